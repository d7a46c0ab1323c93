"""Pins of the oracle against what the pages fix: printed worked examples (tests/golden/,
each with its citation), closed forms, invariants and special cases. CPU only."""
import json
import math
from pathlib import Path

import numpy as np
import pytest

from oracle import mbert_oracle as O

GOLD = Path(__file__).parent / "golden"


def gold(name):
    return json.loads((GOLD / name).read_text())


def printed_equal(values, printed, decimals):
    """``values`` print as ``printed`` when rounded to ``decimals`` places."""
    return np.all(np.abs(np.asarray(values) - np.asarray(printed)) <= 0.5 * 10.0 ** -decimals + 1e-12)


def f32_ulp(x):
    return float(np.spacing(np.float32(abs(x))))


# ------------------------------------------------------------------------------ LayerNorm
def test_layernorm_worked_example():
    g = gold("layernorm_example.json")
    x = np.array(g["input"])
    out = O.layernorm(x, np.ones(4), eps=0.0)
    assert printed_equal(out, g["output"], g["decimals"])
    # the example's mean and (biased) spread, which the normalisation divides by
    assert printed_equal(x.mean(), g["mean"], 4)
    assert printed_equal(np.sqrt(((x - x.mean()) ** 2).mean()), g["std"], 4)


def test_layernorm_properties():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 768)) * 3 + 1.5
    w = 1 + 0.02 * rng.standard_normal(768)
    eps = 1e-5
    y1 = O.layernorm(x, np.ones(768), eps)
    var = x.var(axis=-1)
    assert np.allclose(y1.mean(axis=-1), 0, atol=1e-12)
    assert np.allclose(y1.var(axis=-1), var / (var + eps), rtol=1e-12)
    # weight-only: the weight multiplies, no bias is added
    assert np.allclose(O.layernorm(x, w, eps), y1 * w, rtol=1e-14)
    # shift invariance
    assert np.allclose(O.layernorm(x + 7.0, w, eps), O.layernorm(x, w, eps), atol=1e-10)


# ------------------------------------------------------------------------------ attention core
def test_attention_seed0_table():
    torch = pytest.importorskip("torch")
    g = gold("attention_seed0.json")
    torch.manual_seed(0)
    X = torch.randn(4, 8)
    Wq = torch.randn(8, 4)
    Wk = torch.randn(8, 4)
    Wv = torch.randn(8, 4)
    X, Wq, Wk, Wv = (t.double().numpy() for t in (X, Wq, Wk, Wv))
    Wq, Wk, Wv = (W / math.sqrt(8) for W in (Wq, Wk, Wv))
    Q, K, V = X @ Wq, X @ Wk, X @ Wv
    p = O.attention_probs(Q, K, np.ones((4, 4), dtype=bool))
    assert printed_equal(p, g["weights"], g["decimals"])
    assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-15)
    # the per-sequence attention gives the weighted blend of the values
    o = O.attention_sequence(Q[:, None], K[:, None], V[:, None], True, 64)[:, 0]
    assert np.allclose(o, p @ V, atol=1e-14)


def test_attention_rows_sum_to_one():
    rng = np.random.default_rng(1)
    L, hd = 200, 64
    q, k = rng.standard_normal((L, hd)), rng.standard_normal((L, hd))
    pos = np.arange(L)
    for glob in (True, False):
        p = O.attention_probs(q, k, O.band_allowed(pos, pos, glob, 64))
        assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-13)
        assert np.all(p >= 0)


def test_non_causal_dropping_last_token_changes_earlier_rows():
    """Encoder-only models, 'Bidirectional attention: delete the mask': dropping the last
    token moves the earlier outputs; under a causal mask the gap is exactly 0."""
    rng = np.random.default_rng(2)
    L, hd = 4, 8
    q, k, v = (rng.standard_normal((L, hd)) for _ in range(3))
    full = O.attention_probs(q, k, np.ones((L, L), bool)) @ v
    drop = O.attention_probs(q[:-1], k[:-1], np.ones((L - 1, L - 1), bool)) @ v[:-1]
    assert np.max(np.abs(full[:-1] - drop)) > 1e-3
    causal = np.tril(np.ones((L, L), bool))
    full_c = O.attention_probs(q, k, causal) @ v
    drop_c = O.attention_probs(q[:-1], k[:-1], np.tril(np.ones((L - 1, L - 1), bool))) @ v[:-1]
    assert np.max(np.abs(full_c[:-1] - drop_c)) == 0.0
    # and the encoder layer itself is non-causal on a whole model (tiny dims)
    from workloads import Dims, make_weights
    cfg = O.Config(n_layers=2, hidden=16, n_heads=2, head_dim=8, intermediate=12, vocab=50,
                   half_window=2)
    w = make_weights(Dims(2, 16, 2, 8, 12, 50), "f32", 11)
    ids = np.array([3, 9, 17, 4, 44])
    a, _ = O.encode(ids, [0, 5], w, cfg)
    b, _ = O.encode(ids[:-1], [0, 4], w, cfg)
    assert np.max(np.abs(a[:-1] - b)) > 1e-3


def test_zero_pad_masked_is_invisible_unmasked_is_not():
    """Encoder-only models, 'Padding and the key padding mask': a pad with zero key and value,
    masked, leaves the real outputs exactly unchanged; unmasked, it takes weight > 0."""
    rng = np.random.default_rng(3)
    hd = 8
    q, k, v = (rng.standard_normal((3, 1, hd)) for _ in range(3))
    alone = O.attention_sequence(q, k, v, True, 64)
    qp = np.concatenate([q, rng.standard_normal((1, 1, hd))])
    kp = np.concatenate([k, np.zeros((1, 1, hd))])
    vp = np.concatenate([v, np.zeros((1, 1, hd))])
    masked = O.attention_sequence(qp, kp, vp, True, 64, key_valid=np.array([1, 1, 1, 0]))
    assert np.max(np.abs(masked[:3] - alone)) == 0.0
    unmasked = O.attention_sequence(qp, kp, vp, True, 64)
    p = O.attention_probs(qp[:3, 0], kp[:, 0], np.ones((3, 4), bool))
    assert np.all(p[:, 3] > 0)
    assert np.max(np.abs(unmasked[:3] - alone)) > 1e-3


def _whole_band_attention(q, k, v, is_global, W, key_valid):
    """The plain definition over the whole sequence at once: one [L, L] allowed matrix, no
    query blocks and no clipped key window."""
    L, H, _ = q.shape
    pos = np.arange(L)
    allowed = O.band_allowed(pos, pos, is_global, W)
    if key_valid is not None:
        allowed = allowed & np.asarray(key_valid, bool)[None, :]
    out = np.zeros_like(q)
    for h in range(H):
        out[:, h] = O.attention_probs(q[:, h], k[:, h], allowed) @ v[:, h]
    return out


@pytest.mark.parametrize("L", [1025, 2300])
@pytest.mark.parametrize("is_global,W", [(True, 64), (False, 64), (False, 3)])
@pytest.mark.parametrize("masked", [False, True], ids=["all_keys", "key_mask"])
def test_attention_sequence_blocking_equals_whole_band(L, is_global, W, masked):
    """The oracle's attention walks queries in chunks and, on local layers, scores only the
    keys [a - W, b + W) that a chunk [a, b) can reach. Both are bookkeeping: for every chunk
    size the result must be the plain whole-sequence definition (kgptalkie, "How Does
    Self-Attention Work?"; candding, "ModernBERT", "The alternating attention": a key j is
    read by query i iff |i - j| <= W). Chunks of 1 and 7 put boundaries everywhere, 1024 is
    the default (a ragged last chunk at L = 1025 and 2300), L is one chunk. An off-by-one in
    the clipped window drops or adds the edge key of a chunk's first or last query."""
    rng = np.random.default_rng([L, W, int(is_global), int(masked)])
    H, hd = 2, 8
    q, k, v = (2.0 * rng.standard_normal((L, H, hd)) for _ in range(3))
    key_valid = None
    if masked:
        key_valid = rng.random(L) > 0.3
        key_valid[:: 97] = True  # every local band keeps some real key
    ref = _whole_band_attention(q, k, v, is_global, W, key_valid)
    for chunk in (1, 7, 1024, L):
        got = O.attention_sequence(q, k, v, is_global, W, key_valid=key_valid, chunk=chunk)
        assert np.max(np.abs(got - ref)) <= 1e-12, chunk
    # the comparison is sharp: dropping the last key of each chunk's window is caught
    if not is_global:
        pos = np.arange(L)
        a, b = 0, 7
        allowed = O.band_allowed(pos[a:b], pos[max(0, a - W):b + W - 1], False, W)
        p = O.attention_probs(q[a:b, 0], k[max(0, a - W):b + W - 1, 0], allowed)
        wrong = p @ v[max(0, a - W):b + W - 1, 0]
        if not masked:
            assert np.max(np.abs(wrong[-1] - ref[b - 1, 0])) > 1e-6


# ------------------------------------------------------------------------------ window / schedule
def test_global_layer_schedule():
    g = gold("window_counts.json")
    assert O.global_layers(O.Config()) == g["global_layers"]
    assert len(O.global_layers(O.Config())) == 8


@pytest.mark.parametrize("case", gold("window_counts.json")["cases"])
def test_window_key_counts(case):
    L, qi = case["length"], case["query"]
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((L, 64)) * 0.1, rng.standard_normal((L, 64)) * 0.1
    pos = np.arange(L)
    for glob, key in ((True, "global_keys"), (False, "local_keys")):
        if key not in case:
            continue
        p = O.attention_probs(q, k, O.band_allowed(pos, pos, glob, 64))
        assert int((p[qi] > 0).sum()) == case[key]
        assert int(O.band_allowed(pos, pos, glob, 64)[qi].sum()) == case[key]


def test_window_is_inclusive_not_64_or_128():
    """candding, 'ModernBERT', 'Pitfalls': an exclusive 64 or a 128 half-width are wrong."""
    pos = np.arange(300)
    allowed = O.band_allowed(pos, pos, False, 64)[100]
    assert allowed[36] and allowed[164] and not allowed[35] and not allowed[165]


def test_pair_counts_at_8192():
    g = gold("window_counts.json")["pairs_at_8192"]
    n = g["n"]
    lo_g, hi_g = O.key_ranges([0, n], True, 64)
    lo_l, hi_l = O.key_ranges([0, n], False, 64)
    pg = int((hi_g - lo_g + 1).sum())
    pl = int((hi_l - lo_l + 1).sum())
    assert pg == g["global"] and pl == g["local"]
    assert round(pg / pl, 1) == g["ratio"]


def test_key_ranges_match_band_and_segments():
    cu = [0, 1, 66, 66, 200, 330]
    for glob in (True, False):
        lo, hi = O.key_ranges(cu, glob, 64)
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            if b == a:
                continue
            pos = np.arange(b - a)
            allowed = O.band_allowed(pos, pos, glob, 64)
            for i in range(b - a):
                js = np.nonzero(allowed[i])[0]
                assert lo[a + i] == a + js.min() and hi[a + i] == a + js.max()
                assert len(js) == js.max() - js.min() + 1  # contiguous


# ------------------------------------------------------------------------------ RoPE
def test_rope_inv_freq_printed_values():
    g = gold("rope_inv_freq.json")
    fg = O.rope_inv_freq(g["theta_global"], g["head_dim"])
    fl = O.rope_inv_freq(g["theta_local"], g["head_dim"])
    assert abs(fg[-1] - g["slowest_global"]) <= f32_ulp(g["slowest_global"])
    assert abs(fl[-1] - g["slowest_local"]) <= f32_ulp(g["slowest_local"])
    assert printed_equal(8191 * fg[-1], g["turn_over_8191_tokens_global"], g["decimals_turn"])
    assert fg[0] == 1.0 and fl[0] == 1.0
    assert np.all(np.diff(fg) < 0)  # first pair turns fastest


def test_rope_rotate_half_pairing():
    """candding, 'ModernBERT', 'The two rope tables': rotate-half over the full head, so
    dimension i pairs with i + 32 (not with i + 1)."""
    x = np.zeros((1, 64))
    x[0, 0] = 1.0
    y = O.rope(x, np.array([1]), 10000.0)
    assert np.isclose(y[0, 0], math.cos(1.0)) and np.isclose(y[0, 32], math.sin(1.0))
    assert np.count_nonzero(np.abs(y) > 1e-15) == 2
    x = np.zeros((1, 64))
    x[0, 40] = 1.0  # second half, pair 8: turns by 1 * 10000^(-16/64)
    a = 10000.0 ** (-16 / 64)
    y = O.rope(x, np.array([1]), 10000.0)
    assert np.isclose(y[0, 40], math.cos(a)) and np.isclose(y[0, 8], -math.sin(a))


def test_rope_invariants():
    rng = np.random.default_rng(5)
    T = 50
    pos = rng.integers(0, 8192, size=T)
    x = rng.standard_normal((3, T, 64))
    for theta in (160000.0, 10000.0):
        y = O.rope(x, pos, theta)
        # norm of every (i, i+32) pair is preserved, hence the vector norm too
        assert np.allclose(x[..., :32] ** 2 + x[..., 32:] ** 2, y[..., :32] ** 2 + y[..., 32:] ** 2)
        assert np.allclose(np.linalg.norm(x, axis=-1), np.linalg.norm(y, axis=-1))
        # position 0 is the identity
        assert np.allclose(O.rope(x, np.zeros(T, int), theta), x, atol=0)
        # q(p) . k(p') depends only on p - p'
        q, k = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
        d1 = (O.rope(q, np.array([7]), theta) * O.rope(k, np.array([3]), theta)).sum()
        d2 = (O.rope(q, np.array([1007]), theta) * O.rope(k, np.array([1003]), theta)).sum()
        assert np.isclose(d1, d2, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------------------------ GELU / GeGLU
def test_gelu_printed_values():
    g = gold("gelu_values.json")
    assert printed_equal(O.gelu_erf(np.array(g["inputs"])), g["outputs"], g["decimals"])
    v = float(O.gelu_erf(1.0))
    assert abs(v - g["gelu_erf_at_1"]) <= f32_ulp(g["gelu_erf_at_1"])
    assert abs(v - g["gelu_tanh_at_1"]) > 1e-4


def test_geglu_first_half_is_activated():
    """candding, 'The feed-forward halves'; modernbert-base (Linnet), 'The fused projections':
    the first half of Wi's output goes through GELU, the second half multiplies it."""
    u = np.array([[1.0, 1.0, 1.0, 2.0, 2.0, 2.0]])
    m = O.geglu(u, 3)
    assert np.allclose(m, 2.0 * O.gelu_erf(1.0))
    assert not np.allclose(m, 1.0 * O.gelu_erf(2.0))


# ------------------------------------------------------------------------------ structure
def test_qkv_split_order():
    cfg = O.Config()
    qkv = np.tile(np.arange(3 * 768, dtype=np.float64), (2, 1))
    q, k, v = O.split_qkv(qkv, cfg)
    assert q.shape == (2, 12, 64)
    assert q[0, 5, 7] == 5 * 64 + 7 and k[1, 0, 0] == 768 and v[0, 11, 63] == 2303


def test_parameter_counts():
    g = gold("parameter_counts.json")
    shapes = O.parameter_shapes(O.Config())
    n = {k: int(np.prod(s)) for k, s in shapes.items()}
    assert len(shapes) == g["n_tensors"]
    assert sum(n.values()) == g["total"]
    assert n["embeddings.tok_embeddings.weight"] == g["embedding"]
    assert n["layers.1.attn.Wqkv.weight"] + n["layers.1.attn.Wo.weight"] == g["attention_per_layer"]
    assert n["layers.1.mlp.Wi.weight"] + n["layers.1.mlp.Wo.weight"] == g["mlp_per_layer"]
    assert sum(v for k, v in n.items() if k.startswith("layers.")) == g["layers_total"]
    assert "layers.0.attn_norm.weight" not in shapes and "layers.1.attn_norm.weight" in shapes
    assert not any("bias" in k for k in shapes)


def test_generator_matches_parameter_shapes():
    from workloads import Dims, make_weights
    w = make_weights(Dims(n_layers=3, vocab=64), "bf16", 99)
    shapes = O.parameter_shapes(O.Config(n_layers=3, vocab=64))
    assert w["tok_emb"].shape == shapes["embeddings.tok_embeddings.weight"]
    assert w["layers"][0]["attn_norm"] is None
    for i in range(3):
        for key, name in (("Wqkv", "attn.Wqkv"), ("attn_Wo", "attn.Wo"), ("Wi", "mlp.Wi"),
                          ("mlp_Wo", "mlp.Wo"), ("mlp_norm", "mlp_norm")):
            assert w["layers"][i][key].shape == shapes[f"layers.{i}.{name}.weight"]


# ------------------------------------------------------------------------------ unpad / pool
def test_unpad_against_flat_index_definition():
    rng = np.random.default_rng(6)
    B, Tp = 6, 40
    lengths = np.array([40, 0, 1, 17, 39, 5])
    mask = (np.arange(Tp)[None, :] < lengths[:, None]).astype(int)
    ids_pad = rng.integers(0, 50368, size=(B, Tp))
    u = O.unpad(ids_pad, mask)
    flat = np.flatnonzero(mask.ravel())
    assert np.array_equal(u["indices"], flat)
    assert np.array_equal(u["ids"], ids_pad.ravel()[flat])
    assert np.array_equal(u["cu_seqlens"], np.concatenate([[0], np.cumsum(lengths)]))
    assert np.array_equal(u["pos"], flat % Tp)  # right padding: rank == column
    assert u["max_seqlen"] == 40
    assert np.array_equal(O.positions(u["cu_seqlens"]), u["pos"])


def test_mean_pool_normalize():
    rng = np.random.default_rng(7)
    out = rng.standard_normal((10, 768))
    cu = [0, 4, 4, 10]
    p = O.mean_pool_normalize(out, cu)
    assert np.allclose(np.linalg.norm(p[[0, 2]], axis=-1), 1.0)
    assert np.all(p[1] == 0)
    m = out[4:10].mean(axis=0)
    assert np.allclose(p[2], m / np.linalg.norm(m))


def _tiny():
    from workloads import Dims, make_weights
    cfg = O.Config(n_layers=4, hidden=16, n_heads=2, head_dim=8, intermediate=12, vocab=50,
                   half_window=2)
    w = make_weights(Dims(4, 16, 2, 8, 12, 50), "f32", 12)
    return cfg, w


def test_packed_equals_padded():
    from workloads import pad_batch
    cfg, w = _tiny()
    rng = np.random.default_rng(8)
    lengths = [5, 1, 9, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ids = rng.integers(0, 50, size=cu[-1])
    out, pooled = O.encode(ids, cu, w, cfg)
    ids_pad, mask = pad_batch(ids, cu, 9, pad_id=3)
    out_p, pooled_p = O.encode_padded(ids_pad, mask, w, cfg)
    u = O.unpad(ids_pad, mask)
    assert np.allclose(O.repad(out, u["indices"], 5, 9), out_p, atol=1e-12)
    assert np.allclose(pooled, pooled_p, atol=1e-12)


def test_pooled_in_batch_equals_alone():
    """kgptalkie, 'How Do We Get One Vector per Text?': a text's pooled vector inside a padded
    batch equals the same text run alone."""
    cfg, w = _tiny()
    rng = np.random.default_rng(9)
    a, b = rng.integers(0, 50, size=8), rng.integers(0, 50, size=3)
    _, pooled = O.encode(np.concatenate([a, b]), [0, 8, 11], w, cfg)
    _, alone = O.encode(b, [0, 3], w, cfg)
    assert np.allclose(pooled[1], alone[0], atol=1e-12)


def test_theta_by_layer_kind():
    """kgptalkie, 'How Does RoPE Work With Two Bases?': global layers rotate with base
    160000, local layers with base 10000. Changing only the local base must leave a global
    layer's output unchanged and move a local layer's output (and vice versa)."""
    from dataclasses import replace
    cfg, w = _tiny()
    rng = np.random.default_rng(10)
    x = rng.standard_normal((9, 16))
    seg, pos = [(0, 9, None)], np.arange(9)
    for layer, glob in ((0, True), (1, False), (3, True)):
        base = O.encoder_layer(x, w["layers"][layer], layer, seg, pos, cfg)
        other_local = O.encoder_layer(x, w["layers"][layer], layer, seg, pos,
                                      replace(cfg, theta_local=777.0))
        other_global = O.encoder_layer(x, w["layers"][layer], layer, seg, pos,
                                       replace(cfg, theta_global=777.0))
        assert np.array_equal(base, other_local) == glob
        assert np.array_equal(base, other_global) == (not glob)
