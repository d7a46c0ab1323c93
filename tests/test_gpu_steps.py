"""Per-step parity: every per-step entry point of the C ABI against the oracle's step on the
same seeded inputs. Integer outputs bit-exact; float outputs within TOL_STEP of the oracle's
float64 result (max |err| / max |ref|). Sizes span several 128-row tiles plus a ragged tail."""
import numpy as np
import pytest

from gpu_util import (TOL_STEP, dev, dev_i32, expected_tiles, host, meta_for, rel_err,
                      meta_order, split_meta, torch)
from oracle import mbert_oracle as O
from workloads import (WORKLOADS, cu_from_lengths, draw_lengths, make_batch, pad_batch,
                       random_matrix, rng)

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "bf16", "f16"]
LENGTH_CASES = {
    "one300": [300],
    "edges": [1, 64, 65, 129, 130, 0, 7, 256, 127, 128],
    "one1000": [1000],
    "stream": [8192, 1, 8192, 2001],  # >= 16384 rows: the streaming loads and stores
}


def B():
    from transformer_encoder_amd import binding
    return binding


def dt(name):
    return B().DTYPES[name]


def c4_lengths():
    return draw_lengths(WORKLOADS[4], rng(4, 1))


# ---------------------------------------------------------------------------- meta (exact)
@pytest.mark.parametrize("lengths", [[300], LENGTH_CASES["edges"], [8192], [0], [5, 0, 0, 3],
                                     "c4"], ids=["300", "edges", "8192", "empty", "zeros", "c4"])
def test_pack_meta_bit_exact(lengths):
    if lengths == "c4":
        lengths = list(c4_lengths())
    cu = cu_from_lengths(lengths)
    T, S = int(cu[-1]), len(lengths)
    m = host(meta_for(cu, T))
    counts, pos, first, tiles = split_meta(m, T, S)
    exp_tiles, exp_first = expected_tiles(cu, B().mbert_tile_tokens())
    assert list(counts[:4]) == [T, max(lengths), len(exp_tiles), 0]
    assert np.array_equal(pos, O.positions(cu))
    assert np.array_equal(first, exp_first)
    assert np.array_equal(tiles, exp_tiles)
    check_order(meta_order(m, T, S), exp_tiles)


def check_order(order, tiles):
    """The attention's dispatch order: a permutation of the tiles in which the sequences'
    key-tile counts (64 keys each, capped at 128) never increase, each sequence's tiles
    together and in row order."""
    assert sorted(order.tolist()) == list(range(len(tiles)))
    if len(tiles) == 0:
        return
    L = tiles[order, 3] - tiles[order, 2]
    key = np.minimum((L + 63) // 64, 128)
    assert np.all(np.diff(key) <= 0)
    seq = tiles[order, 2]
    for s0 in np.unique(seq):
        idx = np.flatnonzero(seq == s0)
        assert np.all(np.diff(idx) == 1)                      # together
        assert np.all(np.diff(tiles[order[idx], 0]) > 0)       # in row order


@pytest.mark.parametrize("cu,total,bit", [([0, 5, 3], 3, 1), ([0, 4, 8], 9, 1), ([1, 4], 4, 1),
                                          ([0, 8193], 8193, 2)])
def test_pack_meta_rejects_bad_cu(cu, total, bit):
    S = len(cu) - 1
    meta = torch().zeros(B().mbert_meta_ints(total, S), dtype=torch().int32, device="cuda")
    B().mbert_pack_meta(dev_i32(cu), S, total, 8192, meta)
    st = B().mbert_read_status(meta)
    assert st[3] & bit and st[2] == 0


def _unpad_gpu(ids_pad, mask, max_pos=8192):
    Bn, Tp = mask.shape
    t = torch()
    Tm = Bn * Tp
    bufs = {k: t.full((max(Tm, 1),), -5, dtype=t.int32, device="cuda") for k in ("ids", "indices", "rowmap")}
    cu = t.full((Bn + 1,), -5, dtype=t.int32, device="cuda")
    meta = t.full((B().mbert_meta_ints(Tm, Bn),), -5, dtype=t.int32, device="cuda")
    B().mbert_unpad(dev_i32(ids_pad), dev_i32(mask), Bn, Tp, max_pos, bufs["ids"], bufs["indices"],
                    bufs["rowmap"], cu, meta)
    return {k: host(v) for k, v in bufs.items()}, host(cu), host(meta)


def test_unpad_bit_exact_padded_workload():
    b = make_batch(WORKLOADS[2])
    ref = O.unpad(b["ids_pad"], b["mask"])
    got, cu, meta = _unpad_gpu(b["ids_pad"], b["mask"])
    Bn, Tp = b["mask"].shape
    T = len(ref["ids"])
    counts, pos, first, tiles = split_meta(meta, Bn * Tp, Bn)
    assert list(counts[:4]) == [T, ref["max_seqlen"], len(expected_tiles(ref["cu_seqlens"], 128)[0]), 0]
    assert np.array_equal(cu, ref["cu_seqlens"])
    assert np.array_equal(got["ids"][:T], ref["ids"])
    assert np.array_equal(got["indices"][:T], ref["indices"])
    assert np.array_equal(pos[:T], ref["pos"])
    rowmap = np.full(Bn * Tp, -1)
    rowmap[ref["indices"]] = np.arange(T)
    assert np.array_equal(got["rowmap"], rowmap)
    assert np.array_equal(tiles, expected_tiles(ref["cu_seqlens"], 128)[0])
    check_order(meta_order(meta, Bn * Tp, Bn), tiles)


def test_unpad_edges_and_holes():
    g = np.random.default_rng(5)
    mask = np.zeros((5, 300), dtype=np.int64)
    mask[1] = 1                       # full row
    mask[2, :1] = 1                   # one token
    mask[3, ::3] = 1                  # holes: positions are ranks among real tokens
    mask[4, :257] = 1
    ids_pad = g.integers(0, 50368, size=mask.shape)
    ref = O.unpad(ids_pad, mask)
    got, cu, meta = _unpad_gpu(ids_pad, mask)
    T = len(ref["ids"])
    counts, pos, _, _ = split_meta(meta, mask.size, 5)
    assert counts[0] == T and counts[3] == 0
    assert np.array_equal(cu, ref["cu_seqlens"])
    assert np.array_equal(got["ids"][:T], ref["ids"]) and np.array_equal(pos[:T], ref["pos"])
    assert np.array_equal(got["indices"][:T], ref["indices"])
    mask[0, 3] = 2
    _, _, meta = _unpad_gpu(ids_pad, mask)
    assert meta[3] & B().STATUS_BAD_MASK


@pytest.mark.parametrize("shape", [(4, 4096), (5, 4000), (1, 16385), (3, 1), (3, 0), (0, 5)],
                         ids=["16384-one-workgroup", "20000-three-kernels", "16385", "3x1", "3x0",
                              "0x5"])
def test_unpad_both_paths_bit_exact(shape):
    """Up to 16,384 slots the unpadding runs as one workgroup (one scan pass over the slots),
    beyond as three kernels (count, scan, compact); random masks with holes, an empty row and a
    full row, against the oracle bit for bit, then a row over max_positions and a mask value
    of 2 flagging their status bits the same way."""
    g = np.random.default_rng(shape[0] * 100003 + shape[1])
    mask = (g.random(shape) < 0.6).astype(np.int64)
    if shape[0] > 0:
        mask[0] = 1
    if shape[0] > 2:
        mask[1] = 0
    ids_pad = g.integers(0, 50368, size=shape)
    ref = O.unpad(ids_pad, mask)
    got, cu, meta = _unpad_gpu(ids_pad, mask, max_pos=max(8192, shape[1]))
    T, Bn = len(ref["ids"]), shape[0]
    counts, pos, first, tiles = split_meta(meta, mask.size, Bn)
    assert list(counts[:4]) == [T, ref["max_seqlen"], len(expected_tiles(ref["cu_seqlens"], 128)[0]), 0]
    assert np.array_equal(cu, ref["cu_seqlens"])
    assert np.array_equal(got["ids"][:T], ref["ids"]) and np.array_equal(pos[:T], ref["pos"])
    assert np.array_equal(got["indices"][:T], ref["indices"])
    rowmap = np.full(mask.size, -1)
    rowmap[ref["indices"]] = np.arange(T)
    assert np.array_equal(got["rowmap"][:mask.size], rowmap)  # (buffers hold at least one entry)
    assert np.array_equal(tiles, expected_tiles(ref["cu_seqlens"], 128)[0])
    if ref["max_seqlen"] > 1:
        _, _, meta = _unpad_gpu(ids_pad, mask, max_pos=int(ref["max_seqlen"]) - 1)
        assert meta[3] & B().STATUS_TOO_LONG
    if mask.size:
        mask[-1, -1] = 2
        _, _, meta = _unpad_gpu(ids_pad, mask, max_pos=max(8192, shape[1]))
        assert meta[3] & B().STATUS_BAD_MASK and not meta[3] & B().STATUS_TOO_LONG


@pytest.mark.parametrize("case", list(LENGTH_CASES) + ["c4"])
@pytest.mark.parametrize("W", [64, 3, 0])
def test_key_ranges_bit_exact(case, W):
    lengths = list(c4_lengths()) if case == "c4" else LENGTH_CASES[case]
    cu = cu_from_lengths(lengths)
    T, S = int(cu[-1]), len(lengths)
    meta = meta_for(cu, T)
    t = torch()
    for glob in (True, False):
        lo = t.full((T,), -9, dtype=t.int32, device="cuda")
        hi = t.full((T,), -9, dtype=t.int32, device="cuda")
        B().mbert_attn_key_ranges(meta, T, S, glob, W, lo, hi)
        rlo, rhi = O.key_ranges(cu, glob, W)
        assert np.array_equal(host(lo), rlo) and np.array_equal(host(hi), rhi)


def test_rope_tables():
    cfg = B().mbert_default_config()
    tab = torch().empty(B().mbert_rope_table_floats(cfg), dtype=torch().float32, device="cuda")
    B().mbert_build_rope_tables(cfg, tab)
    got = host(tab).reshape(2, 8192, 32, 2)
    p = np.arange(8192, dtype=np.float64)[:, None]
    for t, theta in enumerate((160000.0, 10000.0)):
        ang = p * O.rope_inv_freq(theta, 64)[None, :]
        assert np.max(np.abs(got[t, :, :, 0] - np.cos(ang))) < 1.2e-7
        assert np.max(np.abs(got[t, :, :, 1] - np.sin(ang))) < 1.2e-7


# ---------------------------------------------------------------------------- row kernels
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("T", [333, 20001], ids=["333", "20001"])
def test_embed_ln(dtype, T):
    """333 rows: the cached stores; 20001 rows (odd, at least 16384): the streaming stores
    and a wave whose second row is past the end."""
    V = 1000
    from workloads import round_to
    E = round_to(random_matrix((V, 768), 31) + 0.3, dtype)
    w = round_to(1 + random_matrix(768, 32) * 0.05, dtype)
    ids = np.random.default_rng(33).integers(0, V, size=T)
    ids[:2] = [0, V - 1]
    t = torch()
    resid = t.empty((T, 768), dtype=t.float32, device="cuda")
    h = t.empty((T, 768), dtype=t.float32 if dtype == "f32" else
                {"bf16": t.bfloat16, "f16": t.float16}[dtype], device="cuda")
    B().mbert_embed_ln(dt(dtype), dev_i32(ids), T, None, dev(E, dtype), V, dev(w, dtype), 1e-5,
                       resid, h)
    ref = O.embed(ids, {"tok_emb": E, "emb_norm": w}, O.Config(vocab=V))
    assert rel_err(host(resid), ref) < TOL_STEP["f32"]
    assert rel_err(host(h), ref) < TOL_STEP[dtype]


def test_embed_ln_bad_id_flags_status():
    V, T = 100, 5
    E = random_matrix((V, 768), 34, dtype="bf16")
    w = np.ones(768)
    ids = np.array([1, 2, V, -1, 3])
    meta = meta_for([0, T], T)
    t = torch()
    resid = t.empty((T, 768), dtype=t.float32, device="cuda")
    h = t.empty((T, 768), dtype=t.bfloat16, device="cuda")
    B().mbert_embed_ln(dt("bf16"), dev_i32(ids), T, meta, dev(E, "bf16"), V, dev(w, "bf16"), 1e-5,
                       resid, h)
    assert B().mbert_read_status(meta)[3] & B().STATUS_BAD_ID
    ref = O.embed([0], {"tok_emb": E, "emb_norm": w}, O.Config(vocab=V))
    assert rel_err(host(resid)[2], ref[0]) < 3e-5
    # a bad id in a row past the device row count is not a real row: no status bit
    meta2 = meta_for([0, 3], 3)
    ids2 = np.array([1, 2, 3, V + 5])
    B().mbert_embed_ln(dt("bf16"), dev_i32(ids2), 4, meta2, dev(E, "bf16"), V, dev(w, "bf16"), 1e-5,
                       resid, h)
    assert not (B().mbert_read_status(meta2)[3] & B().STATUS_BAD_ID)


@pytest.mark.parametrize("dtype", DTYPES)
def test_layernorm(dtype):
    T = 517
    from workloads import round_to
    x = round_to(random_matrix((T, 768), 41) * 3 + 0.7, "f32")
    w = round_to(1 + np.random.default_rng(42).standard_normal(768) * 0.02, dtype)
    t = torch()
    y = t.empty((T, 768), dtype={"f32": t.float32, "bf16": t.bfloat16, "f16": t.float16}[dtype],
                device="cuda")
    B().mbert_layernorm(dt(dtype), dev(x, "f32"), T, None, dev(w, dtype), 1e-5, y)
    assert rel_err(host(y), O.layernorm(x, w, 1e-5)) < TOL_STEP[dtype]


# ---------------------------------------------------------------------------- GEMMs
def _tdt(dtype):
    t = torch()
    return {"f32": t.float32, "bf16": t.bfloat16, "f16": t.float16}[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("lengths", [[120, 180], [8192], [8192, 8192, 131]],
                         ids=["300", "8192", "16515"])
@pytest.mark.parametrize("table", [0, 1, None], ids=["global", "local", "norope"])
def test_qkv_projection(dtype, lengths, table):
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    h = random_matrix((T, 768), 51, dtype=dtype)
    W = random_matrix((2304, 768), 52, dtype=dtype, std=0.02)
    cfg = B().mbert_default_config()
    rope = torch().empty(B().mbert_rope_table_floats(cfg), dtype=torch().float32, device="cuda")
    B().mbert_build_rope_tables(cfg, rope)
    meta = meta_for(cu, T)
    qkv = torch().empty((T, 2304), dtype=_tdt(dtype), device="cuda")
    B().mbert_qkv_rope(dt(dtype), dev(h, dtype), T, meta, dev(W, dtype), rope, 8192, table or 0,
                       table is not None, qkv)
    theta = 160000.0 if table == 0 else 10000.0
    ref = O.qkv_projection(h, W, O.positions(cu), theta, O.Config(), apply_rope=table is not None)
    assert rel_err(host(qkv), ref) < TOL_STEP[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
def test_rope_standalone(dtype):
    cu = cu_from_lengths([77, 300, 5])
    T = int(cu[-1])
    x = random_matrix((T, 2304), 61, dtype=dtype)
    cfg = B().mbert_default_config()
    rope = torch().empty(B().mbert_rope_table_floats(cfg), dtype=torch().float32, device="cuda")
    B().mbert_build_rope_tables(cfg, rope)
    qkv = dev(x, dtype)
    B().mbert_rope(dt(dtype), qkv, T, meta_for(cu, T), rope, 8192, 1, None)
    got = host(qkv)
    q, k, v = O.split_qkv(x, O.Config())
    pos = O.positions(cu)
    rq = O.rope(q.transpose(1, 0, 2), pos, 10000.0).transpose(1, 0, 2).reshape(T, -1)
    rk = O.rope(k.transpose(1, 0, 2), pos, 10000.0).transpose(1, 0, 2).reshape(T, -1)
    assert rel_err(got[:, :768], rq) < TOL_STEP[dtype]
    assert rel_err(got[:, 768:1536], rk) < TOL_STEP[dtype]
    assert np.array_equal(got[:, 1536:], x[:, 1536:])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("K", [768, 1152])
@pytest.mark.parametrize("T", [300, 22000, 45001])
def test_linear_residual(dtype, K, T):
    a = random_matrix((T, K), 71, dtype=dtype)
    W = random_matrix((768, K), 72, dtype=dtype, std=0.02)
    r0 = random_matrix((T, 768), 73, dtype="f32")
    resid = dev(r0, "f32")
    B().mbert_linear_residual(dt(dtype), dev(a, dtype), K, T, None, dev(W, dtype), resid)
    ref = O.residual_linear(r0, a, W)
    assert rel_err(host(resid), ref) < 1e-5


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("T", [300, 4133, 16500])
def test_mlp_in_geglu(dtype, T):
    h = random_matrix((T, 768), 81, dtype=dtype)
    Wi = random_matrix((2304, 768), 82, dtype=dtype, std=0.05)
    m = torch().empty((T, 1152), dtype=_tdt(dtype), device="cuda")
    B().mbert_mlp_in_geglu(dt(dtype), dev(h, dtype), T, None, dev(Wi, dtype), m)
    assert rel_err(host(m), O.mlp_in_geglu(h, Wi, O.Config())) < TOL_STEP[dtype]


def test_geglu_halves_probe():
    """The first half of Wi's rows feeds GELU, the second half multiplies it (candding,
    'The feed-forward halves'): with Wi rows j = a e_0 and 1152 + j = b e_0, h = e_0 gives
    gelu(a) * b, not gelu(b) * a."""
    T = 4
    h = np.zeros((T, 768))
    h[:, 0] = 1.0
    Wi = np.zeros((2304, 768))
    Wi[:1152, 0] = 1.0
    Wi[1152:, 0] = 2.0
    m = torch().empty((T, 1152), dtype=torch().float32, device="cuda")
    B().mbert_mlp_in_geglu(dt("f32"), dev(h, "f32"), T, None, dev(Wi, "f32"), m)
    assert np.allclose(host(m), 2.0 * O.gelu_erf(1.0), rtol=1e-6)


# ---------------------------------------------------------------------------- attention
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("case", ["one300", "edges", "one1000"])
@pytest.mark.parametrize("glob", [True, False], ids=["global", "local"])
@pytest.mark.parametrize("W", [64, 3])
def test_attention(dtype, case, glob, W):
    if glob and W != 64:
        pytest.skip("the window only matters on local layers")
    cu = cu_from_lengths(LENGTH_CASES[case])
    T, S = int(cu[-1]), len(cu) - 1
    qkv = random_matrix((T, 2304), 91, dtype=dtype, std=1.5)
    o = torch().full((T, 768), float("nan"), dtype=_tdt(dtype), device="cuda")
    B().mbert_attention(dt(dtype), dev(qkv, dtype), T, meta_for(cu, T), S, glob, W, o)
    ref = O.attention_varlen(qkv, O.segments_of(cu), glob, O.Config(half_window=W))
    got = host(o)
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) < TOL_STEP[dtype]


@pytest.mark.parametrize("dtype", ["bf16"])
def test_attention_long_global(dtype):
    cu = cu_from_lengths([3000, 2100])
    T, S = int(cu[-1]), 2
    qkv = random_matrix((T, 2304), 92, dtype=dtype, std=1.5)
    for glob in (True, False):
        o = torch().empty((T, 768), dtype=_tdt(dtype), device="cuda")
        B().mbert_attention(dt(dtype), dev(qkv, dtype), T, meta_for(cu, T), S, glob, 64, o)
        ref = O.attention_varlen(qkv, O.segments_of(cu), glob, O.Config())
        assert rel_err(host(o), ref) < TOL_STEP[dtype]


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_attention_random_length_mixes(seed, dtype):
    """Seeded random batches (2-8 sequences of 0-300 tokens, or 2-40 of 0-700: empty
    sequences, single tokens, ragged tails and multi-tile sequences mixed) on both layer kinds
    and several windows; the grid sizes fall on both sides of the split-key bound (256 work
    groups)."""
    g = np.random.default_rng(1000 + seed)
    small = seed < 2  # small batches: grids under the bound
    S = int(g.integers(2, 9 if small else 41))
    lengths = [int(x) for x in g.integers(0, 301 if small else 701, size=S)]
    lengths[int(g.integers(0, S))] = int(g.integers(0, 2))
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    if T == 0:
        pytest.skip("empty batch")
    qkv = random_matrix((T, 2304), 95 + seed, dtype=dtype, std=1.5)
    W = int(g.choice([64, 17, 1]))
    for glob in (True, False):
        o = torch().full((T, 768), float("nan"), dtype=_tdt(dtype), device="cuda")
        B().mbert_attention(dt(dtype), dev(qkv, dtype), T, meta_for(cu, T), S, glob, W, o)
        ref = O.attention_varlen(qkv, O.segments_of(cu), glob, O.Config(half_window=W))
        got = host(o)
        assert np.all(np.isfinite(got)), (lengths, glob, W)
        assert rel_err(got, ref) < TOL_STEP[dtype], (lengths, glob, W)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("glob", [True, False], ids=["global", "local"])
def test_attention_split_and_whole_agree(dtype, glob):
    """A grid of at most one workgroup per CU (256) runs each workgroup's key tiles on two wave
    sets whose softmax states are merged at the end; a larger grid runs them on one. The same
    sequences (the edge lengths) through both: once alone (18 tiles x 12 heads = 216 work
    groups) and three times over (52 x 12 = 624), every copy against the oracle and the two
    runs against each other."""
    one = LENGTH_CASES["edges"]
    cu1, cu3 = cu_from_lengths(one), cu_from_lengths(one * 3)
    T1, T3 = int(cu1[-1]), int(cu3[-1])
    grid = lambda T, S: 12 * ((T + 127) // 128 + S)
    assert grid(T1, len(one)) <= 256 < grid(T3, 3 * len(one))
    qkv1 = random_matrix((T1, 2304), 93, dtype=dtype, std=1.5)
    qkv3 = np.concatenate([qkv1] * 3)
    o1 = torch().full((T1, 768), float("nan"), dtype=_tdt(dtype), device="cuda")
    o3 = torch().full((T3, 768), float("nan"), dtype=_tdt(dtype), device="cuda")
    B().mbert_attention(dt(dtype), dev(qkv1, dtype), T1, meta_for(cu1, T1), len(one), glob, 64, o1)
    B().mbert_attention(dt(dtype), dev(qkv3, dtype), T3, meta_for(cu3, T3), 3 * len(one), glob, 64,
                        o3)
    ref = O.attention_varlen(qkv1, O.segments_of(cu1), glob, O.Config())
    g1, g3 = host(o1), host(o3)
    assert np.all(np.isfinite(g1)) and np.all(np.isfinite(g3))
    assert rel_err(g1, ref) < TOL_STEP[dtype]
    for c in range(3):
        assert rel_err(g3[c * T1:(c + 1) * T1], ref) < TOL_STEP[dtype]
        assert rel_err(g3[c * T1:(c + 1) * T1], g1) < TOL_STEP[dtype]


# ---------------------------------------------------------------------------- final LN + pool
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("case", ["edges", "one1000", "stream"])
def test_final_ln_pool(dtype, case):
    lengths = LENGTH_CASES[case]
    cu = cu_from_lengths(lengths)
    T, S = int(cu[-1]), len(lengths)
    from workloads import round_to
    x = round_to(random_matrix((T, 768), 101) * 2 + 0.1, "f32")
    w = round_to(1 + np.random.default_rng(102).standard_normal(768) * 0.02, dtype)
    t = torch()
    out = t.empty((T, 768), dtype=t.float32, device="cuda")
    pooled = t.full((S, 768), float("nan"), dtype=t.float32, device="cuda")
    part = t.empty(B().mbert_pool_partial_floats(T, S), dtype=t.float32, device="cuda")
    B().mbert_final_ln_pool(dev(x, "f32"), T, meta_for(cu, T), S, dt(dtype), dev(w, dtype), 1e-5,
                            out, pooled, part)
    ref = O.layernorm(x, w, 1e-5)
    assert rel_err(host(out), ref) < 3e-5
    rp = O.mean_pool_normalize(ref, cu)
    assert np.max(np.abs(host(pooled) - rp)) < 2e-5


def test_repad():
    b = make_batch(WORKLOADS[2])
    ref = O.unpad(b["ids_pad"], b["mask"])
    got, _, _ = _unpad_gpu(b["ids_pad"], b["mask"])
    T = len(ref["ids"])
    Bn, Tp = b["mask"].shape
    x = random_matrix((T, 768), 111, dtype="f32")
    t = torch()
    out_pad = t.full((Bn, Tp, 768), float("nan"), dtype=t.float32, device="cuda")
    B().mbert_repad(dev(x, "f32"), dev_i32(got["rowmap"]), Bn, Tp, out_pad)
    assert np.array_equal(host(out_pad), O.repad(x, ref["indices"], Bn, Tp))
