"""The folded LayerNorm one step at a time, in every dtype, against the oracle's LayerNorm
followed by its Linear (candding, "ModernBERT", §"The pre-norm layer and the final norm"):

1. `mbert_linear_residual_stats`: resid += a W^T, plus the new residual rounded to the dtype
   (bit-exact against rounding the GPU's own residual) and its per-64-column chunk mean and
   sum of squared deviations;
2. `mbert_fold_weight` + `mbert_folded_gemm`: the QKV + RoPE and the Wi + GeGLU GEMMs on the
   rounded residual, against O.qkv_projection(O.layernorm(x)) and O.mlp_in_geglu(O.layernorm(x)).

Residual patterns: N(0, 1) rows, and rows carrying three "massive" dimensions of magnitude
3e4 to 5.3e4 (about 81 % of the fp16 maximum: the peak that candding, §"Dtype headroom",
reports for a trained model's residual stream), where the rounded fp16 copy holds values the
LayerNorm output never does. Tolerances: the per-step bar, max |err| / max |ref| <= 3e-5
(fp32), 1e-2 (bf16), 2e-3 (fp16); fp32 residual outputs of 16-bit GEMMs <= 1e-5."""
import numpy as np
import pytest

from gpu_util import TOL_STEP, dev, dev_i32, host, meta_for, rel_err, torch
from oracle import mbert_oracle as O
from workloads import cu_from_lengths, random_matrix

pytestmark = pytest.mark.gpu

MASSIVE_DIMS = (17, 300, 601)


def B():
    from transformer_encoder_amd import binding
    return binding


def _residual(T, pattern, seed):
    g = np.random.default_rng([seed, 7])
    x = g.standard_normal((T, 768))
    if pattern == "massive":
        for d in MASSIVE_DIMS:
            x[:, d] = g.choice([-1.0, 1.0], T) * g.uniform(3.0e4, 5.3e4, T)
    return x.astype(np.float32).astype(np.float64)


def _tdt(dtype):
    t = torch()
    return {"f32": t.float32, "bf16": t.bfloat16, "f16": t.float16}[dtype]


@pytest.mark.parametrize("pattern", ["normal", "massive"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_folded_steps_against_oracle(dtype, pattern):
    t = torch()
    dt = B().DTYPES[dtype]
    cu = cu_from_lengths([450, 1, 249])
    T = int(cu[-1])
    meta = meta_for(cu, T)
    x0 = _residual(T, pattern, 3 if pattern == "normal" else 4)
    a = random_matrix((T, 768), 71, dtype=dtype)
    Wo = random_matrix((768, 768), 72, dtype=dtype, std=0.02)
    resid = t.from_numpy(x0.astype(np.float32)).cuda()
    xs = t.empty((T, 768), dtype=_tdt(dtype), device="cuda")
    stats = t.empty((T, 12, 2), dtype=t.float32, device="cuda")
    B().mbert_linear_residual_stats(dt, dev(a, dtype), 768, T, meta, dev(Wo, dtype), resid,
                                    xs if dtype != "f32" else None, stats)
    x1 = host(resid)
    ref1 = O.residual_linear(x0, a, Wo)
    # the new residual (fp32 storage rounds it relative to its own magnitude), and the
    # update itself on the ordinary columns, where that rounding is far below the update's
    rest = np.setdiff1d(np.arange(768), MASSIVE_DIMS)
    e_all = rel_err(x1, ref1)
    e_upd = rel_err(x1[:, rest] - x0[:, rest], ref1[:, rest] - x0[:, rest])
    print(f"{dtype} {pattern}: residual rel_err={e_all:.3e} update rel_err={e_upd:.3e}", flush=True)
    assert e_all <= 1e-6 and e_upd <= (3e-5 if dtype == "f32" else 1e-5)
    if dtype != "f32":
        assert t.equal(xs, resid.to(_tdt(dtype)))  # rounded once from the new residual
    st = host(stats)
    chunks = x1.reshape(T, 12, 64)
    mean = chunks.mean(axis=2)
    m2 = ((chunks - mean[:, :, None]) ** 2).sum(axis=2)
    scale = np.abs(chunks).max(axis=2)
    assert np.max(np.abs(st[:, :, 0] - mean) / scale) <= 1e-6
    assert np.max(np.abs(st[:, :, 1] - m2) / np.maximum(m2, 1e-30)) <= 1e-4

    # the LayerNorm folded into the QKV + RoPE and Wi + GeGLU GEMMs
    cfg = B().mbert_default_config()
    rope = t.empty(B().mbert_rope_table_floats(cfg), dtype=t.float32, device="cuda")
    B().mbert_build_rope_tables(cfg, rope)
    a_in = xs if dtype != "f32" else resid
    for kind, rows, name in ((B().FOLD_QKV_ROPE, 2304, "qkv"), (B().FOLD_GEGLU, 2304, "geglu")):
        W = random_matrix((rows, 768), 73 + kind, dtype=dtype, std=0.02)
        nw = (1.0 + 0.02 * np.random.default_rng([74 + kind, 0]).standard_normal(768))
        nw = nw.astype(np.float32).astype(np.float64)
        if dtype != "f32":
            nw = host(dev(nw, dtype))  # the norm weight as stored in the dtype
        Wf = t.empty((rows, 768), dtype=_tdt(dtype), device="cuda")
        c = t.empty(rows, dtype=t.float32, device="cuda")
        B().mbert_fold_weight(dt, dev(W, dtype), dev(nw, dtype), rows, Wf, c)
        out_cols = 2304 if kind == B().FOLD_QKV_ROPE else 1152
        out = t.empty((T, out_cols), dtype=_tdt(dtype), device="cuda")
        B().mbert_folded_gemm(dt, kind, a_in, stats, T, meta, Wf, c, 1e-5, rope, 8192, 0, out)
        h = O.layernorm(x1, nw, 1e-5)
        if kind == B().FOLD_QKV_ROPE:
            ref = O.qkv_projection(h, W, O.positions(cu), 160000.0, O.Config())
        else:
            ref = O.mlp_in_geglu(h, W, O.Config())
        e = rel_err(host(out), ref)
        print(f"{dtype} {pattern} folded {name}: rel_err={e:.3e}", flush=True)
        assert e <= TOL_STEP[dtype], name


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("T", [14337, 65537])
def test_folded_persistent_tiles_against_oracle(dtype, T):
    """The folded QKV + RoPE and Wi + GeGLU GEMMs on the persistent 256x256 tiles: 14,337 rows
    (57 row tiles, the last holding one row, so some XCDs' slots have no tile) and 65,537 rows
    (about nine tiles a workgroup, the last again one row). Each against LayerNorm + Linear
    of the oracle on the same rounded residual, at the per-step bar."""
    t = torch()
    dt = B().DTYPES[dtype]
    lengths = [8192] * (T // 8192) + ([T % 8192] if T % 8192 else [])
    cu = cu_from_lengths(lengths)
    meta = meta_for(cu, T)
    x = _residual(T, "normal", 11)
    xs = dev(x, dtype)
    x = host(xs)  # the residual as the GEMM reads it, rounded to the dtype
    chunks = x.reshape(T, 12, 64)
    mean = chunks.mean(axis=2)
    st = np.stack([mean, ((chunks - mean[:, :, None]) ** 2).sum(axis=2)], axis=2)
    stats = t.from_numpy(st.astype(np.float32)).cuda()
    cfg = B().mbert_default_config()
    rope = t.empty(B().mbert_rope_table_floats(cfg), dtype=t.float32, device="cuda")
    B().mbert_build_rope_tables(cfg, rope)
    rows = np.r_[0:300, T // 2 - 150:T // 2 + 150, T - 300:T]  # sampled rows, both ends
    for kind, name in ((B().FOLD_QKV_ROPE, "qkv"), (B().FOLD_GEGLU, "geglu")):
        W = random_matrix((2304, 768), 91 + kind, dtype=dtype, std=0.02)
        nw = host(dev((1.0 + 0.02 * np.random.default_rng([92 + kind, 0]).standard_normal(768)), dtype))
        Wf = t.empty((2304, 768), dtype=_tdt(dtype), device="cuda")
        c = t.empty(2304, dtype=t.float32, device="cuda")
        B().mbert_fold_weight(dt, dev(W, dtype), dev(nw, dtype), 2304, Wf, c)
        out = t.empty((T, 2304 if kind == B().FOLD_QKV_ROPE else 1152), dtype=_tdt(dtype), device="cuda")
        B().mbert_folded_gemm(dt, kind, xs, stats, T, meta, Wf, c, 1e-5, rope, 8192, 1, out)
        h = O.layernorm(x[rows], nw, 1e-5)
        if kind == B().FOLD_QKV_ROPE:
            ref = O.qkv_projection(h, W, O.positions(cu)[rows], 10000.0, O.Config())
        else:
            ref = O.mlp_in_geglu(h, W, O.Config())
        e = rel_err(host(out)[rows], ref)
        print(f"{dtype} T={T} folded {name}: rel_err={e:.3e}", flush=True)
        assert e <= TOL_STEP[dtype], name
