"""End-to-end parity of mbert_encode / mbert_encode_padded against the oracle on the five
workloads (seeded inputs and random-init weights from workloads/).

Tolerances: float32 path max |err| / max |ref| <= 1e-4; 16-bit paths max |err| <= 2e-2 after
the final LayerNorm and cosine >= 0.999 per token and per pooled vector. Workloads 1 and 2
run the oracle live; workloads 3-5 compare sampled rows and the pooled vectors of sampled
sequences with oracle values stored by tests/golden/make_oracle_samples.py."""
from pathlib import Path

import numpy as np
import pytest

from gpu_util import dev_i32, host, min_cos, rel_err, torch
from oracle import mbert_oracle as O
from workloads import WORKLOADS, Dims, make_batch, make_weights, random_batch, workload_weights

pytestmark = pytest.mark.gpu
GOLD = Path(__file__).parent / "golden"

_models = {}


def model_for(wid):
    from transformer_encoder_amd.model import DeviceModel
    if wid not in _models:
        _models.clear()
        torch().cuda.empty_cache()
        _models[wid] = DeviceModel(workload_weights(wid), WORKLOADS[wid].dtype)
    return _models[wid]


def check_16bit(got, ref, what):
    err = float(np.max(np.abs(got - ref)))
    cos = min_cos(got, ref)
    print(f"{what}: max_abs={err:.3e} min_cos={cos:.6f}", flush=True)
    assert err <= 2e-2 and cos >= 0.999, what


def test_w1_fp32_three_layer_cycle():
    wl = WORKLOADS[1]
    b = make_batch(wl)
    m = model_for(1)
    out, pooled, _ = m.encode(dev_i32(b["ids"]), dev_i32(b["cu_seqlens"]))
    ref, rpool = O.encode(b["ids"], b["cu_seqlens"], workload_weights(1), O.Config(n_layers=3))
    e_out, e_pool = rel_err(host(out), ref), rel_err(host(pooled), rpool)
    print(f"w1: rel_err out={e_out:.3e} pooled={e_pool:.3e}", flush=True)
    assert e_out <= 1e-4 and e_pool <= 1e-4


def test_w2_padded_bf16_and_packed_equal():
    wl = WORKLOADS[2]
    b = make_batch(wl)
    m = model_for(2)
    ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
    out_pad, pooled, ws = m.encode_padded(ids_pad, mask)
    ref, rpool = O.encode(b["ids"], b["cu_seqlens"], workload_weights(2), O.Config())
    u = O.unpad(b["ids_pad"], b["mask"])
    got = host(out_pad).reshape(-1, 768)
    check_16bit(got[u["indices"]], ref, "w2 tokens")
    check_16bit(host(pooled), rpool, "w2 pooled")
    pads = np.ones(got.shape[0], bool)
    pads[u["indices"]] = False
    assert np.all(got[pads] == 0.0)
    # the packed cu_seqlens and indices left in the workspace are exact
    L = m.layout(b["mask"].size, b["mask"].shape[0])
    wsn = ws.cpu().numpy()
    cu = np.frombuffer(wsn[L.cu:L.cu + 4 * 9].tobytes(), dtype=np.int32)
    idx = np.frombuffer(wsn[L.indices:L.indices + 4 * len(u["indices"])].tobytes(), dtype=np.int32)
    assert np.array_equal(cu, u["cu_seqlens"]) and np.array_equal(idx, u["indices"])
    # the packed entry point on the unpadded batch gives bitwise the same rows
    out2, pooled2, _ = m.encode(dev_i32(b["ids"]), dev_i32(b["cu_seqlens"]))
    assert np.array_equal(host(out2), got[u["indices"]])
    assert np.array_equal(host(pooled2), host(pooled))


def test_w2_separate_norms_and_fold_agree():
    """The LayerNorms run as separate kernels (the unfolded path) meet the same bar, and the
    two paths agree closely; on the fp32 workload they agree to float rounding."""
    wl = WORKLOADS[2]
    b = make_batch(wl)
    m = model_for(2)
    ids, cu = dev_i32(b["ids"]), dev_i32(b["cu_seqlens"])
    out_f, pool_f, _ = m.encode(ids, cu)
    m.set_fold(False)
    try:
        out_s, pool_s, _ = m.encode(ids, cu)
    finally:
        m.set_fold(True)
    ref, rpool = O.encode(b["ids"], b["cu_seqlens"], workload_weights(2), O.Config())
    check_16bit(host(out_s), ref, "w2 separate norms")
    check_16bit(host(pool_s), rpool, "w2 separate norms pooled")
    check_16bit(host(out_f), host(out_s), "w2 folded vs separate")
    m1 = model_for(1)
    b1 = make_batch(WORKLOADS[1])
    o1f, _, _ = m1.encode(dev_i32(b1["ids"]), dev_i32(b1["cu_seqlens"]))
    m1.set_fold(False)
    try:
        o1s, _, _ = m1.encode(dev_i32(b1["ids"]), dev_i32(b1["cu_seqlens"]))
    finally:
        m1.set_fold(True)
    e = rel_err(host(o1f), host(o1s))
    print(f"w1 folded vs separate: rel_err={e:.3e}", flush=True)
    assert e <= 2e-5


def _sampled(wid):
    f = GOLD / f"oracle_samples_w{wid}.npz"
    if not f.exists():
        pytest.skip(f"{f.name} not generated (tests/golden/make_oracle_samples.py)")
    g = np.load(f, allow_pickle=False)
    b = make_batch(WORKLOADS[wid])
    assert int(g["total"]) == len(b["ids"])
    m = model_for(wid)
    out, pooled, _ = m.encode(dev_i32(b["ids"]), dev_i32(b["cu_seqlens"]))
    o = host(out)
    check_16bit(o[g["rows"]], g["out"].astype(np.float64), f"w{wid} sampled rows")
    check_16bit(host(pooled)[g["seqs"]], g["pooled"].astype(np.float64), f"w{wid} pooled")
    assert np.all(np.isfinite(o))
    nrm = np.linalg.norm(host(pooled), axis=1)
    assert np.allclose(nrm, 1.0, atol=1e-5)


def test_w3_one_8192_sequence_bf16():
    _sampled(3)


def test_w4_loguniform_varlen_bf16():
    _sampled(4)


def test_w5_32x8192_fp16():
    _sampled(5)


@pytest.mark.parametrize("fold", [True, False], ids=["folded", "separate"])
@pytest.mark.parametrize("lengths", [[1], [1, 2, 3], [65, 0, 129], [64, 65, 300, 7]])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_edge_batches_two_layers(lengths, dtype, fold):
    from transformer_encoder_amd.model import DeviceModel
    w = make_weights(Dims(n_layers=2), dtype, 500 + len(lengths))
    b = random_batch(lengths, 77)
    m = DeviceModel(w, dtype, fold=fold)
    assert (m.folded is not None) == fold
    out, pooled, _ = m.encode(dev_i32(b["ids"]), dev_i32(b["cu_seqlens"]))
    ref, rpool = O.encode(b["ids"], b["cu_seqlens"], w, O.Config(n_layers=2))
    if dtype == "f32":
        assert rel_err(host(out), ref) <= 1e-4 and rel_err(host(pooled), rpool) <= 1e-4
    else:
        check_16bit(host(out), ref, f"edges {lengths}")
        nz = [i for i, L in enumerate(lengths) if L > 0]
        check_16bit(host(pooled)[nz], rpool[nz], f"edges pooled {lengths}")
    for i, L in enumerate(lengths):
        if L == 0:
            assert np.all(host(pooled)[i] == 0)


@pytest.mark.parametrize("lengths,tpad", [([37, 0, 5], 37), ([200, 1], 200), ([64, 3, 0, 64, 10], 64)],
                         ids=["3x37", "2x200", "5x64"])
def test_padded_ragged_slots_zero_pads(lengths, tpad):
    """Padded forward on slot counts that are not multiples of 64 (111, 400, 320), into
    outputs filled with NaN first: every pad row comes back exactly zero, every real row and
    pooled vector matches the oracle (an empty row pools to zero)."""
    from transformer_encoder_amd import binding as B
    from transformer_encoder_amd.model import DeviceModel
    w = make_weights(Dims(n_layers=2), "bf16", 900 + len(lengths))
    b = random_batch(lengths, 91)
    Bn = len(lengths)
    ids_pad = np.full((Bn, tpad), 50283, np.int32)
    mask = np.zeros((Bn, tpad), np.int32)
    for i, L in enumerate(lengths):
        ids_pad[i, :L] = b["ids"][b["cu_seqlens"][i]:b["cu_seqlens"][i + 1]]
        mask[i, :L] = 1
    m = DeviceModel(w, "bf16")
    t = torch()
    out = t.full((Bn, tpad, 768), float("nan"), device="cuda")
    pool = t.full((Bn, 768), float("nan"), device="cuda")
    ws = m.workspace(Bn * tpad, Bn)
    B.mbert_encode_padded(m.w, dev_i32(ids_pad), dev_i32(mask), Bn, tpad, ws, ws.numel(), out, pool,
                          None)
    got, gpool = host(out), host(pool)
    ref, rpool = O.encode(b["ids"], b["cu_seqlens"], w, O.Config(n_layers=2))
    real = mask.astype(bool)
    assert np.all(got[~real] == 0.0), "pad rows not zeroed"
    check_16bit(got[real], ref, f"padded {Bn}x{tpad} tokens")
    nz = [i for i, L in enumerate(lengths) if L > 0]
    check_16bit(gpool[nz], rpool[nz], f"padded {Bn}x{tpad} pooled")
    for i, L in enumerate(lengths):
        if L == 0:
            assert np.all(gpool[i] == 0.0)


def test_deterministic_and_graph_replay():
    from transformer_encoder_amd import binding as B
    wl = WORKLOADS[2]
    b = make_batch(wl)
    m = model_for(2)
    t = torch()
    ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
    out1, pool1, ws = m.encode_padded(ids_pad, mask)
    out2, pool2, _ = m.encode_padded(ids_pad, mask, ws=ws)
    ref_out, ref_pool = host(out1), host(pool1)
    assert np.array_equal(ref_out, host(out2)) and np.array_equal(ref_pool, host(pool2))
    s = t.cuda.Stream()
    gout = t.empty_like(out1)
    gpool = t.empty_like(pool1)
    gws = t.empty_like(ws)
    with t.cuda.stream(s):
        g = B.mbert_graph_capture_padded(m.w, ids_pad, mask, 8, 512, gws, gws.numel(), gout, gpool, s)
    try:
        for i in range(3):
            gout.fill_(float("nan"))
            with t.cuda.stream(s):
                B.mbert_graph_launch(g, s)
            s.synchronize()
            assert np.array_equal(host(gout), ref_out), f"replay {i}"
            assert np.array_equal(host(gpool), ref_pool)
            m.encode_padded(ids_pad, mask, ws=ws)  # eager work between replays
            t.cuda.synchronize()
    finally:
        B.mbert_graph_destroy(g)


def test_kernel_timer_counts_launches():
    from transformer_encoder_amd import binding as B
    b = make_batch(WORKLOADS[2])
    m = model_for(2)
    t = torch()
    ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
    ws = m.workspace(8 * 512, 8)
    out = t.empty((8, 512, 768), dtype=t.float32, device="cuda")
    pooled = t.empty((8, 768), dtype=t.float32, device="cuda")
    timer = B.mbert_timer_create(64)
    try:
        # folded LayerNorms: no separate norm kernel; separate: 21 attention + 22 MLP norms
        for fold, kind, n in ((True, B.K_QKV_ROPE, 22), (True, B.K_ATTN_GLOBAL, 8),
                              (True, B.K_ATTN_LOCAL, 14), (True, B.K_LAYERNORM, 0),
                              (False, B.K_LAYERNORM, 43), (False, B.K_WI_GEGLU, 22)):
            m.set_fold(fold)
            B.mbert_timer_reset(timer)
            B.mbert_encode_padded_timed(m.w, ids_pad, mask, 8, 512, ws, ws.numel(), out, pooled,
                                        kind, timer)
            launches, ms = B.mbert_timer_read(timer)
            assert launches == n and (ms > 0) == (n > 0)
    finally:
        m.set_fold(True)
        B.mbert_timer_destroy(timer)
