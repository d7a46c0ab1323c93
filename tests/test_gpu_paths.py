"""Every path the library ships against the oracle directly, not through another GPU run:

* the padded batch-8 forward as `bench.py` times it: the batch split into three groups of
  whole sequences on three streams, captured into one HIP graph and replayed;
* the per-layer entry point `mbert_layer` (separate LayerNorms), one layer at a time on the
  same float32 residual as the oracle's `encoder_layer`, for the global layer 0 (no
  attention norm; the caller leaves the embedding-norm output in h) and the local layers 1
  and 2, and the three layers chained.

Tolerances: float32 max |err| / max |ref| <= 1e-4 (one layer, or the chain); 16-bit per layer
max |err| / max |ref| <= 1e-2, the per-step bar (16-bit GEMM inputs: one rounding of the
dtype, 2^-9 for bf16, with accumulation-order headroom); the full forward 2e-2 max-abs after
the final LayerNorm and cosine >= 0.999 per token and per pooled vector."""
import numpy as np
import pytest

from gpu_util import dev_i32, host, min_cos, rel_err, torch
from oracle import mbert_oracle as O
from workloads import WORKLOADS, Dims, make_batch, make_weights, random_batch, workload_weights

pytestmark = pytest.mark.gpu


def check_16bit(got, ref, what):
    err = float(np.max(np.abs(got - ref)))
    cos = min_cos(got, ref)
    print(f"{what}: max_abs={err:.3e} min_cos={cos:.6f}", flush=True)
    assert err <= 2e-2 and cos >= 0.999, what


def test_benched_grouped_graph_against_oracle():
    """The timed call of the padded workload (three groups, one captured graph, replayed
    twice with eager work between) against the oracle's forward of the same batch."""
    from transformer_encoder_amd import binding as B
    from transformer_encoder_amd.model import DeviceModel
    t = torch()
    wl = WORKLOADS[2]
    b = make_batch(wl)
    w = workload_weights(2)
    m = DeviceModel(w, "bf16")
    ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
    Bn, Tp = b["mask"].shape
    G = 3
    streams = [t.cuda.Stream() for _ in range(G - 1)]
    main = t.cuda.Stream()
    nbytes = B.mbert_workspace_bytes_grouped(m.cfg, m.dtype, Bn, Tp, G)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    out = t.full((Bn, Tp, 768), float("nan"), dtype=t.float32, device="cuda")
    pooled = t.full((Bn, 768), float("nan"), dtype=t.float32, device="cuda")
    t.cuda.synchronize()
    g = B.mbert_graph_capture_padded_grouped(m.w, ids_pad, mask, Bn, Tp, G, ws, nbytes, out,
                                             pooled, streams, main)
    ref, rpool = O.encode(b["ids"], b["cu_seqlens"], w, O.Config())
    u = O.unpad(b["ids_pad"], b["mask"])
    try:
        for rep in range(2):
            B.mbert_graph_launch(g, main)
            main.synchronize()
            got = host(out).reshape(-1, 768)
            check_16bit(got[u["indices"]], ref, f"grouped graph replay {rep} tokens")
            check_16bit(host(pooled), rpool, f"grouped graph replay {rep} pooled")
            pads = np.ones(got.shape[0], bool)
            pads[u["indices"]] = False
            assert np.all(got[pads] == 0.0)
            m.encode_padded(ids_pad, mask)  # eager work between the replays
            t.cuda.synchronize()
            out.fill_(float("nan"))
            pooled.fill_(float("nan"))
    finally:
        B.mbert_graph_destroy(g)


_LENGTHS = [300, 65, 1, 129, 200]


def _layer_case(dtype):
    w = make_weights(Dims(n_layers=3), dtype, 611)
    batch = random_batch(_LENGTHS, 611)
    cu = batch["cu_seqlens"]
    return w, batch, cu


def _run_layer_gpu(m, x, layer, cu):
    """mbert_layer on residual x (float32 [T, 768]); for layer 0 h holds x in the dtype (the
    embedding-norm output is the layer's input as is). Returns the new residual."""
    from transformer_encoder_amd import binding as B
    from transformer_encoder_amd.model import to_device
    t = torch()
    T, S = x.shape[0], len(cu) - 1
    ws = m.workspace(T, S)
    L = m.layout(T, S)
    base = ws.data_ptr()
    wsv = ws.view(t.uint8)
    B.mbert_pack_meta(dev_i32(cu), S, T, 8192, base + L.meta)
    xr = t.from_numpy(np.ascontiguousarray(x.astype(np.float32))).cuda()
    wsv[L.resid:L.resid + 4 * T * 768].copy_(xr.view(t.uint8).reshape(-1))
    if layer == 0:
        hx = to_device(x, m.dtype_name, "cuda")
        ds = hx.element_size()
        wsv[L.h:L.h + ds * T * 768].copy_(hx.contiguous().view(t.uint8).reshape(-1))
    t.cuda.synchronize()
    B.mbert_layer(m.w, layer, T, S, base, ws.numel())
    t.cuda.synchronize()
    return wsv[L.resid:L.resid + 4 * T * 768].view(t.float32).reshape(T, 768).double().cpu().numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_mbert_layer_each_layer_against_oracle(dtype):
    from transformer_encoder_amd.model import DeviceModel
    w, batch, cu = _layer_case(dtype)
    cfg = O.Config(n_layers=3)
    m = DeviceModel(w, dtype)
    pos = O.positions(cu)
    segs = O.segments_of(cu)
    x = O.embed(batch["ids"], w, cfg).astype(np.float32).astype(np.float64)
    tol = 1e-4 if dtype == "f32" else 1e-2
    for layer in range(3):
        ref = O.encoder_layer(x, w["layers"][layer], layer, segs, pos, cfg)
        got = _run_layer_gpu(m, x, layer, cu)
        e = rel_err(got, ref)
        # the layer's own update (the residual's increment) at the same bar
        e_upd = rel_err(got - x, ref - x)
        print(f"{dtype} layer {layer}: rel_err={e:.3e} update rel_err={e_upd:.3e}", flush=True)
        assert e <= tol and e_upd <= (tol if dtype == "f32" else 2e-2), layer
        x = ref.astype(np.float32).astype(np.float64)  # next layer starts from the oracle's


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mbert_layer_chain_against_oracle(dtype):
    """Three mbert_layer calls in a row on one workspace (layer 0's h from mbert_embed_ln),
    then the final norm, against the oracle's 3-layer forward."""
    from transformer_encoder_amd import binding as B
    from transformer_encoder_amd.model import DeviceModel
    t = torch()
    w, batch, cu = _layer_case(dtype)
    m = DeviceModel(w, dtype)
    T, S = len(batch["ids"]), len(cu) - 1
    ws = m.workspace(T, S)
    L = m.layout(T, S)
    base = ws.data_ptr()
    meta = base + L.meta
    ids, cud = dev_i32(batch["ids"]), dev_i32(cu)
    B.mbert_pack_meta(cud, S, T, 8192, meta)
    B.mbert_embed_ln(m.dtype, ids, T, meta, m.tok_emb, m.cfg.vocab, m.emb_norm, 1e-5,
                     base + L.resid, base + L.h)
    for layer in range(3):
        B.mbert_layer(m.w, layer, T, S, base, ws.numel())
    out = t.empty((T, 768), dtype=t.float32, device="cuda")
    pooled = t.empty((S, 768), dtype=t.float32, device="cuda")
    B.mbert_final_ln_pool(base + L.resid, T, meta, S, m.dtype, m.final_norm, 1e-5, out, pooled,
                          base + L.partials)
    ref, rpool = O.encode(batch["ids"], cu, w, O.Config(n_layers=3))
    if dtype == "f32":
        e, ep = rel_err(host(out), ref), rel_err(host(pooled), rpool)
        print(f"f32 chain: rel_err out={e:.3e} pooled={ep:.3e}", flush=True)
        assert e <= 1e-4 and ep <= 1e-4
    else:
        check_16bit(host(out), ref, f"{dtype} chain tokens")
        check_16bit(host(pooled), rpool, f"{dtype} chain pooled")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_mfma_probe_runs_and_is_deterministic(dtype):
    """The MFMA calibration kernel: every workgroup computes the same accumulator sums from the
    same register operands, so thread t of every block writes the same finite value."""
    from transformer_encoder_amd import binding as B
    t = torch()
    blocks = 300
    out = t.full((blocks * 256,), float("nan"), dtype=t.float32, device="cuda")
    B.mbert_mfma_probe(B.DTYPES[dtype], blocks, 50, out)
    t.cuda.synchronize()
    o = host(out).reshape(blocks, 256)
    assert np.all(np.isfinite(o))
    assert np.all(o == o[0:1])


def test_padded_batch_far_above_its_tokens_equals_packed():
    """A padded batch of 16 rows of 2048 slots holding 700-2048 tokens each: the GEMMs get
    the slot count (32,768) as their row bound and the real count (about 22k) on the device,
    so the persistent 256x256 tiles walk the slots of the device count, not of the bound. The
    padded forward's real rows and pooled vectors are bitwise those of the packed forward on
    the unpadded batch (whose GEMMs take the exact host count), its pad rows exactly zero;
    one short sequence of the batch is also checked against the oracle."""
    from transformer_encoder_amd.model import DeviceModel
    from workloads import pad_batch
    g = np.random.default_rng([77, 1])
    lengths = g.integers(700, 2049, size=16)
    b = random_batch(lengths, 77)
    dims = Dims(n_layers=2)
    w = make_weights(dims, "bf16", 77)
    m = DeviceModel(w, "bf16")
    ids_pad, mask = pad_batch(b["ids"], b["cu_seqlens"], 2048)
    out_pad, pooled_pad, _ = m.encode_padded(dev_i32(ids_pad), dev_i32(mask))
    out, pooled, _ = m.encode(dev_i32(b["ids"]), dev_i32(b["cu_seqlens"]))
    got_pad = host(out_pad).reshape(-1, 768)
    u = O.unpad(ids_pad, mask)
    print(f"T={int(b['cu_seqlens'][-1])} slots={mask.size}", flush=True)
    assert np.array_equal(got_pad[u["indices"]], host(out))
    assert np.array_equal(host(pooled_pad), host(pooled))
    pads = np.ones(got_pad.shape[0], bool)
    pads[u["indices"]] = False
    assert np.all(got_pad[pads] == 0.0)
    # the shortest sequence against the oracle (its rows do not depend on the others)
    s = int(np.argmin(lengths))
    cu = b["cu_seqlens"]
    one = {"ids": b["ids"][cu[s]:cu[s + 1]], "cu_seqlens": np.array([0, lengths[s]])}
    ref, rpool = O.encode(one["ids"], one["cu_seqlens"], w, O.Config(n_layers=2))
    check_16bit(host(out)[cu[s]:cu[s + 1]], ref, "shortest sequence tokens")
    check_16bit(host(pooled)[s:s + 1], rpool, "shortest sequence pooled")
