"""The padded forward split into groups of whole sequences on separate streams, eagerly and
through a captured graph replayed several times with eager work in between.

Sequences never interact, but the attention kernel's work split depends on its grid: a grid of
at most 256 workgroups (one per CU) runs each workgroup's key tiles on two wave sets whose
softmax states are merged at the end, which rounds differently. The batch-8 workload in one
stream has 480 attention workgroups (no split); a group of 4 rows or fewer has at most 240, a
row alone 60 (split). So G = 1 is bitwise the single-stream forward of the whole batch, every
G >= 2 is bitwise the rows run one by one, and the two references agree within the
end-to-end tolerance."""
import numpy as np
import pytest

from gpu_util import dev_i32, host, min_cos, torch
from workloads import WORKLOADS, make_batch, workload_weights

pytestmark = pytest.mark.gpu
_model = {}


def _m():
    from transformer_encoder_amd.model import DeviceModel
    if "m" not in _model:
        _model["m"] = DeviceModel(workload_weights(2), "bf16")
    return _model["m"]


def _run_grouped(m, ids_pad, mask, G, streams):
    from transformer_encoder_amd import binding as B
    t = torch()
    Bn, Tp = ids_pad.shape
    nbytes = B.mbert_workspace_bytes_grouped(m.cfg, m.dtype, Bn, Tp, G)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    out = t.empty((Bn, Tp, 768), dtype=t.float32, device="cuda")
    pooled = t.empty((Bn, 768), dtype=t.float32, device="cuda")
    B.mbert_encode_padded_grouped(m.w, ids_pad, mask, Bn, Tp, G, ws, nbytes, out, pooled, streams)
    return out, pooled, ws


def _rows_one_by_one(m, ids_pad, mask):
    outs, pools = [], []
    for r in range(ids_pad.shape[0]):
        o, p, _ = m.encode_padded(ids_pad[r:r + 1].contiguous(), mask[r:r + 1].contiguous())
        outs.append(o.clone())
        pools.append(p.clone())
    return torch().cat(outs), torch().cat(pools)


_refs = {}


def _references():
    """(whole batch in one stream, rows one by one), both single-stream forwards."""
    if not _refs:
        b = make_batch(WORKLOADS[2])
        m = _m()
        ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
        whole_out, whole_pool, _ = m.encode_padded(ids_pad, mask)
        rows_out, rows_pool = _rows_one_by_one(m, ids_pad, mask)
        torch().cuda.synchronize()
        _refs.update(ids_pad=ids_pad, mask=mask, whole=(whole_out, whole_pool),
                     rows=(rows_out, rows_pool), real=b["mask"].astype(bool))
    return _refs


def test_references_agree():
    r = _references()
    (wo, wp), (ro, rp) = r["whole"], r["rows"]
    real = r["real"]
    for what, a, b in (("tokens", host(wo)[real], host(ro)[real]), ("pooled", host(wp), host(rp))):
        err, cos = float(np.max(np.abs(a - b))), min_cos(a, b)
        print(f"{what}: max_abs={err:.3e} min_cos={cos:.6f}", flush=True)
        assert err <= 2e-2 and cos >= 0.999, what
    # pad rows are zeros in both
    assert not np.any(host(wo)[~real]) and not np.any(host(ro)[~real])


@pytest.mark.parametrize("G", [1, 2, 3, 8, 20])
def test_grouped_equals_single_stream(G):
    r = _references()
    m = _m()
    streams = [torch().cuda.Stream() for _ in range(max(G - 1, 0))]
    out, pooled, _ = _run_grouped(m, r["ids_pad"], r["mask"], G, streams)
    torch().cuda.synchronize()
    ref_out, ref_pool = r["whole"] if G == 1 else r["rows"]
    assert torch().equal(out, ref_out) and torch().equal(pooled, ref_pool)


def test_grouped_graph_replays():
    from transformer_encoder_amd import binding as B
    t = torch()
    r = _references()
    m = _m()
    ids_pad, mask = r["ids_pad"], r["mask"]
    _, _, ws1 = m.encode_padded(ids_pad, mask)
    ref_out, ref_pool = r["rows"]  # groups of 2 rows: the split attention, as each row alone
    G, (Bn, Tp) = 4, tuple(ids_pad.shape)
    streams = [t.cuda.Stream() for _ in range(G - 1)]
    nbytes = B.mbert_workspace_bytes_grouped(m.cfg, m.dtype, Bn, Tp, G)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    out = t.zeros((Bn, Tp, 768), dtype=t.float32, device="cuda")
    pooled = t.zeros((Bn, 768), dtype=t.float32, device="cuda")
    main = t.cuda.Stream()
    g = B.mbert_graph_capture_padded_grouped(m.w, ids_pad, mask, Bn, Tp, G, ws, nbytes, out,
                                             pooled, streams, main)
    try:
        for _ in range(3):
            out.zero_()
            B.mbert_graph_launch(g, main)
            main.synchronize()
            assert t.equal(out, ref_out) and t.equal(pooled, ref_pool)
            m.encode_padded(ids_pad, mask, ws=ws1)  # eager work between replays
            t.cuda.synchronize()
    finally:
        B.mbert_graph_destroy(g)
