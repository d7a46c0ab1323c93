"""The padded forward split into groups of whole sequences on separate streams: every output
is bitwise the single-stream forward's (sequences never interact), eagerly and through a
captured graph replayed several times with eager work in between."""
import numpy as np
import pytest

from gpu_util import dev_i32, host, torch
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


@pytest.mark.parametrize("G", [1, 2, 3, 8, 20])
def test_grouped_equals_single_stream(G):
    b = make_batch(WORKLOADS[2])
    m = _m()
    ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
    ref_out, ref_pool, _ = m.encode_padded(ids_pad, mask)
    streams = [torch().cuda.Stream() for _ in range(max(G - 1, 0))]
    out, pooled, _ = _run_grouped(m, ids_pad, mask, G, streams)
    torch().cuda.synchronize()
    assert torch().equal(out, ref_out) and torch().equal(pooled, ref_pool)


def test_grouped_graph_replays():
    from transformer_encoder_amd import binding as B
    t = torch()
    b = make_batch(WORKLOADS[2])
    m = _m()
    ids_pad, mask = dev_i32(b["ids_pad"]), dev_i32(b["mask"])
    ref_out, ref_pool, ws1 = m.encode_padded(ids_pad, mask)
    G, (Bn, Tp) = 4, b["mask"].shape
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
