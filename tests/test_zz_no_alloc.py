"""mbert_encode_noalloc (the forward whose workspace is the library's own fixed device array)
against mbert_encode with a caller workspace: two calls in a row, the second on a smaller
batch, each compared with the existing entry point's outputs on the same inputs (the same
kernels on the same sizes: bitwise equal, and within the 16-bit end-to-end bar of the
oracle's forward), and the size limit rejected before any work is enqueued."""
import numpy as np
import pytest

from gpu_util import dev_i32, host, min_cos, torch
from oracle import mbert_oracle as O
from workloads import Dims, make_weights, random_batch

pytestmark = pytest.mark.gpu


def B():
    from transformer_encoder_amd import binding
    return binding


def test_noalloc_matches_encode_two_calls():
    from transformer_encoder_amd.model import DeviceModel
    t = torch()
    w = make_weights(Dims(n_layers=3), "bf16", 931)
    m = DeviceModel(w, "bf16")
    for lengths in ([1000, 65, 300, 1, 2000], [129, 64, 7]):  # the second call is smaller
        batch = random_batch(lengths, 931 + len(lengths))
        ids, cu = dev_i32(batch["ids"]), dev_i32(batch["cu_seqlens"])
        T, S = len(batch["ids"]), len(lengths)
        out = t.full((T, 768), float("nan"), dtype=t.float32, device="cuda")
        pooled = t.full((S, 768), float("nan"), dtype=t.float32, device="cuda")
        B().mbert_encode_noalloc(m.w, ids, cu, S, T, out, pooled)
        ref_out, ref_pool, _ = m.encode(ids, cu)
        t.cuda.synchronize()
        assert t.equal(out, ref_out) and t.equal(pooled, ref_pool), lengths
        o_ref, p_ref = O.encode(batch["ids"], batch["cu_seqlens"], w, O.Config(n_layers=3))
        got = host(out)
        err = float(np.max(np.abs(got - o_ref)))
        print(f"noalloc T={T}: max_abs={err:.3e}", flush=True)
        assert err <= 2e-2 and min_cos(got, o_ref) >= 0.999
        assert float(np.max(np.abs(host(pooled) - p_ref))) <= 2e-2


def test_noalloc_rejects_oversize_before_launch():
    from transformer_encoder_amd.model import DeviceModel
    t = torch()
    w = make_weights(Dims(n_layers=1), "bf16", 932)
    m = DeviceModel(w, "bf16")
    cap = B().mbert_noalloc_max_bytes()
    assert cap == 64 << 20
    T = 8192
    assert B().mbert_workspace_bytes(m.cfg, m.dtype, T, 1) > cap
    ids = t.zeros(T, dtype=t.int32, device="cuda")
    cu = dev_i32([0, T])
    out = t.full((T, 768), 7.0, dtype=t.float32, device="cuda")
    rc = B().mbert_encode_noalloc(m.w, ids, cu, 1, T, out, None, check=False)
    t.cuda.synchronize()
    assert rc == B().MBERT_ENOSPC
    assert bool((out == 7.0).all())  # nothing ran
