"""The numpy oracle against the independent pure-Python brute force, on tiny inputs.
CPU only. Tiny dims with a window of 2 exercise the band and the layer schedule; real dims
with a handful of tokens exercise the real q|k|v and GeGLU layouts."""
import numpy as np
import pytest

from oracle import brute
from oracle import mbert_oracle as O
from workloads import Dims, make_weights, random_batch


def _run_both(cfg, w, ids, cu, n_layers):
    out, pooled = O.encode(ids, cu, w, cfg, n_layers=n_layers)
    bo, bp = brute.encode(ids, cu, w, n_layers=n_layers, hidden=cfg.hidden,
                          n_heads=cfg.n_heads, head_dim=cfg.head_dim,
                          intermediate=cfg.intermediate, global_every=cfg.global_every,
                          half_window=cfg.half_window, theta_global=cfg.theta_global,
                          theta_local=cfg.theta_local, eps=cfg.eps)
    return out, pooled, np.array(bo), np.array(bp)


@pytest.mark.parametrize("lengths", [[1], [7], [3, 1, 6, 2], [8, 0, 5]])
def test_tiny_dims_window_two(lengths):
    cfg = O.Config(n_layers=4, hidden=16, n_heads=2, head_dim=8, intermediate=12, vocab=50,
                   half_window=2)
    w = make_weights(Dims(4, 16, 2, 8, 12, 50), "f32", 21)
    b = random_batch(lengths, 21, vocab=50)
    out, pooled, bo, bp = _run_both(cfg, w, b["ids"], b["cu_seqlens"], 4)
    assert np.max(np.abs(out - bo)) < 1e-11
    assert np.max(np.abs(pooled - bp)) < 1e-11


def test_tiny_dims_bf16_weights_other_thetas():
    cfg = O.Config(n_layers=3, hidden=16, n_heads=4, head_dim=4, intermediate=8, vocab=30,
                   half_window=1, theta_global=80000.0, theta_local=500.0)
    w = make_weights(Dims(3, 16, 4, 4, 8, 30), "bf16", 22)
    b = random_batch([6, 4], 22, vocab=30)
    out, pooled, bo, bp = _run_both(cfg, w, b["ids"], b["cu_seqlens"], 3)
    assert np.max(np.abs(out - bo)) < 1e-11


@pytest.mark.slow
def test_real_dims_few_tokens():
    cfg = O.Config(n_layers=2)
    w = make_weights(Dims(n_layers=2), "f32", 23)
    b = random_batch([2, 1], 23)
    out, pooled, bo, bp = _run_both(cfg, w, b["ids"], b["cu_seqlens"], 2)
    assert np.max(np.abs(out - bo)) < 1e-10
    assert np.max(np.abs(pooled - bp)) < 1e-10
