"""Parity of the pooling variants and the two heads (kgptalkie, 'The Masked-LM Head' and 'How
Do We Put a Classifier on Top?'; candding, 'Pooling and normalization') against the oracle on
seeded inputs: max |err| / max |ref| within the per-step tolerance of the run dtype."""
import numpy as np
import pytest

from gpu_util import TOL_STEP, dev, dev_i32, host, meta_for, rel_err, torch
from oracle import mbert_oracle as O
from workloads import WORKLOADS, cu_from_lengths, make_batch, random_matrix, rng, round_to

pytestmark = pytest.mark.gpu
DTYPES = ["f32", "bf16", "f16"]
VOCAB = 50368


def B():
    from transformer_encoder_amd import binding
    return binding


def dt(name):
    return B().DTYPES[name]


def _head_weights(dtype, seed, n_labels=4, vocab=VOCAB):
    Wd = random_matrix((768, 768), seed, dtype=dtype, std=0.05)
    nw = round_to(1.0 + random_matrix((768,), seed + 1, std=0.02), dtype)
    E = random_matrix((vocab, 768), seed + 2, dtype=dtype, std=0.02)
    bv = random_matrix((vocab,), seed + 3, dtype=dtype, std=0.02)
    Wc = random_matrix((n_labels, 768), seed + 4, dtype=dtype, std=0.02)
    bc = random_matrix((n_labels,), seed + 5, dtype=dtype, std=0.02)
    return Wd, nw, E, bv, Wc, bc


POOL_CASES = {"edges": [1, 0, 129, 300, 128, 7], "long": [1000, 3]}


@pytest.mark.parametrize("case", list(POOL_CASES))
@pytest.mark.parametrize("mode", [0, 1, 2, 3], ids=["mean", "cls", "mean_l2", "cls_l2"])
def test_pool_modes(case, mode):
    cu = cu_from_lengths(POOL_CASES[case])
    T, S = int(cu[-1]), len(cu) - 1
    out = random_matrix((T, 768), 131, dtype="f32") + 0.3
    pooled = torch().zeros((S, 768), dtype=torch().float32, device="cuda")
    parts = torch().empty(B().mbert_pool_partial_floats(T, S), dtype=torch().float32, device="cuda")
    B().mbert_pool(dev(out, "f32"), T, meta_for(cu, T), S, mode, pooled, parts)
    ref = O.cls_pool(out, cu) if mode & 1 else O.mean_pool(out, cu)
    if mode & 2:
        ref = O.l2_normalize(ref)
    assert rel_err(host(pooled), ref) < 1e-5


def test_pool_mean_l2_equals_final_norm_pooling():
    """Mean pooling with L2 of the final-norm output matches the pooled vector the final-norm
    kernel produces itself to float32 rounding (same rows and order; the fused kernel may
    contract the norm's last multiply into the column sum)."""
    cu = cu_from_lengths([300, 5, 0, 700])
    T, S = int(cu[-1]), len(cu) - 1
    resid = dev(random_matrix((T, 768), 132, dtype="f32"), "f32")
    w = dev(round_to(1.0 + random_matrix((768,), 133, std=0.02), "bf16"), "bf16")
    meta = meta_for(cu, T)
    t = torch()
    out = t.empty((T, 768), dtype=t.float32, device="cuda")
    p1, p2 = (t.empty((S, 768), dtype=t.float32, device="cuda") for _ in range(2))
    parts = t.empty(B().mbert_pool_partial_floats(T, S), dtype=t.float32, device="cuda")
    B().mbert_final_ln_pool(resid, T, meta, S, B().MBERT_BF16, w, 1e-5, out, p1, parts)
    B().mbert_pool(out, T, meta, S, B().POOL_MEAN | B().POOL_L2, p2, parts)
    assert rel_err(host(p1), host(p2)) < 1e-6


def _mlm(dtype, x, T, rows, n_rows):
    Wd, nw, E, bv, _, _ = _head_weights(dtype, 140)
    t = torch()
    nbytes = B().mbert_head_workspace_bytes(dt(dtype), n_rows)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    logits = t.empty((n_rows, VOCAB), dtype=t.float32, device="cuda")
    B().mbert_mlm_head(dt(dtype), dev(x, "f32"), T, None if rows is None else dev_i32(rows), n_rows,
                       dev(Wd, dtype), dev(nw, dtype), 1e-5, dev(E, dtype), dev(bv, dtype), VOCAB,
                       ws, nbytes, logits)
    return host(logits), (Wd, nw, E, bv)


@pytest.mark.parametrize("dtype", DTYPES)
def test_mlm_head_selected_rows(dtype):
    """Scores at selected positions, including an index outside the rows (a zero vector)."""
    T = 300
    x = random_matrix((T, 768), 141, dtype="f32")
    rows = np.array([0, 299, 17, 17, 150, -1, 300, 42], dtype=np.int32)
    got, (Wd, nw, E, bv) = _mlm(dtype, x, T, rows, len(rows))
    xs = np.where(((rows >= 0) & (rows < T))[:, None], x[np.clip(rows, 0, T - 1)], 0.0)
    ref = O.mlm_logits(xs, Wd, nw, E, bv, 1e-5)
    assert rel_err(got, ref) < TOL_STEP[dtype]
    assert np.array_equal(np.argmax(got[:5], axis=1), np.argmax(ref[:5], axis=1)) or dtype != "f32"


@pytest.mark.parametrize("dtype", ["bf16"])
def test_mlm_head_all_rows(dtype):
    """Every position (no row list), at a size that spans several row tiles and a ragged tail."""
    T = 600
    x = random_matrix((T, 768), 142, dtype="f32")
    got, (Wd, nw, E, bv) = _mlm(dtype, x, T, None, T)
    sample = rng(143, 1).choice(T, 40, replace=False)
    ref = O.mlm_logits(x[sample], Wd, nw, E, bv, 1e-5)
    assert rel_err(got[sample], ref) < TOL_STEP[dtype]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n_labels", [4, 1, 37])
def test_classifier_head(dtype, n_labels):
    S = 9
    pooled = random_matrix((S, 768), 151, dtype="f32")
    Wd, nw, _, _, Wc, bc = _head_weights(dtype, 150, n_labels=n_labels, vocab=64)
    t = torch()
    nbytes = B().mbert_head_workspace_bytes(dt(dtype), S)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    logits = t.empty((S, n_labels), dtype=t.float32, device="cuda")
    B().mbert_classifier_head(dt(dtype), dev(pooled, "f32"), S, dev(Wd, dtype), dev(nw, dtype), 1e-5,
                              dev(Wc, dtype), dev(bc, dtype), n_labels, ws, nbytes, logits)
    ref = O.classifier_logits(pooled, Wd, nw, Wc, bc, 1e-5)
    assert rel_err(host(logits), ref) < TOL_STEP[dtype]


def test_classifier_on_encoder_output():
    """The whole classification path of the page: encode, mean pooling without L2, head and
    a 4-label Linear, against the oracle's path on the same packed batch (3 layers)."""
    from transformer_encoder_amd.model import DeviceModel
    from workloads import Dims, make_weights
    t = torch()
    cu = cu_from_lengths([40, 200, 9])
    T, S = int(cu[-1]), 3
    ids = rng(160, 1).integers(0, 50368, T)
    w = make_weights(Dims(n_layers=3), "bf16", 161)
    m = DeviceModel(w, "bf16")
    out, _, _ = m.encode(dev_i32(ids), dev_i32(cu))
    pooled = t.zeros((S, 768), dtype=t.float32, device="cuda")
    parts = t.empty(B().mbert_pool_partial_floats(T, S), dtype=t.float32, device="cuda")
    B().mbert_pool(out, T, meta_for(cu, T), S, B().POOL_MEAN, pooled, parts)
    Wd, nw, _, _, Wc, bc = _head_weights("bf16", 162, vocab=64)
    nbytes = B().mbert_head_workspace_bytes(B().MBERT_BF16, S)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    logits = t.empty((S, 4), dtype=t.float32, device="cuda")
    B().mbert_classifier_head(B().MBERT_BF16, pooled, S, dev(Wd, "bf16"), dev(nw, "bf16"), 1e-5,
                              dev(Wc, "bf16"), dev(bc, "bf16"), 4, ws, nbytes, logits)
    ref_out, _ = O.encode(ids, cu, w, O.Config(n_layers=3))
    ref = O.classifier_logits(O.mean_pool(ref_out, cu), Wd, nw, Wc, bc, 1e-5)
    assert rel_err(host(logits), ref) < 2e-2
