"""Pins of the oracle's heads and pooling variants (kgptalkie, 'The Masked-LM Head' and 'How
Do We Put a Classifier on Top?'; candding, 'Pooling and normalization') against the values
the pages print, closed forms, invariants and the pure-Python brute force. CPU only."""
import json
import math
from pathlib import Path

import numpy as np

from oracle import brute
from oracle import mbert_oracle as O

G = json.loads((Path(__file__).parent / "golden" / "heads.json").read_text())


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_printed_classifier_probabilities_and_loss():
    """softmax of the printed logits gives the printed probabilities, and the loss for label
    0 is minus the log of its probability. The logits are printed to 4 decimals, which moves
    a probability by at most 0.25 * 1e-4."""
    p = O.class_probabilities(G["logits"])
    assert np.allclose(p, G["probabilities"], atol=0.5e-4 + 0.25e-4)
    assert abs(p.sum() - 1.0) < 1e-12
    loss = O.cross_entropy(G["logits"], G["label"])
    assert abs(loss - G["loss"]) < 0.5e-4 + 0.5e-4
    assert abs(loss + math.log(G["probabilities"][0])) < 2e-4


def test_head_parameter_counts():
    D, V, C = G["hidden"], G["vocab"], G["n_labels"]
    assert D * V == G["decoder_weights"]
    shapes = O.parameter_shapes(O.Config())
    assert int(np.prod(shapes["embeddings.tok_embeddings.weight"])) == G["decoder_weights"]
    assert D * C + C == G["classifier_params"]


def test_prediction_head_matches_brute_force():
    D = 12
    x, Wd = _rand((3, D), 1), _rand((D, D), 2, 0.4)
    w = 1.0 + _rand(D, 3, 0.1)
    got = O.prediction_head(x, Wd, w, 1e-5)
    for r in range(3):
        ref = brute.prediction_head(list(x[r]), [list(row) for row in Wd], list(w), 1e-5)
        assert np.allclose(got[r], ref, rtol=1e-12, atol=1e-12)


def test_prediction_head_normalises_each_row():
    """With a unit norm weight every output row has mean 0 and variance var / (var + eps) of
    its GELU input (kgptalkie, 'What Does LayerNorm Do?')."""
    x, Wd = _rand((5, 768), 4), _rand((768, 768), 5, 0.05)
    eps = 1e-5
    h = O.prediction_head(x, Wd, np.ones(768), eps)
    u = O.gelu_erf(x @ Wd.T)
    var = u.var(axis=1)
    assert np.allclose(h.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose(h.var(axis=1), var / (var + eps), rtol=1e-10)


def test_mlm_logits_tied_decoder():
    """With the embedding rows equal to unit vectors the scores are the head output plus the
    bias, column for column; the highest score goes to the row that points along the head
    output (kgptalkie, 'The Masked-LM Head': a word scores high when its embedding row points
    the same way as the head's output)."""
    D = 16
    x, Wd = _rand((2, D), 6), _rand((D, D), 7, 0.3)
    w = np.ones(D)
    b = _rand(D, 8, 0.01)
    got = O.mlm_logits(x, Wd, w, np.eye(D), b, 1e-5)
    assert np.allclose(got - b, O.prediction_head(x, Wd, w, 1e-5), rtol=1e-12, atol=1e-12)
    h = O.prediction_head(x, Wd, w, 1e-5)
    E = _rand((9, D), 9, 0.1)
    E[4] = 3.0 * h[0] / np.linalg.norm(h[0])
    assert int(np.argmax(O.mlm_logits(x[:1], Wd, w, E, np.zeros(9), 1e-5))) == 4


def test_mlm_and_classifier_logits_match_brute_force():
    D, V, C = 8, 11, 4
    x, Wd, w = _rand((2, D), 10), _rand((D, D), 11, 0.5), 1.0 + _rand(D, 12, 0.1)
    E, bv = _rand((V, D), 13), _rand(V, 14)
    Wc, bc = _rand((C, D), 15), _rand(C, 16)
    L = [list(r) for r in Wd]
    got_m = O.mlm_logits(x, Wd, w, E, bv, 1e-5)
    got_c = O.classifier_logits(x, Wd, w, Wc, bc, 1e-5)
    for r in range(2):
        ref_m = brute.mlm_logits(list(x[r]), L, list(w), [list(e) for e in E], list(bv), 1e-5)
        ref_c = brute.classifier_logits(list(x[r]), L, list(w), [list(c) for c in Wc], list(bc), 1e-5)
        assert np.allclose(got_m[r], ref_m, rtol=1e-12, atol=1e-12)
        assert np.allclose(got_c[r], ref_c, rtol=1e-12, atol=1e-12)


def test_pooling_variants():
    """CLS pooling takes row cu[s] (candding, 'Pooling and normalization': index 0); the mean
    of identical rows is that row; mean then L2 is the pinned sentence-vector pooling; empty
    sequences pool to zero."""
    cu = [0, 3, 3, 8]
    out = _rand((8, 5), 17)
    cls = O.cls_pool(out, cu)
    assert np.array_equal(cls[0], out[0]) and np.array_equal(cls[2], out[3])
    assert not cls[1].any() and not O.mean_pool(out, cu)[1].any()
    same = np.tile(out[:1], (8, 1))
    assert np.allclose(O.mean_pool(same, cu)[[0, 2]], out[0], rtol=1e-14)
    assert np.allclose(O.l2_normalize(O.mean_pool(out, cu)), O.mean_pool_normalize(out, cu), rtol=1e-14)
    assert np.allclose(np.linalg.norm(O.l2_normalize(cls)[[0, 2]], axis=1), 1.0)
