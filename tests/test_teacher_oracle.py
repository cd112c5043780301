"""Pins of the teacher top-K oracle (oracle/teacher_oracle.py) to things other
than itself: hand-worked caches with ties (tests/golden/teacher_cases.json),
the defining order property checked pair by pair, invariances, and agreement
with an independent float32 torch implementation (the input generator's)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workload

HERE = os.path.dirname(os.path.abspath(__file__))


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"ln": math.log, "exp": math.exp}))


def _cases():
    with open(os.path.join(HERE, "golden", "teacher_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_teacher_cases(case):
    out = oracle.teacher_topk_reference(np.array(case["Ht"], float), np.array(case["Wt"], float), case["K"])
    assert out["idx"].tolist() == case["expect"]["idx"]
    want = np.array([[_ev(v) for v in row] for row in case["expect"]["logp"]])
    np.testing.assert_allclose(out["logp"], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["lse"], [_ev(v) for v in case["expect"]["lse"]], rtol=0, atol=1e-12)


def _order_property_holds(Z, idx):
    """Every kept id beats every dropped id, and the kept ids are in order:
    larger logit first, equal logits by lower id (checked pair by pair)."""
    N, V = Z.shape
    for r in range(N):
        kept = list(idx[r])
        if len(set(kept)) != len(kept):
            return False
        dropped = [j for j in range(V) if j not in set(kept)]
        beats = lambda a, b: Z[r, a] > Z[r, b] or (Z[r, a] == Z[r, b] and a < b)
        if any(not beats(a, b) for a in kept for b in dropped):
            return False
        if any(not beats(a, b) for a, b in zip(kept, kept[1:])):
            return False
    return True


def test_order_property_on_random_and_tied_rows():
    rng = np.random.default_rng(51)
    Ht = rng.standard_normal((6, 5))
    Wt = rng.standard_normal((40, 5))
    Wt[7] = Wt[3]  # exact ties between ids 3 and 7 in every row
    Wt[20] = Wt[3]
    for K in (1, 5, 17, 40):
        out = oracle.teacher_topk_reference(Ht, Wt, K)
        assert _order_property_holds(out["Z"], out["idx"])


def test_full_vocabulary_is_a_distribution_and_shift_invariant():
    rng = np.random.default_rng(52)
    Ht = rng.standard_normal((4, 6))
    Wt = rng.standard_normal((30, 6))
    full = oracle.teacher_topk_reference(Ht, Wt, 30)
    np.testing.assert_allclose(np.exp(full["logp"]).sum(axis=1), 1.0, rtol=1e-12)
    assert np.all(full["logp"] <= 0)
    # A constant added to every logit of a row (an extra feature with equal
    # weight for all tokens) changes neither the ids nor the log-probs.
    Ht2 = np.concatenate([Ht, np.full((4, 1), 2.5)], axis=1)
    Wt2 = np.concatenate([Wt, np.full((30, 1), -1.7)], axis=1)
    for K in (1, 8):
        a = oracle.teacher_topk_reference(Ht, Wt, K)
        b = oracle.teacher_topk_reference(Ht2, Wt2, K)
        assert np.array_equal(a["idx"], b["idx"])
        np.testing.assert_allclose(a["logp"], b["logp"], atol=1e-12)


def test_agrees_with_generator_float32_path():
    # workload.teacher_topk computes the same cache with torch float32
    # log_softmax + topk: an independent implementation.
    g = torch.Generator().manual_seed(53)
    Ht = torch.randn(64, 32, generator=g)
    Wt = torch.randn(500, 32, generator=g) * 2.0 / math.sqrt(32)
    K = 20
    idx_t, logp_t = workload.teacher_topk(Ht, Wt, K)
    out = oracle.teacher_topk_reference(Ht.double().numpy(), Wt.double().numpy(), K)
    Z = out["Z"]
    for r in range(64):
        srt = np.sort(Z[r])[::-1]
        gap = np.min(np.abs(np.diff(srt[: K + 1])))
        if gap > 1e-4:  # no near-tie that float32 could order differently
            assert idx_t[r].tolist() == out["idx"][r].tolist()
    np.testing.assert_allclose(logp_t.double().numpy(), np.take_along_axis(
        Z, idx_t.long().numpy(), axis=1) - out["lse"][:, None], atol=2e-5)


def test_planted_mistakes_are_caught():
    case = _cases()[2]
    Ht, Wt, K = np.array(case["Ht"], float), np.array(case["Wt"], float), case["K"]
    want_idx = case["expect"]["idx"]
    Z = Ht @ Wt.T
    # ties broken by the higher id instead
    bad = [sorted(range(3), key=lambda j: (-Z[r, j], -j))[:K] for r in range(2)]
    assert bad != want_idx
    # renormalising over the kept K moves the log-probs
    out = oracle.teacher_topk_reference(Ht, Wt, K)
    ren = out["logp"] - np.log(np.exp(out["logp"]).sum(axis=1, keepdims=True))
    want = np.array([[_ev(v) for v in row] for row in case["expect"]["logp"]])
    assert np.abs(ren - want).max() > 1e-2


def test_invalid_k_rejected():
    with pytest.raises(ValueError):
        oracle.teacher_topk_reference(np.ones((1, 2)), np.ones((3, 2)), 4)
    with pytest.raises(ValueError):
        oracle.teacher_topk_reference(np.ones((1, 2)), np.ones((3, 2)), 0)


def test_lse_and_logp_match_scipy():
    import scipy.special as sps

    rng = np.random.default_rng(54)
    Ht = rng.standard_normal((5, 7)) * 3.0
    Wt = rng.standard_normal((60, 7))
    out = oracle.teacher_topk_reference(Ht, Wt, 9)
    Z = Ht @ Wt.T
    np.testing.assert_allclose(out["lse"], sps.logsumexp(Z, axis=1), rtol=1e-13)
    full = sps.log_softmax(Z, axis=1)
    np.testing.assert_allclose(out["logp"], np.take_along_axis(full, out["idx"].astype(np.int64), axis=1),
                               rtol=1e-12, atol=1e-12)
