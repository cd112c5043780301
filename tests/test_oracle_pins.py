"""Pins of the CPU oracle to things other than itself.

Each test fixes the oracle against mathematics the pages imply: hand-worked
closed forms (tests/golden/hand_cases.json), textbook special cases computed
by library routines (scipy's rel_entr, logsumexp, torch's cross_entropy),
exact identities, an inequality, and fp64 central finite differences of the
oracle's own loss. The last group plants mistakes in a copy of the oracle and
checks that the pins catch them.

Pages: "Hugging Face：让知识蒸馏廉价到可大规模运行", section 为什么蒸馏恢复代价高昂
(the three variants are equivalent; Dense KL is the correctness baseline);
"Chunkovaná KL strata ...", section "Čo dopĺňajú podrobnejšie experimenty" (no
renormalisation); "Chunkovaná KL strata ...", section "Kde zostáva dôvod na
opatrnosť" (Cut Cross-Entropy as prior art: the K = 1 case is cross-entropy).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
from oracle import kl_oracle as ko

HERE = os.path.dirname(os.path.abspath(__file__))


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    return float(eval(x, {"__builtins__": {}}, {"ln": math.log, "exp": math.exp, "e": math.e}))


def _arr(a):
    return np.array([[_ev(v) for v in row] for row in a], dtype=np.float64)


def _rand_case(rng, N, d, V, K, wscale=1.0):
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d)) * wscale / math.sqrt(d)
    T = rng.standard_normal((N, V)) * 2.0
    logpt = T - sps.logsumexp(T, axis=1, keepdims=True)
    idx = np.argsort(-logpt, axis=1, kind="stable")[:, :K]
    logp = np.take_along_axis(logpt, idx, axis=1)
    return H, W, idx.astype(np.int32), logp


# --------------------------------------------------------------------------
# hand-worked closed forms
# --------------------------------------------------------------------------
def test_golden_hand_cases():
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        spec = json.load(f)
    assert len(spec["cases"]) >= 4
    for case in spec["cases"]:
        H = _arr(case["H"])
        W = _arr(case["W"])
        idx = np.array(case["idx"], dtype=np.int64)
        logp = _arr(case["logp"])
        g = case.get("grad", 1.0)
        out = oracle.fused_kl_reference(H, W, idx, logp, grad=g)
        ex = case["expect"]
        np.testing.assert_allclose(out["lse"], [_ev(v) for v in ex["lse"]], rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(out["loss_tok"], [_ev(v) for v in ex["loss_tok"]], rtol=0, atol=1e-14,
                                   err_msg=case["name"])
        np.testing.assert_allclose(out["loss"], sum(_ev(v) for v in ex["loss_tok"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(out["dH"], _arr(ex["dH"]), rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(out["dW"], _arr(ex["dW"]), rtol=0, atol=1e-14, err_msg=case["name"])


# --------------------------------------------------------------------------
# special cases that reduce to textbook quantities
# --------------------------------------------------------------------------
def test_full_vocab_teacher_is_textbook_kl():
    """K = V and a full teacher softmax: the loss is KL(p || q) exactly."""
    rng = np.random.default_rng(11)
    N, d, V = 6, 5, 13
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    T = rng.standard_normal((N, V)) * 1.5
    p = sps.softmax(T, axis=1)
    idx = np.tile(np.arange(V), (N, 1))
    out = oracle.fused_kl_reference(H, W, idx, np.log(p))
    q = sps.softmax(H @ W.T, axis=1)
    ref = sps.rel_entr(p, q).sum(axis=1)
    np.testing.assert_allclose(out["loss_tok"], ref, rtol=1e-12, atol=1e-13)
    assert np.all(out["loss_tok"] >= -1e-15)  # Gibbs' inequality when the teacher mass is 1


def test_k1_probability_one_is_cross_entropy():
    """K = 1, p = 1: the loss is cross-entropy against the cached token."""
    rng = np.random.default_rng(12)
    N, d, V = 9, 4, 17
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    tgt = rng.integers(0, V, size=N)
    out = oracle.fused_kl_reference(H, W, tgt[:, None], np.zeros((N, 1)))
    Z = H @ W.T
    ce = sps.logsumexp(Z, axis=1) - Z[np.arange(N), tgt]
    np.testing.assert_allclose(out["loss_tok"], ce, rtol=1e-13, atol=1e-13)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Ht @ Wt.T, torch.tensor(tgt), reduction="sum")
    loss.backward()
    np.testing.assert_allclose(out["loss"], loss.item(), rtol=1e-13)
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_teacher_equal_to_student_on_topk_gives_zero():
    """p_k = q_{idx_k}: every row's loss is exactly zero (unnormalised p)."""
    rng = np.random.default_rng(13)
    N, d, V, K = 7, 6, 40, 5
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    logq = sps.log_softmax(H @ W.T, axis=1)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    out = oracle.fused_kl_reference(H, W, idx, np.take_along_axis(logq, idx, axis=1))
    np.testing.assert_allclose(out["loss_tok"], 0.0, atol=1e-14)


def test_half_of_student_gives_negative_loss():
    """p = q/2 on the top-K: L_r = P_r ln(1/2) < 0 (the loss is not >= 0 when Σp < 1)."""
    rng = np.random.default_rng(14)
    N, d, V, K = 5, 4, 30, 6
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    logq = sps.log_softmax(H @ W.T, axis=1)
    idx = np.stack([rng.choice(V, K, replace=False) for _ in range(N)])
    logp = np.take_along_axis(logq, idx, axis=1) + math.log(0.5)
    out = oracle.fused_kl_reference(H, W, idx, logp)
    Pm = np.exp(logp).sum(axis=1)
    np.testing.assert_allclose(out["loss_tok"], Pm * math.log(0.5), rtol=1e-12, atol=1e-15)


def test_uniform_student_closed_form():
    """W = 0: lse = ln V, L_r = Σ_k p_k logp_k + P_r ln V, G = P_r/V − p."""
    rng = np.random.default_rng(15)
    H, W, idx, logp = _rand_case(rng, 8, 6, 50, 7)
    W = np.zeros_like(W)
    g = 0.75
    out = oracle.fused_kl_reference(H, W, idx, logp, grad=g)
    p = np.exp(logp)
    Pm = p.sum(axis=1)
    V = W.shape[0]
    np.testing.assert_allclose(out["lse"], math.log(V), rtol=1e-15)
    np.testing.assert_allclose(out["loss_tok"], (p * logp).sum(axis=1) + Pm * math.log(V), rtol=1e-13)
    Gref = np.repeat((Pm / V)[:, None], V, axis=1)
    for r in range(H.shape[0]):
        Gref[r, idx[r]] -= p[r]
    np.testing.assert_allclose(out["dlogits"], g * Gref, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(out["dH"], 0.0, atol=1e-15)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(16)
    H, W, idx, logp = _rand_case(rng, 10, 8, 300, 9, wscale=4.0)
    out = oracle.fused_kl_reference(H, W, idx, logp)
    np.testing.assert_allclose(out["lse"], sps.logsumexp(H @ W.T, axis=1), rtol=1e-14)


def test_sparse_form_matches_dense():
    """The pages' equivalence claim: the sparse per-row form gives the dense result."""
    rng = np.random.default_rng(17)
    H, W, idx, logp = _rand_case(rng, 12, 10, 200, 11)
    out = oracle.fused_kl_reference(H, W, idx, logp)
    Z = H @ W.T
    lse = sps.logsumexp(Z, axis=1)
    p = np.exp(logp)
    sparse = (p * (logp - np.take_along_axis(Z, idx, axis=1) + lse[:, None])).sum(axis=1)
    np.testing.assert_allclose(out["loss_tok"], sparse, rtol=1e-12, atol=1e-13)


def test_log_sum_bound():
    """Log-sum inequality: L_r ≥ P_r ln(P_r / Q_r) ≥ P_r ln P_r, Q_r = Σ_k q_{idx_k}."""
    rng = np.random.default_rng(18)
    for trial in range(5):
        H, W, idx, logp = _rand_case(rng, 16, 8, 120, 1 + 3 * trial, wscale=3.0)
        out = oracle.fused_kl_reference(H, W, idx, logp)
        q = sps.softmax(H @ W.T, axis=1)
        P = np.exp(logp).sum(axis=1)
        Q = np.take_along_axis(q, idx, axis=1).sum(axis=1)
        assert np.all(out["loss_tok"] >= P * np.log(P / Q) - 1e-12)
        assert np.all(out["loss_tok"] >= P * np.log(P) - 1e-12)


def test_dlogits_rows_sum_to_zero():
    rng = np.random.default_rng(19)
    H, W, idx, logp = _rand_case(rng, 20, 7, 90, 6)
    out = oracle.fused_kl_reference(H, W, idx, logp, grad=1.3)
    np.testing.assert_allclose(out["dlogits"].sum(axis=1), 0.0, atol=1e-15)


def test_neg_inf_logprob_acts_as_absent():
    rng = np.random.default_rng(20)
    H, W, idx, logp = _rand_case(rng, 6, 5, 60, 4)
    logp_inf = logp.copy()
    logp_inf[:, -1] = -np.inf
    a = oracle.fused_kl_reference(H, W, idx, logp_inf)
    b = oracle.fused_kl_reference(H, W, idx[:, :-1], logp[:, :-1])
    for k in ("loss_tok", "lse", "dH", "dW"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-14, atol=1e-16)


def test_permuting_cache_columns_changes_nothing():
    rng = np.random.default_rng(21)
    H, W, idx, logp = _rand_case(rng, 6, 5, 60, 8)
    perm = rng.permutation(8)
    a = oracle.fused_kl_reference(H, W, idx, logp)
    b = oracle.fused_kl_reference(H, W, idx[:, perm], logp[:, perm])
    for k in ("loss_tok", "dH", "dW"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-14, atol=1e-16)


def test_rows_reference_matches_full():
    rng = np.random.default_rng(22)
    H, W, idx, logp = _rand_case(rng, 15, 6, 70, 5)
    full = oracle.fused_kl_reference(H, W, idx, logp, grad=0.5)
    rows = [0, 3, 14, 7]
    part = oracle.rows_reference(H, W, idx, logp, rows, grad=0.5)
    for k in ("loss_tok", "lse", "dH", "dlogits"):
        np.testing.assert_allclose(part[k], full[k][rows], rtol=1e-14, atol=1e-16)


def test_row_blocks_assemble_dw():
    """dW is the sum over row blocks of dlogitsᵀ H (the full-size GPU check relies on it)."""
    rng = np.random.default_rng(26)
    H, W, idx, logp = _rand_case(rng, 20, 5, 40, 4)
    full = oracle.fused_kl_reference(H, W, idx, logp, grad=0.8)
    dW = np.zeros_like(full["dW"])
    for r0 in range(0, 20, 6):
        rows = list(range(r0, min(20, r0 + 6)))
        part = oracle.rows_reference(H, W, idx, logp, rows, grad=0.8, with_dh=False)
        assert "dH" not in part
        dW += part["dlogits"].T @ H[rows]
    np.testing.assert_allclose(dW, full["dW"], rtol=1e-13, atol=1e-15)


def test_invalid_cache_rejected():
    with pytest.raises(ValueError):
        ko.teacher_grid(np.array([[0, 0]]), np.zeros((1, 2)), 5)
    with pytest.raises(ValueError):
        ko.teacher_grid(np.array([[5]]), np.zeros((1, 1)), 5)
    with pytest.raises(ValueError):
        ko.teacher_grid(np.array([[-1]]), np.zeros((1, 1)), 5)


# --------------------------------------------------------------------------
# gradients against fp64 central finite differences of the oracle's loss
# --------------------------------------------------------------------------
def _fd_errors(fn, H, W, idx, logp, g, entries_H, entries_W, h=1e-6):
    out = fn(H, W, idx, logp, grad=g)
    errs = []
    for (i, j) in entries_H:
        Hp = H.copy(); Hp[i, j] += h
        Hm = H.copy(); Hm[i, j] -= h
        fd = g * (fn(Hp, W, idx, logp)["loss"] - fn(Hm, W, idx, logp)["loss"]) / (2 * h)
        errs.append(abs(fd - out["dH"][i, j]))
    for (i, j) in entries_W:
        Wp = W.copy(); Wp[i, j] += h
        Wm = W.copy(); Wm[i, j] -= h
        fd = g * (fn(H, Wp, idx, logp)["loss"] - fn(H, Wm, idx, logp)["loss"]) / (2 * h)
        errs.append(abs(fd - out["dW"][i, j]))
    scale = max(np.abs(out["dH"]).max(), np.abs(out["dW"]).max())
    return max(errs) / scale


def test_gradients_finite_differences_every_entry_micro():
    rng = np.random.default_rng(23)
    H, W, idx, logp = _rand_case(rng, 4, 3, 7, 2, wscale=2.0)
    eH = [(i, j) for i in range(4) for j in range(3)]
    eW = [(i, j) for i in range(7) for j in range(3)]
    assert _fd_errors(oracle.fused_kl_reference, H, W, idx, logp, 1.7, eH, eW) < 1e-6


def test_gradients_finite_differences_sampled_tiny_config():
    # The tiny fp32 workload's shape (N=128, d=64, V=1000, K=8), 100 seeded entries each.
    rng = np.random.default_rng(24)
    H, W, idx, logp = _rand_case(rng, 128, 64, 1000, 8)
    eH = list(zip(rng.integers(0, 128, 100), rng.integers(0, 64, 100)))
    eW = list(zip(rng.integers(0, 1000, 100), rng.integers(0, 64, 100)))
    assert _fd_errors(oracle.fused_kl_reference, H, W, idx, logp, 1.0, eH, eW) < 1e-6


# --------------------------------------------------------------------------
# planted mistakes: a broken copy of the oracle must fail the pins
# --------------------------------------------------------------------------
def _mutant(kind):
    def fn(H, W, idx, logp, grad=1.0):
        H = ko.to_f64(H); W = ko.to_f64(W)
        P = ko.teacher_grid(idx, logp, W.shape[0])
        if kind == "renormalise":
            P = P / P.sum(axis=1, keepdims=True)
        _, lse, logq = ko.student_log_softmax(H, W)
        L = ko.kl_rows(P, logq)
        q = np.exp(logq)
        if kind == "drop_mass_factor":
            G = grad * (q - P)
        elif kind == "wrong_sign":
            G = grad * (P - q * P.sum(axis=1, keepdims=True))
        else:
            G = grad * (q * P.sum(axis=1, keepdims=True) - P)
        dH = G @ W
        dW = (G.T @ H) if kind != "wrong_row_index" else (G.T @ H)[::-1]
        return {"loss_tok": L, "loss": float(L.sum()), "lse": lse, "dH": dH, "dW": dW}
    return fn


@pytest.mark.parametrize("kind", ["drop_mass_factor", "wrong_sign", "wrong_row_index"])
def test_planted_gradient_mistakes_are_caught(kind):
    rng = np.random.default_rng(25)
    H, W, idx, logp = _rand_case(rng, 4, 3, 7, 2, wscale=2.0)
    eH = [(i, j) for i in range(4) for j in range(3)]
    eW = [(i, j) for i in range(7) for j in range(3)]
    assert _fd_errors(_mutant(kind), H, W, idx, logp, 1.0, eH, eW) > 1e-3


def test_planted_renormalisation_is_caught():
    with open(os.path.join(HERE, "golden", "hand_cases.json")) as f:
        case = json.load(f)["cases"][0]
    out = _mutant("renormalise")(_arr(case["H"]), _arr(case["W"]), np.array(case["idx"]), _arr(case["logp"]))
    assert abs(out["loss_tok"][0] - _ev(case["expect"]["loss_tok"][0])) > 1e-2


# --------------------------------------------------------------------------
# per-token weights and the mean reduction
# --------------------------------------------------------------------------
def test_mask_equals_dropping_rows():
    # A 0/1 mask must give exactly the loss and gradients of the kept rows
    # alone: an independent evaluation on a smaller problem.
    rng = np.random.default_rng(31)
    H, W, idx, logp = _rand_case(rng, 12, 5, 40, 4)
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 1, 0, 1, 1, 0], dtype=bool)
    for red in ("sum", "mean"):
        got = oracle.fused_kl_reference(H, W, idx, logp, grad=0.7, weight=keep.astype(float), reduction=red)
        sub = oracle.fused_kl_reference(H[keep], W, idx[keep], logp[keep], grad=0.7, reduction=red)
        assert math.isclose(got["loss"], sub["loss"], rel_tol=1e-12)
        np.testing.assert_allclose(got["dW"], sub["dW"], rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(got["dH"][keep], sub["dH"], rtol=1e-10, atol=1e-14)
        assert np.all(got["dH"][~keep] == 0.0)
        np.testing.assert_allclose(got["loss_tok"][keep], sub["loss_tok"], rtol=1e-12)


def test_weights_one_hot_and_linearity():
    rng = np.random.default_rng(32)
    H, W, idx, logp = _rand_case(rng, 6, 4, 30, 3)
    base = oracle.fused_kl_reference(H, W, idx, logp)
    for r in range(6):
        e = np.zeros(6); e[r] = 1.0
        assert math.isclose(oracle.fused_kl_reference(H, W, idx, logp, weight=e)["loss"],
                            base["loss_tok"][r], rel_tol=1e-12)
    w1, w2 = rng.random(6), rng.random(6)
    a = oracle.fused_kl_reference(H, W, idx, logp, weight=w1)
    b = oracle.fused_kl_reference(H, W, idx, logp, weight=w2)
    c = oracle.fused_kl_reference(H, W, idx, logp, weight=2.0 * w1 - 3.0 * w2)
    assert math.isclose(c["loss"], 2.0 * a["loss"] - 3.0 * b["loss"], rel_tol=1e-10)
    np.testing.assert_allclose(c["dW"], 2.0 * a["dW"] - 3.0 * b["dW"], rtol=1e-9, atol=1e-13)


def test_mean_reduction_definitions():
    rng = np.random.default_rng(33)
    H, W, idx, logp = _rand_case(rng, 8, 4, 25, 3)
    base = oracle.fused_kl_reference(H, W, idx, logp)
    m = oracle.fused_kl_reference(H, W, idx, logp, reduction="mean")
    assert math.isclose(m["loss"], float(np.mean(base["loss_tok"])), rel_tol=1e-12)
    np.testing.assert_allclose(m["dH"], base["dH"] / 8, rtol=1e-12)
    w = rng.random(8)
    mw = oracle.fused_kl_reference(H, W, idx, logp, weight=w, reduction="mean")
    assert math.isclose(mw["loss"], float(np.dot(w, base["loss_tok"]) / w.sum()), rel_tol=1e-12)
    # Scaling every weight by the same factor leaves the mean unchanged.
    mw5 = oracle.fused_kl_reference(H, W, idx, logp, weight=5.0 * w, reduction="mean")
    assert math.isclose(mw5["loss"], mw["loss"], rel_tol=1e-12)
    np.testing.assert_allclose(mw5["dW"], mw["dW"], rtol=1e-10)
    z = oracle.fused_kl_reference(H, W, idx, logp, weight=np.zeros(8), reduction="mean")
    assert z["loss"] == 0.0 and np.all(z["dW"] == 0.0) and np.all(z["dH"] == 0.0)
    with pytest.raises(ValueError):
        oracle.fused_kl_reference(H, W, idx, logp, reduction="max")


def _weighted(weight, reduction):
    def fn(H, W, idx, logp, grad=1.0):
        return oracle.fused_kl_reference(H, W, idx, logp, grad=grad, weight=weight, reduction=reduction)
    return fn


def test_weighted_mean_gradients_finite_differences():
    rng = np.random.default_rng(34)
    H, W, idx, logp = _rand_case(rng, 4, 3, 7, 2, wscale=2.0)
    w = np.array([0.3, 0.0, 1.4, 0.8])
    eH = [(i, j) for i in range(4) for j in range(3)]
    eW = [(i, j) for i in range(7) for j in range(3)]
    assert _fd_errors(_weighted(w, "mean"), H, W, idx, logp, 1.3, eH, eW) < 1e-6
    assert _fd_errors(_weighted(w, "sum"), H, W, idx, logp, 0.6, eH, eW) < 1e-6


def test_planted_unweighted_gradient_is_caught():
    # A copy that weights the loss but forgets the weights in the gradient.
    rng = np.random.default_rng(35)
    H, W, idx, logp = _rand_case(rng, 4, 3, 7, 2, wscale=2.0)
    w = np.array([0.3, 0.0, 1.4, 0.8])

    def broken(H, W, idx, logp, grad=1.0):
        out = oracle.fused_kl_reference(H, W, idx, logp, grad=grad)
        out["loss"] = float(np.dot(w, out["loss_tok"]))
        return out
    eH = [(i, j) for i in range(4) for j in range(3)]
    eW = [(i, j) for i in range(7) for j in range(3)]
    assert _fd_errors(broken, H, W, idx, logp, 1.0, eH, eW) > 1e-3


# --------------------------------------------------------------------------
# the exact upcast of bf16 inputs
# --------------------------------------------------------------------------
def _bf16_value(bits: int) -> float:
    """The value of a bfloat16 bit pattern, decoded from its fields: 1 sign
    bit, 8 exponent bits (bias 127), 7 fraction bits; exponent 0 is a
    subnormal (or zero) and exponent 255 infinity or NaN."""
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_to_f64_bf16_is_exact():
    """to_f64 of a bfloat16 tensor gives exactly the value each bit pattern
    encodes: zeros of both signs, the smallest and largest subnormals, the
    smallest normal, 1, the largest finite value, infinities, and every
    pattern with a fraction of all ones or a single one."""
    special = [0x0000, 0x8000, 0x0001, 0x807F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
               0x7F80, 0xFF80, 0x4049, 0x3E80]
    special += [(s << 15) | (e << 7) | f for s in (0, 1) for e in range(255)
                for f in (0x7F, 0x01, 0x40)]
    rng = np.random.default_rng(5)
    special += [int(b) for b in rng.integers(0, 1 << 16, 4000) if ((b >> 7) & 0xFF) != 0xFF]
    bits = np.array(special, dtype=np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    got = oracle.to_f64(t)
    want = np.array([_bf16_value(int(b)) for b in bits])
    assert got.dtype == np.float64 and got.shape == want.shape
    assert np.array_equal(got, want)
    # signs of zero survive as well
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # and a 2-D bf16 operand keeps its shape and row order
    m = t[:4000].reshape(40, 100)
    assert np.array_equal(oracle.to_f64(m), want[:4000].reshape(40, 100))
