"""GPU parity on seeded random shapes, both schedules.

Each case draws its shape from its own seed: N in [1, 700], d in [8, 320]
(a multiple of 8 for bf16, of 4 for float32, so rows stay 16-byte aligned),
V in [2, 5000], K in [1, min(V, 128)], a chunk in [1, 600], the dtype, the
upstream gradient, and (half the time) per-position weights with the sum or
the mean. Inputs follow the workloads' recipe (test_gpu_parity._case). Both
the two-pass calls and the one-pass call are compared with the fp64 oracle
at the tolerances of test_gpu_parity.py, and with each other bit for bit.
A second set draws bf16 shapes with d in [264, 1048], not a multiple of 256,
so the dH and dW launches hold full d tiles and a ragged last one read
through the transposing bf16 loads at a nonzero column base.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import _case, _to_dev, assert_parity, kd  # noqa: F401

pytestmark = pytest.mark.gpu


def _shape(i):
    r = np.random.default_rng(9000 + i)
    dtype = "bf16" if r.random() < 0.6 else "f32"
    step = 8 if dtype == "bf16" else 4
    N = int(r.integers(1, 701))
    d = int(r.integers(1, 320 // step + 1)) * step
    V = int(r.integers(2, 5001))
    K = int(r.integers(1, min(V, 128) + 1))
    chunk = int(r.integers(1, 601))
    grad = float(r.uniform(0.2, 2.0))
    weighted = bool(r.random() < 0.5)
    reduction = "mean" if (weighted and r.random() < 0.5) else "sum"
    return N, d, V, K, dtype, chunk, grad, weighted, reduction


def _wide_shape(i):
    r = np.random.default_rng(9500 + i)
    N = int(r.integers(1, 601))
    d = int(r.integers(33, 132)) * 8
    if d % 256 == 0:
        d += 8
    V = int(r.integers(2, 3001))
    K = int(r.integers(1, min(V, 128) + 1))
    chunk = int(r.integers(1, 601))
    grad = float(r.uniform(0.2, 2.0))
    weighted = bool(r.random() < 0.5)
    reduction = "mean" if (weighted and r.random() < 0.5) else "sum"
    return N, d, V, K, "bf16", chunk, grad, weighted, reduction


@pytest.mark.parametrize("i", range(24))
def test_random_shape(kd, i):
    _check(kd, i, _shape(i))


@pytest.mark.parametrize("i", range(8))
def test_random_wide_bf16_shape(kd, i):
    _check(kd, 100 + i, _wide_shape(i))


def _check(kd, i, shape):
    N, d, V, K, dtype, chunk, grad, weighted, red = shape
    what = f"case {i}: N={N} d={d} V={V} K={K} {dtype} chunk={chunk} {red} w={weighted}"
    print(what, flush=True)
    H, W, idx, logp = _case(N, d, V, K, dtype, seed=i)
    w = torch.rand(N, generator=torch.Generator().manual_seed(i)) * 2.0 if weighted else None
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    wd = None if w is None else w.to(Hd.device)
    g = torch.tensor([grad], dtype=torch.float32, device=Hd.device)
    l2, t2, s2 = kd.kl_forward(Hd, Wd, id_, lp, chunk, weight=wd, reduction=red)
    dH2, dW2 = kd.kl_backward(Hd, Wd, id_, lp, s2, g, chunk, weight=wd, reduction=red)
    l1, t1, s1, dH1, dW1 = kd.kl_forward_backward(Hd, Wd, id_, lp, chunk, grad=g, weight=wd,
                                                  reduction=red)
    torch.cuda.synchronize()
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=grad,
                                    weight=None if w is None else w.numpy(), reduction=red)
    got = {"loss": float(l2.item()), "loss_tok": t2.double().cpu().numpy(),
           "lse": s2.double().cpu().numpy(), "dH": dH2.double().cpu().numpy(),
           "dW": dW2.double().cpu().numpy()}
    assert_parity(got, ref, dtype, what)
    for name, a, b in (("loss", l1, l2), ("loss_tok", t1, t2), ("lse", s1, s2), ("dH", dH1, dH2),
                       ("dW", dW1, dW2)):
        assert torch.equal(a, b), (what, name)
