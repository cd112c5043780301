"""GPU parity of per-position weights / masks and the mean reduction.

The oracle's weighted reading is pinned in test_oracle_pins.py (a 0/1 mask
equals dropping the rows, linearity in the weights, finite differences of the
weighted sum and mean). Here the HIP path is compared with it on the same
seeded inputs, at the tolerances of test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import TOL, _case, _to_dev, assert_parity, kd, max_norm_err, rel_err  # noqa: F401

pytestmark = pytest.mark.gpu


def run_weighted(kd, H, W, idx, logp, chunk, weight, reduction, grad=1.0):
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    wd = None if weight is None else weight.to(Hd.device)
    loss, loss_tok, lse = kd.kl_forward(Hd, Wd, id_, lp, chunk, weight=wd, reduction=reduction)
    g = torch.tensor([grad], dtype=torch.float32, device=Hd.device)
    dH, dW = kd.kl_backward(Hd, Wd, id_, lp, lse, g, chunk, weight=wd, reduction=reduction)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "loss_tok": loss_tok.double().cpu().numpy(),
            "lse": lse.double().cpu().numpy(), "dH": dH.double().cpu().numpy(),
            "dW": dW.double().cpu().numpy()}


def _weights(N, seed, zeros=True):
    g = torch.Generator().manual_seed(seed)
    w = torch.rand(N, generator=g) * 2.0
    if zeros:
        w[torch.rand(N, generator=g) < 0.3] = 0.0  # a packed-sequence style mask on top
    return w.contiguous()


@pytest.mark.parametrize("reduction", ["sum", "mean"])
@pytest.mark.parametrize("N,d,V,K,dtype,chunk", [
    (130, 64, 129, 5, "f32", 64),         # ragged rows, one-column last vocab tile
    (300, 160, 2000, 100, "bf16", 256),   # K = 100 over a small vocabulary
    (257, 72, 515, 1, "bf16", 100),       # K = 1, chunk not a multiple of the tile
])
def test_weighted_parity(kd, N, d, V, K, dtype, chunk, reduction):
    H, W, idx, logp = _case(N, d, V, K, dtype, seed=N + V + K)
    w = _weights(N, seed=N)
    got = run_weighted(kd, H, W, idx, logp, chunk, w, reduction, grad=0.8)
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=0.8, weight=w.numpy(), reduction=reduction)
    assert_parity(got, ref, dtype, f"{N},{d},{V},{K},{dtype},{chunk},{reduction}")


def test_unweighted_mean_is_sum_over_n(kd):
    H, W, idx, logp = _case(200, 64, 700, 8, "f32", seed=41)
    got = run_weighted(kd, H, W, idx, logp, 64, None, "mean", grad=1.0)
    ref = oracle.fused_kl_reference(H, W, idx, logp, reduction="mean")
    assert_parity(got, ref, "f32", "mean without weights")


def test_mask_matches_dropped_rows_on_gpu(kd):
    # The HIP path with a 0/1 mask against the HIP path on the kept rows only.
    H, W, idx, logp = _case(320, 96, 1500, 16, "f32", seed=42)
    keep = torch.rand(320, generator=torch.Generator().manual_seed(3)) < 0.6
    for red in ("sum", "mean"):
        got = run_weighted(kd, H, W, idx, logp, 128, keep.float(), red, grad=1.1)
        sub = run_weighted(kd, H[keep].contiguous(), W, idx[keep].contiguous(),
                           logp[keep].contiguous(), 128, None, red, grad=1.1)
        assert rel_err(got["loss"], sub["loss"]) < 1e-5
        assert max_norm_err(got["dW"], sub["dW"]) < 1e-5
        assert max_norm_err(got["dH"][keep.numpy()], sub["dH"]) < 1e-5
        assert np.all(got["dH"][~keep.numpy()] == 0.0)


def test_zero_total_weight_mean_is_zero(kd):
    H, W, idx, logp = _case(96, 32, 300, 4, "bf16", seed=43)
    got = run_weighted(kd, H, W, idx, logp, 32, torch.zeros(96), "mean")
    assert got["loss"] == 0.0
    assert np.all(got["dH"] == 0.0) and np.all(got["dW"] == 0.0)
    assert np.all(np.isfinite(got["loss_tok"]))


def test_autograd_weighted_mean(kd):
    H, W, idx, logp = _case(150, 64, 800, 8, "bf16", seed=44)
    w = _weights(150, seed=45)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    Hd.requires_grad_(True)
    Wd.requires_grad_(True)
    loss = kd.fused_kl(Hd, Wd, id_, lp, chunk=64, weight=w.to(Hd.device), reduction="mean")
    (loss * 3.0).backward()
    torch.cuda.synchronize()
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=3.0, weight=w.numpy(), reduction="mean")
    assert rel_err(loss.item(), ref["loss"]) < TOL["bf16"]["loss"]
    assert max_norm_err(Hd.grad.double().cpu().numpy(), ref["dH"]) < TOL["bf16"]["grad"]
    assert max_norm_err(Wd.grad.double().cpu().numpy(), ref["dW"]) < TOL["bf16"]["grad"]


def test_bad_weight_and_reduction_rejected(kd):
    H, W, idx, logp = _case(16, 16, 50, 2, "f32", seed=46)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    with pytest.raises(ValueError):
        kd.kl_forward(Hd, Wd, id_, lp, 8, reduction="max")
    with pytest.raises(ValueError):
        kd.kl_forward(Hd, Wd, id_, lp, 8, weight=torch.ones(15, device=Hd.device))


def test_check_inputs_flags_each_violation(kd):
    from test_gpu_parity import _case
    H, W, idx, logp = _case(64, 32, 500, 12, "f32", seed=47)
    dev = torch.device("cuda:0")
    assert kd.check_inputs(idx.to(dev), logp.to(dev), 500) == []
    bad = idx.clone(); bad[3, 5] = 500
    assert kd.check_inputs(bad.to(dev), logp.to(dev), 500) == ["id out of range"]
    bad = idx.clone(); bad[10, 7] = bad[10, 2]
    assert kd.check_inputs(bad.to(dev), logp.to(dev), 500) == ["duplicate id"]
    badl = logp.clone(); badl[20, 0] = float("nan")
    assert kd.check_inputs(idx.to(dev), badl.to(dev), 500) == ["log-prob > 0 or NaN"]
    badl = logp.clone(); badl[0, 0] = 0.25; badl[1, 1] = float("-inf")  # -inf is allowed
    assert kd.check_inputs(idx.to(dev), badl.to(dev), 500) == ["log-prob > 0 or NaN"]
    badl = logp.clone(); badl[1, 1] = float("-inf")
    assert kd.check_inputs(idx.to(dev), badl.to(dev), 500) == []
    # the largest K the loss takes: one row with every id distinct, one with a repeat
    big = torch.stack([torch.randperm(20000)[:16383], torch.randperm(20000)[:16383]]).to(torch.int32)
    big[1, 16000] = big[1, 3]
    lp = torch.full(big.shape, -10.0)
    assert kd.check_inputs(big[:1].contiguous().to(dev), lp[:1].contiguous().to(dev), 20000) == []
    assert kd.check_inputs(big.contiguous().to(dev), lp.contiguous().to(dev), 20000) == ["duplicate id"]
