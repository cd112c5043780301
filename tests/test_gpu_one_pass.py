"""GPU parity of the one-pass call (kd_fused_kl_fwd_bwd): loss and gradients
with each chunk's logits projected once and kept in float32 until its
dlogits are formed.

It is checked against the fp64 oracle on the same seeded inputs, at the
tolerances of test_gpu_parity.py, over the same shapes (ragged rows and vocab
tiles, several dW windows, K = 1 and K = V, -inf entries, weights and the
mean), and at full size on sampled rows and on identities that hold at any
size. A second, separate check: it computes the logits, lse, losses and
dlogits with the same float32 operations as the two-pass calls (the same
GEMM and combine, and the correction at a cached id rounded the same way),
so every output equals theirs bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from test_gpu_parity import (  # noqa: F401
    TOL, _case, _to_dev, assert_parity, kd, max_norm_err, rel_err, run_hip)

pytestmark = pytest.mark.gpu


def run_one(kd, H, W, idx, logp, chunk, grad=1.0, weight=None, reduction="sum", need_dH=True,
            need_dW=True):
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    wd = None if weight is None else weight.to(Hd.device)
    g = torch.tensor([grad], dtype=torch.float32, device=Hd.device)
    loss, tok, lse, dH, dW = kd.kl_forward_backward(Hd, Wd, id_, lp, chunk, grad=g, weight=wd,
                                                    reduction=reduction, need_dH=need_dH,
                                                    need_dW=need_dW)
    torch.cuda.synchronize()
    out = {"loss": float(loss.item()), "loss_tok": tok.double().cpu().numpy(),
           "lse": lse.double().cpu().numpy()}
    if dH is not None:
        out["dH"] = dH.double().cpu().numpy()
    if dW is not None:
        out["dW"] = dW.double().cpu().numpy()
    return out


def test_tiny_fp32_workload(kd):
    cfg = workload.config(1)
    H, W, idx, logp = workload.make_inputs(cfg)
    got = run_one(kd, H, W, idx, logp, cfg.chunk)
    assert_parity(got, oracle.fused_kl_reference(H, W, idx, logp), "f32", "cfg1")


def test_small_bf16_workload(kd):
    cfg = workload.config(2)
    H, W, idx, logp = workload.make_inputs(cfg)
    got = run_one(kd, H, W, idx, logp, cfg.chunk)
    assert_parity(got, oracle.fused_kl_reference(H, W, idx, logp), "bf16", "cfg2")


@pytest.mark.parametrize("N,d,V,K,dtype,chunk", [
    (130, 64, 129, 5, "f32", 64),        # ragged rows and a one-column last vocab tile
    (5, 16, 300, 3, "f32", 4),           # fewer rows than a tile, tiny d
    (200, 200, 1000, 17, "bf16", 96),    # d not a multiple of the 64-element stage
    (257, 72, 515, 1, "bf16", 128),      # K = 1
    (64, 32, 40, 40, "f32", 16),         # K = V: the full teacher distribution
    (300, 160, 2000, 100, "bf16", 256),  # K = 100 over a small vocabulary
    (1100, 96, 3000, 20, "bf16", 128),   # 9 chunks: windows of 4, 4 and 1 chunk
    (1536, 256, 8000, 32, "f32", 512),   # fp32 over 3 chunks of 512 rows
    (90, 64, 10000, 8, "f32", 90),       # a row of 10,000 logits: 2 streaming workgroups, ragged
    (64, 8, 300, 4, "bf16", 32),         # d = 8: the smallest bf16 row (16 bytes), one partial stage
    (300, 64, 20000, 16383, "f32", 128), # the largest K (the hit record's 14-bit field), 82% of V cached
    (260, 320, 1100, 9, "bf16", 128),    # d = 320: one full 256-wide d tile and a 64-wide one
    (300, 2880, 1500, 20, "bf16", 128),  # d = 2880 (the gpt-oss head): 11 full d tiles + 64 columns
])
def test_edge_shapes(kd, N, d, V, K, dtype, chunk):
    H, W, idx, logp = _case(N, d, V, K, dtype, seed=N * 7 + V)
    got = run_one(kd, H, W, idx, logp, chunk, grad=0.37)
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=0.37)
    assert_parity(got, ref, dtype, f"{N},{d},{V},{K},{dtype},{chunk}")


@pytest.mark.parametrize("chunk", [1, 7, 100, 1000])
def test_chunk_size_does_not_change_results(kd, chunk):
    cfg = workload.config(1)
    H, W, idx, logp = workload.make_inputs(cfg)
    got = run_one(kd, H, W, idx, logp, chunk)
    assert_parity(got, oracle.fused_kl_reference(H, W, idx, logp), "f32", f"chunk={chunk}")


def test_neg_inf_and_out_of_range_entries(kd):
    # -inf log-probs and ids outside [0, V) both count as p = 0.
    H, W, idx, logp = _case(96, 64, 700, 6, "f32", seed=5)
    logp = logp.clone()
    logp[::3, -2] = float("-inf")
    logp[1, :-1] = float("-inf")
    bad = idx.clone()
    bad[:, -1] = torch.tensor([700, -1, 1 << 30], dtype=torch.int32).repeat(32)
    got = run_one(kd, H, W, bad, logp, 32)
    ref = oracle.fused_kl_reference(H, W, idx[:, :-1].contiguous(), logp[:, :-1].contiguous())
    assert_parity(got, ref, "f32", "-inf / out of range")


@pytest.mark.parametrize("reduction", ["sum", "mean"])
@pytest.mark.parametrize("N,d,V,K,dtype,chunk", [
    (130, 64, 129, 5, "f32", 64),
    (300, 160, 2000, 100, "bf16", 256),
])
def test_weighted_parity(kd, N, d, V, K, dtype, chunk, reduction):
    H, W, idx, logp = _case(N, d, V, K, dtype, seed=N + V + K)
    g = torch.Generator().manual_seed(N)
    w = torch.rand(N, generator=g) * 2.0
    w[torch.rand(N, generator=g) < 0.3] = 0.0
    got = run_one(kd, H, W, idx, logp, chunk, grad=0.8, weight=w, reduction=reduction)
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=0.8, weight=w.numpy(),
                                    reduction=reduction)
    assert_parity(got, ref, dtype, f"{N},{d},{V},{K},{dtype},{chunk},{reduction}")


def test_teacher_equal_to_student_gives_zero_loss(kd):
    H, W, _, _ = _case(64, 32, 500, 8, "f32", seed=6)
    logq = torch.log_softmax(H.double() @ W.double().T, dim=1)
    vals, idx = torch.topk(logq, 8, dim=1)
    got = run_one(kd, H, W, idx.to(torch.int32), vals.float(), 16)
    assert np.abs(got["loss_tok"]).max() < 1e-5


@pytest.mark.parametrize("N,d,V,K,dtype,chunk,weighted", [
    (300, 160, 2000, 100, "bf16", 128, False),
    (1100, 96, 3000, 20, "bf16", 128, True),
    (130, 64, 129, 5, "f32", 64, True),
])
def test_same_results_as_two_pass(kd, N, d, V, K, dtype, chunk, weighted):
    """Same logits, partials and combine, and dlogits from the same float32
    operations: every output is bitwise that of kd_fused_kl_fwd_ex followed
    by kd_fused_kl_bwd_ex."""
    H, W, idx, logp = _case(N, d, V, K, dtype, seed=N + d + 1)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    w = torch.rand(N, generator=torch.Generator().manual_seed(4)).to(Hd.device) if weighted else None
    red = "mean" if weighted else "sum"
    g = torch.full((1,), 1.7, dtype=torch.float32, device=Hd.device)
    l2, t2, s2 = kd.kl_forward(Hd, Wd, id_, lp, chunk, weight=w, reduction=red)
    dH2, dW2 = kd.kl_backward(Hd, Wd, id_, lp, s2, g, chunk, weight=w, reduction=red)
    l1, t1, s1, dH1, dW1 = kd.kl_forward_backward(Hd, Wd, id_, lp, chunk, grad=g, weight=w,
                                                  reduction=red)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(t1, t2) and torch.equal(s1, s2)
    assert torch.equal(dH1, dH2) and torch.equal(dW1, dW2)


def test_dw_accumulate_skip_outputs_and_loss_tok(kd):
    H, W, idx, logp = _case(100, 64, 333, 4, "f32", seed=7)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    _, _, _, _, dW1 = kd.kl_forward_backward(Hd, Wd, id_, lp, 32, need_dH=False)
    acc = dW1.clone()
    kd.kl_forward_backward(Hd, Wd, id_, lp, 32, need_dH=False, dW_out=acc, accumulate=True)
    loss, tok, _, dH_only, none = kd.kl_forward_backward(Hd, Wd, id_, lp, 32, need_dW=False,
                                                         want_loss_tok=False)
    torch.cuda.synchronize()
    assert none is None and tok is None
    assert torch.allclose(acc, 2 * dW1, rtol=1e-6, atol=1e-7)
    ref = oracle.fused_kl_reference(H, W, idx, logp)
    assert rel_err(loss.item(), ref["loss"]) < 1e-4
    assert max_norm_err(dH_only.double().cpu().numpy(), ref["dH"]) < 1e-4


def test_empty_input(kd):
    dev = torch.device("cuda:0")
    H = torch.empty(0, 64, device=dev)
    W = torch.randn(100, 64, device=dev)
    idx = torch.empty(0, 4, dtype=torch.int32, device=dev)
    logp = torch.empty(0, 4, device=dev)
    dW_out = torch.full((100, 64), 3.0, device=dev)
    loss, tok, _, dH, dW = kd.kl_forward_backward(H, W, idx, logp, 16, dW_out=dW_out)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and tok.numel() == 0 and dH.numel() == 0
    assert torch.count_nonzero(dW).item() == 0


def test_bitwise_deterministic(kd):
    H, W, idx, logp = _case(300, 160, 2000, 100, "bf16", seed=8)
    a = run_one(kd, H, W, idx, logp, 128)
    b = run_one(kd, H, W, idx, logp, 128)
    for k in ("loss_tok", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k
    assert a["loss"] == b["loss"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_autograd_one_pass(kd, dtype):
    """fused_kl(one_pass=True): with loss.backward() (upstream gradient 1) the
    gradients are bitwise those of the default two-pass autograd path; with
    another upstream gradient they match the oracle; a second backward
    through the same graph is refused."""
    H, W, idx, logp = _case(300, 96, 2000, 16, dtype, seed=21)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    grads = []
    for one_pass in (False, True):
        h = Hd.clone().requires_grad_(True)
        w = Wd.clone().requires_grad_(True)
        loss = kd.fused_kl(h, w, id_, lp, chunk=128, one_pass=one_pass)
        loss.backward()
        torch.cuda.synchronize()
        grads.append((loss.detach(), h.grad, w.grad))
    (l0, h0, w0), (l1, h1, w1) = grads
    assert torch.equal(l0, l1) and torch.equal(h0, h1) and torch.equal(w0, w1)
    assert h1.dtype == Hd.dtype and w1.dtype == Wd.dtype

    h = Hd.clone().requires_grad_(True)
    w = Wd.clone().requires_grad_(True)
    g = torch.Generator().manual_seed(22)
    wt = torch.rand(300, generator=g).to(Hd.device)
    loss = kd.fused_kl(h, w, id_, lp, chunk=128, weight=wt, reduction="mean", one_pass=True)
    (0.37 * loss).backward(retain_graph=True)
    torch.cuda.synchronize()
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=0.37, weight=wt.cpu().numpy(),
                                    reduction="mean")
    t = TOL[dtype]
    assert rel_err(loss.item(), ref["loss"]) < t["loss"]
    assert max_norm_err(h.grad.double().cpu().numpy(), ref["dH"]) < t["grad"]
    assert max_norm_err(w.grad.double().cpu().numpy(), ref["dW"]) < t["grad"]
    with pytest.raises(RuntimeError):
        loss.backward()


def test_autograd_one_pass_only_h(kd):
    # W frozen: only dH is computed and returned.
    H, W, idx, logp = _case(200, 64, 900, 8, "bf16", seed=23)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    h = Hd.clone().requires_grad_(True)
    loss = kd.fused_kl(h, Wd, id_, lp, chunk=64, one_pass=True)
    loss.backward()
    torch.cuda.synchronize()
    ref = oracle.fused_kl_reference(H, W, idx, logp)
    assert max_norm_err(h.grad.double().cpu().numpy(), ref["dH"]) < TOL["bf16"]["grad"]
    assert Wd.grad is None


# --------------------------------------------------------------------------
# full size: the 8K-token head (the launch configuration bench.py times) and
# the gpt-oss head (d = 2880, V = 201,088, 2,048-row chunks)
# --------------------------------------------------------------------------
def _full_size(kd, cfg, rows_extra):
    H, W, idx, logp = workload.make_inputs(cfg, teacher_device="cuda")
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    loss, tok, lse, dH, dW = kd.kl_forward_backward(Hd, Wd, id_, lp, cfg.chunk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.N + cfg.V + 1)
    rows = sorted(set(rows_extra) | set(rng.integers(0, cfg.N, 8).tolist()))
    ref = oracle.rows_reference(H, oracle.to_f64(W), idx, logp, rows)
    sel = torch.tensor(rows, device=Hd.device)
    assert rel_err(tok[sel].double().cpu().numpy(), ref["loss_tok"]) < 2e-3
    assert rel_err(lse[sel].double().cpu().numpy(), ref["lse"]) < 2e-3
    assert max_norm_err(dH[sel].double().cpu().numpy(), ref["dH"]) < 2e-2
    total = tok.double().sum().item()
    assert abs(loss.item() - total) <= 1e-5 * abs(total)
    dW64 = dW.double()
    assert dW64.sum(dim=0).abs().max().item() < 1e-3 * dW64.abs().max().item() * np.sqrt(cfg.V)
    a = (dW64 * Wd.double()).sum().item()
    b = (dH.double() * Hd.double()).sum().item()
    assert abs(a - b) < 2e-2 * max(abs(a), abs(b), 1e-12)
    del dW64
    # and the two-pass calls on the same inputs
    l2, t2, s2 = kd.kl_forward(Hd, Wd, id_, lp, cfg.chunk)
    dH2, dW2 = kd.kl_backward(Hd, Wd, id_, lp, s2, torch.ones(1, device=Hd.device), cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(loss, l2) and torch.equal(tok, t2) and torch.equal(lse, s2)
    assert torch.equal(dH, dH2) and torch.equal(dW, dW2)


@pytest.mark.timeout(900)
def test_full_size_8k_head(kd):
    cfg = workload.config(3)
    _full_size(kd, cfg, [0, 255, 256, 1023, 1024, 4095, 4096, cfg.N - 1])
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_size_gpt_oss_head(kd):
    cfg = workload.config(5)
    _full_size(kd, cfg, [0, 2047, 2048, 16383, cfg.N - 1])
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_full_size_long_context_262k(kd):
    # The longest point of the long-context sweep: 262,144 tokens in 2,048-row
    # chunks, 64 dW windows of two chunks each.
    cfg = workload.config(4, N=workload.SWEEP_N[-1])
    _full_size(kd, cfg, [0, 2047, 2048, 4095, 4096, cfg.N // 2, cfg.N - 1])
    torch.cuda.empty_cache()
