"""The no-allocation forward entry point (kd_fused_kl_fwd_noalloc) against
the workspace-taking forward (kd_fused_kl_fwd_ex) on the same inputs.

Both run the same kernels in the same order, so every output is compared
bit for bit, and both are also checked against the fp64 oracle at the
tolerances of test_gpu_parity.py. Two calls in a row share the library's
scratch; the second is smaller than the first, so stale contents of the
first call would show up in it.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_kl_loss_chunk_amd import _lib
from test_gpu_parity import _case, _to_dev, assert_parity, kd  # noqa: F401

pytestmark = pytest.mark.gpu


def _noalloc(kd, Hd, Wd, id_, lp, chunk, weight=None, reduction="sum"):
    N = Hd.shape[0]
    loss = torch.empty(1, dtype=torch.float32, device=Hd.device)
    lse = torch.empty(N, dtype=torch.float32, device=Hd.device)
    tok = torch.empty(N, dtype=torch.float32, device=Hd.device)
    kd.kl_forward_noalloc(Hd, Wd, id_, lp, chunk, loss, lse, loss_tok=tok, weight=weight,
                          reduction=reduction)
    return loss, tok, lse


@pytest.mark.parametrize("first,second", [
    # a weighted mean over several prep groups' worth of tiles, then a smaller sum
    ((1100, 96, 3000, 20, "bf16", 128, True), (300, 160, 2000, 100, "bf16", 256, False)),
    ((300, 64, 900, 8, "f32", 64, False), (130, 64, 129, 5, "f32", 32, True)),
])
def test_noalloc_forward_matches_workspace_forward(kd, first, second):
    for N, d, V, K, dtype, chunk, weighted in (first, second):
        H, W, idx, logp = _case(N, d, V, K, dtype, seed=N + V + 3)
        Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
        w = None
        red = "sum"
        if weighted:
            w = torch.rand(N, generator=torch.Generator().manual_seed(N)) * 2.0
            red = "mean"
        wd = None if w is None else w.to(Hd.device)
        l2, t2, s2 = _noalloc(kd, Hd, Wd, id_, lp, chunk, weight=wd, reduction=red)
        l1, t1, s1 = kd.kl_forward(Hd, Wd, id_, lp, chunk, weight=wd, reduction=red)
        torch.cuda.synchronize()
        assert torch.equal(l1, l2) and torch.equal(t1, t2) and torch.equal(s1, s2), (N, d, V)
        ref = oracle.fused_kl_reference(H, W, idx, logp, weight=None if w is None else w.numpy(),
                                        reduction=red)
        got = {"loss": float(l2.item()), "loss_tok": t2.double().cpu().numpy(),
               "lse": s2.double().cpu().numpy()}
        assert_parity(got, ref, dtype, f"noalloc {N},{d},{V},{K},{dtype},{chunk}")


def test_noalloc_without_loss_tok_and_empty(kd):
    H, W, idx, logp = _case(257, 72, 515, 4, "bf16", seed=11)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    loss = torch.empty(1, dtype=torch.float32, device=Hd.device)
    lse = torch.empty(257, dtype=torch.float32, device=Hd.device)
    kd.kl_forward_noalloc(Hd, Wd, id_, lp, 128, loss, lse)
    l1, _, s1 = kd.kl_forward(Hd, Wd, id_, lp, 128, want_loss_tok=False)
    torch.cuda.synchronize()
    assert torch.equal(loss, l1) and torch.equal(lse, s1)
    # N = 0 writes a zero loss
    e = torch.empty(0, 72, dtype=torch.bfloat16, device=Hd.device)
    ei = torch.empty(0, 4, dtype=torch.int32, device=Hd.device)
    el = torch.empty(0, 4, dtype=torch.float32, device=Hd.device)
    loss.fill_(5.0)
    kd.kl_forward_noalloc(e, Wd, ei, el, 16, loss, torch.empty(0, device=Hd.device))
    torch.cuda.synchronize()
    assert loss.item() == 0.0


def test_noalloc_rejects_sizes_beyond_its_scratch(kd):
    # 65,536 positions with K = 200: the bucketed cache alone is 105 MB.
    N, d, V, K, chunk = 65536, 8, 1000, 200, 1024
    need = kd.workspace_bytes(_lib.KD_PASS_FWD, N, d, V, K, chunk, torch.bfloat16)
    assert need > _lib.KD_NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    H = torch.zeros(N, d, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(V, d, dtype=torch.bfloat16, device=dev)
    idx = torch.arange(K, dtype=torch.int32, device=dev).repeat(N, 1).contiguous()  # distinct per row
    logp = torch.zeros(N, K, dtype=torch.float32, device=dev)
    loss = torch.full((1,), 7.0, device=dev)
    lse = torch.full((N,), 7.0, device=dev)
    with pytest.raises(_lib.KDError) as e:
        kd.kl_forward_noalloc(H, W, idx, logp, chunk, loss, lse)
    assert e.value.status == _lib.KD_ERR_WORKSPACE
    torch.cuda.synchronize()
    # nothing was enqueued: the outputs are untouched
    assert loss.item() == 7.0 and bool((lse == 7.0).all())
    # and the same call with the largest accepted chunk group still works
    n2 = 4096
    need2 = kd.workspace_bytes(_lib.KD_PASS_FWD, n2, d, V, K, chunk, torch.bfloat16)
    assert need2 <= _lib.KD_NOALLOC_SCRATCH_BYTES
    kd.kl_forward_noalloc(H[:n2], W, idx[:n2], logp[:n2], chunk, loss, lse[:n2])
    torch.cuda.synchronize()
    assert np.isfinite(loss.item())


def test_noalloc_at_the_8k_head(kd):
    """The 8K-token head in the bench's launch configuration (17 MiB of the
    64 MiB scratch): bitwise the workspace forward's outputs."""
    import workload

    cfg = workload.config(3)
    H, W, idx, logp = workload.make_inputs(cfg, teacher_device="cuda")
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    l2, t2, s2 = _noalloc(kd, Hd, Wd, id_, lp, cfg.chunk)
    l1, t1, s1 = kd.kl_forward(Hd, Wd, id_, lp, cfg.chunk)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2) and torch.equal(t1, t2) and torch.equal(s1, s2)
    del Hd, Wd, id_, lp
    torch.cuda.empty_cache()
