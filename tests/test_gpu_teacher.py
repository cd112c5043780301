"""GPU parity of the offline teacher cache producer (kd_teacher_topk) against
the fp64 oracle (oracle/teacher_oracle.py).

The kernels rank float32 logits and the oracle float64 ones, so where two
logits are closer than the float32 error the two may order them differently.
Each row is therefore checked for what is unique and for validity:
- ids distinct and in range;
- log-probabilities within tolerance of the oracle's value for the same id;
- every kept id within TOL_Z of the oracle's K-th largest logit or above it,
  and no dropped id above that cut by more than TOL_Z;
- wherever the GPU order differs from the oracle's, the two ids' oracle logits
  agree within TOL_Z.
With small-integer inputs every logit is exact in both, and the ids, including
the lower-id-first rule for ties, must match exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from test_gpu_parity import kd  # noqa: F401

pytestmark = pytest.mark.gpu

TOL_Z = 1e-4      # float32 logits vs float64, absolute (logits are O(1..10) here)
TOL_LOGP = 2e-4   # absolute, on log-probabilities


def _run(kd, Ht, Wt, K, chunk):
    dev = torch.device("cuda:0")
    idx, logp, lse = kd.teacher_topk(Ht.to(dev), Wt.to(dev), K, chunk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), logp.double().cpu().numpy(), lse.double().cpu().numpy()


def check_rows(idx, logp, lse, ref, K):
    Z, lse_ref, idx_ref = ref["Z"], ref["lse"], ref["idx"]
    N, V = Z.shape
    for r in range(N):
        ids = idx[r]
        assert len(set(ids.tolist())) == K and ids.min() >= 0 and ids.max() < V, r
        assert abs(lse[r] - lse_ref[r]) < TOL_LOGP, (r, lse[r], lse_ref[r])
        np.testing.assert_allclose(logp[r], Z[r, ids] - lse_ref[r], rtol=0, atol=TOL_LOGP)
        cut = np.sort(Z[r])[::-1][K - 1]
        assert Z[r, ids].min() >= cut - TOL_Z, r
        dropped = np.setdiff1d(np.arange(V), ids)
        if dropped.size:
            assert Z[r, dropped].max() <= cut + TOL_Z, r
        diff = ids != idx_ref[r]
        assert np.all(np.abs(Z[r, ids[diff]] - Z[r, idx_ref[r][diff]]) <= TOL_Z), r


def _inputs(N, d, V, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    Ht = torch.randn(N, d, generator=g)
    Wt = torch.randn(V, d, generator=g) * 2.0 / math.sqrt(d)  # teacher logits with std ≈ 2
    if dtype == "bf16":
        Ht, Wt = Ht.to(torch.bfloat16), Wt.to(torch.bfloat16)
    return Ht.contiguous(), Wt.contiguous()


@pytest.mark.parametrize("N,d,V,K,dtype,chunk", [
    (100, 64, 1000, 8, "f32", 32),          # 4 vocabulary tiles < K = 8: every logit is a candidate
    (300, 128, 5000, 100, "bf16", 128),     # 20 tiles < K = 100: every logit is a candidate
    (257, 72, 70000, 100, "bf16", 256),     # 274 tiles >= K: the tile-maximum threshold; ragged V
    (64, 32, 40, 40, "f32", 16),            # K = V
    (130, 64, 129, 1, "f32", 64),           # K = 1, a one-column last tile
    (200, 96, 3000, 5, "bf16", 1000),       # one chunk, 12 tiles >= K = 5
    (40, 64, 270000, 100, "bf16", 32),      # 1055 tiles: τ searched from memory, not registers
])
def test_teacher_topk_parity(kd, N, d, V, K, dtype, chunk):
    Ht, Wt = _inputs(N, d, V, dtype, seed=N + V + K)
    idx, logp, lse = _run(kd, Ht, Wt, K, chunk)
    ref = oracle.teacher_topk_reference(Ht.double().numpy(), Wt.double().numpy(), K)
    check_rows(idx, logp, lse, ref, K)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_teacher_topk_integer_logits_exact_with_ties(kd, dtype):
    # Entries in {-2..2}: every product and sum is an exact small integer in
    # float32 (and bf16 inputs), so logits tie exactly and often; the ids must
    # equal the oracle's, ties by the lower id first.
    g = torch.Generator().manual_seed(61)
    Ht = torch.randint(-2, 3, (150, 64), generator=g).float()
    Wt = torch.randint(-2, 3, (3000, 64), generator=g).float()
    Wt[2500] = Wt[17]  # duplicate rows: equal logits in every row
    Wt[2999] = Wt[17]
    if dtype == "bf16":
        Ht, Wt = Ht.to(torch.bfloat16), Wt.to(torch.bfloat16)
    K = 50
    idx, logp, lse = _run(kd, Ht.contiguous(), Wt.contiguous(), K, 64)
    ref = oracle.teacher_topk_reference(Ht.double().numpy(), Wt.double().numpy(), K)
    assert np.array_equal(idx, ref["idx"])
    np.testing.assert_allclose(logp, ref["logp"], rtol=0, atol=TOL_LOGP)


@pytest.mark.parametrize("V,chunk", [(20000, 128), (8192, 300)])
def test_teacher_topk_uniform_teacher(kd, V, chunk):
    # A zero head: every logit of every row is 0, so τ = 0 and all V logits
    # are candidates (the lists fill to V entries; V = 20,000 spans three
    # 8192-logit scan workgroups per row, the last one ragged). The kept ids
    # are the K lowest, each with log-probability −ln V.
    N, d, K = 300, 64, 64
    Ht = torch.randn(N, d, generator=torch.Generator().manual_seed(65))
    Wt = torch.zeros(V, d)
    idx, logp, lse = _run(kd, Ht, Wt, K, chunk)
    assert np.array_equal(idx, np.tile(np.arange(K, dtype=idx.dtype), (N, 1)))
    np.testing.assert_allclose(logp, -math.log(V), rtol=0, atol=TOL_LOGP)
    np.testing.assert_allclose(lse, math.log(V), rtol=1e-6, atol=0)


def test_teacher_cache_feeds_the_loss(kd):
    # The producer's cache, used as the loss's teacher input, gives the loss
    # the oracle's cache gives (end to end through both entry points).
    g = torch.Generator().manual_seed(62)
    N, d, V, K = 200, 64, 2000, 16
    Ht = torch.randn(N, d, generator=g)
    Wt = torch.randn(V, d, generator=g) * 2.0 / math.sqrt(d)
    H = torch.randn(N, d, generator=g)
    W = torch.randn(V, d, generator=g) / math.sqrt(d)
    idx, logp, _ = _run(kd, Ht, Wt, K, 64)
    ref = oracle.teacher_topk_reference(Ht.double().numpy(), Wt.double().numpy(), K)
    dev = torch.device("cuda:0")
    loss_gpu_cache, _, _ = kd.kl_forward(H.to(dev), W.to(dev), torch.from_numpy(idx).to(dev),
                                         torch.from_numpy(logp).float().to(dev), 64)
    want = oracle.fused_kl_reference(H, W, ref["idx"], ref["logp"])["loss"]
    assert abs(loss_gpu_cache.item() - want) / abs(want) < 1e-4


def test_teacher_topk_empty(kd):
    dev = torch.device("cuda:0")
    idx, logp, lse = kd.teacher_topk(torch.empty(0, 64, device=dev), torch.randn(100, 64, device=dev), 5)
    torch.cuda.synchronize()
    assert idx.shape == (0, 5) and logp.shape == (0, 5) and lse.shape == (0,)


def test_teacher_topk_full_size_sampled_rows(kd):
    # An 8B-class teacher head (d = 4096, V = 128,256) over 1,536 positions in
    # 1,024-row chunks (a ragged second chunk); 12 sampled rows against the oracle.
    N, d, V, K = 1536, 4096, 128256, 100
    Ht, Wt = _inputs(N, d, V, "bf16", seed=63)
    idx, logp, lse = _run(kd, Ht, Wt, K, 1024)
    rows = np.array([0, 1, 511, 777, 1023, 1024, 1025, 1300, 1499, 1533, 1534, 1535])
    ref = oracle.teacher_topk_reference(Ht[rows].double().numpy(), Wt.double().numpy(), K)
    check_rows(idx[rows], logp[rows], lse[rows], ref, K)


def test_teacher_topk_gpt_oss_vocabulary_sampled_rows(kd):
    # The gpt-oss vocabulary (V = 201,088: a ragged last tile and 25 streaming
    # workgroups per row) with d = 2880, over 2,500 positions in 1,024-row
    # chunks; 10 sampled rows against the oracle.
    N, d, V, K = 2500, 2880, 201088, 100
    Ht, Wt = _inputs(N, d, V, "bf16", seed=66)
    idx, logp, lse = _run(kd, Ht, Wt, K, 1024)
    rows = np.array([0, 1, 1023, 1024, 1500, 2047, 2048, 2400, 2498, 2499])
    ref = oracle.teacher_topk_reference(Ht[rows].double().numpy(), Wt.double().numpy(), K)
    check_rows(idx[rows], logp[rows], lse[rows], ref, K)


def test_teacher_topk_bitwise_repeatable(kd):
    Ht, Wt = _inputs(400, 96, 9000, "bf16", seed=64)
    a = _run(kd, Ht, Wt, 64, 128)
    b = _run(kd, Ht, Wt, 64, 128)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
