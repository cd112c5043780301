"""The library's kernel timing (kd_timing_enable / kd_timing_read), from which
bench.py computes its roofline entry and per-class kernel times.

The launches recorded per kernel class follow the chunk schedule of each call,
every recorded class has a positive duration, a read clears the record, and
timing changes no output bit.
"""
import ctypes

import pytest
import torch

from test_gpu_parity import _case, _to_dev, kd  # noqa: F401

pytestmark = pytest.mark.gpu


def _read(L):
    from chunked_kl_loss_chunk_amd import _lib

    n = len(_lib.KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _lib.check("kd_timing_read", L.kd_timing_read(ms, cnt))
    return {c: (ms[i], cnt[i]) for i, c in enumerate(_lib.KERNEL_CLASSES)}


def _counts(rec):
    return {c: n for c, (_, n) in rec.items()}


# N = 1000 rows in chunks of 128: 7 full chunks and one of 104. V = 3000 gives
# 12 vocabulary tiles, so one prep group covers all 8 chunks, and so does one
# launch of the forward's logit GEMM (up to 16,384 rows). The dW window is
# min(4, 4096 / 128) = 4 chunks, so 2 windows, each with one dlogits launch;
# each window's dH is split over the vocabulary (2 tiles of 256 window rows ×
# 1 d tile, far below the 768 workgroups the split aims at) and reduced once.
N, D, V, K, CHUNK = 1000, 64, 3000, 16, 128
CHUNKS, WINDOWS, FWD_LAUNCHES = 8, 2, 1


def test_timing_follows_the_schedule_and_changes_nothing(kd):
    L = kd.lib()
    H, W, idx, logp = _case(N, D, V, K, "bf16", 11)
    Hd, Wd, id_, lp = _to_dev(H, W, idx, logp)
    g = torch.ones(1, dtype=torch.float32, device=Hd.device)

    def two_pass():
        loss, tok, lse = kd.kl_forward(Hd, Wd, id_, lp, CHUNK)
        dH, dW = kd.kl_backward(Hd, Wd, id_, lp, lse, g, CHUNK)
        return [loss, tok, lse, dH, dW]

    def one_pass():
        return list(kd.kl_forward_backward(Hd, Wd, id_, lp, CHUNK, grad=g))

    ref2, ref1 = two_pass(), one_pass()
    torch.cuda.synchronize()
    _read(L)  # nothing recorded while timing is off
    assert all(n == 0 for n in _counts(_read(L)).values())

    try:
        assert L.kd_timing_enable(1) == 0
        out2 = two_pass()
        torch.cuda.synchronize()
        rec2 = _read(L)
        out1 = one_pass()
        torch.cuda.synchronize()
        rec1 = _read(L)
    finally:
        L.kd_timing_enable(0)

    # The forward: one prep pass; per launch of the logit GEMM (all 8 chunks)
    # a transpose of its chunks of H (bf16), the GEMM and a combine. The
    # backward: the same prep; per window a transpose, one recomputing
    # dlogits GEMM over its chunks, dW and dH (+ reduce).
    assert _counts(rec2) == {"prep": (1 + FWD_LAUNCHES) + (1 + WINDOWS),
                             "fwd_logits": FWD_LAUNCHES, "bwd_dlogits": WINDOWS,
                             "bwd_dh": WINDOWS, "bwd_dw": WINDOWS,
                             "other": FWD_LAUNCHES + WINDOWS, "dl_stream": 0}
    # One pass: no prep groups, the storing logit GEMM, the combine and the
    # streaming dlogits pair per chunk, then the same windows.
    assert _counts(rec1) == {"prep": CHUNKS, "fwd_logits": CHUNKS, "bwd_dlogits": 0,
                             "bwd_dh": WINDOWS, "bwd_dw": WINDOWS, "other": CHUNKS + WINDOWS,
                             "dl_stream": CHUNKS}
    for rec in (rec2, rec1):
        for c, (ms, n) in rec.items():
            if n:
                assert ms > 0.0, (c, ms)
    # a read clears the record
    assert all(n == 0 for n in _counts(_read(L)).values())
    # timing only brackets the launches: every output is bitwise unchanged
    for a, b in zip(out2 + out1, ref2 + ref1):
        assert torch.equal(a, b)

