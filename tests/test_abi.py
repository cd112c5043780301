"""The C ABI on a host without a GPU: the library loads, exports every symbol
the header declares, sizes its workspace, and rejects every invalid argument
before anything is enqueued. Every call below has at least one invalid
argument, so no kernel is ever launched and no pointer is dereferenced."""
import ctypes
import os
import re

import pytest
import torch

from chunked_kl_loss_chunk_amd import _build, _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kd_fused_kl.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    return _lib.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_all_exported(L):
    names = _declared_functions()
    assert "kd_fused_kl_fwd" in names and "kd_fused_kl_bwd" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_status_strings(L):
    assert _lib.status_str(0) == "KD_OK"
    assert _lib.status_str(3) == "KD_ERR_WORKSPACE"
    assert _lib.status_str(4) == "KD_ERR_HIP"
    assert _lib.status_str(99) == "KD_UNKNOWN_STATUS"


def _ws(L, pass_, N, d, V, K, C, dt):
    return L.kd_fused_kl_workspace_bytes(pass_, N, d, V, K, C, dt)


def test_workspace_size_rules(L):
    f, b = _lib.KD_PASS_FWD, _lib.KD_PASS_BWD
    bf, f32 = _lib.KD_BF16, _lib.KD_F32
    # invalid sizes -> 0
    assert _ws(L, f, -1, 64, 1000, 8, 32, f32) == 0
    assert _ws(L, f, 128, 0, 1000, 8, 32, f32) == 0
    assert _ws(L, f, 128, 64, 1000, 1001, 32, f32) == 0  # K > V
    assert _ws(L, f, 128, 64, 1000, 0, 32, f32) == 0
    assert _ws(L, f, 128, 64, 1000, 8, 0, f32) == 0
    assert _ws(L, f, 128, 63, 1000, 8, 32, f32) == 0  # 63*4 bytes is not a multiple of 16
    assert _ws(L, f, 128, 68, 1000, 8, 32, bf) == 0   # 68*2 bytes is not a multiple of 16
    assert _ws(L, f, 128, 64, 1000, 8, 32, 7) == 0
    assert _ws(L, 4, 128, 64, 1000, 8, 32, f32) == 0  # passes: 0 fwd, 1 bwd, 2 teacher, 3 fwd+bwd
    assert _ws(L, -1, 128, 64, 1000, 8, 32, f32) == 0
    assert _ws(L, f, 128, 64, 100000, 20000, 32, f32) == 0  # K beyond the record format
    # valid
    wf = _ws(L, f, 8192, 3072, 128256, 100, 1024, bf)
    wb = _ws(L, b, 8192, 3072, 128256, 100, 1024, bf)
    assert wf > 0 and wb > 0 and wf % 256 == 0 and wb % 256 == 0
    # the backward holds a window of chunks' dlogits: at least C x V_pad bf16
    V_pad = (128256 + 127) // 128 * 128
    assert wb >= 1024 * V_pad * 2
    # the window covers 4096 rows with chunks of 1024 or 2048; one chunk of
    # 8192 is a window of its own, twice as many rows
    assert _ws(L, b, 8192, 3072, 128256, 100, 2048, bf) == wb
    assert _ws(L, b, 8192, 3072, 128256, 100, 8192, bf) > wb
    # Past the prep group of 65,536 rows the backward workspace no longer
    # grows with N; below it, it grows by at most the bucketed cache entries
    # (8 bytes per entry, plus S_r) of the extra rows.
    b64 = _ws(L, b, 65536, 3072, 128256, 100, 1024, bf)
    assert _ws(L, b, 262144, 3072, 128256, 100, 1024, bf) == b64
    assert _ws(L, b, 1 << 20, 3072, 128256, 100, 1024, bf) == b64
    assert 0 < b64 - wb <= (65536 - 8192) * (8 * 100 + 4) + 64 * 1024 * 4 * 4 + 4096
    # past the group the forward workspace grows only by its per-token loss buffer
    w1 = _ws(L, f, 65536, 3072, 128256, 100, 2048, bf)
    w2 = _ws(L, f, 131072, 3072, 128256, 100, 2048, bf)
    w4 = _ws(L, f, 262144, 3072, 128256, 100, 2048, bf)
    assert 0 < w2 - w1 <= 4 * 65536 + 256 and abs((w4 - w2) - 2 * (w2 - w1)) <= 512
    # a chunk larger than N is clamped to N
    assert _ws(L, b, 100, 64, 1000, 8, 4096, f32) == _ws(L, b, 100, 64, 1000, 8, 100, f32)


FAKE = 0x100000  # 16-byte-aligned, never dereferenced (every call is rejected first)


def _fwd(L, **kw):
    a = dict(H=FAKE, W=FAKE, dt=_lib.KD_F32, idx=FAKE, logp=FAKE, N=128, d=64, V=1000, K=8, C=32,
             loss_tok=FAKE, lse=FAKE, loss_sum=FAKE, ws=FAKE, ws_n=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kd_fused_kl_fwd(vp(a["H"]), vp(a["W"]), a["dt"], vp(a["idx"]), vp(a["logp"]), a["N"],
                             a["d"], a["V"], a["K"], a["C"], vp(a["loss_tok"]), vp(a["lse"]),
                             vp(a["loss_sum"]), vp(a["ws"]), a["ws_n"], a["stream"])


def _bwd(L, **kw):
    a = dict(H=FAKE, W=FAKE, dt=_lib.KD_F32, idx=FAKE, logp=FAKE, lse=FAKE, N=128, d=64, V=1000, K=8,
             C=32, grad=FAKE, dH=FAKE, dW=FAKE, acc=0, ws=FAKE, ws_n=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kd_fused_kl_bwd(vp(a["H"]), vp(a["W"]), a["dt"], vp(a["idx"]), vp(a["logp"]),
                             vp(a["lse"]), a["N"], a["d"], a["V"], a["K"], a["C"], vp(a["grad"]),
                             vp(a["dH"]), vp(a["dW"]), a["acc"], vp(a["ws"]), a["ws_n"], a["stream"])


INV, UNS, WSE = _lib.KD_ERR_INVALID_ARG, _lib.KD_ERR_UNSUPPORTED, _lib.KD_ERR_WORKSPACE


@pytest.mark.parametrize("kw,want", [
    (dict(N=-1), INV), (dict(d=0), INV), (dict(V=0), INV), (dict(K=0), INV), (dict(K=1001), INV),
    (dict(C=0), INV), (dict(C=-5), INV), (dict(dt=2), INV), (dict(d=63), INV),
    (dict(K=20000, V=100000), UNS), (dict(V=(1 << 28) + 1), UNS), (dict(V=1 << 22), UNS),
    (dict(H=None), INV), (dict(W=None), INV), (dict(idx=None), INV), (dict(logp=None), INV),
    (dict(lse=None), INV), (dict(loss_sum=None), INV),
    (dict(H=FAKE + 8), INV), (dict(W=FAKE + 4), INV), (dict(idx=FAKE + 2), INV),
    (dict(loss_tok=FAKE + 1), INV), (dict(loss_sum=FAKE + 2), INV),
    (dict(ws=None), WSE), (dict(ws=FAKE + 16), WSE), (dict(ws_n=1024), WSE),
])
def test_forward_rejects_invalid(L, kw, want):
    assert _fwd(L, **kw) == want


@pytest.mark.parametrize("kw,want", [
    (dict(N=-1), INV), (dict(d=0), INV), (dict(K=1001), INV), (dict(C=0), INV), (dict(dt=5), INV),
    (dict(acc=2), INV), (dict(acc=-1), INV),
    (dict(H=None), INV), (dict(W=None), INV), (dict(lse=None), INV), (dict(grad=None), INV),
    (dict(dH=FAKE + 8), INV), (dict(dW=FAKE + 4), INV), (dict(grad=FAKE + 2), INV),
    (dict(ws=None), WSE), (dict(ws_n=4096), WSE),
])
def test_backward_rejects_invalid(L, kw, want):
    assert _bwd(L, **kw) == want


def test_cast_rejects_invalid(L):
    vp = ctypes.c_void_p
    assert L.kd_cast_f32_to_bf16(vp(FAKE), vp(FAKE), -1, None) == INV
    assert L.kd_cast_f32_to_bf16(None, vp(FAKE), 10, None) == INV
    assert L.kd_cast_f32_to_bf16(vp(FAKE), vp(FAKE + 8), 10, None) == INV  # overlap
    assert L.kd_cast_f32_to_bf16(vp(FAKE), vp(FAKE), 0, None) == _lib.KD_OK  # nothing to do


def test_scale_rejects_invalid(L):
    vp = ctypes.c_void_p
    assert L.kd_scale(vp(FAKE), _lib.KD_F32, -1, vp(FAKE), None) == INV
    assert L.kd_scale(vp(FAKE), 2, 10, vp(FAKE), None) == INV
    assert L.kd_scale(None, _lib.KD_F32, 10, vp(FAKE), None) == INV
    assert L.kd_scale(vp(FAKE), _lib.KD_F32, 10, None, None) == INV
    assert L.kd_scale(vp(FAKE + 2), _lib.KD_F32, 10, vp(FAKE), None) == INV   # fp32 needs 4-byte alignment
    assert L.kd_scale(vp(FAKE), _lib.KD_F32, 10, vp(FAKE + 1), None) == INV
    assert L.kd_scale(vp(FAKE), _lib.KD_BF16, 0, vp(FAKE), None) == _lib.KD_OK  # nothing to do


def test_timing_flag_and_read_validated(L):
    assert L.kd_timing_enable(2) == INV
    assert L.kd_timing_enable(-1) == INV
    assert L.kd_timing_read(None, None) == INV
    assert L.kd_timing_enable(0) == _lib.KD_OK


def test_binding_fails_loudly_without_gpu_tensors():
    from chunked_kl_loss_chunk_amd import ops
    H = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        ops.kl_forward(H, torch.zeros(10, 8), torch.zeros(4, 2, dtype=torch.int32),
                       torch.zeros(4, 2), chunk=2)


def test_noalloc_falls_back_to_one_chunk_per_launch_at_the_8k_head(L):
    """At the 8K head the forward projects all 8 chunks in one launch, whose
    workspace exceeds the no-allocation scratch; one chunk per launch fits. So
    the GPU test of the no-allocation forward at that head runs the
    fallback (tests/test_zz_no_alloc.py)."""
    grouped = L.kd_fused_kl_workspace_bytes(_lib.KD_PASS_FWD, 8192, 3072, 128256, 100, 1024,
                                            _lib.KD_BF16)
    assert grouped > _lib.KD_NOALLOC_SCRATCH_BYTES
    # one chunk per launch: the bucketed cache of the group, one transposed
    # chunk, and one chunk's z at the cached ids and partials
    one_chunk = (8192 * 100 * 8 + 8 * 4 * 502 * 4 + 8192 * 4 + 3072 * 1024 * 2
                 + 1024 * 100 * 4 + 1024 * 501 * 8)
    assert one_chunk < _lib.KD_NOALLOC_SCRATCH_BYTES


def test_vocabulary_row_limit(L):
    """The GEMM loaders take 32-bit offsets within a 256-row tile: a padded
    vocabulary row must stay under 8 MiB in the compute dtype."""
    ws = L.kd_fused_kl_workspace_bytes
    for dt, vmax in ((_lib.KD_F32, 2096896), (_lib.KD_BF16, 4194048)):
        for pass_ in (0, 1):
            assert ws(pass_, 128, 64, vmax, 8, 32, dt) > 0
            assert ws(pass_, 128, 64, vmax + 1, 8, 32, dt) == 0


def _fwd_ex(L, **kw):
    a = dict(H=FAKE, W=FAKE, dt=_lib.KD_F32, idx=FAKE, logp=FAKE, w=None, red=0, N=128, d=64, V=1000,
             K=8, C=32, loss_tok=FAKE, lse=FAKE, loss=FAKE, ws=FAKE, ws_n=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kd_fused_kl_fwd_ex(vp(a["H"]), vp(a["W"]), a["dt"], vp(a["idx"]), vp(a["logp"]),
                                vp(a["w"]), a["red"], a["N"], a["d"], a["V"], a["K"], a["C"],
                                vp(a["loss_tok"]), vp(a["lse"]), vp(a["loss"]), vp(a["ws"]),
                                a["ws_n"], a["stream"])


def _bwd_ex(L, **kw):
    a = dict(H=FAKE, W=FAKE, dt=_lib.KD_F32, idx=FAKE, logp=FAKE, w=None, red=0, lse=FAKE, N=128,
             d=64, V=1000, K=8, C=32, grad=FAKE, dH=FAKE, dW=FAKE, acc=0, ws=FAKE, ws_n=1 << 40,
             stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kd_fused_kl_bwd_ex(vp(a["H"]), vp(a["W"]), a["dt"], vp(a["idx"]), vp(a["logp"]),
                                vp(a["w"]), a["red"], vp(a["lse"]), a["N"], a["d"], a["V"], a["K"],
                                a["C"], vp(a["grad"]), vp(a["dH"]), vp(a["dW"]), a["acc"],
                                vp(a["ws"]), a["ws_n"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(red=2), INV), (dict(red=-1), INV), (dict(w=FAKE + 2), INV), (dict(d=63), INV),
    (dict(V=1 << 22), UNS), (dict(ws=None), WSE),
])
def test_weighted_entry_points_reject_invalid(L, kw, want):
    assert _fwd_ex(L, **kw) == want
    assert _bwd_ex(L, **kw) == want


def test_weighted_forward_requires_loss_output(L):
    assert _fwd_ex(L, loss=None) == INV


def _tk(L, **kw):
    a = dict(Ht=FAKE, Wt=FAKE, dt=_lib.KD_BF16, N=64, d=64, V=1000, K=8, C=32, idx=FAKE, logp=FAKE,
             lse=None, ws=FAKE, ws_n=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kd_teacher_topk(vp(a["Ht"]), vp(a["Wt"]), a["dt"], a["N"], a["d"], a["V"], a["K"],
                             a["C"], vp(a["idx"]), vp(a["logp"]), vp(a["lse"]), vp(a["ws"]),
                             a["ws_n"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(K=0), INV), (dict(K=1001), INV), (dict(K=2049, V=5000), UNS), (dict(d=4), INV),
    (dict(Ht=None), INV), (dict(idx=None), INV), (dict(logp=FAKE + 2), INV), (dict(lse=FAKE + 1), INV),
    (dict(ws=None), WSE), (dict(ws_n=1024), WSE), (dict(C=0), INV), (dict(dt=3), INV),
])
def test_teacher_topk_rejects_invalid(L, kw, want):
    assert _tk(L, **kw) == want


def test_teacher_workspace_holds_candidate_lists(L):
    ws = L.kd_fused_kl_workspace_bytes
    n = ws(_lib.KD_PASS_TEACHER, 4096, 4096, 128256, 100, 1024, _lib.KD_BF16)
    assert n >= 1024 * 128256 * 8  # up to V candidates of 8 bytes per row of a chunk
    assert ws(_lib.KD_PASS_TEACHER, 4096, 4096, 128256, 2048, 1024, _lib.KD_BF16) > 0
    assert ws(_lib.KD_PASS_TEACHER, 4096, 4096, 128256, 2049, 1024, _lib.KD_BF16) == 0
    assert ws(4, 4096, 4096, 128256, 100, 1024, _lib.KD_BF16) == 0


@pytest.mark.parametrize("args,want", [
    ((FAKE, FAKE, -1, 8, 100, FAKE), INV), ((FAKE, FAKE, 10, 0, 100, FAKE), INV),
    ((FAKE, FAKE, 10, 101, 100, FAKE), INV), ((FAKE, FAKE, 10, 16384, 20000, FAKE), INV),
    ((FAKE, FAKE, 10, 8, 100, None), INV), ((FAKE, FAKE, 10, 8, 100, FAKE + 2), INV),
    ((None, FAKE, 10, 8, 100, FAKE), INV), ((FAKE, FAKE + 1, 10, 8, 100, FAKE), INV),
])
def test_check_inputs_rejects_invalid(L, args, want):
    vp = ctypes.c_void_p
    idx, logp, N, K, V, flags = args
    assert L.kd_fused_kl_check_inputs(vp(idx), vp(logp), N, K, V, vp(flags), None) == want


def test_one_pass_workspace(L):
    """The one-pass call holds the backward's dlogits window plus one chunk of
    float32 logits, and no bucketed cache: constant in N past the window."""
    ws = L.kd_fused_kl_workspace_bytes
    bf, o, b = _lib.KD_BF16, _lib.KD_PASS_FWD_BWD, _lib.KD_PASS_BWD
    V_pad = (128256 + 255) // 256 * 256
    w1 = ws(o, 8192, 3072, 128256, 100, 1024, bf)
    assert w1 > 0 and w1 % 256 == 0
    assert w1 >= 1024 * V_pad * 4 + 4 * 1024 * V_pad * 2
    # no prep buckets: beyond the per-position loss buffer (4 bytes a row),
    # the size does not grow with N
    w2 = ws(o, 262144, 3072, 128256, 100, 1024, bf)
    assert 0 <= w2 - w1 <= 4 * (262144 - 8192) + 256
    # the extra over the backward is the chunk's logits (and small per-chunk
    # buffers), less the backward's bucketed entries and the three more
    # transposed chunks of H its dlogits launch (one dW window) reads
    wb = ws(b, 8192, 3072, 128256, 100, 1024, bf)
    held_by_bwd = 8 * 100 * 8192 + 3 * 3072 * 1024 * 2 + (1 << 22)
    assert 1024 * V_pad * 4 - held_by_bwd < w1 - wb <= 1024 * V_pad * 4 + (1 << 23)
    # the streaming pass over the stored logits (one-pass loss and teacher
    # cache) takes a workgroup per 8192 logits of a row: chunk x V_pad / 8192
    # workgroups must stay below 2^24
    for pass_ in (o, _lib.KD_PASS_TEACHER):
        assert ws(pass_, 1 << 20, 64, 1 << 16, 8, 1 << 20, _lib.KD_F32) > 0
        assert ws(pass_, 1 << 21, 64, 1 << 16, 8, 1 << 21, _lib.KD_F32) == 0
    for pass_ in (0, 1):
        assert ws(pass_, 1 << 21, 64, 1 << 16, 8, 1 << 21, _lib.KD_F32) > 0


def _fb(L, **kw):
    a = dict(H=FAKE, W=FAKE, dt=_lib.KD_F32, idx=FAKE, logp=FAKE, w=None, red=0, N=128, d=64,
             V=1000, K=8, C=32, grad=FAKE, loss_tok=FAKE, lse=FAKE, loss=FAKE, dH=FAKE, dW=FAKE,
             acc=0, ws=FAKE, ws_n=1 << 40, stream=None)
    a.update(kw)
    vp = ctypes.c_void_p
    return L.kd_fused_kl_fwd_bwd(vp(a["H"]), vp(a["W"]), a["dt"], vp(a["idx"]), vp(a["logp"]),
                                 vp(a["w"]), a["red"], a["N"], a["d"], a["V"], a["K"], a["C"],
                                 vp(a["grad"]), vp(a["loss_tok"]), vp(a["lse"]), vp(a["loss"]),
                                 vp(a["dH"]), vp(a["dW"]), a["acc"], vp(a["ws"]), a["ws_n"],
                                 a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(N=-1), INV), (dict(d=0), INV), (dict(V=0), INV), (dict(K=0), INV), (dict(K=1001), INV),
    (dict(C=0), INV), (dict(dt=2), INV), (dict(d=63), INV), (dict(red=2), INV), (dict(acc=2), INV),
    (dict(K=20000, V=100000), UNS), (dict(V=1 << 22), UNS),
    (dict(H=None), INV), (dict(W=None), INV), (dict(idx=None), INV), (dict(logp=None), INV),
    (dict(lse=None), INV), (dict(loss=None), INV), (dict(grad=None), INV),
    (dict(H=FAKE + 8), INV), (dict(idx=FAKE + 2), INV), (dict(loss_tok=FAKE + 1), INV),
    (dict(loss=FAKE + 2), INV), (dict(grad=FAKE + 2), INV), (dict(dH=FAKE + 8), INV),
    (dict(dW=FAKE + 4), INV), (dict(w=FAKE + 2), INV),
    (dict(ws=None), WSE), (dict(ws=FAKE + 16), WSE), (dict(ws_n=1024), WSE),
])
def test_one_pass_rejects_invalid(L, kw, want):
    assert _fb(L, **kw) == want


def test_launch_grid_limit(L):
    """Every launch holds fewer than 2^24 workgroups of 256 threads (2^32
    work-items): a chunk whose logit tiles (chunk/256 x V/256) reach 2^24 is
    rejected, one just below is accepted; the one-pass streaming pass (a
    workgroup per 8192 stored logits of a row) has its own bound."""
    ws = L.kd_fused_kl_workspace_bytes
    bf = _lib.KD_BF16
    big, below = 1 << 20, (1 << 20) - 256
    for pass_ in (0, 1, 2, 3):
        assert ws(pass_, big, 64, big, 8, big, bf) == 0          # 4096 x 4096 tiles
    for pass_ in (0, 1):
        assert ws(pass_, big, 64, below, 8, big, bf) > 0         # 4096 x 4095 tiles
    # the same chunk with a streaming pass over its stored logits (teacher
    # cache, one-pass call): 2^20 rows x 128 workgroups per row
    assert ws(_lib.KD_PASS_TEACHER, big, 64, below, 8, big, bf) == 0
    assert ws(_lib.KD_PASS_FWD_BWD, big, 64, below, 8, big, bf) == 0
    assert ws(_lib.KD_PASS_FWD_BWD, 1 << 17, 64, below, 8, 1 << 17, bf) == 0  # 2^17 x 128 = 2^24
    assert ws(_lib.KD_PASS_FWD_BWD, 1 << 16, 64, below, 8, 1 << 16, bf) > 0


C_CLIENT = r"""
#include <stdio.h>
#include "kd_fused_kl.h"

int main(void) {
  /* every entry point the header declares, taken by address from C */
  typedef void (*fn_t)(void);
  const fn_t fns[] = {
      (fn_t)kd_status_str, (fn_t)kd_fused_kl_workspace_bytes,
      (fn_t)kd_fused_kl_fwd, (fn_t)kd_fused_kl_bwd,
      (fn_t)kd_fused_kl_fwd_ex, (fn_t)kd_fused_kl_bwd_ex, (fn_t)kd_fused_kl_fwd_noalloc,
      (fn_t)kd_fused_kl_fwd_bwd, (fn_t)kd_teacher_topk,
      (fn_t)kd_fused_kl_check_inputs, (fn_t)kd_cast_f32_to_bf16, (fn_t)kd_scale,
      (fn_t)kd_timing_enable, (fn_t)kd_timing_read};
  for (unsigned i = 0; i < sizeof(fns) / sizeof(fns[0]); ++i)
    if (!fns[i]) return 3;
  size_t ws = kd_fused_kl_workspace_bytes(KD_PASS_FWD_BWD, 8192, 3072, 128256, 100, 1024, KD_BF16);
  int st = kd_fused_kl_fwd(0, 0, KD_F32, 0, 0, -1, 64, 1000, 8, 32, 0, 0, 0, 0, 0, 0);
  printf("%zu %s %d\n", ws, kd_status_str(st), KD_KERNEL_CLASSES);
  return ws > 0 && st == KD_ERR_INVALID_ARG ? 0 : 4;
}
"""


def test_header_is_plain_c(tmp_path):
    """The header compiles as C99 (gcc, no C++), and a C program linked
    against the library calls its host-only entry points."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(_build.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", libdir, "-lkdkl", f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.stdout, run.stderr)
    ws, status, classes = run.stdout.split()
    assert int(ws) == _lib.lib().kd_fused_kl_workspace_bytes(3, 8192, 3072, 128256, 100, 1024, 1)
    assert status == "KD_ERR_INVALID_ARG" and int(classes) == len(_lib.KERNEL_CLASSES)
