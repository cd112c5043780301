"""Python face of the fused, chunked top-K KL loss (thin layer over the C ABI).

PyTorch supplies device memory and the current stream; every step of the loss
runs in the HIP kernels of libkdkl.so. Functions here check shapes and dtypes,
allocate outputs and the workspace with torch, and call the library.

    loss = fused_kl(H, W, topk_idx, topk_logp, chunk=1024)   # autograd-aware
    loss.backward()                                           # dH, dW via HIP

Source: the fused, chunked KL loss of "Hugging Face：让知识蒸馏廉价到可大规模运行"
(section 为什么蒸馏恢复代价高昂, "Fused chunked KL" paragraph), fed by the
offline top-K teacher cache of the same page (section 离线蒸馏).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_DT = {torch.float32: _lib.KD_F32, torch.bfloat16: _lib.KD_BF16}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"H and W must be float32 or bfloat16, got {dt}")
    return _DT[dt]


def workspace_bytes(pass_: int, N: int, d: int, V: int, K: int, chunk: int, dt: torch.dtype) -> int:
    n = _lib.lib().kd_fused_kl_workspace_bytes(int(pass_), N, d, V, K, chunk, dtype_code(dt))
    if n == 0:
        raise ValueError(f"invalid sizes N={N} d={d} V={V} K={K} chunk={chunk} dtype={dt}")
    return int(n)


def _check_inputs(H, W, idx, logp):
    if not (H.is_cuda and W.is_cuda and idx.is_cuda and logp.is_cuda):
        raise ValueError("all inputs must be on the GPU")
    if H.dim() != 2 or W.dim() != 2 or idx.dim() != 2 or logp.dim() != 2:
        raise ValueError("H [N,d], W [V,d], idx [N,K], logp [N,K] expected")
    N, d = H.shape
    V, d2 = W.shape
    if d2 != d or idx.shape != logp.shape or idx.shape[0] != N:
        raise ValueError(f"shape mismatch: H {tuple(H.shape)} W {tuple(W.shape)} "
                         f"idx {tuple(idx.shape)} logp {tuple(logp.shape)}")
    if H.dtype != W.dtype:
        raise TypeError("H and W must share a dtype")
    if idx.dtype != torch.int32 or logp.dtype != torch.float32:
        raise TypeError("topk_idx must be int32 and topk_logp float32")
    for t in (H, W, idx, logp):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    return N, d, V, idx.shape[1]


_RED = {"sum": _lib.KD_REDUCE_SUM, "mean": _lib.KD_REDUCE_MEAN}


def _reduction(reduction: str) -> int:
    if reduction not in _RED:
        raise ValueError(f"reduction must be 'sum' or 'mean', got {reduction!r}")
    return _RED[reduction]


def _check_weight(weight: Optional[torch.Tensor], N: int, dev: torch.device):
    if weight is None:
        return None
    if (weight.shape != (N,) or weight.dtype != torch.float32 or not weight.is_contiguous()
            or weight.device != dev):
        raise ValueError("weight must be a contiguous fp32 [N] tensor on the inputs' device")
    return weight


def kl_forward(H: torch.Tensor, W: torch.Tensor, idx: torch.Tensor, logp: torch.Tensor,
               chunk: int, want_loss_tok: bool = True, weight: Optional[torch.Tensor] = None,
               reduction: str = "sum"
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor], torch.Tensor]:
    """Returns (loss [1] fp32, loss_tok [N] fp32 or None, lse [N] fp32).

    ``loss`` is Σ_r w_r L_r ('sum') or that divided by Σ_r w_r ('mean'), with
    w_r = 1 when ``weight`` is None; ``loss_tok`` holds the unweighted L_r.
    """
    N, d, V, K = _check_inputs(H, W, idx, logp)
    dev = H.device
    dt = dtype_code(H.dtype)
    red = _reduction(reduction)
    weight = _check_weight(weight, N, dev)
    ws_n = workspace_bytes(_lib.KD_PASS_FWD, N, d, V, K, chunk, H.dtype)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    loss_sum = torch.empty(1, dtype=torch.float32, device=dev)
    loss_tok = torch.empty(N, dtype=torch.float32, device=dev) if want_loss_tok else None
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    st = _lib.lib().kd_fused_kl_fwd_ex(_p(H), _p(W), dt, _p(idx), _p(logp), _p(weight), red, N, d,
                                        V, K, chunk, _p(loss_tok), _p(lse), _p(loss_sum), _p(ws),
                                        ws_n, _stream(dev))
    _lib.check("kd_fused_kl_fwd_ex", st)
    return loss_sum, loss_tok, lse


def kl_forward_noalloc(H: torch.Tensor, W: torch.Tensor, idx: torch.Tensor,
                       logp: torch.Tensor, chunk: int, loss: torch.Tensor,
                       lse: torch.Tensor, loss_tok: Optional[torch.Tensor] = None,
                       weight: Optional[torch.Tensor] = None, reduction: str = "sum") -> None:
    """kd_fused_kl_fwd_noalloc: the forward pass into caller-provided outputs,
    with the library's own scratch instead of a workspace. Nothing is
    allocated here or in the library: ``loss`` ([1] fp32), ``lse`` ([N] fp32)
    and ``loss_tok`` ([N] fp32 or None) are written on the current stream.
    Sizes whose forward workspace exceeds KD_NOALLOC_SCRATCH_BYTES raise."""
    N, d, V, K = _check_inputs(H, W, idx, logp)
    dev = H.device
    dt = dtype_code(H.dtype)
    red = _reduction(reduction)
    weight = _check_weight(weight, N, dev)
    for name, t, n in (("loss", loss, 1), ("lse", lse, N), ("loss_tok", loss_tok, N)):
        if t is None and name == "loss_tok":
            continue
        if (t.shape != (n,) or t.dtype != torch.float32 or not t.is_contiguous()
                or t.device != dev):
            raise ValueError(f"{name} must be a contiguous fp32 [{n}] tensor on the inputs' device")
    st = _lib.lib().kd_fused_kl_fwd_noalloc(_p(H), _p(W), dt, _p(idx), _p(logp), _p(weight), red,
                                             N, d, V, K, chunk, _p(loss_tok), _p(lse), _p(loss),
                                             _stream(dev))
    _lib.check("kd_fused_kl_fwd_noalloc", st)


def kl_backward(H: torch.Tensor, W: torch.Tensor, idx: torch.Tensor, logp: torch.Tensor,
                lse: torch.Tensor, grad: torch.Tensor, chunk: int, need_dH: bool = True,
                need_dW: bool = True, dW_out: Optional[torch.Tensor] = None,
                accumulate: bool = False, weight: Optional[torch.Tensor] = None,
                reduction: str = "sum") -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Returns (dH [N,d] in H's dtype or None, dW [V,d] fp32 or None).

    ``grad`` is a 1-element fp32 device tensor: ∂objective/∂loss.
    ``dW_out`` (fp32 [V,d]) is written, or added to when ``accumulate``.
    ``weight`` and ``reduction`` must be those of the forward call.
    """
    N, d, V, K = _check_inputs(H, W, idx, logp)
    dev = H.device
    red = _reduction(reduction)
    weight = _check_weight(weight, N, dev)
    if lse.shape != (N,) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [N] tensor from kl_forward")
    grad = grad.reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    dt = dtype_code(H.dtype)
    ws_n = workspace_bytes(_lib.KD_PASS_BWD, N, d, V, K, chunk, H.dtype)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    dH = torch.empty((N, d), dtype=H.dtype, device=dev) if need_dH else None
    dW = None
    if need_dW:
        if dW_out is not None:
            if dW_out.shape != (V, d) or dW_out.dtype != torch.float32 or not dW_out.is_contiguous():
                raise ValueError("dW_out must be a contiguous fp32 [V,d] tensor")
            dW = dW_out
        else:
            dW = torch.empty((V, d), dtype=torch.float32, device=dev)
            accumulate = False
    st = _lib.lib().kd_fused_kl_bwd_ex(_p(H), _p(W), dt, _p(idx), _p(logp), _p(weight), red,
                                        _p(lse), N, d, V, K, chunk, _p(grad), _p(dH), _p(dW),
                                        1 if accumulate else 0, _p(ws), ws_n, _stream(dev))
    _lib.check("kd_fused_kl_bwd_ex", st)
    return dH, dW


def kl_forward_backward(H: torch.Tensor, W: torch.Tensor, idx: torch.Tensor,
                        logp: torch.Tensor, chunk: int, grad: Optional[torch.Tensor] = None,
                        want_loss_tok: bool = True, need_dH: bool = True, need_dW: bool = True,
                        dW_out: Optional[torch.Tensor] = None, accumulate: bool = False,
                        weight: Optional[torch.Tensor] = None, reduction: str = "sum"):
    """Loss and gradients in one call (kd_fused_kl_fwd_bwd): each chunk's
    logits are projected once and kept only until its dlogits are formed.

    Returns (loss [1], loss_tok [N] or None, lse [N], dH or None, dW or None),
    the results of kl_forward followed by kl_backward with the same
    arguments. ``grad`` (∂objective/∂loss, a 1-element fp32 tensor) defaults
    to 1.
    """
    N, d, V, K = _check_inputs(H, W, idx, logp)
    dev = H.device
    dt = dtype_code(H.dtype)
    red = _reduction(reduction)
    weight = _check_weight(weight, N, dev)
    if grad is None:
        grad = torch.ones(1, dtype=torch.float32, device=dev)
    grad = grad.reshape(1).to(device=dev, dtype=torch.float32).contiguous()
    ws_n = workspace_bytes(_lib.KD_PASS_FWD_BWD, N, d, V, K, chunk, H.dtype)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    loss_tok = torch.empty(N, dtype=torch.float32, device=dev) if want_loss_tok else None
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    dH = torch.empty((N, d), dtype=H.dtype, device=dev) if need_dH else None
    dW = None
    if need_dW:
        if dW_out is not None:
            if dW_out.shape != (V, d) or dW_out.dtype != torch.float32 or not dW_out.is_contiguous():
                raise ValueError("dW_out must be a contiguous fp32 [V,d] tensor")
            dW = dW_out
        else:
            dW = torch.empty((V, d), dtype=torch.float32, device=dev)
            accumulate = False
    st = _lib.lib().kd_fused_kl_fwd_bwd(_p(H), _p(W), dt, _p(idx), _p(logp), _p(weight), red, N,
                                         d, V, K, chunk, _p(grad), _p(loss_tok), _p(lse),
                                         _p(loss), _p(dH), _p(dW), 1 if accumulate else 0, _p(ws),
                                         ws_n, _stream(dev))
    _lib.check("kd_fused_kl_fwd_bwd", st)
    return loss, loss_tok, lse, dH, dW


def teacher_topk(Ht: torch.Tensor, Wt: torch.Tensor, K: int, chunk: int = 1024
                 ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Offline teacher cache of every row: (topk_idx int32 [N,K], topk_logp
    fp32 [N,K], lse fp32 [N]); ids by logit, largest first (ties: lower id
    first), log-probabilities under the full softmax, not renormalised."""
    if not (Ht.is_cuda and Wt.is_cuda):
        raise ValueError("inputs must be on the GPU")
    if Ht.dim() != 2 or Wt.dim() != 2 or Ht.shape[1] != Wt.shape[1]:
        raise ValueError(f"Ht [N,d] and Wt [V,d] expected, got {tuple(Ht.shape)} {tuple(Wt.shape)}")
    if Ht.dtype != Wt.dtype:
        raise TypeError("Ht and Wt must share a dtype")
    if not (Ht.is_contiguous() and Wt.is_contiguous()):
        raise ValueError("inputs must be contiguous")
    N, d = Ht.shape
    V = Wt.shape[0]
    dev = Ht.device
    ws_n = workspace_bytes(_lib.KD_PASS_TEACHER, N, d, V, K, chunk, Ht.dtype)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    idx = torch.empty((N, K), dtype=torch.int32, device=dev)
    logp = torch.empty((N, K), dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    st = _lib.lib().kd_teacher_topk(_p(Ht), _p(Wt), dtype_code(Ht.dtype), N, d, V, K, chunk,
                                     _p(idx), _p(logp), _p(lse), _p(ws), ws_n, _stream(dev))
    _lib.check("kd_teacher_topk", st)
    return idx, logp, lse


def check_inputs(topk_idx: torch.Tensor, topk_logp: torch.Tensor, V: int) -> list:
    """Debug check of the cache's preconditions on the GPU (ids in [0, V) and
    distinct per row, log-probs <= 0 or -inf). Returns the names of the
    violated ones (empty if all hold); synchronises the stream to read them."""
    if not (topk_idx.is_cuda and topk_logp.is_cuda):
        raise ValueError("inputs must be on the GPU")
    if topk_idx.dim() != 2 or topk_idx.shape != topk_logp.shape:
        raise ValueError("topk_idx and topk_logp must both be [N, K]")
    if topk_idx.dtype != torch.int32 or topk_logp.dtype != torch.float32:
        raise TypeError("topk_idx must be int32 and topk_logp float32")
    if not (topk_idx.is_contiguous() and topk_logp.is_contiguous()):
        raise ValueError("inputs must be contiguous")
    N, K = topk_idx.shape
    dev = topk_idx.device
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    st = _lib.lib().kd_fused_kl_check_inputs(_p(topk_idx), _p(topk_logp), N, K, int(V),
                                              _p(flags), _stream(dev))
    _lib.check("kd_fused_kl_check_inputs", st)
    f = int(flags.item())
    names = [(_lib.KD_CHECK_ID_RANGE, "id out of range"), (_lib.KD_CHECK_DUPLICATE, "duplicate id"),
             (_lib.KD_CHECK_LOGP, "log-prob > 0 or NaN")]
    return [n for bit, n in names if f & bit]


def cast_f32_to_bf16(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (round to nearest even) in a HIP kernel."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("expected a contiguous fp32 GPU tensor")
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    st = _lib.lib().kd_cast_f32_to_bf16(_p(x), _p(out), x.numel(), _stream(x.device))
    _lib.check("kd_cast_f32_to_bf16", st)
    return out


def scale_(x: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """x *= s in place on the GPU (x fp32 or bf16, s a 1-element fp32 device
    tensor); nothing but a launch when s == 1."""
    if not (x.is_cuda and x.is_contiguous()):
        raise ValueError("expected a contiguous GPU tensor")
    s = s.reshape(1).to(device=x.device, dtype=torch.float32).contiguous()
    st = _lib.lib().kd_scale(_p(x), dtype_code(x.dtype), x.numel(), _p(s), _stream(x.device))
    _lib.check("kd_scale", st)
    return x


class FusedTopKKL(torch.autograd.Function):
    """Σ over positions of w_r · KL(teacher top-K ‖ student softmax(H Wᵀ)), or
    its weighted mean.

    Two-pass (default): saves only lse [N] between the passes; the backward
    pass recomputes the logits chunk by chunk. One-pass: the forward computes
    the loss and the gradients at an upstream gradient of 1 in one call
    (each chunk projected once) and keeps dH and dW; the backward scales them
    by the upstream gradient (a no-op launch when it is 1). A second backward
    through the same graph is then refused, since the kept gradients were
    scaled in place by the first.
    """

    @staticmethod
    def forward(ctx, H, W, idx, logp, chunk, weight, reduction, one_pass):
        need_dH, need_dW = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        ctx.one_pass = bool(one_pass) and (need_dH or need_dW)
        if ctx.one_pass:
            loss, _, _, dH, dW = kl_forward_backward(
                H, W, idx, logp, chunk, want_loss_tok=False, need_dH=need_dH, need_dW=need_dW,
                weight=weight, reduction=reduction)
            ctx.save_for_backward(dH, dW)
            ctx.w_dtype = W.dtype
            ctx.spent = False
            return loss.reshape(())
        loss, _, lse = kl_forward(H, W, idx, logp, chunk, want_loss_tok=False, weight=weight,
                                  reduction=reduction)
        ctx.save_for_backward(H, W, idx, logp, lse, weight)
        ctx.chunk = chunk
        ctx.reduction = reduction
        return loss.reshape(())

    @staticmethod
    def backward(ctx, grad):
        if ctx.one_pass:
            if ctx.spent:
                raise RuntimeError("fused_kl(one_pass=True) supports one backward per forward")
            ctx.spent = True
            dH, dW = ctx.saved_tensors
            g = grad.reshape(1).to(dtype=torch.float32).contiguous()
            if dH is not None:
                scale_(dH, g)
            if dW is not None:
                scale_(dW, g)
                if ctx.w_dtype == torch.bfloat16:
                    dW = cast_f32_to_bf16(dW)
            return dH, dW, None, None, None, None, None, None
        H, W, idx, logp, lse, weight = ctx.saved_tensors
        need_dH, need_dW = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dH, dW = kl_backward(H, W, idx, logp, lse, grad, ctx.chunk, need_dH=need_dH,
                             need_dW=need_dW, weight=weight, reduction=ctx.reduction)
        if dW is not None and W.dtype == torch.bfloat16:
            dW = cast_f32_to_bf16(dW)
        return dH, dW, None, None, None, None, None, None


def fused_kl(H: torch.Tensor, W: torch.Tensor, topk_idx: torch.Tensor, topk_logp: torch.Tensor,
             chunk: int = 1024, weight: Optional[torch.Tensor] = None,
             reduction: str = "sum", one_pass: bool = False) -> torch.Tensor:
    """Top-K KL distillation loss, summed (or averaged with ``reduction='mean'``)
    over positions with optional per-position ``weight`` (fp32 [N], e.g. a
    0/1 mask for packed sequences); differentiable in H and W.

    ``one_pass=True`` computes the gradients during the forward, projecting
    each chunk once instead of twice (about 25% less time for forward plus
    backward), and holds dH and dW until the backward."""
    _reduction(reduction)
    return FusedTopKKL.apply(H, W, topk_idx, topk_logp, int(chunk), weight, reduction,
                             bool(one_pass))
