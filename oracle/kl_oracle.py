"""Plain, slow, dense fp64 oracle of the top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` (which also compares the result of
its sample with the GPU outputs of the same rows); never by the HIP library
or its binding. It shares no code, table or helper with the GPU path.

Source pages (cited by title and section):

[P1] "Distilação de LLMs mais barata: top-K offline e KL fundida cortam VRAM
     em até 15x" (imasters.com.br)
[P4] "Hugging Face：让知识蒸馏廉价到可大规模运行" (feinterview.poetries.top,
     a translation of the Hugging Face blog post "Making Knowledge
     Distillation Cheap Enough to Run at Scale")
[P5] "Chunkovaná KL strata umožnila destilovať LLM s 32-tisícovým kontextom
     na jednom H200" (aifeed.sk)

What is computed. The three loss variants of [P4, section
为什么蒸馏恢复代价高昂] are stated to be mathematically equivalent, and the
dense one is the authors' correctness baseline, so this oracle IS the dense
variant written out, in float64, with no blocking, fusion or reordering:

1. Student logits Z = H Wᵀ over the full vocabulary: the output projection is
   part of the loss [P4, same section, "Fused chunked KL" paragraph].
2. Student log-probabilities by an explicit, max-shifted softmax over all V
   columns: log q = Z − lse, lse_r = m_r + log Σ_j exp(Z_rj − m_r).
3. Dense teacher-probability grid rebuilt from the cached top-K
   [P4, "Dense KL" paragraph]: P = 0 everywhere, P[r, idx_rk] = exp(logp_rk),
   with no renormalisation of the cut distribution [P5, section
   "Čo dopĺňajú podrobnejšie experimenty"].
4. Forward KL per position, L_r = Σ_j P_rj (log P_rj − log q_rj) with
   0·log 0 = 0, summed over positions into one accumulated loss
   [P1, section "As duas mudanças"; P4 "Fused chunked KL" paragraph].
5. Gradient. The pages name a closed-form gradient but do not print it
   [P4, section 得到的 student]. Writing L_r = Σ_j P_rj log P_rj −
   Σ_j P_rj (Z_rj − lse_r) and using ∂lse_r/∂Z_rj = q_rj gives
   ∂L_r/∂Z_rj = (Σ_j' P_rj') q_rj − P_rj. With an upstream scalar g,
   G = g (q ⊙ rowsum(P) − P), dH = G W and dW = Gᵀ H.

Readings where the pages are silent: the KL direction is KL(teacher ‖
student); the temperature is 1; positions are flattened to N rows; the loss
is a SUM over rows (a mean is the caller's g = 1/N); indices in a row must be
distinct and inside [0, V); a cached log-prob of −inf contributes nothing.

Per-token weights and the mean reduction. The pages mention sequence packing
only as an ablation [P4, section 得到的 student]; packing needs per-position
weights or masks. Reading: with weights w_r the accumulated loss is
Σ_r w_r L_r, and the mean reduction divides it by Σ_r w_r (by N when no
weights are given; a zero total weight gives a zero loss). The per-position
losses L_r themselves stay unweighted. The gradient follows by the chain rule:
G_r = g (w_r / den) (q_r rowsum(P)_r − P_r), with den = Σ_r w_r (mean) or 1
(sum).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "reduction_weights",
    "to_f64",
    "teacher_grid",
    "student_log_softmax",
    "kl_rows",
    "kl_grad_logits",
    "fused_kl_reference",
    "rows_reference",
]


def to_f64(x) -> np.ndarray:
    """Exact upcast to float64 of a numpy array or a CPU torch tensor.

    bfloat16 and float32 values are representable exactly in float64.
    """
    if hasattr(x, "detach"):  # torch tensor, without importing torch here
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _as_index(idx) -> np.ndarray:
    if hasattr(idx, "detach"):
        idx = idx.detach().cpu().numpy()
    return np.asarray(idx, dtype=np.int64)


def teacher_grid(idx, logp, V: int) -> np.ndarray:
    """Dense teacher grid P[N, V] from the top-K cache, not renormalised.

    [P4, 为什么蒸馏恢复代价高昂, "Dense KL" paragraph]; [P5, "Čo dopĺňajú
    podrobnejšie experimenty"]: the kept top-K mass sums to less than one.
    """
    idx = _as_index(idx)
    logp = to_f64(logp)
    if idx.shape != logp.shape or idx.ndim != 2:
        raise ValueError("idx and logp must both be [N, K]")
    N, K = idx.shape
    if K > 0:
        if idx.min() < 0 or idx.max() >= V:
            raise ValueError("teacher index out of [0, V)")
        srt = np.sort(idx, axis=1)
        if np.any(srt[:, 1:] == srt[:, :-1]):
            raise ValueError("teacher indices must be distinct within a row")
    P = np.zeros((N, V), dtype=np.float64)
    rows = np.repeat(np.arange(N), K)
    P[rows, idx.reshape(-1)] = np.exp(logp.reshape(-1))
    return P


def student_log_softmax(H, W):
    """Z = H Wᵀ and its explicit softmax over the full vocabulary.

    Returns (Z, lse, logq), all float64.
    """
    H = to_f64(H)
    W = to_f64(W)
    Z = H @ W.T
    m = Z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(Z - m).sum(axis=1))
    logq = Z - lse[:, None]
    return Z, lse, logq


def kl_rows(P: np.ndarray, logq: np.ndarray) -> np.ndarray:
    """L_r = Σ_j P_rj (log P_rj − log q_rj), taking 0·log 0 = 0."""
    pos = P > 0
    logP = np.log(np.where(pos, P, 1.0))
    terms = np.where(pos, P * (logP - logq), 0.0)
    return terms.sum(axis=1)


def kl_grad_logits(P: np.ndarray, logq: np.ndarray, grad: float = 1.0) -> np.ndarray:
    """∂(g·Σ_r L_r)/∂Z = g (q ⊙ rowsum(P) − P), dense [N, V]."""
    q = np.exp(logq)
    return float(grad) * (q * P.sum(axis=1, keepdims=True) - P)


def reduction_weights(N: int, weight=None, reduction: str = "sum") -> np.ndarray:
    """Per-row factor c_r of the accumulated loss Σ_r c_r L_r.

    sum: c_r = w_r (1 without weights). mean: c_r = w_r / Σ_r' w_r' (1/N
    without weights), and c = 0 when the total weight is 0.
    """
    if reduction not in ("sum", "mean"):
        raise ValueError("reduction must be 'sum' or 'mean'")
    w = np.ones(N) if weight is None else to_f64(weight).reshape(-1)
    if w.shape[0] != N:
        raise ValueError("weight must have one entry per row")
    if reduction == "sum":
        return w
    den = w.sum()
    return w / den if den != 0 else np.zeros(N)


def fused_kl_reference(H, W, idx, logp, grad: float = 1.0, weight=None,
                       reduction: str = "sum") -> dict:
    """Dense forward + backward of the top-K KL loss, all in float64.

    Inputs: H [N, d], W [V, d] (any float dtype; upcast exactly), idx int
    [N, K], logp [N, K], the upstream scalar ``grad`` = ∂objective/∂loss,
    optional per-row ``weight`` [N] and ``reduction`` ('sum' or 'mean').
    Returns loss_tok [N] (unweighted), loss (the reduced total), lse [N],
    dlogits [N, V], dH [N, d], dW [V, d].
    """
    H = to_f64(H)
    W = to_f64(W)
    V = W.shape[0]
    P = teacher_grid(idx, logp, V)
    _, lse, logq = student_log_softmax(H, W)
    loss_tok = kl_rows(P, logq)
    c = reduction_weights(H.shape[0], weight, reduction)
    G = kl_grad_logits(P, logq, grad) * c[:, None]
    dH = G @ W
    dW = G.T @ H
    return {
        "loss_tok": loss_tok,
        "loss": float((c * loss_tok).sum()),
        "lse": lse,
        "dlogits": G,
        "dH": dH,
        "dW": dW,
    }


def rows_reference(H, W, idx, logp, rows, grad: float = 1.0, with_dh: bool = True) -> dict:
    """The same definition evaluated on a subset of rows.

    Every quantity except dW depends on its own row only, so loss_tok, lse,
    dlogits and dH of the selected rows can be checked one by one at sizes
    where the full dense grid would not fit; dW is the sum over row blocks of
    dlogitsᵀ H. ``W`` may be passed already upcast (a float64 array) to avoid
    repeating the conversion; ``with_dh=False`` skips the dH product.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Hs = to_f64(H[rows] if not hasattr(H, "detach") else H[rows.tolist()])
    W64 = W if (isinstance(W, np.ndarray) and W.dtype == np.float64) else to_f64(W)
    idx_s = _as_index(idx)[rows]
    logp_s = to_f64(logp)[rows]
    V = W64.shape[0]
    P = teacher_grid(idx_s, logp_s, V)
    _, lse, logq = student_log_softmax(Hs, W64)
    loss_tok = kl_rows(P, logq)
    G = kl_grad_logits(P, logq, grad)
    out = {"rows": rows, "loss_tok": loss_tok, "lse": lse, "dlogits": G}
    if with_dh:
        out["dH"] = G @ W64
    return out
