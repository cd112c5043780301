"""Plain fp64 oracle of the offline teacher cache: top-K ids and log-probs.

TEST INFRASTRUCTURE ONLY (same rule as kl_oracle.py): imported by ``tests/``
and by the CPU-baseline leg of ``bench.py --workload teacher-cache``, never by
the HIP library or its binding.

Source pages (cited by title and section):

[P1] "Distilação de LLMs mais barata: top-K offline e KL fundida cortam VRAM
     em até 15x", section "As duas mudanças": the teacher runs once, and the
     100 most probable tokens of every position are cached.
[P4] "Hugging Face：让知识蒸馏廉价到可大规模运行", paragraph 离线蒸馏 (the same
     step), and section 为什么蒸馏恢复代价高昂 ("Dense KL" rebuilds the teacher
     grid from the cached top-100).
[P5] "Chunkovaná KL strata umožnila destilovať LLM s 32-tisícovým kontextom
     na jednom H200", section "Čo dopĺňajú podrobnejšie experimenty": the kept
     top-100 is not renormalised.

What is computed, for teacher hidden states Ht [N, d] and the teacher's output
head Wt [V, d], written out with no blocking or reordering:

1. Teacher logits Z = Ht Wtᵀ (fp64).
2. Their log-normaliser over the full vocabulary, lse_r = log Σ_j exp Z_rj.
3. The K most probable tokens of each row: sort the row by logit, largest
   first, equal logits by the lower token id first, and keep the first K ids.
4. Their log-probabilities from the full softmax, logp_rk = Z_r,idx_rk − lse_r
   (not renormalised over the kept K).

Readings: "most probable" ranks by the full-softmax probability, which orders
exactly as the logits do; ties go to the lower id (a deterministic rule the
pages do not state).
"""
from __future__ import annotations

import numpy as np

from .kl_oracle import to_f64

__all__ = ["teacher_logits", "teacher_topk_reference"]


def teacher_logits(Ht, Wt) -> tuple:
    """(Z, lse) in float64 for Ht [N, d] and Wt [V, d]."""
    Z = to_f64(Ht) @ to_f64(Wt).T
    m = Z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(Z - m).sum(axis=1))
    return Z, lse


def teacher_topk_reference(Ht, Wt, K: int) -> dict:
    """Top-K cache of each row: idx int32 [N, K], logp [N, K], lse [N], and
    the logits Z [N, V] (for checking near-ties)."""
    Z, lse = teacher_logits(Ht, Wt)
    N, V = Z.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    idx = np.empty((N, K), dtype=np.int32)
    for r in range(N):
        # Largest logit first; among equal logits the lower id first.
        order = sorted(range(V), key=lambda j: (-Z[r, j], j)) if V <= 64 else \
            np.lexsort((np.arange(V), -Z[r]))
        idx[r] = np.asarray(order[:K], dtype=np.int32)
    logp = np.take_along_axis(Z, idx.astype(np.int64), axis=1) - lse[:, None]
    return {"idx": idx, "logp": logp, "lse": lse, "Z": Z}
