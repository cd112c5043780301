"""Seeded synthetic workloads for the fused, chunked top-K KL distillation loss.

This module only draws inputs. It is shared by the CPU oracle's tests, the GPU
parity tests, ``bench.py`` and ``__graft_entry__.smoke()``; it holds none of
the student-side loss arithmetic and imports neither ``oracle`` nor the HIP
package.

What the inputs stand for (source pages, cited by title and section):

* [P4] "Hugging Face：让知识蒸馏廉价到可大规模运行" (feinterview.poetries.top),
  section 离线蒸馏 and section 为什么蒸馏恢复代价高昂: the teacher runs once,
  and the 100 most probable tokens of every position are cached.
* [P5] "Chunkovaná KL strata umožnila destilovať LLM s 32-tisícovým kontextom
  na jednom H200" (aifeed.sk), section "Dva odlišné zdroje úspory": the cache
  holds the top-100 tokens and their values; section "Čo dopĺňajú podrobnejšie
  experimenty": the cut distribution is not renormalised.
* [P4] section 扩展到长上下文 and [P5] the same section: the isolated loss
  benchmark is a toy output-projection network with no backbone, so hidden
  states are synthetic.

The teacher "cache" here is produced the way such a cache is produced: a
seeded random teacher head W_t projects the same hidden states, a full softmax
over the vocabulary is taken in fp32, and the top-K token ids (int32) and their
log-probabilities (fp32) are kept without renormalisation. Ties in top-K are
measure-zero for continuous draws; the loss is invariant to the order of the K
columns, and both sides of every comparison receive the same cache.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "config", "make_inputs", "cache_digest", "teacher_head_inputs"]


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload shape. ``dtype`` is the dtype of H and W."""

    cid: int
    name: str
    N: int
    d: int
    V: int
    K: int
    chunk: int
    dtype: str  # "f32" or "bf16"

    def with_n(self, N: int) -> "Config":
        return dataclasses.replace(self, N=N)


# The five workloads: a tiny fp32 case the oracle finishes instantly, a small
# bf16 case, a 3.2B-student head at 8K context, the isolated long-context
# loss-kernel sweep (32K .. 256K tokens), and a gpt-oss style 201,088-token
# vocabulary head.
CONFIGS = {
    1: Config(1, "tiny-fp32", 128, 64, 1000, 8, 32, "f32"),
    2: Config(2, "small-bf16", 1024, 512, 32000, 100, 256, "bf16"),
    3: Config(3, "llama3.2b-head-8k", 8192, 3072, 128256, 100, 1024, "bf16"),
    4: Config(4, "long-context-sweep", 32768, 3072, 128256, 100, 2048, "bf16"),
    5: Config(5, "gpt-oss-head-32k", 32768, 2880, 201088, 100, 2048, "bf16"),
}
SWEEP_N = (32768, 65536, 131072, 262144)


def config(cid: int, N: Optional[int] = None) -> Config:
    c = CONFIGS[cid]
    return c.with_n(N) if N is not None else c


def _seeds(cfg: Config):
    # Config 4 is one config id over four token counts; each point gets its
    # own seeds so the four caches are independent draws.
    cid = cfg.cid + (cfg.N // 32768 if cfg.cid == 4 else 0)
    return 1000 + cid, 2000 + cid, 3000 + cid


def _normal(shape, std, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32) * std


def teacher_topk(H32: torch.Tensor, Wt: torch.Tensor, K: int,
                 device: str = "cpu", rows_per_block: int = 1024):
    """Top-K ids and log-probs of a random teacher head, no renormalisation.

    Row-blocked so that the full [N, V] teacher grid never exists at once.
    Returns CPU tensors: idx int32 [N, K], logp float32 [N, K].
    """
    N = H32.shape[0]
    Wt_dev = Wt.to(device)
    idx_out = torch.empty((N, K), dtype=torch.int32)
    logp_out = torch.empty((N, K), dtype=torch.float32)
    for r0 in range(0, N, rows_per_block):
        r1 = min(N, r0 + rows_per_block)
        logits = H32[r0:r1].to(device) @ Wt_dev.T
        logprobs = torch.log_softmax(logits, dim=1)
        vals, ids = torch.topk(logprobs, K, dim=1, largest=True, sorted=True)
        idx_out[r0:r1] = ids.to(torch.int32).cpu()
        logp_out[r0:r1] = vals.cpu()
        del logits, logprobs, vals, ids
    return idx_out, logp_out


def make_inputs(cfg: Config, teacher_device: str = "cpu"):
    """Draw (H, W, idx, logp) for ``cfg`` on the CPU.

    H ~ N(0, 1), W ~ N(0, 1/d), teacher head W_t ~ N(0, 4/d) (discarded after
    use). bf16 workloads round H and W to bfloat16 (round-to-nearest-even) and
    the teacher projects the rounded H. ``teacher_device`` only says where the
    teacher projection runs; the returned tensors are always on the CPU.
    """
    sH, sW, sT = _seeds(cfg)
    H = _normal((cfg.N, cfg.d), 1.0, sH)
    W = _normal((cfg.V, cfg.d), cfg.d ** -0.5, sW)
    if cfg.dtype == "bf16":
        H = H.to(torch.bfloat16)
        W = W.to(torch.bfloat16)
    elif cfg.dtype != "f32":
        raise ValueError(f"unknown dtype {cfg.dtype}")
    Wt = _normal((cfg.V, cfg.d), 2.0 * cfg.d ** -0.5, sT)
    idx, logp = teacher_topk(H.float(), Wt, cfg.K, device=teacher_device)
    del Wt
    return H.contiguous(), W.contiguous(), idx.contiguous(), logp.contiguous()


def cache_digest(idx: torch.Tensor, logp: torch.Tensor) -> str:
    """SHA-256 of a teacher cache, to record which draw a run used."""
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(idx.numpy()).tobytes())
    h.update(np.ascontiguousarray(logp.numpy()).tobytes())
    return h.hexdigest()


def teacher_head_inputs(N: int = 8192, d: int = 4096, V: int = 128256, seed: int = 4000):
    """Teacher-side inputs of the offline cache step: final hidden states
    Ht ~ N(0, 1) [N, d] and an output head Wt ~ N(0, 4/d) [V, d] (teacher
    logits with std ≈ 2), both rounded to bf16, on the CPU. The default shape
    is an 8B-class teacher head (d = 4096, the Llama 3 vocabulary of 128,256)
    over 8K positions, the pages' 8K distillation setting."""
    Ht = _normal((N, d), 1.0, seed).to(torch.bfloat16)
    Wt = _normal((V, d), 2.0 * d ** -0.5, seed + 1).to(torch.bfloat16)
    return Ht.contiguous(), Wt.contiguous()
