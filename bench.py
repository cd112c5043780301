#!/usr/bin/env python
"""Throughput of the fused, chunked top-K KL loss (forward + backward) on one MI355X.

One step = one forward and one backward pass of the whole loss over one batch
of synthetic input: the 3.2B-student output head at 8K context (N=8192 tokens,
d=3072, V=128,256, K=100, chunk=1024, bf16 H/W, fp32 teacher log-probs). That
is the workload the ≥60%-of-bf16-MFMA-peak target is stated for; inputs are
resident in HBM before the timed region starts.

Prints ONE JSON line. Besides tokens/s it reports hardware TFLOP/s (8·N·d·V
per step: forward projection, backward recompute, dH and dW), the pages'
convention (6·N·d·V, recompute not counted), peak HBM, a roofline entry for the
dominant kernel measured live with HIP events on the launch stream, and the
CPU oracle timed on a bounded sample of the same workload. The oracle's result
on that sample is also compared with the GPU outputs of the same rows
(``oracle_check``: per-token loss, lse and dH at the stated tolerances).

    python bench.py [--steps K] [--warmup W] [--workload 8k-head|gpt-oss-head|sweep|small|teacher-cache]

``--workload teacher-cache`` times the offline teacher cache step instead
(top-K ids and log-probs through an 8B-class teacher head) and prints its own
line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3
WORKLOADS = {"small": (2, None), "8k-head": (3, None), "gpt-oss-head": (5, None)}

# The pages' own figures, measured on an NVIDIA H200 with PyTorch: context
# only, never a baseline for this line (other hardware; the 8K rows are whole
# training steps of a 3.2B student, and the isolated-loss rows use a toy head
# whose d, V, K and dtype the pages do not state). Sources: the results table
# of "Destilación de LLMs: Multiverse Computing reduce memoria 15× con 1 GPU"
# (section "Resultados concretos") and the long-context paragraphs of
# "Hugging Face：让知识蒸馏廉价到可大规模运行" (section 扩展到长上下文).
PAGES_CONTEXT_8K = {
    "hardware": "1x NVIDIA H200 (pages' figures; context only)",
    "what": "whole training step at 8K context, 3.2B student, Llama 3.1 8B teacher",
    "tflops_pages_convention": {"online KD": 237, "offline dense KL": 331,
                                "offline forward-chunked KL": 335, "offline fused chunked KL": 304},
    "peak_memory_gb": {"online KD": 102.8, "offline dense KL": 78.3,
                       "offline forward-chunked KL": 61.8, "offline fused chunked KL": 58.3},
}
PAGES_CONTEXT_SWEEP = {
    32768: {"hardware": "H200 (pages' figures; context only)", "what": "isolated loss, toy head",
            "peak_memory_gib": {"fused chunked": 5.45, "dense": 85.2}},
    262144: {"hardware": "H200 (pages' figures; context only)", "what": "isolated loss, toy head",
             "peak_memory_gib": {"fused chunked": 11.6, "next best (chunked)": 134.2},
             "speed": "fused about 3.3x faster per iteration than the next best"},
}


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _gen(cfg, dev):
    import workload

    _log(f"generating {cfg.name} N={cfg.N} d={cfg.d} V={cfg.V} K={cfg.K}")
    H, W, idx, logp = workload.make_inputs(cfg, teacher_device=str(dev))
    return H.to(dev), W.to(dev), idx.to(dev), logp.to(dev), workload.cache_digest(idx, logp)


def _kernel_stats(kd_lib):
    from chunked_kl_loss_chunk_amd import _lib

    n = len(_lib.KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _lib.check("kd_timing_read", kd_lib.kd_timing_read(ms, cnt))
    return {c: {"total_ms": ms[i], "launches": cnt[i]} for i, c in enumerate(_lib.KERNEL_CLASSES)}


TRAFFIC_WORKLOAD = "llama3.2b-head-8k"  # the workload profiles/hbm_traffic.md was taken on


def source_sha256() -> str:
    """sha-256 over the kernel sources (the files of csrc, in sorted order):
    names the kernel version a bench line or a profile was taken on."""
    import hashlib

    src = os.path.join(ROOT, "chunked_kl_loss_chunk_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(src)):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic(kernel: str, workload_name: str = TRAFFIC_WORKLOAD):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this workload and on the current kernel source; else None."""
    if workload_name != TRAFFIC_WORKLOAD:
        return None
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != source_sha256():
        return None
    row = re.search(rf"^\|\s*{kernel}\s*\|[^|]*\|[^|]*\|\s*([0-9.eE+]+)\s*\|", text, re.M)
    return float(row.group(1)) if row else None


def run_gpu(cfg, steps, warmup, dev):
    import torch

    import chunked_kl_loss_chunk_amd as kd

    L = kd.lib()
    H, W, idx, logp, digest = _gen(cfg, dev)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    g = torch.ones(1, dtype=torch.float32, device=dev)
    dW = torch.empty((cfg.V, cfg.d), dtype=torch.float32, device=dev)

    def step():
        _, _, lse = kd.kl_forward(H, W, idx, logp, cfg.chunk, want_loss_tok=False)
        kd.kl_backward(H, W, idx, logp, lse, g, cfg.chunk, dW_out=dW, accumulate=False)

    _log(f"warmup {warmup} steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    _log(f"timing {steps} steps")
    torch.cuda.reset_peak_memory_stats(dev)
    resident = torch.cuda.memory_allocated(dev)
    # The reported loop runs with the library's kernel timing off: no events
    # between the launches of a step. Events on the stream the library
    # launches on (torch's current stream) between steps give per-step times
    # for the median; the wall clock around all steps gives the reported mean.
    L.kd_timing_enable(0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    median_ms = per_step[steps // 2] if steps % 2 else 0.5 * (per_step[steps // 2 - 1] + per_step[steps // 2])
    peak = torch.cuda.max_memory_allocated(dev)
    # A second loop of the same steps with every launch bracketed by HIP
    # events on its stream: the per-class kernel times and the roofline entry.
    _log(f"timing {steps} instrumented steps (per-kernel events)")
    L.kd_timing_enable(1)
    _kernel_stats(L)  # clear
    torch.cuda.synchronize()
    i0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    i1 = time.perf_counter()
    kstats = _kernel_stats(L)
    L.kd_timing_enable(0)
    # The forward and the backward pass, each timed alone.
    _, _, lse = kd.kl_forward(H, W, idx, logp, cfg.chunk, want_loss_tok=False)
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    for _ in range(steps):
        kd.kl_forward(H, W, idx, logp, cfg.chunk, want_loss_tok=False)
    torch.cuda.synchronize()
    f1 = time.perf_counter()
    for _ in range(steps):
        kd.kl_backward(H, W, idx, logp, lse, g, cfg.chunk, dW_out=dW, accumulate=False)
    torch.cuda.synchronize()
    b1 = time.perf_counter()
    # The same step captured once into a HIP graph and replayed: no host
    # launch gaps between the ~60 kernels of a step.
    graph_s = None
    try:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_s = (time.perf_counter() - g0) / steps
        del graph
    except RuntimeError as e:  # capture unsupported here: report the eager number only
        _log(f"graph capture skipped: {e}")
    torch.cuda.synchronize()
    one = _time_one_pass(kd, L, H, W, idx, logp, g, dW, cfg.chunk, steps, warmup, dev)
    return {
        "sec_per_step": (t1 - t0) / steps,
        "instrumented_sec_per_step": (i1 - i0) / steps,
        "median_ms_per_step": median_ms,
        "fwd_sec_per_step": (f1 - f0) / steps,
        "bwd_sec_per_step": (b1 - f1) / steps,
        "graph_sec_per_step": graph_s,
        "kernels": kstats,
        "peak_hbm_bytes": int(peak),
        "resident_bytes": int(resident),
        "cache_sha256": digest,
        "one_pass": one,
        "inputs": (H, W, idx, logp),
    }


def _time_one_pass(kd, L, H, W, idx, logp, g, dW, chunk, steps, warmup, dev):
    """The same loss and gradients through kd_fused_kl_fwd_bwd, which projects
    each chunk once and keeps its float32 logits until its dlogits are formed
    (three logit-sized GEMMs per chunk instead of four)."""
    import torch

    def step():
        kd.kl_forward_backward(H, W, idx, logp, chunk, grad=g, want_loss_tok=False, dW_out=dW,
                               accumulate=False)

    _log(f"one-pass: warmup {max(1, warmup)}, timing {steps} steps")
    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    L.kd_timing_enable(1)
    _kernel_stats(L)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    s = (time.perf_counter() - t0) / steps
    ks = _kernel_stats(L)
    L.kd_timing_enable(0)
    return {"sec_per_step": s, "kernels": ks,
            "peak_hbm_bytes": int(torch.cuda.max_memory_allocated(dev))}


def _host_info():
    """The host the oracle runs on: CPU model, logical CPUs, CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(),
            "cpus_available": len(os.sched_getaffinity(0))}


def cpu_baseline(cfg, H, W, idx, logp, rows):
    """The CPU oracle as it stands, on the first `rows` rows of the workload.
    Returns its result (for the oracle check) and the timing record."""
    import numpy as np  # noqa: F401

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity count
        threads = len(os.sched_getaffinity(0))
    Hs, ids, lps = H[:rows].cpu(), idx[:rows].cpu(), logp[:rows].cpu()
    Wc = W.cpu()
    _log(f"cpu oracle on {rows} rows, {threads} BLAS threads")
    t0 = time.perf_counter()
    ref = oracle.fused_kl_reference(Hs, Wc, ids, lps)
    dt = time.perf_counter() - t0
    return ref, {
        "value": rows / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"first {rows} of {cfg.N} rows of the workload (d={cfg.d}, V={cfg.V}, "
                   f"K={cfg.K}), dense fp64 forward+backward incl. dW; {dt:.1f} s"),
        # the dense oracle's three contractions: Z = H Wᵀ, dH = G W, dW = Gᵀ H
        "gflops": 6.0 * rows * cfg.d * cfg.V / dt / 1e9,
        **_host_info(),
    }


def oracle_check(cfg, H, W, idx, logp, ref, rows):
    """The GPU path in the bench's launch configuration (full workload, its
    chunk size) against the oracle on the sampled rows: per-token loss and lse
    (relative) and dH (max-normalised). Each of these rows depends only on its
    own inputs; dW sums over all rows and is covered by the tests' identities."""
    import numpy as np
    import torch

    import chunked_kl_loss_chunk_amd as kd

    g = torch.ones(1, dtype=torch.float32, device=H.device)
    _, loss_tok, lse = kd.kl_forward(H, W, idx, logp, cfg.chunk, want_loss_tok=True)
    dH, _ = kd.kl_backward(H, W, idx, logp, lse, g, cfg.chunk, need_dW=False)
    torch.cuda.synchronize()
    lt = loss_tok[:rows].double().cpu().numpy()
    ls = lse[:rows].double().cpu().numpy()
    dh = dH[:rows].double().cpu().numpy()
    del dH
    e_loss = float(np.abs(lt - ref["loss_tok"]).max() / max(np.abs(ref["loss_tok"]).max(), 1e-30))
    e_sum = float(abs(lt.sum() - ref["loss"]) / max(abs(ref["loss"]), 1e-30))
    e_lse = float((np.abs(ls - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1e-30)).max())
    e_dh = float(np.abs(dh - ref["dH"]).max() / max(np.abs(ref["dH"]).max(), 1e-30))
    tol_loss, tol_grad = (2e-3, 2e-2) if cfg.dtype == "bf16" else (1e-4, 1e-4)
    return {"rows": rows, "loss_tok_max_norm_err": e_loss, "loss_sum_rel_err": e_sum,
            "lse_max_rel_err": e_lse, "dH_max_norm_err": e_dh,
            "tolerance": {"loss": tol_loss, "grad": tol_grad},
            "pass": bool(e_loss < tol_loss and e_sum < tol_loss and e_lse < tol_loss
                         and e_dh < tol_grad)}


def run_teacher_cache(steps, warmup, dev, no_cpu, cpu_rows):
    """The offline teacher cache step: top-K ids + log-probs of every position
    through an 8B-class teacher head, kd_teacher_topk against torch's
    materialise-then-topk path on the same inputs."""
    import torch

    import chunked_kl_loss_chunk_amd as kd
    import workload

    N, d, V, K, chunk = 8192, 4096, 128256, 100, 1024
    L = kd.lib()
    _log(f"generating teacher head inputs N={N} d={d} V={V}")
    Ht_c, Wt_c = workload.teacher_head_inputs(N, d, V)
    Ht, Wt = Ht_c.to(dev), Wt_c.to(dev)
    torch.cuda.synchronize()

    def step():
        return kd.teacher_topk(Ht, Wt, K, chunk)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    resident = torch.cuda.memory_allocated(dev)
    L.kd_timing_enable(1)
    _kernel_stats(L)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        idx, logp, lse = step()
    torch.cuda.synchronize()
    s = (time.perf_counter() - t0) / steps
    ks = _kernel_stats(L)
    L.kd_timing_enable(0)
    peak = torch.cuda.max_memory_allocated(dev)

    def torch_path():
        for r0 in range(0, N, chunk):
            z = (Ht[r0:r0 + chunk] @ Wt.T).float()
            v, i = torch.topk(torch.log_softmax(z, dim=1), K, dim=1)
        return i, v

    for _ in range(max(1, warmup)):
        torch_path()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        torch_path()
    torch.cuda.synchronize()
    s_torch = (time.perf_counter() - t0) / steps

    # One logit GEMM per chunk (2·N·d·V flops per step); the candidates come
    # from its stored logits.
    gemm_ms = ks["fwd_logits"]["total_ms"]
    achieved = 2.0 * N * d * V * steps / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else 0.0
    out = {
        "metric": "teacher top-K cache tokens/s",
        "value": N / s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": s * 1e3,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded teacher hidden states and head)",
        "config": {"workload": "teacher-head-8k", "N": N, "d": d, "V": V, "K": K, "chunk": chunk},
        "tflops": 2.0 * N * d * V / s / 1e12,
        "frac_of_peak": 2.0 * N * d * V / s / 1e12 / PEAK_BF16_TFLOPS,
        "peak_hbm_bytes": int(peak),
        "resident_input_bytes": int(resident),
        "kernels": {k: {"avg_ms": (v["total_ms"] / v["launches"]) if v["launches"] else 0.0,
                        "launches_per_step": v["launches"] / steps} for k, v in ks.items()},
        "roofline": {"kernel": "fwd_logits (storing its logits)", "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "torch_reference": {"ms_per_step": s_torch * 1e3, "tokens_per_s": N / s_torch,
                            "what": "bf16 matmul per 1024 rows, fp32 log_softmax, torch.topk"},
        "cpu_baseline": None,
        "kernel_source_sha256": source_sha256(),
    }
    if not no_cpu:
        import oracle

        rows = min(cpu_rows, N)
        try:
            from threadpoolctl import threadpool_info

            threads = max([i.get("num_threads", 1) for i in threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        _log(f"cpu oracle on {rows} rows, {threads} BLAS threads")
        t0 = time.perf_counter()
        oracle.teacher_topk_reference(Ht_c[:rows], Wt_c, K)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": rows / dt, "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"first {rows} of {N} rows (d={d}, V={V}, K={K}), "
                                         f"fp64 logits, lse and sort; {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def sweep_fit(lines):
    """Least-squares a + b·N over the sweep's points, for peak HBM (b in bytes
    per token) and for the step time (b in µs per token), with the residual
    of every point: linear growth in N shows as residuals that are small
    against the values."""
    import numpy as np

    N = np.array([float(l["N"]) for l in lines])
    A = np.stack([np.ones_like(N), N], axis=1)
    out = {"N": [int(n) for n in N]}
    for key, scale, unit in (("peak_hbm_bytes", 1.0, "bytes"), ("ms_per_step", 1e3, "us"),
                             ("one_pass_peak_hbm_bytes", 1.0, "bytes")):
        y = np.array([float(l[key]) for l in lines])
        (a, b), *_ = np.linalg.lstsq(A, y, rcond=None)
        res = y - (a + b * N)
        out[key] = {"a": float(a), "b_per_token": float(b * scale), "unit_b": f"{unit}/token",
                    "residuals": [float(x) for x in res],
                    "max_rel_residual": float(np.max(np.abs(res) / np.abs(y)))}
    return out


def run_gemm_ceiling(steps, warmup, dev):
    """torch's bf16 matmul (hipBLASLt) on the three contraction shapes of the
    8K head, with the bench's seeded operands, beside the fused kernels' own
    per-launch times measured in the same process on the same inputs:

      chunk logits  [1024 x 3072] . [3072 x 128256]   (forward; recomputed in the backward)
      window dH     [4096 x 128256] . [128256 x 3072]
      window dW     [128256 x 4096] . [4096 x 3072]   (float32 output where torch offers it)

    The dlogits operand of dH and dW is the real one for the first 4096 rows
    (S_r q − p at the cached ids, rounded to bf16), formed here with torch."""
    import torch

    import chunked_kl_loss_chunk_amd as kd
    import workload

    cfg = workload.config(3)
    L = kd.lib()
    H, W, idx, logp, _ = _gen(cfg, dev)
    C, win = cfg.chunk, 4 * cfg.chunk
    Hc = H[:C].contiguous()
    Hw = H[:win].contiguous()
    with torch.no_grad():
        z = (Hw @ W.T).float()
        q = torch.softmax(z, dim=1)
        del z
        p = torch.exp(logp[:win])
        dl = q * p.sum(dim=1, keepdim=True)
        del q
        dl.scatter_add_(1, idx[:win].long(), -p)
        dl = dl.to(torch.bfloat16)
        dlT = dl.t().contiguous()
    torch.cuda.synchronize()

    def mm_f32(a, b):
        # bf16 operands, float32 output (torch's out_dtype form of mm)
        return torch.mm(a, b, out_dtype=torch.float32)

    if mm_f32(dlT[:256], Hw).dtype != torch.float32:
        raise RuntimeError("torch.mm did not produce a float32 output for the dW case")

    cases = {
        "logits (H_c . W^T)": (lambda: torch.mm(Hc, W.t()), 2.0 * C * cfg.d * cfg.V),
        "logits (W . H_c^T)": (lambda: torch.mm(W, Hc.t()), 2.0 * C * cfg.d * cfg.V),
        "dH (dl . W)": (lambda: torch.mm(dl, W), 2.0 * win * cfg.d * cfg.V),
        "dW (dl^T . H_w, fp32 out)": (lambda: mm_f32(dlT, Hw), 2.0 * win * cfg.d * cfg.V),
        "dW (dl^T . H_w, bf16 out)": (lambda: torch.mm(dlT, Hw), 2.0 * win * cfg.d * cfg.V),
    }
    reps = max(steps, 5)
    lib_ms = {}
    for name, (fn, flops) in cases.items():
        for _ in range(max(warmup, 2)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        lib_ms[name] = {"ms": ms, "tflops": flops / ms / 1e9, "frac_of_peak": flops / ms / 1e9 / PEAK_BF16_TFLOPS}
        _log(f"{name}: {ms:.3f} ms")
    del dl, dlT
    torch.cuda.empty_cache()

    # The fused kernels on the same inputs, same process: per-launch HIP-event
    # times of a full forward + backward step.
    g = torch.ones(1, dtype=torch.float32, device=dev)
    dW = torch.empty((cfg.V, cfg.d), dtype=torch.float32, device=dev)

    def step():
        _, _, lse = kd.kl_forward(H, W, idx, logp, cfg.chunk, want_loss_tok=False)
        kd.kl_backward(H, W, idx, logp, lse, g, cfg.chunk, dW_out=dW, accumulate=False)

    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()
    L.kd_timing_enable(1)
    _kernel_stats(L)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    ks = _kernel_stats(L)
    L.kd_timing_enable(0)
    fused = {k: ks[k]["total_ms"] / ks[k]["launches"] for k in
             ("fwd_logits", "bwd_dlogits", "bwd_dh", "bwd_dw") if ks[k]["launches"]}
    # A logit launch covers several chunks (the forward's group, the
    # backward's window) and dH and dW one window each: compare per chunk
    # and per window with the library's single GEMMs.
    n_chunks = -(-cfg.N // C)
    n_windows = -(-cfg.N // (win))
    per_unit = {"fwd_logits per chunk": ks["fwd_logits"]["total_ms"] / (reps * n_chunks),
                "bwd_dlogits per chunk": ks["bwd_dlogits"]["total_ms"] / (reps * n_chunks),
                "bwd_dh per window": ks["bwd_dh"]["total_ms"] / (reps * n_windows),
                "bwd_dw per window": ks["bwd_dw"]["total_ms"] / (reps * n_windows)}
    best_logits = min(lib_ms["logits (H_c . W^T)"]["ms"], lib_ms["logits (W . H_c^T)"]["ms"])
    ratio = {
        "fwd_logits / best logits GEMM": per_unit["fwd_logits per chunk"] / best_logits,
        "bwd_dlogits / best logits GEMM": per_unit["bwd_dlogits per chunk"] / best_logits,
        "bwd_dh / dH GEMM": per_unit["bwd_dh per window"] / lib_ms["dH (dl . W)"]["ms"],
        "bwd_dw / dW GEMM (fp32 out)": per_unit["bwd_dw per window"] / lib_ms["dW (dl^T . H_w, fp32 out)"]["ms"],
    }
    print(json.dumps({
        "what": "hipBLASLt (torch.mm, bf16 operands) on the fused loss's contraction shapes, "
                "8K head, beside the fused kernels in the same process",
        "config": {"workload": cfg.name, "N": cfg.N, "d": cfg.d, "V": cfg.V, "chunk": C,
                   "window": win},
        "torch_mm": lib_ms,
        "fused_avg_ms_per_launch": fused,
        "fused_ms_per_chunk_or_window": per_unit,
        "fused_over_library": ratio,
        "reps": reps,
        "kernel_source_sha256": source_sha256(),
    }), flush=True)


def run_hbm_copy(steps, warmup, dev):
    """A plain 1 GiB device-to-device copy (torch copy_ of 256 Mi float32):
    the HBM bandwidth one copy kernel reaches, and the reference a counter
    profile of it gives for scaling FETCH_SIZE and WRITE_SIZE to bytes (it
    reads and writes exactly 1 GiB per call)."""
    import torch

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(warmup, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"what": "device copy of 1 GiB (reads 1 GiB, writes 1 GiB)", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "ms": ms, "GB_per_s": 2 * 4 * n / ms / 1e6,
                      "steps": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="8k-head",
                    choices=[*WORKLOADS, "sweep", "teacher-cache", "gemm-ceiling", "hbm-copy"])
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}, WORLD_SIZE={world}): "
              "the loss is built and measured for a single MI355X; the multi-GPU split is "
              "a design note only.", file=sys.stderr)
        sys.exit(2)

    import torch

    import workload

    dev = torch.device("cuda:0")
    if args.workload == "teacher-cache":
        run_teacher_cache(args.steps, args.warmup, dev, args.no_cpu_baseline,
                          min(args.cpu_rows, 1024))
        return
    if args.workload == "sweep":
        lines = []
        for N in workload.SWEEP_N:
            cfg = workload.config(4, N=N)
            r = run_gpu(cfg, args.steps, args.warmup, dev)
            s = r["sec_per_step"]
            line = {
                "workload": cfg.name, "N": N, "d": cfg.d, "V": cfg.V, "K": cfg.K, "chunk": cfg.chunk,
                "ms_per_step": s * 1e3, "tokens_per_s": N / s,
                "tflops": 8 * N * cfg.d * cfg.V / s / 1e12,
                "frac_of_peak": 8 * N * cfg.d * cfg.V / s / 1e12 / PEAK_BF16_TFLOPS,
                "one_pass_ms_per_step": r["one_pass"]["sec_per_step"] * 1e3,
                "one_pass_tokens_per_s": N / r["one_pass"]["sec_per_step"],
                "peak_hbm_bytes": r["peak_hbm_bytes"], "resident_bytes": r["resident_bytes"],
                "peak_hbm_gib": r["peak_hbm_bytes"] / 2**30,
                "one_pass_peak_hbm_bytes": r["one_pass"]["peak_hbm_bytes"],
                "pages_context": PAGES_CONTEXT_SWEEP.get(N),
                "kernel_source_sha256": source_sha256(),
            }
            lines.append(line)
            print(json.dumps(line), flush=True)
            del r
            torch.cuda.empty_cache()
        print(json.dumps({"sweep_fit": sweep_fit(lines)}), flush=True)
        return
    if args.workload == "gemm-ceiling":
        run_gemm_ceiling(args.steps, args.warmup, dev)
        return
    if args.workload == "hbm-copy":
        run_hbm_copy(args.steps, args.warmup, dev)
        return

    cid, _ = WORKLOADS[args.workload]
    cfg = workload.config(cid)
    r = run_gpu(cfg, args.steps, args.warmup, dev)
    s = r["sec_per_step"]
    N, d, V = cfg.N, cfg.d, cfg.V
    flops = 8.0 * N * d * V
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    ks = r["kernels"]
    gemms = ["fwd_logits", "bwd_dlogits", "bwd_dh", "bwd_dw"]
    dom = max(gemms, key=lambda k: ks[k]["total_ms"])
    # Each of the four contractions does 2·rows·d·V flops for the rows a
    # launch covers (a group of chunks, a dW window), so over the timed steps
    # it did 2·N·d·V·steps.
    dom_ms = ks[dom]["total_ms"]
    achieved = 2.0 * N * d * V * args.steps / (dom_ms / 1e3) / 1e12 if dom_ms > 0 else 0.0
    kernels_out = {k: {"avg_ms": (v["total_ms"] / v["launches"]) if v["launches"] else 0.0,
                       "launches_per_step": v["launches"] / args.steps,
                       "ms_per_step": v["total_ms"] / args.steps} for k, v in ks.items()}
    out = {
        "metric": "fused KL fwd+bwd tokens/s",
        "value": N / s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded H, W and random-teacher top-K cache)",
        "config": {"workload": cfg.name, "N": N, "d": d, "V": V, "K": cfg.K, "chunk": cfg.chunk,
                   "global_batch": N, "parallelism": "single-gpu"},
        "tflops": flops / s / 1e12,
        "tflops_pages_convention": 6.0 * N * d * V / s / 1e12,
        "frac_of_peak": flops / s / 1e12 / peak,
        "peak_hbm_bytes": r["peak_hbm_bytes"],
        "resident_input_bytes": r["resident_bytes"],
        "kernels": kernels_out,
        "median_ms_per_step": r["median_ms_per_step"],
        "instrumented_ms_per_step": r["instrumented_sec_per_step"] * 1e3,
        "fwd_ms_per_step": r["fwd_sec_per_step"] * 1e3,
        "bwd_ms_per_step": r["bwd_sec_per_step"] * 1e3,
        "graph_ms_per_step": None if r["graph_sec_per_step"] is None else r["graph_sec_per_step"] * 1e3,
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": _traffic(dom, cfg.name)},
        "cache_sha256": r["cache_sha256"],
        "kernel_source_sha256": source_sha256(),
        "pages_context": PAGES_CONTEXT_8K if cid == 3 else None,
    }
    one = r["one_pass"]
    s1 = one["sec_per_step"]
    out["one_pass"] = {
        "what": ("kd_fused_kl_fwd_bwd: the same loss and gradients with each chunk projected "
                 "once (6·N·d·V GEMM flops) and its float32 logits kept until its dlogits "
                 "are formed; the headline keeps the pages' recompute schedule (8·N·d·V)"),
        "ms_per_step": s1 * 1e3,
        "tokens_per_s": N / s1,
        "tflops": 6.0 * N * d * V / s1 / 1e12,
        "peak_hbm_bytes": one["peak_hbm_bytes"],
        "kernels": {k: {"avg_ms": (v["total_ms"] / v["launches"]) if v["launches"] else 0.0,
                        "launches_per_step": v["launches"] / args.steps,
                        "ms_per_step": v["total_ms"] / args.steps}
                    for k, v in one["kernels"].items() if v["launches"]},
    }
    if not args.no_cpu_baseline:
        H, W, idx, logp = r["inputs"]
        rows = min(args.cpu_rows, N)
        ref, out["cpu_baseline"] = cpu_baseline(cfg, H, W, idx, logp, rows)
        out["oracle_check"] = oracle_check(cfg, H, W, idx, logp, ref, rows)
        del ref
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
