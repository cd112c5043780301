"""The C ABI from a non-Python caller: chunked_kl_loss_chunk_amd/examples/
abi_client (C++, HIP runtime API, built by the host compiler next to the
library) runs the forward and backward passes of the tiny fp32 workload, or
the one-pass call; its outputs are compared with the oracle at the fp32
tolerances, and the two schedules with each other bit for bit."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workload
from test_gpu_parity import TOL, kd, max_norm_err, rel_err  # noqa: F401

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "chunked_kl_loss_chunk_amd", "examples", "abi_client")


def _run_client(tmp_path, cfg, H, W, idx, logp, g, mode):
    src, dst = tmp_path / "in.bin", tmp_path / f"out_{mode}.bin"
    with open(src, "wb") as f:
        np.array([cfg.N, cfg.d, cfg.V, cfg.K, 48], dtype=np.int64).tofile(f)
        H.numpy().astype(np.float32).tofile(f)
        W.numpy().astype(np.float32).tofile(f)
        idx.numpy().astype(np.int32).tofile(f)
        logp.numpy().astype(np.float32).tofile(f)
        np.array([g], dtype=np.float32).tofile(f)
    args = [CLIENT, str(src), str(dst)] + (["one-pass"] if mode == "one-pass" else [])
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    return np.fromfile(dst, dtype=np.float32)


def test_c_abi_client_one_pass_matches_oracle_and_two_pass(kd, tmp_path):
    assert os.path.exists(CLIENT), "abi_client is built by chunked_kl_loss_chunk_amd._build.build()"
    cfg = workload.config(1)
    H, W, idx, logp = workload.make_inputs(cfg)
    two = _run_client(tmp_path, cfg, H, W, idx, logp, 0.6, "two-pass")
    one = _run_client(tmp_path, cfg, H, W, idx, logp, 0.6, "one-pass")
    assert np.array_equal(one, two)
    out = one.astype(np.float64)
    N, d = cfg.N, cfg.d
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=0.6)
    t = TOL["f32"]
    assert rel_err(out[0], ref["loss"]) < t["loss"]
    assert max_norm_err(out[1 + 2 * N:1 + 2 * N + N * d].reshape(N, d), ref["dH"]) < t["grad"]
    assert max_norm_err(out[1 + 2 * N + N * d:].reshape(cfg.V, d), ref["dW"]) < t["grad"]


def test_c_abi_client_matches_oracle(kd, tmp_path):
    assert os.path.exists(CLIENT), "abi_client is built by chunked_kl_loss_chunk_amd._build.build()"
    cfg = workload.config(1)
    H, W, idx, logp = workload.make_inputs(cfg)
    g = 0.6
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([cfg.N, cfg.d, cfg.V, cfg.K, 48], dtype=np.int64).tofile(f)
        H.numpy().astype(np.float32).tofile(f)
        W.numpy().astype(np.float32).tofile(f)
        idx.numpy().astype(np.int32).tofile(f)
        logp.numpy().astype(np.float32).tofile(f)
        np.array([g], dtype=np.float32).tofile(f)
    res = subprocess.run([CLIENT, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    out = np.fromfile(dst, dtype=np.float32).astype(np.float64)
    N, d, V = cfg.N, cfg.d, cfg.V
    loss, tok, lse = out[0], out[1:1 + N], out[1 + N:1 + 2 * N]
    dH = out[1 + 2 * N:1 + 2 * N + N * d].reshape(N, d)
    dW = out[1 + 2 * N + N * d:].reshape(V, d)
    ref = oracle.fused_kl_reference(H, W, idx, logp, grad=g)
    t = TOL["f32"]
    assert rel_err(loss, ref["loss"]) < t["loss"]
    assert rel_err(tok, ref["loss_tok"]) < t["loss"] and rel_err(lse, ref["lse"]) < t["loss"]
    assert max_norm_err(dH, ref["dH"]) < t["grad"] and max_norm_err(dW, ref["dW"]) < t["grad"]
