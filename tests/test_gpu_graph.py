"""The loss under HIP graph capture.

The library allocates nothing, never synchronises and clears its scratch with
kernels (no memset nodes), so a caller may capture a forward + backward step
into a graph and replay it. Each replay here runs on new inputs copied into
the captured buffers, with eager work between replays, and must equal an
eager run on the same inputs bit for bit (the path is deterministic).
"""
import pytest
import torch

from test_gpu_parity import _case, kd  # noqa: F401

pytestmark = pytest.mark.gpu


def _eager(kd, H, W, idx, logp, chunk, weight=None, reduction="sum"):
    loss, tok, lse = kd.kl_forward(H, W, idx, logp, chunk, weight=weight, reduction=reduction)
    g = torch.full((1,), 0.75, dtype=torch.float32, device=H.device)
    dH, dW = kd.kl_backward(H, W, idx, logp, lse, g, chunk, weight=weight, reduction=reduction)
    return loss, tok, lse, dH, dW


@pytest.mark.parametrize("dtype,weighted", [("bf16", False), ("f32", True)])
def test_graph_replays_equal_eager(kd, dtype, weighted):
    dev = torch.device("cuda:0")
    N, d, V, K, chunk = 300, 128, 2000, 16, 64
    H, W, idx, logp = (t.to(dev) for t in _case(N, d, V, K, dtype, seed=71))
    w = torch.rand(N, device=dev) if weighted else None
    red = "mean" if weighted else "sum"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            _eager(kd, H, W, idx, logp, chunk, w, red)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _eager(kd, H, W, idx, logp, chunk, w, red)
    for rep in range(3):
        Hn, Wn, idn, lpn = (t.to(dev) for t in _case(N, d, V, K, dtype, seed=72 + rep))
        H.copy_(Hn)
        W.copy_(Wn)
        idx.copy_(idn)
        logp.copy_(lpn)
        if weighted:
            w.copy_(torch.rand(N, device=dev))
        graph.replay()
        torch.cuda.synchronize()
        ref = _eager(kd, H, W, idx, logp, chunk, w, red)
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "loss_tok", "lse", "dH", "dW"), outs, ref):
            assert torch.equal(a, b), (rep, name)


def _eager_one_pass(kd, H, W, idx, logp, chunk, weight=None, reduction="sum"):
    g = torch.full((1,), 0.75, dtype=torch.float32, device=H.device)
    return kd.kl_forward_backward(H, W, idx, logp, chunk, grad=g, weight=weight,
                                  reduction=reduction)


@pytest.mark.parametrize("dtype,weighted", [("bf16", True), ("f32", False)])
def test_one_pass_graph_replays_equal_eager(kd, dtype, weighted):
    """kd_fused_kl_fwd_bwd captured once; each replay on new inputs equals an
    eager call on them bit for bit."""
    dev = torch.device("cuda:0")
    N, d, V, K, chunk = 700, 96, 3000, 20, 128
    H, W, idx, logp = (t.to(dev) for t in _case(N, d, V, K, dtype, seed=81))
    w = torch.rand(N, device=dev) if weighted else None
    red = "mean" if weighted else "sum"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            _eager_one_pass(kd, H, W, idx, logp, chunk, w, red)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _eager_one_pass(kd, H, W, idx, logp, chunk, w, red)
    for rep in range(3):
        Hn, Wn, idn, lpn = (t.to(dev) for t in _case(N, d, V, K, dtype, seed=82 + rep))
        H.copy_(Hn)
        W.copy_(Wn)
        idx.copy_(idn)
        logp.copy_(lpn)
        if weighted:
            w.copy_(torch.rand(N, device=dev))
        graph.replay()
        torch.cuda.synchronize()
        ref = _eager_one_pass(kd, H, W, idx, logp, chunk, w, red)
        torch.cuda.synchronize()
        for name, a, b in zip(("loss", "loss_tok", "lse", "dH", "dW"), outs, ref):
            assert torch.equal(a, b), (rep, name)


def test_teacher_cache_cast_and_scale_graph_replays_equal_eager(kd):
    """The teacher cache producer, the fp32 -> bf16 cast and the in-place
    scale captured once (every launch on the capturing stream, no memset
    nodes); each replay on new inputs equals eager calls on them bit for bit."""
    dev = torch.device("cuda:0")
    N, d, V, K, chunk = 600, 64, 3000, 12, 256

    def draw(seed):
        g = torch.Generator().manual_seed(seed)
        Ht = torch.randn(N, d, generator=g).to(torch.bfloat16)
        Wt = (torch.randn(V, d, generator=g) * 2 * d ** -0.5).to(torch.bfloat16)
        x = torch.randn(N, 136, generator=g)
        y = torch.randn(N, 72, generator=g).to(torch.bfloat16)
        return Ht.to(dev), Wt.to(dev), x.to(dev), y.to(dev)

    Ht, Wt, x, y0 = draw(91)
    y = y0.clone()
    s = torch.full((1,), 0.5, dtype=torch.float32, device=dev)

    def run():
        idx, logp, lse = kd.teacher_topk(Ht, Wt, K, chunk)
        xb = kd.cast_f32_to_bf16(x)
        kd.scale_(y, s)
        return idx, logp, lse, xb

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    for rep in range(3):
        Hn, Wn, xn, yn = draw(92 + rep)
        Ht.copy_(Hn)
        Wt.copy_(Wn)
        x.copy_(xn)
        y.copy_(yn)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs] + [y.clone()]
        y.copy_(yn)
        ref = list(run()) + [y]
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "logp", "lse", "cast", "scale"), got, ref):
            assert torch.equal(a, b), (rep, name)
