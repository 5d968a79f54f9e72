"""The layer's calls under HIP graph capture (through torch.cuda.graph).

Every entry point only enqueues kernels on the given stream: no allocation,
no memset, no copy, no synchronisation. So a whole training step (routing,
TopK, fine and coarse forward, both backwards) can be captured once and
replayed. Each replay must reproduce the eager step bit for bit, with eager
work and synchronisations between the replays.
"""
import pytest
import torch

from video_dit_trainable_amd import vsa2
from video_dit_trainable_amd.configs import Workload
from video_dit_trainable_amd.inputs import make_gate_inputs, make_grad_out, make_qkv

pytestmark = pytest.mark.gpu

MID = Workload("graph-mid", 61, (8, 16, 32), 1, 4, 128, "bf16", 8, "lowrank", skew=True, train=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vsa2.lib()


def test_captured_step_replays_bitwise():
    w = MID
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_qkv(w))
    x, w_g = (t.to(dev) for t in make_gate_inputs(w, zero_gate=False))
    d_o = make_grad_out(w).to(dev)
    p = vsa2.problem(w.batch, w.heads, w.head_dim, w.grid, w.dtype)
    layer = vsa2.Layer(p, w.topk, w.d_model, device=dev)

    def step():
        layer.forward(q, k, v, x, w_g)
        return layer.backward(q, k, v, x, w_g, d_o)

    g = step()
    torch.cuda.synchronize()
    outs = lambda: [layer.o, layer.o_f, layer.lse, layer.row_ptr, layer.col_idx, layer.col_ptr, layer.row_idx,
                    g["dq"], g["dk"], g["dv"], g["dx"], g["dw_g"]]
    want = [t.clone() for t in outs()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # a warm-up call on the capture stream's side, as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        for t in outs():               # eager work between replays: clobber every output
            t.fill_(-1 if not t.is_floating_point() else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, (a, b) in enumerate(zip(outs(), want)):
            assert torch.equal(a, b), f"replay {replay}: output {n} differs from the eager step"
