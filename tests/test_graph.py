"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library launches only on the caller's stream and allocates nothing,
and its workspaces need no clearing, so its calls capture like any kernel
launch.  The captured sequence mixes the paths: a bf16 ring call, a tiled
K split (partials, then the reduce kernel), an fp32 M = 16 split call, an
fp8 call with a fused GELU epilogue, a bf16 decode call with weights stored
N x K split over K into a bf16 output, and the bf16 ring writing a
saturating fp8 output, the whole-line bf16 kernel (4096 x 4096 x 1024),
and the plain fp32 M = 16 call (A staged through LDS, no workspace).  It
is replayed several times, with
eager work and synchronisations between replays, and every replay must
reproduce the eager results bit for bit (every path is deterministic).
"""
import pytest
import torch

import tiled_gemm_f32_amd as tg
from tiled_gemm_f32_amd.workloads import make_bias, make_random_inputs

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _dev(t):
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cuda().view(torch.float8_e4m3fn)
    return t.cuda()


def test_graph_capture_and_replay(gpu_available):
    A1, B1, _ = make_random_inputs(1024, 1024, 2048, seed=900, dist="normal", dtype="bf16f32")
    A2, B2, _ = make_random_inputs(256, 512, 6000, seed=901, dist="normal", dtype="f32")
    A3, B3, _ = make_random_inputs(16, 4096, 8192, seed=902, dist="normal", dtype="f32")
    A4, B4, _ = make_random_inputs(512, 768, 1024, seed=903, dist="normal", dtype="fp8f32")
    B4t = B4.t().contiguous()
    bias = make_bias(768, seed=904).cuda()
    A1, B1, A2, B2, A3, B3, A4, B4t = (_dev(t) for t in (A1, B1, A2, B2, A3, B3, A4, B4t))
    A5, B5, _ = make_random_inputs(16, 2048, 4096, seed=905, dist="normal", dtype="bf16f32")
    B5t = _dev(B5.t().contiguous())
    A5 = _dev(A5)
    A6, B6, _ = make_random_inputs(4096, 4096, 1024, seed=906, dist="normal", dtype="bf16f32")
    A7, B7, _ = make_random_inputs(16, 4096, 2048, seed=907, dist="normal", dtype="f32")
    A6, B6, A7, B7 = (_dev(t) for t in (A6, B6, A7, B7))
    ws2 = tg.workspace(256, 512, 6000)
    ws3 = tg.workspace(16, 4096, 8192)
    ws5 = tg.workspace(16, 2048, 4096, dtype=tg.GEMM_DTYPE_BF16F32)
    outs = [torch.empty(1024, 1024, device="cuda"), torch.empty(256, 512, device="cuda"),
            torch.empty(16, 4096, device="cuda"), torch.empty(512, 768, device="cuda"),
            torch.empty(16, 2048, dtype=torch.bfloat16, device="cuda"),
            torch.empty(1024, 1024, dtype=torch.float8_e4m3fn, device="cuda"),
            torch.empty(4096, 4096, device="cuda"), torch.empty(16, 4096, device="cuda")]
    names = {k["id"]: k["name"] for k in tg.kernels()}
    for (M, N, K, dt) in [(4096, 4096, 1024, tg.GEMM_DTYPE_BF16F32), (16, 4096, 2048, tg.GEMM_DTYPE_F32)]:
        st, pl = tg.gemm_plan_query(dt, M, N, K, 1.0, A6.data_ptr(), K, B6.data_ptr(), N, 0.0, A6.data_ptr(), N, 0, 0)
        assert st == tg.GEMM_OK and ("lines" in names[pl["kernel_id"]] or "alds" in names[pl["kernel_id"]])

    def sequence():
        tg.gemm(A1, B1, outs[0])
        tg.gemm(A2, B2, outs[1], ws=ws2)
        tg.gemm(A3, B3, outs[2], ws=ws3)
        tg.gemm(A4, B4t, outs[3], op_b="T", bias=bias, activation="gelu", alpha=0.125)
        # weights stored N x K, split over K through the workspace, bf16 output
        tg.gemm(A5, B5t, None, op_b="T", ws=ws5, out=outs[4], out_scale=0.5)
        # the bf16 ring with a saturating fp8 output
        tg.gemm(A1, B1, None, out=outs[5], out_scale=0.01)
        # the whole-line bf16 kernel; the plain fp32 M = 16 call
        tg.gemm(A6, B6, outs[6])
        tg.gemm(A7, B7, outs[7])

    say("[graph] eager reference")
    sequence()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):      # warm up on the capture stream
        sequence()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    say("[graph] capture")
    with torch.cuda.graph(graph):
        sequence()
    torch.cuda.synchronize()

    def bits(t):
        return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t.view(torch.int16) \
            if t.dtype == torch.bfloat16 else t.view(torch.int32)

    for rep in range(4):
        for o in outs:
            bits(o).fill_(-1)              # eager work between replays: NaN patterns
        ws2.fill_(0xFF)
        ws5.fill_(0xFF)
        torch.cuda.synchronize()
        say(f"[graph] replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(bits(o), bits(r)), f"replay {rep}, call {i}"
