"""Streams and graph capture through the C ABI.

* One plan run concurrently on two streams with different inputs: each
  result equals the result of the same run alone (a plan is immutable and the
  library keeps no state between calls).
* tsgemm_run and the MX pack + tsgemm_run_mx_packed step captured into a
  HIP graph (torch.cuda.graph) and replayed several times with new input
  contents copied in between, each replay checked against an eager run.
"""

import numpy as np
import pytest
import torch

import persistent_tile_scheduled_amd as tsg
from workloads import make_inputs, make_mx_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def test_one_plan_two_streams():
    M, N, K = 1024, 768, 1024
    plan = tsg.Plan(M, N, K, "bf16", 256, 256, 64, 4, 3)
    ins = [make_inputs(M, N, K, "bf16", "normal_sqrtk", seed) for seed in (11, 12)]
    dev = [(a.to(DEV), b.to(DEV)) for a, b in ins]
    alone = []
    for a, b in dev:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        plan.run(a, b, c)
        torch.cuda.synchronize()
        alone.append(_bits(c))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    torch.cuda.synchronize()
    for rep in range(3):
        for s, (a, b), c in zip(streams, dev, outs):
            with torch.cuda.stream(s):
                plan.run(a, b, c, stream=s)
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(_bits(outs[i]), alone[i]), f"stream {i}, repetition {rep}"


def test_gemm_graph_replays_match_eager():
    M, N, K = 768, 512, 512
    plan = tsg.Plan(M, N, K, "fp16", 128, 128, 64, 2, 3)
    a = torch.empty((M, K), dtype=torch.float16, device=DEV)
    b = torch.empty((K, N), dtype=torch.float16, device=DEV)
    c = torch.empty((M, N), dtype=torch.float16, device=DEV)
    a0, b0 = make_inputs(M, N, K, "fp16", "uniform", 21)
    a.copy_(a0.to(DEV)); b.copy_(b0.to(DEV))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):       # warm-up outside the capture
        plan.run(a, b, c, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(a, b, c)
    for seed in (22, 23, 24):
        an, bn = make_inputs(M, N, K, "fp16", "uniform", seed)
        a.copy_(an.to(DEV)); b.copy_(bn.to(DEV))
        c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(c)
        ref = torch.empty_like(c)
        plan.run(a, b, ref)
        torch.cuda.synchronize()
        assert np.array_equal(got, _bits(ref)), f"replay with seed {seed}"


def test_mx_packed_step_graph_replays_match_eager():
    M, N, K = 520, 264, 512
    plan = tsg.Plan(M, N, K, "mxfp8", 256, 256, 128, 2, 2, num_workgroups=6)
    A, SFA, B, SFB = [torch.from_numpy(x).to(DEV) for x in make_mx_inputs(M, N, K, seed=31, spread=2)]
    sfp = [torch.empty((plan.mx_packed_scale_bytes(op),), dtype=torch.uint8, device=DEV) for op in (0, 1)]
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)

    def step():
        plan.mx_pack_scales(SFA, sfp[0], 0)
        plan.mx_pack_scales(SFB, sfp[1], 1)
        plan.run_mx_packed(A, sfp[0], B, sfp[1], C)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in (32, 33, 34):
        new = [torch.from_numpy(x).to(DEV) for x in make_mx_inputs(M, N, K, seed=seed, spread=2)]
        for dst, src in zip((A, SFA, B, SFB), new):
            dst.copy_(src)
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _bits(C)
        ref = torch.empty_like(C)
        plan.run_mx(A, SFA, B, SFB, ref)
        torch.cuda.synchronize()
        assert np.array_equal(got, _bits(ref)), f"replay with seed {seed}"
