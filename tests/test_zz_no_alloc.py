"""The allocation-free MX entry point (tsgemm_run_mx_noalloc) through the C ABI.

It packs SFA and SFB into the library's static per-device workspace and runs
the packed-scale kernel, so C must be bit for bit the output of the existing
path with caller-owned packed scales (tsgemm_mx_pack_scales twice, then
tsgemm_run_mx_packed), which is itself bit for bit tsgemm_run_mx.  Two calls in
a row, the second on a smaller problem, show that what the first call left in
the shared workspace does not leak into the second.  Both are also held to the
MX bound against the CPU oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import persistent_tile_scheduled_amd as tsg
from workloads import make_mx_inputs

DEV = torch.device("cuda:0")


def _existing_packed_path(plan, dev_ops, C):
    A, SFA, B, SFB = dev_ops
    sfp = [torch.empty((plan.mx_packed_scale_bytes(op),), dtype=torch.uint8, device=DEV) for op in (0, 1)]
    plan.mx_pack_scales(SFA, sfp[0], 0)
    plan.mx_pack_scales(SFB, sfp[1], 1)
    plan.run_mx_packed(A, sfp[0], B, sfp[1], C)


@pytest.mark.gpu
def test_noalloc_matches_packed_path_twice_shrinking():
    lib = tsg.load()
    # first call: ragged rows and columns, 13 slabs (4 scale groups, the last partial)
    # second call: a smaller problem, fewer blocks and groups than the first
    for (M, N, K, P, seed) in ((1000, 776, 1664, 5, 21), (300, 264, 384, 3, 22)):
        print(f"[case] noalloc {M}x{N}x{K} P={P}", flush=True)
        A, SFA, B, SFB = make_mx_inputs(M, N, K, seed=seed, spread=2)
        dev_ops = [torch.from_numpy(x).to(DEV) for x in (A, SFA, B, SFB)]
        plan = tsg.Plan(M, N, K, "mxfp8", 256, 256, 128, 2, 2, num_workgroups=P)
        C_ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        _existing_packed_path(plan, dev_ops, C_ref)
        buf = torch.full((M * N + 64,), float("nan"), dtype=torch.bfloat16, device=DEV)
        C = buf[: M * N].view(M, N)
        rc = lib.tsgemm_run_mx_noalloc(plan._h, *[t.data_ptr() for t in dev_ops], C.data_ptr(),
                                       torch.cuda.current_stream(DEV).cuda_stream)
        assert rc == tsg.OK, tsg.last_error()
        torch.cuda.synchronize()
        assert torch.isnan(buf[M * N:].float()).all(), "write past the end of C"
        assert torch.equal(C.view(torch.int16), C_ref.view(torch.int16)), "differs from the packed path"
        got = C.cpu().double().numpy()
        c64 = oracle.mx_gemm_f64(A, SFA, B, SFB)
        mag = oracle.mx_gemm_f64(A & 0x7F, SFA, B & 0x7F, SFB)
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - c64) <= 2.0 ** -8 * np.abs(c64) + 2.0 ** -10 * mag)


def test_noalloc_rejects_plans_beyond_the_workspace():
    """(M + N) * K / 32 bytes of packed scales above the 16 MiB workspace are
    refused before anything is launched (no GPU needed)."""
    lib = tsg.load()
    big = tsg.Plan(16384, 16384, 16512, "mxfp8", 256, 256, 128, 8, 2)   # 2 x 8.25 MiB
    assert lib.tsgemm_run_mx_noalloc(big._h, None, None, None, None, None, None) == tsg.EUNSUPPORTED
    assert "static workspace" in tsg.last_error()
    fits = tsg.Plan(16384, 16384, 16384, "mxfp8", 256, 256, 128, 8, 2)  # 2 x 8 MiB: exactly full
    assert lib.tsgemm_run_mx_noalloc(fits._h, None, None, None, None, None, None) == tsg.EINVAL
    assert "NULL" in tsg.last_error()
    fp16 = tsg.Plan(512, 512, 512, "fp16", 128, 128, 64, 2, 2)
    assert lib.tsgemm_run_mx_noalloc(fp16._h, None, None, None, None, None, None) == tsg.EINVAL
