"""Host-side checks of the C ABI (no GPU): the library loads and exports every
function include/tsgemm.h declares; create() validates its arguments; plan
arithmetic; and the scheduler code compiled for the host reproduces the
oracle schedule bit for bit."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import persistent_tile_scheduled_amd as tsg
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "tsgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsgemm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = tsg.load()
    declared = _header_functions()
    assert set(declared) == set(tsg.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("args,code,needle", [
    ((512, 512, 512, 4, 128, 128, 64, 2, 2), tsg.EINVAL, "dtype"),
    ((512, 512, 512, 3, 256, 256, 64, 2, 2), tsg.EUNSUPPORTED, "MXFP8 tile"),
    ((512, 512, 384 + 64, 3, 256, 256, 128, 2, 2), tsg.EINVAL, "multiple of block_K"),
    ((512, 500, 512, 3, 256, 256, 128, 2, 2), tsg.EINVAL, "divisible by 8"),
    ((512, 512, 1 << 23, 3, 256, 256, 128, 2, 2), tsg.EUNSUPPORTED, "exceeds 2^31"),
    ((-1, 512, 512, 1, 128, 128, 64, 2, 2), tsg.EINVAL, ">= 0"),
    ((512, 512, 500, 1, 128, 128, 64, 2, 2), tsg.EINVAL, "multiple of block_K"),
    ((512, 500, 512, 1, 128, 128, 64, 2, 2), tsg.EINVAL, "divisible by 8"),
    ((512, 512, 512, 1, 128, 128, 64, 0, 2), tsg.EINVAL, "group_size"),
    ((512, 512, 512, 1, 128, 128, 64, 2, 1), tsg.EINVAL, "num_stages"),
    ((512, 512, 512, 1, 64, 64, 64, 2, 2), tsg.EUNSUPPORTED, "not compiled"),
    ((512, 512, 512, 1, 128, 256, 64, 2, 2), tsg.EUNSUPPORTED, "not compiled"),
    ((1 << 31, 512, 512, 1, 128, 128, 64, 2, 2), tsg.EINVAL, "2^31"),
    ((512, 512, 1 << 23, 1, 256, 256, 64, 2, 2), tsg.EUNSUPPORTED, "exceeds 2^31"),
])
def test_create_rejects(args, code, needle):
    lib = tsg.load()
    h = lib.tsgemm_create(*args)
    assert not h
    assert needle in tsg.last_error()
    assert lib.tsgemm_last_error_code() == code
    with pytest.raises(tsg.TsgemmError) as e:
        tsg.Plan(*args)
    assert e.value.code == code


def test_error_code_clears_on_success():
    lib = tsg.load()
    assert not lib.tsgemm_create(512, 512, 512, 9, 128, 128, 64, 2, 2)
    assert lib.tsgemm_last_error_code() == tsg.EINVAL
    h = lib.tsgemm_create(512, 512, 512, 1, 128, 128, 64, 2, 2)
    assert h and lib.tsgemm_last_error_code() == tsg.OK and tsg.last_error() == ""
    lib.tsgemm_destroy(h)


@pytest.mark.parametrize("cs", [1, 2, 3])
def test_launch_info_explicit_grid_needs_no_device(cs):
    """With an explicit worker count the grid comes from the plan alone: P and
    the busiest worker's waves ceil(ceil(m_blocks/cs) * n_blocks / (P/cs))."""
    p = tsg.Plan(7 * 128 - 40, 6 * 128, 256, "fp16", 128, 128, 64, 4, 2, num_workgroups=6 * cs, cluster_size=cs)
    lib = tsg.load()
    P, it = ctypes.c_int32(), ctypes.c_int32()
    assert lib.tsgemm_launch_info(p._h, ctypes.byref(P), ctypes.byref(it), None) == tsg.OK
    want = -(-(-(-7 // cs) * 6) // 6)
    assert (P.value, it.value) == (6 * cs, want)
    assert p.trace_rows() == 6 * cs * want
    q = tsg.Plan(512, 512, 512, "fp16", 128, 128, 64, 2, 2, num_workgroups=5, cluster_size=2)
    assert lib.tsgemm_launch_info(q._h, ctypes.byref(P), None, None) == tsg.EINVAL
    assert "clusters" in tsg.last_error()


def test_mx_plan_info_and_dtype_mismatch():
    """An MXFP8 plan: stage = A and B slabs (256 x 128 bytes each) plus 4 scale
    bytes per row; tsgemm_run refuses it and tsgemm_run_mx refuses an fp16
    plan, both before any HIP call."""
    lib = tsg.load()
    p = tsg.Plan(1000, 520, 384, "mxfp8", 256, 256, 128, 8, 3, num_workgroups=6)
    inf = p.info()
    assert (inf["dtype"], inf["lds_slots"], inf["stage_bytes"], inf["lds_bytes"]) == (3, 2, 67584, 135168)
    assert (inf["m_blocks"], inf["n_blocks"], inf["k_blocks"], inf["waves"]) == (4, 3, 3, 2)
    assert inf["threads_per_workgroup"] == 256
    assert lib.tsgemm_run(p._h, None, None, None, None) == tsg.EINVAL
    assert "tsgemm_run_mx" in tsg.last_error()
    with pytest.raises(tsg.TsgemmError):
        tsg.Plan(1000, 520, 384, "mxfp8", 256, 256, 128, 8, 2, waves=8)
    q = tsg.Plan(512, 512, 512, "fp16", 128, 128, 64, 2, 2)
    assert lib.tsgemm_run_mx(q._h, None, None, None, None, None, None) == tsg.EINVAL
    assert "MXFP8" in tsg.last_error()
    assert lib.tsgemm_run_mx_traced(p._h, None, None, None, None, None, None, None) == tsg.EINVAL
    assert "trace" in tsg.last_error()
    assert p.trace_rows() == 6 * 2
    # packed scale arrays: blocks x ceil(k_blocks / 4) groups x 256 rows x 16 bytes
    assert p.mx_packed_scale_bytes(0) == 4 * 1 * 4096 and p.mx_packed_scale_bytes(1) == 3 * 1 * 4096
    big = tsg.Plan(8192, 8192, 8192, "mxfp8", 256, 256, 128, 8, 2)
    assert big.mx_packed_scale_bytes(0) == 32 * 16 * 4096 == 8192 * 8192 // 32
    assert lib.tsgemm_mx_packed_scale_bytes(p._h, 2) == tsg.EINVAL
    assert lib.tsgemm_mx_packed_scale_bytes(q._h, 0) == tsg.EINVAL
    assert lib.tsgemm_mx_pack_scales(p._h, 0, None, None, None) == tsg.EINVAL
    assert lib.tsgemm_run_mx_packed(q._h, None, None, None, None, None, None) == tsg.EINVAL


def test_set_epilogue_validation_and_info():
    lib = tsg.load()
    p = tsg.Plan(1024, 1024, 1024, "bf16", 256, 256, 64, 4, 3)
    assert p.info()["store_block_N"] == 0 and p.info()["lds_bytes"] == 2 * 65536
    assert lib.tsgemm_set_epilogue(p._h, 32) == tsg.EINVAL
    assert lib.tsgemm_set_epilogue(p._h, 64) == tsg.OK
    inf = p.info()
    assert (inf["store_block_N"], inf["lds_slots"], inf["lds_bytes"]) == (64, 2, 2 * 65536 + 256 * 128)
    assert lib.tsgemm_set_waves(p._h, 8) == tsg.EUNSUPPORTED          # chunked epilogue: 4 waves only
    assert lib.tsgemm_set_epilogue(p._h, 0) == tsg.OK and p.info()["store_block_N"] == 0
    q = tsg.Plan(1024, 1024, 1024, "fp16", 128, 128, 64, 4, 5)
    assert q.info()["lds_slots"] == 5
    assert lib.tsgemm_set_epilogue(q._h, 64) == tsg.OK
    assert (q.info()["lds_slots"], q.info()["lds_bytes"]) == (4, 4 * 32768 + 128 * 128)   # ring gives up a slot
    w8 = tsg.Plan(1024, 1024, 1024, "bf16", 256, 256, 64, 4, 3, waves=8)
    assert lib.tsgemm_set_epilogue(w8._h, 64) == tsg.EUNSUPPORTED
    mx = tsg.Plan(1024, 1024, 1024, "mxfp8", 256, 256, 128, 4, 2)
    assert lib.tsgemm_set_epilogue(mx._h, 64) == tsg.EUNSUPPORTED
    assert lib.tsgemm_set_epilogue(mx._h, 0) == tsg.OK


def test_null_plan_calls_fail_cleanly():
    lib = tsg.load()
    assert lib.tsgemm_num_tiles(None) == tsg.EINVAL
    assert lib.tsgemm_set_num_workgroups(None, 4) == tsg.EINVAL
    assert lib.tsgemm_run(None, None, None, None, None) == tsg.EINVAL
    assert "NULL" in tsg.last_error()
    lib.tsgemm_destroy(None)


def test_run_rejects_bad_pointers_before_any_launch():
    plan = tsg.Plan(256, 256, 256, "fp16", 128, 128, 64, 2, 2, num_workgroups=4)
    lib = tsg.load()
    assert lib.tsgemm_run(plan._h, 16, 32, None, None) == tsg.EINVAL       # C NULL
    assert lib.tsgemm_run(plan._h, 16, 0, 48, None) == tsg.EINVAL          # B NULL
    assert lib.tsgemm_run(plan._h, 16, 32, 50, None) == tsg.EINVAL         # misaligned
    assert "aligned" in tsg.last_error()
    # M*N == 0: nothing to do, succeeds without touching pointers
    empty = tsg.Plan(0, 256, 256, "fp16", 128, 128, 64, 2, 2, num_workgroups=4)
    assert lib.tsgemm_run(empty._h, None, None, None, None) == 0


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_plan_info_matches_workload(name):
    w = WORKLOADS[name]
    plan = tsg.Plan(w.M, w.N, w.K, w.dtype, w.block_M, w.block_N, w.block_K, w.group_size,
                    w.num_stages, num_workgroups=w.num_workgroups or 256)
    inf = plan.info()
    mb, nb = -(-w.M // w.block_M), -(-w.N // w.block_N)
    assert (inf["m_blocks"], inf["n_blocks"], inf["k_blocks"]) == (mb, nb, w.K // w.block_K)
    assert inf["num_tiles"] == mb * nb == plan.num_tiles
    P = w.num_workgroups or 256
    assert inf["num_workgroups"] == P and inf["waves"] == -(-mb * nb // P)
    stage = (w.block_M * w.block_K + w.block_K * w.block_N) * 2
    assert inf["stage_bytes"] == stage
    assert inf["lds_slots"] == min(w.num_stages, 160 * 1024 // stage, 5)
    assert inf["lds_bytes"] <= 160 * 1024 and inf["lds_slots"] >= 2
    assert inf["threads_per_workgroup"] == 256


@pytest.mark.parametrize("tile", [(128, 128, 32), (128, 128, 64), (256, 256, 32), (256, 256, 64)])
def test_set_waves(tile):
    """8 waves (2x4 grid, two per SIMD) run the same LDS ring; bad counts are refused."""
    bm, bn, bk = tile
    lib = tsg.load()
    plan = tsg.Plan(1024, 1024, 512, "bf16", bm, bn, bk, 4, 3)
    base = plan.info()
    assert lib.tsgemm_set_waves(plan._h, 8) == 0
    inf = plan.info()
    assert inf["threads_per_workgroup"] == 512
    assert (inf["lds_slots"], inf["lds_bytes"]) == (base["lds_slots"], base["lds_bytes"])
    assert lib.tsgemm_set_waves(plan._h, 6) == tsg.EINVAL and "waves" in tsg.last_error()
    assert plan.info()["threads_per_workgroup"] == 512  # a refused call leaves the plan as it was
    assert lib.tsgemm_set_waves(plan._h, 0) == 0 and plan.info()["threads_per_workgroup"] == 256


def test_sm90_stage_arithmetic():
    """The page's lowered sm_90 GEMM (128x128x32 fp16, 3 stages) reserves 49152 bytes
    of dynamic shared memory: 3 * (128*32 + 32*128) * 2.  Same shape here."""
    plan = tsg.Plan(1024, 1024, 1024, "fp16", 128, 128, 32, 4, 3, num_workgroups=256)
    inf = plan.info()
    assert inf["stage_bytes"] * 3 == 49152 and inf["lds_bytes"] == 49152


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_host_schedule_matches_oracle(name):
    w = WORKLOADS[name]
    P = w.num_workgroups or 256
    plan = tsg.Plan(w.M, w.N, w.K, w.dtype, w.block_M, w.block_N, w.block_K, w.group_size, w.num_stages)
    got = plan.schedule_host(P)
    mb, nb = -(-w.M // w.block_M), -(-w.N // w.block_N)
    want = np.array(oracle.schedule.schedule(P, mb, nb, w.group_size), dtype=np.int32)
    assert np.array_equal(got, want)


def test_host_schedule_sweep_partial_groups():
    rng = np.random.default_rng(5)
    for _ in range(60):
        mb, nb = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        gs, P = int(rng.integers(1, 14)), int(rng.integers(1, 40))
        plan = tsg.Plan(mb * 128, nb * 128, 64, "bf16", 128, 128, 64, gs, 2)
        want = np.array(oracle.schedule.schedule(P, mb, nb, gs), dtype=np.int32)
        assert np.array_equal(plan.schedule_host(P), want), (mb, nb, gs, P)


# ---------------------------------------------------------------- scheduler options
def test_set_schedule_validation_and_info():
    lib = tsg.load()
    plan = tsg.Plan(1000, 1024, 256, "fp16", 128, 128, 64, 4, 2, num_workgroups=12)
    inf = plan.info()
    assert (inf["cluster_size"], inf["column_major"]) == (1, 0)
    assert lib.tsgemm_set_schedule(plan._h, 2, 1) == tsg.EINVAL
    assert lib.tsgemm_set_schedule(plan._h, 0, 0) == tsg.EINVAL and "cluster_size" in tsg.last_error()
    assert lib.tsgemm_set_schedule(plan._h, 1, 3) == 0
    inf = plan.info()
    assert (inf["cluster_size"], inf["column_major"]) == (3, 1)
    # 8 x 8 blocks, clusters of 3 -> 3 cluster rows x 8 = 24 cluster tiles over 4 clusters
    assert inf["waves"] == 6
    out = (ctypes.c_int32 * (4 * plan.num_tiles))()
    assert lib.tsgemm_schedule_host(plan._h, 10, out) == tsg.EINVAL and "clusters of 3" in tsg.last_error()


@pytest.mark.parametrize("cs", [1, 2, 3, 4])
@pytest.mark.parametrize("cm", [False, True])
def test_host_schedule_options_match_oracle(cs, cm):
    rng = np.random.default_rng(100 + 10 * cs + cm)
    for _ in range(40):
        mb, nb = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        gs, P = int(rng.integers(1, 14)), cs * int(rng.integers(1, 12))
        plan = tsg.Plan(mb * 128, nb * 128, 64, "bf16", 128, 128, 64, gs, 2, column_major=cm, cluster_size=cs)
        want = np.array(oracle.schedule.schedule(P, mb, nb, gs, column_major=cm, cluster_size=cs), dtype=np.int32)
        assert np.array_equal(plan.schedule_host(P), want), (mb, nb, gs, P, cs, cm)


@pytest.mark.parametrize("P,X", [(256, 8), (255, 8), (8, 8), (3, 8), (300, 8), (64, 1), (97, 4)])
def test_worker_numbering_is_a_balanced_permutation(P, X):
    """Workgroup b runs on XCD b % X.  The numbering must be a permutation of
    the worker ids; every XCD must hold contiguous runs of them; and the first
    A ids (the workers that have tiles) must be split over the XCDs as evenly
    as possible, so a problem with fewer tiles than workgroups still uses
    every XCD's L2."""
    for A in sorted({1, 2, X - 1 if X > 1 else 1, X, X + 3, P // 3, P // 2, P - 1, P}):
        if not 1 <= A <= P:
            continue
        w = tsg.worker_numbering(P, X, A)
        assert sorted(w.tolist()) == list(range(P)), (P, X, A)
        if X == 1:
            assert w.tolist() == list(range(P))
            continue
        per_xcd = [w[x::X] for x in range(X)]
        counts = [int((ids < A).sum()) for ids in per_xcd]
        assert max(counts) - min(counts) <= 1 and sum(counts) == A, (P, X, A, counts)
        for ids in per_xcd:
            act, idle = ids[ids < A], ids[ids >= A]
            assert np.all(np.diff(act) == 1) and np.all(np.diff(idle) == 1)   # contiguous runs
            assert np.all(ids[:len(act)] < A)                                 # active slots first
    with pytest.raises(tsg.TsgemmError):
        tsg.worker_numbering(P, X, 0)


def test_set_l2_prefetch_validation_and_info():
    lib = tsg.load()
    p = tsg.Plan(1024, 1024, 1024, "fp16", 128, 128, 32, 4, 3)
    assert p.info()["l2_prefetch"] == 1  # on by default for fp16/bf16 plans
    assert lib.tsgemm_set_l2_prefetch(p._h, 0) == tsg.OK and p.info()["l2_prefetch"] == 0
    assert lib.tsgemm_set_l2_prefetch(p._h, 1) == tsg.OK and p.info()["l2_prefetch"] == 1
    for bad in (-1, 2):
        assert lib.tsgemm_set_l2_prefetch(p._h, bad) == tsg.EINVAL
        assert "0 or 1" in tsg.last_error()
    assert lib.tsgemm_set_l2_prefetch(None, 1) == tsg.EINVAL
    assert tsg.Plan(1024, 1024, 1024, "fp16", 128, 128, 32, 4, 3, l2_prefetch=False).info()["l2_prefetch"] == 0
    mx = tsg.Plan(512, 512, 512, "mxfp8", 256, 256, 128, 2, 2)
    assert mx.info()["l2_prefetch"] == 0
    assert lib.tsgemm_set_l2_prefetch(mx._h, 0) == tsg.OK
    assert lib.tsgemm_set_l2_prefetch(mx._h, 1) == tsg.EUNSUPPORTED


def test_info_struct_layout_matches_header(tmp_path):
    """The binding's tsgemm_info mirrors the C struct: every field at the
    offset, and the struct at the size, a C compiler gives the header's."""
    fields = [name for name, _ in tsg.Info._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"tsgemm.h\"\nint main(void) {\n"
                   + "".join(f'    printf("{f} %zu\\n", offsetof(tsgemm_info, {f}));\n' for f in fields)
                   + '    printf("sizeof %zu\\n", sizeof(tsgemm_info));\n    return 0;\n}\n')
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    for f in fields:
        assert int(out[f]) == getattr(tsg.Info, f).offset, f
    assert int(out["sizeof"]) == ctypes.sizeof(tsg.Info)
