"""GPU parity of the block-scaled FP8 (MX) GEMM: tsgemm_run_mx through the C ABI
against the CPU oracle (oracle_mx.c).

Tolerance.  The oracle gives the exact product C64 (binary64, every term exact)
and, from sign-cleared codes, the magnitude sum mag = sum_k |terms|.  The
matrix core adds the scaled products of one instruction with a small internal
error (measured on adversarial inputs spanning 2^-31 .. 2^30: at most about
2^-12.3 of that instruction's magnitude sum), the partial sums accumulate in
fp32 (K/64 additions, relative 2^-24 each) and the result is rounded once to
bf16 (at most 2^-8 relative).  Hence, elementwise,

    |C - C64| <= 2^-8 * |C64| + 2^-10 * mag,

with a margin of 4x on the internal error.  Where every partial sum is exactly
representable (small integer elements, scales near one) the kernel must match
the once-rounded oracle bit for bit.  Schedules (the kernel's own trace) must
match the oracle bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import persistent_tile_scheduled_amd as tsg
from workloads import MX_WORKLOADS, make_mx_inputs, mx_workload_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL_REL, TOL_MAG = 2.0 ** -8, 2.0 ** -10


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _plan(M, N, K, P=0, gs=8, column_major=False, cluster_size=1):
    return tsg.Plan(M, N, K, "mxfp8", 256, 256, 128, gs, 2, num_workgroups=P,
                    column_major=column_major, cluster_size=cluster_size)


def _run(plan, A, SFA, B, SFB, guard=64):
    """C inside a NaN-filled buffer with `guard` sentinels after it."""
    M, N = plan.M, plan.N
    dev = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (A, SFA, B, SFB)]
    buf = torch.full((M * N + guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    C = buf[: M * N].view(M, N)
    plan.run_mx(*dev, C)
    torch.cuda.synchronize()
    assert torch.isnan(buf[M * N:].float()).all(), "write past the end of C"
    return C.cpu().double().numpy()


def _mag(A, SFA, B, SFB):
    return oracle.mx_gemm_f64(A & 0x7F, SFA, B & 0x7F, SFB)


def _check_bound(got, c64, mag, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output (unwritten tile?)"
    err = np.abs(got - c64)
    bound = TOL_REL * np.abs(c64) + TOL_MAG * mag
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[:5].tolist()}, "
                           f"worst err/bound {(err / np.maximum(bound, 1e-300)).max():.3g}")
    fro = np.linalg.norm(got - c64) / max(np.linalg.norm(c64), 1e-300)
    assert fro <= 2.0 ** -8, f"{what}: relative Frobenius error {fro}"
    return float((err / np.maximum(mag, 1e-300)).max()), float(fro)


def _int_codes(rng, shape):
    # E4M3 codes of the integers -2..2 (0xC0 = -2, 0xB8 = -1, 0x00, 0x38 = 1, 0x40 = 2)
    return rng.choice(np.array([0xC0, 0xB8, 0x00, 0x38, 0x40], np.uint8), size=shape)


# ---------------------------------------------------------------- bit-exact cases
@pytest.mark.parametrize("scales", ["unit", "pow2"])
def test_mx_bit_exact_when_sums_are_exact(scales):
    """Integer elements in [-2, 2]; scales 2^0 (unit) or 2^-1..2^1 (pow2): every
    partial sum is a short dyadic number, so the result is the exact product
    rounded once to bf16.  Any mis-paired k, wrong block scale or misplaced
    row/column shows up as a bit difference."""
    rng = np.random.default_rng(21)
    M, N, K = 300, 264, 384           # 2x2 tiles, both ragged; 3 slabs
    print(f"[case] bit-exact {scales} {M}x{N}x{K}", flush=True)
    A, B = _int_codes(rng, (M, K)), _int_codes(rng, (N, K))
    if scales == "unit":
        SFA = np.full((M, K // 32), 127, np.uint8)
        SFB = np.full((N, K // 32), 127, np.uint8)
    else:
        SFA = rng.integers(126, 129, (M, K // 32)).astype(np.uint8)
        SFB = rng.integers(126, 129, (N, K // 32)).astype(np.uint8)
    got = _run(_plan(M, N, K, P=3, gs=1), A, SFA, B, SFB)
    ref_bits, _ = oracle.mx_reference_c(A, SFA, B, SFB, oracle.BF16)
    ref = _bf16_bits_to_f64(ref_bits)
    diff = np.argwhere(got != ref)
    assert len(diff) == 0, f"{len(diff)} elements differ, first {diff[:5].tolist()}"


# ---------------------------------------------------------------- random MX data
MX_CASES = [
    # M, N, K, spread, P, group, column_major, cluster
    (256, 256, 128, 0, 1, 8, False, 1),      # one tile, one slab
    (512, 512, 512, 0, 4, 2, False, 1),
    (1000, 520, 384, 3, 5, 8, False, 1),     # ragged rows and columns, odd slab count
    (300, 1032, 1024, 8, 2, 3, True, 2),     # wide scale spread, column-major, clusters of 2
    (777, 264, 256, 2, 6, 1, False, 3),      # clusters of 3 over 4 row blocks: some ranks idle
    (768, 768, 128, 1, 2, 2, False, 1),      # one slab per tile, 4-5 tiles per worker
    (768, 520, 256, 1, 2, 3, False, 1),      # two slabs per tile, ragged columns, 4-5 tiles per worker
]


@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_s{c[3]}_P{c[4]}")
def test_mx_random_full_compare(case):
    M, N, K, spread, P, gs, cm, cs = case
    print(f"[case] mx {case}", flush=True)
    A, SFA, B, SFB = make_mx_inputs(M, N, K, seed=M + N + K, spread=spread)
    got = _run(_plan(M, N, K, P=P, gs=gs, column_major=cm, cluster_size=cs), A, SFA, B, SFB)
    c64 = oracle.mx_gemm_f64(A, SFA, B, SFB)
    worst, fro = _check_bound(got, c64, _mag(A, SFA, B, SFB), f"mx {case}")
    print(f"  max err/mag {worst:.3g}, rel Frobenius {fro:.3g}", flush=True)


def test_mx_trace_matches_oracle_schedule():
    M, N, K, P = 7 * 256 - 40, 5 * 256, 256, 6
    for cm, cs in [(False, 1), (True, 1), (False, 2), (True, 3)]:
        print(f"[case] mx trace column_major={cm} cluster={cs}", flush=True)
        plan = _plan(M, N, K, P=P * cs, gs=2, column_major=cm, cluster_size=cs)
        A, SFA, B, SFB = make_mx_inputs(M, N, K, seed=5)
        dev = [torch.from_numpy(x).to(DEV) for x in (A, SFA, B, SFB)]
        C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        trace = torch.full((4 * plan.trace_rows(),), -1, dtype=torch.int32, device=DEV)
        plan.run_mx_traced(*dev, C, trace)
        torch.cuda.synchronize()
        rows = trace.cpu().numpy().reshape(-1, 4)
        rows = rows[rows[:, 0] >= 0]
        want = np.array(oracle.schedule.schedule(P * cs, plan.info()["m_blocks"], plan.info()["n_blocks"], 2,
                                                 column_major=cm, cluster_size=cs), dtype=np.int32)
        assert np.array_equal(rows, want)
        _check_bound(C.cpu().double().numpy(), oracle.mx_gemm_f64(A, SFA, B, SFB), _mag(A, SFA, B, SFB),
                     f"traced cm={cm} cs={cs}")


# ---------------------------------------------------------------- packed scales
def _pack_reference(SF, rows, K):
    """The packed layout of tsgemm_mx_pack_scales written out directly:
    [256-row block][group of 16 scale bytes][256 rows][16], zeros past the data."""
    kb = K // 32
    blocks, groups = -(-rows // 256), -(-(K // 128) // 4)
    out = np.zeros((blocks, groups, 256, 16), np.uint8)
    for b in range(blocks):
        for g in range(groups):
            r0, r1 = b * 256, min(rows, b * 256 + 256)
            c0, c1 = g * 16, min(kb, g * 16 + 16)
            out[b, g, : r1 - r0, : c1 - c0] = SF[r0:r1, c0:c1]
    return out.reshape(-1)


@pytest.mark.parametrize("shape", [(300, 264, 384), (520, 776, 1152), (256, 256, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_packed_scales_layout_and_bit_identical_result(shape):
    """tsgemm_mx_pack_scales writes exactly the documented permutation, and
    tsgemm_run_mx_packed on it returns C bit for bit equal to tsgemm_run_mx
    (same products, same order), within the bound of the oracle."""
    M, N, K = shape
    print(f"[case] mx packed {shape}", flush=True)
    A, SFA, B, SFB = make_mx_inputs(M, N, K, seed=K + 1, spread=3)
    plan = _plan(M, N, K, P=5, gs=2)
    dev = [torch.from_numpy(x).to(DEV) for x in (A, SFA, B, SFB)]
    packed = []
    for op, (sf, rows) in enumerate(((dev[1], M), (dev[3], N))):
        sfp = torch.full((plan.mx_packed_scale_bytes(op),), 0xAB, dtype=torch.uint8, device=DEV)
        plan.mx_pack_scales(sf, sfp, op)
        torch.cuda.synchronize()
        assert np.array_equal(sfp.cpu().numpy(), _pack_reference((SFA, SFB)[op], rows, K)), f"operand {op}"
        packed.append(sfp)
    C1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    C2 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    plan.run_mx(*dev, C1)
    plan.run_mx_packed(dev[0], packed[0], dev[2], packed[1], C2)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    _check_bound(C2.cpu().double().numpy(), oracle.mx_gemm_f64(A, SFA, B, SFB), _mag(A, SFA, B, SFB),
                 f"packed {shape}")


# ---------------------------------------------------------------- edge cases
def test_mx_empty_and_zero_k():
    z = torch.zeros(0, dtype=torch.uint8, device=DEV)
    plan = _plan(0, 256, 128)
    plan.run_mx(z.view(0, 128), z.view(0, 4), torch.zeros((256, 128), dtype=torch.uint8, device=DEV),
                torch.zeros((256, 4), dtype=torch.uint8, device=DEV), torch.empty((0, 256), dtype=torch.bfloat16, device=DEV))
    plan = _plan(300, 264, 0)
    C = torch.full((300, 264), float("nan"), dtype=torch.bfloat16, device=DEV)
    e = torch.empty((300, 0), dtype=torch.uint8, device=DEV)
    plan.run_mx(e, e, torch.empty((264, 0), dtype=torch.uint8, device=DEV),
                torch.empty((264, 0), dtype=torch.uint8, device=DEV), C)
    torch.cuda.synchronize()
    assert (C.float() == 0).all()


def test_mx_nan_codes_propagate():
    """OCP MX: a NaN scale (0xFF) makes its whole block NaN, and an E4M3 NaN
    element (S.1111.111) its product.  The rows/columns they touch are NaN in
    the oracle; the kernel must agree on which outputs are NaN."""
    rng = np.random.default_rng(9)
    M, N, K = 256, 256, 256
    A, SFA, B, SFB = make_mx_inputs(M, N, K, seed=9)
    SFA[3, 5] = 0xFF          # row 3 of C
    A[77, 200] = 0x7F         # row 77
    B[140, 17] = 0xFF         # column 140 (negative-signed NaN code)
    SFB[250, 0] = 0xFF        # column 250
    print("[case] mx NaN propagation", flush=True)
    got = _run(_plan(M, N, K, P=1), A, SFA, B, SFB)
    c64 = oracle.mx_gemm_f64(A, SFA, B, SFB)
    assert np.array_equal(np.isnan(got), np.isnan(c64)), \
        f"NaN pattern differs: kernel {np.isnan(got).sum()} NaNs, oracle {np.isnan(c64).sum()}"
    fin = ~np.isnan(c64)
    assert np.all(np.abs(got[fin] - c64[fin]) <= TOL_REL * np.abs(c64[fin]) + TOL_MAG * _mag(A, SFA, B, SFB)[fin])


# ---------------------------------------------------------------- full size, every element
_MX_FULL = {}


def _mx_full_reference(name):
    """Inputs, the oracle's exact product C64, its magnitude sum and C64 rounded
    once to bf16, for one benchmark shape (kept for the next test)."""
    if name not in _MX_FULL:
        _MX_FULL.clear()
        A, SFA, B, SFB = mx_workload_inputs(MX_WORKLOADS[name])
        c64 = oracle.mx_gemm_f64(A, SFA, B, SFB)
        mag = _mag(A, SFA, B, SFB)
        cref = _bf16_bits_to_f64(oracle.round_to(c64, oracle.BF16))
        _MX_FULL[name] = (A, SFA, B, SFB, c64, mag, cref)
    return _MX_FULL[name]


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("name", list(MX_WORKLOADS))
def test_mx_full_size_every_element(name, packed):
    """The benchmarked shape in the launch configuration the benchmark times
    (one workgroup per CU, XCD remap on; scales row-major or packed on the
    device first): every element of C within the bound against the oracle's
    whole product, and the relative Frobenius error against the once-rounded
    oracle over all of C within 1e-3 (the fp16/bf16 criterion; the bf16
    rounding of the exact product alone would use most of it, hence the
    rounded reference)."""
    w = MX_WORKLOADS[name]
    print(f"[case] mx full size {name} packed={packed}", flush=True)
    A, SFA, B, SFB, c64, mag, cref = _mx_full_reference(name)
    plan = _plan(w.M, w.N, w.K, P=w.num_workgroups, gs=w.group_size)
    if packed:
        dev = [torch.from_numpy(x).to(DEV) for x in (A, SFA, B, SFB)]
        sfp = [torch.empty((plan.mx_packed_scale_bytes(op),), dtype=torch.uint8, device=DEV) for op in (0, 1)]
        plan.mx_pack_scales(dev[1], sfp[0], 0)
        plan.mx_pack_scales(dev[3], sfp[1], 1)
        buf = torch.full((w.M * w.N + 256,), float("nan"), dtype=torch.bfloat16, device=DEV)
        plan.run_mx_packed(dev[0], sfp[0], dev[2], sfp[1], buf[: w.M * w.N].view(w.M, w.N))
        torch.cuda.synchronize()
        assert torch.isnan(buf[w.M * w.N:].float()).all(), "write past the end of C"
        got = buf[: w.M * w.N].view(w.M, w.N).cpu().double().numpy()
    else:
        got = _run(plan, A, SFA, B, SFB, guard=256)
    assert np.all(np.isfinite(got)), "non-finite output (unwritten tile?)"
    err = np.abs(got - c64)
    bound = TOL_REL * np.abs(c64) + TOL_MAG * mag
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of the bound, first {bad[:5].tolist()}"
    fro = np.linalg.norm(got - cref) / np.linalg.norm(cref)
    assert fro <= 1e-3, f"relative Frobenius error {fro}"
    d2, r2 = (got - cref) ** 2, cref ** 2
    row = np.sqrt(d2.sum(axis=1) / r2.sum(axis=1)).max()
    col = np.sqrt(d2.sum(axis=0) / r2.sum(axis=0)).max()
    # per row and column (2e-3): one wrong block scale moves its whole row of C by ~6%
    assert row <= 2e-3 and col <= 2e-3, f"worst row {row}, worst column {col}"
    print(f"  max err/bound {(err / bound).max():.3g}, max err/mag {(err / mag).max():.3g}, "
          f"rel. Frobenius vs rounded oracle {fro:.3g} (vs exact {np.linalg.norm(got - c64) / np.linalg.norm(c64):.3g}), "
          f"worst row {row:.3g}, worst column {col:.3g}", flush=True)
