// Persistent, tile-scheduled block-scaled FP8 (MX) GEMM for gfx950 (CDNA4).
//
//   C[m,n] = sum_k x(A[m,k]) * s(SFA[m,k/32]) * x(B[n,k]) * s(SFB[n,k/32])
//
// x() decodes an OCP FP8 E4M3 element, s() an OCP E8M0 scale (2^(e-127)); a
// scale covers 32 consecutive elements along K (OCP Microscaling Formats
// specification v1.0).  The page "[Feature] Introduce tile scheduler #2441"
// lists an MXFP8 block-scaled persistent GEMM among its examples (PR overview,
// changed files: blockscaled_gemm ... mxfp8 ... 1d1d) driven by the same tile
// scheduler, without printing its layouts; the layout here is the plain "1d1d"
// reading: A[M][K] and B[N][K] K-contiguous bytes, SFA[M][K/32] and
// SFB[N][K/32] scale bytes, C[M][N] bf16, fp32 accumulation.
//
// Same structure as the fp16/bf16 kernel: persistent workers on one
// `while valid()` loop over their tiles, a loader running one LDS stage ahead
// with its own scheduler copy, buffer_load ... lds DMA with range-checked
// descriptors (zero fill past the matrix), XOR-swizzled 16-byte LDS chunks.
// Specific to this kernel:
//   * math: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, one E8M0 scale per
//     operand row and 32-deep block); 4 waves in a 2x2 grid, each a 128x128
//     sub-tile = 4x4 blocks of 32x32, all 256 AGPRs as accumulators;
//   * tile 256x256, 128-deep slabs: a stage holds A and B (256 rows x 128
//     bytes each), 64 KiB; two stages.  Scale bytes travel separately, once
//     per group of SG slabs (4 * SG bytes per row: one 16-byte DMA lane per
//     row and 4 slabs) into a two-entry scale ring: fetching them per slab
//     (4 bytes from each of 256 rows, a cache line per lane) cost as much
//     address-unit work as the A and B slabs themselves;
//   * operand layout of the instruction: lane l supplies row l%32; its bytes
//     0-15 are k = 16*(l/32) + 0..15 of the 64-deep step and bytes 16-31 are
//     k = 32 + 16*(l/32) + 0..15; lane l also supplies the scale of row l%32
//     for the step's 32-deep block l/32.  A fragment is therefore two 16-byte
//     LDS reads and a scale one LDS byte read (no register shuffling);
//   * B is the instruction's first operand, so a lane's 16 results run along
//     N.  Its rows are permuted (src row rho -> column pi(rho)) so that a lane
//     holds two runs of 8 consecutive columns and the epilogue writes 16-byte
//     pieces, 32 contiguous bytes per C row and store instruction.
#pragma once

#include "tile_scheduler.h"
#include "tsgemm_device.h"

namespace tsg {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

struct MxArgs {
    const uint8_t* A;    // [M][K] E4M3
    const uint8_t* SFA;  // [M][K/32] E8M0, or packed (see tsgemm_mx_pack_kernel)
    const uint8_t* B;    // [N][K] E4M3
    const uint8_t* SFB;  // [N][K/32] E8M0, or packed
    uint16_t* C;         // [M][N] bf16
    int32_t* trace;      // optional (worker, iter, m, n) per processed tile
    int64_t M, N, K;
    uint32_t m_blocks, n_blocks, k_blocks, group;
    uint32_t P, max_iters, num_xcd;
    uint32_t num_active;  // workers with at least one tile (worker numbering)
    uint32_t cluster, col_major;
    uint32_t n_groups;   // scale groups per tile: ceil(k_blocks / SG)
};

// acc += src0 x src1 with per-row E8M0 scales (byte 0 of each scale
// register, op_sel 0), both operands E4M3.  Accumulator constrained to AGPRs
// as in the fp16/bf16 kernel.  The leading s_nop 1 covers the wait state an
// MFMA needs after a VALU write of one of its source or scale VGPRs (gfx950
// code generation places one, s_nop 0, for that pair): the compiler
// zero-extends the scale bytes with VALU ops it may place right before this
// asm, and it pads only instructions it knows to be MFMAs.  Reading a result
// needs 20 wait states after this 64-cycle MFMA; the epilogue reads a block
// four MFMAs after its last one.
__device__ __forceinline__ void mfma_mx32(f32x16& acc, i32x8 src0, i32x8 src1, uint32_t s0, uint32_t s1) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(acc) : "v"(src0), "v"(src1), "v"(s0), "v"(s1));
}

// The same MFMA with a zero accumulator input (the k == 0 clear).
__device__ __forceinline__ void mfma_mx32_clear(f32x16& acc, i32x8 src0, i32x8 src1, uint32_t s0, uint32_t s1) {
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
                 : "=a"(acc) : "v"(src0), "v"(src1), "v"(s0), "v"(s1));
}

#ifndef TSG_MX_SG
#define TSG_MX_SG 4
#endif
#ifndef TSG_MX_DMA_FIRST
#define TSG_MX_DMA_FIRST 11  // data DMAs of a slab issued in its first k-step of issue (of 16)
#endif
struct MxTraits {
    static constexpr int BM = 256, BN = 256, BK = 128, L = 2;
    static constexpr int THREADS = 256;           // 4 waves, 2 x 2
    static constexpr int WM = 128, WN = 128;      // wave sub-tile
    static constexpr int F = 4;                   // 32x32 blocks per wave side
    static constexpr int A_BYTES = BM * BK;       // 32 KiB
    static constexpr int B_BYTES = BN * BK;       // 32 KiB
    static constexpr int STAGE = A_BYTES + B_BYTES;  // 64 KiB
    static constexpr int SG = TSG_MX_SG;          // slabs per scale group
    static constexpr int SC_ROW = 4 * SG;         // scale bytes per row and group
    static constexpr int SC_OFF = STAGE * L;      // scale ring after the stages
    static constexpr int SC_B = BM * SC_ROW;      // B's part of a ring entry
    static constexpr int SC_ENTRY = (BM + BN) * SC_ROW;
    static constexpr int LDS = SC_OFF + 2 * SC_ENTRY;
    static constexpr int NA = A_BYTES / (1024 * 4);  // 16-byte DMAs per wave and slab for A (8)
    static constexpr int NB = B_BYTES / (1024 * 4);  // ... for B (8)
    static constexpr int ND = NA + NB;
    static constexpr int LPR = SG / 4;            // 16-byte DMA lanes per row and group
    static constexpr int NS = LPR;                // scale DMAs per wave and operand and group (64 rows)
    static constexpr int NSC = 2 * NS;
    // data DMAs of a slab issued in the LAST k-step of the slab two back (with
    // the scale DMAs); the remaining ND - DF go out during the next k-step
    static constexpr int DF = (TSG_MX_DMA_FIRST > 0 && TSG_MX_DMA_FIRST < ND) ? TSG_MX_DMA_FIRST : ND;
    static_assert(SG == 4 || SG == 8, "scale group");
    static_assert(L == 2, "the slabs' DMA counts vary (scale groups): every wait is for all of them");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(BM / 4 == 64 && BN / 4 == 64, "64 scale rows per wave and operand");
};
#ifndef TSG_MX_GAP
#define TSG_MX_GAP 2
#endif
#ifndef TSG_MX_S0
#define TSG_MX_S0 2
#endif
#ifndef TSG_MX_SCALES_FIRST
#define TSG_MX_SCALES_FIRST 1
#endif
constexpr int kMxGap = TSG_MX_GAP;  // MFMAs (64 cycles each) between the last read of a fragment set and its refill
constexpr int kMxS0 = TSG_MX_S0;    // MFMAs a slab's last k-step issues before its wait and barrier

// Column of B (within a 32-column block) that instruction row rho carries:
// rho = 8j + 4h + t  ->  16*(j/2) + 8h + 4*(j%2) + t.  A lane of the result
// with half h then holds columns 8h + 0..7 (values 0-7) and 16 + 8h + 0..7
// (values 8-15).
__device__ __forceinline__ uint32_t mx_col_of_row(uint32_t rho) {
    return 16u * (rho >> 4) + 8u * ((rho >> 2) & 1u) + 4u * ((rho >> 3) & 1u) + (rho & 3u);
}

// Swizzled slot of logical 16-byte chunk c in an LDS row is c ^ swz(row).
// A fragment read has lanes 0-31 on 32 consecutive rows (B: rows pi(rho))
// at one chunk and lanes 32-63 on the same rows at the next chunk.  On
// gfx950 such a 16-byte-per-lane read is conflict-free only if, besides rows
// 0-7 spreading over the 8 slots, rows r and r + 8 also land on different
// slots (measured with the LDS bank-conflict counter: row & 7 alone costs a
// 2-way conflict on every read).  A rows therefore use (row & 7) ^ bit 3 of
// the row; B rows the same function of rho, i.e. bits 0, 1, 3 of the column
// with bit 2 folded in.
__device__ __forceinline__ uint32_t mx_swz_a(uint32_t m) { return (m & 7u) ^ ((m >> 3) & 1u); }
__device__ __forceinline__ uint32_t mx_swz_b(uint32_t n) { return ((n & 3u) | ((n >> 1) & 4u)) ^ ((n >> 2) & 1u); }

// PACKED: SFA and SFB come in the tile-blocked layout of tsgemm_mx_pack_kernel,
// so a wave's share of a scale group is 64 * SC_ROW contiguous bytes (one or two
// cache lines per 8 lanes) instead of 64 rows' worth of separate cache lines.
template <bool PACKED>
__global__ __launch_bounds__(256, 1) void tsgemm_mx_kernel(MxArgs args) {
    using T = MxTraits;
    constexpr int F = T::F, NA = T::NA, NB = T::NB, ND = T::ND, NS = T::NS, NSC = T::NSC, L = T::L;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)smem);

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t stress_ctr = 0;  // race-detection build only (TSG_STRESS)
    const uint32_t wr = wave >> 1, wc = wave & 1u;
    const uint32_t N = (uint32_t)args.N, K = (uint32_t)args.K, KB = K / 32u;
    const uint32_t k_blocks = args.k_blocks;
    const uint32_t wid = worker_of_workgroup(blockIdx.x, args.P, args.num_xcd, args.num_active);

    // ---- DMA source offsets (bytes from the slab origin) ----
    // Instruction q of this wave fills 16-byte LDS positions p = (wave*NA + q)*64
    // + lane: stage row p/8 = (wave*NA + q)*8 + lane/8, slot lane%8.  The lane
    // fetches the logical chunk the swizzle puts at that slot (a function of
    // lane/8 and, through bit 3 of the row, of the parity of q).
    uint32_t voff[ND + NS];
    {
        const uint32_t r8 = lane >> 3, slot = lane & 7u;
#pragma unroll
        for (int q = 0; q < NA; ++q) {
            const uint32_t row = (wave * NA + q) * 8u + r8;
            voff[q] = row * K + ((slot ^ mx_swz_a(row)) * 16u);
        }
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const uint32_t row = (wave * NB + q) * 8u + r8;
            voff[NA + q] = row * K + ((slot ^ mx_swz_b(row)) * 16u);
        }
        // scale instruction i: rows wave*64 + i*64/LPR + lane/LPR, 16-byte part
        // lane%LPR of the group's 4*SG bytes (same offsets for SFA and SFB)
#pragma unroll
        for (int i = 0; i < NS; ++i)
            voff[ND + i] = (wave * 64u + i * (64u / T::LPR) + lane / T::LPR) * (PACKED ? (uint32_t)T::SC_ROW : KB) +
                           (lane % T::LPR) * 16u;
    }

    // ---- per-lane LDS read offsets (bytes from the stage origin) ----
    // The instruction lane (h, r): operand row r, byte halves from chunks
    // 4*ks + h (bytes 0-15) and 4*ks + 2 + h (bytes 16-31) of the 8-chunk row.
    const uint32_t h = lane >> 5, r = lane & 31u;
    const uint32_t a_row = wr * T::WM + r;                     // + 32*fm
    const uint32_t b_row = wc * T::WN + mx_col_of_row(r);      // + 32*fn
    uint32_t a_off[2][2], b_off[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t c = 4u * ks + 2u * j + h;
            a_off[ks][j] = a_row * T::BK + ((c ^ mx_swz_a(a_row)) * 16u);
            b_off[ks][j] = T::A_BYTES + b_row * T::BK + ((c ^ mx_swz_b(b_row)) * 16u);
        }
    // scale byte of block 2*ks + h of the row, from the ring entry's record of
    // the row (4 bytes per slab of the group)
    const uint32_t sa_off = a_row * T::SC_ROW + h, sb_off = T::SC_B + b_row * T::SC_ROW + h;

    // ---- loader: its own scheduler copy, L slabs ahead of the math ----
    // Per tile the loader forms the byte addresses of its first slab of A, B
    // (row blocks m and n, column 0) and of their scales, and the ranges the
    // descriptors may span; per slab it only steps them (A and B by BK bytes,
    // row-major scales by BK/32 bytes, packed scales by one group record per
    // group).  The scalar work between two MFMAs is then a few adds and
    // selects: the wave that issues it also issues the MFMAs.
    //   A: range = rows * K - k0 bytes from the slab origin, rows =
    //      min(M - m0, BM): rows past M read zeros and the range never runs
    //      past row m0 + rows - 1 (B likewise with the columns of C);
    //   row-major scales: rows * K/32 - k0/32 bytes (scale bytes of slabs past
    //      K in a partial last group are never read);
    //   packed scales: one 256-row group record.
    // BM*K is below 2^31 (checked when the plan is created).
    TileScheduler ld;
    ld.setup(args.P, args.m_blocks, args.n_blocks, args.group, args.cluster, args.col_major);
    ld.init(wid);
    constexpr uint32_t kGroupBytes = (uint32_t)T::BM * T::SC_ROW;
    const uint32_t M32 = (uint32_t)args.M;
    uint32_t ld_k = 0, ld_slot = 0, ld_grp = 0;
    uint64_t a_ptr = 0, b_ptr = 0, sa_ptr = 0, sb_ptr = 0;
    uint32_t a_num = 0, b_num = 0, sa_num = 0, sb_num = 0, dec = 0, sdec = 0;
    bool ld_live = false;
    i32x4 rs_a, rs_b, rs_sa, rs_sb;
    uint32_t dma_lds = 0, sc_lds = 0, ld_lds = lds_base;
    bool sc_issue = false;

    // ranges for the loader's current tile; zero past the end of the schedule
    // (the data DMAs then write zeros into a stage nobody reads, so every slab
    // issues the same data DMAs)
    auto tile_ranges = [&]() __attribute__((always_inline)) {
        const bool live = ld.valid();
        ld_live = live;
        const uint32_t m0 = ld.m_idx * T::BM, n0 = ld.n_idx * T::BN;
        const uint32_t rows = live ? (M32 - m0 < (uint32_t)T::BM ? M32 - m0 : (uint32_t)T::BM) : 0u;
        const uint32_t cols = live ? (N - n0 < (uint32_t)T::BN ? N - n0 : (uint32_t)T::BN) : 0u;
        a_ptr = reinterpret_cast<uint64_t>(args.A) + (live ? (uint64_t)m0 * K : 0u);
        b_ptr = reinterpret_cast<uint64_t>(args.B) + (live ? (uint64_t)n0 * K : 0u);
        a_num = rows * K;
        b_num = cols * K;
        dec = live ? (uint32_t)T::BK : 0u;
        if constexpr (PACKED) {
            // group g of row block i: 256 rows x SC_ROW bytes at (i * n_groups + g) * 256 * SC_ROW
            sa_ptr = reinterpret_cast<uint64_t>(args.SFA) + (live ? (uint64_t)ld.m_idx * args.n_groups * kGroupBytes : 0u);
            sb_ptr = reinterpret_cast<uint64_t>(args.SFB) + (live ? (uint64_t)ld.n_idx * args.n_groups * kGroupBytes : 0u);
            sa_num = live ? kGroupBytes : 0u;
            sb_num = sa_num;
        } else {
            sa_ptr = reinterpret_cast<uint64_t>(args.SFA) + (live ? (uint64_t)m0 * KB : 0u);
            sb_ptr = reinterpret_cast<uint64_t>(args.SFB) + (live ? (uint64_t)n0 * KB : 0u);
            sa_num = rows * KB;
            sb_num = cols * KB;
            sdec = live ? (uint32_t)T::BK / 32u : 0u;
        }
    };
    // descriptors and LDS targets of the loader's next slab.  A slab that
    // starts a scale group (k % SG == 0) also fetches the group's scales into
    // ring entry (group count) % 2.
    auto slab_desc = [&]() __attribute__((always_inline)) {
        dma_lds = ld_lds;
        sc_issue = ld_live && (ld_k % T::SG) == 0;
        // wave-uniform by construction; readfirstlane keeps it in an SGPR
        // for the DMA's M0 add
        sc_lds = __builtin_amdgcn_readfirstlane(lds_base + T::SC_OFF + (ld_grp & 1u) * T::SC_ENTRY + wave * 64u * T::SC_ROW);
        rs_a = rsrc_words_u64(a_ptr, a_num);
        rs_b = rsrc_words_u64(b_ptr, b_num);
        rs_sa = rsrc_words_u64(sa_ptr, sa_num);
        rs_sb = rsrc_words_u64(sb_ptr, sb_num);
    };
    // step the loader to the slab after
    auto slab_advance = [&]() __attribute__((always_inline)) {
        ld_grp += sc_issue ? 1u : 0u;
        a_ptr += (uint32_t)T::BK;
        a_num -= dec;
        b_ptr += (uint32_t)T::BK;
        b_num -= dec;
        if constexpr (PACKED) {
            if (sc_issue) {
                sa_ptr += kGroupBytes;
                sb_ptr += kGroupBytes;
            }
        } else {
            sa_ptr += (uint32_t)T::BK / 32u;
            sa_num -= sdec;
            sb_ptr += (uint32_t)T::BK / 32u;
            sb_num -= sdec;
        }
        if (++ld_slot == (uint32_t)L) {
            ld_slot = 0;
            ld_lds -= (L - 1) * T::STAGE;
        } else {
            ld_lds += T::STAGE;
        }
        if (++ld_k == k_blocks) {
            ld_k = 0;
            ld.next_tile();
            tile_ranges();
        }
    };
    auto next_slab = [&]() __attribute__((always_inline)) {
        slab_desc();
        slab_advance();
    };
    // In the main loop the same two steps go out in pieces, each between
    // empty volatile asm statements on the registers it reads and writes: a
    // wave issues one instruction every four cycles and the scaled MFMA keeps
    // the matrix core busy for 64, so fifteen instructions fit in a gap, and
    // the compiler would otherwise hoist the descriptor work into the gap
    // before the k-step's first MFMA next to the loop's own scalar work.
    //   desc 0: LDS targets and whether the slab starts a scale group;
    //   desc 1..4: the A, B, SFA and SFB descriptors;
    //   adv 0: the A and B origins and ranges;  adv 1: the scale origins and
    //   ranges and the group count;  adv 2: LDS slot, slab count, next tile.
    auto desc_piece = [&](auto p_c) __attribute__((always_inline)) {
        constexpr int p = decltype(p_c)::value;
        if constexpr (p == 0) {
            asm volatile("" : "+s"(ld_lds), "+s"(ld_k));
            dma_lds = ld_lds;
            sc_issue = ld_live && (ld_k % T::SG) == 0;
            sc_lds = __builtin_amdgcn_readfirstlane(lds_base + T::SC_OFF + (ld_grp & 1u) * T::SC_ENTRY + wave * 64u * T::SC_ROW);
            asm volatile("" : "+s"(dma_lds), "+s"(sc_lds));
        } else if constexpr (p == 1) {
            asm volatile("" : "+s"(a_ptr), "+s"(a_num));
            rs_a = rsrc_words_u64(a_ptr, a_num);
            asm volatile("" : "+s"(rs_a));
        } else if constexpr (p == 2) {
            asm volatile("" : "+s"(b_ptr), "+s"(b_num));
            rs_b = rsrc_words_u64(b_ptr, b_num);
            asm volatile("" : "+s"(rs_b));
        } else if constexpr (p == 3) {
            asm volatile("" : "+s"(sa_ptr), "+s"(sa_num));
            rs_sa = rsrc_words_u64(sa_ptr, sa_num);
            asm volatile("" : "+s"(rs_sa));
        } else {
            asm volatile("" : "+s"(sb_ptr), "+s"(sb_num));
            rs_sb = rsrc_words_u64(sb_ptr, sb_num);
            asm volatile("" : "+s"(rs_sb));
        }
    };
    auto adv_piece = [&](auto p_c) __attribute__((always_inline)) {
        constexpr int p = decltype(p_c)::value;
        if constexpr (p == 0) {
            asm volatile("" : "+s"(a_ptr), "+s"(b_ptr), "+s"(a_num), "+s"(b_num));
            a_ptr += (uint32_t)T::BK;
            a_num -= dec;
            b_ptr += (uint32_t)T::BK;
            b_num -= dec;
            asm volatile("" : "+s"(a_ptr), "+s"(b_ptr), "+s"(a_num), "+s"(b_num));
        } else if constexpr (p == 1) {
            asm volatile("" : "+s"(sa_ptr), "+s"(sb_ptr), "+s"(sa_num), "+s"(sb_num));
            ld_grp += sc_issue ? 1u : 0u;
            if constexpr (PACKED) {
                if (sc_issue) {
                    sa_ptr += kGroupBytes;
                    sb_ptr += kGroupBytes;
                }
            } else {
                sa_ptr += (uint32_t)T::BK / 32u;
                sa_num -= sdec;
                sb_ptr += (uint32_t)T::BK / 32u;
                sb_num -= sdec;
            }
            asm volatile("" : "+s"(sa_ptr), "+s"(sb_ptr), "+s"(sa_num), "+s"(sb_num));
        } else {
            asm volatile("" : "+s"(ld_lds), "+s"(ld_slot), "+s"(ld_k));
            if (++ld_slot == (uint32_t)L) {
                ld_slot = 0;
                ld_lds -= (L - 1) * T::STAGE;
            } else {
                ld_lds += T::STAGE;
            }
            if (__builtin_expect(++ld_k == k_blocks, 0)) {
                ld_k = 0;
                ld.next_tile();
                tile_ranges();
            }
            asm volatile("" : "+s"(ld_lds), "+s"(ld_slot), "+s"(ld_k));
        }
    };
    tile_ranges();
    // DMA q of a slab in issue order: A and B chunks [0, DF), then (only when
    // the slab starts a scale group) the group's scale DMAs, SFA then SFB, then
    // chunks [DF, ND).
    auto dma_op = [&](auto q_c) __attribute__((always_inline)) {
        constexpr int qq = decltype(q_c)::value;
        constexpr int q = qq < T::DF ? qq + NSC : (qq < T::DF + NSC ? qq - T::DF : qq);
        stress_pause<2>(wave, stress_ctr);
        if constexpr (q < NSC) {
            constexpr int i = q % NS;
            if (sc_issue)
                dma16_at<(q < NS ? 0u : (uint32_t)T::SC_B) + i * 1024u>(sc_lds, voff[ND + i], q < NS ? rs_sa : rs_sb);
        } else if constexpr (q - NSC < NA) {
            // the LDS target is formed inside the DMA's own asm, next to it
            dma16_at<(q - NSC) * 1024u>(dma_lds + wave * NA * 1024u, voff[q - NSC], rs_a);
        } else {
            dma16_at<(uint32_t)T::A_BYTES + (q - NSC - NA) * 1024u>(dma_lds + wave * NB * 1024u, voff[q - NSC], rs_b);
        }
    };

    // ---- fragments and scales: two register sets, the one this k-step's
    // MFMAs read and the one the next k-step's LDS reads fill ----
    f32x16 acc[F][F];
#pragma unroll
    for (int fm = 0; fm < F; ++fm)
#pragma unroll
        for (int fn = 0; fn < F; ++fn) acc[fm][fn] = f32x16{};
    u32x4 fa[2][F][2], fb[2][F][2];
    uint32_t sa[2][F], sb[2][F];

    // per-k-step address registers: stage and scale-record bases folded in
    // once, then register + immediate (32 rows = 4096 bytes of fragment,
    // 32 * SC_ROW of scales).  scb = scale ring entry + 4 * (slab in group).
    uint32_t ra[2], rb[2], rsa, rsb;
    auto set_addr = [&](auto ks_c, uint32_t st, uint32_t scb) __attribute__((always_inline)) {
        constexpr int KS = decltype(ks_c)::value;
        ra[0] = lds_base + st + a_off[KS][0];
        ra[1] = lds_base + st + a_off[KS][1];
        rb[0] = lds_base + st + b_off[KS][0];
        rb[1] = lds_base + st + b_off[KS][1];
        rsa = lds_base + scb + sa_off + 2u * KS;
        rsb = lds_base + scb + sb_off + 2u * KS;
    };
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    // read op r in consumption order of units A0, B0..B3, A1..A3: with
    // TSG_MX_SCALES_FIRST the eight scale bytes first, then the two 16-byte
    // halves of every unit (the compiler zero-extends the scale bytes at the
    // top of the consuming k-step, so they should be the first reads to land);
    // otherwise unit by unit, halves then scale byte.
    constexpr int R = 3 * 2 * F;
    auto read_op = [&](auto set_c, auto r_c) __attribute__((always_inline)) {
        constexpr int SET = decltype(set_c)::value, rr = decltype(r_c)::value;
        constexpr int u = TSG_MX_SCALES_FIRST ? (rr < 2 * F ? rr : (rr - 2 * F) / 2) : rr / 3;
        constexpr int part = TSG_MX_SCALES_FIRST ? (rr < 2 * F ? 2 : (rr - 2 * F) % 2) : rr % 3;
        constexpr bool is_a = (u == 0 || u > F);
        constexpr int f = u == 0 ? 0 : (u > F ? u - F : u - 1);
        if constexpr (is_a) {
            if constexpr (part < 2)
                fa[SET][f][part] = *(const lds_u32x4*)((lds_u8*)(uintptr_t)ra[part] + f * 32 * T::BK);
            else
                sa[SET][f] = *((const lds_u8*)(uintptr_t)rsa + f * 32 * T::SC_ROW);
        } else {
            if constexpr (part < 2)
                fb[SET][f][part] = *(const lds_u32x4*)((lds_u8*)(uintptr_t)rb[part] + f * 32 * T::BK);
            else
                sb[SET][f] = *((const lds_u8*)(uintptr_t)rsb + f * 32 * T::SC_ROW);
        }
    };
    auto read_all = [&](auto set_c, auto ks_c, uint32_t st, uint32_t scb) __attribute__((always_inline)) {
        set_addr(ks_c, st, scb);
        static_for<0, R>([&](auto r_c) __attribute__((always_inline)) { read_op(set_c, r_c); });
    };

    // ---- the MMA's tile scheduler and each lane's place in C ----
    TileScheduler sched;
    sched.setup(args.P, args.m_blocks, args.n_blocks, args.group, args.cluster, args.col_major);
    const uint32_t row0 = wr * T::WM + r, col0 = wc * T::WN + 8u * h;
    const uint32_t lane_off = (row0 * N + col0) * 2u;

    // Interleaved epilogue: a tile's C leaves between MFMAs.  Row block fm
    // (32 rows) is final after MFMA F*fm + F-1 of the tile's last k-step.
    // Blocks fm < kMxEpiFirst are stored in that k-step, two stores after
    // each MFMA from F*fm + F on, so store (fn, half) reads block (fm, fn)
    // F MFMAs after it was last written; block F-1 is final too late and is
    // stored in the next tile's first k-step, two stores after each of its
    // first MFMAs, long before that k-step's first MFMA on it.  That first
    // k-step uses the MFMA with a zero accumulator input (the k == 0 clear).
    // A worker's first tile stores nothing there (empty store window); its
    // last tile stores block F-1 after the loop.
    constexpr int kMxEpiFirst = F - 1;
    static_assert(F * (kMxEpiFirst - 1) + F + F - 1 < F * F, "first-part stores must fit in the k-step");
    __amdgpu_buffer_rsrc_t e_rc = make_rsrc(args.C, 0u);
    uint32_t e_rows = 0, e_cols = 0;
    // the store window of the MMA's current tile (and its trace row)
    auto epi_state = [&]() __attribute__((always_inline)) {
        const uint32_t m_idx = sched.m_idx, n_idx = sched.n_idx;
        if (args.trace != nullptr && threadIdx.x == 0) {
            int32_t* row = args.trace + 4 * ((size_t)wid * args.max_iters + sched.iter);
            *(int4*)row = make_int4((int)wid, (int)sched.iter, (int)m_idx, (int)n_idx);
            store_gap();
        }
        const int64_t m0 = (int64_t)m_idx * T::BM, n0 = (int64_t)n_idx * T::BN;
        e_rows = (uint32_t)((args.M - m0) < T::BM ? (args.M - m0) : T::BM);
        e_cols = (uint32_t)((args.N - n0) < T::BN ? (args.N - n0) : T::BN);
        e_rc = make_rsrc(args.C + (m0 * args.N + n0), ((e_rows - 1u) * N + e_cols) * 2u);
    };
    // store j of row block fm: block (fm, j / 2), values 8 * (j % 2) .. + 7.
    // Lane (h, r) of block (fm, fn) holds row 32*fm + r and columns
    // 32*fn + 8h + 0..7 (values 0-7) and 32*fn + 16 + 8h + 0..7 (values 8-15).
    auto epi_op = [&](auto fm_c, auto j_c) __attribute__((always_inline)) {
        constexpr int fm = decltype(fm_c)::value, j = decltype(j_c)::value;
        constexpr int fn = j / 2, hs = j % 2;
        const f32x16& x = acc[fm][fn];
        const u32x4 v = {cvt_pk<DT_BF16>(x[8 * hs + 0], x[8 * hs + 1]), cvt_pk<DT_BF16>(x[8 * hs + 2], x[8 * hs + 3]),
                         cvt_pk<DT_BF16>(x[8 * hs + 4], x[8 * hs + 5]), cvt_pk<DT_BF16>(x[8 * hs + 6], x[8 * hs + 7])};
        const bool ok = row0 + fm * 32 < e_rows && col0 + 32u * fn + 16u * hs < e_cols;
        __builtin_amdgcn_raw_buffer_store_b128(v, e_rc, (ok ? lane_off : 0x80000000u) + (fn * 32 + 16 * hs) * 2,
                                               fm * 32 * N * 2, TSG_MX_C_CPOL);
    };

    // One 64-deep k-step: 16 MFMAs (fm-major) from register set CUR, with the
    // memory operations for what follows between them: the reads of the next
    // k-step into set NXT and, in a slab's LAST k-step, the DMA of slab
    // phase + L.  LAST first waits for the next slab and passes the workgroup
    // barrier (after S0 MFMAs), then refills the stage just consumed and reads
    // the next slab's first k-step; otherwise the reads take k-step KSN of the
    // current stage.  No read into a set starts within kMxGap MFMAs of the
    // last MFMA that read it.
    // EPH: 0 no stores, 1 the current tile's stores of blocks fm <
    // kMxEpiFirst (its last k-step), 2 the previous tile's block F-1 (the
    // tile's first k-step, whose MFMAs start from zero).
    auto kstep = [&](auto cur_c, auto last_c, auto ksn_c, uint32_t read_st, uint32_t read_scb, auto eph_c) __attribute__((always_inline)) {
        constexpr int EPH = decltype(eph_c)::value;
        constexpr int CUR = decltype(cur_c)::value;
        constexpr int NXT = 1 - CUR;
        constexpr bool LAST = decltype(last_c)::value;
        constexpr int NSTEP = F * F;
        constexpr int S0 = LAST ? kMxS0 : 0;
        constexpr int START = S0 > kMxGap ? S0 : kMxGap;
        constexpr int AVAIL = NSTEP - START - 1;
        constexpr int D = LAST ? T::DF + NSC : ND - T::DF;   // DMA ops [D0, D0 + D) of the issue order
        constexpr int D0 = LAST ? 0 : T::DF + NSC;
        constexpr int DPER = D ? (D + AVAIL - 1) / AVAIL : 0;
        constexpr int PER = (R + AVAIL - 1) / AVAIL;
        static_assert(AVAIL * PER >= R && (D == 0 || AVAIL * DPER >= D), "k-step too short for its memory operations");
        static_assert(START >= 2, "the first k-step's addresses need a gap before its first read");
        // the scale descriptors after the barrier's gap, before the slab's
        // first scale DMA (issue position DF); the loader's three pieces
        // after the first k-step's DMAs
        constexpr int kScaleDesc = START + 1;
        constexpr int kAdvGap = NSTEP - 6;
        static_assert(!LAST || D == 0 || START + T::DF / DPER >= kScaleDesc + 2, "scale descriptors before their DMAs");
        static_assert(LAST || D == 0 || START + (D + DPER - 1) / DPER <= kAdvGap, "the loader steps after the first k-step's DMAs");
        static_for<0, NSTEP>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            constexpr int fm = s / F, fn = s % F;
            const i32x8 b8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(fb[CUR][fn][0], fb[CUR][fn][1], 0, 1, 2, 3, 4, 5, 6, 7));
            const i32x8 a8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(fa[CUR][fm][0], fa[CUR][fm][1], 0, 1, 2, 3, 4, 5, 6, 7));
            if constexpr (EPH == 2)
                mfma_mx32_clear(acc[fm][fn], b8, a8, sb[CUR][fn], sa[CUR][fm]);
            else
                mfma_mx32(acc[fm][fn], b8, a8, sb[CUR][fn], sa[CUR][fm]);
            // LAST: the slab's descriptors, A and B before its first DMA, the
            // scale descriptors before its first scale DMA; the slab's first
            // k-step (!LAST): the loader's step, after that k-step's DMAs of
            // the previous slab (they use the descriptors already formed)
            if constexpr (LAST && s == 0) {
                desc_piece(std::integral_constant<int, 0>{});
                desc_piece(std::integral_constant<int, 1>{});
            }
            if constexpr (LAST && s == 1) desc_piece(std::integral_constant<int, 2>{});
            if constexpr (LAST && s == kScaleDesc) desc_piece(std::integral_constant<int, 3>{});
            if constexpr (LAST && s == kScaleDesc + 1) desc_piece(std::integral_constant<int, 4>{});
            if constexpr (!LAST && s >= kAdvGap && s < kAdvGap + 3)
                adv_piece(std::integral_constant<int, (s >= kAdvGap ? s - kAdvGap : 0)>{});
            if constexpr (!LAST && s == START - 1) {
                asm volatile("" : "+s"(read_st), "+s"(read_scb));
                set_addr(ksn_c, read_st, read_scb);
                asm volatile("" : "+v"(ra[0]), "+v"(ra[1]), "+v"(rb[0]), "+v"(rb[1]), "+v"(rsa), "+v"(rsb));
            }
            if constexpr (LAST && s == S0 - 1) {
                stress_pause<0>(wave, stress_ctr);
                wait_vm<0>();    // slab phase+1 (and its scale group) has landed
                lds_barrier();   // ... for every wave; stage phase and scale entries read are free
                stress_pause<1>(wave, stress_ctr);
                set_addr(ksn_c, read_st, read_scb);
            }
            if constexpr (s >= START) {
                constexpr int i = s - START;
                if constexpr (D) {
                    constexpr int d0 = i * DPER;
                    constexpr int d1 = d0 + DPER < D ? d0 + DPER : D;
                    static_for<d0, d1>([&](auto q_c) __attribute__((always_inline)) {
                        dma_op(std::integral_constant<int, D0 + decltype(q_c)::value>{});
                    });
                }
                constexpr int q0 = i * PER;
                constexpr int q1 = q0 + PER < R ? q0 + PER : R;
                static_for<q0, q1>([&](auto q_c) __attribute__((always_inline)) {
                    read_op(std::integral_constant<int, NXT>{}, q_c);
                });
            }
            if constexpr (EPH == 1 && s >= F && s / F - 1 < kMxEpiFirst) {
                // stores 2(s mod F), 2(s mod F) + 1 of block s / F - 1
                epi_op(std::integral_constant<int, s / F - 1>{}, std::integral_constant<int, 2 * (s % F)>{});
                epi_op(std::integral_constant<int, s / F - 1>{}, std::integral_constant<int, 2 * (s % F) + 1>{});
            } else if constexpr (EPH == 2 && s < F) {
                epi_op(std::integral_constant<int, F - 1>{}, std::integral_constant<int, 2 * s>{});
                epi_op(std::integral_constant<int, F - 1>{}, std::integral_constant<int, 2 * s + 1>{});
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using TRUE_ = std::integral_constant<bool, true>;
    using FALSE_ = std::integral_constant<bool, false>;

    // prologue: slabs 0..L-1 in flight, the first k-step's fragments read
    for (int s = 0; s < L; ++s) {
        if (s + 1 < L) {
            next_slab();
            static_for<0, NSC + ND>([&](auto q_c) __attribute__((always_inline)) { dma_op(q_c); });
        } else {  // the last prologue slab's chunks [DF, ND) and the loader's step follow in the first k-step
            slab_desc();
            static_for<0, T::DF + NSC>([&](auto q_c) __attribute__((always_inline)) { dma_op(q_c); });
        }
    }
    stress_pause<3>(wave, stress_ctr);
    wait_vm<0>();
    lds_barrier();
    auto scale_base = [&](uint32_t grp, uint32_t sub) __attribute__((always_inline)) -> uint32_t {
        return T::SC_OFF + (grp & 1u) * T::SC_ENTRY + sub * 4u;
    };
    read_all(I0{}, I0{}, 0u, scale_base(0u, 0u));

    // two k-steps per slab: set 0 then set 1; the second (LAST) publishes the
    // next slab and reads its first k-step into set 0.  grp counts the scale
    // groups consumed so far exactly as the loader counts those it fetched.
    // The k loop is rotated (the tile's first k-step, then pairs of one
    // slab's last and the next slab's first k-step, then the tile's last
    // k-step) so a tile is one code path and its stores can sit between the
    // MFMAs of its last and the next tile's first k-step.
    uint32_t phase = 0, grp = 0;
    bool pend = false;  // a tile's block F-1 is still to be stored
    for (sched.init(wid); sched.valid(); sched.next_tile()) {
        kstep(I0{}, FALSE_{}, I1{}, (phase % L) * T::STAGE, scale_base(grp, 0u), I2{});
        for (uint32_t k = 0; k + 1u < k_blocks; ++k, ++phase) {
            const uint32_t k_next = k + 1u;
            const uint32_t grp_next = grp + ((k_next % T::SG) == 0u ? 1u : 0u);
            kstep(I1{}, TRUE_{}, I0{}, ((phase + 1u) % L) * T::STAGE, scale_base(grp_next, k_next % T::SG), I0{});
            grp = grp_next;
            kstep(I0{}, FALSE_{}, I1{}, ((phase + 1u) % L) * T::STAGE, scale_base(grp, k_next % T::SG), I0{});
        }
        // the tile's last slab: its LAST k-step reads the next tile's slab 0,
        // which starts a scale group
        epi_state();
        kstep(I1{}, TRUE_{}, I0{}, ((phase + 1u) % L) * T::STAGE, scale_base(grp + 1u, 0u), I1{});
        grp += 1u;
        ++phase;
        pend = true;
    }
    if (pend) {
        gap_nops();  // the last tile's last MFMAs have written their accumulators
        static_for<0, 2 * F>([&](auto j_c) __attribute__((always_inline)) {
            epi_op(std::integral_constant<int, F - 1>{}, j_c);
            store_gap();  // the store may still read its data registers
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    wait_vm<0>();  // no DMA may still target LDS when the workgroup retires
}

}  // namespace tsg
