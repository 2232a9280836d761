// Persistent, tile-scheduled GEMM kernel for gfx950 (CDNA4).
//
//   C[M,N] = A[M,K] * B[K,N], fp16/bf16 in and out, fp32 accumulation.
//
// Method (page "[Feature] Introduce tile scheduler #2441", diff of
// examples/gemm_sm100/gemm_tcgen5mma_ws_persistent.py, gemm_persistent):
//   * a fixed grid of persistent workers; each runs one `while sched.valid()`
//     loop over its tiles (tile_scheduler.h);
//   * the K loop streams A and B slabs through a ring of shared-memory stages:
//     slab counter phase = w * k_blocks + k runs across tiles, stage
//     phase % stages (the review on the page's conversation tab settles the
//     slot index as phase % num_stages);
//   * the MMA accumulates the tile in fp32, clearing the accumulator on k == 0;
//   * the epilogue casts the fp32 tile to the output type and stores it.
// The page's SM100 design (TMA, tcgen05 into TMEM, mbarriers, one warp per
// role) is replaced by what gfx950 offers:
//   * loads: buffer_load ... lds (16 bytes per lane straight into LDS) with a
//     per-slab buffer descriptor whose range check returns zero past the matrix
//     edge (the analogue of TMA's out-of-bounds fill);
//   * the loader runs `stages - 1` slabs ahead of the math with its own
//     scheduler copy, so the next tile's first slabs are in flight while the
//     current tile's epilogue stores drain;
//   * math: v_mfma_f32_16x16x32_{f16,bf16}; A fragments come from
//     K-contiguous LDS rows (ds_read_b128), B fragments from N-contiguous LDS
//     rows through the LDS transpose read ds_read_b64_tr_b16;
//   * LDS rows are XOR-swizzled in 16-byte chunks so fragment reads spread over
//     the banks; the swizzle is applied on the global side of the DMA (each
//     lane fetches the chunk that belongs at its fixed LDS position);
//   * 256 threads = 4 wavefronts in a 2x2 grid, one per SIMD; every wave
//     computes a (BM/2) x (BN/2) sub-tile with its accumulators in registers;
//   * the MFMA is issued with B as its first operand, so a lane's results run
//     along N and the epilogue writes 16 contiguous bytes per lane;
//   * on 256x256x64 tiles each slab's two k-steps reach every accumulator as
//     two MFMAs in a row (PAIR), the second taking its accumulator input from
//     the matrix core's forwarding path.
#pragma once

#include "tile_scheduler.h"
#include "tsgemm_device.h"

namespace tsg {

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int DT, int BM, int BN, int BK, int L, int WGN, int EPI = 0>
struct GemmTraits {
    static constexpr int NW = 2 * WGN;                      // waves: 2 along M x WGN along N
    static constexpr int THREADS = 64 * NW;
    static constexpr int WM = BM / 2, WN = BN / WGN;        // wave sub-tile
    static constexpr int FM = WM / 16, FN = WN / 16;        // 16x16 blocks per wave
    static constexpr int KS = BK / 32;                      // MFMA k-steps per slab
    static constexpr int CA = BK / 8;                       // 16-byte chunks per A row
    static constexpr int CB = BN / 8;                       // 16-byte chunks per B row
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // EPI = 64: the epilogue stages C through an LDS buffer of BM rows x 64
    // columns after the ring (EPI = 0: direct stores from registers)
    static constexpr int CHUNK_OFF = STAGE * L;
    static constexpr int CHUNK_BYTES = EPI ? BM * EPI * 2 : 0;
    static constexpr int LDS = STAGE * L + CHUNK_BYTES;
    static constexpr int NA = A_BYTES / (1024 * NW);        // DMA instructions per wave, A
    static constexpr int NB = B_BYTES / (1024 * NW);        // DMA instructions per wave, B
    static constexpr int NL = NA + NB;
    // DMAs of a slab issued in the LAST k-step of the slab two back; with two
    // k-steps per slab the remaining NL - DF go out during the next k-step
    static constexpr int DF = (BK == 64 && TSG_DMA_FIRST > 0 && TSG_DMA_FIRST < NL) ? TSG_DMA_FIRST : NL;
    static_assert(BK == 32 || BK == 64, "block_K");
    static_assert(FN % 2 == 0 && FM >= 1, "wave tile");
    static_assert(NA >= 1 && NB >= 1 && NA * 1024 * NW == A_BYTES && NB * 1024 * NW == B_BYTES,
                  "slab must split into whole 1 KiB DMAs per wave");
    static_assert(WGN == 2 || WGN == 4, "wave grid");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(EPI == 0 || (EPI == 64 && WGN == 2 && WN % 64 == 0), "chunked epilogue: 64 columns, 4 waves");
    static_assert(CB >= 16, "B swizzle needs 16 chunks per row");
};


// With fewer tiles than workers every active worker owns exactly one tile and
// the others would leave at once.  Instead, each of them warms the L2 of the
// XCD it runs on (workgroup b runs on XCD b % X) with part of the A row panel
// and B column panel that one of that XCD's active workers is about to stream:
// one 4-byte load per 128-byte line, in K order, from the first line the
// active worker's own prologue does not already request.  The idle workers of
// an XCD split its active workers round robin and each one's lines among
// themselves.  Nothing is written; only the timing of the active workers'
// loads depends on it.
template <int BM, int BN, int BK, int L>
__device__ __forceinline__ void warm_l2_for_xcd(const GemmArgs& args) {
    const uint32_t X = args.num_xcd > 1u ? args.num_xcd : 1u;
    const uint32_t P = args.P, A = args.num_active;
    const uint32_t x = blockIdx.x % X, j = blockIdx.x / X;
    const uint32_t slots = P / X + (x < P % X ? 1u : 0u);
    const uint32_t active_x = A / X + (x < A % X ? 1u : 0u);
    const uint32_t first_active = x * (A / X) + (x < A % X ? x : A % X);
    if (active_x == 0u || j < active_x || j >= slots) return;
    const uint32_t i = j - active_x, n_idle = slots - active_x;
    const uint32_t helped = i % active_x;                                 // active worker of this XCD
    const uint32_t part = i / active_x;                                   // this workgroup's share ...
    const uint32_t parts = (n_idle - helped + active_x - 1u) / active_x;  // ... of that many
    TileScheduler s;
    s.setup(P, args.m_blocks, args.n_blocks, args.group, args.cluster, args.col_major);
    s.init(first_active + helped);
    if (!s.valid()) return;
    const uint64_t M = (uint64_t)args.M, N = (uint64_t)args.N, K = (uint64_t)args.K;
    const uint64_t m0 = (uint64_t)s.m_idx * BM, n0 = (uint64_t)s.n_idx * BN;
    const uint32_t rows_a = (uint32_t)(M - m0 < (uint64_t)BM ? M - m0 : (uint64_t)BM);
    const uint32_t cols_b = (uint32_t)(N - n0 < (uint64_t)BN ? N - n0 : (uint64_t)BN);
    const uint32_t row_bytes = (uint32_t)(K * 2u);                      // an A row
    const uint32_t seg_bytes = cols_b * 2u;                             // a B row's part in the panel
    const uint32_t k_lines = (row_bytes + 127u) / 128u;                 // 128-byte lines along K
    const uint32_t kl0 = (uint32_t)L * BK * 2u / 128u;                  // first line past the prologue
    const uint32_t b_touch = (seg_bytes + 127u) / 128u + 1u;            // touches per B row (any alignment)
    const uint32_t per_line = rows_a + 64u * b_touch;                   // A rows + the 64 B rows of a K line
    if (kl0 >= k_lines) return;
    const uint32_t total = (k_lines - kl0) * per_line;
    const uint32_t stride = parts * blockDim.x;
    const uint8_t* a_panel = reinterpret_cast<const uint8_t*>(args.A) + m0 * K * 2u;
    const uint8_t* b_panel = reinterpret_cast<const uint8_t*>(args.B) + n0 * 2u;
    // address of touch `idx`: every address is inside A's rows [m0, m0 + rows_a) or B's rows
    // [0, K) x columns [n0, n0 + cols_b) (out-of-range indexes are clamped onto the last line)
    auto address = [&](uint32_t idx) __attribute__((always_inline)) -> const uint32_t* {
        idx = idx < total ? idx : total - 1u;
        const uint32_t kl = kl0 + idx / per_line, t = idx % per_line;
        if (t < rows_a) {
            const uint32_t off = kl * 128u < row_bytes - 4u ? kl * 128u : row_bytes - 4u;
            return reinterpret_cast<const uint32_t*>(a_panel + (uint64_t)t * row_bytes + off);
        }
        const uint32_t u = t - rows_a, kr = u / b_touch, c = u % b_touch;
        const uint64_t k = (uint64_t)kl * 64u + kr < K ? (uint64_t)kl * 64u + kr : K - 1u;
        const uint32_t off = c * 128u < seg_bytes - 4u ? c * 128u : seg_bytes - 4u;
        return reinterpret_cast<const uint32_t*>(b_panel + k * N * 2u + off);
    };
    uint32_t sink = 0;
    for (uint32_t base = part * blockDim.x + threadIdx.x; base < total; base += 8u * stride) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *address(base + (uint32_t)u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) sink ^= v[u];
    }
    asm volatile("" ::"v"(sink));  // the loads are the point; keep them
}

#ifndef TSG_PAIR
#define TSG_PAIR 1  // 0: no paired-k-step kernels (every plan runs the k-step-by-k-step order)
#endif
// The kernels that run each slab's two k-steps as MFMA pairs on one
// accumulator (PAIR, below): 256x256x64 tiles, four waves, direct stores.
// A plan runs them when its tiles have at least two slabs.
constexpr bool pair_kernel(int bm, int bn, int bk, int wgn, int epi) {
    return TSG_PAIR && TSG_EPI_INTERLEAVE && bm == 256 && bn == 256 && bk == 64 && wgn == 2 && epi == 0;
}

template <int DT, int BM, int BN, int BK, int L, int WGN, int EPI = 0, bool PAIR = false>
__global__ __launch_bounds__(64 * 2 * WGN, 1) void tsgemm_kernel(GemmArgs args) {
    using T = GemmTraits<DT, BM, BN, BK, L, WGN, EPI>;
    constexpr int FM = T::FM, FN = T::FN, KS = T::KS, NA = T::NA, NB = T::NB, NL = T::NL;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
    const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)smem);

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wr = wave / WGN, wc = wave % WGN;  // wave row / column in the 2 x WGN grid
    const uint32_t N = (uint32_t)args.N, K = (uint32_t)args.K;
    const uint32_t k_blocks = args.k_blocks;
    const uint32_t wid = worker_of_workgroup(blockIdx.x, args.P, args.num_xcd, args.num_active);
    uint32_t stress_ctr = 0;  // race-detection build only (TSG_STRESS)
    if (args.prefetch && wid >= args.num_active) {  // a worker without a tile (uniform per workgroup)
        warm_l2_for_xcd<BM, BN, BK, L>(args);
        return;
    }

    // ---- DMA source offsets (bytes from the slab origin) = lane part + uniform part ----
    // Instruction q of this wave fills 16-byte LDS positions p = qe*64 + lane,
    // qe = wave*NA + q (A) or wave*NB + q (B); the lane fetches the logical
    // chunk that the swizzle puts at p.  A's swizzle depends on the lane only;
    // B's also on bits 1 and 3 of the stage row, i.e. on vkey = (qe*64/CB) & 0xA.
    const uint32_t va = ((lane / T::CA) * K + ((lane % T::CA) ^ swz_a<T::CA>(lane / T::CA)) * 8u) * 2u;
    uint32_t ua[NA], ub[NB];
#pragma unroll
    for (int q = 0; q < NA; ++q) ua[q] = (wave * NA + q) * (64u / T::CA) * K * 2u;
#pragma unroll
    for (int q = 0; q < NB; ++q) ub[q] = (wave * NB + q) * (64u / T::CB) * N * 2u;
    uint32_t vb[4];  // indexed by vkey bits (1, 3)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint32_t kr = lane / T::CB + ((v & 1) << 1) + ((v >> 1) << 3);
        vb[v] = ((lane / T::CB) * N + ((lane % T::CB) ^ swz_b(kr)) * 8u) * 2u;
    }
    auto vb_for = [&](uint32_t qe) __attribute__((always_inline)) -> uint32_t {
        const uint32_t key = (qe * (64u / T::CB)) & 0xAu;
        return vb[((key >> 1) & 1u) | ((key >> 3) << 1)];
    };
    // full per-instruction offsets, formed once (an add right before each DMA
    // would stall its issue on the VALU result)
    uint32_t voff[NL];
#pragma unroll
    for (int q = 0; q < NA; ++q) voff[q] = va + ua[q];
#pragma unroll
    for (int q = 0; q < NB; ++q) voff[NA + q] = vb_for(wave * NB + q) + ub[q];

    // ---- per-lane LDS read offsets (bytes from the stage origin) ----
    const uint32_t l16 = lane & 15u, lg = lane >> 4;
    uint32_t a_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        a_off[ks] = (wr * T::WM + l16) * (BK * 2) + (((uint32_t)ks * 4u + lg) ^ swz_a<T::CA>(l16)) * 16u;
    // B fragments: the n columns of a pair of 16x16 blocks (2t, 2t+1) are
    // interleaved so that a lane ends up holding 8 consecutive n of one row:
    // block b, lane group g holds n = 32t + 8g + 4*(b ^ (g & 1)) + 0..3.  A
    // transpose-read lane with chunk offset q = l16 & 3 therefore reads the
    // half (b ^ (q & 1)) of its chunk, which also spreads one read's 16 lanes
    // over 16 distinct bank pairs.
    uint32_t b_off[FN];
    {
        const uint32_t kr0 = 8u * lg + (l16 >> 2);  // k row of the transpose read (ks=0, h=0)
        const uint32_t sw = swz_b(kr0);
#pragma unroll
        for (int t = 0; t < FN / 2; ++t) {
            const uint32_t chunk = (wc * T::WN + 32u * t) / 8u + (l16 & 3u);
            const uint32_t base = T::A_BYTES + kr0 * (BN * 2) + (chunk ^ sw) * 16u;
#pragma unroll
            for (int b = 0; b < 2; ++b) b_off[2 * t + b] = base + 8u * ((uint32_t)b ^ (l16 & 1u));
        }
    }

    // ---- loader: its own scheduler copy, L slabs ahead of the MMA ----
    // Per tile the loader forms the byte address of its first A slab (row
    // block m, column 0) and B slab (row 0, column block n) and the ranges the
    // descriptors may span; per slab it only steps them (A by BK columns, B by
    // BK rows).  The scalar work that sits between two MFMAs is then a few
    // adds and selects instead of 64-bit products and compares: the wave
    // that issues them is the one that issues the MFMAs.
    //   A: range = rows * K * 2 - k0 * 2 bytes from the slab origin, rows =
    //      min(M - m0, BM): rows past M read zeros, and the range never runs
    //      past row m0 + rows - 1 of A;
    //   B: every slab but the tile's last spans BK full rows; the last slab's
    //      range stops at the end of B (columns past N in its last row read
    //      zeros; elsewhere they read finite neighbours that are never stored).
    // BM*K*2 and BK*N*2 are below 2^31 (checked when the plan is created).
    TileScheduler ld;
    ld.setup(args.P, args.m_blocks, args.n_blocks, args.group, args.cluster, args.col_major);
    ld.init(wid);
    uint32_t ld_k = 0;
    uint32_t a_dec = 0, b_cap = 0, b_last = 0;
    const uint32_t M32 = (uint32_t)args.M;
    const uint64_t b_step = (uint64_t)BK * N * 2u;
    // The loader's state is the descriptors themselves (words 0-1: the
    // slab origin, word 2: the range) and the LDS target of its next slab; the
    // DMAs read them in place.
    i32x4 rs_a, rs_b;
    uint32_t dma_lds = lds_base + wave * NA * 1024u;
    // With a slab's DMAs split over two k-steps, the loader steps in the
    // first k-step of a slab (after the split slab's remaining DMAs), else in
    // the slab's last k-step (after all of them).
    constexpr bool kSplitAdvance = KS == 2 && T::DF < NL;
    auto add64 = [](i32x4& r, uint64_t d) __attribute__((always_inline)) {
        const uint64_t a = (((uint64_t)(uint32_t)r.y) << 32 | (uint32_t)r.x) + d;  // stride bits are 0
        r.x = (int)(uint32_t)a;
        r.y = (int)(uint32_t)(a >> 32);
    };

    // ranges for the loader's current tile; zero past the end of the schedule
    // (the DMAs then write zeros into a stage nobody reads, so every slab
    // issues the same instructions)
    auto tile_ranges = [&]() __attribute__((always_inline)) {
        const bool live = ld.valid();
        const uint32_t m0 = ld.m_idx * BM, n0 = ld.n_idx * BN;
        const uint32_t rows = live ? (M32 - m0 < (uint32_t)BM ? M32 - m0 : (uint32_t)BM) : 0u;
        a_dec = live ? BK * 2u : 0u;
        b_cap = live ? (uint32_t)BK * N * 2u : 0u;
        b_last = live ? ((uint32_t)BK * N - n0) * 2u : 0u;
        rs_a = rsrc_words_u64(reinterpret_cast<uint64_t>(args.A) + (live ? (uint64_t)m0 * K * 2u : 0u), rows * K * 2u);
        rs_b = rsrc_words_u64(reinterpret_cast<uint64_t>(args.B) + (live ? (uint64_t)n0 * 2u : 0u),
                              k_blocks == 1u ? b_last : b_cap);
    };
    // Step the loader to the slab after, once every DMA of the current one
    // has been issued.  With one wave per SIMD a wave issues at most one
    // instruction every four cycles, so a 16-cycle MFMA leaves room for three
    // others before the next MFMA can go; a longer run of scalar work in one
    // gap stalls the matrix core.  The step is therefore cut into pieces of at
    // most three scalar instructions, one per gap, in this order:
    //   0: A's origin and range;  1: B's origin;  2: the LDS target (wraps to
    //   slot 0 after slot L-1);  3: B's range for the next slab (the tile's
    //   last slab stops at the end of B);  4: the slab count, and at a tile's
    //   end (rare, branched over) the next tile's descriptors.
    // Each piece starts and ends with an empty volatile asm on the registers
    // it changes: volatile asm keeps its order with the MFMAs (volatile asm
    // too), so the compiler can neither hoist a piece's work above the MFMA
    // before its gap nor sink it past the MFMA after.
    const uint32_t dma_first = dma_lds, dma_wrap = dma_lds + (L - 1) * T::STAGE;
    const uint32_t k_before_last = k_blocks - 2u;  // wraps for k_blocks = 1: every step then starts a tile
    constexpr int kAdvPieces = 5;
    auto adv_piece = [&](auto p_c) __attribute__((always_inline)) {
        constexpr int p = decltype(p_c)::value;
        if constexpr (p == 0) {
            asm volatile("" : "+s"(rs_a));
            add64(rs_a, BK * 2u);
            rs_a.z -= (int)a_dec;
            asm volatile("" : "+s"(rs_a));
        } else if constexpr (p == 1) {
            asm volatile("" : "+s"(rs_b));
            add64(rs_b, b_step);
            asm volatile("" : "+s"(rs_b));
        } else if constexpr (p == 2) {
            asm volatile("" : "+s"(dma_lds));
            dma_lds = dma_lds == dma_wrap ? dma_first : dma_lds + T::STAGE;
            asm volatile("" : "+s"(dma_lds));
        } else if constexpr (p == 3) {
            asm volatile("" : "+s"(rs_b), "+s"(ld_k));
            rs_b.z = (int)(ld_k == k_before_last ? b_last : b_cap);
            asm volatile("" : "+s"(rs_b));
        } else {
            asm volatile("" : "+s"(ld_k));
            if (__builtin_expect(++ld_k == k_blocks, 0)) {
                ld_k = 0;
                ld.next_tile();
                tile_ranges();
            }
            asm volatile("" : "+s"(ld_k), "+s"(rs_a), "+s"(rs_b));
        }
    };
    auto slab_advance = [&]() __attribute__((always_inline)) {
        static_for<0, kAdvPieces>([&](auto p_c) __attribute__((always_inline)) { adv_piece(p_c); });
    };
    tile_ranges();
    // One DMA in one piece (prologue): its LDS target is written to M0 inside
    // the DMA's own asm.
    auto dma_op = [&](auto q_c) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
        if constexpr (q < NA)
            dma16_at<q * 1024u>(dma_lds, voff[q], rs_a);
        else
            dma16_at<(uint32_t)T::A_BYTES + (q - NA) * 1024u>(dma_lds + wave * (NB - NA) * 1024u, voff[q], rs_b);
    };
    // The same DMA in two pieces (main loop): M0 written in the MFMA gap
    // before the one that issues the load, so neither gap carries the wait
    // state an M0 write needs before its LDS-DMA.  Nothing else in the loop
    // writes M0 (the fragment reads do not use it); a load is always issued
    // before the next M0 write, in program order, with an MFMA between each
    // M0 write and its load.
    auto m0_op = [&](auto q_c) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
        if constexpr (q < NA)
            set_m0<q * 1024u>(dma_lds);
        else
            set_m0<(uint32_t)T::A_BYTES + (q - NA) * 1024u>(dma_lds + wave * (NB - NA) * 1024u);
    };
    auto load_op = [&](auto q_c) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;
        stress_pause<2>(wave, stress_ctr);
        const uint32_t v = voff[q];
        if constexpr (q < NA)
            dma16_m0(v, rs_a);
        else
            dma16_m0(v, rs_b);
    };

    // ---- fragments: two register sets for A and B, the one the MFMAs of this
    // k-step read and the one the next k-step's LDS reads fill ----
    f32x4 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
    i16x8 fa[2][FM];
    i16x4 fb[2][FN][2];

    // LDS reads of one k-step: A block fm, and B halves (fn, h) into set SET.
    // The stage base is folded into per-lane address registers once per
    // k-step (ra, rb); each read is then register + immediate.
    uint32_t ra, rb[FN];
    auto set_addr = [&](auto ks_c, uint32_t st) __attribute__((always_inline)) {
        constexpr int KSN = decltype(ks_c)::value;
        ra = lds_base + st + a_off[KSN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) rb[fn] = lds_base + st + b_off[fn] + KSN * 32 * (BN * 2);
    };
    auto read_a = [&](auto set_c, auto fm_c) __attribute__((always_inline)) {
        constexpr int SET = decltype(set_c)::value, fm = decltype(fm_c)::value;
        fa[SET][fm] = __builtin_bit_cast(i16x8, *(const __attribute__((address_space(3))) u32x4*)(
                                               (__attribute__((address_space(3))) uint8_t*)(uintptr_t)ra + fm * 16 * (BK * 2)));
    };
    auto read_b = [&](auto set_c, auto r_c) __attribute__((always_inline)) {
        constexpr int SET = decltype(set_c)::value, r = decltype(r_c)::value;
        constexpr int fn = r / 2, h = r % 2;
        fb[SET][fn][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) uint8_t*)(uintptr_t)rb[fn] + h * 4 * (BN * 2)));
    };
    // read op r of a k-step in consumption order: A block 0, the B halves,
    // then A blocks 1..FM-1
    constexpr int R = FM + 2 * FN;
    auto read_op = [&](auto set_c, auto r_c) __attribute__((always_inline)) {
        constexpr int r = decltype(r_c)::value;
        if constexpr (r == 0 || r > 2 * FN)
            read_a(set_c, std::integral_constant<int, (r == 0 ? 0 : r - 2 * FN)>{});
        else
            read_b(set_c, std::integral_constant<int, r - 1>{});
    };
    auto read_all = [&](auto set_c, auto ks_c, uint32_t st) __attribute__((always_inline)) {
        set_addr(ks_c, st);
        static_for<0, R>([&](auto r_c) __attribute__((always_inline)) { read_op(set_c, r_c); });
    };
    // The address a read op needs, formed one MFMA ahead of the read (an add
    // right before its read would stall the read on the add): read op 0 forms
    // ra, the first half of each B pair forms rb[fn]; the others reuse them.
    auto prep_op = [&](auto ks_c, auto r_c, uint32_t st) __attribute__((always_inline)) {
        constexpr int KSN = decltype(ks_c)::value, r = decltype(r_c)::value;
        if constexpr (r == 0)
            ra = lds_base + st + a_off[KSN];
        else if constexpr (r <= 2 * FN && (r - 1) % 2 == 0)
            rb[(r - 1) / 2] = lds_base + st + b_off[(r - 1) / 2] + KSN * 32 * (BN * 2);
    };

    // ---- the MMA's tile scheduler and each lane's place in C ----
    TileScheduler sched;
    sched.setup(args.P, args.m_blocks, args.n_blocks, args.group, args.cluster, args.col_major);
    const bool swap = (lg & 1u) != 0;  // odd lane groups hold the upper four columns of block 2t
    const uint32_t row0 = wr * T::WM + l16, col0 = wc * T::WN + 8u * lg;
    const uint32_t lane_off = (row0 * N + col0) * 2u;

    // Interleaved epilogue (four waves, two k-steps per slab, direct stores:
    // the 256x256 and 128x128 tiles with 64-deep slabs): a tile's C leaves
    // between MFMAs instead of after them.
    // Row block fm is final after MFMA fm*FN + FN-1 of the tile's last k-step.
    // Blocks fm < kEpiFirst send each of their FN/2 stores kEpiLag + 2t MFMAs
    // later in that k-step; the rest are final too late for it, and their
    // stores go out in the next tile's first k-step, store t of block fm after
    // MFMA (fm - kEpiFirst)*FN + 2t, before that k-step's first MFMA on block
    // fm.  Half and half (4 of 8 blocks) measured best: the last k-step
    // already carries the slab barrier, most of the next slab's DMAs and its
    // first reads.  A tile's first k-step uses the MFMA with a zero
    // accumulator input (the k == 0 clear), so no accumulator is ever cleared
    // by a register write.
    // A worker's first tile stores nothing in its first k-step (an empty
    // store window); its last tile stores the remaining blocks after the
    // loop.  Stores are two MFMAs apart, so a store's data registers stay
    // intact for 32+ cycles before the next conversion overwrites them (two
    // wait states are required, store_gap).
    constexpr bool kEpiInterleave = TSG_EPI_INTERLEAVE && KS == 2 && EPI == 0 && WGN == 2 && FM % 2 == 0 && FN % 2 == 0;
    static_assert(!PAIR || (kEpiInterleave && FM == 8 && FN == 8), "paired k-steps: 256x256x64 tiles, four waves");
    // MFMAs issued between a block's last MFMA and the first read of its
    // accumulators: the MFMAs are asm the compiler cannot see, so the wait
    // for their results is placed here (3 MFMAs, 48+ cycles)
    constexpr int kEpiLag = 3;
    constexpr int kEpiFirst = TSG_EPI_FIRST * FM / 8;  // row blocks stored in the tile's own last k-step
    static_assert(!kEpiInterleave || (kEpiFirst - 1) * FN + FN - 1 + kEpiLag + 2 * (FN / 2 - 1) < FM * FN,
                  "first-part stores must fit in the k-step");
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
        const int64_t m0 = (int64_t)m_idx * BM, n0 = (int64_t)n_idx * BN;
        e_rows = (uint32_t)((args.M - m0) < BM ? (args.M - m0) : BM);
        e_cols = (uint32_t)((args.N - n0) < BN ? (args.N - n0) : BN);
        e_rc = make_rsrc(args.C + (m0 * args.N + n0), ((e_rows - 1u) * N + e_cols) * 2u);
    };
    // store t of row block fm (16 rows x 32 columns of the wave's sub-tile)
    auto epi_op = [&](auto fm_c, auto t_c) __attribute__((always_inline)) {
        constexpr int fm = decltype(fm_c)::value, t = decltype(t_c)::value;
        const f32x4 x = acc[fm][2 * t], y = acc[fm][2 * t + 1];
        const uint32_t x0 = cvt_pk<DT>(x[0], x[1]), x1 = cvt_pk<DT>(x[2], x[3]);
        const uint32_t y0 = cvt_pk<DT>(y[0], y[1]), y1 = cvt_pk<DT>(y[2], y[3]);
        const u32x4 v = swap ? u32x4{y0, y1, x0, x1} : u32x4{x0, x1, y0, y1};
        const bool ok = row0 + fm * 16 < e_rows && col0 + 32u * t < e_cols;
        __builtin_amdgcn_raw_buffer_store_b128(v, e_rc, (ok ? lane_off : 0x80000000u) + t * 64, fm * 16 * N * 2, TSG_C_CPOL);
    };

    // One 32-deep k-step: FM*FN MFMAs (fm-major) from register set CUR,
    // accumulating into tiles that the epilogue left at zero, or (EPH 2) from
    // a zero accumulator input (the k == 0 clear either way), with the
    // memory operations for what follows between them: the
    // DMAs and the reads of the next k-step into set NXT.  No read
    // into a set starts within kGap MFMAs of the last MFMA that read it: an
    // MFMA may still be fetching its operands, and a second wave on the SIMD
    // can delay it.  LAST (the slab's last k-step) first waits for the next
    // slab and passes the workgroup barrier, then issues the DMA of slab
    // phase+L into the stage just consumed and reads the next slab's first
    // k-step; otherwise it reads k-step KSN of the current stage.  SAME (an
    // odd tail slab) refills set CUR after its MFMAs.
    // EPH: 0 no stores, 1 the current tile's stores of blocks fm < kEpiFirst
    // (its last k-step), 2 the previous tile's other stores (the tile's first
    // k-step, whose MFMAs start from zero).
    // One k-step per slab: the stage the k-steps read, stepped along by the
    // k-step itself (a compare and select in an MFMA gap of its own, pinned
    // like the loader's pieces) instead of recomputed from the slab count.
    // It starts one slot behind: the first k-step steps it to slot 1.
    uint32_t st_rd = 0;
    auto next_stage = [](uint32_t& st) __attribute__((always_inline)) {
        asm volatile("" : "+s"(st));
        st = st == (L - 1) * T::STAGE ? 0u : st + T::STAGE;
        asm volatile("" : "+s"(st));
    };
    // STP: read from st_rd, stepped in gap START - 2 (before the first
    // address add that uses it), instead of from read_st.
    auto kstep = [&](auto cur_c, auto last_c, auto ksn_c, uint32_t read_st, auto same_c, auto eph_c, auto stp_c) __attribute__((always_inline)) {
        constexpr int EPH = decltype(eph_c)::value;
        constexpr int CUR = decltype(cur_c)::value;
        constexpr bool SAME = decltype(same_c)::value;
        constexpr int NXT = SAME ? CUR : 1 - CUR;
        constexpr bool LAST = decltype(last_c)::value;
        constexpr bool STP = decltype(stp_c)::value;
        constexpr int NSTEP = FM * FN;
        constexpr int S0 = LAST ? 2 : 0;                   // MFMAs issued before the barrier
        constexpr int START = S0 > kGap ? S0 : kGap;       // first step with memory operations
        constexpr int AVAIL = NSTEP - START - 1;
        static_assert(AVAIL >= 2, "k-step too short for its memory operations");
        static_assert(!STP || START >= 2, "the stage step needs a gap before the first address add");
        static_assert(LAST ? T::DF <= AVAIL + 1 : NL - T::DF <= AVAIL + 1, "every DMA of a slab needs a gap");
        // LAST issues DMAs [0, DF) of slab phase+L; the following first k-step
        // of the next slab issues [DF, NL) of the same slab
        constexpr int D = LAST ? T::DF : (SAME ? 0 : NL - T::DF);
        constexpr int D0 = LAST ? 0 : T::DF;
        // DMA issues are spaced DS MFMAs apart: a burst of them right after the
        // barrier would overflow the texture unit's queue and stall issue
        constexpr int DS = D ? (AVAIL / (D ? D : 1) < dma_spacing(BK) ? (AVAIL / (D ? D : 1) > 0 ? AVAIL / (D ? D : 1) : 1) : dma_spacing(BK)) : 1;
        constexpr int QR = SAME ? 0 : R;                   // reads, spread evenly
        constexpr int PER = QR ? (QR + AVAIL - 1) / AVAIL : 0;
        // The loader's step, in the k-step that issues a slab's last DMAs: in
        // the first gap after all of this k-step's memory operations, or in
        // the last gap after its DMA when the operations fill the k-step (the
        // DMAs read the descriptors in place, so none may follow the step).
        constexpr int MEM_END = START + (D ? (D - 1) * DS + 1 : 0) > START + (PER ? (QR + PER - 1) / (PER ? PER : 1) : 0)
                                    ? START + (D ? (D - 1) * DS + 1 : 0) : START + (PER ? (QR + PER - 1) / (PER ? PER : 1) : 0);
        constexpr int ADV = MEM_END < NSTEP - 1 ? MEM_END : NSTEP - 1;
        static_for<0, NSTEP>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            // row blocks fm in order; within a row the B blocks forward on even
            // rows and backward on odd ones, so consecutive MFMAs share an
            // operand at every row change too (fewer operand bits switch:
            // measured ~1% more MFMA work per joule on random bf16 data)
            constexpr int fm = s / FN, fn = (fm & 1) ? FN - 1 - s % FN : s % FN;
            const i16x8 bv = __builtin_shufflevector(fb[CUR][fn][0], fb[CUR][fn][1], 0, 1, 2, 3, 4, 5, 6, 7);
            if constexpr (EPH == 2)
                mfma16x16x32_clear<DT>(acc[fm][fn], bv, fa[CUR][fm]);
            else
                mfma16x16x32<DT>(acc[fm][fn], bv, fa[CUR][fm]);
            if constexpr (LAST && s == S0 - 1) {
                stress_pause<0>(wave, stress_ctr);
                wait_vm<(L - 2) * NL < 63 ? (L - 2) * NL : 63>();  // slab phase+1 has landed
                lds_barrier();                                       // ... for every wave; stage phase free
                stress_pause<1>(wave, stress_ctr);
            }
            if constexpr (STP && s == START - 2) next_stage(st_rd);
            if constexpr (s + 1 >= START) {
                // addresses of the reads issued in the next step
                constexpr int p0 = (s + 1 - START) * PER;
                constexpr int p1 = p0 + PER < QR ? p0 + PER : QR;
                static_for<p0, (p1 > p0 ? p1 : p0)>([&](auto q_c) __attribute__((always_inline)) {
                    prep_op(ksn_c, q_c, STP ? st_rd : read_st);
                });
            }
            if constexpr (s >= START) {
                constexpr int i = s - START;
                if constexpr (D && i % DS == 0 && i / DS < D) load_op(std::integral_constant<int, D0 + i / DS>{});
                constexpr int q0 = i * PER;
                constexpr int q1 = q0 + PER < QR ? q0 + PER : QR;
                static_for<q0, q1>([&](auto q_c) __attribute__((always_inline)) {
                    read_op(std::integral_constant<int, NXT>{}, q_c);
                });
            }
            // after this gap's DMA (with short k-steps the last DMA can sit in
            // the gap ADV itself): piece p of the loader's step in gap ADV + p,
            // the pieces that do not fit before the k-step's end in its last gap
            if constexpr (kSplitAdvance ? !LAST : LAST) {
                static_for<0, kAdvPieces>([&](auto p_c) __attribute__((always_inline)) {
                    constexpr int p = decltype(p_c)::value;
                    if constexpr (s == (ADV + p < NSTEP - 1 ? ADV + p : NSTEP - 1)) adv_piece(p_c);
                });
            }
            if constexpr (EPH == 1) {
                static_for<0, kEpiFirst>([&](auto fm_c) __attribute__((always_inline)) {
                    static_for<0, FN / 2>([&](auto t_c) __attribute__((always_inline)) {
                        constexpr int fm = decltype(fm_c)::value, t = decltype(t_c)::value;
                        if constexpr (s == fm * FN + FN - 1 + kEpiLag + 2 * t) epi_op(fm_c, t_c);
                    });
                });
            } else if constexpr (EPH == 2) {
                static_for<kEpiFirst, FM>([&](auto fm_c) __attribute__((always_inline)) {
                    static_for<0, FN / 2>([&](auto t_c) __attribute__((always_inline)) {
                        constexpr int fm = decltype(fm_c)::value, t = decltype(t_c)::value;
                        if constexpr (s == (fm - kEpiFirst) * FN + 2 * t) epi_op(fm_c, t_c);
                    });
                });
            }
            // M0 for the DMA issued in the next step, after this step's load
            if constexpr (D && s + 1 >= START && (s + 1 - START) % DS == 0 && (s + 1 - START) / DS < D)
                m0_op(std::integral_constant<int, D0 + (s + 1 - START) / DS>{});
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (SAME) {
            gap_nops();
            set_addr(ksn_c, STP ? st_rd : read_st);
            static_for<0, R>([&](auto r_c) __attribute__((always_inline)) { read_op(cur_c, r_c); });
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using TRUE_ = std::integral_constant<bool, true>;
    using FALSE_ = std::integral_constant<bool, false>;

    // ---- paired k-steps (PAIR) ----
    // Each slab's two 32-deep k-steps go to every accumulator as two MFMAs in
    // a row: (k-step 0, k-step 1) of block (fm, fn), then the next block.  An
    // MFMA whose accumulator input is the previous MFMA's result takes it from
    // the matrix core's forwarding path instead of the register file, and on
    // random data the board's power limit then allows ~4.7% more MFMA work
    // (microbenchmark of the two orders at the limit).  Every accumulator still
    // sees its k-steps in K order, so C is the k-step-by-k-step order's bit
    // for bit.
    // A slab runs in two phases of FM*FN MFMAs: phase 1 on column blocks
    // fn < FN/2, phase 2 (which opens with the slab barrier, as the last
    // k-step does above) on fn >= FN/2, row blocks in order in both.  So the
    // fragments of both k-steps fit the registers of the two sets above:
    //   B blocks fn >= FN/2 are read in phase 1 (from this slab), those below
    //   in phase 2 (from the next slab), each half while the other is in use;
    //   A row block fm is last read by row fm of phase 2, so blocks
    //   fm < kPA2 are refilled from the next slab there, kGap MFMAs after
    //   that row, and the rest early in the next phase 1.
    // Phase 2 forms the next slab's LDS addresses, issues DMAs [0, DF) of slab
    // phase+L into the stage phase 1 finished reading, and (EPH 1, a tile's
    // last slab) stores column blocks fn < FN/2, final since phase 1; phase 1
    // issues DMAs [DF, NL) and the loader's step, and (EPH 2, a tile's first
    // slab) stores the previous tile's blocks fn >= FN/2 before phase 2
    // overwrites them.  CLR: the tile's first slab (zero accumulator inputs).
    constexpr int kPA2 = FM / 2;              // A row blocks refilled in phase 2
    constexpr int kPR2B = 2 * FN;             // phase 2: B reads (fn < FN/2, both k-steps and halves)
    constexpr int kPR2A = 2 * kPA2;           // phase 2: A reads (fm < kPA2, both k-steps)
    constexpr int kPR1A = 2 * (FM - kPA2);    // phase 1: A reads (fm >= kPA2)
    constexpr int kPR1B = 2 * FN;             // phase 1: B reads (fn >= FN/2)
    constexpr int kPStart = kGap > 2 ? kGap : 2;
    constexpr int kPSteps = FM * FN;
    // gap of phase 2's A read i (row block i/2): after the B reads, and kGap
    // MFMAs after the row's last MFMA in this phase
    constexpr auto p2a_gap = [](int i) constexpr {
        int p = kPStart + kPR2B;
        for (int j = 0; j <= i; ++j) {
            const int e = (j / 2) * FN + FN - 1 + kGap;
            p = p > e ? p : e;
            if (j < i) ++p;
        }
        return p;
    };
    constexpr int kPEpi = FM * FN / 4;        // stores per epilogue half
    constexpr int kPEpiGap = kPSteps - 2 * kPEpi + 1;
    i16x8 pa[FM][2];     // A fragments [row block][k-step]
    i16x4 pb[FN][2][2];  // B fragments [column block][k-step][half]
    uint32_t pra[2], prb[FN];
    auto p_addr_a = [&](auto k_c, uint32_t st) __attribute__((always_inline)) {
        pra[decltype(k_c)::value] = lds_base + st + a_off[decltype(k_c)::value];
    };
    auto p_addr_b = [&](auto fn_c, uint32_t st) __attribute__((always_inline)) {
        prb[decltype(fn_c)::value] = lds_base + st + b_off[decltype(fn_c)::value];
    };
    auto p_read_a = [&](auto fm_c, auto k_c) __attribute__((always_inline)) {
        constexpr int fm = decltype(fm_c)::value, k = decltype(k_c)::value;
        pa[fm][k] = __builtin_bit_cast(i16x8, *(const __attribute__((address_space(3))) u32x4*)(
                                              (__attribute__((address_space(3))) uint8_t*)(uintptr_t)pra[k] + fm * 16 * (BK * 2)));
    };
    auto p_read_b = [&](auto fn_c, auto k_c, auto h_c) __attribute__((always_inline)) {
        constexpr int fn = decltype(fn_c)::value, k = decltype(k_c)::value, h = decltype(h_c)::value;
        pb[fn][k][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)((__attribute__((address_space(3))) uint8_t*)(uintptr_t)prb[fn] + (k * 32 + h * 4) * (BN * 2)));
    };
    // B read r of a phase (column blocks from fn0), A read i (row blocks from fm0)
    auto p_read_b_op = [&](auto fn0_c, auto r_c) __attribute__((always_inline)) {
        constexpr int r = decltype(r_c)::value;
        p_read_b(std::integral_constant<int, decltype(fn0_c)::value + r / 4>{}, std::integral_constant<int, (r / 2) % 2>{},
                 std::integral_constant<int, r % 2>{});
    };
    auto p_read_a_op = [&](auto fm0_c, auto i_c) __attribute__((always_inline)) {
        constexpr int i = decltype(i_c)::value;
        p_read_a(std::integral_constant<int, decltype(fm0_c)::value + i / 2>{}, std::integral_constant<int, i % 2>{});
    };
    // the next slab's LDS addresses (phase 2, and the prologue)
    auto p_addr_op = [&](auto q_c, uint32_t st) __attribute__((always_inline)) {
        constexpr int q = decltype(q_c)::value;  // B blocks < FN/2, A (k-steps 0, 1), B blocks >= FN/2
        if constexpr (q < FN / 2)
            p_addr_b(std::integral_constant<int, q>{}, st);
        else if constexpr (q < FN / 2 + 2)
            p_addr_a(std::integral_constant<int, q - FN / 2>{}, st);
        else
            p_addr_b(std::integral_constant<int, q - 2>{}, st);
    };
    auto pstep = [&](auto ph_c, auto clr_c, auto eph_c, uint32_t st_next) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph_c)::value, EPH = decltype(eph_c)::value;
        constexpr bool CLR = decltype(clr_c)::value, LAST = PH == 2;
        constexpr int NSTEP = kPSteps;
        constexpr int S0 = LAST ? 2 : 0;
        constexpr int START = kPStart;
        constexpr int AVAIL = NSTEP - START - 1;
        constexpr int D = LAST ? T::DF : NL - T::DF;
        constexpr int D0 = LAST ? 0 : T::DF;
        constexpr int DS = D ? (AVAIL / (D ? D : 1) < dma_spacing(BK) ? (AVAIL / (D ? D : 1) > 0 ? AVAIL / (D ? D : 1) : 1) : dma_spacing(BK)) : 1;
        constexpr int DMA_END = D ? START + (D - 1) * DS + 1 : 0;
        constexpr int READ_END = LAST ? p2a_gap(kPR2A - 1) + 1 : START + kPR1A + kPR1B;
        constexpr int MEM_END = DMA_END > READ_END ? DMA_END : READ_END;
        constexpr int ADV = MEM_END < NSTEP - 1 ? MEM_END : NSTEP - 1;
        static_assert(LAST ? p2a_gap(kPR2A - 1) < NSTEP && START + kPR2B <= p2a_gap(0) : READ_END <= NSTEP,
                      "every read of a phase needs a gap");
        static_assert(D <= AVAIL + 1 && kPEpiGap >= kEpiLag, "phase too short for its memory operations");
        static_for<0, NSTEP>([&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            constexpr int pr = s / 2, kk = s % 2;  // MFMA pair, k-step within the slab
            constexpr int fm = pr / (FN / 2), j = pr % (FN / 2);
            constexpr int fn = (LAST ? FN / 2 : 0) + ((fm & 1) ? FN / 2 - 1 - j : j);
            const i16x8 bv = __builtin_shufflevector(pb[fn][kk][0], pb[fn][kk][1], 0, 1, 2, 3, 4, 5, 6, 7);
            if constexpr (CLR && kk == 0)
                mfma16x16x32_clear<DT>(acc[fm][fn], bv, pa[fm][kk]);
            else
                mfma16x16x32<DT>(acc[fm][fn], bv, pa[fm][kk]);
            if constexpr (LAST && s == S0 - 1) {
                stress_pause<0>(wave, stress_ctr);
                wait_vm<(L - 2) * NL < 63 ? (L - 2) * NL : 63>();  // slab phase+1 has landed
                lds_barrier();                                       // ... for every wave; stage phase free
                stress_pause<1>(wave, stress_ctr);
            }
            if constexpr (LAST && s < FN + 2) p_addr_op(std::integral_constant<int, s>{}, st_next);
            if constexpr (s >= START) {
                constexpr int i = s - START;
                if constexpr (D && i % DS == 0 && i / DS < D) load_op(std::integral_constant<int, D0 + i / DS>{});
            }
            if constexpr (LAST) {
                if constexpr (s >= START && s - START < kPR2B) p_read_b_op(I0{}, std::integral_constant<int, s - START>{});
                static_for<0, kPR2A>([&](auto i_c) __attribute__((always_inline)) {
                    if constexpr (p2a_gap(decltype(i_c)::value) == s) p_read_a_op(I0{}, i_c);
                });
            } else {
                if constexpr (s >= START && s - START < kPR1A)
                    p_read_a_op(std::integral_constant<int, kPA2>{}, std::integral_constant<int, s - START>{});
                if constexpr (s >= START + kPR1A && s - START - kPR1A < kPR1B)
                    p_read_b_op(std::integral_constant<int, FN / 2>{}, std::integral_constant<int, s - START - kPR1A>{});
            }
            if constexpr (kSplitAdvance ? !LAST : LAST) {
                static_for<0, kAdvPieces>([&](auto p_c) __attribute__((always_inline)) {
                    constexpr int p = decltype(p_c)::value;
                    if constexpr (s == (ADV + p < NSTEP - 1 ? ADV + p : NSTEP - 1)) adv_piece(p_c);
                });
            }
            if constexpr (EPH != 0 && s >= kPEpiGap && (s - kPEpiGap) % 2 == 0) {
                constexpr int e = (s - kPEpiGap) / 2;  // store e: row block e / (FN/4), t within the half
                constexpr int t = (EPH == 1 ? 0 : FN / 4) + e % (FN / 4);
                epi_op(std::integral_constant<int, e / (FN / 4)>{}, std::integral_constant<int, t>{});
            }
            if constexpr (D && s + 1 >= START && (s + 1 - START) % DS == 0 && (s + 1 - START) / DS < D)
                m0_op(std::integral_constant<int, D0 + (s + 1 - START) / DS>{});
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- epilogue: cast and store one finished tile, then clear its
    // accumulators for the next (the k == 0 clear).  Conversions are volatile
    // asm so each stays next to its store instead of all being hoisted.  Lanes
    // outside C get a vector offset past the descriptor's range and are
    // dropped; the row block goes into the scalar offset.

    // Chunked epilogue (the page's store_block_N path: the cast tile goes to
    // shared memory and leaves in 64-column blocks), EPI = 64.  For chunk c
    // (tile columns 64c .. 64c+63) the two waves holding those columns write
    // their 16-byte pieces (row r, chunk-local 16-byte slot j at r*128 +
    // (j ^ (r mod 8))*16, the same swizzle as the A rows); after a barrier all
    // threads copy whole 128-byte rows out with 16-byte stores (8 threads per
    // row, 32 rows per 256 threads and round); a second barrier frees the
    // buffer for the next chunk.  The rounding is the direct path's, so C is
    // bit-identical.
    auto chunked_store = [&](__amdgpu_buffer_rsrc_t rc, uint32_t rows_left, uint32_t cols_left)
                             __attribute__((always_inline)) {
        if constexpr (EPI) {
            constexpr int CH = BN / EPI;          // chunks per tile
            constexpr int WPC = T::WN / EPI;      // chunks per wave column
            constexpr int ROUNDS = BM * 8 / T::THREADS;
            typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
            const uint32_t chunk = lds_base + T::CHUNK_OFF;
            static_for<0, CH>([&](auto c_c) __attribute__((always_inline)) {
                constexpr int c = decltype(c_c)::value;
                if (wc == (uint32_t)(c / WPC)) {
                    static_for<0, FM>([&](auto fm_c) __attribute__((always_inline)) {
                        constexpr int fm = decltype(fm_c)::value;
                        const uint32_t r = row0 + fm * 16;
                        static_for<0, 2>([&](auto tt_c) __attribute__((always_inline)) {
                            constexpr int tt = decltype(tt_c)::value;
                            constexpr int t = (c % WPC) * 2 + tt;
                            const f32x4 x = acc[fm][2 * t], y = acc[fm][2 * t + 1];
                            const uint32_t x0 = cvt_pk<DT>(x[0], x[1]), x1 = cvt_pk<DT>(x[2], x[3]);
                            const uint32_t y0 = cvt_pk<DT>(y[0], y[1]), y1 = cvt_pk<DT>(y[2], y[3]);
                            const u32x4 v = swap ? u32x4{y0, y1, x0, x1} : u32x4{x0, x1, y0, y1};
                            const uint32_t slot = (4u * tt + lg) ^ (r & 7u);
                            *(lds_u32x4*)((__attribute__((address_space(3))) uint8_t*)(uintptr_t)(chunk + r * 128u + slot * 16u)) = v;
                        });
                    });
                }
                stress_pause<4>(wave, stress_ctr);
                lds_barrier();  // the chunk is complete in LDS
                static_for<0, ROUNDS>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    const uint32_t idx = i * T::THREADS + threadIdx.x;
                    const uint32_t r = idx >> 3, j = idx & 7u;
                    const u32x4 v = *(const lds_u32x4*)((__attribute__((address_space(3))) uint8_t*)(uintptr_t)(
                        chunk + r * 128u + ((j ^ (r & 7u)) * 16u)));
                    const uint32_t col = (uint32_t)c * EPI + 8u * j;
                    const bool ok = r < rows_left && col < cols_left;
                    __builtin_amdgcn_raw_buffer_store_b128(v, rc, ok ? (r * N + col) * 2u : 0x80000000u, 0, TSG_C_CPOL);
                    store_gap();
                });
                stress_pause<5>(wave, stress_ctr);
                lds_barrier();  // every read of the chunk done before it is rewritten
            });
            // the k == 0 clear, once for the whole tile: clearing inside the
            // owner-only branches would make every accumulator a merge of two
            // values and spill
            static_for<0, FM>([&](auto fm_c) __attribute__((always_inline)) {
                static_for<0, FN>([&](auto fn_c) __attribute__((always_inline)) {
                    acc[decltype(fm_c)::value][decltype(fn_c)::value] = f32x4{0.f, 0.f, 0.f, 0.f};
                });
            });
        }
    };

    auto epilogue = [&]() __attribute__((always_inline)) {
        gap_nops();  // the tile's last MFMAs have written their accumulators
        const uint32_t m_idx = sched.m_idx, n_idx = sched.n_idx;
        if (args.trace != nullptr && threadIdx.x == 0) {
            int32_t* row = args.trace + 4 * ((size_t)wid * args.max_iters + sched.iter);
            *(int4*)row = make_int4((int)wid, (int)sched.iter, (int)m_idx, (int)n_idx);
            store_gap();
        }
        const int64_t m0 = (int64_t)m_idx * BM, n0 = (int64_t)n_idx * BN;
        const uint32_t rows_left = (uint32_t)((args.M - m0) < BM ? (args.M - m0) : BM);
        const uint32_t cols_left = (uint32_t)((args.N - n0) < BN ? (args.N - n0) : BN);
        const uint32_t c_bytes = ((rows_left - 1u) * N + cols_left) * 2u;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(args.C + (m0 * args.N + n0), c_bytes);
        if constexpr (EPI) {
            chunked_store(rc, rows_left, cols_left);
        } else {
        static_for<0, FM>([&](auto fm_c) __attribute__((always_inline)) {
            constexpr int fm = decltype(fm_c)::value;
            const bool row_ok = row0 + fm * 16 < rows_left;
            static_for<0, FN / 2>([&](auto t_c) __attribute__((always_inline)) {
                constexpr int t = decltype(t_c)::value;
                const f32x4 x = acc[fm][2 * t], y = acc[fm][2 * t + 1];
                const uint32_t x0 = cvt_pk<DT>(x[0], x[1]), x1 = cvt_pk<DT>(x[2], x[3]);
                const uint32_t y0 = cvt_pk<DT>(y[0], y[1]), y1 = cvt_pk<DT>(y[2], y[3]);
                const u32x4 v = swap ? u32x4{y0, y1, x0, x1} : u32x4{x0, x1, y0, y1};
                const bool ok = row_ok && col0 + 32u * t < cols_left;
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, (ok ? lane_off : 0x80000000u) + t * 64,
                                                       fm * 16 * N * 2, TSG_C_CPOL);
                // the store's data registers are read after it issues: two wait
                // states before the next conversion overwrites them
                store_gap();
                acc[fm][2 * t] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc[fm][2 * t + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        }
    };

    // prologue: slabs 0..L-1 in flight (the last one's DMAs [DF, NL) follow in
    // the first k-step), the first k-step's fragments read
    for (int s = 0; s < L; ++s) {
        if (s + 1 < L) {
            static_for<0, NL>([&](auto q_c) __attribute__((always_inline)) { dma_op(q_c); });
            slab_advance();
        } else {
            static_for<0, T::DF>([&](auto q_c) __attribute__((always_inline)) { dma_op(q_c); });
            if constexpr (!kSplitAdvance) slab_advance();
        }
    }
    stress_pause<3>(wave, stress_ctr);
    wait_vm<(L - 2) * NL + T::DF < 63 ? (L - 2) * NL + T::DF : 63>();
    lds_barrier();
    if constexpr (PAIR) {
        // what the first slab's phase 1 expects the previous phase 2 to have read
        static_for<0, FN + 2>([&](auto q_c) __attribute__((always_inline)) { p_addr_op(q_c, 0u); });
        static_for<0, kPR2B>([&](auto r_c) __attribute__((always_inline)) { p_read_b_op(I0{}, r_c); });
        static_for<0, kPR2A>([&](auto i_c) __attribute__((always_inline)) { p_read_a_op(I0{}, i_c); });
    } else {
        read_all(I0{}, I0{}, 0u);
    }

    // Each slab's last k-step publishes the next slab and reads its first
    // fragments into the other register set.  Two k-steps per slab: sets 0/1
    // alternate inside the slab.  One k-step per slab: slabs go in pairs; an
    // odd last slab refills set 0 after its MFMAs so every tile starts on set 0.
    uint32_t phase = 0;
    bool pend = false;  // a tile's second-half stores are still to go out
    for (sched.init(wid); sched.valid(); sched.next_tile()) {
        if constexpr (PAIR) {
            // one code path per tile (k_blocks >= 2): the first slab's two
            // phases clear, the last slab's phase 2 stores
            pstep(I1{}, TRUE_{}, I2{}, 0u);
            pstep(I2{}, TRUE_{}, I0{}, ((phase + 1u) % L) * T::STAGE);
            ++phase;
            for (uint32_t k = 1; k + 1u < k_blocks; ++k, ++phase) {
                pstep(I1{}, FALSE_{}, I0{}, 0u);
                pstep(I2{}, FALSE_{}, I0{}, ((phase + 1u) % L) * T::STAGE);
            }
            pstep(I1{}, FALSE_{}, I0{}, 0u);
            epi_state();  // after the previous tile's last stores
            pstep(I2{}, FALSE_{}, I1{}, ((phase + 1u) % L) * T::STAGE);
            ++phase;
        } else if constexpr (kEpiInterleave) {
            // rotated: the tile's first k-step, then (last k-step of slab k,
            // first k-step of slab k+1) pairs, then its last k-step; one code
            // path per tile, so the accumulators stay put
            kstep(I0{}, FALSE_{}, I1{}, (phase % L) * T::STAGE, FALSE_{}, I2{}, FALSE_{});
            for (uint32_t k = 0; k + 1u < k_blocks; ++k, ++phase) {
                kstep(I1{}, TRUE_{}, I0{}, ((phase + 1u) % L) * T::STAGE, FALSE_{}, I0{}, FALSE_{});
                kstep(I0{}, FALSE_{}, I1{}, ((phase + 1u) % L) * T::STAGE, FALSE_{}, I0{}, FALSE_{});
            }
            epi_state();  // after the previous tile's last stores
            kstep(I1{}, TRUE_{}, I0{}, ((phase + 1u) % L) * T::STAGE, FALSE_{}, I1{}, FALSE_{});
            ++phase;
        } else if constexpr (KS == 2) {
            for (uint32_t k = 0; k < k_blocks; ++k, ++phase) {
                const uint32_t st_cur = (phase % L) * T::STAGE;
                const uint32_t st_next = ((phase + 1u) % L) * T::STAGE;
                kstep(I0{}, FALSE_{}, I1{}, st_cur, FALSE_{}, I0{}, FALSE_{});
                kstep(I1{}, TRUE_{}, I0{}, st_next, FALSE_{}, I0{}, FALSE_{});
            }
        } else {
            uint32_t k = 0;
            for (; k + 1u < k_blocks; k += 2u) {
                kstep(I0{}, TRUE_{}, I0{}, 0u, FALSE_{}, I0{}, TRUE_{});
                kstep(I1{}, TRUE_{}, I0{}, 0u, FALSE_{}, I0{}, TRUE_{});
            }
            if (k < k_blocks) kstep(I0{}, TRUE_{}, I0{}, 0u, TRUE_{}, I0{}, TRUE_{});
        }
        if constexpr (kEpiInterleave)
            pend = true;
        else
            epilogue();
    }
    if constexpr (kEpiInterleave) {
        if (pend) {
            gap_nops();  // the last tile's last MFMAs have written their accumulators
            if constexpr (PAIR) {
                static_for<0, FM>([&](auto fm_c) __attribute__((always_inline)) {
                    static_for<FN / 4, FN / 2>([&](auto t_c) __attribute__((always_inline)) {
                        epi_op(fm_c, t_c);
                        store_gap();
                        __builtin_amdgcn_sched_barrier(0);
                    });
                });
            } else {
                static_for<kEpiFirst, FM>([&](auto fm_c) __attribute__((always_inline)) {
                    static_for<0, FN / 2>([&](auto t_c) __attribute__((always_inline)) {
                        epi_op(fm_c, t_c);
                        store_gap();
                        __builtin_amdgcn_sched_barrier(0);
                    });
                });
            }
        }
    }
    wait_vm<0>();  // no DMA may still target LDS when the workgroup retires
}

}  // namespace tsg
