// Device helpers shared by the GEMM kernels for gfx950 (CDNA4): vector types,
// the MFMA and conversion wrappers, LDS DMA issue, buffer descriptors, waits
// and barriers, and the XOR swizzles of the LDS slab layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tsg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

enum { DT_FP16 = 1, DT_BF16 = 2 };
#ifndef TSG_DMA_SPACING
#define TSG_DMA_SPACING 0  // 0: 4 MFMAs for 64-deep slabs, 3 for 32-deep (measured best on MI355X)
#endif
// MFMAs between consecutive DMA issues of a wave, for block_K = bk
constexpr int dma_spacing(int bk) { return TSG_DMA_SPACING > 0 ? TSG_DMA_SPACING : (bk == 64 ? 4 : 3); }
#ifndef TSG_DMA_FIRST
#define TSG_DMA_FIRST 14  // DMAs per slab issued in its first k-step of issue (0: all)
#endif
#ifndef TSG_EPI_INTERLEAVE
#define TSG_EPI_INTERLEAVE 1  // four-wave, 64-deep-slab kernels: C stores between the MFMAs
#endif
#ifndef TSG_EPI_FIRST
#define TSG_EPI_FIRST 4  // eighths of a wave's row blocks stored in the tile's last k-step
#endif
#ifndef TSG_GAP
#define TSG_GAP 4
#endif
constexpr int kGap = TSG_GAP;  // MFMAs between the last read of a fragment set and its refill

// Cache policy of the fp16/bf16 kernels' stores of C: nt (bit 1,
// non-temporal) | sc1 (bit 4, device scope, written through).  A wave of
// 256x256 tiles has each XCD write 32 tiles = 4 MiB of C, as much as its whole
// L2; stored as ordinary lines they evicted the A and B slabs the XCD's other
// workgroups were still reading, which then came back from beyond the L2 a
// second time.  Streamed past the L2 they do not: at 8192^3 the reads from
// beyond the L2 fall to the tiling's floor (each XCD fetching its 4 A and 8 B
// panels once per wave).  Each store writes 64 contiguous bytes of 16 rows.
#ifndef TSG_C_CPOL
#define TSG_C_CPOL 18
#endif
// The block-scaled kernel keeps ordinary stores: its 32x32 accumulator layout
// writes only 32 contiguous bytes per row and store, and written through
// unmerged those partial lines nearly double the bytes written, while its fp8
// slabs, half the bytes of fp16 ones, already come from beyond the L2 close to
// once per XCD and wave.
#ifndef TSG_MX_C_CPOL
#define TSG_MX_C_CPOL 0
#endif

// Cache policy of the LDS-DMA loads: sc0, so the L1 does not keep the lines.
// A CU requests every byte of a slab once (the other workgroups sharing a
// panel are on other CUs, and meet in the L2), so there is nothing to keep;
// at 8192^3 this was 0.5% faster, elsewhere the same.  (nt, which also stops
// the L2 keeping them, was 30-60% slower: the L2 is where slabs are shared.)
#ifndef TSG_DMA_MOD
#define TSG_DMA_MOD " sc0"
#endif

#ifndef TSG_STRESS
#define TSG_STRESS 0  // 1: race-detection build, pauses at every synchronisation site (tests only)
#endif

// Race-detection build: a pseudo-random pause of 0 to ~2048 cycles, different
// for every wave, site and call, before and after each workgroup barrier and
// before each LDS-DMA.  Shifting the waves against each other this way makes a
// missing wait (a stage refilled while another wave still reads it, or read
// before its data landed) show up as wrong results.  s_sleep always ends, so a
// pause never hangs a wave.  Compiles to nothing in the normal build.
template <int SITE>
__device__ __forceinline__ void stress_pause(uint32_t wave, uint32_t& ctr) {
    if constexpr (TSG_STRESS != 0) {
        ++ctr;
        const uint32_t h = ((wave + 1u) * 0x9E3779B1u) ^ (ctr * 0x85EBCA77u) ^ ((uint32_t)(SITE + 1) * 0xC2B2AE3Du);
        switch ((h ^ (h >> 15)) & 7u) {
            case 3: __builtin_amdgcn_s_sleep(1); break;
            case 4: __builtin_amdgcn_s_sleep(4); break;
            case 5: __builtin_amdgcn_s_sleep(8); break;
            case 6: __builtin_amdgcn_s_sleep(16); break;
            case 7: __builtin_amdgcn_s_sleep(32); break;
            default: break;
        }
    } else {
        (void)wave;
        (void)ctr;
    }
}

// Wait states the compiler cannot place itself, because the instructions
// involved sit inside inline asm (its hazard recognizer does not look into an
// asm block for these pairs).  The counts are the ones gfx950 code generation
// inserts for the same pairs written with compiler-visible instructions:
//   gap_nops:  a 16x16x32 MFMA's result -> a VALU read of it (here the
//              v_accvgpr_read of the conversion): 8 wait states (s_nop 7);
//   store_gap: a 16-byte buffer store -> a write of its data registers: 2
//              (s_nop 1; the compiler adds the same two itself when the
//              writer is an asm block, so this is a second guard).
__device__ __forceinline__ void gap_nops() { asm volatile("s_nop 7" ::: "memory"); }
__device__ __forceinline__ void store_gap() { asm volatile("s_nop 1" ::: "memory"); }
constexpr uint32_t kRawBufferFlags = 0x00020000u;  // gfx9 raw buffer: 32-bit data format, no swizzle

struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    uint16_t* C;
    int32_t* trace;  // optional (worker, iter, m, n) per processed tile
    int64_t M, N, K;
    uint32_t m_blocks, n_blocks, k_blocks, group;
    uint32_t P, max_iters, num_xcd;
    uint32_t num_active;          // workers with at least one tile (worker numbering)
    uint32_t cluster, col_major;  // tile scheduler options
    uint32_t prefetch;            // 1: workers without a tile warm their XCD's L2 (timing only)
};

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
// acc += a * b on the 16x16x32 matrix core.  Written as asm with the
// accumulator constrained to AGPRs: each 16x16 fp32 tile stays in one fixed
// AGPR quad for the whole kernel and the VGPRs are left to the fragments.
template <int DT>
__device__ __forceinline__ void mfma16x16x32(f32x4& acc, i16x8 a, i16x8 b) {
    if constexpr (DT == DT_FP16)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same MFMA with a zero accumulator input (the k == 0 clear): acc = a*b.
template <int DT>
__device__ __forceinline__ void mfma16x16x32_clear(f32x4& acc, i16x8 a, i16x8 b) {
    if constexpr (DT == DT_FP16)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}

// Two fp32 accumulators (held in AGPRs) -> one dword of two 16-bit values
// (low half = a), round to nearest even.  The AGPR reads sit inside the asm so
// they happen at the store that needs them rather than all up front.
template <int DT>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    uint32_t r, t;
    if constexpr (DT == DT_FP16)
        asm volatile("v_accvgpr_read_b32 %0, %2\n\tv_accvgpr_read_b32 %1, %3\n\tv_cvt_pk_f16_f32 %0, %0, %1"
                     : "=&v"(r), "=&v"(t) : "a"(a), "a"(b));
    else
        asm volatile("v_accvgpr_read_b32 %0, %2\n\tv_accvgpr_read_b32 %1, %3\n\tv_cvt_pk_bf16_f32 %0, %0, %1"
                     : "=&v"(r), "=&v"(t) : "a"(a), "a"(b));
    return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kRawBufferFlags);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// All LDS reads of this wave done, then workgroup barrier.  The wait is the
// builtin, not asm, so the compiler's own wait insertion knows every earlier
// LDS read has completed and adds no stale lgkmcnt waits after it; the empty
// asm statements are compiler memory barriers, so no LDS access moves across.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    // gfx9 s_waitcnt: lgkmcnt(0), vmcnt and expcnt left at their maxima
    __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}


// Swizzled 16-byte chunk slot of logical chunk c in LDS row r.
template <int CA>
__device__ __forceinline__ uint32_t swz_a(uint32_t r) {
    // 8 consecutive rows at one logical chunk land on 8 distinct bank groups
    return CA == 8 ? (r & 7u) : ((r >> 1) & 3u);
}
__device__ __forceinline__ uint32_t swz_b(uint32_t kr) {
    // the 4 rows of one transpose read, and the two row octets a wave reads
    // together, land on distinct bank groups
    const uint32_t s = (kr & 1u) | ((kr & 2u) << 1);  // 0,1,4,5 for kr%4 = 0..3
    return s | (((kr >> 3) & 1u) << 3);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Descriptor words from a byte address held in scalar registers.
__device__ __forceinline__ i32x4 rsrc_words_u64(uint64_t a, uint32_t bytes) {
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));  // stride 0
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = (int)kRawBufferFlags;
    return r;
}

// One 16-byte-per-lane DMA from a buffer into LDS, its LDS target base + OFF
// written to M0 inside the same asm (one scalar instruction next to the DMA;
// s_nop: the wait state between an M0 write and the LDS-DMA that uses it).
// Inline asm, so the compiler does not treat every later LDS read as
// dependent on it (it cannot tell the stage being filled from the stage
// being read); the kernel waits on vmcnt itself before the barrier that
// publishes a stage.  Every M0 write in the kernels is inside these helpers:
// no asm operand asks the compiler for a value in M0.
template <uint32_t OFF>
__device__ __forceinline__ void dma16_at(uint32_t lds_base_addr, uint32_t voff, i32x4 rsrc) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen" TSG_DMA_MOD " lds"
                 ::"v"(voff), "s"(rsrc), "s"(lds_base_addr), "i"(OFF)
                 : "memory", "m0", "scc");
}

// The LDS-DMA in two pieces: M0 = base + OFF, and later the load that uses
// it.  The caller keeps other M0 writers out from between them and leaves at
// least one instruction between the two (the M0-to-LDS-DMA wait state).
template <uint32_t OFF>
__device__ __forceinline__ void set_m0(uint32_t lds_base_addr) {
    asm volatile("s_add_u32 m0, %0, %1" ::"s"(lds_base_addr), "i"(OFF) : "m0", "scc");
}
__device__ __forceinline__ void dma16_m0(uint32_t voff, i32x4 rsrc) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen" TSG_DMA_MOD " lds" ::"v"(voff), "s"(rsrc) : "memory");
}

}  // namespace tsg
