// libtsgemm: C ABI around the persistent tile-scheduled GEMM kernels
// (declarations and contracts: include/tsgemm.h).  The kernels themselves
// are compiled in their own translation units (tsgemm_launch.h).
//
// Host conventions follow the lowered host code on page "tilelang" (blog,
// section 1.3): argument checks before any launch, 0 / negative return codes,
// and the failure message kept for a get_last_error() call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "tsgemm.h"
#include "tile_scheduler.h"
#include "tsgemm_launch.h"
#include "tsgemm_mx_kernel.h"

namespace tsg {

// C = 0 when K == 0 (an empty sum): plain 16-byte stores, N % 8 == 0.
__global__ void tsgemm_zero_kernel(uint16_t* C, int64_t count8) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count8) *(u32x4*)(C + 8 * i) = u32x4{0u, 0u, 0u, 0u};
}

// Schedule dump: the same scheduler and worker numbering as the GEMM kernel.
__global__ void tsgemm_schedule_kernel(uint32_t P, uint32_t m_blocks, uint32_t n_blocks,
                                       uint32_t group, uint32_t cluster, uint32_t col_major,
                                       uint32_t num_xcd, uint32_t num_active, uint32_t max_iters, int32_t* out) {
    if (threadIdx.x != 0) return;
    const uint32_t wid = worker_of_workgroup(blockIdx.x, P, num_xcd, num_active);
    TileScheduler s;
    s.setup(P, m_blocks, n_blocks, group, cluster, col_major);
    for (s.init(wid); s.valid(); s.next_tile()) {
        int32_t* row = out + 4 * ((size_t)wid * max_iters + s.iter);
        *(int4*)row = make_int4((int)wid, (int)s.iter, (int)s.m_idx, (int)s.n_idx);
    }
}

}  // namespace tsg

namespace {

using tsg::KernelEntry;
using tsg::kLdsBytes;
constexpr int kMaxSlots = 5;           // deepest compiled LDS ring

thread_local char g_err[512] = "";
thread_local int g_code = 0;

// Every entry point starts by clearing the last error of its thread.
void reset_error() {
    g_err[0] = '\0';
    g_code = 0;
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    g_code = code;
    return code;
}

// Every compiled fp16/bf16 kernel, gathered from the translation units that
// build them (one per dtype and tile shape).
struct KernelTable {
    std::vector<KernelEntry> entries;
    KernelTable() {
        typedef const KernelEntry* (*tu_fn)(int*);
        const tu_fn tus[] = {tsg::TSG_GEMM_TU_FN(1, 128, 32), tsg::TSG_GEMM_TU_FN(1, 128, 64),
                             tsg::TSG_GEMM_TU_FN(1, 256, 32), tsg::TSG_GEMM_TU_FN(1, 256, 64),
                             tsg::TSG_GEMM_TU_FN(2, 128, 32), tsg::TSG_GEMM_TU_FN(2, 128, 64),
                             tsg::TSG_GEMM_TU_FN(2, 256, 32), tsg::TSG_GEMM_TU_FN(2, 256, 64)};
        for (tu_fn f : tus) {
            int n = 0;
            const KernelEntry* e = f(&n);
            entries.insert(entries.end(), e, e + n);
        }
    }
};

const std::vector<KernelEntry>& kernels() {
    static const KernelTable table;  // thread-safe one-time construction
    return table.entries;
}

// Default wavefronts per workgroup for a tile shape (measured on MI355X).
int default_waves(int bm, int bn, int bk) {
    (void)bm; (void)bn; (void)bk;
    return 4;
}

const KernelEntry* find_kernel(int dt, int bm, int bn, int bk, int slots, int waves, int epi) {
    for (const KernelEntry& e : kernels())
        if (e.dt == dt && e.bm == bm && e.bn == bn && e.bk == bk && e.slots == slots && e.waves == waves &&
            e.epi == epi)
            return &e;
    return nullptr;
}

// LDS ring depth in block_K slabs: min(num_stages, (LDS - epilogue buffer) /
// stage, kMaxSlots); 0 when two stages do not fit.
int ring_slots(int bm, int bn, int bk, int stages, int epi = 0) {
    const int stage = (bm * bk + bk * bn) * 2;
    int slots = (kLdsBytes - bm * epi * 2) / stage;
    if (slots > stages) slots = stages;
    if (slots > kMaxSlots) slots = kMaxSlots;
    return slots >= 2 ? slots : 0;
}

bool tile_supported(int bm, int bn, int bk) {
    return (bm == 128 && bn == 128 && (bk == 32 || bk == 64)) ||
           (bm == 256 && bn == 256 && (bk == 32 || bk == 64));
}

// Persistent grid default: one workgroup per compute unit of the device; the
// XCD count (accelerator complex dies, each with its own L2) drives the
// worker renumbering.  Both are queried once per device and cached.
std::atomic<int> g_cu_count[64];
std::atomic<int> g_xcd_count[64];

int device_cus(int* cus, int* xcds) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TSGEMM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    const bool cached = dev >= 0 && dev < 64;
    int n = cached ? g_cu_count[dev].load() : 0;
    int x = cached ? g_xcd_count[dev].load() : 0;
    if (n <= 0 || x <= 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess || n <= 0)
            return fail(TSGEMM_EHIP, "cannot query the compute-unit count: %s", hipGetErrorString(e));
        // Workgroup b of a launch goes to XCD b % (XCD count).  A runtime that
        // cannot report the count gets 1: the renumbering is then the
        // identity, which changes speed only, never C or the schedule.
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0) {
            (void)hipGetLastError();
            x = 1;
        }
        if (cached) {
            g_cu_count[dev].store(n);
            g_xcd_count[dev].store(x);
        }
    }
    *cus = n;
    *xcds = x;
    return TSGEMM_OK;
}

}  // namespace

struct tsgemm_plan {
    int64_t M, N, K;
    int dtype, bm, bn, bk, group, stages, slots;
    int64_t m_blocks, n_blocks, k_blocks, tiles;
    int P;         // 0 = default (compute units)
    int xcd_remap; // 1 = permute workgroups so each XCD runs consecutive worker ids
    int cluster;   // workgroups per cluster (tile scheduler option), >= 1
    int col_major; // 1 = transposed tile walk (tile scheduler option)
    int epi;       // 0 = direct stores, 64 = C staged through LDS in 64-column chunks
    int prefetch;  // 1 = workers without a tile warm their XCD's L2 (fp16/bf16 kernels)
    const KernelEntry* kernel;  // fp16/bf16 kernel; NULL for an MXFP8 plan
};

namespace {

struct Grid {
    uint32_t P, xcds, max_iters;
    uint32_t active;  // workers with at least one tile: whole clusters, at most P
};

bool is_mx(const tsgemm_plan* p) { return p->dtype == TSGEMM_MXFP8; }

// Bytes of one LDS stage: the A and B slabs (and for MXFP8 their scale bytes,
// 4 per row and 128-deep slab).
int stage_bytes_of(int dtype, int bm, int bn, int bk) {
    return dtype == TSGEMM_MXFP8 ? (bm + bn) * (bk + 4) : (bm * bk + bk * bn) * 2;
}

// Waves of the longest-running workgroup: its cluster's share of the
// ceil(m_blocks / cluster) x n_blocks cluster tiles.
uint32_t max_iters_for(const tsgemm_plan* p, uint32_t P) {
    const int64_t clusters = P / (uint32_t)p->cluster;
    const int64_t m_cl = (p->m_blocks + p->cluster - 1) / p->cluster;
    return (uint32_t)((m_cl * p->n_blocks + clusters - 1) / clusters);
}

int resolve_grid(const tsgemm_plan* p, Grid* g) {
    int cus = 0, xcds = 1;
    if (p->P == 0 || p->xcd_remap) {
        int rc = device_cus(&cus, &xcds);
        if (rc != TSGEMM_OK) return rc;
    }
    g->P = (uint32_t)(p->P ? p->P : cus);
    g->xcds = p->xcd_remap ? (uint32_t)xcds : 1u;
    if (g->P % (uint32_t)p->cluster != 0)
        return fail(TSGEMM_EINVAL, "the %u workgroups do not split into clusters of %d", g->P, p->cluster);
    g->max_iters = max_iters_for(p, g->P);
    const int64_t clusters = g->P / (uint32_t)p->cluster;
    const int64_t cluster_tiles = (p->m_blocks + p->cluster - 1) / p->cluster * p->n_blocks;
    g->active = (uint32_t)((cluster_tiles < clusters ? cluster_tiles : clusters) * p->cluster);
    if (g->active == 0) g->active = g->P;  // no tiles: nothing to spread
    return TSGEMM_OK;
}

int run_impl(const tsgemm_plan* p, const void* A, const void* B, void* C, void* stream, int32_t* trace) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (is_mx(p)) return fail(TSGEMM_EINVAL, "an MXFP8 plan runs with tsgemm_run_mx");
    if (p->M == 0 || p->N == 0) return TSGEMM_OK;  // empty output: nothing to launch
    if (!C) return fail(TSGEMM_EINVAL, "C is NULL");
    if (p->K > 0 && (!A || !B)) return fail(TSGEMM_EINVAL, "A or B is NULL");
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) | reinterpret_cast<uintptr_t>(C)) & 15u)
        return fail(TSGEMM_EINVAL, "A, B and C must be 16-byte aligned");
    Grid g;
    int rc = resolve_grid(p, &g);
    if (rc != TSGEMM_OK) return rc;
    tsg::GemmArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = static_cast<uint16_t*>(C);
    a.trace = trace;
    a.M = p->M;
    a.N = p->N;
    a.K = p->K;
    a.m_blocks = (uint32_t)p->m_blocks;
    a.n_blocks = (uint32_t)p->n_blocks;
    a.k_blocks = (uint32_t)p->k_blocks;
    a.group = (uint32_t)p->group;
    a.P = g.P;
    a.max_iters = g.max_iters;
    a.num_xcd = g.xcds;
    a.num_active = g.active;
    a.cluster = (uint32_t)p->cluster;
    a.col_major = (uint32_t)p->col_major;
    a.prefetch = p->prefetch && g.active < g.P ? 1u : 0u;
    (void)hipGetLastError();
    if (p->k_blocks == 0) {
        // empty sum: C = 0 (N % 8 == 0, so 8 elements per thread)
        const int64_t count8 = p->M * p->N / 8;
        const unsigned blocks = (unsigned)((count8 + 255) / 256);
        hipLaunchKernelGGL(tsg::tsgemm_zero_kernel, dim3(blocks), dim3(256), 0,
                           static_cast<hipStream_t>(stream), a.C, count8);
    } else {
        p->kernel->fn(a, g.P, static_cast<hipStream_t>(stream));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TSGEMM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return TSGEMM_OK;
}

// Scale groups per tile column of K (SG slabs each) and bytes of one packed
// scale array for `blocks` row (or column) blocks.
uint32_t mx_groups(const tsgemm_plan* p) {
    return (uint32_t)((p->k_blocks + tsg::MxTraits::SG - 1) / tsg::MxTraits::SG);
}
int64_t mx_packed_bytes(const tsgemm_plan* p, int64_t blocks) {
    return blocks * (int64_t)mx_groups(p) * tsg::MxTraits::BM * tsg::MxTraits::SC_ROW;
}

int run_mx_impl(const tsgemm_plan* p, const void* A, const void* SFA, const void* B, const void* SFB, void* C,
                void* stream, int32_t* trace, bool packed) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (!is_mx(p)) return fail(TSGEMM_EINVAL, "tsgemm_run_mx needs a TSGEMM_MXFP8 plan (dtype %d)", p->dtype);
    if (p->M == 0 || p->N == 0) return TSGEMM_OK;
    if (!C) return fail(TSGEMM_EINVAL, "C is NULL");
    if (p->K > 0 && (!A || !B || !SFA || !SFB)) return fail(TSGEMM_EINVAL, "A, SFA, B or SFB is NULL");
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) | reinterpret_cast<uintptr_t>(C)) & 15u)
        return fail(TSGEMM_EINVAL, "A, B and C must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(SFA) | reinterpret_cast<uintptr_t>(SFB)) & (packed ? 15u : 3u))
        return fail(TSGEMM_EINVAL, packed ? "packed SFA and SFB must be 16-byte aligned"
                                          : "SFA and SFB must be 4-byte aligned");
    Grid g;
    int rc = resolve_grid(p, &g);
    if (rc != TSGEMM_OK) return rc;
    (void)hipGetLastError();
    if (p->k_blocks == 0) {
        const int64_t count8 = p->M * p->N / 8;
        const unsigned blocks = (unsigned)((count8 + 255) / 256);
        hipLaunchKernelGGL(tsg::tsgemm_zero_kernel, dim3(blocks), dim3(256), 0,
                           static_cast<hipStream_t>(stream), static_cast<uint16_t*>(C), count8);
    } else {
        tsg::MxArgs a;
        a.A = static_cast<const uint8_t*>(A);
        a.SFA = static_cast<const uint8_t*>(SFA);
        a.B = static_cast<const uint8_t*>(B);
        a.SFB = static_cast<const uint8_t*>(SFB);
        a.C = static_cast<uint16_t*>(C);
        a.trace = trace;
        a.M = p->M;
        a.N = p->N;
        a.K = p->K;
        a.m_blocks = (uint32_t)p->m_blocks;
        a.n_blocks = (uint32_t)p->n_blocks;
        a.k_blocks = (uint32_t)p->k_blocks;
        a.group = (uint32_t)p->group;
        a.P = g.P;
        a.max_iters = g.max_iters;
        a.num_xcd = g.xcds;
        a.num_active = g.active;
        a.cluster = (uint32_t)p->cluster;
        a.col_major = (uint32_t)p->col_major;
        a.n_groups = mx_groups(p);
        tsg::launch_mx(a, g.P, packed, static_cast<hipStream_t>(stream));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TSGEMM_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return TSGEMM_OK;
}

}  // namespace

extern "C" {

const char* tsgemm_last_error(void) { return g_err; }

int tsgemm_last_error_code(void) { return g_code; }

tsgemm_plan* tsgemm_create(int64_t M, int64_t N, int64_t K, int dtype, int block_M, int block_N,
                           int block_K, int group_size, int num_stages) {
    reset_error();
    if (M < 0 || N < 0 || K < 0) { fail(TSGEMM_EINVAL, "M, N, K must be >= 0"); return nullptr; }
    if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31)) {
        fail(TSGEMM_EINVAL, "M, N and K must be below 2^31"); return nullptr;
    }
    if (dtype != TSGEMM_FP16 && dtype != TSGEMM_BF16 && dtype != TSGEMM_MXFP8) {
        fail(TSGEMM_EINVAL, "dtype must be TSGEMM_FP16 (1), TSGEMM_BF16 (2) or TSGEMM_MXFP8 (3), got %d", dtype);
        return nullptr;
    }
    if (block_M <= 0 || block_N <= 0 || block_K <= 0) { fail(TSGEMM_EINVAL, "block sizes must be positive"); return nullptr; }
    if (group_size < 1) { fail(TSGEMM_EINVAL, "group_size must be >= 1, got %d", group_size); return nullptr; }
    if (num_stages < 2) { fail(TSGEMM_EINVAL, "num_stages must be >= 2, got %d", num_stages); return nullptr; }
    if (K % block_K != 0) {
        fail(TSGEMM_EINVAL, "K (%lld) must be a multiple of block_K (%d)", (long long)K, block_K); return nullptr;
    }
    if (N % 8 != 0 || K % 8 != 0) {
        fail(TSGEMM_EINVAL, "N and K must be divisible by 8 (16-byte rows)"); return nullptr;
    }
    if (dtype == TSGEMM_MXFP8) {
        if (block_M != 256 || block_N != 256 || block_K != 128) {
            fail(TSGEMM_EUNSUPPORTED, "MXFP8 tile %dx%dx%d is not compiled (have 256x256x128)", block_M, block_N, block_K);
            return nullptr;
        }
    } else if (!tile_supported(block_M, block_N, block_K)) {
        fail(TSGEMM_EUNSUPPORTED, "tile %dx%dx%d is not compiled (have 128x128x{32,64}, 256x256x{32,64})",
             block_M, block_N, block_K);
        return nullptr;
    }
    const int64_t lim = int64_t(1) << 31;
    if (dtype == TSGEMM_MXFP8) {
        if (int64_t(block_M) * K >= lim || int64_t(block_N) * K >= lim || int64_t(block_M) * N * 2 >= lim) {
            fail(TSGEMM_EUNSUPPORTED, "a tile's byte extent (block_M*K, block_N*K, block_M*N*2) exceeds 2^31");
            return nullptr;
        }
    } else if (int64_t(block_M) * K * 2 >= lim || int64_t(block_K) * N * 2 >= lim || int64_t(block_M) * N * 2 >= lim) {
        fail(TSGEMM_EUNSUPPORTED, "a tile's byte extent (block_M*K*2, block_K*N*2, block_M*N*2) exceeds 2^31");
        return nullptr;
    }
    const int stage = stage_bytes_of(dtype, block_M, block_N, block_K);
    const int slots = dtype == TSGEMM_MXFP8 ? 2 : ring_slots(block_M, block_N, block_K, num_stages);
    if (slots < 2) { fail(TSGEMM_EUNSUPPORTED, "two %d-byte stages do not fit in LDS", stage); return nullptr; }
    const int64_t mb = (M + block_M - 1) / block_M, nb = (N + block_N - 1) / block_N;
    if (mb * nb >= lim) { fail(TSGEMM_EUNSUPPORTED, "tile count must be below 2^31"); return nullptr; }
    const KernelEntry* k = dtype == TSGEMM_MXFP8
                               ? nullptr
                               : find_kernel(dtype, block_M, block_N, block_K, slots, default_waves(block_M, block_N, block_K), 0);
    if (!k && dtype != TSGEMM_MXFP8) { fail(TSGEMM_EUNSUPPORTED, "no kernel for this configuration"); return nullptr; }
    tsgemm_plan* p = new (std::nothrow) tsgemm_plan;
    if (!p) { fail(TSGEMM_ENOMEM, "out of host memory"); return nullptr; }
    p->M = M; p->N = N; p->K = K;
    p->dtype = dtype; p->bm = block_M; p->bn = block_N; p->bk = block_K;
    p->group = group_size; p->stages = num_stages; p->slots = slots;
    p->m_blocks = mb; p->n_blocks = nb; p->k_blocks = K / block_K; p->tiles = mb * nb;
    p->P = 0; p->xcd_remap = 1; p->cluster = 1; p->col_major = 0; p->epi = 0; p->prefetch = k ? 1 : 0; p->kernel = k;
    return p;
}

int tsgemm_set_num_workgroups(tsgemm_plan* p, int num_workgroups) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (num_workgroups < 0) return fail(TSGEMM_EINVAL, "num_workgroups must be >= 0");
    p->P = num_workgroups;
    return TSGEMM_OK;
}

int tsgemm_set_waves(tsgemm_plan* p, int waves) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (waves == 0) waves = default_waves(p->bm, p->bn, p->bk);
    if (waves != 4 && waves != 8) return fail(TSGEMM_EINVAL, "waves must be 0, 4 or 8, got %d", waves);
    if (is_mx(p)) return waves == 4 ? TSGEMM_OK : fail(TSGEMM_EUNSUPPORTED, "the MXFP8 kernel runs 4 waves");
    const KernelEntry* k = find_kernel(p->dtype, p->bm, p->bn, p->bk, p->slots, waves, p->epi);
    if (!k) return fail(TSGEMM_EUNSUPPORTED, "no %d-wave kernel for this configuration%s", waves,
                        p->epi ? " with the chunked epilogue" : "");
    p->kernel = k;
    return TSGEMM_OK;
}

int tsgemm_set_epilogue(tsgemm_plan* p, int store_block_N) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (store_block_N != 0 && store_block_N != 64)
        return fail(TSGEMM_EINVAL, "store_block_N must be 0 (direct stores) or 64, got %d", store_block_N);
    if (is_mx(p))
        return store_block_N ? fail(TSGEMM_EUNSUPPORTED, "the MXFP8 kernel stores directly") : TSGEMM_OK;
    const int slots = ring_slots(p->bm, p->bn, p->bk, p->stages, store_block_N);
    if (slots < 2) return fail(TSGEMM_EUNSUPPORTED, "two stages and the epilogue buffer do not fit in LDS");
    const KernelEntry* k = find_kernel(p->dtype, p->bm, p->bn, p->bk, slots, p->kernel->waves, store_block_N);
    if (!k) return fail(TSGEMM_EUNSUPPORTED, "no %d-wave kernel with store_block_N %d", p->kernel->waves, store_block_N);
    p->kernel = k;
    p->slots = slots;
    p->epi = store_block_N;
    return TSGEMM_OK;
}

int tsgemm_set_xcd_remap(tsgemm_plan* p, int enable) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (enable != 0 && enable != 1) return fail(TSGEMM_EINVAL, "enable must be 0 or 1");
    p->xcd_remap = enable;
    return TSGEMM_OK;
}

int tsgemm_set_l2_prefetch(tsgemm_plan* p, int enable) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (enable != 0 && enable != 1) return fail(TSGEMM_EINVAL, "enable must be 0 or 1");
    if (enable && is_mx(p)) return fail(TSGEMM_EUNSUPPORTED, "the MXFP8 kernel does not warm the L2");
    p->prefetch = enable;
    return TSGEMM_OK;
}

int tsgemm_set_schedule(tsgemm_plan* p, int column_major, int cluster_size) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (column_major != 0 && column_major != 1) return fail(TSGEMM_EINVAL, "column_major must be 0 or 1");
    if (cluster_size < 1 || cluster_size > 64) return fail(TSGEMM_EINVAL, "cluster_size must be in [1, 64], got %d", cluster_size);
    p->col_major = column_major;
    p->cluster = cluster_size;
    return TSGEMM_OK;
}

int tsgemm_run(const tsgemm_plan* p, const void* A, const void* B, void* C, void* stream) {
    return run_impl(p, A, B, C, stream, nullptr);
}

int tsgemm_run_traced(const tsgemm_plan* p, const void* A, const void* B, void* C, void* stream,
                      int32_t* trace) {
    if (!trace) return fail(TSGEMM_EINVAL, "trace is NULL");
    return run_impl(p, A, B, C, stream, trace);
}

int tsgemm_run_mx(const tsgemm_plan* p, const void* A, const void* SFA, const void* B, const void* SFB, void* C,
                  void* stream) {
    return run_mx_impl(p, A, SFA, B, SFB, C, stream, nullptr, false);
}

int tsgemm_run_mx_traced(const tsgemm_plan* p, const void* A, const void* SFA, const void* B, const void* SFB,
                         void* C, void* stream, int32_t* trace) {
    if (!trace) return fail(TSGEMM_EINVAL, "trace is NULL");
    return run_mx_impl(p, A, SFA, B, SFB, C, stream, trace, false);
}

int64_t tsgemm_mx_packed_scale_bytes(const tsgemm_plan* p, int operand) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (!is_mx(p)) return fail(TSGEMM_EINVAL, "not a TSGEMM_MXFP8 plan (dtype %d)", p->dtype);
    if (operand != 0 && operand != 1) return fail(TSGEMM_EINVAL, "operand must be 0 (SFA) or 1 (SFB), got %d", operand);
    return mx_packed_bytes(p, operand == 0 ? p->m_blocks : p->n_blocks);
}

int tsgemm_mx_pack_scales(const tsgemm_plan* p, int operand, const void* SF, void* SFP, void* stream) {
    const int64_t bytes = tsgemm_mx_packed_scale_bytes(p, operand);
    if (bytes < 0) return (int)bytes;
    if (bytes == 0) return TSGEMM_OK;  // no rows or K == 0: nothing to pack
    if (!SF || !SFP) return fail(TSGEMM_EINVAL, "SF or SFP is NULL");
    if ((reinterpret_cast<uintptr_t>(SF) & 3u) || (reinterpret_cast<uintptr_t>(SFP) & 15u))
        return fail(TSGEMM_EINVAL, "SF must be 4-byte and SFP 16-byte aligned");
    const int64_t rows = operand == 0 ? p->M : p->N;
    const int64_t blocks = operand == 0 ? p->m_blocks : p->n_blocks;
    const int64_t dwords = bytes / 4;
    (void)hipGetLastError();
    tsg::launch_mx_pack(static_cast<const uint8_t*>(SF), static_cast<uint8_t*>(SFP), rows, (uint32_t)(p->K / 32),
                        (uint32_t)blocks, mx_groups(p), (unsigned)((dwords + 255) / 256),
                        static_cast<hipStream_t>(stream));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TSGEMM_EHIP, "pack kernel launch failed: %s", hipGetErrorString(e));
    return TSGEMM_OK;
}

int tsgemm_run_mx_packed(const tsgemm_plan* p, const void* A, const void* SFAP, const void* B, const void* SFBP,
                         void* C, void* stream) {
    return run_mx_impl(p, A, SFAP, B, SFBP, C, stream, nullptr, true);
}

int tsgemm_run_mx_noalloc(const tsgemm_plan* p, const void* A, const void* SFA, const void* B, const void* SFB,
                          void* C, void* stream) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (!is_mx(p)) return fail(TSGEMM_EINVAL, "tsgemm_run_mx_noalloc needs a TSGEMM_MXFP8 plan (dtype %d)", p->dtype);
    if (p->M == 0 || p->N == 0) return TSGEMM_OK;
    // packed SFA at the workspace start, packed SFB at the next 256-byte boundary
    const int64_t a_bytes = mx_packed_bytes(p, p->m_blocks), b_bytes = mx_packed_bytes(p, p->n_blocks);
    const int64_t b_off = (a_bytes + 255) / 256 * 256;
    if (b_off + b_bytes > tsg::kMxScratchBytes)
        return fail(TSGEMM_EUNSUPPORTED,
                    "the packed scales need %lld bytes; the static workspace of tsgemm_run_mx_noalloc holds %lld",
                    (long long)(b_off + b_bytes), (long long)tsg::kMxScratchBytes);
    if (p->k_blocks == 0) return run_mx_impl(p, A, SFA, B, SFB, C, stream, nullptr, false);  // C = 0, no scales
    if (!A || !B || !C || !SFA || !SFB) return fail(TSGEMM_EINVAL, "A, SFA, B, SFB or C is NULL");
    if ((reinterpret_cast<uintptr_t>(SFA) | reinterpret_cast<uintptr_t>(SFB)) & 3u)
        return fail(TSGEMM_EINVAL, "SFA and SFB must be 4-byte aligned");
    void* ws = nullptr;
    hipError_t e = tsg::mx_scratch_address(&ws);
    if (e != hipSuccess) return fail(TSGEMM_EHIP, "workspace address: %s", hipGetErrorString(e));
    uint8_t* sfap = static_cast<uint8_t*>(ws);
    uint8_t* sfbp = sfap + b_off;
    // the pack kernels write every byte of both packed arrays (zeros past the
    // data), so nothing a previous call left in the workspace is read
    int rc = tsgemm_mx_pack_scales(p, 0, SFA, sfap, stream);
    if (rc == TSGEMM_OK) rc = tsgemm_mx_pack_scales(p, 1, SFB, sfbp, stream);
    if (rc != TSGEMM_OK) return rc;
    return run_mx_impl(p, A, sfap, B, sfbp, C, stream, nullptr, true);
}

int64_t tsgemm_num_tiles(const tsgemm_plan* p) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    return p->tiles;
}

int tsgemm_num_workgroups(const tsgemm_plan* p) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    if (p->P) return p->P;
    int cus = 0, xcds = 1;
    int rc = device_cus(&cus, &xcds);
    return rc != TSGEMM_OK ? rc : cus;
}

int tsgemm_launch_info(const tsgemm_plan* p, int32_t* num_workgroups, int32_t* max_iters, int32_t* num_xcds) {
    reset_error();
    if (!p) return fail(TSGEMM_EINVAL, "plan is NULL");
    // the device is consulted only for what the plan leaves to it: the
    // default worker count, and the XCD count when asked for
    int cus = 0, xcds = 1;
    if (p->P == 0 || (num_xcds && p->xcd_remap)) {
        int rc = device_cus(&cus, &xcds);
        if (rc != TSGEMM_OK) return rc;
    }
    const uint32_t P = (uint32_t)(p->P ? p->P : cus);
    if (P % (uint32_t)p->cluster != 0)
        return fail(TSGEMM_EINVAL, "the %u workgroups do not split into clusters of %d", P, p->cluster);
    if (num_workgroups) *num_workgroups = (int32_t)P;
    if (max_iters) *max_iters = (int32_t)max_iters_for(p, P);
    if (num_xcds) *num_xcds = p->xcd_remap ? (int32_t)xcds : 1;
    return TSGEMM_OK;
}

int tsgemm_plan_info(const tsgemm_plan* p, tsgemm_info* info) {
    reset_error();
    if (!p || !info) return fail(TSGEMM_EINVAL, "plan or info is NULL");
    std::memset(info, 0, sizeof(*info));
    info->M = p->M; info->N = p->N; info->K = p->K;
    info->dtype = p->dtype;
    info->block_M = p->bm; info->block_N = p->bn; info->block_K = p->bk;
    info->group_size = p->group;
    info->num_stages = p->stages;
    info->lds_slots = p->slots;
    info->stage_bytes = stage_bytes_of(p->dtype, p->bm, p->bn, p->bk);
    info->lds_bytes = info->stage_bytes * p->slots + (p->epi ? p->bm * p->epi * 2 : 0);
    info->m_blocks = p->m_blocks; info->n_blocks = p->n_blocks;
    info->k_blocks = p->k_blocks; info->num_tiles = p->tiles;
    info->num_workgroups = p->P;  // explicit P only; default resolves at run time
    info->waves = p->P && p->P % p->cluster == 0 ? (int32_t)max_iters_for(p, (uint32_t)p->P) : 0;
    info->threads_per_workgroup = p->kernel ? 64 * p->kernel->waves : tsg::MxTraits::THREADS;
    info->xcd_remap = p->xcd_remap;
    info->cluster_size = p->cluster;
    info->column_major = p->col_major;
    info->store_block_N = p->epi;
    info->l2_prefetch = p->prefetch;
    return TSGEMM_OK;
}

int tsgemm_schedule_host(const tsgemm_plan* p, int num_workgroups, int32_t* out) {
    reset_error();
    if (!p || !out) return fail(TSGEMM_EINVAL, "plan or out is NULL");
    if (num_workgroups <= 0) return fail(TSGEMM_EINVAL, "num_workgroups must be > 0");
    if (num_workgroups % p->cluster != 0)
        return fail(TSGEMM_EINVAL, "the %d workgroups do not split into clusters of %d", num_workgroups, p->cluster);
    tsg::TileScheduler s;
    s.setup((uint32_t)num_workgroups, (uint32_t)p->m_blocks, (uint32_t)p->n_blocks, (uint32_t)p->group,
            (uint32_t)p->cluster, (uint32_t)p->col_major);
    int64_t row = 0;
    for (uint32_t wid = 0; wid < (uint32_t)num_workgroups; ++wid)
        for (s.init(wid); s.valid(); s.next_tile(), ++row) {
            out[4 * row + 0] = (int32_t)wid;
            out[4 * row + 1] = (int32_t)s.iter;
            out[4 * row + 2] = (int32_t)s.m_idx;
            out[4 * row + 3] = (int32_t)s.n_idx;
        }
    if (row != p->tiles) return fail(TSGEMM_EINVAL, "schedule covered %lld of %lld tiles", (long long)row, (long long)p->tiles);
    return TSGEMM_OK;
}

int tsgemm_worker_numbering(int32_t num_workgroups, int32_t num_xcds, int32_t num_active, int32_t* out) {
    reset_error();
    if (!out) return fail(TSGEMM_EINVAL, "out is NULL");
    if (num_workgroups <= 0 || num_xcds <= 0 || num_active <= 0 || num_active > num_workgroups)
        return fail(TSGEMM_EINVAL, "need num_workgroups > 0, num_xcds > 0 and 0 < num_active <= num_workgroups");
    for (int32_t b = 0; b < num_workgroups; ++b)
        out[b] = (int32_t)tsg::worker_of_workgroup((uint32_t)b, (uint32_t)num_workgroups, (uint32_t)num_xcds,
                                                   (uint32_t)num_active);
    return TSGEMM_OK;
}

int tsgemm_dump_schedule(const tsgemm_plan* p, int32_t* out) {
    reset_error();
    if (!p || !out) return fail(TSGEMM_EINVAL, "plan or out is NULL");
    if (p->tiles == 0) return TSGEMM_OK;
    Grid g;
    int rc = resolve_grid(p, &g);
    if (rc != TSGEMM_OK) return rc;
    const size_t n = (size_t)g.P * g.max_iters * 4;
    int32_t* d = nullptr;
    hipError_t e = hipMalloc(&d, n * sizeof(int32_t));
    if (e != hipSuccess) return fail(TSGEMM_ENOMEM, "hipMalloc: %s", hipGetErrorString(e));
    std::vector<int32_t> h(n);
    e = hipMemset(d, 0xFF, n * sizeof(int32_t));
    if (e == hipSuccess) {
        hipLaunchKernelGGL(tsg::tsgemm_schedule_kernel, dim3(g.P), dim3(64), 0, 0, g.P, (uint32_t)p->m_blocks,
                           (uint32_t)p->n_blocks, (uint32_t)p->group, (uint32_t)p->cluster,
                           (uint32_t)p->col_major, g.xcds, g.active, g.max_iters, d);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpy(h.data(), d, n * sizeof(int32_t), hipMemcpyDeviceToHost);
    hipError_t e2 = hipFree(d);
    if (e != hipSuccess) return fail(TSGEMM_EHIP, "schedule kernel: %s", hipGetErrorString(e));
    if (e2 != hipSuccess) return fail(TSGEMM_EHIP, "hipFree: %s", hipGetErrorString(e2));
    // rows are stored at [worker][iter]: reading them in that order sorts them
    int64_t row = 0;
    for (size_t i = 0; i < n; i += 4) {
        if (h[i] < 0) continue;
        if (row >= p->tiles) return fail(TSGEMM_EINVAL, "device schedule visited more than %lld tiles", (long long)p->tiles);
        std::memcpy(out + 4 * row, &h[i], 4 * sizeof(int32_t));
        ++row;
    }
    if (row != p->tiles) return fail(TSGEMM_EINVAL, "device schedule visited %lld of %lld tiles", (long long)row, (long long)p->tiles);
    return TSGEMM_OK;
}

void tsgemm_destroy(tsgemm_plan* p) { delete p; }

}  // extern "C"
