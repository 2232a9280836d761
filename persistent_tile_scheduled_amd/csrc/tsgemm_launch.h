// Host-side launch interface between the C ABI (tsgemm.hip) and the
// translation units that compile the kernels (tsgemm_gemm_tu.hip, once per
// dtype and tile shape; tsgemm_mx_tu.hip), so the kernels build in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsgemm_device.h"

namespace tsg {

struct MxArgs;

constexpr int kLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup

// Ring slots that a launch with `s` requested slots and a chunked-epilogue
// buffer of `epi` columns gets: `s` when they fit in LDS, else 2 (such
// entries are compiled but never selected: the plan caps the slot count).
constexpr int fit_slots(int bm, int bn, int bk, int s, int epi) {
    return ((bm * bk + bk * bn) * 2 * s + bm * epi * 2) <= kLdsBytes ? s : 2;
}

typedef void (*launch_fn)(const GemmArgs&, unsigned grid, hipStream_t);

// One compiled fp16/bf16 kernel: dtype, tile, ring slots, wavefronts, epilogue.
struct KernelEntry {
    int dt, bm, bn, bk, slots, waves, epi;
    launch_fn fn;
};

// The entries one translation unit compiles (its dtype and tile shape).
#define TSG_GEMM_TU_FN(DT, BM, BK) gemm_kernels_##DT##_##BM##_##BK
#define TSG_DECLARE_GEMM_TU(DT, BM, BK) const KernelEntry* TSG_GEMM_TU_FN(DT, BM, BK)(int* count);
TSG_DECLARE_GEMM_TU(1, 128, 32)
TSG_DECLARE_GEMM_TU(1, 128, 64)
TSG_DECLARE_GEMM_TU(1, 256, 32)
TSG_DECLARE_GEMM_TU(1, 256, 64)
TSG_DECLARE_GEMM_TU(2, 128, 32)
TSG_DECLARE_GEMM_TU(2, 128, 64)
TSG_DECLARE_GEMM_TU(2, 256, 32)
TSG_DECLARE_GEMM_TU(2, 256, 64)

// Block-scaled FP8 kernels (tsgemm_mx_tu.hip).
// Workspace of the allocation-free MX entry point: packed SFA then packed SFB
// in one static device array of this many bytes (per device, held until the
// process ends).
constexpr int64_t kMxScratchBytes = int64_t(16) << 20;
// Device address of that array on the current device (looked up once per
// device); hipSuccess or the lookup's error.
hipError_t mx_scratch_address(void** ptr);
void launch_mx(const MxArgs& a, unsigned grid, bool packed, hipStream_t s);
void launch_mx_pack(const uint8_t* SF, uint8_t* SFP, int64_t rows, uint32_t kb_bytes, uint32_t blocks,
                    uint32_t n_groups, unsigned grid, hipStream_t s);

}  // namespace tsg
