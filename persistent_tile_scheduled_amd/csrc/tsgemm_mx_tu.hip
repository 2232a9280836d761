// The block-scaled FP8 (MX) kernels: the GEMM (row-major or packed scales)
// and the scale-packing permutation.
#include <mutex>

#include "tsgemm_launch.h"
#include "tsgemm_mx_kernel.h"

namespace tsg {

// Packed-scale workspace of tsgemm_run_mx_noalloc (see kMxScratchBytes).  In
// host code `scratch` names a host-side stand-in, never the device memory:
// every host use goes through the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) uint8_t scratch[kMxScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device ordinal
}  // namespace

hipError_t mx_scratch_address(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Scale packing for the PACKED kernel: SF[rows][K/32] (row-major E8M0) ->
// SFP[block][group][256][SC_ROW], block = 256-row block, group = SG consecutive
// 128-deep slabs (SC_ROW = 4 * SG bytes of one row).  Rows past `rows` and
// bytes past K/32 are written as 0.  One thread per output dword.
__global__ void tsgemm_mx_pack_kernel(const uint8_t* SF, uint8_t* SFP, int64_t rows, uint32_t kb_bytes,
                                      uint32_t blocks, uint32_t n_groups) {
    constexpr uint32_t DW = MxTraits::SC_ROW / 4;  // dwords per row and group
    const uint64_t total = (uint64_t)blocks * n_groups * MxTraits::BM * DW;
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const uint32_t d = (uint32_t)(t % DW);
    const uint64_t rg = t / DW;                    // ((block * n_groups + group) * 256 + r)
    const uint32_t r = (uint32_t)(rg % MxTraits::BM);
    const uint64_t bg = rg / MxTraits::BM;
    const uint32_t g = (uint32_t)(bg % n_groups), blk = (uint32_t)(bg / n_groups);
    const int64_t row = (int64_t)blk * MxTraits::BM + r;
    const uint32_t col = g * (uint32_t)MxTraits::SC_ROW + d * 4u;   // byte within the row, multiple of 4
    uint32_t v = 0;
    if (row < rows && col < kb_bytes) v = *(const uint32_t*)(SF + row * kb_bytes + col);  // kb_bytes % 4 == 0
    *(uint32_t*)(SFP + t * 4) = v;
}

void launch_mx(const MxArgs& a, unsigned grid, bool packed, hipStream_t s) {
    if (packed)
        hipLaunchKernelGGL(tsgemm_mx_kernel<true>, dim3(grid), dim3(MxTraits::THREADS), 0, s, a);
    else
        hipLaunchKernelGGL(tsgemm_mx_kernel<false>, dim3(grid), dim3(MxTraits::THREADS), 0, s, a);
}

void launch_mx_pack(const uint8_t* SF, uint8_t* SFP, int64_t rows, uint32_t kb_bytes, uint32_t blocks,
                    uint32_t n_groups, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL(tsgemm_mx_pack_kernel, dim3(grid), dim3(256), 0, s, SF, SFP, rows, kb_bytes, blocks, n_groups);
}

}  // namespace tsg
