// The fp16/bf16 kernels of one dtype and tile shape, chosen by the build
// with -DTSG_TU_DT=<1 fp16 | 2 bf16> -DTSG_TU_BM=<128 | 256> -DTSG_TU_BK=<32 | 64>
// (square tiles, BN = BM): every ring depth that fits in LDS, 4 and 8
// wavefronts, direct and chunked epilogue.
#include "tsgemm_launch.h"
#include "tsgemm_kernel.h"

#if !defined(TSG_TU_DT) || !defined(TSG_TU_BM) || !defined(TSG_TU_BK)
#error "build with -DTSG_TU_DT, -DTSG_TU_BM and -DTSG_TU_BK"
#endif

namespace tsg {
namespace {

template <int DT, int BM, int BN, int BK, int L, int WGN, int EPI>
void launch_gemm(const GemmArgs& a, unsigned grid, hipStream_t s) {
    if constexpr (pair_kernel(BM, BN, BK, WGN, EPI)) {
        if (a.k_blocks >= 2u) {  // the paired kernel runs tiles of two slabs or more
            hipLaunchKernelGGL((tsgemm_kernel<DT, BM, BN, BK, L, WGN, EPI, true>), dim3(grid), dim3(64 * 2 * WGN), 0, s, a);
            return;
        }
    }
    hipLaunchKernelGGL((tsgemm_kernel<DT, BM, BN, BK, L, WGN, EPI>), dim3(grid), dim3(64 * 2 * WGN), 0, s, a);
}

constexpr int DT = TSG_TU_DT, BM = TSG_TU_BM, BK = TSG_TU_BK;

#define TSG_ENTRY(S, WGN, EPI) \
    {DT, BM, BM, BK, S, 2 * WGN, EPI, launch_gemm<DT, BM, BM, BK, fit_slots(BM, BM, BK, S, EPI), WGN, EPI>}
#define TSG_SLOTS(WGN, EPI) TSG_ENTRY(2, WGN, EPI), TSG_ENTRY(3, WGN, EPI), TSG_ENTRY(4, WGN, EPI), TSG_ENTRY(5, WGN, EPI)

const KernelEntry kEntries[] = {TSG_SLOTS(2, 0), TSG_SLOTS(4, 0), TSG_SLOTS(2, 64)};

}  // namespace

#define TSG_DEFINE_GEMM_TU(D, M_, K_)                                   \
    const KernelEntry* TSG_GEMM_TU_FN(D, M_, K_)(int* count) {          \
        *count = (int)(sizeof(kEntries) / sizeof(kEntries[0]));         \
        return kEntries;                                                \
    }
TSG_DEFINE_GEMM_TU(TSG_TU_DT, TSG_TU_BM, TSG_TU_BK)

}  // namespace tsg
