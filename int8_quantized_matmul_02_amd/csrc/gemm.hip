// gemm.hip -- instantiation of the tiled int8 MFMA GEMM (gemm_kernel.h) used
// by llmint8_matmul for T > 16 and by llmint8_igemm_i32.
#include "gemm_kernel.h"

namespace llmint8 {

// 256 x 256 block tile, 2 x 2 wavefronts of 128 x 128, 4-stage LDS ring
// (4 x 32 KB), groups of 4 tile rows.
using GemmMain = gemm::Cfg<256, 256, 2, 2, 4, 4>;

hipError_t launch_gemm(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                       const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1)
{
    return gemm::launch<GemmMain>(Xq, CB, T, K, N, ep, s, ev0, ev1);
}

}  // namespace llmint8
