// gemm.hip -- instantiations of the tiled int8 MFMA GEMM (gemm_kernel.h) used
// by llmint8_matmul for T > 16 and by llmint8_igemm_i32.
#include "gemm_kernel.h"

namespace llmint8 {

// 256 x 256 block tile, 2 x 2 wavefronts of 128 x 128, groups of 4 tile
// rows.  With K a multiple of 128 the ring holds two stages of 128 bytes per
// row (every load instruction then fetches whole 128-byte lines), otherwise
// four stages of 64 bytes; 128 KB of LDS either way.  The fp16 pass over
// more than 32 outlier columns (rows padded to 128 bytes) runs through the
// same ring.
//
// Up to K = 6144 the int8 output kernel runs with 2 x 4 wavefronts of
// 128 x 64 instead (two per SIMD, so one issues MFMAs while the other waits
// at a barrier or on LDS; 50 % more fragment reads per MFMA).  Measured on
// MI355X: 242 -> 236 us at 4096 x 4096 x 16384 and 41.8 -> 40.3 us at
// 2048 x 2048 x 8192, but 471 -> 488 us at K = 12288, where the longer main
// loop gains less from the second wavefront than the extra LDS traffic
// costs.  The zero-point and FP8 epilogues spill in that shape and keep four
// wavefronts.
//
// The many-outlier kernel runs with 2 x 4 wavefronts at every K that is a
// multiple of 128, in every variant: its fp16 pass dequantizes the weight
// codes with VALU work between the MFMAs, which the second wavefront per
// SIMD overlaps.  Measured on MI355X: 1284 -> 1191 us at 4096 x 12288 x
// 12288 with threshold 0, 789 -> 735 us at a 4096 x 16384 x 4096 fc2-like
// input (83 % of the columns outliers), 678 -> 651 us with 128 outlier
// columns at 4096 x 12288 x 12288.
using Gemm128 = gemm::Cfg<256, 256, 2, 2, 2, 4, 128>;
using Gemm128W8 = gemm::Cfg<256, 256, 2, 4, 2, 4, 128>;
using Gemm64 = gemm::Cfg<256, 256, 2, 2, 4, 4, 64>;
constexpr int64_t kW8MaxK = 6144;

hipError_t launch_gemm(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                       const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1)
{
    if (K % Gemm128::ROWB == 0 && K <= kW8MaxK && !ep.row_zp && !ep.f8)
        return gemm::launch<Gemm128W8, Gemm128W8>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    if (K % Gemm128::ROWB == 0)
        return gemm::launch<Gemm128, Gemm128W8>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    return gemm::launch<Gemm64>(Xq, CB, T, K, N, ep, s, ev0, ev1);
}

}  // namespace llmint8
