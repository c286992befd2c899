// decode.hip -- instantiation of the weight-streaming kernel (decode_kernel.h)
// used by llmint8_matmul for T <= 16 and by llmint8_igemm_i32.
#include "decode_kernel.h"

namespace llmint8 {

// Each wavefront streams 16 weight rows, 1 KB of each per stage, through two
// LDS stages; four wavefronts per block.
using DecodeMain = decode::CfgLds<2, 1024, 4>;

hipError_t launch_decode(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                         const EpilogueArgs &ep, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1)
{
    return decode::launch_lds<DecodeMain>(Xq, CB, T, K, N, ep, s, ev0, ev1);
}

}  // namespace llmint8
