// decode.hip -- instantiation of the weight-streaming kernel (decode_kernel.h)
// used by llmint8_matmul for T <= 16 and by llmint8_igemm_i32.
#include "decode_kernel.h"

namespace llmint8 {

// Each wavefront streams 16 weight rows, 512 bytes of each per stage, with
// three register buffers (two stages in flight); four wavefronts per block.
// With two or more activation rows the fragments come from the packed layout
// (one contiguous KB per k-step instead of up to 16 row pieces) and the
// block's wavefronts keep in step so that they share each fragment in L1.
using DecodeRows = decode::CfgRs<512, 4, 3, false>;
using DecodePacked = decode::CfgRs<512, 4, 3, true>;

hipError_t launch_decode(const int8_t *Xq, const int8_t *CB, int64_t T, int64_t K, int64_t N,
                         const EpilogueArgs &ep, bool xq_packed, hipStream_t s, hipEvent_t ev0,
                         hipEvent_t ev1)
{
    if (xq_packed)
        return decode::launch_rs<DecodePacked>(Xq, CB, T, K, N, ep, s, ev0, ev1);
    return decode::launch_rs<DecodeRows>(Xq, CB, T, K, N, ep, s, ev0, ev1);
}

}  // namespace llmint8
