// ffn_decode_q41.hip -- decode expert-FFN kernels instantiated for Q4_1 blocks.
#include "ffn_decode.h"

namespace moe {

hipError_t decode_ffn_q41(const DecodeArgs &a, hipStream_t st) {
  hipError_t e = gateup_q<MOE_Q4_1>(a, st);
  if (e != hipSuccess) return e;
  e = down_q<MOE_Q4_1>(a, st);
  return e;
}

}  // namespace moe
