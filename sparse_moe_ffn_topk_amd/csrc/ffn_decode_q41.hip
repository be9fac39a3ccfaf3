// ffn_decode_q41.hip -- decode expert-FFN kernels instantiated for Q4_1 blocks.
#include "ffn_decode.h"

namespace moe {

hipError_t decode_ffn_q41(const DecodeArgs &a0, hipStream_t st) {
  DecodeArgs a = a0;
  hipError_t e = prelude_q<MOE_Q4_1>(a, st);
  if (e != hipSuccess) return e;
  e = gateup_q<MOE_Q4_1>(a, st);
  if (e != hipSuccess) return e;
  e = down_q<MOE_Q4_1>(a, st);
  return e;
}

}  // namespace moe
