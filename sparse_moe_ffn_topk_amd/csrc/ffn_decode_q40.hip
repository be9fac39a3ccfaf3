// ffn_decode_q40.hip -- decode expert-FFN kernels instantiated for Q4_0 blocks.
#include "ffn_decode.h"

namespace moe {

hipError_t decode_ffn_q40(const DecodeArgs &a0, hipStream_t st) {
  DecodeArgs a = a0;
  hipError_t e = prelude_q<MOE_Q4_0>(a, st);
  if (e != hipSuccess) return e;
  e = gateup_q<MOE_Q4_0>(a, st);
  if (e != hipSuccess) return e;
  e = down_q<MOE_Q4_0>(a, st);
  return e;
}

}  // namespace moe
