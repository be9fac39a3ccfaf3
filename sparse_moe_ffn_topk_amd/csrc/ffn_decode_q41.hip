// ffn_decode_q41.hip -- decode expert-FFN kernels instantiated for Q4_1 blocks.
#include "ffn_decode.h"

namespace moe {

hipError_t decode_ffn_q41(const DecodeArgs &a, hipStream_t st) {
  timer_before(3, st);
  hipError_t e = gateup_q<MOE_Q4_1>(a, st);
  timer_after(3, st);
  if (e != hipSuccess) return e;
  timer_before(4, st);
  e = down_q<MOE_Q4_1>(a, st);
  timer_after(4, st);
  return e;
}

}  // namespace moe
