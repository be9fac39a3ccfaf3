// ffn_decode.hip -- dispatch of the decode expert FFNs by block type.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

hipError_t decode_ffn_q41(const DecodeArgs &a, hipStream_t st);
hipError_t decode_ffn_q40(const DecodeArgs &a, hipStream_t st);
hipError_t decode_ffn_q80(const DecodeArgs &a, hipStream_t st);

size_t decode_down_lds_bytes(int k, int F, int SF) {
  // act blocks of 32 floats at a 36-float stride, plus one sum per block
  return (size_t)(k * (F / 32) + SF / 32) * (36 + 1) * sizeof(float);
}

hipError_t launch_decode_ffn(const DecodeArgs &a, hipStream_t st) {
  return a.qtype == MOE_Q4_1 ? decode_ffn_q41(a, st) : (a.qtype == MOE_Q8_0 ? decode_ffn_q80(a, st) : decode_ffn_q40(a, st));
}

}  // namespace moe
