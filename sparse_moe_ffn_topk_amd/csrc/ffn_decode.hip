// ffn_decode.hip -- dispatch of the decode expert FFNs by block type.
#include "moe_common.h"
#include "moe_launch.h"
#include "select_block.h"

namespace moe {

hipError_t decode_ffn_q41(const DecodeArgs &a, hipStream_t st);
hipError_t decode_ffn_q40(const DecodeArgs &a, hipStream_t st);
hipError_t decode_ffn_q80(const DecodeArgs &a, hipStream_t st);

size_t decode_down_lds_bytes(int k, int F, int SF) {
  // act blocks of 32 floats at a 36-float stride, plus one sum per block
  return (size_t)(k * (F / 32) + SF / 32) * (36 + 1) * sizeof(float);
}

int prelude_token_group(int T, int H) {
  if (T < 2 || H > 64 * 2 * 32) return 0;  // two blocks per lane of a 64-lane row
  static int limit[64];                    // max LDS per block, per device (0: not read yet)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (limit[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
    limit[dev] = v;
  }
  const long avail = (long)limit[dev] - (long)sizeof(SelShared);
  const long per = (long)(H / 32) * (XSTRIDE + 1) * (long)sizeof(float);
  // at most 4 tokens per group: a group's inputs then take about a third of a
  // CU's LDS at H = 2048, so two or three groups' blocks share a CU (more waves
  // to hide latency), at the cost of one more pass over the shared weights
  // (from the cache) per extra group
  const int want = T <= 2 ? 2 : 4;
  for (int tg = want; tg >= 2; tg >>= 1)
    if (tg * per <= avail) return tg;
  return 0;
}

hipError_t launch_decode_ffn(const DecodeArgs &a, hipStream_t st) {
  return a.qtype == MOE_Q4_1 ? decode_ffn_q41(a, st) : (a.qtype == MOE_Q8_0 ? decode_ffn_q80(a, st) : decode_ffn_q40(a, st));
}

}  // namespace moe
