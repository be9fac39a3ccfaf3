// probe.hip -- measurement probes of the chip the MoE step runs on (gfx950):
// the streaming-read rate the decode kernels are bounded by, the cost of a
// kernel boundary, and the cost of a cross-XCD exchange inside one kernel.
// Diagnostics only: no part of the MoE step uses them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_q4.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Streaming read: every thread reads 16-byte pieces i, i + stride, ... of the
// buffer (4 pieces in flight per iteration) and folds them into one word,
// which is stored only if it equals a value no fold produces here (the
// stores never happen, the loads cannot be dropped).
__global__ __launch_bounds__(256) void k_probe_stream(const u32x4 *__restrict__ buf, size_t n16,
                                                      uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u && sink) sink[threadIdx.x] = acc;
}

__global__ void k_probe_empty() {}

// All-to-all exchange, `rounds` times: in round r every block stores the
// 64-bit word (r + 1) << 32 | its index to its own slot with a device-scope
// store, then every block reads all slots (device-scope loads) until each
// holds round r + 1.  A value and its round travel in one 64-bit word, so a
// reader needs no fence: it sees the old word or the new one.  The wait is
// bounded: after `spin_limit` reads of a slot without progress the block
// sets status[0] = 1 and leaves the loop, so every wave ends.  Thread 0 of
// block 0 records the 100 MHz real-time counter at the start and end in
// cycles[0..1].  A slot only grows, so a block that runs ahead never hides a
// round from one that lags.
__global__ __launch_bounds__(256) void k_probe_exchange(unsigned long long *__restrict__ slots, int rounds,
                                                        uint32_t spin_limit, uint32_t *__restrict__ status,
                                                        unsigned long long *__restrict__ cycles) {
  const int G = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
  __shared__ int failed;
  if (tid == 0) failed = 0;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int r = 0; r < rounds; r++) {
    const unsigned long long want = (unsigned long long)(r + 1) << 32;
    if (tid == 0) __hip_atomic_store(&slots[b], want | (unsigned)b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int s = tid; s < G; s += blockDim.x) {
      uint32_t n = 0;
      while ((__hip_atomic_load(&slots[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32) < (unsigned)(r + 1)) {
        if (++n >= spin_limit) {
          failed = 1;
          break;
        }
      }
    }
    __syncthreads();
    if (failed) break;
  }
  if (failed && tid == 0) __hip_atomic_store(&status[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (b == 0 && tid == 0) {
    cycles[0] = t0;
    cycles[1] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace

extern "C" {

int moe_probe_stream(const void *buf, size_t bytes, int32_t blocks, uint32_t *sink, moe_stream_t stream) {
  if (!buf || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || blocks < 1) return MOE_EINVAL;
  hipLaunchKernelGGL(k_probe_stream, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)buf,
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

int moe_probe_empty(int32_t blocks, moe_stream_t stream) {
  if (blocks < 1) return MOE_EINVAL;
  hipLaunchKernelGGL(k_probe_empty, dim3(blocks), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

int moe_probe_exchange(int32_t blocks, int32_t rounds, uint32_t spin_limit, void *slots, uint32_t *status,
                       unsigned long long *cycles, moe_stream_t stream) {
  if (blocks < 1 || blocks > 4096 || rounds < 1 || spin_limit < 1 || !slots || !status || !cycles)
    return MOE_EINVAL;
  unsigned long long *s = (unsigned long long *)slots;
  void *args[] = {&s, &rounds, &spin_limit, &status, &cycles};
  // a cooperative launch: every block is resident at once, or the launch fails
  const hipError_t e = hipLaunchCooperativeKernel((const void *)k_probe_exchange, dim3(blocks), dim3(256), args, 0,
                                                  (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : MOE_ELAUNCH;
}

}  // extern "C"
