// moe_common.h -- device helpers shared by the gfx950 kernels of the MoE step.
//
// Q4 blocks (GGUF): Q4_1 = f16 d, f16 m, 16 nibble bytes (20 B, value d*q+m);
// Q4_0 = f16 d, 16 nibble bytes (18 B, value d*(q-8)).  Nibble byte i holds
// element i in its low half and element i+16 in its high half (block layout of
// the diskformer flint_moe_ssd.js page, file header and Q41DOT comment).
//
// Q8_0 = f16 d, 32 signed bytes (34 B, value d*q, element i = byte i; the
// lfm2_moe_ssd.js page's int8 expert plane).
//
// A block's dot with 32 inputs is d*sum(q x) + m*sum(x) (the same page's
// q41dot identity); Q4_0 is the case m = -8d.  Q8_0 takes the same form with
// q' = q + 128 (each byte XOR 0x80, then converted as unsigned) and
// m = -128d.  The per-block input sum is computed once per input vector and
// kept in LDS beside the inputs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_Q4_0 0
#define MOE_Q4_1 1
#define MOE_Q8_0 2

// Dword 3 of a raw buffer resource on gfx9-family parts (gfx950 included):
// 32-bit data format, no swizzle, no stride; out-of-range loads return 0.
#define MOE_RSRC_WORD3 0x00020000

namespace moe {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  // Sizes are rounded up to whole dwords: a dword holding the last byte of an
  // allocation never crosses a page, and Q4_0 loads read 4-byte-aligned words.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)((bytes + 3u) & ~3u),
                                           MOE_RSRC_WORD3);
}

template <int QT> struct QBlock;

// Five dwords of a block as loaded: w[0] carries the f16 scale (and offset),
// the nibble words are extracted by nib().
struct Raw5 {
  uint32_t w[5];
};

template <> struct QBlock<MOE_Q4_1> {
  typedef Raw5 Raw;
  static constexpr int bytes = 20;
  // Block at byte offset `off` (4-byte aligned: rows of 20-byte blocks).
  static __device__ __forceinline__ Raw5 load(rsrc_t r, uint32_t off) {
    Raw5 b;
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    b.w[0] = v.x; b.w[1] = v.y; b.w[2] = v.z; b.w[3] = v.w;
    b.w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(off + 16), 0, 0);
    return b;
  }
  static __device__ __forceinline__ void scales(const Raw5 &b, uint32_t, float &d, float &m) {
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)(b.w[0] & 0xffffu));
    m = (float)__builtin_bit_cast(_Float16, (uint16_t)(b.w[0] >> 16));
  }
  static __device__ __forceinline__ uint32_t nib(const Raw5 &b, uint32_t, int k) { return b.w[1 + k]; }
};

template <> struct QBlock<MOE_Q4_0> {
  typedef Raw5 Raw;
  static constexpr int bytes = 18;
  // Block at byte offset `off` (2-byte aligned): five dwords from the dword
  // boundary at or below it, realigned in registers.
  static __device__ __forceinline__ Raw5 load(rsrc_t r, uint32_t off) {
    uint32_t a = off & ~3u;
    Raw5 b;
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)a, 0, 0);
    b.w[0] = v.x; b.w[1] = v.y; b.w[2] = v.z; b.w[3] = v.w;
    b.w[4] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(a + 16), 0, 0);
    return b;
  }
  static __device__ __forceinline__ void scales(const Raw5 &b, uint32_t off, float &d, float &m) {
    uint16_t db = (off & 2u) ? (uint16_t)(b.w[0] >> 16) : (uint16_t)(b.w[0] & 0xffffu);
    d = (float)__builtin_bit_cast(_Float16, db);
    m = -8.0f * d;
  }
  // Nibble word k = block bytes 2+4k .. 5+4k.
  static __device__ __forceinline__ uint32_t nib(const Raw5 &b, uint32_t off, int k) {
    return (off & 2u) ? b.w[1 + k] : __builtin_amdgcn_alignbyte(b.w[1 + k], b.w[k], 2);
  }
};

// Nine dwords from the dword boundary at or below a Q8_0 block (34 bytes,
// 2-byte aligned).
struct Raw9 {
  uint32_t w[9];
};
template <> struct QBlock<MOE_Q8_0> {
  typedef Raw9 Raw;
  static constexpr int bytes = 34;
  static __device__ __forceinline__ Raw9 load(rsrc_t r, uint32_t off) {
    const uint32_t a = off & ~3u;
    Raw9 b;
    const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(r, (int)a, 0, 0);
    const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(a + 16), 0, 0);
    b.w[0] = v0.x; b.w[1] = v0.y; b.w[2] = v0.z; b.w[3] = v0.w;
    b.w[4] = v1.x; b.w[5] = v1.y; b.w[6] = v1.z; b.w[7] = v1.w;
    b.w[8] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(a + 32), 0, 0);
    return b;
  }
  static __device__ __forceinline__ void scales(const Raw9 &b, uint32_t off, float &d, float &m) {
    const uint16_t db = (off & 2u) ? (uint16_t)(b.w[0] >> 16) : (uint16_t)(b.w[0] & 0xffffu);
    d = (float)__builtin_bit_cast(_Float16, db);
    m = -128.0f * d;
  }
  // Byte word k = block bytes 2+4k .. 5+4k (elements 4k .. 4k+3), as q + 128.
  static __device__ __forceinline__ uint32_t word(const Raw9 &b, uint32_t off, int k) {
    const uint32_t w = (off & 2u) ? b.w[1 + k] : __builtin_amdgcn_alignbyte(b.w[1 + k], b.w[k], 2);
    return w ^ 0x80808080u;
  }
};

// 8 nibbles of 8 bytes (the low halves, or the high halves with sh = 4) as
// exact f16 q in the natural order of the bytes: each nibble is moved into a
// byte of its own, read as an OCP E4M3 byte -- whose value is q 2^-9 for every
// q in 0..15 (subnormal below 8, exponent 1 from 8) -- and scaled by 2^9 by
// the conversion (two values per instruction).
__device__ __forceinline__ half8 nibbles_e4m3(u32x2 nb, uint32_t sh) {
  const uint32_t a = (nb.x >> sh) & 0x0F0F0F0Fu, b = (nb.y >> sh) & 0x0F0F0F0Fu;
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 512.0f, false);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 512.0f, true);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 512.0f, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 512.0f, true);
  const u32x4 v = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
                   __builtin_bit_cast(uint32_t, p3)};
  return __builtin_bit_cast(half8, v);
}

// sum over one nibble word's 8 elements of q*x: low nibbles pair with
// x[4k..4k+3], high nibbles with x[16+4k..16+4k+3].  Each nibble is moved into
// a byte of its own and the bytes are read as OCP E4M3 values -- q 2^-9 for
// every q in 0..15 -- and scaled by 2^9 by the conversion, two per instruction,
// as exact f16 q; each product q*x is then one mixed f16 x f32 fma (exact
// product, one rounding, as an f32 fma of the converted value).
__device__ __forceinline__ void nib_word_dot(uint32_t w, const float4 &xl, const float4 &xh, float &lo,
                                             float &hi) {
  const uint32_t l = w & 0x0F0F0F0Fu, h = (w >> 4) & 0x0F0F0F0Fu;
  const auto l01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(l, 512.0f, false);
  const auto l23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(l, 512.0f, true);
  const auto h01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h, 512.0f, false);
  const auto h23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(h, 512.0f, true);
  lo = __builtin_fmaf((float)l01[0], xl.x, lo);
  lo = __builtin_fmaf((float)l01[1], xl.y, lo);
  lo = __builtin_fmaf((float)l23[0], xl.z, lo);
  lo = __builtin_fmaf((float)l23[1], xl.w, lo);
  hi = __builtin_fmaf((float)h01[0], xh.x, hi);
  hi = __builtin_fmaf((float)h01[1], xh.y, hi);
  hi = __builtin_fmaf((float)h23[0], xh.z, hi);
  hi = __builtin_fmaf((float)h23[1], xh.w, hi);
}

// Q4 block dot with its 32 inputs xb (LDS) and their sum sx.
template <int QT>
__device__ __forceinline__ float block_dot_q4(const Raw5 &b, uint32_t off, const float *xb, float sx) {
  float d, m;
  QBlock<QT>::scales(b, off, d, m);
  float lo = 0.f, hi = 0.f;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    float4 xl = *reinterpret_cast<const float4 *>(xb + 4 * k);
    float4 xh = *reinterpret_cast<const float4 *>(xb + 16 + 4 * k);
    nib_word_dot(QBlock<QT>::nib(b, off, k), xl, xh, lo, hi);
  }
  float q = lo + hi;
  return __builtin_fmaf(d, q, m * sx);
}

// Dot of one loaded block with its 32 inputs xb (LDS) and their sum sx.
template <int QT>
__device__ __forceinline__ float block_dot(const typename QBlock<QT>::Raw &b, uint32_t off, const float *xb,
                                           float sx) {
  if constexpr (QT == MOE_Q8_0) {
    float d, m;
    QBlock<QT>::scales(b, off, d, m);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
      uint32_t w = QBlock<QT>::word(b, off, k);
      asm("" : "+v"(w));  // one v_cvt_f32_ubyteN per byte (see nib_word_dot)
      const float4 xv = *reinterpret_cast<const float4 *>(xb + 4 * k);
      float &acc = (k & 1) ? a1 : a0;
      acc = __builtin_fmaf((float)(w & 0xff), xv.x, acc);
      acc = __builtin_fmaf((float)((w >> 8) & 0xff), xv.y, acc);
      acc = __builtin_fmaf((float)((w >> 16) & 0xff), xv.z, acc);
      acc = __builtin_fmaf((float)(w >> 24), xv.w, acc);
    }
    return __builtin_fmaf(d, a0 + a1, m * sx);
  } else {
    return block_dot_q4<QT>(b, off, xb, sx);
  }
}

// A block's 32 quants as floats (Q4: q, in element order; Q8_0: q + 128) and
// its scale and offset, so that value_i = d * q[i] + m.  For dots of one block
// with several inputs: the conversion is done once.
template <int QT>
__device__ __forceinline__ void block_unpack(const typename QBlock<QT>::Raw &b, uint32_t off, float (&q)[32],
                                             float &d, float &m) {
  QBlock<QT>::scales(b, off, d, m);
  if constexpr (QT == MOE_Q8_0) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      uint32_t w = QBlock<QT>::word(b, off, k);
      asm("" : "+v"(w));  // one v_cvt_f32_ubyteN per byte (see nib_word_dot)
      q[4 * k] = (float)(w & 0xff);
      q[4 * k + 1] = (float)((w >> 8) & 0xff);
      q[4 * k + 2] = (float)((w >> 16) & 0xff);
      q[4 * k + 3] = (float)(w >> 24);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t w = QBlock<QT>::nib(b, off, k);
      uint32_t l = w & 0x0F0F0F0Fu, h = (w >> 4) & 0x0F0F0F0Fu;
      asm("" : "+v"(l));
      asm("" : "+v"(h));
      q[4 * k] = (float)(l & 0xff);
      q[4 * k + 1] = (float)((l >> 8) & 0xff);
      q[4 * k + 2] = (float)((l >> 16) & 0xff);
      q[4 * k + 3] = (float)(l >> 24);
      q[16 + 4 * k] = (float)(h & 0xff);
      q[16 + 4 * k + 1] = (float)((h >> 8) & 0xff);
      q[16 + 4 * k + 2] = (float)((h >> 16) & 0xff);
      q[16 + 4 * k + 3] = (float)(h >> 24);
    }
  }
}

// d * sum_i q[i] x[i] + m * sx for an unpacked block and its 32 inputs xb (LDS).
__device__ __forceinline__ float unpacked_dot(const float (&q)[32], float d, float m, const float *xb, float sx) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const float4 xv = *reinterpret_cast<const float4 *>(xb + 4 * k);
    float &acc = (k & 1) ? a1 : a0;
    acc = __builtin_fmaf(q[4 * k], xv.x, acc);
    acc = __builtin_fmaf(q[4 * k + 1], xv.y, acc);
    acc = __builtin_fmaf(q[4 * k + 2], xv.z, acc);
    acc = __builtin_fmaf(q[4 * k + 3], xv.w, acc);
  }
  return __builtin_fmaf(d, a0 + a1, m * sx);
}

// LDS layout of an input vector: block b's 32 floats at b*XSTRIDE (36 floats:
// a 16-byte pad per block spreads a lane group's 128-bit reads over the banks).
constexpr int XSTRIDE = 36;

// DPP lane moves (gfx9 encodings): row_shr:n moves each lane's value n lanes
// up within its row of 16; with bound_ctrl the first n lanes read 0.
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, true);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ double readlane_d(double v, int lane) {
  const long long b = __builtin_bit_cast(long long, v);
  const int lo = __builtin_amdgcn_readlane((int)b, lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (long long)(unsigned)lo);
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 32):
// the LAST lane of each group (lane % W == W-1) receives the group total.
// For W = 32 the odd rows then add lane 15 of the row below (DPP row_bcast:15,
// rows 1 and 3 written).
template <int W>
__device__ __forceinline__ float group_sum_last(float v) {
  if constexpr (W >= 2) v += dpp_f<DPP_ROW_SHR1>(v);
  if constexpr (W >= 4) v += dpp_f<DPP_ROW_SHR2>(v);
  if constexpr (W >= 8) v += dpp_f<DPP_ROW_SHR4>(v);
  if constexpr (W >= 16) v += dpp_f<DPP_ROW_SHR8>(v);
  if constexpr (W >= 32)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  return v;
}

// Sum of a double over the whole wave (row sums, then the four rows in a
// fixed order); the result is uniform.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<DPP_ROW_SHR1>(v);
  v += dpp_d<DPP_ROW_SHR2>(v);
  v += dpp_d<DPP_ROW_SHR4>(v);
  v += dpp_d<DPP_ROW_SHR8>(v);
  return (readlane_d(v, 15) + readlane_d(v, 31)) + (readlane_d(v, 47) + readlane_d(v, 63));
}

}  // namespace moe
