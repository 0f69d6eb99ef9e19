// Encode and write of one 16-value block (token, KV head, K|V, block) into the
// page pool, NVFP4 and the FP8 baseline, shared by the quantize-on-write
// kernels, the extend kernel's fused chunk write and the decode kernel's fused
// write of each sequence's newest token (gfx950).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): prefill
// quantizes the prompt's keys and values into the NVFP4 cache; each block of 16
// values keeps 8 bytes of packed codes and 1 byte of scale. Page "NVFP4-KV-Cache
// auf der NVIDIA RTX PRO 6000 Blackwell Server Edition" (section "Bytes pro
// Token"): E2M1 values, one E4M3 scale per 16 values, one FP32 scale per tensor.
//
// Every rounding decision is the one on the exact real quotients amax/(6g) and
// x/(E4M3(s) g), "nearest, ties to even": for a power-of-two g through a
// correctly rounded fp32 quotient (proven to take the same decisions), or exact
// comparisons against threshold products; for any other g through comparisons
// in fp64, where every threshold (a few-bit constant times an E4M3 value times
// the 24-bit g, at most 31 significant bits) is exact.
#pragma once

#include "nvfp4kv_device.h"

namespace nvfp4kv {
namespace qenc {

// E4M3 value of a non-negative finite byte k (0..126), exact in fp32 (and fp64).
template <typename T = float>
__device__ inline __attribute__((always_inline)) T e4m3_value(int k) {
  return k < 8 ? (T)k * (T)0x1p-9 : __builtin_ldexp((T)(8 + (k & 7)), (k >> 3) - 10);
}

// Byte of the E4M3 value nearest to amax / six_g (six_g = 6 g), ties to the even
// byte, clamped to 448 (0x7E). Binary search for the first midpoint between
// consecutive E4M3 values that amax does not pass; a tie passes the midpoint
// only when its lower neighbour is odd. T = float is exact for a power-of-two g,
// T = double for any g.
template <typename T>
__device__ inline __attribute__((always_inline)) int scale_byte(T amax, T six_g) {
  int lo = 0, hi = 126;
#pragma unroll
  for (int it = 0; it < 7; ++it) {
    if (lo < hi) {
      const int k = (lo + hi) >> 1;
      const T thr = ((T)0.5 * (e4m3_value<T>(k) + e4m3_value<T>(k + 1))) * six_g;
      const bool pass = amax > thr || (amax == thr && (k & 1));
      lo = pass ? k + 1 : lo;
      hi = pass ? hi : k;
    }
  }
  return lo;
}

// E2M1 code of x for block divisor D = E4M3(s) g: count of the magnitude
// midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (times D) that |x| passes, where
// a tie passes only midpoints whose lower code is odd; sign bit from x.
template <typename T>
__device__ inline __attribute__((always_inline)) uint32_t e2m1_code(float x, T D, bool zero_scale) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const T ax = (T)__builtin_fabsf(x);
  uint32_t c = (uint32_t)(ax > (T)0.25 * D) + (uint32_t)(ax >= (T)0.75 * D) + (uint32_t)(ax > (T)1.25 * D) +
               (uint32_t)(ax >= (T)1.75 * D) + (uint32_t)(ax > (T)2.5 * D) + (uint32_t)(ax >= (T)3.5 * D) +
               (uint32_t)(ax > (T)5.0 * D);
  c = zero_scale ? 0u : c;
  return sign | c;
}

// The threshold path: scale byte by binary search over exact midpoint products,
// codes by seven exact threshold compares per value. amax ignores NaN elements
// (fmax drops them), which then pass no threshold and get magnitude 0.
template <typename T>
__device__ inline __attribute__((always_inline)) void encode_thresholds(const float (&x)[16], float g,
                                                                        uint32_t (&w)[2], int& s) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  s = scale_byte<T>((T)amax, (T)6 * (T)g);
  const T D = e4m3_value<T>(s) * (T)g;
  const bool zs = (s == 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v |= e2m1_code<T>(x[8 * h + i], D, zs) << (4 * i);
    w[h] = v;
  }
}

// The raw bytes of block j of token t, head h, kind (0 K, 1 V): four 16-byte
// pieces (f32) or two (bf16, u[2] and u[3] unused), converted by unpack_block.
// Split from the conversion so that a kernel can issue the loads early and wait
// for them later.
template <bool kBf16>
__device__ inline __attribute__((always_inline)) void load_raw_block(const QuantizeArgs& a, int64_t t, int h,
                                                                     int kind, int j, uint4 (&u)[4]) {
  const int64_t off = t * a.token_stride + (int64_t)h * a.head_stride + j * 16;
  if (kBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(kind ? a.v : a.k) + off);
    u[0] = p[0];
    u[1] = p[1];
    u[2] = u[3] = make_uint4(0, 0, 0, 0);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(kind ? a.v : a.k) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = p[i];
  }
}

template <bool kBf16>
__device__ inline __attribute__((always_inline)) void unpack_block(const uint4 (&u)[4], float (&x)[16]) {
  if (kBf16) {
    const uint32_t w[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[4 * i] = __uint_as_float(u[i].x);
      x[4 * i + 1] = __uint_as_float(u[i].y);
      x[4 * i + 2] = __uint_as_float(u[i].z);
      x[4 * i + 3] = __uint_as_float(u[i].w);
    }
  }
}

// The 16 values of block j of token t, head h, kind (0 K, 1 V) as f32.
__device__ inline __attribute__((always_inline)) void load_block(const QuantizeArgs& a, int64_t t, int h, int kind,
                                                                 int j, float (&x)[16]) {
  const int64_t off = t * a.token_stride + (int64_t)h * a.head_stride + j * 16;
  if (a.bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(kind ? a.v : a.k) + off);
    const uint4 u0 = p[0], u1 = p[1];
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(kind ? a.v : a.k) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = p[i];
      x[4 * i] = f.x;
      x[4 * i + 1] = f.y;
      x[4 * i + 2] = f.z;
      x[4 * i + 3] = f.w;
    }
  }
}

// x / D from r = 1/D correctly rounded: the product x r, its exact remainder
// x - (x r) D (one fma), and one correction step. The result is the correctly
// rounded quotient whenever D carries at most 4 significant bits (every E4M3
// value, and 6, times a power of two), so its nearest-even E2M1 or E4M3
// decision is the decision on the exact real quotient; a CPU test checks this
// for every binary32 x in the binades that can change a code. Written as
// -fma(-rem, r, -q0) so that a zero quotient keeps the sign of x.
__device__ inline __attribute__((always_inline)) float quotient(float x, float D, float r) {
#pragma clang fp contract(off)
  const float q0 = x * r;
  const float rem = __builtin_fmaf(-q0, D, x);
  return -__builtin_fmaf(-rem, r, -q0);
}

// Codes (packed: value i in nibble i % 8 of word i / 8, i.e. the K byte order)
// and scale byte of the 16 values x, for global scale g.
//
// With a power-of-two g, blocks whose values are all finite, whose scale is not
// saturated and not zero take the fast path: the scale byte is the nearest-even
// E4M3 of the quotient amax / (6 g), and every code the nearest-even E2M1 of
// x / D, D = E4M3(s) g, rounded by the hardware f32 -> fp4 conversion (scale
// operand 1.0), which saturates at 6 and keeps the sign. Other blocks (NaN or
// infinite values, amax / (6 g) above 448, a zero scale) take the threshold
// path in fp32, whose products are exact for such g. Any other g takes the
// threshold path in fp64 (kPow2 = false: a separate instantiation, so that the
// kernels of the power-of-two case keep their registers).
template <bool kPow2>
__device__ inline __attribute__((always_inline)) void encode_values(const float (&x)[16], float g, uint32_t (&w)[2],
                                                                    int& s) {
  if (!kPow2) {
    encode_thresholds<double>(x, g, w, s);
    return;
  }
  float ap = __builtin_fabsf(x[0]);  // NaN-propagating max of |x|
#pragma unroll
  for (int i = 1; i < 16; ++i) ap = __builtin_elementwise_maximum(ap, __builtin_fabsf(x[i]));
  const float six_g = 6.0f * g;
  bool fast = ap <= 2688.0f * g;  // 6 * 448 g: false for NaN and infinities
  if (fast) {
    s = (int)f32_to_e4m3(quotient(ap, six_g, 1.0f / six_g));
    fast = s != 0;
  }
  if (fast) {
    const float D = e4m3_to_f32((uint32_t)s) * g;
    const float r = 1.0f / D;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* y = x + 8 * h;
      uint32_t v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, quotient(y[0], D, r), quotient(y[1], D, r), 1.0f, 0);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, quotient(y[2], D, r), quotient(y[3], D, r), 1.0f, 1);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, quotient(y[4], D, r), quotient(y[5], D, r), 1.0f, 2);
      w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, quotient(y[6], D, r), quotient(y[7], D, r), 1.0f, 3);
    }
  } else {
    encode_thresholds<float>(x, g, w, s);
  }
}

// Code of value q (0..15) of a block from its packed words.
__device__ inline __attribute__((always_inline)) uint32_t nibble(const uint32_t (&w)[2], int q) {
  return (w[q >> 3] >> (4 * (q & 7))) & 15u;
}

// Codes and scale byte of block j of token t, head h, kind (0 K, 1 V); kPow2
// must equal a.g_pow2.
template <bool kPow2>
__device__ inline __attribute__((always_inline)) void encode_block(const QuantizeArgs& a, int64_t t, int h, int kind,
                                                                   int j, uint32_t (&w)[2], int& s) {
  float x[16];
  load_block(a, t, h, kind, j, x);
  encode_values<kPow2>(x, a.g, w, s);
}

// Encode block j of token t, KV head h, kind (0 K, 1 V) and write its codes and
// scale to `slot` (>= 0). With `grouped`, a V block whose four-row group is
// written by this call as four consecutive tokens of a.slots (of a.num_tokens)
// is left to the thread of the group's first token, which writes whole words;
// otherwise the block's nibbles are set with atomics.
template <bool kPow2>
__device__ inline __attribute__((always_inline)) void write_block(const QuantizeArgs& a, int64_t t, int64_t slot,
                                                                  int h, int kind, int j, bool grouped) {
  const int64_t page = slot >> 4;
  const int row = (int)(slot & 15);
  uint8_t* slab = a.pool + ((page * a.num_kv_heads + h) * 2 + kind) * (int64_t)kSlab;

  if (kind == 1 && grouped) {
    // V: a code byte holds rows r and r ^ 2 and a 32-bit word rows 4g .. 4g+3 of
    // one page. When this call writes those four rows as four consecutive tokens,
    // the thread of the first one encodes all four and writes whole words.
    const int r4 = row & 3;
    const int64_t tl = t - r4;
    bool full = tl >= 0 && tl + 3 < a.num_tokens;
    const int32_t s0 = full ? a.slots[tl] : -1;
    full = full && s0 >= 0 && (s0 & 3) == 0;
#pragma unroll
    for (int i = 1; i < 4; ++i) full = full && a.slots[tl + i] == s0 + i;
    if (full) {
      if (r4 != 0) return;  // written by the group's first token
      uint32_t c4[4][2];
      int s4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) encode_block<kPow2>(a, t + i, h, 1, j, c4[i], s4[i]);
      // chunk (row/4)*16 + 2j + c holds channels 16j + 8c .. +7; its word wi holds
      // channel q = 8c + 2wi (bytes 0, 1) and q + 1 (bytes 2, 3), rows 0|2 in the
      // even byte and rows 1|3 in the odd one
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          const int q = 8 * c + 2 * wi;
          w[wi] = (nibble(c4[0], q) | (nibble(c4[2], q) << 4)) | ((nibble(c4[1], q) | (nibble(c4[3], q) << 4)) << 8) |
                  ((nibble(c4[0], q + 1) | (nibble(c4[2], q + 1) << 4)) << 16) |
                  ((nibble(c4[1], q + 1) | (nibble(c4[3], q + 1) << 4)) << 24);
        }
        *reinterpret_cast<uint4*>(slab + ((row >> 2) * 16 + 2 * j + c) * 16) = make_uint4(w[0], w[1], w[2], w[3]);
      }
      *reinterpret_cast<uint32_t*>(slab + kCodeBytes + j * 16 + row) =
          (uint32_t)s4[0] | ((uint32_t)s4[1] << 8) | ((uint32_t)s4[2] << 16) | ((uint32_t)s4[3] << 24);
      return;
    }
  }

  uint32_t code[2];
  int s;
  encode_block<kPow2>(a, t, h, kind, j, code, s);
  if (kind == 0) {
    // K: the token's 8 code bytes of block j are contiguous, channel 2i in the low
    // nibble of byte i
    *reinterpret_cast<uint2*>(slab + row * 64 + j * 8) = make_uint2(code[0], code[1]);
    slab[kCodeBytes + row * 8 + j] = (uint8_t)s;
  } else {
    // V, a token alone in its four-row group: channel 16j + e sits in 16-byte
    // chunk (row/4)*16 + 2j + e/8, byte 2*(e%8) + row%2, high nibble for rows with
    // row%4 >= 2; the other nibble of each byte is row r ^ 2 of the same page,
    // which another thread (or another call) may be writing, so the block's
    // nibbles are cleared and set with 32-bit atomics that leave every other bit
    // alone.
    const int sh = 8 * (row & 1) + 4 * ((row >> 1) & 1);
    const uint32_t mask = (0xFu << sh) | (0xFu << (sh + 16));
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t* chunk = reinterpret_cast<uint32_t*>(slab + ((row >> 2) * 16 + 2 * j + c) * 16);
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        const uint32_t val = (nibble(code, 8 * c + 2 * wi) << sh) | (nibble(code, 8 * c + 2 * wi + 1) << (sh + 16));
        __hip_atomic_fetch_and(chunk + wi, ~mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(chunk + wi, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    slab[kCodeBytes + j * 16 + row] = (uint8_t)s;
  }
}

// Block j of token t (of a.num_tokens), KV head h, kind into slot a.slots[t]
// (negative: skipped).
template <bool kPow2>
__device__ inline __attribute__((always_inline)) void quantize_one(const QuantizeArgs& a, int64_t t, int h,
                                                                   int kind, int j) {
  const int32_t slot = a.slots[t];
  if (slot < 0) return;
  write_block<kPow2>(a, t, slot, h, kind, j, true);
}

// FP8 baseline pool: block j of token t, head h, kind into `slot` (>= 0), the
// E4M3 code of x / s for each value (nearest, ties to even, satfinite; s a
// power of two, so x / s is exact in fp32). K: the block's 16 bytes are
// contiguous in the token's row (one 16-byte store). V: value (row r, channel d)
// sits at byte ((r/4)*16 + d/8)*32 + (d%8)*4 + r%4 of the slab, so the block's
// bytes are scattered; every byte belongs to one value, so plain byte stores
// never touch a neighbour's.
constexpr int kFp8Slab = 2048;

__device__ inline __attribute__((always_inline)) void write_block_fp8(const QuantizeArgs& a, int64_t t, int64_t slot,
                                                                      int h, int kind, int j) {
  const int64_t page = slot >> 4;
  const int row = (int)(slot & 15);
  uint8_t* slab = a.pool + ((page * a.num_kv_heads + h) * 2 + kind) * (int64_t)kFp8Slab;
  float x[16];
  load_block(a, t, h, kind, j, x);
  const float inv = kind ? a.inv_v_scale : a.inv_k_scale;
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = f32_to_e4m3(x[i] * inv);
  if (kind == 0) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = c[4 * i] | (c[4 * i + 1] << 8) | (c[4 * i + 2] << 16) | (c[4 * i + 3] << 24);
    *reinterpret_cast<uint4*>(slab + row * 128 + j * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 16 * j + i;
      slab[((row >> 2) * 16 + (d >> 3)) * 32 + (d & 7) * 4 + (row & 3)] = (uint8_t)c[i];
    }
  }
}

}  // namespace qenc
}  // namespace nvfp4kv
