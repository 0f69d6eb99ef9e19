// Internal declarations shared by the HIP sources of libnvfp4kv (not part of the
// public C ABI, see include/nvfp4kv.h for the contract and the pool layout).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kSlab = 1152;     // bytes of one (page, head, K|V) slab
constexpr int kCodeBytes = 1024;
constexpr int kMaxGroup = 16;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Reductions over the four 16-lane rows of a wave64: lane l combines its value
// with lane l ^ 16 (permlane16 swap) or l ^ 32 (permlane32 swap).
__device__ __forceinline__ float xor16_max(float v) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One asynchronous 16-byte-per-lane copy global -> LDS (gfx950 global_load_lds
// dwordx4): lane i reads base + voff and writes LDS address lds + 16 i. It is
// issued from inline assembly so that the compiler, which cannot tell which LDS
// bytes such a copy writes, does not drain all outstanding copies before every
// LDS read; completion is awaited explicitly with wait_dma().
// A wave-uniform copy of a pointer, held in SGPRs (readfirstlane is free when the
// value already is scalar); the copy instructions take their base from SGPRs.
template <typename T>
__device__ __forceinline__ const T* sgpr_ptr(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sgpr_ptr(base)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// The same copy for data read exactly once (the decode kernel's pages): marked
// non-temporal, so that the streamed lines do not displace reusable ones in the
// L2 and the last-level cache. Measured at batch 44 x 32K: the decode kernel
// 301 -> 271 us.
__device__ __forceinline__ void dma16_stream(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sgpr_ptr(base)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Same with 4 bytes per lane (lane i writes LDS address lds + 4 i).
__device__ __forceinline__ void dma4(const int32_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(sgpr_ptr(base)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_dma() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// E4M3 ("fn") code of x: nearest value, ties to the even code, magnitudes above
// 448 saturate to 448, sign kept (also of zero). x must be finite. Written out
// from the format: normal codes 8..126 hold (1 + m/8) 2^(e-7), codes 0..7 hold
// m 2^-9; rounding the binary32 significand to 3 bits with a carry into the
// exponent covers every normal case, and below 2^-6 the value is rounded to a
// multiple of 2^-9 (which reaches code 8 = 2^-6 exactly when it rounds up).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(x);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0x1p-6f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // exact product, nearest-even integer 0..8
  } else {
    const uint32_t bits = u & 0x7FFFFFFFu;
    const uint32_t e = (bits >> 23) - 127u + 7u;  // 1..15 here
    const uint32_t m = bits & 0x7FFFFFu;
    const uint32_t r = m >> 20, rem = m & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ? 1u : 0u;
    code = (e << 3) + r + up;  // a carry out of the mantissa moves to the next exponent
  }
  return sign | code;
}

struct QuantizeArgs {
  const void* k;
  const void* v;
  int32_t bf16;            // 1: sources are bfloat16, 0: float32
  int64_t token_stride;    // elements
  int64_t head_stride;     // elements
  const int32_t* slots;
  int64_t num_tokens;
  uint8_t* pool;
  int32_t num_kv_heads;
  float g;
  int32_t g_pow2;          // 1: g is a power of two (the fast encode applies)
  int32_t fp8;             // 1: the pool is the FP8 baseline
  float inv_k_scale;       // FP8 baseline: 1 / k_scale, 1 / v_scale (powers of two)
  float inv_v_scale;
};

struct AmaxArgs {
  const void* k;
  const void* v;
  int32_t bf16;            // 1: sources are bfloat16, 0: float32
  int64_t token_stride;    // elements
  int64_t head_stride;     // elements
  int64_t num_tokens;
  int32_t num_kv_heads;
  float* partial;          // [kAmaxBlocks][2] workspace
  float* out;              // [2]: max |K|, max |V|
};
constexpr int kAmaxBlocks = 256;

struct DecodeArgs {
  const uint16_t* q;       // bf16 bits [B][Hq][128]
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;           // Hq / Hkv
  int32_t max_seq_len;
  const uint8_t* pool;
  float qk_scale_log2;     // sm_scale * log2(e) * g
  float v_scale;           // g (the partial states carry V in true units)
  int32_t num_splits;
  int32_t num_workgroups;  // persistent workgroups of the decode kernel
  int32_t fp8;             // 1: the pool is the FP8 baseline (K/V scales folded into
                           // qk_scale_log2 and v_scale)
  float* part_o;           // [B][Hq][S][128]
  float* part_ml;          // [B][Hq][S][2]: running max (log2 units), sum
  int32_t write_new;       // 1: the launch first writes token seq_lens[b] - 1 of
                           // every sequence b from nw (token index b) into the pool
  QuantizeArgs nw;         // its sources, pool and scales (nw.slots unused)
  void* out;
  int32_t out_bf16;
  float* lse;
};

struct DequantArgs {
  const uint8_t* pool;
  int32_t num_kv_heads;
  float g;
  int32_t g_pow2;     // 1: g is a power of two (every dequantized value is exact in fp32)
  const int32_t* page_table;
  int64_t pt_stride;
  const int32_t* seq_lens;
  const int64_t* row_offsets;
  int32_t n_seqs;
  int32_t max_seq_len;
  void* k_out;
  void* v_out;
  int32_t out_dtype;  // NVFP4KV_F32, NVFP4KV_BF16 or NVFP4KV_FP8_E4M3
};

struct ExtendArgs {
  const uint16_t* q;       // bf16 bits [C][Hq][128]
  const void* k_pre;       // prefix workspace [P][Hkv][128], bf16 or FP8 E4M3
  const void* v_pre;       // the same, or f16 V^T tiles [ceil(P/64)][Hkv][128][64] (pre_kind 2)
  int32_t pre_kind;        // 0: bf16 rows, 1: FP8 E4M3 rows, 2: bf16 K rows + f16 V^T tiles
  int64_t prefix_len;      // P
  const uint16_t* k_chunk; // bf16 bits [C][Hkv][128]
  const uint16_t* v_chunk;
  int64_t chunk_len;       // C
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;           // Hq / Hkv
  float qk_scale_log2;     // |sm_scale| * log2(e)
  uint32_t q_sign;         // 0x80008000 when sm_scale < 0 (flips the sign of Q), else 0
  float v_mul;             // power of two applied to V before its f16 conversion
  float out_mul;           // 1 / v_mul, applied to the output
  uint16_t* out;           // bf16 bits [C][Hq][128]
  float* lse;              // [C][Hq] natural log, or null
  int32_t tokens_per_block;
  int32_t num_token_blocks;
  int32_t write_chunk;     // 1: also quantize-write the chunk's K/V into an NVFP4 pool
  QuantizeArgs qw;         // that write (chunk K/V, its slots, the pool)
};

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream);
hipError_t launch_amax(const AmaxArgs& a, hipStream_t stream);
// Waves of one decode workgroup, per page format.
int decode_waves_per_split(bool fp8);
// Workgroups of the decode kernel that fit on the device at once, per page format.
int decode_resident_workgroups(int num_cus, bool fp8);
hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream);
// The newest token of every sequence (a.nw, a.page_table, a.seq_lens) into the
// pool, for a global scale that is not a power of two.
hipError_t launch_write_newest(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);
// Chunk tokens per workgroup of the extend kernel for a GQA group size.
int extend_tokens_per_block(int group);
hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream);

// ---- device helpers --------------------------------------------------------

// Decode of an E4M3 (OCP fn) byte held in bits 0..7 of `b` to float (exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8(b, 0);
}

// f16 bit pattern of E4M3(b) / 256 for a non-negative finite byte b (0..0x7E):
// the byte's exponent and mantissa fields land in the f16 fields unchanged, which
// re-biases the exponent by 8 (normal bytes) and maps subnormal bytes onto f16
// subnormals with the same factor. Exact for every byte 0..0x7E.
__device__ __forceinline__ uint32_t e4m3_f16bits_div256(uint32_t b) { return b << 7; }

__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// Two E2M1 codes (byte `sel` of w: low nibble first) to two f16 values, unscaled.
template <int SEL>
__device__ __forceinline__ f16x2 fp4x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace nvfp4kv
