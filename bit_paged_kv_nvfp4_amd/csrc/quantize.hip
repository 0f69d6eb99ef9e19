// Quantize-on-write of K/V rows into the NVFP4 page pool (gfx950).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): initial
// prefill quantizes the prompt's keys and values into the NVFP4 cache; each block
// of 16 values keeps 8 bytes of packed codes and 1 byte of scale. Page
// "NVFP4-KV-Cache auf der NVIDIA RTX PRO 6000 Blackwell Server Edition" (section
// "Bytes pro Token"): E2M1 values, one E4M3 scale per 16 values, one FP32 scale
// per tensor.
//
// One thread encodes one 16-value block (token, KV head, K|V, block); the encode
// and write rules are in quantize_block.h.
#include "nvfp4kv_device.h"
#include "quantize_block.h"

namespace nvfp4kv {
namespace {

// One workgroup per (16 consecutive tokens, KV head, K|V); thread (row, block)
// = (threadIdx / 8, threadIdx % 8) encodes block j of token t0 + row. When the
// 16 tokens fill one page in order (slots s0 .. s0 + 15, s0 a multiple of 16),
// the workgroup owns that page's K or V slab of this head and writes it whole:
// K codes and all scales with plain stores, V code words after the four rows of
// each word have traded codes across lanes. Otherwise each thread writes its
// block alone, as the shared block writer does. (K and V in one 256-thread
// workgroup measured 2-3% slower.)
// kPow2: the pool's global scale is a power of two (the fast encode); any other
// g takes the fp64 threshold encode in its own instantiation. kBf16: the source
// dtype (a.bf16).
template <bool kPow2, bool kBf16>
__global__ __launch_bounds__(128) void k_quantize(QuantizeArgs a) {
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kPage;
  const int kind = blockIdx.z;
  const int row = (threadIdx.x >> 3) & 15;
  const int j = threadIdx.x & 7;
  const int64_t t = t0 + row;
  const bool live = t < a.num_tokens;
  // The row's values are requested before the slots and the workgroup vote, so
  // that the two memory round trips overlap instead of following each other.
  uint4 raw[4];  // rows past the end load the last token (their values are not used)
  qenc::load_raw_block<kBf16>(a, live ? t : a.num_tokens - 1, h, kind, j, raw);
  const int32_t slot = live ? a.slots[t] : -1;
  const int32_t s0 = a.slots[t0];
  const bool whole = __syncthreads_and(live && s0 >= 0 && (s0 & (kPage - 1)) == 0 && slot == s0 + row);
  if (!whole) {
    if (slot >= 0) qenc::write_block<kPow2>(a, t, slot, h, kind, j, true);
    return;
  }
  uint8_t* slab = a.pool + (((int64_t)(s0 / kPage) * a.num_kv_heads + h) * 2 + kind) * (int64_t)kSlab;
  float x[16];
  qenc::unpack_block<kBf16>(raw, x);
  uint32_t w[2];
  int s;
  qenc::encode_values<kPow2>(x, a.g, w, s);
  if (kind == 0) {
    // K: row r holds its 64 code bytes at 64 r (block j at 8 j), scales at 1024 + 8 r + j
    *reinterpret_cast<uint2*>(slab + row * 64 + j * 8) = make_uint2(w[0], w[1]);
    slab[kCodeBytes + row * 8 + j] = (uint8_t)s;
    return;
  }
  // V: the 32 code bytes of block j for rows 4G .. 4G+3 sit in 16-byte chunks
  // 16 G + 2 j + c (c = 0, 1: channels 8c .. 8c+7 of the block); word wi of a
  // chunk holds channels q = 8c + 2 wi and q + 1, each as a byte of rows 0|2 (low
  // nibble row 0) and a byte of rows 1|3. The lane of row 4G + r4 writes the 8
  // bytes of words 2 (r4 & 1), +1 of chunk c = r4 >> 1, i.e. channels 4 r4 .. 4 r4 + 3
  // of the four rows: 16-bit field r4 of each row's packed codes.
  const int r4 = row & 3;
  const int lane = threadIdx.x & 63;  // = (row % 8) * 8 + j
  uint32_t f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int src = lane + 8 * (i - r4);
    const uint32_t lo = (uint32_t)__shfl((int)w[0], src, 64);
    const uint32_t hi = (uint32_t)__shfl((int)w[1], src, 64);
    f[i] = ((r4 >> 1) ? hi : lo) >> (16 * (r4 & 1));
  }
  uint32_t out[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t b[4];  // channels 4 r4 + 2k (low nibble) and + 1 (high nibble) of row i
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (f[i] >> (8 * k)) & 0xFFu;
    out[k] = (b[0] & 15u) | ((b[2] & 15u) << 4) | ((b[1] & 15u) << 8) | ((b[3] & 15u) << 12) |
             ((b[0] >> 4) << 16) | ((b[2] >> 4) << 20) | ((b[1] >> 4) << 24) | ((b[3] >> 4) << 28);
  }
  *reinterpret_cast<uint2*>(slab + ((row >> 2) * 16 + 2 * j + (r4 >> 1)) * 16 + 8 * (r4 & 1)) =
      make_uint2(out[0], out[1]);
  slab[kCodeBytes + j * 16 + row] = (uint8_t)s;
}

// The newest token (position L - 1, L = seq_lens[b]) of every sequence b, token
// b of nw, written into the pool as the decode kernel's fused write does it
// (one workgroup per (sequence, KV head), one thread per 16-value block, V
// nibbles by atomics). The fused decode step runs this first when the global
// scale is not a power of two, so that the decode kernel itself compiles only
// the power-of-two encode.
__global__ __launch_bounds__(64) void k_write_newest(DecodeArgs a) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int j = threadIdx.x;
  const int L = a.seq_lens[b];
  if (L < 1 || j >= 16) return;
  const int64_t slot = (int64_t)a.page_table[(int64_t)b * a.pt_stride + (L - 1) / kPage] * kPage + (L - 1) % kPage;
  qenc::write_block<false>(a.nw, b, slot, h, j >> 3, j & 7, false);
}

// FP8 baseline quantize-on-write: one thread per (token, KV head, K|V, 16-value
// block); the encode and byte layout are in quantize_block.h.
__global__ __launch_bounds__(256) void k_quantize_fp8(QuantizeArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_token = (int64_t)a.num_kv_heads * 16;
  if (idx >= a.num_tokens * per_token) return;
  const int64_t t = idx / per_token;
  const int rem = (int)(idx - t * per_token);
  const int32_t slot = a.slots[t];
  if (slot < 0) return;
  qenc::write_block_fp8(a, t, slot, rem >> 4, (rem >> 3) & 1, rem & 7);
}

// ---- per-tensor amax (global-scale calibration) -----------------------------
// Two launches and no atomics: up to kAmaxBlocks workgroups each reduce a
// grid-stride share of the 16-byte pieces of K and of V into a partial pair in
// the caller's workspace, and one workgroup reduces the partials. fmax drops
// NaN operands, so NaN elements are ignored.
__device__ __forceinline__ float amax16(const void* base, int64_t off, bool bf16) {
  float m = 0.0f;
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w[i] << 16)),
                                             __builtin_fabsf(__uint_as_float(w[i] & 0xFFFF0000u))));
  } else {
    const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(f.x), __builtin_fabsf(f.y)),
                        __builtin_fmaxf(__builtin_fabsf(f.z), __builtin_fabsf(f.w)));
  }
  return m;
}

// Workgroup max of (mk, mv); the result is valid in thread 0.
__device__ __forceinline__ void block_max2(float& mk, float& mv) {
  __shared__ float red[2][4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mk = __builtin_fmaxf(mk, __shfl_xor(mk, o));
    mv = __builtin_fmaxf(mv, __shfl_xor(mv, o));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = mk;
    red[1][w] = mv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    mk = __builtin_fmaxf(__builtin_fmaxf(red[0][0], red[0][1]), __builtin_fmaxf(red[0][2], red[0][3]));
    mv = __builtin_fmaxf(__builtin_fmaxf(red[1][0], red[1][1]), __builtin_fmaxf(red[1][2], red[1][3]));
  }
}

__global__ __launch_bounds__(256) void k_amax_partial(AmaxArgs a) {
  const int per_row = a.bf16 ? 16 : 32;  // 16-byte pieces per (token, head) row of 128 values
  const int vec = a.bf16 ? 8 : 4;
  const int64_t pieces = a.num_tokens * a.num_kv_heads * per_row;
  float mk = 0.0f, mv = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / per_row;
    const int64_t t = row / a.num_kv_heads;
    const int h = (int)(row - t * a.num_kv_heads);
    const int64_t off = t * a.token_stride + (int64_t)h * a.head_stride + (i - row * per_row) * vec;
    mk = __builtin_fmaxf(mk, amax16(a.k, off, a.bf16));
    mv = __builtin_fmaxf(mv, amax16(a.v, off, a.bf16));
  }
  block_max2(mk, mv);
  if (threadIdx.x == 0) {
    a.partial[2 * blockIdx.x] = mk;
    a.partial[2 * blockIdx.x + 1] = mv;
  }
}

__global__ __launch_bounds__(256) void k_amax_final(const float* partial, int n, float* out) {
  float mk = 0.0f, mv = 0.0f;
  for (int i = threadIdx.x; i < n; i += 256) {
    mk = __builtin_fmaxf(mk, partial[2 * i]);
    mv = __builtin_fmaxf(mv, partial[2 * i + 1]);
  }
  block_max2(mk, mv);
  if (threadIdx.x == 0) {
    out[0] = mk;
    out[1] = mv;
  }
}

}  // namespace

hipError_t launch_amax(const AmaxArgs& a, hipStream_t stream) {
  const int64_t pieces = a.num_tokens * a.num_kv_heads * (a.bf16 ? 16 : 32);
  const int64_t want = (pieces + 255) / 256;
  const int blocks = (int)(want < kAmaxBlocks ? want : kAmaxBlocks);
  if (blocks > 0) {
    hipLaunchKernelGGL(k_amax_partial, dim3(blocks), dim3(256), 0, stream, a);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(k_amax_final, dim3(1), dim3(256), 0, stream, a.partial, blocks, a.out);
  return hipGetLastError();
}

hipError_t launch_write_newest(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(k_write_newest, dim3((unsigned)a.batch, (unsigned)a.num_kv_heads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream) {
  const int64_t threads = a.num_tokens * a.num_kv_heads * 16;
  if (threads == 0) return hipSuccess;
  if (a.fp8) {
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(k_quantize_fp8, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  } else {
    const int64_t groups = (a.num_tokens + kPage - 1) / kPage;
    const dim3 grid((unsigned)groups, (unsigned)a.num_kv_heads, 2);
    if (a.g_pow2 && a.bf16)
      hipLaunchKernelGGL((k_quantize<true, true>), grid, dim3(128), 0, stream, a);
    else if (a.g_pow2)
      hipLaunchKernelGGL((k_quantize<true, false>), grid, dim3(128), 0, stream, a);
    else if (a.bf16)
      hipLaunchKernelGGL((k_quantize<false, true>), grid, dim3(128), 0, stream, a);
    else
      hipLaunchKernelGGL((k_quantize<false, false>), grid, dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace nvfp4kv
