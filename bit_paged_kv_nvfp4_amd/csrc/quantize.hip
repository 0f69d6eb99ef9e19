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

__global__ __launch_bounds__(256) void k_quantize(QuantizeArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_token = (int64_t)a.num_kv_heads * 16;
  if (idx >= a.num_tokens * per_token) return;
  const int64_t t = idx / per_token;
  const int rem = (int)(idx - t * per_token);
  qenc::quantize_one(a, t, rem >> 4, (rem >> 3) & 1, rem & 7);
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

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t stream) {
  const int64_t threads = a.num_tokens * a.num_kv_heads * 16;
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (a.fp8)
    hipLaunchKernelGGL(k_quantize_fp8, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
