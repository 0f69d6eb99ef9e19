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
#include <type_traits>

#include "nvfp4kv_device.h"
#include "quantize_block.h"

namespace nvfp4kv {
namespace {

// Max over the kLB lanes of a 16-value block (aligned groups of 2 or 4
// consecutive lanes), NaN-propagating (kNan) or NaN-ignoring, by DPP quad
// permutes.
template <int kLB, bool kNan>
__device__ __forceinline__ float block_lanes_max(float v) {
  auto mx = [](float x, float y) { return kNan ? __builtin_elementwise_maximum(x, y) : __builtin_fmaxf(x, y); };
  v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));  // lane ^ 1
  if (kLB == 4)
    v = mx(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));  // lane ^ 2
  return v;
}

// Codes (nibble i = value i) and scale byte of the kVP values x that one lane
// holds of a 16-value block whose other values sit in the neighbouring lanes of
// its group of kLB = 16 / kVP: the same decisions as qenc::encode_values on the
// whole block (amax over the group, then the fast or the threshold rule).
template <bool kPow2, int kVP>
__device__ __forceinline__ uint32_t encode_part(const float (&x)[kVP], float g, int& s) {
  constexpr int kLB = 16 / kVP;
  float ap = __builtin_fabsf(x[0]);  // NaN-propagating max of |x|
#pragma unroll
  for (int i = 1; i < kVP; ++i) ap = __builtin_elementwise_maximum(ap, __builtin_fabsf(x[i]));
  ap = block_lanes_max<kLB, true>(ap);
  const float six_g = 6.0f * g;
  bool fast = kPow2 && ap <= 2688.0f * g;  // 6 * 448 g: false for NaN and infinities
  if (fast) {
    s = (int)f32_to_e4m3(qenc::quotient(ap, six_g, 1.0f / six_g));
    fast = s != 0;
  }
  uint32_t cw = 0;
  if (fast) {  // the same on every lane of the block
    const float D = e4m3_to_f32((uint32_t)s) * g;
    const float r = 1.0f / D;
    auto q = [&](int i) { return qenc::quotient(x[i], D, r); };
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, q(0), q(1), 1.0f, 0);
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, q(2), q(3), 1.0f, 1);
    if (kVP == 8) {
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, q(4 % kVP), q(5 % kVP), 1.0f, 2);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, q(6 % kVP), q(7 % kVP), 1.0f, 3);
    }
  } else {
    using T = typename std::conditional<kPow2, float, double>::type;
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < kVP; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(x[i]));
    am = block_lanes_max<kLB, false>(am);  // NaN elements are left out of amax
    s = qenc::scale_byte<T>((T)am, (T)6 * (T)g);
    const T D = qenc::e4m3_value<T>(s) * (T)g;
#pragma unroll
    for (int i = 0; i < kVP; ++i) cw |= qenc::e2m1_code<T>(x[i], D, s == 0) << (4 * i);
  }
  return cw;
}

// One workgroup per (16 consecutive tokens, KV head, K|V). When the 16 tokens
// fill one page in order (slots s0 .. s0 + 15, s0 a multiple of 16), the
// workgroup owns that page's K or V slab of this head and writes it whole:
//   - the rows are read with consecutive lanes on consecutive 16-byte pieces
//     (a wave reads 1 KB per instruction), kVP values per lane, so the kLB
//     lanes of a 16-value block share its amax through DPP;
//   - each lane encodes its values and places codes and scale in an image of the
//     slab in LDS (K bytes by plain writes; V bytes, which hold two rows, by LDS
//     ORs into zeroed words);
//   - 72 lanes write the 1,152-byte slab out in 16-byte pieces.
// Otherwise thread (row, block) = (threadIdx / 8, threadIdx % 8) writes its block
// alone, as the shared block writer does. The rows are requested before the
// slots and the workgroup vote, so that the two memory round trips overlap.
// kPow2: the pool's global scale is a power of two (the fast encode); any other
// g takes the fp64 threshold encode in its own instantiation. kBf16: the source
// dtype (a.bf16).
template <bool kPow2, bool kBf16>
__global__ __launch_bounds__(128) void k_quantize(QuantizeArgs a) {
  constexpr int kVP = kBf16 ? 8 : 4;          // values per lane and 16-byte piece
  constexpr int kLanesPerRow = kBf16 ? 16 : 32;
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  constexpr int kLoads = 8 / kRowsPerLoad;    // a wave's 8 rows
  __shared__ __attribute__((aligned(16))) uint8_t img[kSlab];

  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kPage;
  const int kind = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane % kLanesPerRow;        // 16-byte piece of the row
  const int sub = lane / kLanesPerRow;
  const int blk = col * kVP / 16;             // its 16-value block
  const int d0 = col * kVP;                   // its first channel

  const uint8_t* src = static_cast<const uint8_t*>(kind ? a.v : a.k);
  const int esz = kBf16 ? 2 : 4;
  uint4 raw[kLoads];
#pragma unroll
  for (int p = 0; p < kLoads; ++p) {
    const int r = 8 * wave + kRowsPerLoad * p + sub;
    const int64_t t = min(t0 + r, a.num_tokens - 1);  // rows past the end: not used
    raw[p] = *reinterpret_cast<const uint4*>(src + (t * a.token_stride + (int64_t)h * a.head_stride + d0) * esz);
  }
  const int vrow = (tid >> 3) & 15;
  const int64_t vt = t0 + vrow;
  const bool live = vt < a.num_tokens;
  const int32_t slot = live ? a.slots[vt] : -1;
  const int32_t s0 = a.slots[t0];
  const bool whole = __syncthreads_and(live && s0 >= 0 && (s0 & (kPage - 1)) == 0 && slot == s0 + vrow);
  if (!whole) {
    if (slot >= 0) qenc::write_block<kPow2>(a, vt, slot, h, kind, tid & 7, true);
    return;
  }
  if (tid < kSlab / 16) reinterpret_cast<uint4*>(img)[tid] = make_uint4(0, 0, 0, 0);
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kLoads; ++p) {
    const int r = 8 * wave + kRowsPerLoad * p + sub;
    float x[kVP];
    const uint32_t w[4] = {raw[p].x, raw[p].y, raw[p].z, raw[p].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kBf16) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        x[i] = __uint_as_float(w[i]);
      }
    }
    int sb;
    const uint32_t cw = encode_part<kPow2, kVP>(x, a.g, sb);
    const bool first = (col % (16 / kVP)) == 0;  // the block's first lane writes its scale
    if (kind == 0) {
      // K: row r's codes at 64 r, channel d in byte d / 2 (even channel low)
      if (kBf16)
        *reinterpret_cast<uint32_t*>(img + r * 64 + d0 / 2) = cw;
      else
        *reinterpret_cast<uint16_t*>(img + r * 64 + d0 / 2) = (uint16_t)cw;
      if (first) img[kCodeBytes + r * 8 + blk] = (uint8_t)sb;
    } else {
      // V: channel d of row r in byte ((r/4)*16 + d/8)*16 + 2 (d%8) + r%2, high
      // nibble for r%4 >= 2; the lane's kVP channels fall in one 16-byte chunk,
      // two per 32-bit word
      uint32_t* chunk = reinterpret_cast<uint32_t*>(img + (((r >> 2) * 16 + (d0 >> 3)) * 16));
      const int sh = 8 * (r & 1) + 4 * ((r >> 1) & 1);
#pragma unroll
      for (int i = 0; i < kVP / 2; ++i) {
        const int e = (d0 & 7) + 2 * i;  // channels d0 + 2i, + 1: bytes 2e and 2e + 2 of the chunk
        const uint32_t bits = (((cw >> (8 * i)) & 15u) << sh) | (((cw >> (8 * i + 4)) & 15u) << (sh + 16));
        __hip_atomic_fetch_or(chunk + (e >> 1), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (first) img[kCodeBytes + blk * 16 + r] = (uint8_t)sb;
    }
  }
  __syncthreads();
  uint8_t* slab = a.pool + (((int64_t)(s0 / kPage) * a.num_kv_heads + h) * 2 + kind) * (int64_t)kSlab;
  if (tid < kSlab / 16) reinterpret_cast<uint4*>(slab)[tid] = reinterpret_cast<const uint4*>(img)[tid];
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
