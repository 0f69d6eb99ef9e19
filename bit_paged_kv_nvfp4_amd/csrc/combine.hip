// Merge of split-K decode partial states (gfx950).
//
// For every (sequence, query head) the S split states (M_s, Z_s, O_s) written by
// the split kernel are merged: M* = max M_s, w_s = 2^(M_s - M*) (0 for an empty
// split), out = sum w_s O_s / sum w_s Z_s, lse = (M* + log2 sum w_s Z_s) ln 2.
// One wave per (sequence, query head); lane i owns output channels 2i and 2i+1.
// The (M, Z) pairs are read first (lanes stride over the splits); O is read
// only for splits of nonzero weight: an empty split's O is never written (its
// pages were merged into another split's state), and at most 16 O rows are in
// flight at once.
#include "nvfp4kv_device.h"

namespace nvfp4kv {
namespace {

constexpr int kBatch = 16;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(64) void k_decode_combine(DecodeArgs a) {
  const int unit = blockIdx.x;  // b * Hq + qh
  const int lane = threadIdx.x;
  const int S = a.num_splits;
  const float2* __restrict__ ml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)unit * S;
  const float* __restrict__ po = a.part_o + (size_t)unit * S * kHeadDim + 2 * lane;

  float M = -__builtin_inff();
  for (int i = lane; i < S; i += 64) M = __builtin_fmaxf(M, ml[i].x);
  M = wave_max(M);
  float o0 = 0.0f, o1 = 0.0f, Ls = 0.0f;
  if (M != -__builtin_inff()) {
    for (int c0 = 0; c0 < S; c0 += 64) {
      const float2 st = c0 + lane < S ? ml[c0 + lane] : make_float2(-__builtin_inff(), 0.0f);
      const float wl = st.x == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(st.x - M);
      Ls += wl * st.y;
      uint64_t live = __builtin_amdgcn_ballot_w64(wl > 0.0f);  // splits whose O contributes
      while (live) {
        int idx[kBatch];
        float2 v[kBatch];
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          idx[k] = live ? __builtin_ctzll(live) : -1;
          if (live) {
            live &= live - 1;
            ++cnt;
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
          v[k] = idx[k] >= 0 ? *reinterpret_cast<const float2*>(po + (size_t)(c0 + idx[k]) * kHeadDim)
                             : make_float2(0.f, 0.f);
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          if (k < cnt) {
            const float wi = __shfl(wl, idx[k]);
            o0 += wi * v[k].x;
            o1 += wi * v[k].y;
          }
        }
      }
    }
    Ls = wave_sum(Ls);
    const float inv = 1.0f / Ls;
    o0 *= inv;
    o1 *= inv;
  }
  const size_t o = (size_t)unit * kHeadDim + 2 * lane;
  if (a.out_bf16) {
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const uint32_t packed = (uint32_t)f32_to_bf16_bits(o0) | ((uint32_t)f32_to_bf16_bits(o1) << 16);
    *reinterpret_cast<uint32_t*>(out + o) = packed;
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + o) = make_float2(o0, o1);
  }
  if (a.lse && lane == 0)
    a.lse[unit] = (M == -__builtin_inff()) ? -__builtin_inff() : (M + __builtin_log2f(Ls)) * 0.69314718055994530942f;
}

}  // namespace

hipError_t launch_decode_combine(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decode_combine, dim3(a.batch * a.num_q_heads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
