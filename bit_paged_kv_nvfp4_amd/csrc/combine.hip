// Merge of split-K decode partial states (gfx950).
//
// For every (sequence, query head) the S split states (M_s, Z_s, O_s) written by
// the split kernel are merged: M* = max M_s, w_s = 2^(M_s - M*) (0 for an empty
// split), out = sum w_s O_s / sum w_s Z_s, lse = (M* + log2 sum w_s Z_s) ln 2.
// One workgroup per (sequence, query head), one wave per 64 splits (at most 16
// waves, taking every 16th chunk of 64 beyond that); lane i owns output channels
// 2i and 2i+1. Each wave reads its (M, Z) pairs first; O is read only for splits
// of nonzero weight: an empty split's O is never written (its pages were merged
// into another split's state), and at most 16 O rows are in flight per wave.
// With several waves, wave 0 merges their states through LDS the same way.
// Measured with 1024 splits (2 sequences x 64 heads): one wave per (sequence,
// head) took 22-28 us, bounded by its chain of dependent loads.
#include <algorithm>

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

// Waves per (sequence, query head): one per 64 splits, at most kMaxWaves.
constexpr int kMaxWaves = 16;

__global__ __launch_bounds__(64 * kMaxWaves) void k_decode_combine(DecodeArgs a) {
  const int unit = blockIdx.x;  // b * Hq + qh
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int S = a.num_splits;
  const float2* __restrict__ ml = reinterpret_cast<const float2*>(a.part_ml) + (size_t)unit * S;
  const float* __restrict__ po = a.part_o + (size_t)unit * S * kHeadDim + 2 * lane;

  // this wave's splits: chunks of 64 starting at 64 (wave + k nw)
  float M = -__builtin_inff();
  for (int i = 64 * wave + lane; i < S; i += 64 * nw) M = __builtin_fmaxf(M, ml[i].x);
  M = wave_max(M);
  float o0 = 0.0f, o1 = 0.0f, Ls = 0.0f;
  if (M != -__builtin_inff()) {
    for (int c0 = 64 * wave; c0 < S; c0 += 64 * nw) {
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
  }

  if (nw > 1) {
    // merge the waves' states (M_w, Ls_w, O_w relative to 2^M_w) in wave 0
    __shared__ float sM[kMaxWaves], sL[kMaxWaves];
    __shared__ float2 sO[kMaxWaves][64];
    sO[wave][lane] = make_float2(o0, o1);
    if (lane == 0) {
      sM[wave] = M;
      sL[wave] = Ls;
    }
    __syncthreads();
    if (wave != 0) return;
    float Mt = -__builtin_inff();
    for (int w = 0; w < nw; ++w) Mt = __builtin_fmaxf(Mt, sM[w]);
    o0 = o1 = Ls = 0.0f;
    if (Mt != -__builtin_inff()) {
      for (int w = 0; w < nw; ++w) {
        if (sM[w] == -__builtin_inff()) continue;
        const float f = __builtin_amdgcn_exp2f(sM[w] - Mt);
        const float2 ow = sO[w][lane];
        o0 += f * ow.x;
        o1 += f * ow.y;
        Ls += f * sL[w];
      }
    }
    M = Mt;
  }
  if (M != -__builtin_inff()) {
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
  const int nw = std::min(kMaxWaves, std::max(1, (a.num_splits + 63) / 64));
  hipLaunchKernelGGL(k_decode_combine, dim3(a.batch * a.num_q_heads), dim3(64 * nw), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
