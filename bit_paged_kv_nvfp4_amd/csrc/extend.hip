// Extend (chunked-prefill) attention over a dequantized prefix workspace and the
// chunk's own keys and values (gfx950 / CDNA4).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): in the
// extend path the cached NVFP4 prefix is dequantized into a bf16/FP8 workspace
// and attention then runs over it. Here query i of a C-token chunk that follows
// a P-token prefix attends over all P workspace rows and over chunk rows 0..i
// (causal), with query head q reading KV head q / (Hq / Hkv).
//
// Work item: one workgroup of four waves per (KV head, block of chunk tokens).
// Consecutive workgroups take consecutive KV heads, so with Hkv = 8 every block
// of one head runs on one XCD and the head's K/V stream is shared through that
// XCD's L2. A wave owns 32 rows, row = token_in_block * group + head, and per
// 64-key tile computes
//   S^T[64 keys x 32 rows] = K[64 x 128] Q^T      32 x v_mfma_f32_16x16x32_bf16
//   O^T[128 x 32 rows]    += V^T[128 x 64] P^T    32 x v_mfma_f32_16x16x32_f16
// A 16x16x32 MFMA lane (n = lane % 16, G = lane / 16) holds row n of A and
// column n of B with k slots 8G..8G+7, and column n, rows 4G..4G+3 of C. So the
// S^T fragment of a lane (row n; keys 4G..4G+3 of each 16-key block) is already
// a P^T operand: its k slots are keys 4G..4G+3 of block 2ks, then of block
// 2ks+1, and the V^T operand is read with the same key order.
// K and V^T of a tile are staged in LDS (the next tile waits in registers while
// the current one is computed). 16-byte K pieces and 8-byte V^T pieces are
// XOR-swizzled by row, so the 16 rows that a quarter-wave reads hit distinct
// banks. The V^T transpose happens in registers with byte permutes.
// K enters the first product as bf16 (FP8 workspace bytes widen exactly), V the
// second as f16, converted on the way into LDS: exact for every value of
// magnitude below 65504, which covers every NVFP4- or FP8-derived workspace value
// (at g = 1) and every chunk value a model produces.
// Online softmax in fp32, base 2, with a lazy rescale (the running max moves
// only when a tile's max exceeds it by more than 2^8, so P <= 256); P enters
// the second product as f16 (11 significant bits, where bf16 would keep 8 and
// miss the error bar when few keys share the weight), and the row sums add up
// the same rounded values.
#include "nvfp4kv.h"
#include "nvfp4kv_device.h"

namespace nvfp4kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kXWaves = 4;
constexpr int kXRows = 32;  // rows per wave
constexpr int kTile = 64;   // keys per tile
constexpr float kXLazyLog2 = 8.0f;

struct TileRegs {
  uint4 k[4];  // K pieces t + 256 j: key p / 16, channels 8 (p % 16) .. +7
  uint4 v[4];  // V of keys 4 (t / 16) + j, channels 8 (t % 16) .. +7
};

// Raw 8 elements (channels 8c .. 8c+7) of key row kp: prefix rows come from the
// workspace (FP8 bytes land in .x, .y), chunk rows from the chunk, rows past the
// chunk are zero.
__device__ __forceinline__ uint4 load8(const ExtendArgs& a, const void* pre, const uint16_t* chunk, int h,
                                       int64_t kp, int c) {
  uint4 r = make_uint4(0u, 0u, 0u, 0u);
  if (kp < a.prefix_len) {
    const int64_t e = (kp * a.num_kv_heads + h) * kHeadDim + 8 * c;
    if (a.pre_fp8) {
      const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(pre) + e);
      r.x = w.x;
      r.y = w.y;
    } else {
      r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(pre) + e);
    }
  } else if (kp - a.prefix_len < a.chunk_len) {
    r = *reinterpret_cast<const uint4*>(chunk + ((kp - a.prefix_len) * a.num_kv_heads + h) * kHeadDim + 8 * c);
  }
  return r;
}

// Two E4M3 values (as f32) -> two bf16 in one word; exact, since three mantissa
// bits fit in bf16's seven.
__device__ __forceinline__ uint32_t pack_bf16_exact(f32x2 f) {
  return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
}

// The raw elements of key row kp as 8 bf16.
__device__ __forceinline__ uint4 widen8(const ExtendArgs& a, int64_t kp, uint4 r) {
  if (a.pre_fp8 && kp < a.prefix_len) {
    return make_uint4(pack_bf16_exact(__builtin_amdgcn_cvt_pk_f32_fp8(r.x, false)),
                      pack_bf16_exact(__builtin_amdgcn_cvt_pk_f32_fp8(r.x, true)),
                      pack_bf16_exact(__builtin_amdgcn_cvt_pk_f32_fp8(r.y, false)),
                      pack_bf16_exact(__builtin_amdgcn_cvt_pk_f32_fp8(r.y, true)));
  }
  return r;
}

// Two floats -> two f16 (nearest, ties to even) in one word.
__device__ __forceinline__ uint32_t f16x2_rne(float x0, float x1) {
  const f16x2 h = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, h);
}

// The raw elements of key row kp as 8 f16 (the value operand of the second
// product). Exact for every value of magnitude below 65504: the workspace holds
// E4M3 or NVFP4 products, and a bf16 value in f16's normal range needs at most
// 8 of its 11 significant bits.
__device__ __forceinline__ uint4 widen8_f16(const ExtendArgs& a, int64_t kp, uint4 r) {
  uint4 o;
  if (a.pre_fp8 && kp < a.prefix_len) {
    const f32x2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8(r.x, false), f1 = __builtin_amdgcn_cvt_pk_f32_fp8(r.x, true);
    const f32x2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8(r.y, false), f3 = __builtin_amdgcn_cvt_pk_f32_fp8(r.y, true);
    o = make_uint4(f16x2_rne(f0[0], f0[1]), f16x2_rne(f1[0], f1[1]), f16x2_rne(f2[0], f2[1]), f16x2_rne(f3[0], f3[1]));
  } else {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = f16x2_rne(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xFFFF0000u));
    o = make_uint4(h[0], h[1], h[2], h[3]);
  }
  return o;
}

__device__ __forceinline__ void load_tile(const ExtendArgs& a, int h, int64_t base, int t, TileRegs& x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = t + 256 * j;
    x.k[j] = load8(a, a.k_pre, a.k_chunk, h, base + (p >> 4), p & 15);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) x.v[j] = load8(a, a.v_pre, a.v_chunk, h, base + 4 * (t >> 4) + j, t & 15);
}

// k_lds: [key][16 pieces of 16 B], piece c of key r at index r * 16 + (c ^ (r & 15)).
// vt_lds: [channel][16 pieces of 8 B = 4 keys], piece q of channel d at
// d * 16 + (q ^ (d & 15)).
__device__ __forceinline__ void store_tile(const ExtendArgs& a, int64_t base, int t, const TileRegs& x,
                                           uint4* k_lds, uint2* vt_lds) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = t + 256 * j;
    const int r = p >> 4, c = p & 15;
    k_lds[r * 16 + (c ^ (r & 15))] = widen8(a, base + r, x.k[j]);
  }
  const int q = t >> 4, c = t & 15;
  uint4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = widen8_f16(a, base + 4 * q + j, x.v[j]);
  const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
  const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
  const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
  const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // word w of a key holds channels 8c + 2w (low half) and 8c + 2w + 1 (high)
    const int d0 = 8 * c + 2 * w, d1 = d0 + 1;
    vt_lds[d0 * 16 + (q ^ (d0 & 15))] = make_uint2(__builtin_amdgcn_perm(w1[w], w0[w], 0x05040100u),
                                                   __builtin_amdgcn_perm(w3[w], w2[w], 0x05040100u));
    vt_lds[d1 * 16 + (q ^ (d1 & 15))] = make_uint2(__builtin_amdgcn_perm(w1[w], w0[w], 0x07060302u),
                                                   __builtin_amdgcn_perm(w3[w], w2[w], 0x07060302u));
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two finite floats -> two bf16 (nearest, ties to even) in one word.
__device__ __forceinline__ uint32_t bf16x2_rne(float x0, float x1) {
  const f32x2 f = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__global__ __launch_bounds__(64 * kXWaves) __attribute__((amdgpu_waves_per_eu(1))) void k_extend_attn(ExtendArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int n = lane & 15, G = lane >> 4;
  const int Hkv = a.num_kv_heads;
  const int h = blockIdx.x % Hkv;
  const int tb = a.num_token_blocks - 1 - (int)(blockIdx.x / Hkv);  // longest blocks first
  const int grp = a.group;
  const int64_t P = a.prefix_len, C = a.chunk_len;
  const int64_t t_first = (int64_t)tb * a.tokens_per_block;
  const int64_t t_last = min(t_first + a.tokens_per_block, C) - 1;
  const int64_t n_keys = P + t_last + 1;
  const int n_tiles = (int)((n_keys + kTile - 1) / kTile);

  __shared__ uint4 k_lds[kTile * 16];
  __shared__ uint2 vt_lds[kHeadDim * 16];

  TileRegs nxt;
  load_tile(a, h, 0, t, nxt);

  // this lane's rows (one per row block): token, query head; tokens past the
  // chunk (or rows past the block's tokens) are computed but never stored
  int64_t tok[2];
  int qh[2];
  bool valid[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = wave * kXRows + 16 * rb + n;
    const int tl = row / grp;
    tok[rb] = t_first + tl;
    qh[rb] = h * grp + row % grp;
    valid[rb] = tl < a.tokens_per_block && tok[rb] < C;
    if (!valid[rb]) tok[rb] = INT64_MAX / 4;  // sees every key: no masking
  }
  // Q^T operands: column = row, k slots = channels 32 s + 8 G .. +7
  bf16x8 qf[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 u = make_uint4(0u, 0u, 0u, 0u);
      if (valid[rb])
        u = *reinterpret_cast<const uint4*>(a.q + (tok[rb] * a.num_q_heads + qh[rb]) * kHeadDim + 32 * s + 8 * G);
      u.x ^= a.q_sign;
      u.y ^= a.q_sign;
      u.z ^= a.q_sign;
      u.w ^= a.q_sign;
      qf[rb][s] = __builtin_bit_cast(bf16x8, u);
    }
  const float c2 = a.qk_scale_log2;  // >= 0: a negative scale is folded into the sign of Q

  f32x4 oacc[8][2];
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[d][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};
  float lsum[2] = {0.f, 0.f};

  for (int it = 0; it < n_tiles; ++it) {
    const int64_t base = (int64_t)it * kTile;
    __syncthreads();  // every wave is done with the previous tile
    store_tile(a, base, t, nxt, k_lds, vt_lds);
    __syncthreads();
    if (it + 1 < n_tiles) load_tile(a, h, base + kTile, t, nxt);

    // ---- S^T = K Q^T ----
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sacc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int r = 16 * kb + n;
        const bf16x8 kf = __builtin_bit_cast(bf16x8, k_lds[r * 16 + ((4 * s + G) ^ n)]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][s], sacc[kb][rb], 0, 0, 0);
      }

    // ---- mask: key kp is visible to token i iff kp <= P + i ----
    if (base + kTile - 1 > P + t_first) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t kp = base + 16 * kb + 4 * G + r;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            if (kp > P + tok[rb]) sacc[kb][rb][r] = -__builtin_inff();
        }
    }

    // ---- online softmax (base 2, lazy rescale) ----
    float mt[2];
    bool need[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = __builtin_fmaxf(mx, sacc[kb][rb][r]);
      mx = xor32_max(xor16_max(mx));
      mt[rb] = mx * c2;
      need[rb] = mt[rb] > m_ref[rb] + kXLazyLog2;
    }
    if (__builtin_amdgcn_ballot_w64(need[0] || need[1])) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float alpha = need[rb] ? __builtin_amdgcn_exp2f(m_ref[rb] - mt[rb]) : 1.0f;
        m_ref[rb] = need[rb] ? mt[rb] : m_ref[rb];
        lsum[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d][rb] *= alpha;
      }
    }
    // P^T operands: k slots = keys 4G..4G+3 of block 2ks, then of block 2ks + 1
    uint32_t pw[2][2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mu = m_ref[rb] == -__builtin_inff() ? 0.0f : m_ref[rb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const f16x2 ph = {(_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][r], c2, -mu)),
                            (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][r + 1], c2, -mu))};
          lsum[rb] += (float)ph[0] + (float)ph[1];
          pw[rb][kb >> 1][(kb & 1) * 2 + (r >> 1)] = __builtin_bit_cast(uint32_t, ph);
        }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f16x8 pf[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        pf[rb] = __builtin_bit_cast(f16x8, make_uint4(pw[rb][ks][0], pw[rb][ks][1], pw[rb][ks][2], pw[rb][ks][3]));
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int dim = 16 * d + n;
        const uint2 v0 = vt_lds[dim * 16 + ((8 * ks + G) ^ n)];
        const uint2 v1 = vt_lds[dim * 16 + ((8 * ks + 4 + G) ^ n)];
        const f16x8 vf = __builtin_bit_cast(f16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) oacc[d][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[rb], oacc[d][rb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l as bf16; lse in natural log ----
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = xor32_sum(xor16_sum(lsum[rb]));
    if (!valid[rb]) continue;
    const float inv = 1.0f / l;
    uint16_t* o = a.out + (tok[rb] * a.num_q_heads + qh[rb]) * kHeadDim;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const f32x4 v = oacc[d][rb] * inv;
      // channels 16 d + 4 G .. +3 of this row
      *reinterpret_cast<uint2*>(o + 16 * d + 4 * G) = make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
    }
    if (a.lse != nullptr && G == 0) a.lse[tok[rb] * a.num_q_heads + qh[rb]] = (m_ref[rb] + __builtin_log2f(l)) * 0.69314718055994531f;
  }
}

}  // namespace

int extend_tokens_per_block(int group) { return kXWaves * kXRows / group; }

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  if (a.chunk_len == 0) return hipSuccess;
  hipLaunchKernelGGL(k_extend_attn, dim3((unsigned)a.num_token_blocks * (unsigned)a.num_kv_heads),
                     dim3(64 * kXWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
