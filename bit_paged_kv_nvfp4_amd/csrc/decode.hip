// Split-K flash-decoding over the paged NVFP4 cache with in-register dequant
// (gfx950 / CDNA4).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): the decode
// path dequantizes inside the attention kernel instead of expanding the cache
// first. Page "NVFP4-KV-Cache auf der NVIDIA RTX PRO 6000 Blackwell Server
// Edition" (section Geschwindigkeit): the decode kernel multiplies 16-bit queries
// with dequantized NVFP4 keys and values, reading fewer bytes per token.
//
// Work item: one wave64 per (split, KV head, sequence). It owns a contiguous
// range of the sequence's pages and all query heads of the KV group (up to 16),
// so every K/V byte is read once per decode step and shared by the group through
// the matrix cores:
//   S^T[16 tok x 16 heads] = K^[16 x 128] Q^T      4 x v_mfma_f32_16x16x32_f16
//   O^T[128 x 16 heads]   += V^T[128 x 16] P^T     8 x v_mfma_f32_16x16x16_f16
// Lane (n = lane%16, G = lane/16):
//   K: loads 16 B = channels 32G..32G+31 of token n; MFMA step s uses channels
//      32G+8s..+7, and Q is loaded in the same channel order.
//   S^T fragment: head n, tokens 4G..4G+3, which is exactly the P^T operand the
//      PV product needs (k slots ordered tokens 4G+0, +2, +1, +3).
//   V: loads one 16-B chunk = tokens 4G..4G+3 of channel pairs n, 16+n, 32+n,
//      48+n; pair 16q+n feeds two 16-row tiles (even / odd channel of the pair).
// Dequant: v_cvt_scalef32_pk_f16_fp4 turns two codes into exact f16 values (its
// scale operand only carries a power of two, so it is left at 1.0); one
// v_pk_mul_f16 by the E4M3 block scale (as f16, divided by 256 so that every
// scale byte maps exactly) finishes two values. Products of a 2-bit code and a
// 4-bit scale are exact in f16. Q is converted to f16 after a power-of-two
// rescale that puts the group's largest |q| in [2^14, 2^15), so the conversion is
// exact for every element within 2^31 of that maximum. Online softmax runs in
// fp32 in base 2 with a lazy rescale: the running max only moves when a page's
// max exceeds it by more than 2^8, which keeps P <= 256 (exact enough in f16) and
// skips most accumulator rescales.
#include "nvfp4kv_device.h"

namespace nvfp4kv {
namespace {

constexpr float kLazyRescaleLog2 = 8.0f;

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

// Low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

__device__ __forceinline__ f16x2 pk_mul(uint32_t a, uint32_t b) { return as_f16x2(a) * as_f16x2(b); }

struct PageRegs {
  uint4 kc;     // K codes: 32 channels of one token
  uint32_t ks;  // its two K scale bytes
  uint4 vc;     // V codes: 4 tokens x 4 channel pairs
  uint4 vs;     // the matching V scale bytes
};

struct LaneOffsets {
  int k, ks, v, vs;  // byte offsets inside a (page, head) K+V slab pair
};

__device__ __forceinline__ LaneOffsets lane_offsets(int n, int G) {
  LaneOffsets o;
  o.k = n * 64 + G * 16;
  o.ks = kCodeBytes + n * 8 + G * 2;
  o.v = kSlab + (n * 4 + G) * 16;
  o.vs = kSlab + kCodeBytes + (G * 2 + (n >> 3)) * 16;
  return o;
}

__device__ __forceinline__ void load_page(PageRegs& r, const uint8_t* base, const LaneOffsets& o) {
  r.kc = *reinterpret_cast<const uint4*>(base + o.k);
  r.ks = *reinterpret_cast<const uint16_t*>(base + o.ks);
  r.vc = *reinterpret_cast<const uint4*>(base + o.v);
  r.vs = *reinterpret_cast<const uint4*>(base + o.vs);
}

// One page of 16 tokens: S^T = K^ Q^T, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void page_step(const PageRegs& r, int pg, int L, int G, const f16x8 (&qf)[4], float c,
                                          float& m_ref, float& lsum, f32x4 (&acc)[8]) {
  // ---- S^T = K^ Q^T over 4 steps of 32 channels ----
  // scale bytes of finite E4M3 values are <= 0x7E; bit 7 is dropped so that even
  // bytes of never-written (masked) rows decode to finite values
  const uint32_t sk0 = e4m3_f16bits_div256((r.ks & 0x7Fu) * 0x00010001u);
  const uint32_t sk1 = e4m3_f16bits_div256(((r.ks >> 8) & 0x7Fu) * 0x00010001u);
  const uint32_t kw[4] = {r.kc.x, r.kc.y, r.kc.z, r.kc.w};
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t sc = s < 2 ? sk0 : sk1;
    const f16x2 x0 = pk_mul(as_u32(fp4x2_to_f16x2<0>(kw[s])), sc);
    const f16x2 x1 = pk_mul(as_u32(fp4x2_to_f16x2<1>(kw[s])), sc);
    const f16x2 x2 = pk_mul(as_u32(fp4x2_to_f16x2<2>(kw[s])), sc);
    const f16x2 x3 = pk_mul(as_u32(fp4x2_to_f16x2<3>(kw[s])), sc);
    const f16x8 kf = {x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[s], sacc, 0, 0, 0);
  }

  // ---- online softmax (base 2), tokens 4G..4G+3 of head n ----
  float z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = sacc[i] * c;
  if ((pg + 1) * kPage > L) {  // only the last page of a sequence has rows past its end
    const int tok0 = pg * kPage + 4 * G;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (tok0 + i < L) ? z[i] : -__builtin_inff();
  }
  float mx = __builtin_fmaxf(__builtin_fmaxf(z[0], z[1]), __builtin_fmaxf(z[2], z[3]));
  mx = xor16_max(mx);
  mx = xor32_max(mx);
  const bool need = mx > m_ref + kLazyRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    const float m_new = need ? mx : m_ref;
    const float alpha = (m_new == m_ref) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    m_ref = m_new;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(z[i] - m_ref);
  lsum += (p[0] + p[1]) + (p[2] + p[3]);
  const f16x4 pf = {(_Float16)p[0], (_Float16)p[2], (_Float16)p[1], (_Float16)p[3]};

  // ---- O^T += V^T P^T ----
  const uint32_t vw[4] = {r.vc.x, r.vc.y, r.vc.z, r.vc.w};
  const uint32_t vsw[4] = {r.vs.x, r.vs.y, r.vs.z, r.vs.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t r0 = as_u32(fp4x2_to_f16x2<0>(vw[q]));
    const uint32_t r1 = as_u32(fp4x2_to_f16x2<1>(vw[q]));
    const uint32_t r2 = as_u32(fp4x2_to_f16x2<2>(vw[q]));
    const uint32_t r3 = as_u32(fp4x2_to_f16x2<3>(vw[q]));
    const uint32_t s02 = (vsw[q] << 7) & 0x3F803F80u;  // scales of tokens 4G+0, 4G+2
    const uint32_t s13 = (vsw[q] >> 1) & 0x3F803F80u;  // scales of tokens 4G+1, 4G+3
    const f16x2 e0 = pk_mul(pack_lo(r0, r2), s02);
    const f16x2 e1 = pk_mul(pack_lo(r1, r3), s13);
    const f16x2 o0 = pk_mul(pack_hi(r0, r2), s02);
    const f16x2 o1 = pk_mul(pack_hi(r1, r3), s13);
    const f16x4 ve = {e0[0], e0[1], e1[0], e1[1]};
    const f16x4 vo = {o0[0], o0[1], o1[0], o1[1]};
    acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(ve, pf, acc[2 * q], 0, 0, 0);
    acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vo, pf, acc[2 * q + 1], 0, 0, 0);
  }
}

__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_decode_split(DecodeArgs a) {
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int G = lane >> 4;
  const int S = a.num_splits;

  const int L = a.seq_lens[b];
  const int npages = (L + kPage - 1) / kPage;
  const int pps = (npages + S - 1) / S;
  const int pg0 = split * pps;
  const int pg1 = min(pg0 + pps, npages);

  // ---- Q: head n of the group, channels 32G..32G+31, as f16 after rescale ----
  const bool head_ok = n < a.group;
  const int qh = h * a.group + n;
  float qv[32];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((size_t)b * a.num_q_heads + (head_ok ? qh : 0)) * kHeadDim + 32 * G);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 u = head_ok ? qp[i] : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
        qv[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
  float qmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qmax = __builtin_fmaxf(qmax, __builtin_fabsf(qv[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, off));
  int qexp = 0;
  if (qmax > 0.0f) {
    int e2;
    (void)__builtin_frexpf(qmax, &e2);  // qmax = m * 2^e2, m in [0.5, 1)
    qexp = e2 - 15;                      // qmax * 2^-qexp in [2^14, 2^15)
  }
  const float qmul = __builtin_ldexpf(1.0f, -qexp);
  f16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[s][e] = (_Float16)(qv[8 * s + e] * qmul);
  // z (base-2 logit) = S_acc * c: undoes the Q rescale and the 1/256 of the K scales
  const float c = __builtin_ldexpf(a.qk_scale_log2, qexp + 8);

  float m_ref = -__builtin_inff();
  float lsum = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* pt_row = a.page_table + (int64_t)b * a.pt_stride;
  const uint8_t* pool_h = a.pool + (int64_t)h * (2 * kSlab);
  const int64_t page_bytes = (int64_t)a.num_kv_heads * (2 * kSlab);
  const LaneOffsets off = lane_offsets(n, G);

  // Two register sets of raw page bytes in ping-pong: the next page is fetched
  // while the current one is computed, so every wave keeps two pages of loads in
  // flight without register copies between iterations.
  // The prefetch is unconditional (past the split's end it re-reads its last
  // page) so that no branch sits between a load and the wait for older loads.
  PageRegs A, Bq;
  const int last = pg1 - 1;
  if (pg0 < pg1) load_page(A, pool_h + (int64_t)pt_row[pg0] * page_bytes, off);
  for (int pg = pg0; pg < pg1; pg += 2) {
    load_page(Bq, pool_h + (int64_t)pt_row[min(pg + 1, last)] * page_bytes, off);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this page's math
    page_step(A, pg, L, G, qf, c, m_ref, lsum, acc);
    if (pg + 1 >= pg1) break;
    load_page(A, pool_h + (int64_t)pt_row[min(pg + 2, last)] * page_bytes, off);
    __builtin_amdgcn_sched_barrier(0);
    page_step(Bq, pg + 1, L, G, qf, c, m_ref, lsum, acc);
  }

  // ---- partial result of this split ----
  lsum = xor16_sum(lsum);
  lsum = xor32_sum(lsum);
  if (head_ok) {
    const size_t unit = ((size_t)b * a.num_q_heads + qh) * S + split;
    float* po = a.part_o + unit * kHeadDim;
    // acc[2q + par][r] is O^T[channel 32q + 2(4G + r) + par][head n]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v0 = make_float4(acc[2 * q][0], acc[2 * q + 1][0], acc[2 * q][1], acc[2 * q + 1][1]);
      const float4 v1 = make_float4(acc[2 * q][2], acc[2 * q + 1][2], acc[2 * q][3], acc[2 * q + 1][3]);
      *reinterpret_cast<float4*>(po + 32 * q + 8 * G) = v0;
      *reinterpret_cast<float4*>(po + 32 * q + 8 * G + 4) = v1;
    }
    if (G == 0) *reinterpret_cast<float2*>(a.part_ml + unit * 2) = make_float2(m_ref, lsum);
  }
}

// One wave per (sequence, query head): merge the splits' partials.
__global__ __launch_bounds__(64) void k_decode_combine(DecodeArgs a) {
  const int unit = blockIdx.x;  // b * Hq + qh
  const int lane = threadIdx.x;
  const int S = a.num_splits;
  const float* ml = a.part_ml + (size_t)unit * S * 2;
  const float* po = a.part_o + (size_t)unit * S * kHeadDim;
  float M = -__builtin_inff();
  for (int i = 0; i < S; ++i) M = __builtin_fmaxf(M, ml[2 * i]);
  float o0 = 0.0f, o1 = 0.0f, Ls = 0.0f;
  if (M != -__builtin_inff()) {
    for (int i = 0; i < S; ++i) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * i] - M);
      const float2 v = *reinterpret_cast<const float2*>(po + (size_t)i * kHeadDim + 2 * lane);
      Ls += w * ml[2 * i + 1];
      o0 += w * v.x;
      o1 += w * v.y;
    }
    const float inv = (a.v_scale * 256.0f) / Ls;  // V scales were carried as E4M3/256
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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(k_decode_split, dim3(a.num_splits, a.num_kv_heads, a.batch), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_combine, dim3(a.batch * a.num_q_heads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
