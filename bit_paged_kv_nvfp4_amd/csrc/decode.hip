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
//   O^T[128 x 16 heads]   += V^T[128 x 32] P^T     8 x v_mfma_f32_16x16x32_f16
// (the PV product takes two pages, 32 tokens, per MFMA).
// Lane (n = lane%16, G = lane/16):
//   K: loads 16 B = channels 32G..32G+31 of token n; MFMA step s uses channels
//      32G+8s..+7, and Q is loaded in the same channel order.
//   S^T fragment: head n, tokens 4G..4G+3, which is exactly the P^T operand the
//      PV product needs (k slots ordered tokens 4G+0, +2, +1, +3).
//   V: loads one 16-B chunk = channels 8n..8n+7 (half of scale block n/2) of
//      tokens 4G..4G+3, two codes of one channel per byte (tokens 4G+0|4G+2 and
//      4G+1|4G+3), so a conversion yields two k slots directly and the lane needs
//      one word of scales per page; row n of PV tile q is channel 8n + q.
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
#include "quantize_block.h"

namespace nvfp4kv {
namespace {

constexpr float kLazyRescaleLog2 = 8.0f;


__device__ __forceinline__ f16x2 pk_mul(uint32_t a, uint32_t b) { return as_f16x2(a) * as_f16x2(b); }

#ifndef NVFP4KV_DECODE_PAIRS_AHEAD
#define NVFP4KV_DECODE_PAIRS_AHEAD 1
#endif
constexpr int kPairsAhead = NVFP4KV_DECODE_PAIRS_AHEAD;  // pairs of pages in flight while one is computed
constexpr int kRing = 2 * (kPairsAhead + 1);              // LDS slots (pages) per wave
constexpr int kQDmas = 4;  // 1 KB copies of the group's queries (up to 16 heads x 256 B)
static_assert(kRing >= 4, "the query staging area takes the ring's last two slots");

// Page ids reach the wave the same way as page bytes: 64 at a time, copied into
// one of two LDS id buffers one chunk ahead of use. When the issue pointer enters
// a chunk, each lane loads one id of it into a register, and the id of a page is
// then taken with v_readlane (no memory round trip per page). A plain table load
// inside the loop would be a vector load that the compiler drains together with
// every copy in flight.
constexpr int kIdChunk = 64;

// Copy the ids of split-relative pages [64 k, 64 k + 64) (clamped to the split's
// last page) into id buffer k & 1. One vmcnt event.
__device__ __forceinline__ void issue_ids(const int32_t* pt_split, int k, int n_pages, uint32_t ids_lds, int lane) {
  const int rel = min(k * kIdChunk + lane, n_pages - 1);
  dma4(pt_split, (uint32_t)rel * 4u, ids_lds + (k & 1) * (kIdChunk * 4));
}

__device__ __forceinline__ const uint8_t* slab_of(const uint8_t* pool_h, int ids_v, int rel, int64_t page_bytes) {
  const int pid = __builtin_amdgcn_readlane(ids_v, rel % kIdChunk);
  return pool_h + (int64_t)pid * page_bytes;
}


// K^ rows of one MFMA step: channels 32G + 8s .. +7 of the lane's token, exact f16
// (E2M1 code times E4M3 scale / 256).
__device__ __forceinline__ f16x8 k_operand(uint32_t w, uint32_t scale_f16x2) {
  const f16x2 x0 = pk_mul(as_u32(fp4x2_to_f16x2<0>(w)), scale_f16x2);
  const f16x2 x1 = pk_mul(as_u32(fp4x2_to_f16x2<1>(w)), scale_f16x2);
  const f16x2 x2 = pk_mul(as_u32(fp4x2_to_f16x2<2>(w)), scale_f16x2);
  const f16x2 x3 = pk_mul(as_u32(fp4x2_to_f16x2<3>(w)), scale_f16x2);
  return f16x8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

// Both halves of a K scale pair: E4M3 byte SEL of ks as f16 bits (value / 256).
// Rows of never-written bytes may decode to NaN here: their scores are masked.
template <int SEL>
__device__ __forceinline__ uint32_t k_scale_pair(uint32_t ks) {
  return __builtin_amdgcn_perm(0u, ks, SEL == 0 ? 0x0C000C00u : 0x0C010C01u) << 7;
}

// V scale pairs of tokens (4G+0, 4G+2) and (4G+1, 4G+3), as f16 bits (value / 256).
// Bit 7 of each byte is dropped so that never-written bytes of masked rows still
// decode to finite values (their weight is an exact zero, and 0 * inf is NaN).
__device__ __forceinline__ uint32_t v_scales02(uint32_t vs) { return (vs << 7) & 0x3F803F80u; }
__device__ __forceinline__ uint32_t v_scales13(uint32_t vs) { return (vs >> 1) & 0x3F803F80u; }

// V^ of channel 8n + q (q = 0..7) for one page: code bytes 2q (tokens 4G+0 | 4G+2)
// and 2q + 1 (tokens 4G+1 | 4G+3) of the lane's chunk, i.e. k slots ordered
// tokens 4G+0, +2, +1, +3.
template <int Q>
__device__ __forceinline__ void v_operand(const uint4& vc, uint32_t s02, uint32_t s13, f16x2& x02, f16x2& x13) {
  const uint32_t w = Q < 2 ? vc.x : Q < 4 ? vc.y : Q < 6 ? vc.z : vc.w;
  x02 = pk_mul(as_u32(fp4x2_to_f16x2<2 * (Q & 1)>(w)), s02);
  x13 = pk_mul(as_u32(fp4x2_to_f16x2<2 * (Q & 1) + 1>(w)), s13);
}

template <int Q>
__device__ __forceinline__ void pv_tile(const uint4& va, const uint4& vb, uint32_t sa02, uint32_t sa13, uint32_t sb02,
                                        uint32_t sb13, const f16x8& pf, f32x4& acc) {
  f16x2 a02, a13, b02, b13;
  v_operand<Q>(va, sa02, sa13, a02, a13);
  v_operand<Q>(vb, sb02, sb13, b02, b13);
  const f16x8 v = {a02[0], a02[1], a13[0], a13[1], b02[0], b02[1], b13[0], b13[1]};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, pf, acc, 0, 0, 0);
}

// ---- page formats ----------------------------------------------------------
// A format says how one (page, KV head) K+V slab pair travels: its bytes in the
// pool, the per-lane copies into an LDS slot, the registers a lane takes from
// the slot, and the two products of a pair of pages. Lane (n = lane % 16,
// G = lane / 16) computes S^T rows = tokens 4G..4G+3 of both pages for head n,
// and the PV products take channel 8n + q as row n of output tile q.

// NVFP4 pages. An LDS slot holds [K code chunk of lane 0..63 | V code chunk of
// lane 0..63 | 128 K scale bytes | 128 V scale bytes].
struct Nvfp4Page {
  static constexpr int kSlotBytes = 2 * kSlab;  // 2304
  static constexpr int kHeadBytes = 2 * kSlab;  // pool bytes of one (page, head)
  static constexpr int kDmaPerPage = 3;
  static constexpr int kScaleLog2 = 8;          // K and V operands carry E4M3 scale / 256
  // Four workgroups of four waves per CU: LDS (under 40 KB per workgroup of the
  // CU's 160 KB) and registers (at most 128 VGPRs, four waves per SIMD).
  static constexpr int kWaves = 4;
  static constexpr int kWorkgroupsPerCu = 4;

  struct Offsets {
    uint32_t k, v, s;  // per-lane source offsets inside a (page, head) K+V slab pair
  };
  struct Regs {
    uint4 kc;     // K codes: 32 channels of one token
    uint32_t ks;  // its two K scale bytes
    uint4 vc;     // V codes: 8 channels (one half block) x 4 tokens
    uint32_t vs;  // the block's scale bytes of those 4 tokens
  };

  __device__ static __forceinline__ Offsets offsets(int lane) {
    const int n = lane & 15, G = lane >> 4;
    Offsets o;
    o.k = n * 64 + G * 16;                          // 32 K channels of token n
    o.v = kSlab + 16 * lane;                        // V chunk: channels 8n..8n+7, tokens 4G..4G+3
    o.s = lane < 8 ? kCodeBytes + 16 * lane         // lanes 0..7: K scale bytes
                   : kSlab + kCodeBytes + 16 * (lane - 8);  // lanes 8..15: V scale bytes
    return o;
  }

  // The copies of one (page, head) slab pair into an LDS slot (3 vmcnt events).
  __device__ static __forceinline__ void issue(const uint8_t* slab, const Offsets& o, uint32_t slot, int lane) {
    dma16_stream(slab, o.k, slot);
    dma16_stream(slab, o.v, slot + kCodeBytes);
    if (lane < 16) dma16_stream(slab, o.s, slot + 2 * kCodeBytes);
  }

  __device__ static __forceinline__ Regs read(const uint8_t* slot, int lane) {
    const int n = lane & 15, G = lane >> 4;
    Regs r;
    r.kc = *reinterpret_cast<const uint4*>(slot + 16 * lane);
    r.vc = *reinterpret_cast<const uint4*>(slot + kCodeBytes + 16 * lane);
    r.ks = *reinterpret_cast<const uint16_t*>(slot + 2 * kCodeBytes + n * 8 + G * 2);
    r.vs = *reinterpret_cast<const uint32_t*>(slot + 2 * kCodeBytes + 128 + (n >> 1) * 16 + G * 4);
    return r;
  }

  // Encode block j of K (kind 0) or V (kind 1) of token t of the new rows into
  // `slot`. The token is alone in this launch, so V nibbles go in with atomics.
  // Only a power-of-two global scale is written here; for any other g the host
  // writes the new rows with k_write_newest before this launch.
  __device__ static __forceinline__ void write_new(const QuantizeArgs& a, int64_t t, int64_t slot, int h, int kind,
                                                   int j) {
    qenc::write_block<true>(a, t, slot, h, kind, j, false);
  }

  // S^T = K^ Q^T for each page (two independent MFMA chains).
  __device__ static __forceinline__ void scores(const Regs& ra, const Regs& rb, const f16x8 (&qf)[4], f32x4& sa,
                                                f32x4& sb) {
    // Bit 7 of the scale bytes is kept (k_scale_pair): a never-written row past the
    // end of the sequence may score NaN, and pair_step's tail mask replaces its
    // logit by -inf and its weight by an exact 0 before either is used.
    const uint32_t ska0 = k_scale_pair<0>(ra.ks), ska1 = k_scale_pair<1>(ra.ks);
    const uint32_t skb0 = k_scale_pair<0>(rb.ks), skb1 = k_scale_pair<1>(rb.ks);
    const uint32_t kwa[4] = {ra.kc.x, ra.kc.y, ra.kc.z, ra.kc.w};
    const uint32_t kwb[4] = {rb.kc.x, rb.kc.y, rb.kc.z, rb.kc.w};
    sa = f32x4{0.f, 0.f, 0.f, 0.f};
    sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand(kwa[s], s < 2 ? ska0 : ska1), qf[s], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand(kwb[s], s < 2 ? skb0 : skb1), qf[s], sb, 0, 0, 0);
    }
  }

  // O^T += V^T P^T with the 32 tokens as the MFMA reduction: k slots 8G..8G+7 =
  // page A tokens 4G+0, +2, +1, +3, then the same of page B (two codes of one
  // channel share a V code byte: rows 4G+0 | 4G+2 and 4G+1 | 4G+3).
  __device__ static __forceinline__ void pv(const Regs& ra, const Regs& rb, const float (&p)[8], f32x4 (&acc)[8]) {
    const f16x8 pf = {(_Float16)p[0], (_Float16)p[2], (_Float16)p[1], (_Float16)p[3],
                      (_Float16)p[4], (_Float16)p[6], (_Float16)p[5], (_Float16)p[7]};
    const uint32_t sa02 = v_scales02(ra.vs), sa13 = v_scales13(ra.vs);
    const uint32_t sb02 = v_scales02(rb.vs), sb13 = v_scales13(rb.vs);
    pv_tile<0>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[0]);
    pv_tile<1>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[1]);
    pv_tile<2>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[2]);
    pv_tile<3>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[3]);
    pv_tile<4>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[4]);
    pv_tile<5>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[5]);
    pv_tile<6>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[6]);
    pv_tile<7>(ra.vc, rb.vc, sa02, sa13, sb02, sb13, pf, acc[7]);
  }
};

// FP8 E4M3 pages, the baseline the pages compare against (one byte per value,
// per-tensor scales folded into the softmax scale and the output). Pool slab
// pair of one (page, head): K [16 rows][128 channels], then V as 64 chunks of
// 32 B, chunk 16g + n = channels 8n..8n+7 of rows 4g..4g+3, word q = rows
// 4g..4g+3 of channel 8n + q. An LDS slot holds [K channels 32G..32G+15 of
// token n, lane 0..63 | K channels 32G+16..32G+31 | V chunk words 0..3 | V chunk
// words 4..7], 1 KB each.
struct Fp8Page {
  static constexpr int kSlabBytes = 2048;
  static constexpr int kSlotBytes = 2 * kSlabBytes;
  static constexpr int kHeadBytes = 2 * kSlabBytes;
  static constexpr int kDmaPerPage = 4;
  static constexpr int kScaleLog2 = 0;
  // Twice the slot of an NVFP4 page: two waves per workgroup keep a workgroup's
  // LDS at 34 KB, and four workgroups per CU give the same 8 waves' worth of
  // pages in flight per CU in bytes (VGPRs up to 256, two waves per SIMD).
  static constexpr int kWaves = 2;
  static constexpr int kWorkgroupsPerCu = 4;

  struct Offsets {
    uint32_t k, v;
  };
  struct Regs {
    uint4 k0, k1;  // K channels 32G..32G+15 and 32G+16..32G+31 of token n
    uint4 v0, v1;  // V chunk (G, n): words 0..3 and 4..7
  };

  __device__ static __forceinline__ Offsets offsets(int lane) {
    const int n = lane & 15, G = lane >> 4;
    Offsets o;
    o.k = n * 128 + G * 32;
    o.v = kSlabBytes + 32 * lane;
    return o;
  }

  __device__ static __forceinline__ void issue(const uint8_t* slab, const Offsets& o, uint32_t slot, int) {
    // plain copies: the streaming hint that helps the NVFP4 pages measured slower
    // here (73% -> 70% of HBM peak at batch 44 x 32K)
    dma16(slab, o.k, slot);
    dma16(slab, o.k + 16, slot + 1024);
    dma16(slab, o.v, slot + 2048);
    dma16(slab, o.v + 16, slot + 3072);
  }

  __device__ static __forceinline__ Regs read(const uint8_t* slot, int lane) {
    Regs r;
    r.k0 = *reinterpret_cast<const uint4*>(slot + 16 * lane);
    r.k1 = *reinterpret_cast<const uint4*>(slot + 1024 + 16 * lane);
    r.v0 = *reinterpret_cast<const uint4*>(slot + 2048 + 16 * lane);
    r.v1 = *reinterpret_cast<const uint4*>(slot + 3072 + 16 * lane);
    return r;
  }

  __device__ static __forceinline__ void write_new(const QuantizeArgs& a, int64_t t, int64_t slot, int h, int kind,
                                                   int j) {
    qenc::write_block_fp8(a, t, slot, h, kind, j);
  }

  // Four E4M3 bytes of w as exact f16 (the converter's scale operand stays 1.0).
  __device__ static __forceinline__ void f16x4_of(uint32_t w, f16x2& lo, f16x2& hi) {
    lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  }
  // K rows of MFMA step s: channels 32G + 8s .. +7 of the lane's token.
  __device__ static __forceinline__ f16x8 k_op(uint32_t w0, uint32_t w1) {
    f16x2 a, b, c, d;
    f16x4_of(w0, a, b);
    f16x4_of(w1, c, d);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }

  __device__ static __forceinline__ void scores(const Regs& ra, const Regs& rb, const f16x8 (&qf)[4], f32x4& sa,
                                                f32x4& sb) {
    const uint32_t ka[8] = {ra.k0.x, ra.k0.y, ra.k0.z, ra.k0.w, ra.k1.x, ra.k1.y, ra.k1.z, ra.k1.w};
    const uint32_t kb[8] = {rb.k0.x, rb.k0.y, rb.k0.z, rb.k0.w, rb.k1.x, rb.k1.y, rb.k1.z, rb.k1.w};
    sa = f32x4{0.f, 0.f, 0.f, 0.f};
    sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_op(ka[2 * s], ka[2 * s + 1]), qf[s], sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_op(kb[2 * s], kb[2 * s + 1]), qf[s], sb, 0, 0, 0);
    }
  }

  // k slots 8G..8G+7 = page A tokens 4G..4G+3, then page B's; tile q takes word q
  // of each page's chunk (tokens 4G..4G+3 of channel 8n + q).
  __device__ static __forceinline__ void pv(const Regs& ra, const Regs& rb, const float (&p)[8], f32x4 (&acc)[8]) {
    const f16x8 pf = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                      (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
    const uint32_t va[8] = {ra.v0.x, ra.v0.y, ra.v0.z, ra.v0.w, ra.v1.x, ra.v1.y, ra.v1.z, ra.v1.w};
    const uint32_t vb[8] = {rb.v0.x, rb.v0.y, rb.v0.z, rb.v0.w, rb.v1.x, rb.v1.y, rb.v1.z, rb.v1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      f16x2 a0, a1, b0, b1;
      f16x4_of(va[q], a0, a1);
      f16x4_of(vb[q], b0, b1);
      const f16x8 v = {a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, pf, acc[q], 0, 0, 0);
    }
  }
};

// Two pages (32 tokens) per step: the format's S^T products, one online-softmax
// update over the 32 tokens, and the format's PV products. Tokens at or past
// `lim` (the end of the split or of the sequence) are masked.
template <class F>
__device__ __forceinline__ void pair_step(const typename F::Regs& ra, const typename F::Regs& rb, int tok_a, int lim,
                                          int G, const f16x8 (&qf)[4], float c, float& m_ref, float& lsum,
                                          f32x4 (&acc)[8]) {
  f32x4 sa, sb;
  F::scores(ra, rb, qf, sa, sb);

  // ---- online softmax (base 2) over tokens 4G..4G+3 of both pages, head n ----
  // Logits are z = s * c with c > 0 (the query sign absorbs the sign of the
  // softmax scale), so the maximum is taken on the raw scores s and each weight
  // is exp2(fma(s, c, -m)).
  float z[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = sa[i];
    z[4 + i] = sb[i];
  }
  const bool tail = tok_a + 2 * kPage > lim;  // only the last pair of a split has rows to mask
  const int t0 = tok_a + 4 * G;
  if (tail) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = (t0 + i < lim) ? z[i] : -__builtin_inff();
      z[4 + i] = (t0 + kPage + i < lim) ? z[4 + i] : -__builtin_inff();
    }
  }
  float mx = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(z[0], z[1]), __builtin_fmaxf(z[2], z[3])),
                             __builtin_fmaxf(__builtin_fmaxf(z[4], z[5]), __builtin_fmaxf(z[6], z[7])));
  mx = xor16_max(mx);
  mx = xor32_max(mx) * c;
  const bool need = mx > m_ref + kLazyRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    const float m_new = need ? mx : m_ref;
    const float alpha = (m_new == m_ref) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
    lsum *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    m_ref = m_new;
  }
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], c, -m_ref));
  if (tail) {  // exact zeros for masked rows, also when c == 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = (t0 + i < lim) ? p[i] : 0.0f;
      p[4 + i] = (t0 + kPage + i < lim) ? p[4 + i] : 0.0f;
    }
  }
  lsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  F::pv(ra, rb, p, acc);
}

// A value every lane holds the same copy of, moved to scalar registers so that
// what is derived from it (loads of seq_lens, the page table) is scalar too.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A load from read-only memory at an index every lane shares, through the
// scalar path (constant address space): a vector load here would be awaited with
// a wait that also drains every page copy in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int64_t idx) {
  using const_i32 = const __attribute__((address_space(4))) int32_t;
  return ((const_i32*)p)[uniform(idx)];  // address-space cast
}

// Pages of sequence b (0 for a sequence of length 0); b is the same on every lane.
__device__ __forceinline__ int seq_pages(const DecodeArgs& a, int b) {
  return (load_uniform(a.seq_lens, b) + kPage - 1) / kPage;
}
// The same for a per-lane b.
__device__ __forceinline__ int seq_pages_lane(const DecodeArgs& a, int b) { return (a.seq_lens[b] + kPage - 1) / kPage; }

// s_setprio level from the share of `quota` pages still left: 3 above 1/3, 2
// above 1/6, 1 above 1/12, 0 for the rest. Each step down lets the waves that
// trail catch up; the steps sit late, where the spread of finish times forms.
__device__ __forceinline__ void set_priority(int left, int quota) {
  const int level = (int)(left * 3 > quota) + (int)(left * 6 > quota) + (int)(left * 12 > quota);
  switch (level) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// Pages [pg0, pg1) of sequence b, KV head h, for one wave: online-softmax state
// (acc, m_ref, lsum; lsum still per lane) of all query heads of the group.
template <class F>
__device__ __forceinline__ void wave_share(const DecodeArgs& a, int b, int h, int pg0, int pg1, int lane,
                                           uint8_t* ring, int32_t* ids, f32x4 (&acc)[8], float& m_ref,
                                           float& lsum, int& left, int quota) {
  const int n = lane & 15;
  const int G = lane >> 4;
  b = uniform(b);
  h = uniform(h);
  pg0 = uniform(pg0);
  pg1 = uniform(pg1);
  m_ref = -__builtin_inff();
  lsum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (pg0 >= pg1) return;

  const int L = load_uniform(a.seq_lens, b);  // >= 1: the share is not empty
  if (a.write_new) {
    // The sequence's newest token (position L - 1) goes into the pool first,
    // written by the wave whose share holds its page and finished before any
    // copy of that page: 16 lanes, one block (K or V, 16 channels) each.
    const int last = (L - 1) / kPage;
    if (last >= pg0 && last < pg1) {
      if (lane < 16) {
        const int64_t slot =
            (int64_t)load_uniform(a.page_table, (int64_t)b * a.pt_stride + last) * kPage + (L - 1) % kPage;
        F::write_new(a.nw, b, slot, h, lane >> 3, lane & 7);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the row has reached the cache hierarchy
    }
  }
  const bool head_ok = n < a.group;
  const uint8_t* pool_h = a.pool + (int64_t)h * F::kHeadBytes;
  const int64_t page_bytes = (int64_t)a.num_kv_heads * F::kHeadBytes;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
  const uint32_t ids_lds = (uint32_t)(uintptr_t)ids;
  const typename F::Offsets off = F::offsets(lane);
  const int n_pages = pg1 - pg0;
  const int n_pairs = (n_pages + 1) / 2;
  const int lim = min(L, pg1 * kPage);  // tokens of this share end here
  const int32_t* pt_split = a.page_table + (int64_t)b * a.pt_stride + pg0;

  // Start-up: the first two id chunks and the group's queries are copied at
  // once, the first pages go out as soon as the ids have landed, and the queries
  // are converted while those pages are in flight. The queries are staged in the
  // ring's last two slots, which the loop's first refill overwrites only after
  // they have been read.
  const uint32_t q_lds = ring_lds + (kRing - 2) * F::kSlotBytes;
  const uint8_t* qsrc =
      reinterpret_cast<const uint8_t*>(a.q + ((size_t)b * a.num_q_heads + (size_t)h * a.group) * kHeadDim);
  const uint32_t qbytes = (uint32_t)a.group * (kHeadDim * 2);  // 256 .. 4096
  issue_ids(pt_split, 0, n_pages, ids_lds, lane);
  issue_ids(pt_split, 1, n_pages, ids_lds, lane);
#pragma unroll
  for (int k = 0; k < kQDmas; ++k)
    dma16(qsrc, min((uint32_t)(k * 1024 + 16 * lane), qbytes - 16u), q_lds + k * 1024);
  wait_dma<kQDmas>();  // the ids have landed
  int ids_v = ids[lane];  // chunk 0
  // The ring holds kPairsAhead + 1 pairs: one being computed, the others in
  // flight. Pages past the share's end re-read its last page (masked by `lim`),
  // so every iteration issues the same number of copies and the wait count is a
  // constant.
#pragma unroll
  for (int j = 0; j < 2 * kPairsAhead; ++j)
    F::issue(slab_of(pool_h, ids_v, min(j, n_pages - 1), page_bytes), off, ring_lds + j * F::kSlotBytes, lane);
  wait_dma<2 * kPairsAhead * F::kDmaPerPage>();  // the queries have landed

  // ---- Q: head n of the group, channels 32G..32G+31, as f16 after rescale ----
  float qv[32];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(ring + (kRing - 2) * F::kSlotBytes + n * (kHeadDim * 2) + 64 * G);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = head_ok ? qp[i] : make_uint4(0, 0, 0, 0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
        qv[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // staging slots read: free for the refill
  float qmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) qmax = __builtin_fmaxf(qmax, __builtin_fabsf(qv[i]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, o));
  int qexp = 0;
  if (qmax > 0.0f) {
    int e2;
    (void)__builtin_frexpf(qmax, &e2);  // qmax = m * 2^e2, m in [0.5, 1)
    qexp = e2 - 15;                      // qmax * 2^-qexp in [2^14, 2^15)
  }
  // A negative softmax scale is carried by the query's sign (exact), so that the
  // logit multiplier c below is positive.
  const float qmul = a.qk_scale_log2 < 0.0f ? -__builtin_ldexpf(1.0f, -qexp) : __builtin_ldexpf(1.0f, -qexp);
  f16x8 qf[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[st][e] = (_Float16)(qv[8 * st + e] * qmul);
  // z (base-2 logit) = S_acc * c: undoes the Q rescale and the format's scaling
  // of the K operand (1/256 of the E4M3 block scales for NVFP4)
  const float c = __builtin_ldexpf(__builtin_fabsf(a.qk_scale_log2), qexp + F::kScaleLog2);

  int cur = 0;  // ring slot of the current pair's first page
  for (int i = 0; i < n_pairs; ++i) {
    // Issue priority follows the work this wave has left: the hardware favours
    // the oldest wave, which would otherwise finish far ahead of waves started
    // with it while the CU idles at the end.
    set_priority(left, quota);
    left -= 2;
    const int ahead = 2 * (i + kPairsAhead);  // first page of the pair to fetch now
    if (ahead % kIdChunk == 0 && ahead < n_pages) {
      // Entering id chunk k = ahead / 64: its buffer has landed long ago; take
      // its ids into the register and refill the other buffer with chunk k + 1.
      ids_v = ids[((ahead / kIdChunk) & 1) * kIdChunk + lane];
      issue_ids(pt_split, ahead / kIdChunk + 1, n_pages, ids_lds, lane);
    }
    const int nxt = cur == 0 ? kRing - 2 : cur - 2;  // the slot pair freed last iteration
    F::issue(slab_of(pool_h, ids_v, min(ahead, n_pages - 1), page_bytes), off, ring_lds + nxt * F::kSlotBytes,
             lane);
    F::issue(slab_of(pool_h, ids_v, min(ahead + 1, n_pages - 1), page_bytes), off,
             ring_lds + (nxt + 1) * F::kSlotBytes, lane);
    wait_dma<2 * kPairsAhead * F::kDmaPerPage>();  // the current pair's copies have landed
    const typename F::Regs ra = F::read(ring + cur * F::kSlotBytes, lane);
    const typename F::Regs rb = F::read(ring + (cur + 1) * F::kSlotBytes, lane);
    pair_step<F>(ra, rb, (pg0 + 2 * i) * kPage, lim, G, qf, c, m_ref, lsum, acc);
    cur = cur + 2 == kRing ? 0 : cur + 2;
  }
  wait_dma<0>();  // no copy may outlive the wave's use of its LDS
}


// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    v += lane >= o ? t : 0;
  }
  return v;
}

// Work decomposition. The launch's work is the units (b, h, s): split s < S of
// sequence b and KV head h covers pages [s P_b, min((s+1) P_b, n_b)), P_b =
// ceil(n_b / S). In the flattened page space, where (b, h) occupies
// [Hkv cum_b + h n_b, + n_b) (cum_b = pages of the sequences before b), a unit
// starts at its segment's start + min(s P_b, n_b). Workgroup g owns the units
// that start in [g T / W, (g + 1) T / W), T = total pages, W = workgroups (the
// last one owns everything after its start). Its units form at most a few runs
// of consecutive splits of one (b, h); a run is processed as one range of pages,
// its waves taking equal shares, and writes one state (in its first split's
// slot; the run's other splits get empty states).
struct Cursor {
  int b;        // sequence (a.batch: past the end)
  int64_t seg;  // flattened start of segment (b, 0)
  int np;       // pages of sequence b
};

// The first unit in index order that starts at or after flattened page pos: its
// sequence's cursor and (h, s), where s may be S (then the unit is the first of
// (b, h + 1), or of the next sequence). Every lane computes the same.
struct UnitPos {
  Cursor cu;
  int h;
  int s;
};

__device__ __forceinline__ UnitPos locate(const DecodeArgs& a, int64_t pos, int lane) {
  const int S = a.num_splits;
  const int Hkv = a.num_kv_heads;
  // the first b whose segments end at or after pos
  Cursor cu{a.batch, 0, 0};
  int64_t base = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    const int bb = c0 + lane;
    const int np = bb < a.batch ? seq_pages_lane(a, bb) : 0;
    const int64_t incl = wave_incl_scan((int64_t)Hkv * np, lane);  // segments of b <= bb end at base + incl
    const uint64_t hit = __builtin_amdgcn_ballot_w64(bb < a.batch && base + incl >= pos);
    if (hit) {
      const int k = __builtin_ctzll(hit);
      const int64_t incl_k = uniform((int64_t)__shfl(incl, k));
      const int np_k = uniform(__shfl(np, k));
      cu = Cursor{uniform(c0 + k), base + incl_k - (int64_t)Hkv * np_k, np_k};
      break;
    }
    base += uniform((int64_t)__shfl(incl, 63));
  }
  UnitPos u{cu, 0, 0};
  if (cu.b < a.batch && pos > cu.seg) {
    // Here cu.seg < pos <= cu.seg + Hkv np, so np > 0. With rel = pos - cu.seg in
    // [1, Hkv np], segment h = (rel - 1) / np holds offset r = rel - h np in
    // [1, np], and its unit s = ceil(r / P) is the first to start at or after pos
    // (s = S: none does; r = np: the segment's empty trailing splits start
    // exactly at pos).
    const int P = (cu.np + S - 1) / S;
    const int64_t rel = pos - cu.seg;
    u.h = (int)((rel - 1) / cu.np);
    const int64_t r = rel - (int64_t)u.h * cu.np;
    u.s = (int)((r + P - 1) / P);
  }
  return u;
}

// One run: splits s .. s1 of (b, h), np = pages of sequence b. The waves take
// equal shares of its pages, then the last wave to finish merges the shares and
// writes the run's state; the closing barrier frees every ring for the next run.
template <class F>
__device__ __forceinline__ void run(const DecodeArgs& a, int b, int h, int s, int s1, int np, int wave, int lane,
                                    uint8_t* ring_base, int32_t* ids_base, int* waves_done, int& left, int quota) {
  constexpr int kWaves = F::kWaves;
  constexpr int kRingBytes = kRing * F::kSlotBytes;
  const int S = a.num_splits;
  const int P = (np + S - 1) / S;
  const int rp0 = min(s * P, np);
  const int rp1 = min((s1 + 1) * P, np);
  // this wave's share: an even number of pages, so that only the last pair of
  // the share can hold masked rows
  const int share = (((rp1 - rp0 + kWaves - 1) / kWaves) + 1) & ~1;
  const int pg0 = min(rp0 + wave * share, rp1);
  const int pg1 = min(pg0 + share, rp1);

  // The lane index is re-read each run so that the many values derived from it
  // (copy offsets, LDS addresses) are rebuilt here rather than hoisted and kept
  // live across the page loop, where registers are scarce.
  int ln;
  asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
  const int n = ln & 15;
  const int G = ln >> 4;
  uint8_t* const ring = ring_base + wave * kRingBytes;
  f32x4 acc[8];
  float m_ref, lsum;
  wave_share<F>(a, b, h, pg0, pg1, ln, ring, ids_base + wave * (2 * kIdChunk), acc, m_ref, lsum, left, quota);

  // ---- merge the waves' states; the last wave to finish writes the run's ----
  lsum = xor16_sum(lsum);
  lsum = xor32_sum(lsum);  // per head n, on every lane of head n
  {
    // own state into own ring region (its copies have all landed): acc as
    // [q][lane] float4s, then (m, l) per head
    float4* acc_lds = reinterpret_cast<float4*>(ring);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc_lds[q * 64 + ln] = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
    if (G == 0) reinterpret_cast<float2*>(ring + 8 * 64 * 16)[n] = make_float2(m_ref, lsum);
  }
  int prior = 0;
  if (ln == 0) prior = __hip_atomic_fetch_add(waves_done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  prior = __builtin_amdgcn_readfirstlane(prior);
  if (prior == kWaves - 1) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    float mw[kWaves], lw[kWaves];
    float m_all = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float2 ml = reinterpret_cast<const float2*>(ring_base + w * kRingBytes + 8 * 64 * 16)[n];
      mw[w] = ml.x;
      lw[w] = ml.y;
      m_all = __builtin_fmaxf(m_all, ml.x);
    }
    float l_all = 0.0f;
    f32x4 o_all[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) o_all[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      // an empty share has m = -inf and weight 0; so does everything when all are
      const float f = (mw[w] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mw[w] - m_all);
      l_all += f * lw[w];
      const float4* src = reinterpret_cast<const float4*>(ring_base + w * kRingBytes);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = src[q * 64 + ln];
        o_all[q][0] += f * v.x;
        o_all[q][1] += f * v.y;
        o_all[q][2] += f * v.z;
        o_all[q][3] += f * v.w;
      }
    }
    if (n < a.group) {
      const int qh = h * a.group + n;
      const size_t unit = ((size_t)b * a.num_q_heads + qh) * S + s;
      float* po = a.part_o + unit * kHeadDim;
      // o_all[q][r] is O^T[channel 8 (4G + r) + q][head n], in units of
      // 2^-kScaleLog2 of the value scale (NVFP4 V scales travel as E4M3/256)
      const float vs = __builtin_ldexpf(a.v_scale, F::kScaleLog2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 v0 = make_float4(o_all[0][r] * vs, o_all[1][r] * vs, o_all[2][r] * vs, o_all[3][r] * vs);
        const float4 v1 = make_float4(o_all[4][r] * vs, o_all[5][r] * vs, o_all[6][r] * vs, o_all[7][r] * vs);
        *reinterpret_cast<float4*>(po + 32 * G + 8 * r) = v0;
        *reinterpret_cast<float4*>(po + 32 * G + 8 * r + 4) = v1;
      }
      // the run's state, then empty states for its other splits
      float2* pml = reinterpret_cast<float2*>(a.part_ml) + unit;
      for (int k = G; k <= s1 - s; k += 4) pml[k] = k == 0 ? make_float2(m_all, l_all) : make_float2(-__builtin_inff(), 0.0f);
    }
    *waves_done = 0;  // for the next run; the barrier below orders it
  }
  __syncthreads();  // every wave's state has been merged: rings may be reused
}

template <class F>
__device__ __forceinline__ void decode_split(const DecodeArgs& a) {
  constexpr int kWaves = F::kWaves;
  static_assert(kRing * F::kSlotBytes >= 8 * 64 * 16 + 16 * 8, "a wave's state must fit its ring region");
  static_assert(2 * F::kSlotBytes >= 16 * kHeadDim * 2, "the group's queries must fit two ring slots");
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform by construction
  const int lane = threadIdx.x & 63;
  const int S = a.num_splits;
  const int Hkv = a.num_kv_heads;
  const int g = blockIdx.x;
  const int W = gridDim.x;

  __shared__ int waves_done;
  __shared__ __attribute__((aligned(16))) uint8_t ring_all[kWaves][kRing * F::kSlotBytes];
  __shared__ __attribute__((aligned(16))) int32_t ids_all[kWaves][2 * kIdChunk];
  if (threadIdx.x == 0) waves_done = 0;
  __syncthreads();

  // ---- total pages and this workgroup's window (every wave computes the same) ----
  int64_t total = 0;
  for (int c0 = 0; c0 < a.batch; c0 += 64) {
    const int bb = c0 + lane;
    int64_t v = bb < a.batch ? (int64_t)Hkv * seq_pages_lane(a, bb) : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    total += v;
  }
  total = uniform(total);
  const int64_t lo = total * g / W;
  const int64_t hi = g == W - 1 ? INT64_MAX : total * (g + 1) / W;

  // ---- runs ----
  // pages this wave is expected to process (its share of the window), and left
  const int quota = (int)min<int64_t>((min(hi, total) - lo) / kWaves + 1, 1 << 26);  // left * 12 fits int
  int left = quota;
  uint8_t* const ring_base = &ring_all[0][0];
  int32_t* const ids_base = &ids_all[0][0];
  const UnitPos at = locate(a, lo, lane);
  Cursor cu = at.cu;
  int h = at.h;
  int s = at.s;
  while (cu.b < a.batch) {
    if (s >= S) {  // (b, h) exhausted: next head, or next sequence
      s = 0;
      if (++h >= Hkv) {
        h = 0;
        cu.seg += (int64_t)Hkv * cu.np;
        if (++cu.b >= a.batch) break;
        cu.np = seq_pages(a, cu.b);
      }
      continue;
    }
    const int np = cu.np;
    const int P = (np + S - 1) / S;
    const int64_t seg = cu.seg + (int64_t)h * np;
    auto unit_start = [&](int k) -> int64_t { return seg + min((int64_t)k * P, (int64_t)np); };
    if (unit_start(s) >= hi) break;  // the window ends before this unit
    // the run: splits s .. s1 of (b, h), all starting before hi
    int s1 = S - 1;
    if (unit_start(S - 1) >= hi) {
      // last split starting before hi (P > 0 here, since the unit at s starts before hi)
      const int64_t last = (hi - 1 - seg) / P;  // split index of page hi - 1 relative to seg
      s1 = (int)min<int64_t>(last, S - 1);
    }
    run<F>(a, cu.b, h, s, s1, np, wave, lane, ring_base, ids_base, &waves_done, left, quota);
    s = s1 + 1;
  }
}

template <class F>
constexpr int lds_per_workgroup() {
  return F::kWaves * (kRing * F::kSlotBytes + 2 * kIdChunk * 4) + 16;
}
static_assert(Nvfp4Page::kWorkgroupsPerCu * lds_per_workgroup<Nvfp4Page>() <= 160 * 1024,
              "the NVFP4 workgroups of a CU must fit its LDS");
static_assert(Fp8Page::kWorkgroupsPerCu * lds_per_workgroup<Fp8Page>() <= 160 * 1024,
              "the FP8 workgroups of a CU must fit its LDS");
static_assert(lds_per_workgroup<Nvfp4Page>() <= 64 * 1024 && lds_per_workgroup<Fp8Page>() <= 64 * 1024,
              "a workgroup addresses at most 64 KB of LDS");

// Four NVFP4 workgroups of four waves per CU (at most 128 VGPRs: four waves per
// SIMD); four FP8 workgroups of two waves (at most 256 VGPRs).
__global__ __launch_bounds__(64 * Nvfp4Page::kWaves) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_split(
    DecodeArgs a) {
  decode_split<Nvfp4Page>(a);
}
__global__ __launch_bounds__(64 * Fp8Page::kWaves) __attribute__((amdgpu_waves_per_eu(2))) void k_decode_split_fp8(
    DecodeArgs a) {
  decode_split<Fp8Page>(a);
}

}  // namespace

int decode_waves_per_split(bool fp8) { return fp8 ? Fp8Page::kWaves : Nvfp4Page::kWaves; }

// More workgroups than fit would only queue behind the resident ones; the
// kernel's result does not depend on the count.
int decode_resident_workgroups(int num_cus, bool fp8) {
  return (fp8 ? Fp8Page::kWorkgroupsPerCu : Nvfp4Page::kWorkgroupsPerCu) * (num_cus > 0 ? num_cus : 1);
}

hipError_t launch_decode_partial(const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.fp8)
    hipLaunchKernelGGL(k_decode_split_fp8, dim3(a.num_workgroups), dim3(64 * Fp8Page::kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(k_decode_split, dim3(a.num_workgroups), dim3(64 * Nvfp4Page::kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
