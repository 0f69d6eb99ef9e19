// Extend (chunked-prefill) attention over a dequantized prefix workspace and the
// chunk's own keys and values (gfx950 / CDNA4).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): in the
// extend path the cached NVFP4 prefix is dequantized into a bf16/FP8 workspace
// and attention then runs over it. Here query i of a C-token chunk that follows
// a P-token prefix attends over all P workspace rows and over chunk rows 0..i
// (causal), with query head q reading KV head q / (Hq / Hkv).
//
// Work item: one workgroup of eight waves per (KV head, block of chunk tokens),
// one per CU (two waves per SIMD); the eight waves share every K/V tile, so the
// copies and conversions of a tile serve 256 rows. Consecutive workgroups take consecutive KV heads,
// so with Hkv = 8 every block of one head runs on one XCD and the head's K/V
// stream is shared through that XCD's L2. A wave owns 32 rows, row =
// token_in_block * group + head, and per 64-key tile computes
//   S^T[64 keys x 32 rows] = K[64 x 128] Q^T      32 x v_mfma_f32_16x16x32_bf16
//   O^T[128 x 32 rows]    += V^T[128 x 64] P^T    32 x v_mfma_f32_16x16x32_f16
// A 16x16x32 MFMA lane (n = lane % 16, G = lane / 16) holds row n of A and
// column n of B with k slots 8G..8G+7, and column n, rows 4G..4G+3 of C. So the
// S^T fragment of a lane (row n; keys 4G..4G+3 of each 16-key block) is already
// a P^T operand: its k slots are keys 4G..4G+3 of block 2ks, then of block
// 2ks+1, and the V^T operand is read with the same key order.
//
// Tiles: the prefix in 64-key tiles (the last one may be partial), then the
// chunk in 64-key tiles, so that every tile has one source dtype. Each tile's
// K and V rows are copied global -> LDS asynchronously (global_load_lds) into a
// three-stage ring, two tiles ahead of the one being computed. A bf16 K tile
// lands directly in the layout the first product reads; raw V (and FP8 K) are
// then converted by the whole workgroup: V into a transposed f16 tile, FP8 K
// into bf16 (both exact). 16-byte and 8-byte pieces are XOR-swizzled by row so
// that the rows a quarter-wave reads fall in distinct banks.
// K enters the first product as bf16, V the second as f16: V is first
// multiplied by a power of two v_mul (1 unless the caller's bound on |V| exceeds
// 2^15) and the output by 1 / v_mul, so that V stays inside the f16 range; the
// conversion is then exact for magnitudes in [2^-14, 65504] (after the scaling),
// and below 2^-14 the absolute error stays under 2^-25 / v_mul.
// With a pool given, the kernel also quantize-writes the chunk's K/V into it
// (the prefill path's quantize fused into the attention), each workgroup the
// blocks of its own tokens and KV head.
// Online softmax in fp32, base 2, with a lazy rescale (the running max moves
// only when a tile's max exceeds it by more than 2^8, so P <= 256); P enters
// the second product as f16 (11 significant bits, where bf16 would keep 8 and
// miss the error bar when few keys share the weight), and the row sums add up
// the same rounded values, on the matrix cores (an all-ones operand).
#include "nvfp4kv.h"
#include "nvfp4kv_device.h"
#include "quantize_block.h"

namespace nvfp4kv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kXWaves = 8;
constexpr int kXThreads = 64 * kXWaves;
constexpr int kXRows = 32;                  // rows per wave
constexpr int kTile = 64;                   // keys per tile
constexpr int kStages = 3;                  // copies run two tiles ahead
constexpr int kStageBytes = kTile * 256;    // a tile of bf16 rows of one head
constexpr float kXLazyLog2 = 8.0f;

// Barrier for LDS data only: the workgroup's LDS writes are complete and
// visible; outstanding global -> LDS copies are left running.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Two floats -> two bf16 / f16 (nearest, ties to even) in one word.
__device__ __forceinline__ uint32_t bf16x2_rne(float x0, float x1) {
  const f32x2 f = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ uint32_t f16x2_rne(float x0, float x1) {
  const f16x2 h = {(_Float16)x0, (_Float16)x1};
  return __builtin_bit_cast(uint32_t, h);
}
// E4M3 bytes 0,1 (hi = false) or 2,3 of w as two f32 (exact).
__device__ __forceinline__ f32x2 fp8x2(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}
// Two exact E4M3 values as two bf16 (three mantissa bits fit in seven).
__device__ __forceinline__ uint32_t bf16x2_exact(f32x2 f) {
  return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
}

// Prefix workspace kinds: bf16 rows, FP8 E4M3 rows, or bf16 K rows with V as
// f16 tiles already in the PV operand order (NVFP4KV_F16_TILED).
constexpr int kPreBf16 = 0, kPreFp8Rows = 1, kPreTiled = 2;

// One tile: its keys' source rows and dtype.
struct Tile {
  const uint8_t* k;  // K row of the tile's first key, this head
  const uint8_t* v;  // V row of the tile's first key, or the tile's V^T (vtile)
  int n_valid;       // keys of the tile that exist (the rest is masked)
  bool fp8;          // rows are E4M3 bytes (else bf16)
  bool vtile;        // V arrives as a ready f16 V^T tile (16 KB, operand order)
  bool chunk;        // chunk tile (causal mask) or prefix tile
  int64_t first;     // index of the first key in the chunk (chunk tile) or prefix
};

template <int kPre>
__device__ __forceinline__ Tile tile_of(const ExtendArgs& a, int h, int n_pre, int i) {
  Tile x;
  const int64_t Hkv = a.num_kv_heads;
  if (i < n_pre) {
    constexpr bool fp8 = kPre == kPreFp8Rows;
    x.first = (int64_t)i * kTile;
    x.n_valid = (int)min<int64_t>(kTile, a.prefix_len - x.first);
    x.fp8 = fp8;
    x.vtile = kPre == kPreTiled;
    x.chunk = false;
    const int64_t row = (x.first * Hkv + h) * kHeadDim * (fp8 ? 1 : 2);
    x.k = static_cast<const uint8_t*>(a.k_pre) + row;
    x.v = static_cast<const uint8_t*>(a.v_pre) + (x.vtile ? ((int64_t)i * Hkv + h) * (kTile * kHeadDim * 2) : row);
  } else {
    x.first = (int64_t)(i - n_pre) * kTile;
    x.n_valid = (int)min<int64_t>(kTile, a.chunk_len - x.first);
    x.fp8 = false;
    x.vtile = false;
    x.chunk = true;
    const int64_t row = (x.first * Hkv + h) * kHeadDim * 2;
    x.k = reinterpret_cast<const uint8_t*>(a.k_chunk) + row;
    x.v = reinterpret_cast<const uint8_t*>(a.v_chunk) + row;
  }
  return x;
}

// Copies of a tile into one ring stage by wave w (of 8): 4 per wave for bf16
// rows, 2 for FP8 rows. LDS layouts of a stage:
//   K bf16: piece (16 B) c of key r at 16-byte slot r * 16 + (c ^ (r & 15))
//   V bf16: piece c of key r at slot r * 16 + (c ^ ((r >> 1) & 15))
//   K FP8:  piece (16 B = 16 channels) j of key r at slot r * 8 + j
//   V FP8:  piece j of key r at slot r * 8 + (j ^ ((r >> 1) & 7))
// Keys past n_valid copy the tile's last valid row (in bounds; masked later).
//   V^T tile (vtile): the f16 tile lands in the V^T layout below (vt_unit), its
//   16-byte units XOR-swizzled by channel as the conversion pass writes them.
__device__ __forceinline__ void issue_tile(const Tile& x, int hkv, uint32_t k_lds, uint32_t v_lds, int w,
                                           int lane) {
  if (!x.fp8) {
    const uint32_t rs = (uint32_t)hkv * 256;  // bytes between consecutive keys of one head
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int p = (2 * w + j) * 64 + lane;
      const int r = p >> 4, cs = p & 15;
      const uint32_t rr = (uint32_t)min(r, x.n_valid - 1);
      dma16(x.k, rr * rs + 16 * (cs ^ (r & 15)), k_lds + (2 * w + j) * 1024);
      if (x.vtile) {
        // LDS unit p = 8 d + u' holds source unit u' ^ (d & 7) of channel d
        const int d = p >> 3, up = p & 7;
        dma16(x.v, (uint32_t)(d * 128 + 16 * (up ^ (d & 7))), v_lds + (2 * w + j) * 1024);
      } else {
        dma16(x.v, rr * rs + 16 * (cs ^ ((r >> 1) & 15)), v_lds + (2 * w + j) * 1024);
      }
    }
  } else {
    const uint32_t rs = (uint32_t)hkv * 128;
    const int p = w * 64 + lane;
    const int r = p >> 3, cs = p & 7;
    const uint32_t rr = (uint32_t)min(r, x.n_valid - 1);
    dma16(x.k, rr * rs + 16 * cs, k_lds + w * 1024);
    dma16(x.v, rr * rs + 16 * (cs ^ ((r >> 1) & 7)), v_lds + w * 1024);
  }
}

// V^T tile (f16), one 128-byte row per channel d. A PV operand of key half ks
// and lane group G holds keys 32 ks + 4 G .. +3 and 32 ks + 16 + 4 G .. +3 of
// its channel, so 16-byte unit u = 4 ks + G of the row holds exactly those 8
// keys (the second four in its upper 8 bytes), at byte d * 128 + 16 (u ^ (d & 7)):
// one ds_read_b128 per operand, and the 8 rows a group of 8 lanes reads fall in
// 8 different 16-byte bank groups. Keys 4q .. 4q+3 (q < 16) are unit
// 4 (q / 8) + q % 4, half (q / 4) % 2.
__device__ __forceinline__ uint32_t vt_unit(int d, int u) { return d * 128 + 16 * (u ^ (d & 7)); }
__device__ __forceinline__ uint32_t vt_piece(int d, int q) {
  return vt_unit(d, 4 * (q >> 3) + (q & 3)) + 8 * ((q >> 2) & 1);
}

// Workgroup pass over a landed stage: raw V -> V^T (f16); FP8 K -> bf16 K in the
// K-operand layout. Thread t: channels 8c .. 8c+7 (c = t / 32) of keys 2m, 2m+1
// (m = t % 32).
// V is multiplied by vmul (a power of two, 1 unless the caller's bound on |V|
// needs it) before the conversion, so that it stays inside the f16 range.
__device__ __forceinline__ void convert_tile(bool fp8, int t, const uint8_t* k_st, const uint8_t* v_st,
                                             uint8_t* vt, uint8_t* kconv, float vmul) {
  const int c = t >> 5, m = t & 31;
  uint32_t lo[4], hi[4];  // channels (8c + 2e, 8c + 2e + 1) of key 2m and of key 2m + 1, as f16 pairs
  float f0[8], f1[8];     // the same values as f32 (exact)
  if (!fp8) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(v_st + 16 * ((2 * m) * 16 + (c ^ (m & 15))));
    const uint4 a1 = *reinterpret_cast<const uint4*>(v_st + 16 * ((2 * m + 1) * 16 + (c ^ (m & 15))));
    const uint32_t w0[4] = {a0.x, a0.y, a0.z, a0.w}, w1[4] = {a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f0[2 * e] = __uint_as_float(w0[e] << 16);
      f0[2 * e + 1] = __uint_as_float(w0[e] & 0xFFFF0000u);
      f1[2 * e] = __uint_as_float(w1[e] << 16);
      f1[2 * e + 1] = __uint_as_float(w1[e] & 0xFFFF0000u);
    }
  } else {
    const int off = 16 * ((c >> 1) ^ (m & 7)) + 8 * (c & 1);
    const uint2 b0 = *reinterpret_cast<const uint2*>(v_st + (2 * m) * 128 + off);
    const uint2 b1 = *reinterpret_cast<const uint2*>(v_st + (2 * m + 1) * 128 + off);
    const uint32_t w0[2] = {b0.x, b0.y}, w1[2] = {b1.x, b1.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 x0 = fp8x2(w0[e >> 1], e & 1), x1 = fp8x2(w1[e >> 1], e & 1);
      f0[2 * e] = x0[0];
      f0[2 * e + 1] = x0[1];
      f1[2 * e] = x1[0];
      f1[2 * e + 1] = x1[1];
    }
  }
  if (vmul != 1.0f) {  // uniform
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f0[e] *= vmul;
      f1[e] *= vmul;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = f16x2_rne(f0[2 * e], f0[2 * e + 1]);
    hi[e] = f16x2_rne(f1[2 * e], f1[2 * e + 1]);
  }
  if (fp8) {
    // FP8 K: thread t widens 16 channels (piece t % 8) of key t / 8
    const int r = t >> 3, j = t & 7;
    const uint4 kb = *reinterpret_cast<const uint4*>(k_st + r * 128 + 16 * j);
    const uint32_t kw[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint4 o = make_uint4(bf16x2_exact(fp8x2(kw[2 * hh], false)), bf16x2_exact(fp8x2(kw[2 * hh], true)),
                                 bf16x2_exact(fp8x2(kw[2 * hh + 1], false)),
                                 bf16x2_exact(fp8x2(kw[2 * hh + 1], true)));
      const int cc = 2 * j + hh;
      *reinterpret_cast<uint4*>(kconv + 16 * (r * 16 + (cc ^ (r & 15)))) = o;
    }
  }
  // keys 2m, 2m + 1 are half (m & 1) of the 4-key piece m / 2
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int d0 = 8 * c + 2 * e, d1 = d0 + 1;
    *reinterpret_cast<uint32_t*>(vt + vt_piece(d0, m >> 1) + 4 * (m & 1)) =
        __builtin_amdgcn_perm(hi[e], lo[e], 0x05040100u);
    *reinterpret_cast<uint32_t*>(vt + vt_piece(d1, m >> 1) + 4 * (m & 1)) =
        __builtin_amdgcn_perm(hi[e], lo[e], 0x07060302u);
  }
}

template <int kPre>
__global__ __launch_bounds__(kXThreads) __attribute__((amdgpu_waves_per_eu(2))) void k_extend_attn(ExtendArgs a) {
  constexpr bool kPreFp8 = kPre == kPreFp8Rows;
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
  const int n_pre = (int)((P + kTile - 1) / kTile);
  const int n_tiles = n_pre + (int)((t_last + kTile) / kTile);  // chunk keys 0 .. t_last

  // Fused quantize-on-write of the chunk (the prefill path): this workgroup
  // encodes its own tokens' K/V blocks for its KV head into the NVFP4 pool; the
  // attention below reads the bf16 chunk, so the two do not depend on each other.
  if (a.write_chunk) {
    const int64_t n_blk = (t_last - t_first + 1) * 16;
    for (int64_t idx = t; idx < n_blk; idx += kXThreads)
      qenc::quantize_one<true>(a.qw, t_first + idx / 16, h, (int)((idx >> 3) & 1), (int)(idx & 7));
  }

  __shared__ __attribute__((aligned(16))) uint8_t k_ring[kStages][kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t v_ring[kStages][kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kTile * kHeadDim * 2];
  static_assert(kStages * 2 * kStageBytes + kTile * kHeadDim * 2 + kStageBytes <= 160 * 1024,
                "the workgroup's LDS fits a CU");
  __shared__ __attribute__((aligned(16))) uint8_t kconv[kPreFp8 ? kStageBytes : 16];
  const uint32_t k_ring_lds = (uint32_t)reinterpret_cast<uintptr_t>(&k_ring[0][0]);
  const uint32_t v_ring_lds = (uint32_t)reinterpret_cast<uintptr_t>(&v_ring[0][0]);

  // this lane's rows (one per row block): token, query head; rows past the
  // block's tokens or the chunk are computed but never stored
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
  uint4 qraw[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qraw[rb][s] = make_uint4(0u, 0u, 0u, 0u);
      if (valid[rb])
        qraw[rb][s] =
            *reinterpret_cast<const uint4*>(a.q + (tok[rb] * a.num_q_heads + qh[rb]) * kHeadDim + 32 * s + 8 * G);
    }
  bf16x8 qf[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 u = qraw[rb][s];
      u.x ^= a.q_sign;
      u.y ^= a.q_sign;
      u.z ^= a.q_sign;
      u.w ^= a.q_sign;
      // consume the loads here, so that their wait is not placed inside the
      // tile loop (where it would also drain the asynchronous copies)
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      qf[rb][s] = __builtin_bit_cast(bf16x8, u);
    }
  const float c2 = a.qk_scale_log2;  // >= 0: a negative scale is folded into the sign of Q

  f32x4 oacc[8][2];
#pragma unroll
  for (int d = 0; d < 8; ++d)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[d][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};
  // row sums of P on the matrix cores: an all-ones A operand times P^T gives each
  // row's sum in every element of the accumulator column
  f32x4 lacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                      (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};

  // prologue: tiles 0 and 1 in flight
  for (int i = 0; i < 2 && i < n_tiles; ++i)
    issue_tile(tile_of<kPre>(a, h, n_pre, i), Hkv, k_ring_lds + i * kStageBytes, v_ring_lds + i * kStageBytes,
               wave, lane);

  for (int i = 0; i < n_tiles; ++i) {
    const int st = i % kStages;
    const Tile x = tile_of<kPre>(a, h, n_pre, i);
    // this wave's copies of tile i have landed once only tile i+1's are pending
    if (i + 1 >= n_tiles)
      wait_dma<0>();
    else if (kPreFp8 && i + 1 < n_pre)
      wait_dma<2>();
    else
      wait_dma<4>();
    lds_barrier();  // every wave: tile i landed, tile i-1 fully consumed
    if (i + 2 < n_tiles) {
      const int s2 = (i + 2) % kStages;
      issue_tile(tile_of<kPre>(a, h, n_pre, i + 2), Hkv, k_ring_lds + s2 * kStageBytes,
                 v_ring_lds + s2 * kStageBytes, wave, lane);
    }
    if (!x.vtile) {
      convert_tile(x.fp8, t, k_ring[st], v_ring[st], vt, kconv, a.v_mul);
      lds_barrier();  // V^T (and widened K) of tile i complete
    }
    const uint8_t* vsrc = x.vtile ? v_ring[st] : vt;  // a V^T tile that arrived ready, or the converted one

    // ---- S^T = K Q^T ----
    const uint4* kt = reinterpret_cast<const uint4*>(x.fp8 ? kconv : k_ring[st]);
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sacc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, kt[(16 * kb + n) * 16 + ((4 * s + G) ^ n)]);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rb][s], sacc[kb][rb], 0, 0, 0);
      }

    // ---- mask: missing keys; chunk key j is visible to token i iff j <= i ----
    if (x.n_valid < kTile || (x.chunk && x.first + kTile - 1 > t_first)) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * kb + 4 * G + r;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            if (j >= x.n_valid || (x.chunk && x.first + j > tok[rb])) sacc[kb][rb][r] = -__builtin_inff();
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
        lacc[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) oacc[d][rb] *= alpha;
      }
    }
    // P^T operands of key half ks: k slots = keys 4G..4G+3 of block 2ks, then of
    // block 2ks + 1
    f16x8 pf[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float mu = m_ref[rb] == -__builtin_inff() ? 0.0f : m_ref[rb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pf[kb >> 1][rb][4 * (kb & 1) + r] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][r], c2, -mu));
        }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int dim = 16 * d + n;
        const f16x8 vf = __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(vsrc + vt_unit(dim, 4 * ks + G)));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          oacc[d][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[ks][rb], oacc[d][rb], 0, 0, 0);
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) lacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pf[ks][rb], lacc[rb], 0, 0, 0);
  }

  // ---- epilogue: O / l as bf16; lse in natural log ----
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = lacc[rb][0];  // the same row sum in every element
    if (!valid[rb]) continue;
    const float inv = a.out_mul / l;  // out_mul = 1 / v_mul, a power of two
    uint16_t* o = a.out + (tok[rb] * a.num_q_heads + qh[rb]) * kHeadDim;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const f32x4 v = oacc[d][rb] * inv;
      // channels 16 d + 4 G .. +3 of this row
      *reinterpret_cast<uint2*>(o + 16 * d + 4 * G) = make_uint2(bf16x2_rne(v[0], v[1]), bf16x2_rne(v[2], v[3]));
    }
    if (a.lse != nullptr && G == 0)
      a.lse[tok[rb] * a.num_q_heads + qh[rb]] = (m_ref[rb] + __builtin_log2f(l)) * 0.69314718055994531f;
  }
}

}  // namespace

int extend_tokens_per_block(int group) { return kXWaves * kXRows / group; }

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  if (a.chunk_len == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_token_blocks * (unsigned)a.num_kv_heads), block(kXThreads);
  if (a.pre_kind == kPreFp8Rows)
    hipLaunchKernelGGL(k_extend_attn<kPreFp8Rows>, grid, block, 0, stream, a);
  else if (a.pre_kind == kPreTiled)
    hipLaunchKernelGGL(k_extend_attn<kPreTiled>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(k_extend_attn<kPreBf16>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
