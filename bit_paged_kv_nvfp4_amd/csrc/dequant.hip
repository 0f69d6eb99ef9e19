// Extend-path dequantization of a cached NVFP4 prefix into a dense workspace
// (gfx950).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): for
// chunked prefill the cached prefix is dequantized into one workspace shared by
// the layers and attended together with the current chunk.
//
// One wave per (page, KV head, sequence), eight heads' waves to a workgroup. K:
// lane (G, n) reads channels 8n..8n+7 (4 code bytes) and the scale byte of
// tokens G, G+4, G+8, G+12; V: lane (n, G) reads its 16-byte chunk (channels
// 8n..8n+7 of tokens 4G..4G+3) and the four scale bytes of block n/2 for those
// tokens. With a power-of-two g the values E2M1(c) * E4M3(s) * g are exact in
// fp32 and in bf16 (at most 6 significant bits); with any other g the exact
// product has up to 30 significant bits, and every workspace dtype holds its
// nearest-even rounding (one rounding). An FP8 E4M3 workspace (the pages'
// choice) rounds each value once, from its exact value, in both cases.
#include "nvfp4kv.h"
#include "nvfp4kv_device.h"

namespace nvfp4kv {
namespace {


// A 16-byte load of pool bytes read once, marked non-temporal (measured: the
// 163840-token prefix 0.248 -> 0.244 ms into bf16; the same hint on the
// workspace stores made them 2.4x slower, so those stay plain).
__device__ __forceinline__ uint4 load_once(const uint8_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// x g rounded to odd in binary32, for an exact x: the nearest-even product hi,
// its exact error lo = x g - hi (one fma), and, when lo != 0 and the last
// significand bit of hi is even, the binary32 neighbour of hi on the side of
// x g. Rounding that value to nearest even in a format of at most 22
// significant bits (bf16 has 8, E4M3 at most 4) gives the nearest-even
// rounding of x g itself (Boldo and Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", 2008).
__device__ __forceinline__ float product_round_odd(float x, float g) {
#pragma clang fp contract(off)
  const float hi = x * g;
  const float lo = __builtin_fmaf(x, g, -hi);
  uint32_t u = __float_as_uint(hi);
  // same sign as hi: |x g| > |hi|, one step up in magnitude; else one down
  if (lo != 0.0f && !(u & 1u)) u += ((__float_as_uint(lo) ^ u) >> 31) ? 0xFFFFFFFFu : 1u;
  return __uint_as_float(u);
}

// Eight consecutive values of one output row, as one 16-byte store (bf16), two
// (f32) or one 8-byte store (FP8 E4M3). bf16: exact values carry at most 6
// significant bits, so the upper half of each f32 is its bf16 encoding and a
// byte permute packs two; other values (exact = false) are rounded to nearest
// even. FP8: the hardware conversion rounds to nearest even; clamping to +-448
// first (one med3) makes larger magnitudes saturate (a value above 448 rounds to
// 448 or, from 464 on, would overflow the format).
__device__ __forceinline__ void store8(void* base, size_t idx, const float (&v)[8], int dtype, bool exact = true) {
  if (dtype == NVFP4KV_FP8_E4M3) {
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(v[i], -448.0f, 448.0f);
    uint32_t p[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[4 * i], c[4 * i + 1], 0, false);
      p[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[4 * i + 2], c[4 * i + 3], lo, true);
    }
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + idx) = make_uint2(p[0], p[1]);
  } else if (dtype == NVFP4KV_BF16) {
    uint32_t p[4];
    if (exact) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = __builtin_amdgcn_perm(__float_as_uint(v[2 * i + 1]), __float_as_uint(v[2 * i]), 0x07060302u);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        p[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// With kExact (power-of-two g) x holds the exact values E2M1(c) E4M3(s) g, and
// they are stored as they are. Otherwise x holds the unscaled exact values
// E2M1(c) E4M3(s), and each is multiplied by g here with one rounding to the
// workspace dtype.
template <bool kExact>
__device__ __forceinline__ void scale_and_store8(void* base, size_t idx, const float (&x)[8], float g, int dtype) {
  if (kExact) {
    store8(base, idx, x, dtype, true);
    return;
  }
  float v[8];
  if (dtype == NVFP4KV_F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = x[e] * g;  // the one rounding to binary32
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = product_round_odd(x[e], g);
  }
  store8(base, idx, v, dtype, false);
}

// The V side of the NVFP4KV_F16_TILED workspace: key (row) r of KV head h sits
// in tile r / 64 at byte ((r / 64) H + h) 16384: 128 channel rows of 128 bytes,
// key k = r % 64 of channel d at byte d 128 + 16 u + 8 half + 2 pos with
// u = 4 (k / 32) + (k / 4) % 4, half = (k / 16) % 2, pos = k % 4. That is the
// order in which the extend attention's PV operands take the keys (unit u = 4 ks
// + G holds keys 32 ks + 4 G .. +3, then 32 ks + 16 + 4 G .. +3), so its tiles
// are copied into LDS as they are.
__device__ __forceinline__ size_t vt_offset(int64_t r, int h, int H, int d) {
  const int k = (int)(r & 63);
  return ((size_t)(r >> 6) * H + h) * 16384 + d * 128 + 16 * (4 * (k >> 5) + ((k >> 2) & 3)) + 8 * ((k >> 4) & 1) +
         2 * (k & 3);
}

// K rows of one (page, KV head) into the row-major workspace: store i writes
// tokens 4i .. 4i+3; lane (G, n) holds token 4i + G, channels 8n .. 8n+7 (4 code
// bytes; the scale byte of block n/2). Tokens at or past ntok are not written.
template <bool kExact>
__device__ __forceinline__ void dequant_k_page(const DequantArgs& a, const uint8_t* kslab, int64_t row0, int h,
                                               int ntok, int n, int G, int dt) {
  uint32_t kc[4], ks[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * i + G;
    kc[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(kslab + tok * 64 + 4 * n));
    ks[i] = kslab[kCodeBytes + tok * 8 + (n >> 1)];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * i + G;
    if (tok >= ntok) continue;
    const float sc = kExact ? e4m3_to_f32(ks[i]) * a.g : e4m3_to_f32(ks[i]);  // exact either way
    const f32x2 v0 = fp4x2_to_f32x2<0>(kc[i]), v1 = fp4x2_to_f32x2<1>(kc[i]);
    const f32x2 v2 = fp4x2_to_f32x2<2>(kc[i]), v3 = fp4x2_to_f32x2<3>(kc[i]);
    const float v[8] = {v0[0] * sc, v0[1] * sc, v1[0] * sc, v1[1] * sc, v2[0] * sc, v2[1] * sc, v3[0] * sc, v3[1] * sc};
    scale_and_store8<kExact>(a.k_out, ((size_t)(row0 + tok) * a.num_kv_heads + h) * kHeadDim + 8 * n, v, a.g, dt);
  }
}

// The V chunk of lane (n, G) of one slab: channels 8n .. 8n+7 of tokens 4G ..
// 4G+3 (block n/2), unscaled, as val[token 4G + i][channel 8n + e], and the four
// tokens' block scales.
__device__ __forceinline__ void load_v_chunk(const uint8_t* vslab, int lane, int n, int G, float (&val)[4][8],
                                             uint32_t& scales) {
  const uint4 vc = load_once(vslab + 16 * lane);
  scales = *reinterpret_cast<const uint32_t*>(vslab + kCodeBytes + (n >> 1) * 16 + 4 * G);
  const uint32_t vw[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // byte 0: channel 2w of tokens 0|2, byte 1: channel 2w of tokens 1|3,
    // bytes 2, 3: the same for channel 2w + 1
    const f32x2 c0 = fp4x2_to_f32x2<0>(vw[w]), c1 = fp4x2_to_f32x2<1>(vw[w]);
    const f32x2 c2 = fp4x2_to_f32x2<2>(vw[w]), c3 = fp4x2_to_f32x2<3>(vw[w]);
    val[0][2 * w] = c0[0];
    val[2][2 * w] = c0[1];
    val[1][2 * w] = c1[0];
    val[3][2 * w] = c1[1];
    val[0][2 * w + 1] = c2[0];
    val[2][2 * w + 1] = c2[1];
    val[1][2 * w + 1] = c3[0];
    val[3][2 * w + 1] = c3[1];
  }
}

// One workgroup of 8 waves per (page, sequence); wave w takes KV heads w, w + 8,
// ... of the page, so one workgroup writes whole workspace rows (all heads of
// its 16 tokens), and consecutive workgroups write consecutive rows. Measured
// on the 163840-token prefix (8 heads): one wave per (page, head) in head-major
// order took 220 us into bf16, this order 142 us; 4 waves with two heads each
// were 3% slower than 8.
template <bool kExact>
__global__ __launch_bounds__(512) void k_dequant(DequantArgs a) {
  const int pg = blockIdx.x;
  const int s = blockIdx.y;
  const int L = a.seq_lens[s];
  if (pg * kPage >= L) return;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int G = lane >> 4;
  const int64_t pid = a.page_table[(int64_t)s * a.pt_stride + pg];
  const int64_t row0 = a.row_offsets[s] + (int64_t)pg * kPage;
  const int H = a.num_kv_heads;
  const int dt = a.out_dtype;
  const int ntok = min(kPage, L - pg * kPage);

  for (int h = threadIdx.x >> 6; h < H; h += 8) {
    const uint8_t* kslab = a.pool + (pid * H + h) * (int64_t)(2 * kSlab);
    dequant_k_page<kExact>(a, kslab, row0, h, ntok, n, G, dt);
    float val[4][8];
    uint32_t vs;
    load_v_chunk(kslab + kSlab, lane, n, G, val, vs);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * G + i;
      if (tok >= ntok) continue;
      const float e4 = e4m3_to_f32((vs >> (8 * i)) & 0xFFu);
      const float sc = kExact ? e4 * a.g : e4;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = val[i][e] * sc;  // exact: at most 6 significant bits (times 2^k)
      scale_and_store8<kExact>(a.v_out, ((size_t)(row0 + tok) * H + h) * kHeadDim + 8 * n, v, a.g, dt);
    }
  }
}

// The unscaled V values val[i][e] of one lane's chunk times their block scales
// (exact), rounded once to f16: key 4G + i of channel 8n + e, zero where
// `valid` is clear for key i. The product is passed through an empty asm
// operand: left visible, a multiply followed by the f16 rounding is selected
// as one mixed fma with a +0 addend, which turns the product of a -0 code into
// +0.
template <bool kExact>
__device__ __forceinline__ float v_value(const float (&val)[4][8], uint32_t vs, int i, int e, float g, bool valid) {
  const float e4 = e4m3_to_f32((vs >> (8 * i)) & 0xFFu);
  float v = val[i][e] * (kExact ? e4 * g : e4);  // exact
  if (!kExact) v = product_round_odd(v, g);
  asm("" : "+v"(v));
  return valid ? v : 0.0f;
}

// The V^T tile of KV head h for the tile's (up to) four pages. kOwn (the
// sequence's first row a multiple of 64, so it owns its tiles): the whole 16 KB
// tile is written, keys past the sequence's end as zeros. Lane (n, G) takes
// chunk (n, G) of pages 2ks and 2ks + 1 of the tile, which is exactly unit
// u = 4ks + G (keys 32ks + 4G .. +3, then 32ks + 16 + 4G .. +3) of channel rows
// 8n .. 8n+7: one 16-byte store per channel, so every 128-byte channel row is
// written whole by one wave. Otherwise only the sequence's own values are
// stored, one at a time.
template <bool kExact, bool kOwn>
__device__ __forceinline__ void dequant_v_tile(const DequantArgs& a, const int64_t (&pid)[4], int npg, int rows,
                                               int64_t row_t, int h, int lane, int n, int G) {
  const int H = a.num_kv_heads;
#pragma unroll 1
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t x[2][8][2];  // [half][channel e]: keys 32 ks + 16 half + 4G .. +3 as 4 f16
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = 2 * ks + half;
      if (!kOwn && j >= npg) break;
      float val[4][8];
      uint32_t vs = 0;
      if (j < npg) {
        load_v_chunk(a.pool + (pid[j] * H + h) * (int64_t)(2 * kSlab) + kSlab, lane, n, G, val, vs);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) val[i][e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (kOwn) {
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = v_value<kExact>(val, vs, i, e, a.g, kPage * j + 4 * G + i < rows);
          x[half][e][0] = as_u32(f16x2{(_Float16)y[0], (_Float16)y[1]});
          x[half][e][1] = as_u32(f16x2{(_Float16)y[2], (_Float16)y[3]});
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = kPage * j + 4 * G + i;
            if (k < rows)
              *reinterpret_cast<_Float16*>(static_cast<uint8_t*>(a.v_out) + vt_offset(row_t + k, h, H, 8 * n + e)) =
                  (_Float16)v_value<kExact>(val, vs, i, e, a.g, true);
          }
        }
      }
    }
    if (kOwn) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const size_t off = vt_offset(row_t + 32 * ks + 4 * G, h, H, 8 * n + e);  // start of unit 4ks + G
        *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.v_out) + off) =
            make_uint4(x[0][e][0], x[0][e][1], x[1][e][0], x[1][e][1]);
      }
    }
  }
}

// The NVFP4KV_F16_TILED workspace (K as bf16 rows, V as f16 V^T tiles). One
// workgroup of 8 waves per (64-row tile, sequence), wave w taking KV heads w,
// w + 8, ...: the K rows of the tile's (up to) four pages as k_dequant writes
// them, and the head's V^T tile. (With a workgroup per page, four workgroups on
// different XCDs wrote into each 128-byte channel row of a tile, and the
// half-written 64-byte blocks doubled the V bytes that reached HBM.)
template <bool kExact>
__global__ __launch_bounds__(512) void k_dequant_tiled(DequantArgs a) {
  const int t = blockIdx.x;
  const int s = blockIdx.y;
  const int L = a.seq_lens[s];
  if (t * 64 >= L) return;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int G = lane >> 4;
  const int H = a.num_kv_heads;
  const int64_t first = a.row_offsets[s];
  const int rows = min(64, L - 64 * t);  // rows of this sequence in the tile
  const int npg = (rows + kPage - 1) / kPage;
  int64_t pid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pid[j] = j < npg ? a.page_table[(int64_t)s * a.pt_stride + 4 * t + j] : 0;
  const int64_t row_t = first + 64 * (int64_t)t;  // workspace row of the tile's first key

  for (int h = threadIdx.x >> 6; h < H; h += 8) {
    // this loop and the V one over ks stay rolled: unrolled, the kernel took 199
    // VGPRs (two waves per SIMD), rolled 116 (four)
#pragma unroll 1
    for (int j = 0; j < 4; ++j)
      if (j < npg)
        dequant_k_page<kExact>(a, a.pool + (pid[j] * H + h) * (int64_t)(2 * kSlab), row_t + kPage * j, h,
                               min(kPage, rows - kPage * j), n, G, NVFP4KV_BF16);
    if ((first & 63) == 0)
      dequant_v_tile<kExact, true>(a, pid, npg, rows, row_t, h, lane, n, G);
    else
      dequant_v_tile<kExact, false>(a, pid, npg, rows, row_t, h, lane, n, G);
  }
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  const int max_pages = (a.max_seq_len + kPage - 1) / kPage;
  if (a.n_seqs == 0 || max_pages == 0) return hipSuccess;
  if (a.out_dtype == NVFP4KV_F16_TILED) {
    const dim3 grid((max_pages + 3) / 4, a.n_seqs);
    if (a.g_pow2)
      hipLaunchKernelGGL((k_dequant_tiled<true>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((k_dequant_tiled<false>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid(max_pages, a.n_seqs);
  if (a.g_pow2)
    hipLaunchKernelGGL((k_dequant<true>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((k_dequant<false>), grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
