// Extend-path dequantization of a cached NVFP4 prefix into a dense workspace
// (gfx950).
//
// Page "SGLang stores KV cache in 4 bits ..." (section Interpretation): for
// chunked prefill the cached prefix is dequantized into one workspace shared by
// the layers and attended together with the current chunk.
//
// One wave per (page, KV head, sequence). K: lane (t, G) reads channels
// 32G..32G+31 of token t (16 code bytes) and their two scale bytes; V: lane
// (n, G) reads its 16-byte chunk (channels 8n..8n+7 of tokens 4G..4G+3) and the
// four scale bytes of block n/2 for those tokens. Values E2M1(c) * E4M3(s) * g
// are exact in fp32 and in bf16 (at most 6 significant bits); an FP8 E4M3
// workspace (the pages' choice) rounds each of them once, from its exact value.
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

// Eight consecutive values of one output row, as one 16-byte store (bf16), two
// (f32) or one 8-byte store (FP8 E4M3).
__device__ __forceinline__ void store8(void* base, size_t idx, const float (&v)[8], int dtype) {
  if (dtype == NVFP4KV_FP8_E4M3) {
    uint32_t p[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      p[i] = f32_to_e4m3(v[4 * i]) | (f32_to_e4m3(v[4 * i + 1]) << 8) | (f32_to_e4m3(v[4 * i + 2]) << 16) |
             (f32_to_e4m3(v[4 * i + 3]) << 24);
    *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + idx) = make_uint2(p[0], p[1]);
  } else if (dtype == NVFP4KV_BF16) {
    uint32_t p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[i] = (uint32_t)f32_to_bf16_bits(v[2 * i]) | ((uint32_t)f32_to_bf16_bits(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = make_uint4(p[0], p[1], p[2], p[3]);
  } else {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__global__ __launch_bounds__(64) void k_dequant(DequantArgs a) {
  const int pg = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int L = a.seq_lens[s];
  if (pg * kPage >= L) return;
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int G = lane >> 4;
  const int64_t pid = a.page_table[(int64_t)s * a.pt_stride + pg];
  const uint8_t* kslab = a.pool + (pid * a.num_kv_heads + h) * (int64_t)(2 * kSlab);
  const uint8_t* vslab = kslab + kSlab;
  const int64_t row0 = a.row_offsets[s] + (int64_t)pg * kPage;
  const int H = a.num_kv_heads;
  const int dt = a.out_dtype;

  // ---- K: token n, channels 32G..32G+31 (four runs of 8) ----
  if (pg * kPage + n < L) {
    const uint4 kc = load_once(kslab + n * 64 + G * 16);
    const uint32_t ks = *reinterpret_cast<const uint16_t*>(kslab + kCodeBytes + n * 8 + G * 2);
    const float sc0 = e4m3_to_f32(ks & 0xFFu) * a.g;
    const float sc1 = e4m3_to_f32(ks >> 8) * a.g;
    const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
    const size_t base = ((size_t)(row0 + n) * H + h) * kHeadDim + 32 * G;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = w < 2 ? sc0 : sc1;
      const f32x2 v0 = fp4x2_to_f32x2<0>(kw[w]), v1 = fp4x2_to_f32x2<1>(kw[w]);
      const f32x2 v2 = fp4x2_to_f32x2<2>(kw[w]), v3 = fp4x2_to_f32x2<3>(kw[w]);
      const float v[8] = {v0[0] * sc, v0[1] * sc, v1[0] * sc, v1[1] * sc, v2[0] * sc, v2[1] * sc, v3[0] * sc, v3[1] * sc};
      store8(a.k_out, base + 8 * w, v, dt);
    }
  }

  // ---- V: chunk `lane` = channels 8n..8n+7 of tokens 4G..4G+3 (block n/2) ----
  {
    const uint4 vc = load_once(vslab + 16 * lane);
    const uint32_t vs = *reinterpret_cast<const uint32_t*>(vslab + kCodeBytes + (n >> 1) * 16 + 4 * G);
    const uint32_t vw[4] = {vc.x, vc.y, vc.z, vc.w};
    float val[4][8];  // [token 4G + i][channel 8n + e], unscaled
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * G + i;
      if (pg * kPage + tok >= L) continue;
      const float sc = e4m3_to_f32((vs >> (8 * i)) & 0xFFu) * a.g;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = val[i][e] * sc;
      store8(a.v_out, ((size_t)(row0 + tok) * H + h) * kHeadDim + 8 * n, v, dt);
    }
  }
}

}  // namespace

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  const int max_pages = (a.max_seq_len + kPage - 1) / kPage;
  if (a.n_seqs == 0 || max_pages == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant, dim3(max_pages, a.num_kv_heads, a.n_seqs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4kv
