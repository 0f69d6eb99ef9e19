// Host side of the C ABI declared in include/nvfp4kv.h: argument validation (no
// HIP call before it passes) and kernel launches.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "nvfp4kv.h"
#include "nvfp4kv_device.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The NVFP4 global scale g: any finite float in [2^-64, 2^64]. Every dequantized
// value E2M1 * E4M3 * g then lies inside the normal range of fp32 and bf16.
bool valid_global_scale(float g) {
  return isfinite(g) && g >= 0x1p-64f && g <= 0x1p64f;
}

bool is_pow2(float g) {
  int e;
  return isfinite(g) && g > 0.0f && frexpf(g, &e) == 0.5f;
}

// The FP8 baseline's per-tensor scales: powers of two in [2^-64, 2^64], so that
// x / s is exact and the per-value encode is one rounding.
bool valid_pow2_scale(float s) { return valid_global_scale(s) && is_pow2(s); }

int32_t check_pool(const nvfp4kv_pool* pool) {
  if (!pool || !pool->data) return NVFP4KV_ERR_NULL;
  if (pool->num_pages < 1 || pool->num_kv_heads < 1) return NVFP4KV_ERR_SHAPE;
  if (pool->num_pages > ((int64_t)1 << 40) / ((int64_t)pool->num_kv_heads * 2 * NVFP4KV_SLAB_BYTES))
    return NVFP4KV_ERR_SHAPE;
  if (!aligned16(pool->data)) return NVFP4KV_ERR_ALIGN;
  if (!valid_global_scale(pool->global_scale)) return NVFP4KV_ERR_VALUE;
  return NVFP4KV_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? NVFP4KV_OK : NVFP4KV_ERR_HIP; }

int32_t check_fp8_pool(const fp8kv_pool* pool) {
  if (!pool || !pool->data) return NVFP4KV_ERR_NULL;
  if (pool->num_pages < 1 || pool->num_kv_heads < 1) return NVFP4KV_ERR_SHAPE;
  if (pool->num_pages > ((int64_t)1 << 40) / ((int64_t)pool->num_kv_heads * 2 * FP8KV_SLAB_BYTES))
    return NVFP4KV_ERR_SHAPE;
  if (!aligned16(pool->data)) return NVFP4KV_ERR_ALIGN;
  if (!valid_pow2_scale(pool->k_scale) || !valid_pow2_scale(pool->v_scale)) return NVFP4KV_ERR_VALUE;
  return NVFP4KV_OK;
}

// What the kernels need of either pool (validated by check_pool / check_fp8_pool).
struct PoolInfo {
  void* data;
  int32_t num_kv_heads;
  float k_mul;  // NVFP4: g; FP8: k_scale
  float v_mul;  // NVFP4: g; FP8: v_scale
  bool fp8;
};
PoolInfo info_of(const nvfp4kv_pool* p) {
  return PoolInfo{p->data, p->num_kv_heads, p->global_scale, p->global_scale, false};
}
PoolInfo info_of(const fp8kv_pool* p) { return PoolInfo{p->data, p->num_kv_heads, p->k_scale, p->v_scale, true}; }

int32_t quantize_into(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                      int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens, const PoolInfo& pool,
                      void* stream) {
  if (src_dtype != NVFP4KV_F32 && src_dtype != NVFP4KV_BF16) return NVFP4KV_ERR_DTYPE;
  if (num_tokens < 0 || token_stride < 0 || head_stride < 0) return NVFP4KV_ERR_SHAPE;
  if (num_tokens == 0) return NVFP4KV_OK;
  if (!k_src || !v_src || !slot_mapping) return NVFP4KV_ERR_NULL;
  if (num_tokens > ((int64_t)1 << 31) * 256 / ((int64_t)pool.num_kv_heads * 16)) return NVFP4KV_ERR_SHAPE;
  const int64_t vec = src_dtype == NVFP4KV_F32 ? 4 : 8;  // elements per 16 bytes
  if (!aligned16(k_src) || !aligned16(v_src) || token_stride % vec || head_stride % vec ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 3u))
    return NVFP4KV_ERR_ALIGN;
  nvfp4kv::QuantizeArgs a;
  a.k = k_src;
  a.v = v_src;
  a.bf16 = src_dtype == NVFP4KV_BF16;
  a.token_stride = token_stride;
  a.head_stride = head_stride;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  a.pool = static_cast<uint8_t*>(pool.data);
  a.num_kv_heads = pool.num_kv_heads;
  a.g = pool.k_mul;
  a.g_pow2 = is_pow2(pool.k_mul);
  a.fp8 = pool.fp8;
  a.inv_k_scale = 1.0f / pool.k_mul;  // FP8 scales are powers of two: exact
  a.inv_v_scale = 1.0f / pool.v_mul;
  return hip_status(nvfp4kv::launch_quantize(a, static_cast<hipStream_t>(stream)));
}

// Workgroups of the persistent decode grid: the resident count, but at most one
// per kMinGridPages pages of the largest cache the call can hold (batch x KV heads
// x pages of max_seq_len), so that a small batch does not launch a thousand
// workgroups with nothing to read. The kernel's result does not depend on it.
constexpr int64_t kMinGridPages = 8;
int32_t decode_grid(int num_cus, bool fp8, int32_t batch, int32_t num_kv_heads, int32_t max_seq_len) {
  const int64_t resident = nvfp4kv::decode_resident_workgroups(num_cus, fp8);
  const int64_t pages = (int64_t)batch * num_kv_heads * ((max_seq_len + NVFP4KV_PAGE_SIZE - 1) / NVFP4KV_PAGE_SIZE);
  const int64_t want = (pages + kMinGridPages - 1) / kMinGridPages;
  return (int32_t)(want < 1 ? 1 : (want < resident ? want : resident));
}

int32_t default_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len, int32_t num_cus, bool fp8) {
  if (batch < 1 || num_kv_heads < 1 || max_seq_len < 1) return 1;
  if (num_cus <= 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    num_cus = cus;
  }
  const int64_t pages = (max_seq_len + NVFP4KV_PAGE_SIZE - 1) / NVFP4KV_PAGE_SIZE;
  const int64_t segments = (int64_t)batch * num_kv_heads;
  // Splits are the grain at which the persistent workgroups' page windows are
  // cut: about 16 splits per window keeps the windows within about 6% of each
  // other. Consecutive splits in one window share one state, so more splits do
  // not mean more partial-state writes. At least 4 pages per split.
  const int64_t windows = decode_grid(num_cus, fp8, batch, num_kv_heads, max_seq_len);
  int64_t s = (16 * windows + segments - 1) / segments;
  const int64_t max_by_pages = pages / 4 > 1 ? pages / 4 : 1;
  if (s > max_by_pages) s = max_by_pages;
  if (s > NVFP4KV_MAX_SPLITS) s = NVFP4KV_MAX_SPLITS;
  if (s < 1) s = 1;
  return (int32_t)s;
}

}  // namespace

extern "C" {

int64_t nvfp4kv_pool_bytes(int64_t num_pages, int32_t num_kv_heads) {
  if (num_pages < 0 || num_kv_heads < 0) return 0;
  return num_pages * num_kv_heads * 2 * (int64_t)NVFP4KV_SLAB_BYTES;
}

const char* nvfp4kv_status_string(int32_t status) {
  switch (status) {
    case NVFP4KV_OK: return "ok";
    case NVFP4KV_ERR_NULL: return "a required pointer is NULL";
    case NVFP4KV_ERR_SHAPE: return "a size, count or stride is out of range";
    case NVFP4KV_ERR_ALIGN: return "a pointer or stride is not 16-byte aligned";
    case NVFP4KV_ERR_DTYPE: return "unsupported dtype";
    case NVFP4KV_ERR_WORKSPACE: return "workspace too small";
    case NVFP4KV_ERR_VALUE: return "a float argument is out of its allowed set";
    case NVFP4KV_ERR_HIP: return "a HIP runtime call failed";
    case NVFP4KV_ERR_SCRATCH:
      return "the call needs more split-state memory than the library's fixed scratch buffer holds";
    default: return "unknown status";
  }
}

int32_t nvfp4kv_version(void) { return 2; }

int32_t nvfp4kv_check_page_table(const int32_t* page_table, int64_t page_table_stride, const int32_t* seq_lens,
                                 int32_t batch, int32_t max_seq_len, int64_t num_pages, uint8_t* seen,
                                 int64_t* bad_index) {
  if (batch < 0 || page_table_stride < 1 || max_seq_len < 0 || num_pages < 1) return NVFP4KV_ERR_SHAPE;
  if (batch == 0) return NVFP4KV_OK;
  if (!page_table || !seq_lens) return NVFP4KV_ERR_NULL;
  if (seen) memset(seen, 0, (size_t)num_pages);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 0 || L > max_seq_len || L > page_table_stride * NVFP4KV_PAGE_SIZE) {
      if (bad_index) *bad_index = b;
      return NVFP4KV_ERR_SHAPE;
    }
    const int64_t pages = (L + NVFP4KV_PAGE_SIZE - 1) / NVFP4KV_PAGE_SIZE;
    for (int64_t p = 0; p < pages; ++p) {
      const int64_t id = page_table[b * page_table_stride + p];
      if (id < 0 || id >= num_pages || (seen && seen[id])) {
        if (bad_index) *bad_index = b * page_table_stride + p;
        return NVFP4KV_ERR_VALUE;
      }
      if (seen) seen[id] = 1;
    }
  }
  return NVFP4KV_OK;
}

int32_t nvfp4_kv_quantize(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                          int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens,
                          const nvfp4kv_pool* pool, void* stream) {
  if (int32_t e = check_pool(pool)) return e;
  return quantize_into(k_src, v_src, src_dtype, token_stride, head_stride, slot_mapping, num_tokens, info_of(pool),
                       stream);
}

size_t nvfp4_kv_amax_workspace_bytes(void) { return (size_t)nvfp4kv::kAmaxBlocks * 2 * sizeof(float); }

int32_t nvfp4_kv_amax(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                      int64_t head_stride, int64_t num_tokens, int32_t num_kv_heads, float* amax_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (src_dtype != NVFP4KV_F32 && src_dtype != NVFP4KV_BF16) return NVFP4KV_ERR_DTYPE;
  if (num_tokens < 0 || token_stride < 0 || head_stride < 0 || num_kv_heads < 1) return NVFP4KV_ERR_SHAPE;
  if (num_tokens > ((int64_t)1 << 40) / ((int64_t)num_kv_heads * 128)) return NVFP4KV_ERR_SHAPE;
  if (!amax_out || !workspace || (num_tokens > 0 && (!k_src || !v_src))) return NVFP4KV_ERR_NULL;
  if (workspace_bytes < nvfp4_kv_amax_workspace_bytes()) return NVFP4KV_ERR_WORKSPACE;
  const int64_t vec = src_dtype == NVFP4KV_F32 ? 4 : 8;
  if ((num_tokens > 0 && (!aligned16(k_src) || !aligned16(v_src))) || token_stride % vec || head_stride % vec ||
      !aligned16(workspace) || (reinterpret_cast<uintptr_t>(amax_out) & 3u))
    return NVFP4KV_ERR_ALIGN;
  nvfp4kv::AmaxArgs a;
  a.k = k_src;
  a.v = v_src;
  a.bf16 = src_dtype == NVFP4KV_BF16;
  a.token_stride = token_stride;
  a.head_stride = head_stride;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.partial = static_cast<float*>(workspace);
  a.out = amax_out;
  return hip_status(nvfp4kv::launch_amax(a, static_cast<hipStream_t>(stream)));
}

float nvfp4kv_global_scale_tight_for_amax(float amax) {
  if (!(amax >= 0.0f) || !isfinite(amax)) return 0.0f;
  if (amax == 0.0f) return 1.0f;
  // the smallest binary32 g with amax <= 2688 g (an exact comparison in double:
  // 2688 g has at most 29 significant bits)
  float g = (float)((double)amax / 2688.0);
  while (!((double)amax <= 2688.0 * (double)g)) g = nextafterf(g, INFINITY);
  while (g > 0.0f && (double)amax <= 2688.0 * (double)nextafterf(g, 0.0f)) g = nextafterf(g, 0.0f);
  return valid_global_scale(g) ? g : 0.0f;
}

float nvfp4kv_global_scale_for_amax(float amax) {
  if (!(amax >= 0.0f) || !isfinite(amax)) return 0.0f;
  if (amax == 0.0f) return 1.0f;
  double g = 1.0;
  while ((double)amax / (6.0 * g) > 448.0) g *= 2.0;
  while ((double)amax / (6.0 * (g / 2.0)) <= 448.0) g /= 2.0;
  const float gf = (float)g;
  return valid_global_scale(gf) ? gf : 0.0f;
}

int64_t nvfp4kv_tiled_v_bytes(int64_t rows, int32_t num_kv_heads) {
  if (rows < 0 || num_kv_heads < 0) return 0;
  return (rows + 63) / 64 * num_kv_heads * (int64_t)(64 * NVFP4KV_HEAD_DIM * 2);
}

int64_t fp8kv_pool_bytes(int64_t num_pages, int32_t num_kv_heads) {
  if (num_pages < 0 || num_kv_heads < 0) return 0;
  return num_pages * num_kv_heads * 2 * (int64_t)FP8KV_SLAB_BYTES;
}

int32_t fp8_kv_quantize(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                        int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens, const fp8kv_pool* pool,
                        void* stream) {
  if (int32_t e = check_fp8_pool(pool)) return e;
  return quantize_into(k_src, v_src, src_dtype, token_stride, head_stride, slot_mapping, num_tokens, info_of(pool),
                       stream);
}

int32_t nvfp4_paged_decode_attn_default_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                               int32_t num_cus) {
  return default_splits(batch, num_kv_heads, max_seq_len, num_cus, false);
}

int32_t fp8_paged_decode_attn_default_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                             int32_t num_cus) {
  return default_splits(batch, num_kv_heads, max_seq_len, num_cus, true);
}

size_t nvfp4_paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_splits) {
  if (batch < 0 || num_q_heads < 1 || num_splits < 1 || num_splits > NVFP4KV_MAX_SPLITS) return 0;
  const size_t units = (size_t)batch * num_q_heads * num_splits;
  const size_t o_bytes = units * NVFP4KV_HEAD_DIM * sizeof(float);
  const size_t ml_bytes = units * 2 * sizeof(float);
  return o_bytes + ((ml_bytes + 255) & ~(size_t)255);
}

}  // extern "C"

namespace {

bool query_cus(int* cus) {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess &&
         hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && *cus > 0;
}

// Sizes the persistent grid of the decode kernel from the current device (the
// last step before a launch: every argument check has run by then).
int32_t finish_decode(nvfp4kv::DecodeArgs& a) {
  if (a.num_workgroups > 0) return NVFP4KV_OK;
  int cus = 0;
  if (!query_cus(&cus)) return NVFP4KV_ERR_HIP;
  a.num_workgroups = decode_grid(cus, a.fp8 != 0, a.batch, a.num_kv_heads, a.max_seq_len);
  return NVFP4KV_OK;
}

// Shared validation of the decode phases; fills `a` (without out/lse).
int32_t prepare_decode(const void* q, const int32_t* page_table, int64_t page_table_stride, const int32_t* seq_lens,
                       int32_t batch, int32_t num_q_heads, int32_t max_seq_len, const PoolInfo& pool,
                       float sm_scale, int32_t* num_splits, void* workspace, size_t workspace_bytes,
                       nvfp4kv::DecodeArgs& a) {
  if (batch < 0 || num_q_heads < 1 || max_seq_len < 0 || page_table_stride < 1) return NVFP4KV_ERR_SHAPE;
  const int32_t hkv = pool.num_kv_heads;
  if (num_q_heads % hkv != 0) return NVFP4KV_ERR_SHAPE;
  const int32_t group = num_q_heads / hkv;
  if (group < 1 || group > NVFP4KV_MAX_GROUP) return NVFP4KV_ERR_SHAPE;
  if ((int64_t)max_seq_len > page_table_stride * NVFP4KV_PAGE_SIZE) return NVFP4KV_ERR_SHAPE;
  if (*num_splits < 0 || *num_splits > NVFP4KV_MAX_SPLITS) return NVFP4KV_ERR_SHAPE;
  if (!isfinite(sm_scale)) return NVFP4KV_ERR_VALUE;
  if (batch == 0) return NVFP4KV_OK;
  if (!q || !page_table || !seq_lens || !workspace) return NVFP4KV_ERR_NULL;
  if (!aligned16(q) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(page_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return NVFP4KV_ERR_ALIGN;
  // the device's CU count sizes the persistent grid (finish_decode) and the
  // default split count; with num_splits given, no HIP call happens here
  int cus = 0;
  if (*num_splits == 0) {
    if (!query_cus(&cus)) return NVFP4KV_ERR_HIP;
    *num_splits = default_splits(batch, hkv, max_seq_len, cus, pool.fp8);
  }
  const size_t need = nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, *num_splits);
  if (need == 0 || workspace_bytes < need) return NVFP4KV_ERR_WORKSPACE;
  a.q = static_cast<const uint16_t*>(q);
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = hkv;
  a.group = group;
  a.max_seq_len = max_seq_len;
  a.pool = static_cast<const uint8_t*>(pool.data);
  a.qk_scale_log2 = (float)((double)sm_scale * 1.4426950408889634 * (double)pool.k_mul);
  a.v_scale = pool.v_mul;
  a.fp8 = pool.fp8;
  a.num_splits = *num_splits;
  a.num_workgroups = cus > 0 ? decode_grid(cus, pool.fp8, batch, hkv, max_seq_len) : 0;  // 0: finish_decode sets it
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = a.part_o + (size_t)batch * num_q_heads * *num_splits * NVFP4KV_HEAD_DIM;
  a.write_new = 0;
  a.nw = nvfp4kv::QuantizeArgs{};
  a.out = nullptr;
  a.out_bf16 = 0;
  a.lse = nullptr;
  return NVFP4KV_OK;
}

int32_t prepare_combine(const void* workspace, size_t workspace_bytes, int32_t batch, int32_t num_q_heads,
                        int32_t num_splits, void* out, int32_t out_dtype, float* lse, nvfp4kv::DecodeArgs& a) {
  if (out_dtype != NVFP4KV_F32 && out_dtype != NVFP4KV_BF16) return NVFP4KV_ERR_DTYPE;
  if (batch < 0 || num_q_heads < 1 || num_splits < 1 || num_splits > NVFP4KV_MAX_SPLITS) return NVFP4KV_ERR_SHAPE;
  if ((int64_t)batch * num_q_heads > 0x7FFFFFFF) return NVFP4KV_ERR_SHAPE;
  if (batch == 0) return NVFP4KV_OK;
  if (!workspace || !out) return NVFP4KV_ERR_NULL;
  if (!aligned16(workspace) || !aligned16(out) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return NVFP4KV_ERR_ALIGN;
  const size_t need = nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, num_splits);
  if (need == 0 || workspace_bytes < need) return NVFP4KV_ERR_WORKSPACE;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_splits = num_splits;
  a.part_o = static_cast<float*>(const_cast<void*>(workspace));
  a.part_ml = a.part_o + (size_t)batch * num_q_heads * num_splits * NVFP4KV_HEAD_DIM;
  a.out = out;
  a.out_bf16 = out_dtype == NVFP4KV_BF16;
  a.lse = lse;
  return NVFP4KV_OK;
}


int32_t decode_partial(const void* q, const int32_t* page_table, int64_t page_table_stride, const int32_t* seq_lens,
                       int32_t batch, int32_t num_q_heads, int32_t max_seq_len, const PoolInfo& pool, float sm_scale,
                       int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_splits < 1) return NVFP4KV_ERR_SHAPE;  // the caller sizes the workspace for a known count
  nvfp4kv::DecodeArgs a;
  if (int32_t e = prepare_decode(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, pool,
                                 sm_scale, &num_splits, workspace, workspace_bytes, a))
    return e;
  if (batch == 0) return NVFP4KV_OK;
  if (int32_t e = finish_decode(a)) return e;
  return hip_status(nvfp4kv::launch_decode_partial(a, static_cast<hipStream_t>(stream)));
}

// The newest token's K/V rows of each sequence, for the decode launches that
// write them into the pool themselves.
struct NewRows {
  const void* k;
  const void* v;
  int32_t dtype;
  int64_t token_stride;
  int64_t head_stride;
};

// Validates the new rows (as quantize_into does its sources) and points a.nw at
// them; batch rows, one per sequence.
int32_t prepare_new_rows(const NewRows& n, int32_t batch, const PoolInfo& pool, nvfp4kv::DecodeArgs& a) {
  if (n.dtype != NVFP4KV_F32 && n.dtype != NVFP4KV_BF16) return NVFP4KV_ERR_DTYPE;
  if (n.token_stride < 0 || n.head_stride < 0) return NVFP4KV_ERR_SHAPE;
  if (batch == 0) return NVFP4KV_OK;
  if (!n.k || !n.v) return NVFP4KV_ERR_NULL;
  const int64_t vec = n.dtype == NVFP4KV_F32 ? 4 : 8;
  if (!aligned16(n.k) || !aligned16(n.v) || n.token_stride % vec || n.head_stride % vec) return NVFP4KV_ERR_ALIGN;
  a.write_new = 1;
  a.nw.k = n.k;
  a.nw.v = n.v;
  a.nw.bf16 = n.dtype == NVFP4KV_BF16;
  a.nw.token_stride = n.token_stride;
  a.nw.head_stride = n.head_stride;
  a.nw.slots = nullptr;
  a.nw.num_tokens = batch;
  a.nw.pool = static_cast<uint8_t*>(pool.data);
  a.nw.num_kv_heads = pool.num_kv_heads;
  a.nw.g = pool.k_mul;
  a.nw.g_pow2 = is_pow2(pool.k_mul);
  a.nw.fp8 = pool.fp8;
  a.nw.inv_k_scale = 1.0f / pool.k_mul;  // powers of two: exact
  a.nw.inv_v_scale = 1.0f / pool.v_mul;
  return NVFP4KV_OK;
}

int32_t decode_full(const void* q, const int32_t* page_table, int64_t page_table_stride, const int32_t* seq_lens,
                    int32_t batch, int32_t num_q_heads, int32_t max_seq_len, const PoolInfo& pool, float sm_scale,
                    int32_t num_splits, void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                    float* lse, void* stream, const NewRows* new_rows = nullptr) {
  nvfp4kv::DecodeArgs a;
  if (out_dtype != NVFP4KV_F32 && out_dtype != NVFP4KV_BF16) return NVFP4KV_ERR_DTYPE;
  if (int32_t e = prepare_decode(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, pool,
                                 sm_scale, &num_splits, workspace, workspace_bytes, a))
    return e;
  if (new_rows)
    if (int32_t e = prepare_new_rows(*new_rows, batch, pool, a)) return e;
  // the fused step without `out` stops after phase 1 (states in the workspace)
  const bool phase1_only = new_rows && !out;
  if (phase1_only && lse) return NVFP4KV_ERR_NULL;
  if (batch == 0) return NVFP4KV_OK;
  nvfp4kv::DecodeArgs c;
  if (!phase1_only)
    if (int32_t e = prepare_combine(workspace, workspace_bytes, batch, num_q_heads, num_splits, out, out_dtype, lse, c))
      return e;
  if (int32_t e = finish_decode(a)) return e;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // The decode kernel writes the new rows itself only for a power-of-two global
  // scale (the FP8 baseline's scales are powers of two); otherwise a launch of
  // its own writes them first, with the same bytes.
  if (a.write_new && !a.nw.fp8 && !a.nw.g_pow2) {
    if (int32_t e = hip_status(nvfp4kv::launch_write_newest(a, st))) return e;
    a.write_new = 0;
  }
  if (int32_t e = hip_status(nvfp4kv::launch_decode_partial(a, st))) return e;
  if (phase1_only) return NVFP4KV_OK;
  return hip_status(nvfp4kv::launch_decode_combine(c, st));
}

}  // namespace

extern "C" {

int32_t nvfp4_paged_decode_attn_partial(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                        int32_t max_seq_len, const nvfp4kv_pool* pool, float sm_scale,
                                        int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t e = check_pool(pool)) return e;
  return decode_partial(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, info_of(pool),
                        sm_scale, num_splits, workspace, workspace_bytes, stream);
}

int32_t nvfp4_paged_decode_attn(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                                const nvfp4kv_pool* pool, float sm_scale, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* out, int32_t out_dtype, float* lse, void* stream) {
  if (int32_t e = check_pool(pool)) return e;
  return decode_full(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, info_of(pool),
                     sm_scale, num_splits, workspace, workspace_bytes, out, out_dtype, lse, stream);
}

int32_t fp8_paged_decode_attn_partial(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                      int32_t max_seq_len, const fp8kv_pool* pool, float sm_scale,
                                      int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t e = check_fp8_pool(pool)) return e;
  return decode_partial(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, info_of(pool),
                        sm_scale, num_splits, workspace, workspace_bytes, stream);
}

int32_t fp8_paged_decode_attn(const void* q, const int32_t* page_table, int64_t page_table_stride,
                              const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                              const fp8kv_pool* pool, float sm_scale, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, void* out, int32_t out_dtype, float* lse, void* stream) {
  if (int32_t e = check_fp8_pool(pool)) return e;
  return decode_full(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, info_of(pool),
                     sm_scale, num_splits, workspace, workspace_bytes, out, out_dtype, lse, stream);
}

int32_t nvfp4_paged_decode_attn_append(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                                       int64_t new_token_stride, int64_t new_head_stride, const int32_t* page_table,
                                       int64_t page_table_stride, const int32_t* seq_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t max_seq_len, const nvfp4kv_pool* pool,
                                       float sm_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                                       void* out, int32_t out_dtype, float* lse, void* stream) {
  if (int32_t e = check_pool(pool)) return e;
  const NewRows n{k_new, v_new, new_dtype, new_token_stride, new_head_stride};
  return decode_full(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, info_of(pool),
                     sm_scale, num_splits, workspace, workspace_bytes, out, out_dtype, lse, stream, &n);
}

int32_t fp8_paged_decode_attn_append(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                                     int64_t new_token_stride, int64_t new_head_stride, const int32_t* page_table,
                                     int64_t page_table_stride, const int32_t* seq_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t max_seq_len, const fp8kv_pool* pool, float sm_scale,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes, void* out,
                                     int32_t out_dtype, float* lse, void* stream) {
  if (int32_t e = check_fp8_pool(pool)) return e;
  const NewRows n{k_new, v_new, new_dtype, new_token_stride, new_head_stride};
  return decode_full(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len, info_of(pool),
                     sm_scale, num_splits, workspace, workspace_bytes, out, out_dtype, lse, stream, &n);
}

int32_t nvfp4_decode_combine(const void* workspace, size_t workspace_bytes, int32_t batch, int32_t num_q_heads,
                             int32_t num_splits, void* out, int32_t out_dtype, float* lse, void* stream) {
  nvfp4kv::DecodeArgs a;
  if (int32_t e = prepare_combine(workspace, workspace_bytes, batch, num_q_heads, num_splits, out, out_dtype, lse, a))
    return e;
  if (batch == 0) return NVFP4KV_OK;
  return hip_status(nvfp4kv::launch_decode_combine(a, static_cast<hipStream_t>(stream)));
}


int32_t nvfp4_kv_dequant_workspace(const nvfp4kv_pool* pool, const int32_t* page_table, int64_t page_table_stride,
                                   const int32_t* seq_lens, const int64_t* row_offsets, int32_t n_seqs,
                                   int32_t max_seq_len, void* k_out, void* v_out, int32_t out_dtype, void* stream) {
  if (int32_t e = check_pool(pool)) return e;
  if (out_dtype != NVFP4KV_F32 && out_dtype != NVFP4KV_BF16 && out_dtype != NVFP4KV_FP8_E4M3 &&
      out_dtype != NVFP4KV_F16_TILED)
    return NVFP4KV_ERR_DTYPE;
  // f16 holds every dequantized value (at most 2688 g) only for g <= 16
  if (out_dtype == NVFP4KV_F16_TILED && !(pool->global_scale <= 16.0f)) return NVFP4KV_ERR_VALUE;
  if (n_seqs < 0 || max_seq_len < 0 || page_table_stride < 1) return NVFP4KV_ERR_SHAPE;
  if ((int64_t)max_seq_len > page_table_stride * NVFP4KV_PAGE_SIZE) return NVFP4KV_ERR_SHAPE;
  if (n_seqs > 65535 || pool->num_kv_heads > 65535) return NVFP4KV_ERR_SHAPE;
  if (n_seqs == 0 || max_seq_len == 0) return NVFP4KV_OK;
  if (!page_table || !seq_lens || !row_offsets || !k_out || !v_out) return NVFP4KV_ERR_NULL;
  if (!aligned16(k_out) || !aligned16(v_out) || (reinterpret_cast<uintptr_t>(page_table) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(row_offsets) & 7u))
    return NVFP4KV_ERR_ALIGN;
  nvfp4kv::DequantArgs a;
  a.pool = static_cast<const uint8_t*>(pool->data);
  a.num_kv_heads = pool->num_kv_heads;
  a.g = pool->global_scale;
  a.g_pow2 = is_pow2(pool->global_scale);
  a.page_table = page_table;
  a.pt_stride = page_table_stride;
  a.seq_lens = seq_lens;
  a.row_offsets = row_offsets;
  a.n_seqs = n_seqs;
  a.max_seq_len = max_seq_len;
  a.k_out = k_out;
  a.v_out = v_out;
  a.out_dtype = out_dtype;
  return hip_status(nvfp4kv::launch_dequant(a, static_cast<hipStream_t>(stream)));
}

int32_t nvfp4_extend_attn(const void* q, const void* k_prefix, const void* v_prefix, int32_t prefix_dtype,
                          int64_t prefix_len, const void* k_chunk, const void* v_chunk, int64_t chunk_len,
                          int32_t num_q_heads, int32_t num_kv_heads, float sm_scale, float v_bound, void* out,
                          float* lse, const nvfp4kv_pool* chunk_pool, const int32_t* chunk_slots, void* stream) {
  if (chunk_pool) {
    if (int32_t e = check_pool(chunk_pool)) return e;
    if (chunk_pool->num_kv_heads != num_kv_heads) return NVFP4KV_ERR_SHAPE;
  }
  if (prefix_dtype != NVFP4KV_BF16 && prefix_dtype != NVFP4KV_FP8_E4M3 && prefix_dtype != NVFP4KV_F16_TILED)
    return NVFP4KV_ERR_DTYPE;
  // a tiled prefix's V arrives in f16 as it is: no room for a power-of-two scaling
  if (prefix_dtype == NVFP4KV_F16_TILED && prefix_len > 0 && v_bound > 32768.0f) return NVFP4KV_ERR_VALUE;
  if (prefix_len < 0 || chunk_len < 0 || num_q_heads < 1 || num_kv_heads < 1) return NVFP4KV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > NVFP4KV_MAX_GROUP) return NVFP4KV_ERR_SHAPE;
  // element offsets of every operand stay far inside int64
  if (prefix_len > ((int64_t)1 << 40) / ((int64_t)num_kv_heads * 128) ||
      chunk_len > ((int64_t)1 << 31) / ((int64_t)num_q_heads * 128))
    return NVFP4KV_ERR_SHAPE;
  if (!isfinite(sm_scale) || !(v_bound >= 0.0f) || !isfinite(v_bound)) return NVFP4KV_ERR_VALUE;
  if (chunk_len == 0) return NVFP4KV_OK;
  if (!q || !k_chunk || !v_chunk || !out || (prefix_len > 0 && (!k_prefix || !v_prefix))) return NVFP4KV_ERR_NULL;
  if (chunk_pool && !chunk_slots) return NVFP4KV_ERR_NULL;
  if (chunk_slots && (reinterpret_cast<uintptr_t>(chunk_slots) & 3u)) return NVFP4KV_ERR_ALIGN;
  if (!aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(out) ||
      (prefix_len > 0 && (!aligned16(k_prefix) || !aligned16(v_prefix))) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return NVFP4KV_ERR_ALIGN;
  nvfp4kv::ExtendArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_pre = k_prefix;
  a.v_pre = v_prefix;
  a.pre_kind = prefix_dtype == NVFP4KV_FP8_E4M3 ? 1 : prefix_dtype == NVFP4KV_F16_TILED ? 2 : 0;
  a.prefix_len = prefix_len;
  a.k_chunk = static_cast<const uint16_t*>(k_chunk);
  a.v_chunk = static_cast<const uint16_t*>(v_chunk);
  a.chunk_len = chunk_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.qk_scale_log2 = fabsf(sm_scale) * 1.4426950408889634f;
  a.q_sign = sm_scale < 0.0f ? 0x80008000u : 0u;
  // V is brought below 2^15 in magnitude by an exact power of two before its f16
  // conversion, and the output scaled back
  int v_exp = 0;
  while (ldexpf(v_bound, -v_exp) > 32768.0f) ++v_exp;
  a.v_mul = ldexpf(1.0f, -v_exp);
  a.out_mul = ldexpf(1.0f, v_exp);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.tokens_per_block = nvfp4kv::extend_tokens_per_block(a.group);
  const int64_t blocks = (chunk_len + a.tokens_per_block - 1) / a.tokens_per_block;
  if (blocks * num_kv_heads > ((int64_t)1 << 31) - 1) return NVFP4KV_ERR_SHAPE;
  a.num_token_blocks = (int32_t)blocks;
  a.write_chunk = chunk_pool != nullptr;
  if (chunk_pool) {
    nvfp4kv::QuantizeArgs& w = a.qw;
    w.k = k_chunk;
    w.v = v_chunk;
    w.bf16 = 1;
    w.token_stride = (int64_t)num_kv_heads * NVFP4KV_HEAD_DIM;
    w.head_stride = NVFP4KV_HEAD_DIM;
    w.slots = chunk_slots;
    w.num_tokens = chunk_len;
    w.pool = static_cast<uint8_t*>(chunk_pool->data);
    w.num_kv_heads = num_kv_heads;
    w.g = chunk_pool->global_scale;
    w.g_pow2 = is_pow2(chunk_pool->global_scale);
    w.fp8 = 0;
    w.inv_k_scale = w.inv_v_scale = 1.0f;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.write_chunk && !a.qw.g_pow2) {
    // the extend kernel fuses only the power-of-two encode; any other g is
    // written by the quantize kernel first (the same bytes)
    if (int32_t e = hip_status(nvfp4kv::launch_quantize(a.qw, st))) return e;
    a.write_chunk = 0;
  }
  return hip_status(nvfp4kv::launch_extend(a, st));
}

}  // extern "C"

// ---- decode without a caller workspace ----------------------------------------
// The split states of nvfp4_paged_decode_attn_noalloc live in one fixed device
// array per GPU. In host code `scratch` is only a stand-in for the symbol: its
// device address comes from hipGetSymbolAddress, once per device, and only that
// address is ever passed to a kernel.
namespace {

constexpr size_t kScratchBytes = (size_t)NVFP4KV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array (NULL on failure).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

int32_t nvfp4_paged_decode_attn_noalloc(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                        int32_t max_seq_len, const nvfp4kv_pool* pool, float sm_scale,
                                        int32_t num_splits, void* out, int32_t out_dtype, float* lse, void* stream) {
  if (int32_t e = check_pool(pool)) return e;
  if (out_dtype != NVFP4KV_F32 && out_dtype != NVFP4KV_BF16) return NVFP4KV_ERR_DTYPE;
  if (batch < 0 || num_q_heads < 1 || max_seq_len < 0 || page_table_stride < 1) return NVFP4KV_ERR_SHAPE;
  if (num_splits < 0 || num_splits > NVFP4KV_MAX_SPLITS) return NVFP4KV_ERR_SHAPE;
  if (batch == 0) return NVFP4KV_OK;
  // the most splits whose states fit the scratch array
  const size_t per_split = nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, 1);
  if (per_split == 0 || per_split > kScratchBytes) return NVFP4KV_ERR_SCRATCH;
  int32_t fit = (int32_t)(kScratchBytes / per_split < NVFP4KV_MAX_SPLITS ? kScratchBytes / per_split
                                                                          : NVFP4KV_MAX_SPLITS);
  while (fit > 1 && nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, fit) > kScratchBytes) --fit;
  if (num_splits > 0 && nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, num_splits) > kScratchBytes)
    return NVFP4KV_ERR_SCRATCH;
  if (num_splits == 0) {
    int cus = 0;
    if (!query_cus(&cus)) return NVFP4KV_ERR_HIP;
    num_splits = default_splits(batch, pool->num_kv_heads, max_seq_len, cus, false);
    if (num_splits > fit) num_splits = fit;
  }
  // every argument check of the workspace entry point runs before the scratch
  // address is looked up (the only HIP call here that is not a launch)
  nvfp4kv::DecodeArgs a, c;
  const size_t ws_bytes = nvfp4_paged_decode_attn_workspace_bytes(batch, num_q_heads, num_splits);
  void* const kFakeAligned = reinterpret_cast<void*>((uintptr_t)256);  // stands in for the scratch in checks
  if (int32_t e = prepare_decode(q, page_table, page_table_stride, seq_lens, batch, num_q_heads, max_seq_len,
                                 info_of(pool), sm_scale, &num_splits, kFakeAligned, ws_bytes, a))
    return e;
  if (int32_t e = prepare_combine(kFakeAligned, ws_bytes, batch, num_q_heads, num_splits, out, out_dtype, lse, c))
    return e;
  void* ws = scratch_of_current_device();
  if (!ws) return NVFP4KV_ERR_HIP;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = a.part_o + (size_t)batch * num_q_heads * num_splits * NVFP4KV_HEAD_DIM;
  c.part_o = a.part_o;
  c.part_ml = a.part_ml;
  if (int32_t e = finish_decode(a)) return e;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (int32_t e = hip_status(nvfp4kv::launch_decode_partial(a, st))) return e;
  return hip_status(nvfp4kv::launch_decode_combine(c, st));
}

}  // extern "C"
