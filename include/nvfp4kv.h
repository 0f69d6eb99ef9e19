/*
 * nvfp4kv.h — C ABI of the NVFP4 paged-KV attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [LMSYS]  "SGLang stores KV cache in 4 bits: long-context decode throughput
 *            rises 26-30%, and FP8 stalls first under agent concurrency"
 *            (summary of the LMSYS post "Accelerating Long-Context and Agentic
 *            Inference with NVFP4 KV Cache").
 *   [EUROK]  "NVFP4-KV-Cache auf der NVIDIA RTX PRO 6000 Blackwell Server
 *            Edition: Genauigkeit, Nutzer".
 *
 * The library computes four things on the GPU, each in hand-written HIP:
 *   - nvfp4_kv_quantize: quantize-on-write of K/V rows into the NVFP4 pool
 *     ([LMSYS] "Interpretation": initial prefill quantizes the prompt's keys and
 *     values into the NVFP4 cache).
 *   - nvfp4_paged_decode_attn: grouped-query decode attention that reads the
 *     paged NVFP4 cache and dequantizes it inside the kernel ([LMSYS]
 *     "Interpretation"; [EUROK] "Geschwindigkeit": the decode kernel takes 16-bit
 *     queries and NVFP4 keys and values).
 *   - nvfp4_kv_dequant_workspace: the extend path's dequantization of a cached
 *     prefix into a dense workspace ([LMSYS] "Interpretation").
 *   - nvfp4_extend_attn: the extend path's attention of a chunk of queries over
 *     that workspace and the chunk itself ([LMSYS] "Interpretation").
 * and, as the baseline the pages compare against, an FP8 E4M3 paged cache with
 * the same decode machinery (fp8_kv_quantize, fp8_paged_decode_attn).
 *
 * NVFP4 ([EUROK] "Bytes pro Token"; [LMSYS] "Interpretation", "Perspective"):
 * each value is E2M1 (1 sign, 2 exponent, 1 mantissa bit; magnitudes 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6); each 16 contiguous values of a head row share one E4M3 (OCP
 * "fn", max 448) block scale s; a per-tensor float global scale g sits above
 * (1.0 in every experiment the pages report). A value decodes to
 * E2M1(c) * E4M3(s) * g. Encoding: s = E4M3 nearest to amax/(6 g), ties to
 * even, clamped to 448; c = E2M1 nearest to x/(E4M3(s) g), ties to even,
 * saturating at 6, sign bit = sign bit of x; a zero scale gives magnitude-0
 * codes. 8 code bytes + 1 scale byte per 16 values.
 *
 * Pool layout (NVFP4KV_SLAB_BYTES = 1152 per slab):
 *   slab(page p, KV head h, kind k) starts at byte ((p*Hkv + h)*2 + k) * 1152,
 *   k = 0 for K, 1 for V. A slab holds the 16 token rows r of page p for head h:
 *   1024 code bytes (one 4-bit code per value), then 128 scale bytes (block j =
 *   channels 16j..16j+15):
 *     K code (r, d):  byte r*64 + d/2, low nibble for even d, high for odd d
 *     K scale (r, j): byte 1024 + r*8 + j
 *     V code (r, d):  byte ((r/4)*16 + d/8)*16 + 2*(d%8) + r%2,
 *                     low nibble for r%4 < 2, high nibble for r%4 >= 2
 *     V scale (r, j): byte 1024 + j*16 + r
 *   K rows are token-major. V is cut into 64 chunks of 16 bytes; chunk
 *   (r/4)*16 + d/8 holds channels 8(d/8)..+7 of tokens 4(r/4)..+3, and each of
 *   its bytes holds one channel of two tokens (r and r+2), the pairs the decode
 *   kernel's matrix-core operands take along the token axis. A V byte is
 *   therefore shared by two tokens. nvfp4_kv_quantize writes whole V bytes only
 *   where the same call writes every token they hold (a whole page, or a group
 *   of four rows 4G..4G+3). Otherwise it updates only the written token's
 *   nibbles, with atomics. Tokens of one page may therefore be written by
 *   different calls, or by one call in any order.
 *   Token t of a sequence lives at page page_table[t/16], row t%16.
 *
 * Conventions for every entry point:
 *   - The caller owns all memory; the library allocates nothing, keeps no
 *     global mutable state, and is reentrant. The one exception is
 *     nvfp4_paged_decode_attn_noalloc, which keeps its split states in a fixed
 *     device array of the library (see there).
 *   - Arguments named *device* are device pointers; the pool descriptor is a
 *     host pointer to a struct whose data member is a device pointer.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and returns without synchronizing.
 *   - Every host-side check runs before any HIP call; on error nothing is
 *     enqueued and a status > 0 is returned. Device-side data errors (a page id
 *     outside the pool, seq_lens[b] > max_seq_len or beyond the page table row,
 *     a slot outside the pool) are undefined behaviour; nvfp4kv_check_page_table
 *     checks them on host copies.
 */
#ifndef NVFP4KV_H_
#define NVFP4KV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4KV_HEAD_DIM 128
#define NVFP4KV_PAGE_SIZE 16
#define NVFP4KV_SLAB_BYTES 1152
#define NVFP4KV_MAX_GROUP 16     /* query heads per KV head */
#define NVFP4KV_MAX_SPLITS 4096
#define NVFP4KV_ALIGN 16         /* required alignment (bytes) of every device pointer */

enum nvfp4kv_status {
  NVFP4KV_OK = 0,
  NVFP4KV_ERR_NULL = 1,      /* a required pointer is NULL */
  NVFP4KV_ERR_SHAPE = 2,     /* a size, count or stride is out of range */
  NVFP4KV_ERR_ALIGN = 3,     /* a pointer or stride breaks the 16-byte rule */
  NVFP4KV_ERR_DTYPE = 4,     /* unsupported dtype code */
  NVFP4KV_ERR_WORKSPACE = 5, /* workspace smaller than required */
  NVFP4KV_ERR_VALUE = 6,     /* a float argument is not allowed (e.g. global scale) */
  NVFP4KV_ERR_HIP = 7,       /* a HIP runtime call failed */
  NVFP4KV_ERR_SCRATCH = 8    /* nvfp4_paged_decode_attn_noalloc: the states exceed its fixed scratch */
};

/* Element types. NVFP4KV_FP8_E4M3 (OCP E4M3 "fn": 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, largest finite 448, no infinities) is an output type
 * of the extend dequantization only. NVFP4KV_F16_TILED is an extend workspace of
 * two parts: K as bf16 rows [rows][Hkv][128] (as NVFP4KV_BF16), and V as f16 in
 * tiles of 64 rows: row r of KV head h, channel d lies at byte
 *   ((r/64) Hkv + h) 16384 + d 128 + 16 u + 8 ((k/16) % 2) + 2 (k % 4),
 *   k = r % 64, u = 4 (k/32) + (k/4) % 4
 * (nvfp4kv_tiled_v_bytes bytes for `rows` rows): each 16-byte unit holds the
 * eight keys one matrix-core operand of nvfp4_extend_attn takes, so its V tiles
 * are copied into the kernel's local memory unchanged. */
enum nvfp4kv_dtype { NVFP4KV_F32 = 0, NVFP4KV_BF16 = 1, NVFP4KV_FP8_E4M3 = 2, NVFP4KV_F16_TILED = 3 };

/* Bytes of the V part of an NVFP4KV_F16_TILED workspace of `rows` rows. */
int64_t nvfp4kv_tiled_v_bytes(int64_t rows, int32_t num_kv_heads);

/* NVFP4 KV pool of one layer. */
typedef struct nvfp4kv_pool {
  void* data;            /* device, 16-byte aligned, num_pages*num_kv_heads*2*1152 bytes */
  int64_t num_pages;     /* >= 1 */
  int32_t num_kv_heads;  /* >= 1 */
  float global_scale;    /* g: any finite float in [2^-64, 2^64] (1.0 in all workloads) */
} nvfp4kv_pool;

/* Bytes of a pool of num_pages pages and num_kv_heads heads. */
int64_t nvfp4kv_pool_bytes(int64_t num_pages, int32_t num_kv_heads);

/* Static string for a status code (never NULL). */
const char* nvfp4kv_status_string(int32_t status);

/* Library ABI version (incremented on any signature or layout change): 2. */
int32_t nvfp4kv_version(void);

/*
 * Host-side check of the data preconditions the kernels do not check (a page id
 * outside the pool or a length beyond the table makes them read or write out of
 * bounds). It reads HOST copies of the page table and the lengths, runs on the
 * CPU only and makes no HIP call; call it where such inputs are built or in a
 * debug run. For each b < batch: 0 <= seq_lens[b] <= max_seq_len, seq_lens[b] <=
 * page_table_stride * 16, and every page id of the first ceil(seq_lens[b] / 16)
 * entries of row b lies in [0, num_pages). With `seen` (host, num_pages bytes,
 * contents overwritten) it also checks that no physical page holds live tokens of
 * two sequences, or twice in one sequence (the fused decode step writes each
 * sequence's newest page while the others are read). Returns NVFP4KV_OK, or
 * NVFP4KV_ERR_SHAPE for a length and NVFP4KV_ERR_VALUE for a page id, with
 * *bad_index (if not NULL) set to the offending b (lengths) or b *
 * page_table_stride + logical page (ids); NVFP4KV_ERR_NULL / ERR_SHAPE for
 * missing pointers or negative sizes.
 */
int32_t nvfp4kv_check_page_table(const int32_t* page_table, int64_t page_table_stride, const int32_t* seq_lens,
                                 int32_t batch, int32_t max_seq_len, int64_t num_pages, uint8_t* seen,
                                 int64_t* bad_index);

/*
 * Quantize-on-write ([LMSYS] "Interpretation"; format per [EUROK] "Bytes pro
 * Token"). For each token t < num_tokens with slot_mapping[t] >= 0 and each KV
 * head h, encodes K[t][h][0..127] and V[t][h][0..127] as 8 NVFP4 blocks each and
 * writes codes and scales to page slot/16, row slot%16 of `pool` (layout above).
 * Tokens with a negative slot are skipped. Output bytes are a deterministic
 * function of the inputs; distinct tokens must map to distinct slots.
 *   k_src, v_src    device; element (t, h, d) at t*token_stride + h*head_stride + d
 *                   (elements), float32 or bfloat16 per src_dtype
 *   src_dtype       NVFP4KV_F32 or NVFP4KV_BF16
 *   token_stride,
 *   head_stride     elements; multiples of 4 (F32) or 8 (BF16)
 *   slot_mapping    device int32 [num_tokens]
 *   num_tokens      >= 0 (0 is a no-op)
 * Every rounding decision is the one on the exact real quotients amax/(6 g) and
 * x/(E4M3(s) g), for any allowed g: with a power of two through an exact fp32
 * quotient test, otherwise through fp64 comparisons against exact threshold
 * products (slower: about three times the arithmetic per value).
 * Errors: NULL pointers (ERR_NULL); bad dtype (ERR_DTYPE); unaligned pointer or
 * stride (ERR_ALIGN); negative sizes, a non-positive page or head count
 * (ERR_SHAPE); global scale not finite or outside [2^-64, 2^64] (ERR_VALUE).
 */
int32_t nvfp4_kv_quantize(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                          int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens,
                          const nvfp4kv_pool* pool, void* stream);

/*
 * Split count the decode call uses when passed num_splits = 0. The decode
 * kernel keeps up to 4 workgroups of 4 waves resident per compute unit for the
 * whole launch (fewer when the cache is small: at most one workgroup per 8
 * pages of batch x num_kv_heads x ceil(max_seq_len / 16)) and gives each a
 * window of about equal page count, cut at split boundaries. The default makes
 * about 16 splits per window (windows within about 6% of each other), at least
 * 4 pages per split, at most NVFP4KV_MAX_SPLITS.
 * num_cus <= 0 asks the current
 * HIP device for its compute-unit count (the only HIP call of this function).
 * Returns >= 1.
 */
int32_t nvfp4_paged_decode_attn_default_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                               int32_t num_cus);

/* Workspace bytes the decode call needs for the given sizes (num_splits >= 1;
 * pass the resolved split count). Returns 0 for invalid sizes. */
size_t nvfp4_paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_splits);

/*
 * Decode attention over the paged NVFP4 cache ([LMSYS] "Interpretation": decode
 * dequantizes inside the attention kernel; [EUROK] "Geschwindigkeit"; grouped-
 * query attention per [EUROK] "Unterstuetzung in den Engines"). For each
 * sequence b and query head qh (KV head h = qh / (num_q_heads / num_kv_heads)):
 *   out[b][qh] = sum_t softmax_t(sm_scale * q[b][qh] . K^[t]) V^[t],
 *   t < seq_lens[b], K^/V^ the dequantized cache of head h,
 *   lse[b][qh] = natural-log log-sum-exp of the scaled logits.
 * Split-K flash decoding: num_splits ranges of pages per (b, h) are reduced with
 * an online softmax into the workspace, then combined. A sequence of length 0
 * yields out = 0 and lse = -inf.
 *   q               device bf16 [batch][num_q_heads][128], row-major
 *   page_table      device int32 [batch][page_table_stride] physical page ids
 *   seq_lens        device int32 [batch], each in [0, max_seq_len]
 *   max_seq_len     host upper bound of seq_lens (<= page_table_stride*16)
 *   pool            host pointer to the pool descriptor
 *   sm_scale        finite softmax scale (1/sqrt(128) in the workloads)
 *   num_splits      0 = nvfp4_paged_decode_attn_default_splits(..., 0), or 1..4096
 *   workspace       device scratch of >= nvfp4_paged_decode_attn_workspace_bytes
 *                   bytes for the resolved split count; contents are overwritten
 *   out             device [batch][num_q_heads][128], bf16 or f32 per out_dtype
 *   lse             device f32 [batch][num_q_heads], or NULL
 * Limits: num_q_heads % num_kv_heads == 0, 1 <= num_q_heads/num_kv_heads <= 16.
 * Errors: ERR_NULL, ERR_SHAPE (sizes, group, splits, strides), ERR_ALIGN,
 * ERR_DTYPE (out_dtype), ERR_WORKSPACE, ERR_VALUE (sm_scale not finite, global
 * scale), ERR_HIP (launch failure, or the CU-count query when num_splits = 0).
 */
int32_t nvfp4_paged_decode_attn(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                                const nvfp4kv_pool* pool, float sm_scale, int32_t num_splits, void* workspace,
                                size_t workspace_bytes, void* out, int32_t out_dtype, float* lse, void* stream);

/*
 * The two phases of nvfp4_paged_decode_attn, for callers that time, overlap or
 * distribute them (for example, merging states computed on several devices).
 *
 * Phase 1, nvfp4_paged_decode_attn_partial: same inputs and checks as
 * nvfp4_paged_decode_attn, num_splits >= 1 (resolved by the caller). Split s of
 * sequence b covers logical pages [s*P, min((s+1)*P, n_b)), P = ceil(n_b / S),
 * n_b = ceil(seq_lens[b] / 16). For every (b, qh, s) it writes an online-softmax
 * state into the workspace:
 *   M[b][qh][s]      reference exponent (base 2) of the logits of the tokens the
 *                    state covers, -inf for an empty state; not necessarily
 *                    their maximum,
 *   Z[b][qh][s]      sum over those tokens of 2^(x_t log2(e) - M),
 *   O[b][qh][s][128] sum over those tokens of 2^(x_t log2(e) - M) v^_t,
 * with x_t = sm_scale q . k^_t (natural-log logits). State s covers the tokens
 * of splits s..s' for some s' >= s (consecutive splits one workgroup processed
 * together); the states of splits s+1..s' are then empty (M = -inf, Z = 0) and
 * their O is not written. Together the S states cover every token once.
 * Workspace layout: O as f32 [B][Hq][S][128] at byte 0, then (M, Z) as f32
 * pairs [B][Hq][S][2] at byte B*Hq*S*128*4.
 *
 * Phase 2, nvfp4_decode_combine: for every (b, qh) merges the S states:
 *   M* = max_s M, Z* = sum_s 2^(M_s - M*) Z_s, out = sum_s 2^(M_s - M*) O_s / Z*,
 *   lse = (M* + log2 Z*) ln 2; all states empty: out = 0, lse = -inf. The O of
 *   an empty state (M = -inf) is never read.
 * Errors: as nvfp4_paged_decode_attn (ERR_SHAPE for num_splits outside
 * 1..4096, ERR_WORKSPACE when the workspace is smaller than the layout above).
 */
int32_t nvfp4_paged_decode_attn_partial(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                        int32_t max_seq_len, const nvfp4kv_pool* pool, float sm_scale,
                                        int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

int32_t nvfp4_decode_combine(const void* workspace, size_t workspace_bytes, int32_t batch, int32_t num_q_heads,
                             int32_t num_splits, void* out, int32_t out_dtype, float* lse, void* stream);

/*
 * Decode attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and result as nvfp4_paged_decode_attn, without the
 * workspace argument. The split states go to a device array the library holds,
 * NVFP4KV_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, kept from the first call on a
 * GPU until the process ends. That first call also looks up the array's device
 * address (hipGetSymbolAddress); no call allocates anything.
 *   num_splits   0: the default split count, lowered until the states fit the
 *                scratch; otherwise the states of num_splits splits
 *                (nvfp4_paged_decode_attn_workspace_bytes) must fit, else
 *                NVFP4KV_ERR_SCRATCH
 *   all other arguments, results and errors as nvfp4_paged_decode_attn.
 * Every call on one GPU uses the same array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and give wrong results.
 * Calls in order on one stream are safe; nothing in the array needs to start
 * at zero (each call writes every state it reads).
 */
#define NVFP4KV_NOALLOC_SCRATCH_BYTES (64 << 20)
int32_t nvfp4_paged_decode_attn_noalloc(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                        const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                        int32_t max_seq_len, const nvfp4kv_pool* pool, float sm_scale,
                                        int32_t num_splits, void* out, int32_t out_dtype, float* lse, void* stream);

/*
 * One decode step with its quantize-on-write in the same launch ([LMSYS]
 * "Interpretation": each step writes the new token's K/V into the NVFP4 cache
 * and the decode kernel reads the cache dequantizing in registers). For each
 * sequence b with seq_lens[b] >= 1, token L-1 (L = seq_lens[b]) is the newest:
 * its K/V rows k_new[b], v_new[b] are encoded exactly as nvfp4_kv_quantize
 * encodes them and written to slot page_table[b][(L-1)/16]*16 + (L-1)%16 of the
 * pool; then the attention of nvfp4_paged_decode_attn runs over tokens 0..L-1,
 * the new one included. Result: the pool bytes and out/lse of
 * nvfp4_kv_quantize(k_new, v_new, those slots) followed by
 * nvfp4_paged_decode_attn, with one launch fewer.
 *   k_new, v_new    device [batch][num_kv_heads][128] at b*new_token_stride +
 *                   h*new_head_stride + d (elements), float32 or bfloat16 per
 *                   new_dtype (NVFP4KV_F32 / NVFP4KV_BF16); strides multiples
 *                   of 4 (F32) or 8 (BF16)
 *   out             as nvfp4_paged_decode_attn, or NULL (then lse must be NULL):
 *                   the call stops after phase 1 and leaves the partial states
 *                   in the workspace, as nvfp4_paged_decode_attn_partial does,
 *                   for nvfp4_decode_combine
 *   all other arguments as nvfp4_paged_decode_attn.
 * The page holding a sequence's newest token must not be among the first
 * ceil(seq_lens/16) pages of another sequence of the batch (it is written while
 * the others are read). Errors: as nvfp4_paged_decode_attn, plus ERR_NULL,
 * ERR_DTYPE, ERR_SHAPE (negative strides) and ERR_ALIGN for the new rows, and
 * ERR_NULL for an lse without out.
 */
int32_t nvfp4_paged_decode_attn_append(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                                       int64_t new_token_stride, int64_t new_head_stride, const int32_t* page_table,
                                       int64_t page_table_stride, const int32_t* seq_lens, int32_t batch,
                                       int32_t num_q_heads, int32_t max_seq_len, const nvfp4kv_pool* pool,
                                       float sm_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                                       void* out, int32_t out_dtype, float* lse, void* stream);

/*
 * Extend-path dequantization ([LMSYS] "Interpretation": the cached prefix is
 * dequantized into one workspace shared across layers and attended alongside the
 * current chunk). For each listed sequence s and t < seq_lens[s], writes the
 * dequantized K and V rows of every KV head to row row_offsets[s] + t of the
 * dense workspaces k_out / v_out, shaped [rows][num_kv_heads][128]. Each value
 * is the nearest value of the workspace dtype to the exact E2M1 * E4M3 * g, ties
 * to even (one rounding): with a power-of-two g the values (at most 6
 * significant bits) are exact in f32 and bf16; with any other g they carry up
 * to 30 significant bits and are rounded. With NVFP4KV_FP8_E4M3 (the pages' FP8
 * workspace) values of magnitude above 448 become +-448 (saturation); the sign
 * of zero is kept. No value exceeds 2688 g in magnitude.
 *   page_table      device int32 [n_seqs][page_table_stride]
 *   seq_lens        device int32 [n_seqs], prefix tokens to dequantize, each in
 *                   [0, max_seq_len]
 *   row_offsets     device int64 [n_seqs], first workspace row of each sequence
 *   max_seq_len     host upper bound of seq_lens (<= page_table_stride*16)
 *   k_out, v_out    device, f32, bf16 or FP8 E4M3 (one byte) per out_dtype; with
 *                   NVFP4KV_F16_TILED, k_out bf16 rows and v_out f16 tiles (see
 *                   the dtype): every value is the f16 nearest the exact value
 *                   (one rounding; g <= 16, so that no value exceeds the f16
 *                   range). A sequence whose row_offsets entry is a multiple
 *                   of 64 owns its tiles (no other sequence may have rows in
 *                   them): they are written whole, the rows of its last tile
 *                   after its last row as zeros. Any other
 *                   sequence gets only its own rows, one value at a time
 *                   (slower), so sequences may share a tile.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_VALUE (global scale; g
 * above 16 with NVFP4KV_F16_TILED), ERR_HIP.
 */
int32_t nvfp4_kv_dequant_workspace(const nvfp4kv_pool* pool, const int32_t* page_table, int64_t page_table_stride,
                                   const int32_t* seq_lens, const int64_t* row_offsets, int32_t n_seqs,
                                   int32_t max_seq_len, void* k_out, void* v_out, int32_t out_dtype, void* stream);

/*
 * Global-scale calibration hook ([LMSYS] "Perspective": the experiments left
 * the per-tensor FP32 global scale at 1.0, and calibrating it may narrow the
 * accuracy gap to FP8). nvfp4_kv_amax writes max |K| and max |V| over T tokens
 * of every KV head (same source arguments as nvfp4_kv_quantize) to amax_out[0]
 * and amax_out[1] (device f32); NaN elements are ignored. It takes a device
 * workspace of nvfp4_kv_amax_workspace_bytes() bytes (two launches, no atomics,
 * no memset; nothing is allocated). nvfp4kv_global_scale_for_amax (host, pure)
 * returns the smallest power of two g with amax / (6 g) <= 448, so that no
 * block scale saturates and the largest ones use the top of the E4M3 range; 1.0
 * for amax = 0; 0.0 when amax is negative, not finite, or g would fall outside
 * [2^-64, 2^64]. One pool has one g: pass max(amax[0], amax[1]).
 * nvfp4kv_global_scale_tight_for_amax (host, pure) returns the smallest binary32
 * g with amax <= 2688 g ([EUROK] "Bytes pro Token": the global scale is an FP32
 * number), so that the largest block scale is 448 or just below; the same
 * conventions for amax = 0 and invalid input. Values dequantized at g reach at
 * most 2688 g in magnitude: pass that bound as nvfp4_extend_attn's v_bound.
 * Errors: ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_WORKSPACE, ERR_HIP.
 */
size_t nvfp4_kv_amax_workspace_bytes(void);
int32_t nvfp4_kv_amax(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                      int64_t head_stride, int64_t num_tokens, int32_t num_kv_heads, float* amax_out,
                      void* workspace, size_t workspace_bytes, void* stream);
float nvfp4kv_global_scale_for_amax(float amax);
float nvfp4kv_global_scale_tight_for_amax(float amax);

/*
 * ---- FP8 E4M3 baseline ------------------------------------------------------
 * The cache the pages compare NVFP4 against ([LMSYS] "Synopsis", "Perspective";
 * [EUROK] "Bytes pro Token": one byte per value), built with the same decode
 * machinery so that the comparison is between formats, not kernels. Each value
 * is stored as the E4M3 ("fn") code of x / s, with s the per-tensor scale of K
 * or V: the nearest E4M3 value, ties to the even code, magnitudes above 448
 * saturate to +-448, sign kept. It decodes to E4M3(code) * s.
 *
 * FP8 pool layout: each page holds, for each KV head h, a K slab then a V slab
 * of 2048 bytes each: slab(p, h, kind) at byte ((p * Hkv + h) * 2 + kind) * 2048,
 * one code byte per value:
 *   K (row r, channel d): byte r*128 + d
 *   V (row r, channel d): byte ((r/4)*16 + d/8)*32 + (d%8)*4 + r%4
 * (a 32-byte V chunk holds channels 8n..8n+7 of rows 4g..4g+3, channel-major,
 * so that one 32-bit word is the four rows of one channel). Each byte belongs to
 * one value: writes of distinct tokens never touch each other's bytes.
 */
#define FP8KV_SLAB_BYTES 2048

typedef struct fp8kv_pool {
  void* data;            /* device, 16-byte aligned, num_pages*num_kv_heads*2*2048 bytes */
  int64_t num_pages;     /* >= 1 */
  int32_t num_kv_heads;  /* >= 1 */
  float k_scale;         /* per-tensor scales: powers of two in [2^-64, 2^64] */
  float v_scale;
} fp8kv_pool;

/* Bytes of an FP8 pool of num_pages pages and num_kv_heads heads. */
int64_t fp8kv_pool_bytes(int64_t num_pages, int32_t num_kv_heads);

/* Quantize-on-write into the FP8 pool: arguments, slots and errors as
 * nvfp4_kv_quantize (ERR_VALUE: a scale that is not a power of two in range). */
int32_t fp8_kv_quantize(const void* k_src, const void* v_src, int32_t src_dtype, int64_t token_stride,
                        int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens, const fp8kv_pool* pool,
                        void* stream);

/* Decode attention over the FP8 pool: arguments, outputs, partial-state format
 * (phase 2 is nvfp4_decode_combine), workspace size and errors as
 * nvfp4_paged_decode_attn / _partial. The kernel runs four workgroups of two
 * waves per CU (an FP8 page slot is 4 KB of LDS), so its default split count
 * comes from fp8_paged_decode_attn_default_splits. */
int32_t fp8_paged_decode_attn_default_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                                             int32_t num_cus);
int32_t fp8_paged_decode_attn(const void* q, const int32_t* page_table, int64_t page_table_stride,
                              const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, int32_t max_seq_len,
                              const fp8kv_pool* pool, float sm_scale, int32_t num_splits, void* workspace,
                              size_t workspace_bytes, void* out, int32_t out_dtype, float* lse, void* stream);
int32_t fp8_paged_decode_attn_partial(const void* q, const int32_t* page_table, int64_t page_table_stride,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_q_heads,
                                      int32_t max_seq_len, const fp8kv_pool* pool, float sm_scale,
                                      int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);
/* One FP8 decode step with its quantize-on-write in the same launch: arguments,
 * result and errors as nvfp4_paged_decode_attn_append, with the FP8 encode of
 * fp8_kv_quantize. */
int32_t fp8_paged_decode_attn_append(const void* q, const void* k_new, const void* v_new, int32_t new_dtype,
                                     int64_t new_token_stride, int64_t new_head_stride, const int32_t* page_table,
                                     int64_t page_table_stride, const int32_t* seq_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t max_seq_len, const fp8kv_pool* pool, float sm_scale,
                                     int32_t num_splits, void* workspace, size_t workspace_bytes, void* out,
                                     int32_t out_dtype, float* lse, void* stream);

/*
 * Extend-path attention ([LMSYS] "Interpretation": after the cached prefix is
 * dequantized into a workspace, the chunk's queries attend over it and over the
 * chunk). One request: a chunk of C tokens that follows a P-token prefix. Query
 * token i (0 <= i < C), query head qh, attends over all P workspace rows and
 * over chunk rows 0..i (causal), reading KV head qh / (num_q_heads /
 * num_kv_heads):
 *   out[i][qh] = sum_t softmax_t(sm_scale * q[i][qh] . k_t) v_t,
 *   lse[i][qh] = ln sum_t exp(sm_scale * q[i][qh] . k_t)   (natural log)
 * Readings (the page names no mask and no precision for the chunk's own rows):
 * the mask is causal over the chunk, and the chunk's keys and values enter as
 * the bf16 values given here, not via the NVFP4 cache.
 *   q               device bf16 [C][num_q_heads][128], contiguous
 *   k_prefix, v_prefix  device [P][num_kv_heads][128] workspace as written by
 *                   nvfp4_kv_dequant_workspace: NVFP4KV_BF16 or
 *                   NVFP4KV_FP8_E4M3 per prefix_dtype (finite values), or
 *                   NVFP4KV_F16_TILED (K bf16 rows, V f16 tiles whose rows past
 *                   P are finite, as the dequant writes them); may be NULL when
 *                   P = 0. With the tiled V the prefix's V^T tiles need no
 *                   conversion pass in the kernel.
 *   k_chunk, v_chunk    device bf16 [C][num_kv_heads][128], contiguous
 *   out             device bf16 [C][num_q_heads][128]
 *   lse             device f32 [C][num_q_heads] or NULL
 * num_q_heads must be a multiple of num_kv_heads with a quotient of at most 16.
 * Arithmetic: fp32 accumulation on the matrix cores; Q and K enter the first
 * product as bf16; V and the softmax weights enter the second as f16 (the row
 * sums use the same rounded weights).
 *   v_bound         an upper bound of |V| over the workspace and the chunk, or 0
 *                   when every |V| is at most 2^15. V is multiplied by 2^-e, e the
 *                   smallest integer >= 0 with v_bound * 2^-e <= 2^15,
 *                   before its f16 conversion, and the output by 2^e
 *                   (both exact). A workspace dequantized at global scale g is
 *                   bounded by 2688 g; a chunk by its amax (nvfp4_kv_amax). With
 *                   the scaling, V converts exactly for magnitudes in
 *                   [2^(e-14), 2^(e+15)] and smaller values carry an absolute
 *                   error below 2^(e-25); a |V| above 65504 * 2^e becomes
 *                   infinite (a bound that is too small gives a wrong result).
 * All device pointers 16-byte aligned; nothing is allocated; the call is
 * asynchronous on `stream`.
 * Fused quantize-on-write ([LMSYS] "Interpretation": the prefill path writes
 * the prompt's keys and values into the NVFP4 cache): when chunk_pool is not
 * NULL, the same launch also writes chunk token i's K/V to slot chunk_slots[i]
 * of chunk_pool, with exactly the bytes nvfp4_kv_quantize would write (same
 * rules, negative slots skipped; chunk_pool->num_kv_heads must equal
 * num_kv_heads). The attention reads the bf16 chunk, not those bytes.
 *   chunk_pool      NVFP4 pool or NULL (no write)
 *   chunk_slots     device int32 [C] when chunk_pool is given
 * Errors: ERR_NULL, ERR_SHAPE (counts out of range, group > 16, pool heads),
 * ERR_ALIGN, ERR_DTYPE (prefix_dtype), ERR_VALUE (sm_scale not finite, v_bound
 * negative or not finite, or above 2^15 with a tiled prefix, pool global scale),
 * ERR_HIP.
 */
int32_t nvfp4_extend_attn(const void* q, const void* k_prefix, const void* v_prefix, int32_t prefix_dtype,
                          int64_t prefix_len, const void* k_chunk, const void* v_chunk, int64_t chunk_len,
                          int32_t num_q_heads, int32_t num_kv_heads, float sm_scale, float v_bound, void* out,
                          float* lse, const nvfp4kv_pool* chunk_pool, const int32_t* chunk_slots, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H_ */
