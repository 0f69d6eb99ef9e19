/*
 * CPU oracle for NVFP4 paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Plain, slow, scalar C with fp64 arithmetic. Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it. It shares no code, header, table or constant with the GPU library: the
 * pool layout below is re-derived here from its written definition.
 *
 * Sources (web pages; cited by title and section):
 *   [LMSYS]  "SGLang stores KV cache in 4 bits: long-context decode throughput
 *            rises 26-30%, and FP8 stalls first under agent concurrency"
 *            (summary of the LMSYS post "Accelerating Long-Context and Agentic
 *            Inference with NVFP4 KV Cache").
 *   [EUROK]  "NVFP4-KV-Cache auf der NVIDIA RTX PRO 6000 Blackwell Server
 *            Edition: Genauigkeit, Nutzer".
 *
 * What is computed, step by step:
 *   1. E2M1 element decode: a 4-bit float with one sign, two exponent and one
 *      mantissa bit ([EUROK] "Bytes pro Token"). Reading: exponent bias 1, no
 *      infinities or NaN, so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   2. E4M3 block-scale decode: FP8 with four exponent and three mantissa bits
 *      ([EUROK] "Bytes pro Token"). Reading: the OCP "fn" variant, bias 7,
 *      subnormals m/8 * 2^-6, 0x7F/0xFF are NaN, largest finite 448.
 *   3. Block scale of 16 contiguous values ([LMSYS] "Interpretation": one byte
 *      of scale per 16 values): the E4M3 value nearest to amax / (6 g), ties to
 *      the even code, clamped to the largest finite value (satfinite). g is the
 *      per-tensor FP32 scale, 1.0 in every experiment ([LMSYS] "Perspective";
 *      [EUROK] "Bytes pro Token"). The quotient is the exact real number.
 *   4. Element codes: the E2M1 value nearest to x / (dec(s) g), ties to the
 *      even code, saturating at 6; the sign bit is the sign bit of x. When the
 *      scale is zero every code has magnitude 0 (a reading; the pages are
 *      silent).
 *   5. Packing: each code is one nibble; 8 data bytes plus 1 scale byte per 16
 *      values ([LMSYS] "Interpretation"). Where the nibbles sit is the pool
 *      layout below (a storage choice the pages leave open).
 *   6. Dequantization: x^ = E2M1(c) * E4M3(s) * g ([LMSYS] "Interpretation":
 *      decode dequantizes inside the attention kernel).
 *   7. Attention for decode: softmax(sm_scale * q . k^_t) weighted sum of v^_t
 *      over t < seq_len, per query head, with query head q reading KV head
 *      q / (Hq / Hkv) (grouped-query attention, [EUROK] "Unterstuetzung in den
 *      Engines"). Evaluated in fp64 as the plain definition: all logits, their
 *      maximum, exponentials, sums, one division.
 *   8. Extend (chunked-prefill) attention ([LMSYS] "Interpretation": the
 *      extend path dequantizes the cached prefix into a workspace, then runs
 *      attention over it). Query i of a C-token chunk that follows a P-token
 *      prefix attends over all P workspace rows and chunk rows 0..i, with the
 *      same softmax and head grouping as step 7. Readings (the page names no
 *      mask and no precision for the chunk's own keys and values): the mask is
 *      causal over the chunk, and the chunk's keys and values enter as the
 *      bf16 values they arrive in, not via the NVFP4 cache.
 *  10. Global-scale calibration ([LMSYS] "Perspective": the experiments left
 *      the per-tensor FP32 global scale at 1.0 and calibrating it may narrow
 *      the accuracy gap). Reading: the calibrated g is the smallest power of
 *      two with amax / (6 g) <= 448, amax = max |x| over the tensor, so that no
 *      block scale saturates and the largest block scales use the top of the
 *      E4M3 range; g = 1 for an all-zero tensor. The tight variant is the
 *      smallest binary32 g with the same property ([EUROK] "Bytes pro Token"
 *      names the global scale an FP32 number).
 *  11. Any finite g > 0 (steps 3, 4 and 6 take g as an FP32 number): every
 *      threshold of steps 3 and 4 is the product of a few-bit constant, an E4M3
 *      value and g, at most 31 significant bits, so it is exact in double, and so
 *      is every dequantized value E2M1 * E4M3 * g. A dense workspace of another
 *      precision holds the nearest value of that precision to the exact product
 *      (nearest, ties to even; one rounding).
 *   9. FP8 baseline ([LMSYS] "Perspective" and "Synopsis" compare NVFP4 KV
 *      against an FP8 KV cache; [EUROK] "Bytes pro Token" gives FP8 one byte
 *      per value). Each value is stored as the E4M3 code of x / s, s the
 *      per-tensor scale of K or V: the nearest E4M3 value, ties to the even
 *      code, saturating at 448, sign of x kept (the rounding of step 3 applied
 *      to |x|, with den = s). It decodes to E4M3(code) * s. Decode attention
 *      over such a cache is step 7 with these rows.
 *
 * Pool layout (the written definition both sides implement independently):
 *   A pool holds num_pages pages; each page holds, for each KV head h, a K slab
 *   then a V slab of 1152 bytes each:  slab(p, h, kind) starts at byte
 *   ((p * Hkv + h) * 2 + kind) * 1152, kind 0 = K, 1 = V. A slab covers the 16
 *   token rows r of the page and the 128 channels d of the head: 1024 code
 *   bytes, then 128 scale bytes. A code's place is a nibble index
 *   2 * byte + (1 for the high nibble):
 *     K code (row r, channel d): byte r*64 + d/2, high nibble iff d is odd
 *     K scale (row r, block j = d/16): byte 1024 + r*8 + j
 *     V code (row r, channel d): byte ((r/4)*16 + d/8)*16 + 2*(d%8) + r%2,
 *                                high nibble iff r%4 >= 2
 *     V scale (row r, block j): byte 1024 + j*16 + r
 *   (a V code byte holds rows r and r+2 of one channel).
 *   Token t of a sequence lives at page page_table[t/16], row t%16.
 *
 * FP8 pool layout (the baseline's written definition): each page holds, for
 * each KV head h, a K slab then a V slab of 2048 bytes each, slab(p, h, kind) at
 * byte ((p * Hkv + h) * 2 + kind) * 2048, one code byte per value:
 *     K (row r, channel d): byte r*128 + d
 *     V (row r, channel d): byte ((r/4)*16 + d/8)*32 + (d%8)*4 + r%4
 *   (a 32-byte V chunk holds channels 8n..8n+7 of rows 4g..4g+3, channel-major).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 128
#define ORC_PAGE 16
#define ORC_SLAB 1152

/* ---- 1. E2M1 decode ---------------------------------------------------- */
double orc_e2m1_value(int code) {
  int sign = (code >> 3) & 1;
  int e = (code >> 1) & 3;
  int m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* ---- 2. E4M3 decode ---------------------------------------------------- */
double orc_e4m3_value(int byte) {
  int sign = (byte >> 7) & 1;
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp(m / 8.0, -6);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Tables of the step-1 and step-2 values, filled once at load time. */
static double orc_e4m3_table[127];
static double orc_e2m1_table[8];
__attribute__((constructor)) static void orc_fill_tables(void) {
  int k;
  for (k = 0; k < 127; ++k) orc_e4m3_table[k] = orc_e4m3_value(k);
  for (k = 0; k < 8; ++k) orc_e2m1_table[k] = orc_e2m1_value(k);
}

/* ---- 3. block scale: nearest E4M3 to amax / den, ties even, satfinite ---- */
/* Walks the 127 non-negative finite E4M3 values upward; the result moves past
 * value k exactly when amax/den lies above the midpoint of k and k+1, or on it
 * with k odd (so that a tie lands on the even code). All products below carry
 * few significant bits and are exact in double. */
int orc_e4m3_nearest_of_quotient(double amax, double den) {
  int k = 0;
  while (k < 126) {
    double mid = 0.5 * (orc_e4m3_table[k] + orc_e4m3_table[k + 1]);
    double thr = den * mid;
    if (amax > thr || (amax == thr && (k & 1)))
      ++k;
    else
      break;
  }
  return k;
}

/* FP8 E4M3 code of a finite value x (the extend path's FP8 workspace): the
 * nearest E4M3 magnitude, ties to the even code, saturating at 448 (the same
 * rounding as a block scale, applied to |x|), with the sign bit of x. */
int orc_e4m3_code_of(double x) {
  int mag = orc_e4m3_nearest_of_quotient(fabs(x), 1.0);
  return (signbit(x) ? 0x80 : 0) | mag;
}

int orc_scale_byte(float amax, float g) {
  return orc_e4m3_nearest_of_quotient((double)amax, 6.0 * (double)g);
}

/* ---- 4. element code: nearest E2M1 to x / D, ties even, saturating -------- */
int orc_e2m1_code(float x, double D) {
  int sign = signbit(x) ? 8 : 0;
  double ax = fabs((double)x);
  int k = 0;
  if (D == 0.0) return sign; /* zero scale: magnitude 0, sign kept */
  while (k < 7) {
    double mid = 0.5 * (orc_e2m1_table[k] + orc_e2m1_table[k + 1]);
    double thr = D * mid;
    if (ax > thr || (ax == thr && (k & 1)))
      ++k;
    else
      break;
  }
  return sign | k;
}

/* ---- 3+4+5: one block of 16 values ------------------------------------ */
void orc_quantize_block16(const float* x, float g, uint8_t* codes8, uint8_t* scale) {
  float amax = 0.0f;
  int i;
  for (i = 0; i < 16; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  int s = orc_scale_byte(amax, g);
  double D = orc_e4m3_value(s) * (double)g;
  for (i = 0; i < 8; ++i) {
    int lo = orc_e2m1_code(x[2 * i], D);
    int hi = orc_e2m1_code(x[2 * i + 1], D);
    codes8[i] = (uint8_t)(lo | (hi << 4));
  }
  *scale = (uint8_t)s;
}

/* ---- 11. one rounding of an exact value to bf16 ------------------------- */
/* Bit pattern of the bfloat16 value nearest to x (8 significant bits), ties to
 * the even significand, sign kept. x is finite and either zero or inside the
 * normal bf16 range, as every dequantized value with g in [2^-64, 2^64] is. The
 * significand is scaled to [128, 256) exactly, rounded to an integer (the
 * default rounding mode rounds half to even), and scaled back. */
uint16_t orc_bf16_bits_of(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  int e;
  float f;
  uint32_t u;
  if (a == 0.0) return sign;
  frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
  f = (float)ldexp(nearbyint(ldexp(a, 8 - e)), e - 8); /* exact: at most 9 significant bits */
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (u >> 16));
}

void orc_bf16_bits_of_array(const double* x, int64_t n, uint16_t* out) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = orc_bf16_bits_of(x[i]);
}

/* ---- pool addressing (written definition, see header) ------------------- */
int64_t orc_slab_offset(int64_t page, int head, int kind, int num_kv_heads) {
  return ((page * num_kv_heads + head) * 2 + kind) * (int64_t)ORC_SLAB;
}
int orc_code_nibble(int kind, int row, int d) {
  int byte, high;
  if (kind == 0) {
    byte = row * 64 + d / 2;
    high = d % 2;
  } else {
    byte = ((row / 4) * 16 + d / 8) * 16 + 2 * (d % 8) + row % 2;
    high = (row % 4) >= 2;
  }
  return 2 * byte + high;
}
int orc_scale_byte_offset(int kind, int row, int block) {
  if (kind == 0) return 1024 + row * 8 + block;
  return 1024 + block * 16 + row;
}
static void orc_put_nibble(uint8_t* slab, int nibble, int code) {
  uint8_t* b = slab + nibble / 2;
  if (nibble % 2) *b = (uint8_t)((*b & 0x0F) | (code << 4));
  else *b = (uint8_t)((*b & 0xF0) | code);
}
static int orc_get_nibble(const uint8_t* slab, int nibble) {
  int b = slab[nibble / 2];
  return (nibble % 2) ? (b >> 4) : (b & 15);
}
int64_t orc_pool_bytes(int64_t num_pages, int num_kv_heads) {
  return num_pages * num_kv_heads * 2 * (int64_t)ORC_SLAB;
}

static float orc_bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Quantize-on-write of T tokens of K and V ([T][Hkv][128], element strides
 * given) into the pool at slot_mapping[t] = page*16 + row (negative = skip).
 * src_dtype 0 = float32, 1 = bfloat16 bits. Pages are spread over n_threads
 * threads (a V code byte holds two rows of a page, so one page has one writer);
 * each token's codes are computed the same way by any thread. */
typedef struct {
  const void *k_src, *v_src;
  int src_dtype;
  int64_t token_stride, head_stride;
  const int32_t* slot_mapping;
  int64_t t_begin, t_end;
  int num_kv_heads;
  float g;
  uint8_t* pool;
  int part, n_parts; /* this worker writes the pages with page % n_parts == part */
} orc_quant_job;

static void* orc_quant_worker(void* arg) {
  orc_quant_job* J = (orc_quant_job*)arg;
  int64_t t;
  int h, kind, j, i;
  for (t = J->t_begin; t < J->t_end; ++t) {
    int32_t slot = J->slot_mapping[t];
    if (slot < 0) continue;
    int64_t page = slot / ORC_PAGE;
    int row = slot % ORC_PAGE;
    if (page % J->n_parts != J->part) continue; /* V bytes are shared by two rows */
    for (h = 0; h < J->num_kv_heads; ++h) {
      for (kind = 0; kind < 2; ++kind) {
        const void* src = kind == 0 ? J->k_src : J->v_src;
        uint8_t* slab = J->pool + orc_slab_offset(page, h, kind, J->num_kv_heads);
        for (j = 0; j < 8; ++j) {
          float x[16];
          uint8_t codes[8], s;
          for (i = 0; i < 16; ++i) {
            int64_t idx = t * J->token_stride + h * J->head_stride + 16 * j + i;
            x[i] = J->src_dtype == 0 ? ((const float*)src)[idx]
                                     : orc_bf16_to_float(((const uint16_t*)src)[idx]);
          }
          orc_quantize_block16(x, J->g, codes, &s);
          for (i = 0; i < 8; ++i) {
            orc_put_nibble(slab, orc_code_nibble(kind, row, 16 * j + 2 * i), codes[i] & 15);
            orc_put_nibble(slab, orc_code_nibble(kind, row, 16 * j + 2 * i + 1), codes[i] >> 4);
          }
          slab[orc_scale_byte_offset(kind, row, j)] = s;
        }
      }
    }
  }
  return NULL;
}

void orc_quantize_to_pool(const void* k_src, const void* v_src, int src_dtype, int64_t token_stride,
                          int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens,
                          int num_kv_heads, float g, uint8_t* pool, int n_threads) {
  orc_quant_job jobs[256];
  pthread_t th[256];
  int i;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  for (i = 0; i < n_threads; ++i) {
    orc_quant_job* J = &jobs[i];
    J->k_src = k_src;
    J->v_src = v_src;
    J->src_dtype = src_dtype;
    J->token_stride = token_stride;
    J->head_stride = head_stride;
    J->slot_mapping = slot_mapping;
    J->t_begin = 0;
    J->t_end = num_tokens;
    J->part = i;
    J->n_parts = n_threads;
    J->num_kv_heads = num_kv_heads;
    J->g = g;
    J->pool = pool;
  }
  if (n_threads == 1) {
    orc_quant_worker(&jobs[0]);
    return;
  }
  for (i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, orc_quant_worker, &jobs[i]);
  for (i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
}

/* ---- 6. dequantize one token row of one head ------------------------------ */
void orc_dequant_row(const uint8_t* pool, int64_t page, int row, int head, int kind,
                     int num_kv_heads, float g, double* out128) {
  const uint8_t* slab = pool + orc_slab_offset(page, head, kind, num_kv_heads);
  int d;
  for (d = 0; d < ORC_D; ++d) {
    int code = orc_get_nibble(slab, orc_code_nibble(kind, row, d));
    int s = slab[orc_scale_byte_offset(kind, row, d / 16)];
    out128[d] = orc_e2m1_value(code) * orc_e4m3_value(s) * (double)g;
  }
}

/* Extend path: dequantize tokens [0, len) of each listed sequence into a dense
 * workspace [row][Hkv][128] (fp64 here), row = cu_rows[s] + t. */
void orc_dequant_workspace(const uint8_t* pool, int num_kv_heads, float g, const int32_t* page_table,
                           int64_t page_table_stride, const int32_t* seq_lens, const int64_t* cu_rows,
                           int n_seqs, double* k_out, double* v_out) {
  int s, h;
  int64_t t;
  for (s = 0; s < n_seqs; ++s)
    for (t = 0; t < seq_lens[s]; ++t) {
      int64_t page = page_table[s * page_table_stride + t / ORC_PAGE];
      int row = (int)(t % ORC_PAGE);
      for (h = 0; h < num_kv_heads; ++h) {
        int64_t o = ((cu_rows[s] + t) * num_kv_heads + h) * ORC_D;
        orc_dequant_row(pool, page, row, h, 0, num_kv_heads, g, k_out + o);
        orc_dequant_row(pool, page, row, h, 1, num_kv_heads, g, v_out + o);
      }
    }
}

/* ---- 7. decode attention over the dequantized cache ----------------------- */
typedef struct {
  const uint16_t* q; /* bf16 bits [B][Hq][128] */
  const int32_t* page_table;
  int64_t page_table_stride;
  const int32_t* seq_lens;
  int batch, num_q_heads, num_kv_heads;
  const uint8_t* pool;
  float g;
  int fp8;                /* 1: the pool is the FP8 baseline (step 9) */
  float k_scale, v_scale; /* its per-tensor scales */
  double sm_scale;
  double* out; /* [B][Hq][128] */
  double* lse; /* [B][Hq] */
  const int32_t* units; /* optional list of (b*Hq + qh) to compute; NULL = all */
  int n_units;
  int next; /* work counter */
  pthread_mutex_t lock;
} orc_attn_job;

void orc_fp8_dequant_row(const uint8_t* pool, int64_t page, int row, int head, int kind, int num_kv_heads,
                         float scale, double* out128);

/* Decoded K (kind 0) or V (kind 1) row of one head for the attention: from the
 * NVFP4 pool (step 6) or the FP8 baseline pool (step 9). */
static void orc_attn_row(const orc_attn_job* J, int64_t page, int row, int h, int kind, double* out) {
  if (J->fp8)
    orc_fp8_dequant_row(J->pool, page, row, h, kind, J->num_kv_heads, kind ? J->v_scale : J->k_scale, out);
  else
    orc_dequant_row(J->pool, page, row, h, kind, J->num_kv_heads, J->g, out);
}

static void orc_attn_one(orc_attn_job* J, int b, int qh) {
  int group = J->num_q_heads / J->num_kv_heads;
  int h = qh / group;
  int64_t L = J->seq_lens[b];
  double q[ORC_D], kd[ORC_D], vd[ORC_D], acc[ORC_D];
  double* out = J->out + ((int64_t)b * J->num_q_heads + qh) * ORC_D;
  double m = -INFINITY, sum = 0.0;
  double* z;
  int64_t t;
  int d;
  for (d = 0; d < ORC_D; ++d) q[d] = (double)orc_bf16_to_float(J->q[((int64_t)b * J->num_q_heads + qh) * ORC_D + d]);
  for (d = 0; d < ORC_D; ++d) acc[d] = 0.0;
  if (L <= 0) { /* empty sequence: output 0, lse -inf (a reading) */
    for (d = 0; d < ORC_D; ++d) out[d] = 0.0;
    if (J->lse) J->lse[(int64_t)b * J->num_q_heads + qh] = -INFINITY;
    return;
  }
  z = (double*)malloc(sizeof(double) * (size_t)L);
  for (t = 0; t < L; ++t) { /* logits */
    int64_t page = J->page_table[b * J->page_table_stride + t / ORC_PAGE];
    double dot = 0.0;
    orc_attn_row(J, page, (int)(t % ORC_PAGE), h, 0, kd);
    for (d = 0; d < ORC_D; ++d) dot += q[d] * kd[d];
    z[t] = J->sm_scale * dot;
    if (z[t] > m) m = z[t];
  }
  for (t = 0; t < L; ++t) { /* weights and weighted sum of values */
    int64_t page = J->page_table[b * J->page_table_stride + t / ORC_PAGE];
    double w = exp(z[t] - m);
    orc_attn_row(J, page, (int)(t % ORC_PAGE), h, 1, vd);
    sum += w;
    for (d = 0; d < ORC_D; ++d) acc[d] += w * vd[d];
  }
  for (d = 0; d < ORC_D; ++d) out[d] = acc[d] / sum;
  if (J->lse) J->lse[(int64_t)b * J->num_q_heads + qh] = m + log(sum);
  free(z);
}

static void* orc_attn_worker(void* arg) {
  orc_attn_job* J = (orc_attn_job*)arg;
  for (;;) {
    int u;
    pthread_mutex_lock(&J->lock);
    u = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (u >= J->n_units) break;
    {
      int unit = J->units ? J->units[u] : u;
      orc_attn_one(J, unit / J->num_q_heads, unit % J->num_q_heads);
    }
  }
  return NULL;
}

/* Computes out/lse for the listed (b*Hq + qh) units (all when units == NULL),
 * spreading whole units over n_threads threads; the arithmetic of a unit does
 * not depend on the thread count. */
static void orc_attn_run(const uint16_t* q_bf16, const int32_t* page_table, int64_t page_table_stride,
                         const int32_t* seq_lens, int batch, int num_q_heads, int num_kv_heads,
                         const uint8_t* pool, float g, int fp8, float k_scale, float v_scale, double sm_scale,
                         double* out, double* lse, const int32_t* units, int n_units, int n_threads) {
  orc_attn_job J;
  pthread_t th[256];
  int i;
  J.q = q_bf16;
  J.page_table = page_table;
  J.page_table_stride = page_table_stride;
  J.seq_lens = seq_lens;
  J.batch = batch;
  J.num_q_heads = num_q_heads;
  J.num_kv_heads = num_kv_heads;
  J.pool = pool;
  J.g = g;
  J.fp8 = fp8;
  J.k_scale = k_scale;
  J.v_scale = v_scale;
  J.sm_scale = sm_scale;
  J.out = out;
  J.lse = lse;
  J.units = units;
  J.n_units = units ? n_units : batch * num_q_heads;
  J.next = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (n_threads == 1) {
    orc_attn_worker(&J);
  } else {
    for (i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, orc_attn_worker, &J);
    for (i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
  }
  pthread_mutex_destroy(&J.lock);
}

void orc_decode_attn(const uint16_t* q_bf16, const int32_t* page_table, int64_t page_table_stride,
                     const int32_t* seq_lens, int batch, int num_q_heads, int num_kv_heads,
                     const uint8_t* pool, float g, double sm_scale, double* out, double* lse,
                     const int32_t* units, int n_units, int n_threads) {
  orc_attn_run(q_bf16, page_table, page_table_stride, seq_lens, batch, num_q_heads, num_kv_heads, pool, g, 0, 1.0f,
               1.0f, sm_scale, out, lse, units, n_units, n_threads);
}

/* Decode attention over the FP8 baseline pool (steps 7 and 9). */
void orc_fp8_decode_attn(const uint16_t* q_bf16, const int32_t* page_table, int64_t page_table_stride,
                         const int32_t* seq_lens, int batch, int num_q_heads, int num_kv_heads,
                         const uint8_t* pool, float k_scale, float v_scale, double sm_scale, double* out,
                         double* lse, const int32_t* units, int n_units, int n_threads) {
  orc_attn_run(q_bf16, page_table, page_table_stride, seq_lens, batch, num_q_heads, num_kv_heads, pool, 1.0f, 1,
               k_scale, v_scale, sm_scale, out, lse, units, n_units, n_threads);
}


/* ---- 8. extend attention: prefix workspace + causal chunk ---------------- */
/* Value of element idx of a workspace stored as dtype 0 = f32, 1 = bf16 bits,
 * 2 = FP8 E4M3 bytes (the three dtypes the extend dequant writes). */
static double orc_ws_value(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  if (dtype == 1) return (double)orc_bf16_to_float(((const uint16_t*)base)[idx]);
  return orc_e4m3_value(((const uint8_t*)base)[idx]);
}

typedef struct {
  const uint16_t* q;                 /* bf16 bits [C][Hq][128] */
  const void *k_pre, *v_pre;         /* [P][Hkv][128] of pre_dtype */
  int pre_dtype;
  int64_t prefix_len;
  const uint16_t *k_chunk, *v_chunk; /* bf16 bits [C][Hkv][128] */
  int64_t chunk_len;
  int num_q_heads, num_kv_heads;
  double sm_scale;
  double* out; /* [C][Hq][128] */
  double* lse; /* [C][Hq] */
  const int64_t* units; /* optional list of (i*Hq + qh); NULL = all */
  int64_t n_units;
  int64_t next;
  pthread_mutex_t lock;
} orc_ext_job;

/* Key (kind 0) or value (kind 1) channel d of visible row t of KV head h:
 * rows [0, P) are the prefix workspace, rows P + j chunk row j. */
static double orc_ext_kv(const orc_ext_job* J, int kind, int64_t t, int h, int d) {
  if (t < J->prefix_len)
    return orc_ws_value(kind ? J->v_pre : J->k_pre, J->pre_dtype, (t * J->num_kv_heads + h) * ORC_D + d);
  {
    const uint16_t* c = kind ? J->v_chunk : J->k_chunk;
    return (double)orc_bf16_to_float(c[((t - J->prefix_len) * J->num_kv_heads + h) * ORC_D + d]);
  }
}

static void orc_ext_one(orc_ext_job* J, int64_t i, int qh) {
  int group = J->num_q_heads / J->num_kv_heads;
  int h = qh / group;
  int64_t n_vis = J->prefix_len + i + 1; /* causal: chunk rows 0..i */
  double q[ORC_D], acc[ORC_D];
  double m = -INFINITY, sum = 0.0;
  double* z = (double*)malloc(sizeof(double) * (size_t)n_vis);
  double* out = J->out + (i * J->num_q_heads + qh) * ORC_D;
  int64_t t;
  int d;
  for (d = 0; d < ORC_D; ++d) q[d] = (double)orc_bf16_to_float(J->q[(i * J->num_q_heads + qh) * ORC_D + d]);
  for (d = 0; d < ORC_D; ++d) acc[d] = 0.0;
  for (t = 0; t < n_vis; ++t) { /* logits */
    double dot = 0.0;
    for (d = 0; d < ORC_D; ++d) dot += q[d] * orc_ext_kv(J, 0, t, h, d);
    z[t] = J->sm_scale * dot;
    if (z[t] > m) m = z[t];
  }
  for (t = 0; t < n_vis; ++t) { /* weights and weighted sum of values */
    double w = exp(z[t] - m);
    sum += w;
    for (d = 0; d < ORC_D; ++d) acc[d] += w * orc_ext_kv(J, 1, t, h, d);
  }
  for (d = 0; d < ORC_D; ++d) out[d] = acc[d] / sum;
  if (J->lse) J->lse[i * J->num_q_heads + qh] = m + log(sum);
  free(z);
}

static void* orc_ext_worker(void* arg) {
  orc_ext_job* J = (orc_ext_job*)arg;
  for (;;) {
    int64_t u;
    pthread_mutex_lock(&J->lock);
    u = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (u >= J->n_units) break;
    {
      int64_t unit = J->units ? J->units[u] : u;
      orc_ext_one(J, unit / J->num_q_heads, (int)(unit % J->num_q_heads));
    }
  }
  return NULL;
}

/* Computes out/lse for the listed (i*Hq + qh) units (all when units == NULL)
 * over n_threads threads; a unit's arithmetic does not depend on the thread. */
void orc_extend_attn(const uint16_t* q_bf16, const void* k_pre, const void* v_pre, int pre_dtype,
                     int64_t prefix_len, const uint16_t* k_chunk, const uint16_t* v_chunk, int64_t chunk_len,
                     int num_q_heads, int num_kv_heads, double sm_scale, double* out, double* lse,
                     const int64_t* units, int64_t n_units, int n_threads) {
  orc_ext_job J;
  pthread_t th[256];
  int i;
  J.q = q_bf16;
  J.k_pre = k_pre;
  J.v_pre = v_pre;
  J.pre_dtype = pre_dtype;
  J.prefix_len = prefix_len;
  J.k_chunk = k_chunk;
  J.v_chunk = v_chunk;
  J.chunk_len = chunk_len;
  J.num_q_heads = num_q_heads;
  J.num_kv_heads = num_kv_heads;
  J.sm_scale = sm_scale;
  J.out = out;
  J.lse = lse;
  J.units = units;
  J.n_units = units ? n_units : chunk_len * num_q_heads;
  J.next = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (n_threads == 1) {
    orc_ext_worker(&J);
  } else {
    for (i = 0; i < n_threads; ++i) pthread_create(&th[i], NULL, orc_ext_worker, &J);
    for (i = 0; i < n_threads; ++i) pthread_join(th[i], NULL);
  }
  pthread_mutex_destroy(&J.lock);
}


/* ---- 9. FP8 baseline: pool layout, quantize-on-write, row decode ---------- */
#define ORC_FP8_SLAB 2048

int64_t orc_fp8_slab_offset(int64_t page, int head, int kind, int num_kv_heads) {
  return ((page * num_kv_heads + head) * 2 + kind) * (int64_t)ORC_FP8_SLAB;
}

int orc_fp8_byte_offset(int kind, int row, int d) {
  if (kind == 0) return row * 128 + d;
  return ((row / 4) * 16 + d / 8) * 32 + (d % 8) * 4 + row % 4;
}

int64_t orc_fp8_pool_bytes(int64_t num_pages, int num_kv_heads) {
  return num_pages * num_kv_heads * 2 * (int64_t)ORC_FP8_SLAB;
}

/* E4M3 code of x / s: nearest E4M3 magnitude of |x| / s (exact comparisons of
 * |x| against s times each midpoint), ties to the even code, saturating at 448,
 * sign of x. */
int orc_fp8_code(float x, float s) {
  int mag = orc_e4m3_nearest_of_quotient(fabs((double)x), (double)s);
  return (signbit(x) ? 0x80 : 0) | mag;
}

/* Quantize-on-write of T tokens of K and V ([T][Hkv][128], element strides
 * given) into the FP8 pool at slot_mapping[t] = page*16 + row (negative = skip).
 * src_dtype 0 = float32, 1 = bfloat16 bits. Every byte belongs to one (token,
 * head, channel), so write order does not matter. */
void orc_fp8_quantize_to_pool(const void* k_src, const void* v_src, int src_dtype, int64_t token_stride,
                              int64_t head_stride, const int32_t* slot_mapping, int64_t num_tokens,
                              int num_kv_heads, float k_scale, float v_scale, uint8_t* pool) {
  int64_t t;
  int h, kind, d;
  for (t = 0; t < num_tokens; ++t) {
    int32_t slot = slot_mapping[t];
    if (slot < 0) continue;
    for (h = 0; h < num_kv_heads; ++h)
      for (kind = 0; kind < 2; ++kind) {
        const void* src = kind == 0 ? k_src : v_src;
        uint8_t* slab = pool + orc_fp8_slab_offset(slot / ORC_PAGE, h, kind, num_kv_heads);
        for (d = 0; d < ORC_D; ++d) {
          int64_t idx = t * token_stride + h * head_stride + d;
          float x = src_dtype == 0 ? ((const float*)src)[idx] : orc_bf16_to_float(((const uint16_t*)src)[idx]);
          slab[orc_fp8_byte_offset(kind, slot % ORC_PAGE, d)] = (uint8_t)orc_fp8_code(x, kind ? v_scale : k_scale);
        }
      }
  }
}

/* Decoded K (kind 0) or V (kind 1) row of one head: E4M3(code) * scale. */
void orc_fp8_dequant_row(const uint8_t* pool, int64_t page, int row, int head, int kind, int num_kv_heads,
                         float scale, double* out128) {
  const uint8_t* slab = pool + orc_fp8_slab_offset(page, head, kind, num_kv_heads);
  int d;
  for (d = 0; d < ORC_D; ++d) out128[d] = orc_e4m3_value(slab[orc_fp8_byte_offset(kind, row, d)]) * (double)scale;
}


/* ---- 10. global-scale calibration -------------------------------------- */
/* max |x| over T tokens x H heads x 128 channels (element strides given);
 * src_dtype 0 = float32, 1 = bfloat16 bits. */
double orc_amax(const void* src, int src_dtype, int64_t token_stride, int64_t head_stride, int64_t num_tokens,
                int num_heads) {
  double m = 0.0;
  int64_t t;
  int h, d;
  for (t = 0; t < num_tokens; ++t)
    for (h = 0; h < num_heads; ++h)
      for (d = 0; d < ORC_D; ++d) {
        int64_t idx = t * token_stride + h * head_stride + d;
        double x = src_dtype == 0 ? (double)((const float*)src)[idx]
                                  : (double)orc_bf16_to_float(((const uint16_t*)src)[idx]);
        if (fabs(x) > m) m = fabs(x);
      }
  return m;
}

/* Smallest binary32 g with amax / (6 g) <= 448, i.e. amax <= 2688 g (a product
 * of at most 29 significant bits, exact in double); g = 1 for amax = 0. Starts
 * from a float near amax / 2688 and steps one binary32 value at a time. */
float orc_global_scale_tight_for_amax(double amax) {
  float g;
  if (amax <= 0.0) return 1.0f;
  g = (float)(amax / 2688.0);
  while (!(amax <= 2688.0 * (double)g)) g = nextafterf(g, INFINITY);
  while (g > 0.0f && amax <= 2688.0 * (double)nextafterf(g, 0.0f)) g = nextafterf(g, 0.0f);
  return g;
}

/* Smallest power of two g with amax / (6 g) <= 448 (g = 1 for amax = 0). */
double orc_global_scale_for_amax(double amax) {
  double g = 1.0;
  if (amax <= 0.0) return 1.0;
  while (amax / (6.0 * g) > 448.0) g *= 2.0;
  while (amax / (6.0 * (g / 2.0)) <= 448.0) g /= 2.0;
  return g;
}
