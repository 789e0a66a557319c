/*
 * Plain fp64 CPU oracle for paged KV-cache decode.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the GPU library: every layout formula below
 * is written out again from its definition.
 *
 * What it computes, and where the pages define it:
 *  - KV bytes per token = 2 * layers * kv_heads * head_dim * bytes_per_element
 *    (ssdnodes.com, "KV cache vs prompt cache", section "How much memory does
 *    the KV cache use?", the bytes-per-token formula; the 2 counts K and V).
 *  - Each sequence's cache is cut into fixed blocks (default 16 tokens) that
 *    need not be adjacent; a per-sequence block table maps logical block ->
 *    physical block (ahmedhaies.com, "PagedAttention: why LLM serving wastes
 *    most GPU memory", section "The solution: borrow virtual memory from the
 *    OS"; thienlv.com, "PagedAttention là gì?", section "How does
 *    PagedAttention work?").
 *  - A decode step appends the new token's key/value to the cache and reads
 *    the whole cache to attend (news.hamidun.com glossary "KV-Cache", the
 *    prefill/decode paragraph); the new query attends to all previous keys and
 *    values (same page, the mechanism paragraph).
 *  - With grouped-query attention several query heads share one stored K/V
 *    head (ssdnodes.com, same section, the GQA paragraph); query head h reads
 *    kv head h / (q_heads / kv_heads).
 *
 *  - Quantised caches: q8_0 and q4_0 (ssdnodes.com, same page, "Four ways to
 *    make the KV cache smaller", item 2), read as llama.cpp's Q8_0 / Q4_0
 *    block formats: per 32 consecutive head_dim elements one fp16 scale and
 *    32 int8 codes / 32 4-bit codes.
 *
 * Physical layout of one layer of the pool (our choice; the pages fix only
 * "blocks of block_size tokens" and "a block table"): K and V are separate
 * arrays, each indexed [block][kv_head][row][d] in row-major order, where row
 * is the token's position inside its block.
 *
 * Numbers are read exactly from their stored type (fp32, fp16, bf16, or a
 * q8_0 / q4_0 code times its fp16 scale) into double; all attention arithmetic is
 * double. (Quantising a new q8_0 row makes its integer decisions in fp32, as
 * the format's definition does.) No blocking, no online softmax, no split:
 * gather to a contiguous array, then softmax(q.K^T * scale) . V.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_Q8_0 = 3, ORC_Q4_0 = 4 };

static int orc_quantised(int dtype) { return dtype == ORC_Q8_0 || dtype == ORC_Q4_0; }

static size_t orc_elem_bytes(int dtype) { return dtype == ORC_F32 ? 4u : 2u; }

/* IEEE-754 binary16 -> double, from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double orc_half_bits_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int fr = h & 0x3ff;
  double v;
  if (ex == 0) {
    v = ldexp((double)fr, -24); /* subnormal: fr * 2^-14 * 2^-10 */
  } else if (ex == 31) {
    v = fr ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + fr), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double orc_bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double orc_load(const void* base, size_t idx, int dtype) {
  if (dtype == ORC_F32) {
    float f;
    memcpy(&f, (const char*)base + idx * 4u, 4);
    return (double)f;
  }
  uint16_t b;
  memcpy(&b, (const char*)base + idx * 2u, 2);
  return dtype == ORC_F16 ? orc_half_bits_to_double(b) : orc_bf16_bits_to_double(b);
}

/* Exposed so the tests can check the conversions against library routines. */
double orc_elem_to_double(const void* base, int64_t idx, int dtype) {
  return orc_load(base, (size_t)idx, dtype);
}

/*
 * IEEE-754 binary32 value -> binary16 bits, rounded to nearest with ties to
 * even, from the format's definition: the value is scaled by a power of two
 * (exact in double) so that the kept bits are the integer part, and rint()
 * (default rounding mode) rounds it. Overflow gives infinity.
 */
static uint16_t orc_float_to_half_bits(float f) {
  uint16_t sign = signbit(f) ? 0x8000u : 0u;
  if (isnan(f)) return sign | 0x7e00u;
  if (isinf(f)) return sign | 0x7c00u;
  double a = fabs((double)f);
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: a multiple of 2^-24; 1024 units is the smallest normal */
    return sign | (uint16_t)rint(ldexp(a, 24));
  }
  int E;
  frexp(a, &E); /* a = m * 2^E, m in [0.5, 1): a = 1.f * 2^(E-1) */
  int ex = E - 1;
  int units = (int)rint(ldexp(a, 10 - ex)); /* 1.f in units of 2^-10: [1024, 2048] */
  int field = ex + 15;
  if (units == 2048) {
    units = 1024;
    ++field;
  }
  if (field >= 31) return sign | 0x7c00u;
  return sign | (uint16_t)(field << 10) | (uint16_t)(units - 1024);
}

void orc_float_to_half(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_float_to_half_bits(x[i]);
}

/*
 * q8_0 quantisation of one group of 32 consecutive values. ssdnodes.com,
 * "KV cache vs prompt cache", "Four ways to make the KV cache smaller" (item
 * 2) and its FAQ name q8_0 as the cache type that about halves the memory of
 * an f16 cache; its definition is llama.cpp's Q8_0 block: one scale
 * d = max|x| / 127 stored as fp16 and 32 int8 codes round(x / d) (rounding
 * half away from zero, x / d taken as x * (1 / d)), value = d * code. The
 * integer decisions are made in fp32, as that definition does; the codes use
 * the fp32 scale, the stored scale is its fp16 rounding.
 */
static void orc_q8_quantize_group(const float* x, int8_t* codes, uint16_t* d_bits) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 127.0f;
  float id = d != 0.0f ? 1.0f / d : 0.0f;
  for (int i = 0; i < 32; ++i) codes[i] = (int8_t)roundf(x[i] * id);
  *d_bits = orc_float_to_half_bits(d);
}

void orc_q8_quantize(const float* x, int64_t n_groups, int8_t* codes, uint16_t* d_bits) {
  for (int64_t g = 0; g < n_groups; ++g) orc_q8_quantize_group(x + 32 * g, codes + 32 * g, d_bits + g);
}

/*
 * q4_0 quantisation of one group of 32 consecutive values. The same page
 * ("Four ways to make the KV cache smaller", item 2, and the FAQ) names q4_0
 * as the cache type that takes about a quarter of an f16 cache; its
 * definition is llama.cpp's Q4_0 block: m = the value of largest magnitude
 * (the first one on ties), scale d = m / -8 stored as fp16, 4-bit codes
 * q = min(15, trunc(x * (1 / d) + 8.5)), value = (q - 8) * d. Decisions in
 * fp32 (the product and the sum rounded separately), codes from the fp32
 * scale.
 */
static void orc_q4_quantize_group(const float* x, uint8_t* q, uint16_t* d_bits) {
  float amax = 0.0f, m = 0.0f;
  for (int i = 0; i < 32; ++i) {
    if (amax < fabsf(x[i])) {
      amax = fabsf(x[i]);
      m = x[i];
    }
  }
  float d = m / -8.0f;
  float id = d != 0.0f ? 1.0f / d : 0.0f;
  for (int i = 0; i < 32; ++i) {
    float t = x[i] * id;
    t = t + 8.5f;
    int c = (int)(int8_t)t;
    q[i] = (uint8_t)(c < 15 ? c : 15);
  }
  *d_bits = orc_float_to_half_bits(d);
}

void orc_q4_quantize(const float* x, int64_t n_groups, uint8_t* codes, uint16_t* d_bits) {
  for (int64_t g = 0; g < n_groups; ++g) orc_q4_quantize_group(x + 32 * g, codes + 32 * g, d_bits + g);
}

/*
 * Quantised tile of one (block, kv head) in the pool (our layout; the pages fix
 * none): block_size rows of codes, then block_size x head_dim/32 fp16 scales,
 * ordered [row][group] in the K region and [group][row] in the V region.
 * q8_0: the int8 codes in the order the decode's lanes read them. Rows are
 * taken R = min(block_size, 16) at a time (u = r / R, rr = r % R); element d
 * is code j = d % 8 of chunk w = d / 8 (P = head_dim / 8 chunks per row,
 * NV = P / 4); with group k and quarter q of w = 4k + q:
 *   K region: u*R*D + (k/2)*R*64 + (q*R + rr)*16 + (k%2)*8 + j
 *   V region: u*R*D + ((rr%NV)/2)*R*64 + ((rr/NV)*P + w)*16 + (rr%2)*8 + j
 * (one 16-byte unit holds a token's chunks of two groups in K, and one
 * chunk of two consecutive rows in V).
 * q4_0: a word is 4 bytes holding 8 consecutive elements of a row (element j of
 * the word in byte j/2, low nibble for even j); with G = head_dim/32 groups and
 * CB = head_dim/2 code bytes per row, word w = 4k + q of row r (group k,
 * quarter q) lies at byte
 *   K region: r*CB + 4*(q*G + k)                     (words transposed in the row)
 *   V region: (r - r%G)*CB + 4*(w*G + r%G)           (rows interleaved by G)
 * so that one reader's share of a tile (the G words of one quarter of a K row,
 * or one word of G consecutive V rows) is one contiguous run.
 */
static size_t orc_code_row_bytes(int dtype, int head_dim) {
  return dtype == ORC_Q4_0 ? (size_t)head_dim / 2 : (size_t)head_dim;
}

static size_t orc_qtile_bytes(int dtype, int block_size, int head_dim) {
  return (size_t)block_size * orc_code_row_bytes(dtype, head_dim) +
         (size_t)block_size * (head_dim / 32) * 2;
}

static size_t orc_q8_code_offset(int is_v, int row, int d, int block_size, int head_dim) {
  const size_t D = (size_t)head_dim, P = D / 8, NV = P / 4;
  const size_t R = block_size < 16 ? (size_t)block_size : 16;
  const size_t u = (size_t)row / R, rr = (size_t)row % R, w = (size_t)d / 8, j = (size_t)d % 8;
  if (is_v) return u * R * D + ((rr % NV) / 2) * R * 64 + ((rr / NV) * P + w) * 16 + (rr % 2) * 8 + j;
  const size_t k = w / 4, q = w % 4;
  return u * R * D + (k / 2) * R * 64 + (q * R + rr) * 16 + (k % 2) * 8 + j;
}

static size_t orc_q4_word_offset(int is_v, int row, int word, int head_dim) {
  const size_t G = (size_t)head_dim / 32, CB = (size_t)head_dim / 2;
  if (is_v) return ((size_t)row - (size_t)row % G) * CB + 4 * ((size_t)word * G + (size_t)row % G);
  return (size_t)row * CB + 4 * ((size_t)(word % 4) * G + (size_t)(word / 4));
}

static size_t orc_qscale_offset(int dtype, int is_v, int row, int grp, int block_size,
                                int head_dim) {
  size_t codes = (size_t)block_size * orc_code_row_bytes(dtype, head_dim);
  int ng = head_dim / 32;
  return codes + 2 * (size_t)(is_v ? grp * block_size + row : row * ng + grp);
}

/* Value of element d of row `row` in a quantised tile, exact in double:
 * q8_0 scale * code, q4_0 scale * (nibble - 8). */
static double orc_qload(const char* tile, int dtype, int is_v, int row, int d, int block_size,
                        int head_dim) {
  uint16_t h;
  memcpy(&h, tile + orc_qscale_offset(dtype, is_v, row, d / 32, block_size, head_dim), 2);
  double code;
  if (dtype == ORC_Q4_0) {
    uint8_t b;
    memcpy(&b, tile + orc_q4_word_offset(is_v, row, d / 8, head_dim) + (d % 8) / 2, 1);
    code = (double)((d & 1 ? b >> 4 : b & 15) - 8);
  } else {
    int8_t c;
    memcpy(&c, tile + orc_q8_code_offset(is_v, row, d, block_size, head_dim), 1);
    code = (double)c;
  }
  return orc_half_bits_to_double(h) * code;
}

/* ssdnodes.com, "KV cache vs prompt cache", "How much memory does the KV cache
 * use?": bytes per token = 2 * layers * kv_heads * head_dim * bytes/element. */
/* Thread count of the OpenMP loops below (timing runs only; results do not
 * depend on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

int64_t orc_kv_bytes_per_token(int64_t layers, int64_t kv_heads, int64_t head_dim,
                               int64_t bytes_per_elem) {
  return 2 * layers * kv_heads * head_dim * bytes_per_elem;
}

/* Element index of (block, kv_head, row, d) in one layer's K (or V) array. */
static size_t orc_pool_index(int64_t block, int64_t head, int64_t row, int64_t d,
                             int kv_heads, int block_size, int head_dim) {
  return (size_t)((((block * kv_heads) + head) * block_size + row) * head_dim + d);
}

/*
 * Append (news.hamidun.com "KV-Cache", prefill/decode paragraph: each decode
 * step appends the new token's key/value entry to the cache).
 * For sequence s with context length L (the new token included), the new
 * token is logical position p = L - 1; it lives in physical block
 * block_table[s][p / block_size] at row p % block_size. Writes k_new[s][g][:]
 * and v_new[s][g][:] there for every kv head g. Bytes are copied unchanged.
 * Sequences with L <= 0 are skipped.
 */
void orc_append(int batch, int kv_heads, int head_dim, int block_size, int dtype,
                void* k_pool, void* v_pool, const int32_t* block_table, int max_blocks,
                const int32_t* ctx_lens, const void* k_new, const void* v_new) {
  size_t eb = orc_elem_bytes(dtype);
  for (int s = 0; s < batch; ++s) {
    int L = ctx_lens[s];
    if (L <= 0) continue;
    int p = L - 1;
    int32_t blk = block_table[(size_t)s * max_blocks + p / block_size];
    int row = p % block_size;
    if (orc_quantised(dtype)) {
      /* new rows arrive in bf16 and are quantised group by group */
      size_t tb = orc_qtile_bytes(dtype, block_size, head_dim);
      for (int g = 0; g < kv_heads; ++g) {
        for (int is_v = 0; is_v < 2; ++is_v) {
          const void* src = is_v ? v_new : k_new;
          char* tile = (char*)(is_v ? v_pool : k_pool) + ((size_t)blk * kv_heads + g) * tb;
          for (int grp = 0; grp < head_dim / 32; ++grp) {
            float x[32];
            for (int i = 0; i < 32; ++i)
              x[i] = (float)orc_load(src, ((size_t)s * kv_heads + g) * head_dim + grp * 32 + i,
                                     ORC_BF16);
            uint16_t d;
            if (dtype == ORC_Q4_0) {
              uint8_t q[32], packed[16];
              orc_q4_quantize_group(x, q, &d);
              for (int i = 0; i < 16; ++i) packed[i] = (uint8_t)(q[2 * i] | (q[2 * i + 1] << 4));
              for (int w = 0; w < 4; ++w)  /* the group's four words */
                memcpy(tile + orc_q4_word_offset(is_v, row, 4 * grp + w, head_dim),
                       packed + 4 * w, 4);
            } else {
              int8_t codes[32];
              orc_q8_quantize_group(x, codes, &d);
              for (int i = 0; i < 32; ++i)
                memcpy(tile + orc_q8_code_offset(is_v, row, grp * 32 + i, block_size, head_dim),
                       codes + i, 1);
            }
            memcpy(tile + orc_qscale_offset(dtype, is_v, row, grp, block_size, head_dim), &d, 2);
          }
        }
      }
      continue;
    }
    for (int g = 0; g < kv_heads; ++g) {
      size_t dst = orc_pool_index(blk, g, row, 0, kv_heads, block_size, head_dim) * eb;
      size_t src = ((size_t)s * kv_heads + g) * head_dim * eb;
      memcpy((char*)k_pool + dst, (const char*)k_new + src, head_dim * eb);
      memcpy((char*)v_pool + dst, (const char*)v_new + src, head_dim * eb);
    }
  }
}

/*
 * Gather one sequence's first n_tokens K and V rows of kv head g into
 * contiguous double arrays out_k[t][d], out_v[t][d]: logical token t sits in
 * physical block block_table[s][t / block_size], row t % block_size.
 */
void orc_gather(int kv_heads, int head_dim, int block_size, int dtype, const void* k_pool,
                const void* v_pool, const int32_t* bt_row, int n_tokens, int g, double* out_k,
                double* out_v) {
  for (int t = 0; t < n_tokens; ++t) {
    int32_t blk = bt_row[t / block_size];
    int row = t % block_size;
    if (orc_quantised(dtype)) {
      size_t off = ((size_t)blk * kv_heads + g) * orc_qtile_bytes(dtype, block_size, head_dim);
      for (int d = 0; d < head_dim; ++d) {
        out_k[(size_t)t * head_dim + d] =
            orc_qload((const char*)k_pool + off, dtype, 0, row, d, block_size, head_dim);
        out_v[(size_t)t * head_dim + d] =
            orc_qload((const char*)v_pool + off, dtype, 1, row, d, block_size, head_dim);
      }
      continue;
    }
    for (int d = 0; d < head_dim; ++d) {
      size_t i = orc_pool_index(blk, g, row, d, kv_heads, block_size, head_dim);
      out_k[(size_t)t * head_dim + d] = orc_load(k_pool, i, dtype);
      out_v[(size_t)t * head_dim + d] = orc_load(v_pool, i, dtype);
    }
  }
}

/*
 * Softmax attention of one query vector over n contiguous K/V rows, in fp64:
 *   z_t = scale * sum_d q[d] * K[t][d]
 *   p_t = exp(z_t - max z) / sum_u exp(z_u - max z)
 *   out[d] = sum_t p_t * V[t][d]
 */
void orc_attend(int n, int head_dim, const double* q, const double* kc, const double* vc,
                double scale, double* out) {
  double* z = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double mx = -INFINITY;
  for (int t = 0; t < n; ++t) {
    double acc = 0.0;
    for (int d = 0; d < head_dim; ++d) acc += q[d] * kc[(size_t)t * head_dim + d];
    z[t] = scale * acc;
    if (z[t] > mx) mx = z[t];
  }
  double den = 0.0;
  for (int t = 0; t < n; ++t) {
    z[t] = exp(z[t] - mx);
    den += z[t];
  }
  for (int d = 0; d < head_dim; ++d) out[d] = 0.0;
  for (int t = 0; t < n; ++t) {
    double p = z[t] / den;
    for (int d = 0; d < head_dim; ++d) out[d] += p * vc[(size_t)t * head_dim + d];
  }
  free(z);
}

/*
 * Decode attention for a batch, reading the cache through the block tables:
 * for every sequence s and query head h, gather the first ctx_lens[s] rows of
 * kv head h / (q_heads / kv_heads) and attend with q[s][h].
 * q is stored in the cache dtype (bf16 for a quantised cache),
 * [batch][q_heads][head_dim]; out is double
 * [batch][q_heads][head_dim]. Parallel over (sequence, kv head) with OpenMP.
 */
void orc_decode(int batch, int q_heads, int kv_heads, int head_dim, int block_size, int dtype,
                const void* k_pool, const void* v_pool, const int32_t* block_table,
                int max_blocks, const int32_t* ctx_lens, const void* q, double scale,
                double* out) {
  int group = q_heads / kv_heads;
  int npairs = batch * kv_heads;
  int qdt = orc_quantised(dtype) ? ORC_BF16 : dtype; /* q of a quantised cache is bf16 */
#pragma omp parallel for schedule(dynamic, 1)
  for (int pi = 0; pi < npairs; ++pi) {
    int s = pi / kv_heads;
    int g = pi % kv_heads;
    int L = ctx_lens[s];
    size_t n = (size_t)(L > 0 ? L : 1) * head_dim;
    double* kc = (double*)malloc(sizeof(double) * n);
    double* vc = (double*)malloc(sizeof(double) * n);
    double* qd = (double*)malloc(sizeof(double) * head_dim);
    orc_gather(kv_heads, head_dim, block_size, dtype, k_pool, v_pool,
               block_table + (size_t)s * max_blocks, L, g, kc, vc);
    for (int h = g * group; h < (g + 1) * group; ++h) {
      for (int d = 0; d < head_dim; ++d)
        qd[d] = orc_load(q, ((size_t)s * q_heads + h) * head_dim + d, qdt);
      orc_attend(L, head_dim, qd, kc, vc, scale, out + ((size_t)s * q_heads + h) * head_dim);
    }
    free(kc);
    free(vc);
    free(qd);
  }
}

/*
 * The same decode computed as independent partitions of part_tokens tokens
 * (partition i covers tokens [i*part_tokens, min(L, (i+1)*part_tokens))),
 * each reduced to (m_i = max logit, l_i = sum exp(z - m_i),
 * o_i = sum exp(z - m_i) * V), then merged with M = max_i m_i:
 *   out = sum_i exp(m_i - M) o_i / sum_i exp(m_i - M) l_i.
 * The merge is an exact identity of softmax, so in exact arithmetic this
 * equals orc_decode; the tests hold the two together to ~1e-12.
 */
void orc_decode_partitioned(int batch, int q_heads, int kv_heads, int head_dim, int block_size,
                            int dtype, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int max_blocks, const int32_t* ctx_lens,
                            const void* q, double scale, int part_tokens, double* out) {
  int group = q_heads / kv_heads;
  int npairs = batch * q_heads;
#pragma omp parallel for schedule(dynamic, 1)
  for (int pi = 0; pi < npairs; ++pi) {
    int s = pi / q_heads;
    int h = pi % q_heads;
    int g = h / group;
    int L = ctx_lens[s];
    size_t n = (size_t)(L > 0 ? L : 1) * head_dim;
    double* kc = (double*)malloc(sizeof(double) * n);
    double* vc = (double*)malloc(sizeof(double) * n);
    double* qd = (double*)malloc(sizeof(double) * head_dim);
    double* oi = (double*)malloc(sizeof(double) * head_dim);
    double* acc = out + ((size_t)s * q_heads + h) * head_dim;
    orc_gather(kv_heads, head_dim, block_size, dtype, k_pool, v_pool,
               block_table + (size_t)s * max_blocks, L, g, kc, vc);
    for (int d = 0; d < head_dim; ++d)
      qd[d] = orc_load(q, ((size_t)s * q_heads + h) * head_dim + d,
                       orc_quantised(dtype) ? ORC_BF16 : dtype);
    int nparts = (L + part_tokens - 1) / part_tokens;
    double* m = (double*)malloc(sizeof(double) * (size_t)(nparts > 0 ? nparts : 1));
    double* l = (double*)malloc(sizeof(double) * (size_t)(nparts > 0 ? nparts : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)(nparts > 0 ? nparts : 1) * head_dim);
    for (int i = 0; i < nparts; ++i) {
      int t0 = i * part_tokens;
      int t1 = t0 + part_tokens < L ? t0 + part_tokens : L;
      double mi = -INFINITY;
      for (int t = t0; t < t1; ++t) {
        double z = 0.0;
        for (int d = 0; d < head_dim; ++d) z += qd[d] * kc[(size_t)t * head_dim + d];
        z *= scale;
        if (z > mi) mi = z;
      }
      double li = 0.0;
      for (int d = 0; d < head_dim; ++d) oi[d] = 0.0;
      for (int t = t0; t < t1; ++t) {
        double z = 0.0;
        for (int d = 0; d < head_dim; ++d) z += qd[d] * kc[(size_t)t * head_dim + d];
        double e = exp(z * scale - mi);
        li += e;
        for (int d = 0; d < head_dim; ++d) oi[d] += e * vc[(size_t)t * head_dim + d];
      }
      m[i] = mi;
      l[i] = li;
      memcpy(o + (size_t)i * head_dim, oi, sizeof(double) * head_dim);
    }
    double M = -INFINITY;
    for (int i = 0; i < nparts; ++i)
      if (m[i] > M) M = m[i];
    double den = 0.0;
    for (int d = 0; d < head_dim; ++d) acc[d] = 0.0;
    for (int i = 0; i < nparts; ++i) {
      double w = exp(m[i] - M);
      den += w * l[i];
      for (int d = 0; d < head_dim; ++d) acc[d] += w * o[(size_t)i * head_dim + d];
    }
    for (int d = 0; d < head_dim; ++d) acc[d] /= den;
    free(m);
    free(l);
    free(o);
    free(kc);
    free(vc);
    free(qd);
    free(oi);
  }
}
