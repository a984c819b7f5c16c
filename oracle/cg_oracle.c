/*
 * cg_oracle.c -- plain, slow CPU reference of the CacheGen-style KV codec.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the GPU smoke check and the CPU
 * baseline of the benchmark load this library; the GPU library never links,
 * includes or calls it, and the two share no code (not even a header).
 *
 * What it computes, by source (page title and section):
 *  [P2] "CacheGen实战：KV缓存压缩与流式传输在大型语言模型服务中的高效应用"
 *       section 1:   three-part compression -- store differences between
 *                    neighbouring tokens, quantize with a finer step in
 *                    shallow layers and a coarser one in deep layers, and
 *                    entropy-code the differences group by group so frequent
 *                    patterns get short codes;
 *       section 2.1: cut the context into 1.5K-token chunks, encode each at
 *                    three quality levels;
 *       section 2.3: the receiver decodes on the GPU and a fill stage puts
 *                    the KV into the model's cache;
 *       section 3.1: step presets 0.3/0.8/1.2, 0.5/1.0/1.5, 0.8/1.5/2.0.
 *  [P1] "CacheGen：大语言模型推理加速的KV缓存压缩与流式传输技术解析"
 *       「KV缓存的量化压缩机制」: K and V are 16-bit FP16/BF16 tensors;
 *       「量化编码器设计」: statistics are taken per channel and the quantized
 *       integer indices are entropy coded; the coder's statistics may come
 *       from a calibration run on other data (robust tables, below);
 *       「流式传输架构」: the compressed cache travels as independent chunks.
 *  [P3] KV-cache optimisation article (test.idctop.com),
 *       「vLLM中的PagedAttention优化」: KV held in physical blocks that need
 *       not be contiguous, located through a block table.
 *
 * The pages fix none of the bit-level choices (rounding, alphabet, escape,
 * normalisation, stream layout). Those are readings, each marked READING
 * below.
 *
 * Compile: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no SIMD code).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CGO_PROB_BITS 12
#define CGO_M 4096u            /* 2^12: total of every frequency table     */
#define CGO_L 65536u           /* 2^16: lower bound of the rANS state      */
#define CGO_ESC 255            /* escape symbol                            */
#define CGO_LANES 64           /* channels per group                       */
#define CGO_HDR_WORDS 192      /* 3 x 64 words at the head of a group      */

#define CGO_OK 0
#define CGO_ERR_INVALID_ARG (-1)
#define CGO_ERR_UNSUPPORTED (-2)
#define CGO_ERR_CAPACITY (-3)
#define CGO_ERR_CORRUPT (-5)
#define CGO_ERR_TABLE (-6)

#define CGO_F16 0                    /* element types of the KV tensor  */
#define CGO_BF16 1
#define CGO_TABLES_ROBUST 1u         /* tables flag: unseen symbols escape */

#define CGO_TABLE_MAGIC 0x42544743u  /* "CGTB" */
#define CGO_RECORD_MAGIC 0x4B434743u /* "CGCK" */
#define CGO_VERSION 1u

typedef struct {
  int32_t layers;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t chunk_tokens;
  int64_t tokens;
  int32_t dtype;     /* CGO_F16 or CGO_BF16: the element type of x and y */
  int32_t reserved;  /* 0 */
} cgo_shape;

/* ------------------------------------------------------------------------ */
/* Little-endian field access (the container is defined little-endian).     */
/* ------------------------------------------------------------------------ */
static void put_u16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}
static uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format definition.       */
/* [P1]「KV缓存的量化压缩机制」: the cache holds 16-bit FP16 elements.       */
/* ------------------------------------------------------------------------ */
float cgo_half_to_float(uint16_t h) {
  uint32_t sign = h >> 15, e = (h >> 10) & 31u, m = h & 1023u;
  float v;
  if (e == 0) {
    v = ldexpf((float)m, -24);               /* zero or subnormal: m * 2^-24 */
  } else if (e == 31) {
    if (m == 0) {
      v = INFINITY;
    } else {                                  /* NaN: keep the payload bits */
      uint32_t bits = 0x7F800000u | (m << 13);
      memcpy(&v, &bits, 4);
    }
  } else {
    v = ldexpf((float)(1024u + m), (int)e - 25); /* (1.m) * 2^(e-15)        */
  }
  return sign ? -v : v;
}

/* Round to nearest, ties to even. */
uint16_t cgo_float_to_half(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7E00u | ((bits >> 13) & 0x3FFu));
  double a = fabs((double)f);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);  /* halfway past 65504 */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: multiples of 2^-24; 1024 becomes the smallest normal */
    double n = rint(a * ldexp(1.0, 24));
    return (uint16_t)(sign | (uint16_t)n);
  }
  int ex;
  frexp(a, &ex);                 /* a = fr * 2^ex, fr in [0.5, 1)            */
  int E = ex - 1;                /* a in [2^E, 2^(E+1))                       */
  double n = rint(ldexp(a, 10 - E)); /* significand scaled to [1024, 2048]    */
  if (n >= 2048.0) { n = 1024.0; E += 1; }
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((uint32_t)n - 1024u));
}

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> binary32, from the format: sign, 8-bit exponent (bias 127),  */
/* 7-bit fraction. [P1]「KV缓存的量化压缩机制」: BF16 is the other 16-bit    */
/* type the cache may hold.                                                   */
/* ------------------------------------------------------------------------ */
float cgo_bf16_to_float(uint16_t h) {
  uint32_t sign = h >> 15, e = (h >> 7) & 255u, m = h & 127u;
  float v;
  if (e == 0) {
    v = ldexpf((float)m, -133);               /* zero or subnormal: m * 2^-133 */
  } else if (e == 255) {
    if (m == 0) {
      v = INFINITY;
    } else {                                  /* NaN: keep the payload bits  */
      uint32_t bits = 0x7F800000u | (m << 16);
      memcpy(&v, &bits, 4);
    }
  } else {
    v = ldexpf((float)(128u + m), (int)e - 134); /* (1.m) * 2^(e-127)        */
  }
  return sign ? -v : v;
}

/* Round to nearest, ties to even; NaN stays a (quiet) NaN. */
uint16_t cgo_float_to_bf16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7FC0u | ((bits >> 16) & 0x7Fu));
  double a = fabs((double)f);
  /* halfway between the largest finite value (2 - 2^-7) * 2^127 and 2^128;
   * the tie goes to the even neighbour, which is the overflow */
  if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7F80u);
  if (a < ldexp(1.0, -126)) {
    /* subnormal range: multiples of 2^-133; 128 becomes the smallest normal */
    double n = rint(a * ldexp(1.0, 133));
    return (uint16_t)(sign | (uint16_t)n);
  }
  int ex;
  frexp(a, &ex);
  int E = ex - 1;                    /* a in [2^E, 2^(E+1))                   */
  double n = rint(ldexp(a, 7 - E));  /* significand scaled to [128, 256]      */
  if (n >= 256.0) { n = 128.0; E += 1; }
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)((uint32_t)n - 128u));
}

static float elem_to_float(int dtype, uint16_t h) {
  return dtype == CGO_BF16 ? cgo_bf16_to_float(h) : cgo_half_to_float(h);
}
static uint16_t float_to_elem(int dtype, float f) {
  return dtype == CGO_BF16 ? cgo_float_to_bf16(f) : cgo_float_to_half(f);
}

/* ------------------------------------------------------------------------ */
/* Quantization. [P2] section 1: one uniform step per layer group, finer in  */
/* shallow layers; presets in section 3.1.                                    */
/* READING: q = round-half-even(fl32(x / step)) with an IEEE binary32 divide, */
/* clamped to int16; NaN gives 0. Saturation is counted.                       */
/* ------------------------------------------------------------------------ */
int32_t cgo_quantize_dt(int dtype, uint16_t xh, float step, int* saturated, int* is_nan) {
  float x = elem_to_float(dtype, xh);
  if (saturated) *saturated = 0;
  if (is_nan) *is_nan = 0;
  if (isnan(x)) {
    if (is_nan) *is_nan = 1;
    return 0;
  }
  float v = x / step;           /* binary32 division, round to nearest even  */
  float r = rintf(v);           /* round half to even (default rounding mode) */
  if (r > 32767.0f) {
    if (saturated) *saturated = 1;
    return 32767;
  }
  if (r < -32768.0f) {
    if (saturated) *saturated = 1;
    return -32768;
  }
  return (int32_t)r;
}

int32_t cgo_quantize(uint16_t xh, float step, int* saturated, int* is_nan) {
  return cgo_quantize_dt(CGO_F16, xh, step, saturated, is_nan);
}

/* READING: reconstruction = RNE to the element type of fl32(float(q) * step). */
uint16_t cgo_dequantize_dt(int dtype, int32_t q, float step) {
  float v = (float)q * step;    /* one binary32 product, no contraction      */
  return float_to_elem(dtype, v);
}

uint16_t cgo_dequantize(int32_t q, float step) { return cgo_dequantize_dt(CGO_F16, q, step); }

/* Array forms of the scalar definitions above (plain loops, for tests). */
void cgo_half_to_float_array(const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_half_to_float(h[i]);
}
void cgo_float_to_half_array(const float* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_float_to_half(f[i]);
}
void cgo_quantize_array(const uint16_t* xh, int64_t n, float step, int32_t* q) {
  for (int64_t i = 0; i < n; i++) q[i] = cgo_quantize(xh[i], step, 0, 0);
}
void cgo_dequantize_array(const int32_t* q, int64_t n, float step, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_dequantize(q[i], step);
}
void cgo_bf16_to_float_array(const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_bf16_to_float(h[i]);
}
void cgo_float_to_bf16_array(const float* f, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_float_to_bf16(f[i]);
}
void cgo_quantize_array_dt(int dtype, const uint16_t* xh, int64_t n, float step, int32_t* q) {
  for (int64_t i = 0; i < n; i++) q[i] = cgo_quantize_dt(dtype, xh[i], step, 0, 0);
}
void cgo_dequantize_array_dt(int dtype, const int32_t* q, int64_t n, float step, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = cgo_dequantize_dt(dtype, q[i], step);
}

/* ------------------------------------------------------------------------ */
/* Token deltas and symbols. [P2] section 1: only the difference to the      */
/* previous token is stored. READING: differences of the quantized q, taken  */
/* modulo 2^16 so every difference fits int16; the first token of a chunk is */
/* stored raw; |d| <= 127 maps to symbol d+127, anything else to the escape  */
/* symbol 255 followed by the raw 16-bit difference.                          */
/* ------------------------------------------------------------------------ */
int32_t cgo_wrap16(int32_t v) {
  int32_t r = (v + 32768) % 65536;
  if (r < 0) r += 65536;
  return r - 32768;
}

static int symbol_of(int32_t d, uint16_t* payload) {
  *payload = (uint16_t)(d & 0xFFFF);
  if (d >= -127 && d <= 127) return d + 127;
  return CGO_ESC;
}

static int64_t chunk_count(const cgo_shape* s) {
  return (s->tokens + s->chunk_tokens - 1) / s->chunk_tokens;
}

static int64_t chunk_len(const cgo_shape* s, int64_t c) {
  int64_t t0 = c * s->chunk_tokens;
  int64_t n = s->tokens - t0;
  return n < s->chunk_tokens ? n : s->chunk_tokens;
}

static size_t x_index(const cgo_shape* s, int l, int kv, int h, int64_t t, int d) {
  return ((((size_t)l * 2 + kv) * s->kv_heads + h) * (size_t)s->tokens + (size_t)t) *
             s->head_dim + d;
}

static int shape_ok(const cgo_shape* s) {
  return s && s->layers > 0 && s->kv_heads > 0 && s->head_dim > 0 && s->head_dim % 64 == 0 &&
         s->chunk_tokens > 0 && s->tokens > 0 && (s->dtype == CGO_F16 || s->dtype == CGO_BF16) &&
         s->reserved == 0;
}

/* ------------------------------------------------------------------------ */
/* Per-channel statistics. [P1]「量化编码器设计」: statistics are gathered    */
/* channel by channel; [P2] section 1: entropy coding is grouped.             */
/* READING: one table per (layer group, K|V, head, dim); it counts the       */
/* symbols of tokens 1..n-1 of every chunk over every layer of the group     */
/* (the raw first token is not counted).                                      */
/* ------------------------------------------------------------------------ */
void cgo_table_counts(const cgo_shape* s, const uint8_t* layer_group, const float* steps,
                      const uint16_t* X, int g, int kv, int h, int d, uint64_t counts[256],
                      uint64_t stats[4]) {
  memset(counts, 0, 256 * sizeof(uint64_t));
  for (int l = 0; l < s->layers; l++) {
    if (layer_group[l] != g) continue;
    float step = steps[g];
    for (int64_t c = 0; c < chunk_count(s); c++) {
      int64_t t0 = c * s->chunk_tokens, n = chunk_len(s, c);
      int32_t prev = 0;
      for (int64_t i = 0; i < n; i++) {
        int sat, nan_;
        int32_t q = cgo_quantize_dt(s->dtype, X[x_index(s, l, kv, h, t0 + i, d)], step, &sat, &nan_);
        if (stats) {
          stats[0] += 1;
          stats[1] += (uint64_t)sat;
          stats[2] += (uint64_t)nan_;
        }
        if (i > 0) {
          uint16_t pay;
          int sym = symbol_of(cgo_wrap16(q - prev), &pay);
          counts[sym] += 1;
          if (stats && sym == CGO_ESC) stats[3] += 1;
        }
        prev = q;
      }
    }
  }
}

/* READING: normalisation to a 12-bit table (the coder is a 12-bit static
 * rANS). Every observed symbol keeps f >= 1, unobserved symbols get 0; the
 * rounding deficit goes to the most frequent symbol, a surplus is taken from
 * the largest frequency. Ties go to the lowest symbol index. */
void cgo_normalize(const uint64_t counts[256], uint16_t f[256]) {
  uint64_t n = 0;
  for (int s = 0; s < 256; s++) n += counts[s];
  memset(f, 0, 256 * sizeof(uint16_t));
  if (n == 0) {
    f[127] = CGO_M;
    return;
  }
  uint32_t S = 0;
  for (int s = 0; s < 256; s++) {
    if (counts[s] == 0) continue;
    uint64_t v = counts[s] * CGO_M / n;
    f[s] = (uint16_t)(v < 1 ? 1 : v);
    S += f[s];
  }
  if (S < CGO_M) {
    int j = 0;
    for (int s = 1; s < 256; s++)
      if (counts[s] > counts[j]) j = s;
    f[j] = (uint16_t)(f[j] + (CGO_M - S));
    S = CGO_M;
  }
  while (S > CGO_M) {
    int j = 0;
    for (int s = 1; s < 256; s++)
      if (f[s] > f[j]) j = s;
    uint32_t cut = f[j] - 1u;
    if (cut > S - CGO_M) cut = S - CGO_M;
    f[j] = (uint16_t)(f[j] - cut);
    S -= cut;
  }
}

/* READING: robust tables ([P1]「量化编码器设计」: the statistics may come
 * from calibration data other than the tensor coded). Normalise as above;
 * if the escape symbol got no frequency, one unit moves to it from the
 * largest frequency (lowest symbol on ties), so that every delta stays
 * codable: a delta whose symbol has f = 0 is coded as an escape. */
void cgo_normalize_robust(const uint64_t counts[256], uint16_t f[256]) {
  cgo_normalize(counts, f);
  if (f[CGO_ESC] == 0) {
    int j = 0;
    for (int s = 1; s < 256; s++)
      if (f[s] > f[j]) j = s;
    f[j] = (uint16_t)(f[j] - 1u);
    f[CGO_ESC] = 1;
  }
}

/* Cumulative frequencies: b[s] = sum of f over symbols below s. */
static void cumulative(const uint16_t f[256], uint32_t b[256]) {
  uint32_t acc = 0;
  for (int s = 0; s < 256; s++) {
    b[s] = acc;
    acc += f[s];
  }
}

/* ------------------------------------------------------------------------ */
/* Tables blob (format section). Little-endian:                              */
/*   0 magic "CGTB"   4 version   8 layers  12 kv_heads  16 head_dim         */
/*  20 n_groups      24 level_id 28 chunk_tokens  32 tokens (u64)            */
/*  40 f_offset      44 dtype    48 format_bytes (u64)   56 flags  60 zero    */
/*  64 f32 step[G], then u8 layer_group[L], zero pad to f_offset             */
/*     (= align 256), then u16 f[G][2][H][D][256].                           */
/* ------------------------------------------------------------------------ */
uint64_t cgo_tables_f_offset(const cgo_shape* s, int32_t n_groups) {
  return align_up(64 + 4 * (uint64_t)n_groups + (uint64_t)s->layers, 256);
}

uint64_t cgo_tables_format_bytes(const cgo_shape* s, int32_t n_groups) {
  return cgo_tables_f_offset(s, n_groups) +
         (uint64_t)n_groups * 2 * s->kv_heads * s->head_dim * 256 * 2;
}

static size_t table_index(const cgo_shape* s, int g, int kv, int h, int d) {
  return (((size_t)g * 2 + kv) * s->kv_heads + h) * s->head_dim + d;
}

/* Builds the tables of one quality level from X (the tensor to encode, or
 * calibration data for robust tables: flags = CGO_TABLES_ROBUST).
 * stats (optional) = {elements, saturated, nan, escapes}. */
int cgo_build_tables(const cgo_shape* s, int32_t level_id, int32_t n_groups,
                     const uint8_t* layer_group, const float* steps, const uint16_t* X,
                     uint32_t flags, uint8_t* blob, uint64_t blob_cap, uint64_t stats[4]) {
  if (!shape_ok(s) || n_groups < 1 || n_groups > 255) return CGO_ERR_INVALID_ARG;
  if (flags & ~CGO_TABLES_ROBUST) return CGO_ERR_INVALID_ARG;
  for (int l = 0; l < s->layers; l++)
    if (layer_group[l] >= n_groups) return CGO_ERR_INVALID_ARG;
  for (int g = 0; g < n_groups; g++)
    if (!(steps[g] > 0.0f) || isinf(steps[g])) return CGO_ERR_INVALID_ARG;
  uint64_t need = cgo_tables_format_bytes(s, n_groups);
  if (blob_cap < need) return CGO_ERR_CAPACITY;
  memset(blob, 0, need);
  uint64_t foff = cgo_tables_f_offset(s, n_groups);
  put_u32(blob + 0, CGO_TABLE_MAGIC);
  put_u32(blob + 4, CGO_VERSION);
  put_u32(blob + 8, (uint32_t)s->layers);
  put_u32(blob + 12, (uint32_t)s->kv_heads);
  put_u32(blob + 16, (uint32_t)s->head_dim);
  put_u32(blob + 20, (uint32_t)n_groups);
  put_u32(blob + 24, (uint32_t)level_id);
  put_u32(blob + 28, (uint32_t)s->chunk_tokens);
  put_u64(blob + 32, (uint64_t)s->tokens);
  put_u32(blob + 40, (uint32_t)foff);
  put_u32(blob + 44, (uint32_t)s->dtype);
  put_u64(blob + 48, need);
  put_u32(blob + 56, flags);
  for (int g = 0; g < n_groups; g++) {
    uint32_t bits;
    memcpy(&bits, &steps[g], 4);
    put_u32(blob + 64 + 4 * g, bits);
  }
  for (int l = 0; l < s->layers; l++) blob[64 + 4 * n_groups + l] = layer_group[l];
  if (stats) memset(stats, 0, 4 * sizeof(uint64_t));
  uint64_t counts[256];
  uint16_t f[256];
  for (int g = 0; g < n_groups; g++)
    for (int kv = 0; kv < 2; kv++)
      for (int h = 0; h < s->kv_heads; h++)
        for (int d = 0; d < s->head_dim; d++) {
          cgo_table_counts(s, layer_group, steps, X, g, kv, h, d, counts, stats);
          if (flags & CGO_TABLES_ROBUST)
            cgo_normalize_robust(counts, f);
          else
            cgo_normalize(counts, f);
          uint8_t* dst = blob + foff + table_index(s, g, kv, h, d) * 512;
          for (int k = 0; k < 256; k++) put_u16(dst + 2 * k, f[k]);
        }
  return CGO_OK;
}

typedef struct {
  int32_t n_groups, level_id;
  int robust;
  float steps[256];
  uint8_t lg[65536];
  const uint8_t* f;
} blob_view;

static int parse_blob(const cgo_shape* s, const uint8_t* blob, blob_view* v) {
  if (get_u32(blob) != CGO_TABLE_MAGIC || get_u32(blob + 4) != CGO_VERSION) return CGO_ERR_INVALID_ARG;
  if ((int32_t)get_u32(blob + 8) != s->layers || (int32_t)get_u32(blob + 12) != s->kv_heads ||
      (int32_t)get_u32(blob + 16) != s->head_dim || s->layers > 65536)
    return CGO_ERR_INVALID_ARG;
  v->n_groups = (int32_t)get_u32(blob + 20);
  v->level_id = (int32_t)get_u32(blob + 24);
  if ((int32_t)get_u32(blob + 44) != s->dtype) return CGO_ERR_INVALID_ARG;
  uint32_t flags = get_u32(blob + 56);
  if (flags & ~CGO_TABLES_ROBUST) return CGO_ERR_INVALID_ARG;
  v->robust = (flags & CGO_TABLES_ROBUST) != 0;
  if (v->n_groups < 1 || v->n_groups > 255) return CGO_ERR_INVALID_ARG;
  for (int g = 0; g < v->n_groups; g++) {
    uint32_t bits = get_u32(blob + 64 + 4 * g);
    memcpy(&v->steps[g], &bits, 4);
  }
  for (int l = 0; l < s->layers; l++) v->lg[l] = blob[64 + 4 * v->n_groups + l];
  v->f = blob + get_u32(blob + 40);
  return CGO_OK;
}

static void load_table(const cgo_shape* s, const blob_view* v, int g, int kv, int h, int d,
                       uint16_t f[256]) {
  const uint8_t* src = v->f + table_index(s, g, kv, h, d) * 512;
  for (int k = 0; k < 256; k++) f[k] = get_u16(src + 2 * k);
}

/* ------------------------------------------------------------------------ */
/* Entropy coding of one group. [P2] section 1 (grouped entropy coding),     */
/* [P1]「量化编码器设计」(integer indices entropy coded).                       */
/* READING: static rANS with 12-bit frequencies (M = 4096), a 32-bit state   */
/* in [2^16, 2^32) and 16-bit renormalisation words. A group is             */
/* (chunk, layer, K|V, head, 64-channel slice j); lane k codes channel       */
/* 64j+k with its own table and its own state. Word order as the decoder    */
/* reads it:                                                                  */
/*   state>>16 of lanes 0..63, state&0xFFFF of lanes 0..63,                  */
/*   raw q of the first token of lanes 0..63,                                */
/*   then for tokens i = 1..n-1: the renormalisation words of the lanes that */
/*   need one (ascending lane), then the escape payloads (ascending lane).   */
/* The encoder runs i = n-1 down to 1; for each lane it first renormalises   */
/* (emits the low 16 bits when x >= f*2^20) and then codes the symbol:       */
/*   x <- floor(x/f)*4096 + (x mod f) + b.                                    */
/* With robust tables a symbol of frequency 0 is coded as the escape (its   */
/* delta becomes the payload); otherwise it is an error (CGO_ERR_TABLE).    */
/* ------------------------------------------------------------------------ */
static void group_q(const cgo_shape* s, const blob_view* v, const uint16_t* X, int64_t c, int l,
                    int kv, int h, int j, int32_t* q /* [64][n] */, int64_t n) {
  int64_t t0 = c * s->chunk_tokens;
  float step = v->steps[v->lg[l]];
  for (int k = 0; k < CGO_LANES; k++)
    for (int64_t i = 0; i < n; i++)
      q[k * n + i] = cgo_quantize_dt(s->dtype, X[x_index(s, l, kv, h, t0 + i, 64 * j + k)], step, 0, 0);
}

/* Worst case: one renorm word and one escape word per symbol, plus the head. */
int64_t cgo_group_word_bound(int64_t n) { return CGO_LANES * (2 * (n - 1) + 3); }

int64_t cgo_encode_group_q(const int32_t* q /* [64][n] */, int64_t n,
                           const uint16_t* const f_lane[64], int robust, uint16_t* out, int64_t cap) {
  uint32_t b[64][256];
  for (int k = 0; k < CGO_LANES; k++) cumulative(f_lane[k], b[k]);
  int64_t steps = n > 1 ? n - 1 : 0;
  uint16_t* rw = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(steps * 64 + 1));
  uint16_t* ew = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(steps * 64 + 1));
  int* rc = (int*)calloc((size_t)(steps + 1), sizeof(int));
  int* ec = (int*)calloc((size_t)(steps + 1), sizeof(int));
  uint32_t x[64];
  int64_t result = 0;
  for (int k = 0; k < CGO_LANES; k++) x[k] = CGO_L;
  for (int64_t i = n - 1; i >= 1; i--) {
    int64_t slot = i - 1;
    for (int k = 0; k < CGO_LANES; k++) {
      uint16_t pay = 0;
      int sym = symbol_of(cgo_wrap16(q[k * n + i] - q[k * n + i - 1]), &pay);
      if (robust && f_lane[k][sym] == 0) sym = CGO_ESC;
      uint32_t f = f_lane[k][sym];
      if (f == 0) {
        result = CGO_ERR_TABLE;
        goto done;
      }
      if ((uint64_t)x[k] >= ((uint64_t)f << 20)) {
        rw[slot * 64 + rc[slot]++] = (uint16_t)(x[k] & 0xFFFFu);
        x[k] >>= 16;
      }
      x[k] = (x[k] / f) * CGO_M + (x[k] % f) + b[k][sym];
      if (sym == CGO_ESC) ew[slot * 64 + ec[slot]++] = pay;
    }
  }
  {
    int64_t total = CGO_HDR_WORDS;
    for (int64_t i = 0; i < steps; i++) total += rc[i] + ec[i];
    if (total > cap) {
      result = CGO_ERR_CAPACITY;
      goto done;
    }
    int64_t p = 0;
    for (int k = 0; k < CGO_LANES; k++) out[p++] = (uint16_t)(x[k] >> 16);
    for (int k = 0; k < CGO_LANES; k++) out[p++] = (uint16_t)(x[k] & 0xFFFFu);
    for (int k = 0; k < CGO_LANES; k++) out[p++] = (uint16_t)(q[k * n] & 0xFFFF);
    for (int64_t i = 0; i < steps; i++) {
      for (int r = 0; r < rc[i]; r++) out[p++] = rw[i * 64 + r];
      for (int r = 0; r < ec[i]; r++) out[p++] = ew[i * 64 + r];
    }
    result = p;
  }
done:
  free(rw);
  free(ew);
  free(rc);
  free(ec);
  return result;
}

/* Inverse of the above. Writes q[64][n]. Returns CGO_OK or CGO_ERR_CORRUPT
 * (a word read past the end, a final state other than 2^16, or words left). */
int cgo_decode_group_q(const uint16_t* w, int64_t n_words, int64_t n,
                       const uint16_t* const f_lane[64], int32_t* q /* [64][n] */) {
  uint32_t b[64][256];
  for (int k = 0; k < CGO_LANES; k++) cumulative(f_lane[k], b[k]);
  if (n_words < CGO_HDR_WORDS) return CGO_ERR_CORRUPT;
  uint32_t x[64];
  int sym[64];
  int64_t p = 0;
  for (int k = 0; k < CGO_LANES; k++) x[k] = (uint32_t)w[p++] << 16;
  for (int k = 0; k < CGO_LANES; k++) x[k] |= w[p++];
  for (int k = 0; k < CGO_LANES; k++) q[k * n] = (int16_t)w[p++];
  for (int64_t i = 1; i < n; i++) {
    for (int k = 0; k < CGO_LANES; k++) {
      uint32_t slot = x[k] & (CGO_M - 1);
      int s = -1;
      for (int t = 0; t < 256; t++)
        if (f_lane[k][t] > 0 && b[k][t] <= slot && slot < b[k][t] + f_lane[k][t]) {
          s = t;
          break;
        }
      if (s < 0) return CGO_ERR_CORRUPT;
      sym[k] = s;
      x[k] = f_lane[k][s] * (x[k] >> CGO_PROB_BITS) + slot - b[k][s];
    }
    for (int k = 0; k < CGO_LANES; k++)
      if (x[k] < CGO_L) {
        if (p >= n_words) return CGO_ERR_CORRUPT;
        x[k] = (x[k] << 16) | w[p++];
      }
    for (int k = 0; k < CGO_LANES; k++) {
      int32_t d;
      if (sym[k] == CGO_ESC) {
        if (p >= n_words) return CGO_ERR_CORRUPT;
        d = (int16_t)w[p++];
      } else {
        d = sym[k] - 127;
      }
      q[k * n + i] = cgo_wrap16(q[k * n + i - 1] + d);
    }
  }
  for (int k = 0; k < CGO_LANES; k++)
    if (x[k] != CGO_L) return CGO_ERR_CORRUPT;
  if (p != n_words) return CGO_ERR_CORRUPT;
  return CGO_OK;
}

static void lane_tables(const cgo_shape* s, const blob_view* v, int l, int kv, int h, int j,
                        uint16_t (*fbuf)[256], const uint16_t* f_lane[64]) {
  for (int k = 0; k < CGO_LANES; k++) {
    load_table(s, v, v->lg[l], kv, h, 64 * j + k, fbuf[k]);
    f_lane[k] = fbuf[k];
  }
}

/* One group of one chunk, straight from the fp16 tensor and the blob. */
int64_t cgo_encode_group(const cgo_shape* s, const uint8_t* blob, const uint16_t* X, int64_t c,
                         int l, int kv, int h, int j, uint16_t* out, int64_t cap) {
  if (!shape_ok(s)) return CGO_ERR_INVALID_ARG;
  blob_view* v = (blob_view*)malloc(sizeof(blob_view));
  int rc = parse_blob(s, blob, v);
  if (rc != CGO_OK) {
    free(v);
    return rc;
  }
  int64_t n = chunk_len(s, c);
  int32_t* q = (int32_t*)malloc(sizeof(int32_t) * 64 * (size_t)n);
  uint16_t fbuf[64][256];
  const uint16_t* f_lane[64];
  group_q(s, v, X, c, l, kv, h, j, q, n);
  lane_tables(s, v, l, kv, h, j, fbuf, f_lane);
  int64_t r = cgo_encode_group_q(q, n, f_lane, v->robust, out, cap);
  free(q);
  free(v);
  return r;
}

/* ------------------------------------------------------------------------ */
/* Chunk record. [P2] section 2.1 and [P1]「流式传输架构」: every chunk is a  */
/* self-contained, separately transferable unit. READING (layout, LE):       */
/*   0 magic "CGCK"  4 version  8 chunk_index  12 level_id                   */
/*  16 token_start (u64)  24 n_tokens  28 n_groups  32 layers  36 kv_heads   */
/*  40 head_dim  44 data_start  48 record_bytes (u64)  56 data_bytes (u64)   */
/*  64 u64 group_offset[n_groups+1] (from data start, multiples of 16)       */
/*     u32 group_words[n_groups]; zero pad to data_start (align 256);        */
/*     group streams in (layer, K|V, head, slice) order, each zero-padded to */
/*     16 bytes; zero pad to record_bytes (align 256).                        */
/* ------------------------------------------------------------------------ */
static int64_t groups_per_chunk(const cgo_shape* s) {
  return (int64_t)s->layers * 2 * s->kv_heads * (s->head_dim / 64);
}

uint64_t cgo_record_data_start(const cgo_shape* s) {
  int64_t G = groups_per_chunk(s);
  return align_up(64 + 8 * (uint64_t)(G + 1) + 4 * (uint64_t)G, 256);
}

int64_t cgo_encode_chunk(const cgo_shape* s, const uint8_t* blob, const uint16_t* X, int64_t c,
                         uint8_t* out, uint64_t cap) {
  if (!shape_ok(s) || c < 0 || c >= chunk_count(s)) return CGO_ERR_INVALID_ARG;
  blob_view* v = (blob_view*)malloc(sizeof(blob_view));
  int rc = parse_blob(s, blob, v);
  if (rc != CGO_OK) {
    free(v);
    return rc;
  }
  int64_t n = chunk_len(s, c), G = groups_per_chunk(s);
  int64_t bound = cgo_group_word_bound(n);
  uint16_t* words = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)bound);
  int32_t* q = (int32_t*)malloc(sizeof(int32_t) * 64 * (size_t)n);
  uint64_t* offs = (uint64_t*)calloc((size_t)G + 1, sizeof(uint64_t));
  uint32_t* nw = (uint32_t*)calloc((size_t)G, sizeof(uint32_t));
  uint64_t data_cap = 1 << 16, pos = 0;
  uint8_t* data = (uint8_t*)calloc(data_cap, 1);
  uint64_t ds = cgo_record_data_start(s);
  int64_t result = 0;
  int slices = s->head_dim / 64;
  uint16_t fbuf[64][256];
  const uint16_t* f_lane[64];
  int64_t gi = 0;
  for (int l = 0; l < s->layers; l++)
    for (int kv = 0; kv < 2; kv++)
      for (int h = 0; h < s->kv_heads; h++)
        for (int j = 0; j < slices; j++, gi++) {
          group_q(s, v, X, c, l, kv, h, j, q, n);
          lane_tables(s, v, l, kv, h, j, fbuf, f_lane);
          int64_t m = cgo_encode_group_q(q, n, f_lane, v->robust, words, bound);
          if (m < 0) {
            result = m;
            goto done;
          }
          uint64_t padded = align_up(2 * (uint64_t)m, 16);
          while (pos + padded > data_cap) {
            data = (uint8_t*)realloc(data, data_cap * 2);
            memset(data + data_cap, 0, data_cap);
            data_cap *= 2;
          }
          offs[gi] = pos;
          nw[gi] = (uint32_t)m;
          for (int64_t k = 0; k < m; k++) put_u16(data + pos + 2 * k, words[k]);
          pos += padded;
        }
  offs[G] = pos;
  {
    uint64_t rec = align_up(ds + pos, 256);
    if (rec > cap) {
      result = CGO_ERR_CAPACITY;
      goto done;
    }
    memset(out, 0, rec);
    put_u32(out + 0, CGO_RECORD_MAGIC);
    put_u32(out + 4, CGO_VERSION);
    put_u32(out + 8, (uint32_t)c);
    put_u32(out + 12, (uint32_t)v->level_id);
    put_u64(out + 16, (uint64_t)(c * s->chunk_tokens));
    put_u32(out + 24, (uint32_t)n);
    put_u32(out + 28, (uint32_t)G);
    put_u32(out + 32, (uint32_t)s->layers);
    put_u32(out + 36, (uint32_t)s->kv_heads);
    put_u32(out + 40, (uint32_t)s->head_dim);
    put_u32(out + 44, (uint32_t)ds);
    put_u64(out + 48, rec);
    put_u64(out + 56, pos);
    for (int64_t g = 0; g <= G; g++) put_u64(out + 64 + 8 * g, offs[g]);
    for (int64_t g = 0; g < G; g++) put_u32(out + 64 + 8 * (G + 1) + 4 * g, nw[g]);
    memcpy(out + ds, data, pos);
    result = (int64_t)rec;
  }
done:
  free(words);
  free(q);
  free(offs);
  free(nw);
  free(data);
  free(v);
  return result;
}

/* Upper bound of a chunk record's size (every group at its worst case). */
uint64_t cgo_record_bound(const cgo_shape* s, int64_t c) {
  int64_t n = chunk_len(s, c);
  return align_up(cgo_record_data_start(s) +
                      (uint64_t)groups_per_chunk(s) * align_up(2 * (uint64_t)cgo_group_word_bound(n), 16),
                  256);
}

/* ------------------------------------------------------------------------ */
/* Decode of one chunk record. [P2] section 2.3: decode, then fill the       */
/* model's cache. Contiguous target Y[layer][K|V][head][token][dim], or the  */
/* paged pool[layer][K|V][block][head][16][dim] with block = bt[token/16]    */
/* ([P3]「vLLM中的PagedAttention优化」); other pool entries are untouched.    */
/* ------------------------------------------------------------------------ */
static int check_record(const cgo_shape* s, const blob_view* v, const uint8_t* rec,
                        uint64_t rec_bytes, int64_t* c_out) {
  int64_t G = groups_per_chunk(s);
  if (rec_bytes < 64) return CGO_ERR_CORRUPT;
  if (get_u32(rec) != CGO_RECORD_MAGIC || get_u32(rec + 4) != CGO_VERSION) return CGO_ERR_CORRUPT;
  int64_t c = get_u32(rec + 8);
  if (c >= chunk_count(s)) return CGO_ERR_CORRUPT;
  if ((int32_t)get_u32(rec + 12) != v->level_id) return CGO_ERR_CORRUPT;
  if (get_u64(rec + 16) != (uint64_t)(c * s->chunk_tokens)) return CGO_ERR_CORRUPT;
  if (get_u32(rec + 24) != (uint32_t)chunk_len(s, c)) return CGO_ERR_CORRUPT;
  if (get_u32(rec + 28) != (uint32_t)G) return CGO_ERR_CORRUPT;
  if ((int32_t)get_u32(rec + 32) != s->layers || (int32_t)get_u32(rec + 36) != s->kv_heads ||
      (int32_t)get_u32(rec + 40) != s->head_dim)
    return CGO_ERR_CORRUPT;
  uint64_t ds = get_u32(rec + 44), rb = get_u64(rec + 48), db = get_u64(rec + 56);
  if (ds != cgo_record_data_start(s) || rb > rec_bytes || ds + db > rb) return CGO_ERR_CORRUPT;
  uint64_t prev = 0;
  for (int64_t g = 0; g <= G; g++) {
    uint64_t o = get_u64(rec + 64 + 8 * g);
    if (o % 16 != 0 || o < prev || o > db) return CGO_ERR_CORRUPT;
    if (g == 0 && o != 0) return CGO_ERR_CORRUPT;
    if (g == G && o != db) return CGO_ERR_CORRUPT;
    if (g > 0) {
      uint64_t nw = get_u32(rec + 64 + 8 * (G + 1) + 4 * (g - 1));
      if (2 * nw > o - prev) return CGO_ERR_CORRUPT;
    }
    prev = o;
  }
  *c_out = c;
  return CGO_OK;
}

static int decode_chunk_impl(const cgo_shape* s, const uint8_t* blob, const uint8_t* rec,
                             uint64_t rec_bytes, uint16_t* Y, uint16_t* pool, int64_t num_blocks,
                             const int32_t* bt) {
  if (!shape_ok(s)) return CGO_ERR_INVALID_ARG;
  blob_view* v = (blob_view*)malloc(sizeof(blob_view));
  int rc = parse_blob(s, blob, v);
  if (rc != CGO_OK) {
    free(v);
    return rc;
  }
  int64_t c;
  rc = check_record(s, v, rec, rec_bytes, &c);
  if (rc != CGO_OK) {
    free(v);
    return rc;
  }
  int64_t n = chunk_len(s, c), t0 = c * s->chunk_tokens, G = groups_per_chunk(s);
  if (pool) {
    for (int64_t i = 0; i < n; i++) {
      int64_t blk = bt[(t0 + i) / 16];
      if (blk < 0 || blk >= num_blocks) {
        free(v);
        return CGO_ERR_INVALID_ARG;
      }
    }
  }
  uint64_t ds = get_u32(rec + 44);
  int32_t* q = (int32_t*)malloc(sizeof(int32_t) * 64 * (size_t)n);
  uint16_t* words = NULL;
  uint16_t fbuf[64][256];
  const uint16_t* f_lane[64];
  int slices = s->head_dim / 64, H = s->kv_heads, D = s->head_dim;
  int64_t gi = 0;
  rc = CGO_OK;
  for (int l = 0; l < s->layers && rc == CGO_OK; l++)
    for (int kv = 0; kv < 2 && rc == CGO_OK; kv++)
      for (int h = 0; h < H && rc == CGO_OK; h++)
        for (int j = 0; j < slices && rc == CGO_OK; j++, gi++) {
          uint64_t o = get_u64(rec + 64 + 8 * gi);
          uint64_t nw = get_u32(rec + 64 + 8 * (G + 1) + 4 * gi);
          words = (uint16_t*)realloc(words, sizeof(uint16_t) * (size_t)(nw + 1));
          for (uint64_t k = 0; k < nw; k++) words[k] = get_u16(rec + ds + o + 2 * k);
          lane_tables(s, v, l, kv, h, j, fbuf, f_lane);
          rc = cgo_decode_group_q(words, (int64_t)nw, n, f_lane, q);
          if (rc != CGO_OK) break;
          float step = v->steps[v->lg[l]];
          for (int k = 0; k < CGO_LANES; k++)
            for (int64_t i = 0; i < n; i++) {
              uint16_t y = cgo_dequantize_dt(s->dtype, q[k * n + i], step);
              int64_t t = t0 + i;
              int d = 64 * j + k;
              if (pool) {
                int64_t blk = bt[t / 16];
                size_t idx = (((((size_t)l * 2 + kv) * (size_t)num_blocks + (size_t)blk) * H + h) * 16 +
                              (size_t)(t % 16)) * D + d;
                pool[idx] = y;
              } else {
                Y[x_index(s, l, kv, h, t, d)] = y;
              }
            }
        }
  free(words);
  free(q);
  free(v);
  return rc;
}

int cgo_decode_chunk(const cgo_shape* s, const uint8_t* blob, const uint8_t* rec,
                     uint64_t rec_bytes, uint16_t* Y) {
  return decode_chunk_impl(s, blob, rec, rec_bytes, Y, NULL, 0, NULL);
}

int cgo_decode_chunk_paged(const cgo_shape* s, const uint8_t* blob, const uint8_t* rec,
                           uint64_t rec_bytes, uint16_t* pool, int64_t num_blocks,
                           const int32_t* block_table) {
  if (!pool || !block_table || num_blocks <= 0) return CGO_ERR_INVALID_ARG;
  return decode_chunk_impl(s, blob, rec, rec_bytes, NULL, pool, num_blocks, block_table);
}

/* ------------------------------------------------------------------------ */
/* Attention over the restored cache. [P2] section 2.3: the decoded KV is    */
/* filled into the model's cache and used by the model unchanged; [P3]      */
/* 「vLLM中的PagedAttention优化」: attention reads K/V from physical blocks  */
/* through a block table. READING: one new token per layer ("decode step"), */
/* q_heads query heads sharing the kv_heads (query head qh uses kv head      */
/* qh / (q_heads / kv_heads)), scores scale * q . k over the first n_tokens */
/* tokens, softmax, weighted sum of V; all in binary64.                      */
/*   q   element bits [layers][q_heads][head_dim]                           */
/*   o   binary64 [layers][q_heads][head_dim]                               */
/* ------------------------------------------------------------------------ */
int cgo_attend_paged(const cgo_shape* s, int32_t q_heads, const uint16_t* q, const uint16_t* pool,
                     int64_t num_blocks, const int32_t* bt, int64_t n_tokens, double scale,
                     double* o) {
  if (!shape_ok(s) || q_heads < s->kv_heads || q_heads % s->kv_heads != 0 || n_tokens < 1 ||
      num_blocks < 1)
    return CGO_ERR_INVALID_ARG;
  int H = s->kv_heads, D = s->head_dim, G = q_heads / s->kv_heads;
  for (int64_t t = 0; t < n_tokens; t += 16)
    if (bt[t / 16] < 0 || bt[t / 16] >= num_blocks) return CGO_ERR_INVALID_ARG;
  double* sc = (double*)malloc(sizeof(double) * (size_t)n_tokens);
  double* qf = (double*)malloc(sizeof(double) * (size_t)D);
  for (int l = 0; l < s->layers; l++)
    for (int qh = 0; qh < q_heads; qh++) {
      int h = qh / G;
      for (int d = 0; d < D; d++)
        qf[d] = elem_to_float(s->dtype, q[((size_t)l * q_heads + qh) * D + d]);
      double m = -INFINITY;
      for (int64_t t = 0; t < n_tokens; t++) {
        size_t kb = ((((size_t)l * 2 + 0) * (size_t)num_blocks + (size_t)bt[t / 16]) * H + h) * 16 +
                    (size_t)(t % 16);
        double acc = 0.0;
        for (int d = 0; d < D; d++) acc += qf[d] * (double)elem_to_float(s->dtype, pool[kb * D + d]);
        sc[t] = scale * acc;
        if (sc[t] > m) m = sc[t];
      }
      double den = 0.0;
      for (int64_t t = 0; t < n_tokens; t++) {
        sc[t] = exp(sc[t] - m);
        den += sc[t];
      }
      double* out = o + ((size_t)l * q_heads + qh) * D;
      for (int d = 0; d < D; d++) out[d] = 0.0;
      for (int64_t t = 0; t < n_tokens; t++) {
        size_t vb = ((((size_t)l * 2 + 1) * (size_t)num_blocks + (size_t)bt[t / 16]) * H + h) * 16 +
                    (size_t)(t % 16);
        for (int d = 0; d < D; d++) out[d] += sc[t] * (double)elem_to_float(s->dtype, pool[vb * D + d]);
      }
      for (int d = 0; d < D; d++) out[d] /= den;
    }
  free(sc);
  free(qf);
  return CGO_OK;
}
