/*
 * Drives the CPU oracle (oracle/cg_oracle.c) through every entry point on
 * small seeded inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer: table build, chunk encode and decode
 * (contiguous and paged), the group coder, normalisation, attention, and the
 * error paths (capacity, corrupted and truncated records). Exits non-zero on
 * any mismatch; the sanitizers report memory and undefined-behaviour errors.
 * Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t layers, kv_heads, head_dim, chunk_tokens;
  int64_t tokens;
  int32_t dtype, reserved;
} cgo_shape;

int cgo_build_tables(const cgo_shape*, int32_t, int32_t, const uint8_t*, const float*, const uint16_t*,
                     uint32_t, uint8_t*, uint64_t, uint64_t[4]);
uint64_t cgo_tables_format_bytes(const cgo_shape*, int32_t);
int64_t cgo_encode_chunk(const cgo_shape*, const uint8_t*, const uint16_t*, int64_t, uint8_t*, uint64_t);
uint64_t cgo_record_bound(const cgo_shape*, int64_t);
int cgo_decode_chunk(const cgo_shape*, const uint8_t*, const uint8_t*, uint64_t, uint16_t*);
int cgo_decode_chunk_paged(const cgo_shape*, const uint8_t*, const uint8_t*, uint64_t, uint16_t*, int64_t,
                           const int32_t*);
int cgo_attend_paged(const cgo_shape*, int32_t, const uint16_t*, const uint16_t*, int64_t, const int32_t*,
                     int64_t, double, double*);
int64_t cgo_encode_group_q(const int32_t*, int64_t, const uint16_t* const[64], int, uint16_t*, int64_t);
int cgo_decode_group_q(const uint16_t*, int64_t, int64_t, const uint16_t* const[64], int32_t*);
void cgo_normalize(const uint64_t[256], uint16_t[256]);
void cgo_normalize_robust(const uint64_t[256], uint16_t[256]);
int32_t cgo_quantize_dt(int, uint16_t, float, int*, int*);
uint16_t cgo_dequantize_dt(int, int32_t, float);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double unif(void) { return (double)(next_u64() >> 11) / 9007199254740992.0; }

static int failures = 0;
#define CHECK(c, ...)                \
  do {                               \
    if (!(c)) {                      \
      failures++;                    \
      fprintf(stderr, __VA_ARGS__); \
      fputc('\n', stderr);           \
    }                                \
  } while (0)

/* element bits of a random-walk tensor, with rare wide jumps and specials */
static void fill(uint16_t* X, size_t n, int T, int D, int dtype, double spread) {
  for (size_t i = 0; i < n; i++) {
    int t = (int)((i / (size_t)D) % (size_t)T);
    uint16_t prev = t ? X[i - (size_t)D] : 0;
    uint16_t v;
    double u = unif();
    if (u < 0.002) {
      v = (uint16_t)next_u64(); /* any bit pattern: NaN, Inf, subnormal */
    } else if (dtype == 0) {
      v = (uint16_t)(prev + (uint16_t)((int)(spread * (unif() - 0.5))));
      if ((v & 0x7C00) == 0x7C00) v &= 0x3FFF;
    } else {
      v = (uint16_t)(prev + (uint16_t)((int)(spread * (unif() - 0.5))));
      if ((v & 0x7F80) == 0x7F80) v &= 0x3FFF;
    }
    X[i] = v;
  }
}

static void roundtrip(int L, int H, int D, int64_t T, int C, int G, int dtype, uint32_t flags, double spread) {
  cgo_shape s = {L, H, D, C, T, dtype, 0};
  size_t n = (size_t)L * 2 * H * (size_t)T * D;
  uint16_t* X = malloc(n * 2);
  uint16_t* Y = malloc(n * 2);
  fill(X, n, (int)T, D, dtype, spread);
  uint8_t lg[64];
  float steps[8];
  for (int l = 0; l < L; l++) lg[l] = (uint8_t)(l * G / L);
  for (int g = 0; g < G; g++) steps[g] = (float)(0.3 + 0.45 * g + 0.01 * (double)(next_u64() % 7));
  uint64_t fb = cgo_tables_format_bytes(&s, G);
  uint8_t* blob = malloc(fb);
  uint64_t st[4];
  CHECK(cgo_build_tables(&s, 3, G, lg, steps, X, flags, blob, fb - 1, st) == -3, "blob capacity");
  int rc = cgo_build_tables(&s, 3, G, lg, steps, X, flags, blob, fb, st);
  CHECK(rc == 0, "build_tables %d", rc);
  int64_t nch = (T + C - 1) / C;
  int64_t nb = (T + 15) / 16, NB = nb + 2;
  int32_t* bt = malloc(sizeof(int32_t) * (size_t)nb);
  for (int64_t i = 0; i < nb; i++) bt[i] = (int32_t)i;
  for (int64_t i = nb - 1; i > 0; i--) { /* permutation of [0, nb) */
    int64_t j = (int64_t)(next_u64() % (uint64_t)(i + 1));
    int32_t tmp = bt[i];
    bt[i] = bt[j];
    bt[j] = tmp;
  }
  size_t pool_n = (size_t)L * 2 * (size_t)NB * H * 16 * D;
  uint16_t* pool = calloc(pool_n, 2);
  for (int64_t c = 0; c < nch; c++) {
    uint64_t cap = cgo_record_bound(&s, c);
    uint8_t* rec = malloc(cap);
    CHECK(cgo_encode_chunk(&s, blob, X, c, rec, 64) == -3, "record capacity");
    int64_t m = cgo_encode_chunk(&s, blob, X, c, rec, cap);
    CHECK(m > 0 && (uint64_t)m <= cap, "encode_chunk %lld", (long long)m);
    if (m <= 0) {
      free(rec);
      continue;
    }
    CHECK(cgo_decode_chunk(&s, blob, rec, (uint64_t)m, Y) == 0, "decode_chunk");
    CHECK(cgo_decode_chunk_paged(&s, blob, rec, (uint64_t)m, pool, NB, bt) == 0, "decode_chunk_paged");
    CHECK(cgo_decode_chunk(&s, blob, rec, 40, Y) != 0, "short record accepted");
    /* damaged copies: any status, no crash */
    uint8_t* bad = malloc((size_t)m);
    for (int k = 0; k < 6; k++) {
      memcpy(bad, rec, (size_t)m);
      for (int f = 0; f < 1 + k; f++) bad[next_u64() % (uint64_t)m] ^= (uint8_t)(1u << (next_u64() % 8));
      (void)cgo_decode_chunk(&s, blob, bad, (uint64_t)m, Y);
    }
    free(bad);
    free(rec);
  }
  /* decoded = dequant(quant(x)) everywhere (the decode of the damaged copies
   * above may have written Y: decode every chunk again) */
  for (int64_t c = 0; c < nch; c++) {
    uint64_t cap = cgo_record_bound(&s, c);
    uint8_t* rec = malloc(cap);
    int64_t m = cgo_encode_chunk(&s, blob, X, c, rec, cap);
    if (m > 0) (void)cgo_decode_chunk(&s, blob, rec, (uint64_t)m, Y);
    free(rec);
  }
  size_t bad_el = 0;
  for (size_t i = 0; i < n; i++) {
    int l = (int)(i / ((size_t)2 * H * (size_t)T * D));
    float stp = steps[lg[l]];
    uint16_t want = cgo_dequantize_dt(dtype, cgo_quantize_dt(dtype, X[i], stp, 0, 0), stp);
    bad_el += Y[i] != want;
  }
  CHECK(bad_el == 0, "decoded elements differ: %zu", bad_el);
  /* attention over the paged pool */
  int qh = 2 * H;
  uint16_t* q = malloc(sizeof(uint16_t) * (size_t)L * qh * D);
  for (size_t i = 0; i < (size_t)L * qh * D; i++) q[i] = (uint16_t)(dtype ? 0x3F80 : 0x3C00) ^ (uint16_t)(next_u64() & 0x03FF);
  double* o = malloc(sizeof(double) * (size_t)L * qh * D);
  CHECK(cgo_attend_paged(&s, qh, q, pool, NB, bt, T, 1.0 / sqrt((double)D), o) == 0, "attend");
  free(q);
  free(o);
  free(pool);
  free(bt);
  free(blob);
  free(X);
  free(Y);
}

static void group_coder(void) {
  for (int rep = 0; rep < 30; rep++) {
    int64_t n = 1 + (int64_t)(next_u64() % 300);
    int32_t* q = malloc(sizeof(int32_t) * 64 * (size_t)n);
    int32_t* back = malloc(sizeof(int32_t) * 64 * (size_t)n);
    uint16_t fbuf[64][256];
    const uint16_t* f[64];
    uint64_t cnt[256];
    for (int k = 0; k < 64; k++) {
      int32_t v = (int32_t)(next_u64() % 65536) - 32768;
      memset(cnt, 0, sizeof(cnt));
      for (int64_t i = 0; i < n; i++) {
        int32_t d = (unif() < 0.05) ? (int32_t)(next_u64() % 65536) - 32768 : (int32_t)(next_u64() % 9) - 4;
        int32_t nv = v + d;
        nv = ((nv + 32768) % 65536 + 65536) % 65536 - 32768;
        if (i > 0) {
          int32_t w = ((nv - v + 32768) % 65536 + 65536) % 65536 - 32768;
          cnt[(w >= -127 && w <= 127) ? w + 127 : 255]++;
        }
        v = nv;
        q[k * n + i] = v;
      }
      if (rep % 2) cgo_normalize_robust(cnt, fbuf[k]);
      else cgo_normalize(cnt, fbuf[k]);
      f[k] = fbuf[k];
    }
    int64_t cap = 64 * (2 * (n - 1) + 3);
    uint16_t* w = malloc(sizeof(uint16_t) * (size_t)cap);
    int64_t m = cgo_encode_group_q(q, n, f, rep % 2, w, cap);
    CHECK(m >= 192 && m <= cap, "encode_group_q %lld", (long long)m);
    if (m > 0) {
      CHECK(cgo_decode_group_q(w, m, n, f, back) == 0, "decode_group_q");
      CHECK(memcmp(back, q, sizeof(int32_t) * 64 * (size_t)n) == 0, "group round trip");
      CHECK(cgo_decode_group_q(w, m - 1, n, f, back) != 0, "truncated stream accepted");
      CHECK(cgo_encode_group_q(q, n, f, rep % 2, w, 100) < 0 || m <= 100, "group capacity");
    }
    free(w);
    free(q);
    free(back);
  }
}

static void normalisation(void) {
  uint64_t cnt[256];
  uint16_t f[256];
  for (int rep = 0; rep < 200; rep++) {
    int nz = 1 + (int)(next_u64() % 256);
    memset(cnt, 0, sizeof(cnt));
    for (int k = 0; k < nz; k++) cnt[next_u64() % 256] = next_u64() >> (next_u64() % 64);
    if (rep % 3 == 0) memset(cnt, 0, sizeof(cnt));
    if (rep % 2) cgo_normalize_robust(cnt, f);
    else cgo_normalize(cnt, f);
    uint32_t sum = 0;
    for (int k = 0; k < 256; k++) sum += f[k];
    CHECK(sum == 4096, "normalised sum %u", sum);
  }
}

int main(void) {
  /* L, H, D, T, C, groups, dtype, flags, spread */
  roundtrip(4, 2, 64, 1000, 256, 3, 0, 0, 6.0);
  roundtrip(3, 1, 128, 300, 64, 2, 0, 1, 40.0);
  roundtrip(2, 1, 64, 37, 7, 1, 1, 0, 3.0);
  roundtrip(1, 3, 192, 100, 100, 1, 0, 0, 300.0);
  roundtrip(2, 2, 64, 1, 1, 2, 1, 1, 1.0);
  roundtrip(5, 1, 64, 129, 128, 3, 1, 0, 2000.0);
  group_coder();
  normalisation();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle harness: all checks passed\n");
  return 0;
}
