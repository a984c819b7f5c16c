// Drives the host side of libcg (argument checks, size queries, the dispatch
// planner, workspace carving and launch-argument setup) without a GPU, for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer: the kernel
// launchers are replaced by stubs that record their arguments and do no
// device work, and every pointer handed to the library is a fake, aligned
// device address it never dereferences. Exits non-zero on a failed check.
// Test infrastructure only.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "../../kv_cache_compression_encode_amd/csrc/cg_layout.h"

using namespace cg;

static int failures = 0;
#define CHECK(c, ...)                \
  do {                               \
    if (!(c)) {                      \
      ++failures;                    \
      std::fprintf(stderr, __VA_ARGS__); \
      std::fputc('\n', stderr);      \
    }                                \
  } while (0)

namespace cg {
static DecodeArgs g_dec;
static EncodeArgs g_enc;
static WriteArgs g_wr;
static int g_launches = 0;
hipError_t launch_fill_u32(uint32_t*, uint32_t, uint64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_blob_init(const BlobInitArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qcheck(const QCheckArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_hist(const HistArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_norm(const NormArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_encode(const EncodeArgs& a, hipStream_t) { ++g_launches; g_enc = a; return hipSuccess; }
hipError_t launch_layout(const LayoutArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_chunk_scan(const ChunkScanArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_write(const WriteArgs& a, hipStream_t) { ++g_launches; g_wr = a; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs& a, bool, hipStream_t) { ++g_launches; g_dec = a; return hipSuccess; }
hipError_t launch_attend(const AttendArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_attend_reduce(const AttendArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_make_refs(const uint8_t*, const uint64_t*, int32_t, int32_t, cg_chunk_ref*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_copy(void*, const void*, uint64_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_set_ref(cg_chunk_ref*, const uint8_t*, uint64_t, int32_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace cg

static void* fake(uintptr_t k) { return reinterpret_cast<void*>(0x7f0000000000ull + (k << 20)); }

struct Lv {
  std::vector<uint8_t> lg;
  std::vector<float> st;
  cg_level c;
  Lv(int L, int G, int id = 1) : lg(L), st(G) {
    for (int l = 0; l < L; ++l) lg[l] = (uint8_t)((int64_t)l * G / L);
    for (int g = 0; g < G; ++g) st[g] = 0.3f + 0.4f * g;
    c.level_id = id;
    c.n_groups = G;
    c.layer_group = lg.data();
    c.step = st.data();
  }
};

static cg_shape shape(int L, int H, int D, int64_t T, int C, int dt = 0) {
  cg_shape s;
  std::memset(&s, 0, sizeof(s));
  s.layers = L;
  s.kv_heads = H;
  s.head_dim = D;
  s.tokens = T;
  s.chunk_tokens = C;
  s.dtype = dt;
  return s;
}

static void planner() {
  const int Ls[] = {1, 2, 4, 11, 16, 17, 32, 33, 48, 49, 64, 100, 255, 1024};
  const int cus[] = {1, 8, 80, 256, 304, 1024};
  int n = 0;
  for (int L : Ls)
    for (int G : {1, 2, 3, 7})
      for (int H : {1, 8, 32})
        for (int D : {64, 128, 192}) {
          if (G > L) continue;
          cg_shape s = shape(L, H, D, 1 << 14, 1536);
          Lv lv(L, G);
          const int nch = (int)((s.tokens + s.chunk_tokens - 1) / s.chunk_tokens);
          for (int nref : {1, 2, 3, 5, nch}) {
            for (int cu : cus) {
              int32_t out[3] = {0, 0, 0};
              cg_status rc = cg_decode_plan(&s, 1, &lv.c, nref, cu, out);
              CHECK(rc == CG_OK, "plan rc %d", rc);
              CHECK(out[0] >= 1 && out[0] <= kMaxRefsPerBlock && out[2] >= 1 && out[2] <= out[0] &&
                        out[1] >= 0 && out[1] <= nref && out[1] % out[0] == 0,
                    "plan L%d G%d H%d D%d n%d cus%d: %d %d %d", L, G, H, D, nref, cu, out[0], out[1], out[2]);
              ++n;
            }
          }
        }
  std::printf("planner: %d plans\n", n);
}

static void decode_setup() {
  for (int L : {4, 48, 64, 100}) {
    cg_shape s = shape(L, 8, 128, 32768, 1536);
    Lv lv(L, L >= 3 ? 3 : 1);
    const void* tabs[1] = {fake(1)};
    int32_t n = 22;
    g_launches = 0;
    cg_status rc = cg_decode(&s, 1, &lv.c, tabs, (const cg_chunk_ref*)fake(2), n, (uint16_t*)fake(3),
                             (int32_t*)fake(4), nullptr, 0);
    CHECK(rc == CG_OK, "decode rc %d", rc);
    CHECK(g_launches == 2, "decode launches %d", g_launches);
    const DecodeArgs& a = g_dec;
    int lg_max = 0;
    for (int g = 0; g < lv.c.n_groups; ++g) {
      int c = 0;
      for (int l = 0; l < L; ++l) c += lv.lg[l] == g;
      lg_max = c > lg_max ? c : lg_max;
    }
    CHECK(a.item_rounds * kWaves * kChains >= a.refs_per_block * lg_max, "item rounds %d", a.item_rounds);
    const uint64_t rblocks = (uint64_t)(a.split / a.refs_per_block) +
                             (uint64_t)(a.n_refs - a.split + a.refs_per_block2 - 1) / a.refs_per_block2;
    const uint64_t blocks = rblocks * a.g_max * 2 * a.s.H * a.s.S * a.item_rounds;
    CHECK(blocks > 0 && blocks < (1ull << 31), "grid %llu", (unsigned long long)blocks);
    rc = cg_decode_paged(&s, 1, &lv.c, tabs, (const cg_chunk_ref*)fake(2), n, (uint16_t*)fake(3), 2048,
                         (const int32_t*)fake(5), (int32_t*)fake(4), nullptr, 0);
    CHECK(rc == CG_OK, "decode_paged rc %d", rc);
  }
}

static void encode_setup() {
  for (int L : {4, 48, 64}) {
    cg_shape s = shape(L, 8, 128, 32768, 1536);
    Lv lv(L, 3);
    for (int64_t cb : {0, 5, 21}) {
      const int64_t ce = cb == 21 ? 22 : cb + 3;
      const size_t ws = cg_encode_workspace_bytes(&s, cb, ce);
      const size_t bound = cg_encode_bound(&s, cb, ce);
      CHECK(ws > 0 && bound > 0, "encode sizes");
      cg_status rc = cg_encode(&s, &lv.c, fake(1), (const uint16_t*)fake(2), cb, ce, (uint8_t*)fake(3), bound,
                               (uint64_t*)fake(4), fake(5), ws, (int32_t*)fake(6), nullptr, 0);
      CHECK(rc == CG_OK, "encode rc %d", rc);
      CHECK(g_enc.chunks_per_block >= 1 && g_enc.split % g_enc.chunks_per_block == 0, "encode plan");
      rc = cg_encode(&s, &lv.c, fake(1), (const uint16_t*)fake(2), cb, ce, (uint8_t*)fake(3), bound,
                     (uint64_t*)fake(4), fake(5), ws - 1, (int32_t*)fake(6), nullptr, 0);
      CHECK(rc == CG_ERR_INVALID_ARG, "short encode workspace accepted");
    }
  }
}

static void sizes_and_checks() {
  // limits: largest layer count, tokens near the 32-bit slab limit
  cg_shape big = shape(1024, 1, 64, (1ll << 22) - 1, 1 << 20);
  CHECK(cg_tables_bytes(&big, 255) > 0, "big tables");
  CHECK(cg_encode_bound(&big, 0, 4) > 0, "big bound");
  cg_shape over = shape(1024, 1, 64, 1ll << 22, 1 << 20);
  CHECK(cg_tables_bytes(&over, 3) == 0, "layers x tokens >= 2^32 accepted");
  cg_shape ok = shape(4, 2, 64, 1024, 256);
  CHECK(cg_tables_bytes(&ok, 0) == 0 && cg_tables_bytes(&ok, 256) == 0, "group count");
  cg_shape b = ok;
  b.head_dim = 65;
  CHECK(cg_tables_bytes(&b, 3) == 0, "head_dim 65");
  b = ok;
  b.dtype = 2;
  CHECK(cg_tables_bytes(&b, 3) == 0, "dtype 2");
  b = ok;
  b.reserved = 1;
  CHECK(cg_tables_bytes(&b, 3) == 0, "reserved");
  b = ok;
  b.chunk_tokens = 0;
  CHECK(cg_tables_bytes(&b, 3) == 0, "chunk 0");
  CHECK(cg_attend_workspace_bytes(&ok, 3, 100) == 0 && cg_attend_workspace_bytes(&ok, 4, 100) > 0, "attend ws");
  // levels with bad groups or steps
  Lv lv(4, 2);
  lv.lg[3] = 2;
  CHECK(cg_build_tables(&ok, &lv.c, (const uint16_t*)fake(1), fake(2), fake(3), 1 << 24, 0, nullptr, nullptr,
                        0) == CG_ERR_INVALID_ARG,
        "layer group out of range");
  Lv lv2(4, 2);
  lv2.st[1] = std::numeric_limits<float>::quiet_NaN();
  CHECK(cg_build_tables(&ok, &lv2.c, (const uint16_t*)fake(1), fake(2), fake(3), 1 << 24, 0, nullptr, nullptr,
                        0) == CG_ERR_INVALID_ARG,
        "NaN step");
  Lv lv3(4, 2);
  CHECK(cg_build_tables(&ok, &lv3.c, (const uint16_t*)fake(1), fake(2), fake(3), 1 << 24, 2, nullptr, nullptr,
                        0) == CG_ERR_INVALID_ARG,
        "unknown flag");
  CHECK(cg_build_tables(&ok, &lv3.c, (const uint16_t*)fake(1), (uint8_t*)fake(2) + 4, fake(3), 1 << 24, 0,
                        nullptr, nullptr, 0) == CG_ERR_INVALID_ARG,
        "misaligned tables");
  g_launches = 0;
  CHECK(cg_build_tables(&ok, &lv3.c, (const uint16_t*)fake(1), fake(2), fake(3), 1 << 24, 0, nullptr, nullptr,
                        0) == CG_OK,
        "build");
  CHECK(g_launches == 5, "build launches %d", g_launches);  // counts, header, quotient check, hist, norm
  cg_shape wide = shape(64, 8, 128, 1024, 256);
  Lv lw(64, 64);
  CHECK(cg_build_tables_noalloc(&wide, &lw.c, (const uint16_t*)fake(1), fake(2), 0, nullptr, nullptr, 0) ==
            CG_ERR_UNSUPPORTED,
        "noalloc size limit");
  // decoders: bad level counts, null refs, zero refs
  const void* tabs[1] = {fake(1)};
  CHECK(cg_decode(&ok, 0, &lv3.c, tabs, (const cg_chunk_ref*)fake(2), 4, (uint16_t*)fake(3), (int32_t*)fake(4),
                  nullptr, 0) == CG_ERR_INVALID_ARG,
        "no levels");
  CHECK(cg_decode(&ok, 1, &lv3.c, tabs, nullptr, 4, (uint16_t*)fake(3), (int32_t*)fake(4), nullptr, 0) ==
            CG_ERR_INVALID_ARG,
        "null refs");
  CHECK(cg_decode_paged(&ok, 1, &lv3.c, tabs, (const cg_chunk_ref*)fake(2), 4, (uint16_t*)fake(3), 0,
                        (const int32_t*)fake(5), (int32_t*)fake(4), nullptr, 0) == CG_ERR_INVALID_ARG,
        "no pool blocks");
  CHECK(cg_stream_decode_paged(&ok, 1, &lv3.c, tabs, nullptr, nullptr, nullptr, 4, (uint8_t*)fake(6), 1 << 20,
                               (cg_chunk_ref*)fake(2), (uint16_t*)fake(3), 64, (const int32_t*)fake(5),
                               (int32_t*)fake(4), 0, 0) == CG_ERR_INVALID_ARG,
        "stream without host records");
  // level policies
  CHECK(cg_select_level(std::nan("")) == 2 && cg_select_level(-1.0) == 2 && cg_select_level(1.0) == 2 &&
            cg_select_level(1.0000001) == 1 && cg_select_level(5.0) == 1 && cg_select_level(5.0000001) == 0 &&
            cg_select_level(INFINITY) == 0,
        "select_level");
  std::vector<int32_t> lev(100);
  CHECK(cg_recency_levels(100, 10, 40, lev.data()) == CG_OK && lev[99] == 0 && lev[0] == 2, "recency");
  CHECK(cg_recency_levels(100, 41, 40, lev.data()) == CG_ERR_INVALID_ARG, "recency order");
  CHECK(cg_recency_levels(0, 1, 2, lev.data()) == CG_ERR_INVALID_ARG, "recency empty");
}

int main() {
  planner();
  decode_setup();
  encode_setup();
  sizes_and_checks();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host harness: all checks passed\n");
  return 0;
}
