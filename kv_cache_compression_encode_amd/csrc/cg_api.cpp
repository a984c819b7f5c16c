// cg_api.cpp -- C ABI of the gfx950 KV-cache codec: argument checks, buffer
// sizing, workspace carving and kernel launches. No device memory is
// allocated here; every buffer comes from the caller.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <functional>
#include <mutex>
#include <utility>
#include <vector>

#include "cg_layout.h"

using namespace cg;

namespace {

// Shapes the kernels' index arithmetic and grids are sized for.
cg_status check_shape(const cg_shape* sp, Shape* out) {
  if (!sp) return CG_ERR_INVALID_ARG;
  const cg_shape& s = *sp;
  if (s.layers < 1 || s.kv_heads < 1 || s.head_dim < 1 || s.chunk_tokens < 1 || s.tokens < 1 ||
      (s.dtype != CG_DTYPE_F16 && s.dtype != CG_DTYPE_BF16) || s.reserved != 0)
    return CG_ERR_INVALID_ARG;
  if (s.head_dim % 64 != 0) return CG_ERR_UNSUPPORTED;
  if (s.layers > kMaxLayers || s.chunk_tokens > (1 << 20) || s.kv_heads > (1 << 16) ||
      s.head_dim > (1 << 16))
    return CG_ERR_UNSUPPORTED;
  if ((uint64_t)s.layers * (uint64_t)s.tokens >= (1ull << 32)) return CG_ERR_UNSUPPORTED;
  // per-(layer, K|V, head) slabs and per-chunk slices are addressed with
  // 32-bit buffer offsets
  if ((uint64_t)s.tokens * s.head_dim * 2 >= (1ull << 32)) return CG_ERR_UNSUPPORTED;
  const uint64_t gpc = (uint64_t)s.layers * 2 * s.kv_heads * (s.head_dim / 64);
  if (gpc >= (1ull << 31)) return CG_ERR_UNSUPPORTED;
  if (out) {
    out->L = s.layers;
    out->H = s.kv_heads;
    out->D = s.head_dim;
    out->C = s.chunk_tokens;
    out->S = s.head_dim / 64;
    out->T = s.tokens;
    out->dt = s.dtype;
  }
  return CG_OK;
}

cg_status check_level(const cg_level* lv, const Shape& s) {
  if (!lv || !lv->layer_group || !lv->step) return CG_ERR_INVALID_ARG;
  if (lv->n_groups < 1 || lv->n_groups > kMaxGroups) return CG_ERR_INVALID_ARG;
  if (lv->level_id < 0 || lv->level_id > 65535) return CG_ERR_INVALID_ARG;
  for (int l = 0; l < s.L; ++l)
    if (lv->layer_group[l] >= lv->n_groups) return CG_ERR_INVALID_ARG;
  for (int g = 0; g < lv->n_groups; ++g)
    if (!(lv->step[g] > 0.0f) || !std::isfinite(lv->step[g])) return CG_ERR_INVALID_ARG;
  return CG_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

cg_status hip_status(hipError_t e) { return e == hipSuccess ? CG_OK : CG_ERR_HIP; }

hipError_t mark(const cg_profile* prof, bool begin, hipStream_t st) {
  if (!prof) return hipSuccess;
  hipEvent_t ev = begin ? prof->main_begin : prof->main_end;
  return ev ? hipEventRecord(ev, st) : hipSuccess;
}

struct EncodeWs {
  uint64_t gw, gs, go, rb, scratch, total;
};

EncodeWs encode_ws_layout(const Shape& s, int64_t n_ch, uint64_t cap_words) {
  const uint64_t gpc = (uint64_t)groups_per_chunk(s.L, s.H, s.D);
  EncodeWs w;
  uint64_t o = 0;
  w.gw = o;
  o = align_up(o + 4 * gpc * n_ch, 256);
  w.gs = o;
  o = align_up(o + 4 * gpc * n_ch, 256);
  w.go = o;
  o = align_up(o + 8 * (gpc + 1) * n_ch, 256);
  w.rb = o;
  o = align_up(o + 8 * (uint64_t)n_ch, 256);
  w.scratch = o;
  o = align_up(o + 2 * cap_words * gpc * n_ch, 256);
  w.total = o;
  return w;
}

cg_status check_range(const Shape& s, int64_t cb, int64_t ce) {
  const int64_t nch = n_chunks(s.T, s.C);
  if (cb < 0 || ce <= cb || ce > nch) return CG_ERR_INVALID_ARG;
  return CG_OK;
}

}  // namespace

static int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

// Splits n_rec records (decode) or chunks (encode) of each of `sets` table
// sets into workgroups: records [0, split) in blocks of r1, the rest in
// blocks of r2, first-class blocks launched first. One workgroup fits a
// compute unit (its tables fill the LDS). The plan with the shortest
// simulated greedy dispatch (workgroups taken in launch order by the first
// free compute unit) wins. cost(r, last) is a workgroup's time for a block
// of r records, the last of which is `last` / 1024 of a full one.
struct BlockPlan {
  int r1 = 1, split = 0, r2 = 1;
};

// Greedy dispatch of equal-cost workgroups: each goes to the compute unit
// that frees first. The units' finish times are kept as (time, count) groups
// in ascending order, so a run of workgroups costs a few group moves instead
// of one heap operation per workgroup (the multiset of finish times, and so
// the span, is what the per-workgroup simulation gives).
struct Dispatch {
  std::vector<std::pair<int64_t, int64_t>> g;  // finish time -> units, ascending
  explicit Dispatch(int64_t cus) : g{{0, cus}} {}
  void add(int64_t t, int64_t c) {
    auto it = g.begin();
    while (it != g.end() && it->first < t) ++it;
    if (it != g.end() && it->first == t)
      it->second += c;
    else
      g.insert(it, {t, c});
  }
  void run(int64_t jobs, int64_t t) {
    while (jobs > 0) {
      const int64_t t0 = g.front().first, c = g.front().second;
      const int64_t k = c < jobs ? c : jobs;
      if (k == c)
        g.erase(g.begin());
      else
        g.front().second -= k;
      add(t0 + t, k);
      jobs -= k;
    }
  }
  int64_t span() const { return g.back().first; }
};

template <class Cost>
static BlockPlan plan_blocks(int cus, int64_t n_rec, int64_t sets, int max_r, int64_t last, Cost cost) {
  BlockPlan best;
  int64_t best_span = INT64_MAX;
  for (int r1 = 1; r1 <= max_r && r1 <= n_rec; ++r1) {
    for (int r2 = 1; r2 <= r1; ++r2) {
      for (int64_t split = 0; split <= n_rec; split += r1) {
        if (split == n_rec && r2 != 1) continue;  // no second class
        const int64_t n1 = split / r1, n2 = (n_rec - split + r2 - 1) / r2;
        const int64_t rem = (n_rec - split) % r2;
        Dispatch d(cus);
        if (n2 == 0) {
          d.run((n1 - 1) * sets, cost(r1, 1024));
          d.run(sets, cost(r1, last));
        } else {
          d.run(n1 * sets, cost(r1, 1024));
          d.run((n2 - 1) * sets, cost(r2, 1024));
          d.run(sets, cost(rem ? (int)rem : r2, last));  // the block with the last record
        }
        const int64_t span = d.span();
        if (span < best_span) {
          best_span = span;
          best.r1 = r1;
          best.split = (int)split;
          best.r2 = r2;
        }
      }
    }
  }
  return best;
}

static int max_layers_per_group(const Shape& s, const cg_level& lv) {
  int lg_max = 0;
  for (int g = 0; g < lv.n_groups; ++g) {
    int n = 0;
    for (int l = 0; l < s.L; ++l) n += lv.layer_group[l] == g;
    if (n > lg_max) lg_max = n;
  }
  return lg_max;
}

// length of the last of n records in 1/1024 chunk: a call covering the
// sequence's last chunk is taken to end with it (the plan only affects speed)
static int64_t last_len(const Shape& s, bool ends_at_last_chunk) {
  const int64_t nch = n_chunks(s.T, s.C);
  return ends_at_last_chunk ? chunk_len(s.T, s.C, nch - 1) * 1024 / s.C : 1024;
}

// Decode: a workgroup holds R records x (layers of its group) groups, dealt
// to its 16 wavefronts, so a wavefront runs c = ceil(items / 16) chains,
// at most three interleaved at a time (more in further rounds of three);
// workgroup times per chain count are measured on gfx950 (3 chains = 1000).
// A block ending with a short record runs all chains for that length, then
// one chain fewer.
static void plan_decode(const Shape& s, const cg_level& lv, int32_t n_refs, int cus, DecodeArgs* a) {
  static const int kWgCost[kChains + 1] = {0, 380, 710, 1000};
  const int lg_max = max_layers_per_group(s, lv);
  auto chains = [&](int r) { return (r * lg_max + kWaves - 1) / kWaves; };
  auto wg_cost = [&](int c) { return (int64_t)(c / kChains) * kWgCost[kChains] + kWgCost[c % kChains]; };
  int max_r = 1;
  while (max_r < kMaxRefsPerBlock && chains(max_r + 1) <= kChains) ++max_r;
  auto cost = [&](int r, int64_t last) {
    const int64_t rest = r > 1 ? wg_cost(chains(r - 1)) : 0;
    return wg_cost(chains(r)) * last / 1024 + rest * (1024 - last) / 1024 + 5;
  };
  const BlockPlan p = plan_blocks(cus, n_refs, (int64_t)lv.n_groups * 2 * s.H * s.S, max_r,
                                  last_len(s, n_refs == n_chunks(s.T, s.C)), cost);
  a->refs_per_block = p.r1;
  a->split = p.split;
  a->refs_per_block2 = p.r2;
  a->item_rounds = (int32_t)((p.r1 * lg_max + kWaves * kChains - 1) / (kWaves * kChains));
}

// Encode: a workgroup holds R chunks x (layers of its group) groups, dealt
// round-robin to its 16 wavefronts, which encode theirs one after another;
// its time is the longest wavefront's sum of chunk lengths.
static void plan_encode(const Shape& s, const cg_level& lv, int64_t chunk_end, int64_t n, EncodeArgs* a) {
  const int lg_max = max_layers_per_group(s, lv);
  auto cost = [&](int r, int64_t last) {
    int64_t worst = 0;
    for (int w = 0; w < kWaves; ++w) {
      int64_t sum = 0;
      for (int it = w; it < r * lg_max; it += kWaves) sum += it / lg_max == r - 1 ? last : 1024;
      worst = sum > worst ? sum : worst;
    }
    return worst + 5;
  };
  const BlockPlan p = plan_blocks(compute_units(), n, (int64_t)lv.n_groups * 2 * s.H * s.S, 4,
                                  last_len(s, chunk_end == n_chunks(s.T, s.C)), cost);
  a->chunks_per_block = p.r1;
  a->split = p.split;
  a->chunks_per_block2 = p.r2;
}

extern "C" {

int32_t cg_version(void) { return 1; }

const char* cg_status_string(cg_status st) {
  switch (st) {
    case CG_OK: return "ok";
    case CG_ERR_INVALID_ARG: return "invalid argument";
    case CG_ERR_UNSUPPORTED: return "unsupported shape or size";
    case CG_ERR_CAPACITY: return "output buffer too small";
    case CG_ERR_HIP: return "HIP launch or runtime error";
    case CG_ERR_CORRUPT: return "corrupt record or stream";
    case CG_ERR_TABLE: return "symbol missing from frequency table";
    default: return "unknown status";
  }
}

size_t cg_tables_bytes(const cg_shape* shape, int32_t n_groups) {
  Shape s;
  if (check_shape(shape, &s) != CG_OK || n_groups < 1 || n_groups > kMaxGroups) return 0;
  return (size_t)tb_total_bytes(s.L, s.H, s.D, n_groups);
}

size_t cg_tables_format_bytes(const cg_shape* shape, int32_t n_groups) {
  Shape s;
  if (check_shape(shape, &s) != CG_OK || n_groups < 1 || n_groups > kMaxGroups) return 0;
  return (size_t)tb_format_bytes(s.L, s.H, s.D, n_groups);
}

// ---- scratch of the allocation-free table build -----------------------------
// cg_build_tables_noalloc keeps the symbol counts in this file-scope device
// array instead of a caller workspace. Each GPU the library runs on holds its
// own copy until the process ends. In host code the name `scratch` is only a
// stand-in: its device address on each GPU comes from hipGetSymbolAddress
// (scratch_address below), and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[CG_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // per device: the array's device address

// The array's address on the current device, looked up on the first call
// on that device (with it current) and kept.
cg_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CG_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CG_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return CG_OK;
}
}  // namespace

size_t cg_build_workspace_bytes(const cg_shape* shape, int32_t n_groups) {
  Shape s;
  if (check_shape(shape, &s) != CG_OK || n_groups < 1 || n_groups > kMaxGroups) return 0;
  return (size_t)align_up(tb_n_tables(n_groups, s.H, s.D) * 256 * 4, 256);
}

cg_status cg_build_tables(const cg_shape* shape, const cg_level* level, const uint16_t* x_dev,
                          void* tables_dev, void* ws_dev, size_t ws_bytes, uint32_t flags,
                          uint64_t* stats_dev, const cg_profile* prof, hipStream_t stream) {
  Shape s;
  cg_status rc = check_shape(shape, &s);
  if (rc != CG_OK) return rc;
  if (flags & ~(uint32_t)CG_TABLES_ROBUST) return CG_ERR_INVALID_ARG;
  if ((rc = check_level(level, s)) != CG_OK) return rc;
  if (!x_dev || !tables_dev || !ws_dev || !aligned(x_dev, 2) || !aligned(tables_dev, 256) ||
      !aligned(ws_dev, 256) || (stats_dev && !aligned(stats_dev, 8)))
    return CG_ERR_INVALID_ARG;
  const int G = level->n_groups;
  if (ws_bytes < cg_build_workspace_bytes(shape, G)) return CG_ERR_INVALID_ARG;
  const uint64_t ntab = tb_n_tables(G, s.H, s.D);
  if ((uint64_t)s.L * 2 * s.H * s.S >= (1ull << 31) || ntab / 4 + 1 >= (1ull << 31))
    return CG_ERR_UNSUPPORTED;

  uint32_t* counts = static_cast<uint32_t*>(ws_dev);
  uint8_t* blob = static_cast<uint8_t*>(tables_dev);
  hipError_t e = launch_fill_u32(counts, 0, ntab * 256, stream);
  if (e == hipSuccess && stats_dev)
    e = launch_fill_u32(reinterpret_cast<uint32_t*>(stats_dev), 0, 8, stream);
  if (e != hipSuccess) return CG_ERR_HIP;

  BlobInitArgs bi;
  std::memset(&bi, 0, sizeof(bi));
  bi.blob = blob;
  bi.L = s.L;
  bi.H = s.H;
  bi.D = s.D;
  bi.G = G;
  bi.C = s.C;
  bi.level_id = level->level_id;
  bi.dtype = s.dt;
  bi.flags = flags;
  bi.T = s.T;
  for (int g = 0; g < G; ++g) bi.step[g] = level->step[g];
  for (int l = 0; l < s.L; ++l) bi.lg[l] = level->layer_group[l];
  if ((e = launch_blob_init(bi, stream)) != hipSuccess) return CG_ERR_HIP;

  QCheckArgs qa;
  qa.blob = blob;
  qa.qflags = reinterpret_cast<uint32_t*>(blob + tb_qflag_offset(s.L, s.H, s.D, G));
  qa.L = s.L;
  qa.G = G;
  qa.bf = s.dt == kDtypeBf16;
  if ((e = launch_qcheck(qa, stream)) != hipSuccess) return CG_ERR_HIP;

  HistArgs ha;
  ha.s = s;
  ha.x = x_dev;
  ha.blob = blob;
  ha.counts = counts;
  ha.stats = reinterpret_cast<unsigned long long*>(stats_dev);
  ha.G = G;
  if ((e = mark(prof, true, stream)) != hipSuccess) return CG_ERR_HIP;
  if ((e = launch_hist(ha, stream)) != hipSuccess) return CG_ERR_HIP;
  if ((e = mark(prof, false, stream)) != hipSuccess) return CG_ERR_HIP;

  NormArgs na;
  na.counts = counts;
  na.blob = blob;
  na.f_off = tb_f_offset(s.L, G);
  na.enc_off = tb_enc_offset(s.L, s.H, s.D, G);
  na.dec_off = tb_dec_offset(s.L, s.H, s.D, G);
  na.n_tables = (int64_t)ntab;
  na.robust = (flags & CG_TABLES_ROBUST) != 0;
  return hip_status(launch_norm(na, stream));
}

cg_status cg_build_tables_noalloc(const cg_shape* shape, const cg_level* level, const uint16_t* x_dev,
                                  void* tables_dev, uint32_t flags, uint64_t* stats_dev,
                                  const cg_profile* prof, hipStream_t stream) {
  Shape s;
  cg_status rc = check_shape(shape, &s);
  if (rc != CG_OK) return rc;
  if ((rc = check_level(level, s)) != CG_OK) return rc;
  const size_t need = cg_build_workspace_bytes(shape, level->n_groups);
  if (need == 0) return CG_ERR_INVALID_ARG;
  if (need > CG_NOALLOC_SCRATCH_BYTES) return CG_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != CG_OK) return rc;
  // the counts are cleared by cg_build_tables' own fill kernel
  return cg_build_tables(shape, level, x_dev, tables_dev, ws, CG_NOALLOC_SCRATCH_BYTES, flags, stats_dev, prof,
                         stream);
}

size_t cg_encode_bound(const cg_shape* shape, int64_t chunk_begin, int64_t chunk_end) {
  Shape s;
  if (check_shape(shape, &s) != CG_OK || check_range(s, chunk_begin, chunk_end) != CG_OK) return 0;
  const int64_t gpc = groups_per_chunk(s.L, s.H, s.D);
  uint64_t total = 0;
  for (int64_t c = chunk_begin; c < chunk_end; ++c) {
    const uint64_t g = align_up(2 * group_cap_words(chunk_len(s.T, s.C, c)), 16);
    total += align_up(rec_data_start(gpc) + g * (uint64_t)gpc, 256);
  }
  return (size_t)total;
}

size_t cg_encode_workspace_bytes(const cg_shape* shape, int64_t chunk_begin, int64_t chunk_end) {
  Shape s;
  if (check_shape(shape, &s) != CG_OK || check_range(s, chunk_begin, chunk_end) != CG_OK) return 0;
  const uint64_t cap = group_cap_words(chunk_len(s.T, s.C, chunk_begin));
  return (size_t)encode_ws_layout(s, chunk_end - chunk_begin, cap).total;
}

cg_status cg_encode(const cg_shape* shape, const cg_level* level, const void* tables_dev,
                    const uint16_t* x_dev, int64_t chunk_begin, int64_t chunk_end,
                    uint8_t* out_dev, uint64_t out_cap, uint64_t* chunk_offsets_dev, void* ws_dev,
                    size_t ws_bytes, int32_t* status_dev, const cg_profile* prof,
                    hipStream_t stream) {
  Shape s;
  cg_status rc = check_shape(shape, &s);
  if (rc != CG_OK) return rc;
  if ((rc = check_level(level, s)) != CG_OK) return rc;
  if ((rc = check_range(s, chunk_begin, chunk_end)) != CG_OK) return rc;
  if (!tables_dev || !x_dev || !out_dev || !chunk_offsets_dev || !ws_dev || !status_dev ||
      !aligned(tables_dev, 256) || !aligned(x_dev, 2) || !aligned(out_dev, 256) ||
      !aligned(chunk_offsets_dev, 8) || !aligned(ws_dev, 256) || !aligned(status_dev, 4))
    return CG_ERR_INVALID_ARG;
  const int64_t n = chunk_end - chunk_begin;
  const uint64_t cap = group_cap_words(chunk_len(s.T, s.C, chunk_begin));
  const EncodeWs w = encode_ws_layout(s, n, cap);
  if (ws_bytes < w.total) return CG_ERR_INVALID_ARG;
  const int G = level->n_groups;
  const int64_t gpc = groups_per_chunk(s.L, s.H, s.D);
  if ((uint64_t)n * G * 2 * s.H * s.S >= (1ull << 31) || cap >= (1ull << 32)) return CG_ERR_UNSUPPORTED;
  const int gpb = 4;  // groups per copy block (one per wavefront)
  if ((uint64_t)n * (1 + (gpc + gpb - 1) / gpb) >= (1ull << 31)) return CG_ERR_UNSUPPORTED;

  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(status_dev), 0, 1, stream);
  if (e != hipSuccess) return CG_ERR_HIP;

  EncodeArgs ea;
  ea.s = s;
  ea.x = x_dev;
  ea.blob = static_cast<const uint8_t*>(tables_dev);
  ea.G = G;
  ea.chunk_begin = chunk_begin;
  ea.n_chunks = n;
  ea.cap_words = cap;
  plan_encode(s, *level, chunk_end, n, &ea);
  ea.scratch = reinterpret_cast<uint16_t*>(ws + w.scratch);
  ea.group_words = reinterpret_cast<uint32_t*>(ws + w.gw);
  ea.group_start = reinterpret_cast<uint32_t*>(ws + w.gs);
  ea.status = status_dev;
  if ((e = mark(prof, true, stream)) != hipSuccess) return CG_ERR_HIP;
  if ((e = launch_encode(ea, stream)) != hipSuccess) return CG_ERR_HIP;
  if ((e = mark(prof, false, stream)) != hipSuccess) return CG_ERR_HIP;

  LayoutArgs la;
  la.gpc = gpc;
  la.n_chunks = n;
  la.group_words = ea.group_words;
  la.group_off = reinterpret_cast<uint64_t*>(ws + w.go);
  la.rec_bytes = reinterpret_cast<uint64_t*>(ws + w.rb);
  if ((e = launch_layout(la, stream)) != hipSuccess) return CG_ERR_HIP;

  ChunkScanArgs ca;
  ca.n_chunks = n;
  ca.rec_bytes = la.rec_bytes;
  ca.chunk_offsets = chunk_offsets_dev;
  ca.out_cap = out_cap;
  ca.status = status_dev;
  if ((e = launch_chunk_scan(ca, stream)) != hipSuccess) return CG_ERR_HIP;

  WriteArgs wa;
  wa.s = s;
  wa.gpc = gpc;
  wa.chunk_begin = chunk_begin;
  wa.n_chunks = n;
  wa.blob = ea.blob;
  wa.cap_words = cap;
  wa.scratch = ea.scratch;
  wa.group_words = ea.group_words;
  wa.group_start = ea.group_start;
  wa.group_off = la.group_off;
  wa.rec_bytes = la.rec_bytes;
  wa.chunk_offsets = chunk_offsets_dev;
  wa.out = out_dev;
  wa.out_cap = out_cap;
  wa.groups_per_block = gpb;
  return hip_status(launch_write(wa, stream));
}

cg_status cg_make_refs(const uint8_t* base_dev, const uint64_t* offsets_dev, int32_t n,
                       int32_t table, cg_chunk_ref* refs_dev, hipStream_t stream) {
  if (!base_dev || !offsets_dev || !refs_dev || n < 1 || table < 0 || table >= kMaxLevels ||
      !aligned(offsets_dev, 8) || !aligned(refs_dev, 8))
    return CG_ERR_INVALID_ARG;
  return hip_status(launch_make_refs(base_dev, offsets_dev, n, table, refs_dev, stream));
}

static cg_status decode_common(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                               const void* const* tables_dev, const cg_chunk_ref* refs_dev,
                               int32_t n_refs, int32_t* status_dev, DecodeArgs* a) {
  Shape s;
  cg_status rc = check_shape(shape, &s);
  if (rc != CG_OK) return rc;
  if (n_levels < 1 || n_levels > kMaxLevels || !levels || !tables_dev || !refs_dev || n_refs < 1 ||
      !status_dev || !aligned(refs_dev, 8) || !aligned(status_dev, 4))
    return CG_ERR_INVALID_ARG;
  std::memset(a, 0, sizeof(*a));
  int g_max = 0;
  for (int k = 0; k < n_levels; ++k) {
    if ((rc = check_level(&levels[k], s)) != CG_OK) return rc;
    if (!tables_dev[k] || !aligned(tables_dev[k], 256)) return CG_ERR_INVALID_ARG;
    for (int k2 = 0; k2 < k; ++k2)
      if (levels[k2].level_id == levels[k].level_id && tables_dev[k2] != tables_dev[k])
        return CG_ERR_INVALID_ARG;
    a->tables[k] = static_cast<const uint8_t*>(tables_dev[k]);
    a->level_id[k] = levels[k].level_id;
    a->n_groups[k] = levels[k].n_groups;
    if (levels[k].n_groups > g_max) g_max = levels[k].n_groups;
  }
  if ((uint64_t)n_refs * g_max * 2 * s.H * s.S * n_levels * ((s.L + kWaves * kChains - 1) / (kWaves * kChains)) >=
      (1ull << 31))
    return CG_ERR_UNSUPPORTED;
  a->s = s;
  a->refs = refs_dev;
  a->n_refs = n_refs;
  // several levels: records of a workgroup must share a table set, and which
  // set each record names is on the device, so every block of records is
  // launched once per set and decodes its records of that set; the blocks
  // are sized for the level with the most layers per group (runs of records
  // of one level fill them)
  int widest = 0;
  for (int k = 1; k < n_levels; ++k)
    if (max_layers_per_group(s, levels[k]) > max_layers_per_group(s, levels[widest])) widest = k;
  plan_decode(s, levels[widest], n_refs, compute_units(), a);
  a->per_level = n_levels > 1;
  a->n_tables = n_levels;
  a->g_max = g_max;
  a->status = status_dev;
  return CG_OK;
}

cg_status cg_decode_plan(const cg_shape* shape, int32_t n_levels, const cg_level* levels, int32_t n_refs,
                         int32_t compute_units_hint, int32_t* out_host) {
  Shape s;
  cg_status rc = check_shape(shape, &s);
  if (rc != CG_OK) return rc;
  if (!levels || !out_host || n_levels < 1 || n_levels > kMaxLevels || n_refs < 1) return CG_ERR_INVALID_ARG;
  for (int k = 0; k < n_levels; ++k)
    if ((rc = check_level(&levels[k], s)) != CG_OK) return rc;
  int widest = 0;  // as in decode_common
  for (int k = 1; k < n_levels; ++k)
    if (max_layers_per_group(s, levels[k]) > max_layers_per_group(s, levels[widest])) widest = k;
  DecodeArgs a;
  plan_decode(s, levels[widest], n_refs, compute_units_hint > 0 ? compute_units_hint : compute_units(), &a);
  out_host[0] = a.refs_per_block;
  out_host[1] = a.split;
  out_host[2] = a.refs_per_block2;
  return CG_OK;
}

cg_status cg_decode(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                    const void* const* tables_dev, const cg_chunk_ref* refs_dev, int32_t n_refs,
                    uint16_t* y_dev, int32_t* status_dev, const cg_profile* prof,
                    hipStream_t stream) {
  DecodeArgs a;
  cg_status rc = decode_common(shape, n_levels, levels, tables_dev, refs_dev, n_refs, status_dev, &a);
  if (rc != CG_OK) return rc;
  if (!y_dev || !aligned(y_dev, 2)) return CG_ERR_INVALID_ARG;
  a.y = y_dev;
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(status_dev), 0, 1, stream);
  if (e == hipSuccess) e = mark(prof, true, stream);
  if (e == hipSuccess) e = launch_decode(a, false, stream);
  if (e == hipSuccess) e = mark(prof, false, stream);
  return hip_status(e);
}

cg_status cg_decode_paged(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                          const void* const* tables_dev, const cg_chunk_ref* refs_dev,
                          int32_t n_refs, uint16_t* pool_dev, int64_t num_blocks,
                          const int32_t* block_table_dev, int32_t* status_dev,
                          const cg_profile* prof, hipStream_t stream) {
  DecodeArgs a;
  cg_status rc = decode_common(shape, n_levels, levels, tables_dev, refs_dev, n_refs, status_dev, &a);
  if (rc != CG_OK) return rc;
  if (!pool_dev || !aligned(pool_dev, 2) || num_blocks < 1 || num_blocks >= (1ll << 31) ||
      !block_table_dev || !aligned(block_table_dev, 4))
    return CG_ERR_INVALID_ARG;
  // one (layer, K|V) slab of the pool is addressed with 32-bit buffer offsets
  if ((uint64_t)num_blocks * shape->kv_heads * 16 * shape->head_dim * 2 >= (1ull << 32))
    return CG_ERR_UNSUPPORTED;
  a.pool = pool_dev;
  a.num_blocks = num_blocks;
  a.block_table = block_table_dev;
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(status_dev), 0, 1, stream);
  if (e == hipSuccess) e = mark(prof, true, stream);
  if (e == hipSuccess) e = launch_decode(a, true, stream);
  if (e == hipSuccess) e = mark(prof, false, stream);
  return hip_status(e);
}

// Attention: pages per wavefront so that about 16K wavefronts share the
// work (at least 4, at most 64 pages each: one block-table entry per lane).
static int32_t attend_pages_per_wave(const Shape& s, int64_t n_pages) {
  const int64_t total = (int64_t)s.L * s.H * n_pages;
  const int64_t ppw = (total + 16383) / 16384;
  return (int32_t)std::min<int64_t>(64, std::max<int64_t>(4, ppw));
}

static cg_status attend_args(const cg_shape* shape, int32_t q_heads, int64_t n_tokens, AttendArgs* a) {
  Shape s;
  cg_status rc = check_shape(shape, &s);
  if (rc != CG_OK) return rc;
  if (q_heads < s.H || q_heads % s.H != 0 || n_tokens < 1 || n_tokens >= (1ll << 40))
    return CG_ERR_INVALID_ARG;
  if (q_heads / s.H > 16 || (s.D != 64 && s.D != 128 && s.D != 256) || (int64_t)q_heads * s.L >= (1ll << 31))
    return CG_ERR_UNSUPPORTED;
  std::memset(a, 0, sizeof(*a));
  a->s = s;
  a->q_heads = q_heads;
  a->G = q_heads / s.H;
  a->n_tokens = n_tokens;
  a->n_pages = (n_tokens + 15) / 16;
  a->pages_per_wave = attend_pages_per_wave(s, a->n_pages);
  a->n_parts = (a->n_pages + a->pages_per_wave - 1) / a->pages_per_wave;
  return CG_OK;
}

size_t cg_attend_workspace_bytes(const cg_shape* shape, int32_t q_heads, int64_t n_tokens) {
  AttendArgs a;
  if (attend_args(shape, q_heads, n_tokens, &a) != CG_OK) return 0;
  const uint64_t slots = (uint64_t)a.s.L * a.s.H * a.n_parts * a.G;
  return (size_t)(align_up(slots * 2 * 4, 256) + align_up(slots * a.s.D * 4, 256));
}

cg_status cg_attend_paged(const cg_shape* shape, int32_t q_heads, const uint16_t* q_dev,
                          const uint16_t* pool_dev, int64_t num_blocks, const int32_t* block_table_dev,
                          int64_t n_tokens, float scale, float* o_dev, void* ws_dev, size_t ws_bytes,
                          int32_t* status_dev, const cg_profile* prof, hipStream_t stream) {
  AttendArgs a;
  cg_status rc = attend_args(shape, q_heads, n_tokens, &a);
  if (rc != CG_OK) return rc;
  if (!q_dev || !aligned(q_dev, 16) || !pool_dev || !aligned(pool_dev, 16) || num_blocks < 1 ||
      num_blocks >= (1ll << 31) || !block_table_dev || !aligned(block_table_dev, 4) || !o_dev ||
      !aligned(o_dev, 4) || !ws_dev || !aligned(ws_dev, 256) || !status_dev || !aligned(status_dev, 4) ||
      !(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return CG_ERR_INVALID_ARG;
  if (ws_bytes < cg_attend_workspace_bytes(shape, q_heads, n_tokens)) return CG_ERR_INVALID_ARG;
  const uint64_t slots = (uint64_t)a.s.L * a.s.H * a.n_parts * a.G;
  a.q = q_dev;
  a.pool = pool_dev;
  a.num_blocks = num_blocks;
  a.bt = block_table_dev;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.part_ml = static_cast<float*>(ws_dev);
  a.part_o = reinterpret_cast<float*>(static_cast<uint8_t*>(ws_dev) + align_up(slots * 2 * 4, 256));
  a.o = o_dev;
  a.status = status_dev;
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(status_dev), 0, 1, stream);
  if (e == hipSuccess) e = mark(prof, true, stream);
  if (e == hipSuccess) e = launch_attend(a, stream);
  if (e == hipSuccess) e = mark(prof, false, stream);
  if (e == hipSuccess) e = launch_attend_reduce(a, stream);
  return hip_status(e);
}

cg_status cg_stream_decode_paged(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                                 const void* const* tables_dev, const uint8_t* records_host,
                                 const uint64_t* offsets_host, const int32_t* table_of_record_host,
                                 int32_t n_records, uint8_t* staging_dev, uint64_t staging_bytes,
                                 cg_chunk_ref* refs_dev, uint16_t* pool_dev, int64_t num_blocks,
                                 const int32_t* block_table_dev, int32_t* status_dev,
                                 hipStream_t stream, hipStream_t copy_stream) {
  DecodeArgs a;
  cg_status rc = decode_common(shape, n_levels, levels, tables_dev, refs_dev, 1, status_dev, &a);
  if (rc != CG_OK) return rc;
  if (!records_host || !offsets_host || n_records < 1 || !staging_dev || !aligned(staging_dev, 256) ||
      !pool_dev || !aligned(pool_dev, 2) || num_blocks < 1 || num_blocks >= (1ll << 31) ||
      !block_table_dev || !aligned(block_table_dev, 4))
    return CG_ERR_INVALID_ARG;
  if ((uint64_t)num_blocks * shape->kv_heads * 16 * shape->head_dim * 2 >= (1ull << 32))
    return CG_ERR_UNSUPPORTED;
  uint64_t max_rec = 0;
  for (int32_t k = 0; k < n_records; ++k) {
    if (offsets_host[k + 1] < offsets_host[k]) return CG_ERR_INVALID_ARG;
    const uint64_t b = offsets_host[k + 1] - offsets_host[k];
    if (b > max_rec) max_rec = b;
    if (table_of_record_host && (table_of_record_host[k] < 0 || table_of_record_host[k] >= n_levels))
      return CG_ERR_INVALID_ARG;
  }
  const uint64_t half = align_up(max_rec, 256);
  if (2 * half > staging_bytes) return CG_ERR_INVALID_ARG;
  a.pool = pool_dev;
  a.num_blocks = num_blocks;
  a.block_table = block_table_dev;

  hipEvent_t copied[2] = {nullptr, nullptr}, consumed[2] = {nullptr, nullptr};
  hipError_t e = hipSuccess;
  for (int k = 0; k < 2 && e == hipSuccess; ++k) {
    e = hipEventCreateWithFlags(&copied[k], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&consumed[k], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = launch_fill_u32(reinterpret_cast<uint32_t*>(status_dev), 0, 1, stream);
  // the first copy may only overwrite staging once earlier work on `stream` is done
  if (e == hipSuccess) e = hipEventRecord(consumed[0], stream);
  if (e == hipSuccess) e = hipEventRecord(consumed[1], stream);
  for (int32_t k = 0; k < n_records && e == hipSuccess; ++k) {
    const int slot = k & 1;
    uint8_t* dst = staging_dev + slot * half;
    const uint64_t bytes = offsets_host[k + 1] - offsets_host[k];
    // receive: wait until the slot's previous record has been decoded
    e = hipStreamWaitEvent(copy_stream, consumed[slot], 0);
    if (e == hipSuccess)
      e = hipMemcpyAsync(dst, records_host + offsets_host[k], bytes, hipMemcpyHostToDevice, copy_stream);
    if (e == hipSuccess) e = hipEventRecord(copied[slot], copy_stream);
    // decode + fill on `stream` once the record has landed
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, copied[slot], 0);
    if (e == hipSuccess)
      e = launch_set_ref(refs_dev + slot, dst, bytes, table_of_record_host ? table_of_record_host[k] : 0,
                         stream);
    if (e == hipSuccess) {
      a.refs = refs_dev + slot;
      a.n_refs = 1;
      a.refs_per_block = 1;
      a.split = 0;
      a.refs_per_block2 = 1;
      a.per_level = 0;  // one record: its own set
      e = launch_decode(a, true, stream);
    }
    if (e == hipSuccess) e = hipEventRecord(consumed[slot], stream);
  }
  for (int k = 0; k < 2; ++k) {
    if (copied[k]) (void)hipEventDestroy(copied[k]);
    if (consumed[k]) (void)hipEventDestroy(consumed[k]);
  }
  return hip_status(e);
}

// Bandwidth a level needs, in Gbit/s ("CacheGen实战" 2.2: the sender
// switches to a cheaper level as the measured link slows; reading of the
// page's garbled thresholds): level k is taken when the measured bandwidth
// exceeds kLevelNeedGbps[k], trying the highest quality first; the last
// level (fast) needs nothing. A NaN bandwidth exceeds nothing.
static const double kLevelNeedGbps[] = {5.0, 1.0};
static const int32_t kLevels = (int32_t)(sizeof(kLevelNeedGbps) / sizeof(kLevelNeedGbps[0])) + 1;

int32_t cg_select_level(double bandwidth_gbps) {
  int32_t k = 0;
  while (k < kLevels - 1 && !(bandwidth_gbps > kLevelNeedGbps[k])) ++k;
  return k;
}

cg_status cg_recency_levels(int64_t n_chunks, int64_t near_chunks, int64_t far_chunks,
                            int32_t* levels_host) {
  if (!levels_host || n_chunks < 1 || near_chunks < 0 || far_chunks < near_chunks)
    return CG_ERR_INVALID_ARG;
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t dist = n_chunks - 1 - c;
    levels_host[c] = dist < near_chunks ? 0 : (dist >= far_chunks ? 2 : 1);
  }
  return CG_OK;
}

cg_status cg_copy(void* dst_dev, const void* src_dev, uint64_t bytes, hipStream_t stream) {
  if (!dst_dev || !src_dev || bytes % 16 != 0 || !aligned(dst_dev, 16) || !aligned(src_dev, 16))
    return CG_ERR_INVALID_ARG;
  return hip_status(launch_copy(dst_dev, src_dev, bytes, stream));
}

}  // extern "C"
