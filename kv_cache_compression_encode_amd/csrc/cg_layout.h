// cg_layout.h -- byte layouts and launch-argument structs of the gfx950 codec
// library. Internal to the library (host API and kernels).
#pragma once

#include <stdint.h>

#include "../../include/cg.h"

namespace cg {

constexpr uint32_t kTableMagic = 0x42544743u;   // "CGTB"
constexpr uint32_t kRecordMagic = 0x4B434743u;  // "CGCK"
constexpr uint32_t kVersion = 1;
constexpr int kDtypeF16 = 0, kDtypeBf16 = 1;  // element types (shape.dtype)
constexpr uint32_t kTablesRobust = 1u;        // tables flag: unseen symbols escape
constexpr int kLanes = 64;           // channels per group = wavefront width
constexpr int kHdrWords = 192;       // state hi, state lo, raw q0: 3 x 64 words
constexpr uint32_t kM = 4096;        // 12-bit frequency total
constexpr uint32_t kL = 65536;       // rANS state lower bound
constexpr int kEsc = 255;
constexpr int kMaxLevels = 8;
constexpr int kMaxGroups = 255;
constexpr int kMaxLayers = 1024;

// Lookup tables are stored per "set" = the 64 channels of one (layer group,
// K|V, head, 64-dim slice), lane-minor: entry e of lane k is dword e*64 + k,
// so a wavefront reading "its" entries touches 64 different banks and a set
// is copied to LDS as one contiguous block.
// Decoder set (128 KB), per 32-slot word w of a lane's slot range:
//   above[w][64] : bit q (q >= 1) set when a symbol starts at slot 32w + 32 - q
//                  (the start bitmap reversed and shifted up by one), so
//                  popcount(above << (slot & 31)) counts starts after the slot;
//   rankx[w][64] : 256 * (symbols starting at or below slot 32w+31, minus 1)
//                  + byte address of the lane's info column;
//   info[256][64]: rank -> d | (4096 - f) << 8 | b << 20 with d = sym - 127 as
//                  a byte (0x80 = escape).
// info address = rankx[w] - 256 * popcount(above[w] << (slot & 31)).
// above and rankx lie in the first 64 KB so one ds_read2st64 fetches both.
constexpr int kDecDwords = 512;            // per channel
constexpr int kDecBm = 0, kDecRb = 128 * 64, kDecInfo = 256 * 64;  // dword offsets in a set
// Encoder set: [257 rows][64] of (16 f - 1) mod 2^16 | b << 16, indexed by
// the token delta d clamped to [-128, 128], plus 128: row r = 1..255 holds
// symbol r - 1 (d = r - 128), rows 0 and 256 the escape symbol's entry (d
// below -127 or above 127). A symbol that plain tables cannot code (f = 0,
// or an escape of f = 0) holds kEncInvalid. The escape symbol is the last
// in cumulative order, so its b, and hence its entry, exceeds every other
// coded symbol's: entry >= the escape's entry means "escape". 64.25 KB.
constexpr int kEncDwords = 257;            // per channel
constexpr uint32_t kEncInvalid = 0xFFFFFFFFu;
// Decoder ring per chain: 256 16-bit words refilled 128 at a time (one dword
// per lane), plus a 64-word mirror of words 0..63 so a read at
// (p mod 256) + k, k < 64, needs no wrap.
constexpr int kRingWords = 256;
constexpr int kRingMirror = 64;
constexpr int kRingBlock = 128;
constexpr int kChains = 3;  // at most this many groups decoded together by one wavefront
constexpr int kMaxRefsPerBlock = 3;  // records sharing one decode workgroup
constexpr int kWaves = 16;  // wavefronts per workgroup of the codec kernels

__host__ __device__ inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// ---- tables blob -----------------------------------------------------------
__host__ __device__ inline uint64_t tb_f_offset(int L, int G) {
  return align_up(64 + 4 * (uint64_t)G + (uint64_t)L, 256);
}
__host__ __device__ inline uint64_t tb_n_tables(int G, int H, int D) {
  return (uint64_t)G * 2 * H * D;
}
__host__ __device__ inline uint64_t tb_format_bytes(int L, int H, int D, int G) {
  return tb_f_offset(L, G) + tb_n_tables(G, H, D) * 512;
}
// Lookup section (not part of the format): per-group fast-quotient flags,
// encoder tables, decoder tables.
__host__ __device__ inline uint64_t tb_acc_offset(int L, int H, int D, int G) {
  return align_up(tb_format_bytes(L, H, D, G), 256);
}
__host__ __device__ inline uint64_t tb_qflag_offset(int L, int H, int D, int G) {
  return tb_acc_offset(L, H, D, G);
}
__host__ __device__ inline uint64_t tb_enc_offset(int L, int H, int D, int G) {
  return tb_acc_offset(L, H, D, G) + 1024;
}
__host__ __device__ inline uint64_t tb_dec_offset(int L, int H, int D, int G) {
  return tb_enc_offset(L, H, D, G) + tb_n_tables(G, H, D) * kEncDwords * 4;
}
__host__ __device__ inline uint64_t tb_total_bytes(int L, int H, int D, int G) {
  return tb_dec_offset(L, H, D, G) + tb_n_tables(G, H, D) * kDecDwords * 4;
}

// ---- chunk records ---------------------------------------------------------
__host__ __device__ inline int64_t n_chunks(int64_t T, int C) { return (T + C - 1) / C; }
__host__ __device__ inline int64_t chunk_len(int64_t T, int C, int64_t c) {
  int64_t n = T - c * C;
  return n < C ? n : C;
}
__host__ __device__ inline int64_t groups_per_chunk(int L, int H, int D) {
  return (int64_t)L * 2 * H * (D / 64);
}
__host__ __device__ inline uint64_t rec_data_start(int64_t gpc) {
  return align_up(64 + 8 * (uint64_t)(gpc + 1) + 4 * (uint64_t)gpc, 256);
}
// Worst case words of one group of n tokens: one renorm word and one escape
// word per symbol plus the 192-word head.
__host__ __device__ inline uint64_t group_cap_words(int64_t n) {
  return (uint64_t)kLanes * (2 * (uint64_t)(n - 1) + 3);
}

struct Shape {
  int L, H, D, C, S;  // S = D / 64 slices
  int64_t T;
  int dt;             // kDtypeF16 or kDtypeBf16
};

// ---- launch arguments --------------------------------------------------------
struct BlobInitArgs {
  uint8_t* blob;
  int L, H, D, G, C;
  int32_t level_id;
  int32_t dtype;
  uint32_t flags;
  int64_t T;
  float step[kMaxGroups + 1];
  uint8_t lg[kMaxLayers];
};

struct QCheckArgs {
  const uint8_t* blob;
  uint32_t* qflags;
  int L, G;
  bool bf;  // inputs are bfloat16
};

struct HistArgs {
  Shape s;
  const uint16_t* x;
  const uint8_t* blob;
  uint32_t* counts;      // [G][2][H][D][256]
  unsigned long long* stats;  // optional [4]
  int G;
};

struct NormArgs {
  const uint32_t* counts;
  uint8_t* blob;
  uint64_t f_off, enc_off, dec_off;
  int64_t n_tables;
  bool robust;  // kTablesRobust
};

struct EncodeArgs {
  Shape s;
  const uint16_t* x;
  const uint8_t* blob;
  int G;
  int64_t chunk_begin, n_chunks;
  // chunks [0, split) of the call go to workgroups in blocks of
  // chunks_per_block, the rest in blocks of chunks_per_block2
  int32_t chunks_per_block, split, chunks_per_block2;
  uint64_t cap_words;          // per group slot in the scratch
  uint16_t* scratch;           // [n_chunks][gpc][cap_words]
  uint32_t* group_words;       // [n_chunks][gpc]
  uint32_t* group_start;       // [n_chunks][gpc]
  int32_t* status;
};

struct LayoutArgs {
  int64_t gpc;
  int64_t n_chunks;
  const uint32_t* group_words;
  uint64_t* group_off;         // [n_chunks][gpc+1]
  uint64_t* rec_bytes;         // [n_chunks]
};

struct ChunkScanArgs {
  int64_t n_chunks;
  const uint64_t* rec_bytes;
  uint64_t* chunk_offsets;     // [n_chunks+1]
  uint64_t out_cap;
  int32_t* status;
};

struct WriteArgs {
  Shape s;
  int64_t gpc, chunk_begin, n_chunks;
  const uint8_t* blob;
  uint64_t cap_words;
  const uint16_t* scratch;
  const uint32_t* group_words;
  const uint32_t* group_start;
  const uint64_t* group_off;
  const uint64_t* rec_bytes;
  const uint64_t* chunk_offsets;
  uint8_t* out;
  uint64_t out_cap;
  int groups_per_block;
};

struct AttendArgs {
  Shape s;
  int q_heads, G;              // G = q_heads / kv_heads <= 16
  const uint16_t* q;           // [L][q_heads][D] element bits
  const uint16_t* pool;        // [L][2][num_blocks][H][16][D]
  int64_t num_blocks;
  const int32_t* bt;           // [ceil(n_tokens / 16)]
  int64_t n_tokens, n_pages;
  int32_t pages_per_wave;
  int64_t n_parts;             // partials per (layer, kv head)
  float scale_log2e;           // softmax scale * log2(e)
  float* part_ml;              // [L][H][n_parts][G][2]: running max (log2 units), sum
  float* part_o;               // [L][H][n_parts][G][D]: unnormalised output
  float* o;                    // [L][q_heads][D]
  int32_t* status;
};

struct DecodeArgs {
  Shape s;
  const cg_chunk_ref* refs;
  int32_t n_refs;
  // Records [0, split) go to workgroups in blocks of refs_per_block, the
  // rest in blocks of refs_per_block2 (all of a workgroup's records share
  // one table set); first-class blocks come first in launch order.
  int32_t refs_per_block;
  int32_t split;
  int32_t refs_per_block2;
  // per_level: the grid holds one copy of these blocks per table set, and a
  // block decodes only the records of its copy's set (records of several
  // levels in any order); otherwise a block's set is its first record's
  int32_t per_level;
  // workgroups per block of records and table set: a block's groups are
  // decoded 48 (16 wavefronts x 3 chains) per workgroup
  int32_t item_rounds;
  int32_t n_tables;
  int32_t g_max;
  const uint8_t* tables[kMaxLevels];
  int32_t level_id[kMaxLevels];
  int32_t n_groups[kMaxLevels];
  uint16_t* y;            // contiguous output (or null)
  uint16_t* pool;         // paged output (or null)
  int64_t num_blocks;
  const int32_t* block_table;
  int32_t* status;
};

// Launchers (defined next to the kernels).
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, uint64_t n, hipStream_t st);
hipError_t launch_blob_init(const BlobInitArgs& a, hipStream_t st);
hipError_t launch_qcheck(const QCheckArgs& a, hipStream_t st);
hipError_t launch_hist(const HistArgs& a, hipStream_t st);
hipError_t launch_norm(const NormArgs& a, hipStream_t st);
hipError_t launch_encode(const EncodeArgs& a, hipStream_t st);
hipError_t launch_layout(const LayoutArgs& a, hipStream_t st);
hipError_t launch_chunk_scan(const ChunkScanArgs& a, hipStream_t st);
hipError_t launch_write(const WriteArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, bool paged, hipStream_t st);
hipError_t launch_attend(const AttendArgs& a, hipStream_t st);
hipError_t launch_attend_reduce(const AttendArgs& a, hipStream_t st);
hipError_t launch_make_refs(const uint8_t* base, const uint64_t* offs, int32_t n, int32_t table,
                            cg_chunk_ref* refs, hipStream_t st);
hipError_t launch_copy(void* dst, const void* src, uint64_t bytes, hipStream_t st);
hipError_t launch_set_ref(cg_chunk_ref* ref, const uint8_t* record, uint64_t bytes, int32_t table,
                          hipStream_t st);

}  // namespace cg
