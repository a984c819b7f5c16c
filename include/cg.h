/*
 * cg.h -- C ABI of the MI355X (gfx950) CacheGen-style KV-cache codec.
 *
 * The codec compresses an fp16 K/V cache in three steps that the pages
 * describe ("CacheGen实战：KV缓存压缩与流式传输在大型语言模型服务中的高效应用",
 * section 1): quantize with one step per layer group (fine in shallow layers,
 * coarse in deep ones), store token-to-token differences, and entropy-code
 * the differences group by group. The context is cut into chunks (section
 * 2.1: 1.5K tokens) that are encoded, shipped and decoded independently, and
 * the receiver decodes on the GPU straight into the model's cache (section
 * 2.3), which may be paged ("vLLM中的PagedAttention优化" in the KV-cache
 * optimisation article: physical blocks found through a block table).
 *
 * Bit-level definition (the pages leave it open; these are the readings):
 *   x      = fp16 or bfloat16 element ("CacheGen：大语言模型推理加速的KV缓存压缩
 *            与流式传输技术解析", 「KV缓存的量化压缩机制」: the cache is FP16/BF16)
 *   q      = clamp(round_half_even(fl32(x / step[group(layer)])), -32768, 32767), NaN -> 0
 *   d_0    = q[first token of the chunk] (raw);  d_i = wrap16(q_i - q_{i-1})
 *   symbol = d_i + 127 if |d_i| <= 127, else 255 (escape) + raw u16(d_i);
 *            with robust tables also 255 + raw u16(d_i) when the table gives
 *            d_i + 127 frequency 0
 *   tables = per (layer group, K|V, head, dim) symbol counts, normalised to
 *            12-bit frequencies (sum 4096)
 *   coder  = static rANS, 32-bit state in [2^16, 2^32), 16-bit words; a group
 *            = (chunk, layer, K|V, head, 64-dim slice), lane k codes dim
 *            64*slice + k, 64 lanes interleaved word by word
 *   x_hat  = round_half_even to the element type of fl32(float(q) * step)
 *
 * Layouts (all little-endian, element = fp16 or bfloat16 bits as uint16_t):
 *   KV tensor  x[layer][2 (K,V)][kv_head][token][head_dim]
 *   paged pool pool[layer][2][num_blocks][kv_head][16][head_dim]
 *   tables blob, chunk record: see cg_tables_format_bytes / cg_encode.
 *
 * Conventions for every call:
 *   - Pointers named *_dev are device pointers the CALLER allocates and owns;
 *     the library allocates no device memory and keeps no state between calls.
 *   - Calls are asynchronous and ordered on `stream`. The return value only
 *     reports argument checks and launch failures (CG_ERR_INVALID_ARG,
 *     CG_ERR_UNSUPPORTED, CG_ERR_HIP). Errors that depend on data are written
 *     to the device word *status_dev (0 = OK, else a CG_ERR_* code); the call
 *     first resets it to 0. Read it after synchronising the stream.
 *   - Alignment: tables, workspaces, containers and refs must be 256-byte
 *     aligned; x / y / pool must be 2-byte aligned.
 *   - Two calls that share an output or workspace buffer and overlap in time
 *     race; ordering on one stream is enough.
 */
#ifndef CG_H_
#define CG_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t cg_status;
#define CG_OK 0
#define CG_ERR_INVALID_ARG (-1) /* bad argument, shape, pointer or block-table entry */
#define CG_ERR_UNSUPPORTED (-2) /* valid but outside the library's limits          */
#define CG_ERR_CAPACITY (-3)    /* output buffer too small (encode)                  */
#define CG_ERR_HIP (-4)         /* a HIP launch or runtime call failed                */
#define CG_ERR_CORRUPT (-5)     /* a record or stream failed its integrity checks      */
#define CG_ERR_TABLE (-6)       /* a symbol to encode has frequency 0 in the table     */

/* Element types (cg_shape.dtype). */
#define CG_DTYPE_F16 0
#define CG_DTYPE_BF16 1

/* cg_build_tables flags. CG_TABLES_ROBUST: tables meant for tensors other
 * than the one they are built from (calibration data; "CacheGen：…技术解析",
 * 「量化编码器设计」: per-channel statistics drive the coder). The escape
 * symbol keeps a frequency of at least 1 (one unit moves to it from the
 * largest frequency, lowest symbol on ties, when the data had no escape),
 * and cg_encode codes a delta whose symbol has frequency 0 as an escape
 * instead of failing with CG_ERR_TABLE. Decoding is unchanged. */
#define CG_TABLES_ROBUST 1u

/* Shape of one KV cache. head_dim must be a multiple of 64. Limits:
 * layers <= 1024, layers*tokens < 2^32, chunk_tokens <= 1<<20. */
typedef struct cg_shape {
  int32_t layers;       /* L */
  int32_t kv_heads;     /* H */
  int32_t head_dim;     /* D */
  int32_t chunk_tokens; /* C: delta-reset and record unit ("CacheGen实战" 2.1: 1536) */
  int64_t tokens;       /* T */
  int32_t dtype;        /* CG_DTYPE_F16 or CG_DTYPE_BF16: elements of x, y and pool */
  int32_t reserved;     /* 0 */
} cg_shape;

/* One quality level ("CacheGen实战" 3.1: high 0.3/0.8/1.2, balanced
 * 0.5/1.0/1.5, fast 0.8/1.5/2.0). Host pointers. */
typedef struct cg_level {
  int32_t level_id;           /* stored in tables and records, 0..65535        */
  int32_t n_groups;           /* G, 1..255                                      */
  const uint8_t* layer_group; /* [layers], each < n_groups                      */
  const float* step;          /* [n_groups], finite and > 0                      */
} cg_level;

/* Where one chunk record lives, for the decoders. Device array. */
typedef struct cg_chunk_ref {
  const uint8_t* record; /* device pointer to a record written by cg_encode, 256-B aligned */
  uint64_t bytes;        /* readable bytes at `record` (>= the record's size)               */
  int32_t table;         /* index into the decoder's levels / tables arrays                 */
  int32_t reserved;      /* 0                                                             */
} cg_chunk_ref;

/* Optional timing hook. When a call gets a non-null cg_profile, it records
 * main_begin right before and main_end right after its main kernel (k_hist for
 * cg_build_tables, k_encode for cg_encode, k_decode for the decoders) on the
 * call's stream. The events are created and owned by the caller. */
typedef struct cg_profile {
  hipEvent_t main_begin;
  hipEvent_t main_end;
} cg_profile;

/* Library version (1) and a readable name for a status code. */
int32_t cg_version(void);
const char* cg_status_string(cg_status s);

/* ---- frequency tables -------------------------------------------------- */

/* Bytes of a tables blob for `n_groups` layer groups (format section plus the
 * decoder/encoder lookup section that follows it), or 0 for a bad shape. */
size_t cg_tables_bytes(const cg_shape* shape, int32_t n_groups);

/* Bytes of the format section alone: the part a file or another
 * implementation must reproduce. Layout: 64-byte header ("CGTB", version,
 * layers, kv_heads, head_dim, n_groups, level_id, chunk_tokens, tokens u64,
 * f_offset, dtype, format_bytes u64, flags, 0), f32 step[G], u8
 * layer_group[L], zero pad to f_offset (256-aligned), u16 f[G][2][H][D][256].
 * Encoders and decoders take a blob only for a shape of the same layers,
 * kv_heads, head_dim and dtype; tokens and chunk_tokens may differ (tables
 * built on calibration data). */
size_t cg_tables_format_bytes(const cg_shape* shape, int32_t n_groups);

/* Workspace of cg_build_tables (symbol counts), or 0 for a bad shape. */
size_t cg_build_workspace_bytes(const cg_shape* shape, int32_t n_groups);

/* Per-channel statistics ("CacheGen：…技术解析", 「量化编码器设计」: statistics
 * per channel, entropy coding of the integer indices; "CacheGen实战"
 * section 1: grouped entropy coding). Counts the symbols of tokens 1..n-1 of
 * every chunk of x_dev per (layer group, K|V, head, dim), normalises each
 * table to 12 bits and writes the blob to tables_dev (cg_tables_bytes).
 * flags: 0 or CG_TABLES_ROBUST (other bits: CG_ERR_INVALID_ARG).
 * stats_dev (optional, u64[4]) receives {elements, saturated, nan, escapes}.
 * Data errors: none. */
cg_status cg_build_tables(const cg_shape* shape, const cg_level* level, const uint16_t* x_dev,
                          void* tables_dev, void* ws_dev, size_t ws_bytes, uint32_t flags,
                          uint64_t* stats_dev, const cg_profile* prof, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): as
 * cg_build_tables, but the symbol counts live in a static device array of
 * CG_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends, so no workspace argument is needed and the call
 * allocates nothing. Returns CG_ERR_UNSUPPORTED when the counts
 * (cg_build_workspace_bytes) exceed that size (a 7B-shape level of three
 * layer groups needs 25.2 MB), CG_ERR_HIP if the array's address cannot be
 * found. Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (other streams, other threads) race; the array is
 * cleared at the start of each call. */
#define CG_NOALLOC_SCRATCH_BYTES (32u << 20)
cg_status cg_build_tables_noalloc(const cg_shape* shape, const cg_level* level, const uint16_t* x_dev,
                                  void* tables_dev, uint32_t flags, uint64_t* stats_dev,
                                  const cg_profile* prof, hipStream_t stream);

/* ---- encode -------------------------------------------------------------- */

/* Worst-case bytes of the records of chunks [chunk_begin, chunk_end). */
size_t cg_encode_bound(const cg_shape* shape, int64_t chunk_begin, int64_t chunk_end);

/* Workspace of cg_encode for that chunk range, or 0 for a bad range. */
size_t cg_encode_workspace_bytes(const cg_shape* shape, int64_t chunk_begin, int64_t chunk_end);

/* Encodes chunks [chunk_begin, chunk_end) of x_dev with the tables of one
 * level ("CacheGen实战" 2.1: every chunk is pre-encoded per quality level).
 * Writes the chunk records back to back to out_dev and their byte offsets to
 * chunk_offsets_dev[0 .. n] (u64, offsets[n] = total). A record is: 64-byte
 * header ("CGCK", version, chunk_index, level_id, token_start u64, n_tokens,
 * n_groups, layers, kv_heads, head_dim, data_start, record_bytes u64,
 * data_bytes u64), u64 group_offset[n_groups+1] (from the data start,
 * multiples of 16), u32 group_words[n_groups], zero pad to data_start
 * (256-aligned), the group word streams in (layer, K|V, head, slice) order
 * each zero-padded to 16 bytes, zero pad to record_bytes (256-aligned).
 * Data errors: CG_ERR_CAPACITY (total > out_cap; offsets still hold the
 * needed sizes, out_dev is not written), CG_ERR_TABLE, CG_ERR_INVALID_ARG
 * (tables blob does not match the shape). */
cg_status cg_encode(const cg_shape* shape, const cg_level* level, const void* tables_dev,
                    const uint16_t* x_dev,
                    int64_t chunk_begin, int64_t chunk_end, uint8_t* out_dev, uint64_t out_cap,
                    uint64_t* chunk_offsets_dev, void* ws_dev, size_t ws_bytes,
                    int32_t* status_dev, const cg_profile* prof, hipStream_t stream);

/* Fills refs_dev[i] = {base_dev + offsets_dev[i], offsets_dev[i+1] - offsets_dev[i],
 * table, 0} for i < n (a helper to decode what cg_encode wrote). */
cg_status cg_make_refs(const uint8_t* base_dev, const uint64_t* offsets_dev, int32_t n,
                       int32_t table, cg_chunk_ref* refs_dev, hipStream_t stream);

/* ---- decode -------------------------------------------------------------- */

/* Decodes the records named by refs_dev[0 .. n_refs) into the contiguous
 * tensor y_dev ("CacheGen实战" 2.3: parallel GPU decode). Record i is read
 * with tables_dev[refs[i].table], which must have been built for
 * levels[refs[i].table]; records of different levels may be mixed (section
 * 2.1), in any order (a record's header names its chunk). With one level,
 * up to three consecutive references share a workgroup; with several, each
 * table set's records share workgroups in reference order however the
 * levels interleave. Only the token ranges of the given chunks are written.
 * n_levels <= 8. levels and tables_dev are host arrays; tables_dev[k] is a
 * device pointer. Data errors: CG_ERR_CORRUPT (bad record header, group
 * offsets, final rANS state or word count), CG_ERR_INVALID_ARG (table index
 * out of range, blob not matching its level). */
cg_status cg_decode(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                    const void* const* tables_dev, const cg_chunk_ref* refs_dev, int32_t n_refs,
                    uint16_t* y_dev, int32_t* status_dev, const cg_profile* prof,
                    hipStream_t stream);

/* As cg_decode, but the destination is a paged cache: token t of layer l,
 * K|V kv, head h goes to pool_dev[l][kv][block_table_dev[t/16]][h][t%16][:]
 * ("vLLM中的PagedAttention优化": non-contiguous physical blocks). The block
 * table is indexed by absolute token block, int32 [ceil(tokens/16)]. Pool
 * entries of other blocks are not touched. Data errors: as cg_decode, plus
 * CG_ERR_INVALID_ARG when an entry used by a chunk is outside
 * [0, num_blocks) (that chunk is then not written). */
cg_status cg_decode_paged(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                          const void* const* tables_dev, const cg_chunk_ref* refs_dev,
                          int32_t n_refs, uint16_t* pool_dev, int64_t num_blocks,
                          const int32_t* block_table_dev, int32_t* status_dev,
                          const cg_profile* prof, hipStream_t stream);

/* The dispatch plan cg_decode and cg_decode_paged launch for n_refs records
 * of these levels (host only, no device work). A decode workgroup holds the
 * decoder tables of one table set (one layer group, K|V, head and 64-dim
 * slice) and decodes that set's groups of a block of records; records
 * [0, split) go in blocks of records_per_block, the rest in blocks of
 * records_per_block2, and a block's groups are dealt to 16 wavefronts that
 * decode up to three of them at a time as interleaved chains (a layer group
 * of more than 48 layers takes several rounds). The plan minimises a
 * simulated dispatch over compute_units compute units; compute_units <= 0
 * means those of the current device (256 when no device is visible), which
 * is what the decoders plan with. Writes out_host[3] = {records_per_block,
 * split, records_per_block2}. Returns CG_ERR_INVALID_ARG for n_refs < 1, a
 * null pointer or n_levels outside 1..8, and the shape and level checks of
 * cg_decode. */
cg_status cg_decode_plan(const cg_shape* shape, int32_t n_levels, const cg_level* levels, int32_t n_refs,
                         int32_t compute_units, int32_t* out_host);

/* Streaming fill of a paged cache ("CacheGen实战" 2.3: a receive stage, a
 * parallel GPU decode stage and a fill stage run as a pipeline). Records
 * [0, n_records) lie in host memory at records_host + offsets_host[k]
 * (offsets_host has n_records+1 entries; records_host should be pinned, else
 * the copies are synchronous). Record k is copied host-to-device into one of
 * two halves of staging_dev on copy_stream while record k-1 is decoded into
 * pool_dev on stream; table_of_record_host[k] (or 0 when NULL) selects its
 * level. staging_bytes must hold two copies of the largest record;
 * refs_dev holds 2 cg_chunk_ref. Returns after enqueueing all work; the last
 * decode is ordered on stream. Data errors: as cg_decode_paged. */
cg_status cg_stream_decode_paged(const cg_shape* shape, int32_t n_levels, const cg_level* levels,
                                 const void* const* tables_dev, const uint8_t* records_host,
                                 const uint64_t* offsets_host, const int32_t* table_of_record_host,
                                 int32_t n_records, uint8_t* staging_dev, uint64_t staging_bytes,
                                 cg_chunk_ref* refs_dev, uint16_t* pool_dev, int64_t num_blocks,
                                 const int32_t* block_table_dev, int32_t* status_dev,
                                 hipStream_t stream, hipStream_t copy_stream);

/* ---- level policies (host only, no device work) ---------------------------- */

/* Level for one chunk from the bandwidth measured for its transfer, in Gbit/s
 * ("CacheGen实战" 2.2: the sender watches the link and switches compression
 * level). Returns 0 (high quality) above 5 Gbit/s, 1 (balanced) above
 * 1 Gbit/s up to 5, else 2 (fast). The page's comparison operators are
 * garbled; this is the reading. A NaN bandwidth gives 2. The page's fall back
 * to sending text and recomputing the cache is not part of the codec. */
int32_t cg_select_level(double bandwidth_gbps);

/* Recency-based level schedule (the CacheGen technical analysis, dynamic bit
 * allocation: cache close to the generation position keeps more precision).
 * Chunk c of n_chunks lies n_chunks - 1 - c chunks behind the newest one; it
 * gets level 0 (high) when that distance is below near_chunks, level 2
 * (fast) when it is at least far_chunks, else level 1 (balanced). Writes
 * levels_host[n_chunks]. Returns CG_ERR_INVALID_ARG unless
 * 0 <= near_chunks <= far_chunks and n_chunks >= 1. */
cg_status cg_recency_levels(int64_t n_chunks, int64_t near_chunks, int64_t far_chunks,
                            int32_t* levels_host);

/* ---- measurement helper ---------------------------------------------------- */

/* ---- attention over the restored cache -------------------------------- */

/* The consumer of the decoded cache ("CacheGen实战" 2.3: the decoded KV is
 * filled into the model's cache and used unchanged; "vLLM中的PagedAttention
 * 优化": K and V read from 16-token physical blocks through a block table).
 * One new token per layer: for every layer l and query head qh (which reads
 * kv head qh / (q_heads / kv_heads)),
 *   o[l][qh][:] = sum_t softmax_t(scale * q[l][qh] . K[l][t]) V[l][t],  t < n_tokens,
 * with K[l][t] = pool[l][0][bt[t/16]][h][t%16][:], V likewise from pool[l][1].
 *   q_dev    elements of shape->dtype, [layers][q_heads][head_dim], 16-byte aligned
 *   pool_dev [layers][2][num_blocks][kv_heads][16][head_dim] (as cg_decode_paged), 16-byte aligned
 *   o_dev    fp32 [layers][q_heads][head_dim]
 *   ws_dev   cg_attend_workspace_bytes (per-wavefront partial results), 256-byte aligned
 * Limits: q_heads a multiple of kv_heads, at most 16 query heads per kv head
 * (CG_ERR_UNSUPPORTED otherwise), head_dim 64, 128 or 256, n_tokens >= 1.
 * Scores take fp32 sums of exact 16-bit products (matrix cores), the softmax
 * and the weighted sum of V are fp32; the result agrees with the exact value
 * to within a bound stated with the tests. A block-table entry outside
 * [0, num_blocks) writes CG_ERR_INVALID_ARG to *status_dev (its page is
 * skipped). prof (optional) brackets the main kernel (k_attend). */
size_t cg_attend_workspace_bytes(const cg_shape* shape, int32_t q_heads, int64_t n_tokens);
cg_status cg_attend_paged(const cg_shape* shape, int32_t q_heads, const uint16_t* q_dev,
                          const uint16_t* pool_dev, int64_t num_blocks, const int32_t* block_table_dev,
                          int64_t n_tokens, float scale, float* o_dev, void* ws_dev, size_t ws_bytes,
                          int32_t* status_dev, const cg_profile* prof, hipStream_t stream);

/* Plain device copy of `bytes` (a multiple of 16) with the library's launch
 * style; used to calibrate achievable bandwidth and HBM counters. */
cg_status cg_copy(void* dst_dev, const void* src_dev, uint64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CG_H_ */
