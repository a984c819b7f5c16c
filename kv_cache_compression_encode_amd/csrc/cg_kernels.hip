// cg_kernels.hip -- gfx950 (CDNA4, wave64) kernels of the KV-cache codec.
//
// Method (CacheGen实战：KV缓存压缩与流式传输在大型语言模型服务中的高效应用):
//   section 1   quantize per layer group, token deltas, grouped entropy coding
//   section 2.1 1.5K-token chunks, one record per chunk and quality level
//   section 2.3 parallel GPU decode filling the model's (paged) KV cache
// The A100 decoder the page mentions (one CUDA thread per token) is not the
// design here: a token-delta prefix is sequential per channel, so on CDNA4
// one wavefront owns 64 channels of one (chunk, layer, K|V, head) and walks
// the tokens, each lane running its own rANS state; the 64 streams share one
// interleaved word stream placed with ballot + mbcnt prefix counts.
//
// Kernels
//   k_fill_u32     fill (no hipMemset, so calls stay capturable)
//   k_blob_init    tables-blob header, steps, layer groups
//   k_qcheck       per layer group: is x*(1/step), or failing that a two-term
//                  reciprocal, exact for all 65536 inputs of the element type?
//                  (else the IEEE divide is used)
//   k_hist         quantize + delta + symbol, LDS-privatised 64 x 256 counts
//   k_norm         one wavefront per table: 12-bit normalisation, cumulative
//                  frequencies, encoder / decoder lookup tables
//   k_encode       one wavefront per group: backward rANS over the tokens,
//                  words placed backward in a per-group scratch slot
//   k_layout       per chunk: scan of padded group sizes
//   k_chunk_scan   scan of record sizes -> chunk offsets, capacity check
//   k_write        record headers + compaction of the group streams
//   k_decode<P>    fused rANS decode + token prefix + dequantize + store
//                  (P: contiguous or through the block table into 16-token pages)
// Element types: fp16 or bfloat16 (the KV cache holds either: "CacheGen：
// 大语言模型推理加速的KV缓存压缩与流式传输技术解析", 「KV缓存的量化压缩机制」);
// the kernels that touch elements take the type as a template parameter BF.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "cg_layout.h"

namespace cg {

// ---------------------------------------------------------------------------
// wavefront helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, int lane) {
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x - v;
}

// arg max over the wave with the lowest index winning ties
__device__ __forceinline__ void wave_argmax(uint32_t& val, uint32_t& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t v2 = __shfl_xor(val, o), i2 = __shfl_xor(idx, o);
    if (v2 > val || (v2 == val && i2 < idx)) {
      val = v2;
      idx = i2;
    }
  }
}

__device__ __forceinline__ void set_status(int32_t* status, int32_t code) {
  if (status) atomicCAS(status, 0, code);
}

// ---------------------------------------------------------------------------
// element arithmetic (bit-exact definition)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Element bits -> binary32 (exact). bfloat16 is the upper half of a binary32.
template <bool BF>
__device__ __forceinline__ float elem_to_f32(uint16_t h) {
  if constexpr (BF)
    return __uint_as_float((uint32_t)h << 16);
  else
    return h2f(h);
}
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// (float)(int16_t)v with the sign extension folded into the conversion.
__device__ __forceinline__ float cvt_f32_sext16(int32_t v) {
  float r;
  asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_0"
      : "=v"(r)
      : "v"(v));
  return r;
}

// q = clamp(rint_even(fl32(x / step)), -32768, 32767), NaN -> 0.
// Three ways to the quotient, QM:
//   kQuotDiv   the IEEE binary32 divide;
//   kQuotTwo   v = fma(x, r_hi, x * r_lo): a two-term reciprocal, r_hi = 1/step
//              rounded down, r_lo = RN(1/step - r_hi) >= 0, so x * r_lo has
//              the sign of x (+-Inf and overflow stay saturating, NaN NaN);
//              its error is ~2^-48 relative, far inside the quotient's
//              rounding except where the divide rounds onto a tie;
//   kQuotMul   v = x * RN(1/step).
// The two cheap ones are used only for steps where k_qcheck proved that they
// give the same q as the divide for every input of the element type.
// Branch-free; sat / nan_ count saturated and NaN inputs.
constexpr int kQuotDiv = 0, kQuotTwo = 1, kQuotMul = 2;

// The constants of one step, computed once per workgroup.
struct Quot {
  float step;
  float rcp;  // RN(1/step)
  float rhi;  // 1/step rounded down
  float rlo;  // RN(1/step - rhi)
};

__device__ __forceinline__ Quot make_quot(float step) {
  Quot q;
  q.step = step;
  q.rcp = 1.0f / step;
  // rcp * step - 1 with one rounding keeps the sign of the exact value
  q.rhi = __builtin_fmaf(q.rcp, step, -1.0f) > 0.0f ? __uint_as_float(__float_as_uint(q.rcp) - 1u) : q.rcp;
  q.rlo = (float)(1.0 / (double)step - (double)q.rhi);
  return q;
}

template <int QM, bool BF>
__device__ __forceinline__ int32_t quantize(uint16_t xh, const Quot& qc, uint32_t& sat, uint32_t& nan_) {
  constexpr bool FAST = QM != kQuotDiv;
  const float x = elem_to_f32<BF>(xh);
  float v;
  // (the products written as fma with a zero addend round as the plain
  // products do, apart from the sign of a zero quotient, which q does not
  // see; for fp16 inputs the backend then folds the conversion of x into
  // mixed-precision fma instructions)
  if (QM == kQuotMul) {
    v = __builtin_fmaf(x, qc.rcp, 0.0f);  // NaN stays NaN, Inf and overflow saturate below
  } else if (QM == kQuotTwo) {
    v = __builtin_fmaf(x, qc.rhi, __builtin_fmaf(x, qc.rlo, 0.0f));
  } else {
    v = x / qc.step;
  }
  const bool is_nan = v != v;
  const float r = __builtin_rintf(v);
  sat += (r > 32767.0f) | (r < -32768.0f);
  nan_ += is_nan;
  if (FAST) {
    // the conversion instruction gives 0 for NaN and saturates +-Inf and
    // out-of-range values, so one integer clamp finishes the job (k_qcheck
    // compares this path with the exact one below on every fp16 input)
    int32_t i;
    asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(r));
    return i < -32768 ? -32768 : (i > 32767 ? 32767 : i);
  }
  const float c = __builtin_fminf(__builtin_fmaxf(r, -32768.0f), 32767.0f);
  return is_nan ? 0 : (int32_t)c;
}

// x_hat = fp16_RNE(fl32(q * step)): two roundings. The conversion is issued
// as its own instruction: the backend would fuse the multiply and the
// conversion into v_fma_mixlo_f16, which rounds once and differs on ties.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  uint32_t h;
  asm("v_cvt_f16_f32 %0, %1" : "=v"(h) : "v"(v));
  return (uint16_t)h;
}

// bfloat16: round to nearest even, one gfx950 conversion instruction.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

template <bool BF>
__device__ __forceinline__ uint16_t f32_to_elem(float v) {
  if constexpr (BF)
    return f32_to_bf16_bits(v);
  else
    return f32_to_f16_bits(v);
}

// Same, for q held modulo 2^16 in the low half of a 32-bit register.
template <bool BF>
__device__ __forceinline__ uint16_t dequantize_low16(uint32_t q, float step) {
  return f32_to_elem<BF>(cvt_f32_sext16((int32_t)q) * step);
}

// 127 + wrap16(q_t - q_{t-1}) as unsigned: below 255 it is the symbol,
// otherwise the delta needs an escape (symbol 255).
__device__ __forceinline__ uint32_t sym_raw(int32_t q_t, int32_t q_prev) {
  return (uint32_t)((int32_t)(int16_t)(uint32_t)(q_t - q_prev) + 127);
}


// mbcnt with a base: base + number of set bits of m in lanes below this one.
__device__ __forceinline__ uint32_t mbcnt_base(uint64_t m, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, base));
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Values every lane loads from the same address (headers, offsets, layer
// groups). Loads through generic pointers count as per-lane for the
// compiler's divergence analysis; moving them to scalar registers keeps the
// loops that depend on them uniform.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni(uint64_t v) {
  return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v);
}
__device__ __forceinline__ float uni(float v) { return __uint_as_float(uni(__float_as_uint(v))); }
template <typename T>
__device__ __forceinline__ T* uni(T* p) {
  return reinterpret_cast<T*>(uni((uint64_t)reinterpret_cast<uintptr_t>(p)));
}

// ---- wavefront priority from progress ---------------------------------------
// A SIMD issues from its oldest ready wavefront first. In the encoder and
// decoder a workgroup of 16 wavefronts owns the CU (its tables fill the LDS)
// and every wavefront has the same amount of work, so under age order the
// four wavefronts of a SIMD finish one after another, the last ~20 % behind
// the mean and alone on its SIMD at the end, while the workgroup's LDS stays
// held. Each wavefront therefore publishes the tokens it has left in an LDS
// slot every 32 tokens and raises its priority by the number of its SIMD's
// other wavefronts (of its workgroup) with fewer left. Wavefront w runs on
// the SIMD of w + 4, w + 8, ... (the dispatcher's order, measured); were it
// otherwise the priorities would only balance less, never change a result.
// The histogram workgroups (8 wavefronts, two per CU) do the same with their
// one SIMD-mate; they gain less, since the other workgroup fills the SIMD.
constexpr int kProgressPeriod = 32;  // tokens between two updates (a power of two)

__device__ __forceinline__ void set_priority(int p) {
  if (p <= 0) __builtin_amdgcn_s_setprio(0);
  else if (p == 1) __builtin_amdgcn_s_setprio(1);
  else if (p == 2) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(3);
}

// left[WAVES]: tokens each wavefront of the workgroup has left (LDS). Entries
// are read without synchronisation; a stale value only delays the balance.
template <int WAVES>
__device__ __forceinline__ void publish_progress(int* left, int wave, int mine, int lane) {
  static_assert(WAVES == 8 || WAVES == 16, "two or four wavefronts per SIMD");
  if (lane == 0) left[wave] = mine;
  int ahead = uni(left[wave ^ 4]) < mine;
  if (WAVES == 16) ahead += (uni(left[wave ^ 8]) < mine) + (uni(left[wave ^ 12]) < mine);
  set_priority(ahead);
}

// Raw buffer resource over [base, base + bytes): accesses use a per-lane
// offset in a VGPR plus a wave-uniform offset in an SGPR, so address
// arithmetic stays on the scalar unit. The hardware range check covers the
// VGPR offset (loads past `bytes` return 0, stores are dropped); offsets that
// may run past the end therefore go in the VGPR, and the SGPR offset is used
// only where the access is in bounds by construction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

struct BlobHdr {
  uint32_t magic, version, L, H, D, G, level_id, C;
  uint64_t T;
  uint32_t f_offset, dtype;
  uint64_t format_bytes;
  uint32_t flags, z1;
};

__device__ __forceinline__ const BlobHdr* blob_hdr(const uint8_t* b) {
  return reinterpret_cast<const BlobHdr*>(b);
}
__device__ __forceinline__ float blob_step(const uint8_t* b, int g) {
  return uni(reinterpret_cast<const float*>(b + 64)[g]);
}
__device__ __forceinline__ const uint8_t* blob_lg(const uint8_t* b, int G) { return b + 64 + 4 * G; }
__device__ __forceinline__ int layer_group(const uint8_t* b, int G, int l) {
  return uni((uint32_t)blob_lg(b, G)[l]);
}
__device__ __forceinline__ bool blob_ok(const uint8_t* b, const Shape& s, int G) {
  const BlobHdr* bh = reinterpret_cast<const BlobHdr*>(b);
  return uni(bh->magic) == kTableMagic && uni(bh->version) == kVersion && (int)uni(bh->L) == s.L &&
         (int)uni(bh->H) == s.H && (int)uni(bh->D) == s.D && (int)uni(bh->G) == G &&
         (int)uni(bh->dtype) == s.dt && (uni(bh->flags) & ~kTablesRobust) == 0;
}
// Quotient mode of layer group g: bit 0 of the flag = kQuotTwo proven exact,
// bit 1 = kQuotMul proven exact (k_qcheck clears what fails).
__device__ __forceinline__ int qmode(const uint8_t* b, int L, int H, int D, int G, int g) {
  const uint32_t f = uni(reinterpret_cast<const uint32_t*>(b + tb_qflag_offset(L, H, D, G))[g]);
  return (f & 2u) ? kQuotMul : (f & 1u) ? kQuotTwo : kQuotDiv;
}

// ---------------------------------------------------------------------------
// fill / copy / refs
// ---------------------------------------------------------------------------
__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t value, uint64_t n) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

__global__ void k_copy(uint4* __restrict__ dst, const uint4* __restrict__ src, uint64_t n) {
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void k_make_refs(const uint8_t* base, const uint64_t* __restrict__ offs, int32_t n,
                            int32_t table, cg_chunk_ref* __restrict__ refs) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    cg_chunk_ref r;
    r.record = base + offs[i];
    r.bytes = offs[i + 1] - offs[i];
    r.table = table;
    r.reserved = 0;
    refs[i] = r;
  }
}

__global__ void k_set_ref(cg_chunk_ref* ref, const uint8_t* record, uint64_t bytes, int32_t table) {
  if (threadIdx.x == 0) {
    cg_chunk_ref r;
    r.record = record;
    r.bytes = bytes;
    r.table = table;
    r.reserved = 0;
    *ref = r;
  }
}

// ---------------------------------------------------------------------------
// tables blob: header, steps, layer groups, quotient flags
// ---------------------------------------------------------------------------
__global__ void k_blob_init(BlobInitArgs a) {
  const uint64_t foff = tb_f_offset(a.L, a.G);
  const uint64_t fbytes = tb_format_bytes(a.L, a.H, a.D, a.G);
  const uint64_t acc = tb_acc_offset(a.L, a.H, a.D, a.G);
  uint8_t* b = a.blob;
  for (uint64_t i = threadIdx.x; i < foff; i += blockDim.x) {
    uint8_t v = 0;
    if (i >= 64 && i < 64 + 4 * (uint64_t)a.G) {
      uint32_t bits = __float_as_uint(a.step[(i - 64) / 4]);
      v = (uint8_t)(bits >> (8 * ((i - 64) % 4)));
    } else if (i >= 64 + 4 * (uint64_t)a.G && i < 64 + 4 * (uint64_t)a.G + a.L) {
      v = a.lg[i - 64 - 4 * a.G];
    }
    b[i] = v;
  }
  for (uint64_t i = fbytes + threadIdx.x; i < acc; i += blockDim.x) b[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* h = reinterpret_cast<uint32_t*>(b);
    h[0] = kTableMagic;
    h[1] = kVersion;
    h[2] = (uint32_t)a.L;
    h[3] = (uint32_t)a.H;
    h[4] = (uint32_t)a.D;
    h[5] = (uint32_t)a.G;
    h[6] = (uint32_t)a.level_id;
    h[7] = (uint32_t)a.C;
    *reinterpret_cast<uint64_t*>(b + 32) = (uint64_t)a.T;
    h[10] = (uint32_t)foff;
    h[11] = (uint32_t)a.dtype;
    *reinterpret_cast<uint64_t*>(b + 48) = fbytes;
    h[14] = a.flags;
    h[15] = 0;
  }
  uint32_t* qf = reinterpret_cast<uint32_t*>(b + tb_qflag_offset(a.L, a.H, a.D, a.G));
  for (int g = threadIdx.x; g < 256; g += blockDim.x) qf[g] = g < a.G ? 3u : 0u;
}

template <bool BF>
__global__ void k_qcheck(QCheckArgs a) {
  const int g = blockIdx.y;
  const uint32_t xh = blockIdx.x * blockDim.x + threadIdx.x;  // 0 .. 65535
  const Quot qc = make_quot(blob_step(a.blob, g));
  uint32_t s0 = 0, n0 = 0;
  const int32_t qi = quantize<kQuotDiv, BF>((uint16_t)xh, qc, s0, n0);
  const int32_t qf = quantize<kQuotTwo, BF>((uint16_t)xh, qc, s0, n0);
  const int32_t qm = quantize<kQuotMul, BF>((uint16_t)xh, qc, s0, n0);
  if (qf != qi) atomicAnd(&a.qflags[g], ~1u);
  if (qm != qi) atomicAnd(&a.qflags[g], ~2u);
}

// ---------------------------------------------------------------------------
// histogram: one workgroup per (layer, K|V, head, slice); 8 wavefronts split
// the tokens (a wavefront starting inside a chunk re-quantizes the token
// before its range). Counts are privatised in LDS lane-minor, hist[sym][lane],
// so the 64 lanes of an increment hit 64 different banks; row 256 takes the
// first token of each chunk (no symbol). Counts land in HBM in the same
// lane-minor order per table set, so the flush is coalesced.
// ---------------------------------------------------------------------------
constexpr int kHistThreads = 512;
constexpr int kHistWaves = kHistThreads / 64;
constexpr int kHistBatch = 16;

// Tokens [t_begin, t_end) of one (layer, K|V, head, slice) column; xr
// covers the column from token 0 (row t at byte t * row_bytes). Every load
// is in bounds by construction. STATS adds the saturated / NaN counts.
template <int QM, bool STATS, bool BF>
__device__ __forceinline__ void hist_range(__amdgpu_buffer_rsrc_t xr, uint32_t row_bytes, int t_begin,
                                           int t_end, int C, const Quot qc, uint32_t* hist,
                                           int* left, int wave, int lane, uint32_t& sat,
                                           uint32_t& nan_) {
  const uint32_t lane2 = 2u * lane, lane4 = 4u * lane;
  uint32_t* hl = hist + lane;
  int32_t prev = 0;
  int pos = t_begin % C;  // position of the next token inside its chunk
  if (pos != 0) {
    uint32_t d0 = 0, d1 = 0;
    prev = quantize<QM, BF>(
        (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(xr, lane2, (uint32_t)(t_begin - 1) * row_bytes, 0),
        qc, d0, d1);
  }
  auto one = [&](uint16_t xh) {
    uint32_t s0 = 0, n0 = 0;
    const int32_t q = quantize<QM, BF>(xh, qc, s0, n0);
    if (STATS) {
      sat += s0;
      nan_ += n0;
    }
    const uint32_t r = sym_raw(q, prev);
    // byte offset of row min(r, 255), column lane, in one shift-or (the
    // compiler splits it in two)
    uint32_t off;
    asm("v_lshl_or_b32 %0, %1, 8, %2" : "=v"(off) : "v"(r < 255u ? r : 255u), "v"(lane4));
    uint32_t* cell = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(hist) + off);
    atomicAdd(cell, 1u);
    if (__builtin_expect(pos == 0, 0)) {  // a chunk head has no symbol: row 256 counts it instead
      atomicSub(cell, 1u);
      atomicAdd(hl + 256 * 64, 1u);
    }
    prev = q;
    pos = (pos + 1 == C) ? 0 : pos + 1;
  };
  // the rows of the next batch are loaded while the current one is counted
  // (rows past t_end clamp to the last one)
  // (32-bit slots: two 16-bit values packed in one register would make the
  // packing wait for both loads at once)
  auto load_batch = [&](uint32_t* v, int t0) {
    if (t0 + kHistBatch <= t_end) {
      const uint32_t o0 = (uint32_t)t0 * row_bytes;
#pragma unroll
      for (int k = 0; k < kHistBatch; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(xr, lane2, o0 + (uint32_t)k * row_bytes, 0);
    } else {
#pragma unroll
      for (int k = 0; k < kHistBatch; ++k) {
        const int tk = t0 + k < t_end ? t0 + k : t_end - 1;
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(xr, lane2, uni((uint32_t)tk * row_bytes), 0);
      }
    }
  };
  int t = t_begin;
  uint32_t xv[kHistBatch];
  load_batch(xv, t);
  // the first batch lands before the loop: otherwise its pending loads merge
  // into the loop's wait counts and every token waits on the next batch
  __builtin_amdgcn_s_waitcnt(0x0F70);
  static_assert(2 * kHistBatch == kProgressPeriod, "progress every second batch");
  for (; t + kHistBatch <= t_end; t += kHistBatch) {
    if (((t - t_begin) & kHistBatch) == 0) publish_progress<kHistWaves>(left, wave, t_end - t, lane);
    uint32_t xn[kHistBatch];
    load_batch(xn, t + kHistBatch);
#pragma unroll
    for (int k = 0; k < kHistBatch; ++k) one((uint16_t)xv[k]);
#pragma unroll
    for (int k = 0; k < kHistBatch; ++k) xv[k] = xn[k];
  }
#pragma unroll
  for (int k = 0; k < kHistBatch; ++k)
    if (t + k < t_end) one((uint16_t)xv[k]);
}

template <bool BF>
__global__ void __launch_bounds__(kHistThreads) k_hist(HistArgs a) {
  __shared__ uint32_t hist[257 * 64];
  __shared__ int left[kHistWaves];  // tokens each wavefront has left (priorities)
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  for (int i = tid; i < 257 * 64; i += kHistThreads) hist[i] = 0;
  if (tid < kHistWaves) left[tid] = 0x7FFFFFFF;

  const Shape s = a.s;
  int64_t bid = blockIdx.x;
  const int j = (int)(bid % s.S);
  bid /= s.S;
  const int h = (int)(bid % s.H);
  bid /= s.H;
  const int kv = (int)(bid % 2);
  const int l = (int)(bid / 2);
  const int G = a.G;
  const int g = layer_group(a.blob, G, l);
  const Quot qc = make_quot(blob_step(a.blob, g));
  const int qm = qmode(a.blob, s.L, s.H, s.D, G, g);
  __syncthreads();

  const uint16_t* xb = a.x + (((size_t)l * 2 + kv) * s.H + h) * (size_t)s.T * s.D + 64 * j;
  const uint32_t row_bytes = 2u * (uint32_t)s.D;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(xb, (uint32_t)(s.T * row_bytes));
  const int t_begin = (int)(s.T * wave / kHistWaves), t_end = (int)(s.T * (wave + 1) / kHistWaves);
  uint32_t sat = 0, nan_ = 0;
  if (t_begin < t_end) {
#define CG_HIST(QM, ST) \
  hist_range<QM, ST, BF>(xr, row_bytes, t_begin, t_end, s.C, qc, hist, left, wave, lane, sat, nan_)
    if (a.stats) {
      if (qm == kQuotMul) CG_HIST(kQuotMul, true);
      else if (qm == kQuotTwo) CG_HIST(kQuotTwo, true);
      else CG_HIST(kQuotDiv, true);
    } else {
      if (qm == kQuotMul) CG_HIST(kQuotMul, false);
      else if (qm == kQuotTwo) CG_HIST(kQuotTwo, false);
      else CG_HIST(kQuotDiv, false);
    }
#undef CG_HIST
  }
  __syncthreads();
  const size_t set = (((size_t)g * 2 + kv) * s.H + h) * s.S + j;
  uint32_t* counts = a.counts + set * (256 * 64);
  for (int i = tid; i < 256 * 64; i += kHistThreads) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&counts[i], c);
  }
  if (a.stats) {
    // escapes are the histogram's row 255, counted once per workgroup
    const uint32_t st = wave_sum(sat), nn = wave_sum(nan_);
    const uint32_t es = wave == 0 ? wave_sum(hist[255 * 64 + lane]) : 0u;
    if (lane == 0) {
      if (wave == 0) atomicAdd(&a.stats[0], (unsigned long long)(64 * s.T));
      if (st) atomicAdd(&a.stats[1], (unsigned long long)st);
      if (nn) atomicAdd(&a.stats[2], (unsigned long long)nn);
      if (es) atomicAdd(&a.stats[3], (unsigned long long)es);
    }
  }
}

// ---------------------------------------------------------------------------
// normalisation: one wavefront per table; lane k owns symbols 4k .. 4k+3.
// Same rule as the format defines: f = max(1, floor(c*4096/n)) for observed
// symbols, deficit to the most frequent symbol, surplus cut from the largest
// frequency, ties to the lowest symbol.
// ---------------------------------------------------------------------------
constexpr int kNormThreads = 256;

__global__ void __launch_bounds__(kNormThreads) k_norm(NormArgs a) {
  __shared__ uint32_t bm_lds[kNormThreads / 64][128];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * (kNormThreads / 64) + wave;
  const bool active = t < a.n_tables;
  for (int i = lane; i < 128; i += 64) bm_lds[wave][i] = 0;
  uint32_t c[4] = {0, 0, 0, 0}, f[4] = {0, 0, 0, 0}, b[4] = {0, 0, 0, 0};
  uint32_t rank0 = 0, K = 0;
  // table t is channel kk of set t / 64 (sets are lane-minor, 64 channels)
  const int64_t set = t >> 6;
  const int kk = (int)(t & 63);
  if (active) {
    const uint32_t* cs = a.counts + set * (256 * 64) + kk;
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = cs[(4 * lane + k) * 64];
    const uint64_t n = wave_sum((uint64_t)c[0] + c[1] + c[2] + c[3]);
    if (n == 0) {
      if (lane == 127 / 4) f[127 % 4] = kM;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (c[k]) {
          const uint64_t v = (uint64_t)c[k] * kM / n;
          f[k] = v < 1 ? 1u : (uint32_t)v;
        }
      }
      uint32_t S = wave_sum(f[0] + f[1] + f[2] + f[3]);
      if (S < kM) {
        uint32_t bv = c[0], bi = 4 * lane;
#pragma unroll
        for (int k = 1; k < 4; ++k)
          if (c[k] > bv) {
            bv = c[k];
            bi = 4 * lane + k;
          }
        wave_argmax(bv, bi);
        if ((int)(bi >> 2) == lane) f[bi & 3] += kM - S;
        S = kM;
      }
      while (S > kM) {
        uint32_t bv = f[0], bi = 4 * lane;
#pragma unroll
        for (int k = 1; k < 4; ++k)
          if (f[k] > bv) {
            bv = f[k];
            bi = 4 * lane + k;
          }
        wave_argmax(bv, bi);
        uint32_t cut = bv - 1u;
        if (cut > S - kM) cut = S - kM;
        if ((int)(bi >> 2) == lane) f[bi & 3] -= cut;
        S -= cut;
      }
    }
    // robust tables: the escape (symbol 255, lane 63, k = 3) gets at least
    // one unit, taken from the largest frequency (lowest symbol on ties)
    if (a.robust && __shfl(f[3], 63) == 0) {
      uint32_t bv = f[0], bi = 4 * lane;
#pragma unroll
      for (int k = 1; k < 4; ++k)
        if (f[k] > bv) {
          bv = f[k];
          bi = 4 * lane + k;
        }
      wave_argmax(bv, bi);
      if ((int)(bi >> 2) == lane) f[bi & 3] -= 1u;
      if (lane == 63) f[3] = 1u;
    }
    // cumulative frequencies and ranks of the present symbols
    const uint32_t fsum = f[0] + f[1] + f[2] + f[3];
    const uint32_t fex = wave_excl_scan(fsum, lane);
    b[0] = fex;
    b[1] = fex + f[0];
    b[2] = b[1] + f[1];
    b[3] = b[2] + f[2];
    const uint32_t pc = (f[0] > 0) + (f[1] > 0) + (f[2] > 0) + (f[3] > 0);
    rank0 = wave_excl_scan(pc, lane);
    K = __shfl(rank0 + pc, 63);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (f[k]) atomicOr(&bm_lds[wave][b[k] >> 5], 1u << (b[k] & 31));
  }
  __syncthreads();
  if (!active) return;
  // format section: u16 f
  uint16_t* fsec = reinterpret_cast<uint16_t*>(a.blob + a.f_off) + t * 256;
  uint2 fv;
  fv.x = f[0] | (f[1] << 16);
  fv.y = f[2] | (f[3] << 16);
  reinterpret_cast<uint2*>(fsec)[lane] = fv;
  // encoder set: (16 f - 1) mod 2^16 | b << 16 per symbol. The low half
  // gives the encoder both its renormalisation test (x >> 16 above it) and
  // the address of f's reciprocal (8 f, from half of it); the high half is
  // the symbol's start. The escape symbol (255) comes last in cumulative
  // order, so every other coded symbol's entry is below the escape's: the
  // encoder escapes a lane whose entry is at or above it. With robust
  // tables a symbol of frequency 0 gets the escape's entry, so the encoder
  // escapes it; without, it gets kEncInvalid, which is at or above any
  // escape entry, as is the escape of plain tables that saw none; the
  // encoder's escape branch reports kEncInvalid as CG_ERR_TABLE. Rows are
  // indexed by delta + 128 (symbol + 1); the escape's entry fills rows 0
  // and 256, which the clamped deltas beyond +-127 reach.
  uint32_t* enc = reinterpret_cast<uint32_t*>(a.blob + a.enc_off) + set * (kEncDwords * 64) + kk;
  const uint32_t f_esc = __shfl(f[3], 63), b_esc = __shfl(b[3], 63);
  const uint32_t esc_entry = f_esc == 0 ? kEncInvalid : (((16u * f_esc - 1u) & 0xFFFFu) | (b_esc << 16));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int sym = 4 * lane + k;
    uint32_t e = ((16u * f[k] - 1u) & 0xFFFFu) | (b[k] << 16);
    if (sym == 255) e = esc_entry;
    else if (f[k] == 0) e = a.robust ? esc_entry : kEncInvalid;
    if (sym < 255) {
      enc[(sym + 1) * 64] = e;
    } else {
      enc[0] = e;
      enc[256 * 64] = e;
    }
  }
  // decoder set: reversed start bitmap, scaled rank bases, rank -> (d, 4096-f, b)
  uint32_t* dec = reinterpret_cast<uint32_t*>(a.blob + a.dec_off) + set * (kDecDwords * 64) + kk;
  const uint32_t w0 = bm_lds[wave][2 * lane], w1 = bm_lds[wave][2 * lane + 1];
  const uint32_t p0 = __popc(w0), p1 = __popc(w1);
  const uint32_t pex = wave_excl_scan(p0 + p1, lane);  // starts below word 2*lane
  const uint32_t info_col = 4u * kDecInfo + 4u * (uint32_t)kk;
  dec[kDecBm + (2 * lane) * 64] = __builtin_bitreverse32(w0) << 1;
  dec[kDecBm + (2 * lane + 1) * 64] = __builtin_bitreverse32(w1) << 1;
  dec[kDecRb + (2 * lane) * 64] = ((pex + p0 - 1u) << 8) + info_col;
  dec[kDecRb + (2 * lane + 1) * 64] = ((pex + p0 + p1 - 1u) << 8) + info_col;
  uint32_t r = rank0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (f[k]) {
      const uint32_t dbyte = (uint32_t)(4 * lane + k - 127) & 255u;
      dec[kDecInfo + r * 64] = dbyte | ((kM - f[k]) << 8) | (b[k] << 20);
      r += 1;
    }
    if ((uint32_t)(4 * lane + k) >= K) dec[kDecInfo + (4 * lane + k) * 64] = 0;
  }
}

// ---------------------------------------------------------------------------
// encode: one workgroup per (chunk, layer group, K|V, head, slice); its 16
// wavefronts take the layers of the group. The set's encoder table (lane-
// minor, 64.25 KB) and per f = 0..4096 RU(1/f) with 4096 - f packed in (32 KB)
// sit in LDS.
// Exact quotient: floor(x/f) = trunc(fl64(x) * RU(1/f)) for x < 2^32, f <= 2^12
// (the product stays below q+1 by more than the fp64 spacing there).
// The group is coded backward (token n-1 first) and its words are written
// backward into a worst-case scratch slot: per token first the escape
// payloads, then the renormalisation words, so that the decoder, reading
// forward, meets renorm words before escape payloads.
// ---------------------------------------------------------------------------
constexpr int kEncThreads = kWaves * 64;
constexpr int kEncBatch = 16;

// The encoder's scratch slot is a structured buffer of 2-byte records (one
// word each, cap of them), so a store names its word by index and the
// address unit does the doubling: word soff/2 + idx. Stores only, in inline
// assembly (the compiler has no structured 16-bit store); no memory clobber:
// nothing in the kernel reads the scratch it writes, and a clobber would keep
// the next token's table read from moving above the store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_slot_rsrc(const uint16_t* base, uint32_t words) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)2, (int)words, 0x00020000);
}

// word idx (per lane) after the first soff / 2 words of the slot <- v
__device__ __forceinline__ void slot_store(uint32_t v, uint32_t idx, __amdgpu_buffer_rsrc_t sw, uint32_t soff) {
  asm volatile(
      "s_nop 4\n\t"  // VALU-written SGPR operands of the store: see stream_load_async
      "buffer_store_short %0, %1, %2, %3 idxen"
      :
      : "v"(v), "v"(idx), "s"(sw), "s"(uni(soff)));
}

// On the lanes of m: store the low 16 bits of x as word idx after soff / 2,
// then x >>= 16. One masked region with a single VALU shift; the compiler's
// version computes the shift into a temporary and copies it back. No wait
// states before the store: its scalar operands (the slot descriptor, the
// word offset) come from scalar instructions, and tests/asm_hazards.py checks
// in the compiled code that no VALU write of them falls within the five wait
// states a vector-memory read of a VALU-written SGPR needs.
__device__ __forceinline__ void renorm_out(uint32_t& x, uint64_t m, __amdgpu_buffer_rsrc_t sw,
                                           uint32_t idx, uint32_t soff) {
  uint64_t saved;
  asm volatile(
      "s_and_saveexec_b64 %1, %2\n\t"
      "buffer_store_short %0, %3, %4, %5 idxen\n\t"
      "v_lshrrev_b32 %0, 16, %0\n\t"
      "s_mov_b64 exec, %1"
      : "+v"(x), "=&s"(saved)
      : "s"(m), "v"(idx), "s"(sw), "s"(soff)
      : "scc");
}

// A token t >= 1 of a group passes three stages, each started one token
// after the previous one so that its LDS read lands behind a token of other
// work instead of being waited for at once:
//   S1: quantize x_{t-1}, symbol of q_t - q_{t-1}, read the symbol's entry
//   S2: escape test on the entry, read f's reciprocal
//   S3: escape payload, renormalisation word, state update
struct EncTok {
  uint32_t e;    // symbol entry (16 f - 1) mod 2^16 | b << 16 (S1 read)
  uint32_t d16;  // low 16 bits: the wrapped delta, the escape payload
  bool esc;      // this lane codes an escape (wide delta, or robust tables)
  uint64_t me;   // lanes of the wavefront that need one
  double r;      // RU(1/f), 4096 - f in its low 16 bits (S2 read)
};

// The encoder's constant for frequency f, one 8-byte LDS entry at 8 f:
// RU(1/f), rounded up further to 36 significant bits, with 4096 - f in the
// 16 low bits this frees. The stored value exceeds 1/f by a relative 2^-35
// at most, below the 2^-32 / f that keeps trunc(x * r) = floor(x / f) for
// every state x < f * 2^20 (the one below that the renormalisation leaves);
// f = 4096 stays exact (2^-12). f = 0 holds 4096 in a zero value.
__device__ __forceinline__ double enc_rcp(uint32_t f) {
  if (f == 0) return __longlong_as_double(4096);
  double r = 1.0 / (double)f;
  if (__builtin_fma(r, (double)f, -1.0) < 0.0) r = __longlong_as_double(__double_as_longlong(r) + 1);
  const uint64_t u = ((uint64_t)__double_as_longlong(r) + 0xFFFFu) & ~(uint64_t)0xFFFF;
  return __longlong_as_double((long long)(u | (kM - f)));
}

// q_t - q_{t-1} wrapped to 16 bits and sign-extended, in one instruction
// (the SDWA form sign-extends its 16-bit result)
__device__ __forceinline__ int32_t sub_wrap16(int32_t a, int32_t b) {
  int32_t r;
  asm("v_sub_u32_sdwa %0, %1, %2 dst_sel:WORD_0 dst_unused:UNUSED_SEXT src0_sel:DWORD src1_sel:DWORD"
      : "=v"(r)
      : "v"(a), "v"(b));
  return r;
}

// a + (b >> 16) in one instruction (the SDWA form reads b's high half)
__device__ __forceinline__ uint32_t add_hi16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
      : "=v"(r)
      : "v"(a), "v"(b));
  return r;
}

// row0: the lane's column of the encoder table at row 128 (delta 0); the
// entry of delta d is row0[64 * clamp(d, -128, 128)]
template <int QM, bool BF>
__device__ __forceinline__ void enc_s1(EncTok& k, uint16_t xprev, int32_t& qhi, const Quot& qc,
                                       const uint32_t* row0) {
  uint32_t d0 = 0, d1 = 0;
  const int32_t qlo = quantize<QM, BF>(xprev, qc, d0, d1);
  const int32_t d = sub_wrap16(qhi, qlo);
  k.d16 = (uint32_t)d;
  const int32_t m = d < -128 ? -128 : (d > 128 ? 128 : d);
  k.e = row0[m * 64];
  qhi = qlo;
}

// The escape decision compares the entry with the lane's escape entry
// (symbol 255, a wide delta and, with robust tables, every symbol of
// frequency 0; kEncInvalid too). The reciprocal sits at byte 8 f, one past
// half the entry's low half (16 f - 1); kEncInvalid's reaches f = 4096.
__device__ __forceinline__ void enc_s2(EncTok& k, const uint8_t* rcp, uint32_t e_esc) {
  k.esc = k.e >= e_esc;
  k.me = __ballot(k.esc);
  k.r = *reinterpret_cast<const double*>(rcp + ((k.e & 0xFFFFu) >> 1) + 1);
}

// A symbol that plain tables cannot code (frequency 0, or an escape of
// frequency 0) holds kEncInvalid, which counts as an escape, so the escape
// branch is the only place it shows; the call then reports CG_ERR_TABLE.
// (reported from inside the branch: a flag carried to the end of the group
// would be updated by a select on every token)
__device__ __forceinline__ void enc_s3(const EncTok& k, uint32_t& x, uint32_t& P, __amdgpu_buffer_rsrc_t sr,
                                       int32_t* status, int lane) {
  if (k.me) {
    P -= (uint32_t)__popcll(k.me);
    if (k.esc) slot_store(k.d16, mbcnt_base(k.me, 0), sr, 2u * P);
    if (__builtin_expect(__ballot(k.esc && k.e == kEncInvalid) != 0, 0) && lane == 0)
      set_status(status, CG_ERR_TABLE);
  }
  // renormalise when x >= f * 2^20, i.e. x >> 16 >= 16 f (never for
  // f = 4096, whose entry's low half is 65535)
  const uint64_t mr = __ballot((x >> 16) > (k.e & 0xFFFFu));
  P -= (uint32_t)__popcll(mr);
  renorm_out(x, mr, sr, mbcnt_base(mr, 0), 2u * P);
  // x <- floor(x/f)*4096 + x mod f + b = x + floor(x/f)*(4096-f) + b; the
  // quotient is < 2^20 and 4096 - f <= 2^12, so a 24-bit multiply is exact.
  const uint32_t qd = (uint32_t)((double)x * k.r);
  const uint32_t g = (uint32_t)__double_as_longlong(k.r) & 0xFFFFu;
  x = add_hi16(__umul24(qd, g) + x, k.e);
}

// Encodes tokens n-1 .. 1 of a group (backward), then the head. xr covers the
// group's column of x (row t at byte t * row_bytes), sr its scratch slot of
// cap words; every access is in bounds by construction.
template <int QM, bool BF>
__device__ __forceinline__ void encode_group(__amdgpu_buffer_rsrc_t xr, int n, uint32_t row_bytes,
                                             const Quot qc, const uint32_t* ftab,
                                             const uint8_t* rcp, __amdgpu_buffer_rsrc_t sr,
                                             uint32_t cap, int lane, uint32_t& words,
                                             uint32_t& start, int32_t* status, int* left, int wave,
                                             int left_after) {
  const uint32_t lane2 = 2u * lane;
  const uint32_t* row0 = ftab + 128 * 64 + lane;
  const uint32_t e_esc = ftab[lane];  // row 0: the escape's entry
  uint32_t P = cap;
  uint32_t x = kL;
  auto row = [&](int r) { return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(xr, lane2, (uint32_t)r * row_bytes, 0); };
  uint32_t d0 = 0, d1 = 0;
  int32_t qhi = quantize<QM, BF>(row(n - 1), qc, d0, d1);
  if (n >= 3) {
    // a: token in S3, b: in S2, c: in S1. Prologue: token n-1 through S1 and
    // S2, token n-2 through S1.
    EncTok a, b, c;
    enc_s1<QM, BF>(a, row(n - 2), qhi, qc, row0);
    enc_s2(a, rcp, e_esc);
    enc_s1<QM, BF>(b, row(n - 3), qhi, qc, row0);
    // tokens i, i-1, ... enter S1 with x of rows i-1, i-2, ...; the rows of
    // the next batch are loaded while the current one is encoded. Offsets
    // stay scalar: a batch of 16 rows all >= 0 needs no clamp; the last one
    // clamps at 0. (32-bit slots, as in hist_range)
    // rows i0 - 1, ..., i0 - 16 (i0 >= 16: all of them exist)
    auto load_rows = [&](uint32_t* v, int i0) {
      const uint32_t o0 = (uint32_t)(i0 - 1) * row_bytes;
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k)
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(xr, lane2, o0 - (uint32_t)k * row_bytes, 0);
    };
    // the same rows, those below 0 replaced by row 0 (any i0)
    auto load_rows_clamped = [&](uint32_t* v, int i0) {
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k) {
        const int r = i0 - 1 - k > 0 ? i0 - 1 - k : 0;
        v[k] = __builtin_amdgcn_raw_buffer_load_b16(xr, lane2, uni((uint32_t)r * row_bytes), 0);
      }
    };
    int i = n - 3;  // next token to enter S1
    // Three batches of rows in flight: the batch a step encodes was loaded
    // two steps earlier. The renormalisation stores are inline assembly the
    // compiler does not count, so the vmcnt wait it places before a row's
    // first use also covers every operation issued after that row's load
    // beyond the loads it knows of; with the batch loaded one step ahead that
    // wait reached the loads just issued (or, before them, the stores just
    // issued) and exposed a memory round trip every 16 tokens.
    uint32_t xa[kEncBatch], xb[kEncBatch], xc[kEncBatch];
    load_rows_clamped(xa, i);
    load_rows_clamped(xb, i - kEncBatch);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // as in hist_range
    auto advance = [&](uint16_t xprev) {
      enc_s1<QM, BF>(c, xprev, qhi, qc, row0);
      enc_s2(b, rcp, e_esc);
      enc_s3(a, x, P, sr, status, lane);
      a = b;
      b = c;
    };
    static_assert(2 * kEncBatch == kProgressPeriod, "progress every second batch");
    // one step: encode the batch of tokens at, ..., at - 15 and load the
    // batch two ahead; three steps per iteration, rotating the registers.
    // The loop runs while every row it loads exists (at - 32 >= 16), so its
    // loads need no clamp: a clamped variant on one of two paths put a
    // register copy, and a full vmcnt wait, on both.
    auto step16 = [&](uint32_t* cur, uint32_t* ahead, int at) {
      if (at & kEncBatch) publish_progress<kWaves>(left, wave, left_after + at, lane);
      load_rows(ahead, at - 2 * kEncBatch);
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k) advance((uint16_t)cur[k]);
    };
    for (; i >= 5 * kEncBatch; i -= 3 * kEncBatch) {
      step16(xa, xc, i);
      step16(xb, xa, i - kEncBatch);
      step16(xc, xb, i - 2 * kEncBatch);
    }
    // the last batches (at most four), rows moved once per batch
    for (; i >= kEncBatch; i -= kEncBatch) {
      if (i & kEncBatch) publish_progress<kWaves>(left, wave, left_after + i, lane);
      load_rows_clamped(xc, i - 2 * kEncBatch);
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k) advance((uint16_t)xa[k]);
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k) {
        xa[k] = xb[k];
        xb[k] = xc[k];
      }
    }
#pragma unroll
    for (int k = 0; k < kEncBatch; ++k)  // the last i < 16 tokens
      if (k < i) advance((uint16_t)xa[k]);
    // epilogue: the last two tokens leave the pipeline
    enc_s2(b, rcp, e_esc);
    enc_s3(a, x, P, sr, status, lane);
    enc_s3(b, x, P, sr, status, lane);
  } else if (n == 2) {
    EncTok a;
    enc_s1<QM, BF>(a, row(0), qhi, qc, row0);
    enc_s2(a, rcp, e_esc);
    enc_s3(a, x, P, sr, status, lane);
  }
  P -= 64;
  slot_store((uint32_t)qhi, lane, sr, 2u * P);
  P -= 64;
  slot_store(x, lane, sr, 2u * P);
  P -= 64;
  slot_store(x >> 16, lane, sr, 2u * P);
  words = cap - P;
  start = P;
}

// The k-th layer (0-based, ascending) of layer group g, or -1; computed by
// one wavefront with ballots over the blob's layer -> group map.
__device__ __forceinline__ int layer_of_group(const uint8_t* blob, int G, int L, int g, int k, int lane) {
  int base = 0;
  for (int l0 = 0; l0 < L; l0 += 64) {
    const int l = l0 + lane;
    const bool in = l < L && blob_lg(blob, G)[l < L ? l : 0] == g;
    const uint64_t m = __ballot(in);
    const int cnt = __popcll(m);
    if (k < base + cnt) {
      const uint64_t hit = __ballot(in && (int)mbcnt_base(m, 0) == k - base);
      return l0 + __builtin_ctzll(hit);
    }
    base += cnt;
  }
  return -1;
}

__device__ __forceinline__ int layers_in_group(const uint8_t* blob, int G, int L, int g, int lane) {
  int n = 0;
  for (int l0 = 0; l0 < L; l0 += 64) {
    const int l = l0 + lane;
    n += __popcll(__ballot(l < L && blob_lg(blob, G)[l < L ? l : 0] == g));
  }
  return n;
}

// LDS of the encoder, laid out by hand so both tables sit at small fixed
// offsets: the per-frequency constants first (address f * 8), then the
// symbol table.
constexpr int kEncRcpBytes = 8 * (kM + 1);
constexpr int kEncFtabOff = (kEncRcpBytes + 255) / 256 * 256;

template <bool BF>
__global__ void __launch_bounds__(kEncThreads) k_encode(EncodeArgs a) {
  __shared__ __align__(16) uint8_t enc_lds[kEncFtabOff + 4 * kEncDwords * 64];
  __shared__ int left[kWaves];
  double* rcp_tab = reinterpret_cast<double*>(enc_lds);
  uint32_t* ftab = reinterpret_cast<uint32_t*>(enc_lds + kEncFtabOff);
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const Shape s = a.s;
  int64_t bid = blockIdx.x;
  const int j = (int)(bid % s.S);
  bid /= s.S;
  const int h = (int)(bid % s.H);
  bid /= s.H;
  const int kv = (int)(bid % 2);
  bid /= 2;
  const int g = (int)(bid % a.G);
  const int64_t rb = bid / a.G;  // block of chunks within the call
  const int64_t nb1 = a.split / a.chunks_per_block;
  int64_t cl_begin, cl_end;
  if (rb < nb1) {
    cl_begin = rb * a.chunks_per_block;
    cl_end = cl_begin + a.chunks_per_block;
  } else {
    cl_begin = a.split + (rb - nb1) * a.chunks_per_block2;
    cl_end = cl_begin + a.chunks_per_block2 < a.n_chunks ? cl_begin + a.chunks_per_block2 : a.n_chunks;
  }
  const int G = a.G;
  if (!blob_ok(a.blob, s, G)) {
    if (tid == 0) set_status(a.status, CG_ERR_INVALID_ARG);
    return;
  }
  const size_t set = (((size_t)g * 2 + kv) * s.H + h) * s.S + j;
  const uint4* esrc = reinterpret_cast<const uint4*>(
      reinterpret_cast<const uint32_t*>(a.blob + tb_enc_offset(s.L, s.H, s.D, G)) + set * (kEncDwords * 64));
  for (int u = tid; u < kEncDwords * 64 / 4; u += kEncThreads) reinterpret_cast<uint4*>(ftab)[u] = esrc[u];
  for (int f = tid; f <= (int)kM; f += kEncThreads) rcp_tab[f] = enc_rcp((uint32_t)f);
  if (tid < kWaves) left[tid] = 0x7FFFFFFF;
  __syncthreads();

  const Quot qc = make_quot(blob_step(a.blob, g));
  const int qm = qmode(a.blob, s.L, s.H, s.D, G, g);
  const int64_t gpc = groups_per_chunk(s.L, s.H, s.D);
  const uint32_t cap = (uint32_t)a.cap_words;
  // items = (chunk, k-th layer of the group), chunk-major; wavefront w takes
  // items w, w + 16, ...
  const int lg_count = layers_in_group(a.blob, G, s.L, g, lane);
  const int items = (int)(cl_end - cl_begin) * lg_count;
  int my_left = 0;  // tokens of this wavefront's groups not yet encoded
  for (int it = wave; it < items; it += kWaves)
    my_left += (int)chunk_len(s.T, s.C, a.chunk_begin + cl_begin + it / lg_count);
  for (int it = wave; it < items; it += kWaves) {
    const int64_t cl = cl_begin + it / lg_count;  // chunk index within the call
    const int64_t c = a.chunk_begin + cl;
    const int64_t n = chunk_len(s.T, s.C, c), t0 = c * s.C;
    my_left -= (int)n;
    const int l = layer_of_group(a.blob, G, s.L, g, it % lg_count, lane);
    const int64_t gi = (((int64_t)l * 2 + kv) * s.H + h) * s.S + j;
    const int64_t slot = cl * gpc + gi;
    const __amdgpu_buffer_rsrc_t sr = make_slot_rsrc(a.scratch + (size_t)slot * a.cap_words, cap);
    const uint16_t* xb = a.x + ((((size_t)l * 2 + kv) * s.H + h) * (size_t)s.T + t0) * s.D + 64 * j;
    const uint32_t row_bytes = 2u * (uint32_t)s.D;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(xb, (uint32_t)n * row_bytes);
    uint32_t words, start;
#define CG_ENC(QM) \
  encode_group<QM, BF>(xr, (int)n, row_bytes, qc, ftab, enc_lds, sr, cap, lane, words, start, a.status, \
               left, wave, my_left)
    if (qm == kQuotMul) CG_ENC(kQuotMul);
    else if (qm == kQuotTwo) CG_ENC(kQuotTwo);
    else CG_ENC(kQuotDiv);
#undef CG_ENC
    if (lane == 0) {
      a.group_words[slot] = words;
      a.group_start[slot] = start;
    }
  }
  if (lane == 0) left[wave] = 0;
}

// ---------------------------------------------------------------------------
// record layout: one workgroup per chunk; exclusive scan of 16-byte-padded
// group sizes.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 256;

__device__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* sh, uint64_t& total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    uint64_t y = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += y;
    __syncthreads();
  }
  const uint64_t incl = sh[tid];
  total = sh[kScanThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ void __launch_bounds__(kScanThreads) k_layout(LayoutArgs a) {
  __shared__ uint64_t sh[kScanThreads];
  const int64_t c = blockIdx.x;
  const uint32_t* gw = a.group_words + c * a.gpc;
  uint64_t* go = a.group_off + c * (a.gpc + 1);
  uint64_t carry = 0;
  for (int64_t base = 0; base < a.gpc; base += kScanThreads) {
    const int64_t i = base + threadIdx.x;
    const uint64_t sz = i < a.gpc ? align_up(2 * (uint64_t)gw[i], 16) : 0;
    uint64_t tot;
    const uint64_t ex = block_excl_scan_u64(sz, sh, tot);
    if (i < a.gpc) go[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    go[a.gpc] = carry;
    a.rec_bytes[c] = align_up(rec_data_start(a.gpc) + carry, 256);
  }
}

__global__ void __launch_bounds__(kScanThreads) k_chunk_scan(ChunkScanArgs a) {
  __shared__ uint64_t sh[kScanThreads];
  uint64_t carry = 0;
  for (int64_t base = 0; base < a.n_chunks; base += kScanThreads) {
    const int64_t i = base + threadIdx.x;
    const uint64_t sz = i < a.n_chunks ? a.rec_bytes[i] : 0;
    uint64_t tot;
    const uint64_t ex = block_excl_scan_u64(sz, sh, tot);
    if (i < a.n_chunks) a.chunk_offsets[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    a.chunk_offsets[a.n_chunks] = carry;
    if (carry > a.out_cap) set_status(a.status, CG_ERR_CAPACITY);
  }
}

// ---------------------------------------------------------------------------
// record write: block 0 of each chunk writes the header, the offset and word
// tables and the zero padding; the other blocks copy group streams (one
// wavefront per group) from the scratch slots into place.
// ---------------------------------------------------------------------------
constexpr int kWriteThreads = 256;
constexpr int kCopyUnroll = 4;
typedef unsigned int v4u32_t __attribute__((ext_vector_type(4)));

// 16 output bytes from the 32 source bytes lo|hi, starting Q dwords plus
// bs bytes into lo.
template <int Q>
__device__ __forceinline__ uint4 shift_pick(const uint4& lo, const uint4& hi, uint32_t bs) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return make_uint4(__builtin_amdgcn_alignbyte(w[Q + 1], w[Q + 0], bs),
                    __builtin_amdgcn_alignbyte(w[Q + 2], w[Q + 1], bs),
                    __builtin_amdgcn_alignbyte(w[Q + 3], w[Q + 2], bs),
                    __builtin_amdgcn_alignbyte(w[Q + 4], w[Q + 3], bs));
}

// Zero the bytes of a 16-byte output chunk at or past `end` (byte offset o
// of the chunk); the stream ends on a 2-byte boundary.
__device__ __forceinline__ uint32_t keep_below(uint32_t v, uint32_t o, uint32_t end) {
  return o + 4 <= end ? v : (o + 2 <= end ? (v & 0xFFFFu) : 0u);
}

// One wavefront copies words [P, P + nw) of a scratch slot (src, 16-byte
// aligned) to dst as 16-byte chunks, zero-padded to nbytes (a multiple of
// 16). Source reads past the slot return 0 (range-checked VGPR offsets).
template <int Q>
__device__ __forceinline__ void copy_stream_q(__amdgpu_buffer_rsrc_t src, uint32_t a0, uint32_t bs,
                                              uint32_t end, __amdgpu_buffer_rsrc_t dst, uint32_t nbytes,
                                              int lane) {
  for (uint32_t base = 0; base < nbytes; base += 64 * 16 * kCopyUnroll) {
    uint4 lo[kCopyUnroll], hi[kCopyUnroll];
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) {
      const uint32_t off = base + 16u * (64u * k + lane);
      lo[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src, a0 + off, 0, 0));
      hi[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(src, a0 + off + 16, 0, 0));
    }
#pragma unroll
    for (int k = 0; k < kCopyUnroll; ++k) {
      const uint32_t off = base + 16u * (64u * k + lane);
      if (off < nbytes) {
        uint4 v = shift_pick<Q>(lo[k], hi[k], bs);
        if (off + 16 > end) {
          v.x = keep_below(v.x, off, end);
          v.y = keep_below(v.y, off + 4, end);
          v.z = keep_below(v.z, off + 8, end);
          v.w = keep_below(v.w, off + 12, end);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v), dst, off, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void copy_stream(__amdgpu_buffer_rsrc_t src, uint32_t P, uint32_t nw,
                                            __amdgpu_buffer_rsrc_t dst, uint32_t nbytes, int lane) {
  const uint32_t sb = 2u * P, a0 = sb & ~15u, q = (sb & 15u) >> 2, bs = sb & 3u, end = 2u * nw;
  switch (q) {
    case 0: copy_stream_q<0>(src, a0, bs, end, dst, nbytes, lane); break;
    case 1: copy_stream_q<1>(src, a0, bs, end, dst, nbytes, lane); break;
    case 2: copy_stream_q<2>(src, a0, bs, end, dst, nbytes, lane); break;
    default: copy_stream_q<3>(src, a0, bs, end, dst, nbytes, lane); break;
  }
}


__global__ void __launch_bounds__(kWriteThreads) k_write(WriteArgs a) {
  if (uni(a.chunk_offsets[a.n_chunks]) > a.out_cap) return;
  const int64_t nblk = 1 + (a.gpc + a.groups_per_block - 1) / a.groups_per_block;
  const int64_t cl = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int64_t c = a.chunk_begin + cl;
  uint8_t* rec = a.out + uni(a.chunk_offsets[cl]);
  const uint64_t ds = rec_data_start(a.gpc);
  const uint64_t* go = a.group_off + cl * (a.gpc + 1);
  const uint64_t data_bytes = uni(go[a.gpc]);
  const uint64_t rbytes = uni(a.rec_bytes[cl]);
  const int tid = threadIdx.x;
  if (blk == 0) {
    const uint64_t tab_end = 64 + 8 * (uint64_t)(a.gpc + 1) + 4 * (uint64_t)a.gpc;
    uint64_t* ro = reinterpret_cast<uint64_t*>(rec + 64);
    for (int64_t i = tid; i <= a.gpc; i += kWriteThreads) ro[i] = go[i];
    uint32_t* rw = reinterpret_cast<uint32_t*>(rec + 64 + 8 * (a.gpc + 1));
    for (int64_t i = tid; i < a.gpc; i += kWriteThreads) rw[i] = a.group_words[cl * a.gpc + i];
    for (uint64_t i = tab_end + tid; i < ds; i += kWriteThreads) rec[i] = 0;
    for (uint64_t i = ds + data_bytes + tid; i < rbytes; i += kWriteThreads) rec[i] = 0;
    if (tid == 0) {
      uint32_t* h = reinterpret_cast<uint32_t*>(rec);
      h[0] = kRecordMagic;
      h[1] = kVersion;
      h[2] = (uint32_t)c;
      h[3] = blob_hdr(a.blob)->level_id;
      *reinterpret_cast<uint64_t*>(rec + 16) = (uint64_t)(c * a.s.C);
      h[6] = (uint32_t)chunk_len(a.s.T, a.s.C, c);
      h[7] = (uint32_t)a.gpc;
      h[8] = (uint32_t)a.s.L;
      h[9] = (uint32_t)a.s.H;
      h[10] = (uint32_t)a.s.D;
      h[11] = (uint32_t)ds;
      *reinterpret_cast<uint64_t*>(rec + 48) = rbytes;
      *reinterpret_cast<uint64_t*>(rec + 56) = data_bytes;
    }
    return;
  }
  const int wave = wave_id(), lane = tid & 63;
  const int64_t g_begin = (blk - 1) * a.groups_per_block;
  for (int64_t gi = g_begin + wave; gi < g_begin + a.groups_per_block && gi < a.gpc;
       gi += kWriteThreads / 64) {
    const int64_t slot = cl * a.gpc + gi;
    const uint32_t nw = uni(a.group_words[slot]);
    const uint32_t P = uni(a.group_start[slot]);
    const uint64_t g0 = uni(go[gi]), g1 = uni(go[gi + 1]);
    const __amdgpu_buffer_rsrc_t src = make_rsrc(a.scratch + (size_t)slot * a.cap_words, 2u * (uint32_t)a.cap_words);
    const __amdgpu_buffer_rsrc_t dst = make_rsrc(rec + ds + g0, (uint32_t)(g1 - g0));
    copy_stream(src, P, nw, dst, (uint32_t)(g1 - g0), lane);
  }
}

// ---------------------------------------------------------------------------
// decode: one workgroup per (block of records, layer group, K|V, head, slice).
// The set's decoder tables (lane-minor, 128 KB) sit in LDS. The workgroup's
// groups (records x layers of the layer group) are dealt to the wavefronts
// round-robin, so a wavefront holds up to three; it decodes them as
// independent chains interleaved in one instruction stream, so the dependent
// LDS reads of one chain overlap the others'. Per chain a 256-word LDS ring
// (+ 64-word mirror) holds the stream, refilled 128 words ahead with one
// coalesced dword per lane.
//
// Per token and lane (x = rANS state, slot = x & 4095, w = slot >> 5):
//   info = LDS[rankx[w] - 256 * popcount(above[w] << (slot & 31))]
//        = d | (4096 - f) << 8 | b << 20
//   x = x - ((4096 - f) * (x >> 12) + b)      (= f * (x >> 12) + slot - b)
//   x < 2^16: x = x << 16 | next renorm word (ballot + mbcnt)
//   q += d (signed byte); byte 0x80: q += 128 + escape payload
//   y = fp16(fl32(q * step))
// ---------------------------------------------------------------------------
constexpr int kDecThreads = kWaves * 64;
constexpr int kRingStride = kRingWords + kRingMirror;  // 16-bit words per chain

// a * b + c on 24-bit signed operands in one instruction (the compiler would
// split a multiply by -256 into a shift and a subtraction)
__device__ __forceinline__ uint32_t mad_i24(uint32_t a, int32_t b, uint32_t c) {
  uint32_t r;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(b), "v"(c));
  return r;
}

__device__ __forceinline__ uint32_t lds_u32(const uint32_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + byte_off);
}

// x = x << 16 | w on the lanes of m only, the other lanes unchanged: one VALU
// instruction under a narrowed execution mask instead of a shift and a select.
__device__ __forceinline__ void renorm_lanes(uint32_t& x, uint32_t w, uint64_t m) {
  uint64_t saved;
  asm volatile(
      "s_and_saveexec_b64 %1, %2\n\t"
      "v_lshl_or_b32 %0, %0, 16, %3\n\t"
      "s_mov_b64 exec, %1"
      : "+v"(x), "=&s"(saved)
      : "s"(m), "v"(w)
      : "scc");
}

struct Chain {
  __amdgpu_buffer_rsrc_t src;  // the group's padded stream (reads past it give 0)
  __amdgpu_buffer_rsrc_t dst;  // output rows
  uint16_t* ring;
  uint32_t p, loaded, nw;      // words consumed / staged / in the stream
  uint32_t doff;               // byte offset of the current output row in dst
  uint32_t pref;               // per lane: the next 128-word block, one dword each
  uint32_t x, q;               // per lane: rANS state, token value mod 2^16
  int t0;                      // first token (tokens < 2^26: the host's shape limits)
  int n;
  uint32_t bt0, bt1;           // paged: byte offsets of the pages of blocks bt_base + lane, + 64
  int bt_base;
  uint32_t pg_left;            // paged: tokens left in the current page after the last stored one
  bool ok;
  // values carried between the phases of one token (pipelined loop)
  uint32_t above, rankx, info, w;
  uint64_t mr;
  int pref_it;  // pipelined loop: iteration that issued the load now in pref
  // pipelined loop: p and loaded - 128 as byte offsets (2 x words), so the
  // ring address is one mask and add and the refill test one compare
  uint32_t pb, lim_b;
};

struct GroupRef {
  const uint8_t* rec;
  uint64_t ds, dbytes;
  int64_t t0;
  int n;
  int l;
};

// Byte offset in the (layer, K|V) slab of the pool of the first row of head
// h in the page of block-table entry i (0 past the chain's last block).
__device__ __forceinline__ uint32_t page_offset(const DecodeArgs& a, int i, int last, int h,
                                                uint32_t row_bytes) {
  if (i > last) return 0u;
  const uint32_t blk = (uint32_t)a.block_table[i];
  return (blk * (uint32_t)a.s.H + (uint32_t)h) * 16u * row_bytes;
}

// The chain's window of 128 block-table entries from bt_base on, as page
// offsets in two registers (entry bt_base + lane, + 64).
__device__ __forceinline__ void load_pages(const DecodeArgs& a, Chain& c, int h, uint32_t row_bytes, int lane) {
  const int last = (c.t0 + c.n - 1) >> 4;
  c.bt0 = page_offset(a, c.bt_base + lane, last, h, row_bytes);
  c.bt1 = page_offset(a, c.bt_base + 64 + lane, last, h, row_bytes);
}

__device__ __forceinline__ uint32_t page_in_window(const Chain& c, uint32_t bi) {
  return bi < 64 ? (uint32_t)__builtin_amdgcn_readlane(c.bt0, bi)
                 : (uint32_t)__builtin_amdgcn_readlane(c.bt1, bi - 64);
}

template <bool PAGED>
__device__ __forceinline__ uint32_t row_offset(const DecodeArgs& a, Chain& c, int t, int h,
                                               uint32_t row_bytes, int lane) {
  if (!PAGED) return (uint32_t)(t - c.t0) * row_bytes;
  const int b = (t >> 4) - c.bt_base;
  if (__builtin_expect(b >= 128, 0)) {  // next window of 128 block-table entries
    c.bt_base += 128;
    load_pages(a, c, h, row_bytes, lane);
    // wait here, once per 2048 tokens, so the compiler does not have to
    // assume these loads pending (and wait for every store) on each step
    __builtin_amdgcn_s_waitcnt(0x0F70);
  }
  return page_in_window(c, (uint32_t)((t >> 4) - c.bt_base)) + (uint32_t)(t & 15) * row_bytes;
}

// Output row of token i of the chain, from the previous one: the next row of
// the same 16-token page, or at a page boundary the page the block table
// names (contiguous output: always the next row).
template <bool PAGED>
__device__ __forceinline__ void next_row(const DecodeArgs& a, Chain& c, int i, int h, uint32_t row_bytes,
                                         int lane) {
  if (!PAGED || __builtin_expect(c.pg_left != 0, 1)) {  // page boundaries: 1 token in 16
    c.doff += row_bytes;
    if (PAGED) c.pg_left -= 1;
  } else {
    c.doff = row_offset<PAGED>(a, c, c.t0 + i, h, row_bytes, lane);
    c.pg_left = 15;
  }
}

__device__ __forceinline__ void ring_put(Chain& c, uint32_t wbase, uint32_t v, int lane) {
  const uint32_t r = (wbase + 2u * lane) & (kRingWords - 1);
  *reinterpret_cast<uint32_t*>(c.ring + r) = v;
  if (r < (uint32_t)kRingMirror) *reinterpret_cast<uint32_t*>(c.ring + kRingWords + r) = v;
}

// 128 words from word wbase on, one dword per lane; reads past the group's
// padded extent (the prefetch runs ahead of the stream's end) return 0.
__device__ __forceinline__ uint32_t stream_load(const Chain& c, uint32_t wbase, int lane) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(c.src, 4u * lane + 2u * wbase, 0, 0);
}

// Sets up one group: checks its directory entry, stages its first 256 words,
// reads the head and writes token 0. c.ok = false for a damaged entry.
template <bool PAGED, bool BF>
__device__ __forceinline__ void chain_open(const DecodeArgs& a, Chain& c, const GroupRef& gr,
                                           int64_t gpc, int kv, int h, int j, float step,
                                           uint16_t* ring, int lane) {
  const Shape s = a.s;
  c.ok = false;
  const int64_t gi = (((int64_t)gr.l * 2 + kv) * s.H + h) * s.S + j;
  const uint64_t* goffs = reinterpret_cast<const uint64_t*>(gr.rec + 64);
  const uint32_t* gwords = reinterpret_cast<const uint32_t*>(gr.rec + 64 + 8 * (gpc + 1));
  const uint64_t o0 = uni(goffs[gi]), o1 = uni(goffs[gi + 1]);
  const uint32_t nw = uni(gwords[gi]);
  if ((o0 & 15) || (o1 & 15) || o0 > o1 || o1 > gr.dbytes || 2ull * nw > o1 - o0 ||
      nw < (uint32_t)kHdrWords || (o1 - o0) >= (1ull << 32) || (gi == 0 && o0 != 0) ||
      (gi == gpc - 1 && o1 != gr.dbytes)) {
    if (lane == 0) set_status(a.status, CG_ERR_CORRUPT);
    return;
  }
  c.ok = true;
  c.src = make_rsrc(gr.rec + gr.ds + o0, (uint32_t)(o1 - o0));
  c.ring = ring;
  c.nw = nw;
  c.t0 = (int)gr.t0;
  c.n = gr.n;
  {
    const uint32_t v0 = stream_load(c, 0, lane), v1 = stream_load(c, kRingBlock, lane);
    ring_put(c, 0, v0, lane);
    ring_put(c, kRingBlock, v1, lane);
  }
  c.loaded = 2 * kRingBlock;
  c.pref = stream_load(c, c.loaded, lane);
  __builtin_amdgcn_wave_barrier();
  c.x = ((uint32_t)ring[lane] << 16) | ring[64 + lane];
  c.q = ring[128 + lane];
  c.p = kHdrWords;
  const uint32_t row_bytes = 2u * (uint32_t)s.D;
  const size_t col = (size_t)64 * j;
  if (!PAGED) {
    const uint16_t* y0 = a.y + ((((size_t)gr.l * 2 + kv) * s.H + h) * (size_t)s.T + gr.t0) * s.D + col;
    c.dst = make_rsrc(y0, (uint32_t)(gr.n * row_bytes));
  } else {
    const uint16_t* p0 = a.pool + ((size_t)gr.l * 2 + kv) * (size_t)a.num_blocks * s.H * 16 * s.D + col;
    c.dst = make_rsrc(p0, (uint32_t)((uint64_t)a.num_blocks * s.H * 16 * row_bytes));
    c.bt_base = c.t0 >> 4;
    load_pages(a, c, h, row_bytes, lane);
  }
  c.doff = row_offset<PAGED>(a, c, c.t0, h, row_bytes, lane);
  c.pg_left = 15u - (uint32_t)(gr.t0 & 15);
  __builtin_amdgcn_raw_buffer_store_b16(dequantize_low16<BF>(c.q, step), c.dst, 2u * lane, c.doff, 0);
}

__device__ __forceinline__ void chain_close(const DecodeArgs& a, const Chain& c, int lane) {
  const bool bad = (__ballot(c.x != kL) != 0) || (c.p != c.nw);
  if (bad && lane == 0) set_status(a.status, CG_ERR_CORRUPT);
}

// Tokens [i_begin, i_end) of NC chains in lockstep.
template <bool PAGED, int NC, bool BF>
__device__ __forceinline__ void chain_steps(const DecodeArgs& a, Chain* c, int i_begin, int i_end,
                                            const uint32_t* tabs, int h, float step, int lane) {
  const uint32_t lane4 = 4u * lane, lane2 = 2u * lane;
  constexpr uint32_t kRbOff = 4u * (kDecRb - kDecBm);
  const uint32_t row_bytes = 2u * (uint32_t)a.s.D;
  // Retire every outstanding vector-memory load before the loop, so no load
  // issued by an earlier loop is still pending on a register this loop reuses
  // (that would put a vmcnt wait on every step). vmcnt(0), expcnt/lgkmcnt
  // unrestricted.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (int i = i_begin; i < i_end; ++i) {
    bool refill = false;
#pragma unroll
    for (int k = 0; k < NC; ++k) refill |= c[k].loaded - c[k].p < (uint32_t)kRingBlock;
    if (refill) {
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        if (c[k].loaded - c[k].p < (uint32_t)kRingBlock) {
          ring_put(c[k], c[k].loaded, c[k].pref, lane);
          c[k].loaded += kRingBlock;
          c[k].pref = stream_load(c[k], c[k].loaded, lane);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // The three dependent LDS reads of a token are issued chain by chain in
    // phases; a scheduling fence after each phase keeps the compiler from
    // serialising the chains (it would otherwise finish one chain's read
    // chain before starting the next one's).
    uint32_t above[NC], rankx[NC], info[NC], w[NC];
    uint64_t mr[NC];
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const uint32_t ob = ((c[k].x << 3) & 0x7F00u) | lane4;  // word (slot >> 5) of this lane
      above[k] = lds_u32(tabs, ob);
      rankx[k] = lds_u32(tabs, ob + kRbOff);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const uint32_t after = (uint32_t)__popc(above[k] << (c[k].x & 31u));  // starts after the slot
      info[k] = lds_u32(tabs, mad_i24(after, -256, rankx[k]));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const uint32_t x = c[k].x;
      const uint32_t fp = (info[k] >> 8) & 0xFFFu, bs = info[k] >> 20;
      c[k].x = x - (fp * (x >> 12) + bs);
      mr[k] = __ballot(c[k].x < kL);
      const uint16_t* rp = c[k].ring + (c[k].p & (kRingWords - 1));
      w[k] = rp[mbcnt_base(mr[k], 0)];  // every lane reads; only renormalising lanes use it
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      renorm_lanes(c[k].x, w[k], mr[k]);
      c[k].p += (uint32_t)__popcll(mr[k]);
      c[k].q += (uint32_t)(int32_t)(int8_t)(info[k] & 0xFFu);
    }
    uint64_t me[NC];
    bool any_esc = false;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      me[k] = __ballot((info[k] & 0xFFu) == 0x80u);
      any_esc |= me[k] != 0;
    }
    if (any_esc) {
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        if (me[k]) {
          const uint16_t* ep = c[k].ring + (c[k].p & (kRingWords - 1));
          if ((info[k] & 0xFFu) == 0x80u) c[k].q += 128u + ep[mbcnt_base(me[k], 0)];
          c[k].p += (uint32_t)__popcll(me[k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const uint16_t y = dequantize_low16<BF>(c[k].q, step);
      if (PAGED)
        next_row<PAGED>(a, c[k], i, h, row_bytes, lane);
      else
        c[k].doff += row_bytes;
      __builtin_amdgcn_raw_buffer_store_b16(y, c[k].dst, lane2, c[k].doff, 0);
    }
  }
}

// v += 2 * k for wave-uniform values, one scalar instruction
__device__ __forceinline__ void add_twice(uint32_t& v, uint32_t k) {
  asm("s_lshl1_add_u32 %0, %1, %0" : "+s"(v) : "s"(k) : "scc");
}

// ---- software-pipelined chains ---------------------------------------------
// A token of one chain is three phases, each ending in one LDS read that the
// next phase consumes:
//   A: (refill the ring) and read above/rankx of the state's slot word
//   B: read the info entry
//   C: update the state, ballot the lanes that renormalise, read their words
//   D: (consumes C's read) renormalise, advance q, escapes, store the row
// D of a token and A of the next need no LDS round trip between them, so a
// token is three slots. Chain k runs k slots behind chain 0; every slot holds
// one phase of every chain, so each LDS read is covered by a full slot of the
// other chains' work instead of being waited for at once.

// Waits for the stream load issued `age` pipelined iterations ago. Every
// iteration of an NC-chain loop issues NC stores, and a chain stores its
// token right before its refill, so at least NC * (age - 1) + 1 vector-memory
// operations were issued after that load; vector-memory operations complete
// in order, so waiting until no more than that many are outstanding suffices
// and stores issued since then need not drain.
template <int NC>
__device__ __forceinline__ void wait_stream_load(int age) {
  if (age >= 4) {
    if (NC == 3) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  } else if (age >= 2) {
    if (NC == 3) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
  }
}

// The next 128-word block into a register. Issued as inline assembly so the
// compiler does not track it (it would wait at the consumer for every store
// issued since, assuming the load could be the most recent one); the
// consumer waits with wait_stream_load instead, and chain_pipe retires all
// such loads before it returns.
__device__ __forceinline__ uint32_t stream_load_async(const Chain& c, uint32_t wbase, int lane) {
  uint32_t v;
  // s_nop 4: the compiler does not see the SGPR operands of a memory
  // instruction inside inline assembly, so it does not insert the 5 wait
  // states a VALU write of those SGPRs (e.g. a spill reload by v_readlane)
  // needs before they are read
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2, 0 offen"
               : "=&v"(v)
               : "v"(4u * lane + 2u * wbase), "s"(c.src)
               : "memory");
  return v;
}

template <int NC>
__device__ __forceinline__ void ph_a(Chain& c, const uint32_t* tabs, int lane, int it) {
  if (__builtin_expect(c.pb > c.lim_b, 0)) {  // fewer than 128 words staged
    wait_stream_load<NC>(it - c.pref_it);
    ring_put(c, c.loaded, c.pref, lane);
    c.loaded += kRingBlock;
    c.lim_b += 2u * kRingBlock;
    c.pref = stream_load_async(c, c.loaded, lane);
    c.pref_it = it;
    __builtin_amdgcn_wave_barrier();
  }
  const uint32_t ob = ((c.x << 3) & 0x7F00u) | (4u * lane);  // word (slot >> 5) of this lane
  c.above = lds_u32(tabs, ob);
  c.rankx = lds_u32(tabs, ob + 4u * (kDecRb - kDecBm));
}

__device__ __forceinline__ void ph_b(Chain& c, const uint32_t* tabs) {
  const uint32_t after = (uint32_t)__popc(c.above << (c.x & 31u));  // starts after the slot
  c.info = lds_u32(tabs, mad_i24(after, -256, c.rankx));
}

__device__ __forceinline__ void ph_c(Chain& c) {
  const uint32_t x = c.x;
  const uint32_t fp = (c.info >> 8) & 0xFFFu, bs = c.info >> 20;
  c.x = x - (fp * (x >> 12) + bs);
  c.mr = __ballot(c.x < kL);
  const uint16_t* rp =
      reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(c.ring) + (c.pb & (2u * kRingWords - 1)));
  c.w = rp[mbcnt_base(c.mr, 0)];  // every lane reads; only renormalising lanes use it
}

template <bool PAGED, bool BF, bool ADV = true>
__device__ __forceinline__ void ph_d(const DecodeArgs& a, Chain& c, int i, int h, float step,
                                     uint32_t row_bytes, int lane) {
  renorm_lanes(c.x, c.w, c.mr);
  add_twice(c.pb, (uint32_t)__popcll(c.mr));
  c.q += (uint32_t)(int32_t)(int8_t)(c.info & 0xFFu);
  // escapes and refills are rare: as unlikely branches their blocks leave
  // the loop's straight path, which then takes no branch
  const uint64_t me = __ballot((c.info & 0xFFu) == 0x80u);
  if (__builtin_expect(me != 0, 0)) {
    const uint16_t* ep = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(c.ring) +
                                                            (c.pb & (2u * kRingWords - 1)));
    if ((c.info & 0xFFu) == 0x80u) c.q += 128u + ep[mbcnt_base(me, 0)];
    add_twice(c.pb, (uint32_t)__popcll(me));
  }
  const uint16_t y = dequantize_low16<BF>(c.q, step);
  if (ADV) {
    if (PAGED)
      next_row<PAGED>(a, c, i, h, row_bytes, lane);
    else
      c.doff += row_bytes;
  }
  __builtin_amdgcn_raw_buffer_store_b16(y, c.dst, 2u * lane, c.doff, 0);
}

// Paged output of NC chains whose pages start at the same token offset (the
// chunk length a multiple of 16, or equal starts): one page counter for all,
// and every chain's row advanced at the top of the step, instead of a test
// per chain per token.
// pg: tokens left in the current page; bi: the page's index in the chains'
// windows (the same for all: their pages start at the same offset).
template <int NC>
__device__ __forceinline__ void next_rows_in_step(const DecodeArgs& a, Chain* c, int h, uint32_t row_bytes,
                                                  uint32_t& pg, uint32_t& bi, int lane) {
  if (__builtin_expect(pg != 0, 1)) {
#pragma unroll
    for (int k = 0; k < NC; ++k) c[k].doff += row_bytes;
    pg -= 1;
  } else {
    bi += 1;
    if (__builtin_expect(bi == 128, 0)) {  // next windows of 128 block-table entries
#pragma unroll
      for (int k = 0; k < NC; ++k) {
        c[k].bt_base += 128;
        load_pages(a, c[k], h, row_bytes, lane);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // as in row_offset
      bi = 0;
    }
#pragma unroll
    for (int k = 0; k < NC; ++k) c[k].doff = page_in_window(c[k], bi);  // row 0 of the page
    pg = 15;
  }
}

#define CG_SLOT __builtin_amdgcn_sched_barrier(0)

// Tokens [i0, i1) of NC = 2 or 3 chains, i1 > i0, software-pipelined. A
// scheduling fence after every phase keeps each phase's LDS read where it is
// issued (the compiler would sink the reads to the end of a slot).
template <bool PAGED, int NC, bool BF, bool SYNC>
__device__ __forceinline__ void chain_pipe(const DecodeArgs& a, Chain* c, int i0, int i1,
                                           const uint32_t* tabs, int* left, int h, float step,
                                           int lane) {
  static_assert(NC == 2 || NC == 3, "two or three chains");
  static_assert(PAGED || !SYNC, "one page counter: paged output only");
  constexpr bool ADV = !SYNC;  // the row advance: in ph_d, or for all chains per step
  uint32_t pg = SYNC ? c[0].pg_left : 0u;
  uint32_t bi = SYNC ? (uint32_t)(((c[0].t0 + i0 - 1) >> 4) - c[0].bt_base) : 0u;
  const uint32_t row_bytes = 2u * (uint32_t)a.s.D;
  // see chain_steps: no load of an earlier loop may stay pending; the
  // compiler-issued prefetch of chain_open is complete after this wait
  __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    c[k].pref_it = -8;
    c[k].pb = 2u * c[k].p;
    c[k].lim_b = 2u * (c[k].loaded - kRingBlock);
  }
  // prologue (iteration 0): chain 0 runs A, B, C of token i0; chain 1 A, B;
  // chain 2 A
  ph_a<NC>(c[0], tabs, lane, 0);
  CG_SLOT;
  ph_b(c[0], tabs);
  CG_SLOT;
  ph_a<NC>(c[1], tabs, lane, 0);
  CG_SLOT;
  ph_c(c[0]);
  CG_SLOT;
  ph_b(c[1], tabs);
  CG_SLOT;
  if (NC == 3) {
    ph_a<NC>(c[2], tabs, lane, 0);
    CG_SLOT;
  }
  int it = 1;
  const int wave = wave_id();
  for (int i = i0; i < i1 - 1; ++i, ++it) {
    if ((i & (kProgressPeriod - 1)) == 0) publish_progress<kWaves>(left, wave, i1 - i, lane);
    if (SYNC) next_rows_in_step<NC>(a, c, h, row_bytes, pg, bi, lane);
    ph_d<PAGED, BF, ADV>(a, c[0], i, h, step, row_bytes, lane);
    ph_a<NC>(c[0], tabs, lane, it);
    CG_SLOT;
    ph_c(c[1]);
    CG_SLOT;
    if (NC == 3) {
      ph_b(c[2], tabs);
      CG_SLOT;
    }
    ph_b(c[0], tabs);
    CG_SLOT;
    ph_d<PAGED, BF, ADV>(a, c[1], i, h, step, row_bytes, lane);
    ph_a<NC>(c[1], tabs, lane, it);
    CG_SLOT;
    if (NC == 3) {
      ph_c(c[2]);
      CG_SLOT;
    }
    ph_c(c[0]);
    CG_SLOT;
    ph_b(c[1], tabs);
    CG_SLOT;
    if (NC == 3) {
      ph_d<PAGED, BF, ADV>(a, c[2], i, h, step, row_bytes, lane);
      ph_a<NC>(c[2], tabs, lane, it);
      CG_SLOT;
    }
  }
  // epilogue: finish token i1 - 1
  if (SYNC) next_rows_in_step<NC>(a, c, h, row_bytes, pg, bi, lane);
  ph_d<PAGED, BF, ADV>(a, c[0], i1 - 1, h, step, row_bytes, lane);
  ph_c(c[1]);
  if (NC == 3) ph_b(c[2], tabs);
  ph_d<PAGED, BF, ADV>(a, c[1], i1 - 1, h, step, row_bytes, lane);
  if (NC == 3) {
    ph_c(c[2]);
    ph_d<PAGED, BF, ADV>(a, c[2], i1 - 1, h, step, row_bytes, lane);
  }
  // the last prefetches may still be in flight into registers the compiler
  // considers free from here on; the empty uses keep those registers
  // reserved (not reassigned to other values) until the wait
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < NC; ++k) asm volatile("" ::"v"(c[k].pref));
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    c[k].p = c[k].pb >> 1;
    if (SYNC) c[k].pg_left = pg;
  }
}

// NC chains decoded together for their common length, then the longer ones
// finish one at a time.
template <bool PAGED, int NC, bool BF>
__device__ __forceinline__ void run_chains(const DecodeArgs& a, Chain* c, const uint32_t* tabs, int* left,
                                           int h, float step, int lane) {
  int nmin = c[0].n;
#pragma unroll
  for (int k = 1; k < NC; ++k) nmin = c[k].n < nmin ? c[k].n : nmin;
  if constexpr (NC == 1) {
    chain_steps<PAGED, 1, BF>(a, c, 1, nmin, tabs, h, step, lane);
  } else {
    if (nmin > 1) {
      bool same_pages = PAGED;
#pragma unroll
      for (int k = 1; k < NC; ++k) same_pages = same_pages && c[k].pg_left == c[0].pg_left;
      if (same_pages)
        chain_pipe<PAGED, NC, BF, PAGED>(a, c, 1, nmin, tabs, left, h, step, lane);
      else
        chain_pipe<PAGED, NC, BF, false>(a, c, 1, nmin, tabs, left, h, step, lane);
    }
  }
  if constexpr (NC > 1) {
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (c[k].n > nmin) chain_steps<PAGED, 1, BF>(a, &c[k], nmin > 1 ? nmin : 1, c[k].n, tabs, h, step, lane);
  }
#pragma unroll
  for (int k = 0; k < NC; ++k) chain_close(a, c[k], lane);
}

// Several levels: the positions of the references that name table set lvl
// and whose rank among those references lies in [k0, k1), in reference order
// (at most kMaxRefsPerBlock), so a workgroup's records share its set however
// the levels of neighbouring references mix. Each wavefront scans the table
// indices 64 at a time (the results are wave-uniform). With all_refs the
// scan covers every reference; *bad reports one that names no table set.
__device__ __forceinline__ int refs_of_set(const DecodeArgs& a, int lvl, int64_t k0, int64_t k1, int64_t* sel,
                                           bool all_refs, bool* bad, int lane) {
  int found = 0;
  int64_t rank = 0;
  bool b = false;
  for (int64_t base = 0; base < a.n_refs && (rank < k1 || all_refs); base += 64) {
    const int64_t r = base + lane;
    const int t = r < a.n_refs ? a.refs[r].table : -1;
    b |= __ballot(r < a.n_refs && (t < 0 || t >= a.n_tables)) != 0;
    uint64_t m = __ballot(t == lvl);
    const int64_t cnt = __popcll(m);
    if (rank + cnt <= k0 || rank >= k1) {
      rank += cnt;
      continue;
    }
    while (m != 0 && rank < k1) {
      const int bit = __builtin_ctzll(m);
      m &= m - 1;
      if (rank >= k0 && found < kMaxRefsPerBlock) sel[found++] = base + bit;
      ++rank;
    }
  }
  *bad = b;
  return found;
}

template <bool PAGED, bool BF>
__global__ void __launch_bounds__(kDecThreads) k_decode(DecodeArgs a) {
  __shared__ uint32_t tabs[kDecDwords * 64];
  __shared__ uint16_t rings[kWaves * kChains * kRingStride];
  __shared__ int left[kWaves];  // tokens each wavefront has left (priorities)
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const Shape s = a.s;
  int64_t bid = blockIdx.x;
  const int round = (int)(bid % a.item_rounds);  // which 48 of the block's groups
  bid /= a.item_rounds;
  const int j = (int)(bid % s.S);
  bid /= s.S;
  const int h = (int)(bid % s.H);
  bid /= s.H;
  const int kv = (int)(bid % 2);
  bid /= 2;
  const int g = (int)(bid % a.g_max);
  int64_t rb = bid / a.g_max;
  const int64_t nb1 = a.split / a.refs_per_block;
  int lvl = 0;  // several levels: the table set of this copy of the blocks
  if (a.per_level) {
    const int64_t rblocks = nb1 + (a.n_refs - a.split + a.refs_per_block2 - 1) / a.refs_per_block2;
    lvl = (int)(rb / rblocks);
    rb -= lvl * rblocks;
  }
  int64_t r_begin, r_end;
  if (rb < nb1) {
    r_begin = rb * a.refs_per_block;
    r_end = r_begin + a.refs_per_block;
  } else {
    r_begin = a.split + (rb - nb1) * a.refs_per_block2;
    r_end = r_begin + a.refs_per_block2 < a.n_refs ? r_begin + a.refs_per_block2 : a.n_refs;
  }
  const bool first_block = (g == 0 && kv == 0 && h == 0 && j == 0 && lvl == 0);

  // the workgroup's table set: its copy's (several levels), else its first
  // record's, which the other records must share
  const int ti = a.per_level ? lvl : uni(a.refs[r_begin].table);
  if (ti < 0 || ti >= a.n_tables) {
    if (tid == 0 && first_block) set_status(a.status, CG_ERR_INVALID_ARG);
    return;
  }
  const int G = a.n_groups[ti];
  if (g >= G) return;
  const uint8_t* blob = a.tables[ti];
  if (!blob_ok(blob, s, G) ||
      (int32_t)uni(blob_hdr(blob)->level_id) != a.level_id[ti]) {
    if (tid == 0) set_status(a.status, CG_ERR_INVALID_ARG);
    return;
  }
  const int64_t gpc = groups_per_chunk(s.L, s.H, s.D);
  const uint64_t ds_expect = rec_data_start(gpc);
  const int64_t nch = n_chunks(s.T, s.C);

  // the workgroup's references: its block's (one level), else those of its
  // table set with ranks in the block's range (several levels)
  int64_t sel[kMaxRefsPerBlock];
  int nsel = 0;
  if (a.per_level) {
    bool bad_ref = false;
    const bool reporter = first_block && rb == 0;
    nsel = refs_of_set(a, lvl, r_begin, r_end, sel, reporter, &bad_ref, lane);
    if (bad_ref && reporter && tid == 0) set_status(a.status, CG_ERR_INVALID_ARG);
  } else {
    for (int64_t r = r_begin; r < r_end && nsel < kMaxRefsPerBlock; ++r) sel[nsel++] = r;
  }

  // record headers of this workgroup (at most kMaxRefsPerBlock = 3)
  GroupRef rr0, rr1, rr2;
  rr0.l = rr1.l = rr2.l = 0;
  int nrec = 0;
  for (int k = 0; k < nsel; ++k) {
    const int64_t r = sel[k];
    const uint8_t* rec = uni(a.refs[r].record);
    const uint64_t ref_bytes = uni(a.refs[r].bytes);
    const int rti = uni(a.refs[r].table);
    if (rti != ti) {  // another copy decodes it, or no table set has that index
      if (tid == 0 && first_block && (!a.per_level || rti < 0 || rti >= a.n_tables))
        set_status(a.status, CG_ERR_INVALID_ARG);
      continue;
    }
    if (ref_bytes < ds_expect || (reinterpret_cast<uintptr_t>(rec) & 15)) {
      if (tid == 0) set_status(a.status, CG_ERR_CORRUPT);
      continue;
    }
    const uint32_t* rh = reinterpret_cast<const uint32_t*>(rec);
    const int64_t c = uni(rh[2]);
    const uint64_t rbytes = uni(*reinterpret_cast<const uint64_t*>(rec + 48));
    const uint64_t dbytes = uni(*reinterpret_cast<const uint64_t*>(rec + 56));
    bool bad = uni(rh[0]) != kRecordMagic || uni(rh[1]) != kVersion || c >= nch ||
               (int32_t)uni(rh[3]) != a.level_id[ti];
    if (!bad) {
      bad = uni(*reinterpret_cast<const uint64_t*>(rec + 16)) != (uint64_t)(c * s.C) ||
            uni(rh[6]) != (uint32_t)chunk_len(s.T, s.C, c) || uni(rh[7]) != (uint32_t)gpc ||
            (int)uni(rh[8]) != s.L || (int)uni(rh[9]) != s.H || (int)uni(rh[10]) != s.D ||
            uni(rh[11]) != ds_expect || rbytes > ref_bytes || ds_expect + dbytes > rbytes;
    }
    if (bad) {
      if (tid == 0) set_status(a.status, CG_ERR_CORRUPT);
      continue;
    }
    const int64_t n = chunk_len(s.T, s.C, c), t0 = c * s.C;
    if (PAGED) {
      bool bt_bad = false;
      for (int64_t b = (t0 >> 4) + tid; b <= ((t0 + n - 1) >> 4); b += kDecThreads) {
        const int32_t v = a.block_table[b];
        bt_bad |= (v < 0 || (int64_t)v >= a.num_blocks);
      }
      if (__syncthreads_or(bt_bad)) {
        if (tid == 0) set_status(a.status, CG_ERR_INVALID_ARG);
        continue;
      }
    }
    GroupRef& dst = nrec == 0 ? rr0 : nrec == 1 ? rr1 : rr2;
    dst.rec = rec;
    dst.ds = ds_expect;
    dst.dbytes = dbytes;
    dst.t0 = t0;
    dst.n = (int)n;
    ++nrec;
  }
  if (nrec == 0) return;
  // items = (record, k-th layer of the group), record-major; this workgroup
  // decodes items [48 round, 48 round + 48) (a layer group of more than 48
  // layers spreads one record over several workgroups)
  const int lg_count = layers_in_group(blob, G, s.L, g, lane);
  constexpr int kRound = kWaves * kChains;
  const int base = round * kRound;
  const int items = nrec * lg_count - base < kRound ? nrec * lg_count - base : kRound;
  if (items <= 0) return;

  // the set's decoder tables, one contiguous 128 KB block
  const size_t set = (((size_t)g * 2 + kv) * s.H + h) * s.S + j;
  const uint4* dsrc = reinterpret_cast<const uint4*>(
      reinterpret_cast<const uint32_t*>(blob + tb_dec_offset(s.L, s.H, s.D, G)) + set * (kDecDwords * 64));
  for (int u = tid; u < kDecDwords * 64 / 4; u += kDecThreads) reinterpret_cast<uint4*>(tabs)[u] = dsrc[u];
  const float step = blob_step(blob, g);
  if (tid < kWaves) left[tid] = 0x7FFFFFFF;
  __syncthreads();

  // wavefront w takes items w, w + 16, w + 32 of the workgroup's. Deeper
  // layers code more bits per value, so the layer order is turned around in
  // the second record and rotated by half in the third: each wavefront gets
  // a shallow, a deep and a middle layer rather than the same depth three
  // times.
  const int mine = wave < items ? (items - 1 - wave) / kWaves + 1 : 0;
  if (mine == 0) {
    if (lane == 0) left[wave] = 0;
    return;
  }
  Chain c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
    if (k < mine) {
      const int it = base + wave + k * kWaves;
      const int ri = it / lg_count;
      GroupRef gr = ri == 0 ? rr0 : ri == 1 ? rr1 : rr2;
      int li = it - ri * lg_count;
      if (ri == 1) li = lg_count - 1 - li;
      if (ri == 2) li = (li + lg_count / 2) % lg_count;
      gr.l = layer_of_group(blob, G, s.L, g, li, lane);
      chain_open<PAGED, BF>(a, c[k], gr, gpc, kv, h, j, step, rings + (wave * kChains + k) * kRingStride,
                        lane);
    } else {
      c[k].ok = false;
    }
  }
  const bool all_ok = c[0].ok && (mine < 2 || c[1].ok) && (mine < 3 || c[2].ok);
  if (all_ok && mine == 3) {
    run_chains<PAGED, 3, BF>(a, c, tabs, left, h, step, lane);
  } else if (all_ok && mine == 2) {
    run_chains<PAGED, 2, BF>(a, c, tabs, left, h, step, lane);
  } else {
    // one chain, or a damaged directory entry among them: the rest one by one
#pragma unroll
    for (int k = 0; k < kChains; ++k)
      if (c[k].ok) run_chains<PAGED, 1, BF>(a, &c[k], tabs, left, h, step, lane);
  }
  if (lane == 0) left[wave] = 0;
}

// ---------------------------------------------------------------------------
// attention of one new token per layer over the paged cache: the consumer
// of the restored KV ("CacheGen实战" 2.3: the decoded cache is used by the
// model unchanged; "vLLM中的PagedAttention优化": K/V in 16-token physical
// blocks found through a block table). Query head qh reads kv head qh / G.
//
// k_attend: a wavefront takes pages_per_wave consecutive pages of one
// (layer, kv head) and all G <= 16 query heads of that kv head:
//   S = K_page (16 tokens x D) . Q^T (D x 16 head slots) on the matrix
//       cores (v_mfma_f32_16x16x16 f16/bf16, fp32 accumulation; products of
//       two 16-bit elements are exact in fp32);
//   online softmax per head in base 2 (scores pre-scaled by scale*log2 e);
//   O[g][d] += P[t][g] V[t][d] on the vector ALUs in fp32, each lane owning
//       D/64 adjacent dims, P broadcast from LDS.
// It writes its partial (running max, sum, unnormalised O) per head;
// k_attend_reduce merges the partials of a (layer, query head).
//
// MFMA 16x16x16 operand layout (lane i, 4 elements j): A[i%16][4(i/16)+j],
// B[4(i/16)+j][i%16], D[4(i/16)+j][i%16]. The contraction index is free to
// permute as long as A and B agree: k-step 2c+h of lane group i/16 takes
// dims 32c + 8(i/16) + 4h + j, so one 16-byte load per lane gives two steps.
// ---------------------------------------------------------------------------
constexpr int kAttWaves = 4;

typedef _Float16 att_h4 __attribute__((ext_vector_type(4)));
typedef short att_s4 __attribute__((ext_vector_type(4)));
typedef float att_f4 __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ att_f4 mfma16(uint2 a, uint2 b, att_f4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(att_s4, a), __builtin_bit_cast(att_s4, b),
                                                     c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(att_h4, a), __builtin_bit_cast(att_h4, b), c,
                                                 0, 0, 0);
}

// ND = D / 64 dims per lane in the P.V product (D = 64, 128 or 256); GM =
// head slots carried through P.V (4, 8 or 16 >= G; slots >= G see q = 0 and
// are not written)
template <bool BF, int ND, int GM>
__global__ void __launch_bounds__(kAttWaves * 64) k_attend(AttendArgs a) {
  constexpr int D = 64 * ND, KS = D / 32;  // 16-byte loads per lane per page
  __shared__ float p_lds[kAttWaves][16][16];  // [token][head slot]
  __shared__ float al_lds[kAttWaves][16];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int gi = lane & 15, gq = lane >> 4;
  const int h = blockIdx.y, l = blockIdx.z;
  const int64_t part = (int64_t)blockIdx.x * kAttWaves + wave;
  if (part >= a.n_parts) return;
  const Shape s = a.s;
  const int G = a.G;
  const int64_t pg0 = part * a.pages_per_wave;
  const int64_t pg1 = pg0 + a.pages_per_wave < a.n_pages ? pg0 + a.pages_per_wave : a.n_pages;

  // Q as the B operand: slot gi < G is query head h*G + gi, other slots 0
  uint2 qb[KS][2];
  {
    const uint16_t* qrow = a.q + ((size_t)l * a.q_heads + (size_t)h * G + (gi < G ? gi : 0)) * D;
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      uint4 v = gi < G ? *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * gq) : make_uint4(0, 0, 0, 0);
      qb[c][0] = make_uint2(v.x, v.y);
      qb[c][1] = make_uint2(v.z, v.w);
    }
  }
  const size_t kv_stride = (size_t)a.num_blocks * s.H * 16 * D;  // K -> V of a layer
  const uint16_t* kbase = a.pool + (size_t)l * 2 * kv_stride + (size_t)h * 16 * D;
  float m = -__builtin_inff();  // running max of head slot gi (log2 units)
  float lsum = 0.0f;            // this lane's share of the running sum
  float acc_o[GM][ND];
#pragma unroll
  for (int g = 0; g < GM; ++g)
#pragma unroll
    for (int k = 0; k < ND; ++k) acc_o[g][k] = 0.0f;

  // block-table entries of this wavefront's pages, one per lane
  // (pages_per_wave <= 64); an entry out of range is reported and its page
  // skipped (its loads use block 0 so they stay in bounds)
  const int npw = (int)(pg1 - pg0);
  const int32_t bt_lane = lane < npw ? a.bt[pg0 + lane] : 0;
  const bool bt_bad = lane < npw && (bt_lane < 0 || (int64_t)bt_lane >= a.num_blocks);
  const uint64_t bad_pages = __ballot(bt_bad);
  if (bad_pages && lane == 0) set_status(a.status, CG_ERR_INVALID_ARG);
  const int32_t bt_safe = bt_bad ? 0 : bt_lane;

  // one page in registers: K as MFMA A operands, V rows as this lane's dims
  using VT = typename std::conditional<ND == 1, uint16_t, typename std::conditional<ND == 2, uint32_t, uint2>::type>::type;
  auto load_page = [&](int i, uint4* kv, VT* vv) {
    const int32_t blk = __builtin_amdgcn_readlane(bt_safe, i);
    const uint16_t* kp = kbase + (size_t)blk * s.H * 16 * D;
    const uint16_t* vp = kp + kv_stride;
#pragma unroll
    for (int c = 0; c < KS; ++c) kv[c] = *reinterpret_cast<const uint4*>(kp + gi * D + 32 * c + 8 * gq);
    const int64_t left = a.n_tokens - (pg0 + i) * 16;
    const int last = left < 16 ? (int)left - 1 : 15;  // rows past the end re-read the last valid one
#pragma unroll
    for (int t = 0; t < 16; ++t)
      vv[t] = *reinterpret_cast<const VT*>(vp + (t < last ? t : last) * D + ND * lane);
  };
  uint4 kc[KS], kn[KS];
  VT vc[16], vn[16];
  if (npw > 0) load_page(0, kc, vc);
  // the first page lands before the loop, so that the loop's wait counts
  // only cover the page being prefetched (see hist_range)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  for (int i = 0; i < npw; ++i) {
    if (i + 1 < npw) load_page(i + 1, kn, vn);
    const int64_t pg = pg0 + i;
    if (!((bad_pages >> i) & 1)) {
      const int64_t left = a.n_tokens - pg * 16;
      const int nv = left < 16 ? (int)left : 16;  // valid tokens of this page
      // S = K Q^T
      att_f4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < KS; ++c) {
        sc = mfma16<BF>(make_uint2(kc[c].x, kc[c].y), qb[c][0], sc);
        sc = mfma16<BF>(make_uint2(kc[c].z, kc[c].w), qb[c][1], sc);
      }
      // sc[j] = S[token 4 gq + j][slot gi]; tokens past the end do not count
      float sv[4];
      float pm = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[j] = 4 * gq + j < nv ? sc[j] * a.scale_log2e : -__builtin_inff();
        pm = __builtin_fmaxf(pm, sv[j]);
      }
      pm = __builtin_fmaxf(pm, __shfl_xor(pm, 16));
      pm = __builtin_fmaxf(pm, __shfl_xor(pm, 32));
      const float m_new = __builtin_fmaxf(m, pm);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 on the first page
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pj = __builtin_amdgcn_exp2f(sv[j] - m_new);
        p_lds[wave][4 * gq + j][gi] = pj;
        ps += pj;
      }
      lsum = lsum * alpha + ps;
      m = m_new;
      if (gq == 0) al_lds[wave][gi] = alpha;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // O = diag(alpha) O + P^T V (rows past the end have P = 0)
      {
        float al[GM];
#pragma unroll
        for (int g4 = 0; g4 < GM / 4; ++g4)
          *reinterpret_cast<float4*>(&al[4 * g4]) = *reinterpret_cast<const float4*>(&al_lds[wave][4 * g4]);
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
          for (int k = 0; k < ND; ++k) acc_o[g][k] *= al[g];
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float v[ND];
        if constexpr (ND == 1) {
          v[0] = elem_to_f32<BF>(vc[t]);
        } else if constexpr (ND == 2) {
          v[0] = elem_to_f32<BF>((uint16_t)vc[t]);
          v[1] = elem_to_f32<BF>((uint16_t)(vc[t] >> 16));
        } else {
          v[0] = elem_to_f32<BF>((uint16_t)vc[t].x);
          v[1] = elem_to_f32<BF>((uint16_t)(vc[t].x >> 16));
          v[2] = elem_to_f32<BF>((uint16_t)vc[t].y);
          v[3] = elem_to_f32<BF>((uint16_t)(vc[t].y >> 16));
        }
        float pt[GM];
#pragma unroll
        for (int g4 = 0; g4 < GM / 4; ++g4)
          *reinterpret_cast<float4*>(&pt[4 * g4]) = *reinterpret_cast<const float4*>(&p_lds[wave][t][4 * g4]);
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
          for (int k = 0; k < ND; ++k) acc_o[g][k] = __builtin_fmaf(pt[g], v[k], acc_o[g][k]);
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int c = 0; c < KS; ++c) kc[c] = kn[c];
#pragma unroll
    for (int t = 0; t < 16; ++t) vc[t] = vn[t];
  }
  // partial of this wavefront: max and sum per head slot, unnormalised O
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const size_t pbase = (((size_t)l * s.H + h) * a.n_parts + part) * G;
  if (gq == 0 && gi < G) {
    a.part_ml[2 * (pbase + gi)] = m;
    a.part_ml[2 * (pbase + gi) + 1] = lsum;
  }
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g < G) {
      float* po = a.part_o + (pbase + g) * D + ND * lane;
#pragma unroll
      for (int k = 0; k < ND; ++k) po[k] = acc_o[g][k];
    }
  }
}

// One wavefront per (layer, query head): merge the partials.
template <int ND>
__global__ void __launch_bounds__(64) k_attend_reduce(AttendArgs a) {
  constexpr int D = 64 * ND;
  const int lane = threadIdx.x;
  const int qh = blockIdx.x, l = blockIdx.y;
  const int h = qh / a.G, g = qh % a.G;
  const size_t base = ((size_t)l * a.s.H + h) * a.n_parts * a.G + g;  // + part * G
  float M = -__builtin_inff();
  for (int64_t p = 0; p < a.n_parts; ++p) M = __builtin_fmaxf(M, a.part_ml[2 * (base + p * a.G)]);
  float den = 0.0f, o[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) o[k] = 0.0f;
  for (int64_t p = 0; p < a.n_parts; ++p) {
    const size_t i = base + p * a.G;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * i] - M);
    den = __builtin_fmaf(w, a.part_ml[2 * i + 1], den);
    const float* po = a.part_o + i * D + ND * lane;
#pragma unroll
    for (int k = 0; k < ND; ++k) o[k] = __builtin_fmaf(w, po[k], o[k]);
  }
  float* out = a.o + ((size_t)l * a.q_heads + qh) * D + ND * lane;
#pragma unroll
  for (int k = 0; k < ND; ++k) out[k] = o[k] / den;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static unsigned grid_for(uint64_t n, unsigned threads, unsigned cap) {
  uint64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  return (unsigned)(b < cap ? b : cap);
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t value, uint64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 256, 8192)), dim3(256), 0, st, p, value, n);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, uint64_t bytes, hipStream_t st) {
  const uint64_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy, dim3(grid_for(n, 256, 1 << 16)), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n);
  return hipGetLastError();
}

hipError_t launch_make_refs(const uint8_t* base, const uint64_t* offs, int32_t n, int32_t table,
                            cg_chunk_ref* refs, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_make_refs, dim3((n + 255) / 256), dim3(256), 0, st, base, offs, n, table, refs);
  return hipGetLastError();
}

hipError_t launch_set_ref(cg_chunk_ref* ref, const uint8_t* record, uint64_t bytes, int32_t table,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_set_ref, dim3(1), dim3(64), 0, st, ref, record, bytes, table);
  return hipGetLastError();
}

hipError_t launch_blob_init(const BlobInitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_blob_init, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_qcheck(const QCheckArgs& a, hipStream_t st) {
  if (a.bf)
    hipLaunchKernelGGL(k_qcheck<true>, dim3(65536 / 256, a.G), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_qcheck<false>, dim3(65536 / 256, a.G), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_hist(const HistArgs& a, hipStream_t st) {
  const uint64_t blocks = (uint64_t)a.s.L * 2 * a.s.H * a.s.S;
  if (a.s.dt == kDtypeBf16)
    hipLaunchKernelGGL(k_hist<true>, dim3((unsigned)blocks), dim3(kHistThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_hist<false>, dim3((unsigned)blocks), dim3(kHistThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a, hipStream_t st) {
  const uint64_t blocks = (uint64_t)(a.n_tables + 3) / 4;
  hipLaunchKernelGGL(k_norm, dim3((unsigned)blocks), dim3(kNormThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t st) {
  const uint64_t rblocks = (uint64_t)(a.split / a.chunks_per_block) +
                           (uint64_t)(a.n_chunks - a.split + a.chunks_per_block2 - 1) / a.chunks_per_block2;
  const uint64_t blocks = rblocks * a.G * 2 * a.s.H * a.s.S;
  if (a.s.dt == kDtypeBf16)
    hipLaunchKernelGGL(k_encode<true>, dim3((unsigned)blocks), dim3(kEncThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_encode<false>, dim3((unsigned)blocks), dim3(kEncThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_layout, dim3((unsigned)a.n_chunks), dim3(kScanThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_chunk_scan(const ChunkScanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_chunk_scan, dim3(1), dim3(kScanThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_write(const WriteArgs& a, hipStream_t st) {
  const int64_t nblk = 1 + (a.gpc + a.groups_per_block - 1) / a.groups_per_block;
  hipLaunchKernelGGL(k_write, dim3((unsigned)(a.n_chunks * nblk)), dim3(kWriteThreads), 0, st, a);
  return hipGetLastError();
}

template <bool BF, int ND>
static void launch_attend_nd(const AttendArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_parts + kAttWaves - 1) / kAttWaves), (unsigned)a.s.H, (unsigned)a.s.L);
  if (a.G <= 4)
    hipLaunchKernelGGL((k_attend<BF, ND, 4>), grid, dim3(kAttWaves * 64), 0, st, a);
  else if (a.G <= 8)
    hipLaunchKernelGGL((k_attend<BF, ND, 8>), grid, dim3(kAttWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL((k_attend<BF, ND, 16>), grid, dim3(kAttWaves * 64), 0, st, a);
}

template <bool BF>
static hipError_t launch_attend_t(const AttendArgs& a, hipStream_t st) {
  switch (a.s.D) {
    case 64: launch_attend_nd<BF, 1>(a, st); break;
    case 128: launch_attend_nd<BF, 2>(a, st); break;
    case 256: launch_attend_nd<BF, 4>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  return a.s.dt == kDtypeBf16 ? launch_attend_t<true>(a, st) : launch_attend_t<false>(a, st);
}

hipError_t launch_attend_reduce(const AttendArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.q_heads, (unsigned)a.s.L);
  switch (a.s.D) {
    case 64: hipLaunchKernelGGL((k_attend_reduce<1>), grid, dim3(64), 0, st, a); break;
    case 128: hipLaunchKernelGGL((k_attend_reduce<2>), grid, dim3(64), 0, st, a); break;
    case 256: hipLaunchKernelGGL((k_attend_reduce<4>), grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool paged, hipStream_t st) {
  const uint64_t rblocks = (uint64_t)(a.split / a.refs_per_block) +
                           (uint64_t)(a.n_refs - a.split + a.refs_per_block2 - 1) / a.refs_per_block2;
  const uint64_t blocks =
      rblocks * (a.per_level ? a.n_tables : 1) * a.g_max * 2 * a.s.H * a.s.S * a.item_rounds;
  const bool bf = a.s.dt == kDtypeBf16;
  if (paged && bf)
    hipLaunchKernelGGL((k_decode<true, true>), dim3((unsigned)blocks), dim3(kDecThreads), 0, st, a);
  else if (paged)
    hipLaunchKernelGGL((k_decode<true, false>), dim3((unsigned)blocks), dim3(kDecThreads), 0, st, a);
  else if (bf)
    hipLaunchKernelGGL((k_decode<false, true>), dim3((unsigned)blocks), dim3(kDecThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode<false, false>), dim3((unsigned)blocks), dim3(kDecThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace cg
