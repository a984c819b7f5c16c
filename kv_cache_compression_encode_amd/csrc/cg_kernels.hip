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
//   k_qcheck       per layer group: is the 4-flop quotient exact for all 65536
//                  fp16 inputs? (else the IEEE divide is used)
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
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// q = clamp(rint_even(fl32(x / step)), -32768, 32767), NaN -> 0.
// fast: v1 = x*r, e = x - v1*step (exact by FMA), v = v1 + e*r with r = RN(1/step);
// used only for steps where k_qcheck proved it equal to the IEEE quotient for
// every fp16 input.
template <bool COUNT>
__device__ __forceinline__ int32_t quantize(uint16_t xh, float step, float rcp, bool fast,
                                            uint32_t& sat, uint32_t& nan_) {
  const float x = h2f(xh);
  float v;
  if (fast) {
    const float v1 = x * rcp;
    const float e = __builtin_fmaf(-v1, step, x);
    const float v2 = __builtin_fmaf(e, rcp, v1);
    v = (e == e) ? v2 : v1;  // non-finite x: keep x*r (Inf or NaN)
  } else {
    v = x / step;
  }
  if (v != v) {
    if (COUNT) nan_ += 1;
    return 0;
  }
  const float r = __builtin_rintf(v);
  if (r > 32767.0f) {
    if (COUNT) sat += 1;
    return 32767;
  }
  if (r < -32768.0f) {
    if (COUNT) sat += 1;
    return -32768;
  }
  return (int32_t)r;
}

// x_hat = fp16_RNE(fl32(q * step)): two roundings. The empty asm keeps the
// binary32 product as a value; without it the backend may fuse multiply and
// conversion into v_fma_mixlo_f16, which rounds once and differs on ties.
__device__ __forceinline__ uint16_t dequantize(int32_t q, float step) {
  float v = (float)q * step;
  asm volatile("" : "+v"(v));
  return f2h(v);
}

__device__ __forceinline__ int32_t wrap16(int32_t v) { return ((v + 32768) & 0xFFFF) - 32768; }

__device__ __forceinline__ uint32_t symbol_of(int32_t d) {
  return ((uint32_t)(d + 127) <= 254u) ? (uint32_t)(d + 127) : (uint32_t)kEsc;
}

struct BlobHdr {
  uint32_t magic, version, L, H, D, G, level_id, C;
  uint64_t T;
  uint32_t f_offset, z0;
  uint64_t format_bytes, z1;
};

__device__ __forceinline__ const BlobHdr* blob_hdr(const uint8_t* b) {
  return reinterpret_cast<const BlobHdr*>(b);
}
__device__ __forceinline__ float blob_step(const uint8_t* b, int g) {
  return reinterpret_cast<const float*>(b + 64)[g];
}
__device__ __forceinline__ const uint8_t* blob_lg(const uint8_t* b, int G) { return b + 64 + 4 * G; }

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
    h[11] = 0;
    *reinterpret_cast<uint64_t*>(b + 48) = fbytes;
    *reinterpret_cast<uint64_t*>(b + 56) = 0;
  }
  uint32_t* qf = reinterpret_cast<uint32_t*>(b + tb_qflag_offset(a.L, a.H, a.D, a.G));
  for (int g = threadIdx.x; g < 256; g += blockDim.x) qf[g] = g < a.G ? 1u : 0u;
}

__global__ void k_qcheck(QCheckArgs a) {
  const int g = blockIdx.y;
  const uint32_t xh = blockIdx.x * blockDim.x + threadIdx.x;  // 0 .. 65535
  const float step = blob_step(a.blob, g);
  const float rcp = 1.0f / step;
  uint32_t s0 = 0, n0 = 0;
  const int32_t qf = quantize<false>((uint16_t)xh, step, rcp, true, s0, n0);
  const int32_t qi = quantize<false>((uint16_t)xh, step, rcp, false, s0, n0);
  if (qf != qi) atomicAnd(&a.qflags[g], 0u);
}

// ---------------------------------------------------------------------------
// histogram: one workgroup per (layer, K|V, head, slice); 8 wavefronts split
// the tokens; counts privatised in LDS (64 channels x 256 symbols, padded
// stride so lanes with equal symbols hit different banks).
// ---------------------------------------------------------------------------
constexpr int kHistThreads = 512;
constexpr int kHistWaves = kHistThreads / 64;
constexpr int kHistBatch = 8;

__global__ void __launch_bounds__(kHistThreads) k_hist(HistArgs a) {
  __shared__ uint32_t hist[kLanes * kEncLdsStride];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < kLanes * kEncLdsStride; i += kHistThreads) hist[i] = 0;

  const Shape s = a.s;
  int64_t bid = blockIdx.x;
  const int j = (int)(bid % s.S);
  bid /= s.S;
  const int h = (int)(bid % s.H);
  bid /= s.H;
  const int kv = (int)(bid % 2);
  const int l = (int)(bid / 2);
  const int G = a.G;
  const int g = blob_lg(a.blob, G)[l];
  const float step = blob_step(a.blob, g);
  const float rcp = 1.0f / step;
  const uint32_t* qflags = reinterpret_cast<const uint32_t*>(a.blob + tb_qflag_offset(s.L, s.H, s.D, G));
  const bool fast = qflags[g] != 0;
  __syncthreads();

  const uint16_t* __restrict__ xb =
      a.x + (((size_t)l * 2 + kv) * s.H + h) * (size_t)s.T * s.D + 64 * j + lane;
  const int64_t t_begin = s.T * wave / kHistWaves, t_end = s.T * (wave + 1) / kHistWaves;
  uint32_t* my = hist + lane * kEncLdsStride;
  uint32_t sat = 0, nan_ = 0, esc = 0, elems = 0;
  int32_t prev = 0;
  int64_t pos = t_begin % s.C;  // position inside the chunk
  if (t_begin < t_end && pos != 0) {
    uint32_t d0 = 0, d1 = 0;
    prev = quantize<false>(xb[(size_t)(t_begin - 1) * s.D], step, rcp, fast, d0, d1);
  }
  for (int64_t t = t_begin; t < t_end; t += kHistBatch) {
    uint16_t xv[kHistBatch];
#pragma unroll
    for (int k = 0; k < kHistBatch; ++k)
      xv[k] = (t + k < t_end) ? xb[(size_t)(t + k) * s.D] : (uint16_t)0;
#pragma unroll
    for (int k = 0; k < kHistBatch; ++k) {
      if (t + k < t_end) {
        const int32_t q = quantize<true>(xv[k], step, rcp, fast, sat, nan_);
        elems += 1;
        if (pos != 0) {
          const uint32_t sym = symbol_of(wrap16(q - prev));
          atomicAdd(&my[sym], 1u);
          esc += (sym == (uint32_t)kEsc);
        }
        prev = q;
        pos = (pos + 1 == s.C) ? 0 : pos + 1;
      }
    }
  }
  __syncthreads();
  uint32_t* counts = a.counts + ((((size_t)g * 2 + kv) * s.H + h) * s.D + 64 * j) * 256;
  for (int i = tid; i < kLanes * 256; i += kHistThreads) {
    const uint32_t c = hist[(i >> 8) * kEncLdsStride + (i & 255)];
    if (c) atomicAdd(&counts[i], c);
  }
  if (a.stats) {
    const uint32_t e = wave_sum(elems), st = wave_sum(sat), nn = wave_sum(nan_), es = wave_sum(esc);
    if (lane == 0) {
      atomicAdd(&a.stats[0], (unsigned long long)e);
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
  if (active) {
    const uint4 cv = reinterpret_cast<const uint4*>(a.counts + t * 256)[lane];
    c[0] = cv.x;
    c[1] = cv.y;
    c[2] = cv.z;
    c[3] = cv.w;
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
  // encoder table: f | b << 16 per symbol
  uint4 ev;
  ev.x = f[0] | (b[0] << 16);
  ev.y = f[1] | (b[1] << 16);
  ev.z = f[2] | (b[2] << 16);
  ev.w = f[3] | (b[3] << 16);
  reinterpret_cast<uint4*>(a.blob + a.enc_off)[t * 64 + lane] = ev;
  // decoder table: bitmap of symbol starts, rank bases, rank -> (sym, f-1, b)
  uint32_t* dec = reinterpret_cast<uint32_t*>(a.blob + a.dec_off) + t * kDecDwords;
  const uint32_t w0 = bm_lds[wave][2 * lane], w1 = bm_lds[wave][2 * lane + 1];
  const uint32_t p0 = __popc(w0), p1 = __popc(w1);
  const uint32_t pex = wave_excl_scan(p0 + p1, lane);
  dec[2 * lane] = w0;
  dec[2 * lane + 1] = w1;
  dec[128 + 2 * lane] = pex - 1u;
  dec[128 + 2 * lane + 1] = pex + p0 - 1u;
  uint32_t r = rank0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (f[k]) {
      dec[256 + r] = (uint32_t)(4 * lane + k) | ((f[k] - 1u) << 8) | (b[k] << 20);
      r += 1;
    }
    if ((uint32_t)(4 * lane + k) >= K) dec[256 + 4 * lane + k] = 0;
  }
}

// ---------------------------------------------------------------------------
// encode: one workgroup per (chunk, layer group, K|V, head, slice); its 16
// wavefronts take the layers of the group; the group's 64 encoder tables and
// a table of RU(1/f) for f = 1..4096 sit in LDS.
// Exact quotient: floor(x/f) = trunc(fl64(x) * RU(1/f)) for x < 2^32, f <= 2^12.
// ---------------------------------------------------------------------------
constexpr int kEncThreads = kWaves * 64;
constexpr int kEncBatch = 8;

__global__ void __launch_bounds__(kEncThreads) k_encode(EncodeArgs a) {
  __shared__ uint32_t ftab[kLanes * kEncLdsStride];
  __shared__ double rcp_tab[kM + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Shape s = a.s;
  int64_t bid = blockIdx.x;
  const int j = (int)(bid % s.S);
  bid /= s.S;
  const int h = (int)(bid % s.H);
  bid /= s.H;
  const int kv = (int)(bid % 2);
  bid /= 2;
  const int g = (int)(bid % a.G);
  const int64_t cl = bid / a.G;  // chunk index within the call
  const int64_t c = a.chunk_begin + cl;
  const int G = a.G;
  const BlobHdr* bh = blob_hdr(a.blob);
  if (bh->magic != kTableMagic || bh->version != kVersion || (int)bh->L != s.L ||
      (int)bh->H != s.H || (int)bh->D != s.D || (int)bh->G != G) {
    if (tid == 0) set_status(a.status, CG_ERR_INVALID_ARG);
    return;
  }
  const uint64_t enc_off = tb_enc_offset(s.L, s.H, s.D, G);
  const uint32_t* esrc = reinterpret_cast<const uint32_t*>(a.blob + enc_off) +
                         ((((size_t)g * 2 + kv) * s.H + h) * s.D + 64 * j) * kEncDwords;
  for (int u = tid; u < kLanes * kEncDwords / 4; u += kEncThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(esrc)[u];
    uint32_t* d = ftab + (u >> 6) * kEncLdsStride + (u & 63) * 4;
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
  for (int f = tid + 1; f <= (int)kM; f += kEncThreads) {
    double r = 1.0 / (double)f;
    if (__builtin_fma(r, (double)f, -1.0) < 0.0) r = __longlong_as_double(__double_as_longlong(r) + 1);
    rcp_tab[f] = r;
  }
  if (tid == 0) rcp_tab[0] = 0.0;
  __syncthreads();

  const float step = blob_step(a.blob, g);
  const float rcp = 1.0f / step;
  const uint32_t* qflags = reinterpret_cast<const uint32_t*>(a.blob + tb_qflag_offset(s.L, s.H, s.D, G));
  const bool fast = qflags[g] != 0;
  const uint8_t* lg = blob_lg(a.blob, G);
  const int64_t n = chunk_len(s.T, s.C, c), t0 = c * s.C;
  const int64_t gpc = groups_per_chunk(s.L, s.H, s.D);
  const uint32_t* my = ftab + lane * kEncLdsStride;
  bool table_err = false;
  int cnt = 0;
  for (int l = 0; l < s.L; ++l) {
    if (lg[l] != g) continue;
    if ((cnt++ % kWaves) != wave) continue;
    const int64_t gi = (((int64_t)l * 2 + kv) * s.H + h) * s.S + j;
    const int64_t slot = cl * gpc + gi;
    uint16_t* __restrict__ sb = a.scratch + (size_t)slot * a.cap_words;
    const uint16_t* __restrict__ xb =
        a.x + ((((size_t)l * 2 + kv) * s.H + h) * (size_t)s.T + t0) * s.D + 64 * j + lane;
    uint32_t P = (uint32_t)a.cap_words;
    uint32_t x = kL;
    uint32_t d0 = 0, d1 = 0;
    int32_t qhi = quantize<false>(xb[(size_t)(n - 1) * s.D], step, rcp, fast, d0, d1);
    for (int64_t i = n - 1; i >= 1; i -= kEncBatch) {
      uint16_t xv[kEncBatch];
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k)
        xv[k] = (i - 1 - k >= 0) ? xb[(size_t)(i - 1 - k) * s.D] : (uint16_t)0;
#pragma unroll
      for (int k = 0; k < kEncBatch; ++k) {
        if (i - k >= 1) {
          const int32_t qlo = quantize<false>(xv[k], step, rcp, fast, d0, d1);
          const int32_t dlt = wrap16(qhi - qlo);
          const uint32_t sym = symbol_of(dlt);
          const uint32_t e = my[sym];
          uint32_t f = e & 0xFFFFu, bb = e >> 16;
          if (f == 0) {
            table_err = true;
            f = kM;
            bb = 0;
          }
          // escape payloads of this token (read after its renorm words)
          const bool is_esc = sym == (uint32_t)kEsc;
          const uint64_t me = __ballot(is_esc);
          if (me) {
            P -= (uint32_t)__popcll(me);
            if (is_esc) sb[P + mbcnt(me)] = (uint16_t)(dlt & 0xFFFF);
          }
          // renormalise: x >= f * 2^20  <=>  x > (f << 20) - 1 (wraps to ~0 for f = 4096)
          const bool need = x > ((f << 20) - 1u);
          const uint64_t mr = __ballot(need);
          P -= (uint32_t)__popcll(mr);
          if (need) {
            sb[P + mbcnt(mr)] = (uint16_t)(x & 0xFFFFu);
            x >>= 16;
          }
          // x <- floor(x/f)*4096 + x mod f + b  =  x + floor(x/f)*(4096-f) + b
          const uint32_t qd = (uint32_t)((double)x * rcp_tab[f]);
          x = x + qd * (kM - f) + bb;
          qhi = qlo;
        }
      }
    }
    P -= 64;
    sb[P + lane] = (uint16_t)(qhi & 0xFFFF);
    P -= 64;
    sb[P + lane] = (uint16_t)(x & 0xFFFFu);
    P -= 64;
    sb[P + lane] = (uint16_t)(x >> 16);
    if (lane == 0) {
      a.group_words[slot] = (uint32_t)a.cap_words - P;
      a.group_start[slot] = P;
    }
  }
  if (__ballot(table_err) && lane == 0) set_status(a.status, CG_ERR_TABLE);
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

__global__ void __launch_bounds__(kWriteThreads) k_write(WriteArgs a) {
  if (a.chunk_offsets[a.n_chunks] > a.out_cap) return;
  const int64_t nblk = 1 + (a.gpc + a.groups_per_block - 1) / a.groups_per_block;
  const int64_t cl = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int64_t c = a.chunk_begin + cl;
  uint8_t* rec = a.out + a.chunk_offsets[cl];
  const uint64_t ds = rec_data_start(a.gpc);
  const uint64_t* go = a.group_off + cl * (a.gpc + 1);
  const uint64_t data_bytes = go[a.gpc];
  const uint64_t rbytes = a.rec_bytes[cl];
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
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t g_begin = (blk - 1) * a.groups_per_block;
  for (int64_t gi = g_begin + wave; gi < g_begin + a.groups_per_block && gi < a.gpc;
       gi += kWriteThreads / 64) {
    const int64_t slot = cl * a.gpc + gi;
    const uint32_t nw = a.group_words[slot];
    const uint16_t* src = a.scratch + (size_t)slot * a.cap_words + a.group_start[slot];
    uint32_t* dst = reinterpret_cast<uint32_t*>(rec + ds + go[gi]);
    const uint32_t ndw = (uint32_t)((go[gi + 1] - go[gi]) / 4);
    for (uint32_t k = lane; k < ndw; k += 64) {
      const uint32_t w0 = 2 * k < nw ? src[2 * k] : 0u;
      const uint32_t w1 = 2 * k + 1 < nw ? src[2 * k + 1] : 0u;
      dst[k] = w0 | (w1 << 16);
    }
  }
}

// ---------------------------------------------------------------------------
// decode: one workgroup per (record, layer group, K|V, head, slice); the 64
// decoder tables of the slice sit in LDS and each wavefront decodes the
// groups of one layer at a time. Per wavefront a 512-word LDS ring holds the
// stream, refilled 256 words ahead with coalesced 8-byte loads.
//
// Per token and lane: slot = x & 4095; rank = rankbase[slot>>5] +
// popcount(bitmap[slot>>5] << (31 - (slot&31))); (sym, f, b) = info[rank];
// x = f*(x>>12) + slot - b; renormalise from the ring (ballot + mbcnt);
// escape payload likewise; q += d (mod 2^16); y = fp16(fl32(q*step)).
// ---------------------------------------------------------------------------
constexpr int kDecThreads = kWaves * 64;

template <bool PAGED>
__device__ __forceinline__ void decode_group(const DecodeArgs& a, const uint32_t* __restrict__ tabs,
                                             uint16_t* ring, const uint8_t* __restrict__ rec,
                                             uint64_t ds, uint64_t data_bytes, int64_t gpc, int l,
                                             int kv, int h, int j, int64_t t0, int64_t n,
                                             float step, int lane) {
  const Shape s = a.s;
  const int64_t gi = (((int64_t)l * 2 + kv) * s.H + h) * s.S + j;
  const uint64_t* goffs = reinterpret_cast<const uint64_t*>(rec + 64);
  const uint32_t* gwords = reinterpret_cast<const uint32_t*>(rec + 64 + 8 * (gpc + 1));
  const uint64_t o0 = goffs[gi], o1 = goffs[gi + 1];
  const uint32_t nw = gwords[gi];
  if ((o0 & 15) || (o1 & 15) || o0 > o1 || o1 > data_bytes || 2ull * nw > o1 - o0 ||
      nw < (uint32_t)kHdrWords || (gi == 0 && o0 != 0) || (gi == gpc - 1 && o1 != data_bytes)) {
    if (lane == 0) set_status(a.status, CG_ERR_CORRUPT);
    return;
  }
  const uint8_t* __restrict__ gb = rec + ds + o0;
  const uint32_t pw = (uint32_t)((o1 - o0) >> 1);  // readable words, multiple of 8
  auto load4 = [&](uint32_t wbase) -> uint2 {
    const uint32_t w = wbase + 4u * lane;
    if (w + 4u <= pw) return *reinterpret_cast<const uint2*>(gb + 2ull * w);
    return make_uint2(0u, 0u);
  };
  auto put4 = [&](uint32_t wbase, uint2 v) {
    *reinterpret_cast<uint2*>(ring + ((wbase + 4u * lane) & (kRingWords - 1))) = v;
  };
  {
    const uint2 v0 = load4(0), v1 = load4(256);
    put4(0, v0);
    put4(256, v1);
  }
  uint32_t loaded = 512;
  uint2 pref = load4(512);
  __builtin_amdgcn_wave_barrier();

  uint32_t x = ((uint32_t)ring[lane] << 16) | ring[64 + lane];
  int32_t q = (int16_t)ring[128 + lane];
  uint32_t p = kHdrWords;
  const uint32_t* __restrict__ tb = tabs + lane * kDecLdsStride;

  uint16_t* __restrict__ yp = nullptr;
  size_t ystride = 0;
  if (!PAGED) {
    yp = a.y + ((((size_t)l * 2 + kv) * s.H + h) * (size_t)s.T + t0) * s.D + 64 * j + lane;
    ystride = (size_t)s.D;
    yp[0] = dequantize(q, step);
  }
  const size_t pool_base = PAGED ? (((size_t)l * 2 + kv) * (size_t)a.num_blocks) : 0;
  auto pool_ptr = [&](int64_t t) -> uint16_t* {
    const int32_t blk = __builtin_amdgcn_readfirstlane(a.block_table[t >> 4]);
    return a.pool + (((pool_base + (size_t)blk) * s.H + h) * 16 + (size_t)(t & 15)) * s.D + 64 * j + lane;
  };
  if (PAGED) *pool_ptr(t0) = dequantize(q, step);

  for (int64_t i = 1; i < n; ++i) {
    if (loaded - p < 256u) {
      put4(loaded, pref);
      loaded += 256;
      pref = load4(loaded);
      __builtin_amdgcn_wave_barrier();
    }
    const uint32_t slot = x & (kM - 1);
    const uint32_t wi = slot >> 5;
    const uint32_t bm = tb[wi], rb = tb[128 + wi];
    const uint32_t rank = (uint32_t)__popc(bm << (31u - (slot & 31u))) + rb;
    const uint32_t info = tb[256 + (rank & 255u)];
    const uint32_t sym = info & 255u, fm1 = (info >> 8) & 4095u, bsym = info >> 20;
    x = (fm1 + 1u) * (x >> 12) + slot - bsym;
    const bool need = x < kL;
    const uint64_t mr = __ballot(need);
    if (need) x = (x << 16) | ring[(p + mbcnt(mr)) & (kRingWords - 1)];
    p += (uint32_t)__popcll(mr);
    int32_t d = (int32_t)sym - 127;
    const bool is_esc = sym == (uint32_t)kEsc;
    const uint64_t me = __ballot(is_esc);
    if (me) {
      if (is_esc) d = (int16_t)ring[(p + mbcnt(me)) & (kRingWords - 1)];
      p += (uint32_t)__popcll(me);
    }
    q = (int32_t)(int16_t)(q + d);
    const uint16_t y = dequantize(q, step);
    if (PAGED) {
      *pool_ptr(t0 + i) = y;
    } else {
      yp += ystride;
      *yp = y;
    }
  }
  const bool bad = (__ballot(x != kL) != 0) || (p != nw);
  if (bad && lane == 0) set_status(a.status, CG_ERR_CORRUPT);
}

template <bool PAGED>
__global__ void __launch_bounds__(kDecThreads) k_decode(DecodeArgs a) {
  __shared__ uint32_t tabs[kLanes * kDecLdsStride];
  __shared__ uint32_t rings[kWaves * kRingWords / 2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Shape s = a.s;
  int64_t bid = blockIdx.x;
  const int j = (int)(bid % s.S);
  bid /= s.S;
  const int h = (int)(bid % s.H);
  bid /= s.H;
  const int kv = (int)(bid % 2);
  bid /= 2;
  const int g = (int)(bid % a.g_max);
  const int64_t r = bid / a.g_max;
  const bool first_block = (g == 0 && kv == 0 && h == 0 && j == 0);

  const cg_chunk_ref ref = a.refs[r];
  const int ti = ref.table;
  if (ti < 0 || ti >= a.n_tables) {
    if (tid == 0 && first_block) set_status(a.status, CG_ERR_INVALID_ARG);
    return;
  }
  const int G = a.n_groups[ti];
  if (g >= G) return;
  const uint8_t* blob = a.tables[ti];
  const BlobHdr* bh = blob_hdr(blob);
  if (bh->magic != kTableMagic || bh->version != kVersion || (int)bh->L != s.L ||
      (int)bh->H != s.H || (int)bh->D != s.D || (int)bh->G != G ||
      (int32_t)bh->level_id != a.level_id[ti]) {
    if (tid == 0) set_status(a.status, CG_ERR_INVALID_ARG);
    return;
  }
  // record header
  const uint8_t* rec = ref.record;
  const int64_t gpc = groups_per_chunk(s.L, s.H, s.D);
  const uint64_t ds_expect = rec_data_start(gpc);
  if (ref.bytes < ds_expect || (reinterpret_cast<uintptr_t>(rec) & 15)) {
    if (tid == 0) set_status(a.status, CG_ERR_CORRUPT);
    return;
  }
  const uint32_t* rh = reinterpret_cast<const uint32_t*>(rec);
  const int64_t c = rh[2];
  const int64_t nch = n_chunks(s.T, s.C);
  const uint64_t rbytes = *reinterpret_cast<const uint64_t*>(rec + 48);
  const uint64_t dbytes = *reinterpret_cast<const uint64_t*>(rec + 56);
  bool bad = rh[0] != kRecordMagic || rh[1] != kVersion || c >= nch ||
             (int32_t)rh[3] != a.level_id[ti];
  if (!bad) {
    bad = *reinterpret_cast<const uint64_t*>(rec + 16) != (uint64_t)(c * s.C) ||
          rh[6] != (uint32_t)chunk_len(s.T, s.C, c) || rh[7] != (uint32_t)gpc ||
          (int)rh[8] != s.L || (int)rh[9] != s.H || (int)rh[10] != s.D || rh[11] != ds_expect ||
          rbytes > ref.bytes || ds_expect + dbytes > rbytes;
  }
  if (bad) {
    if (tid == 0) set_status(a.status, CG_ERR_CORRUPT);
    return;
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
      return;
    }
  }
  // the 64 decoder tables of this (group, K|V, head, slice)
  const uint32_t* dsrc = reinterpret_cast<const uint32_t*>(blob + tb_dec_offset(s.L, s.H, s.D, G)) +
                         ((((size_t)g * 2 + kv) * s.H + h) * s.D + 64 * j) * kDecDwords;
  for (int u = tid; u < kLanes * kDecDwords / 4; u += kDecThreads) {
    const uint4 v = reinterpret_cast<const uint4*>(dsrc)[u];
    uint32_t* d = tabs + (u >> 7) * kDecLdsStride + (u & 127) * 4;
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
  __syncthreads();
  const float step = blob_step(blob, g);
  const uint8_t* lg = blob_lg(blob, G);
  uint16_t* ring = reinterpret_cast<uint16_t*>(rings + wave * (kRingWords / 2));
  int cnt = 0;
  for (int l = 0; l < s.L; ++l) {
    if (lg[l] != g) continue;
    if ((cnt++ % kWaves) != wave) continue;
    decode_group<PAGED>(a, tabs, ring, rec, ds_expect, dbytes, gpc, l, kv, h, j, t0, n, step, lane);
  }
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

hipError_t launch_blob_init(const BlobInitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_blob_init, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_qcheck(const QCheckArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_qcheck, dim3(65536 / 256, a.G), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_hist(const HistArgs& a, hipStream_t st) {
  const uint64_t blocks = (uint64_t)a.s.L * 2 * a.s.H * a.s.S;
  hipLaunchKernelGGL(k_hist, dim3((unsigned)blocks), dim3(kHistThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a, hipStream_t st) {
  const uint64_t blocks = (uint64_t)(a.n_tables + 3) / 4;
  hipLaunchKernelGGL(k_norm, dim3((unsigned)blocks), dim3(kNormThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t st) {
  const uint64_t blocks = (uint64_t)a.n_chunks * a.G * 2 * a.s.H * a.s.S;
  hipLaunchKernelGGL(k_encode, dim3((unsigned)blocks), dim3(kEncThreads), 0, st, a);
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

hipError_t launch_decode(const DecodeArgs& a, bool paged, hipStream_t st) {
  const uint64_t blocks = (uint64_t)a.n_refs * a.g_max * 2 * a.s.H * a.s.S;
  if (paged)
    hipLaunchKernelGGL(k_decode<true>, dim3((unsigned)blocks), dim3(kDecThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_decode<false>, dim3((unsigned)blocks), dim3(kDecThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace cg
