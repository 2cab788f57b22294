// Streaming (HBM-bound) kernels of the optimizer step: momentum EMA with
// sum-of-squares partials, the fused Lion step, sign + 1-bit pack or int8
// signs, majority vote + update (or the vote as a matrix), the polar update,
// and the small per-problem finalize kernels.  Every kernel reads and writes each element once with 16-byte
// vector accesses where the problem size allows, and reduces in a fixed
// order so results are run-to-run identical.
//
// Sources: SignMuon technical summary (gist.science/ja/paper/2605.16311),
// CacheMuon technical summary (gist.science/ja/paper/2606.16371), LionMuon
// technical summary (gist.science/pt/paper/2605.19811).
#include "sm_internal.hpp"

namespace sm {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = kThreads * 8;  // elements per block iteration
// A launch whose read-modify-write data exceeds the 256 MB Infinity Cache
// streams it with non-temporal accesses (nothing of it would still be cached
// when the next step reads it back); smaller data stays cacheable.
constexpr double kStreamBytes = 256.0 * 1024 * 1024;
static_assert(kChunk == kNormChunk, "the norm partials count chunks of kChunk");

template <typename T>
__device__ __forceinline__ float round_to(float v) {
  return v;
}
template <>
__device__ __forceinline__ float round_to<bf16_t>(float v) {
  return bf2f(f2bf(v));
}

// Loads up to 8 elements starting at e0 (< count); missing ones read as 0.
template <typename T>
__device__ __forceinline__ void load8_tail(const T* p, int64_t e0, int64_t count, bool vec,
                                           float* v) {
  if (vec && e0 + 8 <= count) {
    load8<T>(p + e0, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (e0 + e < count) ? Elem<T>::load(p + e0 + e) : 0.f;
  }
}

// load8_tail for data read once (the gradients): non-temporal 16-byte loads
// keep the streams from evicting what the next kernels read back (the
// momentum, which the Newton-Schulz launches read in place).
template <typename T>
__device__ __forceinline__ void load8_once(const T* p, int64_t e0, int64_t count, bool vec,
                                           float* v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  if (vec && e0 + 8 <= count) {
    if constexpr (sizeof(T) == 2) {
      const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + e0));
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
      }
    } else {
      const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + e0));
      const u32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + e0 + 4));
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = __uint_as_float(w[q]);
    }
  } else {
    load8_tail<T>(p, e0, count, vec, v);
  }
}

template <typename T>
__device__ __forceinline__ void store8_tail(T* p, int64_t e0, int64_t count, bool vec,
                                            const float* v) {
  if (vec && e0 + 8 <= count) {
    store8<T>(p + e0, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e0 + e < count) Elem<T>::store(p + e0 + e, v[e]);
  }
}

// store8_tail for data not read back soon (a Lion step's momentum, the
// weights): non-temporal 16-byte stores.
template <typename T>
__device__ __forceinline__ void store8_once(T* p, int64_t e0, int64_t count, bool vec,
                                            const float* v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  if (vec && e0 + 8 <= count) {
    if constexpr (sizeof(T) == 2) {
      u32x4_t o;
      o.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
      o.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
      o.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
      o.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(p + e0));
    } else {
      u32x4_t a, b;
      a.x = __float_as_uint(v[0]); a.y = __float_as_uint(v[1]);
      a.z = __float_as_uint(v[2]); a.w = __float_as_uint(v[3]);
      b.x = __float_as_uint(v[4]); b.y = __float_as_uint(v[5]);
      b.z = __float_as_uint(v[6]); b.w = __float_as_uint(v[7]);
      __builtin_nontemporal_store(a, reinterpret_cast<u32x4_t*>(p + e0));
      __builtin_nontemporal_store(b, reinterpret_cast<u32x4_t*>(p + e0 + 4));
    }
  } else {
    store8_tail<T>(p, e0, count, vec, v);
  }
}

// beta*m + (1-beta)*g as one fixed float32 sequence: the product (1-beta)*g
// is rounded, then fused with beta*m (one more rounding).  Fixing the order
// keeps sign decisions on the result reproducible off the GPU.
__device__ __forceinline__ float ema32(float beta, float m, float omb, float g) {
  return __fmaf_rn(beta, m, __fmul_rn(omb, g));
}

// Sum-of-squares accumulation shared by every producer of norm partials, so
// that the EMA kernel and the standalone reduction give identical bits:
// entries beyond the problem are loaded as 0 and add exactly nothing.
__device__ __forceinline__ float sumsq8(float acc, const float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __fmaf_rn(v[e], v[e], acc);
  return acc;
}

// Fixed-order block sum: wave butterfly, then wave 0 adds the 4 wave sums.
__device__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = 0.f;
  if (threadIdx.x == 0) r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// Byte of sign bits for 8 entries: bit e set iff v[e] < 0 (NaN, +-0 -> 0).
__device__ __forceinline__ uint32_t neg_byte(const float* v, int64_t e0, int64_t count) {
  uint32_t byte = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e0 + e < count && v[e] < 0.f) byte |= 1u << e;
  return byte;
}

// The sign word of 64 consecutive entries, assembled across the 8 lanes that
// hold them: lane 8q + i of a wave holds the byte of entries 8i..8i+7 of the
// group's word (bit e of the byte = entry 8i + e); every lane of the group
// gets the word.  All lanes of the wave must call it.
__device__ __forceinline__ uint64_t group8_word(uint32_t byte) {
  const int sh = 8 * (threadIdx.x & 7);
  uint32_t lo = sh < 32 ? byte << sh : 0u;
  uint32_t hi = sh >= 32 ? byte << (sh - 32) : 0u;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    lo |= (uint32_t)__shfl_xor((int)lo, o, 64);
    hi |= (uint32_t)__shfl_xor((int)hi, o, 64);
  }
  return ((uint64_t)hi << 32) | lo;
}

// Stores the sign word of the thread's 8-lane group: the thread's entries
// start at e0 = 8 * (thread index in a 64-entry-aligned run), so word e0/64.
__device__ __forceinline__ void store_group_word(uint64_t* bits, int64_t e0, int64_t words,
                                                 uint32_t byte) {
  const uint64_t w = group8_word(byte);
  const int64_t wi = e0 >> 6;
  if ((threadIdx.x & 7) == 0 && wi < words) bits[wi] = w;
}

// Eight int8 signs (-1 iff v[e] < 0, else +1) of entries e0..e0+7, stored
// as one 8-byte word when all are inside and the target is aligned.
__device__ __forceinline__ void store_signs8(int8_t* s, int64_t e0, int64_t count,
                                             const float* v) {
  if (e0 + 8 <= count && (reinterpret_cast<uintptr_t>(s + e0) & 7u) == 0) {
    uint64_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= (uint64_t)(v[e] < 0.f ? 0xFFu : 0x01u) << (8 * e);
    *reinterpret_cast<uint64_t*>(s + e0) = word;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e0 + e < count) s[e0 + e] = v[e] < 0.f ? (int8_t)-1 : (int8_t)1;
  }
}

// ------------------------------------------------------------------ EMA

// The EMA of one problem's chunks part, part + nparts, ...; returns this
// thread's sum of squares of the stored x values.
template <typename TM, typename TG, typename TX>
__device__ __forceinline__ float ema_run(TM* m, const TG* g, TX* xo, int64_t count, float beta,
                                         bool vec, int64_t part, int64_t nparts, bool stream) {
  const float omb = 1.0f - beta;
  float acc = 0.f;
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  for (int64_t ci = part; ci < nchunks; ci += nparts) {
    const int64_t e0 = ci * kChunk + (int64_t)threadIdx.x * 8;
    if (e0 >= count) continue;
    float mv[8], gv[8];
    if (stream) load8_once<TM>(m, e0, count, vec, mv);
    else load8_tail<TM>(m, e0, count, vec, mv);
    load8_once<TG>(g, e0, count, vec, gv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = round_to<TM>(ema32(beta, mv[e], omb, gv[e]));
      mv[e] = v;
      gv[e] = round_to<TX>(v);  // 0 beyond the end: both inputs load as 0
    }
    acc = sumsq8(acc, gv);
    if (stream) store8_once<TM>(m, e0, count, vec, mv);
    else store8_tail<TM>(m, e0, count, vec, mv);
    if (xo) store8_tail<TX>(xo, e0, count, vec, gv);
  }
  return acc;
}

// Problem b = matrix b / per, worker b % per; blocks past the problem's
// norm_parts have nothing to do.
template <typename TM, typename TG>
__global__ __launch_bounds__(kThreads) void k_ema_tbl(EmaTbl t, int per, float beta, bool stream) {
  __shared__ float red[4];
  const int b = blockIdx.y, q = b / per, w = b - q * per;
  const EmaMat& e = t.m[q];
  const int parts = norm_parts(e.count);
  if ((int)blockIdx.x >= parts) return;
  TM* m = static_cast<TM*>(e.mom) + (int64_t)w * e.count;
  const TG* g = static_cast<const TG*>(e.grad) + (int64_t)w * e.count;
  TM* xo = e.x ? static_cast<TM*>(e.x) + (int64_t)w * e.count : nullptr;
  const float acc = ema_run<TM, TG, TM>(m, g, xo, e.count, beta, (e.count % 8) == 0,
                                        blockIdx.x, parts, stream);
  float s = block_sum(acc, red);
  if (threadIdx.x == 0) e.partials[(int64_t)w * kNormParts + blockIdx.x] = s;
}

// LionMuon: ghat = b1*M + (1-b1)*G (direction), M <- b2*M + (1-b2)*G.
template <typename TM, typename TG, typename TX>
__global__ __launch_bounds__(kThreads) void k_lion(PtrTbl mom, PtrTbl grad, int per,
                                                   int64_t count, float b1, float b2, TX* x,
                                                   float* partials, uint64_t* bits,
                                                   int64_t words, int8_t* s8, bool vec,
                                                   bool stream) {
  __shared__ float red[4];
  const int b = blockIdx.y;
  TM* m = (TM*)tbl_addr(mom, b, per, count * (int64_t)sizeof(TM));
  const TG* g = (const TG*)tbl_addr(grad, b, per, count * (int64_t)sizeof(TG));
  TX* xo = x ? x + (int64_t)b * count : nullptr;
  uint64_t* bo = bits ? bits + (int64_t)b * words : nullptr;
  int8_t* so = s8 ? s8 + (int64_t)b * count : nullptr;
  const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
  float acc = 0.f;
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  for (int64_t ci = blockIdx.x; ci < nchunks; ci += gridDim.x) {
    const int64_t e0 = ci * kChunk + (int64_t)threadIdx.x * 8;
    uint32_t byte = 0;
    if (e0 < count) {
      float mv[8], gv[8], dv[8];
      // a large Lion step's momentum streams (see kStreamBytes); a Muon
      // step's stays cacheable, like the G_hat its NS reads next
      if (!stream) load8_tail<TM>(m, e0, count, vec, mv);
      else load8_once<TM>(m, e0, count, vec, mv);
      load8_once<TG>(g, e0, count, vec, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dv[e] = ema32(b1, mv[e], omb1, gv[e]);
        mv[e] = round_to<TM>(ema32(b2, mv[e], omb2, gv[e]));
      }
      if (!stream) store8_tail<TM>(m, e0, count, vec, mv);
      else store8_once<TM>(m, e0, count, vec, mv);
      if (bo) {
        byte = neg_byte(dv, e0, count);
      } else if (so) {
        store_signs8(so, e0, count, dv);
      } else if (xo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dv[e] = round_to<TX>(dv[e]);
        acc = sumsq8(acc, dv);
        store8_tail<TX>(xo, e0, count, vec, dv);
      }
    }
    if (bo) store_group_word(bo, e0, words, byte);
  }
  if (!bo && !so) {
    float s = block_sum(acc, red);
    if (threadIdx.x == 0 && partials) partials[(int64_t)b * kNormParts + blockIdx.x] = s;
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_sumsq(const T* x, int64_t count, float* partials,
                                                    bool vec) {
  __shared__ float red[4];
  const int b = blockIdx.y;
  const T* xp = x + (int64_t)b * count;
  float acc = 0.f;
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  for (int64_t ci = blockIdx.x; ci < nchunks; ci += gridDim.x) {
    const int64_t e0 = ci * kChunk + (int64_t)threadIdx.x * 8;
    if (e0 >= count) continue;
    float v[8];
    load8_tail<T>(xp, e0, count, vec, v);
    acc = sumsq8(acc, v);
  }
  float s = block_sum(acc, red);
  if (threadIdx.x == 0) partials[(int64_t)b * kNormParts + blockIdx.x] = s;
}

// One wave per problem: lane l sums partials l, l + 64, ... in order (fp64),
// then the lanes combine in a fixed butterfly, so the result is the same on
// every run.
__device__ __forceinline__ void finalize_one(const float* p, int parts, float eps, float* out) {
  double s = 0.0;
  for (int i = threadIdx.x; i < parts; i += 64) s += (double)p[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (threadIdx.x == 0) *out = (float)(1.0 / (sqrt(s) + (double)eps));
}

__global__ __launch_bounds__(64) void k_scale_finalize(const float* partials, int parts,
                                                       float eps, float* scale) {
  const int b = blockIdx.x;
  finalize_one(partials + (int64_t)b * kNormParts, parts, eps, scale + b);
}

__global__ __launch_bounds__(64) void k_scale_finalize_tbl(EmaTbl t, int per, float eps) {
  const int b = blockIdx.x, q = b / per, w = b - q * per;
  const EmaMat& e = t.m[q];
  finalize_one(e.partials + (int64_t)w * kNormParts, norm_parts(e.count), eps, e.scale + w);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_sign_pack(const T* x, int64_t count,
                                                        uint64_t* bits, int64_t words,
                                                        bool vec) {
  const int b = blockIdx.y;
  const T* xp = x + (int64_t)b * count;
  uint64_t* bo = bits + (int64_t)b * words;
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  for (int64_t ci = blockIdx.x; ci < nchunks; ci += gridDim.x) {
    const int64_t e0 = ci * kChunk + (int64_t)threadIdx.x * 8;
    uint32_t byte = 0;
    if (e0 < count) {
      float v[8];
      load8_tail<T>(xp, e0, count, vec, v);
      byte = neg_byte(v, e0, count);
    }
    store_group_word(bo, e0, words, byte);
  }
}

// int8 signs: a thread keeps kSignUnroll chunks' loads in flight before it
// writes any signs (with one 16-byte load per thread at a time the int8
// signs ran at 4.8-5.3 TB/s on large inputs, with four 5.6-5.9).  Block
// iteration c takes chunks c * kSignUnroll .. + kSignUnroll - 1.
constexpr int kSignUnroll = 4;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_sign_int8(const T* x, int64_t count, int8_t* s,
                                                        bool vec) {
  const int b = blockIdx.y;
  const T* xp = x + (int64_t)b * count;
  int8_t* sp = s + (int64_t)b * count;
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  for (int64_t c0 = (int64_t)blockIdx.x * kSignUnroll; c0 < nchunks;
       c0 += (int64_t)gridDim.x * kSignUnroll) {
    float v[kSignUnroll][8];
#pragma unroll
    for (int u = 0; u < kSignUnroll; ++u) {
      const int64_t e0 = (c0 + u) * kChunk + (int64_t)threadIdx.x * 8;
      if (c0 + u < nchunks && e0 < count) load8_tail<T>(xp, e0, count, vec, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kSignUnroll; ++u) {
      const int64_t e0 = (c0 + u) * kChunk + (int64_t)threadIdx.x * 8;
      if (c0 + u < nchunks && e0 < count) store_signs8(sp, e0, count, v[u]);
    }
  }
}

// ------------------------------------------------------------------ 1-bit vote

// Per block iteration a tile of 256 sign words (16384 entries).  Phase 1:
// thread t reads word t of every worker (8-byte loads, each worker's 2 KB of
// the tile contiguous) and counts the negatives of its 64 entries in
// bit-sliced form: plane p of the count of entry j is bit j of c[p], and a
// worker's word is added with a ripple of carries through the 7 planes
// (counts up to 64).  The vote of entry j is +1 iff 2 n_neg < M and -1 iff
// 2 n_neg > M (0 on a tie), i.e. n_neg < ceil(M/2) and n_neg > floor(M/2),
// compared plane by plane from the top.  The two 64-bit masks go to LDS.
// Phase 2: thread t takes the tile's 8-entry groups t, t + 256, ...: their
// vote bytes come from LDS, and the weights are read and written with
// 16-byte accesses that are contiguous across the block.
constexpr int kVotePlanes = 7;

__device__ __forceinline__ void bits_less_greater(const uint64_t* c, int k, uint64_t* lt,
                                                  uint64_t* gt) {
  uint64_t l = 0, g = 0, eq = ~0ull;
#pragma unroll
  for (int p = kVotePlanes - 1; p >= 0; --p) {
    if ((k >> p) & 1) {
      l |= eq & ~c[p];
      eq &= c[p];
    } else {
      g |= eq & c[p];
      eq &= ~c[p];
    }
  }
  *lt = l;
  *gt = g;
}

template <typename TW, bool UPDATE, bool STREAM>
__device__ __forceinline__ void vote_bits_tiles(const uint64_t* sg, int M, int64_t stride,
                                                int64_t count, TW* wp, float lr,
                                                int8_t* vote_out, bool vec, int64_t tile0,
                                                int64_t tstep, uint64_t* pos_s,
                                                uint64_t* neg_s) {
  const int64_t words = (count + 63) / 64;
  const int64_t ntiles = (words + kThreads - 1) / kThreads;
  const int k_pos = (M + 1) / 2, k_neg = M / 2;
  for (int64_t tile = tile0; tile < ntiles; tile += tstep) {
    const int64_t wi = tile * kThreads + threadIdx.x;
    uint64_t c[kVotePlanes];
#pragma unroll
    for (int p = 0; p < kVotePlanes; ++p) c[p] = 0;
    if (wi < words) {
      for (int k0 = 0; k0 < M; k0 += 8) {
        uint64_t wd[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)       // all eight loads issued before the adds
          if constexpr (STREAM)
            wd[q] = k0 + q < M ? __builtin_nontemporal_load(sg + (int64_t)(k0 + q) * stride + wi)
                               : 0ull;
          else
            wd[q] = k0 + q < M ? sg[(int64_t)(k0 + q) * stride + wi] : 0ull;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          uint64_t carry = wd[q];
#pragma unroll
          for (int p = 0; p < kVotePlanes; ++p) {
            const uint64_t t = c[p] & carry;
            c[p] ^= carry;
            carry = t;
          }
        }
      }
    }
    uint64_t pos, neg, unused;
    bits_less_greater(c, k_pos, &pos, &unused);   // n_neg < ceil(M/2): +1
    bits_less_greater(c, k_neg, &unused, &neg);   // n_neg > floor(M/2): -1
    pos_s[threadIdx.x] = pos;
    neg_s[threadIdx.x] = neg;
    __syncthreads();
    const uint8_t* pb = reinterpret_cast<const uint8_t*>(pos_s);
    const uint8_t* nb = reinterpret_cast<const uint8_t*>(neg_s);
    const int64_t et = tile * (int64_t)kThreads * 64;
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      const int q = g8 * kThreads + threadIdx.x;   // 8-entry group within the tile
      const int64_t e0 = et + (int64_t)q * 8;
      if (e0 < count) {
        const uint32_t pbyte = pb[q], nbyte = nb[q];
        float wv[8];
        int vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = (int)((pbyte >> e) & 1u) - (int)((nbyte >> e) & 1u);
        // large weights stream past the caches (see kStreamBytes), like the
        // signs above; the vote matrix of a polar step stays cacheable for its
        // norm pass
        if constexpr (UPDATE) {
          if constexpr (STREAM) load8_once<TW>(wp, e0, count, vec, wv);
          else load8_tail<TW>(wp, e0, count, vec, wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) wv[e] = wv[e] - lr * (float)vv[e];  // lr*v exact: one rounding
          if constexpr (STREAM) store8_once<TW>(wp, e0, count, vec, wv);
          else store8_tail<TW>(wp, e0, count, vec, wv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) wv[e] = (float)vv[e];
          store8_tail<TW>(wp, e0, count, vec, wv);
        }
        if (UPDATE && vote_out) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e0 + e < count) vote_out[e0 + e] = (int8_t)vv[e];
        }
      }
    }
    __syncthreads();   // the masks are rewritten by the next tile
  }
}

// Vote over M <= 64 workers from int8 signs, 8 entries per thread: the
// integer sum of the workers' bytes, as the SUM all-reduce of the int8
// variant would deliver it; V = sign(sum), 0 on ties.  UPDATE: W <- rnd_W(
// fp32(W) - lr V) in place (and the vote to vote_out); otherwise V itself is
// written as TW.  sg is the matrix's first worker's signs, the M workers
// `stride` bytes apart; threads first, first + step, ... of the matrix's
// 8-entry groups.
template <int ENC, typename TW, bool UPDATE>
__device__ __forceinline__ void vote_body(const void* sg, int M, int64_t stride, int64_t count,
                                          TW* wp, float lr, int8_t* vote_out, bool vec,
                                          int64_t first, int64_t step) {
  const int64_t n8 = (count + 7) / 8;
  for (int64_t i = first; i < n8; i += step) {
    const int64_t e0 = 8 * i;
    int sum[8];
    static_assert(ENC == 1, "the packed-bit vote runs in vote_bits_tiles");
    {
      const int8_t* sb = static_cast<const int8_t*>(sg);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = 0;
      const bool full = e0 + 8 <= count && (stride & 7) == 0 &&
                        (reinterpret_cast<uintptr_t>(sb + e0) & 7u) == 0;
      if (full) {
        // workers 8 at a time, all 8 loads issued before their sums
        for (int k0 = 0; k0 < M; k0 += 8) {
          uint64_t wd[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            wd[q] = k0 + q < M
                ? *reinterpret_cast<const uint64_t*>(sb + (int64_t)(k0 + q) * stride + e0)
                : 0ull;
#pragma unroll
          for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] += (int)(int8_t)(uint8_t)(wd[q] >> (8 * e));
        }
      } else {
        for (int k = 0; k < M; ++k) {
          const int8_t* src = sb + (int64_t)k * stride + e0;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e0 + e < count) sum[e] += (int)src[e];
        }
      }
    }
    int vv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) vv[e] = (sum[e] > 0) - (sum[e] < 0);
    float wv[8];
    if constexpr (UPDATE) {
      load8_tail<TW>(wp, e0, count, vec, wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = wv[e] - lr * (float)vv[e];  // lr*v is exact: one rounding
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = (float)vv[e];
    }
    store8_tail<TW>(wp, e0, count, vec, wv);
    if (UPDATE && vote_out) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (e0 + e < count) vote_out[e0 + e] = (int8_t)vv[e];
    }
  }
}

template <int ENC, typename TW, bool UPDATE>
__global__ __launch_bounds__(kThreads) void k_vote(const void* signs, int M, int64_t stride,
                                                   int64_t mat_stride, int64_t count, PtrTbl w,
                                                   float lr, int8_t* vote_out, bool vec,
                                                   bool stream) {
  const int j = blockIdx.y;
  const void* sg = ENC == 0
      ? static_cast<const void*>(static_cast<const uint64_t*>(signs) + j * mat_stride)
      : static_cast<const void*>(static_cast<const int8_t*>(signs) + j * mat_stride);
  if constexpr (ENC == 0) {
    __shared__ uint64_t pos_s[kThreads], neg_s[kThreads];
    if (stream)
      vote_bits_tiles<TW, UPDATE, true>(static_cast<const uint64_t*>(sg), M, stride, count,
                                        (TW*)w.p[j], lr, vote_out, vec, blockIdx.x, gridDim.x,
                                        pos_s, neg_s);
    else
      vote_bits_tiles<TW, UPDATE, false>(static_cast<const uint64_t*>(sg), M, stride, count,
                                         (TW*)w.p[j], lr, vote_out, vec, blockIdx.x, gridDim.x,
                                         pos_s, neg_s);
  } else {
    vote_body<ENC, TW, UPDATE>(sg, M, stride, count, (TW*)w.p[j], lr, vote_out, vec,
                               (int64_t)blockIdx.x * kThreads + threadIdx.x,
                               (int64_t)gridDim.x * kThreads);
  }
}

// The vote + update of matrices of different shapes in one launch (one
// matrix per blockIdx.y, described by the table).
template <int ENC, typename TW>
__global__ __launch_bounds__(kThreads) void k_vote_tbl(VoteTbl t, int M, float lr, bool stream) {
  const VoteMat& v = t.m[blockIdx.y];
  if constexpr (ENC == 0) {
    __shared__ uint64_t pos_s[kThreads], neg_s[kThreads];
    if (stream)
      vote_bits_tiles<TW, true, true>(static_cast<const uint64_t*>(v.signs), M, v.stride,
                                      v.count, static_cast<TW*>(v.w), lr, nullptr,
                                      (v.count % 8) == 0, blockIdx.x, gridDim.x, pos_s, neg_s);
    else
      vote_bits_tiles<TW, true, false>(static_cast<const uint64_t*>(v.signs), M, v.stride,
                                       v.count, static_cast<TW*>(v.w), lr, nullptr,
                                       (v.count % 8) == 0, blockIdx.x, gridDim.x, pos_s, neg_s);
  } else {
    vote_body<ENC, TW, true>(v.signs, M, v.stride, v.count, static_cast<TW*>(v.w), lr, nullptr,
                             (v.count % 8) == 0, (int64_t)blockIdx.x * kThreads + threadIdx.x,
                             (int64_t)gridDim.x * kThreads);
  }
}

template <typename TD, typename TW>
__global__ __launch_bounds__(kThreads) void k_polar_update(const TD* d, int64_t count,
                                                           PtrTbl w, float lr, bool vec,
                                                           bool stream) {
  const int j = blockIdx.y;
  const TD* dp = d + (int64_t)j * count;
  TW* wp = (TW*)w.p[j];
  const int64_t n8 = (count + 7) / 8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t e0 = 8 * i;
    float wv[8], dv[8];
    if (stream) {   // large: past the caches (see kStreamBytes)
      load8_once<TW>(wp, e0, count, vec, wv);
      load8_once<TD>(dp, e0, count, vec, dv);
    } else {
      load8_tail<TW>(wp, e0, count, vec, wv);
      load8_tail<TD>(dp, e0, count, vec, dv);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = __fsub_rn(wv[e], __fmul_rn(lr, dv[e]));
    if (stream) store8_once<TW>(wp, e0, count, vec, wv);
    else store8_tail<TW>(wp, e0, count, vec, wv);
  }
}

// q = s + a I for a batch of r x r bf16 matrices (problem p at s + p ss and
// q + p sq), summed in float32 and rounded to bf16.  Eight consecutive
// entries of one row per thread (r % 8 == 0, 16-byte aligned rows); with
// `lower`, entries of 256 x 256 tiles above the diagonal are skipped.
__global__ __launch_bounds__(kThreads) void k_add_identity(const bf16_t* s, int64_t ss,
                                                           bf16_t* q, int64_t sq, int r,
                                                           float a, int lower) {
  const int64_t rr = (int64_t)r * r;
  const bf16_t* sp = s + (int64_t)blockIdx.y * ss;
  bf16_t* qp = q + (int64_t)blockIdx.y * sq;
  for (int64_t e0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8; e0 < rr;
       e0 += (int64_t)gridDim.x * kThreads * 8) {
    float v[8];
    load8<bf16_t>(sp + e0, v);
    const int64_t row = e0 / r;
    const int64_t d = row - (e0 - row * r);   // diagonal entry's offset in the eight
    if (lower && ((e0 - row * r) >> 8) > (row >> 8)) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (d == e) v[e] = __fadd_rn(v[e], a);
    store8<bf16_t>(qp + e0, v);
  }
}

__global__ void k_gather_has_cache(PtrTbl cs, int per, int nprob, int32_t* hc) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nprob) return;
  hc[b] = reinterpret_cast<const int32_t*>(tbl_addr(cs, b, per, 8))[0];
}

__global__ void k_cache_decide(const float* resid, int parts, int nprob, int r,
                               const int32_t* hc, PtrTbl cs, int per, int mode, float gamma,
                               int32_t t32, int32_t* flags, float* err, int32_t* refreshed,
                               PtrTbl diag, bool has_diag) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nprob) return;
  int refresh;
  float e = -1.0f;
  if (mode == 1 || !hc[b]) {
    refresh = 1;
  } else {
    double sum = 0.0;
    for (int i = 0; i < parts; ++i) sum += (double)resid[(int64_t)b * parts + i];
    e = (float)(sqrt(sum) / sqrt((double)r));
    refresh = (mode == 2) ? 0 : !(e <= gamma);
  }
  flags[b] = refresh;
  if (err) err[b] = e;
  if (refreshed) refreshed[b] = refresh;
  if (has_diag) {   // problem b's {err, refreshed} row, by the table of matrices
    float* row = const_cast<float*>(reinterpret_cast<const float*>(tbl_addr(diag, b, per, 8)));
    row[0] = e;
    row[1] = (float)refresh;
  }
  if (refresh) {
    int32_t* st = const_cast<int32_t*>(reinterpret_cast<const int32_t*>(tbl_addr(cs, b, per, 8)));
    st[0] = 1;
    st[1] = t32;
  }
}


// *out = 1 iff some flag of the sets is 1 (one block; __syncthreads_or
// combines the threads).
__global__ __launch_bounds__(kThreads) void k_any_flags(FlagSets fs, int32_t* out) {
  int v = 0;
  for (int a = 0; a < fs.count; ++a)
    for (int i = threadIdx.x; i < fs.n[a]; i += kThreads) v |= fs.f[a][i] == 1;
  v = __syncthreads_or(v);
  if (threadIdx.x == 0) *out = v ? 1 : 0;
}

// The cached Q of every refreshed problem as a whole float32 r x r matrix,
// from the bf16 matrix stored as its 256 x 256 tiles on and below the
// diagonal (entries above come from the mirror tiles).  One 64 x 64 block of
// the output per workgroup, staged through LDS so that a mirror block is
// read along its stored rows and written transposed.
__global__ __launch_bounds__(kThreads) void k_q_store(const bf16_t* src, int64_t sst, int r,
                                                      PtrTbl q, int per, const int32_t* flags) {
  const int b = blockIdx.y;
  if (flags[b] != 1) return;
  __shared__ float tile[64][65];
  const int nb = (r + 63) / 64;
  const int i0 = (blockIdx.x / nb) * 64, j0 = (blockIdx.x % nb) * 64;
  const bool lower = (i0 >> 8) >= (j0 >> 8);
  const bf16_t* sp = src + (int64_t)b * sst;
  // source block: rows (lower ? i0 : j0) .., columns (lower ? j0 : i0) ..
  const int sr0 = lower ? i0 : j0, sc0 = lower ? j0 : i0;
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int a = e >> 6, c = e & 63;
    const int row = sr0 + a, col = sc0 + c;
    const float v = (row < r && col < r) ? bf2f(sp[(int64_t)row * r + col]) : 0.f;
    if (lower) tile[a][c] = v; else tile[c][a] = v;
  }
  __syncthreads();
  float* qp = reinterpret_cast<float*>(const_cast<char*>(
      tbl_addr(q, b, per, (int64_t)r * r * (int64_t)sizeof(float))));
  for (int e = threadIdx.x; e < 64 * 64; e += kThreads) {
    const int a = e >> 6, c = e & 63;
    if (i0 + a < r && j0 + c < r) qp[(int64_t)(i0 + a) * r + (j0 + c)] = tile[a][c];
  }
}

// Float32 cache -> bf16 matrix (round to nearest even), 8 entries per thread.
__global__ __launch_bounds__(kThreads) void k_q_load(PtrTbl q, int per, int r, bf16_t* dst,
                                                     int64_t dst_stride, const int32_t* flags) {
  const int b = blockIdx.y;
  if (flags[b] != 1) return;
  const int64_t rr = (int64_t)r * r;
  const float* src = reinterpret_cast<const float*>(tbl_addr(q, b, per, rr * 4));
  bf16_t* d = dst + (int64_t)b * dst_stride;
  for (int64_t e0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8; e0 < rr;
       e0 += (int64_t)gridDim.x * kThreads * 8) {
    float v[8];
    load8<float>(src + e0, v);
    store8<bf16_t>(d + e0, v);
  }
}

// Compacts the indices of the set flags, in increasing order: a block-wide
// inclusive scan per 256 flags.
__global__ __launch_bounds__(kThreads) void k_compact_flags(const int32_t* flags, int n,
                                                            int32_t* dyn) {
  __shared__ int scan[kThreads];
  int base = 0;
  for (int i0 = 0; i0 < n; i0 += kThreads) {
    const int i = i0 + (int)threadIdx.x;
    const int f = (i < n && flags[i] == 1) ? 1 : 0;
    scan[threadIdx.x] = f;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int v = (int)threadIdx.x >= off ? scan[threadIdx.x - off] : 0;
      __syncthreads();
      scan[threadIdx.x] += v;
      __syncthreads();
    }
    if (f) dyn[1 + base + scan[threadIdx.x] - 1] = i;
    base += scan[kThreads - 1];
    __syncthreads();
  }
  if (threadIdx.x == 0) dyn[0] = base;
}

// Blocks per problem of a grid-stride streaming launch (blockIdx.y = the
// problem) whose problems need at most `need` block iterations each, and
// about `total` blocks in all, never more: blocks run in rounds of what the
// CUs hold at once, and a total just above a whole number of rounds of long
// grid-stride blocks leaves a lone last round.
inline unsigned blocks_per_problem(int64_t need, int nprob, int64_t total) {
  int64_t want = total / (nprob > 0 ? nprob : 1);
  if (want < 1) want = 1;
  return (unsigned)(need < want ? need : want);
}

inline int stream_blocks(int64_t count, int nprob) {
  // enough blocks in flight to fill 256 CUs several times over
  return (int)blocks_per_problem((count + kChunk - 1) / kChunk, nprob, 4096);
}

}  // namespace

// ------------------------------------------------------------------ launchers


sm_status launch_ema_tbl(const EmaMat* mats, int nmat, int per, int mdt, int gdt, float beta,
                         bool finalize, float eps, hipStream_t s) {
  for (int q0 = 0; q0 < nmat; q0 += kEmaMax) {
    const int n = std::min(kEmaMax, nmat - q0);
    EmaTbl t;
    std::memset(&t, 0, sizeof(t));
    int parts = 1;
    double bytes = 0.0;
    for (int q = 0; q < n; ++q) {
      t.m[q] = mats[q0 + q];
      parts = std::max(parts, norm_parts(t.m[q].count));
      bytes += (double)per * t.m[q].count *
               (2.0 * dt_size(mdt) + dt_size(gdt) + (t.m[q].x ? dt_size(mdt) : 0.0));
    }
    double mbytes = 0.0;
    for (int q = 0; q < n; ++q) mbytes += (double)per * t.m[q].count * dt_size(mdt);
    const bool stream = mbytes > kStreamBytes;
    prof_begin(SM_K_EMA, bytes, s);
    SM_DISPATCH_DT(mdt, TM, SM_DISPATCH_DT(gdt, TG,
        hipLaunchKernelGGL((k_ema_tbl<TM, TG>), dim3(parts, n * per), dim3(kThreads), 0, s, t,
                           per, beta, stream)));
    prof_end(s);
    SM_TRY(check_launch());
    if (finalize) {
      double fb = 0.0;
      for (int q = 0; q < n; ++q) fb += (double)per * (norm_parts(t.m[q].count) + 1) * 4.0;
      prof_begin(SM_K_MISC, fb, s);
      hipLaunchKernelGGL(k_scale_finalize_tbl, dim3(n * per), dim3(64), 0, s, t, per, eps);
      prof_end(s);
      SM_TRY(check_launch());
    }
  }
  return SM_OK;
}

sm_status launch_lion(const PtrTbl& mom, const PtrTbl& grad, int per, int nprob, int64_t count,
                      int mdt, int gdt, float beta1, float beta2, void* x, int xdt,
                      float* partials, uint64_t* bits, int64_t words, int8_t* s8,
                      hipStream_t s) {
  if (nprob <= 0 || count <= 0) return SM_OK;
  const bool vec = (count % 8) == 0;
  dim3 grid(norm_parts(count), nprob);
  double bytes = (double)nprob * count * (2.0 * dt_size(mdt) + dt_size(gdt)) +
                 (bits ? (double)nprob * words * 8.0
                       : (s8 ? (double)nprob * count : (double)nprob * count * dt_size(xdt)));
  const bool stream = x == nullptr && (double)nprob * count * dt_size(mdt) > kStreamBytes;
  prof_begin(SM_K_LION, bytes, s);
  SM_DISPATCH_DT(mdt, TM, SM_DISPATCH_DT(gdt, TG, SM_DISPATCH_DT(xdt, TX,
      hipLaunchKernelGGL((k_lion<TM, TG, TX>), grid, dim3(kThreads), 0, s, mom, grad, per,
                         count, beta1, beta2, (TX*)x, partials, bits, words, s8, vec,
                         stream))));
  prof_end(s);
  return check_launch();
}

sm_status launch_sumsq(const void* x, int dt, int nprob, int64_t count, float* partials,
                       hipStream_t s) {
  if (nprob <= 0) return SM_OK;
  const bool vec = (count % 8) == 0;
  dim3 grid(norm_parts(count), nprob);
  prof_begin(SM_K_NORM, (double)nprob * count * dt_size(dt), s);
  SM_DISPATCH_DT(dt, T,
      hipLaunchKernelGGL((k_sumsq<T>), grid, dim3(kThreads), 0, s, (const T*)x, count,
                         partials, vec));
  prof_end(s);
  return check_launch();
}

sm_status launch_scale_finalize(const float* partials, int nprob, int64_t count, float eps,
                                float* scale, hipStream_t s) {
  if (nprob <= 0) return SM_OK;
  const int parts = norm_parts(count);
  prof_begin(SM_K_MISC, (double)nprob * (parts + 1) * 4.0, s);
  hipLaunchKernelGGL(k_scale_finalize, dim3(nprob), dim3(64), 0, s, partials, parts, eps,
                     scale);
  prof_end(s);
  return check_launch();
}

sm_status launch_sign_pack(const void* x, int dt, int nprob, int64_t count, uint64_t* bits,
                           int64_t words, hipStream_t s) {
  if (nprob <= 0 || count <= 0) return SM_OK;
  const bool vec = (count % 8) == 0 && (reinterpret_cast<uintptr_t>(x) % 16) == 0;
  dim3 grid(stream_blocks(count, nprob), nprob);
  prof_begin(SM_K_SIGN_PACK, (double)nprob * ((double)count * dt_size(dt) + words * 8.0), s);
  SM_DISPATCH_DT(dt, T,
      hipLaunchKernelGGL((k_sign_pack<T>), grid, dim3(kThreads), 0, s, (const T*)x, count,
                         bits, words, vec));
  prof_end(s);
  return check_launch();
}

sm_status launch_sign_int8(const void* x, int dt, int nprob, int64_t count, int8_t* s8,
                           hipStream_t s) {
  if (nprob <= 0 || count <= 0) return SM_OK;
  const bool vec = (count % 8) == 0 && (reinterpret_cast<uintptr_t>(x) % 16) == 0;
  // one block iteration per block (up to about a million blocks): short
  // blocks leave a tail of one iteration
  const int64_t nchunks = (count + kChunk - 1) / kChunk;
  dim3 grid(blocks_per_problem((nchunks + kSignUnroll - 1) / kSignUnroll, nprob, 1 << 20),
            nprob);
  prof_begin(SM_K_SIGN_PACK, (double)nprob * count * (dt_size(dt) + 1.0), s);
  SM_DISPATCH_DT(dt, T,
      hipLaunchKernelGGL((k_sign_int8<T>), grid, dim3(kThreads), 0, s, (const T*)x, count, s8,
                         vec));
  prof_end(s);
  return check_launch();
}

sm_status launch_vote(int enc, const void* signs, int M, int64_t stride, int64_t mat_stride,
                      int nmat, int64_t count, const PtrTbl& w, int wdt, float lr,
                      int8_t* vote_out, bool update, hipStream_t s) {
  if (nmat <= 0 || count <= 0) return SM_OK;
  const bool vec = (count % 8) == 0;
  const int64_t n8 = (count + 7) / 8;
  // bits: one block iteration per tile of kThreads words; int8: of kThreads 8-entry groups
  int64_t need = enc == SM_ENC_BITS ? ((count + 63) / 64 + kThreads - 1) / kThreads
                                    : (n8 + kThreads - 1) / kThreads;
  dim3 grid(blocks_per_problem(need, nmat, 4096), nmat);
  const double sign_bytes = enc == SM_ENC_BITS ? M / 8.0 : (double)M;
  double bytes = (double)nmat * count *
                 (sign_bytes + (update ? 2.0 : 1.0) * dt_size(wdt) + (vote_out ? 1.0 : 0.0));
  const bool stream = (double)nmat * count * dt_size(wdt) > kStreamBytes;
  prof_begin(SM_K_VOTE_UPDATE, bytes, s);
  if (enc == SM_ENC_BITS) {
    if (update) {
      SM_DISPATCH_DT(wdt, TW,
          hipLaunchKernelGGL((k_vote<0, TW, true>), grid, dim3(kThreads), 0, s, signs, M,
                             stride, mat_stride, count, w, lr, vote_out, vec, stream));
    } else {
      SM_DISPATCH_DT(wdt, TW,
          hipLaunchKernelGGL((k_vote<0, TW, false>), grid, dim3(kThreads), 0, s, signs, M,
                             stride, mat_stride, count, w, lr, nullptr, vec, stream));
    }
  } else {
    if (update) {
      SM_DISPATCH_DT(wdt, TW,
          hipLaunchKernelGGL((k_vote<1, TW, true>), grid, dim3(kThreads), 0, s, signs, M,
                             stride, mat_stride, count, w, lr, vote_out, vec, stream));
    } else {
      SM_DISPATCH_DT(wdt, TW,
          hipLaunchKernelGGL((k_vote<1, TW, false>), grid, dim3(kThreads), 0, s, signs, M,
                             stride, mat_stride, count, w, lr, nullptr, vec, stream));
    }
  }
  prof_end(s);
  return check_launch();
}

sm_status launch_vote_tbl(int enc, int M, const VoteMat* mats, int nmat, int wdt, float lr,
                          hipStream_t s) {
  for (int q0 = 0; q0 < nmat; q0 += kVoteMax) {
    const int n = std::min(kVoteMax, nmat - q0);
    VoteTbl t;
    std::memset(&t, 0, sizeof(t));
    int64_t need = 1;
    double bytes = 0.0, wbytes = 0.0;
    const double sign_bytes = enc == SM_ENC_BITS ? M / 8.0 : (double)M;
    for (int q = 0; q < n; ++q) {
      t.m[q] = mats[q0 + q];
      const int64_t n8 = (t.m[q].count + 7) / 8;
      const int64_t units = enc == SM_ENC_BITS ? (t.m[q].count + 63) / 64 : n8;
      need = std::max<int64_t>(need, (units + kThreads - 1) / kThreads);
      bytes += (double)t.m[q].count * (sign_bytes + 2.0 * dt_size(wdt));
      wbytes += (double)t.m[q].count * dt_size(wdt);
    }
    const bool stream = wbytes > kStreamBytes;
    // about 64 blocks per CU in all: the matrices' sizes differ, and short
    // blocks even out the launch's tail
    const dim3 grid(blocks_per_problem(need, n, 16384), n);
    prof_begin(SM_K_VOTE_UPDATE, bytes, s);
    if (enc == SM_ENC_BITS) {
      SM_DISPATCH_DT(wdt, TW,
          hipLaunchKernelGGL((k_vote_tbl<0, TW>), grid, dim3(kThreads), 0, s, t, M, lr, stream));
    } else {
      SM_DISPATCH_DT(wdt, TW,
          hipLaunchKernelGGL((k_vote_tbl<1, TW>), grid, dim3(kThreads), 0, s, t, M, lr, stream));
    }
    prof_end(s);
    SM_TRY(check_launch());
  }
  return SM_OK;
}

sm_status launch_polar_update(const void* d, int ddt, int nmat, int64_t count, const PtrTbl& w,
                              int wdt, float lr, hipStream_t s) {
  if (nmat <= 0 || count <= 0) return SM_OK;
  const bool vec = (count % 8) == 0;
  const int64_t n8 = (count + 7) / 8;
  dim3 grid(blocks_per_problem((n8 + kThreads - 1) / kThreads, nmat, 4096), nmat);
  const bool stream = (double)nmat * count * dt_size(wdt) > kStreamBytes;
  prof_begin(SM_K_POLAR_UPDATE, (double)nmat * count * (dt_size(ddt) + 2.0 * dt_size(wdt)), s);
  SM_DISPATCH_DT(ddt, TD, SM_DISPATCH_DT(wdt, TW,
      hipLaunchKernelGGL((k_polar_update<TD, TW>), grid, dim3(kThreads), 0, s, (const TD*)d,
                         count, w, lr, vec, stream)));
  prof_end(s);
  return check_launch();
}


sm_status launch_add_identity(const bf16_t* src, int64_t ss, bf16_t* dst, int64_t sq, int r,
                              int batch, float a, bool lower, hipStream_t s) {
  if (batch <= 0 || r <= 0) return SM_OK;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (r % 8 || ss % 8 || sq % 8 || !al(src) || !al(dst)) return SM_ERR_UNSUPPORTED;
  const int64_t n8 = (int64_t)r * r / 8;
  int64_t want = (2048 + batch - 1) / batch;
  const int64_t need = (n8 + kThreads - 1) / kThreads;
  dim3 grid((unsigned)(need < want ? need : want), batch);
  prof_begin(SM_K_MISC, (double)batch * (lower ? lower_tile_entries(r) : (double)r * r) * 4.0,
             s);
  hipLaunchKernelGGL(k_add_identity, grid, dim3(kThreads), 0, s, src, ss, dst, sq, r, a,
                     lower ? 1 : 0);
  prof_end(s);
  return check_launch();
}


sm_status launch_gather_has_cache(const PtrTbl& cs, int per, int nprob, int32_t* hc,
                                  hipStream_t s) {
  if (nprob <= 0) return SM_OK;
  prof_begin(SM_K_MISC, (double)nprob * 12.0, s);
  hipLaunchKernelGGL(k_gather_has_cache, dim3((nprob + 63) / 64), dim3(64), 0, s, cs, per,
                     nprob, hc);
  prof_end(s);
  return check_launch();
}

sm_status launch_any_flags(const FlagSets& fs, int32_t* out, hipStream_t s) {
  if (fs.count <= 0) return SM_ERR_ARG;
  double bytes = 4.0;
  for (int a = 0; a < fs.count; ++a) bytes += 4.0 * fs.n[a];
  prof_begin(SM_K_MISC, bytes, s);
  hipLaunchKernelGGL(k_any_flags, dim3(1), dim3(kThreads), 0, s, fs, out);
  prof_end(s);
  return check_launch();
}

sm_status launch_q_store(const bf16_t* src, int64_t sst, int r, const PtrTbl& q, int per,
                         const int32_t* flags, int batch, hipStream_t s) {
  if (batch <= 0 || r <= 0) return SM_OK;
  const int nb = (r + 63) / 64;
  // read up to the lower-tile entries, write r^2 floats, per refreshed problem
  prof_begin(SM_K_MISC, (double)batch * ((double)r * r * 2.0 + (double)r * r * 4.0), s);
  hipLaunchKernelGGL(k_q_store, dim3(nb * nb, batch), dim3(kThreads), 0, s, src, sst, r, q, per,
                     flags);
  prof_end(s);
  return check_launch();
}

sm_status launch_compact_flags(const int32_t* flags, int n, int32_t* dyn, hipStream_t s) {
  if (n <= 0) return SM_ERR_ARG;
  prof_begin(SM_K_MISC, 8.0 * n + 4.0, s);
  hipLaunchKernelGGL(k_compact_flags, dim3(1), dim3(kThreads), 0, s, flags, n, dyn);
  prof_end(s);
  return check_launch();
}

sm_status launch_q_load(const PtrTbl& q, int per, int r, bf16_t* dst, int64_t dst_stride,
                        const int32_t* flags, int batch, hipStream_t s) {
  if (batch <= 0 || r <= 0) return SM_OK;
  if (r % 8 || dst_stride % 8) return SM_ERR_UNSUPPORTED;
  const int64_t n8 = (int64_t)r * r / 8;
  int64_t want = (2048 + batch - 1) / batch;
  const int64_t need = (n8 + kThreads - 1) / kThreads;
  dim3 grid((unsigned)(need < want ? need : want), batch);
  prof_begin(SM_K_MISC, (double)batch * (double)r * r * 6.0, s);
  hipLaunchKernelGGL(k_q_load, grid, dim3(kThreads), 0, s, q, per, r, dst, dst_stride, flags);
  prof_end(s);
  return check_launch();
}

sm_status launch_cache_decide(const float* resid_partials, int parts, int nprob, int r,
                              const int32_t* hc, const PtrTbl& cs, int per, int mode,
                              float gamma, int64_t t, int32_t* flags, float* err,
                              int32_t* refreshed, const PtrTbl* diag, hipStream_t s) {
  if (nprob <= 0) return SM_OK;
  PtrTbl dt;
  if (diag) dt = *diag; else std::memset(&dt, 0, sizeof(dt));
  prof_begin(SM_K_MISC, (double)nprob * (parts * 4.0 + 24.0), s);
  hipLaunchKernelGGL(k_cache_decide, dim3((nprob + 63) / 64), dim3(64), 0, s, resid_partials,
                     parts, nprob, r, hc, cs, per, mode, gamma, (int32_t)t, flags, err,
                     refreshed, dt, diag != nullptr);
  prof_end(s);
  return check_launch();
}

}  // namespace sm
