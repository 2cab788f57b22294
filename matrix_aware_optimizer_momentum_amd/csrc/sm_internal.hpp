// Internal declarations shared by the HIP translation units of libsm.
// Device helpers, the operand descriptors of the batched MFMA GEMM, and the
// host-side launchers that the C ABI layer (sm_api.hip) drives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/sm.h"

namespace sm {

// ---------------------------------------------------------------- types

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an IEEE float32)

enum Dt : int { F32 = SM_F32, BF16 = SM_BF16 };

__host__ __device__ inline size_t dt_size(int dt) { return dt == BF16 ? 2 : 4; }

// bfloat16 -> float32 is exact: the 16 stored bits are the float's top half.
__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// float32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
// Written out so that it does not depend on which conversion instruction
// the compiler picks.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
    return (bf16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  return (bf16_t)((u + 0x7FFFu + lsb) >> 16);
}

// Runs __VA_ARGS__ with T the element type of dt (bf16_t or float).
#define SM_DISPATCH_DT(dt, T, ...)                   \
  do {                                               \
    if ((dt) == BF16) {                              \
      typedef bf16_t T;                              \
      __VA_ARGS__;                                   \
    } else {                                         \
      typedef float T;                               \
      __VA_ARGS__;                                   \
    }                                                \
  } while (0)

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store(bf16_t* p, float v) { *p = f2bf(v); }
};

// Eight consecutive elements of a 16-byte-aligned array, as float32.
template <typename T> __device__ __forceinline__ void load8(const T* p, float* v);
template <> __device__ __forceinline__ void load8<float>(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
  uint4 a = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float* v);
template <> __device__ __forceinline__ void store8<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// ---------------------------------------------------------------- pointer tables

// Up to kTbl matrices per launch; problem b of a launch is worker (b % per)
// of matrix (b / per), at byte offset (b % per) * worker_stride_bytes.
constexpr int kTbl = 64;
struct PtrTbl {
  const char* p[kTbl];
};

__device__ __forceinline__ const char* tbl_addr(const PtrTbl& t, int b, int per,
                                                int64_t worker_stride_bytes) {
  return t.p[b / per] + (int64_t)(b % per) * worker_stride_bytes;
}

// ---------------------------------------------------------------- launch accounting

// Brackets every launch with events while profiling is enabled.
// work: flops (GEMMs) or bytes (streaming kernels); bytes: the launch's
// algorithmic HBM bytes (each operand read once, each output written once);
// negative means "same as work".
void prof_begin(int kind, double work, hipStream_t s, double bytes = -1.0);
void prof_end(hipStream_t s);
// Device address of a kind's {executed flops, executed bytes} accumulator
// while profiling is enabled, else null.  Launches whose problems are
// predicated on a device flag record no work on the host; their kernels add
// the work of the problems that ran here.
double* prof_exec_slot(int kind);

// Records a failed HIP call and maps it to SM_ERR_HIP.
sm_status hip_fail(hipError_t e);
sm_status check_launch();

// Returns the status of expr from the calling function unless it is SM_OK.
#define SM_TRY(expr)                    \
  do {                                  \
    sm_status _st = (expr);             \
    if (_st != SM_OK) return _st;       \
  } while (0)


// ---------------------------------------------------------------- streaming kernels

// Partial sums per problem of every sum-of-squares producer: one per block,
// norm_parts(count) blocks (up to kNormParts, the stride of the partials
// array), so that a launch has enough blocks to keep HBM busy.
constexpr int kNormParts = 512;
constexpr int kNormChunk = 2048;   // entries per block iteration
__host__ __device__ inline int norm_parts(int64_t count) {
  const int64_t n = (count + kNormChunk - 1) / kNormChunk;
  return (int)(n < 1 ? 1 : (n > kNormParts ? kNormParts : n));
}

// Single EMA  M <- beta*M + (1-beta)*G over a table of matrices of any
// shapes (the momentum and the gradients of matrix q: `per` workers, count
// entries apart), kEmaMax per launch.  Writes M, the NS input copy x
// ([per][count] in the momentum type, may be null) and the sum-of-squares
// partials of the stored x values ([per][kNormParts], norm_parts(count) of
// them); with `finalize`, also scale = 1 / (||x|| + eps) per problem, as
// launch_scale_finalize.
struct EmaMat {
  void* mom;
  const void* grad;
  void* x;            // NS input copy [per][count] in the momentum type, or null
  float* partials;
  float* scale;
  int64_t count;
};
constexpr int kEmaMax = 64;
struct EmaTbl {
  EmaMat m[kEmaMax];
};
sm_status launch_ema_tbl(const EmaMat* mats, int nmat, int per, int mdt, int gdt, float beta,
                         bool finalize, float eps, hipStream_t s);

// LionMuon fused kernel.  ghat = beta1*M + (1-beta1)*G, M <- beta2*M +
// (1-beta2)*G.  On a Lion step the signs of ghat (decided in float32) are
// packed to bits[nprob][words] (bits != null) or written as int8 signs to
// s8[nprob][count] (s8 != null); otherwise ghat is stored to x in xdt with
// sum-of-squares partials (Muon step input).
sm_status launch_lion(const PtrTbl& mom, const PtrTbl& grad, int per, int nprob, int64_t count,
                      int mdt, int gdt, float beta1, float beta2, void* x, int xdt,
                      float* partials, uint64_t* bits, int64_t words, int8_t* s8,
                      hipStream_t s);

// Sum-of-squares partials of nprob contiguous problems.
sm_status launch_sumsq(const void* x, int dt, int nprob, int64_t count, float* partials,
                       hipStream_t s);

// scale[b] = 1 / (sqrt(sum_i partials[b][i]) + eps) over the norm_parts(count)
// partials of problems of `count` elements
sm_status launch_scale_finalize(const float* partials, int nprob, int64_t count, float eps,
                                float* scale, hipStream_t s);

// Sign + 1-bit pack of nprob contiguous problems of `count` elements into
// bits (problem b at bits + b*words).
sm_status launch_sign_pack(const void* x, int dt, int nprob, int64_t count, uint64_t* bits,
                           int64_t words, hipStream_t s);

// int8 signs (-1 iff x < 0, else +1) of nprob contiguous problems of `count`
// elements into s8 (problem b at s8 + b*count).
sm_status launch_sign_int8(const void* x, int dt, int nprob, int64_t count, int8_t* s8,
                           hipStream_t s);

// Vote of `nmat` matrices from packed bits (enc SM_ENC_BITS; strides in
// uint64 words) or int8 signs (SM_ENC_INT8; strides in bytes): matrix j reads
// signs + j*mat_stride, worker k at + k*stride.  update: W <- rnd(W - lr*V)
// in place at w.p[j] (vote_out optional); otherwise V in {-1, 0, +1} is
// written as wdt to w.p[j].
sm_status launch_vote(int enc, const void* signs, int M, int64_t stride, int64_t mat_stride,
                      int nmat, int64_t count, const PtrTbl& w, int wdt, float lr,
                      int8_t* vote_out, bool update, hipStream_t s);

// Power-method spectral norm of E_b = A_b - B_b (b may be null), batch
// problems of m x n (k_power.hip); ws of spectral_norm_ws_bytes().
int spectral_row_chunks(int batch, int m, int n);
size_t spectral_norm_ws_bytes(int batch, int m, int n);
sm_status launch_spectral_norm(const void* a, const void* b, int dt, int batch, int m, int n,
                               const float* v0, int iters, float* out, void* ws, hipStream_t s);

// One matrix of a multi-shape vote + update: its first worker's signs
// (packed words or int8), the workers `stride` words / bytes apart, its
// entry count and weights.
struct VoteMat {
  const void* signs;
  void* w;
  int64_t stride, count;
};
constexpr int kVoteMax = 96;   // matrices per launch (the table rides in the arguments)
struct VoteTbl {
  VoteMat m[kVoteMax];
};
// Vote + update (W <- rnd(fp32(W) - fp32(lr) * v)) of nmat matrices of any
// shapes, kVoteMax per launch.
sm_status launch_vote_tbl(int enc, int M, const VoteMat* mats, int nmat, int wdt, float lr,
                          hipStream_t s);

// W <- rnd(fp32(W) - fp32(lr*D)) for nmat matrices, D contiguous [nmat][count].
sm_status launch_polar_update(const void* d, int ddt, int nmat, int64_t count, const PtrTbl& w,
                              int wdt, float lr, hipStream_t s);

// q_b = s_b + a I for a batch of r x r bf16 matrices (float32 sum, bf16
// rounding); needs r % 8 == 0, strides % 8 == 0 and 16-byte aligned bases.
// lower: only the 256 x 256 tiles on and below the diagonal (matrices kept
// as their lower triangle of tiles).
sm_status launch_add_identity(const bf16_t* src, int64_t ss, bf16_t* dst, int64_t sq, int r,
                              int batch, float a, bool lower, hipStream_t s);

// Entries of an n x n matrix kept as its 256 x 256 tiles on and below the
// diagonal (row block i holds rows x min(256 (i + 1), n) entries).
inline double lower_tile_entries(int n) {
  double e = 0.0;
  for (int r0 = 0; r0 < n; r0 += 256)
    e += (double)(n - r0 < 256 ? n - r0 : 256) * (r0 + 256 < n ? r0 + 256 : n);
  return e;
}

// has_cache flags of nprob problems: hc[b] = cache_state(b)[0], where problem
// b's {has_cache, a_t} pair is at tbl_addr(cs, b, per, 8).
sm_status launch_gather_has_cache(const PtrTbl& cs, int per, int nprob, int32_t* hc,
                                  hipStream_t s);

// CacheMuon accept/refresh decision per problem (see sm_gram_ns_cached):
// err from the residual partials, flags[b] = 1 to refresh, outputs err /
// refreshed / diag (each optional; problem b's {err, refreshed} float pair
// at tbl_addr(*diag, b, per, 8)), and {1, t} written to cache_state on a
// refresh.
sm_status launch_cache_decide(const float* resid_partials, int parts, int nprob, int r,
                              const int32_t* hc, const PtrTbl& cs, int per, int mode,
                              float gamma, int64_t t, int32_t* flags, float* err,
                              int32_t* refreshed, const PtrTbl* diag, hipStream_t s);

// Flag arrays of up to kTbl sets of problems (f[a] holds n[a] int32 flags).
struct FlagSets {
  const int32_t* f[kTbl];
  int n[kTbl];
  int count;
};
// *out = 1 iff some flag is 1, else 0 (device int32).
sm_status launch_any_flags(const FlagSets& fs, int32_t* out, hipStream_t s);

// Writes the cache of each problem b with flags[b] == 1: the r x r bf16
// matrix src + b*sst, stored as its 256 x 256 tiles on and below the
// diagonal, as a whole float32 matrix at tbl_addr(q, b, per, 4 r^2).
sm_status launch_q_store(const bf16_t* src, int64_t sst, int r, const PtrTbl& q, int per,
                         const int32_t* flags, int batch, hipStream_t s);
// The cache of each problem b with flags[b] == 1 (float32 r x r at
// tbl_addr(q, b, per, 4 r^2)) rounded to bf16 into dst + b*dst_stride;
// needs r % 8 == 0.
sm_status launch_q_load(const PtrTbl& q, int per, int r, bf16_t* dst, int64_t dst_stride,
                        const int32_t* flags, int batch, hipStream_t s);

// ---------------------------------------------------------------- batched MFMA GEMM

enum Layout : int {
  KC = 0,  // operand row i, column k at base + i*ld + k (k contiguous)
  RC = 1   // at base + k*ld + i (row index contiguous)
};

struct GemmOperand {
  const void* p;
  int64_t ld;      // elements
  int64_t stride;  // elements between problems
  int dt;          // F32 / BF16 in memory
  int layout;      // KC / RC
  int tbl;         // 1: problem b lives at tbl.p[b / tbl_per] + (b % tbl_per) * stride
};

// C[b] (M x N) = alpha_b * A[b] B[b] + beta_b * Cin[b] + diag * I
//   A[b] is M x K, B[b] is K x N (B's KC layout stores B^T row-major).
//   alpha_b = alpha * scale[b]^alpha_pow, beta_b = beta * scale[b]^beta_pow.
// Cin has C's dtype.  Optional outputs: C (c_dt), C2 (float32) =
// c2_diag*I + c2_scale*value,
// resid partials ([batch][tiles]) = sum over the tile of (value - I)^2,
// bits ([batch][bits_stride] words): the packed signs of C as stored (bit e
// of word w set iff entry 64 w + e of the row-major M x N result is
// negative; needs N % 64 == 0).
// Problems with pred && pred[b*pred_stride] != pred_val are skipped.
// sym: the result is symmetric (A B with A = B^T, or commuting symmetric
// factors, and a symmetric Cin): only tiles on and below the diagonal are
// computed, each off-diagonal one stored a second time, transposed (C only;
// no C2, resid or bits).
// Operands / outputs flagged `tbl` address problem b through the launch's
// pointer table: entry tbl_off + b / tbl_per, plus (b % tbl_per) * stride.
struct GemmCore {
  GemmOperand a, b;
  const void* cin; int64_t ldcin, scin; int cin_tbl;
  void* c; int64_t ldc, sc; int c_dt; int c_tbl;
  float* c2; int64_t ldc2, sc2; int c2_tbl;
  float* resid;
  uint64_t* bits; int64_t bits_stride;
  const float* scale;
  const int32_t* pred; int pred_stride; int32_t pred_val;
  int M, N, K, batch;
  float alpha; int alpha_pow;
  float beta; int beta_pow;
  float diag;
  float c2_diag, c2_scale;
  int sym;
  int tbl_per, tbl_off;
  // Kernel-time accounting of predicated launches (set by the launcher):
  // each problem that runs adds prof_flops / prof_bytes to prof_exec[0 / 1].
  double* prof_exec; double prof_flops, prof_bytes;
};
// One product set as the host builds it: the per-matrix base pointers
// (CacheMuon's Q caches, Sign-Muon's momenta) ride along in tbl; the launcher
// packs the tables of the sets it groups into one launch table.
struct GemmArgs : GemmCore {
  PtrTbl tbl;
};

// Tiles per problem that the GEMM launch uses for (M, N) (resid partials).
int gemm_tiles(int mfma_dt, int M, int N);

// Launch with MFMA operand type mfma_dt (BF16 -> bf16 MFMA, F32 -> fp32 MFMA).
sm_status launch_gemm(const GemmArgs& g, int mfma_dt, int kind, hipStream_t s);
// Launches the product sets gs (one kind, one MFMA type) in as few launches
// as their operand types / layouts, the table capacity and the group limit
// allow; within a launch the sets run in order of decreasing K.
sm_status launch_gemm_groups(std::vector<GemmArgs>& gs, int mfma_dt, int kind, hipStream_t s);

// ---------------------------------------------------------------- grouped NS GEMM

// One group of batched problems for the persistent NS GEMM:
// C[b] = alpha_b * A[b] B[b]^T (+ identity term), A: M x K, B: N x K in the
// operand sense, bf16, C (M x N) row-major bf16.  An operand with *_kr set is
// stored k-major (K x rows, row-major, leading dimension ld over rows).
// sym: C is symmetric (A == B, or A and B are commuting symmetric matrices,
// as all polynomials in one Gram matrix are), same layout on both sides:
// only tm >= tn tiles are computed, off-diagonal ones are also stored
// transposed.  ident: 1 adds (a I) times the B part (needs K == M), 2 adds
// the A part times (a I) (needs K == N); a = hi + lo as bf16 bit patterns
// (ident_terms 1: hi only).  alpha_b = alpha * scale[b]^alpha_pow (scale may
// be null).  One launch takes up to kNsgMaxGroups groups that use at most
// kNsgMaxTables distinct pointer tables.
constexpr int kNsgMaxGroups = 8;
constexpr int kNsgMaxTables = 4;
struct NsgGroup {
  const bf16_t* a; int64_t lda, sa; int a_kr;
  const bf16_t* b; int64_t ldb, sb; int b_kr;
  // Optional per-matrix addressing of the operands flagged a_tbl / b_tbl
  // (then a / b are unused): problem p is worker p % tbl_per of matrix
  // p / tbl_per, at tbl->p[p / tbl_per] + (p % tbl_per) * s{a,b} elements.
  const PtrTbl* tbl; int tbl_per; int a_tbl, b_tbl;
  bf16_t* c; int64_t ldc, sc;
  const float* scale; int alpha_pow; float alpha;
  int M, N, K, batch;
  int sym;
  int ident, ident_terms;
  uint32_t ident_hi, ident_lo;
  // Lower-triangle storage of symmetric square matrices (Gram-form chain):
  // a_low / b_low mark an operand (KC, K x K) whose 256 x 256 tiles above the
  // diagonal were never written; the kernel reads a panel's entries past its
  // diagonal block from the mirror tiles, transposed.  c_low (symmetric
  // products) stores the tiles on and below the diagonal only.
  int a_low, b_low, c_low;
  // Apply only: instead of C, write the 1-bit signs of its bf16 values
  // (bit = 1 <=> negative, bit j of word w <=> row-major entry 64 w + j) to
  // bits + problem * bits_stride words; needs N % 64 == 0.  With bits_s8
  // the signs are int8 instead (-1 iff negative, else +1; one byte per
  // row-major entry, row pitch N bytes) at the same address, bits_stride
  // still counted in 8-byte words; then bits is 16-byte aligned and
  // bits_stride even.
  uint64_t* bits; int64_t bits_stride; int bits_s8;
  // Optional per-problem store predicate (device int32 per problem): a
  // problem whose flag is not 1 computes its tiles but stores nothing.
  const int32_t* pred;
  // Probe (kind SM_K_PROBE, symmetric, no identity): instead of C, each
  // wave writes the residual partial sum over its 128 x 128 part of the
  // tile of (alpha * value - [row == col])^2 (doubled below the diagonal,
  // whose mirror is not computed) to resid + problem * 4 * lower tiles +
  // 4 * (tm (tm + 1) / 2 + tn) + wave.
  float* resid;
  // Optional device problem list (int32 [1 + batch]: the count, then the
  // indices of the problems to run); the other problems are neither
  // computed nor stored.  In a launch either every group has one or none.
  const int32_t* dyn;
};

// Residual partials per problem that a probe launch writes (4 per lower tile).
inline int ns_probe_parts(int r) {
  const int t = (r + 255) / 256;
  return 4 * (t * (t + 1) / 2);
}

bool gemm_ns_supported(const NsgGroup& g);
// Splits a into bf16 terms hi (+ lo); returns the number of terms whose sum
// is exactly a (1 or 2), or 0 if two do not suffice.
int ns_ident_split(float a, uint32_t* hi_bits, uint32_t* lo_bits);
// Kinds SM_K_GEMM_GRAM and SM_K_GEMM_RR (which differ only in the kernel-time
// accounting) run the symmetric-product kernel: symmetric groups, plus tall
// applies and wide ones with a one-term identity (no signs) riding along; kind
// SM_K_GEMM_APPLY runs the apply kernel (applies only).  Returns
// SM_ERR_UNSUPPORTED for other groups or more than kNsgMaxTables distinct
// tables.
// gate (optional device int32): when it holds 0 at launch time the whole
// launch does nothing (the fresh solve of a CacheMuon step that refreshes
// no problem).  Groups with device problem lists (NsgGroup::dyn) need
// dyn_tiles, a device int32 [kNsgMaxGroups + 1] scratch that a small kernel
// ahead of the launch fills with each group's first tile and the total (so
// that groups of different shapes and lists share a launch); pointer tables
// are addressed by the listed problem.
sm_status launch_gemm_ns(const NsgGroup* groups, int ngroups, int kind, hipStream_t s,
                         const int32_t* gate = nullptr, int32_t* dyn_tiles = nullptr);
// dyn[0] = the number of problems b < n with flags[b] == 1, dyn[1 ..] = those
// b in increasing order (one workgroup).
sm_status launch_compact_flags(const int32_t* flags, int n, int32_t* dyn, hipStream_t s);
// Distinct pointer tables among the groups.
int ns_group_tables(const NsgGroup* groups, int ngroups);
// Workgroups one NS GEMM launch runs at most (one per CU of the device).
int gemm_ns_cus();

}  // namespace sm
