// Newton-Schulz GEMM for bf16 operands with both operands k-contiguous
// ("NT": C = A B^T with A M x K and B N x K, both row-major).
//
// The direct Newton-Schulz step only ever needs this form when the iterate
// is kept in both orientations (X and X^T): the Gram product X X^T reads X
// twice, and the apply product B X reads B and X^T.  The apply epilogue
// writes the next iterate in both orientations.
//
// Tile 256 x 256, 256 threads = 4 waves (2 x 2), each wave 128 x 128 as 4 x 4
// blocks of v_mfma_f32_32x32x16_bf16 (256 float32 accumulators per lane).
// Operands move HBM/L2 -> LDS with gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at the instruction's LDS
// base + 16 l), without passing through registers, into a ring of four 32 KB
// k-stages (k = 32 each).  Step k multiplies stage k, issues the loads of
// stage k + 3 into the buffer stage k - 1 left, and reads the fragments of
// its own second k16 slice and of the first slice of stage k + 1 while its
// MFMAs run (one memory instruction after each MFMA).  Before the step's
// barrier each wave waits for its loads of stage k + 2 only, so the loads of
// a stage have about two steps of MFMA work to arrive.  The barrier is a bare
// s_barrier between compiler memory fences: the loads still in flight target
// buffers nobody reads until a later barrier.
//
// LDS stage layout: A rows then B rows, 64 bytes per row, the four 16-byte k
// chunks of row R stored at chunk position c ^ ((R >> 2) & 3).  Sixteen
// consecutive rows read at one chunk then hit 16 distinct 4-bank groups, so
// the 16-byte fragment reads (and the 16-byte stores) are conflict-free.
//
// Identity fold: the apply product X' = a X + B X needs a X.  Instead of
// reading X again in the epilogue, the k-stages that cover the output's own
// rows add (a I) X (wide) or X (a I) (tall) with one extra MFMA per 32 x 32
// block whose rows meet the stage's k range; with a exact in bf16 (1.5) the
// term is added exactly in float32, as an epilogue add would.
//
// Epilogue: value = alpha_b * acc (+ beta_b * Cin on the general path),
// converted with v_cvt_pk_bf16_f32.  Row-major C: a two-round quad DPP
// shuffle turns each lane's 4 rows x 1 column into 1 row x 4 columns, stored
// as 8-byte chunks.  Transposed outputs (C^T, or the mirror tile of a
// symmetric product) go through a swizzled 32 KB LDS region per wave as
// 16-byte row-contiguous stores.  A symmetric product (A == B) computes only
// tiles with tm >= tn.
#include "sm_internal.hpp"

namespace sm {
namespace nt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 32, NT = 256;
constexpr int STG = (BM + BN) * BK;     // bf16 elements per stage (32 KB)
constexpr int BOFF = BM * BK;           // B rows start here within a stage

struct NtArgs {
  const bf16_t* a; int64_t lda, sa;
  const bf16_t* b; int64_t ldb, sb;
  const bf16_t* cin; int64_t ldcin, scin;
  bf16_t* c; int64_t ldc, sc;
  bf16_t* ct; int64_t ldct, sct;
  const float* scale; int alpha_pow, beta_pow;
  float alpha, beta;
  int M, N, K, batch;
  int sym;
  int tm_fast;
  int ident;          // 0 none, 1: acc += (a I) B-part (wide), 2: acc += A-part (a I) (tall)
  uint32_t ident_bits;  // bf16 bits of a
  int tiles_m, tiles_n, tiles_per_prob;
  int xcd_chunk;      // blocks per XCD after remapping (0: no remap)
};

// Direct-to-LDS loads of one k-stage: each wave fills 4 row groups of A and
// 4 of B, 16 rows x 64 bytes (1 KB) per instruction.  Lane l of a group
// covers row l / 4 and fetches the global k chunk that belongs at position
// l % 4 of that row under the stage swizzle.  Rows past the matrix are
// clamped to its last row and stages past K to the last stage: an operand row
// outside the matrix only feeds accumulator rows / columns that the epilogue
// never stores, and stages past K are prefetched but never multiplied.  The
// loads are therefore unconditional.  Offsets are 32-bit byte offsets from
// the problem's base (the launcher checks that they fit).
struct DmaOffs {
  uint32_t a[4], b[4];
};

__device__ __forceinline__ DmaOffs dma_offsets(int64_t lda, int m0, int M, int64_t ldb, int n0,
                                               int N) {
  DmaOffs o;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane >> 2;
  const int kc = 8 * ((lane & 3) ^ ((lane >> 4) & 3));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grp = wave * 4 + i;
    const int ra = m0 + grp * 16 + rl, rb = n0 + grp * 16 + rl;
    o.a[i] = (uint32_t)(2 * ((ra < M ? ra : M - 1) * lda + kc));
    o.b[i] = (uint32_t)(2 * ((rb < N ? rb : N - 1) * ldb + kc));
  }
  return o;
}

// Byte offset of k-stage k0: stages past K are clamped to the last one.
__device__ __forceinline__ uint32_t stage_koff(int k0, int K) {
  return 2u * (uint32_t)(k0 < K ? k0 : K - BK);
}

// Load q (0..3: A groups, 4..7: B groups) of this wave's share of a stage.
__device__ __forceinline__ void dma_load(bf16_t* S, const char* A, const char* B,
                                         const DmaOffs& o, uint32_t koff, int q) {
  const int grp = (threadIdx.x >> 6) * 4 + (q & 3);
  if (q < 4)
    __builtin_amdgcn_global_load_lds(A + (o.a[q] + koff), S + grp * 16 * BK, 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(B + (o.b[q - 4] + koff), S + BOFF + grp * 16 * BK, 16, 0, 0);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt low
// bits 3:0 and high bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence (no wait for outstanding direct-
// to-LDS loads); the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte fragment of row R, k chunk c (0..3) of a stage operand.
__device__ __forceinline__ bf16x8 frag(const bf16_t* S, int R, int c) {
  return *reinterpret_cast<const bf16x8*>(S + R * BK + 8 * (c ^ ((R >> 2) & 3)));
}

// Identity fragment for the k16 slice `half` (0/1) of the 32-index block
// that a stage of the identity group covers: lane l supplies index l % 32 and
// k = 16 half + 8 (l / 32) + e; the element is a where they agree.
__device__ __forceinline__ bf16x8 ident_frag(int half, uint32_t abits) {
  const int lane = threadIdx.x & 63;
  const int e = (lane & 31) - 16 * half - 8 * (lane >> 5);
  uint32_t w0 = 0u, w1 = 0u, w2 = 0u, w3 = 0u;
  const uint32_t v = abits << (16 * (e & 1));
  if (e >= 0 && e < 8) {
    const int d = e >> 1;
    w0 = d == 0 ? v : 0u; w1 = d == 1 ? v : 0u; w2 = d == 2 ? v : 0u; w3 = d == 3 ? v : 0u;
  }
  const uint4 u = make_uint4(w0, w1, w2, w3);
  return __builtin_bit_cast(bf16x8, u);
}

// The fragments of one k16 slice of this wave's 128 x 128 sub-tile.
struct Frags {
  bf16x8 a[4], b[4];
};

__device__ __forceinline__ void read_frags(Frags& f, const bf16_t* S, int wm, int wn, int s) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = frag(S, wm * 128 + i * 32 + lr, 2 * s + lk);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = frag(S + BOFF, wn * 128 + j * 32 + lr, 2 * s + lk);
}

// One step of the main loop (stage k): the two k16 slices' MFMAs, each
// followed by at most one memory instruction, in this order:
//   slice 0 (f0): reads of this stage's slice-1 fragments into f1, then the
//                 direct-to-LDS loads of stage k + 3 into buffer ld3;
//   slice 1 (f1): reads of stage k + 1's slice-0 fragments into f0.
// sched_barrier keeps the compiler from regrouping them (hoisting the reads
// would need a second set of fragment registers).
template <int IDM, int IB>
__device__ __forceinline__ void nt_step(f32x16 (&acc)[4][4], Frags& f0, Frags& f1,
                                        const bf16_t* cur, const bf16_t* nxt, bf16_t* ld3,
                                        const char* A, const char* B, const DmaOffs& o,
                                        uint32_t koff3, int wm, int wn, bf16x8 id0,
                                        bf16x8 id1) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.a[i], f0.b[j], acc[i][j], 0, 0, 0);
    if (q < 4)
      f1.a[q] = frag(cur, wm * 128 + q * 32 + lr, 2 + lk);
    else if (q < 8)
      f1.b[q - 4] = frag(cur + BOFF, wn * 128 + (q - 4) * 32 + lr, 2 + lk);
    else
      dma_load(ld3, A, B, o, koff3, q - 8);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (IDM == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[IB][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id0, f0.b[j], acc[IB][j], 0, 0, 0);
  } else if constexpr (IDM == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i][IB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0.a[i], id0, acc[i][IB], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.a[i], f1.b[j], acc[i][j], 0, 0, 0);
    if (q < 4)
      f0.a[q] = frag(nxt, wm * 128 + q * 32 + lr, lk);
    else if (q < 8)
      f0.b[q - 4] = frag(nxt + BOFF, wn * 128 + (q - 4) * 32 + lr, lk);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (IDM == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[IB][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(id1, f1.b[j], acc[IB][j], 0, 0, 0);
  } else if constexpr (IDM == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i][IB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1.a[i], id1, acc[i][IB], 0, 0, 0);
  }
}

// ---- epilogue staging: a wave's 128 x 128 bf16 tile in its own 32 KB stage
// array, row-major with 256-byte rows and 16-byte chunk c of row r stored at
// position c ^ (r & 15) (conflict-free for the access patterns below).
__device__ __forceinline__ int sw(int r, int c) {   // element offset of (r, c)
  return r * 128 + 8 * ((c >> 3) ^ (r & 15)) + (c & 7);
}

// Global 128 x 128 sub-matrix (rows r0.., cols c0.., clipped) -> staging.
__device__ __forceinline__ void tile_to_lds(bf16_t* L, const bf16_t* __restrict__ src,
                                            int64_t ld, int r0, int c0, int rows, int cols) {
  const int lane = threadIdx.x & 63, sub = lane & 15, rsel = lane >> 4;
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const int d = it * 4 + rsel, r = r0 + d, c = c0 + sub * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows) {
      const bf16_t* p = src + (int64_t)r * ld + c;
      if (c + 8 <= cols) {
        v = *reinterpret_cast<const uint4*>(p);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < cols) w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    *reinterpret_cast<uint4*>(L + sw(d, sub * 8)) = v;
  }
}

// Staging -> global 128 x 128 sub-matrix at rows r0.., cols c0.. (clipped).
__device__ __forceinline__ void lds_to_tile(const bf16_t* L, bf16_t* __restrict__ dst,
                                            int64_t ld, int r0, int c0, int rows, int cols) {
  const int lane = threadIdx.x & 63, sub = lane & 15, rsel = lane >> 4;
  const bool interior = r0 + 128 <= rows && c0 + 128 <= cols;
#pragma unroll 8
  for (int it = 0; it < 32; ++it) {
    const int d = it * 4 + rsel, r = r0 + d, c = c0 + sub * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(L + sw(d, sub * 8));
    bf16_t* p = dst + (int64_t)r * ld + c;
    if (interior) {
      *reinterpret_cast<uint4*>(p) = v;
    } else if (r < rows) {
      if (c + 8 <= cols) {
        *reinterpret_cast<uint4*>(p) = v;
      } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < cols) p[e] = (bf16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t cvt2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ROLE tags the kernel symbol by its use (Gram / apply / r x r) for profiles;
// IDM selects the identity fold (0 none, 1 wide apply, 2 tall apply).
template <int ROLE, int IDM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_nt(NtArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t S0[STG];
  __shared__ __attribute__((aligned(16))) bf16_t S1[STG];
  __shared__ __attribute__((aligned(16))) bf16_t S2[STG];
  __shared__ __attribute__((aligned(16))) bf16_t S3[STG];
  // XCD-aware remap: consecutive workgroups land on different XCDs; give each
  // XCD a contiguous range of tiles so tiles of one problem share its L2.
  int bid = blockIdx.x;
  if (g.xcd_chunk > 0) bid = (bid & 7) * g.xcd_chunk + (bid >> 3);
  const int prob = bid / g.tiles_per_prob;
  if (prob >= g.batch) return;
  int t = bid - prob * g.tiles_per_prob;
  int tm, tn;
  if (g.sym) {  // lower triangle, row-major: t = tm (tm + 1) / 2 + tn
    tm = (int)((sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
    while ((tm + 1) * (tm + 2) / 2 <= t) ++tm;
    while (tm * (tm + 1) / 2 > t) --tm;
    tn = t - tm * (tm + 1) / 2;
  } else if (g.tm_fast) {  // consecutive tiles share the B-operand row block
    tn = t / g.tiles_m;
    tm = t - tn * g.tiles_m;
  } else {
    tm = t / g.tiles_n;
    tn = t - tm * g.tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const int wr0 = m0 + wm * 128, wc0 = n0 + wn * 128;   // wave sub-tile origin
  const bf16_t* A = g.a + (int64_t)prob * g.sa;
  const bf16_t* B = g.b + (int64_t)prob * g.sb;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Stage j sits in LDS buffer j % 4.  Step k: loads of stage k + 3 go into
  // buffer (k + 3) % 4, whose stage k - 1 was last read in step k - 1; at
  // the end of step k the wave waits for its loads of stage k + 2 (read from
  // step k + 1 on), leaving the 8 loads of stage k + 3 in flight.
  const int nk = g.K / BK;   // a multiple of 4 (the launcher requires K % 128 == 0)
  const DmaOffs dof = dma_offsets(g.lda, m0, g.M, g.ldb, n0, g.N);
  bf16x8 id0, id1;
  if constexpr (IDM != 0) {
    id0 = ident_frag(0, g.ident_bits);
    id1 = ident_frag(1, g.ident_bits);
  } else {
    id0 = id1 = bf16x8{};
  }
  const char* Ab = reinterpret_cast<const char*>(A);
  const char* Bb = reinterpret_cast<const char*>(B);
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_load(S0, Ab, Bb, dof, stage_koff(0, g.K), q);
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_load(S1, Ab, Bb, dof, stage_koff(BK, g.K), q);
#pragma unroll
  for (int q = 0; q < 8; ++q) dma_load(S2, Ab, Bb, dof, stage_koff(2 * BK, g.K), q);
  wait_vm<8>();            // stages 0 and 1 of this wave
  barrier_nofence();
  Frags f0, f1;
  read_frags(f0, S0, wm, wn, 0);
#define SM_NT_STEP(KOFF, CUR, NXT, L3, IDM)                                              \
  {                                                                                    \
    nt_step<IDM, KOFF>(acc, f0, f1, CUR, NXT, L3, Ab, Bb, dof,                         \
                       stage_koff((kt + (KOFF) + 3) * BK, g.K), wm, wn, id0, id1);     \
    wait_vm<8>();                                                                      \
    barrier_nofence();                                                                 \
  }
#define SM_NT_GROUP(IDM)               \
  SM_NT_STEP(0, S0, S1, S3, IDM)       \
  SM_NT_STEP(1, S1, S2, S0, IDM)       \
  SM_NT_STEP(2, S2, S3, S1, IDM)       \
  SM_NT_STEP(3, S3, S0, S2, IDM)
  // With the identity fold, the one group of four stages whose k range
  // equals this wave's 128 output rows (wide) or columns (tall) adds a I:
  // step s of that group covers block s.  The loop is peeled around that
  // group so the accumulators follow a single code path; every wave still
  // runs nk barriers.
  int kt = 0;
  if constexpr (IDM != 0) {
    const int id_kt = (IDM == 1 ? wr0 : wc0) / BK;   // a multiple of 4
    for (; kt < id_kt && kt < nk; kt += 4) {
      SM_NT_GROUP(0)
    }
    if (kt < nk) {
      SM_NT_GROUP(IDM)
      kt += 4;
    }
  }
  for (; kt < nk; kt += 4) {
    SM_NT_GROUP(0)
  }
#undef SM_NT_GROUP
#undef SM_NT_STEP
  // the prefetches past the last stage must land before the buffers are reused
  wait_vm<0>();
  __syncthreads();

  // ---------------- epilogue (the stage buffers are free after the last barrier)
  float alpha = g.alpha, beta = g.beta;
  if (g.scale) {
    const float sc = g.scale[prob];
    for (int p = 0; p < g.alpha_pow; ++p) alpha *= sc;
    for (int p = 0; p < g.beta_pow; ++p) beta *= sc;
  }
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lq = (lane >> 5) * 4;
  bf16_t* L = wave == 0 ? S0 : wave == 1 ? S1 : wave == 2 ? S2 : S3;
  // pk[i][j][q]: bf16 values of rows i*32 + q*8 + lq + {0,1} (.x) and
  // {2,3} (.y) of column j*32 + lr (wave sub-tile coordinates).
  uint2 pk[4][4][4];
  if (g.cin) {
    tile_to_lds(L, g.cin + (int64_t)prob * g.scin, g.ldcin, wr0, wc0, g.M, g.N);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = alpha * acc[i][j][q * 4 + e] +
                   beta * bf2f(L[sw(i * 32 + q * 8 + lq + e, j * 32 + lr)]);
          pk[i][j][q] = make_uint2(cvt2(v[0], v[1]), cvt2(v[2], v[3]));
        }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pk[i][j][q] = make_uint2(cvt2(alpha * acc[i][j][q * 4 + 0], alpha * acc[i][j][q * 4 + 1]),
                                   cvt2(alpha * acc[i][j][q * 4 + 2], alpha * acc[i][j][q * 4 + 3]));
  }
  bf16_t* C = g.c + (int64_t)prob * g.sc;
  const bool mirror = g.sym && tm != tn;     // uniform over the block
  if (g.ct || mirror) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)     // transposed: row = source col
          *reinterpret_cast<uint2*>(L + sw(j * 32 + lr, i * 32 + q * 8 + lq)) = pk[i][j][q];
    __syncthreads();
    if (g.ct) lds_to_tile(L, g.ct + (int64_t)prob * g.sct, g.ldct, wc0, wr0, g.N, g.M);
    if (mirror) lds_to_tile(L, C, g.ldc, wc0, wr0, g.N, g.M);
  }
  // Row-major C: quad shuffles give each lane 1 row x 4 consecutive columns.
  const int cm = lane & 3;
  const int rsel = ((cm & 1) << 1) | (cm >> 1);     // which of the 4 rows this lane ends with
  const int colq = (lr & ~3);
  const bool interior = wr0 + 128 <= g.M && wc0 + 128 <= g.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t v0 = pk[i][j][q].x, v1 = pk[i][j][q].y;   // rows (0,1), (2,3)
        const uint32_t recv = dpp_xor1((cm & 1) ? v0 : v1);
        const uint32_t mine = (cm & 1) ? v1 : v0;
        const uint32_t lo = (cm & 1) ? recv : mine;              // lower column
        const uint32_t hi = (cm & 1) ? mine : recv;
        const uint32_t ra = (lo & 0xFFFFu) | (hi << 16);          // first row, 2 columns
        const uint32_t rb = (lo >> 16) | (hi & 0xFFFF0000u);      // second row, 2 columns
        const uint32_t r2 = dpp_xor2((cm < 2) ? rb : ra);
        const uint32_t keep = (cm < 2) ? ra : rb;
        const uint2 out = (cm < 2) ? make_uint2(keep, r2) : make_uint2(r2, keep);
        const int row = wr0 + i * 32 + q * 8 + lq + rsel;
        const int col = wc0 + j * 32 + colq;
        bf16_t* p = C + (int64_t)row * g.ldc + col;
        if (interior) {
          *reinterpret_cast<uint2*>(p) = out;
        } else if (row < g.M) {
          if (col + 4 <= g.N) {
            *reinterpret_cast<uint2*>(p) = out;
          } else {
            const uint32_t w[2] = {out.x, out.y};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < g.N) p[e] = (bf16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
}

}  // namespace nt

// ------------------------------------------------------------------ launcher

bool gemm_nt_supported(const NtLaunch& L) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!al(L.a) || !al(L.b) || !al(L.c)) return false;
  if (L.lda % 8 || L.ldb % 8 || L.sa % 8 || L.sb % 8 || L.ldc % 8 || L.sc % 8) return false;
  if (L.cin && (!al(L.cin) || L.ldcin % 8 || L.scin % 8)) return false;
  if (L.K % (4 * nt::BK)) return false;  // whole groups of four k-stages
  // operand byte offsets within one problem must fit in 32 bits
  if ((int64_t)L.M * L.lda >= (int64_t)1 << 31 || (int64_t)L.N * L.ldb >= (int64_t)1 << 31)
    return false;   // (byte offsets below 2^32)
  if (L.ct && (!al(L.ct) || L.ldct % 8 || L.sct % 8)) return false;
  return true;
}

sm_status launch_gemm_nt(const NtLaunch& L, int kind, hipStream_t s) {
  using namespace nt;
  if (L.batch <= 0 || L.M <= 0 || L.N <= 0 || L.K <= 0) return SM_OK;
  NtArgs g;
  g.a = L.a; g.lda = L.lda; g.sa = L.sa;
  g.b = L.b; g.ldb = L.ldb; g.sb = L.sb;
  g.cin = L.cin; g.ldcin = L.ldcin; g.scin = L.scin;
  g.c = L.c; g.ldc = L.ldc; g.sc = L.sc;
  g.ct = L.ct; g.ldct = L.ldct; g.sct = L.sct;
  g.scale = L.scale; g.alpha_pow = L.alpha_pow; g.beta_pow = L.beta_pow;
  g.alpha = L.alpha; g.beta = L.beta;
  g.M = L.M; g.N = L.N; g.K = L.K; g.batch = L.batch;
  g.sym = L.sym ? 1 : 0;
  // few row tiles: walk them fastest so the tiles sharing a B row block run
  // together and the (small) A operand stays in L2
  g.tm_fast = (!L.sym && (L.M + BM - 1) / BM <= 4) ? 1 : 0;
  g.ident = L.ident;
  g.ident_bits = L.ident_bits;
  g.tiles_m = (L.M + BM - 1) / BM;
  g.tiles_n = (L.N + BN - 1) / BN;
  g.tiles_per_prob = g.sym ? g.tiles_m * (g.tiles_m + 1) / 2 : g.tiles_m * g.tiles_n;
  const int64_t blocks = (int64_t)g.tiles_per_prob * L.batch;
  // remap only when the grid splits evenly over the 8 XCDs
  g.xcd_chunk = (blocks % 8 == 0) ? (int)(blocks / 8) : 0;
  // a symmetric product is credited with the half it needs (M N K), not 2 M N K
  const double flops = (L.sym ? 1.0 : 2.0) * L.M * (double)L.N * L.K * L.batch;
  prof_begin(kind, flops, s);
  const dim3 grid((unsigned)blocks), block(NT);
  if (L.ident == 1)
    hipLaunchKernelGGL((k_gemm_nt<SM_K_GEMM_APPLY, 1>), grid, block, 0, s, g);
  else if (L.ident == 2)
    hipLaunchKernelGGL((k_gemm_nt<SM_K_GEMM_APPLY, 2>), grid, block, 0, s, g);
  else if (kind == SM_K_GEMM_GRAM)
    hipLaunchKernelGGL((k_gemm_nt<SM_K_GEMM_GRAM, 0>), grid, block, 0, s, g);
  else if (kind == SM_K_GEMM_APPLY)
    hipLaunchKernelGGL((k_gemm_nt<SM_K_GEMM_APPLY, 0>), grid, block, 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm_nt<SM_K_GEMM_RR, 0>), grid, block, 0, s, g);
  prof_end(s);
  return check_launch();
}

}  // namespace sm
