// Batched MFMA GEMM for gfx950 (CDNA4), shared by the Newton-Schulz and
// Gram Newton-Schulz products.
//
//   C[b] = alpha_b * A[b] * B[b] + beta_b * Cin[b] + diag * I     (M x N, K)
//
// Block tile 128 x 128, 256 threads = 4 waves in a 2 x 2 arrangement, each
// wave owning a 64 x 64 sub-tile as 2 x 2 blocks of 32 x 32 MFMA outputs.
// Operands are staged through LDS as [row][k] (k contiguous) in the MFMA
// input type, so every fragment is one 16-byte (bf16) or 8-byte (f32) LDS
// read.  A KC operand (k contiguous in HBM) is copied with 16-byte loads; an
// RC operand (row index contiguous in HBM) is transposed in registers on its
// way into LDS.  Interior tiles with aligned leading dimensions take the
// vector path, edge tiles load element by element with zero fill, so any
// M, N, K >= 1 is handled.
//
// MFMA lane layout relied on (32 x 32 output blocks): for the A operand lane
// l supplies row l % 32, for the B operand column l % 32, each with a group
// of consecutive k selected by l / 32 (A and B use the same k grouping, so
// the order of k inside a group does not matter).  Output register v of lane
// l holds row 8*(v/4) + 4*(l/32) + v%4, column l % 32.
#pragma once

#include "sm_internal.hpp"

namespace sm {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int NT = 256;

template <typename TM> struct Cfg;
template <> struct Cfg<bf16_t> {
  static constexpr int BK = 32;
  static constexpr int LDK = 32 + 8;  // LDS row pitch in elements (80 bytes)
};
template <> struct Cfg<float> {
  static constexpr int BK = 16;
  static constexpr int LDK = 16 + 4;  // 80 bytes
};

template <typename TG, typename TM> struct Conv;
template <> struct Conv<bf16_t, bf16_t> {
  __device__ __forceinline__ static bf16_t cv(bf16_t v) { return v; }
};
template <> struct Conv<float, bf16_t> {
  __device__ __forceinline__ static bf16_t cv(float v) { return f2bf(v); }
};
template <> struct Conv<float, float> {
  __device__ __forceinline__ static float cv(float v) { return v; }
};
template <> struct Conv<bf16_t, float> {
  __device__ __forceinline__ static float cv(bf16_t v) { return bf2f(v); }
};

__device__ __forceinline__ uint32_t pack_bf2(bf16_t lo, bf16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// ------------------------------------------------------------ staging: KC operand
// Tile rows [r0, r0+128), k in [k0, k0+BK) of an operand stored row-major with
// k contiguous: element (r, k) at base[r*ld + k].
template <typename TG, typename TM>
__device__ __forceinline__ void stage_kc(const TG* __restrict__ base, int64_t ld, int r0,
                                         int rows, int k0, int K, bool fast, TM* S) {
  constexpr int BK = Cfg<TM>::BK, LDK = Cfg<TM>::LDK;
  constexpr int VEC = 16 / sizeof(TM);          // elements per 16-byte LDS write
  constexpr int VPR = BK / VEC;                 // vectors per row (4)
  constexpr int NV = (BM * VPR) / NT;           // vectors per thread (2)
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = threadIdx.x + NT * i;
    const int row = v / VPR;
    const int kv = (v % VPR) * VEC;
    TM* dst = S + row * LDK + kv;
    if (fast) {
      const TG* src = base + (int64_t)(r0 + row) * ld + (k0 + kv);
      if constexpr (sizeof(TG) == sizeof(TM)) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {  // float32 in HBM, bf16 in LDS: 8 floats -> 8 bf16
        static_assert(sizeof(TG) == 4 && sizeof(TM) == 2, "f32 -> bf16 staging only");
        float4 x0 = *reinterpret_cast<const float4*>(src);
        float4 x1 = *reinterpret_cast<const float4*>(src + 4);
        uint4 o;
        o.x = pack_bf2(f2bf(x0.x), f2bf(x0.y));
        o.y = pack_bf2(f2bf(x0.z), f2bf(x0.w));
        o.z = pack_bf2(f2bf(x1.x), f2bf(x1.y));
        o.w = pack_bf2(f2bf(x1.z), f2bf(x1.w));
        *reinterpret_cast<uint4*>(dst) = o;
      }
    } else {
      const int r = r0 + row;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int k = k0 + kv + e;
        TG val = (TG)0;
        if (r < rows && k < K) val = base[(int64_t)r * ld + k];
        dst[e] = Conv<TG, TM>::cv(val);
      }
    }
  }
}

// ------------------------------------------------------------ staging: RC operand
// Tile rows [r0, r0+128), k in [k0, k0+BK) of an operand whose row index is
// contiguous: element (r, k) at base[k*ld + r].  Each thread loads KV
// consecutive k for 2 adjacent rows and writes them as two [row][k] vectors.
template <typename TG, typename TM>
__device__ __forceinline__ void stage_rc(const TG* __restrict__ base, int64_t ld, int r0,
                                         int rows, int k0, int K, bool fast, TM* S) {
  constexpr int BK = Cfg<TM>::BK, LDK = Cfg<TM>::LDK;
  constexpr int KV = 16 / sizeof(TM);  // k per LDS vector: 8 (bf16) or 4 (f32)
  static_assert((BK / KV) * (BM / 2) == NT, "one chunk per thread");
  const int rc = (threadIdx.x % (BM / 2)) * 2;
  const int kc = (threadIdx.x / (BM / 2)) * KV;
  __attribute__((aligned(16))) TM v0[KV];
  __attribute__((aligned(16))) TM v1[KV];
  if (fast) {
    const TG* src = base + (int64_t)(k0 + kc) * ld + (r0 + rc);
#pragma unroll
    for (int kk = 0; kk < KV; ++kk) {
      const TG* p = src + (int64_t)kk * ld;
      if constexpr (sizeof(TG) == 2) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        v0[kk] = Conv<TG, TM>::cv((TG)(w & 0xFFFFu));
        v1[kk] = Conv<TG, TM>::cv((TG)(w >> 16));
      } else {
        float2 w = *reinterpret_cast<const float2*>(p);
        v0[kk] = Conv<TG, TM>::cv(w.x);
        v1[kk] = Conv<TG, TM>::cv(w.y);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KV; ++kk) {
      const int k = k0 + kc + kk;
      const int r = r0 + rc;
      TG a = (TG)0, b = (TG)0;
      if (k < K) {
        if (r < rows) a = base[(int64_t)k * ld + r];
        if (r + 1 < rows) b = base[(int64_t)k * ld + r + 1];
      }
      v0[kk] = Conv<TG, TM>::cv(a);
      v1[kk] = Conv<TG, TM>::cv(b);
    }
  }
  TM* d0 = S + rc * LDK + kc;  // 16-byte aligned: LDK*sizeof(TM) and kc*sizeof(TM) are
  TM* d1 = d0 + LDK;            // multiples of 16
  *reinterpret_cast<uint4*>(d0) = *reinterpret_cast<const uint4*>(v0);
  *reinterpret_cast<uint4*>(d1) = *reinterpret_cast<const uint4*>(v1);
}

template <typename TG, typename TM, int LAY>
__device__ __forceinline__ void stage(const TG* base, int64_t ld, int r0, int rows, int k0,
                                      int K, bool fast, TM* S) {
  if constexpr (LAY == KC)
    stage_kc<TG, TM>(base, ld, r0, rows, k0, K, fast, S);
  else
    stage_rc<TG, TM>(base, ld, r0, rows, k0, K, fast, S);
}

// ------------------------------------------------------------ MFMA step

template <typename TM> struct Mma;

template <> struct Mma<bf16_t> {
  // one k-group of 16: fragments are 8 consecutive k at offset 8*(lane/32)
  __device__ __forceinline__ static void step(const bf16_t* As, const bf16_t* Bs, int wm,
                                              int wn, f32x16 (&acc)[2][2]) {
    constexpr int LDK = Cfg<bf16_t>::LDK, BK = Cfg<bf16_t>::BK;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfg[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + lr) * LDK + kk + lk * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfg[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + j * 32 + lr) * LDK + kk + lk * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
    }
  }
};

template <> struct Mma<float> {
  // pairs of 32x32x2 MFMAs over 4 k: lane supplies k = kk + 2*(lane/32) + {0,1}
  __device__ __forceinline__ static void step(const float* As, const float* Bs, int wm, int wn,
                                              f32x16 (&acc)[2][2]) {
    constexpr int LDK = Cfg<float>::LDK, BK = Cfg<float>::BK;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float2 af[2], bfg[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const float2*>(As + (wm * 64 + i * 32 + lr) * LDK + kk + lk * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfg[j] = *reinterpret_cast<const float2*>(Bs + (wn * 64 + j * 32 + lr) * LDK + kk + lk * 2);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i].x, bfg[j].x, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i].y, bfg[j].y, acc[i][j], 0, 0, 0);
        }
    }
  }
};

// ------------------------------------------------------------ kernel

// Base address of problem b of an operand or output.
__device__ __forceinline__ const char* prob_base(const GemmArgs& g, const void* p, int tbl,
                                                 int64_t stride, size_t es, int b) {
  if (tbl) return tbl_addr(g.tbl, b, g.tbl_per, stride * (int64_t)es);
  return reinterpret_cast<const char*>(p) + (int64_t)b * stride * (int64_t)es;
}

struct KArgs {
  GemmArgs g;
  bool a_aligned, b_aligned;
  int tiles_n, tiles;
};

// ROLE (the SM_K_GEMM_* / SM_K_PROBE kind) changes no code; it gives each
// role its own kernel symbol so per-kernel profiles attribute time by role.
template <typename TA, typename TB, typename TM, int LA, int LB, int ROLE>
__global__ __launch_bounds__(NT) void k_gemm(KArgs ka) {
  constexpr int BK = Cfg<TM>::BK, LDK = Cfg<TM>::LDK;
  __shared__ __attribute__((aligned(16))) TM As[BM * LDK];
  __shared__ __attribute__((aligned(16))) TM Bs[BN * LDK];
  __shared__ float red[4];
  const GemmArgs& g = ka.g;
  const int b = blockIdx.y;
  if (g.pred && g.pred[(int64_t)b * g.pred_stride] != g.pred_val) return;
  if (g.prof_exec && blockIdx.x == 0 && threadIdx.x == 0) {
    atomicAdd(g.prof_exec, g.prof_flops);
    atomicAdd(g.prof_exec + 1, g.prof_bytes);
  }

  const int tile = blockIdx.x;
  const int tm = tile / ka.tiles_n, tn = tile % ka.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TA* A = reinterpret_cast<const TA*>(prob_base(g, g.a.p, g.a.tbl, g.a.stride, sizeof(TA), b));
  const TB* B = reinterpret_cast<const TB*>(prob_base(g, g.b.p, g.b.tbl, g.b.stride, sizeof(TB), b));

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const bool a_rows_in = (m0 + BM) <= g.M;
  const bool b_rows_in = (n0 + BN) <= g.N;
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    const bool k_in = (k0 + BK) <= g.K;
    __syncthreads();
    stage<TA, TM, LA>(A, g.a.ld, m0, g.M, k0, g.K, ka.a_aligned && a_rows_in && k_in, As);
    stage<TB, TM, LB>(B, g.b.ld, n0, g.N, k0, g.K, ka.b_aligned && b_rows_in && k_in, Bs);
    __syncthreads();
    Mma<TM>::step(As, Bs, wm, wn, acc);
  }

  // ---------------- epilogue
  float alpha = g.alpha, beta = g.beta;
  if (g.scale) {
    const float s = g.scale[b];
    for (int p = 0; p < g.alpha_pow; ++p) alpha *= s;
    for (int p = 0; p < g.beta_pow; ++p) beta *= s;
  }
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
  const size_t ces = (g.c_dt == BF16) ? 2 : 4;
  const char* cin_b = g.cin ? prob_base(g, g.cin, g.cin_tbl, g.scin, ces, b) : nullptr;
  char* c_b = g.c ? const_cast<char*>(prob_base(g, g.c, g.c_tbl, g.sc, ces, b)) : nullptr;
  float* c2_b =
      g.c2 ? reinterpret_cast<float*>(const_cast<char*>(prob_base(g, g.c2, g.c2_tbl, g.sc2, 4, b)))
           : nullptr;
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + i * 32 + (v >> 2) * 8 + lk * 4 + (v & 3);
        const int col = n0 + wn * 64 + j * 32 + lr;
        if (row < g.M && col < g.N) {
          float val = alpha * acc[i][j][v];
          if (cin_b) {
            const int64_t off = (int64_t)row * g.ldcin + col;
            const float ci = (g.c_dt == BF16)
                                 ? bf2f(reinterpret_cast<const bf16_t*>(cin_b)[off])
                                 : reinterpret_cast<const float*>(cin_b)[off];
            val += beta * ci;
          }
          if (row == col) val += g.diag;
          if (c_b) {
            const int64_t off = (int64_t)row * g.ldc + col;
            if (g.c_dt == BF16)
              reinterpret_cast<bf16_t*>(c_b)[off] = f2bf(val);
            else
              reinterpret_cast<float*>(c_b)[off] = val;
          }
          if (c2_b) {
            c2_b[(int64_t)row * g.ldc2 + col] = g.c2_scale * val + (row == col ? g.c2_diag : 0.f);
          }
          if (g.resid) {
            const float d = val - (row == col ? 1.f : 0.f);
            rs += d * d;
          }
        }
      }
  if (g.resid) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rs += __shfl_xor(rs, o, 64);
    if (lane == 0) red[wave] = rs;
    __syncthreads();
    if (threadIdx.x == 0)
      g.resid[(int64_t)b * ka.tiles + tile] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

// Host-side alignment test for the vector staging path of an operand.
inline bool operand_aligned(const GemmArgs& g, const GemmOperand& o, int mfma_dt) {
  const size_t es = dt_size(o.dt);
  uintptr_t p = reinterpret_cast<uintptr_t>(o.p);
  if (o.tbl) {  // every table entry must satisfy the same alignment
    p = 0;
    const int n = (g.batch + g.tbl_per - 1) / g.tbl_per;
    for (int i = 0; i < n && i < kTbl; ++i) p |= reinterpret_cast<uintptr_t>(g.tbl.p[i]);
  }
  if (o.layout == KC) {
    // 16-byte loads of 16/es elements (two float4 for f32 -> bf16 LDS)
    const int64_t vec = 16 / (int64_t)es;
    return (p % 16 == 0) && (o.ld % vec == 0) && (o.stride % vec == 0);
  }
  // pairs of adjacent rows: 4-byte (bf16) or 8-byte (f32) loads
  (void)mfma_dt;
  return (p % (2 * es) == 0) && (o.ld % 2 == 0) && (o.stride % 2 == 0);
}

template <typename TA, typename TB, typename TM, int LA, int LB>
sm_status launch_t(const GemmArgs& g, int kind, hipStream_t s) {
  KArgs ka;
  ka.g = g;
  ka.a_aligned = operand_aligned(g, g.a, 0);
  ka.b_aligned = operand_aligned(g, g.b, 0);
  const int tiles_m = (g.M + BM - 1) / BM;
  ka.tiles_n = (g.N + BN - 1) / BN;
  ka.tiles = tiles_m * ka.tiles_n;
  dim3 grid(ka.tiles, g.batch);
  const double bytes = ((double)g.M * g.K * dt_size(g.a.dt) + (double)g.N * g.K * dt_size(g.b.dt) +
                        (double)g.M * g.N * (g.c ? dt_size(g.c_dt) : 0)) * g.batch;
  double* exec = g.pred ? prof_exec_slot(kind) : nullptr;
  if (exec) {  // the problems that run report their own work
    ka.g.prof_exec = exec;
    ka.g.prof_flops = 2.0 * g.M * (double)g.N * g.K;
    ka.g.prof_bytes = bytes / g.batch;
    prof_begin(kind, 0.0, s, 0.0);
  } else {
    ka.g.prof_exec = nullptr;
    prof_begin(kind, 2.0 * g.M * (double)g.N * g.K * g.batch, s, bytes);
  }
  switch (kind) {
    case SM_K_GEMM_GRAM:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_GEMM_GRAM>), grid, dim3(NT), 0, s, ka);
      break;
    case SM_K_GEMM_APPLY:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_GEMM_APPLY>), grid, dim3(NT), 0, s, ka);
      break;
    case SM_K_PROBE:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_PROBE>), grid, dim3(NT), 0, s, ka);
      break;
    default:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_GEMM_RR>), grid, dim3(NT), 0, s, ka);
      break;
  }
  prof_end(s);
  return check_launch();
}

}  // namespace gemm
}  // namespace sm
