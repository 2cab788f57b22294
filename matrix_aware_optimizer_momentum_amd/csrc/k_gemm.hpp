// Batched, grouped MFMA GEMM for gfx950 (CDNA4), shared by the Newton-Schulz
// and Gram Newton-Schulz products that the persistent bf16 NS kernel does not
// take (float32 NS, CacheMuon's generic solve, edge layouts).
//
//   C[b] = alpha_b * A[b] * B[b] + beta_b * Cin[b] + diag * I     (M x N, K)
//
// One launch runs up to kGemmMaxGroups product sets of possibly different
// shapes (one block per 128 x 128 output tile per problem, the sets' blocks
// laid end to end in a 1-D grid), so the products of every matrix shape of a
// step share a launch and fill the chip together.
//
// Block tile 128 x 128, 256 threads = 4 waves in a 2 x 2 arrangement, each
// wave owning a 64 x 64 sub-tile as 2 x 2 blocks of 32 x 32 MFMA outputs; a
// float32 launch too small to fill the chip with such tiles takes 64 x 64
// tiles (one 32 x 32 block per wave) instead.
// Operands are staged through LDS as [row][k] (k contiguous) in the MFMA
// input type, so every fragment is one 16-byte (bf16) or 8-byte (f32) LDS
// read.  A KC operand (k contiguous in HBM) is copied with 16-byte loads; an
// RC operand (row index contiguous in HBM) is transposed in registers on its
// way into LDS, except with float32 MFMA input: there it is copied as it
// lies, [k][row], and a fragment is two dword reads (the float32 MFMA takes
// one k per register, so no transpose is needed at all).  Interior tiles
// with aligned leading dimensions take the vector path, edge tiles load
// element by element with zero fill, so any M, N, K >= 1 is handled.
//
// Pipelining: two LDS stages.  The global loads of k-slab t+1 are issued into
// registers before the MFMAs of slab t, and written to the other LDS stage
// after them, so their latency hides behind the MFMAs; one barrier per slab.
// The float32 64 tile keeps two slabs in flight in two register sets.
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

constexpr int BM = 128;      // block tile (the small-problem float32 variant uses 64)
constexpr int BN = 128;
constexpr int NT = 256;
constexpr int kGemmMaxGroups = 8;

// k-slab depth and LDS row pitch per MFMA type and block tile T.
template <typename TM, int T> struct Cfg;
template <int T> struct Cfg<bf16_t, T> {
  static constexpr int BK = 32;
  static constexpr int LDK = 32 + 8;  // LDS row pitch in elements (80 bytes)
};
template <int T> struct Cfg<float, T> {
  // The 64 tile takes 32 k per slab (a wave's one 32 x 32 block then gets 16
  // MFMAs per slab); the 128 tile keeps 16 (its wave issues 32 MFMAs per slab
  // over four blocks already, and a deeper slab would cost the CU blocks).
  static constexpr int BK = T == 64 ? 32 : 16;
  static constexpr int LDK = BK + 4;  // 144 or 80 bytes
  // pitch of a [k][row] stage (RC operands): the two k rows that the halves
  // of a wave read in one fragment load lie 2 * LDR = 32 (mod 64) banks apart
  static constexpr int LDR = T + 16;
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

// ------------------------------------------------------------ staging
// A stage is split in two: load() issues the global loads of one k-slab of
// the tile into registers (raw HBM type), store() converts them to the MFMA
// type and writes them to an LDS stage.  Between the two the loads are in
// flight.

template <typename TG, typename TM, int LAY, int T> struct Stage;

// KC operand: tile rows [r0, r0+T), k in [k0, k0+BK), element (r, k) at
// base[r*ld + k].  Each thread moves NV vectors of VEC consecutive k.
template <typename TG, typename TM, int T> struct Stage<TG, TM, KC, T> {
  static constexpr int BK = Cfg<TM, T>::BK, LDK = Cfg<TM, T>::LDK;
  static constexpr int VEC = 16 / sizeof(TM);   // elements per 16-byte LDS write
  static constexpr int VPR = BK / VEC;          // vectors per row (4)
  static constexpr int NV = (T * VPR) / NT;     // vectors per thread (2 for T = 128)
  static constexpr int ELEMS = T * LDK;         // LDS elements of one stage, as [row][k]
  static_assert(NV >= 1, "every thread moves a vector");
  static_assert((VEC * sizeof(TG)) % 16 == 0, "whole 16-byte global loads");
  __attribute__((aligned(16))) TG raw[NV][VEC];

  __device__ __forceinline__ void load(const TG* __restrict__ base, int64_t ld, int r0,
                                       int rows, int k0, int K, bool fast) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = threadIdx.x + NT * i;
      const int row = v / VPR;
      const int kv = (v % VPR) * VEC;
      if (fast) {
        const uint4* src =
            reinterpret_cast<const uint4*>(base + (int64_t)(r0 + row) * ld + (k0 + kv));
        uint4* dst = reinterpret_cast<uint4*>(raw[i]);
#pragma unroll
        for (int q = 0; q < (int)(VEC * sizeof(TG) / 16); ++q) dst[q] = src[q];
      } else {
        const int r = r0 + row;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int k = k0 + kv + e;
          raw[i][e] = (r < rows && k < K) ? base[(int64_t)r * ld + k] : (TG)0;
        }
      }
    }
  }
  __device__ __forceinline__ void store(TM* S) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = threadIdx.x + NT * i;
      const int row = v / VPR;
      const int kv = (v % VPR) * VEC;
      __attribute__((aligned(16))) TM o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = Conv<TG, TM>::cv(raw[i][e]);
      *reinterpret_cast<uint4*>(S + row * LDK + kv) = *reinterpret_cast<const uint4*>(o);
    }
  }
};

// RC operand: tile rows [r0, r0+T), k in [k0, k0+BK), element (r, k) at
// base[k*ld + r].  A chunk is KV consecutive k of 2 adjacent rows, written as
// two [row][k] vectors; a thread moves NC chunks (for T = 64 with bf16 half
// the threads have none).
template <typename TG, typename TM, int T> struct Stage<TG, TM, RC, T> {
  static constexpr int BK = Cfg<TM, T>::BK, LDK = Cfg<TM, T>::LDK;
  static constexpr int KV = 16 / sizeof(TM);  // k per LDS vector: 8 (bf16) or 4 (f32)
  static constexpr int CHUNKS = (BK / KV) * (T / 2);
  static constexpr int NC = CHUNKS >= NT ? CHUNKS / NT : 1;
  static constexpr int ELEMS = T * LDK;   // LDS elements of one stage, as [row][k]
  static_assert(CHUNKS == NT / 2 || CHUNKS % NT == 0, "chunks spread evenly over the threads");
  TG v0[NC][KV], v1[NC][KV];

  __device__ __forceinline__ void load(const TG* __restrict__ base, int64_t ld, int r0,
                                       int rows, int k0, int K, bool fast) {
    if (CHUNKS < NT && (int)threadIdx.x >= CHUNKS) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int id = threadIdx.x + NT * c;
      const int rc = (id % (T / 2)) * 2;
      const int kc = (id / (T / 2)) * KV;
      if (fast) {
        const TG* src = base + (int64_t)(k0 + kc) * ld + (r0 + rc);
#pragma unroll
        for (int kk = 0; kk < KV; ++kk) {
          const TG* p = src + (int64_t)kk * ld;
          if constexpr (sizeof(TG) == 2) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
            v0[c][kk] = (TG)(w & 0xFFFFu);
            v1[c][kk] = (TG)(w >> 16);
          } else {
            const float2 w = *reinterpret_cast<const float2*>(p);
            v0[c][kk] = w.x;
            v1[c][kk] = w.y;
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
          v0[c][kk] = a;
          v1[c][kk] = b;
        }
      }
    }
  }
  __device__ __forceinline__ void store(TM* S) const {
    if (CHUNKS < NT && (int)threadIdx.x >= CHUNKS) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int id = threadIdx.x + NT * c;
      const int rc = (id % (T / 2)) * 2;
      const int kc = (id / (T / 2)) * KV;
      __attribute__((aligned(16))) TM o0[KV];
      __attribute__((aligned(16))) TM o1[KV];
#pragma unroll
      for (int kk = 0; kk < KV; ++kk) {
        o0[kk] = Conv<TG, TM>::cv(v0[c][kk]);
        o1[kk] = Conv<TG, TM>::cv(v1[c][kk]);
      }
      TM* d0 = S + rc * LDK + kc;  // 16-byte aligned: LDK*sizeof(TM) and kc*sizeof(TM) are
      TM* d1 = d0 + LDK;            // multiples of 16
      *reinterpret_cast<uint4*>(d0) = *reinterpret_cast<const uint4*>(o0);
      *reinterpret_cast<uint4*>(d1) = *reinterpret_cast<const uint4*>(o1);
    }
  }
};

// RC float32 operand with float32 MFMA input: staged without a transpose.
// The LDS stage holds it as [k][row] (rows contiguous, pitch LDR), and each
// thread moves NV 16-byte vectors of 4 consecutive rows at one k; the MFMA
// step reads a lane's two k of a group as two dwords LDR apart.
template <int T> struct Stage<float, float, RC, T> {
  static constexpr int BK = Cfg<float, T>::BK, LDR = Cfg<float, T>::LDR;
  static constexpr int VPK = T / 4;              // vectors per k
  static constexpr int NV = BK * VPK / NT;       // vectors per thread (2)
  static constexpr int ELEMS = BK * LDR;         // LDS elements of one stage, as [k][row]
  static_assert(NV >= 1 && (BK * VPK) % NT == 0, "vectors spread evenly over the threads");
  float4 raw[NV];

  __device__ __forceinline__ void load(const float* __restrict__ base, int64_t ld, int r0,
                                       int rows, int k0, int K, bool fast) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = threadIdx.x + NT * i;
      const int k = k0 + v / VPK;
      const int r = r0 + (v % VPK) * 4;
      if (fast) {
        raw[i] = *reinterpret_cast<const float4*>(base + (int64_t)k * ld + r);
      } else {
        const float* src = base + (int64_t)k * ld;
        const bool kin = k < K;
        raw[i].x = (kin && r < rows) ? src[r] : 0.f;
        raw[i].y = (kin && r + 1 < rows) ? src[r + 1] : 0.f;
        raw[i].z = (kin && r + 2 < rows) ? src[r + 2] : 0.f;
        raw[i].w = (kin && r + 3 < rows) ? src[r + 3] : 0.f;
      }
    }
  }
  __device__ __forceinline__ void store(float* S) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = threadIdx.x + NT * i;
      *reinterpret_cast<float4*>(S + (v / VPK) * LDR + (v % VPK) * 4) = raw[i];
    }
  }
};

// ------------------------------------------------------------ MFMA step

template <typename TM> struct Mma;

// A wave owns WB x WB output blocks of 32 x 32 (WB = 2 for the 128 tile, 1
// for the 64 tile).
template <> struct Mma<bf16_t> {
  // k-groups of 16: fragments are 8 consecutive k at offset 8*(lane/32).  The
  // next group's fragments are read before this group's MFMAs go out.
  template <int WB, int LA, int LB>   // both layouts are staged as [row][k]
  __device__ __forceinline__ static void step(const bf16_t* As, const bf16_t* Bs, int wm,
                                              int wn, f32x16 (&acc)[WB][WB]) {
    constexpr int LDK = Cfg<bf16_t, 64 * WB>::LDK, BK = Cfg<bf16_t, 64 * WB>::BK;
    constexpr int NG = BK / 16;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lk = lane >> 5;
    const bf16_t* pa = As + (wm * 32 * WB + lr) * LDK + lk * 8;
    const bf16_t* pb = Bs + (wn * 32 * WB + lr) * LDK + lk * 8;
    bf16x8 af[2][WB], bfg[2][WB];
#pragma unroll
    for (int i = 0; i < WB; ++i) {
      af[0][i] = *reinterpret_cast<const bf16x8*>(pa + i * 32 * LDK);
      bfg[0][i] = *reinterpret_cast<const bf16x8*>(pb + i * 32 * LDK);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int c = g & 1, n = c ^ 1;
      if (g + 1 < NG) {
#pragma unroll
        for (int i = 0; i < WB; ++i) {
          af[n][i] = *reinterpret_cast<const bf16x8*>(pa + i * 32 * LDK + (g + 1) * 16);
          bfg[n][i] = *reinterpret_cast<const bf16x8*>(pb + i * 32 * LDK + (g + 1) * 16);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // the reads go out ahead of the MFMAs
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[c][i], bfg[c][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// Float32 fragment of output block i of wave row / column w, k-group g: the
// lane's k = 4 g + 2 (lane / 32) + {0, 1} of row 32 (WB w + i) + lane % 32,
// from a [row][k] stage (one 8-byte read) or a [k][row] stage (two dwords).
template <int LAY, int WB>
__device__ __forceinline__ float2 frag_f32(const float* S, int w, int i, int g) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
  if constexpr (LAY == RC) {
    constexpr int LDR = Cfg<float, 64 * WB>::LDR;
    const float* p = S + (g * 4 + lk * 2) * LDR + (w * WB + i) * 32 + lr;
    return make_float2(p[0], p[LDR]);
  } else {
    constexpr int LDK = Cfg<float, 64 * WB>::LDK;
    return *reinterpret_cast<const float2*>(S + ((w * WB + i) * 32 + lr) * LDK + g * 4 + lk * 2);
  }
}

template <> struct Mma<float> {
  // k-groups of 4, each two 32x32x2 MFMAs per output block.  The next
  // group's fragments are read before this group's MFMAs go out.
  template <int WB, int LA, int LB>
  __device__ __forceinline__ static void step(const float* As, const float* Bs, int wm, int wn,
                                              f32x16 (&acc)[WB][WB]) {
    constexpr int NG = Cfg<float, 64 * WB>::BK / 4;
    float2 af[2][WB], bfg[2][WB];
#pragma unroll
    for (int i = 0; i < WB; ++i) {
      af[0][i] = frag_f32<LA, WB>(As, wm, i, 0);
      bfg[0][i] = frag_f32<LB, WB>(Bs, wn, i, 0);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int c = g & 1, n = c ^ 1;
      if (g + 1 < NG) {
#pragma unroll
        for (int i = 0; i < WB; ++i) {
          af[n][i] = frag_f32<LA, WB>(As, wm, i, g + 1);
          bfg[n][i] = frag_f32<LB, WB>(Bs, wn, i, g + 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // the reads go out ahead of the MFMAs
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[c][i].x, bfg[c][j].x, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[c][i].y, bfg[c][j].y, acc[i][j], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// ------------------------------------------------------------ kernel

// Epilogue of an interior tile with a float32 output and none of the rarer
// outputs (second output, residual partials): per 32 x 32 block the Cin
// values are loaded first (all in flight together), then
// value = alpha acc + beta Cin (+ diag on the diagonal), kept in acc (for the
// sign packing) and stored, and stored transposed too for a mirrored tile
// (16-byte aligned output rows: ldc % 4 == 0).
// The same arithmetic, in the same order, as the general epilogue; no
// bounds checks and no per-element branches on launch parameters.
template <bool CIN, int WB>
__device__ __forceinline__ void epilogue_f32_interior(f32x16 (&acc)[WB][WB], float alpha,
                                                      float beta, float diag, const float* cin,
                                                      int64_t ldcin, float* c, int64_t ldc,
                                                      bool mirror, int r0, int c0) {
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j) {
      const int rb = r0 + i * 32;   // row of v = rb + e(v), e(v) = 8 (v / 4) + v % 4
      const int col = c0 + j * 32;
      float ci[16];
      if constexpr (CIN) {
        const float* p = cin + (int64_t)rb * ldcin + col;
#pragma unroll
        for (int v = 0; v < 16; ++v) ci[v] = p[((v >> 2) * 8 + (v & 3)) * ldcin];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rb + (v >> 2) * 8 + (v & 3);
        float val = alpha * acc[i][j][v];
        if constexpr (CIN) val += beta * ci[v];
        if (row == col) val += diag;
        acc[i][j][v] = val;
      }
      if (c) {
        float* p = c + (int64_t)rb * ldc + col;
#pragma unroll
        for (int v = 0; v < 16; ++v) p[((v >> 2) * 8 + (v & 3)) * ldc] = acc[i][j][v];
        if (mirror) {   // rows e(v) of column col: four runs of four consecutive entries
          float* q = c + (int64_t)col * ldc + rb;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            *reinterpret_cast<float4*>(q + 8 * u) =
                make_float4(acc[i][j][4 * u], acc[i][j][4 * u + 1], acc[i][j][4 * u + 2],
                            acc[i][j][4 * u + 3]);
        }
      }
    }
}

// One product set of a launch as the kernel sees it.
struct KGroup {
  GemmCore g;
  int tiles_n, tiles;   // tiles per problem
  int blk_begin;        // first block of the set in the launch grid
  int a_aligned, b_aligned;
};

struct KArgs {
  KGroup grp[kGemmMaxGroups];
  PtrTbl tbl;
  int ngroups;
};

// Base address of problem b of an operand or output.
__device__ __forceinline__ const char* prob_base(const KArgs& ka, const GemmCore& g, const void* p,
                                                 int tbl, int64_t stride, size_t es, int b) {
  if (tbl) {
    const int e = g.tbl_off + b / g.tbl_per;
    return ka.tbl.p[e] + (int64_t)(b % g.tbl_per) * stride * (int64_t)es;
  }
  return reinterpret_cast<const char*>(p) + (int64_t)b * stride * (int64_t)es;
}

// ROLE (the SM_K_GEMM_* / SM_K_PROBE kind) changes no code; it gives each
// role its own kernel symbol so per-kernel profiles attribute time by role.
// T: the square block tile (128, or 64 for launches too small to fill the
// chip with 128 tiles), a wave owning (T / 2)^2 of it.
template <typename TA, typename TB, typename TM, int LA, int LB, int ROLE, int T>
__global__ __launch_bounds__(NT, (T == 128 && sizeof(TM) == 4) ? 3 : 1) void k_gemm(KArgs ka) {
  constexpr int BK = Cfg<TM, T>::BK;
  constexpr int WB = T / 64;   // 32 x 32 blocks per wave and dimension
  constexpr int WT = T / 2;    // wave sub-tile
  using SA = Stage<TA, TM, LA, T>;
  using SB = Stage<TB, TM, LB, T>;
  __shared__ __attribute__((aligned(16))) TM As[2][SA::ELEMS];
  __shared__ __attribute__((aligned(16))) TM Bs[2][SB::ELEMS];
  __shared__ float red[4];
  int gi = 0;
  while (gi + 1 < ka.ngroups && (int)blockIdx.x >= ka.grp[gi + 1].blk_begin) ++gi;
  const KGroup& kg = ka.grp[gi];
  const GemmCore& g = kg.g;
  const int local = (int)blockIdx.x - kg.blk_begin;
  const int b = local / kg.tiles;
  const int tile = local - b * kg.tiles;
  if (g.pred && g.pred[(int64_t)b * g.pred_stride] != g.pred_val) return;
  if (g.prof_exec && tile == 0 && threadIdx.x == 0) {
    atomicAdd(g.prof_exec, g.prof_flops);
    atomicAdd(g.prof_exec + 1, g.prof_bytes);
  }

  int tm, tn;
  if (g.sym) {   // lower-triangle tile u = tm (tm + 1) / 2 + tn, tn <= tm
    tm = (int)((sqrtf(8.f * (float)tile + 1.f) - 1.f) * 0.5f);
    while (tm * (tm + 1) / 2 > tile) --tm;
    while ((tm + 1) * (tm + 2) / 2 <= tile) ++tm;
    tn = tile - tm * (tm + 1) / 2;
  } else {
    tm = tile / kg.tiles_n;
    tn = tile % kg.tiles_n;
  }
  const bool mirror = g.sym && tm != tn;
  const int m0 = tm * T, n0 = tn * T;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TA* A =
      reinterpret_cast<const TA*>(prob_base(ka, g, g.a.p, g.a.tbl, g.a.stride, sizeof(TA), b));
  const TB* B =
      reinterpret_cast<const TB*>(prob_base(ka, g, g.b.p, g.b.tbl, g.b.stride, sizeof(TB), b));

  f32x16 acc[WB][WB];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const bool a_fast_rows = kg.a_aligned && (m0 + T) <= g.M;
  const bool b_fast_rows = kg.b_aligned && (n0 + T) <= g.N;
  const int nk = (g.K + BK - 1) / BK;
  auto load = [&](SA& sa, SB& sb, int kt) {
    const int k0 = kt * BK;
    const bool k_in = (k0 + BK) <= g.K;
    sa.load(A, g.a.ld, m0, g.M, k0, g.K, a_fast_rows && k_in);
    sb.load(B, g.b.ld, n0, g.N, k0, g.K, b_fast_rows && k_in);
  };
  if constexpr (sizeof(TM) == 4 && T == 64) {
    // Two slabs in flight: slab t + 2's loads are issued before slab t's
    // MFMAs, slab t + 1 (loaded one step earlier) goes to LDS after them.
    // One slab's MFMAs (16 per wave) are shorter than a load's latency, so
    // with one slab in flight the loop waited on every load.  The two
    // register sets alternate, hence the loop by pairs.
    SA sa0, sa1;
    SB sb0, sb1;
    load(sa0, sb0, 0);
    if (nk > 1) load(sa1, sb1, 1);
    sa0.store(As[0]);
    sb0.store(Bs[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      if (kt + 2 < nk) load(sa0, sb0, kt + 2);
      Mma<TM>::template step<WB, LA, LB>(As[0], Bs[0], wm, wn, acc);
      if (kt + 1 < nk) {   // stage 1 was last read by slab kt - 1, before the last barrier
        sa1.store(As[1]);
        sb1.store(Bs[1]);
      }
      __syncthreads();
      if (kt + 1 >= nk) break;
      if (kt + 3 < nk) load(sa1, sb1, kt + 3);
      Mma<TM>::template step<WB, LA, LB>(As[1], Bs[1], wm, wn, acc);
      if (kt + 2 < nk) {
        sa0.store(As[0]);
        sb0.store(Bs[0]);
      }
      __syncthreads();
    }
  } else {
    SA sa;
    SB sb;
    load(sa, sb, 0);
    sa.store(As[0]);
    sb.store(Bs[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) load(sa, sb, kt + 1);
      Mma<TM>::template step<WB, LA, LB>(As[cur], Bs[cur], wm, wn, acc);
      if (more) {
        // stage cur ^ 1 was last read by slab kt - 1, before the previous barrier
        sa.store(As[cur ^ 1]);
        sb.store(Bs[cur ^ 1]);
      }
      __syncthreads();
    }
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
  // an input / output is present when its pointer or its table flag is set
  const char* cin_b =
      (g.cin || g.cin_tbl) ? prob_base(ka, g, g.cin, g.cin_tbl, g.scin, ces, b) : nullptr;
  char* c_b = (g.c || g.c_tbl) ? const_cast<char*>(prob_base(ka, g, g.c, g.c_tbl, g.sc, ces, b))
                               : nullptr;
  float* c2_b = (g.c2 || g.c2_tbl) ? reinterpret_cast<float*>(const_cast<char*>(
                                         prob_base(ka, g, g.c2, g.c2_tbl, g.sc2, 4, b)))
                                   : nullptr;
  // uniform parameters, read once (every store below may alias the kernel
  // arguments as far as the compiler knows)
  const bool cbf = g.c_dt == BF16;
  const int Mg = g.M, Ng = g.N;
  const int64_t ldcin = g.ldcin, ldc = g.ldc, ldc2 = g.ldc2;
  const float diag = g.diag, c2_scale = g.c2_scale, c2_diag = g.c2_diag;
  const bool resid = g.resid != nullptr;
  float rs = 0.f;
  const bool interior = (m0 + T) <= Mg && (n0 + T) <= Ng;
  // (a mirrored tile's transposed stores go out as 16-byte vectors)
  const bool vec_ok = !mirror || ((ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(c_b) & 15) == 0);
  // (float32 MFMA kernels only: on the bf16 ones it would cost occupancy)
  if (sizeof(TM) == 4 && !cbf && interior && !c2_b && !resid && vec_ok) {
    const int r0 = m0 + wm * WT + lk * 4, c0 = n0 + wn * WT + lr;
    float* cf = reinterpret_cast<float*>(c_b);
    if constexpr (sizeof(TM) == 4) {
      if (cin_b)
        epilogue_f32_interior<true, WB>(acc, alpha, beta, diag,
                                        reinterpret_cast<const float*>(cin_b), ldcin, cf, ldc,
                                        mirror, r0, c0);
      else
        epilogue_f32_interior<false, WB>(acc, alpha, beta, diag, nullptr, 0, cf, ldc, mirror,
                                         r0, c0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * WT + i * 32 + (v >> 2) * 8 + lk * 4 + (v & 3);
          const int col = n0 + wn * WT + j * 32 + lr;
          float stored = 0.f;
          if (row < Mg && col < Ng) {
            float val = alpha * acc[i][j][v];
            if (cin_b) {
              const int64_t off = (int64_t)row * ldcin + col;
              const float ci = cbf ? bf2f(reinterpret_cast<const bf16_t*>(cin_b)[off])
                                   : reinterpret_cast<const float*>(cin_b)[off];
              val += beta * ci;
            }
            if (row == col) val += diag;
            stored = cbf ? bf2f(f2bf(val)) : val;
            if (c_b) {
              const int64_t off = (int64_t)row * ldc + col;
              const int64_t offt = (int64_t)col * ldc + row;
              if (cbf) {
                reinterpret_cast<bf16_t*>(c_b)[off] = f2bf(val);
                if (mirror) reinterpret_cast<bf16_t*>(c_b)[offt] = f2bf(val);
              } else {
                reinterpret_cast<float*>(c_b)[off] = val;
                if (mirror) reinterpret_cast<float*>(c_b)[offt] = val;
              }
            }
            if (c2_b)
              c2_b[(int64_t)row * ldc2 + col] = c2_scale * val + (row == col ? c2_diag : 0.f);
            if (resid) {
              const float d = val - (row == col ? 1.f : 0.f);
              rs += d * d;
            }
          }
          acc[i][j][v] = stored;
        }
  }
  if (g.bits) {
    // Signs of the stored values, packed: for fixed (i, v) the ballot over
    // the wave of block j holds row R (lanes 0-31) and row R + 4 (lanes
    // 32-63), columns c0 + 32 j + lane % 32, with c0 = n0 + WT wn.
    // N % 64 == 0 makes each row's 64 columns from a multiple of 64 one sign
    // word: with the 128 tile a wave covers a whole word (blocks j = 0, 1),
    // with the 64 tile each wave its 32-bit half.
    const int c0 = n0 + wn * WT;
    if constexpr (WB == 2) {
      uint64_t* bits_b = g.bits + (int64_t)b * g.bits_stride;
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint64_t b0 = __ballot(acc[i][0][v] < 0.f);
          const uint64_t b1 = __ballot(acc[i][1][v] < 0.f);
          const int row = m0 + wm * WT + i * 32 + (v >> 2) * 8 + lk * 4 + (v & 3);
          if (lr == 0 && row < g.M && c0 < g.N) {
            const uint64_t w = lk == 0 ? ((b0 & 0xFFFFFFFFull) | (b1 << 32))
                                       : ((b0 >> 32) | (b1 & 0xFFFFFFFF00000000ull));
            bits_b[((int64_t)row * g.N + c0) >> 6] = w;
          }
        }
    } else {
      uint32_t* half_b = reinterpret_cast<uint32_t*>(g.bits + (int64_t)b * g.bits_stride);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint64_t b0 = __ballot(acc[0][0][v] < 0.f);
        const int row = m0 + wm * WT + (v >> 2) * 8 + lk * 4 + (v & 3);
        if (lr == 0 && row < g.M && n0 < g.N)
          half_b[(((int64_t)row * g.N + n0) >> 6) * 2 + wn] =
              lk == 0 ? (uint32_t)b0 : (uint32_t)(b0 >> 32);
      }
    }
  }
  if (g.resid) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) rs += __shfl_xor(rs, o, 64);
    if (lane == 0) red[wave] = rs;
    __syncthreads();
    if (threadIdx.x == 0)
      g.resid[(int64_t)b * kg.tiles + tile] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

// Host-side alignment test for the vector staging path of an operand.
// vec4_rc: an RC operand staged by 16-byte loads of 4 rows (float32 into a
// float32 MFMA) rather than by pairs of rows.
inline bool operand_aligned(const GemmArgs& g, const GemmOperand& o, bool vec4_rc) {
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
  if (vec4_rc) return (p % 16 == 0) && (o.ld % 4 == 0) && (o.stride % 4 == 0);
  // pairs of adjacent rows: 4-byte (bf16) or 8-byte (f32) loads
  return (p % (2 * es) == 0) && (o.ld % 2 == 0) && (o.stride % 2 == 0);
}

inline bool uses_tbl(const GemmArgs& g) {
  return g.a.tbl || g.b.tbl || g.cin_tbl || g.c_tbl || g.c2_tbl;
}

// Launches n (<= kGemmMaxGroups) product sets of one operand-type / layout
// combination with block tile T; their tables must fit one launch table
// together (the caller, launch_gemm_groups, packs them).
template <typename TA, typename TB, typename TM, int LA, int LB, int T>
sm_status launch_tile(const GemmArgs* gs, int n, int kind, hipStream_t s) {
  KArgs ka;
  std::memset(&ka, 0, sizeof(ka));
  int nt = 0;        // launch table entries used
  int64_t blk = 0;
  double flops = 0.0, bytes = 0.0;
  ka.ngroups = n;
  for (int i = 0; i < n; ++i) {
    const GemmArgs& g = gs[i];
    KGroup& k = ka.grp[i];
    k.g = static_cast<const GemmCore&>(g);
    if (uses_tbl(g)) {
      const int ne = (g.batch + g.tbl_per - 1) / g.tbl_per;
      int off = -1;
      for (int o = 0; o + ne <= nt && off < 0; ++o)   // a set of the launch with the same table
        if (std::memcmp(&ka.tbl.p[o], &g.tbl.p[0], ne * sizeof(const char*)) == 0) off = o;
      if (off < 0) {
        if (nt + ne > kTbl) return SM_ERR_UNSUPPORTED;
        std::memcpy(&ka.tbl.p[nt], &g.tbl.p[0], ne * sizeof(const char*));
        off = nt;
        nt += ne;
      }
      k.g.tbl_off = off;
    } else {
      k.g.tbl_off = 0;
    }
    k.a_aligned = operand_aligned(g, g.a, sizeof(TA) == 4 && sizeof(TM) == 4);
    k.b_aligned = operand_aligned(g, g.b, sizeof(TB) == 4 && sizeof(TM) == 4);
    const int tiles_m = (g.M + T - 1) / T;
    k.tiles_n = (g.N + T - 1) / T;
    k.tiles = g.sym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * k.tiles_n;
    k.blk_begin = (int)blk;
    blk += (int64_t)k.tiles * g.batch;
    // a symmetric product is credited the half it needs
    const double fl = (g.sym ? 1.0 : 2.0) * g.M * (double)g.N * g.K;
    const double by = (double)g.M * g.K * dt_size(g.a.dt) + (double)g.N * g.K * dt_size(g.b.dt) +
                      (double)g.M * g.N * ((g.c || g.c_tbl) ? dt_size(g.c_dt) : 0);
    if (g.pred) {  // the problems that run report their own work
      k.g.prof_exec = prof_exec_slot(kind);
      k.g.prof_flops = fl;
      k.g.prof_bytes = by;
    } else {
      k.g.prof_exec = nullptr;
      flops += fl * g.batch;
      bytes += by * g.batch;
    }
  }
  if (blk == 0) return SM_OK;
  if (blk > 0x7FFFFFFF) return SM_ERR_SHAPE;
  prof_begin(kind, flops, s, bytes);
  const dim3 grid((unsigned)blk);
  switch (kind) {
    case SM_K_GEMM_GRAM:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_GEMM_GRAM, T>), grid, dim3(NT), 0, s, ka);
      break;
    case SM_K_GEMM_APPLY:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_GEMM_APPLY, T>), grid, dim3(NT), 0, s, ka);
      break;
    case SM_K_PROBE:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_PROBE, T>), grid, dim3(NT), 0, s, ka);
      break;
    default:
      hipLaunchKernelGGL((k_gemm<TA, TB, TM, LA, LB, SM_K_GEMM_RR, T>), grid, dim3(NT), 0, s, ka);
      break;
  }
  prof_end(s);
  return check_launch();
}

// Float32 launches with fewer 128 x 128 tiles than two per CU take the 64
// tile (four times the blocks, a quarter of the k-loop work each), unless a
// set writes residual partials (they are laid out per 128 tile).
template <typename TA, typename TB, typename TM, int LA, int LB>
sm_status launch_t(const GemmArgs* gs, int n, int kind, hipStream_t s) {
  if constexpr (sizeof(TM) == 4) {
    int64_t blk = 0;
    bool need128 = false;
    for (int i = 0; i < n; ++i) {
      const GemmArgs& g = gs[i];
      const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
      blk += (g.sym ? tm * (tm + 1) / 2 : tm * tn) * g.batch;
      need128 = need128 || g.resid;
    }
    if (!need128 && blk < 2 * 256) return launch_tile<TA, TB, TM, LA, LB, 64>(gs, n, kind, s);
  }
  return launch_tile<TA, TB, TM, LA, LB, 128>(gs, n, kind, s);
}

}  // namespace gemm
}  // namespace sm
