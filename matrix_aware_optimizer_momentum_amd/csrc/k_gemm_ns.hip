// Persistent grouped bf16 GEMMs for the Newton-Schulz products.
//
// Two kernels: one for symmetric products (the Gram products X X^T, and the
// r x r products of the Gram form, whose operands are commuting symmetric
// matrices) and one for applies ((B + aI) X, X (B + aI), Q X).  One launch
// computes every product of one kind and step of the iteration over up to
// eight groups of batched problems of different shapes: C = alpha_b * A B^T
// per problem, A M x K and B N x K in the "operand" sense, fp32
// accumulation, bf16 output.
//
// Operand storage.  An operand is either k-contiguous (KC: stored rows x K,
// row-major) or k-major (KR: stored K x rows, row-major, i.e. its transpose
// is what is multiplied).  With KR the NS iterate never has to exist in both
// orientations: the wide apply reads X (m x n, contraction over m) as KR, the
// tall Gram X^T X reads X as KR on both sides.  KR fragments come out of LDS
// through the gfx950 transposing read ds_read_b64_tr_b16.
//
// Work split.  The grid is one workgroup per CU (or fewer), walking the flat
// list of 256 x 256 output tiles in rounds of gridDim tiles, in alternating
// direction (snake); workgroups of one XCD take consecutive tiles so that
// they share that XCD's L2, and within a problem the tiles go in bands of
// four tile rows, column by column (ns_tiles.hpp), so that those tiles share
// few operand panels.  Groups are ordered by the caller (largest K
// first), so concurrent tiles have similar work and the snake evens out the
// rest.
//
// Pipeline.  256 threads = 4 waves (2 x 2), each wave 128 x 128 of the tile
// as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16.  Operands go HBM -> LDS with
// direct-to-LDS loads (global_load_lds_dwordx4) into a ring of five 32 KB
// k-stages (k = 32; 160 KB, all of the CU's LDS).  Step k multiplies stage k
// in two k16 slices.  Between them each wave waits for its own loads of
// stage k + 1 and the workgroup meets at a fence-free barrier; the second
// slice then reads stage k + 1's first fragments and issues the loads of
// stage k + 4 into the buffer stage k - 1 used.  So a stage's loads have
// about two and a half steps to land.  The ring runs on across tiles: the
// next tile's first stages load during the current tile's last steps and its
// epilogue.
//
// Epilogue: value = alpha_b * acc, rounded to bf16 with v_cvt_pk_bf16_f32.
// An interior sub-tile goes out through the ring buffer of the stage just
// multiplied (free until the next tile's first barrier) in 64 x 64 chunks,
// so that every store writes whole 128-byte row segments; edge sub-tiles are
// stored element by element straight from registers.  A symmetric product
// (A == B, or two commuting symmetric matrices) computes only tiles with
// tm >= tn and stores each off-diagonal tile a second time, transposed, as
// the mirror tile, unless C is kept as its lower triangle of tiles (the
// Gram form's chain): its consumers then read a panel's entries past the
// diagonal block from the stored tiles, transposed, in k segments of fixed
// operand layouts.  In a vote step the last apply stores the packed signs
// of the values instead (wave ballots).
//
// Identity fold.  The apply X' = a X + B X gets a X from extra MFMAs in the
// k-stages that cover the output's own rows (wide: (a I) X) or columns (tall:
// X (a I)), against an a I fragment; a is split into up to two bf16 terms
// a_hi + a_lo, whose products with bf16 data are exact in fp32.  The Gram
// form's products A (B + aI) use the same fold, and (A + aI)(B + aI) folds
// the identity on both sides (plus a^2 where the two groups meet).
#include "sm_internal.hpp"

#define SM_HD __host__ __device__
#include "ns_tiles.hpp"

namespace sm {
namespace nsg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 32, NT = 256;
constexpr int NBUF = 5;          // k-stage buffers in the LDS ring (160 KB)
constexpr int HALF = 256 * BK;   // bf16 elements of one operand in a stage (16 KB)
constexpr int STG = 2 * HALF;    // a stage: A half, then B half (32 KB)

// Kernel-side group descriptor (the launcher copies NsgGroup into it).
struct Grp {
  const bf16_t* a;
  const bf16_t* b;
  bf16_t* c;
  const float* scale;
  int64_t lda, sa, ldb, sb, ldc, sc;
  int M, N, K, batch;
  int combo;          // instantiation index within the kernel's role
  int a_kr, b_kr;
  int sym;
  int ident;          // 0 none, 1 A side (wide apply), 2 B side (tall apply), 3 both
  uint32_t id_hi, id_lo;   // bf16 bits of the identity terms
  int alpha_pow;
  float alpha;
  int tiles_m, tiles_n, tiles_per_prob, tile_begin;
  int tpp_begin;               // tiles per problem of the groups before this one
  int a_tbl, b_tbl, tbl_per;   // per-matrix operand addressing (see NsgGroup)
  int a_low, b_low;            // operand stored as its lower triangle of tiles
  int c_low;                   // symmetric C: store the lower triangle only
  int tbl;                     // byte offset of the group's table in Args
  uint64_t* bits;              // apply: signs instead of C (see NsgGroup)
  int64_t bits_stride;
  int bits_s8;                 // the signs as int8 (see NsgGroup)
  const int32_t* pred;         // per-problem store predicate (see NsgGroup), or null
  float* resid;                // probe: residual partials (see NsgGroup)
  const int32_t* dyn;          // device problem list (see NsgGroup), or null
};

struct Args {
  Grp g[kNsgMaxGroups];
  PtrTbl tbl[kNsgMaxTables];
  const int32_t* gate;         // launch-wide: nothing to do while *gate == 0
  // With device problem lists (Grp::dyn): the first tile of each group's
  // listed problems and, at [kNsgMaxGroups], the launch's total, written by
  // k_dyn_prefix before the launch; tiles are laid out group by group over
  // the listed problems only.  Null: the static layout.
  const int32_t* dyn_tiles;
  double* prof_exec;           // gated launch while profiling: work added here when it runs
  double prof_flops, prof_bytes;   // per launch
  int ngroups, total_tiles, xcd_chunk;
  int tpp_total;               // tiles per problem over all groups
};
static_assert(sizeof(Args) <= 4096, "kernel arguments stay within 4 KB");

// ---------------------------------------------------------------- LDS layouts
// KC half: 256 operand rows x 64 bytes; the 16-byte k chunk c of row R sits
// at position c ^ ((R >> 2) & 3) (16 consecutive rows read at one chunk hit
// 16 distinct 4-bank groups).
// KR half: 32 k-rows x 512 bytes; the 16-byte column chunk c of k-row r sits
// at position c ^ (4 (r & 3)) (the four k-rows a transposing read touches
// land in four distinct 64-byte bank ranges).

// ---------------------------------------------------------------- lane ids
// The thread id, opaque to the optimizer.  Per-tile code (load offsets,
// fragment offsets, epilogue positions) derives its per-lane values from it
// where they are used: hoisted out of the tile loop they would stay live
// across the k loop and be spilled, and a spill reload waits for every load
// in flight.
__device__ __forceinline__ int fresh_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------- tile decode
// Tile of round r for workgroup v (of stride): rounds alternate direction, so
// with the list ordered from long to short K a workgroup that had a long tile
// in one round tends to get a short one in the next.
__device__ __forceinline__ int tile_of(int r, int v, int stride) {
  return r * stride + ((r & 1) ? stride - 1 - v : v);
}

struct Tile {
  int gi, prob, tm, tn;
};

// A wave-uniform int32 loaded through the scalar unit (counted by lgkmcnt,
// not vmcnt, so it does not wait for the loads in flight); the wait is in the
// same statement.
__device__ __forceinline__ int sload_i32(const int32_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const int32_t* q = reinterpret_cast<const int32_t*>(((uint64_t)hi << 32) | lo);
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q) : "memory");
  return v;
}

// Eight wave-uniform int32 (32-byte aligned) through the scalar unit, as
// sload_i32.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 sload_i32x8(const int32_t* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const int32_t* q = reinterpret_cast<const int32_t*>(((uint64_t)hi << 32) | lo);
  i32x8 v;
  asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q) : "memory");
  return v;
}

// Tile t of the launch; dyn: the layout over the groups' device problem
// lists (see Args::dyn_tiles), else the static one.
__device__ __forceinline__ Tile decode_tile(const Args& A, int t, bool dyn) {
  Tile r;
  int gi = 0, begin = 0;
  if (dyn) {
    const i32x8 first = sload_i32x8(A.dyn_tiles);
#pragma unroll
    for (int q = 1; q < kNsgMaxGroups; ++q)
      if (q < A.ngroups && t >= first[q]) gi = q;
#pragma unroll
    for (int q = 0; q < kNsgMaxGroups; ++q)
      if (q == gi) begin = first[q];
  } else {
#pragma unroll
    for (int q = 1; q < kNsgMaxGroups; ++q)
      if (q < A.ngroups && t >= A.g[q].tile_begin) gi = q;
    begin = A.g[gi].tile_begin;
  }
  const Grp& g = A.g[gi];
  const int local = t - begin;
  r.gi = gi;
  const int pc = local / g.tiles_per_prob;
  r.prob = dyn ? sload_i32(g.dyn + 1 + pc) : pc;
  const int u = local - pc * g.tiles_per_prob;
  ns_tile_coords(u, g.tiles_m, g.tiles_n, g.sym, &r.tm, &r.tn);   // banded walk
  return r;
}

// ---------------------------------------------------------------- DMA side
// Load q of a wave lands at 1 KB * (4 wave + q) within the stage half:
//  KC: operand rows row0 + 16 (4 wave + q) + lane / 4, k chunk of position
//      lane % 4;
//  KR: k-row 2 (4 wave + q) + lane / 32, column chunk of position lane % 32.
// Operand rows past the matrix are clamped to its last row (KC) or last
// column chunk (KR): they only feed outputs that are never stored.  The
// per-lane byte offsets are for stage 0; stage k0 adds k0 * kstride bytes
// (kstride = 2 for KC, 2 ld for KR).
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[4], int kr, int64_t ld, int row0,
                                            int rows) {
  const int tid = fresh_tid(), lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int slot = 4 * wave + q;
    if (!kr) {
      int row = row0 + 16 * slot + (lane >> 2);
      row = row < rows ? row : rows - 1;
      const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
      off[q] = (uint32_t)(2 * ((int64_t)row * ld + 8 * chunk));
    } else {
      const int krow = 2 * slot + (lane >> 5);
      int col = row0 + 8 * ((lane & 31) ^ (4 * (krow & 3)));
      col = col < rows ? col : rows - 8;
      off[q] = (uint32_t)(2 * ((int64_t)krow * ld + col));
    }
  }
}

// Load position: one group of 4 stages of one tile, with the per-lane
// offsets of that tile.
struct LoadPos {
  const char* abase;
  const char* bbase;
  uint32_t aoff[4], boff[4];
  uint32_t akst, bkst;
  int r;        // round of the tile (tile = tile_of(r, workgroup, stride))
  int kg;       // group of 4 stages within the tile
  int nkg;      // groups in the tile
  int sw;       // next group where a lower-stored operand turns to KR reads
  int dyn;      // the layout over device problem lists (Args::dyn_tiles)
  int total;    // tiles of the launch
};

// The first group past the diagonal block of panel p (256 operand rows, two
// groups of 128 k): from there on a lower-stored operand's panel entries
// (p, k) live in the stored tiles (k, p) and are read transposed (KR).
__device__ __forceinline__ int low_switch(int p, int nkg) {
  return 2 * (p + 1) < nkg ? 2 * (p + 1) : nkg;
}

// Load position: group kg of tile t (round r), with the per-lane offsets of
// the operand layouts that group reads.
__device__ __forceinline__ void load_tile_setup(LoadPos& L, const Args& A, int r, int t,
                                                int kg = 0) {
  // The tile index is wave-uniform; readfirstlane states it, so that the
  // decode and the argument reads are scalar (a vector read of the arguments
  // would wait for every load in flight).
  t = __builtin_amdgcn_readfirstlane(t);
  r = __builtin_amdgcn_readfirstlane(r);
  kg = __builtin_amdgcn_readfirstlane(kg);
  const Tile tl = decode_tile(A, t, L.dyn != 0);
  const Grp& g = A.g[tl.gi];
  // the group's table, addressed by its byte offset in the arguments (an
  // index into Args::tbl makes the compiler copy the arguments to scratch)
  const PtrTbl* tb = reinterpret_cast<const PtrTbl*>(reinterpret_cast<const char*>(&A) + g.tbl);
  L.abase = g.a_tbl ? tbl_addr(*tb, tl.prob, g.tbl_per, 2 * g.sa)
                    : reinterpret_cast<const char*>(g.a + (int64_t)tl.prob * g.sa);
  L.bbase = g.b_tbl ? tbl_addr(*tb, tl.prob, g.tbl_per, 2 * g.sb)
                    : reinterpret_cast<const char*>(g.b + (int64_t)tl.prob * g.sb);
  const int nkg = g.K / (4 * BK);
  const int asw = g.a_low ? low_switch(tl.tm, nkg) : nkg;
  const int bsw = g.b_low ? low_switch(tl.tn, nkg) : nkg;
  const int akr = g.a_kr || kg >= asw, bkr = g.b_kr || kg >= bsw;
  dma_offsets(L.aoff, akr, g.lda, tl.tm * 256, g.M);
  dma_offsets(L.boff, bkr, g.ldb, tl.tn * 256, g.N);
  L.akst = akr ? (uint32_t)(2 * g.lda) : 2u;
  L.bkst = bkr ? (uint32_t)(2 * g.ldb) : 2u;
  L.r = r;
  L.kg = kg;
  L.nkg = nkg;
  L.sw = kg < asw ? (kg < bsw && bsw < asw ? bsw : asw) : (kg < bsw ? bsw : nkg);
}

// The group after p: the next group of the same tile, else the first group of
// the workgroup's next tile; past the last tile p itself (its stages are then
// loaded again into buffers that are never multiplied).
__device__ __forceinline__ void load_advance(LoadPos& p, const Args& A, int vid, int stride) {
  if (p.kg + 1 < p.nkg && p.kg + 1 != p.sw) {
    ++p.kg;
  } else {
    // the next tile, or the same tile where an operand turns to KR reads
    // (one setup for both, so that it is inlined once)
    const bool next = p.kg + 1 >= p.nkg;
    const int r = next ? p.r + 1 : p.r;
    const int nt = tile_of(r, vid, stride);
    if (nt < p.total) load_tile_setup(p, A, r, nt, next ? 0 : p.kg + 1);
  }
}

// One direct-to-LDS load: each lane's 16 bytes at base + voff land at LDS
// byte address m0 + 16 lane.  Issued from inline assembly so that the
// compiler, which cannot tell which LDS bytes a pending load writes, does not
// add a wait for all of them before every LDS read: the kernel's own
// s_waitcnt vmcnt and barriers order the buffers (see the pipeline notes).
// The instruction has no register result; M0 is set one wait state ahead.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, uint32_t m0) {
  // The operands are wave-uniform; readfirstlane makes them scalar registers.
  // It returns int: each half goes through uint32_t so that the low half is
  // zero-extended (a sign-extended low half would corrupt the high bits).
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t sm0 = (uint32_t)__builtin_amdgcn_readfirstlane(m0);
  // The hazard recognizer does not look inside inline asm, so the asm keeps
  // its own wait states: 5 between a VALU write of an SGPR (the readfirstlane
  // of the base, which the compiler may place just before) and a memory
  // instruction reading it, and 1 between writing M0 and the LDS DMA.
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(sm0)
               : "memory", "m0");
}

// LDS byte address of a shared array.
__device__ __forceinline__ uint32_t lds_addr(const bf16_t* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// Load q (0..3: A, 4..7: B) of this wave's share of stage s (0..3) of the
// group at L into the stage buffer at LDS byte address sbuf; wbase is this
// wave's first slot (4 wave KB).
__device__ __forceinline__ void dma_load(uint32_t sbuf, uint32_t wbase, const LoadPos& L, int s,
                                         int q) {
  const uint32_t k0 = (uint32_t)(L.kg * 4 * BK + s * BK);
  if (q < 4)
    dma16(L.abase, L.aoff[q] + k0 * L.akst, sbuf + wbase + 1024u * q);
  else
    dma16(L.bbase, L.boff[q - 4] + k0 * L.bkst, sbuf + 2u * HALF + wbase + 1024u * (q - 4));
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt low
// bits 3:0 and high bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// A wave-uniform float loaded through the scalar unit (counted by lgkmcnt,
// not vmcnt, so it does not wait for the loads in flight); the wait is in the
// same statement.
__device__ __forceinline__ float scalar_load(const float* p) {
  // the address is wave-uniform; readfirstlane states it for the compiler
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const float* q = reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
  float v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q) : "memory");
  return v;
}

// A wave-uniform int32 loaded through the scalar unit (see scalar_load).
__device__ __forceinline__ int scalar_load_i32(const int32_t* p) {
  return __builtin_bit_cast(int, scalar_load(reinterpret_cast<const float*>(p)));
}

// Workgroup barrier without a memory fence (no wait for outstanding direct-
// to-LDS loads); the empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- fragments
struct Frags {
  bf16x8 a[4], b[4];
};

// Per-lane LDS element offsets of the fragment reads of one operand half for
// this wave's rows rbase.. (128 rows = 4 blocks of 32): KC uses one offset
// per k16 slice (block i adds 32 rows = i * 32 * BK elements); KR uses one
// per (block, read) pair (slice s adds 16 k-rows = s * 16 * 256 elements).
// Only the layout's own offsets are computed, per tile, so that they are not
// live across the epilogue.
template <int KR>
struct FragOffs;

template <>
struct FragOffs<0> {
  int kc[2];
  __device__ __forceinline__ explicit FragOffs(int rbase) {
    const int lane = fresh_tid() & 63;
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int R = rbase + lr, c = 2 * s + lk;
      kc[s] = R * BK + 8 * (c ^ ((R >> 2) & 3));
    }
  }
};

template <>
struct FragOffs<1> {
  int kr[4][2];
  __device__ __forceinline__ explicit FragOffs(int rbase) {
    const int lane = fresh_tid() & 63;
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int krow = 8 * (g >> 1) + 4 * r + (j >> 2);
        const int col = rbase + 32 * i + 16 * (g & 1) + 4 * (j & 3);
        const int chunk = (col >> 3) ^ (4 * (krow & 3));
        kr[i][r] = krow * 256 + 8 * chunk + (col & 7);
      }
  }
};

// Fragment of block i (32 operand rows), k16 slice s, of an operand half.
template <int KR>
__device__ __forceinline__ bf16x8 frag(const bf16_t* H, const FragOffs<KR>& f, int i, int s) {
  if constexpr (!KR) {
    return *reinterpret_cast<const bf16x8*>(H + f.kc[s] + i * 32 * BK);
  } else {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const bf16_t* p0 = H + f.kr[i][0] + s * 16 * 256;
    const bf16_t* p1 = H + f.kr[i][1] + s * 16 * 256;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(__attribute__((address_space(3))) void*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(__attribute__((address_space(3))) void*)(p1));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(l2.x, l2.y, h2.x, h2.y));
  }
}

// Identity fragment for k16 slice `half` of the 32-index block a stage of the
// identity group covers: lane l supplies index l % 32 and k = 16 half +
// 8 (l / 32) + e; the element is `bits` where they agree.
__device__ __forceinline__ bf16x8 ident_frag(int half, uint32_t bits) {
  const int lane = fresh_tid() & 63;
  const int e = (lane & 31) - 16 * half - 8 * (lane >> 5);
  // selects on lane conditions only (the compiler keeps them as scalar lane
  // masks), so that nothing per lane has to stay live across the k loop
  const uint32_t v = (e & 1) ? bits << 16 : bits;
  const bool in = e >= 0 && e < 8;
  const uint32_t w0 = (in && (e >> 1) == 0) ? v : 0u;
  const uint32_t w1 = (in && (e >> 1) == 1) ? v : 0u;
  const uint32_t w2 = (in && (e >> 1) == 2) ? v : 0u;
  const uint32_t w3 = (in && (e >> 1) == 3) ? v : 0u;
  return __builtin_bit_cast(bf16x8, make_uint4(w0, w1, w2, w3));
}

// The identity terms of a tile: bf16 bit patterns of a_hi and a_lo.
struct Ident {
  uint32_t hi, lo;
};

// Identity fragments of the two k16 slices (a_hi, and a_lo for two terms),
// built once when a tile reaches its identity group.  With the identity on
// both sides (one term), h is the A side's fragment and l the B side's,
// each zero when the group does not carry that side.
struct IdFrags {
  bf16x8 h[2], l[2];
};

#define SM_MFMA(A_, B_, C_) C_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_, B_, C_, 0, 0, 0)

// Identity MFMAs of slice s for block IB.
template <int IDM, int IDT, int IB>
__device__ __forceinline__ void ident_mma(f32x16 (&acc)[4][4], const Frags& f,
                                          const IdFrags& idf, int s) {
  if constexpr (IDM == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) SM_MFMA(idf.h[s], f.b[j], acc[IB][j]);
    if constexpr (IDT == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) SM_MFMA(idf.l[s], f.b[j], acc[IB][j]);
    }
  } else if constexpr (IDM == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) SM_MFMA(f.a[i], idf.h[s], acc[i][IB]);
    if constexpr (IDT == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) SM_MFMA(f.a[i], idf.l[s], acc[i][IB]);
    }
  } else if constexpr (IDM == 3) {
    // (A + aI)(B + aI) = AB + aB + aA + a^2 I, one term: the A side's
    // group covers the wave's rows, the B side's its columns, and where
    // both coincide the a^2 term lands on the diagonal of block (IB, IB).
    // All nine MFMAs run, against zero fragments for a side the group does
    // not carry: under a lane-mask branch the compiler may leave out the
    // skip, and an MFMA issued with no active lanes still accumulates.
    static_assert(IDT == 1, "both-sided identity takes one term");
#pragma unroll
    for (int j = 0; j < 4; ++j) SM_MFMA(idf.h[s], f.b[j], acc[IB][j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) SM_MFMA(f.a[i], idf.l[s], acc[i][IB]);
    SM_MFMA(idf.h[s], idf.l[s], acc[IB][IB]);
  }
}

// One step of the main loop (stage k in buffer cur): the two k16 slices'
// MFMAs, each followed by at most two memory instructions:
//   slice 0 (f0): reads of this stage's slice-1 fragments into f1;
//   then this wave waits for its own loads of stage k + 1 (wait_lenient: a
//   count that an epilogue's stores make safe, see run_tile) and the
//   workgroup meets at a fence-free barrier;
//   slice 1 (f1): reads of stage k + 1's slice-0 fragments into f0, and this
//   wave's direct-to-LDS loads of stage k + 4 (stage ls of the group at L)
//   into buffer ldb, the one stage k - 1 used: every wave is past the
//   barrier, so its MFMAs of stage k - 1 have consumed their reads.
// sched_barrier keeps the compiler from regrouping them (hoisting the reads
// would need a second set of fragment registers).  A KR fragment takes two
// transposing reads.
template <int AKR, int BKR, int IDM, int IDT, int IB>
__device__ __forceinline__ void nsg_step(f32x16 (&acc)[4][4], Frags& f0, Frags& f1,
                                         const bf16_t* cur, const bf16_t* nxt, uint32_t ldb,
                                         uint32_t wbase, const LoadPos& L, int ls,
                                         const FragOffs<AKR>& fa, const FragOffs<BKR>& fb,
                                         const IdFrags& idf, bool wait_lenient) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    SM_MFMA(f0.a[i], f0.b[j], acc[i][j]);
    if (q < 4) f1.a[q] = frag<AKR>(cur, fa, q, 1);
    else if (q < 8) f1.b[q - 4] = frag<BKR>(cur + HALF, fb, q - 4, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  ident_mma<IDM, IDT, IB>(acc, f0, idf, 0);
  __builtin_amdgcn_sched_barrier(0);
  // stage k + 1 must have landed; in steady state the loads of stages k + 2
  // and k + 3 (16) follow it, after an epilogue also its >= 32 stores
  if (wait_lenient) wait_vm<48>(); else wait_vm<16>();
  barrier_nofence();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int i = q >> 2, j = q & 3;
    SM_MFMA(f1.a[i], f1.b[j], acc[i][j]);
    if (q < 4) f0.a[q] = frag<AKR>(nxt, fa, q, 0);
    else if (q < 8) f0.b[q - 4] = frag<BKR>(nxt + HALF, fb, q - 4, 0);
    else dma_load(ldb, wbase, L, ls, q - 8);
    __builtin_amdgcn_sched_barrier(0);
  }
  ident_mma<IDM, IDT, IB>(acc, f1, idf, 1);
}

// The k loop of one tile: nk / 4 groups of 4 steps.  Stages live in a ring
// of NBUF buffers that runs on across tiles: cb is the buffer of the current
// stage.  Step s of group kg loads stage s of the group after it (the load
// position LP is one group ahead: group kg + 1, or the first group of the
// workgroup's next tile), so LP moves on after step 3.  `lenient`: the tile
// follows an epilogue, which issued at least 32 stores after the loads of
// the tile's first stages (or drained them all), so in the tile's first
// three steps at least 48 operations follow the stage being waited for
// (16 stage loads and 32 stores) and vmcnt <= 48 implies it has landed.
// Groups kg0 .. kg1 - 1 of a tile, all read with layouts (AKR, BKR).
template <int AKR, int BKR, int IDM, int IDT>
__device__ __forceinline__ void run_groups(f32x16 (&acc)[4][4], Frags& f0, Frags& f1,
                                           const bf16_t* smem, uint32_t la0, int& cb,
                                           uint32_t wbase, LoadPos& LP, const Args& A, int vid,
                                           int stride, int kg0, int kg1, int id_g, int wm,
                                           int wn, const Ident& id, bool lenient) {
  if (kg0 >= kg1) return;
  const FragOffs<AKR> fa(wm * 128);
  const FragOffs<BKR> fb(wn * 128);
  // slice 0 of the first stage (the step before read it with the layouts of
  // the previous tile or segment, so it is read again with these)
  {
    const bf16_t* c0 = smem + cb * STG;
#pragma unroll
    for (int i = 0; i < 4; ++i) f0.a[i] = frag<AKR>(c0, fa, i, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) f0.b[i] = frag<BKR>(c0 + HALF, fb, i, 0);
  }
  for (int kg = kg0; kg < kg1; ++kg) {
#define SM_NSG_STEP(S_, IDM_)                                                               \
    {                                                                                       \
      const int nb = cb == NBUF - 1 ? 0 : cb + 1;                                           \
      const int lb = cb == 0 ? NBUF - 1 : cb - 1;                                           \
      nsg_step<AKR, BKR, IDM_, IDT, S_>(acc, f0, f1, smem + cb * STG, smem + nb * STG,      \
                                        la0 + (uint32_t)(lb * STG * 2), wbase, LP, S_, fa,  \
                                        fb, idf, lenient && kg == 0 && (S_) < 3);           \
      cb = nb;                                                                              \
    }
#define SM_NSG_GROUP(IDM_) \
    SM_NSG_STEP(0, IDM_)   \
    SM_NSG_STEP(1, IDM_)   \
    SM_NSG_STEP(2, IDM_)   \
    SM_NSG_STEP(3, IDM_)
    if constexpr (IDM == 3) {   // id_g: the A side's group | the B side's << 16
      const bool ia = kg == (id_g & 0xffff), ib = kg == (id_g >> 16);
      if (ia || ib) {
        IdFrags idf;
        const bf16x8 z{};
        idf.h[0] = ia ? ident_frag(0, id.hi) : z;
        idf.h[1] = ia ? ident_frag(1, id.hi) : z;
        idf.l[0] = ib ? ident_frag(0, id.hi) : z;
        idf.l[1] = ib ? ident_frag(1, id.hi) : z;
        SM_NSG_GROUP(3)
      } else {
        IdFrags idf;   // not read: the group has no identity MFMAs
        SM_NSG_GROUP(0)
      }
    } else if constexpr (IDM != 0) {
      if (kg == id_g) {
        IdFrags idf;
        idf.h[0] = ident_frag(0, id.hi);
        idf.h[1] = ident_frag(1, id.hi);
        if constexpr (IDT == 2) {
          idf.l[0] = ident_frag(0, id.lo);
          idf.l[1] = ident_frag(1, id.lo);
        }
        SM_NSG_GROUP(IDM)
      } else {
        IdFrags idf;   // not read: the group has no identity MFMAs
        SM_NSG_GROUP(0)
      }
    } else {
      IdFrags idf;
      SM_NSG_GROUP(0)
    }
#undef SM_NSG_GROUP
#undef SM_NSG_STEP
    // after step 3 the load position moves on; outside the identity branch,
    // whose condition the compiler takes for divergent, the next tile's
    // arguments stay scalar loads
    load_advance(LP, A, vid, stride);
  }
}

template <int AKR, int BKR, int IDM, int IDT>
__device__ __forceinline__ void run_tile(f32x16 (&acc)[4][4], Frags& f0, Frags& f1,
                                         const bf16_t* smem, uint32_t la0, int& cb,
                                         uint32_t wbase, LoadPos& LP, const Args& A, int vid,
                                         int stride, int nkg, int id_g, int wm, int wn,
                                         const Ident& id, bool lenient) {
  run_groups<AKR, BKR, IDM, IDT>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, 0, nkg,
                                 id_g, wm, wn, id, lenient);
}

// A tile with lower-stored operands: k segments of fixed layouts, split where
// an operand's panel passes its diagonal block (asw for A, bsw for B; see
// low_switch).  LOW 3: both operands (symmetric tile, tn <= tm, so B turns
// first); 1: A only, B KR; 2: B only, A KC.  The identity group of a panel
// lies in its diagonal block, before that panel's switch: a B-side (or a
// one-operand) identity falls in the first segment; with the identity on
// both sides (IDM 3) the A side's group may fall in the second.
template <int LOW, int IDM, int IDT>
__device__ __forceinline__ void run_tile_low(f32x16 (&acc)[4][4], Frags& f0, Frags& f1,
                                             const bf16_t* smem, uint32_t la0, int& cb,
                                             uint32_t wbase, LoadPos& LP, const Args& A,
                                             int vid, int stride, int nkg, int asw, int bsw,
                                             int id_g, int wm, int wn, const Ident& id,
                                             bool lenient) {
  static_assert(LOW != 3 || IDM != 1, "an A-side identity group may follow B's switch");
  if constexpr (LOW == 3) {
    run_groups<0, 0, IDM, IDT>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, 0, bsw,
                               id_g, wm, wn, id, lenient);
    run_groups<0, 1, IDM == 3 ? 3 : 0, IDT>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid,
                                            stride, bsw, asw, id_g, wm, wn, id, false);
    run_groups<1, 1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, asw, nkg,
                           id_g, wm, wn, id, false);
  } else if constexpr (LOW == 1) {
    run_groups<0, 1, IDM, IDT>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, 0, asw,
                               id_g, wm, wn, id, lenient);
    run_groups<1, 1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, asw, nkg,
                           id_g, wm, wn, id, false);
  } else {
    run_groups<0, 0, IDM, IDT>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, 0, bsw,
                               id_g, wm, wn, id, lenient);
    run_groups<0, 1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, bsw, nkg,
                           id_g, wm, wn, id, false);
  }
}

// ---------------------------------------------------------------- epilogue
// Quad permutes (every lane written: no old value needed).
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t cvt2(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8-byte store; STREAM marks it non-temporal (for outputs too large to be
// read back from the caches).
template <bool STREAM>
__device__ __forceinline__ void st8(bf16_t* p, uint2 v) {
  if constexpr (STREAM) {
    __builtin_nontemporal_store(v.x, reinterpret_cast<uint32_t*>(p));
    __builtin_nontemporal_store(v.y, reinterpret_cast<uint32_t*>(p) + 1);
  } else {
    *reinterpret_cast<uint2*>(p) = v;
  }
}

// 16-byte store; STREAM marks it non-temporal.
template <bool STREAM>
__device__ __forceinline__ void st16(bf16_t* p, uint4 v) {
  if constexpr (STREAM) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    __builtin_nontemporal_store(v.x, q);
    __builtin_nontemporal_store(v.y, q + 1);
    __builtin_nontemporal_store(v.z, q + 2);
    __builtin_nontemporal_store(v.w, q + 3);
  } else {
    *reinterpret_cast<uint4*>(p) = v;
  }
}

// Stores this wave's interior 128 x 128 sub-tile (origin wr0, wc0) of
// alpha * acc (SCALE false: alpha is 1), or with TRANSPOSED its mirror copy
// (the sub-tile transposed, at (wc0, wr0)), through LDS: four 64 x 64 chunks
// pass through the wave's 8 KB `stage`, written as 8-byte pieces and read
// back as 16-byte row pieces, so that every global store instruction writes
// 8 whole 128-byte row segments.  Straight from registers a store covered
// 64 bytes of 8 rows (normal) or 16 bytes of 32 rows (mirror).  Chunk
// layout: 64 rows of 128 bytes, the 16-byte piece c of row R at position
// c ^ (R & 7).  One wave's LDS accesses execute in order, so the read-back
// sees the chunk's writes and the next chunk's writes follow the reads.
// Issues 32 global stores.
template <bool SCALE, bool STREAM, bool TRANSPOSED>
__device__ __forceinline__ void store_staged(const f32x16 (&acc)[4][4], bf16_t* C, int64_t ldc,
                                             int wr0, int wc0, float alpha, bf16_t* stage) {
  const int lane = fresh_tid() & 63;
  const int lr = lane & 31, lq = (lane >> 5) * 4;
  const int cm = lane & 3;
  const int rsel = ((cm & 1) << 1) | (cm >> 1);   // which of the 4 rows this lane ends with
  const int colq = lr & ~3;
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int J = 0; J < 2; ++J) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // rows i*32 + q*8 + lq + {0,1} (v0) and {2,3} (v1) of column j*32 + lr
            const f32x16& a = acc[2 * I + ii][2 * J + jj];
            uint32_t v0, v1;
            if constexpr (SCALE) {
              v0 = cvt2(alpha * a[q * 4 + 0], alpha * a[q * 4 + 1]);
              v1 = cvt2(alpha * a[q * 4 + 2], alpha * a[q * 4 + 3]);
            } else {
              v0 = cvt2(a[q * 4 + 0], a[q * 4 + 1]);
              v1 = cvt2(a[q * 4 + 2], a[q * 4 + 3]);
            }
            int R, c, off;
            uint2 piece;
            if constexpr (TRANSPOSED) {
              // the 4 rows are 4 consecutive entries of mirror row jj*32 + lr
              R = jj * 32 + lr;
              c = ii * 4 + q;
              off = lq;
              piece = make_uint2(v0, v1);
            } else {
              // two rounds of quad shuffles: 1 row x 4 columns per lane
              const uint32_t recv = dpp_xor1((cm & 1) ? v0 : v1);
              const uint32_t mine = (cm & 1) ? v1 : v0;
              const uint32_t lo = (cm & 1) ? recv : mine;              // lower column
              const uint32_t hi = (cm & 1) ? mine : recv;
              const uint32_t ra = (lo & 0xFFFFu) | (hi << 16);          // first row, 2 columns
              const uint32_t rb = (lo >> 16) | (hi & 0xFFFF0000u);      // second row, 2 columns
              const uint32_t r2 = dpp_xor2((cm < 2) ? rb : ra);
              const uint32_t keep = (cm < 2) ? ra : rb;
              piece = (cm < 2) ? make_uint2(keep, r2) : make_uint2(r2, keep);
              R = ii * 32 + q * 8 + lq + rsel;
              const int col = jj * 32 + colq;
              c = col >> 3;
              off = col & 4;
            }
            *reinterpret_cast<uint2*>(stage + R * 64 + ((c ^ (R & 7)) * 8) + off) = piece;
            // one piece at a time keeps few values live (the k loop's
            // registers are all taken)
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int R = t * 8 + (lane >> 3), c = lane & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + R * 64 + ((c ^ (R & 7)) * 8));
        bf16_t* p = TRANSPOSED ? C + (int64_t)(wc0 + J * 64 + R) * ldc + (wr0 + I * 64 + c * 8)
                               : C + (int64_t)(wr0 + I * 64 + R) * ldc + (wc0 + J * 64 + c * 8);
        st16<STREAM>(p, v);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
}

// Stores a sub-tile that is not wholly inside C, element-checked (and its
// mirror copy when `mirror`), straight from registers: two rounds of quad
// DPP shuffles give each lane 1 row x 4 columns; the mirror's 4 rows are 4
// consecutive entries of one row.
template <bool SCALE, bool STREAM>
__device__ __forceinline__ void epilogue_edge(const f32x16 (&acc)[4][4], bf16_t* C, int64_t ldc,
                                              int M, int N, int wr0, int wc0, float alpha,
                                              bool mirror) {
  const int lane = fresh_tid() & 63;
  const int lr = lane & 31, lq = (lane >> 5) * 4;
  const int cm = lane & 3;
  const int rsel = ((cm & 1) << 1) | (cm >> 1);
  const int colq = lr & ~3;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v0, v1;
        if constexpr (SCALE) {
          v0 = cvt2(alpha * acc[i][j][q * 4 + 0], alpha * acc[i][j][q * 4 + 1]);
          v1 = cvt2(alpha * acc[i][j][q * 4 + 2], alpha * acc[i][j][q * 4 + 3]);
        } else {
          v0 = cvt2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]);
          v1 = cvt2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
        }
        if (!STREAM && mirror) {
          const int trow = wc0 + j * 32 + lr, tcol = wr0 + i * 32 + q * 8 + lq;
          bf16_t* p = C + (int64_t)trow * ldc + tcol;
          if (trow < N) {
            const uint32_t w[2] = {v0, v1};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (tcol + e < M) p[e] = (bf16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
        const uint32_t recv = dpp_xor1((cm & 1) ? v0 : v1);
        const uint32_t mine = (cm & 1) ? v1 : v0;
        const uint32_t lo = (cm & 1) ? recv : mine;
        const uint32_t hi = (cm & 1) ? mine : recv;
        const uint32_t ra = (lo & 0xFFFFu) | (hi << 16);
        const uint32_t rb = (lo >> 16) | (hi & 0xFFFF0000u);
        const uint32_t r2 = dpp_xor2((cm < 2) ? rb : ra);
        const uint32_t keep = (cm < 2) ? ra : rb;
        const uint2 out = (cm < 2) ? make_uint2(keep, r2) : make_uint2(r2, keep);
        const int row = wr0 + i * 32 + q * 8 + lq + rsel;
        const int col = wc0 + j * 32 + colq;
        bf16_t* p = C + (int64_t)row * ldc + col;
        if (row < M) {
          if (col + 4 <= N) {
            st8<STREAM>(p, out);
          } else {
            const uint32_t w[2] = {out.x, out.y};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < N) p[e] = (bf16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
}

// The wave's sub-tile lies wholly inside C or not; readfirstlane states that
// this is wave-uniform, so the choice is one scalar branch per tile.  An
// interior sub-tile goes out through LDS (`stage`: this wave's 8 KB of the
// free ring buffer; the caller has met the workgroup at a barrier, so every
// wave is past its reads of it), 32 stores, 64 with the mirror copy (the
// symmetric kernel's off-diagonal tiles); an edge sub-tile is stored element
// by element and the wave's memory operations drained, so that the next
// tile's first waits hold (see run_tile).
template <bool SCALE, bool STREAM>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[4][4], bf16_t* C, int64_t ldc, int M,
                                         int N, int wr0, int wc0, float alpha, bool mirror,
                                         bf16_t* stage) {
  const int inside =
      __builtin_amdgcn_readfirstlane((wr0 + 128 <= M && wc0 + 128 <= N) ? 1 : 0);
  if (inside) {
    store_staged<SCALE, STREAM, false>(acc, C, ldc, wr0, wc0, alpha, stage);
    if constexpr (!STREAM) {
      if (mirror) store_staged<SCALE, false, true>(acc, C, ldc, wr0, wc0, alpha, stage);
    }
  } else {
    epilogue_edge<SCALE, STREAM>(acc, C, ldc, M, N, wr0, wc0, alpha, mirror);
    wait_vm<0>();
  }
}

// The probe's epilogue: this wave's part of sum (alpha * acc - [row == col])^2
// over the entries inside M x N, times `weight`, as one float at *out (a
// vector store from lane 0); the wave's memory operations are drained, so
// that the next tile's first waits hold (see run_tile).
__device__ __forceinline__ void epilogue_resid(const f32x16 (&acc)[4][4], float* out, int M,
                                               int N, int wr0, int wc0, float alpha,
                                               float weight) {
  const int lane = fresh_tid() & 63;
  const int lr = lane & 31, lq = (lane >> 5) * 4;
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wr0 + 32 * i + 8 * (v >> 2) + lq + (v & 3);
        const int col = wc0 + 32 * j + lr;
        if (row < M && col < N) {
          const float d = __fsub_rn(__fmul_rn(alpha, acc[i][j][v]), row == col ? 1.f : 0.f);
          part = __fmaf_rn(d, d, part);
        }
      }
  // butterfly over the wave; the lane id comes from fresh_tid (a shuffle
  // builtin would derive its own, which the compiler hoists and spills)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int other = __builtin_amdgcn_ds_bpermute((lane ^ o) << 2, __float_as_int(part));
    part = __fadd_rn(part, __int_as_float(other));
  }
  if (lane == 0) *out = __fmul_rn(weight, part);
  wait_vm<0>();
}

// The writelane intrinsic, which this compiler exposes under no builtin
// name.  Going through the intrinsic (not inline asm) keeps the instruction
// visible to the hazard recognizer: v_writelane reads its value from an SGPR
// that the ballot's compare has just written, and needs wait states after it.
extern "C" __device__ int sm_llvm_writelane(int val, int lane, int old)
    __asm("llvm.amdgcn.writelane.i32");

// v[lane] = val (val wave-uniform, lane a constant): v_writelane_b32.
template <int LANE>
__device__ __forceinline__ uint32_t writelane(uint32_t v, uint32_t val) {
  return (uint32_t)sm_llvm_writelane((int)val, LANE, (int)v);
}

// Four int8 signs from four sign bits (bit e set <=> byte e is -1, else +1):
// each bit is moved to the low bit of its byte and scaled by 0xFE, so that
// 0x01 + 0xFE = 0xFF; no byte carries into the next.
__device__ __forceinline__ uint32_t s8x4_of_bits(uint32_t b) {
  const uint32_t spread = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
  return 0x01010101u + 0xFEu * spread;
}

// Writes the signs of this wave's 128 x 128 sub-tile of alpha * acc as packed
// bits (the sign of each value rounded to bf16 exactly as epilogue() rounds
// it, so the bits equal the sign packing of the stored direction): bit = 1
// <=> negative, 64 consecutive columns of a row per 64-bit word (N % 64 ==
// 0, wpr = N / 64 words per row).  A ballot over one accumulator register
// gives 32 columns of two rows (lanes 0-31: row r, 32-63: row r + 4); two
// column blocks make one word per row, placed with writelane into the lane
// that stores it (lane L: row L % 32 of the block, word L / 32).  Issues 4
// stores, then drains this wave's memory operations (fewer stores than the
// lenient wait after a plain epilogue assumes).  S8: the lane expands its
// word into the 64 int8 signs of those entries instead (-1 iff negative,
// else +1; row pitch N bytes from s8) and stores them as four 16-byte
// vectors, 16 stores per wave.
template <bool SCALE, bool S8>
__device__ __forceinline__ void epilogue_bits(const f32x16 (&acc)[4][4], uint64_t* bits,
                                              int8_t* s8, int64_t wpr, int M, int N, int wr0,
                                              int wc0, float alpha) {
  const int lane = fresh_tid() & 63;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t wlo = 0u, whi = 0u;   // this lane's word
    // p: word (columns 64p..64p+63 of the sub-tile); q, e: accumulator
    // register q*4 + e of blocks (i, 2p) and (i, 2p + 1)
#define SM_BITS_QE(P, Q, E)                                                                \
    {                                                                                      \
      float a0 = acc[i][2 * (P)][(Q) * 4 + (E)], a1 = acc[i][2 * (P)][(Q) * 4 + (E) + 1];  \
      float b0 = acc[i][2 * (P) + 1][(Q) * 4 + (E)];                                       \
      float b1 = acc[i][2 * (P) + 1][(Q) * 4 + (E) + 1];                                   \
      if constexpr (SCALE) {                                                               \
        a0 *= alpha; a1 *= alpha; b0 *= alpha; b1 *= alpha;                                \
      }                                                                                    \
      const uint32_t ha = cvt2(a0, a1), hb = cvt2(b0, b1);                                 \
      SM_BITS_H(P, Q, E, 0, ha << 16, hb << 16)                                            \
      SM_BITS_H(P, Q, E, 1, ha & 0xFFFF0000u, hb & 0xFFFF0000u)                            \
    }
    /* register e + h: rows q*8 + e + h (lanes 0-31) and q*8 + 4 + e + h (lanes 32-63) */
#define SM_BITS_H(P, Q, E, H, XA, XB)                                                      \
    {                                                                                      \
      const uint64_t ma = __builtin_amdgcn_ballot_w64(__uint_as_float(XA) < 0.f);          \
      const uint64_t mb = __builtin_amdgcn_ballot_w64(__uint_as_float(XB) < 0.f);          \
      constexpr int L0 = (P) * 32 + (Q) * 8 + (E) + (H);                                   \
      wlo = writelane<L0>(wlo, (uint32_t)ma);                                              \
      whi = writelane<L0>(whi, (uint32_t)mb);                                              \
      wlo = writelane<L0 + 4>(wlo, (uint32_t)(ma >> 32));                                  \
      whi = writelane<L0 + 4>(whi, (uint32_t)(mb >> 32));                                  \
    }
#define SM_BITS_Q(P, Q) SM_BITS_QE(P, Q, 0) SM_BITS_QE(P, Q, 2)
#define SM_BITS_P(P) SM_BITS_Q(P, 0) SM_BITS_Q(P, 1) SM_BITS_Q(P, 2) SM_BITS_Q(P, 3)
    SM_BITS_P(0)
    SM_BITS_P(1)
#undef SM_BITS_P
#undef SM_BITS_Q
#undef SM_BITS_H
#undef SM_BITS_QE
    const int row = wr0 + i * 32 + (lane & 31);
    const int col = wc0 + 64 * (lane >> 5);
    if (row < M && col < N) {
      if constexpr (S8) {
        // columns col .. col + 63 (N % 64 == 0: all inside the row)
        uint4* dst = reinterpret_cast<uint4*>(s8 + (int64_t)row * N + col);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t b16 = ((c < 2 ? wlo : whi) >> (16 * (c & 1))) & 0xFFFFu;
          dst[c] = make_uint4(s8x4_of_bits(b16 & 15u), s8x4_of_bits((b16 >> 4) & 15u),
                              s8x4_of_bits((b16 >> 8) & 15u), s8x4_of_bits(b16 >> 12));
        }
      } else {
        *reinterpret_cast<uint2*>(bits + (int64_t)row * wpr + (col >> 6)) = make_uint2(wlo, whi);
      }
    }
  }
  wait_vm<0>();
}

// ---------------------------------------------------------------- kernel
// Two kernels: one for symmetric products (Gram products and the r x r
// products), one for applies.  Combos per kernel (index = Grp::combo):
// operand layouts and identity mode.
//   SYM:   0 (KC, KC)        1 (KR, KR)
//          2 (KC, KC, B-side id, 1 term)   3 (KC, KC, B-side id, 2 terms)
//          4 (KC, KR, A-side id, 1 term)
//          5 (both lower-stored, B-side id, 1 term)
//          6 (both lower-stored, id on both sides, 1 term)
//          (2 to 4 also take plain applies riding along: tall 2/3, wide 4)
//   APPLY: 0 (KC, KR, A-side id, 1 term)   1 (KC, KC, B-side id, 1 term)
//          2 (KC, KR, A-side id, 2 terms)  3 (KC, KC, B-side id, 2 terms)
//          4 (KC, KR)        5 (KC, KC)
//          6 (A lower-stored, KR)          7 (KC, B lower-stored)
//   PROBE: 0 (KC, KC)       1 (KR, KR)    (symmetric, residual epilogue)
constexpr int ROLE_SYM = 0, ROLE_APPLY = 1, ROLE_PROBE = 2;
template <int ROLE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_ns(Args args) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[NBUF * STG];
  // Read in place from the kernel argument segment, where args is the only
  // explicit argument (offset 0).  Through the parameter itself the compiler
  // copied all of Args to scratch once the kernel had grown past some size.
  (void)args;
  const Args& A = *(const Args*)(__builtin_amdgcn_kernarg_segment_ptr());
  int vid = blockIdx.x;
  if (A.xcd_chunk > 0) vid = (vid & 7) * A.xcd_chunk + (vid >> 3);
  const int stride = gridDim.x;
  int round = 0;
  int t = tile_of(0, vid, stride);
  if (t >= A.total_tiles) return;
  if (A.gate && scalar_load_i32(A.gate) == 0) return;   // uniform over the launch
  const bool dyn = A.dyn_tiles != nullptr;
  int total = A.total_tiles;
  if (dyn) {
    total = sload_i32(A.dyn_tiles + kNsgMaxGroups);
    if (t >= total) return;
  }
  // (with problem lists k_dyn_prefix credits the work of the listed problems)
  if (A.prof_exec && !dyn && blockIdx.x == 0 && threadIdx.x == 0) {
    atomicAdd(A.prof_exec, A.prof_flops);
    atomicAdd(A.prof_exec + 1, A.prof_bytes);
  }

  const int wave = threadIdx.x >> 6;

  // LDS byte address of the ring and of this wave's load slots
  const uint32_t la0 = lds_addr(smem);
  const uint32_t wbase = 4096u * (uint32_t)__builtin_amdgcn_readfirstlane(wave);
  // prologue: the first tile's stages 0..3 into buffers 0..3; the load
  // position then moves one group ahead
  LoadPos LP;
  LP.dyn = dyn ? 1 : 0;
  LP.total = total;
  load_tile_setup(LP, A, 0, t);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int q = 0; q < 8; ++q) dma_load(la0 + (uint32_t)(s * STG * 2), wbase, LP, s, q);
  load_advance(LP, A, vid, stride);
  wait_vm<24>();   // stage 0 of this wave
  barrier_nofence();
  int cb = 0;
  Frags f0, f1;
  f0.a[0] = f0.a[1] = f0.a[2] = f0.a[3] = bf16x8{};
  f0.b[0] = f0.b[1] = f0.b[2] = f0.b[3] = bf16x8{};
  f1 = f0;

  bool lenient = false;
  for (;;) {
    const Tile tc = decode_tile(A, t, dyn);
    const Grp& g = A.g[tc.gi];
    const int nkg = g.K / (4 * BK);
    // this wave's 128 x 128 quarter (wm, wn) of the tile, derived again after
    // the k loop rather than kept live across it
    int wm = (fresh_tid() >> 6) >> 1, wn = (fresh_tid() >> 6) & 1;
    // identity group of this wave: the 128 k-indices equal to its rows / columns
    const int id_g = g.ident == 1   ? 2 * tc.tm + wm
                     : g.ident == 2 ? 2 * tc.tn + wn
                                    : (2 * tc.tm + wm) | ((2 * tc.tn + wn) << 16);
    Ident id;
    id.hi = g.id_hi;
    id.lo = g.id_lo;
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    if constexpr (ROLE == ROLE_SYM) {
      if (g.combo == 0) {
        run_tile<0, 0, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 1) {
        run_tile<1, 1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 2) {
        run_tile<0, 0, 2, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 3) {
        run_tile<0, 0, 2, 2>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 4) {
        run_tile<0, 1, 1, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 5) {
        run_tile_low<3, 2, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg,
                              low_switch(tc.tm, nkg), low_switch(tc.tn, nkg), id_g, wm, wn, id,
                              lenient);
      } else {
        run_tile_low<3, 3, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg,
                              low_switch(tc.tm, nkg), low_switch(tc.tn, nkg), id_g, wm, wn, id,
                              lenient);
      }
    } else if constexpr (ROLE == ROLE_PROBE) {
      if (g.combo == 0) {
        run_tile<0, 0, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else {
        run_tile<1, 1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      }
    } else {
      if (g.combo == 0) {
        run_tile<0, 1, 1, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 1) {
        run_tile<0, 0, 2, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 2) {
        run_tile<0, 1, 1, 2>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 3) {
        run_tile<0, 0, 2, 2>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 4) {
        run_tile<0, 1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 5) {
        run_tile<0, 0, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, id_g, wm, wn, id, lenient);
      } else if (g.combo == 6) {
        run_tile_low<1, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg,
                              low_switch(tc.tm, nkg), nkg, id_g, wm, wn, id, lenient);
      } else {
        run_tile_low<2, 0, 1>(acc, f0, f1, smem, la0, cb, wbase, LP, A, vid, stride, nkg, nkg,
                              low_switch(tc.tn, nkg), id_g, wm, wn, id, lenient);
      }
    }
    wm = (fresh_tid() >> 6) >> 1;
    wn = (fresh_tid() >> 6) & 1;
    const int wr0 = tc.tm * 256 + wm * 128, wc0 = tc.tn * 256 + wn * 128;
    float alpha = g.alpha;
    if (g.scale) {
      const float sc = scalar_load(g.scale + tc.prob);
      for (int p = 0; p < g.alpha_pow; ++p) alpha *= sc;
    }
    // Each kernel compiles only its own epilogues (extra instantiations cost
    // the whole kernel registers).  Symmetric products are scaled (by b, c
    // or 1) and read back by the next launch, so they stay cacheable; the
    // applies are not symmetric, mostly unscaled (alpha is 1 after the first
    // iteration) and their outputs stream out.
    bf16_t* C = g.c + (int64_t)tc.prob * g.sc;
    // The stores go through the ring buffer of the stage just multiplied:
    // the next tile's first loads target the other four, and its stage 4
    // goes there only after the barrier of its first step.  Every wave is
    // past its reads of that stage once all have met here.
    bf16_t* stage = smem + (cb == 0 ? NBUF - 1 : cb - 1) * STG +
                    4096 * __builtin_amdgcn_readfirstlane(fresh_tid() >> 6);
    if (g.pred && scalar_load_i32(g.pred + tc.prob) != 1) {
      // a problem that keeps its output: nothing stored; drained like an edge
      // epilogue, so that the next tile's first waits hold (see run_tile)
      wait_vm<0>();
    } else if constexpr (ROLE == ROLE_PROBE) {
      const int u = tc.tm * (tc.tm + 1) / 2 + tc.tn;
      float* out = g.resid + (int64_t)tc.prob * 4 * g.tiles_per_prob + 4 * u +
                   __builtin_amdgcn_readfirstlane(fresh_tid() >> 6);
      epilogue_resid(acc, out, g.M, g.N, wr0, wc0, alpha, tc.tm != tc.tn ? 2.f : 1.f);
    } else if constexpr (ROLE == ROLE_APPLY) {
      if (g.bits) {   // the last iteration of a vote-mode step: signs only
        uint64_t* bp = g.bits + (int64_t)tc.prob * g.bits_stride;
        if (g.bits_s8) {
          int8_t* sp = reinterpret_cast<int8_t*>(bp);
          if (alpha == 1.f)
            epilogue_bits<false, true>(acc, bp, sp, g.N / 64, g.M, g.N, wr0, wc0, alpha);
          else
            epilogue_bits<true, true>(acc, bp, sp, g.N / 64, g.M, g.N, wr0, wc0, alpha);
        } else {
          if (alpha == 1.f)
            epilogue_bits<false, false>(acc, bp, nullptr, g.N / 64, g.M, g.N, wr0, wc0, alpha);
          else
            epilogue_bits<true, false>(acc, bp, nullptr, g.N / 64, g.M, g.N, wr0, wc0, alpha);
        }
      } else {
        barrier_nofence();
        if (alpha == 1.f)
          epilogue<false, true>(acc, C, g.ldc, g.M, g.N, wr0, wc0, alpha, false, stage);
        else
          epilogue<true, true>(acc, C, g.ldc, g.M, g.N, wr0, wc0, alpha, false, stage);
      }
    } else {
      // an off-diagonal tile of a symmetric product also stores its mirror
      // copy, unless C is kept as its lower triangle
      barrier_nofence();
      epilogue<true, false>(acc, C, g.ldc, g.M, g.N, wr0, wc0, alpha,
                            g.sym && !g.c_low && tc.tm != tc.tn, stage);
    }
    t = tile_of(++round, vid, stride);
    if (t >= total) break;
    // every epilogue issues >= 32 stores or drains (see run_tile)
    lenient = true;
  }
  wait_vm<0>();   // the loads past the last stage target this workgroup's LDS
}

// The tile layout of a launch over its groups' device problem lists: group
// q's listed problems take tiles [out[q], out[q + 1]) (out[kNsgMaxGroups]:
// the total; nothing when the gate holds 0), and the work of the listed
// problems is credited to prof_exec while profiling.  One thread.
struct DynPrefixArgs {
  const int32_t* lists[kNsgMaxGroups];
  int tpp[kNsgMaxGroups];
  double flops[kNsgMaxGroups], bytes[kNsgMaxGroups];   // per listed problem
  int ngroups;
  const int32_t* gate;
  int32_t* out;
  double* prof_exec;
};

__global__ __launch_bounds__(64) void k_dyn_prefix(DynPrefixArgs a) {
  if (threadIdx.x != 0) return;
  const bool run = !a.gate || *a.gate != 0;
  int off = 0;
  double fl = 0.0, by = 0.0;
  for (int q = 0; q < kNsgMaxGroups; ++q) {
    a.out[q] = off;
    if (q < a.ngroups && run) {
      const int c = a.lists[q][0];
      off += c * a.tpp[q];
      fl += c * a.flops[q];
      by += c * a.bytes[q];
    }
  }
  a.out[kNsgMaxGroups] = off;
  if (a.prof_exec && off > 0) {
    atomicAdd(a.prof_exec, fl);
    atomicAdd(a.prof_exec + 1, by);
  }
}

}  // namespace nsg

// ------------------------------------------------------------------ launcher

namespace {
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}
}  // namespace

bool gemm_ns_supported(const NsgGroup& G) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if ((G.a_tbl || G.b_tbl) && (!G.tbl || G.tbl_per < 1 || G.batch > G.tbl_per * kTbl))
    return false;
  auto al_op = [&](const bf16_t* p, int use_tbl) {
    if (!use_tbl) return p != nullptr && al(p);
    for (int q = 0; q < (G.batch + G.tbl_per - 1) / G.tbl_per; ++q)
      if (!G.tbl->p[q] || !al(G.tbl->p[q])) return false;
    return true;
  };
  if (!al_op(G.a, G.a_tbl) || !al_op(G.b, G.b_tbl) || !al(G.c)) return false;
  if (G.lda % 8 || G.ldb % 8 || G.sa % 8 || G.sb % 8 || G.ldc % 4 || G.sc % 4) return false;
  if (G.M < 8 || G.N < 8 || G.K <= 0 || G.K % (4 * nsg::BK)) return false;
  if (G.a_kr && G.M % 8) return false;
  if (G.b_kr && G.N % 8) return false;
  // operand byte offsets within one problem must fit in 32 bits
  const int64_t ea = G.a_kr ? (int64_t)G.K * G.lda : (int64_t)G.M * G.lda;
  const int64_t eb = G.b_kr ? (int64_t)G.K * G.ldb : (int64_t)G.N * G.ldb;
  if (2 * ea >= ((int64_t)1 << 32) || 2 * eb >= ((int64_t)1 << 32)) return false;
  if (G.sym && (G.M != G.N || G.a_kr != G.b_kr || G.a_tbl != G.b_tbl))
    return false;
  if (G.ident && G.ident_terms != 1 && G.ident_terms != 2) return false;
  if (G.bits && (G.sym || G.N % 64 != 0 || (reinterpret_cast<uintptr_t>(G.bits) & 7u) ||
                 G.bits_stride < (int64_t)G.M * (G.N / 64)))
    return false;
  if (G.bits && G.bits_s8 &&
      ((reinterpret_cast<uintptr_t>(G.bits) & 15u) || G.bits_stride % 2 ||
       8 * G.bits_stride < (int64_t)G.M * G.N))
    return false;
  if (G.ident == 1 && G.K != G.M) return false;
  if (G.ident == 2 && G.K != G.N) return false;
  // both sides: symmetric lower-stored products of square matrices, one term
  if (G.ident == 3 &&
      (G.K != G.M || G.K != G.N || !G.sym || !G.a_low || !G.b_low || G.ident_terms != 1))
    return false;
  // lower-stored operands: square KC matrices; C kept lower only when symmetric
  if (G.a_low && (G.a_kr || G.a_tbl || G.M != G.K || G.M % 8)) return false;
  if (G.b_low && (G.b_kr || G.b_tbl || G.N != G.K || G.N % 8)) return false;
  if (G.c_low && !G.sym) return false;
  return true;
}

// Splits a into hi + lo with hi = bf16(a) and lo = bf16(a - hi); returns the
// number of terms needed for the sum to equal a exactly (1 or 2), or 0 if
// two are not enough.
int ns_ident_split(float a, uint32_t* hi_bits, uint32_t* lo_bits) {
  auto bf = [](float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    const uint32_t r = u + 0x7FFFu + ((u >> 16) & 1u);
    return r >> 16;
  };
  auto fl = [](uint32_t b) {
    const uint32_t u = b << 16;
    float x;
    std::memcpy(&x, &u, 4);
    return x;
  };
  const uint32_t h = bf(a);
  const float rem = a - fl(h);
  const uint32_t l = bf(rem);
  *hi_bits = h;
  *lo_bits = l;
  if (rem == 0.f) return 1;
  return (fl(h) + fl(l) == a) ? 2 : 0;
}

int gemm_ns_cus() { return cu_count(); }

int ns_group_tables(const NsgGroup* groups, int ngroups) {
  const PtrTbl* seen[kNsgMaxGroups];
  int n = 0;
  for (int q = 0; q < ngroups && q < kNsgMaxGroups; ++q) {
    const NsgGroup& G = groups[q];
    if (!(G.a_tbl || G.b_tbl)) continue;
    bool found = false;
    for (int i = 0; i < n; ++i) found |= seen[i] == G.tbl;
    if (!found) seen[n++] = G.tbl;
  }
  return n;
}

sm_status launch_gemm_ns(const NsgGroup* groups, int ngroups, int kind, hipStream_t s,
                         const int32_t* gate, int32_t* dyn_tiles) {
  using namespace nsg;
  if (ngroups <= 0 || ngroups > kNsgMaxGroups) return SM_ERR_ARG;
  const bool dyn = groups[0].dyn != nullptr;
  if (dyn && (!dyn_tiles || (reinterpret_cast<uintptr_t>(dyn_tiles) & 31u))) return SM_ERR_ARG;
  DynPrefixArgs dp;
  std::memset(&dp, 0, sizeof(dp));
  const bool apply = kind == SM_K_GEMM_APPLY;
  const bool probe = kind == SM_K_PROBE;
  if (!apply && !probe && kind != SM_K_GEMM_GRAM && kind != SM_K_GEMM_RR) return SM_ERR_ARG;
  Args a;
  std::memset(&a, 0, sizeof(a));
  const PtrTbl* tbls[kNsgMaxTables];
  int ntbl = 0;
  int tiles = 0;
  double flops = 0.0, bytes = 0.0;
  for (int q = 0; q < ngroups; ++q) {
    const NsgGroup& G = groups[q];
    Grp& g = a.g[q];
    g.a = G.a; g.b = G.b; g.c = G.c; g.scale = G.scale;
    g.lda = G.lda; g.sa = G.sa; g.ldb = G.ldb; g.sb = G.sb; g.ldc = G.ldc; g.sc = G.sc;
    g.M = G.M; g.N = G.N; g.K = G.K; g.batch = G.batch;
    g.a_kr = G.a_kr ? 1 : 0;
    g.b_kr = G.b_kr ? 1 : 0;
    g.sym = G.sym ? 1 : 0;
    g.ident = G.ident;
    g.id_hi = G.ident_hi;
    g.id_lo = G.ident_terms == 2 ? G.ident_lo : 0u;
    g.alpha_pow = G.alpha_pow;
    g.alpha = G.alpha;
    g.bits = G.bits;
    g.bits_stride = G.bits_stride;
    g.bits_s8 = G.bits_s8 ? 1 : 0;
    g.pred = G.pred;
    g.resid = G.resid;
    if (probe != (G.resid != nullptr)) return SM_ERR_UNSUPPORTED;
    if (G.bits && !apply) return SM_ERR_UNSUPPORTED;
    if (G.pred && G.bits) return SM_ERR_UNSUPPORTED;
    g.a_tbl = G.a_tbl ? 1 : 0;
    g.b_tbl = G.b_tbl ? 1 : 0;
    g.tbl_per = G.tbl_per;
    g.a_low = G.a_low ? 1 : 0;
    g.b_low = G.b_low ? 1 : 0;
    g.c_low = G.c_low ? 1 : 0;
    if (G.a_tbl || G.b_tbl) {
      int ti = 0;
      while (ti < ntbl && tbls[ti] != G.tbl) ++ti;
      if (ti == ntbl) {
        if (ntbl == kNsgMaxTables) return SM_ERR_UNSUPPORTED;
        tbls[ntbl] = G.tbl;
        a.tbl[ntbl] = *G.tbl;
        ++ntbl;
      }
      g.tbl = (int)(offsetof(Args, tbl) + ti * sizeof(PtrTbl));
    }
    // the instantiation for this group's layouts and identity mode
    int combo = -1;
    const bool two = G.ident && G.ident_terms == 2;
    const int low = (g.a_low ? 1 : 0) | (g.b_low ? 2 : 0);
    if (probe) {
      if (g.sym && !G.ident && !low && !G.c_low && !G.pred && g.a_kr == g.b_kr)
        combo = g.a_kr ? 1 : 0;
    } else if (!apply && g.sym) {
      if (low == 3) {
        if (G.ident == 2 && !two) combo = 5;
        else if (G.ident == 3 && !two) combo = 6;
      } else if (low) {
      } else if (!G.ident && !g.a_kr && !g.b_kr) combo = 0;
      else if (!G.ident && g.a_kr && g.b_kr) combo = 1;
      else if (G.ident == 2 && !g.a_kr && !g.b_kr) combo = two ? 3 : 2;
    } else if (!apply && !G.bits) {   // an apply riding along with symmetric products
      if (low) {
      } else if (G.ident == 1 && !g.a_kr && g.b_kr && !two) combo = 4;
      else if (G.ident == 2 && !g.a_kr && !g.b_kr) combo = two ? 3 : 2;
    } else if (low) {
      if (!G.ident && low == 1 && g.b_kr) combo = 6;
      else if (!G.ident && low == 2 && !g.a_kr) combo = 7;
    } else {
      if (G.ident == 1 && !g.a_kr && g.b_kr) combo = two ? 2 : 0;
      else if (G.ident == 2 && !g.a_kr && !g.b_kr) combo = two ? 3 : 1;
      else if (!G.ident && !g.a_kr && g.b_kr) combo = 4;
      else if (!G.ident && !g.a_kr && !g.b_kr) combo = 5;
    }
    if (combo < 0) return SM_ERR_UNSUPPORTED;
    // the apply kernel compiles only the plain epilogue (the symmetric one
    // stores a plain tile when its group is not symmetric)
    if (apply && g.sym) return SM_ERR_UNSUPPORTED;
    g.combo = combo;
    g.tiles_m = (G.M + 255) / 256;
    g.tiles_n = (G.N + 255) / 256;
    g.tiles_per_prob = g.sym ? g.tiles_m * (g.tiles_m + 1) / 2 : g.tiles_m * g.tiles_n;
    g.tile_begin = tiles;
    g.tpp_begin = a.tpp_total;
    a.tpp_total += g.tiles_per_prob;
    // device problem lists: in every group of the launch or in none
    if ((G.dyn != nullptr) != dyn) return SM_ERR_ARG;
    g.dyn = G.dyn;
    const int64_t gt = (int64_t)g.tiles_per_prob * G.batch;
    if (gt <= 0) return SM_ERR_ARG;
    if ((int64_t)tiles + gt > (int64_t)1 << 30) return SM_ERR_UNSUPPORTED;
    tiles += (int)gt;
    // a symmetric product is credited with the half it needs (M N K)
    flops += (g.sym ? 1.0 : 2.0) * G.M * (double)G.N * G.K * G.batch;
    // stored entries of each operand read once (one operand when A and B
    // are the same matrix), C written once (the 1-bit signs in its place);
    // a lower-stored matrix holds only its tiles on and below the diagonal
    const bool same = G.a == G.b && G.a_kr == G.b_kr && G.a_tbl == G.b_tbl && G.sa == G.sb &&
                      G.a_low == G.b_low;
    const double ea = G.a_low ? lower_tile_entries(G.M) : G.M * (double)G.K;
    const double eb = G.b_low ? lower_tile_entries(G.N) : G.N * (double)G.K;
    const double ec = probe ? 2.0 * ns_probe_parts(G.M)   // the float partials
                      : G.bits ? G.M * (double)G.N / (G.bits_s8 ? 2.0 : 16.0)
                             : (G.c_low ? lower_tile_entries(G.M) : G.M * (double)G.N);
    const double gbytes = 2.0 * ((same ? 0.0 : eb) + ea + ec);
    bytes += gbytes * G.batch;
    dp.lists[q] = G.dyn;
    dp.tpp[q] = g.tiles_per_prob;
    dp.flops[q] = (g.sym ? 1.0 : 2.0) * G.M * (double)G.N * G.K;
    dp.bytes[q] = gbytes;
  }
  a.ngroups = ngroups;
  a.total_tiles = tiles;
  a.gate = gate;
  a.dyn_tiles = dyn ? dyn_tiles : nullptr;
  const int grid = std::min(tiles, cu_count());
  a.xcd_chunk = (grid % 8 == 0) ? grid / 8 : 0;
  double* exec = (gate || dyn) ? prof_exec_slot(kind) : nullptr;
  if (dyn) {   // the tile layout over the lists (and the work they get credited)
    dp.ngroups = ngroups;
    dp.gate = gate;
    dp.out = dyn_tiles;
    dp.prof_exec = exec;
    prof_begin(SM_K_MISC, (kNsgMaxGroups + 1) * 4.0, s);
    hipLaunchKernelGGL(k_dyn_prefix, dim3(1), dim3(64), 0, s, dp);
    prof_end(s);
    SM_TRY(check_launch());
  }
  if (exec) {   // a gated launch reports its work only if it runs
    a.prof_exec = dyn ? nullptr : exec;
    a.prof_flops = flops;
    a.prof_bytes = bytes;
    prof_begin(kind, 0.0, s, 0.0);
  } else {
    prof_begin(kind, flops, s, bytes);
  }
  if (apply)
    hipLaunchKernelGGL((k_gemm_ns<ROLE_APPLY>), dim3(grid), dim3(NT), 0, s, a);
  else if (probe)
    hipLaunchKernelGGL((k_gemm_ns<ROLE_PROBE>), dim3(grid), dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_ns<ROLE_SYM>), dim3(grid), dim3(NT), 0, s, a);
  prof_end(s);
  return check_launch();
}

}  // namespace sm
