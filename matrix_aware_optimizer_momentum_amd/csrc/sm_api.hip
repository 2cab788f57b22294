// C ABI of libsm: argument validation, workspace layout, and the launch
// sequences of the optimizer step.  Every entry point validates its
// arguments on the host before the first HIP call, enqueues its kernels on
// the caller's stream and returns without synchronising.
//
// Sources (short names used below):
//   [SignMuon-ja]  SignMuon technical summary, gist.science/ja/paper/2605.16311
//   [CacheMuon-ja] CacheMuon technical summary, gist.science/ja/paper/2606.16371
//   [LionMuon-pt]  LionMuon technical summary, gist.science/pt/paper/2605.19811
#include "sm_internal.hpp"

#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <vector>

// A captured and instantiated step (sm_step_graph).
struct sm_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace sm {

// ====================================================================== errors

static std::atomic<int> g_last_hip{0};

sm_status hip_fail(hipError_t e) {
  g_last_hip.store((int)e);
  return SM_ERR_HIP;
}

sm_status check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SM_OK : hip_fail(e);
}


// ====================================================================== profiling

namespace {
struct ProfRec {
  int kind;
  double work, bytes;
  hipEvent_t a, b;
};
constexpr size_t kProfMax = 65536;
bool g_prof_on = false;
std::vector<hipEvent_t> g_prof_pool;  // 2 events per record
std::vector<ProfRec> g_prof_recs;
bool g_prof_open = false;
}  // namespace

void prof_begin(int kind, double work, hipStream_t s, double bytes) {
  g_prof_open = false;
  if (!g_prof_on) return;
  const size_t i = g_prof_recs.size();
  if (2 * i + 1 >= g_prof_pool.size()) return;
  ProfRec r{kind, work, bytes < 0.0 ? work : bytes, g_prof_pool[2 * i], g_prof_pool[2 * i + 1]};
  if (hipEventRecord(r.a, s) != hipSuccess) return;
  g_prof_recs.push_back(r);
  g_prof_open = true;
}

void prof_end(hipStream_t s) {
  if (!g_prof_open) return;
  g_prof_open = false;
  (void)hipEventRecord(g_prof_recs.back().b, s);
}

// Executed work of predicated launches, accumulated on the device:
// {flops, bytes} per kernel kind.  Written only by kernels (vector atomics);
// the host reads and clears it with copies while profiling.
__device__ __align__(256) double g_prof_exec[2 * SM_K_NUM_KINDS];
namespace {
double* g_prof_exec_ptr = nullptr;  // device address of g_prof_exec (current device)
}

double* prof_exec_slot(int kind) {
  if (!g_prof_on || !g_prof_exec_ptr || kind < 0 || kind >= SM_K_NUM_KINDS) return nullptr;
  return g_prof_exec_ptr + 2 * kind;
}

// ====================================================================== helpers

namespace {

bool valid_dt(int dt) { return dt == SM_F32 || dt == SM_BF16; }
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}
bool finite(float v) { return std::isfinite(v); }

sm_status check_ns_params(const sm_ns_params* p) {
  if (!p) return SM_ERR_ARG;
  if (p->iters < 1 || p->iters > 64) return SM_ERR_ARG;
  if (!finite(p->a) || !finite(p->b) || !finite(p->c)) return SM_ERR_ARG;
  if (!finite(p->eps) || p->eps < 0.f) return SM_ERR_ARG;
  return SM_OK;
}

sm_status check_shape(int batch, int m, int n) {
  if (batch < 1 || m < 1 || n < 1) return SM_ERR_SHAPE;
  if ((int64_t)m * n >= (int64_t(1) << 31)) return SM_ERR_SHAPE;
  if (batch > 4096) return SM_ERR_SHAPE;
  return SM_OK;
}

// Bump allocator over the caller's workspace; with base == null it only
// measures.  Every buffer starts on a 256-byte boundary.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

PtrTbl tbl_one(const void* p) {
  PtrTbl t;
  std::memset(&t, 0, sizeof(t));
  t.p[0] = static_cast<const char*>(p);
  return t;
}

GemmOperand opnd(const void* p, int64_t ld, int64_t stride, int dt, int layout, int tbl = 0) {
  GemmOperand o;
  o.p = p;
  o.ld = ld;
  o.stride = stride;
  o.dt = dt;
  o.layout = layout;
  o.tbl = tbl;
  return o;
}

GemmArgs gemm_base(int M, int N, int K, int batch) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.M = M;
  g.N = N;
  g.K = K;
  g.batch = batch;
  g.alpha = 1.f;
  g.beta = 0.f;
  g.tbl_per = 1;
  g.tbl_off = 0;
  return g;
}

// ------------------------------------------------------------------ direct NS

struct NsWs {
  void* tmp;    // [batch][m*n] ping-pong iterate, or [batch][3][r*r] Gram-form slots
  void* amat;   // [batch][r*r]
  void* amat2;  // [batch][r*r] (quintic term)
};

void carve_ns(Carver& cv, int dt, int batch, int m, int n, NsWs& w) {
  const int64_t r = m < n ? m : n;
  const size_t es = dt_size(dt);
  w.tmp = cv.take<void>((size_t)batch * std::max<int64_t>((int64_t)m * n, 3 * r * r) * es);
  w.amat = cv.take<void>((size_t)batch * r * r * es);
  w.amat2 = cv.take<void>((size_t)batch * r * r * es);
}

// One batch of same-shaped direct-NS problems: x[batch][m][n] -> out.  With
// xtbl set, x is null and problem p is read from worker p % xper of matrix
// p / xper (the momentum tensors themselves, no contiguous copy).
struct NsJob {
  const void* x;
  void* out;
  NsWs w;
  const float* scale;
  int batch, m, n;
  const PtrTbl* xtbl = nullptr;
  int xper = 1;
  // Vote mode: the last iteration writes the packed signs of X_K here
  // ([batch][bits_stride] words, the layout of launch_sign_pack) instead of
  // out (needs n % 64 == 0).
  uint64_t* bits = nullptr;
  int64_t bits_stride = 0;
  // bits_s8: the signs as int8 instead ([batch][m n] bytes at bits,
  // bits_stride = m n / 8 words; the grouped kernels only)
  bool bits_s8 = false;
};

// The grouped-kernel descriptors of one NS iteration of job j:
//   gram:  A_k = alpha X X^T (wide: X KC on both sides) or X^T X (tall: X KR
//          on both sides), symmetric, alpha = b (c = 0) or 1, times s^2 in
//          the first iteration;
//   rr:    B_k = c (A_k A_k + (b / c) A_k), the quintic term (c != 0);
//   apply: X_{k+1} = (B_k + a I) X_k (wide: A = B_k, B operand = X_k as KR)
//          or X_k (B_k + a I) (tall: A = X_k, B operand = B_k), times s in
//          the first iteration.
struct NsDesc {
  NsgGroup gram, rr, apply;
};

bool ns_desc(const NsJob& j, const void* cur, void* dst, bool first, bool last,
             const sm_ns_params& p, NsDesc& d) {
  const bool wide = j.m <= j.n;
  const int m = j.m, n = j.n, r = wide ? m : n;
  const int64_t mn = (int64_t)m * n, rr = (int64_t)r * r;
  auto bp = [](const void* q) { return static_cast<const bf16_t*>(q); };
  auto mp = [](void* q) { return static_cast<bf16_t*>(q); };
  std::memset(&d, 0, sizeof(d));
  const int tb = (cur == nullptr && j.xtbl) ? 1 : 0;   // cur is the tabled input
  NsgGroup& g = d.gram;
  g.a = bp(cur); g.lda = n; g.sa = mn; g.a_kr = wide ? 0 : 1;
  g.b = bp(cur); g.ldb = n; g.sb = mn; g.b_kr = wide ? 0 : 1;
  g.tbl = j.xtbl; g.tbl_per = j.xper; g.a_tbl = tb; g.b_tbl = tb;
  g.c = mp(j.w.amat); g.ldc = r; g.sc = rr;
  g.scale = j.scale; g.alpha_pow = first && j.scale ? 2 : 0;
  g.alpha = (p.c == 0.f) ? p.b : 1.f;
  g.M = r; g.N = r; g.K = wide ? n : m; g.batch = j.batch; g.sym = 1;
  if (!gemm_ns_supported(g)) return false;
  const void* bmat = j.w.amat;
  if (p.c != 0.f) {
    NsgGroup& q = d.rr;
    q.a = bp(j.w.amat); q.lda = r; q.sa = rr;
    q.b = bp(j.w.amat); q.ldb = r; q.sb = rr;
    q.c = mp(j.w.amat2); q.ldc = r; q.sc = rr;
    q.alpha = p.c;
    q.M = r; q.N = r; q.K = r; q.batch = j.batch; q.sym = 1;
    q.ident = 2;
    q.ident_terms = ns_ident_split(p.b / p.c, &q.ident_hi, &q.ident_lo);
    if (q.ident_terms == 0 || !gemm_ns_supported(q)) return false;
    bmat = j.w.amat2;
  }
  NsgGroup& a = d.apply;
  a.tbl = j.xtbl; a.tbl_per = j.xper;
  if (wide) {
    a.a = bp(bmat); a.lda = r; a.sa = rr;
    a.b = bp(cur); a.ldb = n; a.sb = mn; a.b_kr = 1; a.b_tbl = tb;
    a.ident = 1;
  } else {
    a.a = bp(cur); a.lda = n; a.sa = mn; a.a_tbl = tb;
    a.b = bp(bmat); a.ldb = r; a.sb = rr;
    a.ident = 2;
  }
  a.c = mp(dst); a.ldc = n; a.sc = mn;
  a.scale = j.scale; a.alpha_pow = first && j.scale ? 1 : 0; a.alpha = 1.f;
  a.M = m; a.N = n; a.K = r; a.batch = j.batch;
  a.ident_terms = ns_ident_split(p.a, &a.ident_hi, &a.ident_lo);
  if (last && j.bits) {
    a.bits = j.bits;
    a.bits_stride = j.bits_stride;
    a.bits_s8 = j.bits_s8 ? 1 : 0;
  }
  return a.ident_terms != 0 && gemm_ns_supported(a);
}

// Launches one product kind for all jobs, groups ordered by decreasing K so
// that concurrent tiles carry similar work, as few launches as the group
// and table limits allow.
sm_status launch_ns_groups(std::vector<NsgGroup>& gs, int kind, hipStream_t s,
                           const int32_t* gate = nullptr, int32_t* dyn_tiles = nullptr) {
  std::stable_sort(gs.begin(), gs.end(),
                   [](const NsgGroup& x, const NsgGroup& y) { return x.K > y.K; });
  size_t i = 0;
  while (i < gs.size()) {
    int ng = 1;
    while (i + ng < gs.size() && ng < kNsgMaxGroups &&
           ns_group_tables(gs.data() + i, ng + 1) <= kNsgMaxTables)
      ++ng;
    SM_TRY(launch_gemm_ns(gs.data() + i, ng, kind, s, gate, dyn_tiles));
    i += ng;
  }
  return SM_OK;
}

// ------------------------------------------------------------------ Gram-form NS
// The cubic iteration (c = 0) reaches the same X_K through r x r products,
// which is cheaper when the matrix is far from square.  With S_k = b X_k X_k^T
// and P_k = S_k + aI one direct step is X_{k+1} = P_k X_k, so X_k = Q_k X_0
// with Q_k = P_{k-1} ... P_0.  S_k, P_k and Q_k are all polynomials in
// G = X_0 X_0^T, hence symmetric and commuting, and
//   S_0 = b s^2 x x^T            (the Gram product over the long side)
//   Q_1 = S_0 + aI               (identity fill)
//   T_k = S_k (S_k + aI),  S_{k+1} = T_k (S_k + aI)   (= P_k S_k P_k), k < K-1
//   Q_{k+1} = Q_k (S_k + aI)     (k >= 1)
//   X_K = s Q_K x                (one apply over the long side)
// Every r x r product is a symmetric one (lower-triangle tiles) whose aI
// part comes from the identity fold, so S_k, T_k and Q_k are rounded to
// bf16 once per product, like the direct form's B_k and X_k.  With a
// one-term identity there is no fill: Q_2 = (S_0 + aI)(S_1 + aI) takes the
// identity on both sides, straight from S_0.  Storing P_k
// instead of S_k would round its O(1) diagonal and costs several times the
// error.  Launches L1(k) = {T_k, Q_{k+1}} and L2(k) = {S_{k+1}}, 2K - 1 in
// all; Q_{k+1} (k = 1 .. K-2) may be split by problems between L1(k) and
// L2(k) to fill L1(k)'s last round of tiles (ns_grouped).  Five r x r slots
// per problem: S_k, Q_k, two free ones rotating, and T.
struct GfSlot {
  bf16_t* p;
  int64_t st;   // elements between problems
};

struct GfPlan {
  NsgGroup gram, apply;
  // products per iteration k: T[k] = T_k, S[k] = S_{k+1} (k < K-1),
  // Q[k] = Q_{k+1} (k >= 1); unused entries have batch 0
  std::vector<NsgGroup> T, S, Q;
  GfSlot fill_src, fill_dst;   // Q_1 = S_0 + aI (fill_src.p null: no fill)
  GfSlot qk;                   // where Q_K ends up (lower-stored when gram.c_low)
  int r, batch, tiles;   // tiles: 256 x 256 tiles of one r x r product
  float a;
};

// Problems [p0, p0 + n) of group g (no pointer tables).
NsgGroup ns_subrange(const NsgGroup& g, int p0, int n) {
  NsgGroup h = g;
  h.a = g.a + (int64_t)p0 * g.sa;
  h.b = g.b + (int64_t)p0 * g.sb;
  h.c = g.c + (int64_t)p0 * g.sc;
  if (g.scale) h.scale = g.scale + p0;
  if (g.bits) h.bits = g.bits + (int64_t)p0 * g.bits_stride;
  if (g.pred) h.pred = g.pred + p0;
  h.batch = n;
  return h;
}

// Executed MFMA work of one problem in 256 x 256 tile x 128-deep k-group
// units, for the direct and the Gram form (identity groups included).
int64_t ns_tile_work(int r, int cols, int K, bool gram_form) {
  const int64_t tr = (r + 255) / 256, tc = (cols + 255) / 256;
  const int64_t sym = tr * (tr + 1) / 2;
  const int64_t kr = (r + 127) / 128, kc = (cols + 127) / 128;
  if (!gram_form) return K * (sym * kc + tr * tc * (kr + 1));
  return sym * kc + 3 * (int64_t)(K - 1) * sym * (kr + 1) + tr * tc * kr;
}

// Takes job j in the Gram form if that form's MFMA work is below the direct
// form's (always with `force`: CacheMuon needs Q_K).  The choice depends on
// the job alone (not on the other jobs of the call), so a matrix gets the
// same result from a step as from sm_ns_polar.
bool gf_plan(const NsJob& j, const sm_ns_params& p, GfPlan& g, bool force = false) {
  const int K = p.iters;
  if (p.c != 0.f || K < 2) return false;
  const bool wide = j.m <= j.n;
  const int m = j.m, n = j.n, r = wide ? m : n, cols = wide ? n : m;
  if (!force && ns_tile_work(r, cols, K, true) >= ns_tile_work(r, cols, K, false)) return false;
  const int64_t mn = (int64_t)m * n, rr = (int64_t)r * r;
  auto bp = [](const void* q) { return static_cast<const bf16_t*>(q); };
  auto mp = [](void* q) { return static_cast<bf16_t*>(q); };
  const int tb = (j.x == nullptr && j.xtbl) ? 1 : 0;
  // three of the five r x r slots live in the iterate buffer
  GfSlot slot[4] = {{mp(j.w.amat), rr}, {mp(j.w.amat2), rr}, {mp(j.w.tmp), 3 * rr},
                    {mp(j.w.tmp) + rr, 3 * rr}};
  const GfSlot tslot{mp(j.w.tmp) + 2 * rr, 3 * rr};
  uint32_t id_hi = 0, id_lo = 0;
  const int id_terms = ns_ident_split(p.a, &id_hi, &id_lo);
  if (id_terms == 0) return false;
  // S_k, T_k, Q_k are symmetric: with a one-term identity the products keep
  // only their tiles on and below the diagonal, and read the rest of a panel
  // from the mirror tiles (no mirror stores)
  const int low = id_terms == 1 ? 1 : 0;

  std::memset(&g.gram, 0, sizeof(g.gram));
  NsgGroup& gr = g.gram;
  gr.a = bp(j.x); gr.lda = n; gr.sa = mn; gr.a_kr = wide ? 0 : 1;
  gr.b = bp(j.x); gr.ldb = n; gr.sb = mn; gr.b_kr = wide ? 0 : 1;
  gr.tbl = j.xtbl; gr.tbl_per = j.xper; gr.a_tbl = tb; gr.b_tbl = tb;
  // lower-stored: S_0 goes to Q_1's slot and serves as Q_1 too (Q_2 takes
  // the identity on both sides); else Q_1 = S_0 + aI is filled in
  const GfSlot& s0 = low ? slot[1] : slot[0];
  gr.c = s0.p; gr.ldc = r; gr.sc = s0.st;
  gr.scale = j.scale; gr.alpha_pow = j.scale ? 2 : 0; gr.alpha = p.b;
  gr.M = r; gr.N = r; gr.K = cols; gr.batch = j.batch; gr.sym = 1; gr.c_low = low;
  if (!gemm_ns_supported(gr)) return false;

  // C = A (B + aI) over r x r slots
  auto prod = [&](const GfSlot& A, const GfSlot& B, const GfSlot& C) {
    NsgGroup q;
    std::memset(&q, 0, sizeof(q));
    q.a = A.p; q.lda = r; q.sa = A.st;
    q.b = B.p; q.ldb = r; q.sb = B.st;
    q.c = C.p; q.ldc = r; q.sc = C.st;
    q.alpha = 1.f;
    q.M = r; q.N = r; q.K = r; q.batch = j.batch; q.sym = 1;
    q.ident = 2; q.ident_terms = id_terms; q.ident_hi = id_hi; q.ident_lo = id_lo;
    q.a_low = q.b_low = q.c_low = low;
    return q;
  };
  // slots of S_k and Q_k, and the two free ones (Q_{k+1}, S_{k+1} go there);
  // lower-stored, S_0 and Q_1 share slot 1 until Q_2 is made, and slot 0
  // stands by as S_2's
  int si = low ? 1 : 0, qi = 1, f1 = 2, f2 = 3;
  g.fill_src = low ? GfSlot{nullptr, 0} : slot[si];
  g.fill_dst = slot[qi];
  NsgGroup none;
  std::memset(&none, 0, sizeof(none));
  g.T.assign(K, none);
  g.S.assign(K, none);
  g.Q.assign(K, none);
  for (int k = 0; k < K; ++k) {
    if (k < K - 1) g.T[k] = prod(slot[si], slot[si], tslot);         // T_k
    if (k >= 1) g.Q[k] = prod(slot[qi], slot[si], slot[f1]);        // Q_{k+1}
    if (k == 1 && low) g.Q[k].ident = 3;   // Q_2 = (S_0 + aI)(S_1 + aI)
    if (k < K - 1) g.S[k] = prod(tslot, slot[si], slot[f2]);         // S_{k+1}
    const int os = si, oq = qi;
    if (k >= 1) { qi = f1; f1 = oq; }
    if (k < K - 1) { si = f2; f2 = (k == 0 && low) ? 0 : os; }
  }
  for (int k = 0; k < K; ++k)
    for (const NsgGroup* q : {&g.T[k], &g.S[k], &g.Q[k]})
      if (q->batch && !gemm_ns_supported(*q)) return false;

  std::memset(&g.apply, 0, sizeof(g.apply));
  NsgGroup& a = g.apply;
  const GfSlot& qk = slot[qi];
  g.qk = qk;
  a.tbl = j.xtbl; a.tbl_per = j.xper;
  if (wide) {   // X_K = Q_K x
    a.a = qk.p; a.lda = r; a.sa = qk.st; a.a_low = low;
    a.b = bp(j.x); a.ldb = n; a.sb = mn; a.b_kr = 1; a.b_tbl = tb;
  } else {      // X_K = x Q_K
    a.a = bp(j.x); a.lda = n; a.sa = mn; a.a_tbl = tb;
    a.b = qk.p; a.ldb = r; a.sb = qk.st; a.b_low = low;
  }
  a.c = mp(j.out); a.ldc = n; a.sc = mn;
  a.scale = j.scale; a.alpha_pow = j.scale ? 1 : 0; a.alpha = 1.f;
  a.M = m; a.N = n; a.K = r; a.batch = j.batch;
  if (j.bits) {
    a.bits = j.bits;
    a.bits_stride = j.bits_stride;
    a.bits_s8 = j.bits_s8 ? 1 : 0;
  }
  if (!gemm_ns_supported(a)) return false;
  g.r = r;
  g.batch = j.batch;
  g.tiles = (int)(((r + 255) / 256) * ((r + 255) / 256 + 1) / 2);
  g.a = p.a;
  auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  return r % 8 == 0 && al(j.w.amat) && al(j.w.amat2) &&
         al(j.w.tmp);
}

// Tiles of one launch of group g (256 x 256; lower triangle when symmetric).
int64_t ns_group_tiles(const NsgGroup& g) {
  const int64_t tm = (g.M + 255) / 256, tn = (g.N + 255) / 256;
  return (g.sym ? tm * (tm + 1) / 2 : tm * tn) * g.batch;
}

// Whether the symmetric kernel runs apply g: its combos take the tall apply
// X (B + aI) and the wide (B + aI) X with a one-term identity, not signs.
bool ns_rides_sym(const NsgGroup& g) {
  if (g.sym || g.bits) return false;
  if (g.ident == 2) return !g.a_kr && !g.b_kr;
  return g.ident == 1 && !g.a_kr && g.b_kr && g.ident_terms == 1;
}

// NS on bf16 jobs with the grouped kernels.  Jobs that gf_plan takes run the
// Gram form, the others the direct form.  Direct only: per iteration one
// Gram launch and one apply launch for all jobs.  With Gram-form jobs: their
// Gram products share the first launch with the direct jobs' first Gram
// products; their 2K - 1 r x r launches carry the direct jobs' next
// products along (the direct chain a_0, g_1, a_1, ..., g_{K-1}, one per
// launch, when the symmetric kernel runs their applies; else only the
// Gram products g_1 .. g_{K-1}, with the applies in launches of their own);
// and their applies share the last launch with the direct jobs' last
// apply.  Returns SM_ERR_UNSUPPORTED (nothing launched) if some job does not
// meet the kernels' requirements.
sm_status ns_grouped(const std::vector<NsJob>& jobs, const sm_ns_params& p, hipStream_t s) {
  const int K = p.iters;
  std::vector<const NsJob*> dj;
  std::vector<GfPlan> gf;
  for (const NsJob& j : jobs) {
    GfPlan g;
    if (gf_plan(j, p, g))
      gf.push_back(std::move(g));
    else
      dj.push_back(&j);
  }
  // the direct jobs' products of every iteration
  std::vector<std::vector<NsDesc>> D(K, std::vector<NsDesc>(dj.size()));
  for (int k = 0; k < K; ++k)
    for (size_t i = 0; i < dj.size(); ++i) {
      const NsJob& j = *dj[i];
      const void* cur = k == 0 ? j.x : (((K - k) % 2 == 0) ? j.out : j.w.tmp);
      void* dst = ((K - 1 - k) % 2 == 0) ? j.out : j.w.tmp;
      if (!ns_desc(j, cur, dst, k == 0, k == K - 1, p, D[k][i])) return SM_ERR_UNSUPPORTED;
    }
  const int nrr = gf.empty() ? 0 : 2 * K - 1;   // Gram-form r x r launches
  // ride: the direct chain's applies travel in the r x r launches too
  bool ride = nrr > 0 && !dj.empty() && p.c == 0.f;
  for (int k = 0; ride && k < K - 1; ++k)
    for (size_t i = 0; i < dj.size(); ++i) ride = ride && ns_rides_sym(D[k][i].apply);
  // Riding, a direct job's chain a_0, g_1, a_1, ..., g_{K-1} (2K - 2
  // products, each needing the one before) takes one product per r x r
  // launch, so it skips one of the 2K - 1 launches.  The job's problems may
  // form two cohorts that skip different launches (chosen below to save
  // rounds of the grid); a_0 reads the input through its table and scale, so
  // both cohorts run it in launch 0 (skip >= 1) and it is never split.
  struct Cohort {
    int p0, n, skip;
  };
  std::vector<std::vector<Cohort>> coh(dj.size());
  for (size_t i = 0; i < dj.size(); ++i)
    coh[i] = {{0, D[0][i].apply.batch, std::max(nrr - 1, 1)}};
  // the direct products that travel with r x r launch l
  auto riders_of = [&](int l, std::vector<NsgGroup>& v) {
    for (size_t i = 0; i < dj.size(); ++i) {
      if (!ride) {
        if (l + 1 <= K - 1) v.push_back(D[l + 1][i].gram);
        continue;
      }
      // chain element of each cohort in launch l; equal elements of
      // adjacent cohorts go out as one group
      int c0 = -1, p0 = 0, n = 0;
      auto flush = [&]() {
        if (c0 < 0) return;
        const NsgGroup& g = c0 % 2 == 0 ? D[c0 / 2][i].apply : D[(c0 + 1) / 2][i].gram;
        v.push_back(p0 == 0 && n == g.batch ? g : ns_subrange(g, p0, n));
        c0 = -1;
      };
      for (const Cohort& h : coh[i]) {
        const int c = l == h.skip ? -1 : (l < h.skip ? l : l - 1);
        if (c < 0 || c > 2 * K - 3) { flush(); continue; }
        if (c == c0 && p0 + n == h.p0) { n += h.n; continue; }
        flush();
        c0 = c; p0 = h.p0; n = h.n;
      }
      flush();
    }
  };
  // tiles per problem of a direct job's applies and Gram products
  std::vector<int64_t> tpp_apply(dj.size()), tpp_gram(dj.size());
  for (size_t i = 0; i < dj.size(); ++i) {
    tpp_apply[i] = ns_group_tiles(D[0][i].apply) / D[0][i].apply.batch;
    tpp_gram[i] = ns_group_tiles(D[0][i].gram) / D[0][i].gram.batch;
  }
  // tiles and groups of the direct products in r x r launch l (as riders_of
  // issues them, counted without building them)
  auto riders = [&](int l, int* groups = nullptr) {
    int64_t t = 0;
    int ng = 0;
    for (size_t i = 0; i < dj.size(); ++i) {
      if (!ride) {
        if (l + 1 <= K - 1) { t += tpp_gram[i] * D[l + 1][i].gram.batch; ++ng; }
        continue;
      }
      int c0 = -1;
      for (const Cohort& h : coh[i]) {
        const int c = l == h.skip ? -1 : (l < h.skip ? l : l - 1);
        if (c < 0 || c > 2 * K - 3) { c0 = -1; continue; }
        t += (c % 2 == 0 ? tpp_apply[i] : tpp_gram[i]) * h.n;
        if (c != c0) ++ng;
        c0 = c;
      }
    }
    if (groups) *groups = ng;
    return t;
  };
  // Q_{k+1} (k = 1 .. K-2) goes to L1(k) whole, or its first problems fill
  // L1(k)'s last round of tiles and the rest joins L2(k), whichever needs
  // fewer rounds of the grid (qa[k][job]: problems in L1(k)).
  const int64_t cus = gemm_ns_cus();
  auto rounds = [&](int64_t t) { return (t + cus - 1) / cus; };
  std::vector<std::vector<int>> qa(K, std::vector<int>(gf.size(), 0));
  auto plan_q = [&]() {
    for (int k = 1; k < K; ++k) {
      int64_t tt = 0, qt = 0, st = 0;
      for (size_t i = 0; i < gf.size(); ++i) {
        tt += (int64_t)gf[i].tiles * gf[i].T[k].batch;
        qt += (int64_t)gf[i].tiles * gf[i].Q[k].batch;
        st += (int64_t)gf[i].tiles * gf[i].S[k].batch;
        qa[k][i] = gf[i].Q[k].batch;   // whole, unless split below
      }
      if (k > K - 2) continue;
      const int64_t b1 = tt + riders(2 * k), b2 = st + riders(2 * k + 1);
      int64_t room = rounds(b1) * cus - b1, moved = 0;
      std::vector<int> split(gf.size(), 0);
      for (size_t i = 0; i < gf.size(); ++i) {
        const int n = (int)std::min<int64_t>(gf[i].Q[k].batch, room / gf[i].tiles);
        split[i] = n;
        room -= (int64_t)n * gf[i].tiles;
        moved += (int64_t)n * gf[i].tiles;
      }
      if (rounds(b1) + rounds(b2 + qt - moved) < rounds(b1 + qt) + rounds(b2)) qa[k] = split;
    }
  };
  plan_q();
  auto take_rr = [&](int l, std::vector<NsgGroup>& v) {
    const int k = l / 2;
    for (size_t i = 0; i < gf.size(); ++i) {
      const GfPlan& g = gf[i];
      const NsgGroup& q = g.Q[k];
      if (l % 2 == 0) {   // L1(k): T_k and the first qa problems of Q_{k+1}
        if (g.T[k].batch) v.push_back(g.T[k]);
        if (q.batch && qa[k][i]) v.push_back(ns_subrange(q, 0, qa[k][i]));
      } else {            // L2(k): S_{k+1} and the rest of Q_{k+1}
        if (g.S[k].batch) v.push_back(g.S[k]);
        if (q.batch && qa[k][i] < q.batch)
          v.push_back(ns_subrange(q, qa[k][i], q.batch - qa[k][i]));
      }
    }
  };
  // rounds of the grid over the r x r launches; a launch that would need
  // more than kNsgMaxGroups groups rules the configuration out
  auto rr_rounds = [&]() -> int64_t {
    plan_q();
    int64_t total = 0;
    for (int l = 0; l < nrr; ++l) {
      const int k = l / 2;
      int ng = 0;
      int64_t t = riders(l, &ng);
      for (size_t i = 0; i < gf.size(); ++i) {
        const GfPlan& g = gf[i];
        const int qb = g.Q[k].batch, q1 = qa[k][i];
        const int a = l % 2 == 0 ? g.T[k].batch : g.S[k].batch;
        const int q = l % 2 == 0 ? q1 : qb - q1;
        t += (int64_t)g.tiles * (a + q);
        ng += (a > 0) + (q > 0);
      }
      if (ng > kNsgMaxGroups) return INT64_MAX;
      total += rounds(t);
    }
    return total;
  };
  if (ride && nrr >= 3) {
    // per direct job, the cohorts that need fewest rounds (greedy over the
    // jobs); the choice depends only on the launch shapes, so it is cached
    std::vector<int64_t> key = {K, cus};
    for (const GfPlan& g : gf) key.insert(key.end(), {g.tiles, g.batch});
    for (size_t i = 0; i < dj.size(); ++i)
      key.insert(key.end(), {tpp_apply[i], tpp_gram[i], D[0][i].apply.batch});
    static std::mutex mu;
    static std::map<std::vector<int64_t>, std::vector<std::vector<Cohort>>> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      coh = it->second;
    } else {
      for (size_t i = 0; i < dj.size(); ++i) {
        const int b = D[0][i].apply.batch;
        std::vector<Cohort> best = coh[i];
        int64_t best_r = rr_rounds();
        auto consider = [&](std::vector<Cohort> c) {
          coh[i] = std::move(c);
          const int64_t r = rr_rounds();
          if (r < best_r) { best_r = r; best = coh[i]; }
        };
        for (int s1 = 1; s1 < nrr; ++s1) consider({{0, b, s1}});
        const int step = std::max(1, b / 64);
        for (int n1 = step; n1 < b; n1 += step)
          for (int s1 = 1; s1 < nrr; ++s1)
            for (int s2 = 1; s2 < nrr; ++s2)
              if (s1 != s2) consider({{0, n1, s1}, {n1, b - n1, s2}});
        coh[i] = best;
      }
      if (cache.size() < 256) cache[key] = coh;
    }
    plan_q();
  }
  auto fills = [&]() -> sm_status {
    for (const GfPlan& g : gf)
      if (g.fill_src.p)
        SM_TRY(launch_add_identity(g.fill_src.p, g.fill_src.st, g.fill_dst.p, g.fill_dst.st,
                                   g.r, g.batch, g.a, g.gram.c_low != 0, s));
    return SM_OK;
  };

  if (ride) {
    std::vector<NsgGroup> first, last;
    for (size_t i = 0; i < dj.size(); ++i) first.push_back(D[0][i].gram);
    for (const GfPlan& g : gf) first.push_back(g.gram);
    SM_TRY(launch_ns_groups(first, SM_K_GEMM_GRAM, s));
    SM_TRY(fills());
    for (int l = 0; l < nrr; ++l) {
      std::vector<NsgGroup> v;
      take_rr(l, v);
      riders_of(l, v);
      SM_TRY(launch_ns_groups(v, SM_K_GEMM_RR, s));
    }
    for (size_t i = 0; i < dj.size(); ++i) last.push_back(D[K - 1][i].apply);
    for (const GfPlan& g : gf) last.push_back(g.apply);
    return launch_ns_groups(last, SM_K_GEMM_APPLY, s);
  }
  int l = 0;
  for (int k = 0; k < K; ++k) {
    std::vector<NsgGroup> sym, rr, apply;
    for (size_t i = 0; i < dj.size(); ++i) {
      sym.push_back(D[k][i].gram);
      if (p.c != 0.f) rr.push_back(D[k][i].rr);
      apply.push_back(D[k][i].apply);
    }
    int kind = SM_K_GEMM_GRAM;
    if (k == 0) {
      for (const GfPlan& g : gf) sym.push_back(g.gram);
    } else if (l < nrr) {
      take_rr(l++, sym);
      kind = SM_K_GEMM_RR;
    }
    SM_TRY(launch_ns_groups(sym, kind, s));
    if (k == 0) SM_TRY(fills());
    if (!rr.empty()) SM_TRY(launch_ns_groups(rr, SM_K_GEMM_RR, s));
    if (k == K - 1) {   // the rest of the Gram-form chain, then every last apply
      for (; l < nrr; ++l) {
        std::vector<NsgGroup> v;
        take_rr(l, v);
        SM_TRY(launch_ns_groups(v, SM_K_GEMM_RR, s));
      }
      for (const GfPlan& g : gf) apply.push_back(g.apply);
    }
    SM_TRY(launch_ns_groups(apply, SM_K_GEMM_APPLY, s));
  }
  return SM_OK;
}

// Whether ns_grouped takes job j (checked for the first iteration's
// pointers; later iterations use buffers of the same shapes and alignment).
bool ns_grouped_ok(const NsJob& j, int dt, const sm_ns_params& p) {
  if (dt != BF16) return false;
  GfPlan g;
  if (gf_plan(j, p, g)) return true;
  NsDesc d;
  return ns_desc(j, j.x, j.out, true, p.iters == 1, p, d) &&
         ns_desc(j, j.out, j.w.tmp, false, true, p, d);
}

// Products of one direct NS step on problems of shape m x n (x contiguous):
//   gram:  A = alpha * X X^T       (oriented; Y^T Y for a tall Y)
//   apply: X' = alpha * (B X) + beta * X   (X B^T for a tall Y)
GemmArgs gram_args(const void* x, int dt, int batch, int m, int n) {
  const bool wide = m <= n;
  const int r = wide ? m : n, c = wide ? n : m;
  GemmArgs g = gemm_base(r, r, c, batch);
  const int lay = wide ? KC : RC;
  g.a = opnd(x, n, (int64_t)m * n, dt, lay);
  g.b = opnd(x, n, (int64_t)m * n, dt, lay);
  return g;
}

GemmArgs apply_args(const void* bm, int bm_dt, int bm_tbl, const void* x, int dt, int batch,
                    int m, int n) {
  const bool wide = m <= n;
  const int r = wide ? m : n;
  GemmArgs g = gemm_base(m, n, r, batch);
  if (wide) {  // X' = B X : A = B (r x r), B-operand = X with rows k contiguous
    g.a = opnd(bm, r, (int64_t)r * r, bm_dt, KC, bm_tbl);
    g.b = opnd(x, n, (int64_t)m * n, dt, RC);
  } else {     // Y' = Y B^T : A = Y, B-operand(k, j) = B(j, k)
    g.a = opnd(x, n, (int64_t)m * n, dt, KC);
    g.b = opnd(bm, r, (int64_t)r * r, bm_dt, KC, bm_tbl);
  }
  return g;
}

// X_K of the direct iteration [SignMuon-ja] section 2 (core mechanism 1):
// X_{k+1} = a X_k + (b A_k + c A_k^2) X_k,  A_k = X_k X_k^T, starting from
// X_0 = s x (s = scale[b], or 1 without normalisation).  The scale enters
// the first step's GEMMs: A_0 = s^2 x x^T, X_1 = s (a x + B_0 x).
// This is the path of the jobs that the persistent bf16 kernel does not
// take (float32 above all): per iteration the Gram products of every job go
// out as grouped launches, then the quintic terms, then the applies.
sm_status ns_generic(const std::vector<NsJob>& jobs, int dt, const sm_ns_params& p,
                     hipStream_t s) {
  const int K = p.iters;
  const size_t nj = jobs.size();
  for (const NsJob& j : jobs)
    if (j.bits_s8) return SM_ERR_UNSUPPORTED;   // int8 signs: the grouped kernels only
  std::vector<const void*> cur(nj);
  for (size_t i = 0; i < nj; ++i) cur[i] = jobs[i].x;
  // the iterate of job i read through its pointer table (k == 0 with xtbl)
  auto via_tbl = [&](size_t i, int k) { return k == 0 && jobs[i].xtbl != nullptr; };
  std::vector<GemmArgs> gr, qr, ap;
  for (int k = 0; k < K; ++k) {
    gr.clear();
    qr.clear();
    ap.clear();
    for (size_t i = 0; i < nj; ++i) {
      const NsJob& j = jobs[i];
      const int m = j.m, n = j.n, r = m < n ? m : n;
      const int64_t rr = (int64_t)r * r, mn = (int64_t)m * n;
      const bool first = (k == 0) && j.scale;
      const bool last = k == K - 1;
      const bool tb = via_tbl(i, k);
      void* dst = ((K - 1 - k) % 2 == 0) ? j.out : j.w.tmp;
      // A_k (times b when the quintic term is absent)
      GemmArgs g = gram_args(cur[i], dt, j.batch, m, n);
      if (tb) {
        g.a.tbl = g.b.tbl = 1;
        g.tbl = *j.xtbl;
        g.tbl_per = j.xper;
      }
      g.c = j.w.amat; g.ldc = r; g.sc = rr; g.c_dt = dt;
      g.scale = j.scale; g.alpha_pow = first ? 2 : 0;
      g.alpha = (p.c == 0.f) ? p.b : 1.f;
      g.sym = 1;
      gr.push_back(g);
      const void* bmat = j.w.amat;
      if (p.c != 0.f) {  // B = c A A + b A
        GemmArgs q = gemm_base(r, r, r, j.batch);
        q.a = opnd(j.w.amat, r, rr, dt, KC);
        q.b = opnd(j.w.amat, r, rr, dt, RC);
        q.cin = j.w.amat; q.ldcin = r; q.scin = rr;
        q.c = j.w.amat2; q.ldc = r; q.sc = rr; q.c_dt = dt;
        q.alpha = p.c; q.beta = p.b;
        q.sym = 1;   // c A^2 + b A of a symmetric A
        qr.push_back(q);
        bmat = j.w.amat2;
      }
      GemmArgs a = apply_args(bmat, dt, 0, cur[i], dt, j.batch, m, n);
      a.cin = cur[i]; a.ldcin = n; a.scin = mn;
      if (tb) {
        (m <= n ? a.b : a.a).tbl = 1;
        a.cin_tbl = 1;
        a.tbl = *j.xtbl;
        a.tbl_per = j.xper;
      }
      a.c_dt = dt;   // also the type of Cin, and the rounding the signs are taken after
      if (last && j.bits) {   // signs only: X_K itself is not stored
        a.bits = j.bits;
        a.bits_stride = j.bits_stride;
      } else {
        a.c = dst; a.ldc = n; a.sc = mn;
      }
      a.scale = j.scale; a.alpha_pow = first ? 1 : 0; a.beta_pow = first ? 1 : 0;
      a.alpha = 1.f; a.beta = p.a;
      ap.push_back(a);
      cur[i] = dst;
    }
    SM_TRY(launch_gemm_groups(gr, dt, SM_K_GEMM_GRAM, s));
    if (!qr.empty()) SM_TRY(launch_gemm_groups(qr, dt, SM_K_GEMM_RR, s));
    SM_TRY(launch_gemm_groups(ap, dt, SM_K_GEMM_APPLY, s));
  }
  return SM_OK;
}

sm_status ns_core(const void* x, void* out, const NsWs& w, const float* scale, int dt, int batch,
                  int m, int n, const sm_ns_params& p, hipStream_t s) {
  const NsJob job{x, out, w, scale, batch, m, n};
  if (ns_grouped_ok(job, dt, p)) return ns_grouped(std::vector<NsJob>{job}, p, s);
  return ns_generic(std::vector<NsJob>{job}, dt, p, s);
}

// ------------------------------------------------------------------ Gram NS with cache

struct GramWs {
  float* ga;      // [batch][r*r]  G ping-pong
  float* gb;
  float* t;       // [batch][r*r]  P_k G_k
  float* bq;      // [batch][r*r]  b G + c G^2 (quintic)
  float* qt;      // [batch][r*r]  Q ping-pong partner of the cache
  NsWs ns;        // bf16 Gram-form slots over the same bytes as ga .. qt
  float* resid;   // [batch][tiles]
  int32_t* hc;    // [batch] has_cache snapshot
  int32_t* flags; // [batch] refresh decision
  int32_t* any;   // 1 iff some problem refreshes
  int32_t* any_hc;  // 1 iff some problem has a cache
  int32_t* dyn;   // [1 + batch] the refreshed problems: count, then indices
  int32_t* dyn_tiles;   // [kNsgMaxGroups + 1] tile layout of a launch over such lists
};

// The five float32 r x r buffers of the generic solve are one region; the
// bf16 Gram-form solve (five r x r bf16 slots per problem: NsWs amat, amat2
// and the three-slot tmp) uses its first half.
void carve_gram(Carver& cv, int batch, int m, int n, GramWs& w) {
  const int64_t r = m < n ? m : n;
  const size_t rr = (size_t)batch * r * r * 4;
  char* region = cv.take<char>(5 * rr);
  w.ga = reinterpret_cast<float*>(region);
  w.gb = reinterpret_cast<float*>(region + rr);
  w.t = reinterpret_cast<float*>(region + 2 * rr);
  w.bq = reinterpret_cast<float*>(region + 3 * rr);
  w.qt = reinterpret_cast<float*>(region + 4 * rr);
  w.ns.amat = region;                 // [batch][r*r] bf16
  w.ns.amat2 = region + rr / 2;       // [batch][r*r] bf16
  w.ns.tmp = region + rr;             // [batch][3 r*r] bf16
  w.resid = cv.take<float>((size_t)batch * gemm_tiles(0, (int)r, (int)r) * 4);
  w.hc = cv.take<int32_t>((size_t)batch * 4);
  w.flags = cv.take<int32_t>((size_t)batch * 4);
  w.any = cv.take<int32_t>(4);
  w.any_hc = cv.take<int32_t>(4);
  w.dyn = cv.take<int32_t>((size_t)(batch + 1) * 4);
  w.dyn_tiles = cv.take<int32_t>((size_t)(kNsgMaxGroups + 1) * 4);
}

// The fresh solve of CacheMuon in the Gram form on the persistent MFMA
// kernels (bf16 operands, cubic coefficients): the same chain as the
// Newton-Schulz Gram form (S_k = b G_k, P_k = S_k + aI, so G_{k+1} = P_k G_k
// P_k and Q_{k+1} = P_k Q_k are the products T_k = S_k P_k, S_{k+1} = T_k P_k,
// Q_{k+1} = Q_k P_k).  Every launch runs only the refreshed problems, listed
// on the device per plan (from the decision flags), and nothing when there
// are none (gate `any`); the plans (shape chunks) share each launch.  Q_K
// goes to the caches as whole float32 matrices.
struct GfFresh {
  const GfPlan* plan;
  const int32_t* flags;
  int32_t* dyn;
  const PtrTbl* qtbl;
  int qper;
};

sm_status gram_fresh_gf(const std::vector<GfFresh>& fr, const int32_t* any, int32_t* dyn_tiles,
                        hipStream_t s) {
  if (fr.empty()) return SM_OK;
  const int K = (int)fr[0].plan->T.size();
  auto listed = [](NsgGroup g, int32_t* dyn) {
    g.dyn = dyn;
    return g;
  };
  std::vector<NsgGroup> v;
  for (const GfFresh& f : fr) {
    if ((int)f.plan->T.size() != K || !f.plan->gram.c_low) return SM_ERR_UNSUPPORTED;
    SM_TRY(launch_compact_flags(f.flags, f.plan->batch, f.dyn, s));
    v.push_back(listed(f.plan->gram, f.dyn));
  }
  SM_TRY(launch_ns_groups(v, SM_K_GEMM_GRAM, s, any, dyn_tiles));
  for (int k = 0; k < K; ++k) {
    std::vector<NsgGroup> l1, l2;             // {T_k, Q_{k+1}}, then {S_{k+1}}
    for (const GfFresh& f : fr) {
      const GfPlan& g = *f.plan;
      if (g.T[k].batch) l1.push_back(listed(g.T[k], f.dyn));
      if (g.Q[k].batch) l1.push_back(listed(g.Q[k], f.dyn));
      if (g.S[k].batch) l2.push_back(listed(g.S[k], f.dyn));
    }
    if (!l1.empty()) SM_TRY(launch_ns_groups(l1, SM_K_GEMM_RR, s, any, dyn_tiles));
    if (!l2.empty()) SM_TRY(launch_ns_groups(l2, SM_K_GEMM_RR, s, any, dyn_tiles));
  }
  v.clear();
  for (const GfFresh& f : fr) v.push_back(listed(f.plan->apply, f.dyn));
  SM_TRY(launch_ns_groups(v, SM_K_GEMM_APPLY, s, any, dyn_tiles));
  for (const GfFresh& f : fr) {   // q_store reads the lower-stored Q_K
    const GfPlan& g = *f.plan;
    SM_TRY(launch_q_store(g.qk.p, g.qk.st, g.r, *f.qtbl, f.qper, f.flags, g.batch, s));
  }
  return SM_OK;
}

// One batch of same-shaped CacheMuon problems.  Problem b's Q lives at
// qtbl[b / qper] + (b % qper) * r*r floats, its {has_cache, a_t} pair at
// cstbl[b / qper] + (b % qper) * 2 ints, its diagnostic row (err, refreshed)
// at diag[b / qper] + (b % qper) * 2 floats when has_diag.  The NS input is x
// ([batch][m][n]) or, with xtbl, worker b % xper of matrix b / xper read in
// place (the persistent kernels only: see gram_fast_plan).
struct GramJob {
  const void* x;
  const PtrTbl* xtbl;
  int xper;
  void* d;
  PtrTbl qtbl, cstbl;
  int qper;
  float* err_out;
  int32_t* refr_out;
  PtrTbl diag;
  bool has_diag;
  GramWs w;
  const float* scale;
  int batch, m, n;
};

// The persistent-kernel route of a job (bf16, cubic, one-term identity, and
// shapes the kernels take): the fresh solve's Gram-form chain, the candidate
// D_hat = s Q x (x Q^T when tall) with Q rounded to bf16 (the operand type
// the generic kernel would round it to), and the probe's residual partials
// of D_hat D_hat^T - I.
struct GramFast {
  GfPlan gf;
  NsgGroup ap, pr;
};

bool gram_fast_plan(const GramJob& j, int dt, const sm_ns_params& p, GramFast& f) {
  if (dt != BF16 || p.c != 0.f || p.iters < 2) return false;
  uint32_t hi = 0, lo = 0;
  if (ns_ident_split(p.a, &hi, &lo) != 1) return false;
  NsJob job{j.x, j.d, j.w.ns, j.scale, j.batch, j.m, j.n};
  job.xtbl = j.xtbl;
  job.xper = j.xper;
  if (!gf_plan(job, p, f.gf, true) || !f.gf.gram.c_low) return false;
  const bool wide = j.m <= j.n;
  const int r = wide ? j.m : j.n;
  const int64_t rr = (int64_t)r * r, mn = (int64_t)j.m * j.n;
  const bf16_t* qb = static_cast<const bf16_t*>(j.w.ns.amat);
  const bf16_t* xb = static_cast<const bf16_t*>(j.x);
  const int tb = j.xtbl ? 1 : 0;
  NsgGroup& ap = f.ap;
  std::memset(&ap, 0, sizeof(ap));
  if (wide) {
    ap.a = qb; ap.lda = r; ap.sa = rr;
    ap.b = xb; ap.ldb = j.n; ap.sb = mn; ap.b_kr = 1; ap.b_tbl = tb;
  } else {
    ap.a = xb; ap.lda = j.n; ap.sa = mn; ap.a_tbl = tb;
    ap.b = qb; ap.ldb = r; ap.sb = rr;
  }
  ap.tbl = j.xtbl; ap.tbl_per = j.xper;
  ap.c = static_cast<bf16_t*>(j.d); ap.ldc = j.n; ap.sc = mn;
  ap.scale = j.scale; ap.alpha_pow = j.scale ? 1 : 0; ap.alpha = 1.f;
  ap.M = j.m; ap.N = j.n; ap.K = r; ap.batch = j.batch;
  ap.pred = j.w.hc;
  NsgGroup& pr = f.pr;
  std::memset(&pr, 0, sizeof(pr));
  const bf16_t* db = static_cast<const bf16_t*>(j.d);
  pr.a = db; pr.lda = j.n; pr.sa = mn; pr.a_kr = wide ? 0 : 1;
  pr.b = db; pr.ldb = j.n; pr.sb = mn; pr.b_kr = wide ? 0 : 1;
  pr.alpha = 1.f;
  pr.M = r; pr.N = r; pr.K = wide ? j.n : j.m; pr.batch = j.batch; pr.sym = 1;
  pr.resid = j.w.resid;
  return gemm_ns_supported(ap) && gemm_ns_supported(pr);
}

// The generic route's candidate: D_hat = s * Q x (s * x Q^T for a tall x) and
// the residual partials of D_hat D_hat^T - I, for the problems with a cache.
sm_status gram_generic_candidate(const GramJob& j, int dt, hipStream_t s) {
  GemmArgs g = apply_args(j.qtbl.p[0], F32, 1, j.x, dt, j.batch, j.m, j.n);
  g.tbl = j.qtbl; g.tbl_per = j.qper;
  g.c = j.d; g.ldc = j.n; g.sc = (int64_t)j.m * j.n; g.c_dt = dt;
  g.scale = j.scale; g.alpha_pow = 1;
  g.pred = j.w.hc; g.pred_stride = 1; g.pred_val = 1;
  SM_TRY(launch_gemm(g, dt, SM_K_GEMM_APPLY, s));
  GemmArgs pr = gram_args(j.d, dt, j.batch, j.m, j.n);
  pr.resid = j.w.resid;
  pr.pred = j.w.hc; pr.pred_stride = 1; pr.pred_val = 1;
  return launch_gemm(pr, dt, SM_K_PROBE, s);
}

// The generic route's fresh Gram-NS, predicated on the decision flags:
// G_0 = X X^T, P_k = aI + B_k with B_k = b G_k + c G_k^2, Q_{k+1} = a Q_k +
// B_k Q_k, G_{k+1} = a T_k + T_k B_k with T_k = a G_k + B_k G_k, D = Q_K X.
// The identity parts are added in float32 in the GEMM epilogues; Q_K is
// written straight into the cache.
sm_status gram_generic_fresh(const GramJob& j, int dt, const sm_ns_params& p, hipStream_t s) {
  const GramWs& w = j.w;
  const PtrTbl& qtbl = j.qtbl;
  const int qper = j.qper, batch = j.batch, m = j.m, n = j.n;
  const void* x = j.x;
  const int r = m <= n ? m : n;
  const int64_t rr = (int64_t)r * r;
  const int K = p.iters;
  const bool quintic = p.c != 0.f;
  // Q_k lives in the cache for k == K (mod 2) so that Q_K lands there.
  auto qbuf_is_cache = [&](int k) { return ((K - k) % 2) == 0; };
  auto set_q_out = [&](GemmArgs& g, int k) {  // write Q_k as output c
    if (qbuf_is_cache(k)) { g.c = const_cast<char*>(qtbl.p[0]); g.c_tbl = 1; }
    else { g.c = w.qt; g.c_tbl = 0; }
    g.ldc = r; g.sc = rr; g.c_dt = F32;
  };
  auto pred_fresh = [&](GemmArgs& g) {
    g.pred = w.flags; g.pred_stride = 1; g.pred_val = 1;
    g.tbl = qtbl; g.tbl_per = qper;
  };

  // G_0 = s^2 x x^T, and Q_1 = aI + B_0
  {
    GemmArgs g = gram_args(x, dt, batch, m, n);
    pred_fresh(g);
    g.c = w.ga; g.ldc = r; g.sc = rr; g.c_dt = F32;
    g.scale = j.scale; g.alpha_pow = 2;
    if (!quintic) {
      if (qbuf_is_cache(1)) { g.c2 = reinterpret_cast<float*>(const_cast<char*>(qtbl.p[0])); g.c2_tbl = 1; }
      else { g.c2 = w.qt; g.c2_tbl = 0; }
      g.ldc2 = r; g.sc2 = rr; g.c2_diag = p.a; g.c2_scale = p.b;
    }
    SM_TRY(launch_gemm(g, dt, SM_K_GEMM_GRAM, s));
  }
  auto make_bq = [&](const float* gk, bool write_q1) -> sm_status {
    GemmArgs g = gemm_base(r, r, r, batch);
    pred_fresh(g);
    g.a = opnd(gk, r, rr, F32, KC);
    g.b = opnd(gk, r, rr, F32, RC);
    g.cin = gk; g.ldcin = r; g.scin = rr;
    g.c = w.bq; g.ldc = r; g.sc = rr; g.c_dt = F32;
    g.alpha = p.c; g.beta = p.b;
    if (write_q1) {
      if (qbuf_is_cache(1)) { g.c2 = reinterpret_cast<float*>(const_cast<char*>(qtbl.p[0])); g.c2_tbl = 1; }
      else { g.c2 = w.qt; g.c2_tbl = 0; }
      g.ldc2 = r; g.sc2 = rr; g.c2_diag = p.a; g.c2_scale = 1.f;
    }
    return launch_gemm(g, dt, SM_K_GEMM_RR, s);
  };
  if (quintic) SM_TRY(make_bq(w.ga, true));

  float* gprev = w.ga;
  float* gnew = w.gb;
  for (int k = 1; k < K; ++k) {
    // T = a G + B G
    {
      GemmArgs g = gemm_base(r, r, r, batch);
      pred_fresh(g);
      g.a = quintic ? opnd(w.bq, r, rr, F32, KC) : opnd(gprev, r, rr, F32, KC);
      g.b = opnd(gprev, r, rr, F32, RC);
      g.cin = gprev; g.ldcin = r; g.scin = rr;
      g.c = w.t; g.ldc = r; g.sc = rr; g.c_dt = F32;
      g.alpha = quintic ? 1.f : p.b; g.beta = p.a;
      SM_TRY(launch_gemm(g, dt, SM_K_GEMM_RR, s));
    }
    // G_k = a T + T B
    {
      GemmArgs g = gemm_base(r, r, r, batch);
      pred_fresh(g);
      g.a = opnd(w.t, r, rr, F32, KC);
      g.b = quintic ? opnd(w.bq, r, rr, F32, RC) : opnd(gprev, r, rr, F32, RC);
      g.cin = w.t; g.ldcin = r; g.scin = rr;
      g.c = gnew; g.ldc = r; g.sc = rr; g.c_dt = F32;
      g.alpha = quintic ? 1.f : p.b; g.beta = p.a;
      SM_TRY(launch_gemm(g, dt, SM_K_GEMM_RR, s));
    }
    if (quintic) SM_TRY(make_bq(gnew, false));
    // Q_{k+1} = a Q_k + B_k Q_k
    {
      GemmArgs g = gemm_base(r, r, r, batch);
      pred_fresh(g);
      g.a = quintic ? opnd(w.bq, r, rr, F32, KC) : opnd(gnew, r, rr, F32, KC);
      const bool qc = qbuf_is_cache(k);
      const void* qk = qc ? static_cast<const void*>(qtbl.p[0]) : static_cast<const void*>(w.qt);
      g.b = opnd(qk, r, rr, F32, RC, qc ? 1 : 0);
      g.cin = qk; g.cin_tbl = qc ? 1 : 0; g.ldcin = r; g.scin = rr;
      set_q_out(g, k + 1);
      g.alpha = quintic ? 1.f : p.b; g.beta = p.a;
      SM_TRY(launch_gemm(g, dt, SM_K_GEMM_RR, s));
    }
    float* tmp = gprev; gprev = gnew; gnew = tmp;
  }
  // D = s * Q_K x
  GemmArgs g = apply_args(qtbl.p[0], F32, 1, x, dt, batch, m, n);
  pred_fresh(g);
  g.c = j.d; g.ldc = n; g.sc = (int64_t)m * n; g.c_dt = dt;
  g.scale = j.scale; g.alpha_pow = 1;
  return launch_gemm(g, dt, SM_K_GEMM_APPLY, s);
}

// CacheMuon's orthogonalisation of every problem of the jobs,
// [CacheMuon-ja] core mechanism:
//   candidate (if cached): D_hat = Q X, err = ||D_hat D_hat^T - I||_F / sqrt(r)
//   refresh iff no cache / forced / err > gamma, decided on the device;
//   fresh Gram-NS for the refreshed problems only.
// Jobs on the persistent kernels share their candidate launches (one apply
// and one probe launch for all of them, gated by one device flag: some
// problem has a cache); each job's decision and fresh solve are its own.
sm_status gram_jobs(const std::vector<GramJob>& jobs, int dt, const sm_ns_params& p, float gamma,
                    int mode, int64_t t, hipStream_t s) {
  const size_t nj = jobs.size();
  std::vector<GramFast> fp(nj);
  std::vector<char> fast(nj, 0);
  for (size_t i = 0; i < nj; ++i) {
    fast[i] = gram_fast_plan(jobs[i], dt, p, fp[i]);
    if (!fast[i] && (jobs[i].xtbl || !jobs[i].x)) return SM_ERR_UNSUPPORTED;
  }
  for (const GramJob& j : jobs)
    SM_TRY(launch_gather_has_cache(j.cstbl, j.qper, j.batch, j.w.hc, s));
  if (mode != 1) {
    FlagSets fs;
    std::memset(&fs, 0, sizeof(fs));
    std::vector<NsgGroup> ap, pr;
    int32_t* any_hc = nullptr;
    for (size_t i = 0; i < nj; ++i) {
      if (!fast[i]) continue;
      if (fs.count == kTbl) return SM_ERR_UNSUPPORTED;
      fs.f[fs.count] = jobs[i].w.hc;
      fs.n[fs.count] = jobs[i].batch;
      ++fs.count;
      if (!any_hc) any_hc = jobs[i].w.any_hc;
      ap.push_back(fp[i].ap);
      pr.push_back(fp[i].pr);
    }
    if (any_hc) {
      SM_TRY(launch_any_flags(fs, any_hc, s));
      for (size_t i = 0; i < nj; ++i) {
        if (!fast[i]) continue;
        const GramJob& j = jobs[i];
        const int r = j.m <= j.n ? j.m : j.n;
        SM_TRY(launch_q_load(j.qtbl, j.qper, r, static_cast<bf16_t*>(j.w.ns.amat),
                             (int64_t)r * r, j.w.hc, j.batch, s));
      }
      SM_TRY(launch_ns_groups(ap, SM_K_GEMM_APPLY, s, any_hc));
      SM_TRY(launch_ns_groups(pr, SM_K_PROBE, s, any_hc));
    }
    for (size_t i = 0; i < nj; ++i)
      if (!fast[i]) SM_TRY(gram_generic_candidate(jobs[i], dt, s));
  }
  for (size_t i = 0; i < nj; ++i) {
    const GramJob& j = jobs[i];
    const int r = j.m <= j.n ? j.m : j.n;
    const int parts = fast[i] ? ns_probe_parts(r) : gemm_tiles(dt, r, r);
    SM_TRY(launch_cache_decide(j.w.resid, parts, j.batch, r, j.w.hc, j.cstbl, j.qper, mode,
                               gamma, t, j.w.flags, j.err_out, j.refr_out,
                               j.has_diag ? &j.diag : nullptr, s));
  }
  // fresh solves: the persistent-kernel jobs share their launches, gated by
  // one device flag (some problem of some job refreshes)
  {
    FlagSets fs;
    std::memset(&fs, 0, sizeof(fs));
    std::vector<GfFresh> fr;
    int32_t* any = nullptr;
    int32_t* dyn_tiles = nullptr;
    for (size_t i = 0; i < nj; ++i) {
      if (!fast[i]) continue;
      const GramJob& j = jobs[i];
      fs.f[fs.count] = j.w.flags;
      fs.n[fs.count] = j.batch;
      ++fs.count;
      if (!any) {
        any = j.w.any;
        dyn_tiles = j.w.dyn_tiles;
      }
      fr.push_back(GfFresh{&fp[i].gf, j.w.flags, j.w.dyn, &j.qtbl, j.qper});
    }
    if (any) {
      SM_TRY(launch_any_flags(fs, any, s));
      SM_TRY(gram_fresh_gf(fr, any, dyn_tiles, s));
    }
  }
  for (size_t i = 0; i < nj; ++i)
    if (!fast[i]) SM_TRY(gram_generic_fresh(jobs[i], dt, p, s));
  return SM_OK;
}

// Whether a step's CacheMuon chunk can read its momenta in place (the
// persistent-kernel route takes it with the pointer table).
bool gram_in_place_ok(const GramJob& j, int dt, const sm_ns_params& p) {
  GramFast f;
  return gram_fast_plan(j, dt, p, f);
}

// ------------------------------------------------------------------ step planning

struct Chunk {
  int m, n;
  std::vector<int> mats;  // <= kTbl matrix indices, all of shape m x n
};

std::vector<Chunk> plan_chunks(const sm_matrix* mats, int nmat) {
  std::vector<Chunk> out;
  std::vector<char> used(nmat, 0);
  for (int i = 0; i < nmat; ++i) {
    if (used[i]) continue;
    Chunk c;
    c.m = mats[i].m;
    c.n = mats[i].n;
    for (int j = i; j < nmat; ++j) {
      if (used[j] || mats[j].m != c.m || mats[j].n != c.n) continue;
      used[j] = 1;
      c.mats.push_back(j);
      if ((int)c.mats.size() == kTbl) {
        out.push_back(c);
        c.mats.clear();
      }
    }
    if (!c.mats.empty()) out.push_back(c);
  }
  return out;
}

struct ChunkWs {
  void* x0;          // NS input copy (and the vote matrix of the polar step)
  void* d;
  NsWs ns;
  GramWs gram;
  float* partials;
  float* scale;
  uint64_t* bits;    // packed signs [B][words]   (SM_ENC_BITS)
  int8_t* s8;        // int8 signs   [B][count]   (SM_ENC_INT8)
};

void carve_chunk(Carver& cv, const sm_config& c, const Chunk& ch, ChunkWs& w) {
  const int B = (int)ch.mats.size() * c.M;
  const int64_t count = (int64_t)ch.m * ch.n;
  const size_t es = dt_size(c.mdt);
  const int64_t words = (count + 63) / 64;
  const bool ns_possible = !(c.algo == SM_LION_MUON && c.period == 0) || c.vote_polar;
  std::memset(&w, 0, sizeof(w));
  if (c.encoding == SM_ENC_INT8)
    w.s8 = cv.take<int8_t>((size_t)B * count);
  else
    w.bits = cv.take<uint64_t>((size_t)B * words * 8);
  if (!ns_possible) return;
  w.partials = cv.take<float>((size_t)B * kNormParts * 4);
  w.scale = cv.take<float>((size_t)B * 4);
  w.x0 = cv.take<void>((size_t)B * count * es);
  w.d = cv.take<void>((size_t)B * count * es);
  if (c.algo == SM_CACHE_MUON) carve_gram(cv, B, ch.m, ch.n, w.gram);
  if (c.algo != SM_CACHE_MUON || c.vote_polar) carve_ns(cv, c.mdt, B, ch.m, ch.n, w.ns);
}

sm_status check_config(const sm_config* c) {
  if (!c) return SM_ERR_ARG;
  if (c->algo < SM_SIGN_MUON || c->algo > SM_LION_MUON) return SM_ERR_ARG;
  if (c->update != SM_UPDATE_VOTE && c->update != SM_UPDATE_POLAR) return SM_ERR_ARG;
  if (!valid_dt(c->wdt) || !valid_dt(c->mdt) || !valid_dt(c->gdt)) return SM_ERR_DTYPE;
  if (!finite(c->lr) || !finite(c->beta1) || !finite(c->beta2)) return SM_ERR_ARG;
  if (c->period < 0) return SM_ERR_ARG;
  if (c->cache_mode < 0 || c->cache_mode > 2) return SM_ERR_ARG;
  if (std::isnan(c->gamma)) return SM_ERR_ARG;
  SM_TRY(check_ns_params(&c->ns));
  if (c->M < 1 || c->M > 64) return SM_ERR_UNSUPPORTED;
  if (c->update == SM_UPDATE_POLAR && (c->M != 1 || c->algo == SM_SIGN_MUON))
    return SM_ERR_UNSUPPORTED;
  if (c->encoding != SM_ENC_BITS && c->encoding != SM_ENC_INT8) return SM_ERR_ARG;
  if (c->vote_polar != 0 && c->vote_polar != 1) return SM_ERR_ARG;
  return SM_OK;
}

sm_status check_mats(const sm_config& c, const sm_matrix* mats, int nmat) {
  if (!mats || nmat < 1) return SM_ERR_ARG;
  for (int i = 0; i < nmat; ++i) {
    const sm_matrix& a = mats[i];
    SM_TRY(check_shape(1, a.m, a.n));
    if (!a.w || !a.mom || !a.grad) return SM_ERR_ARG;
    if (!al16(a.w) || !al16(a.mom) || !al16(a.grad)) return SM_ERR_ARG;
    if (c.algo == SM_CACHE_MUON) {
      if (!a.q_cache || !a.cache_state || !al16(a.q_cache) || !al16(a.cache_state))
        return SM_ERR_ARG;
    }
  }
  return SM_OK;
}

size_t step_ws_bytes(const sm_config& c, const std::vector<Chunk>& chunks) {
  Carver cv(nullptr);
  for (const Chunk& ch : chunks) {
    ChunkWs w;
    carve_chunk(cv, c, ch, w);
  }
  return cv.off + 256;
}

}  // namespace
}  // namespace sm

// ====================================================================== C ABI

using namespace sm;

extern "C" {

const char* sm_status_string(int s) {
  switch (s) {
    case SM_OK: return "SM_OK";
    case SM_ERR_ARG: return "SM_ERR_ARG: invalid argument";
    case SM_ERR_SHAPE: return "SM_ERR_SHAPE: invalid shape";
    case SM_ERR_DTYPE: return "SM_ERR_DTYPE: invalid dtype";
    case SM_ERR_WORKSPACE: return "SM_ERR_WORKSPACE: workspace too small";
    case SM_ERR_UNSUPPORTED: return "SM_ERR_UNSUPPORTED: unsupported configuration";
    case SM_ERR_HIP: return "SM_ERR_HIP: HIP runtime error";
    default: return "unknown sm_status";
  }
}

int sm_last_hip_error(void) { return g_last_hip.load(); }

int sm_version(void) { return 4; }

sm_status sm_ns_polar_ws(int dt, int batch, int m, int n, size_t* ws_bytes) {
  if (!ws_bytes) return SM_ERR_ARG;
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  SM_TRY(check_shape(batch, m, n));
  Carver cv(nullptr);
  NsWs w;
  carve_ns(cv, dt, batch, m, n, w);
  cv.take<float>((size_t)batch * kNormParts * 4);
  cv.take<float>((size_t)batch * 4);
  *ws_bytes = cv.off + 256;
  return SM_OK;
}

sm_status sm_ns_polar(const void* x, void* u, int dt, int batch, int m, int n, int normalize,
                      const sm_ns_params* p, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  SM_TRY(check_shape(batch, m, n));
  SM_TRY(check_ns_params(p));
  if (!x || !u || !ws || !al16(x) || !al16(u) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return SM_ERR_ARG;
  if (normalize != 0 && normalize != 1) return SM_ERR_ARG;
  const size_t bytes = (size_t)batch * m * n * dt_size(dt);
  if (overlap(x, bytes, u, bytes)) return SM_ERR_ARG;
  size_t need = 0;
  SM_TRY(sm_ns_polar_ws(dt, batch, m, n, &need));
  if (ws_bytes < need) return SM_ERR_WORKSPACE;
  if (overlap(ws, ws_bytes, x, bytes) || overlap(ws, ws_bytes, u, bytes)) return SM_ERR_ARG;

  Carver cv(ws);
  NsWs w;
  carve_ns(cv, dt, batch, m, n, w);
  float* partials = cv.take<float>((size_t)batch * kNormParts * 4);
  float* scale = cv.take<float>((size_t)batch * 4);
  const int64_t count = (int64_t)m * n;
  if (normalize) {
    SM_TRY(launch_sumsq(x, dt, batch, count, partials, s));
    SM_TRY(launch_scale_finalize(partials, batch, count, p->eps, scale, s));
  }
  return ns_core(x, u, w, normalize ? scale : nullptr, dt, batch, m, n, *p, s);
}

}  // extern "C"

// ------------------------------------------------------------------ static scratch

// Scratch of sm_ns_polar_noalloc: a file-scope device array (each device the
// library runs on holds its own copy until the process ends).  In host code
// `scratch` names a host-side stand-in, never a device address: the device
// address comes from hipGetSymbolAddress, once per device, and only that
// pointer is passed to kernels.
__device__ __align__(256) unsigned char scratch[SM_NS_NOALLOC_MAX_WS];

namespace {
std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device ordinal -> device address of `scratch`

sm_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return SM_OK;
}
}  // namespace

extern "C" {

sm_status sm_ns_polar_noalloc(const void* x, void* u, int dt, int batch, int m, int n,
                              int normalize, const sm_ns_params* p, hipStream_t s) {
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  SM_TRY(check_shape(batch, m, n));
  SM_TRY(check_ns_params(p));
  if (!x || !u || !al16(x) || !al16(u)) return SM_ERR_ARG;
  if (normalize != 0 && normalize != 1) return SM_ERR_ARG;
  size_t need = 0;
  SM_TRY(sm_ns_polar_ws(dt, batch, m, n, &need));
  if (need > (size_t)SM_NS_NOALLOC_MAX_WS) return SM_ERR_WORKSPACE;
  void* ws = nullptr;
  SM_TRY(scratch_address(&ws));
  return sm_ns_polar(x, u, dt, batch, m, n, normalize, p, ws, (size_t)SM_NS_NOALLOC_MAX_WS, s);
}

sm_status sm_gram_ns_cached_ws(int dt, int batch, int m, int n, size_t* ws_bytes) {
  if (!ws_bytes) return SM_ERR_ARG;
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  SM_TRY(check_shape(batch, m, n));
  Carver cv(nullptr);
  GramWs w;
  carve_gram(cv, batch, m, n, w);
  cv.take<float>((size_t)batch * kNormParts * 4);
  cv.take<float>((size_t)batch * 4);
  *ws_bytes = cv.off + 256;
  return SM_OK;
}

sm_status sm_gram_ns_cached(const void* x, void* d, float* q, int32_t* cache_state, float* err,
                            int32_t* refreshed, int dt, int batch, int m, int n, int normalize,
                            const sm_ns_params* p, float gamma, int mode, int64_t t, void* ws,
                            size_t ws_bytes, hipStream_t s) {
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  SM_TRY(check_shape(batch, m, n));
  SM_TRY(check_ns_params(p));
  if (!x || !d || !q || !cache_state || !ws) return SM_ERR_ARG;
  if (!al16(x) || !al16(d) || !al16(q) || !al16(cache_state)) return SM_ERR_ARG;
  if ((err && !al16(err)) || (refreshed && !al16(refreshed))) return SM_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return SM_ERR_ARG;
  if (normalize != 0 && normalize != 1) return SM_ERR_ARG;
  if (mode < 0 || mode > 2 || std::isnan(gamma)) return SM_ERR_ARG;
  const size_t bytes = (size_t)batch * m * n * dt_size(dt);
  if (overlap(x, bytes, d, bytes)) return SM_ERR_ARG;
  size_t need = 0;
  SM_TRY(sm_gram_ns_cached_ws(dt, batch, m, n, &need));
  if (ws_bytes < need) return SM_ERR_WORKSPACE;
  // the workspace must not alias any caller buffer the call reads or writes
  const int r = m < n ? m : n;
  const size_t qbytes = (size_t)batch * r * r * sizeof(float);
  const size_t sbytes = (size_t)batch * 2 * sizeof(int32_t);
  if (overlap(ws, ws_bytes, x, bytes) || overlap(ws, ws_bytes, d, bytes) ||
      overlap(ws, ws_bytes, q, qbytes) || overlap(ws, ws_bytes, cache_state, sbytes) ||
      (err && overlap(ws, ws_bytes, err, (size_t)batch * 4)) ||
      (refreshed && overlap(ws, ws_bytes, refreshed, (size_t)batch * 4)))
    return SM_ERR_ARG;
  if (overlap(q, qbytes, x, bytes) || overlap(q, qbytes, d, bytes)) return SM_ERR_ARG;

  Carver cv(ws);
  GramWs w;
  carve_gram(cv, batch, m, n, w);
  float* partials = cv.take<float>((size_t)batch * kNormParts * 4);
  float* scale = cv.take<float>((size_t)batch * 4);
  if (normalize) {
    SM_TRY(launch_sumsq(x, dt, batch, (int64_t)m * n, partials, s));
    SM_TRY(launch_scale_finalize(partials, batch, (int64_t)m * n, p->eps, scale, s));
  }
  GramJob j;
  std::memset(&j, 0, sizeof(j));
  j.x = x;
  j.xper = 1;
  j.d = d;
  j.qtbl = tbl_one(q);
  j.cstbl = tbl_one(cache_state);
  j.qper = batch;
  j.err_out = err;
  j.refr_out = refreshed;
  j.w = w;
  j.scale = normalize ? scale : nullptr;
  j.batch = batch;
  j.m = m;
  j.n = n;
  return gram_jobs(std::vector<GramJob>{j}, dt, *p, gamma, mode, t, s);
}

sm_status sm_sign_pack(const void* x, int dt, int64_t count, uint64_t* bits, hipStream_t s) {
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  if (count < 0) return SM_ERR_SHAPE;
  if (count == 0) return SM_OK;
  if (!x || !bits) return SM_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(x) % dt_size(dt)) || (reinterpret_cast<uintptr_t>(bits) & 7u))
    return SM_ERR_ARG;
  return launch_sign_pack(x, dt, 1, count, bits, (count + 63) / 64, s);
}

sm_status sm_vote_update(const uint64_t* bits, int M, int64_t words_stride, int64_t count,
                         void* w, int wdt, float lr, int8_t* vote_out, hipStream_t s) {
  if (!valid_dt(wdt)) return SM_ERR_DTYPE;
  if (count < 0) return SM_ERR_SHAPE;
  if (M < 1 || M > 64) return SM_ERR_UNSUPPORTED;
  if (count == 0) return SM_OK;
  if (!bits || !w || !al16(w) || (reinterpret_cast<uintptr_t>(bits) & 7u)) return SM_ERR_ARG;
  if (words_stride < (count + 63) / 64 || !finite(lr)) return SM_ERR_ARG;
  const PtrTbl wt = tbl_one(w);
  return launch_vote(SM_ENC_BITS, bits, M, words_stride, 0, 1, count, wt, wdt, lr, vote_out,
                     true, s);
}

sm_status sm_sign_int8(const void* x, int dt, int64_t count, int8_t* sg, hipStream_t s) {
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  if (count < 0) return SM_ERR_SHAPE;
  if (count == 0) return SM_OK;
  if (!x || !sg || (reinterpret_cast<uintptr_t>(x) % dt_size(dt))) return SM_ERR_ARG;
  if (overlap(x, (size_t)count * dt_size(dt), sg, (size_t)count)) return SM_ERR_ARG;
  return launch_sign_int8(x, dt, 1, count, sg, s);
}

sm_status sm_vote_update_int8(const int8_t* sg, int M, int64_t stride, int64_t count, void* w,
                              int wdt, float lr, int8_t* vote_out, hipStream_t s) {
  if (!valid_dt(wdt)) return SM_ERR_DTYPE;
  if (count < 0) return SM_ERR_SHAPE;
  if (M < 1 || M > 64) return SM_ERR_UNSUPPORTED;
  if (count == 0) return SM_OK;
  if (!sg || !w || !al16(w)) return SM_ERR_ARG;
  if (stride < count || !finite(lr)) return SM_ERR_ARG;
  const PtrTbl wt = tbl_one(w);
  return launch_vote(SM_ENC_INT8, sg, M, stride, 0, 1, count, wt, wdt, lr, vote_out, true, s);
}

sm_status sm_vote(const void* signs, int encoding, int M, int64_t stride, int64_t count, void* v,
                  int vdt, hipStream_t s) {
  if (!valid_dt(vdt)) return SM_ERR_DTYPE;
  if (count < 0) return SM_ERR_SHAPE;
  if (M < 1 || M > 64) return SM_ERR_UNSUPPORTED;
  if (encoding != SM_ENC_BITS && encoding != SM_ENC_INT8) return SM_ERR_ARG;
  if (count == 0) return SM_OK;
  if (!signs || !v || !al16(v)) return SM_ERR_ARG;
  if (encoding == SM_ENC_BITS) {
    if ((reinterpret_cast<uintptr_t>(signs) & 7u) || stride < (count + 63) / 64) return SM_ERR_ARG;
  } else if (stride < count) {
    return SM_ERR_ARG;
  }
  const PtrTbl vt = tbl_one(v);
  return launch_vote(encoding, signs, M, stride, 0, 1, count, vt, vdt, 0.f, nullptr, false, s);
}

sm_status sm_polar_update(void* w, int wdt, const void* d, int ddt, int64_t count, float lr,
                          hipStream_t s) {
  if (!valid_dt(wdt) || !valid_dt(ddt)) return SM_ERR_DTYPE;
  if (count < 0) return SM_ERR_SHAPE;
  if (count == 0) return SM_OK;
  if (!w || !d || !al16(w) || !al16(d) || !finite(lr)) return SM_ERR_ARG;
  if (overlap(w, (size_t)count * dt_size(wdt), d, (size_t)count * dt_size(ddt))) return SM_ERR_ARG;
  const PtrTbl wt = tbl_one(w);
  return launch_polar_update(d, ddt, 1, count, wt, wdt, lr, s);
}

sm_status sm_spectral_norm_ws(int batch, int m, int n, size_t* ws_bytes) {
  if (!ws_bytes) return SM_ERR_ARG;
  SM_TRY(check_shape(batch, m, n));
  *ws_bytes = spectral_norm_ws_bytes(batch, m, n);
  return SM_OK;
}

sm_status sm_spectral_norm(const void* a, const void* b, int dt, int batch, int m, int n,
                           const float* v0, int iters, float* out, void* ws, size_t ws_bytes,
                           hipStream_t s) {
  if (!valid_dt(dt)) return SM_ERR_DTYPE;
  SM_TRY(check_shape(batch, m, n));
  if (!a || !v0 || !out || !ws || iters < 0 || iters > 100000) return SM_ERR_ARG;
  const uintptr_t es = dt_size(dt);
  if ((reinterpret_cast<uintptr_t>(a) % es) || (b && (reinterpret_cast<uintptr_t>(b) % es)))
    return SM_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(v0) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u) ||
      (reinterpret_cast<uintptr_t>(ws) & 255u))
    return SM_ERR_ARG;
  const size_t need = spectral_norm_ws_bytes(batch, m, n);
  if (ws_bytes < need) return SM_ERR_WORKSPACE;
  if (overlap(out, (size_t)batch * 4, ws, ws_bytes) || overlap(v0, (size_t)batch * n * 4, ws, ws_bytes))
    return SM_ERR_ARG;
  return launch_spectral_norm(a, b, dt, batch, m, n, v0, iters, out, ws, s);
}

sm_status sm_step_ws(const sm_config* c, const sm_matrix* mats, int nmat, size_t* ws_bytes) {
  if (!ws_bytes) return SM_ERR_ARG;
  SM_TRY(check_config(c));
  if (!mats || nmat < 1) return SM_ERR_ARG;
  for (int i = 0; i < nmat; ++i) SM_TRY(check_shape(1, mats[i].m, mats[i].n));
  *ws_bytes = step_ws_bytes(*c, plan_chunks(mats, nmat));
  return SM_OK;
}

sm_status sm_step(const sm_config* c, const sm_matrix* mats, int nmat, int64_t t, void* ws,
                  size_t ws_bytes, float* diag, hipStream_t s) {
  SM_TRY(check_config(c));
  SM_TRY(check_mats(*c, mats, nmat));
  if (t < 1 || !ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SM_ERR_ARG;
  if (diag && !al16(diag)) return SM_ERR_ARG;
  const std::vector<Chunk> chunks = plan_chunks(mats, nmat);
  if (ws_bytes < step_ws_bytes(*c, chunks)) return SM_ERR_WORKSPACE;

  const int M = c->M;
  const bool muon_step =
      (c->algo != SM_LION_MUON) || (c->period > 0 && (t % c->period) == 0);
  const bool polar = c->update == SM_UPDATE_POLAR && muon_step;
  // Tables of the chunks' per-matrix pointers.
  struct ChunkRun {
    ChunkWs w;
    PtrTbl mom, grad, wt, qt, cs;
    int nc, B;
    int64_t count, words;
    NsJob job;          // direct NS of this chunk
    GramJob gjob;       // CacheMuon: the chunk's orthogonalisation
    bool grouped;       // job runs in the grouped launches
    bool fused_signs;   // its last product writes the packed signs (no a7/a8 launch)
  };
  std::vector<ChunkRun> runs(chunks.size());
  Carver cv(ws);
  for (size_t ci = 0; ci < chunks.size(); ++ci) {
    const Chunk& ch = chunks[ci];
    ChunkRun& r = runs[ci];
    carve_chunk(cv, *c, ch, r.w);
    r.nc = (int)ch.mats.size();
    r.B = r.nc * M;
    r.count = (int64_t)ch.m * ch.n;
    r.words = (r.count + 63) / 64;
    std::memset(&r.mom, 0, sizeof(r.mom));
    std::memset(&r.grad, 0, sizeof(r.grad));
    std::memset(&r.wt, 0, sizeof(r.wt));
    std::memset(&r.qt, 0, sizeof(r.qt));
    std::memset(&r.cs, 0, sizeof(r.cs));
    for (int j = 0; j < r.nc; ++j) {
      const sm_matrix& a = mats[ch.mats[j]];
      r.mom.p[j] = static_cast<const char*>(a.mom);
      r.grad.p[j] = static_cast<const char*>(a.grad);
      r.wt.p[j] = static_cast<const char*>(a.w);
      r.qt.p[j] = reinterpret_cast<const char*>(a.q_cache);
      r.cs.p[j] = reinterpret_cast<const char*>(a.cache_state);
    }
    // Direct NS input: Sign-Muon's is the momentum itself (Y = M), read in
    // place through the pointer table when the grouped kernel takes it, so
    // a1 writes no copy; LionMuon's is the interpolation Ghat, which only
    // exists as the copy a1 writes.
    r.grouped = false;
    r.fused_signs = false;
    if (c->algo == SM_CACHE_MUON) {
      // diag rows follow the caller's matrix order: the chunk's matrix j
      // (any position in that order) has its M rows at diag + mats[j]*M*2
      GramJob& g = r.gjob;
      std::memset(&g, 0, sizeof(g));
      g.d = r.w.d;
      g.qtbl = r.qt;
      g.cstbl = r.cs;
      g.qper = M;
      g.has_diag = diag != nullptr;
      for (int j = 0; diag && j < r.nc; ++j)
        g.diag.p[j] = reinterpret_cast<const char*>(diag + (int64_t)ch.mats[j] * M * 2);
      g.w = r.w.gram;
      g.scale = r.w.scale;
      g.batch = r.B;
      g.m = ch.m;
      g.n = ch.n;
      // the momenta read in place where the persistent kernels take the chunk
      g.xtbl = &r.mom;
      g.xper = M;
      if (!gram_in_place_ok(g, c->mdt, c->ns)) {
        g.xtbl = nullptr;
        g.xper = 1;
        g.x = r.w.x0;
      }
    }
    if (muon_step && c->algo != SM_CACHE_MUON) {
      r.job = NsJob{r.w.x0, r.w.d, r.w.ns, r.w.scale, r.B, ch.m, ch.n};
      if (c->algo == SM_SIGN_MUON) {
        NsJob tj = r.job;
        tj.x = nullptr;
        tj.xtbl = &r.mom;
        tj.xper = M;
        if (ns_grouped_ok(tj, c->mdt, c->ns)) {
          r.job = tj;
          r.grouped = true;
        }
      }
      if (!r.grouped) r.grouped = ns_grouped_ok(r.job, c->mdt, c->ns);
      if (!r.grouped && c->algo == SM_SIGN_MUON) {  // the generic path reads M in place too
        r.job.x = nullptr;
        r.job.xtbl = &r.mom;
        r.job.xper = M;
      }
      // a7 + a8 fused into the last NS product when the signs are all the
      // step needs from the direction (int8 signs: the grouped kernels only)
      r.fused_signs = false;
      if (!polar && c->encoding == SM_ENC_BITS) {
        NsJob bj = r.job;
        bj.bits = r.w.bits;
        bj.bits_stride = r.words;
        if (r.grouped ? ns_grouped_ok(bj, c->mdt, c->ns) : (ch.n % 64) == 0) {
          r.job = bj;
          r.fused_signs = true;
        }
      } else if (!polar && c->encoding == SM_ENC_INT8 && r.grouped && r.count % 16 == 0) {
        NsJob bj = r.job;
        bj.bits = reinterpret_cast<uint64_t*>(r.w.s8);
        bj.bits_stride = r.count / 8;
        bj.bits_s8 = true;
        if (ns_grouped_ok(bj, c->mdt, c->ns)) {
          r.job = bj;
          r.fused_signs = true;
        }
      }
    }
  }
  // a1 (+ a2 partials): momentum, and the NS input or the Lion signs.  The
  // single EMA of every chunk goes out as one launch over a table of
  // matrices (and one norm finalize).
  if (c->algo == SM_LION_MUON) {
    for (size_t ci = 0; ci < chunks.size(); ++ci) {
      ChunkRun& r = runs[ci];
      if (muon_step)
        SM_TRY(launch_lion(r.mom, r.grad, M, r.B, r.count, c->mdt, c->gdt, c->beta1, c->beta2,
                           r.w.x0, c->mdt, r.w.partials, nullptr, 0, nullptr, s));
      else
        SM_TRY(launch_lion(r.mom, r.grad, M, r.B, r.count, c->mdt, c->gdt, c->beta1, c->beta2,
                           nullptr, c->mdt, nullptr, r.w.bits, r.words, r.w.s8, s));
      if (muon_step)
        SM_TRY(launch_scale_finalize(r.w.partials, r.B, r.count, c->ns.eps, r.w.scale, s));
    }
  } else {
    std::vector<EmaMat> ema;
    for (size_t ci = 0; ci < chunks.size(); ++ci) {
      ChunkRun& r = runs[ci];
      // no copy when the NS reads M in place
      void* x0 = (r.job.xtbl || (c->algo == SM_CACHE_MUON && r.gjob.xtbl)) ? nullptr : r.w.x0;
      for (int j = 0; j < r.nc; ++j) {
        EmaMat e;
        e.mom = const_cast<char*>(r.mom.p[j]);
        e.grad = r.grad.p[j];
        e.x = x0 ? static_cast<char*>(x0) + (int64_t)j * M * r.count * dt_size(c->mdt)
                 : nullptr;
        e.partials = r.w.partials + (int64_t)j * M * kNormParts;
        e.scale = r.w.scale + (int64_t)j * M;
        e.count = r.count;
        ema.push_back(e);
      }
    }
    SM_TRY(launch_ema_tbl(ema.data(), (int)ema.size(), M, c->mdt, c->gdt, c->beta1, muon_step,
                          c->ns.eps, s));
  }
  // a3-a5: the direction.  Direct NS runs all chunks the grouped kernel takes
  // together (one launch per product kind and iteration).
  if (muon_step) {
    std::vector<NsJob> grouped, generic;
    std::vector<GramJob> gjobs;
    for (size_t ci = 0; ci < chunks.size(); ++ci) {
      ChunkRun& r = runs[ci];
      if (c->algo == SM_CACHE_MUON)
        gjobs.push_back(r.gjob);
      else
        (r.grouped ? grouped : generic).push_back(r.job);
    }
    if (!gjobs.empty())
      SM_TRY(gram_jobs(gjobs, c->mdt, c->ns, c->gamma, c->cache_mode, t, s));
    if (!grouped.empty()) SM_TRY(ns_grouped(grouped, c->ns, s));
    if (!generic.empty()) SM_TRY(ns_generic(generic, c->mdt, c->ns, s));
  }
  // a7-a10: signs (packed bits or int8), vote and update (or the polar update)
  const bool int8 = c->encoding == SM_ENC_INT8;
  for (size_t ci = 0; ci < chunks.size(); ++ci) {
    ChunkRun& r = runs[ci];
    if (muon_step) {
      if (polar)
        SM_TRY(launch_polar_update(r.w.d, c->mdt, r.nc, r.count, r.wt, c->wdt, c->lr, s));
      else if (int8 && !r.fused_signs)
        SM_TRY(launch_sign_int8(r.w.d, c->mdt, r.B, r.count, r.w.s8, s));
      else if (!int8 && !r.fused_signs)
        SM_TRY(launch_sign_pack(r.w.d, c->mdt, r.B, r.count, r.w.bits, r.words, s));
    }
  }
  if (polar) return SM_OK;
  std::vector<const void*> sg(chunks.size());
  for (size_t ci = 0; ci < chunks.size(); ++ci)
    sg[ci] = int8 ? (const void*)runs[ci].w.s8 : (const void*)runs[ci].w.bits;
  if (!c->vote_polar) {   // every matrix of every chunk in one launch
    std::vector<VoteMat> vm;
    for (size_t ci = 0; ci < chunks.size(); ++ci) {
      ChunkRun& r = runs[ci];
      const int64_t stride = int8 ? r.count : r.words;
      for (int j = 0; j < r.nc; ++j) {
        VoteMat v;
        v.signs = int8 ? static_cast<const void*>(runs[ci].w.s8 + (int64_t)j * M * stride)
                       : static_cast<const void*>(runs[ci].w.bits + (int64_t)j * M * stride);
        v.w = const_cast<char*>(r.wt.p[j]);
        v.stride = stride;
        v.count = r.count;
        vm.push_back(v);
      }
    }
    return launch_vote_tbl(c->encoding, M, vm.data(), (int)vm.size(), c->wdt, c->lr, s);
  }
  // Optional local polar step on the vote: V (exact in mdt) -> its own
  // normalisation -> NS with the step's settings -> W <- W - lr * D.
  std::vector<NsJob> vjobs, vgen;   // vote NS jobs: persistent kernel / generic path
  for (size_t ci = 0; ci < chunks.size(); ++ci) {
    const Chunk& ch = chunks[ci];
    ChunkRun& r = runs[ci];
    const int64_t stride = int8 ? r.count : r.words;
    PtrTbl vt;
    std::memset(&vt, 0, sizeof(vt));
    for (int j = 0; j < r.nc; ++j)
      vt.p[j] = static_cast<const char*>(r.w.x0) + (int64_t)j * r.count * dt_size(c->mdt);
    SM_TRY(launch_vote(c->encoding, sg[ci], M, stride, (int64_t)M * stride, r.nc, r.count, vt,
                       c->mdt, 0.f, nullptr, false, s));
    SM_TRY(launch_sumsq(r.w.x0, c->mdt, r.nc, r.count, r.w.partials, s));
    SM_TRY(launch_scale_finalize(r.w.partials, r.nc, r.count, c->ns.eps, r.w.scale, s));
    NsJob j{r.w.x0, r.w.d, r.w.ns, r.w.scale, r.nc, ch.m, ch.n};
    (ns_grouped_ok(j, c->mdt, c->ns) ? vjobs : vgen).push_back(j);
  }
  if (!vjobs.empty()) SM_TRY(ns_grouped(vjobs, c->ns, s));
  if (!vgen.empty()) SM_TRY(ns_generic(vgen, c->mdt, c->ns, s));
  for (size_t ci = 0; ci < chunks.size(); ++ci) {
    ChunkRun& r = runs[ci];
    SM_TRY(launch_polar_update(r.w.d, c->mdt, r.nc, r.count, r.wt, c->wdt, c->lr, s));
  }
  return SM_OK;
}

// ------------------------------------------------------------------ HIP graphs of a step

// The step's launches are recorded on a private non-blocking stream (so the
// caller's stream, possibly the null stream, is never in capture), then
// instantiated once.  sm_step only launches kernels (no copies, memsets or
// allocations), so the graph holds kernel nodes alone and their arguments
// (pointers, sizes, hyper-parameters) by value.
sm_status sm_step_graph(const sm_config* c, const sm_matrix* mats, int nmat, int64_t t, void* ws,
                        size_t ws_bytes, float* diag, sm_graph* out) {
  if (!out) return SM_ERR_ARG;
  *out = nullptr;
  SM_TRY(check_config(c));
  SM_TRY(check_mats(*c, mats, nmat));
  if (t < 1 || !ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return SM_ERR_ARG;
  // CacheMuon's kernels record t with each refresh; event pairs of the
  // kernel-time accounting are host-side records, not graph nodes
  if (c->algo == SM_CACHE_MUON || g_prof_on) return SM_ERR_UNSUPPORTED;
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return hip_fail(e);
  }
  const sm_status st = sm_step(c, mats, nmat, t, ws, ws_bytes, diag, cs);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (st != SM_OK || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return st != SM_OK ? st : hip_fail(e);
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e);
  }
  sm_graph h = new (std::nothrow) sm_graph_s{g, x};
  if (!h) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return hip_fail(hipErrorOutOfMemory);
  }
  *out = h;
  return SM_OK;
}

sm_status sm_graph_launch(sm_graph g, hipStream_t s) {
  if (!g) return SM_ERR_ARG;
  const hipError_t e = hipGraphLaunch(g->exec, s);
  return e == hipSuccess ? SM_OK : hip_fail(e);
}

sm_status sm_graph_destroy(sm_graph g) {
  if (!g) return SM_OK;
  const hipError_t e1 = hipGraphExecDestroy(g->exec);
  const hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  if (e1 != hipSuccess) return hip_fail(e1);
  return e2 == hipSuccess ? SM_OK : hip_fail(e2);
}

// ------------------------------------------------------------------ profiling ABI

sm_status sm_profile_enable(int on) {
  if (on) {
    if (g_prof_pool.empty()) {
      g_prof_pool.resize(2 * kProfMax);
      for (size_t i = 0; i < g_prof_pool.size(); ++i) {
        hipError_t e = hipEventCreate(&g_prof_pool[i]);
        if (e != hipSuccess) {
          g_prof_pool.resize(i);
          return hip_fail(e);
        }
      }
      g_prof_recs.reserve(kProfMax);
    }
    if (!g_prof_exec_ptr) {
      void* p = nullptr;
      hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_prof_exec));
      if (e != hipSuccess) return hip_fail(e);
      g_prof_exec_ptr = static_cast<double*>(p);
      const double zero[2 * SM_K_NUM_KINDS] = {};
      e = hipMemcpy(g_prof_exec_ptr, zero, sizeof(zero), hipMemcpyHostToDevice);
      if (e != hipSuccess) return hip_fail(e);
    }
    g_prof_on = true;
  } else {
    g_prof_on = false;
  }
  return SM_OK;
}

sm_status sm_profile_reset(void) {
  g_prof_recs.clear();
  g_prof_open = false;
  if (g_prof_exec_ptr) {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e);
    const double zero[2 * SM_K_NUM_KINDS] = {};
    e = hipMemcpy(g_prof_exec_ptr, zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
  }
  return SM_OK;
}

// Executed {flops, bytes} of a kind's predicated launches so far.
static sm_status read_exec(int kind, double* out2) {
  out2[0] = out2[1] = 0.0;
  if (!g_prof_exec_ptr) return SM_OK;
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e);
  e = hipMemcpy(out2, g_prof_exec_ptr + 2 * kind, 2 * sizeof(double), hipMemcpyDeviceToHost);
  return e == hipSuccess ? SM_OK : hip_fail(e);
}

sm_status sm_profile_read(int kind, double* ms_total, int64_t* launches, double* work) {
  if (kind < 0 || kind >= SM_K_NUM_KINDS || !ms_total || !launches || !work) return SM_ERR_ARG;
  double ms = 0.0, wk = 0.0;
  int64_t n = 0;
  for (const ProfRec& r : g_prof_recs) {
    if (r.kind != kind) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e);
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e);
    ms += t;
    wk += r.work;
    ++n;
  }
  double ex[2];
  SM_TRY(read_exec(kind, ex));
  *ms_total = ms;
  *launches = n;
  *work = wk + ex[0];
  return SM_OK;
}

sm_status sm_profile_read_bytes(int kind, double* bytes) {
  if (kind < 0 || kind >= SM_K_NUM_KINDS || !bytes) return SM_ERR_ARG;
  double b = 0.0;
  for (const ProfRec& r : g_prof_recs)
    if (r.kind == kind) b += r.bytes;
  double ex[2];
  SM_TRY(read_exec(kind, ex));
  *bytes = b + ex[1];
  return SM_OK;
}

const char* sm_kernel_kind_name(int kind) {
  static const char* names[SM_K_NUM_KINDS] = {
      "ema", "norm", "gemm_gram", "gemm_apply", "gemm_rr", "probe",
      "sign_pack", "vote_update", "lion", "polar_update", "misc", "spectral"};
  if (kind < 0 || kind >= SM_K_NUM_KINDS) return "unknown";
  return names[kind];
}

}  // extern "C"
