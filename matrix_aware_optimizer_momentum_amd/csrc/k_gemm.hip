// Dispatch of the batched MFMA GEMM over operand types and layouts, and the
// packing of product sets into grouped launches.
#include "k_gemm.hpp"

namespace sm {

sm_status launch_gemm_bf16_a(const GemmArgs* gs, int n, int kind, hipStream_t s);
sm_status launch_gemm_bf16_b(const GemmArgs* gs, int n, int kind, hipStream_t s);
sm_status launch_gemm_f32(const GemmArgs* gs, int n, int kind, hipStream_t s);

static_assert(sizeof(gemm::KArgs) <= 4096, "kernel arguments of one grouped launch");

int gemm_tiles(int mfma_dt, int M, int N) {
  (void)mfma_dt;
  return ((M + gemm::BM - 1) / gemm::BM) * ((N + gemm::BN - 1) / gemm::BN);
}

namespace {

bool empty_set(const GemmArgs& g) { return g.batch <= 0 || g.M <= 0 || g.N <= 0 || g.K <= 0; }

sm_status check_set(const GemmArgs& g, int mfma_dt) {
  if (g.tbl_per < 1) return SM_ERR_ARG;
  if (g.bits && (g.N % 64) != 0) return SM_ERR_UNSUPPORTED;
  if (g.sym && (g.M != g.N || g.c2 || g.c2_tbl || g.resid || g.bits)) return SM_ERR_UNSUPPORTED;
  if (mfma_dt != BF16 && (g.a.dt != F32 || g.b.dt != F32)) return SM_ERR_UNSUPPORTED;
  if (gemm::uses_tbl(g) && (g.batch + g.tbl_per - 1) / g.tbl_per > kTbl) return SM_ERR_UNSUPPORTED;
  return SM_OK;
}

// Sets that one kernel instantiation can run together.
bool same_kernel(const GemmArgs& x, const GemmArgs& y) {
  return x.a.dt == y.a.dt && x.b.dt == y.b.dt && x.a.layout == y.a.layout &&
         x.b.layout == y.b.layout;
}

// Table entries that sets[0..n) need in one launch (identical tables shared).
int table_entries(const GemmArgs* const* sets, int n) {
  std::vector<const GemmArgs*> seen;
  int used = 0;
  for (int i = 0; i < n; ++i) {
    const GemmArgs& g = *sets[i];
    if (!gemm::uses_tbl(g)) continue;
    const int ne = (g.batch + g.tbl_per - 1) / g.tbl_per;
    bool dup = false;
    for (const GemmArgs* o : seen) {
      const int no = (o->batch + o->tbl_per - 1) / o->tbl_per;
      if (no >= ne && std::memcmp(&o->tbl.p[0], &g.tbl.p[0], ne * sizeof(const char*)) == 0)
        dup = true;
    }
    if (!dup) {
      used += ne;
      seen.push_back(&g);
    }
  }
  return used;
}

sm_status launch_set(const GemmArgs* gs, int n, int mfma_dt, int kind, hipStream_t s) {
  if (mfma_dt == BF16) {
    if (gs[0].a.dt == BF16) return launch_gemm_bf16_a(gs, n, kind, s);
    return launch_gemm_bf16_b(gs, n, kind, s);
  }
  return launch_gemm_f32(gs, n, kind, s);
}

}  // namespace

sm_status launch_gemm(const GemmArgs& g, int mfma_dt, int kind, hipStream_t s) {
  if (empty_set(g)) return SM_OK;
  SM_TRY(check_set(g, mfma_dt));
  return launch_set(&g, 1, mfma_dt, kind, s);
}

sm_status launch_gemm_groups(std::vector<GemmArgs>& gs, int mfma_dt, int kind, hipStream_t s) {
  std::vector<const GemmArgs*> sets;
  for (const GemmArgs& g : gs) {
    if (empty_set(g)) continue;
    SM_TRY(check_set(g, mfma_dt));
    sets.push_back(&g);
  }
  // longest blocks first, so that the short ones fill the tail
  std::stable_sort(sets.begin(), sets.end(),
                   [](const GemmArgs* x, const GemmArgs* y) { return x->K > y->K; });
  std::vector<char> done(sets.size(), 0);
  std::vector<GemmArgs> batch;
  std::vector<const GemmArgs*> pick;
  for (size_t i = 0; i < sets.size(); ++i) {
    if (done[i]) continue;
    pick.clear();
    for (size_t j = i; j < sets.size() && (int)pick.size() < gemm::kGemmMaxGroups; ++j) {
      if (done[j] || !same_kernel(*sets[i], *sets[j])) continue;
      pick.push_back(sets[j]);
      if (table_entries(pick.data(), (int)pick.size()) > kTbl) {
        pick.pop_back();
        continue;
      }
      done[j] = 1;
    }
    batch.clear();
    for (const GemmArgs* p : pick) batch.push_back(*p);
    SM_TRY(launch_set(batch.data(), (int)batch.size(), mfma_dt, kind, s));
  }
  return SM_OK;
}

}  // namespace sm
