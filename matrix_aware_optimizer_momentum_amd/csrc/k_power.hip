// Power-method estimate of the spectral norm of a batch of differences
// E_b = A_b - B_b (m x n, row-major), for the CacheMuon fidelity diagnostic:
// the distance ||D_hat - D_fresh||_sp between a cached direction and the
// fresh one (CacheMuon technical summary, gist.science/ja/paper/2606.16371,
// theoretical analysis and the diagnostic findings of the experiments).
//
// From the caller's start vectors: v = v0 / ||v0||; `iters` times y = E v,
// z = E^T y, v = z / ||z||; then sigma = ||E v||.  Every pass streams A and B
// once (HBM-bound); E is formed on the fly in float32.  The iterate is kept
// unnormalised (z) with per-block partial sums of z^2, and y = (E z) / ||z||
// takes the norm from those partials, so no pass is a one-block reduction.
// Sums run in a fixed order (wave butterflies, fixed row chunks and column
// blocks), so results are run-to-run identical.
#include "sm_internal.hpp"

namespace sm {

namespace {

constexpr int kPT = 256;           // threads per block
constexpr int kRowsPerBlock = 4;   // y = E v: one row per wave
constexpr int kColsPerBlock = kPT * 8;

// Eight consecutive entries of one row of E = a - b (b may be null) from
// column c0; entries past n read as 0.
template <typename T>
__device__ __forceinline__ void diff8(const T* a, const T* b, int64_t c0, int64_t n, bool vec,
                                      float* d) {
  if (vec && c0 + 8 <= n) {
    load8<T>(a + c0, d);
    if (b) {
      float w[8];
      load8<T>(b + c0, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = __fsub_rn(d[e], w[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool in = c0 + e < n;
      const float x = in ? Elem<T>::load(a + c0 + e) : 0.f;
      const float z = (in && b) ? Elem<T>::load(b + c0 + e) : 0.f;
      d[e] = __fsub_rn(x, z);
    }
  }
}

// y[b][row] = (sum_c E_b[row][c] z[b][c]) / ||z_b|| (0 if z_b = 0), with
// ||z_b||^2 the sum of the nb partials zsq[b][*]; z rows are npad long (zero
// past n).
template <typename T>
__global__ __launch_bounds__(kPT) void k_pm_av(const T* a, const T* b, int64_t sp, int m, int n,
                                               int npad, const float* v, const double* zsq,
                                               int nb, float* y, bool vec) {
  const int p = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* vp = v + (int64_t)p * npad;
  const int row = blockIdx.x * kRowsPerBlock + wave;
  if (row >= m) return;
  const int64_t off = (int64_t)p * sp + (int64_t)row * n;
  const T* ar = a + off;
  const T* br = b ? b + off : nullptr;
  float acc = 0.f;
  for (int64_t c0 = (int64_t)lane * 8; c0 < n; c0 += 64 * 8) {
    float d[8];
    diff8<T>(ar, br, c0, n, vec, d);
    const float4 v0 = *reinterpret_cast<const float4*>(vp + c0);
    const float4 v1 = *reinterpret_cast<const float4*>(vp + c0 + 4);
    const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __fmaf_rn(d[e], vv[e], acc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) {
    double s2 = 0.0;
    for (int i = 0; i < nb; ++i) s2 += zsq[(int64_t)p * nb + i];
    y[(int64_t)p * m + row] = s2 > 0.0 ? (float)((double)acc / sqrt(s2)) : 0.f;
  }
}

// zpart[b][chunk][c] = sum over the chunk's rows r of E_b[r][c] y[b][r];
// 8 consecutive columns per thread.
template <typename T>
__global__ __launch_bounds__(kPT) void k_pm_atv(const T* a, const T* b, int64_t sp, int m, int n,
                                                int npad, const float* y, int rows_per_chunk,
                                                float* zpart, bool vec) {
  const int p = blockIdx.z, chunk = blockIdx.y;
  const int64_t c0 = ((int64_t)blockIdx.x * kPT + threadIdx.x) * 8;
  if (c0 >= npad) return;
  const int r0 = chunk * rows_per_chunk;
  const int r1 = min(m, r0 + rows_per_chunk);
  const float* yp = y + (int64_t)p * m;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < r1; ++r) {
    const int64_t off = (int64_t)p * sp + (int64_t)r * n;
    float d[8];
    diff8<T>(a + off, b ? b + off : nullptr, c0, n, vec, d);
    const float yr = yp[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __fmaf_rn(d[e], yr, acc[e]);
  }
  float* zp = zpart + ((int64_t)p * gridDim.y + chunk) * npad + c0;
  *reinterpret_cast<float4*>(zp) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(zp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// Fixed-order block sum in double.
__device__ double block_sum_d(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const double r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// z[b][c] = sum over `parts` rows of x (stride sx; problem stride sp) at
// column c, for c < len (0 up to npad); zsq[b][block] = this block's sum of
// z^2.  With parts = 1 it copies the start vectors into the padded layout.
__global__ __launch_bounds__(kPT) void k_pm_colsum(const float* x, int parts, int64_t sx,
                                                   int64_t sp, int len, int npad, float* z,
                                                   double* zsq) {
  __shared__ double red[4];
  const int p = blockIdx.y;
  const int c = blockIdx.x * kPT + threadIdx.x;
  float val = 0.f;
  if (c < len) {
    const float* xp = x + (int64_t)p * sp + c;
    for (int k = 0; k < parts; ++k) val += xp[(int64_t)k * sx];
  }
  if (c < npad) z[(int64_t)p * npad + c] = val;
  const double s2 = block_sum_d((double)val * (double)val, red);
  if (threadIdx.x == 0) zsq[(int64_t)p * gridDim.x + blockIdx.x] = s2;
}

// out[b] = ||y_b|| (one block per problem, m entries).
__global__ __launch_bounds__(kPT) void k_pm_norm(const float* y, int m, float* out) {
  __shared__ double red[4];
  const int p = blockIdx.x;
  double acc = 0.0;
  for (int c = threadIdx.x; c < m; c += kPT) {
    const double v = y[(int64_t)p * m + c];
    acc += v * v;
  }
  const double nz = sqrt(block_sum_d(acc, red));
  if (threadIdx.x == 0) out[p] = (float)nz;
}

}  // namespace

size_t spectral_norm_ws_bytes(int batch, int m, int n) {
  const int64_t npad = ((int64_t)n + 7) / 8 * 8;
  const int64_t rc = spectral_row_chunks(batch, m, n);
  const int64_t nb = (npad + kPT - 1) / kPT;
  const size_t v = (size_t)batch * npad * 4, y = (size_t)batch * m * 4;
  const size_t z = (size_t)batch * rc * npad * 4, q = (size_t)batch * nb * 8;
  return ((v + 255) / 256 + (y + 255) / 256 + (z + 255) / 256 + (q + 255) / 256) * 256 + 256;
}

int spectral_row_chunks(int batch, int m, int n) {
  const int64_t colblocks = ((int64_t)n + kColsPerBlock - 1) / kColsPerBlock;
  int64_t rc = (2048 + colblocks * batch - 1) / (colblocks * batch);
  const int64_t maxrc = ((int64_t)m + 15) / 16;
  if (rc > maxrc) rc = maxrc;
  if (rc < 1) rc = 1;
  return (int)rc;
}

sm_status launch_spectral_norm(const void* a, const void* b, int dt, int batch, int m, int n,
                               const float* v0, int iters, float* out, void* ws, hipStream_t s) {
  if (batch <= 0) return SM_OK;
  const int64_t npad = ((int64_t)n + 7) / 8 * 8;
  const int nb = (int)((npad + kPT - 1) / kPT);
  const int rc = spectral_row_chunks(batch, m, n);
  const int rows_per_chunk = (m + rc - 1) / rc;
  char* base = static_cast<char*>(ws);
  const size_t vbytes = ((size_t)batch * npad * 4 + 255) / 256 * 256;
  const size_t ybytes = ((size_t)batch * m * 4 + 255) / 256 * 256;
  const size_t zbytes = ((size_t)batch * rc * npad * 4 + 255) / 256 * 256;
  float* v = reinterpret_cast<float*>(base);
  float* y = reinterpret_cast<float*>(base + vbytes);
  float* zpart = reinterpret_cast<float*>(base + vbytes + ybytes);
  double* zsq = reinterpret_cast<double*>(base + vbytes + ybytes + zbytes);
  const int64_t sp = (int64_t)m * n;
  const size_t es = dt_size(dt);
  const bool vec = (n % 8) == 0 && (reinterpret_cast<uintptr_t>(a) & 15u) == 0 &&
                   (!b || (reinterpret_cast<uintptr_t>(b) & 15u) == 0);
  const double pass_bytes = (double)batch * sp * es * (b ? 2.0 : 1.0);
  const dim3 g_av((m + kRowsPerBlock - 1) / kRowsPerBlock, batch);
  const dim3 g_atv((unsigned)((npad + kColsPerBlock - 1) / kColsPerBlock), rc, batch);
  const dim3 g_cs(nb, batch);

  // v <- v0 (padded), with its squared-norm partials
  prof_begin(SM_K_SPECTRAL, (double)batch * n * 8.0, s);
  hipLaunchKernelGGL(k_pm_colsum, g_cs, dim3(kPT), 0, s, v0, 1, (int64_t)0, (int64_t)n, n,
                     (int)npad, v, zsq);
  prof_end(s);
  SM_TRY(check_launch());
  for (int it = 0; it <= iters; ++it) {
    prof_begin(SM_K_SPECTRAL, pass_bytes, s);
    SM_DISPATCH_DT(dt, T,
        hipLaunchKernelGGL((k_pm_av<T>), g_av, dim3(kPT), 0, s, (const T*)a, (const T*)b, sp,
                           m, n, (int)npad, v, zsq, nb, y, vec));
    prof_end(s);
    SM_TRY(check_launch());
    if (it == iters) break;
    prof_begin(SM_K_SPECTRAL, pass_bytes, s);
    SM_DISPATCH_DT(dt, T,
        hipLaunchKernelGGL((k_pm_atv<T>), g_atv, dim3(kPT), 0, s, (const T*)a, (const T*)b, sp,
                           m, n, (int)npad, y, rows_per_chunk, zpart, vec));
    prof_end(s);
    SM_TRY(check_launch());
    prof_begin(SM_K_SPECTRAL, (double)batch * rc * npad * 4.0, s);
    hipLaunchKernelGGL(k_pm_colsum, g_cs, dim3(kPT), 0, s, zpart, rc, (int64_t)npad,
                       (int64_t)rc * npad, n, (int)npad, v, zsq);
    prof_end(s);
    SM_TRY(check_launch());
  }
  prof_begin(SM_K_SPECTRAL, (double)batch * m * 4.0, s);
  hipLaunchKernelGGL(k_pm_norm, dim3(batch), dim3(kPT), 0, s, y, m, out);
  prof_end(s);
  return check_launch();
}

}  // namespace sm
