/*
 * sm.h - C ABI of the MI355X (gfx950) Muon-family optimizer step library.
 *
 * One optimizer step of Sign-Muon, CacheMuon or LionMuon on a set of weight
 * matrices, with M data-parallel workers simulated on one GPU as M gradient
 * streams.  The steps are: momentum EMA, Frobenius normalisation,
 * Newton-Schulz (NS) polar iteration or its Gram form with a cached left
 * transform Q and an orthogonality-residual reuse check, entrywise sign,
 * 1-bit packing, majority vote, and the weight update.
 *
 * Sources (cited below by short name):
 *   [SignMuon-ja]  SignMuon technical summary, gist.science/ja/paper/2605.16311
 *   [SignMuon-abs] SignMuon abstract, fugumt.com/fugumt/paper_check/2605.16311v1
 *                  and hotpaper.ai/paper/2605.16311
 *   [CacheMuon-ja] CacheMuon technical summary, gist.science/ja/paper/2606.16371
 *   [LionMuon-pt]  LionMuon technical summary, gist.science/pt/paper/2605.19811
 *
 * Conventions shared by every call
 *   - Every tensor pointer is DEVICE memory, row-major, contiguous, owned by
 *     the caller, and 16-byte aligned unless a call states otherwise.  The library never allocates device
 *     memory, never frees, and keeps no pointer after a call returns.
 *     Scratch memory is passed in as `ws` (sized by the matching *_ws query).
 *   - All GPU work is enqueued on the stream `s` (0 = null stream) and is
 *     asynchronous; no call synchronises the stream or copies device data to
 *     the host.
 *   - Arguments are validated on the host before any HIP call; a bad
 *     argument returns an SM_ERR_* code and enqueues nothing.  A failed
 *     launch returns SM_ERR_HIP; sm_last_hip_error() then gives the HIP code.
 *     No call aborts or throws across the ABI.
 *   - Arithmetic is float32 (MFMA accumulation in float32).  bf16 values are
 *     rounded from float32 with round-to-nearest-even.
 *   - sign(x) = -1 if x < 0, else +1  (+0, -0 and NaN give +1).
 *   - 1-bit layout: uint64 words, little-endian; bit j of word w holds entry
 *     64*w + j of the row-major matrix in its original orientation; the bit
 *     is 1 iff the entry is negative; unused tail bits are 0.
 *   - Calls on different streams with disjoint buffers are independent.
 */
#ifndef SM_H
#define SM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SM_OK = 0,
  SM_ERR_ARG = 1,          /* null / misaligned / aliased pointer, bad scalar    */
  SM_ERR_SHAPE = 2,        /* non-positive or too large dimension                */
  SM_ERR_DTYPE = 3,        /* dtype not SM_F32 / SM_BF16                         */
  SM_ERR_WORKSPACE = 4,    /* ws too small (query the *_ws call)                 */
  SM_ERR_UNSUPPORTED = 5,  /* valid request outside what the library implements  */
  SM_ERR_HIP = 6           /* a HIP runtime call or launch failed                */
} sm_status;

typedef enum { SM_F32 = 0, SM_BF16 = 1 } sm_dtype;

/* Newton-Schulz parameters: iterations K and polynomial coefficients of
 * X <- a X + b (X X^T) X + c (X X^T)^2 X, and the normalisation guard eps of
 * X = Y / (||Y||_F + eps).  The pages print no coefficients; the cubic
 * default is {5, 1.5f, -0.5f, 0.0f, 1e-7f}.  1 <= iters <= 64. */
typedef struct {
  int32_t iters;
  float a, b, c;
  float eps;
} sm_ns_params;

/* Human-readable name of a status code (static storage, never NULL). */
const char* sm_status_string(int status);

/* Last hipError_t returned by a HIP call inside the library (0 if none). */
int sm_last_hip_error(void);

/* Library ABI version (increments on any signature change). */
int sm_version(void);

/* ------------------------------------------------------------------------
 * Direct Newton-Schulz polar factor.
 * [SignMuon-ja] section 2, core mechanism 1 and algorithm flow step 1: each
 * worker approximates the polar factor of its momentum by a Newton-Schulz
 * iteration; [LionMuon-pt] problem statement: Muon steps with msign(G_hat).
 *
 * x, u : [batch][m][n] in dt.  u receives X_K.  x is read-only and must not
 *        overlap u.  A tall problem (m > n) is iterated on its transpose
 *        (Gram matrix n x n); x and u keep the original orientation.
 *        With bf16 operands, cubic coefficients (c = 0), K >= 2 and a shape
 *        far enough from square, X_K is computed in the Gram form: with
 *        S_k = b X_k X_k^T, X_{k+1} = (S_k + aI) X_k, so X_K = Q_K X_0 with
 *        Q_K the product of the (S_k + aI), all polynomials in X_0 X_0^T
 *        (r x r products instead of r x max(m,n) ones).  It is the same X_K
 *        up to rounding; the choice depends on the problem alone (shape,
 *        dtype, K, coefficients), so sm_step gives a matrix the same bits
 *        as this call.
 * normalize : 1 -> iterate from x / (||x||_F + eps) per problem; 0 -> from x.
 * ws   : scratch of at least sm_ns_polar_ws(...) bytes, 256-byte aligned.
 * Errors: SM_ERR_ARG (null, misaligned, overlap, bad params), SM_ERR_SHAPE
 *        (batch, m or n < 1, or m*n >= 2^31), SM_ERR_DTYPE, SM_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
sm_status sm_ns_polar_ws(int dt, int batch, int m, int n, size_t* ws_bytes);
sm_status sm_ns_polar(const void* x, void* u, int dt, int batch, int m, int n,
                      int normalize, const sm_ns_params* p, void* ws, size_t ws_bytes,
                      hipStream_t s);

/* ------------------------------------------------------------------------
 * sm_ns_polar without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same inputs, outputs, kernels
 * and results (bit for bit) as sm_ns_polar; the scratch is a fixed device
 * array inside the library of SM_NS_NOALLOC_MAX_WS bytes (64 MiB), one per
 * GPU, held until the process ends.  The call allocates nothing and uses
 * no zero-initialised scratch.  Limit: sm_ns_polar_ws(dt, batch, m, n) must
 * not exceed SM_NS_NOALLOC_MAX_WS (about a 2048 x 8192 bf16 problem, or
 * eight 768 x 3072 ones), else SM_ERR_WORKSPACE and nothing is enqueued.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or host threads) race and must be ordered by
 * the caller.  Errors as for sm_ns_polar.
 * ---------------------------------------------------------------------- */
#define SM_NS_NOALLOC_MAX_WS (64u << 20)
sm_status sm_ns_polar_noalloc(const void* x, void* u, int dt, int batch, int m, int n,
                              int normalize, const sm_ns_params* p, hipStream_t s);

/* ------------------------------------------------------------------------
 * CacheMuon orthogonalisation: Gram Newton-Schulz with a cached left
 * transform Q and a residual-based reuse trigger.
 * [CacheMuon-ja] method, core mechanism items 1-3: a refresh runs the fresh
 * Gram-NS solve, which returns the direction and the left transform Q; other
 * steps apply the cached Q to the normalised momentum, D_hat = Q X, and keep
 * it iff err = ||D_hat D_hat^T - I||_F / ||I||_F <= gamma, else refresh.
 *
 * With r = min(m,n) and X the wide orientation of x (x^T when m > n):
 *   fresh: G_0 = X X^T, Q_0 = I; for k < K: P_k = aI + bG_k + cG_k^2,
 *          Q_{k+1} = P_k Q_k, G_{k+1} = P_k G_k P_k; D = Q_K X.
 * x, d  : [batch][m][n] in dt; d receives the direction in x's orientation.
 * q     : [batch][r][r] float32, the cache (caller-owned, persistent state).
 * cache_state : [batch][2] int32 = {has_cache, a_t} (persistent; zero it
 *         before the first step).  a_t is the low 32 bits of t.
 * err   : [batch] float32 out: the probed residual, or -1 if no candidate
 *         was probed (no cache, or mode 1).
 * refreshed : [batch] int32 out: 1 if a fresh solve ran, else 0.
 * mode  : 0 trigger (reuse iff err <= gamma; NaN err refreshes),
 *         1 force fresh every step, 2 force reuse whenever a cache exists.
 * t     : step index (1-based) recorded as a_t on refresh.
 * The accept/refresh decision is taken on the device; nothing is copied to
 * the host.  Errors as for sm_ns_polar, plus SM_ERR_ARG for a bad mode.
 * ---------------------------------------------------------------------- */
sm_status sm_gram_ns_cached_ws(int dt, int batch, int m, int n, size_t* ws_bytes);
sm_status sm_gram_ns_cached(const void* x, void* d, float* q, int32_t* cache_state,
                            float* err, int32_t* refreshed, int dt, int batch, int m,
                            int n, int normalize, const sm_ns_params* p, float gamma,
                            int mode, int64_t t, void* ws, size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------------------
 * Entrywise sign and 1-bit pack.
 * [SignMuon-ja] section 2, algorithm flow steps 2-3 (all-gather variant):
 * workers keep only the entrywise sign of their direction, packed one bit
 * per entry (32x fewer bytes than float32, [SignMuon-ja] communication
 * efficiency).
 * x    : [count] in dt (element-aligned; 16-byte alignment takes the
 *        vector path).   bits : [ceil(count/64)] uint64 out, 8-byte aligned.
 * Errors: SM_ERR_ARG (null/misaligned), SM_ERR_SHAPE (count < 0),
 *         SM_ERR_DTYPE.  count == 0 is a no-op.
 * ---------------------------------------------------------------------- */
sm_status sm_sign_pack(const void* x, int dt, int64_t count, uint64_t* bits, hipStream_t s);

/* ------------------------------------------------------------------------
 * Majority vote and update.
 * [SignMuon-ja] section 2, core mechanism 3 and algorithm flow step 4: the
 * workers' signs are summed as integers and thresholded by sign(); every
 * worker then applies W <- W - eta * vote.
 * bits : [M][words_stride] uint64 (8-byte aligned), worker-major packed
 *        signs (what an all-gather of the workers' 1-bit buffers delivers);
 *        words_stride >= ceil(count/64).
 * V_i  = sign(M - 2 * n_neg_i) in {-1, 0, +1} (0 only on ties, even M).
 * w    : [count] in wdt, updated in place: W <- rnd_W(fp32(W) - fp32(lr)*V),
 *        one float32 rounding, then RNE to bf16 for bf16 weights.
 * vote_out : optional [count] int8 out (NULL to skip; any alignment).
 * Errors: SM_ERR_ARG (null/misaligned, words_stride too small, lr not
 *         finite), SM_ERR_SHAPE (count < 0), SM_ERR_UNSUPPORTED (M < 1 or
 *         M > 64), SM_ERR_DTYPE.
 * ---------------------------------------------------------------------- */
sm_status sm_vote_update(const uint64_t* bits, int M, int64_t words_stride, int64_t count,
                         void* w, int wdt, float lr, int8_t* vote_out, hipStream_t s);

/* ------------------------------------------------------------------------
 * int8 sign encoding (the integer SUM all-reduce variant).
 * [SignMuon-ja] section 2, algorithm flow step 3 (all-reduce variant) and
 * communication efficiency: each entry's sign travels as one int8 (8 bits
 * per entry, 4x fewer bytes than float32), and the workers' signs are
 * summed as integers before the threshold.
 *
 * sm_sign_int8: s[i] = -1 if x[i] < 0 else +1 (+0, -0, NaN -> +1).
 *   x : [count] in dt (element-aligned).  s : [count] int8 out (any
 *   alignment; 8-byte alignment takes the vector path).
 *   Errors: SM_ERR_ARG (null/misaligned x), SM_ERR_SHAPE (count < 0),
 *   SM_ERR_DTYPE.  count == 0 is a no-op.
 * sm_vote_update_int8: sum_i = sum_m s[m][i] (integer), V_i = sign(sum_i)
 *   in {-1, 0, +1} (0 only on ties), then W <- rnd_W(fp32(W) - fp32(lr)*V)
 *   as sm_vote_update.  s : [M][stride] int8, worker m's signs at
 *   s + m*stride (stride >= count, in elements).  The signs must be -1 or
 *   +1 (as sm_sign_int8 writes them); the vote equals sm_vote_update's on
 *   the same signs.  vote_out : optional [count] int8.
 *   Errors: as sm_vote_update (stride < count -> SM_ERR_ARG).
 * ---------------------------------------------------------------------- */
typedef enum { SM_ENC_BITS = 0, SM_ENC_INT8 = 1 } sm_encoding;

sm_status sm_sign_int8(const void* x, int dt, int64_t count, int8_t* s, hipStream_t stream);
sm_status sm_vote_update_int8(const int8_t* s, int M, int64_t stride, int64_t count, void* w,
                              int wdt, float lr, int8_t* vote_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The vote as a matrix, and the dense update (the optional local polar step
 * on the vote).
 * [SignMuon-ja] section 2, algorithm flow step 5, and [SignMuon-abs]: a
 * worker may apply a local polar step to the aggregated sign matrix, at no
 * extra communication cost.  The library reads it as D = NS(V / (||V||_F +
 * eps)) with the step's Newton-Schulz settings, and W <- W - lr*D:
 * sm_vote -> sm_ns_polar (normalize = 1) -> sm_polar_update.
 *
 * sm_vote: V_i = sign(sum_m s_m,i) in {-1, 0, +1} written to v ([count] in
 *   vdt, 16-byte aligned).  signs: packed bits ([M][stride] uint64, 8-byte
 *   aligned, stride >= ceil(count/64) words) for encoding SM_ENC_BITS, or
 *   int8 signs ([M][stride] int8, stride >= count) for SM_ENC_INT8.
 *   Errors: SM_ERR_ARG (null/misaligned, bad encoding, stride too small),
 *   SM_ERR_SHAPE (count < 0), SM_ERR_UNSUPPORTED (M outside 1..64),
 *   SM_ERR_DTYPE.
 * sm_polar_update: w [count] in wdt updated in place, W <- rnd_W(fp32(W) -
 *   fp32(fp32(lr) * D)); d [count] in ddt.  Both 16-byte aligned, not
 *   overlapping.  Errors: SM_ERR_ARG (null/misaligned/overlap, lr not
 *   finite), SM_ERR_SHAPE, SM_ERR_DTYPE.
 * ---------------------------------------------------------------------- */
sm_status sm_vote(const void* signs, int encoding, int M, int64_t stride, int64_t count, void* v,
                  int vdt, hipStream_t stream);
sm_status sm_polar_update(void* w, int wdt, const void* d, int ddt, int64_t count, float lr,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * Spectral norm of a difference (the CacheMuon fidelity diagnostic).
 * [CacheMuon-ja] theoretical analysis: the cached direction's deviation
 * from the exact one is bounded in the spectral norm, ||D_hat - D||_sp <=
 * delta_t; experiments, diagnostic findings: the residual trigger tracks the
 * agreement between cached and fresh updates.  With the cached candidate
 * (sm_gram_ns_cached, mode 2) and the fresh direction (mode 1, on a copy of
 * the cache) of the same momentum, this call measures that distance.
 *
 * Per problem b, with E = a_b - b_b (b == NULL: E = a_b), m x n row-major
 * in dt: v = v0_b / ||v0_b||; `iters` times y = E v, z = E^T y, v = z/||z||
 * (v = 0 once z = 0); out[b] = ||E v||, a lower bound of ||E||_2 that
 * reaches it as iters grows (unless v0_b is orthogonal to E's top right
 * singular vector).  Arithmetic in float32 (norms in double); the sums run
 * in a fixed order.
 * a, b : [batch][m][n] in dt (element-aligned; 16-byte alignment and n % 8
 *        == 0 take the vector path).  v0 : [batch][n] float32, the start
 *        vectors (the caller's, e.g. seeded random).  out : [batch] float32.
 * iters: 0..100000.  ws : at least sm_spectral_norm_ws(...) bytes, 256-byte
 *        aligned.
 * Errors: SM_ERR_ARG (null/misaligned, bad iters, out overlapping ws),
 *         SM_ERR_SHAPE, SM_ERR_DTYPE, SM_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
sm_status sm_spectral_norm_ws(int batch, int m, int n, size_t* ws_bytes);
sm_status sm_spectral_norm(const void* a, const void* b, int dt, int batch, int m, int n,
                           const float* v0, int iters, float* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Whole optimizer step over a set of weight matrices.
 *
 * algo SM_SIGN_MUON  ([SignMuon-ja] section 2, algorithm flow steps 1-4):
 *   per worker M <- beta1*M + (1-beta1)*G, D = NS(M/(||M||_F+eps)),
 *   s = sign(D) packed to bits; V = majority vote; W <- W - lr*V.
 * algo SM_CACHE_MUON ([CacheMuon-ja] core mechanism): as Sign-Muon but D
 *   comes from the cached Gram-NS (q_cache, cache_state per matrix) with
 *   reuse threshold gamma and cache_mode as in sm_gram_ns_cached; update
 *   SM_UPDATE_POLAR (M must be 1) applies W <- W - lr*D, SM_UPDATE_VOTE
 *   votes the signs of D.
 * algo SM_LION_MUON  ([LionMuon-pt] core algorithm items 1-2):
 *   G_hat = beta1*M + (1-beta1)*G, then M <- beta2*M + (1-beta2)*G.  If
 *   period > 0 and t mod period == 0 the direction is NS(G_hat normalised)
 *   (a Muon step), otherwise sign(G_hat) (a Lion step; period 0 = never
 *   Muon).  Signs are voted over the M workers; with SM_UPDATE_POLAR and
 *   M = 1 a Muon step applies W <- W - lr*D instead.
 * encoding: how the signs travel between the a7 and a9 stages, SM_ENC_BITS
 *   (1-bit packing, the all-gather payload) or SM_ENC_INT8 (one int8 per
 *   entry, the SUM all-reduce payload); the vote, and so W, is identical.
 * vote_polar: 1 replaces W <- W - lr*V by the optional polar step on the
 *   vote, W <- W - lr*NS(V/(||V||_F+eps)), with the step's ns settings and
 *   the Newton-Schulz operand type mdt (vote updates only; ignored on a
 *   SM_UPDATE_POLAR Muon step).
 *
 * sm_matrix: m, n > 0; w [m][n] in wdt; mom [M][m][n] in mdt (updated in
 *   place); grad [M][m][n] in gdt (read-only); q_cache [M][r][r] float32 and
 *   cache_state [M][2] int32 for SM_CACHE_MUON, else NULL.
 * mdt is also the Newton-Schulz operand type (bf16 -> bf16 MFMA, f32 ->
 *   f32 MFMA); accumulation is always float32.
 * t: 1-based step index.  ws: at least sm_step_ws(...) bytes.
 * diag: optional device float [nmat][M][2] out = {err, refreshed} per
 *   (matrix, worker) for SM_CACHE_MUON (NULL to skip; ignored otherwise).
 * Errors: SM_ERR_ARG (also a bad encoding or vote_polar), SM_ERR_SHAPE,
 *   SM_ERR_DTYPE, SM_ERR_WORKSPACE, SM_ERR_UNSUPPORTED (M outside 1..64,
 *   POLAR with M != 1, SIGN_MUON with POLAR), SM_ERR_HIP.
 * ---------------------------------------------------------------------- */
typedef enum { SM_SIGN_MUON = 0, SM_CACHE_MUON = 1, SM_LION_MUON = 2 } sm_algo;
typedef enum { SM_UPDATE_VOTE = 0, SM_UPDATE_POLAR = 1 } sm_update;

typedef struct {
  int32_t m, n;
  void* w;
  void* mom;
  const void* grad;
  float* q_cache;
  int32_t* cache_state;
} sm_matrix;

typedef struct {
  int32_t algo;        /* sm_algo                                         */
  int32_t update;      /* sm_update                                       */
  int32_t M;           /* workers, 1..64                                  */
  int32_t wdt, mdt, gdt;
  float lr;
  float beta1;         /* EMA beta (Sign/CacheMuon) or Lion beta1          */
  float beta2;         /* Lion beta2 (LionMuon only)                       */
  int32_t period;      /* LionMuon P, 0 = infinity                         */
  sm_ns_params ns;
  float gamma;         /* CacheMuon residual threshold                     */
  int32_t cache_mode;  /* CacheMuon mode (0 trigger, 1 fresh, 2 reuse)     */
  int32_t encoding;    /* sm_encoding of the signs                         */
  int32_t vote_polar;  /* 1: polar step on the vote before the update      */
} sm_config;

sm_status sm_step_ws(const sm_config* c, const sm_matrix* mats, int nmat, size_t* ws_bytes);
sm_status sm_step(const sm_config* c, const sm_matrix* mats, int nmat, int64_t t,
                  void* ws, size_t ws_bytes, float* diag, hipStream_t s);

/* ------------------------------------------------------------------------
 * One optimizer step recorded as a HIP graph and replayed.
 * [SignMuon-ja] section 2, algorithm flow steps 1-4 and [LionMuon-pt]
 * methodology item 1: the same step, with the same matrices, runs at every
 * iteration t -> t+1; a step of many small matrices is bound by its kernel
 * launches, which one graph launch replaces.
 *
 * sm_step_graph records sm_step(c, mats, nmat, t, ws, ws_bytes, diag) on a
 * private stream, without running it, and returns an instantiated graph in
 * *out.  Arguments as for sm_step; the config and matrix arrays are read
 * during the call only, while the device buffers they name (w, mom, grad,
 * ws, diag) must stay allocated, in place, until sm_graph_destroy: every
 * replay reads and writes them as one sm_step call does.  sm_graph_launch
 * enqueues one replay on s (results bit-identical to sm_step at the
 * recorded t); replays must not overlap one another or other calls that
 * use the same buffers (two graphs may share a workspace).  For SM_LION_MUON the
 * step type follows t (a Muon step iff t % period == 0): record one graph
 * per type.  The recorded kernels do not read t otherwise.
 * Errors: as sm_step; SM_ERR_UNSUPPORTED for SM_CACHE_MUON (its kernels store
 * t with each refresh) or while kernel-time accounting is enabled;
 * SM_ERR_HIP if capture or instantiation fails.  *out is NULL on error.
 * sm_graph_destroy releases the graph and does not wait: call it once the
 * replays enqueued so far have finished.  sm_graph_destroy(NULL) is a no-op.
 * ---------------------------------------------------------------------- */
typedef struct sm_graph_s* sm_graph;
sm_status sm_step_graph(const sm_config* c, const sm_matrix* mats, int nmat, int64_t t,
                        void* ws, size_t ws_bytes, float* diag, sm_graph* out);
sm_status sm_graph_launch(sm_graph g, hipStream_t s);
sm_status sm_graph_destroy(sm_graph g);

/* ------------------------------------------------------------------------
 * Kernel-time accounting (for benchmarks; not part of the method).
 * While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events on its stream, tagged with its kind and its algorithmic work
 * (flops for GEMMs, bytes for streaming kernels).  sm_profile_read waits for
 * the recorded events and returns the totals for one kind;
 * sm_profile_read_bytes returns the kind's algorithmic HBM bytes (every
 * operand read once, every output written once; for streaming kinds the
 * same as the work), from which a GEMM's arithmetic intensity follows.
 * Launches whose problems run only if a device flag says so (CacheMuon's
 * fresh solve and cached candidate) are credited with the work of the
 * problems that actually ran: those kernels add it to a small device-side
 * accumulator, which reading and resetting synchronise the device to copy.
 * Enabling creates an event pool (up to 65536 launches); reading or
 * disabling never allocates.  Not thread-safe; meant for one benchmarking
 * thread, outside timed regions for reads and resets.
 * ---------------------------------------------------------------------- */
enum {
  SM_K_EMA = 0,          /* momentum EMA (+ norm partials)         bytes  */
  SM_K_NORM = 1,         /* sum-of-squares / scale finalize        bytes  */
  SM_K_GEMM_GRAM = 2,    /* X X^T (NS and Gram-NS)                 flops  */
  SM_K_GEMM_APPLY = 3,   /* a X + B X  /  Q X                      flops  */
  SM_K_GEMM_RR = 4,      /* r x r products of Gram-NS / quintic    flops  */
  SM_K_PROBE = 5,        /* residual D D^T - I                     flops  */
  SM_K_SIGN_PACK = 6,    /* sign + 1-bit pack                      bytes  */
  SM_K_VOTE_UPDATE = 7,  /* vote + W update                        bytes  */
  SM_K_LION = 8,         /* fused Lion interpolation/EMA/sign/pack bytes  */
  SM_K_POLAR_UPDATE = 9, /* W <- W - lr D                          bytes  */
  SM_K_MISC = 10,        /* small finalize / copy kernels          bytes  */
  SM_K_SPECTRAL = 11,    /* power-method passes (diagnostic)       bytes  */
  SM_K_NUM_KINDS = 12
};
sm_status sm_profile_enable(int on);
sm_status sm_profile_reset(void);
sm_status sm_profile_read(int kind, double* ms_total, int64_t* launches, double* work);
sm_status sm_profile_read_bytes(int kind, double* bytes);
const char* sm_kernel_kind_name(int kind);

/* ------------------------------------------------------------------------
 * MFMA ceiling probe (for benchmarks; not part of the method).
 * The NS GEMMs are priced against the chip's nominal bf16 dense peak, which
 * assumes every matrix pipe busy at the top shader clock; under a sustained
 * matrix load the clock drops.  This call measures the rate a bf16 GEMM k
 * loop of the NS kernels' tile shape can reach: `blocks` workgroups of four
 * waves, each wave running `iters` k16 slices of sixteen
 * v_mfma_f32_32x32x16_bf16 on a 128x128 float32 accumulator block, with the
 * fragments
 *   mode 0: rotated in registers;
 *   mode 1: read from LDS every slice (no global memory in the loop);
 *   mode 2: as mode 1, plus per two slices the NS kernels' operand staging
 *           (eight 16-byte direct-to-LDS loads per wave from `src`, a wait
 *           for the loads of three steps before, one workgroup barrier).
 * It executes blocks * 4 * iters * 16 * 32768 flops.  out: blocks * 256
 * floats of device memory (caller-owned, 4-byte aligned) that receive
 * per-thread sums of the accumulators.  src (mode 2 only, else ignored):
 * src_bytes of device memory, a power of two from 64 KB to 64 MB, 16-byte
 * aligned, only read (keep it L2-sized to leave out cache misses).
 * blocks: 1..65536, iters: 1..10^7.  SM_ERR_ARG for a bad mode or a null or
 * misaligned pointer, SM_ERR_SHAPE for sizes out of range.  Time it with
 * events on `s`.
 * ---------------------------------------------------------------------- */
sm_status sm_mfma_ceiling(int mode, int blocks, int iters, const void* src, size_t src_bytes,
                          float* out, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* SM_H */
