// C ABI of the fused SO(2) convolution: argument checks, workspace layout and
// the kernel schedules of the forward, backward and double backward.
#include <complex>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/so2conv.h"
#include "gemm.hpp"
#include "ops.hpp"
#include "wigner.hpp"

namespace so2 {
int upload_generators_fwd(const float* host);
int upload_generators_bwd(const float* host);
int upload_generators_dual(const float* host);
}  // namespace so2

using namespace so2;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define SO2_HIP(expr)                                                                       \
  do {                                                                                      \
    int _e = (int)(expr);                                                                   \
    if (_e != 0) return fail(SO2_EHIP, std::string("HIP error in ") + #expr + ": " +       \
                                           hipGetErrorString((hipError_t)_e));              \
  } while (0)

inline size_t al(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------- generators
// G_k^(l) = d/dt D^(l)(exp(t [e_k]_x)) at t = 0, evaluated exactly by a
// complex step through the Wigner recursion: D(I + i h K) = D(I) + i h G + O(h^2).
void compute_generators(float* out) {
  using cd = std::complex<double>;
  const double h = 1e-30;
  const int cross[3][9] = {{0, 0, 0, 0, 0, -1, 0, 1, 0}, {0, 0, 1, 0, 0, 0, -1, 0, 0}, {0, -1, 0, 1, 0, 0, 0, 0, 0}};
  std::memset(out, 0, sizeof(float) * 3 * kGenSize);
  for (int k = 0; k < 3; ++k) {
    cd R[9], D1[9];
    for (int a = 0; a < 9; ++a) R[a] = cd((a % 4 == 0) ? 1.0 : 0.0, h * cross[k][a]);
    wigner_l1<cd>(R, D1);
    float* G = out + k * kGenSize;
    for (int a = 0; a < 9; ++a) G[1 + a] = (float)(D1[a].imag() / h);
    std::vector<cd> prev(D1, D1 + 9), cur;
    int off = 10;
    for (int l = 2; l <= kMaxL; ++l) {
      const int n = 2 * l + 1;
      cur.assign(n * n, cd(0));
      for (int m = -l; m <= l; ++m)
        for (int c = -l; c <= l; ++c) cur[(m + l) * n + c + l] = wig_entry<cd>(l, m, c, D1, prev.data(), l - 1);
      for (int a = 0; a < n * n; ++a) G[off + a] = (float)(cur[a].imag() / h);
      off += n * n;
      prev = cur;
    }
  }
}

std::mutex g_init_mu;
bool g_init_done[64];

int ensure_init() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SO2_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(SO2_EUNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_init_mu);
  if (g_init_done[dev]) return SO2_OK;
  static float table[3 * kGenSize];
  static bool have = false;
  if (!have) {
    compute_generators(table);
    have = true;
  }
  SO2_HIP(upload_generators_fwd(table));
  SO2_HIP(upload_generators_bwd(table));
  SO2_HIP(upload_generators_dual(table));
  g_init_done[dev] = true;
  return SO2_OK;
}

// ---------------------------------------------------------------- checks
int check_cfg(const so2conv_cfg* cfg, Dims* d) {
  if (!cfg) return fail(SO2_EINVAL, "cfg is NULL");
  const int L = cfg->lmax, M = cfg->mmax, C = cfg->channels;
  if (L < 0 || L > kMaxL) return fail(SO2_EUNSUPPORTED, "lmax must be in [0, 6]");
  if (M < 0 || M > L) return fail(SO2_EINVAL, "mmax must be in [0, lmax]");
  if (!lm_supported(L, M)) return fail(SO2_EUNSUPPORTED, "(lmax, mmax) pair has no compiled kernels");
  if (C < 16 || C > 256 || C % 16) return fail(SO2_EUNSUPPORTED, "channels must be a multiple of 16 in [16, 256]");
  if (cfg->n_rbf < 4 || cfg->n_rbf % 4 || cfg->n_rbf > 1024)
    return fail(SO2_EUNSUPPORTED, "n_rbf must be a multiple of 4 in [4, 1024]");
  if (cfg->dtype != SO2_F32) return fail(SO2_EUNSUPPORTED, "only float32 is supported");
  d->L = L;
  d->M = M;
  d->C = C;
  return SO2_OK;
}

int check_graph(const so2conv_graph* g, GraphDev* gd) {
  if (!g) return fail(SO2_EINVAL, "graph is NULL");
  if (g->n_nodes < 0 || g->n_edges < 0) return fail(SO2_EINVAL, "negative graph size");
  if (g->n_edges > 0x3fffffffLL) return fail(SO2_EUNSUPPORTED, "too many edges (int32 edge ids, 2E rows)");
  if (g->n_edges > 0 && (!g->src || !g->dst || !g->src_perm)) return fail(SO2_EINVAL, "graph index arrays are NULL");
  if (!g->dst_ptr || !g->src_ptr) return fail(SO2_EINVAL, "graph CSR arrays are NULL");
  gd->N = g->n_nodes;
  gd->E = g->n_edges;
  gd->src = g->src;
  gd->dst = g->dst;
  gd->shift = g->shift;
  gd->dst_ptr = g->dst_ptr;
  gd->src_perm = g->src_perm;
  gd->src_ptr = g->src_ptr;
  gd->e0 = 0;
  gd->e1 = g->n_edges;
  return SO2_OK;
}

// ---------------------------------------------------------------- layouts
struct SavedLayout {
  size_t S, T, U, Z, V, total;
};
SavedLayout saved_layout(const Dims& d, int n_rbf, long E) {
  (void)n_rbf;
  SavedLayout s;
  size_t o = 0;
  const size_t e = (size_t)E;
  s.S = o; o += al(sizeof(float) * e * (d.L + 1) * d.Ci());
  s.T = o; o += al(sizeof(float) * e * d.wT());
  s.U = o; o += al(sizeof(float) * e * d.wU());
  s.Z = o; o += al(sizeof(float) * e * d.wZ());
  s.V = o; o += al(sizeof(float) * e * d.wZ());
  s.total = o;
  return s;
}

// K chunk of split-K weight-gradient products over edges
void split_plan(long K, int* splits, int* chunk) {
  long c = 4096;
  long s = (K + c - 1) / c;
  if (s > 256) {
    c = ((K + 255) / 256 + 15) / 16 * 16;
    s = (K + c - 1) / c;
  }
  if (s < 1) s = 1;
  *splits = (int)s;
  *chunk = (int)c;
}

struct Arena {
  char* base;
  size_t used;
  float* take(size_t floats) {
    float* p = reinterpret_cast<float*>(base ? base + used : nullptr);
    used += al(sizeof(float) * floats);
    return p;
  }
};

// ---------------------------------------------------------------- gemm helpers
GemmProb prob(const float* A, int lda, const float* B, int ldb, float* C, int ldc, int M, int N, int K, int acc = 0) {
  GemmProb p{};
  p.A = A; p.B = B; p.C = C;
  p.M = M; p.N = N; p.K = K;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc;
  p.k_splits = 1; p.k_chunk = K; p.accumulate = acc;
  return p;
}

// ---------------------------------------------------------------- GEMM timing
// When enabled, every MFMA GEMM launch is bracketed by HIP events on the
// launching stream and its algorithmic flop count (2 M N K summed over the
// launch's problems) is recorded; so2conv_profile_read reports the totals.
struct ProfRec {
  int kind;          // 0 NN, 1 NT, 2 TN
  double flops;
  double bytes;      // algorithmic: A, B read once, C (or the split partials) written once
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

int run_batch(std::vector<GemmProb>& ps, bool TA, bool TB, hipStream_t s) {
  size_t i = 0;
  while (i < ps.size()) {
    GemmBatch b{};
    b.nprob = 0;
    double flops = 0, bytes = 0;
    while (i < ps.size() && b.nprob < kGemmMaxProbs) {
      const GemmProb& q = ps[i];
      flops += 2.0 * q.M * (double)q.N * q.K;
      bytes += 4.0 * ((double)q.M * q.K + (double)q.K * q.N +
                      (double)q.M * q.N * (q.partial ? q.k_splits : 1) * (q.accumulate ? 2 : 1));
      b.p[b.nprob++] = ps[i++];
    }
    if (g_prof_on) {
      ProfRec r{TA ? 2 : (TB ? 1 : 0), flops, bytes, nullptr, nullptr};
      SO2_HIP(hipEventCreate(&r.a));
      SO2_HIP(hipEventCreate(&r.b));
      SO2_HIP(hipEventRecord(r.a, s));
      SO2_HIP(gemm_run(b, TA, TB, s));
      SO2_HIP(hipEventRecord(r.b, s));
      std::lock_guard<std::mutex> lk(g_prof_mu);
      g_prof.push_back(r);
    } else {
      SO2_HIP(gemm_run(b, TA, TB, s));
    }
  }
  return SO2_OK;
}

// Weight gradient G[M][N] (+)= sum over segments of A_s^T B_s, A_s [K_s][lda], B_s [K_s][ldb];
// deterministic split-K through the partial buffer P.
struct TnSeg {
  const float* A;
  int lda;
  const float* B;
  int ldb;
  long K;
};
size_t tn_partial_floats(long K_total_rows, int nseg, int M, int N) {
  int sp, ch;
  split_plan(K_total_rows, &sp, &ch);
  return (size_t)(sp + nseg) * M * N;
}
int run_tn(const TnSeg* segs, int nseg, int M, int N, float* G, int ldg, int accumulate, float* P, hipStream_t s) {
  std::vector<GemmProb> ps;
  int total_splits = 0;
  for (int q = 0; q < nseg; ++q) {
    if (segs[q].K <= 0) continue;
    int sp, ch;
    split_plan(segs[q].K, &sp, &ch);
    GemmProb p = prob(segs[q].A, segs[q].lda, segs[q].B, segs[q].ldb, P + (size_t)total_splits * M * N, N, M, N,
                      (int)segs[q].K);
    p.k_splits = sp;
    p.k_chunk = ch;
    p.partial = 1;
    total_splits += p.k_splits;
    ps.push_back(p);
  }
  if (total_splits == 0) return SO2_OK;
  int r = run_batch(ps, true, false, s);
  if (r) return r;
  SO2_HIP(gemm_reduce(P, total_splits, M, N, G, ldg, accumulate, s));
  return SO2_OK;
}

__global__ void fill_kernel(float* p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}
int fill(float* p, size_t n, hipStream_t s) {
  if (n == 0) return SO2_OK;
  size_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)b), dim3(256), 0, s, p, n, 0.f);
  SO2_HIP(hipGetLastError());
  return SO2_OK;
}

// S = rbf W_rad
int radial(const Dims& d, int n_rbf, long E, const float* rbf, const float* w_rad, float* S, hipStream_t s, int acc = 0) {
  std::vector<GemmProb> ps{prob(rbf, n_rbf, w_rad, (d.L + 1) * d.Ci(), S, (d.L + 1) * d.Ci(), (int)E,
                                (d.L + 1) * d.Ci(), n_rbf, acc)};
  return run_batch(ps, false, false, s);
}

// first linear: U[:, block a] = T[:, block a] W1r_a  (rows = E * rowmul stacked)
void lin1_probs(const Dims& d, const float* T, const float* W1r, float* U, int rows, int acc, std::vector<GemmProb>& ps) {
  for (int a = 0; a <= d.M; ++a) {
    int r, c;
    long off;
    realified_shape(d, 0, a, &r, &c, &off);
    ps.push_back(prob(T + mm_block(a, d.L, d.Ci()), d.wT(), W1r + off, c, U + d.u_block(a), d.wU(), rows, c, r, acc));
  }
}
void lin2_probs(const Dims& d, const float* Z, const float* W2r, float* V, int rows, int acc, std::vector<GemmProb>& ps) {
  for (int a = 0; a <= d.M; ++a) {
    int r, c;
    long off;
    realified_shape(d, 1, a, &r, &c, &off);
    ps.push_back(prob(Z + mm_block(a, d.L, d.C), d.wZ(), W2r + off, c, V + mm_block(a, d.L, d.C), d.wZ(), rows, c, r, acc));
  }
}
// transposed products: Tbar[:, a] = Ubar[:, a] W1r_a^T
void lin1t_probs(const Dims& d, const float* Ub, const float* W1r, float* Tb, int rows, int acc, std::vector<GemmProb>& ps) {
  for (int a = 0; a <= d.M; ++a) {
    int r, c;
    long off;
    realified_shape(d, 0, a, &r, &c, &off);
    ps.push_back(prob(Ub + d.u_block(a), d.wU(), W1r + off, c, Tb + mm_block(a, d.L, d.Ci()), d.wT(), rows, r, c, acc));
  }
}
void lin2t_probs(const Dims& d, const float* Vb, const float* W2r, float* Zb, int rows, int acc, std::vector<GemmProb>& ps) {
  for (int a = 0; a <= d.M; ++a) {
    int r, c;
    long off;
    realified_shape(d, 1, a, &r, &c, &off);
    ps.push_back(prob(Vb + mm_block(a, d.L, d.C), d.wZ(), W2r + off, c, Zb + mm_block(a, d.L, d.C), d.wZ(), rows, r, c, acc));
  }
}

bool all_null(const float* const* p, int n) {
  if (!p) return true;
  for (int i = 0; i < n; ++i)
    if (p[i]) return false;
  return true;
}

int check_weights(const Dims& d, const float* w_rad, const float* const* w1, const float* const* w2) {
  if (!w_rad) return fail(SO2_EINVAL, "w_rad is NULL");
  if (!w1 || !w2) return fail(SO2_EINVAL, "weight pointer arrays are NULL");
  for (int a = 0; a <= d.M; ++a)
    if (!w1[a] || !w2[a]) return fail(SO2_EINVAL, "a weight block pointer is NULL");
  return SO2_OK;
}

size_t ws_weights(const Dims& d) {
  return al(sizeof(float) * realified_size(d, 0)) + al(sizeof(float) * realified_size(d, 1));
}

// largest weight-gradient block (floats): realified blocks and the radial matrix
size_t max_grad_block(const Dims& d, int n_rbf) {
  size_t mx = (size_t)n_rbf * (d.L + 1) * d.Ci();
  for (int second = 0; second < 2; ++second)
    for (int a = 0; a <= d.M; ++a) {
      int r, c;
      long off;
      realified_shape(d, second, a, &r, &c, &off);
      if ((size_t)r * c > mx) mx = (size_t)r * c;
    }
  return mx;
}

size_t primal_floats(const Dims& d) { return (size_t)(d.L + 1) * d.Ci() + d.wT() + d.wU() + 2 * (size_t)d.wZ(); }

// Workspace of one stage for a chunk of `ec` edges out of E.
//   stage 0: forward; 1: backward; 2: double backward.
//   recompute: the per-edge forward state lives in the workspace (saved == NULL).
size_t ws_need(const Dims& d, int n_rbf, long E, long ec, int stage, bool recompute) {
  const size_t e = (size_t)ec;
  const size_t wS = (size_t)(d.L + 1) * d.Ci();
  size_t b = ws_weights(d);
  size_t per = recompute ? primal_floats(d) : 0;
  int nseg = 1;
  if (stage == 1) {
    per += 2 * (size_t)d.wZ() + d.wU() + d.wT() + wS + 9;
    b += ws_weights(d);                               // realified weight gradients
    b += al(sizeof(float) * 3 * (size_t)E);           // per-edge position gradient (all edges)
  } else if (stage == 2) {
    b += 2 * ws_weights(d);                           // direction weights, weight gradients
    per += wS + d.wT() + 3 + d.wU() + 2 * (size_t)d.wZ() + 4 * (size_t)d.wZ() + 2 * (size_t)d.wU() +
           2 * (size_t)d.wT() + 2 * wS;
    nseg = 2;
  }
  b += 24 * 256 + sizeof(float) * per * e;           // per-edge buffers (+ alignment)
  if (stage > 0) {
    int sp, ch;
    split_plan(ec, &sp, &ch);
    b += al(sizeof(float) * (size_t)nseg * (sp + 1) * max_grad_block(d, n_rbf));
  }
  return b + 4096;
}

// edges per chunk that fit in ws_bytes (E if everything fits; 0 if not even 1024 edges do)
long pick_chunk(const Dims& d, int n_rbf, long E, int stage, bool recompute, size_t ws_bytes) {
  if (E == 0) return 0;
  if (ws_need(d, n_rbf, E, E, stage, recompute) <= ws_bytes) return E;
  long lo = 0, hi = E;
  while (hi - lo > 1024) {
    const long mid = (lo + hi) / 2 / 1024 * 1024;
    if (mid <= lo) break;
    if (ws_need(d, n_rbf, E, mid, stage, recompute) <= ws_bytes) lo = mid;
    else hi = mid;
  }
  if (lo == 0 && ws_need(d, n_rbf, E, 1024 < E ? 1024 : E, stage, recompute) <= ws_bytes) lo = 1024 < E ? 1024 : E;
  return lo;
}

struct Primal {
  const float *S, *T, *U, *Z, *V;
};

// forward state of the chunk [g.e0, g.e1) into (S, T, U, Z, V)
int forward_chunk(const Dims& d, int n_rbf, const GraphDev& g, const float* x, const float* pos, const float* rbf,
                  const float* w_rad, const float* W1r, const float* W2r, float* S, float* T, float* U, float* Z,
                  float* V, hipStream_t s) {
  const int ec = (int)(g.e1 - g.e0);
  int r;
  if ((r = radial(d, n_rbf, ec, rbf + (size_t)g.e0 * n_rbf, w_rad, S, s))) return r;
  SO2_HIP(launch_edge_fwd(d, g, x, pos, S, T, s));
  std::vector<GemmProb> ps;
  lin1_probs(d, T, W1r, U, ec, 0, ps);
  if ((r = run_batch(ps, false, false, s))) return r;
  SO2_HIP(launch_gate_fwd(d, ec, U, Z, s));
  ps.clear();
  lin2_probs(d, Z, W2r, V, ec, 0, ps);
  return run_batch(ps, false, false, s);
}

int zero_grads(const Dims& d, int n_rbf, int N, float* gx, float* gpos, float* gw_rad, float* const* gw1,
               float* const* gw2, hipStream_t s) {
  int r;
  const size_t dC = (size_t)d.d() * d.C;
  if (gx && (r = fill(gx, (size_t)N * dC, s))) return r;
  if (gpos && (r = fill(gpos, (size_t)N * 3, s))) return r;
  if (gw_rad && (r = fill(gw_rad, (size_t)n_rbf * (d.L + 1) * d.Ci(), s))) return r;
  for (int a = 0; a <= d.M; ++a) {
    int rr, cc;
    long off;
    realified_shape(d, 0, a, &rr, &cc, &off);
    if (gw1 && gw1[a] && (r = fill(gw1[a], (size_t)(a ? rr / 2 : rr) * cc, s))) return r;
    realified_shape(d, 1, a, &rr, &cc, &off);
    if (gw2 && gw2[a] && (r = fill(gw2[a], (size_t)(a ? rr / 2 : rr) * cc, s))) return r;
  }
  return SO2_OK;
}

}  // namespace

// =====================================================================================
extern "C" {

const char* so2conv_last_error(void) { return g_err.c_str(); }

int so2conv_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return SO2_OK;
}

int so2conv_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  return SO2_OK;
}

int so2conv_profile_read(int kind, int64_t* launches, double* total_ms, double* total_flops, double* total_bytes) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int64_t n = 0;
  double ms = 0, fl = 0, by = 0;
  for (auto& r : g_prof) {
    if (kind >= 0 && r.kind != kind) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(SO2_EHIP, "hipEventSynchronize failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return fail(SO2_EHIP, "hipEventElapsedTime failed");
    ++n;
    ms += t;
    fl += r.flops;
    by += r.bytes;
  }
  if (launches) *launches = n;
  if (total_ms) *total_ms = ms;
  if (total_flops) *total_flops = fl;
  if (total_bytes) *total_bytes = by;
  return SO2_OK;
}

int so2conv_supported(int32_t lmax, int32_t mmax) { return lm_supported(lmax, mmax) ? 1 : 0; }

size_t so2conv_graph_workspace_bytes(int32_t n_nodes, int64_t n_edges) { return graph_ws_bytes(n_nodes, n_edges); }

int so2conv_graph_prepare(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst, int32_t* dst_ptr,
                          int32_t* src_perm, int32_t* src_ptr, int32_t* err_word, void* ws, size_t ws_bytes,
                          void* stream) {
  g_err.clear();
  if (n_nodes < 0 || n_edges < 0) return fail(SO2_EINVAL, "negative graph size");
  if (n_edges > 0x3fffffffLL) return fail(SO2_EUNSUPPORTED, "too many edges");
  if (n_edges > 0 && (!src || !dst || !src_perm)) return fail(SO2_EINVAL, "NULL edge arrays");
  if (!dst_ptr || !src_ptr) return fail(SO2_EINVAL, "NULL CSR outputs");
  if (!ws || ws_bytes < graph_ws_bytes(n_nodes, n_edges)) return fail(SO2_EWORKSPACE, "graph workspace too small");
  SO2_HIP(launch_graph_prepare(n_nodes, n_edges, src, dst, dst_ptr, src_perm, src_ptr, ws, ws_bytes, err_word,
                               (hipStream_t)stream));
  return SO2_OK;
}

size_t so2conv_saved_bytes(const so2conv_cfg* cfg, int64_t n_edges) {
  Dims d;
  if (check_cfg(cfg, &d)) return 0;
  return saved_layout(d, cfg->n_rbf, n_edges).total;
}

size_t so2conv_workspace_bytes(const so2conv_cfg* cfg, int32_t n_nodes, int64_t n_edges, int stage) {
  (void)n_nodes;
  Dims d;
  if (check_cfg(cfg, &d) || stage < 0 || stage > 2) return 0;
  return ws_need(d, cfg->n_rbf, n_edges, n_edges, stage, false);
}

size_t so2conv_chunked_workspace_bytes(const so2conv_cfg* cfg, int32_t n_nodes, int64_t n_edges, int stage,
                                       int64_t chunk_edges) {
  (void)n_nodes;
  Dims d;
  if (check_cfg(cfg, &d) || stage < 0 || stage > 2 || chunk_edges < 1) return 0;
  const long ec = chunk_edges < n_edges ? chunk_edges : n_edges;
  return ws_need(d, cfg->n_rbf, n_edges, ec, stage, true);
}

int so2conv_debug_rotate_gather(const so2conv_cfg* cfg, const so2conv_graph* g, const float* x, const float* pos,
                                const float* rbf, const float* w_rad, float* T_out, void* ws, size_t ws_bytes,
                                void* stream) {
  g_err.clear();
  Dims d;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &d)) || (r = check_graph(g, &gd))) return r;
  if ((r = ensure_init())) return r;
  if (!x || !pos || !rbf || !w_rad || !T_out) return fail(SO2_EINVAL, "NULL input");
  const size_t need = al(sizeof(float) * (size_t)gd.E * (d.L + 1) * d.Ci());
  if (!ws || ws_bytes < need) return fail(SO2_EWORKSPACE, "workspace too small (needs E*(L+1)*2C floats)");
  hipStream_t s = (hipStream_t)stream;
  float* S = static_cast<float*>(ws);
  if ((r = radial(d, cfg->n_rbf, gd.E, rbf, w_rad, S, s))) return r;
  SO2_HIP(launch_edge_fwd(d, gd, x, pos, S, T_out, s));
  return SO2_OK;
}

int so2conv_fwd(const so2conv_cfg* cfg, const so2conv_graph* g, const float* x, const float* pos, const float* rbf,
                const float* w_rad, const float* const* w1, const float* const* w2, float* y, void* saved, void* ws,
                size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &d)) || (r = check_graph(g, &gd))) return r;
  if ((r = check_weights(d, w_rad, w1, w2))) return r;
  if (!x || !pos || (!rbf && gd.E > 0) || !y) return fail(SO2_EINVAL, "NULL input or output");
  if ((r = ensure_init())) return r;
  const int n_rbf = cfg->n_rbf;
  const bool recompute = saved == nullptr;
  if (!ws) return fail(SO2_EWORKSPACE, "workspace is NULL");
  const long ec = pick_chunk(d, n_rbf, gd.E, 0, recompute, ws_bytes);
  if (gd.E > 0 && ec == 0) return fail(SO2_EWORKSPACE, "forward workspace too small for a 1024-edge chunk");
  if (ws_bytes < ws_weights(d)) return fail(SO2_EWORKSPACE, "forward workspace too small");
  hipStream_t s = (hipStream_t)stream;
  Arena ar{static_cast<char*>(ws), 0};
  float* W1r = ar.take(realified_size(d, 0));
  float* W2r = ar.take(realified_size(d, 1));
  const SavedLayout sl = saved_layout(d, n_rbf, gd.E);
  char* st = static_cast<char*>(saved);
  float *S = nullptr, *T = nullptr, *U = nullptr, *Z = nullptr, *V = nullptr;
  if (recompute) {
    S = ar.take((size_t)ec * (d.L + 1) * d.Ci());
    T = ar.take((size_t)ec * d.wT());
    U = ar.take((size_t)ec * d.wU());
    Z = ar.take((size_t)ec * d.wZ());
    V = ar.take((size_t)ec * d.wZ());
  }
  SO2_HIP(launch_realify(d, 0, w1, W1r, s));
  SO2_HIP(launch_realify(d, 1, w2, W2r, s));
  if (gd.E == 0) {
    GraphDev gc = gd;
    gc.e0 = gc.e1 = 0;
    SO2_HIP(launch_node_fwd(d, gc, pos, nullptr, y, 0, s));
    return SO2_OK;
  }
  for (long e0 = 0, c = 0; e0 < gd.E; e0 += ec, ++c) {
    GraphDev gc = gd;
    gc.e0 = e0;
    gc.e1 = e0 + ec < gd.E ? e0 + ec : gd.E;
    float *Sc = S, *Tc = T, *Uc = U, *Zc = Z, *Vc = V;
    if (!recompute) {
      Sc = reinterpret_cast<float*>(st + sl.S) + (size_t)e0 * (d.L + 1) * d.Ci();
      Tc = reinterpret_cast<float*>(st + sl.T) + (size_t)e0 * d.wT();
      Uc = reinterpret_cast<float*>(st + sl.U) + (size_t)e0 * d.wU();
      Zc = reinterpret_cast<float*>(st + sl.Z) + (size_t)e0 * d.wZ();
      Vc = reinterpret_cast<float*>(st + sl.V) + (size_t)e0 * d.wZ();
    }
    if ((r = forward_chunk(d, n_rbf, gc, x, pos, rbf, w_rad, W1r, W2r, Sc, Tc, Uc, Zc, Vc, s))) return r;
    SO2_HIP(launch_node_fwd(d, gc, pos, Vc, y, c > 0, s));
  }
  return SO2_OK;
}

int so2conv_bwd(const so2conv_cfg* cfg, const so2conv_graph* g, const float* x, const float* pos, const float* rbf,
                const float* w_rad, const float* const* w1, const float* const* w2, const void* saved,
                const float* gy, float* gx, float* gpos, float* grbf, float* gw_rad, float* const* gw1,
                float* const* gw2, float* gedge, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &d)) || (r = check_graph(g, &gd))) return r;
  if ((r = check_weights(d, w_rad, w1, w2))) return r;
  if (!x || !pos || !gy || (!rbf && gd.E > 0)) return fail(SO2_EINVAL, "NULL input");
  if ((r = ensure_init())) return r;
  hipStream_t s = (hipStream_t)stream;
  const int n_rbf = cfg->n_rbf, wS = (d.L + 1) * d.Ci();
  if (gd.E == 0) return zero_grads(d, n_rbf, gd.N, gx, gpos, gw_rad, gw1, gw2, s);
  const bool recompute = saved == nullptr;
  if (!ws) return fail(SO2_EWORKSPACE, "workspace is NULL");
  const long ec = pick_chunk(d, n_rbf, gd.E, 1, recompute, ws_bytes);
  if (ec == 0) return fail(SO2_EWORKSPACE, "backward workspace too small for a 1024-edge chunk");
  const SavedLayout sl = saved_layout(d, n_rbf, gd.E);
  const char* st = static_cast<const char*>(saved);
  Arena ar{static_cast<char*>(ws), 0};
  float* W1r = ar.take(realified_size(d, 0));
  float* W2r = ar.take(realified_size(d, 1));
  float* gW1r = ar.take(realified_size(d, 0));
  float* gW2r = ar.take(realified_size(d, 1));
  float* vbar_all = ar.take((size_t)gd.E * 3);
  float *S = nullptr, *T = nullptr, *U = nullptr, *Z = nullptr, *V = nullptr;
  if (recompute) {
    S = ar.take((size_t)ec * wS);
    T = ar.take((size_t)ec * d.wT());
    U = ar.take((size_t)ec * d.wU());
    Z = ar.take((size_t)ec * d.wZ());
    V = ar.take((size_t)ec * d.wZ());
  }
  float* tbar = ar.take((size_t)ec * d.wZ());
  float* Zbar = ar.take((size_t)ec * d.wZ());
  float* Ubar = ar.take((size_t)ec * d.wU());
  float* Tbar = ar.take((size_t)ec * d.wT());
  float* Sbar = ar.take((size_t)ec * wS);
  float* tau1 = ar.take((size_t)ec * 3);
  float* tau2 = ar.take((size_t)ec * 3);
  float* tau3 = ar.take((size_t)ec * 3);
  float* P = ar.take(0);
  float* vbar = gedge ? gedge : vbar_all;
  const bool want_w1 = !all_null(gw1, d.M + 1), want_w2 = !all_null(gw2, d.M + 1);

  SO2_HIP(launch_realify(d, 0, w1, W1r, s));
  SO2_HIP(launch_realify(d, 1, w2, W2r, s));
  for (long e0 = 0, c = 0; e0 < gd.E; e0 += ec, ++c) {
    GraphDev gc = gd;
    gc.e0 = e0;
    gc.e1 = e0 + ec < gd.E ? e0 + ec : gd.E;
    const int n = (int)(gc.e1 - gc.e0);
    const int acc = c > 0;
    Primal pr;
    if (recompute) {
      if ((r = forward_chunk(d, n_rbf, gc, x, pos, rbf, w_rad, W1r, W2r, S, T, U, Z, V, s))) return r;
      pr = {S, T, U, Z, V};
    } else {
      pr = {reinterpret_cast<const float*>(st + sl.S) + (size_t)e0 * wS,
            reinterpret_cast<const float*>(st + sl.T) + (size_t)e0 * d.wT(),
            reinterpret_cast<const float*>(st + sl.U) + (size_t)e0 * d.wU(),
            reinterpret_cast<const float*>(st + sl.Z) + (size_t)e0 * d.wZ(),
            reinterpret_cast<const float*>(st + sl.V) + (size_t)e0 * d.wZ()};
    }
    // E -> N transpose: tbar = R gy[dst], tau1 = rotation torque of <V, R gy>
    SO2_HIP(launch_edge_bwd(d, gc, pos, gy, pr.V, tbar, tau1, s));
    std::vector<GemmProb> ps;
    lin2t_probs(d, tbar, W2r, Zbar, n, 0, ps);
    if ((r = run_batch(ps, false, true, s))) return r;
    if (want_w2) {
      for (int a = 0; a <= d.M; ++a) {
        int rr, cc;
        long off;
        realified_shape(d, 1, a, &rr, &cc, &off);
        TnSeg seg{pr.Z + mm_block(a, d.L, d.C), d.wZ(), tbar + mm_block(a, d.L, d.C), d.wZ(), n};
        if ((r = run_tn(&seg, 1, rr, cc, gW2r + off, cc, acc, P, s))) return r;
      }
    }
    SO2_HIP(launch_gate_bwd(d, n, pr.U, Zbar, Ubar, s));
    ps.clear();
    lin1t_probs(d, Ubar, W1r, Tbar, n, 0, ps);
    if ((r = run_batch(ps, false, true, s))) return r;
    if (want_w1) {
      for (int a = 0; a <= d.M; ++a) {
        int rr, cc;
        long off;
        realified_shape(d, 0, a, &rr, &cc, &off);
        TnSeg seg{pr.T + mm_block(a, d.L, d.Ci()), d.wT(), Ubar + d.u_block(a), d.wU(), n};
        if ((r = run_tn(&seg, 1, rr, cc, gW1r + off, cc, acc, P, s))) return r;
      }
    }
    // N -> E transpose: gx (both halves), Sbar, position torques
    SO2_HIP(launch_node_bwd(d, gc, x, pos, pr.S, Tbar, gx, Sbar, tau2, tau3, acc, s));
    if (grbf) {
      ps.clear();
      ps.push_back(prob(Sbar, wS, w_rad, wS, grbf + (size_t)e0 * n_rbf, n_rbf, n, n_rbf, wS));
      if ((r = run_batch(ps, false, true, s))) return r;
    }
    if (gw_rad) {
      TnSeg seg{rbf + (size_t)e0 * n_rbf, n_rbf, Sbar, wS, n};
      if ((r = run_tn(&seg, 1, n_rbf, wS, gw_rad, wS, acc, P, s))) return r;
    }
    if (gpos || gedge) SO2_HIP(launch_vbar(gc, pos, tau1, tau2, tau3, vbar, s));
  }
  if (want_w2) SO2_HIP(launch_fold_grad(d, 1, gW2r, gw2, s));
  if (want_w1) SO2_HIP(launch_fold_grad(d, 0, gW1r, gw1, s));
  if (gpos) SO2_HIP(launch_node_pos(gd, vbar, gpos, s));
  return SO2_OK;
}

int so2conv_dbwd(const so2conv_cfg* cfg, const so2conv_graph* g, const float* x, const float* pos, const float* rbf,
                 const float* w_rad, const float* const* w1, const float* const* w2, const void* saved,
                 const float* gy, const float* px, const float* ppos, const float* pedge, const float* prbf,
                 const float* pw_rad, const float* const* pw1, const float* const* pw2, float* ggy, float* gx2,
                 float* gpos2, float* grbf2, float* gw_rad2, float* const* gw1_2, float* const* gw2_2, void* ws,
                 size_t ws_bytes, void* stream) {
  g_err.clear();
  Dims d;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &d)) || (r = check_graph(g, &gd))) return r;
  if ((r = check_weights(d, w_rad, w1, w2))) return r;
  if (!x || !pos || !gy || (!rbf && gd.E > 0)) return fail(SO2_EINVAL, "NULL input");
  if (gpos2) return fail(SO2_EUNSUPPORTED, "gpos2 (position second derivatives) is not provided; pass NULL");
  if ((r = ensure_init())) return r;
  const bool has_pw1 = !all_null(pw1, d.M + 1), has_pw2 = !all_null(pw2, d.M + 1);
  if (has_pw1)
    for (int a = 0; a <= d.M; ++a)
      if (!pw1[a]) return fail(SO2_EINVAL, "pw1 must be NULL or hold M+1 non-NULL blocks");
  if (has_pw2)
    for (int a = 0; a <= d.M; ++a)
      if (!pw2[a]) return fail(SO2_EINVAL, "pw2 must be NULL or hold M+1 non-NULL blocks");
  hipStream_t s = (hipStream_t)stream;
  const int n_rbf = cfg->n_rbf, wS = (d.L + 1) * d.Ci();
  if (gd.E == 0) {
    int rr = zero_grads(d, n_rbf, gd.N, gx2, nullptr, gw_rad2, gw1_2, gw2_2, s);
    if (rr) return rr;
    if (ggy) return fill(ggy, (size_t)gd.N * d.d() * d.C, s);
    return SO2_OK;
  }
  const bool recompute = saved == nullptr;
  if (!ws) return fail(SO2_EWORKSPACE, "workspace is NULL");
  const long ec = pick_chunk(d, n_rbf, gd.E, 2, recompute, ws_bytes);
  if (ec == 0) return fail(SO2_EWORKSPACE, "double-backward workspace too small for a 1024-edge chunk");
  const SavedLayout sl = saved_layout(d, n_rbf, gd.E);
  const char* st = static_cast<const char*>(saved);
  Arena ar{static_cast<char*>(ws), 0};
  float* W1r = ar.take(realified_size(d, 0));
  float* W2r = ar.take(realified_size(d, 1));
  float* pW1r = ar.take(realified_size(d, 0));
  float* pW2r = ar.take(realified_size(d, 1));
  float* gW1r = ar.take(realified_size(d, 0));
  float* gW2r = ar.take(realified_size(d, 1));
  float *S = nullptr, *T = nullptr, *U = nullptr, *Z = nullptr, *V = nullptr;
  if (recompute) {
    S = ar.take((size_t)ec * wS);
    T = ar.take((size_t)ec * d.wT());
    U = ar.take((size_t)ec * d.wU());
    Z = ar.take((size_t)ec * d.wZ());
    V = ar.take((size_t)ec * d.wZ());
  }
  float* Sdot = ar.take((size_t)ec * wS);
  float* Tdot = ar.take((size_t)ec * d.wT());
  float* omega = ar.take((size_t)ec * 3);
  float* Udot = ar.take((size_t)ec * d.wU());
  float* Zdot = ar.take((size_t)ec * d.wZ());
  float* Vdot = ar.take((size_t)ec * d.wZ());
  float* G2 = ar.take((size_t)2 * ec * d.wZ());
  float* ZZ = ar.take((size_t)2 * ec * d.wZ());
  float* UU = ar.take((size_t)2 * ec * d.wU());
  float* TT = ar.take((size_t)2 * ec * d.wT());
  float* Sbar = ar.take((size_t)ec * wS);
  float* Sdb = ar.take((size_t)ec * wS);
  float* P = ar.take(0);
  const bool want_w1 = !all_null(gw1_2, d.M + 1), want_w2 = !all_null(gw2_2, d.M + 1);

  SO2_HIP(launch_realify(d, 0, w1, W1r, s));
  SO2_HIP(launch_realify(d, 1, w2, W2r, s));
  if (has_pw1) SO2_HIP(launch_realify(d, 0, pw1, pW1r, s));
  if (has_pw2) SO2_HIP(launch_realify(d, 1, pw2, pW2r, s));
  for (long e0 = 0, c = 0; e0 < gd.E; e0 += ec, ++c) {
    GraphDev gc = gd;
    gc.e0 = e0;
    gc.e1 = e0 + ec < gd.E ? e0 + ec : gd.E;
    const int n = (int)(gc.e1 - gc.e0);
    const int acc = c > 0;
    const float* rbf_c = rbf + (size_t)e0 * n_rbf;
    const float* prbf_c = prbf ? prbf + (size_t)e0 * n_rbf : nullptr;
    Primal pr;
    if (recompute) {
      if ((r = forward_chunk(d, n_rbf, gc, x, pos, rbf, w_rad, W1r, W2r, S, T, U, Z, V, s))) return r;
      pr = {S, T, U, Z, V};
    } else {
      pr = {reinterpret_cast<const float*>(st + sl.S) + (size_t)e0 * wS,
            reinterpret_cast<const float*>(st + sl.T) + (size_t)e0 * d.wT(),
            reinterpret_cast<const float*>(st + sl.U) + (size_t)e0 * d.wU(),
            reinterpret_cast<const float*>(st + sl.Z) + (size_t)e0 * d.wZ(),
            reinterpret_cast<const float*>(st + sl.V) + (size_t)e0 * d.wZ()};
    }

    // ---- tangent (dual) forward along (px, ppos, pedge, prbf, pW)
    if (prbf_c) {
      if ((r = radial(d, n_rbf, n, prbf_c, w_rad, Sdot, s))) return r;
    } else if ((r = fill(Sdot, (size_t)n * wS, s))) {
      return r;
    }
    if (pw_rad) {
      if ((r = radial(d, n_rbf, n, rbf_c, pw_rad, Sdot, s, 1))) return r;
    }
    SO2_HIP(launch_edge_dual(d, gc, x, px, pos, ppos, pedge, pr.S, Sdot, Tdot, omega, s));
    std::vector<GemmProb> ps;
    lin1_probs(d, Tdot, W1r, Udot, n, 0, ps);
    if ((r = run_batch(ps, false, false, s))) return r;
    if (has_pw1) {
      ps.clear();
      lin1_probs(d, pr.T, pW1r, Udot, n, 1, ps);
      if ((r = run_batch(ps, false, false, s))) return r;
    }
    SO2_HIP(launch_gate_dual(d, n, pr.U, Udot, Zdot, s));
    ps.clear();
    lin2_probs(d, Zdot, W2r, Vdot, n, 0, ps);
    if ((r = run_batch(ps, false, false, s))) return r;
    if (has_pw2) {
      ps.clear();
      lin2_probs(d, pr.Z, pW2r, Vdot, n, 1, ps);
      if ((r = run_batch(ps, false, false, s))) return r;
    }
    // dL/dgy = the forward's directional derivative (Eq.(5))
    if (ggy) SO2_HIP(launch_node_dual(d, gc, pos, omega, pr.V, Vdot, ggy, acc, s));

    // ---- reverse of the tangent output with cotangent gy
    SO2_HIP(launch_edge_bwd_dual(d, gc, pos, omega, gy, G2, s));
    ps.clear();
    lin2t_probs(d, G2, W2r, ZZ, 2 * n, 0, ps);     // [Zdot_bar; Zbar]
    if ((r = run_batch(ps, false, true, s))) return r;
    if (has_pw2) {
      ps.clear();
      lin2t_probs(d, G2, pW2r, ZZ + (size_t)n * d.wZ(), n, 1, ps);   // Zbar += tbar pW2^T
      if ((r = run_batch(ps, false, true, s))) return r;
    }
    if (want_w2) {
      for (int a = 0; a <= d.M; ++a) {
        int rr, cc;
        long off;
        realified_shape(d, 1, a, &rr, &cc, &off);
        const int bo = mm_block(a, d.L, d.C);
        TnSeg segs[2] = {{Zdot + bo, d.wZ(), G2 + bo, d.wZ(), n},
                         {pr.Z + bo, d.wZ(), G2 + (size_t)n * d.wZ() + bo, d.wZ(), n}};
        if ((r = run_tn(segs, 2, rr, cc, gW2r + off, cc, acc, P, s))) return r;
      }
    }
    SO2_HIP(launch_gate_dbwd(d, n, pr.U, Udot, ZZ, UU, s));   // [Udot_bar; Ubar]
    ps.clear();
    lin1t_probs(d, UU, W1r, TT, 2 * n, 0, ps);      // [Tdot_bar; Tbar]
    if ((r = run_batch(ps, false, true, s))) return r;
    if (has_pw1) {
      ps.clear();
      lin1t_probs(d, UU, pW1r, TT + (size_t)n * d.wT(), n, 1, ps);   // Tbar += Udot_bar pW1^T
      if ((r = run_batch(ps, false, true, s))) return r;
    }
    if (want_w1) {
      for (int a = 0; a <= d.M; ++a) {
        int rr, cc;
        long off;
        realified_shape(d, 0, a, &rr, &cc, &off);
        const int ao = mm_block(a, d.L, d.Ci()), uo = d.u_block(a);
        TnSeg segs[2] = {{Tdot + ao, d.wT(), UU + uo, d.wU(), n},
                         {pr.T + ao, d.wT(), UU + (size_t)n * d.wU() + uo, d.wU(), n}};
        if ((r = run_tn(segs, 2, rr, cc, gW1r + off, cc, acc, P, s))) return r;
      }
    }
    SO2_HIP(launch_node_bwd_dual(d, gc, x, px, pos, omega, pr.S, Sdot, TT, gx2, Sbar, Sdb, acc, s));
    if (grbf2) {
      float* out = grbf2 + (size_t)e0 * n_rbf;
      ps.clear();
      ps.push_back(prob(Sbar, wS, w_rad, wS, out, n_rbf, n, n_rbf, wS));
      if ((r = run_batch(ps, false, true, s))) return r;
      if (pw_rad) {
        ps.clear();
        ps.push_back(prob(Sdb, wS, pw_rad, wS, out, n_rbf, n, n_rbf, wS, 1));
        if ((r = run_batch(ps, false, true, s))) return r;
      }
    }
    if (gw_rad2) {
      TnSeg segs[2] = {{rbf_c, n_rbf, Sbar, wS, n}, {prbf_c, n_rbf, Sdb, wS, prbf_c ? n : 0}};
      if ((r = run_tn(segs, 2, n_rbf, wS, gw_rad2, wS, acc, P, s))) return r;
    }
  }
  if (want_w2) SO2_HIP(launch_fold_grad(d, 1, gW2r, gw2_2, s));
  if (want_w1) SO2_HIP(launch_fold_grad(d, 0, gW1r, gw1_2, s));
  return SO2_OK;
}

}  // extern "C"
