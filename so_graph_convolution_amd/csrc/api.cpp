// C ABI of the fused SO(2) convolution: argument checks, workspace layout and
// the kernel schedules of the forward, backward and double backward.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/so2conv.h"
#include "api_common.hpp"
#include "gemm.hpp"
#include "ops.hpp"
#include "so3_gen.hpp"
#include "wigner.hpp"

namespace so2 {
int upload_generators_fwd(const float* host);
int upload_generators_bwd(const float* host);
int upload_generators_dual(const float* host);
}  // namespace so2

using namespace so2;

namespace so2 {

namespace {
thread_local std::string g_err;
}  // namespace

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}
void clear_error() { g_err.clear(); }
const char* last_error() { return g_err.c_str(); }
int set_error(int code, const std::string& msg) { return fail(code, msg); }

}  // namespace so2

namespace {

// ---------------------------------------------------------------- generators
// The so(3) generator table is evaluated at compile time (so3_gen.hpp, dual
// numbers through the Wigner recursion), so the copy uploaded here for the
// cooperative rotation-rate tables and the literals inside the kernels are
// the same floats on every host.
constexpr GenTable kGenHost = make_gen_table();

// the kernels apply the generators through two candidate orders per row and
// per column (gen_cand); a table entry outside them would be dropped
bool generators_sparse(const float* table) {
  for (int k = 0; k < 3; ++k)
    for (int l = 1; l <= kMaxL; ++l) {
      const int n = 2 * l + 1;
      const float* G = table + k * kGenSize + gen_off(l);
      for (int i = -l; i <= l; ++i)
        for (int c = -l; c <= l; ++c) {
          if (G[(i + l) * n + c + l] == 0.f) continue;
          int a0, a1, b0, b1;
          gen_cand(k, i, &a0, &a1);   // row i
          gen_cand(k, c, &b0, &b1);   // column c
          if ((c != a0 && c != a1) || (i != b0 && i != b1)) return false;
        }
    }
  return true;
}

std::mutex g_init_mu;
bool g_init_done[64];

int ensure_init() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SO2_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(SO2_EUNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_init_mu);
  if (g_init_done[dev]) return SO2_OK;
  const float* table = kGenHost.v;
  if (!generators_sparse(table))
    return fail(SO2_EUNSUPPORTED, "so(3) generator table outside the two-candidate pattern the kernels use");
  SO2_HIP(upload_generators_fwd(table));
  SO2_HIP(upload_generators_bwd(table));
  SO2_HIP(upload_generators_dual(table));
  g_init_done[dev] = true;
  return SO2_OK;
}

// ---------------------------------------------------------------- checks
// Configuration of one call: sizes and the storage type of the boundary arrays
// and of the per-edge GEMM operands.
struct Ctx {
  Dims d;
  int n_rbf;
  int bf;    // 1: bfloat16 boundary arrays and GEMM operands
  int es;    // bytes per GEMM-operand element
  int debug; // SO2_DEBUG_CHECKS
  int split = 0; // float32 products through bfloat16 pieces (float32 calls without SO2_F32_NATIVE)
  int fused_gate = 0; // SO2_FUSED_GATE
  int ns = 1; // weight sets: one per system (the plain operator has one)
  int nk = 0; // experts of a mixture (0: plain operator)
  int ng = 0; // spherical-grid activation: grid points, and the caller's tables (degree-major rows)
  const float* gG = nullptr;
  const float* gP = nullptr;
  size_t node_floats() const { return (size_t)d.d() * d.C; }   // one node row
  int wS() const { return (d.L + 1) * d.Ci(); }
};

int check_cfg(const so2conv_cfg* cfg, Ctx* c) {
  if (!cfg) return fail(SO2_EINVAL, "cfg is NULL");
  const int L = cfg->lmax, M = cfg->mmax, C = cfg->channels;
  if (L < 0 || L > kMaxL) return fail(SO2_EUNSUPPORTED, "lmax must be in [0, 6]");
  if (M < 0 || M > L) return fail(SO2_EINVAL, "mmax must be in [0, lmax]");
  if (!lm_supported(L, M)) return fail(SO2_EUNSUPPORTED, "(lmax, mmax) pair has no compiled kernels");
  if (C < 16 || C > 256 || C % 16) return fail(SO2_EUNSUPPORTED, "channels must be a multiple of 16 in [16, 256]");
  if (cfg->n_rbf < 4 || cfg->n_rbf % 4 || cfg->n_rbf > 1024)
    return fail(SO2_EUNSUPPORTED, "n_rbf must be a multiple of 4 in [4, 1024]");
  if (cfg->dtype != SO2_F32 && cfg->dtype != SO2_BF16) return fail(SO2_EUNSUPPORTED, "dtype must be SO2_F32 or SO2_BF16");
  if (cfg->flags & ~(SO2_DEBUG_CHECKS | SO2_F32_NATIVE | SO2_FUSED_GATE)) return fail(SO2_EINVAL, "unknown cfg flags");
  const int H = cfg->heads == 0 ? 1 : cfg->heads;
  if (H < 1 || H > kMaxHeads || C % H) return fail(SO2_EUNSUPPORTED, "heads must divide channels, at most 16");
  if (H > 1 && (C / H) % 64 && C / H != 16 && C / H != 32)
    return fail(SO2_EUNSUPPORTED, "channels per head must be 16, 32 or a multiple of 64");
  c->debug = (cfg->flags & SO2_DEBUG_CHECKS) != 0;
  c->d.L = L;
  c->d.M = M;
  c->d.C = C;
  c->d.H = H;
  c->n_rbf = cfg->n_rbf;
  c->bf = cfg->dtype == SO2_BF16;
  c->es = c->bf ? 2 : 4;
  c->split = !c->bf && !(cfg->flags & SO2_F32_NATIVE);
  c->fused_gate = (cfg->flags & SO2_FUSED_GATE) != 0;
  if (cfg->act != SO2_ACT_GATE && cfg->act != SO2_ACT_SWIGLU_S2) return fail(SO2_EINVAL, "unknown activation");
  c->d.s2 = cfg->act == SO2_ACT_SWIGLU_S2;
  if (c->d.s2) {
    if (c->d.q() > 32) return fail(SO2_EUNSUPPORTED, "the grid activation takes at most 32 retained rows");
    if (cfg->n_grid < 1 || cfg->n_grid > 256) return fail(SO2_EUNSUPPORTED, "n_grid must be in [1, 256]");
    c->ng = cfg->n_grid;
    c->gG = cfg->grid_basis;
    c->gP = cfg->grid_proj;
  }
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

// ---------------------------------------------------------------- debug checks
// Word of failed checks of this device (bits as in so2conv_debug_status).
__device__ unsigned g_debug_word;

__global__ void validate_kernel(GraphDev g, const float* __restrict__ pos, const float* __restrict__ rbf, int n_rbf,
                                const float* __restrict__ env, int heads) {
  unsigned bits = 0;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < g.E; e += (long)gridDim.x * blockDim.x) {
    const int j = g.src[e], i = g.dst[e];
    const bool jr = j >= 0 && j < g.N, ir = i >= 0 && i < g.N;
    if (!jr) bits |= 1u;
    if (!ir) bits |= 2u;
    if (e > 0 && g.dst[e - 1] > i) bits |= 4u;
    if (jr && ir) {
      float r2 = 0.f;
      bool fin = true;
      for (int k = 0; k < 3; ++k) {
        const float v = pos[3 * j + k] - pos[3 * i + k] + (g.shift ? g.shift[3 * e + k] : 0.f);
        fin = fin && isfinite(v);
        r2 += v * v;
      }
      if (!fin) bits |= 16u;
      else if (!(r2 > 0.f)) bits |= 8u;
    }
    for (int k = 0; k < n_rbf; ++k)
      if (!isfinite(rbf[(size_t)e * n_rbf + k])) bits |= 16u;
    if (env)
      for (int h = 0; h < heads; ++h)
        if (!isfinite(env[e * heads + h])) bits |= 16u;
  }
  if (bits) atomicOr(&g_debug_word, bits);
}

std::string debug_bits_text(unsigned b) {
  std::string m;
  const char* names[] = {"src out of range", "dst out of range", "dst decreasing", "zero-length edge",
                         "non-finite input"};
  for (int k = 0; k < 5; ++k)
    if (b & (1u << k)) m += (m.empty() ? "" : ", ") + std::string(names[k]);
  return m;
}

// SO2_DEBUG_CHECKS: validate, wait for the verdict, and refuse to compute on bad inputs
int debug_validate(const Ctx& c, const GraphDev& g, const float* pos, const float* rbf, const float* env,
                   hipStream_t s) {
  if (!c.debug) return SO2_OK;
  const unsigned zero = 0;
  SO2_HIP(hipStreamSynchronize(s));
  SO2_HIP(hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &zero, sizeof(zero)));
  if (g.E > 0) {
    long b = (g.E + 255) / 256;
    if (b > 4096) b = 4096;
    hipLaunchKernelGGL(validate_kernel, dim3((unsigned)b), dim3(256), 0, s, g, pos, rbf, c.n_rbf, env, c.d.H);
    SO2_HIP(hipGetLastError());
  }
  SO2_HIP(hipStreamSynchronize(s));
  unsigned w = 0;
  SO2_HIP(hipMemcpyFromSymbol(&w, HIP_SYMBOL(g_debug_word), sizeof(w)));
  if (w) return fail(SO2_EDEVICE, "device-side validation failed: " + debug_bits_text(w));
  return SO2_OK;
}

// ---------------------------------------------------------------- layouts

struct SavedLayout {
  size_t S, T, U, Z, V, total;
};
SavedLayout saved_layout(const Ctx& c, long E) {
  const Dims& d = c.d;
  SavedLayout s;
  size_t o = 0;
  const size_t e = (size_t)E;
  s.S = o; o += al(sizeof(float) * e * c.wS());
  s.T = o; o += al((size_t)c.es * e * d.wT());
  s.U = o; o += al(sizeof(float) * e * d.wU());
  s.Z = o; o += al((size_t)c.es * e * d.wZ());
  s.V = o; o += al(sizeof(float) * e * d.wZ());
  s.total = o;
  return s;
}

// State the backward can keep for the double backward with the same inputs
// and gy: the cotangents Zbar [E, wZ] (float32), Ubar [E, wU] (operand type)
// and Tbar [E, wT] (float32). They equal the cotangents of the tangent chain
// (Zdot_bar, Udot_bar, Tdot_bar) that the double backward's reverse pass
// would otherwise form with one more data-gradient product per linear.
struct BwdSavedLayout {
  size_t Z, U, T, total;
};
BwdSavedLayout bwd_saved_layout(const Ctx& c, long E) {
  const Dims& d = c.d;
  BwdSavedLayout s;
  size_t o = 0;
  const size_t e = (size_t)E;
  s.Z = o; o += al(sizeof(float) * e * d.wZ());
  s.U = o; o += al((size_t)c.es * e * d.wU());
  s.T = o; o += al(sizeof(float) * e * d.wT());
  s.total = o;
  return s;
}
struct BwdRows {
  float* Z;
  void* U;
  float* T;
};
BwdRows bwd_rows(const Ctx& c, const void* sb, long E, long e0) {
  const BwdSavedLayout L = bwd_saved_layout(c, E);
  char* b = static_cast<char*>(const_cast<void*>(sb));
  return {reinterpret_cast<float*>(b + L.Z) + (size_t)e0 * c.d.wZ(), b + L.U + (size_t)c.es * e0 * c.d.wU(),
          reinterpret_cast<float*>(b + L.T) + (size_t)e0 * c.d.wT()};
}

}  // namespace

// K chunk of split-K weight-gradient products over edges (a multiple of the
// GEMM K tile). With `small` (the rows of one system), rows that 4096-row
// chunks would cut into fewer than 32 splits are cut into chunks of 512 to
// 2048 rows, halving until there are 32 splits or the chunk is 512 rows: a
// handful of long splits leaves most CUs idle (measured on MI355X at 17,880
// edges, lmax 4, C 128). The splits of K <= K' rows then stay within
// max(ceil(K' / 4096), min(64, ceil(K' / 512))), which take_partials sizes for.
void so2::split_plan(long K, int* splits, int* chunk, bool small) {
  long c = 4096;
  if (small)
    while (c > 512 && (K + c - 1) / c < 32) c /= 2;
  long s = (K + c - 1) / c;
  if (s > 256) {
    c = ((K + 255) / 256 + kGemmKTile - 1) / kGemmKTile * kGemmKTile;
    s = (K + c - 1) / c;
  }
  if (s < 1) s = 1;
  *splits = (int)s;
  *chunk = (int)c;
}

namespace {

// realified weights of one linear as GEMM B operands: W [rows][cols] and, for
// bfloat16, its transpose (the forward product A.W runs as A.(W^T)^T)
struct Lin {
  const void* W;
  const void* WT;
  const float* U[kMaxL + 1];   // float32: user-layout blocks [k][2h] of orders >= 1 (complex products)
};
struct LinBuf {
  void* W;
  void* WT;
};
LinBuf take_lin(Arena& ar, const Ctx& c, int second) {
  const size_t n = (size_t)realified_size(c.d, second);
  LinBuf b;
  b.W = ar.bytes(n * c.es);
  if (c.bf) {
    b.WT = ar.bytes(n * c.es);
  } else {   // float32: the transposed order-0 block (the data-gradient products read it k-major)
    int r, cc;
    long off;
    realified_shape(c.d, second, 0, &r, &cc, &off);
    b.WT = ar.bytes((size_t)r * cc * sizeof(float));
  }
  return b;
}

std::vector<LinBuf> take_lins(Arena& ar, const Ctx& c, int second) {
  std::vector<LinBuf> v(c.ns);
  for (auto& b : v) b = take_lin(ar, c, second);
  return v;
}
std::vector<float*> take_grads(Arena& ar, const Ctx& c, int second) {
  std::vector<float*> v(c.ns);
  for (auto& g : v) g = ar.take(realified_size(c.d, second));
  return v;
}

// user-layout block a of linear `second`: [k][cols] (a = 0) or [k][2h] (a >= 1)
long user_block(const Dims& d, int second, int a) {
  int r, cc;
  long off;
  realified_shape(d, second, a, &r, &cc, &off);
  return (long)(a ? r / 2 : r) * cc;
}
long user_size(const Dims& d, int second) {
  long n = 0;
  for (int a = 0; a <= d.M; ++a) n += user_block(d, second, a);
  return n;
}
long max_user_block(const Dims& d) {
  long n = 0;
  for (int second = 0; second < 2; ++second)
    for (int a = 0; a <= d.M; ++a) n = std::max(n, user_block(d, second, a));
  return n;
}

// K chunk of the coefficient-gradient products (K = a user block's size)
constexpr long kCoefChunk = 4096;
static_assert(kCoefChunk % kGemmKTile == 0, "coefficient split chunks must be whole K tiles");

// Mixture of linear experts: merged weights of every system per linear
// (block-major: block a holds [S][user_block] at S * (offset of a)), the
// merged weight directions of the double backward, float32 staging of one
// expert block (bfloat16 experts or expert gradients), and the split-K
// partials of the coefficient gradients.
struct MixWs {
  float* merged[2];    // merged weights of each linear; at the end, the per-system gradients
  float* pmerged[2];   // double backward: merged directions; at the end, the first-order gradients
  float *we32, *gwe32, *P;
};
void take_mix(Arena& ar, const Ctx& c, int stage, MixWs* m) {
  *m = MixWs{};
  if (!c.nk) return;
  const size_t mb = (size_t)max_user_block(c.d);
  for (int second = 0; second < 2; ++second) {
    m->merged[second] = ar.take((size_t)c.ns * user_size(c.d, second));
    m->pmerged[second] = stage == 2 ? ar.take((size_t)c.ns * user_size(c.d, second)) : nullptr;
  }
  m->we32 = c.bf ? ar.take((size_t)c.nk * mb) : nullptr;
  m->gwe32 = c.bf && stage > 0 ? ar.take((size_t)c.nk * mb) : nullptr;
  m->P = stage > 0 ? ar.take((size_t)((mb + kCoefChunk - 1) / kCoefChunk) * c.ns * c.nk) : nullptr;
}

// largest weight-gradient block (floats): realified blocks and the radial matrix
size_t max_grad_block(const Ctx& c) {
  size_t mx = (size_t)c.n_rbf * c.wS();
  for (int second = 0; second < 2; ++second)
    for (int a = 0; a <= c.d.M; ++a) {
      int r, cc;
      long off;
      realified_shape(c.d, second, a, &r, &cc, &off);
      if ((size_t)r * cc > mx) mx = (size_t)r * cc;
    }
  return mx;
}

// split-K partials of one order's weight-gradient launch: nseg segments of up
// to ec rows, cut at system borders (each system's rows split on their own,
// at most ceil(rows / 4096) + 1 splits each; the rows of one system, K <= ec,
// at most max(ceil(ec / 4096), min(64, ceil(ec / 512))): chunks of fewer than
// 4096 rows leave under 64 splits, and no chunk is below 512 rows)
float* take_partials(Arena& ar, const Ctx& c, long ec, int nseg) {
  int sp, ch;
  const bool small = c.ns <= 1;
  split_plan(ec, &sp, &ch, small);
  const long fine = small ? std::min<long>(64, (ec + 511) / 512) : 0;
  const long bound = std::max<long>(std::max<long>(sp, (ec + 4095) / 4096), fine) + 1 + (c.ns > 1 ? c.ns : 0);
  return ar.take((size_t)nseg * bound * max_grad_block(c));
}

struct Primal {
  const float* S;
  const void* T;
  const float* U;
  const void* Z;
  const float* V;
};
struct PrimalBuf {
  float* S;
  void* T;
  float* U;
  void* Z;
  float* V;
};
PrimalBuf take_primal(Arena& ar, const Ctx& c, long ec) {
  const Dims& d = c.d;
  const size_t e = (size_t)ec;
  PrimalBuf p;
  p.S = ar.take(e * c.wS());
  p.T = ar.bytes(e * d.wT() * c.es);
  p.U = ar.take(e * d.wU());
  p.Z = ar.bytes(e * d.wZ() * c.es);
  p.V = ar.take(e * d.wZ());
  return p;
}
Primal saved_rows(const Ctx& c, const void* saved, long E, long e0) {
  const SavedLayout sl = saved_layout(c, E);
  const char* st = static_cast<const char*>(saved);
  const Dims& d = c.d;
  return {reinterpret_cast<const float*>(st + sl.S) + (size_t)e0 * c.wS(),
          st + sl.T + (size_t)e0 * d.wT() * c.es,
          reinterpret_cast<const float*>(st + sl.U) + (size_t)e0 * d.wU(),
          st + sl.Z + (size_t)e0 * d.wZ() * c.es,
          reinterpret_cast<const float*>(st + sl.V) + (size_t)e0 * d.wZ()};
}

// m-major grid tables of the spherical-grid activation (NULL with the gate)
float* take_s2(Arena& ar, const Ctx& c) { return c.d.s2 ? ar.take(2 * (size_t)c.ng * c.d.q()) : nullptr; }

struct FwdWs {
  std::vector<LinBuf> W1, W2;
  MixWs mix;
  float *w_rad32, *x32, *y32, *s2t;
  PrimalBuf pr;
};
void layout_fwd(Arena& ar, const Ctx& c, int N, long ec, bool recompute, FwdWs* w) {
  w->s2t = take_s2(ar, c);
  w->W1 = take_lins(ar, c, 0);
  w->W2 = take_lins(ar, c, 1);
  take_mix(ar, c, 0, &w->mix);
  w->w_rad32 = c.bf ? ar.take((size_t)c.n_rbf * c.wS()) : nullptr;
  w->x32 = c.bf ? ar.take((size_t)N * c.node_floats()) : nullptr;
  w->y32 = c.bf ? ar.take((size_t)N * c.node_floats()) : nullptr;
  w->pr = recompute ? take_primal(ar, c, ec) : PrimalBuf{};
}

struct BwdWs {
  std::vector<LinBuf> W1, W2;
  std::vector<float*> gW1r, gW2r;
  MixWs mix;
  float* vbar_all;
  float *w_rad32, *x32, *gy32, *gx32, *gw_rad32, *s2t;
  PrimalBuf pr;
  void *tbar, *Ubar;
  float *Zbar, *Tbar, *Sbar, *tau1, *tau2, *tau3, *P;
};
void layout_bwd(Arena& ar, const Ctx& c, int N, long E, long ec, bool recompute, BwdWs* w) {
  const Dims& d = c.d;
  const size_t e = (size_t)ec;
  w->s2t = take_s2(ar, c);
  w->W1 = take_lins(ar, c, 0);
  w->W2 = take_lins(ar, c, 1);
  w->gW1r = take_grads(ar, c, 0);
  w->gW2r = take_grads(ar, c, 1);
  take_mix(ar, c, 1, &w->mix);
  w->vbar_all = ar.take((size_t)E * 3);
  w->w_rad32 = c.bf ? ar.take((size_t)c.n_rbf * c.wS()) : nullptr;
  w->x32 = c.bf ? ar.take((size_t)N * c.node_floats()) : nullptr;
  w->gy32 = c.bf ? ar.take((size_t)N * c.node_floats()) : nullptr;
  w->gx32 = c.bf ? ar.take((size_t)N * c.node_floats()) : nullptr;
  w->gw_rad32 = c.bf ? ar.take((size_t)c.n_rbf * c.wS()) : nullptr;
  w->pr = recompute ? take_primal(ar, c, ec) : PrimalBuf{};
  w->tbar = ar.bytes(e * d.wZ() * c.es);
  w->Zbar = ar.take(e * d.wZ());
  w->Ubar = ar.bytes(e * d.wU() * c.es);
  w->Tbar = ar.take(e * d.wT());
  w->Sbar = ar.take(e * c.wS());
  w->tau1 = ar.take(e * 3);
  w->tau2 = ar.take(e * 3);
  w->tau3 = ar.take(e * 3);
  w->P = take_partials(ar, c, ec, 1);
}

struct DbwdWs {
  std::vector<LinBuf> W1, W2, pW1, pW2;
  std::vector<float*> gW1r, gW2r, gW1f, gW2f;   // gW*f: first-order weight gradients (mixture directions)
  MixWs mix;
  float *vbar2_all, *p2e, *p2d, *p2s;
  float *w_rad32, *pw_rad32, *x32, *px32, *gy32, *ggy32, *gx2_32, *gw_rad2_32, *s2t;
  PrimalBuf pr;
  void *Tdot, *Zdot, *G2, *UU;
  float *Sdot, *omega, *Udot, *Vdot, *ZZ, *TT, *Sbar, *Sdb, *P;
};
void layout_dbwd(Arena& ar, const Ctx& c, int N, long E, long ec, bool recompute, DbwdWs* w) {
  const Dims& d = c.d;
  const size_t e = (size_t)ec;
  w->s2t = take_s2(ar, c);
  w->W1 = take_lins(ar, c, 0);
  w->W2 = take_lins(ar, c, 1);
  w->pW1 = take_lins(ar, c, 0);
  w->pW2 = take_lins(ar, c, 1);
  w->gW1r = take_grads(ar, c, 0);
  w->gW2r = take_grads(ar, c, 1);
  if (c.nk) {
    w->gW1f = take_grads(ar, c, 0);
    w->gW2f = take_grads(ar, c, 1);
  }
  take_mix(ar, c, 2, &w->mix);
  w->vbar2_all = ar.take((size_t)E * 3);      // position derivative per edge vector (all edges)
  w->p2e = ar.take(e * 6);
  w->p2d = ar.take(e * 6);
  w->p2s = ar.take(e * 6);
  const size_t nf = (size_t)N * c.node_floats(), rf = (size_t)c.n_rbf * c.wS();
  w->w_rad32 = c.bf ? ar.take(rf) : nullptr;
  w->pw_rad32 = c.bf ? ar.take(rf) : nullptr;
  w->gw_rad2_32 = c.bf ? ar.take(rf) : nullptr;
  w->x32 = c.bf ? ar.take(nf) : nullptr;
  w->px32 = c.bf ? ar.take(nf) : nullptr;
  w->gy32 = c.bf ? ar.take(nf) : nullptr;
  w->ggy32 = c.bf ? ar.take(nf) : nullptr;
  w->gx2_32 = c.bf ? ar.take(nf) : nullptr;
  w->pr = recompute ? take_primal(ar, c, ec) : PrimalBuf{};
  w->Sdot = ar.take(e * c.wS());
  w->Tdot = ar.bytes(e * d.wT() * c.es);
  w->omega = ar.take(e * 3);
  w->Udot = ar.take(e * d.wU());
  w->Zdot = ar.bytes(e * d.wZ() * c.es);
  w->Vdot = ar.take(e * d.wZ());
  w->G2 = ar.bytes(2 * e * d.wZ() * c.es);
  w->ZZ = ar.take(2 * e * d.wZ());
  w->UU = ar.bytes(2 * e * d.wU() * c.es);
  w->TT = ar.take(2 * e * d.wT());
  w->Sbar = ar.take(e * c.wS());
  w->Sdb = ar.take(e * c.wS());
  w->P = take_partials(ar, c, ec, 2);
}

// Workspace of one stage for a chunk of `ec` edges out of E.
//   stage 0: forward; 1: backward; 2: double backward.
//   recompute: the per-edge forward state lives in the workspace (saved == NULL).
size_t ws_need(const Ctx& c, int N, long E, long ec, int stage, bool recompute) {
  Arena ar{nullptr, 0};
  if (stage == 0) {
    FwdWs w;
    layout_fwd(ar, c, N, ec, recompute, &w);
  } else if (stage == 1) {
    BwdWs w;
    layout_bwd(ar, c, N, E, ec, recompute, &w);
  } else {
    DbwdWs w;
    layout_dbwd(ar, c, N, E, ec, recompute, &w);
  }
  return ar.used + 4096;
}

// edges per chunk that fit in ws_bytes (E if everything fits; 0 if not even 1024 edges do)
long pick_chunk(const Ctx& c, int N, long E, int stage, bool recompute, size_t ws_bytes) {
  if (E == 0) return 0;
  if (ws_need(c, N, E, E, stage, recompute) <= ws_bytes) return E;
  long lo = 0, hi = E;
  while (hi - lo > 1024) {
    const long mid = (lo + hi) / 2 / 1024 * 1024;
    if (mid <= lo) break;
    if (ws_need(c, N, E, mid, stage, recompute) <= ws_bytes) lo = mid;
    else hi = mid;
  }
  if (lo == 0 && ws_need(c, N, E, 1024 < E ? 1024 : E, stage, recompute) <= ws_bytes) lo = 1024 < E ? 1024 : E;
  return lo;
}

// ---------------------------------------------------------------- gemm helpers
}  // namespace

GemmProb so2::prob(const void* A, int lda, const void* B, int ldb, float* C, int ldc, int M, int N, int K, int acc) {
  GemmProb p{};
  p.A = A; p.B = B; p.C = C;
  p.M = M; p.N = N; p.K = K;
  p.lda = lda; p.ldb = ldb; p.ldc = ldc;
  p.k_splits = 1; p.k_chunk = K; p.accumulate = acc;
  return p;
}

namespace {

const void* offs(const void* p, size_t elems, int es) { return static_cast<const char*>(p) + elems * es; }
void* offs(void* p, size_t elems, int es) { return static_cast<char*>(p) + elems * es; }

// ---------------------------------------------------------------- GEMM timing
// When enabled, every MFMA GEMM launch is bracketed by HIP events on the
// launching stream and its algorithmic flop count (2 M N K summed over the
// launch's problems) is recorded; so2conv_profile_read reports the totals.
struct ProfRec {
  int kind;          // 0 NN, 1 NT, 2 TN (float32); 3 NT, 4 TN (bfloat16); 5 NN, 6 NT, 7 TN (complex float32);
                     // 8 NN, 9 NT, 10 TN (float32 through bfloat16 pieces, kSplitProducts MFMA products each)
  double flops;
  double bytes;      // algorithmic: A, B read once, C (or the split partials) written once
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

constexpr int kSplitProducts = 6;   // bf16 piece products per float32 product of the split GEMMs

}  // namespace

int so2::run_batch(std::vector<GemmProb>& ps, bool TA, bool TB, int op, hipStream_t s, const GateCols* gate) {
  if (ps.empty()) return SO2_OK;
  const bool bf = op == kOpBF16;
  const double es = bf ? 2.0 : 4.0;
  size_t i = 0;
  while (i < ps.size()) {
    GemmBatch b{};
    b.nprob = 0;
    if (gate) {
      b.gC = gate->C;
      b.gL = gate->L;
      b.ldz = gate->ldz;
      b.ldgam = gate->ldgam;
    }
    double flops = 0, bytes = 0;
    while (i < ps.size() && b.nprob < kGemmMaxProbs) {
      const GemmProb& q = ps[i];
      const double f = q.cplx ? 2.0 : 1.0;   // complex: both halves of A and B, real and imaginary C
      flops += (q.cplx ? 3.0 : 1.0) * 2.0 * q.M * (double)q.N * q.K;
      bytes += es * f * ((double)q.M * q.K + (double)q.K * q.N) +
               4.0 * f * (double)q.M * q.N * (q.partial ? q.k_splits : 1) * (q.accumulate ? 2 : 1);
      b.p[b.nprob++] = ps[i++];
    }
    bool split = false;
    auto launch = [&]() -> int {
      if (op == kOpSplit) {
        const int e = gemm_x3_run(b, TA, TB, kSplitProducts, s);
        if (e != hipErrorNotSupported) {
          split = true;
          return e;
        }
      }
      if (bf && !TA && TB) {   // bfloat16 A.B^T: the direct-to-LDS kernel where its layout takes the operands
        const int e = gemm_b16_run(b, s);
        if (e != hipErrorNotSupported) return e;
      }
      if (bf && TA && !TB) {   // bfloat16 A^T.B (weight gradients): register-staged transposed tiles
        const int e = gemm_b16t_run(b, s);
        if (e != hipErrorNotSupported) return e;
      }
      return gemm_run(b, TA, TB, bf, s);   // hipErrorNotSupported for gated problems
    };
    if (g_prof_on) {
      ProfRec r{0, flops, bytes, nullptr, nullptr};
      SO2_HIP(hipEventCreate(&r.a));
      SO2_HIP(hipEventCreate(&r.b));
      SO2_HIP(hipEventRecord(r.a, s));
      const int e = launch();
      if (gate && e == hipErrorNotSupported) {   // nothing ran: the caller takes the ungated products
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
        return kNoFusedGate;
      }
      SO2_HIP(e);
      SO2_HIP(hipEventRecord(r.b, s));
      r.kind = split ? (TA ? 10 : (TB ? 9 : 8))
                     : (ps[0].cplx ? (TA ? 7 : (TB ? 6 : 5)) : (bf ? (TA ? 4 : 3) : (TA ? 2 : (TB ? 1 : 0))));
      std::lock_guard<std::mutex> lk(g_prof_mu);
      g_prof.push_back(r);
    } else {
      const int e = launch();
      if (gate && e == hipErrorNotSupported) return kNoFusedGate;
      SO2_HIP(e);
    }
  }
  return SO2_OK;
}

int so2::run_tn(const TnSeg* segs, int nseg, int M, int N, float* G, int ldg, int accumulate, float* P, int bf,
                hipStream_t s) {
  std::vector<GemmProb> ps;
  int total_splits = 0;
  // a thin side of at most 64 (the radial map's n_rbf rows) becomes the
  // product's columns: the partials then hold G^T and the reduction
  // writes G back transposed
  const bool swap = M <= 64 && N > M && !bf;
  for (int q = 0; q < nseg; ++q) {
    if (segs[q].K <= 0) continue;
    int sp, ch;
    split_plan(segs[q].K, &sp, &ch);
    float* Pq = P + (size_t)total_splits * M * N;
    GemmProb p = swap ? prob(segs[q].B, segs[q].ldb, segs[q].A, segs[q].lda, Pq, M, N, M, (int)segs[q].K)
                      : prob(segs[q].A, segs[q].lda, segs[q].B, segs[q].ldb, Pq, N, M, N, (int)segs[q].K);
    p.k_splits = sp;
    p.k_chunk = ch;
    p.partial = 1;
    total_splits += p.k_splits;
    ps.push_back(p);
  }
  if (total_splits == 0) return SO2_OK;
  int r = run_batch(ps, true, false, bf, s);
  if (r) return r;
  SO2_HIP(swap ? gemm_reduce(P, total_splits, N, M, G, ldg, accumulate, s, 1)
               : gemm_reduce(P, total_splits, M, N, G, ldg, accumulate, s));
  return SO2_OK;
}

namespace {
__global__ void fill_kernel(float* p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void fill16_kernel(unsigned short* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}
}  // namespace

int so2::fill(float* p, size_t n, hipStream_t s) {
  if (n == 0) return SO2_OK;
  size_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)b), dim3(256), 0, s, p, n, 0.f);
  SO2_HIP(hipGetLastError());
  return SO2_OK;
}

namespace {
// zero n elements of the boundary type
int zero(const Ctx& c, void* p, size_t n, hipStream_t s) {
  if (!c.bf) return fill(static_cast<float*>(p), n, s);
  if (n == 0) return SO2_OK;
  size_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  hipLaunchKernelGGL(fill16_kernel, dim3((unsigned)b), dim3(256), 0, s, static_cast<unsigned short*>(p), n);
  SO2_HIP(hipGetLastError());
  return SO2_OK;
}

// float32 view of a boundary input: itself, or its conversion into `tmp`
int f32_in(const Ctx& c, const void* in, float* tmp, size_t n, const float** out, hipStream_t s) {
  if (!in) {
    *out = nullptr;
    return SO2_OK;
  }
  if (!c.bf) {
    *out = static_cast<const float*>(in);
    return SO2_OK;
  }
  SO2_HIP(launch_to_f32(static_cast<const bf16s*>(in), tmp, n, s));
  *out = tmp;
  return SO2_OK;
}
// float32 accumulator of a boundary output: itself, or `tmp` (copied back by f32_out)
float* f32_acc(const Ctx& c, void* out, float* tmp) {
  if (!out) return nullptr;
  return c.bf ? tmp : static_cast<float*>(out);
}
int f32_out(const Ctx& c, const float* tmp, void* out, size_t n, hipStream_t s) {
  if (!out || !c.bf) return SO2_OK;
  SO2_HIP(launch_to_bf16(tmp, static_cast<bf16s*>(out), n, s));
  return SO2_OK;
}

// S = rbf W_rad (float32)
int radial(const Ctx& c, long E, const float* rbf, const float* w_rad, float* S, hipStream_t s, int acc = 0) {
  std::vector<GemmProb> ps{prob(rbf, c.n_rbf, w_rad, c.wS(), S, c.wS(), (int)E, c.wS(), c.n_rbf, acc)};
  return run_batch(ps, false, false, 0, s);
}

// Weights of one linear per system: edges [e[s], e[s+1]) use W[s] (the plain
// operator is one system holding every edge).
struct WSet {
  std::vector<long> e;
  std::vector<Lin> W;
};
// user-layout blocks: the caller's arrays (one system) or each system's
// merged blocks (`merged`, block-major, see sys_blocks)
void sys_blocks(const Ctx& c, int second, float* merged, int sy, void** bp);
WSet wset(const Ctx& c, int second, const std::vector<long>& e, const std::vector<LinBuf>& b,
          const void* const* user, float* merged) {
  WSet w{e, {}};
  for (size_t sy = 0; sy < b.size(); ++sy) {
    Lin l{b[sy].W, b[sy].WT, {}};
    void* bp[kMaxL + 1] = {};
    if (merged) sys_blocks(c, second, merged, (int)sy, bp);
    for (int a = 0; a <= c.d.M; ++a)
      l.U[a] = static_cast<const float*>(merged ? bp[a] : (user ? user[a] : nullptr));
    w.W.push_back(l);
  }
  return w;
}

// complex product of order a >= 1 (float32): see GemmProb
GemmProb prob_cx(const void* A, int lda, int dA, const void* B, int ldb, int dB, float* C, int ldc, int M, int N,
                 int K, float sA, float sB, int acc = 0) {
  GemmProb p = prob(A, lda, B, ldb, C, ldc, M, N, K, acc);
  p.cplx = 1;
  p.dA = dA;
  p.dB = dB;
  p.sA = sA;
  p.sB = sB;
  return p;
}

// Per-order products of linear `second` (0: first, 1: second) over the chunk
// of n edges starting at edge e0, one problem per (system, order):
//   forward   : C[:, out block a] (+)= A[:, in block a]  W_a
//   transposed: C[:, in block a]  (+)= A[:, out block a] W_a^T
// In-blocks: T (first, width wT) or Z (second, width wZ); out-blocks: U (first,
// width wU) or V (second, width wZ). A is an operand buffer, C float32;
// `stacks` copies of the chunk's rows follow each other in A and C (the
// double backward's stacked 2n-row products).
int run_lin(const Ctx& c, int second, bool transposed, const void* A, float* C, const WSet& w, long e0, int n,
            int stacks, int acc, hipStream_t s) {
  const Dims& d = c.d;
  const int win = second ? d.wZ() : d.wT(), wout = second ? d.wZ() : d.wU();
  const int lda = transposed ? wout : win, ldc = transposed ? win : wout;
  std::vector<GemmProb> ps, pc;   // order-0 products; products of orders >= 1 (float32)
  const int op = c.bf ? kOpBF16 : (c.split ? kOpSplit : kOpF32);
  // float32 data-gradient products of order 0 read the transposed weight copy
  bool use_wt = !c.bf && transposed;
  for (const Lin& l : w.W) use_wt = use_wt && l.WT != nullptr;
  for (int q = 0; q < stacks; ++q)
    for (size_t sy = 0; sy < w.W.size(); ++sy) {
      const long lo = std::max(w.e[sy], e0), hi = std::min(w.e[sy + 1], e0 + n);
      if (hi <= lo) continue;
      const long r0 = (long)q * n + (lo - e0);
      const int rows = (int)(hi - lo);
      const Lin& W = w.W[sy];
      const void* Ar = offs(A, (size_t)r0 * lda, c.es);
      float* Cr = C + (size_t)r0 * ldc;
      for (int a = 0; a <= d.M; ++a) {
        int r, cc;
        long off;
        realified_shape(d, second, a, &r, &cc, &off);
        const long ib = mm_block(a, d.L, second ? d.C : d.Ci());
        const long ob = second ? mm_block(a, d.L, d.C) : d.u_block(a);
        if (a > 0 && c.split) {
          // realified: [T+ T-] W_a forward, [U+ U-] W_a^T transposed (W_a [r][cc] row-major)
          if (!transposed)
            pc.push_back(prob(offs(Ar, ib, c.es), win, offs(W.W, off, c.es), cc, Cr + ob, wout, rows, cc, r, acc));
          else
            pc.push_back(prob(offs(Ar, ob, c.es), wout, offs(W.W, off, c.es), cc, Cr + ib, win, rows, r, cc, acc));
          continue;
        }
        if (a > 0 && !c.bf) {
          // (T+ + i T-)(W0 + i W1) forward; (U+ + i U-)(W0 - i W1)^T transposed
          const int k = r / 2, h = cc / 2;
          if (!transposed)
            pc.push_back(prob_cx(offs(Ar, ib, c.es), win, k, W.U[a], cc, h, Cr + ob, wout, rows, h, k, 1.f, 1.f, acc));
          else
            pc.push_back(prob_cx(offs(Ar, ob, c.es), wout, h, W.U[a], cc, h, Cr + ib, win, rows, k, h, 1.f, -1.f, acc));
          continue;
        }
        if (!transposed) {
          if (c.bf)
            ps.push_back(prob(offs(Ar, ib, c.es), win, offs(W.WT, off, c.es), r, Cr + ob, wout, rows, cc, r, acc));
          else
            ps.push_back(prob(offs(Ar, ib, c.es), win, offs(W.W, off, c.es), cc, Cr + ob, wout, rows, cc, r, acc));
        } else if (use_wt) {
          // float32 order 0: A (W^T) with the transposed copy, its rows k-major
          ps.push_back(prob(offs(Ar, ob, c.es), wout, offs(W.WT, off, c.es), r, Cr + ib, win, rows, r, cc, acc));
        } else {
          ps.push_back(prob(offs(Ar, ob, c.es), wout, offs(W.W, off, c.es), cc, Cr + ib, win, rows, r, cc, acc));
        }
      }
    }
  int rr = run_batch(ps, false, (transposed && !use_wt) || c.bf, op, s);
  if (rr) return rr;
  return run_batch(pc, false, transposed, op, s);
}

// The first linear's forward over the chunk of n edges at e0 with the gate in
// the products' epilogue (SO2_FUSED_GATE): the gate columns of order 0 first,
// then every other product of the first linear writes its output U and the
// gated Z together (degree 0: SiLU(u); degree l >= 1: sigmoid(gamma_l) u,
// gamma_l read from the row's gate columns). Runs on the float32 path through
// bfloat16 pieces and on bfloat16 calls; kNoFusedGate without the flag or
// where those kernels do not take the operands (the caller then runs the
// products and the gate kernel).
int run_lin_gated(const Ctx& c, const void* A, float* U, void* Z, const WSet& w, long e0, int n, hipStream_t s) {
  const Dims& d = c.d;
  if (!c.fused_gate || d.s2 || !(c.split || c.bf)) return kNoFusedGate;
  const int win = d.wT(), wout = d.wU(), wz = d.wZ(), L = d.L, C = d.C;
  const int op = c.bf ? kOpBF16 : kOpSplit;
  std::vector<GemmProb> pg, pu;   // gate columns; gated products
  for (size_t sy = 0; sy < w.W.size(); ++sy) {
    const long lo = std::max(w.e[sy], e0), hi = std::min(w.e[sy + 1], e0 + n);
    if (hi <= lo) continue;
    const long r0 = lo - e0;
    const int rows = (int)(hi - lo);
    const Lin& W = w.W[sy];
    const void* Ar = offs(A, (size_t)r0 * win, c.es);
    float* Ur = U + (size_t)r0 * wout;
    void* Zr = offs(Z, (size_t)r0 * wz, c.es);
    for (int a = 0; a <= d.M; ++a) {
      int r, cc;
      long off;
      realified_shape(d, 0, a, &r, &cc, &off);
      const long ib = mm_block(a, L, d.Ci()), ob = d.u_block(a);
      const int nu = a == 0 ? (L + 1) * C : cc;   // the block's gated columns
      // weights as B: W [r][cc] (float32, A.B) or its transpose [cc][r] (bfloat16, A.B^T)
      auto wcols = [&](long col) { return c.bf ? offs(W.WT, off + col * r, c.es) : offs(W.W, off + col, c.es); };
      const int ldb = c.bf ? r : cc;
      if (a == 0 && L > 0)
        pg.push_back(prob(offs(Ar, ib, c.es), win, wcols((long)(L + 1) * C), ldb, Ur + (L + 1) * C, wout, rows, L * C, r));
      GemmProb q = prob(offs(Ar, ib, c.es), win, wcols(0), ldb, Ur + ob, wout, rows, nu, r);
      q.gate = a + 1;
      q.Z = offs(Zr, mm_block(a, L, C), c.es);
      q.gam = Ur + (L + 1) * C;
      pu.push_back(q);
    }
  }
  int rr;
  if ((rr = run_batch(pg, false, c.bf, op, s))) return rr;
  const GateCols gcols{C, L, wz, wout};
  return run_batch(pu, false, c.bf, op, s, &gcols);
}

// weight gradient of linear `second` per system (realified, float32) over the
// chunk of n edges at e0: G[s]_a (+)= sum_q In_q[:, in a]^T Out_q[:, out a] on
// the system's rows. One launch per order covers every system (each split
// over its own rows into its own partials), then one fixed-order reduction
// per system. A system's first chunk overwrites its gradient unless `zeroed`
// (then every chunk accumulates into gradients cleared beforehand).
int run_lin_grad(const Ctx& c, int second, const void* const* in, const void* const* out, int nseg, int n,
                 const WSet& w, long e0, const std::vector<float*>& G, bool zeroed, float* P, hipStream_t s) {
  const Dims& d = c.d;
  const int win = second ? d.wZ() : d.wT(), wout = second ? d.wZ() : d.wU();
  struct Red {
    size_t sy, poff;
    int splits, acc;
  };
  for (int a = 0; a <= d.M; ++a) {
    int r, cc;
    long off;
    realified_shape(d, second, a, &r, &cc, &off);
    const long ib = mm_block(a, d.L, second ? d.C : d.Ci());
    const long ob = second ? mm_block(a, d.L, d.C) : d.u_block(a);
    const bool cx = a > 0 && !c.bf && !c.split;   // float32 complex products into the user layout
    std::vector<GemmProb> ps;
    std::vector<Red> red;
    size_t poff = 0;
    for (size_t sy = 0; sy < w.W.size(); ++sy) {
      const long lo = std::max(w.e[sy], e0), hi = std::min(w.e[sy + 1], e0 + n);
      if (hi <= lo) continue;
      Red rd{sy, poff, 0, zeroed || lo != w.e[sy]};
      for (int q = 0; q < nseg; ++q) {
        int sp, ch;
        split_plan(hi - lo, &sp, &ch, c.ns <= 1);
        const void* Aq = offs(in[q], (size_t)(lo - e0) * win + ib, c.es);
        const void* Bq = offs(out[q], (size_t)(lo - e0) * wout + ob, c.es);
        // float32, orders >= 1: (T+ - i T-)^T (Ubar+ + i Ubar-) straight into the user layout [k][2h]
        GemmProb p = cx ? prob_cx(Aq, win, r / 2, Bq, wout, cc / 2, P + poff, cc, r / 2, cc / 2, (int)(hi - lo),
                                  -1.f, 1.f)
                        : prob(Aq, win, Bq, wout, P + poff, cc, r, cc, (int)(hi - lo));
        p.k_splits = sp;
        p.k_chunk = ch;
        p.partial = 1;
        ps.push_back(p);
        poff += (size_t)sp * (cx ? r / 2 : r) * cc;
        rd.splits += sp;
      }
      red.push_back(rd);
    }
    if (ps.empty()) continue;
    int rr = run_batch(ps, true, false, c.bf ? kOpBF16 : (c.split ? kOpSplit : kOpF32), s);
    if (rr) return rr;
    for (const Red& rd : red)
      SO2_HIP(gemm_reduce(P + rd.poff, rd.splits, cx ? r / 2 : r, cc, G[rd.sy] + off, cc, rd.acc, s));
  }
  return SO2_OK;
}

bool all_null(const void* const* p, int n) {
  if (!p) return true;
  for (int i = 0; i < n; ++i)
    if (p[i]) return false;
  return true;
}

int check_weights(const Dims& d, const void* w_rad, const void* const* w1, const void* const* w2) {
  if (!w_rad) return fail(SO2_EINVAL, "w_rad is NULL");
  if (!w1 || !w2) return fail(SO2_EINVAL, "weight pointer arrays are NULL");
  for (int a = 0; a <= d.M; ++a)
    if (!w1[a] || !w2[a]) return fail(SO2_EINVAL, "a weight block pointer is NULL");
  return SO2_OK;
}

int realify(const Ctx& c, int second, const void* const* w, const LinBuf& b, hipStream_t s) {
  SO2_HIP(launch_realify(c.d, second, w, b.W, b.WT, c.bf, s));
  return SO2_OK;
}

// ---------------------------------------------------------------- mixture of linear experts
// System-dependent mixture (TrimSO(2) page, Appendix C.1: UMA's edge
// projections use system-dependent mixtures of linear experts; Table 2: 64
// experts): system s uses W(s) = sum_k coef[s][k] W^(k) for both linears and
// every order. Experts are stacked per order block as [K][user block].
struct MixIn {
  std::vector<long> e;   // S+1 edge offsets of the systems
  const float* coef;     // [S][K], device, float32
};

// merged (+)= coef . We for every order block of linear `second`: [S][K] x [K][block]
int mix_linear(const Ctx& c, int second, const void* const* we, const float* coef, float* merged, float* we32,
               int acc, hipStream_t s) {
  long off = 0;
  for (int a = 0; a <= c.d.M; ++a) {
    const long pm = user_block(c.d, second, a);
    const float* w32;
    int r;
    if ((r = f32_in(c, we[a], we32, (size_t)c.nk * pm, &w32, s))) return r;
    std::vector<GemmProb> ps{
        prob(coef, c.nk, w32, (int)pm, merged + (size_t)c.ns * off, (int)pm, c.ns, (int)pm, c.nk, acc)};
    if ((r = run_batch(ps, false, false, 0, s))) return r;
    off += pm;
  }
  return SO2_OK;
}

// block pointers of system sy inside a block-major merged buffer
void sys_blocks(const Ctx& c, int second, float* merged, int sy, void** bp) {
  long off = 0;
  for (int a = 0; a <= c.d.M; ++a) {
    const long pm = user_block(c.d, second, a);
    bp[a] = merged + (size_t)c.ns * off + (size_t)sy * pm;
    off += pm;
  }
}

int realify_systems(const Ctx& c, int second, float* merged, const std::vector<LinBuf>& b, hipStream_t s) {
  for (int sy = 0; sy < c.ns; ++sy) {
    void* bp[kMaxL + 1];
    sys_blocks(c, second, merged, sy, bp);
    SO2_HIP(launch_realify(c.d, second, bp, b[sy].W, b[sy].WT, c.bf, s, 1));
  }
  return SO2_OK;
}

// every system's realified gradient of linear `second` folded into a
// block-major merged buffer (float32, user layout)
int fold_systems(const Ctx& c, int second, const std::vector<float*>& G, float* merged, hipStream_t s) {
  for (int sy = 0; sy < c.ns; ++sy) {
    void* bp[kMaxL + 1];
    sys_blocks(c, second, merged, sy, bp);
    SO2_HIP(launch_fold_grad(c.d, second, G[sy], bp, 0, s, !c.bf && !c.split));
  }
  return SO2_OK;
}

// C (+)= A B^T, A [M][K], B [N][K] (float32), split over K with a fixed-order reduction
int nt_split(const float* A, int lda, const float* B, int ldb, float* C, int ldc, int M, int N, long K, int acc,
             float* P, hipStream_t s) {
  const int sp = (int)((K + kCoefChunk - 1) / kCoefChunk);
  GemmProb p = prob(A, lda, B, ldb, P, N, M, N, (int)K);
  p.k_splits = sp;
  p.k_chunk = (int)kCoefChunk;
  p.partial = 1;
  std::vector<GemmProb> ps{p};
  int r = run_batch(ps, false, true, 0, s);
  if (r) return r;
  SO2_HIP(gemm_reduce(P, sp, M, N, C, ldc, acc, s));
  return SO2_OK;
}

// Expert and coefficient gradients of linear `second` from the per-system
// gradients Gm (block-major, float32), for every order block a:
//   gwe[a]  = coefA^T Gm[a] (+ coefB^T Gm2[a])             [K][S] x [S][block]
//   gcoef  (+)= Gm[a] WeA[a]^T (+ Gm2[a] WeB[a]^T)         [S][block] x [block][K]
// The second terms (the double backward's directions on coef and experts)
// are skipped where their operands are null. gcoef accumulates from the
// first product on when gcoef_acc.
int mix_grads(const Ctx& c, int second, const float* Gm, const float* coefA, const void* const* WeA, const float* Gm2,
              const float* coefB, const void* const* WeB, void* const* gwe, float* gcoef, bool gcoef_acc,
              const MixWs& mw, hipStream_t s) {
  long off = 0;
  int r;
  bool cacc = gcoef_acc;
  for (int a = 0; a <= c.d.M; ++a) {
    const long pm = user_block(c.d, second, a);
    const float* GA = Gm + (size_t)c.ns * off;
    const float* GB = Gm2 ? Gm2 + (size_t)c.ns * off : nullptr;
    if (gcoef) {
      const float* w32;
      if ((r = f32_in(c, WeA[a], mw.we32, (size_t)c.nk * pm, &w32, s))) return r;
      if ((r = nt_split(GA, (int)pm, w32, (int)pm, gcoef, c.nk, c.ns, c.nk, pm, cacc, mw.P, s))) return r;
      cacc = true;
      if (GB && WeB && WeB[a]) {
        if ((r = f32_in(c, WeB[a], mw.we32, (size_t)c.nk * pm, &w32, s))) return r;
        if ((r = nt_split(GB, (int)pm, w32, (int)pm, gcoef, c.nk, c.ns, c.nk, pm, 1, mw.P, s))) return r;
      }
    }
    if (gwe && gwe[a]) {
      float* out = c.bf ? mw.gwe32 : static_cast<float*>(gwe[a]);
      std::vector<GemmProb> p1{prob(coefA, c.nk, GA, (int)pm, out, (int)pm, c.nk, (int)pm, c.ns)};
      if ((r = run_batch(p1, true, false, 0, s))) return r;
      if (GB && coefB) {   // accumulates onto the first product: its own launch, after it
        std::vector<GemmProb> p2{prob(coefB, c.nk, GB, (int)pm, out, (int)pm, c.nk, (int)pm, c.ns, 1)};
        if ((r = run_batch(p2, true, false, 0, s))) return r;
      }
      if (c.bf) SO2_HIP(launch_to_bf16(out, static_cast<bf16s*>(gwe[a]), (size_t)c.nk * pm, s));
    }
    off += pm;
  }
  return SO2_OK;
}

// realified weights of both linears per system: the user's (plain operator)
// or the merged mixture
int prepare_weights(const Ctx& c, const MixIn* mx, const void* const* w1, const void* const* w2,
                    const std::vector<LinBuf>& B1, const std::vector<LinBuf>& B2, const MixWs& mw, hipStream_t s) {
  int r;
  if (!mx) {
    if ((r = realify(c, 0, w1, B1[0], s)) || (r = realify(c, 1, w2, B2[0], s))) return r;
    return SO2_OK;
  }
  if ((r = mix_linear(c, 0, w1, mx->coef, mw.merged[0], mw.we32, 0, s))) return r;
  if ((r = realify_systems(c, 0, mw.merged[0], B1, s))) return r;
  if ((r = mix_linear(c, 1, w2, mx->coef, mw.merged[1], mw.we32, 0, s))) return r;
  return realify_systems(c, 1, mw.merged[1], B2, s);
}

std::vector<long> sys_edges(const MixIn* mx, long E) { return mx ? mx->e : std::vector<long>{0, E}; }

int zero_sets(const std::vector<float*>& G, size_t n, hipStream_t s) {
  for (float* g : G) {
    int r = fill(g, n, s);
    if (r) return r;
  }
  return SO2_OK;
}

// ---------------------------------------------------------------- Edge -> Edge activation
int check_act(const Ctx& c) {
  if (c.d.s2 && (!c.gG || !c.gP)) return fail(SO2_EINVAL, "grid_basis or grid_proj is NULL");
  return SO2_OK;
}
// The gate, or the spherical-grid SwiGLU with the call's m-major grid tables
// G [ng][q], P [q][ng] (copied from the caller's degree-major tables into the
// workspace once per call). Inputs U, Udot, Zbar... float32; outputs of the
// operand type.
struct ActTab {
  const float* G = nullptr;
  const float* P = nullptr;
};
int act_tables(const Ctx& c, float* s2t, ActTab* t, hipStream_t s) {
  if (!c.d.s2) return SO2_OK;
  float* Gm = s2t;
  float* Pm = s2t + (size_t)c.ng * c.d.q();
  SO2_HIP(launch_s2_mmajor(c.d.L, c.d.M, c.ng, c.gG, c.gP, Gm, Pm, s));
  t->G = Gm;
  t->P = Pm;
  return SO2_OK;
}
// Z = A(U)
int act_fwd(const Ctx& c, const ActTab& t, long n, const float* U, void* Z, hipStream_t s) {
  if (c.d.s2) SO2_HIP(launch_s2_fwd(n, c.d.q(), c.d.C, c.ng, U, t.G, t.P, Z, c.bf, s));
  else SO2_HIP(launch_gate_fwd(c.d, n, U, Z, c.bf, s));
  return SO2_OK;
}
// Ubar = J(U)^T Zbar
int act_bwd(const Ctx& c, const ActTab& t, long n, const float* U, const float* Zbar, void* Ubar, hipStream_t s) {
  if (c.d.s2) SO2_HIP(launch_s2_bwd(n, c.d.q(), c.d.C, c.ng, U, t.G, t.P, Zbar, Ubar, c.bf, s));
  else SO2_HIP(launch_gate_bwd(c.d, n, U, Zbar, Ubar, c.bf, s));
  return SO2_OK;
}
// Zdot = J(U) Udot
int act_dual(const Ctx& c, const ActTab& t, long n, const float* U, const float* Udot, void* Zdot, hipStream_t s) {
  if (c.d.s2)
    SO2_HIP(launch_s2_dbwd(n, c.d.q(), c.d.C, c.ng, U, t.G, t.P, nullptr, Udot, Zdot, nullptr, c.bf, s));
  else
    SO2_HIP(launch_gate_dual(c.d, n, U, Udot, Zdot, c.bf, s));
  return SO2_OK;
}
// reverse of the tangent chain: Ub = J^T Zb + d/dU <Zdb, J Udot>; Udb = J^T Zdb (may be NULL)
int act_dbwd(const Ctx& c, const ActTab& t, long n, const float* U, const float* Udot, const float* Zdb,
             const float* Zb, void* Udb, void* Ub, hipStream_t s) {
  if (c.d.s2)
    SO2_HIP(launch_s2_rev(n, c.d.q(), c.d.C, c.ng, U, t.G, t.P, Udot, Zdb, Zb, Udb, Ub, c.bf, s));
  else
    SO2_HIP(launch_gate_dbwd(c.d, n, U, Udot, Zdb, Zb, Udb, Ub, c.bf, s));
  return SO2_OK;
}

// forward state of the chunk [g.e0, g.e1) into (S, T, U, Z, V)
int forward_chunk(const Ctx& c, const ActTab& at, const GraphDev& g, const float* x, const float* pos,
                  const float* rbf, const float* w_rad, const WSet& W1, const WSet& W2, const PrimalBuf& p,
                  hipStream_t s) {
  const int ec = (int)(g.e1 - g.e0);
  int r;
  if ((r = radial(c, ec, rbf + (size_t)g.e0 * c.n_rbf, w_rad, p.S, s))) return r;
  SO2_HIP(launch_edge_fwd(c.d, g, x, pos, p.S, p.T, c.bf, s));
  r = run_lin_gated(c, p.T, p.U, p.Z, W1, g.e0, ec, s);   // the gate in the first linear's epilogue
  if (r == kNoFusedGate) {
    if ((r = run_lin(c, 0, false, p.T, p.U, W1, g.e0, ec, 1, 0, s))) return r;
    r = act_fwd(c, at, ec, p.U, p.Z, s);
  }
  if (r) return r;
  return run_lin(c, 1, false, p.Z, p.V, W2, g.e0, ec, 1, 0, s);
}

int zero_grads(const Ctx& c, int N, void* gx, float* gpos, void* gw_rad, void* const* gw1, void* const* gw2,
               hipStream_t s) {
  int r;
  const Dims& d = c.d;
  if (gx && (r = zero(c, gx, (size_t)N * c.node_floats(), s))) return r;
  if (gpos && (r = fill(gpos, (size_t)N * 3, s))) return r;
  if (gw_rad && (r = zero(c, gw_rad, (size_t)c.n_rbf * c.wS(), s))) return r;
  for (int a = 0; a <= d.M; ++a) {
    int rr, cc;
    long off;
    realified_shape(d, 0, a, &rr, &cc, &off);
    if (gw1 && gw1[a] && (r = zero(c, gw1[a], (size_t)(a ? rr / 2 : rr) * cc, s))) return r;
    realified_shape(d, 1, a, &rr, &cc, &off);
    if (gw2 && gw2[a] && (r = zero(c, gw2[a], (size_t)(a ? rr / 2 : rr) * cc, s))) return r;
  }
  return SO2_OK;
}

// forward of the plain operator (mx == NULL) or of the mixture of experts
// (w1, w2: expert stacks)
int conv_fwd(const Ctx& c, const GraphDev& gd, const MixIn* mx, const void* x, const float* pos, const float* rbf,
             const float* env, const void* w_rad, const void* const* w1, const void* const* w2, void* y, void* saved,
             void* ws, size_t ws_bytes, void* stream) {
  int r;
  const Dims& d = c.d;
  if ((r = check_weights(d, w_rad, w1, w2)) || (r = check_act(c))) return r;
  if (!x || !pos || (!rbf && gd.E > 0) || !y) return fail(SO2_EINVAL, "NULL input or output");
  if ((r = ensure_init())) return r;
  if ((r = debug_validate(c, gd, pos, rbf, env, (hipStream_t)stream))) return r;
  const bool recompute = saved == nullptr;
  if (!ws) return fail(SO2_EWORKSPACE, "workspace is NULL");
  const long ec = pick_chunk(c, gd.N, gd.E, 0, recompute, ws_bytes);
  if (gd.E > 0 && ec == 0) return fail(SO2_EWORKSPACE, "forward workspace too small for a 1024-edge chunk");
  if (ws_bytes < ws_need(c, gd.N, gd.E, 0, 0, recompute)) return fail(SO2_EWORKSPACE, "forward workspace too small");
  hipStream_t s = (hipStream_t)stream;
  Arena ar{static_cast<char*>(ws), 0};
  FwdWs w;
  layout_fwd(ar, c, gd.N, ec, recompute, &w);
  const size_t nf = (size_t)gd.N * c.node_floats();
  const float *x32, *wr32;
  if ((r = f32_in(c, x, w.x32, nf, &x32, s))) return r;
  if ((r = f32_in(c, w_rad, w.w_rad32, (size_t)c.n_rbf * c.wS(), &wr32, s))) return r;
  float* y32 = f32_acc(c, y, w.y32);
  if ((r = prepare_weights(c, mx, w1, w2, w.W1, w.W2, w.mix, s))) return r;
  ActTab at;
  if ((r = act_tables(c, w.s2t, &at, s))) return r;
  const std::vector<long> se = sys_edges(mx, gd.E);
  const WSet W1 = wset(c, 0, se, w.W1, w1, w.mix.merged[0]), W2 = wset(c, 1, se, w.W2, w2, w.mix.merged[1]);
  if (gd.E == 0) {
    GraphDev gc = gd;
    gc.e0 = gc.e1 = 0;
    SO2_HIP(launch_node_fwd(d, gc, pos, nullptr, nullptr, y32, 0, s));
    return f32_out(c, y32, y, nf, s);
  }
  for (long e0 = 0, k = 0; e0 < gd.E; e0 += ec, ++k) {
    GraphDev gc = gd;
    gc.e0 = e0;
    gc.e1 = e0 + ec < gd.E ? e0 + ec : gd.E;
    PrimalBuf p = w.pr;
    if (!recompute) {
      const SavedLayout sl = saved_layout(c, gd.E);
      char* st = static_cast<char*>(saved);
      p.S = reinterpret_cast<float*>(st + sl.S) + (size_t)e0 * c.wS();
      p.T = st + sl.T + (size_t)e0 * d.wT() * c.es;
      p.U = reinterpret_cast<float*>(st + sl.U) + (size_t)e0 * d.wU();
      p.Z = st + sl.Z + (size_t)e0 * d.wZ() * c.es;
      p.V = reinterpret_cast<float*>(st + sl.V) + (size_t)e0 * d.wZ();
    }
    if ((r = forward_chunk(c, at, gc, x32, pos, rbf, wr32, W1, W2, p, s))) return r;
    SO2_HIP(launch_node_fwd(d, gc, pos, p.V, env, y32, k > 0, s));
  }
  return f32_out(c, y32, y, nf, s);
}

// backward of the plain operator (mx == NULL) or of the mixture (w1, w2,
// gw1, gw2: expert stacks; gcoef: coefficient gradient)
int conv_bwd(const Ctx& c, const GraphDev& gd, const MixIn* mx, const void* x, const float* pos, const float* rbf,
             const float* env, const void* w_rad, const void* const* w1, const void* const* w2, const void* saved,
             const void* gy, void* gx, float* gpos, float* grbf, float* genv, void* gw_rad, void* const* gw1,
             void* const* gw2, float* gcoef, float* gedge, void* saved_bwd, void* ws, size_t ws_bytes, void* stream) {
  int r;
  const Dims& d = c.d;
  if ((r = check_weights(d, w_rad, w1, w2)) || (r = check_act(c))) return r;
  if (!x || !pos || !gy || (!rbf && gd.E > 0)) return fail(SO2_EINVAL, "NULL input");
  if (genv && !env) return fail(SO2_EINVAL, "genv requested without an envelope");
  if ((r = ensure_init())) return r;
  if ((r = debug_validate(c, gd, pos, rbf, env, (hipStream_t)stream))) return r;
  hipStream_t s = (hipStream_t)stream;
  const int n_rbf = c.n_rbf, wS = c.wS();
  if (gd.E == 0 && !mx) return zero_grads(c, gd.N, gx, gpos, gw_rad, gw1, gw2, s);
  const bool recompute = saved == nullptr;
  if (!ws) return fail(SO2_EWORKSPACE, "workspace is NULL");
  const long ec = pick_chunk(c, gd.N, gd.E, 1, recompute, ws_bytes);
  if (ec == 0) return fail(SO2_EWORKSPACE, "backward workspace too small for a 1024-edge chunk");
  Arena ar{static_cast<char*>(ws), 0};
  BwdWs w;
  layout_bwd(ar, c, gd.N, gd.E, ec, recompute, &w);
  const size_t nf = (size_t)gd.N * c.node_floats();
  const float *x32, *gy32, *wr32;
  if ((r = f32_in(c, x, w.x32, nf, &x32, s))) return r;
  if ((r = f32_in(c, gy, w.gy32, nf, &gy32, s))) return r;
  if ((r = f32_in(c, w_rad, w.w_rad32, (size_t)n_rbf * wS, &wr32, s))) return r;
  float* gx_acc = f32_acc(c, gx, w.gx32);
  float* gwr_acc = f32_acc(c, gw_rad, w.gw_rad32);
  float* vbar = gedge ? gedge : w.vbar_all;
  const bool want_w1 = !all_null(gw1, d.M + 1) || gcoef, want_w2 = !all_null(gw2, d.M + 1) || gcoef;
  if ((r = prepare_weights(c, mx, w1, w2, w.W1, w.W2, w.mix, s))) return r;
  ActTab at;
  if ((r = act_tables(c, w.s2t, &at, s))) return r;
  const std::vector<long> se = sys_edges(mx, gd.E);
  const WSet W1 = wset(c, 0, se, w.W1, w1, w.mix.merged[0]), W2 = wset(c, 1, se, w.W2, w2, w.mix.merged[1]);
  if (mx && want_w1 && (r = zero_sets(w.gW1r, realified_size(d, 0), s))) return r;
  if (mx && want_w2 && (r = zero_sets(w.gW2r, realified_size(d, 1), s))) return r;
  for (long e0 = 0, k = 0; e0 < gd.E; e0 += ec, ++k) {
    GraphDev gc = gd;
    gc.e0 = e0;
    gc.e1 = e0 + ec < gd.E ? e0 + ec : gd.E;
    const int n = (int)(gc.e1 - gc.e0);
    const int acc = k > 0;
    Primal pr;
    if (recompute) {
      if ((r = forward_chunk(c, at, gc, x32, pos, rbf, wr32, W1, W2, w.pr, s))) return r;
      pr = {w.pr.S, w.pr.T, w.pr.U, w.pr.Z, w.pr.V};
    } else {
      pr = saved_rows(c, saved, gd.E, e0);
    }
    // the cotangents go to the caller's saved state when it keeps them
    const BwdRows cb = saved_bwd ? bwd_rows(c, saved_bwd, gd.E, e0) : BwdRows{w.Zbar, w.Ubar, w.Tbar};
    // E -> N transpose: tbar = R gy[dst], tau1 = rotation torque of <V, R gy>
    SO2_HIP(launch_edge_bwd(d, gc, pos, gy32, pr.V, env, w.tbar, w.tau1, genv, c.bf, s));
    if ((r = run_lin(c, 1, true, w.tbar, cb.Z, W2, e0, n, 1, 0, s))) return r;
    if (want_w2) {
      const void* in[1] = {pr.Z};
      const void* out[1] = {w.tbar};
      if ((r = run_lin_grad(c, 1, in, out, 1, n, W2, e0, w.gW2r, mx != nullptr, w.P, s))) return r;
    }
    if ((r = act_bwd(c, at, n, pr.U, cb.Z, cb.U, s))) return r;
    if ((r = run_lin(c, 0, true, cb.U, cb.T, W1, e0, n, 1, 0, s))) return r;
    if (want_w1) {
      const void* in[1] = {pr.T};
      const void* out[1] = {cb.U};
      if ((r = run_lin_grad(c, 0, in, out, 1, n, W1, e0, w.gW1r, mx != nullptr, w.P, s))) return r;
    }
    // N -> E transpose: gx (both halves), Sbar, position torques
    SO2_HIP(launch_node_bwd(d, gc, x32, pos, pr.S, cb.T, gx_acc, w.Sbar, w.tau2, w.tau3, acc, s));
    if (grbf) {
      std::vector<GemmProb> ps{prob(w.Sbar, wS, wr32, wS, grbf + (size_t)e0 * n_rbf, n_rbf, n, n_rbf, wS)};
      if ((r = run_batch(ps, false, true, 0, s))) return r;
    }
    if (gwr_acc) {
      TnSeg seg{rbf + (size_t)e0 * n_rbf, n_rbf, w.Sbar, wS, n};
      if ((r = run_tn(&seg, 1, n_rbf, wS, gwr_acc, wS, acc, w.P, 0, s))) return r;
    }
    if (gpos || gedge) SO2_HIP(launch_vbar(gc, pos, w.tau1, w.tau2, w.tau3, vbar, d.s2, s));
  }
  if (!mx) {
    if (want_w2) SO2_HIP(launch_fold_grad(d, 1, w.gW2r[0], gw2, c.bf, s, !c.bf && !c.split));
    if (want_w1) SO2_HIP(launch_fold_grad(d, 0, w.gW1r[0], gw1, c.bf, s, !c.bf && !c.split));
  } else {
    for (int second = 0; second < 2; ++second) {
      if (!(second ? want_w2 : want_w1)) continue;
      float* gm = w.mix.merged[second];   // the merged weights are no longer needed
      if ((r = fold_systems(c, second, second ? w.gW2r : w.gW1r, gm, s))) return r;
      if ((r = mix_grads(c, second, gm, mx->coef, second ? w2 : w1, nullptr, nullptr, nullptr, second ? gw2 : gw1,
                         gcoef, second == 1 && want_w1, w.mix, s)))
        return r;
    }
  }
  if (gpos) SO2_HIP(launch_node_pos(gd, vbar, gpos, s));
  if ((r = f32_out(c, gx_acc, gx, nf, s))) return r;
  return f32_out(c, gwr_acc, gw_rad, (size_t)n_rbf * wS, s);
}

// double backward of the plain operator (mx == NULL) or of the mixture
// (w1, w2, pw1, pw2, gw1_2, gw2_2: expert stacks; pcoef: direction on the
// coefficients; gcoef2: their derivative)
int conv_dbwd(const Ctx& c, const GraphDev& gd, const MixIn* mx, const void* x, const float* pos, const float* rbf,
              const float* env, const void* w_rad, const void* const* w1, const void* const* w2, const void* saved,
              const void* gy, const void* px, const float* ppos, const float* pedge, const float* prbf,
              const float* penv, const void* pw_rad, const void* const* pw1, const void* const* pw2,
              const float* pcoef, void* ggy, void* gx2, float* gpos2, float* grbf2, float* genv2, void* gw_rad2,
              void* const* gw1_2, void* const* gw2_2, float* gcoef2, const void* saved_bwd, void* ws,
              size_t ws_bytes, void* stream) {
  int r;
  const Dims& d = c.d;
  if ((r = check_weights(d, w_rad, w1, w2)) || (r = check_act(c))) return r;
  if (!x || !pos || !gy || (!rbf && gd.E > 0)) return fail(SO2_EINVAL, "NULL input");
  if ((penv || genv2) && !env) return fail(SO2_EINVAL, "penv or genv2 given without an envelope");
  if ((r = ensure_init())) return r;
  if ((r = debug_validate(c, gd, pos, rbf, env, (hipStream_t)stream))) return r;
  const bool has_pwe1 = !all_null(pw1, d.M + 1), has_pwe2 = !all_null(pw2, d.M + 1);
  // directions on the weights of each system: the user's (plain), or
  // coef pWe + pcoef We (mixture)
  const bool has_pw1 = has_pwe1 || (mx && pcoef), has_pw2 = has_pwe2 || (mx && pcoef);
  // first-order weight gradients per system, needed for the mixture's directions
  const bool first = mx && (pcoef || has_pwe1 || has_pwe2);
  if (has_pwe1)
    for (int a = 0; a <= d.M; ++a)
      if (!pw1[a]) return fail(SO2_EINVAL, "pw1 must be NULL or hold M+1 non-NULL blocks");
  if (has_pwe2)
    for (int a = 0; a <= d.M; ++a)
      if (!pw2[a]) return fail(SO2_EINVAL, "pw2 must be NULL or hold M+1 non-NULL blocks");
  hipStream_t s = (hipStream_t)stream;
  const int n_rbf = c.n_rbf, wS = c.wS();
  if (gd.E == 0 && !mx) {
    int rr = zero_grads(c, gd.N, gx2, gpos2, gw_rad2, gw1_2, gw2_2, s);
    if (rr) return rr;
    if (ggy) return zero(c, ggy, (size_t)gd.N * c.node_floats(), s);
    return SO2_OK;
  }
  const bool recompute = saved == nullptr;
  if (!ws) return fail(SO2_EWORKSPACE, "workspace is NULL");
  const long ec = pick_chunk(c, gd.N, gd.E, 2, recompute, ws_bytes);
  if (ec == 0) return fail(SO2_EWORKSPACE, "double-backward workspace too small for a 1024-edge chunk");
  Arena ar{static_cast<char*>(ws), 0};
  DbwdWs w;
  layout_dbwd(ar, c, gd.N, gd.E, ec, recompute, &w);
  const size_t nf = (size_t)gd.N * c.node_floats(), rf = (size_t)n_rbf * wS;
  const float *x32, *px32, *gy32, *wr32, *pwr32;
  if ((r = f32_in(c, x, w.x32, nf, &x32, s))) return r;
  if ((r = f32_in(c, px, w.px32, nf, &px32, s))) return r;
  if ((r = f32_in(c, gy, w.gy32, nf, &gy32, s))) return r;
  if ((r = f32_in(c, w_rad, w.w_rad32, rf, &wr32, s))) return r;
  if ((r = f32_in(c, pw_rad, w.pw_rad32, rf, &pwr32, s))) return r;
  float* ggy_acc = f32_acc(c, ggy, w.ggy32);
  float* gx2_acc = f32_acc(c, gx2, w.gx2_32);
  float* gwr2_acc = f32_acc(c, gw_rad2, w.gw_rad2_32);
  const bool want_w1 = !all_null(gw1_2, d.M + 1) || gcoef2, want_w2 = !all_null(gw2_2, d.M + 1) || gcoef2;
  if ((r = prepare_weights(c, mx, w1, w2, w.W1, w.W2, w.mix, s))) return r;
  if (!mx) {
    if (has_pw1 && (r = realify(c, 0, pw1, w.pW1[0], s))) return r;
    if (has_pw2 && (r = realify(c, 1, pw2, w.pW2[0], s))) return r;
  } else {
    for (int second = 0; second < 2; ++second) {
      const bool hp = second ? has_pw2 : has_pw1, hwe = second ? has_pwe2 : has_pwe1;
      if (!hp) continue;
      float* pm = w.mix.pmerged[second];
      if (hwe && (r = mix_linear(c, second, second ? pw2 : pw1, mx->coef, pm, w.mix.we32, 0, s))) return r;
      if (pcoef && (r = mix_linear(c, second, second ? w2 : w1, pcoef, pm, w.mix.we32, hwe, s))) return r;
      if ((r = realify_systems(c, second, pm, second ? w.pW2 : w.pW1, s))) return r;
    }
    if (want_w1 && (r = zero_sets(w.gW1r, realified_size(d, 0), s))) return r;
    if (want_w2 && (r = zero_sets(w.gW2r, realified_size(d, 1), s))) return r;
    if (first && want_w1 && (r = zero_sets(w.gW1f, realified_size(d, 0), s))) return r;
    if (first && want_w2 && (r = zero_sets(w.gW2f, realified_size(d, 1), s))) return r;
  }
  ActTab at;
  if ((r = act_tables(c, w.s2t, &at, s))) return r;
  const std::vector<long> se = sys_edges(mx, gd.E);
  const WSet W1 = wset(c, 0, se, w.W1, w1, w.mix.merged[0]), W2 = wset(c, 1, se, w.W2, w2, w.mix.merged[1]);
  const WSet pW1 = wset(c, 0, se, w.pW1, pw1, w.mix.pmerged[0]), pW2 = wset(c, 1, se, w.pW2, pw2, w.mix.pmerged[1]);
  for (long e0 = 0, k = 0; e0 < gd.E; e0 += ec, ++k) {
    GraphDev gc = gd;
    gc.e0 = e0;
    gc.e1 = e0 + ec < gd.E ? e0 + ec : gd.E;
    const int n = (int)(gc.e1 - gc.e0);
    const int acc = k > 0;
    const float* rbf_c = rbf + (size_t)e0 * n_rbf;
    const float* prbf_c = prbf ? prbf + (size_t)e0 * n_rbf : nullptr;
    Primal pr;
    if (recompute) {
      if ((r = forward_chunk(c, at, gc, x32, pos, rbf, wr32, W1, W2, w.pr, s))) return r;
      pr = {w.pr.S, w.pr.T, w.pr.U, w.pr.Z, w.pr.V};
    } else {
      pr = saved_rows(c, saved, gd.E, e0);
    }

    // ---- tangent (dual) forward along (px, ppos, pedge, prbf, pW)
    if (prbf_c) {
      if ((r = radial(c, n, prbf_c, wr32, w.Sdot, s))) return r;
    } else if ((r = fill(w.Sdot, (size_t)n * wS, s))) {
      return r;
    }
    if (pwr32) {
      if ((r = radial(c, n, rbf_c, pwr32, w.Sdot, s, 1))) return r;
    }
    SO2_HIP(launch_edge_dual(d, gc, x32, px32, pos, ppos, pedge, pr.S, w.Sdot, w.Tdot, w.omega, c.bf, s));
    if ((r = run_lin(c, 0, false, w.Tdot, w.Udot, W1, e0, n, 1, 0, s))) return r;
    if (has_pw1 && (r = run_lin(c, 0, false, pr.T, w.Udot, pW1, e0, n, 1, 1, s))) return r;
    if ((r = act_dual(c, at, n, pr.U, w.Udot, w.Zdot, s))) return r;
    if ((r = run_lin(c, 1, false, w.Zdot, w.Vdot, W2, e0, n, 1, 0, s))) return r;
    if (has_pw2 && (r = run_lin(c, 1, false, pr.Z, w.Vdot, pW2, e0, n, 1, 1, s))) return r;
    // dL/dgy = the forward's directional derivative (Eq.(5))
    if (ggy_acc) SO2_HIP(launch_node_dual(d, gc, pos, w.omega, pr.V, w.Vdot, env, penv, ggy_acc, acc, s));

    // ---- reverse of the tangent output with cotangent gy
    SO2_HIP(launch_edge_bwd_dual(d, gc, pos, w.omega, gy32, w.G2, c.bf, pr.V, w.Vdot, env, penv,
                                 gpos2 ? w.p2e : nullptr, genv2, s));
    // The reverse pass's cotangents of the tangent chain (Zdot_bar, Udot_bar,
    // Tdot_bar) depend only on gy and the primal: they are the backward's
    // (Zbar, Ubar, Tbar). With the backward's saved state only the second
    // halves (cotangents of the primal chain) are formed here.
    const BwdRows sb = saved_bwd ? bwd_rows(c, saved_bwd, gd.E, e0) : BwdRows{nullptr, nullptr, nullptr};
    float* Zb = w.ZZ + (size_t)n * d.wZ();
    const float* Zdb = saved_bwd ? sb.Z : w.ZZ;
    void* Ub = offs(w.UU, (size_t)n * d.wU(), c.es);
    const void* Udb = saved_bwd ? sb.U : w.UU;
    float* Tb = w.TT + (size_t)n * d.wT();
    const float* Tdb = saved_bwd ? sb.T : w.TT;
    // [Zdot_bar; Zbar] = G2 W2^T (2n stacked rows)
    if (saved_bwd) {
      if ((r = run_lin(c, 1, true, offs(static_cast<const void*>(w.G2), (size_t)n * d.wZ(), c.es), Zb, W2, e0, n, 1,
                       0, s)))
        return r;
    } else if ((r = run_lin(c, 1, true, w.G2, w.ZZ, W2, e0, n, 2, 0, s))) {
      return r;
    }
    // Zbar += tbar pW2^T
    if (has_pw2 && (r = run_lin(c, 1, true, w.G2, Zb, pW2, e0, n, 1, 1, s))) return r;
    if (want_w2) {
      const void* in[2] = {w.Zdot, pr.Z};
      const void* out[2] = {w.G2, offs(static_cast<const void*>(w.G2), (size_t)n * d.wZ(), c.es)};
      if ((r = run_lin_grad(c, 1, in, out, 2, n, W2, e0, w.gW2r, mx != nullptr, w.P, s))) return r;
      // first-order gradient Z^T tbar (tbar: the first n rows of G2)
      if (first && (r = run_lin_grad(c, 1, &in[1], out, 1, n, W2, e0, w.gW2f, true, w.P, s))) return r;
    }
    // [Udot_bar; Ubar]
    if ((r = act_dbwd(c, at, n, pr.U, w.Udot, Zdb, Zb, saved_bwd ? nullptr : w.UU, Ub, s))) return r;
    // [Tdot_bar; Tbar] = UU W1^T
    if (saved_bwd) {
      if ((r = run_lin(c, 0, true, Ub, Tb, W1, e0, n, 1, 0, s))) return r;
    } else if ((r = run_lin(c, 0, true, w.UU, w.TT, W1, e0, n, 2, 0, s))) {
      return r;
    }
    // Tbar += Udot_bar pW1^T
    if (has_pw1 && (r = run_lin(c, 0, true, Udb, Tb, pW1, e0, n, 1, 1, s))) return r;
    if (want_w1) {
      const void* in[2] = {w.Tdot, pr.T};
      const void* out[2] = {Udb, Ub};
      if ((r = run_lin_grad(c, 0, in, out, 2, n, W1, e0, w.gW1r, mx != nullptr, w.P, s))) return r;
      // first-order gradient T^T Ubar (Ubar: the first n rows of UU)
      if (first && (r = run_lin_grad(c, 0, &in[1], out, 1, n, W1, e0, w.gW1f, true, w.P, s))) return r;
    }
    SO2_HIP(launch_node_bwd_dual(d, gc, x32, px32, pos, w.omega, pr.S, w.Sdot, Tdb, Tb, gx2_acc, w.Sbar, w.Sdb,
                                 gpos2 ? w.p2d : nullptr, gpos2 ? w.p2s : nullptr, acc, s));
    if (gpos2) SO2_HIP(launch_pos2(gc, pos, ppos, pedge, w.omega, w.p2e, w.p2d, w.p2s, w.vbar2_all, d.s2, s));
    if (grbf2) {
      float* out = grbf2 + (size_t)e0 * n_rbf;
      std::vector<GemmProb> ps{prob(w.Sbar, wS, wr32, wS, out, n_rbf, n, n_rbf, wS)};
      if ((r = run_batch(ps, false, true, 0, s))) return r;
      if (pwr32) {
        std::vector<GemmProb> ps2{prob(w.Sdb, wS, pwr32, wS, out, n_rbf, n, n_rbf, wS, 1)};
        if ((r = run_batch(ps2, false, true, 0, s))) return r;
      }
    }
    if (gwr2_acc) {
      TnSeg segs[2] = {{rbf_c, n_rbf, w.Sbar, wS, n}, {prbf_c, n_rbf, w.Sdb, wS, prbf_c ? n : 0}};
      if ((r = run_tn(segs, 2, n_rbf, wS, gwr2_acc, wS, acc, w.P, 0, s))) return r;
    }
  }
  if (!mx) {
    if (want_w2) SO2_HIP(launch_fold_grad(d, 1, w.gW2r[0], gw2_2, c.bf, s, !c.bf && !c.split));
    if (want_w1) SO2_HIP(launch_fold_grad(d, 0, w.gW1r[0], gw1_2, c.bf, s, !c.bf && !c.split));
  } else {
    for (int second = 0; second < 2; ++second) {
      if (!(second ? want_w2 : want_w1)) continue;
      // the merged weights and directions are no longer needed: they take the gradients
      float *gm = w.mix.merged[second], *gf = w.mix.pmerged[second];
      if ((r = fold_systems(c, second, second ? w.gW2r : w.gW1r, gm, s))) return r;
      if (first && (r = fold_systems(c, second, second ? w.gW2f : w.gW1f, gf, s))) return r;
      if ((r = mix_grads(c, second, gm, mx->coef, second ? w2 : w1, first ? gf : nullptr, pcoef,
                         second ? pw2 : pw1, second ? gw2_2 : gw1_2, gcoef2, second == 1 && want_w1, w.mix, s)))
        return r;
    }
  }
  if (gpos2) SO2_HIP(launch_node_pos(gd, w.vbar2_all, gpos2, s));
  if ((r = f32_out(c, ggy_acc, ggy, nf, s))) return r;
  if ((r = f32_out(c, gx2_acc, gx2, nf, s))) return r;
  return f32_out(c, gwr2_acc, gw_rad2, rf, s);
}

}  // namespace

// =====================================================================================
extern "C" {

const char* so2conv_last_error(void) { return last_error(); }

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

int so2conv_generator_table(float* out, int64_t n) {
  const int64_t size = 3 * kGenSize;
  if (!out) return (int)size;
  if (n < size) return fail(SO2_EINVAL, "so2conv_generator_table: output holds fewer than 3 * kGenSize floats");
  std::memcpy(out, kGenHost.v, sizeof(float) * size);
  return (int)size;
}

int so2conv_debug_status(void* stream) {
  clear_error();
  SO2_HIP(hipStreamSynchronize((hipStream_t)stream));
  unsigned w = 0, zero = 0;
  SO2_HIP(hipMemcpyFromSymbol(&w, HIP_SYMBOL(g_debug_word), sizeof(w)));
  if (!w) return SO2_OK;
  SO2_HIP(hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &zero, sizeof(zero)));
  return fail(SO2_EDEVICE, "device-side validation failed: " + debug_bits_text(w));
}

size_t so2conv_graph_workspace_bytes(int32_t n_nodes, int64_t n_edges) { return graph_ws_bytes(n_nodes, n_edges); }

int so2conv_graph_prepare(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst, int32_t* dst_ptr,
                          int32_t* src_perm, int32_t* src_ptr, int32_t* err_word, void* ws, size_t ws_bytes,
                          void* stream) {
  clear_error();
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
  Ctx c;
  if (check_cfg(cfg, &c) || n_edges < 0) return 0;
  return saved_layout(c, n_edges).total;
}

size_t so2conv_saved_bwd_bytes(const so2conv_cfg* cfg, int64_t n_edges) {
  Ctx c;
  if (check_cfg(cfg, &c) || n_edges < 0) return 0;
  return bwd_saved_layout(c, n_edges).total;
}

size_t so2conv_workspace_bytes(const so2conv_cfg* cfg, int32_t n_nodes, int64_t n_edges, int stage) {
  Ctx c;
  if (check_cfg(cfg, &c) || stage < 0 || stage > 2 || n_nodes < 0 || n_edges < 0) return 0;
  return ws_need(c, n_nodes, n_edges, n_edges, stage, false);
}

size_t so2conv_chunked_workspace_bytes(const so2conv_cfg* cfg, int32_t n_nodes, int64_t n_edges, int stage,
                                       int64_t chunk_edges) {
  Ctx c;
  if (check_cfg(cfg, &c) || stage < 0 || stage > 2 || chunk_edges < 1 || n_nodes < 0 || n_edges < 0) return 0;
  const long ec = chunk_edges < n_edges ? chunk_edges : n_edges;
  return ws_need(c, n_nodes, n_edges, ec, stage, true);
}

int so2conv_debug_rotate_gather(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos,
                                const float* rbf, const void* w_rad, void* T_out, void* ws, size_t ws_bytes,
                                void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &c)) || (r = check_graph(g, &gd))) return r;
  if ((r = ensure_init())) return r;
  if (!x || !pos || !rbf || !w_rad || !T_out) return fail(SO2_EINVAL, "NULL input");
  Arena ar{nullptr, 0};
  ar.take((size_t)gd.E * c.wS());
  if (c.bf) {
    ar.take((size_t)gd.N * c.node_floats());
    ar.take((size_t)c.n_rbf * c.wS());
  }
  if (!ws || ws_bytes < ar.used) return fail(SO2_EWORKSPACE, "workspace too small for the rotate-gather hook");
  hipStream_t s = (hipStream_t)stream;
  ar = Arena{static_cast<char*>(ws), 0};
  float* S = ar.take((size_t)gd.E * c.wS());
  float* xt = c.bf ? ar.take((size_t)gd.N * c.node_floats()) : nullptr;
  float* wt = c.bf ? ar.take((size_t)c.n_rbf * c.wS()) : nullptr;
  const float *x32, *w32;
  if ((r = f32_in(c, x, xt, (size_t)gd.N * c.node_floats(), &x32, s))) return r;
  if ((r = f32_in(c, w_rad, wt, (size_t)c.n_rbf * c.wS(), &w32, s))) return r;
  if ((r = radial(c, gd.E, rbf, w32, S, s))) return r;
  SO2_HIP(launch_edge_fwd(c.d, gd, x32, pos, S, T_out, c.bf, s));
  return SO2_OK;
}

int so2conv_fwd(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos, const float* rbf,
                const float* env, const void* w_rad, const void* const* w1, const void* const* w2, void* y,
                void* saved, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &c)) || (r = check_graph(g, &gd))) return r;
  return conv_fwd(c, gd, nullptr, x, pos, rbf, env, w_rad, w1, w2, y, saved, ws, ws_bytes, stream);
}

int so2conv_bwd(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos, const float* rbf,
                const float* env, const void* w_rad, const void* const* w1, const void* const* w2, const void* saved,
                const void* gy, void* gx, float* gpos, float* grbf, float* genv, void* gw_rad, void* const* gw1,
                void* const* gw2, float* gedge, void* saved_bwd, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &c)) || (r = check_graph(g, &gd))) return r;
  return conv_bwd(c, gd, nullptr, x, pos, rbf, env, w_rad, w1, w2, saved, gy, gx, gpos, grbf, genv, gw_rad, gw1, gw2,
                  nullptr, gedge, saved_bwd, ws, ws_bytes, stream);
}

int so2conv_dbwd(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos, const float* rbf,
                 const float* env, const void* w_rad, const void* const* w1, const void* const* w2, const void* saved,
                 const void* gy, const void* px, const float* ppos, const float* pedge, const float* prbf,
                 const float* penv, const void* pw_rad, const void* const* pw1, const void* const* pw2, void* ggy,
                 void* gx2, float* gpos2, float* grbf2, float* genv2, void* gw_rad2, void* const* gw1_2,
                 void* const* gw2_2, const void* saved_bwd, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  int r;
  if ((r = check_cfg(cfg, &c)) || (r = check_graph(g, &gd))) return r;
  return conv_dbwd(c, gd, nullptr, x, pos, rbf, env, w_rad, w1, w2, saved, gy, px, ppos, pedge, prbf, penv, pw_rad,
                   pw1, pw2, nullptr, ggy, gx2, gpos2, grbf2, genv2, gw_rad2, gw1_2, gw2_2, nullptr, saved_bwd, ws,
                   ws_bytes, stream);
}

// ---------------------------------------------------------------- mixture of linear experts entry points
}  // extern "C"

namespace {

int check_mole(const Ctx& c0, const so2mole_cfg* m, long E, Ctx* c, MixIn* mx) {
  *c = c0;
  if (!m) return fail(SO2_EINVAL, "mixture cfg is NULL");
  if (c0.d.s2) return fail(SO2_EUNSUPPORTED, "the mixture of linear experts takes the gated activation only");
  if (m->n_systems < 1 || m->n_systems > 65536) return fail(SO2_EUNSUPPORTED, "n_systems must be in [1, 65536]");
  if (m->n_experts < 4 || m->n_experts > 1024 || m->n_experts % 4)
    return fail(SO2_EUNSUPPORTED, "n_experts must be a multiple of 4 in [4, 1024]");
  if (!m->sys_edge_ptr) return fail(SO2_EINVAL, "sys_edge_ptr is NULL");
  const int64_t* p = m->sys_edge_ptr;
  if (p[0] != 0 || p[m->n_systems] != E) return fail(SO2_EINVAL, "sys_edge_ptr must run from 0 to n_edges");
  for (int s = 0; s < m->n_systems; ++s)
    if (p[s + 1] < p[s]) return fail(SO2_EINVAL, "sys_edge_ptr must be non-decreasing");
  c->ns = m->n_systems;
  c->nk = m->n_experts;
  mx->e.assign(p, p + m->n_systems + 1);
  mx->coef = nullptr;
  return SO2_OK;
}

int check_mole_call(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* m, const float* coef, Ctx* c,
                    GraphDev* gd, MixIn* mx) {
  Ctx c0;
  int r;
  if ((r = check_cfg(cfg, &c0)) || (r = check_graph(g, gd)) || (r = check_mole(c0, m, gd->E, c, mx))) return r;
  if (!coef) return fail(SO2_EINVAL, "coef is NULL");
  mx->coef = coef;
  return SO2_OK;
}

// outputs of a mixture call on a graph without edges: every gradient is zero
int zero_mole_grads(const Ctx& c, void* const* gw1, void* const* gw2, float* gcoef, hipStream_t s) {
  int r;
  for (int second = 0; second < 2; ++second) {
    void* const* gw = second ? gw2 : gw1;
    if (!gw) continue;
    for (int a = 0; a <= c.d.M; ++a)
      if (gw[a] && (r = zero(c, gw[a], (size_t)c.nk * user_block(c.d, second, a), s))) return r;
  }
  if (gcoef && (r = fill(gcoef, (size_t)c.ns * c.nk, s))) return r;
  return SO2_OK;
}

}  // namespace

extern "C" {

size_t so2mole_workspace_bytes(const so2conv_cfg* cfg, const so2mole_cfg* mole, int32_t n_nodes, int64_t n_edges,
                               int stage, int64_t chunk_edges) {
  Ctx c0, c;
  MixIn mx;
  if (check_cfg(cfg, &c0) || stage < 0 || stage > 2 || n_nodes < 0 || n_edges < 0 || chunk_edges < 0) return 0;
  if (check_mole(c0, mole, n_edges, &c, &mx)) return 0;
  if (chunk_edges == 0) return ws_need(c, n_nodes, n_edges, n_edges, stage, false);
  const long ec = chunk_edges > n_edges ? n_edges : chunk_edges;
  return ws_need(c, n_nodes, n_edges, ec, stage, true);
}

int so2mole_fwd(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* mole, const void* x,
                const float* pos, const float* rbf, const float* env, const void* w_rad, const void* const* w1e,
                const void* const* w2e, const float* coef, void* y, void* saved, void* ws, size_t ws_bytes,
                void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  MixIn mx;
  int r;
  if ((r = check_mole_call(cfg, g, mole, coef, &c, &gd, &mx))) return r;
  return conv_fwd(c, gd, &mx, x, pos, rbf, env, w_rad, w1e, w2e, y, saved, ws, ws_bytes, stream);
}

int so2mole_bwd(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* mole, const void* x,
                const float* pos, const float* rbf, const float* env, const void* w_rad, const void* const* w1e,
                const void* const* w2e, const float* coef, const void* saved, const void* gy, void* gx, float* gpos,
                float* grbf, float* genv, void* gw_rad, void* const* gw1e, void* const* gw2e, float* gcoef,
                float* gedge, void* saved_bwd, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  MixIn mx;
  int r;
  if ((r = check_mole_call(cfg, g, mole, coef, &c, &gd, &mx))) return r;
  if (gd.E == 0) {
    if ((r = check_weights(c.d, w_rad, w1e, w2e))) return r;
    hipStream_t s = (hipStream_t)stream;
    if ((r = zero_grads(c, gd.N, gx, gpos, gw_rad, nullptr, nullptr, s))) return r;
    return zero_mole_grads(c, gw1e, gw2e, gcoef, s);
  }
  return conv_bwd(c, gd, &mx, x, pos, rbf, env, w_rad, w1e, w2e, saved, gy, gx, gpos, grbf, genv, gw_rad, gw1e, gw2e,
                  gcoef, gedge, saved_bwd, ws, ws_bytes, stream);
}

int so2mole_dbwd(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* mole, const void* x,
                 const float* pos, const float* rbf, const float* env, const void* w_rad, const void* const* w1e,
                 const void* const* w2e, const float* coef, const void* saved, const void* gy, const void* px,
                 const float* ppos, const float* pedge, const float* prbf, const float* penv, const void* pw_rad,
                 const void* const* pw1e, const void* const* pw2e, const float* pcoef, void* ggy, void* gx2,
                 float* gpos2, float* grbf2, float* genv2, void* gw_rad2, void* const* gw1e_2, void* const* gw2e_2,
                 float* gcoef2, const void* saved_bwd, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  Ctx c;
  GraphDev gd;
  MixIn mx;
  int r;
  if ((r = check_mole_call(cfg, g, mole, coef, &c, &gd, &mx))) return r;
  if (gd.E == 0) {
    if ((r = check_weights(c.d, w_rad, w1e, w2e))) return r;
    hipStream_t s = (hipStream_t)stream;
    if ((r = zero_grads(c, gd.N, gx2, gpos2, gw_rad2, nullptr, nullptr, s))) return r;
    if (ggy && (r = zero(c, ggy, (size_t)gd.N * c.node_floats(), s))) return r;
    return zero_mole_grads(c, gw1e_2, gw2e_2, gcoef2, s);
  }
  return conv_dbwd(c, gd, &mx, x, pos, rbf, env, w_rad, w1e, w2e, saved, gy, px, ppos, pedge, prbf, penv, pw_rad,
                   pw1e, pw2e, pcoef, ggy, gx2, gpos2, grbf2, genv2, gw_rad2, gw1e_2, gw2e_2, gcoef2, saved_bwd, ws,
                   ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- spherical-grid SwiGLU activation
namespace so2 {
namespace {
int check_s2(const so2s2_cfg* cfg, int64_t E) {
  if (!cfg) return fail(SO2_EINVAL, "cfg is NULL");
  if (cfg->rows < 1 || cfg->rows > 32) return fail(SO2_EUNSUPPORTED, "rows must be in [1, 32]");
  if (cfg->channels < 1 || cfg->channels > 65536) return fail(SO2_EUNSUPPORTED, "channels must be in [1, 65536]");
  if (cfg->n_grid < 1 || cfg->n_grid > 256) return fail(SO2_EUNSUPPORTED, "n_grid must be in [1, 256]");
  if (cfg->dtype != SO2_F32) return fail(SO2_EUNSUPPORTED, "the grid activation is float32 only");
  if (cfg->flags) return fail(SO2_EINVAL, "unknown cfg flags");
  if (E < 0) return fail(SO2_EINVAL, "negative edge count");
  return SO2_OK;
}
}  // namespace
}  // namespace so2

extern "C" {

int so2s2_fwd(const so2s2_cfg* cfg, int64_t n_edges, const float* U, const float* G, const float* P, float* Z,
              void* stream) {
  clear_error();
  int r;
  if ((r = check_s2(cfg, n_edges))) return r;
  if (n_edges == 0) return SO2_OK;
  if (!U || !G || !P || !Z) return fail(SO2_EINVAL, "NULL input or output");
  SO2_HIP(launch_s2_fwd(n_edges, cfg->rows, cfg->channels, cfg->n_grid, U, G, P, Z, 0, (hipStream_t)stream));
  return SO2_OK;
}

int so2s2_bwd(const so2s2_cfg* cfg, int64_t n_edges, const float* U, const float* G, const float* P,
              const float* gZ, float* gU, void* stream) {
  clear_error();
  int r;
  if ((r = check_s2(cfg, n_edges))) return r;
  if (n_edges == 0) return SO2_OK;
  if (!U || !G || !P || !gZ || !gU) return fail(SO2_EINVAL, "NULL input or output");
  SO2_HIP(launch_s2_bwd(n_edges, cfg->rows, cfg->channels, cfg->n_grid, U, G, P, gZ, gU, 0, (hipStream_t)stream));
  return SO2_OK;
}

int so2s2_dbwd(const so2s2_cfg* cfg, int64_t n_edges, const float* U, const float* G, const float* P,
               const float* gZ, const float* pU, float* ggZ, float* gU2, void* stream) {
  clear_error();
  int r;
  if ((r = check_s2(cfg, n_edges))) return r;
  if (n_edges == 0) return SO2_OK;
  if (!U || !G || !P || !gZ || !pU) return fail(SO2_EINVAL, "NULL input");
  if (!ggZ && !gU2) return fail(SO2_EINVAL, "no output requested");
  SO2_HIP(launch_s2_dbwd(n_edges, cfg->rows, cfg->channels, cfg->n_grid, U, G, P, gZ, pU, ggZ, gU2, 0,
                         (hipStream_t)stream));
  return SO2_OK;
}

}  // extern "C"

