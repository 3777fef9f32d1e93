// C ABI of the node-to-node spherical projection and of the back-projection
// from the grid (TrimSO(2) page, Appendix B.4, spherical activations):
// argument checks, workspace layout and the schedules of the forward,
// backward and double backward.
#include <algorithm>
#include <string>
#include <vector>

#include "../../include/so2conv.h"
#include "api_common.hpp"
#include "gemm.hpp"
#include "ops.hpp"

using namespace so2;

namespace {

// ---------------------------------------------------------------- spherical projection
struct GridCtx {
  int L, Cin, Ch, Cout, ng, N;
  int d() const { return (L + 1) * (L + 1); }
};

int check_grid(const so2grid_cfg* cfg, int32_t N, GridCtx* g) {
  if (!cfg) return fail(SO2_EINVAL, "cfg is NULL");
  if (cfg->lmax < 0 || cfg->lmax > kMaxL) return fail(SO2_EUNSUPPORTED, "lmax must be in [0, 6]");
  for (int c : {cfg->c_in, cfg->c_h, cfg->c_out})
    if (c < 4 || c > 1024 || c % 4) return fail(SO2_EUNSUPPORTED, "channel counts must be multiples of 4 in [4, 1024]");
  if (cfg->n_grid < 1 || cfg->n_grid > 65536) return fail(SO2_EUNSUPPORTED, "n_grid must be in [1, 65536]");
  if (cfg->dtype != SO2_F32) return fail(SO2_EUNSUPPORTED, "the spherical projection is float32 only");
  if (cfg->flags) return fail(SO2_EINVAL, "unknown cfg flags");
  if (N < 0) return fail(SO2_EINVAL, "negative node count");
  *g = GridCtx{cfg->lmax, cfg->c_in, cfg->c_h, cfg->c_out, cfg->n_grid, N};
  return SO2_OK;
}

// per-(l, m) row problems over all nodes: C[:, j] (+)= op(A[:, j]) with the
// channel map of degree l; rows are node rows j = l^2 + m of [N][d][.]
int grid_rows(const GridCtx& g, const float* A, int wa, const float* Bm, int ldb, bool tb, float* C, int wc,
              int K, int Nn, int acc, hipStream_t s) {
  std::vector<GemmProb> ps;
  for (int l = 0; l <= g.L; ++l)
    for (int m = 0; m < 2 * l + 1; ++m) {
      const int j = l * l + m;
      ps.push_back(prob(A + (size_t)j * wa, g.d() * wa, Bm + (size_t)l * (tb ? Nn : K) * ldb, ldb,
                        C + (size_t)j * wc, g.d() * wc, g.N, Nn, K, acc));
    }
  return run_batch(ps, false, tb, 0, s);
}

// split of the node dimension of the weight-gradient products: about 16
// splits (so that all (l, m) products together fill the GPU), 256..4096 rows
void grid_split(long N, int* splits, int* chunk) {
  long c = ((N + 15) / 16 + kGemmKTile - 1) / kGemmKTile * kGemmKTile;
  c = c < 256 ? 256 : (c > 4096 ? 4096 : c);
  long s = (N + c - 1) / c;
  *splits = (int)(s < 1 ? 1 : s);
  *chunk = (int)c;
}

// Gm_l (+)= sum_m X[:, l^2+m]^T Z[:, l^2+m]  (Gm: [L+1][wx][wz]): every (l, m)
// product in one grouped launch, split over nodes into partials, then one
// fixed-order reduction per degree
int grid_wgrad(const GridCtx& g, const float* X, int wx, const float* Z, int wz, float* Gm, int acc, float* P,
               hipStream_t s) {
  if (g.N == 0) return SO2_OK;
  int sp, ch;
  grid_split(g.N, &sp, &ch);
  std::vector<GemmProb> ps;
  size_t off = 0;
  for (int j = 0; j < g.d(); ++j) {
    GemmProb p = prob(X + (size_t)j * wx, g.d() * wx, Z + (size_t)j * wz, g.d() * wz, P + off, wz, wx, wz, g.N);
    p.k_splits = sp;
    p.k_chunk = ch;
    p.partial = 1;
    ps.push_back(p);
    off += (size_t)sp * wx * wz;
  }
  int r = run_batch(ps, true, false, 0, s);
  if (r) return r;
  off = 0;
  for (int l = 0; l <= g.L; ++l) {
    const int n = (2 * l + 1) * sp;
    SO2_HIP(gemm_reduce(P + off, n, wx, wz, Gm + (size_t)l * wx * wz, wz, acc, s));
    off += (size_t)n * wx * wz;
  }
  return SO2_OK;
}

// partials: every (l, m) product's splits at once, or the channel-map products
// (L+1 segments of one split each)
size_t grid_partials(const GridCtx& g) {
  int sp, ch;
  grid_split(g.N, &sp, &ch);
  const int mx = std::max(std::max(g.Cin, g.Ch), g.Cout);
  return (size_t)std::max(g.d() * sp, g.L + 1) * mx * mx;
}

struct GridWs {
  float *B, *pB, *Y, *Z, *gB, *gB2, *P;
};
void layout_grid(Arena& ar, const GridCtx& g, int stage, GridWs* w) {
  const size_t bsz = (size_t)(g.L + 1) * g.Cin * g.Cout, nf = (size_t)g.N * g.d() * g.Cout;
  *w = GridWs{};
  w->B = ar.take(bsz);
  if (stage == 0) {
    w->Y = ar.take(nf);
    return;
  }
  w->Z = ar.take(nf);
  w->gB = ar.take(bsz);
  if (stage == 2) {
    w->pB = ar.take(bsz);
    w->Y = ar.take(nf);
    w->gB2 = ar.take(bsz);
  }
  w->P = ar.take(grid_partials(g));
}

size_t grid_ws_need(const GridCtx& g, int stage) {
  Arena ar{nullptr, 0};
  GridWs w;
  layout_grid(ar, g, stage, &w);
  return ar.used + 4096;
}

// B_l = W_l A (or += )
int grid_channel_map(const GridCtx& g, const float* W, const float* A, float* B, int acc, hipStream_t s) {
  std::vector<GemmProb> ps;
  for (int l = 0; l <= g.L; ++l)
    ps.push_back(prob(W + (size_t)l * g.Cin * g.Ch, g.Ch, A, g.Cout, B + (size_t)l * g.Cin * g.Cout, g.Cout, g.Cin,
                      g.Cout, g.Ch, acc));
  return run_batch(ps, false, false, 0, s);
}

// gW_l (+)= Gm_l A^T   and   gA (+)= sum_l W_l^T Gm_l
int grid_map_grads(const GridCtx& g, const float* Gm, const float* W, const float* A, float* gW, float* gA, int acc,
                   float* P, hipStream_t s) {
  int r;
  if (gW) {
    std::vector<GemmProb> ps;
    for (int l = 0; l <= g.L; ++l)
      ps.push_back(prob(Gm + (size_t)l * g.Cin * g.Cout, g.Cout, A, g.Cout, gW + (size_t)l * g.Cin * g.Ch, g.Ch, g.Cin,
                        g.Ch, g.Cout, acc));
    if ((r = run_batch(ps, false, true, 0, s))) return r;
  }
  if (gA) {
    std::vector<TnSeg> segs;
    for (int l = 0; l <= g.L; ++l)
      segs.push_back(TnSeg{W + (size_t)l * g.Cin * g.Ch, g.Ch, Gm + (size_t)l * g.Cin * g.Cout, g.Cout, g.Cin});
    if ((r = run_tn(segs.data(), (int)segs.size(), g.Ch, g.Cout, gA, g.Cout, acc, P, 0, s))) return r;
  }
  return SO2_OK;
}

}  // namespace

extern "C" {

// ---------------------------------------------------------------- spherical projection entry points
size_t so2grid_workspace_bytes(const so2grid_cfg* cfg, int32_t n_nodes, int stage) {
  GridCtx g;
  if (check_grid(cfg, n_nodes, &g) || stage < 0 || stage > 2) return 0;
  return grid_ws_need(g, stage);
}

int so2grid_fwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* x, const float* G, const float* W,
                const float* A, float* U, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  GridCtx g;
  int r;
  if ((r = check_grid(cfg, n_nodes, &g))) return r;
  if (!G || !W || !A || (g.N > 0 && (!x || !U))) return fail(SO2_EINVAL, "NULL input or output");
  if (g.N == 0) return SO2_OK;
  if (!ws || ws_bytes < grid_ws_need(g, 0)) return fail(SO2_EWORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  Arena ar{static_cast<char*>(ws), 0};
  GridWs w;
  layout_grid(ar, g, 0, &w);
  if ((r = grid_channel_map(g, W, A, w.B, 0, s))) return r;                          // B_l = W_l A
  if ((r = grid_rows(g, x, g.Cin, w.B, g.Cout, false, w.Y, g.Cout, g.Cin, g.Cout, 0, s))) return r;   // Y = X B
  SO2_HIP(launch_grid_apply(g.L, g.N, g.ng, g.Cout, G, w.Y, U, s));                 // U = G Y
  return SO2_OK;
}

int so2grid_bwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* x, const float* G, const float* W,
                const float* A, const float* gU, float* gx, float* gW, float* gA, void* ws, size_t ws_bytes,
                void* stream) {
  clear_error();
  GridCtx g;
  int r;
  if ((r = check_grid(cfg, n_nodes, &g))) return r;
  if (!G || !W || !A || (g.N > 0 && (!x || !gU))) return fail(SO2_EINVAL, "NULL input");
  hipStream_t s = (hipStream_t)stream;
  if (g.N == 0) {   // no nodes: zero weight gradients
    if (gW && (r = fill(gW, (size_t)(g.L + 1) * g.Cin * g.Ch, s))) return r;
    if (gA && (r = fill(gA, (size_t)g.Ch * g.Cout, s))) return r;
    return SO2_OK;
  }
  if (!ws || ws_bytes < grid_ws_need(g, 1)) return fail(SO2_EWORKSPACE, "workspace too small");
  Arena ar{static_cast<char*>(ws), 0};
  GridWs w;
  layout_grid(ar, g, 1, &w);
  if ((r = grid_channel_map(g, W, A, w.B, 0, s))) return r;
  SO2_HIP(launch_grid_apply_t(g.L, g.N, g.ng, g.Cout, G, gU, w.Z, s));              // Z = G^T gU
  if (gx && (r = grid_rows(g, w.Z, g.Cout, w.B, g.Cout, true, gx, g.Cin, g.Cout, g.Cin, 0, s))) return r;  // Z B^T
  if (gW || gA) {
    if ((r = grid_wgrad(g, x, g.Cin, w.Z, g.Cout, w.gB, 0, w.P, s))) return r;      // Bbar_l = X^T Z
    if ((r = grid_map_grads(g, w.gB, W, A, gW, gA, 0, w.P, s))) return r;
  }
  return SO2_OK;
}

int so2grid_dbwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* x, const float* G, const float* W,
                 const float* A, const float* gU, const float* px, const float* pW, const float* pA, float* ggU,
                 float* gx2, float* gW2, float* gA2, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  GridCtx g;
  int r;
  if ((r = check_grid(cfg, n_nodes, &g))) return r;
  if (!G || !W || !A || (g.N > 0 && (!x || !gU))) return fail(SO2_EINVAL, "NULL input");
  hipStream_t s = (hipStream_t)stream;
  if (g.N == 0) {
    if (gW2 && (r = fill(gW2, (size_t)(g.L + 1) * g.Cin * g.Ch, s))) return r;
    if (gA2 && (r = fill(gA2, (size_t)g.Ch * g.Cout, s))) return r;
    return SO2_OK;
  }
  if (!ws || ws_bytes < grid_ws_need(g, 2)) return fail(SO2_EWORKSPACE, "workspace too small");
  Arena ar{static_cast<char*>(ws), 0};
  GridWs w;
  layout_grid(ar, g, 2, &w);
  const size_t nf = (size_t)g.N * g.d();
  const bool has_pB = pW || pA;
  if ((r = grid_channel_map(g, W, A, w.B, 0, s))) return r;
  if (pW && (r = grid_channel_map(g, pW, A, w.pB, 0, s))) return r;                 // pB = pW A + W pA
  if (pA && (r = grid_channel_map(g, W, pA, w.pB, pW ? 1 : 0, s))) return r;
  SO2_HIP(launch_grid_apply_t(g.L, g.N, g.ng, g.Cout, G, gU, w.Z, s));              // Z = G^T gU
  // dL/dgU = G (px B + x pB)
  if (ggU) {
    if (!px && !has_pB) {
      if ((r = fill(ggU, (size_t)g.N * g.ng * g.Cout, s))) return r;
    } else {
      if (px && (r = grid_rows(g, px, g.Cin, w.B, g.Cout, false, w.Y, g.Cout, g.Cin, g.Cout, 0, s))) return r;
      if (has_pB && (r = grid_rows(g, x, g.Cin, w.pB, g.Cout, false, w.Y, g.Cout, g.Cin, g.Cout, px ? 1 : 0, s)))
        return r;
      SO2_HIP(launch_grid_apply(g.L, g.N, g.ng, g.Cout, G, w.Y, ggU, s));
    }
  }
  // dL/dx = Z pB^T
  if (gx2) {
    if (has_pB) {
      if ((r = grid_rows(g, w.Z, g.Cout, w.pB, g.Cout, true, gx2, g.Cin, g.Cout, g.Cin, 0, s))) return r;
    } else if ((r = fill(gx2, nf * g.Cin, s))) {
      return r;
    }
  }
  // dL/dW = (px^T Z) A^T + Bbar pA^T ; dL/dA = sum W^T (px^T Z) + sum pW^T Bbar
  if (gW2 || gA2) {
    if (gW2 && (r = fill(gW2, (size_t)(g.L + 1) * g.Cin * g.Ch, s))) return r;
    if (gA2 && (r = fill(gA2, (size_t)g.Ch * g.Cout, s))) return r;
    if (px) {
      if ((r = grid_wgrad(g, px, g.Cin, w.Z, g.Cout, w.gB2, 0, w.P, s))) return r;
      if ((r = grid_map_grads(g, w.gB2, W, A, gW2, gA2, 1, w.P, s))) return r;
    }
    if (has_pB) {
      if ((r = grid_wgrad(g, x, g.Cin, w.Z, g.Cout, w.gB, 0, w.P, s))) return r;   // Bbar
      if (pA && gW2) {   // gW2_l += Bbar_l pA^T
        std::vector<GemmProb> ps;
        for (int l = 0; l <= g.L; ++l)
          ps.push_back(prob(w.gB + (size_t)l * g.Cin * g.Cout, g.Cout, pA, g.Cout, gW2 + (size_t)l * g.Cin * g.Ch,
                            g.Ch, g.Cin, g.Ch, g.Cout, 1));
        if ((r = run_batch(ps, false, true, 0, s))) return r;
      }
      if (pW && gA2) {   // gA2 += sum_l pW_l^T Bbar_l
        std::vector<TnSeg> segs;
        for (int l = 0; l <= g.L; ++l)
          segs.push_back(TnSeg{pW + (size_t)l * g.Cin * g.Ch, g.Ch, w.gB + (size_t)l * g.Cin * g.Cout, g.Cout, g.Cin});
        if ((r = run_tn(segs.data(), (int)segs.size(), g.Ch, g.Cout, gA2, g.Cout, 1, w.P, 0, s))) return r;
      }
    }
  }
  return SO2_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- back-projection from the grid
// Z^(l) = H_l (Y A) computed as (H_l Y) A (Appendix B.4, the second
// identity): per node V = H Y ((L+1)^2 x C_h, one streaming pass over the grid
// values), then Z = V A as one product over all node rows.
namespace {
struct BackCtx {
  int L, Ch, Cout, ng, N;
  int d() const { return (L + 1) * (L + 1); }
  long rows() const { return (long)N * d(); }
};
int check_back(const so2grid_cfg* cfg, int32_t N, BackCtx* b) {
  GridCtx g;
  const int r = check_grid(cfg, N, &g);
  if (r) return r;
  if ((long)N * g.d() > 0x7fffffffL) return fail(SO2_EUNSUPPORTED, "too many node rows");
  *b = BackCtx{g.L, g.Ch, g.Cout, g.ng, N};
  return SO2_OK;
}
struct BackWs {
  float *V, *W, *PV, *P;
};
void layout_back(Arena& ar, const BackCtx& b, int stage, BackWs* w) {
  const size_t nv = (size_t)b.rows() * b.Ch;
  *w = BackWs{};
  w->V = ar.take(nv);
  if (stage >= 1) {
    w->W = ar.take(nv);
    int sp, ch;
    split_plan(b.rows(), &sp, &ch);                 // run_tn's partials
    w->P = ar.take((size_t)sp * b.Ch * b.Cout);
  }
  if (stage == 2) w->PV = ar.take(nv);
}
size_t back_ws_need(const BackCtx& b, int stage) {
  Arena ar{nullptr, 0};
  BackWs w;
  layout_back(ar, b, stage, &w);
  return ar.used + 4096;
}
// C [rows][Cout] (+)= V [rows][Ch] A [Ch][Cout]
int back_map(const BackCtx& b, const float* V, const float* A, float* C, int acc, hipStream_t s) {
  std::vector<GemmProb> ps{prob(V, b.Ch, A, b.Cout, C, b.Cout, (int)b.rows(), b.Cout, b.Ch, acc)};
  return run_batch(ps, false, false, kOpF32, s);
}
// T [rows][Ch] = Z [rows][Cout] A^T
int back_map_t(const BackCtx& b, const float* Z, const float* A, float* T, hipStream_t s) {
  std::vector<GemmProb> ps{prob(Z, b.Cout, A, b.Cout, T, b.Ch, (int)b.rows(), b.Ch, b.Cout)};
  return run_batch(ps, false, true, kOpF32, s);
}
// gA [Ch][Cout] (+)= V^T Z over all node rows (fixed-order split-K)
int back_map_grad(const BackCtx& b, const float* V, const float* Z, float* gA, int acc, float* P, hipStream_t s) {
  TnSeg seg{V, b.Ch, Z, b.Cout, b.rows()};
  return run_tn(&seg, 1, b.Ch, b.Cout, gA, b.Cout, acc, P, kOpF32, s);
}
}  // namespace

extern "C" {

size_t so2grid_back_workspace_bytes(const so2grid_cfg* cfg, int32_t n_nodes, int stage) {
  BackCtx b;
  if (check_back(cfg, n_nodes, &b) || stage < 0 || stage > 2) return 0;
  return back_ws_need(b, stage);
}

int so2grid_back_fwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* Y, const float* H, const float* A,
                     float* Z, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  BackCtx b;
  int r;
  if ((r = check_back(cfg, n_nodes, &b))) return r;
  if (!H || !A || (b.N > 0 && (!Y || !Z))) return fail(SO2_EINVAL, "NULL input or output");
  if (b.N == 0) return SO2_OK;
  if (!ws || ws_bytes < back_ws_need(b, 0)) return fail(SO2_EWORKSPACE, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  Arena ar{static_cast<char*>(ws), 0};
  BackWs w;
  layout_back(ar, b, 0, &w);
  SO2_HIP(launch_grid_apply_t(b.L, b.N, b.ng, b.Ch, H, Y, w.V, s, 1));        // V = H Y
  return back_map(b, w.V, A, Z, 0, s);                                          // Z = V A
}

int so2grid_back_bwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* Y, const float* H, const float* A,
                     const float* gZ, float* gY, float* gA, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  BackCtx b;
  int r;
  if ((r = check_back(cfg, n_nodes, &b))) return r;
  if (!H || !A || (b.N > 0 && (!Y || !gZ))) return fail(SO2_EINVAL, "NULL input");
  hipStream_t s = (hipStream_t)stream;
  if (b.N == 0) return gA ? fill(gA, (size_t)b.Ch * b.Cout, s) : SO2_OK;
  if (!ws || ws_bytes < back_ws_need(b, 1)) return fail(SO2_EWORKSPACE, "workspace too small");
  Arena ar{static_cast<char*>(ws), 0};
  BackWs w;
  layout_back(ar, b, 1, &w);
  if (gY) {                                                                     // gY = H^T (gZ A^T)
    if ((r = back_map_t(b, gZ, A, w.W, s))) return r;
    SO2_HIP(launch_grid_apply(b.L, b.N, b.ng, b.Ch, H, w.W, gY, s, 1));
  }
  if (gA) {                                                                     // gA = (H Y)^T gZ
    SO2_HIP(launch_grid_apply_t(b.L, b.N, b.ng, b.Ch, H, Y, w.V, s, 1));
    if ((r = back_map_grad(b, w.V, gZ, gA, 0, w.P, s))) return r;
  }
  return SO2_OK;
}

int so2grid_back_dbwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* Y, const float* H, const float* A,
                      const float* gZ, const float* pY, const float* pA, float* ggZ, float* gY2, float* gA2,
                      void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  BackCtx b;
  int r;
  if ((r = check_back(cfg, n_nodes, &b))) return r;
  if (!H || !A || (b.N > 0 && (!Y || !gZ))) return fail(SO2_EINVAL, "NULL input");
  hipStream_t s = (hipStream_t)stream;
  if (b.N == 0) return gA2 ? fill(gA2, (size_t)b.Ch * b.Cout, s) : SO2_OK;
  if (!ws || ws_bytes < back_ws_need(b, 2)) return fail(SO2_EWORKSPACE, "workspace too small");
  Arena ar{static_cast<char*>(ws), 0};
  BackWs w;
  layout_back(ar, b, 2, &w);
  const size_t ny = (size_t)b.N * b.ng * b.Ch;
  if (pY) SO2_HIP(launch_grid_apply_t(b.L, b.N, b.ng, b.Ch, H, pY, w.PV, s, 1));   // PV = H pY
  // dL/dgZ = (H pY) A + (H Y) pA
  if (ggZ) {
    if (!pY && !pA) {
      if ((r = fill(ggZ, (size_t)b.rows() * b.Cout, s))) return r;
    } else {
      if (pY && (r = back_map(b, w.PV, A, ggZ, 0, s))) return r;
      if (pA) {
        SO2_HIP(launch_grid_apply_t(b.L, b.N, b.ng, b.Ch, H, Y, w.V, s, 1));    // V = H Y
        if ((r = back_map(b, w.V, pA, ggZ, pY ? 1 : 0, s))) return r;
      }
    }
  }
  // dL/dY = H^T (gZ pA^T)
  if (gY2) {
    if (pA) {
      if ((r = back_map_t(b, gZ, pA, w.W, s))) return r;
      SO2_HIP(launch_grid_apply(b.L, b.N, b.ng, b.Ch, H, w.W, gY2, s, 1));
    } else if ((r = fill(gY2, ny, s))) {
      return r;
    }
  }
  // dL/dA = (H pY)^T gZ
  if (gA2) {
    if (pY) {
      if ((r = back_map_grad(b, w.PV, gZ, gA2, 0, w.P, s))) return r;
    } else if ((r = fill(gA2, (size_t)b.Ch * b.Cout, s))) {
      return r;
    }
  }
  return SO2_OK;
}

}  // extern "C"
