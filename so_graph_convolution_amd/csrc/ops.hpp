// Host-side launchers of the convolution's kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include "layout.hpp"
#include "numeric.hpp"

namespace so2 {

struct GraphDev {
  int N;
  long E;
  const int* src;
  const int* dst;
  const float* shift;     // [E,3] or null
  const int* dst_ptr;     // [N+1] incoming-edge ranges (edges sorted by dst)
  const int* src_perm;    // [E] edge ids ordered by (src, edge id)
  const int* src_ptr;     // [N+1] ranges into src_perm
  long e0, e1;            // edge chunk [e0, e1): per-edge buffers are indexed by e - e0
};

// (lmax, mmax) pairs with compiled kernels
bool lm_supported(int L, int M);

// upload the so(3) generator tables to the current device (idempotent per device)
int init_generators();

// Buffers marked "operand" below hold the per-edge inputs of the per-order
// linears: float32, or bfloat16 when the launcher's bf16 flag is set.

// ---- forward
// T[e] (operand; m-major, width q*2C) = S[e] * (R_e [x_src | x_dst])
int launch_edge_fwd(const Dims& d, const GraphDev& g, const float* x, const float* pos, const float* S, void* T,
                    int bf16, hipStream_t s);
// Z (operand) = gate(U)
int launch_gate_fwd(const Dims& d, long E, const float* U, void* Z, int bf16, hipStream_t s);
// y[i] (+)= sum_{e -> i, e in chunk} env[e] R_e^T V[e]  (env: per-edge envelope, null = 1)
int launch_node_fwd(const Dims& d, const GraphDev& g, const float* pos, const float* V, const float* env, float* y,
                    int accumulate, hipStream_t s);

// ---- backward
// tbar[e] (operand) = env_e R_e gy[dst]; tau[e] = torque of env_e <V, R gy> (for the
// position gradient); genv[e] (global index, if not null) = <V, R gy>
int launch_edge_bwd(const Dims& d, const GraphDev& g, const float* pos, const float* gy, const float* V,
                    const float* env, void* tbar, float* tau, float* genv, int bf16, hipStream_t s);
// Ubar (operand) from Zbar (gate backward)
int launch_gate_bwd(const Dims& d, long E, const float* U, const float* Zbar, void* Ubar, int bf16, hipStream_t s);
// gx[n] (both halves), Sbar[e], tau_dst[e], tau_src[e]
int launch_node_bwd(const Dims& d, const GraphDev& g, const float* x, const float* pos, const float* S,
                    const float* Tbar, float* gx, float* Sbar, float* tau_dst, float* tau_src, int accumulate,
                    hipStream_t s);
// vbar[e] = rhat x (tau1 + tau2 + tau3) / rho for the chunk's edges (vbar indexed globally)
// roll != 0: the frame's turn about the edge axis counts (activations that are not roll-invariant)
int launch_vbar(const GraphDev& g, const float* pos, const float* tau1, const float* tau2, const float* tau3,
                float* vbar, int roll, hipStream_t s);
// gpos[n] = sum_out vbar - sum_in vbar over every edge
int launch_node_pos(const GraphDev& g, const float* vbar, float* gpos, hipStream_t s);

// ---- double backward (force-training pattern and general directions)
// Tdot (operand) = Sdot*(R a) + S*(Rdot a + R adot), Rdot from the position direction; also
// writes the per-edge rotation direction omega[e][3]
int launch_edge_dual(const Dims& d, const GraphDev& g, const float* x, const float* px, const float* pos,
                     const float* ppos, const float* pedge, const float* S, const float* Sdot, void* Tdot,
                     float* omega, int bf16, hipStream_t s);
// Zdot (operand)
int launch_gate_dual(const Dims& d, long E, const float* U, const float* Udot, void* Zdot, int bf16, hipStream_t s);
// ydot[i] = sum_e env (Rdot^T V + R^T Vdot) + penv R^T V
int launch_node_dual(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* V,
                     const float* Vdot, const float* env, const float* penv, float* ydot, int accumulate,
                     hipStream_t s);
// G2 (operand) rows [0,E) = env R gy[dst], rows [E,2E) = env Rdot gy[dst] + penv R gy[dst];
// with p2 (not null) also the per-edge torque and rate cotangent [E][6] of ydot's
// rotations; with genv2 (not null, global index) the envelope derivative
int launch_edge_bwd_dual(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* gy,
                         void* G2, int bf16, const float* V, const float* Vdot, const float* env, const float* penv,
                         float* p2, float* genv2, hipStream_t s);
// vbar2[e] (global edge index) = position derivative of the double backward per edge vector,
// from the three [E][6] torque/rate parts (chunk-relative rows)
int launch_pos2(const GraphDev& g, const float* pos, const float* ppos, const float* pedge, const float* omega,
                const float* pe, const float* pd, const float* ps, float* vbar2, int roll, hipStream_t s);
// from (Zdot_bar, Zbar) produce the operands (Udot_bar, Ubar), E rows each;
// Udb NULL: Udot_bar is not written
int launch_gate_dbwd(const Dims& d, long E, const float* U, const float* Udot, const float* Zdb, const float* Zb,
                     void* Udb, void* Ub, int bf16, hipStream_t s);
// gx2 and (Sbar, Sdot_bar) from Tdot_bar (Tdb) and Tbar (Tb), chunk rows each; with p2_dst/p2_src
// (not null) also the per-edge torque and rate cotangent [E][6] of the rotation on gather, per half
int launch_node_bwd_dual(const Dims& d, const GraphDev& g, const float* x, const float* px, const float* pos,
                         const float* omega, const float* S, const float* Sdot, const float* Tdb, const float* Tb,
                         float* gx2, float* Sbar, float* Sdot_bar, float* p2_dst, float* p2_src, int accumulate,
                         hipStream_t s);

// ---- weights
// Wr (realified per order): block 0 = W[0]; block m = [[W_m0, W_m1], [-W_m1, W_m0]].
// float32: w and wr float. bfloat16: w bfloat16 (float32 with in_f32); wr
// holds every block bfloat16 and wrt (if not null) every block transposed
// ([cols][rows]).
int launch_realify(const Dims& d, int second, const void* const* w, void* wr, void* wrt, int bf16, hipStream_t s,
                   int in_f32 = 0);
// fold the realified float32 gradient back: gW_m0 = G00 + G11, gW_m1 = G01 - G10 (m >= 1),
// gW_0 = G_0; gw blocks float32 or bfloat16. user_layout (float32): blocks
// m >= 1 already hold [gW_m0 | gW_m1] ([k][2h], from the complex products) at
// their realified offsets and are copied.
int launch_fold_grad(const Dims& d, int second, const float* gr, void* const* gw, int bf16, hipStream_t s,
                     int user_layout = 0);
// dtype conversions of n elements
int launch_to_f32(const bf16s* in, float* out, size_t n, hipStream_t s);
int launch_to_bf16(const float* in, bf16s* out, size_t n, hipStream_t s);

// realified weight geometry: rows/cols of block a and its offset (floats) in the packed buffer
void realified_shape(const Dims& d, int second, int a, int* rows, int* cols, long* off);
long realified_size(const Dims& d, int second);

// ---- node-to-node spherical projection: per node U = G Y (G: [ng][(L+1)^2]; Y, Z: [N][(L+1)^2][C];
// U: [N][ng][C]) and Z = G^T U
// U = G Y per node (G [ng][d]; basis_t: G given as [d][ng])
int launch_grid_apply(int L, int N, int ng, int C, const float* G, const float* Y, float* U, hipStream_t s,
                      int basis_t = 0);
// Z = G^T U per node (G [ng][d]; basis_t: G given as [d][ng], so Z = H U for H = G^T)
int launch_grid_apply_t(int L, int N, int ng, int C, const float* G, const float* U, float* Z, hipStream_t s,
                        int basis_t = 0);
// spherical-grid SwiGLU activation on edges (s2act.hip); U-shaped arrays
// [E][q][2C], Z-shaped [E][q][C]; float32 inputs, outputs of the operand type
// (bfloat16 when bf16 != 0)
int launch_s2_fwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, void* Z, int bf16,
                  hipStream_t s);
int launch_s2_bwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                  void* gU, int bf16, hipStream_t s);
int launch_s2_dbwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                   const float* pU, void* ggZ, void* gU2, int bf16, hipStream_t s);
// o2 = J^T Zb + d/dU <Za, J Ud>, o1 = J^T Za (o1 may be NULL)
int launch_s2_rev(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* Ud,
                  const float* Za, const float* Zb, void* o1, void* o2, int bf16, hipStream_t s);
// caller's degree-major grid tables -> m-major row order
int launch_s2_mmajor(int L, int M, int ng, const float* G, const float* P, float* Gm, float* Pm, hipStream_t s);

// ---- graph preparation
size_t graph_ws_bytes(int N, long E);
int launch_graph_prepare(int N, long E, const int* src, const int* dst, int* dst_ptr, int* src_perm, int* src_ptr,
                         void* ws, size_t ws_bytes, int* err_word, hipStream_t s);

}  // namespace so2
