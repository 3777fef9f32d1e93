/* so2conv.h -- C ABI of the MI355X fused edgewise SO(2) convolution.
 *
 * The operation (TrimSO(2): Fast and Memory-Efficient Training of Equivariant
 * Interatomic Potentials; Section 2 Eq.(1)-(2), Section 3.2, Appendix A.1-A.2
 * and B.1-B.3): for every directed edge e = (j -> i), j = src[e], i = dst[e],
 *   v_e = pos[j] - pos[i] + shift_e                          (A.1 edge geometry)
 *   D_e = real Wigner-D blocks of the frame R_e, R_e v_e/|v_e| = +z
 *   T_e = s_e * (D_e [x_j | x_i]),  s_e = rbf_e W_rad         (B.1, C.1 radial scaling)
 *   first SO(2) linear per order m (Eq.(1)), gated activation (B.2),
 *   second SO(2) linear, y_i = sum_{e -> i} (J D_e)^T t_e      (B.3)
 * with backward (Section 3.3 Eq.(4)) and double backward (Eq.(5), A.3 Eq.(3)).
 *
 * Conventions (all arrays row-major, contiguous):
 *   L = lmax (0..6), M = mmax (0..L), C = channels (multiple of 16, 16..256),
 *   d = (L+1)^2 node rows in degree-major order (l, m = -l..l), real
 *   orthonormal harmonics without Condon-Shortley phase (Y_1 ~ (y, z, x)).
 *   Node features x, y, gx, gy, px, ggy, gx2: [N, d, C] of the call's dtype.
 *   pos, gpos, ppos: [N, 3] float32.  shift, gedge, pedge: [E, 3] float32.
 *   rbf, grbf, prbf: [E, n_rbf] float32 (n_rbf a multiple of 4).
 *   env, genv, penv, genv2: [E, H] float32 (H = cfg->heads), optional weights
 *   of each message before the receiver sum (Appendix C.1: eSEN and UMA sum
 *   messages with their cutoff envelopes, H = 1; EquiformerV3 applies
 *   attention weights before aggregation, one per head): channel c of the
 *   message belongs to head c / (C / H), and
 *   y_i[:, c] = sum_{e -> i} env[e, head(c)] ((J D_e)^T t_e)[:, c].
 *   NULL env = no weights (then genv, penv and genv2 must be NULL). Like rbf
 *   it is an input: its dependence on positions or on other features (an
 *   attention softmax) is the caller's chain rule through genv / genv2.
 *   w_rad: [n_rbf, (L+1) * 2C], column (l, c_in), c_in < C: source channels.
 *   w1[0]: [(L+1)*2C, (L+1)*C + L*C]  rows (l, c_in); columns (l, c) then the
 *          gate columns (l = 1..L, c).
 *   w1[m]: [(L-m+1)*2C, 2*(L-m+1)*C] = [W_m0 | W_m1], rows (l = m..L, c_in),
 *          u_+ = T_+ W_m0 - T_- W_m1, u_- = T_+ W_m1 + T_- W_m0 (Eq.(1)), "+"
 *          is order +m, "-" is order -m.
 *   w2[0]: [(L+1)*C, (L+1)*C];  w2[m]: [(L-m+1)*C, 2*(L-m+1)*C].
 *   Gate: l = 0 -> SiLU(u); l >= 1 -> sigmoid(gate_{l,c}) * u for every
 *   retained order |m| <= min(l, M). (cfg->act selects the spherical-grid
 *   SwiGLU instead, which changes the first linear's columns; see act.)
 *   Graph: dst non-decreasing (edges grouped by receiver).
 *
 * dtype (cfg->dtype): SO2_F32 -- every array float32, float32 arithmetic.
 *   SO2_BF16 -- node features (x, y, gy, gx, px, ggy, gx2) and weights with
 *   their gradients (w_rad, w1, w2, gw_*, pw_*) are bfloat16; pos, shift, rbf
 *   and their gradients and directions stay float32. Node arrays are widened
 *   to float32 once per call; the per-order products run on bfloat16 matrix
 *   cores (operands rounded to nearest even) with float32 accumulation, and
 *   every other step (rotations, gates, reductions, weight-gradient sums)
 *   computes in float32; outputs are rounded to bfloat16 once at the end.
 *   Arrays typed `void*` below hold elements of the call's dtype.
 *
 * Ownership: every array pointer is a caller-owned DEVICE pointer on the
 * current HIP device, except the pointer arrays w1/w2/gw1/... themselves,
 * which are HOST arrays of M+1 device pointers. The library never allocates
 * device memory: scratch comes from the caller's workspace `ws` (size from
 * so2conv_workspace_bytes), intermediate state kept for differentiation from
 * `saved` (size from so2conv_saved_bytes). Work is enqueued on `stream`
 * (a hipStream_t, NULL = default stream); no call synchronises.
 *
 * Errors: a negative so2_status is returned and so2conv_last_error() gives a
 * message (thread-local). Argument checks happen on the host before any
 * work is enqueued. Outputs are overwritten; a NULL output pointer means "not
 * requested" and its work is skipped. Results are bitwise reproducible for
 * identical inputs (fixed-order reductions, no floating-point atomics).
 */
#ifndef SO2CONV_H
#define SO2CONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SO2_OK = 0,
  SO2_EINVAL = -1,        /* bad argument (null required pointer, bad size, ...) */
  SO2_EUNSUPPORTED = -2,  /* configuration without compiled kernels */
  SO2_EWORKSPACE = -3,    /* workspace or saved buffer too small */
  SO2_EHIP = -4,          /* a HIP runtime call failed */
  SO2_EDEVICE = -5        /* device-side validation failed */
} so2_status;

typedef enum { SO2_F32 = 0, SO2_BF16 = 1 } so2_dtype;

/* cfg->flags */
enum {
  /* Validate the inputs on the device before any compute kernel: edge indices
   * in range, receivers non-decreasing, no zero-length edge, finite positions,
   * shifts, rbf and message weights. The call then synchronises its stream and returns
   * SO2_EDEVICE (message: the failed checks) instead of computing; the word of
   * the last checked call stays readable through so2conv_debug_status. */
  SO2_DEBUG_CHECKS = 2,
  /* float32 calls: run the per-order products on the float32 matrix cores
   * (v_mfma_f32_32x32x2_f32, orders >= 1 as three-product complex GEMMs)
   * instead of the default, which writes every float32 operand as the exact
   * sum of three bfloat16 pieces and multiplies the pieces on the bfloat16
   * matrix cores with float32 accumulation (six piece products per float32
   * product; the three dropped ones sum to below 2^-23 of it). Both give
   * float32-accurate products; the default is faster on gfx950, whose
   * bfloat16 matrix rate is sixteen times its float32 one. */
  SO2_F32_NATIVE = 4,
  /* Gate the first linear's forward products in their epilogue (TrimSO(2)
   * page, Section 3.2 "Recombination with activation"): the gate columns
   * run first, then every other first-linear product writes U and the
   * gated Z together, instead of a separate gate pass over U. Float32 calls
   * through bfloat16 pieces and bfloat16 calls with the gated activation;
   * otherwise ignored. Results are bitwise those without the flag. Off by
   * default: measured on MI355X it is slower (medium workload 438 against
   * 435 ms per step, high-degree 537 against 528), the per-element gate
   * reads and sigmoids in the epilogue costing more than the pass over U
   * they replace. */
  SO2_FUSED_GATE = 8
};

/* cfg->act: the Edge -> Edge activation between the two SO(2) linears
 * (TrimSO(2) page, Appendix C.1 "Implementation": eSEN and UMA recombine with
 * a gated activation, EquiformerV3 uses its spherical-grid activation; Table
 * 2 names it SwiGLU-S2).
 *   SO2_ACT_GATE: the gate described at the top of this file.
 *   SO2_ACT_SWIGLU_S2: the first linear has 2C output channels per retained
 *     row (channels 0..C-1 the value half u_v, C..2C-1 the gate half u_g):
 *       w1[0]: [(L+1)*2C, (L+1)*2C], columns (l, c'), c' in [0, 2C);
 *       w1[m]: [(L-m+1)*2C, 2*(L-m+1)*2C] = [W_m0 | W_m1], columns of each
 *              half (l = m..L, c'), Eq.(1) as above.
 *     Per edge and channel c, over the q retained rows of the edge frame:
 *       v = G u_v,  a = G u_g,  s = SiLU(a) * v,  z = P s
 *     with G = grid_basis [n_grid][q] (the retained basis at n_grid points of
 *     the edge-frame sphere) and P = grid_proj [q][n_grid] (the projection
 *     back), device float32 arrays the calls only read; a row index r counts
 *     the retained rows in degree-major order (l = 0..L, then m =
 *     -min(l,M)..min(l,M)). q <= 32 and n_grid in [1, 256] (else
 *     SO2_EUNSUPPORTED); the compute calls return SO2_EINVAL for NULL tables.
 *     G and P are constants: no gradients are formed for them. The grid
 *     products take float32 operands on the float32 matrix cores in SO2_F32
 *     calls, and bfloat16 operands (the float32 rows, the tables and the
 *     grid values rounded to nearest even) with float32 accumulation in
 *     SO2_BF16 calls; the nonlinearity is float32 in both, and z is stored
 *     in the operand type of the second linear.
 *   The size queries read only act and n_grid. The mixture entry points
 *   (so2mole_*) take SO2_ACT_GATE only. */
enum { SO2_ACT_GATE = 0, SO2_ACT_SWIGLU_S2 = 1 };

/* heads: 0 or 1 = one weight per edge; H > 1 divides channels, C / H is 16,
 * 32 or a multiple of 64, H <= 16 (else SO2_EUNSUPPORTED). */
typedef struct {
  int32_t lmax, mmax, channels, n_rbf, dtype, flags, heads;
  int32_t act;               /* SO2_ACT_GATE or SO2_ACT_SWIGLU_S2 */
  int32_t n_grid;            /* SO2_ACT_SWIGLU_S2: grid points */
  const float* grid_basis;   /* SO2_ACT_SWIGLU_S2: G [n_grid][q], device */
  const float* grid_proj;    /* SO2_ACT_SWIGLU_S2: P [q][n_grid], device */
} so2conv_cfg;

typedef struct {
  int32_t n_nodes;
  int64_t n_edges;
  const int32_t* src;      /* [E] sender j */
  const int32_t* dst;      /* [E] receiver i, non-decreasing */
  const float* shift;      /* [E,3] periodic image shift, or NULL */
  const int32_t* dst_ptr;  /* [N+1] from so2conv_graph_prepare */
  const int32_t* src_perm; /* [E]   from so2conv_graph_prepare */
  const int32_t* src_ptr;  /* [N+1] from so2conv_graph_prepare */
} so2conv_graph;

/* Incoming-edge CSR over receivers (Appendix B.3) and the stable grouping of
 * edges by sender used by the source-side sums of the backward (Eq.(4)).
 * dst_ptr[n] = first edge with dst >= n; src_perm = edge ids sorted stably by
 * src; src_ptr[n] = first position in src_perm with src >= n. err_word
 * (device int, caller-zeroed, may be NULL) gets bits OR-ed in: 1 src out of
 * range, 2 dst out of range, 4 dst decreasing. */
size_t so2conv_graph_workspace_bytes(int32_t n_nodes, int64_t n_edges);
int so2conv_graph_prepare(int32_t n_nodes, int64_t n_edges, const int32_t* src, const int32_t* dst,
                          int32_t* dst_ptr, int32_t* src_perm, int32_t* src_ptr, int32_t* err_word, void* ws,
                          size_t ws_bytes, void* stream);

/* Workspace and saved state.
 * The operator and its derivatives are sums over edges, so every call
 * processes the edges in contiguous chunks whose size the library picks from
 * ws_bytes (one chunk when the workspace is large enough); node outputs are
 * accumulated across chunks in a fixed order, so results do not depend on the
 * chunk size beyond float rounding of that order.
 *   so2conv_saved_bytes: the per-edge forward state (about 56 KB per edge at
 *     lmax 4, C 128 in float32; 41 KB with bfloat16 operands) that
 *     so2conv_fwd writes into `saved` and bwd/dbwd read.
 *   so2conv_workspace_bytes(stage): workspace for one chunk covering all edges
 *     when `saved` is used (stage 0 forward, 1 backward, 2 double backward).
 *   so2conv_chunked_workspace_bytes(stage, chunk_edges): workspace when `saved`
 *     is NULL and chunks of chunk_edges edges recompute the forward state
 *     (bounded memory; backward stages then redo the forward products).
 * Both include the float32 copies of the node arrays of a bfloat16 call, so
 * they depend on n_nodes. */
size_t so2conv_workspace_bytes(const so2conv_cfg* cfg, int32_t n_nodes, int64_t n_edges, int stage);
size_t so2conv_chunked_workspace_bytes(const so2conv_cfg* cfg, int32_t n_nodes, int64_t n_edges, int stage,
                                       int64_t chunk_edges);
size_t so2conv_saved_bytes(const so2conv_cfg* cfg, int64_t n_edges);
/* so2conv_saved_bwd_bytes: the backward's per-edge cotangents of the two
 * linears' outputs and of the first linear's input (Zbar, Ubar, Tbar; 40 KB
 * per edge at lmax 4, C 128 in float32, 34 KB with bfloat16 operands) that
 * so2conv_bwd writes into `saved_bwd` and so2conv_dbwd reads. In force training (Appendix A.3,
 * Eq.(3)) the double backward follows the backward with the same gy; its
 * reverse pass carries gy back through the tangent copy of the forward, and
 * those cotangents depend only on gy and the forward state, so they equal
 * the backward's. With them the double backward runs each linear's
 * data-gradient product on E rows instead of 2E. */
size_t so2conv_saved_bwd_bytes(const so2conv_cfg* cfg, int64_t n_edges);

/* Forward: y [N,d,C]. `saved` (may be NULL) receives the state needed by
 * so2conv_bwd / so2conv_dbwd for the same inputs. */
int so2conv_fwd(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos, const float* rbf,
                const float* env, const void* w_rad, const void* const* w1, const void* const* w2, void* y,
                void* saved, void* ws, size_t ws_bytes, void* stream);

/* so2conv_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * inputs and output y as so2conv_fwd with saved = NULL (no per-edge state is
 * kept; the forward runs in edge chunks that recompute it). The workspace is
 * a fixed 256 MiB device array inside the library, one per GPU, held until
 * the process ends; the call allocates nothing and synchronises nothing.
 * Returns SO2_EWORKSPACE (with a message naming the bytes needed) when a
 * 1024-edge chunk of this configuration does not fit in 256 MiB (for example
 * bfloat16 calls with many nodes, whose float32 node copies live in the
 * workspace); other errors as so2conv_fwd. Every call on one GPU uses that
 * GPU's one array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. */
int so2conv_fwd_noalloc(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos,
                        const float* rbf, const float* env, const void* w_rad, const void* const* w1,
                        const void* const* w2, void* y, void* stream);

/* Backward (vector-Jacobian product with cotangent gy, Section 3.3): gx, gpos,
 * grbf, genv, gw_rad, gw1[m], gw2[m] and gedge = dL/dv_e (for virials). `saved`
 * comes from so2conv_fwd on the same inputs, or is NULL (the forward state is
 * recomputed chunk by chunk). gw1/gw2 may be NULL, or hold NULL entries.
 * saved_bwd (may be NULL; so2conv_saved_bwd_bytes) receives the cotangents
 * a later so2conv_dbwd with the same inputs and gy can reuse. */
int so2conv_bwd(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos, const float* rbf,
                const float* env, const void* w_rad, const void* const* w1, const void* const* w2, const void* saved,
                const void* gy, void* gx, float* gpos, float* grbf, float* genv, void* gw_rad, void* const* gw1,
                void* const* gw2, float* gedge, void* saved_bwd, void* ws, size_t ws_bytes, void* stream);

/* Double backward: derivatives of
 *   L = <px, gx> + <ppos, gpos> + <pedge, gedge> + <prbf, grbf> + <penv, genv> + <pw, gw>
 * (the backward's outputs paired with directions; NULL direction = zero) with
 * respect to gy (ggy = the forward's directional derivative, Eq.(5)), x (gx2),
 * pos (gpos2 [N,3] float32, through the frames and their rotation rates;
 * rbf is an input, so its dependence on positions is the caller's chain
 * rule through grbf2), rbf (grbf2), env (genv2), w_rad, w1, w2. Any output may be NULL;
 * gpos2 costs a further pass over the rotation's generator rows. */
int so2conv_dbwd(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos, const float* rbf,
                 const float* env, const void* w_rad, const void* const* w1, const void* const* w2, const void* saved,
                 const void* gy, const void* px, const float* ppos, const float* pedge, const float* prbf,
                 const float* penv, const void* pw_rad, const void* const* pw1, const void* const* pw2, void* ggy,
                 void* gx2, float* gpos2, float* grbf2, float* genv2, void* gw_rad2, void* const* gw1_2,
                 void* const* gw2_2, const void* saved_bwd, void* ws, size_t ws_bytes, void* stream);

/* Test hook: the first linear's m-major input T (rotation on gather,
 * Appendix B.1) [E, q*2C], block |m| = 0..M: block 0 columns (l, c_in), block
 * m columns [+m (l = m..L, c_in) | -m (l = m..L, c_in)], with the pinned edge
 * frame rows (z >= 0, k = 1/(1+z): (1-x^2k, -xyk, -x), (-xyk, 1-y^2k, -y),
 * (x, y, z); z < 0, k = 1/(1-z): (1-x^2k, -xyk, x), (xyk, y^2k-1, -y), (x, y, z)).
 * T_out has the call's dtype (the stored GEMM operand). Workspace: E*(L+1)*2C
 * floats, plus N*d*C + n_rbf*(L+1)*2C floats for a bfloat16 call (each
 * rounded up to 256 bytes). */
int so2conv_debug_rotate_gather(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos,
                                const float* rbf, const void* w_rad, void* T_out, void* ws, size_t ws_bytes,
                                void* stream);

/* ---- Mixture of linear experts (Appendix C.1, Implementation: UMA's edge
 * projections use system-dependent mixtures of linear experts; Table 2: 64
 * experts for UMA). A batch of S systems: system s owns the receiver-sorted
 * edges [sys_edge_ptr[s], sys_edge_ptr[s+1]) (a structure's nodes form one
 * range, so its incoming edges are contiguous) and float32 coefficients
 * coef[s][0..K). Every edge of system s uses
 *   W1_m(s) = sum_k coef[s][k] W1_m^(k),   W2_m(s) = sum_k coef[s][k] W2_m^(k)
 * for every order m in place of the plain operator's w1[m], w2[m]; w_rad is
 * shared. Expert stacks: w1e[m] is [K][rows][cols] of the plain w1[m] layout
 * (same for w2e, their gradients and directions), in cfg->dtype. The per-order
 * products run as one grouped GEMM over (system, order) problems; weight
 * gradients are per system (split-K over its edges, fixed order), then
 *   gw1e[m][k] = sum_s coef[s][k] gW1_m(s),  gcoef[s][k] = sum_m <W1_m^(k), gW1_m(s)> + (same for W2).
 * The double backward takes directions pw1e, pw2e, pcoef (NULL = zero) as
 * the plain one takes pw1, pw2, and returns gw1e_2, gw2e_2, gcoef2 (the
 * first-order per-system gradients it then needs cost one more weight-gradient
 * product per linear). Every other argument, output and error is as in
 * so2conv_fwd/bwd/dbwd; a graph without edges gives zero gradients.
 * sys_edge_ptr is a HOST array [S+1] with p[0] = 0, p[S] = n_edges,
 * non-decreasing (empty systems allowed); n_systems in [1, 65536]; n_experts a
 * multiple of 4 in [4, 1024]; errors SO2_EINVAL / SO2_EUNSUPPORTED otherwise.
 * Workspace: so2mole_workspace_bytes(stage, chunk_edges): chunk_edges = 0
 * sizes one chunk over all edges that uses `saved` (as so2conv_workspace_bytes);
 * chunk_edges > 0 sizes chunks of that many edges that recompute the forward
 * state when `saved` is NULL (as so2conv_chunked_workspace_bytes).
 * saved_bwd (may be NULL; so2conv_saved_bwd_bytes) as in so2conv_bwd/dbwd: the
 * backward's cotangents, per system formed with that system's merged weights
 * in both calls. */
typedef struct {
  int32_t n_systems;
  int32_t n_experts;
  const int64_t* sys_edge_ptr;
} so2mole_cfg;
size_t so2mole_workspace_bytes(const so2conv_cfg* cfg, const so2mole_cfg* mole, int32_t n_nodes, int64_t n_edges,
                               int stage, int64_t chunk_edges);
int so2mole_fwd(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* mole, const void* x,
                const float* pos, const float* rbf, const float* env, const void* w_rad, const void* const* w1e,
                const void* const* w2e, const float* coef, void* y, void* saved, void* ws, size_t ws_bytes,
                void* stream);
int so2mole_bwd(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* mole, const void* x,
                const float* pos, const float* rbf, const float* env, const void* w_rad, const void* const* w1e,
                const void* const* w2e, const float* coef, const void* saved, const void* gy, void* gx, float* gpos,
                float* grbf, float* genv, void* gw_rad, void* const* gw1e, void* const* gw2e, float* gcoef,
                float* gedge, void* saved_bwd, void* ws, size_t ws_bytes, void* stream);
int so2mole_dbwd(const so2conv_cfg* cfg, const so2conv_graph* g, const so2mole_cfg* mole, const void* x,
                 const float* pos, const float* rbf, const float* env, const void* w_rad, const void* const* w1e,
                 const void* const* w2e, const float* coef, const void* saved, const void* gy, const void* px,
                 const float* ppos, const float* pedge, const float* prbf, const float* penv, const void* pw_rad,
                 const void* const* pw1e, const void* const* pw2e, const float* pcoef, void* ggy, void* gx2,
                 float* gpos2, float* grbf2, float* genv2, void* gw_rad2, void* const* gw1e_2, void* const* gw2e_2,
                 float* gcoef2, const void* saved_bwd, void* ws, size_t ws_bytes, void* stream);

/* ---- Node-to-node spherical projection with fused channel maps (Appendix B.4,
 * spherical activations). Per node i with coefficient rows X_i^(l) = x[i][l^2..(l+1)^2)
 * (n_l x c_in):
 *   U_i = sum_l G_l (X_i^(l) B_l),  B_l = W_l A        (= [sum_l G_l X_i^(l) W_l] A)
 * G: [n_grid, (L+1)^2] float32, column block l = the degree-l basis at the
 * grid points (caller-supplied; any matrix). W: [L+1, c_in, c_h], A: [c_h, c_out],
 * x: [N, (L+1)^2, c_in], U: [N, n_grid, c_out]; float32 only. The library forms
 * B_l once (never the c_h-wide coefficient or grid arrays), runs X B on the
 * matrix cores and applies G per node. Backward: gx = (G^T gU) B^T per degree,
 * gB = X^T (G^T gU), gW = gB A^T, gA = sum_l W_l^T gB_l. Double backward of
 * L = <px, gx> + <pW, gW> + <pA, gA> (NULL direction = zero): ggU, gx2, gW2, gA2.
 * Channel counts: multiples of 4 up to 1024; lmax <= 6; n_grid <= 65536.
 * Workspace from so2grid_workspace_bytes (stage 0 fwd, 1 bwd, 2 dbwd). */
typedef struct {
  int32_t lmax, c_in, c_h, c_out, n_grid, dtype, flags;
} so2grid_cfg;
size_t so2grid_workspace_bytes(const so2grid_cfg* cfg, int32_t n_nodes, int stage);
int so2grid_fwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* x, const float* G, const float* W,
                const float* A, float* U, void* ws, size_t ws_bytes, void* stream);
int so2grid_bwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* x, const float* G, const float* W,
                const float* A, const float* gU, float* gx, float* gW, float* gA, void* ws, size_t ws_bytes,
                void* stream);
int so2grid_dbwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* x, const float* G, const float* W,
                 const float* A, const float* gU, const float* px, const float* pW, const float* pA, float* ggU,
                 float* gx2, float* gW2, float* gA2, void* ws, size_t ws_bytes, void* stream);

/* Back-projection from the grid (TrimSO(2) page, Appendix B.4, Forward
 * computation, the second identity H_l (Y A_out) = (H_l Y) A_out): the grid
 * values after the nonlinearity return to coefficients,
 *   Z^(l) = H_l (Y A),  computed as (H_l Y) A,
 * so the [n_grid x c_out] product Y A is never formed per node. H
 * [(lmax+1)^2][n_grid] stacks the H_l (degree-l rows), a constant (no
 * gradient). Uses cfg->lmax, c_h (grid channels), c_out and n_grid; c_in is
 * not used (it must still be a valid channel count).
 * Arrays (device, float32, row-major): Y, gY, pY, gY2 [n_nodes][n_grid][c_h];
 * H [(lmax+1)^2][n_grid]; A, gA, pA, gA2 [c_h][c_out];
 * Z, gZ, ggZ [n_nodes][(lmax+1)^2][c_out].
 *   fwd : Z
 *   bwd : gY = H^T (gZ A^T), gA = sum over nodes (H Y)^T gZ (either may be NULL)
 *   dbwd: L = <pY, gY> + <pA, gA> (NULL direction = zero):
 *         ggZ = dL/dgZ = (H pY) A + (H Y) pA, gY2 = dL/dY = H^T (gZ pA^T),
 *         gA2 = dL/dA = sum over nodes (H pY)^T gZ (outputs may be NULL)
 * Workspace from so2grid_back_workspace_bytes (stage 0 fwd, 1 bwd, 2 dbwd).
 * Weight-map gradients sum over nodes in a fixed order (bitwise
 * reproducible); errors as for so2grid_fwd. */
size_t so2grid_back_workspace_bytes(const so2grid_cfg* cfg, int32_t n_nodes, int stage);
int so2grid_back_fwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* Y, const float* H, const float* A,
                     float* Z, void* ws, size_t ws_bytes, void* stream);
int so2grid_back_bwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* Y, const float* H, const float* A,
                     const float* gZ, float* gY, float* gA, void* ws, size_t ws_bytes, void* stream);
int so2grid_back_dbwd(const so2grid_cfg* cfg, int32_t n_nodes, const float* Y, const float* H, const float* A,
                      const float* gZ, const float* pY, const float* pA, float* ggZ, float* gY2, float* gA2,
                      void* ws, size_t ws_bytes, void* stream);

/* Spherical-grid SwiGLU activation on edges (SwiGLU-S2; TrimSO(2) page,
 * Table 2 and Appendix C.1 "Implementation": EquiformerV3's Edge -> Edge activation; Appendix
 * B.4: the degree-l basis evaluated at n_g grid points, the nonlinearity on
 * grid values). The pages name the activation without a formula; read here,
 * per edge e and channel c of q coefficient rows with a value half
 * (channels 0..C-1) and a gate half (C..2C-1):
 *   v = G u_v,  a = G u_g,  s = SiLU(a) * v,  z = P s
 * with G [n_grid][rows] (the basis of the retained rows at the grid points)
 * and P [rows][n_grid] (the projection back) supplied by the caller; both are
 * constants (no gradients for them).
 * Arrays (device, float32, row-major): U and pU, gU, gU2 [n_edges][rows][2C];
 * Z and gZ, ggZ [n_edges][rows][C]. rows in [1, 32], channels in
 * [1, 65536], n_grid in [1, 256] (G and P are staged in LDS as matrix-core
 * operands), else SO2_EUNSUPPORTED; NULL inputs or outputs are SO2_EINVAL (in
 * dbwd one of ggZ, gU2 may be NULL: not requested). No workspace;
 * n_edges == 0 is a no-op. Runs asynchronously on `stream`.
 *   fwd : Z
 *   bwd : gU = dZ/dU^T gZ
 *   dbwd: with L = <pU, gU>: ggZ = dL/dgZ (the forward's directional
 *         derivative along pU), gU2 = dL/dU */
typedef struct {
  int32_t rows, channels, n_grid, dtype /* SO2_F32 */, flags /* 0 */;
} so2s2_cfg;
int so2s2_fwd(const so2s2_cfg* cfg, int64_t n_edges, const float* U, const float* G, const float* P, float* Z,
              void* stream);
int so2s2_bwd(const so2s2_cfg* cfg, int64_t n_edges, const float* U, const float* G, const float* P,
              const float* gZ, float* gU, void* stream);
int so2s2_dbwd(const so2s2_cfg* cfg, int64_t n_edges, const float* U, const float* G, const float* P,
               const float* gZ, const float* pU, float* ggZ, float* gU2, void* stream);

/* Measurement hook for the per-order GEMMs (the dense products of Section
 * 3.1 and Eq.(1)). While enabled, every matrix-core GEMM launch is bracketed
 * by HIP events on the launching stream and its algorithmic flop count (2 M N K
 * summed over the launch's problems) and algorithmic bytes (each operand read
 * once, the output written once) are recorded. so2conv_profile_read
 * synchronises on the recorded events and returns the number of launches, the
 * summed event time (ms), flops and bytes for kind 0 (A B), 1 (A B^T),
 * 2 (A^T B, weight gradients) with float32 operands, 3 (A B^T) and 4 (A^T B)
 * with bfloat16 operands, 5 (A B), 6 (A B^T), 7 (A^T B) as complex float32
 * products of orders m >= 1 (flops: the three real products executed), or
 * -1 (all). Host-side state, process-wide. */
int so2conv_profile_enable(int on);
int so2conv_profile_reset(void);
int so2conv_profile_read(int kind, int64_t* launches, double* total_ms, double* total_flops, double* total_bytes);

/* Synchronises `stream` and reports the device-side validation word of the
 * current device left by the last call with SO2_DEBUG_CHECKS (each such call
 * clears it first): SO2_OK if clear, else SO2_EDEVICE with the failed checks in
 * so2conv_last_error() (bits: 1 src out of range, 2 dst out of range,
 * 4 dst decreasing, 8 zero-length edge, 16 non-finite input); the word is
 * cleared. */
int so2conv_debug_status(void* stream);

/* Copies the so(3) generator table the kernels use for the rotation torques
 * and rotation rates (Section 2's frame rotation, differentiated: G_k^(l) =
 * d/dt D^(l)(exp(t [e_k]_x)) at t = 0, k = x, y, z) to host memory `out`
 * (so2conv_generator_table(NULL, 0) floats: generator k's table at offset
 * k * (that count / 3), degree l = 0..6's (2l+1)^2 block row-major at offset
 * sum_{l' < l} (2l'+1)^2 within it, rows and columns in order m = -l..l;
 * the l = 0 block is the single zero). The table is evaluated when the
 * library is compiled; no GPU is needed. Returns the number of floats, or
 * SO2_EINVAL if out is non-NULL and n is smaller. */
int so2conv_generator_table(float* out, int64_t n);

/* message of the last failing call on this thread ("" if none) */
const char* so2conv_last_error(void);
/* 1 if (lmax, mmax) has compiled kernels */
int so2conv_supported(int32_t lmax, int32_t mmax);

#ifdef __cplusplus
}
#endif

#endif /* SO2CONV_H */
