"""CPU oracle for the fused edgewise SO(2) convolution -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module. The product path never calls it.

What it computes (TrimSO(2): Fast and Memory-Efficient Training of Equivariant
Interatomic Potentials, Section 2 Eq.(1)-(2), Appendix A.1-A.2, B.1-B.3):

  for every directed edge e = (j -> i), j = src[e], i = dst[e]:
    v_e   = pos[j] - pos[i] + shift_e,  rhat_e = v_e/|v_e|       (A.1 edge geometry)
    R_e   = edge-frame rotation with R_e rhat_e = zhat              (A.2 frame alignment)
    D_e   = real Wigner-D blocks of R_e                             (A.1 rotation law)
    a_e   = [x_j | x_i]  (source channels first, width 2C)
    s_e   = rbf_e W_rad, one scale per (degree, input channel)      (C.1 radial scaling)
    T_e   = s_e * (D_e a_e), retained orders |m| <= min(l, M)       (B.1 GEMM input)
    first SO(2) linear per order, Eq.(1):
        m = 0 : [u_0 | gamma] = T^(0) W1[0]
        m > 0 : [Q00 Q01; Q10 Q11] = [T_+; T_-][W_m0 W_m1],
                u_+ = Q00 - Q11, u_- = Q10 + Q01
    gate (B.2): l = 0 -> SiLU(u); l >= 1 -> sigmoid(gamma_l) * u for all retained m
      or, with grid tables (G, P) (EquiformerV3's spherical-grid SwiGLU, Appendix
      C.1 "Implementation" and Table 2): the first linear has 2C output channels
      per retained row (value half, then gate half) and the activation is
      s2act_oracle.forward over each edge's retained rows in degree-major order
    second SO(2) linear (same structure, no gate columns) -> t_e
    y_i  += sum_e (J D_e)^T t_e                                     (B.3 inverse rotation)

Backward and double backward are torch.autograd derivatives of this plain
definition (the pages' Eq.(3)-(5) describe these derivatives; the oracle
does not hand-derive them).

Conventions fixed here because the pages leave them open (each is a reading,
stated once more in the repository's design notes):
  * real spherical harmonics, orthonormal, orders m=-l..l, no Condon-Shortley
    phase, so Y_1 = sqrt(3/4pi) (y, z, x);
  * Wigner-D defined by Y(R u) = D(R) Y(u), computed here by exact quadrature
    over the sphere (Gauss-Legendre in cos(theta) x uniform in phi);
  * edge frame: the minimal rotation taking rhat to +z for rhat_z >= 0, and
    for rhat_z < 0 the rotation whose rows are given in `edge_frame` below;
  * order pairing: "+" is order +m (cos type), "-" is order -m (sin type);
  * gate scalars are L*C extra m=0 output columns of the first linear,
    ordered (l = 1..L, c).

Everything runs in float64. The operator and all its derivatives are sums of
per-edge terms, so edges are processed in chunks and the chunk results added;
this is exact and is the only departure from a single pass.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import s2act_oracle

__all__ = ["real_sh", "wigner_d", "edge_frame", "forward", "backward", "double_backward",
           "retained_orders", "q_count", "k_count", "OracleInputs", "to_oracle_inputs", "grid_rows",
           "activation_input"]

DT = torch.float64


# ----------------------------------------------------------------------------- counts
def retained_orders(l: int, M: int):
    """Retained orders of degree l: m with |m| <= min(l, M) (B.1 compact rotation blocks)."""
    k = min(l, M)
    return list(range(-k, k + 1))


def q_count(L: int, M: int) -> int:
    """q_{L,M}: number of retained (l, m) rows (A.2)."""
    return sum(len(retained_orders(l, M)) for l in range(L + 1))


def k_count(L: int, M: int) -> int:
    """K_{L,M}: compact rotation entries per edge (B.1)."""
    return sum(len(retained_orders(l, M)) * (2 * l + 1) for l in range(L + 1))


# ----------------------------------------------------------------------------- harmonics
def _legendre_deriv_coeffs(l: int, m: int) -> np.ndarray:
    """Power-basis coefficients of d^m/dz^m P_l(z)."""
    c = np.polynomial.legendre.leg2poly(np.eye(l + 1)[l])
    return np.polynomial.polynomial.polyder(c, m) if m > 0 else c


def real_sh(l: int, u: torch.Tensor) -> torch.Tensor:
    """Real orthonormal spherical harmonics of degree l at unit vectors u [..., 3].

    Y_{l,0}  = N_l0 P_l(z)
    Y_{l,m}  = sqrt(2) N_lm (d^m P_l/dz^m)(z) Re((x + i y)^m)      m > 0
    Y_{l,-m} = sqrt(2) N_lm (d^m P_l/dz^m)(z) Im((x + i y)^m)      m > 0
    N_lm = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!). (For unit u, (x+iy)^m =
    sin^m(theta) e^{i m phi}, so this is P_l^m(cos theta) cos/sin(m phi)
    without the Condon-Shortley phase.) Returns [..., 2l+1], order m=-l..l.
    """
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    out = [None] * (2 * l + 1)
    cr, ci = torch.ones_like(x), torch.zeros_like(x)     # (x + i y)^0
    for m in range(0, l + 1):
        if m > 0:
            cr, ci = cr * x - ci * y, cr * y + ci * x
        dc = _legendre_deriv_coeffs(l, m)
        q = torch.zeros_like(z)
        for k in range(len(dc) - 1, -1, -1):               # Horner
            q = q * z + float(dc[k])
        n = math.sqrt((2 * l + 1) / (4 * math.pi) * math.factorial(l - m) / math.factorial(l + m))
        if m == 0:
            out[l] = n * q
        else:
            out[l + m] = math.sqrt(2.0) * n * q * cr
            out[l - m] = math.sqrt(2.0) * n * q * ci
    return torch.stack(out, dim=-1)


def _sphere_grid(l: int):
    """Quadrature exact for polynomials of degree <= 2l on the unit sphere:
    Gauss-Legendre with l+1 nodes in cos(theta) times 2l+1 uniform nodes in phi."""
    zs, wz = np.polynomial.legendre.leggauss(l + 1)
    nphi = 2 * l + 1
    phi = 2 * np.pi * np.arange(nphi) / nphi
    Z, P = np.meshgrid(zs, phi, indexing="ij")
    W = np.repeat(wz[:, None], nphi, axis=1) * (2 * np.pi / nphi)
    st = np.sqrt(1 - Z * Z)
    u = np.stack([st * np.cos(P), st * np.sin(P), Z], -1).reshape(-1, 3)
    return torch.tensor(u, dtype=DT), torch.tensor(W.reshape(-1), dtype=DT)


_GRID = {}


def wigner_d(l: int, R: torch.Tensor) -> torch.Tensor:
    """Real Wigner-D block of degree l for rotations R [..., 3, 3]:
    D[m, n] = integral over the sphere of Y_m(R u) Y_n(u) du, evaluated exactly
    by quadrature, so that Y(R u) = D(R) Y(u). Returns [..., 2l+1, 2l+1]."""
    if l not in _GRID:
        u, w = _sphere_grid(l)
        _GRID[l] = (u, w, real_sh(l, u))
    u, w, Yu = _GRID[l]
    Ru = torch.einsum("...ab,gb->...ga", R, u)               # [..., G, 3]
    YRu = real_sh(l, Ru)                                     # [..., G, n]
    return torch.einsum("...gm,gn,g->...mn", YRu, Yu, w)


def edge_frame(rhat: torch.Tensor) -> torch.Tensor:
    """Rotation R with R rhat = +z (the edge frame of A.2), rows given explicitly.

    z >= 0, k = 1/(1+z): rows (1-x^2k, -xyk, -x), (-xyk, 1-y^2k, -y), (x, y, z)
    z <  0, k = 1/(1-z): rows (1-x^2k, -xyk,  x), ( xyk, y^2k-1, -y), (x, y, z)
    """
    x, y, z = rhat[..., 0], rhat[..., 1], rhat[..., 2]
    pos = z >= 0
    zero = torch.zeros_like(z)
    # each branch only sees its own half-line of z, so the unused branch stays finite
    k = torch.where(pos, 1.0 / (1.0 + torch.where(pos, z, zero)), 1.0 / (1.0 - torch.where(pos, zero, z)))
    sgn = torch.where(pos, torch.ones_like(z), -torch.ones_like(z))
    r0 = torch.stack([1 - x * x * k, -x * y * k, -sgn * x], -1)
    r1 = torch.stack([-sgn * x * y * k, sgn * (1 - y * y * k), -y], -1)
    r2 = torch.stack([x, y, z], -1)
    return torch.stack([r0, r1, r2], -2)


def _rot_z(psi: torch.Tensor) -> torch.Tensor:
    c, s = torch.cos(psi), torch.sin(psi)
    o, zr = torch.ones_like(psi), torch.zeros_like(psi)
    return torch.stack([torch.stack([c, -s, zr], -1), torch.stack([s, c, zr], -1),
                        torch.stack([zr, zr, o], -1)], -2)


# ----------------------------------------------------------------------------- inputs
class OracleInputs:
    """float64 torch views of one workload (indices stay int64). `env` (None,
    [E] or [E, H]) weights each message before the receiver sum (TrimSO(2)
    page, Appendix C.1 Implementation: eSEN and UMA sum messages with their
    cutoff envelopes, one weight per edge; EquiformerV3 applies attention
    weights before aggregation, one weight per edge and head, head h covering
    channels [h C/H, (h+1) C/H)). `grid` (None or (G, P)) selects the
    spherical-grid SwiGLU activation instead of the gate (Appendix C.1
    "Implementation": EquiformerV3's Edge -> Edge activation)."""

    def __init__(self, lmax, mmax, channels, pos, x, src, dst, shift, rbf, w_rad, w1, w2, env=None, grid=None):
        self.L, self.M, self.C = lmax, mmax, channels
        self.pos, self.x, self.rbf, self.w_rad = pos, x, rbf, w_rad
        self.w1, self.w2 = list(w1), list(w2)
        self.src, self.dst, self.shift = src, dst, shift
        self.env = env
        # spherical-grid SwiGLU activation (None: the gate): constant tables
        # (G [n_g, q], P [q, n_g]) over the retained rows in degree-major order
        self.grid = grid

    def leaves(self):
        return [self.x, self.pos, self.rbf, self.w_rad] + self.w1 + self.w2 + \
            ([self.env] if self.env is not None else [])


def to_oracle_inputs(d: dict, requires_grad=False) -> OracleInputs:
    cfg = d["cfg"]

    def t(a):
        return torch.tensor(np.asarray(a, dtype=np.float64), dtype=DT, requires_grad=requires_grad)

    grid = None
    if d.get("grid_G") is not None:
        grid = tuple(torch.tensor(np.asarray(d[k], np.float64), dtype=DT) for k in ("grid_G", "grid_P"))
    return OracleInputs(cfg.lmax, cfg.mmax, cfg.channels, t(d["pos"]), t(d["x"]),
                        torch.tensor(d["src"], dtype=torch.int64), torch.tensor(d["dst"], dtype=torch.int64),
                        torch.tensor(np.asarray(d["shift"], np.float64), dtype=DT), t(d["rbf"]),
                        t(d["w_rad"]), [t(w) for w in d["w1"]], [t(w) for w in d["w2"]],
                        t(d["env"]) if d.get("env") is not None else None, grid)


# ----------------------------------------------------------------------------- forward
def _so2_linear(Tp, Tm, W):
    """Eq.(1): [Q00 Q01; Q10 Q11] = [T_+; T_-][W_m0 W_m1]; u_+ = Q00 - Q11, u_- = Q10 + Q01."""
    h = W.shape[1] // 2
    Q = torch.cat([Tp, Tm], 0) @ W
    E = Tp.shape[0]
    Q00, Q01 = Q[:E, :h], Q[:E, h:]
    Q10, Q11 = Q[E:, :h], Q[E:, h:]
    return Q00 - Q11, Q10 + Q01


def _rotated_inputs(inp: OracleInputs, e_idx, D):
    """Rotation on gather (B.1): T^(l)[m, c] = s[l, c] * sum_m' D[m, m'] a[m', c], all rows m."""
    L, C = inp.L, inp.C
    src, dst = inp.src[e_idx], inp.dst[e_idx]
    E = e_idx.shape[0]
    s = (inp.rbf[e_idx] @ inp.w_rad).view(E, L + 1, 2 * C)
    T = []
    for l in range(L + 1):
        blk = slice(l * l, (l + 1) * (l + 1))
        a = torch.cat([inp.x[src, blk, :], inp.x[dst, blk, :]], -1)         # [E, n, 2C]
        T.append(s[:, l, None, :] * (D[l] @ a))
    return T


def rotated_inputs(inp: OracleInputs, e_idx=None):
    """Per degree l, [E', 2l+1, 2C]: the first linear's input before order selection,
    in the pinned edge frame (used to check the rotation-on-gather stage alone)."""
    if e_idx is None:
        e_idx = torch.arange(inp.src.shape[0])
    v = inp.pos[inp.src[e_idx]] - inp.pos[inp.dst[e_idx]] + inp.shift[e_idx]
    R = edge_frame(v / torch.linalg.norm(v, dim=-1, keepdim=True))
    D = [wigner_d(l, R) for l in range(inp.L + 1)]
    return _rotated_inputs(inp, e_idx, D)


def grid_rows(L: int, M: int):
    """The retained rows (l, m) in degree-major order: the row order of the
    spherical-grid activation's tables."""
    return [(l, m) for l in range(L + 1) for m in retained_orders(l, M)]


def _first_linear(inp: OracleInputs, T):
    """Eq.(1) per order on the rotated inputs T (list over l of [E, 2l+1, 2C]):
    u[(l, m)] of width C (gate; gamma[l] the gate columns of degree l >= 1) or
    2C (spherical-grid SwiGLU: value channels, then gate channels; gamma None)."""
    L, M, C = inp.L, inp.M, inp.C
    hw = C if inp.grid is None else 2 * C
    u = {}
    T0 = torch.cat([T[l][:, l, :] for l in range(L + 1)], -1)
    o0 = T0 @ inp.w1[0]
    for l in range(L + 1):
        u[(l, 0)] = o0[:, l * hw:(l + 1) * hw]
    gamma = None
    if inp.grid is None:
        gamma = {l: o0[:, (L + 1) * C + (l - 1) * C:(L + 1) * C + l * C] for l in range(1, L + 1)}
    for m in range(1, M + 1):
        Tp = torch.cat([T[l][:, l + m, :] for l in range(m, L + 1)], -1)
        Tm = torch.cat([T[l][:, l - m, :] for l in range(m, L + 1)], -1)
        up, um = _so2_linear(Tp, Tm, inp.w1[m])
        for k, l in enumerate(range(m, L + 1)):
            u[(l, m)] = up[:, k * hw:(k + 1) * hw]
            u[(l, -m)] = um[:, k * hw:(k + 1) * hw]
    return u, gamma


def activation_input(inp: OracleInputs, e_idx=None):
    """The first linear's output of the edges e_idx as [E', q, width] rows in
    degree-major order (grid_rows): what the Edge -> Edge activation reads."""
    if e_idx is None:
        e_idx = torch.arange(inp.src.shape[0])
    v = inp.pos[inp.src[e_idx]] - inp.pos[inp.dst[e_idx]] + inp.shift[e_idx]
    R = edge_frame(v / torch.linalg.norm(v, dim=-1, keepdim=True))
    D = [wigner_d(l, R) for l in range(inp.L + 1)]
    u, _ = _first_linear(inp, _rotated_inputs(inp, e_idx, D))
    return torch.stack([u[r] for r in grid_rows(inp.L, inp.M)], 1)


def edge_messages(inp: OracleInputs, e_idx: torch.Tensor, roll: torch.Tensor | None = None):
    """Global-frame messages of the edges e_idx: list over l of [E', 2l+1, C].

    `roll` (optional, [E']) replaces R_e by R_z(roll) R_e; the result must not
    depend on it (any frame with R rhat = z is valid)."""
    L, M, C = inp.L, inp.M, inp.C
    src, dst = inp.src[e_idx], inp.dst[e_idx]
    E = e_idx.shape[0]
    v = inp.pos[src] - inp.pos[dst] + inp.shift[e_idx]
    rhat = v / torch.linalg.norm(v, dim=-1, keepdim=True)
    R = edge_frame(rhat)
    if roll is not None:
        R = _rot_z(roll) @ R
    D = [wigner_d(l, R) for l in range(L + 1)]
    T = _rotated_inputs(inp, e_idx, D)
    u, gamma = _first_linear(inp, T)
    if inp.grid is None:
        # gated activation
        z = {}
        for (l, m), val in u.items():
            z[(l, m)] = torch.nn.functional.silu(val) if l == 0 else torch.sigmoid(gamma[l]) * val
    else:
        # spherical-grid SwiGLU over each edge's retained rows
        rows = grid_rows(L, M)
        Z = s2act_oracle.forward(torch.stack([u[r] for r in rows], 1), *inp.grid)
        z = {r: Z[:, k, :] for k, r in enumerate(rows)}
    # second SO(2) linear
    t = {}
    Z0 = torch.cat([z[(l, 0)] for l in range(L + 1)], -1)
    o0 = Z0 @ inp.w2[0]
    for l in range(L + 1):
        t[(l, 0)] = o0[:, l * C:(l + 1) * C]
    for m in range(1, M + 1):
        Zp = torch.cat([z[(l, m)] for l in range(m, L + 1)], -1)
        Zm = torch.cat([z[(l, -m)] for l in range(m, L + 1)], -1)
        tp, tm = _so2_linear(Zp, Zm, inp.w2[m])
        for k, l in enumerate(range(m, L + 1)):
            t[(l, m)] = tp[:, k * C:(k + 1) * C]
            t[(l, -m)] = tm[:, k * C:(k + 1) * C]
    # inverse rotation: msg^(l)[m', c] = sum_{m retained} D[m, m'] t[m, c]
    msgs = []
    for l in range(L + 1):
        ms = retained_orders(l, M)
        Dr = torch.stack([D[l][:, l + m, :] for m in ms], 1)                  # [E, q_l, n_l]
        tl = torch.stack([t[(l, m)] for m in ms], 1)                          # [E, q_l, C]
        msgs.append(Dr.transpose(1, 2) @ tl)
    return msgs


def _chunks(E, chunk, edges=None):
    idx = torch.arange(E) if edges is None else torch.as_tensor(edges, dtype=torch.int64)
    for a in range(0, idx.shape[0], chunk):
        yield idx[a:a + chunk]


def _scatter(inp: OracleInputs, e_idx, msgs, n_nodes):
    d = (inp.L + 1) ** 2
    y = torch.zeros(n_nodes, d, inp.C, dtype=DT)
    dst = inp.dst[e_idx]
    w = None
    if inp.env is not None:
        w = inp.env[e_idx]
        w = w[:, None] if w.dim() == 1 else w.repeat_interleave(inp.C // w.shape[1], dim=1)   # [E', C]
    for l, msg in enumerate(msgs):
        if w is not None:
            msg = msg * w[:, None, :]
        y[:, l * l:(l + 1) * (l + 1), :] = y[:, l * l:(l + 1) * (l + 1), :].index_add(0, dst, msg)
    return y


def forward(inp: OracleInputs, chunk=4096, edges=None, roll=None):
    """y[N, d, C] = sum over edges of inverse-rotated messages at the target node.
    `edges` restricts the sum to a subset of edges (exact for nodes all of whose
    incoming edges are in the subset)."""
    N = inp.x.shape[0]
    E = inp.src.shape[0]
    y = torch.zeros(N, (inp.L + 1) ** 2, inp.C, dtype=DT)
    for e_idx in _chunks(E, chunk, edges):
        r = None if roll is None else roll[e_idx]
        y = y + _scatter(inp, e_idx, edge_messages(inp, e_idx, r), N)
    return y


def _grads(out, wrt, grad_out, create_graph=False):
    g = torch.autograd.grad(out, wrt, grad_out, create_graph=create_graph, allow_unused=True)
    return [torch.zeros_like(w) if gi is None else gi for gi, w in zip(g, wrt)]


def backward(inp: OracleInputs, gy: torch.Tensor, chunk=4096, edges=None, with_edge_grad=False):
    """Vector-Jacobian product of `forward` with cotangent gy.

    Returns dict with gx, gpos, grbf, gw_rad, gw1 (list), gw2 (list), genv (if
    the inputs carry an envelope) and, if requested, gedge [E,3] = dL/dv_e
    (derivative with respect to each edge vector)."""
    leaves = [t.detach().requires_grad_(True) for t in inp.leaves()]
    nw = len(inp.w1)
    has_env = inp.env is not None
    inp2 = OracleInputs(inp.L, inp.M, inp.C, leaves[1], leaves[0], inp.src, inp.dst,
                        inp.shift.detach().clone().requires_grad_(with_edge_grad), leaves[2], leaves[3],
                        leaves[4:4 + nw], leaves[4 + nw:4 + 2 * nw], leaves[4 + 2 * nw] if has_env else None,
                        inp.grid)
    N = inp.x.shape[0]
    acc = [torch.zeros_like(t) for t in leaves]
    gedge = torch.zeros_like(inp.shift) if with_edge_grad else None
    for e_idx in _chunks(inp.src.shape[0], chunk, edges):
        y = _scatter(inp2, e_idx, edge_messages(inp2, e_idx), N)
        wrt = leaves + ([inp2.shift] if with_edge_grad else [])
        g = _grads(y, wrt, gy)
        for k in range(len(leaves)):
            acc[k] += g[k]
        if with_edge_grad:
            gedge += g[-1]
    out = dict(gx=acc[0], gpos=acc[1], grbf=acc[2], gw_rad=acc[3],
               gw1=acc[4:4 + nw], gw2=acc[4 + nw:4 + 2 * nw])
    if has_env:
        out["genv"] = acc[4 + 2 * nw]
    if with_edge_grad:
        out["gedge"] = gedge
    return out


def double_backward(inp: OracleInputs, gy: torch.Tensor, px=None, ppos=None, prbf=None,
                    pw_rad=None, pw1=None, pw2=None, pedge=None, penv=None, chunk=2048, edges=None):
    """Derivatives of L = <px, gx> + <ppos, gpos> + <prbf, grbf> + <pW, gW> (+ <pedge, gedge>)
    (+ <penv, genv>), where (gx, gpos, grbf, gW, gedge, genv) = backward(inp, gy), with
    respect to gy (-> ggy), x, pos, rbf, W_rad, W1, W2 and the envelope (-> genv, if
    the inputs carry one). None directions are zero."""
    leaves = [t.detach().requires_grad_(True) for t in inp.leaves()]
    gyl = gy.detach().clone().requires_grad_(True)
    nw = len(inp.w1)
    has_env = inp.env is not None
    shift = inp.shift.detach().clone().requires_grad_(pedge is not None)
    inp2 = OracleInputs(inp.L, inp.M, inp.C, leaves[1], leaves[0], inp.src, inp.dst, shift,
                        leaves[2], leaves[3], leaves[4:4 + nw], leaves[4 + nw:4 + 2 * nw],
                        leaves[4 + 2 * nw] if has_env else None, inp.grid)
    dirs = [px, ppos, prbf, pw_rad] + list(pw1 or [None] * nw) + list(pw2 or [None] * nw) + \
        ([penv] if has_env else [])
    N = inp.x.shape[0]
    acc = [torch.zeros_like(t) for t in leaves]
    accgy = torch.zeros_like(gy)
    for e_idx in _chunks(inp.src.shape[0], chunk, edges):
        y = _scatter(inp2, e_idx, edge_messages(inp2, e_idx), N)
        wrt = leaves + ([shift] if pedge is not None else [])
        g = _grads(y, wrt, gyl, create_graph=True)
        Lval = torch.zeros((), dtype=DT)
        for gi, p in zip(g, dirs + ([pedge] if pedge is not None else [])):
            if p is not None:
                Lval = Lval + (gi * p).sum()
        if not Lval.requires_grad:
            continue
        h = _grads(Lval, leaves + [gyl], None)
        for k in range(len(leaves)):
            acc[k] += h[k]
        accgy += h[-1]
    out = dict(ggy=accgy, gx=acc[0], gpos=acc[1], grbf=acc[2], gw_rad=acc[3],
               gw1=acc[4:4 + nw], gw2=acc[4 + nw:4 + 2 * nw])
    if has_env:
        out["genv"] = acc[4 + 2 * nw]
    return out
