"""Seeded synthetic inputs for the fused SO(2) convolution.

This module is shared by the CPU oracle, the tests and the benchmark. It holds
no arithmetic of the convolution itself: it draws atom positions in a periodic
box, builds the periodic radius graph, evaluates a Gaussian radial basis on the
edge lengths (a caller-side input of the operator) and draws node features,
weights, incoming gradients and differentiation directions.

Workloads follow the TrimSO(2) page (Appendix C.1, Tables 2-3: lmax, mmax,
channel width, number of radial basis functions, 6 A cutoff) and the operator
sweep recipe of Appendix C.4.2 (N nodes, each picking K distinct targets).
The pages train on OMat24 batches; those are not available, so uniform random
packings of the stated density stand in for them.

Conventions:
  * edge e runs from source j = src[e] to target i = dst[e]; the periodic
    image shift is shift[e] = n_e * box (Cartesian), so the edge vector is
    pos[j] - pos[i] + shift[e] (TrimSO(2) page, Appendix A.1 edge geometry).
  * edges are sorted by (dst, src, image index) with image index
    (nx+1)*9 + (ny+1)*3 + (nz+1), nx,ny,nz in {-1,0,1}.
  * node features are [N, (L+1)^2, C], degree-major, orders m=-l..l.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Config", "CONFIGS", "make_config", "radius_graph_pbc", "gaussian_rbf",
           "random_targets_graph", "make_inputs", "weight_shapes", "swiglu_s2_inputs"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_atoms: int
    box: float            # cubic box edge (A); 0 means a non-periodic sweep graph
    rc: float             # cutoff radius (A)
    lmax: int
    mmax: int
    channels: int         # C (node channels); the message input width is 2C
    n_rbf: int
    dtype: str            # "f32" or "bf16" (features and weights)
    weight_init: str      # "glorot" or "normal_1_over_c"
    seed: int
    n_clusters: int = 0   # dense clusters (Large config)
    cluster_size: int = 0
    cluster_radius: float = 0.0
    min_dist: float = 0.0  # rejection-sample positions until min pair distance >= this
    k_targets: int = 0     # >0: sweep graph, each node picks k distinct targets
    act: str = "gate"      # Edge -> Edge activation: "gate" or "swiglu_s2"
    n_grid: int = 0        # swiglu_s2: grid points of the activation's tables


CONFIGS = {
    # Tiny: FD-checked; 5 A cutoff in an 8 A box gives multi-image edges.
    "T": Config("T", 32, 8.0, 5.0, 2, 2, 16, 8, "f32", "glorot", 0, min_dist=0.5),
    # eSEN-like small.
    "S": Config("S", 2000, (2000 / 0.1) ** (1 / 3), 6.0, 2, 2, 128, 64, "f32", "normal_1_over_c", 1),
    # UMA/eSEN-like medium (the headline workload).
    "M": Config("M", 10000, (10000 / 0.08) ** (1 / 3), 6.0, 4, 2, 128, 64, "f32", "normal_1_over_c", 2),
    # EquiformerV3-like high degree, bf16 features and weights.
    "H": Config("H", 20000, (20000 / 0.1) ** (1 / 3), 5.0, 6, 2, 128, 64, "bf16", "normal_1_over_c", 3),
    # Large single-GPU system with 5% of atoms in dense clusters.
    "X": Config("X", 100000, 100.0, 6.0, 4, 2, 256, 64, "bf16", "normal_1_over_c", 4,
                n_clusters=25, cluster_size=200, cluster_radius=3.0),
    # Context workloads sized like the pages' operator measurements.
    "P1": Config("P1", 399, 20.0, 6.0, 4, 2, 128, 64, "f32", "normal_1_over_c", 5),
    "P2": Config("P2", 512, 20.0, 0.0, 4, 2, 128, 64, "f32", "normal_1_over_c", 6, k_targets=64),
}


def make_config(name: str, **overrides) -> Config:
    """Return a named config, optionally with fields replaced (for small parity cases)."""
    return dataclasses.replace(CONFIGS[name], **overrides) if overrides else CONFIGS[name]


def weight_shapes(lmax: int, mmax: int, channels: int, act: str = "gate"):
    """Shapes of W1[m], W2[m] for m = 0..mmax (input width 2C, output width C).

    act "gate" (hidden width C plus gate columns):
      W1[0]: [(L+1)*2C, (L+1)*C + L*C]  rows (l, c_in); columns (l, c) then gate columns (l=1..L, c)
      W1[m]: [(L-m+1)*2C, 2*(L-m+1)*C]  = [W_{m,0} | W_{m,1}]
    act "swiglu_s2" (hidden width 2C per row: value channels, then gate channels):
      W1[0]: [(L+1)*2C, (L+1)*2C]
      W1[m]: [(L-m+1)*2C, 2*(L-m+1)*2C]
    W2[0]: [(L+1)*C, (L+1)*C]
    W2[m]: [(L-m+1)*C, 2*(L-m+1)*C]
    """
    L, M, C = lmax, mmax, channels
    hw = 2 * C if act == "swiglu_s2" else C
    w1 = [((L + 1) * 2 * C, (L + 1) * hw + (0 if act == "swiglu_s2" else L * C))]
    w2 = [((L + 1) * C, (L + 1) * C)]
    for m in range(1, M + 1):
        nl = L - m + 1
        w1.append((nl * 2 * C, 2 * nl * hw))
        w2.append((nl * C, 2 * nl * C))
    return w1, w2


# ----------------------------------------------------------------------------- graphs

def _image_code(n):
    return (n[..., 0] + 1) * 9 + (n[..., 1] + 1) * 3 + (n[..., 2] + 1)


def _canonical_sort(src, dst, img):
    order = np.lexsort((img, src, dst))
    return order


def radius_graph_pbc(pos: np.ndarray, box: float, rc: float):
    """Directed periodic radius graph (cubic box), every image within rc is an edge.

    Returns src, dst (int32), shift (float32 [E,3], Cartesian) sorted by
    (dst, src, image). Self-edges are excluded only for the zero image.
    Requires rc < box (images n in {-1,0,1}^3 suffice).
    """
    assert rc < box
    pos = np.asarray(pos, dtype=np.float64)
    N = pos.shape[0]
    nc = int(box // rc)
    src_l, dst_l, img_l = [], [], []
    if nc < 3:
        # brute force over the 27 images
        offs = np.array([(a, b, c) for a in (-1, 0, 1) for b in (-1, 0, 1) for c in (-1, 0, 1)])
        for n in offs:
            d = pos[None, :, :] + n * box - pos[:, None, :]   # [i, j, 3] = pos_j + n*box - pos_i
            r2 = (d * d).sum(-1)
            mask = r2 < rc * rc
            if not n.any():
                np.fill_diagonal(mask, False)
            ii, jj = np.nonzero(mask)
            dst_l.append(ii); src_l.append(jj)
            img_l.append(np.broadcast_to(n, (len(ii), 3)))
    else:
        cell = np.floor(pos / box * nc).astype(np.int64) % nc            # [N,3]
        cid = (cell[:, 0] * nc + cell[:, 1]) * nc + cell[:, 2]
        order = np.argsort(cid, kind="stable")
        counts = np.bincount(cid, minlength=nc ** 3)
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
        for a in (-1, 0, 1):
            for b in (-1, 0, 1):
                for c in (-1, 0, 1):
                    raw = cell + np.array([a, b, c])                     # neighbour cell, unwrapped
                    n = np.floor_divide(raw, nc)                          # image of that cell
                    wrapped = raw - n * nc
                    ncid = (wrapped[:, 0] * nc + wrapped[:, 1]) * nc + wrapped[:, 2]
                    cnt = counts[ncid]
                    i_rep = np.repeat(np.arange(N), cnt)
                    first = np.repeat(starts[ncid], cnt)
                    within = np.arange(cnt.sum()) - np.repeat(np.cumsum(cnt) - cnt, cnt)
                    j = order[first + within]
                    nn = n[i_rep]
                    d = pos[j] + nn * box - pos[i_rep]
                    r2 = (d * d).sum(-1)
                    keep = r2 < rc * rc
                    keep &= ~((j == i_rep) & (~nn.any(axis=1)))
                    dst_l.append(i_rep[keep]); src_l.append(j[keep]); img_l.append(nn[keep])
    src = np.concatenate(src_l).astype(np.int64)
    dst = np.concatenate(dst_l).astype(np.int64)
    img = np.concatenate(img_l).astype(np.int64)
    o = _canonical_sort(src, dst, _image_code(img))
    src, dst, img = src[o], dst[o], img[o]
    shift = (img * box).astype(np.float32)
    return src.astype(np.int32), dst.astype(np.int32), shift


def random_targets_graph(rng: np.random.Generator, n: int, k: int):
    """Sweep graph: each node picks k distinct targets uniformly among the other nodes
    (TrimSO(2) page, Appendix C.4.2). Returns src, dst sorted by (dst, src); no shifts."""
    src = np.repeat(np.arange(n), k)
    dst = np.empty(n * k, dtype=np.int64)
    for j in range(n):
        t = rng.choice(n - 1, size=k, replace=False)
        t[t >= j] += 1
        dst[j * k:(j + 1) * k] = t
    o = np.lexsort((src, dst))
    return src[o].astype(np.int32), dst[o].astype(np.int32), np.zeros((n * k, 3), np.float32)


def gaussian_rbf(rho: np.ndarray, n_rbf: int, rc: float) -> np.ndarray:
    """Gaussian radial basis phi_k(rho) = exp(-(rho - mu_k)^2 / (2 sigma^2)),
    mu_k = k rc/(n-1), sigma = rc/(n-1). Computed in float64, returned float32."""
    rho = np.asarray(rho, dtype=np.float64)
    mu = np.linspace(0.0, rc, n_rbf)
    sig = rc / (n_rbf - 1)
    return np.exp(-((rho[:, None] - mu[None, :]) ** 2) / (2 * sig * sig)).astype(np.float32)


def _positions(rng, cfg: Config):
    N, box = cfg.n_atoms, cfg.box
    if cfg.n_clusters:
        centres = rng.random((cfg.n_clusters, 3)) * box
        pts = []
        for cc in centres:
            # uniform in a ball: direction x radius^(1/3)
            d = rng.normal(size=(cfg.cluster_size, 3))
            d /= np.linalg.norm(d, axis=1, keepdims=True)
            r = cfg.cluster_radius * rng.random(cfg.cluster_size) ** (1 / 3)
            pts.append(np.mod(cc + d * r[:, None], box))
        rest = rng.random((N - cfg.n_clusters * cfg.cluster_size, 3)) * box
        pos = np.concatenate(pts + [rest], 0)
    else:
        while True:
            pos = rng.random((N, 3)) * box
            if cfg.min_dist <= 0:
                break
            d = pos[None] - pos[:, None]
            d -= box * np.round(d / box)
            r = np.sqrt((d * d).sum(-1)) + np.eye(N) * 1e9
            if r.min() >= cfg.min_dist:
                break
    pos = pos.astype(np.float32)
    # keep positions strictly inside [0, box) after rounding to float32
    pos = np.where(pos >= np.float32(box), np.float32(0.0), pos)
    return pos


def _weights(rng, cfg: Config):
    w1s, w2s = weight_shapes(cfg.lmax, cfg.mmax, cfg.channels)

    def draw(shape):
        if cfg.weight_init == "glorot":
            a = math.sqrt(6.0 / (shape[0] + shape[1]))
            return rng.uniform(-a, a, size=shape)
        return rng.normal(0.0, 1.0 / math.sqrt(cfg.channels), size=shape)

    w_rad = rng.normal(0.0, 1.0 / math.sqrt(cfg.n_rbf), size=(cfg.n_rbf, (cfg.lmax + 1) * 2 * cfg.channels))
    w1 = [draw(s) for s in w1s]
    w2 = [draw(s) for s in w2s]
    return w_rad, w1, w2


def cosine_envelope(d: dict) -> np.ndarray:
    """Caller-side cutoff envelope per edge, 0.5 (cos(pi rho / rc) + 1) of the edge
    length (a smooth cutoff used as synthetic envelope input; float32)."""
    v = d["pos"][d["src"]].astype(np.float64) - d["pos"][d["dst"]] + d["shift"]
    rho = np.sqrt((v * v).sum(1))
    return (0.5 * (np.cos(np.pi * rho / d["cfg"].rc) + 1.0)).astype(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def make_inputs(cfg: Config, with_directions=True):
    """Draw every input of one workload. Draw order: positions (and cluster
    centres), x, W_rad, W1[0..M], W2[0..M], gy, px, ppos, prbf.

    All floating arrays are float32 (bf16 configs hold bf16-representable
    float32 values for x, weights, gy and px)."""
    rng = np.random.default_rng(cfg.seed)
    L, C = cfg.lmax, cfg.channels
    d = (L + 1) ** 2
    if cfg.k_targets:
        pos = (rng.random((cfg.n_atoms, 3)) * cfg.box).astype(np.float32)
        src, dst, shift = random_targets_graph(rng, cfg.n_atoms, cfg.k_targets)
        rc = float(cfg.box) * math.sqrt(3.0)
    else:
        pos = _positions(rng, cfg)
        src, dst, shift = radius_graph_pbc(pos, cfg.box, cfg.rc)
        rc = cfg.rc
    v = pos[src].astype(np.float64) - pos[dst] + shift
    rho = np.sqrt((v * v).sum(1))
    rbf = gaussian_rbf(rho, cfg.n_rbf, rc)
    x = rng.normal(size=(cfg.n_atoms, d, C)).astype(np.float32)
    w_rad, w1, w2 = _weights(rng, cfg)
    out = dict(cfg=cfg, pos=pos, src=src, dst=dst, shift=shift, rbf=rbf, x=x,
               w_rad=w_rad.astype(np.float32),
               w1=[w.astype(np.float32) for w in w1], w2=[w.astype(np.float32) for w in w2])
    if cfg.act == "swiglu_s2":
        out.update(swiglu_s2_inputs(cfg))
    # with_directions: True (all), False (none) or a tuple naming a prefix of
    # ("gy", "px", "ppos", "prbf"); draws stop after the last one requested, so a
    # prefix draws exactly the same values as the full set.
    if with_directions:
        E = len(src)
        names = ("gy", "px", "ppos", "prbf")
        want = names if with_directions is True else tuple(with_directions)
        last = max(names.index(k) for k in want)
        shapes = {"gy": (cfg.n_atoms, d, C), "px": (cfg.n_atoms, d, C), "ppos": (cfg.n_atoms, 3),
                  "prbf": (E, cfg.n_rbf)}
        for k in names[:last + 1]:
            out[k] = rng.normal(size=shapes[k]).astype(np.float32)
    if cfg.dtype == "bf16":
        for k in ("x", "gy", "px", "w_rad"):
            if k in out:
                out[k] = round_bf16(out[k])
        out["w1"] = [round_bf16(w) for w in out["w1"]]
        out["w2"] = [round_bf16(w) for w in out["w2"]]
    return out


def swiglu_s2_inputs(cfg: Config) -> dict:
    """First-linear weights of the spherical-grid SwiGLU activation (value and
    gate halves per retained row, drawn like the plain weights) and synthetic
    grid tables grid_G [n_grid, q] ~ N(0, 1/q), grid_P [q, n_grid] ~ N(0, 1/n_grid)
    of the size of a grid with n_grid points (the values of the tables do not
    change the work; a model evaluates the retained harmonics at its grid).
    Drawn from a stream of their own, so every other input equals the gated
    workload's."""
    rng = np.random.default_rng(30_000 + cfg.seed)
    L, M, C = cfg.lmax, cfg.mmax, cfg.channels
    q = (L + 1) * (2 * M + 1) - M * (M + 1)
    ng = cfg.n_grid
    if ng < 1:
        raise ValueError("swiglu_s2 needs n_grid >= 1")
    w1s, _ = weight_shapes(L, M, C, "swiglu_s2")

    def draw(shape):
        if cfg.weight_init == "glorot":
            a = math.sqrt(6.0 / (shape[0] + shape[1]))
            return rng.uniform(-a, a, size=shape)
        return rng.normal(0.0, 1.0 / math.sqrt(C), size=shape)
    w1 = [draw(s).astype(np.float32) for s in w1s]
    G = (rng.normal(size=(ng, q)) / math.sqrt(q)).astype(np.float32)
    P = (rng.normal(size=(q, ng)) / math.sqrt(ng)).astype(np.float32)
    return dict(w1=w1, grid_G=G, grid_P=P)


def mixture_inputs(d: dict, n_systems: int, n_experts: int, seed: int = 0, empty_system: bool = False,
                   bf16: bool = False) -> dict:
    """Inputs of the mixture of linear experts (TrimSO(2) page, Appendix C.1,
    UMA's system-dependent mixtures; Table 2: 64 experts): the batch's nodes
    split into n_systems contiguous ranges (one more, empty, system when
    empty_system), their receiver-sorted edge offsets sys_edge_ptr [S+1],
    expert stacks w1e[m] / w2e[m] [K, rows, cols] drawn like the plain weights,
    coefficients coef [S, K] (a softmax of standard normal logits per system;
    the page does not say how UMA forms them, they are an input here) and
    directions pcoef, pw1e, pw2e (standard normal). bf16: experts and their
    directions rounded to bfloat16 values."""
    cfg = d["cfg"]
    rng = np.random.default_rng(10_000 + seed)
    N = cfg.n_atoms
    bounds = [round(N * s / n_systems) for s in range(n_systems + 1)]
    if empty_system:
        bounds = bounds[:1] + bounds[1:2] + bounds[1:]          # system 1 has no nodes
    sys_edge_ptr = np.searchsorted(np.asarray(d["dst"]), bounds).astype(np.int64)
    sys_edge_ptr[0], sys_edge_ptr[-1] = 0, len(d["dst"])
    S = len(bounds) - 1
    w1s, w2s = weight_shapes(cfg.lmax, cfg.mmax, cfg.channels)

    def stack(shapes, scale):
        return [rng.normal(0.0, scale, size=(n_experts,) + s).astype(np.float32) for s in shapes]
    sc = 1.0 / math.sqrt(cfg.channels)
    w1e, w2e = stack(w1s, sc), stack(w2s, sc)
    logits = rng.normal(size=(S, n_experts))
    coef = np.exp(logits - logits.max(1, keepdims=True))
    coef = (coef / coef.sum(1, keepdims=True)).astype(np.float32)
    pcoef = rng.normal(size=(S, n_experts)).astype(np.float32)
    pw1e, pw2e = stack(w1s, 1.0), stack(w2s, 1.0)
    if bf16:
        w1e, w2e = [round_bf16(w) for w in w1e], [round_bf16(w) for w in w2e]
        pw1e, pw2e = [round_bf16(w) for w in pw1e], [round_bf16(w) for w in pw2e]
    return dict(sys_edge_ptr=sys_edge_ptr, w1e=w1e, w2e=w2e, coef=coef, pcoef=pcoef, pw1e=pw1e, pw2e=pw2e)


def attention_weights(d: dict, heads: int, seed: int = 0) -> np.ndarray:
    """Synthetic per-head attention weights [E, heads] (float32): standard
    normal logits per (edge, head), normalised by a softmax over each
    receiver's incoming edges (the weights EquiformerV3 applies before
    aggregation, TrimSO(2) page Appendix C.1; how the model forms the logits
    is outside the operator, they are an input here)."""
    rng = np.random.default_rng(20_000 + seed)
    dst = np.asarray(d["dst"])
    E = len(dst)
    logits = rng.normal(size=(E, heads))
    out = np.zeros((E, heads))
    if E:
        starts = np.flatnonzero(np.r_[True, dst[1:] != dst[:-1]])
        ends = np.r_[starts[1:], E]
        for a, b in zip(starts, ends):
            z = np.exp(logits[a:b] - logits[a:b].max(0))
            out[a:b] = z / z.sum(0)
    return out.astype(np.float32)
