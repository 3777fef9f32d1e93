"""The order pairing of Eq.(1) through the C ABI, against values worked out by
hand (TrimSO(2) page, Section 2 Eq.(1) and Appendix A.2; "+" is order +m).

Same construction as the oracle's pairing pins: one edge 0 -> 1 along +z
(identity frame), radial scale 1, zero order-0 block of the first linear
(every gate 1/2), a single nonzero input row and weight entry; the second
linear passes the order through. With w = 0.75 the expected values are
exact in float32 and bfloat16; the tolerance only absorbs the rounding of the
identity Wigner rows.
"""
import numpy as np
import pytest
import torch

import so_graph_convolution_amd as K

L, M, C, NRBF = 2, 2, 16, 4
W = 0.75


def row(l, m):
    return l * l + l + m


def _weights():
    s1, s2 = K.weight_shapes(K.SO2Config(L, M, C, NRBF))
    return [np.zeros(s, np.float32) for s in s1], [np.zeros(s, np.float32) for s in s2]


def _run(x_row, w1, w2, dtype):
    dev = torch.device("cuda:0")
    ft = torch.bfloat16 if dtype == "bf16" else torch.float32
    cfg = K.SO2Config(L, M, C, NRBF, dtype)
    t = lambda a, dt=torch.float32: torch.tensor(np.ascontiguousarray(a), dtype=dt, device=dev)  # noqa: E731
    g = K.so2conv_graph_prepare(2, t([0], torch.int32), t([1], torch.int32), t(np.zeros((1, 3))))
    x = np.zeros((2, (L + 1) ** 2, C), np.float32)
    x[0, x_row, 0] = 1.0
    rbf = np.zeros((1, NRBF), np.float32)
    rbf[0, 0] = 1.0
    w_rad = np.zeros((NRBF, (L + 1) * 2 * C), np.float32)
    w_rad[0] = 1.0
    y, _ = K.so2conv_fwd(cfg, g, t(x, ft), t([[0, 0, 1.5], [0, 0, 0]]), t(rbf), t(w_rad, ft),
                         [t(w, ft) for w in w1], [t(w, ft) for w in w2])
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def _expect(l, m, val):
    e = np.zeros((2, (L + 1) ** 2, C), np.float32)
    e[1, row(l, m), 1] = val
    return e


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m", [1, 2])
def test_first_linear_cross_weight(m, dtype):
    """Only W_m1[(l=m, c_in=0), (l=m, c=1)] = w. Input on (m, +m): u_- = Q10 + Q01 = +w,
    y = +w/2 on (m, -m). Input on (m, -m): u_+ = Q00 - Q11 = -w, y = -w/2 on (m, +m)."""
    w1, w2 = _weights()
    n = L - m + 1
    w1[m][0, n * C + 1] = W
    w2[m][:, :n * C] = np.eye(n * C)
    tol = 4e-3 if dtype == "bf16" else 1e-6
    np.testing.assert_allclose(_run(row(m, m), w1, w2, dtype), _expect(m, -m, W / 2), rtol=0, atol=tol)
    np.testing.assert_allclose(_run(row(m, -m), w1, w2, dtype), _expect(m, m, -W / 2), rtol=0, atol=tol)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m", [1, 2])
def test_second_linear_cross_weight(m, dtype):
    """First linear passes (l=m, c_in=0) -> (l=m, c=0); only W2's W_m1[(l=m, c=0), (l=m, c=1)] = w.
    Input on (m, +m): t_- = +w/2 on (m, -m); on (m, -m): t_+ = -w/2 on (m, +m)."""
    w1, w2 = _weights()
    n = L - m + 1
    w1[m][0, 0] = 1.0
    w2[m][0, n * C + 1] = W
    tol = 4e-3 if dtype == "bf16" else 1e-6
    np.testing.assert_allclose(_run(row(m, m), w1, w2, dtype), _expect(m, -m, W / 2), rtol=0, atol=tol)
    np.testing.assert_allclose(_run(row(m, -m), w1, w2, dtype), _expect(m, m, -W / 2), rtol=0, atol=tol)
