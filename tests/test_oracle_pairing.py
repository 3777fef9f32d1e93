"""Operator-level pins of the order pairing of the SO(2) linears.

TrimSO(2) page, Section 2 Eq.(1) (restated in Appendix A.2): for order m > 0
the products [Q00 Q01; Q10 Q11] = [T_+; T_-][W_m0 W_m1] are recombined as
u_+ = Q00 - Q11 and u_- = Q10 + Q01. Reading used throughout: "+" is order +m
(the cos-type real harmonic), "-" is order -m (sin-type); with the real
harmonics Y_1 = sqrt(3/4pi) (y, z, x) the l = 1 rows are (m=-1, 0, +1) =
(y, z, x).

Each case here is worked out by hand, not by calling the oracle's own pieces:
one edge 0 -> 1 along +z, so the edge frame and every Wigner block are the
identity; the radial scale is 1 on every (l, channel); the first linear's
order-0 block is zero, so every gate is sigmoid(0) = 1/2; one input row and
one weight entry are nonzero. The expected node output is then a single
number with a sign fixed by Eq.(1). The conjugated pairing
(u_+ = Q00 + Q11, u_- = Q10 - Q01, which is also what swapping the +m and -m
rows consistently in both linears produces) flips that sign, so it fails
here while it passes every invariant and finite-difference pin.
"""
import numpy as np
import pytest
import torch

from oracle import so2conv_oracle as O

DT = torch.float64
L, M, C = 2, 2, 2            # widths kept tiny; two channels to catch channel mix-ups
W = 0.7                      # the one nonzero weight


def row(l, m):
    """Row of (l, m) in a node feature [d, C] (degree blocks, m = -l..l)."""
    return l * l + l + m


def _edge_along_z():
    pos = torch.tensor([[0.0, 0.0, 1.5], [0.0, 0.0, 0.0]], dtype=DT)   # v = pos[src] - pos[dst] = +1.5 z
    src, dst = torch.tensor([0]), torch.tensor([1])
    shift = torch.zeros(1, 3, dtype=DT)
    rbf = torch.ones(1, 1, dtype=DT)
    w_rad = torch.ones(1, (L + 1) * 2 * C, dtype=DT)                    # s = 1 for every (l, c_in)
    return pos, src, dst, shift, rbf, w_rad


def _zero_weights():
    w1 = [torch.zeros((L + 1) * 2 * C, (L + 1) * C + L * C, dtype=DT)]
    w2 = [torch.zeros((L + 1) * C, (L + 1) * C, dtype=DT)]
    for m in range(1, M + 1):
        n = L - m + 1
        w1.append(torch.zeros(n * 2 * C, 2 * n * C, dtype=DT))
        w2.append(torch.zeros(n * C, 2 * n * C, dtype=DT))
    return w1, w2


def _w1_entry(w1, m, l_in, c_in, part, l_out, c_out, val):
    """W1[m] rows are (l = m..L, c_in < 2C); columns [W_m0 | W_m1], each (l = m..L, c < C)."""
    n = L - m + 1
    w1[m][(l_in - m) * 2 * C + c_in, part * n * C + (l_out - m) * C + c_out] = val


def _w2_entry(w2, m, l_in, c_in, part, l_out, c_out, val):
    n = L - m + 1
    w2[m][(l_in - m) * C + c_in, part * n * C + (l_out - m) * C + c_out] = val


def _w2_pass_through(w2, m):
    """Second linear of order m as the identity: W_m0 = I, W_m1 = 0, so t_+ = z_+ and t_- = z_-."""
    n = L - m + 1
    w2[m][:, :n * C] = torch.eye(n * C, dtype=DT)


def _run(x_row, w1, w2):
    pos, src, dst, shift, rbf, w_rad = _edge_along_z()
    x = torch.zeros(2, (L + 1) ** 2, C, dtype=DT)
    x[0, x_row, 0] = 1.0                                               # source node, channel 0
    inp = O.OracleInputs(L, M, C, pos, x, src, dst, shift, rbf, w_rad, w1, w2)
    return O.forward(inp)


def test_frame_of_an_edge_along_z_is_identity():
    R = O.edge_frame(torch.tensor([[0.0, 0.0, 1.0]], dtype=DT))[0]
    assert torch.allclose(R, torch.eye(3, dtype=DT), atol=0)
    for l in range(L + 1):
        assert torch.allclose(O.wigner_d(l, R), torch.eye(2 * l + 1, dtype=DT), atol=1e-13)


@pytest.mark.parametrize("m", [1, 2])
def test_first_linear_cross_weight_on_plus_row(m):
    """x on (l=m, +m); only W_m1[(l=m, c_in=0), (l=m, c=1)] = w.
    T_+ = e, T_- = 0, so Q01 = w and u_- = Q10 + Q01 = +w on (l=m, c=1);
    gate 1/2; second linear passes through: y_dst[(m, -m), 1] = +w/2."""
    w1, w2 = _zero_weights()
    _w1_entry(w1, m, m, 0, 1, m, 1, W)
    _w2_pass_through(w2, m)
    y = _run(row(m, m), w1, w2)
    expect = torch.zeros_like(y)
    expect[1, row(m, -m), 1] = W / 2
    assert torch.allclose(y, expect, atol=1e-13), y[1]


@pytest.mark.parametrize("m", [1, 2])
def test_first_linear_cross_weight_on_minus_row(m):
    """x on (l=m, -m); the same single W_m1 entry. T_- = e, so Q11 = w and
    u_+ = Q00 - Q11 = -w: y_dst[(m, +m), 1] = -w/2."""
    w1, w2 = _zero_weights()
    _w1_entry(w1, m, m, 0, 1, m, 1, W)
    _w2_pass_through(w2, m)
    y = _run(row(m, -m), w1, w2)
    expect = torch.zeros_like(y)
    expect[1, row(m, m), 1] = -W / 2
    assert torch.allclose(y, expect, atol=1e-13), y[1]


@pytest.mark.parametrize("m", [1, 2])
def test_first_linear_diagonal_weight_keeps_the_row(m):
    """Only W_m0[(l=L, c_in=0), (l=m, c=1)] = w, x on (L, -m): Q10 = w, so u_- = +w
    on (l=m, c=1) (degrees mix inside an order, rows keep their sign)."""
    w1, w2 = _zero_weights()
    _w1_entry(w1, m, L, 0, 0, m, 1, W)
    _w2_pass_through(w2, m)
    y = _run(row(L, -m), w1, w2)
    expect = torch.zeros_like(y)
    expect[1, row(m, -m), 1] = W / 2
    assert torch.allclose(y, expect, atol=1e-13), y[1]


@pytest.mark.parametrize("m", [1, 2])
def test_second_linear_cross_weight(m):
    """First linear passes (l=m, c_in=0) -> (l=m, c=0) through W_m0; the second has
    only W_m1[(l=m, c=0), (l=m, c=1)] = w. x on (m, +m): z_+ = 1/2, so
    t_- = Q'10 + Q'01 = +w/2 on (l=m, c=1); x on (m, -m): z_- = 1/2, so
    t_+ = Q'00 - Q'11 = -w/2."""
    w1, w2 = _zero_weights()
    _w1_entry(w1, m, m, 0, 0, m, 0, 1.0)
    _w2_entry(w2, m, m, 0, 1, m, 1, W)
    y = _run(row(m, m), w1, w2)
    expect = torch.zeros_like(y)
    expect[1, row(m, -m), 1] = W / 2
    assert torch.allclose(y, expect, atol=1e-13), y[1]
    y = _run(row(m, -m), w1, w2)
    expect = torch.zeros_like(y)
    expect[1, row(m, m), 1] = -W / 2
    assert torch.allclose(y, expect, atol=1e-13), y[1]


def test_cross_weight_is_a_quarter_turn_about_the_edge():
    """Geometric form of the same sign: with W_10 = 0 and W_11 = I on l = 1, the
    first linear multiplies the order-1 pair by i, a +90 degree turn about the
    edge axis (+z here), taking the x component (row m=+1) to the y component
    (row m=-1) and y to -x."""
    w1, w2 = _zero_weights()
    for c in range(C):
        _w1_entry(w1, 1, 1, c, 1, 1, c, 1.0)
    _w2_pass_through(w2, 1)
    pos, src, dst, shift, rbf, w_rad = _edge_along_z()
    vec = np.array([0.3, -0.8, 0.5])                                    # (x, y, z) of channel 0
    x = torch.zeros(2, (L + 1) ** 2, C, dtype=DT)
    x[0, row(1, 1), 0], x[0, row(1, -1), 0], x[0, row(1, 0), 0] = vec[0], vec[1], vec[2]
    y = O.forward(O.OracleInputs(L, M, C, pos, x, src, dst, shift, rbf, w_rad, w1, w2))
    turned = np.array([-vec[1], vec[0]])                                # R_z(+90) (x, y) = (-y, x)
    got = np.array([y[1, row(1, 1), 0].item(), y[1, row(1, -1), 0].item()])
    np.testing.assert_allclose(got, turned / 2, atol=1e-13)
    assert abs(y[1, row(1, 0), 0].item()) < 1e-13                      # order 0 untouched (W1[0] = 0)
