"""Pins of the oracle's approximate inverse ("[7/7] Experimental GDN/KDA
approximate-inverse QAT", "What does this PR do?": an explicit Neumann
polynomial degree replaces the exact solve; the backward differentiates the
polynomial; "Testing": residual identities, degree validation, gradients of
the actual polynomial).

- Residual identity: (I + L) sum_{m<=d} (-L)^m = I - (-L)^(d+1) (the
  geometric series telescopes); (-L)^(d+1) comes from
  torch.linalg.matrix_power, not from the oracle's loop. A wrong sign, an
  off-by-one degree or a dropped beta fails it.
- Nilpotency: L is strictly lower triangular, so any degree >= n_c - 1 is the
  exact inverse, and the whole forward then equals the exact-solve forward.
- Degree 1 is (I - L) diag(beta), written out by hand.
- The backward equals central finite differences of the Neumann forward, and
  differs from the exact-solve gradient at low degree."""
import numpy as np
import pytest
import torch

from oracle import FMT_E4M3, chunked_bwd, chunked_fwd, wy_factor
from test_oracle_bwd import NAMES, _fd_directional, _loss, _upstream
from test_oracle_fwd import rand_case


def _chunk(seed, n=64, Dk=4, Z=3):
    """One chunk of Z streams; small Dk keeps k_i . k_j of order one and the
    gates stay near 0, so the powers of L stay large enough to tell
    neighbouring degrees apart ((-L)^32 is about 1e-11 here)."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((Z, n, Dk))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    g = -np.log1p(np.exp(rng.standard_normal((Z, n)) - 3.0))
    b = 1 / (1 + np.exp(-rng.standard_normal((Z, n))))
    return tuple(torch.from_numpy(x) for x in (K, g, b))


@pytest.mark.parametrize("d", [1, 3, 7, 15, 31])
def test_residual_identity(d):
    Kc, gc, bc = _chunk(10 + d)
    _, _, L, Td = wy_factor(Kc, gc, bc, solve_degree=d)
    n = L.shape[-1]
    eye = torch.eye(n, dtype=L.dtype).expand_as(L)
    Db = torch.diag_embed(bc)
    rem = torch.linalg.matrix_power(-L, d + 1)
    lhs = (eye + L) @ Td
    rhs = Db - rem @ Db
    scale = float(rhs.abs().max())
    tol = 1e-13 * max(scale, 1.0)
    assert float((lhs - rhs).abs().max()) <= tol
    # the remainder is well above the tolerance, so d +- 1 would fail the identity
    assert float((rem @ Db).abs().max()) > 10 * tol


@pytest.mark.parametrize("n,d", [(64, 63), (20, 31), (5, 7)])
def test_degree_at_least_n_minus_1_is_exact(n, d):
    Kc, gc, bc = _chunk(30 + n, n=n)
    _, _, L, Td = wy_factor(Kc, gc, bc, solve_degree=d)
    _, _, _, Tx = wy_factor(Kc, gc, bc)
    assert float(torch.linalg.matrix_power(L, n).abs().max()) == 0.0
    assert float((Td - Tx).abs().max()) <= 1e-10 * float(Tx.abs().max())


def test_degree_one_closed_form():
    Kc, gc, bc = _chunk(41, n=9, Dk=4, Z=1)
    _, _, L, T1 = wy_factor(Kc, gc, bc, solve_degree=1)
    Ln, bn = L[0].numpy(), bc[0].numpy()
    want = np.zeros((9, 9))
    for i in range(9):
        for j in range(9):
            want[i, j] = ((1.0 if i == j else 0.0) - Ln[i, j]) * bn[j]
    np.testing.assert_allclose(T1[0].numpy(), want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("qdq", [False, True])
def test_forward_at_degree_63_equals_exact(qdq):
    c = rand_case(61, B=2, T=150, Hqk=1, Hv=2, Dk=8, Dv=8)
    kw = dict(state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=8) if qdq else {}
    o1, h1 = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'], **kw)
    o2, h2 = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                         solve_degree=63, **kw)
    tol = 1e-6 if qdq else 1e-10     # QDQ on: an FP32 code may flip at a grid midpoint
    assert float((o1 - o2).norm() / o1.norm()) <= tol
    assert float((h1 - h2).norm() / h1.norm()) <= tol


def test_low_degree_changes_the_forward():
    c = rand_case(62, B=1, T=100, Hqk=1, Hv=2, Dk=4, Dv=4, shift=-2.0)
    o1, _ = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'])
    o3, _ = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                        solve_degree=3)
    assert float((o1 - o3).norm() / o1.norm()) > 1e-4


@pytest.mark.parametrize("d", [1, 3])
def test_backward_of_the_polynomial_matches_fd(d):
    c = rand_case(70 + d, lengths=[70, 9], Hqk=1, Hv=2, Dk=4, Dv=4, shift=-1.0)
    do, dht = _upstream(c, 5)
    scale = 0.6
    grads = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, do, dht,
                        c['h0'], c['cu_seqlens'], solve_degree=d)

    def f(cc):
        return _loss(*(x.numpy() for x in chunked_fwd(
            cc['q'], cc['k'], cc['v'], cc['g'], cc['beta'], scale, cc['h0'],
            cc['cu_seqlens'], solve_degree=d)), do, dht)
    _fd_directional(f, c, grads, np.random.default_rng(6))
    exact = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, do, dht,
                        c['h0'], c['cu_seqlens'])
    for name in ('k', 'beta', 'g'):
        a, b = grads['d' + name], exact['d' + name]
        assert float((a - b).norm() / b.norm()) > 1e-4, name


def test_negative_degree_is_rejected():
    c = rand_case(80, T=10)
    with pytest.raises(ValueError):
        chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'], solve_degree=-1)


def test_names_cover_every_input():
    assert set(NAMES) == {'q', 'k', 'v', 'g', 'beta', 'h0'}
