"""Pins of the oracle's forward: closed forms of the token recurrence, the
chunked form equal to the token recurrence (QDQ off and state QDQ), the exact
solve residual, chunk-size independence, and an independent token-loop
re-derivation of the chunk with W and state QDQ.

Sources: "[1/4] GDN state/W QAT foundation", "What does this PR do?" (exact
recurrent and chunk references; state and W sites; exact triangular solve;
chunk size 64) and "[2/4] GDN/KDA decode QAT with INT8 recurrent state",
"Testing" (257-token trajectories, nonzero initial states, grouped heads,
packed tails, all state scale widths)."""
import numpy as np
import pytest
import torch

from oracle import FMT_E4M3, FMT_INT8, FMT_OFF, chunked_fwd, recurrent_fwd, wy_factor
from oracle.qdq import qdq32


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rand_case(seed, B=1, T=40, Hqk=1, Hv=2, Dk=8, Dv=8, lengths=None, h0=True,
              shift=0.0, retention=False):
    rng = np.random.default_rng(seed)
    if lengths is not None:
        B, T = 1, sum(lengths)
    q = rng.standard_normal((B, T, Hqk, Dk))
    k = rng.standard_normal((B, T, Hqk, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, Dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, Hv))))
    if retention:
        g = np.log(rng.uniform(0.9, 0.999, (B, T, Hv)))
    else:
        g = -np.log1p(np.exp(rng.standard_normal((B, T, Hv)) + shift))
    N = B if lengths is None else len(lengths)
    hz = 0.5 * rng.standard_normal((N, Hv, Dk, Dv)) if h0 else None
    cu = None if lengths is None else np.concatenate([[0], np.cumsum(lengths)])
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=hz, cu_seqlens=cu)


# ---------------------------------------------------------------- closed forms

def _both(c, scale=0.7, **kw):
    o1, h1 = recurrent_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, c['h0'],
                           c['cu_seqlens'], **kw)
    o2, h2 = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, c['h0'],
                         c['cu_seqlens'], **kw)
    return (o1, h1), (o2.numpy(), h2.numpy())


def test_closed_form_zero_beta_is_pure_decay():
    c = rand_case(10, T=70, Hv=2, Dk=6, Dv=5)
    c['beta'][:] = 0.0
    G = np.cumsum(c['g'][0], axis=0)                      # [T, H]
    want_o = 0.7 * np.exp(G)[:, :, None] * np.einsum('hkv,thk->thv', c['h0'][0],
                                                      np.repeat(c['q'][0], 2, axis=1))
    want_h = np.exp(G[-1])[:, None, None] * c['h0'][0]
    for o, h in _both(c):
        assert rel(o[0], want_o) < 1e-13 and rel(h[0], want_h) < 1e-13


def test_closed_form_orthonormal_keys_is_linear_attention():
    Dk, T = 80, 70
    c = rand_case(11, T=T, Hqk=1, Hv=1, Dk=Dk, Dv=4, h0=False)
    c['k'][0, :, 0, :] = np.eye(Dk)[:T]
    c['g'][:] = 0.0
    c['beta'][:] = 1.0
    q, k, v = c['q'][0, :, 0], c['k'][0, :, 0], c['v'][0, :, 0]
    want_o = 0.7 * np.tril(q @ k.T) @ v
    want_h = k.T @ v
    for o, h in _both(c):
        assert rel(o[0, :, 0], want_o) < 1e-13 and rel(h[0, 0], want_h) < 1e-13


def test_closed_form_repeated_key_overwrites():
    c = rand_case(12, T=67, Hqk=1, Hv=1, Dk=5, Dv=3, h0=False)
    kk = np.random.default_rng(0).standard_normal(5)
    kk /= np.linalg.norm(kk)
    c['k'][0, :, 0, :] = kk
    c['g'][:] = 0.0
    c['beta'][:] = 1.0
    want_h = np.outer(kk, c['v'][0, -1, 0])
    for o, h in _both(c):
        assert rel(h[0, 0], want_h) < 1e-12


def test_closed_form_scalar_state_is_exponential_smoothing():
    c = rand_case(13, T=130, Hqk=1, Hv=2, Dk=1, Dv=3)
    c['k'][:] = 1.0
    c['q'][:] = 1.0
    s = c['h0'][0, :, 0, :].copy()                        # [H, Dv]
    want = []
    for t in range(130):
        a = np.exp(c['g'][0, t])[:, None]
        b = c['beta'][0, t][:, None]
        s = a * (1 - b) * s + b * c['v'][0, t]
        want.append(s.copy())
    want = 0.7 * np.stack(want)
    for o, h in _both(c):
        assert rel(o[0], want) < 1e-13


# ------------------------------------------------- chunked == recurrent

CASES = [
    dict(seed=1, B=2, T=257, Hqk=2, Hv=2, Dk=16, Dv=16),
    dict(seed=2, lengths=[257, 3, 70, 1, 64], Hqk=1, Hv=3, Dk=8, Dv=12),
    dict(seed=3, B=1, T=3, Hqk=1, Hv=1, Dk=4, Dv=4),
    dict(seed=4, B=1, T=200, Hqk=2, Hv=4, Dk=8, Dv=8, shift=2.0),
    dict(seed=5, B=1, T=130, Hqk=1, Hv=2, Dk=8, Dv=8, retention=True, h0=False),
]


@pytest.mark.parametrize("case", CASES)
def test_chunked_equals_recurrent_qdq_off(case):
    c = rand_case(**case)
    (o1, h1), (o2, h2) = _both(c)
    assert rel(o2, o1) < 1e-12
    assert rel(h2, h1) < 1e-12


@pytest.mark.parametrize("case", CASES[:2])
def test_chunk_size_independence(case):
    c = rand_case(**case)
    args = (c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'], c['cu_seqlens'])
    o64, h64 = chunked_fwd(*args, chunk=64)
    o16, h16 = chunked_fwd(*args, chunk=16)
    o7, h7 = chunked_fwd(*args, chunk=7)
    assert rel(o16, o64) < 1e-12 and rel(h16, h64) < 1e-12
    assert rel(o7, o64) < 1e-12 and rel(h7, h64) < 1e-12


@pytest.mark.parametrize("n,shift", [(64, 0.0), (64, 2.0), (1, 0.0), (37, 0.0)])
def test_solve_reproduces_diag_beta(n, shift):
    rng = np.random.default_rng(n)
    K = rng.standard_normal((8, n, 32))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    g = -np.log1p(np.exp(rng.standard_normal((8, n)) + shift))
    b = 1 / (1 + np.exp(-rng.standard_normal((8, n))))
    gam, Gam, L, T = wy_factor(torch.tensor(K), torch.tensor(g), torch.tensor(b))
    A = torch.eye(n, dtype=torch.float64) + L
    res = (A @ T - torch.diag_embed(torch.tensor(b))).abs().max().item()
    assert res <= 1e-12
    assert torch.all(L.triu() == 0)                       # strictly lower
    assert torch.all(T.triu(1) == 0)                      # lower triangular


# ------------------------------------------------- state QDQ placement

@pytest.mark.parametrize("fmt", [FMT_E4M3, FMT_INT8])
@pytest.mark.parametrize("block_v", [4, 8, 16])
def test_state_qdq_chunked_equals_recurrent_with_qdq_at_chunk_starts(fmt, block_v):
    c = rand_case(21, lengths=[130, 64, 5], Hqk=1, Hv=2, Dk=8, Dv=16, retention=True)
    (o1, h1), (o2, h2) = _both(c, state_fmt=fmt, block_v=block_v)
    assert rel(o2, o1) < 1e-12
    assert rel(h2, h1) < 1e-12
    (o0, _), _ = _both(c)
    assert rel(o1, o0) > 1e-4                              # the QDQ did something


# ------------------------------------------------- W QDQ: token-loop re-derivation

def _token_loop_chunked(c, scale, state_fmt, w_fmt, block_v, chunk=64):
    """Chunk semantics rebuilt from token recurrences only (no solve, no gate
    matrices): W is minus the response of the per-token writes to a unit
    initial state with zero values, U the response to the values with a zero
    initial state; then the chunk is replayed token by token with the writes
    forced to Vnew = U - Wq Sq."""
    q, k, v, g, beta = (np.asarray(c[n], np.float64) for n in ('q', 'k', 'v', 'g', 'beta'))
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    cu = c['cu_seqlens'] if c['cu_seqlens'] is not None else [b * T for b in range(B + 1)]
    qf = np.repeat(q.reshape(-1, Hqk, Dk), G, axis=1)
    kf = np.repeat(k.reshape(-1, Hqk, Dk), G, axis=1)
    vf, gf, bf = v.reshape(-1, Hv, Dv), g.reshape(-1, Hv), beta.reshape(-1, Hv)
    o = np.zeros_like(vf)
    hts, wcodes = [], []
    for n in range(len(cu) - 1):
        S = np.zeros((Hv, Dk, Dv)) if c['h0'] is None else c['h0'][n].copy()
        for t0 in range(cu[n], cu[n + 1], chunk):
            t1 = min(t0 + chunk, cu[n + 1])
            X = np.broadcast_to(np.eye(Dk), (Hv, Dk, Dk)).copy()   # unit initial state
            Y = np.zeros((Hv, Dk, Dv))
            Wr, Ur = [], []
            for t in range(t0, t1):
                a = np.exp(gf[t])[:, None, None]
                X, Y = a * X, a * Y
                uw = bf[t][:, None] * (0.0 - np.einsum('hkc,hk->hc', X, kf[t]))
                uu = bf[t][:, None] * (vf[t] - np.einsum('hkc,hk->hc', Y, kf[t]))
                X = X + kf[t][:, :, None] * uw[:, None, :]
                Y = Y + kf[t][:, :, None] * uu[:, None, :]
                Wr.append(-uw)
                Ur.append(uu)
            W = np.stack(Wr, axis=1)                  # [H, n, Dk]
            U = np.stack(Ur, axis=1)                  # [H, n, Dv]
            if w_fmt != FMT_OFF:
                Wq, wc, _ = qdq32(W.astype(np.float32), w_fmt, (1, 2))
                wcodes.append(wc)
                Wq = Wq.astype(np.float64)
            else:
                Wq = W
            if state_fmt != FMT_OFF:
                x = S.astype(np.float32).reshape(Hv, Dk, Dv // block_v, block_v)
                Sq = qdq32(x, state_fmt, (1, 3))[0].reshape(Hv, Dk, Dv).astype(np.float64)
            else:
                Sq = S
            Vnew = U - Wq @ Sq
            Z = Sq.copy()
            for i, t in enumerate(range(t0, t1)):
                Z = np.exp(gf[t])[:, None, None] * Z + kf[t][:, :, None] * Vnew[:, i][:, None, :]
                o[t] = scale * np.einsum('hkv,hk->hv', Z, qf[t])
            S = Z
        hts.append(S)
    return o.reshape(v.shape), np.stack(hts), wcodes


@pytest.mark.parametrize("state_fmt,w_fmt", [(FMT_OFF, FMT_E4M3), (FMT_E4M3, FMT_E4M3),
                                             (FMT_INT8, FMT_INT8), (FMT_INT8, FMT_OFF)])
def test_w_qdq_matches_token_loop_rederivation(state_fmt, w_fmt):
    c = rand_case(31, lengths=[150, 7, 64], Hqk=1, Hv=2, Dk=8, Dv=8, retention=True)
    want_o, want_h, want_wc = _token_loop_chunked(c, 0.6, state_fmt, w_fmt, block_v=4)
    rec = {}
    o, h = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.6, c['h0'],
                       c['cu_seqlens'], state_fmt=state_fmt, w_fmt=w_fmt, block_v=4,
                       record=rec)
    assert rel(o.numpy(), want_o) < 1e-10
    assert rel(h.numpy(), want_h) < 1e-10
    if w_fmt != FMT_OFF:
        got_wc = [wc for seq in rec['W'] for (wc, _) in seq]
        assert len(got_wc) == len(want_wc)
        for a, b in zip(got_wc, want_wc):
            np.testing.assert_array_equal(a, b)


def test_qdq_changes_output_and_offsets_are_small():
    """The pages' integration check: enabling QDQ changes the output
    ("[1/4]", "What does this PR do?", Megatron adapters)."""
    c = rand_case(41, T=256, Hqk=1, Hv=2, Dk=32, Dv=32, retention=True)
    args = (c['q'], c['k'], c['v'], c['g'], c['beta'], 0.2, c['h0'], None)
    o0, _ = chunked_fwd(*args)
    os_, _ = chunked_fwd(*args, state_fmt=FMT_E4M3, block_v=16)
    ow, _ = chunked_fwd(*args, w_fmt=FMT_E4M3)
    osw, _ = chunked_fwd(*args, state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=16)
    r_s, r_w, r_sw = rel(os_, o0), rel(ow, o0), rel(osw, o0)
    assert 1e-3 < r_s < 0.1
    assert 1e-6 < r_w < 0.1
    assert r_sw > 1e-3


def test_power_of_two_equivariance_with_qdq():
    """Scaling v and h0 by 2**k scales o and ht by exactly 2**k with both QDQ
    sites on (scales follow the amax; W does not depend on v)."""
    c = rand_case(42, T=100, Hqk=1, Hv=2, Dk=8, Dv=8)
    args = dict(state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=4)
    o1, h1 = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.3, c['h0'], **args)
    o2, h2 = chunked_fwd(c['q'], c['k'], 8.0 * c['v'], c['g'], c['beta'], 0.3,
                         8.0 * c['h0'], **args)
    assert torch.equal(o2, 8.0 * o1) and torch.equal(h2, 8.0 * h1)


# ------------------------------------------------- two-precision read copy

def test_read_profile_chunked_equals_token_recurrence_with_read_offsets():
    """The chunk form of the two-precision profile (reads through the
    per-column E4M3 copy of the chunk's incoming state, carry in FP32)
    equals the token recurrence that reads S - a E, E the read offset taken
    at each chunk start and a its decay ("[5/8] ReplaySSM state QAT and
    two-precision GDN", "What does this PR do?")."""
    c = rand_case(31, lengths=[130, 64, 5], Hqk=1, Hv=2, Dk=8, Dv=16, retention=True)
    (o1, h1), (o2, h2) = _both(c, read_fmt=FMT_E4M3)
    assert rel(o2, o1) < 1e-12
    assert rel(h2, h1) < 1e-12
    (o0, h0), _ = _both(c)
    assert rel(o1, o0) > 1e-4 and rel(h1, h0) > 1e-5        # the read copy did something
    (oq, hq), _ = _both(c, state_fmt=FMT_E4M3, block_v=16)
    assert rel(h1, hq) > 1e-5                              # and it is not the quantized carry


def test_read_profile_zero_beta_keeps_the_anchor_exact():
    """With beta = 0 nothing is written: the anchor only decays, so ht is
    the exact decay of h0 (read errors never reach it), while each output
    reads the per-column E4M3 copy of the chunk's incoming state, decayed:
    o_t = scale (exp(gamma_t) QDQ_R(S_c))^T q_t."""
    c = rand_case(32, T=150, Hqk=1, Hv=2, Dk=8, Dv=4)
    c['beta'] = np.zeros_like(c['beta'])
    scale = 0.6
    o, ht = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, c['h0'],
                        read_fmt=FMT_E4M3)
    o, ht = o.numpy(), ht.numpy()
    cum = np.cumsum(c['g'][0], axis=0)                       # [T, Hv]
    np.testing.assert_allclose(ht[0], np.exp(cum[-1])[:, None, None] * c['h0'][0], rtol=1e-13)
    for t in (0, 5, 63, 64, 100, 149):
        c0 = 64 * (t // 64)
        Sc = c['h0'][0] * (np.exp(cum[c0 - 1]) if c0 > 0 else np.ones(2))[:, None, None]
        r, _, _ = qdq32(Sc.astype(np.float32), FMT_E4M3, (1,))
        decay = np.exp(cum[t] - (cum[c0 - 1] if c0 > 0 else 0.0))
        want = scale * np.einsum('hkv,hk->hv', decay[:, None, None] * r.astype(np.float64),
                                 c['q'][0, t, [0, 0]])
        np.testing.assert_allclose(o[0, t], want, rtol=1e-12, atol=1e-15)


def test_read_profile_refuses_a_quantized_carry():
    c = rand_case(33, T=10, Hqk=1, Hv=1, Dk=4, Dv=4)
    with pytest.raises(ValueError):
        chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                    state_fmt=FMT_E4M3, read_fmt=FMT_E4M3)
