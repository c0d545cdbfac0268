"""Pins of the oracle's backward.

QDQ off: the chunked backward (reverse mode through the WY form) equals
central finite differences of the token recurrence, an independent path.
QDQ on: the identity straight-through gradient ("[1/4] GDN state/W QAT
foundation", "What does this PR do?": identity STE; "[2/4] ...", usage:
pass-through backward) is the exact gradient of a frozen-offset surrogate,
F(x) = chunked forward with every QDQ(z) replaced by z + e, where e is the
QDQ offset recorded at the base point; finite differences of F pin it.
Inputs cover grouped heads, packed sequences, nonzero initial states and an
upstream final-state gradient ("[2/4] ...", "Testing": first-order
input/state gradients)."""
import numpy as np
import pytest
import torch

from oracle import FMT_E4M3, FMT_INT8, FMT_OFF, chunked_bwd, chunked_fwd, recurrent_fwd
from oracle.chunked import qdq_ste
from test_oracle_fwd import rand_case

NAMES = ['q', 'k', 'v', 'g', 'beta', 'h0']


def _loss(o, h, do, dht):
    return float(np.sum(np.asarray(o) * do) + np.sum(np.asarray(h) * dht))


def _fd_directional(f, c, grads, rng, n_dir=3, eps=1e-6):
    """For each input tensor, compare <grad, u> with the central difference
    of f along random directions u."""
    worst = 0.0
    for name in NAMES:
        if c.get(name) is None:
            continue
        for _ in range(n_dir):
            u = rng.standard_normal(c[name].shape)
            cp, cm = dict(c), dict(c)
            cp[name] = c[name] + eps * u
            cm[name] = c[name] - eps * u
            fd = (f(cp) - f(cm)) / (2 * eps)
            an = float(np.sum(grads['d' + name].numpy() * u))
            err = abs(fd - an) / max(abs(fd), abs(an), 1e-8)
            worst = max(worst, err)
            assert err < 1e-6, (name, fd, an)
    return worst


def _upstream(c, seed):
    rng = np.random.default_rng(seed)
    o_shape = c['v'].shape
    N = c['h0'].shape[0] if c['h0'] is not None else (
        len(c['cu_seqlens']) - 1 if c['cu_seqlens'] is not None else c['v'].shape[0])
    Hv, Dk, Dv = c['v'].shape[2], c['q'].shape[3], c['v'].shape[3]
    return rng.standard_normal(o_shape), 0.3 * rng.standard_normal((N, Hv, Dk, Dv))


def test_bwd_qdq_off_elementwise_fd_tiny():
    c = rand_case(51, T=5, Hqk=1, Hv=2, Dk=3, Dv=3)
    do, dht = _upstream(c, 1)
    scale = 0.8
    for chunk in (64, 2):
        grads = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, do, dht,
                            c['h0'], chunk=chunk)
        for name in NAMES:
            x = c[name]
            fd = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                cp, cm = dict(c), dict(c)
                cp[name] = x.copy()
                cm[name] = x.copy()
                cp[name][idx] += 1e-6
                cm[name][idx] -= 1e-6
                lp = _loss(*recurrent_fwd(cp['q'], cp['k'], cp['v'], cp['g'], cp['beta'],
                                          scale, cp['h0']), do, dht)
                lm = _loss(*recurrent_fwd(cm['q'], cm['k'], cm['v'], cm['g'], cm['beta'],
                                          scale, cm['h0']), do, dht)
                fd[idx] = (lp - lm) / 2e-6
            got = grads['d' + name].numpy()
            np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("case", [
    dict(seed=52, lengths=[70, 3, 64], Hqk=1, Hv=2, Dk=4, Dv=4),
    dict(seed=53, B=2, T=130, Hqk=2, Hv=4, Dk=4, Dv=8, shift=2.0),
])
def test_bwd_qdq_off_directional_fd_vs_recurrent(case):
    c = rand_case(**case)
    do, dht = _upstream(c, 2)
    scale = 0.5
    grads = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, do, dht,
                        c['h0'], c['cu_seqlens'])

    def f(cc):
        return _loss(*recurrent_fwd(cc['q'], cc['k'], cc['v'], cc['g'], cc['beta'], scale,
                                    cc['h0'], cc['cu_seqlens']), do, dht)
    _fd_directional(f, c, grads, np.random.default_rng(3))


class _Frozen:
    """Records QDQ offsets at the base point, then replays them as a frozen
    additive offset (smooth surrogate)."""

    def __init__(self):
        self.offsets = []
        self.mode = 'record'
        self.i = 0

    def __call__(self, x, fmt, tile_axes, sink):
        if self.mode == 'record':
            y = qdq_ste(x, fmt, tile_axes, sink)
            self.offsets.append((y - x).detach().clone())
            return y
        e = self.offsets[self.i]
        self.i += 1
        return x + e


@pytest.mark.parametrize("state_fmt,w_fmt,block_v,read_fmt", [(FMT_E4M3, FMT_E4M3, 4, FMT_OFF),
                                                              (FMT_INT8, FMT_OFF, 8, FMT_OFF),
                                                              (FMT_OFF, FMT_E4M3, 8, FMT_OFF),
                                                              (FMT_OFF, FMT_OFF, 8, FMT_E4M3),
                                                              (FMT_OFF, FMT_INT8, 8, FMT_E4M3)])
def test_bwd_ste_equals_frozen_offset_surrogate_gradient(state_fmt, w_fmt, block_v, read_fmt):
    """read_fmt: the two-precision read copy ("[5/8] ReplaySSM state QAT and
    two-precision GDN", "Testing": first-order gradients) through the same
    surrogate: its offset is frozen at every read, the FP32 carry is not."""
    c = rand_case(54, lengths=[100, 3, 64], Hqk=1, Hv=2, Dk=4, Dv=8, retention=True)
    do, dht = _upstream(c, 4)
    scale = 0.5
    kw = dict(state_fmt=state_fmt, w_fmt=w_fmt, block_v=block_v, read_fmt=read_fmt)
    grads = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, do, dht,
                        c['h0'], c['cu_seqlens'], **kw)
    fr = _Frozen()
    o_base, h_base = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, c['h0'],
                                 c['cu_seqlens'], site_fn=fr, **kw)
    assert any(float(e.abs().max()) > 0 for e in fr.offsets)    # QDQ was active
    fr.mode = 'replay'

    def f(cc):
        fr.i = 0
        o, h = chunked_fwd(cc['q'], cc['k'], cc['v'], cc['g'], cc['beta'], scale, cc['h0'],
                           cc['cu_seqlens'], site_fn=fr, **kw)
        assert fr.i == len(fr.offsets)
        return _loss(o.numpy(), h.numpy(), do, dht)

    # the surrogate reproduces the quantized forward at the base point
    o_q, h_q = chunked_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], scale, c['h0'],
                           c['cu_seqlens'], **kw)
    assert torch.equal(o_base, o_q) and torch.equal(h_base, h_q)
    assert abs(f(c) - _loss(o_q.numpy(), h_q.numpy(), do, dht)) < 1e-9
    _fd_directional(f, c, grads, np.random.default_rng(5))


def test_bwd_ste_differs_from_qdq_off_gradient():
    c = rand_case(55, T=128, Hqk=1, Hv=2, Dk=8, Dv=8, retention=True)
    do, dht = _upstream(c, 6)
    g_off = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.4, do, dht, c['h0'])
    g_on = chunked_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.4, do, dht, c['h0'],
                       state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=4)
    d = float((g_on['dk'] - g_off['dk']).norm() / g_off['dk'].norm())
    assert d > 1e-4
