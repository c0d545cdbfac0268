"""Pins of the decode-continuation oracle (oracle/decode.py).

"[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What does this PR
do?" (exact chunk prefill of an explicit prefix, then token-state writes
through the state quantizer, identity straight-through gradients through
initial states and the continuation) and "Testing" (257-token trajectories,
nonzero initial states, grouped heads, packed tails, both readouts, split
carry, all state scale widths, first-order input/state gradients).

What fixes each part, independently of oracle/decode.py's own loop:
  * state format off: the decode and the prefill + decode are the plain
    gated delta rule, which the token recurrence of oracle/recurrent.py
    (numpy, pinned by closed forms) computes;
  * readout before the write: a write after every token is the recurrent
    oracle's state QDQ with a chunk of one token, whose output is read
    before the next QDQ; the decode's final state is that run's final state
    through one more QDQ;
  * readout after the write: each output is scale * QDQ(S_t)^T q_t with S_t
    the recurrent oracle's state after token t;
  * closed forms: beta = 0 and g = 0 keep the written initial state;
  * split carry: continuing from a returned state is bit-identical
    (the write is idempotent);
  * gradients: central finite differences of the recurrent oracle (format
    off) and of the frozen-offset surrogate (format on)."""
import numpy as np
import pytest
import torch

from oracle import FMT_E4M3, FMT_INT8, FMT_OFF, qdq32, recurrent_fwd
from oracle.chunked import qdq_ste
from oracle.decode import (READOUT_AFTER_WRITE, READOUT_BEFORE_WRITE, decode_bwd, decode_fwd,
                           prefill_decode_bwd, prefill_decode_fwd)
from oracle.recurrent import qdq_state64
from test_oracle_fwd import rand_case


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _seqs(c):
    T = c['q'].shape[1]
    if c['cu_seqlens'] is None:
        return [(b * T, (b + 1) * T) for b in range(c['q'].shape[0])]
    cu = [int(x) for x in c['cu_seqlens']]
    return list(zip(cu[:-1], cu[1:]))


def _flat(x, lo, hi):
    return x.reshape(-1, *x.shape[2:])[lo:hi][None]


def _recurrent_reference(c, scale, prefix_len, state_fmt, block_v, readout):
    """Prefill + decode composed from the token recurrence alone, sequence by
    sequence: the prefix with state QDQ at 64-token chunk starts, then the
    decode tokens as chunks of one token (QDQ before each), and for the
    after-write readout one recurrent run per token."""
    Hv, Dv = c['v'].shape[2], c['v'].shape[3]
    o = np.zeros(c['v'].shape).reshape(-1, Hv, Dv)
    hts = []
    for n, (bos, eos) in enumerate(_seqs(c)):
        hi = min(bos + prefix_len, eos)
        h0 = None if c['h0'] is None else c['h0'][n:n + 1]
        args = lambda lo, up: [_flat(c[x], lo, up) for x in ('q', 'k', 'v', 'g', 'beta')]
        o_p, h_mid = recurrent_fwd(*args(bos, hi), scale, h0, state_fmt=state_fmt,
                                   block_v=block_v, chunk=64)
        o[bos:hi] = o_p[0]
        o_d, h_end = recurrent_fwd(*args(hi, eos), scale, h_mid, state_fmt=state_fmt,
                                   block_v=block_v, chunk=1)
        if readout == READOUT_BEFORE_WRITE:
            o[hi:eos] = o_d[0]
        else:
            G = Hv // c['q'].shape[2]
            qf = np.repeat(c['q'].reshape(-1, c['q'].shape[2], c['q'].shape[3]), G, axis=1)
            for t in range(hi, eos):
                _, h_t = recurrent_fwd(*args(hi, t + 1), scale, h_mid, state_fmt=state_fmt,
                                       block_v=block_v, chunk=1)
                St = qdq_state64(h_t[0], state_fmt, block_v) if state_fmt else h_t[0]
                o[t] = scale * np.einsum('hkv,hk->hv', St, qf[t])
        hts.append(qdq_state64(h_end[0], state_fmt, block_v) if state_fmt else h_end[0])
    return o.reshape(c['v'].shape), np.stack(hts)


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("readout", [READOUT_BEFORE_WRITE, READOUT_AFTER_WRITE])
def test_decode_state_off_is_the_token_recurrence(readout):
    c = rand_case(301, lengths=[257, 3, 40], Hqk=1, Hv=2, Dk=6, Dv=5)
    o, ht = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.6, c['h0'],
                       c['cu_seqlens'], readout=readout)
    o_r, h_r = recurrent_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.6, c['h0'],
                             c['cu_seqlens'])
    assert rel(o.numpy(), o_r) < 1e-12 and rel(ht.numpy(), h_r) < 1e-12


@pytest.mark.parametrize("fmt,block_v", [(FMT_E4M3, 4), (FMT_E4M3, 8), (FMT_INT8, 4),
                                         (FMT_INT8, 8)])
def test_decode_before_write_is_recurrence_with_a_qdq_per_token(fmt, block_v):
    c = rand_case(302, B=2, T=257, Hqk=1, Hv=2, Dk=4, Dv=8, retention=True)
    o, ht = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                       state_fmt=fmt, block_v=block_v)
    o_r, h_r = _recurrent_reference(c, 0.5, 0, fmt, block_v, READOUT_BEFORE_WRITE)
    assert rel(o.numpy(), o_r) < 1e-12 and rel(ht.numpy(), h_r) < 1e-12
    # the writes matter: without them the outputs move
    o_off, _ = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'])
    assert rel(o.numpy(), o_off.numpy()) > 1e-4


@pytest.mark.parametrize("fmt", [FMT_E4M3, FMT_INT8])
def test_decode_after_write_reads_the_written_state(fmt):
    c = rand_case(303, lengths=[20, 7], Hqk=1, Hv=2, Dk=4, Dv=8)
    o, ht = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                       c['cu_seqlens'], state_fmt=fmt, block_v=4, readout=READOUT_AFTER_WRITE)
    o_r, h_r = _recurrent_reference(c, 0.5, 0, fmt, 4, READOUT_AFTER_WRITE)
    assert rel(o.numpy(), o_r) < 1e-12 and rel(ht.numpy(), h_r) < 1e-12
    o_b, _ = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                        c['cu_seqlens'], state_fmt=fmt, block_v=4)
    assert rel(o.numpy(), o_b.numpy()) > 1e-4          # the two readouts differ


@pytest.mark.parametrize("fmt", [FMT_E4M3, FMT_INT8])
def test_decode_closed_form_no_write_strength_no_decay(fmt):
    """beta = 0, g = 0: the state stays the written initial state, so both
    readouts give scale * QDQ(h_in)^T q_t and ht = QDQ(h_in)."""
    c = rand_case(304, T=9, Hqk=1, Hv=2, Dk=4, Dv=8)
    c['beta'][:] = 0.0
    c['g'][:] = 0.0
    x = c['h0'][0].astype(np.float32).reshape(2, 4, 2, 4)
    hq = qdq32(x, fmt, tile_axes=(1, 3))[0].reshape(2, 4, 8).astype(np.float64)
    want_o = 0.5 * np.einsum('hkv,thk->thv', hq, np.repeat(c['q'][0], 2, axis=1))
    for readout in (READOUT_BEFORE_WRITE, READOUT_AFTER_WRITE):
        o, ht = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, c['h0'],
                           state_fmt=fmt, block_v=4, readout=readout)
        assert rel(o[0].numpy(), want_o) < 1e-13 and rel(ht[0].numpy(), hq) < 1e-15


def test_decode_representable_state_passes_through_the_write():
    """An INT8 state that is already on its tile's grid (integers times a
    power of two, the largest magnitude 127 steps) is written unchanged."""
    rng = np.random.default_rng(305)
    codes = rng.integers(-127, 128, size=(1, 2, 4, 8)).astype(np.float64)
    codes[..., 0, 0] = 127.0
    codes[..., 0, 4] = -127.0
    h = codes * 2.0 ** -9
    c = rand_case(305, T=3, Hqk=1, Hv=2, Dk=4, Dv=8)
    c['beta'][:] = 0.0
    c['g'][:] = 0.0
    o, ht = decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 1.0, h, state_fmt=FMT_INT8,
                       block_v=4)
    assert np.array_equal(ht.numpy(), h)


@pytest.mark.parametrize("fmt,readout", [(FMT_INT8, READOUT_BEFORE_WRITE),
                                         (FMT_E4M3, READOUT_AFTER_WRITE),
                                         (FMT_OFF, READOUT_BEFORE_WRITE)])
def test_decode_split_carry_is_bit_identical(fmt, readout):
    c = rand_case(306, B=2, T=257, Hqk=1, Hv=2, Dk=4, Dv=8)
    kw = dict(state_fmt=fmt, block_v=4, readout=readout)
    x = [c[n] for n in ('q', 'k', 'v', 'g', 'beta')]
    o, ht = decode_fwd(*x, 0.5, c['h0'], **kw)
    for a in (1, 64, 100):
        o1, h1 = decode_fwd(*[y[:, :a] for y in x], 0.5, c['h0'], **kw)
        o2, h2 = decode_fwd(*[y[:, a:] for y in x], 0.5, h1, **kw)
        assert torch.equal(torch.cat([o1, o2], dim=1), o) and torch.equal(h2, ht)
        # the same continuation through `start` on the whole buffer
        o3, h3 = decode_fwd(*x, 0.5, h1, start=a, **kw)
        assert torch.equal(o3[:, a:], o[:, a:]) and not o3[:, :a].any() and torch.equal(h3, ht)


@pytest.mark.parametrize("prefix_len,fmt,block_v,readout", [
    (64, FMT_INT8, 4, READOUT_BEFORE_WRITE),
    (70, FMT_E4M3, 8, READOUT_BEFORE_WRITE),
    (64, FMT_OFF, 8, READOUT_AFTER_WRITE),
    (0, FMT_E4M3, 4, READOUT_BEFORE_WRITE),
    (200, FMT_INT8, 8, READOUT_BEFORE_WRITE),
])
def test_prefill_decode_is_the_composed_recurrence(prefix_len, fmt, block_v, readout):
    """Packed tails: one sequence shorter than the prefix (all prefill), one
    of 257 tokens, one of 3."""
    c = rand_case(307, lengths=[257, 3, 130], Hqk=1, Hv=2, Dk=4, Dv=8, retention=True)
    o, ht = prefill_decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, prefix_len,
                               c['h0'], c['cu_seqlens'], state_fmt=fmt, block_v=block_v,
                               readout=readout)
    o_r, h_r = _recurrent_reference(c, 0.5, prefix_len, fmt, block_v, readout)
    assert rel(o.numpy(), o_r) < 1e-12 and rel(ht.numpy(), h_r) < 1e-12


def test_prefill_decode_after_write_readout_short():
    c = rand_case(308, lengths=[80, 66], Hqk=1, Hv=2, Dk=4, Dv=8)
    o, ht = prefill_decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, 64, c['h0'],
                               c['cu_seqlens'], state_fmt=FMT_E4M3, block_v=4,
                               readout=READOUT_AFTER_WRITE)
    o_r, h_r = _recurrent_reference(c, 0.5, 64, FMT_E4M3, 4, READOUT_AFTER_WRITE)
    assert rel(o.numpy(), o_r) < 1e-12 and rel(ht.numpy(), h_r) < 1e-12


def test_prefill_decode_grouped_heads_and_w_qdq():
    """Grouped heads; W QDQ applies in the prefill only (the decode has no W)."""
    c = rand_case(309, B=2, T=130, Hqk=2, Hv=4, Dk=4, Dv=8)
    kw = dict(state_fmt=FMT_INT8, block_v=8)
    o_w, h_w = prefill_decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, 64, c['h0'],
                                  w_fmt=FMT_E4M3, **kw)
    o_n, h_n = prefill_decode_fwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, 64, c['h0'],
                                  **kw)
    o_r, h_r = _recurrent_reference(c, 0.5, 64, FMT_INT8, 8, READOUT_BEFORE_WRITE)
    assert rel(o_n.numpy(), o_r) < 1e-12 and rel(h_n.numpy(), h_r) < 1e-12
    d = rel(o_w.numpy(), o_n.numpy())
    assert 1e-5 < d < 0.1


# ----------------------------------------------------------------- backward

NAMES = ('q', 'k', 'v', 'g', 'beta', 'h0')


def _upstream(c, seed):
    rng = np.random.default_rng(seed)
    N = c['h0'].shape[0]
    Hv, Dk, Dv = c['v'].shape[2], c['q'].shape[3], c['v'].shape[3]
    return rng.standard_normal(c['v'].shape), 0.3 * rng.standard_normal((N, Hv, Dk, Dv))


def _loss(o, h, do, dht):
    return float(np.sum(np.asarray(o) * do) + np.sum(np.asarray(h) * dht))


def _fd_check(f, c, grads, seed, eps=1e-6, n_dir=3):
    rng = np.random.default_rng(seed)
    for name in NAMES:
        for _ in range(n_dir):
            u = rng.standard_normal(c[name].shape)
            cp, cm = dict(c), dict(c)
            cp[name] = c[name] + eps * u
            cm[name] = c[name] - eps * u
            fd = (f(cp) - f(cm)) / (2 * eps)
            an = float(np.sum(grads[name].numpy() * u))
            assert abs(fd - an) <= 1e-6 * max(abs(fd), abs(an), 1e-8), (name, fd, an)


def test_decode_bwd_state_off_matches_fd_of_recurrence():
    c = rand_case(310, lengths=[9, 4], Hqk=1, Hv=2, Dk=3, Dv=4)
    do, dht = _upstream(c, 1)
    for readout in (READOUT_BEFORE_WRITE, READOUT_AFTER_WRITE):
        gr = decode_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.7, do, dht, c['h0'],
                        c['cu_seqlens'], readout=readout)
        gr = {n: gr['dh_in' if n == 'h0' else 'd' + n] for n in NAMES}

        def f(cc):
            return _loss(*recurrent_fwd(cc['q'], cc['k'], cc['v'], cc['g'], cc['beta'], 0.7,
                                        cc['h0'], cc['cu_seqlens']), do, dht)
        _fd_check(f, c, gr, 2)


def test_prefill_decode_bwd_state_off_matches_fd_of_recurrence():
    c = rand_case(311, lengths=[70, 5], Hqk=1, Hv=2, Dk=3, Dv=4)
    do, dht = _upstream(c, 3)
    gr = prefill_decode_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.7, 64, do, dht,
                            c['h0'], c['cu_seqlens'])
    gr = {n: gr['d' + n] for n in NAMES}

    def f(cc):
        return _loss(*recurrent_fwd(cc['q'], cc['k'], cc['v'], cc['g'], cc['beta'], 0.7,
                                    cc['h0'], cc['cu_seqlens']), do, dht)
    _fd_check(f, c, gr, 4)


class _Frozen:
    """Records each QDQ's offset at the base point, then replays it as a
    constant additive offset (the smooth surrogate whose exact gradient the
    identity straight-through estimator is)."""

    def __init__(self):
        self.offsets, self.mode, self.i = [], 'record', 0

    def __call__(self, x, fmt, tile_axes, sink):
        if self.mode == 'record':
            y = qdq_ste(x, fmt, tile_axes, sink)
            self.offsets.append((y - x).detach().clone())
            return y
        e = self.offsets[self.i]
        self.i += 1
        return x + e


@pytest.mark.parametrize("fmt,w_fmt,readout,prefix_len", [
    (FMT_INT8, FMT_OFF, READOUT_BEFORE_WRITE, 0),
    (FMT_E4M3, FMT_OFF, READOUT_AFTER_WRITE, 0),
    (FMT_INT8, FMT_E4M3, READOUT_AFTER_WRITE, 64),
    (FMT_E4M3, FMT_OFF, READOUT_BEFORE_WRITE, 70),
])
def test_ste_gradient_is_the_frozen_offset_surrogate_gradient(fmt, w_fmt, readout, prefix_len):
    c = rand_case(312, lengths=[100, 3, 66], Hqk=1, Hv=2, Dk=4, Dv=8, retention=True)
    do, dht = _upstream(c, 5)
    kw = dict(state_fmt=fmt, block_v=4, readout=readout)
    x = [c[n] for n in ('q', 'k', 'v', 'g', 'beta')]
    if prefix_len:
        gr = prefill_decode_bwd(*x, 0.5, prefix_len, do, dht, c['h0'], c['cu_seqlens'],
                                w_fmt=w_fmt, **kw)
        gr = {n: gr['d' + n] for n in NAMES}
        run = lambda cc, sf: prefill_decode_fwd(*[cc[n] for n in ('q', 'k', 'v', 'g', 'beta')],
                                                0.5, prefix_len, cc['h0'], cc['cu_seqlens'],
                                                w_fmt=w_fmt, site_fn=sf, **kw)
    else:
        gr = decode_bwd(*x, 0.5, do, dht, c['h0'], c['cu_seqlens'], **kw)
        gr = {n: gr['dh_in' if n == 'h0' else 'd' + n] for n in NAMES}
        run = lambda cc, sf: decode_fwd(*[cc[n] for n in ('q', 'k', 'v', 'g', 'beta')], 0.5,
                                        cc['h0'], cc['cu_seqlens'], site_fn=sf, **kw)
    fr = _Frozen()
    o_b, h_b = run(c, fr)
    assert any(float(e.abs().max()) > 0 for e in fr.offsets)
    o_q, h_q = run(c, None)
    assert torch.equal(o_b, o_q) and torch.equal(h_b, h_q)
    fr.mode = 'replay'

    def f(cc):
        fr.i = 0
        o, h = run(cc, fr)
        assert fr.i == len(fr.offsets)
        return _loss(o.numpy(), h.numpy(), do, dht)
    _fd_check(f, c, gr, 6)


def test_decode_gradient_reaches_the_prefix():
    """Gradients flow from decode outputs back into prefill tokens and h0."""
    c = rand_case(313, B=1, T=80, Hqk=1, Hv=2, Dk=4, Dv=8, retention=True)
    do = np.zeros(c['v'].shape)
    do[:, 64:] = np.random.default_rng(7).standard_normal(do[:, 64:].shape)
    gr = prefill_decode_bwd(c['q'], c['k'], c['v'], c['g'], c['beta'], 0.5, 64, do, None,
                            c['h0'], state_fmt=FMT_INT8, block_v=4)
    assert float(gr['dk'][:, :64].abs().max()) > 1e-3
    assert float(gr['dh0'].abs().max()) > 1e-6
