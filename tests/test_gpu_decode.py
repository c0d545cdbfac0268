"""Decode continuation on the GPU (gdn_decode_fwd / gdn_decode_bwd, and the
chunk prefill with prefix_len, through the C ABI) against the float64
oracle of oracle/decode.py on the same seeded inputs.

"[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What does this PR
do?" (exact chunk prefill of an explicit prefix, then token-state writes
with E4M3 / INT8 state QDQ, gradients through the initial state and the
continuation) and "Testing" (257-token trajectories, nonzero initial
states, grouped heads, packed tails, both readouts, split carry, all state
scale widths, first-order input/state gradients).

Bars (rel-L2): format off: o <= 3e-3 (bf16 output) or 1e-5 (FP32), ht <= 1e-5;
format on: o and ht <= 1e-2, each written state's codes differ from the
oracle's on at most 1e-3 of the elements (one-step flips where the FP32
value sits on a rounding midpoint) and its scales agree to 1e-3 (a scale
is the tile amax over q_max, so it carries the state's own FP32-vs-float64
difference, which grows over a 257-write trajectory to ~1e-4, and any
earlier flip that lands on the amax element). Gradients: format off <= 3e-3,
on <= 1e-2. Split carry is bit-identical."""
import math

import numpy as np
import pytest
import torch

import gdn_inputs
from gateddeltanet_chunked_recurrence_amd import binding as B
from oracle.decode import decode_bwd, decode_fwd, prefill_decode_bwd, prefill_decode_fwd
from parity_util import code_bytes, draw, head_subset, rel, say

pytestmark = pytest.mark.gpu

OFF, E4M3, INT8 = 0, 1, 2
BEFORE, AFTER = B.READOUT_BEFORE_WRITE, B.READOUT_AFTER_WRITE


def _spec(**kw):
    base = dict(B=2, T=257, Hqk=1, Hv=2, Dk=128, Dv=128, dtype='bf16', gate='softplus',
                shift=0.0, h0=True, state_fmt=INT8, w_fmt=OFF, block_v=64)
    base.update(kw)
    return base


def _scale(spec):
    return 1.0 / math.sqrt(spec['Dk'])


def _o_bar(spec):
    if spec['state_fmt'] != OFF:
        return 1e-2
    return 1e-5 if spec['dtype'] == 'f32' else 3e-3


def _h_bar(spec):
    return 1e-2 if spec['state_fmt'] != OFF else 1e-5


def _full(x):
    """CPU float64 copies of every input with the heads as drawn (grouped
    query/key heads kept), so the oracle's dq, dk are per query/key head
    like the GPU's."""
    return dict(q=x['q'].double().cpu(), k=x['k'].double().cpu(), v=x['v'].double().cpu(),
                g=x['g'].double().cpu(), beta=x['beta'].double().cpu(),
                h0=None if x['h0'] is None else x['h0'].double().cpu(), cu=x['cu_list'],
                do=x['do'].double().cpu(), dht=x['dht'].double().cpu())


def _decode_rows(x, spec, start):
    """Packed token rows the decode writes (tokens start..len-1 of each sequence)."""
    T = x['q'].shape[1]
    bounds = (list(zip(x['cu_list'][:-1], x['cu_list'][1:])) if x['cu_list'] is not None
              else [(b * T, (b + 1) * T) for b in range(x['q'].shape[0])])
    rows = [t for lo, hi in bounds for t in range(min(lo + start, hi), hi)]
    return torch.tensor(rows, dtype=torch.long), bounds


def _decode_saved_views(saved, x, spec, start):
    a = B.make_decode_args(x['q'], x['k'], x['v'], x['g'], x['beta'], None, x['h0'],
                           x['cu_seqlens'], start, spec['state_fmt'], spec['block_v'], 0)
    lib = B.load_library()
    total = lib.gdn_decode_saved_bytes(a)
    raw = saved.cpu()
    assert raw.numel() == total
    N = x['N']
    slots = x['q'].shape[0] * x['q'].shape[1] + N
    Hv, Dk, Dv, bv = spec['Hv'], spec['Dk'], spec['Dv'], spec['block_v']
    codes = raw[:slots * Hv * Dk * Dv].view(slots, Hv, Dk, Dv)
    off = (slots * Hv * Dk * Dv + 255) // 256 * 256
    scales = raw[off: off + slots * Hv * (Dv // bv) * 4].view(torch.float32).view(slots, Hv, Dv // bv)
    return codes, scales


def _check_written_states(x, spec, saved, rec, heads, start):
    """Every written state (first write and one per decode token) against the
    oracle's record of the same writes."""
    codes, scales = _decode_saved_views(saved, x, spec, start)
    _, bounds = _decode_rows(x, spec, start)
    fmt, bv = spec['state_fmt'], spec['block_v']
    flips = total = 0
    worst_scale = 0.0
    for n, (lo, hi) in enumerate(bounds):
        first = min(lo + start, hi)
        writes = rec['S'][n]
        assert len(writes) == hi - first + 1
        for j, (c_ref, d_ref) in enumerate(writes):
            slot = first + n + j
            want = code_bytes(np.asarray(c_ref), fmt)            # [Z, Dk, Dv/bv, bv]
            got = codes[slot][heads].numpy().reshape(want.shape)
            a = np.where(got == 0x80, 0, got) if fmt == E4M3 else got
            b = np.where(want == 0x80, 0, want) if fmt == E4M3 else want
            flips += int((a != b).sum())
            total += a.size
            d_got = scales[slot][heads].double().numpy()
            d_want = np.asarray(d_ref, np.float64).reshape(d_got.shape)
            worst_scale = max(worst_scale, float(np.max(np.abs(d_got - d_want) / d_want)))
    frac = flips / max(total, 1)
    say(f"  written states: code flips {flips}/{total} = {frac:.2e}, scale rel max {worst_scale:.2e}")
    assert frac <= 1e-3 and worst_scale <= 1e-3


DECODE_CASES = [
    # (name, spec overrides, start, readout)
    ('int8_bv64_before', dict(), 0, BEFORE),
    ('int8_bv64_after', dict(), 0, AFTER),
    ('e4m3_bv16_after_gqa', dict(Hqk=2, Hv=4, state_fmt=E4M3, block_v=16), 0, AFTER),
    ('e4m3_bv32_before_start9', dict(state_fmt=E4M3, block_v=32), 9, BEFORE),
    ('int8_bv128_dv128', dict(block_v=128), 0, BEFORE),
    ('e4m3_bv256_dv256_after', dict(Dv=256, block_v=256, state_fmt=E4M3, T=130), 0, AFTER),
    ('int8_dk64_dv256_bv64', dict(Dk=64, Dv=256, T=100), 0, BEFORE),
    ('off_bf16', dict(state_fmt=OFF), 0, BEFORE),
    ('off_fp32_dk64', dict(state_fmt=OFF, dtype='f32', Dk=64, Dv=64, T=120), 0, AFTER),
    ('int8_fp32_dk128', dict(dtype='f32', T=90), 0, BEFORE),
    ('packed_tails', dict(B=1, lengths=[257, 3, 1, 0, 70], Hqk=2, Hv=4, state_fmt=E4M3), 0, AFTER),
    ('no_h0_dv64', dict(h0=False, Dv=64, block_v=16, T=64), 0, BEFORE),
]


def _decode_run(spec, seed, start, readout, save=True):
    x = draw(spec, seed, bwd=True)
    o, ht, saved = B.gdn_decode_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], _scale(spec),
                                    x['h0'], x['cu_seqlens'], start, spec['state_fmt'],
                                    spec['block_v'], readout, save_for_backward=save,
                                    out=torch.zeros(*x['v'].shape, dtype=x['q'].dtype,
                                                    device='cuda'))
    torch.cuda.synchronize()
    return x, o, ht, saved


@pytest.mark.parametrize("name,over,start,readout", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_forward_parity(name, over, start, readout):
    spec = _spec(**over)
    say(f"decode fwd {name}: {spec} start={start} readout={readout}")
    x, o, ht, saved = _decode_run(spec, 101, start, readout)
    heads = list(range(spec['Hv']))
    sub = head_subset(x, spec, heads)
    rec = {}
    o_ref, ht_ref = decode_fwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'], _scale(spec),
                               sub['h0'], sub['cu'], start, spec['state_fmt'], spec['block_v'],
                               readout, record=rec)
    rows, _ = _decode_rows(x, spec, start)
    o_f = o.reshape(-1, spec['Hv'], spec['Dv']).float().cpu()
    o_r = o_ref.reshape(-1, spec['Hv'], spec['Dv'])
    assert torch.isfinite(o_f[rows]).all() and torch.isfinite(ht).all()
    r_o, r_h = rel(o_f[rows], o_r[rows]), rel(ht.cpu(), ht_ref)
    say(f"  rel-L2 o={r_o:.3e} ht={r_h:.3e}")
    assert r_o <= _o_bar(spec) and r_h <= _h_bar(spec)
    # tokens before `start` are left untouched (zeros here)
    mask = torch.ones(o_f.shape[0], dtype=torch.bool)
    mask[rows] = False
    assert not o_f[mask].any()
    if spec['state_fmt'] != OFF:
        _check_written_states(x, spec, saved, rec, heads, start)
    assert B.device_errors() == 0


@pytest.mark.parametrize("fmt,readout", [(INT8, BEFORE), (E4M3, AFTER), (OFF, AFTER)])
def test_decode_split_carry_is_bit_identical(fmt, readout):
    """Continuing a decode from its returned state equals the unsplit run
    bit for bit (the write is idempotent; the per-token arithmetic does not
    depend on where the run started)."""
    spec = _spec(state_fmt=fmt, T=257, B=2)
    x = draw(spec, 7)
    kw = dict(state_fmt=fmt, block_v=64, readout=readout)
    args = lambda y: [y[n] for n in ('q', 'k', 'v', 'g', 'beta')]
    o, ht, _ = B.gdn_decode_fwd(*args(x), _scale(spec), x['h0'], **kw)
    for a in (1, 64, 200):
        part = lambda lo, hi: {n: x[n][:, lo:hi].contiguous() for n in ('q', 'k', 'v', 'g', 'beta')}
        o1, h1, _ = B.gdn_decode_fwd(*args(part(0, a)), _scale(spec), x['h0'], **kw)
        o2, h2, _ = B.gdn_decode_fwd(*args(part(a, 257)), _scale(spec), h1, **kw)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([o1, o2], dim=1), o), a
        assert torch.equal(h2, ht), a
        # the same continuation through `start` on the whole buffer
        o3 = torch.zeros_like(o)
        o3, h3, _ = B.gdn_decode_fwd(*args(x), _scale(spec), h1, start=a, out=o3, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o3[:, a:], o[:, a:]) and torch.equal(h3, ht), a


PREFILL_CASES = [
    ('p64_int8_before', dict(), 64, BEFORE),
    ('p70_e4m3_after_w', dict(state_fmt=E4M3, w_fmt=E4M3), 70, AFTER),
    ('p64_packed_tails_gqa', dict(B=1, lengths=[257, 40, 3, 130], Hqk=2, Hv=4), 64, BEFORE),
    ('p128_off', dict(state_fmt=OFF), 128, AFTER),
    ('p0_decode_only', dict(state_fmt=E4M3, block_v=32), 0, BEFORE),
    ('p64_fp32_dk64', dict(dtype='f32', Dk=64, Dv=64, T=150, block_v=32), 64, AFTER),
]


@pytest.mark.parametrize("name,over,P,readout", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_decode_forward_and_backward_parity(name, over, P, readout):
    spec = _spec(**over)
    say(f"prefill+decode {name}: {spec} prefix={P} readout={readout}")
    x = draw(spec, 202, bwd=True)
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'],
              readout=readout)
    o, ht, saved = B.gdn_prefill_decode_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], P,
                                            _scale(spec), x['h0'], x['cu_seqlens'],
                                            save_for_backward=True, **kw)
    grads = B.gdn_prefill_decode_bwd(x['q'], x['k'], x['v'], x['g'], x['beta'], saved, x['do'],
                                     x['dht'], _scale(spec), x['h0'], x['cu_seqlens'],
                                     grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert B.device_errors() == 0
    sub = _full(x)
    o_ref, ht_ref = prefill_decode_fwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'],
                                       _scale(spec), P, sub['h0'], sub['cu'], **kw)
    r_o, r_h = rel(o.float().cpu(), o_ref), rel(ht.cpu(), ht_ref)
    say(f"  rel-L2 o={r_o:.3e} ht={r_h:.3e}")
    assert r_o <= _o_bar(spec) and r_h <= _h_bar(spec)
    want = prefill_decode_bwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'], _scale(spec),
                              P, sub['do'], sub['dht'], sub['h0'], sub['cu'], **kw)
    bar = 1e-2 if (spec['state_fmt'] != OFF or spec['w_fmt'] != OFF) else 3e-3
    for n in ('dq', 'dk', 'dv', 'dg', 'dbeta', 'dh0'):
        a = grads[n].float().cpu()
        assert torch.isfinite(a).all(), n
        r = rel(a, want[n])
        say(f"  {n}: rel-L2 {r:.3e}")
        assert r <= bar, (n, r)


BWD_CASES = [
    ('int8_before', dict(), 0, BEFORE),
    ('e4m3_after_gqa_bv16', dict(Hqk=2, Hv=4, state_fmt=E4M3, block_v=16), 0, AFTER),
    ('int8_dv256_bv256_after', dict(Dv=256, block_v=256, T=100), 0, AFTER),
    ('off_fp32_dk64', dict(state_fmt=OFF, dtype='f32', Dk=64, Dv=64, T=120), 0, BEFORE),
    ('e4m3_start33_packed', dict(B=1, lengths=[100, 5, 40], state_fmt=E4M3), 33, BEFORE),
]


@pytest.mark.parametrize("name,over,start,readout", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_decode_backward_parity(name, over, start, readout):
    spec = _spec(**over)
    say(f"decode bwd {name}: {spec} start={start} readout={readout}")
    x, o, ht, saved = _decode_run(spec, 303, start, readout)
    g = B.gdn_decode_bwd(x['q'], x['k'], x['v'], x['g'], x['beta'], saved, x['do'], x['dht'],
                         _scale(spec), x['h0'], x['cu_seqlens'], grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert B.device_errors() == 0
    sub = _full(x)
    want = decode_bwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'], _scale(spec),
                      sub['do'], sub['dht'], sub['h0'], sub['cu'], start, spec['state_fmt'],
                      spec['block_v'], readout)
    rows, _ = _decode_rows(x, spec, start)
    bar = 1e-2 if spec['state_fmt'] != OFF else 3e-3
    for n in ('dq', 'dk', 'dv', 'dg', 'dbeta'):
        a = g[n].float().cpu()
        a = a.reshape(-1, *a.shape[2:])[rows]
        b = want[n].reshape(-1, *want[n].shape[2:])[rows]
        assert torch.isfinite(a).all(), n
        r = rel(a, b)
        say(f"  {n}: rel-L2 {r:.3e}")
        assert r <= bar, (n, r)
    r = rel(g['dh_in'].cpu(), want['dh_in'])
    say(f"  dh_in: rel-L2 {r:.3e}")
    assert r <= bar


def test_decode_saved_stamp_refuses_another_policy():
    """A decode backward under another readout than the forward that wrote
    the saved buffer gets NaN gradients and the stamp flag, not silent
    numbers."""
    spec = _spec(T=70)
    x, o, ht, saved = _decode_run(spec, 5, 0, BEFORE)
    saved.gdn_decode = dict(saved.gdn_decode, readout=AFTER)
    g = B.gdn_decode_bwd(x['q'], x['k'], x['v'], x['g'], x['beta'], saved, x['do'], x['dht'],
                         _scale(spec), x['h0'], x['cu_seqlens'], grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert B.device_errors() == B.DEVERR_SAVED_STAMP
    assert torch.isnan(g['dq']).all() and torch.isnan(g['dh_in']).all()


def test_decode_moderate_size_sampled_heads():
    """257-token trajectories at H = 16, Dk = Dv = 128 (the chunk path's
    head size), E4M3 writes after a 64-token prefill; compared on sampled
    heads."""
    spec = _spec(B=4, Hqk=16, Hv=16, state_fmt=E4M3, w_fmt=E4M3)
    x = draw(spec, 11, bwd=True)
    o, ht, saved = B.gdn_prefill_decode_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], 64,
                                            _scale(spec), x['h0'], state_fmt=E4M3, w_fmt=E4M3,
                                            block_v=64, readout=AFTER)
    torch.cuda.synchronize()
    heads = [0, 7, 15]
    sub = head_subset(x, spec, heads)
    o_ref, ht_ref = prefill_decode_fwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'],
                                       _scale(spec), 64, sub['h0'], None, state_fmt=E4M3,
                                       w_fmt=E4M3, block_v=64, readout=AFTER)
    r_o, r_h = rel(o[:, :, heads].float().cpu(), o_ref), rel(ht[:, heads].cpu(), ht_ref)
    say(f"  rel-L2 o={r_o:.3e} ht={r_h:.3e}")
    assert r_o <= 1e-2 and r_h <= 1e-2
