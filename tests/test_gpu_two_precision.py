"""The two-precision profile on the GPU against the oracle ("[5/8] ReplaySSM
state QAT and two-precision GDN", "What does this PR do?" and "Usage": an
FP32 recurrence anchor, a dynamic E4M3 read copy grouped by 128 key channels
per value row, read errors never overwriting the anchor; "Testing":
first-order gradients).

Chunk-path reading (oracle/chunked.py): every read of a chunk's incoming
state (W S in Vnew, Q S in O) uses the per-value-column E4M3 copy Sr; the
carry keeps S in FP32. The forward is compared in full on small cases with
ragged chunks, grouped heads, packed sequences and h0 (bar 1e-2, QDQ on),
the saved read copy value by value against the oracle's record (one-step
code flips counted), the saved FP32 anchors against the oracle's states, a
closed form (beta = 0: ht is the exact decay of h0), and every gradient."""
import math

import numpy as np
import pytest
import torch

import gdn_inputs
from gateddeltanet_chunked_recurrence_amd import binding as B
from oracle.qdq import round_e4m3
from parity_util import draw, gpu_bwd, gpu_fwd, oracle_bwd, oracle_fwd, rel, say, seq_bounds

pytestmark = pytest.mark.gpu

OFF, E4M3, INT8 = 0, 1, 2
READ = dict(read_fmt=E4M3)

CASES = [
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=257, Hqk=2, Hv=4, state_fmt=OFF, w_fmt=OFF,
                                        h0=True)),
    ('varlen_int8_gqa4x16_d128', dict(lengths=[130, 0, 64, 3, 70], Hqk=1, Hv=2, state_fmt=OFF,
                                      w_fmt=E4M3)),
    ('long_e4m3_t65536_h32_dk128_dv256', dict(T=700, Hqk=1, Hv=2, state_fmt=OFF, w_fmt=INT8)),
]


def _full_sub(x):
    sub = dict(q=x['q'].double().cpu(), k=x['k'].double().cpu(), v=x['v'].double().cpu(),
               g=x['g'].double().cpu(), beta=x['beta'].double().cpu(),
               h0=None if x['h0'] is None else x['h0'].double().cpu(), cu=x['cu_list'])
    if 'do' in x:
        sub['do'] = x['do'].double().cpu()
        sub['dht'] = x['dht'].double().cpu()
    return sub


@pytest.mark.parametrize("name,over", CASES)
def test_two_precision_forward_matches_oracle(name, over):
    spec = gdn_inputs.spec(name, **over)
    say(f"two-precision fwd {spec}")
    x = draw(spec, 13)
    o, ht, saved = gpu_fwd(x, spec, save=True, **READ)
    assert torch.isfinite(o.float()).all() and torch.isfinite(ht).all()
    sub = _full_sub(x)
    rec = {}
    o_ref, ht_ref = oracle_fwd(sub, spec, record=rec, **READ)
    r_o, r_h = rel(o.float(), o_ref), rel(ht, ht_ref)
    o_off, ht_off = oracle_fwd(sub, spec)
    eff = rel(o_ref, o_off)
    say(f"  rel-L2 O={r_o:.3e} ht={r_h:.3e}; read-copy effect on O {eff:.3e}")
    assert r_o <= 1e-2 and r_h <= 1e-2
    # saved: the state section holds the read copy (codes times column
    # scales), the anchor section the FP32 state, per chunk slot
    lay = B.saved_layout(B.make_fwd_args(x['q'], x['k'], x['v'], x['g'], x['beta'], None, x['h0'],
                                         x['cu_seqlens'], OFF, spec['w_fmt'], 64, read_fmt=E4M3))
    Hv, Dk, Dv = spec['Hv'], spec['Dk'], spec['Dv']
    raw = saved.cpu()
    sr = raw[lay.off_state:lay.off_state + lay.num_slots * Hv * Dk * Dv * 4].view(torch.float32)
    sr = sr.view(lay.num_slots, Hv, Dk, Dv)
    an = raw[lay.off_anchor:lay.off_anchor + lay.num_slots * Hv * Dk * Dv * 4].view(torch.float32)
    an = an.view(lay.num_slots, Hv, Dk, Dv)
    # per column, the saved values are codes times the column scale, and the
    # column maximum is the code 448: so the scale is max / 448 and the codes
    # follow (rounded onto the grid); compare both with the oracle's record
    n_el = n_flip = 0
    worst_scale = worst_anchor = 0.0
    for n, (bos, eos) in enumerate(seq_bounds(x, spec)):
        for c in range((eos - bos + 63) // 64):
            slot = n + bos // 64 + c
            codes, d = rec['R'][0 if x['cu_list'] is None else n][c]
            codes = codes.reshape(-1, Hv, Dk, Dv)
            d = d.reshape(-1, Hv, 1, Dv)
            codes, d = (codes[n], d[n]) if x['cu_list'] is None else (codes[0], d[0])
            got = sr[slot].numpy()
            amax = np.abs(got).max(axis=1, keepdims=True)
            dg = np.where(amax > 0, amax / np.float32(448.0), d).astype(np.float32)
            cg = round_e4m3((got / dg).astype(np.float32))
            live = amax[:, 0] > 0
            worst_scale = max(worst_scale, float(np.max(np.abs(dg / d - 1)[:, 0][live], initial=0)))
            n_el += codes.size
            n_flip += int(np.sum(cg != codes))
        h0n = x['h0'][n].cpu() if x['h0'] is not None else torch.zeros(Hv, Dk, Dv)
        worst_anchor = max(worst_anchor, rel(an[n + bos // 64], h0n) if eos > bos else 0.0)
    frac = n_flip / max(n_el, 1)
    say(f"  read copy: {n_flip}/{n_el} codes differ ({frac:.2e}); max column scale rel diff "
        f"{worst_scale:.2e}; first anchor vs h0 {worst_anchor:.1e}")
    assert frac <= 1e-3 and worst_scale <= 1e-4 and worst_anchor == 0.0
    assert eff > 30 * r_o or r_o < 2e-3


def test_two_precision_zero_beta_anchor_is_exact_decay():
    """beta = 0: nothing is written, so the FP32 anchor only decays and ht is
    h0 times exp(sum g), while the quantized-carry profile's ht is not."""
    spec = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=1, T=300, Hqk=1, Hv=2, state_fmt=OFF,
                           w_fmt=OFF, h0=True, shift=-2.0)
    x = draw(spec, 14)
    x['beta'] = torch.zeros_like(x['beta'])
    _, ht, _ = gpu_fwd(x, spec, **READ)
    want = x['h0'][0].double().cpu() * torch.exp(x['g'][0].double().cpu().sum(0))[:, None, None]
    r = rel(ht[0], want)
    _, htq, _ = gpu_fwd(x, dict(spec, state_fmt=E4M3))
    rq = rel(htq[0], want)
    say(f"  beta = 0: ht vs exact decay {r:.2e} (quantized carry {rq:.2e})")
    assert r < 1e-5 and rq > 100 * r


@pytest.mark.parametrize("name,over", CASES[:2])
def test_two_precision_backward_matches_oracle(name, over):
    spec = gdn_inputs.spec(name, **over)
    say(f"two-precision bwd {spec}")
    x = draw(spec, 15, bwd=True)
    _, _, saved = gpu_fwd(x, spec, save=True, **READ)
    got = gpu_bwd(x, spec, saved)               # the profile comes from the saved buffer
    want = oracle_bwd(_full_sub(x), spec, **READ)
    off = oracle_bwd(_full_sub(x), spec)
    for n in ('dq', 'dk', 'dv', 'dg', 'dbeta', 'dh0'):
        if n not in want:
            continue
        r = rel(got[n].float(), want[n])
        say(f"  {n}: rel-L2 {r:.3e} (read-copy effect {rel(want[n], off[n]):.2e})")
        assert torch.isfinite(got[n].float()).all() and r <= 1e-2, (n, r)
