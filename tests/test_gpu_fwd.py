"""Forward parity of the HIP path (through the C ABI) against the float64
oracle on the same seeded inputs.

Bars: QDQ off rel-L2 <= 2e-3 on O and ht; QDQ on rel-L2 <= 1e-2. Small cases
span several chunks and ragged tails and are compared in full; the five
named workloads run at full size on the GPU and are compared on sampled
value heads (heads are independent, so the oracle computes exactly those).
Exported QDQ codes and scales are compared with the oracle's, since the QDQ
effect on O alone can sit below the tolerance."""
import numpy as np
import pytest
import torch

import gdn_inputs
from gateddeltanet_chunked_recurrence_amd import binding as B
from parity_util import (code_bytes, draw, gpu_fwd, head_subset, oracle_fwd, rel, saved_views,
                         say, seq_bounds)

pytestmark = pytest.mark.gpu

OFF, E4M3, INT8 = 0, 1, 2


def _bar(spec):
    return 2e-3 if (spec['state_fmt'] == OFF and spec['w_fmt'] == OFF) else 1e-2


def _check_fwd(spec, seed, heads, save=True, code_checks=True):
    say(f"fwd {spec} seed={seed} heads={heads}")
    x = draw(spec, seed)
    o, ht, saved = gpu_fwd(x, spec, save=save)
    assert torch.isfinite(o.float()).all() and torch.isfinite(ht).all()
    sub = head_subset(x, spec, heads)
    rec = {}
    o_ref, ht_ref = oracle_fwd(sub, spec, record=rec)
    r_o = rel(o[:, :, heads].float(), o_ref)
    r_h = rel(ht[:, heads], ht_ref)
    say(f"  rel-L2 O={r_o:.3e} ht={r_h:.3e}")
    bar = _bar(spec)
    assert r_o <= bar and r_h <= bar
    if save and code_checks:
        _check_codes(x, spec, saved, rec, heads)
    assert B.device_errors() == 0                  # no bounded wait gave up
    return x, o, ht, r_o, r_h


def _canon(codes, fmt):
    """E4M3 codes 0x80 (-0) and 0x00 (+0) dequantize to the same zero; the
    GPU can produce an exact zero where the oracle has a tiny signed value."""
    codes = np.asarray(codes)
    return np.where(codes == 0x80, 0, codes) if fmt == E4M3 else codes


def _check_codes(x, spec, saved, rec, heads):
    """Exported codes and scales vs the oracle's record of the same sites.
    Codes may differ where the FP32 value sits within rounding noise of a
    grid midpoint (a one-step flip); scales follow the tile amax, a computed
    FP32 value, so they agree to its precision (~2^-16 relative)."""
    sv = saved_views(saved, x, spec)
    bounds = seq_bounds(x, spec)
    n_el = n_flip = 0
    max_scale_rel = 0.0
    for n, (bos, eos) in enumerate(bounds):
        nchunks = (eos - bos + 63) // 64
        for c in range(nchunks):
            slot = n + bos // 64 + c
            if spec['state_fmt']:
                # oracle record: per sequence n, chunk c: codes [Z, Dk, nb, bv], Z = heads
                # (varlen) or B*heads (batched)
                cz, dz = rec['S'][0 if x['cu_list'] is None else n][c]
                Hs = len(heads)
                if x['cu_list'] is None:
                    cz = cz.reshape(-1, Hs, *cz.shape[1:])[n]
                    dz = dz.reshape(-1, Hs, *dz.shape[1:])[n]
                want = _canon(code_bytes(cz.reshape(Hs, spec['Dk'], spec['Dv']),
                                         spec['state_fmt']), spec['state_fmt'])
                got = _canon(sv['S'][slot, heads].numpy(), spec['state_fmt'])
                n_el += want.size
                n_flip += int((got != want).sum())
                dg = sv['dS'][slot, heads].numpy()
                dw = dz.reshape(Hs, -1)
                max_scale_rel = max(max_scale_rel, float(np.max(np.abs(dg / dw - 1))))
            if spec['w_fmt']:
                cz, dz = rec['W'][0 if x['cu_list'] is None else n][c]
                Hs = len(heads)
                if x['cu_list'] is None:
                    cz = cz.reshape(-1, Hs, *cz.shape[1:])[n]
                    dz = dz.reshape(-1, Hs)[n]
                t0 = bos + 64 * c
                t1 = min(t0 + 64, eos)
                want = _canon(code_bytes(cz, spec['w_fmt']), spec['w_fmt'])   # [Hs, nc, Dk]
                got = _canon(sv['W'][t0:t1][:, heads].permute(1, 0, 2).numpy(), spec['w_fmt'])
                n_el += want.size
                n_flip += int((got != want).sum())
                dg = sv['dW'][slot, heads].numpy()
                max_scale_rel = max(max_scale_rel, float(np.max(np.abs(dg / dz.reshape(-1) - 1))))
    frac = n_flip / max(n_el, 1)
    say(f"  codes: {n_flip}/{n_el} differ ({frac:.2e}); max scale rel diff {max_scale_rel:.2e}")
    assert frac <= 1e-3
    assert max_scale_rel <= 1e-4


# ------------------------------------------------------------ small, full compare

SMALL = [
    # (name, overrides)
    ('tiny_fp32', {}),
    ('tiny_fp32', dict(T=257, Hqk=1, Hv=3, h0=True)),
    ('tiny_fp32', dict(T=200, state_fmt=E4M3, w_fmt=E4M3, block_v=32, h0=True)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=257, Hqk=2, Hv=4)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=1, T=300, Hqk=1, Hv=2, state_fmt=OFF, w_fmt=OFF,
                                        shift=0.0, h0=True)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=1, T=130, Hqk=1, Hv=2, Dk=64, Dv=256, block_v=16,
                                        gate='retention')),
    ('varlen_int8_gqa4x16_d128', dict(lengths=[257, 3, 70, 1, 64, 130], Hqk=2, Hv=4)),
    ('varlen_int8_gqa4x16_d128', dict(lengths=[100, 65], Hqk=1, Hv=2, state_fmt=INT8,
                                      w_fmt=INT8, block_v=32, gate='retention')),
    ('varlen_int8_gqa4x16_d128', dict(lengths=[200, 64], Hqk=1, Hv=2, state_fmt=OFF, w_fmt=E4M3,
                                      Dv=64)),
    ('long_e4m3_t65536_h32_dk128_dv256', dict(T=1000, Hqk=2, Hv=2)),
    # mixed formats at the two sites (each state-kernel format pair is covered)
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=1, T=260, Hqk=1, Hv=2, state_fmt=INT8, w_fmt=E4M3,
                                        h0=True)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=1, T=199, Hqk=1, Hv=2, state_fmt=E4M3, w_fmt=INT8,
                                        Dk=64, Dv=128, block_v=32)),
    # one 64-wide value block per head, varlen with short and empty-tail sequences
    ('varlen_int8_gqa4x16_d128', dict(lengths=[130, 64, 1, 65], Hqk=1, Hv=2, Dv=64,
                                      state_fmt=E4M3, w_fmt=E4M3, block_v=64, h0=True)),
    # state scale tiles wider than one 64-column value block: the workgroup
    # spans the tile (8 or 16 waves), both QDQ sites on or mixed formats
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=1, T=200, Hqk=1, Hv=2, block_v=128, h0=True)),
    ('long_e4m3_t65536_h32_dk128_dv256', dict(T=300, Hqk=1, Hv=2, block_v=256, w_fmt=INT8)),
    ('varlen_int8_gqa4x16_d128', dict(lengths=[130, 3, 70], Hqk=1, Hv=2, Dv=256, block_v=128,
                                      h0=True)),
    ('varlen_int8_gqa4x16_d128', dict(lengths=[100, 65], Hqk=1, Hv=2, Dk=64, Dv=256, block_v=256,
                                      state_fmt=E4M3, w_fmt=E4M3)),
    # empty sequences first, between and last: their ht is h0, they own no chunk
    ('varlen_int8_gqa4x16_d128', dict(lengths=[0, 130, 0, 64, 1, 0], Hqk=1, Hv=2,
                                      state_fmt=E4M3, w_fmt=E4M3, h0=True)),
]


@pytest.mark.parametrize("name,over", SMALL)
def test_fwd_small_full_parity(name, over):
    spec = gdn_inputs.spec(name, **over)
    _check_fwd(spec, seed=11, heads=list(range(spec['Hv'])))


def test_fwd_qdq_off_bf16_meets_2e3_and_internal_error_small():
    """QDQ off with bf16 I/O: O's own bf16 rounding costs ~1.6e-3, so the
    kernel's internal error must stay far below it; ht (FP32) shows it."""
    spec = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=1, T=1024, Hqk=2, Hv=2,
                           state_fmt=OFF, w_fmt=OFF, shift=0.0, h0=True)
    _, _, _, r_o, r_h = _check_fwd(spec, seed=12, heads=[0, 1])
    assert r_h <= 2e-4


# ------------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("name,heads", [
    ('tiny_fp32', [0, 1]),
    ('fwd_e4m3_b4_t4096_h16_d128', [0, 9]),
    ('varlen_int8_gqa4x16_d128', [0, 13]),
    ('long_e4m3_t65536_h32_dk128_dv256', [5]),
])
def test_fwd_workload_parity(name, heads):
    spec = gdn_inputs.spec(name)
    _check_fwd(spec, seed=gdn_inputs.ORDER.index(name) + 1, heads=heads)


def test_fwd_workload5_forward_parity():
    spec = gdn_inputs.spec('fwd_bwd_e4m3_b2_t8192_h16_d128')
    _check_fwd(spec, seed=5, heads=[3])


# ------------------------------------------------------------ properties

def test_fwd_deterministic_and_split_carry():
    spec = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=1, T=640, Hqk=2, Hv=4, h0=True)
    x = draw(spec, 21)
    o1, h1, _ = gpu_fwd(x, spec)
    o2, h2, _ = gpu_fwd(x, spec)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    # split carry at a chunk boundary: run 384 tokens, continue from ht
    cut = 384
    xa = dict(x, q=x['q'][:, :cut].contiguous(), k=x['k'][:, :cut].contiguous(),
              v=x['v'][:, :cut].contiguous(), g=x['g'][:, :cut].contiguous(),
              beta=x['beta'][:, :cut].contiguous())
    xb = dict(x, q=x['q'][:, cut:].contiguous(), k=x['k'][:, cut:].contiguous(),
              v=x['v'][:, cut:].contiguous(), g=x['g'][:, cut:].contiguous(),
              beta=x['beta'][:, cut:].contiguous())
    oa, ha, _ = gpu_fwd(xa, dict(spec, T=cut))
    xb['h0'] = ha
    ob, hb, _ = gpu_fwd(xb, dict(spec, T=640 - cut))
    assert torch.equal(torch.cat([oa, ob], dim=1), o1)
    assert torch.equal(hb, h1)


def test_fwd_qdq_effect_visible_and_tracked():
    """Slow-decay gates make the state QDQ visible in O; the GPU must sit far
    closer to the QDQ oracle than the QDQ oracle sits to the QDQ-off one."""
    spec = gdn_inputs.spec('long_e4m3_t65536_h32_dk128_dv256', T=2048, Hqk=2, Hv=2, Dv=128)
    x = draw(spec, 31)
    o, ht, _ = gpu_fwd(x, spec)
    sub = head_subset(x, spec, [0, 1])
    o_q, _ = oracle_fwd(sub, spec)
    o_off, _ = oracle_fwd(sub, spec, state_fmt=OFF, w_fmt=OFF)
    r_gpu = rel(o.float(), o_q)
    r_eff = rel(o_q, o_off)
    say(f"  gpu vs oracle {r_gpu:.3e}; qdq effect {r_eff:.3e}")
    assert r_eff > 5 * r_gpu


def test_fwd_fp16_operand_range_is_checked():
    """With both QDQ sites on, the masked Q K^T operand is kept in fp16; an
    entry beyond its +-65504 range (q . k that large: unnormalised inputs)
    raises the device error flag instead of passing an infinity on silently.
    Normalised inputs of the same shape raise nothing."""
    spec = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=1, T=128, Hqk=1, Hv=1)
    x = draw(spec, 77)
    assert B.device_errors() == 0
    gpu_fwd(x, spec)
    assert B.device_errors() == 0
    big = dict(x)
    big["q"] = (x["q"].float() * 1000.0).to(torch.bfloat16).contiguous()
    big["k"] = (x["k"].float() * 1000.0).to(torch.bfloat16).contiguous()
    gpu_fwd(big, spec)
    assert B.device_errors() == B.DEVERR_P_RANGE


@pytest.mark.parametrize("name,over", [
    ('fwd_e4m3_b4_t4096_h16_d128', dict()),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=1000, Hqk=4, Hv=8, state_fmt=INT8)),
    ('long_e4m3_t65536_h32_dk128_dv256', dict(T=8192)),
    ('fwd_bwd_e4m3_b2_t8192_h16_d128', dict()),
    # four items only: fewer than the CUs the chain leaves, no head
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=1, T=256, Hqk=1, Hv=1)),
    # Dk 64, INT8 W, 32-wide scale tiles, ragged last chunk, h0
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=3, T=777, Hqk=2, Hv=6, Dk=64, Dv=64, w_fmt=INT8,
                                        block_v=32, h0=True)),
    # the general state kernel: QDQ off, INT8 state with W off, 128- and 256-wide tiles
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=2048, state_fmt=OFF, w_fmt=OFF, h0=True)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=1500, Hqk=4, Hv=8, state_fmt=INT8, w_fmt=OFF)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=1000, Hqk=2, Hv=4, block_v=128, w_fmt=INT8)),
    ('long_e4m3_t65536_h32_dk128_dv256', dict(T=2048, Hqk=4, Hv=4, block_v=256)),
    ('fwd_e4m3_b4_t4096_h16_d128', dict(B=2, T=900, Hqk=2, Hv=2, Dk=64, Dv=128, state_fmt=OFF,
                                        w_fmt=E4M3)),
])
def test_fwd_overlapped_schedule_equals_serial(name, over):
    """gdn_chunk_fwd runs the prep's remainder concurrently with the state
    chain (ready flags per chunk) where the state kernel leaves CUs idle; its
    outputs and saved buffer equal the serial two-stage schedule bit for bit,
    and no bounded wait gives up."""
    import math
    spec = gdn_inputs.spec(name, **over)
    x = draw(spec, 31)
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    sc = 1.0 / math.sqrt(spec['Dk'])
    o1, h1, s1 = B.gdn_chunk_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], sc, x['h0'],
                                 save_for_backward=True, **kw)
    plan = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], sc, x['h0'], save=True, **kw)
    assert plan.schedule()['overlapped']
    plan.saved.zero_()
    plan.prep()
    plan.state()
    torch.cuda.synchronize()
    assert B.device_errors() == 0
    assert torch.equal(o1, plan.o) and torch.equal(h1, plan.ht)
    s_serial = plan.saved.clone()
    plan.saved.zero_()
    plan.o.zero_()
    plan.forward()
    torch.cuda.synchronize()
    assert B.device_errors() == 0
    assert torch.equal(o1, plan.o) and torch.equal(h1, plan.ht)
    assert torch.equal(s_serial, plan.saved)
    say(f"  {name} {over}: overlapped == serial")


@pytest.mark.parametrize("over", [dict(), dict(state_fmt=OFF, w_fmt=OFF)])
def test_fwd_overlapped_reads_no_stale_workspace(over):
    """The overlapped forward reads each chunk's operands after its ready
    flag: with the workspace still holding another input's operands from the
    call before, every call equals the serial schedule on its own input."""
    import math
    spec = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=2, T=2048, **over)
    xs = [draw(spec, 41), draw(spec, 42)]
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    sc = 1.0 / math.sqrt(spec['Dk'])
    ref = []
    for x in xs:
        p = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], sc, x['h0'], **kw)
        p.prep()
        p.state()
        ref.append((p.o.clone(), p.ht.clone()))
    live = {n: xs[0][n].clone() for n in ('q', 'k', 'v', 'g', 'beta')}
    plan = B.FwdPlan(live['q'], live['k'], live['v'], live['g'], live['beta'], sc, None, **kw)
    assert plan.schedule()['overlapped']
    for i in (0, 1, 0, 1, 1, 0):
        for n in live:
            live[n].copy_(xs[i][n])
        plan.forward()
        torch.cuda.synchronize()
        assert B.device_errors() == 0
        assert torch.equal(plan.o, ref[i][0]) and torch.equal(plan.ht, ref[i][1]), i
    say("  overlapped calls alternating inputs on one workspace: each equals its serial run")


@pytest.mark.parametrize("over", [
    dict(),                                             # INT8 state, W off: the general kernel
    dict(state_fmt=E4M3, w_fmt=E4M3),                   # both sites on: the split kernel
    dict(lengths=[0, 700, 1, 130, 0, 2048], state_fmt=E4M3, w_fmt=INT8, block_v=32),
])
def test_fwd_overlapped_packed_equals_serial(over):
    """Packed sequences (cu_seqlens) take the overlapped forward with an item
    order and split that a setup kernel derives from the lengths on the
    device (longest sequences first within each chunk index); o, ht and the
    saved buffer equal the two stages run one after the other, with empty
    and one-token sequences too, and no bounded wait gives up."""
    import math
    spec = gdn_inputs.spec('varlen_int8_gqa4x16_d128', **over)
    x = draw(spec, 71)
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    sc = 1.0 / math.sqrt(spec['Dk'])
    plan = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], sc, x['h0'], x['cu_seqlens'],
                     save=True, **kw)
    sch = plan.schedule()
    assert sch['overlapped'] and sch['items'] == -1 and sch['head_items'] == -1
    plan.saved.zero_()
    plan.prep()
    plan.state()
    torch.cuda.synchronize()
    assert B.device_errors() == 0
    o_s, h_s, s_s = plan.o.clone(), plan.ht.clone(), plan.saved.clone()
    for _ in range(2):
        plan.saved.zero_()
        plan.o.zero_()
        plan.forward()
        torch.cuda.synchronize()
        assert B.device_errors() == 0
        assert torch.equal(plan.o, o_s) and torch.equal(plan.ht, h_s)
        assert torch.equal(plan.saved, s_s)
    say(f"  packed {over}: overlapped == serial")


@pytest.mark.parametrize("packed", [False, True])
def test_fwd_overlapped_prefix_equals_serial(packed):
    """With prefix_len (the prefill of a decode continuation) the overlapped
    forward builds and consumes only the chunks of each sequence's prefix:
    equal-length sequences size the schedule from the prefix, packed ones
    cap every length in the setup kernel. o (prefix rows), ht and the saved
    buffer equal the two stages in series."""
    import math
    over = dict(lengths=[300, 1500, 64, 2048, 0, 777]) if packed else dict(B=2, T=1024)
    name = 'varlen_int8_gqa4x16_d128' if packed else 'fwd_e4m3_b4_t4096_h16_d128'
    spec = gdn_inputs.spec(name, state_fmt=E4M3, w_fmt=E4M3, **over)
    x = draw(spec, 73)
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    sc = 1.0 / math.sqrt(spec['Dk'])
    plan = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], sc, x['h0'], x['cu_seqlens'],
                     save=True, prefix_len=700, **kw)
    sch = plan.schedule()
    assert sch['overlapped']
    if not packed:
        assert sch['items'] == 11 * 2 * spec['Hv']      # 700 tokens: 11 chunks per sequence
    plan.saved.zero_()
    plan.o.zero_()
    plan.prep()
    plan.state()
    torch.cuda.synchronize()
    assert B.device_errors() == 0
    o_s, h_s, s_s = plan.o.clone(), plan.ht.clone(), plan.saved.clone()
    for _ in range(2):
        plan.saved.zero_()
        plan.o.zero_()
        plan.forward()
        torch.cuda.synchronize()
        assert B.device_errors() == 0
        assert torch.equal(plan.o, o_s) and torch.equal(plan.ht, h_s)
        assert torch.equal(plan.saved, s_s)
    say(f"  prefix 700, packed={packed}: overlapped == serial")
