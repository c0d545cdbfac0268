"""Helpers shared by the GPU parity tests: run the HIP path through the
binding, run the oracle on the same (device-drawn) inputs for a subset of
value heads, and compare."""
import math
import sys

import numpy as np
import torch

import gdn_inputs
from gateddeltanet_chunked_recurrence_amd import binding as B
from oracle import chunked_fwd, chunked_bwd


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel(a, b):
    a = torch.as_tensor(a).double().cpu()
    b = torch.as_tensor(b).double().cpu()
    den = float(b.norm())
    return float((a - b).norm()) / max(den, 1e-300)


def draw(spec, seed, bwd=False):
    return gdn_inputs.make_inputs(spec, seed, device='cuda', bwd=bwd)


def gpu_fwd(x, spec, save=False, **over):
    p = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    p.update(over)
    o, ht, saved = B.gdn_chunk_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'],
                                   scale=1.0 / math.sqrt(spec['Dk']), h0=x['h0'],
                                   cu_seqlens=x['cu_seqlens'], save_for_backward=save, **p)
    torch.cuda.synchronize()
    return o, ht, saved


def head_subset(x, spec, heads):
    """CPU float64 copies restricted to value heads `heads`; the query/key
    head of each is gathered so the subset has Hqk = Hv = len(heads)."""
    G = spec['Hv'] // spec['Hqk']
    qk = [h // G for h in heads]
    sub = dict(q=x['q'][:, :, qk].double().cpu(), k=x['k'][:, :, qk].double().cpu(),
               v=x['v'][:, :, heads].double().cpu(), g=x['g'][:, :, heads].double().cpu(),
               beta=x['beta'][:, :, heads].double().cpu(),
               h0=None if x['h0'] is None else x['h0'][:, heads].double().cpu(),
               cu=x['cu_list'])
    if 'do' in x:
        sub['do'] = x['do'][:, :, heads].double().cpu()
        sub['dht'] = x['dht'][:, heads].double().cpu()
    return sub


def oracle_fwd(sub, spec, record=None, **over):
    p = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    p.update(over)
    return chunked_fwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'],
                       1.0 / math.sqrt(spec['Dk']), sub['h0'], sub['cu'], record=record, **p)


def oracle_bwd(sub, spec, **over):
    p = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    p.update(over)
    return chunked_bwd(sub['q'], sub['k'], sub['v'], sub['g'], sub['beta'],
                       1.0 / math.sqrt(spec['Dk']), sub['do'], sub['dht'], sub['h0'], sub['cu'],
                       **p)


def seq_bounds(x, spec):
    if x['cu_list'] is not None:
        return list(zip(x['cu_list'][:-1], x['cu_list'][1:]))
    T = spec['T']
    return [(b * T, (b + 1) * T) for b in range(spec['B'])]


def saved_views(saved, x, spec, **over):
    """Decode the saved buffer into (state codes/values, state scales, W codes,
    W scales) as CPU tensors (see gdn_saved_layout in include/gdn.h)."""
    p = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    p.update(over)
    a = B.make_fwd_args(x['q'], x['k'], x['v'], x['g'], x['beta'], None, x['h0'],
                        x['cu_seqlens'], p['state_fmt'], p['w_fmt'], p['block_v'])
    lay = B.saved_layout(a)
    raw = saved.cpu()
    Hv, Dk, Dv = spec['Hv'], spec['Dk'], spec['Dv']
    ns = lay.num_slots
    out = {}
    if p['state_fmt']:
        out['S'] = raw[lay.off_state: lay.off_state + ns * Hv * Dk * Dv].view(ns, Hv, Dk, Dv)
        out['dS'] = raw[lay.off_state_scale: lay.off_state_scale + ns * Hv * (Dv // p['block_v']) * 4] \
            .view(torch.float32).view(ns, Hv, Dv // p['block_v'])
    else:
        out['S'] = raw[lay.off_state: lay.off_state + ns * Hv * Dk * Dv * 4].view(torch.float32) \
            .view(ns, Hv, Dk, Dv)
    if p['w_fmt']:
        ntok = x['q'].shape[0] * x['q'].shape[1]
        out['W'] = raw[lay.off_w: lay.off_w + ntok * Hv * Dk].view(ntok, Hv, Dk)
        out['dW'] = raw[lay.off_w_scale: lay.off_w_scale + ns * Hv * 4].view(torch.float32) \
            .view(ns, Hv)
    out['num_slots'] = ns
    return out


def code_bytes(codes, fmt):
    """Oracle code values -> the one-byte encoding the kernels export."""
    from oracle.qdq import e4m3_encode
    c = np.asarray(codes)
    if fmt == 1:
        return e4m3_encode(c)
    return c.astype(np.int8).view(np.uint8)


def gpu_bwd(x, spec, saved, grad_dtype=torch.float32, **over):
    p = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    p.update(over)
    g = B.gdn_chunk_bwd(x['q'], x['k'], x['v'], x['g'], x['beta'], saved, x['do'],
                        dht=x['dht'], scale=1.0 / math.sqrt(spec['Dk']), h0=x['h0'],
                        cu_seqlens=x['cu_seqlens'], grad_dtype=grad_dtype, **p)
    torch.cuda.synchronize()
    assert B.device_errors() == 0                   # saved stamp matched, no wait gave up
    return g
