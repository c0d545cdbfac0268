"""gdn_chunk_fwd_noalloc (the forward for callers that cannot allocate
device memory) against gdn_chunk_fwd through the C ABI: the same kernels on
the library's fixed scratch array instead of a caller workspace, so the
outputs are bit-identical. Two calls in a row, the second on a smaller
input (the array keeps the first call's contents), then a problem too large
for the array, which is refused before any launch."""
import pytest
import torch

import gdn_inputs
from gateddeltanet_chunked_recurrence_amd import binding as B
from parity_util import draw, gpu_fwd, head_subset, oracle_fwd, rel, say

pytestmark = pytest.mark.gpu


def _noalloc(x, spec):
    o, ht = B.gdn_chunk_fwd_noalloc(x['q'], x['k'], x['v'], x['g'], x['beta'],
                                    scale=spec['Dk'] ** -0.5, h0=x['h0'],
                                    cu_seqlens=x['cu_seqlens'], state_fmt=spec['state_fmt'],
                                    w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    torch.cuda.synchronize()
    return o, ht


def test_noalloc_forward_matches_workspace_forward_twice():
    big = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=2, T=1000, Hqk=2, Hv=4, h0=True)
    small = gdn_inputs.spec('varlen_int8_gqa4x16_d128', lengths=[130, 3, 64], Hqk=1, Hv=2)
    for spec, seed in ((big, 41), (small, 42)):
        say(f"noalloc forward {spec}")
        x = draw(spec, seed)
        o_ref, ht_ref, _ = gpu_fwd(x, spec)
        o, ht = _noalloc(x, spec)
        assert torch.equal(o, o_ref) and torch.equal(ht, ht_ref)
        heads = [0, 1]
        want_o, want_h = oracle_fwd(head_subset(x, spec, heads), spec)
        r_o, r_h = rel(o[:, :, heads].float(), want_o), rel(ht[:, heads], want_h)
        say(f"  rel-L2 vs oracle O={r_o:.3e} ht={r_h:.3e}")
        assert r_o <= 1e-2 and r_h <= 1e-2
    assert B.device_errors() == 0


def test_noalloc_refuses_a_problem_above_its_scratch():
    spec = gdn_inputs.spec('fwd_e4m3_b4_t4096_h16_d128', B=1, T=4096, Hqk=16, Hv=16)
    x = draw(spec, 43)
    with pytest.raises(B.GdnError, match='noalloc'):
        _noalloc(x, spec)
