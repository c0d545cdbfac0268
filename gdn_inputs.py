"""Seeded synthetic inputs for the chunked gated delta rule.

Shared by the tests, smoke() and bench.py, and the only module that both the
oracle side and the HIP side of a comparison use. It draws random tensors and
shapes them; it holds none of the method's arithmetic.

Recipe (same for every workload; numbers per workload in WORKLOADS):
  q, k  ~ N(0, 1), L2-normalised per token in FP32, then cast to the input
          dtype (bf16 round-to-nearest-even, or kept FP32)
  v     ~ N(0, 1), cast to the input dtype
  beta  = sigmoid(N(0, 1))                                   (FP32)
  g     = -softplus(N(0, 1) + shift)   for gate = 'softplus'   (FP32)
          log(U[0.9, 0.999])           for gate = 'retention'
  h0    ~ N(0, 0.1^2) (FP32) when the workload has an initial state
  do    ~ N(0, 1) (input dtype), dht ~ N(0, 0.1^2) (FP32) for the backward
Draw order is fixed (q, k, v, beta, g, h0, do, dht) so a seed pins the data.
"""
import torch

FMT_OFF, FMT_E4M3, FMT_INT8 = 0, 1, 2

WORKLOADS = {
    'tiny_fp32': dict(B=1, T=128, Hqk=2, Hv=2, Dk=64, Dv=64, dtype='f32',
                      gate='softplus', shift=0.0, h0=False,
                      state_fmt=FMT_OFF, w_fmt=FMT_OFF, block_v=64),
    'fwd_e4m3_b4_t4096_h16_d128': dict(B=4, T=4096, Hqk=16, Hv=16, Dk=128, Dv=128,
                                       dtype='bf16', gate='softplus', shift=2.0, h0=False,
                                       state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=64),
    'varlen_int8_gqa4x16_d128': dict(B=1, lengths=[257, 1000, 3, 4096, 640], Hqk=4, Hv=16,
                                     Dk=128, Dv=128, dtype='bf16', gate='softplus', shift=0.0,
                                     h0=True, state_fmt=FMT_INT8, w_fmt=FMT_OFF, block_v=64),
    'long_e4m3_t65536_h32_dk128_dv256': dict(B=1, T=65536, Hqk=32, Hv=32, Dk=128, Dv=256,
                                             dtype='bf16', gate='retention', shift=0.0,
                                             h0=False, state_fmt=FMT_E4M3, w_fmt=FMT_E4M3,
                                             block_v=64),
    'fwd_bwd_e4m3_b2_t8192_h16_d128': dict(B=2, T=8192, Hqk=16, Hv=16, Dk=128, Dv=128,
                                           dtype='bf16', gate='softplus', shift=0.0, h0=True,
                                           state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=64,
                                           bwd=True),
    # decode continuation: 257-token trajectories, a 64-token chunk prefill,
    # then token-state writes
    'decode_e4m3_b4_t257_p64_h16_d128': dict(B=4, T=257, Hqk=16, Hv=16, Dk=128, Dv=128,
                                             dtype='bf16', gate='softplus', shift=0.0, h0=True,
                                             state_fmt=FMT_E4M3, w_fmt=FMT_E4M3, block_v=64,
                                             bwd=True, prefix_len=64),
}

# The five workloads in the order the parity suite and the bench refer to them.
ORDER = ['tiny_fp32', 'fwd_e4m3_b4_t4096_h16_d128', 'varlen_int8_gqa4x16_d128',
         'long_e4m3_t65536_h32_dk128_dv256', 'fwd_bwd_e4m3_b2_t8192_h16_d128']


def spec(name, **overrides):
    s = dict(WORKLOADS[name])
    s.update(overrides)
    return s


def _to_dtype(x, dtype):
    return x.to(torch.bfloat16) if dtype == 'bf16' else x.to(torch.float32)


def make_inputs(s, seed, device='cpu', bwd=None):
    """Draw one workload. Returns a dict of tensors on `device`:
    q, k [B, T, Hqk, Dk]; v [B, T, Hv, Dv]; g, beta [B, T, Hv] (FP32);
    h0 [N, Hv, Dk, Dv] or None; cu_seqlens (int32, N+1) or None;
    do [B, T, Hv, Dv], dht [N, Hv, Dk, Dv] when bwd; plus 'cu_list' (python
    offsets or None) and 'N'."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if 'lengths' in s:
        lens = list(s['lengths'])
        B, T = 1, sum(lens)
        cu = [0]
        for n in lens:
            cu.append(cu[-1] + n)
    else:
        B, T = s['B'], s['T']
        cu = None
    N = len(cu) - 1 if cu is not None else B
    Hqk, Hv, Dk, Dv = s['Hqk'], s['Hv'], s['Dk'], s['Dv']
    f32 = dict(device=device, dtype=torch.float32, generator=gen)

    q = torch.randn(B, T, Hqk, Dk, **f32)
    k = torch.randn(B, T, Hqk, Dk, **f32)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn(B, T, Hv, Dv, **f32)
    beta = torch.sigmoid(torch.randn(B, T, Hv, **f32))
    if s['gate'] == 'softplus':
        g = -torch.nn.functional.softplus(torch.randn(B, T, Hv, **f32) + s['shift'])
    elif s['gate'] == 'retention':
        g = torch.log(0.9 + 0.099 * torch.rand(B, T, Hv, **f32))
    else:
        raise ValueError(s['gate'])
    h0 = 0.1 * torch.randn(N, Hv, Dk, Dv, **f32) if s['h0'] else None
    out = dict(q=_to_dtype(q, s['dtype']).contiguous(), k=_to_dtype(k, s['dtype']).contiguous(),
               v=_to_dtype(v, s['dtype']).contiguous(), g=g.contiguous(),
               beta=beta.contiguous(), h0=h0, N=N, cu_list=cu,
               cu_seqlens=None if cu is None else torch.tensor(cu, dtype=torch.int32,
                                                                device=device))
    if bwd if bwd is not None else s.get('bwd', False):
        out['do'] = _to_dtype(torch.randn(B, T, Hv, Dv, **f32), s['dtype']).contiguous()
        out['dht'] = 0.1 * torch.randn(N, Hv, Dk, Dv, **f32)
    return out
