"""Throughput of the chunked gated delta rule forward with FP8 E4M3 state and
W fake QDQ on one MI355X, against the bf16 MFMA roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one gdn_chunk_fwd call over B=4 sequences of T=4096 tokens, 16
heads, Dk = Dv = 128, state E4M3 with [128, 64] scale tiles, W E4M3 per
(chunk, head): the whole forward path (gates, gated K K^T, exact solve, W/U,
both QDQ sites, the sequential state recurrence, the output) runs in one
kernel launch, with inputs resident in HBM. Prints one JSON line.

Roofline: algorithmic FLOPs per token and head at full 64x64 tiles,
F = 2 (3 C Dk + 2 C Dv + 3 Dk Dv) + C^2 / 3 (C = 64; K K^T, W, Q K^T; U, P V;
W S, K^T Vnew, Q S; the solve) = 181 589 for Dk = Dv = 128, divided by the
kernel's average duration (HIP events around the timed launches on the
launch stream), against the dense bf16 MFMA peak of 2.5 PFLOP/s.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunk fwd(+bwd) tokens/s and % bf16 MFMA peak, FP8 state+W QDQ on"
WORKLOAD = 'fwd_e4m3_b4_t4096_h16_d128'
PEAK_BF16_TFLOPS = 2500.0
CHUNK = 64


def flops_per_token_head(Dk, Dv, C=CHUNK):
    return 2 * (3 * C * Dk + 2 * C * Dv + 3 * Dk * Dv) + C * C / 3.0


def bytes_algorithmic(spec):
    """Minimum HBM bytes of one forward: read q, k, v (bf16), g, beta (FP32),
    h0 if any; write o (bf16) and ht (FP32)."""
    B, T, Hqk, Hv, Dk, Dv = (spec[k] for k in ('B', 'T', 'Hqk', 'Hv', 'Dk', 'Dv'))
    tok = B * T
    rd = tok * (2 * Hqk * Dk * 2 + Hv * Dv * 2 + 2 * Hv * 4)
    wr = tok * Hv * Dv * 2 + B * Hv * Dk * Dv * 4
    return rd + wr


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, 'gateddeltanet_chunked_recurrence_amd', 'csrc')
    for f in sorted(os.listdir(csrc)):
        if f.endswith(('.hip', '.h', '.cpp')):
            h.update(open(os.path.join(csrc, f), 'rb').read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, 'profiles', f'{kernel}_{WORKLOAD}_traffic.json')
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get('source_hash') != src_hash:
        return None
    return d.get('bytes_per_launch')


def cpu_baseline(spec, seed):
    """The float64 oracle on a bounded sample of the same workload: `nseq` of
    the B sequences, full length, all heads (sequences are independent)."""
    import torch

    import gdn_inputs
    from oracle import chunked_fwd
    nseq = 3
    s = dict(spec, B=nseq)
    x = gdn_inputs.make_inputs(s, seed, device='cpu')
    args = [x[n].double() for n in ('q', 'k', 'v', 'g', 'beta')]
    t = time.perf_counter()
    chunked_fwd(*args, 1.0 / math.sqrt(spec['Dk']), None, None, state_fmt=spec['state_fmt'],
                w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    dt = time.perf_counter() - t
    ntok = nseq * spec['T']
    return dict(value=ntok / dt, unit='tokens/s', cores=torch.get_num_threads(), kind='oracle',
                sample=f'{nseq} of {spec["B"]} sequences x {spec["T"]} tokens x {spec["Hv"]} heads '
                       f'(float64 chunked oracle, {dt:.1f} s)')


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument('--gpus', type=int, default=1)
    ap.add_argument('--steps', type=int, default=50)
    ap.add_argument('--warmup', type=int, default=10)
    ap.add_argument('--no-cpu-baseline', action='store_true')
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get('WORLD_SIZE', '1')) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(heads/sequences shard with no communication; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gdn_inputs
    from gateddeltanet_chunked_recurrence_amd import binding as B

    spec = gdn_inputs.spec(WORKLOAD)
    x = gdn_inputs.make_inputs(spec, seed=2, device='cuda')
    scale = 1.0 / math.sqrt(spec['Dk'])
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])

    def step():
        return B.gdn_chunk_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], scale=scale, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / args.steps          # one launch per step
    ms_per_step = wall * 1e3 / args.steps

    tokens = spec['B'] * spec['T']
    token_heads = tokens * spec['Hv']
    flops = flops_per_token_head(spec['Dk'], spec['Dv']) * token_heads
    achieved = flops / (kern_ms * 1e-3) / 1e12
    src = source_hash()
    traffic = measured_traffic('gdn_fwd_kernel', src)
    out = dict(
        metric=METRIC, value=tokens / (ms_per_step * 1e-3), unit='tokens/s', n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True,
        scaling='weak', vs_baseline=None, dtype='bf16', data='synthetic',
        config=dict(workload=WORKLOAD, B=spec['B'], T=spec['T'], Hqk=spec['Hqk'],
                    Hv=spec['Hv'], Dk=spec['Dk'], Dv=spec['Dv'], chunk=CHUNK,
                    state_qdq='e4m3', w_qdq='e4m3', block_v=spec['block_v'], parallelism='1gpu'),
        roofline=dict(bound='mfma', achieved=achieved, peak=PEAK_BF16_TFLOPS, unit='TFLOP/s',
                      frac=achieved / PEAK_BF16_TFLOPS, traffic=traffic),
        kernel_ms=kern_ms, gflop_per_step=flops / 1e9,
        hbm_gbs_algorithmic=bytes_algorithmic(spec) / (kern_ms * 1e-3) / 1e9,
        source_hash=src)
    if not args.no_cpu_baseline:
        out['cpu_baseline'] = cpu_baseline(spec, seed=2)
    print(json.dumps(out), flush=True)


if __name__ == '__main__':
    main()
