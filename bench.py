"""Throughput of the chunked gated delta rule forward with FP8 E4M3 state and
W fake QDQ on one MI355X, against the bf16 MFMA roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-bwd] [--copy-calibration]

One step = one forward over B=4 sequences of T=4096 tokens, 16 heads,
Dk = Dv = 128, state E4M3 with [128, 64] scale tiles, W E4M3 per (chunk,
head), inputs resident in HBM: the forward's two stages, as gdn_chunk_fwd
runs them (gdn_chunk_fwd_prep: gates, gated K K^T, exact solve, W and its
QDQ, U, masked Q K^T for every chunk and head; gdn_chunk_fwd_state: the state
QDQ and sequential recurrence, and the output). Prints one JSON line.

Algorithmic FLOPs per token and head at full 64x64 tiles (C = 64):
  prep   2 (3 C Dk + C Dv) + C^2 / 3   (K K^T, Q K^T, W; U; the solve)
  state  2 (3 Dk Dv + C Dv)            (W S, Q S, K^T Vnew; P Vnew)
  total 181 589 for Dk = Dv = 128.
`roofline` is the dominant (longer) kernel's own FLOPs per launch divided by
its average duration, timed with HIP events on the launch stream around each
stage of every timed step; `roofline_path` is the same for the whole forward.
Peak: dense bf16 MFMA, 2.5 PFLOP/s.
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


def flops_prep(Dk, Dv, C=CHUNK):
    return 2 * (3 * C * Dk + C * Dv) + C * C / 3.0


def flops_state(Dk, Dv, C=CHUNK):
    return 2 * (3 * Dk * Dv + C * Dv)


def flops_per_token_head(Dk, Dv, C=CHUNK):
    return flops_prep(Dk, Dv, C) + flops_state(Dk, Dv, C)


def bytes_algorithmic(spec):
    """Minimum HBM bytes of one forward: read q, k, v (bf16), g, beta (FP32),
    h0 if any; write o (bf16) and ht (FP32)."""
    B, T, Hqk, Hv, Dk, Dv = (spec[k] for k in ('B', 'T', 'Hqk', 'Hv', 'Dk', 'Dv'))
    tok = B * T
    rd = tok * (2 * Hqk * Dk * 2 + Hv * Dv * 2 + 2 * Hv * 4)
    wr = tok * Hv * Dv * 2 + B * Hv * Dk * Dv * 4
    return rd + wr


# Sources each timed kernel is compiled from; a committed counter summary is
# used only while these files are unchanged.
KERNEL_SOURCES = {
    'gdn_state_split_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h',
                               'gdn_fwd_state_split.hip'),
    'gdn_prep_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h', 'gdn_fwd_prep.hip'),
}


def source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, 'gateddeltanet_chunked_recurrence_amd', 'csrc')
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(csrc, f), 'rb').read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, src_hash):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    counter reads for a device copy of known size) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    (else None)."""
    p = os.path.join(ROOT, 'profiles', f'{kernel}_{WORKLOAD}_traffic.json')
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get('source_hash') != src_hash:
        return None
    return d.get('bytes_per_launch')


def cpu_baseline(spec, seed, min_seconds=10.0):
    """The float64 oracle on the same workload (all B sequences, full length,
    all heads), repeated until at least `min_seconds` of CPU work."""
    import torch

    import gdn_inputs
    from oracle import chunked_fwd
    x = gdn_inputs.make_inputs(spec, seed, device='cpu')
    args = [x[n].double() for n in ('q', 'k', 'v', 'g', 'beta')]
    reps, t = 0, time.perf_counter()
    while True:
        chunked_fwd(*args, 1.0 / math.sqrt(spec['Dk']), None, None, state_fmt=spec['state_fmt'],
                    w_fmt=spec['w_fmt'], block_v=spec['block_v'])
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    ntok = reps * spec['B'] * spec['T']
    return dict(value=ntok / dt, unit='tokens/s', cores=torch.get_num_threads(), kind='oracle',
                sample=f'{reps} passes over the whole workload ({spec["B"]} x {spec["T"]} tokens, '
                       f'{spec["Hv"]} heads; float64 chunked oracle, {dt:.1f} s)')


def time_fwd_bwd(steps, warmup):
    """Forward (saving for the backward) + backward on the forward+backward
    workload (B=2, T=8192, H=16, Dk=Dv=128, E4M3 state and W, initial state,
    dO and dS_final given). Returns per-step milliseconds of each part."""
    import torch

    import gdn_inputs
    from gateddeltanet_chunked_recurrence_amd import binding as B
    name = 'fwd_bwd_e4m3_b2_t8192_h16_d128'
    spec = gdn_inputs.spec(name)
    x = gdn_inputs.make_inputs(spec, seed=2, device='cuda', bwd=True)
    scale = 1.0 / math.sqrt(spec['Dk'])
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])

    def fwd():
        return B.gdn_chunk_fwd(x['q'], x['k'], x['v'], x['g'], x['beta'], scale=scale,
                               h0=x['h0'], save_for_backward=True, **kw)

    def bwd(saved):
        return B.gdn_chunk_bwd(x['q'], x['k'], x['v'], x['g'], x['beta'], saved, x['do'],
                               x['dht'], scale=scale, h0=x['h0'], **kw)

    for _ in range(warmup):
        bwd(fwd()[2])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    for i in range(steps):
        ev[3 * i].record(stream)
        saved = fwd()[2]
        ev[3 * i + 1].record(stream)
        bwd(saved)
        ev[3 * i + 2].record(stream)
    torch.cuda.synchronize()
    f = sum(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps)) / steps
    b = sum(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps)) / steps
    tokens = spec['B'] * spec['T']
    return dict(workload=name, fwd_ms=f, bwd_ms=b, tokens_per_s=tokens / ((f + b) * 1e-3),
                steps=steps)


def time_neumann_prep(x, spec, scale, kw, steps, degrees=(3, 31)):
    """Prep-stage milliseconds on the same workload with the opt-in Neumann
    solve of each degree in place of the exact solve (the state stage does
    not change)."""
    import torch

    from gateddeltanet_chunked_recurrence_amd import binding as B
    out = {}
    stream = torch.cuda.current_stream()
    for d in degrees:
        plan = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], scale=scale, solve_degree=d,
                         **kw)
        plan.prep()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            plan.prep()
        e1.record(stream)
        torch.cuda.synchronize()
        out[str(d)] = e0.elapsed_time(e1) / steps
    return dict(prep_ms_by_degree=out, steps=steps)


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters (each copy reads and writes `nbytes`)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device='cuda').fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes=nbytes, reps=reps)), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument('--gpus', type=int, default=1)
    ap.add_argument('--steps', type=int, default=50)
    ap.add_argument('--warmup', type=int, default=10)
    ap.add_argument('--no-cpu-baseline', action='store_true')
    ap.add_argument('--no-bwd', action='store_true', help='skip the forward+backward and Neumann-solve timings')
    ap.add_argument('--copy-calibration', action='store_true',
                    help='only run a 1 GiB device copy (counter calibration)')
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get('WORLD_SIZE', '1')) != 1:
        print("bench.py measures one GPU and has no multi-GPU path: sequences and heads "
              "are independent, so a multi-GPU run would shard them with no communication",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import gdn_inputs
    from gateddeltanet_chunked_recurrence_amd import binding as B

    spec = gdn_inputs.spec(WORKLOAD)
    x = gdn_inputs.make_inputs(spec, seed=2, device='cuda')
    scale = 1.0 / math.sqrt(spec['Dk'])
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])

    plan = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], scale=scale, **kw)

    for _ in range(args.warmup):
        plan.prep()
        plan.state()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        plan.prep()
        ev[2 * i + 1].record(stream)
        plan.state()
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prep_ms = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)) / args.steps
    state_ms = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(args.steps)) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    tokens = spec['B'] * spec['T']
    th = tokens * spec['Hv']
    Dk, Dv = spec['Dk'], spec['Dv']
    f_prep, f_state = flops_prep(Dk, Dv) * th, flops_state(Dk, Dv) * th
    dom = 'gdn_state_split_kernel' if state_ms >= prep_ms else 'gdn_prep_kernel'
    dom_ms, dom_flops = (state_ms, f_state) if state_ms >= prep_ms else (prep_ms, f_prep)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    path_ms = prep_ms + state_ms
    path = (f_prep + f_state) / (path_ms * 1e-3) / 1e12
    src = source_hash(dom)
    traffic = measured_traffic(dom, src)
    out = dict(
        metric=METRIC, value=tokens / (ms_per_step * 1e-3), unit='tokens/s', n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True,
        scaling='weak', vs_baseline=None, dtype='bf16', data='synthetic',
        config=dict(workload=WORKLOAD, B=spec['B'], T=spec['T'], Hqk=spec['Hqk'],
                    Hv=spec['Hv'], Dk=Dk, Dv=Dv, chunk=CHUNK,
                    state_qdq='e4m3', w_qdq='e4m3', block_v=spec['block_v'], parallelism='1gpu'),
        roofline=dict(bound='mfma', achieved=achieved, peak=PEAK_BF16_TFLOPS, unit='TFLOP/s',
                      frac=achieved / PEAK_BF16_TFLOPS, traffic=traffic, kernel=dom),
        roofline_path=dict(bound='mfma', achieved=path, peak=PEAK_BF16_TFLOPS, unit='TFLOP/s',
                           frac=path / PEAK_BF16_TFLOPS),
        kernel_ms=dict(gdn_prep_kernel=prep_ms, gdn_state_split_kernel=state_ms),
        gflop_per_step=(f_prep + f_state) / 1e9,
        hbm_gbs_algorithmic=bytes_algorithmic(spec) / (path_ms * 1e-3) / 1e9,
        source_hash=src)
    if not args.no_bwd:
        out['fwd_bwd'] = time_fwd_bwd(steps=max(3, args.steps // 5), warmup=2)
        out['neumann_solve'] = time_neumann_prep(x, spec, scale, kw, steps=max(3, args.steps // 5))
    if not args.no_cpu_baseline:
        out['cpu_baseline'] = cpu_baseline(spec, seed=2)
    print(json.dumps(out), flush=True)


if __name__ == '__main__':
    main()
