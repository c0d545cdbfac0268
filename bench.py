"""Throughput of the chunked gated delta rule forward with FP8 E4M3 state and
W fake QDQ on one MI355X, against the bf16 MFMA roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-bwd] [--no-configs] [--copy-calibration]

One step = one forward over B=4 sequences of T=4096 tokens, 16 heads,
Dk = Dv = 128, state E4M3 with [128, 64] scale tiles, W E4M3 per (chunk,
head), inputs resident in HBM: the forward's two stages, as gdn_chunk_fwd
runs them (gdn_chunk_fwd_prep: gates, gated K K^T, exact solve, W and its
QDQ, U, masked Q K^T for every chunk and head; gdn_chunk_fwd_state: the state
QDQ and sequential recurrence, and the output). Prints one JSON line.

Timing protocol: W untimed warmup steps, then exactly K steps between two
device synchronizations. Before each step a 512 MB buffer is written, so
the 256 MB last-level cache holds none of the step's inputs; HIP events on
the launch stream bracket each stage of each step (the flush is outside
them). `ms_per_step` is the median step time, with p10 and p90 beside it;
`value` = tokens / ms_per_step. The other workloads (the tiny FP32 case, the
packed varlen INT8 case, the long-context case, and forward + backward) are
timed the same way in `configs` and `fwd_bwd`.

Algorithmic FLOPs per token and head at full 64x64 tiles (C = 64):
  prep   2 (3 C Dk + C Dv) + C^2 / 3   (K K^T, Q K^T, W; U; the solve)
  state  2 (3 Dk Dv + C Dv)            (W S, Q S, K^T Vnew; P Vnew)
  total 181 589 for Dk = Dv = 128.
`roofline` is the dominant (longer) kernel's own FLOPs per launch divided by
its median duration; `roofline_path` is the same for the whole forward.
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
HBM_PEAK_GBS = 8000.0
CHUNK = 64
FLUSH_BYTES = 512 << 20


def flops_prep(Dk, Dv, C=CHUNK):
    return 2 * (3 * C * Dk + C * Dv) + C * C / 3.0


def flops_state(Dk, Dv, C=CHUNK):
    return 2 * (3 * Dk * Dv + C * Dv)


def flops_bwd(Dk, Dv, C=CHUNK):
    return 2 * (6 * C * Dk + 4 * C * Dv + 6 * Dk * Dv) + 2 * C * C / 3.0


def spec_tokens(spec):
    return sum(spec['lengths']) if 'lengths' in spec else spec['B'] * spec['T']


def bytes_algorithmic(spec):
    """Minimum HBM bytes of one forward: read q, k, v, g, beta and h0 once,
    write o and ht once (bf16 or FP32 io as the workload has it)."""
    esz = 4 if spec['dtype'] == 'f32' else 2
    tok = spec_tokens(spec)
    N = len(spec['lengths']) if 'lengths' in spec else spec['B']
    Hqk, Hv, Dk, Dv = spec['Hqk'], spec['Hv'], spec['Dk'], spec['Dv']
    rd = tok * (2 * Hqk * Dk * esz + Hv * Dv * esz + 2 * Hv * 4)
    rd += N * Hv * Dk * Dv * 4 if spec['h0'] else 0
    wr = tok * Hv * Dv * esz + N * Hv * Dk * Dv * 4
    return rd + wr


# Sources each timed kernel is compiled from; a committed counter summary is
# used only while these files are unchanged.
KERNEL_SOURCES = {
    'gdn_state_split_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h',
                               'gdn_fwd_state_split.hip'),
    'gdn_prep_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h', 'gdn_fwd_prep.hip'),
    'gdn_state_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h', 'gdn_fwd_state.hip'),
    'gdn_fwd_kernel': ('gdn_device.h', 'gdn_launch.h', 'gdn_fwd.hip'),
    'bwd_img_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h', 'gdn_bwd_state.hip'),
    'bwd_state_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h', 'gdn_bwd_state.hip'),
    'bwd_local_kernel': ('gdn_device.h', 'gdn_images.h', 'gdn_launch.h', 'gdn_bwd_local.hip'),
}
BWD_KERNELS = ('bwd_img_kernel', 'bwd_state_kernel', 'bwd_local_kernel')
FWD_KERNELS = ('gdn_state_split_kernel', 'gdn_prep_kernel', 'gdn_state_kernel', 'gdn_fwd_kernel')


def state_kernel_of(spec):
    """The kernel that runs the state stage of a forward workload."""
    if spec['dtype'] == 'f32':
        return 'gdn_fwd_kernel'
    split = spec['state_fmt'] != 0 and spec['w_fmt'] != 0 and spec['block_v'] <= 64
    return 'gdn_state_split_kernel' if split else 'gdn_state_kernel'


def source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, 'gateddeltanet_chunked_recurrence_amd', 'csrc')
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(csrc, f), 'rb').read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by what the
    counter reads for a device copy of known size) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    (else None)."""
    if kernel not in KERNEL_SOURCES:
        return None
    p = os.path.join(ROOT, 'profiles', f'{kernel}_{workload}_traffic.json')
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get('source_hash') != source_hash(kernel):
        return None
    return d.get('bytes_per_launch')


def host_threads():
    """Host CPUs this process may run on (the affinity mask: on a shared GPU
    box that is its CPU share, which os.cpu_count() does not show)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(spec, seed, min_seconds=10.0):
    """The float64 oracle, untuned, on the same workload: whole passes over
    all B sequences at full length and all heads, repeated until at least
    `min_seconds` of CPU work, with torch's CPU threads (its BLAS included)
    set to the host CPUs this process may use."""
    import torch

    import gdn_inputs
    from oracle import chunked_fwd
    threads = host_threads()
    torch.set_num_threads(threads)
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
    ntok = reps * spec_tokens(spec)
    return dict(value=ntok / dt, unit='tokens/s', cores=torch.get_num_threads(), kind='oracle',
                host_cpu_count=os.cpu_count(),
                sample=f'{reps} passes over the whole workload ({spec["B"]} x {spec["T"]} tokens, '
                       f'{spec["Hv"]} heads; float64 chunked oracle, {dt:.1f} s)')


def _stats(xs):
    xs = sorted(xs)
    q = lambda f: xs[min(len(xs) - 1, max(0, int(round(f * (len(xs) - 1)))))]
    return dict(median=q(0.5), p10=q(0.1), p90=q(0.9))


def time_fwd(spec, seed, steps, warmup, flush):
    """Per-step times (ms) of the forward on one workload, flushing the
    last-level cache before each step (outside the timed events): `total`
    times gdn_chunk_fwd (the overlapped schedule where it applies); `prep`
    and `state` time the two stages run one after the other, for the
    per-kernel rooflines, and `serial` their sum."""
    import torch

    import gdn_inputs
    from gateddeltanet_chunked_recurrence_amd import binding as B
    x = gdn_inputs.make_inputs(spec, seed, device='cuda')
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
    plan = B.FwdPlan(x['q'], x['k'], x['v'], x['g'], x['beta'], scale=1.0 / math.sqrt(spec['Dk']),
                     h0=x['h0'], cu_seqlens=x['cu_seqlens'], **kw)
    for _ in range(warmup):
        plan.forward()
        plan.prep()
        plan.state()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        plan.forward()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        flush.fill_((i + 1) & 0xFF)
        ev[i][2].record(stream)
        plan.prep()
        ev[i][3].record(stream)
        plan.state()
        ev[i][4].record(stream)
    torch.cuda.synchronize()
    total = [e[0].elapsed_time(e[1]) for e in ev]
    prep = [e[2].elapsed_time(e[3]) for e in ev]
    state = [e[3].elapsed_time(e[4]) for e in ev]
    serial = [e[2].elapsed_time(e[4]) for e in ev]
    return dict(total=_stats(total), prep=_stats(prep), state=_stats(state), serial=_stats(serial),
                wall_s=wall)


def fwd_record(name, spec, t, state_kernel):
    """Bench figures of one forward workload from its stage timings."""
    tokens = spec_tokens(spec)
    th = tokens * spec['Hv']
    Dk, Dv = spec['Dk'], spec['Dv']
    f_prep, f_state = flops_prep(Dk, Dv) * th, flops_state(Dk, Dv) * th
    p_ms, s_ms, tot = t['prep']['median'], t['state']['median'], t['total']['median']
    if state_kernel == 'gdn_fwd_kernel':            # FP32 inputs: one fused kernel does all of it
        dom, dom_ms, dom_f = state_kernel, s_ms, f_prep + f_state
    elif s_ms >= p_ms:
        dom, dom_ms, dom_f = state_kernel, s_ms, f_state
    else:
        dom, dom_ms, dom_f = 'gdn_prep_kernel', p_ms, f_prep
    ach = dom_f / (dom_ms * 1e-3) / 1e12
    path = (f_prep + f_state) / (tot * 1e-3) / 1e12
    traffic = measured_traffic(dom, name)
    return dict(
        workload=name, tokens=tokens, ms=t['total'], tokens_per_s=tokens / (tot * 1e-3),
        kernel_ms=dict(prep=t['prep'], state=t['state']), serial_ms=t['serial'],
        roofline=dict(bound='mfma', achieved=ach, peak=PEAK_BF16_TFLOPS, unit='TFLOP/s',
                      frac=ach / PEAK_BF16_TFLOPS, traffic=traffic, kernel=dom),
        roofline_path=dict(bound='mfma', achieved=path, peak=PEAK_BF16_TFLOPS, unit='TFLOP/s',
                           frac=path / PEAK_BF16_TFLOPS),
        hbm_gbs_algorithmic=bytes_algorithmic(spec) / (tot * 1e-3) / 1e9,
        gflop=(f_prep + f_state) / 1e9)


def time_fwd_bwd(steps, warmup, flush, solve_degree=0):
    """Forward (saving for the backward) + backward on the forward+backward
    workload (B=2, T=8192, H=16, Dk=Dv=128, E4M3 state and W, initial state,
    dO and dS_final given), per-step medians."""
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
                               h0=x['h0'], save_for_backward=True, solve_degree=solve_degree,
                               **kw)

    def bwd(saved):
        return B.gdn_chunk_bwd(x['q'], x['k'], x['v'], x['g'], x['beta'], saved, x['do'],
                               x['dht'], scale=scale, h0=x['h0'])

    for _ in range(warmup):
        bwd(fwd()[2])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        saved = fwd()[2]
        ev[i][1].record(stream)
        bwd(saved)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    f = _stats([e[0].elapsed_time(e[1]) for e in ev])
    b = _stats([e[1].elapsed_time(e[2]) for e in ev])
    tokens = spec['B'] * spec['T']
    th = tokens * spec['Hv']
    fl = (flops_prep(128, 128) + flops_state(128, 128) + flops_bwd(128, 128)) * th
    tot = f['median'] + b['median']
    ach = fl / (tot * 1e-3) / 1e12
    return dict(workload=name, solve_degree=solve_degree, fwd_ms=f, bwd_ms=b,
                tokens_per_s=tokens / (tot * 1e-3),
                steps=steps, bwd_bytes_counted={k: measured_traffic(k, name) for k in BWD_KERNELS},
                roofline_path=dict(bound='mfma', achieved=ach, peak=PEAK_BF16_TFLOPS,
                                   unit='TFLOP/s', frac=ach / PEAK_BF16_TFLOPS))


def time_decode(steps, warmup, flush):
    """Decode continuation on the 257-token workload: the 64-token chunk
    prefill plus 193 token-state writes (E4M3, readout after the write),
    forward (saving for the backward) and backward, per-step medians."""
    import torch

    import gdn_inputs
    from gateddeltanet_chunked_recurrence_amd import binding as B
    name = 'decode_e4m3_b4_t257_p64_h16_d128'
    spec = gdn_inputs.spec(name)
    x = gdn_inputs.make_inputs(spec, seed=2, device='cuda')
    P, scale = spec['prefix_len'], 1.0 / math.sqrt(spec['Dk'])
    kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'],
              readout=B.READOUT_AFTER_WRITE)
    args = [x[n] for n in ('q', 'k', 'v', 'g', 'beta')]

    def fwd():
        return B.gdn_prefill_decode_fwd(*args, P, scale, x['h0'], save_for_backward=True, **kw)

    def bwd(saved):
        return B.gdn_prefill_decode_bwd(*args, saved, x['do'], x['dht'], scale, x['h0'])

    for _ in range(warmup):
        bwd(fwd()[2])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        flush.fill_(i & 0xFF)
        ev[i][0].record(stream)
        saved = fwd()[2]
        ev[i][1].record(stream)
        bwd(saved)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    f = _stats([e[0].elapsed_time(e[1]) for e in ev])
    b = _stats([e[1].elapsed_time(e[2]) for e in ev])
    tokens = spec['B'] * spec['T']
    return dict(workload=name, fwd_ms=f, bwd_ms=b, decode_tokens_per_seq=spec['T'] - P,
                tokens_per_s=tokens / ((f['median'] + b['median']) * 1e-3), steps=steps)


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
    ap.add_argument('--no-configs', action='store_true', help='skip the other forward workloads')
    ap.add_argument('--workload', default=WORKLOAD, help='forward workload of the headline line')
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

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device='cuda')
    spec = gdn_inputs.spec(args.workload)
    t = time_fwd(spec, 2, args.steps, args.warmup, flush)
    head = fwd_record(args.workload, spec, t, state_kernel_of(spec))
    ms = t['total']['median']
    tokens = spec_tokens(spec)
    out = dict(
        metric=METRIC, value=tokens / (ms * 1e-3), unit='tokens/s', n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=ms,
        ms_per_step_p10=t['total']['p10'], ms_per_step_p90=t['total']['p90'],
        higher_is_better=True, scaling='weak', vs_baseline=None, dtype='bf16', data='synthetic',
        config=dict(workload=args.workload, B=spec['B'],
                    **({'lengths': spec['lengths']} if 'lengths' in spec else {'T': spec['T']}),
                    Hqk=spec['Hqk'], Hv=spec['Hv'], Dk=spec['Dk'], Dv=spec['Dv'], chunk=CHUNK,
                    state_qdq=['off', 'e4m3', 'int8'][spec['state_fmt']],
                    w_qdq=['off', 'e4m3', 'int8'][spec['w_fmt']], block_v=spec['block_v'],
                    parallelism='1gpu'),
        roofline=head['roofline'], roofline_path=head['roofline_path'],
        kernel_ms=head['kernel_ms'], ms_serial_stages=head['serial_ms'], gflop_per_step=head['gflop'],
        hbm_gbs_algorithmic=head['hbm_gbs_algorithmic'],
        whole_forward_traffic=dict(
            bytes_algorithmic=bytes_algorithmic(spec),
            bytes_counted={k: measured_traffic(k, args.workload) for k in FWD_KERNELS
                           if k in ('gdn_prep_kernel', state_kernel_of(spec))}),
        protocol=dict(flush_bytes_between_steps=FLUSH_BYTES, stat='median over steps',
                      timed_wall_s=t['wall_s']),
        source_hash={k: source_hash(k) for k in KERNEL_SOURCES})
    if not args.no_configs:
        cfgs = {}
        for name, steps in (('tiny_fp32', 20), ('varlen_int8_gqa4x16_d128', 20),
                            ('long_e4m3_t65536_h32_dk128_dv256', 5)):
            s = gdn_inputs.spec(name)
            cfgs[name] = fwd_record(name, s, time_fwd(s, 2, steps, 2, flush), state_kernel_of(s))
            torch.cuda.empty_cache()
        out['configs'] = cfgs
    if not args.no_bwd:
        out['fwd_bwd'] = time_fwd_bwd(steps=max(3, args.steps // 5), warmup=2, flush=flush)
        x = gdn_inputs.make_inputs(spec, 2, device='cuda')
        kw = dict(state_fmt=spec['state_fmt'], w_fmt=spec['w_fmt'], block_v=spec['block_v'])
        out['neumann_solve'] = time_neumann_prep(x, spec, 1.0 / math.sqrt(spec['Dk']), kw,
                                                 steps=max(3, args.steps // 5))
        out['fwd_bwd_neumann_d3'] = time_fwd_bwd(steps=max(3, args.steps // 5), warmup=2,
                                                 flush=flush, solve_degree=3)
        out['decode'] = time_decode(steps=max(3, args.steps // 5), warmup=2, flush=flush)
    if not args.no_cpu_baseline:
        out['cpu_baseline'] = cpu_baseline(spec, seed=2)
    print(json.dumps(out), flush=True)


if __name__ == '__main__':
    main()
