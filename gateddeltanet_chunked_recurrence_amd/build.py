"""Builds libgdn_hip.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m gateddeltanet_chunked_recurrence_amd.build   [-j N] [--debug]

Every source is compiled by hipcc for --offload-arch=gfx950 with packed FP32
instructions disabled, then linked into one shared library next to this file.
"""
import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, 'csrc')
INCLUDE = os.path.join(os.path.dirname(HERE), 'include')
LIB = os.path.join(HERE, 'libgdn_hip.so')
BUILD_DIR = os.path.join(os.path.dirname(HERE), '_build')
SOURCES = ['gdn_abi.cpp', 'gdn_qdq.hip', 'gdn_guard.hip', 'gdn_fwd.hip', 'gdn_fwd_prep.hip',
           'gdn_fwd_state.hip', 'gdn_fwd_state_split.hip', 'gdn_bwd.hip',
           'gdn_bwd_state.hip', 'gdn_bwd_local.hip', 'gdn_decode.hip']
HIPCC = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')

COMMON = ['-std=c++17', '-O3', '-fPIC', '--offload-arch=gfx950',
          '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
          '-I', CSRC, '-I', INCLUDE, '-Wall', '-Wno-unused-function']


def _compile(src, debug):
    out = os.path.join(BUILD_DIR, src + '.o')
    lang = ['-x', 'hip'] if src.endswith('.hip') else ['-x', 'hip']
    cmd = [HIPCC] + COMMON + lang + (['-g'] if debug else []) + \
        ['-c', os.path.join(CSRC, src), '-o', out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if 'packed-fp32-ops' not in ln]
    return src, r.returncode, '\n'.join(msgs), out


def build(jobs=4, debug=False, verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    objs = []
    for src, rc, msg, out in results:
        if msg.strip() and (rc != 0 or verbose):
            print(f'--- {src}\n{msg}', file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f'hipcc failed on {src}')
        objs.append(out)
    tmp = LIB + '.tmp'
    # --no-undefined: a kernel whose host stub was not emitted fails the build,
    # not the first dlopen
    cmd = [HIPCC, '-shared', '-fPIC', '--offload-arch=gfx950', '-Wl,--no-undefined', '-o', tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError('link failed:\n' + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == '__main__':
    ap = argparse.ArgumentParser()
    ap.add_argument('-j', type=int, default=4)
    ap.add_argument('--debug', action='store_true')
    ap.add_argument('-v', action='store_true')
    args = ap.parse_args()
    print(build(args.j, args.debug, args.v))
