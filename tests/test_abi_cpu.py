"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/gdn.h declares, and rejects bad arguments before any launch with the
documented status codes ("explicit early rejection" and "rejected before
launch": "[1/4] GDN state/W QAT foundation", "What does this PR do?" and
"Testing"). No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

from gateddeltanet_chunked_recurrence_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, 'include', 'gdn.h')).read()
    src = re.sub(r'/\*.*?\*/', '', src, flags=re.S)
    return sorted(set(re.findall(r'^\s*(?:const\s+)?\w+\**\s+\**(gdn_\w+)\s*\(', src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert {'gdn_chunk_fwd', 'gdn_chunk_bwd', 'gdn_qdq_state', 'gdn_decode_fwd',
            'gdn_decode_bwd', 'gdn_decode_saved_bytes', 'gdn_decode_bwd_workspace_bytes'} <= set(names)
    lib = B.load_library()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.gdn_abi_version() == 8


def _args(**kw):
    fake = ctypes.c_void_p(0x10000)          # aligned, never dereferenced on these paths
    a = B.FwdArgs(B=1, T=128, Hqk=2, Hv=4, Dk=128, Dv=128, num_seqs=1, io_dtype=B.GDN_BF16,
                  scale=0.1, policy=B.QdqPolicy(B.QDQ_E4M3, B.QDQ_E4M3, 64, 64))
    for name in ('q', 'k', 'v', 'g', 'beta', 'o'):
        setattr(a, name, fake)
    for k, v in kw.items():
        if k in ('state_fmt', 'w_fmt', 'block_v', 'chunk_size', 'solve_degree', 'read_fmt'):
            setattr(a.policy, k, v)
        else:
            setattr(a, k, v)
    return a


BAD = [
    (dict(chunk_size=32), B.GDN_E_UNSUPPORTED, 'chunk_size'),
    (dict(state_fmt=3), B.GDN_E_UNSUPPORTED, 'format'),
    (dict(w_fmt=-1), B.GDN_E_UNSUPPORTED, 'format'),
    (dict(block_v=48), B.GDN_E_UNSUPPORTED, 'block_v'),
    (dict(Dv=64, block_v=128), B.GDN_E_INVALID, 'does not divide'),
    (dict(block_v=512), B.GDN_E_UNSUPPORTED, 'block_v'),
    (dict(io_dtype=1, Dk=64, block_v=128), B.GDN_E_UNSUPPORTED, 'block_v up to 64'),
    (dict(Hv=6, Hqk=4), B.GDN_E_INVALID, 'multiple'),
    (dict(Dk=96), B.GDN_E_UNSUPPORTED, 'Dk'),
    (dict(Dv=512), B.GDN_E_UNSUPPORTED, 'Dv'),
    (dict(io_dtype=1), B.GDN_E_UNSUPPORTED, 'FP32'),
    (dict(io_dtype=7), B.GDN_E_INVALID, 'io_dtype'),
    (dict(num_seqs=2), B.GDN_E_INVALID, 'num_seqs'),
    (dict(B=2, cu_seqlens=ctypes.c_void_p(0x20000)), B.GDN_E_INVALID, 'cu_seqlens'),
    (dict(scale=float('nan')), B.GDN_E_INVALID, 'scale'),
    (dict(q=None), B.GDN_E_INVALID, 'q is NULL'),
    (dict(o=None), B.GDN_E_INVALID, 'o is NULL'),
    (dict(k=ctypes.c_void_p(0x10004)), B.GDN_E_INVALID, 'aligned'),
    (dict(T=-1), B.GDN_E_INVALID, 'bad sizes'),
    # the Neumann degree is 2^j - 1 (j = 1..6), never rounded to a supported one
    (dict(solve_degree=2), B.GDN_E_UNSUPPORTED, 'solve_degree'),
    (dict(solve_degree=5), B.GDN_E_UNSUPPORTED, 'solve_degree'),
    (dict(solve_degree=127), B.GDN_E_UNSUPPORTED, 'solve_degree'),
    (dict(solve_degree=-1), B.GDN_E_UNSUPPORTED, 'solve_degree'),
    (dict(solve_degree=3, io_dtype=1, Dk=64), B.GDN_E_UNSUPPORTED, 'Neumann'),
    # the two-precision read copy: E4M3 or off, never with a quantized carry,
    # built for Dk = 128 and bf16 inputs
    (dict(read_fmt=2, state_fmt=0), B.GDN_E_UNSUPPORTED, 'read_fmt'),
    (dict(read_fmt=5, state_fmt=0), B.GDN_E_UNSUPPORTED, 'read_fmt'),
    (dict(read_fmt=1), B.GDN_E_INVALID, 'replaces the state'),
    (dict(read_fmt=1, state_fmt=0, Dk=64), B.GDN_E_UNSUPPORTED, 'Dk = 128'),
    (dict(prefix_len=-1), B.GDN_E_INVALID, 'prefix_len'),
]


@pytest.mark.parametrize("kw,status,msg", BAD)
def test_forward_rejects_before_launch(kw, status, msg):
    lib = B.load_library()
    a = _args(**kw)
    got = lib.gdn_chunk_fwd(ctypes.byref(a), None)
    assert got == status
    assert msg in lib.gdn_last_error().decode()


def test_forward_schedule_host_logic():
    """gdn_fwd_schedule: where gdn_chunk_fwd overlaps the operand build with
    the state recurrence, and how it splits the (chunk, head) items. The head
    is items - R * chunks / r in whole rounds of CUs, R = CUs - the state
    workgroups (N Hv Dv / 64, or Dv / block_v per head for 128- and 256-wide
    tiles), r = 3.7 for the split state kernel (both QDQ sites on, tiles up
    to 64 wide; 3.0 where two prep workgroups share a CU: Dv <= 128 with the
    exact solve) and 1.75 for the general one; numbers worked by hand here."""
    big = dict(B=4, T=4096, Hqk=16, Hv=16, num_seqs=4)
    sch = B.fwd_schedule(_args(**big), 256)
    # 64 chunks x 64 (sequence, head) pairs; 128 state workgroups leave R = 128;
    # 4096 - 128 * 64 / 3.0 = 1365.3 -> 5 rounds of 256
    assert sch == dict(overlapped=True, items=4096, head_items=1280, rest_blocks=128)
    # 304 CUs: R = 176; 4096 - 176 * 64 / 3.0 = 341.3 -> 1 round of 304
    assert B.fwd_schedule(_args(**big), 304) == dict(overlapped=True, items=4096, head_items=304,
                                                      rest_blocks=176)
    # a long sequence: the remainder alone outlasts the chain, so no head
    sch = B.fwd_schedule(_args(B=1, T=65536, Hqk=32, Hv=32, Dv=256, num_seqs=1), 256)
    assert sch == dict(overlapped=True, items=32768, head_items=0, rest_blocks=128)
    # the general state kernel: its chain alone outlasts the remainder
    for kw in (dict(big, state_fmt=B.QDQ_OFF), dict(big, w_fmt=B.QDQ_OFF),
               dict(big, state_fmt=B.QDQ_OFF, w_fmt=B.QDQ_OFF)):
        assert B.fwd_schedule(_args(**kw), 256) == dict(overlapped=True, items=4096, head_items=0,
                                                         rest_blocks=128), kw
    # 128-wide tiles: one workgroup per head and tile, 64 in all, R = 192
    assert B.fwd_schedule(_args(**dict(big, block_v=128)), 256) == dict(
        overlapped=True, items=4096, head_items=0, rest_blocks=192)
    # QDQ off with Dv 64 and 128 heads: 8192 items, R = 128;
    # 8192 - 128 * 64 / 1.75 = 3510.9 -> 14 rounds of 256
    many = dict(B=8, T=4096, Hqk=16, Hv=16, Dv=64, num_seqs=8, state_fmt=B.QDQ_OFF,
                w_fmt=B.QDQ_OFF)
    assert B.fwd_schedule(_args(**many), 256) == dict(overlapped=True, items=8192, head_items=3584,
                                                       rest_blocks=128)
    serial = [
        dict(big, state_fmt=B.QDQ_OFF, read_fmt=B.QDQ_E4M3),   # two-precision profile
        dict(big, io_dtype=B.GDN_F32, Dk=64, Dv=64),
        dict(big, T=192),                                   # 3 chunks
        dict(big, prefix_len=128),                          # 2 chunks
        dict(B=2, T=4096, Hqk=32, Hv=32, Dv=256, num_seqs=2),   # 256 state workgroups
        # packed sequences beyond the setup kernel's limits
        dict(B=1, T=4096, Hqk=16, Hv=16, num_seqs=1025, cu_seqlens=ctypes.c_void_p(0x20000)),
        dict(B=1, T=4095 * 64 + 1, Hqk=1, Hv=1, num_seqs=2, cu_seqlens=ctypes.c_void_p(0x20000)),
    ]
    for kw in serial:
        sch = B.fwd_schedule(_args(**kw), 256)
        assert sch['overlapped'] is False, kw
    # packed sequences: the device derives the items and the head from the lengths
    packed = dict(B=1, T=4096, Hqk=16, Hv=16, num_seqs=2, cu_seqlens=ctypes.c_void_p(0x20000))
    assert B.fwd_schedule(_args(**packed), 256) == dict(overlapped=True, items=-1, head_items=-1,
                                                         rest_blocks=192)
    with pytest.raises(B.GdnError):
        B.fwd_schedule(_args(**big), -1)
    with pytest.raises(B.GdnError):
        B.fwd_schedule(_args(Hv=3), 256)


def test_no_overlap_switch_makes_the_schedule_serial():
    """GDN_NO_OVERLAP (read once per process) turns the overlapped schedules
    off: checked in a child process that loads the library with it set."""
    import subprocess
    import sys
    code = ("import ctypes, sys; sys.path.insert(0, %r); "
            "from tests.test_abi_cpu import _args; "
            "from gateddeltanet_chunked_recurrence_amd import binding as B; "
            "print(B.fwd_schedule(_args(B=4, T=4096, Hqk=16, Hv=16, num_seqs=4), 256)['overlapped'])"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    for env, want in ((dict(GDN_NO_OVERLAP='1'), 'False'), (dict(), 'True')):
        e = {k: v for k, v in os.environ.items() if k != 'GDN_NO_OVERLAP'}
        e.update(env)
        out = subprocess.run([sys.executable, '-c', code], env=e, capture_output=True, text=True,
                             timeout=120)
        assert out.returncode == 0, out.stderr
        assert out.stdout.strip().splitlines()[-1] == want


def test_forward_workspace_is_sized_and_required():
    """bf16 inputs need the prep kernel's scratch: its size follows the
    per-(slot, head) image sizes, a missing or short workspace is rejected
    with GDN_E_WORKSPACE, and FP32 inputs (fused path) need none."""
    lib = B.load_library()
    a = _args()
    n = lib.gdn_fwd_workspace_bytes(ctypes.byref(a))
    slots = 1 + 2                                       # N + ceil(128 / 64)
    # W codes, K^T, P hi/lo (bf16, K^T and P rows unpadded), gate block (1 KB), U (FP32), W
    # scale, the ready flag of the overlapped schedule; once per call the two item counters
    # and the CU admission table (8 x 264 words)
    per = 64 * 128 * 2 + 128 * 64 * 2 + 2 * 64 * 64 * 2 + 1024 + 128 * 64 * 4 + 4 + 4
    fixed = 8 + 8 * 264 * 4
    assert n >= slots * 4 * per + fixed and n <= slots * 4 * per + fixed + 5 * 256
    assert lib.gdn_chunk_fwd(ctypes.byref(a), None) == B.GDN_E_WORKSPACE
    assert 'workspace' in lib.gdn_last_error().decode()
    a.workspace = ctypes.c_void_p(0x40000)
    a.workspace_bytes = n - 1
    assert lib.gdn_chunk_fwd(ctypes.byref(a), None) == B.GDN_E_WORKSPACE
    off = _args(w_fmt=B.QDQ_OFF)                        # W as hi + lo planes
    assert lib.gdn_fwd_workspace_bytes(ctypes.byref(off)) >= n + slots * 4 * 64 * 128 * 2
    f32 = _args(io_dtype=B.GDN_F32, Dk=64)
    assert lib.gdn_fwd_workspace_bytes(ctypes.byref(f32)) == 0
    assert lib.gdn_fwd_workspace_bytes(ctypes.byref(_args(Dk=96))) == 0


def test_empty_problem_is_a_no_op():
    lib = B.load_library()
    a = _args(T=0, q=None, k=None, v=None, g=None, beta=None, o=None)
    assert lib.gdn_chunk_fwd(ctypes.byref(a), None) == B.GDN_OK


def test_saved_layout_sizes():
    lib = B.load_library()
    a = _args(B=2, T=100, num_seqs=2)
    lay = B.saved_layout(a)
    assert lay.num_slots == 2 + 4                            # N + ceil(200 / 64)
    assert lay.off_state == 0
    assert lay.off_state_scale >= lay.num_slots * 4 * 128 * 128
    assert lay.off_w >= lay.off_state_scale + lay.num_slots * 4 * 2 * 4
    assert lay.off_w_scale >= lay.off_w + 200 * 4 * 128
    assert lay.off_x >= lay.off_w_scale + lay.num_slots * 4 * 4
    assert lay.off_meta >= lay.off_x + lay.num_slots * 4 * 64 * 64 * 4   # X, bf16 inputs
    assert lay.total_bytes == lay.off_meta + 256                        # the policy stamp
    assert lay.total_bytes == lib.gdn_saved_bytes(ctypes.byref(a))
    a.policy.state_fmt = B.QDQ_OFF
    a.policy.w_fmt = B.QDQ_OFF
    lay = B.saved_layout(a)
    assert lay.off_state_scale >= lay.num_slots * 4 * 128 * 128 * 4
    assert lay.off_w == lay.off_state_scale and lay.off_w_scale == lay.off_w
    f32 = _args(B=2, T=100, num_seqs=2, io_dtype=B.GDN_F32, Dk=64, Dv=64)
    lay = B.saved_layout(f32)
    assert lay.off_meta == lay.off_x                         # no X for FP32 inputs


def test_backward_rejects_before_launch():
    lib = B.load_library()
    fake = ctypes.c_void_p(0x10000)
    a = B.BwdArgs(fwd=_args(saved=fake), do_=fake, dq=fake, dk=fake, dv=fake, dg=fake,
                  dbeta=fake, grad_dtype=B.GDN_BF16)
    assert lib.gdn_chunk_bwd(ctypes.byref(a), None) == B.GDN_E_WORKSPACE
    assert 'workspace' in lib.gdn_last_error().decode()
    a.workspace = fake
    a.workspace_bytes = lib.gdn_bwd_workspace_bytes(ctypes.byref(a)) - 1
    assert lib.gdn_chunk_bwd(ctypes.byref(a), None) == B.GDN_E_WORKSPACE
    a.do_ = None
    assert lib.gdn_chunk_bwd(ctypes.byref(a), None) == B.GDN_E_INVALID
    a.do_ = fake
    a.fwd.saved = None
    assert lib.gdn_chunk_bwd(ctypes.byref(a), None) == B.GDN_E_INVALID
    a.fwd.saved = fake
    a.grad_dtype = 5
    assert lib.gdn_chunk_bwd(ctypes.byref(a), None) == B.GDN_E_INVALID


def test_backward_of_the_neumann_solve_is_accepted():
    """The backward differentiates the approximate inverse's polynomial: a
    valid degree passes the backward's policy checks (it stops at the missing
    workspace here) and its workspace includes the dL/dX section."""
    lib = B.load_library()
    fake = ctypes.c_void_p(0x10000)
    a = B.BwdArgs(fwd=_args(saved=fake, solve_degree=7), do_=fake, dq=fake, dk=fake, dv=fake,
                  dg=fake, dbeta=fake, grad_dtype=B.GDN_BF16)
    assert lib.gdn_chunk_bwd(ctypes.byref(a), None) == B.GDN_E_WORKSPACE
    exact = B.BwdArgs(fwd=_args(saved=fake), do_=fake, dq=fake, dk=fake, dv=fake, dg=fake,
                      dbeta=fake, grad_dtype=B.GDN_BF16)
    slots = 1 + 2
    assert (lib.gdn_bwd_workspace_bytes(ctypes.byref(a)) -
            lib.gdn_bwd_workspace_bytes(ctypes.byref(exact))) >= slots * 4 * 64 * 64 * 4
    for d in (1, 3, 7, 15, 31, 63):                   # every admitted degree passes the forward checks
        f = _args(solve_degree=d)
        assert lib.gdn_fwd_workspace_bytes(ctypes.byref(f)) > 0


def test_qdq_state_rejects_before_launch():
    lib = B.load_library()
    fake = ctypes.c_void_p(0x10000)
    cases = [((fake, fake, None, None, 2, 128, 128, 64, 0), B.GDN_E_UNSUPPORTED),
             ((fake, fake, None, None, 2, 128, 128, 48, 1), B.GDN_E_UNSUPPORTED),
             ((fake, fake, None, None, 2, 128, 96, 64, 1), B.GDN_E_INVALID),
             ((None, fake, None, None, 2, 128, 128, 64, 1), B.GDN_E_INVALID),
             ((fake, ctypes.c_void_p(0x10008), None, None, 2, 128, 128, 64, 2), B.GDN_E_INVALID),
             ((fake, fake, None, None, 0, 128, 128, 64, 1), B.GDN_OK)]
    for args, status in cases:
        assert lib.gdn_qdq_state(*args, None) == status, args


def test_binding_backward_takes_the_forward_policy():
    """The saved buffer carries the policy of the forward that wrote it; the
    binding's backward takes omitted policy arguments from it and refuses a
    different one (the C ABI checks the same stamp on the device)."""
    import torch
    saved = torch.zeros(16, dtype=torch.uint8)
    saved.gdn_policy = dict(state_fmt=B.QDQ_E4M3, w_fmt=B.QDQ_E4M3, block_v=64, solve_degree=3)
    x = torch.zeros(1, 4, 1, 64)
    g = torch.zeros(1, 4, 1)
    for bad in (dict(solve_degree=0), dict(state_fmt=B.QDQ_INT8), dict(block_v=32)):
        with pytest.raises(ValueError, match=list(bad)[0]):
            B.gdn_chunk_bwd(x, x, x, g, g, saved, x, **bad)


def test_noalloc_forward_refuses_above_its_scratch():
    """gdn_chunk_fwd_noalloc has a fixed scratch array (64 MiB per GPU): a
    problem whose forward workspace is larger is refused before any launch,
    with GDN_E_UNSUPPORTED and a message naming the entry point."""
    lib = B.load_library()
    a = _args(T=4096, Hqk=16, Hv=16)
    assert lib.gdn_fwd_workspace_bytes(ctypes.byref(a)) > B.NOALLOC_SCRATCH_BYTES
    assert lib.gdn_chunk_fwd_noalloc(ctypes.byref(a), None) == B.GDN_E_UNSUPPORTED
    assert 'noalloc' in lib.gdn_last_error().decode()
    bad = _args(chunk_size=32)                        # the ordinary checks come first
    assert lib.gdn_chunk_fwd_noalloc(ctypes.byref(bad), None) == B.GDN_E_UNSUPPORTED
    assert 'chunk_size' in lib.gdn_last_error().decode()


# ------------------------------------------------------------------ decode
def _dargs(**kw):
    fake = ctypes.c_void_p(0x10000)
    a = B.DecodeArgs(B=1, T=257, Hqk=2, Hv=4, Dk=128, Dv=128, num_seqs=1, io_dtype=B.GDN_BF16,
                     scale=0.1, start=64, state_fmt=B.QDQ_INT8, block_v=64,
                     readout=B.READOUT_BEFORE_WRITE)
    for name in ('q', 'k', 'v', 'g', 'beta', 'o'):
        setattr(a, name, fake)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


DECODE_BAD = [
    (dict(state_fmt=3), B.GDN_E_UNSUPPORTED, 'format'),
    (dict(block_v=48), B.GDN_E_UNSUPPORTED, 'block_v'),
    (dict(Dv=64, block_v=128), B.GDN_E_INVALID, 'does not divide'),
    (dict(readout=2), B.GDN_E_INVALID, 'readout'),
    (dict(start=-1), B.GDN_E_INVALID, 'start'),
    (dict(Hv=6, Hqk=4), B.GDN_E_INVALID, 'multiple'),
    (dict(Dk=96), B.GDN_E_UNSUPPORTED, 'Dk'),
    (dict(Dv=32), B.GDN_E_UNSUPPORTED, 'Dv'),
    (dict(io_dtype=3), B.GDN_E_INVALID, 'io_dtype'),
    (dict(num_seqs=2), B.GDN_E_INVALID, 'num_seqs'),
    (dict(scale=float('inf')), B.GDN_E_INVALID, 'scale'),
    (dict(v=None), B.GDN_E_INVALID, 'v is NULL'),
    (dict(o=None), B.GDN_E_INVALID, 'o is NULL'),
    (dict(h_in=ctypes.c_void_p(0x10008)), B.GDN_E_INVALID, 'aligned'),
]


@pytest.mark.parametrize("kw,status,msg", DECODE_BAD)
def test_decode_forward_rejects_before_launch(kw, status, msg):
    lib = B.load_library()
    a = _dargs(**kw)
    assert lib.gdn_decode_fwd(ctypes.byref(a), None) == status
    assert msg in lib.gdn_last_error().decode()


def test_decode_saved_bytes_and_backward_checks():
    """Saved written states: one per decode step plus the first write of each
    sequence, in B*T + N slots (codes, then scales, then the stamp); the
    backward needs that buffer and, with grouped heads, its workspace."""
    lib = B.load_library()
    a = _dargs()
    slots = 257 + 1
    codes = slots * 4 * 128 * 128
    scales = slots * 4 * 2 * 4
    r256 = lambda x: (x + 255) // 256 * 256
    assert lib.gdn_decode_saved_bytes(ctypes.byref(a)) == r256(r256(codes) + scales) + 256
    off = _dargs(state_fmt=B.QDQ_OFF)
    assert lib.gdn_decode_saved_bytes(ctypes.byref(off)) == r256(codes * 4) + 256
    assert lib.gdn_decode_saved_bytes(ctypes.byref(_dargs(readout=7))) == 0
    fake = ctypes.c_void_p(0x10000)
    b = B.DecodeBwdArgs(fwd=_dargs(), do_=fake, dq=fake, dk=fake, dv=fake, dg=fake, dbeta=fake,
                        grad_dtype=B.GDN_BF16)
    assert lib.gdn_decode_bwd(ctypes.byref(b), None) == B.GDN_E_INVALID      # no saved buffer
    assert 'saved' in lib.gdn_last_error().decode()
    b.fwd.saved = fake
    need = lib.gdn_decode_bwd_workspace_bytes(ctypes.byref(b))
    # partial dq, dk, dg, dbeta per token, value head and group of 64-column
    # slabs (Dv 128 with 64-wide scale tiles: two groups), 2 Dk + 4 floats each
    assert need == r256(257 * 4 * 2 * (2 * 128 + 4) * 4)
    assert lib.gdn_decode_bwd(ctypes.byref(b), None) == B.GDN_E_WORKSPACE
    b.fwd.Hqk = 4                                                 # no head groups, two slab groups
    assert lib.gdn_decode_bwd_workspace_bytes(ctypes.byref(b)) == r256(257 * 4 * 2 * 260 * 4)
    b.fwd.block_v = 128                                           # one tile spans the head
    assert lib.gdn_decode_bwd_workspace_bytes(ctypes.byref(b)) == 0
    b.fwd.block_v = 64
    b.grad_dtype = 9
    assert lib.gdn_decode_bwd(ctypes.byref(b), None) == B.GDN_E_INVALID
