"""ctypes binding of include/gdn.h: argument marshalling only.

The functions below take torch tensors that already live on a ROCm device,
allocate the outputs with torch (device memory plumbing), fill the C argument
structs with raw device pointers and call the HIP library on torch's current
stream. No step of the computation runs here. If libgdn_hip.so is missing the
import of this module's functions fails loudly; there is no fallback.
"""
import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'libgdn_hip.so')

GDN_OK, GDN_E_INVALID, GDN_E_UNSUPPORTED, GDN_E_WORKSPACE, GDN_E_HIP = 0, -1, -2, -3, -4
QDQ_OFF, QDQ_E4M3, QDQ_INT8 = 0, 1, 2
GDN_BF16, GDN_F32 = 0, 1

c_i32, c_i64, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class QdqPolicy(ctypes.Structure):
    _fields_ = [('state_fmt', c_i32), ('w_fmt', c_i32), ('block_v', c_i32), ('chunk_size', c_i32),
                ('solve_degree', c_i32), ('read_fmt', c_i32)]


class FwdArgs(ctypes.Structure):
    _fields_ = [('B', c_i32), ('T', c_i32), ('Hqk', c_i32), ('Hv', c_i32), ('Dk', c_i32),
                ('Dv', c_i32), ('num_seqs', c_i32), ('io_dtype', c_i32), ('scale', c_f32),
                ('prefix_len', c_i32), ('policy', QdqPolicy), ('q', c_vp), ('k', c_vp), ('v', c_vp), ('g', c_vp),
                ('beta', c_vp), ('h0', c_vp), ('cu_seqlens', c_vp), ('o', c_vp), ('ht', c_vp),
                ('saved', c_vp), ('workspace', c_vp), ('workspace_bytes', c_sz)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [('B', c_i32), ('T', c_i32), ('Hqk', c_i32), ('Hv', c_i32), ('Dk', c_i32),
                ('Dv', c_i32), ('num_seqs', c_i32), ('io_dtype', c_i32), ('scale', c_f32),
                ('start', c_i32), ('state_fmt', c_i32), ('block_v', c_i32), ('readout', c_i32),
                ('q', c_vp), ('k', c_vp), ('v', c_vp), ('g', c_vp), ('beta', c_vp),
                ('h_in', c_vp), ('cu_seqlens', c_vp), ('o', c_vp), ('ht', c_vp), ('saved', c_vp)]


class DecodeBwdArgs(ctypes.Structure):
    _fields_ = [('fwd', DecodeArgs), ('do_', c_vp), ('dht', c_vp), ('grad_dtype', c_i32),
                ('dq', c_vp), ('dk', c_vp), ('dv', c_vp), ('dg', c_vp), ('dbeta', c_vp),
                ('dh_in', c_vp), ('workspace', c_vp), ('workspace_bytes', c_sz)]


READOUT_BEFORE_WRITE, READOUT_AFTER_WRITE = 0, 1


class SavedLayout(ctypes.Structure):
    _fields_ = [('num_slots', c_i64), ('off_state', c_i64), ('off_state_scale', c_i64),
                ('off_w', c_i64), ('off_w_scale', c_i64), ('off_x', c_i64), ('off_anchor', c_i64),
                ('off_meta', c_i64), ('total_bytes', c_i64)]


class BwdArgs(ctypes.Structure):
    _fields_ = [('fwd', FwdArgs), ('do_', c_vp), ('dht', c_vp), ('grad_dtype', c_i32),
                ('dq', c_vp), ('dk', c_vp), ('dv', c_vp), ('dg', c_vp), ('dbeta', c_vp),
                ('dh0', c_vp), ('workspace', c_vp), ('workspace_bytes', c_sz)]


_LIB = None


def load_library():
    """Load libgdn_hip.so (built in-tree by build.py); raise if it is absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f'{LIB_PATH} is missing: build it with '
                           'python -m gateddeltanet_chunked_recurrence_amd.build')
    lib = ctypes.CDLL(LIB_PATH)
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_abi_version.restype = c_i32
    for name, argt in (('gdn_chunk_fwd', [ctypes.POINTER(FwdArgs), c_vp]),
                       ('gdn_chunk_fwd_noalloc', [ctypes.POINTER(FwdArgs), c_vp]),
                       ('gdn_chunk_fwd_prep', [ctypes.POINTER(FwdArgs), c_vp]),
                       ('gdn_chunk_fwd_state', [ctypes.POINTER(FwdArgs), c_vp]),
                       ('gdn_chunk_bwd', [ctypes.POINTER(BwdArgs), c_vp]),
                       ('gdn_saved_layout', [ctypes.POINTER(FwdArgs), ctypes.POINTER(SavedLayout)]),
                       ('gdn_qdq_state', [c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32,
                                          c_i32, c_vp]),
                       ('gdn_decode_fwd', [ctypes.POINTER(DecodeArgs), c_vp]),
                       ('gdn_decode_bwd', [ctypes.POINTER(DecodeBwdArgs), c_vp])):
        f = getattr(lib, name)
        f.argtypes = argt
        f.restype = c_i32
    lib.gdn_fwd_schedule.argtypes = [ctypes.POINTER(FwdArgs), c_i32, ctypes.POINTER(c_i32)]
    lib.gdn_fwd_schedule.restype = c_i32
    lib.gdn_device_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
    lib.gdn_device_errors.restype = c_i32
    lib.gdn_saved_bytes.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.gdn_saved_bytes.restype = c_sz
    lib.gdn_fwd_workspace_bytes.argtypes = [ctypes.POINTER(FwdArgs)]
    lib.gdn_fwd_workspace_bytes.restype = c_sz
    lib.gdn_bwd_workspace_bytes.argtypes = [ctypes.POINTER(BwdArgs)]
    lib.gdn_bwd_workspace_bytes.restype = c_sz
    lib.gdn_decode_saved_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.gdn_decode_saved_bytes.restype = c_sz
    lib.gdn_decode_bwd_workspace_bytes.argtypes = [ctypes.POINTER(DecodeBwdArgs)]
    lib.gdn_decode_bwd_workspace_bytes.restype = c_sz
    _LIB = lib
    return lib


class GdnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f'gdn status {status}: {msg}')
        self.status = status


def _check(status):
    if status != GDN_OK:
        raise GdnError(status, load_library().gdn_last_error().decode())


DEVERR_LDS_WAIT, DEVERR_FLAG_WAIT, DEVERR_SAVED_STAMP, DEVERR_P_RANGE = 1, 2, 4, 8


def fwd_schedule(args, cus=0):
    """gdn_fwd_schedule: the schedule gdn_chunk_fwd takes for these FwdArgs on
    a device of `cus` CUs (0: the current one), as a dict (overlapped, items,
    head_items, rest_blocks)."""
    out = (c_i32 * 4)()
    _check(load_library().gdn_fwd_schedule(ctypes.byref(args), cus, out))
    return dict(overlapped=bool(out[0]), items=out[1], head_items=out[2], rest_blocks=out[3])


def device_errors():
    """Sticky device error flags of the current device (synchronizes, then
    reads and clears them); 0 when no kernel reported a problem."""
    v = ctypes.c_uint32(0)
    _check(load_library().gdn_device_errors(ctypes.byref(v)))
    return int(v.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_fwd_args(q, k, v, g, beta, scale, h0, cu_seqlens, state_fmt, w_fmt, block_v,
                  o=None, ht=None, saved=None, num_seqs=None, solve_degree=0, read_fmt=0,
                  prefix_len=0):
    """Fill the forward argument struct from tensor shapes and pointers."""
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if num_seqs is None:
        num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    io = GDN_F32 if q.dtype == torch.float32 else GDN_BF16
    a = FwdArgs(B=B, T=T, Hqk=Hqk, Hv=Hv, Dk=Dk, Dv=Dv, num_seqs=num_seqs, io_dtype=io,
                scale=float(1.0 / math.sqrt(Dk) if scale is None else scale),
                prefix_len=prefix_len,
                policy=QdqPolicy(state_fmt, w_fmt, block_v, 64, solve_degree, read_fmt))
    for name, t in (('q', q), ('k', k), ('v', v), ('g', g), ('beta', beta), ('h0', h0),
                    ('cu_seqlens', cu_seqlens), ('o', o), ('ht', ht), ('saved', saved)):
        setattr(a, name, _ptr(t))
    return a


def saved_layout(args):
    lay = SavedLayout()
    _check(load_library().gdn_saved_layout(ctypes.byref(args), ctypes.byref(lay)))
    return lay


def gdn_chunk_fwd(q, k, v, g, beta, scale=None, h0=None, cu_seqlens=None, state_fmt=QDQ_OFF,
                  w_fmt=QDQ_OFF, block_v=64, output_final_state=True, save_for_backward=False,
                  solve_degree=0, read_fmt=QDQ_OFF, prefix_len=0, out=None):
    """Chunked forward on q's device and torch's current stream.

    q, k [B, T, Hqk, Dk], v [B, T, Hv, Dv] (bf16, or FP32 with Dk = 64);
    g, beta [B, T, Hv] FP32; h0 [N, Hv, Dk, Dv] FP32 or None; cu_seqlens int32
    [N + 1] (B = 1) or None. solve_degree: 0 for the exact solve, or a
    Neumann degree 1, 3, 7, 15, 31, 63 (bf16 inputs). read_fmt: QDQ_E4M3 for
    the two-precision profile (FP32 carry, E4M3 read copy; state_fmt off).
    prefix_len > 0 runs only the first prefix_len tokens of every sequence
    (o of later tokens is left as it was). out: optional preallocated o.
    Returns (o, ht or None, saved uint8 buffer or None).
    """
    lib = load_library()
    dev = q.device
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    o = torch.empty(B, T, Hv, Dv, dtype=q.dtype, device=dev) if out is None else out
    ht = torch.empty(N, Hv, Dk, Dv, dtype=torch.float32, device=dev) if output_final_state else None
    a = make_fwd_args(q, k, v, g, beta, scale, h0, cu_seqlens, state_fmt, w_fmt, block_v, o, ht,
                      solve_degree=solve_degree, read_fmt=read_fmt, prefix_len=prefix_len)
    saved = None
    if save_for_backward:
        nbytes = lib.gdn_saved_bytes(ctypes.byref(a))
        if nbytes == 0:
            _check(lib.gdn_chunk_fwd(ctypes.byref(a), None))     # reports the shape error
        saved = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        # the policy travels with the buffer, so the backward cannot pick another
        saved.gdn_policy = dict(state_fmt=state_fmt, w_fmt=w_fmt, block_v=block_v,
                                solve_degree=solve_degree, read_fmt=read_fmt,
                                prefix_len=prefix_len)
        a.saved = _ptr(saved)
    wbytes = lib.gdn_fwd_workspace_bytes(ctypes.byref(a))
    ws = torch.empty(wbytes, dtype=torch.uint8, device=dev) if wbytes else None
    a.workspace = _ptr(ws)
    a.workspace_bytes = wbytes
    _check(lib.gdn_chunk_fwd(ctypes.byref(a), _stream(dev)))
    return o, ht, saved


NOALLOC_SCRATCH_BYTES = 64 << 20


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, scale=None, h0=None, cu_seqlens=None,
                          state_fmt=QDQ_OFF, w_fmt=QDQ_OFF, block_v=64, output_final_state=True,
                          out=None):
    """gdn_chunk_fwd through the allocation-free entry point: the library
    uses its fixed per-GPU scratch array instead of a workspace. `out` may
    pass preallocated (o, ht); otherwise they are allocated here (by torch,
    outside the library call). Returns (o, ht or None)."""
    lib = load_library()
    dev = q.device
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    if out is None:
        o = torch.empty(B, T, Hv, Dv, dtype=q.dtype, device=dev)
        ht = torch.empty(N, Hv, Dk, Dv, dtype=torch.float32, device=dev) \
            if output_final_state else None
    else:
        o, ht = out
    a = make_fwd_args(q, k, v, g, beta, scale, h0, cu_seqlens, state_fmt, w_fmt, block_v, o, ht)
    _check(lib.gdn_chunk_fwd_noalloc(ctypes.byref(a), _stream(dev)))
    return o, ht


class FwdPlan:
    """Forward arguments, outputs and workspace prepared once, for running
    the two forward stages (prep, state) as separate calls on the current
    stream: plan.prep(); plan.state(), or both in one call: plan.forward().
    Outputs: plan.o, plan.ht, and plan.saved (the backward's saved buffer)
    with save=True; prefix_len > 0 runs only the first prefix_len tokens of
    every sequence (the other rows of plan.o are not written)."""

    def __init__(self, q, k, v, g, beta, scale=None, h0=None, cu_seqlens=None,
                 state_fmt=QDQ_OFF, w_fmt=QDQ_OFF, block_v=64, solve_degree=0, read_fmt=QDQ_OFF,
                 save=False, prefix_len=0):
        lib = load_library()
        dev = q.device
        B, T, Hqk, Dk = q.shape
        Hv, Dv = v.shape[2], v.shape[3]
        N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
        self.o = torch.empty(B, T, Hv, Dv, dtype=q.dtype, device=dev)
        self.ht = torch.empty(N, Hv, Dk, Dv, dtype=torch.float32, device=dev)
        self._keep = (q, k, v, g, beta, h0, cu_seqlens)
        self.args = make_fwd_args(q, k, v, g, beta, scale, h0, cu_seqlens, state_fmt, w_fmt,
                                  block_v, self.o, self.ht, solve_degree=solve_degree,
                                  read_fmt=read_fmt, prefix_len=prefix_len)
        self.saved = None
        if save:
            self.saved = torch.empty(lib.gdn_saved_bytes(ctypes.byref(self.args)), dtype=torch.uint8,
                                     device=dev)
            self.args.saved = _ptr(self.saved)
        wbytes = lib.gdn_fwd_workspace_bytes(ctypes.byref(self.args))
        self.ws = torch.empty(wbytes, dtype=torch.uint8, device=dev) if wbytes else None
        self.args.workspace = _ptr(self.ws)
        self.args.workspace_bytes = wbytes
        self.dev = dev

    def forward(self):
        """The whole forward in one call (gdn_chunk_fwd: the overlapped
        schedule where it applies)."""
        _check(load_library().gdn_chunk_fwd(ctypes.byref(self.args), _stream(self.dev)))

    def schedule(self, cus=0):
        return fwd_schedule(self.args, cus)

    def prep(self):
        _check(load_library().gdn_chunk_fwd_prep(ctypes.byref(self.args), _stream(self.dev)))

    def state(self):
        _check(load_library().gdn_chunk_fwd_state(ctypes.byref(self.args), _stream(self.dev)))


def gdn_chunk_bwd(q, k, v, g, beta, saved, do, dht=None, scale=None, h0=None, cu_seqlens=None,
                  state_fmt=None, w_fmt=None, block_v=None, grad_dtype=None, solve_degree=None,
                  read_fmt=None, prefix_len=None, out=None):
    """Backward of gdn_chunk_fwd (identity straight-through at both QDQ sites)
    from the forward's `saved` buffer. Returns dict dq, dk, dv, dg, dbeta, dh0.
    Policy arguments left as None are taken from the policy the forward
    attached to `saved`; one that is given must equal it. out: optional dict
    of preallocated gradient tensors (with prefix_len only prefix tokens are
    written, so a decode backward may fill the rest)."""
    pol = dict(state_fmt=state_fmt, w_fmt=w_fmt, block_v=block_v, solve_degree=solve_degree,
               read_fmt=read_fmt, prefix_len=prefix_len)
    defaults = dict(state_fmt=QDQ_OFF, w_fmt=QDQ_OFF, block_v=64, solve_degree=0,
                    read_fmt=QDQ_OFF, prefix_len=0)
    fwd_pol = getattr(saved, 'gdn_policy', None)
    for key, val in pol.items():
        if fwd_pol is not None:
            fv = fwd_pol.get(key, defaults[key])
            if val is None:
                pol[key] = fv
            elif val != fv and not (key == 'block_v' and fwd_pol['state_fmt'] == QDQ_OFF):
                raise ValueError(f'{key}={val} differs from the forward that wrote `saved` '
                                 f'({key}={fv})')
        elif val is None:
            pol[key] = defaults[key]
    state_fmt, w_fmt, block_v, solve_degree, read_fmt, prefix_len = (
        pol[k_] for k_ in ('state_fmt', 'w_fmt', 'block_v', 'solve_degree', 'read_fmt',
                           'prefix_len'))
    lib = load_library()
    dev = q.device
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    gd = q.dtype if grad_dtype is None else grad_dtype
    out = out if out is not None else dict(dq=torch.empty(B, T, Hqk, Dk, dtype=gd, device=dev),
               dk=torch.empty(B, T, Hqk, Dk, dtype=gd, device=dev),
               dv=torch.empty(B, T, Hv, Dv, dtype=gd, device=dev),
               dg=torch.empty(B, T, Hv, dtype=torch.float32, device=dev),
               dbeta=torch.empty(B, T, Hv, dtype=torch.float32, device=dev),
               dh0=torch.empty(N, Hv, Dk, Dv, dtype=torch.float32, device=dev)
               if h0 is not None else None)
    fa = make_fwd_args(q, k, v, g, beta, scale, h0, cu_seqlens, state_fmt, w_fmt, block_v,
                       saved=saved, solve_degree=solve_degree, read_fmt=read_fmt,
                       prefix_len=prefix_len)
    a = BwdArgs(fwd=fa, do_=_ptr(do), dht=_ptr(dht),
                grad_dtype=GDN_F32 if gd == torch.float32 else GDN_BF16,
                dq=_ptr(out['dq']), dk=_ptr(out['dk']), dv=_ptr(out['dv']), dg=_ptr(out['dg']),
                dbeta=_ptr(out['dbeta']), dh0=_ptr(out['dh0']))
    nbytes = lib.gdn_bwd_workspace_bytes(ctypes.byref(a))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    a.workspace = _ptr(ws)
    a.workspace_bytes = ws.numel()
    _check(lib.gdn_chunk_bwd(ctypes.byref(a), _stream(dev)))
    return out


def gdn_qdq_state(x, fmt, block_v, return_codes=False, out=None):
    """QDQ of FP32 states x [n, Dk, Dv] per [Dk, block_v] tile.
    Returns (y, scales [n, Dv / block_v], codes uint8 or None)."""
    lib = load_library()
    n, Dk, Dv = x.shape
    y = torch.empty_like(x) if out is None else out
    scales = torch.empty(n, Dv // block_v if block_v and Dv % block_v == 0 else 1,
                         dtype=torch.float32, device=x.device)
    codes = torch.empty(n, Dk, Dv, dtype=torch.uint8, device=x.device) if return_codes else None
    _check(lib.gdn_qdq_state(_ptr(x), _ptr(y), _ptr(scales), _ptr(codes), n, Dk, Dv, block_v, fmt,
                             _stream(x.device)))
    return y, scales, codes


# --------------------------------------------------------------- decode
def make_decode_args(q, k, v, g, beta, scale, h_in, cu_seqlens, start, state_fmt, block_v,
                     readout, o=None, ht=None, saved=None):
    """Fill the decode argument struct from tensor shapes and pointers."""
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    num_seqs = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    io = GDN_F32 if q.dtype == torch.float32 else GDN_BF16
    a = DecodeArgs(B=B, T=T, Hqk=Hqk, Hv=Hv, Dk=Dk, Dv=Dv, num_seqs=num_seqs, io_dtype=io,
                   scale=float(1.0 / math.sqrt(Dk) if scale is None else scale), start=start,
                   state_fmt=state_fmt, block_v=block_v, readout=readout)
    for name, t in (('q', q), ('k', k), ('v', v), ('g', g), ('beta', beta), ('h_in', h_in),
                    ('cu_seqlens', cu_seqlens), ('o', o), ('ht', ht), ('saved', saved)):
        setattr(a, name, _ptr(t))
    return a


def gdn_decode_fwd(q, k, v, g, beta, scale=None, h_in=None, cu_seqlens=None, start=0,
                   state_fmt=QDQ_OFF, block_v=64, readout=READOUT_BEFORE_WRITE,
                   save_for_backward=False, out=None):
    """Decode steps over tokens [start, len) of every sequence from h_in,
    each followed by a write of the state through the state quantizer.
    Shapes as gdn_chunk_fwd. out: optional preallocated o (tokens before
    `start` are left as they are). Returns (o, ht, saved or None); ht is the
    last written state."""
    lib = load_library()
    dev = q.device
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    o = torch.empty(B, T, Hv, Dv, dtype=q.dtype, device=dev) if out is None else out
    ht = torch.empty(N, Hv, Dk, Dv, dtype=torch.float32, device=dev)
    a = make_decode_args(q, k, v, g, beta, scale, h_in, cu_seqlens, start, state_fmt, block_v,
                         readout, o, ht)
    saved = None
    if save_for_backward:
        nbytes = lib.gdn_decode_saved_bytes(ctypes.byref(a))
        if nbytes == 0:
            _check(lib.gdn_decode_fwd(ctypes.byref(a), None))   # reports the argument error
        saved = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        saved.gdn_decode = dict(start=start, state_fmt=state_fmt, block_v=block_v,
                                readout=readout)
        a.saved = _ptr(saved)
    _check(lib.gdn_decode_fwd(ctypes.byref(a), _stream(dev)))
    return o, ht, saved


def gdn_decode_bwd(q, k, v, g, beta, saved, do, dht=None, scale=None, h_in=None, cu_seqlens=None,
                   grad_dtype=None, out=None):
    """Backward of gdn_decode_fwd (identity straight-through at every write)
    from its saved buffer, under the policy the forward attached to it.
    Returns dict dq, dk, dv, dg, dbeta, dh_in (dh_in when h_in is given);
    only decode tokens are written."""
    pol = getattr(saved, 'gdn_decode', None)
    if pol is None:
        raise ValueError('`saved` does not come from gdn_decode_fwd(save_for_backward=True)')
    lib = load_library()
    dev = q.device
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else B
    gd = q.dtype if grad_dtype is None else grad_dtype
    if out is None:
        out = dict(dq=torch.empty(B, T, Hqk, Dk, dtype=gd, device=dev),
                   dk=torch.empty(B, T, Hqk, Dk, dtype=gd, device=dev),
                   dv=torch.empty(B, T, Hv, Dv, dtype=gd, device=dev),
                   dg=torch.empty(B, T, Hv, dtype=torch.float32, device=dev),
                   dbeta=torch.empty(B, T, Hv, dtype=torch.float32, device=dev))
    out['dh_in'] = torch.empty(N, Hv, Dk, Dv, dtype=torch.float32, device=dev) \
        if h_in is not None else None
    fa = make_decode_args(q, k, v, g, beta, scale, h_in, cu_seqlens, pol['start'],
                          pol['state_fmt'], pol['block_v'], pol['readout'], saved=saved)
    a = DecodeBwdArgs(fwd=fa, do_=_ptr(do), dht=_ptr(dht),
                      grad_dtype=GDN_F32 if gd == torch.float32 else GDN_BF16,
                      dq=_ptr(out['dq']), dk=_ptr(out['dk']), dv=_ptr(out['dv']),
                      dg=_ptr(out['dg']), dbeta=_ptr(out['dbeta']), dh_in=_ptr(out['dh_in']))
    nbytes = lib.gdn_decode_bwd_workspace_bytes(ctypes.byref(a))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    a.workspace = _ptr(ws)
    a.workspace_bytes = nbytes
    _check(lib.gdn_decode_bwd(ctypes.byref(a), _stream(dev)))
    return out


def gdn_prefill_decode_fwd(q, k, v, g, beta, prefix_len, scale=None, h0=None, cu_seqlens=None,
                           state_fmt=QDQ_OFF, w_fmt=QDQ_OFF, block_v=64,
                           readout=READOUT_BEFORE_WRITE, save_for_backward=False):
    """Decode continuation: the exact chunk prefill of the first prefix_len
    tokens of every sequence (gdn_chunk_fwd with prefix_len), then decode
    steps over the rest from the prefill's final state (gdn_decode_fwd with
    start = prefix_len), into one o. Returns (o, ht, saved); saved is the
    pair of both calls' buffers (or None)."""
    o, h_mid, s_pre = None, h0, None
    if prefix_len > 0:
        o, h_mid, s_pre = gdn_chunk_fwd(q, k, v, g, beta, scale, h0, cu_seqlens, state_fmt, w_fmt,
                                        block_v, True, save_for_backward, prefix_len=prefix_len)
    o, ht, s_dec = gdn_decode_fwd(q, k, v, g, beta, scale, h_mid, cu_seqlens, prefix_len,
                                  state_fmt, block_v, readout, save_for_backward, out=o)
    saved = None
    if save_for_backward:
        saved = dict(prefill=s_pre, decode=s_dec, h_mid=h_mid, prefix_len=prefix_len)
    return o, ht, saved


def gdn_prefill_decode_bwd(q, k, v, g, beta, saved, do, dht=None, scale=None, h0=None,
                           cu_seqlens=None, grad_dtype=None):
    """Backward of gdn_prefill_decode_fwd: the decode backward (its dh_in is
    the gradient of the prefill's final state), then the prefill's chunk
    backward with that as dht, into one set of gradients. Returns dict dq,
    dk, dv, dg, dbeta, dh0 (dh0 when h0 is given)."""
    P = saved['prefix_len']
    h_mid = saved['h_mid']
    out = gdn_decode_bwd(q, k, v, g, beta, saved['decode'], do, dht, scale, h_mid, cu_seqlens,
                         grad_dtype)
    dh_mid = out.pop('dh_in')
    if P > 0:
        res = gdn_chunk_bwd(q, k, v, g, beta, saved['prefill'], do, dh_mid, scale, h0, cu_seqlens,
                            grad_dtype=grad_dtype, out=dict(out, dh0=None if h0 is None else
                                                            torch.empty_like(h0)))
        out['dh0'] = res['dh0']
    else:
        out['dh0'] = dh_mid
    return out
