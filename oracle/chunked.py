"""Oracle: chunked (WY-form) gated delta rule with state/W fake QDQ, and its
identity straight-through backward (float64, plain PyTorch CPU ops).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path.

Sources. "[1/4] GDN state/W QAT foundation", "What does this PR do?": dynamic
FP8 E4M3 fake QDQ at the recurrent-state and WY-activation (W) sites of the
chunked training path, chunk size 64, exact triangular solve, identity
straight-through gradients, the forward's quantized W reused by the
backward. "[2/4] GDN/KDA decode QAT with INT8 recurrent state", "What does
this PR do?": INT8 state with per-head [Dk, block_v] scales. The pages give
no formulas; the chunk form below is derived from the token recurrence in
oracle/recurrent.py (substituting the token update into itself over a
chunk) and tested equal to it.

Per (sequence, value head) and chunk of n <= C tokens (sequence-relative;
positions i, j = 1..n) with incoming state S:

    gamma_i   = g_1 + ... + g_i                       (chunk-local cumsum)
    Gam_ij    = exp(gamma_i - gamma_j) for i >= j, else 0
    L_ij      = beta_i (k_i . k_j) Gam_ij   for i > j, else 0
    T         = (I + L)^-1 diag(beta)                 (exact solve: (I+L) T = diag(beta))
    W         = T diag(exp(gamma)) K,   U = T V
    Wq        = QDQ_W(W)     one scale per (sequence, chunk, head) over [n, Dk]
    Sq        = QDQ_S(S)     one scale per [Dk, block_v] tile
    Vnew      = U - Wq Sq
    O         = scale (diag(exp(gamma)) Q Sq + ((Q K^T) * Gam) Vnew)
    S_next    = exp(gamma_n) Sq + (diag(exp(gamma_n - gamma)) K)^T Vnew

ht is the last S_next, not quantized. Each QDQ is the FP32 function of
oracle/qdq.py applied to fl32 of its float64 argument; its backward is the
identity.

Opt-in approximate inverse ("[7/7] Experimental GDN/KDA approximate-inverse
QAT", "What does this PR do?"): a solve policy with an explicit Neumann
polynomial degree d replaces the exact solve by

    T_d       = (sum_{m=0..d} (-L)^m) diag(beta)

and the backward differentiates that polynomial (autograd through the same
sum). L is strictly lower triangular, so (-L)^n = 0 for n >= n_c and any
d >= n_c - 1 gives the exact inverse.

Opt-in two-precision profile ("[5/8] ReplaySSM state QAT and two-precision
GDN", "What does this PR do?" and "Usage": the state quantizer disabled, an
FP32 recurrence anchor, and a dynamic E4M3 read quantizer grouped by 128 key
channels per value row, whose errors never overwrite the anchor). On the
chunk path, read here as: with read_fmt set (state_fmt must be off) every
read of the chunk's incoming state uses Sr = QDQ_R(S), one scale per value
column over all Dk key channels, while the carry keeps S:

    Vnew      = U - Wq Sr
    O         = scale (diag(exp(gamma)) Q Sr + ((Q K^T) * Gam) Vnew)
    S_next    = exp(gamma_n) S + (diag(exp(gamma_n - gamma)) K)^T Vnew
"""
import math

import numpy as np
import torch

from .qdq import FMT_OFF, qdq32


class _QdqSte(torch.autograd.Function):
    """Fake QDQ forward (FP32, oracle/qdq.py), identity backward."""

    @staticmethod
    def forward(ctx, x, fmt, tile_axes, sink):
        x32 = x.detach().to(torch.float32).cpu().numpy()
        out, c, d = qdq32(x32, fmt, tile_axes)
        if sink is not None:
            sink.append((c, d))
        return torch.from_numpy(out.astype(np.float64))

    @staticmethod
    def backward(ctx, gout):
        return gout, None, None, None


def qdq_ste(x, fmt, tile_axes, sink=None):
    if fmt == FMT_OFF:
        return x
    return _QdqSte.apply(x, fmt, tile_axes, sink)


def gate_matrix(gam):
    """Gam_ij = exp(gamma_i - gamma_j) for i >= j, else 0.  gam: [Z, n]."""
    n = gam.shape[-1]
    lower = torch.ones(n, n, dtype=torch.bool).tril()
    diff = (gam[:, :, None] - gam[:, None, :]).masked_fill(~lower, 0.0)
    return torch.exp(diff) * lower


def neumann_poly(L, degree):
    """sum_{m=0..degree} (-L)^m, term by term ("[7/7]", "What does this PR
    do?": the explicit Neumann polynomial of the approximate inverse)."""
    eye = torch.eye(L.shape[-1], dtype=L.dtype).expand_as(L)
    term, acc = eye, eye
    for _ in range(degree):
        term = term @ (-L)
        acc = acc + term
    return acc


def wy_factor(Kc, gc, bc, solve_degree=0):
    """Chunk-local gate cumsum, L, and T with (I + L) T = diag(beta), or with
    solve_degree > 0 the Neumann polynomial of that degree in place of
    (I + L)^-1. Kc: [Z, n, Dk], gc, bc: [Z, n]. Returns (gamma, Gam, L, T)."""
    gam = torch.cumsum(gc, dim=-1)
    Gam = gate_matrix(gam)
    n = Kc.shape[1]
    strict = torch.ones(n, n, dtype=torch.bool).tril(-1)
    L = (bc[:, :, None] * (Kc @ Kc.transpose(1, 2)) * Gam) * strict
    if solve_degree:
        return gam, Gam, L, neumann_poly(L, solve_degree) @ torch.diag_embed(bc)
    eye = torch.eye(n, dtype=Kc.dtype).expand_as(L)
    T = torch.linalg.solve_triangular(eye + L, torch.diag_embed(bc), upper=False)
    return gam, Gam, L, T


def _chunk_loop(Q, K, V, g, beta, S, scale, state_fmt, w_fmt, block_v, chunk,
                rec, site_fn, solve_degree=0, read_fmt=FMT_OFF):
    """Z independent (sequence, head) streams of equal length.
    Q, K: [Z, L, Dk]; V: [Z, L, Dv]; g, beta: [Z, L]; S: [Z, Dk, Dv]."""
    Z, Lseq, Dk = Q.shape
    Dv = V.shape[2]
    outs = []
    for r0 in range(0, Lseq, chunk):
        r1 = min(r0 + chunk, Lseq)
        Qc, Kc, Vc = Q[:, r0:r1], K[:, r0:r1], V[:, r0:r1]
        gam, Gam, _, T = wy_factor(Kc, g[:, r0:r1], beta[:, r0:r1], solve_degree)
        W = T @ (torch.exp(gam)[:, :, None] * Kc)
        U = T @ Vc
        Wq = W if w_fmt == FMT_OFF else site_fn(W, w_fmt, (1, 2),
                                                None if rec is None else rec['W'])
        if state_fmt == FMT_OFF:
            Sq = S
        else:
            Sq = site_fn(S.reshape(Z, Dk, Dv // block_v, block_v), state_fmt, (1, 3),
                         None if rec is None else rec['S']).reshape(Z, Dk, Dv)
        # the state as read: Sq, or the two-precision read copy (one scale
        # per value column over the Dk key channels)
        Sr = Sq if read_fmt == FMT_OFF else site_fn(S, read_fmt, (1,),
                                                    None if rec is None else rec['R'])
        Vnew = U - Wq @ Sr
        P = (Qc @ Kc.transpose(1, 2)) * Gam
        outs.append(scale * (torch.exp(gam)[:, :, None] * (Qc @ Sr) + P @ Vnew))
        gl = gam[:, -1]
        Kd = torch.exp(gl[:, None] - gam)[:, :, None] * Kc
        S = torch.exp(gl)[:, None, None] * Sq + Kd.transpose(1, 2) @ Vnew
    return torch.cat(outs, dim=1), S


def _as64(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.to(torch.float64)
    return torch.as_tensor(np.asarray(x, np.float64))


def chunked_fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None,
                state_fmt=FMT_OFF, w_fmt=FMT_OFF, block_v=64, chunk=64,
                record=None, site_fn=None, solve_degree=0, read_fmt=FMT_OFF):
    """q, k: [B, T, Hqk, Dk]; v: [B, T, Hv, Dv]; g, beta: [B, T, Hv];
    h0: [N, Hv, Dk, Dv] or None; cu_seqlens: N+1 offsets (B must be 1).
    float64 torch tensors (autograd flows through them) or arrays.
    Returns (o [B, T, Hv, Dv], ht [N, Hv, Dk, Dv]) as float64 tensors.

    record: optional dict; receives per-sequence lists of exported QDQ codes
    and scales: record['S'][n][c] = (codes [Hv or B*Hv, Dk, Dv/bv, bv],
    d [..., 1, Dv/bv, 1]), record['W'][n][c] = (codes [.., n_c, Dk], d).

    site_fn: optional replacement for the QDQ step, called as
    site_fn(x, fmt, tile_axes, sink) at every site in a fixed order (W then
    S, chunk by chunk); used by the tests' frozen-offset surrogate.

    solve_degree: 0 for the exact solve, else the Neumann polynomial degree
    (any d >= 1) in its place.

    read_fmt: the two-precision profile's read quantizer (state_fmt must be
    off); record['R'][n][c] = (codes [Z, Dk, Dv], d [Z, 1, Dv]). Site order
    per chunk: W, S, then R."""
    site_fn = qdq_ste if site_fn is None else site_fn
    if solve_degree < 0:
        raise ValueError("solve_degree must be 0 (exact) or a polynomial degree >= 1")
    if read_fmt != FMT_OFF and state_fmt != FMT_OFF:
        raise ValueError("the two-precision read copy replaces the state quantizer")
    q, k, v, g, beta, h0 = map(_as64, (q, k, v, g, beta, h0))
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    if Hv % Hqk or (state_fmt != FMT_OFF and Dv % block_v):
        raise ValueError("need Hv % Hqk == 0 and Dv % block_v == 0")
    qv = torch.repeat_interleave(q, G, dim=2)      # value head h reads h // G
    kv = torch.repeat_interleave(k, G, dim=2)
    if record is not None:
        record.setdefault('S', [])
        record.setdefault('W', [])
        record.setdefault('R', [])

    def streams(x, lo, hi):      # [B, T, H, D] -> [B*H, hi-lo, D]
        x = x[:, lo:hi]
        return x.permute(0, 2, 1, *range(3, x.dim())).reshape(
            x.shape[0] * x.shape[2], hi - lo, *x.shape[3:])

    if cu_seqlens is None:
        bounds = [(0, T)]
        S0 = torch.zeros(B * Hv, Dk, Dv, dtype=torch.float64) if h0 is None \
            else h0.reshape(B * Hv, Dk, Dv)
    else:
        assert B == 1
        cu = [int(x) for x in cu_seqlens]
        bounds = list(zip(cu[:-1], cu[1:]))
    o_parts, ht_parts = [], []
    for n, (lo, hi) in enumerate(bounds):
        if cu_seqlens is not None:
            S0 = torch.zeros(Hv, Dk, Dv, dtype=torch.float64) if h0 is None else h0[n]
        rec = None if record is None else {'S': [], 'W': [], 'R': []}
        if hi > lo:
            o_n, S_n = _chunk_loop(streams(qv, lo, hi), streams(kv, lo, hi),
                                   streams(v, lo, hi),
                                   streams(g[..., None], lo, hi)[..., 0],
                                   streams(beta[..., None], lo, hi)[..., 0],
                                   S0, scale, state_fmt, w_fmt, block_v, chunk, rec,
                                   site_fn, solve_degree, read_fmt)
        else:
            o_n, S_n = torch.zeros(S0.shape[0], 0, Dv, dtype=torch.float64), S0
        if record is not None:
            record['S'].append(rec['S'])
            record['W'].append(rec['W'])
            record['R'].append(rec['R'])
        Bn = B if cu_seqlens is None else 1
        o_parts.append(o_n.reshape(Bn, Hv, hi - lo, Dv).permute(0, 2, 1, 3))
        ht_parts.append(S_n.reshape(Bn, Hv, Dk, Dv))
    o = torch.cat(o_parts, dim=1)
    ht = torch.cat(ht_parts, dim=0)
    return o, ht


def chunked_bwd(q, k, v, g, beta, scale, do, dht=None, h0=None, cu_seqlens=None,
                state_fmt=FMT_OFF, w_fmt=FMT_OFF, block_v=64, chunk=64, site_fn=None,
                solve_degree=0, read_fmt=FMT_OFF):
    """Reverse-mode derivative of chunked_fwd with every QDQ's Jacobian taken
    as the identity (identity straight-through estimator). The forward values
    of Sq and Wq are used inside every product, as the saved quantized W is
    in the pages' backward.

    Returns dict of float64 tensors: dq, dk, dv, dg, dbeta, dh0 (dh0 is
    present when h0 is given, and is d/d h0 of the same loss)."""
    leaves = {}
    for name, x in (('q', q), ('k', k), ('v', v), ('g', g), ('beta', beta), ('h0', h0)):
        if x is None:
            continue
        t = _as64(x).clone().requires_grad_(True)
        leaves[name] = t
    o, ht = chunked_fwd(leaves['q'], leaves['k'], leaves['v'], leaves['g'],
                        leaves['beta'], scale, leaves.get('h0'), cu_seqlens,
                        state_fmt, w_fmt, block_v, chunk, site_fn=site_fn,
                        solve_degree=solve_degree, read_fmt=read_fmt)
    outs, grads = [o], [_as64(do)]
    if dht is not None:
        outs.append(ht)
        grads.append(_as64(dht))
    names = list(leaves)
    res = torch.autograd.grad(outs, [leaves[n] for n in names], grads,
                              allow_unused=True)
    out = {}
    for n, r in zip(names, res):
        out['d' + n] = torch.zeros_like(leaves[n]) if r is None else r.detach()
    return out


def default_scale(Dk):
    return 1.0 / math.sqrt(Dk)
