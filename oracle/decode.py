"""Oracle: decode continuation of the gated delta rule with token-state
writes through the state quantizer (float64, plain PyTorch CPU ops), and
its identity straight-through backward (autograd).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path.

Source: "[2/4] GDN/KDA decode QAT with INT8 recurrent state". "What does
this PR do?": an explicit prefix length selects exact chunk prefill
followed by token-state writes; recurrent states are FP8 E4M3 or signed
symmetric dynamic INT8 with per-head [Dk, block_v] scales, nearest-even
rounding and identity straight-through gradients; gradients flow through
initial states and the continuation. "Testing": 257-token trajectories,
nonzero initial states, grouped heads, packed tails, both readouts, split
carry, all state scale widths, first-order input/state gradients.

The pages give no formulas. Readings (plainest ones the rest supports):

  * A decode step is one token of the gated delta rule of
    oracle/recurrent.py, after which the updated state is written to the
    recurrent-state cache through the state quantizer; the next token reads
    the state as written.
  * The state handed to the decode (the prefill's final state, or the
    initial state when there is no prefix) is written to the cache the same
    way before the first decode token.
  * "Both readouts": the token's output is read from the updated state
    either before its write (the value the update computed) or after it
    (the state as written). Both include the token's own write, as the
    chunk path's output does.
  * The decode's final state is the last state written (the cache content).
  * Exact chunk prefill: the chunk path of oracle/chunked.py (state QDQ at
    chunk starts, W QDQ per the policy, exact solve) over the first
    `prefix_len` tokens of every sequence; its final state, not quantized,
    is the state handed over.

Per (sequence, value head), with S the state as handed over:

    S   <- QDQ(S)                                  (first write)
    for each decode token t:
        S   <- exp(g_t) S
        u_t  = beta_t (v_t - S^T k_t)
        S   <- S + k_t u_t^T
        o_before = scale S^T q_t
        S   <- QDQ(S)                              (token-state write)
        o_after  = scale S^T q_t
        o_t  = o_before or o_after (the readout)
    ht = S

QDQ is the FP32 function of oracle/qdq.py on fl32 of its float64 argument,
one scale per [Dk, block_v] tile; identity when the state format is off.
"""
import numpy as np
import torch

from .chunked import _as64, chunked_fwd, qdq_ste
from .qdq import FMT_OFF

READOUT_BEFORE_WRITE = 0
READOUT_AFTER_WRITE = 1


def _bounds(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = [int(x) for x in cu_seqlens]
    return list(zip(cu[:-1], cu[1:]))


def _decode_loop(Q, K, V, g, beta, S, scale, state_fmt, block_v, readout, site_fn, sink):
    """Z = Hv streams of one sequence. Q, K: [Z, L, Dk]; V: [Z, L, Dv];
    g, beta: [Z, L]; S: [Z, Dk, Dv] the state handed over. Returns the
    outputs [Z, L, Dv] and the last written state."""
    Z, Lseq, Dk = Q.shape
    Dv = V.shape[2]

    def write(x):
        if state_fmt == FMT_OFF:
            return x
        y = site_fn(x.reshape(Z, Dk, Dv // block_v, block_v), state_fmt, (1, 3), sink)
        return y.reshape(Z, Dk, Dv)

    S = write(S)
    outs = []
    for t in range(Lseq):
        S = torch.exp(g[:, t])[:, None, None] * S
        u = beta[:, t][:, None] * (V[:, t] - torch.einsum('zkv,zk->zv', S, K[:, t]))
        S = S + K[:, t][:, :, None] * u[:, None, :]
        o_before = scale * torch.einsum('zkv,zk->zv', S, Q[:, t])
        S = write(S)
        if readout == READOUT_AFTER_WRITE:
            outs.append(scale * torch.einsum('zkv,zk->zv', S, Q[:, t]))
        else:
            outs.append(o_before)
    o = torch.stack(outs, dim=1) if outs else torch.zeros(Z, 0, Dv, dtype=torch.float64)
    return o, S


def decode_fwd(q, k, v, g, beta, scale, h_in=None, cu_seqlens=None, start=0,
               state_fmt=FMT_OFF, block_v=64, readout=READOUT_BEFORE_WRITE,
               record=None, site_fn=None):
    """Decode steps over tokens [start, len) of every sequence, from h_in.

    q, k: [B, T, Hqk, Dk]; v: [B, T, Hv, Dv]; g, beta: [B, T, Hv];
    h_in: [N, Hv, Dk, Dv] or None (zero); cu_seqlens: N+1 offsets (B == 1).
    Returns (o [B, T, Hv, Dv] with zeros before `start` of each sequence,
    ht [N, Hv, Dk, Dv]) as float64 tensors; autograd flows through them.

    record: optional dict; record['S'][n] receives the (codes, d) of every
    write of sequence n in order (the first write, then one per token).
    site_fn: optional replacement of the QDQ step (see chunked_fwd)."""
    site_fn = qdq_ste if site_fn is None else site_fn
    q, k, v, g, beta, h_in = map(_as64, (q, k, v, g, beta, h_in))
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if Hv % Hqk or (state_fmt != FMT_OFF and Dv % block_v):
        raise ValueError("need Hv % Hqk == 0 and Dv % block_v == 0")
    if readout not in (READOUT_BEFORE_WRITE, READOUT_AFTER_WRITE):
        raise ValueError("readout must be READOUT_BEFORE_WRITE or READOUT_AFTER_WRITE")
    G = Hv // Hqk
    # token-major [B*T, H, D] views; value head h reads query/key head h // G
    qf = torch.repeat_interleave(q.reshape(B * T, Hqk, Dk), G, dim=1)
    kf = torch.repeat_interleave(k.reshape(B * T, Hqk, Dk), G, dim=1)
    vf, gf, bf = v.reshape(B * T, Hv, Dv), g.reshape(B * T, Hv), beta.reshape(B * T, Hv)
    if record is not None:
        record.setdefault('S', [])
    o_rows, ht = [], []
    pos = 0
    for n, (bos, eos) in enumerate(_bounds(B, T, cu_seqlens)):
        S0 = torch.zeros(Hv, Dk, Dv, dtype=torch.float64) if h_in is None else h_in[n]
        lo = min(bos + start, eos)
        sink = [] if record is not None else None
        o_n, S_n = _decode_loop(qf[lo:eos].transpose(0, 1), kf[lo:eos].transpose(0, 1),
                                vf[lo:eos].transpose(0, 1), gf[lo:eos].T, bf[lo:eos].T,
                                S0, scale, state_fmt, block_v, readout, site_fn, sink)
        if record is not None:
            record['S'].append(sink)
        o_rows.append(torch.zeros(lo - pos, Hv, Dv, dtype=torch.float64))
        o_rows.append(o_n.transpose(0, 1))
        pos = eos
        ht.append(S_n)
    o = torch.cat(o_rows, dim=0).reshape(B, T, Hv, Dv)
    return o, torch.stack(ht, dim=0)


def prefill_decode_fwd(q, k, v, g, beta, scale, prefix_len, h0=None, cu_seqlens=None,
                       state_fmt=FMT_OFF, w_fmt=FMT_OFF, block_v=64,
                       readout=READOUT_BEFORE_WRITE, record=None, site_fn=None):
    """Exact chunk prefill of the first `prefix_len` tokens of every sequence
    (chunked_fwd, chunk 64, from h0), then decode_fwd over the rest from the
    prefill's final state. Returns (o [B, T, Hv, Dv], ht [N, Hv, Dk, Dv]).

    record: optional dict; record['prefill'] receives chunked_fwd's record
    of each sequence's prefix, record['S'] decode_fwd's writes."""
    q, k, v, g, beta, h0 = map(_as64, (q, k, v, g, beta, h0))
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    bounds = _bounds(B, T, cu_seqlens)
    o_pre, h_mid = [], []
    rec_pre = None if record is None else {}
    for n, (bos, eos) in enumerate(bounds):
        hi = min(bos + prefix_len, eos)
        flat = lambda x: x.reshape(B * T, *x.shape[2:])[bos:hi][None]
        h0n = None if h0 is None else h0[n:n + 1]
        r = None if record is None else {}
        o_n, ht_n = chunked_fwd(flat(q), flat(k), flat(v), flat(g), flat(beta), scale, h0n,
                                None, state_fmt, w_fmt, block_v, 64, record=r,
                                site_fn=site_fn)
        if record is not None:
            rec_pre.setdefault('S', []).append(r['S'][0])
            rec_pre.setdefault('W', []).append(r['W'][0])
        o_pre.append((bos, hi, o_n[0]))
        h_mid.append(ht_n[0])
    o_dec, ht = decode_fwd(q, k, v, g, beta, scale, torch.stack(h_mid, dim=0), cu_seqlens,
                           prefix_len, state_fmt, block_v, readout, record, site_fn)
    rows = o_dec.reshape(B * T, Hv, Dv)
    parts, pos = [], 0
    for (bos, hi, o_n), (_, eos) in zip(o_pre, bounds):
        parts += [o_n, rows[hi:eos]]
    o = torch.cat(parts, dim=0).reshape(B, T, Hv, Dv)
    if record is not None:
        record['prefill'] = rec_pre
    return o, ht


def _grads(fn, tensors, do, dht):
    leaves = {}
    for name, x in tensors.items():
        if x is not None:
            leaves[name] = _as64(x).clone().requires_grad_(True)
    o, ht = fn(leaves)
    outs, grads = [o], [_as64(do)]
    if dht is not None:
        outs.append(ht)
        grads.append(_as64(dht))
    res = torch.autograd.grad(outs, list(leaves.values()), grads, allow_unused=True)
    return {'d' + n: (torch.zeros_like(leaves[n]) if r is None else r.detach())
            for n, r in zip(leaves, res)}


def decode_bwd(q, k, v, g, beta, scale, do, dht=None, h_in=None, cu_seqlens=None, start=0,
               state_fmt=FMT_OFF, block_v=64, readout=READOUT_BEFORE_WRITE, site_fn=None):
    """Reverse-mode derivative of decode_fwd with every write's Jacobian the
    identity (identity straight-through); the written values are used in
    every product. Returns dict dq, dk, dv, dg, dbeta and dh_in (when h_in
    is given). Tokens before `start` get zero gradients."""
    fn = lambda L: decode_fwd(L['q'], L['k'], L['v'], L['g'], L['beta'], scale, L.get('h_in'),
                              cu_seqlens, start, state_fmt, block_v, readout, site_fn=site_fn)
    return _grads(fn, dict(q=q, k=k, v=v, g=g, beta=beta, h_in=h_in), do, dht)


def prefill_decode_bwd(q, k, v, g, beta, scale, prefix_len, do, dht=None, h0=None,
                       cu_seqlens=None, state_fmt=FMT_OFF, w_fmt=FMT_OFF, block_v=64,
                       readout=READOUT_BEFORE_WRITE, site_fn=None):
    """Reverse-mode derivative of prefill_decode_fwd (identity
    straight-through at every QDQ site, prefill and decode). Returns dict
    dq, dk, dv, dg, dbeta and dh0 (when h0 is given)."""
    fn = lambda L: prefill_decode_fwd(L['q'], L['k'], L['v'], L['g'], L['beta'], scale,
                                      prefix_len, L.get('h0'), cu_seqlens, state_fmt, w_fmt,
                                      block_v, readout, site_fn=site_fn)
    return _grads(fn, dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), do, dht)
