"""Oracle: token-by-token gated delta rule (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path.

What it computes ("[1/4] GDN state/W QAT foundation", "What does this PR
do?": GatedDeltaNet training, exact recurrent reference, fla-core 0.5.1
conventions). The pages print no formula; the plainest reading of the
gated delta rule, per sequence and value head, from S = h0 (or 0):

    S   <- exp(g_t) * S                       (decay, g_t <= 0)
    u_t  = beta_t * (v_t - S^T k_t)           (delta-rule correction)
    S   <- S + k_t u_t^T                      (write)
    o_t  = scale * S^T q_t                    (read after the write)
    ht   = S after the last token

S is Dk x Dv. Grouped heads: value head h reads query/key head
h // (Hv // Hqk). Packed sequences (cu_seqlens) are independent, each with
its own h0/ht.

Optional state QDQ (reading of where the state site sits on the chunked
path, "[1/4]" "What does this PR do?"): before the first token of every
chunk of `chunk` tokens (sequence-relative), S <- QDQ(S) with one scale per
[Dk, block_v] tile, evaluated in FP32 on fl32(S). The final state is
returned without QDQ.

Optional two-precision read copy ("[5/8] ReplaySSM state QAT and
two-precision GDN", "What does this PR do?": an FP32 recurrence anchor and a
quantized copy used for reads, whose errors never overwrite the anchor),
chunk-path reading: at the first token of every chunk the read offset
E = S - QDQ_R(S) is taken (one scale per value column over all Dk key
channels) and decays with the state, so every read in the chunk (the
delta-rule prediction S^T k_t and the readout S^T q_t) sees S - a E, a the
decay since the chunk start, while the writes go to the anchor S itself.
"""
import numpy as np

from .qdq import FMT_OFF, qdq32


def _seq_bounds(T_total, B, cu_seqlens):
    if cu_seqlens is None:
        T = T_total // B
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = [int(x) for x in cu_seqlens]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def qdq_state64(S, fmt, block_v):
    """QDQ of a float64 [H, Dk, Dv] state: fl32, FP32 QDQ per [Dk, block_v]
    tile, back to float64."""
    H, Dk, Dv = S.shape
    x = S.astype(np.float32).reshape(H, Dk, Dv // block_v, block_v)
    out, _, _ = qdq32(x, fmt, tile_axes=(1, 3))
    return out.reshape(H, Dk, Dv).astype(np.float64)


def recurrent_fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None,
                  state_fmt=FMT_OFF, block_v=64, chunk=64, read_fmt=FMT_OFF):
    """q, k: [B, T, Hqk, Dk]; v: [B, T, Hv, Dv]; g, beta: [B, T, Hv].
    With cu_seqlens (length N+1) B must be 1 and T is the packed length.
    h0: [N, Hv, Dk, Dv] or None.  Returns (o [B, T, Hv, Dv], ht [N, Hv, Dk, Dv])
    in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, Hqk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    G = Hv // Hqk
    qf = np.repeat(q.reshape(B * T, Hqk, Dk), G, axis=1)   # [BT, Hv, Dk]
    kf = np.repeat(k.reshape(B * T, Hqk, Dk), G, axis=1)
    vf = v.reshape(B * T, Hv, Dv)
    gf = g.reshape(B * T, Hv)
    bf = beta.reshape(B * T, Hv)
    seqs = _seq_bounds(B * T, B, cu_seqlens)
    o = np.zeros((B * T, Hv, Dv))
    ht = np.zeros((len(seqs), Hv, Dk, Dv))
    for n, (bos, eos) in enumerate(seqs):
        S = np.zeros((Hv, Dk, Dv)) if h0 is None else np.array(h0[n], np.float64)
        E = np.zeros((Hv, Dk, Dv))                   # read offset (two-precision)
        a = np.ones(Hv)                              # its decay since the chunk start
        for t in range(bos, eos):
            if state_fmt != FMT_OFF and (t - bos) % chunk == 0:
                S = qdq_state64(S, state_fmt, block_v)
            if read_fmt != FMT_OFF and (t - bos) % chunk == 0:
                r, _, _ = qdq32(S.astype(np.float32), read_fmt, tile_axes=(1,))
                E = S - r.astype(np.float64)
                a = np.ones(Hv)
            S = np.exp(gf[t])[:, None, None] * S
            a = np.exp(gf[t]) * a
            u = bf[t][:, None] * (vf[t] - np.einsum('hkv,hk->hv', S - a[:, None, None] * E, kf[t]))
            S = S + kf[t][:, :, None] * u[:, None, :]
            o[t] = scale * np.einsum('hkv,hk->hv', S - a[:, None, None] * E, qf[t])
        ht[n] = S
    return o.reshape(B, T, Hv, Dv), ht
