"""fp64 CPU oracle for jagged (padding-free) attention, forward and backward.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module.  It shares no code with the HIP
library: no kernels, headers, helpers or constants.  Everything here is the
plain textbook definition, written out in float64 with numpy, one
(sequence, head) at a time, materialising each score matrix.

Sources (cited by page title and section):
  [FMHA]  "cuTile Kernels -- FMHA Implementation": "Attention Basics" (the
          definition softmax(Q K^T * scale) V and the causal mask that sets
          future scores to -inf), "Flash Attention Algorithm" and "Kernel
          Pseudocode" (the online-softmax recurrence), "cuTile Implementation"
          (the causal tile bound Tc / mask_start and the rule offs_m >= offs_n).
  [JFA]   "Optimizing Jagged Flash Attention with TLX: The Road Toward SOTA
          FA4 on Blackwell": "Introduction" (sequences packed contiguously,
          boundaries in an offsets tensor, no padded tokens), "1. The
          Challenge" (broadcast-Q: one dense Q for every sequence, so dQ is the
          sum over the whole batch), "Loop peeling" (bulk pass to
          aligned = (klen // BLOCK_N) * BLOCK_N, then a masked tail).

Readings where the pages are silent (each also listed in the design notes):
  * lse is the natural-log log-sum-exp of the scaled, masked scores.
  * A sequence with no keys gives O = 0 and lse = -inf, and contributes no
    gradient.
  * Causal positions are local to a sequence and top-left aligned: query i
    sees keys j <= i (also when, in broadcast mode, Lq differs from L_b).
  * The backward is the exact derivative of the forward: dP = dO V^T,
    delta_i = sum_d dO_id O_id, dS = P o (dP - delta), dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO.  The pages do not print it.
  * Sliding window ([JFA] "3. Attention Variants: the flexibility of TLX",
    block-sparse part, and "Conclusion" name windowing support without a
    rule): with the causal mask and a window of W keys, query i sees keys j
    with i - W < j <= i (W <= 0: no window).  A query row that sees no key
    (possible in broadcast mode when i - W >= L) gives O = 0, lse = -inf and
    no gradient, like a sequence with no keys.
  * Grouped-query attention ([JFA] "3. Attention Variants: the flexibility
    of TLX", block-sparse part, and "Conclusion" name GQA support without
    defining it): with H query heads and H_kv = H / G key/value heads, query
    head h attends with key/value head h // G (consecutive query heads share
    one), so that head's dK and dV are the sums over its G query heads.

Layouts (numpy arrays, any float dtype; converted to float64 on entry):
  k, v         [T, H_kv, d], T = offsets[-1]; H_kv divides H (H_kv = H: plain
               multi-head attention)
  broadcast:   q [H, Lq, d]; out, dout [B, H, Lq, d]; lse [B, H, Lq];
               dq [H, Lq, d] (sum over sequences)
  self:        q, out, dout, dq [T, H, d]; lse [T, H]
  dk, dv       [T, H_kv, d]
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def causal_visible(n_q: int, n_k: int, window: int = 0) -> np.ndarray:
    """Boolean [n_q, n_k]: True where query i may see key j, i.e. j <= i
    ([FMHA] "cuTile Implementation": keep a score where offs_m >= offs_n),
    and, with a window of W > 0 keys, j > i - W."""
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    vis = j <= i
    if window > 0:
        vis = vis & (j > i - window)
    return vis


def sequence_scores(qb, kb, scale: float, causal: bool, window: int = 0) -> np.ndarray:
    """S = scale * Q K^T, future scores (and, with a window, scores of keys
    W or more positions back) set to -inf when causal ([FMHA] "Attention
    Basics")."""
    s = scale * (_f64(qb) @ _f64(kb).T)
    if causal:
        s = np.where(causal_visible(s.shape[0], s.shape[1], window), s, -np.inf)
    return s


def sequence_forward(qb, kb, vb, scale: float, causal: bool, window: int = 0):
    """One (sequence, head): returns (O [n,d], lse [n], P [n,L]).

    P = softmax(S) row-wise with the row maximum subtracted first; O = P V;
    lse = m + ln(sum_j exp(S_ij - m)) ([FMHA] "Attention Basics").
    """
    qb, kb, vb = _f64(qb), _f64(kb), _f64(vb)
    n, d = qb.shape
    L = kb.shape[0]
    if L == 0:
        return np.zeros((n, vb.shape[1])), np.full(n, -np.inf), np.zeros((n, 0))
    s = sequence_scores(qb, kb, scale, causal, window)
    m = s.max(axis=1)
    seen = np.isfinite(m)  # rows that see at least one key
    e = np.exp(s - np.where(seen, m, 0.0)[:, None])
    l = e.sum(axis=1)
    p = e / np.where(seen, l, 1.0)[:, None]
    lse = np.where(seen, np.where(seen, m, 0.0) + np.log(np.where(seen, l, 1.0)), -np.inf)
    return p @ vb, lse, p


def sequence_backward(qb, kb, vb, dob, scale: float, causal: bool, window: int = 0):
    """One (sequence, head): returns (dQ [n,d], dK [L,d], dV [L,d]).

    The derivative of O = softmax(scale Q K^T) V: with P and O recomputed by
    sequence_forward, dP = dO V^T, delta = rowsum(dO o O), dS = P o (dP -
    delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
    """
    qb, kb, vb, dob = _f64(qb), _f64(kb), _f64(vb), _f64(dob)
    L = kb.shape[0]
    if L == 0:
        return np.zeros_like(qb), np.zeros((0, qb.shape[1])), np.zeros((0, vb.shape[1]))
    o, _, p = sequence_forward(qb, kb, vb, scale, causal, window)
    delta = (dob * o).sum(axis=1)
    dp = dob @ vb.T
    ds = p * (dp - delta[:, None])
    return scale * (ds @ kb), scale * (ds.T @ qb), p.T @ dob


def _group(H: int, H_kv: int) -> int:
    """Query heads per key/value head."""
    if H_kv < 1 or H % H_kv:
        raise ValueError(f"{H} query heads do not split into groups over {H_kv} key/value heads")
    return H // H_kv


def _seq_bounds(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return [(int(off[b]), int(off[b + 1])) for b in range(off.size - 1)]


def jagged_forward(q, k, v, offsets, scale: float, causal: bool, broadcast_q: bool, window: int = 0):
    """Forward over a packed batch ([JFA] "Introduction": sequence b owns the
    packed rows offsets[b]..offsets[b+1]-1 of K and V; in self mode also of
    Q; [JFA] "1. The Challenge": in broadcast mode every sequence attends
    with the same dense Q)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bounds = _seq_bounds(offsets)
    B = len(bounds)
    H = q.shape[0] if broadcast_q else q.shape[1]
    G = _group(H, k.shape[1])
    if broadcast_q:
        Lq = q.shape[1]
        out = np.zeros((B, H, Lq, v.shape[2]))
        lse = np.zeros((B, H, Lq))
    else:
        out = np.zeros((q.shape[0], H, v.shape[2]))
        lse = np.zeros((q.shape[0], H))
    for b, (s0, s1) in enumerate(bounds):
        for h in range(H):
            qb = q[h] if broadcast_q else q[s0:s1, h]
            o, ls, _ = sequence_forward(qb, k[s0:s1, h // G], v[s0:s1, h // G], scale, causal, window)
            if broadcast_q:
                out[b, h], lse[b, h] = o, ls
            else:
                out[s0:s1, h], lse[s0:s1, h] = o, ls
    return out, lse


def jagged_backward(q, k, v, offsets, scale: float, causal: bool, broadcast_q: bool, dout, window: int = 0):
    """Backward over a packed batch.  In broadcast mode dQ is the sum of the
    per-sequence dQ over the whole batch ([JFA] "1. The Challenge")."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    bounds = _seq_bounds(offsets)
    H = q.shape[0] if broadcast_q else q.shape[1]
    G = _group(H, k.shape[1])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b, (s0, s1) in enumerate(bounds):
        for h in range(H):
            kb, vb = k[s0:s1, h // G], v[s0:s1, h // G]
            if broadcast_q:
                g = sequence_backward(q[h], kb, vb, dout[b, h], scale, causal, window)
                dq[h] += g[0]
            else:
                g = sequence_backward(q[s0:s1, h], kb, vb, dout[s0:s1, h], scale, causal, window)
                dq[s0:s1, h] = g[0]
            dk[s0:s1, h // G] += g[1]
            dv[s0:s1, h // G] += g[2]
    return dq, dk, dv


def broadcast_dq_rows(q, k, v, offsets, scale: float, causal: bool, dout, rows):
    """dQ[h, i, :] for the listed (h, i) pairs in broadcast mode, one query
    row at a time.  Every quantity on a row of the definition depends only
    on that row: p = softmax row i of sequence b, o = p V_b, delta = dO_b[i].o,
    ds = p o (dO_b[i] V_b^T - delta), dQ[h,i] = scale * sum_b ds K_b."""
    out = []
    bounds = _seq_bounds(offsets)
    G = _group(q.shape[0], k.shape[1])
    for (h, i) in rows:
        qi = _f64(q[h, i:i + 1])
        acc = np.zeros(q.shape[2])
        for b, (s0, s1) in enumerate(bounds):
            if s1 == s0:
                continue
            kb, vb = _f64(k[s0:s1, h // G]), _f64(v[s0:s1, h // G])
            s = scale * (qi @ kb.T)[0]
            if causal:
                s = np.where(np.arange(s1 - s0) <= i, s, -np.inf)
            e = np.exp(s - s.max())
            p = e / e.sum()
            o = p @ vb
            do = _f64(dout[b, h, i])
            ds = p * (vb @ do - do @ o)
            acc += scale * (ds @ kb)
        out.append(acc)
    return np.array(out)


def online_forward_sequence(qb, kb, vb, scale: float, causal: bool, BM: int, BN: int):
    """The tiled online-softmax recurrence of [FMHA] "Flash Attention
    Algorithm" / "Kernel Pseudocode", in float64, for one (sequence, head).

    Queries are cut into tiles of BM rows.  For each query tile a running
    maximum m (-inf), running sum l (0) and accumulator acc (0) are carried
    across key tiles of BN keys: m_new = max(m, rowmax(S_tile)), correction =
    exp(m - m_new), l = l*correction + rowsum(exp(S_tile - m_new)), acc =
    acc*correction + exp(S_tile - m_new) V_tile, m = m_new; finally O =
    acc / l.  With a causal mask the key loop stops after tile
    Tc = cdiv(min((bid+1)*BM, L), BN) and only tiles from mask_start =
    (bid*BM)//BN on are masked ([FMHA] "cuTile Implementation").  Otherwise the
    loop is peeled: unmasked tiles up to aligned = (L//BN)*BN, then at most
    one masked tail tile ([JFA] "Loop peeling").  Returns (O, lse).
    """
    qb, kb, vb = _f64(qb), _f64(kb), _f64(vb)
    n, L = qb.shape[0], kb.shape[0]
    out = np.zeros((n, vb.shape[1]))
    lse = np.full(n, -np.inf)
    if L == 0:
        return out, lse
    for bid in range((n + BM - 1) // BM):
        r0, r1 = bid * BM, min(n, (bid + 1) * BM)
        rows = np.arange(r0, r1)
        m = np.full(r1 - r0, -np.inf)
        l = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, vb.shape[1]))
        if causal:
            Tc = -(-min((bid + 1) * BM, L) // BN)
            mask_start = (bid * BM) // BN
        else:
            Tc = -(-L // BN)
            mask_start = L // BN  # == aligned // BN: only the partial tail is masked
        for j in range(Tc):
            c0, c1 = j * BN, min(L, (j + 1) * BN)
            s = scale * (qb[r0:r1] @ kb[c0:c1].T)
            if j >= mask_start:
                cols = np.arange(c0, c1)
                keep = cols[None, :] < L
                if causal:
                    keep = keep & (rows[:, None] >= cols[None, :])
                s = np.where(keep, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            corr = np.exp(m - m_new)
            p = np.exp(s - m_new[:, None])
            l = l * corr + p.sum(axis=1)
            acc = acc * corr[:, None] + p @ vb[c0:c1]
            m = m_new
        out[r0:r1] = acc / l[:, None]
        lse[r0:r1] = m + np.log(l)
    return out, lse
