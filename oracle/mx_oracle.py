"""fp64 CPU oracle for the MXFP8 jagged attention forward.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may use this module.  It shares no code with the HIP
library.  It decodes the FP8 formats by their definitions, dequantizes the
inputs, and computes the attention in float64 one (sequence, head) at a
time, with the softmax output quantized block by block as the method says.

Sources:
  [JFA]  "Optimizing Jagged Flash Attention with TLX: The Road Toward SOTA FA4
         on Blackwell", "Low-precision (MXFP8) attention": the two products
         of the forward take block-scaled FP8 operands (E4M3 elements, E8M0
         per-block scale factors), and the softmax output P is quantized to
         FP8 on the fly before its product with V.
  The formats are those of the OCP Microscaling (MX) specification, which
  the page's "MXFP8" names: an E4M3 element has a sign, 4 exponent bits
  (bias 7) and 3 mantissa bits, no infinities, and S.1111.111 as NaN (so the
  largest magnitude is 448); an E8M0 scale is the power of two 2^(c - 127)
  (c = 255: NaN); a block is 32 consecutive elements along the reduction
  dimension of a product, with one scale.  Quantizing a block of values x
  takes the scale X = 2^(floor(log2 max|x|) - 8) (8 = E4M3's largest
  exponent) and the element x / X rounded to the nearest E4M3 value, ties
  to the even code, saturating at +-448.

Readings where the page is silent (each also listed in the design notes):
  * Inputs arrive quantized: Q and K as E4M3 with one scale per 32
    consecutive head-dim elements of a row; V transposed, as E4M3
    [H_kv, d, T_pad] (T_pad = total_len rounded up to 64, columns past
    total_len zero) with one scale per 32 consecutive keys of the packed
    key index, [H_kv, T_pad / 32, d].  Key blocks follow the packed index:
    a block may hold keys of two sequences.
  * P is quantized per query row and per key block of that same packed
    index (32 keys; keys outside the row's visible set have P = 0).
  * The softmax statistics stay unquantized: l = sum of P, lse = log of the
    sum of exp(scores), and O = (quantized P) V / l.  So a one-key row gives
    O = v * q(P) / P, not v.
  * Which reference the exponentials are taken against does not matter as
    long as it is a whole power of two: E4M3's grid is closed under
    multiplication by powers of two (outside the subnormal and saturated
    ends, which the block scale keeps away from the block maximum), so the
    quantized block, times its scale, scales with the reference and the
    ratio O is unchanged.  This function uses the ceiling of the row's
    largest score in log2 units.
  * No sliding window; d = 128.

The backward (the same page says the variant covers both directions and
gives no more detail; readings, each also in the design notes):
  * Every product takes block-scaled FP8 operands blocked along its own
    reduction dimension, so each tensor arrives in the encodings its
    products need: Q, K, V and dO row-wise (blocks of 32 along d) for
    S = scale Q K^T and dP = dO V^T; Q and dO blocked along the query axis
    for dK = scale dS^T Q and dV = P^T dO; K blocked along the key axis for
    dQ = scale dS K.  The query-blocked encodings are transposed, with one
    scale per 32 queries of a head-dim column: broadcast Q^T [H, d, Lq_pad],
    scales [H, Lq_pad / 32, d], dO^T [B, H, d, Lq_pad], scales
    [B, H, Lq_pad / 32, d] (Lq_pad = Lq rounded up to 64, queries from 0);
    self mode Q^T and dO^T [H, d, T_pad], scales [H, T_pad / 32, d] (the
    packed token index, as for keys); K^T [H_kv, d, T_pad], scales
    [H_kv, T_pad / 32, d], the layout of the forward's V^T.  Padding
    columns are zero.
  * P = exp(S - lse) with the forward's lse; delta = rowsum(dO o O) with the
    row-wise dO and the forward's O as stored; dS = P o (dP - delta).  These
    stay unquantized; the operands they feed are quantized on the fly with
    the block rule of the forward: P and dS per key column in blocks of 32
    queries (the query axis's blocks above) for dV and dK, and dS per query
    row in blocks of 32 keys of the packed index for dQ.  The softmax scale
    multiplies the products' results, not dS.
  * The gradients are float32 sums; dK, dV of a key / value head sum over its
    query heads, and broadcast dQ over the sequences.

Layouts (numpy uint8 codes):
  broadcast: q8 [H, Lq, d], q_scale [H, Lq, d/32]; out [B, H, Lq, d],
             lse [B, H, Lq]; do8 [B, H, Lq, d], do_scale [B, H, Lq, d/32]
  self:      q8 [T, H, d], q_scale [T, H, d/32]; out [T, H, d], lse [T, H];
             do8 [T, H, d], do_scale [T, H, d/32]
  k8, v8 [T, H_kv, d], k_scale, v_scale [T, H_kv, d/32]
  vt8, kt8 [H_kv, d, T_pad], vt_scale, kt_scale [H_kv, T_pad/32, d]
  qt8, dot8 and their scales: as in the backward's readings above
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8
# A quantization decision counts as fragile when its input lies within this
# relative distance of a rounding boundary: a float32 computation of the same
# value (relative error near 1e-6) may land on the other side.
FRAGILE_REL = 2.0 ** -15
# Bound on a float32 score's error relative to the sum of the magnitudes of
# its products (sum over d of |q_d k_d|): the block-scaled matrix instruction
# accumulates the 128 exact products in float32 steps, up to 128 roundings.
SCORE_REL = 2.0 ** -17


def decode_e4m3(codes) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode_e8m0(codes) -> np.ndarray:
    """float64 values 2^(c - 127) of E8M0 codes (NaN for 255)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def _grid() -> np.ndarray:
    """The non-negative E4M3 values, in code order (increasing)."""
    return decode_e4m3(np.arange(127, dtype=np.uint8))


_GRID = _grid()
_MIDS = (_GRID[1:] + _GRID[:-1]) / 2.0


def quantize_e4m3(x) -> np.ndarray:
    """x rounded to the nearest E4M3 value, ties to the even code,
    saturating at +-448 (float64 in, float64 on the grid out)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_GRID, a, side="left"), 0, len(_GRID) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _GRID[lo]
    dhi = _GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    q = np.where(pick_hi, _GRID[hi], _GRID[lo])
    return np.copysign(q, x)


def block_scale_exponent(amax: float):
    """floor(log2 amax) - 8 for amax > 0: the block's scale is 2 to this."""
    return math.floor(math.log2(amax)) - E4M3_EMAX


def quantize_block(p: np.ndarray):
    """One MX block of non-negative values: (dequantized values, scale
    exponent or None for an all-zero block, dev).  dev[j] is how far element
    j's dequantized value can move if its input, or the block maximum, is
    off by a relative FRAGILE_REL (the other side of a rounding boundary or
    of a power of two): 0 where the decision is robust."""
    p = np.asarray(p, dtype=np.float64)
    amax = float(p.max()) if p.size else 0.0
    if amax == 0.0:
        return np.zeros_like(p), None, np.zeros_like(p)
    se = block_scale_exponent(amax)
    q = quantize_e4m3(p / 2.0 ** se) * 2.0 ** se
    dev = np.zeros_like(p)
    for f_max in (1.0 - FRAGILE_REL, 1.0, 1.0 + FRAGILE_REL):
        se_alt = block_scale_exponent(amax * f_max)
        for f in (1.0 - FRAGILE_REL, 1.0 + FRAGILE_REL):
            alt = quantize_e4m3(p * f / 2.0 ** se_alt) * 2.0 ** se_alt
            dev = np.maximum(dev, np.abs(alt - q))
    # inputs moved by FRAGILE_REL move robust outputs by at most that much too
    dev = np.where(dev <= 2.0 * FRAGILE_REL * np.abs(q), 0.0, dev)
    return q, se, dev


def dequantize_rows(x8, scale8) -> np.ndarray:
    """E4M3 codes [..., d] with E8M0 scales [..., d / 32] -> float64."""
    v = decode_e4m3(x8)
    s = decode_e8m0(scale8)
    return v * np.repeat(s, BLOCK, axis=-1)


def dequantize_vt(vt8, vt_scale, total_len: int) -> np.ndarray:
    """V from its transposed E4M3 codes [H_kv, d, T_pad] and key-block scales
    [H_kv, T_pad / 32, d] -> float64 [total_len, H_kv, d]."""
    v = decode_e4m3(vt8)                                       # [Hkv, d, Tp]
    s = np.repeat(decode_e8m0(vt_scale), BLOCK, axis=1)        # [Hkv, Tp, d]
    return (v.transpose(0, 2, 1) * s)[:, :total_len].transpose(1, 0, 2)


def sequence_forward(q, k, v, s0: int, scale: float, causal: bool):
    """One (sequence, head): q [n_q, d], k, v [L, d] float64 (dequantized),
    s0 = the sequence's first packed key index.  Returns (o [n_q, d],
    lse [n_q], allow [n_q, d]): allow bounds how far o can move when a
    fragile quantization decision (see quantize_block) goes the other way,
    sum over those keys of dev |v| / l; 0 where every decision is robust."""
    n_q, d = q.shape
    L = k.shape[0]
    o = np.zeros((n_q, d))
    lse = np.full(n_q, -np.inf)
    allow = np.zeros((n_q, d))
    if L == 0 or n_q == 0:
        return o, lse, allow
    x = (q @ k.T) * (scale / math.log(2.0))                  # scores in log2 units
    vis = np.ones((n_q, L), dtype=bool)
    if causal:
        vis = np.arange(L)[None, :] <= np.arange(n_q)[:, None]
    kabs = s0 + np.arange(L)
    blocks = kabs // BLOCK
    for i in range(n_q):
        cols = np.nonzero(vis[i])[0]
        if cols.size == 0:
            continue
        xi = x[i, cols]
        ref = math.ceil(float(xi.max()))
        p = np.exp2(xi - ref)
        l = float(p.sum())
        phat = np.zeros_like(p)
        dev = np.zeros_like(p)
        for b in np.unique(blocks[cols]):
            sel = blocks[cols] == b
            phat[sel], _, dev[sel] = quantize_block(p[sel])
        o[i] = (phat @ v[cols]) / l
        allow[i] = (dev @ np.abs(v[cols])) / l
        lse[i] = (ref + math.log2(l)) * math.log(2.0)
    return o, lse, allow


def jagged_forward(q8, q_scale, k8, k_scale, vt8, vt_scale, offsets, scale: float, causal: bool,
                   broadcast_q: bool, H_kv: int | None = None):
    """MXFP8 forward over a packed batch.  Returns (out, lse, allow) with
    out / lse in the bf16 path's layouts (float64) and allow of out's shape
    (see sequence_forward)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    B = len(offsets) - 1
    T = int(offsets[-1])
    Q = dequantize_rows(q8, q_scale)
    K = dequantize_rows(k8, k_scale)
    V = dequantize_vt(vt8, vt_scale, T)
    H = Q.shape[0] if broadcast_q else Q.shape[1]
    Hkv = K.shape[1] if H_kv is None else H_kv
    G = H // Hkv
    d = Q.shape[-1]
    if broadcast_q:
        Lq = Q.shape[1]
        out = np.zeros((B, H, Lq, d))
        lse = np.full((B, H, Lq), -np.inf)
    else:
        out = np.zeros((T, H, d))
        lse = np.full((T, H), -np.inf)
    frag = np.zeros_like(out)
    for b in range(B):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        for h in range(H):
            kk, vv = K[s0:s1, h // G], V[s0:s1, h // G]
            if broadcast_q:
                o, ls, fr = sequence_forward(Q[h], kk, vv, s0, scale, causal)
                out[b, h], lse[b, h], frag[b, h] = o, ls, fr
            else:
                o, ls, fr = sequence_forward(Q[s0:s1, h], kk, vv, s0, scale, causal)
                out[s0:s1, h], lse[s0:s1, h], frag[s0:s1, h] = o, ls, fr
    return out, lse, frag


# ---------------------------------------------------------------- backward

def _floor_log2(a):
    """floor(log2 a) for a > 0, exactly (from the binary exponent)."""
    _, e = np.frexp(a)
    return e.astype(np.float64) - 1.0


def quantize_along(x, pos, axis: int, eps=None):
    """MX quantization of a 2-D array along `axis`: the elements whose
    positions pos // 32 agree (pos: consecutive integers, one per index of
    that axis) form one block, per index of the other axis.  Each block takes
    the block rule of quantize_block.  Returns (q, dev): dev[i] bounds how
    far element i's dequantized value can move when every input element j of
    its block is off by up to eps[j] (default FRAGILE_REL |x|), through a
    rounding decision or the block's scale going the other way; 0 where no
    decision can flip."""
    x = np.asarray(x, dtype=np.float64)
    eps = FRAGILE_REL * np.abs(x) if eps is None else np.asarray(eps, dtype=np.float64)
    if axis == 0:
        q, dev = quantize_along(x.T, pos, 1, eps.T)
        return q.T, dev.T
    R, n = x.shape
    pos = np.asarray(pos, dtype=np.int64)
    if n == 0:
        return np.zeros_like(x), np.zeros_like(x)
    first = int(pos[0]) // BLOCK
    blk = pos // BLOCK - first
    slot = pos % BLOCK
    nb = int(blk[-1]) + 1
    xb = np.zeros((R, nb, BLOCK))
    eb = np.zeros((R, nb, BLOCK))
    xb[:, blk, slot] = x
    eb[:, blk, slot] = eps
    amax = np.abs(xb).max(axis=-1, keepdims=True)
    live = amax > 0
    se = np.where(live, _floor_log2(np.where(live, amax, 1.0)) - E4M3_EMAX, 0.0)
    qb = np.where(live, quantize_e4m3(xb * np.exp2(-se)) * np.exp2(se), 0.0)
    E = eb.max(axis=-1, keepdims=True)
    dev = np.zeros_like(xb)
    sgn = np.sign(xb)
    for a_alt in (amax - E, amax, amax + E):
        ok = a_alt > 0
        se_alt = np.where(ok, _floor_log2(np.where(ok, a_alt, 1.0)) - E4M3_EMAX, se)
        for s in (-1.0, 1.0):
            xa = xb + s * eb * sgn
            alt = quantize_e4m3(xa * np.exp2(-se_alt)) * np.exp2(se_alt)
            dev = np.maximum(dev, np.abs(alt - qb))
    dev = np.where((dev <= 2.0 * eb) | ~live, 0.0, dev)
    return qb[:, blk, slot], dev[:, blk, slot]


def dequantize_cols(x8, scale8, n: int, p0: int = 0) -> np.ndarray:
    """Positions p0 .. p0 + n - 1 of transposed E4M3 codes [..., d, n_pad]
    with scales per 32 positions of the last axis, [..., n_pad / 32, d]
    -> float64 [..., n, d]."""
    pos = np.arange(p0, p0 + n)
    v = decode_e4m3(np.asarray(x8)[..., p0:p0 + n])
    s = decode_e8m0(np.asarray(scale8)[..., pos // BLOCK, :])
    return np.swapaxes(v, -1, -2) * s


def sequence_backward(qr, qc, kr, kc, vr, dor, doc, o, lse, qpos, kpos, scale: float, causal: bool):
    """One (sequence, head) of the MXFP8 backward, float64.

    qr, dor [n_q, d], kr, vr [L, d]: row-wise dequantized Q, dO, K, V; qc,
    doc [n_q, d]: Q and dO from their query-blocked encodings; kc [L, d]: K
    from its key-blocked encoding; o [n_q, d] and lse [n_q]: the forward's
    output (as stored) and log-sum-exp; qpos [n_q], kpos [L]: the positions
    whose // 32 gives each query's and key's block.

    Returns (dq, dk, dv, allow_dq, allow_dk, allow_dv): the gradients and, per
    element, the bound of quantize_along's dev carried through each product
    (0 where every decision is robust).  The input error bounds of a float32
    computation: P within (FRAGILE_REL + |scale| SCORE_REL |q| |k|) of itself
    (the score's error moves exp by that much, relatively); dS within that
    error times |dP - delta| plus FRAGILE_REL P (|dO| |V|^T + |dO| |O|) (the
    float32 sums of dP and delta)."""
    qr, qc, kr, kc, vr, dor, doc, o = (np.asarray(x, dtype=np.float64) for x in (qr, qc, kr, kc, vr, dor, doc, o))
    lse = np.asarray(lse, dtype=np.float64)
    n_q, L = qr.shape[0], kr.shape[0]
    if n_q == 0 or L == 0:
        z = lambda r, c: np.zeros((r, c))
        return z(n_q, qc.shape[1]), z(L, qc.shape[1]), z(L, doc.shape[1]), \
            z(n_q, qc.shape[1]), z(L, qc.shape[1]), z(L, doc.shape[1])
    s = scale * (qr @ kr.T)
    vis = np.ones((n_q, L), dtype=bool)
    if causal:
        vis = np.arange(L)[None, :] <= np.arange(n_q)[:, None]
    vis = vis & np.isfinite(lse)[:, None]
    p = np.where(vis, np.exp(np.where(vis, s - np.where(np.isfinite(lse), lse, 0.0)[:, None], 0.0)), 0.0)
    dp = dor @ vr.T
    delta = (dor * o).sum(axis=1)
    ds = p * (dp - delta[:, None])
    eps_p = p * (FRAGILE_REL + abs(scale) * SCORE_REL * (np.abs(qr) @ np.abs(kr).T))
    eps_ds = eps_p * np.abs(dp - delta[:, None]) \
        + FRAGILE_REL * p * (np.abs(dor) @ np.abs(vr).T + (np.abs(dor) * np.abs(o)).sum(axis=1)[:, None])
    pq, dev_p = quantize_along(p, qpos, 0, eps_p)
    dsq, dev_q = quantize_along(ds, qpos, 0, eps_ds)
    dsk, dev_k = quantize_along(ds, kpos, 1, eps_ds)
    a = abs(scale)
    dv = pq.T @ doc
    dk = scale * (dsq.T @ qc)
    dq = scale * (dsk @ kc)
    return dq, dk, dv, a * (dev_k @ np.abs(kc)), a * (dev_q.T @ np.abs(qc)), dev_p.T @ np.abs(doc)


def dequantize_backward_inputs(t: dict, broadcast_q: bool):
    """float64 views of every encoding of an MXFP8 backward input set (numpy
    codes under the layout names of this module's header): Qr, Qc, Kr, Kc,
    Vr, dOr, dOc in the row layouts of q8, k8 and do8."""
    T = int(np.asarray(t["offsets"])[-1])
    Qr = dequantize_rows(t["q8"], t["q_scale"])
    Kr = dequantize_rows(t["k8"], t["k_scale"])
    Vr = dequantize_rows(t["v8"], t["v_scale"])
    dOr = dequantize_rows(t["do8"], t["do_scale"])
    Kc = np.swapaxes(dequantize_cols(t["kt8"], t["kt_scale"], T), 0, 1)          # [T, H_kv, d]
    if broadcast_q:
        Lq = Qr.shape[1]
        Qc = dequantize_cols(t["qt8"], t["qt_scale"], Lq)                      # [H, Lq, d]
        dOc = dequantize_cols(t["dot8"], t["dot_scale"], Lq)                   # [B, H, Lq, d]
    else:
        Qc = np.swapaxes(dequantize_cols(t["qt8"], t["qt_scale"], T), 0, 1)      # [T, H, d]
        dOc = np.swapaxes(dequantize_cols(t["dot8"], t["dot_scale"], T), 0, 1)   # [T, H, d]
    return Qr, Qc, Kr, Kc, Vr, dOr, dOc


def backward_item(t: dict, deq, out, lse, b: int, h: int, scale: float, causal: bool, broadcast_q: bool):
    """sequence_backward of sequence b and query head h of a packed batch
    (deq: dequantize_backward_inputs(t); out, lse: the forward's)."""
    Qr, Qc, Kr, Kc, Vr, dOr, dOc = deq
    off = np.asarray(t["offsets"], dtype=np.int64)
    s0, s1 = int(off[b]), int(off[b + 1])
    H = Qr.shape[0] if broadcast_q else Qr.shape[1]
    hk = h // (H // Kr.shape[1])
    kpos = np.arange(s0, s1)
    if broadcast_q:
        Lq = Qr.shape[1]
        return sequence_backward(Qr[h], Qc[h], Kr[s0:s1, hk], Kc[s0:s1, hk], Vr[s0:s1, hk], dOr[b, h], dOc[b, h],
                                 out[b, h], lse[b, h], np.arange(Lq), kpos, scale, causal)
    return sequence_backward(Qr[s0:s1, h], Qc[s0:s1, h], Kr[s0:s1, hk], Kc[s0:s1, hk], Vr[s0:s1, hk],
                             dOr[s0:s1, h], dOc[s0:s1, h], out[s0:s1, h], lse[s0:s1, h], kpos, kpos, scale,
                             causal)


def jagged_backward(t: dict, out, lse, scale: float, causal: bool, broadcast_q: bool):
    """MXFP8 backward over a packed batch.  t: numpy codes of every encoding
    (q8, q_scale, qt8, qt_scale, k8, k_scale, kt8, kt_scale, v8, v_scale,
    do8, do_scale, dot8, dot_scale) and offsets; out, lse: the forward's.
    Returns (dq, dk, dv, allow_dq, allow_dk, allow_dv), dq in q8's layout
    (broadcast: summed over the sequences), dk / dv [T, H_kv, d] summed over
    each group's query heads."""
    deq = dequantize_backward_inputs(t, broadcast_q)
    Qr, Kr = deq[0], deq[2]
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    off = np.asarray(t["offsets"], dtype=np.int64)
    H = Qr.shape[0] if broadcast_q else Qr.shape[1]
    G = H // Kr.shape[1]
    dq, adq = np.zeros_like(Qr), np.zeros_like(Qr)
    dk, adk = np.zeros_like(Kr), np.zeros_like(Kr)
    dv, adv = np.zeros_like(Kr), np.zeros_like(Kr)
    for b in range(len(off) - 1):
        s0, s1 = int(off[b]), int(off[b + 1])
        for h in range(H):
            g = backward_item(t, deq, out, lse, b, h, scale, causal, broadcast_q)
            if broadcast_q:
                dq[h] += g[0]
                adq[h] += g[3]
            else:
                dq[s0:s1, h] = g[0]
                adq[s0:s1, h] = g[3]
            dk[s0:s1, h // G] += g[1]
            dv[s0:s1, h // G] += g[2]
            adk[s0:s1, h // G] += g[4]
            adv[s0:s1, h // G] += g[5]
    return dq, dk, dv, adq, adk, adv
