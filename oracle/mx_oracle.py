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

Layouts (numpy uint8 codes):
  broadcast: q8 [H, Lq, d], q_scale [H, Lq, d/32]; out [B, H, Lq, d],
             lse [B, H, Lq]
  self:      q8 [T, H, d], q_scale [T, H, d/32]; out [T, H, d], lse [T, H]
  k8 [T, H_kv, d], k_scale [T, H_kv, d/32]
  vt8 [H_kv, d, T_pad], vt_scale [H_kv, T_pad/32, d]
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
