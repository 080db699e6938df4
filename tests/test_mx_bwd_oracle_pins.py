"""Pins of the MXFP8 backward oracle (oracle/mx_oracle.py, sequence_backward
and what it calls) against things other than itself: the already pinned
per-block rule, the plain gradient where quantization is switched off, closed
forms, which encoding each product reads, where the blocks fall, the E4M3
format's error bound and power-of-two invariance."""
from __future__ import annotations

import math

import numpy as np
import pytest

import workloads as wl
from oracle import jfa_oracle as jo
from oracle import mx_oracle as mo


def _rng(seed):
    return np.random.default_rng(seed)


def test_quantize_along_matches_the_block_rule():
    """Each block of quantize_along is quantize_block of its elements, with
    blocks cut at multiples of 32 of the given positions, along either axis."""
    rng = _rng(1)
    for trial in range(30):
        R, n = int(rng.integers(1, 5)), int(rng.integers(1, 130))
        p0 = int(rng.integers(0, 200))
        pos = np.arange(p0, p0 + n)
        x = rng.standard_normal((R, n)) * 2.0 ** rng.integers(-12, 4, (R, n))
        x[rng.uniform(size=(R, n)) < 0.1] = 0.0
        if trial % 3 == 0:
            x = np.abs(x)
        q, dev = mo.quantize_along(x, pos, 1)
        qt, devt = mo.quantize_along(x.T, pos, 0)
        assert np.array_equal(qt.T, q) and np.array_equal(devt.T, dev)
        for r in range(R):
            for b in np.unique(pos // 32):
                sel = pos // 32 == b
                qb, _, db = mo.quantize_block(np.abs(x[r, sel]))
                assert np.array_equal(np.abs(q[r, sel]), qb)
                assert np.array_equal(np.sign(q[r, sel]) * np.sign(x[r, sel]) >= 0, np.ones(sel.sum(), bool))
                assert np.array_equal(dev[r, sel], db)


def test_quantize_along_fragile_closed_forms():
    # amax 1.9 sets the scale 2^-8; 1.0625 is the midpoint of 1 and 1.125
    q, dev = mo.quantize_along(np.array([[1.9, 1.0625, -1.0625]]), np.arange(3), 1)
    assert np.array_equal(q[0], [1.75, 1.0, -1.0]) and np.array_equal(dev[0], [0.0, 0.125, 0.125])
    # an absolute error bound larger than the distance to the midpoint flips it
    q, dev = mo.quantize_along(np.array([[1.9, 1.1]]), np.arange(2), 1, eps=np.array([[0.0, 0.04]]))
    assert q[0, 1] == 1.125 and dev[0, 1] == 0.125
    q, dev = mo.quantize_along(np.array([[1.9, 1.1]]), np.arange(2), 1, eps=np.array([[0.0, 0.01]]))
    assert not dev.any()
    # a block maximum just below a power of two: the scale could be the next
    # one up, where 2 - 2^-20 no longer saturates (1.75 -> 2)
    q, dev = mo.quantize_along(np.array([[2.0 * (1 - 2.0 ** -20), 0.3]]), np.arange(2), 1)
    assert q[0, 0] == 1.75 and dev[0, 0] == 0.25
    # an all-zero block
    q, dev = mo.quantize_along(np.zeros((2, 40)), np.arange(40), 1)
    assert not q.any() and not dev.any()


def _plain_case(rng, n_q, L, d=128, causal=False):
    q, k, v, do = (rng.standard_normal(s) for s in ((n_q, d), (L, d), (L, d), (n_q, d)))
    return q, k, v, do


def _identity_quantizer(x, pos, axis, eps=None):
    x = np.asarray(x, dtype=np.float64)
    return x.copy(), np.zeros_like(x)


@pytest.mark.parametrize("causal", [False, True])
def test_unquantized_backward_is_the_plain_gradient(causal, monkeypatch):
    """With the on-the-fly quantization switched off and one value per
    tensor in every encoding, the backward is the textbook gradient (the
    plain oracle's, itself pinned to torch autograd), given the exact O and
    lse."""
    monkeypatch.setattr(mo, "quantize_along", _identity_quantizer)
    rng = _rng(2)
    for n_q, L, scale in ((37, 37, 0.09), (64, 100, -0.2), (5, 70, 0.3)):
        q, k, v, do = _plain_case(rng, n_q, L)
        o, lse, _ = jo.sequence_forward(q, k, v, scale, causal, 0)
        dq, dk, dv, aq, ak, av = mo.sequence_backward(q, q, k, k, v, do, do, o, lse, np.arange(n_q),
                                                      np.arange(L) + 3, scale, causal)
        rq, rk, rv = jo.sequence_backward(q, k, v, do, scale, causal, 0)
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))
        assert not (aq.any() or ak.any() or av.any())


def test_each_product_reads_its_own_encoding():
    """dQ reads the key-blocked K (and nothing else query- or key-blocked),
    dK the query-blocked Q, dV the query-blocked dO; the row-wise encodings
    feed S, dP and delta, hence everything."""
    rng = _rng(3)
    n_q, L, scale = 40, 70, 0.1
    qr, kr, vr, dor = _plain_case(rng, n_q, L)
    qc, kc, doc = (x + 0.05 * rng.standard_normal(x.shape) for x in (qr, kr, dor))
    o, lse, _ = jo.sequence_forward(qr, kr, vr, scale, False, 0)
    o = o + 0.01 * rng.standard_normal(o.shape)
    args = dict(qr=qr, qc=qc, kr=kr, kc=kc, vr=vr, dor=dor, doc=doc, o=o)

    def run(**over):
        a = dict(args, **over)
        return mo.sequence_backward(a["qr"], a["qc"], a["kr"], a["kc"], a["vr"], a["dor"], a["doc"], a["o"], lse,
                                    np.arange(n_q), np.arange(L), scale, False)[:3]

    base = run()
    for name, touched in (("qc", {1}), ("kc", {0}), ("doc", {2}), ("qr", {0, 1, 2}), ("kr", {0, 1, 2}),
                          ("vr", {0, 1}), ("dor", {0, 1}), ("o", {0, 1})):
        alt = run(**{name: args[name] * 2.0 ** 0.5})
        for i in range(3):
            same = np.array_equal(alt[i], base[i])
            assert same == (i not in touched), (name, "dq dk dv".split()[i])
    # and dK is linear in the query-blocked Q given the rest (powers of two
    # keep every quantized operand as it was)
    two = run(qc=2 * qc)
    np.testing.assert_array_equal(two[1], 2 * base[1])


def test_single_key_closed_form():
    """One query, one key, lse = the score: P = 1 (exact in E4M3), dV = the
    query-blocked dO row, and dS = dO.v - dO.o = 0 with O = v."""
    rng = _rng(4)
    for _ in range(10):
        q, k, v, do = _plain_case(rng, 1, 1)
        doc = do * 0.75
        s = 0.3 * float(q[0] @ k[0])
        dq, dk, dv, *_ = mo.sequence_backward(q, q, k, k, v, do, doc, v.copy(), np.array([s]), [0], [0], 0.3, False)
        np.testing.assert_array_equal(dv, doc)
        assert np.abs(dk).max() < 1e-12 and np.abs(dq).max() < 1e-12


def _e4m3_rel(x):
    """A lone positive value under the block rule: 3 fraction bits, nearest
    (ties to even), 1.75 times the power of two at most."""
    e = math.floor(math.log2(x))
    m = x / 2.0 ** e
    f = round(m * 8)  # Python's round: ties to even
    return min(f / 8, 1.75) * 2.0 ** e


def test_two_keys_closed_form():
    """One query, two keys: each key column's block holds one query, so
    dV[j] = q(P_j) dO with q the lone-value rule, whatever the other key."""
    rng = _rng(5)
    for _ in range(20):
        q, k, v, do = _plain_case(rng, 1, 2)
        scale = 0.2
        s = scale * (q @ k.T)[0]
        lse = float(np.log(np.exp(s).sum()))
        p = np.exp(s - lse)
        o = p @ v
        _, _, dv, *_ = mo.sequence_backward(q, q, k, k, v, do, do, o[None], np.array([lse]), [0], [5, 6], scale,
                                            False)
        for j in range(2):
            np.testing.assert_allclose(dv[j], _e4m3_rel(p[j]) * do[0], rtol=1e-14, atol=0)


def _column_case(p_col, qpos):
    """One key whose column of P over the queries is p_col (through lse),
    score 0, and one-hot query-blocked dO rows: dV's first entries are then
    the quantized column."""
    n_q, d = len(p_col), 128
    q = np.zeros((n_q, d))
    k = np.zeros((1, d))
    v = np.zeros((1, d))
    lse = -np.log(p_col)
    do = np.zeros((n_q, d))
    doc = np.eye(n_q, d)
    o = np.zeros((n_q, d))
    _, _, dv, *_ = mo.sequence_backward(q, q, k, k, v, do, doc, o, lse, qpos, [0], 1.0, False)
    return dv[0, :n_q]


def test_p_blocks_follow_the_query_axis():
    """P is quantized per key column in blocks of 32 queries.  A small value
    beside 1.0 in its block sits on the coarse grid (2^-17 steps); beside only
    small values it keeps three fraction bits."""
    small = 1.3 * 2.0 ** -17
    p = np.array([1.0, small, small, 2.0 ** -17])
    # self mode: packed positions 30..33 straddle two blocks
    got = _column_case(p, np.arange(30, 34))
    np.testing.assert_allclose(got, [1.0, 2.0 ** -17, 1.25 * 2.0 ** -17, 2.0 ** -17], rtol=1e-12)
    # one block
    got = _column_case(p, np.arange(0, 4))
    np.testing.assert_allclose(got, [1.0, 2.0 ** -17, 2.0 ** -17, 2.0 ** -17], rtol=1e-12)


def test_jagged_query_blocks_by_mode():
    """In broadcast mode the query blocks start at query 0 for every
    sequence; in self mode they follow the packed index."""
    t = _mx_case([30, 40], 1, 1, 8, True, seed=6)
    a, out, lse = t
    deq = mo.dequantize_backward_inputs(a, True)
    g_b1 = mo.backward_item(a, deq, out, lse, 1, 0, 0.1, False, True)
    Qr, Qc, Kr, Kc, Vr, dOr, dOc = deq
    ref = mo.sequence_backward(Qr[0], Qc[0], Kr[30:70, 0], Kc[30:70, 0], Vr[30:70, 0], dOr[1, 0], dOc[1, 0],
                               out[1, 0], lse[1, 0], np.arange(8), np.arange(30, 70), 0.1, False)
    for x, y in zip(g_b1, ref):
        np.testing.assert_array_equal(x, y)
    a, out, lse = _mx_case([30, 40], 1, 1, 0, False, seed=7)
    deq = mo.dequantize_backward_inputs(a, False)
    g = mo.backward_item(a, deq, out, lse, 1, 0, 0.1, False, False)
    Qr, Qc, Kr, Kc, Vr, dOr, dOc = deq
    sl = slice(30, 70)
    ref = mo.sequence_backward(Qr[sl, 0], Qc[sl, 0], Kr[sl, 0], Kc[sl, 0], Vr[sl, 0], dOr[sl, 0], dOc[sl, 0],
                               out[sl, 0], lse[sl, 0], np.arange(30, 70), np.arange(30, 70), 0.1, False)
    for x, y in zip(g, ref):
        np.testing.assert_array_equal(x, y)


def test_ds_blocks_follow_the_key_axis():
    """dS is quantized per query row in blocks of 32 keys for dQ: one query,
    keys at packed positions 30..33 with dS = (1, small, small, 2^-17) through
    dP (delta = 0), one-hot key-blocked K."""
    d = 128
    small = 1.3 * 2.0 ** -17
    target = np.array([1.0, small, small, 2.0 ** -17])
    L = 4
    q = np.zeros((1, d))
    k = np.zeros((L, d))
    lse = np.array([0.0])          # P = exp(0 - 0) = 1 on every key
    v = np.zeros((L, d))
    v[:, 0] = target               # dP = dO v^T = target with dO = e0
    do = np.zeros((1, d))
    do[0, 0] = 1.0
    o = np.zeros((1, d))           # delta = 0
    kc = np.eye(L, d)
    for kp, want in ((np.arange(30, 34), [1.0, 2.0 ** -17, 1.25 * 2.0 ** -17, 2.0 ** -17]),
                     (np.arange(0, 4), [1.0, 2.0 ** -17, 2.0 ** -17, 2.0 ** -17])):
        dq, *_ = mo.sequence_backward(q, q, k, kc, v, do, do, o, lse, [0], kp, 1.0, False)
        np.testing.assert_allclose(dq[0, :L], want, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_within_the_format_error_of_the_plain_gradient(causal):
    """Every quantized P or dS element is within 2^-3 of itself plus 2^-17 of
    its block's largest magnitude of the exact value (three fraction bits,
    saturation at 1.75 times the top power of two, subnormal steps), so each
    gradient is within that much, carried through its product, of the
    unquantized one; and quantization does change it."""
    rng = _rng(8)
    n_q, L, scale = 50, 90, 0.15
    q, k, v, do = _plain_case(rng, n_q, L)
    o, lse, p = jo.sequence_forward(q, k, v, scale, causal, 0)
    dq, dk, dv, *_ = mo.sequence_backward(q, q, k, k, v, do, do, o, lse, np.arange(n_q), np.arange(L), scale,
                                          causal)
    rq, rk, rv = jo.sequence_backward(q, k, v, do, scale, causal, 0)
    ds = p * (do @ v.T - (do * o).sum(axis=1)[:, None])
    for got, ref, x, op, a, name in ((dv, rv, p.T, do, 1.0, "dv"), (dk, rk, ds.T, q, scale, "dk"),
                                     (dq, rq, ds, k, scale, "dq")):
        bound = abs(a) * (2.0 ** -3 * np.abs(x) @ np.abs(op)
                          + 2.0 ** -16 * np.abs(x).max(axis=1, keepdims=True) * np.abs(op).sum(axis=0)[None, :])
        err = np.abs(got - ref)
        assert (err <= bound + 1e-12).all(), name
        assert err.max() > 0, name


def _mx_case(lengths, H, H_kv, Lq, bq, seed, consistent=False, scale_fwd=0.1):
    t = wl.make_mx_bwd_tensors(lengths, H, H_kv, 128, Lq, bq, seed=seed, consistent=consistent)
    a = {n: (v.numpy() if hasattr(v, "numpy") else v) for n, v in t.items()}
    out, lse, _ = mo.jagged_forward(a["q8"], a["q_scale"], a["k8"], a["k_scale"], a["vt8"], a["vt_scale"],
                                    a["offsets"], scale_fwd, False, bq)
    return a, out, lse


def test_gradients_scale_with_powers_of_two_of_do():
    """dO twice as large (both encodings' scales one up): every gradient and
    allowance exactly twice."""
    for bq in (True, False):
        a, out, lse = _mx_case([3, 37, 0, 30], 2, 1, 8, bq, seed=9)
        g0 = mo.jagged_backward(a, out, lse, 0.1, True, bq)
        b = dict(a)
        b["do_scale"] = a["do_scale"] + 1
        b["dot_scale"] = a["dot_scale"] + 1
        g1 = mo.jagged_backward(b, out, lse, 0.1, True, bq)
        for x, y in zip(g0, g1):
            np.testing.assert_array_equal(y, 2 * x)


def test_dequantized_column_layouts_by_brute_force():
    rng = _rng(10)
    for bq in (True, False):
        t = wl.make_mx_bwd_tensors([3, 37, 0, 30], 2, 1, 128, 40, bq, seed=11, consistent=False)
        a = {n: (v.numpy() if hasattr(v, "numpy") else v) for n, v in t.items()}
        T = t["total_len"]
        Qr, Qc, Kr, Kc, Vr, dOr, dOc = mo.dequantize_backward_inputs(a, bq)
        dec = lambda c, s: mo.decode_e4m3(c) * 2.0 ** (int(s) - 127)
        for _ in range(300):
            j, tt = int(rng.integers(128)), int(rng.integers(T))
            assert Kc[tt, 0, j] == dec(a["kt8"][0, j, tt], a["kt_scale"][0, tt // 32, j])
            assert Vr[tt, 0, j] == dec(a["v8"][tt, 0, j], a["v_scale"][tt, 0, j // 32])
            h, b = int(rng.integers(2)), int(rng.integers(4))
            if bq:
                i = int(rng.integers(40))
                assert Qc[h, i, j] == dec(a["qt8"][h, j, i], a["qt_scale"][h, i // 32, j])
                assert dOc[b, h, i, j] == dec(a["dot8"][b, h, j, i], a["dot_scale"][b, h, i // 32, j])
                assert dOr[b, h, i, j] == dec(a["do8"][b, h, i, j], a["do_scale"][b, h, i, j // 32])
            else:
                assert Qc[tt, h, j] == dec(a["qt8"][h, j, tt], a["qt_scale"][h, tt // 32, j])
                assert dOc[tt, h, j] == dec(a["dot8"][h, j, tt], a["dot_scale"][h, tt // 32, j])
                assert dOr[tt, h, j] == dec(a["do8"][tt, h, j], a["do_scale"][tt, h, j // 32])


@pytest.mark.parametrize("bq", [True, False])
def test_jagged_backward_sums_per_sequence_and_group(bq):
    """The batch entry point: dK / dV of a key / value head are the sums over
    its query heads, broadcast dQ the sum over the sequences."""
    a, out, lse = _mx_case([3, 37, 0, 30], 4, 2, 8, bq, seed=12)
    dq, dk, dv, *_ = mo.jagged_backward(a, out, lse, 0.09, True, bq)
    deq = mo.dequantize_backward_inputs(a, bq)
    off = a["offsets"]
    rq, rk, rv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for b in range(4):
        s0, s1 = int(off[b]), int(off[b + 1])
        for h in range(4):
            g = mo.backward_item(a, deq, out, lse, b, h, 0.09, True, bq)
            if bq:
                rq[h] = rq[h] + g[0]
            else:
                rq[s0:s1, h] = g[0]
            rk[s0:s1, h // 2] += g[1]
            rv[s0:s1, h // 2] += g[2]
    np.testing.assert_array_equal(dq, rq)
    np.testing.assert_array_equal(dk, rk)
    np.testing.assert_array_equal(dv, rv)
