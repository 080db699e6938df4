"""Pins of the MXFP8 oracle (oracle/mx_oracle.py) against things other than
itself: torch's own float8 formats, brute force over every E4M3 code, closed
forms of the block rule, the invariance the oracle's reading relies on, and
plain attention where quantization is exact."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import jfa_oracle as jo
from oracle import mx_oracle as mo


def test_e4m3_decoding_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = mo.decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # the format's landmarks
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0xFE] == -448.0


def test_e8m0_decoding_matches_torch_float8_e8m0fnu():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    got = mo.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127


def _brute_quantize(x):
    """Nearest non-negative E4M3 value by exhaustive search (ties: even
    code), sign restored, magnitudes above 448 saturated."""
    grid = mo.decode_e4m3(np.arange(127, dtype=np.uint8))
    out = np.empty_like(x)
    for i, v in enumerate(x):
        a = min(abs(v), 448.0)
        d = np.abs(grid - a)
        best = np.flatnonzero(d == d.min())
        code = best[0] if best.size == 1 else best[best % 2 == 0][0]
        out[i] = math.copysign(grid[code], v)
    return out


def test_quantize_matches_brute_force_midpoints_and_saturation():
    rng = np.random.default_rng(3)
    grid = mo.decode_e4m3(np.arange(127, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([rng.uniform(-500, 500, 2000), rng.uniform(-2, 2, 2000) * 2.0 ** rng.integers(-12, 3, 2000),
                        mids, -mids, grid, [0.0, 448.0, 449.0, 463.9, 464.0, 479.0, 1e6, -1e6]])
    assert np.array_equal(mo.quantize_e4m3(x), _brute_quantize(x))


def test_quantize_matches_torch_cast_below_overflow():
    rng = np.random.default_rng(4)
    x = rng.uniform(-463, 463, 5000) * 2.0 ** rng.integers(-14, 1, 5000)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(mo.quantize_e4m3(x.astype(np.float32).astype(np.float64)), ref)


def test_block_rule_closed_forms():
    # amax 3: scale 2^(1 - 8); 3 and 1 are on the grid, exact
    q, se, _ = mo.quantize_block(np.array([3.0, 1.0]))
    assert se == -7 and np.array_equal(q, [3.0, 1.0])
    # amax with mantissa 1.9: 1.9 * 256 = 486.4 saturates to 448 = 1.75 * 256
    q, se, _ = mo.quantize_block(np.array([1.9, 0.5]))
    assert se == -8 and q[0] == 1.75 and q[1] == 0.5
    # an element 2^-20 below the maximum: 2^-12 of the scale, half of the
    # smallest subnormal step rounds to zero; 2^-16 is two steps, exact
    q, _, _ = mo.quantize_block(np.array([1.0, 2.0 ** -20, 2.0 ** -16]))
    assert np.array_equal(q, [1.0, 0.0, 2.0 ** -16])
    q, se, dev = mo.quantize_block(np.zeros(5))
    assert se is None and not q.any() and not dev.any()


def test_block_quantization_scales_with_powers_of_two():
    """The reading that the exponentials' reference may be any power of two
    rests on this: quantizing 2^k p gives 2^k times quantizing p."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        p = rng.uniform(0, 1, 32) * 2.0 ** rng.integers(-20, 1, 32)
        k = int(rng.integers(-30, 30))
        q0, _, _ = mo.quantize_block(p)
        q1, _, _ = mo.quantize_block(p * 2.0 ** k)
        assert np.array_equal(q1, q0 * 2.0 ** k)


def test_fragile_decisions_and_their_deviation():
    # with amax 1.9 the scale is 2^-8, and 1.0625 maps to 272, the midpoint
    # of 256 and 288: it rounds to 1.0 (the even code) or, moved up, to
    # 1.125, one step of 2^-3 away
    q, _, dev = mo.quantize_block(np.array([1.9, 1.0625]))
    assert q[1] == 1.0 and dev[1] == 0.125 and dev[0] == 0.0
    _, _, dev = mo.quantize_block(np.array([1.9, 1.3]))
    assert not dev.any()
    # amax just below a power of two: the scale could be the next one up,
    # where 2 - 2^-20 no longer saturates (1.75 -> 2)
    q, _, dev = mo.quantize_block(np.array([2.0 * (1 - 2.0 ** -20), 0.3]))
    assert q[0] == 1.75 and dev[0] == 0.25


def test_exact_p_reduces_to_plain_attention():
    """With all scores equal, P = 1 on every visible key, which E4M3 holds
    exactly: the MXFP8 forward equals the textbook forward."""
    rng = np.random.default_rng(6)
    for causal in (False, True):
        L, d = 45, 128
        q = rng.standard_normal((L, d))
        k = np.zeros((L, d))
        v = rng.standard_normal((L, d))
        o, lse, allow = mo.sequence_forward(q, k, v, 17, 0.1, causal)
        ro, rl, _ = jo.sequence_forward(q, k, v, 0.1, causal, 0)
        # every block maximum is exactly 1, a power of two: a float32 value
        # just below it would take the next scale down and saturate at 0.875
        assert (allow > 0).all()
        np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)


def test_single_key_closed_form():
    rng = np.random.default_rng(7)
    d = 128
    for _ in range(20):
        q = rng.standard_normal((1, d))
        k = rng.standard_normal((1, d))
        v = rng.standard_normal((1, d))
        scale = 0.3
        o, lse, _ = mo.sequence_forward(q, k, v, 5, scale, False)
        s = float((q @ k.T)[0, 0]) * scale
        x = s / math.log(2)
        p = 2.0 ** (x - math.ceil(x))
        w = mo.quantize_e4m3(np.array([p * 2.0 ** (8 - math.floor(math.log2(p)))]))[0] \
            * 2.0 ** (math.floor(math.log2(p)) - 8) / p
        np.testing.assert_allclose(o[0], w * v[0], rtol=1e-13, atol=1e-15)
        assert abs(lse[0] - s) < 1e-12


def test_key_blocks_follow_the_packed_index():
    """Keys at packed positions 30, 31 | 32, 33 fall in two blocks.  A small
    P beside a large one is quantized on the large one's coarse grid; the
    same small P in the next block, beside only small ones, is exact."""
    d = 128
    P = np.array([1.0, 1.5 * 2.0 ** -17, 1.5 * 2.0 ** -17, 2.0 ** -17])
    x = np.log2(P)
    scale = 0.5
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k = np.zeros((4, d))
    k[:, 0] = x * math.log(2) / scale
    v = np.eye(4, d)
    o, _, _ = mo.sequence_forward(q, k, v, 30, scale, False)
    l = P.sum()
    # block {30, 31}: scale 2^-8, 1.5 * 2^-17 is 1.5 subnormal steps -> 2 steps
    # block {32, 33}: both exact
    np.testing.assert_allclose(o[0, :4] * l, [1.0, 2.0 ** -16, 1.5 * 2.0 ** -17, 2.0 ** -17], rtol=1e-12)
    # starting at packed position 0 the four keys share one block: both
    # 1.5-step values round to 2 steps (ties to even), 2^-17 is one step
    o, _, _ = mo.sequence_forward(q, k, v, 0, scale, False)
    np.testing.assert_allclose(o[0, :4] * l, [1.0, 2.0 ** -16, 2.0 ** -16, 2.0 ** -17], rtol=1e-12)


def test_quantized_forward_within_the_format_error_of_plain_attention():
    """E4M3 keeps 3 mantissa bits: each P moves by at most 2^-4 of itself
    (2^-3 where the block maximum saturates), so O moves by at most 2^-3 of
    max |v| from the unquantized forward on the same dequantized inputs."""
    rng = np.random.default_rng(8)
    for causal in (False, True):
        L, d = 70, 128
        q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
        o, lse, _ = mo.sequence_forward(q, k, v, 3, 0.2, causal)
        ro, rl, _ = jo.sequence_forward(q, k, v, 0.2, causal, 0)
        assert np.max(np.abs(o - ro)) <= 2.0 ** -3 * np.abs(v).max()
        np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-12)
        assert np.max(np.abs(o - ro)) > 0  # quantization does something


def test_dequantized_layouts_by_brute_force():
    """jagged_forward's dequantization of Q, K and the transposed V,
    checked element by element from the layout definitions."""
    import workloads as wl
    t = wl.make_mx_tensors([3, 37, 0, 30], 2, 1, 128, 8, True, seed=9)
    q8, qs, k8, ks = (t[n].numpy() for n in ("q8", "q_scale", "k8", "k_scale"))
    vt8, vts = t["vt8"].numpy(), t["vt_scale"].numpy()
    T = t["total_len"]
    Q = mo.dequantize_rows(q8, qs)
    K = mo.dequantize_rows(k8, ks)
    V = mo.dequantize_vt(vt8, vts, T)
    rng = np.random.default_rng(10)
    for _ in range(300):
        h, i, j = int(rng.integers(2)), int(rng.integers(8)), int(rng.integers(128))
        assert Q[h, i, j] == mo.decode_e4m3(q8[h, i, j]) * 2.0 ** (int(qs[h, i, j // 32]) - 127)
        tt = int(rng.integers(T))
        assert K[tt, 0, j] == mo.decode_e4m3(k8[tt, 0, j]) * 2.0 ** (int(ks[tt, 0, j // 32]) - 127)
        assert V[tt, 0, j] == mo.decode_e4m3(vt8[0, j, tt]) * 2.0 ** (int(vts[0, tt // 32, j]) - 127)


@pytest.mark.parametrize("bq", [True, False])
def test_jagged_forward_per_sequence(bq):
    """The batch entry point gives each (sequence, head) what
    sequence_forward gives on its rows, with the grouped head mapping."""
    import workloads as wl
    t = wl.make_mx_tensors([3, 37, 0, 30], 4, 2, 128, 8, bq, seed=11)
    arr = {n: t[n].numpy() for n in ("q8", "q_scale", "k8", "k_scale", "vt8", "vt_scale", "offsets")}
    out, lse, fr = mo.jagged_forward(arr["q8"], arr["q_scale"], arr["k8"], arr["k_scale"], arr["vt8"],
                                     arr["vt_scale"], arr["offsets"], 0.09, True, bq)
    Q = mo.dequantize_rows(arr["q8"], arr["q_scale"])
    K = mo.dequantize_rows(arr["k8"], arr["k_scale"])
    V = mo.dequantize_vt(arr["vt8"], arr["vt_scale"], t["total_len"])
    off = arr["offsets"]
    for b in range(4):
        s0, s1 = int(off[b]), int(off[b + 1])
        for h in range(4):
            qq = Q[h] if bq else Q[s0:s1, h]
            o, ls, _ = mo.sequence_forward(qq, K[s0:s1, h // 2], V[s0:s1, h // 2], s0, 0.09, True)
            got_o = out[b, h] if bq else out[s0:s1, h]
            got_l = lse[b, h] if bq else lse[s0:s1, h]
            np.testing.assert_array_equal(got_o, o)
            np.testing.assert_array_equal(got_l, ls)
