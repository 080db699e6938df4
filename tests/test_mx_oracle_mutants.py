"""Plant plausible mistakes in the MXFP8 oracle (on the CPU) and check that
its pins catch each one: evidence that the pins constrain every part of it.
"""
import math

import numpy as np
import pytest

from oracle import mx_oracle as mo
from tests import test_mx_oracle_pins as pins


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


_orig_quantize = mo.quantize_e4m3
_orig_decode = mo.decode_e4m3
_orig_seq = mo.sequence_forward


def _mut_scale_minus7(amax):
    return math.floor(math.log2(amax)) - 7


def _mut_ties_up(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), mo.E4M3_MAX)
    g = mo._GRID
    hi = np.clip(np.searchsorted(g, a, side="left"), 0, len(g) - 1)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (g[hi] - a) <= (a - g[lo])
    return np.copysign(np.where(pick_hi, g[hi], g[lo]), x)


def _mut_no_saturation(x):
    x = np.asarray(x, dtype=np.float64)
    q = _orig_quantize(x)
    # values past 448 keep rounding on the grid's next binade (480, 512)
    big = np.abs(x) > 464
    return np.where(big, np.copysign(np.round(np.abs(x) / 32) * 32, x), q)


def _mut_decode_bias8(codes):
    return _orig_decode(codes) / 2.0


def _mut_blocks_relative(q, k, v, s0, scale, causal):
    return _orig_seq(q, k, v, 0, scale, causal)


def _mut_l_quantized(q, k, v, s0, scale, causal):
    o, lse, allow = _orig_seq(q, k, v, s0, scale, causal)
    # normalise by the sum of the quantized weights instead (rows sum to 1)
    n_q, L = q.shape[0], k.shape[0]
    if L == 0:
        return o, lse, allow
    x = (q @ k.T) * (scale / math.log(2.0))
    vis = np.ones((n_q, L), dtype=bool)
    if causal:
        vis = np.arange(L)[None, :] <= np.arange(n_q)[:, None]
    for i in range(n_q):
        cols = np.nonzero(vis[i])[0]
        if cols.size == 0:
            continue
        xi = x[i, cols]
        p = np.exp2(xi - math.ceil(xi.max()))
        blocks = (s0 + cols) // mo.BLOCK
        ph = np.zeros_like(p)
        for b in np.unique(blocks):
            ph[blocks == b] = mo.quantize_block(p[blocks == b])[0]
        o[i] = (ph @ v[cols]) / ph.sum()
    return o, lse, allow


def _mut_vt_scale_swapped(vt8, vt_scale, total_len):
    v = mo.decode_e4m3(vt8)
    s = np.repeat(mo.decode_e8m0(vt_scale), mo.BLOCK, axis=1)
    s = s[:, ::-1, :]  # key blocks in the wrong order
    return (v.transpose(0, 2, 1) * s)[:, :total_len].transpose(1, 0, 2)


def _mut_row_blocks16(x8, scale8):
    v = mo.decode_e4m3(x8)
    s = mo.decode_e8m0(scale8)
    return v * np.tile(s, 2)[..., : v.shape[-1] // 16].repeat(16, axis=-1)


MUTANTS = {
    "scale_exponent_minus_7": ("block_scale_exponent", _mut_scale_minus7),
    "ties_round_up": ("quantize_e4m3", _mut_ties_up),
    "no_saturation": ("quantize_e4m3", _mut_no_saturation),
    "e4m3_bias_8": ("decode_e4m3", _mut_decode_bias8),
    "key_blocks_per_sequence": ("sequence_forward", _mut_blocks_relative),
    "sum_of_quantized_p": ("sequence_forward", _mut_l_quantized),
    "v_scale_blocks_reordered": ("dequantize_vt", _mut_vt_scale_swapped),
    "row_blocks_of_16": ("dequantize_rows", _mut_row_blocks16),
}


def _pin_suite():
    return [
        ("e4m3_torch", pins.test_e4m3_decoding_matches_torch_float8_e4m3fn),
        ("brute_quantize", pins.test_quantize_matches_brute_force_midpoints_and_saturation),
        ("torch_cast", pins.test_quantize_matches_torch_cast_below_overflow),
        ("closed_forms", pins.test_block_rule_closed_forms),
        ("invariance", pins.test_block_quantization_scales_with_powers_of_two),
        ("fragile", pins.test_fragile_decisions_and_their_deviation),
        ("exact_p", pins.test_exact_p_reduces_to_plain_attention),
        ("single_key", pins.test_single_key_closed_form),
        ("packed_blocks", pins.test_key_blocks_follow_the_packed_index),
        ("format_error", pins.test_quantized_forward_within_the_format_error_of_plain_attention),
        ("layouts", pins.test_dequantized_layouts_by_brute_force),
    ]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(mo, attr, fn)
    caught = [pin for pin, run in _pin_suite() if _fails(run)]
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    assert not [pin for pin, run in _pin_suite() if _fails(run)]
