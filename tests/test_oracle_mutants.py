"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one.  This is evidence that the pins constrain every part of the
oracle, not a test of the library.
"""
import numpy as np
import pytest

from oracle import jfa_oracle as jo
from tests import test_oracle_pins as pins


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _mut_scores_no_scale(qb, kb, scale, causal, window=0):
    s = jo._f64(qb) @ jo._f64(kb).T
    if causal:
        s = np.where(jo.causal_visible(*s.shape), s, -np.inf)
    return s


def _mut_scores_wrong_causal(qb, kb, scale, causal, window=0):
    s = scale * (jo._f64(qb) @ jo._f64(kb).T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j < i, s, -np.inf) if s.shape[0] > 1 else s
    return s


def _mut_scores_off_by_one(qb, kb, scale, causal, window=0):
    s = scale * (jo._f64(qb) @ jo._f64(kb).T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        s = np.where(j <= i + 1, s, -np.inf)
    return s


def _mut_scores_window_off_by_one(qb, kb, scale, causal, window=0):
    s = scale * (jo._f64(qb) @ jo._f64(kb).T)
    if causal:
        i = np.arange(s.shape[0])[:, None]
        j = np.arange(s.shape[1])[None, :]
        vis = j <= i
        if window > 0:
            vis = vis & (j >= i - window)
        s = np.where(vis, s, -np.inf)
    return s


def _make_bwd_mutant(kind):
    orig = jo.sequence_backward

    def bwd(qb, kb, vb, dob, scale, causal, window=0):
        qb, kb, vb, dob = (jo._f64(x) for x in (qb, kb, vb, dob))
        if kb.shape[0] == 0:
            return orig(qb, kb, vb, dob, scale, causal)
        o, _, p = jo.sequence_forward(qb, kb, vb, scale, causal)
        delta = (dob * o).sum(axis=1)
        dp = dob @ vb.T
        if kind == "no_delta":
            ds = p * dp
        elif kind == "delta_sign":
            ds = p * (dp + delta[:, None])
        else:
            ds = p * (dp - delta[:, None])
        dq = scale * (ds @ kb)
        dk = scale * (ds.T @ qb)
        dv = p.T @ dob
        if kind == "dq_no_scale":
            dq = ds @ kb
        if kind == "dv_no_p":
            dv = np.ones_like(p).T @ dob / p.shape[1]
        if kind == "dk_uses_k":
            dk = scale * (ds.T @ (qb + 0.0 * qb) - 0.0) + 1e-3 * kb
        return dq, dk, dv
    return bwd


def _mut_lse_log2(qb, kb, vb, scale, causal, window=0):
    o, lse, p = ORIG_FWD(qb, kb, vb, scale, causal)
    return o, lse / np.log(2.0), p


ORIG_FWD = jo.sequence_forward


def _mut_softmax_no_max_shift(qb, kb, vb, scale, causal, window=0):
    o, lse, p = ORIG_FWD(qb, kb, vb, scale, causal)
    return o, lse - 0.5, p


def _mut_jagged_dq_overwrite(q, k, v, offsets, scale, causal, broadcast_q, dout, window=0):
    q64, k64, v64, d64 = (jo._f64(x) for x in (q, k, v, dout))
    dq = np.zeros_like(q64)
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    for b, (s0, s1) in enumerate(jo._seq_bounds(offsets)):
        for h in range(k64.shape[1]):
            if broadcast_q:
                g = jo.sequence_backward(q64[h], k64[s0:s1, h], v64[s0:s1, h], d64[b, h], scale, causal)
                if s1 > s0:
                    dq[h] = g[0]  # planted: '=' where the batch sum needs '+='
            else:
                g = jo.sequence_backward(q64[s0:s1, h], k64[s0:s1, h], v64[s0:s1, h], d64[s0:s1, h],
                                         scale, causal)
                dq[s0:s1, h] = g[0]
            dk[s0:s1, h], dv[s0:s1, h] = g[1], g[2]
    return dq, dk, dv


def _mut_gqa_interleaved_heads(q, k, v, offsets, scale, causal, broadcast_q, window=0):
    """Grouped heads mapped round-robin (h % H_kv) instead of by group."""
    q, k, v = jo._f64(q), jo._f64(k), jo._f64(v)
    bounds = jo._seq_bounds(offsets)
    H = q.shape[0] if broadcast_q else q.shape[1]
    Hkv = k.shape[1]
    B, Lq = len(bounds), (q.shape[1] if broadcast_q else 0)
    out = np.zeros((B, H, Lq, v.shape[2])) if broadcast_q else np.zeros((q.shape[0], H, v.shape[2]))
    lse = np.zeros((B, H, Lq)) if broadcast_q else np.zeros((q.shape[0], H))
    for b, (s0, s1) in enumerate(bounds):
        for h in range(H):
            qb = q[h] if broadcast_q else q[s0:s1, h]
            o, ls, _ = jo.sequence_forward(qb, k[s0:s1, h % Hkv], v[s0:s1, h % Hkv], scale, causal)
            if broadcast_q:
                out[b, h], lse[b, h] = o, ls
            else:
                out[s0:s1, h], lse[s0:s1, h] = o, ls
    return out, lse


def _mut_gqa_dkv_overwrite(q, k, v, offsets, scale, causal, broadcast_q, dout, window=0):
    """dK / dV of a shared head keep only the last query head of the group."""
    q, k, v, dout = jo._f64(q), jo._f64(k), jo._f64(v), jo._f64(dout)
    bounds = jo._seq_bounds(offsets)
    H = q.shape[0] if broadcast_q else q.shape[1]
    G = H // k.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b, (s0, s1) in enumerate(bounds):
        for h in range(H):
            kb, vb = k[s0:s1, h // G], v[s0:s1, h // G]
            if broadcast_q:
                g = jo.sequence_backward(q[h], kb, vb, dout[b, h], scale, causal)
                dq[h] += g[0]
            else:
                g = jo.sequence_backward(q[s0:s1, h], kb, vb, dout[s0:s1, h], scale, causal)
                dq[s0:s1, h] = g[0]
            dk[s0:s1, h // G] = g[1]
            dv[s0:s1, h // G] = g[2]
    return dq, dk, dv


def _pin_suite():
    """Every pin, as (name, callable) pairs; a mutant must fail at least one."""
    return [
        ("rows_sum", lambda: [pins.test_softmax_rows_sum_to_one(c) for c in (False, True)]),
        ("single_key", lambda: [pins.test_single_key_returns_v_exactly(b) for b in (True, False)]),
        ("causal_row0", pins.test_causal_first_row_returns_first_value),
        ("dense_bcast", lambda: [pins.test_equal_lengths_broadcast_is_dense_attention(c) for c in (False, True)]),
        ("sdpa_causal", pins.test_single_sequence_causal_is_sdpa_is_causal),
        ("block_diag", lambda: [pins.test_self_mode_is_block_diagonal_dense_attention(c) for c in (False, True)]),
        ("dq_sum", pins.test_broadcast_dq_is_sum_of_per_sequence_dq),
        ("fd", lambda: [pins.test_finite_differences(b, c) for b in (True, False) for c in (False, True)]),
        ("gqa_self", lambda: [pins.test_gqa_self_mode_is_sdpa_grouped_query(c, 4, 2) for c in (False, True)]),
        ("gqa_bcast", lambda: [pins.test_gqa_broadcast_is_sdpa_grouped_query(c) for c in (False, True)]),
        ("window_self", lambda: [pins.test_window_self_mode_is_sdpa_with_a_band_mask(w) for w in (1, 3)]),
        ("window_bcast", pins.test_window_broadcast_rows_that_see_no_key),
    ]


MUTANTS = {
    "scores_without_scale": ("sequence_scores", _mut_scores_no_scale),
    "causal_strict_lower": ("sequence_scores", _mut_scores_wrong_causal),
    "causal_off_by_one": ("sequence_scores", _mut_scores_off_by_one),
    "bwd_no_delta": ("sequence_backward", _make_bwd_mutant("no_delta")),
    "bwd_delta_sign": ("sequence_backward", _make_bwd_mutant("delta_sign")),
    "bwd_dq_no_scale": ("sequence_backward", _make_bwd_mutant("dq_no_scale")),
    "bwd_dv_wrong": ("sequence_backward", _make_bwd_mutant("dv_no_p")),
    "bwd_dk_extra_term": ("sequence_backward", _make_bwd_mutant("dk_uses_k")),
    "lse_base2": ("sequence_forward", _mut_lse_log2),
    "lse_shifted": ("sequence_forward", _mut_softmax_no_max_shift),
    "bcast_dq_overwrite": ("jagged_backward", _mut_jagged_dq_overwrite),
    "window_off_by_one": ("sequence_scores", _mut_scores_window_off_by_one),
    "gqa_interleaved_heads": ("jagged_forward", _mut_gqa_interleaved_heads),
    "gqa_dkv_overwrite": ("jagged_backward", _mut_gqa_dkv_overwrite),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(jo, attr, fn)
    caught = [pin for pin, run in _pin_suite() if _fails(run)]
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    assert not [pin for pin, run in _pin_suite() if _fails(run)]
