"""Parity at the full sizes of the larger workloads, through the C-ABI, in
the launch configuration bench.py times.

The oracle cannot redo a whole workload in seconds, so the outputs are
sampled: every head of a few sequences (the longest, the shortest and
seeded random ones) for O, lse, dK, dV (and self-attention dQ), and a few
whole rows of the broadcast-Q dQ, each computed one by one by the oracle.
"""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import jfa_oracle as jo
from tests._parity import compare, compare_lse

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import jagged_flashattention_fwd_amd as m
    m.lib()
    return m


def f64(t):
    return t.detach().to("cpu").double().numpy()


def _sample_sequences(lengths, n_random, seed):
    rng = np.random.default_rng(seed)
    L = np.asarray(lengths)
    picks = {int(np.argmax(L)), int(np.argmin(L))}
    while len(picks) < 2 + n_random:
        picks.add(int(rng.integers(0, len(L))))
    return sorted(picks)


def _run_full(jfa, idx):
    w = wl.workload(idx)
    print(f"full-size {w.name}: generating", flush=True)
    t = wl.make_workload(w, device="cuda")
    scale = w.scale
    out, lse = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], scale, w.causal, w.broadcast_q,
                                 window=w.window)
    dq, dk, dv = jfa.attention_bwd(t["q"], t["k"], t["v"], t["offsets"], scale, w.causal, w.broadcast_q,
                                   out, lse, t["dout"], window=w.window)
    torch.cuda.synchronize()
    for name, x in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        finite = torch.isfinite(x) if name != "lse" else (torch.isfinite(x) | torch.isneginf(x))
        assert bool(finite.all()), f"{name} has non-finite values"
    print(f"full-size {w.name}: library done, checking samples", flush=True)
    return w, t, out, lse, dq, dk, dv


def _check_sequences(w, t, out, lse, dq, dk, dv, seqs, kv_heads):
    """Every query head of the listed key / value heads (one each without
    grouped heads): O, lse (and self-mode dQ) per query head, dK / dV as the
    sum over the group's query heads."""
    off = t["offsets"].cpu().numpy()
    G = w.H // w.kv_heads
    for b in seqs:
        s0, s1 = int(off[b]), int(off[b + 1])
        for hk in kv_heads:
            kb, vb = f64(t["k"][s0:s1, hk]), f64(t["v"][s0:s1, hk])
            sk, sv = 0.0, 0.0
            for h in range(hk * G, (hk + 1) * G):
                if w.broadcast_q:
                    qb, dob = f64(t["q"][h]), f64(t["dout"][b, h])
                    o_g, l_g = f64(out[b, h]), f64(lse[b, h])
                else:
                    qb, dob = f64(t["q"][s0:s1, h]), f64(t["dout"][s0:s1, h])
                    o_g, l_g = f64(out[s0:s1, h]), f64(lse[s0:s1, h])
                o_r, l_r, _ = jo.sequence_forward(qb, kb, vb, w.scale, w.causal, w.window)
                gq, gk, gv = jo.sequence_backward(qb, kb, vb, dob, w.scale, w.causal, w.window)
                sk, sv = sk + gk, sv + gv
                tag = f"{w.name} seq {b} (L={s1 - s0}) head {h}"
                compare(f"O {tag}", o_g, o_r)
                compare_lse(f"lse {tag}", l_g, l_r)
                if not w.broadcast_q:
                    compare(f"dQ {tag}", f64(dq[s0:s1, h]), gq)
            tag = f"{w.name} seq {b} (L={s1 - s0}) key/value head {hk}"
            compare(f"dK {tag}", f64(dk[s0:s1, hk]), sk)
            compare(f"dV {tag}", f64(dv[s0:s1, hk]), sv)


def _check_broadcast_dq_rows(w, t, dq, rows):
    off = t["offsets"].cpu().numpy()
    G = w.H // w.kv_heads
    for h in sorted({h for h, _ in rows}):
        # one head's K, V, dO on the host as float32 (the oracle widens each slice)
        hk = h // G
        k = t["k"][:, hk:hk + 1].float().cpu().numpy()
        v = t["v"][:, hk:hk + 1].float().cpu().numpy()
        do = t["dout"][:, h:h + 1].float().cpu().numpy()
        q = t["q"][h:h + 1].float().cpu().numpy()
        mine = [(0, i) for hh, i in rows if hh == h]
        ref = jo.broadcast_dq_rows(q, k, v, off, w.scale, w.causal, do, mine)
        got = np.stack([f64(dq[h, i]) for _, i in mine])
        compare(f"dQ {w.name} head {h} rows {[i for _, i in mine]}", got, ref)


@pytest.mark.timeout(900)
def test_full_prod_bcast(jfa):
    w, t, out, lse, dq, dk, dv = _run_full(jfa, 2)
    seqs = _sample_sequences(t["lengths"], 4, seed=202)
    _check_sequences(w, t, out, lse, dq, dk, dv, seqs, range(w.H))
    _check_broadcast_dq_rows(w, t, dq, [(0, 0), (0, 255), (3, 130), (2, 77)])


@pytest.mark.timeout(900)
def test_full_long_causal(jfa):
    w, t, out, lse, dq, dk, dv = _run_full(jfa, 3)
    seqs = _sample_sequences(t["lengths"], 2, seed=303)
    _check_sequences(w, t, out, lse, dq, dk, dv, seqs, [0, 7, 15])


@pytest.mark.timeout(900)
def test_full_skew_bcast(jfa):
    w, t, out, lse, dq, dk, dv = _run_full(jfa, 4)
    L = np.asarray(t["lengths"])
    long_ids = np.nonzero(L >= 4096)[0]
    seqs = sorted(set(_sample_sequences(L, 3, seed=404)) | {int(long_ids[0])})
    _check_sequences(w, t, out, lse, dq, dk, dv, seqs, [0, 5])
    _check_broadcast_dq_rows(w, t, dq, [(1, 0), (1, 511), (6, 300)])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx", [5, 6])
def test_full_dense_llm(jfa, idx):
    w, t, out, lse, dq, dk, dv = _run_full(jfa, idx)
    seqs = _sample_sequences(t["lengths"], 3, seed=500 + idx)
    _check_sequences(w, t, out, lse, dq, dk, dv, seqs, range(w.H))


@pytest.mark.timeout(900)
def test_full_prod_bcast_grouped_query(jfa):
    w, t, out, lse, dq, dk, dv = _run_full(jfa, "prod_bcast_gqa")
    assert dk.shape[1] == 1
    seqs = _sample_sequences(t["lengths"], 3, seed=707)
    _check_sequences(w, t, out, lse, dq, dk, dv, seqs, [0])
    _check_broadcast_dq_rows(w, t, dq, [(0, 0), (3, 200)])


@pytest.mark.timeout(900)
def test_full_long_causal_window(jfa):
    w, t, out, lse, dq, dk, dv = _run_full(jfa, "long_causal_8k_window")
    seqs = _sample_sequences(t["lengths"], 2, seed=808)
    _check_sequences(w, t, out, lse, dq, dk, dv, seqs, [0, 9])
