"""Parity at the full sizes of the larger workloads, through the C-ABI, in
the launch configuration bench.py times.

prod_bcast, long_causal_8k and skew_bcast are compared over their whole O,
lse, dQ, dK and dV tensors.  The oracle's per-(sequence, head) functions run in a
process pool (tests/_oracle_pool.py).  The variant workloads are sampled:
every head of a few sequences, and a few whole broadcast dQ rows.
"""
import math
import time

import numpy as np
import pytest

import workloads as wl
from oracle import jfa_oracle as jo
from tests._oracle_pool import WholeLse, WholeTensor, run_items
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


def _check_whole(w, t, out, lse, dq, dk, dv, heads, acc=None):
    """Every (sequence, head) of the listed heads (plain heads, H_kv = H):
    O, lse, dK, dV (and self-attention dQ) item by item, broadcast dQ of
    those heads summed over every sequence in fp64; each statistic over the
    whole tensor.  With `acc` (accumulators of an earlier call over other
    heads) the statistics continue and are checked by the caller."""
    assert w.kv_heads == w.H
    off = t["offsets"].cpu().numpy()
    B, bq, scale = w.B, w.broadcast_q, w.scale
    t0 = time.perf_counter()
    host = {}
    for h in heads:
        host[h] = {
            "k": t["k"][:, h].float().cpu().numpy(),
            "v": t["v"][:, h].float().cpu().numpy(),
            "q": (t["q"][h] if bq else t["q"][:, h]).float().cpu().numpy(),
            "do": (t["dout"][:, h] if bq else t["dout"][:, h]).float().cpu().numpy(),
            "o": (out[:, h] if bq else out[:, h]).float().cpu().numpy(),
            "lse": (lse[:, h] if bq else lse[:, h]).cpu().numpy(),
            "dq": (dq[h] if bq else dq[:, h]).cpu().numpy(),
            "dk": dk[:, h].cpu().numpy(),
            "dv": dv[:, h].cpu().numpy(),
        }
    print(f"  host copies of heads {list(heads)}: {time.perf_counter() - t0:.1f} s", flush=True)
    items, cost, where = [], [], []
    for h in heads:
        x = host[h]
        for b in range(B):
            s0, s1 = int(off[b]), int(off[b + 1])
            qb = x["q"] if bq else x["q"][s0:s1]
            dob = x["do"][b] if bq else x["do"][s0:s1]
            items.append((qb, x["k"][s0:s1], x["v"][s0:s1], dob, scale, w.causal, w.window))
            cost.append(qb.shape[0] * max(s1 - s0, 1))
            where.append((h, b, s0, s1))
    if acc is None:
        chk = {n: WholeTensor(f"{n} {w.name}") for n in ("O", "dQ", "dK", "dV")}
        chk_lse = WholeLse(f"lse {w.name}")
    else:
        chk, chk_lse = acc
    ref_dq = {h: np.zeros_like(host[h]["dq"], dtype=np.float64) for h in heads} if bq else None
    done = 0
    for i, (o_r, l_r, q_r, k_r, v_r) in run_items(items, cost):
        h, b, s0, s1 = where[i]
        x = host[h]
        if bq:
            chk["O"].add(x["o"][b], o_r)
            chk_lse.add(x["lse"][b], l_r)
            ref_dq[h] += q_r
        else:
            chk["O"].add(x["o"][s0:s1], o_r)
            chk_lse.add(x["lse"][s0:s1], l_r)
            chk["dQ"].add(x["dq"][s0:s1], q_r)
        chk["dK"].add(x["dk"][s0:s1], k_r)
        chk["dV"].add(x["dv"][s0:s1], v_r)
        done += 1
        if done % max(1, len(items) // 8) == 0:
            print(f"  oracle {done}/{len(items)} items, {time.perf_counter() - t0:.1f} s", flush=True)
    if bq:
        for h in heads:
            chk["dQ"].add(host[h]["dq"], ref_dq[h])
    if acc is not None:
        return
    for c in chk.values():
        c.check()
    chk_lse.check()


@pytest.mark.timeout(900)
def test_full_prod_bcast(jfa):
    """The whole of every output, all 1024 sequences and 4 heads."""
    w, t, out, lse, dq, dk, dv = _run_full(jfa, 2)
    _check_whole(w, t, out, lse, dq, dk, dv, range(w.H))


@pytest.mark.timeout(900)
def test_full_long_causal(jfa):
    """The whole of every output, all 64 sequences and 16 heads."""
    w, t, out, lse, dq, dk, dv = _run_full(jfa, 3)
    _check_whole(w, t, out, lse, dq, dk, dv, range(w.H))


@pytest.mark.timeout(900)
def test_full_skew_bcast(jfa):
    """The whole of every output: dQ summed over all 4096 sequences, and O,
    lse, dK, dV of every sequence (the 410 long ones included), all 8 heads
    (two at a time, to bound the host copies)."""
    w, t, out, lse, dq, dk, dv = _run_full(jfa, 4)
    acc = ({n: WholeTensor(f"{n} {w.name}") for n in ("O", "dQ", "dK", "dV")}, WholeLse(f"lse {w.name}"))
    for h0 in range(0, w.H, 2):
        _check_whole(w, t, out, lse, dq, dk, dv, [h0, h0 + 1], acc=acc)
    for c in acc[0].values():
        c.check()
    acc[1].check()


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
