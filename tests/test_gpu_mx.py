"""MXFP8 forward on the GPU against the fp64 MXFP8 oracle (oracle/mx_oracle.py).

Inputs are random E4M3 / E8M0 codes (workloads.make_mx_tensors).  O is
compared element by element with the bar of the bf16 path (max abs 2e-2
plus, per element, the oracle's allowance for quantization decisions that a
float32 computation may take the other way; rel-L2 5e-3) and lse with its
max-abs bar; lse does not depend on the quantization of P."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import mx_oracle as mo
from tests._parity import LSE_MAX_ABS, MAX_ABS, REL_L2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import jagged_flashattention_fwd_amd as m
    m.lib()
    return m


def _run(jfa, t, bq, causal, scale):
    dev = torch.device("cuda:0")
    g = {n: t[n].to(dev) for n in ("q8", "q_scale", "k8", "k_scale", "vt8", "vt_scale", "offsets")}
    out, lse = jfa.attention_fwd_mxfp8(g["q8"], g["q_scale"], g["k8"], g["k_scale"], g["vt8"], g["vt_scale"],
                                       g["offsets"], scale, causal, bq)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _oracle(t, bq, causal, scale):
    a = {n: t[n].cpu().numpy() for n in ("q8", "q_scale", "k8", "k_scale", "vt8", "vt_scale", "offsets")}
    return mo.jagged_forward(a["q8"], a["q_scale"], a["k8"], a["k_scale"], a["vt8"], a["vt_scale"], a["offsets"],
                             scale, causal, bq)


def _compare(name, got_o, got_l, ref_o, ref_l, allow):
    assert np.all(np.isfinite(got_o)), f"{name}: non-finite O"
    err = np.abs(got_o - ref_o)
    excess = err - allow
    worst = float(excess.max()) if excess.size else 0.0
    robust = allow == 0
    worst_robust = float(err[robust].max()) if robust.any() else 0.0
    beyond = float(np.mean(err > MAX_ABS)) if err.size else 0.0
    d2 = float(np.sum((got_o - ref_o) ** 2))
    r2 = float(np.sum(ref_o ** 2))
    rel = math.sqrt(d2 / r2) if r2 > 0 else math.sqrt(d2)
    ninf = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(got_l), ninf), f"{name}: lse -inf pattern"
    lerr = float(np.max(np.abs(got_l[~ninf] - ref_l[~ninf]))) if (~ninf).any() else 0.0
    print(f"  {name}: O max |err| where every decision is robust {worst_robust:.3e}, max |err| - allowance "
          f"{worst:.3e} (max allowance {allow.max():.2e}), share of |err| > {MAX_ABS}: {beyond:.1e}, "
          f"rel L2 {rel:.3e}, lse max abs {lerr:.3e}", flush=True)
    assert worst_robust <= MAX_ABS, f"{name}: O error {worst_robust:.3e}"
    assert worst <= MAX_ABS, f"{name}: O error {worst:.3e} beyond the allowance"
    assert beyond <= 1e-3, f"{name}: {beyond:.1e} of the elements past {MAX_ABS}"
    assert rel <= REL_L2, f"{name}: O rel L2 {rel:.3e}"
    assert lerr <= LSE_MAX_ABS, f"{name}: lse {lerr:.3e}"


CASES = [
    # (lengths, H, H_kv, Lq, broadcast_q, causal)
    ([5, 40, 0, 33, 100, 1, 64, 130, 257], 2, 2, 40, True, False),
    ([5, 40, 0, 33, 100, 1, 64, 130, 257], 2, 1, 300, True, True),
    ([300, 1, 65, 0, 129], 2, 1, 0, False, False),
    ([600, 31, 64, 200], 4, 2, 0, False, True),
    ([64, 128, 192], 2, 2, 256, True, False),
    ([1], 1, 1, 1, True, False),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_mx_forward_matches_oracle(jfa, case):
    lengths, H, H_kv, Lq, bq, causal = CASES[case]
    print(f"mx case {case}: lengths={lengths[:6]}.. H={H} H_kv={H_kv} Lq={Lq} bq={bq} causal={causal}", flush=True)
    t = wl.make_mx_tensors(lengths, H, H_kv, 128, Lq, bq, seed=100 + case)
    scale = 1.0 / math.sqrt(128)
    got_o, got_l = _run(jfa, t, bq, causal, scale)
    ref_o, ref_l, allow = _oracle(t, bq, causal, scale)
    _compare(f"case {case}", got_o, got_l, ref_o, ref_l, allow)


def test_mx_forward_sharper_scores(jfa):
    """A larger scale: sharper softmax rows, block maxima far apart."""
    lengths = [70, 300, 33, 129]
    t = wl.make_mx_tensors(lengths, 2, 2, 128, 64, True, seed=7)
    got_o, got_l = _run(jfa, t, True, False, 0.6)
    ref_o, ref_l, allow = _oracle(t, True, False, 0.6)
    _compare("sharp", got_o, got_l, ref_o, ref_l, allow)


def test_mx_forward_negative_scale(jfa):
    lengths = [70, 130, 1]
    t = wl.make_mx_tensors(lengths, 2, 2, 128, 40, True, seed=8)
    got_o, got_l = _run(jfa, t, True, False, -1.0 / math.sqrt(128))
    ref_o, ref_l, allow = _oracle(t, True, False, -1.0 / math.sqrt(128))
    _compare("negative scale", got_o, got_l, ref_o, ref_l, allow)


def test_mx_forward_prod_bcast_sampled(jfa):
    """prod_bcast's shapes (1024 sequences of U[64, 2048] keys, 4 heads,
    256 broadcast queries) at full size: every output finite; three
    sequences and all their heads against the oracle."""
    w = wl.workload("prod_bcast")
    t = wl.make_mx_workload(w, device="cuda:0")
    scale = 1.0 / math.sqrt(128)
    got_o, got_l = _run(jfa, t, True, False, scale)
    off = t["offsets"].cpu().numpy()
    rng = np.random.default_rng(41)
    for b in [int(x) for x in rng.choice(w.B, size=3, replace=False)]:
        s0, s1 = int(off[b]), int(off[b + 1])
        sub = {n: t[n].cpu() for n in ("q8", "q_scale")}
        k8, ks = t["k8"][s0:s1].cpu().numpy(), t["k_scale"][s0:s1].cpu().numpy()
        Q = mo.dequantize_rows(sub["q8"].numpy(), sub["q_scale"].numpy())
        K = mo.dequantize_rows(k8, ks)
        # V of the sequence's keys only: codes [H_kv, d, s0:s1], scales of their blocks
        vt = t["vt8"][:, :, s0:s1].cpu().numpy()
        vs = t["vt_scale"].cpu().numpy()[:, (np.arange(s0, s1) // 32), :]          # [H_kv, L, d]
        V = (mo.decode_e4m3(vt).transpose(0, 2, 1) * mo.decode_e8m0(vs)).transpose(1, 0, 2)
        for h in range(w.H):
            o, ls, allow = mo.sequence_forward(Q[h], K[:, h], V[:, h], s0, scale, False)
            _compare(f"prod_bcast seq {b} head {h}", got_o[b, h], got_l[b, h], o, ls, allow)
