"""MXFP8 backward on the GPU against the fp64 MXFP8 backward oracle
(oracle/mx_oracle.py, jagged_backward).

Inputs are seeded random E4M3 / E8M0 codes in every encoding
(workloads.make_mx_bwd_tensors), either one tensor per name whose row-wise
and axis-blocked encodings hold the same values, or every encoding drawn on
its own (so that a kernel reading one encoding for another fails).  O and
lse are the oracle's MXFP8 forward, rounded to bf16 / fp32, and go to both
sides.  dQ, dK and dV are compared element by element with the bar of the
bf16 path: max abs 2e-2 beyond the oracle's per-element allowance for
float32-fragile quantization decisions, the same 2e-2 where every decision
is robust, and rel-L2 5e-3 of the error beyond the allowance.  The raw rel-L2
is printed too: a P block whose largest value is exactly 1 (a causal row's
first key, where P = exp(S - lse) = 1 up to rounding) takes the scale 2^-8
or, a rounding below, 2^-9 with 1 saturating to 0.875, so whole columns may
legitimately differ by 1/8."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import mx_oracle as mo
from tests._parity import MAX_ABS, REL_L2

pytestmark = pytest.mark.gpu

ENC = ("q8", "q_scale", "qt8", "qt_scale", "k8", "k_scale", "kt8", "kt_scale", "v8", "v_scale", "do8", "do_scale",
       "dot8", "dot_scale")


@pytest.fixture(scope="module")
def jfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import jagged_flashattention_fwd_amd as m
    m.lib()
    return m


def _np(t):
    return {n: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for n, v in t.items()}


def _forward_inputs(a, bq, causal, scale):
    """O (bf16-rounded) and lse (fp32-rounded) of the oracle's MXFP8 forward,
    as float64, and as the device tensors the library reads."""
    out, lse, _ = mo.jagged_forward(a["q8"], a["q_scale"], a["k8"], a["k_scale"], a["vt8"], a["vt_scale"],
                                    a["offsets"], scale, causal, bq)
    o_bf = torch.from_numpy(out).to(torch.bfloat16)
    l_32 = torch.from_numpy(lse).to(torch.float32)
    return o_bf.double().numpy(), l_32.double().numpy(), o_bf, l_32


def _run(jfa, t, bq, causal, scale, o_bf, l_32):
    dev = torch.device("cuda:0")
    g = {n: t[n].to(dev) for n in ENC}
    dq, dk, dv = jfa.attention_bwd_mxfp8(g, t["offsets"].to(dev), scale, causal, bq, o_bf.to(dev), l_32.to(dev))
    torch.cuda.synchronize()
    return [x.cpu().double().numpy() for x in (dq, dk, dv)]


def _compare(name, got, ref, allow):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return
    err = np.abs(got - ref)
    worst = float((err - allow).max())
    robust = allow == 0
    worst_robust = float(err[robust].max()) if robust.any() else 0.0
    r2 = float(np.sum(ref ** 2))
    rn = math.sqrt(r2) if r2 > 0 else 1.0
    rel_raw = math.sqrt(float(np.sum(err ** 2))) / rn
    # the part of the error that no fragile decision explains
    rel = math.sqrt(float(np.sum(np.maximum(err - allow, 0.0) ** 2))) / rn
    print(f"  {name}: max |err| where every decision is robust {worst_robust:.3e}, max |err| - allowance "
          f"{worst:.3e} (max allowance {allow.max():.2e}, max |ref| {np.abs(ref).max():.2e}), rel L2 beyond the "
          f"allowance {rel:.3e} (raw {rel_raw:.3e})", flush=True)
    assert worst_robust <= MAX_ABS, f"{name}: error {worst_robust:.3e}"
    assert worst <= MAX_ABS, f"{name}: error {worst:.3e} beyond the allowance"
    assert rel <= REL_L2, f"{name}: rel L2 {rel:.3e} beyond the allowance"


CASES = [
    # (lengths, H, H_kv, Lq, broadcast_q, causal, consistent)
    ([5, 40, 0, 33, 100, 1, 64, 130, 257], 2, 2, 40, True, False, True),
    ([5, 40, 0, 33, 100, 1, 64, 130, 257], 2, 1, 300, True, True, False),
    ([300, 1, 65, 0, 129], 2, 1, 0, False, False, False),
    ([600, 31, 64, 200], 4, 2, 0, False, True, True),
    ([64, 128, 192], 2, 2, 256, True, False, False),
    ([1], 1, 1, 1, True, False, True),
    ([129, 3, 250], 2, 2, 64, True, True, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_mx_backward_matches_oracle(jfa, case):
    lengths, H, H_kv, Lq, bq, causal, cons = CASES[case]
    print(f"mx bwd case {case}: lengths={lengths[:6]}.. H={H} H_kv={H_kv} Lq={Lq} bq={bq} causal={causal} "
          f"consistent={cons}", flush=True)
    t = wl.make_mx_bwd_tensors(lengths, H, H_kv, 128, Lq, bq, seed=200 + case, consistent=cons)
    a = _np(t)
    scale = 1.0 / math.sqrt(128)
    o64, l64, o_bf, l_32 = _forward_inputs(a, bq, causal, scale)
    got = _run(jfa, t, bq, causal, scale, o_bf, l_32)
    ref = mo.jagged_backward(a, o64, l64, scale, causal, bq)
    for i, name in enumerate(("dq", "dk", "dv")):
        _compare(f"case {case} {name}", got[i], ref[i], ref[3 + i])


@pytest.mark.parametrize("scale", [0.6, -0.3, 0.0])
def test_mx_backward_other_scales(jfa, scale):
    """Sharper rows, a negative scale, and scale 0 (uniform P, dK = dQ = 0)."""
    lengths = [70, 300, 33, 129]
    t = wl.make_mx_bwd_tensors(lengths, 2, 2, 128, 64, True, seed=9, consistent=False)
    a = _np(t)
    o64, l64, o_bf, l_32 = _forward_inputs(a, True, False, scale)
    got = _run(jfa, t, True, False, scale, o_bf, l_32)
    ref = mo.jagged_backward(a, o64, l64, scale, False, True)
    for i, name in enumerate(("dq", "dk", "dv")):
        _compare(f"scale {scale} {name}", got[i], ref[i], ref[3 + i])
    if scale == 0.0:
        assert not got[0].any() and not got[1].any()


def test_mx_backward_prod_bcast_sampled(jfa):
    """prod_bcast's shapes (1024 sequences of U[64, 2048] keys, 4 heads, 256
    broadcast queries) at full size, in the launch configuration the bench
    times: every output finite; dK / dV of three sequences (every head)
    against the oracle; two whole dQ rows per head, each the sum over all
    1024 sequences of the oracle's one-row backward.  O and lse are the
    oracle's unquantized fp64 forward of the dequantized inputs (any O and
    lse are valid backward inputs; these are close to the forward's)."""
    from oracle import jfa_oracle as jo
    from tests._oracle_pool import run_calls
    w = wl.workload("prod_bcast")
    print("mx bwd prod_bcast: generating", flush=True)
    t = wl.make_mx_bwd_workload(w, device="cuda:0")
    a = _np(t)
    scale = w.scale
    off = a["offsets"]
    B, H, Lq = w.B, w.H, w.Lq
    Qr = mo.dequantize_rows(a["q8"], a["q_scale"])
    Qc = mo.dequantize_cols(a["qt8"], a["qt_scale"], Lq)

    def seq_kv(b):
        s0, s1 = int(off[b]), int(off[b + 1])
        Kr = mo.dequantize_rows(a["k8"][s0:s1], a["k_scale"][s0:s1])
        Vr = mo.dequantize_rows(a["v8"][s0:s1], a["v_scale"][s0:s1])
        Kc = np.swapaxes(mo.dequantize_cols(a["kt8"], a["kt_scale"], s1 - s0, s0), 0, 1)
        return s0, s1, Kr, Kc, Vr

    print("mx bwd prod_bcast: O and lse (oracle forward)", flush=True)
    out = np.zeros((B, H, Lq, 128))
    lse = np.full((B, H, Lq), -np.inf)
    items, where = [], []
    kv = {}
    for b in range(B):
        s0, s1, Kr, Kc, Vr = seq_kv(b)
        kv[b] = (s0, s1, Kr, Kc, Vr)
        if s1 > s0:
            for h in range(H):
                items.append((np.float32(Qr[h]), np.float32(Kr[:, h]), np.float32(Vr[:, h]), scale, False, 0))
                where.append((b, h))
    for i, (o, ls, _) in run_calls("oracle.jfa_oracle", "sequence_forward", items, [len(x[1]) for x in items]):
        b, h = where[i]
        out[b, h], lse[b, h] = o, ls
    o_bf = torch.from_numpy(out).to(torch.bfloat16)
    l_32 = torch.from_numpy(lse).to(torch.float32)
    o64, l64 = o_bf.double().numpy(), l_32.double().numpy()
    print("mx bwd prod_bcast: library", flush=True)
    dq, dk, dv = _run(jfa, t, True, False, scale, o_bf, l_32)
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert np.all(np.isfinite(x)), f"{name} has non-finite values"
    dOr_all = mo.dequantize_rows(a["do8"], a["do_scale"])                 # [B, H, Lq, d]
    rng = np.random.default_rng(43)
    for b in [int(x) for x in rng.choice(B, size=3, replace=False)]:
        s0, s1, Kr, Kc, Vr = kv[b]
        dOc = mo.dequantize_cols(a["dot8"][b], a["dot_scale"][b], Lq)       # [H, Lq, d]
        for h in range(H):
            g = mo.sequence_backward(Qr[h], Qc[h], Kr[:, h], Kc[:, h], Vr[:, h], dOr_all[b, h], dOc[h], o64[b, h],
                                     l64[b, h], np.arange(Lq), np.arange(s0, s1), scale, False)
            _compare(f"prod_bcast seq {b} head {h} dk", dk[s0:s1, h], g[1], g[4])
            _compare(f"prod_bcast seq {b} head {h} dv", dv[s0:s1, h], g[2], g[5])
    print("mx bwd prod_bcast: dQ rows", flush=True)
    rows = {h: sorted(int(i) for i in rng.choice(Lq, size=2, replace=False)) for h in range(H)}
    f32 = lambda x: np.ascontiguousarray(x, dtype=np.float32)  # dequantized values are exact in float32
    items, where = [], []
    for b in range(B):
        s0, s1, Kr, Kc, Vr = kv[b]
        if s1 == s0:
            continue
        dOc_b = mo.dequantize_cols(a["dot8"][b], a["dot_scale"][b], Lq)
        for h, ri in rows.items():
            items.append((f32(Qr[h, ri]), f32(Qc[h, ri]), f32(Kr[:, h]), f32(Kc[:, h]), f32(Vr[:, h]),
                          f32(dOr_all[b, h, ri]), f32(dOc_b[h, ri]), o64[b, h, ri], l64[b, h, ri], ri,
                          np.arange(s0, s1), scale, False))
            where.append(h)
    ref = {h: np.zeros((2, 128)) for h in range(H)}
    allow = {h: np.zeros((2, 128)) for h in range(H)}
    for k, g in run_calls("oracle.mx_oracle", "sequence_backward", items, [len(x[2]) for x in items]):
        ref[where[k]] += g[0]
        allow[where[k]] += g[3]
    for h, ri in rows.items():
        for r, i in enumerate(ri):
            _compare(f"prod_bcast dq head {h} row {i}", dq[h, i], ref[h][r], allow[h][r])


def test_mx_forward_backward_long_causal_sampled(jfa):
    """long_causal_8k's shapes (64 sequences of logU[128, 8192] keys, 16
    heads, self mode, causal) at full size, forward and backward in the
    launch configuration the bench times: every output finite; three
    sequences (the shortest and two near 1.5K keys), two heads each, against
    the oracle.  The backward reads O and lse of the sampled rows from the
    oracle's MXFP8 forward and the library's own forward elsewhere (rows of
    other sequences do not enter these sequences' gradients)."""
    w = wl.workload("long_causal_8k")
    print("mx long_causal_8k: generating", flush=True)
    t = wl.make_mx_bwd_workload(w, device="cuda:0")
    scale = w.scale
    dev = torch.device("cuda:0")
    out, lse = jfa.attention_fwd_mxfp8(t["q8"], t["q_scale"], t["k8"], t["k_scale"], t["vt8"], t["vt_scale"],
                                       t["offsets"], scale, True, False)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
    a = _np(t)
    off = a["offsets"]
    L = np.diff(off)
    seqs = [int(np.argmin(L))] + [int(b) for b in np.argsort(np.abs(L - 1500))[:2]]
    heads = [0, 11]
    Qr = mo.dequantize_rows(a["q8"], a["q_scale"])
    Kr = mo.dequantize_rows(a["k8"], a["k_scale"])
    Vc = mo.dequantize_vt(a["vt8"], a["vt_scale"], t["total_len"])
    out_in, lse_in = out.clone(), lse.clone()
    ref_f = {}
    for b in seqs:
        s0, s1 = int(off[b]), int(off[b + 1])
        for h in heads:
            o, ls, allow = mo.sequence_forward(Qr[s0:s1, h], Kr[s0:s1, h], Vc[s0:s1, h], s0, scale, True)
            _compare(f"long_causal_8k fwd seq {b} (L={s1 - s0}) head {h} O", out[s0:s1, h].float().cpu().double().numpy(),
                     o, allow)
            lerr = float(np.max(np.abs(lse[s0:s1, h].cpu().double().numpy() - ls)))
            assert lerr <= 2e-2, f"lse {lerr:.3e}"
            out_in[s0:s1, h] = torch.from_numpy(o).to(torch.bfloat16).to(dev)
            lse_in[s0:s1, h] = torch.from_numpy(ls).to(torch.float32).to(dev)
    print("mx long_causal_8k: backward", flush=True)
    g = {n: t[n] for n in ENC}
    dq, dk, dv = jfa.attention_bwd_mxfp8(g, t["offsets"], scale, True, False, out_in, lse_in)
    torch.cuda.synchronize()
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(x).all()), f"{name} has non-finite values"
    o64 = out_in.float().cpu().double().numpy()
    l64 = lse_in.cpu().double().numpy()
    deq = mo.dequantize_backward_inputs(a, False)
    for b in seqs:
        s0, s1 = int(off[b]), int(off[b + 1])
        for h in heads:
            r = mo.backward_item(a, deq, o64, l64, b, h, scale, True, False)
            for i, (name, x) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
                _compare(f"long_causal_8k seq {b} (L={s1 - s0}) head {h} {name}",
                         x[s0:s1, h].cpu().double().numpy(), r[i], r[3 + i])
