"""GPU parity of jfa_bwd (called through the C-ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import jfa_oracle as jo
from tests._parity import compare, to64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import jagged_flashattention_fwd_amd as m
    m.lib()
    return m


def _run(jfa, t, bq, causal, scale):
    out, lse = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], scale, causal, bq)
    dq, dk, dv = jfa.attention_bwd(t["q"], t["k"], t["v"], t["offsets"], scale, causal, bq, out, lse,
                                   t["dout"])
    torch.cuda.synchronize()
    return dq, dk, dv


def _check_case(jfa, lengths, H, d, Lq, bq, causal, seed, std=1.0, scale=None):
    print(f"bwd case lengths={list(lengths)[:8]}.. H={H} d={d} Lq={Lq} bq={bq} causal={causal}",
          flush=True)
    t = wl.make_tensors(lengths, H, d, Lq, bq, std=std, seed=seed, device="cuda")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq, dk, dv = _run(jfa, t, bq, causal, scale)
    rq, rk, rv = jo.jagged_backward(to64(t["q"]), to64(t["k"]), to64(t["v"]),
                                    t["offsets"].cpu().numpy(), scale, causal, bq, to64(t["dout"]))
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        ma, rl = compare(name, to64(got), ref)
        print(f"  {name}: max abs {ma:.2e}  rel L2 {rl:.2e}", flush=True)


EDGE = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 0, 255, 256, 257, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bq,causal", [(True, False), (True, True), (False, False), (False, True)])
def test_bwd_edge_lengths(jfa, d, bq, causal):
    _check_case(jfa, EDGE, 2, d, 70 if bq else 0, bq, causal, seed=21)


@pytest.mark.parametrize("Lq", [1, 32, 63, 64, 65, 256, 300])
def test_bwd_broadcast_lq(jfa, Lq):
    _check_case(jfa, [5, 130, 1, 64, 700, 129], 3, 128, Lq, True, False, seed=100 + Lq)


# Short sequences against many broadcast queries (the regime of skew_bcast's
# short sequences): P and dS are large, and dV / dK sum their rounding over
# all 512 queries.
@pytest.mark.parametrize("std", [0.5, 1.0])
def test_bwd_short_sequences_many_queries(jfa, std):
    _check_case(jfa, [2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 1, 7], 2, 128, 512, True, False, seed=31, std=std)


def test_bwd_broadcast_dq_many_chunks(jfa):
    """One head and more sequences than compute units: the broadcast dQ runs
    256 sequence chunks and sums their partials with a 256-leaf tree."""
    lengths = wl.draw_lengths(("uniform", 1, 90), 300, 77)
    _check_case(jfa, lengths, 1, 128, 64, True, False, seed=77)


@pytest.mark.parametrize("lengths", [[512] * 5, [1000] * 3])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_equal_lengths(jfa, lengths, causal):
    """The dense LLM regime at reduced batch: equal lengths in self mode
    (a whole number of tiles, and a ragged tail)."""
    _check_case(jfa, lengths, 4, 128, 0, False, causal, seed=len(lengths) + 40)


@pytest.mark.parametrize("idx", [0, 1])
def test_bwd_workloads_full(jfa, idx):
    w = wl.workload(idx)
    lengths = wl.draw_lengths(w.lengths, w.B, idx)
    _check_case(jfa, lengths, w.H, w.d, w.Lq, w.broadcast_q, w.causal, seed=idx, std=w.std)


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True)])
def test_bwd_bitwise_deterministic(jfa, bq, causal):
    t = wl.make_tensors([300, 17, 900, 64, 1, 513], 4, 128, 256 if bq else 0, bq, seed=9, device="cuda")
    a = _run(jfa, t, bq, causal, 0.08)
    b = _run(jfa, t, bq, causal, 0.08)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("bq,causal", [(True, True), (False, True), (False, False)])
def test_bwd_dynamic_handout_reused_workspace(jfa, bq, causal):
    """Causal or self-attention tiles come from hand-out counters past each
    workgroup's first zigzag tiles: with more tiles than that, three calls on
    one workspace into NaN-filled outputs must each cover every tile once and
    agree bitwise, and match the oracle."""
    rng = np.random.default_rng(33)
    lengths = [int(x) for x in rng.integers(1, 300 if not bq else 400, size=500)]
    H, d, Lq = 2, 128, (200 if bq else 0)
    t = wl.make_tensors(lengths, H, d, Lq, bq, seed=33, device="cuda")
    B, T = len(lengths), int(sum(lengths))
    assert H * sum(-(-L // 128) for L in lengths) > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    scale = 0.09
    out, lse = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], scale, causal, bq)
    ws = jfa.workspace(T, B, H, Lq, d, causal, bq, 1, "cuda")
    res = []
    for _ in range(3):
        dq = torch.full(tuple(t["q"].shape), float("nan"), dtype=torch.float32, device="cuda")
        dk = torch.full((T, H, d), float("nan"), dtype=torch.float32, device="cuda")
        dv = torch.full((T, H, d), float("nan"), dtype=torch.float32, device="cuda")
        jfa.jfa_bwd(t["q"], t["k"], t["v"], t["offsets"], B, H, Lq, d, scale, causal, bq, out, lse, t["dout"],
                    dq, dk, dv, T, ws)
        torch.cuda.synchronize()
        res.append((dq, dk, dv))
    for r in res[1:]:
        for x, y in zip(res[0], r):
            assert torch.equal(x, y)
    rq, rk, rv = jo.jagged_backward(to64(t["q"]), to64(t["k"]), to64(t["v"]), t["offsets"].cpu().numpy(), scale,
                                    causal, bq, to64(t["dout"]))
    for name, got, ref in (("dQ", res[0][0], rq), ("dK", res[0][1], rk), ("dV", res[0][2], rv)):
        compare(name, to64(got), ref)


def test_bwd_single_key_dv_is_column_sum_of_dout(jfa):
    # One key: P = 1 for every query, so dV = sum of dO over the query rows
    # and dK = 0 (dS = P (dP - delta) = 0 when delta = dP).
    lengths = [1, 3, 1]
    H, d, Lq = 2, 128, 40
    t = wl.make_tensors(lengths, H, d, Lq, True, seed=17, device="cuda")
    dq, dk, dv = _run(jfa, t, True, False, 0.1)
    off = t["offsets"].cpu().numpy()
    for b in (0, 2):
        ref = to64(t["dout"][b]).sum(axis=1)  # [H, d]
        np.testing.assert_allclose(to64(dv[off[b]]), ref, rtol=1e-5, atol=1e-4)
        assert float(dk[off[b]].abs().max()) < 1e-3


@pytest.mark.parametrize("bq,causal", [(True, False), (True, True), (False, False), (False, True)])
def test_bwd_negative_scale_d128(jfa, bq, causal):
    """Negative scale on the d = 128 kernels (the row terms -lse / scale
    change sign, and the forward keeps the minimum raw score), at the
    workloads' magnitude 1/sqrt(d).  (At |scale| = 0.3 the softmax is 3.4x
    sharper and dQ / dK reach max-abs 6e-2 for either sign, rel-L2 2.7e-3:
    the rounding of delta from the bf16 output, not the sign.)"""
    _check_case(jfa, [3, 77, 130, 300, 1], 2, 128, 70 if bq else 0, bq, causal, seed=7, scale=-1.0 / math.sqrt(128))


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True)])
def test_bwd_single_sequence(jfa, bq, causal):
    """B = 1: one sequence, several key tiles."""
    _check_case(jfa, [777], 3, 128, 300 if bq else 0, bq, causal, seed=8)


def test_bwd_rejects_zero_scale(jfa):
    t = wl.make_tensors([5, 9], 2, 128, 16, True, seed=3, device="cuda")
    out, lse = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.0, False, True)
    with pytest.raises(RuntimeError, match="INVALID_ARG"):
        jfa.attention_bwd(t["q"], t["k"], t["v"], t["offsets"], 0.0, False, True, out, lse, t["dout"])


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True)])
def test_bwd_sequence_permutation(jfa, bq, causal):
    """Permuting the order of the sequences permutes dK, dV (and self-mode
    dQ) the same way, bitwise; the broadcast dQ, a sum over sequences taken
    in length order (all lengths distinct here), is unchanged bitwise."""
    lengths = [300, 1, 64, 129, 0, 700, 33, 256]
    H, d, Lq = 2, 128, 100
    t = wl.make_tensors(lengths, H, d, Lq if bq else 0, bq, seed=12, device="cuda")
    perm = [5, 2, 7, 0, 4, 1, 6, 3]
    off = t["offsets"].cpu().numpy()
    plen = [lengths[p] for p in perm]
    pt = {"offsets": torch.from_numpy(wl.offsets_from_lengths(plen)).cuda()}
    rows = torch.cat([torch.arange(int(off[p]), int(off[p + 1])) for p in perm]).cuda()
    pt["k"], pt["v"] = t["k"][rows].contiguous(), t["v"][rows].contiguous()
    pt["q"] = t["q"] if bq else t["q"][rows].contiguous()
    pt["dout"] = t["dout"][perm].contiguous() if bq else t["dout"][rows].contiguous()
    a = _run(jfa, t, bq, causal, 0.09)
    b = _run(jfa, pt, bq, causal, 0.09)
    if bq:
        assert torch.equal(b[0], a[0])
    else:
        assert torch.equal(b[0], a[0][rows])
    assert torch.equal(b[1], a[1][rows]) and torch.equal(b[2], a[2][rows])
