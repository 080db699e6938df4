"""GPU parity of grouped-query attention (jfa_fwd_gqa / jfa_bwd_gqa through
the C-ABI) against the fp64 oracle: key / value heads shared by groups of
consecutive query heads, dK / dV summed over each group."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import jfa_oracle as jo
from tests._parity import compare, compare_lse, to64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def jfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import jagged_flashattention_fwd_amd as m
    m.lib()
    return m


def _case(jfa, lengths, H, H_kv, d, Lq, bq, causal, seed):
    print(f"gqa case lengths={list(lengths)[:8]}.. H={H} H_kv={H_kv} d={d} Lq={Lq} bq={bq} causal={causal}",
          flush=True)
    t = wl.make_tensors(lengths, H, d, Lq, bq, seed=seed, device="cuda")
    k = t["k"][:, :H_kv].contiguous()
    v = t["v"][:, :H_kv].contiguous()
    scale = 1.0 / math.sqrt(d)
    out, lse = jfa.attention_fwd(t["q"], k, v, t["offsets"], scale, causal, bq)
    dq, dk, dv = jfa.attention_bwd(t["q"], k, v, t["offsets"], scale, causal, bq, out, lse, t["dout"])
    torch.cuda.synchronize()
    off = t["offsets"].cpu().numpy()
    ro, rl = jo.jagged_forward(to64(t["q"]), to64(k), to64(v), off, scale, causal, bq)
    compare("O", to64(out), ro)
    compare_lse("lse", to64(lse), rl)
    rq, rk, rv = jo.jagged_backward(to64(t["q"]), to64(k), to64(v), off, scale, causal, bq, to64(t["dout"]))
    assert dk.shape == (int(off[-1]), H_kv, d)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, to64(got), ref)
    return out, lse, dq, dk, dv


EDGE = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 0, 255, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bq,causal", [(True, False), (True, True), (False, False), (False, True)])
@pytest.mark.parametrize("H,H_kv", [(4, 2), (3, 1)])
def test_gqa_edge_lengths(jfa, d, bq, causal, H, H_kv):
    _case(jfa, EDGE, H, H_kv, d, 70 if bq else 0, bq, causal, seed=5)


def test_gqa_many_sequences_broadcast(jfa):
    rng = np.random.default_rng(8)
    lengths = [int(x) for x in rng.integers(1, 600, size=120)]
    _case(jfa, lengths, 8, 2, 128, 256, True, False, seed=8)


def test_gqa_with_one_group_per_head_is_the_plain_call(jfa):
    """H_kv = H through the grouped entry points equals the plain calls bitwise."""
    lengths = [5, 300, 64, 129]
    H, d, Lq = 2, 128, 96
    t = wl.make_tensors(lengths, H, d, Lq, True, seed=3, device="cuda")
    B, T = len(lengths), int(sum(lengths))
    o1, l1 = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.1, False, True)
    ws = jfa.workspace(T, B, H, Lq, d, False, True, 0, "cuda")
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    jfa.jfa_fwd(t["q"], t["k"], t["v"], t["offsets"], B, H, Lq, d, 0.1, False, True, o2, l2, T, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
