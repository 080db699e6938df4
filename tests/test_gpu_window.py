"""GPU parity of the causal sliding window (jfa_fwd_ex / jfa_bwd_ex through
the C-ABI) against the fp64 oracle: query i sees keys i - W < j <= i; in
broadcast mode rows past the last key's window see nothing (O = 0,
lse = -inf, no gradient)."""
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


def _case(jfa, lengths, H, H_kv, d, Lq, bq, window, seed):
    print(f"window case lengths={list(lengths)[:8]}.. H={H} H_kv={H_kv} d={d} Lq={Lq} bq={bq} W={window}",
          flush=True)
    t = wl.make_tensors(lengths, H, d, Lq, bq, seed=seed, device="cuda")
    k = t["k"][:, :H_kv].contiguous()
    v = t["v"][:, :H_kv].contiguous()
    scale = 1.0 / math.sqrt(d)
    out, lse = jfa.attention_fwd(t["q"], k, v, t["offsets"], scale, True, bq, window=window)
    dq, dk, dv = jfa.attention_bwd(t["q"], k, v, t["offsets"], scale, True, bq, out, lse, t["dout"],
                                   window=window)
    torch.cuda.synchronize()
    off = t["offsets"].cpu().numpy()
    ro, rl = jo.jagged_forward(to64(t["q"]), to64(k), to64(v), off, scale, True, bq, window=window)
    compare("O", to64(out), ro)
    compare_lse("lse", to64(lse), rl)
    rq, rk, rv = jo.jagged_backward(to64(t["q"]), to64(k), to64(v), off, scale, True, bq, to64(t["dout"]),
                                    window=window)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        compare(name, to64(got), ref)
    return rl


EDGE = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 0, 255, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bq", [True, False])
@pytest.mark.parametrize("window", [1, 17, 64, 100, 300])
def test_window_edge_lengths(jfa, d, bq, window):
    rl = _case(jfa, EDGE, 2, 2, d, 290 if bq else 0, bq, window, seed=11)
    if bq and window < 290:
        assert np.isneginf(rl).any()  # some broadcast rows see no key


@pytest.mark.parametrize("bq", [True, False])
def test_window_grouped_query_heads(jfa, bq):
    _case(jfa, EDGE, 4, 2, 128, 160 if bq else 0, bq, 48, seed=12)


def test_window_many_sequences_broadcast(jfa):
    rng = np.random.default_rng(13)
    lengths = [int(x) for x in rng.integers(1, 900, size=80)]
    _case(jfa, lengths, 4, 4, 128, 256, True, 200, seed=13)


def test_window_many_sequences_self(jfa):
    rng = np.random.default_rng(14)
    lengths = [int(x) for x in rng.integers(1, 900, size=40)]
    _case(jfa, lengths, 2, 2, 128, 0, False, 130, seed=14)


def test_window_wider_than_every_sequence_is_causal(jfa):
    """A window of at least the longest sequence masks nothing beyond the
    causal rule: the result is the plain causal one up to rounding."""
    t = wl.make_tensors(EDGE, 2, 128, 0, False, seed=15, device="cuda")
    scale = 1.0 / math.sqrt(128)
    o1, l1 = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], scale, True, False, window=400)
    o0, l0 = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], scale, True, False)
    torch.cuda.synchronize()
    compare("O", to64(o1), to64(o0), max_abs=8e-3, rel_l2=2e-3)
    compare_lse("lse", to64(l1), to64(l0), max_abs=1e-4)


def test_window_without_causal_is_rejected(jfa):
    t = wl.make_tensors([5, 9], 2, 128, 0, False, seed=16, device="cuda")
    with pytest.raises(RuntimeError):
        jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.1, False, False, window=4)
