"""The allocation-free forward entry point, jfa_fwd_noalloc, through the
C-ABI: its output equals jfa_fwd_ex's (same kernels, workspace from torch)
bitwise, on two calls in a row, the second with a smaller input, and meets
the oracle bar."""
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


def _outputs(t, bq, B, H, Lq, d, T):
    shape_o = (B, H, Lq, d) if bq else (T, H, d)
    shape_l = (B, H, Lq) if bq else (T, H)
    return (torch.full(shape_o, float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full(shape_l, float("nan"), dtype=torch.float32, device="cuda"))


def _case(jfa, lengths, H, H_kv, d, Lq, bq, causal, window, seed):
    print(f"noalloc case B={len(lengths)} H={H}/{H_kv} d={d} Lq={Lq} bq={bq} causal={causal} window={window}",
          flush=True)
    t = wl.make_tensors(lengths, H, d, Lq, bq, seed=seed, device="cuda", with_dout=False)
    if H_kv < H:
        t["k"], t["v"] = t["k"][:, :H_kv].contiguous(), t["v"][:, :H_kv].contiguous()
    B, T = len(lengths), int(sum(lengths))
    scale = 1.0 / math.sqrt(d)
    out_a, lse_a = _outputs(t, bq, B, H, Lq, d, T)
    jfa.jfa_fwd_noalloc(t["q"], t["k"], t["v"], t["offsets"], B, H, H_kv, Lq, d, scale, causal, window, bq,
                        out_a, lse_a, T)
    out_b, lse_b = _outputs(t, bq, B, H, Lq, d, T)
    ws = jfa.workspace(T, B, H, Lq, d, causal, bq, 0, "cuda", H_kv=H_kv)
    jfa.jfa_fwd_ex(t["q"], t["k"], t["v"], t["offsets"], B, H, H_kv, Lq, d, scale, causal, window, bq, out_b,
                   lse_b, T, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    ref_o, ref_l = jo.jagged_forward(to64(t["q"]), to64(t["k"]), to64(t["v"]), t["offsets"].cpu().numpy(), scale,
                                     causal, bq, window=window)
    compare("O", to64(out_a), ref_o)
    compare_lse("lse", to64(lse_a), ref_l)


def test_noalloc_forward_two_calls_second_smaller(jfa):
    rng = np.random.default_rng(5)
    big = [int(x) for x in rng.integers(0, 900, size=600)]
    _case(jfa, big, 4, 4, 128, 256, True, False, 0, seed=51)
    small = [int(x) for x in rng.integers(1, 400, size=9)]
    _case(jfa, small, 4, 2, 128, 0, False, True, 100, seed=52)


def test_noalloc_forward_rejects_sizes_beyond_its_scratch(jfa):
    # 1000 heads x (8192 sequences + rows / 256) tiles of 32 bytes: far beyond 16 MiB
    t = wl.make_tensors([3, 5], 2, 128, 0, False, seed=1, device="cuda", with_dout=False)
    out, lse = _outputs(t, False, 2, 2, 0, 128, 8)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        jfa.jfa_fwd_noalloc(t["q"], t["k"], t["v"], t["offsets"], 8192, 1000, 1000, 0, 128, 0.1, 0, 0, 0, out, lse,
                            1 << 30)
