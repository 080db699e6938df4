"""The useful-FLOP convention of bench.py against the numbers the FMHA guide
prints ("cuTile Kernels -- FMHA Implementation", "Performance Results"):
dense attention, 4*head_dim flops per (query, key) pair and head, over the
full S x S, with batch*heads*head_dim = 8192 behind every printed row."""
import os

import numpy as np
import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.strip() and not line.startswith("#"):
            out.append([float(x) for x in line.split()])
    return out


def test_b300_sweep_matches_flop_convention():
    # batch*heads = 64, head_dim = 128: 64 equal-length dense sequences, one head
    # each, i.e. per the library's count 4*d*H*pairs with pairs = sum L^2.
    for seq, ms, tflops in _rows("cutile_b300_fmha_sweep.txt"):
        S = int(seq)
        fwd, _ = bench.useful_flops([S] * 64, 1, 128, 0, False, False)
        assert fwd == 4 * S * S * 8192
        got = fwd / (ms * 1e-3) / 1e12
        assert got == pytest.approx(tflops, rel=0.006), (S, got, tflops)


def test_spark_steps_match_flop_convention():
    fwd, _ = bench.useful_flops([2048] * 64, 1, 128, 0, False, False)
    for _, ms, tflops in _rows("cutile_spark_fmha_steps.txt"):
        assert fwd / (ms * 1e-3) / 1e12 == pytest.approx(tflops, rel=0.015)


def test_visible_pairs_closed_forms():
    L = [1, 5, 64]
    assert bench.visible_pairs(L, 0, True, False) == 1 + 15 + 64 * 65 // 2
    assert bench.visible_pairs(L, 0, False, False) == 1 + 25 + 64 * 64
    assert bench.visible_pairs(L, 7, False, True) == 7 * 70
    # broadcast causal: query i sees min(i+1, L) keys
    assert bench.visible_pairs([3], 5, True, True) == 1 + 2 + 3 + 3 + 3
    assert bench.useful_flops(L, 2, 64, 7, False, True) == (4 * 64 * 2 * 490, 10 * 64 * 2 * 490)


def test_bench_refuses_more_than_one_gpu():
    assert bench.main(["--gpus", "2"]) == 2


@pytest.mark.parametrize("bq", [False, True])
def test_visible_pairs_with_a_window_by_brute_force(bq):
    """Query i sees key j when j <= i, i - W < j and j < L: counted pair by
    pair on small cases, against the closed forms bench.py uses."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        L = [int(x) for x in rng.integers(0, 40, size=5)]
        W = int(rng.integers(1, 50))
        Lq = int(rng.integers(1, 60)) if bq else 0
        n = 0
        for Lb in L:
            for i in range(Lq if bq else Lb):
                n += sum(1 for j in range(Lb) if j <= i and j > i - W)
        assert bench.visible_pairs(L, Lq, True, bq, W) == n
    # a window at least as long as every sequence is the plain causal count
    assert bench.visible_pairs([5, 9], 12, True, bq, 64) == bench.visible_pairs([5, 9], 12, True, bq)


def test_kernel_names_map_to_timing_labels():
    """rocprofv3 kernel names (templates, anonymous namespace) map to the
    library's timing labels the traffic summaries are keyed by."""
    names = {
        "void jfa::(anonymous namespace)::fwd_kernel_dma<128, 8, 32, false, true>(jfa::FwdArgs, jfa::TileRec const*)":
            "fwd_kernel",
        "void jfa::(anonymous namespace)::fwd_kernel<64, 8, 32, true, false>(jfa::FwdArgs)": "fwd_kernel",
        "void jfa::(anonymous namespace)::dkdv_pair_kernel<false, true>(jfa::BwdArgs, jfa::TileRec const*)":
            "dkdv_kernel",
        "void jfa::(anonymous namespace)::dq_bcast_kernel<128, false>(jfa::BwdArgs)": "dq_kernel",
        "void jfa::(anonymous namespace)::dq_reduce<64>(float const*, float*, int, int, int, int, int)": "dq_reduce",
        "jfa::(anonymous namespace)::sched_expand(jfa::SchedArgs, jfa::Schedule)": None,
        "__amd_rocclr_copyBuffer": None,
    }
    for n, lab in names.items():
        assert bench.label_of(n) == lab, n


def test_committed_traffic_summaries_parse():
    """Every committed traffic summary names a timing label and holds a byte
    count per launch; measured_traffic reads it while the sources match."""
    d = bench.PROFILE_DIR
    files = [f for f in os.listdir(d) if f.startswith("traffic_") and f.endswith(".txt")]
    assert files
    for f in files:
        stem = f[len("traffic_"):-len(".txt")]
        label = next((k for k in bench.LABEL_SYMBOLS if stem.startswith(k + "_")), None)
        assert label is not None, f
        vals = dict(line.split(":", 1) for line in open(os.path.join(d, f)) if ":" in line and not line.startswith("#"))
        assert float(vals["hbm_bytes_per_launch"]) > 0
        if vals["source_digest"].strip() == bench.kernel_source_digest():
            assert bench.measured_traffic(label, stem[len(label) + 1:]) == float(vals["hbm_bytes_per_launch"])
