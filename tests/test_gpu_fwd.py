"""GPU parity of jfa_fwd (called through the C-ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest

import workloads as wl
from oracle import jfa_oracle as jo
from oracle import schedule_ref as sr
from tests._parity import compare, compare_lse, to64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# Tile geometry this test expects of the library (checked against the
# library's own report before use).
def fwd_bm(bq, causal):
    """Query rows of a forward tile (every mode)."""
    return 256
BWD_BN = 128


@pytest.fixture(scope="module")
def jfa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import jagged_flashattention_fwd_amd as m
    m.lib()
    return m


def _run_case(jfa, lengths, H, d, Lq, bq, causal, seed, std=1.0, scale=None):
    t = wl.make_tensors(lengths, H, d, Lq, bq, std=std, seed=seed, device="cuda", with_dout=False)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    print(f"fwd case lengths={list(lengths)[:8]}.. H={H} d={d} Lq={Lq} bq={bq} causal={causal}",
          flush=True)
    out, lse = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], scale, causal, bq)
    torch.cuda.synchronize()
    ref_o, ref_lse = jo.jagged_forward(to64(t["q"]), to64(t["k"]), to64(t["v"]),
                                       t["offsets"].cpu().numpy(), scale, causal, bq)
    compare("O", to64(out), ref_o)
    compare_lse("lse", to64(lse), ref_lse)
    return t, out, lse


EDGE = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 0, 255, 256, 257, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bq,causal", [(True, False), (True, True), (False, False), (False, True)])
def test_fwd_edge_lengths(jfa, d, bq, causal):
    _run_case(jfa, EDGE, 2, d, 70 if bq else 0, bq, causal, seed=11)


@pytest.mark.parametrize("Lq", [1, 32, 255, 256, 257, 512])
def test_fwd_broadcast_lq(jfa, Lq):
    _run_case(jfa, [5, 130, 1, 64, 700], 3, 128, Lq, True, False, seed=Lq)


def test_fwd_negative_and_zero_scale(jfa):
    _run_case(jfa, [3, 77, 130], 2, 64, 40, True, False, seed=5, scale=-0.3)
    _run_case(jfa, [3, 77, 130], 2, 128, 0, False, True, seed=6, scale=0.0)


@pytest.mark.parametrize("bq,causal", [(True, False), (True, True), (False, False), (False, True)])
def test_fwd_negative_scale_d128(jfa, bq, causal):
    """A negative scale turns the running maximum into the minimum of the
    raw scores: the d = 128 kernel's branch for it, in every mode."""
    _run_case(jfa, [3, 77, 130, 300, 1], 2, 128, 70 if bq else 0, bq, causal, seed=7, scale=-0.3)


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True)])
def test_fwd_single_sequence(jfa, bq, causal):
    """B = 1: one sequence (several tiles of it in self mode)."""
    _run_case(jfa, [777], 3, 128, 300 if bq else 0, bq, causal, seed=8)


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True)])
def test_fwd_sequence_permutation(jfa, bq, causal):
    """Permuting the order of the sequences permutes O and lse the same way,
    bitwise (each output row is computed from its own sequence only)."""
    lengths = [300, 1, 64, 129, 0, 700, 33, 256]
    H, d, Lq = 2, 128, 100
    t = wl.make_tensors(lengths, H, d, Lq if bq else 0, bq, seed=12, device="cuda", with_dout=False)
    perm = [5, 2, 7, 0, 4, 1, 6, 3]
    off = t["offsets"].cpu().numpy()
    plen = [lengths[p] for p in perm]
    poff = torch.from_numpy(wl.offsets_from_lengths(plen)).cuda()
    rows = torch.cat([torch.arange(int(off[p]), int(off[p + 1])) for p in perm]).cuda()
    k, v = t["k"][rows].contiguous(), t["v"][rows].contiguous()
    q = t["q"] if bq else t["q"][rows].contiguous()
    o1, l1 = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.09, causal, bq)
    o2, l2 = jfa.attention_fwd(q, k, v, poff, 0.09, causal, bq)
    torch.cuda.synchronize()
    if bq:
        assert torch.equal(o2, o1[perm]) and torch.equal(l2, l1[perm])
    else:
        assert torch.equal(o2, o1[rows]) and torch.equal(l2, l1[rows])


@pytest.mark.parametrize("lengths", [[512] * 5, [1000] * 3])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_dense_equal_lengths(jfa, lengths, causal):
    """The dense LLM regime at reduced batch: equal lengths in self mode
    (a whole number of tiles, and a ragged tail)."""
    _run_case(jfa, lengths, 4, 128, 0, False, causal, seed=len(lengths) + 40)


@pytest.mark.parametrize("idx", [0, 1])
def test_fwd_workloads_full(jfa, idx):
    w = wl.workload(idx)
    lengths = wl.draw_lengths(w.lengths, w.B, idx)
    _run_case(jfa, lengths, w.H, w.d, w.Lq, w.broadcast_q, w.causal, seed=idx, std=w.std)


def test_single_key_sequences_return_v_bitwise(jfa):
    lengths = [1, 1, 5, 1]
    H, d, Lq = 2, 128, 33
    t = wl.make_tensors(lengths, H, d, Lq, True, seed=3, device="cuda", with_dout=False)
    out, _ = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.1, False, True)
    off = t["offsets"].cpu().numpy()
    for b in (0, 1, 3):
        v = t["v"][off[b]]  # [H, d]
        assert torch.equal(out[b], v[:, None, :].expand(H, Lq, d))
    # causal self-attention: row 0 of every sequence returns V row 0
    t = wl.make_tensors([7, 1, 130], H, d, 0, False, seed=4, device="cuda", with_dout=False)
    out, _ = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.1, True, False)
    for s in t["offsets"].cpu().numpy()[:-1]:
        assert torch.equal(out[s], t["v"][s])


def test_fwd_deterministic(jfa):
    t = wl.make_tensors([300, 17, 900, 64], 4, 128, 256, True, seed=9, device="cuda", with_dout=False)
    a = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.08, False, True)
    b = jfa.attention_fwd(t["q"], t["k"], t["v"], t["offsets"], 0.08, False, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("bq,causal", [(True, False), (False, True)])
def test_fwd_dynamic_handout_reused_workspace(jfa, bq, causal):
    """More tiles than two per workgroup, so most come from the hand-out
    counter; three calls on one workspace into NaN-filled outputs must each
    cover every tile once (the counter restarts per call) and agree bitwise."""
    rng = np.random.default_rng(21)
    lengths = [int(x) for x in rng.integers(1, 300, size=700 if bq else 900)]
    H, d, Lq = 2, 128, (300 if bq else 0)
    t = wl.make_tensors(lengths, H, d, Lq, bq, seed=21, device="cuda", with_dout=False)
    B, T = len(lengths), int(sum(lengths))
    n_tiles = B * H * -(-Lq // fwd_bm(bq, causal)) if bq else H * sum(-(-L // fwd_bm(bq, causal)) for L in lengths)
    assert n_tiles > 2 * torch.cuda.get_device_properties(0).multi_processor_count
    ws = jfa.workspace(T, B, H, Lq, d, causal, bq, 0, "cuda")
    outs = []
    for _ in range(3):
        out = torch.full((B, H, Lq, d) if bq else (T, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H, Lq) if bq else (T, H), float("nan"), dtype=torch.float32, device="cuda")
        jfa.jfa_fwd(t["q"], t["k"], t["v"], t["offsets"], B, H, Lq, d, 0.09, causal, bq, out, lse, T, ws)
        torch.cuda.synchronize()
        outs.append((out, lse))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    ref_o, ref_lse = jo.jagged_forward(to64(t["q"]), to64(t["k"]), to64(t["v"]), t["offsets"].cpu().numpy(),
                                       0.09, causal, bq)
    compare("O", to64(outs[0][0]), ref_o)
    compare_lse("lse", to64(outs[0][1]), ref_lse)


@pytest.mark.parametrize("pass_", [0, 1])
@pytest.mark.parametrize("bq,causal", [(True, 0), (False, 0), (False, 1)])
def test_schedule_bit_exact(jfa, pass_, bq, causal):
    lengths = wl.draw_lengths(("mix", 0.1, (0, 40), (300, 3000)), 777, 21)
    H, Lq = 3, 300
    block, P = jfa.jfa_schedule_params(pass_, causal, int(bq), 128)
    props = torch.cuda.get_device_properties(0)
    expect_block = fwd_bm(bq, causal) if pass_ == 0 else BWD_BN
    assert (block, P) == (expect_block, props.multi_processor_count)
    off = torch.from_numpy(wl.offsets_from_lengths(lengths)).cuda()
    T = int(off[-1])
    ws = jfa.workspace(T, len(lengths), H, Lq if bq else 0, 128, 0, bq, pass_, "cuda")
    ref = sr.schedule(lengths, H, Lq if bq else 0, bq, pass_, expect_block, expect_block,
                      props.multi_processor_count)
    cap = len(ref) + 5
    tiles = torch.full((cap, 4), -7, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int64, device="cuda")
    jfa.jfa_debug_schedule(off, len(lengths), H, Lq if bq else 0, causal, bq, pass_, T, tiles, n, ws)
    torch.cuda.synchronize()
    assert int(n.item()) == len(ref)
    got = tiles.cpu().numpy()
    assert np.array_equal(got[:len(ref)], np.array(ref, dtype=np.int32))
    assert np.all(got[len(ref):] == -7)


DQ_BM = 256  # query rows of the self-attention backward's dQ tiles


@pytest.mark.parametrize("list_", [0, 1, 2])
@pytest.mark.parametrize("name", ["tiny_bcast", "self_causal_1k", "prod_bcast", "long_causal_8k", "skew_bcast",
                                  "prod_bcast_gqa", "dense_llm_1k"])
def test_schedule_bit_exact_on_workload_offsets(jfa, name, list_):
    """Every tile list the library builds (forward query tiles, backward key
    tiles, self-attention dQ query tiles), on each workload's own seeded
    offsets, equals the integer reference, key / value head included."""
    w = wl.workload(name)
    if list_ == 2 and w.broadcast_q:
        pytest.skip("the dQ query-tile list exists in self-attention mode only")
    lengths = wl.draw_lengths(w.lengths, w.B, wl.WORKLOADS.index(w))
    B, H, Hkv, Lq, bq = w.B, w.H, w.kv_heads, w.Lq, w.broadcast_q
    block, P = jfa.jfa_schedule_params(1 if list_ == 1 else 0, w.causal, int(bq), w.d)
    assert block == (BWD_BN if list_ == 1 else fwd_bm(bq, w.causal))
    blk = {0: fwd_bm(bq, w.causal), 1: BWD_BN, 2: DQ_BM}[list_]
    off = torch.from_numpy(wl.offsets_from_lengths(lengths)).cuda()
    T = int(off[-1])
    ws = jfa.workspace(T, B, H, Lq, w.d, w.causal, bq, 0 if list_ == 0 else 1, "cuda", H_kv=Hkv)
    ref = sr.schedule(lengths, Hkv if list_ == 1 else H, Lq, bq, 1 if list_ == 1 else 0, blk, blk, P, G=H // Hkv)
    cap = len(ref) + 3
    tiles = torch.full((cap, 5), -7, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int64, device="cuda")
    jfa.jfa_debug_schedule_ex(off, B, H, Hkv, Lq, w.causal, bq, list_, T, tiles, n, ws)
    torch.cuda.synchronize()
    print(f"schedule {name} list {list_}: {len(ref)} tiles", flush=True)
    assert int(n.item()) == len(ref)
    got = tiles.cpu().numpy()
    assert np.array_equal(got[:len(ref)], np.array(ref, dtype=np.int32))
    assert np.all(got[len(ref):] == -7)
