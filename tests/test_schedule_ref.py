"""Pins of the integer schedule reference: every tile exactly once, closed-form
counts, longest-first order and the zigzag hand-out ("Optimizing Jagged Flash
Attention with TLX", "Scheduling jagged tiles across SMs")."""
import itertools

import numpy as np
import pytest

from oracle import schedule_ref as sr


def _expected_tiles(lengths, H, Lq, broadcast_q, pass_, BM, BN):
    """Brute force: every (b, h, block) whose block holds at least one query
    row (forward) or key row (backward), found by scanning rows one by one."""
    out = set()
    for b, L in enumerate(lengths):
        for h in range(H):
            if pass_ == 0:
                n_rows = Lq if broadcast_q else L
                for r in range(n_rows):
                    out.add((b, h, r // BM))
            else:
                for r in range(L):
                    out.add((b, h, r // BN))
    return out


CASES = [
    ([5, 0, 17, 3, 17, 1], 2, 9, True, 4, 8),
    ([5, 0, 17, 3, 17, 1], 3, 0, False, 4, 8),
    ([64, 63, 65, 128, 1, 2, 0], 1, 64, True, 64, 32),
    ([1000, 7, 513, 512, 0], 4, 0, False, 128, 64),
]


@pytest.mark.parametrize("pass_", [0, 1])
@pytest.mark.parametrize("lengths,H,Lq,bq,BM,BN", CASES)
def test_every_tile_exactly_once(lengths, H, Lq, bq, BM, BN, pass_):
    tiles = sr.schedule(lengths, H, Lq, bq, pass_, BM, BN, P=5)
    triples = [t[:3] for t in tiles]
    assert len(triples) == len(set(triples))
    assert set(triples) == _expected_tiles(lengths, H, Lq, bq, pass_, BM, BN)


def test_closed_form_counts_equal_lengths():
    B, H, Lq, L, BM, BN = 7, 3, 100, 300, 32, 64
    lengths = [L] * B
    assert len(sr.schedule(lengths, H, Lq, True, 0, BM, BN, 4)) == B * H * 4      # cdiv(100, 32)
    assert len(sr.schedule(lengths, H, 0, False, 0, BM, BN, 4)) == B * H * 10     # cdiv(300, 32)
    assert len(sr.schedule(lengths, H, Lq, True, 1, BM, BN, 4)) == B * H * 5      # cdiv(300, 64)


def test_longest_first_and_stable():
    lengths = [3, 9, 9, 1, 0, 9, 4]
    tiles = sr.schedule(lengths, 2, 8, True, 0, 4, 4, P=3)
    seq = [t[0] for t in tiles]
    firsts = [b for b, _ in itertools.groupby(seq)]
    assert firsts == [1, 2, 5, 6, 0, 3, 4]
    lens = [lengths[b] for b in seq]
    assert all(a >= b for a, b in zip(lens, lens[1:]))


def test_block_order_inside_sequence():
    tiles = sr.schedule([10], 2, 0, False, 0, 4, 4, P=2)
    assert [t[1:3] for t in tiles] == [(0, 2), (0, 1), (0, 0), (1, 2), (1, 1), (1, 0)]
    tiles = sr.schedule([10], 2, 0, False, 1, 4, 4, P=2)
    assert [t[1:3] for t in tiles] == [(0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (1, 2)]


@pytest.mark.parametrize("P", [1, 2, 5, 8])
def test_zigzag(P):
    T = 4 * P + 3
    slots = [sr.zigzag_slot(t, P) for t in range(T)]
    for p in range(T // P):
        chunk = slots[p * P:(p + 1) * P]
        assert sorted(chunk) == list(range(P))
        assert chunk == (list(range(P)) if p % 2 == 0 else list(range(P - 1, -1, -1)))
    # a slot's tile count differs by at most one from any other slot's
    counts = np.bincount(slots, minlength=P)
    assert counts.max() - counts.min() <= 1


def test_broadcast_backward_is_head_major():
    lengths = [300, 5, 129]
    tiles = sr.schedule(lengths, 3, 16, True, 1, 64, 128, P=4)
    heads = [t[1] for t in tiles]
    assert heads == sorted(heads)
    # within a head: sequences longest first, blocks ascending
    h0 = [(t[0], t[2]) for t in tiles if t[1] == 0]
    assert h0 == [(0, 0), (0, 1), (0, 2), (2, 0), (2, 1), (1, 0)]
    # self-attention backward keeps the sequence-major order
    tiles = sr.schedule(lengths, 3, 0, False, 1, 64, 128, P=4)
    assert [t[:3] for t in tiles[:4]] == [(0, 0, 0), (0, 0, 1), (0, 0, 2), (0, 1, 0)]
