"""Integer reference for the persistent tile schedule.  TEST INFRASTRUCTURE.

Only tests/ may use this module; it shares no code with the HIP library.

What the schedule follows ("Optimizing Jagged Flash Attention with TLX",
"Scheduling jagged tiles across SMs"): in the forward a tile's cost grows
with its sequence's key length, so work is sorted by K/V workload, longest
first, and handed to the persistent workers in a zigzag (boustrophedon):
even passes fill workers left to right, odd passes right to left.  The
backward's tiles are (batch, head, K/V block) triples of a valid-tile list,
block-innermost so consecutive tiles reuse the same data.

The rules, in the order they are applied (tile sizes BM, BN and the worker
count P are parameters; tie-breaks are this library's reading):
  1. L_b = offsets[b+1] - offsets[b].
  2. Sequence order: by L_b descending; equal lengths keep ascending b.
  3. Tiles per sequence:
       forward, broadcast Q:   H * cdiv(Lq, BM)   (also when L_b == 0: those
                               tiles write O = 0, lse = -inf)
       forward, self:          H * cdiv(L_b, BM)
       backward (both modes):  H * cdiv(L_b, BN)
  4. The sequences' tiles are concatenated in that order (an exclusive
     prefix sum of the counts gives each sequence's first tile).  Inside a
     sequence: heads ascending, and for each head the blocks in cost order,
     heaviest first -- forward query blocks descending (a causal query
     block sees more keys the later it is), backward key blocks ascending
     (a causal key block is seen by more query blocks the earlier it is).
     Broadcast-Q backward only: the list is head-major instead -- all of
     head 0's tiles (sequences in the order of rule 2, blocks ascending),
     then head 1's, and so on.
  5. Tile t goes to worker slot: pass p = t // P, s = t % P,
     slot = s if p is even else P - 1 - s.
  6. With grouped-query heads (G query heads per key/value head), a tile
     of query head h reads key/value head h // G.  The backward's key tiles
     are per key/value head instead (one tile covers the G query heads of
     its group): rules 3-5 with H // G heads, each tile recorded with the
     group's first query head hk * G and hk.

The self-attention backward's dQ pass walks query tiles by the forward's
rules (pass 0) with its own block size.
"""
from __future__ import annotations


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def sequence_order(lengths) -> list:
    return sorted(range(len(lengths)), key=lambda b: (-int(lengths[b]), b))


def tiles_of_sequence(L: int, H: int, Lq: int, broadcast_q: bool, pass_: int, BM: int, BN: int):
    """(h, block) pairs of one sequence, in schedule order."""
    if pass_ == 0:
        nblk = cdiv(Lq, BM) if broadcast_q else cdiv(L, BM)
        blocks = list(range(nblk - 1, -1, -1))
    else:
        nblk = cdiv(L, BN)
        blocks = list(range(nblk))
    return [(h, blk) for h in range(H) for blk in blocks]


def zigzag_slot(t: int, P: int) -> int:
    p, s = divmod(t, P)
    return s if p % 2 == 0 else P - 1 - s


def schedule(lengths, H: int, Lq: int, broadcast_q: bool, pass_: int, BM: int, BN: int, P: int,
             G: int = 0):
    """Full tile list in tile order t = 0, 1, ...: [(b, h, block, slot), ...],
    or with G > 0 query heads per key/value head [(b, h, block, h // G,
    slot), ...]; for the backward's key tiles (pass 1) with G > 0, H counts
    key/value heads and the records are (b, hk * G, block, hk, slot)."""
    triples = []
    for b in sequence_order(lengths):
        for (h, blk) in tiles_of_sequence(int(lengths[b]), H, Lq, broadcast_q, pass_, BM, BN):
            triples.append((b, h, blk))
    if pass_ == 1 and broadcast_q:
        triples = [x for h in range(H) for x in triples if x[1] == h]
    if G and pass_ == 1:
        # key tiles per key/value head: H here counts key/value heads
        return [(b, hk * G, blk, hk, zigzag_slot(t, P)) for t, (b, hk, blk) in enumerate(triples)]
    if G:
        return [(b, h, blk, h // G, zigzag_slot(t, P)) for t, (b, h, blk) in enumerate(triples)]
    return [(b, h, blk, zigzag_slot(t, P)) for t, (b, h, blk) in enumerate(triples)]
