"""Pins of the fp64 oracle against what the mathematics and the pages fix.

None of these re-types the oracle's formulas: each compares it with a closed
form, an invariant, a library routine used the way the FMHA guide uses
PyTorch SDPA for correctness ("cuTile Kernels -- FMHA Implementation",
"Performance Results"), or finite differences.
"""
import math

import numpy as np
import pytest
import torch

from oracle import jfa_oracle as jo

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def _offsets(lengths):
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    return off


# ---------------------------------------------------------------- P1 ------
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    q, k, v = _rand(7, 5), _rand(9, 5), _rand(9, 3)
    _, _, p = jo.sequence_forward(q, k, v, 0.7, causal)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    if causal:  # no weight on future keys
        assert np.all(p[np.triu_indices(7, k=1, m=9)] == 0)


# ---------------------------------------------------------------- P2 ------
@pytest.mark.parametrize("broadcast_q", [True, False])
def test_single_key_returns_v_exactly(broadcast_q):
    H, d, Lq = 3, 8, 5
    lengths = [1, 4, 1]
    off = _offsets(lengths)
    T = int(off[-1])
    k, v = _rand(T, H, d), _rand(T, H, d)
    q = _rand(H, Lq, d) if broadcast_q else _rand(T, H, d)
    scale = 0.37
    out, lse = jo.jagged_forward(q, k, v, off, scale, False, broadcast_q)
    for b in (0, 2):
        s = int(off[b])
        for h in range(H):
            if broadcast_q:
                assert np.array_equal(out[b, h], np.broadcast_to(v[s, h], (Lq, d)))
                np.testing.assert_allclose(lse[b, h], scale * (q[h] @ k[s, h]), rtol=1e-15)
            else:
                assert np.array_equal(out[s, h], v[s, h])
                np.testing.assert_allclose(lse[s, h], scale * (q[s, h] @ k[s, h]), rtol=1e-15)


def test_causal_first_row_returns_first_value():
    q, k, v = _rand(6, 4), _rand(6, 4), _rand(6, 4)
    o, lse, _ = jo.sequence_forward(q, k, v, 0.5, True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == 0.5 * (q[0] @ k[0])


def test_empty_sequence():
    H, d, Lq = 2, 4, 3
    off = _offsets([3, 0, 2])
    k, v = _rand(5, H, d), _rand(5, H, d)
    q = _rand(H, Lq, d)
    out, lse = jo.jagged_forward(q, k, v, off, 0.5, False, True)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    dout = _rand(3, H, Lq, d)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, 0.5, False, True, dout)
    dq_wo, _, _ = jo.jagged_backward(q, k, v, _offsets([3, 2]), 0.5, False, True, dout[[0, 2]])
    np.testing.assert_allclose(dq, dq_wo, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P3 ------
@pytest.mark.parametrize("broadcast_q,causal", [(True, False), (False, True), (True, True)])
def test_sequence_permutation(broadcast_q, causal):
    H, d, Lq = 2, 6, 5
    lengths = [3, 7, 1, 5]
    perm = [2, 0, 3, 1]
    off = _offsets(lengths)
    T = int(off[-1])
    k, v = _rand(T, H, d), _rand(T, H, d)
    q = _rand(H, Lq, d) if broadcast_q else _rand(T, H, d)
    dout = _rand(len(lengths), H, Lq, d) if broadcast_q else _rand(T, H, d)

    def rows(b):
        return np.arange(off[b], off[b + 1])

    idx = np.concatenate([rows(b) for b in perm])
    off_p = _offsets([lengths[b] for b in perm])
    q_p = q if broadcast_q else q[idx]
    dout_p = dout[perm] if broadcast_q else dout[idx]
    o, lse = jo.jagged_forward(q, k, v, off, 0.4, causal, broadcast_q)
    o_p, lse_p = jo.jagged_forward(q_p, k[idx], v[idx], off_p, 0.4, causal, broadcast_q)
    g = jo.jagged_backward(q, k, v, off, 0.4, causal, broadcast_q, dout)
    g_p = jo.jagged_backward(q_p, k[idx], v[idx], off_p, 0.4, causal, broadcast_q, dout_p)
    if broadcast_q:
        np.testing.assert_allclose(o_p, o[perm], atol=1e-12)
        np.testing.assert_allclose(lse_p, lse[perm], atol=1e-12)
        np.testing.assert_allclose(g_p[0], g[0], atol=1e-12)  # dQ is a batch sum
    else:
        np.testing.assert_allclose(o_p, o[idx], atol=1e-12)
        np.testing.assert_allclose(lse_p, lse[idx], atol=1e-12)
        np.testing.assert_allclose(g_p[0], g[0][idx], atol=1e-12)
    np.testing.assert_allclose(g_p[1], g[1][idx], atol=1e-12)
    np.testing.assert_allclose(g_p[2], g[2][idx], atol=1e-12)


# ---------------------------------------------------------------- P4 ------
@pytest.mark.parametrize("n,L,BM,BN,causal", [
    (37, 53, 16, 8, False), (37, 53, 16, 8, True), (64, 64, 32, 32, True),
    (5, 130, 128, 64, False), (130, 130, 64, 64, True), (1, 1, 16, 16, False),
    (20, 3, 8, 4, True)])
def test_online_recurrence_matches_materialised(n, L, BM, BN, causal):
    q, k, v = _rand(n, 12), _rand(L, 12), _rand(L, 7)
    o, lse, _ = jo.sequence_forward(q, k, v, 0.3, causal)
    o2, lse2 = jo.online_forward_sequence(q, k, v, 0.3, causal, BM, BN)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P5 ------
def _sdpa(q, k, v, scale, mask=None, causal=False, gqa=False):
    """fp64 CPU SDPA with autograd; q [..., n, d], k/v [..., L, d] (gqa: k/v
    with fewer heads, torch's own grouped-query mapping)."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=None if mask is None else torch.tensor(mask),
        is_causal=causal, scale=scale, enable_gqa=gqa)
    return o, (tq, tk, tv)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 1), (3, 3)])
def test_gqa_self_mode_is_sdpa_grouped_query(causal, H, H_kv):
    """Grouped-query attention: B equal-length sequences in self mode against
    torch's SDPA with enable_gqa (its own head mapping and its autograd sums
    dK / dV over each group)."""
    B, L, d = 2, 7, 5
    scale = 0.4
    off = _offsets([L] * B)
    q, dout = _rand(B * L, H, d), _rand(B * L, H, d)
    k, v = _rand(B * L, H_kv, d), _rand(B * L, H_kv, d)
    out, lse = jo.jagged_forward(q, k, v, off, scale, causal, False)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, scale, causal, False, dout)
    dense = lambda x: x.reshape(B, L, x.shape[1], d).transpose(0, 2, 1, 3).copy()  # noqa: E731
    packed = lambda x: x.transpose(0, 2, 1, 3).reshape(B * L, x.shape[1], d)  # noqa: E731
    o_ref, (tq, tk, tv) = _sdpa(dense(q), dense(k), dense(v), scale, causal=causal, gqa=True)
    np.testing.assert_allclose(out, packed(o_ref.detach().numpy()), rtol=1e-12, atol=1e-12)
    o_ref.backward(torch.tensor(dense(dout)))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, packed(t.grad.numpy()), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_broadcast_is_sdpa_grouped_query(causal):
    """Broadcast mode with grouped-query heads: equal lengths against SDPA
    with the dense Q repeated over the batch and enable_gqa."""
    B, H, H_kv, Lq, L, d = 3, 4, 2, 5, 8, 6
    scale = 1 / math.sqrt(d)
    off = _offsets([L] * B)
    k, v = _rand(B * L, H_kv, d), _rand(B * L, H_kv, d)
    q = _rand(H, Lq, d)
    dout = _rand(B, H, Lq, d)
    out, _ = jo.jagged_forward(q, k, v, off, scale, causal, True)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, scale, causal, True, dout)
    kd = k.reshape(B, L, H_kv, d).transpose(0, 2, 1, 3)
    vd = v.reshape(B, L, H_kv, d).transpose(0, 2, 1, 3)
    qd = np.broadcast_to(q, (B, H, Lq, d)).copy()
    mask = np.tril(np.ones((Lq, L), dtype=bool)) if causal else None
    o_ref, (tq, tk, tv) = _sdpa(qd, kd, vd, scale, mask=mask, gqa=True)
    np.testing.assert_allclose(out, o_ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    o_ref.backward(torch.tensor(dout))
    np.testing.assert_allclose(dq, tq.grad.sum(0).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy().transpose(0, 2, 1, 3).reshape(B * L, H_kv, d),
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy().transpose(0, 2, 1, 3).reshape(B * L, H_kv, d),
                               rtol=1e-10, atol=1e-12)


def _band(n_q, n_k, window):
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return (j <= i) & (j > i - window)


@pytest.mark.parametrize("window", [1, 3, 6, 100])
def test_window_self_mode_is_sdpa_with_a_band_mask(window):
    """Causal sliding window: equal lengths in self mode against SDPA with the
    explicit band mask i - W < j <= i, forward and autograd gradients."""
    B, H, L, d = 2, 2, 9, 4
    scale = 0.6
    off = _offsets([L] * B)
    q, k, v, dout = (_rand(B * L, H, d) for _ in range(4))
    out, lse = jo.jagged_forward(q, k, v, off, scale, True, False, window=window)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, scale, True, False, dout, window=window)
    dense = lambda x: x.reshape(B, L, H, d).transpose(0, 2, 1, 3).copy()  # noqa: E731
    packed = lambda x: x.transpose(0, 2, 1, 3).reshape(B * L, H, d)  # noqa: E731
    mask = _band(L, L, window)
    o_ref, (tq, tk, tv) = _sdpa(dense(q), dense(k), dense(v), scale, mask=mask)
    np.testing.assert_allclose(out, packed(o_ref.detach().numpy()), rtol=1e-12, atol=1e-12)
    o_ref.backward(torch.tensor(dense(dout)))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, packed(t.grad.numpy()), rtol=1e-10, atol=1e-12)
    s = scale * torch.tensor(dense(q)) @ torch.tensor(dense(k)).transpose(-1, -2)
    s = s.masked_fill(~torch.tensor(mask), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy().transpose(0, 2, 1).reshape(B * L, H),
                               rtol=1e-12, atol=1e-12)


def test_window_broadcast_rows_that_see_no_key():
    """Broadcast mode, window W: query rows i >= L + W - 1 see no key of a
    length-L sequence: O = 0, lse = -inf, and they add nothing to dQ, dK, dV
    (the other rows match SDPA with the band mask)."""
    H, Lq, d, W = 2, 10, 3, 2
    lengths = [4, 1, 7]
    off = _offsets(lengths)
    T = sum(lengths)
    q, k, v = _rand(H, Lq, d), _rand(T, H, d), _rand(T, H, d)
    dout = _rand(len(lengths), H, Lq, d)
    out, lse = jo.jagged_forward(q, k, v, off, 0.5, True, True, window=W)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, 0.5, True, True, dout, window=W)
    dq_ref = np.zeros_like(dq)
    for b, L in enumerate(lengths):
        s0 = int(off[b])
        seen = np.arange(Lq) < L + W - 1
        assert np.all(out[b][:, ~seen] == 0) and np.all(np.isneginf(lse[b][:, ~seen]))
        mask = _band(int(seen.sum()), L, W)
        kd, vd = k[s0:s0 + L].transpose(1, 0, 2), v[s0:s0 + L].transpose(1, 0, 2)
        o_ref, (tq, tk, tv) = _sdpa(q[:, seen], kd.copy(), vd.copy(), 0.5, mask=mask)
        np.testing.assert_allclose(out[b][:, seen], o_ref.detach().numpy(), rtol=1e-12, atol=1e-12)
        o_ref.backward(torch.tensor(dout[b][:, seen].copy()))
        dq_ref[:, seen] += tq.grad.numpy()
        np.testing.assert_allclose(dk[s0:s0 + L], tk.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv[s0:s0 + L], tv.grad.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-10, atol=1e-12)


def test_window_wider_than_every_sequence_is_plain_causal():
    lengths = [5, 2, 8]
    off = _offsets(lengths)
    q, k, v, dout = (_rand(sum(lengths), 2, 3) for _ in range(4))
    a = jo.jagged_forward(q, k, v, off, 0.7, True, False, window=8)
    b = jo.jagged_forward(q, k, v, off, 0.7, True, False)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    ga = jo.jagged_backward(q, k, v, off, 0.7, True, False, dout, window=8)
    gb = jo.jagged_backward(q, k, v, off, 0.7, True, False, dout)
    for x, y in zip(ga, gb):
        np.testing.assert_array_equal(x, y)


def test_gqa_rejects_heads_that_do_not_split():
    off = _offsets([3])
    with pytest.raises(ValueError):
        jo.jagged_forward(_rand(3, 4, 2), _rand(3, 3, 2), _rand(3, 3, 2), off, 1.0, False, False)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_broadcast_is_dense_attention(causal):
    B, H, Lq, L, d = 3, 2, 6, 9, 8
    scale = 1 / math.sqrt(d)
    off = _offsets([L] * B)
    k, v = _rand(B * L, H, d), _rand(B * L, H, d)
    q = _rand(H, Lq, d)
    dout = _rand(B, H, Lq, d)
    out, lse = jo.jagged_forward(q, k, v, off, scale, causal, True)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, scale, causal, True, dout)
    kd = k.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    vd = v.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    qd = np.broadcast_to(q, (B, H, Lq, d)).copy()
    mask = np.tril(np.ones((Lq, L), dtype=bool)) if causal else None
    o_ref, (tq, tk, tv) = _sdpa(qd, kd, vd, scale, mask=mask)
    np.testing.assert_allclose(out, o_ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    s = scale * torch.tensor(qd) @ torch.tensor(kd).transpose(-1, -2)
    if causal:
        s = s.masked_fill(~torch.tensor(mask), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)
    o_ref.backward(torch.tensor(dout))
    np.testing.assert_allclose(dq, tq.grad.sum(0).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy().transpose(0, 2, 1, 3).reshape(B * L, H, d),
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy().transpose(0, 2, 1, 3).reshape(B * L, H, d),
                               rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_self_mode_is_batched_dense_attention(causal):
    """The dense LLM regime: B sequences of one length in self mode are a
    batched dense attention [B, H, L, d] (causal: SDPA's is_causal)."""
    B, H, L, d = 3, 2, 7, 6
    scale = 1 / math.sqrt(d)
    off = _offsets([L] * B)
    q, k, v, dout = (_rand(B * L, H, d) for _ in range(4))
    out, lse = jo.jagged_forward(q, k, v, off, scale, causal, False)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, scale, causal, False, dout)
    dense = lambda x: x.reshape(B, L, H, d).transpose(0, 2, 1, 3).copy()  # noqa: E731
    packed = lambda x: x.transpose(0, 2, 1, 3).reshape(B * L, H, d)  # noqa: E731
    o_ref, (tq, tk, tv) = _sdpa(dense(q), dense(k), dense(v), scale, causal=causal)
    np.testing.assert_allclose(out, packed(o_ref.detach().numpy()), rtol=1e-12, atol=1e-12)
    o_ref.backward(torch.tensor(dense(dout)))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, packed(t.grad.numpy()), rtol=1e-10, atol=1e-12)
    s = scale * torch.tensor(dense(q)) @ torch.tensor(dense(k)).transpose(-1, -2)
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(L, L, dtype=torch.bool)), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy().transpose(0, 2, 1).reshape(B * L, H),
                               rtol=1e-12, atol=1e-12)


def test_single_sequence_causal_is_sdpa_is_causal():
    T, H, d = 11, 3, 4
    q, k, v, dout = _rand(T, H, d), _rand(T, H, d), _rand(T, H, d), _rand(T, H, d)
    off = _offsets([T])
    out, _ = jo.jagged_forward(q, k, v, off, 0.5, True, False)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, 0.5, True, False, dout)
    o_ref, (tq, tk, tv) = _sdpa(*(x.transpose(1, 0, 2) for x in (q, k, v)), 0.5, causal=True)
    np.testing.assert_allclose(out, o_ref.detach().numpy().transpose(1, 0, 2), atol=1e-12)
    o_ref.backward(torch.tensor(dout.transpose(1, 0, 2).copy()))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.numpy().transpose(1, 0, 2), atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_self_mode_is_block_diagonal_dense_attention(causal):
    lengths = [4, 1, 6, 3]
    H, d = 2, 5
    off = _offsets(lengths)
    T = int(off[-1])
    q, k, v, dout = _rand(T, H, d), _rand(T, H, d), _rand(T, H, d), _rand(T, H, d)
    out, lse = jo.jagged_forward(q, k, v, off, 0.6, causal, False)
    dq, dk, dv = jo.jagged_backward(q, k, v, off, 0.6, causal, False, dout)
    seg = np.repeat(np.arange(len(lengths)), lengths)
    mask = seg[:, None] == seg[None, :]
    if causal:
        mask &= np.arange(T)[None, :] <= np.arange(T)[:, None]
    o_ref, (tq, tk, tv) = _sdpa(*(x.transpose(1, 0, 2) for x in (q, k, v)), 0.6, mask=mask)
    np.testing.assert_allclose(out, o_ref.detach().numpy().transpose(1, 0, 2), atol=1e-12)
    o_ref.backward(torch.tensor(dout.transpose(1, 0, 2).copy()))
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, t.grad.numpy().transpose(1, 0, 2), atol=1e-11)


# ---------------------------------------------------------------- P6 ------
def test_broadcast_dq_is_sum_of_per_sequence_dq():
    H, d, Lq = 2, 4, 3
    lengths = [5, 2, 7]
    off = _offsets(lengths)
    T = int(off[-1])
    q, k, v = _rand(H, Lq, d), _rand(T, H, d), _rand(T, H, d)
    dout = _rand(3, H, Lq, d)
    dq, _, _ = jo.jagged_backward(q, k, v, off, 0.8, False, True, dout)
    acc = np.zeros_like(dq)
    for b in range(3):
        s0, s1 = off[b], off[b + 1]
        g = jo.jagged_backward(q, k[s0:s1], v[s0:s1], _offsets([lengths[b]]), 0.8, False, True,
                               dout[b:b + 1])
        acc += g[0]
    np.testing.assert_allclose(dq, acc, rtol=1e-13, atol=1e-13)


def test_delta_identity():
    # rowsum(dO o O) == rowsum(P o dP) with dP = dO V^T: O = P V.
    q, k, v, do = _rand(5, 3), _rand(8, 3), _rand(8, 4), _rand(5, 4)
    o, _, p = jo.sequence_forward(q, k, v, 0.9, False)
    np.testing.assert_allclose((do * o).sum(1), (p * (do @ v.T)).sum(1), rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_dq_rows_match_full_backward(causal):
    H, d, Lq = 2, 4, 6
    lengths = [5, 0, 9, 2]
    off = _offsets(lengths)
    T = int(off[-1])
    q, k, v = _rand(H, Lq, d), _rand(T, H, d), _rand(T, H, d)
    dout = _rand(4, H, Lq, d)
    dq, _, _ = jo.jagged_backward(q, k, v, off, 0.5, causal, True, dout)
    rows = [(0, 0), (1, 5), (0, 3)]
    r = jo.broadcast_dq_rows(q, k, v, off, 0.5, causal, dout, rows)
    for n, (h, i) in enumerate(rows):
        np.testing.assert_allclose(r[n], dq[h, i], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P7 ------
def _fd_check(broadcast_q, causal, lengths, H=2, d=3, Lq=4, eps=1e-6):
    off = _offsets(lengths)
    T = int(off[-1])
    k, v = _rand(T, H, d), _rand(T, H, d)
    q = _rand(H, Lq, d) if broadcast_q else _rand(T, H, d)
    dout = _rand(len(lengths), H, Lq, d) if broadcast_q else _rand(T, H, d)
    scale = 0.7

    def loss(q_, k_, v_):
        return float((jo.jagged_forward(q_, k_, v_, off, scale, causal, broadcast_q)[0] * dout).sum())

    grads = jo.jagged_backward(q, k, v, off, scale, causal, broadcast_q, dout)
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][i] += eps
            args_m[which][i] -= eps
            fd[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("broadcast_q,causal", [(True, False), (True, True), (False, False), (False, True)])
def test_finite_differences(broadcast_q, causal):
    _fd_check(broadcast_q, causal, [3, 1, 5])
