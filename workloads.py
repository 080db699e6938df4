"""Seeded synthetic inputs for jagged attention: the one module both sides share.

This module draws sequence lengths and bf16 tensors and nothing else: it holds
no attention arithmetic.  The oracle (CPU, fp64) and the HIP library are both
fed from what it returns.

The five workloads stand in for the production shapes of "Optimizing Jagged
Flash Attention with TLX" (Performance section: a dense broadcast Q against
jagged K/V at varying sparsity), whose data is not public.  Each is given by
its sizes and length distribution:

  tiny_bcast      broadcast Q, B=4,    H=2,  d=64,  Lq=32,  L ~ U[1,64]
  self_causal_1k  self-attn, causal, B=32,  H=8,  d=128,        L ~ U[1,1024]
  prod_bcast      broadcast Q, B=1024, H=4,  d=128, Lq=256, L ~ U[64,2048]
  long_causal_8k  self-attn, causal, B=64,  H=16, d=128,        L ~ logU[128,8192]
  skew_bcast      broadcast Q, B=4096, H=8,  d=128, Lq=512,
                  90% L ~ U[1,32], 10% L ~ U[4096,16384], values N(0, 0.5)

and two of the dense LLM regime (equal-length Q/K/V, B=768, H=4, d=128),
at sequence length 1024, self-attention without and with the causal mask:

  dense_llm_1k         self-attn,         B=768, H=4, d=128, L = 1024
  dense_llm_1k_causal  self-attn, causal, B=768, H=4, d=128, L = 1024

and two of the attention variants the pages name (grouped-query heads and a
sliding window), on the shapes above:

  prod_bcast_gqa         prod_bcast with one key/value head for the 4 query heads
  long_causal_8k_window  long_causal_8k with a causal window of 1024 keys

Lengths are drawn with numpy's PCG64 from the seed; integer draws are
inclusive.  Log-uniform lengths are round(exp(U(ln lo, ln hi))) clipped to
[lo, hi].  In skew_bcast exactly round(0.1*B) sequences, at seeded random
positions, are long.  Tensor values are fp32 normal draws times the
workload's standard deviation, rounded to bf16 (round to nearest even), made
with a torch generator on the target device so large inputs never pass
through host memory.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

try:  # torch is only needed to materialise tensors
    import torch
except ImportError:  # pragma: no cover
    torch = None


@dataclass(frozen=True)
class Workload:
    name: str
    broadcast_q: bool
    causal: bool
    B: int
    H: int
    d: int
    Lq: int  # query rows of the shared Q (broadcast mode); 0 in self mode
    lengths: tuple  # ("uniform", lo, hi) | ("loguniform", lo, hi) | ("mix", frac_long, (lo,hi), (lo,hi))
    std: float = 1.0
    tags: tuple = field(default_factory=tuple)
    H_kv: int = 0  # key / value heads (grouped-query attention); 0: H
    window: int = 0  # causal sliding window in keys; 0: none

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = [
    Workload("tiny_bcast", True, False, 4, 2, 64, 32, ("uniform", 1, 64)),
    Workload("self_causal_1k", False, True, 32, 8, 128, 0, ("uniform", 1, 1024)),
    Workload("prod_bcast", True, False, 1024, 4, 128, 256, ("uniform", 64, 2048)),
    Workload("long_causal_8k", False, True, 64, 16, 128, 0, ("loguniform", 128, 8192)),
    Workload("skew_bcast", True, False, 4096, 8, 128, 512,
             ("mix", 0.1, (1, 32), (4096, 16384)), std=0.5),
    # The pages' second regime: dense LLM attention, equal-length Q/K/V.
    Workload("dense_llm_1k", False, False, 768, 4, 128, 0, ("uniform", 1024, 1024)),
    Workload("dense_llm_1k_causal", False, True, 768, 4, 128, 0, ("uniform", 1024, 1024)),
    # Attention variants on the shapes above.
    Workload("prod_bcast_gqa", True, False, 1024, 4, 128, 256, ("uniform", 64, 2048), H_kv=1),
    Workload("long_causal_8k_window", False, True, 64, 16, 128, 0, ("loguniform", 128, 8192), window=1024),
]


def workload(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return WORKLOADS[index_or_name]
    for w in WORKLOADS:
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)


def draw_lengths(spec: tuple, B: int, seed: int) -> np.ndarray:
    """Sequence lengths (int64 [B]) for a length spec, from numpy PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kind = spec[0]
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        return rng.integers(lo, hi + 1, size=B, dtype=np.int64)
    if kind == "loguniform":
        lo, hi = spec[1], spec[2]
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)
    if kind == "mix":
        frac, (slo, shi), (llo, lhi) = spec[1], spec[2], spec[3]
        n_long = int(round(frac * B))
        lengths = rng.integers(slo, shi + 1, size=B, dtype=np.int64)
        pos = rng.choice(B, size=n_long, replace=False)
        lengths[pos] = rng.integers(llo, lhi + 1, size=n_long, dtype=np.int64)
        return lengths
    raise ValueError(f"unknown length spec {spec!r}")


def offsets_from_lengths(lengths) -> np.ndarray:
    """int64 [B+1]: offsets[0] = 0, offsets[b+1] = offsets[b] + lengths[b]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.size + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def _normal_bf16(shape, std, gen, device, chunk_elems=1 << 28):
    """bf16 tensor of fp32 N(0,1)*std draws, produced in chunks on `device`."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        tmp = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:e].copy_(tmp)  # fp32 -> bf16, round to nearest even
        del tmp
    return out


def make_tensors(lengths, H: int, d: int, Lq: int, broadcast_q: bool, std: float = 1.0,
                 seed: int = 0, device="cpu", with_dout: bool = True):
    """Seeded q, k, v, dout (bf16) and offsets (int64) for one jagged batch.

    Layouts: k, v [T, H, d] with T = sum(lengths).  Broadcast mode: q [H, Lq, d],
    dout [B, H, Lq, d].  Self mode: q, dout [T, H, d].
    """
    if torch is None:  # pragma: no cover
        raise RuntimeError("torch is required to build tensors")
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    B = lengths.size
    dev = torch.device(device)
    gens = []
    for i in range(4):
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 7919 + 104729 * (i + 1))
        gens.append(g)
    q_shape = (H, Lq, d) if broadcast_q else (T, H, d)
    o_shape = (B, H, Lq, d) if broadcast_q else (T, H, d)
    t = {
        "offsets": torch.from_numpy(off).to(dev),
        "q": _normal_bf16(q_shape, std, gens[0], dev),
        "k": _normal_bf16((T, H, d), std, gens[1], dev),
        "v": _normal_bf16((T, H, d), std, gens[2], dev),
    }
    if with_dout:
        t["dout"] = _normal_bf16(o_shape, std, gens[3], dev)
    t["lengths"] = lengths
    t["total_len"] = T
    return t


def make_workload(w, seed: int | None = None, device="cpu", with_dout: bool = True):
    """Tensors for a named workload (seed defaults to the workload's index)."""
    if not isinstance(w, Workload):
        w = workload(w)
    if seed is None:
        seed = WORKLOADS.index(w)
    lengths = draw_lengths(w.lengths, w.B, seed)
    t = make_tensors(lengths, w.H, w.d, w.Lq, w.broadcast_q, w.std, seed, device, with_dout)
    if w.kv_heads < w.H:  # the first H_kv heads of the draw
        t["k"] = t["k"][:, :w.kv_heads].contiguous()
        t["v"] = t["v"][:, :w.kv_heads].contiguous()
    t["workload"] = w
    return t


# MXFP8 inputs ("Low-precision (MXFP8) attention"): random E4M3 element codes
# and E8M0 scale codes, drawn directly as integers (no quantization happens
# here).  Element magnitude codes are uniform over exponent fields 4..8
# (values 2^-3 .. 3.75) with a random sign; scale codes are 125..127 (scales
# 1/4, 1/2, 1).  V comes transposed, [H_kv, d, T_pad] with T_pad = T rounded
# up to 64 and zero codes past T, its scales per 32 keys of the packed index,
# [H_kv, T_pad / 32, d].
MX_CODE_LO, MX_CODE_HI = 0x20, 0x47
MX_SCALE_LO, MX_SCALE_HI = 125, 127


def _mx_codes(shape, gen, device):
    mag = torch.randint(MX_CODE_LO, MX_CODE_HI + 1, shape, generator=gen, device=device, dtype=torch.int32)
    sign = torch.randint(0, 2, shape, generator=gen, device=device, dtype=torch.int32) * 0x80
    return (mag | sign).to(torch.uint8)


def _mx_scales(shape, gen, device):
    return torch.randint(MX_SCALE_LO, MX_SCALE_HI + 1, shape, generator=gen, device=device,
                         dtype=torch.int32).to(torch.uint8)


def make_mx_tensors(lengths, H: int, H_kv: int, d: int, Lq: int, broadcast_q: bool, seed: int = 0,
                    device="cpu"):
    """Seeded MXFP8 inputs: q8 / q_scale, k8 / k_scale, vt8 / vt_scale (uint8
    codes) and offsets.  Layouts: q8 [H, Lq, d] (broadcast) or [T, H, d],
    q_scale the same with d / 32; k8 [T, H_kv, d], k_scale [T, H_kv, d / 32];
    vt8 [H_kv, d, T_pad], vt_scale [H_kv, T_pad / 32, d]."""
    if torch is None:  # pragma: no cover
        raise RuntimeError("torch is required to build tensors")
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    T_pad = max(64, -(-T // 64) * 64)
    dev = torch.device(device)
    gens = []
    for i in range(6):
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 6007 + 7919 * (i + 1))
        gens.append(g)
    nb = d // 32
    q_shape = (H, Lq, d) if broadcast_q else (T, H, d)
    vt8 = _mx_codes((H_kv, d, T_pad), gens[4], dev)
    vt8[:, :, T:] = 0
    return {
        "offsets": torch.from_numpy(off).to(dev),
        "q8": _mx_codes(q_shape, gens[0], dev),
        "q_scale": _mx_scales(q_shape[:-1] + (nb,), gens[1], dev),
        "k8": _mx_codes((T, H_kv, d), gens[2], dev),
        "k_scale": _mx_scales((T, H_kv, nb), gens[3], dev),
        "vt8": vt8,
        "vt_scale": _mx_scales((H_kv, T_pad // 32, d), gens[5], dev),
        "lengths": lengths,
        "total_len": T,
        "t_pad": T_pad,
    }


def make_mx_workload(w, seed: int | None = None, device="cpu"):
    """MXFP8 inputs for a named workload's shapes (seed: the workload's index)."""
    if not isinstance(w, Workload):
        w = workload(w)
    if seed is None:
        seed = WORKLOADS.index(w)
    lengths = draw_lengths(w.lengths, w.B, seed)
    t = make_mx_tensors(lengths, w.H, w.kv_heads, w.d, w.Lq, w.broadcast_q, seed, device)
    t["workload"] = w
    return t


def _tile_encodings(codes, tiles, n: int, n_pad: int):
    """Row and column encodings of one tensor given as E4M3 codes [..., n, d]
    and one E8M0 code per 32 x 32 tile, [..., n_pad / 32, d / 32]: the row
    encoding's scales [..., n, d / 32] and the transposed codes [..., d, n_pad]
    (zero past n) with scales [..., n_pad / 32, d].  Both dequantize to the
    same values."""
    row_scale = tiles.repeat_interleave(32, dim=-2)[..., :n, :]
    col_codes = torch.zeros(codes.shape[:-2] + (codes.shape[-1], n_pad), dtype=torch.uint8, device=codes.device)
    col_codes[..., :n] = codes.transpose(-1, -2)
    col_scale = tiles.repeat_interleave(32, dim=-1)
    return row_scale.contiguous(), col_codes.contiguous(), col_scale.contiguous()


def make_mx_bwd_tensors(lengths, H: int, H_kv: int, d: int, Lq: int, broadcast_q: bool, seed: int = 0,
                        consistent: bool = True, device="cpu"):
    """Seeded MXFP8 inputs of the forward and the backward: every encoding of
    Q, K, V and dO (layouts in oracle/mx_oracle.py's header) and offsets.

    consistent=True: each tensor is one set of E4M3 codes with one E8M0 scale
    per 32 x 32 tile (32 positions of its query / key axis by 32 head-dim
    elements), so that its row-wise and its transposed, axis-blocked encoding
    hold the same values, as two quantizations of one tensor would nearly.
    consistent=False: every encoding drawn on its own (codes and scales), so
    that a kernel reading one encoding in place of another differs."""
    if torch is None:  # pragma: no cover
        raise RuntimeError("torch is required to build tensors")
    lengths = np.asarray(lengths, dtype=np.int64)
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    B = len(lengths)
    T_pad = max(64, -(-T // 64) * 64)
    Lq_pad = max(64, -(-Lq // 64) * 64) if broadcast_q else 0
    dev = torch.device(device)
    gens = []
    for i in range(16):
        g = torch.Generator(device=dev)
        g.manual_seed(seed * 7001 + 104729 * (i + 1))
        gens.append(g)
    nb = d // 32
    out = {"offsets": torch.from_numpy(off).to(dev), "lengths": lengths, "total_len": T, "t_pad": T_pad,
           "lq_pad": Lq_pad}

    def packed(name, heads, gi):
        # [T, heads, d] row encoding; transposed [heads, d, T_pad] along the packed index
        codes = _mx_codes((heads, T, d), gens[gi], dev)
        if consistent:
            tiles = _mx_scales((heads, T_pad // 32, nb), gens[gi + 1], dev)
            rs, cc, cs = _tile_encodings(codes, tiles, T, T_pad)
        else:
            rs = _mx_scales((heads, T, nb), gens[gi + 1], dev)
            cc = _mx_codes((heads, d, T_pad), gens[gi + 2], dev)
            cc[:, :, T:] = 0
            cs = _mx_scales((heads, T_pad // 32, d), gens[gi + 3], dev)
        out[name + "8"] = codes.permute(1, 0, 2).contiguous()
        out[name + "_scale"] = rs.permute(1, 0, 2).contiguous()
        out[name + "t8"] = cc
        out[name + "t_scale"] = cs

    def dense(name, lead, gi):
        # [*lead, Lq, d] row encoding; transposed [*lead, d, Lq_pad] from query 0
        codes = _mx_codes(lead + (Lq, d), gens[gi], dev)
        if consistent:
            tiles = _mx_scales(lead + (Lq_pad // 32, nb), gens[gi + 1], dev)
            rs, cc, cs = _tile_encodings(codes, tiles, Lq, Lq_pad)
        else:
            rs = _mx_scales(lead + (Lq, nb), gens[gi + 1], dev)
            cc = _mx_codes(lead + (d, Lq_pad), gens[gi + 2], dev)
            cc[..., Lq:] = 0
            cs = _mx_scales(lead + (Lq_pad // 32, d), gens[gi + 3], dev)
        out[name + "8"] = codes
        out[name + "_scale"] = rs
        out[name + "t8"] = cc
        out[name + "t_scale"] = cs

    packed("k", H_kv, 0)
    packed("v", H_kv, 4)
    if broadcast_q:
        dense("q", (H,), 8)
        dense("do", (B, H), 12)
    else:
        packed("q", H, 8)
        packed("do", H, 12)
    return out


def make_mx_bwd_workload(w, seed: int | None = None, consistent: bool = True, device="cpu"):
    """make_mx_bwd_tensors for a named workload's shapes (seed: the workload's index)."""
    if not isinstance(w, Workload):
        w = workload(w)
    if seed is None:
        seed = WORKLOADS.index(w)
    lengths = draw_lengths(w.lengths, w.B, seed)
    t = make_mx_bwd_tensors(lengths, w.H, w.kv_heads, w.d, w.Lq, w.broadcast_q, seed, consistent, device)
    t["workload"] = w
    return t
