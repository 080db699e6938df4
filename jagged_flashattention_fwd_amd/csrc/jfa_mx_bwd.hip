// MXFP8 jagged attention backward on gfx950 (d = 128).
//
// "Optimizing Jagged Flash Attention with TLX", "Low-precision (MXFP8)
// attention": the backward, like the forward, runs its products on
// block-scaled FP8 operands (E4M3 elements, one E8M0 scale per 32 elements
// along the product's reduction dimension), quantizing the softmax output
// (and here also dS) on the fly.  Each input arrives in the encodings its
// products need (layouts in include/jfa.h):
//   S    = Q K^T     Q, K row-wise                  (reduction over d)
//   dP   = dO V^T    dO, V row-wise                 (reduction over d)
//   dV  += P^T dO    dO blocked along the queries   (reduction over queries)
//   dK  += dS^T Q    Q blocked along the queries    (reduction over queries)
//   dQ  += dS K      K blocked along the keys       (reduction over keys)
// with P = exp(S scale - lse), delta = rowsum(dO o O) (row-wise dO, the
// forward's O as stored) and dS = P o (dP - delta), all float32; P and dS
// are quantized per key column in blocks of 32 queries for dV and dK, dS per
// query row in blocks of 32 keys of the packed index for dQ, with the block
// rule of the forward (scale 2^(floor(log2 amax) - 8), nearest E4M3, ties to
// even, capped at 448).  The softmax scale multiplies dK and dQ.
//
// Kernels, in launch order:
//   delta_mx_kernel  -delta (the dP products below start from it) and
//                    lse * log2(e) per query row.
//   dkdv_mx_kernel   persistent over tiles of 128 keys of one (sequence,
//                    key / value head), eight waves in four pairs of 32
//                    keys, two waves per SIMD: both waves of a pair hold the
//                    keys' row-wise K and V in registers, one takes the
//                    first 32 queries of each step and accumulates dV, the
//                    other the last 32 and accumulates dK, and each hands its
//                    partner the quantized block the partner's product
//                    needs.  The group's query heads stream in steps of 64
//                    queries through LDS (row-wise Q and dO, query-blocked
//                    Q^T and dO^T, their scales, lse and -delta).  A lane
//                    owns one key, so the quantization along the queries is
//                    a per-lane block of the score layout.
//   dq_mx_kernel     the forward's structure: a lane owns one query row,
//                    keys stream in steps of 64 of the packed index (row-wise
//                    K and V, key-blocked K^T).  Self mode: persistent over
//                    tiles of 256 query rows, writing dQ.  Broadcast: one
//                    workgroup per (head, 256-row query block, chunk of
//                    sequences), writing a float32 partial that dq_reduce
//                    (jfa_bwd.hip) sums in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_mx.hpp"
#include "jfa_timing.hpp"

namespace jfa {
namespace {

// Row copies into LDS (as in the forward): rows of 128 bytes padded to 144,
// nine lanes per row, so a copy moves 7 rows and the first chunk of an
// eighth; transposed rows of 64 bytes padded to 80, five lanes per row, 12
// rows and the four chunks of a thirteenth.  Two copies starting one (four)
// rows apart cover a wave's 8 (16) rows; the overhang into the next row
// writes that row's own data, or lands in the gap after the tile.
constexpr int RB = 144, TB = 80;
__device__ __forceinline__ uint32_t row_voff(int l, uint32_t stride) {
  return (uint32_t)(l / 9) * stride + ((l % 9) < 8 ? (uint32_t)(l % 9) * 16u : 0u);
}
__device__ __forceinline__ uint32_t trow_voff(int l, uint32_t stride) {
  return (uint32_t)(l / 5) * stride + ((l % 5) < 4 ? (uint32_t)(l % 5) * 16u : 0u);
}

// ---------------------------------------------------------------- delta --
// -delta, delta = sum over d of dequant(dO) o O, and lse * log2(e), per
// query row (the dP products of both kernels below start from -delta, so
// that dS = P o dP' takes no subtraction).  Eight threads per row of 128,
// 16 elements (half a scale block) each.
__global__ __launch_bounds__(256) void delta_mx_kernel(const uint16_t* __restrict__ out,
                                                       const uint8_t* __restrict__ do8,
                                                       const uint8_t* __restrict__ do_scale,
                                                       const float* __restrict__ lse, float* __restrict__ delta,
                                                       float* __restrict__ lse2, int64_t rows) {
  constexpr int D = 128, TPR = 8;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = gtid; e < rows * TPR; e += stride) {
    const int64_t row = e / TPR;
    const int c = (int)(e % TPR);
    const u32x4 codes = *reinterpret_cast<const u32x4*>(do8 + row * D + c * 16);
    const u32x4 o0 = *reinterpret_cast<const u32x4*>(out + row * D + c * 16);
    const u32x4 o1 = *reinterpret_cast<const u32x4*>(out + row * D + c * 16 + 8);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[w], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes[w], true);
      const uint32_t oa = w < 2 ? o0[2 * w] : o1[2 * w - 4];
      const uint32_t ob = w < 2 ? o0[2 * w + 1] : o1[2 * w - 3];
      acc += lo[0] * bf16_lo(oa);
      acc += lo[1] * bf16_hi(oa);
      acc += hi[0] * bf16_lo(ob);
      acc += hi[1] * bf16_hi(ob);
    }
    acc *= __builtin_amdgcn_ldexpf(1.f, (int)do_scale[row * 4 + c / 2] - 127);
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (c == 0) {
      delta[row] = -acc;
      lse2[row] = lse[row] * LOG2E;
    }
  }
}

// ------------------------------------------------------------- dK / dV --
struct MxB {
  // Waves w and w + 4 form a pair over the same 32 keys: wave w takes the
  // step's first 32 queries and accumulates dV, wave w + 4 the other 32 and
  // dK; each hands its partner the quantized operand the partner needs.
  static constexpr int NW = 8, BQ = 64, BK = NW / 2 * 32, D = 128, NBUF = 3, DEP = 2;
  static constexpr int RW = BQ / NW, TW = D / NW;  // Q / dO rows and transposed rows copied per wave
  static constexpr int NRC = (RW + 6) / 7, NTC = (TW + 11) / 12;  // copies per wave of each
  static_assert(RW >= 7 && TW >= 12, "copy geometry");
  static_assert(BK == MX_BK, "the key tiles of the schedule");
  static constexpr int OFF_Q = 0;                          // Q rows [64][144]
  static constexpr int OFF_DO = OFF_Q + BQ * RB + 16;      // dO rows
  static constexpr int OFF_QT = OFF_DO + BQ * RB + 16;     // Q^T rows [128 d][80]
  static constexpr int OFF_DOT = OFF_QT + D * TB + 64;     // dO^T rows
  static constexpr int OFF_QS = OFF_DOT + D * TB + 64;     // Q row scale words [64]
  static constexpr int OFF_DOS = OFF_QS + BQ * 4;          // dO row scale words
  static constexpr int OFF_QTS = OFF_DOS + BQ * 4;         // Q^T scales [2 query blocks][128 d]
  static constexpr int OFF_DOTS = OFF_QTS + 2 * D;         // dO^T scales
  static constexpr int OFF_L = OFF_DOTS + 2 * D;           // lse * log2(e) [64]
  static constexpr int OFF_DL = OFF_L + BQ * 4;            // -delta [64]
  static constexpr int BUF = OFF_DL + BQ * 4;
  // Copies per wave per step: Q, dO, Q^T, dO^T, and one dword copy each of
  // the four scale arrays, lse and delta.
  static constexpr int IPS = 2 * NRC + 2 * NTC + 6;
  static constexpr int NST = 4 * 16;  // stores per wave at a tile end: dV or dK, 16 per head-dim tile
  static constexpr int NST_WAIT = NST < 63 ? NST : 63;
  static_assert(BUF % 16 == 0, "buffer alignment");
  static_assert(NBUF * BUF <= 160 * 1024, "LDS");
  static_assert(NBUF >= DEP + 1, "a buffer is refilled only after every wave has left it");
  static constexpr int NKV = 12;          // loads of a tile's K / V operands and of the next tile record
  // At a tile end at most one step's copies stay in flight before the next
  // tile's K / V loads and this tile's stores are issued.
  static_assert(DEP * IPS <= 63 && IPS + NKV <= 63, "vector-memory counter");
};

// Two 16-byte global reads forming one lane's 32 operand bytes.
__device__ __forceinline__ i32x8 ld32x2(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p0);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p1);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(MxB::NW * WAVE, 1) void dkdv_mx_kernel(BwdMxArgs a) {
  using C = MxB;
  constexpr int BQ = C::BQ, BK = C::BK, D = C::D, NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS, NST_WAIT = C::NST_WAIT;
  constexpr int NW = C::NW, RW = C::RW, TW = C::TW, NRC = C::NRC, NTC = C::NTC;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][C::BUF];

  __shared__ __attribute__((aligned(16))) u32x4 xw[NW][WAVE];  // operand words handed to the partner
  __shared__ uint32_t xc[NW][WAVE];                           // and their block scale codes

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int role = wave / (NW / 2);  // 0: queries 0..31 of a step, dV; 1: queries 32..63, dK
  const int kw = wave % (NW / 2);    // key group of the pair
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_ktiles;
  const int H = a.H, Lq = a.Lq, Hkv = a.Hkv, G = a.G;
  const int64_t total = a.total_len;
  const float c2 = a.scale_log2;

  const int64_t t0 = zigzag_tile(0, slot, a.P);
  if (t0 >= T) return;

  // ---- per-lane copy geometry
  const uint32_t rstride = BCAST ? (uint32_t)D : (uint32_t)H * D;          // between Q / dO rows
  const uint32_t sstride = BCAST ? 4u : (uint32_t)H * 4;                   // between row scale words, lse, delta
  const uint32_t tpad = BCAST ? (uint32_t)a.lq_pad : (uint32_t)a.t_pad;   // between transposed rows
  const uint32_t voff_r = row_voff(l, rstride);
  const uint32_t voff_t = trow_voff(l, tpad);
  const uint32_t nqb = tpad / 32;  // query blocks per transposed row

  struct Tp {
    int64_t s0;
    int L, hk, b, k0;  // k0: local index of the tile's first key
    int nq;            // queries of the sequence (broadcast: Lq)
    int j0, nj;        // steps j0 .. j0 + nj - 1 per query head (64-query units of Lq / of the packed index)
    int jp0, jp1;      // steps [jp0, jp1) need no mask
  };
  auto tparams = [&](const TileRec& r) {
    Tp p;
    p.s0 = r.s0;
    p.L = r.L;
    p.hk = r.hk;
    p.b = r.b;
    p.k0 = r.blk * BK;
    p.nq = BCAST ? Lq : r.L;
    const int k_last = min(p.k0 + BK, r.L) - 1;  // the tile's last key
    // queries that see a key of the tile: q >= k0 when causal
    const int q_first = CAUSAL ? p.k0 : 0;
    const int64_t base = BCAST ? 0 : r.s0;       // position of local query 0 on the step axis
    if (q_first >= p.nq) {
      p.j0 = 0;
      p.nj = 0;
    } else {
      p.j0 = (int)((base + q_first) / BQ);
      p.nj = (int)((base + p.nq - 1) / BQ) - p.j0 + 1;
    }
    // plain steps: every query of the step exists and (causal) sees every key
    // of the tile
    const int64_t lo = base + (CAUSAL ? (int64_t)k_last : 0);  // first position whose query sees all keys
    const int64_t hi = base + p.nq;                            // end of the queries
    p.jp0 = (int)((lo + BQ - 1) / BQ);
    p.jp1 = (int)(hi / BQ);
    return p;
  };

  // ---- the step stream: steps (query head gi, step j) of the current and
  // the next tile, issued DEP ahead of their use.  Each wave copies RW rows
  // of Q and dO, TW rows of Q^T and dO^T, and RW words of each scale array,
  // lse and delta.
  int g_iss = 0, g_cmp = 0, iss_cur = 0, iss_nxt = 0;
  const int64_t qt_bytes = (int64_t)H * D * tpad;
  const int64_t dot_bytes = BCAST ? (int64_t)a.B * H * D * tpad : (int64_t)H * D * tpad;
  // part 0: the row copies and the small ones (after a step's first
  // barrier), 1: the transposed rows (after its second), 2: both.  Splitting
  // keeps a workgroup's 112 copies from queueing behind each other at once.
  auto issue_next = [&](const Tp& cp, const Tp& np, bool has_nxt, int part) {
    const int ncur = cp.nj * G, nnxt = np.nj * G;
    const bool cur = iss_cur < ncur;
    if (!(cur || (has_nxt && iss_nxt < nnxt))) return;
    const Tp& p = cur ? cp : np;
    const int s = cur ? iss_cur : iss_nxt;
    const int gi = s / p.nj, j = p.j0 + s % p.nj;
    const int h = p.hk * G + gi;
    const int64_t pos = (int64_t)j * BQ + wave * RW;  // this wave's first Q / dO row on the step axis
    const int64_t avail = BCAST ? (int64_t)Lq - pos : total - pos;
    const int nrow = (int)max((int64_t)0, min(avail, (int64_t)(RW + 1)));
    const int nsc = min(nrow, RW);
    int64_t qrow, drow, qt_off, dot_off;
    if constexpr (BCAST) {
      qrow = (int64_t)h * Lq + pos;
      drow = ((int64_t)p.b * H + h) * Lq + pos;
      qt_off = ((int64_t)h * D + wave * TW) * tpad + (int64_t)j * BQ;
      dot_off = (((int64_t)p.b * H + h) * D + wave * TW) * tpad + (int64_t)j * BQ;
    } else {
      qrow = drow = pos * H + h;
      qt_off = dot_off = ((int64_t)h * D + wave * TW) * tpad + (int64_t)j * BQ;
    }
    const int64_t sc_q = ((int64_t)h * nqb + 2 * j) * D + wave * (2 * D / NW);
    const int64_t sc_d = BCAST ? (((int64_t)p.b * H + h) * nqb + 2 * j) * D + wave * (2 * D / NW) : sc_q;
    const uint32_t buf = lds_addr(smem[(uint32_t)g_iss % NBUF]);
    if (part != 1) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q8 + qrow * D, nrow * (int)rstride);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.do8 + drow * D, nrow * (int)rstride);
      const uint32_t qd = buf + C::OFF_Q + wave * RW * RB, dd = buf + C::OFF_DO + wave * RW * RB;
#pragma unroll
      for (int c = 0; c < NRC; ++c) {
        const int r = min(7 * c, RW - 7);
        dma_copy16_buf(rq, voff_r, (uint32_t)r * rstride, qd + r * RB);
        dma_copy16_buf(rd, voff_r, (uint32_t)r * rstride, dd + r * RB);
      }
    }
    if (part != 0) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.qt8 + qt_off, (int)min(qt_bytes - qt_off, (int64_t)(TW + 1) * tpad));
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dot8 + dot_off, (int)min(dot_bytes - dot_off, (int64_t)(TW + 1) * tpad));
      const uint32_t qd = buf + C::OFF_QT + wave * TW * TB, dd = buf + C::OFF_DOT + wave * TW * TB;
#pragma unroll
      for (int c = 0; c < NTC; ++c) {
        const int r = min(12 * c, TW - 12);
        dma_copy16_buf(rq, voff_t, (uint32_t)r * tpad, qd + r * TB);
        dma_copy16_buf(rd, voff_t, (uint32_t)r * tpad, dd + r * TB);
      }
    }
    if (part != 1 && l < RW) {
      const uint32_t so = (uint32_t)l * sstride, sb = (uint32_t)wave * RW * 4;
      dma_copy4_buf(make_rsrc(a.q_scale + qrow * 4, nsc * (int)sstride), so, 0, buf + C::OFF_QS + sb);
      dma_copy4_buf(make_rsrc(a.do_scale + drow * 4, nsc * (int)sstride), so, 0, buf + C::OFF_DOS + sb);
      dma_copy4_buf(make_rsrc(a.lse2 + drow, nsc * (int)sstride), so, 0, buf + C::OFF_L + sb);
      dma_copy4_buf(make_rsrc(a.delta + drow, nsc * (int)sstride), so, 0, buf + C::OFF_DL + sb);
      dma_copy4_buf(make_rsrc(a.qt_scale + sc_q, 2 * D / NW), (uint32_t)l * 4, 0, buf + C::OFF_QTS + sb);
      dma_copy4_buf(make_rsrc(a.dot_scale + sc_d, 2 * D / NW), (uint32_t)l * 4, 0, buf + C::OFF_DOTS + sb);
    }
    if (part == 0) return;
    if (cur) ++iss_cur;
    else ++iss_nxt;
    ++g_iss;
  };
  auto wait_step = [&](int gi) {
    const int after = g_iss - 1 - gi;
    if (after >= 1) wait_vmcnt<IPS>();
    else wait_vmcnt<0>();
  };

  // ---- K and V of this wave's 32 keys (B operands of S and dP): lane (key,
  // g) holds bytes 16 g .. 16 g + 15 of the blocks 2 kk and 2 kk + 1, and its
  // scale word shifted so that byte 2 kk is block 2 kk + g's scale.  Keys
  // past the sequence read its first row; their columns are never stored.
  i32x8 kop[2], vop[2];
  uint32_t ksc = 0, vsc = 0;
  auto load_kv = [&](const Tp& p) {
    int key = p.k0 + kw * 32 + lc;
    key = key < p.L ? key : 0;
    const int64_t row = (p.s0 + key) * Hkv + p.hk;
    const uint8_t* kr = a.k8 + row * D;
    const uint8_t* vr = a.v8 + row * D;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      kop[kk] = ld32x2(kr + 64 * kk + 16 * g, kr + 64 * kk + 32 + 16 * g);
      vop[kk] = ld32x2(vr + 64 * kk + 16 * g, vr + 64 * kk + 32 + 16 * g);
    }
    ksc = *reinterpret_cast<const uint32_t*>(a.k_scale + row * 4) >> (8 * g);
    vsc = *reinterpret_cast<const uint32_t*>(a.v_scale + row * 4) >> (8 * g);
  };

  // dV (role 0) or dK (role 1) of this wave's 32 keys, key by d: the
  // quantized operand of the products is their A side (a key per row, the
  // scaled product's A and B layouts being the same), so register
  // 4 i4 + e of head-dim tile dt is key 8 i4 + 4 g + e at d = 32 dt + lc.
  f32x16 acc[4];
  // dV, or dK = scale * acc, of a tile: NST bounded buffer stores per wave,
  // each writing two whole 128-byte rows (lanes 0-31 one key, lanes 32-63
  // the key 4 further) straight from the registers.  The whole byte offset
  // stays in the lane operand, which the range check covers; the asm hides
  // the lane part from loop-invariant hoisting.
  auto store_out = [&](const Tp& p, bool live) {
    const int k0 = p.k0 + kw * 32;
    const int nv = live ? max(0, min(p.L - k0, 32)) : 0;
    const uint32_t kstride = (uint32_t)Hkv * D * 4;
    const int64_t row0 = (p.s0 + k0) * Hkv + p.hk;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((role ? a.dk : a.dv) + row0 * D, nv * (int)kstride);
    const float sc = role ? a.scale : 1.f;
    uint32_t sb = (uint32_t)(4 * g) * kstride + (uint32_t)lc * 4;
    asm volatile("" : "+v"(sb));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(live ? acc[dt][i4 * 4 + e] * sc : 0.f), ro,
                                                sb + (uint32_t)(8 * i4 + e) * kstride + (uint32_t)(dt * 128), 0, 0);
  };

  Tp cp = tparams(a.ktiles[t0]);
  load_kv(cp);
  // The record of the tile after the next, loaded by lane 0 of wave 0 one
  // tile ahead and handed to every wave through LDS at the tile start, so
  // that no wave waits for it there.
  __shared__ TileRec s_rec;
  TileRec nrec{};
  {
    const int64_t t1 = zigzag_tile(1, slot, a.P);
    if (wave == 0 && l == 0 && t1 < T) nrec = a.ktiles[t1];
  }
  store_out(cp, false);  // stores that write nothing: every tile start sees NST stores after its loads

  __shared__ int s_next;
  unsigned int fetched = 0;
  for (int64_t pass = 0;; ++pass) {
    const int nsteps = cp.nj * G;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
    {
      const int need = min(DEP, nsteps);
      if (iss_cur < need) {
        while (iss_cur < need) issue_next(cp, cp, false, 2);
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<NST_WAIT>();  // (at most 63: the counter's range; waiting for more is safe)
      }
    }
    if (wave == 0 && l == 0) {
      if (pass > 0) s_next = (int)fetched;
      s_rec = nrec;
    }
    barrier_lds();
    const int64_t tn = pass == 0 ? zigzag_tile(1, slot, a.P)
                                 : 2 * (int64_t)a.P + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
    const bool has_nxt = tn < T;
    if (has_nxt && wave == 0 && l == 0) fetched = atomicAdd(a.ktile_ctr, 1u);
    const Tp np = has_nxt ? tparams(s_rec) : cp;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) asm volatile("" : "+v"(kop[kk]), "+v"(vop[kk]));
    asm volatile("" : "+v"(ksc), "+v"(vsc));
    const int g_first = g_cmp;
    const int key = cp.k0 + kw * 32 + lc;           // this lane's key (local)
    const bool wave_live = cp.k0 + kw * 32 < cp.L;  // the pair has a key of the sequence
    const int64_t base = BCAST ? 0 : cp.s0;

    auto step = [&](int j, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      if (g_cmp != g_first) wait_step(g_cmp);
      barrier_lds();
      issue_next(cp, np, has_nxt, 0);
      const char* buf = smem[(uint32_t)g_cmp % NBUF];
      ++g_cmp;
      const int qbase = (int)((int64_t)j * BQ - base);  // local index of the step's first query
      const int qt = role;
      uint32_t wq[4], wd[4], cpq = 127, cdq = 127;
      if (wave_live) {
        // S and dP for queries qt * 32 .. qt * 32 + 31 x this pair's 32 keys:
        // lane (key, g) holds query rows qt * 32 + (i / 4) * 8 + 4 g + i % 4
        const char* qr = buf + C::OFF_Q + (qt * 32 + lc) * RB;
        const char* dr = buf + C::OFF_DO + (qt * 32 + lc) * RB;
        const uint32_t qsw = *reinterpret_cast<const uint32_t*>(buf + C::OFF_QS + (qt * 32 + lc) * 4) >> (8 * g);
        const uint32_t dsw = *reinterpret_cast<const uint32_t*>(buf + C::OFF_DOS + (qt * 32 + lc) * 4) >> (8 * g);
        // dP' = dP - delta: the products start from the rows' -delta
        f32x16 dp;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4 nd = *reinterpret_cast<const f32x4*>(buf + C::OFF_DL + (qt * 32 + r * 8 + 4 * g) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[r * 4 + e] = nd[e];
        }
        f32x16 s = mfma_mx<0, 0>(lds_read32x2(qr + 16 * g, qr + 32 + 16 * g), kop[0], f32x16{}, (int)qsw, (int)ksc);
        s = mfma_mx<2, 2>(lds_read32x2(qr + 64 + 16 * g, qr + 96 + 16 * g), kop[1], s, (int)qsw, (int)ksc);
        dp = mfma_mx<0, 0>(lds_read32x2(dr + 16 * g, dr + 32 + 16 * g), vop[0], dp, (int)dsw, (int)vsc);
        dp = mfma_mx<2, 2>(lds_read32x2(dr + 64 + 16 * g, dr + 96 + 16 * g), vop[1], dp, (int)dsw, (int)vsc);
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = qt * 32 + r * 8 + 4 * g;
          const f32x4 lv = *reinterpret_cast<const f32x4*>(buf + C::OFF_L + row * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = r * 4 + e;
            float pv = fast_exp2(s[i] * c2 - lv[e]);
            if constexpr (MASKED) {
              const int q = qbase + row + e;
              const bool ok = q >= 0 && q < cp.nq && (!CAUSAL || key <= q);
              pv = ok ? pv : 0.f;
            }
            p[i] = pv;
            ds[i] = pv * dp[i];
          }
        }
        quantize_block32<false>(p, wq, &cpq);
        quantize_block32<true>(ds, wd, &cdq);
        // the partner accumulates with the other product's operand: role 0
        // hands over its dS block, role 1 its P block
        xw[wave][l] = role ? u32x4{wq[0], wq[1], wq[2], wq[3]} : u32x4{wd[0], wd[1], wd[2], wd[3]};
        xc[wave][l] = role ? cpq : cdq;
      }
      barrier_lds();
      issue_next(cp, np, has_nxt, 1);
      if (!wave_live) return;
      const u32x4 xo = xw[wave ^ (NW / 2)][l];
      const uint32_t xcode = xc[wave ^ (NW / 2)][l];
      // role 0: dV += P^T dO with P of both query blocks; role 1: dK +=
      // dS^T Q (the quantized P or dS as the A operand, dO^T or Q^T rows as
      // the B operand).  Block 0 is the role-0 wave's, block 1 the role-1
      // wave's; lane half g takes block g's scale.
      i32x8 bop;
      uint32_t bsc;
      if (role == 0) {
        bop = i32x8{(int)wq[0], (int)wq[1], (int)wq[2], (int)wq[3], (int)xo[0], (int)xo[1], (int)xo[2], (int)xo[3]};
        bsc = g == 0 ? cpq : xcode;
      } else {
        bop = i32x8{(int)xo[0], (int)xo[1], (int)xo[2], (int)xo[3], (int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        bsc = g == 0 ? xcode : cdq;
      }
      const int off_a = role ? C::OFF_QT : C::OFF_DOT;
      const int off_s = role ? C::OFF_QTS : C::OFF_DOTS;
      uint32_t asc = 0;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        asc |= (uint32_t)(*reinterpret_cast<const uint8_t*>(buf + off_s + g * D + dt * 32 + lc)) << (8 * dt);
      static_for<0, 4>([&](auto dt_tag) {
        constexpr int dt = decltype(dt_tag)::value;
        const char* ar = buf + off_a + (dt * 32 + lc) * TB;
        acc[dt] = mfma_mx<0, dt>(bop, lds_read32x2(ar + 16 * g, ar + 32 + 16 * g), acc[dt], (int)bsc, (int)asc);
      });
    };
    for (int gi = 0; gi < G; ++gi)
      for (int jj = 0; jj < cp.nj; ++jj) {
        const int j = cp.j0 + jj;
        if (j >= cp.jp0 && j < cp.jp1) step(j, std::false_type{});
        else step(j, std::true_type{});
      }

    // s_next and s_rec are rewritten at the next tile start: a tile without
    // steps has no barrier of its own after the waves read them
    if (nsteps == 0) barrier_lds();
    wait_vmcnt<IPS>();
    if (has_nxt) {
      load_kv(np);
      const int64_t t2 = 2 * (int64_t)a.P + fetched;  // the tile after np
      if (wave == 0 && l == 0 && t2 < T) nrec = a.ktiles[t2];
    }
    store_out(cp, true);
    if (!has_nxt) break;
    cp = np;
    iss_cur = iss_nxt;
    iss_nxt = 0;
  }
}

// ------------------------------------------------------------------ dQ --
struct MxQ {
  static constexpr int NW = 8, BN = 64, BM = NW * 32, D = 128, NBUF = 3, DEP = 2;
  static constexpr int OFF_K = 0;                       // K rows [64][144]
  static constexpr int OFF_V = OFF_K + BN * RB + 16;    // V rows
  static constexpr int OFF_KT = OFF_V + BN * RB + 16;   // K^T rows [128 d][80]
  static constexpr int OFF_KS = OFF_KT + D * TB + 64;   // K row scale words [64]
  static constexpr int OFF_VS = OFF_KS + BN * 4;        // V row scale words
  static constexpr int OFF_KTS = OFF_VS + BN * 4;       // K^T scales [2 key blocks][128 d]
  static constexpr int BUF = OFF_KTS + 2 * D;
  static_assert(BM == MX_BM, "the query tiles of the schedule");
  static constexpr int IPS = 9;                         // K, V, K^T (two each), three scale copies
  static constexpr int NST = 4 * 4;                     // dQ stores per wave
  static_assert(BUF % 16 == 0, "buffer alignment");
  static_assert(NBUF * BUF <= 160 * 1024, "LDS");
  static_assert(NBUF >= DEP + 1, "a buffer is refilled only after every wave has left it");
  static_assert(DEP * IPS + 12 + NST <= 63, "vector-memory counter");  // 12: loads of a tile's row operands
};

template <bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(MxQ::NW * WAVE, 1) void dq_mx_kernel(BwdMxArgs a) {
  using C = MxQ;
  constexpr int BN = C::BN, BM = C::BM, D = C::D, NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS, NST = C::NST;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][C::BUF];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const int H = a.H, Lq = a.Lq, Hkv = a.Hkv, G = a.G;
  const int64_t total = a.total_len;
  const float c2 = a.scale_log2;

  // ---- work: self mode, persistent over the query tiles; broadcast, item
  // (head, query block, chunk) walks the chunk's sequences
  const int slot = BCAST ? 0 : logical_slot(blockIdx.x, a.P);
  const int64_t T = BCAST ? 0 : *a.n_qtiles;
  int item_h = 0, item_qb = 0, item_c = 0, n_seg = 0;
  if constexpr (BCAST) {
    const int item = blockIdx.x;
    item_c = item % a.dq_chunks;
    item_qb = (item / a.dq_chunks) % a.dq_qblocks;
    item_h = item / (a.dq_chunks * a.dq_qblocks);
    n_seg = (a.B - item_c + a.dq_chunks - 1) / a.dq_chunks;
  }
  auto seg_rec = [&](int64_t i) {
    if constexpr (BCAST) {
      TileRec r;
      r.b = a.seq_order[item_c + i * a.dq_chunks];
      int64_t s0;
      r.L = (int)seq_range(a.offsets, r.b, total, &s0);
      r.s0 = s0;
      r.h = item_h;
      r.blk = item_qb;
      r.hk = item_h / G;
      r.pad = 0;
      return r;
    } else {
      return a.qtiles[i];
    }
  };
  const int64_t t0 = BCAST ? 0 : zigzag_tile(0, slot, a.P);
  if (!BCAST && t0 >= T) return;

  const uint32_t kstride = (uint32_t)Hkv * D;  // bytes between K / V rows
  const uint32_t tpad = (uint32_t)a.t_pad;     // bytes between K^T rows
  const uint32_t voff_k = row_voff(l, kstride);
  const uint32_t voff_t = trow_voff(l, tpad);
  const uint32_t nbk = tpad / 32;

  struct Tp {
    int64_t s0;
    int L, h, hk, b, q0, n_kv, J0;
    int lead, n_plain;  // steps [0, lead) and [n_plain, n_kv) take the masked body
  };
  auto tparams = [&](const TileRec& r) {
    Tp p;
    p.s0 = r.s0;
    p.L = r.L;
    p.h = r.h;
    p.hk = r.hk;
    p.b = r.b;
    p.q0 = r.blk * BM;
    const int nq = BCAST ? Lq : r.L;
    int kv_end = r.L;
    if (CAUSAL) kv_end = min(kv_end, min(p.q0 + BM, nq));
    p.J0 = (int)(r.s0 / BN);
    p.n_kv = kv_end > 0 ? (int)((r.s0 + kv_end - 1) / BN) - p.J0 + 1 : 0;
    p.lead = (r.s0 % BN != 0 && p.n_kv > 0) ? 1 : 0;
    const int lim = CAUSAL ? min(kv_end, p.q0 + 1) : kv_end;
    const int full = (int)((r.s0 + lim) / BN) - p.J0;
    p.n_plain = min(max(full, p.lead), p.n_kv);
    return p;
  };

  int g_iss = 0, g_cmp = 0, iss_cur = 0, iss_nxt = 0;
  const int64_t kt_bytes = (int64_t)Hkv * D * tpad;
  // part 0: K and V rows and their scales (after the step's barrier), 1: the
  // K^T rows and scales (after the first key half's dS), 2: both.
  auto issue_next = [&](const Tp& cp, const Tp& np, bool has_nxt, int part) {
    const bool cur = iss_cur < cp.n_kv;
    if (!(cur || (has_nxt && iss_nxt < np.n_kv))) return;
    const Tp& p = cur ? cp : np;
    const int J = p.J0 + (cur ? iss_cur : iss_nxt);
    const int64_t krow = (int64_t)J * BN + wave * 8;
    const int nrow = (int)max((int64_t)0, min(total - krow, (int64_t)9));
    const int nsc = min(nrow, 8);
    const int64_t row = krow * Hkv + p.hk;
    const int64_t t_off = ((int64_t)p.hk * D + wave * 16) * tpad + (int64_t)J * BN;
    const uint32_t buf = lds_addr(smem[(uint32_t)g_iss % NBUF]);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k8 + row * D, nrow * (int)kstride);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v8 + row * D, nrow * (int)kstride);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(a.kt8 + t_off, (int)min(kt_bytes - t_off, (int64_t)(17 * tpad)));
    if (part != 1) {
      const uint32_t kd = buf + C::OFF_K + wave * 8 * RB;
      dma_copy16_buf(rk, voff_k, 0, kd);
      dma_copy16_buf(rk, voff_k, kstride, kd + RB);
      const uint32_t vd = buf + C::OFF_V + wave * 8 * RB;
      dma_copy16_buf(rv, voff_k, 0, vd);
      dma_copy16_buf(rv, voff_k, kstride, vd + RB);
      if (l < 8) {
        dma_copy4_buf(make_rsrc(a.k_scale + row * 4, nsc * Hkv * 4), (uint32_t)l * Hkv * 4, 0,
                      buf + C::OFF_KS + wave * 32);
        dma_copy4_buf(make_rsrc(a.v_scale + row * 4, nsc * Hkv * 4), (uint32_t)l * Hkv * 4, 0,
                      buf + C::OFF_VS + wave * 32);
      }
    }
    if (part == 0) return;
    const uint32_t td = buf + C::OFF_KT + wave * 16 * TB;
    dma_copy16_buf(rt, voff_t, 0, td);
    dma_copy16_buf(rt, voff_t, 4 * tpad, td + 4 * TB);
    if (l < 8) {
      dma_copy4_buf(make_rsrc(a.kt_scale + ((int64_t)p.hk * nbk + 2 * J) * D + wave * 32, 32), (uint32_t)l * 4, 0,
                    buf + C::OFF_KTS + wave * 32);
    }
    if (cur) ++iss_cur;
    else ++iss_nxt;
    ++g_iss;
  };
  auto wait_step = [&](int gi) {
    const int after = g_iss - 1 - gi;
    if (after >= 1) wait_vmcnt<IPS>();
    else wait_vmcnt<0>();
  };

  // ---- this lane's query row: Q and dO (B operands of S^T and dP^T, laid
  // out as the forward's Q), lse * log2(e) and delta.  Rows past the
  // queries read the block's first row; they are never stored.
  i32x8 qop[2], dop[2];
  uint32_t qsc = 0, dsc = 0;
  float lq2 = 0.f, dlt = 0.f;  // lse * log2(e) and -delta of this lane's row
  auto load_q = [&](const Tp& p) {
    const int nq = BCAST ? Lq : p.L;
    int qi = p.q0 + wave * 32 + lc;
    qi = qi < nq ? qi : p.q0 < nq ? p.q0 : 0;
    const int64_t qrow = BCAST ? (int64_t)p.h * Lq + qi : (p.s0 + qi) * H + p.h;
    const int64_t drow = BCAST ? ((int64_t)p.b * H + p.h) * Lq + qi : qrow;
    const uint8_t* qr = a.q8 + qrow * D;
    const uint8_t* dr = a.do8 + drow * D;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      qop[kk] = ld32x2(qr + 64 * kk + 16 * g, qr + 64 * kk + 32 + 16 * g);
      dop[kk] = ld32x2(dr + 64 * kk + 16 * g, dr + 64 * kk + 32 + 16 * g);
    }
    qsc = *reinterpret_cast<const uint32_t*>(a.q_scale + qrow * 4) >> (8 * g);
    dsc = *reinterpret_cast<const uint32_t*>(a.do_scale + drow * 4) >> (8 * g);
    lq2 = a.lse2[drow];
    dlt = a.delta[drow];
  };

  f32x16 acc[4];
  // dQ rows of a self-mode tile (scale applied), or the broadcast partial
  auto store_out = [&](const Tp& p, int nrows) {
    __amdgpu_buffer_rsrc_t ro;
    uint32_t rowb;
    float sc;
    if constexpr (BCAST) {
      const int64_t item = ((int64_t)item_h * a.dq_qblocks + item_qb) * a.dq_chunks + item_c;
      ro = make_rsrc(a.dq_part + (item * BM + wave * 32) * D, nrows > 0 ? 32 * D * 4 : 0);
      rowb = D * 4;
      sc = 1.f;
    } else {
      const int r0 = p.q0 + wave * 32;
      const int nv = max(0, min(nrows - r0, 32));
      ro = make_rsrc(a.dq + ((p.s0 + r0) * H + p.h) * D, nv * H * D * 4);
      rowb = (uint32_t)H * D * 4;
      sc = a.scale;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[dt][i4 * 4 + e] * sc;
        const uint32_t off = (uint32_t)lc * rowb + (uint32_t)(dt * 32 + i4 * 8 + g * 4) * 4u;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, off, 0, 0);
      }
  };

#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  if constexpr (BCAST) {
    if (n_seg == 0) {  // a chunk without sequences: its partial is zero
      store_out(Tp{}, 1);
      return;
    }
  }
  Tp cp = tparams(seg_rec(t0));
  load_q(cp);
  if constexpr (!BCAST) store_out(cp, 0);  // stores that write nothing, as at every later tile start

  __shared__ int s_next;
  unsigned int fetched = 0;
  for (int64_t pass = 0;; ++pass) {
    const int64_t s0 = cp.s0;
    const int L = cp.L, q0 = cp.q0, n_kv = cp.n_kv;
    const int nq = BCAST ? Lq : L;
    const int qrow = q0 + wave * 32 + lc;
    if constexpr (!BCAST) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
    }
    {
      const int need = min(DEP, n_kv);
      if (iss_cur < need) {
        while (iss_cur < need) issue_next(cp, cp, false, 2);
        wait_vmcnt<0>();
      } else if (BCAST) {
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<NST>();
      }
    }
    int64_t tn;
    if constexpr (BCAST) {
      barrier_lds();
      tn = pass + 1;
    } else {
      if (pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
      barrier_lds();
      tn = pass == 0 ? zigzag_tile(1, slot, a.P) : 2 * (int64_t)a.P + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
    }
    const bool has_nxt = BCAST ? tn < n_seg : tn < T;
    if constexpr (!BCAST) {
      if (has_nxt && wave == 0 && l == 0) fetched = atomicAdd(a.qtile_ctr, 1u);
    }
    const Tp np = has_nxt ? tparams(seg_rec(tn)) : cp;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) asm volatile("" : "+v"(qop[kk]), "+v"(dop[kk]));
    asm volatile("" : "+v"(qsc), "+v"(dsc), "+v"(lq2), "+v"(dlt));
    // dP' = dP - delta of this lane's row: the dP products of every step
    // start from it
    f32x16 ndel;
#pragma unroll
    for (int i = 0; i < 16; ++i) ndel[i] = dlt;
    const int g_first = g_cmp;

    auto kv_step = [&](int j, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      if (g_cmp != g_first) wait_step(g_cmp);
      barrier_lds();
      issue_next(cp, np, has_nxt, 0);
      const char* buf = smem[(uint32_t)g_cmp % NBUF];
      const int kbase = (cp.J0 + j) * BN - (int)s0;
      uint32_t sw[8];
      uint32_t ssc = 127;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const char* kr = buf + C::OFF_K + (kt * 32 + lc) * RB;
        const char* vr = buf + C::OFF_V + (kt * 32 + lc) * RB;
        const uint32_t ksw = *reinterpret_cast<const uint32_t*>(buf + C::OFF_KS + (kt * 32 + lc) * 4) >> (8 * g);
        const uint32_t vsw = *reinterpret_cast<const uint32_t*>(buf + C::OFF_VS + (kt * 32 + lc) * 4) >> (8 * g);
        f32x16 s = mfma_mx<0, 0>(lds_read32x2(kr + 16 * g, kr + 32 + 16 * g), qop[0], f32x16{}, (int)ksw, (int)qsc);
        s = mfma_mx<2, 2>(lds_read32x2(kr + 64 + 16 * g, kr + 96 + 16 * g), qop[1], s, (int)ksw, (int)qsc);
        f32x16 dp = mfma_mx<0, 0>(lds_read32x2(vr + 16 * g, vr + 32 + 16 * g), dop[0], ndel, (int)vsw, (int)dsc);
        dp = mfma_mx<2, 2>(lds_read32x2(vr + 64 + 16 * g, vr + 96 + 16 * g), dop[1], dp, (int)vsw, (int)dsc);
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(s[i] * c2 - lq2);
          if constexpr (MASKED) {
            const int key = kbase + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
            const bool ok = key >= 0 && key < L && (!CAUSAL || key <= qrow);
            pv = ok ? pv : 0.f;
          }
          ds[i] = pv * dp[i];
        }
        uint32_t w[4], code;
        quantize_block32<true>(ds, w, &code);
#pragma unroll
        for (int q = 0; q < 4; ++q) sw[kt * 4 + q] = w[q];
        ssc = g == kt ? code : ssc;
        if (kt == 0) issue_next(cp, np, has_nxt, 1);
      }
      const i32x8 sop = i32x8{(int)sw[0], (int)sw[1], (int)sw[2], (int)sw[3],
                              (int)sw[4], (int)sw[5], (int)sw[6], (int)sw[7]};
      // dQ^T += K^T dS^T over the step's 64 keys, 4 head-dim tiles of 32
      uint32_t tsw = 0;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        tsw |= (uint32_t)(*reinterpret_cast<const uint8_t*>(buf + C::OFF_KTS + g * D + dt * 32 + lc)) << (8 * dt);
      static_for<0, 4>([&](auto dt_tag) {
        constexpr int dt = decltype(dt_tag)::value;
        const char* tr = buf + C::OFF_KT + (dt * 32 + lc) * TB;
        acc[dt] = mfma_mx<dt, 0>(lds_read32x2(tr + 16 * g, tr + 32 + 16 * g), sop, acc[dt], (int)tsw, (int)ssc);
      });
      ++g_cmp;
    };
    for (int j = 0; j < cp.lead; ++j) kv_step(j, std::true_type{});
    for (int j = cp.lead; j < cp.n_plain; ++j) kv_step(j, std::false_type{});
    for (int j = max(cp.n_plain, cp.lead); j < n_kv; ++j) kv_step(j, std::true_type{});

    if (has_nxt) load_q(np);
    if constexpr (!BCAST) store_out(cp, nq);
    if (!has_nxt) break;
    cp = np;
    iss_cur = iss_nxt;
    iss_nxt = 0;
  }
  if constexpr (BCAST) store_out(cp, 1);
}

}  // namespace

hipError_t launch_bwd_mx(const BwdMxArgs& a, hipStream_t st) {
  const int64_t rows = a.broadcast_q ? (int64_t)a.B * a.H * a.Lq : a.total_len * a.H;
  hipError_t e;
  if (rows > 0) {
    const int64_t want = (rows * 8 + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    JFA_TIMED_LAUNCH(K_DELTA_MX, st, delta_mx_kernel, dim3(blocks), dim3(256), 0, st, a.out, a.do8, a.do_scale,
                     a.lse, a.delta, a.lse2, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 blk(MxB::NW * WAVE);
  if (a.causal) {
    if (a.broadcast_q) JFA_TIMED_LAUNCH(K_DKDV_MX, st, (dkdv_mx_kernel<true, true>), dim3(a.P), blk, 0, st, a);
    else JFA_TIMED_LAUNCH(K_DKDV_MX, st, (dkdv_mx_kernel<true, false>), dim3(a.P), blk, 0, st, a);
  } else {
    if (a.broadcast_q) JFA_TIMED_LAUNCH(K_DKDV_MX, st, (dkdv_mx_kernel<false, true>), dim3(a.P), blk, 0, st, a);
    else JFA_TIMED_LAUNCH(K_DKDV_MX, st, (dkdv_mx_kernel<false, false>), dim3(a.P), blk, 0, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 qblk(MxQ::NW * WAVE);
  if (a.broadcast_q) {
    const dim3 grid((unsigned)(a.H * a.dq_qblocks * a.dq_chunks));
    if (a.causal) JFA_TIMED_LAUNCH(K_DQ_MX, st, (dq_mx_kernel<true, true>), grid, qblk, 0, st, a);
    else JFA_TIMED_LAUNCH(K_DQ_MX, st, (dq_mx_kernel<false, true>), grid, qblk, 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_dq_reduce(a.dq_part, a.dq, a.H, a.Lq, 128, MX_BM, a.dq_qblocks, a.dq_chunks, a.scale, st);
  }
  if (a.causal) JFA_TIMED_LAUNCH(K_DQ_MX, st, (dq_mx_kernel<true, false>), dim3(a.P), qblk, 0, st, a);
  else JFA_TIMED_LAUNCH(K_DQ_MX, st, (dq_mx_kernel<false, false>), dim3(a.P), qblk, 0, st, a);
  return hipGetLastError();
}

}  // namespace jfa
