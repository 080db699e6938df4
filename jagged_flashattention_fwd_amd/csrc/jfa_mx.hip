// MXFP8 jagged attention forward on gfx950 (d = 128).
//
// "Optimizing Jagged Flash Attention with TLX", "Low-precision (MXFP8)
// attention": both products of the forward take block-scaled FP8 operands
// (E4M3 elements, one E8M0 scale per 32 elements along the product's
// reduction dimension), and the softmax output P is quantized to FP8 on the
// fly.  Here the products are
//   S^T  = K Q^T    v_mfma_scale_f32_32x32x64_f8f6f4, reduction over d
//   O^T += V^T P^T  the same instruction, reduction over 64 keys
// (operand layout in jfa_mx.hpp).
//
// Inputs (one reading of the page, which gives none): Q and K rows as E4M3
// with one scale per 32 head-dim elements; V transposed, [H_kv, d, T_pad]
// (T_pad = total_len rounded up to 64), with one scale per 32 keys of the
// packed key index, [H_kv, T_pad / 32, d].  Key steps follow that index (64
// keys from a multiple of 64), so a step's two scale blocks are whole; keys
// of a neighbouring sequence in a step are masked.
//
// P: the running maximum is kept at whole numbers (log2 units).  P is
// exp2(s c - m), its block maximum b over 32 keys of a query row gives the
// scale 2^(floor(log2 b) - 8), and P / scale, capped at 448, is rounded to
// E4M3 by the conversion instruction (nearest, ties to even).  Because E4M3's
// grid is closed under powers of two, the quantized block times its scale
// does not depend on which whole-number reference m is used.  The row sums
// l take the unquantized P; O = (quantized P) V / l, lse = (m + log2 l) ln 2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_mx.hpp"
#include "jfa_timing.hpp"

namespace jfa {
namespace {

struct Mx {
  static constexpr int NW = 8, BN = 64, BM = NW * 32, D = 128, NBUF = 4, DEP = 2;
  // K rows: 128 bytes + 16 of padding (16-byte reads of 16 consecutive rows
  // hit 16 distinct bank groups); V^T rows (64 keys): 64 + 16.
  static constexpr int K_RB = 144, V_RB = 80;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_V = OFF_K + BN * K_RB + 16;        // after the K copies' overhang
  static constexpr int OFF_KS = OFF_V + D * V_RB + 64;        // after the V copies' overhang
  static constexpr int OFF_VS = OFF_KS + BN * 4;              // [2 key blocks][128 d]
  static constexpr int BUF = OFF_VS + 2 * D;
  // Copies per wave per step: K (8 rows, 7 per copy: starts 0 and 1), V^T
  // (16 rows, 12 per copy: starts 0 and 4), K scales, V scales.
  static constexpr int IPS = 6;
  static constexpr int NST = 2 * 4 + 1;  // stores per wave at a tile end: O pieces and lse
  static_assert(BUF % 16 == 0, "buffer alignment");
  static_assert(NBUF * BUF <= 160 * 1024, "LDS");
  static_assert(DEP * IPS + NST <= 63, "vector-memory counter");
};

template <bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(Mx::NW * WAVE, 1) void fwd_mx_kernel(FwdMxArgs a, const TileRec* __restrict__ tiles) {
  using C = Mx;
  constexpr int BN = C::BN, BM = C::BM, D = C::D, NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS, NST = C::NST;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][C::BUF];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_tiles;
  const int H = a.H, Lq = a.Lq, Hkv = a.Hkv;
  const int64_t total = a.total_len;
  // A negative scale is folded into Q: the sign bits of its E4M3 codes flip
  // at its load (exact), so that every score below is (-q) k with the
  // scale's magnitude and the softmax keeps one form.
  const float c2 = __builtin_fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80808080u : 0u;

  const int64_t t0 = zigzag_tile(0, slot, a.P);
  if (t0 >= T) return;

  // ---- per-lane copy geometry (fixed for the kernel)
  const uint32_t kstride = (uint32_t)Hkv * D;  // bytes between K rows
  const uint32_t tpad = (uint32_t)a.t_pad;     // bytes between V^T rows
  const uint32_t voff_k = (uint32_t)(l / 9) * kstride + ((l % 9) < 8 ? (uint32_t)(l % 9) * 16u : 0u);
  const uint32_t voff_v = (uint32_t)(l / 5) * tpad + ((l % 5) < 4 ? (uint32_t)(l % 5) * 16u : 0u);
  const uint32_t nbk = tpad / 32;  // key blocks per V^T row

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
    // a step is plain when its keys all exist and (causal) all precede the
    // tile's first query row
    const int lim = CAUSAL ? min(kv_end, p.q0 + 1) : kv_end;
    const int full = (int)((r.s0 + lim) / BN) - p.J0;
    p.n_plain = min(max(full, p.lead), p.n_kv);
    return p;
  };

  // ---- the step stream (as in the bf16 forward): g_iss / g_cmp steps
  // issued / computed; iss_cur / iss_nxt of the current / next tile.
  int g_iss = 0, g_cmp = 0, iss_cur = 0, iss_nxt = 0;
  __amdgpu_buffer_rsrc_t j_rk = make_rsrc(a.k8, 0), j_rv = make_rsrc(a.vt8, 0);
  __amdgpu_buffer_rsrc_t j_rks = make_rsrc(a.k_scale, 0), j_rvs = make_rsrc(a.vt_scale, 0);
  uint32_t j_buf = 0;
  bool j_on = false;
  auto prep_next = [&](const Tp& cp, const Tp& np, bool has_nxt) {
    const bool cur = iss_cur < cp.n_kv;
    j_on = cur || (has_nxt && iss_nxt < np.n_kv);
    if (!j_on) return;
    const Tp& p = cur ? cp : np;
    const int J = p.J0 + (cur ? iss_cur : iss_nxt);
    // K: this wave's 8 rows (and the one after), rows past the tensor read as zeros
    const int64_t krow = (int64_t)J * BN + wave * 8;
    const int krows = (int)max((int64_t)0, min(total - krow, (int64_t)9));
    j_rk = make_rsrc(a.k8 + (krow * Hkv + p.hk) * D, krows * (int)kstride);
    const int ksr = (int)max((int64_t)0, min(total - krow, (int64_t)8));
    j_rks = make_rsrc(a.k_scale + (krow * Hkv + p.hk) * 4, ksr * Hkv * 4);
    // V^T: this wave's 16 d-rows (and the one after, inside the tensor), keys
    // 64 J .. 64 J + 63
    const int64_t vrow = (int64_t)p.hk * D + wave * 16;
    const int64_t vbytes = (int64_t)Hkv * D * tpad - (vrow * tpad + (int64_t)J * BN);
    j_rv = make_rsrc(a.vt8 + vrow * tpad + (int64_t)J * BN, (int)min(vbytes, (int64_t)(17 * tpad)));
    j_rvs = make_rsrc(a.vt_scale + ((int64_t)p.hk * nbk + 2 * J) * D + wave * 32, 32);
    j_buf = lds_addr(smem[(uint32_t)g_iss % NBUF]);
    if (cur) ++iss_cur;
    else ++iss_nxt;
    ++g_iss;
  };
  auto issue_copies = [&](int part) {  // 0: K and scales, 1: V^T
    if (!j_on) return;
    if (part != 1) {
      const uint32_t kd = j_buf + C::OFF_K + wave * 8 * C::K_RB;
      dma_copy16_buf(j_rk, voff_k, 0, kd);
      dma_copy16_buf(j_rk, voff_k, kstride, kd + C::K_RB);
      if (l < 8) {
        dma_copy4_buf(j_rks, (uint32_t)l * Hkv * 4, 0, j_buf + C::OFF_KS + wave * 32);
        dma_copy4_buf(j_rvs, (uint32_t)l * 4, 0, j_buf + C::OFF_VS + wave * 32);
      }
    }
    if (part != 0) {
      const uint32_t vd = j_buf + C::OFF_V + wave * 16 * C::V_RB;
      dma_copy16_buf(j_rv, voff_v, 0, vd);
      dma_copy16_buf(j_rv, voff_v, 4 * tpad, vd + 4 * C::V_RB);
    }
  };
  auto wait_step = [&](int gi) {
    const int after = g_iss - 1 - gi;
    if (after >= 1) wait_vmcnt<IPS>();
    else wait_vmcnt<0>();
  };

  // ---- Q operand (B of S^T = K Q^T): lane (query row, g) holds bytes
  // 16 g .. 16 g + 15 of blocks 2 kk and 2 kk + 1 for kk = 0, 1; its scale
  // word shifted so that byte 2 kk is block 2 kk + g's scale.
  i32x8 qop[2];
  uint32_t qsc = 0;
  auto load_q = [&](const Tp& p) {
    const int nq = BCAST ? Lq : p.L;
    int qi = p.q0 + wave * 32 + lc;
    qi = qi < nq ? qi : p.q0 < nq ? p.q0 : 0;
    const int64_t row = BCAST ? (int64_t)p.h * Lq + qi : (p.s0 + qi) * H + p.h;
    const uint8_t* qr = a.q8 + row * D;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(qr + 64 * kk + 16 * g);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(qr + 64 * kk + 32 + 16 * g);
      qop[kk] = i32x8{(int)(x0[0] ^ qsign), (int)(x0[1] ^ qsign), (int)(x0[2] ^ qsign), (int)(x0[3] ^ qsign),
                      (int)(x1[0] ^ qsign), (int)(x1[1] ^ qsign), (int)(x1[2] ^ qsign), (int)(x1[3] ^ qsign)};
    }
    qsc = *reinterpret_cast<const uint32_t*>(a.q_scale + row * 4) >> (8 * g);
  };

  f32x16 oacc[4];
  float m2 = -INFINITY, lsum = 0.f;
  // O = acc / l (bf16) and lse of a tile: NST bounded buffer stores per wave
  auto store_out = [&](const Tp& p, int nrows) {
    const int r0 = p.q0 + wave * 32;
    const int nv = max(0, min(nrows - r0, 32));
    const int64_t orow0 = BCAST ? ((int64_t)p.b * H + p.h) * Lq + r0 : (p.s0 + r0) * H + p.h;
    const int ostride = BCAST ? D : H * D;
    const int lstride = BCAST ? 1 : H;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + orow0 * D, nv * ostride * 2);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + orow0, nv * lstride * 4);
    const float lt = sum_across_halves(lsum);
    const float inv = lt > 0.f ? fast_rcp(lt) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        uint32_t w[2][2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i4 = 2 * p2 + k;
          w[k][0] = pack_bf16x2(oacc[dt][i4 * 4 + 0] * inv, oacc[dt][i4 * 4 + 1] * inv);
          w[k][1] = pack_bf16x2(oacc[dt][i4 * 4 + 2] * inv, oacc[dt][i4 * 4 + 3] * inv);
        }
        const uint32_t s0w = g ? w[0][0] : w[1][0], s1w = g ? w[0][1] : w[1][1];
        const uint32_t r0w = (uint32_t)__shfl_xor((int)s0w, 32), r1w = (uint32_t)__shfl_xor((int)s1w, 32);
        u32x4 v;
        if (g == 0) v = u32x4{w[0][0], w[0][1], r0w, r1w};
        else v = u32x4{r0w, r1w, w[1][0], w[1][1]};
        const int d0 = dt * 32 + p2 * 16 + g * 8;
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, (lc * ostride + d0) * 2, 0, 0);
      }
    const float lse = lt > 0.f ? (m2 + fast_log2(lt)) * LN2 : -INFINITY;
    const uint32_t loff = g == 0 ? (uint32_t)(lc * lstride * 4) : 0xfffffff0u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, loff, 0, 0);
  };

  Tp cp = tparams(tiles[t0]);
  load_q(cp);
  {
    // stores that write nothing, so that every tile start sees the same
    // operations after its Q loads
    lsum = 0.f;
    m2 = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
    store_out(cp, 0);
  }

  __shared__ int s_next;
  unsigned int fetched = 0;
  for (int64_t pass = 0;; ++pass) {
    const int64_t s0 = cp.s0;
    const int L = cp.L, q0 = cp.q0, n_kv = cp.n_kv;
    const int nq = BCAST ? Lq : L;
    const int qrow = q0 + wave * 32 + lc;  // this lane's query row (local)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
    m2 = -INFINITY;
    lsum = 0.f;

    // tile start: its first min(DEP, n_kv) steps were normally issued during
    // the previous tile; only the previous tile's stores may be outstanding
    {
      const int need = min(DEP, n_kv);
      if (iss_cur < need) {
        while (iss_cur < need) {
          prep_next(cp, cp, false);
          issue_copies(2);
        }
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<NST>();
      }
    }
    if (pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
    barrier_lds();
    const int64_t tn = pass == 0 ? zigzag_tile(1, slot, a.P)
                                 : 2 * (int64_t)a.P + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
    const bool has_nxt = tn < T;
    if (has_nxt && wave == 0 && l == 0) fetched = atomicAdd(a.tile_ctr, 1u);
    const Tp np = has_nxt ? tparams(tiles[tn]) : cp;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) asm volatile("" : "+v"(qop[kk]));
    asm volatile("" : "+v"(qsc));
    const int g_first = g_cmp;

    auto kv_step = [&](int j, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      if (g_cmp != g_first) wait_step(g_cmp);
      barrier_lds();
      prep_next(cp, np, has_nxt);
      issue_copies(0);
      const char* buf = smem[(uint32_t)g_cmp % NBUF];
      const int kbase = (cp.J0 + j) * BN - (int)s0;  // local index of the step's first key

      // ---- S^T = K Q^T: 2 key subtiles x 2 halves of d
      f32x16 sacc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const char* kr = buf + C::OFF_K + (kt * 32 + lc) * C::K_RB;
        const uint32_t ksw = *reinterpret_cast<const uint32_t*>(buf + C::OFF_KS + (kt * 32 + lc) * 4) >> (8 * g);
        const i32x8 k0 = lds_read32x2(kr + 16 * g, kr + 32 + 16 * g);
        const i32x8 k1 = lds_read32x2(kr + 64 + 16 * g, kr + 96 + 16 * g);
        sacc[kt] = mfma_mx<0, 0>(k0, qop[0], f32x16{}, (int)ksw, (int)qsc);
        sacc[kt] = mfma_mx<2, 2>(k1, qop[1], sacc[kt], (int)ksw, (int)qsc);
      }
      // ---- row maximum (log2 units).  Unmasked steps reduce the raw scores
      // and fold the scale into the exponent's fma below; masked steps scale
      // first and set masked keys to -inf.
      float mt = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if constexpr (MASKED) {
            float x = sacc[kt][i] * c2;
            const int key = kbase + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
            const bool ok = key >= 0 && key < L && (!CAUSAL || key <= qrow);
            x = ok ? x : -INFINITY;
            sacc[kt][i] = x;
            mt = fmaxf(mt, x);
          } else {
            mt = fmaxf(mt, sacc[kt][i]);
          }
        }
      issue_copies(1);
      mt = max_across_halves(mt);
      if constexpr (!MASKED) mt *= c2;
      // the running maximum moves in whole numbers, and only past a slack of 8
      if (__builtin_expect(__any(mt > m2 + 8.f), 0)) {
        if (mt > m2 + 8.f) {
          const float mn = ceilf(mt);
          const float alpha = m2 == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(m2 - mn));
          m2 = mn;
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
        }
      }
      const float mref = m2 == -INFINITY ? 0.f : m2;
      // ---- P, its row sum, and its E4M3 codes per 32-key block
      uint32_t pb[8];      // B operand: [block 0: 4 words][block 1: 4 words]
      uint32_t pscale = 127;
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float p[16];
        float bm = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = MASKED ? fast_exp2(sacc[kt][i] - mref) : fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -mref));
          ls += p[i];
          bm = fmaxf(bm, p[i]);
        }
        bm = max_across_halves(bm);
        const uint32_t be = __float_as_uint(bm) >> 23;  // biased exponent of the block maximum
        const bool live = be >= 27u;                      // maximum at least 2^-100, else the block is 0
        const float cap = live ? mx_block_cap(be) : 0.f;  // 448 times the block scale, before the division
        const float scale = live ? mx_block_scale(be) : 1.f;
        const uint32_t code = live ? be - 8u : 127u;      // E8M0 of 2^(floor(log2 bm) - 8)
        pscale = g == kt ? code : pscale;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float* v = p + 4 * q;
          uint32_t x = cvt_e4m3x2_scaled<false>(fminf(v[0], cap), fminf(v[1], cap), scale, 0u);
          w[q] = cvt_e4m3x2_scaled<true>(fminf(v[2], cap), fminf(v[3], cap), scale, x);
        }
        // lo = keys 4g + {0..3, 8..11}, hi = keys 16 + 4g + {0..3, 8..11}:
        // the lower half takes the upper half's lo, the upper half the
        // lower half's hi, so that lane half g holds keys 16 g .. 16 g + 15
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          auto sw = __builtin_amdgcn_permlane32_swap(w[q], w[2 + q], false, false);
          pb[kt * 4 + 2 * q] = sw[0];
          pb[kt * 4 + 2 * q + 1] = sw[1];
        }
      }
      lsum += ls;
      const i32x8 pop = i32x8{(int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3],
                              (int)pb[4], (int)pb[5], (int)pb[6], (int)pb[7]};
      // ---- O^T += V^T P^T over the step's 64 keys, 4 head-dim tiles of 32
      uint32_t vsw = 0;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vsw |= (uint32_t)(*reinterpret_cast<const uint8_t*>(buf + C::OFF_VS + g * D + dt * 32 + lc)) << (8 * dt);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* vr = buf + C::OFF_V + (dt * 32 + lc) * C::V_RB;
        const i32x8 vo = lds_read32x2(vr + 16 * g, vr + 32 + 16 * g);
        switch (dt) {
          case 0: oacc[0] = mfma_mx<0, 0>(vo, pop, oacc[0], (int)vsw, (int)pscale); break;
          case 1: oacc[1] = mfma_mx<1, 0>(vo, pop, oacc[1], (int)vsw, (int)pscale); break;
          case 2: oacc[2] = mfma_mx<2, 0>(vo, pop, oacc[2], (int)vsw, (int)pscale); break;
          default: oacc[3] = mfma_mx<3, 0>(vo, pop, oacc[3], (int)vsw, (int)pscale); break;
        }
      }
      ++g_cmp;
    };
    for (int j = 0; j < cp.lead; ++j) kv_step(j, std::true_type{});
    for (int j = cp.lead; j < cp.n_plain; ++j) kv_step(j, std::false_type{});
    for (int j = max(cp.n_plain, cp.lead); j < n_kv; ++j) kv_step(j, std::true_type{});

    // a tile without steps has no barrier after the waves read s_next,
    // which wave 0 rewrites at the next tile start
    if (g_cmp == g_first) barrier_lds();
    // the next tile's Q rows, then this tile's stores
    if (has_nxt) load_q(np);
    store_out(cp, nq);
    if (!has_nxt) break;
    cp = np;
    iss_cur = iss_nxt;
    iss_nxt = 0;
  }
}

}  // namespace

hipError_t launch_fwd_mx(const FwdMxArgs& a, hipStream_t stream) {
  const dim3 grid(a.P), block(Mx::NW * WAVE);
  if (a.causal) {
    if (a.broadcast_q) JFA_TIMED_LAUNCH(K_FWD_MX, stream, (fwd_mx_kernel<true, true>), grid, block, 0, stream, a, a.tiles);
    else JFA_TIMED_LAUNCH(K_FWD_MX, stream, (fwd_mx_kernel<true, false>), grid, block, 0, stream, a, a.tiles);
  } else {
    if (a.broadcast_q) JFA_TIMED_LAUNCH(K_FWD_MX, stream, (fwd_mx_kernel<false, true>), grid, block, 0, stream, a, a.tiles);
    else JFA_TIMED_LAUNCH(K_FWD_MX, stream, (fwd_mx_kernel<false, false>), grid, block, 0, stream, a, a.tiles);
  }
  return hipGetLastError();
}

}  // namespace jfa
