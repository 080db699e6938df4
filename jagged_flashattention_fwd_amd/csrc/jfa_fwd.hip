// Jagged flash-attention forward for gfx950.
//
// Computes O = softmax(scale * Q K^T) V and lse = log sum exp(scale * Q K^T)
// for every (sequence, head) of a packed batch, with the online-softmax
// recurrence of "cuTile Kernels -- FMHA Implementation" ("Flash Attention
// Algorithm"): running maximum, running sum and accumulator carried over K/V
// tiles.  Sequences are packed with no padding and delimited by an offsets
// tensor ("Optimizing Jagged Flash Attention with TLX", "Introduction"); in
// broadcast mode one dense Q is shared by all sequences ("1. The
// Challenge").
//
// Work unit: a tile = BM query rows of one (sequence, head).  The kernel is
// persistent ("2.1 Structural changes"): P workgroups walk a device-built,
// longest-first tile list in zigzag order ("Scheduling jagged tiles across
// SMs").  Wave w of a workgroup owns QW consecutive query rows.
//
// Per K/V step of 64 keys the math is done transposed, S^T = K Q^T, so a lane
// owns one query column: the row max and row sum of the online softmax are
// per-lane register reductions plus one cross-half swap, and P^T is already
// the B operand of O^T += V^T P^T.  K and V are staged row-major in LDS
// (double buffered, loads of the next step overlap the math of this one); K
// feeds the A operand with 16-byte reads and V^T is read with the LDS
// transpose read.  The K/V loop is peeled ("Loop peeling"): a mask-free bulk
// and masked tail / causal-diagonal steps.  Scores are exponentiated with
// exp2 after folding log2(e) into the scale ("exp2 + flush_to_zero"), and the
// final normalisation uses the hardware reciprocal ("Approximate Division").
// The running maximum is only moved when a new maximum exceeds it by more
// than 2^8 (in exp2 units); until then exponentials are taken against the
// stale maximum, which leaves O and lse unchanged up to rounding and skips
// most rescaling of the accumulator.
#include <type_traits>

#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

constexpr float RESCALE_SLACK = 8.0f;  // log2 units

template <int D, int NW, int QW, bool CAUSAL, bool BCAST>
struct Fwd {
  static constexpr int NT = NW * WAVE;
  static constexpr int BN = FWD_KV_STEP;
  static constexpr int QS = QW / 32;   // 32-row query subtiles per wave
  static constexpr int BM = NW * QW;
  static constexpr int KS = D / 16;    // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;    // 32-wide head-dim tiles of O^T
  static constexpr int TILE_BYTES = tile_bytes<BN, D>();
  // d = 128: K/V rows go straight from global memory to LDS (three padded
  // rows per copy), DEP steps ahead of the one being computed, in a ring of
  // DEP + 1 buffers.  Each wave copies RPW rows of K and of V per step, IPS
  // copies; the vector-memory counter can hold at most 63 outstanding
  // operations, which bounds DEP.
  // d = 64: rows are staged through registers one step ahead.
  static constexpr bool DMA = D == 128;
  static constexpr int RPW = BN / NW;
  static constexpr int CPT = PadRowCopy::copies(RPW);
  static constexpr int IPS = 2 * CPT;
  static constexpr int DEP = DMA ? ((2 * IPS <= 63) ? 3 : 2) : 1;
  static constexpr int NBUF = DEP + 1;
  static constexpr int BUF_BYTES = TILE_BYTES + PadRowCopy::GAP;
  static_assert(!DMA || (TileGeom<D>::ROW_BYTES == 19 * 16 && RPW >= 3), "copy geometry");
};

template <int D, int NW, int QW, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(NW * WAVE, 1) void fwd_kernel(FwdArgs a) {
  using C = Fwd<D, NW, QW, CAUSAL, BCAST>;
  constexpr int BN = C::BN, QS = C::QS, BM = C::BM, KS = C::KS, DT = C::DT, NT = C::NT;
  constexpr int NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][2][C::BUF_BYTES];  // [buffer][K, V]

  const int tid = threadIdx.x;
  const int wave = tid / WAVE, l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_tiles;
  const int H = a.H;
  const int64_t ld = (int64_t)H * D;  // packed row stride (elements)
  const float c2 = a.scale_log2;

  for (int64_t pass = 0;; ++pass) {
    const int64_t t = zigzag_tile(pass, slot, a.P);
    if (t >= T) break;
    const TileRec tile = a.tiles[t];
    int64_t s0;
    const int L = (int)seq_range(a.offsets, tile.b, a.total_len, &s0);
    const int h = tile.h;
    const int q0 = tile.blk * BM;
    const int nq = BCAST ? a.Lq : L;
    const int wq0 = q0 + wave * (QS * 32);  // first query row of this wave

    // ---- Q^T operand (B): lane (lc, g) holds Q[row][8*(2ks+g) .. +7].
    bf16x8 qreg[QS][KS];
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      const int qi = wq0 + s * 32 + lc;
      const uint16_t* qrow = BCAST ? a.q + ((int64_t)h * a.Lq + qi) * D
                                   : a.q + ((s0 + qi) * H + h) * (int64_t)D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (qi < nq) {
          qreg[s][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + ks * 16 + g * 8));
        } else {
          qreg[s][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
      }
    }

    f32x16 oacc[DT][QS];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < QS; ++s) oacc[dt][s] = f32x16{};
    float m2[QS], lsum[QS];
#pragma unroll
    for (int s = 0; s < QS; ++s) { m2[s] = -INFINITY; lsum[s] = 0.f; }

    int kv_end = L;
    if (CAUSAL) kv_end = min(kv_end, min(q0 + BM, nq));
    const int n_kv = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    const int n_bulk = CAUSAL ? min(q0 / BN, L / BN) : L / BN;

    const uint16_t* kbase = a.k + (s0 * H + h) * (int64_t)D;
    const uint16_t* vbase = a.v + (s0 * H + h) * (int64_t)D;
    TileLoader<BN, D, NT> kl, vl;
    // Copies K/V step j into ring buffer j % NBUF (d = 128 path).  Rows past
    // the sequence end repeat its last row: finite values that the mask
    // discards, and never an address outside the tensor.
    const PadRowCopy pc;
    auto issue = [&](int j) {
      constexpr int RPW = C::RPW, RB = TileGeom<D>::ROW_BYTES;
      const int base_row = min(j * BN + wave * RPW, L - 1);
      const int last = L - 1 - base_row;
      const uint16_t* kb = kbase + (int64_t)base_row * ld;
      const uint16_t* vb = vbase + (int64_t)base_row * ld;
      const uint32_t kd = lds_addr(smem[j % NBUF][0]) + wave * RPW * RB;
      const uint32_t vd = lds_addr(smem[j % NBUF][1]) + wave * RPW * RB;
#pragma unroll
      for (int k = 0; k < C::CPT; ++k) {
        const int R = PadRowCopy::start(k, RPW);
        const uint32_t vo = pc.voff(R, last, (uint32_t)(ld * 2));
        dma_copy16(kb, vo, kd + R * RB);
        dma_copy16(vb, vo, vd + R * RB);
      }
    };

    __syncthreads();  // the previous tile's readers are done with LDS
    if constexpr (C::DMA) {
      wait_vmcnt<0>();  // Q rows (and the last tile's stores) are not counted below
      for (int jj = 0; jj < DEP && jj < n_kv; ++jj) issue(jj);
    } else {
      if (n_kv > 0) {
        kl.load(kbase, ld, min(BN, L), tid);
        vl.load(vbase, ld, min(BN, L), tid);
        kl.store(smem[0][0], tid);
        vl.store(smem[0][1], tid);
      }
      __syncthreads();
    }

    // One K/V step of BN keys.  MASKED is a compile-time constant: the
    // bulk steps carry no mask code at all; only the tail step and the
    // causal diagonal steps take the masked body.
    auto kv_step = [&](int j, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int buf = j % NBUF;
      const int k0 = j * BN;
      if constexpr (C::DMA) {
        // Wait for this wave's copies of step j (later steps may still be in
        // flight), then for every wave's; step j-1's buffer is then free.
        const int ahead = min(DEP, n_kv - j) - 1;
        if constexpr (DEP >= 3) {
          if (ahead >= 2) wait_vmcnt<2 * IPS>();
          else if (ahead == 1) wait_vmcnt<IPS>();
          else wait_vmcnt<0>();
        } else {
          if (ahead >= 1) wait_vmcnt<IPS>();
          else wait_vmcnt<0>();
        }
        barrier_lds();
        if (j + DEP < n_kv) issue(j + DEP);
      } else if (j + 1 < n_kv) {
        const int nxt = k0 + BN;
        kl.load(kbase + (int64_t)nxt * ld, ld, min(BN, L - nxt), tid);
        vl.load(vbase + (int64_t)nxt * ld, ld, min(BN, L - nxt), tid);
      }
      // Causal: a wave whose last query row precedes this step's first key
      // sees none of it.
      const bool active = !(CAUSAL && MASKED) || (k0 <= wq0 + QS * 32 - 1);
      if (active) {
        const char* Ks = smem[buf][0];
        const char* Vs = smem[buf][1];
        // ---- S^T = K Q^T : two 32-key subtiles x QS query subtiles.
        f32x16 sacc[2][QS];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s = 0; s < QS; ++s) sacc[kt][s] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const bf16x8 ka = lds_read16(Ks, tile_off<D>(kt * 32 + lc, ks * 2 + g));
#pragma unroll
            for (int s = 0; s < QS; ++s) sacc[kt][s] = mfma32(ka, qreg[s][ks], sacc[kt][s]);
          }
        }
        // ---- online softmax, one query per lane (both halves of a row agree).
        uint32_t pk[2][2][QS][4];  // [kt][k-half][s][bf16 pairs]
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          const int qi = wq0 + s * 32 + lc;
          float mt = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float x = sacc[kt][s][i] * c2;
              if (MASKED) {
                const int key = k0 + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
                const bool ok = key < L && (!CAUSAL || key <= qi);
                x = ok ? x : -INFINITY;
              }
              sacc[kt][s][i] = x;
              mt = fmaxf(mt, x);
            }
          mt = max_across_halves(mt);
          const bool need = mt > m2[s] + RESCALE_SLACK;
          if (__builtin_expect(__any(need), 0)) {
            const float alpha = need ? fast_exp2(m2[s] - mt) : 1.f;
            m2[s] = need ? mt : m2[s];
            lsum[s] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt][s] *= alpha;
          }
          const float mref = m2[s] == -INFINITY ? 0.f : m2[s];
          float ls = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = hh * 8 + e * 2;
                const float p0 = fast_exp2(sacc[kt][s][i] - mref);
                const float p1 = fast_exp2(sacc[kt][s][i + 1] - mref);
                ls += p0 + p1;
                pk[kt][hh][s][e] = pack_bf16x2(p0, p1);
              }
          lsum[s] += ls;
        }
        // ---- O^T += V^T P^T.  k-slots of P^T (B operand) for k-half hh of
        // key subtile kt are keys kt*32 + hh*16 + {4g..4g+3, 8+4g..8+4g+3}; the
        // transpose read of V delivers the same keys.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int r0 = kt * 32 + hh * 16 + g * 4;
            bf16x8 va[DT];
            if constexpr (C::DMA) {
              // lane's transpose-read address: row r0 + j, column 16*(G&1) + 4q
              const int jj = (l & 15) >> 2, cq = ((l >> 4) & 1) * 16 + (l & 3) * 4;
              const uint32_t a0 = lds_addr(Vs + tile_off_col4<D>(r0 + jj, cq));
              lds_operand_tr_x4(a0, a0 + 8 * TileGeom<D>::ROW_BYTES, va);
            } else {
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) va[dt] = lds_operand_tr<D>(Vs, r0, r0 + 8, dt * 32);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
              for (int s = 0; s < QS; ++s) {
                const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[kt][hh][s][0], pk[kt][hh][s][1],
                                                                    pk[kt][hh][s][2], pk[kt][hh][s][3]});
                oacc[dt][s] = mfma32(va[dt], pb, oacc[dt][s]);
              }
            }
          }
      }
      if constexpr (!C::DMA) {
        if (j + 1 < n_kv) {
          kl.store(smem[buf ^ 1][0], tid);
          vl.store(smem[buf ^ 1][1], tid);
        }
        __syncthreads();
      }
    };
    const int n_plain = min(n_bulk, n_kv);
    for (int j = 0; j < n_plain; ++j) kv_step(j, std::false_type{});
    for (int j = n_plain; j < n_kv; ++j) kv_step(j, std::true_type{});

    // ---- epilogue: O = acc / l (bf16), lse = (m + log2 l) * ln 2.
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      const int qi = wq0 + s * 32 + lc;
      const float lt = sum_across_halves(lsum[s]);
      const float inv = lt > 0.f ? fast_rcp(lt) : 0.f;
      if (qi < nq) {
        uint16_t* orow = BCAST ? a.out + (((int64_t)tile.b * H + h) * a.Lq + qi) * D
                               : a.out + ((s0 + qi) * H + h) * (int64_t)D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = dt * 32 + i4 * 8 + g * 4;
            u32x2 w;
            w[0] = pack_bf16x2(oacc[dt][s][i4 * 4 + 0] * inv, oacc[dt][s][i4 * 4 + 1] * inv);
            w[1] = pack_bf16x2(oacc[dt][s][i4 * 4 + 2] * inv, oacc[dt][s][i4 * 4 + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d0) = w;
          }
        if (g == 0) {
          const float lse = lt > 0.f ? (m2[s] + fast_log2(lt)) * LN2 : -INFINITY;
          if (BCAST)
            a.lse[((int64_t)tile.b * H + h) * a.Lq + qi] = lse;
          else
            a.lse[(s0 + qi) * H + h] = lse;
        }
      }
    }
  }
}

template <int D, int NW, int QW, bool CAUSAL, bool BCAST>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  JFA_TIMED_LAUNCH(K_FWD, stream, (fwd_kernel<D, NW, QW, CAUSAL, BCAST>), dim3(a.P), dim3(NW * WAVE), 0,
                   stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  // 32 query rows per wave; broadcast tiles of 256 rows use 8 waves (two
  // per SIMD, so one wave's matrix ops overlap the other's softmax).
  if (a.broadcast_q) {
    return a.causal ? launch_fwd_t<D, FWD_BM_BCAST / 32, 32, true, true>(a, stream)
                    : launch_fwd_t<D, FWD_BM_BCAST / 32, 32, false, true>(a, stream);
  }
  return a.causal ? launch_fwd_t<D, FWD_BM_SELF / 32, 32, true, false>(a, stream)
                  : launch_fwd_t<D, FWD_BM_SELF / 32, 32, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_fwd_d<64>(a, stream);
  return launch_fwd_d<128>(a, stream);
}

}  // namespace jfa
