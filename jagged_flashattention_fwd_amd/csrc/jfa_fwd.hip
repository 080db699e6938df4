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
// SMs").  Each workgroup is 4 waves; wave w owns QW consecutive query rows.
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
#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

constexpr float RESCALE_SLACK = 8.0f;  // log2 units

template <int D, int QW, bool CAUSAL, bool BCAST>
struct Fwd {
  static constexpr int NW = 4;
  static constexpr int NT = NW * WAVE;
  static constexpr int BN = FWD_KV_STEP;
  static constexpr int QS = QW / 32;   // 32-row query subtiles per wave
  static constexpr int BM = NW * QW;
  static constexpr int KS = D / 16;    // MFMA k-steps over the head dim
  static constexpr int DT = D / 32;    // 32-wide head-dim tiles of O^T
  static constexpr int TILE_BYTES = tile_bytes<BN, D>();
};

template <int D, int QW, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdArgs a) {
  using C = Fwd<D, QW, CAUSAL, BCAST>;
  constexpr int BN = C::BN, QS = C::QS, BM = C::BM, KS = C::KS, DT = C::DT, NT = C::NT;
  __shared__ __attribute__((aligned(16))) char smem[2][2][C::TILE_BYTES];  // [buffer][K, V]

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

    __syncthreads();  // the previous tile's readers are done with LDS
    if (n_kv > 0) {
      kl.load(kbase, ld, min(BN, L), tid);
      vl.load(vbase, ld, min(BN, L), tid);
      kl.store(smem[0][0], tid);
      vl.store(smem[0][1], tid);
    }
    __syncthreads();

    for (int j = 0; j < n_kv; ++j) {
      const int buf = j & 1;
      const int k0 = j * BN;
      if (j + 1 < n_kv) {
        const int nxt = k0 + BN;
        kl.load(kbase + (int64_t)nxt * ld, ld, min(BN, L - nxt), tid);
        vl.load(vbase + (int64_t)nxt * ld, ld, min(BN, L - nxt), tid);
      }
      // Causal: a wave whose last query row precedes this step's first key
      // sees none of it.
      const bool active = !CAUSAL || (k0 <= wq0 + QS * 32 - 1);
      if (active) {
        const char* Ks = smem[buf][0];
        const char* Vs = smem[buf][1];
        const bool masked = j >= n_bulk;
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
              if (masked) {
                const int key = k0 + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
                const bool ok = key < L && (!CAUSAL || key <= qi);
                x = ok ? x : -INFINITY;
              }
              sacc[kt][s][i] = x;
              mt = fmaxf(mt, x);
            }
          mt = max_across_halves(mt);
          const bool need = mt > m2[s] + RESCALE_SLACK;
          if (__any(need)) {
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
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const bf16x8 va = lds_operand_tr<D>(Vs, r0, r0 + 8, dt * 32);
#pragma unroll
              for (int s = 0; s < QS; ++s) {
                const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[kt][hh][s][0], pk[kt][hh][s][1],
                                                                    pk[kt][hh][s][2], pk[kt][hh][s][3]});
                oacc[dt][s] = mfma32(va, pb, oacc[dt][s]);
              }
            }
          }
      }
      if (j + 1 < n_kv) {
        kl.store(smem[buf ^ 1][0], tid);
        vl.store(smem[buf ^ 1][1], tid);
      }
      __syncthreads();
    }

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

template <int D, int QW, bool CAUSAL, bool BCAST>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  JFA_TIMED_LAUNCH(K_FWD, stream, (fwd_kernel<D, QW, CAUSAL, BCAST>), dim3(a.P), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  if (a.broadcast_q) {
    return a.causal ? launch_fwd_t<D, FWD_BM_BCAST / 4, true, true>(a, stream)
                    : launch_fwd_t<D, FWD_BM_BCAST / 4, false, true>(a, stream);
  }
  return a.causal ? launch_fwd_t<D, FWD_BM_SELF / 4, true, false>(a, stream)
                  : launch_fwd_t<D, FWD_BM_SELF / 4, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_fwd_d<64>(a, stream);
  return launch_fwd_d<128>(a, stream);
}

}  // namespace jfa
