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
// d = 128: tiles past each workgroup's first two come from a global hand-out
// counter (runtime balance) rather than the static zigzag order.
constexpr bool DYN_FWD = true;

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
  // rows per copy), DEP = 2 steps ahead of the one being computed, in a ring
  // of 4 buffers.  Each wave copies RPW rows of K and of V per step, IPS
  // copies; the vector-memory counter can hold at most 63 outstanding
  // operations.
  // d = 64: rows are staged through registers one step ahead.
  static constexpr bool DMA = D == 128;
  static constexpr int RPW = BN / NW;
  static constexpr int CPT = PadRowCopy::copies(RPW);
  static constexpr int IPS = 2 * CPT;
  static constexpr int DEP = DMA ? 2 : 1;
  static constexpr int NBUF = DMA ? 4 : 2;
  static_assert((NBUF & (NBUF - 1)) == 0, "ring index by mask");
  static constexpr int BUF_BYTES = TILE_BYTES + PadRowCopy::GAP;
  static_assert(!DMA || (TileGeom<D>::ROW_BYTES == PadRowCopy::ROW_BYTES && RPW >= 3), "copy geometry");
  // V tiles of the direct-copy form are only read with the transposing read
  // (32 lanes take 64 bytes from each of 4 consecutive rows): 320-byte rows
  // put those rows 64 bytes apart modulo the 256 bytes of the LDS banks, so
  // the 32 lanes touch every bank once.  Rows of 304 bytes (K) overlap by
  // 16 bytes between neighbours there.
  using VCopy = PadRowCopyN<20>;
  static constexpr int ROW_BYTES_V = DMA ? VCopy::ROW_BYTES : TileGeom<D>::ROW_BYTES;
  static constexpr int BUF_BYTES_V = BN * ROW_BYTES_V + VCopy::GAP;
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
  const int64_t ld = (int64_t)a.Hkv * D;  // K / V row stride (elements)
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
    // A window cuts steps anywhere: every step takes the masked body then.
    const int n_bulk = a.window > 0 ? 0 : CAUSAL ? min(q0 / BN, L / BN) : L / BN;
    // First step with a key inside some row's window (the tile's first row
    // sees keys from q0 - window + 1 on); the steps before it are skipped.
    const int j0 = CAUSAL && a.window > 0 ? min(max(0, q0 - a.window + 1) / BN, n_kv) : 0;

    const uint16_t* kbase = a.k + (s0 * a.Hkv + tile.hk) * (int64_t)D;
    const uint16_t* vbase = a.v + (s0 * a.Hkv + tile.hk) * (int64_t)D;
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
      for (int jj = j0; jj < j0 + DEP && jj < n_kv; ++jj) issue(jj);
    } else {
      if (n_kv > j0) {
        const int r0 = j0 * BN;
        kl.load(kbase + (int64_t)r0 * ld, ld, min(BN, L - r0), tid);
        vl.load(vbase + (int64_t)r0 * ld, ld, min(BN, L - r0), tid);
        kl.store(smem[j0 % NBUF][0], tid);
        vl.store(smem[j0 % NBUF][1], tid);
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
                const bool ok = key < L && (!CAUSAL || (key <= qi && (a.window <= 0 || key > qi - a.window)));
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
    for (int j = j0; j < n_plain; ++j) kv_step(j, std::false_type{});
    for (int j = max(n_plain, j0); j < n_kv; ++j) kv_step(j, std::true_type{});

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

// d = 128 form of the kernel.  K/V steps form one stream over this
// workgroup's tiles: copies run DEP steps ahead across tile boundaries, and
// are issued from inside S^T products.  Non-causal tiles are
// software-pipelined: each iteration runs the S^T products of step j + 1
// with the softmax of step j between them, then the PV products of step j.
// The next tile's Q rows are loaded before the current tile's O / lse are
// stored, and the stores are bounded buffer stores of a fixed count per
// wave, so the wait at the next tile start covers exactly the copies and Q
// loads and lets the stores drain.
template <int D, int NW, int QW, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(NW * WAVE, 1) void fwd_kernel_dma(FwdArgs a, const TileRec* __restrict__ tiles) {
  using C = Fwd<D, NW, QW, CAUSAL, BCAST>;
  static_assert(C::DMA, "direct-copy form");
  constexpr int BN = C::BN, QS = C::QS, BM = C::BM, KS = C::KS, DT = C::DT;
  constexpr int NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS, RPW = C::RPW, RB = TileGeom<D>::ROW_BYTES;
  constexpr int RBV = C::ROW_BYTES_V;
  // Stores per wave at a tile end: O (DT * 2 pieces of 16 bytes) and lse, per subtile.
  constexpr int NST = QS * (2 * DT + 1);
  static_assert(DEP * IPS + NST <= 63, "vector-memory counter");
  __shared__ __attribute__((aligned(16))) char smem_k[NBUF][C::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) char smem_v[NBUF][C::BUF_BYTES_V];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_tiles;
  const int H = a.H, Lq = a.Lq;
  const int64_t ld = (int64_t)a.Hkv * D;  // K / V row stride (elements)
  // A negative scale is folded into Q: the sign bits of the Q operand are
  // flipped at its load, so that every score below is (-q) k with the
  // scale's magnitude, and the softmax keeps one form (the row maximum of
  // the raw scores).  The products are exact; the matrix unit's sums of
  // them may round differently from those of q k, within the same error.
  const float c2 = __builtin_fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  // This lane's source byte offset within a K copy (304-byte rows in LDS)
  // and a V copy (320-byte rows), relative to the copy's first row.
  const uint32_t rstride = (uint32_t)(ld * 2);
  const uint32_t voff_k = PadRowCopy::lane_row(l) * rstride + PadRowCopy::lane_byte(l);
  const uint32_t voff_v = C::VCopy::lane_row(l) * rstride + C::VCopy::lane_byte(l);

  const int64_t t0 = zigzag_tile(0, slot, a.P);
  if (t0 >= T) return;

  // Per-tile values, with the addresses of the tile's row 0 of K and V.
  struct Tp {
    int64_t s0;
    int L, h, b, q0, n_kv, n_bulk;
    int j0;  // first step: the steps before it lie wholly outside every row's window
    const uint16_t* kb;
    const uint16_t* vb;
  };
  auto tparams = [&](const TileRec& r) {
    Tp p;
    p.s0 = r.s0;
    p.L = r.L;
    p.h = r.h;
    p.b = r.b;
    p.kb = a.k + (r.s0 * a.Hkv + r.hk) * (int64_t)D;
    p.vb = a.v + (r.s0 * a.Hkv + r.hk) * (int64_t)D;
    p.q0 = r.blk * BM;
    const int nq = BCAST ? Lq : r.L;
    int kv_end = r.L;
    if (CAUSAL) kv_end = min(kv_end, min(p.q0 + BM, nq));
    p.n_kv = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    // A window cuts steps anywhere: every step takes the masked body then.
    p.n_bulk = a.window > 0 ? 0 : min(CAUSAL ? min(p.q0 / BN, r.L / BN) : r.L / BN, p.n_kv);
    p.j0 = CAUSAL && a.window > 0 ? min(max(0, p.q0 - a.window + 1) / BN, p.n_kv) : 0;
    return p;
  };

  // ---- the step stream.  g_iss / g_cmp: steps issued / computed so far
  // over the whole stream; iss_cur / iss_nxt: steps of the current / next
  // tile issued.
  int g_iss = 0, g_cmp = 0, iss_cur = 0, iss_nxt = 0;
  // The prepared step: buffer resources over this wave's K and V source
  // rows of it (the rows that exist, at most RPW + 1: a copy's overhang
  // reaches one row past the run; rows past the sequence end read as
  // zeros) and its ring buffer.  Past the stream's last step the copies
  // still go out, over empty ranges (they read nothing and at most write
  // zeros into the ring buffer the next step would take, which no wave
  // reads again), so that no branch splits the code they sit in.
  __amdgpu_buffer_rsrc_t j_rk = make_rsrc(a.k, 0), j_rv = make_rsrc(a.v, 0);
  uint32_t j_kd = 0, j_vd = 0;
  auto prep_next = [&](const Tp& cp, const Tp& np, bool has_nxt) {
    const int nn = has_nxt ? np.n_kv - np.j0 : 0;
    const bool cur = iss_cur < cp.n_kv - cp.j0;
    const int buf = (int)((uint32_t)g_iss % NBUF);
    j_kd = lds_addr(smem_k[buf]) + wave * RPW * RB;
    j_vd = lds_addr(smem_v[buf]) + wave * RPW * RBV;
    if (!(cur || iss_nxt < nn)) {
      j_rk = make_rsrc(a.k, 0);
      j_rv = make_rsrc(a.v, 0);
      return;
    }
    const int L_ = cur ? cp.L : np.L;
    const int j = cur ? cp.j0 + iss_cur : np.j0 + iss_nxt;
    const int base_row = j * BN + wave * RPW;
    const int rows = max(0, min(L_ - base_row, RPW + 1));
    // byte offset of the row within the sequence (a 32 x 32-bit product)
    const uint64_t roff = (uint64_t)(uint32_t)base_row * rstride;
    j_rk = make_rsrc(reinterpret_cast<const char*>(cur ? cp.kb : np.kb) + roff, rows * (int)rstride);
    j_rv = make_rsrc(reinterpret_cast<const char*>(cur ? cp.vb : np.vb) + roff, rows * (int)rstride);
    if (cur) ++iss_cur;
    else ++iss_nxt;
    ++g_iss;
  };
  // Copies [k0, k1) of the prepared step (K for k < CPT, V after); the
  // copy's first row goes into the scalar offset.
  auto issue_copies = [&](int k0, int k1) {
#pragma unroll
    for (int k = k0; k < k1; ++k) {
      const int R = PadRowCopy::start(k % C::CPT, RPW);
      if (k < C::CPT) dma_copy16_buf(j_rk, voff_k, R * rstride, j_kd + R * RB);
      else dma_copy16_buf(j_rv, voff_v, R * rstride, j_vd + R * RBV);
    }
  };

  // ---- Q^T operand (B): lane (lc, g) holds Q[row][8*(2ks+g) .. +7].
  // Rows past the last query read row 0 of the block (finite, never stored).
  bf16x8 qreg[QS][KS];
  auto load_q = [&](const Tp& p) {
    const int nq = BCAST ? Lq : p.L;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      int qi = p.q0 + wave * (QS * 32) + s * 32 + lc;
      qi = qi < nq ? qi : p.q0 < nq ? p.q0 : 0;
      const uint16_t* qrow = BCAST ? a.q + ((int64_t)p.h * Lq + qi) * D : a.q + ((p.s0 + qi) * H + p.h) * (int64_t)D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + g * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] ^= qsign;
        qreg[s][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };

  // ---- O = acc / l (bf16) and lse = (m + log2 l) * ln 2 of a tile: NST
  // buffer stores per wave, bounded to the tile's rows (nrows = 0 stores
  // nothing).
  f32x16 oacc[DT][QS];
  float m2[QS], lsum[QS];
  auto store_out = [&](const Tp& p, int nrows) {
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      const int r0 = p.q0 + wave * (QS * 32) + s * 32;  // first row of the subtile
      const int nv = max(0, min(nrows - r0, 32));        // its valid rows
      const int64_t orow0 = BCAST ? ((int64_t)p.b * H + p.h) * Lq + r0 : (p.s0 + r0) * H + p.h;
      const int ostride = BCAST ? D : H * D;             // elements between rows
      const int lstride = BCAST ? 1 : H;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + orow0 * D, nv * ostride * 2);
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + orow0, nv * lstride * 4);
      const float lt = sum_across_halves(lsum[s]);
      const float inv = lt > 0.f ? fast_rcp(lt) : 0.f;
      // Register group i4 of lane (row, g) holds columns dt*32 + 8 i4 + 4g
      // + 0..3.  Lanes l and l + 32 trade one group of each pair (2p, 2p+1)
      // so that each then holds 8 consecutive columns, 16 + 8g .. of 16p:
      // one 16-byte store per lane and pair.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int p2 = 0; p2 < 2; ++p2) {
          uint32_t w[2][2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int i4 = 2 * p2 + k;
            w[k][0] = pack_bf16x2(oacc[dt][s][i4 * 4 + 0] * inv, oacc[dt][s][i4 * 4 + 1] * inv);
            w[k][1] = pack_bf16x2(oacc[dt][s][i4 * 4 + 2] * inv, oacc[dt][s][i4 * 4 + 3] * inv);
          }
          // g = 0 sends group 2p+1 and receives the partner's group 2p;
          // g = 1 sends group 2p and receives the partner's group 2p+1.
          const uint32_t s0w = g ? w[0][0] : w[1][0], s1w = g ? w[0][1] : w[1][1];
          const uint32_t r0w = (uint32_t)__shfl_xor((int)s0w, 32), r1w = (uint32_t)__shfl_xor((int)s1w, 32);
          u32x4 v;
          if (g == 0) v = u32x4{w[0][0], w[0][1], r0w, r1w};
          else v = u32x4{r0w, r1w, w[1][0], w[1][1]};
          const int d0 = dt * 32 + p2 * 16 + g * 8;
          __builtin_amdgcn_raw_buffer_store_b128(v, ro, (lc * ostride + d0) * 2, 0, 0);
        }
      const float lse = lt > 0.f ? (m2[s] + fast_log2(lt)) * LN2 : -INFINITY;
      // lanes of the second half hold the same row: their store is dropped
      const uint32_t loff = g == 0 ? (uint32_t)(lc * lstride * 4) : 0xfffffff0u;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), rl, loff, 0, 0);
    }
  };

  Tp cp = tparams(tiles[t0]);
  load_q(cp);
  {
    // Stores that write nothing: the first tile start sees the same
    // operations after its Q loads as every later one.
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      lsum[s] = 0.f;
      m2[s] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][s] = f32x16{};
    }
    store_out(cp, 0);
  }

  // Tile hand-out: each workgroup takes its first two tiles by the zigzag
  // order (passes 0 and 1) and every later one from a global counter over
  // the rest of the longest-first list, one tile ahead: the index for pass
  // p + 2 is fetched at the start of pass p (one lane of wave 0, a vector
  // atomic) and shared through LDS at the start of pass p + 1.  Its latency
  // hides behind a whole tile; the compiler's wait for it falls at the tile
  // start, where everything but the previous tile's stores has landed.
  __shared__ int s_next;
  unsigned int fetched = 0;
  for (int64_t pass = 0;; ++pass) {
    const int64_t s0 = cp.s0;
    const int L = cp.L, h = cp.h, q0 = cp.q0, n_kv = cp.n_kv;
    const int nq = BCAST ? Lq : L;
    const int wq0 = q0 + wave * (QS * 32);  // first query row of this wave
    (void)s0;
    (void)h;

#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int s = 0; s < QS; ++s) oacc[dt][s] = f32x16{};
#pragma unroll
    for (int s = 0; s < QS; ++s) { m2[s] = -INFINITY; lsum[s] = 0.f; }

    // Tile start: normally its first min(DEP, n_kv) steps were issued during
    // the previous tile, before its Q loads for this tile, and only the
    // previous tile's NST stores may be outstanding after those.
    {
      const int need = min(DEP, n_kv - cp.j0);
      if (iss_cur < need) {
        while (iss_cur < need) {
          prep_next(cp, cp, false);  // this tile's steps only
          issue_copies(0, 2 * C::CPT);
        }
        wait_vmcnt<0>();
      } else {
        wait_vmcnt<NST>();
      }
    }
    if (DYN_FWD && pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
    if (DYN_FWD) barrier_lds();
    const int64_t tn = !DYN_FWD ? zigzag_tile(pass + 1, slot, a.P)
                       : pass == 0 ? zigzag_tile(1, slot, a.P)
                                   : 2 * (int64_t)a.P + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
    const bool has_nxt = tn < T;
    if (DYN_FWD && has_nxt && wave == 0 && l == 0) fetched = atomicAdd(a.tile_ctr, 1u);
    const Tp np = has_nxt ? tparams(tiles[tn]) : cp;
#pragma unroll
    for (int s = 0; s < QS; ++s)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = __builtin_bit_cast(u32x4, qreg[s][ks]);
        asm volatile("" : "+v"(x));
        qreg[s][ks] = __builtin_bit_cast(bf16x8, x);
      }
    const int g_first = g_cmp;  // stream index of this tile's step 0

    // One K/V step of BN keys.  MASKED is a compile-time constant: the
    // bulk steps carry no mask code at all; only the tail step and the
    // causal diagonal steps take the masked body.
    // S^T = K Q^T of stream step gi into sacc; the K operand of k-step
    // ks + 1 is read before the products of k-step ks, and hook(ks) runs
    // after them; the prepared step's copies go out between the k-steps
    // when COPY is true.
    auto s_phase = [&](int gi, f32x16 (&sacc)[2][QS], auto&& hook, auto copy_tag) {
      constexpr bool COPY = decltype(copy_tag)::value;
      const char* Ks = smem_k[(uint32_t)gi % NBUF];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < QS; ++s) sacc[kt][s] = f32x16{};
      bf16x8 ka[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) ka[kt] = lds_read16(Ks, tile_off<D>(kt * 32 + lc, g));
      static_for<0, KS>([&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        bf16x8 kn[2];
        if constexpr (ks + 1 < KS) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) kn[kt] = lds_read16(Ks, tile_off<D>(kt * 32 + lc, (ks + 1) * 2 + g));
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s = 0; s < QS; ++s) sacc[kt][s] = mfma32(ka[kt], qreg[s][ks], sacc[kt][s]);
        constexpr int PER = (2 * C::CPT + KS - 1) / KS;
        if constexpr (COPY) issue_copies(ks * PER, min((ks + 1) * PER, 2 * C::CPT));
        hook(ks_tag);
        if constexpr (ks + 1 < KS) {
          ka[0] = kn[0];
          ka[1] = kn[1];
        }
      });
    };
    // O^T += V^T P^T of stream step gi, in 8 pieces (key group (kt, hh) x
    // head-dim tiles 2 h, 2 h + 1); the transposed V reads of each piece
    // are issued before the products of the piece before.
    const int jj = (l & 15) >> 2, cq = ((l >> 4) & 1) * 16 + (l & 3) * 4;
    auto pv_phase = [&](int gi, const uint32_t (&pk)[2][2][QS][4]) {
      const char* Vs = smem_v[(uint32_t)gi % NBUF];
      uint32_t va[4];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int r0 = (grp >> 1) * 32 + (grp & 1) * 16 + g * 4;
        va[grp] = lds_addr(Vs + tile_off_col4<D, RBV>(r0 + jj, cq));
      }
      i16x4 xv[2][4];
      static_assert(DT == 4, "two pieces of two head-dim tiles per key group");
      tr4_issue<0>(va[0], va[0] + 8 * RBV, xv[0]);
      static_for<0, 8>([&](auto pc_tag) {
        constexpr int pc = decltype(pc_tag)::value;
        constexpr int grp = pc >> 1, hf = pc & 1;
        constexpr int kt = grp >> 1, hh = grp & 1;
        if constexpr (pc + 1 < 8) {
          constexpr int ng = (pc + 1) >> 1, nh = (pc + 1) & 1;
          tr4_issue<nh * 128>(va[ng], va[ng] + 8 * RBV, xv[(pc + 1) & 1]);
          tr4_wait<4>(xv[pc & 1]);
        } else {
          tr4_wait<0>(xv[pc & 1]);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int s = 0; s < QS; ++s) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[kt][hh][s][0], pk[kt][hh][s][1],
                                                                pk[kt][hh][s][2], pk[kt][hh][s][3]});
            oacc[2 * hf + k][s] = mfma32(tr4_operand(xv[pc & 1], k), pb, oacc[2 * hf + k][s]);
          }
      });
    };
    auto kv_step = [&](int j, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int k0 = j * BN;
      // Wait for this wave's copies of step j (steps issued after it may
      // still be in flight), then for every wave's; the ring buffer of the
      // step before is then free.  Steps issued before the tile start were
      // waited for there.
      if (g_cmp != g_first) {
        const int after = g_iss - 1 - g_cmp;
        if constexpr (DEP >= 3) {
          if (after >= 2) wait_vmcnt<2 * IPS>();
          else if (after == 1) wait_vmcnt<IPS>();
          else wait_vmcnt<0>();
        } else {
          if (after >= 1) wait_vmcnt<IPS>();
          else wait_vmcnt<0>();
        }
      }
      barrier_lds();
      prep_next(cp, np, has_nxt);
      // Causal: a wave whose last query row precedes this step's first key
      // sees none of it.
      const bool active = !(CAUSAL && MASKED) || (k0 <= wq0 + QS * 32 - 1);
      if (!active) {
        issue_copies(0, 2 * C::CPT);
      } else {
        // ---- S^T = K Q^T : two 32-key subtiles x QS query subtiles; the
        // next step's copies are issued between the k-steps.
        f32x16 sacc[2][QS];
        s_phase(g_cmp, sacc, [](auto) {}, std::true_type{});
        // ---- online softmax, one query per lane (both halves of a row agree).
        uint32_t pk[2][2][QS][4];  // [kt][k-half][s][bf16 pairs]
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          const int qi = wq0 + s * 32 + lc;
          // Row maximum in exp2 units.  Unmasked steps reduce the raw
          // scores and fold the scale into the exponent's fma below; masked
          // steps scale first and set masked scores to -inf.
          float mt;
          if constexpr (MASKED) {
            mt = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                float x = sacc[kt][s][i] * c2;
                const int key = k0 + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
                const bool ok = key < L && (!CAUSAL || (key <= qi && (a.window <= 0 || key > qi - a.window)));
                x = ok ? x : -INFINITY;
                sacc[kt][s][i] = x;
                mt = fmaxf(mt, x);
              }
            mt = max_across_halves(mt);
          } else {
            float r = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int i = 0; i < 16; ++i) r = fmaxf(r, sacc[kt][s][i]);
            mt = max_across_halves(r) * c2;
          }
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
                float p0, p1;
                if constexpr (MASKED) {
                  p0 = fast_exp2(sacc[kt][s][i] - mref);
                  p1 = fast_exp2(sacc[kt][s][i + 1] - mref);
                } else {
                  p0 = fast_exp2(__builtin_fmaf(sacc[kt][s][i], c2, -mref));
                  p1 = fast_exp2(__builtin_fmaf(sacc[kt][s][i + 1], c2, -mref));
                }
                ls += p0 + p1;
                pk[kt][hh][s][e] = pack_bf16x2(p0, p1);
              }
          lsum[s] += ls;
        }
        // ---- O^T += V^T P^T.  k-slots of P^T (B operand) for k-half hh of
        // key subtile kt are keys kt*32 + hh*16 + {4g..4g+3, 8+4g..8+4g+3}; the
        // transpose read of V delivers the same keys.
        pv_phase(g_cmp, pk);
      }
      ++g_cmp;
    };
    if constexpr (CAUSAL) {
      const int n_plain = cp.n_bulk;
      for (int j = cp.j0; j < n_plain; ++j) kv_step(j, std::false_type{});
      for (int j = max(n_plain, cp.j0); j < n_kv; ++j) kv_step(j, std::true_type{});
    } else if (n_kv > 0) {
      // Software-pipelined steps: the S products of step j + 1 run beside
      // the softmax of step j (split into pieces between their k-steps), then
      // the PV products of step j.  Only the last step of a tile can be
      // masked (keys past the sequence end); it runs after the loop.
      // Step j's V stays in use until its PV products, so the copies issued
      // after the barrier of iteration j go to the buffer of step j - 1 (the
      // stream's next step is j + 3); the tile's last step issues one more
      // after a barrier of its own, and the stream stays DEP steps ahead.
      // This wave's copies of stream step gi landed, with iss steps' copies out.
      auto wait_step = [&](int gi, int iss) {
        const int after = iss - 1 - gi;
        if constexpr (DEP >= 3) {
          if (after >= 2) wait_vmcnt<2 * IPS>();
          else if (after == 1) wait_vmcnt<IPS>();
          else wait_vmcnt<0>();
        } else {
          if (after >= 1) wait_vmcnt<IPS>();
          else wait_vmcnt<0>();
        }
      };
      // Softmax of one step in pieces: sm_max (row maximum; the masked form
      // scales and masks the scores in place), sm_rescale (lazy rescale of
      // the running state; returns the reference exponent), sm_exp (P of key
      // subtile kt, k-half hh, as packed bf16) and sm_sum.
      float rmax[QS], mref[QS], lsp[QS];
      auto sm_max = [&](auto masked_tag, int k0, f32x16 (&sacc)[2][QS], int kt) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          float r;
          if constexpr (MASKED) {
            r = kt == 0 ? -INFINITY : rmax[s];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float x = sacc[kt][s][i] * c2;
              const int key = k0 + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
              x = key < L ? x : -INFINITY;
              sacc[kt][s][i] = x;
              r = fmaxf(r, x);
            }
          } else {
            r = kt == 0 ? -INFINITY : rmax[s];
#pragma unroll
            for (int i = 0; i < 16; ++i) r = fmaxf(r, sacc[kt][s][i]);
          }
          rmax[s] = r;
        }
      };
      auto sm_rescale = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          float mt;
          if constexpr (MASKED) mt = max_across_halves(rmax[s]);
          else mt = max_across_halves(rmax[s]) * c2;
          const bool need = mt > m2[s] + RESCALE_SLACK;
          if (__builtin_expect(__any(need), 0)) {
            const float alpha = need ? fast_exp2(m2[s] - mt) : 1.f;
            m2[s] = need ? mt : m2[s];
            lsum[s] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt][s] *= alpha;
          }
          mref[s] = m2[s] == -INFINITY ? 0.f : m2[s];
          lsp[s] = 0.f;
        }
      };
      auto sm_exp = [&](auto masked_tag, const f32x16 (&sacc)[2][QS], int kt, int hh, uint32_t (&pk)[2][2][QS][4]) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int s = 0; s < QS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = hh * 8 + e * 2;
            float p0, p1;
            if constexpr (MASKED) {
              p0 = fast_exp2(sacc[kt][s][i] - mref[s]);
              p1 = fast_exp2(sacc[kt][s][i + 1] - mref[s]);
            } else {
              p0 = fast_exp2(__builtin_fmaf(sacc[kt][s][i], c2, -mref[s]));
              p1 = fast_exp2(__builtin_fmaf(sacc[kt][s][i + 1], c2, -mref[s]));
            }
            lsp[s] += p0 + p1;
            pk[kt][hh][s][e] = pack_bf16x2(p0, p1);
          }
      };
      auto sm_sum = [&]() {
#pragma unroll
        for (int s = 0; s < QS; ++s) lsum[s] += lsp[s];
      };
      // One pipelined iteration: step j's softmax (scores in sa) and PV,
      // beside step j + 1's S products (into sb).
      uint32_t pk[2][2][QS][4];
      auto iter = [&](int j, f32x16 (&sa)[2][QS], f32x16 (&sb)[2][QS]) {
        const int gj = g_first + j;
        // The next step's copy preparation (addresses only) runs before the
        // wait and the barrier, beside the other waves' arrival; the wait
        // counts the steps whose copies are out, which excludes it.
        const int iss0 = g_iss;
        prep_next(cp, np, has_nxt);
        wait_step(gj + 1, iss0);
        barrier_lds();
        using F = std::false_type;
        s_phase(gj + 1, sb, [&](auto ks_tag) {
          constexpr int ks = decltype(ks_tag)::value;
          if constexpr (ks == 0) sm_max(F{}, 0, sa, 0);
          if constexpr (ks == 1) {
            sm_max(F{}, 0, sa, 1);
            sm_rescale(F{});
          }
          if constexpr (ks >= 2 && ks < 6) sm_exp(F{}, sa, (ks - 2) >> 1, (ks - 2) & 1, pk);
          if constexpr (ks == 6) sm_sum();
        }, std::true_type{});
        pv_phase(gj, pk);
        ++g_cmp;
      };
      auto last = [&](auto masked_tag, int j, f32x16 (&sa)[2][QS]) {
        barrier_lds();  // every wave has left the buffer of step j - 1
        prep_next(cp, np, has_nxt);
        issue_copies(0, 2 * C::CPT);
        sm_max(masked_tag, j * BN, sa, 0);
        sm_max(masked_tag, j * BN, sa, 1);
        sm_rescale(masked_tag);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) sm_exp(masked_tag, sa, kt, hh, pk);
        sm_sum();
        pv_phase(g_first + j, pk);
        ++g_cmp;
      };
      f32x16 sa[2][QS], sb[2][QS];
      // prologue: step 0's S products, with no copies (each tile issues
      // one copy step per iteration and one in its last step)
      barrier_lds();
      s_phase(g_first, sa, [](auto) {}, std::false_type{});
      int j = 0;
      for (; j + 2 < n_kv; j += 2) {
        iter(j, sa, sb);
        iter(j + 1, sb, sa);
      }
      if (j + 1 < n_kv) {
        iter(j, sa, sb);
        ++j;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s = 0; s < QS; ++s) sa[kt][s] = sb[kt][s];
      }
      if (cp.n_bulk < n_kv) last(std::true_type{}, j, sa);
      else last(std::false_type{}, j, sa);
    }

    // A tile without steps has no barrier after the waves read s_next,
    // which wave 0 rewrites at the next tile start.
    if (DYN_FWD && g_cmp == g_first) barrier_lds();
    // Tile end: the next tile's Q rows, then this tile's O and lse.
    if (has_nxt) load_q(np);
    store_out(cp, nq);
    if (!has_nxt) {
      wait_vmcnt<0>();  // no copy into LDS outlives the workgroup
      break;
    }
    cp = np;
    iss_cur = iss_nxt;
    iss_nxt = 0;
  }
}

template <int D, int NW, int QW, bool CAUSAL, bool BCAST>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  if constexpr (D == 128) {
    JFA_TIMED_LAUNCH(K_FWD, stream, (fwd_kernel_dma<D, NW, QW, CAUSAL, BCAST>), dim3(a.P), dim3(NW * WAVE), 0,
                     stream, a, a.tiles);
  } else {
    JFA_TIMED_LAUNCH(K_FWD, stream, (fwd_kernel<D, NW, QW, CAUSAL, BCAST>), dim3(a.P), dim3(NW * WAVE), 0,
                     stream, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t stream) {
  // 32 query rows per wave; tiles of 256 rows use 8 waves (two per SIMD,
  // so one wave's matrix ops overlap the other's softmax).
  if (a.broadcast_q) {
    return a.causal ? launch_fwd_t<D, FWD_BM / 32, 32, true, true>(a, stream)
                    : launch_fwd_t<D, FWD_BM / 32, 32, false, true>(a, stream);
  }
  return a.causal ? launch_fwd_t<D, FWD_BM / 32, 32, true, false>(a, stream)
                  : launch_fwd_t<D, FWD_BM / 32, 32, false, false>(a, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_fwd_d<64>(a, stream);
  return launch_fwd_d<128>(a, stream);
}

}  // namespace jfa
