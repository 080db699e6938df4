// Jagged flash-attention backward for gfx950.
//
// The gradient of O = softmax(scale Q K^T) V, with P recomputed from the
// forward's lse:  dP = dO V^T,  delta_i = sum_d dO_id O_id,
// dS = P o (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// In broadcast mode dQ is summed over every sequence of the batch
// ("Optimizing Jagged Flash Attention with TLX", "1. The Challenge").
//
// Kernels, in launch order:
//   delta_kernel        streaming pre-pass: delta = rowsum(dO o O) (O as
//                       stored), lse * log2(e), and the bf16 row terms of
//                       -lse / scale and -delta, per query row.
//   delta_exact_kernel  delta again, exactly, for sequences of at most 128
//                       keys and, in causal broadcast mode, the first 128
//                       query rows of every sequence (jfa_dkdv.hip).
//   dkdv_kernel         dK and dV (jfa_dkdv.hip).
//   dq_kernel           dQ.  Self-attention: persistent, a tile is 128 query
//                       rows, looping over K/V steps recomputing S^T, dP^T,
//                       dS^T and accumulating dQ^T += K^T dS^T.  Broadcast Q:
//                       one workgroup per (head, 256-row query block, chunk of
//                       sequences) writes a private fp32 partial, summed by
//   dq_reduce           with a fixed pairwise tree (bitwise reproducible) --
//                       per-workgroup partials instead of a contended
//                       reduce-add into one buffer, which "Multi-stage dQ
//                       staging" names the main backward bottleneck.
// Loops are peeled ("Loop peeling"): the causal diagonal blocks take the
// masked path, the rest do not.
#include <type_traits>

#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

// Threshold of the two-term bf16 dS operand in dQ: rounding dS to bf16 costs
// up to 2^-9 of each value, summed over many keys; where a subtile holds a
// value above this, the rounded remainder is multiplied in as well.
constexpr float SPLIT_DS = 0.25f;

// ------------------------------------------------------------- delta ----
// Rows of d elements; D/8 threads per row, 16 bytes each.  Also writes the
// row's lse in base-2 units (lse * log2(e)), the form the dQ kernels read, and
// the row terms (row_terms) of -lse / scale and -delta that the dK/dV kernel
// folds into its score products.  Broadcast rows whose delta the exact pass
// (delta_exact_kernel, after this one) writes are not read here.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    float* __restrict__ delta, float* __restrict__ lse2,
                                                    u32x4* __restrict__ term_l, u32x4* __restrict__ term_d,
                                                    float inv_scale, int64_t rows, const int64_t* __restrict__ offsets,
                                                    int64_t total_len, int HLq, int Lq, int causal) {
  constexpr int TPR = D / 8;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // Broadcast rows (HLq > 0) whose delta the exact pass writes (sequences of
  // 1 .. BWD_BN keys; with the causal mask also the first BWD_BN query rows
  // of every sequence) skip the O / dO reads.  A row's flag is found one
  // iteration ahead, so that its offsets read overlaps the row before.
  auto exact_row = [&](int64_t row) {
    if (HLq <= 0 || row >= rows) return false;
    // (32-bit division where the row index fits: the 64-bit one costs
    // several times more)
    int b, q;
    if (rows <= 0x7fffffffll) {
      const uint32_t r32 = (uint32_t)row;
      b = (int)(r32 / (uint32_t)HLq);
      q = (int)(r32 % (uint32_t)Lq);
    } else {
      b = (int)(row / HLq);
      q = (int)(row % Lq);
    }
    int64_t s0;
    const int64_t L = seq_range(offsets, b, total_len, &s0);
    return L > 0 && (L <= BWD_BN || (causal && q < BWD_BN));
  };
  bool exact_nxt = exact_row(gtid / TPR);
  for (int64_t e = gtid; e < rows * TPR; e += stride) {
    const int64_t row = e / TPR;
    const int c = (int)(e % TPR);
    const bool exact = exact_nxt;
    u32x4 o = u32x4{0u, 0u, 0u, 0u}, g = u32x4{0u, 0u, 0u, 0u};
    if (!exact) {
      o = *reinterpret_cast<const u32x4*>(out + row * D + c * 8);
      g = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
    }
    exact_nxt = exact_row((e + stride) / TPR);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_lo(o[i]) * bf16_lo(g[i]);
      acc += bf16_hi(o[i]) * bf16_hi(g[i]);
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (c == 0) {
      lse2[row] = lse[row] * LOG2E;
      term_l[row] = row_terms(-lse[row] * inv_scale);
      if (!exact) {
        delta[row] = acc;
        term_d[row] = row_terms(-acc);
      }
    }
  }
}

// --------------------------------------------------------- dQ reduce ----
// dq[h][q][:] = scale * sum over the NC partials of (h, q-block), summed as a
// perfect binary tree over MAXP leaves (leaves c >= NC are zero), left
// operand first.  Partials: [H][n_qb][NC][BM][d].  Adding a zero leaf or a
// zero subtree is exact, so the walk stops at NP = the least power of two
// >= NC, which gives the same sums as all MAXP leaves.
constexpr int MAXP = 256;

// Sum of the perfect binary tree over leaves base .. base + N - 1 of the
// chunk partials (leaves >= NC are zero), left operand first.
template <int N>
__device__ __forceinline__ float dq_tree(const float* p0, int64_t stride, int NC, int base) {
  static_assert(N >= 1 && N <= 128 && (N & (N - 1)) == 0, "power-of-two leaf count");
  float s[8];
#pragma unroll
  for (int w = 0; w < N; ++w) {
    float x = base + w < NC ? p0[(int64_t)(base + w) * stride] : 0.f;
    // Leaf w closes one subtree per trailing one bit of w: merge them.
    int lvl = 0;
#pragma unroll
    for (int z = 0; z < 7; ++z) {
      if (((w >> z) & 1) && lvl == z) {
        x = s[z] + x;
        lvl = z + 1;
      }
    }
    s[lvl] = x;
  }
  // the root of the N-leaf tree sits at level log2(N)
  constexpr int ROOT = N >= 128 ? 7 : N >= 64 ? 6 : N >= 32 ? 5 : N >= 16 ? 4 : N >= 8 ? 3 : N >= 4 ? 2 : N >= 2 ? 1 : 0;
  return s[ROOT];
}

template <int NP>
__global__ __launch_bounds__(256) void dq_reduce(const float* __restrict__ part, float* __restrict__ dq,
                                                 int H, int Lq, int d, int BM, int n_qb, int NC, float scale) {
  static_assert(NP >= 1 && NP <= MAXP && (NP & (NP - 1)) == 0, "power-of-two leaf count");
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)H * Lq * d;
  if (e >= n) return;
  const int col = (int)(e % d);
  const int64_t hq = e / d;
  const int q = (int)(hq % Lq), h = (int)(hq / Lq);
  const int qb = q / BM, r = q - qb * BM;
  const int64_t stride = (int64_t)BM * d;  // between the partials of consecutive chunks
  const float* p0 = part + (((int64_t)h * n_qb + qb) * NC) * stride + (int64_t)r * d + col;
  float sum;
  if constexpr (NP <= 128) {
    sum = dq_tree<NP>(p0, stride, NC, 0);
  } else {
    // the root of a 256-leaf tree joins its two 128-leaf halves
    static_assert(NP == 2 * 128, "two halves");
    const float left = dq_tree<128>(p0, stride, NC, 0);
    sum = left + dq_tree<128>(p0, stride, NC, 128);
  }
  dq[e] = sum * scale;
}

// ------------------------------------------------------------------ dQ ----
// dQ for a block of BM = NW*32 query rows: loop over the K/V rows it sees,
// recompute S^T = K Q^T and dP^T = V dO^T, form dS^T = P^T o (dP^T - delta)
// and accumulate dQ^T += K^T dS^T in registers.  One lane owns one query
// row (the forward's layout), so lse and delta are per-lane scalars.
//   self mode:      persistent over the query-block tile list; a tile sees
//                   its own sequence and writes its dQ rows.
//   broadcast mode: one workgroup per (head, query block, chunk); chunk c
//                   takes every NC-th sequence of the length-sorted order
//                   (so chunks get alike mixes of lengths), and writes its
//                   fp32 partial for dq_reduce.
template <int D, int NW, bool CAUSAL, bool BCAST>
struct DqCfg {
  static constexpr int NT = NW * WAVE;
  static constexpr int BN = DQ_KV_STEP;
  static constexpr int BM = NW * 32;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE_BYTES = tile_bytes<BN, D>();
  // d = 128: K/V rows go straight to LDS, three padded rows per copy; each
  // wave copies RPW rows of K and of V per step (IPS copies).
  static constexpr bool DMA = D == 128;
  static constexpr int RPW = BN / NW;
  static constexpr int CPT = PadRowCopy::copies(RPW);
  static constexpr int IPS = 2 * CPT;
  static constexpr int DEP = DMA ? ((2 * IPS <= 63) ? 3 : 2) : 1;
  static constexpr int NBUF = DEP + 1;
  static constexpr int BUF_BYTES = TILE_BYTES + PadRowCopy::GAP;
  static_assert(!DMA || (TileGeom<D>::ROW_BYTES == 19 * 16 && RPW >= 3), "copy geometry");
};

template <int D, int NW, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(NW * WAVE, 1) void dq_kernel(BwdArgs a) {
  using C = DqCfg<D, NW, CAUSAL, BCAST>;
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, DT = C::DT, NT = C::NT;
  constexpr int NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][2][C::BUF_BYTES];  // [buffer][K, V]
  const int tid = threadIdx.x;
  const int wave = tid / WAVE, l = tid % WAVE, g = l / 32, lc = l % 32;
  const PadRowCopy pc;
  const int H = a.H;
  const int64_t ld = (int64_t)a.Hkv * D;  // K / V row stride
  const float c2 = a.scale_log2;

  bf16x8 qreg[KS], doreg[KS];
  float lse2 = INFINITY, del = 0.f;
  f32x16 dqa[DT];
  TileLoader<BN, D, NT> kl, vl;

  // Rows of Q (B operand Q^T) for this wave's query rows.
  auto load_rows = [&](const uint16_t* rowp, bool ok, bf16x8* dst) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *reinterpret_cast<const u32x4*>(rowp + ks * 16 + g * 8);
      dst[ks] = __builtin_bit_cast(bf16x8, x);
    }
  };

  // One K/V step: S^T, dP^T, dS^T, dQ^T += K^T dS^T, two 32-key halves in turn.
  auto step_math = [&](const char* Ks, const char* Vs, int k0, int L, int qi, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int jj = (l & 15) >> 2, cq = ((l >> 4) & 1) * 16 + (l & 3) * 4;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // dP^T starts from -delta (a lane's registers all belong to its query
      // row), so that dS^T = P^T o dP' takes no subtraction.
      f32x16 sacc = f32x16{}, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) dpacc[i] = -del;
      // K / V operands of k-step ks + 1 are read before the products of
      // k-step ks.
      bf16x8 kc = lds_read16(Ks, tile_off<D>(kt * 32 + lc, g));
      bf16x8 vc = lds_read16(Vs, tile_off<D>(kt * 32 + lc, g));
      static_for<0, KS>([&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        bf16x8 kn, vn;
        if constexpr (ks + 1 < KS) {
          const int off = tile_off<D>(kt * 32 + lc, (ks + 1) * 2 + g);
          kn = lds_read16(Ks, off);
          vn = lds_read16(Vs, off);
        }
        sacc = mfma32(kc, qreg[ks], sacc);
        dpacc = mfma32(vc, doreg[ks], dpacc);
        if constexpr (ks + 1 < KS) {
          kc = kn;
          vc = vn;
        }
      });
      uint32_t ta[2];
      i16x4 xk[2][4];
      if constexpr (C::DMA) {
        // The first transposed K reads of dQ^T's products go out before
        // the dS arithmetic.
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          ta[hh] = lds_addr(Ks + tile_off_col4<D>(kt * 32 + hh * 16 + g * 4 + jj, cq));
        tr4_issue<0>(ta[0], ta[0] + 8 * TileGeom<D>::ROW_BYTES, xk[0]);
      }
      // C layout: lane owns query qi; register i is key
      // k0 + kt*32 + 8*(i/4) + 4g + i%4.
      float dsf[16];
      float dsmax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(sacc[i] * c2 - lse2);
        if (MASKED) {
          const int key = k0 + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          const bool ok = key < L && (!CAUSAL || (key <= qi && (a.window <= 0 || key > qi - a.window)));
          pv = ok ? pv : 0.f;
        }
        dsf[i] = pv * dpacc[i];
        dsmax = fmaxf(dsmax, fabsf(dsf[i]));
      }
      // dQ sums dS over many keys (all keys of a chunk of sequences in
      // broadcast mode): large dS values are carried as two bf16 terms.
      const bool split = __any(dsmax > SPLIT_DS);
      uint32_t hi[2][4], lo[2][4];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        hi[i >> 3][(i & 7) >> 1] = pack_bf16x2(dsf[i], dsf[i + 1]);
        lo[i >> 3][(i & 7) >> 1] = 0u;
      }
      if (split) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) split_bf16x2(dsf[i], dsf[i + 1], &hi[i >> 3][(i & 7) >> 1], &lo[i >> 3][(i & 7) >> 1]);
      }
      // dQ^T += K^T dS^T; K^T by transpose read, keys in the order of the
      // dS^T registers.
      if constexpr (C::DMA) {
        // 4 pieces (k-half hh x head-dim tiles 2 hf, 2 hf + 1), each
        // piece's reads issued before the products of the piece before.
        static_assert(DT == 4, "two pieces of two head-dim tiles per k-half");
        static_for<0, 4>([&](auto pc_tag) {
          constexpr int pc = decltype(pc_tag)::value;
          constexpr int hh = pc >> 1, hf = pc & 1;
          if constexpr (pc + 1 < 4) {
            constexpr int nh = (pc + 1) >> 1, nf = (pc + 1) & 1;
            tr4_issue<nf * 128>(ta[nh], ta[nh] + 8 * TileGeom<D>::ROW_BYTES, xk[(pc + 1) & 1]);
            tr4_wait<4>(xk[pc & 1]);
          } else {
            tr4_wait<0>(xk[pc & 1]);
          }
          const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{hi[hh][0], hi[hh][1], hi[hh][2], hi[hh][3]});
#pragma unroll
          for (int k = 0; k < 2; ++k) dqa[2 * hf + k] = mfma32(tr4_operand(xk[pc & 1], k), db, dqa[2 * hf + k]);
          if (split) {
            const bf16x8 dl = __builtin_bit_cast(bf16x8, u32x4{lo[hh][0], lo[hh][1], lo[hh][2], lo[hh][3]});
#pragma unroll
            for (int k = 0; k < 2; ++k) dqa[2 * hf + k] = mfma32(tr4_operand(xk[pc & 1], k), dl, dqa[2 * hf + k]);
          }
        });
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r0 = kt * 32 + hh * 16 + g * 4;
          bf16x8 ka[DT];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) ka[dt] = lds_operand_tr<D>(Ks, r0, r0 + 8, dt * 32);
          const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{hi[hh][0], hi[hh][1], hi[hh][2], hi[hh][3]});
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) dqa[dt] = mfma32(ka[dt], db, dqa[dt]);
          if (split) {
            const bf16x8 dl = __builtin_bit_cast(bf16x8, u32x4{lo[hh][0], lo[hh][1], lo[hh][2], lo[hh][3]});
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) dqa[dt] = mfma32(ka[dt], dl, dqa[dt]);
          }
        }
      }
    }
  };

  // All K/V steps of one sequence (rows s0.. of head h), with the same ring
  // discipline as the forward.  `after_prologue` runs once the first copies
  // are in flight (loads of per-sequence rows go there).
  auto sequence = [&](int64_t s0, int L, int hk, int q0, int wq0, int qi, auto after_prologue) {
    int kv_end = L;
    if (CAUSAL) kv_end = min(kv_end, q0 + BM);
    const int n_kv = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    const int n_bulk = a.window > 0 ? 0 : CAUSAL ? min(q0 / BN, L / BN) : L / BN;  // window: all masked
    // First step with a key inside some row's window; earlier steps are skipped.
    const int j0 = CAUSAL && a.window > 0 ? min(max(0, q0 - a.window + 1) / BN, n_kv) : 0;
    const uint16_t* kbase = a.k + (s0 * a.Hkv + hk) * (int64_t)D;
    const uint16_t* vbase = a.v + (s0 * a.Hkv + hk) * (int64_t)D;
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
    __syncthreads();  // earlier readers of the ring are done
    if constexpr (C::DMA) {
      wait_vmcnt<0>();
      for (int jj = j0; jj < j0 + DEP && jj < n_kv; ++jj) issue(jj);
      after_prologue();
    } else {
      after_prologue();
      if (n_kv > j0) {
        const int r0 = j0 * BN;
        kl.load(kbase + (int64_t)r0 * ld, ld, min(BN, L - r0), tid);
        vl.load(vbase + (int64_t)r0 * ld, ld, min(BN, L - r0), tid);
        kl.store(smem[j0 % NBUF][0], tid);
        vl.store(smem[j0 % NBUF][1], tid);
      }
      __syncthreads();
    }
    auto kv_step = [&](int j, auto masked_tag) {
      const int buf = j % NBUF;
      const int k0 = j * BN;
      if constexpr (C::DMA) {
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
      const bool active = !(CAUSAL && decltype(masked_tag)::value) || (k0 <= wq0 + 31);
      if (active) step_math(smem[buf][0], smem[buf][1], k0, L, qi, masked_tag);
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
  };

  if constexpr (!BCAST) {
    const int slot = logical_slot(blockIdx.x, a.P_dq);
    const int64_t T = *a.n_qtiles;
    // Tile hand-out: the first tile by slot, every later one from a global
    // counter over the rest of the list, fetched one tile ahead (one lane of
    // wave 0, a vector atomic) and shared through LDS at the next tile start.
    __shared__ int s_next;
    unsigned int fetched = 0;
    for (int64_t pass = 0;; ++pass) {
      if (pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
      __syncthreads();
      const int64_t t = pass == 0 ? (int64_t)slot : a.P_dq + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
      if (t >= T) break;
      if (wave == 0 && l == 0) fetched = atomicAdd(a.qtile_ctr, 1u);
      const TileRec tile = a.qtiles[t];
      int64_t s0;
      const int L = (int)seq_range(a.offsets, tile.b, a.total_len, &s0);
      const int h = tile.h;
      const int q0 = tile.blk * BM;
      const int wq0 = q0 + wave * 32;
      const int qi = wq0 + lc;
      const bool q_ok = qi < L;
      load_rows(a.q + ((s0 + qi) * H + h) * (int64_t)D, q_ok, qreg);
      load_rows(a.dout + ((s0 + qi) * H + h) * (int64_t)D, q_ok, doreg);
      lse2 = q_ok ? a.lse[(s0 + qi) * H + h] * LOG2E : INFINITY;
      del = q_ok ? a.delta[(s0 + qi) * H + h] : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};
      sequence(s0, L, tile.hk, q0, wq0, qi, [] {});
      if (q_ok) {
        float* dst = a.dq + ((s0 + qi) * H + h) * (int64_t)D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = dqa[dt][i4 * 4 + e] * a.scale;
            *reinterpret_cast<f32x4*>(dst + dt * 32 + i4 * 8 + g * 4) = v;
          }
      }
    }
  } else {
    const int NC = a.dq_chunks, n_qb = a.dq_qblocks, Lq = a.Lq;
    const int item = blockIdx.x;
    const int h = item / (n_qb * NC);
    const int rem = item - h * n_qb * NC;
    const int qb = rem / NC, c = rem - qb * NC;
    const int q0 = qb * BM;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + lc;
    const bool q_ok = qi < Lq;
    load_rows(a.q + ((int64_t)h * Lq + qi) * D, q_ok, qreg);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};
    for (int r = c; r < a.B; r += NC) {
      const int b = a.seq_order[r];
      int64_t s0;
      const int L = (int)seq_range(a.offsets, b, a.total_len, &s0);
      if (L <= 0) continue;
      const int64_t row = ((int64_t)b * H + h) * Lq + qi;
      sequence(s0, L, h / a.G, q0, wq0, qi, [&] {
        load_rows(a.dout + row * D, q_ok, doreg);
        lse2 = q_ok ? a.lse[row] * LOG2E : INFINITY;
        del = q_ok ? a.delta[row] : 0.f;
      });
    }
    // this chunk's fp32 partial, rows q0.. of (h, qb): [BM][D]
    float* dst = a.dq_part + (int64_t)item * BM * D + (int64_t)(wave * 32 + lc) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dqa[dt][i4 * 4 + e];
        *reinterpret_cast<f32x4*>(dst + dt * 32 + i4 * 8 + g * 4) = v;
      }
  }
}

// Row position of row r of a tile stored with the 4 x 4 transpose within each
// group of 16 rows (its own inverse).
__device__ __forceinline__ int kperm_row(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// Broadcast dQ, d = 128.  One workgroup per (head, 256-row query block,
// chunk); its K/V steps form one stream over the chunk's sequences, copied DEP
// steps ahead across sequence boundaries and issued from inside the S^T / dP^T
// products of the step DEP before.  The next sequence's dO rows, lse and
// delta are loaded at the start of the current one.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(DQ_BM_BCAST * 2, 1) void dq_bcast_kernel(BwdArgs a) {
  constexpr int NW = DQ_BM_BCAST / 32;
  using C = DqCfg<D, NW, CAUSAL, true>;
  static_assert(C::DMA, "direct-copy form");
  constexpr int BN = C::BN, BM = C::BM, KS = C::KS, DT = C::DT;
  constexpr int NBUF = C::NBUF, DEP = C::DEP, IPS = C::IPS, RPW = C::RPW, RB = TileGeom<D>::ROW_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][2][C::BUF_BYTES];  // [buffer][K, V]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const PadRowCopy pc;
  const int H = a.H, Lq = a.Lq, B = a.B;
  const int64_t ld = (int64_t)a.Hkv * D;  // K / V row stride
  const float c2 = a.scale_log2;

  const int NC = a.dq_chunks, n_qb = a.dq_qblocks;
  const int item = blockIdx.x;
  const int h = item / (n_qb * NC);
  const int hk = h / a.G;  // key / value head
  const int rem = item - h * n_qb * NC;
  const int qb = rem / NC, c = rem - qb * NC;
  const int q0 = qb * BM;
  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + lc;
  const bool q_ok = qi < Lq;

  // Q^T operand (B) of this lane's query row; rows past Lq are zero.
  bf16x8 qreg[KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)h * Lq + (q_ok ? qi : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + g * 8);
      if (!q_ok) x = u32x4{0u, 0u, 0u, 0u};
      qreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
  f32x16 dqa[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};

  // A sequence of the chunk: packed rows [s0, s0 + L), its dO / lse / delta
  // rows, and its K/V step counts.
  struct Sq {
    int64_t s0, row;
    int L, n_kv, n_bulk, r;
    int j0;              // first step: the steps before it lie wholly outside every row's window
    const uint16_t* kb;  // K / V rows s0 of head h
    const uint16_t* vb;
  };
  auto seq_at = [&](int r) {
    Sq q;
    q.r = r;
    const int b = a.seq_order[r];
    q.L = (int)seq_range(a.offsets, b, a.total_len, &q.s0);
    q.row = ((int64_t)b * H + h) * Lq;
    q.kb = a.k + (q.s0 * a.Hkv + hk) * (int64_t)D;
    q.vb = a.v + (q.s0 * a.Hkv + hk) * (int64_t)D;
    int kv_end = q.L;
    if (CAUSAL) kv_end = min(kv_end, q0 + BM);
    q.n_kv = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    q.n_bulk = a.window > 0 ? 0 : min(CAUSAL ? min(q0 / BN, q.L / BN) : q.L / BN, q.n_kv);  // window: all masked
    q.j0 = CAUSAL && a.window > 0 ? min(max(0, q0 - a.window + 1) / BN, q.n_kv) : 0;
    return q;
  };
  // The first sequence of the chunk at or after position r with keys to
  // visit (r >= B: none).
  auto next_valid = [&](int r) {
    Sq q;
    q.r = B;
    q.n_kv = 0;
    q.j0 = 0;
    for (; r < B; r += NC) {
      q = seq_at(r);
      if (q.n_kv > q.j0) break;
      q.r = B;
    }
    return q;
  };

  // ---- the step stream (as in the forward).  The K tile is read both ways
  // (16-byte reads of 16 consecutive key rows for S^T, transposing reads of
  // 4 rows for dQ^T += K^T dS^T): key row r of a step sits at row position
  // perm(r), the 4 x 4 transpose within each group of 16 rows, which keeps
  // both reads free of bank conflicts with 304-byte rows (as the Q / dO
  // tiles of the dK / dV kernel).  Position p of a copy takes key row
  // perm(p) of the step, fixed per lane and copy; V is read one way only.
  int g_iss = 0, g_cmp = 0, iss_cur = 0, iss_nxt = 0;
  const uint16_t* j_k = a.k;
  const uint16_t* j_v = a.v;
  uint32_t j_kd = 0, j_vd = 0;
  int j_last = 0, j_lastk = 0;
  bool j_on = false;
  int kperm[C::CPT];
#pragma unroll
  for (int k = 0; k < C::CPT; ++k)
    kperm[k] = kperm_row(wave * RPW + PadRowCopy::start(k, RPW) + (int)PadRowCopy::lane_row(l));
  auto prep_next = [&](const Sq& cp, const Sq& np, bool has_nxt) {
    const int nn = has_nxt ? np.n_kv - np.j0 : 0;
    const bool cur = iss_cur < cp.n_kv - cp.j0;
    j_on = cur || iss_nxt < nn;
    if (!j_on) return;
    const int L_ = cur ? cp.L : np.L;
    const int j = cur ? cp.j0 + iss_cur : np.j0 + iss_nxt;
    const int base_row = min(j * BN + wave * RPW, L_ - 1);
    // byte offsets of rows within the sequence (32 x 32-bit products); K from
    // the step's first row (j BN < L), V from this wave's first
    const uint64_t roff = (uint64_t)(uint32_t)base_row * (uint32_t)(ld * 2);
    const uint64_t koff = (uint64_t)(uint32_t)(j * BN) * (uint32_t)(ld * 2);
    j_k = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(cur ? cp.kb : np.kb) + koff);
    j_v = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(cur ? cp.vb : np.vb) + roff);
    j_last = L_ - 1 - base_row;
    j_lastk = L_ - 1 - j * BN;
    const int buf = (int)((uint32_t)g_iss % NBUF);
    j_kd = lds_addr(smem[buf][0]) + wave * RPW * RB;
    j_vd = lds_addr(smem[buf][1]) + wave * RPW * RB;
    if (cur) ++iss_cur;
    else ++iss_nxt;
    ++g_iss;
  };
  auto issue_copies = [&](int k0, int k1) {
    if (!j_on) return;
#pragma unroll
    for (int k = k0; k < k1; ++k) {
      const int R = PadRowCopy::start(k % C::CPT, RPW);
      if (k < C::CPT) {
        const uint32_t vo = (uint32_t)min(kperm[k], j_lastk) * (uint32_t)(ld * 2) + pc.byte;
        dma_copy16(j_k, vo, j_kd + R * RB);
      } else {
        dma_copy16(j_v, pc.voff(R, j_last, (uint32_t)(ld * 2)), j_vd + R * RB);
      }
    }
  };

  // Per-sequence operands of this lane's query row: dO (A operand of dP^T's
  // B side), lse * log2(e) and delta; the next sequence's are loaded ahead.
  bf16x8 doreg[KS], don[KS];
  float lse2 = INFINITY, del = 0.f, lse2n = INFINITY, deln = 0.f;
  auto load_seq = [&](const Sq& q) {
    const int64_t row = q.row + (q_ok ? qi : 0);
    const uint16_t* dr = a.dout + row * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) don[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dr + ks * 16 + g * 8));
    lse2n = a.lse2[row];
    deln = a.delta[row];
  };

  Sq cp = next_valid(c);
  if (cp.r < B) load_seq(cp);
  while (cp.r < B) {
    const Sq np = next_valid(cp.r + NC);
    const bool has_nxt = np.r < B;
    // This sequence's operands (loaded during the previous one, so only the
    // copies issued since, which the prefetched steps need anyway, are
    // waited for with them).
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = __builtin_bit_cast(u32x4, don[ks]);
      asm volatile("" : "+v"(x));
      doreg[ks] = __builtin_bit_cast(bf16x8, x);
    }
    asm volatile("" : "+v"(lse2n), "+v"(deln));
    lse2 = q_ok ? lse2n : INFINITY;
    del = q_ok ? deln : 0.f;
    if (has_nxt) load_seq(np);
    const int L = cp.L, n_kv = cp.n_kv;
    {
      const int need = min(DEP, n_kv - cp.j0);
      if (iss_cur < need) {
        while (iss_cur < need) {
          prep_next(cp, np, has_nxt);
          issue_copies(0, 2 * C::CPT);
        }
      }
    }
    auto kv_step = [&](int j, auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int buf = (int)((uint32_t)g_cmp % NBUF);
      const int k0 = j * BN;
      // Wait for this wave's copies of the step: the copies issued after it
      // may stay in flight.  (Copies issued before this sequence's operand
      // loads were already waited for with them, and the next sequence's
      // operand loads, issued before any later copy, need no wait here.)
      {
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
      const bool active = !(CAUSAL && MASKED) || (k0 <= wq0 + 31);
      if (!active) {
        issue_copies(0, 2 * C::CPT);
      } else {
        const char* Ks = smem[buf][0];
        const char* Vs = smem[buf][1];
        const int jj = (l & 15) >> 2, cq = ((l >> 4) & 1) * 16 + (l & 3) * 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x16 sacc = f32x16{}, dpacc = f32x16{};
          // K / V operands of k-step ks + 1 are read before the products of
          // k-step ks.
          const int kpos = kperm_row(kt * 32 + lc);  // row position of this lane's key
          bf16x8 kc = lds_read16(Ks, tile_off<D>(kpos, g));
          bf16x8 vc = lds_read16(Vs, tile_off<D>(kt * 32 + lc, g));
          static_for<0, KS>([&](auto ks_tag) {
            constexpr int ks = decltype(ks_tag)::value;
            bf16x8 kn, vn;
            if constexpr (ks + 1 < KS) {
              kn = lds_read16(Ks, tile_off<D>(kpos, (ks + 1) * 2 + g));
              vn = lds_read16(Vs, tile_off<D>(kt * 32 + lc, (ks + 1) * 2 + g));
            }
            sacc = mfma32(kc, qreg[ks], sacc);
            dpacc = mfma32(vc, doreg[ks], dpacc);
            if (kt == 0) {
              constexpr int PER = (2 * C::CPT + KS - 1) / KS;
              issue_copies(ks * PER, min((ks + 1) * PER, 2 * C::CPT));
            }
            if constexpr (ks + 1 < KS) {
              kc = kn;
              vc = vn;
            }
          });
          // The first transposed K reads of dQ^T's products go out before
          // the dS arithmetic.
          uint32_t ta[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) ta[hh] = lds_addr(Ks + tile_off_col4<D>(kperm_row(kt * 32 + hh * 16 + g * 4 + jj), cq));
          // rows r and r + 8 (r < 8 within its group) sit 2 positions apart
          i16x4 xk[2][4];
          tr4_issue<0>(ta[0], ta[0] + 2 * RB, xk[0]);
          // C layout: lane owns query qi; register i is key
          // k0 + kt*32 + 8*(i/4) + 4g + i%4.
          float dsf[16];
          float dsmax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pv = fast_exp2(sacc[i] * c2 - lse2);
            if (MASKED) {
              const int key = k0 + kt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
              const bool ok = key < L && (!CAUSAL || (key <= qi && (a.window <= 0 || key > qi - a.window)));
              pv = ok ? pv : 0.f;
            }
            dsf[i] = pv * (dpacc[i] - del);
            dsmax = fmaxf(dsmax, fabsf(dsf[i]));
          }
          const bool split = __any(dsmax > SPLIT_DS);
          uint32_t hi[2][4], lo[2][4];
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            hi[i >> 3][(i & 7) >> 1] = pack_bf16x2(dsf[i], dsf[i + 1]);
            lo[i >> 3][(i & 7) >> 1] = 0u;
          }
          if (split) {
#pragma unroll
            for (int i = 0; i < 16; i += 2) split_bf16x2(dsf[i], dsf[i + 1], &hi[i >> 3][(i & 7) >> 1], &lo[i >> 3][(i & 7) >> 1]);
          }
          // dQ^T += K^T dS^T in 4 pieces (k-half hh x head-dim tiles 2 hf,
          // 2 hf + 1); each piece's transposed reads are issued before the
          // products of the piece before.
          static_for<0, 4>([&](auto pc_tag) {
            constexpr int pc = decltype(pc_tag)::value;
            constexpr int hh = pc >> 1, hf = pc & 1;
            if constexpr (pc + 1 < 4) {
              constexpr int nh = (pc + 1) >> 1, nf = (pc + 1) & 1;
              tr4_issue<nf * 128>(ta[nh], ta[nh] + 2 * RB, xk[(pc + 1) & 1]);
              tr4_wait<4>(xk[pc & 1]);
            } else {
              tr4_wait<0>(xk[pc & 1]);
            }
            const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{hi[hh][0], hi[hh][1], hi[hh][2], hi[hh][3]});
#pragma unroll
            for (int k = 0; k < 2; ++k) dqa[2 * hf + k] = mfma32(tr4_operand(xk[pc & 1], k), db, dqa[2 * hf + k]);
            if (split) {
              const bf16x8 dl = __builtin_bit_cast(bf16x8, u32x4{lo[hh][0], lo[hh][1], lo[hh][2], lo[hh][3]});
#pragma unroll
              for (int k = 0; k < 2; ++k) dqa[2 * hf + k] = mfma32(tr4_operand(xk[pc & 1], k), dl, dqa[2 * hf + k]);
            }
          });
        }
      }
      ++g_cmp;
    };
    for (int j = cp.j0; j < cp.n_bulk; ++j) kv_step(j, std::false_type{});
    for (int j = max(cp.n_bulk, cp.j0); j < n_kv; ++j) kv_step(j, std::true_type{});
    cp = np;
    iss_cur = iss_nxt;
    iss_nxt = 0;
  }
  // this chunk's fp32 partial, rows q0.. of (h, qb): [BM][D]
  float* dst = a.dq_part + (int64_t)item * BM * D + (int64_t)(wave * 32 + lc) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = dqa[dt][i4 * 4 + e];
      *reinterpret_cast<f32x4*>(dst + dt * 32 + i4 * 8 + g * 4) = v;
    }
}

// ------------------------------------------------------- group sum ----
// Grouped-query heads: the dK / dV of a key / value head is the sum over the
// query heads that share it, taken here in ascending head order from the
// per-query-head slices the dK / dV kernel wrote.  One thread per 16 bytes of
// the output.
__global__ __launch_bounds__(256) void group_sum_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst,
                                                        int64_t n, int Hkv, int G, int D4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int64_t t = e / ((int64_t)Hkv * D4);
    const int rem = (int)(e - t * Hkv * D4);
    const int hk = rem / D4, c = rem - hk * D4;
    const f32x4* s = src + (t * Hkv * G + (int64_t)hk * G) * D4 + c;
    f32x4 acc = s[0];
    for (int i = 1; i < G; ++i) acc += s[(int64_t)i * D4];
    dst[e] = acc;
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  const int64_t rows = a.broadcast_q ? (int64_t)a.B * a.H * a.Lq : a.total_len * a.H;
  if (rows > 0) {
    const int64_t work = rows * (D / 8);
    const int64_t want = (work + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    JFA_TIMED_LAUNCH(K_DELTA, st, (delta_kernel<D>), dim3(blocks), dim3(256), 0, st, a.out, a.dout, a.lse, a.delta,
                     a.lse2, reinterpret_cast<u32x4*>(a.term_l), reinterpret_cast<u32x4*>(a.term_d),
                     1.0f / a.scale, rows, a.offsets, a.total_len, a.broadcast_q ? a.H * a.Lq : 0, a.Lq, a.causal);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_dkdv(a, st);
  if (e != hipSuccess) return e;
  if (a.broadcast_q) {
    const int items = a.H * a.dq_qblocks * a.dq_chunks;
    if constexpr (D == 128) {
      if (a.causal)
        JFA_TIMED_LAUNCH(K_DQ, st, (dq_bcast_kernel<D, true>), dim3(items), dim3(DQ_BM_BCAST * 2), 0, st, a);
      else
        JFA_TIMED_LAUNCH(K_DQ, st, (dq_bcast_kernel<D, false>), dim3(items), dim3(DQ_BM_BCAST * 2), 0, st, a);
    } else {
      if (a.causal)
        JFA_TIMED_LAUNCH(K_DQ, st, (dq_kernel<D, DQ_BM_BCAST / 32, true, true>), dim3(items), dim3(DQ_BM_BCAST * 2), 0, st, a);
      else
        JFA_TIMED_LAUNCH(K_DQ, st, (dq_kernel<D, DQ_BM_BCAST / 32, false, true>), dim3(items), dim3(DQ_BM_BCAST * 2), 0, st, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_dq_reduce(a.dq_part, a.dq, a.H, a.Lq, D, DQ_BM_BCAST, a.dq_qblocks, a.dq_chunks, a.scale, st);
  }
  // Tiles of 256 rows: 8 waves, two per SIMD, as in the forward.
  if (a.causal)
    JFA_TIMED_LAUNCH(K_DQ, st, (dq_kernel<D, DQ_BM / 32, true, false>), dim3(a.P_dq), dim3(DQ_BM * 2), 0, st, a);
  else
    JFA_TIMED_LAUNCH(K_DQ, st, (dq_kernel<D, DQ_BM / 32, false, false>), dim3(a.P_dq), dim3(DQ_BM * 2), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_group_sum(const float* src, float* dst, int64_t total_len, int H, int Hkv, int d,
                            hipStream_t stream) {
  const int64_t n = total_len * Hkv * (d / 4);
  if (n == 0) return hipSuccess;
  const int64_t want = (n + 255) / 256;
  const int blocks = (int)(want < 4096 ? want : 4096);
  JFA_TIMED_LAUNCH(K_GROUP_SUM, stream, group_sum_kernel, dim3(blocks), dim3(256), 0, stream,
                   reinterpret_cast<const f32x4*>(src), reinterpret_cast<f32x4*>(dst), n, Hkv, H / Hkv, d / 4);
  return hipGetLastError();
}

hipError_t launch_dq_reduce(const float* part, float* dq, int H, int Lq, int d, int BM, int n_qb, int NC,
                            float scale, hipStream_t st) {
  const int64_t n = (int64_t)H * Lq * d;
  if (n == 0) return hipSuccess;
  int np2 = 1;
  while (np2 < NC) np2 <<= 1;
  const dim3 grid((unsigned)((n + 255) / 256));
#define JFA_DQ_REDUCE(NPV)                                                                                     \
  case NPV:                                                                                                    \
    JFA_TIMED_LAUNCH(K_DQ_REDUCE, st, dq_reduce<NPV>, grid, dim3(256), 0, st, part, dq, H, Lq, d, BM, n_qb, NC, \
                     scale);                                                                                   \
    break;
  switch (np2) {
    JFA_DQ_REDUCE(1)
    JFA_DQ_REDUCE(2)
    JFA_DQ_REDUCE(4)
    JFA_DQ_REDUCE(8)
    JFA_DQ_REDUCE(16)
    JFA_DQ_REDUCE(32)
    JFA_DQ_REDUCE(64)
    JFA_DQ_REDUCE(128)
    JFA_DQ_REDUCE(256)
    default: return hipErrorInvalidValue;
  }
#undef JFA_DQ_REDUCE
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.broadcast_q && a.dq_chunks > MAXP) return hipErrorInvalidValue;
  if (a.d == 64) return launch_bwd_d<64>(a, stream);
  return launch_bwd_d<128>(a, stream);
}

}  // namespace jfa
