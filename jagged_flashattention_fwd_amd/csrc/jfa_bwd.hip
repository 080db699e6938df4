// Jagged flash-attention backward for gfx950.
//
// The gradient of O = softmax(scale Q K^T) V, with P recomputed from the
// forward's lse:  dP = dO V^T,  delta_i = sum_d dO_id O_id,
// dS = P o (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// In broadcast mode dQ is summed over every sequence of the batch
// ("Optimizing Jagged Flash Attention with TLX", "1. The Challenge").
//
// Kernels, in launch order:
//   delta_kernel   streaming pre-pass, delta = rowsum(dO o O) (O as stored).
//   dkdv_kernel    persistent; a tile is 128 keys of one (sequence, head), its
//                  K/V held in registers while query blocks of 64 rows stream
//                  through LDS -- the K/V-outer, dense-Q-inner loop of
//                  "Scheduling jagged tiles across SMs".  Per query block:
//                  S = Q K^T, dP = dO V^T, P, dS, dV += P^T dO, dK += dS^T Q
//                  and, in broadcast mode, the fifth product dQ += dS K
//                  ("2-CTA collaborative MMA (backward)" counts five GEMMs per
//                  K/V block).  Broadcast dQ goes to a private fp32 partial
//                  per workgroup instead of a contended reduce-add into one
//                  buffer ("Multi-stage dQ staging" names that reduce-add the
//                  main backward bottleneck); the tile list is handed out
//                  statically, so each partial sums in a fixed order.
//   dq_reduce      sums the partials with a fixed pairwise tree (bitwise
//                  reproducible), times scale.
//   dq_self_kernel self-attention dQ: a tile is 128 query rows; loops over
//                  K/V steps recomputing S^T, dP^T, dS^T and accumulating
//                  dQ^T += K^T dS^T.  No atomics.
// Loops are peeled ("Loop peeling"): the causal diagonal blocks take the
// masked path, the rest do not.
#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

constexpr int NW = 4;
constexpr int NT = NW * WAVE;
// Split thresholds of the two-term bf16 operands in dV and dK (see dkdv_kernel).
constexpr float SPLIT_P = 1.0f / 16.0f;
constexpr float SPLIT_DS = 0.25f;

// ------------------------------------------------------------- delta ----
// Rows of d elements; D/8 threads per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    float* __restrict__ delta, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = gtid; e < rows * TPR; e += stride) {
    const int64_t row = e / TPR;
    const int c = (int)(e % TPR);
    const u32x4 o = *reinterpret_cast<const u32x4*>(out + row * D + c * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_lo(o[i]) * bf16_lo(g[i]);
      acc += bf16_hi(o[i]) * bf16_hi(g[i]);
    }
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
    if (c == 0) delta[row] = acc;
  }
}

// ------------------------------------------------------------- dK / dV ----
constexpr int PDP_PAD = 4;  // fp32 row padding of the P o dP staging tile

template <int D, bool CAUSAL, bool BCAST>
struct DkdvSmem {
  static constexpr int QB = BWD_QB;
  static constexpr int BN = BWD_BN;
  static constexpr int QTILE = tile_bytes<QB, D>();
  char q[2][QTILE];
  char dout[2][QTILE];
  float lse2[2][QB];
  float delta[2][QB];
  float dpart[4][QB];  // per-wave partial row sums of P o dP
  int split[4];        // per-wave: dS carried as two bf16 terms
  char k[BCAST ? tile_bytes<BN, D>() : 16];
  union {
    struct {
      char hi[BN * TR_ONLY_ROW_BYTES_64];  // dS as [key][query], bf16 high terms
      char lo[BN * TR_ONLY_ROW_BYTES_64];  // bf16 remainders (zero where not split)
    } ds;
    float pdp[BN][QB + PDP_PAD];  // P o dP as [key][query]
  } u;
};

template <int D, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int QB = BWD_QB, BN = BWD_BN, KS = D / 16, DT = D / 32;
  using Smem = DkdvSmem<D, CAUSAL, BCAST>;
  __shared__ __attribute__((aligned(16))) Smem sm;

  const int tid = threadIdx.x;
  const int wave = tid / WAVE, l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_ktiles;
  const int H = a.H, Lq = a.Lq;
  const int64_t ld = (int64_t)H * D;
  const float c2 = a.scale_log2;

  float* part = nullptr;
  if (BCAST) {
    // This workgroup's private dQ partial [H][Lq][D], cleared first.
    const int64_t n = (int64_t)H * Lq * D;
    part = a.dq_part + (int64_t)slot * n;
    for (int64_t i = (int64_t)tid * 4; i < n; i += NT * 4)
      *reinterpret_cast<f32x4*>(part + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int64_t pass = 0;; ++pass) {
    const int64_t t = zigzag_tile(pass, slot, a.P);
    if (t >= T) break;
    const TileRec tile = a.ktiles[t];
    int64_t s0;
    const int L = (int)seq_range(a.offsets, tile.b, a.total_len, &s0);
    const int h = tile.h;
    const int k0 = tile.blk * BN;         // first key of the tile
    const int kw = k0 + wave * 32 + lc;   // this lane's key
    const bool key_ok = kw < L;
    const int nq = BCAST ? Lq : L;
    // When the tile holds every key of its sequence, delta is recomputed
    // here as rowsum(P o dP) from fp32 P and dP, instead of rowsum(dO o O)
    // from the bf16-rounded O: for short sequences P is large and the O
    // rounding would otherwise dominate the dK and dQ error.
    const bool exact_delta = L <= BN;

    // K and V rows of this lane's key as B operands (B[d][key] = K[key][d]).
    bf16x8 kreg[KS], vreg[KS];
    {
      const uint16_t* kr = a.k + ((s0 + kw) * H + h) * (int64_t)D;
      const uint16_t* vr = a.v + ((s0 + kw) * H + h) * (int64_t)D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (key_ok) {
          x = *reinterpret_cast<const u32x4*>(kr + ks * 16 + g * 8);
          y = *reinterpret_cast<const u32x4*>(vr + ks * 16 + g * 8);
        }
        kreg[ks] = __builtin_bit_cast(bf16x8, x);
        vreg[ks] = __builtin_bit_cast(bf16x8, y);
      }
    }
    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dk[dt] = f32x16{}; dv[dt] = f32x16{}; }

    // Query blocks that can see a key of this tile.
    const int m_first = CAUSAL ? k0 / QB : 0;
    const int m_end = (nq + QB - 1) / QB;        // exclusive
    // Blocks whose rows all lie at or after the tile's last key need no causal mask.
    const int m_nomask = CAUSAL ? (k0 + BN - 1 + QB - 1) / QB : 0;

    const uint16_t* qbase = BCAST ? a.q + (int64_t)h * Lq * D : a.q + (s0 * H + h) * (int64_t)D;
    const int64_t qld = BCAST ? D : ld;
    const uint16_t* dobase = BCAST ? a.dout + ((int64_t)tile.b * H + h) * Lq * D
                                   : a.dout + (s0 * H + h) * (int64_t)D;
    const float* lse_base = BCAST ? a.lse + ((int64_t)tile.b * H + h) * Lq : a.lse + s0 * H + h;
    float* del_base = BCAST ? a.delta + ((int64_t)tile.b * H + h) * Lq : a.delta + s0 * H + h;
    const int64_t sld = BCAST ? 1 : H;  // stride between rows of lse / delta

    TileLoader<QB, D, NT> ql, dol;
    float sv = 0.f;  // lse2 (threads 0..63) or delta (64..127) of the next block
    auto load_block = [&](int m) {
      const int r0 = m * QB;
      const int nr = min(QB, nq - r0);
      ql.load(qbase + (int64_t)r0 * qld, qld, nr, tid);
      dol.load(dobase + (int64_t)r0 * qld, qld, nr, tid);
      if (tid < QB) {
        sv = tid < nr ? lse_base[(int64_t)(r0 + tid) * sld] * LOG2E : INFINITY;
      } else if (tid < 2 * QB) {
        const int r = tid - QB;
        sv = r < nr ? del_base[(int64_t)(r0 + r) * sld] : 0.f;
      }
    };
    auto store_block = [&](int buf) {
      ql.store(sm.q[buf], tid);
      dol.store(sm.dout[buf], tid);
      if (tid < QB) sm.lse2[buf][tid] = sv;
      else if (tid < 2 * QB) sm.delta[buf][tid - QB] = sv;
    };

    __syncthreads();  // the previous tile's readers are done with LDS
    if (m_first < m_end) {
      load_block(m_first);
      store_block(0);
    }
    if (BCAST) {
      TileLoader<BN, D, NT> kl;
      kl.load(a.k + (s0 * H + h) * (int64_t)D + (int64_t)k0 * ld, ld, min(BN, L - k0), tid);
      kl.store(sm.k, tid);
    }
    __syncthreads();

    for (int m = m_first; m < m_end; ++m) {
      const int buf = (m - m_first) & 1;
      if (m + 1 < m_end) load_block(m + 1);
      const char* Qs = sm.q[buf];
      const char* Ds = sm.dout[buf];
      const bool diag = CAUSAL && m < m_nomask;

      // S = Q K^T and dP = dO V^T for query subtile s (32 rows) of the block.
      // C layout: lane owns key kw; register i is query row
      // m*QB + s*32 + 8*(i/4) + 4g + i%4.
      auto scores = [&](int s, f32x16& sacc, f32x16& dpacc) {
        sacc = f32x16{};
        dpacc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = tile_off<D>(s * 32 + lc, ks * 2 + g);
          sacc = mfma32(lds_read16(Qs, off), kreg[ks], sacc);
          dpacc = mfma32(lds_read16(Ds, off), vreg[ks], dpacc);
        }
      };
      auto probs = [&](int s, const f32x16& sacc, float* pf) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = s * 32 + i4 * 8 + g * 4;
          const f32x4 ls = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][r]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i4 * 4 + e;
            const float pv = fast_exp2(sacc[i] * c2 - ls[e]);
            bool ok = key_ok;
            if (diag) ok = ok && (kw <= m * QB + r + e);
            pf[i] = ok ? pv : 0.f;
          }
        }
      };

      if (exact_delta) {
        // delta = rowsum(P o dP) over every key of the sequence (all in this
        // tile); S and dP are recomputed below.
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          f32x16 sacc, dpacc;
          scores(s, sacc, dpacc);
          float pf[16];
          probs(s, sacc, pf);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = pf[i4 * 4 + e] * dpacc[i4 * 4 + e];
            *reinterpret_cast<f32x4*>(&sm.u.pdp[wave * 32 + lc][s * 32 + i4 * 8 + g * 4]) = v;
          }
        }
        __syncthreads();
        {
          const int q = tid & (QB - 1), kq = tid >> 6;  // 4 ranges of 32 keys
          float acc = 0.f;
#pragma unroll 8
          for (int kk = 0; kk < 32; ++kk) acc += sm.u.pdp[kq * 32 + kk][q];
          sm.dpart[kq][q] = acc;
        }
        __syncthreads();
        if (tid < QB) {
          const float dsum = (sm.dpart[0][tid] + sm.dpart[1][tid]) + (sm.dpart[2][tid] + sm.dpart[3][tid]);
          sm.delta[buf][tid] = dsum;
          // the self-attention dQ kernel runs next and reads it
          if (!BCAST && m * QB + tid < nq) del_base[(int64_t)(m * QB + tid) * sld] = dsum;
        }
        __syncthreads();
      }

      bool split_ds_any = false;
#pragma unroll 1
      for (int s = 0; s < 2; ++s) {
        f32x16 sacc, dpacc;
        scores(s, sacc, dpacc);
        float pf[16], dsf[16];
        probs(s, sacc, pf);
        float pmax = 0.f, dsmax = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 dl = *reinterpret_cast<const f32x4*>(&sm.delta[buf][s * 32 + i4 * 8 + g * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i4 * 4 + e;
            dsf[i] = pf[i] * (dpacc[i] - dl[e]);
            pmax = fmaxf(pmax, pf[i]);
            dsmax = fmaxf(dsmax, fabsf(dsf[i]));
          }
        }
        // Rounding P or dS to bf16 costs up to 2^-9 of each value, and dV /
        // dK / dQ sum that error over many queries or keys.  Where a value is
        // large (short or sharply peaked sequences) the operand is split into
        // a truncated bf16 high part and a rounded bf16 remainder and the
        // product is taken twice; elsewhere one rounded bf16 operand is used.
        const bool split_p = __any(pmax > SPLIT_P);
        const bool split_ds = __any(dsmax > SPLIT_DS);
        split_ds_any = split_ds_any || split_ds;
        uint32_t pp[2][4], dsp[2][4], plo[2][4], dslo[2][4];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const int hh = i >> 3, e = (i & 7) >> 1;
          if (split_p) {
            split_bf16x2(pf[i], pf[i + 1], &pp[hh][e], &plo[hh][e]);
          } else {
            pp[hh][e] = pack_bf16x2(pf[i], pf[i + 1]);
            plo[hh][e] = 0u;
          }
          if (split_ds) {
            split_bf16x2(dsf[i], dsf[i + 1], &dsp[hh][e], &dslo[hh][e]);
          } else {
            dsp[hh][e] = pack_bf16x2(dsf[i], dsf[i + 1]);
            dslo[hh][e] = 0u;
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS: A operands are transposed reads
        // of the query-major tiles; k-slots = the query rows of the P / dS
        // register pairs.
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r0 = s * 32 + hh * 16 + g * 4;
          const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pp[hh][0], pp[hh][1], pp[hh][2], pp[hh][3]});
          const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{dsp[hh][0], dsp[hh][1], dsp[hh][2], dsp[hh][3]});
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 doa = lds_operand_tr<D>(Ds, r0, r0 + 8, dt * 32);
            const bf16x8 qa = lds_operand_tr<D>(Qs, r0, r0 + 8, dt * 32);
            dv[dt] = mfma32(doa, pb, dv[dt]);
            dk[dt] = mfma32(qa, db, dk[dt]);
            if (split_p) {
              const bf16x8 pl = __builtin_bit_cast(bf16x8, u32x4{plo[hh][0], plo[hh][1], plo[hh][2], plo[hh][3]});
              dv[dt] = mfma32(doa, pl, dv[dt]);
            }
            if (split_ds) {
              const bf16x8 dl = __builtin_bit_cast(bf16x8, u32x4{dslo[hh][0], dslo[hh][1], dslo[hh][2], dslo[hh][3]});
              dk[dt] = mfma32(qa, dl, dk[dt]);
            }
          }
        }
        if (BCAST) {
          // dS (two bf16 terms) to LDS as [key][query]: this wave's 32 key rows.
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int col = s * 32 + i4 * 8 + g * 4;
            const int off = tile_off_col4<QB, TR_ONLY_ROW_BYTES_64>(wave * 32 + lc, col);
            const int hh = i4 >> 1, e0 = (i4 & 1) * 2;
            *reinterpret_cast<u32x2*>(sm.u.ds.hi + off) = u32x2{dsp[hh][e0], dsp[hh][e0 + 1]};
            *reinterpret_cast<u32x2*>(sm.u.ds.lo + off) = u32x2{dslo[hh][e0], dslo[hh][e0 + 1]};
          }
        }
      }

      if (BCAST) {
        if (l == 0) sm.split[wave] = split_ds_any ? 1 : 0;
        if (m == m_first) __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bool any_split = (sm.split[0] | sm.split[1] | sm.split[2] | sm.split[3]) != 0;
        // dQ[q][d] (block) = sum over the tile's 128 keys of dS[q][key] K[key][d].
        // Wave w: query subtile (w & 1), head-dim tiles of half (w >> 1).
        constexpr int DTW = DT / 2;
        const int qs = wave & 1;
        f32x16 dqa[DTW];
#pragma unroll
        for (int x = 0; x < DTW; ++x) dqa[x] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < BN / 16; ++kk) {
          const int kr0 = kk * 16 + g * 8;
          const bf16x8 ahi = lds_operand_tr<QB, TR_ONLY_ROW_BYTES_64>(sm.u.ds.hi, kr0, kr0 + 4, qs * 32);
          bf16x8 alo = ahi;
          if (any_split) alo = lds_operand_tr<QB, TR_ONLY_ROW_BYTES_64>(sm.u.ds.lo, kr0, kr0 + 4, qs * 32);
#pragma unroll
          for (int x = 0; x < DTW; ++x) {
            const int dt = (wave >> 1) * DTW + x;
            const bf16x8 kb = lds_operand_tr<D>(sm.k, kr0, kr0 + 4, dt * 32);
            dqa[x] = mfma32(ahi, kb, dqa[x]);
            if (any_split) dqa[x] = mfma32(alo, kb, dqa[x]);
          }
        }
        // C layout: lane -> head-dim column, registers -> query rows.
#pragma unroll
        for (int x = 0; x < DTW; ++x) {
          const int dcol = ((wave >> 1) * DTW + x) * 32 + lc;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = m * QB + qs * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
            if (q < Lq) {
              float* dst = part + ((int64_t)h * Lq + q) * D + dcol;
              unsafeAtomicAdd(dst, dqa[x][i]);
            }
          }
        }
      }
      if (m + 1 < m_end) store_block(buf ^ 1);
      __syncthreads();
    }

    // dK = scale * dS^T Q, dV = P^T dO for this lane's key; C layout: lane ->
    // key, registers -> head-dim rows 8*(i/4) + 4g + i%4 of each 32-wide tile.
    if (key_ok) {
      float* dkr = a.dk + ((s0 + kw) * H + h) * (int64_t)D;
      float* dvr = a.dv + ((s0 + kw) * H + h) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = dt * 32 + i4 * 8 + g * 4;
          f32x4 kv, vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[e] = dk[dt][i4 * 4 + e] * a.scale;
            vv[e] = dv[dt][i4 * 4 + e];
          }
          *reinterpret_cast<f32x4*>(dkr + d0) = kv;
          *reinterpret_cast<f32x4*>(dvr + d0) = vv;
        }
    }
  }
}

// --------------------------------------------------------- dQ reduce ----
// dq[e] = scale * sum_{w < P} part[w][e], summed as a perfect binary tree
// over MAXP leaves (leaves w >= P are zero), left operand first.
constexpr int MAXP = 256;

__global__ __launch_bounds__(256) void dq_reduce(const float* __restrict__ part, float* __restrict__ dq,
                                                 int64_t n, int P, float scale) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float s[9];
#pragma unroll
  for (int w = 0; w < MAXP; ++w) {
    float x = w < P ? part[(int64_t)w * n + e] : 0.f;
    // Leaf w closes one subtree per trailing one bit of w: merge them.
    int lvl = 0;
#pragma unroll
    for (int z = 0; z < 8; ++z) {
      if (((w >> z) & 1) && lvl == z) {
        x = s[z] + x;
        lvl = z + 1;
      }
    }
    s[lvl] = x;
  }
  dq[e] = s[8] * scale;
}

// ------------------------------------------------ self-attention dQ ----
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dq_self_kernel(BwdArgs a) {
  constexpr int BN = DQ_KV_STEP, KS = D / 16, DT = D / 32, BM = DQ_BM;
  __shared__ __attribute__((aligned(16))) char smem[2][2][tile_bytes<BN, D>()];  // [buffer][K, V]
  const int tid = threadIdx.x;
  const int wave = tid / WAVE, l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P_dq);
  const int64_t T = *a.n_qtiles;
  const int H = a.H;
  const int64_t ld = (int64_t)H * D;
  const float c2 = a.scale_log2;

  for (int64_t pass = 0;; ++pass) {
    const int64_t t = zigzag_tile(pass, slot, a.P_dq);
    if (t >= T) break;
    const TileRec tile = a.qtiles[t];
    int64_t s0;
    const int L = (int)seq_range(a.offsets, tile.b, a.total_len, &s0);
    const int h = tile.h;
    const int q0 = tile.blk * BM;
    const int wq0 = q0 + wave * 32;
    const int qi = wq0 + lc;
    const bool q_ok = qi < L;

    bf16x8 qreg[KS], doreg[KS];
    {
      const uint16_t* qr = a.q + ((s0 + qi) * H + h) * (int64_t)D;
      const uint16_t* dr = a.dout + ((s0 + qi) * H + h) * (int64_t)D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (q_ok) {
          x = *reinterpret_cast<const u32x4*>(qr + ks * 16 + g * 8);
          y = *reinterpret_cast<const u32x4*>(dr + ks * 16 + g * 8);
        }
        qreg[ks] = __builtin_bit_cast(bf16x8, x);
        doreg[ks] = __builtin_bit_cast(bf16x8, y);
      }
    }
    const float lse2 = q_ok ? a.lse[(s0 + qi) * H + h] * LOG2E : INFINITY;
    const float del = q_ok ? a.delta[(s0 + qi) * H + h] : 0.f;

    f32x16 dqa[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dqa[dt] = f32x16{};

    int kv_end = L;
    if (CAUSAL) kv_end = min(kv_end, q0 + BM);
    const int n_kv = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    const int n_bulk = CAUSAL ? min(q0 / BN, L / BN) : L / BN;

    const uint16_t* kbase = a.k + (s0 * H + h) * (int64_t)D;
    const uint16_t* vbase = a.v + (s0 * H + h) * (int64_t)D;
    TileLoader<BN, D, NT> kl, vl;
    __syncthreads();
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
      const bool active = !CAUSAL || (k0 <= wq0 + 31);
      if (active) {
        const char* Ks = smem[buf][0];
        const char* Vs = smem[buf][1];
        const bool masked = j >= n_bulk;
        uint32_t dsp[2][2][4];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int off = tile_off<D>(kt * 32 + lc, ks * 2 + g);
            sacc = mfma32(lds_read16(Ks, off), qreg[ks], sacc);
            dpacc = mfma32(lds_read16(Vs, off), doreg[ks], dpacc);
          }
          // C layout: lane owns query qi; register i is key
          // k0 + kt*32 + 8*(i/4) + 4g + i%4.
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            float dsv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              float pv = fast_exp2(sacc[i + e] * c2 - lse2);
              if (masked) {
                const int key = k0 + kt * 32 + ((i + e) >> 2) * 8 + g * 4 + ((i + e) & 3);
                const bool ok = key < L && (!CAUSAL || key <= qi);
                pv = ok ? pv : 0.f;
              }
              dsv[e] = pv * (dpacc[i + e] - del);
            }
            dsp[kt][i >> 3][(i & 7) >> 1] = pack_bf16x2(dsv[0], dsv[1]);
          }
        }
        // dQ^T += K^T dS^T; K^T through the transpose read, keys in the
        // order of the dS^T registers.
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int r0 = kt * 32 + hh * 16 + g * 4;
            const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{dsp[kt][hh][0], dsp[kt][hh][1], dsp[kt][hh][2], dsp[kt][hh][3]});
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
              dqa[dt] = mfma32(lds_operand_tr<D>(Ks, r0, r0 + 8, dt * 32), db, dqa[dt]);
          }
      }
      if (j + 1 < n_kv) {
        kl.store(smem[buf ^ 1][0], tid);
        vl.store(smem[buf ^ 1][1], tid);
      }
      __syncthreads();
    }

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
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  const int64_t rows = a.broadcast_q ? (int64_t)a.B * a.H * a.Lq : a.total_len * a.H;
  if (rows > 0) {
    const int64_t work = rows * (D / 8);
    const int64_t want = (work + 255) / 256;
    const int blocks = (int)(want < 4096 ? want : 4096);
    JFA_TIMED_LAUNCH(K_DELTA, st, (delta_kernel<D>), dim3(blocks), dim3(256), 0, st, a.out, a.dout, a.delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.broadcast_q) {
    if (a.causal)
      JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, true, true>), dim3(a.P), dim3(256), 0, st, a);
    else
      JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, false, true>), dim3(a.P), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)a.H * a.Lq * D;
    JFA_TIMED_LAUNCH(K_DQ_REDUCE, st, dq_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.dq_part, a.dq, n,
                       a.P, a.scale);
    return hipGetLastError();
  }
  if (a.causal)
    JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, true, false>), dim3(a.P), dim3(256), 0, st, a);
  else
    JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, false, false>), dim3(a.P), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.causal)
    JFA_TIMED_LAUNCH(K_DQ_SELF, st, (dq_self_kernel<D, true>), dim3(a.P_dq), dim3(256), 0, st, a);
  else
    JFA_TIMED_LAUNCH(K_DQ_SELF, st, (dq_self_kernel<D, false>), dim3(a.P_dq), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.broadcast_q && a.P > MAXP) return hipErrorInvalidValue;
  if (a.d == 64) return launch_bwd_d<64>(a, stream);
  return launch_bwd_d<128>(a, stream);
}

}  // namespace jfa
