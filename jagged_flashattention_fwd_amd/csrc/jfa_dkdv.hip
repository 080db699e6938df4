// dK / dV of jagged flash attention on gfx950, and the exact-delta pre-pass.
//
// dV = P^T dO and dK = scale dS^T Q with P recomputed from the forward's lse
// and dS = P o (dO V^T - delta) ("Optimizing Jagged Flash Attention with TLX",
// "2-CTA collaborative MMA (backward)"; the tiles follow the K/V-outer,
// dense-Q-inner loop of "Scheduling jagged tiles across SMs").
//
// d = 64 runs dkdv_kernel, described here; d = 128 runs dkdv_pair_kernel (its
// own description below), which splits each 32-key group's work between two
// waves of one SIMD.
//
// dkdv_kernel is persistent.  A tile is 128 keys of one (sequence, head); each
// of the 4 waves keeps its 32 keys' K and V rows in registers as MFMA
// operands and accumulates their dK^T / dV^T.  Query blocks of 64 rows (Q, dO
// and each row's terms of -lse / scale and -delta) stream through a ring of 3
// LDS buffers, copied straight
// from global memory (16 bytes per lane, 3 rows per copy) two blocks ahead of
// use; the stream runs on across tile boundaries, and the copies are issued
// from inside the previous block's first products.  The next tile's V rows
// are copied to a per-wave LDS area during the tile's last block; at the
// tile end they are read from there and the next tile's K rows loaded, then
// the dK / dV stores go through a per-wave LDS transpose (the same area)
// into whole 128-byte segments and drain while the next tile computes.  Each
// block is two 32-row subtiles, ordered so that the vector-ALU work of a
// subtile (P and dS) sits
// beside matrix-core work of the other (S and dP of subtile 1, dV and dK of
// subtile 0) in one basic block; with one wave per SIMD that overlap is the
// only latency hiding there is.
//
// The row terms enter as one extra k-step of the S and dP products (three
// bf16 terms times ones, row_terms), so the accumulators hold S - lse / scale
// and dP - delta: P = exp2(c S'), dS = P o dP', with no per-row values held
// in registers or read per element.
//
// Masks are compile-time variants chosen per block: blocks that cross the
// causal diagonal, the key tile at a sequence end and the last (partial)
// query block take the masked body; every other block carries no mask code.
#include <type_traits>

#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

// Two-term bf16 operands: rounding P or dS to bf16 costs up to 2^-9 of each
// value, and dV / dK sum that error over many queries.  Where a subtile holds
// a large value (short or sharply peaked sequences) the rounded remainder
// x - bf16(x) is multiplied in as well.
constexpr float SPLIT_P = 0.25f;
constexpr float SPLIT_DS = 1.0f;

template <int D>
struct Dkdv {
  static constexpr int NW = 4;
  static constexpr int QB = BWD_QB;  // query rows per block (two subtiles)
  static constexpr int BN = BWD_BN;  // keys per tile (32 per wave)
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int RB = TileGeom<D>::ROW_BYTES;
  static constexpr int TILE = QB * RB;
  // d = 128: rows are copied straight from global memory into LDS, three
  // padded rows per copy (PadRowCopy); a wave's 16 rows of a tile take 6.
  static constexpr bool DMA = D == 128;
  static constexpr int NBUF = 3;
  // One ring buffer: Q tile, dO tile, then the 64 rows' terms of -lse / scale
  // and of -delta (16 bytes per row; waves 2 and 3 copy the same rows as waves
  // 0 and 1, which keeps the number of copies equal across waves).  Each tile
  // is followed by the gap that absorbs the overhang of its last row copy.
  static constexpr int GAP = PadRowCopy::GAP;
  static constexpr int OFF_DO = TILE + GAP;
  static constexpr int OFF_TL = OFF_DO + TILE + GAP;
  static constexpr int OFF_TD = OFF_TL + QB * 16;
  static constexpr int BUF = OFF_TD + QB * 16;
  static constexpr int RPW = QB / NW;                  // rows per wave per tile
  static constexpr int CPT = PadRowCopy::copies(RPW);  // copies per wave per tile
  static_assert(!DMA || (RB == 19 * 16 && RPW >= 3), "copy geometry");
  static constexpr int IPS = 2 * CPT + 1;  // copies per wave per block
  static_assert(IPS <= 63, "one block of copies must fit the vector-memory counter");
  static_assert(NBUF * BUF <= 160 * 1024, "LDS");
};

// Issue the transposed reads of DT head-dim operand tiles for the 8 k-slots at
// rows (row0 .. row0+3) and (row0+8 .. row0+11), where `addr` already holds
// this lane's row and column and OFF is the byte offset of row0; the second
// group of rows lies R2 bytes after the first (8 rows unless the tile's rows
// are permuted).  Nothing waits here: tr_wait<N> below makes the values
// available.
template <int OFF, int RB, int R2 = 8 * RB>
__device__ __forceinline__ void tr_issue4(uint32_t addr, i16x4 (&x)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%9\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:%15\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:%16"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
        "=&v"(x[7])
      : "v"(addr), "i"(OFF), "i"(OFF + R2), "i"(OFF + 64), "i"(OFF + R2 + 64), "i"(OFF + 128),
        "i"(OFF + R2 + 128), "i"(OFF + 192), "i"(OFF + R2 + 192));
}
template <int OFF, int RB>
__device__ __forceinline__ void tr_issue2(uint32_t addr, i16x4 (&x)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%5\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %4 offset:%8"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(addr), "i"(OFF), "i"(OFF + 8 * RB), "i"(OFF + 64), "i"(OFF + 8 * RB + 64));
  x[4] = x[5] = x[6] = x[7] = i16x4{0, 0, 0, 0};
}
template <int D, int OFF, int RB, int R2 = 8 * RB>
__device__ __forceinline__ void tr_issue(uint32_t addr, i16x4 (&x)[8]) {
  if constexpr (D == 128) tr_issue4<OFF, RB, R2>(addr, x);
  else tr_issue2<OFF, RB>(addr, x);
}
// Wait until at most N LDS reads of this wave are outstanding; the values in
// x become defined by this statement, so their users are ordered after it.
template <int N>
__device__ __forceinline__ void tr_wait(i16x4 (&x)[8]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7])
               : "i"(N));
}
__device__ __forceinline__ bf16x8 tr_operand(const i16x4 (&x)[8], int dt) {
  struct P { i16x4 a, b; } p = {x[2 * dt], x[2 * dt + 1]};
  return __builtin_bit_cast(bf16x8, p);
}

// Direct global -> LDS copies (global_load_lds_dword: 4 bytes per lane into
// LDS at M0 + 4 * lane), written as asm so that the compiler does not treat
// them as pending writes to every LDS buffer and drain them before each LDS
// read; completion is tracked with wait_vmcnt instead.  Nothing else in these
// kernels uses M0, and each statement sets it before its copy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from a per-lane address.
__device__ __forceinline__ void copy_gather16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0");
}
#pragma clang diagnostic pop



// Operand reads of S = Q K^T and dP = dO V^T for one subtile: for each
// k-step ks the 16-byte chunk (2ks + g) of this lane's query row, of Q and
// of dO, issued in the order q0 d0 q1 d1 ... (`addr` holds this lane's row
// and chunk g; OFF is the subtile's row offset).  With d = 128 the 16 reads
// are two statements; qd_wait<N> then makes pair ks available with N = the
// number of reads issued after it.
template <int OFF, int OFFD>
__device__ __forceinline__ void qd_issue4(uint32_t addr, u32x4* q, u32x4* d) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16"
      : "=&v"(q[0]), "=&v"(d[0]), "=&v"(q[1]), "=&v"(d[1]), "=&v"(q[2]), "=&v"(d[2]), "=&v"(q[3]), "=&v"(d[3])
      : "v"(addr), "i"(OFF), "i"(OFFD), "i"(OFF + 32), "i"(OFFD + 32), "i"(OFF + 64), "i"(OFFD + 64),
        "i"(OFF + 96), "i"(OFFD + 96));
}
template <int N>
__device__ __forceinline__ void lgkm_wait2(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
// The row terms of this lane's query row, of -lse / scale (at OFFL) and of
// -delta (at OFFD), as A operands of the extra k-step (`addr` holds the row's
// 16 * row; both lane halves read the row's 16 bytes, which meet the zero
// half of the ones operand in the upper k-slots).
template <int OFFL, int OFFD>
__device__ __forceinline__ void tm_issue(uint32_t addr, u32x4& tl, u32x4& td) {
  asm volatile("ds_read_b128 %0, %2 offset:%3\n\tds_read_b128 %1, %2 offset:%4"
               : "=&v"(tl), "=&v"(td)
               : "v"(addr), "i"(OFFL), "i"(OFFD));
}

// Residual of a packed bf16 pair: bf16(a - hi.a), bf16(b - hi.b).
__device__ __forceinline__ uint32_t bf16x2_residual(float a, float b, uint32_t hi) {
  return pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}

template <int D, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a, const TileRec* __restrict__ tiles) {
  using C = Dkdv<D>;
  constexpr int QB = C::QB, BN = C::BN, KS = C::KS, DT = C::DT, NBUF = C::NBUF, RB = C::RB;
  constexpr int NT = C::NW * WAVE;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][C::BUF];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_ktiles;
  const int H = a.H, Lq = a.Lq;
  const int64_t ld = (int64_t)H * D;
  const float c2 = a.scale_log2;

  // This lane's part of a transposed read (see lds_operand_tr): row j of the
  // 4-row group, 4 columns at 16 * (G & 1) + 4 q.
  const int trs = l & 15;
  const uint32_t tr_lane = (uint32_t)((g * 4 + (trs >> 2)) * RB + (((((l >> 4) & 1) << 4) + ((trs & 3) << 2)) << 1));

  // Work flows across tile boundaries.  Query blocks form one stream over
  // this workgroup's tiles and are copied two blocks ahead of the compute,
  // into the next tile's first blocks while the current tile finishes.  The
  // next tile's K / V rows are loaded into registers before the current
  // tile's dK / dV are stored, so that the stores drain while the next tile
  // computes.
  const int64_t t0 = zigzag_tile(0, slot, a.P);
  if (t0 >= T) return;

  const int64_t qs = BCAST ? (int64_t)D : ld;          // row stride of Q / dO
  const int64_t sld = BCAST ? 1 : H;                    // row stride of the per-row arrays
  // Per-tile values, with the tile's row-0 addresses of Q, dO and this
  // wave's row terms of -lse / scale (even waves) or -delta (odd waves).
  struct Tp {
    int64_t s0;
    int L, h, hk, b, k0, m_first, m_end, nq;  // hk: the key / value head of query head h
    const uint16_t* qb;
    const uint16_t* db;
    const u32x4* vb;
  };
  auto tparams = [&](const TileRec& r) {
    Tp p;
    p.s0 = r.s0;
    p.L = r.L;
    p.h = r.h;
    p.hk = r.hk;
    p.b = r.b;
    p.k0 = r.blk * BN;
    p.nq = BCAST ? Lq : r.L;
    p.m_first = CAUSAL ? p.k0 / QB : 0;                 // query blocks that can see a key of the tile
    p.m_end = max((p.nq + QB - 1) / QB, p.m_first);     // exclusive
    // Window: rows past k0 + BN - 2 + window see no key of the tile.
    if (CAUSAL && a.window > 0) p.m_end = max(min(p.m_end, (p.k0 + BN - 2 + a.window) / QB + 1), p.m_first);
    p.qb = BCAST ? a.q + (int64_t)r.h * Lq * D : a.q + (r.s0 * H + r.h) * (int64_t)D;
    p.db = BCAST ? a.dout + ((int64_t)r.b * H + r.h) * Lq * D : a.dout + (r.s0 * H + r.h) * (int64_t)D;
    p.vb = reinterpret_cast<const u32x4*>((wave & 1) ? a.term_d : a.term_l) +
           (BCAST ? ((int64_t)r.b * H + r.h) * Lq : r.s0 * H + r.h);
    return p;
  };

  // One query block's copies into a ring buffer.  With d = 128 they are
  // prepared before the block (which block, source rows, buffer) and issued
  // from inside the block's first matrix-core phase (issue_rows / issue_vec),
  // where their scalar address work overlaps the products.  Rows past the
  // last query repeat it: finite values the masked body discards.
  // The prepared job: this wave's first Q / dO source rows of the block, this
  // lane's row terms of -lse / scale (even waves) or -delta (odd waves), the ring
  // buffer's LDS address, rows i > j_last repeat row j_last, and the number
  // of vector-memory operations the job issues (0: none).
  const uint16_t* j_q = a.q;
  const uint16_t* j_d = a.q;
  const u32x4* j_v = reinterpret_cast<const u32x4*>(a.term_l);
  uint32_t j_lds = 0;  // ring buffer
  uint32_t j_ldw = 0;  // this wave's first row in it
  int j_last = 0, j_n = 0;
  // Copies [k0, k1) of this wave's 2 * CPT for the prepared block (Q for
  // k < CPT, dO after), three padded rows each (PadRowCopy).
  const PadRowCopy pc;
  auto issue_rows = [&](int k0, int k1) {
    if constexpr (C::DMA) {
      if (j_n == 0) return;
#pragma unroll
      for (int k = k0; k < k1; ++k) {
        const int R = PadRowCopy::start(k % C::CPT, C::RPW);
        const uint32_t voff = pc.voff(R, j_last, (uint32_t)(qs * 2));
        if (k < C::CPT) dma_copy16(j_q, voff, j_ldw + R * RB);
        else dma_copy16(j_d, voff, j_ldw + C::OFF_DO + R * RB);
      }
    }
  };
  auto issue_vec = [&]() {
    if constexpr (C::DMA) {
      if (j_n == 0) return;
      copy_gather16(j_v, j_lds + C::OFF_TL + (wave & 1) * QB * 16);
    }
  };
  // d = 64: the block is staged through registers right away (the job then
  // issues nothing).
  auto stage_now = [&](const uint16_t* qbase, const uint16_t* dobase, int64_t rbase, int nq, int j, char* buf) {
    const int r0 = j * QB;
    TileLoader<QB, D, NT> ql, dol;
    const int nr = min(QB, nq - r0);
    ql.load(qbase + (int64_t)r0 * qs, qs, nr, tid);
    dol.load(dobase + (int64_t)r0 * qs, qs, nr, tid);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (tid < 2 * QB) {
      const int r = tid & (QB - 1);
      const int64_t ri = rbase + (int64_t)min(r0 + r, nq - 1) * sld;
      v = reinterpret_cast<const u32x4*>(tid < QB ? a.term_l : a.term_d)[ri];
    }
    ql.store(buf, tid);
    dol.store(buf + C::OFF_DO, tid);
    if (tid < 2 * QB) reinterpret_cast<u32x4*>(buf + C::OFF_TL)[tid] = v;
  };

  // Issue state of the block stream.
  int ring_iss = 0, ring_cmp = 0;  // ring buffers of the next issued / computed block
  int iss_cur = 0, iss_nxt = 0;    // blocks of the current / next tile issued so far
  // Prepares the next block of the stream (the current tile's, then the next
  // tile's), if there is one, and advances the stream.
  auto prep_next = [&](const Tp& cp, const Tp& np, bool has_nxt) {
    j_n = 0;
    const int nbc = cp.m_end - cp.m_first;
    const int nbn = has_nxt ? np.m_end - np.m_first : 0;
    const bool cur = iss_cur < nbc;
    if (!cur && iss_nxt >= nbn) return;
    const int nq_ = cur ? cp.nq : np.nq;
    const int j = cur ? cp.m_first + iss_cur : np.m_first + iss_nxt;
    if constexpr (C::DMA) {
      const int base_row = min(j * QB + wave * C::RPW, nq_ - 1);
      // byte offset of the row (a 32 x 32-bit product)
      const uint64_t roff = (uint64_t)(uint32_t)base_row * (uint32_t)(qs * 2);
      j_q = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(cur ? cp.qb : np.qb) + roff);
      j_d = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(cur ? cp.db : np.db) + roff);
      j_v = (cur ? cp.vb : np.vb) + (int64_t)min(j * QB + l, nq_ - 1) * sld;
      j_lds = lds_addr(smem[ring_iss]);
      j_ldw = j_lds + wave * C::RPW * RB;
      j_last = nq_ - 1 - base_row;
      j_n = C::IPS;
    } else {
      const int64_t rbase = BCAST ? ((int64_t)(cur ? cp.b : np.b) * H + (cur ? cp.h : np.h)) * Lq
                                  : (cur ? cp.s0 : np.s0) * H + (cur ? cp.h : np.h);
      stage_now(cur ? cp.qb : np.qb, cur ? cp.db : np.db, rbase, nq_, j, smem[ring_iss]);
    }
    if (cur) ++iss_cur;
    else ++iss_nxt;
    ring_iss = ring_iss == NBUF - 1 ? 0 : ring_iss + 1;
  };
  auto issue_now = [&]() {
    issue_rows(0, 2 * C::CPT);
    issue_vec();
  };

  // Waits until at most n vector-memory operations of this wave are
  // outstanding, for n one of the counts the block stream produces.
  auto wait_n = [&](int n) {
    if constexpr (C::DMA) {
      if (n >= C::IPS) wait_vmcnt<C::IPS>();
      else wait_vmcnt<0>();
    }
  };

  // K and V rows of this lane's key of tile p as B operands (B[d][key] =
  // K[key][d]).  Lanes past the sequence end read its last key (finite
  // values; those keys are masked and never stored).
  u32x4 kraw[KS], vraw[KS];
  auto load_rows = [&](const Tp& p, const uint16_t* base, u32x4 (&x)[KS]) {
    const int kc = min(p.k0 + wave * 32 + lc, p.L - 1);
    const uint16_t* r = base + ((p.s0 + kc) * a.Hkv + p.hk) * (int64_t)D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) x[ks] = *reinterpret_cast<const u32x4*>(r + ks * 16);
  };
  auto load_kv = [&](const Tp& p) {
    load_rows(p, a.k, kraw);
    load_rows(p, a.v, vraw);
  };

  // Per-wave LDS area (8 KB): the next tile's V rows, copied during the
  // tile's last query block, and then the staging of the dK / dV stores.
  // Row r holds key k0 + 32 wave + r; its 16-byte chunk c sits at slot
  // c ^ (r & 15), so that the operand reads (one row per lane, one chunk
  // column per read) are free of bank conflicts.
  __shared__ __attribute__((aligned(16))) char wstage[C::NW][32 * 256];
  constexpr int VDMA = D == 128 ? 8 : 0;  // copies per wave (4 rows each)
  auto issue_v_next = [&](const Tp& p) {
    if constexpr (VDMA > 0) {
      const uint16_t* vb = a.v + ((p.s0 + p.k0) * a.Hkv + p.hk) * (int64_t)D;
      const uint32_t lds0 = lds_addr(wstage[wave]);
      // The lane index through an opaque copy: the offsets below are then
      // computed here, once per tile, rather than hoisted out of the block
      // loop and kept live through every block.
      int lo = l;
      asm volatile("" : "+v"(lo));
      const int rl = lo >> 4, slot = lo & 15;
#pragma unroll
      for (int i = 0; i < VDMA; ++i) {
        const int r = 4 * i + rl;
        const int kr = min(wave * 32 + r, p.L - 1 - p.k0);
        const uint32_t voff = (uint32_t)kr * (uint32_t)(a.Hkv * D * 2) + (uint32_t)(((slot ^ (r & 15))) * 16);
        dma_copy16(vb, voff, lds0 + i * 1024);
      }
    }
  };
  auto read_v_staged = [&]() {
    const char* base = wstage[wave];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      vraw[ks] = *reinterpret_cast<const u32x4*>(base + lc * 256 + (((2 * ks + g) ^ (lc & 15)) * 16));
  };

  // dK = scale * dS^T Q and dV = P^T dO of this lane's keys.  The C layout
  // (lane -> key, registers -> head-dim rows 8*(i/4) + 4g + i%4 of each
  // 32-wide tile) gives 32-byte pieces of 32 rows per register group; each
  // 32 x 32 chunk is transposed through a per-wave LDS area so that every
  // store writes whole 128-byte segments of 8 rows.  Buffer stores bounded to
  // the tile's first nvalid keys: every wave issues exactly 8 * DT of them
  // whatever its keys, and stores past the bound are dropped, so the K / V
  // wait at the next tile start has a fixed count.
  constexpr int SRS = 36;  // staging row stride in floats
  static_assert(32 * SRS * 4 <= 32 * 256, "staging fits the per-wave area");
  auto store_dkdv = [&](const Tp& p, int nvalid, const f32x16 (&dk)[DT], const f32x16 (&dv)[DT]) {
    const int64_t row0 = (p.s0 + p.k0) * H + p.h;
    const int nrec = nvalid * H * D * 4;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.dk + row0 * D, nrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.dv + row0 * D, nrec);
    float* st = reinterpret_cast<float*>(wstage[wave]);
    const int rk8 = l >> 3, rc = (l & 7) * 4;  // read side: key 8r + rk8, columns rc .. rc+3
    auto chunk = [&](const f32x16& acc, float mul, const __amdgpu_buffer_rsrc_t& rs, int dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i4 * 4 + e] * mul;
        *reinterpret_cast<f32x4*>(st + lc * SRS + i4 * 8 + g * 4) = v;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + (r * 8 + rk8) * SRS + rc);
        const int off = ((wave * 32 + r * 8 + rk8) * H * D + dt * 32 + rc) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, 0);
      }
    };
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) chunk(dk[dt], a.scale, rk, dt);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) chunk(dv[dt], 1.0f, rv, dt);
  };

  Tp cp = tparams(tiles[t0]);
  load_kv(cp);
  {
    // Stores that write nothing: the first tile start sees the same
    // operations after its K / V loads as every later one.
    f32x16 z[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) z[dt] = f32x16{};
    store_dkdv(cp, 0, z, z);
  }

  // Tile hand-out.  Causal or self-attention tiles differ in cost: each
  // workgroup takes its first two tiles by the zigzag order and every later
  // one from a global counter over the rest of the list (every dK / dV
  // element is written once by one lane, so the results do not depend on the
  // assignment).  The index for pass p + 2 is fetched at the start of pass p
  // (one lane of wave 0, a vector atomic) and shared through LDS at the
  // tile-start barrier of pass p + 1, where the compiler's wait for it falls
  // behind the wait for everything but the stores.  Non-causal broadcast
  // tiles all cost the same: the static zigzag order alone.
  constexpr bool DYN = CAUSAL || !BCAST;
  __shared__ int s_next;
  unsigned int fetched = 0;
  for (int64_t pass = 0;; ++pass) {
    // The next tile: known here in the static order, at the tile start
    // (handoff) otherwise.
    const int64_t tn0 = zigzag_tile(pass + 1, slot, a.P);
    bool has_nxt = !DYN && tn0 < T;
    Tp np = has_nxt ? tparams(tiles[tn0]) : cp;
    auto handoff = [&]() {
      if constexpr (DYN) {
        const int64_t tn = pass == 0 ? tn0 : 2 * (int64_t)a.P + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
        has_nxt = tn < T;
        if (has_nxt && wave == 0 && l == 0) fetched = atomicAdd(a.ktile_ctr, 1u);
        if (has_nxt) np = tparams(tiles[tn]);
      }
    };
    bool v_staged = false;  // the next tile's V rows are on their way to LDS
    int vm_last = 0;        // copies of the block in progress, issued after them
    const int L = cp.L;
    const int k0 = cp.k0;                 // first key of the tile
    const int kw = k0 + wave * 32 + lc;   // this lane's key
    const bool key_ok = kw < L;
    const int nq = BCAST ? Lq : L;
    const int m_first = cp.m_first, m_end = cp.m_end;
    const int nb = m_end - m_first;
    // Blocks m < m_diag hold a row before the tile's last key.
    const int m_diag = CAUSAL ? (k0 + BN - 1 + QB - 1) / QB : 0;
    const bool tile_partial = k0 + BN > L || a.window > 0;  // a window cuts blocks anywhere
    const int m_full = nq / QB;  // blocks m < m_full have all QB rows

    bf16x8 kreg[KS], vreg[KS];
    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) { dk[dt] = f32x16{}; dv[dt] = f32x16{}; }

    // Lane bases of the LDS reads (the buffer address is added per block).
    const uint32_t qd_lane = (uint32_t)(lc * RB + g * 16);
    const uint32_t tm_lane = (uint32_t)(lc * 16);
    // B operand of the row-term k-step: ones in k-slots 0..2, zeros elsewhere.
    const bf16x8 ones3 = __builtin_bit_cast(bf16x8, g == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});

    // S = Q K^T and dP = dO V^T of subtile S_ from the operand reads q / d
    // (issued by qd_issue; W0 = reads issued after the last pair, so pair ks
    // waits for W0 + 2 (KS - 1 - ks)).  C layout: lane owns key kw; register
    // i is query row S_*32 + 8*(i/4) + 4g + i%4.
    // After each k-step, hook(ks) runs vector work beside it, and a
    // scheduling barrier keeps that order.
    auto mma_scores = [&](auto w_tag, auto lo_tag, auto hi_tag, u32x4* q, u32x4* d, f32x16& sacc, f32x16& dpacc,
                          auto&& hook) {
      constexpr int W0 = decltype(w_tag)::value;
      static_for<decltype(lo_tag)::value, decltype(hi_tag)::value>([&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        lgkm_wait2<W0 + 2 * (KS - 1 - ks)>(q[ks], d[ks]);
        sacc = mfma32(__builtin_bit_cast(bf16x8, q[ks]), kreg[ks], sacc);
        dpacc = mfma32(__builtin_bit_cast(bf16x8, d[ks]), vreg[ks], dpacc);
        hook(ks_tag);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto qd_issue = [&](auto s_tag, uint32_t base, u32x4* q, u32x4* d) {
      constexpr int S_ = decltype(s_tag)::value;
      qd_issue4<S_ * 32 * RB, S_ * 32 * RB + C::OFF_DO>(base, q, d);
      if constexpr (KS == 8) qd_issue4<S_ * 32 * RB + 128, S_ * 32 * RB + C::OFF_DO + 128>(base, q + 4, d + 4);
    };
    auto tm_read = [&](auto s_tag, uint32_t base, u32x4& tl, u32x4& td) {
      constexpr int S_ = decltype(s_tag)::value;
      tm_issue<C::OFF_TL + S_ * 32 * 16, C::OFF_TD + S_ * 32 * 16>(base, tl, td);
    };

    // P and dS of registers 4*i4 .. 4*i4+3 (query rows s*32 + 8*i4 + 4g + e)
    // of subtile s of block m, from its S - lse / scale and dP - delta.
    auto pds = [&](auto masked_tag, int m, int s, const f32x16& sc, const f32x16& dc, int i4, float (&p4)[4],
                   float (&d4)[4]) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const int r = s * 32 + i4 * 8 + g * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i4 * 4 + e;
        float pv = fast_exp2(sc[i] * c2);
        if constexpr (MASKED) {
          const int row = m * QB + r + e;
          bool ok = key_ok && row < nq;
          if constexpr (CAUSAL) ok = ok && kw <= row && (a.window <= 0 || kw > row - a.window);
          pv = ok ? pv : 0.f;
        }
        p4[e] = pv;
        d4[e] = pv * dc[i];
      }
    };

    // P and dS of subtile s as packed bf16 MFMA B operands pp / dsp (pair
    // hh: query rows s*32 + hh*16 + 4g + {0..3, 8..11}); pmax / dsmax
    // collect max |value|.
    auto probs = [&](auto masked_tag, int m, int s, const f32x16& sc, const f32x16& dc, uint32_t (&pp)[2][4],
                     uint32_t (&dsp)[2][4], float& pmax, float& dsmax, int i4) {
      {
        float p4[4], d4[4];
        pds(masked_tag, m, s, sc, dc, i4, p4, d4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pmax = fmaxf(pmax, p4[e]);
          dsmax = fmaxf(dsmax, fabsf(d4[e]));
        }
        pp[i4 >> 1][(i4 & 1) * 2] = pack_bf16x2(p4[0], p4[1]);
        pp[i4 >> 1][(i4 & 1) * 2 + 1] = pack_bf16x2(p4[2], p4[3]);
        dsp[i4 >> 1][(i4 & 1) * 2] = pack_bf16x2(d4[0], d4[1]);
        dsp[i4 >> 1][(i4 & 1) * 2 + 1] = pack_bf16x2(d4[2], d4[3]);
      }
    };

    // dV^T += dO^T P and dK^T += Q^T dS for subtile s: the A operands are
    // transposed reads of the query-major dO / Q tiles at the same query rows
    // as the k-slots of the P / dS register pairs.  Reads: dO(hh0) Q(hh0)
    // dO(hh1) Q(hh1), each group waited with the later ones in flight.
    auto dvdk = [&](auto s_tag, uint32_t tb, const uint32_t (&pp)[2][4], const uint32_t (&dsp)[2][4],
                    auto&& hook) {
      constexpr int s = decltype(s_tag)::value;
      constexpr int OF0 = (s * 32) * RB, OF1 = (s * 32 + 16) * RB;
      constexpr int NR = 2 * DT;  // reads per group
      const bf16x8 p0 = __builtin_bit_cast(bf16x8, u32x4{pp[0][0], pp[0][1], pp[0][2], pp[0][3]});
      const bf16x8 p1 = __builtin_bit_cast(bf16x8, u32x4{pp[1][0], pp[1][1], pp[1][2], pp[1][3]});
      const bf16x8 d0 = __builtin_bit_cast(bf16x8, u32x4{dsp[0][0], dsp[0][1], dsp[0][2], dsp[0][3]});
      const bf16x8 d1 = __builtin_bit_cast(bf16x8, u32x4{dsp[1][0], dsp[1][1], dsp[1][2], dsp[1][3]});
      i16x4 xo0[8], xq0[8], xo1[8], xq1[8];
      tr_issue<D, OF0 + C::OFF_DO, RB>(tb, xo0);
      tr_issue<D, OF0, RB>(tb, xq0);
      tr_wait<NR>(xo0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dv[dt] = mfma32(tr_operand(xo0, dt), p0, dv[dt]);
      hook(std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
      tr_issue<D, OF1 + C::OFF_DO, RB>(tb, xo1);
      tr_wait<NR>(xq0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dk[dt] = mfma32(tr_operand(xq0, dt), d0, dk[dt]);
      hook(std::integral_constant<int, 1>{});
      __builtin_amdgcn_sched_barrier(0);
      tr_issue<D, OF1, RB>(tb, xq1);
      tr_wait<NR>(xo1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dv[dt] = mfma32(tr_operand(xo1, dt), p1, dv[dt]);
      hook(std::integral_constant<int, 2>{});
      __builtin_amdgcn_sched_barrier(0);
      tr_wait<0>(xq1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dk[dt] = mfma32(tr_operand(xq1, dt), d1, dk[dt]);
      hook(std::integral_constant<int, 3>{});
      __builtin_amdgcn_sched_barrier(0);
    };

    // Remainder products of subtile s where a P (dV) or dS (dK) value is
    // large: P / dS are recomputed from S / dP and their residuals against
    // the packed operands multiplied in.
    auto fixup = [&](auto masked_tag, auto s_tag, int m, const char* buf, const f32x16& sc, const f32x16& dc,
                     const uint32_t (&pp)[2][4], const uint32_t (&dsp)[2][4], bool fix_p, bool fix_ds) {
      constexpr int s = decltype(s_tag)::value;
      // Opaque copies: the values below are recomputed here rather than
      // kept alive from the main path through the whole block.
      f32x16 sc2 = sc, dc2 = dc;
      asm volatile("" : "+v"(sc2), "+v"(dc2));
      const uint32_t tb = lds_addr(buf) + tr_lane;
      auto half = [&](auto hh_tag) {
        constexpr int hh = decltype(hh_tag)::value;
        u32x4 plo, dlo;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i4 = 2 * hh + k;
          float p4[4], d4[4];
          pds(masked_tag, m, s, sc2, dc2, i4, p4, d4);
          plo[2 * k] = bf16x2_residual(p4[0], p4[1], pp[hh][2 * k]);
          plo[2 * k + 1] = bf16x2_residual(p4[2], p4[3], pp[hh][2 * k + 1]);
          dlo[2 * k] = bf16x2_residual(d4[0], d4[1], dsp[hh][2 * k]);
          dlo[2 * k + 1] = bf16x2_residual(d4[2], d4[3], dsp[hh][2 * k + 1]);
        }
        if (fix_p) {
          i16x4 xo[8];
          tr_issue<D, (s * 32 + hh * 16) * RB + C::OFF_DO, RB>(tb, xo);
          tr_wait<0>(xo);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) dv[dt] = mfma32(tr_operand(xo, dt), __builtin_bit_cast(bf16x8, plo), dv[dt]);
        }
        if (fix_ds) {
          i16x4 xq[8];
          tr_issue<D, (s * 32 + hh * 16) * RB, RB>(tb, xq);
          tr_wait<0>(xq);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) dk[dt] = mfma32(tr_operand(xq, dt), __builtin_bit_cast(bf16x8, dlo), dk[dt]);
        }
      };
      half(std::integral_constant<int, 0>{});
      half(std::integral_constant<int, 1>{});
    };

    // One query block, every LDS read issued explicitly so that its latency
    // overlaps other work:
    //   1. Row terms(0), Q/dO(0) reads; S0, dP0 from the row-term k-step.
    //   2. Row terms(1), Q/dO(1) reads; P0, dS0 (vector ALU) beside S1, dP1.
    //   3. dV/dK of subtile 0 beside P1, dS1.
    //   4. dV/dK of subtile 1.
    auto block = [&](auto masked_tag, int m, const char* buf) {
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using W0 = std::integral_constant<int, 0>;
      using K0 = std::integral_constant<int, 0>;
      using KE = std::integral_constant<int, KS>;
      const uint32_t lb = lds_addr(buf);
      const uint32_t qb = lb + qd_lane, tmb = lb + tm_lane, tb = lb + tr_lane;
      uint32_t pa[2][4], dsa[2][4], pb[2][4], dsb[2][4];
      u32x4 q[KS], d[KS], tl, td;
      auto none = [](auto) {};
      // S / dP accumulators start from the row-term k-step (its reads issued
      // first and waited for with up to 15 operand reads after them in flight;
      // the counter holds no more).
      tm_read(S0{}, tmb, tl, td);
      qd_issue(S0{}, qb, q, d);
      lgkm_wait2<(2 * KS > 15 ? 15 : 2 * KS)>(tl, td);
      f32x16 sa = mfma32(__builtin_bit_cast(bf16x8, tl), ones3, f32x16{});
      f32x16 da = mfma32(__builtin_bit_cast(bf16x8, td), ones3, f32x16{});
      // The next block's copies, spread over the k-steps.
      auto copy_hook = [&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        constexpr int PER = (2 * C::CPT + KS - 1) / KS;
        issue_rows(ks * PER, min((ks + 1) * PER, 2 * C::CPT));
        if constexpr (ks == KS - 1) issue_vec();
      };
      mma_scores(W0{}, K0{}, KE{}, q, d, sa, da, copy_hook);

      // P0 / dS0 in four row groups, one after every KS/4 k-steps of S1 / dP1.
      tm_read(S1{}, tmb, tl, td);
      qd_issue(S1{}, qb, q, d);
      lgkm_wait2<(2 * KS > 15 ? 15 : 2 * KS)>(tl, td);
      f32x16 sb = mfma32(__builtin_bit_cast(bf16x8, tl), ones3, f32x16{});
      f32x16 db = mfma32(__builtin_bit_cast(bf16x8, td), ones3, f32x16{});
      float pmax = 0.f, dsmax = 0.f;
      auto p0_hook = [&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        if constexpr (ks % (KS / 4) == KS / 4 - 1) probs(masked_tag, m, 0, sa, da, pa, dsa, pmax, dsmax, ks / (KS / 4));
      };
      mma_scores(W0{}, K0{}, KE{}, q, d, sb, db, p0_hook);

      // P1 / dS1 beside dV / dK of subtile 0.
      float pmax1 = 0.f, dsmax1 = 0.f;
      auto p1_hook = [&](auto g_tag) {
        probs(masked_tag, m, 1, sb, db, pb, dsb, pmax1, dsmax1, decltype(g_tag)::value);
      };
      dvdk(S0{}, tb, pa, dsa, p1_hook);
      dvdk(S1{}, tb, pb, dsb, none);
      const bool f0p = pmax > SPLIT_P, f0d = dsmax > SPLIT_DS;
      const bool f1p = pmax1 > SPLIT_P, f1d = dsmax1 > SPLIT_DS;
      if (__builtin_expect(__any(f0p || f0d || f1p || f1d), 0)) {
        fixup(masked_tag, S0{}, m, buf, sa, da, pa, dsa, __any(f0p), __any(f0d));
        fixup(masked_tag, S1{}, m, buf, sb, db, pb, dsb, __any(f1p), __any(f1d));
      }
    };

    // The K / V registers are consumed here, on every path and outside the
    // loops, so that the compiler's own wait for those loads (it sees the 8 *
    // DT stores after them) happens once per tile.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      asm volatile("" : "+v"(kraw[ks]), "+v"(vraw[ks]));
      kreg[ks] = __builtin_bit_cast(bf16x8, kraw[ks]);
      vreg[ks] = __builtin_bit_cast(bf16x8, vraw[ks]);
    }
    if (nb > 0) {
      // Tile start.  Normally the first two blocks were issued during the
      // previous tile, before its K / V loads for this tile, and only the
      // previous tile's 8 * DT stores may be outstanding after those.
      {
        const int need = min(nb, 2);
        if (iss_cur < need) {
          while (iss_cur < need) {
            prep_next(cp, cp, false);  // this tile's blocks only
            issue_now();
          }
          wait_vmcnt<0>();
        } else {
          static_assert(8 * DT <= 63, "store count");
          wait_vmcnt<8 * DT>();
        }
        if (DYN && pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
        barrier_lds();  // the block's copies landed for every wave; the previous block's readers are done
        handoff();
      }
      // Blocks [m0, m1) with one body (a loop per mask variant, rather than
      // a branch per block, keeps register allocation to one body at a time).
      // Block m + 2 goes to the ring buffer block m - 1 used, which every
      // wave has left once block m's barrier returns.
      auto run = [&](auto masked_tag, int m0, int m1) {
        for (int m = m0; m < m1; ++m) {
          if (m != m_first) {
            wait_n(vm_last);
            barrier_lds();
          }
          prep_next(cp, np, has_nxt);
          vm_last = j_n;
          // The tile's last block copies the next tile's V rows first (the
          // tile end waits for them with this block's own copies in flight).
          if constexpr (VDMA > 0) {
            if (m == m_end - 1 && has_nxt) {
              issue_v_next(np);
              v_staged = true;
            }
          }
          block(masked_tag, m, smem[ring_cmp]);
          ring_cmp = ring_cmp == NBUF - 1 ? 0 : ring_cmp + 1;
        }
      };
      if (tile_partial) {
        run(std::true_type{}, m_first, m_end);
      } else {
        // masked: causal diagonal blocks, then the partial last block
        const int u0 = CAUSAL ? min(max(m_diag, m_first), m_end) : m_first;
        const int u1 = max(u0, min(m_full, m_end));
        run(std::true_type{}, m_first, u0);
        run(std::false_type{}, u0, u1);
        run(std::true_type{}, u1, m_end);
      }
    } else {
      // A tile with no query block (causal broadcast keys past the queries).
      if (DYN && pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
      if (DYN) barrier_lds();
      handoff();
    }

    // Tile end: the next tile's K / V loads, then this tile's stores.
    if (has_nxt) {
      if (v_staged) {
        wait_n(vm_last);
        asm volatile("" ::: "memory");  // the reads below stay after the wait
        read_v_staged();
      } else {
        load_rows(np, a.v, vraw);
      }
      load_rows(np, a.k, kraw);
    }
    store_dkdv(cp, min(L - k0, BN), dk, dv);
    if (!has_nxt) break;
    cp = np;
    iss_cur = iss_nxt;
    iss_nxt = 0;
  }
}

// ============================================== dK / dV, d = 128, 8 waves --
// The same tiles, block stream and results as dkdv_kernel, with the work of
// each 32-key group split between two waves so that two waves share every
// SIMD and one's vector work runs beside the other's matrix products:
//   score wave (waves 0-3):    K rows of its keys; S = Q K^T (+ the -lse /
//                              scale row terms), P = exp2(c S'), masked;
//                              P to LDS; dV += P^T dO.
//   gradient wave (waves 4-7): V rows of the same keys; dP = dO V^T (+ the
//                              -delta row terms); after P arrives,
//                              dS = P o dP', dK += dS^T Q.
// P passes lane to lane (both waves own the same key per lane and the same
// query rows per register), through a 32 KB area.  Each wave holds one
// operand set (K or V) and one fp32 accumulator (dV or dK, key by d, so that
// its stores write whole 128-byte rows straight from the registers), half of
// dkdv_kernel's, so that it fits in the 256 registers of a wave sharing its
// SIMD.  The iterations are software-pipelined (the back of one block beside
// the front of the next) in one stream across tiles: between two tiles a
// transition runs the back of one tile's last block beside the front of the
// next tile's first, and the finished tile's stores drain during the next
// iteration.
struct Pair {
  static constexpr int NW = 8, NG = 4;  // waves; key groups of 32 keys (one score + one gradient wave each)
  static constexpr int QB = BWD_QB, BN = BWD_BN, D = 128, KS = 8, DT = 4;
  static constexpr int RB = TileGeom<128>::ROW_BYTES;
  static constexpr int TILE = QB * RB;
  static constexpr int NBUF = 3;
  static constexpr int GAP = PadRowCopy::GAP;
  static constexpr int OFF_DO = TILE + GAP;
  static constexpr int OFF_TL = OFF_DO + TILE + GAP;
  static constexpr int OFF_TD = OFF_TL + QB * 16;
  static constexpr int BUF = OFF_TD + QB * 16;
  static constexpr int RPW = QB / NW;                  // rows per wave per tile
  static constexpr int CPT = PadRowCopy::copies(RPW);  // copies per wave per tile
  static constexpr int IPS = 2 * CPT + 1;              // copies per wave per block
  // P hand-over as fp16, two areas (consecutive iterations): [area]
  // [subtile][key group][register group][lane] x 8 bytes.
  static constexpr int XBYTES = 2 * 2 * NG * 4 * WAVE * 8;
  static_assert(RB == 19 * 16 && RPW >= 3, "copy geometry");
  static_assert(NBUF * BUF + XBYTES + 64 <= 160 * 1024, "LDS");
  // Q / dO tiles are read both ways: 16-byte reads of 16 consecutive query
  // rows (S = Q K^T, dP = dO V^T) and transposing reads of 4 consecutive
  // rows x 64 bytes per 32 lanes (dV += P^T dO, dK += dS^T Q).  Query
  // row r of a tile sits at row position perm(r): within each group of 16
  // rows the 4 x 4 transpose (r = 4 m + i at 4 i + m).  Any 16 consecutive
  // rows then still take 16 distinct positions modulo 16, and 4 consecutive
  // rows 4 m .. 4 m + 3 take positions m, m + 4, m + 8, m + 12, whose 64-byte
  // windows of a 304-byte row are 64 bytes apart modulo the 256 bytes of
  // the LDS banks: both reads are free of bank conflicts.  perm is its own
  // inverse.
  __host__ __device__ static constexpr int perm(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }
};

// Eight 16-byte LDS reads at OFF + 32 ks (k-step ks of a 128-wide row, the
// lane's chunk already in `addr`), not waited for.
template <int OFF>
__device__ __forceinline__ void rows_issue8(uint32_t addr, u32x4 (&x)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%9\n\t"
      "ds_read_b128 %1, %8 offset:%10\n\t"
      "ds_read_b128 %2, %8 offset:%11\n\t"
      "ds_read_b128 %3, %8 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %8 offset:%14\n\t"
      "ds_read_b128 %6, %8 offset:%15\n\t"
      "ds_read_b128 %7, %8 offset:%16"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(addr), "i"(OFF), "i"(OFF + 32), "i"(OFF + 64), "i"(OFF + 96), "i"(OFF + 128), "i"(OFF + 160),
        "i"(OFF + 192), "i"(OFF + 224));
}
// One 16-byte LDS read at byte offset OFF from `addr`, not waited for.
template <int OFF>
__device__ __forceinline__ void lds_read16_issue(uint32_t addr, u32x4& x) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(x) : "v"(addr), "i"(OFF));
}
template <int N>
__device__ __forceinline__ void lgkm_wait1(u32x4& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

template <bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(512, 1) void dkdv_pair_kernel(BwdArgs a, const TileRec* __restrict__ tiles) {
  using C = Pair;
  constexpr int QB = C::QB, BN = C::BN, KS = C::KS, DT = C::DT, NBUF = C::NBUF, RB = C::RB, D = C::D;
  __shared__ __attribute__((aligned(16))) char smem[NBUF][C::BUF];
  __shared__ __attribute__((aligned(16))) char xchg[C::XBYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int kgrp = wave & (C::NG - 1);  // key group: keys 32 kgrp .. 32 kgrp + 31 of the tile
  const bool grad = wave >= C::NG;      // gradient wave (V, dP, dS, dK); else score wave (K, S, P, dV)
  const int l = tid % WAVE, g = l / 32, lc = l % 32;
  const int slot = logical_slot(blockIdx.x, a.P);
  const int64_t T = *a.n_ktiles;
  const int H = a.H, Lq = a.Lq;
  const int64_t ld = (int64_t)H * D;
  const float c2 = a.scale_log2;

  // This lane's part of a transposed read (see lds_operand_tr): row g * 4 +
  // (trs >> 2) of a group of 16 sits at position C::perm of it, and the
  // rows 8 further at 2 positions further.
  const int trs = l & 15;
  const uint32_t tr_lane =
      (uint32_t)(C::perm(g * 4 + (trs >> 2)) * RB + (((((l >> 4) & 1) << 4) + ((trs & 3) << 2)) << 1));
  constexpr int TR2 = 2 * RB;

  const int64_t t0 = zigzag_tile(0, slot, a.P);
  if (t0 >= T) return;

  const int64_t qs = BCAST ? (int64_t)D : ld;  // row stride of Q / dO
  const int64_t sld = BCAST ? 1 : H;           // row stride of the per-row arrays
  // A tile: 128 keys of one sequence and key / value head hk, against the
  // query blocks m_first .. m_end - 1 of each of its ng query heads h ..
  // h + ng - 1 (ng = G with grouped heads, one dK / dV accumulator for the
  // group); its block stream is head-major, nb = ng * nbh blocks.
  struct Tp {
    int64_t s0;
    int L, h, hk, b, k0, m_first, m_end, nq, nbh, nb;
    const uint16_t* qb;  // Q, dO, row terms of the first query head
    const uint16_t* db;
    const u32x4* vb;
  };
  const int ng = a.G;
  const int64_t hs_qd = BCAST ? (int64_t)Lq * D : (int64_t)D;  // Q / dO: next query head
  const int64_t hs_row = BCAST ? (int64_t)Lq : 1;              // row terms: next query head
  auto tparams = [&](const TileRec& r) {
    Tp p;
    p.s0 = r.s0;
    p.L = r.L;
    p.h = r.h;
    p.hk = r.hk;
    p.b = r.b;
    p.k0 = r.blk * BN;
    p.nq = BCAST ? Lq : r.L;
    p.m_first = CAUSAL ? p.k0 / QB : 0;
    p.m_end = max((p.nq + QB - 1) / QB, p.m_first);
    if (CAUSAL && a.window > 0) p.m_end = max(min(p.m_end, (p.k0 + BN - 2 + a.window) / QB + 1), p.m_first);
    p.nbh = p.m_end - p.m_first;
    p.nb = ng * p.nbh;
    p.qb = BCAST ? a.q + (int64_t)r.h * Lq * D : a.q + (r.s0 * H + r.h) * (int64_t)D;
    p.db = BCAST ? a.dout + ((int64_t)r.b * H + r.h) * Lq * D : a.dout + (r.s0 * H + r.h) * (int64_t)D;
    p.vb = reinterpret_cast<const u32x4*>((wave & 1) ? a.term_d : a.term_l) +
           (BCAST ? ((int64_t)r.b * H + r.h) * Lq : r.s0 * H + r.h);
    return p;
  };

  // The block stream, as in dkdv_kernel: each wave fills its 8 row
  // positions of the Q and dO tiles (three padded rows per copy) and copies
  // one row-term array (even waves -lse / scale, odd waves -delta) of the
  // block two ahead.  The copies read through buffer resources over the
  // block's rows that exist (rows past the last query read as zeros); the
  // source row of each position (C::perm) is fixed per lane and copy.
  __amdgpu_buffer_rsrc_t j_rq = make_rsrc(a.q, 0), j_rd = make_rsrc(a.q, 0);
  const u32x4* j_v = reinterpret_cast<const u32x4*>(a.term_l);
  uint32_t j_lds = 0, j_ldw = 0;
  int j_n = 0;
  const uint32_t rstride = (uint32_t)(qs * 2);
  uint32_t cvoff[C::CPT];
#pragma unroll
  for (int k = 0; k < C::CPT; ++k)
    cvoff[k] = (uint32_t)C::perm(wave * C::RPW + PadRowCopy::start(k, C::RPW) + (int)PadRowCopy::lane_row(l)) * rstride +
               PadRowCopy::lane_byte(l);
  auto issue_rows = [&](int k0, int k1) {
    if (j_n == 0) return;
#pragma unroll
    for (int k = k0; k < k1; ++k) {
      const int R = PadRowCopy::start(k % C::CPT, C::RPW);
      if (k < C::CPT) dma_copy16_buf(j_rq, cvoff[k % C::CPT], 0, j_ldw + R * RB);
      else dma_copy16_buf(j_rd, cvoff[k % C::CPT], 0, j_ldw + C::OFF_DO + R * RB);
    }
  };
  auto issue_vec = [&]() {
    if (j_n == 0) return;
    copy_gather16(j_v, j_lds + C::OFF_TL + (wave & 1) * QB * 16);
  };
  int ring_iss = 0, ring_cmp = 0;
  int iss_cur = 0, iss_nxt = 0;
  // position of the current tile's next block to issue: query head gi
  // (0 .. ng-1), block j - m_first (0 .. nbh-1).  The stream runs at most
  // one block ahead, so of the next tile only its first block (head 0,
  // block m_first) is ever issued early.
  int cur_gi = 0, cur_jb = 0;
  auto prep_next = [&](const Tp& cp, const Tp& np, bool has_nxt) {
    j_n = 0;
    const int nbn = has_nxt ? np.nb : 0;
    const bool cur = iss_cur < cp.nb;
    if (!cur && iss_nxt >= min(nbn, 1)) return;
    // the block: query head gi, block j of the current tile, or the next
    // tile's first block
    const int gi = cur ? cur_gi : 0;
    const int j = cur ? cp.m_first + cur_jb : np.m_first;
    const int nq_ = cur ? cp.nq : np.nq;
    // the block's rows that exist, up to the one past it (the last copy's
    // overhang)
    const int rows = max(0, min(nq_ - j * QB, QB + 1));
    const uint64_t roff = (uint64_t)(uint32_t)(j * QB) * rstride;
    j_rq = make_rsrc(reinterpret_cast<const char*>((cur ? cp.qb : np.qb) + gi * hs_qd) + roff, rows * (int)rstride);
    j_rd = make_rsrc(reinterpret_cast<const char*>((cur ? cp.db : np.db) + gi * hs_qd) + roff, rows * (int)rstride);
    j_v = (cur ? cp.vb : np.vb) + gi * hs_row + (int64_t)min(j * QB + l, nq_ - 1) * sld;
    j_lds = lds_addr(smem[ring_iss]);
    j_ldw = j_lds + wave * C::RPW * RB;
    j_n = C::IPS;
    // (value selects, not a branch over which counter to bump: the latter
    // becomes an increment through a selected address, which puts the
    // counters in scratch memory)
    const int c1 = cur ? 1 : 0;
    const int jb1 = cur_jb + c1;
    const bool wrap = jb1 == cp.nbh;
    iss_cur += c1;
    iss_nxt += 1 - c1;
    cur_jb = wrap ? 0 : jb1;
    cur_gi += wrap ? 1 : 0;
    ring_iss = ring_iss == NBUF - 1 ? 0 : ring_iss + 1;
  };
  auto issue_now = [&]() {
    issue_rows(0, 2 * C::CPT);
    issue_vec();
  };
  auto wait_n = [&](int n) {
    if (n >= C::IPS) wait_vmcnt<C::IPS>();
    else wait_vmcnt<0>();
  };

  // This wave's operand rows (K for a score wave, V for a gradient wave) of
  // its key, as B operands; lanes past the sequence end read its last key.
  u32x4 kvraw[KS];
  auto load_rows = [&](const Tp& p) {
    const int kc = min(p.k0 + kgrp * 32 + lc, p.L - 1);
    const uint16_t* r = (grad ? a.v : a.k) + ((p.s0 + kc) * a.Hkv + p.hk) * (int64_t)D + g * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kvraw[ks] = *reinterpret_cast<const u32x4*>(r + ks * 16);
  };

  // dV (score wave) or scale * dK (gradient wave) of this wave's keys.  The
  // accumulators hold them key by d: register 4 i4 + e of head-dim tile dt
  // is key 8 i4 + 4 g + e of the wave's 32 at d = 32 dt + lc, so each
  // 4-byte store writes two whole 128-byte runs (lanes 0-31 one key, lanes
  // 32-63 the key 4 further); bounded buffer stores (keys past the sequence
  // end are dropped), 16 * DT per wave.  A store's byte offset is this
  // lane's part (key kgrp * 32 + 4 g, d = lc) plus the register's, added per
  // store, so that the whole offset stays in the lane operand, which the
  // range check covers; st_base hides the lane part from loop-invariant
  // hoisting, which would keep all the sums live.
  const uint32_t st_lane = (uint32_t)(((kgrp * 32 + 4 * g) * a.Hkv * D + lc) * 4);
  auto st_base = [&]() {
    uint32_t b = st_lane;
    asm volatile("" : "+v"(b));
    return b;
  };
  auto store_acc = [&](const Tp& p, int nvalid, const f32x16 (&acc)[DT]) {
    const int64_t row0 = (p.s0 + p.k0) * a.Hkv + p.hk;  // dK / dV are [total_len, H_kv, d]
    const int nrec = nvalid * a.Hkv * D * 4;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((grad ? a.dk : a.dv) + row0 * D, nrec);
    const float mul = grad ? a.scale : 1.0f;
    const uint32_t sb = st_base();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[dt][i4 * 4 + e] * mul), rs,
                                                sb + (uint32_t)(((8 * i4 + e) * a.Hkv * D + dt * 32) * 4), 0, 0);
  };
  // Zero dV / dK for a tile without query blocks: 16-byte stores of whole
  // 128-byte runs (lane l: key l / 8 of each group of 8, chunk l % 8).
  auto store_zero = [&](const Tp& p, int nvalid) {
    const int64_t row0 = (p.s0 + p.k0) * a.Hkv + p.hk;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((grad ? a.dk : a.dv) + row0 * D, nvalid * a.Hkv * D * 4);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, rs,
                                               (uint32_t)(((kgrp * 32 + r * 8 + (l >> 3)) * a.Hkv * D + dt * 32 + (l & 7) * 4) * 4), 0, 0);
  };

  Tp cp = tparams(tiles[t0]);

  constexpr bool DYN = CAUSAL || !BCAST;
  __shared__ int s_next;
  unsigned int fetched = 0;
  // The tile after the current one, known from the current tile's start.
  Tp np = cp;
  bool has_nxt = false;
  // At the start barrier of the tile of pass p: its successor (static
  // zigzag, or past the first two passes the hand-out counter, whose next
  // value one lane fetches now and passes on at the next tile start).
  auto start_duties = [&](int64_t p) {
    const int64_t tn0 = zigzag_tile(p + 1, slot, a.P);
    if constexpr (DYN) {
      const int64_t tn = p == 0 ? tn0 : 2 * (int64_t)a.P + (uint32_t)__builtin_amdgcn_readfirstlane(s_next);
      has_nxt = tn < T;
      if (has_nxt && wave == 0 && l == 0) fetched = atomicAdd(a.ktile_ctr, 1u);
      if (has_nxt) np = tparams(tiles[tn]);
    } else {
      has_nxt = tn0 < T;
      if (has_nxt) np = tparams(tiles[tn0]);
    }
  };

  // A tile's lane and loop values: this lane's key, the query rows, and per
  // query head the blocks [0, u0) and [u1, nbh) that take the masked front.
  struct Tv {
    int kw, nq, nb, nbh, m_first, u0, u1;
    bool key_ok;
  };
  auto tvals = [&](const Tp& p) {
    Tv v;
    v.kw = p.k0 + kgrp * 32 + lc;
    v.key_ok = v.kw < p.L;
    v.nq = p.nq;
    v.nb = p.nb;
    v.nbh = p.nbh;
    v.m_first = p.m_first;
    const int m_diag = CAUSAL ? (p.k0 + BN - 1 + QB - 1) / QB : 0;
    const bool tile_partial = p.k0 + BN > p.L || a.window > 0;
    const int m_full = p.nq / QB;
    v.u0 = tile_partial ? p.nbh : CAUSAL ? min(max(m_diag, p.m_first), p.m_end) - p.m_first : 0;
    v.u1 = tile_partial ? p.nbh : max(v.u0, min(m_full, p.m_end) - p.m_first);
    return v;
  };

  bf16x8 kv[KS];
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // B operand of the row-term k-step: ones in k-slots 0..2.
  const bf16x8 ones3 = __builtin_bit_cast(bf16x8, g == 0 ? u32x4{0x3F803F80u, 0x3F80u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u});
  // Lane bases: this lane's query row and chunk g of the role's row tile,
  // its row term, and its 16-byte slots of the hand-over area.
  const uint32_t row_lane = (uint32_t)(C::perm(lc) * RB + g * 16) + (grad ? (uint32_t)C::OFF_DO : 0u);
  const uint32_t tm_lane = (uint32_t)(lc * 16) + (grad ? (uint32_t)C::OFF_TD : (uint32_t)C::OFF_TL);
  u32x2* const xw = reinterpret_cast<u32x2*>(xchg) + (kgrp * 4) * WAVE + l;  // + ((xs * 2 + s) * NG * 4 + i4) * WAVE

  // Carried from one iteration to the next, in one register array for
  // both roles: the score wave's P of the block just scored as packed
  // bf16 B operands (carry[8 s + 4 hh + k], subtile s, pair hh) and their
  // rounded remainders (carry[16 + ...]), plus the largest value per
  // subtile; the gradient wave's dP' of that block (carry[16 s + i] as
  // fp32 bits).
  uint32_t carry[32];
  float pmaxc[2] = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 32; ++i) carry[i] = 0u;

  // Front of an iteration: S (score wave) or dP (gradient wave) of block
  // m, each subtile from its row-term k-step and KS k-steps of LDS rows
  // (three reads ahead) against the registers.  The score wave turns S
  // into P, writes it to hand-over area xs for the gradient wave and keeps
  // it packed; the gradient wave keeps dP'.
  auto front = [&](auto masked_tag, const Tv& tv, int m, const char* buf, int xs) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const uint32_t lb = lds_addr(buf);
    f32x16 sc[2];
    // score wave: P of register group I4 of subtile S_ (rows S_ * 32 + 8 I4 + 4 g + e)
    auto p_rows = [&](auto s_tag, auto i4_tag) __attribute__((always_inline)) {
      constexpr int S_ = decltype(s_tag)::value, I4 = decltype(i4_tag)::value;
      const int r = S_ * 32 + I4 * 8 + g * 4;
      float p4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = fast_exp2(sc[S_][I4 * 4 + e] * c2);
        if constexpr (MASKED) {
          const int row = m * QB + r + e;
          bool ok = tv.key_ok && row < tv.nq;
          if constexpr (CAUSAL) ok = ok && tv.kw <= row && (a.window <= 0 || tv.kw > row - a.window);
          pv = ok ? pv : 0.f;
        }
        p4[e] = pv;
        pmaxc[S_] = fmaxf(pmaxc[S_], pv);
      }
      xw[((xs * 2 + S_) * C::NG * 4 + I4) * WAVE] = u32x2{pack_f16x2(p4[0], p4[1]), pack_f16x2(p4[2], p4[3])};
      const uint32_t h0 = pack_bf16x2(p4[0], p4[1]), h1 = pack_bf16x2(p4[2], p4[3]);
      constexpr int c = 8 * S_ + 4 * (I4 >> 1) + (I4 & 1) * 2;
      carry[c] = h0;
      carry[c + 1] = h1;
      carry[16 + c] = bf16x2_residual(p4[0], p4[1], h0);
      carry[16 + c + 1] = bf16x2_residual(p4[2], p4[3], h1);
    };
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    if (!grad) pmaxc[0] = pmaxc[1] = 0.f;
    static_for<0, 2>([&](auto s_tag) {
      constexpr int s = decltype(s_tag)::value;
      constexpr int LA = 3;  // row reads in flight ahead of the products
      u32x4 rw[KS], tmv;
      const uint32_t rb = lb + row_lane;
      lds_read16_issue<s * 32 * 16>(lb + tm_lane, tmv);
      static_for<0, LA>([&](auto k_tag) {
        constexpr int k = decltype(k_tag)::value;
        lds_read16_issue<s * 32 * RB + 32 * k>(rb, rw[k]);
      });
      lgkm_wait1<LA>(tmv);
      sc[s] = mfma32(__builtin_bit_cast(bf16x8, tmv), ones3, f32x16{});
      static_for<0, KS>([&](auto ks_tag) {
        constexpr int ks = decltype(ks_tag)::value;
        // reads issued after this k-step's: ks + 1 .. ks + LA - 1 (and any
        // hand-over writes, which only make the wait conservative)
        lgkm_wait1<(KS - 1 - ks < LA - 1 ? KS - 1 - ks : LA - 1)>(rw[ks]);
        if constexpr (ks + LA < KS) lds_read16_issue<s * 32 * RB + 32 * (ks + LA)>(rb, rw[ks + LA]);
        sc[s] = mfma32(__builtin_bit_cast(bf16x8, rw[ks]), kv[ks], sc[s]);
        if constexpr (s == 1 && (ks & 1)) {
          // score wave: P of subtile 0 beside subtile 1's products
          if (!grad) p_rows(Z{}, std::integral_constant<int, (ks >> 1)>{});
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
    if (!grad) {
      static_for<0, 4>([&](auto i4_tag) { p_rows(O{}, i4_tag); });
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        carry[i] = __float_as_uint(sc[0][i]);
        carry[16 + i] = __float_as_uint(sc[1][i]);
      }
    }
  };

  // Back of an iteration: dV += P^T dO (score wave) or dK += dS^T Q
  // (gradient wave, dS = P o dP' with P from hand-over area xs) of the
  // block before, one instruction stream for both: the packed P or dS (its
  // registers read as the A operand give P^T / dS^T, a key per row) times
  // transposed reads of the dO or Q tile at the query rows of its k-slots
  // (pair hh: rows s * 32 + 16 hh + 4 g + {0..3, 8..11}) as the B operand,
  // so that the accumulator holds key rows by d columns.  Where a subtile
  // holds a value above its threshold the rounded remainders are multiplied
  // in as well.
  auto back = [&](const char* buf, int xs) __attribute__((always_inline)) {
    const uint32_t tbr = lds_addr(buf) + tr_lane + (grad ? 0u : (uint32_t)C::OFF_DO);
    static_for<0, 2>([&](auto s_tag) {
      constexpr int s = decltype(s_tag)::value;
      constexpr int OF0 = (s * 32) * RB, OF1 = (s * 32 + 16) * RB;
      const u32x2* xr = reinterpret_cast<const u32x2*>(xchg) + (((xs * 2 + s) * C::NG + kgrp) * 4) * WAVE + l;
      i16x4 x0[8], x1[8];
      tr_issue<D, OF0, RB, TR2>(tbr, x0);
      tr_issue<D, OF1, RB, TR2>(tbr, x1);
      // gradient wave: dS of register group i4 = P (fp16, from the score
      // wave's lanes) times dP'
      auto ds4 = [&](int i4, float (&d4)[4]) __attribute__((always_inline)) {
        const u32x2 pv = xr[i4 * WAVE];
        const float pf[4] = {f16_lo(pv[0]), f16_hi(pv[0]), f16_lo(pv[1]), f16_hi(pv[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) d4[e] = pf[e] * __uint_as_float(carry[16 * s + i4 * 4 + e]);
      };
      uint32_t op[2][4];
      bool big;
      if (grad) {
        float dsmax = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float d4[4];
          ds4(i4, d4);
#pragma unroll
          for (int e = 0; e < 4; ++e) dsmax = fmaxf(dsmax, fabsf(d4[e]));
          op[i4 >> 1][(i4 & 1) * 2] = pack_bf16x2(d4[0], d4[1]);
          op[i4 >> 1][(i4 & 1) * 2 + 1] = pack_bf16x2(d4[2], d4[3]);
        }
        big = dsmax > SPLIT_DS;
      } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int k = 0; k < 4; ++k) op[hh][k] = carry[8 * s + 4 * hh + k];
        big = pmaxc[s] > SPLIT_P;
      }
      const bf16x8 o0 = __builtin_bit_cast(bf16x8, u32x4{op[0][0], op[0][1], op[0][2], op[0][3]});
      const bf16x8 o1 = __builtin_bit_cast(bf16x8, u32x4{op[1][0], op[1][1], op[1][2], op[1][3]});
      tr_wait<2 * DT>(x0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(o0, tr_operand(x0, dt), acc[dt]);
      tr_wait<0>(x1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(o1, tr_operand(x1, dt), acc[dt]);
      if (__builtin_expect(__any(big), 0)) {
        u32x4 lo[2];
        if (grad) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            float d4[4];
            ds4(i4, d4);
            lo[i4 >> 1][(i4 & 1) * 2] = bf16x2_residual(d4[0], d4[1], op[i4 >> 1][(i4 & 1) * 2]);
            lo[i4 >> 1][(i4 & 1) * 2 + 1] = bf16x2_residual(d4[2], d4[3], op[i4 >> 1][(i4 & 1) * 2 + 1]);
          }
        } else {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int k = 0; k < 4; ++k) lo[hh][k] = carry[16 + 8 * s + 4 * hh + k];
        }
        // reads and their wait in one statement: on this rare path the
        // compiler may move registers freely
        bf16x8 y[4];
        lds_operand_tr_x4(tbr + OF0, tbr + OF0 + TR2, y);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(__builtin_bit_cast(bf16x8, lo[0]), y[dt], acc[dt]);
        lds_operand_tr_x4(tbr + OF1, tbr + OF1 + TR2, y);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32(__builtin_bit_cast(bf16x8, lo[1]), y[dt], acc[dt]);
      }
    });
  };

  // The operand registers are taken where a first front needs them, so that
  // the compiler's wait for their loads happens once per tile.
  auto take_kv = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      asm volatile("" : "+v"(kvraw[ks]));
      kv[ks] = __builtin_bit_cast(bf16x8, kvraw[ks]);
    }
  };
  // The front of a tile's first block (query head 0, block m_first).
  auto front_first = [&](const Tv& tv, const char* buf, int xs) __attribute__((always_inline)) {
    if (tv.u0 > 0 || tv.u1 <= 0) front(std::true_type{}, tv, tv.m_first, buf, xs);
    else front(std::false_type{}, tv, tv.m_first, buf, xs);
  };

  // One stream of iterations across tiles.  Iteration i of a tile runs the
  // back of block i - 1 and then the front of block i, with one barrier per
  // iteration; blocks stream one ahead through a ring of 3 buffers, so the
  // ring holds the back's block, the front's block and the copies in
  // flight.  Between two tiles one transition runs the back of the first
  // tile's last block beside the front of the next tile's first block (the
  // next tile's start: its successor, the copies of its second block); each
  // wave issues the first tile's stores right after that back, and they
  // drain during the front and the next iteration.  Hand-over areas
  // alternate by iteration across tiles.
  int ring_back = 0;
  int xlast = 1;       // hand-over area of the last front
  Tp pv = cp;          // the tile whose last back is pending
  bool pend = false;   // ... if any
  bool cv = true;      // cp is a tile to start
  for (int64_t pass = 0;; ++pass) {
    // ---- transition: the back of pv's last block (pend), the start of cp (cv)
    const Tv tv = tvals(cp);
    const bool fr = cv && tv.nb > 0;
    if (fr) load_rows(cp);                // the last front has used the rows it replaces
    asm volatile("" ::: "memory");        // the row loads stay ahead of the wait that counts them
    bool own0 = false;
    if (fr && iss_cur < 1) {
      prep_next(cp, cp, false);           // cp's first block, not issued yet (the first tile's,
      issue_now();                        // or one after a tile without blocks)
      own0 = true;
    }
    // this wave's copies of cp's first block, issued before the row loads
    // (and any stores), or just now
    if (own0 || !fr) wait_vmcnt<0>();
    else wait_vmcnt<KS>();
    if constexpr (!DYN) {
      if (cv) start_duties(pass);
    }
    if (DYN && cv && pass > 0 && wave == 0 && l == 0) s_next = (int)fetched;
    barrier_lds();
    if (cv) {
      if constexpr (DYN) start_duties(pass);
      prep_next(cp, np, has_nxt);         // cp's second block, or the next tile's first
      issue_now();
    }
    if (pend) {
      back(smem[ring_back], xlast);
      store_acc(pv, min(pv.L - pv.k0, BN), acc);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
    }
    if (fr) {
      take_kv();
      front_first(tv, smem[ring_cmp], xlast ^ 1);
      xlast ^= 1;
      ring_back = ring_cmp;
      ring_cmp = ring_cmp == NBUF - 1 ? 0 : ring_cmp + 1;
    } else {
      // (a definition on this path too, so that the rows of the tile before
      // are dead during the back above)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[ks] = bf16x8{};
    }
    const bool stores_out = pend;
    if (!cv) break;
    // every wave has read the hand-out index before wave 0 writes the next
    // one (a tile of two or more blocks has iteration barriers in between)
    if (DYN && tv.nb <= 1) barrier_lds();

    if (tv.nb == 0) {
      store_zero(cp, min(cp.L - cp.k0, BN));  // a tile without query blocks
      pend = false;
    } else {
      const int nb = tv.nb, nbh = tv.nbh;
      // iteration i (1 <= i < nb); its front is block m of the stream's current query head
      auto iter = [&](auto masked_tag, int i, int m) __attribute__((always_inline)) {
        // this wave's copies of block i (issued at the transition before
        // the 16 * DT stores of the tile before, when i = 1)
        static_assert(16 * DT >= 63, "wait count");
        if (i == 1 && stores_out) wait_vmcnt<63>();
        else wait_vmcnt<0>();
        barrier_lds();  // every wave's copies landed; block i - 2's buffer and hand-over area free
        // Block i + 1 (the next tile's first block at i = nb - 1)
        prep_next(cp, np, has_nxt);
        issue_rows(0, C::CPT);  // Q rows and row terms now, dO rows after the back:
        issue_vec();            // a workgroup's 56 copies queue behind each other
        back(smem[ring_back], xlast);
        issue_rows(C::CPT, 2 * C::CPT);
        front(masked_tag, tv, m, smem[ring_cmp], xlast ^ 1);
        xlast ^= 1;
        ring_back = ring_cmp;  // the next iteration's back reads this block
        ring_cmp = ring_cmp == NBUF - 1 ? 0 : ring_cmp + 1;
      };
      // iterations [max(i0, 1), i1) of the head whose blocks start at
      // iteration hb (a loop per mask variant keeps register allocation to
      // one body at a time)
      auto run = [&](auto masked_tag, int i0, int i1, int hb) __attribute__((always_inline)) {
        for (int i = max(i0, 1); i < i1; ++i) iter(masked_tag, i, tv.m_first + (i - hb));
      };
      for (int i0 = 0; i0 < nb; i0 += nbh) {
        run(std::true_type{}, i0, i0 + tv.u0, i0);
        run(std::false_type{}, i0 + tv.u0, i0 + tv.u1, i0);
        run(std::true_type{}, i0 + tv.u1, i0 + nbh, i0);
      }
      pend = true;
    }
    pv = cp;
    cv = has_nxt;
    if (cv) {
      // the stream's position moves on to the next tile, whose first block
      // may already be issued
      cur_gi = iss_nxt > 0 && np.nbh == 1 ? 1 : 0;
      cur_jb = iss_nxt > 0 && np.nbh > 1 ? 1 : 0;
      iss_cur = iss_nxt;
      iss_nxt = 0;
      cp = np;
    }
  }
}

// ----------------------------------------------------------- exact delta --
// For a sequence with at most BWD_BN keys, delta_i = sum_k P_ik dP_ik from
// fp32 P and dP (the same quantity as rowsum(dO o O), without the bf16
// rounding of the stored O, which dominates the dK and dQ error when P is
// large).  In causal broadcast mode the same holds for the first BWD_BN
// query rows of any sequence: they see only keys below BWD_BN, and few of
// them, so their P is large too, and dQ sums such rows over every sequence.
// (Self-attention rows are not summed across sequences; their error stays
// within the bar, and the pass would cost a workgroup per (sequence, head).)
// A workgroup takes query rows 128 z .. 128 z + 127 (z = blockIdx.z) of one
// head for each sequence it visits: in causal broadcast mode for z = 0 one
// sequence per workgroup, otherwise a walk over the short sequences from
// the end of the length-sorted order.  Wave w takes rows 32w .. 32w+31
// with the transposed score layout S^T = K Q^T (lane -> query, registers
// -> keys), so each lane sums its registers and the two halves of the wave
// are added.
template <int D, bool CAUSAL, bool BCAST>
__global__ __launch_bounds__(256) void delta_exact_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  static_assert(BWD_BN == 128, "the causal rows of block 0 see keys below 128 only");
  const int h = blockIdx.y;
  const int H = a.H, Lq = a.Lq;
  const int wave = threadIdx.x / WAVE, l = threadIdx.x % WAVE, g = l / 32, lc = l % 32;
  const int qw = blockIdx.z * 128 + wave * 32;
  // Rows of sequence b: query block blockIdx.z against its first Lk keys.
  auto rows_of = [&](int b, int L, int64_t s0) {
    const int Lk = min(L, BWD_BN);  // keys any row of this workgroup sees
    const int nq = BCAST ? Lq : L;
    if (qw >= nq) return;
    const int q = qw + lc;
    const int qc = min(q, nq - 1);
    const uint16_t* qrow = BCAST ? a.q + ((int64_t)h * Lq + qc) * D : a.q + ((s0 + qc) * H + h) * (int64_t)D;
    const int64_t ri = BCAST ? ((int64_t)b * H + h) * Lq + qc : (s0 + qc) * H + h;
    const uint16_t* dorow = a.dout + ri * D;
    bf16x8 qr[KS], dr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + ks * 16 + g * 8));
      dr[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dorow + ks * 16 + g * 8));
    }
    const float ls2 = a.lse2[ri];
    const float c2 = a.scale_log2;
    float acc = 0.f;
    // K and V of each 32-key half are loaded one half ahead, so that a
    // sequence's key halves cost one load latency, not one each
    u32x4 kn[KS], vn[KS];
    auto load_kv = [&](int kt) {
      const int key = min(kt * 32 + lc, Lk - 1);
      const uint16_t* kr = a.k + ((s0 + key) * a.Hkv + h / a.G) * (int64_t)D;
      const uint16_t* vr = a.v + ((s0 + key) * a.Hkv + h / a.G) * (int64_t)D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kn[ks] = *reinterpret_cast<const u32x4*>(kr + ks * 16 + g * 8);
        vn[ks] = *reinterpret_cast<const u32x4*>(vr + ks * 16 + g * 8);
      }
    };
    load_kv(0);
    for (int kt = 0; kt * 32 < Lk; ++kt) {
      bf16x8 kc[KS], vc[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kc[ks] = __builtin_bit_cast(bf16x8, kn[ks]);
        vc[ks] = __builtin_bit_cast(bf16x8, vn[ks]);
      }
      if ((kt + 1) * 32 < Lk) load_kv(kt + 1);
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        st = mfma32(kc[ks], qr[ks], st);
        dpt = mfma32(vc[ks], dr[ks], dpt);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kt * 32 + 8 * (i / 4) + 4 * g + (i % 4);
        bool ok = kk < Lk;
        if (CAUSAL) ok = ok && kk <= q && (a.window <= 0 || kk > q - a.window);
        const float p = ok ? fast_exp2(st[i] * c2 - ls2) : 0.f;
        acc += p * dpt[i];
      }
    }
    acc = sum_across_halves(acc);
    if (g == 0 && q < nq) {
      a.delta[ri] = acc;
      reinterpret_cast<u32x4*>(a.term_d)[ri] = row_terms(-acc);
    }
  };
  if (CAUSAL && BCAST && blockIdx.z == 0) {
    // every sequence: the first 128 query rows see keys below 128 only
    const int b = blockIdx.x;
    int64_t s0;
    const int L = (int)seq_range(a.offsets, b, a.total_len, &s0);
    if (L > 0) rows_of(b, L, s0);
    return;
  }
  // The sequences of at most BWD_BN keys sit at the end of the
  // length-sorted order (longest first): workgroup x takes ranks
  // B - 1 - x, B - 1 - x - gridDim.x, ... until a longer sequence.
  for (int r = a.B - 1 - (int)blockIdx.x; r >= 0; r -= (int)gridDim.x) {
    const int b = a.seq_order[r];
    int64_t s0;
    const int L = (int)seq_range(a.offsets, b, a.total_len, &s0);
    if (L > BWD_BN) break;
    if (L > 0) rows_of(b, L, s0);
  }
}

constexpr int DELTA_EXACT_WG = 256;  // workgroups per (head, query block) over the short sequences

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t st) {
  const int nqb = a.broadcast_q ? (a.Lq + 127) / 128 : 1;
  // causal broadcast: a workgroup per sequence (every sequence's first query
  // block); otherwise workgroups walk the short sequences of the sorted order
  const int gx = a.broadcast_q && a.causal ? a.B : min(a.B, DELTA_EXACT_WG);
  const dim3 eg((unsigned)gx, (unsigned)a.H, (unsigned)nqb);
  if (a.broadcast_q) {
    if (a.causal) JFA_TIMED_LAUNCH(K_DELTA_EXACT, st, (delta_exact_kernel<D, true, true>), eg, dim3(256), 0, st, a);
    else JFA_TIMED_LAUNCH(K_DELTA_EXACT, st, (delta_exact_kernel<D, false, true>), eg, dim3(256), 0, st, a);
  } else {
    if (a.causal) JFA_TIMED_LAUNCH(K_DELTA_EXACT, st, (delta_exact_kernel<D, true, false>), eg, dim3(256), 0, st, a);
    else JFA_TIMED_LAUNCH(K_DELTA_EXACT, st, (delta_exact_kernel<D, false, false>), eg, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128) {
    if (a.broadcast_q) {
      if (a.causal) JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_pair_kernel<true, true>), dim3(a.P), dim3(512), 0, st, a, a.ktiles);
      else JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_pair_kernel<false, true>), dim3(a.P), dim3(512), 0, st, a, a.ktiles);
    } else {
      if (a.causal) JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_pair_kernel<true, false>), dim3(a.P), dim3(512), 0, st, a, a.ktiles);
      else JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_pair_kernel<false, false>), dim3(a.P), dim3(512), 0, st, a, a.ktiles);
    }
  } else {
    if (a.broadcast_q) {
      if (a.causal) JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, true, true>), dim3(a.P), dim3(256), 0, st, a, a.ktiles);
      else JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, false, true>), dim3(a.P), dim3(256), 0, st, a, a.ktiles);
    } else {
      if (a.causal) JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, true, false>), dim3(a.P), dim3(256), 0, st, a, a.ktiles);
      else JFA_TIMED_LAUNCH(K_DKDV, st, (dkdv_kernel<D, false, false>), dim3(a.P), dim3(256), 0, st, a, a.ktiles);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return launch_d<64>(a, stream);
  return launch_d<128>(a, stream);
}

}  // namespace jfa

