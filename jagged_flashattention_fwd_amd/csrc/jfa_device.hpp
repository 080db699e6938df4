// Device-side building blocks for the gfx950 (CDNA4) jagged attention kernels.
//
// Everything here is written for one wave of 64 lanes and the bf16 matrix
// core instruction v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, C 32x32 fp32).
// Operand lane layouts of that instruction (checked on the device):
//   A:  lane l holds A[l % 32][8*(l/32) + 0..7]
//   B:  lane l holds B[8*(l/32) + 0..7][l % 32]
//   C:  lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l % 32]
// LDS tiles are row-major bf16 with padded rows (TileGeom).  The LDS serves
// 256 bytes per cycle: a 16-byte read takes 16 lanes per cycle, the
// transposing read ds_read_b64_tr_b16 32 lanes (4 rows x 64 bytes).  Rows of
// 304 bytes keep 16-byte reads of 16 consecutive rows free of bank
// conflicts; under the transposing read, neighbouring rows overlap by 16
// bytes (a two-way conflict, seen in the SQ_LDS_BANK_CONFLICT counter).
// Tiles read only by the transposing read use 320-byte rows, which are free
// of conflicts there (no conflict cycles counted).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace jfa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) short lds_short;

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// f(integral_constant<int, i>) for i = B .. E-1, at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- math --
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}
// Two-term bf16 split of a pair: hi = the values truncated to bf16, lo = the
// remainders rounded to bf16, so hi + lo carries about 16 significant bits.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t* hi, uint32_t* lo) {
  const uint32_t ua = __float_as_uint(a) & 0xffff0000u, ub = __float_as_uint(b) & 0xffff0000u;
  *hi = (ua >> 16) | ub;
  f32x2 r = {a - __uint_as_float(ua), b - __uint_as_float(ub)};
  *lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
}
// fp32 pair -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x as three bf16 values whose sum is exactly x (the first two truncate the
// value and its remainder to 8 significant bits; the last remainder has at
// most 8 left), then five zeros: eight bf16 MFMA operand slots.  Multiplied by
// ones in the matching slots of the other operand, one extra k-step adds x to
// every product of the row in the fp32 accumulator.
__device__ __forceinline__ u32x4 row_terms(float x) {
  const uint32_t u0 = __float_as_uint(x) & 0xffff0000u;
  const float r1 = x - __uint_as_float(u0);
  const uint32_t u1 = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(u1);
  return u32x4{(u0 >> 16) | u1, __float_as_uint(r2) >> 16, 0u, 0u};
}

// Full-row reductions for the transposed score layout, where lanes l and
// l+32 hold the two halves of one row: after the swap every lane sees both.
__device__ __forceinline__ float max_across_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float min_across_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ------------------------------------------------------------- LDS tiles --
// Row-major bf16 tile with D columns, rows padded to ROW_BYTES.  The padding
// is chosen so that 16-byte reads of 16 consecutive rows at one column hit
// 16 distinct 16-byte bank groups (ROW_BYTES / 16 is odd).  Because the
// layout is affine in (row, column), every operand address is one per-lane
// base plus a compile-time constant, which the LDS instructions take as an
// immediate offset.
template <int D>
struct TileGeom {
  static_assert(D == 64 || D == 128, "tile width");
  static constexpr int ROW_BYTES = D == 128 ? 304 : 208;
};
// Byte offset of (row, 16-byte chunk).
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * TileGeom<D>::ROW_BYTES + (chunk << 4);
}
// Byte offset of element column `col` of `row`.
template <int D, int RB = TileGeom<D>::ROW_BYTES>
__device__ __forceinline__ int tile_off_col4(int row, int col) {
  return row * RB + (col << 1);
}
template <int R, int D>
constexpr int tile_bytes() { return R * TileGeom<D>::ROW_BYTES; }

__device__ __forceinline__ bf16x8 lds_read16(const char* lds, int off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + off));
}
__device__ __forceinline__ void lds_write16(char* lds, int off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}

// ds_read_b64_tr_b16: within each 16-lane group, source lane s = 4j + q
// supplies 4 consecutive 16-bit values of row j at columns 4q..4q+3; lane i of
// the group receives column i of rows 0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* lds, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)((lds_short*)((__attribute__((address_space(3))) char*)(lds + off))));
}

// MFMA operand with the k index running along the rows of a row-major LDS
// tile X[k][n] (e.g. V^T from V[key][d]): lane l receives X[k][n0 + l%32] for
// its 8 k-slots.  `krow(r, g)` gives the first of the 4 rows delivered by read
// r (0 or 1) to lane group g = l/32; rows krow..krow+3 fill k-slots 4r..4r+3.
template <int D, int RB = TileGeom<D>::ROW_BYTES>
__device__ __forceinline__ bf16x8 lds_operand_tr(const char* lds, int krow0, int krow1, int n0) {
  const int l = lane_id();
  const int s = l & 15, j = s >> 2, q = s & 3, G = l >> 4;
  const int col = n0 + ((G & 1) << 4) + (q << 2);
  i16x4 a = lds_read_tr(lds, tile_off_col4<D, RB>(krow0 + j, col));
  i16x4 b = lds_read_tr(lds, tile_off_col4<D, RB>(krow1 + j, col));
  struct P { i16x4 x, y; } p = {a, b};
  return __builtin_bit_cast(bf16x8, p);
}

// 32-bit LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// Four MFMA A operands of a transposed 128-wide tile (head-dim tiles 0..3)
// from one key group, with the transpose read issued directly: a0 / a1 are
// this lane's LDS addresses for the group's first and second 4-row read.
// The builtin form of the instruction makes the compiler drain every
// outstanding direct-to-LDS copy before it; this form waits only for its
// own reads (lgkmcnt), and its results depend on that wait.
__device__ __forceinline__ void lds_operand_tr_x4(uint32_t a0, uint32_t a1, bf16x8 out[4]) {
  i16x4 x0, y0, x1, y1, x2, y2, x3, y3;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:64\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:128\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:192\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0), "=&v"(y0), "=&v"(x1), "=&v"(y1), "=&v"(x2), "=&v"(y2), "=&v"(x3), "=&v"(y3)
      : "v"(a0), "v"(a1)
      : "memory");
  struct P { i16x4 x, y; };
  out[0] = __builtin_bit_cast(bf16x8, P{x0, y0});
  out[1] = __builtin_bit_cast(bf16x8, P{x1, y1});
  out[2] = __builtin_bit_cast(bf16x8, P{x2, y2});
  out[3] = __builtin_bit_cast(bf16x8, P{x3, y3});
}

// Four transposed reads (rows a0 / a1, column byte offsets OFF and OFF +
// 64) issued without waiting: two MFMA operands.  tr4_wait<N> makes them
// available once at most N later LDS reads of this wave are outstanding.
template <int OFF>
__device__ __forceinline__ void tr4_issue(uint32_t a0, uint32_t a1, i16x4 (&x)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(a0), "v"(a1), "i"(OFF), "i"(OFF + 64));
}
template <int N>
__device__ __forceinline__ void tr4_wait(i16x4 (&x)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : "i"(N));
}
__device__ __forceinline__ bf16x8 tr4_operand(const i16x4 (&x)[4], int k) {
  struct P { i16x4 a, b; } p = {x[2 * k], x[2 * k + 1]};
  return __builtin_bit_cast(bf16x8, p);
}

// ------------------------------------------------------ global <-> LDS ----
// A tile of R rows x D bf16 columns is copied by NT threads, 16 bytes each
// per step; row r of the tile is global row (base + r * ld) and rows at or
// beyond `nrows` read as zero.
template <int R, int D, int NT>
struct TileLoader {
  static constexpr int CPR = D / 8;              // chunks per row
  static constexpr int N = R * CPR / NT;         // chunks per thread
  static_assert(R * CPR % NT == 0, "tile must split evenly");
  u32x4 v[N];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, c = idx % CPR;
      if (r < nrows) {
        v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * ld + c * 8);
      } else {
        v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      const int r = idx / CPR, c = idx % CPR;
      lds_write16(lds, tile_off<D>(r, c), v[i]);
    }
  }
};

// ------------------------------------------------------------ sequences --
// Rows [s0, s0 + L) of the packed tensors belong to sequence b.  Offsets are
// clamped into [0, total] so that malformed offsets can never address memory
// outside the packed tensors (results are then meaningless, but in bounds).
__device__ __forceinline__ int64_t seq_range(const int64_t* __restrict__ off, int b, int64_t total,
                                             int64_t* s0_out) {
  int64_t s0 = off[b], e = off[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > total ? total : s0);
  e = e < s0 ? s0 : (e > total ? total : e);
  *s0_out = s0;
  return e - s0;
}

// ------------------------------------------------- direct global -> LDS --
typedef __attribute__((address_space(3))) void lds_void;


// 16 bytes per lane from base (wave-uniform) + voff (per lane) straight into
// LDS at lds + 16 * lane (global_load_lds_dwordx4, 1 KB per wave).  Written
// as asm so that the compiler does not treat it as a pending write to every
// LDS buffer and drain it before each LDS read; completion is tracked with
// wait_vmcnt.  readfirstlane states the uniformity of the addresses where
// the compiler cannot prove it, and costs nothing where they already sit in
// scalar registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_copy16(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t r = (uint64_t)(uintptr_t)base;
  const uint64_t ru = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(r >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)r);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"((const void*)(uintptr_t)ru), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0");
}
// The same copy through a buffer resource: 16 bytes per lane from byte
// soff + voff of the resource into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds).  The range check covers soff + voff: a
// lane at or past the resource's size reads nothing and writes zeros to its
// 16 bytes of LDS (checked on the device).  soff is wave-uniform.
__device__ __forceinline__ void dma_copy16_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rs),
               "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "m0");
}
#pragma clang diagnostic pop

// Buffer resource over [base, base + nbytes): buffer stores at byte offsets
// past nbytes are dropped by the hardware, which bounds-checks them per lane.
// Both values are wave-uniform; readfirstlane keeps the descriptor in scalar
// registers where the compiler cannot prove that.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  const uint64_t r = (uint64_t)(uintptr_t)base;
  const uint64_t ru = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(r >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)r);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)ru, (short)0, __builtin_amdgcn_readfirstlane(nbytes),
                                           0x00020000);
}

// Rows of 256 data bytes padded to NCH 16-byte chunks in LDS (NCH = 19:
// 304-byte rows; 20: 320-byte rows), copied with dma_copy16: one copy fills
// 3 whole rows and the first 64 - 3 NCH chunks of a fourth.  Lane l moves
// chunk l % NCH of row l / NCH; chunks 16 .. NCH - 1 are padding (those
// lanes re-read chunk 0 into it).  A run of n >= 3 rows takes ceil(n / 3)
// copies starting at rows min(3 k, n - 3); the overhang into the row after
// the run writes the values that row's own copy writes, or lands in the
// GAP bytes kept after the tile.
template <int NCH>
struct PadRowCopyN {
  static constexpr int GAP = 128;
  static_assert(NCH >= 16 && 64 / NCH == 3 && (64 - 3 * NCH) * 16 <= GAP, "three rows and part of a fourth");
  static constexpr int ROW_BYTES = NCH * 16;
  uint32_t row;   // row of this lane within a copy (0..3)
  uint32_t byte;  // byte offset of its chunk within the row
  __device__ __forceinline__ PadRowCopyN() : row(lane_row(lane_id())), byte(lane_byte(lane_id())) {}
  __device__ static constexpr uint32_t lane_row(int l) { return (uint32_t)(l / NCH); }
  __device__ static constexpr uint32_t lane_byte(int l) { return (l % NCH) < 16 ? (uint32_t)(l % NCH) * 16u : 0u; }
  static constexpr int copies(int n) { return (n + 2) / 3; }
  static constexpr int start(int k, int n) { return 3 * k < n - 3 ? 3 * k : n - 3; }
  // Per-lane source offset of copy k of a run whose rows past `last` repeat
  // row `last`; stride = global row stride in bytes.
  __device__ __forceinline__ uint32_t voff(int R, int last, uint32_t stride) const {
    return (uint32_t)min(R + (int)row, last) * stride + byte;
  }
};
using PadRowCopy = PadRowCopyN<19>;

// s_waitcnt with only the vector-memory counter constrained (at most n
// operations of this wave still outstanding; n <= 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that also orders this wave's earlier LDS reads before
// it (lgkmcnt(0)), without waiting for outstanding global loads: the
// direct-to-LDS pipelines account for those with wait_vmcnt.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ----------------------------------------------------------- schedule ----
// Tile t of the concatenated list goes to worker slot zigzag_slot(t, P):
// pass t / P fills slots left to right when even, right to left when odd.
__device__ __forceinline__ int64_t zigzag_tile(int64_t pass, int slot, int P) {
  return pass * P + ((pass & 1) ? (P - 1 - slot) : slot);
}
__device__ __forceinline__ int zigzag_slot(int64_t t, int P) {
  const int64_t p = t / P;
  const int s = (int)(t - p * P);
  return (p & 1) ? (P - 1 - s) : s;
}
// Persistent workgroup w runs worker slot logical_slot(w): hardware places
// workgroup w on XCD w % 8, so consecutive slots (which receive consecutive
// tiles, often of the same sequence) are packed onto the same XCD and its L2.
__device__ __forceinline__ int logical_slot(int w, int P) {
  const int per = P / 8;
  if (per * 8 != P) return w;
  return (w & 7) * per + (w >> 3);
}

}  // namespace jfa
