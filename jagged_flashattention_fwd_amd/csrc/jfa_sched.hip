// On-device tile scheduler for the persistent kernels.
//
// "Optimizing Jagged Flash Attention with TLX", "Scheduling jagged tiles
// across SMs", sorts the forward's tiles by K/V workload, longest first, and
// hands them to the persistent workers in a zigzag; the backward walks a list
// of valid (batch, head, K/V block) tiles, block-innermost.  That page does
// the sorting on the host.  Here it runs on the device from the offsets
// tensor, so no length ever crosses to the host and nothing synchronises:
//   1. one workgroup sorts the sequences by length, descending (ties: lower
//      index first), counts each sequence's tiles and takes an exclusive
//      prefix sum of the counts in sorted order;
//   2. one workgroup per sequence writes that sequence's tiles -- heads
//      ascending, blocks heaviest first -- at its prefix-sum position
//      (broadcast-Q backward: head-major, see sched_expand).
// The persistent kernels then take tile t in zigzag order (jfa_device.hpp).
#include "jfa_device.hpp"
#include "jfa_internal.hpp"
#include "jfa_timing.hpp"

namespace jfa {

namespace {

constexpr int SORT_THREADS = 1024;

__device__ __forceinline__ int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ int64_t tiles_of(int64_t L, int H, int Lq, int broadcast_q, int pass, int blk) {
  if (pass == 0) return (int64_t)H * cdiv64(broadcast_q ? Lq : L, blk);
  return (int64_t)H * cdiv64(L, blk);
}

// Single workgroup: bitonic sort of N = 2^k keys, then a chunked exclusive
// scan of the per-sequence tile counts.  Thread t holds keys c * 1024 + t;
// compare-exchange stages between lanes of one wave go through register
// shuffles, the others through LDS (two barriers each), so a sort of N keys
// takes 2 log2(N / 64) (log2(N / 64) + 1) / 2 barriers instead of one per
// stage.
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long x, int m) {
  const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)x, m);
  const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(x >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}
// New value of element i after the stage (k, j) compare-exchange with its
// partner i ^ j holding y: the lower index of an ascending (i & k == 0) pair
// keeps the minimum.
__device__ __forceinline__ unsigned long long bitonic_pick(int i, int k, int j, unsigned long long x,
                                                           unsigned long long y) {
  const bool up = (i & k) == 0, lower = (i & j) == 0;
  const unsigned long long mn = x < y ? x : y, mx = x < y ? y : x;
  return lower == up ? mn : mx;
}

__global__ __launch_bounds__(SORT_THREADS) void sched_sort_scan(SchedArgs a, Schedule s, int N) {
  extern __shared__ __attribute__((aligned(16))) unsigned long long keys[];
  __shared__ int64_t wsum[SORT_THREADS / WAVE];
  constexpr int EMAX = MAX_B / SORT_THREADS;
  const int tid = threadIdx.x;
  const int B = a.B;
  const int E = (N + SORT_THREADS - 1) / SORT_THREADS;  // keys per thread
  unsigned long long v[EMAX];
#pragma unroll
  for (int c = 0; c < EMAX; ++c) {
    const int i = c * SORT_THREADS + tid;
    unsigned long long k = ~0ull;
    if (c < E && i < B) {
      int64_t s0;
      const int64_t L = seq_range(a.offsets, i, a.total_len, &s0);
      unsigned long long Lc = L > 0xffffffffll ? 0xffffffffull : (unsigned long long)L;
      k = ((0xffffffffull - Lc) << 32) | (unsigned long long)i;
    }
    v[c] = k;
  }
  for (int k = 2; k <= N; k <<= 1) {
    int j = k >> 1;
    for (; j >= WAVE; j >>= 1) {
#pragma unroll
      for (int c = 0; c < EMAX; ++c)
        if (c < E && c * SORT_THREADS + tid < N) keys[c * SORT_THREADS + tid] = v[c];
      __syncthreads();
#pragma unroll
      for (int c = 0; c < EMAX; ++c) {
        const int i = c * SORT_THREADS + tid;
        if (c < E && i < N) v[c] = bitonic_pick(i, k, j, v[c], keys[i ^ j]);
      }
      __syncthreads();
    }
    for (; j > 0; j >>= 1) {
#pragma unroll
      for (int c = 0; c < EMAX; ++c) {
        const int i = c * SORT_THREADS + tid;
        if (c < E) v[c] = bitonic_pick(i, k, j, v[c], shfl_xor_u64(v[c], j));
      }
    }
  }
#pragma unroll
  for (int c = 0; c < EMAX; ++c)
    if (c < E && c * SORT_THREADS + tid < N) keys[c * SORT_THREADS + tid] = v[c];
  __syncthreads();
  // Chunked exclusive scan over ranks 0..B-1: a shuffle scan inside each
  // wave, then the totals of the waves before.
  const int per = (B + SORT_THREADS - 1) / SORT_THREADS;
  const int r0 = tid * per, r1 = min(B, r0 + per);
  // a sequence's length comes back out of its key (every length is at
  // most total_len, below 2^31)
  auto len_of = [](unsigned long long key) { return (int64_t)(0xffffffffull - (key >> 32)); };
  int64_t local = 0;
  for (int r = r0; r < r1; ++r) {
    const int b = (int)(keys[r] & 0xffffffffull);
    s.order[r] = b;
    local += tiles_of(len_of(keys[r]), a.H, a.Lq, a.broadcast_q, a.pass, a.blk);
  }
  const int lane = tid % WAVE, wv = tid / WAVE;
  int64_t incl = local;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const int64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == WAVE - 1) wsum[wv] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  int64_t total = 0;
  for (int w = 0; w < SORT_THREADS / WAVE; ++w) total += wsum[w];
  // Positions are clamped to the list's capacity, which well-formed offsets
  // never reach.
  int64_t run = before + incl - local;  // exclusive prefix of this chunk
  for (int r = r0; r < r1; ++r) {
    s.cum[r] = run < s.max_tiles ? run : s.max_tiles;
    run += tiles_of(len_of(keys[r]), a.H, a.Lq, a.broadcast_q, a.pass, a.blk);
  }
  if (tid == SORT_THREADS - 1) {
    const int64_t T = total < s.max_tiles ? total : s.max_tiles;
    s.cum[B] = T;
    s.n_tiles[0] = T;
    s.n_tiles[1] = 0;  // the forward's dynamic hand-out counter
  }
}

// One workgroup per sorted rank: write that sequence's tiles.
__global__ __launch_bounds__(256) void sched_expand(SchedArgs a, Schedule s) {
  const int r = blockIdx.x;
  const int b = s.order[r];
  const int64_t start = s.cum[r];
  const int64_t n = s.cum[r + 1] - start;
  if (n <= 0) return;
  int64_t s0;
  const int64_t L = seq_range(a.offsets, b, a.total_len, &s0);
  const int64_t nblk = a.pass == 0 ? cdiv64(a.broadcast_q ? a.Lq : L, a.blk) : cdiv64(L, a.blk);
  if (nblk <= 0) return;
  // Broadcast-Q backward: the list is head-major (all tiles of head 0, then
  // head 1, ...), so at any time the persistent workgroups read one head's
  // 64-128 KB of Q, which stays resident in L2 beside the K / V streams.
  // Every sequence has the same tile count in every head, so head h's part
  // of the list starts at h * (T / H) and this sequence's tiles at cum[r] / H.
  const bool head_major = a.pass == 1 && a.broadcast_q;
  const int64_t T = s.cum[a.B];
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
    const int h = (int)(j / nblk);
    const int64_t i = j - (int64_t)h * nblk;
    const int blk = (int)(a.pass == 0 ? nblk - 1 - i : i);
    const int64_t pos = head_major ? h * (T / a.H) + start / a.H + i : start + j;
    const TileRec rec = a.kv_tiles ? TileRec{b, h * a.G, blk, (int)L, s0, h, 0} : TileRec{b, h, blk, (int)L, s0, h / a.G, 0};
    if (pos < s.max_tiles) s.tiles[pos] = rec;
  }
}

// Tile list in list order, `ncol` int32 per tile: b, h, block, worker slot
// (ncol = 4) or b, h, block, key / value head, worker slot (ncol = 5).
__global__ __launch_bounds__(256) void sched_dump(Schedule s, int P, int32_t* out, int64_t cap, int64_t* n_out,
                                                  int ncol) {
  const int64_t T = *s.n_tiles;
  const int64_t n = T < cap ? T : cap;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (int64_t)gridDim.x * blockDim.x) {
    const TileRec r = s.tiles[t];
    int32_t* o = out + ncol * t;
    o[0] = r.b;
    o[1] = r.h;
    o[2] = r.blk;
    if (ncol == 5) o[3] = r.hk;
    o[ncol - 1] = zigzag_slot(t, P);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_out = T;
}

}  // namespace

hipError_t init_schedule_kernels() {
  // Sorting MAX_B keys needs 64 KiB of dynamic LDS.
  return hipFuncSetAttribute(reinterpret_cast<const void*>(sched_sort_scan),
                             hipFuncAttributeMaxDynamicSharedMemorySize, MAX_B * 8);
}

hipError_t launch_schedule(const SchedArgs& a, const Schedule& s, hipStream_t stream) {
  int N = WAVE;  // at least one wave of keys: the shuffle stages span whole waves
  while (N < a.B) N <<= 1;
  JFA_TIMED_LAUNCH(K_SCHED_SORT, stream, sched_sort_scan, dim3(1), dim3(SORT_THREADS), (size_t)N * 8, stream, a, s, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  JFA_TIMED_LAUNCH(K_SCHED_EXPAND, stream, sched_expand, dim3(a.B), dim3(256), 0, stream, a, s);
  return hipGetLastError();
}

hipError_t launch_schedule_dump(const Schedule& s, int P, int32_t* out, int64_t cap, int64_t* n_out, int ncol,
                                hipStream_t stream) {
  JFA_TIMED_LAUNCH(K_SCHED_DUMP, stream, sched_dump, dim3(256), dim3(256), 0, stream, s, P, out, cap, n_out, ncol);
  return hipGetLastError();
}

}  // namespace jfa
