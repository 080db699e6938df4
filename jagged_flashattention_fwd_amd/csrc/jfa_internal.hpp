// Internal (library-private) launch interface shared by the host API and the
// kernel translation units.  Not part of the C-ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa {

// One tile of a persistent kernel's work list: sequence b, head h, block blk,
// and the sequence's (clamped) packed row range [s0, s0 + L), so that a
// kernel needs no second dependent load to find its rows.
struct TileRec {
  int b, h, blk, L;
  int64_t s0;
  int hk;   // key / value head of query head h (h / G; h with plain heads)
  int pad;
};
static_assert(sizeof(TileRec) == 32, "tile record layout");

// Tile sizes.  Forward: a tile is BM query rows of one (sequence, head),
// streamed against K/V in steps of KV_STEP keys.  Backward: a tile is BN key
// rows of one (sequence, head), streamed against query blocks of QB rows.
constexpr int FWD_KV_STEP = 64;
constexpr int FWD_BM = 256;        // forward tile: 8 waves x 32 query rows
constexpr int BWD_BN = 128;        // 4 waves x 32 key rows
constexpr int BWD_QB = 64;         // query rows per step of the dK/dV kernel
constexpr int DQ_BM = 256;         // self-attention dQ kernel: 8 waves x 32 query rows
constexpr int DQ_BM_BCAST = 256;   // broadcast dQ kernel: 8 waves x 32 query rows
constexpr int DQ_KV_STEP = 64;
constexpr int MAX_B = 8192;        // single-workgroup sequence sort
constexpr float MIN_BWD_SCALE = 0x1p-100f;  // smallest |scale| the backward accepts

struct Schedule {
  int* order;         // [B]
  int64_t* cum;       // [B+1]
  TileRec* tiles;     // [max_tiles]
  int64_t* n_tiles;   // [2]: tile count, then the forward's hand-out counter (reset by the sort)
  int64_t max_tiles;  // capacity of `tiles`
};

struct SchedArgs {
  const int64_t* offsets;
  int64_t total_len;
  int B, H, Lq, broadcast_q, pass, blk;
  int G;  // query heads per key / value head (the tile records' hk = h / G)
  // 1: the tiles are per key / value head (H above is H_kv): each covers the
  // G query heads of its group, its record carries the group's first query
  // head h = hk * G and hk.  0: per query head.
  int kv_tiles = 0;
};

// Once per device, with it current: kernel attributes of the scheduler.
hipError_t init_schedule_kernels();
hipError_t launch_schedule(const SchedArgs& a, const Schedule& s, hipStream_t stream);
hipError_t launch_schedule_dump(const Schedule& s, int P, int32_t* out, int64_t cap, int64_t* n_out, int ncol,
                                hipStream_t stream);

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int64_t* offsets;
  uint16_t* out;
  float* lse;
  const TileRec* tiles;
  const int64_t* n_tiles;
  unsigned int* tile_ctr;  // tiles handed out past the first two per workgroup (starts at 0)
  int64_t total_len;
  int B, H, Lq, d;
  int Hkv, G;        // key / value heads; G = H / Hkv query heads share one
  int window;        // causal sliding window in keys (query i sees i - window < j <= i); 0: none
  float scale_log2;  // softmax scale times log2(e)
  int causal, broadcast_q;
  int P;             // persistent workgroups
};
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// MXFP8 forward (d = 128): E4M3 codes and E8M0 scale codes, layouts as in
// jfa_fwd_mxfp8.
struct FwdMxArgs {
  const uint8_t* q8;
  const uint8_t* q_scale;
  const uint8_t* k8;
  const uint8_t* k_scale;
  const uint8_t* vt8;
  const uint8_t* vt_scale;
  const int64_t* offsets;
  uint16_t* out;
  float* lse;
  const TileRec* tiles;
  const int64_t* n_tiles;
  unsigned int* tile_ctr;
  int64_t total_len;
  int64_t t_pad;  // keys per V^T row: total_len rounded up to 64
  int B, H, Lq;
  int Hkv, G;
  float scale_log2;
  int causal, broadcast_q;
  int P;
};
hipError_t launch_fwd_mx(const FwdMxArgs& a, hipStream_t stream);

// MXFP8 backward (d = 128): E4M3 / E8M0 codes of every encoding, layouts as
// in jfa_bwd_mxfp8.
struct BwdMxArgs {
  const uint8_t* q8;  const uint8_t* q_scale;    // row-wise
  const uint8_t* qt8; const uint8_t* qt_scale;   // query-blocked, transposed
  const uint8_t* k8;  const uint8_t* k_scale;    // row-wise
  const uint8_t* kt8; const uint8_t* kt_scale;   // key-blocked, transposed
  const uint8_t* v8;  const uint8_t* v_scale;    // row-wise
  const uint8_t* do8; const uint8_t* do_scale;   // row-wise
  const uint8_t* dot8; const uint8_t* dot_scale; // query-blocked, transposed
  const int64_t* offsets;
  const uint16_t* out;    // the forward's O (bf16)
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;           // [rows] scratch: -delta (the dP products start from it)
  float* lse2;            // [rows] scratch: lse * log2(e)
  float* dq_part;         // broadcast-mode dQ partials, as in BwdArgs
  const int* seq_order;
  int dq_qblocks, dq_chunks;
  const TileRec* ktiles;  // key tiles of MX_BK keys per (sequence, key / value head)
  const int64_t* n_ktiles;
  unsigned int* ktile_ctr;
  const TileRec* qtiles;  // self mode: query tiles of MX_BM rows
  const int64_t* n_qtiles;
  unsigned int* qtile_ctr;
  int64_t total_len;
  int64_t t_pad;          // total_len rounded up to 64
  int lq_pad;             // broadcast: Lq rounded up to 64
  int B, H, Lq;
  int Hkv, G;
  float scale, scale_log2;
  int causal, broadcast_q;
  int P;
};
constexpr int MX_BK = 128;  // keys per tile of the MXFP8 dK / dV kernel: 4 waves x 32
constexpr int MX_BM = 256;  // query rows per tile of the MXFP8 dQ kernel: 8 waves x 32
hipError_t launch_bwd_mx(const BwdMxArgs& a, hipStream_t stream);
// dq[h][q][:] = scale * the sum over the NC partials of (h, q-block), as
// the broadcast dQ of the bf16 backward (jfa_bwd.hip).
hipError_t launch_dq_reduce(const float* part, float* dq, int H, int Lq, int d, int BM, int n_qb, int NC,
                            float scale, hipStream_t stream);

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int64_t* offsets;
  const uint16_t* out;
  const float* lse;
  const uint16_t* dout;
  float* dq;
  float* dk;
  float* dv;
  float* delta;           // [rows] scratch: delta per query row
  float* lse2;            // [rows] scratch: lse * log2(e) per query row
  // [rows][8] bf16 scratch: -lse / scale (term_l) and -delta (term_d) of each
  // query row as three bf16 terms (t0 + t1 + t2 within 2^-24 of it), then
  // five zeros: the extra k-step that folds the row terms into the score
  // products of the dK / dV kernel.
  uint16_t* term_l;
  uint16_t* term_d;
  float* dq_part;         // [H][n_qb][NC][DQ_BM_BCAST][d] broadcast-mode partials
  const int* seq_order;   // sequences sorted by length (broadcast dQ chunks)
  int dq_qblocks;         // n_qb = cdiv(Lq, DQ_BM_BCAST)
  int dq_chunks;          // NC
  const TileRec* ktiles;  // key-block tiles (dK/dV kernel)
  const int64_t* n_ktiles;
  unsigned int* ktile_ctr;  // key tiles handed out past the zigzag ones (starts at 0)
  const TileRec* qtiles;  // query-block tiles (self-attention dQ kernel)
  const int64_t* n_qtiles;
  unsigned int* qtile_ctr;  // query tiles handed out past the first one per workgroup
  int B, H, Lq, d;
  int Hkv, G;             // key / value heads; G = H / Hkv query heads share one
  int window;             // causal sliding window in keys; 0: none
  int64_t total_len;
  float scale;
  float scale_log2;
  int causal, broadcast_q;
  int P;       // persistent workgroups of the dK/dV kernel (== number of partials)
  int P_dq;    // persistent workgroups of the self-attention dQ kernel
};
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
// Grouped heads: dst[t][g][:] = sum over i < H / Hkv, ascending, of
// src[t][g * (H / Hkv) + i][:] (fp32 rows of d elements).
hipError_t launch_group_sum(const float* src, float* dst, int64_t total_len, int H, int Hkv, int d,
                            hipStream_t stream);
// Exact delta for short sequences, then dK / dV (delta and lse2 must hold the
// pre-pass values).
hipError_t launch_dkdv(const BwdArgs& a, hipStream_t stream);

}  // namespace jfa
