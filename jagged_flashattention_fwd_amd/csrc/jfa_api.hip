// Host side of the C-ABI (include/jfa.h): argument checks, workspace
// carving, template dispatch and launches on the caller's stream.  Nothing
// here allocates or frees device memory, and nothing synchronises unless
// JFA_DEBUG=1 asks for the offsets check.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "jfa.h"
#include "jfa_internal.hpp"

namespace jfa {
namespace {

constexpr int MAX_DEVICES = 64;

// Scratch of jfa_fwd_noalloc: the forward's workspace (sort keys, prefix
// sums, tile list, hand-out counter) in a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never uses this name as
// an address: each device's copy is reached through the pointer that
// hipGetSymbolAddress returns at that device's set-up.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)JFA_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

// Per-device set-up, done once per device with that device current: the
// compute-unit count, the kernel attributes the launches rely on, and the
// device address of this device's scratch array.
struct DeviceState {
  int cus = 0;
  int rc = JFA_ERR_HIP;
  char* scratch = nullptr;  // this device's copy of `scratch` (null if the lookup failed)
};
DeviceState g_dev[MAX_DEVICES];
std::once_flag g_dev_once[MAX_DEVICES];

int device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return JFA_ERR_HIP;
  std::call_once(g_dev_once[dev], [dev] {
    DeviceState& st = g_dev[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return;
    if (init_schedule_kernels() != hipSuccess) return;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr != nullptr)
      st.scratch = static_cast<char*>(ptr);
    else
      (void)hipGetLastError();  // only jfa_fwd_noalloc needs it; it reports the failure
    st.cus = n;
    st.rc = JFA_OK;
  });
  *out = &g_dev[dev];
  return g_dev[dev].rc;
}

// Compute units of the current device.
int cu_count(int* out) {
  DeviceState* st = nullptr;
  const int rc = device_state(&st);
  if (rc != JFA_OK) return rc;
  *out = st->cus;
  return JFA_OK;
}

// JFA_DEBUG=1 in the environment: check the offsets tensor on the host
// before launching (one synchronous copy of B + 1 values).
bool debug_checks() {
  static const bool on = [] {
    const char* e = getenv("JFA_DEBUG");
    return e && e[0] == '1';
  }();
  return on;
}

// offsets[0] = 0, non-decreasing, offsets[B] = total_len ("Optimizing Jagged
// Flash Attention with TLX", "Introduction": sequence b owns the packed rows
// offsets[b] .. offsets[b+1]-1).
int check_offsets_sync(const int64_t* offsets, int B, int64_t total_len, hipStream_t st) {
  std::vector<int64_t> h((size_t)B + 1);
  if (hipMemcpyAsync(h.data(), offsets, sizeof(int64_t) * h.size(), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return JFA_ERR_HIP;
  if (h[0] != 0 || h[B] != total_len) return JFA_ERR_INVALID_ARG;
  for (int b = 0; b < B; ++b)
    if (h[b + 1] < h[b]) return JFA_ERR_INVALID_ARG;
  return JFA_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Query rows of a forward tile (8 waves, two per SIMD, in every mode).
int fwd_block_rows() { return FWD_BM; }

// Upper bound on a pass's tile count that needs only host-known sizes:
// sum_b cdiv(L_b, blk) <= cdiv(total_len, blk) + B.
int64_t max_tiles(int pass, int64_t total_len, int B, int H, int Lq, int broadcast_q) {
  if (pass == 0) {
    const int bm = fwd_block_rows();
    if (broadcast_q) return (int64_t)B * H * cdiv(Lq, bm);
    return (int64_t)H * (cdiv(total_len, bm) + B);
  }
  return (int64_t)H * (cdiv(total_len, BWD_BN) + B);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Broadcast-mode dQ work split: n_qb query blocks of DQ_BM_BCAST rows per
// head, and nc sequence chunks, so that H * n_qb * nc fills but does not
// exceed the P compute units (at most 256 chunks, at most B).
void dq_split(int B, int H, int Lq, int P, int* n_qb, int* nc) {
  *n_qb = (int)cdiv(Lq, DQ_BM_BCAST);
  int c = P / (H * *n_qb);
  if (c > B) c = B;
  if (c > 256) c = 256;
  if (c < 1) c = 1;
  *nc = c;
}

struct Layout {
  size_t sched_a[4];  // order, cum, n_tiles, tiles
  size_t sched_b[4];
  int64_t cap_a = 0, cap_b = 0;
  size_t delta = 0, lse2 = 0, term_l = 0, term_d = 0, dq_part = 0;
  size_t dk_heads = 0, dv_heads = 0;  // grouped heads: dK / dV per query head before the group sum
  size_t sched_end = 0;               // end of the tile lists (the layout's first part)
  size_t total = 0;
};

void place_schedule(size_t* at, size_t off[4], int B, int64_t cap) {
  off[0] = *at; *at = align256(*at + sizeof(int) * (size_t)B);
  off[1] = *at; *at = align256(*at + sizeof(int64_t) * ((size_t)B + 1));
  off[2] = *at; *at = align256(*at + 2 * sizeof(int64_t));
  off[3] = *at; *at = align256(*at + sizeof(TileRec) * (size_t)cap);
}

Layout layout(int pass, int64_t total_len, int B, int H, int Hkv, int Lq, int d, int broadcast_q, int P) {
  Layout L;
  size_t at = 0;
  if (pass == 0) {
    L.cap_a = max_tiles(0, total_len, B, H, Lq, broadcast_q);
    place_schedule(&at, L.sched_a, B, L.cap_a);
    L.sched_end = at;
  } else {
    L.cap_a = max_tiles(1, total_len, B, H, Lq, broadcast_q);
    place_schedule(&at, L.sched_a, B, L.cap_a);
    if (!broadcast_q) {
      L.cap_b = max_tiles(0, total_len, B, H, Lq, broadcast_q);
      place_schedule(&at, L.sched_b, B, L.cap_b);
    }
    L.sched_end = at;
    const size_t rows = broadcast_q ? (size_t)B * H * Lq : (size_t)total_len * H;
    L.delta = at; at = align256(at + sizeof(float) * rows);
    L.lse2 = at; at = align256(at + sizeof(float) * rows);
    L.term_l = at; at = align256(at + 16 * rows);
    L.term_d = at; at = align256(at + 16 * rows);
    if (broadcast_q) {
      int n_qb, nc;
      dq_split(B, H, Lq, P, &n_qb, &nc);
      L.dq_part = at;
      at = align256(at + sizeof(float) * (size_t)H * n_qb * nc * DQ_BM_BCAST * d);
    }
    if (Hkv < H && d == 64) {  // d = 128 sums each group inside the dK / dV kernel
      L.dk_heads = at; at = align256(at + sizeof(float) * (size_t)total_len * H * d);
      L.dv_heads = at; at = align256(at + sizeof(float) * (size_t)total_len * H * d);
    }
  }
  L.total = at;
  return L;
}

Schedule schedule_at(char* ws, const size_t off[4], int64_t cap) {
  Schedule s;
  s.order = reinterpret_cast<int*>(ws + off[0]);
  s.cum = reinterpret_cast<int64_t*>(ws + off[1]);
  s.n_tiles = reinterpret_cast<int64_t*>(ws + off[2]);
  s.tiles = reinterpret_cast<TileRec*>(ws + off[3]);
  s.max_tiles = cap;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_sizes(int64_t total_len, int B, int H, int Lq, int d, int broadcast_q) {
  if (B < 1 || H < 1 || total_len < 0) return JFA_ERR_INVALID_ARG;
  if (broadcast_q && Lq < 1) return JFA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return JFA_ERR_UNSUPPORTED;
  if (B > MAX_B) return JFA_ERR_UNSUPPORTED;
  // Row and element indices inside a sequence are 32-bit.
  if (total_len > (int64_t)INT32_MAX || (broadcast_q && (int64_t)Lq * H > (int64_t)INT32_MAX))
    return JFA_ERR_UNSUPPORTED;
  if (H > 65535) return JFA_ERR_UNSUPPORTED;
  return JFA_OK;
}

// Grouped heads: H_kv key / value heads, each shared by H / H_kv query heads.
int check_heads(int H, int Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return JFA_ERR_INVALID_ARG;
  return JFA_OK;
}

// Sliding window: W >= 0 keys (0: none), only with the causal mask.
int check_window(int causal, int window) {
  if (window < 0) return JFA_ERR_INVALID_ARG;
  if (window > 0 && !causal) return JFA_ERR_UNSUPPORTED;
  return JFA_OK;
}

int workers(int pass, int* P) {
  int cus = 0;
  const int rc = cu_count(&cus);
  if (rc != JFA_OK) return rc;
  (void)pass;
  *P = cus;  // one persistent workgroup per compute unit
  return JFA_OK;
}

}  // namespace
}  // namespace jfa

using namespace jfa;

extern "C" {

const char* jfa_status_string(int status) {
  switch (status) {
    case JFA_OK: return "JFA_OK";
    case JFA_ERR_INVALID_ARG: return "JFA_ERR_INVALID_ARG: invalid argument";
    case JFA_ERR_UNSUPPORTED: return "JFA_ERR_UNSUPPORTED: unsupported size or head dim";
    case JFA_ERR_WORKSPACE: return "JFA_ERR_WORKSPACE: workspace too small";
    case JFA_ERR_HIP: return "JFA_ERR_HIP: HIP runtime error";
    default: return "JFA: unknown status";
  }
}

int jfa_schedule_params(int pass, int causal, int broadcast_q, int d, int* block_rows, int* workers_out) {
  if (!block_rows || !workers_out || (pass != 0 && pass != 1)) return JFA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return JFA_ERR_UNSUPPORTED;
  (void)causal;
  (void)broadcast_q;
  *block_rows = pass == 0 ? fwd_block_rows() : BWD_BN;
  return workers(pass, workers_out);
}

size_t jfa_workspace_size_gqa(int64_t total_len, int B, int H, int H_kv, int Lq, int d, int causal,
                              int broadcast_q, int pass) {
  (void)causal;
  if (pass != 0 && pass != 1) return 0;
  if (check_sizes(total_len, B, H, Lq, d, broadcast_q) != JFA_OK || check_heads(H, H_kv) != JFA_OK) return 0;
  int P = 0;
  if (workers(pass, &P) != JFA_OK) return 0;
  return layout(pass, total_len, B, H, H_kv, broadcast_q ? Lq : 0, d, broadcast_q, P).total;
}

size_t jfa_workspace_size(int64_t total_len, int B, int H, int Lq, int d, int causal, int broadcast_q, int pass) {
  return jfa_workspace_size_gqa(total_len, B, H, H, Lq, d, causal, broadcast_q, pass);
}

}  // extern "C"

namespace jfa {
namespace {

// Keys per row of the MXFP8 forward's transposed V: total_len rounded up to
// a whole 64-key step (at least one).
int64_t mxfp8_t_pad(int64_t total_len) { return total_len <= 0 ? 64 : (total_len + 63) / 64 * 64; }

// Argument checks shared by the forward entry points (everything but the
// workspace).
int check_fwd_args(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
                   int Lq, int d, float scale, int causal, int window, int broadcast_q, const void* out,
                   const float* lse, int64_t total_len) {
  if (!q || !k || !v || !offsets || !out || !lse) return JFA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) || (reinterpret_cast<uintptr_t>(offsets) & 7))
    return JFA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return JFA_ERR_INVALID_ARG;
  int rc = check_sizes(total_len, B, H, Lq, d, broadcast_q);
  if (rc != JFA_OK) return rc;
  rc = check_heads(H, H_kv);
  if (rc != JFA_OK) return rc;
  return check_window(causal, window);
}

// The forward's launches on a checked workspace `ws` laid out by `lay`
// (Lq already 0 in self mode).
int fwd_launch(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv, int Lq,
               int d, float scale, int causal, int window, int broadcast_q, void* out, float* lse,
               int64_t total_len, char* ws, const Layout& lay, int P, hipStream_t st) {
  const Schedule s = schedule_at(ws, lay.sched_a, lay.cap_a);
  SchedArgs sa{offsets, total_len, B, H, Lq, broadcast_q ? 1 : 0, 0, fwd_block_rows(), H / H_kv};
  if (launch_schedule(sa, s, st) != hipSuccess) return JFA_ERR_HIP;

  FwdArgs fa;
  fa.q = static_cast<const uint16_t*>(q);
  fa.k = static_cast<const uint16_t*>(k);
  fa.v = static_cast<const uint16_t*>(v);
  fa.offsets = offsets;
  fa.out = static_cast<uint16_t*>(out);
  fa.lse = lse;
  fa.tiles = s.tiles;
  fa.n_tiles = s.n_tiles;
  fa.tile_ctr = reinterpret_cast<unsigned int*>(s.n_tiles + 1);
  fa.total_len = total_len;
  fa.B = B; fa.H = H; fa.Lq = Lq; fa.d = d;
  fa.Hkv = H_kv; fa.G = H / H_kv;
  fa.window = window;
  fa.scale_log2 = scale * 1.4426950408889634f;
  fa.causal = causal ? 1 : 0;
  fa.broadcast_q = broadcast_q ? 1 : 0;
  fa.P = P;
  if (launch_fwd(fa, st) != hipSuccess) return JFA_ERR_HIP;
  return JFA_OK;
}

}  // namespace
}  // namespace jfa

extern "C" {

int jfa_fwd_ex(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
               int Lq, int d, float scale, int causal, int window, int broadcast_q, void* out, float* lse,
               int64_t total_len, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_fwd_args(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse,
                          total_len);
  if (rc != JFA_OK) return rc;
  if (!workspace || !aligned16(workspace)) return JFA_ERR_INVALID_ARG;
  if (!broadcast_q) Lq = 0;
  int P = 0;
  rc = workers(0, &P);
  if (rc != JFA_OK) return rc;
  const Layout lay = layout(0, total_len, B, H, H_kv, Lq, d, broadcast_q, P);
  if (workspace_bytes < lay.total) return JFA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    rc = check_offsets_sync(offsets, B, total_len, st);
    if (rc != JFA_OK) return rc;
  }
  return fwd_launch(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, total_len,
                    static_cast<char*>(workspace), lay, P, st);
}

int jfa_fwd_mxfp8(const void* q8, const void* q_scale, const void* k8, const void* k_scale, const void* vt8,
                  const void* vt_scale, const int64_t* offsets, int B, int H, int H_kv, int Lq, int d, float scale,
                  int causal, int broadcast_q, void* out, float* lse, int64_t total_len, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (!q_scale || !k_scale || !vt_scale) return JFA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q_scale) & 3) || (reinterpret_cast<uintptr_t>(k_scale) & 3) ||
      (reinterpret_cast<uintptr_t>(vt_scale) & 3))
    return JFA_ERR_INVALID_ARG;
  int rc = check_fwd_args(q8, k8, vt8, offsets, B, H, H_kv, Lq, d, scale, causal, 0, broadcast_q, out, lse,
                          total_len);
  if (rc != JFA_OK) return rc;
  if (d != 128) return JFA_ERR_UNSUPPORTED;
  // The MXFP8 kernels bound their copies of transposed rows with 32-bit
  // byte counts of up to 17 rows of T_pad keys.
  if (mxfp8_t_pad(total_len) > (int64_t)(INT32_MAX / 32)) return JFA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace)) return JFA_ERR_INVALID_ARG;
  if (!broadcast_q) Lq = 0;
  int P = 0;
  rc = workers(0, &P);
  if (rc != JFA_OK) return rc;
  const Layout lay = layout(0, total_len, B, H, H_kv, Lq, d, broadcast_q, P);
  if (workspace_bytes < lay.total) return JFA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    rc = check_offsets_sync(offsets, B, total_len, st);
    if (rc != JFA_OK) return rc;
  }
  const Schedule s = schedule_at(static_cast<char*>(workspace), lay.sched_a, lay.cap_a);
  SchedArgs sa{offsets, total_len, B, H, Lq, broadcast_q ? 1 : 0, 0, fwd_block_rows(), H / H_kv};
  if (launch_schedule(sa, s, st) != hipSuccess) return JFA_ERR_HIP;
  FwdMxArgs fa;
  fa.q8 = static_cast<const uint8_t*>(q8);
  fa.q_scale = static_cast<const uint8_t*>(q_scale);
  fa.k8 = static_cast<const uint8_t*>(k8);
  fa.k_scale = static_cast<const uint8_t*>(k_scale);
  fa.vt8 = static_cast<const uint8_t*>(vt8);
  fa.vt_scale = static_cast<const uint8_t*>(vt_scale);
  fa.offsets = offsets;
  fa.out = static_cast<uint16_t*>(out);
  fa.lse = lse;
  fa.tiles = s.tiles;
  fa.n_tiles = s.n_tiles;
  fa.tile_ctr = reinterpret_cast<unsigned int*>(s.n_tiles + 1);
  fa.total_len = total_len;
  fa.t_pad = mxfp8_t_pad(total_len);
  fa.B = B; fa.H = H; fa.Lq = Lq;
  fa.Hkv = H_kv; fa.G = H / H_kv;
  fa.scale_log2 = scale * 1.4426950408889634f;
  fa.causal = causal ? 1 : 0;
  fa.broadcast_q = broadcast_q ? 1 : 0;
  fa.P = P;
  if (launch_fwd_mx(fa, st) != hipSuccess) return JFA_ERR_HIP;
  return JFA_OK;
}

int64_t jfa_mxfp8_t_pad(int64_t total_len) { return total_len < 0 ? -1 : mxfp8_t_pad(total_len); }

int jfa_bwd_mxfp8(const void* q8, const void* q_scale, const void* qt8, const void* qt_scale, const void* k8,
                  const void* k_scale, const void* kt8, const void* kt_scale, const void* v8,
                  const void* v_scale, const void* do8, const void* do_scale, const void* dot8,
                  const void* dot_scale, const int64_t* offsets, int B, int H, int H_kv, int Lq, int d,
                  float scale, int causal, int broadcast_q, const void* out, const float* lse, float* dq,
                  float* dk, float* dv, int64_t total_len, void* workspace, size_t workspace_bytes,
                  void* stream) {
  const void* codes[] = {q8, qt8, k8, kt8, v8, do8, dot8, out, dq, dk, dv, workspace};
  const void* scales[] = {q_scale, qt_scale, k_scale, kt_scale, v_scale, do_scale, dot_scale, lse};
  for (const void* p : codes)
    if (!p || !aligned16(p)) return JFA_ERR_INVALID_ARG;
  for (const void* p : scales)
    if (!p || (reinterpret_cast<uintptr_t>(p) & 3)) return JFA_ERR_INVALID_ARG;
  if (!offsets || (reinterpret_cast<uintptr_t>(offsets) & 7)) return JFA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return JFA_ERR_INVALID_ARG;
  int rc = check_sizes(total_len, B, H, Lq, d, broadcast_q);
  if (rc != JFA_OK) return rc;
  rc = check_heads(H, H_kv);
  if (rc != JFA_OK) return rc;
  if (d != 128) return JFA_ERR_UNSUPPORTED;
  // The MXFP8 kernels bound their copies of transposed rows with 32-bit
  // byte counts of up to 17 rows of T_pad keys.
  if (mxfp8_t_pad(total_len) > (int64_t)(INT32_MAX / 32)) return JFA_ERR_UNSUPPORTED;
  if (!broadcast_q) Lq = 0;
  int P = 0;
  rc = workers(1, &P);
  if (rc != JFA_OK) return rc;
  const Layout lay = layout(1, total_len, B, H, H_kv, Lq, d, broadcast_q, P);
  if (workspace_bytes < lay.total) return JFA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    rc = check_offsets_sync(offsets, B, total_len, st);
    if (rc != JFA_OK) return rc;
  }
  char* ws = static_cast<char*>(workspace);
  const Schedule sk = schedule_at(ws, lay.sched_a, lay.cap_a);
  SchedArgs sa{offsets, total_len, B, H_kv, Lq, broadcast_q ? 1 : 0, 1, MX_BK, H / H_kv};
  sa.kv_tiles = 1;
  if (launch_schedule(sa, sk, st) != hipSuccess) return JFA_ERR_HIP;
  Schedule sq{};
  if (!broadcast_q) {
    sq = schedule_at(ws, lay.sched_b, lay.cap_b);
    SchedArgs sb{offsets, total_len, B, H, Lq, 0, 0, MX_BM, H / H_kv};
    if (launch_schedule(sb, sq, st) != hipSuccess) return JFA_ERR_HIP;
  }
  BwdMxArgs ba;
  ba.q8 = static_cast<const uint8_t*>(q8);
  ba.q_scale = static_cast<const uint8_t*>(q_scale);
  ba.qt8 = static_cast<const uint8_t*>(qt8);
  ba.qt_scale = static_cast<const uint8_t*>(qt_scale);
  ba.k8 = static_cast<const uint8_t*>(k8);
  ba.k_scale = static_cast<const uint8_t*>(k_scale);
  ba.kt8 = static_cast<const uint8_t*>(kt8);
  ba.kt_scale = static_cast<const uint8_t*>(kt_scale);
  ba.v8 = static_cast<const uint8_t*>(v8);
  ba.v_scale = static_cast<const uint8_t*>(v_scale);
  ba.do8 = static_cast<const uint8_t*>(do8);
  ba.do_scale = static_cast<const uint8_t*>(do_scale);
  ba.dot8 = static_cast<const uint8_t*>(dot8);
  ba.dot_scale = static_cast<const uint8_t*>(dot_scale);
  ba.offsets = offsets;
  ba.out = static_cast<const uint16_t*>(out);
  ba.lse = lse;
  ba.dq = dq;
  ba.dk = dk;
  ba.dv = dv;
  ba.delta = reinterpret_cast<float*>(ws + lay.delta);
  ba.lse2 = reinterpret_cast<float*>(ws + lay.lse2);
  ba.dq_part = broadcast_q ? reinterpret_cast<float*>(ws + lay.dq_part) : nullptr;
  ba.seq_order = sk.order;
  ba.dq_qblocks = 0;
  ba.dq_chunks = 0;
  if (broadcast_q) dq_split(B, H, Lq, P, &ba.dq_qblocks, &ba.dq_chunks);
  ba.ktiles = sk.tiles;
  ba.n_ktiles = sk.n_tiles;
  ba.ktile_ctr = reinterpret_cast<unsigned int*>(sk.n_tiles + 1);
  ba.qtiles = broadcast_q ? nullptr : sq.tiles;
  ba.n_qtiles = broadcast_q ? nullptr : sq.n_tiles;
  ba.qtile_ctr = broadcast_q ? nullptr : reinterpret_cast<unsigned int*>(sq.n_tiles + 1);
  ba.total_len = total_len;
  ba.t_pad = mxfp8_t_pad(total_len);
  ba.lq_pad = broadcast_q ? (int)mxfp8_t_pad(Lq) : 0;
  ba.B = B; ba.H = H; ba.Lq = Lq;
  ba.Hkv = H_kv; ba.G = H / H_kv;
  ba.scale = scale;
  ba.scale_log2 = scale * 1.4426950408889634f;
  ba.causal = causal ? 1 : 0;
  ba.broadcast_q = broadcast_q ? 1 : 0;
  ba.P = P;
  if (launch_bwd_mx(ba, st) != hipSuccess) return JFA_ERR_HIP;
  return JFA_OK;
}

int jfa_fwd_noalloc(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
                    int Lq, int d, float scale, int causal, int window, int broadcast_q, void* out, float* lse,
                    int64_t total_len, void* stream) {
  int rc = check_fwd_args(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse,
                          total_len);
  if (rc != JFA_OK) return rc;
  if (!broadcast_q) Lq = 0;
  // The forward's layout does not depend on the worker count: its size is
  // checked against the scratch before any device call.
  const Layout lay = layout(0, total_len, B, H, H_kv, Lq, d, broadcast_q, 1);
  if (lay.total > NOALLOC_SCRATCH_BYTES) return JFA_ERR_WORKSPACE;
  DeviceState* dst = nullptr;
  rc = device_state(&dst);
  if (rc != JFA_OK) return rc;
  if (!dst->scratch) return JFA_ERR_HIP;
  return fwd_launch(q, k, v, offsets, B, H, H_kv, Lq, d, scale, causal, window, broadcast_q, out, lse, total_len,
                    dst->scratch, lay, dst->cus, reinterpret_cast<hipStream_t>(stream));
}

int jfa_fwd(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int Lq,
            int d, float scale, int causal, int broadcast_q, void* out, float* lse, int64_t total_len,
            void* workspace, size_t workspace_bytes, void* stream) {
  return jfa_fwd_ex(q, k, v, offsets, B, H, H, Lq, d, scale, causal, 0, broadcast_q, out, lse, total_len,
                    workspace, workspace_bytes, stream);
}

int jfa_bwd_ex(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
               int Lq, int d, float scale, int causal, int window, int broadcast_q, const void* out,
               const float* lse, const void* dout, float* dq, float* dk, float* dv, int64_t total_len,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !offsets || !out || !lse || !dout || !dq || !dk || !dv || !workspace)
    return JFA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) || (reinterpret_cast<uintptr_t>(offsets) & 7))
    return JFA_ERR_INVALID_ARG;
  // The dK / dV kernel folds -lse / scale into its score products, which
  // needs |scale| >= 2^-100 (then |lse / scale| stays finite in fp32).
  if (!isfinite(scale) || !(fabsf(scale) >= MIN_BWD_SCALE)) return JFA_ERR_INVALID_ARG;
  int rc = check_sizes(total_len, B, H, Lq, d, broadcast_q);
  if (rc != JFA_OK) return rc;
  rc = check_heads(H, H_kv);
  if (rc != JFA_OK) return rc;
  rc = check_window(causal, window);
  if (rc != JFA_OK) return rc;
  if (!broadcast_q) Lq = 0;
  int P = 0;
  rc = workers(1, &P);
  if (rc != JFA_OK) return rc;
  const Layout lay = layout(1, total_len, B, H, H_kv, Lq, d, broadcast_q, P);
  if (workspace_bytes < lay.total) return JFA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (debug_checks()) {
    rc = check_offsets_sync(offsets, B, total_len, st);
    if (rc != JFA_OK) return rc;
  }
  char* ws = static_cast<char*>(workspace);
  const Schedule sk = schedule_at(ws, lay.sched_a, lay.cap_a);
  // Key tiles: d = 128, one per key / value head (its G query heads summed
  // in the dK / dV kernel); d = 64, one per query head.
  const bool kv_tiles = d == 128;
  SchedArgs sa{offsets, total_len, B, kv_tiles ? H_kv : H, Lq, broadcast_q ? 1 : 0, 1, BWD_BN, H / H_kv};
  sa.kv_tiles = kv_tiles ? 1 : 0;
  if (launch_schedule(sa, sk, st) != hipSuccess) return JFA_ERR_HIP;
  Schedule sq{};
  if (!broadcast_q) {
    sq = schedule_at(ws, lay.sched_b, lay.cap_b);
    SchedArgs sb{offsets, total_len, B, H, Lq, 0, 0, DQ_BM, H / H_kv};  // self-attention dQ query tiles
    if (launch_schedule(sb, sq, st) != hipSuccess) return JFA_ERR_HIP;
  }
  BwdArgs ba;
  ba.q = static_cast<const uint16_t*>(q);
  ba.k = static_cast<const uint16_t*>(k);
  ba.v = static_cast<const uint16_t*>(v);
  ba.offsets = offsets;
  ba.out = static_cast<const uint16_t*>(out);
  ba.lse = lse;
  ba.dout = static_cast<const uint16_t*>(dout);
  // Grouped heads at d = 64: the dK / dV kernel writes one slice per query
  // head, summed over each group afterwards.
  const bool grouped = H_kv < H && !kv_tiles;
  ba.dq = dq;
  ba.dk = grouped ? reinterpret_cast<float*>(ws + lay.dk_heads) : dk;
  ba.dv = grouped ? reinterpret_cast<float*>(ws + lay.dv_heads) : dv;
  ba.delta = reinterpret_cast<float*>(ws + lay.delta);
  ba.lse2 = reinterpret_cast<float*>(ws + lay.lse2);
  ba.term_l = reinterpret_cast<uint16_t*>(ws + lay.term_l);
  ba.term_d = reinterpret_cast<uint16_t*>(ws + lay.term_d);
  ba.dq_part = broadcast_q ? reinterpret_cast<float*>(ws + lay.dq_part) : nullptr;
  ba.seq_order = sk.order;
  ba.dq_qblocks = 0;
  ba.dq_chunks = 0;
  if (broadcast_q) dq_split(B, H, Lq, P, &ba.dq_qblocks, &ba.dq_chunks);
  ba.ktiles = sk.tiles;
  ba.n_ktiles = sk.n_tiles;
  ba.ktile_ctr = reinterpret_cast<unsigned int*>(sk.n_tiles + 1);
  ba.qtiles = broadcast_q ? nullptr : sq.tiles;
  ba.n_qtiles = broadcast_q ? nullptr : sq.n_tiles;
  ba.qtile_ctr = broadcast_q ? nullptr : reinterpret_cast<unsigned int*>(sq.n_tiles + 1);
  ba.B = B; ba.H = H; ba.Lq = Lq; ba.d = d;
  ba.Hkv = H_kv; ba.G = H / H_kv;
  ba.window = window;
  ba.total_len = total_len;
  ba.scale = scale;
  ba.scale_log2 = scale * 1.4426950408889634f;
  ba.causal = causal ? 1 : 0;
  ba.broadcast_q = broadcast_q ? 1 : 0;
  ba.P = P;
  ba.P_dq = P;
  if (launch_bwd(ba, st) != hipSuccess) return JFA_ERR_HIP;
  if (grouped) {
    if (launch_group_sum(ba.dk, dk, total_len, H, H_kv, d, st) != hipSuccess) return JFA_ERR_HIP;
    if (launch_group_sum(ba.dv, dv, total_len, H, H_kv, d, st) != hipSuccess) return JFA_ERR_HIP;
  }
  return JFA_OK;
}

int jfa_bwd(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int Lq,
            int d, float scale, int causal, int broadcast_q, const void* out, const float* lse,
            const void* dout, float* dq, float* dk, float* dv, int64_t total_len, void* workspace,
            size_t workspace_bytes, void* stream) {
  return jfa_bwd_ex(q, k, v, offsets, B, H, H, Lq, d, scale, causal, 0, broadcast_q, out, lse, dout, dq, dk,
                    dv, total_len, workspace, workspace_bytes, stream);
}

int jfa_debug_schedule_ex(const int64_t* offsets, int B, int H, int H_kv, int Lq, int causal, int broadcast_q,
                          int list, int64_t total_len, int32_t* tiles, int64_t cap, int64_t* n_tiles,
                          void* workspace, size_t workspace_bytes, void* stream) {
  (void)causal;
  if (!offsets || !tiles || !n_tiles || !workspace || cap < 0 || list < 0 || list > 2)
    return JFA_ERR_INVALID_ARG;
  if (list == 2 && broadcast_q) return JFA_ERR_INVALID_ARG;  // the query-tile list is self-attention only
  // The schedule does not depend on d; the size checks need a supported one.
  int rc = check_sizes(total_len, B, H, Lq, 128, broadcast_q);
  if (rc != JFA_OK) return rc;
  rc = check_heads(H, H_kv);
  if (rc != JFA_OK) return rc;
  if (!broadcast_q) Lq = 0;
  const int pass = list == 0 ? 0 : 1;
  int P = 0;
  rc = workers(pass, &P);
  if (rc != JFA_OK) return rc;
  // The backward's own workspace layout, so that the same workspace serves.
  // Only the tile lists, at the front of the pass's layout, are used here.
  const Layout lay = layout(pass, total_len, B, H, H_kv, Lq, 128, broadcast_q, P);
  if (workspace_bytes < lay.sched_end) return JFA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const Schedule s = list == 2 ? schedule_at(ws, lay.sched_b, lay.cap_b) : schedule_at(ws, lay.sched_a, lay.cap_a);
  const int blk = list == 0 ? fwd_block_rows() : list == 1 ? BWD_BN : DQ_BM;
  // the d = 128 lists: key tiles per key / value head
  SchedArgs sa{offsets, total_len, B, list == 1 ? H_kv : H, Lq, broadcast_q ? 1 : 0, pass, blk, H / H_kv};
  sa.kv_tiles = list == 1 ? 1 : 0;
  if (list == 2) sa.pass = 0;  // query tiles: the forward's per-sequence rule
  if (launch_schedule(sa, s, st) != hipSuccess) return JFA_ERR_HIP;
  if (launch_schedule_dump(s, P, tiles, cap, n_tiles, 5, st) != hipSuccess) return JFA_ERR_HIP;
  return JFA_OK;
}

int jfa_debug_schedule(const int64_t* offsets, int B, int H, int Lq, int causal, int broadcast_q, int pass,
                       int64_t total_len, int32_t* tiles, int64_t cap, int64_t* n_tiles, void* workspace,
                       size_t workspace_bytes, void* stream) {
  (void)causal;
  if (!offsets || !tiles || !n_tiles || !workspace || cap < 0 || (pass != 0 && pass != 1))
    return JFA_ERR_INVALID_ARG;
  int rc = check_sizes(total_len, B, H, Lq, 128, broadcast_q);
  if (rc != JFA_OK) return rc;
  if (!broadcast_q) Lq = 0;
  int P = 0;
  rc = workers(pass, &P);
  if (rc != JFA_OK) return rc;
  const Layout lay = layout(pass, total_len, B, H, H, Lq, 64, broadcast_q, P);
  if (workspace_bytes < lay.total) return JFA_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Schedule s = schedule_at(static_cast<char*>(workspace), lay.sched_a, lay.cap_a);
  SchedArgs sa{offsets, total_len, B, H, Lq, broadcast_q ? 1 : 0, pass,
               pass == 0 ? fwd_block_rows() : BWD_BN, 1};
  if (launch_schedule(sa, s, st) != hipSuccess) return JFA_ERR_HIP;
  if (launch_schedule_dump(s, P, tiles, cap, n_tiles, 4, st) != hipSuccess) return JFA_ERR_HIP;
  return JFA_OK;
}

}  // extern "C"
