/*
 * jfa.h -- C-ABI of the gfx950 (MI355X) jagged flash-attention library,
 * libjfa.so.
 *
 * The operation.  For every sequence b of a packed batch and every head h,
 *     O = softmax(scale * Q K^T) V,   lse = log sum_j exp(scale * (Q K^T)_ij)
 * ("cuTile Kernels -- FMHA Implementation", "Attention Basics"), computed
 * with the online-softmax recurrence ("Flash Attention Algorithm") directly
 * on packed, padding-free K/V addressed through an offsets tensor
 * ("Optimizing Jagged Flash Attention with TLX", "Introduction"), plus the
 * backward pass.  Two modes:
 *   broadcast_q = 1: one dense Q [H, Lq, d] is shared by every sequence, so
 *                    dQ is the sum of the per-sequence dQ over the whole
 *                    batch ("1. The Challenge").
 *   broadcast_q = 0: self-attention; Q is packed like K/V.
 * causal = 1 masks future keys ("Attention Basics"): query i of a sequence
 * sees keys j <= i, positions counted from the start of the sequence
 * (top-left aligned, also when Lq differs from the sequence length).
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers on the current HIP device, and
 *     16-byte aligned.  The caller owns all memory; the library keeps no
 *     pointer after a call returns and never allocates or frees.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without synchronising.  Results are valid once the
 *     stream has executed the work.  Calls that share a workspace must not
 *     overlap.
 *   - bf16 tensors are passed as raw 16-bit storage.  Supported head dims:
 *     d = 64 and d = 128.  B <= 8192 sequences.
 *   - offsets: int64 [B+1], offsets[0] = 0, non-decreasing,
 *     offsets[B] = total_len.  Sequence b owns packed rows
 *     offsets[b] .. offsets[b+1]-1.  It is read on the device only; values
 *     outside [0, total_len] are clamped (the results are then meaningless
 *     but no memory outside the tensors is touched).
 *   - Layouts (row-major, contiguous):
 *       k, v            bf16 [total_len, H, d]
 *       broadcast:  q   bf16 [H, Lq, d]
 *                   out, dout bf16 [B, H, Lq, d];  lse fp32 [B, H, Lq]
 *                   dq  fp32 [H, Lq, d]  (sum over all sequences)
 *       self:       q, out, dout bf16 [total_len, H, d]; lse fp32 [total_len, H]
 *                   dq  fp32 [total_len, H, d]; Lq is ignored
 *       dk, dv          fp32 [total_len, H, d]
 *   - lse is the natural-log log-sum-exp.  A sequence with no keys yields
 *     O = 0, lse = -inf (broadcast mode) and no gradient contribution.
 *   - Every call returns a jfa_status.  Argument errors are detected on the
 *     host before anything is enqueued; JFA_ERR_HIP reports a failed HIP
 *     runtime call or kernel launch.
 *   - Offsets are device data, so their values are not checked by default
 *     (see the clamping above).  With JFA_DEBUG=1 in the environment,
 *     jfa_fwd / jfa_bwd (and the _ex forms) first copy the offsets to the
 *     host, synchronising `stream`, and return JFA_ERR_INVALID_ARG unless
 *     offsets[0] = 0, offsets[b] <= offsets[b+1] and offsets[B] = total_len.
 */
#ifndef JFA_H
#define JFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, non-finite scale */
  JFA_ERR_UNSUPPORTED = 2, /* d not in {64,128}, B above the supported maximum */
  JFA_ERR_WORKSPACE = 3,   /* workspace_bytes smaller than jfa_workspace_size() */
  JFA_ERR_HIP = 4          /* HIP runtime error or failed launch */
} jfa_status;

/* Workspace bytes needed by jfa_fwd (pass = 0) or jfa_bwd (pass = 1) for
 * these sizes (tile lists, per-row scratch of the backward, the broadcast
 * dQ partials; the size depends on the current device's compute-unit
 * count).  Returns 0 for arguments the calls would reject (a valid size is
 * never 0).  No work is enqueued. */
size_t jfa_workspace_size(int64_t total_len, int B, int H, int Lq, int d, int causal, int broadcast_q, int pass);

/* Forward.  Writes out (bf16) and lse (fp32) in the layouts above.
 * Scheduling (sequence sort by length, tile list) runs on the device. */
int jfa_fwd(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int Lq,
            int d, float scale, int causal, int broadcast_q, void* out, float* lse, int64_t total_len,
            void* workspace, size_t workspace_bytes, void* stream);

/* Backward: the exact derivative of the forward, dP = dO V^T,
 * delta = rowsum(dO o O), dS = P o (dP - delta), dQ = scale dS K,
 * dK = scale dS^T Q, dV = P^T dO (five products per K/V block,
 * "Optimizing Jagged Flash Attention with TLX", "2-CTA collaborative MMA";
 * broadcast dQ summed over the batch, "1. The Challenge").  `out` and `lse`
 * must come from jfa_fwd with identical arguments; `dout` is dL/dO.  Writes
 * dq, dk, dv (fp32) in the layouts above.  The result is bitwise
 * reproducible for a given device: every reduction runs in a fixed order
 * (broadcast-mode dQ is summed from per-workgroup partials by a fixed
 * pairwise tree, never by atomics).  |scale| must be at least 2^-100
 * (JFA_ERR_INVALID_ARG otherwise, scale = 0 included): the dK / dV kernel
 * folds -lse / scale into its score products. */
int jfa_bwd(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int Lq,
            int d, float scale, int causal, int broadcast_q, const void* out, const float* lse,
            const void* dout, float* dq, float* dk, float* dv, int64_t total_len, void* workspace,
            size_t workspace_bytes, void* stream);

/* Grouped-query attention and the sliding window ("Optimizing Jagged Flash
 * Attention with TLX", "3. Attention Variants: the flexibility of TLX" and
 * "Conclusion" name both without giving a rule; these are the usual ones).
 *
 * Grouped-query heads: k and v hold H_kv heads, [total_len, H_kv, d], and
 * query head h attends with key/value head h / (H / H_kv), so consecutive
 * query heads share one; dk and dv are [total_len, H_kv, d], each the sum
 * over the H / H_kv query heads of the group.  H_kv must divide H
 * (JFA_ERR_INVALID_ARG otherwise); H_kv = H is plain multi-head attention.
 * With H_kv < H the backward sums each group in a fixed order, so results
 * stay bitwise reproducible: for d = 128 inside the dK / dV kernel (one tile
 * per key / value head walks the group's query heads in ascending order);
 * for d = 64 from per-query-head dK / dV in the workspace
 * (2 * total_len * H * d fp32), summed per group in ascending head order.
 *
 * Sliding window: window = W > 0 (with causal = 1 only; JFA_ERR_UNSUPPORTED
 * otherwise, JFA_ERR_INVALID_ARG for W < 0) lets query i see keys j with
 * i - W < j <= i; window = 0 is no window.  A query row that sees no key
 * (broadcast mode, i - W >= L_b) gives O = 0, lse = -inf and no gradient.
 * Key steps and query blocks wholly outside every row's window are skipped;
 * the steps and blocks that remain take the masked path.
 *
 * jfa_fwd and jfa_bwd above are these with H_kv = H and window = 0.  Every
 * other argument, layout and rule is as above. */
size_t jfa_workspace_size_gqa(int64_t total_len, int B, int H, int H_kv, int Lq, int d, int causal,
                              int broadcast_q, int pass);
int jfa_fwd_ex(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
               int Lq, int d, float scale, int causal, int window, int broadcast_q, void* out, float* lse,
               int64_t total_len, void* workspace, size_t workspace_bytes, void* stream);
int jfa_bwd_ex(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
               int Lq, int d, float scale, int causal, int window, int broadcast_q, const void* out,
               const float* lse, const void* dout, float* dq, float* dk, float* dv, int64_t total_len,
               void* workspace, size_t workspace_bytes, void* stream);

/* MXFP8 forward ("Optimizing Jagged Flash Attention with TLX",
 * "Low-precision (MXFP8) attention": both products take block-scaled FP8
 * operands, E4M3 elements with one E8M0 scale per 32 elements along the
 * product's reduction dimension, and the softmax output P is quantized to
 * FP8 on the fly).  d = 128 only (JFA_ERR_UNSUPPORTED otherwise); no
 * sliding window.  Inputs are uint8 codes (OCP MX formats: E4M3 with bias
 * 7, no infinities, 0x7F / 0xFF NaN; E8M0 code c = 2^(c - 127)):
 *   q8        broadcast [H, Lq, 128], self [total_len, H, 128]   (16-byte aligned)
 *   q_scale   q8's shape with 128 -> 4: block j = elements 32j .. 32j+31 (4-byte aligned)
 *   k8        [total_len, H_kv, 128], k_scale [total_len, H_kv, 4]
 *   vt8       V transposed, [H_kv, 128, T_pad], T_pad = jfa_mxfp8_t_pad(total_len)
 *             (total_len rounded up to 64; columns past total_len are read as
 *             keys of no sequence and may hold anything finite)
 *   vt_scale  [H_kv, T_pad / 32, 128]: one scale per 32 keys of the packed
 *             key index (block j = packed keys 32j .. 32j+31, which may span
 *             two sequences) and head-dim element
 * P is quantized per query row and per 32-key block of that same packed
 * index: with b the block's largest P (keys outside the row's visible set
 * have P = 0), scale 2^(floor(log2 b) - 8), elements P / scale rounded to
 * the nearest E4M3 (ties to even) and capped at 448.  The softmax
 * statistics are not quantized: O = (quantized P) V / l with l the sum of
 * P, and lse = log sum exp(scale * q.k) as in jfa_fwd.  out, lse, offsets,
 * the workspace (jfa_workspace_size_gqa with pass 0), the modes and the
 * error rules are those of jfa_fwd_ex; total_len above 2^26 (T_pad past
 * (2^31 - 1) / 32) returns JFA_ERR_UNSUPPORTED. */
int jfa_fwd_mxfp8(const void* q8, const void* q_scale, const void* k8, const void* k_scale, const void* vt8,
                  const void* vt_scale, const int64_t* offsets, int B, int H, int H_kv, int Lq, int d, float scale,
                  int causal, int broadcast_q, void* out, float* lse, int64_t total_len, void* workspace,
                  size_t workspace_bytes, void* stream);
/* Keys per row of the MXFP8 forward's transposed V for a packed length
 * (total_len rounded up to a multiple of 64, at least 64); -1 if negative.
 * The same rounding gives Lq_pad for the MXFP8 backward's broadcast Q^T. */
int64_t jfa_mxfp8_t_pad(int64_t total_len);

/* MXFP8 backward (the same page gives the variant for both directions):
 * every product takes block-scaled FP8 operands blocked along its own
 * reduction dimension, so each tensor comes in the encodings its products
 * need, and P and dS are quantized on the fly.  With S = scale Q K^T,
 * P = exp(S - lse), dP = dO V^T, delta = rowsum(dO o O), dS = P o (dP - delta):
 *   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K,
 * where S and dP read the row-wise Q, K, dO, V (blocks of 32 along d), dV
 * and dK the query-blocked dO and Q, dQ the key-blocked K; delta uses the
 * row-wise dO and `out` as stored.  P and dS are quantized per key column
 * in blocks of 32 queries for dV and dK, dS per query row in blocks of 32
 * keys of the packed index for dQ, each block with the rule of
 * jfa_fwd_mxfp8 (scale 2^(floor(log2 amax) - 8), nearest E4M3, ties to
 * even, capped at +-448).  d = 128 only; no sliding window.  Inputs (uint8
 * codes; codes 16-byte aligned, scales 4-byte aligned):
 *   q8, q_scale      row-wise Q, as in jfa_fwd_mxfp8
 *   qt8, qt_scale    Q blocked along the queries, transposed:
 *                    broadcast [H, 128, Lq_pad], scales [H, Lq_pad / 32, 128]
 *                    (Lq_pad = jfa_mxfp8_t_pad(Lq), blocks from query 0);
 *                    self [H, 128, T_pad], scales [H, T_pad / 32, 128]
 *                    (blocks of the packed index)
 *   k8, k_scale      row-wise K, as in jfa_fwd_mxfp8
 *   kt8, kt_scale    K blocked along the keys, transposed: [H_kv, 128, T_pad],
 *                    scales [H_kv, T_pad / 32, 128] (the layout of vt8)
 *   v8, v_scale      row-wise V: [total_len, H_kv, 128], [total_len, H_kv, 4]
 *   do8, do_scale    row-wise dO: broadcast [B, H, Lq, 128], [B, H, Lq, 4];
 *                    self [total_len, H, 128], [total_len, H, 4]
 *   dot8, dot_scale  dO blocked along the queries, transposed: broadcast
 *                    [B, H, 128, Lq_pad], [B, H, Lq_pad / 32, 128]; self
 *                    [H, 128, T_pad], [H, T_pad / 32, 128]
 * Padding columns of the transposed encodings may hold anything finite.
 * out (bf16) and lse are the MXFP8 forward's outputs; dq, dk, dv are fp32 in
 * the layouts of jfa_bwd_ex (dk, dv [total_len, H_kv, 128], each summed over
 * its query heads; broadcast dq summed over the sequences).  Any finite scale
 * is accepted.  The workspace is that of jfa_bwd_ex:
 * jfa_workspace_size_gqa(total_len, B, H, H_kv, Lq, 128, causal,
 * broadcast_q, 1) bytes.  Offsets, modes and error rules as in jfa_bwd_ex;
 * the total_len limit of jfa_fwd_mxfp8 applies. */
int jfa_bwd_mxfp8(const void* q8, const void* q_scale, const void* qt8, const void* qt_scale, const void* k8,
                  const void* k_scale, const void* kt8, const void* kt_scale, const void* v8,
                  const void* v_scale, const void* do8, const void* do_scale, const void* dot8,
                  const void* dot_scale, const int64_t* offsets, int B, int H, int H_kv, int Lq, int d,
                  float scale, int causal, int broadcast_q, const void* out, const float* lse, float* dq,
                  float* dk, float* dv, int64_t total_len, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): jfa_fwd_ex without the workspace
 * arguments.  Its scratch (the tile schedule: sort keys, prefix sums, tile
 * list, hand-out counter) is a static device array inside the library, one
 * copy per GPU, JFA_NOALLOC_MAX_WORKSPACE bytes, held until the process
 * ends.  Calls whose forward workspace (jfa_workspace_size_gqa, pass 0)
 * would exceed it return JFA_ERR_WORKSPACE before anything is enqueued.
 * Nothing is allocated or freed and nothing synchronises (JFA_DEBUG's
 * offsets check does not apply here).  Every call on a GPU uses that GPU's
 * one array, and each call rewrites all of the scratch it reads, so calls
 * in sequence on any streams that are ordered are fine; calls that can run
 * concurrently on one GPU (different unsynchronised streams or host
 * threads) race and give wrong results. */
#define JFA_NOALLOC_MAX_WORKSPACE (16u << 20)
int jfa_fwd_noalloc(const void* q, const void* k, const void* v, const int64_t* offsets, int B, int H, int H_kv,
                    int Lq, int d, float scale, int causal, int window, int broadcast_q, void* out, float* lse,
                    int64_t total_len, void* stream);

/* Tile geometry the library uses on the current device for a pass:
 * *block_rows = query rows per forward tile (pass 0) or key rows per
 * backward tile (pass 1); *workers = persistent workgroups that share the
 * tile list.  Host-only. */
int jfa_schedule_params(int pass, int causal, int broadcast_q, int d, int* block_rows, int* workers);

/* Test hooks for the tile schedule ("Optimizing Jagged Flash Attention with
 * TLX", "Scheduling jagged tiles across SMs": sequences sorted by K/V
 * workload, longest first, and tiles handed to the persistent workers in a
 * zigzag).  Each builds a tile list exactly as jfa_fwd / jfa_bwd do and
 * copies it to `tiles` (device int32), in list order; *n_tiles (device
 * int64) receives the full tile count; at most `cap` tiles are written.
 * total_len is offsets[B], passed so that the workspace is sized on the
 * host without reading the offsets.
 *   jfa_debug_schedule: pass 0 = forward query tiles, 1 = backward key
 *     tiles; [cap][4] = b, h, block, worker slot; workspace of that pass.
 *   jfa_debug_schedule_ex: list 0 = forward query tiles, 1 = backward key
 *     tiles as the d = 128 backward builds them (one per key / value head,
 *     h = the group's first query head), 2 = the self-attention backward's
 *     dQ query tiles (broadcast_q = 0 only); H_kv key / value heads as in
 *     jfa_fwd_ex; [cap][5] = b, h, block, key / value head, worker slot;
 *     workspace of the forward (list 0) or backward (lists 1, 2). */
int jfa_debug_schedule(const int64_t* offsets, int B, int H, int Lq, int causal, int broadcast_q,
                       int pass, int64_t total_len, int32_t* tiles, int64_t cap, int64_t* n_tiles,
                       void* workspace, size_t workspace_bytes, void* stream);
int jfa_debug_schedule_ex(const int64_t* offsets, int B, int H, int H_kv, int Lq, int causal, int broadcast_q,
                          int list, int64_t total_len, int32_t* tiles, int64_t cap, int64_t* n_tiles,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing for measurement tools (not thread-safe; host-only
 * bookkeeping).  jfa_timing_enable(capacity) creates 2*capacity hipEvents and
 * from then on brackets every kernel launch of the library with two events
 * on the launch stream (capacity 0 turns timing off and frees the events).
 * At most `capacity` launches are recorded between two reads; later ones are
 * not timed.  jfa_timing_read(kernel, ...) waits for the recorded events,
 * then returns the number of completed launches of kernel number `kernel`
 * (0 <= kernel < the count at which jfa_kernel_name returns NULL) and their
 * summed device time in milliseconds since the last jfa_timing_reset. */
int jfa_timing_enable(int capacity);
int jfa_timing_reset(void);
int jfa_timing_read(int kernel, int64_t* launches, double* total_ms);
const char* jfa_kernel_name(int kernel);

/* Static, human-readable name of a jfa_status value. */
const char* jfa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H */
