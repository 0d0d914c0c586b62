/*
 * oscar.h -- C ABI of the MI355X (gfx950) library for attention-aware INT2 KV caching.
 *
 * The method (OSCAR, as described by the "Together AI open-sources OSCAR" article, the OSCAR
 * overview page and the OSCAR study note): per request the KV cache holds a BF16 sink (first
 * 64 tokens), a BF16 recent window (last 256 tokens, current token included) and, between
 * them, a history whose keys and values are rotated by R = U . H_Had . P_br, clipped,
 * group-quantised to INT2 (4 codes per byte, per-group scale and zero) and paged. Decode
 * attention runs the BF16 and INT2 segments in separate kernels and merges them with an
 * online-softmax (log-sum-exp) combine. A demote kernel moves the oldest recent token into
 * the history each step. A TriAxialKV-style mixed history (TriAxialKV reading note,
 * section 4) adds an INT4 page pool above an address offset and decodes it in
 * bitwidth-homogeneous splits.
 *
 * General contract
 *  - Every pointer argument named *_host is host memory; every other pointer is device memory
 *    on the current HIP device. The caller allocates and owns every buffer. The library never
 *    allocates device memory and keeps no global state (oscar_decode_step_noalloc aside: its
 *    workspace is a fixed array of the library on each device).
 *  - All work is enqueued asynchronously on `stream` (0 = the default stream), and no call
 *    synchronises the stream, with two offline exceptions documented at their declarations:
 *    oscar_codebook_fit (waits for `stream` each iteration) and oscar_rotation_from_covariance
 *    (host computation, no device work).
 *  - Arguments are validated on the host (scalars, null pointers, sizes); on a validation error
 *    nothing is enqueued and a negative status is returned. Device-resident values (lengths,
 *    page ids) are not read by the host: lengths above max_seq_len are clamped, and page ids
 *    outside [0, pool_pages) are skipped (their tokens contribute nothing) and flagged in the
 *    workspace error word (decode) -- they never cause an out-of-bounds access.
 *  - A launch failure reported by HIP returns OSCAR_ERR_LAUNCH.
 *  - Row-vector convention: a key row x is stored rotated as x . R; R is row-major [d][d] fp32.
 *
 * Fixed values of this build: page_size 16 tokens; head_dim 64 or 128; group_size == head_dim
 * in the paged kernels (any divisor of head_dim in oscar_quantize_pack); Hq/Hkv in {1,2,4,8};
 * sink_len and recent_len multiples of 16 with sink_len <= 256, 16 <= recent_len <= 1024.
 *
 * ---------------------------------------------------------------------------------------------
 * Data layouts (all little-endian; "bf16" = IEEE bfloat16 bit pattern)
 *
 * History page ("page-head" = one page of one kv-head; a page holds 16 token slots).
 *   INT2 page-head, d = head_dim: 64 lane chunks of (K: d/16 bytes, then V: d/16 bytes), then
 *   16 x 8 bytes of metadata. Total 4*d*2 + 128 bytes (1152 at d = 128, 640 at d = 64).
 *   INT4 page-head: 64 key parts of d/8 bytes (lane order), then 64 value parts of d/8 bytes,
 *   then 128 bytes of metadata: lane L's key part at byte L*d/8, its value part at (64 + L)*d/8
 *   (so a 16-byte load per lane of either part reads 1 KB of whole lines at d = 128).
 *   Total 4*d*4 + 128 bytes (2176 at d = 128).
 *   A page = num_kv_heads consecutive page-heads. Page id p < int4_page_offset is an INT2 page
 *   at pool + p*P2; page id p >= int4_page_offset is an INT4 page at
 *   pool + int4_page_offset*P2 + (p - int4_page_offset)*P4 (P2, P4 = page bytes). A single
 *   compare of the id decides the width, as in the TriAxialKV dual pool.
 *   Metadata of token slot t (0..15): bf16 {sK, zK, sV, zV} at byte 8*t of the metadata block,
 *   where (s, z) are the group's scale and zero: x_hat = s*code + z (rotated basis).
 *   Codes are 32-bit little-endian words inside each lane's key or value part (word a = bytes
 *   4a..4a+3 of the part):
 *   INT2 key of slot t, channel ch:  kk = ch/32, g = (ch%32)/8, m = (ch%8)/2, hf = ch%2;
 *       lane L = 16*g + t, word a = kk/2, bit 8*(kk%2) + 2*m + 16*hf.
 *   INT2 value of slot t, channel ch: nb = ch/16, c = ch%16, g = t/4, m = (t%4)/2, hf = t%2;
 *       lane L = 16*g + c, word a = nb/4, bit 2*(nb%4) + 8*m + 16*hf.
 *   INT4 key of slot t, channel ch:  kk = ch/32, g = (ch%32)/8, m = (ch%8)/2, hf = ch%2;
 *       lane L = 16*g + t, word a = kk, bit 4*m + 16*hf.
 *   INT4 value of slot t, channel ch: nb = ch/16, c = ch%16, g = t/4, m = (t%4)/2, hf = t%2;
 *       lane L = 16*g + c, word a = nb/2, bit 4*(nb%2) + 8*m + 16*hf.
 *   (These orders put the codes each matrix-core lane needs into its own 16-byte load.)
 *
 * BF16 page-head (sink/recent window, and the full-BF16 baseline cache): 16 tokens of K then V.
 *   K element (t, ch) at bf16 index ((g*16 + t)*(d/32) + kk)*8 + i with kk = ch/32,
 *       g = (ch%32)/8, i = ch%8.
 *   V element (t, ch) at bf16 index 16*d + ((g*16 + c)*(d/16) + nb)*4 + r with nb = ch/16,
 *       c = ch%16, g = t/4, r = t%4.
 *   64*d bytes per page-head (8192 at d = 128).
 *
 * Window (BF16 sink + recent of a batch): [batch][num_kv_heads][W pages][BF16 page-head] with
 *   W = (sink_len + recent_len)/16. Position p < sink_len lives in window page p/16, slot p%16.
 *   Position p >= sink_len lives in ring slot s = p % recent_len: window page
 *   sink_len/16 + s/16, slot s%16. With T tokens in cache the recent window is
 *   [max(sink_len, T - recent_len), T) and the history is [sink_len, T - recent_len).
 *
 * Cache state per request b: seq_len[b] = T (tokens in cache, current token included) and,
 *   for a mixed cache, n_int4[b] = number of history tokens stored at 4 bits. History slot k of
 *   width w lives in page table[b*pt_stride + k/16] (INT2: page_table, INT4: page_table4),
 *   slot k%16. INT2 history count = max(0, T - sink_len - recent_len) - n_int4[b].
 * ---------------------------------------------------------------------------------------------
 */
#ifndef OSCAR_H_
#define OSCAR_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  OSCAR_OK = 0,
  OSCAR_ERR_INVALID_ARG = -1, /* null pointer, out-of-range scalar, inconsistent sizes      */
  OSCAR_ERR_UNSUPPORTED = -2, /* valid request this build does not implement (e.g. d=96)    */
  OSCAR_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required            */
  OSCAR_ERR_LAUNCH = -4       /* a kernel launch failed (hipGetLastError after the launch)  */
} oscar_status_t;

/* Shape and policy of one attention layer's cache. */
typedef struct oscar_layout {
  int32_t num_q_heads;      /* Hq                                                            */
  int32_t num_kv_heads;     /* Hkv; query head h reads kv-head h / (Hq/Hkv)                  */
  int32_t head_dim;         /* d: 64 or 128                                                  */
  int32_t group_size;       /* quantisation group along head_dim (== head_dim when paged)    */
  int32_t sink_len;         /* BF16 sink tokens (64)                                         */
  int32_t recent_len;       /* BF16 recent window tokens (256)                               */
  int32_t page_size;        /* tokens per page: must be 16                                   */
  int32_t mixed;            /* 0: INT2 history only; 1: INT2 + INT4 pools                    */
  int64_t int4_page_offset; /* mixed: page ids >= this are INT4 pages                        */
  int64_t pool_pages;       /* number of valid page ids in the pool arena                    */
  float clip_k, clip_v;     /* INT2 clip ratios c_K, c_V (study note, case 2: 0.96, 0.92)    */
  float clip_k4, clip_v4;   /* INT4 clip ratios (1.0: no clipping)                           */
  /* INT2 Lloyd-Max codebooks (OSCAR overview page, the paragraph that sets OSCAR beside
   * TurboQuant): NULL for the uniform levels 0..3, else a device table [Hkv][2][4] of fp16
   * patterns (K levels, then V levels, per kv-head), 4-byte aligned, each row four finite,
   * strictly increasing levels l_0 < l_1 < l_2 < l_3 (the library reads it on the device and
   * cannot check that; other contents give meaningless codes, never a fault). A group
   * coordinate u = (clip(x) - z)/s gets code [u > t_0] + [u >= t_1] + [u > t_2] with
   * t_j = (l_j + l_{j+1})/2 (fp32), and restores as z + s*l[code]. INT4 tokens keep the
   * uniform levels. Owned by the caller; read by prefill, demote, decode and step. */
  const uint16_t* codebook;
} oscar_layout_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* oscar_status_string(oscar_status_t status);

/* Library version string. */
const char* oscar_version(void);

/* Byte sizes of the layouts above; 0 if the layout is invalid. */
size_t oscar_page_bytes(const oscar_layout_t* layout, int32_t bits);   /* bits: 2, 4 or 16 */
size_t oscar_window_bytes(const oscar_layout_t* layout, int32_t batch);
size_t oscar_pool_bytes(const oscar_layout_t* layout);                  /* whole arena        */

/*
 * Group quantise already-rotated fp32 rows (the bit-exact parity surface; OSCAR overview page,
 * method paragraph; clip constants from the study note, case 2).
 *   x           [rows][dim] fp32 (device)
 *   codes       [rows][dim*bits/8] bytes, canonical order: code i of a row at byte i/(8/bits),
 *               bits (i%(8/bits))*bits (LSB first)
 *   scale_zero  [rows][dim/group][2] bf16 patterns (s, z)
 * Per group: lo = clip*min, hi = clip*max (fp32), s = bf16(fp32(hi-lo)/(2^bits-1)),
 * z = bf16(lo), code = clamp(rint_even(fp32(fp32(clamp(x,lo,hi) - z)/s)), 0, 2^bits-1), and all
 * codes 0 when s == 0. bits in {2, 4}; group divides dim; dim <= 1024; 0 < clip <= 1.
 */
oscar_status_t oscar_quantize_pack(int64_t rows, int32_t dim, int32_t group, int32_t bits,
                                   float clip, const float* x, uint8_t* codes,
                                   uint16_t* scale_zero, hipStream_t stream);

/*
 * INT2 group quantise + pack of already-rotated fp32 rows with a Lloyd-Max codebook (OSCAR
 * overview page, the paragraph that sets OSCAR beside TurboQuant): the grid (s, z) and the
 * packing of oscar_quantize_pack with bits = 2; the code of a coordinate
 * u = fp32(fp32(clamp(x,lo,hi) - z)/s) is [u > t_0] + [u >= t_1] + [u > t_2] with
 * t_j = (l_j + l_{j+1})/2 in fp32 (the nearest level, ties to the even code); all codes 0 when
 * s == 0. levels: host array of four fp16 patterns, finite and strictly increasing (else
 * OSCAR_ERR_INVALID_ARG). The levels 0, 1, 2, 3 give exactly oscar_quantize_pack's codes.
 */
oscar_status_t oscar_quantize_pack_codebook(int64_t rows, int32_t dim, int32_t group, float clip,
                                            const float* x, const uint16_t* levels, uint8_t* codes,
                                            uint16_t* scale_zero, hipStream_t stream);

/*
 * Lloyd-Max fit of INT2 codebooks on the GPU (OSCAR overview page, the paragraph that sets OSCAR
 * beside TurboQuant; Lloyd-Max after Max, 1960). For each kv-head h the calibration rows
 * x[h] ([n_rows][head_dim] bf16, device) are rotated by rot[h] ([head_dim][head_dim] fp32,
 * device) exactly as the cache writers rotate a token, each row gets the INT2 grid with `clip`
 * (group = head_dim), and the coordinates u = fp32(fp32(clamp(x,lo,hi) - z)/s) of every channel
 * (rows with s == 0 are left out) are the samples. Starting from the levels 0, 1, 2, 3, each
 * iteration puts thresholds at the midpoints of the levels (fp64), assigns every sample to the
 * nearest level (on a threshold: the even level) and moves each level to its cell mean (fp64; an
 * empty cell keeps its level); a kv-head stops after the first iteration in which no level moved
 * by more than `tol`, or after max_iter iterations.
 *   levels_out    host [Hkv][4] fp64 fitted levels
 *   patterns_out  host [Hkv][4] their fp16 patterns (round to nearest even): one half of a codebook
 *                 table row (fit K with rot_k, clip_k and V with rot_v, clip_v)
 *   iters_out     host [Hkv] iterations run (may be NULL)
 * Synchronous: returns after `stream` has drained (each iteration copies its partial sums back).
 * Workspace: oscar_codebook_workspace_bytes(num_kv_heads, n_rows, head_dim) bytes of device memory.
 * head_dim in {64, 128}; n_rows >= 0 (0: the uniform levels come back); max_iter >= 1; tol >= 0.
 */
size_t oscar_codebook_workspace_bytes(int32_t num_kv_heads, int32_t n_rows, int32_t head_dim);
oscar_status_t oscar_codebook_fit(int32_t num_kv_heads, int32_t n_rows, int32_t head_dim, const void* x,
                                  const float* rot, float clip, int32_t max_iter, double tol,
                                  void* workspace, size_t workspace_bytes, double* levels_out,
                                  uint16_t* patterns_out, int32_t* iters_out, hipStream_t stream);

/*
 * Build the cache of a batch from full prefixes (prefill): writes the sink and recent windows
 * into `window` and rotates (K by rot_k, V by rot_v), clips, quantises and packs every history
 * token into its page (OSCAR overview page, method paragraph; news article, cache layout).
 *   seq_len      [batch] int32, T of each request (<= max_seq_len)
 *   k, v         [batch][Hkv][max_seq_len][d] bf16, positions 0..T-1 used
 *   token_bits   [batch][max_seq_len] uint8 (2 or 4), width of each history token (mixed
 *                caches only; NULL = all INT2). INT2 and INT4 tokens take consecutive slots
 *                of their own page tables in position order.
 *   rot_k, rot_v [Hkv][d][d] fp32
 *   page_table   [batch][pt_stride] int32 INT2 history pages; page_table4 the INT4 pages
 *                (mixed only, else may be NULL)
 *   n_int4_out   [batch] int32 written with the INT4 history count (may be NULL)
 */
oscar_status_t oscar_kv_prefill(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                                const int32_t* seq_len, const void* k, const void* v,
                                const uint8_t* token_bits, const float* rot_k, const float* rot_v,
                                void* pool, const int32_t* page_table, const int32_t* page_table4,
                                int32_t pt_stride, void* window, int32_t* n_int4_out,
                                hipStream_t stream);

/*
 * One decode step's cache update for every request (OSCAR overview page, method paragraph;
 * study note, SGLang case): with T = seq_len[b], if T >= sink_len + recent_len the oldest recent
 * token (position T - recent_len) is read from the window, rotated, clipped, quantised, packed
 * into the next history slot of its width (demote_bits[b], 2 if NULL) and the new token
 * (new_k/new_v [batch][Hkv][d] bf16) is written into the freed recent slot; otherwise the new
 * token is written at position T of the window. seq_len_out[b] = T + 1 and
 * n_int4_out[b] = n_int4[b] + (width == 4) are written when the pointers are not NULL; they
 * must not alias seq_len / n_int4. n_int4 may be NULL for an INT2-only cache.
 */
oscar_status_t oscar_kv_demote(const oscar_layout_t* layout, int32_t batch, const int32_t* seq_len,
                               const int32_t* n_int4, const void* new_k, const void* new_v,
                               const uint8_t* demote_bits, const float* rot_k, const float* rot_v,
                               void* pool, const int32_t* page_table, const int32_t* page_table4,
                               int32_t pt_stride, void* window, int32_t* seq_len_out,
                               int32_t* n_int4_out, hipStream_t stream);

/* Workspace bytes oscar_decode_attn needs for this batch and length bound. */
size_t oscar_decode_workspace_bytes(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len);

/*
 * Decode attention over the three-segment cache (OSCAR overview page, method paragraph; news
 * article, key/value rotations): for query head h of request b, logits are
 * softmax_scale*q.k over the BF16 sink/recent tokens and softmax_scale*(q.R_K).x_hat over
 * history tokens; one softmax over all of them; out = sum_BF16 p v + (sum_hist p x_hat_V).R_V^T.
 * Computed as bitwidth-homogeneous splits (BF16 / INT2 / INT4 pages) with fp32 accumulation,
 * merged by log-sum-exp (one merge workgroup per request and kv-head).
 *   q          [batch][Hq][d] bf16
 *   out        [batch][Hq][d] fp32
 *   softmax_scale 0 -> 1/sqrt(d)
 *   workspace  >= oscar_decode_workspace_bytes(); word 0 (uint32) is OR-ed with 1 when a page
 *              id outside [0, pool_pages) was skipped (the caller clears it). Contents are scratch between calls; calls
 *              that overlap in time must not share a workspace.
 *   Page tables are read only at indices below pt_stride (longer histories are cut there).
 */
oscar_status_t oscar_decode_attn(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                                 const void* q, const int32_t* seq_len, const int32_t* n_int4,
                                 const void* window, const void* pool, const int32_t* page_table,
                                 const int32_t* page_table4, int32_t pt_stride,
                                 const float* rot_k, const float* rot_v, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, float* out,
                                 hipStream_t stream);

/*
 * oscar_decode_attn with timing: identical work, plus events[0..3] (n_events >= 4, all created by
 * the caller): events[0] recorded on `stream` before the split kernel (BF16 window, INT2 and INT4
 * history pages in one launch), events[1] and events[2] stamped by the runtime at that kernel's
 * start and end (hipExtLaunchKernel), events[3] recorded after the merge kernel. events[1..2] time
 * the split kernel alone, events[2..3] the merge (with the gap between the launches).
 */
oscar_status_t oscar_decode_attn_profiled(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                                          const void* q, const int32_t* seq_len, const int32_t* n_int4,
                                          const void* window, const void* pool, const int32_t* page_table,
                                          const int32_t* page_table4, int32_t pt_stride, const float* rot_k,
                                          const float* rot_v, float softmax_scale, void* workspace,
                                          size_t workspace_bytes, float* out, hipEvent_t* events,
                                          int32_t n_events, hipStream_t stream);

/*
 * One whole decode step (OSCAR overview page, method paragraph; study note, SGLang case): the
 * cache update of oscar_kv_demote (new_k/new_v appended, the oldest recent token demoted) and the
 * attention of oscar_decode_attn over the updated cache, in the same kernels (split and merge,
 * one launch each). The cache after the call -- pool, window, seq_len_out, n_int4_out (both outputs required here, not
 * aliasing the inputs) -- is bit for bit what the two calls in sequence leave. The attention is
 * the same function of the updated cache; it reads the cache as it stands before the step and
 * takes the demoted token (same codes as the demote writes) and the new token as one-token
 * partials, so its output agrees with the two-call sequence to fp32 rounding, not bit for bit.
 * Arguments follow the two calls above; max_seq_len bounds the updated lengths (T + 1). A request
 * with no room for the new token (seq_len >= max_seq_len) is left as it is -- no demote, no
 * append, seq_len_out = seq_len -- attends over its cache with its lengths cut to max_seq_len, and
 * sets bit 1 of workspace word 0.
 */
oscar_status_t oscar_decode_step(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                                 const int32_t* seq_len, const int32_t* n_int4, const void* new_k,
                                 const void* new_v, const uint8_t* demote_bits, const void* q,
                                 const float* rot_k, const float* rot_v, void* pool,
                                 const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                 void* window, int32_t* seq_len_out, int32_t* n_int4_out,
                                 float softmax_scale, void* workspace, size_t workspace_bytes, float* out,
                                 hipStream_t stream);

/*
 * oscar_decode_step with timing: identical work, plus hipEventRecord on `stream` of events[0..3]
 * (n_events >= 4, created by the caller), placed as in oscar_decode_attn_profiled.
 */
oscar_status_t oscar_decode_step_profiled(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                                          const int32_t* seq_len, const int32_t* n_int4, const void* new_k,
                                          const void* new_v, const uint8_t* demote_bits, const void* q,
                                          const float* rot_k, const float* rot_v, void* pool,
                                          const int32_t* page_table, const int32_t* page_table4,
                                          int32_t pt_stride, void* window, int32_t* seq_len_out,
                                          int32_t* n_int4_out, float softmax_scale, void* workspace,
                                          size_t workspace_bytes, float* out, hipEvent_t* events,
                                          int32_t n_events, hipStream_t stream);

/* Bytes of the library-held workspace of oscar_decode_step_noalloc (per device). */
#define OSCAR_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): oscar_decode_step with the same arguments and results
 * but no workspace argument. Its workspace is a device array of OSCAR_NOALLOC_SCRATCH_BYTES held by
 * the library on each device it runs on until the process ends; the call allocates nothing.
 *   Rejected with OSCAR_ERR_WORKSPACE (before any device work) when
 *   oscar_decode_workspace_bytes(layout, batch, max_seq_len) > OSCAR_NOALLOC_SCRATCH_BYTES (for
 *   d = 128, 32 query and 8 kv heads: batch up to 256 at any length).
 *   Every call on a device shares that device's array and leaves its contents behind; nothing in
 *   it needs to start at zero. Calls that overlap in time on one device race (one stream, or
 *   ordered streams, per device). The report word of the workspace (skipped page id, no room) is
 *   not returned here; a request left without room still shows as seq_len_out = seq_len.
 *   The first call on a device looks up the array's device address (hipGetSymbolAddress) with
 *   that device current; OSCAR_ERR_LAUNCH if that fails.
 */
oscar_status_t oscar_decode_step_noalloc(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                                         const int32_t* seq_len, const int32_t* n_int4, const void* new_k,
                                         const void* new_v, const uint8_t* demote_bits, const void* q,
                                         const float* rot_k, const float* rot_v, void* pool,
                                         const int32_t* page_table, const int32_t* page_table4,
                                         int32_t pt_stride, void* window, int32_t* seq_len_out,
                                         int32_t* n_int4_out, float softmax_scale, float* out,
                                         hipStream_t stream);

/*
 * In-house BF16 baseline: the full context of each request in BF16 pages (BF16 page-head
 * layout; page = Hkv page-heads, page ids index `pages`). Writes every position of k/v
 * ([batch][Hkv][max_seq_len][d] bf16, T = seq_len[b]) into the pages of `page_table`.
 */
oscar_status_t oscar_bf16_fill(const oscar_layout_t* layout, int32_t batch, int32_t max_seq_len,
                               const int32_t* seq_len, const void* k, const void* v, void* pages,
                               int64_t num_pages, const int32_t* page_table, int32_t pt_stride,
                               hipStream_t stream);

/* Workspace bytes for oscar_bf16_decode_attn. */
size_t oscar_bf16_decode_workspace_bytes(const oscar_layout_t* layout, int32_t batch,
                                         int32_t max_seq_len);

/*
 * In-house BF16 decode attention (the speed-up denominator): plain softmax(scale q K^T) V over
 * all T tokens of each request from a full-BF16 paged cache, split-K with a log-sum-exp merge.
 * Same q/out/workspace conventions as oscar_decode_attn; ids outside [0, num_pages) skipped.
 */
oscar_status_t oscar_bf16_decode_attn(const oscar_layout_t* layout, int32_t batch,
                                      int32_t max_seq_len, const void* q, const int32_t* seq_len,
                                      const void* pages, int64_t num_pages,
                                      const int32_t* page_table, int32_t pt_stride,
                                      float softmax_scale, void* workspace, size_t workspace_bytes,
                                      float* out, hipStream_t stream);

/* ------------------------------------------------------------------ TriAxialKV bit allocation */

/* Allocation methods of oscar_allocate_bits. */
enum { OSCAR_ALLOC_GREEDY = 0, OSCAR_ALLOC_EXHAUSTIVE = 1 };

/*
 * INT2/INT4 width per tag class (TriAxialKV reading note, section 3): minimise
 * sum_k D_k(b_k) subject to sum_k N_k b_k <= budget_bits * sum_k N_k, b_k in {2, 4}. Host
 * function: every pointer is host memory and nothing is enqueued on a device.
 *   d2, d4       [n_classes] distortion of class k at 2 and at 4 bits (finite)
 *   counts       [n_classes] tokens of class k (0 .. 2^50)
 *   budget_bits  average bits per element the allocation may spend (>= 2)
 *   method       OSCAR_ALLOC_GREEDY: raise classes from 2 to 4 bits in descending order of the
 *                gain per extra bit rho_k = (D_k(2) - D_k(4)) / (2 N_k) (ties: lower class index
 *                first); classes without a positive gain or without tokens stay at 2; the first
 *                class whose raise would exceed the budget ends it.
 *                OSCAR_ALLOC_EXHAUSTIVE: the least total distortion over all 2^n_classes choices
 *                that meet the budget (n_classes <= 24, else OSCAR_ERR_UNSUPPORTED); among equal
 *                costs any one is returned.
 *   bits_out     [n_classes] written with 2 or 4
 *   cost_out     optional: sum_k D_k(bits_out[k])
 * The budget test allows 1e-9 bits of slack for the rounding of budget_bits * sum N_k.
 */
oscar_status_t oscar_allocate_bits(int32_t n_classes, const double* d2, const double* d4,
                                   const int64_t* counts, double budget_bits, int32_t method,
                                   uint8_t* bits_out, double* cost_out);

/*
 * Token widths from tag classes (TriAxialKV reading note, sections 3-4: the class allocation
 * routes every token to the INT2 or the INT4 pool): token_bits[b][t] = class_bits[tags[b][t]]
 * for t < seq_len[b] (device arrays [batch][max_seq_len]; positions at or past seq_len[b] are
 * not written). A tag outside [0, n_classes) routes to 2 bits. class_bits is a host array of
 * n_classes <= 64 entries, each 2 or 4, copied into the launch. The result feeds the
 * token_bits argument of oscar_kv_prefill.
 */
oscar_status_t oscar_route_tokens(int32_t batch, int32_t max_seq_len, const int32_t* seq_len,
                                  const int32_t* tags, int32_t n_classes, const uint8_t* class_bits,
                                  uint8_t* token_bits, hipStream_t stream);

/* ------------------------------------------------------------------ calibration statistics */

/*
 * Workspace bytes of the calibration calls for n_rows calibration queries per query head
 * (n_tokens of oscar_calib_query_cov, n_queries of oscar_calib_value_cov).
 */
size_t oscar_calib_workspace_bytes(int32_t num_kv_heads, int32_t gq, int32_t n_rows, int32_t head_dim);

/*
 * Query covariance of every kv-head ("Together AI open-sources OSCAR", section on what makes OSCAR
 * different): cov[kv] = (1/N) sum_h sum_n q^T q over the gq query heads of the kv-head and the
 * N = n_tokens calibration queries of each. Its eigenvectors (descending eigenvalues) are U_Q of
 * R_K = U_Q . H . P_br (the eigendecomposition is a host step).
 *   q     [num_kv_heads][gq][n_tokens][head_dim] bf16 (device)
 *   cov   [num_kv_heads][head_dim][head_dim] fp32 (device)
 * bf16 products are exact on the matrix cores; sums are fp32, in a fixed order (deterministic).
 * head_dim 64 or 128.
 */
oscar_status_t oscar_calib_query_cov(int32_t num_kv_heads, int32_t gq, int32_t n_tokens, int32_t head_dim,
                                     const void* q, void* workspace, size_t workspace_bytes, float* cov,
                                     hipStream_t stream);

/*
 * Score-weighted value covariance (same section): cov[kv] = (1/N) sum_h (S_h V)^T (S_h V) with
 * S_h = softmax(scale q_h K^T) over a calibration context (rows over its n_ctx keys), for the
 * N = n_queries calibration queries of each of the gq heads. Eigenvectors give U_S of R_V.
 *   q     [num_kv_heads][gq][n_queries][head_dim] bf16; k, v [num_kv_heads][n_ctx][head_dim] bf16
 *   softmax_scale 0 -> 1/sqrt(head_dim)
 *   cov   [num_kv_heads][head_dim][head_dim] fp32
 * S V is formed in fp32 (probabilities enter the product as bf16 high + low parts) and its Gram
 * matrix from bf16 high + low parts of each element (about 16 significant bits).
 */
oscar_status_t oscar_calib_value_cov(int32_t num_kv_heads, int32_t gq, int32_t n_queries, int32_t n_ctx,
                                     int32_t head_dim, const void* q, const void* k, const void* v,
                                     float softmax_scale, void* workspace, size_t workspace_bytes, float* cov,
                                     hipStream_t stream);

/*
 * Rotations from covariances ("Together AI open-sources OSCAR", section on what makes OSCAR
 * different): for each of n_mats symmetric matrices C (C_Q for R_K, C_S for R_V) forms
 * R = U . H . P_br, where U holds the eigenvectors of C as columns in descending eigenvalue
 * order, each column's largest-magnitude entry (the first, on ties) made positive; H is the
 * orthonormal Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H, H], [H, -H]], scaled by
 * 1/sqrt(d)) and P_br the bit-reversal permutation with P[i, rev(i)] = 1, so that
 * R[i][j] = sum_k U[i][k] H[k][rev(j)]. Host function: every pointer is host memory, nothing is
 * enqueued on a device. The eigenvectors come from the cyclic Jacobi method in fp64 on the
 * symmetric part (C + C^T)/2 of each input; R is formed in fp64 and rounded once to fp32.
 *   cov_host      [n_mats][d][d] fp64, finite (else OSCAR_ERR_INVALID_ARG)
 *   rot_host      [n_mats][d][d] fp32 out, row-major (a row x is rotated as x . R)
 *   eigvals_host  [n_mats][d] fp64 out, descending (may be NULL)
 *   eigvecs_host  [n_mats][d][d] fp64 out, U row-major (eigenvector j in column j; may be NULL)
 * head_dim: a power of two, at most 256 (larger: OSCAR_ERR_UNSUPPORTED). Synchronous, about
 * 0.1 s per matrix at d = 128.
 */
oscar_status_t oscar_rotation_from_covariance(int32_t n_mats, int32_t head_dim, const double* cov_host,
                                              float* rot_host, double* eigvals_host, double* eigvecs_host);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H_ */
