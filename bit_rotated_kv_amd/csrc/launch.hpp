// Host-side launchers of the OSCAR kernels and the parameter blocks they take. The C ABI in
// api.hip validates arguments and calls these; they only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

// Cache geometry shared by every kernel.
struct Dims {
  int batch, hq, hkv, gq, d, sink, recent, wpages;  // wpages = (sink + recent) / 16
  int mixed;
  int64_t off4;        // first INT4 page id (mixed) / pool_pages (INT2 only)
  int64_t pool_pages;  // valid page ids are [0, pool_pages)
  int max_seq_len;
  int pt_stride;
};

// Workspace carve-up of a decode call (all device pointers).
struct DecodeWs {
  uint32_t* flags;         // [64]; word 0 bit 0: skipped page id
  // query operands, when precomputed (qpre): [width 2, 4][B * Hkv][high, low][gq][d] fp16 and
  // [width][B * Hkv][gq][4] fp32 {sum of high parts, sum of low parts, 2^E, 0}
  uint16_t* qop;
  float* qhs;
  int qpre;
  float* part_o;           // [B][Hkv][NS][gq][d]
  float* part_lse;         // [B][Hkv][NS][gq]  (log2 units)
  // Slots per (b, kv), in order: nwin window slots (one per window workgroup; in a fused step the
  // last is the new token's), S2 INT2 history slots, S4 INT4 history slots, and in a fused step
  // one more history slot for the demoted token. Slots below nwin are in the original basis.
  int ns;
  int nwin;                // window workgroups per (b, kv): ceil(window pages / 4) (+1 in a step)
  int s2, s4;              // split slots per width
  int ppw;                 // pages per wavefront in a history split (4 waves per split), <= 64
};

constexpr int kMaxSlots = 3200;  // history partial slots per (request, kv-head)
// wavefronts of a decode split workgroup (6 was measured slower than 4 at both batch sizes)
constexpr int kSplitWaves = 4;

struct DecodeArgs {
  Dims dm;
  const uint16_t* q;         // [B][Hq][d] bf16
  const int32_t* seq_len;
  const int32_t* n_int4;     // may be null
  const uint8_t* window;
  const uint8_t* pool;
  const int32_t* pt2;
  const int32_t* pt4;
  const float* rot_k;
  const float* rot_v;
  const uint16_t* codebook;  // INT2 codebook table [Hkv][K, V][4] fp16, or null (uniform levels)
  float scale_log2e;         // softmax scale * log2(e)
  float* out;                // [B][Hq][d] fp32
  DecodeWs ws;
  int step;                  // fused decode step: demote + append ride along (CacheWriteArgs)
  hipEvent_t* events;        // host: optional, 4 events: before the query prologue (if any),
                             // before the split, after it, after the merge
};

struct CacheWriteArgs {
  Dims dm;
  const int32_t* seq_len;
  const int32_t* n_int4;
  const uint16_t* k;         // prefill: [B][Hkv][max_seq_len][d]; demote: [B][Hkv][d]
  const uint16_t* v;
  const uint8_t* bits;       // prefill: [B][max_seq_len]; demote: [B]; may be null
  const float* rot_k;
  const float* rot_v;
  float clip_k, clip_v, clip_k4, clip_v4;
  const uint16_t* codebook;  // INT2 codebook table [Hkv][K, V][4] fp16, or null (uniform levels)
  uint8_t* pool;
  const int32_t* pt2;
  const int32_t* pt4;
  uint8_t* window;
  int32_t* seq_len_out;
  int32_t* n_int4_out;
};

struct Bf16Args {
  Dims dm;                   // pool_pages = number of BF16 pages
  const uint16_t* q;
  const int32_t* seq_len;
  const uint16_t* k;         // fill: [B][Hkv][max_seq_len][d]
  const uint16_t* v;
  uint8_t* pages;
  const int32_t* pt;
  float scale_log2e;
  float* out;
  float* part_o;             // [B][Hkv][S][gq][d]
  float* part_lse;           // [B][Hkv][S][gq]
  uint32_t* flags;
  int s, ppw;
};

hipError_t launch_quantize_pack(int64_t rows, int dim, int group, int bits, float clip, const float* x,
                                uint8_t* codes, uint16_t* sz, const uint16_t* levels, hipStream_t stream);
hipError_t launch_prefill(const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_demote(const CacheWriteArgs& a, hipStream_t stream);
// Decode attention; with a.step, also the demote + append of `cw` (a fused decode step).
hipError_t launch_decode(const DecodeArgs& a, const CacheWriteArgs& cw, hipStream_t stream);
hipError_t launch_bf16_fill(const Bf16Args& a, hipStream_t stream);
hipError_t launch_bf16_decode(const Bf16Args& a, hipStream_t stream);

}  // namespace oscar
