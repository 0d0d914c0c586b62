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

// Workspace carve-up of a decode call (all device pointers) and the plan scalars the split and
// merge kernels share.
//
// Work plan: every (request, kv-head) has a cost sequence -- the step's demote and one-token
// partials (cost step_cost, fused step only), the INT2 history pages (1 each), the INT4 history
// pages (2 each: twice the bytes), the BF16 window as one block (win_cost) -- cut into n_b equal
// cost ranges ("units"), one workgroup each. The kv-heads of a request share its unit count, and
// the counts are apportioned to the requests by cost from the device lengths: n_b = 1 + a share
// of units_per_kv - batch (cumulative rounding, so the shares add up exactly). Unit j of request b
// and kv-head kv is workgroup hkv * (first_b + j) + kv.
struct DecodeWs {
  uint32_t* flags;         // [64]; word 0: bit 0 skipped page id, bit 1 step refused (no room)
  float* part_o;           // [units][3][gq][d]: a unit's window, INT2 and INT4 partials
  float* part_lse;         // [units][3][gq] (log2 units); -inf where the unit has no such segment
  float* step_o;           // [B][Hkv][2][gq][d]: the demoted token (rotated basis), the new token
  float* step_lse;         // [B][Hkv][2][gq]
  int32_t* req_units;      // [B][2]: first unit and unit count of each request (written by the split)
  int units_per_kv;        // workgroups per kv-head (>= batch); grid = hkv * units_per_kv
  int nw;                  // wavefronts per split workgroup
  int step_cost;           // cost of the step segment (0 outside a fused step)
  int win_cost;            // cost of the BF16 window block
  int interleave;          // one request, INT2-only, wide workgroups: unit 0 of each kv-head runs the
                           // step and the window, units 1 .. units_per_kv-1 take the history pages
                           // interleaved (page p: unit 1 + p mod (units_per_kv - 1))
};

// wavefronts of a split workgroup at large batch, and when a few (request, kv-head) pairs must fill
// the chip
#ifndef OSCAR_WIDE_WAVES
#define OSCAR_WIDE_WAVES 16
#endif
constexpr int kSplitWaves = 4;
constexpr int kSplitWavesWide = OSCAR_WIDE_WAVES;
constexpr int kMaxSlots = 3200;  // partial slots per (request, kv-head) of the BF16 baseline

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
  hipEvent_t* events;        // host: optional, 4 events: before the split, the split's start and
                             // stop stamps, after the merge
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
// Split workgroups of `nw` wavefronts a compute unit of the current device holds (0 if unknown).
int split_workgroups_per_cu(int d, int gq, bool cb, bool mixed, int nw);
hipError_t launch_bf16_fill(const Bf16Args& a, hipStream_t stream);
hipError_t launch_bf16_decode(const Bf16Args& a, hipStream_t stream);

}  // namespace oscar
