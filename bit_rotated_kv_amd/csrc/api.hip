// C ABI of the OSCAR gfx950 library (declared and documented in include/oscar.h): host-side
// validation, workspace planning and kernel launches. Nothing here touches device memory.
#include <math.h>
#include <algorithm>
#include <string.h>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

using namespace oscar;

namespace {

// Upper bound of the decode split's workgroups per kv-head (besides one per request): the plan
// shares this many out at most, so the workspace size does not depend on the device.
constexpr int kMaxUnits = 2048;
// Wide split workgroups (16 wavefronts) are used for GQA width 4 when this few (request, kv-head)
// pairs would otherwise give each compute unit two or fewer 4-wavefront workgroups.
#ifndef OSCAR_WIDE_MAX_GROUPS
#define OSCAR_WIDE_MAX_GROUPS 16
#endif
constexpr int kWideMaxGroups = OSCAR_WIDE_MAX_GROUPS;
// Plan costs: an INT2 history page costs 1, an INT4 page 2 (in the kernels); the step and the BF16
// window are chains of latencies and cost about the pages their workgroup streams meanwhile.
// Per-workgroup timelines of one 100K-token request (16-wavefront workgroups streaming ~19 pages
// per us): the window segment takes ~6 us and its unit then ends ~1 us after the history-only
// units of its compute die, the step unit ~0.3 us after; a sweep of the two costs put the split's
// end lowest at 200 (step) and 150 (window). 4-wavefront workgroups stream ~6-7 pages per us.
#ifndef OSCAR_STEP_COST_WIDE
#define OSCAR_STEP_COST_WIDE 200
#endif
#ifndef OSCAR_WIN_COST_WIDE
#define OSCAR_WIN_COST_WIDE 150
#endif
#ifndef OSCAR_STEP_COST
#define OSCAR_STEP_COST 64
#endif
#ifndef OSCAR_WIN_COST
#define OSCAR_WIN_COST 96
#endif
int step_cost(int nw) { return nw >= kSplitWavesWide ? OSCAR_STEP_COST_WIDE : OSCAR_STEP_COST; }
int window_cost(int nw) { return nw >= kSplitWavesWide ? OSCAR_WIN_COST_WIDE : OSCAR_WIN_COST; }

// Smallest unit the plan aims for (cost of 16 INT2 pages): below it the per-workgroup overhead (query
// prologue, workgroup merge, one more partial to merge) outweighs the spread.
constexpr int kMinUnitCost = 16;
// Interleaved one-request plan: its unit 0 runs the step and window (together ~7 us), so the
// history units should stream at least this many pages each for it to pay off.
constexpr int kInterleaveMinPages = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

oscar_status_t check_layout(const oscar_layout_t* L) {
  if (!L) return OSCAR_ERR_INVALID_ARG;
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0 || L->num_q_heads % L->num_kv_heads) return OSCAR_ERR_INVALID_ARG;
  if (L->head_dim <= 0 || L->group_size <= 0 || L->head_dim % L->group_size) return OSCAR_ERR_INVALID_ARG;
  if (L->sink_len < 0 || L->recent_len <= 0 || L->page_size <= 0) return OSCAR_ERR_INVALID_ARG;
  if (L->mixed != 0 && L->mixed != 1) return OSCAR_ERR_INVALID_ARG;
  if (L->pool_pages < 0) return OSCAR_ERR_INVALID_ARG;
  if (L->mixed && (L->int4_page_offset < 0 || L->int4_page_offset > L->pool_pages)) return OSCAR_ERR_INVALID_ARG;
  const float clips[4] = {L->clip_k, L->clip_v, L->clip_k4, L->clip_v4};
  for (float c : clips)
    if (!(c > 0.0f && c <= 1.0f)) return OSCAR_ERR_INVALID_ARG;
  const int gq = L->num_q_heads / L->num_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return OSCAR_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return OSCAR_ERR_UNSUPPORTED;
  if (L->group_size != L->head_dim) return OSCAR_ERR_UNSUPPORTED;
  if (L->page_size != kPage) return OSCAR_ERR_UNSUPPORTED;
  if (L->sink_len % kPage || L->recent_len % kPage || L->sink_len > 256 || L->recent_len > 1024)
    return OSCAR_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(L->codebook) % 4) return OSCAR_ERR_INVALID_ARG;
  return OSCAR_OK;
}

// Four finite, strictly increasing fp16 levels.
bool levels_ok(const uint16_t* levels) {
  if (!levels) return false;
  float prev = -__builtin_huge_valf();
  for (int j = 0; j < 4; ++j) {
    const float l = host_f16_to_f32(levels[j]);
    if (!(l > prev) || l == __builtin_huge_valf()) return false;
    prev = l;
  }
  return true;
}

Dims make_dims(const oscar_layout_t* L, int batch, int max_seq_len, int pt_stride) {
  Dims d;
  d.batch = batch;
  d.hq = L->num_q_heads;
  d.hkv = L->num_kv_heads;
  d.gq = L->num_q_heads / L->num_kv_heads;
  d.d = L->head_dim;
  d.sink = L->sink_len;
  d.recent = L->recent_len;
  d.wpages = (L->sink_len + L->recent_len) / kPage;
  d.mixed = L->mixed;
  d.off4 = L->mixed ? L->int4_page_offset : L->pool_pages;
  d.pool_pages = L->pool_pages;
  d.max_seq_len = max_seq_len;
  d.pt_stride = pt_stride;
  return d;
}

int choose_ppw(int64_t total_pages, int waves, int64_t target = 512) {
  int64_t p = (total_pages + (int64_t)waves * target - 1) / ((int64_t)waves * target);
  if (p < 1) p = 1;
  if (p > 64) p = 64;
  return (int)p;
}

struct DecodePlan {
  int nw, units_per_kv, step_cost, win_cost;
  size_t off_po, off_pl, off_so, off_sl, off_ru, total;
};


int split_waves(const oscar_layout_t* L, int batch) {
  const int gq = L->num_q_heads / L->num_kv_heads;
  return (gq == 4 && (int64_t)batch * L->num_kv_heads <= kWideMaxGroups) ? kSplitWavesWide : kSplitWaves;
}

// Units per kv-head the split shares out: one round of workgroups on the device (every compute unit
// holding as many as it can), at least one per request, no more than the cost bound of the batch at
// max_seq_len allows with kMinUnitCost per unit, and at most the workspace bound.
// `resident` < 0: the bound itself (workspace sizing).
int units_per_kv(const oscar_layout_t* L, int batch, int max_seq_len, int step, int64_t resident) {
  const int64_t bound = std::max<int64_t>(batch, kMaxUnits / L->num_kv_heads);
  if (resident < 0) return (int)bound;
  const int64_t hp = (std::max(0, max_seq_len - L->sink_len - L->recent_len) + kPage - 1) / kPage;
  const int64_t cost = (step ? step_cost(split_waves(L, batch)) : 0) +
                       window_cost(split_waves(L, batch)) + hp * (L->mixed ? 2 : 1);
  const int64_t by_cost = (batch * cost + kMinUnitCost - 1) / kMinUnitCost;
  const int64_t want = std::min(resident / L->num_kv_heads, by_cost);
  return (int)std::min<int64_t>(bound, std::max<int64_t>(batch, want));
}

// Workgroups of the split kernel the current device holds at once (an estimate of 256 compute
// units with two workgroups each when the device cannot be queried).
int64_t resident_workgroups(const oscar_layout_t* L, int nw) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  int per_cu = split_workgroups_per_cu(L->head_dim, L->num_q_heads / L->num_kv_heads, L->codebook != nullptr,
                                       L->mixed != 0, nw);
  if (per_cu <= 0) per_cu = nw == kSplitWavesWide ? 1 : 2;
  return (int64_t)cus * per_cu;
}

// Split plan of a decode call (units_per_kv from units_per_kv()); the workspace layout covers the
// fused step's slots whether or not `step` is set, so one size serves both entry points.
DecodePlan plan_decode(const oscar_layout_t* L, int batch, int step, int upk) {
  DecodePlan p;
  p.nw = split_waves(L, batch);
  p.units_per_kv = upk;
  p.step_cost = step ? step_cost(p.nw) : 0;
  p.win_cost = window_cost(p.nw);
  const int gq = L->num_q_heads / L->num_kv_heads;
  const size_t units = (size_t)L->num_kv_heads * upk;
  const size_t groups = (size_t)batch * L->num_kv_heads;
  p.off_po = kAlign;
  p.off_pl = p.off_po + align_up(units * 3 * gq * L->head_dim * 4);
  p.off_so = p.off_pl + align_up(units * 3 * gq * 4);
  p.off_sl = p.off_so + align_up(groups * 2 * gq * L->head_dim * 4);
  p.off_ru = p.off_sl + align_up(groups * 2 * gq * 4);
  p.total = p.off_ru + align_up((size_t)batch * 2 * 4);
  return p;
}

struct Bf16Plan {
  int ppw, s;
  size_t off_po, off_pl, total;
};

Bf16Plan plan_bf16(const oscar_layout_t* L, int batch, int max_seq_len) {
  Bf16Plan p;
  const int pages = (max_seq_len + kPage - 1) / kPage;
  p.ppw = choose_ppw((int64_t)batch * L->num_kv_heads * pages, 4);
  p.s = (pages + 4 * p.ppw - 1) / (4 * p.ppw);
  // fewer splits when the merge could not hold them all
  while (p.s > kMaxSlots && p.ppw < 64) {
    p.ppw *= 2;
    p.s = (pages + 4 * p.ppw - 1) / (4 * p.ppw);
  }
  if (p.s < 1) p.s = 1;
  const int gq = L->num_q_heads / L->num_kv_heads;
  const size_t nsl = (size_t)batch * L->num_kv_heads * p.s * gq;
  p.off_po = kAlign;
  p.off_pl = p.off_po + align_up(nsl * L->head_dim * 4);
  p.total = p.off_pl + align_up(nsl * 4);
  return p;
}

size_t page_bytes(const oscar_layout_t* L, int bits) {
  if (bits == 16) return (size_t)L->num_kv_heads * bf16_page_head_bytes(L->head_dim);
  return (size_t)L->num_kv_heads * qpage_head_bytes(L->head_dim, bits);
}

}  // namespace

// Workspace of oscar_decode_step_noalloc: one file-scope array per device (its code object's copy),
// zero at load and never freed. Host code uses the address hipGetSymbolAddress returns for the
// current device, never the array's name (which is a host-side stand-in, not a device address).
constexpr size_t kStaticScratchBytes = OSCAR_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
oscar_status_t scratch_on_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return OSCAR_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return OSCAR_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return OSCAR_OK;
}
}  // namespace

extern "C" {

const char* oscar_status_string(oscar_status_t s) {
  switch (s) {
    case OSCAR_OK: return "OSCAR_OK";
    case OSCAR_ERR_INVALID_ARG: return "OSCAR_ERR_INVALID_ARG";
    case OSCAR_ERR_UNSUPPORTED: return "OSCAR_ERR_UNSUPPORTED";
    case OSCAR_ERR_WORKSPACE: return "OSCAR_ERR_WORKSPACE";
    case OSCAR_ERR_LAUNCH: return "OSCAR_ERR_LAUNCH";
  }
  return "OSCAR_ERR_UNKNOWN";
}

const char* oscar_version(void) { return "oscar-mi355x 0.1.0 gfx950"; }

size_t oscar_page_bytes(const oscar_layout_t* L, int32_t bits) {
  if (check_layout(L) != OSCAR_OK || (bits != 2 && bits != 4 && bits != 16)) return 0;
  return page_bytes(L, bits);
}

size_t oscar_window_bytes(const oscar_layout_t* L, int32_t batch) {
  if (check_layout(L) != OSCAR_OK || batch < 0) return 0;
  return (size_t)batch * L->num_kv_heads * ((L->sink_len + L->recent_len) / kPage) * bf16_page_head_bytes(L->head_dim);
}

size_t oscar_pool_bytes(const oscar_layout_t* L) {
  if (check_layout(L) != OSCAR_OK) return 0;
  if (!L->mixed) return (size_t)L->pool_pages * page_bytes(L, 2);
  return (size_t)L->int4_page_offset * page_bytes(L, 2) + (size_t)(L->pool_pages - L->int4_page_offset) * page_bytes(L, 4);
}

oscar_status_t oscar_quantize_pack(int64_t rows, int32_t dim, int32_t group, int32_t bits, float clip, const float* x,
                                   uint8_t* codes, uint16_t* scale_zero, hipStream_t stream) {
  if (rows < 0 || dim <= 0 || group <= 0 || dim % group) return OSCAR_ERR_INVALID_ARG;
  if (bits != 2 && bits != 4) return OSCAR_ERR_INVALID_ARG;
  if (group % (8 / bits)) return OSCAR_ERR_INVALID_ARG;
  if (!(clip > 0.0f && clip <= 1.0f)) return OSCAR_ERR_INVALID_ARG;
  if (dim > 1024) return OSCAR_ERR_UNSUPPORTED;
  if (rows == 0) return OSCAR_OK;
  if (!x || !codes || !scale_zero) return OSCAR_ERR_INVALID_ARG;
  return launch_quantize_pack(rows, dim, group, bits, clip, x, codes, scale_zero, nullptr, stream) == hipSuccess
             ? OSCAR_OK
             : OSCAR_ERR_LAUNCH;
}

oscar_status_t oscar_quantize_pack_codebook(int64_t rows, int32_t dim, int32_t group, float clip, const float* x,
                                            const uint16_t* levels, uint8_t* codes, uint16_t* scale_zero,
                                            hipStream_t stream) {
  if (rows < 0 || dim <= 0 || group <= 0 || dim % group || group % 4) return OSCAR_ERR_INVALID_ARG;
  if (!(clip > 0.0f && clip <= 1.0f) || !levels_ok(levels)) return OSCAR_ERR_INVALID_ARG;
  if (dim > 1024) return OSCAR_ERR_UNSUPPORTED;
  if (rows == 0) return OSCAR_OK;
  if (!x || !codes || !scale_zero) return OSCAR_ERR_INVALID_ARG;
  return launch_quantize_pack(rows, dim, group, 2, clip, x, codes, scale_zero, levels, stream) == hipSuccess
             ? OSCAR_OK
             : OSCAR_ERR_LAUNCH;
}

oscar_status_t oscar_kv_prefill(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const int32_t* seq_len,
                                const void* k, const void* v, const uint8_t* token_bits, const float* rot_k,
                                const float* rot_v, void* pool, const int32_t* page_table, const int32_t* page_table4,
                                int32_t pt_stride, void* window, int32_t* n_int4_out, hipStream_t stream) {
  oscar_status_t st = check_layout(L);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || max_seq_len < 0 || pt_stride < 0) return OSCAR_ERR_INVALID_ARG;
  if (batch == 0) return OSCAR_OK;
  if (!seq_len || !k || !v || !rot_k || !rot_v || !window) return OSCAR_ERR_INVALID_ARG;
  const int hist_max = max_seq_len - L->sink_len - L->recent_len;
  if (hist_max > 0) {
    if (!pool || !page_table || pt_stride <= 0) return OSCAR_ERR_INVALID_ARG;
    if (L->mixed && !page_table4) return OSCAR_ERR_INVALID_ARG;
  }
  CacheWriteArgs a{};
  a.dm = make_dims(L, batch, max_seq_len, pt_stride);
  a.seq_len = seq_len;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.bits = L->mixed ? token_bits : nullptr;
  a.rot_k = rot_k;
  a.rot_v = rot_v;
  a.clip_k = L->clip_k;
  a.clip_v = L->clip_v;
  a.clip_k4 = L->clip_k4;
  a.clip_v4 = L->clip_v4;
  a.codebook = L->codebook;
  a.pool = static_cast<uint8_t*>(pool);
  a.pt2 = page_table;
  a.pt4 = page_table4;
  a.window = static_cast<uint8_t*>(window);
  a.n_int4_out = n_int4_out;
  return launch_prefill(a, stream) == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

// Validates the demote arguments and fills `a`; batch == 0 is valid (nothing to do).
static oscar_status_t build_demote(const oscar_layout_t* L, int32_t batch, const int32_t* seq_len,
                                   const int32_t* n_int4, const void* new_k, const void* new_v,
                                   const uint8_t* demote_bits, const float* rot_k, const float* rot_v, void* pool,
                                   const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                   void* window, int32_t* seq_len_out, int32_t* n_int4_out, CacheWriteArgs* out) {
  oscar_status_t st = check_layout(L);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || pt_stride <= 0) return OSCAR_ERR_INVALID_ARG;
  if (batch == 0) return OSCAR_OK;
  if (!seq_len || !new_k || !new_v || !rot_k || !rot_v || !pool || !page_table || !window) return OSCAR_ERR_INVALID_ARG;
  if (L->mixed && !page_table4) return OSCAR_ERR_INVALID_ARG;
  if (seq_len_out && (const void*)seq_len_out == (const void*)seq_len) return OSCAR_ERR_INVALID_ARG;
  if (n_int4_out && n_int4 && (const void*)n_int4_out == (const void*)n_int4) return OSCAR_ERR_INVALID_ARG;
  CacheWriteArgs a{};
  a.dm = make_dims(L, batch, 0, pt_stride);
  a.seq_len = seq_len;
  a.n_int4 = n_int4;
  a.k = static_cast<const uint16_t*>(new_k);
  a.v = static_cast<const uint16_t*>(new_v);
  a.bits = L->mixed ? demote_bits : nullptr;
  a.rot_k = rot_k;
  a.rot_v = rot_v;
  a.clip_k = L->clip_k;
  a.clip_v = L->clip_v;
  a.clip_k4 = L->clip_k4;
  a.clip_v4 = L->clip_v4;
  a.codebook = L->codebook;
  a.pool = static_cast<uint8_t*>(pool);
  a.pt2 = page_table;
  a.pt4 = page_table4;
  a.window = static_cast<uint8_t*>(window);
  a.seq_len_out = seq_len_out;
  a.n_int4_out = n_int4_out;
  *out = a;
  return OSCAR_OK;
}

oscar_status_t oscar_kv_demote(const oscar_layout_t* L, int32_t batch, const int32_t* seq_len, const int32_t* n_int4,
                               const void* new_k, const void* new_v, const uint8_t* demote_bits, const float* rot_k,
                               const float* rot_v, void* pool, const int32_t* page_table, const int32_t* page_table4,
                               int32_t pt_stride, void* window, int32_t* seq_len_out, int32_t* n_int4_out,
                               hipStream_t stream) {
  CacheWriteArgs a{};
  const oscar_status_t st = build_demote(L, batch, seq_len, n_int4, new_k, new_v, demote_bits, rot_k, rot_v, pool,
                                         page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, &a);
  if (st != OSCAR_OK || batch == 0) return st;
  return launch_demote(a, stream) == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

size_t oscar_decode_workspace_bytes(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len) {
  if (check_layout(L) != OSCAR_OK || batch < 0 || max_seq_len < 0) return 0;
  // the largest plan any device gets; the layout has the fused step's slots in both entry points
  return plan_decode(L, batch, 1, units_per_kv(L, batch, max_seq_len, 1, -1)).total;
}

// Validates the decode arguments and fills `out`; batch == 0 is valid (nothing to do).
static oscar_status_t build_decode(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const void* q,
                                   const int32_t* seq_len, const int32_t* n_int4, const void* window, const void* pool,
                                   const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                   const float* rot_k, const float* rot_v, float softmax_scale, void* workspace,
                                   size_t workspace_bytes, float* out, int step, DecodeArgs* args) {
  oscar_status_t st = check_layout(L);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || max_seq_len < 0 || pt_stride < 0 || !(softmax_scale >= 0.0f)) return OSCAR_ERR_INVALID_ARG;
  if (batch == 0) return OSCAR_OK;
  if (!q || !seq_len || !window || !rot_k || !rot_v || !out) return OSCAR_ERR_INVALID_ARG;
  const int hist_max = max_seq_len - L->sink_len - L->recent_len;
  if (hist_max > 0) {
    if (!pool || !page_table || pt_stride <= 0) return OSCAR_ERR_INVALID_ARG;
    if (L->mixed && !page_table4) return OSCAR_ERR_INVALID_ARG;
  }
  const DecodePlan p =
      plan_decode(L, batch, step,
                  units_per_kv(L, batch, max_seq_len, step, resident_workgroups(L, split_waves(L, batch))));
  if (!workspace || workspace_bytes < p.total) return OSCAR_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  DecodeArgs a{};
  a.dm = make_dims(L, batch, max_seq_len, pt_stride);
  a.q = static_cast<const uint16_t*>(q);
  a.seq_len = seq_len;
  a.n_int4 = L->mixed ? n_int4 : nullptr;
  a.window = static_cast<const uint8_t*>(window);
  a.pool = static_cast<const uint8_t*>(pool);
  a.pt2 = page_table;
  a.pt4 = page_table4;
  a.rot_k = rot_k;
  a.rot_v = rot_v;
  a.codebook = L->codebook;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)L->head_dim);
  a.scale_log2e = scale * 1.4426950408889634f;
  a.out = out;
  a.ws.flags = reinterpret_cast<uint32_t*>(ws);
  a.ws.part_o = reinterpret_cast<float*>(ws + p.off_po);
  a.ws.part_lse = reinterpret_cast<float*>(ws + p.off_pl);
  a.ws.step_o = reinterpret_cast<float*>(ws + p.off_so);
  a.ws.step_lse = reinterpret_cast<float*>(ws + p.off_sl);
  a.ws.req_units = reinterpret_cast<int32_t*>(ws + p.off_ru);
  a.ws.units_per_kv = p.units_per_kv;
  a.ws.nw = p.nw;
  a.ws.step_cost = p.step_cost;
  a.ws.win_cost = p.win_cost;
  // One request in wide workgroups over an INT2-only cache: history pages interleaved over units
  // 1 .. n-1 (no device-side plan, so page ids load before the length is read), when the history
  // at max_seq_len gives those units at least kInterleaveMinPages pages each.
  const int64_t hp_max = (std::max(0, hist_max) + kPage - 1) / kPage;
  a.ws.interleave = batch == 1 && p.nw == kSplitWavesWide && !L->mixed && p.units_per_kv >= 2 &&
                    hp_max >= (int64_t)kInterleaveMinPages * (p.units_per_kv - 1);
  a.step = step;
  *args = a;
  return OSCAR_OK;
}

static oscar_status_t decode_impl(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const void* q,
                                  const int32_t* seq_len, const int32_t* n_int4, const void* window, const void* pool,
                                  const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                  const float* rot_k, const float* rot_v, float softmax_scale, void* workspace,
                                  size_t workspace_bytes, float* out, hipEvent_t* events, hipStream_t stream) {
  DecodeArgs a{};
  const oscar_status_t st = build_decode(L, batch, max_seq_len, q, seq_len, n_int4, window, pool, page_table,
                                         page_table4, pt_stride, rot_k, rot_v, softmax_scale, workspace,
                                         workspace_bytes, out, 0, &a);
  if (st != OSCAR_OK || batch == 0) return st;
  a.events = events;
  const CacheWriteArgs none{};
  return launch_decode(a, none, stream) == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

oscar_status_t oscar_decode_attn(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const void* q,
                                 const int32_t* seq_len, const int32_t* n_int4, const void* window, const void* pool,
                                 const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                 const float* rot_k, const float* rot_v, float softmax_scale, void* workspace,
                                 size_t workspace_bytes, float* out, hipStream_t stream) {
  return decode_impl(L, batch, max_seq_len, q, seq_len, n_int4, window, pool, page_table, page_table4, pt_stride,
                     rot_k, rot_v, softmax_scale, workspace, workspace_bytes, out, nullptr, stream);
}

oscar_status_t oscar_decode_attn_profiled(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len,
                                          const void* q, const int32_t* seq_len, const int32_t* n_int4,
                                          const void* window, const void* pool, const int32_t* page_table,
                                          const int32_t* page_table4, int32_t pt_stride, const float* rot_k,
                                          const float* rot_v, float softmax_scale, void* workspace,
                                          size_t workspace_bytes, float* out, hipEvent_t* events, int32_t n_events,
                                          hipStream_t stream) {
  if (!events || n_events < 4) return OSCAR_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return OSCAR_ERR_INVALID_ARG;
  return decode_impl(L, batch, max_seq_len, q, seq_len, n_int4, window, pool, page_table, page_table4, pt_stride,
                     rot_k, rot_v, softmax_scale, workspace, workspace_bytes, out, events, stream);
}

static oscar_status_t step_impl(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const int32_t* seq_len,
                                const int32_t* n_int4, const void* new_k, const void* new_v,
                                const uint8_t* demote_bits, const void* q, const float* rot_k, const float* rot_v,
                                void* pool, const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                void* window, int32_t* seq_len_out, int32_t* n_int4_out, float softmax_scale,
                                void* workspace, size_t workspace_bytes, float* out, hipEvent_t* events,
                                hipStream_t stream) {
  if (!seq_len_out) return OSCAR_ERR_INVALID_ARG;
  if (L && L->mixed && !n_int4_out) return OSCAR_ERR_INVALID_ARG;
  CacheWriteArgs cw{};
  oscar_status_t st = build_demote(L, batch, seq_len, n_int4, new_k, new_v, demote_bits, rot_k, rot_v, pool,
                                   page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, &cw);
  if (st != OSCAR_OK) return st;
  DecodeArgs a{};
  // the attention reads the cache as it stands before the step (lengths seq_len, n_int4); the
  // demoted and the appended token enter as one-token partials
  st = build_decode(L, batch, max_seq_len, q, seq_len, n_int4, window, pool, page_table, page_table4, pt_stride,
                    rot_k, rot_v, softmax_scale, workspace, workspace_bytes, out, 1, &a);
  if (st != OSCAR_OK || batch == 0) return st;
  a.events = events;
  return launch_decode(a, cw, stream) == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

oscar_status_t oscar_decode_step(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const int32_t* seq_len,
                                 const int32_t* n_int4, const void* new_k, const void* new_v,
                                 const uint8_t* demote_bits, const void* q, const float* rot_k, const float* rot_v,
                                 void* pool, const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                 void* window, int32_t* seq_len_out, int32_t* n_int4_out, float softmax_scale,
                                 void* workspace, size_t workspace_bytes, float* out, hipStream_t stream) {
  return step_impl(L, batch, max_seq_len, seq_len, n_int4, new_k, new_v, demote_bits, q, rot_k, rot_v, pool,
                   page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, softmax_scale, workspace,
                   workspace_bytes, out, nullptr, stream);
}

oscar_status_t oscar_decode_step_profiled(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len,
                                          const int32_t* seq_len, const int32_t* n_int4, const void* new_k,
                                          const void* new_v, const uint8_t* demote_bits, const void* q,
                                          const float* rot_k, const float* rot_v, void* pool,
                                          const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                          void* window, int32_t* seq_len_out, int32_t* n_int4_out,
                                          float softmax_scale, void* workspace, size_t workspace_bytes, float* out,
                                          hipEvent_t* events, int32_t n_events, hipStream_t stream) {
  if (!events || n_events < 4) return OSCAR_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return OSCAR_ERR_INVALID_ARG;
  return step_impl(L, batch, max_seq_len, seq_len, n_int4, new_k, new_v, demote_bits, q, rot_k, rot_v, pool,
                   page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, softmax_scale, workspace,
                   workspace_bytes, out, events, stream);
}

oscar_status_t oscar_decode_step_noalloc(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len,
                                         const int32_t* seq_len, const int32_t* n_int4, const void* new_k,
                                         const void* new_v, const uint8_t* demote_bits, const void* q,
                                         const float* rot_k, const float* rot_v, void* pool,
                                         const int32_t* page_table, const int32_t* page_table4, int32_t pt_stride,
                                         void* window, int32_t* seq_len_out, int32_t* n_int4_out,
                                         float softmax_scale, float* out, hipStream_t stream) {
  oscar_status_t st = check_layout(L);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || max_seq_len < 0) return OSCAR_ERR_INVALID_ARG;
  // the device-independent bound of the plan, so acceptance does not depend on the device
  if (oscar_decode_workspace_bytes(L, batch, max_seq_len) > kStaticScratchBytes) return OSCAR_ERR_WORKSPACE;
  if (batch == 0) return step_impl(L, batch, max_seq_len, seq_len, n_int4, new_k, new_v, demote_bits, q, rot_k,
                                   rot_v, pool, page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out,
                                   softmax_scale, nullptr, 0, out, nullptr, stream);
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != OSCAR_OK) return st;
  return step_impl(L, batch, max_seq_len, seq_len, n_int4, new_k, new_v, demote_bits, q, rot_k, rot_v, pool,
                   page_table, page_table4, pt_stride, window, seq_len_out, n_int4_out, softmax_scale, ws,
                   kStaticScratchBytes, out, nullptr, stream);
}

oscar_status_t oscar_bf16_fill(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const int32_t* seq_len,
                               const void* k, const void* v, void* pages, int64_t num_pages,
                               const int32_t* page_table, int32_t pt_stride, hipStream_t stream) {
  oscar_status_t st = check_layout(L);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || max_seq_len < 0 || num_pages < 0) return OSCAR_ERR_INVALID_ARG;
  if (batch == 0 || max_seq_len == 0) return OSCAR_OK;
  if (!seq_len || !k || !v || !pages || !page_table) return OSCAR_ERR_INVALID_ARG;
  if (pt_stride <= 0) return OSCAR_ERR_INVALID_ARG;
  Bf16Args a{};
  a.dm = make_dims(L, batch, max_seq_len, pt_stride);
  a.dm.pool_pages = num_pages;
  a.seq_len = seq_len;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.pages = static_cast<uint8_t*>(pages);
  a.pt = page_table;
  return launch_bf16_fill(a, stream) == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

size_t oscar_bf16_decode_workspace_bytes(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len) {
  if (check_layout(L) != OSCAR_OK || batch < 0 || max_seq_len < 0) return 0;
  return plan_bf16(L, batch, max_seq_len).total;
}

oscar_status_t oscar_bf16_decode_attn(const oscar_layout_t* L, int32_t batch, int32_t max_seq_len, const void* q,
                                      const int32_t* seq_len, const void* pages, int64_t num_pages,
                                      const int32_t* page_table, int32_t pt_stride, float softmax_scale,
                                      void* workspace, size_t workspace_bytes, float* out, hipStream_t stream) {
  oscar_status_t st = check_layout(L);
  if (st != OSCAR_OK) return st;
  if (batch < 0 || max_seq_len < 0 || num_pages < 0 || pt_stride < 0 || !(softmax_scale >= 0.0f))
    return OSCAR_ERR_INVALID_ARG;
  if (batch == 0) return OSCAR_OK;
  if (!q || !seq_len || !pages || !page_table || !out) return OSCAR_ERR_INVALID_ARG;
  if (pt_stride <= 0) return OSCAR_ERR_INVALID_ARG;
  const Bf16Plan p = plan_bf16(L, batch, max_seq_len);
  if (p.s > kMaxSlots) return OSCAR_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total) return OSCAR_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Bf16Args a{};
  a.dm = make_dims(L, batch, max_seq_len, pt_stride);
  a.dm.pool_pages = num_pages;
  a.q = static_cast<const uint16_t*>(q);
  a.seq_len = seq_len;
  a.pages = static_cast<uint8_t*>(const_cast<void*>(pages));
  a.pt = page_table;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)L->head_dim);
  a.scale_log2e = scale * 1.4426950408889634f;
  a.out = out;
  a.flags = reinterpret_cast<uint32_t*>(ws);
  a.part_o = reinterpret_cast<float*>(ws + p.off_po);
  a.part_lse = reinterpret_cast<float*>(ws + p.off_pl);
  a.s = p.s;
  a.ppw = p.ppw;
  return launch_bf16_decode(a, stream) == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

}  // extern "C"
