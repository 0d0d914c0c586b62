// Decode attention over the three-segment cache (OSCAR overview page, method paragraph: the INT2
// kernel unpacks codes, restores scale/zero and accumulates in floating point, the BF16 kernel
// handles sink/recent, an online-softmax merge combines them; news article: keys stored as x.R_K,
// values as v.R_V). TriAxialKV reading note, section 4: bitwidth-homogeneous splits (INT2 pages,
// INT4 pages) merged by log-sum-exp.
//
// Kernels of one decode call, in stream order:
//   split        one launch, one workgroup per unit of a device-side work plan: a unit is a cost
//                range of its request's sequence [step | INT2 pages | INT4 pages | BF16 window]
//                and runs the segments that range holds (the fused step's demote and new-token
//                partials, window pages, history pages of each width), writing (o, lse) partials
//                per query head. Workgroups are 4 wavefronts, or 16 at small GQA-4 batches. Each
//                history segment forms its query operands itself: q' = (q . R_K) * scale *
//                log2(e), split into fp16 high/low matrix-core operands scaled per channel for the
//                code unpacking below.
//   merge        per (request, kv-head): LSE-merge the history partials (rotated basis), apply
//                R_V^T, LSE-merge with the BF16 window partials, write the fp32 output; in a fused
//                step it also writes the new token into its window slot.
//
// Fused decode step (demote the oldest recent token, append the new one, attend): the attention
// must see the demoted token quantised and the new token in the window, but nothing has to wait
// for the cache writes. The step workgroup rotates and quantises the demoted token with the
// demote's own arithmetic, stores its codes into the history slot that the history workgroups do
// not read yet (it lies past their token count), and adds two one-token partials: the demoted
// token (rotated basis, history side) and the new token (window side). The window role skips the
// ring slot of the demoted token, whose BF16 copy the merge then overwrites with the new token.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16 for QK^T and, over a pair of pages, for PV; BF16
// variants for the window): the 16 tokens of a page on the M rows of QK^T, the query heads of the
// GQA group on the N columns. The QK^T result layout (lane l holds tokens 4*(l/16)+r of head
// l%16) is the A-operand layout of PV (rows = heads, k = tokens); at GQA 4 and 8 the logits are
// spread over the wavefront for the softmax and gathered back with DPP moves. Codes reach the
// matrix cores as fp16 subnormals: masking a code c at bit p of a half-word gives the fp16 value
// c * 2^(p-24); the 2^(24-p) factor is folded into the query operand (keys) or applied once to the
// accumulator (values). Query and softmax weights are split into high + low fp16 parts (~22
// significant bits); the two parts sit in spare columns (QK^T) and spare rows (PV). Each
// wavefront streams its contiguous page range through a load ring of page pairs (six pages, four
// in 16-wavefront workgroups), its page ids fetched a chunk of 60 at a time.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "demote.hpp"
#include "timeline.hpp"

namespace oscar {

#ifdef OSCAR_TIMELINE
__device__ uint64_t g_timeline[kTimelineSplitRows + kTimelineMergeRows][kTimelineCols];
#endif

constexpr float kNegInf = -__builtin_huge_valf();
#ifndef OSCAR_HIST_PIPE2
#define OSCAR_HIST_PIPE2 6
#endif
#ifndef OSCAR_HIST_PIPE4
#define OSCAR_HIST_PIPE4 6
#endif
// history pages in the per-wave load ring (INT2 page-heads are 1152 B, INT4 2176 B at d = 128)
constexpr int kHistPipe2 = OSCAR_HIST_PIPE2;
constexpr int kHistPipe4 = OSCAR_HIST_PIPE4;
#ifndef OSCAR_WIDE_RING
#define OSCAR_WIDE_RING 4
#endif
constexpr int kBf16Pipe = 2;   // BF16 pages in the per-wave load ring (8 KB each)

__device__ __forceinline__ float4_t mfma32_f16(const u32x4_t& a, const half8_t& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma32_bf16(const u32x4_t& a, const u32x4_t& b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ float4_t mfma16_bf16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, float4_t c) {
  const u32x2_t av = {a0, a1}, bv = {b0, b1};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, av), __builtin_bit_cast(short4_t, bv),
                                                   c, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ uint32_t row_shr_or_zero(uint32_t v) {
  if constexpr (N >= 16) return 0u;
  else return dpp_row_shr<N>(v);
}

// Sum / maximum over each aligned group of N adjacent lanes (N = 1, 2, 4, 8 or 16), every lane of
// the group receiving it: quad swaps, then the half-row and row mirrors (DPP, no LDS traffic).
// Every lane of the wavefront must be active.
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "lane group of 1..16");
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f<0x141>(v);
  if constexpr (N >= 16) v += dpp_f<0x140>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float lanes_max(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "lane group of 1..16");
  if constexpr (N >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

// v plus the value of the lane 16 apart (lane l and l ^ 16), and the same 32 lanes apart: a lane
// swap of v with itself puts each lane's own value and its partner's in the two results.
__device__ __forceinline__ float rows_sum16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float rows_sum32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ------------------------------------------------------------------ split bookkeeping
struct HistCounts {
  int T, hist, n2, n4;
};
__device__ inline HistCounts hist_counts(const DecodeArgs& a, int b) {
  HistCounts c;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > a.dm.max_seq_len ? a.dm.max_seq_len : T);
  c.T = T;
  c.hist = max(0, T - a.dm.sink - a.dm.recent);
  int n4 = (a.dm.mixed && a.n_int4) ? a.n_int4[b] : 0;
  n4 = n4 < 0 ? 0 : (n4 > c.hist ? c.hist : n4);
  c.n4 = n4;
  c.n2 = c.hist - n4;
  return c;
}

// ------------------------------------------------------------------ work plan (device side)
// A request's n units cut its cost sequence [step | INT2 pages | INT4 pages | window] into n equal
// cost ranges: an INT2 page costs 1, an INT4 page 2, the step step_cost and the BF16 window (sink
// and recent pages, taken as one block by all wavefronts of its unit at once) win_cost; a page, the
// step or the window belongs to the unit that holds its first cost position. The step and the
// window are latency-bound, and their costs are the pages their unit would stream meanwhile; at
// the two ends of the sequence they fall to different units. Requests get units in proportion to
// their cost. Every wavefront that needs the plan computes it from the device lengths (the host
// knows only max_seq_len), so the workgroups of a launch agree without communicating.
constexpr int kInt4PageCost = 2;

struct ReqCost {
  int p2, p4;    // history pages of each width (cut at the page-table stride)
  int cost;      // whole cost sequence
};

__device__ inline ReqCost request_cost(const DecodeArgs& a, int b) {
  const HistCounts c = hist_counts(a, b);
  ReqCost r;
  r.p2 = min((c.n2 + kPage - 1) / kPage, a.dm.pt_stride);
  r.p4 = min((c.n4 + kPage - 1) / kPage, a.dm.pt_stride);
  r.cost = a.ws.step_cost + r.p2 + kInt4PageCost * r.p4 + a.ws.win_cost;
  return r;
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum over the lanes of a wavefront.
__device__ __forceinline__ int64_t wave_scan_i64(int64_t v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

// Units of the requests before a request whose predecessors' costs add up to `cum`, minus the one
// unit each of them holds at least: floor(extra * cum / C + 1/2) (cumulative rounding, so the
// shares of all requests add up to `extra` exactly).
__device__ __forceinline__ int64_t unit_share(int64_t extra, int64_t cum, int64_t total) {
  return total > 0 ? (2 * extra * cum + total) / (2 * total) : 0;
}

struct RequestUnits {
  int b;           // request (-1: none)
  int first, n;    // units per kv-head before the request, and its own
  ReqCost rc;
};

// The request that holds unit `key` of every kv-head, with its units. Wave-level: every lane
// returns the same.
__device__ RequestUnits request_units(const DecodeArgs& a, int key) {
  const int B = a.dm.batch, lane = threadIdx.x % kWave;
  if (B == 1) {   // one request holds every unit
    RequestUnits r;
    r.b = 0;
    r.first = 0;
    r.n = a.ws.units_per_kv;
    r.rc = request_cost(a, 0);
    return r;
  }
  const int64_t extra = max(0, a.ws.units_per_kv - B);
  int64_t total = 0;
  for (int b0 = 0; b0 < B; b0 += kWave) {
    const int b = b0 + lane;
    total += b < B ? request_cost(a, b).cost : 0;
  }
  total = wave_sum_i64(total);
  RequestUnits r;
  r.b = -1;
  r.first = r.n = 0;
  r.rc = ReqCost{0, 0, 0};
  int64_t carry = 0;
  for (int b0 = 0; b0 < B; b0 += kWave) {
    const int b = b0 + lane;
    const ReqCost rc = b < B ? request_cost(a, b) : ReqCost{0, 0, 0};
    const int64_t incl = wave_scan_i64(rc.cost, lane) + carry;
    const int first = b + (int)unit_share(extra, incl - rc.cost, total);
    const int next = b + 1 + (int)unit_share(extra, incl, total);
    const bool hit = b < B && first <= key && key < next;
    const uint64_t m = __ballot(hit);
    if (m) {
      const int l = __builtin_ctzll(m);
      r.b = __shfl(b, l, kWave);
      r.first = __shfl(first, l, kWave);
      r.n = __shfl(next - first, l, kWave);
      r.rc.p2 = __shfl(rc.p2, l, kWave);
      r.rc.p4 = __shfl(rc.p4, l, kWave);
      r.rc.cost = __shfl(rc.cost, l, kWave);
      return r;
    }
    carry = __shfl(incl, kWave - 1, kWave);
  }
  return r;
}

// Segments of the unit with cost range [c0, c1) of a request's sequence.
struct Segments {
  bool step;
  bool window;    // all window pages
  int p20, p21;   // INT2 history pages
  int p40, p41;   // INT4 history pages
};

__device__ __forceinline__ int ceil_pos(int x, int y) { return x <= 0 ? 0 : (x + y - 1) / y; }

__device__ inline Segments unit_segments(const DecodeArgs& a, const ReqCost& rc, int c0, int c1) {
  const int S = a.ws.step_cost;
  const int base2 = S, base4 = base2 + rc.p2, basew = base4 + kInt4PageCost * rc.p4;
  Segments sg;
  sg.step = S > 0 && c0 == 0 && c1 > 0;
  sg.window = c0 <= basew && basew < c1;
  sg.p20 = min(max(c0 - base2, 0), rc.p2);
  sg.p21 = min(max(c1 - base2, 0), rc.p2);
  sg.p40 = min(ceil_pos(c0 - base4, kInt4PageCost), rc.p4);
  sg.p41 = min(ceil_pos(c1 - base4, kInt4PageCost), rc.p4);
  return sg;
}

// Cost range of unit j of a request with n units (32-bit division when the products fit).
__device__ __forceinline__ void unit_range(const RequestUnits& r, int j, int& c0, int& c1) {
  const uint64_t hi = (uint64_t)(j + 1) * (uint32_t)r.rc.cost;
  if (hi <= 0xFFFFFFFFull) {
    c0 = (int)((uint32_t)j * (uint32_t)r.rc.cost / (uint32_t)r.n);
    c1 = (int)((uint32_t)hi / (uint32_t)r.n);
  } else {
    c0 = (int)((uint64_t)j * (uint32_t)r.rc.cost / (uint32_t)r.n);
    c1 = (int)(hi / (uint32_t)r.n);
  }
}

// ------------------------------------------------------------------ query prologue
// Thread (column group cg, part) of an NT-thread workgroup holds rows part*QR .. part*QR+QR-1 of
// columns 4cg .. 4cg+3 of R_K (float4 loads issued with the segment's first loads).
template <int D, int NT>
struct QRotRows {
  static constexpr int CG = D / 4;      // column groups of 4
  static constexpr int NPQ = NT / CG;   // parts of a column group
  static constexpr int QR = D / NPQ;    // rows per part
  static_assert(NPQ * CG == NT && NPQ * QR == D, "the rotation rows split evenly over the threads");
  float4 r[QR];
  __device__ void load(const float* rot, int tid) {
    const int cg = tid % CG, part = tid / CG;
#pragma unroll
    for (int i = 0; i < QR; ++i) r[i] = *reinterpret_cast<const float4*>(rot + (size_t)(part * QR + i) * D + 4 * cg);
  }
};

template <int D, int GQ, int NW>
struct HistQueryLds {
  float qs[GQ][D];               // queries of the group (fp32)
  float ps[NW][GQ][D];           // per-wavefront partial products
  uint16_t op[2][GQ][D];         // fp16 operands: high parts, low parts
  float hsc[GQ][4];              // per head: sum of high parts, sum of low parts, 2^E
};

// Words of the group's bf16 queries that each thread loads.
template <int D, int GQ, int NT>
constexpr int kQueryWords = (GQ * D / 2 + NT - 1) / NT;

// The queries of a (request, kv-head) group that a thread of the prologue needs. Direct: the thread
// loads the bf16 queries of its own rotation rows (GQ heads x QR rows, when that is a few words);
// otherwise the group is staged through LDS, each thread loading kQueryWords words of it.
template <int D, int GQ, int NT>
struct QueryIn {
  static constexpr int QR = QRotRows<D, NT>::QR;
  static constexpr bool direct = QR % 2 == 0 && GQ * QR / 2 <= 8;
  static constexpr int W = direct ? GQ * QR / 2 : kQueryWords<D, GQ, NT>;
  uint32_t w[W];
  // q: the group's queries [GQ][D] bf16
  __device__ void load(const uint16_t* q, int tid) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(q);
    if constexpr (direct) {
      const int part = tid / QRotRows<D, NT>::CG;
#pragma unroll
      for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int i = 0; i < QR / 2; ++i) w[h * (QR / 2) + i] = src[(h * D + part * QR) / 2 + i];
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        const int e = tid + NT * i;
        w[i] = e < GQ * D / 2 ? src[e] : 0u;
      }
    }
  }
};

// Sum of x[0..N) as a tree of adjacent pairs ((x0 + x1) + (x2 + x3)) + ...
template <int N>
__device__ __forceinline__ float sum_adjacent_tree(float (&x)[N]) {
#pragma unroll
  for (int w = N; w > 1; w /= 2)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) x[i] = x[2 * i] + x[2 * i + 1];
  return x[0];
}

// Query operands of the GQ heads of a (request, kv-head) for code width BITS, into LDS (L.op,
// L.hsc), by one workgroup of NW wavefronts. v = q'_j (rotated, log2-scaled) is split on a
// power-of-two grid Delta = 2^(ceil(log2 max|v|) - 11): v_hi = Delta*rint(v/Delta) has at most 11
// significant bits, so its fp16 operand is exact and every partial sum of c*v_hi over a head is an
// exact fp32 multiple of Delta (|sum| <= 15 * 128 * 2^11 Delta < 2^24 Delta); v_lo = v - v_hi
// carries the rest. The products see v as fp16 operands scaled per code bit position p (a code c at
// bit p of its fp16 slot has the value c*2^(p-24)): operand = v*2^(24-p-E), one exponent E per
// head. Operand column c of the products holds the high parts of head c for c < GQ and the low
// parts of head c-GQ for GQ <= c < 2GQ.
// LUT: the key operand holds codebook levels (normal fp16 values, no bit-position factor), so
// every channel takes p = 0 and the products carry 2^(24-E) instead of 2^-E.
// A callable run by every wavefront between its query products and the prologue's first barrier.
struct NoHook {
  __device__ void operator()() const {}
};

template <int BITS, int D, int GQ, int NW, bool LUT = false, typename Hook = NoHook>
__device__ void query_operands(const QRotRows<D, NW * kWave>& rr, const QueryIn<D, GQ, NW * kWave>& qin,
                               HistQueryLds<D, GQ, NW>& L, float scale_log2e, Hook&& hook = Hook{}) {
  constexpr int NT = NW * kWave;
  constexpr int CG = QRotRows<D, NT>::CG, QR = QRotRows<D, NT>::QR;
  using QI = QueryIn<D, GQ, NT>;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  if constexpr (!QI::direct) {
#pragma unroll
    for (int i = 0; i < QI::W; ++i) {
      const int e = tid + NT * i;
      if (e < GQ * D / 2) {
        float* qf = &L.qs[0][0];
        qf[2 * e] = bf16_bits_to_f32(qin.w[i] & 0xFFFFu);
        qf[2 * e + 1] = bf16_bits_to_f32(qin.w[i] >> 16);
      }
    }
    __syncthreads();
  }
  {
    const int cg = tid % CG, part = tid / CG;
#pragma unroll
    for (int h = 0; h < GQ; ++h) {
      float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < QR; ++i) {
        float x;
        if constexpr (QI::direct) {
          const uint32_t wd = qin.w[h * (QR / 2) + i / 2];
          x = bf16_bits_to_f32((i & 1) ? (wd >> 16) : (wd & 0xFFFFu));
        } else {
          x = L.qs[h][part * QR + i];
        }
        acc.x = fmaf(x, rr.r[i].x, acc.x);
        acc.y = fmaf(x, rr.r[i].y, acc.y);
        acc.z = fmaf(x, rr.r[i].z, acc.z);
        acc.w = fmaf(x, rr.r[i].w, acc.w);
      }
#pragma unroll
      for (int o = CG; o < kWave; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o, kWave);
        acc.y += __shfl_xor(acc.y, o, kWave);
        acc.z += __shfl_xor(acc.z, o, kWave);
        acc.w += __shfl_xor(acc.w, o, kWave);
      }
      if (lane < CG) *reinterpret_cast<float4*>(&L.ps[wave][h][4 * cg]) = acc;
    }
  }
  OSCAR_TL_SPLIT(11);
  hook();
  __syncthreads();
  OSCAR_TL_SPLIT(15);
  constexpr int NC = D / kWave;  // channels per lane in the head pass
  for (int h = wave; h < GQ; h += NW) {
    float v[NC];
    float vmax = 0.0f, me = 0.0f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int j = lane + kWave * k;
      float parts[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) parts[w] = L.ps[w][h][j];
      v[k] = sum_adjacent_tree<NW>(parts) * scale_log2e;
      const int m = (j % 8) / 2;
      const int p = LUT ? 0 : (BITS == 2 ? 2 * m : 4 * (m % 2));
      vmax = fmaxf(vmax, fabsf(v[k]));
      me = fmaxf(me, ldexpf(fabsf(v[k]), 24 - p));
    }
    vmax = wave_max(vmax);
    me = wave_max(me);
    int e = 0, ev = 0;
    if (me > 0.0f) {
      frexpf(me, &e);
      e -= 15;
    }
    if (vmax > 0.0f) frexpf(vmax, &ev);  // vmax < 2^ev
    float sh = 0.0f, sl = 0.0f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int j = lane + kWave * k;
      const int m = (j % 8) / 2;
      const int p = LUT ? 0 : (BITS == 2 ? 2 * m : 4 * (m % 2));
      const float v_hi = ldexpf(rintf(ldexpf(v[k], 11 - ev)), ev - 11);
      const float v_lo = v[k] - v_hi;
      sh += v_hi;
      sl += v_lo;
      L.op[0][h][j] = (uint16_t)f32_to_f16_bits(ldexpf(v_hi, 24 - p - e));
      L.op[1][h][j] = (uint16_t)f32_to_f16_bits(ldexpf(v_lo, 24 - p - e));
    }
    sh = wave_sum(sh);   // exact: a sum of multiples of Delta below 2^24 Delta
    sl = wave_sum(sl);
    if (lane == 0) {
      L.hsc[h][0] = sh;
      L.hsc[h][1] = sl;
      L.hsc[h][2] = ldexpf(1.0f, LUT ? e - 24 : e);
      L.hsc[h][3] = 0.0f;
    }
  }
  __syncthreads();
}

// The operands of query_operands as registers: lane (g, c) gets operand column c and the constants
// of head c % GQ.
template <int BITS, int D, int GQ, int NW, bool LUT = false, typename Hook = NoHook>
__device__ void hist_query_operands(const QRotRows<D, NW * kWave>& rr, const QueryIn<D, GQ, NW * kWave>& qin,
                                    HistQueryLds<D, GQ, NW>& L, float scale_log2e, half8_t (&bq)[D / 32], float& uh,
                                    float& ul, float& esc, Hook&& hook = Hook{}) {
  const int lane = threadIdx.x % kWave, g = lane / 16, c = lane % 16;
  query_operands<BITS, D, GQ, NW, LUT>(rr, qin, L, scale_log2e, hook);
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const u32x4_t z = {0, 0, 0, 0};
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(&L.op[c < GQ ? 0 : 1][c % GQ][32 * kk + 8 * g]);
    bq[kk] = __builtin_bit_cast(half8_t, c < 2 * GQ ? w : z);
  }
  uh = L.hsc[c % GQ][0];
  ul = L.hsc[c % GQ][1];
  esc = L.hsc[c % GQ][2];
}

// ------------------------------------------------------------------ per-wave softmax state
template <int D, int GQ>
struct WaveState {
  float m_run, m_thr, l_part, z_part;  // m_thr = m_run + 8: a logit above it triggers a rescale
  float4_t o[D / 16];
  __device__ void init() {
    m_run = kNegInf;
    m_thr = kNegInf;
    l_part = 0.0f;
    z_part = 0.0f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) o[nb] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
};

// Online-softmax update given NL logits of this lane (4 per page: tokens 4g+r of head h =
// lane%16); returns the probabilities. Rescales only when the maximum exceeds the running max by
// more than 8 (log2 units), so probabilities stay below 2^8.
template <int D, int GQ, int NL>
__device__ __forceinline__ void softmax_page(WaveState<D, GQ>& st, const float (&lg)[NL], float (&p)[NL], int lane) {
  const int h = lane % 16, g = lane / 16;
  float mx = lg[0];
#pragma unroll
  for (int i = 1; i < NL; ++i) mx = fmaxf(mx, lg[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
  const bool need = (h < GQ) && (mx > st.m_run + 8.0f);
  if (__any(need)) {
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = (st.m_run == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.l_part *= alpha;
    st.z_part *= alpha;
    st.m_run = m_new;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, (4 * g + r) % GQ, kWave);
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) st.o[nb][r] *= ar;
    }
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) p[i] = (h < GQ && lg[i] != kNegInf) ? __builtin_amdgcn_exp2f(lg[i] - st.m_run) : 0.0f;
}

// Writes the wave's state to LDS and merges the 4 waves of the workgroup into one partial
// (o normalised, lse in log2 units). VSH_BITS selects the value-code scale restore.
// nws: the first nws wavefronts hold states to merge (the others hold none and only help with the
// outputs). The loops over wavefronts are unrolled to NW with the weights predicated, so every LDS
// read of an output is issued before the first is used.
template <int D, int GQ, int VSH_BITS, bool REDIST = false, int NW = 4>
__device__ void workgroup_merge(const WaveState<D, GQ>& st, float (*o_lds)[2 * GQ][D], float (*st_lds)[3][8],
                                float* part_o, float* part_lse) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane / 16, h = lane % 16;
  float l_tot = st.l_part, z_tot = st.z_part;
  // All on the vector units (no LDS round trip): row rotations, then lane swaps across rows.
  if constexpr (REDIST) {
    // lanes c, c+GQ, ... of a row share a head: fold them first (a row rotated by 8, then by 4, ...
    // down to GQ, sums the lanes of c's residue class mod GQ)
    if constexpr (GQ <= 8) {
      l_tot += dpp_row_ror<8>(l_tot);
      z_tot += dpp_row_ror<8>(z_tot);
    }
    if constexpr (GQ <= 4) {
      l_tot += dpp_row_ror<4>(l_tot);
      z_tot += dpp_row_ror<4>(z_tot);
    }
    if constexpr (GQ <= 2) {
      l_tot += dpp_row_ror<2>(l_tot);
      z_tot += dpp_row_ror<2>(z_tot);
    }
    if constexpr (GQ <= 1) {
      l_tot += dpp_row_ror<1>(l_tot);
      z_tot += dpp_row_ror<1>(z_tot);
    }
  }
  l_tot = rows_sum16(l_tot);
  l_tot = rows_sum32(l_tot);
  z_tot = rows_sum16(z_tot);
  z_tot = rows_sum32(z_tot);
  // every wavefront writes its state (one that ran no page holds the empty state: m = -inf, sums
  // 0), so the reduction below reads all NW entries without per-wavefront branches
  if (g == 0 && h < GQ) {
    st_lds[wave][0][h] = st.m_run;
    st_lds[wave][1][h] = l_tot;
    st_lds[wave][2][h] = z_tot;
  }
  // FOLD (GQA 4 and 8): the high and low rows of a head are added in registers before the state
  // goes to LDS. At GQA 4 they are 16 lanes apart (rows c and c + 4: lane groups 0 and 1), at GQA 8
  // 32 lanes apart (rows c and c + 8: lane groups 0-1 and 2-3); one lane-swap instruction takes the
  // accumulators of two adjacent 16-column blocks nb = 2k, 2k+1 at once, and their sums land side by
  // side, so every write covers 32 consecutive columns of one head. Other widths store both rows.
  constexpr bool FOLD = (GQ == 4 || GQ == 8) && D % 32 == 0;
  if constexpr (FOLD) {
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t a0 = __float_as_uint(st.o[2 * k][r]), a1 = __float_as_uint(st.o[2 * k + 1][r]);
        float sum;
        if constexpr (GQ == 4) {
          const auto sw = __builtin_amdgcn_permlane16_swap(a0, a1, false, false);
          // lanes 0-15: block 2k, rows r and r + 4; lanes 16-31: block 2k + 1
          sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          if (lane < 32) o_lds[wave][r][32 * k + lane] = sum;
        } else {
          const auto sw = __builtin_amdgcn_permlane32_swap(a0, a1, false, false);
          // lanes 0-31: block 2k, rows 4g + r (g < 2) and their low rows; lanes 32-63: block 2k + 1
          sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          o_lds[wave][4 * (g % 2) + r][32 * k + 16 * (g / 2) + h] = sum;
        }
      }
  } else {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (row < 2 * GQ) o_lds[wave][row][16 * nb + h] = st.o[nb][r];
      }
  }
  OSCAR_TL_SPLIT(12);
  __syncthreads();
  OSCAR_TL_SPLIT(13);
  // With at least twice as many threads as outputs, SPLIT adjacent lanes share an output, each
  // folding every SPLIT-th wavefront; their maxima and sums are combined across the lanes (DPP).
  constexpr int SPLIT = NW * kWave >= 2 * GQ * D ? NW * kWave / (GQ * D) : 1;
  if constexpr (SPLIT >= 2) {
    static_assert(NW % SPLIT == 0 && SPLIT <= 16 && (SPLIT & (SPLIT - 1)) == 0, "lane groups of the merge");
    constexpr int WPS = NW / SPLIT;
    const int idx = tid / SPLIT, s = tid % SPLIT;
    const int hh = idx / D, ch = idx % D, nb = ch / 16;
    float mw[WPS];
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < WPS; ++i) {
      mw[i] = st_lds[s + SPLIT * i][0][hh];
      M = fmaxf(M, mw[i]);
    }
    M = lanes_max<SPLIT>(M);
    float L = 0.0f, Z = 0.0f, O = 0.0f;
#pragma unroll
    for (int i = 0; i < WPS; ++i) {
      const int w = s + SPLIT * i;
      const bool live = mw[i] != kNegInf;
      const float aw = live ? __builtin_amdgcn_exp2f(mw[i] - M) : 0.0f;
      L = fmaf(aw, st_lds[w][1][hh], L);
      Z = fmaf(aw, st_lds[w][2][hh], Z);
      O = fmaf(aw, FOLD ? o_lds[w][hh][ch] : o_lds[w][hh][ch] + o_lds[w][GQ + hh][ch], O);
    }
    L = lanes_sum<SPLIT>(L);
    Z = lanes_sum<SPLIT>(Z);
    O = lanes_sum<SPLIT>(O);
    float vscale = 1.0f;
    if (VSH_BITS == 2) vscale = ldexpf(1.0f, 24 - 2 * (nb % 4));
    if (VSH_BITS == 4) vscale = ldexpf(1.0f, 24 - 4 * (nb % 2));
    const bool empty = (M == kNegInf) || !(L > 0.0f);
    if (s == 0) {
      part_o[hh * D + ch] = empty ? 0.0f : (O * vscale + Z) / L;
      if (ch == 0) part_lse[hh] = empty ? kNegInf : M + log2f(L);
    }
    OSCAR_TL_SPLIT(14);
    return;
  }
  for (int idx = tid; idx < GQ * D; idx += NW * kWave) {
    const int hh = idx / D, ch = idx % D, nb = ch / 16;
    float mw[NW];
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mw[w] = st_lds[w][0][hh];
      M = fmaxf(M, mw[w]);
    }
    float L = 0.0f, Z = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const bool live = mw[w] != kNegInf;
      const float aw = live ? __builtin_amdgcn_exp2f(mw[w] - M) : 0.0f;
      const float lw = st_lds[w][1][hh], zw = st_lds[w][2][hh];
      const float ow = FOLD ? o_lds[w][hh][ch] : o_lds[w][hh][ch] + o_lds[w][GQ + hh][ch];
      L = fmaf(aw, lw, L);
      Z = fmaf(aw, zw, Z);
      O = fmaf(aw, ow, O);
    }
    float vscale = 1.0f;
    if (VSH_BITS == 2) vscale = ldexpf(1.0f, 24 - 2 * (nb % 4));
    if (VSH_BITS == 4) vscale = ldexpf(1.0f, 24 - 4 * (nb % 2));
    const bool empty = (M == kNegInf) || !(L > 0.0f);
    part_o[hh * D + ch] = empty ? 0.0f : (O * vscale + Z) / L;
    if (ch == 0) part_lse[hh] = empty ? kNegInf : M + log2f(L);
  }
  OSCAR_TL_SPLIT(14);
}

// ------------------------------------------------------------------ page pipeline
// Runs proc(buf, pg) for pg in [wp0, wp1) while the loads of the next NB-1 pages are in flight.
// Buffers are indexed by compile-time constants (the ring is fully unrolled), and every load is
// issued unconditionally -- out-of-range prefetches read a fixed dummy page-head that stays in
// cache -- so the compiler waits exactly for the buffer about to be used.
template <int NB, typename Page, typename LoadF, typename ProcF>
__device__ __forceinline__ void page_pipeline(int wp0, int wp1, LoadF&& load, ProcF&& proc) {
  Page buf[NB];
  bool ok[NB];
#pragma unroll
  for (int k = 0; k < NB - 1; ++k) ok[k] = load(buf[k], wp0 + k);
  for (int pg = wp0; pg < wp1; pg += NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      ok[(k + NB - 1) % NB] = load(buf[(k + NB - 1) % NB], pg + k + NB - 1);
      if (pg + k < wp1) proc(buf[k], ok[k], pg + k);
    }
  }
}

// ------------------------------------------------------------------ BF16 page-heads
template <int D>
struct Bf16Page {
  u32x4_t ka[D / 32];  // key lane chunk: 8 bf16 per k-step
  u32x4_t va[D / 32];  // value lane chunk: two 16-channel blocks per uint4
};

template <int D>
__device__ __forceinline__ void load_bf16_page(Bf16Page<D>& pr, const uint8_t* ph, int lane) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) pr.ka[kk] = *reinterpret_cast<const u32x4_t*>(ph + lane * (D / 2) + 16 * kk);
#pragma unroll
  for (int j = 0; j < D / 32; ++j) pr.va[j] = *reinterpret_cast<const u32x4_t*>(ph + 32 * D + lane * (D / 2) + 16 * j);
}

template <int D, int GQ>
__device__ __forceinline__ void process_bf16_page(WaveState<D, GQ>& st, const Bf16Page<D>& pr, const u32x4_t* bq,
                                                  const bool valid[4], float sl2e, int lane) {
  const int h = lane % 16;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) acc = mfma32_bf16(pr.ka[kk], bq[kk], acc);
  float lg[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lg[r] = valid[r] ? acc[r] * sl2e : kNegInf;
  float p[4];
  softmax_page<D, GQ, 4>(st, lg, p, lane);
  st.l_part += (p[0] + p[1]) + (p[2] + p[3]);
  uint32_t hb[4], lb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    hb[r] = f32_to_bf16_bits(p[r]);
    lb[r] = f32_to_bf16_bits(p[r] - bf16_bits_to_f32(hb[r]));
  }
  const uint32_t l01 = lb[0] | (lb[1] << 16), l23 = lb[2] | (lb[3] << 16);
  const uint32_t s01 = row_shr_or_zero<GQ>(l01), s23 = row_shr_or_zero<GQ>(l23);
  const uint32_t a01 = h < GQ ? (hb[0] | (hb[1] << 16)) : (h < 2 * GQ ? s01 : 0u);
  const uint32_t a23 = h < GQ ? (hb[2] | (hb[3] << 16)) : (h < 2 * GQ ? s23 : 0u);
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    const u32x4_t& v = pr.va[nb / 2];
    const uint32_t b0 = (nb & 1) ? v[2] : v[0];
    const uint32_t b1 = (nb & 1) ? v[3] : v[1];
    st.o[nb] = mfma16_bf16(a01, a23, b0, b1, st.o[nb]);
  }
}

template <int D, int GQ>
__device__ __forceinline__ void load_bf16_query(u32x4_t* bq, const uint16_t* q, size_t qrow_base, int lane) {
  const int g = lane / 16, h = lane % 16;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    bq[kk] = u32x4_t{0, 0, 0, 0};
    if (h < GQ) bq[kk] = *reinterpret_cast<const u32x4_t*>(q + (qrow_base + h) * D + 32 * kk + 8 * g);
  }
}

// ------------------------------------------------------------------ step segment (fused decode step)
template <int D, int GQ>
struct StepLds {
  uint16_t xs[1 + GQ][D];   // demoted key (row 0) and the queries (rows 1..GQ), bf16
  uint16_t xv[D];           // demoted value, bf16
  uint16_t nk[D], nv[D];    // the new token, bf16
  float xr[2][D];           // rotated demoted key, value
  float vq[GQ][D];          // rotated, log2-scaled queries
  uint8_t cs[2][D];         // codes of the demoted key, value
  uint32_t szs[2];          // their bf16 (scale, zero)
};

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Whether request b's fused step runs: the cache must have room for the new token
// (seq_len < max_seq_len). A request without room is left as it is -- no demote, no append, its
// length unchanged, flag bit 1 -- and its attention covers the cache as it stands.
__device__ __forceinline__ bool step_active(const DecodeArgs& a, int b) {
  return a.step && a.seq_len[b] < a.dm.max_seq_len;
}

// The fp32 rotation entries of a wavefront's 32-column slice (rotation_entries per k-step), loaded
// in H parts of D/16/H k-steps (the first part before anything waits; wide workgroups, bound to 128
// registers, hold half a slice at a time).
template <int D, int H>
struct RotEntries {
  static constexpr int KP = D / 16 / H;   // k-steps per part
  float r[KP][8];
  __device__ void load(const float* rot, int w, int part, int lane) {
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) rotation_entries<D>(rot, w, part * KP + kk, lane, r[kk]);
  }
};

// rotate_rows_loaded on entries in registers, part by part: the same products in the same order.
template <int D, int H, typename XPtr>
__device__ __forceinline__ float16v_t rotate_rows_entries(RotEntries<D, H>& re, const float* rot, int w, XPtr x,
                                                          int stride, int nrows, int lane) {
  constexpr int KP = RotEntries<D, H>::KP;
  float16v_t acc = {};
#pragma unroll
  for (int part = 0; part < H; ++part) {
    if (part > 0) {
      __builtin_amdgcn_sched_barrier(0);   // the next part's loads reuse this part's registers
      re.load(rot, w, part, lane);
    }
#pragma unroll
    for (int kk = 0; kk < KP; ++kk) {
      bf16x8_t hi, mid, lo;
      split_rotation(re.r[kk], hi, mid, lo);
      acc = rotation_step(rotation_a(x, stride, nrows, part * KP + kk, lane), hi, mid, lo, acc);
    }
  }
  return acc;
}

// The step work of (request b, kv-head kv), with T = seq_len[b] tokens before the step. Demote
// (T >= sink + recent): the token at T - recent is read from its ring slot, rotated and quantised
// with the demote kernel's own arithmetic (same rotation order, same grid), and its codes go into
// its history slot, which no history segment reads yet (it lies past their token count); its
// one-token partial -- lse = q' . k_hat, o = v_hat, rotated basis -- fills step slot 0 (lse = -inf
// without a demote). The new token's one-token partial -- lse = scale * log2(e) * q . k_new,
// o = v_new -- fills step slot 1. Both logits are summed in fp64 from exact products. The lengths
// after the step are written here too; the new token's window copy is written by the merge, after
// every window read.
// The segment is a chain of latencies, so every global load is issued before anything waits on
// one: the lengths, then at once the demoted token, the queries, the new token, the page id of the
// history slot, the codebooks and each wavefront's rotation slices.
template <int D, int GQ, int NW>
__device__ void step_seg(const DecodeArgs& a, const CacheWriteArgs& cw, int b, int kv, StepLds<D, GQ>& L) {
  constexpr int SL = D / 32;   // 32-column slices of the rotation
  constexpr int NT = NW * kWave;
  constexpr int ROWS = 4 + GQ; // demoted key, demoted value, new key, new value, queries
  constexpr int PER = (ROWS * D + NT - 1) / NT;
  // the value slices go to their own wavefronts when there are enough of them
  constexpr bool VPAR = NW >= 2 * SL;
  const Dims& dm = a.dm;
  const int bk = b * dm.hkv + kv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  // cache-side lengths exactly as the demote kernel reads them
  const int T = a.seq_len[b] < 0 ? 0 : a.seq_len[b];
  const bool active = step_active(a, b);
  const int n4 = (dm.mixed && a.n_int4) ? a.n_int4[b] : 0;
  const bool demote = active && T >= dm.sink + dm.recent;
  const int bw = (demote && dm.mixed && cw.bits && cw.bits[b] == 4) ? 4 : 2;
  const int dslot = bw == 4 ? n4 : T - dm.sink - dm.recent - n4;
  const int64_t page = demote ? demote_page(cw, b, dslot, bw) : -1;
  const size_t qrow = (size_t)b * dm.hq + (size_t)kv * GQ;
  const int64_t pb = bf16_page_head_bytes(D);
  int opg = 0, ot = 0;
  if (demote) window_slot(T - dm.recent, dm, opg, ot);
  const uint16_t* og = reinterpret_cast<const uint16_t*>(a.window + ((size_t)bk * dm.wpages + opg) * pb);
  uint16_t v[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid + NT * e;
    const int r = idx / D, ch = idx % D;
    uint16_t x = 0;
    if (idx < ROWS * D) {
      if (r == 0) x = demote ? og[bf16_key_index(D, ot, ch)] : (uint16_t)0;
      else if (r == 1) x = demote ? og[bf16_value_index(D, ot, ch)] : (uint16_t)0;
      else if (r == 2) x = cw.k[(size_t)bk * D + ch];
      else if (r == 3) x = cw.v[(size_t)bk * D + ch];
      else x = a.q[(qrow + r - 4) * D + ch];
    }
    v[e] = x;
  }
  const Codebook cbk = load_codebook(cw.codebook, kv, 0);
  const Codebook cbv = load_codebook(cw.codebook, kv, 1);
  // one slice per wavefront: K slices on wavefronts 0..SL-1, V slices on SL..2SL-1 (or, with fewer
  // wavefronts, on 0..SL-1 again after their K products)
  constexpr int H = NW >= 16 ? 2 : 1;
  RotEntries<D, H> re;
  const int vw = VPAR ? wave - SL : wave;
  const bool vwave = VPAR ? (wave >= SL && wave < 2 * SL) : wave < SL;
  const float* rk = a.rot_k + (size_t)kv * D * D;
  const float* rvp = a.rot_v + (size_t)kv * D * D;
  if (wave < SL) re.load(rk, wave, 0, lane);
  else if (vwave) re.load(rvp, vw, 0, lane);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = tid + NT * e;
    const int r = idx / D, ch = idx % D;
    if (idx < ROWS * D) {
      if (r == 0) L.xs[0][ch] = v[e];
      else if (r == 1) L.xv[ch] = v[e];
      else if (r == 2) L.nk[ch] = v[e];
      else if (r == 3) L.nv[ch] = v[e];
      else L.xs[r - 3][ch] = v[e];
    }
  }
  __syncthreads();
  OSCAR_TL_SPLIT(9);
  // one matrix-core pass rotates the key (row 0, the demote's own arithmetic) and the queries
  // (rows 1..GQ) with R_K; a second rotates the value with R_V
  if (wave < SL) {
    const float16v_t acc = rotate_rows_entries<D, H>(re, rk, wave, &L.xs[0][0], D, 1 + GQ, lane);
    const int n = 32 * wave + lane % 32;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int m = 8 * (j / 4) + 4 * (lane / 32) + j % 4;
      if (m == 0)
        L.xr[0][n] = acc[j];
      else if (m <= GQ)
        L.vq[m - 1][n] = acc[j] * a.scale_log2e;
    }
  }
  if (vwave) {
    if (!VPAR) re.load(rvp, vw, 0, lane);
    const float16v_t accv = rotate_rows_entries<D, H>(re, rvp, vw, L.xv, D, 1, lane);
    if (lane < 32) L.xr[1][32 * vw + lane] = accv[0];
  }
  __syncthreads();
  OSCAR_TL_SPLIT(10);
  if (demote && wave < 2) {
    const float clip = bw == 4 ? (wave ? cw.clip_v4 : cw.clip_k4) : (wave ? cw.clip_v : cw.clip_k);
    quantize_token<D>(L.xr[wave], clip, bw, L.cs[wave], &L.szs[wave], lane, wave ? cbv : cbk);
  }
  __syncthreads();
  if (demote) {
    store_token<D>(cw, page, kv, bw, dslot % kPage, 0, L.cs[0], L.szs[0], tid, NT);
    store_token<D>(cw, page, kv, bw, dslot % kPage, 1, L.cs[1], L.szs[1], tid, NT);
  }
  OSCAR_TL_SPLIT(11);
  float* po_d = a.ws.step_o + ((size_t)bk * 2) * GQ * D;
  float* pl_d = a.ws.step_lse + ((size_t)bk * 2) * GQ;
  float* po_n = po_d + GQ * D;
  float* pl_n = pl_d + GQ;
  const double sk = __uint_as_float(L.szs[0] << 16), zk = __uint_as_float(L.szs[0] & 0xFFFF0000u);
  const float sv = __uint_as_float(L.szs[1] << 16), zv = __uint_as_float(L.szs[1] & 0xFFFF0000u);
  // restored values: z + s * level (the code itself, or the codebook's level of an INT2 code)
  const bool lvk = bw == 2 && cw.codebook != nullptr;
  auto level = [&](const Codebook& cb, uint32_t code) { return lvk ? codebook_level(cb, code) : (float)code; };
  for (int h = wave; h < GQ; h += NW) {
    double ld = 0.0, ln = 0.0;
    for (int ch = lane; ch < D; ch += kWave) {
      if (demote) ld += (double)L.vq[h][ch] * (sk * (double)level(cbk, L.cs[0][ch]) + zk);
      if (active) ln += (double)bf16_bits_to_f32(L.xs[1 + h][ch]) * (double)bf16_bits_to_f32(L.nk[ch]);
    }
    ld = wave_sum_f64(ld);
    ln = wave_sum_f64(ln);
    if (lane == 0) {
      pl_d[h] = demote ? (float)ld : kNegInf;
      pl_n[h] = active ? (float)(ln * (double)a.scale_log2e) : kNegInf;
    }
  }
  for (int idx = tid; idx < GQ * D; idx += NT) {
    const int ch = idx % D;
    po_d[idx] = demote ? fmaf(sv, level(cbv, L.cs[1][ch]), zv) : 0.0f;
    po_n[idx] = active ? bf16_bits_to_f32(L.nv[ch]) : 0.0f;
  }
  if (kv == 0 && tid == 0) {
    if (cw.seq_len_out) cw.seq_len_out[b] = active ? T + 1 : a.seq_len[b];
    if (cw.n_int4_out) cw.n_int4_out[b] = n4 + ((demote && bw == 4) ? 1 : 0);
    if (!active) atomicOr(a.ws.flags, 2u);
  }
}

// Window segment: the window pages w0, w0 + ws, w0 + 2 ws, ... of (b, kv) (sink pages, then the
// recent ring); wavefront w takes the w-th, (w + NW)-th, ... of them, with the next page loading
// while one is processed (single pages with many wavefronts: each has at most one or two). In a
// fused step the ring slot of the demoted token (position T - recent) is left to the step segment.
template <int D, int GQ, int NW>
__device__ void window_seg(const DecodeArgs& a, int b, int kv, int w0, int ws, float* po, float* pl,
                           float (*o_lds)[2 * GQ][D], float (*st_lds)[3][8]) {
  const Dims& dm = a.dm;
  const int bk = b * dm.hkv + kv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane / 16;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const bool skip_demoted = step_active(a, b);
  u32x4_t bq[D / 32];
  load_bf16_query<D, GQ>(bq, a.q, (size_t)b * dm.hq + (size_t)kv * GQ, lane);
  WaveState<D, GQ> st;
  st.init();
  const int64_t pb = bf16_page_head_bytes(D);
  const uint8_t* wbase = a.window + (size_t)bk * dm.wpages * pb;
  auto process = [&](const Bf16Page<D>& cur, int pg) {
    bool valid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * g + r;
      if (pg < dm.sink / kPage) {
        valid[r] = kPage * pg + t < T;
      } else if (T <= dm.sink) {
        valid[r] = false;
      } else {
        const int sl = kPage * (pg - dm.sink / kPage) + t;
        int back = (T - 1 - sl) % dm.recent;
        if (back < 0) back += dm.recent;
        valid[r] = T - 1 - back >= dm.sink && !(skip_demoted && back == dm.recent - 1);
      }
    }
    process_bf16_page<D, GQ>(st, cur, bq, valid, a.scale_log2e, lane);
  };
  const int w1 = dm.wpages, stride = NW * ws;
  int pg = w0 + wave * ws;
  if constexpr (NW >= 8) {
    for (; pg < w1; pg += stride) {
      Bf16Page<D> cur;
      load_bf16_page<D>(cur, wbase + pg * pb, lane);
      process(cur, pg);
    }
  } else {
    Bf16Page<D> cur, nxt;
    if (pg < w1) load_bf16_page<D>(cur, wbase + pg * pb, lane);
    for (; pg < w1; pg += stride) {
      if (pg + stride < w1) load_bf16_page<D>(nxt, wbase + (pg + stride) * pb, lane);
      process(cur, pg);
      cur = nxt;
    }
  }
  // wavefronts past the unit's window pages hold the empty state
  workgroup_merge<D, GQ, 16, false, NW>(st, o_lds, st_lds, po, pl);
}

// ------------------------------------------------------------------ INT2 / INT4 history pages
// For GQA widths 4 and 8 the QK^T result is redistributed with DPP so that every lane owns whole
// (token, head) logits (1 per lane at GQ 4, 2 at GQ 8); each lane then loads only its own tokens'
// scale/zero and the softmax arithmetic runs on all 64 lanes. The PV operand is gathered back
// with DPP. Widths 1 and 2 keep the QK^T result layout (4 tokens per lane on the first GQ lanes
// of each row).
template <int GQ>
struct Redist {
  static constexpr bool on = GQ == 4 || GQ == 8;
  static constexpr int per_lane = GQ == 8 ? 2 : 1;   // logits per lane when redistributed
  static constexpr int meta_words = GQ == 4 ? 2 : (GQ == 8 ? 4 : 8);
};

template <int BITS, int D, int GQ>
struct QPage {
  static constexpr int CW = D * BITS / 128;  // 32-bit words of one lane's key or value part
  uint32_t kw[CW], vw[CW];
  uint32_t mt[Redist<GQ>::meta_words];
};

// Raw buffer descriptor of one page-head (gfx9 family: base, stride 0, size in bytes, word 3
// 0x00020000): the page's loads then take the same per-lane byte offsets on every page, and a
// byte past the page-head would read as zero instead of touching the next one. A descriptor of
// size 0 (prefetches past the range, page ids outside the pool) makes every load of the page an
// out-of-range read: zeros, no memory access, so such a load completes as soon as the loads
// issued before it have.
// Cache policy of the history page loads: nt (streaming) where every load instruction of a wavefront
// covers whole 128-byte lines: the codes at d <= 128 (an INT2 lane chunk of 8 or 16 bytes; an INT4
// key or value part of 8 or 16 bytes, the parts of all lanes consecutive) and the metadata at GQA 4
// and 8. A page-head is read once per step, so it should not displace what the step re-reads from
// the L2 (R_K, page tables, query operands). Where two instructions share lines (d = 256, the
// metadata at other widths) a non-allocating load would fetch the line twice: default policy there.
template <int BITS, int D, int GQ>
constexpr int kPageLoadPolicy = (D <= 128 && (GQ == 4 || GQ == 8)) ? 2 : 0;

template <int BITS, int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t qpage_rsrc(uint64_t head, bool live) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(head), (short)0,
                                           live ? 4 * D * BITS + kMetaBytes : 0, kRawBufferFlags);
}

template <int BITS, int D, int GQ>
__device__ __forceinline__ void load_qpage(QPage<BITS, D, GQ>& pr, uint64_t head, bool live, int lane) {
  constexpr int CW = QPage<BITS, D, GQ>::CW;
  constexpr int POL = kPageLoadPolicy<BITS, D, GQ>;
  const int g = lane / 16, c = lane % 16;
  const __amdgpu_buffer_rsrc_t r = qpage_rsrc<BITS, D>(head, live);
  if constexpr (BITS == 2 && CW == 1) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, 0, POL);
    pr.kw[0] = v[0];
    pr.vw[0] = v[1];
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int j = 0; j < 2 * CW / 4; ++j) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 8 * CW + 16 * j, 0, POL);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = 4 * j + e;
        if (w < CW) pr.kw[w] = v[e];
        else pr.vw[w - CW] = v[e];
      }
    }
  } else if constexpr (CW == 2) {  // INT4: key parts of all lanes, then value parts
    const u32x2_t k = __builtin_amdgcn_raw_buffer_load_b64(r, lane * 8, 0, POL);
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, 64 * 8 + lane * 8, 0, POL);
    pr.kw[0] = k[0];
    pr.kw[1] = k[1];
    pr.vw[0] = v[0];
    pr.vw[1] = v[1];
  } else {
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) {
      const u32x4_t k = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 4 * CW + 16 * j, 0, POL);
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, 64 * 4 * CW + lane * 4 * CW + 16 * j, 0, POL);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pr.kw[4 * j + e] = k[e];
        pr.vw[4 * j + e] = v[e];
      }
    }
  }
  constexpr int meta = 4 * D * BITS;
  if constexpr (GQ == 4) {
    const u32x2_t m = __builtin_amdgcn_raw_buffer_load_b64(r, meta + 8 * (4 * g + c / 4), 0, POL);
    pr.mt[0] = m[0];
    pr.mt[1] = m[1];
  } else if constexpr (GQ == 8) {
    const u32x4_t m = __builtin_amdgcn_raw_buffer_load_b128(r, meta + 8 * (4 * g + 2 * (c / 8)), 0, POL);
#pragma unroll
    for (int e = 0; e < 4; ++e) pr.mt[e] = m[e];
  } else {
    const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, meta + 32 * g, 0, POL);
    const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, meta + 32 * g + 16, 0, POL);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr.mt[e] = a[e];
      pr.mt[4 + e] = b[e];
    }
  }
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// fp16 high part in the low half, fp16 low part (W - high) in the high half (built as a half pair,
// so the two conversions write the two halves in place)
__device__ __forceinline__ uint32_t split_f16(float w) {
  half2_t v;
  v.x = (_Float16)w;
  v.y = (_Float16)(w - (float)v.x);
  return __builtin_bit_cast(uint32_t, v);
}

// Two products p0*s0, p1*s1 split as split_f16 does, packed by part: `hi` holds the fp16 high
// parts (token 0 in the low half), `lo` the fp16 of each product minus its high part. Each mixed
// multiply-add writes its half in place (the compiler would build the halves apart and pack them).
// The trailing s_nop gives a DPP read of either result the two wait states it needs after a vector
// write (the compiler does not see the writes inside the statement).
__device__ __forceinline__ void split_f16_pair(float p0, float s0, float p1, float s1, uint32_t& hi, uint32_t& lo) {
  asm("v_fma_mixlo_f16 %0, %2, %3, 0\n\t"
      "v_fma_mixhi_f16 %0, %4, %5, 0\n\t"
      "v_fma_mixlo_f16 %1, %2, %3, -%0 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %4, %5, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(hi), "=&v"(lo)
      : "v"(p0), "v"(s0), "v"(p1), "v"(s1));
}

// QK^T of one page: rows = the 16 token slots, columns = query operand columns (high parts of
// the GQ heads in columns 0..GQ-1, low parts in GQ..2GQ-1, so one product covers both parts).
// LUT: the codes become their codebook levels (two per byte permute) instead of subnormal slots.
template <int BITS, int D, int GQ, bool LUT = false>
__device__ __forceinline__ float4_t qk_page(const QPage<BITS, D, GQ>& pr, const half8_t* bq, const Codebook& cbk) {
  constexpr int NKK = D / 32;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4_t av;
    if constexpr (LUT) {
      const uint32_t z = codebook_spread(pr.kw[kk / 2], kk & 1);
#pragma unroll
      for (int m = 0; m < 4; ++m) av[m] = codebook_levels2(cbk, z, m);
    } else if constexpr (BITS == 2) {
      const uint32_t w = (kk & 1) ? (pr.kw[kk / 2] >> 8) : pr.kw[kk / 2];
      av[0] = w & 0x00030003u;
      av[1] = w & 0x000C000Cu;
      av[2] = w & 0x00300030u;
      av[3] = w & 0x00C000C0u;
    } else {
      const uint32_t w = pr.kw[kk], w1 = pr.kw[kk] >> 8;
      av[0] = w & 0x000F000Fu;
      av[1] = w & 0x00F000F0u;
      av[2] = w1 & 0x000F000Fu;
      av[3] = w1 & 0x00F000F0u;
    }
    acc = mfma32_f16(av, bq[kk], acc);
  }
  return acc;
}

// History logit s*X + z*U of one token and head: X = (X_hi + X_lo) * 2^E from the high-part
// product (an exact multiple of the query grid) and the low-part product, U = sum of the query
// operand (per head). Formed in fp32 (a few roundings of the larger of s*X and z*U; the two
// nearly cancel only as far as the group's zero point exceeds the spread of its values).
__device__ __forceinline__ float hist_logit(float s, float z, float xh, float xl, float esc, float u) {
  return fmaf(s, (xh + xl) * esc, z * u);
}
__device__ __forceinline__ float hist_logit_x(float s, float z, float x, float esc, float u) {
  return fmaf(s, x * esc, z * u);
}

// B operand words of the PV product for value columns 16nb..16nb+15 of one page: the codes of the
// lane's 4 token slots as fp16 subnormal slots (or, with LUT, as their codebook levels).
template <int BITS, int D, int GQ, bool LUT>
__device__ __forceinline__ void value_words(const QPage<BITS, D, GQ>& pr, int nb, const Codebook& cbv, uint32_t& b0,
                                            uint32_t& b1) {
  if constexpr (LUT) {
    b0 = codebook_levels2(cbv, codebook_spread(pr.vw[nb / 4], false), nb % 4);
    b1 = codebook_levels2(cbv, codebook_spread(pr.vw[nb / 4], true), nb % 4);
  } else if constexpr (BITS == 2) {
    const uint32_t w = pr.vw[nb / 4];
    const uint32_t mask = 0x00030003u << (2 * (nb % 4));
    b0 = w & mask;
    b1 = (w >> 8) & mask;
  } else {
    const uint32_t w = pr.vw[nb / 2];
    const uint32_t mask = 0x000F000Fu << (4 * (nb % 2));
    b0 = w & mask;
    b1 = (w >> 8) & mask;
  }
}

// PV product of a page pair, one 16x16x32 product per 16 value columns: the reduction runs over
// the lane group's 4 token slots of the first page, then the same 4 slots of the second, in A
// (probabilities) and B (codes) alike. `a` = {first page's A words, second page's A words}.
template <int BITS, int D, int GQ, bool LUT>
__device__ __forceinline__ void pv_pair(WaveState<D, GQ>& st, const QPage<BITS, D, GQ>& p0,
                                        const QPage<BITS, D, GQ>& p1, const u32x4_t& a, const Codebook& cbv) {
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    u32x4_t b;
    uint32_t w0, w1, w2, w3;
    value_words<BITS, D, GQ, LUT>(p0, nb, cbv, w0, w1);
    value_words<BITS, D, GQ, LUT>(p1, nb, cbv, w2, w3);
    b[0] = w0;
    b[1] = w1;
    b[2] = w2;
    b[3] = w3;
    st.o[nb] = mfma32_f16(a, __builtin_bit_cast(half8_t, b), st.o[nb]);
  }
}

// Rescale of the PV accumulators by alpha of each row's head. Row 4*g+r of the accumulators is
// head (4g+r) mod GQ (rows GQ..2GQ-1 hold the low parts of heads 0..GQ-1); alpha of head hh is
// read from a lane that owns hh.
template <int D, int GQ>
__device__ __forceinline__ void rescale_rows(WaveState<D, GQ>& st, float alpha, int lane) {
  const int g = lane / 16;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float ar;
    if constexpr (GQ == 8) {
      const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), r));
      const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 4 + r));
      ar = (g & 1) ? a1 : a0;
    } else if constexpr (GQ == 4) {
      ar = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), r));
    } else {
      ar = __shfl(alpha, (4 * g + r) % GQ, kWave);
    }
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.o[nb][r] *= ar;
  }
}

// Online softmax over redistributed logits (NL per lane, all of head lane%GQ). No page maximum
// is formed on the common path: probabilities are taken against the running maximum, and only
// when some logit exceeds it by more than 8 (log2 units) is the maximum rebuilt across the lanes
// of each head and the state rescaled, so every probability stays below 2^8.
template <int D, int GQ, int NL>
__device__ __forceinline__ void redist_softmax(WaveState<D, GQ>& st, const float (&lg)[NL], float (&p)[NL], int lane) {
  bool over = false;
#pragma unroll
  for (int i = 0; i < NL; ++i) over |= lg[i] > st.m_thr;
  if (__any(over)) {
    float mx = lg[0];
#pragma unroll
    for (int i = 1; i < NL; ++i) mx = fmaxf(mx, lg[i]);
#pragma unroll
    for (int o = GQ; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);  // 0 while m_run is -inf
    st.l_part *= alpha;
    st.z_part *= alpha;
    st.m_run = m_new;
    st.m_thr = m_new + 8.0f;
    rescale_rows<D, GQ>(st, alpha, lane);
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) p[i] = __builtin_amdgcn_exp2f(lg[i] - st.m_run);  // 0 for -inf logits
}

// Logits per lane and history page: GQA 4 and 8 spread the 16 x GQ logits of a page over the
// wavefront; other widths keep the 4 token slots of the lane's row.
template <int GQ>
constexpr int kPageLogits = GQ == 4 ? 1 : (GQ == 8 ? 2 : 4);

// Logits of one page from its QK^T result `acc` (column c < GQ: high-part product of head c,
// column GQ + c: low-part product). `lim` = tokens of the history from the page's first slot on:
// slots at or past it get -inf. `lim` is uniform and below kPage only on the last page of a
// range: the empty volatile asm keeps the masks behind a branch (the compiler would otherwise
// compute and select them on every page).
template <int BITS, int D, int GQ>
__device__ __forceinline__ void page_logits(const QPage<BITS, D, GQ>& pr, float4_t acc, float uq, float esc, int lim,
                                            int lane, float (&lg)[kPageLogits<GQ>]) {
  const int g = lane / 16, c = lane % 16;
  if constexpr (GQ == 4) {
    // lane (g, c) takes token 4g + c/4 of head c%4. Lanes c < 4 first add the high part (own
    // column) and the low part (column c + 4) of every row, then lane c passes row r on to lane
    // 4r + c.
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = acc[r] + dpp_row_shl_f<4>(acc[r]);
    float x = y[0];
    x = dpp_row_shr_into<4, 0x2>(x, y[1]);
    x = dpp_row_shr_into<8, 0x4>(x, y[2]);
    x = dpp_row_shr_into<12, 0x8>(x, y[3]);
    lg[0] = hist_logit_x(lo_bf16(pr.mt[0]), hi_bf16(pr.mt[0]), x, esc, uq);
    if (lim < kPage) {
      asm volatile("");
      lg[0] = 4 * g + c / 4 < lim ? lg[0] : kNegInf;
    }
  } else if constexpr (GQ == 8) {
    // lane (g, c): tokens 4g + 2(c/8) + {0, 1} of head c%8. Its own column holds one part of
    // head c%8 (high for c < 8, low for c >= 8) and lane c^8 the other: each lane keeps the rows
    // of its tokens and passes its partner the rows of the partner's tokens (x + y, added in
    // either order, is the same sum).
    const bool lo8 = c < 8;
    const float x0 = (lo8 ? acc[0] : acc[2]) + dpp_row_ror<8>(lo8 ? acc[2] : acc[0]);
    const float x1 = (lo8 ? acc[1] : acc[3]) + dpp_row_ror<8>(lo8 ? acc[3] : acc[1]);
    lg[0] = hist_logit_x(lo_bf16(pr.mt[0]), hi_bf16(pr.mt[0]), x0, esc, uq);
    lg[1] = hist_logit_x(lo_bf16(pr.mt[2]), hi_bf16(pr.mt[2]), x1, esc, uq);
    if (lim < kPage) {
      asm volatile("");
      const int t0 = 4 * g + 2 * (c / 8);
      lg[0] = t0 < lim ? lg[0] : kNegInf;
      lg[1] = t0 + 1 < lim ? lg[1] : kNegInf;
    }
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float xl = __uint_as_float(dpp_row_shl<GQ>(__float_as_uint(acc[r])));
      lg[r] = hist_logit(lo_bf16(pr.mt[2 * r]), hi_bf16(pr.mt[2 * r]), acc[r], xl, esc, uq);
    }
    if (lim < kPage) {
      asm volatile("");
#pragma unroll
      for (int r = 0; r < 4; ++r) lg[r] = 4 * g + r < lim ? lg[r] : kNegInf;
    }
  }
}

// Probability and zero-point sums of one page, and its A words of the PV product: row c of the
// lane group holds fp16 parts of p * s_V for the group's 4 token slots (high parts of head c in
// rows c < GQ, low parts in rows GQ + c).
template <int BITS, int D, int GQ>
__device__ __forceinline__ void page_operand(WaveState<D, GQ>& st, const QPage<BITS, D, GQ>& pr,
                                             const float (&p)[kPageLogits<GQ>], uint32_t psel, int lane,
                                             uint32_t& a01, uint32_t& a23) {
  const int c = lane % 16;
  if constexpr (GQ == 4) {
    st.l_part += p[0];
    st.z_part = fmaf(p[0], hi_bf16(pr.mt[1]), st.z_part);
    // row c < 4 holds the fp16 high parts of head c for tokens 4g..4g+3 (lanes c, c+4, c+8,
    // c+12), row 4 + c the low parts (lanes c, c+4, c+8, c+12 seen from row 4 + c: offsets -4, 0,
    // +4, +8); rows 8..15 are zero (selector bytes 0x0C). Lanes 8..15 of y, u, v8 keep whatever
    // they hold: the selector zeroes those rows.
    const uint32_t P = split_f16(p[0] * lo_bf16(pr.mt[1]));
    // lane c takes tokens 4g + j from lanes 4j + c%4: P itself, and P rotated by 4, 8, 12 lanes
    // (rotating right by 12 reads lane c + 4). Rows c < 4 pair (own, c+4) and (c+8, c+12); rows
    // 4..7 pair (c-4, own) and (c+4, c+8).
    const uint32_t r4 = dpp_row_ror_u<4>(P), r8 = dpp_row_ror_u<8>(P), r12 = dpp_row_ror_u<12>(P);
    const bool b0 = c < 4;
    a01 = __builtin_amdgcn_perm(b0 ? r12 : r4, P, psel);
    a23 = __builtin_amdgcn_perm(b0 ? r4 : r12, r8, psel);
  } else if constexpr (GQ == 8) {
    st.l_part += p[0] + p[1];
    st.z_part = fmaf(p[0], hi_bf16(pr.mt[1]), fmaf(p[1], hi_bf16(pr.mt[3]), st.z_part));
    uint32_t P0, L0;   // fp16 high parts of both tokens, and their low parts
    split_f16_pair(p[0], lo_bf16(pr.mt[1]), p[1], lo_bf16(pr.mt[3]), P0, L0);
    // row c < 8: high parts of head c, tokens 4g, 4g+1 (own) and 4g+2, 4g+3 (lane c+8);
    // row c >= 8: low parts of head c-8, tokens 4g, 4g+1 (lane c-8) and 4g+2, 4g+3 (own)
    a01 = dpp_row_shr_into<8, 0xC>(P0, L0);
    a23 = dpp_row_shl_into<8, 0x3>(L0, P0);
  } else {
    float W[4];
    float lsum = 0.0f, zsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      W[r] = p[r] * lo_bf16(pr.mt[2 * r + 1]);
      lsum += p[r];
      zsum = fmaf(p[r], hi_bf16(pr.mt[2 * r + 1]), zsum);
    }
    st.l_part += lsum;
    st.z_part += zsum;
    const uint32_t q0 = split_f16(W[0]), q1 = split_f16(W[1]), q2 = split_f16(W[2]), q3 = split_f16(W[3]);
    const uint32_t s01 = row_shr_or_zero<GQ>(pack_hi16(q0, q1)), s23 = row_shr_or_zero<GQ>(pack_hi16(q2, q3));
    a01 = c < GQ ? pack_lo16(q0, q1) : (c < 2 * GQ ? s01 : 0u);
    a23 = c < GQ ? pack_lo16(q2, q3) : (c < 2 * GQ ? s23 : 0u);
  }
}

// Softmax and PV product of a page pair given the QK^T results of both pages; `lim0`, `lim1` as
// in page_logits (0 masks a whole page). The online-softmax update covers both pages at once.
template <int BITS, int D, int GQ, bool LUT>
__device__ __forceinline__ void process_qpair(WaveState<D, GQ>& st, const QPage<BITS, D, GQ>& pr0,
                                              const QPage<BITS, D, GQ>& pr1, float4_t acc0, float4_t acc1,
                                              float uq, float esc, uint32_t psel, int lim0, int lim1, int lane,
                                              const Codebook& cbv) {
  constexpr int NL = kPageLogits<GQ>;
  float l0[NL], l1[NL];
  page_logits<BITS, D, GQ>(pr0, acc0, uq, esc, lim0, lane, l0);
  page_logits<BITS, D, GQ>(pr1, acc1, uq, esc, lim1, lane, l1);
  float lg[2 * NL], p[2 * NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    lg[i] = l0[i];
    lg[NL + i] = l1[i];
  }
  if constexpr (Redist<GQ>::on) redist_softmax<D, GQ, 2 * NL>(st, lg, p, lane);
  else softmax_page<D, GQ, 2 * NL>(st, lg, p, lane);
  float p0[NL], p1[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    p0[i] = p[i];
    p1[i] = p[NL + i];
  }
  uint32_t w0, w1, w2, w3;
  page_operand<BITS, D, GQ>(st, pr0, p0, psel, lane, w0, w1);
  page_operand<BITS, D, GQ>(st, pr1, p1, psel, lane, w2, w3);
  u32x4_t a;
  a[0] = w0;
  a[1] = w1;
  a[2] = w2;
  a[3] = w3;
  pv_pair<BITS, D, GQ, LUT>(st, pr0, pr1, a, cbv);
}

#ifndef OSCAR_PROGRESS_PRIORITY
#define OSCAR_PROGRESS_PRIORITY 1
#endif
// Issue priority from progress: a compute unit runs two history workgroups, and the sequencer
// prefers the older wavefront among equal priorities, so the workgroup dispatched second would
// trail by a fifth of its run and finish alone. A wavefront instead takes priority 3 - (4 * done
// / total): the ones behind win issue until the two workgroups move in step.
__device__ __forceinline__ void progress_priority(int done, int total) {
  if constexpr (OSCAR_PROGRESS_PRIORITY) {
    const int level = total > 0 ? (4 * done) / total : 3;
    if (level <= 0) __builtin_amdgcn_s_setprio(3);
    else if (level == 1) __builtin_amdgcn_s_setprio(2);
    else if (level == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
}

// Page ids of a chunk of a wavefront's pages: lane i holds the id of page cb + i, or 0 at or past
// wp1 (such pages are never loaded); a raw buffer load bounded at wp1 reads them, so no lane is
// masked off and the loaded register needs no copy. Chunks start kIdChunk pages apart, so the last four lanes repeat the next chunk's first ids
// and every prefetch of a trip finds its id in the current chunk; the next chunk is loaded a whole
// chunk ahead and is only copied when it becomes current, so its load is not waited on early. page_index turns a page's id (read from its
// lane onto the scalar unit) into its index relative to the first page of the width's region, -1 for
// ids outside [first, lim) (another width's or outside the pool: skipped and flagged); the page's
// address is then formed on the scalar unit.
constexpr int kIdChunk = 60;   // a multiple of both ring depths (4 and 6 pages)

__device__ __forceinline__ int page_chunk(const int32_t* pt, int cb, int wp1, int lane) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(pt), (short)0, (int)(4 * max(wp1, 0)), kRawBufferFlags);
  return __builtin_amdgcn_raw_buffer_load_b32(r, 4 * (cb + lane), 0, 0);
}

__device__ __forceinline__ int page_index(int id, int first, int lim) {
  return (id >= first && id < lim) ? id - first : -1;
}

// History segment: pages [p0, p1) of width BITS of (b, kv), split into contiguous ranges of the NW
// wavefronts; the workgroup's partial (rotated basis) goes to po / pl. LUT (INT2 with a codebook):
// codes enter both products as their codebook levels.
// PRE: the rotation rows (rr) are already loaded, and the queries (qin) too when q_ready.
template <int BITS, int D, int GQ, int NW, bool LUT = false, bool PRE = false>
__device__ void hist_seg(const DecodeArgs& a, int b, int kv, int p0, int p1, float* po, float* pl,
                         float (*o_lds)[2 * GQ][D], float (*st_lds)[3][8], HistQueryLds<D, GQ, NW>& qlds,
                         QRotRows<D, NW * kWave>& rr, QueryIn<D, GQ, NW * kWave>& qin, bool q_ready) {
  constexpr int NT = NW * kWave;
  // Load ring of NB page buffers, taken as NB/2 page pairs (compile-time indices). With six pages
  // (below GQA 8) the QK^T products run one pair ahead: the matrix cores work on pair k+1 while the vector units
  // run the softmax of pair k, and the loads of pair k+2 are in flight. Wide workgroups (four
  // wavefronts per SIMD, 128 registers each) keep four pages: the loads of pair k+1 in flight while
  // pair k is processed, and the other wavefronts of the SIMD fill the gaps.
  constexpr int NB = NW >= 8 ? OSCAR_WIDE_RING : (BITS == 2 ? kHistPipe2 : kHistPipe4);
  // at GQA 8 the products are formed right before their softmax: the two results held one pair
  // ahead do not fit the register bound of three workgroups per compute unit
  constexpr bool AHEAD = NB >= 6 && GQ < 8 && NW < 8;
  static_assert(NB % 2 == 0 && NB >= 4 && kIdChunk % NB == 0, "the ring holds whole page pairs");
  // the furthest prefetch of a chunk's last trip reads lane kIdChunk + NB - 3 of the current chunk
  static_assert(kIdChunk + NB - 3 < kWave, "every prefetch of a trip finds its id in the current chunk");
  const Dims& dm = a.dm;
  const int tid = threadIdx.x, lane = tid % kWave, c = lane % 16;
  const int wave = uniform(tid / kWave);
  const int ppw = (p1 - p0 + NW - 1) / NW;
  const int wp0 = uniform(min(p0 + wave * ppw, p1));
  const int wp1 = uniform(min(wp0 + ppw, p1));
  const int32_t* pt = (BITS == 2 ? a.pt2 : a.pt4) + (size_t)b * dm.pt_stride;
  const size_t qbase = (size_t)b * dm.hq + (size_t)kv * GQ;

  // Loads first, side by side: the page ids of this wavefront's first two chunks, the rows of R_K and
  // the queries of the group for the query prologue.
  // region of this width's page ids: INT2 ids [0, off4), INT4 ids [off4, pool_pages) (ids are 32-bit)
  const int64_t off4 = dm.mixed ? dm.off4 : dm.pool_pages;
  const int id_first = BITS == 2 ? 0 : (int)min<int64_t>(off4, INT32_MAX);
  const int id_lim = (int)min<int64_t>(BITS == 2 ? off4 : dm.pool_pages, INT32_MAX);
  int cur = page_chunk(pt, wp0, wp1, lane);
  int nxt = page_chunk(pt, wp0 + kIdChunk, wp1, lane);
  if (!PRE) rr.load(a.rot_k + (size_t)kv * D * D, tid);
  if (!PRE || !q_ready) qin.load(a.q + qbase * D, tid);
  const HistCounts hc = hist_counts(a, b);
  const int ntok = uniform(BITS == 2 ? hc.n2 : hc.n4);   // so every page limit is a scalar

  // byte selector of the PV operand gather at GQA width 4 (lo/lo halves on lanes 0..3 of a row,
  // hi/hi halves on lanes 4..7, zero elsewhere)
  const uint32_t psel = c < 4 ? 0x05040100u : (c < 8 ? 0x03020706u : 0x0C0C0C0Cu);
  WaveState<D, GQ> st;
  st.init();
  if (dm.pool_pages > 0) {
    int cbase = wp0;
    // Page-head address of a page (uniform): invalid ids and the prefetches past the range read
    // zeros without touching memory.
    const int64_t head = qpage_head_bytes(D, BITS);
    const uint64_t region = (uint64_t)a.pool + (BITS == 2 ? 0 : (uint64_t)(off4 * qpage_head_bytes(D, 2) * dm.hkv));
    auto load = [&](QPage<BITS, D, GQ>& pr, int pg) -> bool {
      const int li = pg - cbase;
      const int id = page_index(__builtin_amdgcn_readlane(cur, min(li, kWave - 1)), id_first, id_lim);
      const bool live = pg < wp1 && id >= 0;
      const uint64_t ad = region + (uint64_t)(((int64_t)max(id, 0) * dm.hkv + kv) * head);
      load_qpage<BITS, D, GQ>(pr, ad, live, lane);
      return live;
    };
    QPage<BITS, D, GQ> buf[NB];
    bool ok[NB];
#pragma unroll
    for (int k = 0; k < NB - 2; ++k) ok[k] = load(buf[k], wp0 + k);
    __builtin_amdgcn_sched_barrier(0);  // every prefetch is issued before the query prologue waits
    half8_t bq[D / 32];
    float uh, ul, esc;
    hist_query_operands<BITS, D, GQ, NW, LUT>(rr, qin, qlds, a.scale_log2e, bq, uh, ul, esc);
    OSCAR_TL_SPLIT(3);
    const float uq = uh + ul;   // sum of the query operand of this lane's head
    const Codebook cbk = load_codebook(LUT ? a.codebook : nullptr, kv, 0);
    const Codebook cbv = load_codebook(LUT ? a.codebook : nullptr, kv, 1);
    float4_t acc0, acc1;
    if constexpr (AHEAD) {
      acc0 = qk_page<BITS, D, GQ, LUT>(buf[0], bq, cbk);
      acc1 = qk_page<BITS, D, GQ, LUT>(buf[1], bq, cbk);
    }
    for (int pg = wp0; pg < wp1; pg += NB) {
      progress_priority(pg - wp0, wp1 - wp0);
      if (pg - cbase >= kIdChunk) {   // the next chunk of page ids becomes the current one
        cur = nxt;
        cbase += kIdChunk;
        nxt = page_chunk(pt, cbase + kIdChunk, wp1, lane);
      }
#pragma unroll
      for (int k = 0; k < NB; k += 2) {
        ok[(k + NB - 2) % NB] = load(buf[(k + NB - 2) % NB], pg + k + NB - 2);
        ok[(k + NB - 1) % NB] = load(buf[(k + NB - 1) % NB], pg + k + NB - 1);
        if (pg + k < wp1) {
          float4_t n0, n1;
          if constexpr (AHEAD) {
            n0 = qk_page<BITS, D, GQ, LUT>(buf[(k + 2) % NB], bq, cbk);
            n1 = qk_page<BITS, D, GQ, LUT>(buf[(k + 3) % NB], bq, cbk);
          } else {
            acc0 = qk_page<BITS, D, GQ, LUT>(buf[k], bq, cbk);
            acc1 = qk_page<BITS, D, GQ, LUT>(buf[k + 1], bq, cbk);
          }
          // a page past the range is masked; a page id outside the pool or of the other width is
          // masked and flagged (every page of the range carries at least one token)
          if (ok[k] || ok[k + 1]) {
            process_qpair<BITS, D, GQ, LUT>(st, buf[k], buf[k + 1], acc0, acc1, uq, esc, psel,
                                            ok[k] ? ntok - (pg + k) * kPage : 0,
                                            ok[k + 1] ? ntok - (pg + k + 1) * kPage : 0, lane, cbv);
          }
          if ((!ok[k] || (!ok[k + 1] && pg + k + 1 < wp1)) && lane == 0) atomicOr(a.ws.flags, 1u);
          if constexpr (AHEAD) {
            acc0 = n0;
            acc1 = n1;
          }
        }
      }
    }
  } else if (lane == 0 && wp0 < wp1) {
    atomicOr(a.ws.flags, 1u);
  }
  OSCAR_TL_SPLIT(4);
  // the merge buffers share LDS with the query prologue: every wavefront is past its prologue
  __syncthreads();
  OSCAR_TL_SPLIT(8);
  // wavefronts past the segment's pages hold the empty state
  workgroup_merge<D, GQ, LUT ? 0 : BITS, Redist<GQ>::on, NW>(st, o_lds, st_lds, po, pl);
}

// History segment of a one-request launch with interleaved pages (INT2-only cache, wide
// workgroups): history page p belongs to history unit p mod nunits and, within it, to wavefront
// (p / nunits) mod NW, so wavefront w of unit `unit` takes pages unit + nunits * (w + NW * r),
// r = 0, 1, ... Which pages a wavefront may take does not depend on the request's length, so its
// page ids, the rotation rows and the queries all load at once, before the length is known; the
// length only bounds r. Units differ by at most one page, and so do the wavefronts of a unit.
// LUT as in hist_seg.
template <int D, int GQ, int NW, bool LUT = false>
__device__ void hist_seg_b1(const DecodeArgs& a, int kv, int unit, int nunits, float* po, float* pl,
                            float (*o_lds)[2 * GQ][D], float (*st_lds)[3][8], HistQueryLds<D, GQ, NW>& qlds) {
  constexpr int BITS = 2, NT = NW * kWave, NB = OSCAR_WIDE_RING;
  static_assert(NB % 2 == 0 && NB >= 4 && kIdChunk % NB == 0, "the ring holds whole page pairs");
  static_assert(kIdChunk + NB - 3 < kWave, "every prefetch of a trip finds its id in the current chunk");
  const Dims& dm = a.dm;
  const int tid = threadIdx.x, lane = tid % kWave, c = lane % 16;
  const int wave = uniform(tid / kWave);
  const int base = unit + nunits * wave, stride = nunits * NW;
  // Page ids of list entries cb .. cb + 63 of this wavefront (lane i: entry cb + i); entries past the
  // page table's row read as 0 and are never used (the length bounds the list below).
  const __amdgpu_buffer_rsrc_t ptr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.pt2), (short)0, (int)(4 * max(dm.pt_stride, 0)), kRawBufferFlags);
  auto chunk = [&](int cb) -> int {
    const int64_t pg = (int64_t)base + (int64_t)stride * (cb + lane);
    const int off = pg < dm.pt_stride ? (int)pg : dm.pt_stride;
    return __builtin_amdgcn_raw_buffer_load_b32(ptr, 4 * off, 0, 0);
  };
  // the rotation rows and the queries first: the query products wait for them, and a wait on a
  // load waits for every load issued before it (the page ids come from the page table in HBM,
  // while the rotation rows are mostly in L2)
  QRotRows<D, NT> rr;
  QueryIn<D, GQ, NT> qin;
  rr.load(a.rot_k + (size_t)kv * D * D, tid);
  qin.load(a.q + (size_t)kv * GQ * D, tid);
  int cur = chunk(0);
  int nxt = chunk(kIdChunk);
  const HistCounts hc = hist_counts(a, 0);
  const int ntok = uniform(hc.n2);
  const int npages = min((ntok + kPage - 1) / kPage, dm.pt_stride);
  const int R = uniform(npages > base ? (npages - base + stride - 1) / stride : 0);   // this wavefront's pages
  OSCAR_TL_SPLIT(1);
  OSCAR_TL_SPLIT_VALUE(6, 4u | ((uint32_t)(R * NW) << 8));
  OSCAR_TL_SPLIT(2);

  const uint32_t psel = c < 4 ? 0x05040100u : (c < 8 ? 0x03020706u : 0x0C0C0C0Cu);
  WaveState<D, GQ> st;
  st.init();
  if (dm.pool_pages > 0) {
    int cbase = 0;
    const int64_t head = qpage_head_bytes(D, BITS);
    const int id_lim = (int)min<int64_t>(dm.pool_pages, INT32_MAX);
    const uint64_t region = (uint64_t)a.pool;
    auto load = [&](QPage<BITS, D, GQ>& pr, int r) -> bool {
      const int li = r - cbase;
      const int id = page_index(__builtin_amdgcn_readlane(cur, min(li, kWave - 1)), 0, id_lim);
      const bool live = r < R && id >= 0;
      const uint64_t ad = region + (uint64_t)(((int64_t)max(id, 0) * dm.hkv + kv) * head);
      load_qpage<BITS, D, GQ>(pr, ad, live, lane);
      return live;
    };
    QPage<BITS, D, GQ> buf[NB];
    bool ok[NB];
    // The first pages load before the length is known (they only need their ids): a page past the
    // history is read and then masked. They are requested once the wavefront's query products are
    // done, i.e. once its rotation rows have arrived: requested at entry, their traffic delayed the
    // rotation rows, which every wavefront waits for at the prologue's barrier. The rest of the
    // ring goes by the length.
    half8_t bq[D / 32];
    float uh, ul, esc;
    hist_query_operands<BITS, D, GQ, NW, LUT>(rr, qin, qlds, a.scale_log2e, bq, uh, ul, esc, [&]() {
#pragma unroll
      for (int k = 0; k < NB - 2; ++k) {
        const int id = page_index(__builtin_amdgcn_readlane(cur, k), 0, id_lim);
        load_qpage<BITS, D, GQ>(buf[k], region + (uint64_t)(((int64_t)max(id, 0) * dm.hkv + kv) * head), id >= 0,
                                lane);
        ok[k] = id >= 0;
      }
      OSCAR_TL_SPLIT(9);
    });
    OSCAR_TL_SPLIT(3);
#pragma unroll
    for (int k = 0; k < NB - 2; ++k) ok[k] = ok[k] && k < R;
    const float uq = uh + ul;
    const Codebook cbk = load_codebook(LUT ? a.codebook : nullptr, kv, 0);
    const Codebook cbv = load_codebook(LUT ? a.codebook : nullptr, kv, 1);
    for (int r = 0; r < R; r += NB) {
      progress_priority(r, R);
      if (r - cbase >= kIdChunk) {   // the next chunk of page ids becomes the current one
        cur = nxt;
        cbase += kIdChunk;
        nxt = chunk(cbase + kIdChunk);
      }
#pragma unroll
      for (int k = 0; k < NB; k += 2) {
        ok[(k + NB - 2) % NB] = load(buf[(k + NB - 2) % NB], r + k + NB - 2);
        ok[(k + NB - 1) % NB] = load(buf[(k + NB - 1) % NB], r + k + NB - 1);
        if (r + k < R) {
          const float4_t acc0 = qk_page<BITS, D, GQ, LUT>(buf[k], bq, cbk);
          const float4_t acc1 = qk_page<BITS, D, GQ, LUT>(buf[k + 1], bq, cbk);
          const int t0 = (base + stride * (r + k)) * kPage;   // first token of each page
          const int t1 = t0 + stride * kPage;
          if (ok[k] || ok[k + 1]) {
            process_qpair<BITS, D, GQ, LUT>(st, buf[k], buf[k + 1], acc0, acc1, uq, esc, psel,
                                            ok[k] ? ntok - t0 : 0, ok[k + 1] ? ntok - t1 : 0, lane, cbv);
          }
          if ((!ok[k] || (!ok[k + 1] && r + k + 1 < R)) && lane == 0) atomicOr(a.ws.flags, 1u);
        }
        if (r == 0 && k == 0) OSCAR_TL_SPLIT(10);
      }
    }
  } else if (lane == 0 && R > 0) {
    atomicOr(a.ws.flags, 1u);
  }
  OSCAR_TL_SPLIT(4);
  OSCAR_TL_SPLIT(8);
  // o_lds and st_lds are not shared with the query prologue's LDS: the state goes out at once, and
  // the merge's own barrier waits for the other wavefronts
  workgroup_merge<D, GQ, LUT ? 0 : BITS, Redist<GQ>::on, NW>(st, o_lds, st_lds, po, pl);
}

// LDS of the segments (one at a time per workgroup); 16-byte aligned for the vector reads of the
// query operands
template <int D, int GQ, int NW>
union alignas(16) SplitScratch {
  HistQueryLds<D, GQ, NW> hist;
  StepLds<D, GQ> step;
  float o[NW][2 * GQ][D];   // workgroup merge of the history and window segments
};

// Workgroups of a split launch that a compute unit should hold: three at GQA 8 in an INT2-only
// cache (the register count is then bounded to fit), one of the wide workgroups, else what the
// resources give.
// LDS of the one-request launch: the merge buffer has its own space, so a wavefront writes its
// state as soon as its pages are done, while others still read the query prologue's LDS.
template <int D, int GQ, int NW>
struct alignas(16) SplitB1Scratch {
  union alignas(16) Seg {
    HistQueryLds<D, GQ, NW> hist;
    StepLds<D, GQ> step;
  } seg;
  float o[NW][2 * GQ][D];   // workgroup merge of the history or window segment
};

template <int GQ, bool MIXED, int NW>
constexpr int kSplitMinBlocks = NW >= 16 ? 1 : (NW >= 8 ? 2 : ((GQ == 8 && !MIXED) ? 3 : 1));

// One workgroup per unit of the work plan: workgroup g is unit (g / Hkv) of kv-head g % Hkv. It
// runs the segments its cost range holds, in order: the step, window pages, INT2 pages, INT4 pages,
// each writing its own partial (window: original basis; history: rotated basis); the partials of
// kinds the unit does not hold get lse = -inf. The first unit of kv-head 0 of each request records
// the request's units for the merge.
// CB: the INT2 history uses the codebook table of the decode arguments. MIXED: the cache has INT4
// pages (an INT2-only launch carries no INT4 segment, which keeps its register count down).
// Wide workgroups (NW = 16, one per compute unit) load their rotation rows before the plan (the
// kv-head does not depend on it).
template <int D, int GQ, bool CB, bool MIXED, int NW>
__global__ __launch_bounds__(NW * kWave, (kSplitMinBlocks<GQ, MIXED, NW>)) void split_kernel(DecodeArgs a,
                                                                                         CacheWriteArgs cw) {
  constexpr int NT = NW * kWave;
  constexpr bool PRE = NW >= 16;
  __shared__ float st_lds[NW][3][8];
  __shared__ SplitScratch<D, GQ, NW> scr;
  OSCAR_TL_SPLIT(0);
#ifdef OSCAR_TIMELINE
  OSCAR_TL_SPLIT_VALUE(7, timeline_placement());
#endif
  const int hkv = a.dm.hkv;
  const int g = blockIdx.x, kv = g % hkv, tid = threadIdx.x;
  QRotRows<D, NT> rr;
  QueryIn<D, GQ, NT> qin;
  if constexpr (PRE) rr.load(a.rot_k + (size_t)kv * D * D, tid);
  const RequestUnits ru = request_units(a, g / hkv);   // the same in every wavefront
  OSCAR_TL_SPLIT(1);
  if (ru.b >= 0) {
    const int j = g / hkv - ru.first;
    int c0, c1;
    unit_range(ru, j, c0, c1);
    const Segments sg = unit_segments(a, ru.rc, c0, c1);
    float* po = a.ws.part_o + (size_t)g * 3 * GQ * D;
    float* pl = a.ws.part_lse + (size_t)g * 3 * GQ;
    const bool has[3] = {sg.window, sg.p20 < sg.p21, MIXED && sg.p40 < sg.p41};
    if (tid < 3 * GQ && !has[tid / GQ]) pl[tid] = kNegInf;
    if (kv == 0 && j == 0 && tid == 0) {
      a.ws.req_units[2 * ru.b] = ru.first;
      a.ws.req_units[2 * ru.b + 1] = ru.n;
    }
    OSCAR_TL_SPLIT_VALUE(6, (sg.step ? 1u : 0u) | (has[0] ? 2u : 0u) | (has[1] ? 4u : 0u) | (has[2] ? 8u : 0u) |
                                ((uint32_t)(has[1] ? sg.p21 - sg.p20 : sg.p41 - sg.p40) << 8));
    if (sg.step) {
      step_seg<D, GQ, NW>(a, cw, ru.b, kv, scr.step);
      __syncthreads();
    }
    if (has[0]) {
      window_seg<D, GQ, NW>(a, ru.b, kv, 0, 1, po, pl, scr.o, st_lds);
      __syncthreads();
    }
    OSCAR_TL_SPLIT(2);
    if (has[1]) {
      hist_seg<2, D, GQ, NW, CB, PRE>(a, ru.b, kv, sg.p20, sg.p21, po + GQ * D, pl + GQ, scr.o, st_lds, scr.hist,
                                       rr, qin, false);
      __syncthreads();
    }
    if constexpr (MIXED) {
      if (has[2])
        hist_seg<4, D, GQ, NW>(a, ru.b, kv, sg.p40, sg.p41, po + 2 * GQ * D, pl + 2 * GQ, scr.o, st_lds, scr.hist,
                               rr, qin, false);
    }
  }
  OSCAR_TL_SPLIT(5);
}

// The split launch of one request over an INT2-only cache in wide workgroups, with interleaved
// history pages: unit 0 of each kv-head runs the step and the window; units 1 .. n-1 share the
// history page by page (hist_seg_b1), so none of them waits for a work plan.
template <int D, int GQ, bool CB, int NW>
__global__ __launch_bounds__(NW * kWave, 1) void split_b1_kernel(DecodeArgs a, CacheWriteArgs cw) {
  __shared__ float st_lds[NW][3][8];
  __shared__ SplitB1Scratch<D, GQ, NW> scr;
  OSCAR_TL_SPLIT(0);
#ifdef OSCAR_TIMELINE
  OSCAR_TL_SPLIT_VALUE(7, timeline_placement());
#endif
  const int hkv = a.dm.hkv;
  const int g = blockIdx.x, kv = g % hkv, tid = threadIdx.x, u = g / hkv;
  float* po = a.ws.part_o + (size_t)g * 3 * GQ * D;
  float* pl = a.ws.part_lse + (size_t)g * 3 * GQ;
  if (u == 0) {
    if (tid < 2 * GQ) pl[GQ + tid] = kNegInf;   // no history partials
    if (kv == 0 && tid == 0) {
      a.ws.req_units[0] = 0;
      a.ws.req_units[1] = a.ws.units_per_kv;
    }
    OSCAR_TL_SPLIT(1);
    OSCAR_TL_SPLIT_VALUE(6, (a.step ? 1u : 0u) | 2u);
    if (a.step) {
      step_seg<D, GQ, NW>(a, cw, 0, kv, scr.seg.step);
      __syncthreads();
    }
    window_seg<D, GQ, NW>(a, 0, kv, 0, 1, po, pl, scr.o, st_lds);
    OSCAR_TL_SPLIT(2);
  } else {
    if (tid < 2 * GQ) pl[tid < GQ ? tid : GQ + tid] = kNegInf;   // no window or INT4 partials
    hist_seg_b1<D, GQ, NW, CB>(a, kv, u - 1, a.ws.units_per_kv - 1, po + GQ * D, pl + GQ, scr.o, st_lds,
                               scr.seg.hist);
  }
  OSCAR_TL_SPLIT(5);
}

// ------------------------------------------------------------------ merge
// One 1024-thread workgroup per (request, kv-head, group of HPW query heads) merges every partial
// of the (request, kv-head) for its heads, in one pass -- the window, INT2 and INT4 partials of each
// of the request's units (found through the unit table the split writes; kinds a unit does not hold
// carry lse = -inf) and the step's two one-token partials: each thread folds
// its slots with a running maximum (lse in log2 units), the threads' states are combined through
// LDS, the history sum (rotated basis of the values) is un-rotated with R_V^T (each R_V row read
// once per workgroup) and added to the window sum.
constexpr int kMergeThreads = 1024;
// The merge is latency-bound: a launch gets the fewest query heads per workgroup (HW) that still
// fits one workgroup per compute unit (a merge workgroup's LDS holds R_V, so a unit runs one).
constexpr int kMergeWorkgroupsPerRound = 256;

struct MergeState {
  float m, wsum;   // running maximum (log2) and weight sum
  float4 ah, aw;   // weighted history / window sums of this thread's float4 column
};
struct MergeCtx {
  int first, units; // the request's units
  int kv, bk;
  int n;           // slots: 3 per unit (window, INT2, INT4; one per unit in the interleaved launch), then 2 step slots in a fused step
  const float* rv; // R_V of the kv-head [D][D]
  int grp, hh, c4, tid;   // hh: query head within the kv group
};

// Partial slot i of a merge: its lse and o addresses (lse slot, o row of head hh) and whether it
// is in the original basis (window) or the rotated one (history).
template <int D, int GQ>
__device__ __forceinline__ void merge_slot(const DecodeArgs& a, const MergeCtx& c, int i, size_t& lse_at,
                                           size_t& o_at, bool& window, bool& step) {
  // interleaved one-request launch: unit 0 holds only the window partial, the others only INT2
  const bool il = a.ws.interleave != 0;
  const int nu = il ? c.units : 3 * c.units;
  step = i >= nu;
  if (step) {
    const size_t s = (size_t)c.bk * 2 + (i - nu);
    lse_at = s * GQ + c.hh;
    o_at = (s * GQ + c.hh) * D;
    window = i - nu == 1;
    return;
  }
  const int j = il ? i : i / 3, kind = il ? (i == 0 ? 0 : 1) : i - 3 * j;
  window = kind == 0;
  const size_t slot = ((size_t)a.dm.hkv * (c.first + j) + c.kv) * 3 + kind;
  lse_at = slot * GQ + c.hh;
  o_at = (slot * GQ + c.hh) * D;
}

// Folds slots base + grp + k*NG (k < MS) into the thread's state: every load is issued before any
// is consumed; `hook` runs between the two.
template <int D, int GQ, int MS, int NG, typename Hook = NoHook>
__device__ __forceinline__ void merge_fold(const DecodeArgs& a, MergeState& st, const MergeCtx& c, int base,
                                           Hook&& hook = Hook{}) {
  float lv[MS];
  float4 vv[MS];
  bool use[MS], win[MS];
#pragma unroll
  for (int k = 0; k < MS; ++k) {
    const int i = base + c.grp + k * NG;
    size_t la = 0, oa = 0;
    bool window = false, step = false;
    const bool live = i < c.n;
    if (live) merge_slot<D, GQ>(a, c, i, la, oa, window, step);
    use[k] = live;
    win[k] = window;
    const float* pl = step ? a.ws.step_lse : a.ws.part_lse;
    const float* po = step ? a.ws.step_o : a.ws.part_o;
    lv[k] = live ? pl[la] : kNegInf;
    vv[k] = live ? *reinterpret_cast<const float4*>(po + oa + 4 * c.c4) : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  hook();   // loads that are needed later go out behind this batch's
#pragma unroll
  for (int k = 0; k < MS; ++k) {
    // slots past the last and empty partials (lse = -inf: no such segment, or no token) weigh 0
    const float l = use[k] ? lv[k] : kNegInf;
    const bool live = l != kNegInf;
    const float m_new = fmaxf(st.m, l);
    const float sc = st.m == m_new ? 1.0f : __builtin_amdgcn_exp2f(st.m - m_new);   // 0 when m is -inf
    const float w = live ? __builtin_amdgcn_exp2f(l - m_new) : 0.0f;
    st.m = m_new;
    st.wsum = fmaf(st.wsum, sc, w);
    const float4 v = live ? vv[k] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    const float wh = win[k] ? 0.0f : w, ww = win[k] ? w : 0.0f;
    st.ah.x = fmaf(st.ah.x, sc, wh * v.x);
    st.ah.y = fmaf(st.ah.y, sc, wh * v.y);
    st.ah.z = fmaf(st.ah.z, sc, wh * v.z);
    st.ah.w = fmaf(st.ah.w, sc, wh * v.w);
    st.aw.x = fmaf(st.aw.x, sc, ww * v.x);
    st.aw.y = fmaf(st.aw.y, sc, ww * v.y);
    st.aw.z = fmaf(st.aw.z, sc, ww * v.z);
    st.aw.w = fmaf(st.aw.w, sc, ww * v.w);
  }
}

template <int D, int GQ, int HW>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeArgs a, CacheWriteArgs cw) {
  constexpr int NT = kMergeThreads;
  constexpr int C4 = D / 4;           // float4 columns of a partial
  constexpr int TPH = NT / HW;        // threads per head
  constexpr int NG = TPH / C4;        // slot groups per head
  constexpr int SUB = NT / (HW * D);  // combine: threads per output column (adjacent lanes)
  constexpr int GPS = NG / SUB;       // slot groups per combine thread (4)
  constexpr int NP = NT / D;          // un-rotation: threads per R_V row (adjacent lanes)
  constexpr int RP = D / NP;          // contiguous entries of the row per thread
  constexpr int AS = D + 4;           // padded LDS row of a group's sums
  static_assert(GPS * SUB == NG && NP * RP == D && SUB <= 16 && NP <= 16 && RP % 4 == 0, "merge thread layout");
  __shared__ __attribute__((aligned(16))) float acc_h[NG][HW][AS];
  __shared__ __attribute__((aligned(16))) float acc_w[NG][HW][AS];
  __shared__ float m_s[NG][HW], w_s[NG][HW];
  __shared__ float hsum[HW][D], wsum_s[HW][D], wtot_s[HW];
  OSCAR_TL_MERGE(0);
  const Dims& dm = a.dm;
  const int bk = blockIdx.x / (GQ / HW), h0 = HW * (blockIdx.x % (GQ / HW));
  const int kv = bk % dm.hkv, b = bk / dm.hkv;
  const int tid = threadIdx.x;
  const int hl = tid / TPH, r = tid % TPH, c4 = r % C4, grp = r / C4;
  // fused step: the new token's window slot is written at the end (every window read of the step
  // is done). Its length is fetched now as a vector load (an atomic load is never scalarised): it
  // then shares the round trip of the partial loads instead of stalling the wavefront ahead of them.
  const bool ring_wg = a.step && h0 == 0 && tid < 2 * D;
  const int t_len = ring_wg ? __hip_atomic_load(a.seq_len + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
  // one request owns every unit (no table read); otherwise the table the split wrote
  const bool single = dm.batch == 1;
  const int first = single ? 0 : a.ws.req_units[2 * b];
  const int units = single ? a.ws.units_per_kv : a.ws.req_units[2 * b + 1];
  const int n = (a.ws.interleave ? units : 3 * units) + (a.step ? 2 : 0);
  // Slots are taken up to 12 at a time per thread: every load of a batch is issued (slots no segment
  // wrote are not read) before any is consumed, and the first batch's loads share one round trip
  // with the R_V staging.
  MergeState ms_st{kNegInf, 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  const MergeCtx mc{first, units, kv, bk, n, a.rot_v + (size_t)kv * D * D, grp, h0 + hl, c4, tid};
  // the thread's RP contiguous entries of its R_V row for the un-rotation, requested right behind
  // the first batch of partials (so the fold waits for the partials only; R_V is read straight into
  // registers, not staged in LDS)
  const int uj = tid / NP, upart = tid % NP;
  float4 rvr[RP / 4];
  auto load_rv = [&]() {
#pragma unroll
    for (int e = 0; e < RP / 4; ++e)
      rvr[e] = *reinterpret_cast<const float4*>(mc.rv + (size_t)uj * D + RP * upart + 4 * e);
  };
  const int per_thread = (n + NG - 1) / NG;   // uniform
  if (per_thread <= 4) {
    merge_fold<D, GQ, 4, NG>(a, ms_st, mc, 0, load_rv);
  } else if (per_thread <= 12) {
    merge_fold<D, GQ, 12, NG>(a, ms_st, mc, 0, load_rv);
  } else {
    merge_fold<D, GQ, 8, NG>(a, ms_st, mc, 0, load_rv);
    for (int base = 8 * NG; base < n; base += 8 * NG) merge_fold<D, GQ, 8, NG>(a, ms_st, mc, base);
  }
  OSCAR_TL_MERGE(1);
  *reinterpret_cast<float4*>(&acc_h[grp][hl][4 * c4]) = ms_st.ah;
  *reinterpret_cast<float4*>(&acc_w[grp][hl][4 * c4]) = ms_st.aw;
  if (c4 == 0) {
    m_s[grp][hl] = ms_st.m;
    w_s[grp][hl] = ms_st.wsum;
  }
  __syncthreads();
  // Combine the groups of each output column: lane group of SUB threads per column, thread `sub`
  // taking groups sub, sub + SUB, ... (so the lanes of a half-wavefront read distinct banks); the
  // maximum and the sums are folded across the SUB lanes.
  {
    const int col = tid / SUB, sub = tid % SUB;
    const int h2 = col / D, ch = col % D;
    float mg[GPS];
    float M = kNegInf;
#pragma unroll
    for (int q = 0; q < GPS; ++q) {
      mg[q] = m_s[sub + SUB * q][h2];
      M = fmaxf(M, mg[q]);
    }
    M = lanes_max<SUB>(M);
    float hs = 0.0f, ws = 0.0f, W = 0.0f;
#pragma unroll
    for (int q = 0; q < GPS; ++q) {
      const int gg = sub + SUB * q;
      const float e = mg[q] == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(mg[q] - M);
      hs = fmaf(e, acc_h[gg][h2][ch], hs);
      ws = fmaf(e, acc_w[gg][h2][ch], ws);
      W = fmaf(e, w_s[gg][h2], W);
    }
    hs = lanes_sum<SUB>(hs);
    ws = lanes_sum<SUB>(ws);
    W = lanes_sum<SUB>(W);
    if (sub == 0) {
      hsum[h2][ch] = hs;
      wsum_s[h2][ch] = ws;
      if (ch == 0) wtot_s[h2] = W;
    }
  }
  __syncthreads();
  OSCAR_TL_MERGE(3);
  // un-rotation: thread (j, part) forms part of out[h][j] = sum_i hsum[h][i] R_V[j][i] over
  // i = RP part .. RP part + RP - 1 (its registers); the parts are folded across the NP lanes of row j
  {
    const int j = uj, part = upart;
    float acc[HW];
#pragma unroll
    for (int h2 = 0; h2 < HW; ++h2) acc[h2] = 0.0f;
#pragma unroll
    for (int k = 0; k < RP; ++k) {
      const float4& r4 = rvr[k / 4];
      const float rji = (k % 4 == 0) ? r4.x : ((k % 4 == 1) ? r4.y : ((k % 4 == 2) ? r4.z : r4.w));
#pragma unroll
      for (int h2 = 0; h2 < HW; ++h2) acc[h2] = fmaf(hsum[h2][RP * part + k], rji, acc[h2]);
    }
#pragma unroll
    for (int h2 = 0; h2 < HW; ++h2) acc[h2] = lanes_sum<NP>(acc[h2]);
    if (part == 0) {
#pragma unroll
      for (int h2 = 0; h2 < HW; ++h2) {
        const float W = wtot_s[h2];
        const size_t o = ((size_t)b * dm.hq + (size_t)kv * GQ + h0 + h2) * D + j;
        a.out[o] = W > 0.0f ? (acc[h2] + wsum_s[h2][j]) / W : 0.0f;
      }
    }
  }
  OSCAR_TL_MERGE(5);
  if (ring_wg && t_len < dm.max_seq_len) {   // the step ran for this request (it had room)
    // the new token takes its window slot (the demoted token's ring slot, or position T), as the
    // demote kernel writes it
    int pgw, t;
    window_slot(t_len < 0 ? 0 : t_len, dm, pgw, t);
    const int sel = tid / D, ch = tid % D;
    uint16_t* pg = reinterpret_cast<uint16_t*>(cw.window + ((size_t)bk * dm.wpages + pgw) * bf16_page_head_bytes(D));
    pg[sel ? bf16_value_index(D, t, ch) : bf16_key_index(D, t, ch)] = (sel ? cw.v : cw.k)[(size_t)bk * D + ch];
  }
}

// ------------------------------------------------------------------ BF16 baseline split
template <int D, int GQ>
__global__ __launch_bounds__(256) void bf16_paged_split_kernel(Bf16Args a) {
  __shared__ float o_lds[4][2 * GQ][D];
  __shared__ float st_lds[4][3][8];
  const Dims& dm = a.dm;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane / 16;
  const int s = blockIdx.x % a.s;
  const int bk = blockIdx.x / a.s;
  const int kv = bk % dm.hkv, b = bk / dm.hkv;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int npages = min((T + kPage - 1) / kPage, dm.pt_stride);
  const int pg0 = s * 4 * a.ppw;
  if (pg0 >= npages) return;
  const int wp0 = pg0 + wave * a.ppw;
  const int wp1 = min(wp0 + a.ppw, npages);
  u32x4_t bq[D / 32];
  load_bf16_query<D, GQ>(bq, a.q, (size_t)b * dm.hq + (size_t)kv * GQ, lane);
  WaveState<D, GQ> st;
  st.init();
  const int my_pid = (wp0 + lane < wp1) ? a.pt[(size_t)b * dm.pt_stride + wp0 + lane] : -1;
  const int64_t pbytes = bf16_page_head_bytes(D);
  if (dm.pool_pages > 0) {
    page_pipeline<kBf16Pipe, Bf16Page<D>>(
        wp0, wp1,
        [&](Bf16Page<D>& pr, int pg) -> bool {
          const int64_t page = pg < wp1 ? (int64_t)__builtin_amdgcn_readlane(my_pid, pg - wp0) : -1;
          const bool valid = page >= 0 && page < dm.pool_pages;
          load_bf16_page<D>(pr, a.pages + (valid ? (page * dm.hkv + kv) * pbytes : 0), lane);
          return valid;
        },
        [&](const Bf16Page<D>& pr, bool valid, int pg) {
          if (valid) {
            bool tv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) tv[r] = kPage * pg + 4 * g + r < T;
            process_bf16_page<D, GQ>(st, pr, bq, tv, a.scale_log2e, lane);
          } else if (lane == 0) {
            atomicOr(a.flags, 1u);
          }
        });
  } else if (lane == 0) {
    atomicOr(a.flags, 1u);
  }
  const size_t pbase = ((size_t)b * dm.hkv + kv) * a.s + s;
  workgroup_merge<D, GQ, 16>(st, o_lds, st_lds, a.part_o + pbase * GQ * D, a.part_lse + pbase * GQ);
}

// ------------------------------------------------------------------ BF16 baseline merge
// LSE-merge of n partial slots (slot i at slot_of(i)) for one query head into o[D] and its lse.
// All lse values are fetched first; the weighted sum then issues independent float4 loads.
template <int D>
__device__ void merge_slots(const float* po, const float* pl, size_t sbase, int gq, int hh, int n, int first, int n_a,
                            int base_b, float* wl, float* red, float (*acc_s)[D], float* o_out, float* lse_out) {
  constexpr int C4 = D / 4;          // float4 columns
  constexpr int NG = 256 / C4;       // slot groups
  const int tid = threadIdx.x;
  auto slot_of = [&](int i) { return i < n_a ? first + i : base_b + (i - n_a); };
  float m = kNegInf;
  for (int i = tid; i < n; i += 256) {
    const float l = pl[(sbase + slot_of(i)) * gq + hh];
    wl[i] = l;
    m = fmaxf(m, l);
  }
  red[tid] = m;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float ws = 0.0f;
  for (int i = tid; i < n; i += 256) {
    const float w = (M == kNegInf || wl[i] == kNegInf) ? 0.0f : exp2f(wl[i] - M);
    wl[i] = w;
    ws += w;
  }
  red[tid] = ws;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float W = red[0];
  const int c4 = tid % C4, grp = tid / C4;
  float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int i = grp; i < n; i += NG) {
    const float w = wl[i];
    const float4 v = *reinterpret_cast<const float4*>(po + ((sbase + slot_of(i)) * gq + hh) * D + 4 * c4);
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  acc_s[grp][4 * c4 + 0] = acc.x;
  acc_s[grp][4 * c4 + 1] = acc.y;
  acc_s[grp][4 * c4 + 2] = acc.z;
  acc_s[grp][4 * c4 + 3] = acc.w;
  __syncthreads();
  if (tid < D) {
    float o = 0.0f;
    for (int gg = 0; gg < NG; ++gg) o += acc_s[gg][tid];
    o_out[tid] = W > 0.0f ? o / W : 0.0f;
  }
  if (tid == 0) *lse_out = (M == kNegInf || !(W > 0.0f)) ? kNegInf : M + log2f(W);
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(256) void bf16_merge_kernel(Bf16Args a) {
  __shared__ float wl[kMaxSlots];
  __shared__ float red[256];
  __shared__ float acc_s[256 / (D / 4)][D];
  __shared__ float o_s[D];
  __shared__ float lse_s[1];
  const Dims& dm = a.dm;
  const int hq_i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int gq = dm.gq, kv = hq_i / gq, hh = hq_i % gq;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int n = (min((T + kPage - 1) / kPage, dm.pt_stride) + 4 * a.ppw - 1) / (4 * a.ppw);
  const size_t sbase = ((size_t)b * dm.hkv + kv) * a.s;
  merge_slots<D>(a.part_o, a.part_lse, sbase, gq, hh, n, 0, n, 0, wl, red, acc_s, o_s, &lse_s[0]);
  if (tid < D) a.out[((size_t)b * dm.hq + hq_i) * D + tid] = o_s[tid];
}

// ------------------------------------------------------------------ launchers
template <int D, int GQ, bool CB, bool MIXED, int NW>
static const void* split_symbol() {
  return reinterpret_cast<const void*>(&split_kernel<D, GQ, CB, MIXED, NW>);
}

// The split kernel instance of a launch (wide workgroups exist for GQA width 4 only; `il`: the
// interleaved one-request launch, INT2-only).
template <int D, int GQ>
static const void* split_function(bool cb, bool mixed, int nw, bool il = false) {
  if constexpr (GQ == 4) {
    if (nw == kSplitWavesWide) {
      if (il) {
        if (mixed) return nullptr;
        return cb ? reinterpret_cast<const void*>(&split_b1_kernel<D, GQ, true, kSplitWavesWide>)
                  : reinterpret_cast<const void*>(&split_b1_kernel<D, GQ, false, kSplitWavesWide>);
      }
      if (mixed) return cb ? split_symbol<D, GQ, true, true, kSplitWavesWide>() : split_symbol<D, GQ, false, true, kSplitWavesWide>();
      return cb ? split_symbol<D, GQ, true, false, kSplitWavesWide>() : split_symbol<D, GQ, false, false, kSplitWavesWide>();
    }
  }
  if (nw != kSplitWaves) return nullptr;
  if (mixed) return cb ? split_symbol<D, GQ, true, true, kSplitWaves>() : split_symbol<D, GQ, false, true, kSplitWaves>();
  return cb ? split_symbol<D, GQ, true, false, kSplitWaves>() : split_symbol<D, GQ, false, false, kSplitWaves>();
}

static const void* split_function_of(int d, int gq, bool cb, bool mixed, int nw) {
#define OSCAR_DISPATCH(DD, GG) \
  if (d == DD && gq == GG) return split_function<DD, GG>(cb, mixed, nw);
  OSCAR_DISPATCH(128, 1) OSCAR_DISPATCH(128, 2) OSCAR_DISPATCH(128, 4) OSCAR_DISPATCH(128, 8)
  OSCAR_DISPATCH(64, 1) OSCAR_DISPATCH(64, 2) OSCAR_DISPATCH(64, 4) OSCAR_DISPATCH(64, 8)
#undef OSCAR_DISPATCH
  return nullptr;
}

int split_workgroups_per_cu(int d, int gq, bool cb, bool mixed, int nw) {
  const void* f = split_function_of(d, gq, cb, mixed, nw);
  int n = 0;
  if (!f || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, nw * kWave, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <int D, int GQ>
static hipError_t launch_decode_t(const DecodeArgs& a, const CacheWriteArgs& cw, hipStream_t stream) {
  const Dims& dm = a.dm;
  const void* f = split_function<D, GQ>(a.codebook != nullptr, dm.mixed != 0, a.ws.nw, a.ws.interleave != 0);
  if (!f) return hipErrorInvalidValue;
  // the timing variant records event 0, then brackets the split kernel with the dispatch's own
  // start and stop stamps (events 1 and 2), so its interval is the kernel's execution time
  if (a.events) (void)hipEventRecord(a.events[0], stream);
  const dim3 grid(dm.hkv * a.ws.units_per_kv), block(a.ws.nw * kWave);
  DecodeArgs args = a;
  CacheWriteArgs cwa = cw;
  void* kargs[] = {&args, &cwa};
  hipError_t e = a.events ? hipExtLaunchKernel(f, grid, block, kargs, 0, stream, a.events[1], a.events[2], 0)
                          : hipLaunchKernel(f, grid, block, kargs, 0, stream);
  if (e != hipSuccess) return e;
  const int groups = dm.batch * dm.hkv;
  bool merged = false;
  if constexpr (GQ >= 2) {
    if (groups * GQ <= kMergeWorkgroupsPerRound) {
      hipLaunchKernelGGL((merge_kernel<D, GQ, 1>), dim3(groups * GQ), dim3(kMergeThreads), 0, stream, a, cw);
      merged = true;
    }
  }
  if constexpr (GQ >= 4) {
    if (!merged && groups * GQ / 2 <= kMergeWorkgroupsPerRound) {
      hipLaunchKernelGGL((merge_kernel<D, GQ, 2>), dim3(groups * GQ / 2), dim3(kMergeThreads), 0, stream, a, cw);
      merged = true;
    }
  }
  if (!merged) hipLaunchKernelGGL((merge_kernel<D, GQ, GQ>), dim3(groups), dim3(kMergeThreads), 0, stream, a, cw);
  if (a.events) (void)hipEventRecord(a.events[3], stream);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, const CacheWriteArgs& cw, hipStream_t stream) {
  if (a.dm.batch == 0) return hipSuccess;
  const int d = a.dm.d, gq = a.dm.gq;
#define OSCAR_DISPATCH(DD, GG) \
  if (d == DD && gq == GG) return launch_decode_t<DD, GG>(a, cw, stream);
  OSCAR_DISPATCH(128, 1) OSCAR_DISPATCH(128, 2) OSCAR_DISPATCH(128, 4) OSCAR_DISPATCH(128, 8)
  OSCAR_DISPATCH(64, 1) OSCAR_DISPATCH(64, 2) OSCAR_DISPATCH(64, 4) OSCAR_DISPATCH(64, 8)
#undef OSCAR_DISPATCH
  return hipErrorInvalidValue;
}

template <int D, int GQ>
static hipError_t launch_bf16_decode_t(const Bf16Args& b, hipStream_t stream) {
  hipLaunchKernelGGL((bf16_paged_split_kernel<D, GQ>), dim3(b.dm.batch * b.dm.hkv * b.s), dim3(256), 0, stream, b);
  hipLaunchKernelGGL((bf16_merge_kernel<D>), dim3(b.dm.hq, b.dm.batch), dim3(256), 0, stream, b);
  return hipGetLastError();
}

hipError_t launch_bf16_decode(const Bf16Args& b, hipStream_t stream) {
  if (b.dm.batch == 0) return hipSuccess;
  const int d = b.dm.d, gq = b.dm.gq;
#define OSCAR_DISPATCH(DD, GG) \
  if (d == DD && gq == GG) return launch_bf16_decode_t<DD, GG>(b, stream);
  OSCAR_DISPATCH(128, 1) OSCAR_DISPATCH(128, 2) OSCAR_DISPATCH(128, 4) OSCAR_DISPATCH(128, 8)
  OSCAR_DISPATCH(64, 1) OSCAR_DISPATCH(64, 2) OSCAR_DISPATCH(64, 4) OSCAR_DISPATCH(64, 8)
#undef OSCAR_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace oscar

#ifdef OSCAR_TIMELINE
// Diagnostic library only: copies the timeline table (rows of 8 uint64, split rows then merge rows)
// to host memory, or clears it. Synchronous.
extern "C" int oscar_timeline_read(void* host, size_t bytes) {
  if (bytes > sizeof(oscar::g_timeline)) bytes = sizeof(oscar::g_timeline);
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(oscar::g_timeline), bytes, 0, hipMemcpyDeviceToHost);
}
extern "C" int oscar_timeline_clear(void) {
  static uint64_t zero[oscar::kTimelineSplitRows + oscar::kTimelineMergeRows][oscar::kTimelineCols];
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(oscar::g_timeline), zero, sizeof(zero), 0, hipMemcpyHostToDevice);
}
#endif
