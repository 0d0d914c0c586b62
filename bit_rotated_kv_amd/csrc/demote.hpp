// Device code shared by the cache writers and the fused decode step: history page-head
// addressing, packed code stores, the rotation on the matrix cores (one arithmetic for every
// writer), and the per-step demote of the oldest recent token.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace oscar {

__device__ inline bool page_ok(int64_t page, int bits, const Dims& dm) {
  if (page < 0 || page >= dm.pool_pages) return false;
  if (!dm.mixed) return bits == 2;
  return bits == 2 ? page < dm.off4 : page >= dm.off4;
}

__device__ inline uint8_t* page_head_mut(uint8_t* pool, int64_t page, int kv, const Dims& dm) {
  return const_cast<uint8_t*>(page_head_addr(pool, page, kv, dm.hkv, dm.d, dm.mixed ? dm.off4 : dm.pool_pages));
}

// Key codes of slot t: whole 32-bit words owned by the slot (plain stores).
__device__ inline void store_key_codes(uint8_t* ph, int d, int bits, int t, const uint8_t* cs, int tid, int nthr) {
  const int cb = d * bits / 32;  // bytes of one lane's key part
  const int nwl = cb / 4;
  for (int idx = tid; idx < 4 * nwl; idx += nthr) {
    const int g = idx / nwl, a = idx % nwl;
    uint32_t w = 0;
    if (bits == 2) {
      for (int k2 = 0; k2 < 2; ++k2)
        for (int m = 0; m < 4; ++m)
          for (int hf = 0; hf < 2; ++hf) {
            const int ch = 32 * (2 * a + k2) + 8 * g + 2 * m + hf;
            w |= (uint32_t)cs[ch] << (8 * k2 + 2 * m + 16 * hf);
          }
    } else {
      for (int m = 0; m < 4; ++m)
        for (int hf = 0; hf < 2; ++hf) {
          const int ch = 32 * a + 8 * g + 2 * m + hf;
          w |= (uint32_t)cs[ch] << (4 * m + 16 * hf);
        }
    }
    reinterpret_cast<uint32_t*>(ph + key_part_offset(bits, cb, 16 * g + t))[a] = w;
  }
}

// Value codes of slot t: each word is shared by the 4 slots of a token group, so the slot's bits
// are replaced with atomic and/or.
__device__ inline void store_value_codes(uint8_t* ph, int d, int bits, int t, const uint8_t* cs, int tid, int nthr) {
  const int cb = d * bits / 32;
  const int nwl = cb / 4;
  const int g = t / 4, m = (t % 4) / 2, hf = t % 2;
  for (int idx = tid; idx < 16 * nwl; idx += nthr) {
    const int c = idx / nwl, a = idx % nwl;
    uint32_t mask = 0, val = 0;
    if (bits == 2) {
      for (int n4 = 0; n4 < 4; ++n4) {
        const int ch = 16 * (4 * a + n4) + c;
        const int bit = 2 * n4 + 8 * m + 16 * hf;
        mask |= 3u << bit;
        val |= (uint32_t)cs[ch] << bit;
      }
    } else {
      for (int n2 = 0; n2 < 2; ++n2) {
        const int ch = 16 * (2 * a + n2) + c;
        const int bit = 4 * n2 + 8 * m + 16 * hf;
        mask |= 15u << bit;
        val |= (uint32_t)cs[ch] << bit;
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(ph + value_part_offset(bits, cb, 16 * g + c)) + a;
    atomicAnd(dst, ~mask);
    atomicOr(dst, val);
  }
}

// ------------------------------------------------------------------ rotation on the matrix cores
// x_rot = x . R for bf16 rows x and the fp32 rotation R of a kv-head, with
// v_mfma_f32_32x32x16_bf16. R is split exactly into three bf16 parts, R = R_hi + R_mid + R_lo (each
// the round-to-nearest-even bf16 of what the previous parts leave; 8 + 8 + 8 significant bits
// cover fp32's 24), so every product x_k * R_part[k][n] is exact and only the fp32 accumulation
// rounds. The accumulation order is fixed -- 16-channel k-steps in ascending order, and within a
// k-step the parts lo, mid, hi -- and a row's result depends on that row alone, so the prefill,
// the demote and the fused decode step give a token the same x_rot and the same codes. The
// prefill holds its wavefront's slice of R in registers across tiles (RotSlice, rotate_tile);
// the single-row writers read it as fp32 and split it one k-step at a time (rotate_rows_loaded) in the
// same order.
//
// Operand layout of the 32x32x16 product (lane l, row/column m = n = l % 32): A holds row m,
// channels 16*kk + 8*(l/32) .. +7; B holds those channels of output column n; the 16 accumulators
// of lane l are rows 8*(j/4) + 4*(l/32) + j%4 of column n.
typedef float float16v_t __attribute__((ext_vector_type(16)));

// The three bf16 parts of the rotation entries r[0..7] (exact: r = hi + mid + lo). Each part is the
// round-to-nearest-even bf16 of what the previous parts leave (the hardware conversion,
// v_cvt_pk_bf16_f32, two entries per instruction); the residuals are exact fp32 differences.
__device__ __forceinline__ void split_rotation(const float (&r)[8], bf16x8_t& hi, bf16x8_t& mid, bf16x8_t& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)r[i];
    const float r1 = r[i] - (float)h;   // exact
    const __bf16 m = (__bf16)r1;
    const float r2 = r1 - (float)m;     // exact, at most 8 significant bits
    hi[i] = h;
    mid[i] = m;
    lo[i] = (__bf16)r2;                 // exact
  }
}

// The rotation entries of lane `lane` for k-step kk of the slice of wavefront w (column 32w + l%32).
template <int D>
__device__ __forceinline__ void rotation_entries(const float* rot, int w, int kk, int lane, float (&r)[8]) {
  const int n = 32 * w + lane % 32;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = rot[(size_t)(16 * kk + 8 * (lane / 32) + i) * D + n];
}

// A operand of lane `lane` for k-step kk: row lane % 32 of x (zero for rows >= nrows).
template <typename XPtr>
__device__ __forceinline__ bf16x8_t rotation_a(XPtr x, int stride, int nrows, int kk, int lane) {
  const int m = lane % 32;
  u32x4_t w = {0, 0, 0, 0};
  if (m < nrows) w = *reinterpret_cast<const u32x4_t*>(x + (size_t)m * stride + 16 * kk + 8 * (lane / 32));
  return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ float16v_t rotation_step(const bf16x8_t& a, const bf16x8_t& hi, const bf16x8_t& mid,
                                                    const bf16x8_t& lo, float16v_t acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, mid, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, acc, 0, 0, 0);
}

template <int D>
struct RotSlice {
  static constexpr int KS = D / 16;       // k-steps
  static constexpr int SLICES = D / 32;   // 32-column slices (wavefronts 0..SLICES-1 hold one)
  bf16x8_t hi[KS], mid[KS], lo[KS];
  // wavefront w < SLICES: columns 32w .. 32w+31 of rot ([D][D] fp32, row-major)
  __device__ void load(const float* rot, int w, int lane) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float r[8];
      rotation_entries<D>(rot, w, kk, lane, r);
      split_rotation(r, hi[kk], mid[kk], lo[kk]);
    }
  }
};

// Rows 0..31 of x (bf16 bits; row m at x + m * stride, rows m >= nrows read as zero) times the
// wavefront's slice of R held in registers. Returns the accumulators of lane `lane`.
template <int D, typename XPtr>
__device__ __forceinline__ float16v_t rotate_tile(const RotSlice<D>& rs, XPtr x, int stride, int nrows, int lane) {
  bf16x8_t a[RotSlice<D>::KS];
#pragma unroll
  for (int kk = 0; kk < RotSlice<D>::KS; ++kk) a[kk] = rotation_a(x, stride, nrows, kk, lane);
  float16v_t acc = {};
#pragma unroll
  for (int kk = 0; kk < RotSlice<D>::KS; ++kk) acc = rotation_step(a[kk], rs.hi[kk], rs.mid[kk], rs.lo[kk], acc);
  return acc;
}

// rotate_tile for the single-row writers: the slice of wavefront w is read from rot as fp32 (every
// entry loaded before the first product, one round trip to memory) and split as in RotSlice; the
// same products in the same order.
template <int D, typename XPtr>
__device__ __forceinline__ float16v_t rotate_rows_loaded(const float* rot, int w, XPtr x, int stride, int nrows,
                                                         int lane) {
  float r[D / 16][8];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) rotation_entries<D>(rot, w, kk, lane, r[kk]);
  float16v_t acc = {};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    bf16x8_t hi, mid, lo;
    split_rotation(r[kk], hi, mid, lo);
    acc = rotation_step(rotation_a(x, stride, nrows, kk, lane), hi, mid, lo, acc);
  }
  return acc;
}

// ------------------------------------------------------------------ demote
// Page id of history slot `slot` of width bw for request b; -1 when the slot lies past the page
// table.
__device__ inline int64_t demote_page(const CacheWriteArgs& a, int b, int slot, int bw) {
  const int32_t* pt = (bw == 4 ? a.pt4 : a.pt2) + (size_t)b * a.dm.pt_stride;
  return (slot >= 0 && slot / kPage < a.dm.pt_stride) ? pt[slot / kPage] : -1;
}

// Window page and slot that hold position p (p >= 0): sink page p / 16 below the sink length,
// else recent-ring slot p mod recent.
__device__ inline void window_slot(int p, const Dims& dm, int& pgw, int& t) {
  if (p < dm.sink) {
    pgw = p / kPage;
    t = p % kPage;
  } else {
    const int s = p % dm.recent;
    pgw = dm.sink / kPage + s / kPage;
    t = s % kPage;
  }
}

// One wavefront: range of the rotated token xr[0..D), clipped grid of width bw, and its codes
// (cs) and packed bf16 (scale, zero) (szs, scale in the low half); INT2 codes follow the codebook
// when one is given.
template <int D>
__device__ inline void quantize_token(const float* xr, float clip, int bw, uint8_t* cs, uint32_t* szs, int lane,
                                      const Codebook& cb) {
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  for (int c = lane; c < D; c += kWave) {
    mn = fminf(mn, xr[c]);
    mx = fmaxf(mx, xr[c]);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int levels = (1 << bw) - 1;
  const QuantGrid g = make_grid(mn, mx, clip, levels);
  if (bw == 2 && cb.on)
    for (int c = lane; c < D; c += kWave) cs[c] = (uint8_t)cb_code(xr[c], g, cb);
  else
    for (int c = lane; c < D; c += kWave) cs[c] = (uint8_t)quant_code(xr[c], g, levels);
  if (lane == 0) *szs = g.s_bits | (g.z_bits << 16);
}

// Stores the codes and (scale, zero) of one token -- key (sel 0) or value (sel 1) -- into slot
// ts of history page `page` (skipped for an id outside the pool or of the other width).
template <int D>
__device__ inline void store_token(const CacheWriteArgs& a, int64_t page, int kv, int bw, int ts, int sel,
                                   const uint8_t* cs, uint32_t szs, int tid, int nthr) {
  if (!page_ok(page, bw, a.dm)) return;
  uint8_t* ph = page_head_mut(a.pool, page, kv, a.dm);
  if (sel == 0)
    store_key_codes(ph, D, bw, ts, cs, tid, nthr);
  else
    store_value_codes(ph, D, bw, ts, cs, tid, nthr);
  if (tid == 0) reinterpret_cast<uint32_t*>(ph + 4 * D * bw)[2 * ts + sel] = szs;
}

// One workgroup per (K or V, kv-head, request). With T = seq_len[b] >= sink + recent, the token at
// position T - recent (the oldest of the recent window) is read from its ring slot, rotated
// (x . R), clipped, quantised and packed into the next history slot of its width; the new token
// then takes the freed ring slot (else position T of the window). The rotation column and the
// request's page id are fetched before anything waits on them.
template <int D>
__device__ inline void demote_block(const CacheWriteArgs& a, int sel, int kv, int b) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[D];
  __shared__ float xr[D];
  __shared__ uint8_t cs[D];
  __shared__ uint32_t szs;
  const Dims& dm = a.dm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const float* rot = (sel ? a.rot_v : a.rot_k) + (size_t)kv * D * D;
  const int T = a.seq_len[b] < 0 ? 0 : a.seq_len[b];
  const int64_t pb = bf16_page_head_bytes(D);
  uint8_t* wb = a.window + (size_t)(b * dm.hkv + kv) * dm.wpages * pb;
  const bool demote = T >= dm.sink + dm.recent;
  const int n4 = (dm.mixed && a.n_int4) ? a.n_int4[b] : 0;
  int bw = 2;
  if (demote) {
    bw = (dm.mixed && a.bits && a.bits[b] == 4) ? 4 : 2;
    const int hist_before = T - dm.sink - dm.recent;
    const int slot = bw == 4 ? n4 : hist_before - n4;
    const int64_t page = demote_page(a, b, slot, bw);
    int pgw, t;
    window_slot(T - dm.recent, dm, pgw, t);
    const uint16_t* pg = reinterpret_cast<const uint16_t*>(wb + pgw * pb);
    if (tid < D) xs[tid] = pg[sel ? bf16_value_index(D, t, tid) : bf16_key_index(D, t, tid)];
    __syncthreads();
    if (wave < D / 32) {
      const float16v_t acc = rotate_rows_loaded<D>(rot, wave, xs, D, 1, lane);
      if (lane < 32) xr[32 * wave + lane] = acc[0];   // row 0
    }
    __syncthreads();
    if (wave == 0) {
      const float clip = bw == 4 ? (sel ? a.clip_v4 : a.clip_k4) : (sel ? a.clip_v : a.clip_k);
      quantize_token<D>(xr, clip, bw, cs, &szs, lane, load_codebook(a.codebook, kv, sel));
    }
    __syncthreads();
    store_token<D>(a, page, kv, bw, slot % kPage, sel, cs, szs, tid, 256);
    __syncthreads();
  }
  {
    int pgw, t;
    window_slot(T, dm, pgw, t);
    uint16_t* pg = reinterpret_cast<uint16_t*>(wb + pgw * pb);
    const size_t src = ((size_t)b * dm.hkv + kv) * D;
    if (tid < D) {
      if (sel == 0)
        pg[bf16_key_index(D, t, tid)] = a.k[src + tid];
      else
        pg[bf16_value_index(D, t, tid)] = a.v[src + tid];
    }
  }
  if (sel == 0 && kv == 0 && tid == 0) {
    if (a.seq_len_out) a.seq_len_out[b] = T + 1;
    if (a.n_int4_out) a.n_int4_out[b] = n4 + ((demote && bw == 4) ? 1 : 0);
  }
}

}  // namespace oscar
