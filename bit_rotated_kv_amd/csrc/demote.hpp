// Device code shared by the cache writers and the fused decode step: history page-head
// addressing, packed code stores, the fp32 rotation in a fixed summation order, and the per-step
// demote of the oldest recent token.
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
  const int cb = d * bits / 32;  // bytes of the key part of a lane chunk
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
    reinterpret_cast<uint32_t*>(ph + (size_t)(16 * g + t) * 2 * cb)[a] = w;
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
    uint32_t* dst = reinterpret_cast<uint32_t*>(ph + (size_t)(16 * g + c) * 2 * cb + cb) + a;
    atomicAnd(dst, ~mask);
    atomicOr(dst, val);
  }
}

// ------------------------------------------------------------------ rotation order
// x_rot[j] = sum_i x[i] R[i][j] in fp32, always in the same order so that the prefill and the
// demote write identical codes for a token: the input channels are split into four quarters, each
// quarter is a fused-multiply-add chain in ascending order, and the quarter sums are added as
// (q0 + q1) + (q2 + q3). A workgroup of 256 threads holds column j of R split in 256/D parts
// (thread (j, part)) in registers.
template <int D>
struct RotCol {
  static constexpr int NP = 256 / D;  // parts per column
  static constexpr int RP = D / NP;   // rows per part
  float r[RP];
  __device__ void load(const float* rot, int j, int part) {
#pragma unroll
    for (int i = 0; i < RP; ++i) r[i] = rot[(part * RP + i) * D + j];
  }
  // partial sum of this part over the input row x (LDS, broadcast reads)
  __device__ float part_sum(const float* x, int part) const {
    constexpr int Q = D / 4;
    float qa = 0.0f, qb = 0.0f;
#pragma unroll
    for (int i = 0; i < Q; ++i) qa = fmaf(x[part * RP + i], r[i], qa);
    if constexpr (RP == 2 * Q) {
#pragma unroll
      for (int i = 0; i < Q; ++i) qb = fmaf(x[part * RP + Q + i], r[Q + i], qb);
      return qa + qb;
    } else {
      return qa;
    }
  }
  // combines the NP part sums (stride apart) into the final value
  __device__ static float combine(const float* p, int stride) {
    if constexpr (NP == 2) return p[0] + p[stride];
    else return (p[0] + p[stride]) + (p[2 * stride] + p[3 * stride]);
  }
};

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
// (cs) and packed bf16 (scale, zero) (szs, scale in the low half).
template <int D>
__device__ inline void quantize_token(const float* xr, float clip, int bw, uint8_t* cs, uint32_t* szs, int lane) {
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  for (int c = lane; c < D; c += kWave) {
    mn = fminf(mn, xr[c]);
    mx = fmaxf(mx, xr[c]);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int levels = (1 << bw) - 1;
  const QuantGrid g = make_grid(mn, mx, clip, levels);
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
  constexpr int NP = RotCol<D>::NP;
  __shared__ float xs[D];
  __shared__ float parts[NP][D];
  __shared__ float xr[D];
  __shared__ uint8_t cs[D];
  __shared__ uint32_t szs;
  const Dims& dm = a.dm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int j = tid % D, part = tid / D;
  RotCol<D> rc;
  rc.load((sel ? a.rot_v : a.rot_k) + (size_t)kv * D * D, j, part);
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
    if (tid < D) xs[tid] = bf16_bits_to_f32(pg[sel ? bf16_value_index(D, t, tid) : bf16_key_index(D, t, tid)]);
    __syncthreads();
    parts[part][j] = rc.part_sum(xs, part);
    __syncthreads();
    if (tid < D) xr[tid] = RotCol<D>::combine(&parts[0][tid], D);
    __syncthreads();
    if (wave == 0) {
      const float clip = bw == 4 ? (sel ? a.clip_v4 : a.clip_k4) : (sel ? a.clip_v : a.clip_k);
      quantize_token<D>(xr, clip, bw, cs, &szs, lane);
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
