// Cache writers: prefill (sink/recent windows and rotated+quantised history pages), the per-step
// demote of the oldest recent token (OSCAR overview page, method paragraph; study note, SGLang
// case), and the fill of the full-BF16 baseline cache.
#include "common.hpp"
#include "launch.hpp"
#include "demote.hpp"

namespace oscar {

// Position held by window page j, slot t when T tokens are in cache, or -1 if the slot is empty.
// Sink pages hold positions 0..sink-1; ring slot s holds the latest position p < T with
// p % recent == s, when p >= sink.
__device__ inline int window_position(int j, int t, int T, int sink, int recent) {
  if (j < sink / kPage) {
    const int p = kPage * j + t;
    return (p < T) ? p : -1;
  }
  if (T <= sink) return -1;
  const int s = kPage * (j - sink / kPage) + t;
  int back = (T - 1 - s) % recent;
  if (back < 0) back += recent;
  const int p = T - 1 - back;
  return (p >= sink) ? p : -1;
}

// ------------------------------------------------------------------ prefill: window + counts
__global__ __launch_bounds__(256) void prefill_window_kernel(CacheWriteArgs a) {
  const Dims& dm = a.dm;
  const int kv = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = dm.d;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int64_t pb = bf16_page_head_bytes(d);
  uint8_t* wb = a.window + (size_t)(b * dm.hkv + kv) * dm.wpages * pb;
  const size_t src = ((size_t)b * dm.hkv + kv) * dm.max_seq_len;
  for (int idx = tid; idx < dm.wpages * kPage * d; idx += 256) {
    const int slot = idx / d, ch = idx % d, j = slot / kPage, t = slot % kPage;
    const int p = window_position(j, t, T, dm.sink, dm.recent);
    const uint16_t kb = p >= 0 ? a.k[(src + p) * d + ch] : (uint16_t)0;
    const uint16_t vb = p >= 0 ? a.v[(src + p) * d + ch] : (uint16_t)0;
    uint16_t* pg = reinterpret_cast<uint16_t*>(wb + j * pb);
    pg[bf16_key_index(d, t, ch)] = kb;
    pg[bf16_value_index(d, t, ch)] = vb;
  }
  if (kv == 0 && a.n_int4_out) {
    __shared__ int red[256];
    int cnt = 0;
    const int h1 = T - dm.recent;
    if (a.bits && dm.mixed)
      for (int p = dm.sink + tid; p < h1; p += 256) cnt += a.bits[(size_t)b * dm.max_seq_len + p] == 4;
    red[tid] = cnt;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    if (tid == 0) a.n_int4_out[b] = red[0];
  }
}

// ------------------------------------------------------------------ prefill: history pages
// One workgroup per (32-position chunk of the history, kv-head, request).
template <int D>
__global__ __launch_bounds__(256) void prefill_hist_kernel(CacheWriteArgs a) {
  constexpr int CH = 32;                    // positions per workgroup
  constexpr int NP = RotCol<D>::NP;
  __shared__ float xs[CH * D];              // inputs, then rotated rows
  __shared__ float parts[NP][CH * D];
  __shared__ uint8_t cs[CH * D];
  __shared__ uint32_t szs[CH];
  __shared__ int slot_s[CH];
  __shared__ int bits_s[CH];
  __shared__ int red[256];
  const Dims& dm = a.dm;
  const int chunk = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int hist = T - dm.sink - dm.recent;
  if (CH * chunk >= hist) return;
  const int n = min(CH, hist - CH * chunk);
  const int p0 = dm.sink + CH * chunk;
  const uint8_t* bitsrow = (a.bits && dm.mixed) ? a.bits + (size_t)b * dm.max_seq_len : nullptr;

  // slot of each token: its rank among history tokens of the same width
  int before4 = 0;
  if (bitsrow) {
    int cnt = 0;
    for (int p = dm.sink + tid; p < p0; p += 256) cnt += bitsrow[p] == 4;
    red[tid] = cnt;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    before4 = red[0];
  }
  if (tid == 0) {
    int c4 = before4;
    for (int i = 0; i < n; ++i) {
      const int p = p0 + i;
      const int bw = (bitsrow && bitsrow[p] == 4) ? 4 : 2;
      bits_s[i] = bw;
      slot_s[i] = bw == 4 ? c4 : (p - dm.sink) - c4;
      c4 += bw == 4;
    }
  }
  const size_t src = ((size_t)b * dm.hkv + kv) * dm.max_seq_len;
  const int j = tid % D, part = tid / D;
  for (int sel = 0; sel < 2; ++sel) {
    const uint16_t* xsrc = sel ? a.v : a.k;
    RotCol<D> rc;
    rc.load((sel ? a.rot_v : a.rot_k) + (size_t)kv * D * D, j, part);
    __syncthreads();
    for (int idx = tid; idx < CH * D; idx += 256) {
      const int i = idx / D, c = idx % D;
      xs[idx] = i < n ? bf16_bits_to_f32(xsrc[(src + p0 + i) * D + c]) : 0.0f;
    }
    __syncthreads();
    for (int t = 0; t < n; ++t) parts[part][t * D + j] = rc.part_sum(xs + t * D, part);
    __syncthreads();
    for (int idx = tid; idx < n * D; idx += 256) xs[idx] = RotCol<D>::combine(&parts[0][idx], CH * D);
    __syncthreads();
    for (int i = wave; i < n; i += 4) {
      const int bw = bits_s[i];
      const float clip = bw == 4 ? (sel ? a.clip_v4 : a.clip_k4) : (sel ? a.clip_v : a.clip_k);
      float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
      for (int c = lane; c < D; c += kWave) {
        mn = fminf(mn, xs[i * D + c]);
        mx = fmaxf(mx, xs[i * D + c]);
      }
      mn = wave_min(mn);
      mx = wave_max(mx);
      const int levels = (1 << bw) - 1;
      const QuantGrid g = make_grid(mn, mx, clip, levels);
      for (int c = lane; c < D; c += kWave) cs[i * D + c] = (uint8_t)quant_code(xs[i * D + c], g, levels);
      if (lane == 0) szs[i] = g.s_bits | (g.z_bits << 16);
    }
    __syncthreads();
    // each wave writes the tokens it quantised
    for (int i = wave; i < n; i += 4) {
      const int bw = bits_s[i], slot = slot_s[i];
      const int32_t* pt = (bw == 4 ? a.pt4 : a.pt2) + (size_t)b * dm.pt_stride;
      if (slot / kPage >= dm.pt_stride) continue;
      const int64_t page = pt[slot / kPage];
      if (!page_ok(page, bw, dm)) continue;
      uint8_t* ph = page_head_mut(a.pool, page, kv, dm);
      const int t = slot % kPage;
      if (sel == 0)
        store_key_codes(ph, D, bw, t, cs + i * D, lane, kWave);
      else
        store_value_codes(ph, D, bw, t, cs + i * D, lane, kWave);
      if (lane == 0) reinterpret_cast<uint32_t*>(ph + 4 * D * bw)[2 * t + sel] = szs[i];
    }
  }
}

// ------------------------------------------------------------------ demote (one decode step)
// One workgroup per (K or V, kv-head, request): rotates, quantises and packs its half of the
// oldest recent token, then writes its half of the new token into the freed recent slot.
template <int D>
__global__ __launch_bounds__(256) void demote_kernel(CacheWriteArgs a) {
  demote_block<D>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ------------------------------------------------------------------ BF16 baseline cache fill
__global__ __launch_bounds__(256) void bf16_fill_kernel(Bf16Args a) {
  const Dims& dm = a.dm;
  const int j = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = dm.d;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  if (kPage * j >= T || j >= dm.pt_stride) return;
  const int64_t page = a.pt[(size_t)b * dm.pt_stride + j];
  if (page < 0 || page >= dm.pool_pages) return;
  uint16_t* pg = reinterpret_cast<uint16_t*>(a.pages + (page * dm.hkv + kv) * bf16_page_head_bytes(d));
  const size_t src = ((size_t)b * dm.hkv + kv) * dm.max_seq_len;
  for (int idx = tid; idx < kPage * d; idx += 256) {
    const int t = idx / d, ch = idx % d, p = kPage * j + t;
    pg[bf16_key_index(d, t, ch)] = p < T ? a.k[(src + p) * d + ch] : (uint16_t)0;
    pg[bf16_value_index(d, t, ch)] = p < T ? a.v[(src + p) * d + ch] : (uint16_t)0;
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_prefill(const CacheWriteArgs& a, hipStream_t stream) {
  const Dims& dm = a.dm;
  if (dm.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_window_kernel, dim3(dm.hkv, dm.batch), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int hmax = dm.max_seq_len - dm.sink - dm.recent;
  if (hmax <= 0) return hipSuccess;
  const dim3 grid((hmax + 31) / 32, dm.hkv, dm.batch);
  if (dm.d == 128)
    hipLaunchKernelGGL(prefill_hist_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_hist_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_demote(const CacheWriteArgs& a, hipStream_t stream) {
  const Dims& dm = a.dm;
  if (dm.batch == 0) return hipSuccess;
  if (dm.d == 128)
    hipLaunchKernelGGL(demote_kernel<128>, dim3(2, dm.hkv, dm.batch), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(demote_kernel<64>, dim3(2, dm.hkv, dm.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bf16_fill(const Bf16Args& a, hipStream_t stream) {
  const Dims& dm = a.dm;
  const int pages = (dm.max_seq_len + kPage - 1) / kPage;
  if (dm.batch == 0 || pages == 0) return hipSuccess;
  hipLaunchKernelGGL(bf16_fill_kernel, dim3(pages, dm.hkv, dm.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace oscar
