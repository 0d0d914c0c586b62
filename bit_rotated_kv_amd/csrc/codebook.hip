// Lloyd-Max fit of the INT2 codebook on the GPU (OSCAR overview page, the paragraph that sets OSCAR
// beside TurboQuant: a Lloyd-Max codebook with the attention-aware rotation). The samples are the
// group coordinates u = (clip(x) - z) / s of a kv-head's calibration rows, rotated and gridded
// exactly as the cache writers rotate and grid a token (so a fitted level sits where the encoder
// will put codes). Lloyd's iteration (Max, "Quantizing for minimum distortion", 1960) alternates
// nearest-level cells -- thresholds at the midpoints of the levels -- and cell means:
//   * cb_coord_kernel: once per fit, rotates 64-row chunks on the matrix cores and writes every
//     coordinate (fp32, the quantiser's own quotient; NaN marks a row whose scale is 0);
//   * cb_stats_kernel: once per iteration, the per-cell count and fp64 sum of the coordinates
//     under the current thresholds, as per-workgroup partials;
//   * the host adds the partials in a fixed order, moves each level to its cell mean (an empty cell
//     keeps its level) and stops a kv-head once no level moves by more than the tolerance.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "common.hpp"
#include "launch.hpp"
#include "demote.hpp"

namespace oscar {
namespace {

constexpr int kCoordRows = 64;       // rows per coordinate workgroup
constexpr int kStatsBlocks = 64;     // partials per kv-head and iteration
constexpr size_t kWsAlign = 256;

size_t ws_align(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct FitWs {
  float* u;                 // [Hkv][n][D] coordinates
  double* thr;              // [Hkv][3] thresholds of the current iteration
  double* psum;             // [Hkv][kStatsBlocks][4]
  unsigned long long* pcnt; // [Hkv][kStatsBlocks][4]
};

size_t fit_ws_layout(int hkv, int64_t n, int d, uint8_t* base, FitWs* ws) {
  size_t off = 0;
  const size_t u_off = off;
  off += ws_align((size_t)hkv * n * d * 4);
  const size_t t_off = off;
  off += ws_align((size_t)hkv * 3 * 8);
  const size_t s_off = off;
  off += ws_align((size_t)hkv * kStatsBlocks * 4 * 8);
  const size_t c_off = off;
  off += ws_align((size_t)hkv * kStatsBlocks * 4 * 8);
  if (ws && base) {
    ws->u = reinterpret_cast<float*>(base + u_off);
    ws->thr = reinterpret_cast<double*>(base + t_off);
    ws->psum = reinterpret_cast<double*>(base + s_off);
    ws->pcnt = reinterpret_cast<unsigned long long*>(base + c_off);
  }
  return off;
}

// Workgroup (chunk, kv): rows [64 chunk, 64 chunk + 64) of x[kv] ([n][D] bf16). Wavefront w < D/32
// holds the 32-column slice w of R in registers (as the prefill does) and rotates two 32-row tiles;
// then four threads per row find the row's range, form the INT2 grid and write its coordinates.
template <int D>
__global__ __launch_bounds__(256) void cb_coord_kernel(const uint16_t* __restrict__ x, const float* __restrict__ rot,
                                                       int64_t n, float clip, float* __restrict__ u) {
  constexpr int CH = kCoordRows;
  constexpr int XS = D + 8, RS = D + 8;
  constexpr int SL = RotSlice<D>::SLICES;
  __shared__ __attribute__((aligned(16))) uint16_t xs[CH][XS];
  __shared__ float xr[CH][RS];
  const int kv = blockIdx.y, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t r0 = (int64_t)blockIdx.x * CH;
  const int nr = (int)min((int64_t)CH, n - r0);
  RotSlice<D> rs;
  if (wave < SL) rs.load(rot + (size_t)kv * D * D, wave, lane);
  const uint16_t* src = x + ((size_t)kv * n + r0) * D;
  for (int idx = tid; idx < CH * D / 8; idx += 256) {
    const int row = idx / (D / 8), c8 = idx % (D / 8);
    u32x4_t w = {0, 0, 0, 0};
    if (row < nr) w = *reinterpret_cast<const u32x4_t*>(src + (size_t)row * D + 8 * c8);
    *reinterpret_cast<u32x4_t*>(&xs[row][8 * c8]) = w;
  }
  __syncthreads();
  if (wave < SL) {
#pragma unroll
    for (int tile = 0; tile < CH / 32; ++tile) {
      const float16v_t acc = rotate_tile<D>(rs, &xs[32 * tile][0], XS, nr - 32 * tile, lane);
#pragma unroll
      for (int j = 0; j < 16; ++j)
        xr[32 * tile + 8 * (j / 4) + 4 * (lane / 32) + j % 4][32 * wave + lane % 32] = acc[j];
    }
  }
  __syncthreads();
  constexpr int QC = D / 4;
  const int i = tid / 4, q = tid % 4;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  for (int c = 0; c < QC; ++c) {
    mn = fminf(mn, xr[i][q * QC + c]);
    mx = fmaxf(mx, xr[i][q * QC + c]);
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  if (i < nr) {
#pragma clang fp contract(off)
    const QuantGrid g = make_grid(mn, mx, clip, 3);
    float* dst = u + ((size_t)kv * n + r0 + i) * D + q * QC;
    for (int c = 0; c < QC; c += 4) {
      float4 o;
      float* of = &o.x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xc = fminf(fmaxf(xr[i][q * QC + c + e], g.lo), g.hi);
        of[e] = g.s == 0.0f ? __builtin_nanf("") : __fdiv_rn(xc - g.z, g.s);
      }
      *reinterpret_cast<float4*>(dst + c) = o;
    }
  }
}

__device__ __forceinline__ double shfl_xor_f64(double v, int o) {
  const unsigned long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(b & 0xFFFFFFFFull), o, kWave), hi = __shfl_xor((int)(b >> 32), o, kWave);
  return __longlong_as_double(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Workgroup (blk, kv): per-cell count and fp64 sum of the coordinates u[kv][i], i = blk*1024 + 4t +
// e (strided by the grid), under thresholds thr[kv]; a coordinate on a threshold goes to the even
// cell ([u > t0] + [u >= t1] + [u > t2]); NaN coordinates are skipped.
__global__ __launch_bounds__(256) void cb_stats_kernel(const float* __restrict__ u, int64_t per_head,
                                                       const double* __restrict__ thr, double* __restrict__ psum,
                                                       unsigned long long* __restrict__ pcnt) {
  __shared__ double s_sum[4][4];
  __shared__ unsigned long long s_cnt[4][4];
  const int kv = blockIdx.y, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const double t0 = thr[kv * 3 + 0], t1 = thr[kv * 3 + 1], t2 = thr[kv * 3 + 2];
  const float4* src = reinterpret_cast<const float4*>(u + (size_t)kv * per_head);
  const int64_t n4 = per_head / 4;
  double sum[4] = {0.0, 0.0, 0.0, 0.0};
  unsigned cnt[4] = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 v = src[i];
    const float ve[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double xd = ve[e];
      if (!(xd == xd)) continue;
      const int c = (int)(xd > t0) + (int)(xd >= t1) + (int)(xd > t2);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sum[k] += c == k ? xd : 0.0;
        cnt[k] += c == k ? 1u : 0u;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    double s = sum[k];
    unsigned long long m = cnt[k];
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      s += shfl_xor_f64(s, o);
      m += (unsigned long long)(unsigned)__shfl_xor((int)(unsigned)m, o, kWave);
    }
    if (lane == 0) {
      s_sum[wave][k] = s;
      s_cnt[wave][k] = m;
    }
  }
  __syncthreads();
  if (tid < 4) {
    double s = 0.0;
    unsigned long long m = 0;
    for (int w = 0; w < 4; ++w) {
      s += s_sum[w][tid];
      m += s_cnt[w][tid];
    }
    const size_t o = ((size_t)kv * gridDim.x + blockIdx.x) * 4 + tid;
    psum[o] = s;
    pcnt[o] = m;
  }
}

// fp64 -> fp16 pattern, round to nearest even (finite input).
uint16_t host_f64_to_f16(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  const double a = fabs(x);
  if (a >= 65520.0) return sign | 0x7C00u;                     // beyond the halfway point to 2^16
  if (a < 0x1p-14) return sign | (uint16_t)rint(a * 0x1p24);   // subnormal (1024 -> the smallest normal)
  int k;
  frexp(a, &k);                                                 // a = f 2^k, f in [0.5, 1)
  int e = k - 1;
  double m = rint((ldexp(a, -e) - 1.0) * 1024.0);
  if (m == 1024.0) {
    m = 0.0;
    ++e;
  }
  if (e > 15) return sign | 0x7C00u;
  return sign | (uint16_t)(((e + 15) << 10) | (int)m);
}

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" {

size_t oscar_codebook_workspace_bytes(int32_t num_kv_heads, int32_t n_rows, int32_t head_dim) {
  if (num_kv_heads <= 0 || n_rows < 0 || (head_dim != 64 && head_dim != 128)) return 0;
  return fit_ws_layout(num_kv_heads, n_rows, head_dim, nullptr, nullptr);
}

oscar_status_t oscar_codebook_fit(int32_t num_kv_heads, int32_t n_rows, int32_t head_dim, const void* x,
                                  const float* rot, float clip, int32_t max_iter, double tol, void* workspace,
                                  size_t workspace_bytes, double* levels_out, uint16_t* patterns_out,
                                  int32_t* iters_out, hipStream_t stream) {
  if (num_kv_heads <= 0 || n_rows < 0 || max_iter < 1 || !(tol >= 0.0) || !(clip > 0.0f && clip <= 1.0f))
    return OSCAR_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return OSCAR_ERR_UNSUPPORTED;
  if (!levels_out || !patterns_out) return OSCAR_ERR_INVALID_ARG;
  if (n_rows > 0 && (!x || !rot)) return OSCAR_ERR_INVALID_ARG;
  // per-workgroup cell counts are reduced in 32 bits: at most 2^31 coordinates per partial
  if ((int64_t)n_rows * head_dim > ((int64_t)kStatsBlocks << 31) || num_kv_heads > 65535) return OSCAR_ERR_UNSUPPORTED;
  const int hkv = num_kv_heads;
  const int64_t per_head = (int64_t)n_rows * head_dim;
  std::vector<double> lv((size_t)hkv * 4);
  std::vector<int> iters(hkv, 0);
  std::vector<char> live(hkv, 1);
  for (int h = 0; h < hkv; ++h)
    for (int j = 0; j < 4; ++j) lv[(size_t)h * 4 + j] = (double)j;   // the uniform levels
  FitWs ws{};
  if (n_rows > 0) {
    if (!workspace || workspace_bytes < fit_ws_layout(hkv, n_rows, head_dim, nullptr, nullptr))
      return OSCAR_ERR_WORKSPACE;
    fit_ws_layout(hkv, n_rows, head_dim, static_cast<uint8_t*>(workspace), &ws);
    const dim3 cgrid((unsigned)((n_rows + kCoordRows - 1) / kCoordRows), hkv);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (head_dim == 128)
      hipLaunchKernelGGL(cb_coord_kernel<128>, cgrid, dim3(256), 0, stream, xb, rot, (int64_t)n_rows, clip, ws.u);
    else
      hipLaunchKernelGGL(cb_coord_kernel<64>, cgrid, dim3(256), 0, stream, xb, rot, (int64_t)n_rows, clip, ws.u);
    if (hipGetLastError() != hipSuccess) return OSCAR_ERR_LAUNCH;
  }
  std::vector<double> thr((size_t)hkv * 3), psum((size_t)hkv * kStatsBlocks * 4);
  std::vector<unsigned long long> pcnt((size_t)hkv * kStatsBlocks * 4);
  for (int it = 1; it <= max_iter; ++it) {
    bool any = false;
    for (int h = 0; h < hkv; ++h) any |= live[h] != 0;
    if (!any) break;
    for (int h = 0; h < hkv; ++h)
      for (int j = 0; j < 3; ++j) thr[(size_t)h * 3 + j] = 0.5 * (lv[(size_t)h * 4 + j] + lv[(size_t)h * 4 + j + 1]);
    std::fill(psum.begin(), psum.end(), 0.0);
    std::fill(pcnt.begin(), pcnt.end(), 0ull);
    if (n_rows > 0) {
      if (hipMemcpyAsync(ws.thr, thr.data(), thr.size() * 8, hipMemcpyHostToDevice, stream) != hipSuccess)
        return OSCAR_ERR_LAUNCH;
      hipLaunchKernelGGL(cb_stats_kernel, dim3(kStatsBlocks, hkv), dim3(256), 0, stream, ws.u, per_head, ws.thr,
                         ws.psum, ws.pcnt);
      if (hipGetLastError() != hipSuccess) return OSCAR_ERR_LAUNCH;
      if (hipMemcpyAsync(psum.data(), ws.psum, psum.size() * 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipMemcpyAsync(pcnt.data(), ws.pcnt, pcnt.size() * 8, hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipStreamSynchronize(stream) != hipSuccess)
        return OSCAR_ERR_LAUNCH;
    }
    for (int h = 0; h < hkv; ++h) {
      if (!live[h]) continue;
      double moved = 0.0;
      for (int j = 0; j < 4; ++j) {
        double s = 0.0;
        unsigned long long m = 0;
        for (int k = 0; k < kStatsBlocks; ++k) {
          s += psum[((size_t)h * kStatsBlocks + k) * 4 + j];
          m += pcnt[((size_t)h * kStatsBlocks + k) * 4 + j];
        }
        if (m > 0) {
          const double nl = s / (double)m;
          moved = fmax(moved, fabs(nl - lv[(size_t)h * 4 + j]));
          lv[(size_t)h * 4 + j] = nl;
        }
      }
      iters[h] = it;
      if (moved <= tol) live[h] = 0;
    }
  }
  for (int h = 0; h < hkv; ++h) {
    for (int j = 0; j < 4; ++j) {
      levels_out[(size_t)h * 4 + j] = lv[(size_t)h * 4 + j];
      patterns_out[(size_t)h * 4 + j] = host_f64_to_f16(lv[(size_t)h * 4 + j]);
    }
    if (iters_out) iters_out[h] = iters[h];
  }
  return OSCAR_OK;
}

}  // extern "C"
