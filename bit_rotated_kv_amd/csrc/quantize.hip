// Canonical group quantise + pack of already-rotated fp32 rows (OSCAR overview page, method
// paragraph: clip, quantise, pack four 2-bit codes per byte; scale/zero restore).
#include "common.hpp"
#include "launch.hpp"

namespace oscar {

// One wavefront per (row, group). Each lane owns whole output bytes: lane j packs the
// 8/bits consecutive codes of byte j, so no cross-lane exchange is needed. With a codebook
// (INT2 only) the codes are its nearest-level decisions on the same grid.
__global__ __launch_bounds__(256) void quantize_pack_kernel(int64_t rows, int dim, int group, int bits,
                                                            float clip, const float* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint16_t* __restrict__ sz, Codebook cb) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int ng = dim / group;
  const int per = 8 / bits;
  const int levels = (1 << bits) - 1;
  const int64_t total = rows * ng;
  for (int64_t task = (int64_t)blockIdx.x * 4 + wave; task < total; task += (int64_t)gridDim.x * 4) {
    const int64_t row = task / ng;
    const int gi = (int)(task % ng);
    const float* xp = x + row * dim + (int64_t)gi * group;
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    for (int i = lane; i < group; i += kWave) {
      const float v = xp[i];
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    const QuantGrid g = make_grid(mn, mx, clip, levels);
    uint8_t* cp = codes + row * (dim / per) + (int64_t)gi * (group / per);
    for (int j = lane; j < group / per; j += kWave) {
      uint32_t b = 0;
      if (cb.on)
        for (int e = 0; e < per; ++e) b |= cb_code(xp[j * per + e], g, cb) << (bits * e);
      else
        for (int e = 0; e < per; ++e) b |= quant_code(xp[j * per + e], g, levels) << (bits * e);
      cp[j] = (uint8_t)b;
    }
    if (lane == 0) {
      sz[task * 2 + 0] = (uint16_t)g.s_bits;
      sz[task * 2 + 1] = (uint16_t)g.z_bits;
    }
  }
}

hipError_t launch_quantize_pack(int64_t rows, int dim, int group, int bits, float clip, const float* x,
                                uint8_t* codes, uint16_t* sz, const uint16_t* levels, hipStream_t stream) {
  Codebook cb{};
  cb.on = levels != nullptr;
  if (cb.on) {
    // thresholds as the kernels form them: fp32 midpoints of the fp16 levels (exact)
    float l[4];
    for (int j = 0; j < 4; ++j) l[j] = host_f16_to_f32(levels[j]);
    cb.lut_lo = levels[0] | ((uint32_t)levels[1] << 16);
    cb.lut_hi = levels[2] | ((uint32_t)levels[3] << 16);
    cb.t0 = (l[0] + l[1]) * 0.5f;
    cb.t1 = (l[1] + l[2]) * 0.5f;
    cb.t2 = (l[2] + l[3]) * 0.5f;
  }
  const int64_t tasks = rows * (dim / group);
  if (tasks == 0) return hipSuccess;
  int64_t blocks = (tasks + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quantize_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rows, dim, group, bits,
                     clip, x, codes, sz, cb);
  return hipGetLastError();
}

}  // namespace oscar
