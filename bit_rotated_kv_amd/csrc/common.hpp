// Shared device/host helpers of the OSCAR gfx950 kernels: layout arithmetic, bf16/fp16 bit
// conversions, matrix-core operand types and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <string.h>
#include <stdint.h>

#include "oscar.h"

namespace oscar {

constexpr int kPage = 16;       // tokens per page
constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kMetaBytes = 128; // 16 token slots x {sK, zK, sV, zV} bf16

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ layout sizes
__host__ __device__ inline int64_t qpage_head_bytes(int d, int bits) { return 4LL * d * bits + kMetaBytes; }
__host__ __device__ inline int64_t bf16_page_head_bytes(int d) { return 64LL * d; }
__host__ __device__ inline int lane_chunk_bytes(int d, int bits) { return d * bits / 32; }  // K part; V part same

// Byte address of page-head (page, kv) in the pool arena. Pages below off4 are INT2 pages,
// pages at or above it INT4 pages stacked after the INT2 region.
__device__ inline const uint8_t* page_head_addr(const uint8_t* pool, int64_t page, int kv, int hkv, int d,
                                                int64_t off4) {
  const int64_t p2 = qpage_head_bytes(d, 2) * hkv;
  if (page < off4) return pool + page * p2 + (int64_t)kv * qpage_head_bytes(d, 2);
  const int64_t p4 = qpage_head_bytes(d, 4) * hkv;
  return pool + off4 * p2 + (page - off4) * p4 + (int64_t)kv * qpage_head_bytes(d, 4);
}

// Pointer into global memory (address space 1): loads through it are global loads, also where
// the address was assembled from scalar registers.
template <typename T>
using GPtr = const __attribute__((address_space(1))) T*;

// ------------------------------------------------------------------ number formats
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// fp16 pattern -> fp32 on the host (exact for every pattern; NaN patterns map to NaN).
inline float host_f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  uint32_t u;
  if (e == 0x1Fu) {
    u = sign | 0x7F800000u | (m << 13);
  } else if (e != 0) {
    u = sign | ((e + 112u) << 23) | (m << 13);
  } else {
    float f = (float)m * 0x1p-24f;   // subnormal: m * 2^-24, exact
    return sign ? -f : f;
  }
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// ------------------------------------------------------------------ wavefront reductions
// Whole-wavefront reductions without LDS traffic: butterflies inside each 16-lane row on the DPP
// network (quad permutes [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors), after which
// every lane of a row holds the row's result; the four row results are read as scalars and
// combined. Every lane of the wavefront must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f<0xB1>(v));
  v = fminf(v, dpp_f<0x4E>(v));
  v = fminf(v, dpp_f<0x141>(v));
  v = fminf(v, dpp_f<0x140>(v));
  return fminf(fminf(lane_f(v, 0), lane_f(v, 16)), fminf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// DPP row shift right by N lanes inside each 16-lane row: lane l reads lane l-N (lanes whose
// source falls outside the row read 0).
template <int N>
__device__ __forceinline__ uint32_t dpp_row_shr(uint32_t v) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + N, 0xF, 0xF, false);
}
// DPP row shift left: lane l reads lane l+N of its row (0 outside the row).
template <int N>
__device__ __forceinline__ uint32_t dpp_row_shl(uint32_t v) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xF, 0xF, false);
}
// DPP move with a bank mask: lanes of the 4-lane banks set in BANKS receive src from the lane
// that CTRL selects; the other lanes keep old. Selecting by bank mask keeps the move
// unconditional: a data-dependent select around a DPP move may be turned into a branch, and a
// DPP move executed under a narrowed exec mask reads inactive source lanes as invalid.
template <int CTRL, int BANKS>
__device__ __forceinline__ uint32_t dpp_into(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, 0xF, BANKS, false);
}
template <int N, int BANKS>
__device__ __forceinline__ uint32_t dpp_row_shr_into(uint32_t old, uint32_t src) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return dpp_into<0x110 + N, BANKS>(old, src);
}
template <int N, int BANKS>
__device__ __forceinline__ uint32_t dpp_row_shl_into(uint32_t old, uint32_t src) {
  static_assert(N >= 1 && N <= 15, "row shift 1..15");
  return dpp_into<0x100 + N, BANKS>(old, src);
}
template <int N, int BANKS>
__device__ __forceinline__ float dpp_row_shr_into(float old, float src) {
  return __uint_as_float(dpp_row_shr_into<N, BANKS>(__float_as_uint(old), __float_as_uint(src)));
}
// DPP row rotate right by N lanes inside each 16-lane row.
template <int N>
__device__ __forceinline__ float dpp_row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF,
                                                               false));
}
template <int N>
__device__ __forceinline__ uint32_t dpp_row_ror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xF, 0xF, true);   // every lane has a source
}
// DPP row shift left by N lanes (lane c reads lane c + N of its row; the last N lanes read 0).
template <int N>
__device__ __forceinline__ float dpp_row_shl_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x100 + N, 0xF, 0xF,
                                                               true));
}
// Word 3 of a raw (untyped, unswizzled) buffer descriptor: loads at or past its size return zeros
// without touching memory.
constexpr int kRawBufferFlags = 0x00020000;
// Wave-uniform copy of a value (the compiler treats the result as scalar).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------------ exact group quantiser
// Quantiser decision in fp32, operation by operation with multiply-add contraction switched off
// (c*max - c*min must not become one fused operation): lo = c*min, hi = c*max,
// s = bf16(fp32(hi - lo)/L), z = bf16(lo), code = clamp(rint_even(fp32(clamp(x,lo,hi) - z)/s), 0, L).
struct QuantGrid {
  float lo, hi, s, z;
  float rs;                 // hardware reciprocal of s (estimate for quant_code)
  uint32_t s_bits, z_bits;
};

__device__ __forceinline__ QuantGrid make_grid(float mn, float mx, float clip, int levels) {
#pragma clang fp contract(off)
  QuantGrid g;
  g.lo = clip * mn;
  g.hi = clip * mx;
  const float s32 = __fdiv_rn(g.hi - g.lo, (float)levels);
  g.s_bits = f32_to_bf16_bits(s32);
  g.z_bits = f32_to_bf16_bits(g.lo);
  g.s = bf16_bits_to_f32(g.s_bits);
  g.z = bf16_bits_to_f32(g.z_bits);
  g.rs = __builtin_amdgcn_rcpf(g.s);
  return g;
}

// The quotient t = fl(d / s) only feeds rint, so it is first estimated as d * rcp(s): the hardware
// reciprocal is within 1 ulp, the estimate within 2^-17 of d / s for |t| < 32, and the correctly
// rounded quotient within 2^-19. Unless the estimate lies within 2^-14 of a rounding midpoint
// k + 1/2 (or is not below 32 in magnitude, or not a number), both round to the same integer.
// quant_code_fast returns the code of the estimate and sets `redo` in those cases, where
// quant_code_exact (the correctly rounded division) decides; quant_code chains the two. Every
// variant returns the code of the exact rule.
// (branch-free: the clamps are median-of-three, the tests combine with bitwise operators)
__device__ __forceinline__ uint32_t quant_code_fast(float x, const QuantGrid& g, int levels, bool& redo) {
#pragma clang fp contract(off)
  const float xc = __builtin_amdgcn_fmed3f(x, g.lo, g.hi);
  const float t = (xc - g.z) * g.rs;
  redo = (g.s != 0.0f) & (!(fabsf(t) < 32.0f) | (fabsf(__builtin_amdgcn_fractf(t) - 0.5f) <= 0x1p-14f));
  const float r = __builtin_amdgcn_fmed3f(rintf(t), 0.0f, (float)levels);
  return g.s == 0.0f ? 0u : (uint32_t)r;
}

__device__ __forceinline__ uint32_t quant_code_exact(float x, const QuantGrid& g, int levels) {
#pragma clang fp contract(off)
  if (g.s == 0.0f) return 0u;
  const float xc = fminf(fmaxf(x, g.lo), g.hi);
  const float t = __fdiv_rn(xc - g.z, g.s);
  return (uint32_t)fminf(fmaxf(rintf(t), 0.0f), (float)levels);
}

__device__ __forceinline__ uint32_t quant_code(float x, const QuantGrid& g, int levels) {
  bool redo;
  const uint32_t c = quant_code_fast(x, g, levels, redo);
  return redo ? quant_code_exact(x, g, levels) : c;
}

// ------------------------------------------------------------------ INT2 codebook
// Lloyd-Max codebook of the INT2 history (OSCAR overview page, the paragraph that sets OSCAR beside
// TurboQuant): four increasing fp16 levels l_0..l_3 replace the uniform levels 0..3 of the group
// coordinate u = (clip(x) - z) / s, so a code restores as z + s * l[code]. A code is the nearest
// level: [u > t_0] + [u >= t_1] + [u > t_2] with the midpoints t_j = (l_j + l_{j+1}) / 2 (exact in
// fp32), which sends a u on a threshold to the even code -- the levels 0, 1, 2, 3 give back the
// uniform round-half-to-even code. The table holds [kv-head][K, V][4] fp16 patterns.
struct Codebook {
  uint32_t lut_lo, lut_hi;      // fp16 patterns l_0 | l_1 << 16 and l_2 | l_3 << 16
  uint32_t plane_lo, plane_hi;  // byte planes: low bytes of l_0..l_3, high bytes of l_0..l_3
  float t0, t1, t2;             // decision thresholds
  bool on;                      // false: the uniform levels (this struct is then unused)
};

__device__ __forceinline__ Codebook load_codebook(const uint16_t* table, int kv, int sel) {
  Codebook c;
  c.on = table != nullptr;
  c.lut_lo = 0x3C000000u;   // uniform levels 0, 1, 2, 3
  c.lut_hi = 0x42004000u;
  if (c.on) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(table + ((size_t)kv * 2 + sel) * 4);
    c.lut_lo = p[0];
    c.lut_hi = p[1];
  }
  c.plane_lo = __builtin_amdgcn_perm(c.lut_hi, c.lut_lo, 0x06040200u);
  c.plane_hi = __builtin_amdgcn_perm(c.lut_hi, c.lut_lo, 0x07050301u);
  const float l0 = f16_bits_to_f32(c.lut_lo & 0xFFFFu), l1 = f16_bits_to_f32(c.lut_lo >> 16);
  const float l2 = f16_bits_to_f32(c.lut_hi & 0xFFFFu), l3 = f16_bits_to_f32(c.lut_hi >> 16);
  // uniform values: kept in scalar registers
  c.t0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, (l0 + l1) * 0.5f)));
  c.t1 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, (l1 + l2) * 0.5f)));
  c.t2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, (l2 + l3) * 0.5f)));
  return c;
}

// Level of a code (fp32 value of its fp16 pattern).
__device__ __forceinline__ float codebook_level(const Codebook& c, uint32_t code) {
  const uint32_t w = code < 2 ? c.lut_lo : c.lut_hi;
  return f16_bits_to_f32((code & 1u) ? (w >> 16) : (w & 0xFFFFu));
}

// Levels of packed codes in two byte permutes. codebook_spread copies byte 0 of each half-word of
// w (bytes 1 and 3 when odd) into both bytes of that half-word; codebook_levels2 then takes the
// codes at bits 2m..2m+1 of those bytes and returns their fp16 levels, the low half-word's code
// in the low half: the selector bytes are (c, 4 + c) per half-word, which pick the low and high
// byte of l[c] from the two byte planes.
__device__ __forceinline__ uint32_t codebook_spread(uint32_t w, bool odd) {
  return __builtin_amdgcn_perm(w, w, odd ? 0x03030101u : 0x02020000u);
}
__device__ __forceinline__ uint32_t codebook_levels2(const Codebook& c, uint32_t z, int m) {
  // the selector as one v_and_or_b32 (the compiler would spend an AND and an OR with literals)
  uint32_t sel;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(sel) : "v"(z >> (2 * m)), "s"(0x03030303u), "v"(0x04000400u));
  return __builtin_amdgcn_perm(c.plane_hi, c.plane_lo, sel);
}

// Codebook decisions with the estimate / exact split of quant_code: the estimate decides unless it
// lies within 2^-14 of a threshold (or is not below 32 in magnitude, or not a number).
__device__ __forceinline__ uint32_t cb_code_of(float t, const Codebook& c) {
  return (uint32_t)(t > c.t0) + (uint32_t)(t >= c.t1) + (uint32_t)(t > c.t2);
}

__device__ __forceinline__ uint32_t cb_code_fast(float x, const QuantGrid& g, const Codebook& c, bool& redo) {
#pragma clang fp contract(off)
  const float xc = __builtin_amdgcn_fmed3f(x, g.lo, g.hi);
  const float t = (xc - g.z) * g.rs;
  const float near = fminf(fminf(fabsf(t - c.t0), fabsf(t - c.t1)), fabsf(t - c.t2));
  redo = (g.s != 0.0f) & (!(fabsf(t) < 32.0f) | !(near > 0x1p-14f));
  return g.s == 0.0f ? 0u : cb_code_of(t, c);
}

__device__ __forceinline__ uint32_t cb_code_exact(float x, const QuantGrid& g, const Codebook& c) {
#pragma clang fp contract(off)
  if (g.s == 0.0f) return 0u;
  const float xc = fminf(fmaxf(x, g.lo), g.hi);
  return cb_code_of(__fdiv_rn(xc - g.z, g.s), c);
}

__device__ __forceinline__ uint32_t cb_code(float x, const QuantGrid& g, const Codebook& c) {
  bool redo;
  const uint32_t k = cb_code_fast(x, g, c, redo);
  return redo ? cb_code_exact(x, g, c) : k;
}

// ------------------------------------------------------------------ history code placement
// Byte offset of lane l's key / value part in a history page-head (cb = bytes of one part,
// d * bits / 32). INT2: a lane's two parts sit together (a 2*cb-byte lane chunk). INT4: the 64 key
// parts, then the 64 value parts, so that at d <= 128 one load instruction of a wavefront reads
// consecutive whole 128-byte lines of either part.
__host__ __device__ inline size_t key_part_offset(int bits, int cb, int lane) {
  return bits == 2 ? (size_t)lane * 2 * cb : (size_t)lane * cb;
}
__host__ __device__ inline size_t value_part_offset(int bits, int cb, int lane) {
  return bits == 2 ? (size_t)lane * 2 * cb + cb : (size_t)(64 + lane) * cb;
}

// BF16 page-head element offsets (in bf16 units).
__host__ __device__ inline int bf16_key_index(int d, int t, int ch) {
  const int kk = ch / 32, g = (ch % 32) / 8, i = ch % 8;
  return ((g * 16 + t) * (d / 32) + kk) * 8 + i;
}
__host__ __device__ inline int bf16_value_index(int d, int t, int ch) {
  const int nb = ch / 16, c = ch % 16, g = t / 4, r = t % 4;
  return 16 * d + ((g * 16 + c) * (d / 16) + nb) * 4 + r;
}

}  // namespace oscar
