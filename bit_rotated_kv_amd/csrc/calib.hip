// Calibration statistics of the rotations on the GPU ("Together AI open-sources OSCAR", section on
// what makes OSCAR different): the query covariance C_Q = (1/N) sum_n q_n^T q_n, summed over the
// query heads of a kv-head, and the score-weighted value covariance C_S = (1/N) (S V)^T (S V) with
// S = softmax(scale q K^T) over a calibration context. Their eigenvectors (host, fp64) give
// R = U . H . P_br.
//
// Both are Gram matrices of rows (queries; rows of S V), formed on the matrix cores
// (v_mfma_f32_32x32x16_bf16) in chunks of whole 256-row sub-chunks whose partial sums are added in
// chunk order.
// bf16 rows are exact operands; fp32 rows (S V) are split into bf16 high and low parts and the
// three leading products (hi.hi, hi.lo, lo.hi) are accumulated, for about 16 significant bits per
// element. S V comes from a flash-attention pass: for a tile of 32 context keys, S^T = K Q^T on the
// matrix cores puts one query in each lane (its softmax state stays in the lane), and the
// probabilities enter the S V product as bf16 high + low parts.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "oscar.h"

namespace oscar {
namespace {

typedef float float16v_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float16v_t mfma32(const bf16x8_t& a, const bf16x8_t& b, float16v_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) { return (uint16_t)f32_to_bf16_bits(x); }

constexpr int kGramRows = 256;   // rows per staged sub-chunk of a Gram workgroup
constexpr int kGramTargetWorkgroups = 512;   // about two workgroups per compute unit

// Sub-chunks of 256 rows per Gram workgroup: as few as keep the launch near two workgroups per CU
// (fewer partial Gram matrices to write and add).
inline int gram_subchunks(int hkv, int64_t rows) {
  const int64_t subs = ((int64_t)hkv * ((rows + kGramRows - 1) / kGramRows) + kGramTargetWorkgroups - 1) /
                       kGramTargetWorkgroups;
  return (int)(subs < 1 ? 1 : (subs > 64 ? 64 : subs));
}
inline int64_t gram_chunks(int hkv, int64_t rows) {
  const int64_t per = (int64_t)kGramRows * gram_subchunks(hkv, rows);
  return (rows + per - 1) / per;
}

// ------------------------------------------------------------------ Gram of rows
// Workgroup (chunk, kv): rows [chunk * subs * 256, ...) of the kv-head's rows x[kv] ([R][D], bf16
// or fp32), in sub-chunks of 256 rows: each is transposed into LDS (channel-major) and multiplied
// by itself, the products accumulating in registers in row order. Wavefront w < D/32 owns the
// output rows 32w .. 32w+31 (all D/32 column tiles). Writes the chunk's partial Gram (fp32 [D][D]).
template <int D, bool F32>
__global__ __launch_bounds__(256) void gram_kernel(const void* x, int64_t rows, int subs, float* partial) {
  constexpr int NP = F32 ? 2 : 1;       // bf16 parts per element
  constexpr int RP = kGramRows + 8;     // padded row pitch of the transposed tile (bf16)
  constexpr int CT = D / 32;            // 32-wide tiles per dimension
  constexpr int TPC = 256 / D;          // staging threads per channel
  constexpr int NGI = kGramRows / 8 / TPC;   // 8-row groups per staging thread
  constexpr int GB = NGI < 4 ? NGI : 4;      // groups whose loads are issued together
  __shared__ __attribute__((aligned(16))) uint16_t xt[NP][D][RP];
  const int chunk = blockIdx.x, kv = blockIdx.y;
  const int nchunks = gridDim.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int c = tid % D, ph = tid / D;
  float16v_t acc[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) acc[t] = float16v_t{};
  for (int sc = 0; sc < subs; ++sc) {
    const int64_t r0 = ((int64_t)chunk * subs + sc) * kGramRows;
    if (r0 >= rows) break;
    const int n = (int)min<int64_t>(kGramRows, rows - r0);
    const size_t base = ((size_t)kv * rows + r0) * D + c;   // element index of (row r0, channel c)
    if (sc > 0) __syncthreads();   // the previous sub-chunk's products have read the tile
    if constexpr (!F32) {
      // bf16 rows: thread (channel quad cq, phase ph) loads 8 bytes (4 channels) of each row of its
      // 8-row groups, all loads in flight at once (a wavefront instruction reads whole row
      // segments), then byte-permutes them into one 16-byte channel-major piece per channel
      constexpr int NQ = D / 4, PH = 256 / NQ, GPT = kGramRows / 8 / PH;
      const int cq = tid % NQ, rph = tid / NQ;
      const uint16_t* xb = static_cast<const uint16_t*>(x) + ((size_t)kv * rows + r0) * D + 4 * cq;
      u32x2_t w[GPT][8];
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * (rph + PH * gi) + e;
          w[gi][e] = r < n ? *reinterpret_cast<const u32x2_t*>(xb + (uint32_t)(r * D)) : u32x2_t{0u, 0u};
        }
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int g = rph + PH * gi;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          const uint32_t sel = (ch & 1) ? 0x07060302u : 0x05040100u;   // high or low half-words
          u32x4_t piece;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            piece[k] = __builtin_amdgcn_perm(w[gi][2 * k + 1][ch / 2], w[gi][2 * k][ch / 2], sel);
          *reinterpret_cast<u32x4_t*>(&xt[0][4 * cq + ch][8 * g]) = piece;
        }
      }
    } else
    // fp32 rows: thread (channel c, phase ph) gathers 8 consecutive rows of its channel per group
    // (each load instruction reads consecutive channels of one row) and stores the bf16 high and low
    // parts as 16-byte pieces of the channel-major tiles; the loads of GB groups go out before any
    // is used
    for (int gb = 0; gb < NGI; gb += GB) {
      float v[GB][8];
#pragma unroll
      for (int gi = 0; gi < GB; ++gi)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * (ph + TPC * (gb + gi)) + e;
          float x32 = 0.0f;
          if (r < n) {
            if constexpr (F32)
              x32 = static_cast<const float*>(x)[base + (uint32_t)(r * D)];
            else
              x32 = bf16_bits_to_f32(static_cast<const uint16_t*>(x)[base + (uint32_t)(r * D)]);
          }
          v[gi][e] = x32;
        }
#pragma unroll
      for (int gi = 0; gi < GB; ++gi) {
        const int g = ph + TPC * (gb + gi);
        u32x4_t hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h0 = bf16_rne(v[gi][2 * e]), h1 = bf16_rne(v[gi][2 * e + 1]);
          hi[e] = h0 | (h1 << 16);
          if constexpr (F32)
            lo[e] = (uint32_t)bf16_rne(v[gi][2 * e] - bf16_bits_to_f32(h0)) |
                    ((uint32_t)bf16_rne(v[gi][2 * e + 1] - bf16_bits_to_f32(h1)) << 16);
        }
        *reinterpret_cast<u32x4_t*>(&xt[0][c][8 * g]) = hi;
        if constexpr (F32) *reinterpret_cast<u32x4_t*>(&xt[NP - 1][c][8 * g]) = lo;
      }
    }
    __syncthreads();
    if (wave < CT) {
      const int m = 32 * wave + lane % 32;
      for (int kk = 0; kk < kGramRows / 16; ++kk) {
        const int k0 = 16 * kk + 8 * (lane / 32);
        bf16x8_t a[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) a[p] = *reinterpret_cast<const bf16x8_t*>(&xt[p][m][k0]);
#pragma unroll
        for (int t = 0; t < CT; ++t) {
          const int nn = 32 * t + lane % 32;
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&xt[0][nn][k0]);
          if constexpr (F32) {
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&xt[1][nn][k0]);
            acc[t] = mfma32(a[1], bh, acc[t]);   // lo . hi
            acc[t] = mfma32(a[0], bl, acc[t]);   // hi . lo
          }
          acc[t] = mfma32(a[0], bh, acc[t]);     // hi . hi
        }
      }
    }
  }
  if (wave < CT) {
    float* out = partial + ((size_t)kv * nchunks + chunk) * D * D;
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        out[(size_t)(32 * wave + 8 * (j / 4) + 4 * (lane / 32) + j % 4) * D + 32 * t + lane % 32] = acc[t][j];
  }
}

// cov[kv] = (sum over chunks of partial[kv][chunk], in chunk order) * inv_n
template <int D>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* partial, int nchunks, float inv_n, float* cov) {
  const int kv = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const float* p = partial + (size_t)kv * nchunks * D * D + e;
  float s = 0.0f;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) s += p[(size_t)c * D * D];
  cov[(size_t)kv * D * D + e] = s * inv_n;
}

template <int D, bool F32>
hipError_t launch_gram(const void* x, int hkv, int64_t rows, float inv_n, float* partial, float* cov,
                       hipStream_t stream) {
  const int subs = gram_subchunks(hkv, rows);
  const int nchunks = (int)gram_chunks(hkv, rows);
  hipLaunchKernelGGL((gram_kernel<D, F32>), dim3(nchunks, hkv), dim3(256), 0, stream, x, rows, subs, partial);
  hipLaunchKernelGGL((gram_reduce_kernel<D>), dim3((D * D + 255) / 256, hkv), dim3(256), 0, stream, partial, nchunks,
                     inv_n, cov);
  return hipGetLastError();
}

// ------------------------------------------------------------------ S V rows (flash attention)
// Workgroup (query block of 128, head h, kv-head): wavefront w takes queries 128 bx + 32 w .. +31
// of head h. Per tile of 32 context keys (K row-major and V channel-major in LDS):
//   S^T = K Q^T (A = K rows, B = the wavefront's queries, held in registers): lane l holds query
//     l % 32 and keys 8(j/4) + 4(l/32) + j%4 (j < 16), so the online softmax of a query is the
//     lane's 16 values and those of lane l ^ 32;
//   O^T += V^T P^T with P as exact bf16 high + low parts: the B operand of k-step kk needs keys
//     16kk + 8(l/32) .. +7, four of which come from lane l ^ 32.
// Writes S V = O / l (fp32) as rows h * Nq + query of the kv-head.
template <int D>
__global__ __launch_bounds__(256) void calib_sv_kernel(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                                       int nq, int nctx, float scale_log2e, float* sv) {
  constexpr int KS = D / 16;     // k-steps over channels
  constexpr int CT = D / 32;     // channel tiles of O^T
  constexpr int KP = D + 8;      // padded K row (bf16)
  constexpr int VP = 32 + 8;     // padded V^T row (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t ks[32][KP];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D][VP];
  const int h = blockIdx.y, kv = blockIdx.z, gq = gridDim.y;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, half = lane / 32;
  const int qi = 128 * blockIdx.x + 32 * wave + lane % 32;   // this lane's query
  const uint16_t* qrow = q + (((size_t)kv * gq + h) * nq + qi) * D;
  const uint16_t* kb = k + (size_t)kv * nctx * D;
  const uint16_t* vb = v + (size_t)kv * nctx * D;
  bf16x8_t bq[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4_t w = {0, 0, 0, 0};
    if (qi < nq) w = *reinterpret_cast<const u32x4_t*>(qrow + 16 * kk + 8 * half);
    bq[kk] = __builtin_bit_cast(bf16x8_t, w);
  }
  float16v_t o[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) o[t] = float16v_t{};
  float m_run = -__builtin_huge_valf(), l_run = 0.0f;
  // A tile's loads go out two tiles ahead into registers (K: 16-byte pieces; V: thread (channel, key
  // group) gathers 8 keys of one channel), and are written to LDS when the tile's turn comes.
  constexpr int KPT = 32 * D / 8 / 256, VIT = 4 * D / 256;
  struct TileRegs {
    u32x4_t kw[KPT];
    u32x4_t vw[VIT];
  };
  auto fetch = [&](int k0, TileRegs& R) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + 256 * i, r = idx / (D / 8), c8 = idx % (D / 8);
      R.kw[i] = u32x4_t{0, 0, 0, 0};
      if (k0 + r < nctx) R.kw[i] = *reinterpret_cast<const u32x4_t*>(kb + (size_t)(k0 + r) * D + 8 * c8);
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int idx = tid + 256 * i, c = idx % D, g = idx / D;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r0 = k0 + 8 * g + 2 * e;
        const uint32_t lo = r0 < nctx ? vb[(size_t)r0 * D + c] : 0u;
        const uint32_t hi = r0 + 1 < nctx ? vb[(size_t)(r0 + 1) * D + c] : 0u;
        R.vw[i][e] = lo | (hi << 16);
      }
    }
  };
  auto stage = [&](const TileRegs& R) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + 256 * i, r = idx / (D / 8), c8 = idx % (D / 8);
      *reinterpret_cast<u32x4_t*>(&ks[r][8 * c8]) = R.kw[i];
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int idx = tid + 256 * i, c = idx % D, g = idx / D;
      *reinterpret_cast<u32x4_t*>(&vt[c][8 * g]) = R.vw[i];
    }
  };
  TileRegs ra, rb;
  fetch(0, ra);
  fetch(32, rb);
  for (int k0 = 0; k0 < nctx; k0 += 32) {
    // tiles alternate between the two register sets (k0 / 32 even: ra); the set just written to
    // LDS takes the loads of the tile two ahead
    const bool even = ((k0 / 32) & 1) == 0;
    if (even) {
      stage(ra);
      fetch(k0 + 64, ra);
    } else {
      stage(rb);
      fetch(k0 + 64, rb);
    }
    __syncthreads();
    float16v_t s = {};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      s = mfma32(*reinterpret_cast<const bf16x8_t*>(&ks[lane % 32][16 * kk + 8 * half]), bq[kk], s);
    float p[16], mx = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int key = k0 + 8 * (j / 4) + 4 * half + j % 4;
      p[j] = key < nctx ? s[j] * scale_log2e : -__builtin_huge_valf();
      mx = fmaxf(mx, p[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 while m_run is -inf
    float ps = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      p[j] = __builtin_amdgcn_exp2f(p[j] - m_new);
      ps += p[j];
    }
    l_run = l_run * alpha + (ps + __shfl_xor(ps, 32, kWave));
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < CT; ++t) o[t] *= alpha;
    float pr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) pr[j] = __shfl_xor(p[j], 32, kWave);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // keys 16kk + 8 half .. +7 of this lane's query: lanes l < 32 own the first four and take the
      // next four from lane l + 32; lanes l >= 32 take the first four from lane l - 32
      float e8[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        e8[e] = half == 0 ? p[8 * kk + e] : pr[8 * kk + 4 + e];
        e8[4 + e] = half == 0 ? pr[8 * kk + e] : p[8 * kk + 4 + e];
      }
      bf16x8_t ph, pl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t hb = bf16_rne(e8[e]);
        ph[e] = __builtin_bit_cast(__bf16, hb);
        pl[e] = __builtin_bit_cast(__bf16, bf16_rne(e8[e] - bf16_bits_to_f32(hb)));
      }
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&vt[32 * t + lane % 32][16 * kk + 8 * half]);
        o[t] = mfma32(av, pl, o[t]);
        o[t] = mfma32(av, ph, o[t]);
      }
    }
    __syncthreads();
  }
  if (qi < nq) {
    const float inv_l = 1.0f / l_run;
    float* out = sv + (((size_t)kv * gq + h) * nq + qi) * D;
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int j = 0; j < 16; ++j) out[32 * t + 8 * (j / 4) + 4 * half + j % 4] = o[t][j] * inv_l;
  }
}

size_t gram_partial_bytes(int hkv, int64_t rows, int d) {
  return (size_t)hkv * gram_chunks(hkv, rows) * d * d * 4;
}

bool supported(int d) { return d == 64 || d == 128; }

}  // namespace
}  // namespace oscar

using namespace oscar;

extern "C" {

size_t oscar_calib_workspace_bytes(int32_t num_kv_heads, int32_t gq, int32_t n_rows, int32_t head_dim) {
  if (num_kv_heads <= 0 || gq <= 0 || n_rows <= 0 || !supported(head_dim)) return 0;
  const int64_t rows = (int64_t)gq * n_rows;
  // Gram partials, plus the fp32 rows of S V for the value covariance
  return 256 + gram_partial_bytes(num_kv_heads, rows, head_dim) + (size_t)num_kv_heads * rows * head_dim * 4;
}

oscar_status_t oscar_calib_query_cov(int32_t num_kv_heads, int32_t gq, int32_t n_tokens, int32_t head_dim,
                                     const void* q, void* workspace, size_t workspace_bytes, float* cov,
                                     hipStream_t stream) {
  if (num_kv_heads <= 0 || gq <= 0 || n_tokens <= 0) return OSCAR_ERR_INVALID_ARG;
  if (!supported(head_dim)) return OSCAR_ERR_UNSUPPORTED;
  if (!q || !cov || !workspace) return OSCAR_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)gq * n_tokens;
  if ((rows + kGramRows - 1) / kGramRows > 65535) return OSCAR_ERR_UNSUPPORTED;
  if (workspace_bytes < 256 + gram_partial_bytes(num_kv_heads, rows, head_dim)) return OSCAR_ERR_WORKSPACE;
  float* partial = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + 256);
  const float inv_n = 1.0f / (float)n_tokens;
  const hipError_t e = head_dim == 128 ? launch_gram<128, false>(q, num_kv_heads, rows, inv_n, partial, cov, stream)
                                       : launch_gram<64, false>(q, num_kv_heads, rows, inv_n, partial, cov, stream);
  return e == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

oscar_status_t oscar_calib_value_cov(int32_t num_kv_heads, int32_t gq, int32_t n_queries, int32_t n_ctx,
                                     int32_t head_dim, const void* q, const void* k, const void* v,
                                     float softmax_scale, void* workspace, size_t workspace_bytes, float* cov,
                                     hipStream_t stream) {
  if (num_kv_heads <= 0 || gq <= 0 || n_queries <= 0 || n_ctx <= 0 || !(softmax_scale >= 0.0f))
    return OSCAR_ERR_INVALID_ARG;
  if (!supported(head_dim)) return OSCAR_ERR_UNSUPPORTED;
  if (!q || !k || !v || !cov || !workspace) return OSCAR_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)gq * n_queries;
  if ((rows + kGramRows - 1) / kGramRows > 65535 || gq > 65535 || num_kv_heads > 65535) return OSCAR_ERR_UNSUPPORTED;
  if (workspace_bytes < oscar_calib_workspace_bytes(num_kv_heads, gq, n_queries, head_dim)) return OSCAR_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* partial = reinterpret_cast<float*>(ws + 256);
  float* sv = reinterpret_cast<float*>(ws + 256 + gram_partial_bytes(num_kv_heads, rows, head_dim));
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  const float sl2e = scale * 1.4426950408889634f;
  const dim3 grid((n_queries + 127) / 128, gq, num_kv_heads);
  const uint16_t* qb = static_cast<const uint16_t*>(q);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  if (head_dim == 128)
    hipLaunchKernelGGL(calib_sv_kernel<128>, grid, dim3(256), 0, stream, qb, kb, vb, n_queries, n_ctx, sl2e, sv);
  else
    hipLaunchKernelGGL(calib_sv_kernel<64>, grid, dim3(256), 0, stream, qb, kb, vb, n_queries, n_ctx, sl2e, sv);
  if (hipGetLastError() != hipSuccess) return OSCAR_ERR_LAUNCH;
  const float inv_n = 1.0f / (float)n_queries;
  const hipError_t e = head_dim == 128 ? launch_gram<128, true>(sv, num_kv_heads, rows, inv_n, partial, cov, stream)
                                       : launch_gram<64, true>(sv, num_kv_heads, rows, inv_n, partial, cov, stream);
  return e == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

}  // extern "C"
