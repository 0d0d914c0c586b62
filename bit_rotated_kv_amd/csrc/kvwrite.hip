// Cache writers: prefill (sink/recent windows and rotated+quantised history pages), the per-step
// demote of the oldest recent token (OSCAR overview page, method paragraph; study note, SGLang
// case), and the fill of the full-BF16 baseline cache.
#include <algorithm>
#include <type_traits>

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
// One workgroup per (window page, kv-head, request); the first page's workgroup of kv-head 0 also
// counts the request's INT4 history tokens. Every element of the thread is loaded before any is
// stored: the page could alias the inputs as far as the compiler knows, so a loop of load-store
// pairs would wait out one memory round trip per element.
__global__ __launch_bounds__(256) void prefill_window_kernel(CacheWriteArgs a) {
  constexpr int kItems = kPage * 128 / 256;   // elements per thread at the largest head_dim
  const Dims& dm = a.dm;
  const int j = blockIdx.x, kv = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = dm.d;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int64_t pb = bf16_page_head_bytes(d);
  uint16_t* pg = reinterpret_cast<uint16_t*>(a.window + ((size_t)(b * dm.hkv + kv) * dm.wpages + j) * pb);
  const size_t src = ((size_t)b * dm.hkv + kv) * dm.max_seq_len;
  uint16_t kx[kItems], vx[kItems];
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int idx = tid + 256 * i, t = idx / d, ch = idx % d;
    const int p = idx < kPage * d ? window_position(j, t, T, dm.sink, dm.recent) : -1;
    kx[i] = p >= 0 ? a.k[(src + p) * d + ch] : (uint16_t)0;
    vx[i] = p >= 0 ? a.v[(src + p) * d + ch] : (uint16_t)0;
  }
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int idx = tid + 256 * i, t = idx / d, ch = idx % d;
    if (idx < kPage * d) {
      pg[bf16_key_index(d, t, ch)] = kx[i];
      pg[bf16_value_index(d, t, ch)] = vx[i];
    }
  }
  if (j == 0 && kv == 0 && a.n_int4_out) {
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

// The window's K (sel 0) or V (sel 1) halves of pages j = x, x + nx, ... of one (request, kv-head),
// copied by NT threads (thread t of them): the INT2-only prefill spreads the window over the
// workgroups of its own launch. Every element a thread copies is loaded before any is stored.
template <int NT>
__device__ void window_slice(const CacheWriteArgs& a, int b, int kv, int sel, int T, int x, int nx, int t) {
  constexpr int kItems = (kPage * 128 + NT - 1) / NT;   // elements per thread and page, at most
  const Dims& dm = a.dm;
  const int d = dm.d;
  const int64_t pb = bf16_page_head_bytes(d);
  const uint16_t* src = (sel ? a.v : a.k) + ((size_t)b * dm.hkv + kv) * dm.max_seq_len * d;
  for (int j = x; j < dm.wpages; j += nx) {
    uint16_t* pg = reinterpret_cast<uint16_t*>(a.window + ((size_t)(b * dm.hkv + kv) * dm.wpages + j) * pb);
    uint16_t e[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int idx = t + NT * i, tk = idx / d, ch = idx % d;
      const int p = idx < kPage * d ? window_position(j, tk, T, dm.sink, dm.recent) : -1;
      e[i] = p >= 0 ? src[(size_t)p * d + ch] : (uint16_t)0;
    }
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int idx = t + NT * i, tk = idx / d, ch = idx % d;
      if (idx < kPage * d) pg[sel ? bf16_value_index(d, tk, ch) : bf16_key_index(d, tk, ch)] = e[i];
    }
  }
}

// ------------------------------------------------------------------ prefill: history pages
// One workgroup per (run of kPrefillChunks 64-position chunks of the history, kv-head, request x
// {K, V}). Wavefront w holds the 32-column slice w of R (three bf16 parts) in registers for the
// whole run. Per chunk: the rows are rotated on the matrix cores (rotate_tile, two 32-row tiles),
// each row is clipped, quantised and packed with the demote's grid and code functions (so every
// token gets the codes the demote would give it), and the next chunk's rows are already loading.
// In an INT2-only cache a chunk starts on a page boundary and owns whole pages: its key and value
// words are assembled whole and stored plainly. In a mixed cache INT2 and INT4 tokens take
// consecutive slots of their own tables, so a chunk shares its edge pages with its neighbours and
// value bits are merged per slot.
constexpr int kPrefillChunk = 64;
constexpr int kPrefillChunks = 8;

// CBK: INT2 codes follow the codebook table of the arguments (a separate instantiation keeps the
// uniform quantiser's code unchanged).
template <int D, bool CBK>
__global__ __launch_bounds__(256, 2) void prefill_hist_kernel(CacheWriteArgs a) {
  constexpr int CH = kPrefillChunk;
  constexpr int XS = D + 8;     // bf16 row pitch (16-byte pad)
  constexpr int RS = D + 8;     // fp32 row pitch: the two lane halves of an accumulator store
                                // (rows 4 apart) fall on disjoint banks
  constexpr int CSP = D + 4;    // code row pitch: rows two apart no longer share banks
  constexpr int SL = RotSlice<D>::SLICES;
  constexpr int XW = CH * D / 8 / 256;   // 16-byte row pieces per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[CH][XS];
  __shared__ float xr[CH][RS];
  __shared__ __attribute__((aligned(16))) uint8_t cs[CH][CSP];
  __shared__ uint32_t szs[CH];
  __shared__ int slot_s[CH];
  __shared__ int bits_s[CH];
  __shared__ int red[256];
  // INT2-only caches: page ids of the run's pages, resolved once (-1: outside the table or not a
  // valid INT2 page), so the stores of a chunk wait on no table load
  constexpr int RUN_PAGES = kPrefillChunks * CH / kPage;
  __shared__ int64_t page_s[RUN_PAGES];
  const Dims& dm = a.dm;
  const int kv = blockIdx.y, b = blockIdx.z / 2, sel = blockIdx.z % 2;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int hist = T - dm.sink - dm.recent;
  const int chunk0 = kPrefillChunks * blockIdx.x;
  if (CH * chunk0 >= hist) return;
  const int nchunks = min(kPrefillChunks, (hist - CH * chunk0 + CH - 1) / CH);
  const uint8_t* bitsrow = (a.bits && dm.mixed) ? a.bits + (size_t)b * dm.max_seq_len : nullptr;
  const uint16_t* src = (sel ? a.v : a.k) + ((size_t)b * dm.hkv + kv) * dm.max_seq_len * D;
  RotSlice<D> rs;
  if (wave < SL) rs.load((sel ? a.rot_v : a.rot_k) + (size_t)kv * D * D, wave, lane);
  const Codebook cb = load_codebook(CBK ? a.codebook : nullptr, kv, sel);
  // rows of a chunk: thread pieces tid + 256 e (row = piece / (D/8), 8 channels each)
  auto load_rows = [&](int chunk, u32x4_t (&w)[XW]) {
    const int p0 = dm.sink + CH * chunk, n = min(CH, hist - CH * chunk);
#pragma unroll
    for (int e = 0; e < XW; ++e) {
      const int idx = tid + 256 * e, row = idx / (D / 8), c8 = idx % (D / 8);
      w[e] = u32x4_t{0, 0, 0, 0};
      if (row < n) w[e] = *reinterpret_cast<const u32x4_t*>(src + (size_t)(p0 + row) * D + 8 * c8);
    }
  };
  u32x4_t xw[XW];
  load_rows(chunk0, xw);
  if (!dm.mixed && tid < RUN_PAGES) {
    const int pi = CH * chunk0 / kPage + tid;
    const int64_t page = pi < dm.pt_stride ? (int64_t)a.pt2[(size_t)b * dm.pt_stride + pi] : -1;
    page_s[tid] = page_ok(page, 2, dm) ? page : -1;
  }
  // INT4 tokens before the run (mixed caches): slots are ranks among tokens of the same width
  int c4 = 0;
  if (bitsrow) {
    int cnt = 0;
    for (int p = dm.sink + tid; p < dm.sink + CH * chunk0; p += 256) cnt += bitsrow[p] == 4;
    red[tid] = cnt;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) red[tid] += red[tid + o];
      __syncthreads();
    }
    c4 = red[0];
    __syncthreads();
  }
  for (int ci = 0; ci < nchunks; ++ci) {
    const int chunk = chunk0 + ci;
    const int n = min(CH, hist - CH * chunk);
    const int p0 = dm.sink + CH * chunk;
#pragma unroll
    for (int e = 0; e < XW; ++e) {
      const int idx = tid + 256 * e;
      *reinterpret_cast<u32x4_t*>(&xs[idx / (D / 8)][8 * (idx % (D / 8))]) = xw[e];
    }
    if (bitsrow) {
      // mixed widths: slots are ranks among the tokens of the same width (one thread, in order)
      if (tid == 0) {
        for (int i = 0; i < n; ++i) {
          const int p = p0 + i;
          const int bw = bitsrow[p] == 4 ? 4 : 2;
          bits_s[i] = bw;
          slot_s[i] = bw == 4 ? c4 : (p - dm.sink) - c4;
          c4 += bw == 4;
        }
      }
    } else if (tid < n) {
      bits_s[tid] = 2;
      slot_s[tid] = p0 + tid - dm.sink;
    }
    __syncthreads();
    if (ci + 1 < nchunks) load_rows(chunk + 1, xw);   // in flight during this chunk
    if (wave < SL) {
#pragma unroll
      for (int tile = 0; tile < CH / 32; ++tile) {
        const float16v_t acc = rotate_tile<D>(rs, &xs[32 * tile][0], XS, n - 32 * tile, lane);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          xr[32 * tile + 8 * (j / 4) + 4 * (lane / 32) + j % 4][32 * wave + lane % 32] = acc[j];
      }
    }
    __syncthreads();
    // row i = tid / 4: four threads, D/4 channels each (every lane takes part in the reductions)
    {
      constexpr int QC = D / 4;
      const int i = tid / 4, q = tid % 4;
      const bool live = i < n;
      const int bw = live ? bits_s[i] : 2;
      float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
      if (live)
        for (int c = 0; c < QC; ++c) {
          mn = fminf(mn, xr[i][q * QC + c]);
          mx = fmaxf(mx, xr[i][q * QC + c]);
        }
#pragma unroll
      for (int o = 1; o < 4; o <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      }
      if (live) {
        const float clip = bw == 4 ? (sel ? a.clip_v4 : a.clip_k4) : (sel ? a.clip_v : a.clip_k);
        const int levels = (1 << bw) - 1;
        const QuantGrid g = make_grid(mn, mx, clip, levels);
        uint32_t redo = 0;   // channels whose code the exact division decides (rare)
        if (CBK && bw == 2) {
#pragma unroll
          for (int c4 = 0; c4 < QC / 4; ++c4) {
            const float4 x4 = *reinterpret_cast<const float4*>(&xr[i][q * QC + 4 * c4]);
            const float xe[4] = {x4.x, x4.y, x4.z, x4.w};
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bool r;
              packed |= cb_code_fast(xe[e], g, cb, r) << (8 * e);
              redo |= (uint32_t)r << (4 * c4 + e);
            }
            *reinterpret_cast<uint32_t*>(&cs[i][q * QC + 4 * c4]) = packed;
          }
          while (redo) {
            const int c = __builtin_ctz(redo);
            redo &= redo - 1;
            cs[i][q * QC + c] = (uint8_t)cb_code_exact(xr[i][q * QC + c], g, cb);
          }
        } else {
#pragma unroll
          for (int c4 = 0; c4 < QC / 4; ++c4) {
            const float4 x4 = *reinterpret_cast<const float4*>(&xr[i][q * QC + 4 * c4]);
            const float xe[4] = {x4.x, x4.y, x4.z, x4.w};
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bool r;
              packed |= quant_code_fast(xe[e], g, levels, r) << (8 * e);
              redo |= (uint32_t)r << (4 * c4 + e);
            }
            *reinterpret_cast<uint32_t*>(&cs[i][q * QC + 4 * c4]) = packed;
          }
          while (redo) {
            const int c = __builtin_ctz(redo);
            redo &= redo - 1;
            cs[i][q * QC + c] = (uint8_t)quant_code_exact(xr[i][q * QC + c], g, levels);
          }
        }
        if (q == 0) szs[i] = g.s_bits | (g.z_bits << 16);
      }
    }
    __syncthreads();
    if (!dm.mixed) {
      // INT2, whole pages: slot = position - sink, so token i sits in page (CH*chunk + i)/16, slot i%16
      constexpr int CB = D * 2 / 32;   // bytes of one lane-chunk part (key or value)
      constexpr int NWL = CB / 4;      // words of it
      const int64_t* pgs = page_s + CH * ci / kPage;   // the chunk's pages
      // (scale, zero) of each token
      for (int i = tid; i < n; i += 256) {
        const int64_t page = pgs[i / kPage];
        if (page >= 0)
          reinterpret_cast<uint32_t*>(page_head_mut(a.pool, page, kv, dm) + 4 * D * 2)[2 * (i % kPage) + sel] = szs[i];
      }
      if (sel == 0) {
        // key words: (token, g, a), each owned by one slot
        for (int idx = tid; idx < n * 4 * NWL; idx += 256) {
          const int i = idx / (4 * NWL), g = (idx / NWL) % 4, aw = idx % NWL;
          const int t = i % kPage;
          const int64_t page = pgs[i / kPage];
          if (page < 0) continue;
          uint32_t w = 0;
          for (int k2 = 0; k2 < 2; ++k2)
            for (int m = 0; m < 4; ++m)
              for (int hf = 0; hf < 2; ++hf)
                w |= (uint32_t)cs[i][32 * (2 * aw + k2) + 8 * g + 2 * m + hf] << (8 * k2 + 2 * m + 16 * hf);
          reinterpret_cast<uint32_t*>(page_head_mut(a.pool, page, kv, dm) + (size_t)(16 * g + t) * 2 * CB)[aw] = w;
        }
      } else {
        // value words: (page, token group g', channel c, a), all four slots of a group at once
        const int npg = (n + kPage - 1) / kPage;
        for (int idx = tid; idx < npg * 64 * NWL; idx += 256) {
          const int j = idx / (64 * NWL), r = idx % (64 * NWL);
          const int gg = r / (16 * NWL), c = (r / NWL) % 16, aw = r % NWL;
          const int64_t page = pgs[j];
          if (page < 0) continue;
          uint32_t w = 0;
          for (int m = 0; m < 2; ++m)
            for (int hf = 0; hf < 2; ++hf) {
              const int i = kPage * j + 4 * gg + 2 * m + hf;
              if (i >= n) continue;
              for (int n4 = 0; n4 < 4; ++n4)
                w |= (uint32_t)cs[i][16 * (4 * aw + n4) + c] << (2 * n4 + 8 * m + 16 * hf);
            }
          reinterpret_cast<uint32_t*>(page_head_mut(a.pool, page, kv, dm) + (size_t)(16 * gg + c) * 2 * CB + CB)[aw] = w;
        }
      }
    } else {
      // mixed widths: each wavefront stores the tokens it owns, merging value bits per slot
      for (int i = wave; i < n; i += 4) {
        const int bw = bits_s[i], slot = slot_s[i];
        const int32_t* pt = (bw == 4 ? a.pt4 : a.pt2) + (size_t)b * dm.pt_stride;
        if (slot / kPage >= dm.pt_stride) continue;
        store_token<D>(a, pt[slot / kPage], kv, bw, slot % kPage, sel, cs[i], szs[i], lane, kWave);
      }
    }
    __syncthreads();   // xs, xr, cs and the slot tables are rewritten by the next chunk
  }
}

// ------------------------------------------------------------------ prefill: INT2-only history
// The uniform INT2 code of x on grid g from the estimate t = (clamp(x) - z) * rcp(s), as
// quant_code_fast decides it: `redo` is set where the correctly rounded quotient must decide (t within
// 2^-14 of a rounding midpoint, |t| not below 32, t not a number -- which a zero scale also gives,
// its reciprocal being infinite; quant_code_exact then returns 0 as the rule does).
__device__ __forceinline__ uint32_t int2_code_estimate(float x, const QuantGrid& g, bool& redo) {
#pragma clang fp contract(off)
  const float xc = __builtin_amdgcn_fmed3f(x, g.lo, g.hi);
  const float t = (xc - g.z) * g.rs;
  const float r = rintf(t);
  redo = !(fabsf(t) < 32.0f) | !(fabsf(t - r) < 0.5f - 0x1p-14f);
  return (uint32_t)__builtin_amdgcn_fmed3f(r, 0.0f, 3.0f);
}

// Rows of a chunk in LDS without padding: 16-byte piece c of row r sits at slot c ^ swz(r) of the
// row, so the 16 lanes of a 256-byte LDS pass that read one piece of 16 consecutive rows (the A
// operand below) hit 16 different slots. At d = 128 a row is one pass wide (swz = r mod 16); at
// d = 64 two rows share a pass (swz = (r / 2) mod 8).
template <int D>
__device__ __forceinline__ int piece_swizzle(int r) {
  return D == 128 ? r % 16 : (r / 2) % 8;
}

// A operand (rows row0..row0+31, k-step kk) of the 32x32x16 product from the swizzled rows.
template <int D>
__device__ __forceinline__ bf16x8_t swizzled_rotation_a(const uint16_t* x, int row0, int kk, int lane) {
  const int m = row0 + lane % 32, c = 2 * kk + lane / 32;
  return __builtin_bit_cast(bf16x8_t,
                            *reinterpret_cast<const u32x4_t*>(x + m * D + 8 * (c ^ piece_swizzle<D>(m))));
}

// Both 32-row tiles of a chunk (swizzled rows; rows past the chunk's history are zeros there) times
// the wavefront's slice of R: rotate_tile's products in rotate_tile's order for each tile, the two
// tiles' chains interleaved so each hides the other's matrix-core latency.
template <int D>
__device__ __forceinline__ void rotate_swizzled_pair(const RotSlice<D>& rs, const uint16_t* x, int lane,
                                                     float16v_t& acc0, float16v_t& acc1) {
  acc0 = float16v_t{};
  acc1 = float16v_t{};
#pragma unroll
  for (int kk = 0; kk < RotSlice<D>::KS; ++kk) {
    const bf16x8_t a0 = swizzled_rotation_a<D>(x, 0, kk, lane);
    const bf16x8_t a1 = swizzled_rotation_a<D>(x, 32, kk, lane);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, rs.lo[kk], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, rs.lo[kk], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, rs.mid[kk], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, rs.mid[kk], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, rs.hi[kk], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, rs.hi[kk], acc1, 0, 0, 0);
  }
}

// 16 bytes per lane from a raw buffer (byte offset voff of the lane) straight into LDS: lane L
// writes bytes 16L..16L+15 from `lds`, which must be the same for the whole wavefront.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Wait until at most N vector memory operations of the wavefront are outstanding (loads into LDS
// included), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier after the wavefront's LDS operations. The compiler's own barrier would also
// wait for every row load still streaming into LDS, which is what the loads run ahead to avoid.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Threads of the INT2 prefill: 4 rotating wavefronts, and 64 rows x 4 * (D / 64) quantising threads.
template <int D>
constexpr int kPrefillThreads = 256 + 64 * 4 * (D / 64);

// The history of an INT2-only cache (every token takes consecutive INT2 slots, so a chunk of 64
// positions owns 4 whole pages), with the rotation and code rule of prefill_hist_kernel. One
// workgroup per compute unit and (run of `run` chunks, kv-head, request x {K, V}): wavefronts 0..3
// rotate (matrix cores) and issue every load, the other wavefronts (8 at d = 128, two per SIMD; 4 at
// d = 64) quantise and store, one chunk apart, so the matrix cores and the vector units work at
// once. In iteration i the rotating wavefronts publish chunk i's page ids, issue chunk i+1's
// page-id loads and chunk i+2's row loads (straight into the third of three LDS row buffers), and
// rotate chunk i; the quantising ones quantise and store chunk i-1. A load is thus never waited on
// behind the stores (one counter covers both), a chunk's rows have two iterations to arrive, and
// the rotated rows and page ids passed between the sides are double-buffered, so one workgroup
// barrier per iteration orders them all (each side runs its own loop with as many barriers, so
// neither side's registers stay live in the other's).
// A quantising thread (row, a, q), a < NWL = D/64 words per lane part, q < 4, takes 16 channels and
// assembles whole page-head words in registers:
//  * keys: key word (g, a) of a token holds channels 64a + 32k2 + 8g + j (k2 < 2, j < 8) at bit
//    8k2 + 2(j/2) + 16(j%2): thread q takes word (q, a) and stores it;
//  * values: value word (column cv, a) of a group of 4 tokens holds channels 64a + 16n4 + cv
//    (n4 < 4) of tokens 2m + hf at bit 2n4 + 8m + 16hf: thread q places its row's codes of columns
//    4q + u (u < 4) of word a; the 4 rows of a group are the 4 lanes of a quad, where two DPP swaps
//    and ORs complete the words, and the lane of row r stores column 4q + r.
// Lane l of a quantising wavefront: r = l % 4 (row within its group), q = (l / 4) % 4, s = l / 16
// (a = s % NWL, row group s / NWL).
template <int D, bool CBK>
__global__ __launch_bounds__(kPrefillThreads<D>, 1) void prefill_int2_kernel(CacheWriteArgs a, int run) {
  constexpr int CH = kPrefillChunk;
  constexpr int RS = D + 16;    // fp32 row pitch: consecutive rows 16 banks apart
  constexpr int SL = RotSlice<D>::SLICES;
  constexpr int CB = D * 2 / 32;         // bytes of a lane's key (or value) part
  constexpr int NWL = CB / 4;            // its words
  constexpr int RPW = 16 / NWL;          // rows per quantising wavefront
  constexpr int XW = CH * D * 2 / 1024 / 4;   // 1 KB row blocks of a chunk per rotating wavefront
  constexpr int CP = CH / kPage;              // pages of a chunk
  static_assert(NWL == 1 || NWL == 2, "d = 64 or 128");
  // three row buffers as separate arrays: the compiler then sees that reading one does not wait
  // for the loads still streaming into another
  __shared__ __attribute__((aligned(16))) uint16_t xs0[CH * D];
  __shared__ __attribute__((aligned(16))) uint16_t xs1[CH * D];
  __shared__ __attribute__((aligned(16))) uint16_t xs2[CH * D];
  __shared__ __attribute__((aligned(16))) float xr[2][CH][RS];
  __shared__ int64_t pgs[2][CP];
  const Dims& dm = a.dm;
  const int kv = blockIdx.y, b = blockIdx.z / 2, sel = blockIdx.z % 2;
  const int tid = threadIdx.x, lane = tid % kWave;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > dm.max_seq_len ? dm.max_seq_len : T);
  const int hist = T - dm.sink - dm.recent;
  const int chunk0 = run * blockIdx.x;
  // the window of this (request, kv-head, K or V) is shared among the launch's runs (the cache has
  // no INT4 tokens: its count is 0)
  if (a.n_int4_out && blockIdx.x == 0 && kv == 0 && sel == 0 && tid == 0) a.n_int4_out[b] = 0;
  if (CH * chunk0 >= hist) {   // no history chunk for the workgroup: only its window pages
    window_slice<kPrefillThreads<D>>(a, b, kv, sel, T, blockIdx.x, gridDim.x, tid);
    return;
  }
  const int nchunks = min(run, (hist - CH * chunk0 + CH - 1) / CH);
  if (tid < 256) {
    // rotating wavefronts: they also issue every load of the kernel (rows, page ids) ahead of its
    // use, so no load waits behind the quantising wavefronts' stores
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint16_t* src = (sel ? a.v : a.k) + ((size_t)b * dm.hkv + kv) * dm.max_seq_len * D;
    // a chunk's rows into row buffer `buf`, through a raw buffer descriptor over its n rows (pieces
    // of rows at or past n arrive as zeros; a chunk past the history has n = 0 and reads nothing).
    // Each load writes one 1 KB block of the buffer, lane L its 16-byte slot L; the global piece it
    // fetches is the one the swizzle puts in that slot.
    int goff[XW];
#pragma unroll
    for (int e = 0; e < XW; ++e) {
      const int slot = 64 * (XW * wave + e) + lane;
      const int row = slot / (D / 8), c = (slot % (D / 8)) ^ piece_swizzle<D>(row);
      goff[e] = 16 * (row * (D / 8) + c);
    }
    auto load_rows = [&](int chunk, uint16_t* buf) {
      const int p0 = dm.sink + CH * chunk;
      // uniform by construction; said so, or the compiler may place it in a vector register and
      // loop over the "distinct" descriptors
      const int n = __builtin_amdgcn_readfirstlane(max(0, min(CH, hist - CH * chunk)));
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(src + (size_t)p0 * D), (short)0, n * D * 2, kRawBufferFlags);
#pragma unroll
      for (int e = 0; e < XW; ++e)
        buffer_load_lds16(r, buf + 512 * (XW * wave + e), goff[e]);
    };
    // page id of page tid % CP of a chunk through a raw buffer descriptor over the request's page
    // table (a page past it reads as 0 and is dropped when published), kept as loaded until it is
    // published an iteration later, so the load is not waited on at once
    const __amdgpu_buffer_rsrc_t ptr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.pt2 + (size_t)b * dm.pt_stride), (short)0, 4 * dm.pt_stride, kRawBufferFlags);
    auto load_page = [&](int chunk) -> int32_t {
      return __builtin_amdgcn_raw_buffer_load_b32(ptr, 4 * (CP * chunk + tid % CP), 0, 0);
    };
    RotSlice<D> rs;
    if (wave < SL) rs.load((sel ? a.rot_v : a.rot_k) + (size_t)kv * D * D, wave, lane);
    // Every iteration issues the same loads (past the run: an empty row range, a page id that is
    // not published), so the count of loads in flight is the same on every path.
    int32_t pv = load_page(chunk0);
    load_rows(chunk0, xs0);
    load_rows(chunk0 + 1, xs1);
    wait_vmem<XW>();   // everything but chunk 1's rows
    lds_barrier();
    // iteration i on row buffers cur (chunk i) and ahead (chunk i+2); the loop steps through the
    // three buffers in turn, so each access names its buffer
    auto iteration = [&](int i, const uint16_t* cur, uint16_t* ahead) {
      if (i > nchunks) return;
      // chunk i's page ids (read by the quantising wavefronts in iteration i+1)
      if (tid < CP && i < nchunks)
        pgs[i % 2][tid] = CP * (chunk0 + i) + tid < dm.pt_stride && page_ok((int64_t)pv, 2, dm) ? (int64_t)pv : -1;
      pv = load_page(chunk0 + i + 1);
      load_rows(chunk0 + i + 2, ahead);
      if (i < nchunks && wave < SL) {
        float16v_t acc0, acc1;
        rotate_swizzled_pair<D>(rs, cur, lane, acc0, acc1);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = 8 * (j / 4) + 4 * (lane / 32) + j % 4, col = 32 * wave + lane % 32;
          xr[i % 2][r][col] = acc0[j];
          xr[i % 2][32 + r][col] = acc1[j];
        }
      }
      wait_vmem<XW>();   // chunk i+1's rows and page ids have arrived (chunk i+2's may still stream in)
      lds_barrier();
    };
    for (int i = 0; i < nchunks + 1; i += 3) {
      iteration(i, xs0, xs2);
      iteration(i + 1, xs1, xs0);
      iteration(i + 2, xs2, xs1);
    }
    wait_vmem<0>();   // no load may still write this workgroup's LDS once its wavefronts end
    return;
  }
  // quantising wavefronts: stores only (the window pages of the workgroup first, while the rotating
  // wavefronts load the rotation and the first chunks)
  const int ct = tid - 256;
  window_slice<kPrefillThreads<D> - 256>(a, b, kv, sel, T, blockIdx.x, gridDim.x, ct);
  // the K and V workgroups run separately instantiated quantiser loops (SELV = 0: keys, 1: values),
  // so the channel map, the bit positions and the word choice are compile-time constants
  auto quantise = [&](auto selc) {
    constexpr int SELV = decltype(selc)::value;
    const Codebook cb = load_codebook(CBK ? a.codebook : nullptr, kv, SELV);
    const float clip = SELV ? a.clip_v : a.clip_k;
    const int r4 = lane % 4, q = (lane / 4) % 4, s4 = lane / 16;
    const int wa = s4 % NWL;                                   // word a of the thread
    const int row = RPW * (ct / kWave) + 4 * (s4 / NWL) + r4;  // its row of the chunk
    const int vbase = 8 * (r4 / 2) + 16 * (r4 % 2);            // value words: bit 8m + 16hf of the row's token
    // channel of the thread's value e = 4c + u: keys 64a + 32(c/2) + 8q + 4(c%2) + u, values
    // 64a + 16c + 4q + u
    auto chan4 = [&](int c) { return SELV == 0 ? 64 * wa + 32 * (c / 2) + 8 * q + 4 * (c % 2) : 64 * wa + 16 * c + 4 * q; };
    // bit of value e in its word: keys 8(c/2) + 4(c%2) + 2(u/2) + 16(u%2) (one word), values
    // vbase + 2c in word u (column 4q + u)
    auto bit_of = [&](int e) {
      const int c = e / 4, u = e % 4;
      return SELV == 0 ? 8 * (c / 2) + 4 * (c % 2) + 2 * (u / 2) + 16 * (u % 2) : vbase + 2 * c;
    };
    __syncthreads();
    for (int i = 0; i < nchunks + 1; ++i) {
      if (i >= 1) {
        // quantise and store chunk i-1 from the rotated rows of its buffer
        const int chunk = chunk0 + i - 1, qb = (i - 1) % 2;
        const int n = min(CH, hist - CH * chunk);
        const bool live = row < n;
        float x[16];
  #pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 v = *reinterpret_cast<const float4*>(&xr[qb][row][chan4(c)]);
          x[4 * c] = v.x;
          x[4 * c + 1] = v.y;
          x[4 * c + 2] = v.z;
          x[4 * c + 3] = v.w;
        }
        float mn = x[0], mx = x[0];
  #pragma unroll
        for (int e = 1; e < 16; ++e) {
          mn = fminf(mn, x[e]);
          mx = fmaxf(mx, x[e]);
        }
        // the row's threads: lanes 4q + r4 of the DPP row (q < 4), and for two words the same lanes
        // of the DPP row 16 lanes away
        mn = fminf(mn, dpp_row_ror<4>(mn));
        mx = fmaxf(mx, dpp_row_ror<4>(mx));
        mn = fminf(mn, dpp_row_ror<8>(mn));
        mx = fmaxf(mx, dpp_row_ror<8>(mx));
        if constexpr (NWL == 2) {
          mn = fminf(mn, __shfl_xor(mn, 16, kWave));
          mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        }
        const QuantGrid g = make_grid(mn, mx, clip, 3);
        // A row whose whole estimate range [t(lo), t(hi)] lies in (-0.5, 3.5) (so |t| < 32 and the
        // rounded estimate needs no clamp) takes the short form of the uniform rule; t is monotone
        // in x, so the bound holds for every clamped value of the row. Other rows (a zero or tiny
        // scale, a zero point far off the range) take int2_code_estimate.
        bool short_row = false;
        if (!CBK) {
  #pragma clang fp contract(off)
          const float tlo = (g.lo - g.z) * g.rs, thi = (g.hi - g.z) * g.rs;
          short_row = g.s > 0.0f && tlo > -0.5f && thi < 3.5f;
        }
        uint32_t w[4];   // keys: w[0] only; values: column 4q + u in w[u]
  #pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = 0;
        auto word_of = [&](int e) { return SELV == 0 ? 0 : e % 4; };
        uint32_t redo = 0;
        if (CBK) {
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
            bool r;
            w[word_of(e)] |= cb_code_fast(x[e], g, cb, r) << bit_of(e);
            redo |= (uint32_t)r << e;
          }
        } else if (short_row) {
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
  #pragma clang fp contract(off)
            const float t = (__builtin_amdgcn_fmed3f(x[e], g.lo, g.hi) - g.z) * g.rs;
            const float rt_ = rintf(t);
            redo |= (uint32_t)!(fabsf(t - rt_) < 0.5f - 0x1p-14f) << e;
            w[word_of(e)] |= (uint32_t)rt_ << bit_of(e);
          }
        } else {
  #pragma unroll
          for (int e = 0; e < 16; ++e) {
            bool r;
            w[word_of(e)] |= int2_code_estimate(x[e], g, r) << bit_of(e);
            redo |= (uint32_t)r << e;
          }
        }
        // the rare codes the correctly rounded quotient decides
        while (redo) {
          const int e = __builtin_ctz(redo);
          redo &= redo - 1;
          const float xv = xr[qb][row][chan4(e / 4) + e % 4];
          const uint32_t code = CBK ? cb_code_exact(xv, g, cb) : quant_code_exact(xv, g, 3);
          const int sh = bit_of(e);
  #pragma unroll
          for (int k = 0; k < 4; ++k)
            if (k == word_of(e)) w[k] = (w[k] & ~(3u << sh)) | (code << sh);
        }
        const int64_t page = pgs[qb][row / kPage];
        uint8_t* ph = page >= 0 ? page_head_mut(a.pool, page, kv, dm) : nullptr;
        const int t = row % kPage;
        if (SELV == 0) {
          if (live && ph) reinterpret_cast<uint32_t*>(ph + (size_t)(16 * q + t) * 2 * CB)[wa] = w[0];
        } else {
          // rows past the history add nothing; the quad's 4 rows complete the group's words
  #pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t v = live ? w[k] : 0u;
            v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true);   // quad swap 1,0,3,2
            v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true);   // quad swap 2,3,0,1
            w[k] = v;
          }
          const uint32_t v = r4 == 0 ? w[0] : (r4 == 1 ? w[1] : (r4 == 2 ? w[2] : w[3]));
          if ((row & ~3) < n && ph)
            reinterpret_cast<uint32_t*>(ph + (size_t)(16 * (t / 4) + 4 * q + r4) * 2 * CB + CB)[wa] = v;
        }
        if (live && ph && wa == 0 && q == 0)
          reinterpret_cast<uint32_t*>(ph + 4 * D * 2)[2 * t + SELV] = g.s_bits | (g.z_bits << 16);
      }
      __syncthreads();
    }
  };
  if (sel == 0) quantise(std::integral_constant<int, 0>{});
  else quantise(std::integral_constant<int, 1>{});
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
  const int hmax = dm.max_seq_len - dm.sink - dm.recent;
  // an INT2-only cache with history positions has its window copied by the history launch
  if (dm.mixed || hmax <= 0) {
    hipLaunchKernelGGL(prefill_window_kernel, dim3(dm.wpages, dm.hkv, dm.batch), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (hmax <= 0) return hipSuccess;
  const int runs = (hmax + kPrefillChunk * kPrefillChunks - 1) / (kPrefillChunk * kPrefillChunks);
  const dim3 grid(runs, dm.hkv, 2 * dm.batch);   // z: request x {K, V}
  if (!dm.mixed) {
    // INT2-only: one 8-wavefront workgroup per compute unit, each taking an equal run of chunks of
    // its (request, kv-head, K or V) so that the launch fills the device in whole rounds
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    const int64_t hchunks = (hmax + kPrefillChunk - 1) / kPrefillChunk;
    const int64_t groups = (int64_t)dm.hkv * 2 * dm.batch;
    int64_t run = std::max<int64_t>(1, (hchunks * groups + cus - 1) / cus);
    const int64_t per_group = (hchunks + run - 1) / run;
    run = (hchunks + per_group - 1) / per_group;
    const dim3 g2((unsigned)per_group, dm.hkv, 2 * dm.batch);
    const int r = (int)run;
    const dim3 b128(kPrefillThreads<128>), b64(kPrefillThreads<64>);
    if (a.codebook) {
      if (dm.d == 128)
        hipLaunchKernelGGL((prefill_int2_kernel<128, true>), g2, b128, 0, stream, a, r);
      else
        hipLaunchKernelGGL((prefill_int2_kernel<64, true>), g2, b64, 0, stream, a, r);
    } else {
      if (dm.d == 128)
        hipLaunchKernelGGL((prefill_int2_kernel<128, false>), g2, b128, 0, stream, a, r);
      else
        hipLaunchKernelGGL((prefill_int2_kernel<64, false>), g2, b64, 0, stream, a, r);
    }
  } else if (a.codebook) {
    if (dm.d == 128)
      hipLaunchKernelGGL((prefill_hist_kernel<128, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_hist_kernel<64, true>), grid, dim3(256), 0, stream, a);
  } else {
    if (dm.d == 128)
      hipLaunchKernelGGL((prefill_hist_kernel<128, false>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_hist_kernel<64, false>), grid, dim3(256), 0, stream, a);
  }
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
