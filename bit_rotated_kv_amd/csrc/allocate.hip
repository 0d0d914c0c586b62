// TriAxialKV bit allocation and token routing (TriAxialKV reading note, section 3: INT2 or INT4
// per tag class, minimising the summed attention-output distortion under an average-bit budget,
// greedily by gain per extra bit or exhaustively for small class counts; section 4: the dual
// INT2/INT4 pool that the routed token widths fill).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "oscar.h"

namespace {

constexpr int kMaxExhaustiveClasses = 24;
constexpr int kMaxRouteClasses = 64;
constexpr double kBudgetSlack = 1e-9;   // bits of slack on the budget test (rounding of B * sum N)

bool is_finite(double x) { return x == x && x != HUGE_VAL && x != -HUGE_VAL; }

// Greedy: raise classes from 2 to 4 bits in descending order of rho_k = (D_k(2) - D_k(4)) / (2 N_k)
// (ties: lower class index first); classes without a positive gain or without tokens stay at 2;
// the first class whose raise would exceed the budget ends the allocation.
void greedy(int n, const double* d2, const double* d4, const int64_t* counts, double allowed, int64_t used,
            uint8_t* bits) {
  std::vector<double> rho(n);
  for (int k = 0; k < n; ++k) rho[k] = (d2[k] - d4[k]) / (2.0 * std::max((double)counts[k], 1e-300));
  std::vector<int> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return rho[a] > rho[b]; });
  for (int k = 0; k < n; ++k) bits[k] = 2;
  double u = (double)used;
  for (int k : order) {
    if (d2[k] - d4[k] <= 0.0 || counts[k] == 0) continue;
    if (u + 2.0 * (double)counts[k] > allowed + kBudgetSlack) break;
    bits[k] = 4;
    u += 2.0 * (double)counts[k];
  }
}

// Exhaustive: every 2/4 choice, visited in reflected Gray-code order (one class changes per step),
// with the weight kept exactly in integers and the cost in extended precision; keeps the first
// feasible choice of least cost.
void exhaustive(int n, const double* d2, const double* d4, const int64_t* counts, double allowed, int64_t used,
                uint8_t* bits) {
  long double cost = 0.0L;
  for (int k = 0; k < n; ++k) cost += d2[k];
  int64_t w = used;
  uint32_t state = 0, best = 0;
  bool have = (double)w <= allowed + kBudgetSlack;
  long double best_cost = have ? cost : 0.0L;
  for (uint64_t i = 1; i < (1ull << n); ++i) {
    const int k = __builtin_ctzll(i);
    state ^= 1u << k;
    if ((state >> k) & 1u) {
      w += 2 * counts[k];
      cost += (long double)d4[k] - (long double)d2[k];
    } else {
      w -= 2 * counts[k];
      cost += (long double)d2[k] - (long double)d4[k];
    }
    if ((double)w <= allowed + kBudgetSlack && (!have || cost < best_cost)) {
      have = true;
      best = state;
      best_cost = cost;
    }
  }
  for (int k = 0; k < n; ++k) bits[k] = ((best >> k) & 1u) ? 4 : 2;
}

struct RouteArgs {
  int batch, max_seq_len, n_classes;
  const int32_t* seq_len;
  const int32_t* tags;
  uint8_t* bits;
  uint8_t class_bits[kMaxRouteClasses];
};

// token_bits[b][t] = class_bits[tags[b][t]] for t < seq_len[b]; four positions per thread.
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int b = blockIdx.y;
  int T = a.seq_len[b];
  T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
  const int t0 = 4 * (blockIdx.x * 256 + threadIdx.x);
  const size_t row = (size_t)b * a.max_seq_len;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t = t0 + e;
    if (t >= T) break;
    const int tag = a.tags[row + t];
    a.bits[row + t] = (tag >= 0 && tag < a.n_classes) ? a.class_bits[tag] : (uint8_t)2;
  }
}

}  // namespace

extern "C" {

oscar_status_t oscar_allocate_bits(int32_t n_classes, const double* d2, const double* d4, const int64_t* counts,
                                   double budget_bits, int32_t method, uint8_t* bits_out, double* cost_out) {
  if (n_classes < 0 || (method != OSCAR_ALLOC_GREEDY && method != OSCAR_ALLOC_EXHAUSTIVE))
    return OSCAR_ERR_INVALID_ARG;
  if (!is_finite(budget_bits) || budget_bits < 2.0) return OSCAR_ERR_INVALID_ARG;
  if (n_classes == 0) {
    if (cost_out) *cost_out = 0.0;
    return OSCAR_OK;
  }
  if (!d2 || !d4 || !counts || !bits_out) return OSCAR_ERR_INVALID_ARG;
  if (method == OSCAR_ALLOC_EXHAUSTIVE && n_classes > kMaxExhaustiveClasses) return OSCAR_ERR_UNSUPPORTED;
  int64_t total = 0;
  for (int k = 0; k < n_classes; ++k) {
    if (counts[k] < 0 || counts[k] > ((int64_t)1 << 50) || !is_finite(d2[k]) || !is_finite(d4[k]))
      return OSCAR_ERR_INVALID_ARG;
    total += counts[k];
  }
  const double allowed = budget_bits * (double)total;
  if (method == OSCAR_ALLOC_GREEDY)
    greedy(n_classes, d2, d4, counts, allowed, 2 * total, bits_out);
  else
    exhaustive(n_classes, d2, d4, counts, allowed, 2 * total, bits_out);
  if (cost_out) {
    double c = 0.0;
    for (int k = 0; k < n_classes; ++k) c += bits_out[k] == 4 ? d4[k] : d2[k];
    *cost_out = c;
  }
  return OSCAR_OK;
}

oscar_status_t oscar_route_tokens(int32_t batch, int32_t max_seq_len, const int32_t* seq_len, const int32_t* tags,
                                  int32_t n_classes, const uint8_t* class_bits, uint8_t* token_bits,
                                  hipStream_t stream) {
  if (batch < 0 || max_seq_len < 0 || n_classes < 0 || n_classes > kMaxRouteClasses) return OSCAR_ERR_INVALID_ARG;
  if (batch == 0 || max_seq_len == 0) return OSCAR_OK;
  if (!seq_len || !tags || !token_bits || (n_classes > 0 && !class_bits)) return OSCAR_ERR_INVALID_ARG;
  if (batch > 65535) return OSCAR_ERR_UNSUPPORTED;
  RouteArgs a{};
  a.batch = batch;
  a.max_seq_len = max_seq_len;
  a.n_classes = n_classes;
  a.seq_len = seq_len;
  a.tags = tags;
  a.bits = token_bits;
  for (int k = 0; k < n_classes; ++k) {
    if (class_bits[k] != 2 && class_bits[k] != 4) return OSCAR_ERR_INVALID_ARG;
    a.class_bits[k] = class_bits[k];
  }
  const unsigned blocks = (unsigned)((max_seq_len + 1023) / 1024);
  hipLaunchKernelGGL(route_kernel, dim3(blocks, batch), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? OSCAR_OK : OSCAR_ERR_LAUNCH;
}

}  // extern "C"
