// Offline rotation construction behind the C ABI (host code only; nothing runs on a device).
//
// "Together AI open-sources OSCAR", section on what makes OSCAR different: keys are rotated by
// R_K = U_Q . H . P_br and values by R_V = U_S . H . P_br, where U is the eigenbasis of an
// attention covariance (C_Q for keys, C_S for values), H the orthonormal Sylvester Hadamard
// matrix of size head_dim and P_br the bit-reversal permutation (P[i, rev(i)] = 1).
//
// The eigenbasis comes from the cyclic Jacobi method in fp64: plane rotations, each zeroing one
// off-diagonal pair, swept row by row over the upper triangle until the off-diagonal mass is
// negligible. Jacobi is slow (O(d^3) per sweep, a few sweeps) but simple and accurate to the
// last bits for symmetric matrices, which suits an offline step run once per layer.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "oscar.h"

namespace {

constexpr int kMaxRotationDim = 256;
constexpr int kMaxSweeps = 64;

// Eigen-decomposition of the symmetric a [d][d] (destroyed): eigenvalues into w, eigenvectors as
// the columns of v [d][d]. Returns false if the sweeps did not converge.
bool jacobi_eigen(int d, double* a, double* w, double* v) {
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) v[i * d + j] = i == j ? 1.0 : 0.0;
  double total = 0.0;
  for (int i = 0; i < d * d; ++i) total += a[i] * a[i];
  bool converged = false;
  for (int sweep = 0; sweep < kMaxSweeps && !converged; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < d; ++p)
      for (int q = p + 1; q < d; ++q) off += a[p * d + q] * a[p * d + q];
    // off-diagonal mass below (1e-17)^2 of the matrix: the remaining rotations are below
    // rounding level of every entry
    if (off <= 1e-34 * total || off == 0.0) {
      converged = true;
      break;
    }
    for (int p = 0; p < d - 1; ++p) {
      for (int q = p + 1; q < d; ++q) {
        const double apq = a[p * d + q];
        if (apq == 0.0) continue;
        const double app = a[p * d + p], aqq = a[q * d + q];
        // rotation angle zeroing a_pq: t = tan(phi) is the smaller root of t^2 + 2 theta t - 1 = 0
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        // a <- J^T a J with J = identity except J_pp = J_qq = c, J_pq = s, J_qp = -s
        for (int k = 0; k < d; ++k) {
          const double akp = a[k * d + p], akq = a[k * d + q];
          a[k * d + p] = c * akp - s * akq;
          a[k * d + q] = s * akp + c * akq;
        }
        for (int k = 0; k < d; ++k) {
          const double apk = a[p * d + k], aqk = a[q * d + k];
          a[p * d + k] = c * apk - s * aqk;
          a[q * d + k] = s * apk + c * aqk;
        }
        a[p * d + q] = 0.0;
        a[q * d + p] = 0.0;
        for (int k = 0; k < d; ++k) {
          const double vkp = v[k * d + p], vkq = v[k * d + q];
          v[k * d + p] = c * vkp - s * vkq;
          v[k * d + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  for (int i = 0; i < d; ++i) w[i] = a[i * d + i];
  return converged;
}

int bit_reverse(int i, int bits) {
  int r = 0;
  for (int b = 0; b < bits; ++b)
    if (i >> b & 1) r |= 1 << (bits - 1 - b);
  return r;
}

int popcount(unsigned x) {
  int n = 0;
  for (; x; x &= x - 1) ++n;
  return n;
}

}  // namespace

extern "C" oscar_status_t oscar_rotation_from_covariance(int32_t n_mats, int32_t head_dim, const double* cov_host,
                                                         float* rot_host, double* eigvals_host,
                                                         double* eigvecs_host) {
  if (n_mats < 0 || head_dim < 1 || (head_dim & (head_dim - 1))) return OSCAR_ERR_INVALID_ARG;
  if (head_dim > kMaxRotationDim) return OSCAR_ERR_UNSUPPORTED;
  if (n_mats == 0) return OSCAR_OK;
  if (!cov_host || !rot_host) return OSCAR_ERR_INVALID_ARG;
  const int d = head_dim;
  int bits = 0;
  while ((1 << bits) < d) ++bits;
  for (int64_t i = 0; i < (int64_t)n_mats * d * d; ++i)
    if (!isfinite(cov_host[i])) return OSCAR_ERR_INVALID_ARG;
  std::vector<double> a((size_t)d * d), v((size_t)d * d), w(d), u((size_t)d * d);
  std::vector<int> order(d);
  const double hs = 1.0 / sqrt((double)d);
  for (int m = 0; m < n_mats; ++m) {
    const double* c = cov_host + (size_t)m * d * d;
    // the symmetric part of the input (a covariance accumulated in floating point may differ
    // from its transpose by rounding)
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) a[i * d + j] = 0.5 * (c[i * d + j] + c[j * d + i]);
    if (!jacobi_eigen(d, a.data(), w.data(), v.data())) return OSCAR_ERR_UNSUPPORTED;
    // descending eigenvalues (equal ones keep their Jacobi order)
    for (int i = 0; i < d; ++i) order[i] = i;
    for (int i = 1; i < d; ++i) {
      const int o = order[i];
      int j = i;
      for (; j > 0 && w[order[j - 1]] < w[o]; --j) order[j] = order[j - 1];
      order[j] = o;
    }
    // U: column j = eigenvector order[j], its largest-magnitude entry (first such) made positive
    for (int j = 0; j < d; ++j) {
      const int col = order[j];
      int imax = 0;
      for (int i = 1; i < d; ++i)
        if (fabs(v[i * d + col]) > fabs(v[imax * d + col])) imax = i;
      const double sg = v[imax * d + col] < 0.0 ? -1.0 : 1.0;
      for (int i = 0; i < d; ++i) u[i * d + j] = sg * v[i * d + col];
    }
    // R = U . H . P_br: (U H)[i][m] = sum_k U[i][k] H[k][m] with H[k][m] = (-1)^popcount(k & m) / sqrt(d),
    // and (A P_br)[i][j] = A[i][rev(j)]; formed in fp64, rounded once to fp32
    float* r = rot_host + (size_t)m * d * d;
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        const int col = bit_reverse(j, bits);
        double acc = 0.0;
        for (int k = 0; k < d; ++k) acc += (popcount((unsigned)(k & col)) & 1) ? -u[i * d + k] : u[i * d + k];
        r[i * d + j] = (float)(acc * hs);
      }
    if (eigvals_host)
      for (int j = 0; j < d; ++j) eigvals_host[(size_t)m * d + j] = w[order[j]];
    if (eigvecs_host) memcpy(eigvecs_host + (size_t)m * d * d, u.data(), sizeof(double) * d * d);
  }
  return OSCAR_OK;
}
