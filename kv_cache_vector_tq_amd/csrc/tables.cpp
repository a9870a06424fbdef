// Host-side construction of the constant tables (double precision, then
// rounded): Lloyd-Max codebooks for N(0,1) scaled by 1/sqrt(d) and stored as
// half-precision values (the pages leave the storage precision open), the dense
// Haar rotation from Gaussian draws by Householder QR, Rademacher signs for
// the Hadamard variant, and the QJL matrix.
//
// Codebook: each rotated coordinate of a unit vector is close to N(0, 1/d)
// and is quantised with a precomputed MSE-optimal scalar quantiser
// ("TurboQuant on a 16GB MacBook", "Why this caught my eye"; "aither-kvcache"
// README, "Algorithm").  Built by Lloyd iteration (cell centroid =
// conditional mean, boundary = midpoint), started from evenly spaced levels,
// kept symmetric by iterating the positive half, stopped below 1e-14.
// Rotation: a fixed random orthogonal matrix (README "Algorithm" step 2); the
// Q factor of a Gaussian matrix with the signs of diag(R) folded in is Haar
// distributed.
#include <cmath>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

double pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

double upper_tail(double x) {
  if (x == INFINITY) return 0.0;
  if (x == -INFINITY) return 1.0;
  return 0.5 * std::erfc(x / std::sqrt(2.0));
}

// P(a < X <= b), from the tail nearer the cell for accuracy.
double mass(double a, double b) {
  if (a >= 0.0) return upper_tail(a) - upper_tail(b);
  if (b <= 0.0) return upper_tail(-b) - upper_tail(-a);
  return 1.0 - upper_tail(b) - upper_tail(-a);
}

}  // namespace

std::vector<double> lloyd_max_normal(int bits) {
  const int levels = 1 << bits, half = levels / 2;
  std::vector<double> pos(half), nxt(half), edge(half + 1);
  for (int k = 0; k < half; ++k) pos[k] = (k + 0.5) * 2.0 / half;
  for (int it = 0; it < 1000000; ++it) {
    edge[0] = 0.0;
    for (int k = 1; k < half; ++k) edge[k] = 0.5 * (pos[k - 1] + pos[k]);
    edge[half] = INFINITY;
    double delta = 0.0;
    for (int k = 0; k < half; ++k) {
      nxt[k] = (pdf(edge[k]) - pdf(edge[k + 1])) / mass(edge[k], edge[k + 1]);
      delta = std::fmax(delta, std::fabs(nxt[k] - pos[k]));
    }
    pos.swap(nxt);
    if (delta < 1e-14) break;
  }
  std::vector<double> out(levels);
  for (int k = 0; k < half; ++k) {
    out[half + k] = pos[k];
    out[half - 1 - k] = -pos[k];
  }
  return out;
}

void codebook_f32(int bits, int d, float* centroids, float* boundaries) {
  std::vector<double> unit = lloyd_max_normal(bits);
  const int L = 1 << bits;
  const double scale = 1.0 / std::sqrt(static_cast<double>(d));
  // levels are stored as half-precision values (rounded once from double)
  std::vector<float> c(L);
  for (int k = 0; k < L; ++k) c[k] = static_cast<float>(static_cast<_Float16>(unit[k] * scale));
  if (centroids) std::memcpy(centroids, c.data(), L * sizeof(float));
  if (boundaries)
    for (int k = 0; k + 1 < L; ++k)
      boundaries[k] = static_cast<float>(0.5 * (static_cast<double>(c[k]) + static_cast<double>(c[k + 1])));
}

// Householder QR of the d x d row-major matrix g; writes Q (row-major, f32)
// scaled so that R has a positive diagonal.
void haar_rotation_f32(const double* g, int d, float* out) {
  std::vector<double> a(g, g + static_cast<size_t>(d) * d);  // working copy, row-major
  std::vector<double> vs(static_cast<size_t>(d) * d, 0.0);     // reflector k in row k (entries k..d-1)
  std::vector<double> rdiag(d);
  for (int k = 0; k < d; ++k) {
    double nrm = 0.0;
    for (int i = k; i < d; ++i) nrm += a[i * d + k] * a[i * d + k];
    nrm = std::sqrt(nrm);
    const double x0 = a[k * d + k];
    const double alpha = (x0 >= 0.0) ? -nrm : nrm;  // R_kk = alpha
    double* v = &vs[static_cast<size_t>(k) * d];
    for (int i = k; i < d; ++i) v[i] = a[i * d + k];
    v[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += v[i] * v[i];
    if (vn > 0.0) {
      const double inv = 1.0 / std::sqrt(vn);
      for (int i = k; i < d; ++i) v[i] *= inv;
      for (int j = k; j < d; ++j) {
        double s = 0.0;
        for (int i = k; i < d; ++i) s += v[i] * a[i * d + j];
        for (int i = k; i < d; ++i) a[i * d + j] -= 2.0 * v[i] * s;
      }
    }
    rdiag[k] = a[k * d + k];
  }
  // Q = H_0 H_1 ... H_{d-1}: apply reflectors to the identity, last first.
  std::vector<double> q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* v = &vs[static_cast<size_t>(k) * d];
    for (int j = 0; j < d; ++j) {
      double s = 0.0;
      for (int i = k; i < d; ++i) s += v[i] * q[i * d + j];
      for (int i = k; i < d; ++i) q[i * d + j] -= 2.0 * v[i] * s;
    }
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const double sgn = (rdiag[j] < 0.0) ? -1.0 : 1.0;
      out[i * d + j] = static_cast<float>(q[i * d + j] * sgn);
    }
}

}  // namespace tq
