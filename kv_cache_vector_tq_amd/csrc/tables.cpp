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
// Seeded draws: when the caller passes no draws, the Gaussian matrices come
// from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) keyed by the
// seed, turned into normals by the Box-Muller transform.
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

namespace {

// One Philox4x32 round: two 32x32 -> 64-bit products, the counter words
// permuted and mixed with the key.
inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c[0];
  const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c[2];
  const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
  const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
  const uint32_t n0 = hi1 ^ c[1] ^ k[0], n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

}  // namespace

void philox4x32_10(uint32_t ctr[4], const uint32_t key[2]) {
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {  // key schedule: Weyl increments (golden ratio, sqrt(3) - 1)
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    philox_round(ctr, k);
  }
}

// Draws 2j and 2j+1 of stream `stream` come from Philox block j: counter
// (j mod 2^32, j / 2^32, stream, 0), key (seed mod 2^32, seed / 2^32).  Its
// words give two 53-bit uniforms u1 = (w0 >> 5, w1 >> 6), u2 = (w2 >> 5,
// w3 >> 6) in [0, 1), and Box-Muller gives sqrt(-2 ln(1 - u1)) cos(2 pi u2)
// and sqrt(-2 ln(1 - u1)) sin(2 pi u2).
void seed_normals(uint64_t seed, int stream, int64_t n, double* out) {
  const uint32_t key[2] = {static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32)};
  const double two_pi = 6.283185307179586;
  for (int64_t j = 0; 2 * j < n; ++j) {
    uint32_t c[4] = {static_cast<uint32_t>(j), static_cast<uint32_t>(static_cast<uint64_t>(j) >> 32),
                     static_cast<uint32_t>(stream), 0u};
    philox4x32_10(c, key);
    const double u1 = (static_cast<double>(c[0] >> 5) * 67108864.0 + static_cast<double>(c[1] >> 6)) *
                      (1.0 / 9007199254740992.0);
    const double u2 = (static_cast<double>(c[2] >> 5) * 67108864.0 + static_cast<double>(c[3] >> 6)) *
                      (1.0 / 9007199254740992.0);
    const double rad = std::sqrt(-2.0 * std::log(1.0 - u1));
    out[2 * j] = rad * std::cos(two_pi * u2);
    if (2 * j + 1 < n) out[2 * j + 1] = rad * std::sin(two_pi * u2);
  }
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
