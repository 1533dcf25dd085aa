// Host-side codebook builder for the two RVQ stages: kvq_build_codebooks.
//
// Stage 1 is the 2^b-level Lloyd-Max quantizer of N(0, 1/d) (VeloxQuant-MLX blog, "rvq"
// tag page, "The pipeline, as it actually runs": a Gaussian codebook; "turboquant" tag
// page, "Kernel 2": a Lloyd-Max codebook). 1/d is the variance of one coordinate of a
// rotated unit vector. Stage 2 is the 2^b-level Lloyd-Max quantizer of a zero-mean Laplace
// density ("Laplacian-fit") whose variance equals the stage-1 distortion mse_g/d, so the
// codebooks are analytical and need no data ("kivi" tag page, second post, "Where KIVI
// fits"). Boundaries are midpoints of neighbouring centroids ("rvq" tag page, "What
// 'quantize' means here, precisely").
//
// Both densities are symmetric and log-concave, so the Lloyd-Max quantizer is unique and
// symmetric: only the positive half is iterated (cells [0, t1], [t1, t2], ..., [t_m, inf)
// with t_k the midpoints) and mirrored. Iteration runs in double precision until no
// centroid moves by more than 1e-15 (the float32 tables need about 1e-8).

#include <cmath>
#include <cstring>

#include "kvq.h"

namespace {

constexpr double kInvSqrt2Pi = 0.39894228040143267794;  // 1/sqrt(2 pi)
constexpr double kInvSqrt2 = 0.70710678118654752440;

double gauss_pdf(double x) { return kInvSqrt2Pi * std::exp(-0.5 * x * x); }
double gauss_upper_tail(double x) { return 0.5 * std::erfc(x * kInvSqrt2); }  // P(X > x)

// E[X | a < X < b], X ~ N(0,1), 0 <= a < b (b may be +inf).
double gauss_cell_mean(double a, double b) {
  if (std::isinf(b)) return gauss_pdf(a) / gauss_upper_tail(a);
  return (gauss_pdf(a) - gauss_pdf(b)) / (gauss_upper_tail(a) - gauss_upper_tail(b));
}

// E[X | a < X < b], X ~ Laplace(0, beta), 0 <= a < b (b may be +inf).
// With the density exp(-|x|/beta)/(2 beta): integral of x e^{-x/beta} = -beta (x + beta) e^{-x/beta}.
double laplace_cell_mean(double a, double b, double beta) {
  if (std::isinf(b)) return a + beta;
  const double ea = std::exp(-a / beta), eb = std::exp(-b / beta);
  return ((a + beta) * ea - (b + beta) * eb) / (ea - eb);
}

// Positive-half centroids of the unit-variance quantizer with 2^bits levels.
void lloyd_max_half(int bits, bool laplace, double* pos) {
  const int m = 1 << (bits - 1);
  const double beta = kInvSqrt2;  // Laplace scale with variance 2 beta^2 = 1
  // Start from evenly spaced points; any ordered start converges to the unique optimum.
  for (int k = 0; k < m; ++k) pos[k] = (k + 0.5) * (laplace ? 4.0 : 3.0) / m;
  double t[9];
  for (int it = 0; it < 200000; ++it) {
    t[0] = 0.0;
    for (int k = 1; k < m; ++k) t[k] = 0.5 * (pos[k - 1] + pos[k]);
    t[m] = INFINITY;
    double move = 0.0;
    for (int k = 0; k < m; ++k) {
      const double c = laplace ? laplace_cell_mean(t[k], t[k + 1], beta) : gauss_cell_mean(t[k], t[k + 1]);
      move = std::fmax(move, std::fabs(c - pos[k]));
      pos[k] = c;
    }
    if (move < 1e-15) break;
  }
}

// Unit-Gaussian distortion of a centroid-condition quantizer: 1 - E[Q^2].
double gauss_distortion(int bits, const double* pos) {
  const int m = 1 << (bits - 1);
  double eq2 = 0.0;
  for (int k = 0; k < m; ++k) {
    const double lo = (k == 0) ? 0.0 : 0.5 * (pos[k - 1] + pos[k]);
    const double hi_tail = (k == m - 1) ? 0.0 : gauss_upper_tail(0.5 * (pos[k] + pos[k + 1]));
    eq2 += 2.0 * pos[k] * pos[k] * (gauss_upper_tail(lo) - hi_tail);
  }
  return 1.0 - eq2;
}

// Full ascending float32 table from the positive half, and float32 midpoint boundaries.
void fill_tables(int bits, const double* pos, double sigma, float* c, float* b) {
  const int m = 1 << (bits - 1), k = 1 << bits;
  for (int i = 0; i < m; ++i) {
    const float v = static_cast<float>(sigma * pos[i]);
    c[m + i] = v;
    c[m - 1 - i] = -v;
  }
  for (int i = 0; i + 1 < k; ++i)
    b[i] = static_cast<float>(0.5 * (static_cast<double>(c[i]) + static_cast<double>(c[i + 1])));
}

}  // namespace

extern "C" kvq_status kvq_build_codebooks(int32_t d, int32_t bits, const int8_t* signs, kvq_codebooks* out) {
  if (out == nullptr) return KVQ_ERR_ARG;
  if (d < KVQ_MIN_D || d > KVQ_MAX_D) return KVQ_ERR_SHAPE;
  if (bits < 1 || bits > KVQ_MAX_BITS) return KVQ_ERR_SHAPE;
  if (signs != nullptr)
    for (int j = 0; j < d; ++j)
      if (signs[j] != 1 && signs[j] != -1) return KVQ_ERR_ARG;

  kvq_codebooks cb;
  std::memset(&cb, 0, sizeof(cb));
  cb.d = d;
  cb.bits = bits;
  cb.elems_per_word = 32 / bits;
  // Any other head dimension is rotated zero-padded to the next power of two P (its codes
  // are those of all P rotated coordinates), so the tables are those of P.
  int p = 8;
  while (p < d) p *= 2;
  cb.n_words = (p + cb.elems_per_word - 1) / cb.elems_per_word;

  double g[8], l[8];
  lloyd_max_half(bits, false, g);
  lloyd_max_half(bits, true, l);
  cb.mse_g = gauss_distortion(bits, g);
  cb.sigma1 = 1.0 / std::sqrt(static_cast<double>(p));
  cb.sigma2 = std::sqrt(cb.mse_g) * cb.sigma1;
  fill_tables(bits, g, cb.sigma1, cb.c1, cb.b1);
  fill_tables(bits, l, cb.sigma2, cb.c2, cb.b2);
  if (signs != nullptr)
    for (int j = 0; j < d; ++j)
      if (signs[j] < 0) cb.sign_bits[j >> 5] |= 1u << (j & 31);
  *out = cb;
  return KVQ_OK;
}

extern "C" const char* kvq_status_str(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument (null pointer or inconsistent codebooks)";
    case KVQ_ERR_SHAPE: return "unsupported shape (d must be in [8,1024], bits in 1..4, sizes >= 0)";
    case KVQ_ERR_ALIGN: return "misaligned buffer (fp16 and packed-word buffers need 16-byte, norm buffers 4-byte alignment)";
    case KVQ_ERR_RANGE: return "out of range (s_offset + S exceeds S_cap, or a size overflows)";
    case KVQ_ERR_DEVICE: return "HIP launch failed";
  }
  return "unknown status";
}
