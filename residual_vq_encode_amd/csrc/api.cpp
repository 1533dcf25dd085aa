// C ABI entry points of libkvq: argument validation (host only, before any HIP call),
// per-call kernel constants derived from a kvq_codebooks struct, and the launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <limits>

#include "kvq.h"
#include "params.h"
#include "qjl_params.h"

namespace kvq {
hipError_t launch_encode(const EncodeArgs& a, int d, int bits, int stages, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, int bits, int stages, hipStream_t stream);
hipError_t launch_attend(const AttendArgs& a, int d, int bits, int nqw, hipStream_t stream);
hipError_t launch_qjl(const QjlArgs& a, int d, int m, hipStream_t stream);
hipError_t attend_scratch(void** ptr);
}  // namespace kvq

static_assert(kvq::kAttendScratchBytes == KVQ_ATTEND_SCRATCH_BYTES, "the header states the scratch size");

namespace {

using kvq::AttendArgs;
using kvq::DecodeArgs;
using kvq::EncodeArgs;
using kvq::RowMap;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// a * b without overflow (both >= 0); false on overflow.
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *out = a * b;
  return true;
}

// One stage's tables as the kernels rely on them: 2^bits finite centroids, strictly
// ascending and exactly antisymmetric (c[k] == -c[L-1-k]), and boundaries that are the
// float32 roundings of the midpoints of neighbouring centroids, computed in double ("rvq" tag
// page, "What 'quantize' means here, precisely": counting boundary crossings picks the
// nearest centroid only when the boundaries are those midpoints). Antisymmetry then makes
// the middle boundary +0.0, which the kernels' sign-bit quantizers (bits <= 2) assume, and
// the 3- and 4-bit bucket tables are derived from these boundaries.
bool stage_tables_ok(const float* c, const float* b, int bits) {
  const int L = 1 << bits;
  for (int k = 0; k < L; ++k) {
    if (!std::isfinite(c[k]) || c[k] != -c[L - 1 - k]) return false;
    if (k + 1 < L && !(c[k] < c[k + 1])) return false;
  }
  for (int k = 0; k + 1 < L; ++k) {
    const float mid = static_cast<float>((static_cast<double>(c[k]) + static_cast<double>(c[k + 1])) * 0.5);
    uint32_t got, want;
    std::memcpy(&got, &b[k], 4);
    std::memcpy(&want, &mid, 4);
    if (got != want) return false;  // bit equality: the middle boundary must be +0.0, not -0.0
  }
  return true;
}

kvq_status check_codebooks(const kvq_codebooks* cb) {
  if (cb == nullptr) return KVQ_ERR_ARG;
  if (cb->d < KVQ_MIN_D || cb->d > KVQ_MAX_D) return KVQ_ERR_SHAPE;
  if (cb->bits < 1 || cb->bits > KVQ_MAX_BITS) return KVQ_ERR_SHAPE;
  const int epw = 32 / cb->bits, p = kvq::rotation_length(cb->d);
  if (cb->elems_per_word != epw || cb->n_words != (p + epw - 1) / epw) return KVQ_ERR_ARG;
  if (!stage_tables_ok(cb->c1, cb->b1, cb->bits) || !stage_tables_ok(cb->c2, cb->b2, cb->bits)) return KVQ_ERR_ARG;
  return KVQ_OK;
}

// The codec kernels walk their tiles with 32-bit indices: a launch may hold at most INT_MAX.
kvq_status check_tiles(int64_t n_vec, int64_t vectors_per_tile) {
  return (n_vec + vectors_per_tile - 1) / vectors_per_tile > std::numeric_limits<int32_t>::max() ? KVQ_ERR_RANGE
                                                                                                 : KVQ_OK;
}

// Sign of rotated coordinate j; the padding coordinates (j >= d) take +1.
int sign_of(const kvq_codebooks* cb, int j) {
  return j < cb->d && ((cb->sign_bits[j >> 5] >> (j & 31)) & 1u) ? -1 : 1;
}

// Validates the shared shape/range arguments; on success returns the vector count.
kvq_status check_sizes(const kvq_codebooks* cb, int64_t B, int64_t H, int64_t S, int64_t S_cap,
                       int64_t s_offset, int64_t* n_vec) {
  if (B < 0 || H < 0 || S < 0) return KVQ_ERR_SHAPE;
  if (S_cap < 0 || s_offset < 0 || s_offset > S_cap || S > S_cap - s_offset) return KVQ_ERR_RANGE;
  int64_t bh, n, rows, words, elems, bytes;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, S, &n) || !mul_ok(bh, S_cap, &rows) ||
      !mul_ok(rows, cb->n_words, &words) || !mul_ok(words, 4, &bytes) ||
      !mul_ok(n, cb->d, &elems) || !mul_ok(elems, 2, &bytes))
    return KVQ_ERR_RANGE;
  *n_vec = n;
  return KVQ_OK;
}

RowMap row_map(int64_t S, int64_t S_cap, int64_t s_offset) {
  RowMap m;
  m.S = S > 0 ? S : 1;
  m.S_cap = S_cap;
  m.s_offset = s_offset;
  m.inv_S = 1.0f / static_cast<float>(m.S);
  m.contiguous = (S == S_cap && s_offset == 0) ? 1 : 0;
  return m;
}

// Bucket table of one stage (bits >= 3). The kernel scales a value t (true units) to the
// float32 w = t / (2R), compares it in that form, and reads entry
// j = RNE(v * sub * kTabBuckets) / sub of v = clamp(RN32(w + 1/2), 0, 1) (see kTabBuckets).
// Every v that reaches entry j lies in [(sub j - 1/2), (sub j + sub - 1/2)] / (sub * kTabBuckets)
// (ties either way), so every w that does lies in that interval shifted by -1/2 and widened
// by the rounding of w + 1/2 (at most 2^-24; 2^-23 is allowed), or beyond the end of [-1/2,
// 1/2] for the two end entries. With the thresholds as float32 values tw_k = RN32(b_k / (2R)),
// base_j counts those below the widened interval and thr_j is the one inside it (+inf if
// none), so that
// base_j + [w > thr_j] = #{k : w > tw_k}, the count of boundaries the value exceeds taken in
// float32 on w. Fails if a bucket would hold two thresholds or they are not increasing.
struct Buckets {
  double two_r;  // 2R: true units per unit of w
  float thr[kvq::kTabEntries];
  int32_t base[kvq::kTabEntries];
};

bool make_buckets(const float* bnd, int bits, int sub, double inv_sqrt_d, Buckets* bk) {
  const int nt = (1 << bits) - 1;
  double tmax = 0.0;
  for (int k = 0; k < nt; ++k) {
    if (!std::isfinite(bnd[k]) || (k > 0 && !(bnd[k] > bnd[k - 1]))) return false;
    tmax = std::fmax(tmax, std::fabs(static_cast<double>(bnd[k])));
  }
  if (!(tmax > 0.0)) return false;
  // thresholds land in about [-0.45, 0.45]; 2R is adjusted so that the kernel's scale
  // 1 / (sqrt(d) 2R) is a float32 value exactly (one rounding less in every decision)
  bk->two_r = inv_sqrt_d / static_cast<double>(static_cast<float>(inv_sqrt_d / (2.25 * tmax)));
  float tw[15];
  for (int k = 0; k < nt; ++k) tw[k] = static_cast<float>(static_cast<double>(bnd[k]) / bk->two_r);
  const double step = 1.0 / (static_cast<double>(sub) * kvq::kTabBuckets), slack = std::ldexp(1.0, -23);
  for (int j = 0; j < kvq::kTabEntries; ++j) {
    const double lo = (sub * j - 0.5) * step - 0.5 - slack, hi = (sub * j + sub - 0.5) * step - 0.5 + slack;
    int below = 0, inside = 0;
    float thr = std::numeric_limits<float>::infinity();
    for (int k = 0; k < nt; ++k) {
      if (static_cast<double>(tw[k]) < lo) {
        ++below;
      } else if (static_cast<double>(tw[k]) <= hi) {
        ++inside;
        thr = tw[k];
      }
    }
    if (inside > 1) return false;
    bk->thr[j] = thr;
    bk->base[j] = below;
  }
  return true;
}

float as_float(int32_t v) {
  float f;
  std::memcpy(&f, &v, sizeof(f));
  return f;
}

kvq_status fill_encode_args(const kvq_codebooks* cb, EncodeArgs* a) {
  const int d = kvq::rotation_length(cb->d), bits = cb->bits;  // the rotation's length
  const double inv_sqrt_d = 1.0 / std::sqrt(static_cast<double>(d));
  a->dh = cb->d;
  std::memset(a->wpair, 0, sizeof(a->wpair));
  std::memset(a->tab1, 0, sizeof(a->tab1));
  std::memset(a->tab2, 0, sizeof(a->tab2));
  a->k2_scale = 0.f;
  a->cm2[0] = a->cm2[1] = 0.f;
  if (bits == 1) {
    a->k_scale = static_cast<float>(inv_sqrt_d);  // NX = -y_true
    a->r12 = 1.f;
    a->cm2[0] = cb->c1[1];
  } else if (bits == 2) {
    const double T1 = cb->b1[2], T2 = cb->b2[2];
    a->k_scale = static_cast<float>((2.0 / T1) * inv_sqrt_d);
    a->r12 = static_cast<float>(T1 / T2);
    a->cm2[0] = static_cast<float>((static_cast<double>(cb->c1[3]) - cb->c1[2]) / T2);  // h in units 2/T2
  } else {
    Buckets b1, b2;
    if (!make_buckets(cb->b1, bits, 16, inv_sqrt_d, &b1) || !make_buckets(cb->b2, bits, 8, inv_sqrt_d, &b2))
      return KVQ_ERR_ARG;
    a->k_scale = static_cast<float>(inv_sqrt_d / b1.two_r);
    a->k2_scale = static_cast<float>(inv_sqrt_d / b2.two_r);
    a->r12 = 0.f;
    // stage 2 compares w2 = y_true / (2 R2) + (-c1[m] / (2 R2)) for stage-1 code m
    auto offset2 = [&](int m) { return static_cast<float>(-static_cast<double>(cb->c1[m]) / b2.two_r); };
    for (int j = 0; j < kvq::kTabEntries; ++j) {
      const int m = b1.base[j];
      const bool has = b1.thr[j] != std::numeric_limits<float>::infinity();
      a->tab1[j][0] = b1.thr[j];
      a->tab1[j][1] = as_float(m);
      a->tab1[j][2] = offset2(m);
      a->tab1[j][3] = offset2(has ? m + 1 : m);
      a->tab2[j][0] = b2.thr[j];
      a->tab2[j][1] = as_float(b2.base[j]);
    }
  }
  for (int m = 0; m < d / 2; ++m)
    a->wpair[m] =
        kvq::kOnePair ^ ((sign_of(cb, 2 * m) < 0 ? 0x8000u : 0u) | (sign_of(cb, 2 * m + 1) < 0 ? 0x80000000u : 0u));
  return KVQ_OK;
}

// stages = 2: entry (i1 << bits) | i2 is c1[i1] + c2[i2]; stages = 1: entry i1 << bits is c1[i1].
void fill_decode_args(const kvq_codebooks* cb, int stages, DecodeArgs* a) {
  const int d = kvq::rotation_length(cb->d), bits = cb->bits, k = 1 << bits;  // the rotation's length
  a->inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
  a->dh = cb->d;
  std::memset(a->ztab, 0, sizeof(a->ztab));
  for (int i1 = 0; i1 < k; ++i1) {
    if (stages == 1) {
      a->ztab[i1 << bits] = cb->c1[i1];
    } else {
      for (int i2 = 0; i2 < k; ++i2) a->ztab[(i1 << bits) | i2] = cb->c1[i1] + cb->c2[i2];  // one float32 add
    }
  }
  std::memset(a->xmask, 0, sizeof(a->xmask));
  for (int m = 0; m < d / 2; ++m)
    a->xmask[m] = (sign_of(cb, 2 * m) < 0 ? 0x8000u : 0u) | (sign_of(cb, 2 * m + 1) < 0 ? 0x80000000u : 0u);
}

kvq_status encode_pack(const kvq_codebooks* cb, int stages, const uint16_t* x, int64_t B, int64_t H, int64_t S,
                       uint32_t* packed1, uint32_t* packed2, float* norms, int64_t S_cap, int64_t s_offset,
                       void* stream) {
  kvq_status st = check_codebooks(cb);
  if (st != KVQ_OK) return st;
  if (stages == 0 && (cb->bits != 1 || !is_pow2(cb->d))) return KVQ_ERR_SHAPE;
  int64_t n_vec = 0;
  st = check_sizes(cb, B, H, S, S_cap, s_offset, &n_vec);
  if (st != KVQ_OK) return st;
  if (n_vec == 0) return KVQ_OK;
  if (x == nullptr || packed1 == nullptr || (stages == 2 && packed2 == nullptr) || norms == nullptr)
    return KVQ_ERR_ARG;
  if (!aligned(x, 16) || !aligned(packed1, 16) || (stages == 2 && !aligned(packed2, 16)) || !aligned(norms, 4))
    return KVQ_ERR_ALIGN;
  st = check_tiles(n_vec, kvq::encode_tile_vectors(cb->d, cb->bits));
  if (st != KVQ_OK) return st;

  EncodeArgs a;
  a.x = x;
  a.p1 = packed1;
  a.p2 = stages == 2 ? packed2 : nullptr;
  a.norms = norms;
  a.n_vec = n_vec;
  a.map = row_map(S, S_cap, s_offset);
  st = fill_encode_args(cb, &a);
  if (st != KVQ_OK) return st;
  const hipError_t e = kvq::launch_encode(a, cb->d, cb->bits, stages, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

kvq_status unpack_decode(const kvq_codebooks* cb, int stages, const uint32_t* packed1, const uint32_t* packed2,
                         const float* norms, int64_t B, int64_t H, int64_t S_cap, int64_t s_offset, int64_t S,
                         uint16_t* x_out, void* stream) {
  kvq_status st = check_codebooks(cb);
  if (st != KVQ_OK) return st;
  int64_t n_vec = 0;
  st = check_sizes(cb, B, H, S, S_cap, s_offset, &n_vec);
  if (st != KVQ_OK) return st;
  if (n_vec == 0) return KVQ_OK;
  if (packed1 == nullptr || (stages == 2 && packed2 == nullptr) || x_out == nullptr) return KVQ_ERR_ARG;
  if (!aligned(x_out, 16) || !aligned(packed1, 16) || (stages == 2 && !aligned(packed2, 16)) || !aligned(norms, 4))
    return KVQ_ERR_ALIGN;
  st = check_tiles(n_vec, kvq::decode_tile_vectors(cb->d));
  if (st != KVQ_OK) return st;

  DecodeArgs a;
  a.p1 = packed1;
  a.p2 = stages == 2 ? packed2 : nullptr;
  a.norms = norms;
  a.x = x_out;
  a.n_vec = n_vec;
  a.map = row_map(S, S_cap, s_offset);
  fill_decode_args(cb, stages, &a);
  const hipError_t e = kvq::launch_decode(a, cb->d, cb->bits, stages, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

}  // namespace

extern "C" kvq_status kvq_rvq_encode_pack(const kvq_codebooks* cb, const uint16_t* x, int64_t B, int64_t H,
                                          int64_t S, uint32_t* packed1, uint32_t* packed2, float* norms,
                                          int64_t S_cap, int64_t s_offset, void* stream) {
  return encode_pack(cb, 2, x, B, H, S, packed1, packed2, norms, S_cap, s_offset, stream);
}

extern "C" kvq_status kvq_rvq_unpack_decode(const kvq_codebooks* cb, const uint32_t* packed1,
                                            const uint32_t* packed2, const float* norms, int64_t B, int64_t H,
                                            int64_t S_cap, int64_t s_offset, int64_t S, uint16_t* x_out,
                                            void* stream) {
  return unpack_decode(cb, 2, packed1, packed2, norms, B, H, S_cap, s_offset, S, x_out, stream);
}

extern "C" kvq_status kvq_mse_encode_pack(const kvq_codebooks* cb, const uint16_t* x, int64_t B, int64_t H,
                                          int64_t S, uint32_t* packed, float* norms, int64_t S_cap,
                                          int64_t s_offset, void* stream) {
  return encode_pack(cb, 1, x, B, H, S, packed, nullptr, norms, S_cap, s_offset, stream);
}

extern "C" kvq_status kvq_mse_unpack_decode(const kvq_codebooks* cb, const uint32_t* packed, const float* norms,
                                            int64_t B, int64_t H, int64_t S_cap, int64_t s_offset, int64_t S,
                                            uint16_t* x_out, void* stream) {
  return unpack_decode(cb, 1, packed, nullptr, norms, B, H, S_cap, s_offset, S, x_out, stream);
}

extern "C" kvq_status kvq_rabitq_encode_pack(const kvq_codebooks* cb, const uint16_t* x, int64_t B, int64_t H,
                                             int64_t S, uint32_t* packed, float* norms, int64_t S_cap,
                                             int64_t s_offset, void* stream) {
  return encode_pack(cb, 0, x, B, H, S, packed, nullptr, norms, S_cap, s_offset, stream);
}

// ------------------------------------------------------------------------------ QJL sketch

extern "C" kvq_status kvq_qjl_supported(int32_t d, int32_t m) {
  if (d != 32 && d != 64 && d != 128 && d != 256) return KVQ_ERR_SHAPE;
  if (m < 32 || m > 256 || m % 32 != 0) return KVQ_ERR_SHAPE;
  if (kvq::qjl_lds_need(d, m) > kvq::kQjlLdsMax) return KVQ_ERR_SHAPE;
  return KVQ_OK;
}

extern "C" kvq_status kvq_qjl_encode_pack(const uint16_t* sketch, int32_t d, int32_t m, const uint16_t* x,
                                          int64_t B, int64_t H, int64_t S, uint32_t* packed, uint16_t* norms,
                                          int64_t S_cap, int64_t s_offset, void* stream) {
  kvq_status st = kvq_qjl_supported(d, m);
  if (st != KVQ_OK) return st;
  if (B < 0 || H < 0 || S < 0) return KVQ_ERR_SHAPE;
  if (S_cap < 0 || s_offset < 0 || s_offset > S_cap || S > S_cap - s_offset) return KVQ_ERR_RANGE;
  int64_t bh, n_vec, rows, words, elems, bytes;
  if (!mul_ok(B, H, &bh) || !mul_ok(bh, S, &n_vec) || !mul_ok(bh, S_cap, &rows) || !mul_ok(rows, m / 32, &words) ||
      !mul_ok(words, 4, &bytes) || !mul_ok(n_vec, d, &elems) || !mul_ok(elems, 2, &bytes))
    return KVQ_ERR_RANGE;
  if ((n_vec + 31) / 32 > std::numeric_limits<int32_t>::max() / 2) return KVQ_ERR_RANGE;
  if (n_vec == 0) return KVQ_OK;
  if (sketch == nullptr || x == nullptr || packed == nullptr || norms == nullptr) return KVQ_ERR_ARG;
  if (!aligned(sketch, 16) || !aligned(x, 16) || !aligned(packed, 16) || !aligned(norms, 2)) return KVQ_ERR_ALIGN;
  kvq::QjlArgs a;
  a.x = x;
  a.sketch = sketch;
  a.packed = packed;
  a.norms = norms;
  a.n_vec = n_vec;
  a.map = row_map(S, S_cap, s_offset);
  const hipError_t e = kvq::launch_qjl(a, d, m, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

// ------------------------------------------------------------------------------ attention

namespace {

// How the attention splits its work. With d = 64 or 128 and b = 1, 2 or 4 (d b >= 128) the
// partial pass runs on the matrix cores: a wave serves 16 query vectors of one key/value
// head (nqw = 16; the query vectors of a head are cut into groups of 16, the last one
// padded) and takes 32 cached positions per iteration. Otherwise a wave serves nqw query
// vectors of a head (the largest of 4, 2, 1 that divides the query vectors per head; 1 at
// d = 1024, where their state does not fit the registers) and a multiple of the lane
// layout's positions per iteration. The cached positions are cut into chunks of whole
// iterations, enough of them that the partial pass has about 2048 waves (several per SIMD;
// longer chunks amortise each wave's query rotation and its final merge, and leave fewer
// partial results to combine), at least 4 (matrix path) or 8 iterations per chunk, and at
// most 4096 chunks.
constexpr int64_t kMaxAttendSplits = 4096;  // chunks per query vector the combine kernel takes

struct AttendPlan {
  int64_t n_q = 0;
  int32_t chunk = 0, n_splits = 0, nqw = 1;
  int64_t ws_bytes = 0;
};

bool attend_on_matrix_cores(int32_t d, int32_t bits) {
  return (d == 64 || d == 128) && bits != 3 && d * bits >= 128;
}

kvq_status attend_plan(int32_t d, int32_t bits, int64_t B, int64_t Hq, int64_t Sq, int64_t Hkv, int64_t S_kv,
                       AttendPlan* p) {
  if (d < KVQ_MIN_D || d > KVQ_MAX_D || !is_pow2(d)) return KVQ_ERR_SHAPE;
  if (bits < 1 || bits > KVQ_MAX_BITS) return KVQ_ERR_SHAPE;
  if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 0) return KVQ_ERR_SHAPE;
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return KVQ_ERR_SHAPE;
  if (S_kv < 1 || S_kv > (int64_t(1) << 40)) return KVQ_ERR_RANGE;
  int64_t bh = 0, n_q = 0, gq = 0;
  if (!mul_ok(B, Hq, &bh) || !mul_ok(bh, Sq, &n_q)) return KVQ_ERR_RANGE;
  if (Hq > 0 && !mul_ok(Hq / Hkv, Sq, &gq)) return KVQ_ERR_RANGE;
  const bool mat = attend_on_matrix_cores(d, bits);
  int nqw = 1;
  int64_t vw = 0, min_iters = 8, waves_per_split = 0;  // positions per iteration
  if (mat) {
    nqw = 16;
    vw = 32;
    min_iters = 4;
    waves_per_split = gq > 0 ? (n_q / gq) * ((gq + 15) / 16) : 0;
  } else {
    if (d <= 512) nqw = gq % 4 == 0 ? 4 : gq % 2 == 0 ? 2 : 1;
    const int64_t cm = (nqw > 1 && d >= 32) ? 16 : 32;  // coordinates per lane
    const int64_t c = d < cm ? d : cm;
    vw = 64 / (d / c);
    waves_per_split = n_q / nqw;
  }
  const int64_t want_waves = 2048;
  const int64_t splits0 = waves_per_split > 0 ? (want_waves + waves_per_split - 1) / waves_per_split : 1;
  int64_t chunk = (S_kv + splits0 - 1) / splits0;
  chunk = (chunk + vw - 1) / vw * vw;
  if (chunk < min_iters * vw) chunk = min_iters * vw;
  const int64_t min_chunk = (S_kv + kMaxAttendSplits - 1) / kMaxAttendSplits;  // the combine's limit
  if (chunk < min_chunk) chunk = (min_chunk + vw - 1) / vw * vw;
  if (chunk > (int64_t(1) << 30)) chunk = int64_t(1) << 30;
  const int64_t n_splits = (S_kv + chunk - 1) / chunk;
  int64_t units = 0, ws = 0, waves = 0;
  if (!mul_ok(n_q, n_splits, &units) || !mul_ok(units, (d + 4) * 4, &ws) ||
      !mul_ok(waves_per_split, n_splits, &waves))
    return KVQ_ERR_RANGE;
  if (waves / kvq::kWavesPerBlock > std::numeric_limits<int32_t>::max() ||
      n_q > std::numeric_limits<int32_t>::max() / 16)  // combine blocks: n_q * (d / 64)
    return KVQ_ERR_RANGE;
  p->n_q = n_q;
  p->chunk = static_cast<int32_t>(chunk);
  p->n_splits = static_cast<int32_t>(n_splits);
  p->nqw = nqw;
  p->ws_bytes = ws;
  return KVQ_OK;
}

}  // namespace

extern "C" kvq_status kvq_rvq_attend_workspace_size(int32_t d, int32_t bits, int64_t B, int64_t Hq, int64_t Sq,
                                                    int64_t Hkv, int64_t S_kv, int64_t* bytes) {
  if (bytes == nullptr) return KVQ_ERR_ARG;
  AttendPlan p;
  const kvq_status st = attend_plan(d, bits, B, Hq, Sq, Hkv, S_kv, &p);
  if (st != KVQ_OK) return st;
  *bytes = p.ws_bytes;
  return KVQ_OK;
}

namespace {

// The attention's checks and launch. With use_scratch the partial records go to the
// library's device scratch (looked up after every host check has passed, so a rejected
// call still touches no device state) and workspace / workspace_bytes are ignored.
kvq_status attend(const kvq_codebooks* cbk, const kvq_codebooks* cbv, const uint16_t* q, int64_t B, int64_t Hq,
                  int64_t Sq, int64_t Hkv, const uint32_t* k_packed1, const uint32_t* k_packed2, const float* k_norms,
                  const uint32_t* v_packed1, const uint32_t* v_packed2, const float* v_norms, int64_t S_cap,
                  int64_t S_kv, float scale, void* workspace, int64_t workspace_bytes, bool use_scratch, uint16_t* out,
                  void* stream) {
  kvq_status st = check_codebooks(cbk);
  if (st != KVQ_OK) return st;
  st = check_codebooks(cbv);
  if (st != KVQ_OK) return st;
  if (cbk->d != cbv->d || cbk->bits != cbv->bits) return KVQ_ERR_SHAPE;
  if (B < 0 || Hq < 0 || Sq < 0 || Hkv < 0) return KVQ_ERR_SHAPE;
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return KVQ_ERR_SHAPE;
  if (Hkv > std::numeric_limits<int32_t>::max() || Sq > std::numeric_limits<int32_t>::max() ||
      (Hkv > 0 && Hq / Hkv > std::numeric_limits<int32_t>::max()))
    return KVQ_ERR_RANGE;
  if (S_kv < 1 || S_cap < S_kv) return KVQ_ERR_RANGE;
  AttendPlan p;
  st = attend_plan(cbk->d, cbk->bits, B, Hq, Sq, Hkv, S_kv, &p);
  if (st != KVQ_OK) return st;
  // the caches: [B, Hkv, S_cap, n_words] words and [B, Hkv, S_cap] norms must be addressable
  int64_t rows = 0, words = 0, bytes = 0;
  if (!mul_ok(B, Hkv, &rows) || !mul_ok(rows, S_cap, &rows) || !mul_ok(rows, cbk->n_words, &words) ||
      !mul_ok(words, 4, &bytes))
    return KVQ_ERR_RANGE;
  if (p.n_q == 0) return KVQ_OK;
  if (!std::isfinite(scale)) return KVQ_ERR_ARG;
  if (q == nullptr || k_packed1 == nullptr || k_packed2 == nullptr || k_norms == nullptr || v_packed1 == nullptr ||
      v_packed2 == nullptr || v_norms == nullptr || (!use_scratch && workspace == nullptr) || out == nullptr)
    return KVQ_ERR_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || (!use_scratch && !aligned(workspace, 16)) || !aligned(k_packed1, 16) ||
      !aligned(k_packed2, 16) || !aligned(v_packed1, 16) || !aligned(v_packed2, 16) || !aligned(k_norms, 4) ||
      !aligned(v_norms, 4))
    return KVQ_ERR_ALIGN;
  if (use_scratch) {
    if (p.ws_bytes > kvq::kAttendScratchBytes) return KVQ_ERR_RANGE;
    if (kvq::attend_scratch(&workspace) != hipSuccess) return KVQ_ERR_DEVICE;
  } else if (workspace_bytes < p.ws_bytes) {
    return KVQ_ERR_RANGE;
  }

  AttendArgs a;
  a.q = q;
  a.k1 = k_packed1;
  a.k2 = k_packed2;
  a.kn = k_norms;
  a.v1 = v_packed1;
  a.v2 = v_packed2;
  a.vn = v_norms;
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.n_q = p.n_q;
  a.S_cap = S_cap;
  a.S_kv = S_kv;
  a.Hkv = static_cast<int32_t>(Hkv);
  a.group = static_cast<int32_t>(Hq / Hkv);
  a.Sq = static_cast<int32_t>(Sq);
  a.chunk = p.chunk;
  a.n_splits = p.n_splits;
  const double inv_sqrt_d = 1.0 / std::sqrt(static_cast<double>(cbk->d));
  a.qscale = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634 * inv_sqrt_d);  // log2(e)
  a.inv_sqrt_d = static_cast<float>(inv_sqrt_d);
  const int k = 1 << cbk->bits;
  std::memset(a.ztab_k, 0, sizeof(a.ztab_k));
  std::memset(a.ztab_v, 0, sizeof(a.ztab_v));
  for (int i1 = 0; i1 < k; ++i1)
    for (int i2 = 0; i2 < k; ++i2) {
      a.ztab_k[(i1 << cbk->bits) | i2] = cbk->c1[i1] + cbk->c2[i2];  // one float32 add
      a.ztab_v[(i1 << cbv->bits) | i2] = cbv->c1[i1] + cbv->c2[i2];
    }
  std::memcpy(a.ksign, cbk->sign_bits, sizeof(a.ksign));
  std::memcpy(a.vsign, cbv->sign_bits, sizeof(a.vsign));
  const hipError_t e = kvq::launch_attend(a, cbk->d, cbk->bits, p.nqw, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_DEVICE;
}

}  // namespace

extern "C" kvq_status kvq_rvq_attend(const kvq_codebooks* cbk, const kvq_codebooks* cbv, const uint16_t* q,
                                     int64_t B, int64_t Hq, int64_t Sq, int64_t Hkv, const uint32_t* k_packed1,
                                     const uint32_t* k_packed2, const float* k_norms, const uint32_t* v_packed1,
                                     const uint32_t* v_packed2, const float* v_norms, int64_t S_cap, int64_t S_kv,
                                     float scale, void* workspace, int64_t workspace_bytes, uint16_t* out,
                                     void* stream) {
  return attend(cbk, cbv, q, B, Hq, Sq, Hkv, k_packed1, k_packed2, k_norms, v_packed1, v_packed2, v_norms, S_cap, S_kv,
                scale, workspace, workspace_bytes, false, out, stream);
}

extern "C" kvq_status kvq_rvq_attend_noalloc(const kvq_codebooks* cbk, const kvq_codebooks* cbv, const uint16_t* q,
                                             int64_t B, int64_t Hq, int64_t Sq, int64_t Hkv,
                                             const uint32_t* k_packed1, const uint32_t* k_packed2,
                                             const float* k_norms, const uint32_t* v_packed1,
                                             const uint32_t* v_packed2, const float* v_norms, int64_t S_cap,
                                             int64_t S_kv, float scale, uint16_t* out, void* stream) {
  return attend(cbk, cbv, q, B, Hq, Sq, Hkv, k_packed1, k_packed2, k_norms, v_packed1, v_packed2, v_norms, S_cap, S_kv,
                scale, nullptr, 0, true, out, stream);
}
