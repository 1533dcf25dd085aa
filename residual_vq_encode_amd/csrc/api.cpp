// C ABI entry points of libkvq: argument validation (host only, before any HIP call),
// per-call kernel constants derived from a kvq_codebooks struct, and the launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <limits>

#include "kvq.h"
#include "params.h"

namespace kvq {
hipError_t launch_encode(const EncodeArgs& a, int d, int bits, int stages, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int d, int bits, int stages, hipStream_t stream);
}  // namespace kvq

namespace {

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

kvq_status check_codebooks(const kvq_codebooks* cb) {
  if (cb == nullptr) return KVQ_ERR_ARG;
  if (cb->d < KVQ_MIN_D || cb->d > KVQ_MAX_D || !is_pow2(cb->d)) return KVQ_ERR_SHAPE;
  if (cb->bits < 1 || cb->bits > KVQ_MAX_BITS) return KVQ_ERR_SHAPE;
  const int epw = 32 / cb->bits;
  if (cb->elems_per_word != epw || cb->n_words != (cb->d + epw - 1) / epw) return KVQ_ERR_ARG;
  return KVQ_OK;
}

int sign_of(const kvq_codebooks* cb, int j) { return ((cb->sign_bits[j >> 5] >> (j & 31)) & 1u) ? -1 : 1; }

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

// Bucket table for the positive thresholds of one stage (bits >= 3). The bucket width is
// 0.9 of the smallest gap between consecutive thresholds (0 included), so every bucket
// [j, j+1) in table units holds at most one threshold; thresholds are the float32 values
// RN32(t_k * unit) and m_base(j) counts those below j, so m = m_base + [u > thr] counts
// every threshold below u exactly.
struct Buckets {
  double unit;               // table units per true unit
  int jmax;                  // last bucket; its entry has every threshold below it
  float thr[48];
  int32_t mbase[48];
};

bool make_buckets(const float* bnd, int bits, Buckets* bk, int max_entries) {
  const int half = 1 << (bits - 1);
  const int nt = half - 1;                 // positive thresholds b[half .. 2*half - 2]
  const float* t = bnd + half;
  double gap = t[0];
  for (int k = 1; k < nt; ++k) gap = std::fmin(gap, static_cast<double>(t[k]) - t[k - 1]);
  bk->unit = 1.0 / (0.9 * gap);
  float tf[8];
  for (int k = 0; k < nt; ++k) tf[k] = static_cast<float>(static_cast<double>(t[k]) * bk->unit);
  bk->jmax = static_cast<int>(std::floor(tf[nt - 1])) + 1;
  if (bk->jmax + 1 > max_entries) return false;
  for (int j = 0; j <= bk->jmax; ++j) {
    int below = 0;
    float inside = std::numeric_limits<float>::max();
    for (int k = 0; k < nt; ++k) {
      if (tf[k] < static_cast<float>(j)) ++below;
      else if (tf[k] < static_cast<float>(j + 1)) inside = tf[k];
    }
    bk->thr[j] = inside;
    bk->mbase[j] = below;
  }
  return true;
}

float as_float(int32_t v) {
  float f;
  std::memcpy(&f, &v, sizeof(f));
  return f;
}

kvq_status fill_encode_args(const kvq_codebooks* cb, EncodeArgs* a) {
  const int d = cb->d, bits = cb->bits, k = 1 << bits, half = k / 2;
  const double inv_sqrt_d = 1.0 / std::sqrt(static_cast<double>(d));
  std::memset(a->xmask, 0, sizeof(a->xmask));
  std::memset(a->tab1, 0, sizeof(a->tab1));
  std::memset(a->tab2, 0, sizeof(a->tab2));
  a->j1max = a->j2max = 0;
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
    if (!make_buckets(cb->b1, bits, &b1, kvq::kTab1Max) || !make_buckets(cb->b2, bits, &b2, kvq::kTab2Max))
      return KVQ_ERR_ARG;
    a->k_scale = static_cast<float>(b1.unit * inv_sqrt_d);
    a->r12 = static_cast<float>(b2.unit / b1.unit);
    a->j1max = b1.jmax;
    a->j2max = b2.jmax;
    for (int j = 0; j <= b1.jmax; ++j) {
      const int m = b1.mbase[j];
      const bool has = b1.thr[j] != std::numeric_limits<float>::max();
      a->tab1[j][0] = b1.thr[j];
      a->tab1[j][1] = as_float(m);
      a->tab1[j][2] = static_cast<float>(cb->c1[half + m] * b2.unit);
      a->tab1[j][3] = static_cast<float>(cb->c1[half + (has ? m + 1 : m)] * b2.unit);
    }
    for (int j = 0; j <= b2.jmax; ++j) {
      a->tab2[j][0] = b2.thr[j];
      a->tab2[j][1] = as_float(b2.mbase[j]);
    }
  }
  for (int m = 0; m < d / 2; ++m)
    a->xmask[m] = (sign_of(cb, 2 * m) < 0 ? 0x8000u : 0u) | (sign_of(cb, 2 * m + 1) < 0 ? 0x80000000u : 0u);
  return KVQ_OK;
}

// stages = 2: entry (i1 << bits) | i2 is c1[i1] + c2[i2]; stages = 1: entry i1 << bits is c1[i1].
void fill_decode_args(const kvq_codebooks* cb, int stages, DecodeArgs* a) {
  const int d = cb->d, bits = cb->bits, k = 1 << bits;
  a->inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
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
  int64_t n_vec = 0;
  st = check_sizes(cb, B, H, S, S_cap, s_offset, &n_vec);
  if (st != KVQ_OK) return st;
  if (n_vec == 0) return KVQ_OK;
  if (x == nullptr || packed1 == nullptr || (stages == 2 && packed2 == nullptr) || norms == nullptr)
    return KVQ_ERR_ARG;
  if (!aligned(x, 16) || !aligned(packed1, 16) || (stages == 2 && !aligned(packed2, 16)) || !aligned(norms, 4))
    return KVQ_ERR_ALIGN;

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
