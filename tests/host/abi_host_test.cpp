// Host-only test of libkvq's C ABI, built with AddressSanitizer and UBSan against the launch
// stubs of launch_stubs.cpp (no GPU, nothing launched): codebook construction for every
// supported (d, bits), every argument check of every entry point, the argument blocks the
// checks hand to the launchers, and the attention plan. Device pointers are fake, aligned
// addresses; the stubs never dereference them. Prints "ok" and exits 0 when every check
// holds.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "kvq.h"
#include "launch_stubs.h"

namespace {

int g_fail = 0;

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

template <typename T>
T* fake(uintptr_t addr) {
  return reinterpret_cast<T*>(addr);
}

// ------------------------------------------------------------------------------ codebooks

void test_codebooks() {
  kvq_codebooks cb;
  for (int d = 8; d <= 1024; d *= 2) {
    std::vector<int8_t> neg(d, -1);
    for (int bits = 1; bits <= 4; ++bits) {
      CHECK(kvq_build_codebooks(d, bits, nullptr, &cb) == KVQ_OK);
      const int L = 1 << bits, epw = 32 / bits;
      CHECK(cb.d == d && cb.bits == bits && cb.elems_per_word == epw);
      CHECK(cb.n_words == (d + epw - 1) / epw);
      for (int k = 0; k < L; ++k) {
        CHECK(cb.c1[k] == -cb.c1[L - 1 - k]);  // exactly antisymmetric
        CHECK(cb.c2[k] == -cb.c2[L - 1 - k]);
      }
      for (int k = 0; k + 1 < L; ++k) {
        CHECK(cb.c1[k] < cb.c1[k + 1] && cb.c2[k] < cb.c2[k + 1]);
        CHECK(cb.c1[k] < cb.b1[k] && cb.b1[k] < cb.c1[k + 1]);
        CHECK(cb.c2[k] < cb.b2[k] && cb.b2[k] < cb.c2[k + 1]);
      }
      uint32_t mid;  // the middle boundary is +0 (sign bit clear)
      std::memcpy(&mid, &cb.b1[L / 2 - 1], 4);
      CHECK(mid == 0u);
      std::memcpy(&mid, &cb.b2[L / 2 - 1], 4);
      CHECK(mid == 0u);
      CHECK(std::fabs(cb.sigma1 - 1.0 / std::sqrt(static_cast<double>(d))) < 1e-15);
      for (int w = 0; w < KVQ_MAX_D / 32; ++w) CHECK(cb.sign_bits[w] == 0u);
      CHECK(kvq_build_codebooks(d, bits, neg.data(), &cb) == KVQ_OK);
      for (int j = 0; j < KVQ_MAX_D; ++j) CHECK(((cb.sign_bits[j >> 5] >> (j & 31)) & 1u) == (j < d ? 1u : 0u));
    }
    neg[d - 1] = 0;  // not a sign
    CHECK(kvq_build_codebooks(d, 2, neg.data(), &cb) == KVQ_ERR_ARG);
  }
  // a head dimension that is not a power of two: the tables, word count and sigma1 are those
  // of its rotation length P (the next power of two), the signs its own
  for (int d : {9, 13, 24, 40, 72, 96, 100, 200, 576, 1016, 1023}) {
    int p = 8;
    while (p < d) p *= 2;
    std::vector<int8_t> neg(d, -1);
    for (int bits = 1; bits <= 4; ++bits) {
      kvq_codebooks cp;
      CHECK(kvq_build_codebooks(d, bits, neg.data(), &cb) == KVQ_OK);
      CHECK(kvq_build_codebooks(p, bits, nullptr, &cp) == KVQ_OK);
      const int epw = 32 / bits;
      CHECK(cb.d == d && cb.n_words == (p + epw - 1) / epw && cb.n_words == cp.n_words);
      CHECK(cb.sigma1 == cp.sigma1 && cb.sigma2 == cp.sigma2);
      CHECK(std::memcmp(cb.c1, cp.c1, sizeof(cb.c1)) == 0 && std::memcmp(cb.b2, cp.b2, sizeof(cb.b2)) == 0);
      for (int j = 0; j < KVQ_MAX_D; ++j) CHECK(((cb.sign_bits[j >> 5] >> (j & 31)) & 1u) == (j < d ? 1u : 0u));
    }
  }
  CHECK(kvq_build_codebooks(128, 2, nullptr, nullptr) == KVQ_ERR_ARG);
  for (int d : {-8, 0, 4, 7, 1025, 1032, 2048}) CHECK(kvq_build_codebooks(d, 2, nullptr, &cb) == KVQ_ERR_SHAPE);
  for (int bits : {0, 5, -1}) CHECK(kvq_build_codebooks(128, bits, nullptr, &cb) == KVQ_ERR_SHAPE);
}

// ------------------------------------------------------------------------- bucket tables

// The 3- and 4-bit encoders quantize through bucket tables built on the host: a value is
// scaled to w, the entry is read at the byte offset that the bits of v + 2^13 (stage 1,
// 16-byte entries) or v + 2^14 (stage 2, 8-byte entries) give under a mask, for
// v = clamp(w + 1/2, 0, 1), and the code is the entry's count plus [w > its threshold].
// This replays those float32 steps (the same roundings: std::fma, float adds) on the tables
// the host hands to the launch and checks (a) that the lookup equals a plain count of the
// thresholds for every w of a dense sweep, far outside the table's range, and around every
// threshold and bucket edge, (b) that the thresholds and the stage-2 offsets are the
// codebook's boundaries and centroids in w units, and (c) that the whole two-stage decision
// agrees with the float64 definition (count the boundaries y exceeds, then those its
// residual exceeds) except within 1e-5 relative of a boundary, with an exact zero taking
// the code below the middle boundary.

uint32_t as_u32(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

float clamp01(float v) { return v < 0.f ? 0.f : (v > 1.f ? 1.f : v); }

// entry of w in a table of `stride` floats per entry (4: stage 1, 2: stage 2)
const float* table_entry(const float* tab, int stride, float w) {
  const float v = clamp01(w + 0.5f);
  const float magic = stride == 4 ? 8192.0f : 16384.0f;
  const uint32_t mask = stride == 4 ? 0x7F0u : 0x3F8u;
  const uint32_t off = as_u32(v + magic) & mask;  // bytes
  const int entry = static_cast<int>(off / (4u * stride));
  CHECK(entry >= 0 && entry < kvq::kTabEntries);
  return tab + std::min(entry, kvq::kTabEntries - 1) * stride;
}

int table_code(const float* tab, int stride, float w) {
  const float* e = table_entry(tab, stride, w);
  return static_cast<int>(as_u32(e[1])) + (w > e[0] ? 1 : 0);
}

// the distinct thresholds a table holds, ascending
std::vector<float> table_thresholds(const float* tab, int stride) {
  std::vector<float> t;
  for (int j = 0; j < kvq::kTabEntries; ++j)
    if (!std::isinf(tab[j * stride])) t.push_back(tab[j * stride]);
  std::sort(t.begin(), t.end());
  t.erase(std::unique(t.begin(), t.end()), t.end());
  return t;
}

void check_lookup_against_count(const float* tab, int stride, const std::vector<float>& tw) {
  std::vector<float> ws;
  for (int i = -(1 << 16); i <= (1 << 16); ++i) ws.push_back(static_cast<float>(i) / 98304.0f);
  for (float far : {0.75f, 1.0f, 3.0f, 50.0f, 1e30f}) {
    ws.push_back(far);
    ws.push_back(-far);
  }
  const int sub = stride == 4 ? 16 : 8;
  for (int j = 0; j <= kvq::kTabBuckets; ++j) {  // bucket edges: half-way between grid points
    float e = static_cast<float>((sub * j - 0.5) / (sub * kvq::kTabBuckets) - 0.5);
    for (int k = 0; k < 4; ++k) e = std::nextafter(e, -1.0f);
    for (int k = 0; k < 8; ++k, e = std::nextafter(e, 2.0f)) ws.push_back(e);
  }
  for (float t : tw) {
    float e = t;
    for (int k = 0; k < 4; ++k) e = std::nextafter(e, -1.0f);
    for (int k = 0; k < 8; ++k, e = std::nextafter(e, 2.0f)) ws.push_back(e);
  }
  ws.push_back(0.0f);
  int bad = 0;
  for (float w : ws) {
    int count = 0;
    for (float t : tw) count += w > t ? 1 : 0;
    bad += table_code(tab, stride, w) != count ? 1 : 0;
  }
  CHECK(bad == 0);
}

void test_bucket_tables() {
  float* nr = fake<float>(0x40000);
  for (int d : {8, 64, 128, 1024}) {
    for (int bits : {3, 4}) {
      kvq_codebooks cb;
      CHECK(kvq_build_codebooks(d, bits, nullptr, &cb) == KVQ_OK);
      kvq::g_stub = kvq::StubLog{};
      CHECK(kvq_rvq_encode_pack(&cb, fake<uint16_t>(0x10000), 1, 1, 1, fake<uint32_t>(0x20000),
                                fake<uint32_t>(0x30000), nr, 1, 0, nullptr) == KVQ_OK);
      const kvq::EncodeArgs& a = kvq::g_stub.enc;
      const float* t1 = &a.tab1[0][0];
      const float* t2 = &a.tab2[0][0];
      const int L = 1 << bits;
      const std::vector<float> tv1 = table_thresholds(t1, 4), tv2 = table_thresholds(t2, 2);
      CHECK(static_cast<int>(tv1.size()) == L - 1 && static_cast<int>(tv2.size()) == L - 1);
      if (static_cast<int>(tv1.size()) != L - 1 || static_cast<int>(tv2.size()) != L - 1) continue;
      CHECK(tv1[L / 2 - 1] == 0.0f && tv2[L / 2 - 1] == 0.0f);  // the middle boundary 0
      check_lookup_against_count(t1, 4, tv1);
      check_lookup_against_count(t2, 2, tv2);

      // (b) w = t / (2R): the thresholds are the boundaries, the offsets minus the centroids
      const double sqd = std::sqrt(static_cast<double>(d));
      const double two_r1 = 1.0 / (sqd * a.k_scale), two_r2 = 1.0 / (sqd * a.k2_scale);
      for (int k = 0; k < L - 1; ++k) {
        CHECK(std::fabs(tv1[k] * two_r1 - cb.b1[k]) <= 1e-6 * two_r1);
        CHECK(std::fabs(tv2[k] * two_r2 - cb.b2[k]) <= 1e-6 * two_r2);
      }
      for (int j = 0; j < kvq::kTabEntries; ++j) {
        const int m = static_cast<int>(as_u32(t1[4 * j + 1]));
        const int m_hi = m + (std::isinf(t1[4 * j]) ? 0 : 1);
        CHECK(m >= 0 && m_hi < L);
        if (m < 0 || m_hi >= L) continue;
        CHECK(std::fabs(-t1[4 * j + 2] * two_r2 - cb.c1[m]) <= 1e-6 * two_r2);
        CHECK(std::fabs(-t1[4 * j + 3] * two_r2 - cb.c1[m_hi]) <= 1e-6 * two_r2);
      }

      // (c) the two-stage decision for a unit-norm vector (K = k_scale): y' = y_true sqrt(d)
      std::mt19937_64 rng(1000 + 10 * d + bits);
      std::normal_distribution<double> gauss(0.0, cb.sigma1);
      std::uniform_real_distribution<double> wide(-1.0, 1.0);
      const float K = a.k_scale, K2 = a.k2_scale;  // n = 1
      int bad = 0, near = 0;
      for (int i = 0; i < 400000; ++i) {
        const double y = i == 0 ? 0.0 : (i % 4 == 3 ? wide(rng) : gauss(rng));
        const float yp = static_cast<float>(y * sqd);
        const double yt = static_cast<double>(yp) / sqd;
        const float w1 = std::fma(yp, K, 0.0f);
        const float* e = table_entry(t1, 4, w1);
        const bool gt = w1 > e[0];
        const int c1 = static_cast<int>(as_u32(e[1])) + (gt ? 1 : 0);
        const float w2 = std::fma(yp, K2, gt ? e[3] : e[2]);
        const int c2 = table_code(t2, 2, w2);
        int o1 = 0, o2 = 0;
        for (int k = 0; k < L - 1; ++k) o1 += yt > cb.b1[k] ? 1 : 0;
        const double r = yt - cb.c1[o1];
        for (int k = 0; k < L - 1; ++k) o2 += r > cb.b2[k] ? 1 : 0;
        if (i == 0) CHECK(c1 == L / 2 - 1 && c2 == o2);
        if (c1 == o1 && c2 == o2) continue;
        bool allowed = false;
        if (c1 != o1) {
          for (int k = 0; k < L - 1; ++k)
            allowed |= std::abs(c1 - o1) == 1 &&
                       std::fabs(yt - cb.b1[k]) <= 1e-5 * std::fmax(std::fabs(cb.b1[k]), cb.sigma1);
        } else {
          for (int k = 0; k < L - 1; ++k)
            allowed |= std::abs(c2 - o2) == 1 &&
                       std::fabs(r - cb.b2[k]) <= 1e-5 * std::fmax(std::fabs(cb.b2[k]), cb.sigma2);
        }
        near += allowed ? 1 : 0;
        bad += allowed ? 0 : 1;
      }
      CHECK(bad == 0);
      CHECK(near <= 2);
    }
  }
}

// ------------------------------------------------------------------------ encode / decode

void test_encode_decode() {
  kvq_codebooks cb;
  CHECK(kvq_build_codebooks(128, 2, nullptr, &cb) == KVQ_OK);
  uint16_t* x = fake<uint16_t>(0x10000);
  uint32_t* p1 = fake<uint32_t>(0x20000);
  uint32_t* p2 = fake<uint32_t>(0x30000);
  float* nr = fake<float>(0x40000);
  kvq::g_stub = kvq::StubLog{};

  // contiguous cache: row map is the identity
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.encode_calls == 1 && kvq::g_stub.enc.n_vec == 30 && kvq::g_stub.enc.map.contiguous == 1);
  CHECK(kvq::g_stub.d == 128 && kvq::g_stub.bits == 2 && kvq::g_stub.stages == 2);
  CHECK(kvq::g_stub.enc.x == x && kvq::g_stub.enc.p1 == p1 && kvq::g_stub.enc.p2 == p2 && kvq::g_stub.enc.norms == nr);
  // a window of a larger cache
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 100, 7, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.enc.map.contiguous == 0 && kvq::g_stub.enc.map.S == 5 && kvq::g_stub.enc.map.S_cap == 100 &&
        kvq::g_stub.enc.map.s_offset == 7);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 100, 95, nullptr) == KVQ_OK);  // ends at S_cap
  // range, shape, alignment, null checks
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 100, 96, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 4, 0, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 100, -1, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_encode_pack(&cb, x, -1, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_SHAPE);
  CHECK(kvq_rvq_encode_pack(&cb, x, int64_t(1) << 40, int64_t(1) << 40, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_encode_pack(&cb, fake<uint16_t>(0x10002), 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, fake<uint32_t>(0x20004), p2, nr, 5, 0, nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, fake<float>(0x40002), 5, 0, nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq_rvq_encode_pack(&cb, nullptr, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, nullptr, nr, 5, 0, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_rvq_encode_pack(nullptr, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_ARG);
  kvq_codebooks bad = cb;
  bad.n_words = 9;
  CHECK(kvq_rvq_encode_pack(&bad, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_ARG);
  bad = cb;
  bad.d = 1025;  // above the largest head dimension
  CHECK(kvq_rvq_encode_pack(&bad, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_SHAPE);
  bad.d = 64;  // its word count is not that of d = 64
  CHECK(kvq_rvq_encode_pack(&bad, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_ERR_ARG);
  // a padded head dimension: the launcher gets d, and the arguments the rotation length's
  // tables with d / 8 real chunks per row; the sign code takes powers of two only
  kvq_codebooks c96, c96b1;
  CHECK(kvq_build_codebooks(96, 2, nullptr, &c96) == KVQ_OK && kvq_build_codebooks(96, 1, nullptr, &c96b1) == KVQ_OK);
  CHECK(kvq_rvq_encode_pack(&c96, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.d == 96 && kvq::g_stub.enc.dh == 96 && kvq::g_stub.enc.n_vec == 30);
  CHECK(kvq_rvq_unpack_decode(&c96, p1, p2, nr, 2, 3, 5, 0, 5, x, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.d == 96 && kvq::g_stub.dec.dh == 96 && kvq::g_stub.dec.inv_sqrt_d == 1.0f / std::sqrt(128.0f));
  CHECK(kvq_rabitq_encode_pack(&c96b1, x, 1, 1, 8, p1, nr, 8, 0, nullptr) == KVQ_ERR_SHAPE);
  kvq_codebooks c100;  // rows that are not 16-byte aligned: the same arguments, d elements a row
  CHECK(kvq_build_codebooks(100, 3, nullptr, &c100) == KVQ_OK && c100.n_words == 13);
  CHECK(kvq_rvq_encode_pack(&c100, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.d == 100 && kvq::g_stub.enc.dh == 100);
  CHECK(kvq_rvq_encode_pack(&cb, x, 2, 3, 5, p1, p2, nr, 5, 0, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.enc.dh == 128);
  kvq::g_stub = kvq::StubLog{};
  const int before = kvq::g_stub.encode_calls;
  CHECK(kvq_rvq_encode_pack(&cb, nullptr, 0, 3, 5, nullptr, nullptr, nullptr, 5, 0, nullptr) == KVQ_OK);  // empty
  CHECK(kvq::g_stub.encode_calls == before);

  // single-stage codec and the sign code go through the same launcher with fewer stages
  CHECK(kvq_mse_encode_pack(&cb, x, 1, 1, 8, p1, nr, 8, 0, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.stages == 1 && kvq::g_stub.enc.p2 == nullptr);
  kvq_codebooks cb1;
  CHECK(kvq_build_codebooks(128, 1, nullptr, &cb1) == KVQ_OK);
  CHECK(kvq_rabitq_encode_pack(&cb1, x, 1, 1, 8, p1, nr, 8, 0, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.stages == 0 && kvq::g_stub.bits == 1);
  CHECK(kvq_rabitq_encode_pack(&cb, x, 1, 1, 8, p1, nr, 8, 0, nullptr) == KVQ_ERR_SHAPE);  // 2-bit codebooks

  // decode
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nr, 2, 3, 100, 7, 5, x, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.decode_calls == 1 && kvq::g_stub.dec.n_vec == 30 && kvq::g_stub.dec.map.s_offset == 7);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nullptr, 2, 3, 5, 0, 5, x, nullptr) == KVQ_OK);  // unit mode
  CHECK(kvq::g_stub.dec.norms == nullptr && kvq::g_stub.dec.map.contiguous == 1);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nr, 2, 3, 100, 96, 5, x, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, nullptr, nr, 2, 3, 5, 0, 5, x, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nr, 2, 3, 5, 0, 5, fake<uint16_t>(0x10008), nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq_mse_unpack_decode(&cb, p1, nr, 1, 1, 8, 0, 8, x, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.stages == 1);
}

// Codebook structs that break what the kernels assume (ascending, exactly antisymmetric
// tables whose boundaries are the float32 midpoints of neighbouring centroids, so the middle
// boundary is +0.0) are rejected with KVQ_ERR_ARG before anything is launched, at every bit
// width and by every entry point that takes them.
void test_tampered_codebooks() {
  uint16_t* x = fake<uint16_t>(0x10000);
  uint32_t* p1 = fake<uint32_t>(0x20000);
  uint32_t* p2 = fake<uint32_t>(0x30000);
  float* nr = fake<float>(0x40000);
  for (int bits = 1; bits <= 4; ++bits) {
    kvq_codebooks cb;
    CHECK(kvq_build_codebooks(128, bits, nullptr, &cb) == KVQ_OK);
    const int L = 1 << bits;
    auto rejected = [&](const kvq_codebooks& bad) {
      kvq::g_stub = kvq::StubLog{};
      bool ok = kvq_rvq_encode_pack(&bad, x, 1, 2, 8, p1, p2, nr, 8, 0, nullptr) == KVQ_ERR_ARG &&
                kvq_rvq_unpack_decode(&bad, p1, p2, nr, 1, 2, 8, 0, 8, x, nullptr) == KVQ_ERR_ARG &&
                kvq_mse_encode_pack(&bad, x, 1, 2, 8, p1, nr, 8, 0, nullptr) == KVQ_ERR_ARG;
      return ok && kvq::g_stub.encode_calls == 0 && kvq::g_stub.decode_calls == 0;
    };
    kvq_codebooks bad = cb;
    bad.b1[L / 2 - 1] = -0.0f;  // middle boundary -0
    CHECK(rejected(bad));
    bad = cb;
    bad.b2[L / 2 - 1] = -0.0f;
    CHECK(rejected(bad));
    bad = cb;
    bad.c1[L - 1] = std::nextafter(cb.c1[L - 1], 1.0f);  // breaks antisymmetry (and the last midpoint)
    CHECK(rejected(bad));
    bad = cb;
    bad.c2[0] = std::nextafter(cb.c2[0], -1.0f);
    CHECK(rejected(bad));
    bad = cb;
    bad.b1[0] = std::nextafter(cb.b1[0], -1.0f);  // a boundary one ulp off its midpoint
    CHECK(rejected(bad));
    bad = cb;
    bad.b2[L - 2] = std::nextafter(cb.b2[L - 2], 1.0f);
    CHECK(rejected(bad));
    bad = cb;  // both tables scaled together: still antisymmetric, still midpoints; accepted
    for (int k = 0; k < L; ++k) bad.c1[k] *= 2.0f;
    for (int k = 0; k + 1 < L; ++k) bad.b1[k] *= 2.0f;
    CHECK(kvq_rvq_encode_pack(&bad, x, 1, 2, 8, p1, p2, nr, 8, 0, nullptr) == KVQ_OK);
    bad = cb;
    for (int k = 0; k < L; ++k) std::swap(bad.c1[k], bad.c1[L - 1 - k]);  // descending
    for (int k = 0; k + 1 < L; ++k) bad.b1[k] = -bad.b1[k];
    if (bits > 1) {
      for (int k = 0; k < (L - 1) / 2; ++k) std::swap(bad.b1[k], bad.b1[L - 2 - k]);
      CHECK(rejected(bad));
    }
    bad = cb;
    bad.c1[0] = -std::numeric_limits<float>::infinity();
    bad.c1[L - 1] = std::numeric_limits<float>::infinity();
    CHECK(rejected(bad));
  }
  // the attention takes the same checks
  kvq_codebooks ck, cv;
  CHECK(kvq_build_codebooks(128, 2, nullptr, &ck) == KVQ_OK);
  cv = ck;
  cv.b1[1] = -0.0f;
  int64_t need = 0;
  CHECK(kvq_rvq_attend_workspace_size(128, 2, 1, 32, 1, 8, 4096, &need) == KVQ_OK);
  CHECK(kvq_rvq_attend(&ck, &cv, x, 1, 32, 1, 8, p1, p2, nr, p1, p2, nr, 4096, 4096, 0.1f,
                       fake<void>(0x50000), need, x, nullptr) == KVQ_ERR_ARG);
}

// The kernels index their tiles with 32-bit integers: a launch needing more than INT_MAX
// tiles is refused with KVQ_ERR_RANGE on the host (at d = 1024 the butterfly kernels hold 2
// vectors per tile, at d = 256 8; the matrix-core encodes at d = 128 and 256 and the decode
// at d = 128 hold 16).
void test_tile_limit() {
  uint16_t* x = fake<uint16_t>(0x10000);
  uint32_t* p1 = fake<uint32_t>(0x20000);
  uint32_t* p2 = fake<uint32_t>(0x30000);
  float* nr = fake<float>(0x40000);
  const int64_t imax = std::numeric_limits<int32_t>::max();
  kvq_codebooks cb;
  CHECK(kvq_build_codebooks(1024, 2, nullptr, &cb) == KVQ_OK);
  kvq::g_stub = kvq::StubLog{};
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 2 * imax, p1, p2, nr, 2 * imax, 0, nullptr) == KVQ_OK);
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 2 * imax + 1, p1, p2, nr, 2 * imax + 1, 0, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nr, 1, 1, 2 * imax, 0, 2 * imax, x, nullptr) == KVQ_OK);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nr, 1, 1, 2 * imax + 2, 0, 2 * imax + 2, x, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq::g_stub.encode_calls == 1 && kvq::g_stub.decode_calls == 1);
  CHECK(kvq_build_codebooks(128, 2, nullptr, &cb) == KVQ_OK);
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 16 * imax, p1, p2, nr, 16 * imax, 0, nullptr) == KVQ_OK);
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 16 * imax + 1, p1, p2, nr, 16 * imax + 1, 0, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_rvq_unpack_decode(&cb, p1, p2, nr, 1, 1, 16 * imax + 1, 0, 16 * imax + 1, x, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_build_codebooks(256, 2, nullptr, &cb) == KVQ_OK);  // matrix cores
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 16 * imax, p1, p2, nr, 16 * imax, 0, nullptr) == KVQ_OK);
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 16 * imax + 1, p1, p2, nr, 16 * imax + 1, 0, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_build_codebooks(256, 3, nullptr, &cb) == KVQ_OK);  // butterfly
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 8 * imax, p1, p2, nr, 8 * imax, 0, nullptr) == KVQ_OK);
  CHECK(kvq_rvq_encode_pack(&cb, x, 1, 1, 8 * imax + 1, p1, p2, nr, 8 * imax + 1, 0, nullptr) == KVQ_ERR_RANGE);
}

// The allocation-free attention: the same checks as kvq_rvq_attend, all on the host before
// the scratch is looked up; plans beyond the scratch are refused with KVQ_ERR_RANGE; a good
// call launches with the scratch address as its workspace.
void test_attend_noalloc() {
  kvq_codebooks ck, cv;
  CHECK(kvq_build_codebooks(128, 2, nullptr, &ck) == KVQ_OK);
  CHECK(kvq_build_codebooks(128, 2, nullptr, &cv) == KVQ_OK);
  uint16_t* q = fake<uint16_t>(0x10000);
  uint16_t* out = fake<uint16_t>(0x11000);
  uint32_t* p1 = fake<uint32_t>(0x20000);
  uint32_t* p2 = fake<uint32_t>(0x30000);
  float* nr = fake<float>(0x40000);
  kvq::g_stub = kvq::StubLog{};
  CHECK(kvq_rvq_attend_noalloc(&ck, &cv, q, 1, 32, 1, 8, p1, p2, nr, p1, p2, nr, 32768, 32768, 0.1f, out, nullptr) ==
        KVQ_OK);
  CHECK(kvq::g_stub.attend_calls == 1 && kvq::g_stub.scratch_lookups == 1);
  CHECK(kvq::g_stub.att.ws == reinterpret_cast<float*>(uintptr_t(0x7000000)));
  // 131072 query vectors of one position each need 131072 x 132 x 4 bytes (69 MB) of records
  int64_t need = 0;
  CHECK(kvq_rvq_attend_workspace_size(128, 2, 1, 32, 4096, 8, 4096, &need) == KVQ_OK);
  CHECK(need > KVQ_ATTEND_SCRATCH_BYTES);
  CHECK(kvq_rvq_attend_noalloc(&ck, &cv, q, 1, 32, 4096, 8, p1, p2, nr, p1, p2, nr, 4096, 4096, 0.1f, out, nullptr) ==
        KVQ_ERR_RANGE);
  // argument errors come before the lookup
  CHECK(kvq_rvq_attend_noalloc(&ck, &cv, q, 1, 32, 1, 8, p1, p2, nr, p1, p2, nr, 4096, 4096, 0.1f, nullptr, nullptr) ==
        KVQ_ERR_ARG);
  CHECK(kvq_rvq_attend_noalloc(&ck, &cv, q, 1, 32, 1, 7, p1, p2, nr, p1, p2, nr, 4096, 4096, 0.1f, out, nullptr) ==
        KVQ_ERR_SHAPE);
  CHECK(kvq_rvq_attend_noalloc(&ck, &cv, fake<uint16_t>(0x10002), 1, 32, 1, 8, p1, p2, nr, p1, p2, nr, 4096, 4096,
                               0.1f, out, nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq::g_stub.attend_calls == 1 && kvq::g_stub.scratch_lookups == 1);
}

// ------------------------------------------------------------------------------ QJL

void test_qjl() {
  for (int d : {32, 64, 128, 256})
    for (int m = 32; m <= 256; m += 32) {
      const bool fits = (static_cast<int64_t>(m) * d + 4 * 32 * d) * 2 <= 160 * 1024;
      CHECK(kvq_qjl_supported(d, m) == (fits ? KVQ_OK : KVQ_ERR_SHAPE));
    }
  for (int d : {8, 16, 512, 1024, 100}) CHECK(kvq_qjl_supported(d, 64) == KVQ_ERR_SHAPE);
  for (int m : {0, 16, 48, 288}) CHECK(kvq_qjl_supported(128, m) == KVQ_ERR_SHAPE);
  uint16_t* sk = fake<uint16_t>(0x50000);
  uint16_t* x = fake<uint16_t>(0x10000);
  uint32_t* p = fake<uint32_t>(0x20000);
  uint16_t* nr = fake<uint16_t>(0x40002);  // fp16 norms need 2-byte alignment only
  kvq::g_stub = kvq::StubLog{};
  CHECK(kvq_qjl_encode_pack(sk, 128, 96, x, 2, 4, 33, p, nr, 40, 7, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.qjl_calls == 1 && kvq::g_stub.m == 96 && kvq::g_stub.qjl.n_vec == 2 * 4 * 33);
  CHECK(kvq::g_stub.qjl.map.contiguous == 0 && kvq::g_stub.qjl.map.S_cap == 40);
  CHECK(kvq_qjl_encode_pack(sk, 128, 100, x, 2, 4, 33, p, nr, 40, 7, nullptr) == KVQ_ERR_SHAPE);
  CHECK(kvq_qjl_encode_pack(sk, 128, 96, x, 2, 4, 33, p, nr, 40, 8, nullptr) == KVQ_ERR_RANGE);
  CHECK(kvq_qjl_encode_pack(nullptr, 128, 96, x, 2, 4, 33, p, nr, 40, 7, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_qjl_encode_pack(fake<uint16_t>(0x50008), 128, 96, x, 2, 4, 33, p, nr, 40, 7, nullptr) == KVQ_ERR_ALIGN);
  CHECK(kvq_qjl_encode_pack(sk, 128, 96, x, 2, 4, 33, p, fake<uint16_t>(0x40001), 40, 7, nullptr) == KVQ_ERR_ALIGN);
}

// ------------------------------------------------------------------------------ attention

void test_attend() {
  kvq_codebooks ck, cv, c3;
  CHECK(kvq_build_codebooks(128, 2, nullptr, &ck) == KVQ_OK);
  CHECK(kvq_build_codebooks(128, 2, nullptr, &cv) == KVQ_OK);
  CHECK(kvq_build_codebooks(128, 3, nullptr, &c3) == KVQ_OK);
  uint16_t* q = fake<uint16_t>(0x10000);
  uint16_t* out = fake<uint16_t>(0x18000);
  uint32_t* k1 = fake<uint32_t>(0x20000);
  uint32_t* k2 = fake<uint32_t>(0x30000);
  uint32_t* v1 = fake<uint32_t>(0x40000);
  uint32_t* v2 = fake<uint32_t>(0x50000);
  float* kn = fake<float>(0x60000);
  float* vn = fake<float>(0x70000);
  void* ws = fake<void>(0x100000);
  struct Shape {
    int64_t B, Hq, Sq, Hkv, S_cap, S_kv;
  };
  const Shape shapes[] = {{1, 32, 1, 8, 32768, 32768}, {2, 8, 3, 2, 1000, 999}, {1, 4, 1, 4, 5, 1},
                          {3, 6, 2, 3, 70000, 65537}, {1, 1, 1, 1, 1 << 20, 1 << 20}};
  for (int bits : {1, 2, 3, 4})
    for (int d : {8, 64, 128, 1024})
      for (const Shape& s : shapes) {
        kvq_codebooks a, b;
        CHECK(kvq_build_codebooks(d, bits, nullptr, &a) == KVQ_OK);
        CHECK(kvq_build_codebooks(d, bits, nullptr, &b) == KVQ_OK);
        int64_t need = -1;
        CHECK(kvq_rvq_attend_workspace_size(d, bits, s.B, s.Hq, s.Sq, s.Hkv, s.S_kv, &need) == KVQ_OK);
        CHECK(need > 0);
        kvq::g_stub = kvq::StubLog{};
        CHECK(kvq_rvq_attend(&a, &b, q, s.B, s.Hq, s.Sq, s.Hkv, k1, k2, kn, v1, v2, vn, s.S_cap, s.S_kv, 0.1f, ws,
                             need, out, nullptr) == KVQ_OK);
        const kvq::AttendArgs& p = kvq::g_stub.att;
        CHECK(kvq::g_stub.attend_calls == 1);
        CHECK(p.n_q == s.B * s.Hq * s.Sq && p.group == s.Hq / s.Hkv && p.Hkv == s.Hkv && p.Sq == s.Sq);
        // the chunks cover the cached positions, none of them empty, within the combine's limit
        CHECK(p.n_splits >= 1 && p.n_splits <= 4096 && p.chunk >= 1);
        CHECK(static_cast<int64_t>(p.chunk) * p.n_splits >= s.S_kv);
        CHECK(static_cast<int64_t>(p.chunk) * (p.n_splits - 1) < s.S_kv);
        // one record of d + 4 floats per (query vector, chunk) fits the workspace
        CHECK(p.n_q * p.n_splits * (d + 4) * 4 <= need);
        CHECK(kvq_rvq_attend(&a, &b, q, s.B, s.Hq, s.Sq, s.Hkv, k1, k2, kn, v1, v2, vn, s.S_cap, s.S_kv, 0.1f, ws,
                             need - 1, out, nullptr) == KVQ_ERR_RANGE);
      }
  int64_t need = 0;
  CHECK(kvq_rvq_attend_workspace_size(128, 2, 1, 32, 1, 8, 4096, &need) == KVQ_OK);
  const auto call = [&](const kvq_codebooks* a, const kvq_codebooks* b, int64_t Hq, int64_t Hkv, int64_t S_cap,
                        int64_t S_kv, float scale, void* w, int64_t wb, uint16_t* o) {
    return kvq_rvq_attend(a, b, q, 1, Hq, 1, Hkv, k1, k2, kn, v1, v2, vn, S_cap, S_kv, scale, w, wb, o, nullptr);
  };
  CHECK(call(&ck, &cv, 32, 8, 4096, 4096, 0.1f, ws, need, out) == KVQ_OK);
  CHECK(call(&ck, &c3, 32, 8, 4096, 4096, 0.1f, ws, need, out) == KVQ_ERR_SHAPE);   // different bits
  kvq_codebooks k96, v96;  // the attention takes powers of two only
  CHECK(kvq_build_codebooks(96, 2, nullptr, &k96) == KVQ_OK && kvq_build_codebooks(96, 2, nullptr, &v96) == KVQ_OK);
  CHECK(call(&k96, &v96, 32, 8, 4096, 4096, 0.1f, ws, need, out) == KVQ_ERR_SHAPE);
  CHECK(call(&ck, &cv, 30, 8, 4096, 4096, 0.1f, ws, need, out) == KVQ_ERR_SHAPE);   // Hq % Hkv
  CHECK(call(&ck, &cv, 32, 8, 4095, 4096, 0.1f, ws, need, out) == KVQ_ERR_RANGE);   // S_kv > S_cap
  CHECK(call(&ck, &cv, 32, 8, 4096, 0, 0.1f, ws, need, out) == KVQ_ERR_RANGE);      // S_kv < 1
  CHECK(call(&ck, &cv, 32, 8, 4096, 4096, NAN, ws, need, out) == KVQ_ERR_ARG);
  CHECK(call(&ck, &cv, 32, 8, 4096, 4096, INFINITY, ws, need, out) == KVQ_ERR_ARG);
  CHECK(call(&ck, &cv, 32, 8, 4096, 4096, 0.1f, nullptr, need, out) == KVQ_ERR_ARG);
  CHECK(call(&ck, &cv, 32, 8, 4096, 4096, 0.1f, fake<void>(0x100004), need, out) == KVQ_ERR_ALIGN);
  CHECK(call(&ck, &cv, 32, 8, 4096, 4096, 0.1f, ws, need, fake<uint16_t>(0x18002)) == KVQ_ERR_ALIGN);
  CHECK(call(nullptr, &cv, 32, 8, 4096, 4096, 0.1f, ws, need, out) == KVQ_ERR_ARG);
  CHECK(kvq_rvq_attend_workspace_size(128, 2, 1, 32, 1, 8, 4096, nullptr) == KVQ_ERR_ARG);
  CHECK(kvq_rvq_attend_workspace_size(96, 2, 1, 32, 1, 8, 4096, &need) == KVQ_ERR_SHAPE);
  CHECK(kvq_rvq_attend_workspace_size(128, 5, 1, 32, 1, 8, 4096, &need) == KVQ_ERR_SHAPE);
  CHECK(kvq_rvq_attend_workspace_size(128, 2, 1, 32, 1, 8, 0, &need) == KVQ_ERR_RANGE);
  // no query vectors: nothing to do, no pointer is looked at
  kvq::g_stub = kvq::StubLog{};
  CHECK(kvq_rvq_attend(&ck, &cv, nullptr, 0, 32, 1, 8, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 4096,
                       4096, 0.1f, nullptr, 0, nullptr, nullptr) == KVQ_OK);
  CHECK(kvq::g_stub.attend_calls == 0);
}

void test_status_text() {
  for (int s = -7; s <= 2; ++s) CHECK(kvq_status_str(static_cast<kvq_status>(s)) != nullptr);
}

}  // namespace

int main() {
  test_codebooks();
  test_encode_decode();
  test_tampered_codebooks();
  test_tile_limit();
  test_bucket_tables();
  test_qjl();
  test_attend();
  test_attend_noalloc();
  test_status_text();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
