// HIP kernels for gfx950 (MI355X): softmax attention of fp16 queries over a packed
// two-stage RVQ key/value cache, without reconstructing either cache.
//
// Method (VeloxQuant-MLX blog, "turboquant" tag page, "Kernel 5": one FlashAttention-style
// pass decodes each key as c1[i1] + c2[i2] on the fly and keeps an online softmax, so the
// dequantized keys are never written). Here both caches stay packed and the whole pass runs
// in the rotated domain. The rotation R = H diag(s) / sqrt(D) is orthonormal and a cached
// vector is n R^T z, with z = c1[i1] + c2[i2] its dequantized rotated coordinates, so
//   q . k_t = n_t (R_k q) . z_t        and        sum_t p_t v_t = R_v^T (sum_t p_t n_t z_t):
// the query is rotated once, every key costs one table lookup and one FMA per coordinate,
// every value one lookup and one FMA, and the output is rotated back once per query.
//
// Work split (flash decoding): the cached positions [0, S_kv) are cut into chunks. One wave
// handles up to 4 query vectors that read the same key/value head, over one chunk, with the
// codec's lane layout (L lanes per head vector, C coordinates per lane, 64 / L cached
// positions per iteration; C = 16 when a wave serves several queries); each key and value
// is decoded once for all of them. Each group of L lanes keeps its own online-softmax state,
// the groups are merged at the end of the chunk, and each query's (max, sum, accumulator)
// for the chunk goes to the caller's workspace.
// attend_combine merges the chunks of each query vector (one block per vector) and rotates
// the result back.
// Scores are kept in base-2 units (the query carries log2(e)), so the exponentials are
// single v_exp_f32 instructions.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <climits>

#include "device.h"
#include "params.h"

namespace kvq {

// Waves per SIMD the partial kernel is compiled for: 3 (168 registers per lane), 2 when a
// wave carries 4 queries (their rotated queries and accumulators alone take 128 registers).
template <int NQW>
constexpr int attend_waves_per_eu() {
  return NQW == 4 ? 2 : 3;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Softmax reference slack (base-2 units): a lane group's exponentials are taken against a
// reference that is moved only when a score exceeds it by more than this, so the running
// state is rescaled a few times per chunk instead of at every new maximum; the weights stay
// below 2^8 and the sums lose nothing (their relative precision is what matters).
constexpr float kRefSlack = 8.f;

// b = 1, 2 or 4: the codes of P = 4 / b consecutive coordinates fill one nibble of a packed
// word. One byte made of a nibble of each stream (stage 1 low, stage 2 high) indexes a table
// of the P dequantized values c1[i1] + c2[i2], so a lane reads P coordinates with one LDS
// load and one shift.
template <int BITS>
constexpr int nibble_coords() {
  return BITS == 3 ? 0 : 4 / BITS;
}

// The table: entry e holds, for p < P, c1[i1] + c2[i2] with i1 = code p of nibble e & 15 and
// i2 = code p of nibble e >> 4, taken from zt[(i1 << BITS) | i2].
template <int BITS>
__device__ __forceinline__ void fill_nibble_table(const float* zt, float* tab) {
  constexpr int P = nibble_coords<BITS>();
  constexpr uint32_t M = (1u << BITS) - 1u;
  for (int e = threadIdx.x; e < 256; e += kBlockThreads)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t i1 = (e >> (BITS * p)) & M, i2 = ((e >> 4) >> (BITS * p)) & M;
      tab[e * P + p] = zt[(i1 << BITS) | i2];
    }
}

// z[j] (j < C) of this lane from its words of both streams (codes of coordinate j at bits
// [BITS j, BITS j + BITS) of the lane's word sequence).
template <int BITS, int C, int NWL>
__device__ __forceinline__ void nibble_z(const uint32_t (&w1)[NWL], const uint32_t (&w2)[NWL], const float* tab,
                                         float (&z)[C]) {
  constexpr int P = nibble_coords<BITS>();
  constexpr int NIB = C / P;  // nibbles per stream that hold this lane's codes
#pragma unroll
  for (int w = 0; w < (NIB + 7) / 8; ++w) {
    // byte k of lo: nibbles 2k of both words; of hi: nibbles 2k + 1
    const uint32_t lo = (w1[w] & 0x0F0F0F0Fu) | ((w2[w] << 4) & 0xF0F0F0F0u);
    const uint32_t hi = ((w1[w] >> 4) & 0x0F0F0F0Fu) | (w2[w] & 0xF0F0F0F0u);
#pragma unroll
    for (int t = 0; t < 8 && 8 * w + t < NIB; ++t) {
      const uint32_t e = ((t & 1 ? hi : lo) >> (8 * (t >> 1))) & 0xFFu;
      const int j0 = P * (8 * w + t);
      if constexpr (P == 4) {
        const float4 v = reinterpret_cast<const float4*>(tab)[e];
        z[j0] = v.x; z[j0 + 1] = v.y; z[j0 + 2] = v.z; z[j0 + 3] = v.w;
      } else if constexpr (P == 2) {
        const float2 v = reinterpret_cast<const float2*>(tab)[e];
        z[j0] = v.x; z[j0 + 1] = v.y;
      } else {
        z[j0] = tab[e];
      }
    }
  }
}

// The inverse rotation of this lane's slice in float32: z <- diag(s_v) H z / sqrt(D) for the
// lane's C coordinates [C q, C q + C) (H in registers, then across the L lanes of the
// vector; cross_stage leaves the lane's result multiplied by (-1)^popcount(q)). vsg holds
// the value signs, bit c of word c / 32.
template <int D, int CM>
__device__ __forceinline__ void unrotate_f32(float (&z)[(Layout<D, CM>::C)], int q, float inv_sqrt_d,
                                             const uint32_t* vsg) {
  using G = Layout<D, CM>;
  constexpr int C = G::C, LOG_L = G::LOG_L;
  lane_stages<C, 1>(z);
  cross_stages<C, LOG_L>(z, q);
  const float K = (__builtin_popcount(q) & 1) ? -inv_sqrt_d : inv_sqrt_d;
  const uint32_t sw = vsg[(C * q) >> 5] >> ((C * q) & 31);
#pragma unroll
  for (int j = 0; j < C; ++j) z[j] = __uint_as_float(__float_as_uint(z[j] * K) ^ (((sw >> j) & 1u) << 31));
}

// Coordinates per lane of the attention layout: 16 when a wave serves several queries
// (their rotated queries and accumulators are 2 * NQW * C registers per lane), else 32.
template <int D, int NQW>
constexpr int attend_cm() {
  return (NQW > 1 && D >= 32 && D <= 512) ? 16 : 32;
}

// One wave: NQW query vectors that read the same key/value head (consecutive query heads of
// one group, or consecutive query positions), over one chunk of cached positions. Each key
// and value is decoded once for all NQW queries.
template <int D, int BITS, int NQW>
__global__ __launch_bounds__(kBlockThreads, attend_waves_per_eu<NQW>()) void attend_partial(const AttendArgs a) {
  constexpr int CM = attend_cm<D, NQW>();
  using G = Layout<D, CM>;
  using S = CodeShape<D, BITS, CM>;
  constexpr int C = G::C, L = G::L, LOG_L = G::LOG_L, VW = G::VW, CH = G::CH, NWL = S::NWL;
  constexpr int NZ = 1 << (2 * BITS);
  constexpr int P = nibble_coords<BITS>();
  constexpr int NT = P ? 256 * P : NZ;  // floats per LDS table

  // z tables: by nibble pair (b = 1, 2, 4) or by (i1 << b) | i2 (b = 3)
  __shared__ __align__(16) float ztk[NT];
  __shared__ __align__(16) float ztv[NT];
  __shared__ uint32_t kx[D / 2];  // key signs as fp16 sign-bit masks, one word per coordinate pair
  __shared__ uint32_t vsg[(D + 31) / 32];  // value signs, bit c of word c / 32
  constexpr bool CST = S::STAGED && !S::DIRECT3;  // codes regrouped through LDS
  __shared__ uint32_t cstage[CST ? kWavesPerBlock : 1][CST ? 2 * S::CSTREAM : 1];
  for (int i = threadIdx.x; i < (D + 31) / 32; i += kBlockThreads) vsg[i] = a.vsign[i];
  if constexpr (P != 0) {
    fill_nibble_table<BITS>(a.ztab_k, ztk);
    fill_nibble_table<BITS>(a.ztab_v, ztv);
  } else {
    for (int i = threadIdx.x; i < NZ; i += kBlockThreads) {
      ztk[i] = a.ztab_k[i];
      ztv[i] = a.ztab_v[i];
    }
  }
  for (int m = threadIdx.x; m < D / 2; m += kBlockThreads) {
    const uint32_t s0 = (a.ksign[(2 * m) >> 5] >> ((2 * m) & 31)) & 1u;
    const uint32_t s1 = (a.ksign[(2 * m + 1) >> 5] >> ((2 * m + 1) & 31)) & 1u;
    kx[m] = (s0 ? 0x8000u : 0u) | (s1 ? 0x80000000u : 0u);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane & (L - 1);
  const int vl = lane >> LOG_L;
  uint32_t* cs = cstage[CST ? wv : 0];

  // Unit u of this wave: (b, hkv, chunk, query group), the query group fastest, so the waves
  // of a block read the same packed keys and values.
  const int64_t GQ = static_cast<int64_t>(a.group) * a.Sq;  // query vectors per key/value head
  const int64_t NG = GQ / NQW;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wv;
  if (u >= (a.n_q / NQW) * a.n_splits) return;  // wave-uniform; no barrier follows
  const int64_t qg = u % NG;
  const int64_t r = u / NG;
  const int sp = static_cast<int>(r % a.n_splits);
  const int64_t bh = r / a.n_splits;  // b * Hkv + hkv
  const int64_t b = bh / a.Hkv, hkv = bh % a.Hkv;
  const int64_t Hq = static_cast<int64_t>(a.Hkv) * a.group;
  int64_t qv[NQW];
#pragma unroll
  for (int k = 0; k < NQW; ++k) {
    const int64_t qi = qg * NQW + k;
    qv[k] = (b * Hq + hkv * a.group + qi / a.Sq) * a.Sq + qi % a.Sq;
  }

  // 1. This lane's slices of the rotated queries, y = H diag(s_k) q (every group of L lanes
  //    holds a copy): stages 1-2 from v_dot2 on the fp16 pairs with the signs as weights,
  //    the rest in registers and across the group's lanes.
  float qs[NQW][C];
  // (R q)_j = lane value * (-1)^popcount(q) / sqrt(D); scale and log2(e) ride along
  const float qk = (__builtin_popcount(q) & 1) ? -a.qscale : a.qscale;
#pragma unroll
  for (int k = 0; k < NQW; ++k) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + qv[k] * D + q * C);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint4 v = qp[c];
      const uint32_t xh[4] = {v.x, v.y, v.z, v.w};
      const uint32_t w[4] = {kPP ^ kx[q * (C / 2) + 4 * c], kPP ^ kx[q * (C / 2) + 4 * c + 1],
                             kPP ^ kx[q * (C / 2) + 4 * c + 2], kPP ^ kx[q * (C / 2) + 4 * c + 3]};
      float o[8];
      dot2_stages8(xh, w, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) qs[k][8 * c + j] = o[j];
    }
    lane_stages<C, 4>(qs[k]);
    cross_stages<C, LOG_L>(qs[k], q);
#pragma unroll
    for (int j = 0; j < C; ++j) qs[k][j] *= qk;
  }

  // 2. The chunk's cached positions, 64 / L per iteration (one per lane group), with the next
  //    iteration's packed words and norms loaded while the current ones are used.
  const int64_t t0 = static_cast<int64_t>(sp) * a.chunk;
  const int64_t t1 = t0 + a.chunk < a.S_kv ? t0 + a.chunk : a.S_kv;
  const int64_t rowbase = bh * a.S_cap;
  uint32_t nk1[NWL], nk2[NWL], nv1[NWL], nv2[NWL];
  float nkn = 0.f, nvn = 0.f;
  auto fetch = [&](int64_t base) {
    const int64_t t = base + vl < t1 ? base + vl : t1 - 1;  // past the chunk: re-read its last key
    const int64_t row = rowbase + t;
    load_lane_words<D, BITS, CM>(a.k1, row, q, nk1);
    load_lane_words<D, BITS, CM>(a.k2, row, q, nk2);
    load_lane_words<D, BITS, CM>(a.v1, row, q, nv1);
    load_lane_words<D, BITS, CM>(a.v2, row, q, nv2);
    nkn = a.kn[row];
    nvn = a.vn[row];
  };
  float m[NQW], l[NQW];  // softmax reference (base 2) and sum of weights of this lane group
  float acc[NQW][C];     // running sum of weight * n_v * z_v, this lane's coordinates
#pragma unroll
  for (int k = 0; k < NQW; ++k) {
    m[k] = -FLT_MAX;
    l[k] = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) acc[k][j] = 0.f;
  }

  fetch(t0);
  for (int64_t base = t0; base < t1; base += VW) {
    uint32_t k1[NWL], k2[NWL], v1[NWL], v2[NWL];
#pragma unroll
    for (int i = 0; i < NWL; ++i) { k1[i] = nk1[i]; k2[i] = nk2[i]; v1[i] = nv1[i]; v2[i] = nv2[i]; }
    const float kn = nkn, vn = nvn;
    if (base + VW < t1) fetch(base + VW);
    const bool valid = base + vl < t1;

    // scores (base 2) = n_k * (scaled R q) . z_k, summed over the group's lanes
    float z[C];
    if constexpr (P != 0) nibble_z<BITS>(k1, k2, ztk, z);
    else codes_to_z<D, BITS, true, CM>(k1, k2, ztk, cs, lane, vl, q, z);
    float w[NQW];
#pragma unroll
    for (int k = 0; k < NQW; ++k) {
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < C; ++j) d4[j & 3] = __builtin_fmaf(qs[k][j], z[j], d4[j & 3]);
      const float dot = lane_sum<LOG_L>((d4[0] + d4[1]) + (d4[2] + d4[3]));  // every lane takes part
      const float sc = valid ? dot * kn : -FLT_MAX;
      // online softmax against the reference m (see kRefSlack)
      if (sc > m[k] + kRefSlack) {
        const float f = exp2_fast(m[k] - sc);
        l[k] *= f;
#pragma unroll
        for (int j = 0; j < C; ++j) acc[k][j] *= f;
        m[k] = sc;
      }
      const float e = valid ? exp2_fast(sc - m[k]) : 0.f;
      l[k] += e;
      w[k] = e * vn;
    }

    if constexpr (P != 0) nibble_z<BITS>(v1, v2, ztv, z);
    else codes_to_z<D, BITS, true, CM>(v1, v2, ztv, cs, lane, vl, q, z);
#pragma unroll
    for (int k = 0; k < NQW; ++k)
#pragma unroll
      for (int j = 0; j < C; ++j) acc[k][j] = __builtin_fmaf(w[k], z[j], acc[k][j]);
  }

  // 3. Merge the lane groups (lanes with equal q), rotate the accumulator back (every lane
  //    group holds the merged state), then group 0 writes each query's record.
#pragma unroll
  for (int k = 0; k < NQW; ++k) {
#pragma unroll
    for (int off = L; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m[k], off), lo = __shfl_xor(l[k], off);
      const float M = __builtin_fmaxf(m[k], mo);
      const float f1 = exp2_fast(m[k] - M), f2 = exp2_fast(mo - M);
      l[k] = l[k] * f1 + lo * f2;
#pragma unroll
      for (int j = 0; j < C; ++j) acc[k][j] = acc[k][j] * f1 + __shfl_xor(acc[k][j], off) * f2;
      m[k] = M;
    }
    unrotate_f32<D, CM>(acc[k], q, a.inv_sqrt_d, vsg);
    if (vl == 0) {
      float* ws = a.ws + (qv[k] * a.n_splits + sp) * (D + 4);
      if (q == 0) {
        ws[0] = m[k];
        ws[1] = l[k];
      }
      float4* wa = reinterpret_cast<float4*>(ws + 4 + q * C);
#pragma unroll
      for (int c = 0; c < C / 4; ++c)
        wa[c] = make_float4(acc[k][4 * c], acc[k][4 * c + 1], acc[k][4 * c + 2], acc[k][4 * c + 3]);
    }
  }
}

// ------------------------------------------------------------------- matrix-core partial pass

// The same partial results on the matrix cores (d = 64 or 128, b = 1, 2 or 4). One wave takes
// up to 16 query vectors of one key/value head over one chunk, 32 cached positions per
// iteration, with v_mfma_f32_16x16x32_f16:
//   scores^T [32 positions x 16 queries] = Z_k [32 x d] . Q^T [d x 16]   (two 16-row blocks)
//   out^T [d x 16 queries] += Z_v^T [d x 32] . P^T [32 x 16]
// Every float32 operand is split into fp16 hi + lo (hi = RN16(v), lo = RN16(v - hi), their
// sum within 2^-22 |v| of v) and a product takes three MFMAs (hi.hi + hi.lo + lo.hi), so the
// scores and sums carry float32-level error. Rows of the score product are keys: lane l
// supplies key l % 16 of the block with coordinates (d/4) (l / 16) + 8 s + [0, 8) at k-step s
// (the same coordinate order in both operands), decoded straight from the packed words
// through an LDS table of (hi, lo) pairs indexed by one nibble of each code stream. It
// receives the scores of keys 4 (l / 16) + [0, 4) for query l % 16, which after the softmax
// are exactly the lane's own P^T operand of the value product. The values are decoded the
// same way into an LDS tile [32 keys][d] (hi and lo planes) and read back transposed with
// ds_read_b64_tr_b16, which hands lane l coordinate l % 16 of four consecutive keys.
// Queries are rotated once per wave (in the codec's lane layout), divided by their largest
// coordinate so their fp16 parts cannot overflow; the value weights p n_v are kept against
// their own softmax-style reference for the same reason, and both are put back in float32.

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaKeys = 32;  // cached positions per iteration
constexpr int kMfmaQ = 16;     // query vectors per wave

// fp16 hi + lo parts of v, packed in pairs: (hi(v0) | hi(v1) << 16) and the same for lo.
__device__ __forceinline__ uint2 split_pair(float v0, float v1) {
  const half2_t h = {static_cast<_Float16>(v0), static_cast<_Float16>(v1)};
  const half2_t lo = {static_cast<_Float16>(v0 - static_cast<float>(h[0])),
                      static_cast<_Float16>(v1 - static_cast<float>(h[1]))};
  return make_uint2(__builtin_bit_cast(uint32_t, h), __builtin_bit_cast(uint32_t, lo));
}

// Table of the matrix path: entry e (a nibble of each stream, P = 4 / b coordinates) holds the
// fp16 hi parts of the P values c1[i1] + c2[i2] (in pairs, P / 2 words) then their lo parts;
// at P = 1 one word, hi | lo << 16.
template <int BITS>
__device__ __forceinline__ void fill_mfma_table(const float* zt, uint32_t* tab) {
  constexpr int P = 4 / BITS;
  constexpr uint32_t M = (1u << BITS) - 1u;
  for (int e = threadIdx.x; e < 256; e += kBlockThreads) {
    float z[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t i1 = (e >> (BITS * p)) & M, i2 = ((e >> 4) >> (BITS * p)) & M;
      z[p] = zt[(i1 << BITS) | i2];
    }
    if constexpr (P == 1) {
      const uint2 hl = split_pair(z[0], 0.f);
      tab[e] = (hl.x & 0xFFFFu) | (hl.y << 16);
    } else {
#pragma unroll
      for (int p = 0; p < P; p += 2) {
        const uint2 hl = split_pair(z[p], z[p + 1]);
        tab[e * P + p / 2] = hl.x;
        tab[e * P + P / 2 + p / 2] = hl.y;
      }
    }
  }
}

// The nibble bytes of a lane's words: byte k of lo[w] indexes coordinates of nibble 2k of
// word w (stage 1 low, stage 2 high), of hi[w] nibble 2k + 1.
template <int NWG>
__device__ __forceinline__ void nibble_bytes(const uint32_t (&w1)[NWG], const uint32_t (&w2)[NWG], uint32_t (&lo)[NWG],
                                             uint32_t (&hi)[NWG]) {
#pragma unroll
  for (int w = 0; w < NWG; ++w) {
    lo[w] = (w1[w] & 0x0F0F0F0Fu) | ((w2[w] << 4) & 0xF0F0F0F0u);
    hi[w] = ((w1[w] >> 4) & 0x0F0F0F0Fu) | (w2[w] & 0xF0F0F0F0u);
  }
}

// The fp16 hi and lo parts of the lane's coordinates 8 S .. 8 S + 7 (of its slice), packed
// as 8 halfs each (one MFMA operand).
template <int BITS, int NWG, int S>
__device__ __forceinline__ void table_operand(const uint32_t (&lo)[NWG], const uint32_t (&hi)[NWG],
                                              const uint32_t* tab, u32x4_t& oh, u32x4_t& ol) {
  constexpr int P = 4 / BITS;
  constexpr int N0 = S * 8 / P;  // first nibble of the step
  auto idx = [&](int t) -> uint32_t { return (((t & 1) ? hi[t >> 3] : lo[t >> 3]) >> (8 * ((t & 7) >> 1))) & 0xFFu; };
  if constexpr (P == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint2 e = reinterpret_cast<const uint2*>(tab)[idx(N0 + k)];
      oh[k] = e.x;
      ol[k] = e.y;
    }
  } else if constexpr (P == 4) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4 e = reinterpret_cast<const uint4*>(tab)[idx(N0 + k)];
      oh[2 * k] = e.x;
      oh[2 * k + 1] = e.y;
      ol[2 * k] = e.z;
      ol[2 * k + 1] = e.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t e0 = tab[idx(N0 + 2 * k)], e1 = tab[idx(N0 + 2 * k + 1)];
      oh[k] = (e0 & 0xFFFFu) | (e1 << 16);
      ol[k] = (e0 >> 16) | (e1 & 0xFFFF0000u);
    }
  }
}

// The key operand of one score MFMA: the lane's coordinates 4 J .. 4 J + 3 (of its slice) as
// 8 fp16 k-slots holding each coordinate's hi and lo parts, taken from the table entries
// as they are: (hi 01, lo 01, hi 23, lo 23) at b = 2, (hi 01, hi 23, lo 01, lo 23) at b = 1,
// (hi 0, lo 0, hi 1, lo 1, ...) at b = 4. The query operands repeat each coordinate's hi
// (and, in the second product, lo) part in the matching slots, so two MFMAs give the exact
// product of the split key and query values with no operand shuffling.
template <int BITS, int NWG, int J>
__device__ __forceinline__ u32x4_t key_operand(const uint32_t (&lo)[NWG], const uint32_t (&hi)[NWG],
                                               const uint32_t* tab) {
  constexpr int P = 4 / BITS;
  auto idx = [&](int t) -> uint32_t { return (((t & 1) ? hi[t >> 3] : lo[t >> 3]) >> (8 * ((t & 7) >> 1))) & 0xFFu; };
  if constexpr (P == 2) {
    const uint2 e0 = reinterpret_cast<const uint2*>(tab)[idx(2 * J)];
    const uint2 e1 = reinterpret_cast<const uint2*>(tab)[idx(2 * J + 1)];
    return u32x4_t{e0.x, e0.y, e1.x, e1.y};
  } else if constexpr (P == 4) {
    const uint4 e = reinterpret_cast<const uint4*>(tab)[idx(J)];
    return u32x4_t{e.x, e.y, e.z, e.w};
  } else {
    return u32x4_t{tab[idx(4 * J)], tab[idx(4 * J + 1)], tab[idx(4 * J + 2)], tab[idx(4 * J + 3)]};
  }
}

// The query operands for key_operand's slots: p0, p1 are the (hi, lo) fp16 pairs of the
// coordinates (4 J, 4 J + 1) and (4 J + 2, 4 J + 3); h selects the hi (0) or lo (1) parts.
template <int BITS>
__device__ __forceinline__ u32x4_t query_operand(uint2 p0, uint2 p1, int h) {
  constexpr int P = 4 / BITS;
  const uint32_t a = h ? p0.y : p0.x, b = h ? p1.y : p1.x;
  if constexpr (P == 2) {
    return u32x4_t{a, a, b, b};
  } else if constexpr (P == 4) {
    return u32x4_t{a, b, a, b};
  } else {  // each slot pair holds one coordinate's (hi, lo): repeat that coordinate's part
    return u32x4_t{(a & 0xFFFFu) * 0x10001u, (a >> 16) * 0x10001u, (b & 0xFFFFu) * 0x10001u, (b >> 16) * 0x10001u};
  }
}

__device__ __forceinline__ f32x4_t mfma2(const u32x4_t& a, const u32x4_t& b1, const u32x4_t& b2, f32x4_t c) {
  const f16x8_t A = __builtin_bit_cast(f16x8_t, a);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8_t, b1), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(f16x8_t, b2), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma3(const u32x4_t& ah, const u32x4_t& al, const u32x4_t& bh, const u32x4_t& bl,
                                         f32x4_t c) {
  const f16x8_t Ah = __builtin_bit_cast(f16x8_t, ah), Al = __builtin_bit_cast(f16x8_t, al);
  const f16x8_t Bh = __builtin_bit_cast(f16x8_t, bh), Bl = __builtin_bit_cast(f16x8_t, bl);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bh, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Bl, c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Bh, c, 0, 0, 0);
}

template <int D, int BITS>
__global__ __launch_bounds__(kBlockThreads, 2) void attend_mfma(const AttendArgs a) {
  constexpr int P = 4 / BITS;
  constexpr int NW = D * BITS / 32;   // words per vector per stream
  constexpr int CPL = D / 4;          // coordinates of a key per lane
  constexpr int NWG = CPL * BITS / 32;
  constexpr int KS = D / 32;          // k-steps of the score product
  constexpr int CB = D / 16;          // 16-coordinate blocks of the value product
  static_assert(NWG >= 1 && D >= 64 && D <= 128, "matrix path: d = 64 or 128, d b >= 128");
  // Prologue and epilogue: the codec's lane layout with 8 coordinates per lane, so a wave
  // rotates VW = 512 / D query rows per pass and passes stop at the group's real rows (a GQA
  // group of 4 takes one pass at d = 128 instead of rotating all 16 MFMA rows).
  using G = Layout<D, 8>;
  constexpr int C = G::C, L = G::L, LOG_L = G::LOG_L, VW = G::VW;
  constexpr int NPASS = kMfmaQ / VW;  // passes over the 16 rows
  constexpr int VT = kMfmaKeys * D;   // halfs per plane of the value tile

  // The block's LDS in one struct, small tables first: every table address is then a lane
  // offset plus an immediate below 64 KiB, which the LDS instructions encode themselves (as
  // separate variables the tables landed above the 64 KiB value tile, and each lookup paid
  // for an address add).
  struct Smem {
    alignas(16) uint32_t tabk[256 * P];
    alignas(16) uint32_t tabv[256 * P];
    alignas(16) uint32_t kx[D / 2];
    alignas(16) uint32_t vsg[(D + 31) / 32];
    alignas(16) float nrm[kWavesPerBlock][2 * kMfmaKeys];  // the iteration's key, value norms
    alignas(16) uint16_t vtile[kWavesPerBlock][2 * VT];    // hi plane, lo plane
  };
  __shared__ Smem sm;
  auto& tabk = sm.tabk;
  auto& tabv = sm.tabv;
  auto& kx = sm.kx;
  auto& vsg = sm.vsg;
  auto& nrm = sm.nrm;
  auto& vtile = sm.vtile;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;  // MFMA column: query; row of the key operand: key within a block
  const int g = lane >> 4;  // k-group: coordinates [CPL g, CPL g + CPL) of a key
  uint16_t* vt = vtile[wv];
  float* stage = reinterpret_cast<float*>(vt);  // [16][D] float32: queries in, results out

  // unit u = (b, hkv, chunk, query group of 16), the query group fastest
  const int64_t GQ = static_cast<int64_t>(a.group) * a.Sq;  // query vectors per key/value head
  const int64_t NQG = (GQ + kMfmaQ - 1) / kMfmaQ;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wv;
  const int64_t n_bh = static_cast<int64_t>(a.n_q / GQ);  // B * Hkv
  const bool active = u < n_bh * NQG * a.n_splits;  // wave-uniform
  const int64_t qg = u % NQG;
  const int64_t r = u / NQG;
  const int sp = static_cast<int>(r % a.n_splits);
  const int64_t bh = r / a.n_splits;
  const int64_t bb = bh / a.Hkv, hkv = bh % a.Hkv;
  const int64_t Hq = static_cast<int64_t>(a.Hkv) * a.group;
  const int nq = static_cast<int>(GQ - qg * kMfmaQ < kMfmaQ ? GQ - qg * kMfmaQ : kMfmaQ);
  auto qvec = [&](int i) -> int64_t {  // query vector index of the group's i-th query
    const int64_t qi = qg * kMfmaQ + i;
    return (bb * Hq + hkv * a.group + qi / a.Sq) * a.Sq + qi % a.Sq;
  };
  static_assert(C == 8 && NPASS * VW == kMfmaQ, "one 16-byte chunk of each query row per lane");
  const int q = lane & (L - 1), vl = lane >> LOG_L;  // row p VW + vl of pass p, coordinates [8 q, 8 q + 8)

  // Positions, 32 per iteration: block k of 16 keys, lane (n, g) loads key 16 k + n's words of
  // its coordinate slice, and lane l the norms of key l % 32 (shared through LDS); the next
  // iteration's are loaded while the current ones are used.
  const int64_t t0 = static_cast<int64_t>(sp) * a.chunk;
  const int64_t t1 = t0 + a.chunk < a.S_kv ? t0 + a.chunk : a.S_kv;
  const int64_t rowbase = bh * a.S_cap;
  uint32_t nk1[2][NWG], nk2[2][NWG], nv1[2][NWG], nv2[2][NWG];
  float nkn, nvn;
  auto fetch = [&](int64_t base) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t t = base + 16 * k + n < t1 ? base + 16 * k + n : t1 - 1;
      const int64_t row = rowbase + t;
      load_words<NWG>(a.k1 + row * NW + g * NWG, nk1[k]);
      load_words<NWG>(a.k2 + row * NW + g * NWG, nk2[k]);
      load_words<NWG>(a.v1 + row * NW + g * NWG, nv1[k]);
      load_words<NWG>(a.v2 + row * NW + g * NWG, nv2[k]);
    }
    const int64_t tn = base + (lane & 31) < t1 ? base + (lane & 31) : t1 - 1;
    nkn = a.kn[rowbase + tn];
    nvn = a.vn[rowbase + tn];
  };

  // Before the block's tables are built, start the loads: this lane's part of query rows
  // p VW + vl (zero past the group's nq rows) and the first positions.
  // The chunk records this lane writes at the end (row p VW + vl of each pass, and the header
  // of query n for lanes g = 0) are located here, where the index arithmetic hides behind
  // the loads, rather than on the epilogue's critical path.
  uint4 qraw[NPASS];
  int64_t rec[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    qraw[p] = make_uint4(0u, 0u, 0u, 0u);
    rec[p] = 0;
  }
  int64_t hdr = 0;
  if (active) {
#pragma unroll
    for (int p = 0; p < NPASS; ++p)
      if (p * VW < nq && p * VW + vl < nq) {
        const int64_t qv = qvec(p * VW + vl);
        qraw[p] = reinterpret_cast<const uint4*>(a.q + qv * D + q * C)[0];
        rec[p] = (qv * a.n_splits + sp) * (D + 4) + 4 + q * C;
      }
    fetch(t0);
    if (n < nq) hdr = (qvec(n) * a.n_splits + sp) * (D + 4);
  }

  fill_mfma_table<BITS>(a.ztab_k, tabk);
  fill_mfma_table<BITS>(a.ztab_v, tabv);
  for (int m = threadIdx.x; m < D / 2; m += kBlockThreads) {
    const uint32_t s0 = (a.ksign[(2 * m) >> 5] >> ((2 * m) & 31)) & 1u;
    const uint32_t s1 = (a.ksign[(2 * m + 1) >> 5] >> ((2 * m + 1) & 31)) & 1u;
    kx[m] = (s0 ? 0x8000u : 0u) | (s1 ? 0x80000000u : 0u);
  }
  for (int i = threadIdx.x; i < (D + 31) / 32; i += kBlockThreads) vsg[i] = a.vsign[i];
  __syncthreads();
  if (!active) return;  // no barrier follows

  // 1. Rotated queries y = H diag(s_k) q (scaled by qscale) into stage[16][D]: rows below nq
  //    rotated (their lanes past nq hold zeros), whole passes past nq written as zeros.
  {
    const float qk = (__builtin_popcount(q) & 1) ? -a.qscale : a.qscale;
    const uint32_t w[4] = {kPP ^ kx[q * 4], kPP ^ kx[q * 4 + 1], kPP ^ kx[q * 4 + 2], kPP ^ kx[q * 4 + 3]};
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      float y[C] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (p * VW < nq) {  // wave-uniform
        const uint32_t xh[4] = {qraw[p].x, qraw[p].y, qraw[p].z, qraw[p].w};
        dot2_stages8(xh, w, y);
        lane_stages<C, 4>(y);
        cross_stages<C, LOG_L>(y, q);
      }
      float4* dst = reinterpret_cast<float4*>(stage + (p * VW + vl) * D + q * C);
      dst[0] = make_float4(y[0] * qk, y[1] * qk, y[2] * qk, y[3] * qk);
      dst[1] = make_float4(y[4] * qk, y[5] * qk, y[6] * qk, y[7] * qk);
    }
  }
  wave_lds_fence();

  // 2. Query operands: lane (n, g) takes query n's coordinates [CPL g, CPL g + CPL), divided by
  //    the query's largest magnitude qn (0 for padding queries).
  constexpr int HS = CPL / 4;  // score MFMA pairs per key block: 4 coordinates of the lane each
  u32x4_t qb1[HS], qb2[HS];
  float qn;
  {
    float qv[CPL];
#pragma unroll
    for (int c = 0; c < CPL / 4; ++c) {
      const float4 v = reinterpret_cast<const float4*>(stage + n * D + CPL * g)[c];
      qv[4 * c] = v.x; qv[4 * c + 1] = v.y; qv[4 * c + 2] = v.z; qv[4 * c + 3] = v.w;
    }
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(qv[j]));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    qn = mx;
    const float inv = mx > 0.f ? 1.0f / mx : 0.f;
#pragma unroll
    for (int j = 0; j < HS; ++j) {
      const uint2 p0 = split_pair(qv[4 * j] * inv, qv[4 * j + 1] * inv);
      const uint2 p1 = split_pair(qv[4 * j + 2] * inv, qv[4 * j + 3] * inv);
      qb1[j] = query_operand<BITS>(p0, p1, 0);
      qb2[j] = query_operand<BITS>(p0, p1, 1);
    }
  }
  wave_lds_fence();

  // Softmax state of query n: reference m (base 2) of the scores and this lane's sum l of
  // 2^(s - m); the value weights 2^(s - m) n_v are kept against their own reference mv of
  // s + log2 n_v (so they fit fp16 whatever the norms), and the accumulator is put back on m
  // at the end.
  float m = -FLT_MAX, mv = -FLT_MAX, l = 0.f;
  f32x4_t acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float* nw = nrm[wv];

  for (int64_t base = t0; base < t1; base += kMfmaKeys) {
    uint32_t k1[2][NWG], k2[2][NWG], v1[2][NWG], v2[2][NWG];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int w = 0; w < NWG; ++w) {
        k1[k][w] = nk1[k][w]; k2[k][w] = nk2[k][w]; v1[k][w] = nv1[k][w]; v2[k][w] = nv2[k][w];
      }
    wave_lds_fence();
    if (lane < 32) {
      nw[lane] = nkn;
      nw[kMfmaKeys + lane] = nvn;
    }
    wave_lds_fence();
    float kn[2][4], vn[2][4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float4 a4 = reinterpret_cast<const float4*>(nw + 16 * k + 4 * g)[0];
      const float4 b4 = reinterpret_cast<const float4*>(nw + kMfmaKeys + 16 * k + 4 * g)[0];
      kn[k][0] = a4.x; kn[k][1] = a4.y; kn[k][2] = a4.z; kn[k][3] = a4.w;
      vn[k][0] = b4.x; vn[k][1] = b4.y; vn[k][2] = b4.z; vn[k][3] = b4.w;
    }
    if (base + kMfmaKeys < t1) fetch(base + kMfmaKeys);

    // scores^T of the two key blocks
    f32x4_t sc[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t lo[NWG], hi[NWG];
      nibble_bytes<NWG>(k1[k], k2[k], lo, hi);
      sc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      static_for<0, HS>([&](auto ji) {
        constexpr int J = decltype(ji)::value;
        sc[k] = mfma2(key_operand<BITS, NWG, J>(lo, hi, tabk), qb1[J], qb2[J], sc[k]);
      });
    }

    // online softmax of query n over the 32 keys (keys 16 k + 4 g + j in this lane)
    float s[2][4], sv[2][4], mloc = -FLT_MAX, mvloc = -FLT_MAX;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool valid = base + 16 * k + 4 * g + j < t1;
        s[k][j] = valid ? sc[k][j] * qn * kn[k][j] : -FLT_MAX;
        sv[k][j] = valid ? s[k][j] + __builtin_amdgcn_logf(vn[k][j]) : -FLT_MAX;  // v_log_f32: log2
        mloc = __builtin_fmaxf(mloc, s[k][j]);
        mvloc = __builtin_fmaxf(mvloc, sv[k][j]);
      }
    mloc = __builtin_fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = __builtin_fmaxf(mloc, __shfl_xor(mloc, 32));
    mvloc = __builtin_fmaxf(mvloc, __shfl_xor(mvloc, 16));
    mvloc = __builtin_fmaxf(mvloc, __shfl_xor(mvloc, 32));
    if (mloc > m + kRefSlack) {
      l *= exp2_fast(m - mloc);
      m = mloc;
    }
    if (mvloc > mv + kRefSlack) {
      const float f = exp2_fast(mv - mvloc);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] *= f;
      mv = mvloc;
    }
    u32x4_t ph, pl;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        l += exp2_fast(s[k][j] - m);
        pw[j] = exp2_fast(sv[k][j] - mv);
      }
      const uint2 h0 = split_pair(pw[0], pw[1]), h1 = split_pair(pw[2], pw[3]);
      ph[2 * k] = h0.x;
      pl[2 * k] = h0.y;
      ph[2 * k + 1] = h1.x;
      pl[2 * k + 1] = h1.y;
    }

    // values of the 32 keys into the tile (row = key, 8-half chunks swizzled by row & 7)
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t lo[NWG], hi[NWG];
      nibble_bytes<NWG>(v1[k], v2[k], lo, hi);
      const int row = 16 * k + n;
      static_for<0, KS>([&](auto si) {
        constexpr int S = decltype(si)::value;
        u32x4_t vh, vlo;
        table_operand<BITS, NWG, S>(lo, hi, tabv, vh, vlo);
        const int ch = ((CPL * g + 8 * S) >> 3) ^ (row & 7);
        *reinterpret_cast<u32x4_t*>(vt + row * D + 8 * ch) = vh;
        *reinterpret_cast<u32x4_t*>(vt + VT + row * D + 8 * ch) = vlo;
      });
    }
    wave_lds_fence();

    // out^T += Z_v^T P^T: lane (n, g) reads coordinate 16 cb + n of keys 4 g + [0, 4) and
    // 16 + 4 g + [0, 4) (its k-slots 8 g + [0, 8)), transposed out of the tile
    {
      const int jr = n >> 2, jc = n & 3;  // this lane addresses row kb + jr, coordinates 4 jc..
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        u32x4_t vh, vlo;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int row = 16 * hlf + 4 * g + jr;
          const int ch = (2 * cb + (jc >> 1)) ^ (row & 7);
          const int off = row * D + 8 * ch + 4 * (jc & 1);
          typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
          const i16x4_t th = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)((__attribute__((address_space(3))) uint16_t*)(vt + off)));
          const i16x4_t tl = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)((__attribute__((address_space(3))) uint16_t*)(vt + VT + off)));
          const u32x2_t uh = __builtin_bit_cast(u32x2_t, th), ul = __builtin_bit_cast(u32x2_t, tl);
          vh[2 * hlf] = uh[0]; vh[2 * hlf + 1] = uh[1];
          vlo[2 * hlf] = ul[0]; vlo[2 * hlf + 1] = ul[1];
        }
        acc[cb] = mfma3(vh, vlo, ph, pl, acc[cb]);
      }
    }
  }

  // 5. The query's sum over the four lane groups, its accumulator (coordinates 16 cb + 4 g +
  //    [0, 4) of query n) through LDS into the codec's layout, rotated back, written.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  wave_lds_fence();
  const float back = exp2_fast(mv - m);  // accumulator from reference mv onto m
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
    reinterpret_cast<float4*>(stage + n * D + 16 * cb + 4 * g)[0] =
        make_float4(acc[cb][0] * back, acc[cb][1] * back, acc[cb][2] * back, acc[cb][3] * back);
  wave_lds_fence();
  if (g == 0 && n < nq) {
    float* ws = a.ws + hdr;
    ws[0] = m;
    ws[1] = l;
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    if (p * VW >= nq) break;  // wave-uniform: the group's rows are done
    const int i = p * VW + vl;
    const float4 v0 = reinterpret_cast<const float4*>(stage + i * D + q * C)[0];
    const float4 v1 = reinterpret_cast<const float4*>(stage + i * D + q * C)[1];
    float z[C] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    unrotate_f32<D, 8>(z, q, a.inv_sqrt_d, vsg);
    if (i < nq) {
      float4* wa = reinterpret_cast<float4*>(a.ws + rec[p]);
      wa[0] = make_float4(z[0], z[1], z[2], z[3]);
      wa[1] = make_float4(z[4], z[5], z[6], z[7]);
    }
  }
}

constexpr int kCombineThreads = 256;
constexpr int kMaxSplits = 4096;  // chunks per query vector (the host plan keeps below this)

// Coordinates per combine block.
template <int D>
constexpr int combine_slice() {
  return D < 64 ? D : 64;
}

// One block per (query vector, slice of 64 coordinates), in two passes so that no load waits
// on another: the chunks' maxima give M = max_s m_s, the weights f_s = 2^(m_s - M) (kept in
// LDS) and S = sum_s f_s l_s; then thread t sums f_s u_s over the chunks s = t / Q4 mod G of
// its coordinate quad t mod Q4 (Q4 quads in the slice, G = 256 / Q4 groups), the G partial
// sums meet in LDS, and out = RN16(sum / S). The records u_s are already rotated back.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void attend_combine(const AttendArgs a) {
  constexpr int SL = combine_slice<D>();
  constexpr int Q4 = SL / 4;
  constexpr int NG = kCombineThreads / Q4;

  __shared__ float fs[kMaxSplits];
  __shared__ float red[2][kCombineThreads / 64];
  __shared__ float4 pa[NG][Q4];
  const int64_t qv = blockIdx.x / (D / SL);
  const int c0 = static_cast<int>(blockIdx.x % (D / SL)) * SL;
  const float* wq = a.ws + qv * a.n_splits * (D + 4);
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

  // The records' coordinate quads of the first CPF chunks of this thread are loaded first:
  // they do not depend on pass 1, so their latency overlaps it.
  constexpr int CPF = 16;
  const int qd = t % Q4, grp = t / Q4;
  float4 pre[CPF];
#pragma unroll
  for (int r = 0; r < CPF; ++r) {
    const int sp = grp + r * NG;
    pre[r] = sp < a.n_splits ? reinterpret_cast<const float4*>(wq + sp * (D + 4) + 4 + c0)[qd]
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // pass 1: M, the weights, S; each chunk header {m, l} is read once, as one 8-byte load,
  // and kept in registers (a thread owns at most kMaxSplits / kCombineThreads chunks)
  constexpr int HPT = kMaxSplits / kCombineThreads;
  float2 ml[HPT];
  float M = -FLT_MAX;
#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int sp = t + k * kCombineThreads;
    ml[k] = sp < a.n_splits ? *reinterpret_cast<const float2*>(wq + sp * (D + 4)) : make_float2(-FLT_MAX, 0.f);
    M = __builtin_fmaxf(M, ml[k].x);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = __builtin_fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red[0][wv] = M;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kCombineThreads / 64; ++k) M = __builtin_fmaxf(M, red[0][k]);
  float S = 0.f;
#pragma unroll
  for (int k = 0; k < HPT; ++k) {
    const int sp = t + k * kCombineThreads;
    if (sp < a.n_splits) {
      const float f = exp2_fast(ml[k].x - M);
      fs[sp] = f;
      S += f * ml[k].y;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) S += __shfl_xor(S, off);
  if (lane == 0) red[1][wv] = S;
  __syncthreads();
  S = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineThreads / 64; ++k) S += red[1][k];

  // pass 2: sum_s f_s u_s over this block's coordinates
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int r = 0; r < CPF; ++r) {
    const int sp = grp + r * NG;
    const float f = sp < a.n_splits ? fs[sp] : 0.f;
    acc.x = __builtin_fmaf(f, pre[r].x, acc.x);
    acc.y = __builtin_fmaf(f, pre[r].y, acc.y);
    acc.z = __builtin_fmaf(f, pre[r].z, acc.z);
    acc.w = __builtin_fmaf(f, pre[r].w, acc.w);
  }
#pragma unroll 8
  for (int sp = grp + CPF * NG; sp < a.n_splits; sp += NG) {
    const float f = fs[sp];
    const float4 v = reinterpret_cast<const float4*>(wq + sp * (D + 4) + 4 + c0)[qd];
    acc.x = __builtin_fmaf(f, v.x, acc.x);
    acc.y = __builtin_fmaf(f, v.y, acc.y);
    acc.z = __builtin_fmaf(f, v.z, acc.z);
    acc.w = __builtin_fmaf(f, v.w, acc.w);
  }
  pa[grp][qd] = acc;
  __syncthreads();
  if (t < Q4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int k = 0; k < NG; ++k) {
      const float4 u = pa[k][t];
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    const float r = 1.0f / S;
    const half2_t h0 = {static_cast<_Float16>(v.x * r), static_cast<_Float16>(v.y * r)};
    const half2_t h1 = {static_cast<_Float16>(v.z * r), static_cast<_Float16>(v.w * r)};
    reinterpret_cast<uint2*>(a.out + qv * D + c0)[t] =
        make_uint2(__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1));
  }
}

// ------------------------------------------------------------------------------ dispatch

template <int D, int BITS, int NQW>
static hipError_t launch_attend_t(const AttendArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AttendArgs*>(&a)};
  const int64_t units = (a.n_q / NQW) * a.n_splits;
  const int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > INT_MAX || a.n_q * (D / combine_slice<D>()) > INT_MAX) return hipErrorInvalidValue;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attend_partial<D, BITS, NQW>),
                                 dim3(static_cast<int>(blocks)), dim3(kBlockThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&attend_combine<D>),
                         dim3(static_cast<int>(a.n_q * (D / combine_slice<D>()))), dim3(kCombineThreads), args, 0,
                         stream);
}

// The matrix-core partial pass (16 query vectors per wave unit), then the combine.
template <int D, int BITS>
static hipError_t launch_attend_mfma_t(const AttendArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AttendArgs*>(&a)};
  const int64_t gq = static_cast<int64_t>(a.group) * a.Sq;
  const int64_t units = (a.n_q / gq) * ((gq + kMfmaQ - 1) / kMfmaQ) * a.n_splits;
  const int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > INT_MAX || a.n_q * (D / combine_slice<D>()) > INT_MAX) return hipErrorInvalidValue;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attend_mfma<D, BITS>),
                                 dim3(static_cast<int>(blocks)), dim3(kBlockThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&attend_combine<D>),
                         dim3(static_cast<int>(a.n_q * (D / combine_slice<D>()))), dim3(kCombineThreads), args, 0,
                         stream);
}

template <int D, int BITS>
static auto attend_nqw(int nqw) -> hipError_t (*)(const AttendArgs&, hipStream_t) {
  if constexpr ((D == 64 || D == 128) && BITS != 3 && D * BITS >= 128) {
    if (nqw == kMfmaQ) return launch_attend_mfma_t<D, BITS>;
  }
  if (nqw == 1) return launch_attend_t<D, BITS, 1>;
  if constexpr (D <= 512) {
    if (nqw == 2) return launch_attend_t<D, BITS, 2>;
    if (nqw == 4) return launch_attend_t<D, BITS, 4>;
  }
  return nullptr;
}

template <int D>
static auto attend_fn(int bits, int nqw) -> hipError_t (*)(const AttendArgs&, hipStream_t) {
  switch (bits) {
    case 1: return attend_nqw<D, 1>(nqw);
    case 2: return attend_nqw<D, 2>(nqw);
    case 3: return attend_nqw<D, 3>(nqw);
    case 4: return attend_nqw<D, 4>(nqw);
    default: return nullptr;
  }
}

// Launcher used by api.cpp: both kernels on `stream`, the combine after the partials.
// nqw: query vectors per wave: 16 selects the matrix-core pass (d = 64 or 128, b = 1, 2 or
// 4, d b >= 128); else 1, 2 or 4 (a divisor of group * Sq; 1 for d = 1024).
// ------------------------------------------------------------------------------ scratch

// Device scratch of the allocation-free attention entry point (kvq_rvq_attend_noalloc): the
// per-(query vector, chunk) records of the partial pass live here instead of in a caller's
// workspace. One copy per device, held from the library's load until the process ends. The
// partial pass rewrites every record the combine pass reads, so nothing needs clearing
// between calls; calls that overlap on one device share it and race.
static __device__ __align__(256) float scratch[kAttendScratchBytes / sizeof(float)];

// Device address of this device's scratch array, looked up with the device current at the
// first call on each device and kept (a host-side use of the array's name would be a
// host-side stand-in, not its device address). Two threads racing on the first call both
// store the same address.
hipError_t attend_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_attend(const AttendArgs& a, int d, int bits, int nqw, hipStream_t stream) {
  hipError_t (*f)(const AttendArgs&, hipStream_t) = nullptr;
  switch (d) {
    case 8: f = attend_fn<8>(bits, nqw); break;
    case 16: f = attend_fn<16>(bits, nqw); break;
    case 32: f = attend_fn<32>(bits, nqw); break;
    case 64: f = attend_fn<64>(bits, nqw); break;
    case 128: f = attend_fn<128>(bits, nqw); break;
    case 256: f = attend_fn<256>(bits, nqw); break;
    case 512: f = attend_fn<512>(bits, nqw); break;
    case 1024: f = attend_fn<1024>(bits, nqw); break;
    default: break;
  }
  return f ? f(a, stream) : hipErrorInvalidValue;
}

}  // namespace kvq
