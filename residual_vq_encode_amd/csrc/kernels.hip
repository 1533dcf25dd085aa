// HIP kernels for gfx950 (MI355X): fused encode+pack and unpack+decode of the two-stage
// residual-VQ KV-cache codec.
//
// Method (VeloxQuant-MLX blog): "rvq" tag page, "The pipeline, as it actually runs"
// (normalise, rotate, stage-1 Gaussian codebook, residual, stage-2 Laplacian-fit codebook,
// two separately packed streams), "What 'quantize' means here, precisely" (a code is the
// number of boundaries the value exceeds) and "The kernel" (float32 residual, LSB-first
// packing into uint32 words); "turboquant" tag page, "Kernel 3" (y = H diag(s) x / sqrt(D),
// the sign flip before the butterfly) and "Kernel 5" (dequantized coordinate
// c1[i1] + c2[i2]).
//
// The pages' Metal kernel runs one threadgroup per vector and one thread per coordinate,
// stages codes in threadgroup memory and packs them after a barrier. Here a vector of D
// coordinates is spread over L = D / C lanes of a 64-wide wavefront, C = min(D, 32)
// consecutive coordinates per lane, so a wave works on 64 / L vectors at a time (a tile):
//  * the tile (64 * C fp16 values, contiguous in HBM) is streamed into the wave's own LDS
//    buffer with coalesced 16-byte direct-to-LDS loads (global_load_lds_dwordx4); each lane
//    reads its C coordinates back. The 16-byte chunks are XOR-swizzled so those reads are
//    bank-conflict free. The next tile's loads are issued as soon as the current tile has
//    left LDS, so they fly while the current tile is computed;
//  * the Walsh-Hadamard transform runs its log2 C low stages in registers and its log2 L
//    high stages across lanes (DPP quad permutes / row rotates, or ds_swizzle), each
//    butterfly output one instruction (see cross_stage). The sign flip diag(s) is an exact
//    XOR of fp16 sign bits; the first two stages read the flipped fp16 pairs directly
//    (v_dot2 with (1, 1) and (1, -1) weights: one instruction per output, exact products);
//  * quantization is branch-free; codes are shifted into their words with v_alignbit /
//    shift-or as they are produced, so no code leaves registers (3-bit codes, whose 10-code
//    words straddle lanes, are regrouped through LDS).
// Small per-lane state (32 coordinates) keeps many waves resident per SIMD, and a tile is
// short, so loads of some waves overlap the arithmetic of others and the launch has little
// tail. No MFMA: the transform is O(D log D) additions with +-1 coefficients, and the
// kernel is bound by HBM bandwidth, not by a dense contraction.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>

#include "params.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// How one vector of D coordinates maps onto lanes.
template <int D>
struct Layout {
  static constexpr int C = D < 32 ? D : 32;       // coordinates per lane
  static constexpr int L = D / C;                 // lanes per vector
  static constexpr int LOG_L = __builtin_ctz(L);  // butterfly stages across lanes
  static constexpr int VW = 64 / L;               // vectors per wave tile
  static constexpr int CH = C / 8;                // 16-byte input chunks per lane
  static_assert(D >= 8 && D <= 1024 && (D & (D - 1)) == 0, "D must be a power of two in [8, 1024]");
};

// Residency targets (waves per SIMD); the register allocator is held to 512 / target VGPRs.
constexpr int kEncodeWavesPerEU = 4;
constexpr int kDecodeWavesPerEU = 4;

// ------------------------------------------------------------------------------ helpers

// LDS chunk swizzle for a wave buffer of 64 rows (one per lane) x CH 16-byte chunks. Any
// 16 consecutive lanes then touch 16 distinct 16-byte bank groups, both when a lane writes
// chunk (64k + lane) of the tile and when lane r reads chunk c of its own row r.
template <int CH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CH >= 16) {
    return row & 15;
  } else {
    return (row / (16 / CH)) & (CH - 1);
  }
}

// Orders this wave's LDS accesses: LDS operations of one wave are executed in order, so
// only the compiler needs to be kept from moving accesses across.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Explicit waits: every vector-memory operation of this wave has completed (the tile's
// direct-to-LDS loads have landed), and every LDS operation of this wave has completed
// (the tile buffer may be overwritten).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Cache-policy operand of the direct-to-LDS load: NT (non-temporal). The input is read
// exactly once, so it should not displace anything in the caches.
constexpr int kNonTemporal = 2;

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// fp16x2 dot products with a float32 addend, the non-accumulating (VOP3P) form: the
// compiler otherwise picks the accumulating v_dot2c and spends a move zeroing each
// destination. `w` holds two fp16 weights (low half weighs the pair's first element);
// NEG selects the VOP3P source modifiers applied to it: 0 = (w0, w1), 1 = (w0, -w1),
// 2 = (-w0, -w1), 3 = (-w0, w1). With w = (s_a, s_b), the rotation's signs for the pair,
// this multiplies the pair by (+-s_a, +-s_b) exactly: the sign flip costs nothing.
constexpr uint32_t kPP = 0x3C003C00u;  // fp16 (+1, +1)

template <int NEG>
__device__ __forceinline__ float dot2_f16(uint32_t pair, uint32_t w) {
  float r;
  if constexpr (NEG == 0) asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(pair), "v"(w));
  if constexpr (NEG == 1) asm("v_dot2_f32_f16 %0, %1, %2, 0 neg_hi:[0,1,0]" : "=v"(r) : "v"(pair), "v"(w));
  if constexpr (NEG == 2)
    asm("v_dot2_f32_f16 %0, %1, %2, 0 neg_lo:[0,1,0] neg_hi:[0,1,0]" : "=v"(r) : "v"(pair), "v"(w));
  if constexpr (NEG == 3) asm("v_dot2_f32_f16 %0, %1, %2, 0 neg_lo:[0,1,0]" : "=v"(r) : "v"(pair), "v"(w));
  return r;
}
template <int NEG>
__device__ __forceinline__ float dot2_f16(uint32_t pair, uint32_t w, float addend) {
  float r;
  if constexpr (NEG == 0) asm("v_dot2_f32_f16 %0, %1, %2, %3" : "=v"(r) : "v"(pair), "v"(w), "v"(addend));
  if constexpr (NEG == 1)
    asm("v_dot2_f32_f16 %0, %1, %2, %3 neg_hi:[0,1,0]" : "=v"(r) : "v"(pair), "v"(w), "v"(addend));
  if constexpr (NEG == 2)
    asm("v_dot2_f32_f16 %0, %1, %2, %3 neg_lo:[0,1,0] neg_hi:[0,1,0]" : "=v"(r) : "v"(pair), "v"(w), "v"(addend));
  if constexpr (NEG == 3)
    asm("v_dot2_f32_f16 %0, %1, %2, %3 neg_lo:[0,1,0]" : "=v"(r) : "v"(pair), "v"(w), "v"(addend));
  return r;
}

// The value held by lane (lane ^ M). M = 1, 2: DPP quad permutes; M = 8: DPP row rotate
// by 8 (within a 16-lane row that is lane ^ 8); M = 4, 16: ds_swizzle in bit-mask mode
// (and 0x1f, xor M, within each group of 32 lanes).
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  const int b = __builtin_bit_cast(int, v);
  int r;
  if constexpr (M == 1) {
    r = __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (M == 2) {
    r = __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (M == 8) {
    r = __builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true);  // row_ror:8
  } else {
    static_assert(M == 4 || M == 16, "partner mask");
    r = __builtin_amdgcn_ds_swizzle(b, 0x1F | (M << 10));
  }
  return __builtin_bit_cast(float, r);
}

// One butterfly stage across lanes: lane pairs (p, p ^ M), p the one with that bit clear,
// must become (a + b, a - b) for their values (a, b). Each lane instead computes
// fma(partner, beta, own) with beta = +1 on the lower lane and -1 on the upper one: the
// lower lane gets a + b, the upper lane b - a = -(a - b), each exactly one rounding of the
// true result. The upper lane's results are thus negated; applied from the lowest lane bit
// up, the negations compose to a per-lane sign (-1)^popcount(q) on the finished transform
// (q = the lane's index within its vector), which the caller folds into its scale. (Before
// the stage on bit t, the sign of a lane depends only on its lower bits, so both lanes of
// a pair carry the same sign and beta is always +-1 as stated.)
template <int C, int M>
__device__ __forceinline__ void cross_stage(float (&y)[C], float beta) {
  if constexpr (M == 1 || M == 2 || M == 8) {
    // v_fmac_f32 with the partner read through DPP: one instruction per output. (The
    // compiler keeps a separate v_mov_b32_dpp in front of a v_fmac, so this is written
    // out.) A DPP source must not have been written by a VALU instruction in the two
    // preceding issue slots; each group starts with s_nop 1 (two wait states), and inside a
    // group every instruction reads only the register it writes.
    static_assert(C % 8 == 0, "groups of 8");
#pragma unroll
    for (int i = 0; i < C; i += 8) {
#define KVQ_FMAC_DPP(CTRL)                                                                    \
  asm("s_nop 1\n"                                                                            \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"                     \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                        \
      : "+v"(y[i]), "+v"(y[i + 1]), "+v"(y[i + 2]), "+v"(y[i + 3]), "+v"(y[i + 4]), "+v"(y[i + 5]), \
        "+v"(y[i + 6]), "+v"(y[i + 7])                                                       \
      : "v"(beta))
      if constexpr (M == 1) {
        KVQ_FMAC_DPP("quad_perm:[1,0,3,2]");
      } else if constexpr (M == 2) {
        KVQ_FMAC_DPP("quad_perm:[2,3,0,1]");
      } else {
        KVQ_FMAC_DPP("row_ror:8");
      }
#undef KVQ_FMAC_DPP
    }
  } else {
#pragma unroll
    for (int i = 0; i < C; ++i) y[i] = __builtin_fmaf(xor_lane<M>(y[i]), beta, y[i]);
  }
}

template <int C, int LOG_L>
__device__ __forceinline__ void cross_stages(float (&y)[C], int q) {
  if constexpr (LOG_L >= 1) cross_stage<C, 1>(y, (q & 1) ? -1.f : 1.f);
  if constexpr (LOG_L >= 2) cross_stage<C, 2>(y, (q & 2) ? -1.f : 1.f);
  if constexpr (LOG_L >= 3) cross_stage<C, 4>(y, (q & 4) ? -1.f : 1.f);
  if constexpr (LOG_L >= 4) cross_stage<C, 8>(y, (q & 8) ? -1.f : 1.f);
  if constexpr (LOG_L >= 5) cross_stage<C, 16>(y, (q & 16) ? -1.f : 1.f);
}

// Sum over the L lanes of a vector (xor butterfly: every lane ends with the same value,
// since float addition is commutative).
template <int LOG_L>
__device__ __forceinline__ float lane_sum(float s) {
  if constexpr (LOG_L >= 1) s += xor_lane<1>(s);
  if constexpr (LOG_L >= 2) s += xor_lane<2>(s);
  if constexpr (LOG_L >= 3) s += xor_lane<4>(s);
  if constexpr (LOG_L >= 4) s += xor_lane<8>(s);
  if constexpr (LOG_L >= 5) s += xor_lane<16>(s);
  return s;
}

// In-register butterfly stages h = H0, 2 H0, ..., C/2 (natural order: lower <- a + b,
// upper <- a - b).
template <int C, int H0>
__device__ __forceinline__ void lane_stages(float (&y)[C]) {
#pragma unroll
  for (int h = H0; h < C; h <<= 1) {
#pragma unroll
    for (int p = 0; p < C / (2 * h); ++p) {
#pragma unroll
      for (int j = 0; j < h; ++j) {
        const float u = y[p * 2 * h + j], w = y[p * 2 * h + h + j];
        y[p * 2 * h + j] = u + w;
        y[p * 2 * h + h + j] = u - w;
      }
    }
  }
}

// Issues the direct-to-LDS loads of one tile (64 rows of CH chunks, row r = lane r's
// slice): instruction k writes LDS slots [64k, 64k + 64) (lane i -> slot 64k + i), and slot
// s = r*CH + c' of row r receives the row's global chunk c' ^ swz(r). Rows at or past
// nrows (the last, partial tile) re-read row nrows - 1, so every load stays inside the
// input; those rows are never used.
template <int CH>
__device__ __forceinline__ void dma_tile(uint4* buf, const uint4* src, int nrows, int lane) {
  const char* base = reinterpret_cast<const char*>(src);  // wave-uniform
  if (nrows == 64) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int slot = k * 64 + lane, r = slot / CH, c = (slot % CH) ^ swz<CH>(r);
      const uint32_t off = static_cast<uint32_t>(r * CH + c) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, kNonTemporal);
    }
  } else {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int slot = k * 64 + lane, r = slot / CH, c = (slot % CH) ^ swz<CH>(r);
      const int rr = r < nrows ? r : nrows - 1;
      const uint32_t off = static_cast<uint32_t>(rr * CH + c) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, kNonTemporal);
    }
  }
}

// Cache row of flattened input vector v0 + i: (v / S) * S_cap + s_offset + v % S.
// CONTIG (S == S_cap, s_offset == 0, chosen on the host) compiles to v0 + i. i < 64.
template <bool CONTIG>
__device__ __forceinline__ int64_t cache_row(const RowMap& m, int64_t v0, int i) {
  if constexpr (CONTIG) return v0 + i;
  const int64_t q0 = v0 / m.S;          // once per tile (wave-uniform)
  const int64_t s0 = v0 - q0 * m.S;
  int64_t t = s0 + i;                   // < S + 64
  int64_t q;
  if (m.S > 64) {
    q = (t >= m.S) ? 1 : 0;
  } else {                              // t < 128: the float quotient is within one
    const int ti = static_cast<int>(t), Si = static_cast<int>(m.S);
    int qi = static_cast<int>(static_cast<float>(ti) * m.inv_S);
    int r = ti - qi * Si;
    if (r < 0) { --qi; r += Si; } else if (r >= Si) { ++qi; r -= Si; }
    q = qi;
  }
  return (q0 + q) * m.S_cap + m.s_offset + (t - q * m.S);
}

// Packed words, written with non-temporal stores (nothing in this kernel reads them back,
// so they should not displace anything in the caches). dst is aligned to the store width.
template <int N>
__device__ __forceinline__ void store_words(uint32_t* dst, const uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const u32x4_t v = {w[i], w[i + 1], w[i + 2], w[i + 3]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst) + i / 4);
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const u32x2_t v = {w[i], w[i + 1]};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(dst) + i / 2);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) __builtin_nontemporal_store(w[i], dst + i);
  }
}

template <int N>
__device__ __forceinline__ void load_words(const uint32_t* src, uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const uint4 q = reinterpret_cast<const uint4*>(src)[i / 4];
      w[i] = q.x; w[i + 1] = q.y; w[i + 2] = q.z; w[i + 3] = q.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const uint2 q = reinterpret_cast<const uint2*>(src)[i / 2];
      w[i] = q.x; w[i + 1] = q.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = src[i];
  }
}

// Masks over the code fields of one word holding `cnt` codes of BITS bits.
template <int BITS>
constexpr uint32_t field_ones(int cnt) {  // bit 0 of every field
  uint32_t m = 0;
  for (int k = 0; k < cnt; ++k) m |= 1u << (BITS * k);
  return m;
}

// 3-bit codes held one per byte (bits 0..2 of each byte) <-> 10-code words (bits 3k..3k+2).
__device__ __forceinline__ uint32_t pack4x3(uint32_t e) {  // 4 byte codes -> 12 bits
  uint32_t x = e & 0x07070707u;
  x = (x | (x >> 5)) & 0x003F003Fu;
  return (x | (x >> 10)) & 0xFFFu;
}
__device__ __forceinline__ uint32_t unpack4x3(uint32_t v) {  // 12 bits -> 4 byte codes
  uint32_t x = v & 0xFFFu;
  x = (x | (x << 10)) & 0x003F003Fu;
  return (x | (x << 5)) & 0x07070707u;
}

// ------------------------------------------------------------------------------ encode

// Stage-1 and stage-2 codes of one coordinate (bits >= 3, bucket tables), as the count of
// boundaries below the value: the quantizers are symmetric, so the code is
// half + m (value > 0) or half - 1 - m (value <= 0), m = number of positive thresholds
// below the magnitude. nx = -y * unit1 (sign bit = [y > 0]); ay = |y'| for stage 2.
template <int BITS>
__device__ __forceinline__ void codes_bucket(float nx, float ay, float K2, int j1max, int j2max,
                                             const float4* t1s, const float2* t2s, uint32_t* c1,
                                             uint32_t* c2) {
  constexpr uint32_t HALF = 1u << (BITS - 1);
  const uint32_t p1 = __float_as_uint(nx) >> 31;
  const float ax = __builtin_fabsf(nx);
  const int j1 = static_cast<int>(__builtin_fminf(ax, static_cast<float>(j1max)));
  const float4 e = t1s[j1];
  const bool gt = ax > e.x;
  const uint32_t m1 = __float_as_uint(e.y) + (gt ? 1u : 0u);
  const float cm = gt ? e.w : e.z;
  const float x2 = __builtin_fmaf(ay, K2, -cm);  // residual magnitude in stage-2 units
  const uint32_t p2 = p1 ^ (__float_as_uint(x2) >> 31);
  const float ax2 = __builtin_fabsf(x2);
  const int j2 = static_cast<int>(__builtin_fminf(ax2, static_cast<float>(j2max)));
  const float2 e2 = t2s[j2];
  const uint32_t m2 = __float_as_uint(e2.y) + (ax2 > e2.x ? 1u : 0u);
  *c1 = p1 ? HALF + m1 : HALF - 1u - m1;
  *c2 = p2 ? HALF + m2 : HALF - 1u - m2;
}

// STAGES = 2: the two-stage residual codec (both code streams); STAGES = 1: the single-stage
// codec ("turboquant" tag page, "Kernel 3": rotate, then the nearest Gaussian Lloyd-Max
// centroid), stream 1 only.
template <int D, int BITS, bool CONTIG, int STAGES>
__global__ __launch_bounds__(kBlockThreads, kEncodeWavesPerEU) void encode_kernel(const EncodeArgs a) {
  using G = Layout<D>;
  constexpr int C = G::C, L = G::L, LOG_L = G::LOG_L, VW = G::VW, CH = G::CH;
  constexpr int EPW = 32 / BITS;                     // codes per word
  constexpr int NW = (D + EPW - 1) / EPW;            // words per vector per stream
  constexpr bool STAGED = BITS == 3 && L > 1;        // 10-code words straddle lanes
  constexpr int NWL = STAGED ? (NW + L - 1) / L : (L == 1 ? NW : C / EPW);  // words stored per lane
  constexpr int HALFM1 = (1 << (BITS - 1)) - 1;
  constexpr int CSTREAM = 64 * C / 4 + 4;            // STAGED: dwords per code stream (+ read pad)
  constexpr bool TWO = STAGES == 2;                  // stage 2 computed and stored

  __shared__ uint4 stage[kWavesPerBlock][64 * CH];
  __shared__ float4 t1s[BITS >= 3 ? kTab1Max : 1];
  __shared__ float2 t2s[BITS >= 3 ? kTab2Max : 1];
  __shared__ uint32_t cstage[STAGED ? kWavesPerBlock : 1][STAGED ? STAGES * CSTREAM : 1];
  if constexpr (BITS >= 3) {
    for (int i = threadIdx.x; i < kTab1Max; i += kBlockThreads)
      t1s[i] = make_float4(a.tab1[i][0], a.tab1[i][1], a.tab1[i][2], a.tab1[i][3]);
    for (int i = threadIdx.x; i < kTab2Max; i += kBlockThreads) t2s[i] = make_float2(a.tab2[i][0], a.tab2[i][1]);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int q = lane & (L - 1);   // this lane's part of its vector: coordinates [C q, C q + C)
  const int vl = lane >> LOG_L;   // its vector within the tile
  uint4* buf = stage[wv];
  // tile indices fit in 32 bits (checked at launch)
  const int n_tiles = static_cast<int>((a.n_vec + VW - 1) / VW);
  const int stride = static_cast<int>(gridDim.x) * kWavesPerBlock;
  const uint4* x16 = reinterpret_cast<const uint4*>(a.x);  // tile t starts at chunk 64 CH t
  // this lane's row inside the tile buffer: chunk c sits at slot (lane*CH + c) ^ swz(lane),
  // i.e. at `rbase ^ c` since the swizzle only touches the low log2(CH) bits
  const int rbase = lane * CH + swz<CH>(lane);
  // the transform of lane q comes out multiplied by (-1)^popcount(q) (see cross_stage)
  const bool negated = (__builtin_popcount(q) & 1) != 0;
  // fp16 weights (s_2p, s_2p+1) of this lane's C/2 coordinate pairs: the rotation's signs
  uint32_t wt[C / 2];
#pragma unroll
  for (int p = 0; p < C / 2; ++p) wt[p] = kPP ^ a.xmask[q * (C / 2) + p];

  int tile = static_cast<int>(blockIdx.x) * kWavesPerBlock + wv;
  if (tile < n_tiles) {
    const int64_t v0 = static_cast<int64_t>(tile) * VW;
    const int nv = static_cast<int>(a.n_vec - v0 < VW ? a.n_vec - v0 : VW);
    dma_tile<CH>(buf, x16 + static_cast<int64_t>(tile) * 64 * CH, nv * L, lane);
  }
  // The previous tile's results wait in registers until the current tile has been read out
  // of LDS: storing them right after they are computed would put the stores between the
  // next tile's loads and the wait for those loads, and the wait (which counts stores too)
  // would then also wait for the stores to be acknowledged.
  uint32_t w1[NWL], w2[NWL];
  float n_prev = 0.f;
  int64_t row_prev = -1;  // -1: nothing to store (first tile, or a lane past the last vector)
  for (; tile < n_tiles; tile += stride) {
    const int64_t v0 = static_cast<int64_t>(tile) * VW;
    const int nv = static_cast<int>(a.n_vec - v0 < VW ? a.n_vec - v0 : VW);

    // 1. The tile is in LDS once this wave's loads have landed. Read this lane's C
    //    coordinates chunk by chunk; each chunk (8 coordinates) goes straight into the
    //    squared norm and into the first two butterfly stages.
    //    Walsh-Hadamard transform of the sign-flipped vector, unnormalised: y' = H (s . x).
    //    Stages 1-2 of every 4 coordinates (fp16 pairs P0, P1 with sign weights W0, W1)
    //    come from v_dot2 with a float32 addend: s0 = P0.W0, d0 = P0.(W0 with the second
    //    weight negated), then P1.W1 + s0, P1.(w, -w) + d0, P1.(-w, -w) + s0,
    //    P1.(-w, w) + d0: 6 instructions for 4 outputs, exact products.
    // The wave raises its issue priority while it drains LDS and issues the next tile's
    // loads and the previous tile's stores, so those requests leave early, and drops it
    // again for the arithmetic.
    __builtin_amdgcn_s_setprio(2);
    wait_vmem();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float y[C];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint4 v = buf[rbase ^ c];
      const uint32_t xh[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2_t h = __builtin_bit_cast(half2_t, xh[i]);
        acc[i] = __builtin_amdgcn_fdot2(h, h, acc[i], false);
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t w0 = wt[4 * c + 2 * g], w1 = wt[4 * c + 2 * g + 1];
        const float s0 = dot2_f16<0>(xh[2 * g], w0);
        const float d0 = dot2_f16<1>(xh[2 * g], w0);
        float* o = y + 8 * c + 4 * g;
        o[0] = dot2_f16<0>(xh[2 * g + 1], w1, s0);
        o[1] = dot2_f16<1>(xh[2 * g + 1], w1, d0);
        o[2] = dot2_f16<2>(xh[2 * g + 1], w1, s0);
        o[3] = dot2_f16<3>(xh[2 * g + 1], w1, d0);
      }
    }
    wait_lds();

    // 2. Store the previous tile, then start loading the next tile into the buffer this
    //    tile has just left. Lanes hold consecutive slices of consecutive vectors, so a
    //    wave writes contiguous runs.
    if (row_prev >= 0) {
      if (q == 0) __builtin_nontemporal_store(n_prev, a.norms + row_prev);
      if constexpr (STAGED) {
#pragma unroll
        for (int k = 0; k < NWL; ++k) {
          const int w = q + L * k;
          if (w < NW) {
            __builtin_nontemporal_store(w1[k], a.p1 + row_prev * NW + w);
            if constexpr (TWO) __builtin_nontemporal_store(w2[k], a.p2 + row_prev * NW + w);
          }
        }
      } else {
        store_words<NWL>(a.p1 + row_prev * NW + q * NWL, w1);
        if constexpr (TWO) store_words<NWL>(a.p2 + row_prev * NW + q * NWL, w2);
      }
    }
    {
      const int nt = tile + stride;
      if (nt < n_tiles) {
        const int64_t w0 = static_cast<int64_t>(nt) * VW;
        const int nvn = static_cast<int>(a.n_vec - w0 < VW ? a.n_vec - w0 : VW);
        dma_tile<CH>(buf, x16 + static_cast<int64_t>(nt) * 64 * CH, nvn * L, lane);
      }
    }

    __builtin_amdgcn_s_setprio(0);

    // 3. Remaining butterfly stages: in registers, then across the vector's lanes.
    lane_stages<C, 4>(y);
    cross_stages<C, LOG_L>(y, q);
    const float n = __builtin_sqrtf(lane_sum<LOG_L>((acc[0] + acc[1]) + (acc[2] + acc[3])));
    __builtin_amdgcn_sched_barrier(0);

    // 4. Quantize both stages and pack. K maps the raw transform to the stage-1 unit with
    //    the sign flipped: NX = fma(y', -K, +0) = -(y_true * unit1) (K carries the lane's
    //    sign). Adding +0 turns an exact zero into +0, so sign(NX) is exactly [y_true > 0]
    //    (the count semantics at the middle boundary 0). A zero vector gets K = 0, so
    //    y_true = 0. The stage-2 value X2 = (|y_true| - cm) * unit2 is formed from y'
    //    directly (K2 = |K| * r12), one rounding.
    float K = (n > 0.f) ? a.k_scale * __builtin_amdgcn_rcpf(n) : 0.f;  // v_rcp_f32: 1 ulp
    const float K2 = K * a.r12;
    if (negated) K = -K;
    if constexpr (!STAGED) {
#pragma unroll
      for (int w = 0; w < NWL; ++w) {
        const int jlo = w * EPW;
        const int jhi = (w + 1) * EPW < C ? (w + 1) * EPW : C;
        const int cnt = jhi - jlo;
        uint32_t u1 = 0, u2 = 0;
#pragma unroll
        for (int j = jhi - 1; j >= jlo; --j) {  // highest code first: code jlo ends in bits [0, BITS)
          const float nx = __builtin_fmaf(y[j], -K, 0.0f);
          const float ax = __builtin_fabsf(nx);
          if constexpr (BITS == 1) {
            // stage 1: [y > 0] is the sign bit of NX; stage 2: sign of the residual magnitude
            u1 = __builtin_amdgcn_alignbit(u1, __float_as_uint(nx), 31);
            const float x2 = __builtin_fmaf(__builtin_fabsf(y[j]), K2, -a.cm2[0]);
            u2 = __builtin_amdgcn_alignbit(u2, __float_as_uint(x2), 31);
          } else if constexpr (BITS == 2) {
            // Unit 2/T1: bit 31 of NX is P = [y > 0], bit 30 is O = [|NX| >= 2] = [|y| >= T1].
            u1 = __builtin_amdgcn_alignbit(u1, __float_as_uint(nx), 30);
            // U = |NX| - 2 is |y| - T1 in units 2/T1. T1 is the midpoint of the two centroid
            // magnitudes c0 < c1, so the residual magnitude |y| - c (c the nearer one) is
            // sign(U) * (|U| T1/2 - h), h = (c1 - c0)/2. W = (|U| T1/2 - h) in stage-2 units
            // 2/T2 = |U| r12 - cm2[0]: its bit 31 is sign(W), bit 30 is [|W| >= 2] = [|r| >= T2].
            const float u = ax - 2.0f;
            const float w = __builtin_fmaf(__builtin_fabsf(u), a.r12, -a.cm2[0]);
            u2 = __builtin_amdgcn_alignbit(u2, __float_as_uint(w), 30);
          } else {
            // bucket tables: m = number of positive thresholds below |y|, in table units
            u1 = __builtin_amdgcn_alignbit(u1, __float_as_uint(nx), 31);
            const int j1 = static_cast<int>(__builtin_fminf(ax, static_cast<float>(a.j1max)));
            const float4 e = t1s[j1];
            const bool gt = ax > e.x;
            u1 = (u1 << (BITS - 1)) | (__float_as_uint(e.y) + (gt ? 1u : 0u));
            const float cm = gt ? e.w : e.z;
            const float x2 = __builtin_fmaf(__builtin_fabsf(y[j]), K2, -cm);
            u2 = __builtin_amdgcn_alignbit(u2, __float_as_uint(x2), 31);
            const float ax2 = __builtin_fabsf(x2);
            const int j2 = static_cast<int>(__builtin_fminf(ax2, static_cast<float>(a.j2max)));
            const float2 e2 = t2s[j2];
            u2 = (u2 << (BITS - 1)) | (__float_as_uint(e2.y) + (ax2 > e2.x ? 1u : 0u));
          }
        }
        // Word fixups. Each field holds (P, low) with P = [value > 0] for stage 1 and
        // Q = [residual magnitude < 0] for stage 2. Stage 2's sign is P2 = P1 xor Q (the
        // residual of a non-positive y is the negated magnitude). A field with P = 0 counts
        // downward from the middle: its low bits are (2^(BITS-1) - 1) - m = m xor
        // (2^(BITS-1) - 1); at BITS = 2 that low bit is O xor P xor 1 from the [>= T] bit the
        // alignbit stored.
        const uint32_t ones = field_ones<BITS>(cnt);
        const uint32_t hi = ones << (BITS - 1);
        if constexpr (BITS == 2) {
          // stage 2 holds (sign(W), [|W| >= 2]); its residual-magnitude sign is
          // Q = sign(U) xor sign(W) with sign(U) = not O, so P2 = P xor not O xor sign(W)
          u2 ^= ((u1 ^ (u1 >> 1) ^ ones) & ones) << 1;
          u1 ^= ~(u1 >> 1) & ones;
          u2 ^= ~(u2 >> 1) & ones;
        } else {
          u2 ^= u1 & hi;
        }
        if constexpr (BITS >= 3) {
          const uint32_t n1 = ~(u1 >> (BITS - 1)) & ones;
          const uint32_t n2 = ~(u2 >> (BITS - 1)) & ones;
          u1 ^= n1 * static_cast<uint32_t>(HALFM1);
          u2 ^= n2 * static_cast<uint32_t>(HALFM1);
        }
        w1[w] = u1;
        w2[w] = u2;
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // 3-bit codes: one byte per code into LDS (lane l's C codes at bytes [C l, C l + C) of
      // each stream, i.e. vector vl's codes at [D vl, D vl + D)), then lane q of a vector
      // packs words q, q + L, ... from ten consecutive bytes each.
      uint32_t* cs = cstage[wv];
#pragma unroll
      for (int d4 = 0; d4 < C / 4; ++d4) {
        uint32_t b1 = 0, b2 = 0;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          const int j = 4 * d4 + i;
          uint32_t c1, c2;
          codes_bucket<BITS>(__builtin_fmaf(y[j], -K, 0.0f), __builtin_fabsf(y[j]), K2, a.j1max, a.j2max, t1s,
                             t2s, &c1, &c2);
          b1 = (b1 << 8) | c1;
          b2 = (b2 << 8) | c2;
        }
        cs[lane * (C / 4) + d4] = b1;
        if constexpr (TWO) cs[CSTREAM + lane * (C / 4) + d4] = b2;
      }
      wave_lds_fence();
#pragma unroll
      for (int k = 0; k < NWL; ++k) {
        const int w = q + L * k;
        const int wc = w < NW ? w : NW - 1;           // lanes without a k-th word repeat the last
        const int base = vl * D + 10 * wc;            // byte offset of the word's first code
        const int s = (base & 3) * 8;                 // 0 or 16 (base is even)
        const int cnt = D - 10 * wc < 10 ? D - 10 * wc : 10;
        const uint32_t keep = cnt == 10 ? 0x3FFFFFFFu : (1u << (3 * cnt)) - 1u;
#pragma unroll
        for (int st = 0; st < STAGES; ++st) {
          const uint32_t* p = cs + st * CSTREAM + (base >> 2);
          const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
          const uint32_t e0 = __builtin_amdgcn_alignbit(d1, d0, s);
          const uint32_t e1 = __builtin_amdgcn_alignbit(d2, d1, s);
          const uint32_t e2 = d2 >> s;
          const uint32_t wd = (pack4x3(e0) | (pack4x3(e1) << 12) | (pack4x3(e2 & 0xFFFFu) << 24)) & keep;
          if (st == 0) w1[k] = wd; else w2[k] = wd;
        }
      }
      wave_lds_fence();
    }
    n_prev = n;
    row_prev = (vl < nv) ? cache_row<CONTIG>(a.map, v0, vl) : -1;
  }
  if (row_prev >= 0) {
    if (q == 0) __builtin_nontemporal_store(n_prev, a.norms + row_prev);
    if constexpr (STAGED) {
#pragma unroll
      for (int k = 0; k < NWL; ++k) {
        const int w = q + L * k;
        if (w < NW) {
          __builtin_nontemporal_store(w1[k], a.p1 + row_prev * NW + w);
          if constexpr (TWO) __builtin_nontemporal_store(w2[k], a.p2 + row_prev * NW + w);
        }
      }
    } else {
      store_words<NWL>(a.p1 + row_prev * NW + q * NWL, w1);
      if constexpr (TWO) store_words<NWL>(a.p2 + row_prev * NW + q * NWL, w2);
    }
  }
}

// ------------------------------------------------------------------------------ decode

// STAGES = 2: z = c1[i1] + c2[i2]; STAGES = 1: z = c1[i1] (the host fills the table so that
// entry (i1 << BITS) holds the right value in both cases).
template <int D, int BITS, bool CONTIG, int STAGES>
__global__ __launch_bounds__(kBlockThreads, kDecodeWavesPerEU) void decode_kernel(const DecodeArgs a) {
  using G = Layout<D>;
  constexpr int C = G::C, L = G::L, LOG_L = G::LOG_L, VW = G::VW, CH = G::CH;
  constexpr int EPW = 32 / BITS;
  constexpr int NW = (D + EPW - 1) / EPW;
  constexpr bool STAGED = BITS == 3 && L > 1;
  constexpr int NWL = STAGED ? (NW + L - 1) / L : (L == 1 ? NW : C / EPW);
  constexpr uint32_t MASK = (1u << BITS) - 1;
  constexpr int NZ = 1 << (2 * BITS);
  constexpr int CSTREAM = 64 * C / 4;  // STAGED: dwords per code stream
  constexpr bool TWO = STAGES == 2;

  __shared__ uint4 stage[kWavesPerBlock][64 * CH];
  __shared__ uint4 smask[D / 8];
  __shared__ float zt[NZ];
  __shared__ uint32_t cstage[STAGED ? kWavesPerBlock : 1][STAGED ? STAGES * CSTREAM : 1];
  for (int i = threadIdx.x; i < NZ; i += kBlockThreads) zt[i] = a.ztab[i];
  for (int i = threadIdx.x; i < D / 2; i += kBlockThreads) reinterpret_cast<uint32_t*>(smask)[i] = a.xmask[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane & (L - 1);
  const int vl = lane >> LOG_L;
  uint4* buf = stage[wv];
  const int n_tiles = static_cast<int>((a.n_vec + VW - 1) / VW);
  const int stride = static_cast<int>(gridDim.x) * kWavesPerBlock;
  const bool negated = (__builtin_popcount(q) & 1) != 0;

  // Software pipeline: the packed words and norm of the next tile are loaded into
  // registers while the current tile is computed, and the current tile's output is stored
  // at the start of the next iteration, after those loads have been issued.
  uint32_t nw1[NWL], nw2[NWL];  // next tile's words (STAGED: words q, q + L, ... of the vector)
  float nnrm = 1.0f;
  auto fetch = [&](int t) {
    const int64_t t0 = static_cast<int64_t>(t) * VW;
    const int tnv = static_cast<int>(a.n_vec - t0 < VW ? a.n_vec - t0 : VW);
    // lanes past the last vector read vector t0 (valid) and store nothing
    const int64_t row = cache_row<CONTIG>(a.map, t0, vl < tnv ? vl : 0);
    if constexpr (STAGED) {
#pragma unroll
      for (int k = 0; k < NWL; ++k) {
        const int w = q + L * k < NW ? q + L * k : NW - 1;
        nw1[k] = a.p1[row * NW + w];
        nw2[k] = TWO ? a.p2[row * NW + w] : 0u;
      }
    } else {
      load_words<NWL>(a.p1 + row * NW + q * NWL, nw1);
      if constexpr (TWO) {
        load_words<NWL>(a.p2 + row * NW + q * NWL, nw2);
      } else {
#pragma unroll
        for (int k = 0; k < NWL; ++k) nw2[k] = 0u;
      }
    }
    nnrm = a.norms ? a.norms[row] : 1.0f;
  };
  u32x4_t out[CH];          // previous tile's output chunks (chunk 64k + lane of that tile)
  int out_tile = -1, out_rows = 0;
  auto flush = [&]() {
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.x) + static_cast<int64_t>(out_tile) * 64 * CH;
#pragma unroll
    for (int k = 0; k < CH; ++k)
      if ((k * 64 + lane) / CH < out_rows) __builtin_nontemporal_store(out[k], dst + k * 64 + lane);
  };

  int tile = static_cast<int>(blockIdx.x) * kWavesPerBlock + wv;
  if (tile < n_tiles) fetch(tile);
  for (; tile < n_tiles; tile += stride) {
    const int64_t v0 = static_cast<int64_t>(tile) * VW;
    const int nv = static_cast<int>(a.n_vec - v0 < VW ? a.n_vec - v0 : VW);
    __builtin_amdgcn_s_setprio(2);
    uint32_t w1[NWL], w2[NWL];
#pragma unroll
    for (int k = 0; k < NWL; ++k) { w1[k] = nw1[k]; w2[k] = nw2[k]; }
    const float nrm = nnrm;
    if (out_tile >= 0) flush();
    if (tile + stride < n_tiles) fetch(tile + stride);
    __builtin_amdgcn_s_setprio(0);

    // 1. Codes of this lane's C coordinates, as (i1, i2) pairs -> z = c1[i1] + c2[i2].
    float z[C];
    if constexpr (!STAGED) {
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const uint32_t i1 = (w1[j / EPW] >> (BITS * (j % EPW))) & MASK;
        const uint32_t i2 = (w2[j / EPW] >> (BITS * (j % EPW))) & MASK;
        z[j] = zt[(i1 << BITS) | i2];
      }
    } else {
      // lane q of a vector unpacks its words q, q + L, ... into one byte per code in LDS
      uint32_t* cs = cstage[wv];
#pragma unroll
      for (int k = 0; k < NWL; ++k) {
        const int w = q + L * k;
        if (w < NW) {
          const int base = vl * D + 10 * w;  // even
          const int cnt = D - 10 * w < 10 ? D - 10 * w : 10;  // even
#pragma unroll
          for (int st = 0; st < STAGES; ++st) {
            const uint32_t wd = st == 0 ? w1[k] : w2[k];
            const uint32_t e0 = unpack4x3(wd), e1 = unpack4x3(wd >> 12), e2 = unpack4x3(wd >> 24);
            uint16_t* h = reinterpret_cast<uint16_t*>(cs + st * CSTREAM) + (base >> 1);
            const uint16_t hv[5] = {static_cast<uint16_t>(e0), static_cast<uint16_t>(e0 >> 16),
                                    static_cast<uint16_t>(e1), static_cast<uint16_t>(e1 >> 16),
                                    static_cast<uint16_t>(e2)};
#pragma unroll
            for (int i = 0; i < 5; ++i)
              if (2 * i < cnt) h[i] = hv[i];
          }
        }
      }
      wave_lds_fence();
#pragma unroll
      for (int d4 = 0; d4 < C / 4; ++d4) {
        const uint32_t b1 = cs[lane * (C / 4) + d4], b2 = TWO ? cs[CSTREAM + lane * (C / 4) + d4] : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t i1 = (b1 >> (8 * i)) & MASK, i2 = (b2 >> (8 * i)) & MASK;
          z[4 * d4 + i] = zt[(i1 << BITS) | i2];
        }
      }
      wave_lds_fence();
    }

    // 2. Inverse rotation: H z (H symmetric), in registers then across lanes; then the
    //    scale n / sqrt(D) (carrying the lane's sign) and the final sign flip.
    lane_stages<C, 1>(z);
    cross_stages<C, LOG_L>(z, q);
    float K = nrm * a.inv_sqrt_d;
    if (negated) K = -K;
    uint32_t o[C / 2];
#pragma unroll
    for (int m = 0; m < C / 2; ++m) {
      const half2_t h = {static_cast<_Float16>(z[2 * m] * K), static_cast<_Float16>(z[2 * m + 1] * K)};
      o[m] = __builtin_bit_cast(uint32_t, h);
    }

    // 3. Exact sign flip (XOR of fp16 sign bits) and transpose through LDS into the chunk
    //    order of the (contiguous) output tile, for coalesced 16-byte stores.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint4 mk = smask[q * CH + c];
      buf[lane * CH + (c ^ swz<CH>(lane))] =
          make_uint4(o[4 * c] ^ mk.x, o[4 * c + 1] ^ mk.y, o[4 * c + 2] ^ mk.z, o[4 * c + 3] ^ mk.w);
    }
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int g = k * 64 + lane, r = g / CH, c = g % CH;
      const uint4 v = buf[r * CH + (c ^ swz<CH>(r))];
      out[k] = u32x4_t{v.x, v.y, v.z, v.w};
    }
    wave_lds_fence();
    out_tile = tile;
    out_rows = nv * L;
  }
  if (out_tile >= 0) flush();
}

// ------------------------------------------------------------------------------ dispatch

// Blocks of one kernel resident on the whole current device at once.
static int resident_blocks(const void* f) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kBlockThreads, 0) != hipSuccess) return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

// Persistent grid: as many blocks as fit on the device at once (every wave resident from
// the start, walking tiles with a grid stride and loading its next tile while it computes
// the current one), fewer if there are fewer tiles. The resident count is cached per
// kernel (one value per process; all MI355X devices have the same count).
static hipError_t launch(const void* f, void* args, int64_t n_vec, int vw, int* cap, hipStream_t stream) {
  const int64_t tiles = (n_vec + vw - 1) / vw;
  if (tiles > INT_MAX) return hipErrorInvalidValue;
  if (*cap <= 0) *cap = resident_blocks(f);  // a benign race: every caller computes the same value
  if (*cap <= 0) return hipErrorInvalidValue;
  const int64_t want = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  const int blocks = static_cast<int>(want < *cap ? want : *cap);
  void* a[] = {args};
  return hipLaunchKernel(f, dim3(blocks), dim3(kBlockThreads), a, 0, stream);
}

template <int D, int BITS, int STAGES>
static hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t stream) {
  static int cap[2] = {0, 0};
  const bool c = a.map.contiguous != 0;
  const void* f = c ? reinterpret_cast<const void*>(&encode_kernel<D, BITS, true, STAGES>)
                    : reinterpret_cast<const void*>(&encode_kernel<D, BITS, false, STAGES>);
  return launch(f, const_cast<EncodeArgs*>(&a), a.n_vec, Layout<D>::VW, &cap[c ? 1 : 0], stream);
}

template <int D, int BITS, int STAGES>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  static int cap[2] = {0, 0};
  const bool c = a.map.contiguous != 0;
  const void* f = c ? reinterpret_cast<const void*>(&decode_kernel<D, BITS, true, STAGES>)
                    : reinterpret_cast<const void*>(&decode_kernel<D, BITS, false, STAGES>);
  return launch(f, const_cast<DecodeArgs*>(&a), a.n_vec, Layout<D>::VW, &cap[c ? 1 : 0], stream);
}

#define KVQ_FOR_BITS(MACRO, D, S) \
  case 1: return MACRO<D, 1, S>; case 2: return MACRO<D, 2, S>; case 3: return MACRO<D, 3, S>; case 4: return MACRO<D, 4, S>;

template <int D>
static auto encode_fn(int bits, int stages) -> hipError_t (*)(const EncodeArgs&, hipStream_t) {
  if (stages == 2) {
    switch (bits) { KVQ_FOR_BITS(launch_encode_t, D, 2) }
  } else if (stages == 1) {
    switch (bits) { KVQ_FOR_BITS(launch_encode_t, D, 1) }
  }
  return nullptr;
}
template <int D>
static auto decode_fn(int bits, int stages) -> hipError_t (*)(const DecodeArgs&, hipStream_t) {
  if (stages == 2) {
    switch (bits) { KVQ_FOR_BITS(launch_decode_t, D, 2) }
  } else if (stages == 1) {
    switch (bits) { KVQ_FOR_BITS(launch_decode_t, D, 1) }
  }
  return nullptr;
}

#define KVQ_FOR_D(FN, bits, stages)               \
  switch (d) {                                    \
    case 8: f = FN<8>(bits, stages); break;       \
    case 16: f = FN<16>(bits, stages); break;     \
    case 32: f = FN<32>(bits, stages); break;     \
    case 64: f = FN<64>(bits, stages); break;     \
    case 128: f = FN<128>(bits, stages); break;   \
    case 256: f = FN<256>(bits, stages); break;   \
    case 512: f = FN<512>(bits, stages); break;   \
    case 1024: f = FN<1024>(bits, stages); break; \
    default: break;                               \
  }

// Launchers used by api.cpp. Return hipErrorInvalidValue for an unsupported (d, bits,
// stages) or more than 2^31 - 1 tiles.
hipError_t launch_encode(const EncodeArgs& a, int d, int bits, int stages, hipStream_t stream) {
  hipError_t (*f)(const EncodeArgs&, hipStream_t) = nullptr;
  KVQ_FOR_D(encode_fn, bits, stages)
  return f ? f(a, stream) : hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int d, int bits, int stages, hipStream_t stream) {
  hipError_t (*f)(const DecodeArgs&, hipStream_t) = nullptr;
  KVQ_FOR_D(decode_fn, bits, stages)
  return f ? f(a, stream) : hipErrorInvalidValue;
}

}  // namespace kvq
