// HIP kernels for gfx950 (MI355X): fused encode+pack and unpack+decode of the two-stage
// residual-VQ KV-cache codec, one head vector per lane.
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
// stages codes in threadgroup memory and packs them after a barrier. Here each lane of a
// 64-wide wavefront owns a whole vector (D <= 128 coordinates in registers):
//  * a wave streams 64 consecutive vectors (one tile) straight from HBM into its own LDS
//    buffer with coalesced 16-byte direct-to-LDS loads (global_load_lds_dwordx4), then each
//    lane reads its row back; the 16-byte chunks are XOR-swizzled so the lane-per-row reads
//    are bank-conflict free. The next tile's loads are issued as soon as the current tile
//    has left LDS, so they fly while the current tile is computed (software pipelining
//    without spending registers on the prefetch);
//  * the Walsh-Hadamard transform runs entirely in registers (log2 D butterfly stages, no
//    cross-lane traffic, no barriers). The sign flip diag(s) is an exact XOR of the fp16
//    sign bits with per-pair masks read from a small LDS table (every lane reads the same
//    address, a broadcast); the first stage reads the flipped fp16 pairs directly
//    (v_dot2 with (1, 1) and (1, -1): one instruction per output, exact products);
//  * quantization is branch-free; codes are shifted into their words with v_alignbit /
//    shift-or as they are produced, so no code ever leaves registers.
// No MFMA: the transform is O(D log D) additions with +-1 coefficients, and the kernel is
// bound by HBM bandwidth, not by a dense contraction.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <utility>

#include "params.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------------------ helpers

// LDS chunk swizzle for a wave buffer of 64 rows x CH 16-byte chunks. Any 16 consecutive
// lanes then touch 16 distinct 16-byte bank groups, both when a lane writes chunk
// (64k + lane) of the tile and when lane r reads chunk c of row r.
template <int CH>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CH >= 16) {
    return row & 15;
  } else {
    return (row / (16 / CH)) & (CH - 1);
  }
}

// Orders this wave's LDS accesses around the transpose: LDS operations of one wave are
// executed in order, so only the compiler needs to be kept from moving accesses across.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Explicit waits: every vector-memory operation of this wave has completed (the tile's
// direct-to-LDS loads have landed), and every LDS read and scalar load of this wave has
// returned (the tile buffer may be overwritten; asm-issued scalar loads are usable).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// fp16x2 dot product with a float32 addend, the non-accumulating (VOP3P) form: the
// compiler otherwise picks the accumulating v_dot2c and spends a move zeroing each
// destination. `w` holds two fp16 weights (low half weighs the pair's first element).
constexpr uint32_t kPP = 0x3C003C00u;  // (+1, +1)
constexpr uint32_t kPM = 0xBC003C00u;  // (+1, -1)
constexpr uint32_t kMM = 0xBC00BC00u;  // (-1, -1)
constexpr uint32_t kMP = 0x3C00BC00u;  // (-1, +1)
__device__ __forceinline__ float dot2_f16(uint32_t pair, uint32_t w, float addend, bool zero_addend) {
  float r;
  if (zero_addend) {
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(pair), "s"(w));
  } else {
    asm("v_dot2_f32_f16 %0, %1, %2, %3" : "=v"(r) : "v"(pair), "s"(w), "v"(addend));
  }
  return r;
}

// Issues the direct-to-LDS loads of one tile: instruction k writes LDS slots
// [64k, 64k + 64) (lane i -> slot 64k + i), and slot s = r*CH + c' of row r receives
// the row's global chunk c' ^ swz(r). Rows at or past nv (the last, partial tile) re-read
// row nv - 1, so every load stays inside the input; those lanes' results are never stored.
template <int CH>
__device__ __forceinline__ void dma_tile(uint4* buf, const uint4* src, int nv, int lane) {
  const char* base = reinterpret_cast<const char*>(src);  // wave-uniform
  if (nv == 64) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int slot = k * 64 + lane, r = slot / CH, c = (slot % CH) ^ swz<CH>(r);
      const uint32_t off = static_cast<uint32_t>(r * CH + c) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int slot = k * 64 + lane, r = slot / CH, c = (slot % CH) ^ swz<CH>(r);
      const int rr = r < nv ? r : nv - 1;
      const uint32_t off = static_cast<uint32_t>(rr * CH + c) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, 0);
    }
  }
}

// Cache row of flattened input vector v0 + lane: (v / S) * S_cap + s_offset + v % S.
// CONTIG (S == S_cap, s_offset == 0, chosen on the host) compiles to v0 + lane.
template <bool CONTIG>
__device__ __forceinline__ int64_t cache_row(const RowMap& m, int64_t v0, int lane) {
  if constexpr (CONTIG) return v0 + lane;
  const int64_t q0 = v0 / m.S;          // once per tile (wave-uniform)
  const int64_t s0 = v0 - q0 * m.S;
  int64_t t = s0 + lane;                // < S + 64
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

template <int N>
__device__ __forceinline__ void store_words(uint32_t* dst, const uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      reinterpret_cast<uint4*>(dst)[i / 4] = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 2) reinterpret_cast<uint2*>(dst)[i / 2] = make_uint2(w[i], w[i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = w[i];
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

// ------------------------------------------------------------------------------ encode

template <int D, int BITS, bool CONTIG>
__global__ __launch_bounds__(kBlockThreads, 2) void encode_l1(const EncodeArgs a) {
  static_assert(D >= 8 && D <= 128 && (D & (D - 1)) == 0, "one vector per lane needs D <= 128");
  constexpr int CH = D / 8;                 // 16-byte chunks per vector
  constexpr int EPW = 32 / BITS;            // codes per word
  constexpr int NW = (D + EPW - 1) / EPW;   // words per vector per stream
  constexpr int HALFM1 = (1 << (BITS - 1)) - 1;

  __shared__ uint4 stage[kWavesPerBlock][64 * CH];
  __shared__ uint4 smask[CH];  // per-pair fp16 sign masks, 8 pairs per 16 bytes
  __shared__ float4 t1s[kTab1Max];
  __shared__ float2 t2s[kTab2Max];
  for (int i = threadIdx.x; i < D / 2; i += kBlockThreads) reinterpret_cast<uint32_t*>(smask)[i] = a.xmask[i];
  if constexpr (BITS >= 3) {
    for (int i = threadIdx.x; i < kTab1Max; i += kBlockThreads)
      t1s[i] = make_float4(a.tab1[i][0], a.tab1[i][1], a.tab1[i][2], a.tab1[i][3]);
    for (int i = threadIdx.x; i < kTab2Max; i += kBlockThreads) t2s[i] = make_float2(a.tab2[i][0], a.tab2[i][1]);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  uint4* buf = stage[wv];
  // tile indices fit in 32 bits: 2^31 tiles of 64 vectors of >= 16 bytes exceed any HBM
  const int n_tiles = static_cast<int>((a.n_vec + 63) >> 6);
  const int stride = static_cast<int>(gridDim.x) * kWavesPerBlock;
  const uint4* x16 = reinterpret_cast<const uint4*>(a.x);
  // this lane's row inside the tile buffer: chunk c sits at slot (lane*CH + c) ^ swz(lane),
  // i.e. at `rbase ^ c` since the swizzle only touches the low log2(CH) bits
  const int rbase0 = lane * CH + swz<CH>(lane);

  int tile = static_cast<int>(blockIdx.x) * kWavesPerBlock + wv;
  if (tile < n_tiles) {
    const int64_t v0 = static_cast<int64_t>(tile) << 6;
    dma_tile<CH>(buf, x16 + v0 * CH, static_cast<int>(a.n_vec - v0 < 64 ? a.n_vec - v0 : 64), lane);
  }
  for (; tile < n_tiles; tile += stride) {
    const int64_t v0 = static_cast<int64_t>(tile) << 6;
    const int nv = static_cast<int>(a.n_vec - v0 < 64 ? a.n_vec - v0 : 64);

    // 1. The tile is in LDS once this wave's loads have landed; read this lane's row,
    //    then start loading the next tile into the same buffer.
    wait_vmem();
    // `tile >> 31` is 0; it makes the lane's addresses loop-variant so they are recomputed
    // (one instruction each) rather than held in 2*CH registers across the loop
    const int rbase = rbase0 + (tile >> 31);
    uint32_t xh[D / 2];  // this lane's vector: fp16 pairs, sign-flipped
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint4 q = buf[rbase ^ c];
      const uint4 m = smask[c + (tile >> 31)];  // same address in every lane: a broadcast
      xh[4 * c] = q.x ^ m.x; xh[4 * c + 1] = q.y ^ m.y; xh[4 * c + 2] = q.z ^ m.z; xh[4 * c + 3] = q.w ^ m.w;
    }
    wait_lds();
    {
      const int nt = tile + stride;
      if (nt < n_tiles) {
        const int64_t w0 = static_cast<int64_t>(nt) << 6;
        dma_tile<CH>(buf, x16 + w0 * CH, static_cast<int>(a.n_vec - w0 < 64 ? a.n_vec - w0 : 64),
                     lane + (tile >> 31));
      }
    }

    // 2. Norm: sum of squares of the fp16 inputs, four float32 accumulators.
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 2; ++m) {
      const half2_t h = __builtin_bit_cast(half2_t, xh[m]);
      acc[m & 3] = __builtin_amdgcn_fdot2(h, h, acc[m & 3], false);
    }
    const float n = __builtin_sqrtf((acc[0] + acc[1]) + (acc[2] + acc[3]));

    // 3. Walsh-Hadamard transform of the sign-flipped vector, unnormalised: y' = H (s . x).
    //    The first two butterfly stages of every 4 coordinates (fp16 pairs P0, P1) come
    //    from v_dot2 with fp16 (+-1, +-1) weights and a float32 addend: s0 = P0.(1,1),
    //    d0 = P0.(1,-1), then P1.(1,1) + s0, P1.(1,-1) + d0, P1.(-1,-1) + s0, P1.(-1,1) + d0:
    //    6 instructions for 4 outputs, exact products. The remaining stages are float32
    //    additions in registers.
    float y[D];
#pragma unroll
    for (int q = 0; q < D / 4; ++q) {
      const float s0 = dot2_f16(xh[2 * q], kPP, 0.0f, true);
      const float d0 = dot2_f16(xh[2 * q], kPM, 0.0f, true);
      y[4 * q] = dot2_f16(xh[2 * q + 1], kPP, s0, false);
      y[4 * q + 1] = dot2_f16(xh[2 * q + 1], kPM, d0, false);
      y[4 * q + 2] = dot2_f16(xh[2 * q + 1], kMM, s0, false);
      y[4 * q + 3] = dot2_f16(xh[2 * q + 1], kMP, d0, false);
    }
#pragma unroll
    for (int h = 4; h < D; h <<= 1) {
#pragma unroll
      for (int p = 0; p < D / (2 * h); ++p) {
#pragma unroll
        for (int j = 0; j < h; ++j) {
          const float u = y[p * 2 * h + j], w = y[p * 2 * h + h + j];
          y[p * 2 * h + j] = u + w;
          y[p * 2 * h + h + j] = u - w;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 4. Quantize both stages and pack. K maps the raw transform to the stage-1 unit with
    //    the sign flipped: NX = fma(y', -K, +0) = -(y_true * unit1). Adding +0 turns an exact
    //    zero into +0, so sign(NX) is exactly [y_true > 0] (the count semantics at the middle
    //    boundary 0). A zero vector gets K = 0, so y_true = 0. The stage-2 value
    //    X2 = (|y_true| - cm) * unit2 is formed from y' directly (K2 = |K| * r12), one rounding.
    const float K = (n > 0.f) ? a.k_scale / n : 0.f;
    const float K2 = __builtin_fabsf(K) * a.r12;
    uint32_t w1[NW], w2[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int jlo = w * EPW;
      const int jhi = (w + 1) * EPW < D ? (w + 1) * EPW : D;
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
          const float cm = (ax >= 2.0f) ? a.cm2[1] : a.cm2[0];
          // residual magnitude |y| - cm in stage-2 units 2/T2: its sign bit is Q, bit 30 is [|r| >= T2]
          const float x2 = __builtin_fmaf(__builtin_fabsf(y[j]), K2, -cm);
          u2 = __builtin_amdgcn_alignbit(u2, __float_as_uint(x2), 30);
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
      // Q = [residual magnitude < 0] for stage 2. Stage 2's sign is P2 = P1 xor Q (the residual
      // of a non-positive y is the negated magnitude). A field with P = 0 counts downward
      // from the middle: its low bits are (2^(BITS-1) - 1) - m = m xor (2^(BITS-1) - 1);
      // at BITS = 2 that low bit is O xor P xor 1 from the [>= T] bit the alignbit stored.
      const uint32_t ones = field_ones<BITS>(cnt);
      const uint32_t hi = ones << (BITS - 1);
      u2 ^= u1 & hi;
      if constexpr (BITS == 2) {
        u1 ^= ~(u1 >> 1) & ones;
        u2 ^= ~(u2 >> 1) & ones;
      } else if constexpr (BITS >= 3) {
        const uint32_t n1 = ~(u1 >> (BITS - 1)) & ones;
        const uint32_t n2 = ~(u2 >> (BITS - 1)) & ones;
        u1 ^= n1 * static_cast<uint32_t>(HALFM1);
        u2 ^= n2 * static_cast<uint32_t>(HALFM1);
      }
      w1[w] = u1;
      w2[w] = u2;
      __builtin_amdgcn_sched_barrier(0);
    }

    // 5. Stores: each lane writes its own norm and 2 x NW words; lanes hold consecutive
    //    vectors, so a wave writes contiguous runs.
    if (lane < nv) {
      const int64_t row = cache_row<CONTIG>(a.map, v0, lane);
      a.norms[row] = n;
      store_words<NW>(a.p1 + row * NW, w1);
      store_words<NW>(a.p2 + row * NW, w2);
    }
  }
}

// ------------------------------------------------------------------------------ decode

template <int D, int BITS, bool CONTIG>
__global__ __launch_bounds__(kBlockThreads, 2) void decode_l1(const DecodeArgs a) {
  static_assert(D >= 8 && D <= 128 && (D & (D - 1)) == 0, "one vector per lane needs D <= 128");
  constexpr int CH = D / 8;
  constexpr int EPW = 32 / BITS;
  constexpr int NW = (D + EPW - 1) / EPW;
  constexpr uint32_t MASK = (1u << BITS) - 1;
  constexpr int NZ = 1 << (2 * BITS);

  __shared__ uint4 stage[kWavesPerBlock][64 * CH];
  __shared__ uint4 smask[CH];  // per-pair fp16 sign masks, 8 pairs per 16 bytes
  __shared__ float zt[NZ];
  for (int i = threadIdx.x; i < NZ; i += kBlockThreads) zt[i] = a.ztab[i];
  for (int i = threadIdx.x; i < D / 2; i += kBlockThreads) reinterpret_cast<uint32_t*>(smask)[i] = a.xmask[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  uint4* buf = stage[wv];
  const int64_t n_tiles = (a.n_vec + 63) >> 6;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;

  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wv; tile < n_tiles; tile += stride) {
    const int64_t v0 = tile << 6;
    const int nv = static_cast<int>(a.n_vec - v0 < 64 ? a.n_vec - v0 : 64);
    const int64_t row = cache_row<CONTIG>(a.map, v0, lane < nv ? lane : 0);

    uint32_t w1[NW], w2[NW];
    load_words<NW>(a.p1 + row * NW, w1);
    load_words<NW>(a.p2 + row * NW, w2);
    const float nrm = a.norms ? a.norms[row] : 1.0f;

    // dequantize in the rotated domain: z = c1[i1] + c2[i2]
    float z[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const uint32_t i1 = (w1[j / EPW] >> (BITS * (j % EPW))) & MASK;
      const uint32_t i2 = (w2[j / EPW] >> (BITS * (j % EPW))) & MASK;
      z[j] = zt[(i1 << BITS) | i2];
    }
    // inverse rotation: H z (H symmetric), then scale and the final sign flip
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
#pragma unroll
      for (int p = 0; p < D / (2 * h); ++p) {
#pragma unroll
        for (int j = 0; j < h; ++j) {
          const float u = z[p * 2 * h + j], w = z[p * 2 * h + h + j];
          z[p * 2 * h + j] = u + w;
          z[p * 2 * h + h + j] = u - w;
        }
      }
    }
    const float K = nrm * a.inv_sqrt_d;
    uint32_t o[D / 2];
#pragma unroll
    for (int m = 0; m < D / 2; ++m) {
      const half2_t h = {static_cast<_Float16>(z[2 * m] * K), static_cast<_Float16>(z[2 * m + 1] * K)};
      o[m] = __builtin_bit_cast(uint32_t, h);
    }

    // apply the final sign flip (exact XOR of fp16 sign bits; the mask reads are
    // broadcasts), transpose back through LDS and write the tile with coalesced stores
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint4 mk = smask[c + (tile >> 62)];
      buf[lane * CH + (c ^ swz<CH>(lane))] =
          make_uint4(o[4 * c] ^ mk.x, o[4 * c + 1] ^ mk.y, o[4 * c + 2] ^ mk.z, o[4 * c + 3] ^ mk.w);
    }
    wave_lds_fence();
    uint4* dst = reinterpret_cast<uint4*>(a.x) + v0 * CH;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int g = k * 64 + lane, r = g / CH, c = g % CH;
      const uint4 q = buf[r * CH + (c ^ swz<CH>(r))];
      if (r < nv) dst[g] = q;
    }
    wave_lds_fence();
  }
}

// ------------------------------------------------------------------------------ dispatch

template <int D, int BITS>
static hipError_t launch_encode_t(const EncodeArgs& a, int blocks, hipStream_t stream) {
  void* args[] = {const_cast<EncodeArgs*>(&a)};
  const void* f = a.map.contiguous ? reinterpret_cast<const void*>(&encode_l1<D, BITS, true>)
                                   : reinterpret_cast<const void*>(&encode_l1<D, BITS, false>);
  return hipLaunchKernel(f, dim3(blocks), dim3(kBlockThreads), args, 0, stream);
}

template <int D, int BITS>
static hipError_t launch_decode_t(const DecodeArgs& a, int blocks, hipStream_t stream) {
  void* args[] = {const_cast<DecodeArgs*>(&a)};
  const void* f = a.map.contiguous ? reinterpret_cast<const void*>(&decode_l1<D, BITS, true>)
                                   : reinterpret_cast<const void*>(&decode_l1<D, BITS, false>);
  return hipLaunchKernel(f, dim3(blocks), dim3(kBlockThreads), args, 0, stream);
}

#define KVQ_FOR_BITS(MACRO, D) \
  case 1: return MACRO<D, 1>; case 2: return MACRO<D, 2>; case 3: return MACRO<D, 3>; case 4: return MACRO<D, 4>;

template <int D>
static auto encode_fn(int bits) -> hipError_t (*)(const EncodeArgs&, int, hipStream_t) {
  switch (bits) { KVQ_FOR_BITS(launch_encode_t, D) }
  return nullptr;
}
template <int D>
static auto decode_fn(int bits) -> hipError_t (*)(const DecodeArgs&, int, hipStream_t) {
  switch (bits) { KVQ_FOR_BITS(launch_decode_t, D) }
  return nullptr;
}

// Launchers used by api.cpp. Return hipErrorInvalidValue for an unsupported (d, bits).
hipError_t launch_encode(const EncodeArgs& a, int d, int bits, int blocks, hipStream_t stream) {
  hipError_t (*f)(const EncodeArgs&, int, hipStream_t) = nullptr;
  switch (d) {
    case 8: f = encode_fn<8>(bits); break;
    case 16: f = encode_fn<16>(bits); break;
    case 32: f = encode_fn<32>(bits); break;
    case 64: f = encode_fn<64>(bits); break;
    case 128: f = encode_fn<128>(bits); break;
    default: break;
  }
  return f ? f(a, blocks, stream) : hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int d, int bits, int blocks, hipStream_t stream) {
  hipError_t (*f)(const DecodeArgs&, int, hipStream_t) = nullptr;
  switch (d) {
    case 8: f = decode_fn<8>(bits); break;
    case 16: f = decode_fn<16>(bits); break;
    case 32: f = decode_fn<32>(bits); break;
    case 64: f = decode_fn<64>(bits); break;
    case 128: f = decode_fn<128>(bits); break;
    default: break;
  }
  return f ? f(a, blocks, stream) : hipErrorInvalidValue;
}

}  // namespace kvq
