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
// stages codes in threadgroup memory and packs them after a barrier. Here:
//  * at D = 128 and 256 (encode_mx_kernel; not 3 bits at 256) a wave takes 16 vectors at a
//    time and runs the transform on the matrix cores as H_(D/32) (x) H_32: 2 D / 32
//    v_mfma_f32_16x16x32_f16 products of an fp16 +-1 H_32 slice with the sign-flipped fp16
//    inputs (exact products, float32 sums) and log2(D / 32) float32 butterfly stages across
//    the 32-coordinate blocks; each lane then quantizes 8 coordinates of every output
//    block, and 4 x 4 transposes of the code pieces across lane groups (v_permlane32_swap,
//    v_permlane16_swap) give each lane group a contiguous quarter of the vector's words;
//  * at every other D (encode_kernel) a vector of P coordinates (P = D, or the next power
//    of two for other head dimensions) is spread over L = P / C lanes of a 64-wide
//    wavefront, C = min(P, 32) consecutive coordinates per lane, and the Walsh-Hadamard
//    transform runs its log2 C low stages in registers and its log2 L high stages across
//    lanes (DPP quad permutes / row rotates, or ds_swizzle), each butterfly output one
//    instruction (see cross_stage); the sign flip diag(s) is exact, folded into the fp16
//    weights of the first two stages (v_dot2 with (+-1, +-1) weights, exact products);
//  * in both, a tile is streamed into the wave's own LDS buffer with coalesced 16-byte
//    direct-to-LDS loads (dwords for rows that are not 16-byte aligned), XOR-swizzled so
//    the lanes' reads back are bank-conflict free, and the next tile's loads are issued as
//    soon as the current tile has left LDS, so they fly while it is computed;
//  * quantization is branch-free; codes are shifted into their words with v_alignbit /
//    shift-or as they are produced (3-bit codes, whose 10-code words straddle lanes, are
//    cut from 96-bit slices and, for a contiguous cache, written back through LDS as one
//    run of 16-byte stores).
// The grids are persistent: every wave stays resident and walks tiles with a grid stride.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>

#include "device.h"
#include "params.h"

namespace kvq {

// Residency targets (waves per SIMD); the register allocator is held to 512 / target VGPRs.
constexpr int kEncodeWavesPerEU = 4;
constexpr int kDecodeWavesPerEU = 4;

// The cache-window encodes (general row mapping) at 3 and 4 bits need about 165-180
// registers: held to 128 they spilled 150-250 bytes per lane and ran 1.5-3x slower than the
// contiguous encode (b = 4 window 95 us against 30 us on [1,8,32768,128]); at 3 waves per
// SIMD they run at 35 and 39 us.
template <int BITS, bool CONTIG>
constexpr int encode_waves_per_eu() {
  return (!CONTIG && BITS >= 3) ? 3 : kEncodeWavesPerEU;
}

// The matrix-core encode at D = 256 holds twice the values per lane (64 transform outputs):
// held to 128 registers it spilled, so it runs 3 waves per SIMD.
template <int D>
constexpr int mx_waves_per_eu() {
  return D == 128 ? kEncodeWavesPerEU : 3;
}

// ------------------------------------------------------------------------------ quantizers

// Codes of y[JLO..JHI) for both stages, LSB-first with code JLO in bits [0, BITS) (as one
// packed word holds them). y is the raw transform H diag(s) x of the vector's coordinates
// and K the per-vector scale with the sign the caller's transform leaves on y folded in
// (bits <= 2: NX = fma(y, -K, +0) is the value in stage-1 units with its sign flipped;
// bits >= 3: w1 = fma(y, K, +0)). K2 = |K| r12 (bits <= 2) and K2s (bits >= 3, carrying the
// same sign as K) are the stage-2 scales; t1s / t2s are the LDS bucket tables (bits >= 3).
template <int BITS, int STAGES, int JLO, int JHI, int N>
__device__ __forceinline__ void quantize_run(const float (&y)[N], float K, float K2, float K2s, const EncodeArgs& a,
                                             const float4* t1s, const float2* t2s, uint32_t& w1o, uint32_t& w2o) {
  constexpr int jlo = JLO, jhi = JHI, cnt = jhi - jlo;
  static_assert(0 <= JLO && JLO < JHI && JHI <= N, "code range inside the values");
  uint32_t u1 = 0, u2 = 0;
#pragma unroll
  for (int j = jhi - 1; j >= jlo; --j) {  // highest code first: code jlo ends in bits [0, BITS)
    // STAGES = 0 takes +K: then the sign bit is [y_true < 0] (zeros of either sign give
    // +0), and the word is complemented below to [y_true >= 0]
    const float nx = __builtin_fmaf(y[j], STAGES == 0 ? K : -K, 0.0f);
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
      // Bucket tables: the code is base + [w > thr] of the entry that the bucket of
      // v = clamp(w + 1/2, 0, 1) selects (the clamp is the add's output modifier). The
      // entry's byte offset is read from the bits of v + 2^13 (spacing 2^-10: sixteen
      // times the bucket count) and of v2 + 2^14 (spacing 2^-9, eight-byte entries). A code
      // is below 2^BITS, so it is added to the shifted word rather than or-ed in: the
      // comparison's carry then goes straight into the word (one shift, one add-with-carry).
      const float w1 = __builtin_fmaf(y[j], K, 0.0f);
      const float v1 = __builtin_amdgcn_fmed3f(w1 + 0.5f, 0.0f, 1.0f);
      const uint32_t o1 = __float_as_uint(v1 + 8192.0f) & 0x7F0u;
      const float4 e = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(t1s) + o1);
      const bool gt = w1 > e.x;
      u1 = ((u1 << BITS) + __float_as_uint(e.y)) + (gt ? 1u : 0u);
      const float w2 = __builtin_fmaf(y[j], K2s, gt ? e.w : e.z);
      const float v2 = __builtin_amdgcn_fmed3f(w2 + 0.5f, 0.0f, 1.0f);
      const uint32_t o2 = __float_as_uint(v2 + 16384.0f) & 0x3F8u;
      const float2 e2 = *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(t2s) + o2);
      u2 = ((u2 << BITS) + __float_as_uint(e2.y)) + (w2 > e2.x ? 1u : 0u);
    }
  }
  // Word fixups. Each field holds (P, low) with P = [value > 0] for stage 1 and
  // Q = [residual magnitude < 0] for stage 2. Stage 2's sign is P2 = P1 xor Q (the
  // residual of a non-positive y is the negated magnitude). A field with P = 0 counts
  // downward from the middle: its low bits are (2^(BITS-1) - 1) - m = m xor
  // (2^(BITS-1) - 1); at BITS = 2 that low bit is O xor P xor 1 from the [>= T] bit the
  // alignbit stored.
  // (BITS >= 3 fields are the codes themselves.)
  const uint32_t ones = field_ones<BITS>(cnt);
  if constexpr (BITS == 2) {
    // stage 2 holds (sign(W), [|W| >= 2]); its residual-magnitude sign is
    // Q = sign(U) xor sign(W) with sign(U) = not O, so P2 = P xor not O xor sign(W)
    u2 ^= ((u1 ^ (u1 >> 1) ^ ones) & ones) << 1;
    u1 ^= ~(u1 >> 1) & ones;
    u2 ^= ~(u2 >> 1) & ones;
  } else if constexpr (BITS == 1) {
    u2 ^= u1;
  }
  if constexpr (STAGES == 0) u1 = ~u1 & ones;
  w1o = u1;
  w2o = u2;
}

// ------------------------------------------------------------------------------ encode

// STAGES = 2: the two-stage residual codec (both code streams); STAGES = 1: the single-stage
// codec ("turboquant" tag page, "Kernel 3": rotate, then the nearest Gaussian Lloyd-Max
// centroid), stream 1 only; STAGES = 0 (BITS = 1 only): the 1-bit sign code [y >= 0] of
// the rotated vector with its norm ("rvq" tag page, "A fusion this codebase had already
// proven out": rotate, binarize, pack and magnitude in one kernel), stream 1 only.
// D is the rotation length. ROWS (see kRowsFull): input rows of a.dh < D elements (a head
// dimension that is not a power of two) are loaded densely, 16-byte chunks (kRowsChunks) or
// dwords (kRowsRagged), and the missing coordinates read as zeros, which is the zero-padded
// vector the codec rotates.
template <int D, int BITS, bool CONTIG, int STAGES, int ROWS = kRowsFull>
__global__ __launch_bounds__(kBlockThreads, (encode_waves_per_eu<BITS, CONTIG>())) void encode_kernel(const EncodeArgs a) {
  using G = Layout<D>;
  constexpr int C = G::C, L = G::L, LOG_L = G::LOG_L, VW = G::VW, CH = G::CH;
  constexpr int EPW = 32 / BITS;                     // codes per word
  constexpr int NW = (D + EPW - 1) / EPW;            // words per vector per stream
  constexpr bool STAGED = BITS == 3 && L > 1;        // 10-code words straddle lanes
  // words stored per lane: STAGED lanes store the (3 or 4) words that start in their slice
  constexpr int NWL = STAGED ? 4 : (L == 1 ? NW : C / EPW);
  constexpr bool TWO = STAGES == 2;                  // stage 2 computed and stored
  static_assert(STAGES != 0 || BITS == 1, "the sign code is one bit per coordinate");
  static_assert(!STAGED || C == 32, "a 3-bit lane slice is 96 bits");

  __shared__ uint4 stage[kWavesPerBlock][64 * CH];
  // bucket tables (BITS >= 3): 128 slots, every offset the 7-bit masks can form; the slots
  // past the last entry are never reached by a v in [0, 1] and hold "no threshold"
  constexpr int TSLOTS = BITS >= 3 ? 128 : 1;
  __shared__ float4 t1s[TSLOTS];
  __shared__ float2 t2s[TSLOTS];
  if constexpr (BITS >= 3) {
    for (int i = threadIdx.x; i < TSLOTS; i += kBlockThreads) {
      const bool in = i < kTabEntries;
      t1s[i] = in ? make_float4(a.tab1[i][0], a.tab1[i][1], a.tab1[i][2], a.tab1[i][3])
                  : make_float4(__builtin_inff(), 0.f, 0.f, 0.f);
      t2s[i] = in ? make_float2(a.tab2[i][0], a.tab2[i][1]) : make_float2(__builtin_inff(), 0.f);
    }
  }
  // 3-bit codes into a contiguous cache: a tile's words are one run of VW * NW words per
  // stream (16-byte aligned when that count is a multiple of 4). The lanes' own words are 3
  // or 4 scattered dwords each, so they are dropped into LDS and the wave writes the run
  // back with 16-byte stores.
  constexpr int TW = VW * NW;
  constexpr bool RUN3 = STAGED && CONTIG && TW % 4 == 0;
  constexpr int NSTREAM = TWO ? 2 : 1;
  __shared__ uint32_t pk[RUN3 ? kWavesPerBlock : 1][RUN3 ? NSTREAM * TW : 1];
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
  // STAGED: lane q's codes are bits [96 q, 96 q + 96) of the vector's code stream without the
  // two spare bits of each word (word w = stream bits [30 w, 30 w + 30)). The lane stores the
  // words that start in its slice: the first starts at bit o of the slice, 3 or 4 of them.
  const int s_off = STAGED ? (30 - (96 * q) % 30) % 30 : 0;
  const int s_word = STAGED ? (96 * q + s_off) / 30 : 0;
  // fp16 weights (s_2p, s_2p+1) of this lane's C/2 coordinate pairs: the rotation's signs
  uint32_t wt[C / 2];
#pragma unroll
  for (int p = 0; p < C / 2; ++p) wt[p] = a.wpair[q * (C / 2) + p];

  // kRowsChunks: tile t's rows start at chunk t VW dch, and this lane's chunk c of its slice
  // is chunk C q / 8 + c of its vector, real when below dch. kRowsRagged: tile t's rows are
  // the elements [t VW dh, (t + 1) VW dh), a whole number of dwords (VW is even) that lands
  // densely in the buffer; a tile of an odd element count (the last one, at an odd dh) has
  // its last element read from HBM on its own (see ragged_pairs).
  const int dh = ROWS == kRowsFull ? D : a.dh;
  const int dch = dh / 8;
  uint32_t* const b32 = reinterpret_cast<uint32_t*>(buf);
  auto load_tile = [&](int t, int nvt) {
    if constexpr (ROWS == kRowsChunks) {
      dma_dense<CH>(buf, x16 + static_cast<int64_t>(t) * VW * dch, nvt * dch, lane);
    } else if constexpr (ROWS == kRowsRagged) {
      dma_dwords<C / 2>(b32, reinterpret_cast<const uint32_t*>(a.x) + static_cast<int64_t>(t) * (VW * dh / 2),
                        (nvt * dh) >> 1, lane);
    } else {
      dma_tile<CH>(buf, x16 + static_cast<int64_t>(t) * 64 * CH, nvt * L, lane);
    }
  };
  int tile = static_cast<int>(blockIdx.x) * kWavesPerBlock + wv;
  if (tile < n_tiles) {
    const int64_t v0 = static_cast<int64_t>(tile) * VW;
    const int nv = static_cast<int>(a.n_vec - v0 < VW ? a.n_vec - v0 : VW);
    load_tile(tile, nv);
  }
  // The previous tile's results wait in registers until the current tile has been read out
  // of LDS: storing them right after they are computed would put the stores between the
  // next tile's loads and the wait for those loads, and the wait (which counts stores too)
  // would then also wait for the stores to be acknowledged.
  uint32_t w1[NWL], w2[NWL];
  float n_prev = 0.f;
  int64_t row_prev = -1;  // -1: nothing to store (first tile, or a lane past the last vector)
  int64_t v0_prev = -1;   // RUN3: the previous tile's first vector (-1: none) and its count
  int nv_prev = 0;
  // Stores the previous tile's norms and words.
  auto store_prev = [&]() {
    if constexpr (RUN3) {
      if (row_prev >= 0 && q == 0) __builtin_nontemporal_store(n_prev, a.norms + row_prev);
      if (v0_prev < 0) return;  // wave-uniform
      uint32_t* pw = pk[wv];
      if (row_prev >= 0) {
        const int base = vl * NW + s_word;
#pragma unroll
        for (int k = 0; k < NWL; ++k) {
          if (k < 3 || s_off == 0) {
            pw[base + k] = w1[k];
            if constexpr (TWO) pw[TW + base + k] = w2[k];
          }
        }
      }
      wave_lds_fence();
      const int valid = nv_prev * NW;  // words of the run that belong to vectors
      static_assert(TW / 4 <= 64, "one 16-byte chunk per lane");
#pragma unroll
      for (int st = 0; st < NSTREAM; ++st) {
        uint32_t* dst = (st == 0 ? a.p1 : a.p2) + v0_prev * NW;
        if (4 * lane + 4 <= valid) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(pw + st * TW + 4 * lane);
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst) + lane);
        } else if (4 * lane < valid) {
          for (int e = 4 * lane; e < valid; ++e) __builtin_nontemporal_store(pw[st * TW + e], dst + e);
        }
      }
      wave_lds_fence();  // the reads above complete before the next tile's words land
    } else if (row_prev >= 0) {
      if (q == 0) __builtin_nontemporal_store(n_prev, a.norms + row_prev);
      if constexpr (STAGED) {
#pragma unroll
        for (int k = 0; k < NWL; ++k) {
          if (k < 3 || s_off == 0) {
            __builtin_nontemporal_store(w1[k], a.p1 + row_prev * NW + s_word + k);
            if constexpr (TWO) __builtin_nontemporal_store(w2[k], a.p2 + row_prev * NW + s_word + k);
          }
        }
      } else {
        store_words<NWL>(a.p1 + row_prev * NW + q * NWL, w1);
        if constexpr (TWO) store_words<NWL>(a.p2 + row_prev * NW + q * NWL, w2);
      }
    }
  };
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
    uint32_t xr[ROWS == kRowsRagged ? C / 2 : 1];
    if constexpr (ROWS == kRowsRagged)
      ragged_pairs<C>(b32, a.x + static_cast<int64_t>(tile) * VW * dh, vl, q * C, dh, nv * dh, xr);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      uint4 v;
      if constexpr (ROWS == kRowsChunks) {
        const int cv = q * CH + c;
        v = cv < dch ? buf[vl * dch + cv] : make_uint4(0u, 0u, 0u, 0u);
      } else if constexpr (ROWS == kRowsRagged) {
        v = make_uint4(xr[4 * c], xr[4 * c + 1], xr[4 * c + 2], xr[4 * c + 3]);
      } else {
        v = buf[rbase ^ c];
      }
      const uint32_t xh[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2_t h = __builtin_bit_cast(half2_t, xh[i]);
        acc[i] = __builtin_amdgcn_fdot2(h, h, acc[i], false);
      }
      const uint32_t w[4] = {wt[4 * c], wt[4 * c + 1], wt[4 * c + 2], wt[4 * c + 3]};
      float o[8];
      dot2_stages8(xh, w, o);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[8 * c + j] = o[j];
    }
    wait_lds();

    // 2. Store the previous tile, then start loading the next tile into the buffer this
    //    tile has just left. Lanes hold consecutive slices of consecutive vectors, so a
    //    wave writes contiguous runs.
    store_prev();
    {
      const int nt = tile + stride;
      if (nt < n_tiles) {
        const int64_t w0 = static_cast<int64_t>(nt) * VW;
        const int nvn = static_cast<int>(a.n_vec - w0 < VW ? a.n_vec - w0 : VW);
        load_tile(nt, nvn);
      }
    }

    __builtin_amdgcn_s_setprio(0);

    // 3. Remaining butterfly stages: in registers, then across the vector's lanes.
    lane_stages<C, 4>(y);
    cross_stages<C, LOG_L>(y, q);
    // v_sqrt_f32 (within 1 ulp): the correctly rounded sqrtf costs a dozen more instructions
    // per tile for denormal scaling and the last-bit fix-up. The sum of squares of fp16 values
    // is 0 or a normal float32, and the stored norm is held to 1e-6 relative, so neither is
    // needed.
    const float ss = lane_sum<LOG_L>((acc[0] + acc[1]) + (acc[2] + acc[3]));
    const float n = __builtin_amdgcn_sqrtf(ss);
    __builtin_amdgcn_sched_barrier(0);

    // 4. Quantize both stages and pack. BITS <= 2: K maps the raw transform to the stage-1
    //    unit with the sign flipped: NX = fma(y', -K, +0) = -(y_true * unit1) (K carries the
    //    lane's sign). Adding +0 turns an exact zero into +0, so sign(NX) is exactly
    //    [y_true > 0] (the count semantics at the middle boundary 0). A zero vector gets
    //    K = 0, so y_true = 0. The stage-2 value X2 = (|y_true| - cm) * unit2 is formed from
    //    y' directly (K2 = |K| * r12), one rounding.
    //    BITS >= 3 compare w1 = fma(y', K, +0) = y_true / (2 R1) and
    //    w2 = fma(y', K2s, -c1[m] / (2 R2)) = (y_true - c1[m]) / (2 R2) (K2s carries the lane's
    //    sign as K does) with thresholds in the same units: an exact zero gives w1 = +0, which
    //    does not exceed the middle threshold 0.
    //    BITS >= 3 take both scales as RN32(k / sqrt(ss)), through v_rsq_f64: the stage-2
    //    decision on y_true - c1[m] carries |y_true| times the scale's relative error, which
    //    the finer codes turn into flips at their boundaries; the float32 chain (square
    //    root, reciprocal, product) would round three times.
    float K, K2s = 0.f;
    if constexpr (BITS >= 3) {
      const double r = (ss > 0.f) ? __builtin_amdgcn_rsq(static_cast<double>(ss)) : 0.0;
      K = static_cast<float>(static_cast<double>(a.k_scale) * r);
      K2s = static_cast<float>(static_cast<double>(a.k2_scale) * r);
      if (negated) K2s = -K2s;
    } else {
      K = (n > 0.f) ? a.k_scale * __builtin_amdgcn_rcpf(n) : 0.f;  // v_rcp_f32: 1 ulp
    }
    const float K2 = K * a.r12;
    if (negated) K = -K;
    // Codes of this lane's coordinates [jlo, jhi) of both stages, LSB-first with code jlo in
    // bits [0, BITS) (as one packed word holds them).
    auto pack_range = [&](auto first, auto end, uint32_t& w1o, uint32_t& w2o) {
      quantize_run<BITS, STAGES, decltype(first)::value, decltype(end)::value>(y, K, K2, K2s, a, t1s, t2s, w1o, w2o);
    };
    if constexpr (!STAGED) {
      static_for<0, NWL>([&](auto wi) {
        constexpr int w = decltype(wi)::value;
        pack_range(Int<w * EPW>{}, Int<((w + 1) * EPW < C ? (w + 1) * EPW : C)>{}, w1[w], w2[w]);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      // 3-bit codes, 32 per lane: each stream's codes go into the lane's 96-bit slice of the
      // stream (code j at slice bits [3 j, 3 j + 3)): codes 0-9, 11-20 and 22-31 as three
      // 30-bit groups, codes 10 and 21 across the dword boundaries. A word is the 30 bits
      // starting at its offset, from two consecutive slice dwords (or the last one and the
      // first dword of the next lane's slice; zero past the vector's end).
      uint32_t g1[3], g2[3], c10[2], c21[2];
      static_for<0, 3>([&](auto ki) {
        constexpr int k = decltype(ki)::value;
        pack_range(Int<11 * k>{}, Int<11 * k + 10>{}, g1[k], g2[k]);
        __builtin_amdgcn_sched_barrier(0);
      });
      pack_range(Int<10>{}, Int<11>{}, c10[0], c10[1]);
      pack_range(Int<21>{}, Int<22>{}, c21[0], c21[1]);
      __builtin_amdgcn_sched_barrier(0);
      // lanes whose slice starts at a word boundary take other dword pairs for words 1 and 2;
      // the choice is a bit-select with a lane mask (a ternary here becomes a branch)
      const uint32_t at0 = s_off == 0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int st = 0; st < STAGES; ++st) {
        const uint32_t ga = st == 0 ? g1[0] : g2[0], gb = st == 0 ? g1[1] : g2[1], gc = st == 0 ? g1[2] : g2[2];
        const uint32_t d0 = ga | (c10[st] << 30);
        const uint32_t d1 = (c10[st] >> 2) | (gb << 1) | (c21[st] << 31);
        const uint32_t d2 = (c21[st] >> 1) | (gc << 2);
        uint32_t nb = static_cast<uint32_t>(__shfl(static_cast<int>(d0), lane + 1));
        if (q == L - 1) nb = 0u;
        constexpr uint32_t M30 = 0x3FFFFFFFu;
        const uint32_t e0 = __builtin_amdgcn_alignbit(d1, d0, s_off) & M30;
        const uint32_t e1 = ((__builtin_amdgcn_alignbit(d1, d0, 30) & at0) |
                             (__builtin_amdgcn_alignbit(d2, d1, s_off - 2) & ~at0)) & M30;
        const uint32_t e2 = ((__builtin_amdgcn_alignbit(d2, d1, 28) & at0) |
                             (__builtin_amdgcn_alignbit(nb, d2, s_off - 4) & ~at0)) & M30;
        const uint32_t e3 = __builtin_amdgcn_alignbit(nb, d2, 26) & M30;  // stored only when s_off == 0
        if (st == 0) {
          w1[0] = e0; w1[1] = e1; w1[2] = e2; w1[3] = e3;
        } else {
          w2[0] = e0; w2[1] = e1; w2[2] = e2; w2[3] = e3;
        }
      }
    }
    n_prev = n;
    {
      // computed for every lane, then selected (a lane-dependent call site would split the
      // loop body into branches and raise register pressure)
      const int64_t r = cache_row<CONTIG>(a.map, v0, vl);
      row_prev = (vl < nv) ? r : -1;
    }
    v0_prev = v0;
    nv_prev = nv;
  }
  store_prev();
}

// ------------------------------------------------------------------------------ encode, matrix cores

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Byte r of kWalsh8 holds bit t = parity(r & t) for r, t < 8: the eight Walsh functions of
// length 8, i.e. the sign pattern of row r of the 8 x 8 Sylvester Hadamard matrix.
constexpr uint64_t kWalsh8 = 0x963C5AF066CCAA00ull;

// The encodes of D = 128 and 256 with their transform on the matrix cores. The Sylvester
// matrix factors as H_D = H_NB (x) H_32 (NB = D / 32 = 4 or 8): entry (32 g + r, 32 k + c) is
// (-1)^popcount(g & k) H_32[r][c]. So each 32-coordinate input block x_k of a vector is first
// transformed on its own, z_k = H_32 x_k, and output block g is sum_k (-1)^popcount(g & k) z_k:
// log2(NB) more butterfly stages across the blocks. For a tile of 16 vectors the z_k are 2 NB
// products v_mfma_f32_16x16x32_f16 (A = a 16 x 32 slice of H_32, B = input block k of the 16
// vectors), whose +-1 entries and fp16 inputs multiply exactly, summed in float32; the stages
// across the blocks are float32 adds in registers. The rotation's signs diag(s) are applied
// to the fp16 inputs first (an XOR of sign bits), as the butterfly kernel does through its
// weights.
//
// Why the matrix cores: the butterfly kernel spends about 6.5 VALU instructions per
// coordinate on the transform, as many as its quantizers and packing together, and a wave's
// last tile is computed after the input stream has ended; here (D = 128) the transform is 8
// MFMAs and 64 adds per 16-vector tile, about 280 VALU instructions in all against 450,
// which shortens both the arithmetic that the memory stream has to hide and that tail.
//
// MFMA layout (16x16x32): lane l supplies row l % 16 of A and column l % 16 of B, each with
// the 8 k-values 8 (l / 16) + [0, 8), and receives D[4 (l / 16) + i][l % 16], i < 4. B's
// columns are the tile's vectors: lane l works on vector v = l % 16 together with the lanes
// of the same v in the other three groups g = l / 16, and supplies the coordinates
// 32 k + 8 g + [0, 8) of input block k (one 16-byte chunk). A's row m of output half mh
// carries H_32 row 8 (m >> 2) + 4 mh + (m & 3), so that lane group g receives the block
// coordinates 8 g + 4 mh + i: over the two halves, 8 consecutive coordinates of every block,
// and of every output block after the stages across blocks. Their codes are 8 consecutive
// fields of one packed word (BITS = 4) or a quarter or half of one (BITS = 1, 2); NB / 4
// transposes of those pieces across the four lane groups (v_permlane32_swap, then
// v_permlane16_swap), each over blocks NB / 4 apart, leave lane group g with output blocks
// [g NB / 4, (g + 1) NB / 4), i.e. the vector's words [g NW / 4, (g + 1) NW / 4), stored as
// one contiguous run. At BITS = 3 (D = 128) a piece is 24 bits and the transpose leaves lane
// group g with the 96-bit slice of the code stream that holds codes [32 g, 32 g + 32); the
// 30-bit words (10 codes and 2 spare bits each) are cut from the slices as in the butterfly
// kernel, and a contiguous cache receives each tile's 208 words per stream through LDS as
// one run of 16-byte stores.
template <int D, int BITS, bool CONTIG, int STAGES>
__global__ __launch_bounds__(kBlockThreads, (mx_waves_per_eu<D>())) void encode_mx_kernel(const EncodeArgs a) {
  constexpr int NB = D / 32;             // 32-coordinate blocks of a vector
  constexpr int BPG = NB / 4;            // output blocks each lane group stores
  constexpr int CPV = D / 8;             // 16-byte chunks per vector
  constexpr int TV = kMxTile;            // vectors per tile: the MFMA's 16 columns
  constexpr int TCH = TV * CPV;          // chunks per tile
  constexpr int EPW = 32 / BITS;         // codes per word
  constexpr int NW = (D + EPW - 1) / EPW;  // words per vector per stream
  constexpr bool B3 = BITS == 3;         // 10-code words straddle the lane groups' slices
  constexpr int WPL = B3 ? 4 : NW / 4;   // words each lane group holds per stream (B3: 3 or 4)
  constexpr int WB = B3 ? 0 : NW / NB;   // words of one 32-coordinate block per stream
  constexpr bool TWO = STAGES == 2;
  constexpr int NSTREAM = TWO ? 2 : 1;
  constexpr int TW = TV * NW;            // words of a tile per stream
  constexpr bool RUN = B3 && CONTIG;     // B3 words to a contiguous cache: one run through LDS
  constexpr bool MASKS_LDS = NB > 4;     // the sign masks of 8 blocks would hold 32 registers
  static_assert(TV == 16 && (NB == 4 || NB == 8), "16 vectors of 4 or 8 blocks: one MFMA column per vector");
  static_assert(!B3 || NB == 4, "3-bit slices: 4 blocks, one per lane group");
  static_assert(STAGES != 0 || BITS == 1, "the sign code is one bit per coordinate");
  static_assert(!RUN || (TW % 4 == 0 && TW / 4 <= 64), "a tile's run is at most one 16-byte chunk per lane");

  __shared__ u32x4_t stage[kWavesPerBlock][TCH];
  __shared__ uint32_t pk[RUN ? kWavesPerBlock : 1][RUN ? NSTREAM * TW : 1];
  // MASKS_LDS: the sign-bit masks of diag(s) for chunk 4 k + g of every vector, at [4 k + g]
  __shared__ u32x4_t smask[MASKS_LDS ? 4 * NB : 1];
  if constexpr (MASKS_LDS) {
    for (int i = threadIdx.x; i < 4 * NB; i += kBlockThreads)
      smask[i] = u32x4_t{a.wpair[4 * i] ^ kOnePair, a.wpair[4 * i + 1] ^ kOnePair, a.wpair[4 * i + 2] ^ kOnePair,
                         a.wpair[4 * i + 3] ^ kOnePair};
    if constexpr (BITS < 3) __syncthreads();
  }
  constexpr int TSLOTS = BITS >= 3 ? 128 : 1;
  __shared__ float4 t1s[TSLOTS];
  __shared__ float2 t2s[TSLOTS];
  if constexpr (BITS >= 3) {
    for (int i = threadIdx.x; i < TSLOTS; i += kBlockThreads) {
      const bool in = i < kTabEntries;
      t1s[i] = in ? make_float4(a.tab1[i][0], a.tab1[i][1], a.tab1[i][2], a.tab1[i][3])
                  : make_float4(__builtin_inff(), 0.f, 0.f, 0.f);
      t2s[i] = in ? make_float2(a.tab2[i][0], a.tab2[i][1]) : make_float2(__builtin_inff(), 0.f);
    }
    __syncthreads();
  }

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int v = lane & 15;  // this lane's vector in the tile
  const int g = lane >> 4;  // its lane group: input coordinates 32 k + 8 g + [0, 8)
  // B3: the slice of lane group g is stream bits [96 g, 96 g + 96); its first word starts
  // s_off bits in (word s_word), and it holds 4 word starts when s_off = 0 (g = 0), else 3
  const int s_off = B3 ? (30 - (96 * g) % 30) % 30 : 0;
  const int s_word = B3 ? (96 * g + s_off) / 30 : 0;
  u32x4_t* buf = stage[wv];
  const int n_tiles = static_cast<int>((a.n_vec + TV - 1) / TV);  // fits (checked on the host)
  const int stride = static_cast<int>(gridDim.x) * kWavesPerBlock;
  const char* xb = reinterpret_cast<const char*>(a.x);

  // Direct-to-LDS loads of tile t: instruction k fills slots [64k, 64k + 64); slot s holds
  // chunk (s % CPV) ^ row of vector row = s / CPV, so the 8 lanes of an LDS read phase
  // (consecutive vectors, one chunk each) hit 8 distinct 16-byte bank groups. Rows past the
  // input's end re-read its last vector: every load stays inside the input, and those rows
  // are never stored.
  auto dma = [&](int t) {
    const int64_t t0 = static_cast<int64_t>(t) * TV;
    const int nv = static_cast<int>(a.n_vec - t0 < TV ? a.n_vec - t0 : TV);
    const char* base = xb + t0 * (2 * D);  // wave-uniform
#pragma unroll
    for (int k = 0; k < TCH / 64; ++k) {
      const int s = k * 64 + lane, r = s / CPV, p = s % CPV;
      const int rr = (nv == TV || r < nv) ? r : nv - 1;
      const uint32_t off = static_cast<uint32_t>(rr * CPV + (p ^ r)) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, kNonTemporal);
    }
  };

  int tile = static_cast<int>(blockIdx.x) * kWavesPerBlock + wv;
  if (tile < n_tiles) dma(tile);

  // Per-wave constants, computed while the first tile is in flight: the sign-bit masks of
  // diag(s) over this lane's input chunks 4 k + g, and the A operands of the two output
  // halves (row m = v: H_32 row 8 (v >> 2) + 4 mh + (v & 3) at columns 8 g + t, t < 8, as
  // fp16 +-1 pairs).
  u32x4_t mk[MASKS_LDS ? 1 : NB];
  if constexpr (!MASKS_LDS) {
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) mk[k][i] = a.wpair[4 * (4 * k + g) + i] ^ kOnePair;
  }
  f16x8_t ah[2];
#pragma unroll
  for (int mh = 0; mh < 2; ++mh) {
    const int r = 8 * (v >> 2) + 4 * mh + (v & 3);
    const uint32_t pat = static_cast<uint32_t>(kWalsh8 >> (8 * (r & 7))) & 0xFFu;
    const uint32_t f = (__builtin_popcount((r >> 3) & g) & 1) ? 0x80008000u : 0u;
    u32x4_t w;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      w[p] = (kOnePair | (((pat >> (2 * p)) & 1u) << 15) | (((pat >> (2 * p + 1)) & 1u) << 31)) ^ f;
    ah[mh] = __builtin_bit_cast(f16x8_t, w);
  }

  // The previous tile's words wait in registers until this tile has left LDS, so the
  // loop-top wait (which counts stores too) covers stores issued a compute phase earlier.
  uint32_t o1[WPL], o2[WPL];
  float n_prev = 0.f;
  int64_t row_prev = -1;  // -1: nothing to store (first tile, or a lane past the last vector)
  int64_t v0_prev = -1;   // RUN: the previous tile's first vector (-1: none) and its count
  int nv_prev = 0;
  auto store_prev = [&]() {
    if constexpr (RUN) {
      if (row_prev >= 0 && g == 0) __builtin_nontemporal_store(n_prev, a.norms + row_prev);
      if (v0_prev < 0) return;  // wave-uniform
      uint32_t* pw = pk[wv];
      if (row_prev >= 0) {
        const int base = v * NW + s_word;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k < 3 || s_off == 0) {
            pw[base + k] = o1[k];
            if constexpr (TWO) pw[TW + base + k] = o2[k];
          }
        }
      }
      wave_lds_fence();
      const int valid = nv_prev * NW;  // words of the run that belong to vectors
#pragma unroll
      for (int st = 0; st < NSTREAM; ++st) {
        uint32_t* dst = (st == 0 ? a.p1 : a.p2) + v0_prev * NW;
        if (4 * lane + 4 <= valid) {
          const u32x4_t w = *reinterpret_cast<const u32x4_t*>(pw + st * TW + 4 * lane);
          __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(dst) + lane);
        } else if (4 * lane < valid) {
          for (int e = 4 * lane; e < valid; ++e) __builtin_nontemporal_store(pw[st * TW + e], dst + e);
        }
      }
      wave_lds_fence();  // the reads above complete before the next tile's words land
    } else if (row_prev >= 0) {
      if (g == 0) __builtin_nontemporal_store(n_prev, a.norms + row_prev);
      if constexpr (B3) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k < 3 || s_off == 0) {
            __builtin_nontemporal_store(o1[k], a.p1 + row_prev * NW + s_word + k);
            if constexpr (TWO) __builtin_nontemporal_store(o2[k], a.p2 + row_prev * NW + s_word + k);
          }
        }
      } else {
        store_words<WPL>(a.p1 + row_prev * NW + g * WPL, o1);
        if constexpr (TWO) store_words<WPL>(a.p2 + row_prev * NW + g * WPL, o2);
      }
    }
  };

  for (; tile < n_tiles; tile += stride) {
    const int64_t v0 = static_cast<int64_t>(tile) * TV;
    const int nv = static_cast<int>(a.n_vec - v0 < TV ? a.n_vec - v0 : TV);

    // 1. This lane's fp16 coordinates: chunk 4 k + g of its vector is its B operand of input
    //    block k.
    wait_vmem();
    u32x4_t bq[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) bq[k] = buf[v * CPV + ((4 * k + g) ^ v)];
    wait_lds();

    // 2. Store the previous tile, then load the next one into the buffer just read.
    store_prev();
    if (tile + stride < n_tiles) dma(tile + stride);

    // 3. diag(s) on the fp16 inputs, the blocks' transforms z_k (register i of half mh is
    //    block coordinate 8 g + 4 mh + i), then the log2(NB) stages across the blocks: output
    //    block gb = sum_k (-1)^popcount(gb & k) z_k.
    f32x4_t y4[NB][2];
    if constexpr (NB == 4) {
      f32x4_t z[NB][2];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const f16x8_t bx = __builtin_bit_cast(f16x8_t, bq[k] ^ mk[k]);
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) z[k][mh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[mh], bx, f32x4_t{}, 0, 0, 0);
      }
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float s0 = z[0][mh][i] + z[1][mh][i], d0 = z[0][mh][i] - z[1][mh][i];
          const float s1 = z[2][mh][i] + z[3][mh][i], d1 = z[2][mh][i] - z[3][mh][i];
          y4[0][mh][i] = s0 + s1;
          y4[1][mh][i] = d0 + d1;
          y4[2][mh][i] = s0 - s1;
          y4[3][mh][i] = d0 - d1;
        }
    } else {
      f32x4_t z[NB][2];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const f16x8_t bx = __builtin_bit_cast(f16x8_t, bq[k] ^ smask[4 * k + g]);
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) z[k][mh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[mh], bx, f32x4_t{}, 0, 0, 0);
      }
      // element by element: all the stages of one (mh, i) before the next
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t[NB];
#pragma unroll
          for (int k = 0; k < NB; ++k) t[k] = z[k][mh][i];
#pragma unroll
          for (int h = 1; h < NB; h *= 2)
#pragma unroll
            for (int k = 0; k < NB; ++k)
              if ((k & h) == 0) {
                const float p = t[k], q = t[k + h];
                t[k] = p + q;
                t[k + h] = p - q;
              }
#pragma unroll
          for (int k = 0; k < NB; ++k) y4[k][mh][i] = t[k];
        }
    }

    // 4. Norm: squares of the fp16 values summed in float32, the four lane groups of the
    //    vector added in a fixed order (every lane forms the same sum).
    float ss;
    {
      float s2[2] = {0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NB; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t e = bq[k][i];
          const half2_t p = __builtin_bit_cast(half2_t, e);
          s2[i & 1] = __builtin_amdgcn_fdot2(p, p, s2[i & 1], false);
        }
      }
      const float part = s2[0] + s2[1];
      const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
      const float p2 = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);  // groups g and g ^ 2
      const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(p2), __float_as_uint(p2), false, false);
      ss = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);              // and g ^ 1
    }
    const float n = __builtin_amdgcn_sqrtf(ss);  // v_sqrt_f32, within 1 ulp
    float K, K2 = 0.f, K2s = 0.f;
    if constexpr (BITS >= 3) {
      const double rs = (ss > 0.f) ? __builtin_amdgcn_rsq(static_cast<double>(ss)) : 0.0;
      K = static_cast<float>(static_cast<double>(a.k_scale) * rs);
      K2s = static_cast<float>(static_cast<double>(a.k2_scale) * rs);
    } else {
      K = (n > 0.f) ? a.k_scale * __builtin_amdgcn_rcpf(n) : 0.f;
      K2 = K * a.r12;
    }

    // 5. Codes: output block gb's coordinates 8 g + [0, 8) of this lane give piece gb
    //    (8 BITS bits).
    uint32_t pc1[NB], pc2[NB];
#pragma unroll
    for (int gb = 0; gb < NB; ++gb) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = y4[gb][0][i];
        y[4 + i] = y4[gb][1][i];
      }
      quantize_run<BITS, STAGES, 0, 8>(y, K, K2, K2s, a, t1s, t2s, pc1[gb], pc2[gb]);
    }

    // 6. Transpose the pieces across the lane groups, BPG times: in round r, piece
    //    BPG j + r of group g' goes to group j, slot g' (two swaps across lane halves, then
    //    two across 16-lane rows), so group g holds the pieces of output blocks BPG g + r
    //    from groups 0..3 in order, i.e. the vector's words [g WPL, g WPL + WPL) once joined.
    auto gather = [&](const uint32_t (&pc)[NB], uint32_t (&o)[WPL]) {
#pragma unroll
      for (int r = 0; r < BPG; ++r) {
        uint32_t w[4] = {pc[r], pc[BPG + r], pc[2 * BPG + r], pc[3 * BPG + r]};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const auto sw = __builtin_amdgcn_permlane32_swap(w[j], w[j + 2], false, false);
          w[j] = sw[0];
          w[j + 2] = sw[1];
        }
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const auto sw = __builtin_amdgcn_permlane16_swap(w[j], w[j + 1], false, false);
          w[j] = sw[0];
          w[j + 1] = sw[1];
        }
        if constexpr (BITS == 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) o[WB * r + j] = w[j];
        } else if constexpr (BITS == 3) {
          // the 96-bit slice as three dwords, then the 30-bit words starting in it (the last
          // one reads on into the next group's slice; zero past the vector's end)
          const uint32_t d0 = w[0] | (w[1] << 24);
          const uint32_t d1 = (w[1] >> 8) | (w[2] << 16);
          const uint32_t d2 = (w[2] >> 16) | (w[3] << 8);
          uint32_t nb = static_cast<uint32_t>(__shfl(static_cast<int>(d0), lane + 16));
          if (g == NB - 1) nb = 0u;
          constexpr uint32_t M30 = 0x3FFFFFFFu;
          const uint32_t at0 = s_off == 0 ? 0xFFFFFFFFu : 0u;  // a bit-select, not a branch
          o[0] = __builtin_amdgcn_alignbit(d1, d0, s_off) & M30;
          o[1] = ((__builtin_amdgcn_alignbit(d1, d0, 30) & at0) |
                  (__builtin_amdgcn_alignbit(d2, d1, s_off - 2) & ~at0)) & M30;
          o[2] = ((__builtin_amdgcn_alignbit(d2, d1, 28) & at0) |
                  (__builtin_amdgcn_alignbit(nb, d2, s_off - 4) & ~at0)) & M30;
          o[3] = __builtin_amdgcn_alignbit(nb, d2, 26) & M30;  // stored only when s_off == 0
        } else if constexpr (BITS == 2) {
          o[WB * r] = w[0] | (w[1] << 16);
          o[WB * r + 1] = w[2] | (w[3] << 16);
        } else {
          o[WB * r] = w[0] | (w[1] << 8) | (w[2] << 16) | (w[3] << 24);
        }
      }
    };
    gather(pc1, o1);
    if constexpr (TWO) gather(pc2, o2);

    n_prev = n;
    {
      const int64_t r = cache_row<CONTIG>(a.map, v0, v);
      row_prev = (v < nv) ? r : -1;
    }
    v0_prev = v0;
    nv_prev = nv;
  }
  store_prev();
}

// ------------------------------------------------------------------------------ decode

// STAGES = 2: z = c1[i1] + c2[i2]; STAGES = 1: z = c1[i1] (the host fills the table so that
// entry (i1 << BITS) holds the right value in both cases). D is the rotation length. ROWS
// (see kRowsFull): output rows of a.dh < D elements (a head dimension that is not a power of
// two) take the first a.dh of the D reconstructed coordinates, written as dense 16-byte
// chunks (kRowsChunks) or dwords (kRowsRagged).
template <int D, int BITS, bool CONTIG, int STAGES, int ROWS = kRowsFull>
__global__ __launch_bounds__(kBlockThreads, kDecodeWavesPerEU) void decode_kernel(const DecodeArgs a) {
  using G = Layout<D>;
  using S = CodeShape<D, BITS>;
  constexpr int C = G::C, L = G::L, LOG_L = G::LOG_L, VW = G::VW, CH = G::CH;
  constexpr int NWL = S::NWL;
  constexpr int NZ = 1 << (2 * BITS);
  constexpr bool TWO = STAGES == 2;
  // 1- and 2-bit codes: dequantize groups of GS = 4 / BITS coordinates through a 256-entry
  // table that also does the first log2(GS) butterfly stages (codes_to_groups)
  constexpr bool GROUPS = BITS <= 2;
  constexpr int GS = 4 / BITS;

  __shared__ uint4 stage[kWavesPerBlock][64 * CH];
  __shared__ uint4 smask[D / 8];
  __shared__ float zt[GROUPS ? 1 : NZ];  // per-coordinate table (b >= 3)
  __shared__ GroupEntry<BITS <= 2 ? BITS : 2> gt[GROUPS ? 256 : 1];
  constexpr bool CST = S::STAGED && !S::DIRECT3;  // codes regrouped through LDS
  __shared__ uint32_t cstage[CST ? kWavesPerBlock : 1][CST ? STAGES * S::CSTREAM : 1];
  if constexpr (!GROUPS)
    for (int i = threadIdx.x; i < NZ; i += kBlockThreads) zt[i] = a.ztab[i];
  if constexpr (GROUPS) {
    // entry n1 | n2 << 4: coordinate t of the group has codes (i1, i2) = bits t of n1 and
    // of n2 (BITS = 1), or bit pairs t (BITS = 2); the same float32 sums and differences as
    // the first stages of lane_stages
    for (int i = threadIdx.x; i < 256; i += kBlockThreads) {
      constexpr uint32_t M = (1u << BITS) - 1u;
      float zz[GS];
#pragma unroll
      for (int t = 0; t < GS; ++t)
        zz[t] = a.ztab[(((i >> (BITS * t)) & M) << BITS) | ((i >> (4 + BITS * t)) & M)];
      if constexpr (GS == 2) {
        gt[i] = make_float2(zz[0] + zz[1], zz[0] - zz[1]);
      } else {
        const float s0 = zz[0] + zz[1], d0 = zz[0] - zz[1], s1 = zz[2] + zz[3], d1 = zz[2] - zz[3];
        gt[i] = make_float4(s0 + s1, d0 + d1, s0 - s1, d0 - d1);
      }
    }
  }
  for (int i = threadIdx.x; i < D / 2; i += kBlockThreads) reinterpret_cast<uint32_t*>(smask)[i] = a.xmask[i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane & (L - 1);
  const int vl = lane >> LOG_L;
  uint4* buf = stage[wv];
  uint32_t* cs = cstage[CST ? wv : 0];
  const int n_tiles = static_cast<int>((a.n_vec + VW - 1) / VW);
  const int stride = static_cast<int>(gridDim.x) * kWavesPerBlock;
  const bool negated = (__builtin_popcount(q) & 1) != 0;

  // Software pipeline: the packed words and norm of the next tile are loaded into
  // registers while the current tile is computed, and the current tile's output is stored
  // at the start of the next iteration, after those loads have been issued.
  uint32_t nw1[NWL], nw2[NWL];
  float nnrm = 1.0f;
  auto fetch = [&](int t) {
    const int64_t t0 = static_cast<int64_t>(t) * VW;
    const int tnv = static_cast<int>(a.n_vec - t0 < VW ? a.n_vec - t0 : VW);
    // lanes past the last vector read vector t0 (valid) and store nothing
    const int64_t row = cache_row<CONTIG>(a.map, t0, vl < tnv ? vl : 0);
    load_lane_words<D, BITS>(a.p1, row, q, nw1);
    if constexpr (TWO) {
      load_lane_words<D, BITS>(a.p2, row, q, nw2);
    } else {
#pragma unroll
      for (int k = 0; k < NWL; ++k) nw2[k] = 0u;
    }
    nnrm = a.norms ? a.norms[row] : 1.0f;
  };
  u32x4_t out[CH];          // previous tile's output chunks (chunk 64k + lane of that tile)
  int out_tile = -1, out_rows = 0;
  const int dh = ROWS == kRowsFull ? D : a.dh;  // elements of an output row
  const int dch = dh / 8;                        // and its chunks (kRowsChunks)
  auto flush = [&]() {
    if constexpr (ROWS != kRowsFull) {
      // chunk s of the tile's dense output (rows of dch chunks; out_rows is its chunk count)
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.x) + static_cast<int64_t>(out_tile) * VW * dch;
#pragma unroll
      for (int k = 0; k < CH; ++k)
        if (k * 64 + lane < out_rows) __builtin_nontemporal_store(out[k], dst + k * 64 + lane);
    } else {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.x) + static_cast<int64_t>(out_tile) * 64 * CH;
#pragma unroll
      for (int k = 0; k < CH; ++k)
        if ((k * 64 + lane) / CH < out_rows) __builtin_nontemporal_store(out[k], dst + k * 64 + lane);
    }
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

    // 1. Codes of this lane's C coordinates -> z = c1[i1] + c2[i2] (or c1[i1]).
    float z[C];
    if constexpr (GROUPS) codes_to_groups<D, BITS, TWO>(w1, w2, gt, z);
    else codes_to_z<D, BITS, TWO>(w1, w2, zt, cs, lane, vl, q, z);

    // 2. Inverse rotation: H z (H symmetric), scaled by n / sqrt(D) (carrying the lane's
    //    sign), then the final sign flip as an exact XOR of fp16 sign bits.
    float K = nrm * a.inv_sqrt_d;
    if (negated) K = -K;
    uint32_t o[C / 2];
    unrotate_f16<D, 32, GROUPS ? GS : 1>(z, K, q, o);

    // 3. Transpose through LDS into the chunk order of the (contiguous) output tile, for
    //    coalesced 16-byte stores.
    if constexpr (ROWS != kRowsRagged) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint4 mk = smask[q * CH + c];
        buf[lane * CH + (c ^ swz<CH>(lane))] =
            make_uint4(o[4 * c] ^ mk.x, o[4 * c + 1] ^ mk.y, o[4 * c + 2] ^ mk.z, o[4 * c + 3] ^ mk.w);
      }
    } else {
      // the tile's rows as dense fp16 elements (element vl dh + c of the tile is coordinate c
      // of vector vl), then dword stores of the whole run (the tile starts on a dword: VW is
      // even) and the last element of an odd run on its own
      wave_lds_fence();
      uint16_t* b16 = reinterpret_cast<uint16_t*>(buf);
      const int cq = q * C;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint4 mk = smask[q * CH + c];
        const uint32_t pr[4] = {o[4 * c] ^ mk.x, o[4 * c + 1] ^ mk.y, o[4 * c + 2] ^ mk.z, o[4 * c + 3] ^ mk.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = cq + 8 * c + 2 * i, e = vl * dh + j;
          if (j < dh) b16[e] = static_cast<uint16_t>(pr[i] & 0xFFFFu);
          if (j + 1 < dh) b16[e + 1] = static_cast<uint16_t>(pr[i] >> 16);
        }
      }
      wave_lds_fence();
      const int n = nv * dh, ndw = n >> 1;
      const int64_t first = static_cast<int64_t>(tile) * VW * dh;  // even
      const uint32_t* b32 = reinterpret_cast<const uint32_t*>(buf);
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.x) + (first >> 1);
#pragma unroll
      for (int k = 0; k < C / 2; ++k) {
        const int sidx = k * 64 + lane;
        if (sidx < ndw) __builtin_nontemporal_store(b32[sidx], dst + sidx);
      }
      if ((n & 1) && lane == 0) a.x[first + n - 1] = b16[n - 1];
      wave_lds_fence();  // the reads above complete before the next tile's elements land
      continue;
    }
    wave_lds_fence();
    if constexpr (ROWS == kRowsChunks) {
      // dense output chunk s = 64k + lane is chunk cv = s % dch of vector s / dch, which row
      // (s / dch) L + cv / CH of the tile holds as its chunk cv % CH
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int sidx = k * 64 + lane, vv = sidx / dch, cv = sidx - vv * dch;
        const int r = vv * L + cv / CH, c = cv % CH;
        const uint4 v = r < 64 ? buf[r * CH + (c ^ swz<CH>(r))] : make_uint4(0u, 0u, 0u, 0u);
        out[k] = u32x4_t{v.x, v.y, v.z, v.w};
      }
    } else {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int g = k * 64 + lane, r = g / CH, c = g % CH;
        const uint4 v = buf[r * CH + (c ^ swz<CH>(r))];
        out[k] = u32x4_t{v.x, v.y, v.z, v.w};
      }
    }
    wave_lds_fence();
    out_tile = tile;
    out_rows = ROWS == kRowsChunks ? nv * dch : nv * L;
  }
  if (out_tile >= 0) flush();
}

// ------------------------------------------------------------------------------ dispatch

// Compute units of the current device and blocks of one kernel resident per CU.
static bool residency(const void* f, int* cus, int* per_cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, f, kBlockThreads, 0) != hipSuccess) return false;
  if (*per_cu < 1) *per_cu = 1;
  return *cus > 0;
}

// Persistent grid: at most as many blocks as fit on the device at once (every wave resident
// from the start, walking tiles with a grid stride and loading its next tile while it
// computes the current one), fewer if there are fewer tiles. The residency is asked once per
// kernel (one value per process; all MI355X devices have the same counts).
//
// A wave's last tile is computed after the input stream has ended, so a launch ends with the
// last round's arithmetic on the busiest SIMD. With balance set, the grid takes the number
// of resident blocks per CU (from the most that fit down to 2) whose last round puts the
// fewest waves on one SIMD (a block's waves sit on the four SIMDs of its CU), preferring
// more blocks on ties: the matrix-core encode's 16384 tiles on 256 CUs run as 3 blocks per
// CU (5 rounds of 3072 waves and a last round of 1024, one wave per SIMD) rather than 4
// (4 full rounds). The decodes and the 3- and 4-bit matrix-core encodes keep every resident
// block: a decode's last round is short and the writes of the others' tiles hide it, and
// the 3- and 4-bit encodes are held by their arithmetic, which more waves in flight
// overlap better (4 blocks per CU: 3.5 % faster at 3 bits, the same at 4).
static hipError_t launch(const void* f, void* args, int64_t n_vec, int vw, int* cap, bool balance,
                         hipStream_t stream) {
  const int64_t tiles = (n_vec + vw - 1) / vw;
  if (tiles > INT_MAX) return hipErrorInvalidValue;
  // cap[0]: CUs, cap[1]: resident blocks per CU (a benign race: every caller computes the same)
  if (cap[0] <= 0 && !residency(f, &cap[0], &cap[1])) return hipErrorInvalidValue;
  const int64_t cus = cap[0], per_cu = cap[1];
  const int64_t want = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  int64_t blocks = cus * per_cu;
  if (balance && want > blocks) {
    int64_t best_last = INT64_MAX;
    const int64_t kmin = per_cu < 2 ? per_cu : 2;
    for (int64_t k = per_cu; k >= kmin; --k) {
      const int64_t waves = cus * k * kWavesPerBlock;
      const int64_t last = tiles - ((tiles + waves - 1) / waves - 1) * waves;  // tiles of the last round
      const int64_t per_simd = (last + cus * kWavesPerBlock - 1) / (cus * kWavesPerBlock);
      if (per_simd < best_last) {
        best_last = per_simd;
        blocks = cus * k;
      }
    }
  }
  if (want < blocks) blocks = want;
  void* a[] = {args};
  return hipLaunchKernel(f, dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), a, 0, stream);
}

template <int D, int BITS, int STAGES, int ROWS>
static hipError_t launch_encode_t(const EncodeArgs& a, hipStream_t stream) {
  static int cap[2][2] = {{0, 0}, {0, 0}};
  const bool c = a.map.contiguous != 0;
  if constexpr (encode_on_matrix_cores(D, BITS) && ROWS == kRowsFull) {
    const void* f = c ? reinterpret_cast<const void*>(&encode_mx_kernel<D, BITS, true, STAGES>)
                      : reinterpret_cast<const void*>(&encode_mx_kernel<D, BITS, false, STAGES>);
    return launch(f, const_cast<EncodeArgs*>(&a), a.n_vec, kMxTile, cap[c ? 1 : 0], BITS < 3, stream);
  } else {
    const void* f = c ? reinterpret_cast<const void*>(&encode_kernel<D, BITS, true, STAGES, ROWS>)
                      : reinterpret_cast<const void*>(&encode_kernel<D, BITS, false, STAGES, ROWS>);
    return launch(f, const_cast<EncodeArgs*>(&a), a.n_vec, Layout<D>::VW, cap[c ? 1 : 0], true, stream);
  }
}

template <int D, int BITS, int STAGES, int ROWS>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  static int cap[2][2] = {{0, 0}, {0, 0}};
  const bool c = a.map.contiguous != 0;
  const void* f = c ? reinterpret_cast<const void*>(&decode_kernel<D, BITS, true, STAGES, ROWS>)
                    : reinterpret_cast<const void*>(&decode_kernel<D, BITS, false, STAGES, ROWS>);
  return launch(f, const_cast<DecodeArgs*>(&a), a.n_vec, Layout<D>::VW, cap[c ? 1 : 0], false, stream);
}

}  // namespace kvq
