// Device-side building blocks shared by the codec kernels (codec.h) and the
// attention kernels over the packed cache (attend.hip): the lane layout of a head vector,
// the Walsh-Hadamard butterfly in registers and across lanes, the direct-to-LDS tile load,
// cache-row arithmetic, word loads and stores, and the 3-bit code regrouping helpers.
// gfx950 (MI355X) only.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include <stdint.h>

#include "params.h"

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// How one vector of D coordinates maps onto lanes: C = min(D, CM) consecutive coordinates
// per lane (CM = 32 for the codec kernels; the attention kernels use 16 to leave registers
// for several queries).
template <int D, int CM = 32>
struct Layout {
  static constexpr int C = D < CM ? D : CM;       // coordinates per lane
  static constexpr int L = D / C;                 // lanes per vector
  static constexpr int LOG_L = __builtin_ctz(L);  // butterfly stages across lanes
  static constexpr int VW = 64 / L;               // vectors per wave tile
  static constexpr int CH = C / 8;                // 16-byte input chunks per lane
  static_assert(D >= 8 && D <= 1024 && (D & (D - 1)) == 0, "D must be a power of two in [8, 1024]");
  static_assert(CM >= 8 && L <= 32, "at least 8 coordinates per lane, at most 32 lanes per vector");
};


// ------------------------------------------------------------------------------ helpers

// Compile-time integer, and a loop over [I, N) whose body sees the index as one (so code
// that indexes register arrays with it stays fully unrolled).
template <int V>
struct Int {
  static constexpr int value = V;
};
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}


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

// Butterfly stages 1 and 2 of 8 coordinates straight from their fp16 pairs: xh[k] holds
// coordinates (2k, 2k + 1) and w[k] the fp16 weights (s_2k, s_2k+1), the rotation's signs for
// that pair. v_dot2_f32_f16 multiplies a pair by the weights exactly and adds a float32
// addend; its VOP3P neg_lo / neg_hi modifiers flip the weights' signs for free, so each
// 4-coordinate group takes 6 instructions: s = P0.(w0, w1), d = P0.(w0, -w1), then
// P1.(w2, w3) + s, P1.(w2, -w3) + d, P1.(-w2, -w3) + s, P1.(-w2, w3) + d.
// The twelve instructions are one asm block ending in s_nop 2: on gfx950 a VALU instruction
// reading a DOT result needs 3 wait states, which the compiler inserts for its own dot
// instructions but cannot know about for inline asm. (Inside the block the partial sums are
// read only as the addend of the same opcode, which needs none.) Written as asm because the
// compiler otherwise picks the accumulating v_dot2c and spends a move per product.
constexpr uint32_t kPP = kOnePair;  // fp16 (+1, +1)

__device__ __forceinline__ void dot2_stages8(const uint32_t (&xh)[4], const uint32_t (&w)[4], float (&o)[8]) {
  float s0, d0, s1, d1;
  asm("v_dot2_f32_f16 %8, %12, %16, 0\n"
      "v_dot2_f32_f16 %9, %12, %16, 0 neg_hi:[0,1,0]\n"
      "v_dot2_f32_f16 %10, %14, %18, 0\n"
      "v_dot2_f32_f16 %11, %14, %18, 0 neg_hi:[0,1,0]\n"
      "v_dot2_f32_f16 %0, %13, %17, %8\n"
      "v_dot2_f32_f16 %1, %13, %17, %9 neg_hi:[0,1,0]\n"
      "v_dot2_f32_f16 %2, %13, %17, %8 neg_lo:[0,1,0] neg_hi:[0,1,0]\n"
      "v_dot2_f32_f16 %3, %13, %17, %9 neg_lo:[0,1,0]\n"
      "v_dot2_f32_f16 %4, %15, %19, %10\n"
      "v_dot2_f32_f16 %5, %15, %19, %11 neg_hi:[0,1,0]\n"
      "v_dot2_f32_f16 %6, %15, %19, %10 neg_lo:[0,1,0] neg_hi:[0,1,0]\n"
      "v_dot2_f32_f16 %7, %15, %19, %11 neg_lo:[0,1,0]\n"
      "s_nop 2"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(s0), "=&v"(d0), "=&v"(s1), "=&v"(d1)
      : "v"(xh[0]), "v"(xh[1]), "v"(xh[2]), "v"(xh[3]), "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]));
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

// Direct-to-LDS loads of a tile of padded rows: the tile's nchunks real 16-byte chunks
// (rows of dch chunks, contiguous in HBM from src) land densely in LDS slots [0, nchunks);
// instruction k writes slots [64k, 64k + 64), and lanes past nchunks re-read the tile's last
// chunk, so every load stays inside the input. NI instructions cover up to 64 NI chunks.
template <int NI>
__device__ __forceinline__ void dma_dense(uint4* buf, const uint4* src, int nchunks, int lane) {
  const char* base = reinterpret_cast<const char*>(src);  // wave-uniform
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    if (64 * k < nchunks) {  // wave-uniform
      const int s = k * 64 + lane;
      const uint32_t off = static_cast<uint32_t>(s < nchunks ? s : nchunks - 1) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, kNonTemporal);
    }
  }
}

// Direct-to-LDS loads of ndw >= 1 consecutive dwords from src (4-byte aligned) into
// buf32[0, ndw): instruction k writes slots [64k, 64k + 64), lanes past ndw re-read the last
// dword, so every load stays inside the input. NI instructions cover up to 64 NI dwords.
template <int NI>
__device__ __forceinline__ void dma_dwords(uint32_t* buf32, const uint32_t* src, int ndw, int lane) {
  const char* base = reinterpret_cast<const char*>(src);  // wave-uniform
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    if (64 * k < ndw) {  // wave-uniform
      const int s = k * 64 + lane;
      const uint32_t off = static_cast<uint32_t>(s < ndw ? s : ndw - 1) * 4u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf32 + k * 64), 4, 0, kNonTemporal);
    }
  }
}

// The fp16 coordinates [cq, cq + C) of vector vl of a tile of n elements (rows of dh, C even)
// held densely in LDS as dwords by dma_dwords, as C / 2 fp16 pairs, zero from coordinate dh
// on. The lane's first element e0 = vl dh + cq sits in the upper half of a dword when e0 is
// odd; its pairs are then re-cut across the dword boundaries. A tile of odd n has only
// (n - 1) / 2 dwords in LDS (the last dword would reach past the input); its last element
// tx[n - 1] is read from HBM by the lanes that need it (tx: the tile's first element).
// Reads past the vector's row stay inside the buffer and are masked.
template <int C>
__device__ __forceinline__ void ragged_pairs(const uint32_t* b32, const uint16_t* tx, int vl, int cq, int dh, int n,
                                             uint32_t (&xr)[C / 2]) {
#pragma unroll
  for (int p = 0; p < C / 2; ++p) xr[p] = 0u;
  if (cq >= dh) return;  // the lane's slice is all padding
  const int e0 = vl * dh + cq, bi = e0 >> 1;
  uint32_t w[C / 2 + 1];
#pragma unroll
  for (int k = 0; k <= C / 2; ++k) w[k] = b32[bi + k];
  if (n & 1) {              // wave-uniform
    const int mdw = n >> 1;  // the dword left out: its low half is element n - 1
    if (mdw >= bi && mdw <= bi + C / 2) {
      const uint32_t xl = tx[n - 1];
#pragma unroll
      for (int k = 0; k <= C / 2; ++k)
        if (bi + k == mdw) w[k] = xl;
    }
  }
  const bool odd = (e0 & 1) != 0;
#pragma unroll
  for (int p = 0; p < C / 2; ++p) {
    const uint32_t pr = odd ? __builtin_amdgcn_alignbit(w[p + 1], w[p], 16) : w[p];
    const int c = cq + 2 * p;
    xr[p] = c + 1 < dh ? pr : (c < dh ? (pr & 0xFFFFu) : 0u);
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


// ------------------------------------------------------------------------------ code access

// Where a lane finds the codes of its C coordinates in a packed stream.
template <int D, int BITS, int CM = 32>
struct CodeShape {
  static constexpr int C = Layout<D, CM>::C, L = Layout<D, CM>::L;
  static constexpr int EPW = 32 / BITS;                // codes per word
  static constexpr int NW = (D + EPW - 1) / EPW;       // words per vector per stream
  static constexpr bool STAGED = BITS == 3 && L > 1;   // 10-code words straddle lanes
  // STAGED with 32 codes per lane: the lane's codes are bits [96 q, 96 q + 96) of the
  // vector's stream without the words' two spare bits, which always lie in the four
  // consecutive words from floor(96 q / 30) on; the lane loads those and takes its codes
  // out in registers (slice3_codes)
  static constexpr bool DIRECT3 = STAGED && C == 32;
  static constexpr bool SUB = !STAGED && L > 1 && C < EPW;  // a word holds several lanes' codes
  // words a lane loads per stream: its own NWL consecutive words, or for DIRECT3 the four
  // words that hold its slice, or for other STAGED shapes words q, q + L, ... of the vector
  // (regrouped through LDS by stage_codes), or for SUB the one word holding its codes,
  // shifted so that they start at bit 0
  static constexpr int NWL = DIRECT3 ? 4 : STAGED ? (NW + L - 1) / L : SUB ? 1 : (L == 1 ? NW : C / EPW);
  static constexpr int CSTREAM = 64 * C / 4;           // STAGED: LDS dwords per stream per wave
};

// Loads the words of one stream that lane q of the vector in cache row `row` needs.
template <int D, int BITS, int CM = 32>
__device__ __forceinline__ void load_lane_words(const uint32_t* p, int64_t row, int q,
                                                uint32_t (&w)[CodeShape<D, BITS, CM>::NWL]) {
  using S = CodeShape<D, BITS, CM>;
  if constexpr (S::DIRECT3) {
    // words a .. a + 3, a = floor(96 q / 30); a + 3 is the word holding the vector's last
    // code when q = L - 1, so every index is inside the row
    const uint32_t* src = p + row * S::NW + (96 * q) / 30;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = src[k];
  } else if constexpr (S::STAGED) {
#pragma unroll
    for (int k = 0; k < S::NWL; ++k) {
      const int wi = q + S::L * k < S::NW ? q + S::L * k : S::NW - 1;
      w[k] = p[row * S::NW + wi];
    }
  } else if constexpr (S::SUB) {
    w[0] = p[row * S::NW + (q * S::C) / S::EPW] >> (BITS * ((q * S::C) % S::EPW));
  } else {
    load_words<S::NWL>(p + row * S::NW + q * S::NWL, w);
  }
}

// STAGED only: lane q of vector vl unpacks its words q, q + L, ... into one byte per code at
// bytes [D vl, D vl + D) of the wave's LDS stream `cs` (every lane of the vector writes a
// disjoint part; the caller orders these writes before the reads of codes_of).
template <int D, int BITS, int CM = 32>
__device__ __forceinline__ void stage_codes(const uint32_t (&w)[CodeShape<D, BITS, CM>::NWL], uint32_t* cs, int vl,
                                            int q) {
  using S = CodeShape<D, BITS, CM>;
#pragma unroll
  for (int k = 0; k < S::NWL; ++k) {
    const int wi = q + S::L * k;
    if (wi < S::NW) {
      const int base = vl * D + 10 * wi;                    // even
      const int cnt = D - 10 * wi < 10 ? D - 10 * wi : 10;  // even
      const uint32_t e0 = unpack4x3(w[k]), e1 = unpack4x3(w[k] >> 12), e2 = unpack4x3(w[k] >> 24);
      uint16_t* h = reinterpret_cast<uint16_t*>(cs) + (base >> 1);
      const uint16_t hv[5] = {static_cast<uint16_t>(e0), static_cast<uint16_t>(e0 >> 16),
                              static_cast<uint16_t>(e1), static_cast<uint16_t>(e1 >> 16),
                              static_cast<uint16_t>(e2)};
#pragma unroll
      for (int i = 0; i < 5; ++i)
        if (2 * i < cnt) h[i] = hv[i];
    }
  }
}

// DIRECT3: the lane's 96-bit slice from its four words w[0..3] (word a = floor(96 q / 30),
// the slice starting at bit o = 96 q - 30 a of its 30 code bits): d[0..2] with code j of
// the lane in bits [3 j, 3 j + 3) of the 96. Spare bits (30, 31) of the words are dropped.
__device__ __forceinline__ void slice3_words(const uint32_t (&w)[4], int q, uint32_t (&d)[3]) {
  const uint32_t o = static_cast<uint32_t>(96 * q - 30 * ((96 * q) / 30));  // 0, 6, 12, 18 or 24
  d[0] = __builtin_amdgcn_ubfe(w[0], o, 30u - o) | (w[1] << (30u - o));
  d[1] = __builtin_amdgcn_ubfe(w[1], o + 2u, 28u - o) | (w[2] << (28u - o));
  d[2] = __builtin_amdgcn_ubfe(w[2], o + 4u, 26u - o) | (w[3] << (26u - o));
}

// Code j (0 <= j < 32) of a DIRECT3 slice; codes 10 and 21 straddle dwords.
template <int J>
__device__ __forceinline__ uint32_t slice3_code(const uint32_t (&d)[3]) {
  if constexpr (J < 10) return __builtin_amdgcn_ubfe(d[0], 3u * J, 3u);
  else if constexpr (J == 10) return __builtin_amdgcn_alignbit(d[1], d[0], 30) & 7u;
  else if constexpr (J < 21) return __builtin_amdgcn_ubfe(d[1], 3u * J - 32u, 3u);
  else if constexpr (J == 21) return __builtin_amdgcn_alignbit(d[2], d[1], 31) & 7u;
  else return __builtin_amdgcn_ubfe(d[2], 3u * J - 64u, 3u);
}

// Code of local coordinate j (0 <= j < C) of this lane, from its own words (not STAGED).
template <int D, int BITS, int CM = 32>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[CodeShape<D, BITS, CM>::NWL], int j) {
  using S = CodeShape<D, BITS, CM>;
  return (w[j / S::EPW] >> (BITS * (j % S::EPW))) & ((1u << BITS) - 1u);
}

// Dequantized rotated-domain coordinates z[j] = table[(i1 << BITS) | i2] of this lane
// (i2 = 0 when TWO is false). `zt` is the LDS table, `cs` the wave's LDS staging area for
// STAGED codes other than DIRECT3 (two streams of CSTREAM dwords; unused otherwise).
template <int D, int BITS, bool TWO, int CM = 32>
__device__ __forceinline__ void codes_to_z(const uint32_t (&w1)[CodeShape<D, BITS, CM>::NWL],
                                           const uint32_t (&w2)[CodeShape<D, BITS, CM>::NWL], const float* zt,
                                           uint32_t* cs, int lane, int vl, int q, float (&z)[Layout<D, CM>::C]) {
  using S = CodeShape<D, BITS, CM>;
  constexpr int C = S::C;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  if constexpr (BITS == 4 && !S::SUB) {
    // a word holds 8 codes, one per nibble: the table index (i1 << 4) | i2 of coordinates
    // 0, 2, 4, 6 of a word are the bytes of one interleave of the two streams' words, those
    // of coordinates 1, 3, 5, 7 the bytes of another
#pragma unroll
    for (int k = 0; k < S::NWL; ++k) {
      const uint32_t a = w1[k], b = TWO ? w2[k] : 0u;
      const uint32_t ev = ((a << 4) & 0xF0F0F0F0u) | (b & 0x0F0F0F0Fu);
      const uint32_t od = (a & 0xF0F0F0F0u) | ((b >> 4) & 0x0F0F0F0Fu);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (8 * k + 2 * i < C) z[8 * k + 2 * i] = zt[(ev >> (8 * i)) & 0xFFu];
        if (8 * k + 2 * i + 1 < C) z[8 * k + 2 * i + 1] = zt[(od >> (8 * i)) & 0xFFu];
      }
    }
  } else if constexpr (!S::STAGED) {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const uint32_t i1 = code_at<D, BITS, CM>(w1, j);
      const uint32_t i2 = TWO ? code_at<D, BITS, CM>(w2, j) : 0u;
      z[j] = zt[(i1 << BITS) | i2];
    }
  } else if constexpr (S::DIRECT3) {
    uint32_t d1[3], d2[3] = {0u, 0u, 0u};
    slice3_words(w1, q, d1);
    if constexpr (TWO) slice3_words(w2, q, d2);
    static_for<0, 32>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      const uint32_t i1 = slice3_code<j>(d1);
      const uint32_t i2 = TWO ? slice3_code<j>(d2) : 0u;
      z[j] = zt[(i1 << 3) | i2];
    });
  } else {
    stage_codes<D, BITS, CM>(w1, cs, vl, q);
    if constexpr (TWO) stage_codes<D, BITS, CM>(w2, cs + S::CSTREAM, vl, q);
    wave_lds_fence();
#pragma unroll
    for (int d4 = 0; d4 < C / 4; ++d4) {
      const uint32_t b1 = cs[lane * (C / 4) + d4];
      const uint32_t b2 = TWO ? cs[S::CSTREAM + lane * (C / 4) + d4] : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t i1 = (b1 >> (8 * i)) & MASK, i2 = (b2 >> (8 * i)) & MASK;
        z[4 * d4 + i] = zt[(i1 << BITS) | i2];
      }
    }
    wave_lds_fence();
  }
}

// 1- and 2-bit codes: z after the first log2(G) butterfly stages, straight from a group
// table. A nibble of a stream word holds the codes of G = 4 / BITS consecutive coordinates;
// the two streams' nibbles n1 | n2 << 4 index 256 entries of G floats, the float32
// operations of the table lookups z = c1[i1] + c2[i2] followed by lane_stages' first stages
// (BITS = 2: {z0 + z1, z0 - z1}; BITS = 1: the two stages over four coordinates). The even
// and the odd nibbles of a word take their indices from the bytes of two interleaved words.
template <int BITS>
using GroupEntry = typename std::conditional<BITS == 2, float2, float4>::type;

template <int D, int BITS, bool TWO, int CM = 32>
__device__ __forceinline__ void codes_to_groups(const uint32_t (&w1)[CodeShape<D, BITS, CM>::NWL],
                                                const uint32_t (&w2)[CodeShape<D, BITS, CM>::NWL],
                                                const GroupEntry<BITS>* gt, float (&z)[Layout<D, CM>::C]) {
  using S = CodeShape<D, BITS, CM>;
  constexpr int C = S::C, G = 4 / BITS;
  static_assert(BITS == 1 || BITS == 2, "four code bits per nibble");
  static_assert(!S::STAGED && !S::SUB, "a lane's own words");
#pragma unroll
  for (int k = 0; k < S::NWL; ++k) {
    const uint32_t a = w1[k], b = TWO ? w2[k] : 0u;
    const uint32_t ev = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);  // nibbles 0, 2, 4, 6
    const uint32_t od = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);  // nibbles 1, 3, 5, 7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = S::EPW * k + 2 * G * i;  // first coordinate of nibble 2i of word k
      if (j < C) {
        const GroupEntry<BITS> e = gt[(ev >> (8 * i)) & 0xFFu];
        z[j] = e.x;
        z[j + 1] = e.y;
        if constexpr (G == 4) {
          z[j + 2] = e.z;
          z[j + 3] = e.w;
        }
      }
      if (j + G < C) {
        const GroupEntry<BITS> f = gt[(od >> (8 * i)) & 0xFFu];
        z[j + G] = f.x;
        z[j + G + 1] = f.y;
        if constexpr (G == 4) {
          z[j + G + 2] = f.z;
          z[j + G + 3] = f.w;
        }
      }
    }
  }
}

// The inverse rotation of this lane's slice and the conversion to fp16 pairs:
// o = RN16(K * (H z)) per coordinate pair, H applied in registers then across the L lanes
// of the vector. K must carry the lane's sign (-1)^popcount(q) (see cross_stage); the
// caller applies the final diag(s) to the fp16 pairs (an XOR of sign bits). H0 > 1: z has
// had the in-register stages below H0 already (codes_to_groups).
template <int D, int CM = 32, int H0 = 1>
__device__ __forceinline__ void unrotate_f16(float (&z)[(Layout<D, CM>::C)], float K, int q,
                                             uint32_t (&o)[(Layout<D, CM>::C) / 2]) {
  constexpr int C = Layout<D, CM>::C;
  lane_stages<C, H0>(z);
  cross_stages<C, Layout<D, CM>::LOG_L>(z, q);
#pragma unroll
  for (int m = 0; m < C / 2; ++m) {
    const half2_t h = {static_cast<_Float16>(z[2 * m] * K), static_cast<_Float16>(z[2 * m + 1] * K)};
    o[m] = __builtin_bit_cast(uint32_t, h);
  }
}

}  // namespace kvq
