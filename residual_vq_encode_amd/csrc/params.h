// Kernel parameter blocks of libkvq (internal; not part of the C ABI).
//
// Both kernels take one of these by value, so everything a launch needs (pointers,
// sizes, per-call constants, the rotation's signs in the form each kernel uses, small
// lookup tables) travels in the kernel-argument segment and no device memory is
// allocated. The host fills them from a kvq_codebooks struct (api.cpp).
#pragma once

#include <stdint.h>

namespace kvq {

constexpr int kWaveSize = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWaveSize * kWavesPerBlock;
// Bucket tables of the 3- and 4-bit quantizers. A value t of either stage is scaled to
// w = t / (2R) (R: a little more than the stage's largest threshold magnitude), compared
// in that form, and located through v = clamp(w + 1/2, 0, 1): the entry is
// RNE(v * kTabSub * kTabBuckets) / kTabSub, i.e. the kTabBuckets + 1 entries split [0, 1]
// evenly. The integer is taken from the float32 bits of v + 2^e, whose spacing is
// 1 / (kTabSub * kTabBuckets) in [2^e, 2^(e+1)): masked, they are the entry's byte offset.
// Stage 1 entries are 16 bytes (kTabSub = 16, e = 13), stage 2 entries 8 bytes (kTabSub = 8,
// e = 14).
constexpr uint32_t kOnePair = 0x3C003C00u;  // two fp16 1.0 values

constexpr int kTabBuckets = 64;
constexpr int kTabEntries = kTabBuckets + 1;

// Vectors per wave tile of the matrix-core encode (the 16 columns of its MFMA).
constexpr int kMxTile = 16;

// Rotation length of head dimension d: the power of two >= d. A head dimension that is not
// a power of two is rotated zero-padded to it, and its codes are those of all P rotated
// coordinates.
constexpr int rotation_length(int d) {
  int p = 8;
  while (p < d) p *= 2;
  return p;
}

// How the fp16 rows of head dimension d sit against the rotation length p the kernels run
// at: d = p (kRowsFull); d a multiple of 8 below p, rows of d / 8 16-byte chunks
// (kRowsChunks); any other d, rows of d elements that are not 16-byte aligned (kRowsRagged).
// Either way the p - d missing coordinates are the zeros of the padded vector.
constexpr int kRowsFull = 0;
constexpr int kRowsChunks = 1;
constexpr int kRowsRagged = 2;
constexpr int row_mode(int d) {
  return d == rotation_length(d) ? kRowsFull : (d % 8 == 0 ? kRowsChunks : kRowsRagged);
}

// The encodes of D = 128 (every bit width) and D = 256 (1, 2 and 4 bits) run their
// transform on the matrix cores; every other shape (padded ones included) takes the
// butterfly kernel.
constexpr bool encode_on_matrix_cores(int d, int bits) {
  return (d == 128 && bits >= 1) || (d == 256 && bits >= 1 && bits != 3);
}

// Vectors per wave tile (the unit of work of the persistent grids, indexed with 32-bit
// integers): the matrix-core encode takes 16; the butterfly kernels spread a vector over
// p / min(p, 32) lanes of a 64-lane wave, p the rotation length.
constexpr int64_t butterfly_tile_vectors(int p) { return 64 / (p / (p < 32 ? p : 32)); }
constexpr int64_t encode_tile_vectors(int d, int bits) {
  return encode_on_matrix_cores(d, bits) ? kMxTile : butterfly_tile_vectors(rotation_length(d));
}
constexpr int64_t decode_tile_vectors(int d) { return butterfly_tile_vectors(rotation_length(d)); }

// Where token s of (b, h) lands in a cache whose token axis has capacity S_cap:
// row(v) = (v / S) * S_cap + s_offset + v % S for the flattened input index v.
struct RowMap {
  int64_t S, S_cap, s_offset;
  float inv_S;         // 1/S, used for the small quotients of S <= 64
  int32_t contiguous;  // S == S_cap and s_offset == 0: row(v) = v
};

struct EncodeArgs {
  const uint16_t* x;  // fp16 [n_vec, d]
  int32_t dh;         // head dimension d: fp16 elements of an input row (at most p)
  uint32_t* p1;       // [rows, n_words]
  uint32_t* p2;
  float* norms;       // [rows]
  int64_t n_vec;
  RowMap map;
  // Per-vector scale: the quantizer works on X = y_true * unit, and the kernel forms
  // -X = fma(y', -k_scale / n, +0) from the raw transform y' = H diag(s) x (bits <= 2);
  // bits >= 3: w1 = fma(y', k_scale / n, +0) = y_true / (2 R1) (R1 chosen so that
  // k_scale = 1 / (sqrt(d) 2 R1) is exact).
  float k_scale;
  float r12;          // stage-2 units per stage-1 unit (bits <= 2)
  float k2_scale;     // bits >= 3: w2 = fma(y', k2_scale / n, -c1[m] / (2 R2)), exact too
  float cm2[2];       // bits = 1: cm2[0] = stage-1 centroid magnitude in stage-2 units;
                      // bits = 2: cm2[0] = half the gap between the two centroid magnitudes,
                      // in stage-2 units
  // bits >= 3 bucket tables (see kTabBuckets): stage 1 {threshold in w1, count of
  // thresholds below the bucket (int bits), -c1[count] / (2 R2), the same for count + 1};
  // stage 2 {threshold in w2, count below}. A bucket without a threshold holds +inf
  // (never exceeded).
  float tab1[kTabEntries][4];
  float tab2[kTabEntries][2];
  // Per-pair fp16 weights (s_2m, s_2m+1) of the first butterfly stages: the pair (1, 1)
  // with the sign bit of each coordinate the rotation negates set (bit 15: coordinate 2m,
  // bit 31: 2m + 1). The host folds the signs into the pair so the kernel's prologue only
  // loads them; each wave sees only a few tiles, so its setup counts.
  uint32_t wpair[512];
};

struct DecodeArgs {
  const uint32_t* p1;
  const uint32_t* p2;
  const float* norms;  // nullptr: unit reconstructions
  uint16_t* x;         // fp16 [n_vec, d]
  int32_t dh;          // head dimension d: fp16 elements of an output row (at most p)
  int64_t n_vec;
  RowMap map;
  float inv_sqrt_d;    // 1 / sqrt(p), p the rotation length
  float ztab[256];     // c1[i1] + c2[i2] (float32 sum), index (i1 << bits) | i2
  uint32_t xmask[512]; // per-pair XOR masks flipping fp16 sign bits (the final diag(s))
};

}  // namespace kvq

namespace kvq {

// Attention over a packed cache (attend.hip): scores of the query against every cached key
// and the softmax-weighted sum of the cached values, both caches read packed.
// Bytes of device scratch behind kvq_rvq_attend_noalloc: 32 MiB holds the partial records
// of a decode step (a few query positions) at every supported d up to 16 query heads per
// key/value head.
constexpr int64_t kAttendScratchBytes = int64_t(32) << 20;

struct AttendArgs {
  const uint16_t* q;                // fp16 [B, Hq, Sq, d]
  const uint32_t* k1;               // key cache streams [B, Hkv, S_cap, n_words]
  const uint32_t* k2;
  const float* kn;                  // key norms [B, Hkv, S_cap]
  const uint32_t* v1;               // value cache streams
  const uint32_t* v2;
  const float* vn;
  float* ws;                        // per (query vector, split): {m, l, 0, 0, acc[d]}
  uint16_t* out;                    // fp16 [B, Hq, Sq, d]
  int64_t n_q;                      // B * Hq * Sq query vectors
  int64_t S_cap, S_kv;
  int32_t Hkv, group, Sq;           // group = Hq / Hkv query heads per key/value head
  int32_t chunk, n_splits;          // keys per split, splits per query vector
  float qscale;                     // scale * log2(e) / sqrt(d): scores come out in base-2 units
  float inv_sqrt_d;
  float ztab_k[256];                // c1[i1] + c2[i2] of the key codebooks, index (i1 << bits) | i2
  float ztab_v[256];                // the same for the value codebooks
  uint32_t ksign[32];               // bit j: the key rotation negates coordinate j
  uint32_t vsign[32];               // the same for the values
};

}  // namespace kvq
