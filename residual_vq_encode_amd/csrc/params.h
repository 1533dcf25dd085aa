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
constexpr int kTab1Max = 24;  // stage-1 bucket table entries (bits >= 3)
constexpr int kTab2Max = 40;  // stage-2 bucket table entries (bits >= 3)

// Where token s of (b, h) lands in a cache whose token axis has capacity S_cap:
// row(v) = (v / S) * S_cap + s_offset + v % S for the flattened input index v.
struct RowMap {
  int64_t S, S_cap, s_offset;
  float inv_S;         // 1/S, used for the small quotients of S <= 64
  int32_t contiguous;  // S == S_cap and s_offset == 0: row(v) = v
};

struct EncodeArgs {
  const uint16_t* x;  // fp16 [n_vec, d]
  uint32_t* p1;       // [rows, n_words]
  uint32_t* p2;
  float* norms;       // [rows]
  int64_t n_vec;
  RowMap map;
  // Per-vector scale: the quantizer works on X = y_true * unit, and the kernel forms
  // -X = fma(y', -k_scale / n, +0) from the raw transform y' = H diag(s) x.
  float k_scale;
  float r12;          // stage-2 units per stage-1 unit
  float cm2[2];       // bits = 1: cm2[0] = stage-1 centroid magnitude in stage-2 units;
                      // bits = 2: cm2[0] = half the gap between the two centroid magnitudes,
                      // in stage-2 units
  int32_t j1max, j2max;  // bits >= 3: last bucket index of each table
  // bits >= 3 bucket tables: {threshold, count below the bucket (int bits), centroid
  // magnitude below/above the threshold in stage-2 units} and {threshold, count below}.
  float tab1[kTab1Max][4];
  float tab2[kTab2Max][2];
  // Per-pair XOR masks flipping fp16 sign bits: pair m covers coordinates 2m (bit 15)
  // and 2m + 1 (bit 31).
  uint32_t xmask[512];
};

struct DecodeArgs {
  const uint32_t* p1;
  const uint32_t* p2;
  const float* norms;  // nullptr: unit reconstructions
  uint16_t* x;         // fp16 [n_vec, d]
  int64_t n_vec;
  RowMap map;
  float inv_sqrt_d;
  float ztab[256];     // c1[i1] + c2[i2] (float32 sum), index (i1 << bits) | i2
  uint32_t xmask[512]; // per-pair XOR masks flipping fp16 sign bits (the final diag(s))
};

}  // namespace kvq

namespace kvq {

// Attention over a packed cache (attend.hip): scores of the query against every cached key
// and the softmax-weighted sum of the cached values, both caches read packed.
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
