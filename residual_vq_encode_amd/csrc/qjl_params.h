// Kernel parameter block and launch geometry of the 1-bit sign-sketch encoder (qjl.hip;
// internal, not part of the C ABI), shared with the host-side checks in api.cpp. The sketch
// matrix stays in the caller's device memory; everything else travels by value in the
// kernel-argument segment.
#pragma once

#include <stdint.h>

#include "params.h"

namespace kvq {

struct QjlArgs {
  const uint16_t* x;       // fp16 [n_vec, d]
  const uint16_t* sketch;  // fp16 [m, d], row-major
  uint32_t* packed;        // [rows, m / 32]: bit j of word w is [ (S x)_{32 w + j} >= 0 ]
  uint16_t* norms;         // fp16 [rows]
  int64_t n_vec;
  RowMap map;
};

constexpr int kQjlTile = 32;  // keys per wave tile: the 32 columns of one MFMA block

// Waves per block: each holds a tile of 32 keys (64 d bytes) in LDS next to the one copy
// of the sketch the block shares. At d = 128, m = 128 a block takes 64 KiB, so two blocks
// (two waves per SIMD) share a CU. Measured on the Llama-layer keys: 4 waves per block
// 19.0 us, 8 waves 20.9 us, 16 waves (one block per CU) 19.7 us; the sketch held in
// registers instead of LDS 20.6 us. The loads alone take 15.4 us and the arithmetic alone
// 11-13 us, so the remaining loss is their imperfect overlap.
template <int D>
constexpr int qjl_waves() {
  return 4;
}

constexpr int64_t kQjlLdsMax = 160 * 1024;  // LDS per workgroup (and per CU) on gfx950

// LDS bytes of one block: the sketch (m rows of d fp16) and one tile per wave.
template <int D>
constexpr int64_t qjl_lds_bytes(int m) {
  return (static_cast<int64_t>(m) * D + static_cast<int64_t>(qjl_waves<D>()) * kQjlTile * D) * 2;
}

// LDS bytes a launch needs for head dimension d and sketch size m (0: unsupported d).
inline int64_t qjl_lds_need(int d, int m) {
  switch (d) {
    case 32: return qjl_lds_bytes<32>(m);
    case 64: return qjl_lds_bytes<64>(m);
    case 128: return qjl_lds_bytes<128>(m);
    case 256: return qjl_lds_bytes<256>(m);
    default: return 0;
  }
}

}  // namespace kvq
