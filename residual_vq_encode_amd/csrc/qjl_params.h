// Kernel parameter block of the 1-bit sign-sketch encoder (qjl.hip; internal, not part of
// the C ABI). The sketch matrix stays in the caller's device memory; everything else
// travels by value in the kernel-argument segment.
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

}  // namespace kvq
