// Dispatch of the codec kernels (codec.h) for head dimensions whose fp16 rows are not
// 16-byte aligned (d not a multiple of 8): the rows are moved as dwords (see kRowsRagged).
// Kept apart from kernels.hip so the two halves of the kernel set compile in parallel.
#include "codec.h"

namespace kvq {

#define KVQ_RAGGED_BITS(MACRO, D, S)                                                                   \
  case 1: return MACRO<D, 1, S, kRowsRagged>; case 2: return MACRO<D, 2, S, kRowsRagged>;              \
  case 3: return MACRO<D, 3, S, kRowsRagged>; case 4: return MACRO<D, 4, S, kRowsRagged>;

template <int D>
static auto encode_ragged_fn(int bits, int stages) -> hipError_t (*)(const EncodeArgs&, hipStream_t) {
  if (stages == 2) {
    switch (bits) { KVQ_RAGGED_BITS(launch_encode_t, D, 2) }
  } else if (stages == 1) {
    switch (bits) { KVQ_RAGGED_BITS(launch_encode_t, D, 1) }
  }
  return nullptr;  // the sign code takes powers of two only
}
template <int D>
static auto decode_ragged_fn(int bits, int stages) -> hipError_t (*)(const DecodeArgs&, hipStream_t) {
  if (stages == 2) {
    switch (bits) { KVQ_RAGGED_BITS(launch_decode_t, D, 2) }
  } else if (stages == 1) {
    switch (bits) { KVQ_RAGGED_BITS(launch_decode_t, D, 1) }
  }
  return nullptr;
}

#define KVQ_RAGGED_P(FN)                  \
  switch (p) {                            \
    case 16: f = FN<16>(bits, stages); break;     \
    case 32: f = FN<32>(bits, stages); break;     \
    case 64: f = FN<64>(bits, stages); break;     \
    case 128: f = FN<128>(bits, stages); break;   \
    case 256: f = FN<256>(bits, stages); break;   \
    case 512: f = FN<512>(bits, stages); break;   \
    case 1024: f = FN<1024>(bits, stages); break; \
    default: break;                       \
  }

// p: the rotation length (16 to 1024: d is at least 9).
hipError_t launch_encode_ragged(const EncodeArgs& a, int p, int bits, int stages, hipStream_t stream) {
  hipError_t (*f)(const EncodeArgs&, hipStream_t) = nullptr;
  KVQ_RAGGED_P(encode_ragged_fn)
  return f ? f(a, stream) : hipErrorInvalidValue;
}

hipError_t launch_decode_ragged(const DecodeArgs& a, int p, int bits, int stages, hipStream_t stream) {
  hipError_t (*f)(const DecodeArgs&, hipStream_t) = nullptr;
  KVQ_RAGGED_P(decode_ragged_fn)
  return f ? f(a, stream) : hipErrorInvalidValue;
}

}  // namespace kvq
