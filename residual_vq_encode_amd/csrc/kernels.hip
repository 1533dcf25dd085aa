// Dispatch of the codec kernels (codec.h) for head dimensions that are powers of two or
// multiples of 8; other head dimensions go to kernels_ragged.hip.
#include "codec.h"

namespace kvq {

hipError_t launch_encode_ragged(const EncodeArgs& a, int p, int bits, int stages, hipStream_t stream);
hipError_t launch_decode_ragged(const DecodeArgs& a, int p, int bits, int stages, hipStream_t stream);

#define KVQ_FOR_BITS(MACRO, D, S, R)                                                        \
  case 1: return MACRO<D, 1, S, R>; case 2: return MACRO<D, 2, S, R>; case 3: return MACRO<D, 3, S, R>; \
  case 4: return MACRO<D, 4, S, R>;

// ROWS = kRowsChunks: the head dimension is a multiple of 8 below the rotation length D (so
// at least 24, and D at least 32); the sign code takes powers of two only.
template <int D, int ROWS>
static auto encode_fn(int bits, int stages) -> hipError_t (*)(const EncodeArgs&, hipStream_t) {
  if constexpr (ROWS == kRowsChunks && D < 32) {
    return nullptr;
  } else {
    if (stages == 2) {
      switch (bits) { KVQ_FOR_BITS(launch_encode_t, D, 2, ROWS) }
    } else if (stages == 1) {
      switch (bits) { KVQ_FOR_BITS(launch_encode_t, D, 1, ROWS) }
    } else if (stages == 0 && bits == 1 && ROWS == kRowsFull) {
      return launch_encode_t<D, 1, 0, kRowsFull>;
    }
    return nullptr;
  }
}
template <int D, int ROWS>
static auto decode_fn(int bits, int stages) -> hipError_t (*)(const DecodeArgs&, hipStream_t) {
  if constexpr (ROWS == kRowsChunks && D < 32) {
    return nullptr;
  } else {
    if (stages == 2) {
      switch (bits) { KVQ_FOR_BITS(launch_decode_t, D, 2, ROWS) }
    } else if (stages == 1) {
      switch (bits) { KVQ_FOR_BITS(launch_decode_t, D, 1, ROWS) }
    }
    return nullptr;
  }
}

#define KVQ_FOR_P(FN, bits, stages, chunks)                                                            \
  switch (p) {                                                                                     \
    case 8: f = FN<8, kRowsFull>(bits, stages); break;                                               \
    case 16: f = FN<16, kRowsFull>(bits, stages); break;                                             \
    case 32: f = chunks ? FN<32, kRowsChunks>(bits, stages) : FN<32, kRowsFull>(bits, stages); break;  \
    case 64: f = chunks ? FN<64, kRowsChunks>(bits, stages) : FN<64, kRowsFull>(bits, stages); break;  \
    case 128: f = chunks ? FN<128, kRowsChunks>(bits, stages) : FN<128, kRowsFull>(bits, stages); break; \
    case 256: f = chunks ? FN<256, kRowsChunks>(bits, stages) : FN<256, kRowsFull>(bits, stages); break; \
    case 512: f = chunks ? FN<512, kRowsChunks>(bits, stages) : FN<512, kRowsFull>(bits, stages); break; \
    case 1024: f = chunks ? FN<1024, kRowsChunks>(bits, stages) : FN<1024, kRowsFull>(bits, stages); break; \
    default: break;                                                                                \
  }

// Launchers used by api.cpp (d the head dimension in [8, 1024]; the kernels run at its
// rotation length). Return hipErrorInvalidValue for an unsupported (d, bits, stages) or more
// than 2^31 - 1 tiles.
hipError_t launch_encode(const EncodeArgs& a, int d, int bits, int stages, hipStream_t stream) {
  if (d < 8 || d > 1024 || a.dh != d) return hipErrorInvalidValue;
  const int p = rotation_length(d), mode = row_mode(d);
  if (mode == kRowsRagged) return launch_encode_ragged(a, p, bits, stages, stream);
  hipError_t (*f)(const EncodeArgs&, hipStream_t) = nullptr;
  KVQ_FOR_P(encode_fn, bits, stages, mode == kRowsChunks)
  return f ? f(a, stream) : hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int d, int bits, int stages, hipStream_t stream) {
  if (d < 8 || d > 1024 || a.dh != d) return hipErrorInvalidValue;
  const int p = rotation_length(d), mode = row_mode(d);
  if (mode == kRowsRagged) return launch_decode_ragged(a, p, bits, stages, stream);
  hipError_t (*f)(const DecodeArgs&, hipStream_t) = nullptr;
  KVQ_FOR_P(decode_fn, bits, stages, mode == kRowsChunks)
  return f ? f(a, stream) : hipErrorInvalidValue;
}

}  // namespace kvq
