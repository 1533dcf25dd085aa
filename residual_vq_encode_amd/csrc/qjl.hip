// HIP kernel for gfx950 (MI355X): the QJL key encoder, a 1-bit Johnson-Lindenstrauss sign
// sketch fused with bit packing and the key norm.
//
// Method (VeloxQuant-MLX blog, "turboquant" tag page, "Kernel 4: QJL Encode"): for a fixed
// sketch matrix S [m, d] and every key vector x, the m signs of S x, bit j set when
// (S x)_j >= 0, packed LSB-first so that bit j of the packed sequence is sketch dimension j
// (byte k, bit i of the pages' byte layout is bit 8k + i here; on a little-endian machine
// the bytes are the same), plus the norm |x| rounded to fp16.
//
// S x for a tile of 32 keys is a dense [m x d] x [d x 32] product, so it runs on the matrix
// cores: v_mfma_f32_32x32x16_f16 multiplies the fp16 operands exactly and accumulates in
// float32. The tile is streamed into the wave's LDS buffer with direct-to-LDS 16-byte loads;
// the sketch sits in LDS for the whole (persistent) block, one copy shared by its waves.
//
// MFMA layout (32x32x16): lane l supplies row l % 32 of the A block and column l % 32 of the
// B block, each with the 8 k-values 8 (l / 32) + [0, 8) of the 16-wide k-step, and receives
// the 16 results D[8 (j / 4) + 4 (l / 32) + j % 4][l % 32], j < 16. A = sketch rows (M), B =
// keys (N). The sketch rows are fed in the order that makes lane half h = l / 32 receive
// sketch dimensions 32 mb + 16 h + j of M-block mb in register j, so each lane turns its 16
// results into 16 consecutive sign bits and the two halves of a 32-bit word meet in lanes l
// and l ^ 32.
#include <hip/hip_runtime.h>

#include <climits>

#include "device.h"
#include "qjl_params.h"

namespace kvq {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// LDS chunk swizzle: chunk c of row r (a sketch row or a key of the tile) is stored at
// position c ^ (r & mask), so the 32 rows an MFMA operand read touches spread over the
// banks instead of all hitting one 16-byte group.
template <int D>
constexpr int qjl_chunk_mask() {
  return (D / 8 < 16 ? D / 8 : 16) - 1;
}


template <int D, int MB, bool CONTIG>
__global__ __launch_bounds__(qjl_waves<D>() * 64) void qjl_encode_kernel(const QjlArgs a) {
  constexpr int WPB = qjl_waves<D>();
  constexpr int CPV = D / 8;              // 16-byte chunks per key and per sketch row
  constexpr int SWM = qjl_chunk_mask<D>();
  constexpr int KS = D / 16;              // MFMA k-steps
  constexpr int TCH = kQjlTile * CPV;     // chunks per tile
  static_assert(TCH % 64 == 0, "a tile is a whole number of 1 KiB direct-to-LDS loads");

  extern __shared__ u32x4_t lds[];
  u32x4_t* sk = lds;  // sketch, MB * 32 rows
  {
    const u32x4_t* sg = reinterpret_cast<const u32x4_t*>(a.sketch);
    for (int i = threadIdx.x; i < MB * 32 * CPV; i += WPB * 64) {
      const int r = i / CPV, c = i % CPV;
      sk[r * CPV + (c ^ (r & SWM))] = sg[i];
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4_t* buf = lds + MB * 32 * CPV + wv * TCH;
  const int v = lane & 31;  // this lane's key in the tile (MFMA column)
  const int h = lane >> 5;  // k-values 8h..8h+7 of each step; sketch dims 16h..16h+15 of each 32
  // sketch row (within an M-block) feeding MFMA row v: row 8 (j/4) + 4 h' + j % 4 must carry
  // sketch dimension 16 h' + j
  const int srow = 16 * ((v >> 2) & 1) + 4 * (v >> 3) + (v & 3);
  const int n_tiles = static_cast<int>((a.n_vec + kQjlTile - 1) / kQjlTile);  // < 2^31 (host)
  const int stride = static_cast<int>(gridDim.x) * WPB;
  const char* xb = reinterpret_cast<const char*>(a.x);

  // Direct-to-LDS loads of tile t: instruction k fills slots [64k, 64k + 64); slot s holds
  // chunk (s % CPV) ^ (key & SWM) of key s / CPV. Keys past the input's end re-read its last
  // key, so every load stays inside the input; their results are never stored.
  auto dma = [&](int t) {
    const int64_t v0 = static_cast<int64_t>(t) * kQjlTile;
    const int nv = static_cast<int>(a.n_vec - v0 < kQjlTile ? a.n_vec - v0 : kQjlTile);
    const char* base = xb + v0 * (2 * D);  // wave-uniform
#pragma unroll
    for (int k = 0; k < TCH / 64; ++k) {
      const int s = k * 64 + lane, kv = s / CPV, p = s % CPV;
      const int rv = kv < nv ? kv : nv - 1;
      const uint32_t off = static_cast<uint32_t>(rv * CPV + (p ^ (kv & SWM))) * 16u;
      __builtin_amdgcn_global_load_lds((gptr_t)(base + off), (lptr_t)(buf + k * 64), 16, 0, kNonTemporal);
    }
  };

  int tile = static_cast<int>(blockIdx.x) * WPB + wv;
  if (tile < n_tiles) dma(tile);

  // results of the previous tile, stored after the next tile's loads have been issued
  uint32_t words[MB];
  uint16_t nrm16 = 0;
  int64_t row = -1;  // cache row of this lane's key; -1: nothing held

  for (; tile < n_tiles; tile += stride) {
    const int64_t v0 = static_cast<int64_t>(tile) * kQjlTile;
    const int nv = static_cast<int>(a.n_vec - v0 < kQjlTile ? a.n_vec - v0 : kQjlTile);
    wait_vmem();  // this tile has landed (and the stores issued before it are done)
    f16x8_t b[KS];  // key v, k-values 16 ks + 8 h + [0, 8)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) b[ks] = __builtin_bit_cast(f16x8_t, buf[v * CPV + ((2 * ks + h) ^ (v & SWM))]);
    wait_lds();  // the buffer may now be refilled
    if (tile + stride < n_tiles) dma(tile + stride);

    if (row >= 0) {
      constexpr int PER = MB % 2 == 0 ? MB / 2 : MB;  // words stored by each lane half
      if (MB % 2 == 0 || h == 0) {
        uint32_t part[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) part[i] = words[(MB % 2 == 0 ? h * PER : 0) + i];
        store_words<PER>(a.packed + row * MB + (MB % 2 == 0 ? h * PER : 0), part);
      }
      if (h == 0) a.norms[row] = nrm16;
    }

    // |x|: squares of the fp16 values summed in float32 (v_dot2_f32_f16), both lane halves
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, b[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // through a scalar: bit-casting the vector element w[i] directly compiled to w[0]
        // for every i
        const uint32_t e = w[i];
        const half2_t p = __builtin_bit_cast(half2_t, e);
        ss = __builtin_amdgcn_fdot2(p, p, ss, false);
      }
    }
    ss += __shfl_xor(ss, 32);
    const float nrm = __builtin_amdgcn_sqrtf(ss);  // v_sqrt_f32, within 1 ulp (the fp16 result is held to 1e-6)

    // S x on the matrix cores, MBC M-blocks at a time (independent accumulators, k-steps
    // outermost), then their signs: register j of M-block mb is sketch dimension
    // 32 mb + 16 h + j. The sign bit of (value + 0) is [value < 0] (adding +0 turns a -0
    // into +0, which counts as >= 0); the chain shifts the highest dimension in first so
    // dimension j ends at bit j.
    constexpr int MBC = MB % 2 == 0 ? 2 : 1;
#pragma unroll
    for (int m0 = 0; m0 < MB; m0 += MBC) {
      f32x16_t acc[MBC];
#pragma unroll
      for (int i = 0; i < MBC; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int i = 0; i < MBC; ++i) {
          const f16x8_t sa =
              __builtin_bit_cast(f16x8_t, sk[(32 * (m0 + i) + srow) * CPV + ((2 * ks + h) ^ (srow & SWM))]);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa, b[ks], acc[i], 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < MBC; ++i) {
        uint32_t u = 0;
#pragma unroll
        for (int j = 15; j >= 0; --j) u = __builtin_amdgcn_alignbit(u, __float_as_uint(acc[i][j] + 0.0f), 31);
        const uint32_t hw = ~u & 0xFFFFu;
        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hw), 32));
        words[m0 + i] = h == 0 ? (hw | (other << 16)) : (other | (hw << 16));
      }
    }
    nrm16 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(nrm));
    row = v < nv ? cache_row<CONTIG>(a.map, v0, v) : -1;
  }

  if (row >= 0) {
    constexpr int PER = MB % 2 == 0 ? MB / 2 : MB;
    if (MB % 2 == 0 || h == 0) {
      uint32_t part[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) part[i] = words[(MB % 2 == 0 ? h * PER : 0) + i];
      store_words<PER>(a.packed + row * MB + (MB % 2 == 0 ? h * PER : 0), part);
    }
    if (h == 0) a.norms[row] = nrm16;
  }
}

// --------------------------------------------------------------------------------- launch

template <int D, int MB>
static hipError_t launch_qjl_t(const QjlArgs& a, hipStream_t stream) {
  const void* f = a.map.contiguous ? reinterpret_cast<const void*>(&qjl_encode_kernel<D, MB, true>)
                                   : reinterpret_cast<const void*>(&qjl_encode_kernel<D, MB, false>);
  const int64_t lds = qjl_lds_bytes<D>(MB * 32);
  static int cap[2] = {0, 0};  // resident blocks on the device, asked once per kernel
  int& c = cap[a.map.contiguous ? 1 : 0];
  if (c == 0) {
    int per_cu = 0, dev = 0, cus = 0;
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, qjl_waves<D>() * 64, lds);
    if (e != hipSuccess) return e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    c = (per_cu > 0 ? per_cu : 1) * cus;
  }
  const int64_t tiles = (a.n_vec + kQjlTile - 1) / kQjlTile;
  if (tiles > INT_MAX / 2) return hipErrorInvalidValue;
  const int64_t want = (tiles + qjl_waves<D>() - 1) / qjl_waves<D>();
  const int blocks = static_cast<int>(want < c ? want : c);
  void* args[] = {const_cast<QjlArgs*>(&a)};
  return hipLaunchKernel(f, dim3(blocks), dim3(qjl_waves<D>() * 64), args, static_cast<size_t>(lds), stream);
}

template <int D>
static hipError_t launch_qjl_d(const QjlArgs& a, int m, hipStream_t stream) {
  // m = 32 MB; the sketch and the tiles fit the LDS (checked on the host)
  switch (m / 32) {
    case 1: return launch_qjl_t<D, 1>(a, stream);
    case 2: return launch_qjl_t<D, 2>(a, stream);
    case 3: return launch_qjl_t<D, 3>(a, stream);
    case 4: return launch_qjl_t<D, 4>(a, stream);
    case 5: if constexpr (qjl_lds_bytes<D>(160) <= kQjlLdsMax) return launch_qjl_t<D, 5>(a, stream); break;
    case 6: if constexpr (qjl_lds_bytes<D>(192) <= kQjlLdsMax) return launch_qjl_t<D, 6>(a, stream); break;
    case 7: if constexpr (qjl_lds_bytes<D>(224) <= kQjlLdsMax) return launch_qjl_t<D, 7>(a, stream); break;
    case 8: if constexpr (qjl_lds_bytes<D>(256) <= kQjlLdsMax) return launch_qjl_t<D, 8>(a, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// Launcher used by api.cpp.
hipError_t launch_qjl(const QjlArgs& a, int d, int m, hipStream_t stream) {
  switch (d) {
    case 32: return launch_qjl_d<32>(a, m, stream);
    case 64: return launch_qjl_d<64>(a, m, stream);
    case 128: return launch_qjl_d<128>(a, m, stream);
    case 256: return launch_qjl_d<256>(a, m, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
