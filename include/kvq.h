/*
 * kvq.h - C ABI of the MI355X two-stage residual-VQ KV-cache codec (libkvq.so).
 *
 * The method (VeloxQuant-MLX blog, "rvq" tag page, "The pipeline, as it actually runs"):
 * each head_dim vector of a [B, H, S, D] fp16 key or value tensor is normalised (its
 * norm kept), rotated by a sign-flipped, normalised Walsh-Hadamard transform, quantized
 * against a Gaussian Lloyd-Max codebook, its residual quantized against a Laplacian-fit
 * codebook, and the two b-bit index streams are bit-packed into uint32 words, each
 * stream separately. Decoding inverts every step except the quantization.
 *
 * Conventions shared by every entry point:
 *   - No exceptions cross this boundary and nothing aborts: every call returns a
 *     kvq_status. Argument checks run on the host before any HIP call, so a rejected
 *     call touches no device state.
 *   - The caller owns every buffer. The library allocates nothing, frees nothing and
 *     keeps no global state; `cb` is only read during the call.
 *   - Device calls enqueue on `stream` (a hipStream_t; NULL means the default stream)
 *     and return without synchronising. A fault inside a kernel surfaces at the
 *     caller's next synchronisation, not as a return code.
 *   - Calls that overlap on one stream are ordered; on different streams they may run
 *     concurrently and must not write the same words.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = -1,    /* a required pointer is NULL, or a codebook struct is inconsistent */
  KVQ_ERR_SHAPE = -2,  /* d outside [8, 1024] (or not a power of two where stated); bits not in 1..4; B, H, S < 0 */
  KVQ_ERR_ALIGN = -3,  /* an fp16 or packed-word buffer not 16-byte aligned, or a norm buffer not 4-byte aligned */
  KVQ_ERR_RANGE = -4,  /* s_offset < 0, s_offset + S > S_cap, a size overflows 64 bits, or a
                          launch would need more than 2^31 - 1 tiles (the kernels index tiles
                          with 32-bit integers; a tile is 2 to 64 vectors, by kernel and d) */
  KVQ_ERR_DEVICE = -5  /* the HIP launch reported an error */
} kvq_status;

#define KVQ_MIN_D 8
#define KVQ_MAX_D 1024
#define KVQ_MAX_BITS 4

/*
 * Codebooks and rotation signs for one (d, bits) pair. Plain data, 416 bytes; build it
 * with kvq_build_codebooks and treat it as read-only.
 *
 * The rotation length P is d rounded up to a power of two (P = d when d is one). The
 * Walsh-Hadamard transform exists at powers of two only, so a head dimension such as 96, 100
 * or 576 is rotated as the vector padded with P - d zeros, and all P rotated coordinates are
 * coded (the zeros add nothing to the norm, and the rotated vector keeps unit norm).
 *
 * c1/b1: stage-1 centroids (2^bits, ascending) and boundaries (2^bits - 1): the
 *        Lloyd-Max quantizer of N(0, sigma1^2), sigma1^2 = 1/P (the variance of one
 *        coordinate of a rotated unit vector).
 * c2/b2: stage-2 tables: the Lloyd-Max quantizer of a zero-mean Laplace density whose
 *        variance is the stage-1 distortion, sigma2^2 = mse_g * sigma1^2.
 *        Boundaries are the float32-rounded midpoints of neighbouring centroids (blog,
 *        "rvq" tag page, "What 'quantize' means here, precisely"); both tables are exactly
 *        antisymmetric, so the middle boundary is +0.0.
 * sign_bits: bit j (word j/32, bit j%32) set <=> the rotation multiplies coordinate j by -1
 *        (j < d; the padding coordinates take +1 and their bits are ignored).
 */
typedef struct kvq_codebooks {
  int32_t d;               /* head dimension */
  int32_t bits;            /* bits per code, per stage */
  int32_t elems_per_word;  /* floor(32 / bits) codes in each uint32 word */
  int32_t n_words;         /* ceil(P / elems_per_word) words per vector per stream */
  float c1[16];
  float b1[15];
  float c2[16];
  float b2[15];
  double sigma1;           /* 1/sqrt(P) */
  double sigma2;           /* sqrt(mse_g) * sigma1 */
  double mse_g;            /* distortion of the unit-variance Gaussian Lloyd-Max quantizer */
  uint32_t sign_bits[KVQ_MAX_D / 32];
} kvq_codebooks;

/*
 * kvq_build_codebooks - host only, no device calls.
 *   d     head dimension in [8, 1024]
 *   bits  bits per code per stage, 1..4
 *   signs host array of d entries, each +1 or -1 (the rotation's sign vector), or NULL
 *         for all +1
 *   out   host struct to fill
 * Lloyd-Max iteration in double precision for both densities (the pages: "rvq" tag page,
 * "The pipeline, as it actually runs" names a Gaussian and a Laplacian-fit codebook;
 * "turboquant" tag page, "Kernel 2" names Lloyd-Max; the "kivi" tag page's second post,
 * "Where KIVI fits", calls RVQ's codebooks analytical, needing no calibration).
 * Returns KVQ_ERR_ARG for a NULL out or a sign entry other than +-1, KVQ_ERR_SHAPE for
 * d or bits out of range.
 */
kvq_status kvq_build_codebooks(int32_t d, int32_t bits, const int8_t* signs, kvq_codebooks* out);

/*
 * kvq_rvq_encode_pack - device. Encodes N = B*H*S vectors in one kernel launch.
 *   cb        host pointer to codebooks from kvq_build_codebooks (read during the call)
 *   x         device fp16 [B, H, S, d], contiguous, 16-byte aligned (raw IEEE half bits)
 *   B, H, S   sizes (>= 0; any of them 0 means nothing to do)
 *   packed1   device uint32 [B, H, S_cap, n_words], 16-byte aligned: stage-1 codes
 *   packed2   device uint32 [B, H, S_cap, n_words], 16-byte aligned: stage-2 codes
 *   norms     device float32 [B, H, S_cap], 4-byte aligned: ||x|| of each vector
 *   S_cap     capacity of the cache's token axis (S_cap >= s_offset + S)
 *   s_offset  token s of x is written at cache position s_offset + s (appending one
 *             decode step at a time is S = 1, s_offset = step)
 *   stream    hipStream_t or NULL
 * Word layout (blog, "rvq" tag page, "The kernel"): code j of a vector (j < P) goes to word
 * j / elems_per_word at bits [(j % elems_per_word) * bits, ... + bits), LSB first; bits
 * past the last code are 0. Code value = the number of boundaries the value exceeds
 * ("What 'quantize' means here, precisely"), stage 1 on the rotated coordinate
 * y = (H diag(s) x)_j / (sqrt(P) ||x||) of x padded with zeros to length P, stage 2 on the
 * float32 residual y - c1[code1]. A zero vector stores norm 0 and the codes of y = 0.
 * Errors: KVQ_ERR_ARG, KVQ_ERR_SHAPE, KVQ_ERR_ALIGN, KVQ_ERR_RANGE (checked before any
 * HIP call), KVQ_ERR_DEVICE (launch error). The packed outputs and x must not overlap.
 */
kvq_status kvq_rvq_encode_pack(const kvq_codebooks* cb, const uint16_t* x,
                               int64_t B, int64_t H, int64_t S,
                               uint32_t* packed1, uint32_t* packed2, float* norms,
                               int64_t S_cap, int64_t s_offset, void* stream);

/*
 * kvq_rvq_unpack_decode - device. Decodes cache positions [s_offset, s_offset + S) of
 * every (b, h) in one launch.
 *   packed1/packed2  device uint32 [B, H, S_cap, n_words] (layout as above)
 *   norms            device float32 [B, H, S_cap], or NULL for unit-norm reconstructions
 *   x_out            device fp16 [B, H, S, d], contiguous, 16-byte aligned
 * Each coordinate is dequantized as c1[i1] + c2[i2] in the rotated domain (blog,
 * "turboquant" tag page, "Kernel 5"), rotated back by diag(s) H / sqrt(P) (H is
 * symmetric and H H = P I), scaled by the norm and rounded to fp16 (nearest-even); the
 * first d of the P coordinates are written.
 * Errors as for kvq_rvq_encode_pack.
 */
kvq_status kvq_rvq_unpack_decode(const kvq_codebooks* cb,
                                 const uint32_t* packed1, const uint32_t* packed2,
                                 const float* norms,
                                 int64_t B, int64_t H, int64_t S_cap, int64_t s_offset, int64_t S,
                                 uint16_t* x_out, void* stream);

/*
 * kvq_mse_encode_pack - device. The single-stage codec: the same normalisation, rotation
 * and stage-1 Gaussian Lloyd-Max quantization as kvq_rvq_encode_pack, without the residual
 * stage (blog, "turboquant" tag page, "Kernel 3": randomized Hadamard rotation followed by
 * the nearest-centroid quantize; counting boundary crossings gives the same index, "rvq"
 * tag page, "What 'quantize' means here, precisely"). Only cb's c1/b1 tables and signs
 * are used.
 *   packed    device uint32 [B, H, S_cap, n_words], 16-byte aligned: the codes, with the
 *             word layout of kvq_rvq_encode_pack's packed1 (and the same values)
 *   other arguments and errors as for kvq_rvq_encode_pack
 */
kvq_status kvq_mse_encode_pack(const kvq_codebooks* cb, const uint16_t* x,
                               int64_t B, int64_t H, int64_t S,
                               uint32_t* packed, float* norms,
                               int64_t S_cap, int64_t s_offset, void* stream);

/*
 * kvq_mse_unpack_decode - device. Inverse of kvq_mse_encode_pack: each coordinate is
 * dequantized as c1[i] (blog, "turboquant" tag page, "Kernel 2", dequantize: a gather of
 * the centroid), rotated back by diag(s) H / sqrt(P), scaled by the norm (or not, for
 * norms = NULL) and rounded to fp16 (nearest-even). Arguments and errors as for
 * kvq_rvq_unpack_decode with the single code stream `packed`.
 */
kvq_status kvq_mse_unpack_decode(const kvq_codebooks* cb, const uint32_t* packed, const float* norms,
                                 int64_t B, int64_t H, int64_t S_cap, int64_t s_offset, int64_t S,
                                 uint16_t* x_out, void* stream);

/*
 * kvq_rabitq_encode_pack - device. 1-bit sign codes of the rotated vector with its norm,
 * in one pass (blog, "rvq" tag page, "A fusion this codebase had already proven out": a
 * RaBitQ encoder that rotates, binarizes with y >= 0, packs the sign bits and writes the
 * magnitude). Bit j of a vector is [y_j >= 0] for y = H diag(s) x (the rotation of
 * kvq_rvq_encode_pack; the positive scale does not change a sign), so a zero vector gets
 * every bit set. Bits are packed LSB-first, 32 per word: bit j at word j / 32, bit j % 32;
 * bits past d are 0.
 *   cb        from kvq_build_codebooks(d, 1, signs): only d and the signs are used;
 *             bits != 1 or a d that is not a power of two is KVQ_ERR_SHAPE
 *   packed    device uint32 [B, H, S_cap, ceil(d / 32)], 16-byte aligned
 *   norms     device float32 [B, H, S_cap]: ||x|| (the magnitude)
 *   other arguments and errors as for kvq_rvq_encode_pack
 */
kvq_status kvq_rabitq_encode_pack(const kvq_codebooks* cb, const uint16_t* x,
                                  int64_t B, int64_t H, int64_t S,
                                  uint32_t* packed, float* norms,
                                  int64_t S_cap, int64_t s_offset, void* stream);

/*
 * kvq_qjl_supported - host. KVQ_OK when kvq_qjl_encode_pack takes head dimension d and
 * sketch size m: d in {32, 64, 128, 256}, m a multiple of 32 in [32, 256], and the sketch
 * (2 m d bytes) plus the kernel's key tiles fit the 160 KiB of LDS of one workgroup
 * (every such m at d <= 128, m <= 192 at d = 256). KVQ_ERR_SHAPE otherwise.
 */
kvq_status kvq_qjl_supported(int32_t d, int32_t m);

/*
 * kvq_qjl_encode_pack - device. The QJL key encoder (blog, "turboquant" tag page,
 * "Kernel 4: QJL Encode"): for every key x the m signs of S x, bit j = [(S x)_j >= 0],
 * packed LSB-first (bit j of the sequence at word j / 32, bit j % 32; the pages' byte k,
 * bit i is bit 8k + i, the same bytes on a little-endian machine), and the key norm
 * ||x|| rounded to fp16 (nearest-even). The dot products multiply the fp16 values exactly
 * and sum them in float32 (matrix cores), so a sign may differ from that of the exact dot
 * only when |exact| <= d * 2^-24 * sum_i |S_ji x_i|.
 *   sketch    device fp16 [m, d], row-major, 16-byte aligned, owned by the caller
 *   d, m      see kvq_qjl_supported
 *   x         device fp16 [B, H, S, d], contiguous, 16-byte aligned
 *   packed    device uint32 [B, H, S_cap, m / 32], 16-byte aligned
 *   norms     device fp16 [B, H, S_cap], 2-byte aligned
 *   S_cap, s_offset, stream as for kvq_rvq_encode_pack
 * Errors: KVQ_ERR_SHAPE (unsupported d or m, negative sizes), KVQ_ERR_ARG (null pointer),
 * KVQ_ERR_ALIGN, KVQ_ERR_RANGE (s_offset + S > S_cap, overflow), KVQ_ERR_DEVICE (launch
 * error); all but the last are checked before any HIP call. B * H * S == 0 returns KVQ_OK
 * without touching any pointer.
 */
kvq_status kvq_qjl_encode_pack(const uint16_t* sketch, int32_t d, int32_t m, const uint16_t* x,
                               int64_t B, int64_t H, int64_t S,
                               uint32_t* packed, uint16_t* norms,
                               int64_t S_cap, int64_t s_offset, void* stream);

/*
 * kvq_rvq_attend - device. Softmax attention of fp16 queries over a packed two-stage key
 * cache and value cache, without reconstructing either (blog, "turboquant" tag page,
 * "Kernel 5": keys decoded as c1[i1] + c2[i2] on the fly inside a FlashAttention-style
 * online softmax). For every query vector (b, h, s):
 *     out = sum_t p_t vhat_t,   p = softmax_t(scale * q . khat_t),   t in [0, S_kv)
 * where khat_t and vhat_t are the float32 reconstructions n_t diag(s) H z_t / sqrt(d) that
 * kvq_rvq_unpack_decode would round to fp16 (no rounding is applied to them here). Every
 * query attends to all S_kv cached positions (no mask). The work runs in the rotated
 * domain: q . khat_t = n_t (R q) . z_t, and the weighted sum of values is rotated back once.
 *   cbk, cbv     codebooks of the key and of the value cache (same d and bits, d a power
 *                of two; the sign vectors may differ)
 *   q            device fp16 [B, Hq, Sq, d], contiguous, 16-byte aligned
 *   Hkv          key/value heads; Hq must be a multiple of Hkv (query head h reads
 *                key/value head h / (Hq / Hkv))
 *   k_packed1/2, k_norms, v_packed1/2, v_norms
 *                caches written by kvq_rvq_encode_pack: [B, Hkv, S_cap, n_words] and
 *                [B, Hkv, S_cap]; positions [0, S_kv) are read
 *   S_cap, S_kv  cache capacity and valid length, 1 <= S_kv <= S_cap
 *   scale        softmax scale (finite; 1/sqrt(d) for standard attention)
 *   workspace    device scratch of at least kvq_rvq_attend_workspace_size bytes, 16-byte
 *                aligned, owned by the caller; its contents are overwritten
 *   out          device fp16 [B, Hq, Sq, d], contiguous, 16-byte aligned
 * Errors: KVQ_ERR_ARG (null pointer, non-finite scale, inconsistent codebooks),
 * KVQ_ERR_SHAPE (codebooks of different d or bits, d not a power of two, negative sizes, Hq not a multiple of
 * Hkv), KVQ_ERR_ALIGN, KVQ_ERR_RANGE (S_kv out of range, workspace too small, overflow),
 * KVQ_ERR_DEVICE. B * Hq * Sq == 0 returns KVQ_OK without touching any pointer.
 */
kvq_status kvq_rvq_attend(const kvq_codebooks* cbk, const kvq_codebooks* cbv, const uint16_t* q,
                          int64_t B, int64_t Hq, int64_t Sq, int64_t Hkv,
                          const uint32_t* k_packed1, const uint32_t* k_packed2, const float* k_norms,
                          const uint32_t* v_packed1, const uint32_t* v_packed2, const float* v_norms,
                          int64_t S_cap, int64_t S_kv, float scale,
                          void* workspace, int64_t workspace_bytes, uint16_t* out, void* stream);

/*
 * kvq_rvq_attend_workspace_size - host. Workspace bytes kvq_rvq_attend needs for these
 * sizes (d and bits as in the codebooks; B, Hq, Sq, Hkv, S_kv as passed to kvq_rvq_attend).
 * Errors: KVQ_ERR_ARG (bytes NULL), KVQ_ERR_SHAPE (d not a power of two in range, bits out
 * of range, negative sizes, Hq not a multiple of Hkv), KVQ_ERR_RANGE (S_kv < 1 or overflow).
 */
kvq_status kvq_rvq_attend_workspace_size(int32_t d, int32_t bits, int64_t B, int64_t Hq, int64_t Sq, int64_t Hkv,
                                         int64_t S_kv, int64_t* bytes);

/*
 * kvq_rvq_attend_noalloc - device. kvq_rvq_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same checks, kernels and result, with the partial results in a device
 * scratch array the library holds instead of a caller's workspace. Arguments as for
 * kvq_rvq_attend, without workspace and workspace_bytes.
 *   Scratch: KVQ_ATTEND_SCRATCH_BYTES (32 MiB) per device, part of the library's code object
 *   (each device the library runs on holds one copy until the process ends). Its address is
 *   looked up at the first call on each device. Nothing in it needs clearing between calls.
 *   Every call on one device uses that device's copy: calls that overlap on one device (on
 *   different streams, or from several threads) race and must be ordered by the caller.
 * Errors: as kvq_rvq_attend, and KVQ_ERR_RANGE when these sizes need more than
 * KVQ_ATTEND_SCRATCH_BYTES (kvq_rvq_attend_workspace_size tells how much), checked on the
 * host before any HIP call. Nothing is allocated or freed.
 */
#define KVQ_ATTEND_SCRATCH_BYTES (32ll << 20)
kvq_status kvq_rvq_attend_noalloc(const kvq_codebooks* cbk, const kvq_codebooks* cbv, const uint16_t* q,
                                  int64_t B, int64_t Hq, int64_t Sq, int64_t Hkv,
                                  const uint32_t* k_packed1, const uint32_t* k_packed2, const float* k_norms,
                                  const uint32_t* v_packed1, const uint32_t* v_packed2, const float* v_norms,
                                  int64_t S_cap, int64_t S_kv, float scale, uint16_t* out, void* stream);

/* Static text for a status code; never NULL. */
const char* kvq_status_str(kvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
