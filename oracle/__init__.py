"""Checker for the two-stage residual-VQ KV-cache codec: a plain, slow CPU oracle.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
anything in this package: only the tests, the smoke check of the package entry point
and the CPU-baseline leg of the benchmark use it. The oracle shares no code with the
HIP library: it has its own codebook builder, its own Hadamard matrix, its own
quantizer (argmin over centroids rather than a boundary count) and its own packing.

Sources it follows (the VeloxQuant-MLX blog pages):
  * "rvq" tag page, sections "The pipeline, as it actually runs" (rotate, stage-1
    Gaussian codebook, residual, stage-2 Laplacian-fit codebook, two packed streams),
    "What 'quantize' means here, precisely" (boundaries are midpoints of sorted
    centroids; counting crossings gives the nearest centroid) and "The kernel"
    (float32 residual, LSB-first packing of b-bit codes into uint32 words).
  * "turboquant" tag page, "Kernel 2" (nearest-centroid argmin, first minimum wins),
    "Kernel 3" (randomized Hadamard rotation y = H diag(s) x / sqrt(D), sign flip applied
    before the butterfly) and "Kernel 5" (dequantized key = c1[i1] + c2[i2]).

Modules:
  codebooks  Lloyd-Max scalar quantizers for N(0, 1/D) and for a Laplace density whose
             variance is the stage-1 distortion; float32 tables.
  rvq        encode (normalize, rotate, quantize twice, pack) and decode.
  packing    LSB-first b-bit packing into uint32 words and its inverse.
  flips      the comparison rule between a device result and the oracle.
  attend     softmax attention over packed key/value caches (the plain definition).
"""
