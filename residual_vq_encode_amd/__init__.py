"""Python binding of libkvq, the MI355X two-stage residual-VQ KV-cache codec.

Argument marshalling only: every step of the encode and decode runs in the HIP kernels
of libkvq.so (built in place by ``python -m residual_vq_encode_amd.build``). PyTorch is
used for device memory and streams; tensors are passed to the C ABI as raw pointers on
the current torch stream. There is no fallback path: if the library is missing or the
tensors are not on a GPU, the calls raise.

    cb = build_codebooks(d=128, bits=2, signs=s)           # host, once
    p1, p2, norms = encode(x, cb)                          # x: fp16 [B, H, S, D] on cuda
    x_hat = decode(p1, p2, norms, cb)                      # fp16 [B, H, S, D]

The lower-level calls kvq_rvq_encode_pack / kvq_rvq_unpack_decode mirror the C ABI
(including S_cap / s_offset for writing into and reading from a preallocated cache);
kvq_mse_encode_pack / kvq_mse_unpack_decode (and encode_mse / decode_mse) are the
single-stage codec: stage 1 only, one code stream. kvq_rabitq_encode_pack (encode_rabitq)
writes 1-bit sign codes of the rotated vector with its norm; kvq_qjl_encode_pack
(encode_qjl) writes the 1-bit sign sketch of S x for a caller's fp16 sketch matrix S with
fp16 norms; kvq_rvq_attend (attend) is softmax attention over packed key/value caches.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "KvqError", "Codebooks", "load", "library_path", "build_codebooks", "kvq_build_codebooks",
    "kvq_rvq_encode_pack", "kvq_rvq_unpack_decode", "kvq_mse_encode_pack", "kvq_mse_unpack_decode",
    "kvq_rvq_attend", "kvq_rvq_attend_workspace_size", "kvq_rvq_attend_noalloc", "ATTEND_SCRATCH_BYTES", "kvq_rabitq_encode_pack", "kvq_qjl_encode_pack",
    "kvq_qjl_supported", "kvq_status_str", "encode", "decode", "encode_mse", "decode_mse", "encode_rabitq",
    "encode_qjl", "attend", "n_words", "PreparedLaunch", "prepare_encode", "prepare_decode",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libkvq.so"

STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_ARG", -2: "KVQ_ERR_SHAPE", -3: "KVQ_ERR_ALIGN",
          -4: "KVQ_ERR_RANGE", -5: "KVQ_ERR_DEVICE"}


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({kvq_status_str(status)})")


class Codebooks(ctypes.Structure):
    """Mirror of kvq_codebooks (include/kvq.h)."""
    _fields_ = [
        ("d", ctypes.c_int32), ("bits", ctypes.c_int32),
        ("elems_per_word", ctypes.c_int32), ("n_words", ctypes.c_int32),
        ("c1", ctypes.c_float * 16), ("b1", ctypes.c_float * 15),
        ("c2", ctypes.c_float * 16), ("b2", ctypes.c_float * 15),
        ("sigma1", ctypes.c_double), ("sigma2", ctypes.c_double), ("mse_g", ctypes.c_double),
        ("sign_bits", ctypes.c_uint32 * 32),
    ]

    @property
    def levels(self) -> int:
        return 1 << self.bits

    def tables(self):
        """(c1, b1, c2, b2) as Python lists of the used entries."""
        k = self.levels
        return list(self.c1[:k]), list(self.b1[:k - 1]), list(self.c2[:k]), list(self.b2[:k - 1])

    def signs(self) -> list[int]:
        return [-1 if (self.sign_bits[j >> 5] >> (j & 31)) & 1 else 1 for j in range(self.d)]


assert ctypes.sizeof(Codebooks) == 416

_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load() -> ctypes.CDLL:
    """Load libkvq.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m residual_vq_encode_amd.build`")
    lib = ctypes.CDLL(path)
    i64, ptr = ctypes.c_int64, ctypes.c_void_p
    lib.kvq_build_codebooks.argtypes = [ctypes.c_int32, ctypes.c_int32, ptr, ctypes.POINTER(Codebooks)]
    lib.kvq_build_codebooks.restype = ctypes.c_int
    lib.kvq_rvq_encode_pack.argtypes = [ctypes.POINTER(Codebooks), ptr, i64, i64, i64, ptr, ptr, ptr, i64, i64, ptr]
    lib.kvq_rvq_encode_pack.restype = ctypes.c_int
    lib.kvq_rvq_unpack_decode.argtypes = [ctypes.POINTER(Codebooks), ptr, ptr, ptr, i64, i64, i64, i64, i64, ptr, ptr]
    lib.kvq_rvq_unpack_decode.restype = ctypes.c_int
    lib.kvq_mse_encode_pack.argtypes = [ctypes.POINTER(Codebooks), ptr, i64, i64, i64, ptr, ptr, i64, i64, ptr]
    lib.kvq_mse_encode_pack.restype = ctypes.c_int
    lib.kvq_mse_unpack_decode.argtypes = [ctypes.POINTER(Codebooks), ptr, ptr, i64, i64, i64, i64, i64, ptr, ptr]
    lib.kvq_mse_unpack_decode.restype = ctypes.c_int
    lib.kvq_rvq_attend.argtypes = [ctypes.POINTER(Codebooks), ctypes.POINTER(Codebooks), ptr, i64, i64, i64, i64,
                                   ptr, ptr, ptr, ptr, ptr, ptr, i64, i64, ctypes.c_float, ptr, i64, ptr, ptr]
    lib.kvq_rvq_attend.restype = ctypes.c_int
    lib.kvq_rvq_attend_noalloc.argtypes = [ctypes.POINTER(Codebooks), ctypes.POINTER(Codebooks), ptr, i64, i64, i64,
                                           i64, ptr, ptr, ptr, ptr, ptr, ptr, i64, i64, ctypes.c_float, ptr, ptr]
    lib.kvq_rvq_attend_noalloc.restype = ctypes.c_int
    lib.kvq_rvq_attend_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, i64, i64, i64, i64, i64,
                                                   ctypes.POINTER(ctypes.c_int64)]
    lib.kvq_rvq_attend_workspace_size.restype = ctypes.c_int
    lib.kvq_status_str.argtypes = [ctypes.c_int]
    lib.kvq_rabitq_encode_pack.argtypes = [ctypes.POINTER(Codebooks), ptr, i64, i64, i64, ptr, ptr, i64, i64, ptr]
    lib.kvq_rabitq_encode_pack.restype = ctypes.c_int
    lib.kvq_qjl_supported.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.kvq_qjl_supported.restype = ctypes.c_int
    lib.kvq_qjl_encode_pack.argtypes = [ptr, ctypes.c_int32, ctypes.c_int32, ptr, i64, i64, i64, ptr, ptr, i64, i64,
                                        ptr]
    lib.kvq_qjl_encode_pack.restype = ctypes.c_int
    lib.kvq_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def kvq_status_str(status: int) -> str:
    return load().kvq_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise KvqError(status, what)


def rotation_length(d: int) -> int:
    """The power of two (at least 8) that head dimension d is rotated at: a d that is not a
    power of two is zero-padded to it, and all of its rotated coordinates are coded."""
    p = 8
    while p < d:
        p *= 2
    return p


def n_words(d: int, bits: int) -> int:
    """Packed words per vector per stream for head dimension d."""
    epw = 32 // bits
    return (rotation_length(d) + epw - 1) // epw


def kvq_build_codebooks(d: int, bits: int, signs=None) -> Codebooks:
    """Host call. signs: None (all +1) or a sequence/array/tensor of d values in {+1, -1}."""
    cb = Codebooks()
    buf = None
    if signs is not None:
        vals = [int(v) for v in (signs.tolist() if hasattr(signs, "tolist") else signs)]
        if len(vals) != d:
            raise ValueError(f"signs must have {d} entries")
        buf = (ctypes.c_int8 * d)(*vals)
    _check(load().kvq_build_codebooks(int(d), int(bits), buf, ctypes.byref(cb)), "kvq_build_codebooks")
    return cb


build_codebooks = kvq_build_codebooks


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _require_cuda(*tensors) -> None:
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("kvq kernels need GPU tensors (no CPU path exists)")


def kvq_rvq_encode_pack(cb: Codebooks, x, packed1, packed2, norms, s_offset: int = 0, stream=None) -> None:
    """x: fp16 [B, H, S, d] contiguous; packed1/packed2: int32/uint32 [B, H, S_cap, n_words];
    norms: float32 [B, H, S_cap]. Writes token s of x at cache position s_offset + s."""
    import torch
    _require_cuda(x, packed1, packed2, norms)
    if x.dtype != torch.float16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp16 [B, H, S, d] tensor")
    B, H, S, d = x.shape
    if d != cb.d:
        raise ValueError(f"x has d={d}, codebooks have d={cb.d}")
    S_cap = packed1.shape[2]
    for name, t, shape in (("packed1", packed1, (B, H, S_cap, cb.n_words)),
                           ("packed2", packed2, (B, H, S_cap, cb.n_words)),
                           ("norms", norms, (B, H, S_cap))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with shape {shape}, got {tuple(t.shape)}")
    if packed1.element_size() != 4 or packed2.element_size() != 4 or norms.dtype != torch.float32:
        raise ValueError("packed streams must be 32-bit integers and norms float32")
    _check(load().kvq_rvq_encode_pack(ctypes.byref(cb), _ptr(x), B, H, S, _ptr(packed1), _ptr(packed2),
                                      _ptr(norms), S_cap, int(s_offset), _stream_handle(stream)),
           "kvq_rvq_encode_pack")


class PreparedLaunch:
    """One C ABI call with its arguments validated and marshalled once (prepare_encode,
    prepare_decode): calling it only makes the C call and checks the status, so a loop of
    launches is not held up by Python-side checks. The tensors it was prepared with must stay
    alive and keep their storage."""
    __slots__ = ("_fn", "_args", "_what", "_keep")

    def __init__(self, fn, args, what, keep):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != 0:
            raise KvqError(status, self._what)


def prepare_encode(cb: Codebooks, x, packed1, packed2, norms, s_offset: int = 0, stream=None,
                   stages: int = 2) -> PreparedLaunch:
    """kvq_rvq_encode_pack (stages=2) or kvq_mse_encode_pack (stages=1, packed2 ignored) on
    these tensors, validated as by those calls, as a PreparedLaunch."""
    import torch
    _require_cuda(x, packed1, packed2 if stages == 2 else None, norms)
    if x.dtype != torch.float16 or x.dim() != 4 or not x.is_contiguous() or x.shape[3] != cb.d:
        raise ValueError("x must be a contiguous fp16 [B, H, S, d] tensor matching the codebooks")
    B, H, S, _ = x.shape
    S_cap = packed1.shape[2]
    for name, t in (("packed1", packed1),) + ((("packed2", packed2),) if stages == 2 else ()):
        _check_stream(cb, name, t, B, H, S_cap)
    if tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float32 or not norms.is_contiguous():
        raise ValueError(f"norms must be contiguous float32 {(B, H, S_cap)}")
    cbp = ctypes.pointer(cb)
    lib = load()
    if stages == 2:
        args = (cbp, _ptr(x), B, H, S, _ptr(packed1), _ptr(packed2), _ptr(norms), S_cap, int(s_offset),
                _stream_handle(stream))
        return PreparedLaunch(lib.kvq_rvq_encode_pack, args, "kvq_rvq_encode_pack", (cb, x, packed1, packed2, norms))
    args = (cbp, _ptr(x), B, H, S, _ptr(packed1), _ptr(norms), S_cap, int(s_offset), _stream_handle(stream))
    return PreparedLaunch(lib.kvq_mse_encode_pack, args, "kvq_mse_encode_pack", (cb, x, packed1, norms))


def prepare_decode(cb: Codebooks, packed1, packed2, norms, out, s_offset: int = 0, stream=None,
                   stages: int = 2) -> PreparedLaunch:
    """kvq_rvq_unpack_decode (stages=2) or kvq_mse_unpack_decode (stages=1, packed2 ignored)
    into out, validated as by those calls, as a PreparedLaunch."""
    import torch
    _require_cuda(packed1, packed2 if stages == 2 else None, norms, out)
    if out.dtype != torch.float16 or out.dim() != 4 or not out.is_contiguous() or out.shape[3] != cb.d:
        raise ValueError("out must be a contiguous fp16 [B, H, S, d] tensor")
    B, H, S, _ = out.shape
    S_cap = packed1.shape[2]
    for name, t in (("packed1", packed1),) + ((("packed2", packed2),) if stages == 2 else ()):
        _check_stream(cb, name, t, B, H, S_cap)
    if norms is not None and (tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float32
                              or not norms.is_contiguous()):
        raise ValueError(f"norms must be contiguous float32 {(B, H, S_cap)}")
    cbp = ctypes.pointer(cb)
    lib = load()
    if stages == 2:
        args = (cbp, _ptr(packed1), _ptr(packed2), _ptr(norms), B, H, S_cap, int(s_offset), S, _ptr(out),
                _stream_handle(stream))
        return PreparedLaunch(lib.kvq_rvq_unpack_decode, args, "kvq_rvq_unpack_decode", (cb, packed1, packed2, norms, out))
    args = (cbp, _ptr(packed1), _ptr(norms), B, H, S_cap, int(s_offset), S, _ptr(out), _stream_handle(stream))
    return PreparedLaunch(lib.kvq_mse_unpack_decode, args, "kvq_mse_unpack_decode", (cb, packed1, norms, out))


def kvq_rvq_unpack_decode(cb: Codebooks, packed1, packed2, norms, out, s_offset: int = 0, stream=None) -> None:
    """Decodes cache positions [s_offset, s_offset + S) into out: fp16 [B, H, S, d].
    norms=None gives unit reconstructions."""
    import torch
    _require_cuda(packed1, packed2, norms, out)
    if out.dtype != torch.float16 or out.dim() != 4 or not out.is_contiguous() or out.shape[3] != cb.d:
        raise ValueError("out must be a contiguous fp16 [B, H, S, d] tensor")
    B, H, S, _ = out.shape
    S_cap = packed1.shape[2]
    for name, t, shape in (("packed1", packed1, (B, H, S_cap, cb.n_words)),
                           ("packed2", packed2, (B, H, S_cap, cb.n_words))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with shape {shape}, got {tuple(t.shape)}")
    if norms is not None and (tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float32
                              or not norms.is_contiguous()):
        raise ValueError(f"norms must be contiguous float32 {(B, H, S_cap)}")
    _check(load().kvq_rvq_unpack_decode(ctypes.byref(cb), _ptr(packed1), _ptr(packed2), _ptr(norms),
                                        B, H, S_cap, int(s_offset), S, _ptr(out), _stream_handle(stream)),
           "kvq_rvq_unpack_decode")


def encode(x, cb: Codebooks, stream=None):
    """Allocate outputs and encode x (fp16 [B, H, S, d] on cuda). Returns (packed1, packed2, norms)."""
    import torch
    B, H, S, d = x.shape
    p1 = torch.empty((B, H, S, cb.n_words), dtype=torch.int32, device=x.device)
    p2 = torch.empty_like(p1)
    norms = torch.empty((B, H, S), dtype=torch.float32, device=x.device)
    kvq_rvq_encode_pack(cb, x, p1, p2, norms, 0, stream)
    return p1, p2, norms


def decode(packed1, packed2, norms, cb: Codebooks, stream=None):
    """Allocate the output and decode every cache position. Returns fp16 [B, H, S, d]."""
    import torch
    B, H, S, _ = packed1.shape
    out = torch.empty((B, H, S, cb.d), dtype=torch.float16, device=packed1.device)
    kvq_rvq_unpack_decode(cb, packed1, packed2, norms, out, 0, stream)
    return out


def _check_stream(cb: Codebooks, name: str, t, B: int, H: int, S_cap: int) -> None:
    shape = (B, H, S_cap, cb.n_words)
    if tuple(t.shape) != shape or not t.is_contiguous() or t.element_size() != 4:
        raise ValueError(f"{name} must be a contiguous 32-bit integer tensor of shape {shape}, got {tuple(t.shape)}")


def kvq_mse_encode_pack(cb: Codebooks, x, packed, norms, s_offset: int = 0, stream=None) -> None:
    """Single-stage encode. x: fp16 [B, H, S, d] contiguous; packed: int32/uint32
    [B, H, S_cap, n_words]; norms: float32 [B, H, S_cap]."""
    import torch
    _require_cuda(x, packed, norms)
    if x.dtype != torch.float16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp16 [B, H, S, d] tensor")
    B, H, S, d = x.shape
    if d != cb.d:
        raise ValueError(f"x has d={d}, codebooks have d={cb.d}")
    S_cap = packed.shape[2]
    _check_stream(cb, "packed", packed, B, H, S_cap)
    if tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float32 or not norms.is_contiguous():
        raise ValueError(f"norms must be contiguous float32 {(B, H, S_cap)}")
    _check(load().kvq_mse_encode_pack(ctypes.byref(cb), _ptr(x), B, H, S, _ptr(packed), _ptr(norms), S_cap,
                                      int(s_offset), _stream_handle(stream)), "kvq_mse_encode_pack")


def kvq_mse_unpack_decode(cb: Codebooks, packed, norms, out, s_offset: int = 0, stream=None) -> None:
    """Single-stage decode of cache positions [s_offset, s_offset + S) into out: fp16
    [B, H, S, d]; norms=None gives unit reconstructions."""
    import torch
    _require_cuda(packed, norms, out)
    if out.dtype != torch.float16 or out.dim() != 4 or not out.is_contiguous() or out.shape[3] != cb.d:
        raise ValueError("out must be a contiguous fp16 [B, H, S, d] tensor")
    B, H, S, _ = out.shape
    S_cap = packed.shape[2]
    _check_stream(cb, "packed", packed, B, H, S_cap)
    if norms is not None and (tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float32
                              or not norms.is_contiguous()):
        raise ValueError(f"norms must be contiguous float32 {(B, H, S_cap)}")
    _check(load().kvq_mse_unpack_decode(ctypes.byref(cb), _ptr(packed), _ptr(norms), B, H, S_cap, int(s_offset), S,
                                        _ptr(out), _stream_handle(stream)), "kvq_mse_unpack_decode")


def encode_mse(x, cb: Codebooks, stream=None):
    """Allocate outputs and run the single-stage encode. Returns (packed, norms)."""
    import torch
    B, H, S, d = x.shape
    p = torch.empty((B, H, S, cb.n_words), dtype=torch.int32, device=x.device)
    norms = torch.empty((B, H, S), dtype=torch.float32, device=x.device)
    kvq_mse_encode_pack(cb, x, p, norms, 0, stream)
    return p, norms


def decode_mse(packed, norms, cb: Codebooks, stream=None):
    """Allocate the output and run the single-stage decode. Returns fp16 [B, H, S, d]."""
    import torch
    B, H, S, _ = packed.shape
    out = torch.empty((B, H, S, cb.d), dtype=torch.float16, device=packed.device)
    kvq_mse_unpack_decode(cb, packed, norms, out, 0, stream)
    return out


def kvq_rvq_attend_workspace_size(d: int, bits: int, B: int, Hq: int, Sq: int, Hkv: int, S_kv: int) -> int:
    """Workspace bytes kvq_rvq_attend needs (host call)."""
    out = ctypes.c_int64(0)
    _check(load().kvq_rvq_attend_workspace_size(int(d), int(bits), int(B), int(Hq), int(Sq), int(Hkv), int(S_kv),
                                                ctypes.byref(out)),
           "kvq_rvq_attend_workspace_size")
    return out.value


def kvq_rvq_attend(cbk: Codebooks, cbv: Codebooks, q, kcache, vcache, S_kv: int, scale: float, workspace, out,
                   stream=None) -> None:
    """Attention of q (fp16 [B, Hq, Sq, d]) over cached positions [0, S_kv) of packed caches
    kcache = (packed1, packed2, norms) and vcache (the same), each [B, Hkv, S_cap, n_words] /
    [B, Hkv, S_cap]. workspace: a device tensor of at least kvq_rvq_attend_workspace_size
    bytes; out: fp16 [B, Hq, Sq, d]."""
    import torch
    k1, k2, kn = kcache
    v1, v2, vn = vcache
    _require_cuda(q, k1, k2, kn, v1, v2, vn, workspace, out)
    if q.dtype != torch.float16 or q.dim() != 4 or not q.is_contiguous() or q.shape[3] != cbk.d:
        raise ValueError("q must be a contiguous fp16 [B, Hq, Sq, d] tensor")
    if out.dtype != torch.float16 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 tensor shaped like q")
    B, Hq, Sq, _ = q.shape
    Hkv, S_cap = k1.shape[1], k1.shape[2]
    for name, t in (("k_packed1", k1), ("k_packed2", k2), ("v_packed1", v1), ("v_packed2", v2)):
        _check_stream(cbk, name, t, B, Hkv, S_cap)
    for name, t in (("k_norms", kn), ("v_norms", vn)):
        if tuple(t.shape) != (B, Hkv, S_cap) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32 {(B, Hkv, S_cap)}")
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().kvq_rvq_attend(ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q), B, Hq, Sq, Hkv, _ptr(k1), _ptr(k2),
                                 _ptr(kn), _ptr(v1), _ptr(v2), _ptr(vn), S_cap, int(S_kv), float(scale),
                                 _ptr(workspace), nbytes, _ptr(out), _stream_handle(stream)), "kvq_rvq_attend")


# Device scratch behind kvq_rvq_attend_noalloc (KVQ_ATTEND_SCRATCH_BYTES in include/kvq.h).
ATTEND_SCRATCH_BYTES = 32 << 20


def kvq_rvq_attend_noalloc(cbk: Codebooks, cbv: Codebooks, q, kcache, vcache, S_kv: int, scale: float, out,
                           stream=None) -> None:
    """kvq_rvq_attend without a workspace: the partial results go to the library's per-device
    scratch (at most ATTEND_SCRATCH_BYTES; larger plans raise KVQ_ERR_RANGE). Nothing is
    allocated; calls that overlap on one device share the scratch and race."""
    import torch
    k1, k2, kn = kcache
    v1, v2, vn = vcache
    _require_cuda(q, k1, k2, kn, v1, v2, vn, out)
    if q.dtype != torch.float16 or q.dim() != 4 or not q.is_contiguous() or q.shape[3] != cbk.d:
        raise ValueError("q must be a contiguous fp16 [B, Hq, Sq, d] tensor")
    if out.dtype != torch.float16 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp16 tensor shaped like q")
    B, Hq, Sq, _ = q.shape
    Hkv, S_cap = k1.shape[1], k1.shape[2]
    for name, t in (("k_packed1", k1), ("k_packed2", k2), ("v_packed1", v1), ("v_packed2", v2)):
        _check_stream(cbk, name, t, B, Hkv, S_cap)
    for name, t in (("k_norms", kn), ("v_norms", vn)):
        if tuple(t.shape) != (B, Hkv, S_cap) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32 {(B, Hkv, S_cap)}")
    _check(load().kvq_rvq_attend_noalloc(ctypes.byref(cbk), ctypes.byref(cbv), _ptr(q), B, Hq, Sq, Hkv, _ptr(k1),
                                         _ptr(k2), _ptr(kn), _ptr(v1), _ptr(v2), _ptr(vn), S_cap, int(S_kv),
                                         float(scale), _ptr(out), _stream_handle(stream)), "kvq_rvq_attend_noalloc")


def attend(q, kcache, vcache, cbk: Codebooks, cbv: Codebooks, S_kv: int, scale=None, stream=None):
    """Allocate the workspace and output and run kvq_rvq_attend. scale defaults to 1/sqrt(d)."""
    import math
    import torch
    B, Hq, Sq, d = q.shape
    Hkv = kcache[0].shape[1]
    ws = torch.empty(max(16, kvq_rvq_attend_workspace_size(d, cbk.bits, B, Hq, Sq, Hkv, S_kv)) // 4,
                     dtype=torch.float32,
                     device=q.device)
    out = torch.empty_like(q)
    kvq_rvq_attend(cbk, cbv, q, kcache, vcache, S_kv, 1.0 / math.sqrt(d) if scale is None else scale, ws, out, stream)
    return out


def kvq_rabitq_encode_pack(cb: Codebooks, x, packed, norms, s_offset: int = 0, stream=None) -> None:
    """1-bit sign codes [y >= 0] of the rotated vector. cb: built with bits = 1 (only d and the
    signs are used); x: fp16 [B, H, S, d] contiguous; packed: int32/uint32
    [B, H, S_cap, ceil(d / 32)]; norms: float32 [B, H, S_cap]."""
    import torch
    _require_cuda(x, packed, norms)
    if cb.bits != 1:
        raise ValueError("the sign code takes codebooks built with bits = 1")
    if x.dtype != torch.float16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp16 [B, H, S, d] tensor")
    B, H, S, d = x.shape
    if d != cb.d:
        raise ValueError(f"x has d={d}, codebooks have d={cb.d}")
    S_cap = packed.shape[2]
    _check_stream(cb, "packed", packed, B, H, S_cap)
    if tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float32 or not norms.is_contiguous():
        raise ValueError(f"norms must be contiguous float32 {(B, H, S_cap)}")
    _check(load().kvq_rabitq_encode_pack(ctypes.byref(cb), _ptr(x), B, H, S, _ptr(packed), _ptr(norms), S_cap,
                                         int(s_offset), _stream_handle(stream)), "kvq_rabitq_encode_pack")


def encode_rabitq(x, cb: Codebooks, stream=None):
    """Allocate outputs and write the 1-bit sign codes. Returns (packed, norms)."""
    import torch
    B, H, S, d = x.shape
    p = torch.empty((B, H, S, cb.n_words), dtype=torch.int32, device=x.device)
    norms = torch.empty((B, H, S), dtype=torch.float32, device=x.device)
    kvq_rabitq_encode_pack(cb, x, p, norms, 0, stream)
    return p, norms


def kvq_qjl_supported(d: int, m: int) -> bool:
    """Whether the sign-sketch encoder takes head dimension d and sketch size m (host call)."""
    return load().kvq_qjl_supported(int(d), int(m)) == 0


def kvq_qjl_encode_pack(sketch, x, packed, norms, s_offset: int = 0, stream=None) -> None:
    """1-bit sign sketch. sketch: fp16 [m, d] contiguous; x: fp16 [B, H, S, d] contiguous;
    packed: int32/uint32 [B, H, S_cap, m / 32] (bit j of the sequence = [(S x)_j >= 0]);
    norms: fp16 [B, H, S_cap]. Writes token s at cache position s_offset + s."""
    import torch
    _require_cuda(sketch, x, packed, norms)
    if sketch.dtype != torch.float16 or sketch.dim() != 2 or not sketch.is_contiguous():
        raise ValueError("sketch must be a contiguous fp16 [m, d] tensor")
    if x.dtype != torch.float16 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp16 [B, H, S, d] tensor")
    m, d = sketch.shape
    B, H, S, dx = x.shape
    if dx != d:
        raise ValueError(f"x has d={dx}, the sketch has d={d}")
    S_cap = packed.shape[2]
    if tuple(packed.shape) != (B, H, S_cap, m // 32) or not packed.is_contiguous() or packed.element_size() != 4:
        raise ValueError(f"packed must be a contiguous 32-bit integer tensor of shape {(B, H, S_cap, m // 32)}")
    if tuple(norms.shape) != (B, H, S_cap) or norms.dtype != torch.float16 or not norms.is_contiguous():
        raise ValueError(f"norms must be contiguous float16 {(B, H, S_cap)}")
    _check(load().kvq_qjl_encode_pack(_ptr(sketch), int(d), int(m), _ptr(x), B, H, S, _ptr(packed), _ptr(norms),
                                      S_cap, int(s_offset), _stream_handle(stream)), "kvq_qjl_encode_pack")


def encode_qjl(x, sketch, stream=None):
    """Allocate outputs and write the sign sketch. Returns (packed, norms)."""
    import torch
    B, H, S, d = x.shape
    m = sketch.shape[0]
    p = torch.empty((B, H, S, m // 32), dtype=torch.int32, device=x.device)
    norms = torch.empty((B, H, S), dtype=torch.float16, device=x.device)
    kvq_qjl_encode_pack(sketch, x, p, norms, 0, stream)
    return p, norms
