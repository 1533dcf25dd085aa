"""The C ABI library on the host: exports, struct layout, codebooks, argument checks.

Nothing here launches a kernel: every call either is host-only (kvq_build_codebooks,
kvq_status_str) or is rejected by the host-side argument checks before any HIP call.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import residual_vq_encode_amd as kvq
from oracle import codebooks as ocb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvq_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = kvq.load()
    names = _declared_functions()
    assert names == ["kvq_build_codebooks", "kvq_mse_encode_pack", "kvq_mse_unpack_decode", "kvq_qjl_encode_pack",
                     "kvq_qjl_supported", "kvq_rabitq_encode_pack", "kvq_rvq_attend", "kvq_rvq_attend_noalloc",
                     "kvq_rvq_attend_workspace_size",
                     "kvq_rvq_encode_pack", "kvq_rvq_unpack_decode", "kvq_status_str"]
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(kvq_\w+)", out))
    assert set(names) <= exported


def test_struct_layout_matches_header():
    """Compile the header with gcc and compare sizeof/offsetof with the ctypes mirror."""
    fields = [f for f, _ in kvq.Codebooks._fields_]
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"kvq.h\"\nint main(void){printf(\"%zu\", sizeof(kvq_codebooks));"
    for f in fields:
        src += f'printf(" %zu", offsetof(kvq_codebooks, {f}));'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "probe.c")
        exe = os.path.join(td, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(kvq.Codebooks) == 416
    assert vals[1:] == [getattr(kvq.Codebooks, f).offset for f in fields]


@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebooks_match_oracle_bit_exactly(d, bits):
    """The library's C++ Lloyd-Max builder and the oracle's numpy one are independent
    implementations of the same fixed point; the float32 tables must agree exactly."""
    rng = np.random.default_rng(d * 10 + bits)
    signs = np.where(rng.integers(0, 2, d) == 1, -1, 1)
    cb = kvq.build_codebooks(d, bits, signs)
    t = ocb.build_tables(d, bits)
    c1, b1, c2, b2 = (np.array(v, np.float32) for v in cb.tables())
    assert c1.tobytes() == t.c1.tobytes() and b1.tobytes() == t.b1.tobytes()
    assert c2.tobytes() == t.c2.tobytes() and b2.tobytes() == t.b2.tobytes()
    assert cb.d == d and cb.bits == bits and cb.elems_per_word == 32 // bits
    assert cb.n_words == -(-d // (32 // bits))
    assert cb.signs() == signs.tolist()
    assert abs(cb.sigma1 - t.sigma1) < 1e-15 and abs(cb.sigma2 / t.sigma2 - 1) < 1e-12


def test_build_codebooks_rejects():
    lib = kvq.load()
    cb = kvq.Codebooks()
    for d in (0, 4, 7, 1025, 2048, -8):
        assert lib.kvq_build_codebooks(d, 2, None, ctypes.byref(cb)) == -2
    for d in (8, 9, 12, 100, 1023, 1024):  # any head dimension in [8, 1024]
        assert lib.kvq_build_codebooks(d, 2, None, ctypes.byref(cb)) == 0 and cb.n_words == kvq.n_words(d, 2)
    for b in (0, 5, -1):
        assert lib.kvq_build_codebooks(128, b, None, ctypes.byref(cb)) == -2
    assert lib.kvq_build_codebooks(128, 2, None, None) == -1
    bad = (ctypes.c_int8 * 8)(1, 1, 0, 1, 1, 1, 1, 1)
    assert lib.kvq_build_codebooks(8, 2, bad, ctypes.byref(cb)) == -1
    assert kvq.kvq_status_str(-3).startswith("misaligned") and kvq.kvq_status_str(99) == "unknown status"


def _enc(cb, x, B, H, S, p1, p2, nrm, S_cap, s_off):
    lib = kvq.load()
    return lib.kvq_rvq_encode_pack(cb, x, B, H, S, p1, p2, nrm, S_cap, s_off, None)


def _dec(cb, p1, p2, nrm, B, H, S_cap, s_off, S, out):
    lib = kvq.load()
    return lib.kvq_rvq_unpack_decode(cb, p1, p2, nrm, B, H, S_cap, s_off, S, out, None)


def test_host_side_argument_checks():
    """Every rejection below happens before any HIP call (fake pointers are never used)."""
    cb = kvq.build_codebooks(128, 2)
    pcb = ctypes.byref(cb)
    A = 0x10000  # a 16-byte aligned fake address: only reached by calls that must reject
    # null codebooks / inconsistent codebooks
    assert _enc(None, A, 1, 1, 1, A, A, A, 1, 0) == -1
    broken = kvq.Codebooks.from_buffer_copy(cb)
    broken.n_words = 7
    assert _enc(ctypes.byref(broken), A, 1, 1, 1, A, A, A, 1, 0) == -1
    broken = kvq.Codebooks.from_buffer_copy(cb)
    broken.d = 1025  # above the largest head dimension
    assert _enc(ctypes.byref(broken), A, 1, 1, 1, A, A, A, 1, 0) == -2
    broken.d = 64   # the word count of d = 128
    assert _enc(ctypes.byref(broken), A, 1, 1, 1, A, A, A, 1, 0) == -1
    # shapes and ranges
    assert _enc(pcb, A, -1, 1, 1, A, A, A, 1, 0) == -2
    assert _enc(pcb, A, 1, 1, 5, A, A, A, 4, 0) == -4        # S > S_cap
    assert _enc(pcb, A, 1, 1, 2, A, A, A, 4, 3) == -4        # s_offset + S > S_cap
    assert _enc(pcb, A, 1, 1, 1, A, A, A, 4, -1) == -4
    assert _enc(pcb, A, 1 << 40, 1 << 20, 1, A, A, A, 1, 0) == -4   # overflow
    # nothing to do: OK without touching any pointer
    assert _enc(pcb, None, 0, 32, 8, None, None, None, 8, 0) == 0
    assert _dec(pcb, None, None, None, 4, 0, 8, 0, 8, None) == 0
    # null and misaligned buffers
    assert _enc(pcb, None, 1, 1, 1, A, A, A, 1, 0) == -1
    assert _enc(pcb, A, 1, 1, 1, A, None, A, 1, 0) == -1
    assert _enc(pcb, A + 8, 1, 1, 1, A, A, A, 1, 0) == -3
    assert _enc(pcb, A, 1, 1, 1, A + 4, A, A, 1, 0) == -3
    assert _enc(pcb, A, 1, 1, 1, A, A, A + 2, 1, 0) == -3
    assert _dec(pcb, A, A, None, 1, 1, 4, 0, 4, A + 2) == -3
    assert _dec(pcb, None, A, None, 1, 1, 4, 0, 4, A) == -1
    assert _dec(pcb, A, A, None, 1, 1, 4, 2, 4, A) == -4


def test_single_stage_host_side_argument_checks():
    """The single-stage entry points share the checks; the second stream is not needed."""
    lib = kvq.load()
    cb = kvq.build_codebooks(128, 2)
    pcb = ctypes.byref(cb)
    A = 0x10000
    enc = lambda *a: lib.kvq_mse_encode_pack(*a, None)
    dec = lambda *a: lib.kvq_mse_unpack_decode(*a, None)
    assert enc(None, A, 1, 1, 1, A, A, 1, 0) == -1
    assert enc(pcb, A, 1, 1, 5, A, A, 4, 0) == -4
    assert enc(pcb, None, 0, 3, 3, None, None, 3, 0) == 0
    assert enc(pcb, None, 1, 1, 1, A, A, 1, 0) == -1
    assert enc(pcb, A, 1, 1, 1, None, A, 1, 0) == -1
    assert enc(pcb, A, 1, 1, 1, A, None, 1, 0) == -1
    assert enc(pcb, A, 1, 1, 1, A + 4, A, 1, 0) == -3
    assert enc(pcb, A + 2, 1, 1, 1, A, A, 1, 0) == -3
    assert dec(pcb, None, None, 1, 1, 4, 0, 4, A) == -1
    assert dec(pcb, A, None, 1, 1, 4, 0, 4, A + 2) == -3
    assert dec(pcb, A, None, 1, 1, 4, 2, 4, A) == -4
    assert dec(pcb, None, None, 0, 1, 4, 0, 4, None) == 0


def test_attend_host_side_argument_checks():
    """Every rejection happens on the host; the workspace size follows the documented plan."""
    lib = kvq.load()
    cb = kvq.build_codebooks(128, 2)
    cb4 = kvq.build_codebooks(128, 4)
    cb64 = kvq.build_codebooks(64, 2)
    A = 0x10000
    P = ctypes.byref

    def att(cbk=cb, cbv=cb, q=A, B=1, Hq=4, Sq=1, Hkv=2, ptrs=(A, A, A, A, A, A), S_cap=100, S_kv=50, scale=0.1,
            ws=A, wsb=1 << 30, out=A):
        return lib.kvq_rvq_attend(P(cbk) if cbk is not None else None, P(cbv) if cbv is not None else None, q, B, Hq,
                                  Sq, Hkv, *ptrs, S_cap, S_kv, scale, ws, wsb, out, None)

    assert att(cbk=None) == -1
    assert att(cbv=cb4) == -2 and att(cbv=cb64) == -2
    assert att(Hq=3) == -2 and att(Hkv=0) == -2 and att(B=-1) == -2
    assert att(S_kv=0) == -4 and att(S_kv=101) == -4
    assert att(B=0) == 0 and att(Hq=0, Hkv=0) == 0 and att(Sq=0) == 0
    assert att(scale=float("inf")) == -1 and att(scale=float("nan")) == -1
    assert att(q=None) == -1 and att(ws=None) == -1 and att(out=None) == -1
    assert att(ptrs=(A, A, None, A, A, A)) == -1
    assert att(q=A + 2) == -3 and att(out=A + 8) == -3 and att(ws=A + 4) == -3
    assert att(ptrs=(A + 4, A, A, A, A, A)) == -3 and att(ptrs=(A, A, A + 2, A, A, A)) == -3
    need = kvq.kvq_rvq_attend_workspace_size(128, 2, 1, 4, 1, 2, 50)
    assert need > 0 and att(wsb=need - 1) == -4
    assert lib.kvq_rvq_attend_workspace_size(128, 2, 1, 4, 1, 2, 50, None) == -1
    with pytest.raises(kvq.KvqError):
        kvq.kvq_rvq_attend_workspace_size(96, 2, 1, 4, 1, 2, 50)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_rvq_attend_workspace_size(128, 2, 1, 4, 1, 2, 0)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_rvq_attend_workspace_size(128, 2, 1, 4, 1, 3, 50)
    with pytest.raises(kvq.KvqError):
        kvq.kvq_rvq_attend_workspace_size(128, 5, 1, 4, 1, 2, 50)
    # plan. Matrix path (d = 64 or 128, b = 1, 2, 4, d b >= 128): 16 query vectors per wave
    # unit, units per split = heads x ceil(queries per head / 16), chunks of 32-position
    # iterations, at least 4. Otherwise nqw query vectors per wave (4, 2 or 1, dividing the
    # query vectors per head), chunks of 64 / (d / 16) positions with nqw > 1, else
    # 64 / (d / 32), at least 8 iterations. Both: about 2048 waves, at most 4096 chunks.
    for (d, bits, B, Hq, Sq, Hkv, S_kv) in ((128, 2, 1, 32, 1, 8, 32768), (128, 2, 1, 1, 1, 1, 5),
                                            (128, 3, 4, 8, 3, 4, 1000), (128, 3, 1, 32, 1, 32, 1),
                                            (64, 1, 2, 6, 1, 2, 700), (64, 2, 2, 6, 1, 2, 700),
                                            (1024, 2, 1, 8, 1, 2, 3000), (16, 4, 1, 4, 2, 1, 77),
                                            (128, 4, 1, 1, 1, 1, 10 ** 7), (128, 3, 1, 1, 1, 1, 10 ** 7),
                                            (128, 1, 2, 40, 1, 2, 5000)):
        nq = B * Hq * Sq
        gq = (Hq // Hkv) * Sq
        if d in (64, 128) and bits != 3 and d * bits >= 128:
            vw, min_it, per_split = 32, 4, (nq // gq) * -(-gq // 16)
        else:
            nqw = (4 if gq % 4 == 0 else 2 if gq % 2 == 0 else 1) if d <= 512 else 1
            cm = 16 if nqw > 1 and d >= 32 else 32
            vw, min_it, per_split = 64 // (d // min(d, cm)), 8, nq // nqw
        splits0 = -(-2048 // per_split)
        chunk = -(-S_kv // splits0)
        chunk = max(-(-chunk // vw) * vw, min_it * vw)
        min_chunk = -(-S_kv // 4096)
        if chunk < min_chunk:
            chunk = -(-min_chunk // vw) * vw
        n_splits = -(-S_kv // chunk)
        assert kvq.kvq_rvq_attend_workspace_size(d, bits, B, Hq, Sq, Hkv, S_kv) == nq * n_splits * (d + 4) * 4, \
            (d, bits, B, Hq, Sq, Hkv, S_kv)


def test_python_binding_rejects_cpu_tensors():
    import torch
    cb = kvq.build_codebooks(128, 2)
    x = torch.zeros(1, 1, 4, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        kvq.encode(x, cb)


def test_sign_code_host_checks():
    """kvq_rabitq_encode_pack: bits must be 1; the shared size, pointer and alignment checks
    run before any HIP call (no GPU here)."""
    lib = kvq.load()
    A = 1 << 20
    cb1, cb2 = kvq.build_codebooks(128, 1), kvq.build_codebooks(128, 2)

    def enc(cb=cb1, x=A, B=1, H=2, S=3, p=A, n=A, S_cap=3, s_off=0):
        return lib.kvq_rabitq_encode_pack(None if cb is None else ctypes.byref(cb), x, B, H, S, p, n, S_cap, s_off,
                                          None)

    assert enc(cb=None) == -1
    assert enc(cb=cb2) == -2
    assert enc(B=-1) == -2
    assert enc(S=4) == -4 and enc(s_off=1) == -4
    assert enc(B=0) == 0 and enc(S=0) == 0
    assert enc(x=None) == -1 and enc(p=None) == -1 and enc(n=None) == -1
    assert enc(x=A + 2) == -3 and enc(p=A + 4) == -3 and enc(n=A + 2) == -3


def test_qjl_host_checks():
    """kvq_qjl_supported's shape table and kvq_qjl_encode_pack's checks before any HIP call."""
    lib = kvq.load()
    # the sketch (2 m d bytes) and one 32-key tile per wave (4 waves) fit the 160 KiB of LDS
    # of a gfx950 workgroup
    ok = {(d, m) for d in (32, 64, 128, 256) for m in range(32, 257, 32)
          if 2 * m * d + 4 * 32 * d * 2 <= 160 * 1024}
    assert (128, 256) in ok and (256, 192) in ok and (256, 224) not in ok
    assert (64, 256) in ok and (32, 256) in ok
    for d in (16, 32, 48, 64, 128, 256, 512):
        for m in (0, 16, 32, 64, 96, 100, 128, 160, 192, 224, 256, 288, 512):
            assert (lib.kvq_qjl_supported(d, m) == 0) == ((d, m) in ok), (d, m)
            assert kvq.kvq_qjl_supported(d, m) == ((d, m) in ok)
    A = 1 << 20

    def enc(sk=A, d=128, m=128, x=A, B=1, H=2, S=3, p=A, n=A, S_cap=3, s_off=0):
        return lib.kvq_qjl_encode_pack(sk, d, m, x, B, H, S, p, n, S_cap, s_off, None)

    assert enc(d=96) == -2 and enc(m=100) == -2 and enc(d=256, m=224) == -2 and enc(m=288) == -2
    assert enc(H=-1) == -2
    assert enc(S_cap=2) == -4 and enc(s_off=1) == -4 and enc(s_off=-1) == -4
    assert enc(B=0) == 0 and enc(S=0, S_cap=0) == 0
    assert enc(sk=None) == -1 and enc(x=None) == -1 and enc(p=None) == -1 and enc(n=None) == -1
    assert enc(sk=A + 8) == -3 and enc(x=A + 2) == -3 and enc(p=A + 4) == -3 and enc(n=A + 1) == -3
