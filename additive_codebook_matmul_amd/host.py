"""ctypes binding of the host (CPU) GEMV library (libaqlm_host.so, C ABI in
include/aqlm_host.h).

Argument marshalling only: numpy arrays are checked for dtype, shape and
contiguity and their host pointers are handed to aqlm_host_gemv. This is a
separate entry point for activations in host memory; the GPU binding never
calls it. If the library has not been built, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from ._lib import AQLM_CODES_PACKED, AQLM_OK, STATUS_NAMES, AqlmError, AqlmLayerStruct

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(_PKG_DIR, "libaqlm_host.so")
HOST_EXPORTED_SYMBOLS = ("aqlm_host_gemv", "aqlm_host_isa")

_hlib: Optional[ctypes.CDLL] = None


def load_host_library() -> ctypes.CDLL:
    global _hlib
    if _hlib is not None:
        return _hlib
    if not os.path.exists(HOST_LIB_PATH):
        raise RuntimeError(f"host library not found at {HOST_LIB_PATH}; build it with "
                           "`python -m additive_codebook_matmul_amd.build`")
    lib = ctypes.CDLL(HOST_LIB_PATH)
    lib.aqlm_host_gemv.argtypes = [ctypes.POINTER(AqlmLayerStruct), ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32]
    lib.aqlm_host_gemv.restype = ctypes.c_int
    lib.aqlm_host_isa.argtypes = []
    lib.aqlm_host_isa.restype = ctypes.c_char_p
    _hlib = lib
    return lib


def host_isa() -> str:
    """Instruction set the host library selected ("avx2" or "scalar")."""
    return load_host_library().aqlm_host_isa().decode()


def host_gemv(codes: np.ndarray, codebooks: np.ndarray, scales: np.ndarray, x: np.ndarray,
              threads: int = 0, out: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x . W^T on the host for 1..8 activation rows (aqlm_host_gemv).

    codes [out, in/g, M] uint8 (B = 8) or uint16 (B > 8), or the bit-packed
    stream as a 1-D uint32 array; codebooks [M, 2**B, g] float16; scales [out]
    float16; x [batch, in] float16. Returns [batch, out] float16. threads <= 0
    lets the OpenMP runtime choose.
    """
    lib = load_host_library()
    if codes.ndim not in (1, 3) or codebooks.ndim != 3 or scales.ndim != 1 or x.ndim != 2:
        raise ValueError("codes [out, in/g, M] or a packed stream, codebooks [M, 2**B, g], "
                         "scales [out], x [batch, in]")
    Mc, ncode, g = codebooks.shape
    if ncode < 2 or ncode & (ncode - 1):
        raise ValueError("codebook size must be a power of two")
    B = ncode.bit_length() - 1
    M, n_out = Mc, scales.shape[0]
    packed = codes.ndim == 1
    if packed:
        if x.shape[1] % g:
            raise ValueError("in must be a multiple of g")
        J = x.shape[1] // g
        if codes.dtype != np.uint32 or codes.size != (n_out * J * M * B + 31) // 32:
            raise ValueError("a packed code stream is ceil(out*in/g*M*B/32) uint32 words")
    else:
        n_out_c, J, Mcodes = codes.shape
        if Mcodes != M or n_out_c != n_out:
            raise ValueError("codes, codebooks and scales disagree in shape")
        if codes.dtype != (np.uint8 if B <= 8 else np.uint16):
            raise ValueError(f"codes dtype {codes.dtype} does not match {B}-bit codes")
    for a, name in ((codebooks, "codebooks"), (scales, "scales"), (x, "x")):
        if a.dtype != np.float16:
            raise ValueError(f"{name} must be float16")
    if x.shape[1] != J * g:
        raise ValueError(f"x must be [batch, {J * g}]")
    arrs = [np.ascontiguousarray(a) for a in (codes, codebooks, scales, x)]
    codes, codebooks, scales, x = arrs
    batch = x.shape[0]
    if out is None:
        out = np.empty((batch, n_out), dtype=np.float16)
    elif out.shape != (batch, n_out) or out.dtype != np.float16 or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous float16 [batch, out] array")
    st = AqlmLayerStruct(int(n_out), int(J * g), int(M), int(B), int(g),
                         AQLM_CODES_PACKED if packed else 0,
                         codes.ctypes.data, codebooks.ctypes.data, scales.ctypes.data)
    status = lib.aqlm_host_gemv(ctypes.byref(st), x.ctypes.data, batch, out.ctypes.data,
                                int(threads))
    if status != AQLM_OK:
        raise AqlmError(status, STATUS_NAMES.get(status, str(status)))
    return out
