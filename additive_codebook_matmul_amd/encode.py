"""Toy encoder: dense float16 weights -> the packed AQLM format, on the GPU.

A thin driver over the aqlm_encode_* kernels of libaqlm_mi355x.so (C ABI in
include/aqlm_encode.h): it allocates the device buffers with torch and calls
the kernels in the order the algorithm takes; every arithmetic step runs in
the kernels. The method is residual k-means codebooks and greedy
nearest-codeword codes under the plain squared error (no calibration data, no
training); see include/aqlm_encode.h for the exact rules, which the CPU
oracle of the toy encoder follows bit for bit.
"""
from __future__ import annotations

import ctypes
from typing import Sequence, Tuple

import numpy as np
import torch

from ._lib import _check, load_library

ENCODE_SYMBOLS = ("aqlm_encode_normalize", "aqlm_encode_init", "aqlm_encode_assign",
                  "aqlm_encode_update", "aqlm_encode_round")

_ready = False


def _lib():
    global _ready
    lib = load_library()
    if not _ready:
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.aqlm_encode_normalize.argtypes = [P, I64, I64, P, P, P]
        lib.aqlm_encode_init.argtypes = [P, I64, I32, P, I32, P, P]
        lib.aqlm_encode_assign.argtypes = [P, I64, I32, P, I32, P, I32, I32, P, P]
        lib.aqlm_encode_update.argtypes = [P, I64, I32, P, I32, I32, I32, P, P, P]
        lib.aqlm_encode_round.argtypes = [P, I64, P, P, P]
        for name in ENCODE_SYMBOLS:
            getattr(lib, name).restype = ctypes.c_int
        _ready = True
    return lib


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def normalize(W: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """(scales [out] float16, vecs [out, in] float32) of a dense float16 layer."""
    if W.dtype != torch.float16 or W.dim() != 2 or not W.is_cuda or not W.is_contiguous():
        raise ValueError("W must be a contiguous float16 [out, in] tensor on the GPU")
    out, n_in = W.shape
    scales = torch.empty(out, dtype=torch.float16, device=W.device)
    vecs = torch.empty((out, n_in), dtype=torch.float32, device=W.device)
    with torch.cuda.device(W.device):
        _check(_lib().aqlm_encode_normalize(W.data_ptr(), out, n_in, scales.data_ptr(),
                                            vecs.data_ptr(), _stream(W.device)))
    return scales, vecs


def assign(vecs: torch.Tensor, centroids: torch.Tensor, codes: torch.Tensor, M: int, m: int,
           residual: torch.Tensor = None) -> None:
    """codes[:, m] = nearest centroid of each row of vecs [n, g]; optional residual."""
    n, g = vecs.shape
    with torch.cuda.device(vecs.device):
        _check(_lib().aqlm_encode_assign(vecs.data_ptr(), n, g, centroids.data_ptr(),
                                         centroids.shape[0], codes.data_ptr(), M, m,
                                         _ptr(residual), _stream(vecs.device)))


def update(vecs: torch.Tensor, codes: torch.Tensor, M: int, m: int, centroids: torch.Tensor,
           workspace: torch.Tensor) -> None:
    """Move every centroid with vectors to their (fixed-point exact) mean."""
    n, g = vecs.shape
    with torch.cuda.device(vecs.device):
        _check(_lib().aqlm_encode_update(vecs.data_ptr(), n, g, codes.data_ptr(),
                                         centroids.shape[0], M, m, centroids.data_ptr(),
                                         workspace.data_ptr(), _stream(vecs.device)))


def encode_layer(W: torch.Tensor, M: int, B: int, g: int, iters: int,
                 init_indices: Sequence[np.ndarray]) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Encode a dense float16 layer [out, in] into (codes [out, in/g, M],
    codebooks [M, 2**B, g] float16, scales [out] float16) on W's device.

    init_indices[m] holds the 2**B seeded starting vectors of codebook m's
    k-means (int64, values below out * in / g); iters Lloyd iterations per
    codebook."""
    if not (1 <= M <= 8 and 8 <= B <= 16 and g in (8, 16)):
        raise ValueError("need 1 <= M <= 8, 8 <= B <= 16, g in (8, 16)")
    out, n_in = W.shape
    if n_in % g:
        raise ValueError("in must be a multiple of g")
    if len(init_indices) < M:
        raise ValueError("one array of starting indices per codebook")
    dev = W.device
    K = 2 ** B
    n = out * n_in // g
    lib = _lib()
    scales, vecs = normalize(W)
    r = vecs.view(n, g)                      # residual, updated in place
    codes = torch.empty((out, n_in // g, M), dtype=torch.uint8 if B == 8 else torch.int16,
                        device=dev)
    books = torch.empty((M, K, g), dtype=torch.float16, device=dev)
    cents = torch.empty((K, g), dtype=torch.float32, device=dev)
    ws = torch.empty(K * (g + 1), dtype=torch.int64, device=dev)
    with torch.cuda.device(dev):
        stream = _stream(dev)
        for m in range(M):
            idx = torch.from_numpy(np.ascontiguousarray(init_indices[m], dtype=np.int64)).to(dev)
            if idx.numel() != K:
                raise ValueError(f"codebook {m}: need {K} starting indices")
            _check(lib.aqlm_encode_init(r.data_ptr(), n, g, idx.data_ptr(), K, cents.data_ptr(),
                                        stream))
            for _ in range(iters):
                assign(r, cents, codes, M, m)
                update(r, codes, M, m, cents, ws)
            _check(lib.aqlm_encode_round(cents.data_ptr(), K * g, books[m].data_ptr(),
                                         cents.data_ptr(), stream))
            assign(r, cents, codes, M, m, residual=r)
    return codes, books, scales
