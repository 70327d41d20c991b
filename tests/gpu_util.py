"""Helpers for GPU parity tests: move seeded numpy inputs to the device and
compare library outputs with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from additive_codebook_matmul_amd import AqlmLayer

# Acceptance tolerance of a product: |y - y_ref| <= 1e-2 * sum_i |x_i w_i|.
REL_TOL = 1e-2
# Tight gate derived from the arithmetic (fp16 rounding of y, of W in the
# lookup path or of the codeword sum in the matrix-core path, and float32
# accumulation together stay below ~1e-3 of sum |x w|); it catches dropped or
# duplicated groups that the loose tolerance cannot see.
TIGHT_TOL = 1e-3


def device():
    return torch.device("cuda:0")


def to_dev_codes(codes: np.ndarray) -> torch.Tensor:
    if codes.dtype == np.uint16:
        codes = codes.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(codes)).to(device())


def dev_layer(codes, books, scales) -> AqlmLayer:
    return AqlmLayer(to_dev_codes(codes),
                     torch.from_numpy(np.ascontiguousarray(books)).to(device()),
                     torch.from_numpy(np.ascontiguousarray(scales)).to(device()))


def dev_x(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(device())


def bits(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.asarray(t, dtype=np.float16).view(np.uint16)


def assert_bit_exact(w_gpu: np.ndarray, w_ref: np.ndarray, what: str = ""):
    g, r = bits(w_gpu), bits(w_ref)
    if not np.array_equal(g, r):
        idx = np.argwhere(g != r)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} mismatching weights; first at {i}: "
                             f"gpu 0x{int(g[i]):04x} oracle 0x{int(r[i]):04x}")


def assert_product(y_gpu, y_ref, bound, what: str = "", tight: float = TIGHT_TOL):
    y = np.asarray(y_gpu.detach().cpu().numpy() if isinstance(y_gpu, torch.Tensor) else y_gpu)
    ok = oracle.within_tolerance(y, y_ref, bound, rel=REL_TOL)
    if not ok.all():
        idx = np.argwhere(~ok)
        i = tuple(idx[0])
        raise AssertionError(f"{what}: {len(idx)} outputs outside 1e-2*sum|xw|; first at {i}: "
                             f"gpu {float(y[i])!r} oracle {y_ref[i]!r} bound {bound[i]!r}")
    err = np.abs(y.astype(np.float64) - y_ref)
    rel = np.where(bound > 0, err / np.where(bound > 0, bound, 1), err)
    assert rel.max() <= tight, f"{what}: tight gate {rel.max():.3e} > {tight}"
    return float(rel.max())
