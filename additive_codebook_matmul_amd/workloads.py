"""Seeded synthetic workloads: layer shapes, schemes and input generators.

This module only draws random inputs of the right shapes and value
distributions. It holds none of the method's arithmetic (no decode, no
product), so both the HIP path and the CPU oracle can take their inputs
from it without sharing any computation.

Packed format (one quantized linear layer, out x in):
  codes      [out, in/g, M]   uint8 (B = 8) or uint16 (B > 8), m fastest
  codebooks  [M, 2**B, g]     float16
  scales     [out]            float16
  x          [batch, in]      float16

Value distributions: codes uniform over [0, 2**B); codebook entries drawn
from N(0, 0.02) in float64 then rounded to float16; scales U(0.5, 1.5)
rounded to float16; x standard normal rounded to float16. The random
generator is numpy's PCG64 (default_rng), drawn in the order codes,
codebooks, scales, x, so that the batch size changes only x.

Shapes follow the linear layers of Llama-2-7B (hidden 4096, MLP 11008) and
Llama-2-70B (hidden 8192, MLP 28672, grouped-query k/v of 1024 rows); the
schemes are the pages' "2x8" (two 8-bit codebooks) and "1x16" (one 16-bit
codebook) with codeword length g = 8, plus a g = 16 variant of 1x16, and a
set of general schemes (1..8 codebooks of 8..16-bit codes, g = 8 or 16).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np


@dataclass(frozen=True)
class Scheme:
    """An additive codebook scheme: M codebooks of 2**B codewords of length g."""
    M: int
    B: int
    g: int

    @property
    def name(self) -> str:
        return f"{self.M}x{self.B}g{self.g}"

    @property
    def code_dtype(self):
        return np.uint8 if self.B <= 8 else np.uint16


S2x8 = Scheme(2, 8, 8)
S1x16 = Scheme(1, 16, 8)
S1x16g16 = Scheme(1, 16, 16)


@dataclass(frozen=True)
class Layer:
    name: str
    out_features: int
    in_features: int
    scheme: Scheme
    seed: int
    packed: bool = False  # codes handed over bit-packed (pack_codes) rather than one per element


@dataclass(frozen=True)
class Workload:
    """A named set of layers and the batch sizes each is run at."""
    name: str
    index: int
    layers: Tuple[Layer, ...]
    batches: Tuple[int, ...]
    description: str = ""


_LLAMA2_7B = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
              ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
              ("down", 4096, 11008))
_LLAMA2_70B = (("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192),
               ("o", 8192, 8192), ("gate", 28672, 8192), ("up", 28672, 8192),
               ("down", 8192, 28672))


def _layers(index: int, shapes, scheme: Scheme) -> Tuple[Layer, ...]:
    return tuple(Layer(n, o, i, scheme, 1000 * index + li)
                 for li, (n, o, i) in enumerate(shapes))


def _gemm_layers(index: int) -> Tuple[Layer, ...]:
    out = []
    li = 0
    for scheme in (S1x16g16, S2x8):
        for n, o, i in (("up", 11008, 4096), ("down", 4096, 11008)):
            out.append(Layer(f"{n}_{scheme.name}", o, i, scheme, 1000 * index + li))
            li += 1
    return tuple(out)


# Schemes beyond the three named ones: more codebooks, wider codes, both
# codeword lengths (M x B bits, g), on a Llama-2-7B attention-shaped layer.
GENERAL_SCHEMES = (Scheme(1, 8, 8), Scheme(3, 8, 8), Scheme(4, 8, 8), Scheme(4, 8, 16),
                   Scheme(8, 8, 16), Scheme(1, 12, 8), Scheme(2, 12, 16), Scheme(2, 16, 8))


# The same, with codes bit-packed: B bits per code whatever B is, so that the
# codes cost exactly M*B/g bits per weight.
PACKED_SCHEMES = (Scheme(1, 12, 8), Scheme(2, 12, 16), Scheme(2, 10, 8), Scheme(3, 9, 16))


def _general_layers(index: int) -> Tuple[Layer, ...]:
    plain = tuple(Layer(f"q_{s.name}", 4096, 4096, s, 1000 * index + li)
                  for li, s in enumerate(GENERAL_SCHEMES))
    base = len(plain)
    packed = tuple(Layer(f"q_{s.name}_packed", 4096, 4096, s, 1000 * index + base + li, True)
                   for li, s in enumerate(PACKED_SCHEMES))
    return plain + packed


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in (
        Workload("single_2x8_512x1024", 1,
                 (Layer("single", 512, 1024, S2x8, 1000),), (1,),
                 "one 512x1024 layer, scheme 2x8 g8, batch 1"),
        Workload("llama2_7b_2x8", 2, _layers(2, _LLAMA2_7B, S2x8), (1,),
                 "Llama-2-7B linear layers, scheme 2x8 g8, batch 1"),
        Workload("llama2_7b_1x16", 3, _layers(3, _LLAMA2_7B, S1x16), (1, 4, 8),
                 "Llama-2-7B linear layers, scheme 1x16 g8, batch 1/4/8"),
        Workload("llama2_70b_1x16", 4, _layers(4, _LLAMA2_70B, S1x16), (1,),
                 "Llama-2-70B linear layers, scheme 1x16 g8, batch 1"),
        Workload("gemm_mlp", 5, _gemm_layers(5), (16, 128, 2048),
                 "MLP-shaped layers (11008x4096, 4096x11008), schemes 1x16 g16 "
                 "and 2x8 g8, batch 16/128/2048"),
        Workload("general_schemes", 6, _general_layers(6), (1, 8, 16),
                 "4096x4096 layers under general schemes (M = 1..8 codebooks, "
                 "B = 8..16 bits, g = 8/16), batch 1/8/16"),
    )
}


@dataclass
class LayerData:
    layer: Layer
    codes: np.ndarray       # [out, in/g, M] uint8/uint16
    codebooks: np.ndarray   # [M, 2**B, g] float16
    scales: np.ndarray      # [out] float16

    @property
    def scheme(self) -> Scheme:
        return self.layer.scheme


def make_packed(out_features: int, in_features: int, scheme: Scheme, seed: int,
                codebook_std: float = 0.02,
                scale_range: Tuple[float, float] = (0.5, 1.5)) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.random.Generator]:
    """Draw (codes, codebooks, scales) and return the generator for x."""
    if in_features % scheme.g:
        raise ValueError("in_features must be a multiple of the group size")
    rng = np.random.default_rng(seed)
    J = in_features // scheme.g
    codes = rng.integers(0, 2 ** scheme.B, size=(out_features, J, scheme.M),
                         dtype=scheme.code_dtype)
    codebooks = rng.normal(0.0, codebook_std,
                           size=(scheme.M, 2 ** scheme.B, scheme.g)).astype(np.float16)
    scales = rng.uniform(scale_range[0], scale_range[1], size=out_features).astype(np.float16)
    return codes, codebooks, scales, rng


def make_layer(layer: Layer) -> LayerData:
    codes, codebooks, scales, _ = make_packed(layer.out_features, layer.in_features,
                                              layer.scheme, layer.seed)
    return LayerData(layer, codes, codebooks, scales)


def make_x(layer: Layer, batch: int) -> np.ndarray:
    """x for a layer at a batch size: the draw that follows the layer's weights."""
    _, _, _, rng = make_packed(layer.out_features, layer.in_features, layer.scheme,
                               layer.seed)
    return rng.standard_normal((batch, layer.in_features)).astype(np.float16)


def make_x_only(batch: int, in_features: int, seed: int) -> np.ndarray:
    """A standalone fp16 activation batch (for cases with no layer attached)."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((batch, in_features)).astype(np.float16)


def small_case(out_features: int, in_features: int, scheme: Scheme, batch: int,
               seed: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """A small random layer plus x, for parity at sizes the oracle finishes fast."""
    codes, codebooks, scales, rng = make_packed(out_features, in_features, scheme, seed)
    x = rng.standard_normal((batch, in_features)).astype(np.float16)
    return codes, codebooks, scales, x


def pack_codes(codes: np.ndarray, B: int) -> np.ndarray:
    """The bit-packed storage of a code array: code i of the flattened array
    occupies bits i*B .. i*B+B-1 of a stream of little-endian 32-bit words,
    least significant bit first. Returns ceil(n*B/32) uint32 words."""
    flat = np.asarray(codes).reshape(-1).astype(np.uint64)
    nwords = (flat.size * B + 31) // 32
    words = np.zeros(nwords + 1, dtype=np.uint64)
    bit = np.arange(flat.size, dtype=np.uint64) * np.uint64(B)
    word = (bit >> np.uint64(5)).astype(np.int64)
    shifted = flat << (bit & np.uint64(31))
    # codes occupy disjoint bits, so adding them into a word never carries
    np.add.at(words, word, shifted & np.uint64(0xFFFFFFFF))
    np.add.at(words, word + 1, shifted >> np.uint64(32))
    return words[:nwords].astype(np.uint32)


def workload_bytes(layer: Layer, batch: int) -> Dict[str, int]:
    """Byte counts of the packed tensors and activations of one layer."""
    s = layer.scheme
    J = layer.in_features // s.g
    if layer.packed:
        code_bytes = (layer.out_features * J * s.M * s.B + 31) // 32 * 4
    else:
        code_bytes = layer.out_features * J * s.M * np.dtype(s.code_dtype).itemsize
    return {
        "codes": code_bytes,
        "codebooks": s.M * (2 ** s.B) * s.g * 2,
        "scales": layer.out_features * 2,
        "x": batch * layer.in_features * 2,
        "y": batch * layer.out_features * 2,
    }


# ---------------------------------------------------------------------------
# Inputs of the toy encoder: a dense float16 weight matrix and the seeded
# starting indices of each codebook's k-means. Random draws only; the encoder's
# arithmetic lives in the library and, separately, in the oracle.
# ---------------------------------------------------------------------------
def make_dense_weight(out_features: int, in_features: int, seed: int,
                      std: float = 0.02) -> np.ndarray:
    """A dense weight matrix [out, in]: N(0, std) drawn in float64, rounded to float16."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, std, size=(out_features, in_features)).astype(np.float16)


def kmeans_init_indices(n_vectors: int, K: int, M: int, seed: int) -> List[np.ndarray]:
    """For each of M codebooks, K starting vector indices: K distinct indices
    drawn uniformly when n_vectors >= K, otherwise a random permutation of all
    vectors repeated to length K. int64, one array per codebook."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(M):
        if n_vectors >= K:
            idx = rng.choice(n_vectors, size=K, replace=False)
        else:
            idx = np.resize(rng.permutation(n_vectors), K)
        out.append(np.ascontiguousarray(idx, dtype=np.int64))
    return out
