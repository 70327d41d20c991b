"""ctypes binding of the HIP library (libaqlm_mi355x.so).

Argument marshalling only: torch tensors are checked for device, dtype,
shape, contiguity and alignment, and their device pointers and the current
HIP stream are handed to the C entry points. Every step of the computation
runs in the library's kernels. There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libaqlm_mi355x.so")

AQLM_OK = 0
STATUS_NAMES = {0: "AQLM_OK", 1: "AQLM_ERR_NULL", 2: "AQLM_ERR_SHAPE", 3: "AQLM_ERR_SCHEME",
                4: "AQLM_ERR_ALIGN", 5: "AQLM_ERR_BATCH", 6: "AQLM_ERR_HIP",
                7: "AQLM_ERR_WORKSPACE", 8: "AQLM_ERR_SCRATCH"}
EXPORTED_SYMBOLS = ("aqlm_dequant", "aqlm_gemv", "aqlm_gemv_batched", "aqlm_gemv_workspace_size",
                    "aqlm_gemv_ws", "aqlm_gemm", "aqlm_gemm_workspace_size", "aqlm_gemm_ws",
                    "aqlm_gemm_noalloc", "aqlm_status_string", "aqlm_abi_version")
ABI_VERSION = 5
# bytes of the library's static scratch array (AQLM_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 64 << 20
AQLM_CODES_PACKED = 1
SCHEMES = {(2, 8, 8): "2x8", (1, 16, 8): "1x16", (1, 16, 16): "1x16g16"}


class AqlmLayerStruct(ctypes.Structure):
    """Mirror of struct aqlm_layer in include/aqlm.h."""
    _fields_ = [
        ("out_features", ctypes.c_int64),
        ("in_features", ctypes.c_int64),
        ("num_codebooks", ctypes.c_int32),
        ("nbits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("codes", ctypes.c_void_p),
        ("codebooks", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
    ]


class AqlmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the built library (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not found at {LIB_PATH}; build it with "
            "`python -m additive_codebook_matmul_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lp = ctypes.POINTER(AqlmLayerStruct)
    lib.aqlm_dequant.argtypes = [lp, ctypes.c_void_p, ctypes.c_void_p]
    lib.aqlm_dequant.restype = ctypes.c_int
    for name in ("aqlm_gemv", "aqlm_gemm", "aqlm_gemm_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = [lp, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.aqlm_gemm_workspace_size.argtypes = [lp, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    lib.aqlm_gemm_workspace_size.restype = ctypes.c_int
    lib.aqlm_gemm_ws.argtypes = [lp, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.aqlm_gemm_ws.restype = ctypes.c_int
    lib.aqlm_gemv_batched.argtypes = [lp, ctypes.POINTER(ctypes.c_void_p),
                                      ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32,
                                      ctypes.c_int64, ctypes.c_void_p]
    lib.aqlm_gemv_batched.restype = ctypes.c_int
    lib.aqlm_gemv_workspace_size.argtypes = [lp, ctypes.c_int32, ctypes.c_int64,
                                             ctypes.POINTER(ctypes.c_int64)]
    lib.aqlm_gemv_workspace_size.restype = ctypes.c_int
    lib.aqlm_gemv_ws.argtypes = [lp, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                 ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p]
    lib.aqlm_gemv_ws.restype = ctypes.c_int
    lib.aqlm_status_string.argtypes = [ctypes.c_int]
    lib.aqlm_status_string.restype = ctypes.c_char_p
    lib.aqlm_abi_version.argtypes = []
    lib.aqlm_abi_version.restype = ctypes.c_int
    if lib.aqlm_abi_version() != ABI_VERSION:
        raise RuntimeError("libaqlm_mi355x.so ABI version mismatch; rebuild the library")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().aqlm_status_string(status).decode()


def _check(status: int) -> None:
    if status != AQLM_OK:
        raise AqlmError(status, status_string(status))


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class AqlmLayer:
    """A quantized linear layer held as device tensors in the packed format.

    codes      [out, in/g, M]  torch.uint8 (B = 8) or torch.int16/uint16 bits (B > 8),
               or the bit-packed stream: a 1-D torch.int32/uint32 tensor of
               ceil(out * in/g * M * B / 32) words (then in_features is required)
    codebooks  [M, 2**B, g]    torch.float16
    scales     [out]           torch.float16
    """

    def __init__(self, codes: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor,
                 in_features: Optional[int] = None):
        if codebooks.dim() != 3 or scales.dim() != 1 or codes.dim() not in (1, 3):
            raise ValueError("codes [out, in/g, M] (or a packed 1-D stream), "
                             "codebooks [M, 2**B, g], scales [out]")
        M, ncode, g = codebooks.shape
        out = scales.shape[0]
        if ncode < 2 or ncode & (ncode - 1):
            raise ValueError("codebook size must be a power of two")
        B = ncode.bit_length() - 1
        self.packed = codes.dim() == 1
        if self.packed:
            if in_features is None or in_features % g:
                raise ValueError("a packed code stream needs in_features, a multiple of g")
            J = in_features // g
            if codes.dtype not in (torch.int32, torch.uint32):
                raise ValueError("a packed code stream is 32-bit words")
            if codes.numel() != (out * J * M * B + 31) // 32:
                raise ValueError("packed code stream length does not match the layer")
        else:
            out_c, J, Mcodes = codes.shape
            if Mcodes != M or out_c != out:
                raise ValueError("codes, codebooks and scales disagree in shape")
            want = (torch.uint8,) if B <= 8 else (torch.int16, torch.uint16)
            if codes.dtype not in want:
                raise ValueError(f"codes dtype {codes.dtype} does not match {B}-bit codes")
        if codebooks.dtype != torch.float16 or scales.dtype != torch.float16:
            raise ValueError("codebooks and scales must be float16")
        for t in (codes, codebooks, scales):
            if not t.is_cuda:
                raise ValueError("all tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")
        if not (codes.device == codebooks.device == scales.device):
            raise ValueError("all tensors must be on one device")
        self.codes, self.codebooks, self.scales = codes, codebooks, scales
        self.out_features, self.in_features = int(out), int(J * g)
        self.M, self.B, self.g = int(M), int(B), int(g)
        self.device = codes.device
        self._struct = AqlmLayerStruct(self.out_features, self.in_features, self.M, self.B, self.g,
                                       AQLM_CODES_PACKED if self.packed else 0, codes.data_ptr(),
                                       codebooks.data_ptr(), scales.data_ptr())

    @property
    def scheme(self) -> str:
        return SCHEMES.get((self.M, self.B, self.g), f"{self.M}x{self.B}g{self.g}")

    @property
    def general(self) -> bool:
        """True when the scheme runs the library's general kernels."""
        return (self.M, self.B, self.g) not in SCHEMES

    def _check_x(self, x: torch.Tensor) -> torch.Tensor:
        if x.dim() != 2 or x.shape[1] != self.in_features:
            raise ValueError(f"x must be [batch, {self.in_features}]")
        if x.dtype != torch.float16 or not x.is_contiguous() or x.device != self.device:
            raise ValueError("x must be a contiguous float16 tensor on the layer's device")
        return x

    def dequant(self, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        lib = load_library()
        if out is None:
            out = torch.empty((self.out_features, self.in_features), dtype=torch.float16,
                              device=self.device)
        elif (out.shape != (self.out_features, self.in_features) or out.dtype != torch.float16
              or not out.is_contiguous() or out.device != self.device):
            raise ValueError("out must be a contiguous float16 [out, in] tensor on the device")
        with torch.cuda.device(self.device):
            _check(lib.aqlm_dequant(ctypes.byref(self._struct), out.data_ptr(),
                                    _stream_handle(self.device)))
        return out

    def _product(self, fn_name: str, x: torch.Tensor, out: Optional[torch.Tensor]) -> torch.Tensor:
        lib = load_library()
        x = self._check_x(x)
        batch = x.shape[0]
        if out is None:
            out = torch.empty((batch, self.out_features), dtype=torch.float16, device=self.device)
        elif (out.shape != (batch, self.out_features) or out.dtype != torch.float16
              or not out.is_contiguous() or out.device != self.device):
            raise ValueError("out must be a contiguous float16 [batch, out] tensor on the device")
        with torch.cuda.device(self.device):
            _check(getattr(lib, fn_name)(ctypes.byref(self._struct), x.data_ptr(), batch,
                                         out.data_ptr(), _stream_handle(self.device)))
        return out

    def gemv(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
             workspace: bool = True) -> torch.Tensor:
        """y = x . W^T for 1..8 activation rows (codebook-lookup path).

        With workspace=True (the default) the call goes through aqlm_gemv_ws
        with a workspace taken from torch's allocator on the current stream
        (used by the codebook-sliced 1x16 kernel at one row); workspace=False
        calls aqlm_gemv, which needs none.
        """
        if not workspace:
            return self._product("aqlm_gemv", x, out)
        return gemv_batched([self], [x], None if out is None else [out])[0]

    def workspace_bytes(self, batch: int) -> int:
        """Device workspace aqlm_gemm_ws needs for this batch (0: none)."""
        n = ctypes.c_int64(0)
        _check(load_library().aqlm_gemm_workspace_size(ctypes.byref(self._struct), int(batch),
                                                       ctypes.byref(n)))
        return n.value

    def gemm(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
             workspace: bool = True) -> torch.Tensor:
        """y = x . W^T for any number of activation rows (matrix-core path).

        With workspace=True (the default) the call goes through aqlm_gemm_ws
        with a workspace taken from torch's allocator on the current stream;
        workspace=False calls aqlm_gemm, which needs none.
        """
        if not workspace:
            return self._product("aqlm_gemm", x, out)
        lib = load_library()
        x = self._check_x(x)
        batch = x.shape[0]
        if out is None:
            out = torch.empty((batch, self.out_features), dtype=torch.float16, device=self.device)
        elif (out.shape != (batch, self.out_features) or out.dtype != torch.float16
              or not out.is_contiguous() or out.device != self.device):
            raise ValueError("out must be a contiguous float16 [batch, out] tensor on the device")
        need = self.workspace_bytes(batch)
        ws = torch.empty(need, dtype=torch.uint8, device=self.device) if need else None
        with torch.cuda.device(self.device):
            _check(lib.aqlm_gemm_ws(ctypes.byref(self._struct), x.data_ptr(), batch,
                                    out.data_ptr(), ws.data_ptr() if ws is not None else None,
                                    need, _stream_handle(self.device)))
        return out

    def gemm_noalloc(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The product of gemm() (aqlm_gemm_ws's kernels and bits) through
        aqlm_gemm_noalloc, whose scratch memory is the library's static device
        array: the call allocates nothing on the device (pass `out` to keep
        the output allocation out of it too). Calls on one GPU that overlap in
        time race on that array."""
        return self._product("aqlm_gemm_noalloc", x, out)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        """Pick the lookup path for <= 8 rows and the matrix-core path above."""
        return self.gemv(x) if x.shape[0] <= 8 else self.gemm(x)


def gemv_batched(layers, xs, outs=None, workspace: bool = True):
    """y_i = x_i . W_i^T for several layers in one call.

    layers: sequence of AqlmLayer; xs: sequence of [batch, in_i] float16 tensors
    (one per layer, all with the same batch, may repeat); outs: optional
    preallocated [batch, out_i] tensors. Returns the list of outputs. With
    workspace=True (the default) the call is aqlm_gemv_ws with a workspace
    from torch's allocator on the current stream; workspace=False calls
    aqlm_gemv_batched.
    """
    lib = load_library()
    n = len(layers)
    if len(xs) != n or (outs is not None and len(outs) != n):
        raise ValueError("one x (and one out) per layer")
    if n == 0:
        return []
    batch = xs[0].shape[0]
    device = layers[0].device
    ys = []
    for i, (L, x) in enumerate(zip(layers, xs)):
        x = L._check_x(x)
        if x.shape[0] != batch or L.device != device:
            raise ValueError("all layers share the batch size and the device")
        if outs is None:
            ys.append(torch.empty((batch, L.out_features), dtype=torch.float16, device=device))
        else:
            o = outs[i]
            if (o.shape != (batch, L.out_features) or o.dtype != torch.float16
                    or not o.is_contiguous() or o.device != device):
                raise ValueError("out tensors must be contiguous float16 [batch, out] on the device")
            ys.append(o)
    structs = (AqlmLayerStruct * n)(*[L._struct for L in layers])
    xp = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    yp = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    with torch.cuda.device(device):
        if not workspace:
            _check(lib.aqlm_gemv_batched(structs, xp, yp, n, batch, _stream_handle(device)))
            return ys
        need = ctypes.c_int64(0)
        _check(lib.aqlm_gemv_workspace_size(structs, n, batch, ctypes.byref(need)))
        ws = torch.empty(need.value, dtype=torch.uint8, device=device) if need.value else None
        _check(lib.aqlm_gemv_ws(structs, xp, yp, n, batch,
                                ws.data_ptr() if ws is not None else None, need.value,
                                _stream_handle(device)))
    return ys


def gemv_workspace_bytes(layers, batch: int) -> int:
    """Device workspace aqlm_gemv_ws needs for these layers at this batch (0: none)."""
    n = len(layers)
    structs = (AqlmLayerStruct * n)(*[L._struct for L in layers])
    need = ctypes.c_int64(0)
    _check(load_library().aqlm_gemv_workspace_size(structs, n, int(batch), ctypes.byref(need)))
    return need.value


def raw_call(fn_name: str, struct: AqlmLayerStruct, *args) -> int:
    """Call an entry point with a hand-built descriptor (for boundary tests)."""
    lib = load_library()
    return getattr(lib, fn_name)(ctypes.byref(struct), *args)
