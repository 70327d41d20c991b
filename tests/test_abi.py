"""The C-ABI library on the host: it loads, exports every declared entry point,
and rejects bad arguments before anything is launched (no GPU needed: every
call here fails validation or is a batch == 0 no-op, so no kernel starts)."""
import ctypes
import os
import re

import pytest

from additive_codebook_matmul_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aqlm.h")

FAKE = 0x10000      # a 16-byte aligned address that is never dereferenced
MISALIGNED = 0x10008


def _declared_functions(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"AQLM_API\s+[\w\s\*]*?\b(aqlm_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared_functions() == sorted(_lib.EXPORTED_SYMBOLS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = _lib.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.aqlm_abi_version() == _lib.ABI_VERSION


def test_host_library_exports_every_declared_symbol():
    from additive_codebook_matmul_amd import host
    if not os.path.exists(host.HOST_LIB_PATH):
        from additive_codebook_matmul_amd.build import build_host_library
        build_host_library(verbose=False)
    declared = _declared_functions(os.path.join(ROOT, "include", "aqlm_host.h"))
    assert declared == sorted(host.HOST_EXPORTED_SYMBOLS)
    lib = host.load_host_library()
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layout_matches_header():
    # int64, int64, 4 x int32, 3 pointers
    assert ctypes.sizeof(_lib.AqlmLayerStruct) == 8 + 8 + 16 + 3 * 8
    assert _lib.AqlmLayerStruct.codes.offset == 32


def test_status_strings():
    for st in range(9):
        assert _lib.status_string(st) != "unknown status"
    assert _lib.status_string(99) == "unknown status"
    assert _lib.status_string(0) == "ok"


def _layer(M=2, B=8, g=8, out=64, n_in=128, codes=FAKE, books=FAKE, scales=FAKE, flags=0):
    return _lib.AqlmLayerStruct(out, n_in, M, B, g, flags, codes, books, scales)


ENTRY = {
    "aqlm_dequant": lambda s, x, b, y: _lib.raw_call("aqlm_dequant", s, y, None),
    "aqlm_gemv": lambda s, x, b, y: _lib.raw_call("aqlm_gemv", s, x, b, y, None),
    "aqlm_gemm": lambda s, x, b, y: _lib.raw_call("aqlm_gemm", s, x, b, y, None),
    "aqlm_gemm_ws": lambda s, x, b, y: _lib.raw_call("aqlm_gemm_ws", s, x, b, y, FAKE, 1 << 40,
                                                     None),
    "aqlm_gemm_noalloc": lambda s, x, b, y: _lib.raw_call("aqlm_gemm_noalloc", s, x, b, y, None),
}


@pytest.mark.parametrize("fn", sorted(ENTRY))
def test_null_layer_pointer(fn):
    lib = _lib.load_library()
    f = getattr(lib, fn)
    if fn == "aqlm_dequant":
        assert f(None, FAKE, None) == 1
    elif fn == "aqlm_gemm_ws":
        assert f(None, FAKE, 1, FAKE, FAKE, 1 << 40, None) == 1
    else:
        assert f(None, FAKE, 1, FAKE, None) == 1


@pytest.mark.parametrize("fn", sorted(ENTRY))
@pytest.mark.parametrize("case,status", [
    (dict(codes=0), 1), (dict(books=0), 1), (dict(scales=0), 1),
    (dict(M=0), 3), (dict(M=9), 3), (dict(B=7), 3), (dict(B=17), 3), (dict(g=4), 3),
    (dict(g=32), 3), (dict(M=-1), 3),
    (dict(out=0), 2), (dict(n_in=0), 2), (dict(n_in=100), 2), (dict(out=-5), 2),
    (dict(flags=2), 2), (dict(flags=-1), 2), (dict(out=1 << 40), 2),
    (dict(M=1, B=16, g=16, n_in=136), 2),
    (dict(codes=MISALIGNED), 4), (dict(books=MISALIGNED), 4), (dict(scales=MISALIGNED), 4),
])
def test_layer_validation(fn, case, status):
    s = _layer(**case)
    assert ENTRY[fn](s, FAKE, 1, FAKE) == status


@pytest.mark.parametrize("fn", sorted(ENTRY))
def test_output_pointer_validation(fn):
    s = _layer()
    assert ENTRY[fn](s, FAKE, 1, 0) == 1
    assert ENTRY[fn](s, FAKE, 1, MISALIGNED) == 4


@pytest.mark.parametrize("fn", ["aqlm_gemv", "aqlm_gemm", "aqlm_gemm_ws", "aqlm_gemm_noalloc"])
def test_input_pointer_and_batch_validation(fn):
    s = _layer()
    assert ENTRY[fn](s, 0, 1, FAKE) == 1
    assert ENTRY[fn](s, MISALIGNED, 1, FAKE) == 4
    assert ENTRY[fn](s, FAKE, -1, FAKE) == 5
    # batch == 0 is a no-op that launches nothing, even with unusable pointers
    assert ENTRY[fn](s, 0, 0, 0) == 0


def test_batch_limits():
    s = _layer()
    assert ENTRY["aqlm_gemv"](s, FAKE, 9, FAKE) == 5
    assert ENTRY["aqlm_gemm"](s, FAKE, 1 << 40, FAKE) == 5
    assert ENTRY["aqlm_gemm_ws"](s, FAKE, 1 << 40, FAKE) == 5
    assert ENTRY["aqlm_gemm_noalloc"](s, FAKE, 1 << 40, FAKE) == 5


def _ws_size(s, batch):
    n = ctypes.c_int64(-1)
    st = _lib.load_library().aqlm_gemm_workspace_size(ctypes.byref(s), batch, ctypes.byref(n))
    return st, n.value


def test_workspace_size():
    """Host-side sizing: the workspace form covers the three dedicated schemes
    (element or bit-packed codes) with in/g a multiple of 8 from 17 rows to
    128, and above that wherever its workspace stays within 64 MiB and its
    timing model beats the decoded-tile kernel that aqlm_gemm would run; it
    then holds at least the re-laid activations (in x 16*ceil(batch/16)
    float16 values). At 1..16 rows it reads x in place and needs none."""
    mlp = dict(out=4096, n_in=11008)
    for M, B, g in ((2, 8, 8), (1, 16, 8), (1, 16, 16)):
        for batch in (17, 33, 64, 100, 128):
            st, n = _ws_size(_layer(M, B, g, **mlp), batch)
            bp = 16 * min(8, {5: 6, 7: 8}.get((batch + 15) // 16, (batch + 15) // 16))
            assert st == 0 and n >= 11008 * bp * 2, (M, B, g, batch, n)
            assert n % 16 == 0
    assert _ws_size(_layer(**mlp), 0) == (0, 0)
    assert _ws_size(_layer(**mlp), 16) == (0, 0)                     # K split: skinny tiles
    assert _ws_size(_layer(out=11008, n_in=4096), 1) == (0, 0)      # one tile, x read in place
    assert _ws_size(_layer(out=11008, n_in=4096), 17)[1] > 0         # re-laid activations
    assert _ws_size(_layer(out=300, n_in=1024), 8) == (0, 0)         # few row blocks: skinny
    assert _ws_size(_layer(**mlp), 129)[1] > 0                       # two blocks of 128 rows
    assert _ws_size(_layer(**mlp), 1024)[1] >= 11008 * 1024 * 2      # 8 blocks of 128 rows
    assert _ws_size(_layer(**mlp), 4096) == (0, 0)                   # would pass 64 MiB
    up = dict(out=11008, n_in=4096)
    assert _ws_size(_layer(**up), 1024)[1] >= 4096 * 1024 * 2        # modelled 141 us, tile 150
    assert _ws_size(_layer(**up), 2048) == (0, 0)                    # modelled 259 us, tile 247
    assert _ws_size(_layer(1, 16, 8, **up), 200) == (0, 0)           # 1x16: the tile kernel
    assert _ws_size(_layer(1, 16, 8, **mlp), 200)[1] > 0             # 32 tiles: this form
    assert _ws_size(_layer(3, 8, 8, **mlp), 64) == (0, 0)            # general scheme
    assert _ws_size(_layer(flags=1, **mlp), 64) == _ws_size(_layer(**mlp), 64)  # same bytes
    assert _ws_size(_layer(3, 8, 8, flags=1, **mlp), 64) == (0, 0)   # general, bit-packed
    assert _ws_size(_layer(out=64, n_in=36 * 8), 64) == (0, 0)       # in/g not a multiple of 8
    assert _ws_size(_layer(codes=0, **mlp), 64) == (1, 0)
    assert _ws_size(_layer(**mlp), -1) == (5, 0)
    assert _lib.load_library().aqlm_gemm_workspace_size(ctypes.byref(_layer()), 1, None) == 1


def test_workspace_validation():
    """Errors of aqlm_gemm_ws that stop the call before any launch."""
    s = _layer(out=4096, n_in=11008)
    st, need = _ws_size(s, 64)
    assert st == 0 and need > 0
    f = _lib.load_library().aqlm_gemm_ws
    assert f(ctypes.byref(s), FAKE, 64, FAKE, None, need, None) == 1
    assert f(ctypes.byref(s), FAKE, 64, FAKE, MISALIGNED, need, None) == 4
    assert f(ctypes.byref(s), FAKE, 64, FAKE, FAKE, need - 1, None) == 7
    assert f(ctypes.byref(s), FAKE, 0, FAKE, None, 0, None) == 0     # batch 0: no-op


def test_noalloc_rejects_calls_beyond_the_static_scratch():
    """aqlm_gemm_noalloc returns AQLM_ERR_SCRATCH, before any launch, when the
    workspace form would need more than the static scratch array holds."""
    f = _lib.load_library().aqlm_gemm_noalloc
    big = None
    for out, n_in in ((1024, 1 << 18), (1024, 1 << 19)):
        for batch in (100, 128):
            s = _layer(out=out, n_in=n_in)
            st, need = _ws_size(s, batch)
            if st == 0 and need > _lib.STATIC_SCRATCH_BYTES:
                big = (s, batch)
                break
        if big:
            break
    assert big is not None, "no shape needs more than the static scratch"
    s, batch = big
    assert f(ctypes.byref(s), FAKE, batch, FAKE, None) == 8
    assert "64 MiB" in _lib.status_string(8)


def test_binding_rejects_cpu_tensors_without_calling_the_library():
    import torch
    codes = torch.zeros((4, 2, 2), dtype=torch.uint8)
    books = torch.zeros((2, 256, 8), dtype=torch.float16)
    scales = torch.zeros(4, dtype=torch.float16)
    with pytest.raises(ValueError):
        _lib.AqlmLayer(codes, books, scales)
    with pytest.raises(ValueError):
        _lib.AqlmLayer(codes.to(torch.int16), books, scales)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        _lib.load_library()


def test_batched_validation():
    lib = _lib.load_library()
    n = 2
    structs = (_lib.AqlmLayerStruct * n)(_layer(), _layer(M=9))
    xs = (ctypes.c_void_p * n)(FAKE, FAKE)
    ys = (ctypes.c_void_p * n)(FAKE, FAKE + 0x1000)
    f = lib.aqlm_gemv_batched
    assert f(structs, xs, ys, -1, 1, None) == 2
    assert f(structs, xs, ys, 5000, 1, None) == 2
    assert f(structs, xs, ys, n, 9, None) == 5
    assert f(structs, xs, ys, n, -1, None) == 5
    assert f(None, xs, ys, n, 1, None) == 1
    assert f(structs, None, ys, n, 1, None) == 1
    # the second layer has an unsupported scheme: nothing launches
    assert f(structs, xs, ys, n, 1, None) == 3
    good = (_lib.AqlmLayerStruct * n)(_layer(), _layer())
    bad_y = (ctypes.c_void_p * n)(FAKE, MISALIGNED)
    assert f(good, xs, bad_y, n, 1, None) == 4
    null_x = (ctypes.c_void_p * n)(FAKE, 0)
    assert f(good, null_x, ys, n, 1, None) == 1
    # no-ops launch nothing
    assert f(good, xs, ys, 0, 1, None) == 0
    assert f(good, xs, ys, n, 0, None) == 0


def _gemv_ws_size(layers, batch):
    n = len(layers)
    arr = (_lib.AqlmLayerStruct * n)(*layers) if n else None
    v = ctypes.c_int64(-1)
    st = _lib.load_library().aqlm_gemv_workspace_size(arr, n, batch, ctypes.byref(v))
    return st, v.value


def test_gemv_workspace_size():
    """The codebook-sliced 1x16 kernel's workspace: 8 float32 sums per output
    row (rounded to 256 bytes) for 1x16 g8 layers at one activation row with
    in/8 a multiple of 8, at most 4096 groups and at least 2^19 codes, when
    those layers hold at least 2^22 codes together; none for anything else."""
    big = _layer(1, 16, 8, out=11008, n_in=4096)                         # 5.6 M codes
    assert _gemv_ws_size([big], 1) == (0, 8 * 11008 * 4)
    assert _gemv_ws_size([big], 2) == (0, 0)                              # batch 1 only
    q = _layer(1, 16, 8, out=4096, n_in=4096)                             # 2^21 codes
    assert _gemv_ws_size([q], 1) == (0, 0)                                # alone: too few
    assert _gemv_ws_size([q, q], 1) == (0, 2 * 8 * 4096 * 4)              # 2^22 together
    assert _gemv_ws_size([q, q, q], 1) == (0, 3 * 8 * 4096 * 4)
    assert _gemv_ws_size([_layer(2, 8, 8, out=11008, n_in=4096)], 1) == (0, 0)   # 2x8
    assert _gemv_ws_size([_layer(1, 16, 16, out=11008, n_in=8192)], 1) == (0, 0)  # g16
    small = _layer(1, 16, 8, out=100, n_in=4096)                          # below 2^19: never
    assert _gemv_ws_size([small, big], 1) == (0, 8 * 11008 * 4)
    assert _gemv_ws_size([_layer(1, 16, 8, out=8200, n_in=4096)], 1) == (0, (8 * 8200 * 4 + 255) // 256 * 256)
    assert _gemv_ws_size([_layer(1, 16, 8, out=16384, n_in=36 * 8 * 8 + 8)], 1) == (0, 0)  # in/8 % 8
    assert _gemv_ws_size([_layer(1, 16, 8, out=1200, n_in=28672)], 1)[1] > 0  # 7 chunks per row
    assert _gemv_ws_size([_layer(1, 16, 8, out=1200, n_in=40960)], 1) == (0, 0)  # > 4096 groups
    three = [big, _layer(2, 8, 8, out=4096, n_in=4096), q]
    assert _gemv_ws_size(three, 1) == (0, 8 * 11008 * 4 + 8 * 4096 * 4)
    assert _gemv_ws_size(three, 0) == (0, 0)
    assert _gemv_ws_size([], 1) == (0, 0)
    assert _gemv_ws_size([_layer(M=9)], 1) == (3, 0)
    assert _gemv_ws_size([big], 9) == (5, 0)
    assert _lib.load_library().aqlm_gemv_workspace_size(None, 1, 1, None) == 1


def test_gemv_ws_validation():
    """Errors of aqlm_gemv_ws that stop the call before any launch."""
    f = _lib.load_library().aqlm_gemv_ws
    one = (_lib.AqlmLayerStruct * 1)(_layer(1, 16, 8, out=11008, n_in=4096))
    xs = (ctypes.c_void_p * 1)(FAKE)
    ys = (ctypes.c_void_p * 1)(FAKE + 0x1000)
    need = 8 * 11008 * 4
    assert f(one, xs, ys, 1, 1, None, need, None) == 1
    assert f(one, xs, ys, 1, 1, MISALIGNED, need, None) == 4
    assert f(one, xs, ys, 1, 1, FAKE, need - 1, None) == 7
    assert f(one, xs, ys, 1, 9, FAKE, need, None) == 5
    assert f(one, None, ys, 1, 1, FAKE, need, None) == 1
    assert f(one, xs, ys, -1, 1, FAKE, need, None) == 2
    bad_y = (ctypes.c_void_p * 1)(MISALIGNED)
    assert f(one, xs, bad_y, 1, 1, FAKE, need, None) == 4
    assert f(one, xs, ys, 1, 0, None, 0, None) == 0   # batch 0: no-op
    assert f(one, xs, ys, 0, 1, None, 0, None) == 0   # no layers: no-op


@pytest.mark.parametrize("M,B,g", [(1, 8, 8), (3, 8, 8), (8, 8, 16), (1, 12, 8), (2, 12, 16),
                                   (2, 16, 8), (8, 16, 16), (4, 9, 8), (5, 15, 16)])
def test_general_schemes_accepted(M, B, g):
    """Every M in 1..8, B in 8..16, g in {8, 16} passes validation (batch 0 launches nothing)."""
    s = _layer(M=M, B=B, g=g, n_in=16 * g)
    for fn in ("aqlm_gemv", "aqlm_gemm"):
        assert ENTRY[fn](s, FAKE, 0, FAKE) == 0
    # the same descriptor with a bad pointer is still rejected before any launch
    assert ENTRY["aqlm_gemv"](_layer(M=M, B=B, g=g, n_in=16 * g, codes=MISALIGNED), FAKE, 1, FAKE) == 4


# ---------------------------------------------------------------------------
# toy encoder entry points (include/aqlm_encode.h): exported, and validated on
# the host before any launch
# ---------------------------------------------------------------------------
def test_encode_header_symbols_exported():
    from additive_codebook_matmul_amd import encode as ENC
    declared = _declared_functions(os.path.join(ROOT, "include", "aqlm_encode.h"))
    assert declared == sorted(ENC.ENCODE_SYMBOLS)
    lib = _lib.load_library()
    for name in declared:
        assert hasattr(lib, name), name


def test_encode_validation():
    from additive_codebook_matmul_amd import encode as ENC
    lib = ENC._lib()
    F, F2 = FAKE, FAKE + 0x100000
    # normalize(W, out, in, scales, vecs)
    assert lib.aqlm_encode_normalize(None, 4, 8, F, F2, None) == 1
    assert lib.aqlm_encode_normalize(F, 0, 8, F, F2, None) == 2
    assert lib.aqlm_encode_normalize(F, 4, 0, F, F2, None) == 2
    assert lib.aqlm_encode_normalize(MISALIGNED, 4, 8, F, F2, None) == 4
    # init(vecs, n, g, idx, K, cents)
    assert lib.aqlm_encode_init(F, 10, 8, None, 256, F2, None) == 1
    assert lib.aqlm_encode_init(F, 10, 12, F, 256, F2, None) == 3
    assert lib.aqlm_encode_init(F, 10, 8, F, 300, F2, None) == 3
    assert lib.aqlm_encode_init(F, 10, 8, F, 128, F2, None) == 3
    assert lib.aqlm_encode_init(F, 0, 8, F, 256, F2, None) == 2
    # assign(vecs, n, g, cents, K, codes, M, m, residual)
    assert lib.aqlm_encode_assign(F, 0, 8, F2, 256, F, 2, 0, None, None) == 0   # n == 0: no-op
    assert lib.aqlm_encode_assign(F, 10, 8, F2, 256, None, 2, 0, None, None) == 1
    assert lib.aqlm_encode_assign(F, 10, 8, F2, 256, F, 2, 2, None, None) == 2  # m >= M
    assert lib.aqlm_encode_assign(F, 10, 8, F2, 256, F, 9, 0, None, None) == 2
    assert lib.aqlm_encode_assign(F, 10, 8, F2, 1 << 17, F, 2, 0, None, None) == 3
    assert lib.aqlm_encode_assign(F, 10, 8, F2, 256, MISALIGNED, 2, 0, None, None) == 4
    assert lib.aqlm_encode_assign(F, 10, 8, F2, 256, F, 2, 0, F + 16, None) == 2  # partial overlap
    # update(vecs, n, g, codes, K, M, m, cents, ws)
    assert lib.aqlm_encode_update(F, 10, 8, F, 256, 2, 0, F2, None, None) == 1
    assert lib.aqlm_encode_update(F, 0, 8, F, 256, 2, 0, F2, F, None) == 2
    assert lib.aqlm_encode_update(F, 10, 16, F, 256, 2, 0, F2, MISALIGNED, None) == 4
    # round(cents, count, books, rounded)
    assert lib.aqlm_encode_round(F, 0, F2, None, None) == 0
    assert lib.aqlm_encode_round(None, 8, F2, None, None) == 1
    assert lib.aqlm_encode_round(F, -1, F2, None, None) == 2
