"""aqlm_gemm_noalloc: the workspace product with the library's static scratch.

Called through the C-ABI and compared bit for bit with aqlm_gemm_ws (the same
kernels, the workspace from torch), and with the oracle at the product
tolerance, over consecutive calls whose inputs shrink: the scratch keeps the
previous call's contents, which no call may read.
"""
import numpy as np
import pytest
import torch

import oracle
from additive_codebook_matmul_amd import _lib, workloads as WL
from gpu_util import assert_product, bits, dev_layer, dev_x, device

pytestmark = pytest.mark.gpu

SCHEMES = {"2x8": WL.S2x8, "1x16": WL.S1x16, "1x16g16": WL.S1x16g16}


def _noalloc(layer, x, batch):
    y = torch.empty((batch, layer.out_features), dtype=torch.float16, device=device())
    st = _lib.raw_call("aqlm_gemm_noalloc", layer._struct, x.data_ptr(), batch, y.data_ptr(),
                       None)
    assert st == 0, _lib.status_string(st)
    torch.cuda.synchronize()
    return y


def _ws(layer, x, batch):
    need = layer.workspace_bytes(batch)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device())
    y = torch.empty((batch, layer.out_features), dtype=torch.float16, device=device())
    st = _lib.raw_call("aqlm_gemm_ws", layer._struct, x.data_ptr(), batch, y.data_ptr(),
                       ws.data_ptr(), need, None)
    assert st == 0, _lib.status_string(st)
    torch.cuda.synchronize()
    return y, need


# (scheme, out, in, batch): a split-K call with re-laid activations first, then
# smaller ones: fewer activation rows, another scheme, a call needing no scratch
CALLS = [("2x8", 4096, 11008, 128), ("1x16g16", 1000, 4096, 40), ("2x8", 4096, 11008, 33),
         ("1x16", 2000, 2048, 17), ("2x8", 300, 1024, 8)]


def test_noalloc_matches_workspace_form_over_consecutive_calls():
    needs = []
    for i, (sname, out, n_in, batch) in enumerate(CALLS):
        s = SCHEMES[sname]
        codes, books, scales, x = WL.small_case(out, n_in, s, batch, seed=100 + i)
        layer = dev_layer(codes, books, scales)
        xd = dev_x(x)
        y0, need = _ws(layer, xd, batch)
        assert need <= _lib.STATIC_SCRATCH_BYTES
        needs.append(need)
        y1 = _noalloc(layer, xd, batch)
        assert np.array_equal(bits(y1), bits(y0)), (sname, out, n_in, batch)
        rows = np.unique(np.concatenate([[0, out - 1],
                                         np.random.default_rng(i).choice(out, min(out, 256),
                                                                         replace=False)]))
        y_ref, bound = oracle.forward_rows(x, codes, books, scales, rows)
        assert_product(y1.cpu().numpy()[:, rows], y_ref, bound,
                       f"noalloc {sname} {out}x{n_in} b{batch}")
    # the sequence went from a large scratch need to smaller ones and to none
    assert needs[0] > needs[1] > 0 and needs[0] > needs[2] > 0 and needs[-1] == 0


def test_noalloc_repeated_call_same_bits():
    s = SCHEMES["1x16g16"]
    codes, books, scales, x = WL.small_case(4096, 11008, s, 64, seed=7)
    layer = dev_layer(codes, books, scales)
    xd = dev_x(x)
    assert layer.workspace_bytes(64) > 0
    a = bits(_noalloc(layer, xd, 64))
    b = bits(_noalloc(layer, xd, 64))
    assert np.array_equal(a, b)
    assert np.array_equal(a, bits(layer.gemm_noalloc(xd)))
