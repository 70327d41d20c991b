"""GPU parity of the batched product's routes above 128 activation rows.

With a workspace the call runs the workspace form (blocks of 128 activation
rows) unless aqlm_gemm would run the decoded-tile kernel and the library's
timing model gives that kernel the call, or the workspace would pass 64 MiB;
without one, aqlm_gemm runs the decoded-tile kernel (1x16 and 1x16 g16 from
129 rows, 2x8 from 512 rows on grids of at least 160 blocks) or the wide
tiles. Each case checks which route the workspace size announces, then the
outputs of sampled activation rows (first, last and seeded others) against
the oracle at the product tolerance; calls that need no workspace give the
bits of aqlm_gemm.
"""
import numpy as np
import pytest

import oracle
from additive_codebook_matmul_amd import workloads as WL
from gpu_util import assert_product, bits, dev_layer, dev_x

pytestmark = pytest.mark.gpu

SCHEMES = {"2x8": WL.S2x8, "1x16": WL.S1x16, "1x16g16": WL.S1x16g16}

# (scheme, out, in, batch, workspace form taken)
CASES = [("2x8", 11008, 4096, 640, True),      # 5 blocks of 128 rows (tile: 2 rounds)
         ("2x8", 4096, 11008, 1536, True),     # 12 blocks of 128 rows
         ("2x8", 11008, 4096, 2048, False),    # the decoded-tile kernel, 3 rounds
         ("1x16g16", 11008, 4096, 448, False),  # the decoded-tile kernel below 512 rows
         ("1x16g16", 4096, 11008, 576, True),
         ("1x16", 11008, 1024, 200, False),    # one ragged block of 256 rows
         ("1x16", 4096, 11008, 896, False)]


def _tokens(batch, n=64, seed=2):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, batch - 1], rng.choice(batch, n - 2, replace=False)]))


@pytest.mark.parametrize("scheme,out,n_in,batch,ws_form", CASES, ids=lambda v: str(v))
def test_route_matches_oracle(scheme, out, n_in, batch, ws_form):
    codes, books, scales, x = WL.small_case(out, n_in, SCHEMES[scheme], batch,
                                            seed=out + n_in + batch)
    L = dev_layer(codes, books, scales)
    assert (L.workspace_bytes(batch) > 0) == ws_form
    toks = _tokens(batch)
    y_ref, bound = oracle.forward(x[toks], codes, books, scales)
    xd = dev_x(x)
    y_ws = L.gemm(xd, workspace=True)
    y_plain = L.gemm(xd, workspace=False)
    assert_product(y_ws.cpu().numpy()[toks], y_ref, bound, f"gemm {scheme} {out}x{n_in} b{batch}")
    assert_product(y_plain.cpu().numpy()[toks], y_ref, bound,
                   f"gemm {scheme} {out}x{n_in} b{batch} no workspace")
    if not ws_form:
        assert np.array_equal(bits(y_ws), bits(y_plain))
