"""GPU parity of the whole step on seeded random shapes.

Each case (tests/random_shapes.py) runs build, attention, accept, update and
the commit of the accepted path on the GPU and compares every output with
the oracle: bit-exact for trees, argmax, paths, M and the cache; attention
within 1e-2 (bf16) or 1e-4 (fp32) beyond the output's own rounding to its
storage type, with the plain max-abs error printed beside it.  The shapes
reach launch plans the named workloads do not: GQA groups 1 to 16, trees of
2 to 128 nodes, empty and edge-aligned prefixes, head dim 64 and 128 in
both dtypes.

Short prefixes give rows with a handful of visible keys, whose outputs come
close to single values of V (|out| up to about 3).  There the bf16 rounding
of the output alone is up to 2^-9 |out|, about 6e-3, and the probabilities
the P V product takes in bf16 add about as much again: an emulation with
exact scores, bf16 probabilities and a correctly rounded output reaches a
plain max-abs of 9.0e-3 on case 1.  So the plain 1e-2 bar is not asserted
here; the named workloads, whose long prefixes keep |out| small, assert it.
"""
import pytest

import random_shapes as R
from test_gpu_parity import run_full_check, run_update_tree_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", range(R.N_CASES))
def test_random_shape(case):
    run_full_check(R.make_case(case), raw_bar=False)


@pytest.mark.parametrize("case", range(2, R.N_CASES, 3))
def test_random_shape_update_tree(case):
    """The all-node update of M (every verified node's transition)."""
    run_update_tree_check(R.make_case(case))

