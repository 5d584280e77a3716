"""The random-shape cases stay inside the library's documented limits and
build valid trees on the oracle (the GPU sweep runs them)."""
import numpy as np
import pytest

import oracle as O
import random_shapes as R


@pytest.mark.parametrize("case", range(R.N_CASES))
def test_case_within_limits(case):
    spec = R.random_spec(case)
    assert 1 <= spec["kmax"] <= 127
    assert 0 <= spec["n_draft"] <= R.MAX_DRAFT
    assert all(0 <= k <= spec["kmax"] for k in spec["stage_k_ret"])
    assert spec["Hq"] % spec["Hkv"] == 0 and spec["D"] in (64, 128)
    assert spec["B"] * (spec["kmax"] + 1) * spec["Hq"] <= R.MAX_ROWS or spec["B"] == 1
    w = R.make_case(case)
    tree = O.build_tree(w.cfg, w.draft_parent, w.draft_token, w.draft_conf, w.n_draft,
                        w.root_token, w.prefix_len, w.m_ids)
    n = tree["n_nodes"]
    assert ((n >= 1) & (n <= spec["kmax"] + 1)).all()
    assert (np.asarray(w.prefix_len) == np.asarray(spec["prefix_list"])).all()
