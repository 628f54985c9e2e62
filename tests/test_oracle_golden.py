"""Regression pin of the oracle: recomputing the stored tiny fp32 case (tests/golden/, written
by tests/golden/make_golden.py from the oracle) must reproduce it exactly. The pages print no
worked example, so this guards the oracle against unintended change, not against the pages."""
import importlib.util
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_maker():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_oracle_reproduces_golden_fixture():
    mk = _load_maker()
    with open(mk.PATH) as f:
        stored = json.load(f)
    mk.PARAMS.update(stored["params"])
    got = mk.compute()
    assert got["idx"] == stored["idx"]
    for key in ("csa_entries_first4", "hca_entries_first2", "o_csa", "lse_csa", "o_hca", "lse_hca"):
        assert np.array_equal(np.asarray(got[key]), np.asarray(stored[key])), key
