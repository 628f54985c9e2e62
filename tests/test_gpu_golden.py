"""The GPU library against the stored oracle results of the tiny fp32 case (tests/golden/):
compressed entries, top-k sets and attention, at the fp32 tolerances."""
import importlib.util
import json
import os

import numpy as np
import pytest
import torch

from tests._common import check_attention, check_idx, np_

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_gpu_matches_golden_fixture():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_attention_hca_amd import workloads as W
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    with open(mk.PATH) as f:
        ref = json.load(f)
    mk.PARAMS.update(ref["params"])
    c = mk.case()
    c.t = {k: v.to("cuda") for k, v in c.t.items()}
    got = W.tiny_fp32(c)
    torch.cuda.synchronize()
    csa = np_(got["csa"].data).astype(np.float64)
    hca = np_(got["hca"].data).astype(np.float64)
    yc, yh = np.asarray(ref["csa_entries_first4"]), np.asarray(ref["hca_entries_first2"])
    assert np.abs(csa[:4] - yc).max() <= 1e-5 * max(1.0, np.abs(yc).max())
    assert np.abs(hca[:2] - yh).max() <= 1e-5 * max(1.0, np.abs(yh).max())
    check_idx(np_(got["idx"]), np.asarray(ref["idx"]), "golden top-k")
    check_attention(np_(got["o_csa"]), np_(got["lse_csa"]), np.asarray(ref["o_csa"]), np.asarray(ref["lse_csa"]),
                    "fp32", "golden csa")
    check_attention(np_(got["o_hca"]), np_(got["lse_hca"]), np.asarray(ref["o_hca"]), np.asarray(ref["lse_hca"]),
                    "fp32", "golden hca")
