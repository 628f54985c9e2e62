"""Pins of the oracle's chunked-prefill query (DeepSeek-V4 page, Method section: CSA and HCA
paragraphs, with the sliding-window branch).

split_window=True lets attention see each raw window row after the oracle's own split-layout
encoding (FP8 E4M3 non-RoPE dims with a power-of-two row scale, bf16 RoPE dims). When every
raw row is exactly representable in that layout the option must change nothing, bit for bit;
when it is not, the outputs must differ, and only through the window rows."""
import numpy as np
import torch

import synth
from oracle import codecs
from oracle import compress as OC
from oracle import pipeline as OP
from tests._common import case_numpy


def _case(exact):
    c = synth.chunked_prefill(seed=1205, prefixes=(128, 256, 384), chunk=128, device="cpu")
    if exact:
        # entries +-1/2, +-1, +-2 and 0: exact in bf16 and, under any power-of-two row scale that
        # keeps the row maximum within E4M3's range, exact in E4M3 too
        g = torch.Generator().manual_seed(7)
        vals = torch.tensor([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0])
        pick = torch.randint(0, len(vals), c.t["raw"].shape, generator=g)
        c.t["raw"] = synth.bf16_bits(vals[pick])
    return c


def _queries(c, split):
    p = c.params
    a = case_numpy(c)
    ent = {b: OP.prefill_chunk_entries(p, a, b) for b in range(p["S"])}
    picks = [0, 63, 127, 128, 200, 300, 383]
    return [OP.prefill_query(p, a, qi, lambda b: ent[b][1], lambda b: ent[b][3], split_window=split) for qi in picks]


def test_exactly_representable_window_rows_are_unchanged():
    c = _case(exact=True)
    raw = codecs.decode_bf16(case_numpy(c, keys={"raw"})["raw"])
    dn, dr = c.params["d_nope"], c.params["d_rope"]
    assert np.array_equal(OC.decode(OC.encode(raw, "split", dn, dr), "split"), raw)
    for r0, r1 in zip(_queries(c, False), _queries(c, True)):
        for k in ("idx", "o_csa", "lse_csa", "o_hca", "lse_hca"):
            assert np.array_equal(r0[k], r1[k]), k


def test_general_window_rows_change_attention_only():
    c = _case(exact=False)
    changed = False
    for r0, r1 in zip(_queries(c, False), _queries(c, True)):
        assert np.array_equal(r0["idx"], r1["idx"])  # the indexer never reads the window
        changed = changed or not np.array_equal(r0["o_hca"], r1["o_hca"])
        # FP8 rounding of the window rows moves the output by far less than its scale
        for k in ("o_csa", "o_hca"):
            assert np.max(np.abs(r0[k] - r1[k])) <= 0.1 * np.max(np.abs(r0[k])), k
    assert changed
