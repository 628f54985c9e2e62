"""GPU parity of the grouped output projection (grouped_out_proj) against the
oracle's float64 product: the decode shape (4 queries, 8 groups of 8 heads x
512 dims into 1024 features each), many ragged rows, odd widths (the K tail),
a K split over 8 waves, strided inputs and outputs, bf16 and float32 outputs."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import codecs
from oracle import projection as OP
from tests._common import bf16_ulp, np_

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_hca_amd as H
    return H


def _f64(t):
    return codecs.decode_bf16(np_(t.view(torch.int16)).view(np.uint16))


@pytest.mark.parametrize("n,G,K,N,extra_x,extra_y,ydt", [
    (4, 8, 4096, 1024, 0, 0, "bf16"),        # decode: o [4, 64, 512] -> 8 groups of 4096 -> 1024
    (4, 8, 4096, 1024, 0, 0, "f32"),
    (300, 4, 512, 256, 64, 16, "bf16"),      # many rows (ragged last 128-row block): LDS-tiled blocks
    (270, 2, 64, 192, 0, 0, "f32"),          # many rows, features not a multiple of 128: 4 x 4 tiles per wave
    (37, 3, 96, 48, 8, 3, "f32"),            # odd widths: K tail steps, one 16-wide tile per wave
    (1, 1, 4096, 16, 0, 0, "f32"),           # one tile: K split over 8 waves
])
def test_grouped_projection_vs_oracle(H, n, G, K, N, extra_x, extra_y, ydt):
    print(f"grouped projection n={n} G={G} K={K} N={N} y={ydt}", flush=True)
    sys.stdout.flush()
    g = synth.generator(1019)
    xf = synth.normal(g, (n, G * K + extra_x))
    wf = synth.normal(g, (G, N, K), std=K ** -0.5)
    x = xf.to(torch.bfloat16).cuda()
    w = wf.to(torch.bfloat16).cuda()
    dt = torch.bfloat16 if ydt == "bf16" else torch.float32
    ybuf = torch.full((n, G * N + extra_y), float("nan"), dtype=dt, device="cuda")
    y = ybuf[:, :G * N]
    H.grouped_out_proj(x, w, y)
    y2 = torch.empty_like(ybuf)[:, :G * N]
    H.grouped_out_proj(x, w, y2)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "not deterministic"
    if extra_y:
        assert bool(torch.isnan(ybuf[:, G * N:].float()).all()), "wrote past the output row"
    xd, wd = _f64(x.cpu()), _f64(w.cpu())
    ref = OP.grouped_projection(xd[:, :G * K], wd)
    mag = OP.grouped_projection(np.abs(xd[:, :G * K]), np.abs(wd))
    got = y.float().double().cpu().numpy()
    # float32 accumulation of K products in any order, then the output's own rounding
    bound = 2.0 ** -17 * mag + (bf16_ulp(ref) if ydt == "bf16" else 2.0 ** -24 * np.abs(ref))
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err {err.max():.3e}, {np.count_nonzero(err > bound)} beyond the bound"
