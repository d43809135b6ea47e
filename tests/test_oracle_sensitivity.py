"""The sharp cases the GPU encode tests use can tell the pool and the rotary apart.

For each case of tests/sharp_cases.py the oracle is run as written and with one step
ablated: the pool replaced by the mean pool (a zero pool query, the uniform-attention
special case of the "UForm" page's FAQ on attention vs mean pooling), or the rotary
coordinates wired wrongly (all zero, two axes exchanged, axes rotated; "One Omni Model":
1-D, 2-D and 3-D coordinates). Each ablated output must miss the GPU bar of its test by
at least ten times, so a GPU path with that mistake cannot pass.
"""
import numpy as np
import pytest

import oracle
from tests import sharp_cases as S
from tests.gpu_util import ABS_MAX


@pytest.mark.parametrize("kind", ["text", "image", "video"])
def test_mean_pool_misses_the_pooled_bar_tenfold(kind):
    w, batch = S.pool_case(kind)
    x0, pos, cu = S.frontend(w, batch)
    pooled = oracle.forward(w, x0, pos, cu)
    mean = oracle.forward(S.mean_pool_weights(w), x0, pos, cu)
    d = np.abs(mean - pooled).max()
    print(f"{kind}: mean pool vs attention pool max |diff| {d:.3e} = {d / ABS_MAX:.1f} x the bar")
    assert d >= 10 * ABS_MAX


@pytest.mark.parametrize("kind", ["text", "image", "video"])
def test_wrong_rotary_coordinates_miss_the_trace_bar_tenfold(kind):
    w, batch = S.rotary_case(kind)
    x0, pos, cu = S.frontend(w, batch)
    ref = S.residual_trace(w, x0, pos, cu)[-1]
    for name, p in S.position_ablations(kind, pos).items():
        alt = S.residual_trace(w, x0, p, cu)[-1]
        rel = np.linalg.norm(alt - ref) / np.linalg.norm(ref)
        print(f"{kind}: {name}: residual after block 2 moves by {rel:.3f} = {rel / S.TRACE_REL:.1f} x the bar")
        assert rel >= 10 * S.TRACE_REL, name
