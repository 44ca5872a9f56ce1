"""The numpy rendering of the K-blocked weight layout used by the GPU pack test,
checked element by element against the layout's definition in moe_rocm.h
(tile t, step s, tile row r, element e of the step: source row per the SwiGLU
pairing, chunk c = slot ^ swizzle(r) of the step, slot = e // per-chunk)."""

import numpy as np
import pytest

from tests.test_gpu_blocked import pack_ref


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("swiglu_i", [0, 256])
def test_pack_ref_matches_definition(fp8, swiglu_i):
    rng = np.random.default_rng(3 + int(fp8) + swiglu_i)
    dt = np.uint8 if fp8 else np.uint16
    step, per = (64, 16) if fp8 else (32, 8)
    n, rows, K = 2, 512, 256
    w = rng.integers(0, 200, size=(n, rows, K)).astype(dt)
    out = pack_ref(w, swiglu_i, fp8)
    assert out.shape == (n, rows // 256, K // step, 256, step)
    for _ in range(3000):
        m, t, s, r, e = (int(rng.integers(x)) for x in (n, rows // 256, K // step, 256, step))
        swz = (r >> 2) & 3
        c = (e // per) ^ swz
        if swiglu_i:
            srow = t * 128 + r if r < 128 else swiglu_i + t * 128 + (r - 128)
        else:
            srow = t * 256 + r
        assert out[m, t, s, r, e] == w[m, srow, s * step + c * per + e % per]
    # a permutation of the source: every element appears once
    assert np.array_equal(np.sort(out.reshape(-1)), np.sort(w.reshape(-1)))
