"""Properties of the seeded synthetic inputs (shared by oracle and GPU path)."""
import math

import numpy as np
import pytest

from lora_inputs import (CONFIGS, bf16_bits_of, gen_linear, gen_mlp, make_codebook,
                         to_bf16_values)


def test_codebook_properties():
    from scipy.special import ndtr
    cb = make_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[-1] == 1.0 and 0.0 in cb
    assert (cb > 0).sum() == 8 and (cb < 0).sum() == 7
    # the positive levels are normal quantiles at evenly spaced probabilities
    pos = cb[cb > 0].astype(np.float64)
    scale = 1.0 / pos.max()
    # undo the normalisation with the largest quantile, then check spacing
    p_max = 0.5 * ((1 - 1 / 32) + (1 - 1 / 30))
    from scipy.special import ndtri
    z = pos * ndtri(p_max)
    p = ndtr(z)
    assert np.allclose(np.diff(p), np.diff(p).mean(), atol=1e-6)


def test_inputs_are_exact_in_storage_dtype():
    li = gen_linear(32, 64, 48, 8, 16.0, "bf16")
    for a in (li.X, li.W, li.A, li.B, li.dY):
        assert a.dtype == np.float32
        assert np.array_equal(to_bf16_values(a), a)
    lf = gen_linear(32, 64, 48, 8, 16.0, "f32")
    assert not np.array_equal(to_bf16_values(lf.X), lf.X)


def test_inputs_are_seeded_and_distributed():
    a = gen_linear(256, 512, 512, 8, 16.0, "f32")
    b = gen_linear(256, 512, 512, 8, 16.0, "f32")
    assert np.array_equal(a.X, b.X) and np.array_equal(a.B, b.B)
    assert abs(a.X.std() - 1.0) < 0.01 and abs(a.W.std() - 0.02) < 0.001
    assert np.abs(a.A).max() <= 1 / math.sqrt(512)
    assert abs(a.A.std() - (1 / math.sqrt(512)) / math.sqrt(3)) < 1e-3
    c = gen_linear(256, 512, 512, 8, 16.0, "f32", seed=1)
    assert not np.array_equal(a.X, c.X)


def test_q4_inputs_layout():
    m = gen_mlp(4, 128, 256, 4, 16.0, "bf16", q4=True)
    q = m.q4["gate"]
    assert q.codes.shape == (256, 64) and q.codes.dtype == np.uint8
    assert q.absmax.shape == (256 * 128 // 64,) and (q.absmax >= 0).all()
    assert m.W["gate"] is None
    lo = q.codes & 15; hi = q.codes >> 4
    assert lo.max() == 15 and hi.max() == 15 and lo.min() == 0


def test_config_table():
    assert CONFIGS[3]["d"] == 4096 and CONFIGS[3]["f"] == 14336
    assert CONFIGS[1]["alpha"] / CONFIGS[1]["r"] == 2.0
    assert CONFIGS[4]["alpha"] / CONFIGS[4]["r"] == 0.25
