"""Seeded generators: determinism and the stated recipe (CPU only)."""
import numpy as np
import torch

import datagen
from oracle import formats as F


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(10000) * np.exp(rng.uniform(-20, 20, 10000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(datagen.f32_to_bf16_bits(x), ref)


def test_config1_recipe_and_determinism():
    w, x = datagen.config1()
    w2, x2 = datagen.config1()
    assert np.array_equal(w, w2) and np.array_equal(x, x2)
    assert w.shape == (64, 256) and x.shape == (512, 256)
    wv = F.bf16_bits_to_f64(w)
    assert (np.abs(wv) > 0.2).sum() >= 100          # the x20 outliers
    xv = F.bf16_bits_to_f64(x)
    rms = np.sqrt((xv ** 2).mean(axis=0))
    assert set(np.argsort(rms)[-2:]) == {7, 130}


def test_config5_forced_blocks_out_of_window():
    p, e8, forced = datagen.config5(experts=2, rows=8, k=256, forced_frac=0.1)
    assert p.shape == (2, 2, 8, 128) and e8.shape == (2, 2, 8, 8)
    for g in range(2):
        k = e8[g].astype(int) - 127
        out = (k.max() - k) > 17
        assert np.array_equal(out, forced[g])
