"""The seeded input generators: determinism, block independence, bf16 rounding."""

import numpy as np

import datagen


def test_blocks_are_independent_and_deterministic():
    w = datagen.Workload("t", 5, 2100, 16, 4, "normal", True)
    full = datagen.logits(w)
    again = datagen.logits(w, blocks=[2, 0])
    assert np.array_equal(again[:52], full[2048:])
    assert np.array_equal(again[52:], full[:1024])
    assert np.array_equal(datagen.row_ends(w), 16 - 2100 + np.arange(2100) + 1)


def test_specials_fractions():
    w = datagen.Workload("s", 104, 1024, 4000, 4, "specials", True)
    x = datagen.logits(w)
    n = x.size
    assert abs(np.isposinf(x).sum() / n - 0.001) < 0.0002
    assert abs(np.isneginf(x).sum() / n - 0.001) < 0.0002
    assert abs(np.isnan(x).sum() / n - 0.0005) < 0.0001


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.00390625, 1.01171875, -2.0, np.inf, -np.inf, np.finfo(np.float32).max, 0.0, -0.0],
                 np.float32)
    b = datagen.bf16_bits(f)
    # 1.00390625 = 0x3F808000 is a tie and rounds to even 0x3F80; 1.01171875 =
    # 0x3F818000 rounds up to 0x3F82; the largest finite fp32 rounds to +inf.
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x7F80, 0xFF80, 0x7F80, 0x0000, 0x8000]
    assert np.isnan(datagen.bf16_to_f32(datagen.bf16_bits(np.array([np.nan], np.float32))))[0]


def test_rank_slices():
    g = np.arange(2 * 24, dtype=np.float32).reshape(2, 24)
    s = datagen.rank_slices(g, 8)
    assert s.shape == (8, 2, 3)
    assert s[3, 1].tolist() == [27.0, 35.0, 43.0]


def test_robust_workloads_share_one_base():
    import numpy as np
    base = datagen.logits(datagen.WORKLOADS["robust"], blocks=[7])
    plus = datagen.logits(datagen.WORKLOADS["robust_plus100"], blocks=[7])
    scal = datagen.logits(datagen.WORKLOADS["robust_scale1e8"], blocks=[7])
    assert np.array_equal(plus, base + np.float32(100.0))
    assert np.array_equal(scal, base * np.float32(1e-8))
    ends = datagen.row_ends(datagen.WORKLOADS["robust"])
    assert ends[0] == 1 and ends[-1] == 8192
