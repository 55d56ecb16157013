"""Host rules of the dispatch-table search: cost prior, residual regression, candidate choice, keep/revert."""

import math

import numpy as np
import pytest

from dense_gemm_transformer_amd import search as S


def _cfg(tm, tn, tk, wgs, split=1, launches=1, variant=S.VARIANT_TILED, threads=256, key=""):
    return S.Config(variant, tm, tn, tk, split, threads, wgs, launches, key or f"{tm}x{tn}x{tk}/{split}")


SQ = S.Shape(4096, 4096, 4096, "f32", "f32")


def test_floor_is_the_larger_roofline_term():
    assert SQ.floor_s() == pytest.approx(2 * 4096 ** 3 / 157.3e12)
    narrow = S.Shape(16, 4096, 4096, "f16", "f16")
    assert narrow.floor_s() == pytest.approx(2 * (16 * 4096 + 4096 * 4096 + 16 * 4096) / 8e12)
    assert S.efficiency(narrow, 2 * narrow.floor_s()) == pytest.approx(0.5)


def test_occupancy_follows_registers_and_lds():
    assert S.occupancy(SQ, _cfg(64, 64, 16, 4096)) == 4       # 16 accumulators per wave
    assert S.occupancy(SQ, _cfg(128, 128, 16, 1024)) == 2     # 64
    assert S.occupancy(SQ, _cfg(256, 256, 16, 256)) == 1      # 256
    bf = S.Shape(4096, 4096, 4096, "bf16", "f32")
    assert S.occupancy(bf, _cfg(128, 128, 128, 1024)) == 1    # 2·256·136·2 B = 136 KiB of LDS: one workgroup
    assert S.occupancy(bf, _cfg(128, 128, 64, 1024)) == 2     # 72 KiB: two
    assert S.occupancy(SQ, _cfg(16, 16, 4096, 256, variant=S.VARIANT_STREAM, threads=512)) == 1


def test_rounds_and_fill_have_a_knee_at_the_slot_count():
    full = S.features(SQ, _cfg(128, 128, 16, 256 * 2))        # exactly one round of 2 per CU
    assert (full.rounds, full.fill) == (1, 1.0)
    over = S.features(SQ, _cfg(128, 128, 16, 256 * 2 + 1))    # one workgroup more: a second, nearly empty round
    assert over.rounds == 2 and over.fill == pytest.approx((513 / 512) / 2)
    assert S.prior_s(SQ, over) > S.prior_s(SQ, full) * 1.9


def test_prior_is_monotone_and_prices_split_and_launches():
    base = _cfg(128, 128, 16, 1024)
    t = S.prior_s(SQ, S.features(SQ, base))
    assert t >= SQ.floor_s()
    big = S.Shape(4096, 4096, 8192, "f32", "f32")
    assert S.prior_s(big, S.features(big, base)) > t
    # a split doubles the workgroups and adds partial traffic and a reducer launch
    split = _cfg(128, 128, 16, 2048 + 4096 * 4096 // 1024, split=2, launches=2)
    f = S.features(SQ, split)
    assert f.extra_bytes == 2 * 4 * 4096 * 4096 * 2 and f.launches == 2
    assert S.main_workgroups(SQ, split) == 2048
    assert S.prior_s(SQ, f) > t


def test_regression_recovers_planted_coefficients_and_names_their_sign():
    rng = np.random.default_rng(1)
    beta = np.array([0.05, 0.0, 0.2, -0.3, -0.14, 0.1, 0.6, -0.05, 0.02])
    m = S.ResidualModel(ridge=1e-6)
    for _ in range(200):
        f = S.Features(occ=int(rng.choice([1, 2, 4])), rounds=int(rng.integers(1, 6)), fill=float(rng.uniform(0.2, 1)),
                       split=int(rng.choice([1, 2, 4, 8])), launches=int(rng.integers(1, 3)), l2_bytes=0.0,
                       extra_bytes=0.0, half=bool(rng.integers(0, 2)), slices=float(rng.choice([4, 12, 48, 256])),
                       tile_area=int(rng.choice([4096, 16384, 32768, 65536])))
        prior = 1e-4
        m.add(f, prior, prior * math.exp(f.vector() @ beta + rng.normal(0, 1e-3)))
    m.fit()
    assert np.allclose(m.beta, beta, atol=5e-3)
    rep = {name: (coef, verdict) for name, coef, verdict in m.report()}
    assert rep["log2 split"][1] == "model OVERprices"          # negative coefficient: measured faster than priced
    assert rep["extra rounds"][1] == "model UNDERprices"
    assert m.report()[0][0] == "16-bit operands"  # sorted by size
    # the fitted model's uncertainty is small inside the data and grows far outside it
    inside = S.Features(2, 2, 0.6, 2, 1, 0.0, 0.0)
    outside = S.Features(2, 60, 0.6, 2, 1, 0.0, 0.0)
    assert m.std(inside) < m.std(outside)


def test_unfitted_model_returns_the_prior():
    m = S.ResidualModel()
    f = S.features(SQ, _cfg(128, 128, 16, 1024))
    assert m.predict_s(f, 1e-3) == 1e-3 and m.std(f) == 1.0 and m.report() == []


def test_constraints_drop_thin_splits_and_starved_grids():
    shape = S.Shape(8192, 768, 768, "f32", "f32")
    cands = [_cfg(64, 64, 16, 1536), _cfg(64, 64, 16, 1536 * 8, split=8, launches=2),
             _cfg(64, 64, 16, 1536 * 32, split=32, launches=2), _cfg(256, 256, 16, 32, key="tiny grid")]
    kept = S.constrained(shape, cands)
    # split 8 leaves 96 of K per split (6 slices of 16); split 32 leaves 24 (< 2 slices); 32 workgroups vs 1536
    assert [c.key for c in kept] == [cands[0].key, cands[1].key]
    # a small grid stays when nothing of its variant fills the chip
    only_small = S.constrained(shape, [_cfg(256, 256, 16, 32, key="only")])
    assert [c.key for c in only_small] == ["only"]


def test_choose_spends_budget_on_best_predictions_then_uncertainty_and_keeps_the_incumbent():
    shape = S.Shape(8192, 3072, 768, "bf16", "bf16")
    cands = [_cfg(64, 64, 64, 6144, key="a"), _cfg(128, 128, 64, 1536, key="b"), _cfg(256, 128, 64, 768, key="c"),
             _cfg(256, 256, 64, 384, key="d"), _cfg(128, 128, 64, 3072 + 24576, split=2, launches=2, key="e")]
    m = S.ResidualModel()
    picked = S.choose(shape, cands, m, budget=2, explore=1, incumbent_key="e")
    keys = [c.key for c in picked]
    preds = sorted(cands, key=lambda c: S.prior_s(shape, S.features(shape, c)))
    assert keys[:2] == [preds[0].key, preds[1].key]
    assert len(keys) == 4 and keys[-1] == "e" or (len(keys) == 3 and "e" in keys)
    assert len(set(keys)) == len(keys)


def test_decide_replaces_only_on_a_consistent_paired_gain():
    inc = [100.0, 101.0, 99.0, 100.0, 102.0, 100.0, 98.0]
    faster = [v * 0.95 for v in inc]
    d = S.decide(inc, faster)
    assert not d.keep_incumbent and d.wins == 7 and d.ratio == pytest.approx(0.95)
    assert S.decide(inc, [v * 0.995 for v in inc]).keep_incumbent      # inside the 1 % margin
    mixed = [90.0, 110.0, 90.0, 110.0, 90.0, 110.0, 90.0]               # median gain, but 4 of 7 rounds only
    assert S.decide([100.0] * 7, mixed).keep_incumbent
    with pytest.raises(AssertionError):
        S.decide([1.0, 2.0], [1.0])
