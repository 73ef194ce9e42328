"""The synthetic workloads against the statistics the pages print, and the
oracle's predictor/pre-activation steps against closed forms.

* The power law of activations (page "PowerInfer: Fast Large Language Model
  Serving with a Consumer-grade GPU", section «Метод»): the top 26% (OPT) and
  43% (Llama-2-70B) most frequently active neurons carry 80% of the mass.
* The predictor (page "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU
  Konsumen", section «Prediktor Kepadatan Adaptif»): logit = pre-activation +
  independent N(0, s2) noise, so the predicted-active fraction, recall and
  precision have closed forms over the bivariate normal.
* Union of a batch: E|U|/F = mean_i 1 - (1 - q_i)^B.

Activations here are computed by the oracle, so a mistake in the oracle's
predictor or pre-activation (a dropped bias, a transposed operand, a missing
W1 stage) moves these statistics far outside the tolerances.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import scipy.special as sp

import oracle
from synth import CONFIGS, NOISE_VAR, expected_top_share, make_layer, make_tokens, powerlaw_profile, solve_alpha
from tests.conftest import GOLDEN

M9 = json.load(open(os.path.join(GOLDEN, "powerlaw_m9.json")))


def _empirical_top_share(freq, mass, top_fraction):
    """Rank by frequency (ties: larger mass first, then lower index) and return the top share."""
    order = np.lexsort((np.arange(freq.size), -mass, -freq))
    k = int(math.ceil(top_fraction * freq.size))
    return float(mass[order[:k]].sum() / mass.sum())


def test_alpha_calibration_closed_form():
    a_opt = solve_alpha(M9["opt"]["top_fraction"], M9["opt"]["mass_share"], 16384, 0.10)
    a_llama = solve_alpha(M9["llama2_70b"]["top_fraction"], M9["llama2_70b"]["mass_share"], 28672, 0.10)
    assert abs(a_opt - 0.8158) < 2e-3 and abs(a_llama - 0.6327) < 2e-3
    assert abs(expected_top_share(powerlaw_profile(16384, a_opt, 0.10, None), 0.26) - 0.80) < 1e-6
    p = powerlaw_profile(2048, 1.0, 0.10, None)
    assert abs(p.mean() - 0.10) < 1e-9 and p.max() <= 0.95 and p.min() >= 0.005


@pytest.mark.slow
@pytest.mark.parametrize("name,key,tokens", [("opt6.7b", "opt", 2048), ("llama70b", "llama2_70b", 1024)])
def test_power_law_mass_share(name, key, tokens):
    """Empirical top-X% mass share of oracle activations on the generated workload is 0.80 +- 0.02."""
    cfg = dataclasses.replace(CONFIGS[name], d=256, rank=None)
    L = make_layer(cfg, 0)
    H = L.to_host()
    x = make_tokens(cfg, tokens).numpy()
    pre = oracle.true_preactivation(H, x)                          # [T][F] of the masked projection
    if cfg.act == "relu":
        act = np.maximum(pre, 0.0)
    else:
        u = x.astype(np.float64) @ np.asarray(H["w_up"], dtype=np.float64).T
        act = np.abs(np.maximum(pre, 0.0) * u)
    freq = (pre > 0).mean(axis=0)
    share = _empirical_top_share(freq, act.sum(axis=0), M9[key]["top_fraction"])
    assert abs(share - M9[key]["mass_share"]) < 0.02, share
    assert abs(freq.mean() - 0.10) < 0.01


def _pair_positive(mu, s2):
    """P(h > 0 and h + n > 0) for h ~ N(mu, 1), n ~ N(0, s2) independent (numerical integral)."""
    h = np.linspace(-8, 8, 8001)[None, :] + mu[:, None]
    dens = np.exp(-0.5 * (h - mu[:, None]) ** 2) / math.sqrt(2 * math.pi)
    f = np.where(h > 0, dens * sp.ndtr(h / math.sqrt(s2)), 0.0)
    return f.sum(axis=1) * (h[0, 1] - h[0, 0])


def test_predictor_matches_closed_forms():
    cfg = dataclasses.replace(CONFIGS["opt6.7b"], d=1024, ffn=4096, rank=256)
    L = make_layer(cfg, 0)
    H = L.to_host()
    x = make_tokens(cfg, 256).numpy()
    v = oracle.predictor_logits(H, x)
    h = oracle.true_preactivation(H, x)
    n = v - h
    xn = (x.astype(np.float64) ** 2).sum(axis=1) / cfg.d
    # logit - pre-activation: variance s2 |x|^2/d, uncorrelated with the pre-activation
    assert abs(n.var(axis=1).mean() / (NOISE_VAR * xn.mean()) - 1.0) < 0.03
    assert abs(np.corrcoef(n.ravel(), (h - H["b"]).ravel())[0, 1]) < 0.02
    # predicted active, recall, precision
    mu = sp.ndtri(L.p)
    q = sp.ndtr(mu / math.sqrt(1 + NOISE_VAR))
    both = _pair_positive(mu, NOISE_VAR)
    pm, m = v > 0, h > 0
    assert abs(pm.mean() - q.mean()) < 0.004
    assert abs((pm & m).sum() / m.sum() - both.sum() / L.p.sum()) < 0.02
    assert abs((pm & m).sum() / pm.sum() - both.sum() / q.sum()) < 0.02


def test_union_fraction_closed_form():
    cfg = dataclasses.replace(CONFIGS["opt175b"], d=512, ffn=2048, rank=None, wtype="f16")
    L = make_layer(cfg, 0)
    H = L.to_host()
    B, nb = 8, 64
    x = make_tokens(cfg, B * nb).numpy().reshape(nb, B, cfg.d)
    frac = np.mean([oracle.union(oracle.threshold(oracle.decision_values(H, x[k]))).mean() for k in range(nb)])
    expect = np.mean(1.0 - (1.0 - L.p) ** B)
    assert abs(frac - expect) < 0.01, (frac, expect)


def test_adaptive_rank_and_layer_means():
    cfg = CONFIGS["falcon40b"]
    from synth import layer_mean
    means = np.array([layer_mean(cfg, i) for i in range(cfg.layers)])
    assert means.min() >= 0.03 and means.max() <= 0.12
    ranks = [cfg.layer_rank(m) for m in means]
    assert set(ranks) == {512, 1024}
    assert all((r == 512) == (m < 0.05) for r, m in zip(ranks, means))


def test_generator_is_deterministic():
    cfg = dataclasses.replace(CONFIGS["opt6.7b"], d=128, ffn=256, rank=32)
    a, b = make_layer(cfg, 5), make_layer(cfg, 5)
    for k, t in a.tensors().items():
        if t is not None:
            assert bool((t == getattr(b, k)).all()), k
    assert not bool((make_layer(cfg, 6).p_w2 == a.p_w2).all())
