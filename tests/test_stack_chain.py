"""Chaining of a deep stack keeps its tokens independent (oracle and generator, CPU).

A stack runs each token through every layer (page "PowerInfer: Mesin Inferensi LLM Cepat
dengan GPU Konsumen", introduction). PowerInfer's premise is that cold neurons depend on
the input while hot ones fire across inputs (page "Tüketici sınıfı GPU takılı PC'lerde
yüksek hızlı büyük dil modeli serving", header bullets). The chaining therefore must not
drive different tokens onto one input at depth. With the layer's expected output
subtracted before the rms normalisation, at every depth of full-depth stacks (96 layers
of the OPT-175B shape, 32 of the OPT-6.7B shape, at reduced width):
* the mean pairwise cosine of the 8 tokens' inputs stays near 0;
* the union of their predicted masks stays near its closed form E|U|/F = mean(1 - (1 - q)^8),
  q_i = Phi(mu_i / sqrt(1 + s2)) the predicted-active probability of neuron i;
* at one token per step, each token's active fraction stays near mean(q).
Without the subtraction the same stacks collapse (mean cosine above 0.9, union near the
single-token fraction) within a few layers, which the last test shows.
"""
import dataclasses
import math

import numpy as np
import pytest
import scipy.special as sp

import oracle
from synth import CONFIGS, make_layer, make_tokens

pytestmark = pytest.mark.slow


def _mean_cos(x):
    xn = x.astype(np.float64)
    xn = xn / np.linalg.norm(xn, axis=1, keepdims=True)
    c = xn @ xn.T
    n = x.shape[0]
    return (c.sum() - n) / (n * (n - 1))


def _chain(cfg, batch, tokens=8, center=True):
    """Yields (layer, mean pairwise cosine of the inputs, mean union fraction, expected)."""
    x = make_tokens(cfg, tokens).numpy()
    steps = [x[s:s + batch] for s in range(0, tokens, batch)]
    for li in range(cfg.layers):
        L = make_layer(cfg, li, chain_batch=batch)
        H = L.to_host()
        cos = _mean_cos(np.concatenate(steps))
        res = [oracle.layer_forward(H, xs) for xs in steps]
        q = sp.ndtr(sp.ndtri(L.p) / math.sqrt(1.0 + cfg.noise_var))
        expect = float(np.mean(1.0 - (1.0 - q) ** batch))
        frac = float(np.mean([r["n_active"] for r in res])) / cfg.ffn
        yield li, cos, frac, expect
        c = H["glue_center"] if center else None
        steps = [oracle.glue(r["y"], xs, c) for r, xs in zip(res, steps)]


@pytest.mark.parametrize("name,layers", [("opt175b", 96), ("opt6.7b", 32)])
def test_deep_stack_keeps_tokens_independent_batch8(name, layers):
    cfg = dataclasses.replace(CONFIGS[name], layers=layers, d=1024, ffn=4096, rank=256)
    coss = []
    for li, cos, frac, expect in _chain(cfg, 8):
        coss.append(cos)
        assert abs(cos) < 0.1, f"layer {li}: mean pairwise cosine {cos:.3f}"
        assert abs(frac - expect) < 0.05, f"layer {li}: union {frac:.3f} against {expect:.3f}"
    assert abs(np.mean(coss)) < 0.04, np.mean(coss)


@pytest.mark.parametrize("name,layers", [("opt175b", 96), ("opt6.7b", 32)])
def test_deep_stack_keeps_tokens_independent_batch1(name, layers):
    cfg = dataclasses.replace(CONFIGS[name], layers=layers, d=1024, ffn=4096, rank=256)
    coss = []
    for li, cos, frac, expect in _chain(cfg, 1):
        coss.append(cos)
        assert abs(cos) < 0.1, f"layer {li}: mean pairwise cosine {cos:.3f}"
        assert abs(frac - expect) < 0.02, f"layer {li}: active fraction {frac:.3f} against {expect:.3f}"
    assert abs(np.mean(coss)) < 0.04, np.mean(coss)


def test_plain_rms_chaining_collapses():
    """The reason for the subtraction: the plain rms chaining drives the tokens together."""
    cfg = dataclasses.replace(CONFIGS["opt175b"], layers=10, d=1024, ffn=4096, rank=256)
    last = None
    for li, cos, frac, expect in _chain(cfg, 8, center=False):
        last = (cos, frac, expect)
    cos, frac, expect = last
    assert cos > 0.9 and frac < 0.6 * expect, last
