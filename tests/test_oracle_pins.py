"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-worked
examples (tests/golden), the textbook dense FFN, brute-force bit loops, closed
forms and invariants. A dropped bias, a wrong sign, a transposed operand, a
swapped nibble or an off-by-one in the compaction fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_layer, scaled
from synth.gen import quantize_q4_0
from tests.conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _layer_dict(act, w_up, b, w_down_t, w_gate=None, wtype="f32", rank=0, **extra):
    w_up = np.asarray(w_up, dtype=np.float64)
    d = dict(d=w_up.shape[1], ffn=w_up.shape[0], rank=rank, act=act, wtype=wtype, threshold=0.0,
             w_up=w_up, w_gate=None if w_gate is None else np.asarray(w_gate, dtype=np.float64),
             w_down_t=np.asarray(w_down_t, dtype=np.float64), b=np.asarray(b, dtype=np.float64),
             s_up=None, s_gate=None, s_down=None, p_w1=None, p_w2=None, p_b=None)
    d.update(extra)
    return d


# ---------------------------------------------------------------------------------- golden

def test_golden_relu_tiny():
    g = _golden("relu_tiny.json")
    L = _layer_dict("relu", g["w_up"], g["b"], g["w_down_t"])
    x = np.array(g["x"], dtype=np.float64)
    np.testing.assert_array_equal(oracle.true_preactivation(L, x), g["h"])
    m = oracle.threshold(oracle.decision_values(L, x))
    np.testing.assert_array_equal(m, g["mask"])
    for t in range(2):
        y = oracle.sparse_ffn(L, x[t], oracle.compact(m[t]))
        np.testing.assert_array_equal(y[0], g["y_per_token"][t])
    r = oracle.layer_forward(L, x)
    np.testing.assert_array_equal(r["idx"], g["union_idx"])
    np.testing.assert_array_equal(r["y"], g["y_union"])


def test_golden_sqrelu_tiny():
    g = _golden("sqrelu_tiny.json")
    L = _layer_dict("sqrelu", g["w_up"], g["b"], g["w_down_t"])
    x = np.array(g["x"], dtype=np.float64)
    m = oracle.threshold(oracle.decision_values(L, x))
    np.testing.assert_array_equal(m, g["mask"])
    for t in range(2):
        y = oracle.sparse_ffn(L, x[t], oracle.compact(m[t]))
        np.testing.assert_array_equal(y[0], g["y_per_token"][t])
    r = oracle.layer_forward(L, x)
    np.testing.assert_array_equal(r["idx"], g["union_idx"])
    np.testing.assert_array_equal(r["y"], g["y_union"])


def test_golden_reglu_tiny():
    g = _golden("reglu_tiny.json")
    L = _layer_dict("reglu", g["w_up"], g["b"], g["w_down_t"], w_gate=g["w_gate"])
    x = np.array(g["x"], dtype=np.float64)
    np.testing.assert_array_equal(oracle.true_preactivation(L, x), g["g"])
    r = oracle.layer_forward(L, x)
    np.testing.assert_array_equal(r["mask"], g["mask"])
    np.testing.assert_array_equal(r["y"], g["y"])


def test_golden_per_token_tiny():
    """A predictor that misses a neuron one token activates: union and per-token differ by hand."""
    g = _golden("per_token_tiny.json")
    L = _layer_dict("relu", g["w_up"], g["b"], g["w_down_t"], rank=2,
                    p_w1=np.array(g["p_w1"], dtype=np.float64), p_w2=np.array(g["p_w2"], dtype=np.float64),
                    p_b=np.array(g["p_b"], dtype=np.float64))
    x = np.array(g["x"], dtype=np.float64)
    v = oracle.decision_values(L, x)
    np.testing.assert_array_equal(v, g["v"])
    m = oracle.threshold(v)
    np.testing.assert_array_equal(m, g["mask"])
    r = oracle.layer_forward(L, x)
    np.testing.assert_array_equal(r["idx"], g["union_idx"])
    np.testing.assert_array_equal(r["y"], g["y_union"])
    np.testing.assert_array_equal(oracle.per_token_ffn(L, x, m), g["y_per_token"])


def test_golden_predictor_tiny():
    g = _golden("predictor_tiny.json")
    w_up = np.zeros((4, 3))
    L = _layer_dict("relu", w_up, np.zeros(4), np.zeros((4, 3)), rank=2,
                    p_w1=np.array(g["p_w1"], dtype=np.float64), p_w2=np.array(g["p_w2"], dtype=np.float64),
                    p_b=np.array(g["p_b"], dtype=np.float64))
    v = oracle.decision_values(L, np.array(g["x"], dtype=np.float64))
    np.testing.assert_array_equal(v, g["v"])
    np.testing.assert_array_equal(oracle.threshold(v), g["mask"])


def test_golden_mask_words():
    g = _golden("mask_words_f128.json")
    m = np.zeros(g["ffn"], dtype=bool)
    m[g["active"]] = True
    w = oracle.mask_words(m)
    assert [int(v) for v in w[0]] == [int(s) for s in g["words"]]
    np.testing.assert_array_equal(oracle.compact(m), g["idx"])
    np.testing.assert_array_equal(oracle.words_to_mask(w, g["ffn"])[0], m)


def test_golden_q4_0_block():
    g = _golden("q4_0_block.json")
    codes = np.array(g["code_bytes"], dtype=np.uint8).reshape(1, 16)
    scales = np.array([g["scale"]], dtype=np.float16)
    np.testing.assert_array_equal(oracle.dequant_q4_0(codes, scales), g["values"])


def test_golden_q4_0_quantizer():
    """The generator's quantiser (input side) against a hand-worked block, read back by the oracle."""
    g = _golden("q4_0_quantize.json")
    w = torch.tensor([g["w"]], dtype=torch.float32)
    codes, scales = quantize_q4_0(w)
    assert float(scales[0, 0]) == g["scale"]
    c = codes.numpy()[0, 0]
    q = np.concatenate([c & 0xF, c >> 4])
    np.testing.assert_array_equal(q, g["codes"])
    np.testing.assert_array_equal(oracle.dequant_q4_0(codes.numpy(), scales.numpy())[0], g["stored"])


def test_golden_hot_first_order():
    g = _golden("hot_first_order.json")
    np.testing.assert_array_equal(oracle.hot_first_order(np.array(g["p"])), g["perm"])


# ------------------------------------------------------------------------- threshold, compaction

def test_threshold_special_values():
    v = np.array([0.0, -0.0, 2.0 ** -20, -(2.0 ** -20), 1e-45, -1e-45, np.inf, -np.inf, np.nan, 1.0, -1.0],
                 dtype=np.float32)
    np.testing.assert_array_equal(oracle.threshold(v),
                                  [False, False, True, False, True, False, True, False, False, True, False])
    # a zero predictor row with zero bias gives exactly 0 -> inactive
    L = _layer_dict("relu", np.zeros((1, 2)), [0.0], np.zeros((1, 2)), rank=1,
                    p_w1=np.ones((1, 2)), p_w2=np.zeros((1, 1)), p_b=np.zeros(1))
    assert not oracle.threshold(oracle.decision_values(L, np.ones((1, 2))))[0, 0]
    L["p_b"] = np.array([2.0 ** -20])
    assert oracle.threshold(oracle.decision_values(L, np.ones((1, 2))))[0, 0]


def _brute_words(m):
    words = []
    for w in range(len(m) // 64):
        acc = 0
        for j in range(64):
            if m[64 * w + j]:
                acc |= 1 << j
        words.append(acc)
    return words


def test_compaction_brute_force_low_bits():
    """Every pattern of the first 12 neurons (rest off) of a 64-neuron word, plus all single bits."""
    for pat in range(1 << 12):
        m = np.zeros(64, dtype=bool)
        for j in range(12):
            m[j] = bool((pat >> j) & 1)
        assert int(oracle.mask_words(m)[0, 0]) == _brute_words(m)[0]
        assert list(oracle.compact(m)) == [i for i in range(64) if m[i]]
    for j in range(128):
        m = np.zeros(128, dtype=bool)
        m[j] = True
        assert [int(v) for v in oracle.mask_words(m)[0]] == _brute_words(m)
        assert list(oracle.compact(m)) == [j]


@pytest.mark.parametrize("ffn,density", [(64, 0.5), (128, 0.03), (4096, 0.1), (4096, 0.9), (640, 0.0), (640, 1.0)])
def test_compaction_random_against_loops(ffn, density):
    rng = np.random.default_rng(ffn + int(density * 100))
    for _ in range(5):
        m = rng.random(ffn) < density
        assert [int(v) for v in oracle.mask_words(m)[0]] == _brute_words(m)
        idx = oracle.compact(m)
        assert list(idx) == [i for i in range(ffn) if m[i]]
        assert idx.dtype == np.int32
        assert np.all(np.diff(idx) > 0)
        np.testing.assert_array_equal(oracle.words_to_mask(oracle.mask_words(m), ffn)[0], m)


def test_union_is_or():
    m = np.array([[1, 0, 0, 1], [0, 0, 1, 1], [0, 0, 0, 0]], dtype=bool)
    np.testing.assert_array_equal(oracle.union(m), [True, False, True, True])


# ----------------------------------------------------------------------- sparse FFN vs dense

def _random_layer(rng, act, ffn=256, d=64, wtype="f32"):
    s = 1.0 / math.sqrt(d)
    w_up = rng.normal(0, s, (ffn, d))
    w_gate = rng.normal(0, s, (ffn, d)) if act == "reglu" else None
    w_down_t = rng.normal(0, s, (ffn, d))
    b = rng.normal(-1.0, 0.5, ffn)
    L = _layer_dict(act, w_up, b, w_down_t, w_gate=w_gate)
    if wtype == "f16":
        for k in ("w_up", "w_gate", "w_down_t"):
            if L[k] is not None:
                L[k] = L[k].astype(np.float16)
        L["wtype"] = "f16"
    return L


def _dense_relu(L, x):
    """Textbook dense ReLU FFN: W_down relu(W_up x + b), with W_down = w_down_t^T."""
    W_up = np.asarray(L["w_up"], dtype=np.float64)
    W_down = np.asarray(L["w_down_t"], dtype=np.float64).T
    return (W_down @ np.maximum(W_up @ x + L["b"], 0.0))


def _dense_sqrelu(L, x):
    """Textbook dense Squared-ReLU FFN: W_down relu(W_up x + b)^2."""
    W_up = np.asarray(L["w_up"], dtype=np.float64)
    W_down = np.asarray(L["w_down_t"], dtype=np.float64).T
    return W_down @ np.square(np.maximum(W_up @ x + L["b"], 0.0))


def _dense_reglu(L, x):
    Wg = np.asarray(L["w_gate"], dtype=np.float64)
    Wu = np.asarray(L["w_up"], dtype=np.float64)
    W_down = np.asarray(L["w_down_t"], dtype=np.float64).T
    return W_down @ (np.maximum(Wg @ x + L["b"], 0.0) * (Wu @ x))


@pytest.mark.parametrize("wtype", ["f32", "f16"])
def test_true_mask_sparse_equals_dense_relu(wtype):
    rng = np.random.default_rng(1)
    L = _random_layer(rng, "relu", wtype=wtype)
    for _ in range(8):
        x = rng.normal(size=64)
        r = oracle.layer_forward(L, x[None])
        assert 0 < r["n_active"] < L["ffn"]
        np.testing.assert_allclose(r["y"][0], _dense_relu(L, x), rtol=0, atol=1e-12)


def test_true_mask_sparse_equals_dense_sqrelu():
    rng = np.random.default_rng(12)
    L = _random_layer(rng, "sqrelu")
    for _ in range(8):
        x = rng.normal(size=64)
        r = oracle.layer_forward(L, x[None])
        assert 0 < r["n_active"] < L["ffn"]
        np.testing.assert_allclose(r["y"][0], _dense_sqrelu(L, x), rtol=0, atol=1e-12)
    # a single neuron gives h_i^2 w_down_t[i]; a listed inactive neuron gives nothing
    x = rng.normal(size=64)
    h = np.asarray(L["w_up"]) @ x + L["b"]
    i, j = int(np.argmax(h)), int(np.argmin(h))
    np.testing.assert_allclose(oracle.sparse_ffn(L, x, np.array([i]))[0], h[i] ** 2 * np.asarray(L["w_down_t"])[i],
                               rtol=1e-15, atol=0)
    np.testing.assert_array_equal(oracle.sparse_ffn(L, x, np.array([j]))[0], np.zeros(64))


def test_true_mask_sparse_equals_dense_reglu():
    rng = np.random.default_rng(2)
    L = _random_layer(rng, "reglu")
    for _ in range(8):
        x = rng.normal(size=64)
        r = oracle.layer_forward(L, x[None])
        assert 0 < r["n_active"] < L["ffn"]
        np.testing.assert_allclose(r["y"][0], _dense_reglu(L, x), rtol=0, atol=1e-12)


def test_all_active_empty_and_single_neuron():
    rng = np.random.default_rng(3)
    L = _random_layer(rng, "relu")
    x = rng.normal(size=64)
    np.testing.assert_allclose(oracle.sparse_ffn(L, x, np.arange(L["ffn"]))[0], _dense_relu(L, x), atol=1e-12)
    np.testing.assert_array_equal(oracle.sparse_ffn(L, x, np.array([], dtype=np.int32))[0], np.zeros(64))
    h = np.asarray(L["w_up"]) @ x + L["b"]
    i = int(np.argmax(h))
    np.testing.assert_allclose(oracle.sparse_ffn(L, x, np.array([i]))[0], h[i] * np.asarray(L["w_down_t"])[i],
                               rtol=1e-15, atol=0)
    # a neuron whose pre-activation is negative contributes nothing even if listed
    j = int(np.argmin(h))
    np.testing.assert_array_equal(oracle.sparse_ffn(L, x, np.array([j]))[0], np.zeros(64))


def test_batch_union_equals_per_token_equals_dense():
    """With the true mask, the union over a batch gives each token its own dense FFN."""
    rng = np.random.default_rng(4)
    for act in ("relu", "reglu", "sqrelu"):
        L = _random_layer(rng, act)
        X = rng.normal(size=(8, 64))
        r = oracle.layer_forward(L, X)
        dense = {"relu": _dense_relu, "reglu": _dense_reglu, "sqrelu": _dense_sqrelu}[act]
        for t in range(8):
            np.testing.assert_allclose(r["y"][t], dense(L, X[t]), atol=1e-12)
            own = oracle.layer_forward(L, X[t][None])
            np.testing.assert_allclose(r["y"][t], own["y"][0], atol=1e-12)


def test_per_token_true_mask_equals_dense_and_single_token_equals_union():
    """Per-token masking with the true mask gives each token its dense FFN (every activation
    family); at one token it is the union path; with a random mask it is the per-token sum of
    the chosen neurons' terms, one neuron at a time."""
    rng = np.random.default_rng(21)
    dense = {"relu": _dense_relu, "reglu": _dense_reglu, "sqrelu": _dense_sqrelu}
    for act in ("relu", "reglu", "sqrelu"):
        L = _random_layer(rng, act)
        X = rng.normal(size=(6, 64))
        m = oracle.threshold(oracle.true_preactivation(L, X))
        y = oracle.per_token_ffn(L, X, m)
        for t in range(6):
            np.testing.assert_allclose(y[t], dense[act](L, X[t]), atol=1e-12)
            one = oracle.layer_forward(L, X[t][None])
            np.testing.assert_allclose(y[t], one["y"][0], atol=1e-12)
        mr = rng.random((6, L["ffn"])) < 0.3
        yr = oracle.per_token_ffn(L, X, mr)
        for t in range(2):
            terms = [oracle.sparse_ffn(L, X[t], np.array([i], dtype=np.int32))[0] for i in np.flatnonzero(mr[t])]
            np.testing.assert_allclose(yr[t], np.sum(terms, axis=0), atol=1e-12)


def test_q4_0_layer_sparse_equals_dense_on_dequantised_weights():
    rng = np.random.default_rng(5)
    d, ffn = 128, 192
    w = torch.from_numpy(rng.normal(0, 1 / math.sqrt(d), (ffn, d)).astype(np.float32))
    wd = torch.from_numpy(rng.normal(0, 1 / math.sqrt(d), (ffn, d)).astype(np.float32))
    cu, su = quantize_q4_0(w)
    cd, sd = quantize_q4_0(wd)
    L = dict(d=d, ffn=ffn, rank=0, act="relu", wtype="q4_0", threshold=0.0, w_up=cu.numpy(), s_up=su.numpy(),
             w_gate=None, s_gate=None, w_down_t=cd.numpy(), s_down=sd.numpy(), b=rng.normal(-1, 0.5, ffn),
             p_w1=None, p_w2=None, p_b=None)
    Wu = oracle.dequant_q4_0(cu.numpy(), su.numpy())
    Wd = oracle.dequant_q4_0(cd.numpy(), sd.numpy())
    # the dequantised rows are close to the unquantised ones (round-trip bound below)
    assert np.max(np.abs(Wu - w.numpy())) <= np.max(su.numpy().astype(np.float64)) + 1e-12
    for _ in range(4):
        x = rng.normal(size=d)
        r = oracle.layer_forward(L, x[None])
        dense = Wd.T @ np.maximum(Wu @ x + L["b"], 0.0)
        np.testing.assert_allclose(r["y"][0], dense, atol=1e-12)


# ------------------------------------------------------------------------------ Q4_0 round trip

def test_q4_0_round_trip_bound():
    rng = np.random.default_rng(6)
    w = torch.from_numpy(rng.normal(0, 1, (64, 256)).astype(np.float32))
    w[3, 32:64] = 0.0                                      # an all-zero block
    codes, scales = quantize_q4_0(w)
    deq = oracle.dequant_q4_0(codes.numpy(), scales.numpy()).reshape(64, 8, 32)
    ref = w.numpy().astype(np.float64).reshape(64, 8, 32)
    s = scales.numpy().astype(np.float64)[..., None]
    err = np.abs(deq - ref)
    safe = np.where(s > 0, s, 1.0)
    clipped = np.rint(ref / safe) > 7                      # code would be 16: stored as 15
    # unclipped elements are within s/2; clipped ones store 7*s, within s of the block's absmax
    assert np.all(err[~clipped] <= (np.broadcast_to(s, err.shape) / 2)[~clipped] + 1e-12)
    np.testing.assert_allclose(deq[clipped], (7 * np.broadcast_to(s, err.shape))[clipped], rtol=0, atol=0)
    # s = fp16(absmax/8) may be rounded down by 2^-11 relative, so absmax <= 8 s (1 + 2^-11)
    assert np.all(err[clipped] <= np.broadcast_to(s, err.shape)[clipped] * (1 + 2.0 ** -8))
    np.testing.assert_array_equal(deq[3, 1], np.zeros(32))
    assert np.all(codes.numpy()[3, 1] == 0x88)
    # (q - 8) * s is exact in float32 as well as float64
    q = np.concatenate([codes.numpy() & 0xF, codes.numpy() >> 4], axis=-1).astype(np.float32)
    f32 = ((q - 8) * scales.numpy().astype(np.float32)[..., None])
    np.testing.assert_array_equal(f32.astype(np.float64), deq)


# ----------------------------------------------------------------------------- permutation

def test_hot_first_permutation_invariance():
    cfg = scaled(CONFIGS["falcon40b"], d=128, ffn=512, rank=64)
    gen = make_layer(cfg, 3)
    layer = gen.to_host()
    perm = oracle.hot_first_order(gen.p)
    assert np.all(np.diff(gen.p[perm]) <= 0)
    P = oracle.permute_layer(layer, perm)
    x = np.random.default_rng(7).normal(size=(4, 128)).astype(np.float16)
    r0 = oracle.layer_forward(layer, x)
    r1 = oracle.layer_forward(P, x)
    np.testing.assert_array_equal(r1["mask"], r0["mask"][:, perm])
    np.testing.assert_array_equal(np.sort(perm[r1["idx"]]), r0["idx"])
    np.testing.assert_allclose(r1["y"], r0["y"], rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------ glue

def test_glue_properties():
    rng = np.random.default_rng(8)
    y = rng.normal(0, 3.0, size=(3, 256))
    x_prev = rng.normal(size=(3, 256)).astype(np.float16)
    y[1] = 0.0
    out = oracle.glue(y, x_prev)
    assert out.dtype == np.float16
    np.testing.assert_array_equal(out[1], x_prev[1])
    for t in (0, 2):
        rms = np.sqrt(np.mean(out[t].astype(np.float64) ** 2))
        assert abs(rms - 1.0) < 1e-3
        # scaling y by a power of two changes nothing (bit for bit)
        np.testing.assert_array_equal(oracle.glue(y[t:t + 1] * 8.0, x_prev[t:t + 1])[0], out[t])
        # direction is preserved within fp16 rounding
        np.testing.assert_allclose(out[t].astype(np.float64), y[t] / np.sqrt(np.mean(y[t] ** 2)),
                                   rtol=2.0 ** -11, atol=2.0 ** -24)
    out32 = oracle.glue(y, x_prev.astype(np.float32))
    assert out32.dtype == np.float32


# ------------------------------------------------------------------------------- band

def _num(v):
    return float(v) if not isinstance(v, str) else {"inf": np.inf, "-inf": -np.inf, "nan": np.nan}[v]


def test_golden_band():
    """The exclusion band: strict |v - theta| < 1e-4 in float64, on hand-worked values
    (exactly 1e-4 away is outside; 5e-5 off a nonzero theta is inside; inf and NaN are outside)."""
    g = _golden("band.json")
    for case in g["cases"]:
        v = np.array([_num(x) for x in case["v"]], dtype=np.float64)
        np.testing.assert_array_equal(oracle.band(v, case["theta"]), case["band"])
        # the same values as a [1][F] batch give the same answer row-wise
        np.testing.assert_array_equal(oracle.band(v[None, :], case["theta"])[0], case["band"])
    c = g["float32_case"]
    np.testing.assert_array_equal(oracle.band(np.array(c["v"], dtype=np.float32), c["theta"]), c["band"])
    assert oracle.THRESHOLD_BAND == 1e-4


# ------------------------------------------------------------------------------ stacks

def _golden_stack_layers(g, hot_prefix=0):
    a, b = g["layer_a"], g["layer_b"]
    A = _layer_dict("relu", a["w_up"], a["b"], a["w_down_t"], glue_center=np.array(a["glue_center"], float))
    B = _layer_dict("relu", b["w_up"], b["b"], b["w_down_t"], rank=1,
                    p_w1=np.array(b["p_w1"], float), p_w2=np.array(b["p_w2"], float),
                    p_b=np.array(b["p_b"], float), glue_center=np.array(b["glue_center"], float),
                    hot_prefix=hot_prefix)
    return A, B


def test_golden_stack_two_layers():
    """stack_forward on a hand-worked two-layer, two-token stack (chaining vector, all-zero
    pass-through, a predictor miss, union against per-token batches), and the same numbers
    from an explicit layer_forward -> glue loop."""
    g = _golden("stack_two_layers.json")
    A, B = _golden_stack_layers(g)
    x0 = np.array(g["x0"], dtype=np.float16)
    # one token at a time
    for t in range(2):
        res = oracle.stack_forward([A, B], x0[t:t + 1])
        np.testing.assert_array_equal(res[0]["x"][0], x0[t])
        np.testing.assert_array_equal(res[0]["y"][0], g["y_a"][t])
        np.testing.assert_array_equal(res[0]["mask"][0], g["mask_a"][t])
        np.testing.assert_array_equal(res[1]["x"][0], g["x1"][t])
        assert res[1]["x"].dtype == np.float16
        np.testing.assert_array_equal(res[1]["v"][0], g["v_b"][t])
        np.testing.assert_array_equal(res[1]["mask"][0], g["mask_b"][t])
        np.testing.assert_array_equal(res[1]["y"][0], g["y_b_per_token"][t])
    # both tokens as one batch (union of the batch's masks)
    res = oracle.stack_forward([A, B], x0)
    np.testing.assert_array_equal(res[1]["x"], g["x1"])
    np.testing.assert_array_equal(res[1]["y"], g["y_b_batch"])
    assert [r["n_active"] for r in res] == g["n_active_batch"]
    # the explicit loop with the golden's own numbers
    r0 = oracle.layer_forward(A, x0)
    x1 = oracle.glue(r0["y"], x0, np.array(g["layer_a"]["glue_center"], float))
    np.testing.assert_array_equal(x1, g["x1"])
    r1 = oracle.layer_forward(B, x1)
    np.testing.assert_array_equal(r1["y"], res[1]["y"])


def test_glue_center_identities():
    """glue(y, c) = glue(y - c, 0) whenever y is not all zero; c = 0 is the plain rms glue;
    a token with y == c, or y == 0 while c != 0, passes x through."""
    rng = np.random.default_rng(21)
    d = 128
    y = rng.normal(0, 2.0, size=(4, d))
    c = rng.normal(0, 0.5, size=d)
    x_prev = rng.normal(size=(4, d)).astype(np.float16)
    y[1] = c
    y[2] = 0.0
    out = oracle.glue(y, x_prev, c)
    np.testing.assert_array_equal(out[1], x_prev[1])
    np.testing.assert_array_equal(out[2], x_prev[2])
    for t in (0, 3):
        np.testing.assert_array_equal(out[t], oracle.glue(y[t:t + 1] - c, x_prev[t:t + 1])[0])
        np.testing.assert_array_equal(oracle.glue(y[t:t + 1], x_prev[t:t + 1], np.zeros(d))[0],
                                      oracle.glue(y[t:t + 1], x_prev[t:t + 1])[0])
        u = y[t] - c
        np.testing.assert_allclose(out[t].astype(np.float64), u / np.sqrt(np.mean(u * u)),
                                   rtol=2.0 ** -11, atol=2.0 ** -24)


# ------------------------------------------------------------------------ hot prefix

def test_hot_prefix_taken_without_prediction():
    """A hot prefix of H stored neurons is always computed: H = ffn gives the dense FFN (the
    true mask, textbook numpy), H = 0 the predictor's mask, and in between the prefix's
    exact ReLU plus the predicted tail. Prefix decisions are +inf, never in the band."""
    cfg = scaled(CONFIGS["opt6.7b"], d=64, ffn=128, rank=16)
    H = make_layer(cfg, 3).to_host()
    x = np.random.default_rng(5).normal(size=(3, 64)).astype(np.float16)
    x64 = x.astype(np.float64)
    w_up = H["w_up"].astype(np.float64)
    w_dn = H["w_down_t"].astype(np.float64)
    b = H["b"].astype(np.float64)
    relu = np.maximum(x64 @ w_up.T + b, 0.0)
    dense = relu @ w_dn
    pred = oracle.predictor_logits(H, x) > 0
    for hp in (0, 40, 128):
        L = dict(H, hot_prefix=hp)
        v = oracle.decision_values(L, x)
        assert np.all(np.isinf(v[:, :hp])) and not np.any(oracle.band(v[:, :hp]))
        m = pred.copy()
        m[:, :hp] = True
        for t in range(3):
            r = oracle.layer_forward(L, x[t:t + 1])
            np.testing.assert_array_equal(r["mask"][0], m[t])
            np.testing.assert_allclose(r["y"][0], (m[t] * relu[t]) @ w_dn, rtol=0, atol=1e-12)
        if hp == 128:
            r = oracle.layer_forward(L, x)
            np.testing.assert_allclose(r["y"], dense, rtol=0, atol=1e-12)
