"""fp64 statement of the neuron-aware sparse FFN, step by step.

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke()``
and ``bench.py``'s cpu_baseline leg, never by the HIP path.

Pages cited (by title and section):

* P1 = "Tüketici sınıfı GPU takılı PC'lerde yüksek hızlı büyük dil modeli serving"
* P2 = "PowerInfer: Fast Large Language Model Serving with a Consumer-grade GPU" (КПД)
* P3 = "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU Konsumen"

What the method computes, per FFN layer and token x (all in float64 here):

1. A decision value per neuron. With a predictor (P3 «Prediktor Kepadatan
   Adaptif»: only neurons predicted active are processed; predictors differ
   in size per layer, P2 «Метод»): a low-rank linear map
   ``v = W2 (W1 x) + b_p``. Without one, the true pre-activation of the masked
   projection, ``v = W x + b``.
2. The mask ``m_i = [v_i > theta]`` (strict), theta = 0, i.e. "sigmoid(v) > 0.5"
   taken without evaluating the sigmoid.
3. The index list of active neurons, ascending. For a batch of B tokens, the
   union of the B masks.
4. For each active neuron i, its row of the up (and gate) projection and its
   column of the down projection, used directly without forming a dense
   matrix (P3 «Operator yang Sadar Neuron»: the operators work on individual
   row and column vectors):
   ReLU ``a_i = max(W_up[i] . x + b_i, 0)``;
   ReGLU ``a_i = max(W_gate[i] . x + b_i, 0) * (W_up[i] . x)``;
   Squared-ReLU ``a_i = max(W_up[i] . x + b_i, 0) ** 2``;
   ``y = sum_i a_i * W_down[:, i]`` (stored neuron-major as ``w_down_t[i]``).
   P1 (header bullets, «Kısıtlar ve SSS») restricts the method to ReLU / ReGLU
   / Squared-ReLU models.
5. Q4_0 weights (P1 «Kuantizasyon ve uyumluluk»): each block of 32 elements
   along d stores an fp16 scale s and 4-bit codes q; the weight is (q - 8) * s.
6. Hot-first layout (P3 «Penempatan dan Pengelolaan Neuron»: neurons are
   placed by hotness and a neuron table maps each one back to its original
   position): neurons reordered by descending activation probability, the
   table ``perm[k]`` = original id of stored neuron k. The output is unchanged.

Readings taken where the pages are silent (each is a named choice):

* The predictor is linear and low rank with no hidden nonlinearity; its bias
  is the masked projection's bias.
* ``v == theta`` (including -0.0) is inactive; NaN is inactive.
* A batch uses the union of its tokens' masks for every token; ReLU zeroes
  the neurons a token does not itself activate. Per-token masking (each token on
  its own mask only, :func:`per_token_ffn`) is the alternative the library offers
  as a mode; with the true mask the two agree.
* ReGLU: only the gate has a bias; the mask is taken on the gate.
* Squared-ReLU (named, not defined, by the pages): ``max(h, 0) ** 2`` of the up
  projection; like ReLU it has one row per neuron and the mask is taken on it.
* Layers of a stack are chained by ``x_next = fp16((y - c) / rms(y - c))`` (the
  pages give no layer between FFNs), with ``c`` a fixed per-layer vector that
  the input generator supplies: the expected y of the layer, so that the
  tokens' common component is removed and each token's x keeps its own
  direction through the stack. An all-zero y (or y == c) passes x through.
* A hot prefix of H stored neurons (the hot neurons that PowerInfer keeps
  resident and computes without asking the predictor) is always taken: their
  decision value is +inf, and the activation itself zeroes the inactive ones.
* Decision values within 1e-4 of theta form an exclusion band: there a
  float32 evaluation may legitimately decide either way.
"""
from __future__ import annotations

import numpy as np

THRESHOLD_BAND = 1e-4


# ------------------------------------------------------------------------------------------
# weights
# ------------------------------------------------------------------------------------------

def dequant_q4_0(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q4_0 rows to float64 (P1 «Kuantizasyon ve uyumluluk»).

    ``codes`` uint8 ``[..., nb, 16]``: byte j of a block holds element j in its
    low nibble and element j + 16 in its high nibble. ``scales`` fp16
    ``[..., nb]``. Element value = (q - 8) * s. Returns ``[..., nb * 32]``."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0x0F).astype(np.float64)
    hi = (codes >> 4).astype(np.float64)
    q = np.concatenate([lo, hi], axis=-1)                     # [..., nb, 32]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)[..., None]
    w = (q - 8.0) * s
    return w.reshape(*w.shape[:-2], w.shape[-2] * 32)


def rows_f64(layer: dict, which: str, rows=None) -> np.ndarray:
    """Rows of one stored projection (``which`` in up/gate/down_t) as float64."""
    w = layer["w_" + which]
    if rows is not None:
        w = w[rows]
    if layer["wtype"] == "q4_0":
        s = layer[{"up": "s_up", "gate": "s_gate", "down_t": "s_down"}[which]]
        if rows is not None:
            s = s[rows]
        return dequant_q4_0(w, s)
    return np.asarray(w).astype(np.float64)


def _masked_name(layer: dict) -> str:
    return "gate" if layer["act"] == "reglu" else "up"


# ------------------------------------------------------------------------------------------
# steps 1-3: decision value, threshold, compaction
# ------------------------------------------------------------------------------------------

def predictor_logits(layer: dict, x: np.ndarray) -> np.ndarray:
    """``v = W2 (W1 x) + b_p`` for each token (P3 «Prediktor Kepadatan Adaptif»). x: [B][d]."""
    x64 = np.atleast_2d(np.asarray(x)).astype(np.float64)
    w1 = np.asarray(layer["p_w1"]).astype(np.float64)
    w2 = np.asarray(layer["p_w2"]).astype(np.float64)
    z = x64 @ w1.T                                             # [B][r]
    return z @ w2.T + np.asarray(layer["p_b"]).astype(np.float64)


def true_preactivation(layer: dict, x: np.ndarray) -> np.ndarray:
    """``W x + b`` of the masked projection (up for ReLU, gate for ReGLU), every neuron."""
    x64 = np.atleast_2d(np.asarray(x)).astype(np.float64)
    w = rows_f64(layer, _masked_name(layer))
    return x64 @ w.T + np.asarray(layer["b"]).astype(np.float64)


def decision_values(layer: dict, x: np.ndarray) -> np.ndarray:
    """Decision value of every neuron for each token x ``[B][d]``.

    With a predictor, its logits; without, the true pre-activation. The first
    ``layer["hot_prefix"]`` stored neurons (default 0) are computed for every
    token without a prediction (P1 header bullets and «CPU/GPU hibrit çıkarım
    yöntemi»: hot neurons are preloaded and always computed; P3 «Penempatan dan
    Pengelolaan Neuron»): their value is +inf, so they are always above the
    threshold and never inside the exclusion band."""
    v = predictor_logits(layer, x) if layer["rank"] > 0 else true_preactivation(layer, x)
    h = int(layer.get("hot_prefix", 0) or 0)
    if h > 0:
        v = np.array(v, dtype=np.float64, copy=True)
        v[:, :h] = np.inf
    return v


def threshold(v: np.ndarray, theta: float = 0.0) -> np.ndarray:
    """Mask bit per neuron: strictly above the threshold."""
    return np.asarray(v) > theta


def band(v: np.ndarray, theta: float = 0.0) -> np.ndarray:
    """Neurons whose decision value lies strictly within ``THRESHOLD_BAND`` of theta.

    There the float32 evaluation of a kernel and this float64 one may legitimately
    decide differently, so mask checks exclude these neurons and count them. The
    distance is taken in float64; exactly 1e-4 away is outside the band; +-inf and
    NaN are outside."""
    with np.errstate(invalid="ignore"):
        return np.abs(np.asarray(v, dtype=np.float64) - theta) < THRESHOLD_BAND


def mask_words(m: np.ndarray) -> np.ndarray:
    """Pack bool ``[B][F]`` (F % 64 == 0) into uint64 ``[B][F/64]``; bit j of word w is neuron 64w + j."""
    m = np.atleast_2d(np.asarray(m, dtype=bool))
    B, F = m.shape
    if F % 64:
        raise ValueError("F must be a multiple of 64")
    weights = np.left_shift(np.uint64(1), np.arange(64, dtype=np.uint64))
    bits = m.reshape(B, F // 64, 64).astype(np.uint64)
    return np.bitwise_or.reduce(bits * weights, axis=-1)


def words_to_mask(words: np.ndarray, ffn: int) -> np.ndarray:
    words = np.atleast_2d(np.asarray(words, dtype=np.uint64))
    bits = (words[..., None] >> np.arange(64, dtype=np.uint64)) & np.uint64(1)
    return bits.reshape(words.shape[0], -1)[:, :ffn].astype(bool)


def union(m: np.ndarray) -> np.ndarray:
    """OR of the per-token masks of a batch."""
    return np.any(np.atleast_2d(m), axis=0)


def compact(m: np.ndarray) -> np.ndarray:
    """Ascending int32 indices of the set bits of a 1-D mask."""
    return np.flatnonzero(np.asarray(m, dtype=bool)).astype(np.int32)


# ------------------------------------------------------------------------------------------
# step 4: the sparse FFN on an index list
# ------------------------------------------------------------------------------------------

def sparse_ffn(layer: dict, x: np.ndarray, idx: np.ndarray, chunk: int = 2048) -> np.ndarray:
    """``y[t] = sum_{i in idx} a_{t,i} W_down[:, i]`` with the activation of the layer.

    Reads only the rows of the active neurons (P3 «Operator yang Sadar
    Neuron»). ``idx`` is processed in ascending chunks only to bound memory.
    Returns float64 ``[B][d]``."""
    x64 = np.atleast_2d(np.asarray(x)).astype(np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    y = np.zeros((x64.shape[0], layer["d"]), dtype=np.float64)
    b = np.asarray(layer["b"]).astype(np.float64)
    for c0 in range(0, idx.size, chunk):
        rows = idx[c0:c0 + chunk]
        if layer["act"] == "relu":
            h = x64 @ rows_f64(layer, "up", rows).T + b[rows]
            a = np.maximum(h, 0.0)
        elif layer["act"] == "sqrelu":
            h = x64 @ rows_f64(layer, "up", rows).T + b[rows]
            a = np.maximum(h, 0.0) ** 2
        elif layer["act"] == "reglu":
            g = x64 @ rows_f64(layer, "gate", rows).T + b[rows]
            u = x64 @ rows_f64(layer, "up", rows).T
            a = np.maximum(g, 0.0) * u
        else:
            raise ValueError(layer["act"])
        y += a @ rows_f64(layer, "down_t", rows)
    return y


def per_token_ffn(layer: dict, x: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Per-token masking of a batch: ``y[t] = sum over i with m[t, i] of a_{t,i} W_down[:, i]``.

    Each token is processed on its own predicted neurons only, the operator of P3
    «Operator yang Sadar Neuron» applied one token at a time with the mask P3
    «Prediktor Kepadatan Adaptif» gives that token; the alternative to the union reading
    for batches. Returns float64 ``[B][d]``."""
    x = np.atleast_2d(np.asarray(x))
    m = np.atleast_2d(np.asarray(m, dtype=bool))
    y = np.zeros((x.shape[0], layer["d"]), dtype=np.float64)
    for t in range(x.shape[0]):
        y[t] = sparse_ffn(layer, x[t:t + 1], compact(m[t]))[0]
    return y


def layer_forward(layer: dict, x: np.ndarray) -> dict:
    """Steps 1-4 for one batch x ``[B][d]``: v, per-token masks, band, union idx, y."""
    x = np.atleast_2d(np.asarray(x))
    v = decision_values(layer, x)
    m = threshold(v, layer.get("threshold", 0.0))
    idx = compact(union(m))
    y = sparse_ffn(layer, x, idx)
    return {"v": v, "mask": m, "band": band(v, layer.get("threshold", 0.0)), "idx": idx,
            "n_active": int(idx.size), "y": y}


# ------------------------------------------------------------------------------------------
# step 6: hot-first layout; layer chaining
# ------------------------------------------------------------------------------------------

def hot_first_order(p: np.ndarray) -> np.ndarray:
    """Neuron table: stored position k holds original neuron ``perm[k]``, by descending p (stable)."""
    return np.argsort(-np.asarray(p, dtype=np.float64), kind="stable").astype(np.int32)


_ROW_ARRAYS = ("w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down", "b", "p_w2", "p_b")


def permute_layer(layer: dict, perm: np.ndarray) -> dict:
    """The same layer with its neurons stored in the order ``perm`` (P3 «Penempatan dan Pengelolaan Neuron»)."""
    out = dict(layer)
    for k in _ROW_ARRAYS:
        if layer.get(k) is not None:
            out[k] = np.asarray(layer[k])[perm]
    out["neuron_table"] = np.asarray(perm, dtype=np.int32)
    return out


def glue(y: np.ndarray, x_prev: np.ndarray, center=None) -> np.ndarray:
    """Next layer's input per token: ``u = y - c``, ``x_next = u / sqrt(mean(u^2))``,
    rounded to x's storage type (fp16 stacks to fp16, nearest even; fp32 stacks to fp32).

    ``center`` is the layer's fixed vector c ``[d]`` (None: zero). A token whose y is all
    zero (empty mask), or whose u is all zero, passes x_prev through unchanged."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    x_prev = np.atleast_2d(np.asarray(x_prev))
    c = np.zeros(y.shape[1]) if center is None else np.asarray(center, dtype=np.float64)
    out = np.empty(y.shape, dtype=x_prev.dtype)
    for t in range(y.shape[0]):
        u = y[t] - c
        ss = float(np.sum(u * u))
        if ss == 0.0 or not np.any(y[t] != 0.0):
            out[t] = x_prev[t]
        else:
            out[t] = (u / np.sqrt(ss / y.shape[1])).astype(x_prev.dtype)
    return out


def stack_forward(layers, x0: np.ndarray):
    """Run a stack one batch at a time (P3 intro: each token passes through the whole
    model before the next), chaining layer l to l + 1 by :func:`glue` with layer l's
    ``glue_center``. Returns per-layer results, each with the layer's input ``x``."""
    x = np.atleast_2d(np.asarray(x0))
    results = []
    for layer in layers:
        r = layer_forward(layer, x)
        r["x"] = x
        results.append(r)
        x = glue(r["y"], x, layer.get("glue_center"))
    return results
