"""Helpers that compare the HIP path (through the C ABI) with the fp64 oracle.

Inputs come from ``synth`` only. The oracle never reads a value the HIP path produced:
where a decision value lies within the oracle's exclusion band (|v - theta| < 1e-4) both
decisions are valid, so the expected y is the oracle's own y corrected by the oracle's own
contribution of each band neuron the HIP path decided the other way.
"""
import dataclasses

import numpy as np
import torch

import activation_sparse_ffn_layer_amd as pi
import oracle
from synth import Layer

TOL = {"f32": 1e-5, "f16": 2e-3, "q4_0": 1e-2}


def words_to_bool(words: torch.Tensor, ffn: int) -> np.ndarray:
    w = words.cpu().numpy().view(np.uint64)
    return oracle.words_to_mask(w, ffn)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    if nb == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def make_ctx(layers, max_batch=8):
    d = max(L.d for L in layers)
    f = max(L.ffn for L in layers)
    r = max(max(L.rank for L in layers), 8)
    return pi.Context(max_batch=max_batch, max_d=d, max_ffn=f, max_rank=r)


def run_layer(ctx, ffn: "pi.Ffn", x: torch.Tensor, with_logits=False):
    L = ffn.layer
    B = x.shape[0]
    dev = x.device
    y = torch.full((B, L.d), float("nan"), dtype=torch.float32, device=dev)
    mask = torch.zeros((B, L.ffn // 64), dtype=torch.int64, device=dev)
    idx = torch.full((L.ffn,), -1, dtype=torch.int32, device=dev)
    n = torch.full((1,), -1, dtype=torch.int32, device=dev)
    pi.layer(ctx, ffn, x, y, mask, idx, n)
    out = {"y": y, "mask": mask, "idx": idx, "n": n}
    if with_logits:
        logits = torch.full((B, L.ffn), float("nan"), dtype=torch.float32, device=dev)
        m2 = torch.zeros_like(mask)
        i2 = torch.full_like(idx, -1)
        n2 = torch.full_like(n, -1)
        pi.predict(ctx, ffn, x, m2, i2, n2, logits)
        out.update(logits=logits, mask_p=m2, idx_p=i2, n_p=n2)
    torch.cuda.synchronize()
    return out


def check_layer(host: dict, x_host: np.ndarray, out: dict, tol: float, check_logits=False, v=None, ref=None):
    """Assert parity of one batch; returns (#band neurons, #band neurons decided differently).

    ``v``: the oracle's decision values of x_host when already computed. ``ref``: a dict that
    receives the expected y (``ref["y"]``, [B][d] float64)."""
    ffn = host["ffn"]
    if v is None:
        v = oracle.decision_values(host, x_host)
    m_or = oracle.threshold(v, host["threshold"])
    band = oracle.band(v, host["threshold"])
    m_gpu = words_to_bool(out["mask"], ffn)
    B = x_host.shape[0]
    assert m_gpu.shape == (B, ffn)
    diff = m_gpu != m_or
    assert not np.any(diff & ~band), f"{int(np.sum(diff & ~band))} mask bits differ outside the band"
    # compaction of the GPU's own mask: bit exact
    u_gpu = oracle.union(m_gpu)
    n = int(out["n"].item())
    assert n == int(u_gpu.sum())
    np.testing.assert_array_equal(out["idx"][:n].cpu().numpy(), oracle.compact(u_gpu))
    if check_logits:
        lg = out["logits"].cpu().numpy().astype(np.float64)
        fin = np.isfinite(v)                       # hot-prefix neurons: +inf on both sides
        np.testing.assert_array_equal(lg[~fin], v[~fin])
        if fin.any():
            assert np.max(np.abs(lg[fin] - v[fin])) < oracle.THRESHOLD_BAND, np.max(np.abs(lg[fin] - v[fin]))
        np.testing.assert_array_equal(words_to_bool(out["mask_p"], ffn), m_gpu)
        assert int(out["n_p"].item()) == n
        np.testing.assert_array_equal(out["idx_p"][:n].cpu().numpy(), out["idx"][:n].cpu().numpy())
    # y: the oracle's y on its own union, corrected for band neurons decided the other way
    u_or = oracle.union(m_or)
    y_ref = oracle.sparse_ffn(host, x_host, oracle.compact(u_or))
    for i in np.flatnonzero(u_gpu & ~u_or):
        y_ref = y_ref + oracle.sparse_ffn(host, x_host, np.array([i]))
    for i in np.flatnonzero(u_or & ~u_gpu):
        y_ref = y_ref - oracle.sparse_ffn(host, x_host, np.array([i]))
    y = out["y"].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y))
    for t in range(B):
        if np.all(y_ref[t] == 0.0):
            assert np.all(y[t] == 0.0)
        else:
            e = rel_l2(y[t], y_ref[t])
            assert e <= tol, f"token {t}: rel L2 {e:.3e} > {tol}"
    if ref is not None:
        ref["y"] = y_ref
    return int(band.sum()), int(np.sum(diff))


def check_dump_layer(host: dict, dump: dict, layer: int, tol: float, next_x=None):
    """Teacher-forced parity of one layer of a recorded stack (pi_stack_run_dump): for every
    step, the oracle takes the layer's recorded input and the recorded mask words, index
    list, count and y are checked as in :func:`check_layer`. With ``next_x`` (the next layer's
    recorded inputs [S][B][d]), the chaining is checked too: the next input is within
    2 * tol + 1e-3 (relative L2 per token) of the oracle's glue of the oracle's y (the
    layer's expected output subtracted). Host arrays in ``dump``: x [S][L][B][d], mask
    [S][L][B][W], idx [S][L][stride], n [S][L], y [S][L][B][d]. Returns (band, flips)."""
    xs = dump["x"][:, layer]
    S, B, d = xs.shape
    W = host["ffn"] // 64
    v_all = oracle.decision_values(host, xs.reshape(S * B, d)).reshape(S, B, -1)
    bands = flips = 0
    for s in range(S):
        out = {"mask": torch.from_numpy(np.ascontiguousarray(dump["mask"][s, layer, :, :W])),
               "idx": torch.from_numpy(dump["idx"][s, layer]), "n": torch.tensor([int(dump["n"][s, layer])]),
               "y": torch.from_numpy(dump["y"][s, layer])}
        ref = {}
        nb, nf = check_layer(host, xs[s], out, tol, v=v_all[s], ref=ref)
        bands += nb
        flips += nf
        if next_x is not None:
            want = oracle.glue(ref["y"], xs[s], host.get("glue_center"))
            for t in range(B):
                e = rel_l2(next_x[s, t].astype(np.float64), want[t].astype(np.float64))
                assert e <= 2 * tol + 1e-3, f"step {s} token {t}: next input off by rel L2 {e:.3e}"
    return bands, flips


def check_layer_per_token(host: dict, x_host: np.ndarray, out: dict, tol: float):
    """Parity of one batch under per-token masking: masks as in check_layer; y[t] is the
    oracle's FFN of token t on its own mask, corrected for band neurons the HIP path decided
    the other way for that token. Returns the number of such band decisions."""
    ffn = host["ffn"]
    v = oracle.decision_values(host, x_host)
    m_or = oracle.threshold(v, host["threshold"])
    band = oracle.band(v, host["threshold"])
    m_gpu = words_to_bool(out["mask"], ffn)
    B = x_host.shape[0]
    diff = m_gpu != m_or
    assert not np.any(diff & ~band), f"{int(np.sum(diff & ~band))} mask bits differ outside the band"
    u_gpu = oracle.union(m_gpu)
    n = int(out["n"].item())
    assert n == int(u_gpu.sum())
    np.testing.assert_array_equal(out["idx"][:n].cpu().numpy(), oracle.compact(u_gpu))
    y_ref = oracle.per_token_ffn(host, x_host, m_or)
    for t, i in zip(*np.nonzero(diff)):
        c = oracle.sparse_ffn(host, x_host[t], np.array([i], dtype=np.int32))[0]
        y_ref[t] = y_ref[t] + c if m_gpu[t, i] else y_ref[t] - c
    y = out["y"].cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y))
    for t in range(B):
        if np.all(y_ref[t] == 0.0):
            assert np.all(y[t] == 0.0)
        else:
            e = rel_l2(y[t], y_ref[t])
            assert e <= tol, f"token {t}: rel L2 {e:.3e} > {tol}"
    return int(np.sum(diff))


def layer_with(layer: Layer, **kw) -> Layer:
    return dataclasses.replace(layer, **kw)
