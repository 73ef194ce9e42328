"""Parity of the HIP path (through the C ABI) with the fp64 oracle on seeded synthetic inputs.

Masks: bit exact outside the exclusion band |v| < 1e-4 (band neurons counted). Index
lists: bit exact with the mask they come from. Decision values: within the band width of
the oracle's. y: max per-token relative L2 within 1e-5 (fp32 weights), 2e-3 (fp16),
1e-2 (Q4_0). Identical decision values (pi_compact): bit exact with no exclusion.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_decision_values, make_layer, make_tokens
from tests.parity_util import (TOL, check_layer, check_layer_per_token, make_ctx, rel_l2, run_layer,
                               words_to_bool)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import activation_sparse_ffn_layer_amd as pi


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ threshold + compaction

@pytest.mark.parametrize("B,ffn", [(1, 64), (1, 2048), (2, 320), (5, 16384), (8, 49152), (1, 49152)])
def test_compact_identical_decision_values(B, ffn):
    _say(f"compact B={B} ffn={ffn}")
    v = make_decision_values(B, ffn, seed=1000 * B + ffn)
    ctx = pi.Context(max_batch=8, max_d=64, max_ffn=ffn, max_rank=0)
    vd = torch.from_numpy(v).cuda()
    mask = torch.zeros((B, ffn // 64), dtype=torch.int64, device="cuda")
    idx = torch.full((ffn,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    pi.compact(ctx, vd, 0.0, mask, idx, n)
    torch.cuda.synchronize()
    m = oracle.threshold(v, 0.0)
    np.testing.assert_array_equal(mask.cpu().numpy().view(np.uint64), oracle.mask_words(m))
    ref = oracle.compact(oracle.union(m))
    assert int(n.item()) == ref.size
    np.testing.assert_array_equal(idx[:ref.size].cpu().numpy(), ref)


def test_compact_every_low_pattern():
    """All 4096 patterns of a word's low 12 bits (plus random high bits), 64 words per call."""
    ffn = 64 * 64
    ctx = pi.Context(max_batch=1, max_d=64, max_ffn=ffn, max_rank=0)
    rng = np.random.default_rng(7)
    mask = torch.zeros((1, ffn // 64), dtype=torch.int64, device="cuda")
    idx = torch.full((ffn,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for call in range(64):
        pats = np.arange(call * 64, call * 64 + 64)
        bits = np.zeros((64, 64), dtype=bool)
        for j in range(12):
            bits[:, j] = (pats >> j) & 1
        bits[:, 12:] = rng.random((64, 52)) < 0.3
        v = np.where(bits.reshape(1, ffn), 1.0, -1.0).astype(np.float32)
        pi.compact(ctx, torch.from_numpy(v).cuda(), 0.0, mask, idx, n)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(words_to_bool(mask, ffn)[0], bits.reshape(ffn))
        ref = oracle.compact(bits.reshape(ffn))
        assert int(n.item()) == ref.size
        np.testing.assert_array_equal(idx[:ref.size].cpu().numpy(), ref)


# ------------------------------------------------------------------------ layer parity

def _cfg(name, **kw):
    return dataclasses.replace(CONFIGS[name], **kw)


CASES = {
    # name: (config, layer id, tokens, batch)
    "tiny": (_cfg("tiny"), 0, 16, 1),
    "opt-small": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 0, 8, 1),
    "opt-full": (_cfg("opt6.7b"), 3, 3, 1),
    "falcon-full-r1024": (_cfg("falcon40b"), 0, 2, 1),
    "llama-full-reglu": (_cfg("llama70b"), 0, 2, 1),
    "llama-small-truemask": (_cfg("llama70b", d=1024, ffn=4096, rank=None), 0, 4, 1),
    "opt175-full-q4": (_cfg("opt175b"), 0, 2, 1),
    "opt175-small-q4-b2": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 0, 4, 2),
    "q4-truemask-ragged": (_cfg("opt175b", d=544, ffn=320, rank=None), 0, 4, 1),
    "f16-ragged": (_cfg("opt6.7b", d=520, ffn=320, rank=136), 0, 4, 1),
    "f16-b2": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 1, 8, 2),
    "f16-b4": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 1, 8, 4),
    "f16-b8": (_cfg("opt6.7b", d=2048, ffn=8192, rank=1024), 1, 16, 8),
    "reglu-b8": (_cfg("llama70b", d=1024, ffn=4096, rank=512), 1, 8, 8),
    "f32-b3": (_cfg("tiny"), 0, 9, 3),
    # Q4_0 batches of 3..8 (quarter-block down lanes), ReGLU on Q4_0, x in column windows
    "q4-b4": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 1, 8, 4),
    "q4-b8": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 2, 16, 8),
    "q4-b5-ragged": (_cfg("opt175b", d=544, ffn=320, rank=136), 0, 10, 5),
    "q4-reglu-b8": (_cfg("opt175b", act="reglu", d=1024, ffn=2048, rank=512), 0, 8, 8),
    "q4-truemask-b8": (_cfg("opt175b", d=544, ffn=320, rank=None), 0, 8, 8),
    "reglu-truemask-b8": (_cfg("llama70b", d=1024, ffn=4096, rank=None), 0, 8, 8),
    "f16-b8-xwindows": (_cfg("opt6.7b", d=12288, ffn=2048, rank=512), 0, 8, 8),
    "opt175-full-q4-b8": (_cfg("opt175b"), 0, 8, 8),
    # x larger than 64 KiB: the up GEMV over column slices of x (last slice narrower)
    "reglu-b8-cols": (_cfg("llama70b", d=8192, ffn=4096, rank=512), 0, 8, 8),
    "sqrelu-q4-b4-cols": (_cfg("opt175b", act="sqrelu", d=16896, ffn=2048, rank=512), 0, 8, 4),
    "f16-b3-cols-ragged": (_cfg("opt6.7b", d=8200, ffn=320, rank=136), 0, 6, 3),
    "f16-b1-cols": (_cfg("opt6.7b", d=33280, ffn=512, rank=136), 0, 2, 1),
    # Squared-ReLU (one up row per neuron, a = max(h, 0)^2) on every path
    "sqrelu-small": (_cfg("opt6.7b", act="sqrelu", d=1024, ffn=4096, rank=512), 0, 8, 1),
    "sqrelu-full": (_cfg("opt6.7b", act="sqrelu"), 2, 2, 1),
    "sqrelu-b8": (_cfg("opt6.7b", act="sqrelu", d=1024, ffn=4096, rank=512), 1, 16, 8),
    "sqrelu-truemask-b3": (_cfg("opt6.7b", act="sqrelu", d=1024, ffn=2048, rank=None), 0, 6, 3),
    "sqrelu-q4-b2": (_cfg("opt175b", act="sqrelu", d=2048, ffn=4096, rank=512), 0, 4, 2),
    "sqrelu-b32-mfma": (_cfg("opt6.7b", act="sqrelu", d=1024, ffn=4096, rank=512), 2, 32, 32),
    # batched path on the matrix cores (9..64 tokens)
    "relu-b16-mfma": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 2, 32, 16),
    "reglu-b64-mfma": (_cfg("llama70b", d=1024, ffn=4096, rank=512), 2, 64, 64),
    "reglu-b40-truemask-mfma": (_cfg("llama70b", d=1024, ffn=4096, rank=None), 3, 40, 40),
    "llama-full-b64-mfma": (_cfg("llama70b"), 1, 64, 64),
    # batch sizes between the classes: 6 and 7 tokens on the 8-token vector kernels, 12 on the
    # matrix cores
    "f16-b6": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 2, 12, 6),
    "q4-b7": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 3, 14, 7),
    "relu-b12-mfma": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 3, 24, 12),
    "reglu-b7-cols": (_cfg("llama70b", d=8192, ffn=4096, rank=512), 1, 7, 7),
    # Q4_0 at 3 tokens (the 4-token kernels with a padded token) over a ragged last slice
    "q4-b3-ragged": (_cfg("opt175b", d=800, ffn=640, rank=136), 0, 6, 3),
}


@pytest.mark.parametrize("case", list(CASES))
def test_layer_parity(case):
    cfg, li, T, B = CASES[case]
    _say(f"layer parity {case}: d={cfg.d} ffn={cfg.ffn} rank={cfg.rank} {cfg.wtype} {cfg.act} B={B}")
    L = make_layer(cfg, li, device="cuda")
    H = L.to_host()
    X = make_tokens(cfg, T, device="cuda", stream=li + 1)
    ctx = make_ctx([L], max_batch=max(8, B))
    ffn = pi.Ffn(ctx, L)
    bands = flips = 0
    for s in range(T // B):
        x = X[s * B:(s + 1) * B].contiguous()
        out = run_layer(ctx, ffn, x, with_logits=True)
        nb, nf = check_layer(H, x.cpu().numpy(), out, TOL[cfg.wtype], check_logits=True)
        bands += nb
        flips += nf
    _say(f"  {case}: band neurons {bands}, decided differently {flips}")


# hot prefix: the first H stored neurons are taken without a prediction (H not a multiple of
# 8 leaves a mask byte half predicted; H = ffn is the dense FFN)
HP_CASES = {
    "hp-f16-b1": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 0, 4, 1, 300),
    "hp-f16-b1-ragged": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 1, 4, 1, 101),
    "hp-q4-b1-cols": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 0, 4, 1, 517),
    "hp-f16-b4": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 2, 8, 4, 256),
    "hp-reglu-b2": (_cfg("llama70b", d=1024, ffn=4096, rank=512), 0, 4, 2, 77),
    "hp-relu-b16-mfma": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 2, 32, 16, 333),
    "hp-all-b1": (_cfg("opt6.7b", d=1024, ffn=2048, rank=512), 0, 2, 1, 2048),
}


@pytest.mark.parametrize("case", list(HP_CASES))
def test_layer_parity_hot_prefix(case):
    cfg, li, T, B, hp = HP_CASES[case]
    _say(f"hot-prefix parity {case}: d={cfg.d} ffn={cfg.ffn} rank={cfg.rank} {cfg.wtype} {cfg.act} B={B} H={hp}")
    L = dataclasses.replace(make_layer(cfg, li, device="cuda"), hot_prefix=hp)
    H = L.to_host()
    X = make_tokens(cfg, T, device="cuda", stream=li + 3)
    ctx = make_ctx([L], max_batch=max(8, B))
    ffn = pi.Ffn(ctx, L)
    for s in range(T // B):
        x = X[s * B:(s + 1) * B].contiguous()
        out = run_layer(ctx, ffn, x, with_logits=True)
        check_layer(H, x.cpu().numpy(), out, TOL[cfg.wtype], check_logits=True)
        m = words_to_bool(out["mask"], cfg.ffn)
        assert m[:, :hp].all(), "a hot-prefix neuron is missing from a token's mask"
        assert bool(torch.all(out["logits"][:, :hp] == float("inf")))


# per-token masking: each token gets only its own predicted neurons (vector and matrix paths)
PT_CASES = {
    "pt-f16-b3": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 1, 6, 3),
    "pt-sqrelu-b8": (_cfg("opt6.7b", act="sqrelu", d=1024, ffn=4096, rank=512), 1, 16, 8),
    "pt-reglu-b8-cols": (_cfg("llama70b", d=8192, ffn=4096, rank=512), 0, 8, 8),
    "pt-q4-b4": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 1, 8, 4),
    "pt-q4-b8": (_cfg("opt175b", d=2048, ffn=8192, rank=512), 2, 16, 8),
    "pt-truemask-b8": (_cfg("llama70b", d=1024, ffn=4096, rank=None), 0, 8, 8),
    "pt-relu-b16-mfma": (_cfg("opt6.7b", d=1024, ffn=4096, rank=512), 2, 32, 16),
    "pt-reglu-b64-mfma": (_cfg("llama70b", d=1024, ffn=4096, rank=512), 2, 64, 64),
}


@pytest.mark.parametrize("case", list(PT_CASES))
def test_layer_parity_per_token(case):
    cfg, li, T, B = PT_CASES[case]
    _say(f"per-token parity {case}: d={cfg.d} ffn={cfg.ffn} rank={cfg.rank} {cfg.wtype} {cfg.act} B={B}")
    L = make_layer(cfg, li, device="cuda")
    H = L.to_host()
    X = make_tokens(cfg, T, device="cuda", stream=li + 2)
    ctx = make_ctx([L], max_batch=max(8, B))
    ffn = pi.Ffn(ctx, L)
    flips = 0
    differ = 0
    for s in range(T // B):
        x = X[s * B:(s + 1) * B].contiguous()
        ctx.set_mask_mode("per_token")
        out = run_layer(ctx, ffn, x)
        flips += check_layer_per_token(H, x.cpu().numpy(), out, TOL[cfg.wtype])
        ctx.set_mask_mode("union")
        out_u = run_layer(ctx, ffn, x)
        differ += int(torch.sum(torch.any(out_u["y"] != out["y"], dim=1)).item())
    if cfg.rank is not None:
        assert differ > 0, "per-token and union masking gave the same y for every token"
    _say(f"  {case}: band decisions taken the other way {flips}; tokens whose y differs from the union's {differ}")


def test_stack_per_token_mode_graph_and_switch():
    """The mode reaches captured stack steps: per-token graph == per-token eager, a one-layer
    stack equals pi_layer in that mode, and switching back to the union restores its result."""
    cfg = _cfg("opt6.7b", layers=3, d=1024, ffn=4096, rank=512)
    layers = [make_layer(cfg, i, device="cuda") for i in range(cfg.layers)]
    X = make_tokens(cfg, 8, device="cuda")
    ctx = make_ctx(layers, max_batch=4)
    ffns = [pi.Ffn(ctx, L) for L in layers]

    def run(graph, nl=3):
        y = torch.empty((8, cfg.d), dtype=torch.float32, device="cuda")
        pi.stack_run(ctx, ffns[:nl], X, 4, y, None, use_graph=graph)
        return y

    y_u = run(True)
    ctx.set_mask_mode("per_token")
    y_pg, y_pe = run(True), run(False)
    y1 = run(True, nl=1)
    ctx.set_mask_mode("union")
    y_u2 = run(True)
    ctx.set_mask_mode("per_token")
    out = run_layer(ctx, ffns[0], X[:4].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y_pg, y_pe), "per-token graph and eager runs differ"
    assert torch.equal(y_u, y_u2), "the union result changed after a mode round trip"
    assert not torch.equal(y_u, y_pg), "the mode had no effect on the stack"
    assert torch.equal(y1[:4], out["y"]), "one-layer stack and pi_layer differ in per-token mode"
    check_layer_per_token(layers[0].to_host(), X[:4].cpu().numpy(), out, TOL["f16"])


def test_empty_and_full_masks():
    cfg = _cfg("opt6.7b", d=1024, ffn=2048, rank=512)
    L = make_layer(cfg, 0, device="cuda")
    x = make_tokens(cfg, 2, device="cuda")
    ctx = make_ctx([L])
    for bias, expect in ((-60.0, 0), (60.0, cfg.ffn)):
        L2 = dataclasses.replace(L, b=torch.full_like(L.b, bias), p_b=torch.full_like(L.p_b, bias))
        ffn = pi.Ffn(ctx, L2)
        out = run_layer(ctx, ffn, x[:1])
        assert int(out["n"].item()) == expect
        check_layer(L2.to_host(), x[:1].cpu().numpy(), out, TOL["f16"])
        if expect == 0:
            assert torch.all(out["y"] == 0)


def test_predict_then_sparse_ffn_equals_layer_bitwise():
    cfg = _cfg("opt6.7b", d=2048, ffn=8192, rank=512)
    L = make_layer(cfg, 2, device="cuda")
    x = make_tokens(cfg, 4, device="cuda")
    ctx = make_ctx([L])
    ffn = pi.Ffn(ctx, L)
    for B in (1, 4):
        xb = x[:B].contiguous()
        out = run_layer(ctx, ffn, xb)
        mask = torch.zeros_like(out["mask"])
        idx = torch.full_like(out["idx"], -1)
        n = torch.full_like(out["n"], -1)
        pi.predict(ctx, ffn, xb, mask, idx, n)
        y = torch.empty_like(out["y"])
        pi.sparse_ffn(ctx, ffn, xb, idx, n, y)
        torch.cuda.synchronize()
        assert torch.equal(mask, out["mask"]) and int(n.item()) == int(out["n"].item())
        assert torch.equal(y, out["y"])
        out2 = run_layer(ctx, ffn, xb)
        assert torch.equal(out2["y"], out["y"]), "layer is not deterministic"


@pytest.mark.parametrize("B", [1, 3, 8])
def test_predict_then_sparse_ffn_equals_layer_bitwise_q4(B):
    """Same identity on Q4_0 weights, with x in column windows at 8 tokens (d = 12288)."""
    cfg = _cfg("opt175b", ffn=2048, rank=512)
    L = make_layer(cfg, 1, device="cuda")
    x = make_tokens(cfg, B, device="cuda")
    ctx = make_ctx([L])
    ffn = pi.Ffn(ctx, L)
    out = run_layer(ctx, ffn, x)
    mask = torch.zeros_like(out["mask"])
    idx = torch.full_like(out["idx"], -1)
    n = torch.full_like(out["n"], -1)
    pi.predict(ctx, ffn, x, mask, idx, n)
    y = torch.empty_like(out["y"])
    pi.sparse_ffn(ctx, ffn, x, idx, n, y)
    torch.cuda.synchronize()
    assert torch.equal(mask, out["mask"]) and int(n.item()) == int(out["n"].item())
    assert torch.equal(y, out["y"])
    check_layer(L.to_host(), x.cpu().numpy(), out, TOL["q4_0"])


def test_sparse_ffn_on_oracle_index_list():
    """pi_sparse_ffn on an index list the oracle computed (input-side: from synth data)."""
    cfg = _cfg("llama70b", d=1024, ffn=4096, rank=None)
    L = make_layer(cfg, 5, device="cuda")
    H = L.to_host()
    x = make_tokens(cfg, 2, device="cuda")
    ctx = make_ctx([L])
    ffn = pi.Ffn(ctx, L)
    xh = x.cpu().numpy()
    idx_h = oracle.compact(oracle.union(oracle.threshold(oracle.decision_values(H, xh))))
    idx = torch.from_numpy(np.concatenate([idx_h, np.zeros(cfg.ffn - idx_h.size, np.int32)])).cuda()
    n = torch.tensor([idx_h.size], dtype=torch.int32, device="cuda")
    y = torch.empty((2, cfg.d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(ctx, ffn, x, idx, n, y)
    torch.cuda.synchronize()
    ref = oracle.sparse_ffn(H, xh, idx_h)
    for t in range(2):
        assert rel_l2(y[t].cpu().numpy(), ref[t]) <= TOL["f16"]


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_sparse_ffn_column_slices_on_oracle_index_list(act):
    """pi_sparse_ffn at 8 tokens with fp32 weights and x above 64 KiB (column-sliced up
    GEMV) on the oracle's union list with out-of-range entries mixed in (skipped), and on
    an empty list (y = 0)."""
    cfg = _cfg("tiny", act=act, d=2560, ffn=1024)
    L = make_layer(cfg, 1, device="cuda")
    H = L.to_host()
    B = 8
    x = make_tokens(cfg, B, device="cuda")
    ctx = make_ctx([L])
    ffn = pi.Ffn(ctx, L)
    xh = x.cpu().numpy()
    idx_h = oracle.compact(oracle.union(oracle.threshold(oracle.decision_values(H, xh))))
    assert idx_h.size > 0
    lst = np.insert(idx_h, [0, idx_h.size // 2, idx_h.size], [-1, cfg.ffn + 5, -7]).astype(np.int32)
    idx = torch.from_numpy(np.concatenate([lst, np.zeros(cfg.ffn + 3 - lst.size, np.int32)])).cuda()
    n = torch.tensor([lst.size], dtype=torch.int32, device="cuda")
    y = torch.empty((B, cfg.d), dtype=torch.float32, device="cuda")
    pi.sparse_ffn(ctx, ffn, x, idx, n, y)
    torch.cuda.synchronize()
    ref = oracle.sparse_ffn(H, xh, idx_h)
    for t in range(B):
        assert rel_l2(y[t].cpu().numpy(), ref[t]) <= TOL["f32"]
    n.zero_()
    pi.sparse_ffn(ctx, ffn, x, idx, n, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


# ------------------------------------------------------------------------------- glue

@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
@pytest.mark.parametrize("centered", [False, True])
def test_glue(dtype, centered):
    rng = np.random.default_rng(11)
    B, d = 4, 4096
    c = rng.normal(0, 1.5, d).astype(np.float32) if centered else None
    y = rng.normal(0, 2.5, (B, d)).astype(np.float32)
    y[1] = 0
    if centered:
        y[3] = c + rng.normal(0, 0.5, d).astype(np.float32)   # mostly the common component
        y[2] = c                                              # nothing but it: x passes through
    xp = rng.normal(0, 1, (B, d)).astype(np.float16 if dtype == torch.float16 else np.float32)
    ctx = pi.Context(max_batch=4, max_d=d, max_ffn=64, max_rank=0)
    xo = torch.empty((B, d), dtype=dtype, device="cuda")
    pi.glue(ctx, torch.from_numpy(y).cuda(), torch.from_numpy(xp).cuda(), xo,
            None if c is None else torch.from_numpy(c).cuda())
    torch.cuda.synchronize()
    ref = oracle.glue(y.astype(np.float64), xp, None if c is None else c.astype(np.float64))
    got = xo.cpu().numpy()
    np.testing.assert_array_equal(got[1], xp[1])
    if centered:
        np.testing.assert_array_equal(got[2], xp[2])
    if dtype == torch.float16:
        # fp32 arithmetic then one rounding to fp16: at most one fp16 ulp from the fp64 result
        ulp = np.spacing(np.abs(ref.astype(np.float16))).astype(np.float64)
        assert np.all(np.abs(got.astype(np.float64) - ref.astype(np.float64)) <= ulp)
    else:
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------------------ stacks

@pytest.mark.parametrize("act", ["relu", "sqrelu"])
def test_stack_true_mask_chain_matches_oracle(act):
    cfg = _cfg("opt6.7b", layers=3, d=1024, ffn=4096, rank=None, act=act)
    layers = [make_layer(cfg, i, device="cuda") for i in range(cfg.layers)]
    X = make_tokens(cfg, 4, device="cuda")
    ctx = make_ctx(layers, max_batch=1)
    ffns = [pi.Ffn(ctx, L) for L in layers]
    y = torch.empty((4, cfg.d), dtype=torch.float32, device="cuda")
    nlog = torch.zeros((4, cfg.layers), dtype=torch.int32, device="cuda")
    pi.stack_run(ctx, ffns, X, 1, y, nlog, use_graph=True)
    y2 = torch.empty_like(y)
    pi.stack_run(ctx, ffns, X, 1, y2, None, use_graph=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "graph and eager runs differ"
    hosts = [L.to_host() for L in layers]
    for t in range(4):
        res = oracle.stack_forward(hosts, X[t:t + 1].cpu().numpy())
        assert rel_l2(y[t].cpu().numpy(), res[-1]["y"][0]) <= TOL["f16"]
        got_n = nlog[t].cpu().numpy()
        want_n = np.array([r["n_active"] for r in res])
        assert np.all(np.abs(got_n - want_n) <= 2), (got_n, want_n)


def test_stack_predictor_graph_equals_eager_and_is_deterministic():
    cfg = _cfg("opt6.7b", layers=4, d=1024, ffn=4096, rank=512)
    layers = [make_layer(cfg, i, device="cuda") for i in range(cfg.layers)]
    X = make_tokens(cfg, 8, device="cuda")
    ctx = make_ctx(layers, max_batch=2)
    ffns = [pi.Ffn(ctx, L) for L in layers]
    outs = []
    for use_graph in (True, True, False):
        y = torch.empty((8, cfg.d), dtype=torch.float32, device="cuda")
        pi.stack_run(ctx, ffns, X, 2, y, None, use_graph=use_graph)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    # the first layer of each step is teacher-free: check it against the oracle directly
    H0 = layers[0].to_host()
    out = run_layer(ctx, ffns[0], X[:2].contiguous())
    check_layer(H0, X[:2].cpu().numpy(), out, TOL["f16"])


@pytest.mark.parametrize("d,B", [(8192, 1), (8192, 2), (4096, 1), (4096, 4), (8192, 8), (12288, 3)])
def test_stack_glue_of_partials_equals_layer_by_layer(d, B):
    """The stack hands each layer's down partial sums (8 groups at 1..2 tokens, 16 at 3..8
    tokens) to the next layer's glue: at one token the
    glue-sum kernel and stage 1, at 2..8 tokens one workgroup per token (1 to 3 chunks of
    columns per thread). Chaining pi_layer and pi_glue by hand, which sums them first, gives
    the same y up to rounding."""
    cfg = _cfg("falcon40b", layers=3, d=d, ffn=4096, rank=512)
    layers = [make_layer(cfg, i, device="cuda") for i in range(cfg.layers)]
    T = 2 * B
    X = make_tokens(cfg, T, device="cuda", stream=5)
    ctx = make_ctx(layers, max_batch=B)
    ffns = [pi.Ffn(ctx, L) for L in layers]
    y_stack = torch.empty((T, d), dtype=torch.float32, device="cuda")
    pi.stack_run(ctx, ffns, X, B, y_stack, None, use_graph=True)
    for s in range(T // B):
        x = X[s * B:(s + 1) * B].contiguous()
        for li, f in enumerate(ffns):
            out = run_layer(ctx, f, x)
            if li + 1 < len(ffns):
                xn = torch.empty_like(x)
                pi.glue(ctx, out["y"], x, xn, layers[li].glue_center)
                x = xn
        torch.cuda.synchronize()
        for t in range(B):
            e = rel_l2(y_stack[s * B + t].cpu().numpy(), out["y"][t].cpu().numpy())
            assert e <= TOL["f16"], f"step {s} token {t}: rel L2 {e:.3e}"


@pytest.mark.parametrize("B", [3, 8])
def test_stack_glue_fp32_rows_equals_layer_by_layer(B):
    """The same with fp32 rows and no predictor (true mask): the 2..8-token glue keeps x in
    fp32."""
    cfg = _cfg("tiny", layers=3, d=1536, ffn=2048)
    layers = [make_layer(cfg, i, device="cuda") for i in range(cfg.layers)]
    T = 2 * B
    X = make_tokens(cfg, T, device="cuda", stream=6)
    ctx = make_ctx(layers, max_batch=B)
    ffns = [pi.Ffn(ctx, L) for L in layers]
    y_stack = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    pi.stack_run(ctx, ffns, X, B, y_stack, None, use_graph=True)
    for s in range(T // B):
        x = X[s * B:(s + 1) * B].contiguous()
        for li, f in enumerate(ffns):
            out = run_layer(ctx, f, x)
            if li + 1 < len(ffns):
                xn = torch.empty_like(x)
                pi.glue(ctx, out["y"], x, xn, layers[li].glue_center)
                x = xn
        torch.cuda.synchronize()
        for t in range(B):
            e = rel_l2(y_stack[s * B + t].cpu().numpy(), out["y"][t].cpu().numpy())
            assert e <= TOL["f32"], f"step {s} token {t}: rel L2 {e:.3e}"


@pytest.mark.parametrize("B", [1, 2])
def test_stack_glue_passes_x_through_an_all_zero_layer(B):
    """A layer whose predictor marks no neuron gives y = 0, and the chaining then hands the
    next layer the same x. At one token the next layer's stage 1 takes that branch in its own
    glue, at two tokens the glue kernel does. Either way the second layer's y equals one
    pi_layer call on the stack's input, bit for bit."""
    cfg = _cfg("opt6.7b", layers=2, d=1024, ffn=2048, rank=512)
    L0 = make_layer(cfg, 0, device="cuda")
    L0 = dataclasses.replace(L0, b=torch.full_like(L0.b, -60.0), p_b=torch.full_like(L0.p_b, -60.0))
    L1 = make_layer(cfg, 1, device="cuda")
    T = 2 * B
    X = make_tokens(cfg, T, device="cuda", stream=9)
    ctx = make_ctx([L0, L1], max_batch=B)
    ffns = [pi.Ffn(ctx, L0), pi.Ffn(ctx, L1)]
    y_stack = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    nlog = torch.zeros((T // B, 2), dtype=torch.int32, device="cuda")
    pi.stack_run(ctx, ffns, X, B, y_stack, nlog, use_graph=True)
    torch.cuda.synchronize()
    assert torch.all(nlog[:, 0] == 0) and torch.all(nlog[:, 1] > 0)
    for s in range(T // B):
        out = run_layer(ctx, ffns[1], X[s * B:(s + 1) * B].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(y_stack[s * B:(s + 1) * B], out["y"]), f"step {s}"


def test_stack_graph_follows_rebuilt_layers():
    """A stack step captured as a graph holds its layers' weight pointers. Destroying the
    layers and wrapping other weights (on handles the allocator may place at the same
    addresses) must not replay the old graph: the graph run equals the eager run."""
    cfg = _cfg("opt6.7b", layers=2, d=1024, ffn=2048, rank=512)
    X = make_tokens(cfg, 2, device="cuda")
    ctx = make_ctx([make_layer(cfg, 0, device="cuda")], max_batch=1)
    ys = []
    for seed in (0, 1):
        layers = [make_layer(cfg, i, master=seed, device="cuda") for i in range(cfg.layers)]
        ffns = [pi.Ffn(ctx, L) for L in layers]
        yg = torch.empty((2, cfg.d), dtype=torch.float32, device="cuda")
        ye = torch.empty_like(yg)
        pi.stack_run(ctx, ffns, X, 1, yg, None, use_graph=True)
        pi.stack_run(ctx, ffns, X, 1, ye, None, use_graph=False)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), f"seed {seed}: graph and eager runs differ"
        ys.append(yg)
        for f in ffns:
            f.close()
    assert not torch.equal(ys[0], ys[1])


# ------------------------------------------------------------------------ Q4_0 dequantisation

def test_q4_dequant_bitwise_equals_oracle():
    """The kernels' in-register Q4_0 unpacking, dumped by pi_q4_dequant, equals the oracle's
    (q - 8) * s bit for bit (both exact): on quantised random rows with an all-zero block, a
    block of equal magnitudes, extreme and subnormal scales, and on stored rows of an
    OPT-175B-shaped layer (P1 «Kuantizasyon ve uyumluluk»)."""
    from synth import quantize_q4_0
    g = torch.Generator().manual_seed(5)
    w = torch.randn((64, 1024), generator=g, dtype=torch.float32) * 0.05
    w[0, :32] = 0.0                       # all-zero block: s = 0, q = 8
    w[1, 32:64] = 0.25                    # every element at the absmax: codes clip to 15
    w[2, 64:96] *= 1e4                    # large scale
    w[3, 96:128] *= 1e-6                  # fp16-subnormal scale
    codes, scales = quantize_q4_0(w)
    sets = [(codes, scales)]
    cfg = dataclasses.replace(CONFIGS["opt175b"], ffn=1024, rank=256)
    L = make_layer(cfg, 0, device="cuda")
    rows = torch.tensor([0, 1, 511, 1023])
    sets.append((L.w_down_t.reshape(1024, -1, 16)[rows].cpu(), L.s_down[rows].cpu()))
    sets.append((L.w_up.reshape(1024, -1, 16)[rows].cpu(), L.s_up[rows].cpu()))
    ctx = make_ctx([L])
    for c, sc in sets:
        c = c.contiguous()
        sc = sc.contiguous()
        n, nb = sc.shape
        out = torch.full((n, nb * 32), float("nan"), dtype=torch.float32, device="cuda")
        pi.q4_dequant(ctx, c.cuda(), sc.view(torch.int16).cuda(), out)
        torch.cuda.synchronize()
        want = oracle.dequant_q4_0(c.numpy(), sc.numpy()).astype(np.float32)
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
            f"{int((got != want).sum())} of {got.size} dequantised weights differ"


# ------------------------------------------------------------------------ permutation

def test_hot_first_permutation_on_device():
    cfg = _cfg("falcon40b", d=1024, ffn=4096, rank=512)
    L = make_layer(cfg, 7, device="cuda")
    perm = pi.hot_first_order(L.p)
    np.testing.assert_array_equal(perm, oracle.hot_first_order(L.p))
    ctx = make_ctx([L])
    pd = torch.from_numpy(perm).cuda()

    def pr(t):
        if t is None:
            return None
        out = torch.empty_like(t)
        pi.permute_rows(ctx, t, out, pd)
        return out

    P = dataclasses.replace(L, w_up=pr(L.w_up), w_down_t=pr(L.w_down_t), b=pr(L.b), p_w2=pr(L.p_w2), p_b=pr(L.p_b))
    torch.cuda.synchronize()
    H, HP = L.to_host(), P.to_host()
    ref = oracle.permute_layer(H, perm)
    for k in ("w_up", "w_down_t", "b", "p_w2", "p_b"):
        np.testing.assert_array_equal(HP[k], ref[k])
    x = make_tokens(cfg, 2, device="cuda")
    ffn_p = pi.Ffn(ctx, P, neuron_table=pd)
    out = run_layer(ctx, ffn_p, x[:1])
    check_layer(HP, x[:1].cpu().numpy(), out, TOL["f16"])
    ffn = pi.Ffn(ctx, L)
    out0 = run_layer(ctx, ffn, x[:1])
    assert rel_l2(out["y"].cpu().numpy(), out0["y"].cpu().numpy()) <= TOL["f16"]


# ----------------------------------------------------------------------------- errors

def test_invalid_arguments_enqueue_nothing():
    cfg = _cfg("opt6.7b", d=1024, ffn=2048, rank=512)
    L = make_layer(cfg, 0, device="cuda")
    ctx = make_ctx([L], max_batch=2)
    ffn = pi.Ffn(ctx, L)
    x = make_tokens(cfg, 4, device="cuda")
    y = torch.empty((4, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(pi.PiError, match="invalid argument"):
        pi.layer(ctx, ffn, x, y)                       # B = 4 > max_batch 2
    with pytest.raises(pi.PiError, match="not 16-byte aligned"):
        pi.layer(ctx, ffn, x[:1], y.view(-1)[1:].view(-1)[: cfg.d].view(1, cfg.d))
    bad = dataclasses.replace(L, ffn=2000)
    with pytest.raises(pi.PiError, match="multiple of 64"):
        pi.Ffn(ctx, bad)
    big = pi.Context(max_batch=80, max_d=1024, max_ffn=2048, max_rank=512)
    f2 = pi.Ffn(big, L)
    x70 = make_tokens(cfg, 70, device="cuda")
    y70 = torch.empty((70, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(pi.PiError, match="unsupported"):
        pi.layer(big, f2, x70, y70)                    # above the 64-token batched path
    q4 = dataclasses.replace(CONFIGS["opt175b"], d=1024, ffn=2048, rank=512)
    Lq = make_layer(q4, 0, device="cuda")
    fq = pi.Ffn(big, Lq)
    with pytest.raises(pi.PiError, match="unsupported"):
        pi.layer(big, fq, x70[:12].contiguous(), y70[:12])  # Q4_0 above 8 tokens


def test_stack_batched_graph_equals_eager():
    cfg = _cfg("llama70b", layers=3, d=1024, ffn=4096, rank=512)
    layers = [make_layer(cfg, i, device="cuda") for i in range(cfg.layers)]
    X = make_tokens(cfg, 32, device="cuda")
    ctx = make_ctx(layers, max_batch=16)
    ffns = [pi.Ffn(ctx, L) for L in layers]
    outs = []
    for use_graph in (True, False):
        y = torch.empty((32, cfg.d), dtype=torch.float32, device="cuda")
        pi.stack_run(ctx, ffns, X, 16, y, None, use_graph=use_graph)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.all(torch.isfinite(outs[0]))


# ---------------------------------------------------------------- stacks at the bench's shapes

STACKS = {
    # name: (config, layers, tokens, batch)
    "opt6.7b-b1": (_cfg("opt6.7b", layers=3), 3, 2, 1),
    "falcon40b-b1": (_cfg("falcon40b", layers=3), 3, 2, 1),   # 4 down partial sums into the glue
    "llama70b-b2": (_cfg("llama70b", layers=2), 2, 4, 2),     # 4 partial sums through k_reduce
    "opt175b-q4-b8": (_cfg("opt175b", layers=2), 2, 8, 8),
    "llama70b-b64": (_cfg("llama70b", layers=2), 2, 64, 64),
}


@pytest.mark.parametrize("case", list(STACKS))
def test_stack_full_size_graph_equals_eager(case):
    """Full layer shapes in the launch configuration bench.py times (a HIP graph per step):
    the graph and eager runs agree bit for bit, the output is finite, and the first layer's
    union count is the oracle's up to the neurons inside its exclusion band."""
    cfg, nl, T, B = STACKS[case]
    _say(f"stack {case}: {nl} layers d={cfg.d} ffn={cfg.ffn} B={B}")
    layers = [make_layer(cfg, i, device="cuda") for i in range(nl)]
    X = make_tokens(cfg, T, device="cuda", stream=99)
    ctx = make_ctx(layers, max_batch=B)
    ffns = [pi.Ffn(ctx, L) for L in layers]
    outs, logs = [], []
    for use_graph in (True, False):
        y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
        nlog = torch.zeros((T // B, nl), dtype=torch.int32, device="cuda")
        pi.stack_run(ctx, ffns, X, B, y, nlog, use_graph=use_graph)
        outs.append(y)
        logs.append(nlog)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "graph and eager runs differ"
    assert torch.equal(logs[0], logs[1])
    assert torch.all(torch.isfinite(outs[0]))
    H0 = layers[0].to_host()
    for s in range(T // B):
        xh = X[s * B:(s + 1) * B].cpu().numpy()
        v = oracle.decision_values(H0, xh)
        u = oracle.union(oracle.threshold(v, H0["threshold"]))
        nb = int(oracle.union(oracle.band(v, H0["threshold"])).sum())
        got = int(logs[0][s, 0].item())
        assert abs(got - int(u.sum())) <= nb, (got, int(u.sum()), nb)
