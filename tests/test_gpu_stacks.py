"""Whole stacks as bench.py times them, checked layer by layer against the fp64 oracle.

The stacks are built by bench.py's own builder (seeded weights, hot-first permutation,
chaining vectors for the step's batch size) and fed the bench's token stream. One run of
pi_stack_run_dump records every layer's input, mask words, index list, count and output;
its final outputs are checked to equal, bit for bit, those of the HIP-graph run bench.py
times. Each checked layer is then compared with the oracle teacher-forced on the layer's
recorded input (per layer: predict, skip the inactive neurons, compute the active ones;
page "PowerInfer: Mesin Inferensi LLM Cepat dengan GPU Konsumen", section «Fase Online»):
masks bit exact outside the exclusion band, index lists and counts exact, y within the
tolerance of the weight type, and the chaining into the next layer within 2 * tol + 1e-3.
"""
import gc
import sys

import numpy as np
import pytest
import torch

import bench
from synth import CONFIGS, make_tokens
from tests.parity_util import TOL, check_dump_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import activation_sparse_ffn_layer_amd as pi


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bench_tokens(cfg, B, T):
    """The first T timed tokens of bench.py (after its 8 warm-up steps)."""
    X = make_tokens(cfg, 8 * B + T, device="cuda", stream=12345)
    return X[8 * B:].contiguous()


def _run(name, B, T, check_layers, mask_mode="union"):
    cfg = CONFIGS[name]
    _say(f"stack {name}: {cfg.layers} layers d={cfg.d} ffn={cfg.ffn} B={B} tokens={T}")
    ctx = pi.Context(max_batch=B, max_d=cfg.d, max_ffn=cfg.ffn, max_rank=max(cfg.layer_rank(0.2), 8))
    ctx.set_mask_mode(mask_mode)
    layers, ffns = bench.build_stack(cfg, 0, pi, ctx, batch=B, mask_mode=mask_mode)
    nl = len(layers)
    X = _bench_tokens(cfg, B, T)
    S = T // B
    xdt = torch.float32 if cfg.wtype == "f32" else torch.float16
    stride = max(L.ffn for L in layers)
    dx = torch.zeros((S, nl, B, cfg.d), dtype=xdt, device="cuda")
    dm = torch.zeros((S, nl, B, stride // 64), dtype=torch.int64, device="cuda")
    di = torch.full((S, nl, stride), -1, dtype=torch.int32, device="cuda")
    dn = torch.full((S, nl), -1, dtype=torch.int32, device="cuda")
    dy = torch.zeros((S, nl, B, cfg.d), dtype=torch.float32, device="cuda")
    y_dump = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    n_dump = torch.zeros((S, nl), dtype=torch.int32, device="cuda")
    pi.stack_run_dump(ctx, ffns, X, B, y_dump, n_dump, x=dx, mask=dm, idx=di, n=dn, y=dy, ffn_stride=stride)
    y_graph = torch.empty_like(y_dump)
    n_graph = torch.zeros_like(n_dump)
    pi.stack_run(ctx, ffns, X, B, y_graph, n_graph, use_graph=True)
    torch.cuda.synchronize()
    assert torch.equal(y_dump, y_graph), "the recorded run and the graph run bench.py times differ"
    assert torch.equal(n_dump, n_graph) and torch.equal(n_dump, dn)
    assert torch.equal(dy[:, -1].reshape(T, cfg.d), y_graph), "recorded last-layer y differs from y_out"
    assert torch.equal(dx[:, 0].reshape(T, cfg.d), X), "recorded first-layer input differs from the tokens"
    dump = {"x": dx.cpu().numpy(), "mask": dm.cpu().numpy(), "idx": di.cpu().numpy(), "n": dn.cpu().numpy(),
            "y": dy.cpu().numpy()}
    unions = dn.float().mean(dim=0).cpu().numpy() / cfg.ffn
    profiles = [L.p for L in layers]
    del dx, dm, di, dy
    bands = flips = 0
    for li in check_layers:
        H = layers[li].to_host()
        nxt = dump["x"][:, li + 1] if li + 1 < nl else None
        nb, nf = check_dump_layer(H, dump, li, TOL[cfg.wtype], next_x=nxt)
        bands += nb
        flips += nf
        _say(f"  layer {li}: rank {H['rank']} hot_prefix {H['hot_prefix']} mean union {unions[li]:.4f} "
             f"band {nb} decided differently {nf}")
        del H
    _say(f"  {name} B={B}: {len(check_layers)} layers checked; band neurons {bands}, decided differently {flips}")
    del layers, ffns, ctx
    gc.collect()
    torch.cuda.empty_cache()
    return unions, profiles


@pytest.mark.timeout(900)
def test_opt67b_b1_every_layer():
    _run("opt6.7b", 1, 8, list(range(32)))


@pytest.mark.timeout(900)
def test_falcon40b_b1_hot_first_with_rank512_layers():
    cfg = CONFIGS["falcon40b"]
    from synth import layer_mean
    r512 = [i for i in range(cfg.layers) if cfg.layer_rank(layer_mean(cfg, i)) == 512]
    extra = [i for i in r512 if i >= 8][:3]
    assert len(extra) == 3
    _run("falcon40b", 1, 2, list(range(8)) + extra + [cfg.layers - 1])


@pytest.mark.timeout(900)
def test_llama70b_b1_first_and_last_layers():
    _run("llama70b", 1, 2, [0, 1, 2, 3, 78, 79])


@pytest.mark.timeout(900)
def test_llama70b_b64_first_and_last_layers():
    _run("llama70b", 64, 64, [0, 1, 2, 3, 78, 79])


@pytest.mark.timeout(900)
def test_opt175b_b1_first_and_last_layers():
    _run("opt175b", 1, 2, [0, 1, 2, 3, 94, 95])


@pytest.mark.timeout(900)
def test_opt175b_b8_first_and_last_layers_and_union():
    """At batch 8 the tokens stay independent through all 96 layers: the union of the
    predicted masks stays near its closed form (about 0.43 of the neurons)."""
    unions, profiles = _run("opt175b", 8, 8, [0, 1, 2, 3, 94, 95])
    import math
    import scipy.special as sp
    cfg = CONFIGS["opt175b"]
    expect = np.array([np.mean(1.0 - (1.0 - sp.ndtr(sp.ndtri(p) / math.sqrt(1.0 + cfg.noise_var))) ** 8)
                       for p in profiles])
    _say(f"  union per layer: min {unions.min():.3f} mean {unions.mean():.3f} max {unions.max():.3f}; "
         f"closed form {expect.mean():.3f}")
    dev = np.abs(unions - expect)
    assert dev.max() < 0.06 and abs(unions.mean() - expect.mean()) < 0.03, (dev.max(), unions.mean(), expect.mean())
