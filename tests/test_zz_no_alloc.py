"""pi_layer_noalloc, the entry point for callers that cannot allocate device memory: no
context, its scratch the library's fixed device array. Checked against pi_layer on a context
(bitwise: the same kernels on the same inputs) and against the fp64 oracle (masks exact
outside the exclusion band, y within the weight type's tolerance), on two calls in a row,
the second with a smaller layer and batch, so the second runs on the array the first left."""
import dataclasses
import sys

import pytest
import torch

from synth import CONFIGS, make_layer, make_tokens
from tests.parity_util import TOL, check_layer, make_ctx, run_layer

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import activation_sparse_ffn_layer_amd as pi


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _noalloc(L, x, with_outputs=True):
    B = x.shape[0]
    y = torch.full((B, L.d), float("nan"), dtype=torch.float32, device="cuda")
    if not with_outputs:
        pi.layer_noalloc(L, x, y)
        return {"y": y}
    mask = torch.zeros((B, L.ffn // 64), dtype=torch.int64, device="cuda")
    idx = torch.full((L.ffn,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    pi.layer_noalloc(L, x, y, mask, idx, n)
    return {"y": y, "mask": mask, "idx": idx, "n": n}


CALLS = [
    # (config, layer id, batch): the first call is the larger one
    (dataclasses.replace(CONFIGS["opt175b"], d=12288, ffn=8192, rank=1024), 0, 8),
    (dataclasses.replace(CONFIGS["opt6.7b"], d=1024, ffn=4096, rank=512), 1, 1),
]


def test_noalloc_layer_equals_layer_on_two_calls():
    for k, (cfg, li, B) in enumerate(CALLS):
        _say(f"no-alloc call {k}: d={cfg.d} ffn={cfg.ffn} rank={cfg.rank} {cfg.wtype} B={B}")
        L = make_layer(cfg, li, device="cuda")
        x = make_tokens(cfg, B, device="cuda", stream=40 + k)
        got = _noalloc(L, x)
        torch.cuda.synchronize()
        ctx = make_ctx([L], max_batch=8)
        want = run_layer(ctx, pi.Ffn(ctx, L), x)
        n = int(want["n"].item())
        assert int(got["n"].item()) == n
        assert torch.equal(got["mask"], want["mask"]), "mask words differ from pi_layer's"
        assert torch.equal(got["idx"][:n], want["idx"][:n]), "index list differs from pi_layer's"
        assert torch.equal(got["y"], want["y"]), "y differs from pi_layer's"
        check_layer(L.to_host(), x.cpu().numpy(), got, TOL[cfg.wtype])
        # without the optional outputs (the fixed array holds them)
        y_only = _noalloc(L, x, with_outputs=False)
        torch.cuda.synchronize()
        assert torch.equal(y_only["y"], want["y"])


def test_noalloc_rejects_sizes_beyond_its_array():
    cfg = dataclasses.replace(CONFIGS["opt6.7b"], d=1024, ffn=2048, rank=512)
    L = make_layer(cfg, 0, device="cuda")
    x = make_tokens(cfg, 9, device="cuda")
    y = torch.empty((9, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(pi.PiError, match="unsupported"):
        pi.layer_noalloc(L, x, y)                                   # 9 tokens > 8
    wide = dataclasses.replace(L, d=16384)
    with pytest.raises(pi.PiError, match="unsupported"):
        pi.layer_noalloc(wide, x[:1].contiguous(), y[:1])           # d above 12288 (host check)
    with pytest.raises(pi.PiError, match="invalid argument"):
        pi.layer_noalloc(dataclasses.replace(L, ffn=2000), x[:1].contiguous(), y[:1])
