#!/usr/bin/env python
"""Sparse-FFN decode throughput on one MI355X.

A step is one pass of the whole hot path over one batch: every layer of the stack runs the
low-rank predictor, the threshold and compaction, the gathered up/gate rows with their
activation and the scattered down columns, chained layer to layer by the centred rms glue.
The default workload is the largest: the OPT-175B-shaped stack (96 ReLU layers, d=12288,
ffn=49152, Q4_0 weights, rank-1024 fp16 predictor) at batch 1, with seeded synthetic weights
and tokens resident in HBM before timing starts.

Prints one JSON line: tokens/s over the timed steps, a roofline entry for the kernel that
takes the most time (algorithmic bytes per launch over its HIP-event-timed duration, against
MI355X's 8 TB/s), and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import dataclasses
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-FFN tokens/s at batch 1 (layer stack) + % of HBM peak on active bytes"
HBM_PEAK_GBS = 8000.0
WBYTES = {"f32": 4.0, "f16": 2.0, "q4_0": 18.0 / 32.0}
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
COPY_CAL_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed steps (one batch through the stack each)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="opt175b")
    ap.add_argument("--batch", type=int, default=None, help="tokens per step (default: the workload's first batch)")
    ap.add_argument("--layers", type=int, default=None, help="override the stack depth (exploration only)")
    ap.add_argument("--act", choices=["relu", "reglu", "sqrelu"], default=None,
                    help="override the workload's activation family (e.g. the Squared-ReLU variant)")
    ap.add_argument("--mask", choices=["union", "per_token"], default="union",
                    help="masking of a batch: the union of the tokens' masks, or each token's own")
    ap.add_argument("--hot-prefix", default="0",
                    help="stored neurons of every layer taken without a prediction: a count, or 'auto' "
                         "for the count the bytes model picks per layer (hot-first layouts)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--profile-steps", type=int, default=16, help="steps of the per-kernel event pass")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (3 times), the reference for HBM counters")
    return ap.parse_args()


def kernel_source_hash():
    """Hash of the HIP sources; a recorded counter reading is used only while it matches."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "activation_sparse_ffn_layer_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:12]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` on ``workload`` from the FETCH_SIZE/WRITE_SIZE table
    in profiles/, scaled by the plain-copy calibration; None when absent or taken on other
    kernel sources."""
    try:
        with open(TRAFFIC_TABLE, encoding="utf-8") as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    src = kernel_source_hash()
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 8 and cells[0] == workload and cells[1] == kernel and cells[2] == src:
            try:
                return float(cells[7])
            except ValueError:
                return None
    return None


def stream_read_gbs():
    """Achievable HBM read rate of this GPU: the library GEMV of a 2 GiB fp16 matrix with a
    vector (torch matmul -> rocBLAS; it reads each matrix byte once), best of 5, timed with
    events. On MI355X this reads at about 5.9 TB/s, where torch's own sum of the same bytes
    reaches about 4.0 TB/s."""
    import torch
    m = torch.ones((131072, 8192), dtype=torch.float16, device="cuda")  # 2 GiB
    v = torch.ones((8192, 1), dtype=torch.float16, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    m @ v
    torch.cuda.synchronize()
    for _ in range(5):
        e0.record()
        m @ v
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del m, v
    torch.cuda.empty_cache()
    return (1 << 31) / best / 1e9


def calibrate_copy():
    """A device-to-device copy of exactly 1 GiB, three times: reads and writes 1 GiB each."""
    import torch
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {COPY_CAL_BYTES} bytes 3 times")


def hot_prefix_auto(L, B):
    """Hot-prefix length that minimises a layer's expected bytes (hot-first layouts): a prefix
    neuron saves its predictor row (2r bytes) but reads its up (gate) and down rows whether it
    fires or not; a predicted neuron reads them with probability q_B = 1 - (1 - q)^B, q its
    predicted-active probability Phi(mu / sqrt(1 + s2)). The prefix is the longest run from
    the hottest neuron over which the cumulative saving keeps growing."""
    import numpy as np
    if L.rank <= 0:
        return 0
    c = np.cumsum(hot_prefix_gain(L, B))
    h = int(np.argmax(c)) + 1
    return h if c[h - 1] > 0 else 0


def hot_prefix_gain(L, B):
    """Expected bytes a prefix saves per neuron, in stored (hot-first) order: its predictor row
    (2r bytes) less its up (gate) and down rows, read even when it would not have fired."""
    import scipy.special as sp
    from synth import NOISE_VAR
    q = sp.ndtr(sp.ndtri(L.p) / math.sqrt(1.0 + NOISE_VAR))
    qb = 1.0 - (1.0 - q) ** B
    k = 3 if L.act == "reglu" else 2
    rows = k * L.d * WBYTES[L.wtype]
    return 2.0 * L.rank - (1.0 - qb) * rows


def build_stack(cfg, seed, pi, ctx, batch=1, mask_mode="union", hot_prefix="0"):
    """Generate every layer in device memory; hot-first workloads are permuted on the device.
    Each layer's chaining vector is computed for ``batch`` tokens per step under ``mask_mode``."""
    import torch
    from synth import make_layer
    layers, ffns, tables = [], [], []
    for li in range(cfg.layers):
        L = make_layer(cfg, li, master=seed, device="cuda", chain_batch=batch, chain_mode=mask_mode)
        table = None
        if cfg.hot_first:
            perm = torch.from_numpy(pi.hot_first_order(L.p)).cuda()

            def pr(t):
                if t is None:
                    return None
                out = torch.empty_like(t)
                pi.permute_rows(ctx, t, out, perm)
                return out
            L = dataclasses.replace(L, w_up=pr(L.w_up), w_gate=pr(L.w_gate), w_down_t=pr(L.w_down_t),
                                    s_up=pr(L.s_up), s_gate=pr(L.s_gate), s_down=pr(L.s_down), b=pr(L.b),
                                    p_w2=pr(L.p_w2), p_b=pr(L.p_b), p=L.p[perm.cpu().numpy()])
            table = perm
        if hot_prefix != "0" and L.rank > 0:
            hp = hot_prefix_auto(L, batch) if hot_prefix == "auto" else min(int(hot_prefix), L.ffn)
            L = dataclasses.replace(L, hot_prefix=hp)
        layers.append(L)
        tables.append(table)
        ffns.append(pi.Ffn(ctx, L, neuron_table=table))
        if li % 8 == 7:
            torch.cuda.synchronize()
            log(f"  generated {li + 1}/{cfg.layers} layers")
    torch.cuda.synchronize()
    return layers, ffns


def up_cols(L, B):
    """Whether the library runs the up GEMV as its own kernel (k_up_cols) rather than in stage 2
    for this predictor layer and batch of 1..8 tokens: x (padded to the batch class 1/2/4/8)
    above 64 KiB, Q4_0 rows, d >= 8192, or 5..8 tokens."""
    nb = 1 if B <= 1 else 2 if B <= 2 else 4 if B <= 4 else 8
    big_x = nb * L.d * (4 if L.wtype == "f32" else 2) > 65536
    return B <= 8 and L.rank > 0 and (big_x or L.wtype == "q4_0" or L.d >= 8192 or nb >= 8)


def kernel_bytes(cls, L, B, n_list):
    """Algorithmic bytes moved by the launches of one kernel class on one layer.

    n_list: active (union) counts of the launches. Batches above 8 tokens run the matrix-core
    path, whose stage-2 and true-mask kernels do not include the activations."""
    w = WBYTES[L.wtype]
    xe = 4 if L.wtype == "f32" else 2
    d, F, r = L.d, L.ffn, L.rank
    k_up = 2 if L.act == "reglu" else 1
    if B > 8:
        if cls == "stage1":
            return len(n_list) * (r * d * 2 + B * d * 2 + B * r * 4)
        if cls == "stage2":  # the matrix-core stage 2 reads every predictor row
            return len(n_list) * (F * r * 2 + F * 4 + B * r * 4 + (B + 1) * F / 8)
        if cls == "truemask":
            return len(n_list) * (F * d * 2 + F * 4 + B * d * 2 + (B + 1) * F / 8)
        if cls == "up":
            return sum(n * (k_up * d * 2 + 4 + 4 + 2 * B) + B * d * 2 for n in n_list)
        if cls == "down":
            return sum(n * (d * 2 + 4 + 2 * B) for n in n_list)
        raise KeyError(cls)
    if cls == "stage1":
        return len(n_list) * (r * d * 2 + B * d * xe + B * r * 4)
    up_rows = lambda n: n * (k_up * d * w + 4 + 4 * B)  # noqa: E731  (rows, bias, a written)
    Fp = F - getattr(L, "hot_prefix", 0)  # neurons with a prediction (predictor rows read)
    if cls == "stage2" and up_cols(L, B):  # predictor stage 2 + threshold only
        return len(n_list) * (Fp * r * 2 + Fp * 4 + B * r * 4 + (B + 1) * F / 8)
    if cls == "stage2":  # predictor stage 2 + threshold + own active neurons' up (gate) rows
        return sum(Fp * r * 2 + Fp * 4 + B * r * 4 + (B + 1) * F / 8 + B * d * xe + up_rows(n) for n in n_list)
    if cls == "truemask":  # threshold GEMV + (ReGLU) own active neurons' up rows
        extra = (lambda n: up_rows(n)) if L.act == "reglu" else (lambda n: n * 4 * B)  # noqa: E731
        return sum(F * d * w + F * 4 + B * d * xe + (B + 1) * F / 8 + extra(n) for n in n_list)
    if cls == "up":
        return sum(up_rows(n) + 4 * n + B * d * xe for n in n_list)
    if cls == "down":  # active down rows, their a and the index list (partial sums are overhead)
        return sum(n * (d * w + 4 + 4 * B) + (B + 1) * F / 8 for n in n_list)
    raise KeyError(cls)


def step_bytes(layers, B, nlog_rows):
    """Algorithmic bytes of every step: predictor (or true-mask GEMV), active rows and the
    small vectors, from the measured union counts (nlog_rows[step][layer])."""
    total = 0.0
    for row in nlog_rows:
        for L, n in zip(layers, row):
            if L.rank > 0:
                total += kernel_bytes("stage1", L, B, [n]) + kernel_bytes("stage2", L, B, [n])
            else:
                total += kernel_bytes("truemask", L, B, [n])
            if B > 8 or up_cols(L, B):
                total += kernel_bytes("up", L, B, [n])
            total += kernel_bytes("down", L, B, [n])
    return total


def cpu_model():
    """The host CPU's model name (lscpu), or /proc/cpuinfo's, or None."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().startswith("Model name:"):
                return ln.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, layers, x_tokens, B, budget_s, mask_mode="union"):
    """The fp64 oracle, as it stands, on a bounded sample: one batch of B tokens chained
    through the stack (union or per-token masking, like the GPU step) until the time budget
    runs out. Layers are copied to the host one at a time as the oracle reaches them (not timed)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    x = x_tokens[:B].cpu().numpy()
    done = 0
    elapsed = 0.0
    for L in layers:
        H = L.to_host()
        t0 = time.perf_counter()
        r = oracle.layer_forward(H, x)
        y = oracle.per_token_ffn(H, x, r["mask"]) if mask_mode == "per_token" else r["y"]
        x = oracle.glue(y, x, H["glue_center"])
        elapsed += time.perf_counter() - t0
        done += 1
        del H
        if elapsed >= budget_s:
            break
    frac = done / len(layers)
    return {"value": B * frac / elapsed, "unit": "tokens/s", "cores": int(threads), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"one batch of {B} token(s) through {done} of the {len(layers)} layers "
                      f"({frac:.3f} of a step) in {elapsed:.1f} s of fp64 numpy compute, scaled to a whole "
                      f"step; weight copies to host not timed"}


def main():
    args = parse()
    if args.gpus != 1:
        log(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).")
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch
    import activation_sparse_ffn_layer_amd as pi
    from synth import CONFIGS, make_tokens

    cfg = CONFIGS[args.config]
    if args.layers:
        cfg = dataclasses.replace(cfg, layers=args.layers)
    if args.act:
        cfg = dataclasses.replace(cfg, act=args.act)
    B = args.batch if args.batch else cfg.batches[0]
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    max_rank = max(cfg.layer_rank(0.2), 8)
    ctx = pi.Context(max_batch=B, max_d=cfg.d, max_ffn=cfg.ffn, max_rank=max_rank)
    ctx.set_mask_mode(args.mask)
    log(f"generating {cfg.layers} layers of {cfg.name} on the GPU")
    t0 = time.perf_counter()
    layers, ffns = build_stack(cfg, args.seed, pi, ctx, batch=B, mask_mode=args.mask, hot_prefix=args.hot_prefix)
    log(f"  {sum(L.nbytes() for L in layers) / 1e9:.2f} GB of weights in {time.perf_counter() - t0:.1f} s")
    T_w, T = args.warmup * B, args.steps * B
    X = make_tokens(cfg, T_w + T, master=args.seed, device="cuda", stream=12345)
    xw, xt = X[:T_w].contiguous(), X[T_w:].contiguous()
    y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    yw = torch.empty((max(T_w, B), cfg.d), dtype=torch.float32, device="cuda")
    nlog = torch.zeros((args.steps, cfg.layers), dtype=torch.int32, device="cuda")
    use_graph = not args.no_graph
    if T_w:
        pi.stack_run(ctx, ffns, xw, B, yw[:T_w], None, use_graph=use_graph)
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    pi.stack_run(ctx, ffns, xt, B, y, nlog, use_graph=use_graph)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed_s = max(wall, gpu_ms / 1e3)
    ms_per_step = elapsed_s * 1e3 / args.steps
    value = T / elapsed_s
    nl = nlog.cpu().numpy()
    active_bytes = step_bytes(layers, B, nl.tolist())
    frac_active = active_bytes / elapsed_s / (HBM_PEAK_GBS * 1e9)
    log(f"timed: {args.steps} steps in {elapsed_s * 1e3:.2f} ms ({value:.1f} tok/s), "
        f"{active_bytes / args.steps / 1e6:.1f} MB/step, {100 * frac_active:.1f}% of HBM peak on active bytes")

    # per-kernel event pass on the first timed tokens
    ps = min(args.profile_steps, args.steps)
    nprof = torch.zeros((ps, cfg.layers), dtype=torch.int32, device="cuda")
    yp = torch.empty((ps * B, cfg.d), dtype=torch.float32, device="cuda")
    prof = pi.stack_profile(ctx, ffns, xt[:ps * B].contiguous(), B, yp, nprof)
    npl = nprof.cpu().numpy()
    kb = {}
    for cls in ("stage1", "stage2", "truemask", "up", "down"):
        tot = 0.0
        for li, L in enumerate(layers):
            if (cls in ("stage1", "stage2") and L.rank == 0) or (cls == "truemask" and L.rank > 0):
                continue
            if cls == "up" and B <= 8 and not up_cols(L, B):
                continue
            tot += kernel_bytes(cls, L, B, npl[:, li].tolist())
        kb[cls] = tot
    # the reduction of the down partials moves no algorithmic bytes: it is reported, not ranked
    dom = max((k for k in kb if prof[k][1] > 0), key=lambda k: prof[k][0])
    for k, (ms, cnt) in prof.items():
        if cnt:
            gbs = kb.get(k, float("nan")) / (ms * 1e-3) / 1e9 if k in kb else float("nan")
            log(f"  {k:9s} {cnt:6d} launches  avg {1e3 * ms / cnt:8.2f} us  {gbs:8.1f} GB/s")
    dms, dcnt = prof[dom]
    bytes_per_launch = kb[dom] / dcnt
    achieved = bytes_per_launch / (dms / dcnt * 1e-3) / 1e9
    workload_key = f"{cfg.name} b{B}"
    traffic = recorded_traffic(workload_key, dom)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic),
                "bytes_per_launch": round(bytes_per_launch), "avg_launch_us": round(1e3 * dms / dcnt, 3)}

    stream_gbs = stream_read_gbs()
    log(f"stream read: {stream_gbs:.0f} GB/s achievable; the path moves "
        f"{active_bytes / elapsed_s / 1e9:.0f} GB/s of active bytes")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layers, xt, B, args.cpu_seconds, args.mask)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"f16": "f16", "f32": "f32", "q4_0": "q4_0+f16"}[cfg.wtype],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}-shaped {cfg.act} FFN stack, batch {B}", "layers": cfg.layers, "d": cfg.d,
                   "ffn": cfg.ffn, "rank": cfg.rank, "weights": cfg.wtype, "batch": B, "seed": args.seed,
                   "hot_first": cfg.hot_first, "graph": use_graph, "mask": args.mask,
                   "hot_prefix": int(sum(getattr(L, "hot_prefix", 0) for L in layers))},
        "hbm_frac_active": round(frac_active, 4),
        "stream_read_gbs": round(stream_gbs, 1),
        "frac_of_stream_read": round(active_bytes / elapsed_s / 1e9 / stream_gbs, 4),
        "active_mb_per_step": round(active_bytes / args.steps / 1e6, 2),
        # the bytes model's expected saving of the hot prefixes per step (hot-first layouts)
        "hot_prefix_saved_mb_per_step": round(sum(float(hot_prefix_gain(L, B)[:L.hot_prefix].sum())
                                                  for L in layers if getattr(L, "hot_prefix", 0) > 0) / 1e6, 3),
        "mean_active": round(float(nl.mean()) / cfg.ffn, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
