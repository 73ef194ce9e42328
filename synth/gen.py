"""Seeded synthetic inputs for the activation-sparse FFN: weights, predictor, tokens.

This module only *draws* inputs. It holds none of the FFN arithmetic (no
predictor evaluation, no thresholding, no compaction, no dequantisation, no
activation); both the HIP path and the fp64 oracle consume the arrays it
returns. Large matrices are drawn with ``torch`` on the requested device so a
full-size stack can be generated in device memory; small per-neuron vectors
are drawn with numpy on the host.

Recipe (one layer of one workload):

* Activation profile: a power law over a seeded random neuron order.
  Neuron ``order[k-1]`` gets rank ``k`` (1-based) and activation probability
  ``p = clip(c * k**-alpha, 0.005, 0.95)``, with ``c`` bisected so that
  ``mean(p)`` is the layer's target mean active fraction. PowerInfer reports
  that neuron activations follow a power law: a few hot neurons fire across
  inputs and many cold ones are input dependent (page "Tüketici sınıfı GPU
  takılı PC'lerde yüksek hızlı büyük dil modeli serving", section «PowerInfer'in
  çözmeye çalıştığı sorun»).
* Bias of the masked projection: ``b_i = Phi^-1(p_i)``. With weight rows of
  variance 1/d and x ~ N(0, 1), ``w_i . x`` is close to N(0, 1), so
  P(w_i . x + b_i > 0) is p_i.
* Masked projection with a low-rank predictor of rank r, built so that the
  predictor logit is the true pre-activation plus independent noise of
  variance s2: ``W1 ~ N(0, 1/d) [r][d]`` and ``W2 ~ N(0, (1 + s2)/r) [ffn][r]``
  (both stored fp16) give logit rows ``p_i = (W2 W1)_i``. The masked row is
  ``w_i = p_i / (1 + s2) + e_i`` with ``e_i`` a Gaussian direction made
  orthogonal to ``p_i`` and scaled to ``|e_i|^2 = s2 |p_i|^2 / (1 + s2)^2``.
  Then ``n_i = p_i - w_i`` is orthogonal to ``w_i`` with ``|n_i|^2`` close to
  s2 and ``|w_i|^2`` close to 1, so for x ~ N(0, I) the logit
  ``p_i . x + b_i = (w_i . x + b_i) + n_i . x`` is the pre-activation plus
  noise N(0, s2) independent of it. The predictor bias is ``b`` itself.
* Every other weight element is N(0, 1/d). ReLU layers mask the up
  projection; ReGLU layers mask the gate (which carries the bias) and leave
  the up projection bias-free. The down projection is drawn neuron-major
  (``w_down_t[i]`` is neuron i's output column).
* Q4_0 storage: see :func:`quantize_q4_0`.
* Tokens: x ~ N(0, 1), stored fp16 (fp32 for fp32 workloads).
* Chaining vector of a stack: ``glue_center = sum_i E[a_i] * w_down_t[i]`` (fp32 [d], from
  the drawn down weights before storage rounding), the layer's expected output. It is
  subtracted before the next layer's normalisation, which removes the component that every
  token's y shares, so that deep ReLU stacks keep their tokens' inputs independent.
  E[a_i] is taken for x ~ N(0, I): the pre-activation is ``h ~ N(b_i, sh_i^2)`` and the
  predictor logit ``h + n`` with independent ``n ~ N(0, sn_i^2)``, where by the construction
  above ``sh_i^2 = |p_i|^2 / (1 + s2)`` and ``sn_i^2 = |p_i|^2 s2 / (1 + s2)`` (without a
  predictor, ``sh_i`` is the drawn row's norm and the mask is h > 0). A token's activation
  counts where its own logit is positive, and in a batch of B tokens under the union also
  where another token's is (probability ``1 - (1 - q_i)^(B-1)``, ``q_i = P(h + n > 0)``):
  ``E[a] = E[f(h) P(n > -h)] + E[f(h) P(n <= -h)] (1 - (1 - q)^(B-1))`` with f the ReLU or
  its square, by quadrature over h. ReGLU layers have none (their gate and up rows are drawn
  independently, so the expected activation is zero). The vector therefore depends on the
  batch size and masking the stack is run with (``make_layer``'s ``chain_batch`` and
  ``chain_mode``).
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import scipy.special as sp
import torch

from .configs import P_MAX, P_MIN, StackConfig

# Tensor ids within a (workload, layer) seed namespace.
_T_ORDER, _T_MEAN, _T_W1, _T_W2, _T_E, _T_UP, _T_DOWN, _T_PLAIN = range(8)
_T_TOKENS = 100


def seed_of(master: int, workload: int, layer: int, tensor: int) -> int:
    """63-bit seed for one tensor, from numpy's SeedSequence spawn tree."""
    ss = np.random.SeedSequence(master, spawn_key=(workload, layer, tensor))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def np_rng(master: int, workload: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_of(master, workload, layer, tensor)))


def torch_gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------------------------------------
# activation profile
# --------------------------------------------------------------------------------------------

def _clipped_powerlaw(base: np.ndarray, c: float) -> np.ndarray:
    return np.clip(c * base, P_MIN, P_MAX)


def powerlaw_profile(ffn: int, alpha: float, mean: float, rng: Optional[np.random.Generator]) -> np.ndarray:
    """Per-neuron activation probability p (float64 [ffn]).

    With ``rng`` None the neurons are in rank order (neuron 0 hottest)."""
    if not (P_MIN < mean < P_MAX):
        raise ValueError("mean active fraction out of range")
    rank = np.arange(1, ffn + 1, dtype=np.float64)
    base = rank ** (-alpha)
    lo, hi = 0.0, 1.0
    while _clipped_powerlaw(base, hi).mean() < mean:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _clipped_powerlaw(base, mid).mean() < mean:
            lo = mid
        else:
            hi = mid
    p_by_rank = _clipped_powerlaw(base, 0.5 * (lo + hi))
    if rng is None:
        return p_by_rank
    order = rng.permutation(ffn)          # neuron order[k] has rank k+1
    p = np.empty(ffn, dtype=np.float64)
    p[order] = p_by_rank
    return p


def expected_relu_mass(p: np.ndarray) -> np.ndarray:
    """E[max(h, 0)] for h ~ N(mu, 1) with P(h > 0) = p, i.e. mu = Phi^-1(p).

    Closed form mu*Phi(mu) + phi(mu). Used only to calibrate the profile exponent."""
    mu = sp.ndtri(p)
    return mu * sp.ndtr(mu) + np.exp(-0.5 * mu * mu) / math.sqrt(2.0 * math.pi)


def expected_top_share(p: np.ndarray, top_fraction: float) -> float:
    """Share of expected activation mass carried by the most frequently active neurons."""
    order = np.argsort(-p, kind="stable")
    mass = expected_relu_mass(p)[order]
    k = int(math.ceil(top_fraction * p.size))
    return float(mass[:k].sum() / mass.sum())


def chain_activation(b, sh, sn, act: str, batch: int, mode: str = "union", points: int = 801) -> torch.Tensor:
    """E[a_i] of each neuron for x ~ N(0, I) (input-side calibration of the chaining vector).

    ``h ~ N(b, sh^2)``; ``sn`` the predictor noise std (None: no predictor, mask h > 0).
    Under the union of a batch of ``batch`` tokens a neuron a token does not predict itself
    still counts when another token predicts it. Quadrature over h on +-8 sh, in float64 on
    the device of ``sh`` (torch tensors or arrays)."""
    sh = torch.as_tensor(sh, dtype=torch.float64)
    dev = sh.device
    b = torch.as_tensor(b, dtype=torch.float64, device=dev)
    if act == "reglu":
        return torch.zeros_like(b)
    g = torch.linspace(-8.0, 8.0, points, dtype=torch.float64, device=dev)
    wq = torch.exp(-0.5 * g * g) / math.sqrt(2.0 * math.pi) * (g[1] - g[0])
    h = b[:, None] + sh[:, None] * g[None, :]
    f = torch.clamp_min(h, 0.0)
    if act == "sqrelu":
        f = f * f
    elif act != "relu":
        raise ValueError(act)
    if sn is None:
        return (f * wq).sum(dim=1)
    sn = torch.as_tensor(sn, dtype=torch.float64, device=dev)
    pv = torch.special.ndtr(h / sn[:, None])                      # P(logit > 0 | h)
    own = (f * pv * wq).sum(dim=1)
    if mode == "per_token" or batch <= 1:
        return own
    other = (f * (1.0 - pv) * wq).sum(dim=1)
    q = (pv * wq).sum(dim=1)
    return own + other * (1.0 - (1.0 - q) ** (batch - 1))


@functools.lru_cache(maxsize=None)
def solve_alpha(top_fraction: float, share: float, ffn: int, mean: float) -> float:
    """Power-law exponent at which the top ``top_fraction`` of neurons carry ``share`` of the mass."""
    lo, hi = 0.05, 4.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        s = expected_top_share(powerlaw_profile(ffn, mid, mean, None), top_fraction)
        if s < share:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


# --------------------------------------------------------------------------------------------
# Q4_0 storage
# --------------------------------------------------------------------------------------------

def quantize_q4_0(w: torch.Tensor, chunk_rows: int = 2048, values: bool = False):
    """Quantise rows of ``w`` [rows][d] (d % 32 == 0) to Q4_0 storage.

    Per block of 32 consecutive elements of a row: scale ``s = fp16(absmax / 8)``
    (round to nearest even) and codes ``q = clamp(rint(w / s) + 8, 0, 15)``
    (ties to even, the quotient taken in float64 with the fp16-rounded s); an
    all-zero block has s = 0 and every code 8. Storage is struct-of-arrays:
    codes ``uint8 [rows][d/32][16]`` where byte j of a block holds element j in
    its low nibble and element j + 16 in its high nibble, and scales
    ``float16 [rows][d/32]``. The stored value of an element is (q - 8) * s.

    With ``values`` also returns, as fp32 ``[rows][d]``, the value each code was chosen
    to stand for, (q - 8) * s, taken from the quantiser's own rounding (before the codes
    are packed). The generator uses it only to calibrate the chaining vector; the kernels
    and the oracle decode the packed codes themselves.
    """
    rows, d = w.shape
    if d % 32:
        raise ValueError("Q4_0 needs d % 32 == 0")
    nb = d // 32
    codes = torch.empty((rows, nb, 16), dtype=torch.uint8, device=w.device)
    scales = torch.empty((rows, nb), dtype=torch.float16, device=w.device)
    vals = torch.empty((rows, d), dtype=torch.float32, device=w.device) if values else None
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        blk = w[r0:r1].reshape(r1 - r0, nb, 32).to(torch.float64)
        s16 = (blk.abs().amax(dim=-1) / 8.0).to(torch.float16)
        s64 = s16.to(torch.float64).unsqueeze(-1)
        safe = torch.where(s64 > 0, s64, torch.ones_like(s64))
        q = torch.where(s64 > 0, torch.round(blk / safe) + 8.0, torch.full_like(blk, 8.0))
        q = q.clamp_(0.0, 15.0)
        if values:
            vals[r0:r1] = ((q - 8.0) * s64).reshape(r1 - r0, d).to(torch.float32)
        q = q.to(torch.uint8)
        codes[r0:r1] = q[..., :16] | (q[..., 16:] << 4)
        scales[r0:r1] = s16
    if values:
        return codes, scales, vals
    return codes, scales


# --------------------------------------------------------------------------------------------
# layers and tokens
# --------------------------------------------------------------------------------------------

@dataclass
class Layer:
    """One FFN layer as stored for the kernels (all tensors on one device).

    ``w_up``/``w_gate``/``w_down_t`` are ``[ffn][d]`` neuron-major (fp32, fp16),
    or Q4_0 codes ``uint8 [ffn][d/32][16]`` with fp16 scales ``s_*``.
    ``b`` is the bias of the masked projection (up for ReLU, gate for ReGLU).
    """
    d: int
    ffn: int
    rank: int
    act: str
    wtype: str
    threshold: float
    w_up: torch.Tensor
    w_gate: Optional[torch.Tensor]
    w_down_t: torch.Tensor
    s_up: Optional[torch.Tensor]
    s_gate: Optional[torch.Tensor]
    s_down: Optional[torch.Tensor]
    b: torch.Tensor
    p_w1: Optional[torch.Tensor]
    p_w2: Optional[torch.Tensor]
    p_b: Optional[torch.Tensor]
    p: np.ndarray          # activation probability profile (host)
    mean: float
    alpha: float
    glue_center: Optional[torch.Tensor] = None   # fp32 [d] chaining vector, None for ReGLU
    hot_prefix: int = 0    # stored neurons [0, hot_prefix) taken without a prediction

    def tensors(self):
        return {k: getattr(self, k) for k in ("w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down",
                                              "b", "p_w1", "p_w2", "p_b", "glue_center")}

    def to_host(self) -> dict:
        """Plain numpy copy of every stored array plus the scalar fields."""
        out = {k: (None if v is None else v.detach().cpu().numpy()) for k, v in self.tensors().items()}
        out.update(d=self.d, ffn=self.ffn, rank=self.rank, act=self.act, wtype=self.wtype,
                   threshold=self.threshold, hot_prefix=self.hot_prefix)
        return out

    def nbytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.tensors().values() if v is not None)


def _randn(shape, std, seed, device):
    g = torch_gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std)


def layer_mean(cfg: StackConfig, layer: int, master: int = 0) -> float:
    lo, hi = cfg.mean_active
    if lo == hi:
        return lo
    return float(np_rng(master, cfg.index, layer, _T_MEAN).uniform(lo, hi))


def make_layer(cfg: StackConfig, layer: int, master: int = 0, device="cpu", chain_batch: int = 1,
               chain_mode: str = "union") -> Layer:
    """One seeded layer of ``cfg``. ``chain_batch`` / ``chain_mode``: the batch size and masking
    (union or per_token) the stack will run with, which its chaining vector is computed for."""
    d, ffn = cfg.d, cfg.ffn
    mean = layer_mean(cfg, layer, master)
    if cfg.alpha is not None:
        alpha = cfg.alpha
    else:
        alpha = solve_alpha(cfg.mass_share[0], cfg.mass_share[1], ffn, mean)
    p = powerlaw_profile(ffn, alpha, mean, np_rng(master, cfg.index, layer, _T_ORDER))
    b = torch.from_numpy(sp.ndtri(p).astype(np.float32)).to(device)
    r = cfg.layer_rank(mean)
    sd = 1.0 / math.sqrt(d)
    s = lambda t: seed_of(master, cfg.index, layer, t)  # noqa: E731

    p_w1 = p_w2 = p_b = None
    if r > 0:
        s2 = cfg.noise_var
        p_w1 = _randn((r, d), sd, s(_T_W1), device).to(torch.float16)
        p_w2 = _randn((ffn, r), math.sqrt((1.0 + s2) / r), s(_T_W2), device).to(torch.float16)
        w_mask = _randn((ffn, d), sd, s(_T_E), device)
        w1f = p_w1.to(torch.float32)
        step = 4096
        for r0 in range(0, ffn, step):
            pr = p_w2[r0:r0 + step].to(torch.float32) @ w1f            # logit rows
            e = w_mask[r0:r0 + step]
            pn2 = (pr * pr).sum(dim=1, keepdim=True)
            e.sub_(pr * ((e * pr).sum(dim=1, keepdim=True) / pn2))     # orthogonal to the logit row
            e.mul_(torch.sqrt(s2 * pn2 / (1.0 + s2) ** 2 / (e * e).sum(dim=1, keepdim=True)))
            e.add_(pr, alpha=1.0 / (1.0 + s2))
            del pr, pn2
        del w1f
        p_b = b.clone()
    else:
        w_mask = _randn((ffn, d), sd, s(_T_UP), device)
    w_down = _randn((ffn, d), sd, s(_T_DOWN), device)
    w_plain = _randn((ffn, d), sd, s(_T_PLAIN), device) if cfg.act == "reglu" else None
    chain = cfg.act != "reglu"

    def store(w, values=False):
        """Stored form (weights, Q4_0 scales) and, with ``values``, what it stands for in fp32."""
        if w is None:
            return None, None, None
        if cfg.wtype == "f32":
            return w, None, (w if values else None)
        if cfg.wtype == "f16":
            h = w.to(torch.float16)
            return h, None, (h.to(torch.float32) if values else None)
        if cfg.wtype == "q4_0":
            if values:
                return quantize_q4_0(w, values=True)
            return (*quantize_q4_0(w), None)
        raise ValueError(cfg.wtype)

    m_w, m_s, m_val = store(w_mask, chain)
    del w_mask
    dn_w, dn_s, dn_val = store(w_down, chain)
    del w_down
    pl_w, pl_s, _ = store(w_plain)
    del w_plain
    glue_center = None
    if chain:
        # spreads of the stored masked rows' pre-activation and of the predictor's noise
        sig_h = torch.sqrt((m_val * m_val).sum(dim=1))
        sig_n = None
        if r > 0:
            w1f = p_w1.to(torch.float32)
            sig_n = torch.empty(ffn, dtype=torch.float32, device=device)
            for r0 in range(0, ffn, 4096):
                nr = p_w2[r0:r0 + 4096].to(torch.float32) @ w1f - m_val[r0:r0 + 4096]
                sig_n[r0:r0 + 4096] = torch.sqrt((nr * nr).sum(dim=1))
                del nr
            del w1f
        ea = chain_activation(torch.from_numpy(sp.ndtri(p)).to(device), sig_h, sig_n, cfg.act, chain_batch,
                              chain_mode).to(torch.float32)
        glue_center = (ea.unsqueeze(0) @ dn_val).squeeze(0).contiguous()
        del ea, sig_h, sig_n
    del m_val, dn_val
    if cfg.act in ("relu", "sqrelu"):
        up, s_up, gate, s_gate = m_w, m_s, None, None
    elif cfg.act == "reglu":
        up, s_up, gate, s_gate = pl_w, pl_s, m_w, m_s
    else:
        raise ValueError(cfg.act)
    return Layer(d=d, ffn=ffn, rank=r, act=cfg.act, wtype=cfg.wtype, threshold=0.0,
                 w_up=up, w_gate=gate, w_down_t=dn_w, s_up=s_up, s_gate=s_gate, s_down=dn_s,
                 b=b, p_w1=p_w1, p_w2=p_w2, p_b=p_b, p=p, mean=mean, alpha=alpha, glue_center=glue_center)


def make_tokens(cfg: StackConfig, count: int, master: int = 0, device="cpu", stream: int = 0) -> torch.Tensor:
    """``count`` tokens x ~ N(0, 1) of width d: fp16, or fp32 for fp32 workloads."""
    x = _randn((count, cfg.d), 1.0, seed_of(master, cfg.index, stream, _T_TOKENS), device)
    return x if cfg.wtype == "f32" else x.to(torch.float16)


def make_decision_values(batch: int, ffn: int, seed: int, special: bool = True) -> np.ndarray:
    """Synthetic fp32 decision values ``[batch][ffn]`` for the threshold/compaction entry.

    Mostly N(-1.2, 1) (about 11% above zero) with runs of exact +0, -0, the
    smallest positive and negative subnormals and normals, +-inf, and all-zero
    / all-positive 64-neuron words mixed in when ``special`` is set."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.normal(-1.2, 1.0, size=(batch, ffn)).astype(np.float32)
    if special and ffn >= 64:
        tiny = np.array([0.0, -0.0, 1e-45, -1e-45, 1.1754944e-38, -1.1754944e-38, np.inf, -np.inf,
                         2.0 ** -20, -(2.0 ** -20)], dtype=np.float32)
        for t in range(batch):
            pos = rng.choice(ffn, size=min(ffn // 8, 4 * tiny.size), replace=False)
            v[t, pos] = rng.choice(tiny, size=pos.size)
            w = rng.integers(0, ffn // 64)
            v[t, 64 * w:64 * w + 64] = -1.0          # an all-inactive word
            w = rng.integers(0, ffn // 64)
            v[t, 64 * w:64 * w + 64] = 1.0           # an all-active word
    return v
