"""Seeded synthetic inputs shaped like the workloads of the Averis paper's experiments.

This module holds no step of the method: it only draws numbers.  The same bytes feed the
HIP path and the CPU oracle.  The data stands in for Qwen3 activations and output gradients
during DCLM pre-training, which are not available here; it imitates the structure the pages
describe: a coherent rank-one column mean shared by all tokens, a few channels where the mean
dominates the largest entries, and SwiGLU-style non-odd nonlinear inputs
("均值偏置的诅咒与祝福" explainer, paper.rainbus.top, sections 核心方法 and 实验结果;
gist.science German summary, Technische Zusammenfassung §2).

Every tensor is drawn in fp64 from numpy.random.default_rng(SeedSequence(seed)) with child
streams in a fixed order, then rounded once to fp32 and, for bf16 tensors, from fp32 to bf16
with round-to-nearest-even.  Arrays are returned as numpy fp32 (the exact values of the
bf16 tensors) plus a `dtype` tag; `to_torch` produces the tensor the GPU receives.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Qwen3-0.6B-shaped linears at l = 16384 tokens: (name, m = in features, n = out features).
SWEEP_LAYERS = [
    ("q", 1024, 2048),
    ("k", 1024, 1024),
    ("v", 1024, 1024),
    ("o", 2048, 1024),
    ("gate", 1024, 3072),
    ("up", 1024, 3072),
    ("down", 3072, 1024),
]


@dataclass
class Linear:
    """One linear layer's inputs: X [l, m], D [l, n], W [m, n] (pages' orientation Y = X W)."""
    name: str
    x: np.ndarray
    w: np.ndarray
    d: np.ndarray | None
    dtype: str  # "f32" or "bf16": the element type handed to the GPU
    meta: dict = field(default_factory=dict)


def _round(a, dtype):
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return a32
    # fp32 -> bf16, round to nearest even, on the bit pattern (finite inputs only)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def _mean_vector(rng, m, target_rms, n_spikes, spike=20.0):
    g = rng.standard_normal(m)
    mu = target_rms * g / np.sqrt(np.mean(g * g))
    idx = rng.choice(m, size=n_spikes, replace=False) if n_spikes else np.zeros(0, int)
    mu[idx] *= spike
    return mu


def _n_spikes(m):
    return max(1, int(round(0.001 * m)))


def _grad(rng, l, n, dtype):
    """D = 1 mu_D^T + E, E ~ N(0, 1e-6) (std 1e-3), RMS(mu_D) = the residual RMS."""
    e = rng.standard_normal((l, n)) * 1e-3
    mu_d = _mean_vector(rng, n, 1e-3, 0)
    return _round(e + mu_d[None, :], dtype)


def tiny(seed=0):
    """Forward-only check case: X fp32 [256, 128] = 1 mu^T + R, mu_j ~ N(0, 16), R ~ N(0, 1);
    W fp32 [128, 128] ~ N(0, 0.02^2)."""
    ss = np.random.SeedSequence(seed)
    r_mu, r_r, r_w = [np.random.default_rng(s) for s in ss.spawn(3)]
    mu = r_mu.standard_normal(128) * 4.0
    r = r_r.standard_normal((256, 128))
    w = r_w.standard_normal((128, 128)) * 0.02
    return Linear("tiny", _round(mu[None, :] + r, "f32"), _round(w, "f32"), None, "f32")


def up_proj_like(seed, l, m, n, dtype="bf16", name="up_proj"):
    """X = bf16(1 mu^T + R): R ~ Student-t(4), mu = 3 x RMS(t4) x g / rms(g) with 0.1 % of the
    channels scaled x20; D as in `_grad`; W ~ N(0, 0.02^2) [m, n]."""
    ss = np.random.SeedSequence(seed)
    r_mu, r_r, r_d, r_w = [np.random.default_rng(s) for s in ss.spawn(4)]
    mu = _mean_vector(r_mu, m, 3.0 * np.sqrt(2.0), _n_spikes(m))
    r = r_r.standard_t(4, size=(l, m))
    x = _round(r + mu[None, :], dtype)
    d = _grad(r_d, l, n, dtype)
    w = _round(r_w.standard_normal((m, n)) * 0.02, dtype)
    return Linear(name, x, w, d, dtype)


def down_proj_like(seed, l, m, n, dtype="bf16", name="down_proj"):
    """X = bf16(silu(A) * B + 1 mu^T) with A, B ~ N(0, 1); mu as in up_proj_like with rms(R)
    measured on the draw; D and W as in up_proj_like."""
    ss = np.random.SeedSequence(seed)
    r_mu, r_a, r_b, r_d, r_w = [np.random.default_rng(s) for s in ss.spawn(5)]
    a = r_a.standard_normal((l, m))
    b = r_b.standard_normal((l, m))
    r = a / (1.0 + np.exp(-a)) * b
    del a, b
    mu = _mean_vector(r_mu, m, 3.0 * float(np.sqrt(np.mean(r * r))), _n_spikes(m))
    x = _round(r + mu[None, :], dtype)
    d = _grad(r_d, l, n, dtype)
    w = _round(r_w.standard_normal((m, n)) * 0.02, dtype)
    return Linear(name, x, w, d, dtype)


def up_proj(seed=1, l=8192):
    """Qwen3-0.6B-shaped up_proj: l = 8192 (b = 4, s = 2048), m = 1024, n = 3072, bf16."""
    return up_proj_like(seed, l, 1024, 3072)


def down_proj(seed=2, l=16384):
    """down_proj: l = 16384, m = 3072, n = 1024, bf16, SwiGLU-like input."""
    return down_proj_like(seed, l, 3072, 1024)


def sweep(seed=3, l=16384):
    """The seven Qwen3-0.6B-shaped linears at l = 16384, each drawn as up_proj_like."""
    return [up_proj_like([seed, j], l, m, n, name=nm) for j, (nm, m, n) in enumerate(SWEEP_LAYERS)]


def sweep_device(seed=3, l=16384, device="cuda"):
    """The seven sweep linears drawn directly on the device, for timing: the up_proj_like recipe
    (X = bf16(1 mu^T + R), R ~ Student-t(4) as Z / sqrt(V / 4) with V ~ chi2(4); D = bf16(1 mu_D^T
    + N(0, 1e-6)); W ~ N(0, 0.02^2)) from torch's generator seeded with `seed`.  The values are
    not those of `sweep` (a different generator); the full-size sweep parity test copies these
    draws to the oracle.
    Returns [(name, x, d, w)] of bf16 tensors, x [l, m], d [l, n], w [m, n]."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for name, m, n in SWEEP_LAYERS:
        def normal(*shape):
            return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

        def mean_vec(k, rms, spikes):
            g = normal(k)
            mu = rms * g / torch.sqrt(torch.mean(g * g))
            if spikes:
                idx = torch.randperm(k, generator=gen, device=device)[:spikes]
                mu[idx] *= 20.0
            return mu

        mu = mean_vec(m, 3.0 * 2.0 ** 0.5, _n_spikes(m))
        v = sum(normal(l, m) ** 2 for _ in range(4))
        x = (normal(l, m) / torch.sqrt(v / 4.0) + mu[None, :]).to(torch.bfloat16)
        del v
        d = (normal(l, n) * 1e-3 + mean_vec(n, 1e-3, 0)[None, :]).to(torch.bfloat16)
        w = (normal(m, n) * 0.02).to(torch.bfloat16)
        out.append((name, x, d, w))
    return out


def layer_device(seed=3, l=16384, device="cuda", shared=True, cat=False):
    """The seven linears of one Qwen3-0.6B-shaped transformer layer at l tokens, drawn on the
    device with the recipe of `sweep_device`.  shared=True: q, k and v read the same input
    X [l, 1024] and gate and up the same X [l, 1024], as in the layer (the attention and MLP
    inputs after their norms); o and down have inputs of their own.  Every linear has its own
    output gradient and weight.  cat=True (with shared): the output gradients and the weights
    of q/k/v, and those of gate/up, are adjacent column blocks of one tensor each (D [l, 4096],
    W [1024, 4096]; D [l, 6144], W [1024, 6144]), the storage of a fused projection; the values
    are the same.  Returns [(name, x, d, w)]; shared inputs are one tensor."""
    import torch
    layers = sweep_device(seed, l, device)
    if not shared:
        return layers
    x_attn, x_mlp = layers[0][1], layers[4][1]
    out = []
    for name, x, d, w in layers:
        if name in ("k", "v"):
            x = x_attn
        elif name == "up":
            x = x_mlp
        out.append((name, x, d, w))
    if cat:
        for names in (("q", "k", "v"), ("gate", "up")):
            idx = [i for i, c in enumerate(out) if c[0] in names]
            dp = torch.cat([out[i][2] for i in idx], 1)
            wp = torch.cat([out[i][3] for i in idx], 1)
            off = 0
            for i in idx:
                name, x, d, _ = out[i]
                n = d.shape[1]
                out[i] = (name, x, dp[:, off:off + n], wp[:, off:off + n])
                off += n
    return out


def activations_device(seed, l, m, device="cuda"):
    """One activation matrix X [l, m] bf16 drawn on the device with the up_proj_like recipe
    (X = bf16(1 mu^T + R), R ~ Student-t(4), spike channels x20), for timing only."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    g = normal(m)
    mu = 3.0 * 2.0 ** 0.5 * g / torch.sqrt(torch.mean(g * g))
    idx = torch.randperm(m, generator=gen, device=device)[:_n_spikes(m)]
    mu[idx] *= 20.0
    v = sum(normal(l, m) ** 2 for _ in range(4))
    x = (normal(l, m) / torch.sqrt(v / 4.0) + mu[None, :]).to(torch.bfloat16)
    return x


def activations_device_chunked(seed, l, m, device="cuda", chunk=65536):
    """activations_device for large l: the same recipe drawn in blocks of `chunk` rows (one
    mean vector for all rows), so the fp32 temporaries stay at a few blocks' size."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    g = normal(m)
    mu = 3.0 * 2.0 ** 0.5 * g / torch.sqrt(torch.mean(g * g))
    idx = torch.randperm(m, generator=gen, device=device)[:_n_spikes(m)]
    mu[idx] *= 20.0
    x = torch.empty((l, m), dtype=torch.bfloat16, device=device)
    for r0 in range(0, l, chunk):
        r1 = min(l, r0 + chunk)
        v = sum(normal(r1 - r0, m) ** 2 for _ in range(4))
        x[r0:r1] = (normal(r1 - r0, m) / torch.sqrt(v / 4.0) + mu[None, :]).to(torch.bfloat16)
        del v
    return x


def down_proj_device(seed, l, m, n, device="cuda"):
    """The down_proj_like recipe drawn on the device, for timing: X = bf16(silu(A) * B + 1 mu^T)
    with A, B ~ N(0, 1), mu as in up_proj_like with rms(R) measured on the draw; D = bf16(1 mu_D^T
    + N(0, 1e-6)); W ~ N(0, 0.02^2) [m, n].  Returns bf16 (x [l, m], d [l, n], w [m, n])."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    a = normal(l, m)
    r = torch.nn.functional.silu(a) * normal(l, m)
    del a
    g = normal(m)
    mu = 3.0 * torch.sqrt(torch.mean(r * r)) * g / torch.sqrt(torch.mean(g * g))
    idx = torch.randperm(m, generator=gen, device=device)[:_n_spikes(m)]
    mu[idx] *= 20.0
    x = (r + mu[None, :]).to(torch.bfloat16)
    del r
    gd = normal(n)
    d = (normal(l, n) * 1e-3 + (1e-3 * gd / torch.sqrt(torch.mean(gd * gd)))[None, :]).to(torch.bfloat16)
    w = (normal(m, n) * 0.02).to(torch.bfloat16)
    return x, d, w


@dataclass
class MoE:
    """Expert-contiguous MoE FFN inputs.  offsets [E+1] over the routed rows; per expert e,
    rows offsets[e]:offsets[e+1] of x_gate (token states, shared by gate and up), x_down,
    d_gateup and d_down; w_gate/w_up [E, hidden, ffn], w_down [E, ffn, hidden]."""
    offsets: np.ndarray
    x: np.ndarray
    x_down: np.ndarray
    d_gateup: np.ndarray
    d_down: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    dtype: str = "bf16"


def zipf_topk_counts(rng, tokens, experts, topk, s=1.1):
    """Distinct top-k experts per token by Gumbel-top-k over p_e ~ (e + 1)^-s.
    Returns (expert ids [tokens, topk], counts [experts])."""
    logp = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(tokens, experts))
    ids = np.argsort(-(logp[None, :] + g), axis=1)[:, :topk]
    counts = np.bincount(ids.ravel(), minlength=experts)
    return ids, counts


def moe(seed=4, tokens=8192, hidden=2048, ffn=768, experts=64, topk=8, dtype="bf16"):
    """Top-8 Zipf(1.1) routing of 8192 tokens over 64 experts; token states [tokens, hidden]
    drawn as up_proj_like, gathered per expert; the down-projection input and the output
    gradients drawn per routed row as in up_proj_like."""
    ss = np.random.SeedSequence(seed)
    r_route, r_x, r_xd, r_dg, r_dd, r_w = [np.random.default_rng(s) for s in ss.spawn(6)]
    ids, counts = zipf_topk_counts(r_route, tokens, experts, topk)
    offsets = np.zeros(experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    states = up_proj_like(r_x.integers(1 << 62), tokens, hidden, 8, dtype).x
    order = np.argsort(ids.ravel(), kind="stable")  # routed rows grouped by expert
    x = states[order // topk]
    L = int(offsets[-1])
    x_down = up_proj_like(r_xd.integers(1 << 62), L, ffn, 8, dtype).x
    d_gu = _grad(r_dg, L, ffn, dtype)
    d_dn = _grad(r_dd, L, hidden, dtype)
    w = r_w.standard_normal((3, experts, hidden, ffn)) * 0.02
    w_gate = _round(w[0], dtype)
    w_up = _round(w[1], dtype)
    w_down = _round(np.ascontiguousarray(np.swapaxes(w[2], 1, 2)), dtype)
    return MoE(offsets, x, x_down, d_gu, d_dn, w_gate, w_up, w_down, dtype)


def moe_device(seed=4, tokens=8192, hidden=2048, ffn=768, experts=64, topk=8, device="cuda"):
    """The MoE workload drawn on the device, for timing: Zipf(1.1) top-8 routing of the tokens
    (host, as in `moe`), token states drawn like `activations_device` and gathered per expert,
    the down projection's input likewise, output gradients N(0, 1e-6) plus their own mean,
    weights N(0, 0.02^2) stacked per expert.  Returns (x [L, hidden], x_down [L, ffn],
    d_gate [L, ffn], d_up [L, ffn], d_dn [L, hidden], w_gate [E * hidden, ffn],
    w_up [E * hidden, ffn], w_down [E * ffn, hidden], offsets [E + 1] host int64), bf16
    tensors; the gate and up projections have output gradients of their own."""
    import torch
    ids, counts = zipf_topk_counts(np.random.default_rng(seed), tokens, experts, topk)
    offsets = np.zeros(experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(ids.ravel(), kind="stable")
    L = int(offsets[-1])
    states = activations_device(seed * 10 + 1, tokens, hidden, device)
    x = states[torch.from_numpy(order // topk).to(device)].contiguous()
    del states
    x_down = activations_device(seed * 10 + 2, L, ffn, device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 10 + 3)

    def grad(cols):
        g = torch.randn(cols, generator=gen, device=device)
        mu = 1e-3 * g / torch.sqrt(torch.mean(g * g))
        return (torch.randn(L, cols, generator=gen, device=device) * 1e-3 + mu[None, :]).to(torch.bfloat16)

    d_gate, d_up, d_dn = grad(ffn), grad(ffn), grad(hidden)
    w = [(torch.randn(experts * r, c, generator=gen, device=device) * 0.02).to(torch.bfloat16)
         for r, c in ((hidden, ffn), (hidden, ffn), (ffn, hidden))]
    return x, x_down, d_gate, d_up, d_dn, w[0], w[1], w[2], offsets


def to_torch(a, dtype, device):
    """Hand the exact values to torch as fp32 or bf16 (no rounding: values are representable)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)
