"""A short synthetic training run of a small transformer whose linears are FP4: BF16 vs vanilla
FP4 vs Averis.

The model is a decoder-only transformer (pre-norm RMSNorm blocks, causal multi-head attention,
SwiGLU feed-forward), the shape of a Qwen3 block at small width.  Every linear of every block --
q, k, v, o, gate, up, down -- is the W4A4G4 autograd linear of `autograd.py` (forward, input
gradient and weight gradient all FP4 GEMMs in the HIP library, with or without the mean-residual
split); the embedding, the norms, the attention scores and softmax, and the output head stay in
torch (fp32 attention on contiguous operands).  The data are token sequences of a fixed random
sparse Markov chain (each token has a few likely successors), so the achievable loss is the
chain's entropy rate; the model learns next-token prediction by cross-entropy with AdamW.

The explainer (section 实验结果) reports that the split narrows FP4 training's loss gap to
BF16 on real pre-training; this synthetic run has no dataset and no pretrained weights and
claims no parity with those numbers: it shows the layer working inside a transformer's
training loop and lets one compare the three variants' loss curves qualitatively.

    python -m fp4_quantized_amd.transformer_demo [steps]
"""
from __future__ import annotations

import math
import sys

import torch
import torch.nn.functional as F

from . import averis as av
from .autograd import averis_linear


class Linear(torch.nn.Module):
    """y = x W (W [in, out] fp32 master weight), as a bf16 matmul or the FP4 autograd linear."""

    def __init__(self, d_in, d_out, mode, fmt, gen, device):
        super().__init__()
        self.w = torch.nn.Parameter(torch.randn(d_in, d_out, generator=gen, device=device) * d_in ** -0.5)
        self.mode, self.fmt = mode, fmt

    def forward(self, x):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).to(torch.bfloat16)
        w = self.w.to(torch.bfloat16)
        if self.mode == "bf16":
            y = x2 @ w
        else:
            y = averis_linear(x2, w, self.fmt, split=self.mode == "averis")
        return y.reshape(*lead, -1)


class Block(torch.nn.Module):
    def __init__(self, d, heads, ffn, mode, fmt, gen, device):
        super().__init__()
        mk = lambda i, o: Linear(i, o, mode, fmt, gen, device)  # noqa: E731
        self.q, self.k, self.v, self.o = mk(d, d), mk(d, d), mk(d, d), mk(d, d)
        self.gate, self.up, self.down = mk(d, ffn), mk(d, ffn), mk(ffn, d)
        self.n1 = torch.nn.Parameter(torch.ones(d, device=device))
        self.n2 = torch.nn.Parameter(torch.ones(d, device=device))
        self.heads = heads

    @staticmethod
    def rms(x, g):
        x = x.float()
        return x * torch.rsqrt(x.square().mean(-1, keepdim=True) + 1e-6) * g

    def forward(self, x):
        b, s, d = x.shape
        h = self.rms(x, self.n1)
        q, k, v = (f(h).float().view(b, s, self.heads, -1).transpose(1, 2).contiguous() for f in (self.q, self.k, self.v))
        att = (q @ k.transpose(-1, -2).contiguous()) / math.sqrt(q.shape[-1])
        mask = torch.ones(s, s, dtype=torch.bool, device=x.device).triu(1)
        att = att.masked_fill(mask, float("-inf")).softmax(-1)
        a = (att @ v).transpose(1, 2).reshape(b, s, d)
        x = x + self.o(a).float()
        h = self.rms(x, self.n2)
        return x + self.down(F.silu(self.gate(h).float()) * self.up(h).float()).float()


class TinyLM(torch.nn.Module):
    def __init__(self, vocab, d, heads, ffn, layers, seq, mode, fmt=av.MXFP4, seed=0, device="cuda"):
        super().__init__()
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        self.emb = torch.nn.Parameter(torch.randn(vocab, d, generator=g, device=device) * 0.5)
        self.pos = torch.nn.Parameter(torch.randn(seq, d, generator=g, device=device) * 0.1)
        self.blocks = torch.nn.ModuleList([Block(d, heads, ffn, mode, fmt, g, device) for _ in range(layers)])
        self.nf = torch.nn.Parameter(torch.ones(d, device=device))
        self.head = torch.nn.Parameter(torch.randn(d, vocab, generator=g, device=device) * d ** -0.5)

    def forward(self, tok):
        x = self.emb[tok] + self.pos[: tok.shape[1]]
        for blk in self.blocks:
            x = blk(x)
        return Block.rms(x, self.nf) @ self.head


def markov_chain(vocab, fanout=4, seed=1, device="cuda"):
    """Transition matrix of a random sparse chain: each token's successors are `fanout` random
    tokens with Zipf(1) weights.  Returns (P [vocab, vocab], entropy rate in nats)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    P = torch.zeros(vocab, vocab, device=device)
    w = 1.0 / torch.arange(1, fanout + 1, device=device, dtype=torch.float32)
    w = w / w.sum()
    for t in range(vocab):
        succ = torch.randperm(vocab, generator=g, device=device)[:fanout]
        P[t, succ] = w
    # stationary distribution by power iteration, then the entropy rate
    pi = torch.full((vocab,), 1.0 / vocab, device=device)
    for _ in range(200):
        pi = pi @ P
    ent = -(P * torch.log(P.clamp_min(1e-30))).sum(1)
    return P, float((pi * ent).sum())


def sample_batch(P, batch, seq, gen):
    vocab = P.shape[0]
    tok = torch.empty(batch, seq + 1, dtype=torch.long, device=P.device)
    tok[:, 0] = torch.randint(0, vocab, (batch,), generator=gen, device=P.device)
    for i in range(seq):
        tok[:, i + 1] = torch.multinomial(P[tok[:, i]], 1, generator=gen).squeeze(1)
    return tok[:, :-1], tok[:, 1:]


def run(mode, fmt=av.MXFP4, steps=200, vocab=512, d=512, heads=8, ffn=1536, layers=2, batch=16, seq=256,
        lr=3e-3, pool=64, device="cuda"):
    """Train one variant ('bf16', 'vanilla' or 'averis') on a pool of `pool` batches, cycled.
    Returns (training losses, held-out loss on 4 unseen batches, entropy rate of the chain)."""
    P, h = markov_chain(vocab, device=device)
    model = TinyLM(vocab, d, heads, ffn, layers, seq, mode, fmt, device=device)
    opt = torch.optim.AdamW(model.parameters(), lr=lr, weight_decay=0.0)
    gen = torch.Generator(device=device)
    gen.manual_seed(7)
    data = [sample_batch(P, batch, seq, gen) for _ in range(pool)]
    held = [sample_batch(P, batch, seq, gen) for _ in range(4)]
    losses = []
    for it in range(steps):
        x, y = data[it % len(data)]
        logits = model(x)
        loss = F.cross_entropy(logits.float().reshape(-1, vocab), y.reshape(-1))
        opt.zero_grad(set_to_none=True)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    with torch.no_grad():
        ev = sum(float(F.cross_entropy(model(x).float().reshape(-1, vocab), y.reshape(-1))) for x, y in held) / 4
    return losses, ev, h


def main(steps=300):
    rows = []
    for name, mode, fmt in (("bf16", "bf16", av.MXFP4), ("MXFP4 vanilla", "vanilla", av.MXFP4),
                            ("MXFP4 Averis", "averis", av.MXFP4), ("NVFP4 vanilla", "vanilla", av.NVFP4),
                            ("NVFP4 Averis", "averis", av.NVFP4)):
        ls, ev, h = run(mode, fmt, steps)
        tail = sum(ls[-20:]) / 20
        rows.append((name, ls[0], tail, ev, h))
        print(f"{name:14s} cross-entropy: first {ls[0]:.3f}, last 20 steps {tail:.3f}, held-out {ev:.3f} "
              f"(entropy rate {h:.3f}, log vocab {math.log(512):.3f})", flush=True)
    return rows


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 300)
