"""The pages' attention modules computed in bf16 by PyTorch (CPU autograd):
a yardstick for the gradient tolerance, not an oracle.

"Differential Transformer V2" article, DiffAttnV1 and DiffAttnV2 pseudo-code,
run the way a bf16 model runs them: every tensor op in bf16 (PyTorch's CPU
kernels accumulate matrix products and reductions in fp32 and round each
result to bf16), lambda computed in fp32 and cast to the activation dtype
(Wilsontomass's module in the nanoGPT issue "How best to implement a
differential transformer?").  The error of these gradients against the fp64
oracle says what bf16 arithmetic costs the method on a given input; the GPU
gradients may be off by at most twice as much (the form flash-attention's own
tests use).  Dense T x T maps: small sizes only.
"""
import math

import torch


def _causal_softmax(S, softmax1):
    T = S.shape[-1]
    S = S.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    if softmax1:  # one more logit 0 (Hacker News item 41780844), dropped after the softmax
        S = torch.cat([S, torch.zeros_like(S[..., :1])], dim=-1)
        return torch.softmax(S, dim=-1)[..., :-1]
    return torch.softmax(S, dim=-1)


def v2_grads(q, k, v, lam, dout, softmax1=False):
    """Gradients (dq, dk, dv, dlam) of sum(dout * out) for DiffAttnV2 in bf16;
    q [B,T,Hq,d], k, v [B,T,Hkv,d], lam [B,T,Hq/2] logits, dout [B,T,Hq/2,d]."""
    q, k, v = [t.detach().cpu().to(torch.bfloat16).requires_grad_(True) for t in (q, k, v)]
    lam = lam.detach().cpu().to(torch.bfloat16).requires_grad_(True)
    d = q.shape[-1]
    G = q.shape[2] // k.shape[2]
    qh = q.transpose(1, 2)                                   # [B,Hq,T,d]
    kh = k.repeat_interleave(G, dim=2).transpose(1, 2)
    vh = v.repeat_interleave(G, dim=2).transpose(1, 2)
    P = _causal_softmax(torch.matmul(qh, kh.transpose(-1, -2).contiguous()) / math.sqrt(d), softmax1)
    attn = torch.matmul(P, vh).transpose(1, 2)               # [B,T,Hq,d]
    out = attn[:, :, 0::2] - torch.sigmoid(lam)[..., None] * attn[:, :, 1::2]
    (out.float() * dout.detach().cpu().float()).sum().backward()
    return q.grad, k.grad, v.grad, lam.grad


def v1_grads(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer, dout, softmax1=False):
    """Gradients of sum(dout * out) for DiffAttnV1 in bf16 (q*, k* [B,H,T,d],
    v [B,H,T,2d], lambda vectors fp32 [d]); returns the nine gradients in the
    order of the inputs."""
    ts = [t.detach().cpu().to(torch.bfloat16).requires_grad_(True) for t in (q1, q2, k1, k2, v)]
    ls = [t.detach().cpu().float().requires_grad_(True) for t in (lq1, lk1, lq2, lk2)]
    q1, q2, k1, k2, v = ts
    d = q1.shape[-1]
    li = 0.8 - 0.6 * math.exp(-0.3 * layer)
    lam = (torch.exp((ls[0] * ls[1]).sum()) - torch.exp((ls[2] * ls[3]).sum()) + li).to(torch.bfloat16)
    a = []
    for q, k in ((q1, k1), (q2, k2)):
        P = _causal_softmax(torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(d), softmax1)
        a.append(torch.matmul(P, v))                         # [B,H,T,2d]
    D = a[0] - lam * a[1]
    y = D * torch.rsqrt((D * D).mean(-1, keepdim=True) + 1e-5) * (1.0 - li)
    (y.transpose(1, 2).float() * dout.detach().cpu().float()).sum().backward()
    return [t.grad for t in ts] + [t.grad for t in ls]
