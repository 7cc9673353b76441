"""Float64 reference of the decoder's forward and gradients (plain PyTorch
autograd on the CPU). Written from the model definition alone - pre-norm
RMSNorm without a final norm, half-split rotary positions, causal softmax
attention, SwiGLU, untied or tied tables, mean cross-entropy (MojoLearn 162M
model card, comparison table) - and independent of the oracle's reduction
orders. It pins the oracle's mathematics: the oracle must agree with it to
the tolerances a binary32 computation allows.
"""
from __future__ import annotations

import numpy as np
import torch


def layout(cfg):
    """(name, shape) of every parameter in checkpoint order, written out here
    from the model definition: the input table [V, d]; per layer the attention
    norm gain [d], Wq, Wk, Wv, Wo [d, d], the MLP norm gain [d], Wg, Wu [F, d],
    Wd [d, F]; the output table [V, d] unless it is tied to the input table.
    Linear weights are [out_features, in_features]."""
    V, d, F = cfg["vocab"], cfg["d_model"], cfg["ffn_hidden"]
    out = [("E_in", (V, d))]
    for l in range(cfg["n_layers"]):
        out.append((f"l{l}.attn_norm", (d,)))
        out += [(f"l{l}.W{x}", (d, d)) for x in "qkvo"]
        out.append((f"l{l}.mlp_norm", (d,)))
        out += [(f"l{l}.Wg", (F, d)), (f"l{l}.Wu", (F, d)), (f"l{l}.Wd", (d, F))]
    if not cfg["tied"]:
        out.append(("W_out", (V, d)))
    return out


def unpack(cfg, flat):
    out, o = {}, 0
    for name, shape in layout(cfg):
        n = int(np.prod(shape))
        out[name] = flat[o:o + n].reshape(shape)
        o += n
    return out


def rope64(x, T, hd, theta):
    # x [B, T, H, hd]
    h2 = hd // 2
    i = torch.arange(h2, dtype=torch.float64)
    inv = theta ** (-(2.0 * i) / hd)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    c, s = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    x0, x1 = x[..., :h2], x[..., h2:]
    return torch.cat([x0 * c - x1 * s, x1 * c + x0 * s], dim=-1)


def loss64(cfg, flat, inputs, targets):
    p = unpack(cfg, flat)
    B, T = inputs.shape
    d, H, hd, eps = cfg["d_model"], cfg["n_heads"], cfg["head_dim"], cfg["rms_eps"]
    ids = torch.as_tensor(inputs, dtype=torch.long)
    h = p["E_in"][ids]                                           # [B, T, d]

    def rms(x, w):
        return x / torch.sqrt((x * x).mean(-1, keepdim=True) + eps) * w

    mask = torch.ones(T, T, dtype=torch.bool).tril()
    for l in range(cfg["n_layers"]):
        xn = rms(h, p[f"l{l}.attn_norm"])
        q = (xn @ p[f"l{l}.Wq"].T).view(B, T, H, hd)
        k = (xn @ p[f"l{l}.Wk"].T).view(B, T, H, hd)
        v = (xn @ p[f"l{l}.Wv"].T).view(B, T, H, hd)
        q, k = rope64(q, T, hd, cfg["rope_theta"]), rope64(k, T, hd, cfg["rope_theta"])
        s = torch.einsum("bihc,bjhc->bhij", q, k) / np.sqrt(hd)
        s = s.masked_fill(~mask, float("-inf"))
        a = torch.softmax(s, dim=-1)
        o = torch.einsum("bhij,bjhc->bihc", a, v).reshape(B, T, d)
        h = h + o @ p[f"l{l}.Wo"].T
        xn2 = rms(h, p[f"l{l}.mlp_norm"])
        g = xn2 @ p[f"l{l}.Wg"].T
        u = xn2 @ p[f"l{l}.Wu"].T
        h = h + (torch.nn.functional.silu(g) * u) @ p[f"l{l}.Wd"].T
    Wout = p["E_in"] if cfg["tied"] else p["W_out"]
    logits = h @ Wout.T
    return torch.nn.functional.cross_entropy(logits.reshape(B * T, -1),
                                             torch.as_tensor(targets, dtype=torch.long).reshape(-1))


def loss_and_grad(cfg, params32, inputs, targets):
    flat = torch.tensor(np.asarray(params32, dtype=np.float64), requires_grad=True)
    loss = loss64(cfg, flat, inputs, targets)
    loss.backward()
    return float(loss.detach()), flat.grad.numpy()
