"""Plain PyTorch forward pass of the decoder from a safetensors export.

This is how the trained weights run outside this library (model card,
"Anywhere else: safetensors + PyTorch"): ordinary PyTorch ops with PyTorch's
own summation orders, by default in float64. It agrees with the library's
logits only to rounding, never bit for bit, and nothing in the library calls
it; it exists to check an export and to serve the weights elsewhere.

The architecture is the one the library trains: embedding lookup; per layer
pre-norm RMSNorm (x / sqrt(mean(x^2) + eps) * gain), q/k/v projections,
rotary embedding on q and k (half-split pairs (i, i + hd/2), angle
t * theta^(-2i/hd)), causal softmax attention with scale 1/sqrt(hd), output
projection plus residual, RMSNorm, SwiGLU (silu(g) * u) and down projection
plus residual; no final norm; logits = h W_out^T (W_out = E_in when tied).
Linear weights are [out_features, in_features].
"""
from __future__ import annotations

import json
import math
import struct

import numpy as np
import torch

_META_INT = ("vocab", "d_model", "n_layers", "n_heads", "head_dim", "ffn_hidden", "tied")


def load(src) -> tuple[dict, dict]:
    """(shape metadata, {name: float32 tensor}) from a safetensors path or bytes.
    Reads the format directly: u64 header length, JSON table, raw little-endian data."""
    if isinstance(src, (bytes, bytearray, memoryview)):
        blob = bytes(src)
    else:
        with open(src, "rb") as f:
            blob = f.read()
    (n,) = struct.unpack("<Q", blob[:8])
    table = json.loads(blob[8:8 + n])
    meta = table.pop("__metadata__", {})
    data = memoryview(blob)[8 + n:]
    tensors = {}
    for name, t in table.items():
        if t["dtype"] != "F32":
            raise ValueError(f"{name}: dtype {t['dtype']}, expected F32")
        b, e = t["data_offsets"]
        a = np.frombuffer(data[b:e], dtype="<f4").reshape(t["shape"])
        tensors[name] = torch.from_numpy(a.copy())
    cfg = {k: int(meta[k]) for k in _META_INT}
    cfg["rope_theta"] = float(np.float32(meta["rope_theta"]))
    cfg["rms_eps"] = float(np.float32(meta["rms_eps"]))
    return cfg, tensors


def forward_logits(cfg: dict, tensors: dict, ids, dtype=torch.float64, device="cpu") -> torch.Tensor:
    """Logits [B, T, vocab] for token ids [B, T] (int array or tensor)."""
    d, H, hd, L = cfg["d_model"], cfg["n_heads"], cfg["head_dim"], cfg["n_layers"]
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    W = {k: v.to(device=device, dtype=dtype) for k, v in tensors.items()}
    ids = torch.as_tensor(np.asarray(ids), dtype=torch.long, device=device)
    B, T = ids.shape
    half = hd // 2
    inv = theta ** (-(2.0 * torch.arange(half, dtype=torch.float64)) / hd)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = ang.cos().to(device, dtype), ang.sin().to(device, dtype)
    causal = torch.ones(T, T, dtype=torch.bool, device=device).tril()

    def rms(x, w):
        return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * w

    def rope(t):                                   # [B, H, T, hd]
        a, b = t[..., :half], t[..., half:]
        return torch.cat([a * cos - b * sin, b * cos + a * sin], dim=-1)

    def heads(t):
        return t.view(B, T, H, hd).transpose(1, 2)

    x = W["E_in"][ids]
    for l in range(L):
        p = f"l{l}."
        xn = rms(x, W[p + "attn_norm"])
        q, k, v = (heads(xn @ W[p + w].T) for w in ("Wq", "Wk", "Wv"))
        s = (rope(q) @ rope(k).transpose(-1, -2)) / math.sqrt(hd)
        att = torch.softmax(s.masked_fill(~causal, float("-inf")), dim=-1)
        o = (att @ v).transpose(1, 2).reshape(B, T, d)
        x = x + o @ W[p + "Wo"].T
        xn = rms(x, W[p + "mlp_norm"])
        g, u = xn @ W[p + "Wg"].T, xn @ W[p + "Wu"].T
        x = x + (torch.nn.functional.silu(g) * u) @ W[p + "Wd"].T
    out = W["E_in"] if cfg["tied"] else W["W_out"]
    return x @ out.T
