"""Helpers shared by the GPU tests: device tensors from numpy, bit comparison
with a first-difference report, and the stage-by-stage divergence finder."""
from __future__ import annotations

import numpy as np


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def empty(n, dtype="float32"):
    import torch
    return torch.empty(int(n), dtype=getattr(torch, dtype), device="cuda")


def canon(a) -> np.ndarray:
    """Bits with every NaN mapped to one pattern: NaN payloads are not part of
    the contract (x86 and gfx950 propagate them differently)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()
    u[np.isnan(a)] = 0x7FC00000
    return u


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a, b = canon(a), canon(b)
    return a.shape == b.shape and np.array_equal(a, b)


def diff_report(name: str, got: np.ndarray, want: np.ndarray, limit: int = 5) -> str:
    g = np.ascontiguousarray(got, dtype=np.float32).ravel()
    w = np.ascontiguousarray(want, dtype=np.float32).ravel()
    if g.size != w.size:
        return f"{name}: size {g.size} != {w.size}"
    bad = np.nonzero(canon(g) != canon(w))[0]
    if bad.size == 0:
        return f"{name}: equal"
    rows = ", ".join(f"[{i}] {g[i]!r} vs {w[i]!r}" for i in bad[:limit])
    return f"{name}: {bad.size} of {g.size} differ; first {rows}"


def assert_bits(name: str, got, want) -> None:
    assert bits_equal(got, want), diff_report(name, got, want)


STAGES = [(0, "layer input"), (1, "attn norm"), (2, "attn 1/rms"), (3, "q|k|v rotated"), (4, "P"),
          (5, "attn out"), (6, "mid residual"), (7, "mlp norm"), (8, "mlp 1/rms"), (9, "g|u"),
          (10, "swiglu")]


def first_divergence(gpu_model, orc_model, cfg) -> str:
    """Walks the forward stages in order and names the first that differs."""
    T, BH = cfg["seq_len"], cfg["batch"] * cfg["n_heads"]
    for l in range(cfg["n_layers"]):
        for sid, name in STAGES:
            g, o = gpu_model.read_stage(sid, l), orc_model.stage(sid, l)
            if sid == 4:  # only j <= i is defined
                mask = np.tril(np.ones((T, T), bool))[None].repeat(BH, 0).ravel()
                g, o = g[mask], o[mask]
            if not bits_equal(g, o):
                return f"layer {l} {name}: " + diff_report(name, g, o)
    for sid, name in ((11, "final hidden"), (12, "d-logits"), (13, "row losses")):
        g, o = gpu_model.read_stage(sid, 0), orc_model.stage(sid, 0)
        if not bits_equal(g, o):
            return diff_report(name, g, o)
    return "forward stages all equal"
