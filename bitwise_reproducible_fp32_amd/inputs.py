"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module only draws numbers: model shapes, initial parameters, token ids,
uniform test matrices and the learning-rate table. It holds none of the
training step's arithmetic, so both sides of every parity check receive the
same input bytes and compute everything else on their own.

Workloads (stand-ins for data the pages use but do not publish):
  * c0 - the two-block byte-level LM (mojolearn project page, "Handing training
    off between vendors": 34,944 FP32 parameters, real text). The text is
    replaced by an order-2 Markov source over 256 byte values.
  * c3 - a 6-layer, d=384 decoder with untied 50,257-entry tables.
  * c4 - the 162,147,840-parameter decoder of the MojoLearn 162M model card
    ("Compared with GPT-3 Small" and "Training" tables). FineWeb-Edu BPE ids are
    replaced by i.i.d. truncated Zipf(1.1) ids over 50,257 entries.
Initial parameters follow the model card's "Training" table: N(0, 0.02) for
matrices and tables, 1 + N(0, 0.02) for norm gains, drawn with NumPy's
default_rng tensor by tensor in checkpoint order (float64, then cast).
"""
from __future__ import annotations

import math

import numpy as np

CONFIGS = {
    "c0": dict(vocab=256, d_model=32, n_layers=2, n_heads=4, head_dim=8, ffn_hidden=96,
               tied=1, batch=8, seq_len=64, micro=1),
    "c3": dict(vocab=50257, d_model=384, n_layers=6, n_heads=6, head_dim=64, ffn_hidden=1024,
               tied=0, batch=4, seq_len=1024, micro=4),
    "c4": dict(vocab=50257, d_model=768, n_layers=12, n_heads=12, head_dim=64, ffn_hidden=2048,
               tied=0, batch=4, seq_len=2048, micro=64),
}
HYPER = dict(rope_theta=10000.0, rms_eps=1e-6, beta1=0.9, beta2=0.95, adam_eps=1e-8,
             weight_decay=0.1)
INIT_SEED = 93261


def make_config(name: str | None = None, **over) -> dict:
    """A full model config (shape + hyper-parameters) from a preset and overrides."""
    cfg = dict(CONFIGS[name]) if name else {}
    cfg.update(HYPER)
    cfg.update(over)
    return cfg


def param_shapes(cfg: dict) -> list[tuple[str, tuple[int, ...], str]]:
    """(name, shape, kind) in canonical checkpoint order; kind is 'table' or 'gain'."""
    V, d, F = cfg["vocab"], cfg["d_model"], cfg["ffn_hidden"]
    out = [("E_in", (V, d), "table")]
    for l in range(cfg["n_layers"]):
        out += [(f"l{l}.attn_norm", (d,), "gain"), (f"l{l}.Wq", (d, d), "table"),
                (f"l{l}.Wk", (d, d), "table"), (f"l{l}.Wv", (d, d), "table"),
                (f"l{l}.Wo", (d, d), "table"), (f"l{l}.mlp_norm", (d,), "gain"),
                (f"l{l}.Wg", (F, d), "table"), (f"l{l}.Wu", (F, d), "table"),
                (f"l{l}.Wd", (d, F), "table")]
    if not cfg["tied"]:
        out.append(("W_out", (V, d), "table"))
    return out


def param_count(cfg: dict) -> int:
    return sum(int(np.prod(s)) for _, s, _ in param_shapes(cfg))


def init_params(cfg: dict, seed: int = INIT_SEED) -> np.ndarray:
    """Step-0 parameters as one flat float32 array in canonical order."""
    rng = np.random.default_rng(seed)
    parts = []
    for _, shape, kind in param_shapes(cfg):
        x = rng.normal(0.0, 0.02, size=shape)
        if kind == "gain":
            x = 1.0 + x
        parts.append(x.astype(np.float32).ravel())
    return np.concatenate(parts)


# ------------------------------------------------------------------ token data
def markov_bytes(n: int, seed: int = 1) -> np.ndarray:
    """n bytes from a seeded order-2 Markov source: each context (a, b) has 8
    successors drawn uniformly with Dirichlet(1) weights."""
    rng = np.random.default_rng(seed)
    succ = rng.integers(0, 256, size=(256, 256, 8))
    w = rng.dirichlet(np.ones(8), size=(256, 256))
    cw = np.cumsum(w, axis=2)
    out = np.empty(n, dtype=np.int32)
    start = rng.integers(0, 256, size=2)
    out[0], out[1] = start[0], start[1]
    u = rng.random(n)
    for t in range(2, n):
        a, b = out[t - 2], out[t - 1]
        k = int(np.searchsorted(cw[a, b], u[t], side="right"))
        out[t] = succ[a, b, min(k, 7)]
    return out


_MARKOV_CACHE: dict[int, np.ndarray] = {}


def c0_batch(step: int, batch: int = 8, seq_len: int = 64) -> tuple[np.ndarray, np.ndarray]:
    """Step `step` (0-based) of the byte LM: windows batch*step .. batch*step+batch-1
    of a non-overlapping split of the Markov stream into seq_len+1 bytes."""
    need = (batch * (step + 1)) * (seq_len + 1)
    n = 1 << max(16, math.ceil(math.log2(need)))
    if n not in _MARKOV_CACHE:
        _MARKOV_CACHE[n] = markov_bytes(n)
    s = _MARKOV_CACHE[n][: need].reshape(-1, seq_len + 1)[batch * step: batch * (step + 1)]
    return np.ascontiguousarray(s[:, :-1]), np.ascontiguousarray(s[:, 1:])


def zipf_cdf(vocab: int, alpha: float = 1.1) -> np.ndarray:
    k = np.arange(vocab, dtype=np.float64)
    p = (k + 1.0) ** (-alpha)
    c = np.cumsum(p)
    return c / c[-1]


_ZIPF_CACHE: dict[tuple[int, float], np.ndarray] = {}


def zipf_ids(count: int, vocab: int, seed, alpha: float = 1.1) -> np.ndarray:
    """i.i.d. truncated Zipf ids, P(k) proportional to (k+1)^-alpha for k < vocab,
    by binary64 inverse CDF."""
    key = (vocab, alpha)
    if key not in _ZIPF_CACHE:
        _ZIPF_CACHE[key] = zipf_cdf(vocab, alpha)
    u = np.random.default_rng(seed).random(count)
    ids = np.searchsorted(_ZIPF_CACHE[key], u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def zipf_batch(cfg: dict, micro_index: int) -> tuple[np.ndarray, np.ndarray]:
    """Micro-batch `micro_index` (0-based over the whole run): batch windows of
    seq_len+1 Zipf ids from default_rng([5, micro_index])."""
    B, T = cfg["batch"], cfg["seq_len"]
    w = zipf_ids(B * (T + 1), cfg["vocab"], [5, micro_index]).reshape(B, T + 1)
    return np.ascontiguousarray(w[:, :-1]), np.ascontiguousarray(w[:, 1:])


def batch_for(name: str, cfg: dict, step: int, micro: int) -> tuple[np.ndarray, np.ndarray]:
    """Inputs/targets for 1-based optimizer step `step`, micro-batch `micro`."""
    if name == "c0":
        return c0_batch(step - 1, cfg["batch"], cfg["seq_len"])
    return zipf_batch(cfg, (step - 1) * cfg["micro"] + micro)


def lr_at(name: str, t: int) -> float:
    """Learning rate of 1-based step t, rounded to binary32. The byte LM uses a
    constant 1e-3; c3/c4 use the model card's 250-step linear warmup to 6e-4
    followed by a cosine decay to 6e-5 at step 5,000 (binary64, then rounded)."""
    if name == "c0":
        return float(np.float32(1e-3))
    peak, floor, warm, total = 6e-4, 6e-5, 250, 5000
    if t <= warm:
        lr = peak * t / warm
    else:
        prog = (t - warm) / (total - warm)
        lr = floor + 0.5 * (peak - floor) * (1.0 + math.cos(math.pi * prog))
    return float(np.float32(lr))


def uniform(shape, seed: int = 7) -> np.ndarray:
    """float32 uniform(-1, 1) test data."""
    return np.random.default_rng(seed).uniform(-1.0, 1.0, size=shape).astype(np.float32)
