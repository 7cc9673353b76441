"""Identity cards of the oracle's stages and state arrays (test side).

A card is (tag, dtype, count, SHA-256 hex) of one stage's exact bytes: the
per-stage hashes that the mojolearn PyPI page ("What bitwise identity means")
uses as the check of the identity claim. This module writes the computation
order and the tag strings out on its own, from the forward pass as the model
card describes it (pre-norm block: attention norm, q/k/v with rotary
positions, causal softmax, attention output, residual, MLP norm, SwiGLU), and
hashes with the oracle's SHA-256. It shares nothing with the library's card
code, so a wrong order or tag on either side shows up as a mismatch.
"""
from __future__ import annotations

import numpy as np

import oracle

# (oracle stage id, tag suffix) per layer in the order the forward computes them:
# the layer input, the attention norm's 1/rms then its output, rotated q|k|v,
# the probabilities, the attention output, the mid-layer residual, the MLP
# norm's 1/rms then its output, g|u, the SwiGLU output.
LAYER_STAGES = [(0, "h_in"), (2, "r1"), (1, "xn1"), (3, "qkv"), (4, "P"), (5, "O"), (6, "h_mid"),
                (8, "r2"), (7, "xn2"), (9, "gu"), (10, "a")]
# then the model-level stages: final hidden state, logit gradient, row losses
FINAL_STAGES = [(11, "h_L"), (12, "dlogits"), (13, "loss_rows")]
# state arrays in oracle.Model.read numbering
STATE = [(0, "params"), (1, "grad"), (2, "adam_m"), (3, "adam_v")]


def oracle_cards(model: "oracle.Model", state: bool = True) -> list[tuple[str, str, int, str]]:
    """Cards of every stage of the model's last forward, in computation order,
    then (state=True) of params, gradient accumulator and both moments."""
    out = []
    for layer in range(model.cfg["n_layers"]):
        for sid, name in LAYER_STAGES:
            a = model.stage(sid, layer)
            out.append((f"L{layer}.{name}", "f32", int(a.size), oracle.sha256(a.tobytes())))
    for sid, name in FINAL_STAGES:
        a = model.stage(sid, 0)
        out.append((name, "f32", int(a.size), oracle.sha256(a.tobytes())))
    if state:
        for w, name in STATE:
            a = model.read(w)
            out.append((name, "f32", int(a.size), oracle.sha256(a.tobytes())))
    return out
