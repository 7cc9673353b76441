"""Stage identity cards: the order in which the training step produces its
stages, and the first-divergence diff of two card lists.

A card is (tag, dtype, count, sha256 hex) of one stage's exact bytes in the
canonical export layout (mlb_read_stage). Two runs that agree bit for bit have
equal cards everywhere; the first unequal card in computation order names the
stage where they start to differ. This module holds no arithmetic of the
method; it only orders and compares cards produced by the library or by a
reference implementation.
"""
from __future__ import annotations

from typing import NamedTuple

# per-layer stages in the order the forward pass computes them
# (stage ids of mlb_read_stage: 0 h_in, 2 r1, 1 xn1, 3 qkv, 4 P, 5 O, 6 h_mid,
#  8 r2, 7 xn2, 9 gu, 10 a), then the model-level ones (11 h_L, 12 dlogits,
#  13 loss_rows)
LAYER_ORDER = (0, 2, 1, 3, 4, 5, 6, 8, 7, 9, 10)
FINAL_ORDER = (11, 12, 13)
STAGE_NAMES = ("h_in", "xn1", "r1", "qkv", "P", "O", "h_mid", "xn2", "r2", "gu", "a", "h_L", "dlogits",
               "loss_rows")
STATE_NAMES = ("params", "grad", "adam_m", "adam_v")


class Card(NamedTuple):
    tag: str
    dtype: str
    count: int
    sha256: str


def stage_tag(stage: int, layer: int) -> str:
    return f"L{layer}.{STAGE_NAMES[stage]}" if stage <= 10 else STAGE_NAMES[stage]


def card_order(n_layers: int) -> list[tuple[int, int]]:
    """(stage, layer) pairs in computation order."""
    out = [(st, l) for l in range(n_layers) for st in LAYER_ORDER]
    return out + [(st, 0) for st in FINAL_ORDER]


def first_divergence(a: list[Card], b: list[Card]) -> Card | None:
    """The first card of `a` whose tag, dtype, count or hash differs from `b`'s
    card at the same position (or the first one past the shorter list); None
    when the lists agree."""
    for x, y in zip(a, b):
        if x != y:
            return x
    if len(a) != len(b):
        return (a if len(a) > len(b) else b)[min(len(a), len(b))]
    return None
