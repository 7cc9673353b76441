"""Stage identity cards and the first-divergence diff (host logic and oracle,
CPU): equal runs give equal cards; a planted change in one rule of the profile
(a sabotage arm of the oracle) is reported at the first stage that rule
touches."""
import numpy as np
import pytest

import oracle
from bitwise_reproducible_fp32_amd import inputs as I
from bitwise_reproducible_fp32_amd.cards import Card, card_order, first_divergence, stage_tag
from oracle_cards import FINAL_STAGES, LAYER_STAGES, oracle_cards as cards_of


def test_first_divergence_logic():
    a = [Card("x", "f32", 3, "aa"), Card("y", "f32", 3, "bb"), Card("z", "f32", 1, "cc")]
    assert first_divergence(a, list(a)) is None
    b = [a[0], Card("y", "f32", 3, "bd"), Card("z", "f32", 1, "ee")]
    assert first_divergence(a, b).tag == "y"
    assert first_divergence(a, a[:2]).tag == "z"
    assert first_divergence(a[:1], a).tag == "y"


def test_card_order_follows_the_forward_pass():
    order = [stage_tag(s, l) for s, l in card_order(2)]
    assert order[:4] == ["L0.h_in", "L0.r1", "L0.xn1", "L0.qkv"]
    assert order.index("L0.a") < order.index("L1.h_in")
    assert order[-3:] == ["h_L", "dlogits", "loss_rows"]
    # the library's order and tags equal the test side's own literal list
    literal = [f"L{l}.{n}" for l in range(2) for _, n in LAYER_STAGES] + [n for _, n in FINAL_STAGES]
    assert order == literal
    # and the library's stage ids name the same stages as the oracle's export
    assert [s for s, l in card_order(2)] == [s for l in range(2) for s, _ in LAYER_STAGES] + \
        [s for s, _ in FINAL_STAGES]


def oracle_cards(arm: str | None):
    cfg = I.make_config("c0")
    oracle.set_sabotage(oracle.SABOTAGE[arm] if arm else 0)
    try:
        m = oracle.Model(cfg, I.init_params(cfg))
        x, y = I.c0_batch(0, cfg["batch"], cfg["seq_len"])
        m.forward(x, y)
        m.backward()
        return cards_of(m)
    finally:
        oracle.set_sabotage(0)


@pytest.fixture(scope="module")
def clean_cards():
    return oracle_cards(None)


def test_cards_are_deterministic(clean_cards):
    assert first_divergence(clean_cards, oracle_cards(None)) is None


@pytest.mark.parametrize("arm,first", [("gemm_reverse_k", "L0.qkv"), ("w64_mirror_pairing", "L0.r1"),
                                       ("softmax_divide", "L0.P"), ("libm_log", "loss_rows")])
def test_planted_rule_change_is_located(clean_cards, arm, first):
    bad = oracle_cards(arm)
    d = first_divergence(clean_cards, bad)
    assert d is not None and d[0] == first, (arm, d)
