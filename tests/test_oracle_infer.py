"""Pins of the inference surface of the oracle (CPU): the argmax rule (largest
value, lowest index on ties, NaN below every number), the inference loss equal
to the training forward's loss bit for bit, and greedy choices equal to a brute
force argmax of the kept logits."""
import math

import numpy as np

import oracle
from bitwise_reproducible_fp32_amd import inputs as I


def test_argmax_rule():
    nan, inf = float("nan"), float("inf")
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1                 # tie: lowest index
    assert oracle.argmax([nan, 1.0, nan, 5.0, nan]) == 3            # NaN below every number
    assert oracle.argmax([nan, nan]) == 0                           # all NaN: 0
    assert oracle.argmax([-inf, -inf, -inf]) == 0
    assert oracle.argmax([-0.0, 0.0]) == 0 and oracle.argmax([0.0, -0.0]) == 0   # equal values
    assert oracle.argmax([-inf, nan, -5.0]) == 2
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = rng.integers(-4, 5, size=rng.integers(1, 300)).astype(np.float32)   # many ties
        assert oracle.argmax(x) == int(np.argmax(x))                # numpy: first maximum


def test_infer_loss_equals_training_loss():
    cfg = I.make_config("c0")
    init = I.init_params(cfg)
    x, y = I.c0_batch(0, cfg["batch"], cfg["seq_len"])
    train = oracle.Model(cfg, init).forward(x, y)
    logits, loss = oracle.Model(cfg, init).infer(x, y)
    assert np.float32(loss).tobytes() == np.float32(train).tobytes()
    assert logits.shape == (cfg["batch"] * cfg["seq_len"], cfg["vocab"])
    # the kept logits give the same loss through the standalone cross-entropy rule
    closs, rows, _ = oracle.cross_entropy(logits, y.ravel())
    assert closs.tobytes() == np.float32(loss).tobytes()
    assert math.isfinite(float(loss)) and np.all(np.isfinite(rows))


def test_greedy_is_argmax_of_kept_logits():
    cfg = I.make_config("c0")
    m = oracle.Model(cfg, I.init_params(cfg))
    x, _ = I.c0_batch(0, cfg["batch"], cfg["seq_len"])
    logits, _ = m.infer(x)
    T = cfg["seq_len"]
    for pos in (0, 17, T - 1):
        want = [int(np.argmax(logits.reshape(cfg["batch"], T, -1)[b, pos])) for b in range(cfg["batch"])]
        assert list(m.greedy_next(x, pos)) == want
