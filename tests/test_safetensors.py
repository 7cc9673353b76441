"""The safetensors export (mlb_safetensors, host-only, no device) and the plain
PyTorch forward that runs exported weights elsewhere.

Pins:
- An independent reader (the safetensors package) recovers every tensor of
  the canonical order with its name and shape.
- The data section is the oracle checkpoint's parameter array byte for byte
  (model card, "Anywhere else: safetensors + PyTorch").
- The float64 PyTorch forward agrees with the oracle's FP32 logits to within
  TOL times the largest |logit| of the batch, and picks the same greedy token
  wherever the top two logits are more than twice that apart. PyTorch sums in
  its own order, so this is a tolerance check, not part of the bitwise claim.
  TOL = 1e-5: the FP32 forward's rounding error at these sizes, relative to
  the logit scale, measured at most 1.0e-6 (6-layer model, 128 tokens) and
  2.1e-7 (byte LM), with a margin of ten or more; the pages report a 3.8e-5
  absolute gap for their trained 162M model.
"""
import json
import struct

import numpy as np
import pytest

import oracle
import bitwise_reproducible_fp32_amd as mlb
from bitwise_reproducible_fp32_amd import inputs as I
from bitwise_reproducible_fp32_amd import torch_forward as TF

TOL = 1e-5


def trained_c0():
    """The byte LM after four oracle training steps (weights moved off init)."""
    cfg = I.make_config("c0")
    o = oracle.Model(cfg, I.init_params(cfg))
    for s in range(1, 5):
        x, y = I.batch_for("c0", cfg, s, 0)
        o.forward(x, y)
        o.backward()
        o.adamw(I.lr_at("c0", s))
    return cfg, o


@pytest.mark.parametrize("name,over", [("c0", {}), ("c3", {"batch": 1, "seq_len": 128}), ("c0", {"tied": 0})])
def test_image_layout_and_independent_reader(name, over):
    st_numpy = pytest.importorskip("safetensors.numpy")
    cfg = I.make_config(name, **over)
    p = I.init_params(cfg)
    blob = mlb.safetensors_bytes(cfg, p)
    (n,) = struct.unpack("<Q", blob[:8])
    assert n % 8 == 0 and (8 + n) % 8 == 0
    assert blob[8 + n:] == p.tobytes()                       # parameter array unchanged
    table = json.loads(blob[8:8 + n])
    meta = table["__metadata__"]
    for k in ("vocab", "d_model", "n_layers", "n_heads", "head_dim", "ffn_hidden", "tied"):
        assert int(meta[k]) == int(cfg[k]), k
    assert np.float32(meta["rms_eps"]) == np.float32(cfg["rms_eps"])
    assert np.float32(meta["rope_theta"]) == np.float32(cfg["rope_theta"])
    got = st_numpy.load(blob)
    shapes = I.param_shapes(cfg)
    assert set(got) == {nm for nm, _, _ in shapes}
    off = 0
    for nm, shape, _ in shapes:
        size = int(np.prod(shape))
        assert got[nm].dtype == np.float32 and got[nm].shape == shape, nm
        assert got[nm].tobytes() == p[off:off + size].tobytes(), nm
        off += size
    assert off == p.size


def test_data_section_is_checkpoint_parameter_array():
    cfg, o = trained_c0()
    ck = o.save()
    nb = o.n * 4
    hdr = len(ck) - 3 * nb
    blob = mlb.safetensors_bytes(cfg, o.params)
    (n,) = struct.unpack("<Q", blob[:8])
    assert blob[8 + n:] == ck[hdr:hdr + nb]


def test_refusals():
    cfg = I.make_config("c0")
    with pytest.raises(ValueError):
        mlb.safetensors_bytes(cfg, np.zeros(3, np.float32))
    bad = dict(cfg, d_model=33)
    with pytest.raises(Exception):
        mlb.safetensors_bytes(bad, np.zeros(10, np.float32))


def _agree(cfg, logits_fp32, ids):
    ctx, tensors = TF.load(mlb.safetensors_bytes(cfg, cfg["_params"]))
    ref = TF.forward_logits(ctx, tensors, ids).reshape(-1, cfg["vocab"]).numpy()
    got = logits_fp32.astype(np.float64)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max() / scale
    assert err <= TOL, err
    top2 = np.sort(ref, axis=1)[:, -2:]
    clear = (top2[:, 1] - top2[:, 0]) > 2 * TOL * scale
    mine = np.array([oracle.argmax(r) for r in logits_fp32])
    assert (mine[clear] == ref.argmax(1)[clear]).all()
    return clear.mean()


def test_torch_forward_agrees_with_oracle_byte_lm():
    cfg, o = trained_c0()
    x, _ = I.batch_for("c0", cfg, 5, 0)
    logits, _ = o.infer(x)
    cfg["_params"] = o.params
    assert _agree(cfg, logits, x.reshape(cfg["batch"], cfg["seq_len"])) > 0.9


def test_torch_forward_agrees_with_oracle_decoder():
    cfg = I.make_config("c3", batch=1, seq_len=128)
    p = I.init_params(cfg)
    o = oracle.Model(cfg, p)
    x = np.random.default_rng(3).integers(0, cfg["vocab"], (1, 128)).astype(np.int32)
    logits, _ = o.infer(x)
    cfg["_params"] = p
    assert _agree(cfg, logits, x) > 0.9


def test_torch_forward_catches_a_wrong_tensor():
    """The cross-check is sensitive: swapping two layers' Wq breaks agreement."""
    cfg, o = trained_c0()
    x, _ = I.batch_for("c0", cfg, 5, 0)
    logits, _ = o.infer(x)
    ctx, t = TF.load(mlb.safetensors_bytes(cfg, o.params))
    t["l0.Wq"], t["l1.Wq"] = t["l1.Wq"], t["l0.Wq"]
    ref = TF.forward_logits(ctx, t, x.reshape(cfg["batch"], cfg["seq_len"])).reshape(-1, cfg["vocab"]).numpy()
    assert np.abs(ref - logits).max() > 100 * TOL * np.abs(ref).max()
