"""Named refusals of the library, driven through a model handle.

The pages ask for a refusal by name instead of a silently different result
(mojolearn PyPI page, "What bitwise identity means": an explicit refusal when
the promise cannot be met) and for a load that verifies every array digest
(MojoLearn 162M model card, "Using the model"). Each case below makes one call
that must be refused with its status code, then checks that the state the
library holds (parameters, accumulated gradient, both moments, step) is
bit-identical to what it was before the call, and that the model still trains
on afterwards with the oracle's bits.
"""
import ctypes as C
import hashlib
import struct

import numpy as np
import pytest

import oracle
from bitwise_reproducible_fp32_amd import inputs as I
from gpu_util import dev

pytestmark = pytest.mark.gpu

HDR = 256


@pytest.fixture(scope="module")
def mlb():
    import bitwise_reproducible_fp32_amd as m
    return m


@pytest.fixture(scope="module")
def cfg():
    return I.make_config("c0")


def batch(step):
    x, y = I.c0_batch(step - 1)
    return dev(x.astype(np.int32)), dev(y.astype(np.int32))


def state(mlb, m):
    return [m.read(w).tobytes() for w in (mlb.PARAMS, mlb.GRAD, mlb.ADAM_M, mlb.ADAM_V)] + [m.step]


@pytest.fixture()
def trained(mlb, cfg):
    """A byte-LM model after one step (non-zero moments, step 1) and its bytes."""
    m = mlb.Model(cfg, I.init_params(cfg))
    x, y = batch(1)
    m.forward_loss(x, y)
    m.backward()
    m.adamw_step(I.lr_at("c0", 1))
    blob = m.save()
    yield m, blob
    m.close()


def refused(mlb, status, fn, *args):
    with pytest.raises(mlb.MlbError) as e:
        fn(*args)
    assert e.value.name == status, str(e.value)


def reseal(b: bytearray) -> bytes:
    """Recomputes the header digest (SHA-256 of the first 192 bytes)."""
    b[192:224] = hashlib.sha256(bytes(b[:192])).digest()
    return bytes(b)


def continues_like_oracle(mlb, cfg, m, blob):
    """After the refusals the model takes step 2 with the oracle's bits."""
    o = oracle.Model(cfg, I.init_params(cfg, seed=1))
    o.load(blob)
    x, y = batch(2)
    xo, yo = I.c0_batch(1)
    assert m.forward_loss(x, y).tobytes() == o.forward(xo, yo).tobytes()
    m.backward()
    o.backward()
    m.adamw_step(I.lr_at("c0", 2))
    o.adamw(I.lr_at("c0", 2))
    assert m.save() == o.save()


def test_load_refuses_corrupt_bytes(mlb, cfg, trained):
    m, blob = trained
    before = state(mlb, m)
    nb = (len(blob) - HDR) // 3
    cases = []
    for region in range(3):                     # one flipped byte in params, m, v
        b = bytearray(blob)
        b[HDR + region * nb + 1234] ^= 0x01
        cases.append((f"payload {region}", bytes(b)))
    b = bytearray(blob)
    b[80] ^= 0x01                               # step field, digest not resealed
    cases.append(("header byte", bytes(b)))
    b = bytearray(blob)
    b[100] ^= 0x80                              # stored params digest
    cases.append(("stored digest", bytes(b)))
    cases.append(("truncated", blob[:-1]))
    cases.append(("truncated header", blob[:HDR - 1]))
    cases.append(("extended", blob + b"\0"))
    b = bytearray(blob)
    b[76] = 1                                   # padding inside the sealed part, resealed
    cases.append(("padding", reseal(b)))
    b = bytearray(blob)
    b[240] = 1                                  # padding after the header digest
    cases.append(("tail padding", bytes(b)))
    b = bytearray(blob)
    b[88:96] = struct.pack("<Q", m.n - 1)       # parameter count, resealed
    cases.append(("count", reseal(b)))
    for name, bad in cases:
        with pytest.raises(mlb.MlbError) as e:
            m.load(bad)
        assert e.value.name == "MLB_E_CORRUPT", (name, str(e.value))
        assert state(mlb, m) == before, name
    continues_like_oracle(mlb, cfg, m, blob)


def test_load_refuses_other_profile_or_config(mlb, cfg, trained):
    m, blob = trained
    before = state(mlb, m)
    cases = []
    b = bytearray(blob)
    b[12:16] = struct.pack("<I", 2)              # profile version
    cases.append(("profile", reseal(b), "MLB_E_PROFILE_MISMATCH"))
    b = bytearray(blob)
    b[8:12] = struct.pack("<I", 2)               # format version
    cases.append(("format", reseal(b), "MLB_E_PROFILE_MISMATCH"))
    b = bytearray(blob)
    b[0:8] = b"MLBCKPT2"
    cases.append(("magic", reseal(b), "MLB_E_PROFILE_MISMATCH"))
    b = bytearray(blob)
    b[16:20] = struct.pack("<I", 257)            # vocab
    cases.append(("vocab", reseal(b), "MLB_E_CONFIG_MISMATCH"))
    b = bytearray(blob)
    b[48:52] = struct.pack("<I", 65)             # seq_len
    cases.append(("seq_len", reseal(b), "MLB_E_CONFIG_MISMATCH"))
    b = bytearray(blob)
    b[52:56] = struct.pack("<f", 500000.0)       # rope theta
    cases.append(("rope_theta", reseal(b), "MLB_E_CONFIG_MISMATCH"))
    b = bytearray(blob)
    b[72:76] = struct.pack("<f", 0.0)            # weight decay
    cases.append(("weight_decay", reseal(b), "MLB_E_CONFIG_MISMATCH"))
    for name, bad, status in cases:
        with pytest.raises(mlb.MlbError) as e:
            m.load(bad)
        assert e.value.name == status, (name, str(e.value))
        assert state(mlb, m) == before, name
    # the resealed bytes are otherwise well formed: the original loads
    m.load(blob)
    assert state(mlb, m) == before
    continues_like_oracle(mlb, cfg, m, blob)


def test_call_order_refusals(mlb, cfg, trained):
    m, blob = trained
    before = state(mlb, m)
    refused(mlb, "MLB_E_STATE", m.backward)               # no forward
    refused(mlb, "MLB_E_STATE", m.adamw_step, 1e-3)       # no backward since the step
    assert state(mlb, m) == before
    x, y = batch(2)
    m.forward_loss(x, y)
    refused(mlb, "MLB_E_STATE", m.infer, x, y)            # forward pending its backward
    refused(mlb, "MLB_E_STATE", m.greedy_next, x, 3)
    refused(mlb, "MLB_E_STATE", m.set_overlap, True)
    m.backward()
    g1 = m.read(mlb.GRAD).tobytes()
    refused(mlb, "MLB_E_STATE", m.backward)               # second backward of one forward
    assert m.read(mlb.GRAD).tobytes() == g1               # nothing added twice
    refused(mlb, "MLB_E_STATE", m.save)                   # gradient pending
    assert state(mlb, m)[0] == before[0] and state(mlb, m)[2:] == before[2:]
    o = oracle.Model(cfg, I.init_params(cfg, seed=1))
    o.load(blob)
    xo, yo = I.c0_batch(1)
    o.forward(xo, yo)
    o.backward()
    assert m.read(mlb.GRAD).tobytes() == o.grad.tobytes()
    m.adamw_step(I.lr_at("c0", 2))
    o.adamw(I.lr_at("c0", 2))
    assert m.save() == o.save()


def test_bad_token_refusals(mlb, cfg, trained):
    m, blob = trained
    before = state(mlb, m)
    x, y = I.c0_batch(1)
    for name, xi, yi in (("input = vocab", np.where(np.arange(x.size).reshape(x.shape) == 77, 256, x), y),
                         ("input < 0", np.where(np.arange(x.size).reshape(x.shape) == 0, -1, x), y),
                         ("target = vocab", x, np.where(np.arange(y.size).reshape(y.shape) == 511, 256, y)),
                         ("target huge", x, np.where(np.arange(y.size).reshape(y.shape) == 5, 2 ** 31 - 1, y))):
        xd, yd = dev(xi.astype(np.int32)), dev(yi.astype(np.int32))
        refused(mlb, "MLB_E_BAD_TOKEN", m.forward_loss, xd, yd)
        refused(mlb, "MLB_E_STATE", m.backward)           # no usable forward
        refused(mlb, "MLB_E_BAD_TOKEN", m.infer, xd, yd)
        assert state(mlb, m) == before, name
    continues_like_oracle(mlb, cfg, m, blob)


def test_init_refusals(mlb, cfg):
    import torch
    L = mlb.lib()
    c = mlb.config(cfg)
    need = mlb.workspace_bytes(cfg)
    arena = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    base = arena.data_ptr() + (-arena.data_ptr()) % 256
    init = I.init_params(cfg)
    h = C.c_void_p()
    stream = torch.cuda.current_stream().cuda_stream
    rc = L.mlb_init(C.byref(c), 0, init.ctypes.data, base, need - 256, stream, C.byref(h))
    assert mlb.STATUS[rc] == "MLB_E_ARENA_TOO_SMALL" and not h.value
    rc = L.mlb_init(C.byref(c), 0, init.ctypes.data, base + 4, need, stream, C.byref(h))
    assert mlb.STATUS[rc] == "MLB_E_INVALID_ARG" and not h.value
    bad = mlb.config(dict(cfg, head_dim=7, d_model=28))          # odd head width: no rotary pairs
    rc = L.mlb_init(C.byref(bad), 0, None, base, need, stream, C.byref(h))
    assert mlb.STATUS[rc] == "MLB_E_UNSUPPORTED" and not h.value
    bad = mlb.config(dict(cfg, seq_len=48))                      # not a multiple of 32
    rc = L.mlb_init(C.byref(bad), 0, None, base, need, stream, C.byref(h))
    assert mlb.STATUS[rc] == "MLB_E_UNSUPPORTED" and not h.value
    bad = mlb.config(dict(cfg))
    bad.abi_version = 2
    rc = L.mlb_init(C.byref(bad), 0, None, base, need, stream, C.byref(h))
    assert mlb.STATUS[rc] == "MLB_E_INVALID_ARG" and not h.value
    rc = L.mlb_init(C.byref(c), 0, init.ctypes.data, base, need, stream, C.byref(h))
    assert rc == 0 and h.value
    assert L.mlb_destroy(h) == 0


def test_host_buffer_and_argument_refusals(mlb, cfg, trained):
    m, blob = trained
    L = mlb.lib()
    n = C.c_size_t()
    small = np.zeros(len(blob) - 1, np.uint8)
    assert mlb.STATUS[L.mlb_save(m.h, small.ctypes.data, small.size, C.byref(n))] == "MLB_E_IO"
    assert n.value == len(blob)
    out = np.zeros(m.n - 1, np.float32)
    assert mlb.STATUS[L.mlb_read(m.h, mlb.PARAMS, out.ctypes.data, out.nbytes)] == "MLB_E_IO"
    assert mlb.STATUS[L.mlb_read(m.h, 7, out.ctypes.data, out.nbytes + 4)] == "MLB_E_INVALID_ARG"
    x, _ = batch(2)
    refused(mlb, "MLB_E_INVALID_ARG", m.greedy_next, x, cfg["seq_len"])
    refused(mlb, "MLB_E_INVALID_ARG", m.greedy_next, x, -1)
    assert m.save() == blob
