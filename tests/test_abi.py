"""CPU checks of the C ABI boundary: the library loads, exports every symbol the
headers declare, and refuses invalid or unsupported configs by name. No call
here touches a GPU."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

from bitwise_reproducible_fp32_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mlb():
    import bitwise_reproducible_fp32_amd as m
    if not os.path.exists(m.LIB_PATH):
        from bitwise_reproducible_fp32_amd import build
        build.build()
    return m


def declared_symbols():
    names = set()
    for h in ("mlb.h", "mlb_prim.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(mlb_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(mlb):
    mlb.lib()   # PyTorch's HIP runtime first (see test_one_hip_runtime_in_the_process)
    lib = C.CDLL(mlb.LIB_PATH)
    syms = declared_symbols()
    assert len(syms) >= 25
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) <= set(mlb._SIGS), set(syms) - set(mlb._SIGS)


def test_status_names_and_profile(mlb):
    L = mlb.lib()
    for code, name in mlb.STATUS.items():
        assert L.mlb_status_name(code).decode() == name
    assert L.mlb_profile_version() == 1


def test_param_count_matches_pages(mlb):
    assert mlb.param_count(I.make_config("c0")) == 34944
    assert mlb.param_count(I.make_config("c4")) == 162147840


def test_workspace_fits_the_162m_model(mlb):
    n = mlb.workspace_bytes(I.make_config("c4"))
    assert 4 * 4 * 162147840 < n < 64 << 30


@pytest.mark.parametrize("over,status", [
    (dict(d_model=30), "MLB_E_INVALID_ARG"),          # heads * head_dim != d_model
    (dict(head_dim=7, n_heads=4, d_model=28), "MLB_E_UNSUPPORTED"),
    (dict(ffn_hidden=100), "MLB_E_UNSUPPORTED"),
    (dict(batch=1025), "MLB_E_UNSUPPORTED"),          # > 65,536 tokens per micro-batch
    (dict(vocab=0), "MLB_E_INVALID_ARG"),
    (dict(rms_eps=float("nan")), "MLB_E_INVALID_ARG"),
])
def test_bad_configs_refused(mlb, over, status):
    with pytest.raises(mlb.MlbError) as e:
        mlb.workspace_bytes(I.make_config("c0", **over))
    assert e.value.name == status


def test_abi_version_checked(mlb):
    c = mlb.config(I.make_config("c0"))
    c.abi_version = 99
    n = C.c_size_t()
    assert mlb.lib().mlb_workspace_bytes(C.byref(c), C.byref(n)) == -1


def test_null_arguments_refused(mlb):
    L = mlb.lib()
    c = mlb.config(I.make_config("c0"))
    h = C.c_void_p()
    assert L.mlb_init(C.byref(c), 1, None, None, 0, None, C.byref(h)) == -1   # no arena
    assert L.mlb_init(C.byref(c), 1, None, None, 0, None, None) == -1         # no handle slot
    assert L.mlb_backward(None) == -1
    assert L.mlb_adamw_step(None, 1.0) == -1
    n = C.c_size_t()
    assert L.mlb_save(None, None, 0, C.byref(n)) == -1
    assert L.mlb_destroy(None) == 0


def test_one_hip_runtime_in_the_process(mlb):
    """The binding loads PyTorch's HIP runtime before the library, so a process
    holds one copy of it. PyTorch's wheel carries its own, under the same
    soname; loaded second, it would be a second runtime in which the library's
    device pointers and streams are invalid."""
    code = ("import bitwise_reproducible_fp32_amd as m; m.lib(); import torch; "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1", r.stdout
