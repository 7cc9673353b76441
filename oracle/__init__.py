"""ctypes front end of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package. The arithmetic
lives in oracle.cpp; this file marshals numpy arrays and builds the library.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "oracle.cpp")
# -ffp-contract=off: no implicit mul+add fusion; x86-64-v3 baseline (AVX2+FMA).
CXXFLAGS = ["-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-fPIC", "-shared", "-std=c++17"]


def build(compiler: str = "g++", out: str = LIB_PATH, extra: list[str] | None = None) -> str:
    """Compiles oracle.cpp; the new library replaces the old one by rename, so a
    process that has the old one loaded keeps running on it."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [compiler, *CXXFLAGS, *(extra or []), "-o", tmp, SRC]
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(tmp, out)
    return out


_lib = None
F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
I64P = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
U8P = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
i64, f32, i32 = C.c_int64, C.c_float, C.c_int


class Cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("vocab", "d_model", "n_layers", "n_heads", "head_dim",
                                          "ffn_hidden", "tied", "batch", "seq_len")] + \
               [(n, C.c_float) for n in ("rope_theta", "rms_eps", "beta1", "beta2", "adam_eps",
                                          "weight_decay")]


def cfg_struct(cfg: dict) -> Cfg:
    return Cfg(*[int(cfg[n]) for n, t in Cfg._fields_ if t is C.c_int32],
               *[float(cfg[n]) for n, t in Cfg._fields_ if t is C.c_float])


def argmax(x) -> int:
    """Index of the largest entry: NaN below every number, ties to the lowest index."""
    x = f32a(x).ravel()
    return int(lib().orc_argmax(x, x.size))


def splitmix64(seed: int, n: int) -> np.ndarray:
    """The first n SplitMix64 outputs from seed (uint64)."""
    out = np.empty(n, np.uint64)
    lib().orc_splitmix64(C.c_uint64(seed), n, out.ctypes.data_as(C.POINTER(C.c_uint64)))
    return out


def seed_params(cfg: dict, seed: int) -> np.ndarray:
    """Step-0 parameters drawn from seed by the profile's own generator."""
    c = cfg_struct(cfg)
    out = np.empty(lib().orc_param_count(C.byref(c)), np.float32)
    lib().orc_seed_params(C.byref(c), C.c_uint64(seed), out)
    return out


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    L = C.CDLL(path)
    sig = {
        "orc_set_threads": (None, [i32]), "orc_get_threads": (i32, []), "orc_ftz_daz_set": (i32, []),
        "orc_set_sabotage": (i32, [i32]), "orc_sabotage_count": (i32, []),
        "orc_exp": (f32, [f32]), "orc_log": (f32, [f32]), "orc_fma": (f32, [f32, f32, f32]),
        "orc_exp_array": (None, [F32P, F32P, i64]), "orc_log_array": (None, [F32P, F32P, i64]),
        "orc_fma_array": (None, [F32P, F32P, F32P, F32P, i64]),
        "orc_sigmoid_array": (None, [F32P, F32P, i64]),
        "orc_sum64": (f32, [F32P, i64]), "orc_dot64": (f32, [F32P, F32P, i64]),
        "orc_max64": (f32, [F32P, i64]),
        "orc_gemm": (i32, [i64, i64, i64, i64, C.c_void_p, i64, i64, C.c_void_p, i64, i64,
                           C.c_void_p, i64, i32, f32, i32, i32]),
        "orc_gemm_rows": (i32, [i64, i64, i64, i64, C.c_void_p, i64, i64, C.c_void_p, i64, i64,
                                I64P, i64, C.c_void_p, i64, i32, f32, i32, i32]),
        "orc_rmsnorm_fwd": (None, [F32P, F32P, i64, i64, f32, F32P, F32P]),
        "orc_rmsnorm_bwd": (None, [F32P, F32P, F32P, F32P, i64, i64, F32P, F32P]),
        "orc_rope_table": (None, [i64, i64, f32, F32P, F32P]),
        "orc_rope_fwd": (None, [C.c_void_p, i64, i64, i64, i64, i64, F32P, F32P]),
        "orc_rope_bwd": (None, [C.c_void_p, i64, i64, i64, i64, i64, F32P, F32P]),
        "orc_attn_scale": (f32, [i64]),
        "orc_attention_fwd": (None, [i64, i64, i64, i64, C.c_void_p, C.c_void_p, C.c_void_p, i64,
                                     C.c_void_p, C.c_void_p, i64]),
        "orc_attention_bwd": (None, [i64, i64, i64, i64, C.c_void_p, C.c_void_p, C.c_void_p, i64,
                                     C.c_void_p, C.c_void_p, C.c_void_p, i64, C.c_void_p,
                                     C.c_void_p, C.c_void_p]),
        "orc_swiglu_fwd": (None, [F32P, i64, i64, i64, F32P, i64]),
        "orc_swiglu_bwd": (None, [F32P, i64, F32P, i64, i64, i64, F32P]),
        "orc_cross_entropy": (f32, [F32P, I32P, i64, i64, F32P, F32P]),
        "orc_embed_scatter": (None, [I32P, F32P, i64, i64, F32P]),
        "orc_bias_correction": (f32, [f32, i64]),
        "orc_adamw": (None, [F32P, F32P, F32P, F32P, i64, f32, f32, f32, f32, f32, f32, f32]),
        "orc_sha256": (None, [U8P, i64, U8P]),
        "orc_param_count": (i64, [C.POINTER(Cfg)]),
        "orc_splitmix64": (None, [C.c_uint64, i64, C.POINTER(C.c_uint64)]),
        "orc_model_infer": (C.c_int, [C.c_void_p, I32P, C.c_void_p, C.c_void_p, C.POINTER(C.c_float)]),
        "orc_argmax": (i64, [F32P, i64]),
        "orc_seed_params": (None, [C.POINTER(Cfg), C.c_uint64, F32P]),
        "orc_model_new": (C.c_void_p, [C.POINTER(Cfg), F32P]),
        "orc_model_free": (None, [C.c_void_p]),
        "orc_model_forward": (i32, [C.c_void_p, I32P, I32P, C.POINTER(C.c_float)]),
        "orc_model_backward": (i32, [C.c_void_p]),
        "orc_model_adamw": (i32, [C.c_void_p, f32]),
        "orc_model_read": (None, [C.c_void_p, i32, F32P]),
        "orc_model_step": (i64, [C.c_void_p]),
        "orc_model_save": (i64, [C.c_void_p, C.c_void_p, i64]),
        "orc_model_load": (i32, [C.c_void_p, U8P, i64]),
        "orc_model_stage": (i64, [C.c_void_p, i32, i32, C.c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = L
    return L


def lib():
    return load()


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


SABOTAGE = {"gemm_reverse_k": 1, "gemm_kc512": 2, "gemm_pairwise_chunks": 3, "gemm_mul_add": 4,
            "w64_mirror_pairing": 5, "w32_lanes": 6, "libm_exp": 7, "ftz_daz": 8,
            "softmax_divide": 9, "adamw_decoupled": 10, "scatter_reverse": 11, "libm_log": 12,
            "rms_dw_unchunked": 13, "swiglu_bwd_spelling": 14, "ds_spelling": 15, "w64_blocks": 16}


def set_sabotage(arm: int) -> None:
    if lib().orc_set_sabotage(int(arm)) != 0:
        raise ValueError("unknown sabotage arm")


def f32a(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def exp(x):
    x = f32a(x); y = np.empty_like(x); lib().orc_exp_array(x.ravel(), y.ravel(), x.size); return y


def log(x):
    x = f32a(x); y = np.empty_like(x); lib().orc_log_array(x.ravel(), y.ravel(), x.size); return y


def fma(a, b, c):
    a, b, c = np.broadcast_arrays(f32a(a), f32a(b), f32a(c))
    a, b, c = f32a(a), f32a(b), f32a(c)
    y = np.empty_like(a)
    lib().orc_fma_array(a.ravel(), b.ravel(), c.ravel(), y.ravel(), a.size)
    return y


def sum64(v): v = f32a(v); return np.float32(lib().orc_sum64(v, v.size))
def dot64(a, b): a, b = f32a(a), f32a(b); return np.float32(lib().orc_dot64(a, b, a.size))
def max64(v): v = f32a(v); return np.float32(lib().orc_max64(v, v.size))


def gemm(A, B, M, N, K, sam, sak, sbk, sbn, C=None, ldc=None, kseg=0, mode=0, scale=1.0,
         krange=0, outmask=0):
    """Raw strided G1024 contraction; A and B are flat float32 buffers."""
    ldc = N if ldc is None else ldc
    if C is None:
        C = np.zeros(max(1, M * ldc), dtype=np.float32)
    rc = lib().orc_gemm(M, N, K, kseg, _p(A), sam, sak, _p(B), sbk, sbn, _p(C), ldc, mode,
                        scale, krange, outmask)
    if rc != 0:
        raise ValueError("orc_gemm: bad arguments")
    return C


def gemm_rows(A, B, M, N, K, sam, sak, sbk, sbn, rows, kseg=0, mode=0, scale=1.0, krange=0,
              outmask=0, C=None):
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if C is None:
        C = np.zeros((len(rows), N), dtype=np.float32)
    rc = lib().orc_gemm_rows(M, N, K, kseg, _p(A), sam, sak, _p(B), sbk, sbn, rows, len(rows),
                             _p(C), N, mode, scale, krange, outmask)
    if rc != 0:
        raise ValueError("orc_gemm_rows: bad arguments")
    return C


def linear(X, W):
    """Y = X W^T for X [M,K], W [N,K] (the forward form)."""
    X, W = f32a(X), f32a(W)
    M, K = X.shape
    N = W.shape[0]
    return gemm(X, W, M, N, K, K, 1, 1, K).reshape(M, N)


def rmsnorm_fwd(x, w, eps):
    x, w = f32a(x), f32a(w)
    rows, d = x.shape
    y = np.empty_like(x); r = np.empty(rows, np.float32)
    lib().orc_rmsnorm_fwd(x, w, rows, d, eps, y, r)
    return y, r


def rmsnorm_bwd(dy, x, w, r):
    dy, x, w, r = f32a(dy), f32a(x), f32a(w), f32a(r)
    rows, d = x.shape
    dx = np.empty_like(x); dw = np.empty(d, np.float32)
    lib().orc_rmsnorm_bwd(dy, x, w, r, rows, d, dx, dw)
    return dx, dw


def rope_table(T, hd, theta):
    c = np.empty((T, hd // 2), np.float32); s = np.empty_like(c)
    lib().orc_rope_table(T, hd, theta, c, s)
    return c, s


def attention_fwd(q, k, v):
    """q, k, v [BH, T, hd] contiguous. Returns P [BH, T, T] (upper part 0), O [BH, T, hd]."""
    q, k, v = f32a(q), f32a(k), f32a(v)
    BH, T, hd = q.shape
    P = np.zeros((BH, T, T), np.float32); O = np.zeros((BH, T, hd), np.float32)
    lib().orc_attention_fwd(BH, 1, T, hd, _p(q), _p(k), _p(v), hd, _p(P), _p(O), hd)
    return P, O


def attention_bwd(q, k, v, P, O, dO):
    q, k, v, P, O, dO = map(f32a, (q, k, v, P, O, dO))
    BH, T, hd = q.shape
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    lib().orc_attention_bwd(BH, 1, T, hd, _p(q), _p(k), _p(v), hd, _p(P), _p(O), _p(dO), hd,
                            _p(dq), _p(dk), _p(dv))
    return dq, dk, dv


def cross_entropy(logits, targets):
    logits = f32a(logits); targets = np.ascontiguousarray(targets, dtype=np.int32)
    N, V = logits.shape
    loss_rows = np.empty(N, np.float32); dl = np.empty_like(logits)
    loss = lib().orc_cross_entropy(logits, targets.ravel(), N, V, loss_rows, dl)
    return np.float32(loss), loss_rows, dl


def embed_scatter(ids, dh, dE):
    ids = np.ascontiguousarray(ids, dtype=np.int32).ravel(); dh = f32a(dh)
    out = f32a(dE).copy()
    lib().orc_embed_scatter(ids, dh, len(ids), dh.shape[1], out)
    return out


def sha256(b: bytes | np.ndarray) -> str:
    a = np.frombuffer(bytes(b) if not isinstance(b, np.ndarray) else b.tobytes(), dtype=np.uint8)
    out = np.zeros(32, np.uint8)
    lib().orc_sha256(np.ascontiguousarray(a), a.size, out)
    return out.tobytes().hex()


class Model:
    """The oracle's training state for one model config."""

    def __init__(self, cfg: dict, init_params: np.ndarray):
        self.cfg = dict(cfg)
        self._c = cfg_struct(cfg)
        self.n = lib().orc_param_count(C.byref(self._c))
        init = f32a(init_params)
        if init.size != self.n:
            raise ValueError("init size mismatch")
        self.h = lib().orc_model_new(C.byref(self._c), init)
        if not self.h:
            raise ValueError("bad config")

    def __del__(self):
        try:
            if getattr(self, "h", None) and _lib is not None:
                _lib.orc_model_free(self.h)
        except Exception:
            pass
        self.h = None

    def forward(self, inputs, targets) -> np.float32:
        x = np.ascontiguousarray(inputs, dtype=np.int32).ravel()
        y = np.ascontiguousarray(targets, dtype=np.int32).ravel()
        out = C.c_float()
        if lib().orc_model_forward(self.h, x, y, C.byref(out)) != 0:
            raise ValueError("token out of range")
        return np.float32(out.value)

    def backward(self) -> None:
        if lib().orc_model_backward(self.h) != 0:
            raise RuntimeError("backward without forward")

    def adamw(self, lr: float) -> None:
        if lib().orc_model_adamw(self.h, lr) != 0:
            raise RuntimeError("adamw without gradient")

    def read(self, which: int) -> np.ndarray:
        out = np.empty(self.n, np.float32)
        lib().orc_model_read(self.h, which, out)
        return out

    params = property(lambda s: s.read(0))
    grad = property(lambda s: s.read(1))
    adam_m = property(lambda s: s.read(2))
    adam_v = property(lambda s: s.read(3))

    @property
    def step(self) -> int:
        return lib().orc_model_step(self.h)

    def save(self) -> bytes:
        n = lib().orc_model_save(self.h, None, 0)
        buf = np.zeros(n, np.uint8)
        if lib().orc_model_save(self.h, _p(buf), n) != n:
            raise RuntimeError("save refused")
        return buf.tobytes()

    def load(self, b: bytes) -> None:
        a = np.frombuffer(b, dtype=np.uint8).copy()
        rc = lib().orc_model_load(self.h, a, a.size)
        if rc != 0:
            raise ValueError(f"load refused ({rc})")

    def infer(self, inputs, targets=None):
        """Inference forward: (logits [tokens, vocab], mean loss or None)."""
        x = np.ascontiguousarray(inputs, dtype=np.int32).ravel()
        y = None if targets is None else np.ascontiguousarray(targets, dtype=np.int32).ravel()
        N = x.size
        logits = np.empty((N, self.cfg["vocab"]), np.float32)
        loss = C.c_float()
        rc = lib().orc_model_infer(self.h, x, None if y is None else y.ctypes.data, logits.ctypes.data,
                                   C.byref(loss))
        if rc != 0:
            raise ValueError("token out of range")
        return logits, (None if y is None else np.float32(loss.value))

    def greedy_next(self, inputs, position: int) -> np.ndarray:
        """Next token of each sequence after `position`: argmax of that
        position's logits (lowest index on ties)."""
        logits, _ = self.infer(inputs)
        B, T = self.cfg["batch"], self.cfg["seq_len"]
        rows = logits.reshape(B, T, -1)[:, position, :]
        return np.array([argmax(r) for r in rows], np.int32)

    def stage(self, stage: int, layer: int = 0) -> np.ndarray:
        n = lib().orc_model_stage(self.h, stage, layer, None)
        out = np.empty(n, np.float32)
        lib().orc_model_stage(self.h, stage, layer, _p(out))
        return out
