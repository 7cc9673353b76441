"""Bitwise-reproducible FP32 training step on MI355X (gfx950).

A thin ctypes binding of libmlb.so (include/mlb.h, include/mlb_prim.h). Every
step of the computation runs in the library's HIP kernels; this module only
marshals arguments. PyTorch provides device memory (the arena, test tensors)
and the current HIP stream. There is no CPU path: if the library is missing,
importing the binding raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmlb.so")

MLB_ABI_VERSION = 1
STATUS = {0: "MLB_OK", -1: "MLB_E_INVALID_ARG", -2: "MLB_E_UNSUPPORTED", -3: "MLB_E_DEVICE",
          -4: "MLB_E_ARENA_TOO_SMALL", -5: "MLB_E_BAD_TOKEN", -6: "MLB_E_STATE", -7: "MLB_E_CORRUPT",
          -8: "MLB_E_PROFILE_MISMATCH", -9: "MLB_E_CONFIG_MISMATCH", -10: "MLB_E_IO"}
PARAMS, GRAD, ADAM_M, ADAM_V = 0, 1, 2, 3


class MlbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class Config(C.Structure):
    _fields_ = [("abi_version", C.c_uint32)] + \
               [(n, C.c_uint32) for n in ("vocab", "d_model", "n_layers", "n_heads", "head_dim",
                                          "ffn_hidden", "tied", "batch", "seq_len")] + \
               [(n, C.c_float) for n in ("rope_theta", "rms_eps", "beta1", "beta2", "adam_eps",
                                         "weight_decay")]


def config(cfg: dict) -> Config:
    return Config(MLB_ABI_VERSION, *[int(cfg[n]) for n, t in Config._fields_[1:] if t is C.c_uint32],
                  *[float(cfg[n]) for n, t in Config._fields_ if t is C.c_float])


class Stat(C.Structure):
    _fields_ = [("site", C.c_char * 48), ("kernel", C.c_char * 96), ("launches", C.c_int64),
                ("ms", C.c_double), ("flops", C.c_double), ("bytes", C.c_double)]


_lib = None
vp, i64, i32, f32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
_SIGS = {
    "mlb_param_count": (i64, [C.POINTER(Config)]),
    "mlb_workspace_bytes": (i32, [C.POINTER(Config), C.POINTER(sz)]),
    "mlb_init": (i32, [C.POINTER(Config), C.c_uint64, vp, vp, sz, vp, C.POINTER(vp)]),
    "mlb_forward_loss": (i32, [vp, vp, vp, C.POINTER(f32)]),
    "mlb_backward": (i32, [vp]),
    "mlb_adamw_step": (i32, [vp, f32]),
    "mlb_save": (i32, [vp, vp, sz, C.POINTER(sz)]),
    "mlb_load": (i32, [vp, vp, sz]),
    "mlb_read": (i32, [vp, i32, vp, sz]),
    "mlb_safetensors": (i32, [C.POINTER(Config), vp, vp, sz, C.POINTER(sz)]),
    "mlb_read_stage": (i32, [vp, i32, i32, vp, sz, C.POINTER(sz)]),
    "mlb_step": (C.c_uint64, [vp]),
    "mlb_set_overlap": (i32, [vp, i32]),
    "mlb_infer": (i32, [vp, vp, vp, vp, C.POINTER(f32)]),
    "mlb_greedy_next": (i32, [vp, vp, i32, vp]),
    "mlb_stage_card": (i32, [vp, i32, i32, vp]),
    "mlb_state_card": (i32, [vp, i32, vp]),
    "mlb_stats_enable": (i32, [vp, i32]),
    "mlb_stats_read": (i32, [vp, C.POINTER(Stat), i32, C.POINTER(i32)]),
    "mlb_stats_sites": (i32, [vp, C.c_char_p]),
    "mlb_destroy": (i32, [vp]),
    "mlb_status_name": (C.c_char_p, [i32]),
    "mlb_last_error_message": (C.c_char_p, []),
    "mlb_profile_version": (C.c_uint32, []),
    "mlb_prim_gemm": (i32, [i64, i64, i64, i64, vp, i64, i32, vp, i64, i32, vp, i64, i32, i32, i32, f32,
                            i64, i64, i64, i64, i64, i64, i64, i64, i32, i32, i32, vp, sz, vp]),
    "mlb_prim_gemm_pair": (i32, [i64, i64, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                 i32, i32, i32, vp, sz, vp]),
    "mlb_prim_rmsnorm_fwd": (i32, [vp, vp, i64, i64, f32, vp, vp, vp]),
    "mlb_prim_rmsnorm_bwd": (i32, [vp, vp, vp, vp, i64, i64, vp, vp, vp, sz, vp]),
    "mlb_prim_rope": (i32, [vp, i64, i64, i64, i64, i64, f32, i32, vp]),
    "mlb_prim_attention_fwd": (i32, [i64, i64, i64, i64, vp, vp, vp, i64, vp, vp, i64, i32, vp]),
    "mlb_prim_attention_bwd": (i32, [i64, i64, i64, i64, vp, vp, vp, i64, vp, vp, vp, i64, vp, vp, vp,
                                     i32, vp, sz, vp]),
    "mlb_prim_swiglu_fwd": (i32, [vp, i64, i64, vp, vp]),
    "mlb_prim_swiglu_bwd": (i32, [vp, vp, i64, i64, vp, vp]),
    "mlb_prim_cross_entropy": (i32, [vp, vp, i64, i64, vp, vp, vp, vp]),
    "mlb_prim_embed_scatter": (i32, [vp, vp, i64, i64, i64, vp, vp, sz, vp]),
    "mlb_prim_embed_scatter_noalloc": (i32, [vp, vp, i64, i64, i64, vp, vp]),
    "mlb_prim_adamw": (i32, [vp, vp, vp, vp, i64, f32, f32, f32, f32, f32, i64, vp]),
    "mlb_prim_unary": (i32, [vp, vp, i64, i32, vp]),
    "mlb_diag_mfma": (i32, [i32, vp, vp, vp, vp, i64, vp]),
}


def lib():
    """The loaded HIP library. Raises if it has not been built: there is no fallback.

    PyTorch is imported first: its wheel carries its own HIP runtime, which the
    library must share (both are named libamdhip64.so.7 to the dynamic loader,
    which reuses whichever copy is loaded first). Loading the library first
    would bring in a second runtime for PyTorch, and device memory and streams
    of one would be invalid in the other."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (the HIP runtime the library links against)
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with bitwise_reproducible_fp32_amd/build.py "
                              "(or __graft_entry__.build()); there is no CPU fallback")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise MlbError(status, lib().mlb_last_error_message().decode())


def param_count(cfg: dict) -> int:
    return int(lib().mlb_param_count(C.byref(config(cfg))))


def workspace_bytes(cfg: dict) -> int:
    n = sz()
    check(lib().mlb_workspace_bytes(C.byref(config(cfg)), C.byref(n)))
    return n.value


def safetensors_bytes(cfg: dict, params: np.ndarray) -> bytes:
    """A safetensors file image of `params` (canonical order, float32): the
    parameter array byte for byte behind a JSON tensor table (mlb_safetensors)."""
    p = np.ascontiguousarray(params, dtype=np.float32)
    if p.size != param_count(cfg):
        raise ValueError(f"{p.size} parameters, config needs {param_count(cfg)}")
    c, n = config(cfg), sz()
    check(lib().mlb_safetensors(C.byref(c), None, None, 0, C.byref(n)))
    buf = np.zeros(n.value, np.uint8)
    check(lib().mlb_safetensors(C.byref(c), p.ctypes.data, buf.ctypes.data, n.value, C.byref(n)))
    return buf.tobytes()


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class CardStruct(C.Structure):
    _fields_ = [("tag", C.c_char * 32), ("dtype", C.c_char * 8), ("count", C.c_uint64),
                ("sha256", C.c_uint8 * 32)]


class Model:
    """One training state on the current GPU; the arena is a torch uint8 tensor."""

    def __init__(self, cfg: dict, init_params: np.ndarray | None = None, device: str = "cuda:0", stream=None,
                 seed: int = 0):
        """init_params: step-0 parameters in canonical order, or None to draw
        them from seed with the library's own generator."""
        import torch
        self.cfg = dict(cfg)
        self._c = config(cfg)
        self.n = param_count(cfg)
        init = None
        if init_params is not None:
            init = np.ascontiguousarray(init_params, dtype=np.float32)
            if init.size != self.n:
                raise ValueError(f"init has {init.size} values, the model {self.n}")
        torch.cuda.set_device(torch.device(device))
        nbytes = workspace_bytes(cfg)
        self.arena = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-self.arena.data_ptr()) % 256
        self._stream_obj = stream if stream is not None else torch.cuda.current_stream(device)
        h = vp()
        check(lib().mlb_init(C.byref(self._c), C.c_uint64(seed), None if init is None else init.ctypes.data,
                             self.arena.data_ptr() + off, nbytes, self._stream_obj.cuda_stream, C.byref(h)))
        self.h = h

    def close(self) -> None:
        if getattr(self, "h", None) and self.h.value:
            lib().mlb_destroy(self.h)
            self.h = vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward_loss(self, inputs, targets) -> np.float32:
        """inputs/targets: int32 device tensors of batch*seq_len ids."""
        out = f32()
        check(lib().mlb_forward_loss(self.h, inputs.data_ptr(), targets.data_ptr(), C.byref(out)))
        return np.float32(out.value)

    def backward(self) -> None:
        check(lib().mlb_backward(self.h))

    def adamw_step(self, lr: float) -> None:
        check(lib().mlb_adamw_step(self.h, float(lr)))

    def save(self) -> bytes:
        n = sz()
        check(lib().mlb_save(self.h, None, 0, C.byref(n)))
        buf = np.zeros(n.value, np.uint8)
        check(lib().mlb_save(self.h, buf.ctypes.data, n.value, C.byref(n)))
        return buf.tobytes()

    def load(self, blob: bytes) -> None:
        a = np.frombuffer(blob, dtype=np.uint8)
        check(lib().mlb_load(self.h, a.ctypes.data, a.size))

    def read(self, which: int) -> np.ndarray:
        out = np.empty(self.n, np.float32)
        check(lib().mlb_read(self.h, which, out.ctypes.data, out.nbytes))
        return out

    def export_safetensors(self, path=None) -> bytes:
        """The current parameters as a safetensors image (written to `path` if given)."""
        blob = safetensors_bytes(self.cfg, self.read(PARAMS))
        if path is not None:
            with open(path, "wb") as f:
                f.write(blob)
        return blob

    def read_stage(self, stage: int, layer: int = 0) -> np.ndarray:
        n = sz()
        check(lib().mlb_read_stage(self.h, stage, layer, None, 0, C.byref(n)))
        out = np.empty(n.value, np.float32)
        check(lib().mlb_read_stage(self.h, stage, layer, out.ctypes.data, out.nbytes, C.byref(n)))
        return out

    @property
    def step(self) -> int:
        return int(lib().mlb_step(self.h))

    def _card(self, c: "CardStruct"):
        from .cards import Card
        return Card(c.tag.decode(), c.dtype.decode(), int(c.count), bytes(c.sha256).hex())

    def stage_card(self, stage: int, layer: int = 0):
        c = CardStruct()
        check(lib().mlb_stage_card(self.h, stage, layer, C.byref(c)))
        return self._card(c)

    def state_card(self, which: int):
        c = CardStruct()
        check(lib().mlb_state_card(self.h, which, C.byref(c)))
        return self._card(c)

    def cards(self, state: bool = True) -> list:
        """Identity cards of every stage of the last forward (computation order),
        then of the state arrays."""
        from .cards import card_order
        out = [self.stage_card(st, l) for st, l in card_order(self.cfg["n_layers"])]
        if state:
            out += [self.state_card(w) for w in (PARAMS, GRAD, ADAM_M, ADAM_V)]
        return out

    def infer(self, inputs, targets=None, logits=None):
        """Inference forward on device int32 ids; optional device logits
        [tokens, vocab] to fill; returns the mean loss when targets are given."""
        loss = f32()
        check(lib().mlb_infer(self.h, _ptr(inputs), None if targets is None else _ptr(targets),
                              None if logits is None else _ptr(logits),
                              None if targets is None else C.byref(loss)))
        return None if targets is None else np.float32(loss.value)

    def greedy_next(self, inputs, position: int) -> np.ndarray:
        """Next token of every sequence after `position` (lowest index on ties)."""
        out = np.empty(self.cfg["batch"], np.int32)
        check(lib().mlb_greedy_next(self.h, _ptr(inputs), int(position), out.ctypes.data))
        return out

    def set_overlap(self, on: bool) -> None:
        """Backward weight-gradient work on the library's second stream (default off)."""
        check(lib().mlb_set_overlap(self.h, int(bool(on))))

    def stats_enable(self, on: bool = True) -> None:
        check(lib().mlb_stats_enable(self.h, int(on)))

    def stats_sites(self, sites=None) -> None:
        """Time only these call sites (an iterable of names); None times all."""
        check(lib().mlb_stats_sites(self.h, None if not sites else ",".join(sites).encode()))

    def stats(self) -> list[dict]:
        """Per-site launch statistics since stats_enable (see mlb_stats_read)."""
        n = i32()
        check(lib().mlb_stats_read(self.h, None, 0, C.byref(n)))
        arr = (Stat * max(1, n.value))()
        check(lib().mlb_stats_read(self.h, arr, n.value, C.byref(n)))
        return [dict(site=a.site.decode(), kernel=a.kernel.decode(), launches=a.launches, ms=a.ms,
                     flops=a.flops, bytes=a.bytes) for a in arr[:n.value]]


# ------------------------------------------------------------------ primitives
def gemm(A, B, C_, M, N, K, lda, a_kc, ldb, b_kc, ldc, kseg=0, krange=0, outmask=0, mode=0, scale=1.0,
         batch=1, heads=1, sA=(0, 0), sB=(0, 0), sC=(0, 0), tile=-1, split=-1, simple=0, ws=None,
         stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(lib().mlb_prim_gemm(M, N, K, kseg, _ptr(A), lda, int(a_kc), _ptr(B), ldb, int(b_kc), _ptr(C_), ldc,
                              krange, outmask, mode, float(scale), batch, heads, sA[0], sA[1], sB[0], sB[1],
                              sC[0], sC[1], tile, split, simple, _ptr(ws), ws_bytes, _stream(stream)))


def gemm_pair(p0, p1, K, a_kc, b_kc, mode=0, ws=None, stream=None):
    """p0, p1: (A, lda, B, ldb, C, ldc, M, N) of two contractions over K with one layout."""
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    (A0, lda0, B0, ldb0, C0, ldc0, M0, N0), (A1, lda1, B1, ldb1, C1, ldc1, M1, N1) = p0, p1
    check(lib().mlb_prim_gemm_pair(M0, N0, M1, N1, K, _ptr(A0), lda0, _ptr(B0), ldb0, _ptr(C0), ldc0, _ptr(A1), lda1,
                                   _ptr(B1), ldb1, _ptr(C1), ldc1, int(a_kc), int(b_kc), mode, _ptr(ws), ws_bytes,
                                   _stream(stream)))


def rmsnorm_fwd(x, w, eps, y, r, stream=None):
    rows, d = x.shape
    check(lib().mlb_prim_rmsnorm_fwd(_ptr(x), _ptr(w), rows, d, float(eps), _ptr(y), _ptr(r), _stream(stream)))


def rmsnorm_bwd(dy, x, w, r, dx, dw, ws, stream=None):
    rows, d = x.shape
    check(lib().mlb_prim_rmsnorm_bwd(_ptr(dy), _ptr(x), _ptr(w), _ptr(r), rows, d, _ptr(dx), _ptr(dw), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def rope(x, B, T, H, hd, ld, theta, backward=0, stream=None):
    check(lib().mlb_prim_rope(_ptr(x), B, T, H, hd, ld, float(theta), int(backward), _stream(stream)))


def attention_fwd(B, H, T, hd, q, k, v, ld, P, O, ldo, tiled=0, stream=None):
    check(lib().mlb_prim_attention_fwd(B, H, T, hd, _ptr(q), _ptr(k), _ptr(v), ld, _ptr(P), _ptr(O), ldo,
                                       int(tiled), _stream(stream)))


def attention_bwd(B, H, T, hd, q, k, v, ld, P, O, dO, ldo, dq, dk, dv, ws, tiled=0, stream=None):
    check(lib().mlb_prim_attention_bwd(B, H, T, hd, _ptr(q), _ptr(k), _ptr(v), ld, _ptr(P), _ptr(O), _ptr(dO), ldo,
                                       _ptr(dq), _ptr(dk), _ptr(dv), int(tiled), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))


def tiled_to_dense(P: np.ndarray, T: int) -> np.ndarray:
    """[..., T*T] in the 32x32 tile layout -> [..., T, T] row-major (host, numpy)."""
    nt = T // 32
    x = P.reshape(-1, nt, nt, 32, 32)
    return np.ascontiguousarray(x.transpose(0, 1, 3, 2, 4)).reshape(-1, T, T)


def swiglu_fwd(gu, rows, F, a, stream=None):
    check(lib().mlb_prim_swiglu_fwd(_ptr(gu), rows, F, _ptr(a), _stream(stream)))


def swiglu_bwd(dA, gu, rows, F, dgu, stream=None):
    check(lib().mlb_prim_swiglu_bwd(_ptr(dA), _ptr(gu), rows, F, _ptr(dgu), _stream(stream)))


def cross_entropy(logits, targets, N, V, loss_rows, dl, loss_dev, stream=None):
    check(lib().mlb_prim_cross_entropy(_ptr(logits), _ptr(targets), N, V, _ptr(loss_rows), _ptr(dl),
                                       _ptr(loss_dev), _stream(stream)))


def embed_scatter(ids, dh, N, d, V, dE, ws, stream=None):
    check(lib().mlb_prim_embed_scatter(_ptr(ids), _ptr(dh), N, d, V, _ptr(dE), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))


def adamw(p, g, m, v, n, lr, b1, b2, eps, wd, t, stream=None):
    check(lib().mlb_prim_adamw(_ptr(p), _ptr(g), _ptr(m), _ptr(v), n, float(lr), float(b1), float(b2),
                               float(eps), float(wd), int(t), _stream(stream)))


def unary(x, y, n, which, stream=None):
    check(lib().mlb_prim_unary(_ptr(x), _ptr(y), n, which, _stream(stream)))


def diag_mfma(variant, A, B, Cin, D, nwaves, stream=None):
    check(lib().mlb_diag_mfma(variant, _ptr(A), _ptr(B), _ptr(Cin), _ptr(D), nwaves, _stream(stream)))
