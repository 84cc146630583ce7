"""Thin ctypes binding of libmtdec.so (include/mt.h).

Argument marshalling only: every step of the decoder runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.
There is no fallback: if the library is not built, importing this module
fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmtdec.so")

MT_OK = 0
MT_ERR_INVALID_ARG = -1
MT_ERR_CACHE_FULL = -2
MT_ERR_HIP = -3
MT_ERR_OOM = -4
MT_ERR_UNSUPPORTED = -5

MT_DECODE_AUTO = 0
MT_DECODE_KERNELS = 1
MT_DECODE_PERSISTENT = 2
MT_DECODE_BATCHED = 3

MT_FLAG_W4A8 = 1
MT_FLAG_DENSE_F16 = 2
MT_FLAG_DENSE_F32 = 4

# Names declared in include/mt.h; the CPU test checks the library exports all.
EXPORTED = ("mt_pack_int4", "mt_pack_f16", "mt_create", "mt_prefill", "mt_decode_step", "mt_reset",
            "mt_position", "mt_kv_cache", "mt_check", "mt_set_decode_path", "mt_destroy",
            "mt_last_error", "mt_debug_dequant", "mt_debug_matmul", "mt_debug_trace",
            "mt_prefill_seq", "mt_reset_seq", "mt_position_seq", "mt_cfg_combine", "mt_prefill_noalloc")


class mt_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("vocab", ctypes.c_int32), ("group", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("t_cap", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class mt_int4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p)]


class mt_weights(ctypes.Structure):
    _fields_ = [("tok_emb", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("ln_final", ctypes.c_void_p), ("ln", ctypes.c_void_p),
                ("proj", ctypes.POINTER(mt_int4)), ("dense", ctypes.POINTER(ctypes.c_void_p))]


class MTError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed with status {code}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m audio_midi_transformer_amd.build` "
                          "(or __graft_entry__.build())")
    # torch carries its own HIP runtime; it must be loaded before this
    # library's.  In the other order this library's device queries fail
    # (mt_create reports "hipGetDevice failed").
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.mt_pack_int4.argtypes = [vp, i32, i32, vp, vp]
    L.mt_pack_f16.argtypes = [vp, i64, vp]
    L.mt_create.argtypes = [ctypes.POINTER(mt_config), ctypes.POINTER(mt_weights), ctypes.c_int, vp,
                            ctypes.POINTER(vp)]
    L.mt_prefill.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp]
    L.mt_decode_step.argtypes = [vp, vp, vp, vp, vp]
    L.mt_reset.argtypes = [vp]
    L.mt_position.argtypes = [vp, ctypes.POINTER(i32)]
    L.mt_kv_cache.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp)]
    L.mt_check.argtypes = [vp]
    L.mt_set_decode_path.argtypes = [vp, i32]
    L.mt_destroy.argtypes = [vp]
    L.mt_destroy.restype = None
    L.mt_last_error.argtypes = []
    L.mt_last_error.restype = ctypes.c_char_p
    L.mt_debug_dequant.argtypes = [vp, i32, i32, vp, vp]
    L.mt_debug_matmul.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    L.mt_debug_trace.argtypes = [vp, vp, i64]
    L.mt_prefill_seq.argtypes = [vp, i32, vp, i32, vp, i32, vp, vp, vp]
    L.mt_prefill_noalloc.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp]
    L.mt_reset_seq.argtypes = [vp, i32]
    L.mt_position_seq.argtypes = [vp, i32, ctypes.POINTER(i32)]
    L.mt_cfg_combine.argtypes = [vp, i32, i32, ctypes.c_float, vp, vp, vp, vp]
    for name in ("mt_pack_int4", "mt_pack_f16", "mt_create", "mt_prefill", "mt_decode_step", "mt_reset",
                 "mt_position", "mt_kv_cache", "mt_check", "mt_set_decode_path",
                 "mt_debug_dequant", "mt_debug_matmul", "mt_debug_trace",
                 "mt_prefill_seq", "mt_reset_seq", "mt_position_seq", "mt_cfg_combine", "mt_prefill_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def check(rc: int, where: str) -> None:
    if rc != MT_OK:
        raise MTError(rc, where, lib().mt_last_error().decode(errors="replace"))


# ---------------------------------------------------------------- C names


def mt_pack_int4(W: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Host packer: [N, K] float32 -> (q uint8 [N, K/2], s float32 [N, K/32])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    q = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N, K // 32), dtype=np.float32)
    check(lib().mt_pack_int4(W.ctypes.data, N, K, q.ctypes.data, s.ctypes.data), "mt_pack_int4")
    return q, s


def mt_pack_f16(W: np.ndarray) -> np.ndarray:
    """Host binary16 packer: float32 array -> float16 array of the same shape
    (round to nearest, ties to even, done by the library)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    out = np.empty(W.shape, dtype=np.float16)
    check(lib().mt_pack_f16(W.ctypes.data, W.size, out.ctypes.data), "mt_pack_f16")
    return out


def cfg_combine(logits, cfg: float, guided=None, next=None, token_pair=None, store_guided: bool = True,
                stream=None):
    """mt_cfg_combine on device tensors: logits [2 Np, V] float32 (rows
    0 .. Np-1 conditional, row Np + i the partner of row i) -> (guided
    [Np, V] or None, next [Np] int64, token_pair [2 Np] int64)."""
    import torch
    n2, V = logits.shape
    if n2 % 2:
        raise ValueError("cfg_combine needs an even number of rows")
    Np = n2 // 2
    if store_guided and guided is None:
        guided = torch.empty((Np, V), dtype=torch.float32, device=logits.device)
    if next is None:
        next = torch.empty((Np,), dtype=torch.int64, device=logits.device)
    if token_pair is None:
        token_pair = torch.empty((n2,), dtype=torch.int64, device=logits.device)
    check(lib().mt_cfg_combine(_ptr(logits), Np, V, float(cfg), _ptr(guided) if store_guided else None,
                               _ptr(next), _ptr(token_pair), _stream(stream)), "mt_cfg_combine")
    return (guided if store_guided else None), next, token_pair


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def hip_copy(dst_ptr: int, src_ptr: int, nbytes: int, stream=None) -> None:
    """Device-to-device copy on the given stream (test and bench helper)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_void_p]
    rc = hip.hipMemcpyAsync(dst_ptr, src_ptr, nbytes, 3, _stream(stream))
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed with {rc}")


class Decoder:
    """Owns one mt_model.  Inputs and outputs are torch tensors on the GPU."""

    def __init__(self, weights, batch: int, t_cap: int, eps: float = 1e-5,
                 packed: Optional[Sequence[Tuple[np.ndarray, np.ndarray]]] = None, flags: int = 0):
        import torch
        s = weights.shape
        self.shape, self.batch, self.t_cap = s, batch, t_cap
        self.L, self.d, self.H, self.F, self.V = s.n_layers, s.d_model, s.n_heads, s.d_ff, s.vocab
        cfg = mt_config(s.n_layers, s.d_model, s.n_heads, 64, s.d_ff, s.vocab, 32, batch, t_cap,
                        eps, flags)
        keep = []
        dense_dt = np.float16 if flags & MT_FLAG_DENSE_F16 else np.float32 if flags & MT_FLAG_DENSE_F32 else None
        projs = (mt_int4 * (4 * s.n_layers))()
        dense = None
        if dense_dt is None:
            if packed is None:
                packed = pack_weights(weights)
            for i, (q, sc) in enumerate(packed):
                keep += [q, sc]
                projs[i] = mt_int4(q.ctypes.data, sc.ctypes.data)
        else:
            dense = (ctypes.c_void_p * (4 * s.n_layers))()
            for i, W in enumerate(dense_weights(weights, dense_dt)):
                keep.append(W)
                dense[i] = W.ctypes.data
        ln = np.ascontiguousarray(np.stack([np.stack([weights.ln1_g[l], weights.ln1_b[l],
                                                      weights.ln2_g[l], weights.ln2_b[l]])
                                            for l in range(s.n_layers)]), dtype=np.float32)
        lnf = np.ascontiguousarray(np.stack([weights.lnf_g, weights.lnf_b]), dtype=np.float32)
        emb = np.ascontiguousarray(weights.tok_emb, dtype=np.float32)
        head = np.ascontiguousarray(weights.lm_head, dtype=np.float32)
        w = mt_weights(emb.ctypes.data, head.ctypes.data, lnf.ctypes.data, ln.ctypes.data, projs,
                       ctypes.cast(dense, ctypes.POINTER(ctypes.c_void_p)) if dense is not None else None)
        h = ctypes.c_void_p()
        check(lib().mt_create(ctypes.byref(cfg), ctypes.byref(w), 0, _stream(None), ctypes.byref(h)),
              "mt_create")
        self._h = h
        self.device = torch.device("cuda", torch.cuda.current_device())

    # -- lifetime
    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().mt_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    # -- calls
    def _outputs(self, logits, nxt):
        import torch
        if logits is None:
            logits = torch.empty((self.batch, self.V), dtype=torch.float32, device=self.device)
        if nxt is None:
            nxt = torch.empty((self.batch,), dtype=torch.int64, device=self.device)
        return logits, nxt

    def prefill(self, tokens=None, prefix=None, logits=None, next=None, stream=None):
        logits, next = self._outputs(logits, next)
        S = 0 if tokens is None else int(tokens.shape[-1])
        P = 0 if prefix is None else int(prefix.shape[-2])
        if tokens is not None:
            assert tokens.dtype.is_floating_point is False and tokens.is_contiguous()
        if prefix is not None:
            assert prefix.is_contiguous() and prefix.shape[-1] == self.d
        check(lib().mt_prefill(self._h, _ptr(tokens), S, _ptr(prefix), P, _ptr(logits), _ptr(next),
                               _stream(stream)), "mt_prefill")
        return logits, next

    def prefill_noalloc(self, tokens=None, prefix=None, logits=None, next=None, stream=None):
        """mt_prefill_noalloc: mt_prefill on the library's fixed device
        workspace (no allocation by the library)."""
        logits, next = self._outputs(logits, next)
        S = 0 if tokens is None else int(tokens.shape[-1])
        P = 0 if prefix is None else int(prefix.shape[-2])
        if prefix is not None:
            assert prefix.is_contiguous() and prefix.shape[-1] == self.d
        check(lib().mt_prefill_noalloc(self._h, _ptr(tokens), S, _ptr(prefix), P, _ptr(logits), _ptr(next),
                                       _stream(stream)), "mt_prefill_noalloc")
        return logits, next

    def prefill_seq(self, b: int, tokens=None, prefix=None, logits=None, next=None, stream=None):
        """Sequence b only (ragged batch): tokens [S] and/or prefix [P, d] ->
        (logits [V], next [1])."""
        import torch
        if logits is None:
            logits = torch.empty((self.V,), dtype=torch.float32, device=self.device)
        if next is None:
            next = torch.empty((1,), dtype=torch.int64, device=self.device)
        S = 0 if tokens is None else int(tokens.shape[-1])
        P = 0 if prefix is None else int(prefix.shape[-2])
        if prefix is not None:
            assert prefix.is_contiguous() and prefix.shape[-1] == self.d
        check(lib().mt_prefill_seq(self._h, b, _ptr(tokens), S, _ptr(prefix), P, _ptr(logits), _ptr(next),
                                   _stream(stream)), "mt_prefill_seq")
        return logits, next

    def reset_seq(self, b: int) -> None:
        check(lib().mt_reset_seq(self._h, b), "mt_reset_seq")

    def position_seq(self, b: int) -> int:
        t = ctypes.c_int32()
        check(lib().mt_position_seq(self._h, b, ctypes.byref(t)), "mt_position_seq")
        return t.value

    def decode_step(self, token, logits=None, next=None, stream=None):
        logits, next = self._outputs(logits, next)
        check(lib().mt_decode_step(self._h, _ptr(token), _ptr(logits), _ptr(next), _stream(stream)),
              "mt_decode_step")
        return logits, next

    def reset(self) -> None:
        check(lib().mt_reset(self._h), "mt_reset")

    @property
    def position(self) -> int:
        t = ctypes.c_int32()
        check(lib().mt_position(self._h, ctypes.byref(t)), "mt_position")
        return t.value

    def check(self) -> None:
        check(lib().mt_check(self._h), "mt_check")

    def set_decode_path(self, path: int) -> None:
        check(lib().mt_set_decode_path(self._h, path), "mt_set_decode_path")

    def kv_cache(self, stream=None):
        """Copies of the K and V caches as torch tensors [L, B, t_cap, H, 64]."""
        import torch
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        check(lib().mt_kv_cache(self._h, ctypes.byref(k), ctypes.byref(v)), "mt_kv_cache")
        shape = (self.L, self.batch, self.t_cap, self.H, 64)
        out = []
        for p in (k, v):
            t = torch.empty(shape, dtype=torch.float32, device=self.device)
            hip_copy(t.data_ptr(), p.value, t.numel() * 4, stream)
            out.append(t)
        return out[0], out[1]

    def kv_pointers(self) -> Tuple[int, int]:
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        check(lib().mt_kv_cache(self._h, ctypes.byref(k), ctypes.byref(v)), "mt_kv_cache")
        return k.value, v.value

    def debug_dequant(self, layer: int, proj: int, stream=None):
        import torch
        N, K = self.proj_shape(proj)
        out = torch.empty((N, K), dtype=torch.float32, device=self.device)
        check(lib().mt_debug_dequant(self._h, layer, proj, _ptr(out), _stream(stream)), "mt_debug_dequant")
        return out

    def debug_matmul(self, layer: int, proj: int, x, force_gemm: bool = False, stream=None):
        import torch
        N, K = self.proj_shape(proj)
        assert x.shape[-1] == K and x.is_contiguous()
        M = int(x.shape[0])
        y = torch.empty((M, N), dtype=torch.float32, device=self.device)
        check(lib().mt_debug_matmul(self._h, layer, proj | (0x100 if force_gemm else 0), _ptr(x), M,
                                    _ptr(y), _stream(stream)), "mt_debug_matmul")
        return y

    def debug_trace(self) -> np.ndarray:
        """Phase timestamps of the last persistent step: [256, L + 1, 24]
        (needs MT_TRACE=1 when the model was created)."""
        out = np.zeros((256, self.L + 1, 24), dtype=np.uint64)
        check(lib().mt_debug_trace(self._h, out.ctypes.data, out.size), "mt_debug_trace")
        return out

    def proj_shape(self, proj: int) -> Tuple[int, int]:
        d, F = self.d, self.F
        return [(3 * d, d), (d, d), (F, d), (d, F)][proj]


def dense_weights(weights, dtype=np.float32):
    """Every projection as a contiguous row-major array of `dtype`, in
    mt_weights.dense order; float16 values come from the library's packer
    (mt_pack_f16: round to nearest, ties to even)."""
    out = []
    for l in range(weights.shape.n_layers):
        for W in (weights.w_qkv[l], weights.w_o[l], weights.w_up[l], weights.w_down[l]):
            W = np.ascontiguousarray(W, dtype=np.float32)
            out.append(mt_pack_f16(W) if dtype == np.float16 else W)
    return out


def pack_weights(weights):
    """Canonical INT4 form of every projection, in mt_weights.proj order."""
    out = []
    for l in range(weights.shape.n_layers):
        for W in (weights.w_qkv[l], weights.w_o[l], weights.w_up[l], weights.w_down[l]):
            out.append(mt_pack_int4(W))
    return out
