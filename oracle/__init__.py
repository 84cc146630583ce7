"""CPU oracle for the MuScriptor INT4 decoder step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The library path never imports this
package, and this package never imports the library.  See mt_oracle.c for
what is computed and which passages of the pages each step follows.

Parity status: every exported function is pinned by tests/test_oracle_pins.py
(closed forms, special cases, invariants, brute force on tiny inputs).
Fidelity to the real MuScriptor checkpoint is parity unpinned: the weights
are gated and absent, and the positional scheme is not on the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mt_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libmt_oracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: no fast-math, no FP contraction."""
    if os.path.exists(_LIB_PATH) and not force:
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
           "-Wall", "-Wextra", "-Wno-unused-parameter",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        i64 = ctypes.c_int64
        L.oracle_quantize_int4.argtypes = [_f32p, i64, i64, _u8p, _f32p]
        L.oracle_dequantize_int4.argtypes = [_u8p, _f32p, i64, i64, _f32p]
        L.oracle_matmul.argtypes = [_f32p, i64, i64, _f32p, i64, _f32p]
        L.oracle_round_half.argtypes = [_f32p, i64, _f32p]
        L.oracle_quantize_act_int8.argtypes = [_f32p, i64, i64, _i8p, _f32p]
        L.oracle_matmul_w4a8.argtypes = [_f32p, i64, i64, _u8p, _f32p, i64, _f32p]
        L.oracle_model_set_w4a8.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.oracle_layernorm.argtypes = [_f32p, i64, i64, _f32p, _f32p, ctypes.c_float, _f32p]
        L.oracle_gelu.argtypes = [_f32p, i64, _f32p]
        L.oracle_attention.argtypes = [_f32p, _f32p, _f32p, i64, i64, _f32p]
        L.oracle_model_new.argtypes = [i64, i64, i64, i64, i64, i64, i64, ctypes.c_float]
        L.oracle_model_new.restype = ctypes.c_void_p
        L.oracle_model_free.argtypes = [ctypes.c_void_p]
        L.oracle_model_free.restype = None
        L.oracle_model_set_embed.argtypes = [ctypes.c_void_p, _f32p, _f32p, _f32p, _f32p]
        L.oracle_model_set_layer.argtypes = [ctypes.c_void_p, i64] + [_f32p] * 8 + [ctypes.c_int]
        L.oracle_model_position.argtypes = [ctypes.c_void_p]
        L.oracle_model_position.restype = i64
        L.oracle_model_reset.argtypes = [ctypes.c_void_p]
        L.oracle_model_reset.restype = None
        L.oracle_model_kv.argtypes = [ctypes.c_void_p, ctypes.POINTER(_f32p), ctypes.POINTER(_f32p)]
        L.oracle_model_forward.argtypes = [ctypes.c_void_p, _i64p, i64, _f32p, i64, _f32p, _i64p, _f32p]
        L.oracle_model_forward_seq.argtypes = [ctypes.c_void_p, i64, _i64p, i64, _f32p, i64, _f32p, _i64p]
        L.oracle_model_position_seq.argtypes = [ctypes.c_void_p, i64]
        L.oracle_model_position_seq.restype = i64
        L.oracle_model_reset_seq.argtypes = [ctypes.c_void_p, i64]
        L.oracle_cfg_combine.argtypes = [_f32p, i64, i64, ctypes.c_float, _f32p, _i64p]
        _lib = L
    return _lib


def _f32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def quantize_int4(W: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """[N, K] float32 -> (q uint8 [N, K/2], s float32 [N, K/32])."""
    W = _f32(W)
    N, K = W.shape
    q = np.zeros((N, K // 2), dtype=np.uint8)
    s = np.zeros((N, K // 32), dtype=np.float32)
    _check(lib().oracle_quantize_int4(_p(W, _f32p), N, K, _p(q, _u8p), _p(s, _f32p)), "quantize")
    return q, s


def dequantize_int4(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = _f32(s)
    N, K = q.shape[0], q.shape[1] * 2
    out = np.zeros((N, K), dtype=np.float32)
    _check(lib().oracle_dequantize_int4(_p(q, _u8p), _p(s, _f32p), N, K, _p(out, _f32p)), "dequantize")
    return out


def matmul(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    """A [M, K] times W [N, K] transposed -> [M, N]."""
    A, W = _f32(A), _f32(W)
    M, K = A.shape
    N = W.shape[0]
    assert W.shape[1] == K
    Y = np.zeros((M, N), dtype=np.float32)
    _check(lib().oracle_matmul(_p(A, _f32p), M, K, _p(W, _f32p), N, _p(Y, _f32p)), "matmul")
    return Y


def round_half(X: np.ndarray) -> np.ndarray:
    """IEEE binary16 rounding (ties to even) of float32 values, returned as float32."""
    X = _f32(X)
    out = np.empty_like(X)
    _check(lib().oracle_round_half(_p(X, _f32p), X.size, _p(out, _f32p)), "round_half")
    return out


def cfg_combine(logits: np.ndarray, cfg: float) -> Tuple[np.ndarray, np.ndarray]:
    """Classifier-free guidance over row pairs: logits [2 Np, V] (rows
    0 .. Np-1 conditional, row Np + i the unconditional partner of row i)
    -> (guided float32 [Np, V], next int64 [Np])."""
    lg = _f32(logits)
    n2, V = lg.shape
    assert n2 % 2 == 0 and n2 > 0
    g = np.empty((n2 // 2, V), dtype=np.float32)
    nx = np.empty(n2 // 2, dtype=np.int64)
    _check(lib().oracle_cfg_combine(_p(lg, _f32p), n2 // 2, V, float(cfg), _p(g, _f32p), _p(nx, _i64p)),
           "cfg_combine")
    return g, nx


def quantize_act_int8(X: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """W4A8 activation codes: [M, K] float32 -> (codes int8 [M, K], scales float32 [M, K/32])."""
    X = _f32(np.atleast_2d(X))
    M, K = X.shape
    q = np.zeros((M, K), dtype=np.int8)
    s = np.zeros((M, K // 32), dtype=np.float32)
    _check(lib().oracle_quantize_act_int8(_p(X, _f32p), M, K, _p(q, _i8p), _p(s, _f32p)), "quantize_act")
    return q, s


def matmul_w4a8(A: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W4A8 product of rows A [M, K] with packed INT4 weights (q [N, K/2], s [N, K/32]) -> [M, N]."""
    A = _f32(np.atleast_2d(A))
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = _f32(s)
    M, K = A.shape
    N = q.shape[0]
    assert q.shape[1] * 2 == K
    Y = np.zeros((M, N), dtype=np.float32)
    _check(lib().oracle_matmul_w4a8(_p(A, _f32p), M, K, _p(q, _u8p), _p(s, _f32p), N, _p(Y, _f32p)),
           "matmul_w4a8")
    return Y


def layernorm(X: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    X = _f32(np.atleast_2d(X))
    M, d = X.shape
    g, b = _f32(g), _f32(b)
    Y = np.zeros_like(X)
    _check(lib().oracle_layernorm(_p(X, _f32p), M, d, _p(g, _f32p), _p(b, _f32p), eps,
                                  _p(Y, _f32p)), "layernorm")
    return Y


def gelu(X: np.ndarray) -> np.ndarray:
    X = _f32(X)
    Y = np.zeros_like(X)
    _check(lib().oracle_gelu(_p(X, _f32p), X.size, _p(Y, _f32p)), "gelu")
    return Y


def attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray) -> np.ndarray:
    """q [H, 64]; kc, vc [T, H, 64] -> [H, 64]."""
    q, kc, vc = _f32(q), _f32(kc), _f32(vc)
    T, H = kc.shape[0], kc.shape[1]
    out = np.zeros((H, 64), dtype=np.float32)
    _check(lib().oracle_attention(_p(q, _f32p), _p(kc, _f32p), _p(vc, _f32p), T, H,
                                  _p(out, _f32p)), "attention")
    return out


class OracleModel:
    """B sequences in lockstep over one fixed-capacity FP32 KV cache."""

    def __init__(self, n_layers: int, d_model: int, n_heads: int, d_ff: int, vocab: int,
                 batch: int, t_cap: int, eps: float = 1e-5):
        self.L, self.d, self.H, self.F, self.V = n_layers, d_model, n_heads, d_ff, vocab
        self.B, self.t_cap = batch, t_cap
        self._h = lib().oracle_model_new(n_layers, d_model, n_heads, d_ff, vocab, batch, t_cap, eps)
        if not self._h:
            raise ValueError("oracle_model_new rejected the configuration or ran out of memory")

    @classmethod
    def from_weights(cls, w, batch: int, t_cap: int, eps: float = 1e-5, quantize: bool = True,
                     w4a8: bool = False, dense: Optional[str] = None):
        """dense: None (INT4 unless quantize is False), "f32" (unquantised
        projections) or "f16" (projections rounded to binary16 first)."""
        s = w.shape
        m = cls(s.n_layers, s.d_model, s.n_heads, s.d_ff, s.vocab, batch, t_cap, eps)
        if w4a8:
            m.set_w4a8(True)
        if dense is not None:
            if dense not in ("f16", "f32") or w4a8:
                raise ValueError(f"dense must be 'f16' or 'f32' without w4a8 (got {dense!r})")
            quantize = False
        conv = round_half if dense == "f16" else (lambda a: a)
        m.set_embed(w.tok_emb, w.lm_head, w.lnf_g, w.lnf_b)
        for l in range(s.n_layers):
            m.set_layer(l, conv(w.w_qkv[l]), conv(w.w_o[l]), conv(w.w_up[l]), conv(w.w_down[l]),
                        w.ln1_g[l], w.ln1_b[l], w.ln2_g[l], w.ln2_b[l], quantize=quantize)
        return m

    def close(self) -> None:
        if self._h:
            lib().oracle_model_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_embed(self, tok_emb, lm_head, lnf_g, lnf_b) -> None:
        arrs = [_f32(x) for x in (tok_emb, lm_head, lnf_g, lnf_b)]
        _check(lib().oracle_model_set_embed(self._h, *[_p(a, _f32p) for a in arrs]), "set_embed")

    def set_layer(self, l, wqkv, wo, wup, wdown, g1, b1, g2, b2, quantize: bool = True) -> None:
        arrs = [_f32(x) for x in (wqkv, wo, wup, wdown, g1, b1, g2, b2)]
        _check(lib().oracle_model_set_layer(self._h, l, *[_p(a, _f32p) for a in arrs],
                                            1 if quantize else 0), "set_layer")

    def set_w4a8(self, on: bool) -> None:
        """Run the four projections as the W4A8 product (INT8 activation codes)."""
        _check(lib().oracle_model_set_w4a8(self._h, 1 if on else 0), "set_w4a8")

    @property
    def position(self) -> int:
        return int(lib().oracle_model_position(self._h))

    def reset(self) -> None:
        lib().oracle_model_reset(self._h)

    def forward(self, tokens: Optional[np.ndarray] = None, prefix: Optional[np.ndarray] = None,
                return_hidden: bool = False):
        """tokens [B, S] int64 and/or prefix [B, P, d] -> (logits [B, V], next [B])."""
        B, d = self.B, self.d
        if tokens is None:
            tokens = np.zeros((B, 0), dtype=np.int64)
        if prefix is None:
            prefix = np.zeros((B, 0, d), dtype=np.float32)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64).reshape(B, -1)
        prefix = _f32(prefix).reshape(B, -1, d)
        S, P = tokens.shape[1], prefix.shape[1]
        logits = np.zeros((B, self.V), dtype=np.float32)
        nxt = np.zeros((B,), dtype=np.int64)
        hid = np.zeros((B, d), dtype=np.float32)
        rc = lib().oracle_model_forward(self._h, _p(tokens, _i64p) if S else None, S,
                                        _p(prefix, _f32p) if P else None, P,
                                        _p(logits, _f32p), _p(nxt, _i64p), _p(hid, _f32p))
        if rc == -2:
            raise OverflowError("oracle cache full")
        _check(rc, "forward")
        return (logits, nxt, hid) if return_hidden else (logits, nxt)

    def position_seq(self, b: int) -> int:
        return int(lib().oracle_model_position_seq(self._h, b))

    def reset_seq(self, b: int) -> None:
        _check(lib().oracle_model_reset_seq(self._h, b), "reset_seq")

    def forward_seq(self, b: int, tokens: Optional[np.ndarray] = None, prefix: Optional[np.ndarray] = None):
        """Sequence b only (ragged batch): tokens [S] int64 and/or prefix [P, d],
        appended at that sequence's own position -> (logits [V], next)."""
        d = self.d
        tokens = np.zeros((0,), np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64).reshape(-1)
        prefix = np.zeros((0, d), np.float32) if prefix is None else _f32(prefix).reshape(-1, d)
        S, P = tokens.shape[0], prefix.shape[0]
        logits = np.zeros((self.V,), dtype=np.float32)
        nxt = np.zeros((1,), dtype=np.int64)
        rc = lib().oracle_model_forward_seq(self._h, b, _p(tokens, _i64p) if S else None, S,
                                            _p(prefix, _f32p) if P else None, P, _p(logits, _f32p), _p(nxt, _i64p))
        if rc == -2:
            raise OverflowError("oracle cache full")
        _check(rc, "forward_seq")
        return logits, int(nxt[0])

    def kv(self) -> Tuple[np.ndarray, np.ndarray]:
        """Views of the cache, [L, B, T_cap, H, 64] each (valid until close)."""
        k, v = _f32p(), _f32p()
        _check(lib().oracle_model_kv(self._h, ctypes.byref(k), ctypes.byref(v)), "kv")
        shape = (self.L, self.B, self.t_cap, self.H, 64)
        n = int(np.prod(shape))
        K = np.ctypeslib.as_array(k, shape=(n,)).reshape(shape)
        Vv = np.ctypeslib.as_array(v, shape=(n,)).reshape(shape)
        return K, Vv
