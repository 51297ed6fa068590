"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only callers.  The GPU library never imports this
package, and this package imports nothing from the GPU library.

Arrays are numpy: bf16 tensors travel as their raw uint16 bit patterns,
metadata as int32, results come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Result codes of oracle_check (mirrors the enum in oracle.c).
OK, BAD_SHAPE, BAD_CU_Q_LENS, BAD_CONTEXT, TOO_LONG, BAD_PAGE, BAD_SLOT, DUP_SLOT = range(8)


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into a shared library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load(path: str | None = None):
    """Load the compiled oracle, compiling it first only if it is not built."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    i32, f64, P = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_check.restype = i32
    lib.oracle_check.argtypes = [i32] * 8 + [P] * 4
    lib.oracle_scatter.restype = None
    lib.oracle_scatter.argtypes = [i32] * 4 + [P] * 5
    lib.oracle_attention.restype = None
    lib.oracle_attention.argtypes = [i32] * 7 + [P] * 6 + [f64, i32, P]
    lib.oracle_attention_rows.restype = None
    lib.oracle_attention_rows.argtypes = [i32] * 7 + [P] * 6 + [f64, i32, i32, P, P, P]
    lib.oracle_num_threads.restype = i32
    lib.oracle_num_threads.argtypes = []
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def num_threads(lib=None) -> int:
    return (lib or load()).oracle_num_threads()


def check(page_table, cu_q_lens, context_lens, slot_mapping, *, num_q_heads, num_kv_heads,
          head_dim, page_size, num_pages, lib=None) -> int:
    """Preconditions of the call; returns OK or the first violated rule."""
    lib = lib or load()
    pt, cu, ctx, sm = _i32(page_table), _i32(cu_q_lens), _i32(context_lens), _i32(slot_mapping)
    R = len(ctx)
    T = int(sm.shape[0])
    max_pages = pt.shape[1] if pt.ndim == 2 else 0
    if cu.shape[0] != R + 1:
        return BAD_CU_Q_LENS
    return lib.oracle_check(R, T, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                            max_pages, _ptr(pt), _ptr(cu), _ptr(ctx), _ptr(sm))


def scatter(k_cache, v_cache, k_new, v_new, slot_mapping, *, page_size, lib=None):
    """Return copies of the caches with every new K/V row written to its slot."""
    lib = lib or load()
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    kn, vn, sm = _u16(k_new), _u16(v_new), _i32(slot_mapping)
    T, Hkv, D = kn.shape
    lib.oracle_scatter(T, Hkv, D, page_size, _ptr(kn), _ptr(vn), _ptr(sm), _ptr(kc), _ptr(vc))
    return kc, vc


def attention(q, k_cache, v_cache, page_table, cu_q_lens, context_lens, *, scale, causal,
              lib=None) -> np.ndarray:
    """Exact softmax attention of every query row; returns float64 [T, Hq, D]."""
    lib = lib or load()
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    pt, cu, ctx = _i32(page_table), _i32(cu_q_lens), _i32(context_lens)
    T, Hq, D = q.shape
    _, S, Hkv, _ = kc.shape
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lib.oracle_attention(len(ctx), T, Hq, Hkv, D, S, pt.shape[1], _ptr(q), _ptr(kc), _ptr(vc),
                         _ptr(pt), _ptr(cu), _ptr(ctx), float(scale), int(bool(causal)), _ptr(out))
    return out


def attention_rows(q, k_cache, v_cache, page_table, cu_q_lens, context_lens, tokens, heads, *,
                   scale, causal, lib=None) -> np.ndarray:
    """Exact attention of the listed (token, q head) pairs only; float64 [n, D]."""
    lib = lib or load()
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    pt, cu, ctx = _i32(page_table), _i32(cu_q_lens), _i32(context_lens)
    ts, hs = _i32(tokens), _i32(heads)
    T, Hq, D = q.shape
    _, S, Hkv, _ = kc.shape
    out = np.zeros((len(ts), D), dtype=np.float64)
    lib.oracle_attention_rows(len(ctx), T, Hq, Hkv, D, S, pt.shape[1], _ptr(q), _ptr(kc), _ptr(vc),
                              _ptr(pt), _ptr(cu), _ptr(ctx), float(scale), int(bool(causal)),
                              len(ts), _ptr(ts), _ptr(hs), _ptr(out))
    return out


def forward(q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens, slot_mapping,
            *, scale, causal, lib=None):
    """Check, scatter into copies of the caches, then attend.

    Returns (out float64 [T,Hq,D], k_cache', v_cache').  Raises ValueError when
    a precondition fails.
    """
    lib = lib or load()
    T, Hq, D = q.shape
    P, S, Hkv, _ = k_cache.shape
    rc = check(page_table, cu_q_lens, context_lens, slot_mapping, num_q_heads=Hq,
               num_kv_heads=Hkv, head_dim=D, page_size=S, num_pages=P, lib=lib)
    if rc != OK:
        raise ValueError(f"oracle precondition failed (code {rc})")
    kc, vc = scatter(k_cache, v_cache, k_new, v_new, slot_mapping, page_size=S, lib=lib)
    out = attention(q, kc, vc, page_table, cu_q_lens, context_lens, scale=scale, causal=causal,
                    lib=lib)
    return out, kc, vc
