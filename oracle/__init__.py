"""CPU oracle for the batched speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports it and has no fallback to it.

`spec_oracle.c` holds the arithmetic (plain double-precision loops; see its
header for the passages of the pages it follows).  This module only builds
that file with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB = os.path.join(_HERE, "libspec_oracle.so")

F32, BF16 = 0, 1
SAMPLE, GREEDY, POINT = 0, 1, 2
(FAULT_NONE, FAULT_NO_CLAMP, FAULT_UNSCALED_TAU, FAULT_RESAMPLE_P, FAULT_GREEDY_RULE,
 FAULT_FILTER_P_ONLY) = range(6)

_lib = None


def build(force: bool = True) -> str:
    """Compile spec_oracle.c into libspec_oracle.so (gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
               "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # SPEC_ORACLE_LIB: another build of this source to load instead (the
        # sanitizer run of tests/run_sanitized.py); never rebuilt here
        path = os.environ.get("SPEC_ORACLE_LIB") or _LIB
        if path == _LIB and (not os.path.exists(_LIB)
                             or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_verify.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, D,
                                      i32, i32, i32, P, P, P, P, P, P, P, P, P, P, i32, D, P,
                                      P, P]
        lib.oracle_verify.restype = i32
        lib.oracle_draw_cdf.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, D,
                                        i32, i32, P, i32, D]
        lib.oracle_draw_cdf.restype = i32
        lib.oracle_draw_index.argtypes = [P, i32, D, P]
        lib.oracle_draw_index.restype = i32
        lib.oracle_filter_row.argtypes = [P, i32, i32, D, i32, D, P, P, P]
        lib.oracle_filter_row.restype = i32
        lib.oracle_ngram_draft.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P]
        lib.oracle_ngram_draft.restype = i32
        lib.oracle_gamma_control.argtypes = [P, P, P, P, P, i32, i32, D, D, D, D, i32, P, P]
        lib.oracle_gamma_control.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("logits must be float32 or bf16 bit patterns stored as uint16")


@dataclass
class OracleResult:
    tokens: np.ndarray      # int32 [B, G+1], -1 padded
    n_accepted: np.ndarray  # int32 [B]
    new_len: np.ndarray     # int32 [B]
    px: np.ndarray          # float64 [B, G]; NaN where the position was not tested
    qx: np.ndarray          # float64 [B, G]
    z: np.ndarray           # float64 [B]; normaliser of the drawn distribution
    m: np.ndarray           # float64 [B, 2G+1]; raw-logit max of t_0..t_G, d_0..d_{G-1}
    s: np.ndarray           # float64 [B, 2G+1]; sum exp((l - m) / T)
    draw_pos: np.ndarray    # int32 [B]; position drawn from, -1 if none
    zero_resid: np.ndarray  # int32 [B]; 1 where the residual mass was exactly 0
    fmargin: np.ndarray     # float64 [B]; smallest top-p margin (relative mass) of the rows
    flo: np.ndarray         # float64 [B]; normalised CDF just below the drawn token (NaN: none)
    fhi: np.ndarray         # float64 [B]; normalised CDF at the drawn token


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def verify(target, draft, tokens, uniforms, gamma, kv_len=None, *, temperature=1.0,
           mode=SAMPLE, fault=FAULT_NONE, threads=0, top_k=0, top_p=1.0) -> OracleResult:
    """Run the oracle over a batch.

    target: [B, G+1, V] float32 or uint16 (bf16 bits); draft: [B, G, V] same
    dtype (may be None in greedy and point mode, which ignore it); tokens:
    int32 [B, G]; uniforms:
    float32 [B, G+1] (may be None in greedy mode); gamma: int32 [B];
    kv_len: int32 [B] or None.  threads=0 uses the OpenMP default.  top_k
    (0: off) and top_p (1: off) filter p and q alike before the walk.
    """
    lib = _load()
    target = np.ascontiguousarray(target)
    B, G1, V = target.shape
    G = G1 - 1
    dt = _dtype_code(target)
    if mode == POINT:
        draft = None
    if draft is not None:
        draft = np.ascontiguousarray(draft, dtype=target.dtype)
        if draft.shape != (B, G, V):
            raise ValueError("draft shape must be [B, G, V]")
    tokens = _c(tokens, np.int32).reshape(B, G)
    uniforms = _c(uniforms, np.float32)
    if uniforms is not None:
        uniforms = uniforms.reshape(B, G + 1)
    gamma = _c(gamma, np.int32).reshape(B)
    kv_len = _c(kv_len, np.int32)
    out_tokens = np.empty((B, G + 1), np.int32)
    out_n = np.empty(B, np.int32)
    out_len = np.empty(B, np.int32)
    px = np.empty((B, G), np.float64)
    qx = np.empty((B, G), np.float64)
    z = np.empty(B, np.float64)
    m = np.empty((B, 2 * G + 1), np.float64)
    s = np.empty((B, 2 * G + 1), np.float64)
    pos = np.empty(B, np.int32)
    zr = np.empty(B, np.int32)
    fm = np.empty(B, np.float64)
    flo = np.empty(B, np.float64)
    fhi = np.empty(B, np.float64)
    rc = lib.oracle_verify(_ptr(target), _ptr(draft), dt, _ptr(tokens), _ptr(uniforms),
                           _ptr(gamma), _ptr(kv_len), B, G, V, float(temperature), int(mode),
                           int(fault), int(threads), _ptr(out_tokens), _ptr(out_n),
                           _ptr(out_len), _ptr(px), _ptr(qx), _ptr(z), _ptr(m), _ptr(s),
                           _ptr(pos), _ptr(zr), int(top_k), float(top_p), _ptr(fm),
                           _ptr(flo), _ptr(fhi))
    if rc != 0:
        raise ValueError(f"oracle refused its arguments (code {rc})")
    return OracleResult(out_tokens, out_n, out_len, px, qx, z, m, s, pos, zr, fm, flo, fhi)


def draw_cdf(target, draft, tokens, uniforms, gamma, row, *, temperature=1.0, mode=SAMPLE,
             top_k=0, top_p=1.0):
    """Normalised CDF (C_j / Z, float64 [V]) of the distribution the oracle
    drew row `row`'s last token from, and the position it was drawn at."""
    lib = _load()
    target = np.ascontiguousarray(target)
    B, G1, V = target.shape
    G = G1 - 1
    draft = None if mode == POINT else np.ascontiguousarray(draft, dtype=target.dtype)
    tokens = _c(tokens, np.int32).reshape(B, G)
    uniforms = _c(uniforms, np.float32).reshape(B, G + 1)
    gamma = _c(gamma, np.int32).reshape(B)
    cdf = np.empty(V, np.float64)
    pos = lib.oracle_draw_cdf(_ptr(target), _ptr(draft), _dtype_code(target), _ptr(tokens),
                              _ptr(uniforms), _ptr(gamma), None, B, G, V, float(temperature),
                              int(mode), int(row), _ptr(cdf), int(top_k), float(top_p))
    return cdf, int(pos)


def draw_index(w, u):
    """The oracle's inverse-CDF draw over given non-negative weights:
    (index, Z).  Test hook for the tie-break and the fallback rule."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    z = ctypes.c_double(0.0)
    j = _load().oracle_draw_index(_ptr(w), int(w.size), float(u), ctypes.byref(z))
    if j < 0:
        raise ValueError("oracle refused its arguments")
    return int(j), float(z.value)


def filter_row(logits, *, temperature=1.0, top_k=0, top_p=1.0, margin=False):
    """The filtered distribution softmax(l/T) restricted to top-k then top-p
    (float64 [V]) of one stored logit row, and its logit threshold (and, with
    margin=True, how far the top-p crossing is from the cut, relative to the
    kept mass; +inf when top-p cuts nothing)."""
    lib = _load()
    logits = np.ascontiguousarray(logits)
    prob = np.empty(logits.shape[-1], np.float64)
    tau = ctypes.c_double(0.0)
    mg = ctypes.c_double(0.0)
    rc = lib.oracle_filter_row(_ptr(logits), _dtype_code(logits), logits.shape[-1],
                               float(temperature), int(top_k), float(top_p), _ptr(prob),
                               ctypes.byref(tau), ctypes.byref(mg))
    if rc != 0:
        raise ValueError("oracle refused the row or its arguments")
    return (prob, tau.value, mg.value) if margin else (prob, tau.value)


@dataclass
class DraftResult:
    draft: np.ndarray    # int32 [B, gamma], -1 after the draft
    length: np.ndarray   # int32 [B]
    n: np.ndarray        # int32 [B]; the n-gram length that matched, -1 if none
    pos: np.ndarray      # int32 [B]; where the copied continuation starts, -1 if none


def ngram_draft(context, ctx_len, *, n_min=1, n_max=4, gamma=4) -> DraftResult:
    """Prompt-lookup drafting over int32 contexts [B, stride] with lengths
    ctx_len [B] (see oracle_ngram_draft in spec_oracle.c)."""
    lib = _load()
    context = np.ascontiguousarray(context, dtype=np.int32)
    B, stride = context.shape
    ctx_len = np.ascontiguousarray(ctx_len, dtype=np.int32).reshape(B)
    draft = np.empty((B, gamma), np.int32)
    length = np.empty(B, np.int32)
    n = np.empty(B, np.int32)
    pos = np.empty(B, np.int32)
    rc = lib.oracle_ngram_draft(_ptr(context), _ptr(ctx_len), B, stride, int(n_min), int(n_max),
                                int(gamma), _ptr(draft), _ptr(length), _ptr(n), _ptr(pos))
    if rc != 0:
        raise ValueError("oracle refused the drafting arguments")
    return DraftResult(draft, length, n, pos)


def gamma_control(state, n_accepted=None, gamma_used=None, *, active=None, gamma_limit=None,
                  gamma_max=4, decay=0.9, prior_alpha=0.6, prior_weight=2.0, draft_cost=0.05,
                  batch_off=0):
    """Adaptive draft length (see oracle_gamma_control in spec_oracle.c).

    state: float64 [B, 2] {A, T}, updated in place.  n_accepted, gamma_used:
    int32 [B] of the previous round (both None: no previous round).  Returns
    (gamma int32 [B], alpha float64 [B])."""
    lib = _load()
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous and state.ndim == 2 and state.shape[1] == 2):
        raise ValueError("state must be a C-contiguous float64 [B, 2] array")
    B = state.shape[0]
    opt = lambda a: None if a is None else np.ascontiguousarray(a, dtype=np.int32).reshape(B)
    n_accepted, gamma_used, active, gamma_limit = map(opt, (n_accepted, gamma_used, active,
                                                            gamma_limit))
    gamma = np.empty(B, np.int32)
    alpha = np.empty(B, np.float64)
    rc = lib.oracle_gamma_control(_ptr(n_accepted), _ptr(gamma_used), _ptr(active),
                                  _ptr(gamma_limit), _ptr(state), B, int(gamma_max), float(decay),
                                  float(prior_alpha), float(prior_weight), float(draft_cost),
                                  int(batch_off), _ptr(gamma), _ptr(alpha))
    if rc != 0:
        raise ValueError("oracle refused the controller arguments")
    return gamma, alpha
