"""fp64 CPU oracle for the batched verify step of speculative decoding.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.  It shares
no code with the GPU library and imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential sums in
ascending token id, OpenMP across independent requests / rows).  This module
only compiles it with gcc, loads it with ctypes and marshals numpy arrays.

Inputs are numpy arrays: fp32 logits as ``float32``; bf16 logits as the raw
``uint16`` bit patterns (the top half of an IEEE binary32), which the C side
widens exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_default = None

FP32 = 0
BF16 = 1

# Decisions whose uniform lies closer than this to the threshold it is
# compared with (accept ratio or normalised CDF boundary) are "flagged":
# a path computing in lower precision may legitimately decide them the
# other way.
FLAG_BAND = 1e-6


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source into a shared library with gcc.
    No fast-math: IEEE double semantics are kept."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
         "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (when missing or stale)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
        compile_source(SOURCE, _LIB)
    return _LIB


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return FP32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("logits must be float32 or uint16 (bf16 bit patterns), got %s" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    a = np.asarray(a)
    if a.dtype != dt:
        raise TypeError("expected %s, got %s" % (dt, a.dtype))
    return np.ascontiguousarray(a)


class Oracle:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i32, i64, dbl, ci = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_double, ctypes.c_int)
        lib.oracle_softmax_stats.argtypes = [vp, ci, i64, i32, dbl, vp, vp]
        lib.oracle_softmax_stats.restype = ci
        lib.oracle_verify.argtypes = [vp, vp, ci, vp, vp, vp, dbl, i32, i32, i32, vp, vp, vp, vp]
        lib.oracle_verify.restype = ci
        lib.oracle_verify_greedy.argtypes = [vp, ci, vp, vp, i32, i32, i32, vp, vp, vp]
        lib.oracle_verify_greedy.restype = ci
        lib.oracle_acceptance_counts.argtypes = [vp, vp, i32, i32, vp]
        lib.oracle_acceptance_counts.restype = ci
        lib.oracle_choose_k.argtypes = [vp, i32, dbl, i32, i32, vp, vp, vp, vp]
        lib.oracle_choose_k.restype = ci
        lib.oracle_ngram_propose.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp]
        lib.oracle_ngram_propose.restype = ci
        lib.oracle_tree_verify_greedy.argtypes = [vp, ci, vp, vp, vp, i32, i32, i32, vp, vp, vp]
        lib.oracle_tree_verify_greedy.restype = ci
        lib.oracle_tree_mask.argtypes = [vp, vp, i32, i32, vp, vp]
        lib.oracle_tree_mask.restype = ci
        lib.oracle_sampling_floor.argtypes = [vp, ci, ctypes.c_int64, i32, ctypes.c_double, i32,
                                              ctypes.c_double, vp, vp]
        lib.oracle_sampling_floor.restype = ci
        self.lib = lib
        self.path = path

    def softmax_stats(self, logits: np.ndarray, temperature: float):
        """Row max and sum_t exp((l_t - max)/T) in fp64 for a [..., V] array."""
        logits = np.ascontiguousarray(logits)
        code = _dtype_code(logits)
        V = logits.shape[-1]
        rows = logits.size // V
        m = np.empty(rows, np.float64)
        z = np.empty(rows, np.float64)
        rc = self.lib.oracle_softmax_stats(_ptr(logits), code, rows, V, float(temperature),
                                           _ptr(m), _ptr(z))
        if rc != 0:
            raise ValueError("oracle_softmax_stats rejected its arguments")
        return m.reshape(logits.shape[:-1]), z.reshape(logits.shape[:-1])

    def verify(self, target, draft, draft_tokens, uniforms, temperature, k_per_req=None):
        """One stochastic verify step.

        target [B, K+1, V], draft [B, K, V] or None (one-hot drafts),
        draft_tokens [B, K] int32, uniforms [B, K+1] float32, k_per_req [B]
        int32 or None.  Returns out_tokens [B, K+1], num_accepted [B],
        accept_prob [B, K] (fp64), min_margin [B] (fp64) and flagged [B].
        """
        target = np.ascontiguousarray(target)
        code = _dtype_code(target)
        B, K1, V = target.shape
        K = K1 - 1
        if draft is not None:
            draft = np.ascontiguousarray(draft)
            if draft.dtype != target.dtype or draft.shape != (B, K, V):
                raise ValueError("draft must match target dtype and be [B, K, V]")
        draft_tokens = _c(draft_tokens, np.int32).reshape(B, K)
        uniforms = _c(uniforms, np.float32).reshape(B, K + 1)
        kp = None if k_per_req is None else _c(k_per_req, np.int32).reshape(B)
        out = np.empty((B, K + 1), np.int32)
        nacc = np.empty(B, np.int32)
        ap = np.empty((B, K), np.float64)
        mm = np.empty(B, np.float64)
        rc = self.lib.oracle_verify(_ptr(target), _ptr(draft), code, _ptr(draft_tokens), _ptr(kp),
                                    _ptr(uniforms), float(temperature), B, K, V,
                                    _ptr(out), _ptr(nacc), _ptr(ap), _ptr(mm))
        if rc != 0:
            raise ValueError("oracle_verify rejected its arguments")
        return {"out_tokens": out, "num_accepted": nacc, "accept_prob": ap, "min_margin": mm,
                "flagged": mm < FLAG_BAND}

    def verify_greedy(self, target, draft_tokens, k_per_req=None):
        """One greedy verify step; returns out_tokens, num_accepted, argmax."""
        target = np.ascontiguousarray(target)
        code = _dtype_code(target)
        B, K1, V = target.shape
        K = K1 - 1
        draft_tokens = _c(draft_tokens, np.int32).reshape(B, K)
        kp = None if k_per_req is None else _c(k_per_req, np.int32).reshape(B)
        out = np.empty((B, K + 1), np.int32)
        nacc = np.empty(B, np.int32)
        am = np.empty((B, K + 1), np.int32)
        rc = self.lib.oracle_verify_greedy(_ptr(target), code, _ptr(draft_tokens), _ptr(kp),
                                           B, K, V, _ptr(out), _ptr(nacc), _ptr(am))
        if rc != 0:
            raise ValueError("oracle_verify_greedy rejected its arguments")
        return {"out_tokens": out, "num_accepted": nacc, "argmax": am}


    def acceptance_counts(self, num_accepted, K, k_per_req=None, counters=None):
        """Per-position (drafted, tested, accepted) counts of one step, added
        to ``counters`` ([3, K] uint64, zeros if None); returns the array."""
        nacc = _c(num_accepted, np.int32)
        B = nacc.size
        kp = None if k_per_req is None else _c(k_per_req, np.int32).reshape(B)
        cnt = np.zeros((3, K), np.uint64) if counters is None else counters
        if cnt.dtype != np.uint64 or cnt.shape != (3, K) or not cnt.flags.c_contiguous:
            raise ValueError("counters must be a contiguous uint64 [3, K] array")
        rc = self.lib.oracle_acceptance_counts(_ptr(nacc), _ptr(kp), B, K, _ptr(cnt))
        if rc != 0:
            raise ValueError("oracle_acceptance_counts rejected its arguments")
        return cnt

    def choose_k(self, counters, c, k_min, k_max):
        """(k, alpha_test, alpha_draft, speedup at k) from [3, K] counters."""
        cnt = _c(counters, np.uint64)
        K = cnt.shape[-1]
        at = ctypes.c_double()
        ad = ctypes.c_double()
        sp = ctypes.c_double()
        k = ctypes.c_int32()
        rc = self.lib.oracle_choose_k(_ptr(cnt), K, float(c), int(k_min), int(k_max),
                                      ctypes.byref(at), ctypes.byref(ad), ctypes.byref(k),
                                      ctypes.byref(sp))
        if rc != 0:
            raise ValueError("oracle_choose_k rejected its arguments")
        return k.value, at.value, ad.value, sp.value


    def ngram_propose(self, context, context_len, n_min, n_max, K):
        """n-gram drafter: context [B, L_stride] int32, context_len [B] int32.
        Returns (draft_tokens [B, K] int32, k_per_req [B] int32)."""
        ctx = _c(context, np.int32)
        if ctx.ndim != 2:
            raise ValueError("context must be [B, L]")
        B, Ls = ctx.shape
        ln = _c(context_len, np.int32).reshape(B)
        drafts = np.empty((B, K), np.int32)
        kp = np.empty(B, np.int32)
        rc = self.lib.oracle_ngram_propose(_ptr(ctx), _ptr(ln), B, Ls, int(n_min), int(n_max), int(K),
                                           _ptr(drafts), _ptr(kp))
        if rc != 0:
            raise ValueError("oracle_ngram_propose rejected its arguments")
        return drafts, kp


    def tree_verify_greedy(self, target, node_tokens, parents, n_nodes=None):
        """Greedy tree verify: target [B, N+1, V], node_tokens / parents
        [B, N] int32, n_nodes [B] int32 or None.  Returns out_tokens
        [B, N+1], path_nodes [B, N], num_accepted [B]."""
        target = np.ascontiguousarray(target)
        code = _dtype_code(target)
        B, N1, V = target.shape
        N = N1 - 1
        tok = _c(node_tokens, np.int32).reshape(B, N)
        par = _c(parents, np.int32).reshape(B, N)
        nn = None if n_nodes is None else _c(n_nodes, np.int32).reshape(B)
        out = np.empty((B, N + 1), np.int32)
        path = np.empty((B, N), np.int32)
        nacc = np.empty(B, np.int32)
        rc = self.lib.oracle_tree_verify_greedy(_ptr(target), code, _ptr(tok), _ptr(par), _ptr(nn),
                                                B, N, V, _ptr(out), _ptr(path), _ptr(nacc))
        if rc != 0:
            raise ValueError("oracle_tree_verify_greedy rejected its arguments")
        return {"out_tokens": out, "path_nodes": path, "num_accepted": nacc}

    def tree_mask(self, parents, n_nodes=None):
        """Ancestor-or-self attention mask [B, N, N] uint8 and depth [B, N]
        int32 of flattened draft trees (parents [B, N] int32)."""
        par = _c(parents, np.int32)
        B, N = par.shape
        nn = None if n_nodes is None else _c(n_nodes, np.int32).reshape(B)
        mask = np.empty((B, N, N), np.uint8)
        depth = np.empty((B, N), np.int32)
        if self.lib.oracle_tree_mask(_ptr(par), _ptr(nn), B, N, _ptr(mask), _ptr(depth)) != 0:
            raise ValueError("oracle_tree_mask rejected its arguments")
        return mask, depth


    def sampling_floor(self, logits, temperature, top_k, top_p):
        """Per-row floor of the top-k / top-p processed distribution:
        logits [..., V] float32 or bf16 bits; returns (floor [...] float32,
        margin [...] float64)."""
        logits = np.ascontiguousarray(logits)
        code = _dtype_code(logits)
        V = logits.shape[-1]
        rows = logits.size // V
        fl = np.empty(logits.shape[:-1], np.float32)
        mg = np.empty(logits.shape[:-1], np.float64)
        rc = self.lib.oracle_sampling_floor(_ptr(logits), code, rows, V, float(temperature),
                                            int(top_k), float(top_p), _ptr(fl), _ptr(mg))
        if rc != 0:
            raise ValueError("oracle_sampling_floor rejected its arguments")
        return fl, mg

    def verify_processed(self, target, draft, draft_tokens, uniforms, temperature, top_k, top_p,
                         k_per_req=None):
        """One stochastic verify step on the processed distributions: each
        target and draft row keeps the tokens at or above its floor (every
        other logit set to -inf), then the plain verify step runs on those
        rows.  Adds 'target_floor', 'draft_floor' and 'flagged' also for rows
        whose floor lies within the flag band of a top-p boundary."""
        target = np.ascontiguousarray(target)
        tf, tm = self.sampling_floor(target, temperature, top_k, top_p)
        tv = _as_f32(target)
        tproc = np.where(tv >= tf[..., None], tv, np.float32(-np.inf)).astype(np.float32)
        dproc, df, dm = None, None, None
        if draft is not None:
            draft = np.ascontiguousarray(draft)
            df, dm = self.sampling_floor(draft, temperature, top_k, top_p)
            dv = _as_f32(draft)
            dproc = np.where(dv >= df[..., None], dv, np.float32(-np.inf)).astype(np.float32)
        r = self.verify(tproc, dproc, draft_tokens, uniforms, temperature, k_per_req)
        B, K1 = tf.shape
        kb = np.full(B, K1 - 1) if k_per_req is None else np.asarray(k_per_req)
        near = np.zeros(B, bool)
        for b in range(B):
            near[b] = np.any(tm[b, :kb[b] + 1] < FLAG_BAND)
            if dm is not None:
                near[b] |= np.any(dm[b, :kb[b]] < FLAG_BAND)
        r.update(target_floor=tf, draft_floor=df, floor_flagged=near,
                 flagged=r["flagged"] | near)
        return r


def _as_f32(a):
    """float32 values of float32 logits or bf16 bits (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            _default = Oracle(build())
    return _default


def softmax_stats(logits, temperature):
    return default().softmax_stats(logits, temperature)


def verify(target, draft, draft_tokens, uniforms, temperature, k_per_req=None):
    return default().verify(target, draft, draft_tokens, uniforms, temperature, k_per_req)


def verify_greedy(target, draft_tokens, k_per_req=None):
    return default().verify_greedy(target, draft_tokens, k_per_req)


def acceptance_counts(num_accepted, K, k_per_req=None, counters=None):
    return default().acceptance_counts(num_accepted, K, k_per_req, counters)


def choose_k(counters, c, k_min, k_max):
    return default().choose_k(counters, c, k_min, k_max)


def ngram_propose(context, context_len, n_min, n_max, K):
    return default().ngram_propose(context, context_len, n_min, n_max, K)


def tree_verify_greedy(target, node_tokens, parents, n_nodes=None):
    return default().tree_verify_greedy(target, node_tokens, parents, n_nodes)


def tree_mask(parents, n_nodes=None):
    return default().tree_mask(parents, n_nodes)


def sampling_floor(logits, temperature, top_k, top_p):
    return default().sampling_floor(logits, temperature, top_k, top_p)


def verify_processed(target, draft, draft_tokens, uniforms, temperature, top_k, top_p,
                     k_per_req=None):
    return default().verify_processed(target, draft, draft_tokens, uniforms, temperature, top_k,
                                      top_p, k_per_req)
