"""ctypes binding of libspecdec.so: argument marshalling only.

Every step of the verify path runs in the HIP kernels behind the C ABI
(include/specdec.h).  This module checks shapes, dtypes, devices and
contiguity of torch tensors, hands their device pointers and the current HIP
stream to the library, and turns a negative status into an exception.  When
the library is not built or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

from . import _build

FP32 = 0
BF16 = 1

_lock = threading.Lock()
_lib = None
_workspaces = {}


class SpecdecError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


def library_path() -> str:
    return _build.LIB


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libspecdec.so (building it first only if it does not exist)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = _build.LIB
        if not os.path.exists(path):
            if not build_if_missing:
                raise RuntimeError("libspecdec.so is not built; run "
                                   "python -m speculative_decoding_verification_10_amd._build")
            _build.build()
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz, f32, ci = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_size_t, ctypes.c_float, ctypes.c_int)
        lib.specdec_status_string.argtypes = [ci]
        lib.specdec_status_string.restype = ctypes.c_char_p
        lib.specdec_version.argtypes = []
        lib.specdec_version.restype = ctypes.c_char_p
        lib.specdec_workspace_init.argtypes = [vp, sz, vp]
        lib.specdec_workspace_init.restype = ci
        lib.specdec_workspace_errors.argtypes = [vp, vp, ci, vp]
        lib.specdec_workspace_errors.restype = ci
        lib.specdec_debug_bounded_wait.argtypes = [ctypes.c_uint64, ctypes.c_int32]
        lib.specdec_debug_bounded_wait.restype = ci
        lib.specdec_softmax_stats_workspace_bytes.argtypes = [i64, i32, ci]
        lib.specdec_softmax_stats_workspace_bytes.restype = sz
        lib.specdec_softmax_stats.argtypes = [vp, ci, i64, i32, f32, vp, vp, vp, sz, vp]
        lib.specdec_softmax_stats.restype = ci
        lib.specdec_verify_workspace_bytes.argtypes = [i32, i32, i32, ci, ci]
        lib.specdec_verify_workspace_bytes.restype = sz
        lib.specdec_verify.argtypes = [vp, vp, ci, vp, vp, vp, f32, i32, i32, i32,
                                       vp, vp, vp, vp, sz, vp]
        lib.specdec_verify.restype = ci
        lib.specdec_verify_timed.argtypes = [vp, vp, ci, vp, vp, vp, f32, i32, i32, i32,
                                             vp, vp, vp, vp, sz, vp, vp]
        lib.specdec_verify_timed.restype = ci
        lib.specdec_verify_noalloc.argtypes = [vp, vp, ci, vp, vp, vp, f32, i32, i32, i32,
                                               vp, vp, vp, vp]
        lib.specdec_verify_noalloc.restype = ci
        lib.specdec_verify_greedy_workspace_bytes.argtypes = [i32, i32, i32, ci]
        lib.specdec_verify_greedy_workspace_bytes.restype = sz
        lib.specdec_verify_greedy.argtypes = [vp, ci, vp, vp, i32, i32, i32, vp, vp, vp,
                                              vp, sz, vp]
        lib.specdec_verify_greedy.restype = ci
        lib.specdec_verify_greedy_timed.argtypes = [vp, ci, vp, vp, i32, i32, i32, vp, vp, vp,
                                                    vp, sz, vp, vp]
        lib.specdec_verify_greedy_timed.restype = ci
        lib.specdec_verify_processed_workspace_bytes.argtypes = [i32, i32, i32, ci, ci]
        lib.specdec_verify_processed_workspace_bytes.restype = sz
        lib.specdec_verify_processed.argtypes = [vp, vp, ci, vp, vp, vp, f32, i32, f32, i32, i32,
                                                 i32, vp, vp, vp, vp, sz, vp]
        lib.specdec_verify_processed.restype = ci
        lib.specdec_verify_processed_timed.argtypes = [vp, vp, ci, vp, vp, vp, f32, i32, f32, i32,
                                                       i32, i32, vp, vp, vp, vp, sz, vp, vp]
        lib.specdec_verify_processed_timed.restype = ci
        lib.specdec_sampling_floors.argtypes = [vp, ci, i64, i32, f32, i32, f32, vp, vp]
        lib.specdec_sampling_floors.restype = ci
        lib.specdec_tree_verify_greedy_workspace_bytes.argtypes = [i32, i32, i32, ci]
        lib.specdec_tree_verify_greedy_workspace_bytes.restype = sz
        lib.specdec_tree_verify_greedy.argtypes = [vp, ci, vp, vp, vp, i32, i32, i32, vp, vp, vp,
                                                   vp, sz, vp]
        lib.specdec_tree_verify_greedy.restype = ci
        lib.specdec_tree_verify_greedy_timed.argtypes = [vp, ci, vp, vp, vp, i32, i32, i32, vp, vp,
                                                         vp, vp, sz, vp, vp]
        lib.specdec_tree_verify_greedy_timed.restype = ci
        lib.specdec_tree_mask.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        lib.specdec_tree_mask.restype = ci
        lib.specdec_acceptance_counts.argtypes = [vp, vp, i32, i32, vp, vp]
        lib.specdec_acceptance_counts.restype = ci
        lib.specdec_ngram_propose.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
        lib.specdec_ngram_propose.restype = ci
        lib.specdec_read_stream.argtypes = [vp, sz, vp, vp, vp]
        lib.specdec_read_stream.restype = ci
        dbl = ctypes.c_double
        lib.specdec_choose_k.argtypes = [vp, i32, dbl, i32, i32, vp, vp, vp, vp]
        lib.specdec_choose_k.restype = ci
        _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load().specdec_status_string(status).decode()
    except Exception:  # pragma: no cover - only reached when the library is broken
        return "status %d" % status


def version() -> str:
    return load().specdec_version().decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("logits must be torch.float32 or torch.bfloat16, got %s" % t.dtype)


def _check(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Workspace:
    """Device scratch for the library, zero-filled when allocated so that the
    error word at offset 0 starts clear (no other initialisation is needed).
    The workspaces this module caches are kept per device, stream and entry
    point."""

    def __init__(self, nbytes: int, device):
        self.nbytes = int(nbytes)
        self.tensor = torch.zeros(max(self.nbytes, 256), dtype=torch.uint8, device=torch.device(device))
        self.device = self.tensor.device

    def ptr(self) -> int:
        return self.tensor.data_ptr()


def workspace_errors(ws: Workspace, clear: bool = True) -> int:
    """The workspace's error word (specdec_workspace_errors), read after
    every call enqueued on the current stream; cleared when ``clear``.
    Synchronises with that stream to return the value."""
    out = torch.empty((1,), dtype=torch.int32, device=ws.device)
    rc = load().specdec_workspace_errors(ws.ptr(), out.data_ptr(), int(bool(clear)), _stream(ws.device))
    if rc != 0:
        raise SpecdecError(rc, "specdec_workspace_errors")
    return int(out.item()) & 0xFFFFFFFF


def debug_bounded_wait(wait_ticks: int = 0, withhold_tile: int = -1) -> None:
    """specdec_debug_bounded_wait: for tests of the error path only; (0, -1)
    restores the defaults."""
    rc = load().specdec_debug_bounded_wait(int(wait_ticks), int(withhold_tile))
    if rc != 0:
        raise SpecdecError(rc, "specdec_debug_bounded_wait")


def cached_workspaces():
    """The workspaces this module allocated for calls made without one, keyed
    by (device index, stream, entry point)."""
    return dict(_workspaces)


def _workspace(nbytes: int, device: torch.device, ws: Optional[Workspace], kind: str) -> Workspace:
    if ws is not None:
        if ws.nbytes < nbytes or ws.device != device:
            raise ValueError("workspace too small (%d < %d) or on the wrong device" % (ws.nbytes, nbytes))
        return ws
    key = (device.index, _stream(device), kind)
    cur = _workspaces.get(key)
    if cur is None or cur.nbytes < nbytes:
        cur = Workspace(nbytes, device)
        _workspaces[key] = cur
    return cur


def verify_workspace_bytes(B, K, V, dtype_code, one_hot) -> int:
    return int(load().specdec_verify_workspace_bytes(B, K, V, dtype_code, int(bool(one_hot))))


def verify(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: torch.Tensor,
           uniforms: torch.Tensor, temperature: float, k_per_req: Optional[torch.Tensor] = None,
           accept_prob: bool = False, workspace: Optional[Workspace] = None, out=None,
           events=None, top_k: Optional[int] = None, top_p: Optional[float] = None):
    """Stochastic verify step (specdec_verify).

    target [B, K+1, V], draft [B, K, V] or None (one-hot drafts), both fp32 or
    bf16; draft_tokens [B, K] int32; uniforms [B, K+1] fp32; k_per_req [B]
    int32 or None.  Returns (out_tokens [B, K+1], num_accepted [B],
    accept_prob [B, K] or None).  ``out`` may hold preallocated
    (out_tokens, num_accepted, accept_prob) tensors.  ``events``: three
    torch.cuda.Event (enable_timing=True) or None entries, taken at the row
    kernel's start, its end and the end of the call's last kernel
    (specdec_verify_timed).  ``top_k`` / ``top_p``: run the step on the
    top-k / top-p processed distributions (specdec_verify_processed; None =
    that filter off).
    """
    lib = load()
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", target.dtype, (B, K + 1, V), dev)
    if draft is not None:
        _check(draft, "draft", target.dtype, (B, K, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _check(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    if k_per_req is not None:
        _check(k_per_req, "k_per_req", torch.int32, (B,), dev)
    if out is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        ap = torch.empty((B, K), dtype=torch.float32, device=dev) if accept_prob else None
    else:
        out_tokens, nacc, ap = out
        _check(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
        _check(nacc, "num_accepted", torch.int32, (B,), dev)
        if ap is not None:
            _check(ap, "accept_prob", torch.float32, (B, K), dev)
    processed = top_k is not None or top_p is not None
    if processed:
        nbytes = int(lib.specdec_verify_processed_workspace_bytes(B, K, V, code, int(draft is None)))
        ws = _workspace(nbytes, dev, workspace, "verify_processed")
        args = (_ptr(target), _ptr(draft), code, _ptr(draft_tokens), _ptr(k_per_req), _ptr(uniforms),
                float(temperature), int(top_k or 0), float(1.0 if top_p is None else top_p), B, K, V,
                _ptr(out_tokens), _ptr(nacc), _ptr(ap), ws.ptr(), ws.nbytes, _stream(dev))
        if events is None:
            rc = lib.specdec_verify_processed(*args)
            what = "specdec_verify_processed"
        else:
            if len(events) != 3:
                raise ValueError("events must hold three entries")
            rc = lib.specdec_verify_processed_timed(
                *args, (ctypes.c_void_p * 3)(*[_event_handle(e, dev) for e in events]))
            what = "specdec_verify_processed_timed"
        if rc != 0:
            raise SpecdecError(rc, what)
        return out_tokens, nacc, ap
    nbytes = verify_workspace_bytes(B, K, V, code, draft is None)
    ws = _workspace(nbytes, dev, workspace, "verify")
    if events is None:
        rc = lib.specdec_verify(_ptr(target), _ptr(draft), code, _ptr(draft_tokens),
                                _ptr(k_per_req), _ptr(uniforms), float(temperature), B, K, V,
                                _ptr(out_tokens), _ptr(nacc), _ptr(ap), ws.ptr(), ws.nbytes,
                                _stream(dev))
        what = "specdec_verify"
    else:
        if len(events) != 3:
            raise ValueError("events must hold three entries")
        handles = (ctypes.c_void_p * 3)(*[_event_handle(e, dev) for e in events])
        rc = lib.specdec_verify_timed(_ptr(target), _ptr(draft), code, _ptr(draft_tokens),
                                      _ptr(k_per_req), _ptr(uniforms), float(temperature), B, K,
                                      V, _ptr(out_tokens), _ptr(nacc), _ptr(ap), ws.ptr(),
                                      ws.nbytes, _stream(dev), handles)
        what = "specdec_verify_timed"
    if rc != 0:
        raise SpecdecError(rc, what)
    return out_tokens, nacc, ap


def _event_handle(ev, device: torch.device):
    """The hipEvent_t of a torch.cuda.Event (None -> NULL).  torch creates the
    event lazily at its first record, so an event never recorded is recorded
    once on the current stream first."""
    if ev is None:
        return None
    h = int(ev.cuda_event)
    if h == 0:
        ev.record(torch.cuda.current_stream(device))
        h = int(ev.cuda_event)
    if h == 0:
        raise ValueError("could not obtain the event's handle")
    return h


def verify_greedy(target: torch.Tensor, draft_tokens: torch.Tensor,
                  k_per_req: Optional[torch.Tensor] = None, argmax: bool = False,
                  workspace: Optional[Workspace] = None, out=None, events=None):
    """Greedy verify step (specdec_verify_greedy).  Returns (out_tokens,
    num_accepted, argmax [B, K+1] or None).  ``events``: three
    torch.cuda.Event (enable_timing=True) or None entries, taken at the
    argmax pass's start and end and the end of the call
    (specdec_verify_greedy_timed)."""
    lib = load()
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", target.dtype, (B, K + 1, V), dev)
    _check(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    if k_per_req is not None:
        _check(k_per_req, "k_per_req", torch.int32, (B,), dev)
    if out is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        am = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if argmax else None
    else:
        out_tokens, nacc, am = out
        _check(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
        _check(nacc, "num_accepted", torch.int32, (B,), dev)
        if am is not None:
            _check(am, "argmax", torch.int32, (B, K + 1), dev)
    nbytes = int(lib.specdec_verify_greedy_workspace_bytes(B, K, V, code))
    ws = _workspace(nbytes, dev, workspace, "greedy")
    args = (_ptr(target), code, _ptr(draft_tokens), _ptr(k_per_req), B, K, V, _ptr(out_tokens),
            _ptr(nacc), _ptr(am), ws.ptr(), ws.nbytes, _stream(dev))
    if events is None:
        rc = lib.specdec_verify_greedy(*args)
        what = "specdec_verify_greedy"
    else:
        if len(events) != 3:
            raise ValueError("events must hold three entries")
        rc = lib.specdec_verify_greedy_timed(
            *args, (ctypes.c_void_p * 3)(*[_event_handle(e, dev) for e in events]))
        what = "specdec_verify_greedy_timed"
    if rc != 0:
        raise SpecdecError(rc, what)
    return out_tokens, nacc, am


def tree_verify_greedy(target: torch.Tensor, node_tokens: torch.Tensor, parents: torch.Tensor,
                       n_nodes: Optional[torch.Tensor] = None, path: bool = True,
                       workspace: Optional[Workspace] = None, out=None, events=None):
    """Greedy verification of flattened draft trees
    (specdec_tree_verify_greedy): target [B, N+1, V] (row 0 after the root,
    row i + 1 after node i), node_tokens / parents [B, N] int32, n_nodes [B]
    int32 or None.  Returns (out_tokens [B, N+1], num_accepted [B],
    path_nodes [B, N] or None).  ``events`` as for verify_greedy."""
    lib = load()
    if target.dim() != 3:
        raise ValueError("target must be [B, N+1, V]")
    B, N1, V = target.shape
    N = N1 - 1
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", target.dtype, (B, N + 1, V), dev)
    _check(node_tokens, "node_tokens", torch.int32, (B, N), dev)
    _check(parents, "parents", torch.int32, (B, N), dev)
    if n_nodes is not None:
        _check(n_nodes, "n_nodes", torch.int32, (B,), dev)
    if out is None:
        out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev)
        nacc = torch.empty((B,), dtype=torch.int32, device=dev)
        pn = torch.empty((B, N), dtype=torch.int32, device=dev) if path else None
    else:
        out_tokens, nacc, pn = out
        _check(out_tokens, "out_tokens", torch.int32, (B, N + 1), dev)
        _check(nacc, "num_accepted", torch.int32, (B,), dev)
        if pn is not None:
            _check(pn, "path_nodes", torch.int32, (B, N), dev)
    nbytes = int(lib.specdec_tree_verify_greedy_workspace_bytes(B, N, V, code))
    ws = _workspace(nbytes, dev, workspace, "greedy")
    args = (_ptr(target), code, _ptr(node_tokens), _ptr(parents), _ptr(n_nodes), B, N, V,
            _ptr(out_tokens), _ptr(pn), _ptr(nacc), ws.ptr(), ws.nbytes, _stream(dev))
    if events is None:
        rc = lib.specdec_tree_verify_greedy(*args)
        what = "specdec_tree_verify_greedy"
    else:
        if len(events) != 3:
            raise ValueError("events must hold three entries")
        rc = lib.specdec_tree_verify_greedy_timed(
            *args, (ctypes.c_void_p * 3)(*[_event_handle(e, dev) for e in events]))
        what = "specdec_tree_verify_greedy_timed"
    if rc != 0:
        raise SpecdecError(rc, what)
    return out_tokens, nacc, pn


def tree_mask(parents: torch.Tensor, n_nodes: Optional[torch.Tensor] = None):
    """Ancestor-or-self attention mask [B, N, N] uint8 and depth [B, N] int32
    of flattened draft trees (specdec_tree_mask)."""
    lib = load()
    if parents.dim() != 2:
        raise ValueError("parents must be [B, N]")
    B, N = parents.shape
    dev = parents.device
    _check(parents, "parents", torch.int32, (B, N), dev)
    if n_nodes is not None:
        _check(n_nodes, "n_nodes", torch.int32, (B,), dev)
    mask = torch.empty((B, N, N), dtype=torch.uint8, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    rc = lib.specdec_tree_mask(_ptr(parents), _ptr(n_nodes), B, N, _ptr(mask), _ptr(depth),
                               _stream(dev))
    if rc != 0:
        raise SpecdecError(rc, "specdec_tree_mask")
    return mask, depth


def sampling_floors(logits: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0):
    """Per-row floor of the top-k / top-p processed distribution of a
    [..., V] tensor (specdec_sampling_floors): the kept tokens of a row are
    those with logit >= its floor.  Returns fp32 of shape [...]."""
    lib = load()
    if logits.dim() < 1:
        raise ValueError("logits must have a vocabulary axis")
    V = logits.shape[-1]
    rows = logits.numel() // V if V > 0 else 0
    dev = logits.device
    code = _dtype_code(logits)
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    fl = torch.empty(logits.shape[:-1], dtype=torch.float32, device=dev)
    rc = lib.specdec_sampling_floors(_ptr(logits), code, rows, V, float(temperature), int(top_k),
                                     float(top_p), _ptr(fl), _stream(dev))
    if rc != 0:
        raise SpecdecError(rc, "specdec_sampling_floors")
    return fl


def softmax_stats(logits: torch.Tensor, temperature: float, workspace: Optional[Workspace] = None):
    """Row max and sum_t exp((l_t - max)/T) of a [..., V] tensor
    (specdec_softmax_stats).  Returns two fp32 tensors of shape [...]."""
    lib = load()
    if logits.dim() < 1:
        raise ValueError("logits must have a vocabulary axis")
    V = logits.shape[-1]
    rows = logits.numel() // V if V > 0 else 0
    dev = logits.device
    code = _dtype_code(logits)
    if not logits.is_contiguous():
        raise ValueError("logits must be contiguous")
    rmax = torch.empty(logits.shape[:-1], dtype=torch.float32, device=dev)
    rsum = torch.empty(logits.shape[:-1], dtype=torch.float32, device=dev)
    nbytes = int(lib.specdec_softmax_stats_workspace_bytes(rows, V, code))
    ws = _workspace(nbytes, dev, workspace, "stats")
    rc = lib.specdec_softmax_stats(_ptr(logits), code, rows, V, float(temperature), _ptr(rmax),
                                   _ptr(rsum), ws.ptr(), ws.nbytes, _stream(dev))
    if rc != 0:
        raise SpecdecError(rc, "specdec_softmax_stats")
    return rmax, rsum


def acceptance_counts(num_accepted: torch.Tensor, K: int, k_per_req: Optional[torch.Tensor] = None,
                      counters: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-position (drafted, tested, accepted) counts of one verify step
    (specdec_acceptance_counts), added on the device to ``counters``: an
    int64 [3, K] tensor holding the uint64 counters (zeros when None).
    Returns the counters."""
    lib = load()
    dev = num_accepted.device
    B = num_accepted.numel()
    _check(num_accepted, "num_accepted", torch.int32, (B,), dev)
    if k_per_req is not None:
        _check(k_per_req, "k_per_req", torch.int32, (B,), dev)
    if counters is None:
        counters = torch.zeros((3, K), dtype=torch.int64, device=dev)
    _check(counters, "counters", torch.int64, (3, K), dev)
    rc = lib.specdec_acceptance_counts(_ptr(num_accepted), _ptr(k_per_req), B, int(K),
                                       _ptr(counters), _stream(dev))
    if rc != 0:
        raise SpecdecError(rc, "specdec_acceptance_counts")
    return counters


def choose_k(counters, c: float, k_min: int, k_max: int):
    """Draft length from [3, K] counters (specdec_choose_k, on the host):
    returns (k, alpha_test, alpha_draft, speedup at k)."""
    import numpy as np
    lib = load()
    if isinstance(counters, torch.Tensor):
        counters = counters.detach().cpu().numpy()
    cnt = np.ascontiguousarray(counters).view(np.uint64) if counters.dtype == np.int64 else \
        np.ascontiguousarray(counters, dtype=np.uint64)
    if cnt.ndim != 2 or cnt.shape[0] != 3:
        raise ValueError("counters must be [3, K]")
    K = cnt.shape[1]
    at, ad, sp = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    k = ctypes.c_int32()
    rc = lib.specdec_choose_k(cnt.ctypes.data, K, float(c), int(k_min), int(k_max),
                              ctypes.byref(at), ctypes.byref(ad), ctypes.byref(k), ctypes.byref(sp))
    if rc != 0:
        raise SpecdecError(rc, "specdec_choose_k")
    return k.value, at.value, ad.value, sp.value


def ngram_propose(context: torch.Tensor, context_len: torch.Tensor, n_min: int, n_max: int,
                  K: int, out=None):
    """n-gram (prompt-lookup) drafter (specdec_ngram_propose).  context
    [B, L] int32, context_len [B] int32, both on the device.  Returns
    (draft_tokens [B, K] int32, k_per_req [B] int32)."""
    lib = load()
    if context.dim() != 2:
        raise ValueError("context must be [B, L]")
    B, Ls = context.shape
    dev = context.device
    _check(context, "context", torch.int32, (B, Ls), dev)
    _check(context_len, "context_len", torch.int32, (B,), dev)
    if out is None:
        drafts = torch.empty((B, K), dtype=torch.int32, device=dev)
        kpr = torch.empty((B,), dtype=torch.int32, device=dev)
    else:
        drafts, kpr = out
        _check(drafts, "draft_tokens", torch.int32, (B, K), dev)
        _check(kpr, "k_per_req", torch.int32, (B,), dev)
    rc = lib.specdec_ngram_propose(_ptr(context), _ptr(context_len), B, Ls, int(n_min), int(n_max),
                                   int(K), _ptr(drafts), _ptr(kpr), _stream(dev))
    if rc != 0:
        raise SpecdecError(rc, "specdec_ngram_propose")
    return drafts, kpr
