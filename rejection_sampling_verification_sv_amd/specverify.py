"""Python binding of libspecverify: argument marshalling only.

Each ``sv_*`` function here has the name of the C entry point it calls. It
checks that the tensors are contiguous device tensors of the expected dtype
and shape, allocates outputs (and a zero-filled workspace) with PyTorch when
the caller does not pass them, and forwards raw device pointers and the HIP
stream of the call (``stream=``, default: the current stream). Everything the
binding allocates or zero-fills for a call is enqueued on that same stream,
so it is ordered before the call's kernels. Every step of the computation runs in the library's HIP
kernels; there is no CPU or PyTorch fallback: a missing library or a CPU
tensor raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import threading
from typing import Dict, Optional

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libspecverify.so")

SV_OK = 0
SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_ERRF_TOKEN = 0x1
SV_ERRF_TEMPERATURE = 0x2
SV_ERRF_PARENT = 0x4
SV_ERRF_NONFINITE = 0x8
SV_ERRF_INTERNAL = 0x10
SV_MAX_K = 63
SV_MAX_TREE_NODES = 1024

_DTYPES = {torch.float32: SV_DTYPE_F32, torch.bfloat16: SV_DTYPE_BF16}

_c_i32 = ctypes.c_int32
_c_ptr = ctypes.c_void_p
_c_size = ctypes.c_size_t

_lib = None
_lib_lock = threading.Lock()


class SpecVerifyError(RuntimeError):
    """A non-SV_OK status from the library."""


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m rejection_sampling_verification_sv_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.sv_status_string.argtypes = [ctypes.c_int]
        lib.sv_status_string.restype = ctypes.c_char_p
        lib.sv_chain_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, ctypes.c_int]
        lib.sv_chain_workspace_bytes.restype = _c_size
        lib.sv_verify_chain.argtypes = [
            _c_ptr, _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr,
        ]
        lib.sv_verify_chain.restype = ctypes.c_int
        lib.sv_tree_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, ctypes.c_int]
        lib.sv_tree_workspace_bytes.restype = _c_size
        lib.sv_verify_tree_greedy.argtypes = [
            _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr,
        ]
        lib.sv_verify_tree_greedy.restype = ctypes.c_int
        lib.sv_tree_sampling_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, ctypes.c_int]
        lib.sv_tree_sampling_workspace_bytes.restype = _c_size
        lib.sv_verify_tree_sampling.argtypes = [
            _c_ptr, _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr,
        ]
        lib.sv_verify_tree_sampling.restype = ctypes.c_int
        lib.sv_build_tree_mask.argtypes = [_c_ptr, _c_i32, _c_ptr, _c_ptr, _c_ptr]
        lib.sv_build_tree_mask.restype = ctypes.c_int
        lib.sv_sample_workspace_bytes.argtypes = [_c_i32, _c_i32, ctypes.c_int]
        lib.sv_sample_workspace_bytes.restype = _c_size
        lib.sv_sample_rows.argtypes = [
            _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr,
        ]
        lib.sv_sample_rows.restype = ctypes.c_int
        lib.sv_verify_chain_noalloc.argtypes = [
            _c_ptr, _c_ptr, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
        ]
        lib.sv_verify_chain_noalloc.restype = ctypes.c_int
        lib.sv_lm_head_chain_workspace_bytes.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32]
        lib.sv_lm_head_chain_workspace_bytes.restype = _c_size
        lib.sv_lm_head_logits.argtypes = [_c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr]
        lib.sv_lm_head_logits.restype = ctypes.c_int
        lib.sv_verify_chain_lm_head.argtypes = [
            _c_ptr, _c_ptr, _c_i32, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i32, _c_i32, _c_i32,
            _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr,
        ]
        lib.sv_verify_chain_lm_head.restype = ctypes.c_int
        lib.sv_chain_launches.argtypes = [_c_i32, _c_i32, _c_i32, ctypes.c_int, _c_i32, _c_i32]
        lib.sv_chain_launches.restype = _c_i32
        lib.sv_chain_form.argtypes = [_c_i32, _c_i32, _c_i32, ctypes.c_int, _c_i32, _c_i32]
        lib.sv_chain_form.restype = _c_i32
        lib.sv_time_next_stream_pass.argtypes = [_c_ptr, _c_ptr]
        lib.sv_time_next_stream_pass.restype = ctypes.c_int
        _lib = lib
        return lib


def library():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


def sv_status_string(status: int) -> str:
    return _load().sv_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != SV_OK:
        raise SpecVerifyError(f"{what}: {sv_status_string(status)}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")
    return _DTYPES[t.dtype]


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None, device=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); the library has no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(device, stream) -> int:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


@contextlib.contextmanager
def _on_call_stream(device, stream):
    """Make the call's stream current for the body: the binding's allocations,
    zero-fills and the library's launches are then all ordered on it (the
    caching allocator also ties every tensor allocated here to that stream).
    Yields (call stream, the stream that was current before)."""
    outer = torch.cuda.current_stream(device)
    s = outer if stream is None else stream
    with torch.cuda.stream(s):
        yield s, outer


def _used_on(s, outer, tensors) -> None:
    """Caller tensors read or written on a stream other than the caller's
    current one: tell the caching allocator, so that freeing them on the
    caller's side cannot hand their memory out while the call still runs."""
    if s == outer:
        return
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.device.type == "cuda":
            t.record_stream(s)


def _stream_ordered(fn):
    """Run a binding call with its ``stream=`` argument (default: the current
    stream) made current, so that the outputs, err_flags and workspace the
    binding allocates and zero-fills are ordered before the library's
    kernels on that stream; then record that stream on every tensor argument
    when it is not the caller's current one."""

    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        first = args[0] if args else None
        if not isinstance(first, torch.Tensor) or first.device.type != "cuda":
            return fn(*args, stream=stream, **kw)  # the body raises the argument error
        with _on_call_stream(first.device, stream) as (s, outer):
            out = fn(*args, stream=s, **kw)
            _used_on(s, outer, list(args) + list(kw.values()))
        return out

    return call


def sv_time_next_stream_pass(before: Optional[torch.cuda.Event], after: Optional[torch.cuda.Event]) -> None:
    """Arm this thread's next chain / tree call to launch its streaming pass with
    ``before`` and ``after`` as start / stop events (both None disarms).

    The events must be timing events that exist on the device already (recorded
    at least once); ``before.elapsed_time(after)`` then gives that kernel's
    duration once the stream has run past it.
    """
    if (before is None) != (after is None):
        raise ValueError("pass both events or neither")
    handles = [None, None]
    if before is not None:
        for i, e in enumerate((before, after)):
            if not e.cuda_event:
                raise ValueError("record each event once before arming it (the handle is created lazily)")
            handles[i] = e.cuda_event
    _check(_load().sv_time_next_stream_pass(handles[0], handles[1]), "sv_time_next_stream_pass")


# Zero-filled workspaces, one per (device, stream): the library returns every
# workspace to all-zero counters at the end of each call, so a workspace can
# be reused by the next call on the same stream. A call whose err_flags show
# SV_ERRF_INTERNAL leaves it dirty: reset_workspaces() zero-fills them again.
# Each entry is (workspace, the stream it serves); the workspace is allocated
# and zero-filled on that stream, so the fill is ordered before the first
# kernel that uses it, and a workspace replaced by a larger one is only
# handed out again by the caching allocator to work ordered after its last
# use on that stream.
_workspaces: Dict[tuple, tuple] = {}


def reset_workspaces() -> None:
    """Zero-fill every cached workspace (after a call raised SV_ERRF_INTERNAL).

    Each fill is enqueued on the stream its workspace serves, behind the
    calls already enqueued there.
    """
    for ws, s in _workspaces.values():
        with torch.cuda.stream(s):
            ws.zero_()


def workspace(device, nbytes: int, stream=None) -> torch.Tensor:
    """The cached zero-filled workspace of (device, stream) with at least
    ``nbytes`` bytes (``stream`` None: the device's current stream)."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    key = (torch.device(device).index, s.cuda_stream)
    ent = _workspaces.get(key)
    if ent is None or ent[0].numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = (ws, s)
        return ws
    return ent[0]


def sv_chain_workspace_bytes(B: int, K: int, V: int, dtype: torch.dtype) -> int:
    return int(_load().sv_chain_workspace_bytes(B, K, V, _DTYPES[dtype]))


def sv_chain_launches(B: int, K: int, V: int, dtype: torch.dtype, rows_aligned: bool = True,
                      with_entropy: bool = False) -> int:
    """Kernel launches ``sv_verify_chain`` makes for this shape on the current
    device: 1 (statistics and sampling in one launch) or 2; 0 if invalid."""
    return int(_load().sv_chain_launches(B, K, V, _DTYPES[dtype], int(rows_aligned), int(with_entropy)))


def sv_chain_form(B: int, K: int, V: int, dtype: torch.dtype, rows_aligned: bool = True,
                  with_entropy: bool = False) -> int:
    """``sv_chain_form``: 1 small call, 2 one launch with ticket queues, 3 two
    launches (0: invalid sizes or B = 0), on the current device."""
    return int(_load().sv_chain_form(B, K, V, _DTYPES[dtype], int(rows_aligned), int(with_entropy)))


def sv_tree_workspace_bytes(B: int, N: int, V: int, dtype: torch.dtype) -> int:
    return int(_load().sv_tree_workspace_bytes(B, N, V, _DTYPES[dtype]))


def _chain_prepare(target, draft, draft_tokens, temperature, uniforms, accept_len, out_tokens, p_draft, q_draft,
                   residual_mass, entropy, err_flags, want_probs, want_entropy):
    """Check a chain call's tensors and allocate the outputs the caller did
    not pass (on the current stream, which the public calls make the call's
    stream). Returns (B, K, V, dtype code, output dict)."""
    if target.dim() != 3:
        raise ValueError("target must be [B, K+1, V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    code = _dtype_code(target)
    _dev(target, "target")
    if K > 0:
        _dev(draft, "draft", dtype=target.dtype, shape=(B, K, V), device=dev)
        _dev(draft_tokens, "draft_tokens", dtype=torch.int32, shape=(B, K), device=dev)
    if temperature is not None:
        _dev(temperature, "temperature", dtype=torch.float32, shape=(B,), device=dev)
    _dev(uniforms, "uniforms", dtype=torch.float32, shape=(B, K1), device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {
        "accept_len": torch.empty((B,), **i32) if accept_len is None
        else _dev(accept_len, "accept_len", torch.int32, (B,), dev),
        "out_tokens": torch.empty((B, K1), **i32) if out_tokens is None
        else _dev(out_tokens, "out_tokens", torch.int32, (B, K1), dev),
        "err_flags": torch.zeros((1,), **i32) if err_flags is None
        else _dev(err_flags, "err_flags", torch.int32, (1,), dev),
    }
    if want_probs:
        out["p_draft"] = torch.empty((B, K), **f32) if p_draft is None else _dev(p_draft, "p_draft", torch.float32, (B, K), dev)
        out["q_draft"] = torch.empty((B, K), **f32) if q_draft is None else _dev(q_draft, "q_draft", torch.float32, (B, K), dev)
        out["residual_mass"] = (torch.empty((B,), **f32) if residual_mass is None
                                else _dev(residual_mass, "residual_mass", torch.float32, (B,), dev))
    if entropy is not None:
        out["entropy"] = _dev(entropy, "entropy", torch.float32, (B, 2 * K + 1), dev)
    elif want_entropy:
        out["entropy"] = torch.empty((B, 2 * K + 1), **f32)
    return B, K, V, code, out


def _chain_pointers(target, draft, draft_tokens, temperature, uniforms, B, K, V, code, o):
    return (_ptr(target), _ptr(draft) if K > 0 else None, code, _ptr(draft_tokens) if K > 0 else None,
            _ptr(temperature), _ptr(uniforms), B, K, V,
            _ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o.get("p_draft")), _ptr(o.get("q_draft")),
            _ptr(o.get("residual_mass")), _ptr(o.get("entropy")), _ptr(o["err_flags"]))


@_stream_ordered
def sv_verify_chain(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
                    temperature: Optional[torch.Tensor], uniforms: torch.Tensor, *,
                    accept_len=None, out_tokens=None, p_draft=None, q_draft=None, residual_mass=None,
                    entropy=None, err_flags=None, workspace_tensor=None, stream=None, want_probs: bool = True,
                    want_entropy: bool = False) -> dict:
    """Chain verification (``sv_verify_chain``). Shapes as in include/specverify.h.

    Returns a dict with ``accept_len [B]``, ``out_tokens [B,K+1]``, and when
    ``want_probs`` ``p_draft``, ``q_draft [B,K]``, ``residual_mass [B]``, when
    ``want_entropy`` (or an ``entropy`` tensor is passed) ``entropy [B,2K+1]``,
    plus ``err_flags [1]``. Outputs are ready once the stream has been
    synchronised.
    """
    lib = _load()
    B, K, V, code, out = _chain_prepare(target, draft, draft_tokens, temperature, uniforms, accept_len, out_tokens,
                                        p_draft, q_draft, residual_mass, entropy, err_flags, want_probs,
                                        want_entropy)
    dev = target.device
    nbytes = int(lib.sv_chain_workspace_bytes(B, K, V, code))
    ws = workspace(dev, nbytes, stream) if workspace_tensor is None else workspace_tensor
    st = lib.sv_verify_chain(*_chain_pointers(target, draft, draft_tokens, temperature, uniforms, B, K, V, code, out),
                             _ptr(ws), ws.numel(), _stream_handle(dev, stream))
    _check(st, "sv_verify_chain")
    return out


@_stream_ordered
def sv_verify_chain_noalloc(target: torch.Tensor, draft: Optional[torch.Tensor],
                            draft_tokens: Optional[torch.Tensor], temperature: Optional[torch.Tensor],
                            uniforms: torch.Tensor, *, accept_len=None, out_tokens=None, p_draft=None, q_draft=None,
                            residual_mass=None, entropy=None, err_flags=None, stream=None, want_probs: bool = True,
                            want_entropy: bool = False) -> dict:
    """``sv_verify_chain_noalloc``: chain verification on the library's static
    per-GPU scratch array, no workspace. The library allocates nothing; to
    allocate nothing here either, pass every output tensor (and err_flags).
    Calls that overlap in time on one GPU race (they share the array)."""
    lib = _load()
    B, K, V, code, out = _chain_prepare(target, draft, draft_tokens, temperature, uniforms, accept_len, out_tokens,
                                        p_draft, q_draft, residual_mass, entropy, err_flags, want_probs,
                                        want_entropy)
    st = lib.sv_verify_chain_noalloc(
        *_chain_pointers(target, draft, draft_tokens, temperature, uniforms, B, K, V, code, out),
        _stream_handle(target.device, stream))
    _check(st, "sv_verify_chain_noalloc")
    return out


def sv_lm_head_chain_workspace_bytes(B: int, K: int, V: int, H: int) -> int:
    return int(_load().sv_lm_head_chain_workspace_bytes(B, K, V, H))


@_stream_ordered
def sv_lm_head_logits(hidden: torch.Tensor, head_weight: torch.Tensor, *, logits=None, stream=None) -> torch.Tensor:
    """The LM head alone (``sv_lm_head_logits``): ``hidden [..., H]`` bf16
    through ``head_weight [V, H]`` bf16 -> logits ``[..., V]`` bf16."""
    lib = _load()
    H = hidden.shape[-1]
    V = head_weight.shape[0]
    dev = hidden.device
    _dev(hidden, "hidden", torch.bfloat16)
    _dev(head_weight, "head_weight", torch.bfloat16, (V, H), dev)
    M = hidden.numel() // H
    shape = tuple(hidden.shape[:-1]) + (V,)
    logits = (torch.empty(shape, dtype=torch.bfloat16, device=dev) if logits is None
              else _dev(logits, "logits", torch.bfloat16, shape, dev))
    _check(lib.sv_lm_head_logits(_ptr(hidden), _ptr(head_weight), M, H, V, _ptr(logits), _stream_handle(dev, stream)),
           "sv_lm_head_logits")
    return logits


@_stream_ordered
def sv_verify_chain_lm_head(hidden: torch.Tensor, head_weight: torch.Tensor, draft: Optional[torch.Tensor],
                            draft_tokens: Optional[torch.Tensor], temperature: Optional[torch.Tensor],
                            uniforms: torch.Tensor, *, target_logits=None, accept_len=None, out_tokens=None,
                            p_draft=None, q_draft=None, residual_mass=None, err_flags=None, workspace_tensor=None,
                            stream=None, want_probs: bool = True) -> dict:
    """Chain verification with the target's LM head in the call
    (``sv_verify_chain_lm_head``): ``hidden [B, K+1, H]`` and ``head_weight
    [V, H]`` bf16 give the target logits (returned as ``target_logits``), the
    rest as :func:`sv_verify_chain`."""
    lib = _load()
    if hidden.dim() != 3:
        raise ValueError("hidden must be [B, K+1, H]")
    B, K1, H = hidden.shape
    V = head_weight.shape[0]
    dev = hidden.device
    _dev(hidden, "hidden", torch.bfloat16)
    _dev(head_weight, "head_weight", torch.bfloat16, (V, H), dev)
    target_logits = (torch.empty((B, K1, V), dtype=torch.bfloat16, device=dev) if target_logits is None
                     else _dev(target_logits, "target_logits", torch.bfloat16, (B, K1, V), dev))
    _, K, _, code, out = _chain_prepare(target_logits, draft, draft_tokens, temperature, uniforms, accept_len,
                                        out_tokens, p_draft, q_draft, residual_mass, None, err_flags, want_probs,
                                        False)
    nbytes = int(lib.sv_lm_head_chain_workspace_bytes(B, K, V, H))
    ws = workspace(dev, nbytes, stream) if workspace_tensor is None else workspace_tensor
    st = lib.sv_verify_chain_lm_head(
        _ptr(hidden), _ptr(head_weight), H, _ptr(target_logits), _ptr(draft) if K > 0 else None,
        _ptr(draft_tokens) if K > 0 else None, _ptr(temperature), _ptr(uniforms), B, K, V,
        _ptr(out["accept_len"]), _ptr(out["out_tokens"]), _ptr(out.get("p_draft")), _ptr(out.get("q_draft")),
        _ptr(out.get("residual_mass")), _ptr(out["err_flags"]), _ptr(ws), ws.numel(), _stream_handle(dev, stream))
    _check(st, "sv_verify_chain_lm_head")
    out["target_logits"] = target_logits
    return out


def sv_sample_workspace_bytes(R: int, V: int, dtype: torch.dtype) -> int:
    return int(_load().sv_sample_workspace_bytes(R, V, _DTYPES[dtype]))


@_stream_ordered
def sv_sample_rows(logits: torch.Tensor, temperature: Optional[torch.Tensor], uniforms: torch.Tensor, *,
                   out_tokens=None, out_prob=None, err_flags=None, workspace_tensor=None, stream=None,
                   want_prob: bool = True) -> dict:
    """Draft-side sampling (``sv_sample_rows``): one token per row of
    ``logits [R, V]`` from its temperature softmax, with ``uniforms [R]``.

    Returns a dict with ``tokens [R]`` int32, ``prob [R]`` float32 (when
    ``want_prob``) and ``err_flags [1]``. Outputs are ready once the stream
    has been synchronised.
    """
    lib = _load()
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = logits.shape
    dev = logits.device
    code = _dtype_code(logits)
    _dev(logits, "logits")
    if temperature is not None:
        _dev(temperature, "temperature", dtype=torch.float32, shape=(R,), device=dev)
    _dev(uniforms, "uniforms", dtype=torch.float32, shape=(R,), device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    out_tokens = torch.empty((R,), **i32) if out_tokens is None else _dev(out_tokens, "out_tokens", torch.int32, (R,), dev)
    if want_prob:
        out_prob = (torch.empty((R,), dtype=torch.float32, device=dev) if out_prob is None
                    else _dev(out_prob, "out_prob", torch.float32, (R,), dev))
    err_flags = torch.zeros((1,), **i32) if err_flags is None else _dev(err_flags, "err_flags", torch.int32, (1,), dev)
    nbytes = int(lib.sv_sample_workspace_bytes(R, V, code))
    ws = workspace(dev, nbytes, stream) if workspace_tensor is None else workspace_tensor
    st = lib.sv_sample_rows(_ptr(logits), code, _ptr(temperature), _ptr(uniforms), R, V, _ptr(out_tokens),
                            _ptr(out_prob) if want_prob else None, _ptr(err_flags), _ptr(ws), ws.numel(),
                            _stream_handle(dev, stream))
    _check(st, "sv_sample_rows")
    out = {"tokens": out_tokens, "err_flags": err_flags}
    if want_prob:
        out["prob"] = out_prob
    return out


@_stream_ordered
def sv_verify_tree_greedy(target: torch.Tensor, node_tokens: torch.Tensor, parents: torch.Tensor, *,
                          accept_len=None, path_nodes=None, next_token=None, err_flags=None,
                          workspace_tensor=None, stream=None) -> dict:
    """Greedy tree verification (``sv_verify_tree_greedy``)."""
    lib = _load()
    if target.dim() != 3:
        raise ValueError("target must be [B, N+1, V]")
    B, N1, V = target.shape
    N = N1 - 1
    dev = target.device
    code = _dtype_code(target)
    _dev(target, "target")
    _dev(node_tokens, "node_tokens", torch.int32, (B, N), dev)
    _dev(parents, "parents", torch.int32, (N,), dev)
    i32 = dict(dtype=torch.int32, device=dev)
    accept_len = torch.empty((B,), **i32) if accept_len is None else _dev(accept_len, "accept_len", torch.int32, (B,), dev)
    path_nodes = torch.empty((B, N), **i32) if path_nodes is None else _dev(path_nodes, "path_nodes", torch.int32, (B, N), dev)
    next_token = torch.empty((B,), **i32) if next_token is None else _dev(next_token, "next_token", torch.int32, (B,), dev)
    err_flags = torch.zeros((1,), **i32) if err_flags is None else _dev(err_flags, "err_flags", torch.int32, (1,), dev)
    nbytes = int(lib.sv_tree_workspace_bytes(B, N, V, code))
    ws = workspace(dev, nbytes, stream) if workspace_tensor is None else workspace_tensor
    st = lib.sv_verify_tree_greedy(
        _ptr(target), code, _ptr(node_tokens), _ptr(parents), B, N, V,
        _ptr(accept_len), _ptr(path_nodes), _ptr(next_token), _ptr(err_flags),
        _ptr(ws), ws.numel(), _stream_handle(dev, stream))
    _check(st, "sv_verify_tree_greedy")
    return {"accept_len": accept_len, "path_nodes": path_nodes, "next_token": next_token, "err_flags": err_flags}


def sv_tree_sampling_workspace_bytes(B: int, N: int, V: int, dtype: torch.dtype) -> int:
    return int(_load().sv_tree_sampling_workspace_bytes(B, N, V, _DTYPES[dtype]))


@_stream_ordered
def sv_verify_tree_sampling(target: torch.Tensor, draft: torch.Tensor, node_tokens: torch.Tensor,
                            parents: torch.Tensor, temperature: Optional[torch.Tensor], uniforms: torch.Tensor, *,
                            accept_len=None, path_nodes=None, next_token=None, err_flags=None,
                            workspace_tensor=None, stream=None) -> dict:
    """Sampling verification of a candidate tree (``sv_verify_tree_sampling``).

    ``target`` and ``draft`` are ``[B, N+1, V]`` logits of one dtype,
    ``node_tokens [B, N]`` and ``parents [N]`` int32, ``temperature [B]``
    (or None for 1) and ``uniforms [B, N+1]`` float32. Returns a dict with
    ``accept_len [B]``, ``path_nodes [B, N]``, ``next_token [B]`` and
    ``err_flags [1]``.
    """
    lib = _load()
    if target.dim() != 3:
        raise ValueError("target must be [B, N+1, V]")
    B, N1, V = target.shape
    N = N1 - 1
    dev = target.device
    code = _dtype_code(target)
    _dev(target, "target")
    _dev(draft, "draft", target.dtype, (B, N1, V), dev)
    _dev(node_tokens, "node_tokens", torch.int32, (B, N), dev)
    _dev(parents, "parents", torch.int32, (N,), dev)
    if temperature is not None:
        _dev(temperature, "temperature", torch.float32, (B,), dev)
    _dev(uniforms, "uniforms", torch.float32, (B, N1), dev)
    i32 = dict(dtype=torch.int32, device=dev)
    accept_len = torch.empty((B,), **i32) if accept_len is None else _dev(accept_len, "accept_len", torch.int32, (B,), dev)
    path_nodes = torch.empty((B, N), **i32) if path_nodes is None else _dev(path_nodes, "path_nodes", torch.int32, (B, N), dev)
    next_token = torch.empty((B,), **i32) if next_token is None else _dev(next_token, "next_token", torch.int32, (B,), dev)
    err_flags = torch.zeros((1,), **i32) if err_flags is None else _dev(err_flags, "err_flags", torch.int32, (1,), dev)
    nbytes = int(lib.sv_tree_sampling_workspace_bytes(B, N, V, code))
    ws = workspace(dev, nbytes, stream) if workspace_tensor is None else workspace_tensor
    st = lib.sv_verify_tree_sampling(
        _ptr(target), _ptr(draft), code, _ptr(node_tokens), _ptr(parents), _ptr(temperature), _ptr(uniforms),
        B, N, V, _ptr(accept_len), _ptr(path_nodes), _ptr(next_token), _ptr(err_flags),
        _ptr(ws), ws.numel(), _stream_handle(dev, stream))
    _check(st, "sv_verify_tree_sampling")
    return {"accept_len": accept_len, "path_nodes": path_nodes, "next_token": next_token, "err_flags": err_flags}


@_stream_ordered
def sv_build_tree_mask(parents: torch.Tensor, *, mask=None, err_flags=None, stream=None) -> dict:
    """Tree ancestor mask (``sv_build_tree_mask``): uint8 ``[N, N]``."""
    lib = _load()
    _dev(parents, "parents", torch.int32)
    if parents.dim() != 1:
        raise ValueError("parents must be 1-D")
    N = parents.shape[0]
    dev = parents.device
    mask = torch.empty((N, N), dtype=torch.uint8, device=dev) if mask is None else _dev(mask, "mask", torch.uint8, (N, N), dev)
    err_flags = torch.zeros((1,), dtype=torch.int32, device=dev) if err_flags is None else _dev(err_flags, "err_flags", torch.int32, (1,), dev)
    st = lib.sv_build_tree_mask(_ptr(parents), N, _ptr(mask), _ptr(err_flags), _stream_handle(dev, stream))
    _check(st, "sv_build_tree_mask")
    return {"mask": mask, "err_flags": err_flags}


class PreparedChainCall:
    """``sv_verify_chain`` with every argument checked and marshalled once.

    Calling the object only enqueues the kernels (one ctypes call), so a
    launch loop is not limited by Python-side argument checking. The tensors
    passed at construction are kept alive and reused by every call.
    """

    def _init(self, target, draft, draft_tokens, temperature, uniforms, *, stream=None, want_probs=True,
              want_entropy=False):
        B, K1, V = target.shape
        K = K1 - 1
        dev = target.device
        self.out = {
            "accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((B, K1), dtype=torch.int32, device=dev),
            "err_flags": torch.zeros((1,), dtype=torch.int32, device=dev),
        }
        if want_probs:
            self.out["p_draft"] = torch.empty((B, K), dtype=torch.float32, device=dev)
            self.out["q_draft"] = torch.empty((B, K), dtype=torch.float32, device=dev)
            self.out["residual_mass"] = torch.empty((B,), dtype=torch.float32, device=dev)
        if want_entropy:
            self.out["entropy"] = torch.empty((B, 2 * K + 1), dtype=torch.float32, device=dev)
        # one checked call through the regular path validates every argument
        sv_verify_chain(target, draft, draft_tokens, temperature, uniforms, stream=stream,
                        want_probs=want_probs, **self.out)
        lib = _load()
        code = _dtype_code(target)
        self._ws = workspace(dev, int(lib.sv_chain_workspace_bytes(B, K, V, code)), stream)
        self._keep = (target, draft, draft_tokens, temperature, uniforms)
        o = self.out
        self._fn = lib.sv_verify_chain
        self._args = (
            _ptr(target), _ptr(draft) if K > 0 else None, code, _ptr(draft_tokens) if K > 0 else None,
            _ptr(temperature), _ptr(uniforms), B, K, V,
            _ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o.get("p_draft")), _ptr(o.get("q_draft")),
            _ptr(o.get("residual_mass")), _ptr(o.get("entropy")), _ptr(o["err_flags"]), _ptr(self._ws),
            self._ws.numel(), _stream_handle(dev, stream))

    def __init__(self, *args, stream=None, **kw):
        # outputs and the workspace are allocated and zero-filled on the
        # stream the calls will run on (the caller's current one by default)
        first = args[0]
        with _on_call_stream(first.device, stream) as (s, outer):
            self._init(*args, stream=s, **kw)
            _used_on(s, outer, list(args))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            _check(st, "sv_verify_chain")
        return self.out


class PreparedSampleCall:
    """``sv_sample_rows`` with every argument checked and marshalled once
    (calling the object only enqueues the kernels)."""

    def _init(self, logits, temperature, uniforms, *, stream=None, want_prob=True):
        R, V = logits.shape
        dev = logits.device
        self.out = {"tokens": torch.empty((R,), dtype=torch.int32, device=dev),
                    "err_flags": torch.zeros((1,), dtype=torch.int32, device=dev)}
        if want_prob:
            self.out["prob"] = torch.empty((R,), dtype=torch.float32, device=dev)
        sv_sample_rows(logits, temperature, uniforms, stream=stream, want_prob=want_prob,
                       out_tokens=self.out["tokens"], out_prob=self.out.get("prob"), err_flags=self.out["err_flags"])
        lib = _load()
        self._ws = workspace(dev, int(lib.sv_sample_workspace_bytes(R, V, _dtype_code(logits))), stream)
        self._keep = (logits, temperature, uniforms)
        o = self.out
        self._fn = lib.sv_sample_rows
        self._args = (_ptr(logits), _dtype_code(logits), _ptr(temperature), _ptr(uniforms), R, V, _ptr(o["tokens"]),
                      _ptr(o.get("prob")), _ptr(o["err_flags"]), _ptr(self._ws), self._ws.numel(),
                      _stream_handle(dev, stream))

    def __init__(self, *args, stream=None, **kw):
        # outputs and the workspace are allocated and zero-filled on the
        # stream the calls will run on (the caller's current one by default)
        first = args[0]
        with _on_call_stream(first.device, stream) as (s, outer):
            self._init(*args, stream=s, **kw)
            _used_on(s, outer, list(args))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            _check(st, "sv_sample_rows")
        return self.out


class PreparedTreeCall:
    """``sv_verify_tree_greedy`` with every argument checked and marshalled once
    (the tree counterpart of :class:`PreparedChainCall`)."""

    def _init(self, target, node_tokens, parents, *, stream=None):
        B, N1, V = target.shape
        N = N1 - 1
        dev = target.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.out = {
            "accept_len": torch.empty((B,), **i32),
            "path_nodes": torch.empty((B, N), **i32),
            "next_token": torch.empty((B,), **i32),
            "err_flags": torch.zeros((1,), **i32),
        }
        sv_verify_tree_greedy(target, node_tokens, parents, stream=stream, **self.out)
        lib = _load()
        code = _dtype_code(target)
        self._ws = workspace(dev, int(lib.sv_tree_workspace_bytes(B, N, V, code)), stream)
        self._keep = (target, node_tokens, parents)
        o = self.out
        self._fn = lib.sv_verify_tree_greedy
        self._args = (
            _ptr(target), code, _ptr(node_tokens), _ptr(parents), B, N, V,
            _ptr(o["accept_len"]), _ptr(o["path_nodes"]), _ptr(o["next_token"]), _ptr(o["err_flags"]),
            _ptr(self._ws), self._ws.numel(), _stream_handle(dev, stream))

    def __init__(self, *args, stream=None, **kw):
        # outputs and the workspace are allocated and zero-filled on the
        # stream the calls will run on (the caller's current one by default)
        first = args[0]
        with _on_call_stream(first.device, stream) as (s, outer):
            self._init(*args, stream=s, **kw)
            _used_on(s, outer, list(args))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            _check(st, "sv_verify_tree_greedy")
        return self.out


class PreparedTreeSamplingCall:
    """``sv_verify_tree_sampling`` with every argument checked and marshalled
    once (calling the object only enqueues the kernels)."""

    def _init(self, target, draft, node_tokens, parents, temperature, uniforms, *, stream=None):
        B, N1, V = target.shape
        N = N1 - 1
        dev = target.device
        i32 = dict(dtype=torch.int32, device=dev)
        self.out = {
            "accept_len": torch.empty((B,), **i32),
            "path_nodes": torch.empty((B, N), **i32),
            "next_token": torch.empty((B,), **i32),
            "err_flags": torch.zeros((1,), **i32),
        }
        sv_verify_tree_sampling(target, draft, node_tokens, parents, temperature, uniforms, stream=stream,
                                **self.out)
        lib = _load()
        code = _dtype_code(target)
        self._ws = workspace(dev, int(lib.sv_tree_sampling_workspace_bytes(B, N, V, code)), stream)
        self._keep = (target, draft, node_tokens, parents, temperature, uniforms)
        o = self.out
        self._fn = lib.sv_verify_tree_sampling
        self._args = (
            _ptr(target), _ptr(draft), code, _ptr(node_tokens), _ptr(parents), _ptr(temperature), _ptr(uniforms),
            B, N, V, _ptr(o["accept_len"]), _ptr(o["path_nodes"]), _ptr(o["next_token"]), _ptr(o["err_flags"]),
            _ptr(self._ws), self._ws.numel(), _stream_handle(dev, stream))

    def __init__(self, *args, stream=None, **kw):
        # outputs and the workspace are allocated and zero-filled on the
        # stream the calls will run on (the caller's current one by default)
        first = args[0]
        with _on_call_stream(first.device, stream) as (s, outer):
            self._init(*args, stream=s, **kw)
            _used_on(s, outer, list(args))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            _check(st, "sv_verify_tree_sampling")
        return self.out


class PreparedLMHeadChainCall:
    """``sv_verify_chain_lm_head`` with every argument checked and marshalled
    once (calling the object only enqueues the kernels)."""

    def _init(self, hidden, head_weight, draft, draft_tokens, temperature, uniforms, *, stream=None):
        B, K1, H = hidden.shape
        V = head_weight.shape[0]
        K = K1 - 1
        dev = hidden.device
        self.out = sv_verify_chain_lm_head(hidden, head_weight, draft, draft_tokens, temperature, uniforms,
                                           stream=stream)
        lib = _load()
        self._ws = workspace(dev, int(lib.sv_lm_head_chain_workspace_bytes(B, K, V, H)), stream)
        self._keep = (hidden, head_weight, draft, draft_tokens, temperature, uniforms)
        o = self.out
        self._fn = lib.sv_verify_chain_lm_head
        self._args = (
            _ptr(hidden), _ptr(head_weight), H, _ptr(o["target_logits"]), _ptr(draft) if K > 0 else None,
            _ptr(draft_tokens) if K > 0 else None, _ptr(temperature), _ptr(uniforms), B, K, V,
            _ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o.get("p_draft")), _ptr(o.get("q_draft")),
            _ptr(o.get("residual_mass")), _ptr(o["err_flags"]), _ptr(self._ws), self._ws.numel(),
            _stream_handle(dev, stream))

    def __init__(self, *args, stream=None, **kw):
        first = args[0]
        with _on_call_stream(first.device, stream) as (s, outer):
            self._init(*args, stream=s, **kw)
            _used_on(s, outer, list(args))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            _check(st, "sv_verify_chain_lm_head")
        return self.out


class PreparedLMHeadLogitsCall:
    """``sv_lm_head_logits`` marshalled once (the LM head alone)."""

    def _init(self, hidden, head_weight, *, stream=None):
        H = hidden.shape[-1]
        V = head_weight.shape[0]
        dev = hidden.device
        self.logits = sv_lm_head_logits(hidden, head_weight, stream=stream)
        self._keep = (hidden, head_weight)
        self._fn = _load().sv_lm_head_logits
        self._args = (_ptr(hidden), _ptr(head_weight), hidden.numel() // H, H, V, _ptr(self.logits),
                      _stream_handle(dev, stream))

    def __init__(self, *args, stream=None, **kw):
        first = args[0]
        with _on_call_stream(first.device, stream) as (s, outer):
            self._init(*args, stream=s, **kw)
            _used_on(s, outer, list(args))

    def __call__(self):
        st = self._fn(*self._args)
        if st != SV_OK:
            _check(st, "sv_lm_head_logits")
        return self.logits
