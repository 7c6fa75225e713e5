"""Speculative-decoding verification over the vocabulary on MI355X (gfx950).

Thin Python binding of ``libspecverify.so`` (declared in
``include/spec_verify.h``).  It only marshals arguments: it checks dtypes,
shapes, devices and contiguity, allocates outputs and a scratch workspace
with torch when the caller passes none, and hands raw device pointers plus the
current HIP stream to the C ABI.  Every step of the verification runs in the
library's HIP kernels; there is no CPU path.

Entry points (same names as the C ABI):
  spec_verify_chain(target, draft, draft_tokens, uniforms, temperature, ...)
  spec_verify_chain_pointmass(target, draft_tokens, uniforms, temperature, ...)
  spec_verify_tree_greedy(target, parents, tokens, ...)
  spec_verify_tree_stochastic(target, draft, parents, tokens, uniforms, temperature, ...)
  spec_outcome_topk(logits, draft_tokens, temperature, ncache, ...)
  spec_cache_lookup(accept_len, out_tokens, cache_k, cache_a, ...)
  spec_tree_build(draft_logits, temperature, width, max_depth, budget, ...)
and the *_workspace_bytes sizing functions.
"""
from __future__ import annotations

import ctypes as _ct
import os as _os

__all__ = [
    "SV_DTYPE_F32", "SV_DTYPE_BF16", "SV_MAX_VOCAB", "SpecVerifyError", "library_path", "load_library",
    "spec_verify_chain", "spec_verify_tree_greedy", "spec_verify_chain_workspace_bytes",
    "spec_verify_chain_pointmass", "spec_verify_chain_pointmass_workspace_bytes",
    "spec_outcome_topk", "spec_outcome_topk_workspace_bytes", "spec_cache_lookup",
    "spec_tree_build", "spec_tree_build_workspace_bytes", "spec_verify_tree_stochastic",
    "spec_verify_tree_stochastic_workspace_bytes",
    "spec_verify_tree_greedy_workspace_bytes", "spec_verify_status_string",
    "spec_verify_chain_noalloc", "SV_NOALLOC_SCRATCH_BYTES",
]

SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_MAX_VOCAB = 1 << 29  # largest vocabulary size V any entry point accepts
SV_NOALLOC_SCRATCH_BYTES = 1 << 24  # static scratch of spec_verify_chain_noalloc per GPU

_HERE = _os.path.dirname(_os.path.abspath(__file__))
# Another build of the same sources (for instance one whose host code is
# built with address and undefined-behaviour sanitizers) can be loaded
# instead by naming it here; there is no other library and no fallback.
_LIB_PATH = _os.environ.get("SPEC_VERIFY_LIB") or _os.path.join(_HERE, "libspecverify.so")
_lib = None


class SpecVerifyError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {spec_verify_status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libspecverify.so (built by exact_draft_verification_amd.build).

    Raises RuntimeError if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not _os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing; build it with `python -m exact_draft_verification_amd.build`")
    # torch ships its own HIP runtime under the same soname; importing torch
    # first makes the library bind to that one, so streams and device
    # pointers from torch are valid in it.
    _torch()
    lib = _ct.CDLL(_LIB_PATH)
    P, I32, SZ, D = _ct.c_void_p, _ct.c_int32, _ct.c_size_t, _ct.c_double
    lib.spec_verify_status_string.argtypes = [I32]
    lib.spec_verify_status_string.restype = _ct.c_char_p
    lib.spec_verify_chain_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.spec_verify_chain_workspace_bytes.restype = SZ
    lib.spec_verify_tree_greedy_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.spec_verify_tree_greedy_workspace_bytes.restype = SZ
    chain_args = [P, P, I32, P, P, I32, I32, I32, D, P, P, P, P, SZ, P]
    lib.spec_verify_chain_pointmass_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.spec_verify_chain_pointmass_workspace_bytes.restype = SZ
    pointmass_args = [P, I32, P, P, I32, I32, I32, D, P, P, P, P, SZ, P]
    lib.spec_outcome_topk_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.spec_outcome_topk_workspace_bytes.restype = SZ
    outcome_args = [P, I32, P, I32, I32, I32, D, I32, P, P, P, P, P, SZ, P]
    greedy_args = [P, I32, P, P, I32, I32, I32, P, P, P, P, SZ, P]
    lib.spec_verify_tree_stochastic_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.spec_verify_tree_stochastic_workspace_bytes.restype = SZ
    stochastic_args = [P, P, I32, P, P, P, I32, I32, I32, D, P, P, P, P, P, SZ, P]
    lib.spec_cache_lookup.argtypes = [P, P, I32, I32, P, P, I32, P, P]
    lib.spec_cache_lookup.restype = I32
    lib.spec_tree_build_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.spec_tree_build_workspace_bytes.restype = SZ
    build_args = [P, I32, P, I32, I32, I32, D, I32, I32, I32, P, P, P, P, P, P, SZ, P]
    lib.spec_verify_chain_noalloc.argtypes = [P, P, I32, P, P, I32, I32, I32, D, P, P, P, P]
    lib.spec_verify_chain_noalloc.restype = I32
    # the product entry points, and their instrumented twins (one more
    # argument: the hipEvent_t array the benchmark times kernels with)
    for name, args in (("spec_verify_chain", chain_args),
                       ("spec_verify_chain_pointmass", pointmass_args),
                       ("spec_outcome_topk", outcome_args),
                       ("spec_verify_tree_greedy", greedy_args),
                       ("spec_verify_tree_stochastic", stochastic_args),
                       ("spec_tree_build", build_args)):
        for fn, extra in ((name, []), (name + "_timed", [P])):
            f = getattr(lib, fn)
            f.argtypes = args + extra
            f.restype = I32
    _lib = lib
    return lib


def spec_verify_status_string(status: int) -> str:
    return load_library().spec_verify_status_string(int(status)).decode()


def spec_verify_chain_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_chain_workspace_bytes(B, gamma, V, dtype))


def spec_verify_chain_pointmass_workspace_bytes(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_chain_pointmass_workspace_bytes(B, gamma, V, dtype))


def spec_outcome_topk_workspace_bytes(R: int, gamma: int, V: int, dtype: int, ncache: int) -> int:
    return int(load_library().spec_outcome_topk_workspace_bytes(R, gamma, V, dtype, ncache))


def spec_tree_build_workspace_bytes(R: int, M: int, V: int, dtype: int, W: int, max_depth: int,
                                    budget: int) -> int:
    return int(load_library().spec_tree_build_workspace_bytes(R, M, V, dtype, W, max_depth, budget))


def spec_verify_tree_stochastic_workspace_bytes(B: int, n: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_tree_stochastic_workspace_bytes(B, n, V, dtype))


def spec_verify_tree_greedy_workspace_bytes(B: int, n: int, V: int, dtype: int) -> int:
    return int(load_library().spec_verify_tree_greedy_workspace_bytes(B, n, V, dtype))


# ----------------------------------------------------------------- helpers --

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, shape, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return None if t is None else _ct.c_void_p(t.data_ptr())


def _nbytes(t):
    return t.numel() * t.element_size()


def _new(shape, dtype, device, stream):
    """torch.empty for a tensor the library writes on `stream`.  A tensor
    allocated while another stream is current is marked as used on `stream`,
    so torch's allocator does not hand its memory to other work while
    `stream` may still be writing it (when `stream` is the current stream,
    as under graph capture, the allocation already belongs to it)."""
    torch = _torch()
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return _ct.c_void_p(stream.cuda_stream)


def _invoke(lib, name, phase_events, *args):
    """Calls the entry point `name`, or, when phase_events (a sequence of
    hipEvent_t handles) is given, its instrumented twin `name`_timed, which
    records them around the dominant kernel (benchmark timing only)."""
    if phase_events is None:
        return getattr(lib, name)(*args)
    arr = (_ct.c_void_p * len(phase_events))(*[_ct.c_void_p(int(e)) for e in phase_events])
    return getattr(lib, name + "_timed")(*args, _ct.cast(arr, _ct.c_void_p))


_ws_cache: dict = {}


def _workspace(nbytes: int, device, stream):
    """A scratch workspace reused across calls on one device and stream (calls
    on one stream never overlap; the library needs no initialised contents)."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (str(device), int(stream.cuda_stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = _new(max(nbytes, 256), torch.uint8, device, stream)
        _ws_cache[key] = ws
    return ws


# ------------------------------------------------------------- entry points --

def spec_verify_chain(target, draft, draft_tokens, uniforms, temperature, *, accept_len=None,
                      out_tokens=None, final_dist=None, want_dist=False, workspace=None,
                      stream=None, phase_events=None):
    """Chain verification on the GPU.

    target [B, gamma+1, V] and draft [B, gamma, V] (float32 or bfloat16, same
    dtype), draft_tokens int32 [B, gamma], uniforms float32 [B, gamma+1],
    temperature > 0.  Returns (accept_len [B], out_tokens [B, gamma+1],
    final_dist [B, V] or None).  The call is asynchronous on `stream`
    (default: the current stream)."""
    torch = _torch()
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, g1, V = target.shape
    g = g1 - 1
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", (B, g1, V), device=dev)
    _check(draft, "draft", (B, g, V), dtype=target.dtype, device=dev)
    _check(draft_tokens, "draft_tokens", (B, g), dtype=torch.int32, device=dev)
    _check(uniforms, "uniforms", (B, g1), dtype=torch.float32, device=dev)
    if accept_len is None:
        accept_len = _new(B, torch.int32, dev, stream)
    if out_tokens is None:
        out_tokens = _new((B, g1), torch.int32, dev, stream)
    if final_dist is None and want_dist:
        final_dist = _new((B, V), torch.float32, dev, stream)
    _check(accept_len, "accept_len", (B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", (B, g1), dtype=torch.int32, device=dev)
    if final_dist is not None:
        _check(final_dist, "final_dist", (B, V), dtype=torch.float32, device=dev)
    need = spec_verify_chain_workspace_bytes(B, g, V, code)
    if need == 0:
        raise SpecVerifyError(2, "spec_verify_chain")
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    st = _invoke(lib, "spec_verify_chain", phase_events, _ptr(target), _ptr(draft), code,
                 _ptr(draft_tokens), _ptr(uniforms), B, g, V, float(temperature), _ptr(accept_len),
                 _ptr(out_tokens), _ptr(final_dist), _ptr(workspace), _nbytes(workspace), _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_chain")
    return accept_len, out_tokens, final_dist


def spec_verify_chain_noalloc(target, draft, draft_tokens, uniforms, temperature, *,
                              accept_len=None, out_tokens=None, final_dist=None, want_dist=False,
                              stream=None):
    """Chain verification through the allocation-free entry point: the
    library uses its static per-GPU scratch instead of a workspace.  Same
    arguments and results as spec_verify_chain (outputs the caller does not
    pass are allocated here, by torch, not by the library)."""
    torch = _torch()
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, g1, V = target.shape
    g = g1 - 1
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", (B, g1, V), device=dev)
    _check(draft, "draft", (B, g, V), dtype=target.dtype, device=dev)
    _check(draft_tokens, "draft_tokens", (B, g), dtype=torch.int32, device=dev)
    _check(uniforms, "uniforms", (B, g1), dtype=torch.float32, device=dev)
    if accept_len is None:
        accept_len = _new(B, torch.int32, dev, stream)
    if out_tokens is None:
        out_tokens = _new((B, g1), torch.int32, dev, stream)
    if final_dist is None and want_dist:
        final_dist = _new((B, V), torch.float32, dev, stream)
    _check(accept_len, "accept_len", (B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", (B, g1), dtype=torch.int32, device=dev)
    if final_dist is not None:
        _check(final_dist, "final_dist", (B, V), dtype=torch.float32, device=dev)
    st = lib.spec_verify_chain_noalloc(_ptr(target), _ptr(draft), code, _ptr(draft_tokens),
                                       _ptr(uniforms), B, g, V, float(temperature),
                                       _ptr(accept_len), _ptr(out_tokens), _ptr(final_dist),
                                       _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_chain_noalloc")
    return accept_len, out_tokens, final_dist


def spec_verify_chain_pointmass(target, draft_tokens, uniforms, temperature, *, accept_len=None,
                                out_tokens=None, final_dist=None, want_dist=False,
                                workspace=None, stream=None, phase_events=None):
    """Point-mass chain verification on the GPU (no draft logits).

    target [B, gamma+1, V] (float32 or bfloat16), draft_tokens int32
    [B, gamma], uniforms float32 [B, gamma+1], temperature > 0.  Returns
    (accept_len [B], out_tokens [B, gamma+1], final_dist [B, V] or None)."""
    torch = _torch()
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V]")
    B, g1, V = target.shape
    g = g1 - 1
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", (B, g1, V), device=dev)
    _check(draft_tokens, "draft_tokens", (B, g), dtype=torch.int32, device=dev)
    _check(uniforms, "uniforms", (B, g1), dtype=torch.float32, device=dev)
    if accept_len is None:
        accept_len = _new(B, torch.int32, dev, stream)
    if out_tokens is None:
        out_tokens = _new((B, g1), torch.int32, dev, stream)
    if final_dist is None and want_dist:
        final_dist = _new((B, V), torch.float32, dev, stream)
    _check(accept_len, "accept_len", (B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", (B, g1), dtype=torch.int32, device=dev)
    if final_dist is not None:
        _check(final_dist, "final_dist", (B, V), dtype=torch.float32, device=dev)
    need = spec_verify_chain_pointmass_workspace_bytes(B, g, V, code)
    if need == 0:
        raise SpecVerifyError(2, "spec_verify_chain_pointmass")
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    st = _invoke(lib, "spec_verify_chain_pointmass", phase_events, _ptr(target), code,
                 _ptr(draft_tokens), _ptr(uniforms), B, g, V, float(temperature), _ptr(accept_len),
                 _ptr(out_tokens), _ptr(final_dist), _ptr(workspace), _nbytes(workspace), _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_chain_pointmass")
    return accept_len, out_tokens, final_dist


def spec_outcome_topk(logits, draft_tokens, temperature, ncache, *, out_k=None, out_a=None,
                      out_p=None, hit=None, workspace=None, stream=None, phase_events=None):
    """Outcome scores and the ncache most probable outcomes on the GPU.

    logits [R, gamma+1, V] (float32 or bfloat16), draft_tokens int32
    [R, gamma].  Returns (k [R, ncache] int32, a [R, ncache] int32,
    p [R, ncache] float64, hit [R] float64)."""
    torch = _torch()
    lib = load_library()
    if logits.dim() != 3:
        raise ValueError("logits must be [R, gamma+1, V]")
    R, g1, V = logits.shape
    g = g1 - 1
    dev = logits.device
    code = _dtype_code(logits)
    _check(logits, "logits", (R, g1, V), device=dev)
    _check(draft_tokens, "draft_tokens", (R, g), dtype=torch.int32, device=dev)
    ncache = int(ncache)
    if out_k is None:
        out_k = _new((R, ncache), torch.int32, dev, stream)
    if out_a is None:
        out_a = _new((R, ncache), torch.int32, dev, stream)
    if out_p is None:
        out_p = _new((R, ncache), torch.float64, dev, stream)
    if hit is None:
        hit = _new(R, torch.float64, dev, stream)
    _check(out_k, "out_k", (R, ncache), dtype=torch.int32, device=dev)
    _check(out_a, "out_a", (R, ncache), dtype=torch.int32, device=dev)
    _check(out_p, "out_p", (R, ncache), dtype=torch.float64, device=dev)
    _check(hit, "hit", (R,), dtype=torch.float64, device=dev)
    need = spec_outcome_topk_workspace_bytes(R, g, V, code, ncache)
    if need == 0:
        raise SpecVerifyError(2, "spec_outcome_topk")
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    st = _invoke(lib, "spec_outcome_topk", phase_events, _ptr(logits), code, _ptr(draft_tokens), R,
                 g, V, float(temperature), ncache, _ptr(out_k), _ptr(out_a), _ptr(out_p),
                 _ptr(hit), _ptr(workspace), _nbytes(workspace),
                 _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_outcome_topk")
    return out_k, out_a, out_p, hit


def spec_verify_tree_stochastic(target_logits, draft_logits, parents, tokens, uniforms,
                                temperature, *, want_dist=False, accept_len=None,
                                accept_node=None, out_tokens=None, final_dist=None,
                                workspace=None, stream=None, phase_events=None):
    """Stochastic tree verification on the GPU.

    target_logits, draft_logits [B, n, V] (float32 or bfloat16), parents and
    tokens int32 [B, n], uniforms float32 [B, n] (column 0 drives the draw).
    Returns (accept_len [B], accept_node [B], out_tokens [B, n], final_dist
    [B, V] or None)."""
    torch = _torch()
    lib = load_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, n, V]")
    B, n, V = target_logits.shape
    dev = target_logits.device
    code = _dtype_code(target_logits)
    _check(target_logits, "target_logits", (B, n, V), device=dev)
    _check(draft_logits, "draft_logits", (B, n, V), dtype=target_logits.dtype, device=dev)
    _check(parents, "parents", (B, n), dtype=torch.int32, device=dev)
    _check(tokens, "tokens", (B, n), dtype=torch.int32, device=dev)
    _check(uniforms, "uniforms", (B, n), dtype=torch.float32, device=dev)
    if accept_len is None:
        accept_len = _new(B, torch.int32, dev, stream)
    if accept_node is None:
        accept_node = _new(B, torch.int32, dev, stream)
    if out_tokens is None:
        out_tokens = _new((B, n), torch.int32, dev, stream)
    if want_dist and final_dist is None:
        final_dist = _new((B, V), torch.float32, dev, stream)
    _check(accept_len, "accept_len", (B,), dtype=torch.int32, device=dev)
    _check(accept_node, "accept_node", (B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", (B, n), dtype=torch.int32, device=dev)
    if final_dist is not None:
        _check(final_dist, "final_dist", (B, V), dtype=torch.float32, device=dev)
    need = spec_verify_tree_stochastic_workspace_bytes(B, n, V, code)
    if need == 0:
        raise SpecVerifyError(2, "spec_verify_tree_stochastic")
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    st = _invoke(lib, "spec_verify_tree_stochastic", phase_events, _ptr(target_logits),
                 _ptr(draft_logits), code, _ptr(parents), _ptr(tokens), _ptr(uniforms), B, n, V,
                 float(temperature), _ptr(accept_len), _ptr(accept_node), _ptr(out_tokens),
                 _ptr(final_dist), _ptr(workspace), _nbytes(workspace),
                 _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_tree_stochastic")
    return accept_len, accept_node, out_tokens, final_dist


def spec_tree_build(draft_logits, temperature, width, max_depth, budget, *, child_row=None,
                    parents=None, tokens=None, node_row=None, score=None, n_nodes=None,
                    workspace=None, stream=None, phase_events=None):
    """Best-first draft-tree construction on the GPU.

    draft_logits [R, M, V] (float32 or bfloat16): one row per potential node;
    child_row optional int32 [M, width].  Returns (parents, tokens, node_row
    [R, budget] int32, score [R, budget] float64, n_nodes [R] int32)."""
    torch = _torch()
    lib = load_library()
    if draft_logits.dim() != 3:
        raise ValueError("draft_logits must be [R, M, V]")
    R, M, V = draft_logits.shape
    dev = draft_logits.device
    code = _dtype_code(draft_logits)
    W, budget = int(width), int(budget)
    _check(draft_logits, "draft_logits", (R, M, V), device=dev)
    if child_row is not None:
        _check(child_row, "child_row", (M, W), dtype=torch.int32, device=dev)

    def out(t, name, shape, dt):
        if t is None:
            t = _new(shape, dt, dev, stream)
        _check(t, name, shape, dtype=dt, device=dev)
        return t

    parents = out(parents, "parents", (R, budget), torch.int32)
    tokens = out(tokens, "tokens", (R, budget), torch.int32)
    node_row = out(node_row, "node_row", (R, budget), torch.int32)
    score = out(score, "score", (R, budget), torch.float64)
    n_nodes = out(n_nodes, "n_nodes", (R,), torch.int32)
    need = spec_tree_build_workspace_bytes(R, M, V, code, W, int(max_depth), budget)
    if need == 0:
        raise SpecVerifyError(2, "spec_tree_build")
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    st = _invoke(lib, "spec_tree_build", phase_events, _ptr(draft_logits), code, _ptr(child_row),
                 R, M, V, float(temperature), W, int(max_depth), budget, _ptr(parents),
                 _ptr(tokens), _ptr(node_row), _ptr(score), _ptr(n_nodes), _ptr(workspace),
                 _nbytes(workspace), _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_tree_build")
    return parents, tokens, node_row, score, n_nodes


def spec_cache_lookup(accept_len, out_tokens, cache_k, cache_a, *, slot=None, stream=None):
    """Speculation-cache lookup on the GPU: for each block, the first cache
    slot whose outcome (k, a) is the verified one (k = accept_len,
    a = out_tokens[k]), else -1.  accept_len [R], out_tokens [R, gamma+1],
    cache_k and cache_a [R, ncache], all int32.  Returns slot [R] int32."""
    torch = _torch()
    lib = load_library()
    if out_tokens.dim() != 2 or cache_k.dim() != 2:
        raise ValueError("out_tokens must be [R, gamma+1] and cache_k [R, ncache]")
    R, g1 = out_tokens.shape
    ncache = cache_k.shape[1]
    dev = out_tokens.device
    _check(accept_len, "accept_len", (R,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", (R, g1), dtype=torch.int32, device=dev)
    _check(cache_k, "cache_k", (R, ncache), dtype=torch.int32, device=dev)
    _check(cache_a, "cache_a", (R, ncache), dtype=torch.int32, device=dev)
    if slot is None:
        slot = _new(R, torch.int32, dev, stream)
    _check(slot, "slot", (R,), dtype=torch.int32, device=dev)
    st = lib.spec_cache_lookup(_ptr(accept_len), _ptr(out_tokens), R, g1 - 1, _ptr(cache_k),
                               _ptr(cache_a), ncache, _ptr(slot), _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_cache_lookup")
    return slot


def spec_verify_tree_greedy(target, parents, tokens, *, accept_len=None, accept_node=None,
                            out_tokens=None, workspace=None, stream=None, phase_events=None):
    """Greedy tree verification on the GPU.

    target [B, n, V] (float32 or bfloat16), parents and tokens int32 [B, n].
    Returns (accept_len [B], accept_node [B], out_tokens [B, n])."""
    torch = _torch()
    lib = load_library()
    if target.dim() != 3:
        raise ValueError("target must be [B, n, V]")
    B, n, V = target.shape
    dev = target.device
    code = _dtype_code(target)
    _check(target, "target", (B, n, V), device=dev)
    _check(parents, "parents", (B, n), dtype=torch.int32, device=dev)
    _check(tokens, "tokens", (B, n), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = _new(B, torch.int32, dev, stream)
    if accept_node is None:
        accept_node = _new(B, torch.int32, dev, stream)
    if out_tokens is None:
        out_tokens = _new((B, n), torch.int32, dev, stream)
    _check(accept_len, "accept_len", (B,), dtype=torch.int32, device=dev)
    _check(accept_node, "accept_node", (B,), dtype=torch.int32, device=dev)
    _check(out_tokens, "out_tokens", (B, n), dtype=torch.int32, device=dev)
    need = spec_verify_tree_greedy_workspace_bytes(B, n, V, code)
    if need == 0:
        raise SpecVerifyError(2, "spec_verify_tree_greedy")
    if workspace is None:
        workspace = _workspace(need, dev, stream)
    st = _invoke(lib, "spec_verify_tree_greedy", phase_events, _ptr(target), code, _ptr(parents),
                 _ptr(tokens), B, n, V, _ptr(accept_len), _ptr(accept_node), _ptr(out_tokens),
                 _ptr(workspace), _nbytes(workspace),
                 _stream_handle(stream, dev))
    if st != 0:
        raise SpecVerifyError(st, "spec_verify_tree_greedy")
    return accept_len, accept_node, out_tokens
