"""Python binding of libmds.so, the MI355X Markov draft-sampling library.

Argument marshalling only: every step of the path runs in the HIP kernels of
libmds.so. Tensors are torch CUDA (ROCm) tensors; the calls enqueue work on
the current torch stream (or the given one) and return without synchronising.
The C entry points are declared in include/mds.h; the functions here carry
the same names without the ``mds_`` prefix.

The library must have been built in-tree (``python -m
markov_draft_sampling_amd.build``); importing this module does not build it,
and every call fails with an error if it is missing.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "F32", "BF16", "MdsError", "library_path", "abi_version", "draft_workspace_bytes", "verify_workspace_bytes",
    "new_workspace", "workspace_status", "verify_slot_offsets", "markov_w2_tiled_bytes", "tile_markov_w2",
    "markov_draft_loop", "markov_draft_loop_noalloc", "markov_draft_loop_timed", "rejection_verify",
    "debug_noise", "debug_gumbel", "debug_top_p", "STATUS_BAD_ANCHOR", "STATUS_BAD_DRAFT", "STATUS_BAD_INDEX", "SALT_DRAFT", "SALT_ACCEPT",
    "SALT_RESAMPLE",
]

F32, BF16 = 0, 1
STATUS_BAD_ANCHOR, STATUS_BAD_DRAFT, STATUS_BAD_INDEX = 1, 2, 8
SALT_DRAFT, SALT_ACCEPT, SALT_RESAMPLE = 1 << 30, 1, 2
DRAFT_FP64_GUMBEL, DRAFT_W2_TILED = 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class MdsError(RuntimeError):
    pass


def library_path() -> str:
    return os.path.join(_HERE, "libmds.so")


_c_int, _c_i64, _c_sz, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "mds_abi_version": ([], _c_int),
    "mds_status_string": ([_c_int], ctypes.c_char_p),
    "mds_last_error": ([], ctypes.c_char_p),
    "mds_draft_workspace_bytes": ([_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_c_sz)], _c_int),
    "mds_verify_workspace_bytes": ([_c_int, _c_int, _c_int, _c_int, _c_int, ctypes.POINTER(_c_sz)], _c_int),
    "mds_markov_draft_loop": ([_c_int] * 4 + [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int,
                                              _c_i64, _c_i64, _vp, _vp, _vp, _c_sz, _vp], _c_int),
    "mds_markov_draft_loop_timed": ([_c_int] * 4 + [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                    _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _c_sz, _vp, _vp, _vp,
                                                    ctypes.POINTER(_c_int)], _c_int),
    "mds_rejection_verify": ([_c_int] * 3 + [_vp, _c_i64, _vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _vp, _c_sz, _vp], _c_int),
    "mds_markov_draft_loop_ex": ([_c_int] * 4 + [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _c_int, _vp,
                                                 _vp, _vp, _c_int, _vp, _c_int, _c_i64, _c_i64, _vp, _vp,
                                                 ctypes.c_uint32, _vp, _c_sz, _vp, _vp, _vp, ctypes.POINTER(_c_int)],
                                 _c_int),
    "mds_draft_topk_workspace_bytes": ([_c_int] * 5 + [ctypes.POINTER(_c_sz)], _c_int),
    "mds_markov_w2_tiled_bytes": ([_c_int, _c_int, ctypes.POINTER(_c_sz)], _c_int),
    "mds_tile_markov_w2": ([_c_int, _c_int, _vp, _vp, _c_sz, _vp], _c_int),
    "mds_markov_draft_loop_topk": ([_c_int] * 5 + [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _c_int, _vp,
                                                   _vp, _vp, _c_int, _vp, _c_int, _c_i64, _c_i64, _vp, _vp,
                                                   ctypes.c_uint32, _vp, _c_sz, _vp, _vp, _vp], _c_int),
    "mds_draft_lm_head": ([_c_int] * 4 + [_vp, _c_i64, _vp, _vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp], _c_int),
    "mds_markov_draft_loop_from_hidden": ([_c_int] * 5 + [_vp, _c_i64, _vp, _vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp,
                                                          _vp, _vp, _vp, _vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp,
                                                          _c_sz, _vp, _vp, _vp], _c_int),
    "mds_rejection_verify_indexed": ([_c_int] * 3 + [_vp, _c_i64, _vp, _c_int, _c_i64, _c_i64, _c_int, _vp, _vp, _vp,
                                                     _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp],
                                     _c_int),
    "mds_debug_noise": ([_c_int, _vp, _c_i64, _c_i64, ctypes.c_uint32, _vp, _vp, _vp], _c_int),
    "mds_debug_gumbel": ([_c_int, _vp, _vp, _vp], _c_int),
    "mds_verify_slot_offsets": ([_c_int, ctypes.POINTER(_c_sz), ctypes.POINTER(_c_sz)], _c_int),
    "mds_markov_draft_loop_noalloc": ([_c_int] * 4 + [_vp, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                      _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp], _c_int),
    "mds_debug_top_p": ([_c_int, _c_int, _vp, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp], _c_int),
}


def _lib():
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise MdsError(f"{path} is missing: build it with `python -m markov_draft_sampling_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def _check(rc: int, what: str):
    if rc != 0:
        lib = _lib()
        msg = lib.mds_last_error().decode()
        raise MdsError(f"{what}: {lib.mds_status_string(rc).decode()} ({rc}): {msg}")


def abi_version() -> int:
    return _lib().mds_abi_version()


def draft_workspace_bytes(B: int, K: int, V: int, r: int) -> int:
    out = _c_sz()
    _check(_lib().mds_draft_workspace_bytes(B, K, V, r, ctypes.byref(out)), "draft_workspace_bytes")
    return out.value


def verify_workspace_bytes(B: int, K: int, V: int, has_top_p: bool, has_draft_lse: bool) -> int:
    out = _c_sz()
    _check(_lib().mds_verify_workspace_bytes(B, K, V, int(has_top_p), int(has_draft_lse), ctypes.byref(out)),
           "verify_workspace_bytes")
    return out.value


def verify_slot_offsets(b: int) -> tuple[int, int]:
    """Byte offsets of request b's arrival counter and final-draw key in a
    verification workspace (host only)."""
    c, k = _c_sz(), _c_sz()
    _check(_lib().mds_verify_slot_offsets(b, ctypes.byref(c), ctypes.byref(k)), "verify_slot_offsets")
    return c.value, k.value


def new_workspace(nbytes: int, device=None):
    """A zeroed uint8 device buffer usable as a workspace (zeroed once: the
    library never clears its sticky status word)."""
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


def workspace_status(ws) -> int:
    """The sticky status word (MDS_STATUS_* bits); synchronises on the read."""
    return int(ws[:4].view(dtype=__import__("torch").int32).item())


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise MdsError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return _vp(s.cuda_stream)


def _need(cond, msg):
    if not cond:
        raise MdsError(msg)


def _draft_args(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens, draft_lse,
                workspace):
    import torch
    _need(base.is_cuda, "tensors must be on the GPU")
    _need(base.dim() == 3 and base.stride(2) == 1, "base must be [B, >=K, V] with unit column stride")
    _need(cache.dim() == 3 and cache.stride(2) == 1, "cache must be [B, K, V] with unit column stride")
    B, K = draft_tokens.shape
    V = base.shape[2]
    _need(base.shape[0] == B and base.shape[1] >= K, "base must hold K rows per request")
    _need(tuple(cache.shape) == (B, K, V), "cache must be [B, K, V]")
    _need(w1.dtype == torch.bfloat16 and w2.dtype == torch.bfloat16, "w1 and w2 must be bf16")
    _need(w1.is_contiguous() and w2.is_contiguous() and w1.shape == w2.shape and w1.shape[0] == V,
          "w1 and w2 must be contiguous [V, r]")
    _need(anchor_tokens.dtype == torch.int32 and anchor_tokens.numel() == B, "anchor_tokens must be int32 [B]")
    _need(anchor_pos.dtype == torch.int64 and anchor_pos.numel() == B, "anchor_pos must be int64 [B]")
    _need(temperature.dtype == torch.float32 and temperature.numel() == B, "temperature must be float32 [B]")
    _need(seeds.dtype == torch.int64 and seeds.numel() == B, "seeds must be int64 [B]")
    _need(draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous(), "draft_tokens must be int32 [B, K]")
    for t in (anchor_tokens, anchor_pos, temperature, seeds):
        _need(t.is_contiguous(), "per-request arrays must be contiguous")
    if draft_lse is not None:
        _need(draft_lse.dtype == torch.float32 and draft_lse.is_contiguous() and draft_lse.numel() == B * K,
              "draft_lse must be float32 [B, K]")
    if workspace is not None:
        _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(),
              "workspace must be a contiguous uint8 tensor")
    r = w1.shape[1]
    return (B, K, V, r, _ptr(base), _dtype_code(base), base.stride(0), base.stride(1), _ptr(w1), _ptr(w2),
            _ptr(anchor_tokens), _ptr(anchor_pos), _ptr(temperature), _ptr(seeds), _ptr(cache), _dtype_code(cache),
            cache.stride(0), cache.stride(1), _ptr(draft_tokens), _ptr(draft_lse), _ptr(workspace),
            0 if workspace is None else workspace.numel())


def markov_draft_loop(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens,
                      draft_lse=None, workspace=None, stream=None):
    """Run the K-step Markov draft loop (mds_markov_draft_loop); K = draft_tokens.shape[1].

    Writes cache [B, K, V], draft_tokens [B, K] int32 and, if given,
    draft_lse [B, K] float32. Returns the workspace used.
    """
    B, K = draft_tokens.shape
    if workspace is None:
        workspace = new_workspace(draft_workspace_bytes(B, K, base.shape[2], w1.shape[1]), base.device)
    args = _draft_args(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens, draft_lse,
                       workspace)
    _check(_lib().mds_markov_draft_loop(*args, _stream(stream, base.device)), "markov_draft_loop")
    return workspace


def markov_draft_loop_noalloc(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens,
                              draft_lse, status, stream=None) -> None:
    """markov_draft_loop whose scratch lives inside the library (no workspace;
    K * B <= 1024). status: int32/uint32 device tensor of one element, the
    sticky status word (zeroed by the caller)."""
    _need(status.numel() == 1 and status.element_size() == 4 and status.is_cuda, "status: one 4-byte device word")
    args = _draft_args(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens, draft_lse,
                       None)
    # _draft_args ends with (workspace ptr, workspace bytes): replaced by the status word
    _check(_lib().mds_markov_draft_loop_noalloc(*args[:-2], _vp(status.data_ptr()), _stream(stream, base.device)),
           "markov_draft_loop_noalloc")


def markov_draft_loop_timed(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens,
                            draft_lse, workspace, ev_begin, ev_end, stream=None) -> int:
    """markov_draft_loop recording ev_begin / ev_end (torch.cuda.Event with
    timing) around the Markov step kernel launches; returns how many
    launches that span held (K)."""
    import torch
    args = _draft_args(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens, draft_lse,
                       workspace)
    st = stream if stream is not None else torch.cuda.current_stream(base.device)
    for e in (ev_begin, ev_end):  # torch creates the underlying HIP event on its first record
        if not e.cuda_event:
            e.record(st)
    n = _c_int(0)
    _check(_lib().mds_markov_draft_loop_timed(*args, _stream(stream, base.device), _vp(ev_begin.cuda_event),
                                              _vp(ev_end.cuda_event), ctypes.byref(n)), "markov_draft_loop_timed")
    return n.value


def rejection_verify(target, cache, draft_tokens, temperature, seeds, anchor_pos, out_tokens, num_accepted,
                     draft_lse=None, top_p=None, workspace=None, stream=None):
    """Rejection-sampling verification (mds_rejection_verify).

    target: float32 [B*(K+1), V] (unit column stride); cache as written by the
    draft loop; writes out_tokens [B, K+1] int32 and num_accepted [B] int32.
    """
    import torch
    B, K = draft_tokens.shape
    V = target.shape[1]
    _need(target.is_cuda and target.dtype == torch.float32, "target must be a float32 GPU tensor")
    _need(target.dim() == 2 and target.shape[0] == B * (K + 1) and target.stride(1) == 1,
          "target must be [B*(K+1), V] with unit column stride")
    _need(cache.dim() == 3 and tuple(cache.shape) == (B, K, V) and cache.stride(2) == 1, "cache must be [B, K, V]")
    _need(out_tokens.dtype == torch.int32 and out_tokens.is_contiguous() and out_tokens.numel() == B * (K + 1),
          "out_tokens must be int32 [B, K+1]")
    _need(num_accepted.dtype == torch.int32 and num_accepted.numel() == B, "num_accepted must be int32 [B]")
    _need(draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous(), "draft_tokens must be int32 [B, K]")
    if top_p is not None:
        _need(top_p.dtype == torch.float32 and top_p.numel() == B and top_p.is_contiguous(), "top_p: float32 [B]")
    if draft_lse is not None:
        _need(draft_lse.dtype == torch.float32 and draft_lse.numel() == B * K, "draft_lse: float32 [B, K]")
    if workspace is None:
        workspace = new_workspace(verify_workspace_bytes(B, K, V, top_p is not None, draft_lse is not None),
                                  target.device)
    rc = _lib().mds_rejection_verify(B, K, V, _ptr(target), target.stride(0), _ptr(cache), _dtype_code(cache),
                                     cache.stride(0), cache.stride(1), _ptr(draft_lse), _ptr(draft_tokens),
                                     _ptr(temperature), _ptr(top_p), _ptr(seeds), _ptr(anchor_pos), _ptr(out_tokens),
                                     _ptr(num_accepted), _ptr(workspace), workspace.numel(),
                                     _stream(stream, target.device))
    _check(rc, "rejection_verify")
    return workspace


def markov_w2_tiled_bytes(V: int, r: int) -> int:
    out = _c_sz()
    _check(_lib().mds_markov_w2_tiled_bytes(V, r, ctypes.byref(out)), "markov_w2_tiled_bytes")
    return out.value


def tile_markov_w2(w2, out=None, stream=None):
    """w2 bf16 [V, r] -> bf16 [ceil(V/16), 16*r] holding it in the tiled order
    of mds_tile_markov_w2 (for markov_draft_loop_ex(w2_tiled=True)), written
    into `out` when given, else into a new tensor; returns it."""
    import torch
    _need(w2.is_cuda and w2.dtype == torch.bfloat16 and w2.dim() == 2 and w2.is_contiguous(),
          "w2 must be a contiguous bf16 [V, r] GPU tensor")
    V, r = w2.shape
    n = markov_w2_tiled_bytes(V, r) // 2
    if out is None:
        out = torch.empty((n // (16 * r), 16 * r), dtype=torch.bfloat16, device=w2.device)
    _need(out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (n // (16 * r), 16 * r),
          "out must be a contiguous bf16 [ceil(V/16), 16 r] tensor")
    _check(_lib().mds_tile_markov_w2(V, r, _ptr(w2), _ptr(out), 2 * n, _stream(stream, w2.device)), "tile_markov_w2")
    return out


def markov_draft_loop_ex(base, w1, w2, anchor_tokens, idx_map, sample_pos, temperature, seeds, cache, draft_tokens,
                         row_mapping=None, draft_lse=None, fp64_gumbel=False, workspace=None, stream=None,
                         events=None, w2_tiled=False):
    """Draft loop with request-state indexing and options (mds_markov_draft_loop_ex).

    idx_map int32 [B, K] (state slot per row and step, < 0 inert) or None
    (slot = batch row), sample_pos int64 [B, K] (predicted position P; the
    draw is keyed by P - 1), temperature / seeds [n_slots], row_mapping int32
    [n_slots] or None, cache [n_cache_rows, K, V]; fp64_gumbel: float64 Gumbel
    variates and scores; w2_tiled: w2 is tile_markov_w2's output for the
    [V, r] matrix (w1 [V, r] gives r). base, anchor_tokens, draft_tokens,
    draft_lse are batch-indexed. events: optional (begin, end) torch.cuda.Event pair
    recorded around the Markov step launches; then returns (workspace, number
    of launches).
    """
    import torch
    B, K = draft_tokens.shape
    V = base.shape[2]
    _need(base.is_cuda and base.dim() == 3 and base.stride(2) == 1 and base.shape[0] == B and base.shape[1] >= K,
          "base must be a GPU tensor [B, >=K, V] with unit column stride")
    _need(cache.dim() == 3 and cache.shape[1] == K and cache.shape[2] == V and cache.stride(2) == 1,
          "cache must be [n_cache_rows, K, V] with unit column stride")
    _need(w1.dtype == torch.bfloat16 and w2.dtype == torch.bfloat16 and w1.is_contiguous() and w2.is_contiguous()
          and w1.dim() == 2 and w1.shape[0] == V, "w1 and w2 must be contiguous bf16, w1 [V, r]")
    r = w1.shape[1]
    if w2_tiled:
        _need(tuple(w2.shape) == ((V + 15) // 16, 16 * r), "tiled w2 must be tile_markov_w2's [ceil(V/16), 16 r]")
    else:
        _need(w2.shape == w1.shape, "w2 must be [V, r]")
    _need(anchor_tokens.dtype == torch.int32 and anchor_tokens.numel() == B and anchor_tokens.is_contiguous(),
          "anchor_tokens must be int32 [B]")
    if idx_map is not None:
        _need(idx_map.dtype == torch.int32 and idx_map.numel() == B * K and idx_map.is_contiguous(),
              "idx_map must be int32 [B, K]")
    _need(sample_pos.dtype == torch.int64 and sample_pos.numel() == B * K and sample_pos.is_contiguous(),
          "sample_pos must be int64 [B, K]")
    n_slots = temperature.numel()
    _need(temperature.dtype == torch.float32 and temperature.is_contiguous(), "temperature must be float32 [n_slots]")
    _need(seeds.dtype == torch.int64 and seeds.numel() == n_slots and seeds.is_contiguous(),
          "seeds must be int64 [n_slots]")
    if row_mapping is not None:
        _need(row_mapping.dtype == torch.int32 and row_mapping.numel() == n_slots and row_mapping.is_contiguous(),
              "row_mapping must be int32 [n_slots]")
    _need(draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous(), "draft_tokens must be int32 [B, K]")
    if draft_lse is not None:
        _need(draft_lse.dtype == torch.float32 and draft_lse.is_contiguous() and draft_lse.numel() == B * K,
              "draft_lse must be float32 [B, K]")
    if workspace is None:
        workspace = new_workspace(draft_workspace_bytes(B, K, V, w1.shape[1]), base.device)
    ev = (None, None)
    if events is not None:
        st = stream if stream is not None else torch.cuda.current_stream(base.device)
        for e in events:  # torch creates the underlying HIP event on its first record
            if not e.cuda_event:
                e.record(st)
        ev = (_vp(events[0].cuda_event), _vp(events[1].cuda_event))
    n = _c_int(0)
    rc = _lib().mds_markov_draft_loop_ex(
        B, K, V, w1.shape[1], _ptr(base), _dtype_code(base), base.stride(0), base.stride(1), _ptr(w1), _ptr(w2),
        _ptr(anchor_tokens), _ptr(idx_map), _ptr(sample_pos), n_slots, _ptr(temperature), _ptr(seeds),
        _ptr(row_mapping), cache.shape[0], _ptr(cache), _dtype_code(cache), cache.stride(0), cache.stride(1),
        _ptr(draft_tokens), _ptr(draft_lse), (DRAFT_FP64_GUMBEL if fp64_gumbel else 0) | (DRAFT_W2_TILED if w2_tiled
                                                                                           else 0), _ptr(workspace),
        workspace.numel(), _stream(stream, base.device), ev[0], ev[1], ctypes.byref(n))
    _check(rc, "markov_draft_loop_ex")
    return (workspace, n.value) if events is not None else workspace


def draft_topk_workspace_bytes(B: int, K: int, V: int, r: int, topk: int) -> int:
    out = _c_sz()
    _check(_lib().mds_draft_topk_workspace_bytes(B, K, V, r, topk, ctypes.byref(out)), "draft_topk_workspace_bytes")
    return out.value


def markov_draft_loop_topk(base, w1, w2, anchor_tokens, idx_map, sample_pos, temperature, seeds, cache, draft_tokens,
                           topk, row_mapping=None, draft_lse=None, fp64_gumbel=False, workspace=None, stream=None,
                           events=None):
    """Top-k Markov drafting (mds_markov_draft_loop_topk).

    Arguments as for markov_draft_loop_ex, plus topk (candidates per row,
    1..256). events: optional (begin, end) torch.cuda.Event pair recorded
    around the candidate-selection launch.
    """
    import torch
    B, K = draft_tokens.shape
    V = base.shape[2]
    _need(base.is_cuda and base.dim() == 3 and base.stride(2) == 1 and base.shape[0] == B and base.shape[1] >= K,
          "base must be a GPU tensor [B, >=K, V] with unit column stride")
    _need(cache.dim() == 3 and cache.shape[1] == K and cache.shape[2] == V and cache.stride(2) == 1,
          "cache must be [n_cache_rows, K, V] with unit column stride")
    _need(w1.dtype == torch.bfloat16 and w2.dtype == torch.bfloat16 and w1.is_contiguous() and w2.is_contiguous()
          and w1.shape == w2.shape and w1.shape[0] == V, "w1 and w2 must be contiguous bf16 [V, r]")
    _need(anchor_tokens.dtype == torch.int32 and anchor_tokens.numel() == B and anchor_tokens.is_contiguous(),
          "anchor_tokens must be int32 [B]")
    if idx_map is not None:
        _need(idx_map.dtype == torch.int32 and idx_map.numel() == B * K and idx_map.is_contiguous(),
              "idx_map must be int32 [B, K]")
    _need(sample_pos.dtype == torch.int64 and sample_pos.numel() == B * K and sample_pos.is_contiguous(),
          "sample_pos must be int64 [B, K]")
    n_slots = temperature.numel()
    _need(temperature.dtype == torch.float32 and temperature.is_contiguous(), "temperature must be float32 [n_slots]")
    _need(seeds.dtype == torch.int64 and seeds.numel() == n_slots and seeds.is_contiguous(),
          "seeds must be int64 [n_slots]")
    if row_mapping is not None:
        _need(row_mapping.dtype == torch.int32 and row_mapping.numel() == n_slots and row_mapping.is_contiguous(),
              "row_mapping must be int32 [n_slots]")
    _need(draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous(), "draft_tokens must be int32 [B, K]")
    if draft_lse is not None:
        _need(draft_lse.dtype == torch.float32 and draft_lse.is_contiguous() and draft_lse.numel() == B * K,
              "draft_lse must be float32 [B, K]")
    if workspace is None:
        workspace = new_workspace(draft_topk_workspace_bytes(B, K, V, w1.shape[1], int(topk)), base.device)
    ev = (None, None)
    if events is not None:
        st = stream if stream is not None else torch.cuda.current_stream(base.device)
        for e in events:  # torch creates the underlying HIP event on its first record
            if not e.cuda_event:
                e.record(st)
        ev = (_vp(events[0].cuda_event), _vp(events[1].cuda_event))
    rc = _lib().mds_markov_draft_loop_topk(
        B, K, V, w1.shape[1], int(topk), _ptr(base), _dtype_code(base), base.stride(0), base.stride(1), _ptr(w1),
        _ptr(w2), _ptr(anchor_tokens), _ptr(idx_map), _ptr(sample_pos), n_slots, _ptr(temperature), _ptr(seeds),
        _ptr(row_mapping), cache.shape[0], _ptr(cache), _dtype_code(cache), cache.stride(0), cache.stride(1),
        _ptr(draft_tokens), _ptr(draft_lse), DRAFT_FP64_GUMBEL if fp64_gumbel else 0, _ptr(workspace),
        workspace.numel(), _stream(stream, base.device), ev[0], ev[1])
    _check(rc, "markov_draft_loop_topk")
    return workspace


def draft_lm_head(hidden, lm_head, out, K, stream=None, events=None):
    """Base draft logits from the draft LM head (mds_draft_lm_head).

    hidden bf16 [B*K, H] (row b*K + k, unit column stride), lm_head bf16
    [V, H] contiguous, out float32 or bf16 [B, >=K, V] with unit column
    stride (rows k < K are written). events: optional (begin, end)
    torch.cuda.Event pair recorded around the launch.
    """
    import torch
    V, H = lm_head.shape
    _need(hidden.is_cuda and hidden.dtype == torch.bfloat16 and hidden.dim() == 2 and hidden.shape[1] == H
          and hidden.stride(1) == 1 and hidden.shape[0] % K == 0, "hidden must be bf16 [B*K, H] with unit column stride")
    B = hidden.shape[0] // K
    _need(lm_head.dtype == torch.bfloat16 and lm_head.is_contiguous(), "lm_head must be contiguous bf16 [V, H]")
    _need(out.dim() == 3 and out.shape[0] == B and out.shape[1] >= K and out.shape[2] == V and out.stride(2) == 1,
          "out must be [B, >=K, V] with unit column stride")
    ev = (None, None)
    if events is not None:
        st = stream if stream is not None else torch.cuda.current_stream(hidden.device)
        for e in events:  # torch creates the underlying HIP event on its first record
            if not e.cuda_event:
                e.record(st)
        ev = (_vp(events[0].cuda_event), _vp(events[1].cuda_event))
    rc = _lib().mds_draft_lm_head(B, K, V, H, _ptr(hidden), hidden.stride(0), _ptr(lm_head), _ptr(out),
                                  _dtype_code(out), out.stride(0), out.stride(1), _stream(stream, hidden.device),
                                  ev[0], ev[1])
    _check(rc, "draft_lm_head")


def _event_ptrs(events, stream, device):
    """(begin, end) void pointers of an optional torch.cuda.Event pair."""
    import torch
    if events is None:
        return (None, None)
    st = stream if stream is not None else torch.cuda.current_stream(device)
    for e in events:  # torch creates the underlying HIP event on its first record
        if not e.cuda_event:
            e.record(st)
    return (_vp(events[0].cuda_event), _vp(events[1].cuda_event))


def markov_draft_loop_from_hidden(hidden, lm_head, base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache,
                                  draft_tokens, draft_lse=None, workspace=None, stream=None, events=None):
    """The draft LM head then the K-step draft loop in one call
    (mds_markov_draft_loop_from_hidden); K = draft_tokens.shape[1].

    hidden bf16 [B*K, H], lm_head bf16 [V, H] as for draft_lm_head; base
    float32 or bf16 [B, >=K, V] receives the base logits of steps 1..K-1
    (its step-0 rows are scratch). The rest as for markov_draft_loop.
    events: optional (begin, end) torch.cuda.Event pair recorded around the
    call's launches. Returns the workspace used.
    """
    import torch
    B, K = draft_tokens.shape
    V, H = lm_head.shape
    _need(hidden.is_cuda and hidden.dtype == torch.bfloat16 and hidden.dim() == 2 and hidden.shape[1] == H
          and hidden.stride(1) == 1 and hidden.shape[0] == B * K, "hidden must be bf16 [B*K, H] with unit column stride")
    _need(lm_head.dtype == torch.bfloat16 and lm_head.is_contiguous(), "lm_head must be contiguous bf16 [V, H]")
    if workspace is None:
        workspace = new_workspace(draft_workspace_bytes(B, K, V, w1.shape[1]), base.device)
    args = _draft_args(base, w1, w2, anchor_tokens, anchor_pos, temperature, seeds, cache, draft_tokens, draft_lse,
                       workspace)
    ev = _event_ptrs(events, stream, base.device)
    rc = _lib().mds_markov_draft_loop_from_hidden(*args[:4], H, _ptr(hidden), hidden.stride(0), _ptr(lm_head),
                                                  *args[4:], _stream(stream, base.device), ev[0], ev[1])
    _check(rc, "markov_draft_loop_from_hidden")
    return workspace


def rejection_verify_indexed(target, cache, draft_tokens, idx_map, temperature, seeds, anchor_pos, out_tokens,
                             num_accepted, row_mapping=None, draft_lse=None, top_p=None, workspace=None,
                             stream=None):
    """Verification with request-state indexing (mds_rejection_verify_indexed).

    idx_map int32 [B] (state slot per request, < 0 padding); temperature,
    seeds, top_p [n_slots]; row_mapping int32 [n_slots] or None; cache
    [n_cache_rows, K, V].
    """
    import torch
    B, K = draft_tokens.shape
    V = target.shape[1]
    _need(target.is_cuda and target.dtype == torch.float32 and target.dim() == 2 and target.shape[0] == B * (K + 1)
          and target.stride(1) == 1, "target must be float32 [B*(K+1), V] with unit column stride")
    _need(cache.dim() == 3 and cache.shape[1] == K and cache.shape[2] == V and cache.stride(2) == 1,
          "cache must be [n_cache_rows, K, V]")
    _need(idx_map.dtype == torch.int32 and idx_map.numel() == B and idx_map.is_contiguous(), "idx_map must be int32 [B]")
    n_slots = temperature.numel()
    _need(temperature.dtype == torch.float32 and temperature.is_contiguous(), "temperature must be float32 [n_slots]")
    _need(seeds.dtype == torch.int64 and seeds.numel() == n_slots and seeds.is_contiguous(),
          "seeds must be int64 [n_slots]")
    if top_p is not None:
        _need(top_p.dtype == torch.float32 and top_p.numel() == n_slots and top_p.is_contiguous(),
              "top_p must be float32 [n_slots]")
    if row_mapping is not None:
        _need(row_mapping.dtype == torch.int32 and row_mapping.numel() == n_slots and row_mapping.is_contiguous(),
              "row_mapping must be int32 [n_slots]")
    _need(out_tokens.dtype == torch.int32 and out_tokens.is_contiguous() and out_tokens.numel() == B * (K + 1),
          "out_tokens must be int32 [B, K+1]")
    _need(num_accepted.dtype == torch.int32 and num_accepted.numel() == B, "num_accepted must be int32 [B]")
    _need(draft_tokens.dtype == torch.int32 and draft_tokens.is_contiguous(), "draft_tokens must be int32 [B, K]")
    if draft_lse is not None:
        _need(draft_lse.dtype == torch.float32 and draft_lse.numel() == B * K, "draft_lse: float32 [B, K]")
    if workspace is None:
        workspace = new_workspace(verify_workspace_bytes(B, K, V, top_p is not None, draft_lse is not None),
                                  target.device)
    rc = _lib().mds_rejection_verify_indexed(
        B, K, V, _ptr(target), target.stride(0), _ptr(cache), _dtype_code(cache), cache.stride(0), cache.stride(1),
        cache.shape[0], _ptr(draft_lse), _ptr(draft_tokens), _ptr(idx_map), n_slots, _ptr(temperature), _ptr(top_p),
        _ptr(seeds), _ptr(row_mapping), _ptr(anchor_pos), _ptr(out_tokens), _ptr(num_accepted), _ptr(workspace),
        workspace.numel(), _stream(stream, target.device))
    _check(rc, "rejection_verify_indexed")
    return workspace


def debug_noise(cols, seed: int, pos_key: int, salt: int):
    """Device Philox words and float32 Gumbel variates for int32 columns `cols`."""
    import torch
    _need(cols.is_cuda and cols.dtype == torch.int32 and cols.is_contiguous(), "cols must be int32 on the GPU")
    words = torch.empty(cols.numel(), dtype=torch.int32, device=cols.device)
    g = torch.empty(cols.numel(), dtype=torch.float32, device=cols.device)
    _check(_lib().mds_debug_noise(cols.numel(), _ptr(cols), int(seed), int(pos_key), int(salt), _ptr(words), _ptr(g),
                                  _stream(None, cols.device)), "debug_noise")
    return words, g


def debug_gumbel(words):
    """float32 Gumbel variates the kernels derive from 32-bit words (int32 tensor)."""
    import torch
    _need(words.is_cuda and words.dtype == torch.int32 and words.is_contiguous(), "words must be int32 on the GPU")
    g = torch.empty(words.numel(), dtype=torch.float32, device=words.device)
    _check(_lib().mds_debug_gumbel(words.numel(), _ptr(words), _ptr(g), _stream(None, words.device)), "debug_gumbel")
    return g


def debug_top_p(target, temperature, top_p):
    """Exact top-p kept set per row as verification computes it.

    target: float32 [rows, V] on the GPU; temperature, top_p: float32 [rows].
    Returns (tau uint32-as-int64, cut, log_z, on) tensors of [rows].
    """
    import torch
    rows, V = target.shape
    _need(target.is_cuda and target.dtype == torch.float32 and target.stride(1) == 1, "target: float32 [rows, V]")
    ws = new_workspace(verify_workspace_bytes(rows, 1, V, True, True), target.device)
    tau = torch.empty(rows, dtype=torch.int32, device=target.device)
    cut = torch.empty(rows, dtype=torch.int32, device=target.device)
    log_z = torch.empty(rows, dtype=torch.float32, device=target.device)
    on = torch.empty(rows, dtype=torch.int32, device=target.device)
    _check(_lib().mds_debug_top_p(rows, V, _ptr(target), target.stride(0), _ptr(temperature), _ptr(top_p), _ptr(tau),
                                  _ptr(cut), _ptr(log_z), _ptr(on), _ptr(ws), ws.numel(), _stream(None, target.device)),
           "debug_top_p")
    return tau.to(torch.int64) & 0xFFFFFFFF, cut, log_z, on
