"""ctypes binding of libpa.so (see include/pa.h for the contract).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, a non-zero status becomes ``PAError``.  Every
step of the path runs in the library's HIP kernels; there is no fallback.
torch is imported before the library is loaded so that both share the one HIP
runtime torch ships (same SONAME).
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpa.so")
_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

PA_OK = 0


class PAError(RuntimeError):
    """A libpa.so call returned a non-zero status."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {pa_status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


_lib = None
_lib_lock = threading.Lock()


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is not built; run `python -m paged_kv_cache_310_amd.build` "
                "(there is no non-HIP implementation of this path)")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        lib.pa_status_string.argtypes = [i32]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_append_kv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, vp]
        lib.pa_append_kv.restype = i32
        lib.pa_copy_blocks.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, i32, vp]
        lib.pa_copy_blocks.restype = i32
        lib.pa_append_kv_layers.argtypes = [vp, vp, vp, vp, i32, vp, i64, i64, i32, i32, i32,
                                            i32, vp]
        lib.pa_append_kv_layers.restype = i32
        lib.pa_copy_blocks_layers.argtypes = [vp, vp, i32, vp, i64, i64, i32, i32, i32, i32, vp]
        lib.pa_copy_blocks_layers.restype = i32
        lib.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        lib.pa_decode_workspace_size.restype = i32
        lib.pa_decode_default_workers.argtypes = [ctypes.POINTER(i32)]
        lib.pa_decode_default_workers.restype = i32
        lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i64,
                                  ctypes.c_float, vp, vp, vp, vp, sz, i32, i32, vp]
        lib.pa_decode.restype = i32
        lib.pa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                          i64, ctypes.c_float, vp, vp, vp, i32, i32, vp]
        lib.pa_decode_noalloc.restype = i32
        lib.pa_decode_shared.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                         i64, ctypes.c_float, vp, vp, vp, vp, i32, vp, vp, sz,
                                         i32, i32, vp]
        lib.pa_decode_shared.restype = i32
        lib.pa_decode_shared_workspace_size.argtypes = [i32, i32, i32, i32, i32,
                                                        ctypes.POINTER(sz)]
        lib.pa_decode_shared_workspace_size.restype = i32
        lib.pa_prefill.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i64, i32, i32, i32,
                                   i32, i64, ctypes.c_float, i32, vp]
        lib.pa_prefill.restype = i32
        lib.pa_prefill_split.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i64, i32, i32,
                                         i32, i32, i64, ctypes.c_float, i32, i32, vp, sz, vp]
        lib.pa_prefill_split.restype = i32
        lib.pa_prefill_split_plan.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32,
                                              ctypes.POINTER(i32), ctypes.POINTER(sz)]
        lib.pa_prefill_split_plan.restype = i32
        lib.pa_read_probe.argtypes = [vp, vp, i64, vp, i64, i32, i32, i32, vp]
        lib.pa_read_probe.restype = i32
        lib.pa_set_decode_events.argtypes = [vp, vp]
        lib.pa_set_decode_events.restype = i32
        _lib = lib
        return lib


def pa_status_string(status: int) -> str:
    return _load().pa_status_string(int(status)).decode()


# The current stream's handle as an int, without building a torch Stream
# object (about 30x cheaper per call); torch.cuda.current_stream otherwise.
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _ptr(t: Optional[torch.Tensor]):
    # ctypes passes an int (or None) for a c_void_p argument.
    return None if t is None else t.data_ptr()


def _device_index(device: torch.device) -> int:
    return device.index if device.index is not None else torch.cuda.current_device()


def _stream(device: torch.device, stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _current_raw_stream is not None:
        return _current_raw_stream(_device_index(device))
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DTYPES[t.dtype]


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_cache(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _need(k_cache.is_cuda and k_cache.dim() == 4 and k_cache.is_contiguous(),
          "k_cache must be a contiguous CUDA tensor [num_blocks, num_kv_heads, block_size, head_dim]")
    shape = k_cache.shape
    _need(v_cache.dtype == k_cache.dtype and v_cache.shape == shape and v_cache.is_contiguous()
          and v_cache.get_device() == k_cache.get_device(), "v_cache must match k_cache")
    return shape


def _call(name: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(name, status)


def pa_append_kv(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None) -> None:
    """Write ``k_new[t]``/``v_new[t]`` into slot ``slot_mapping[t]`` of the pools."""
    nb, hkv, bs, d = _check_cache(k_cache, v_cache)
    t = slot_mapping.numel()
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
          and slot_mapping.get_device() == k_cache.get_device(),
          "slot_mapping must be int64 on the pool device")
    for x in (k_new, v_new):
        _need(x.shape == (t, hkv, d) and x.dtype == k_cache.dtype and x.is_contiguous()
              and x.get_device() == k_cache.get_device(),
              "k_new/v_new must be [num_tokens, num_kv_heads, head_dim]")
    _call("pa_append_kv", _load().pa_append_kv(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), t, nb, hkv,
        bs, d, _dtype_code(k_cache), _stream(k_cache.device, stream)))


def pa_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """Copy whole blocks ``(src, dst)`` of both pools."""
    nb, hkv, bs, d = _check_cache(k_cache, v_cache)
    _need(block_mapping.dtype == torch.int64 and block_mapping.is_contiguous()
          and block_mapping.get_device() == k_cache.get_device() and block_mapping.numel() % 2 == 0,
          "block_mapping must be int64 [num_pairs, 2] on the pool device")
    _call("pa_copy_blocks", _load().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_mapping), block_mapping.numel() // 2, nb, hkv, bs,
        d, _dtype_code(k_cache), _stream(k_cache.device, stream)))


def _layer_pools(k_caches, v_caches):
    """Checks per-layer pools (same shape, dtype, device) and returns their
    shape and host arrays of their device pointers."""
    _need(len(k_caches) == len(v_caches) and len(k_caches) > 0,
          "k_caches and v_caches must be equally long, non-empty sequences of pools")
    shape = _check_cache(k_caches[0], v_caches[0])
    for k, v in zip(k_caches, v_caches):
        _need(_check_cache(k, v) == shape and k.dtype == k_caches[0].dtype
              and k.get_device() == k_caches[0].get_device(),
              "every layer's pools must match layer 0's")
    return shape, _ptr_array(k_caches), _ptr_array(v_caches)


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


def pa_append_kv_layers(k_caches, v_caches, k_new, v_new, slot_mapping, stream=None) -> None:
    """``pa_append_kv`` for every layer ``l`` (pools ``k_caches[l]``,
    ``v_caches[l]``, new rows ``k_new[l]``, ``v_new[l]``), one slot mapping for
    all layers, in one launch per 32 layers."""
    (nb, hkv, bs, d), kp, vp = _layer_pools(k_caches, v_caches)
    layers = len(k_caches)
    ref = k_caches[0]
    t = slot_mapping.numel()
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
          and slot_mapping.get_device() == ref.get_device(),
          "slot_mapping must be int64 on the pool device")
    _need(len(k_new) == layers and len(v_new) == layers, "one k_new and one v_new per layer")
    for x in list(k_new) + list(v_new):
        _need(x.shape == (t, hkv, d) and x.dtype == ref.dtype and x.is_contiguous()
              and x.get_device() == ref.get_device(),
              "k_new/v_new must be [num_tokens, num_kv_heads, head_dim]")
    _call("pa_append_kv_layers", _load().pa_append_kv_layers(
        kp, vp, _ptr_array(k_new), _ptr_array(v_new), layers, _ptr(slot_mapping), t, nb, hkv, bs,
        d, _dtype_code(ref), _stream(ref.device, stream)))


def pa_copy_blocks_layers(k_caches, v_caches, block_mapping, stream=None) -> None:
    """``pa_copy_blocks`` for every layer's pools, one pair list for all
    layers, in one launch per 32 layers."""
    (nb, hkv, bs, d), kp, vp = _layer_pools(k_caches, v_caches)
    ref = k_caches[0]
    _need(block_mapping.dtype == torch.int64 and block_mapping.is_contiguous()
          and block_mapping.get_device() == ref.get_device() and block_mapping.numel() % 2 == 0,
          "block_mapping must be int64 [num_pairs, 2] on the pool device")
    _call("pa_copy_blocks_layers", _load().pa_copy_blocks_layers(
        kp, vp, len(k_caches), _ptr(block_mapping), block_mapping.numel() // 2, nb, hkv, bs, d,
        _dtype_code(ref), _stream(ref.device, stream)))


def pa_decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             num_workers: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _call("pa_decode_workspace_size", _load().pa_decode_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers, ctypes.byref(out)))
    return int(out.value)


# Workspace sizes by (current device, sizes): the size is a pure function of
# them (the default worker count depends on the device's compute units).
_workspace_sizes = {}


def _decode_need(size_fn, device_index: int, b: int, hq: int, hkv: int, d: int,
                 num_workers: int) -> int:
    key = (size_fn, device_index, b, hq, hkv, d, num_workers)
    need = _workspace_sizes.get(key)
    if need is None:
        with torch.cuda.device(device_index):
            need = size_fn(b, hq, hkv, d, num_workers)
        if len(_workspace_sizes) >= 4096:   # batch sizes vary from step to step: stay bounded
            _workspace_sizes.clear()
        _workspace_sizes[key] = need
    return need


def pa_decode_default_workers() -> int:
    out = ctypes.c_int(0)
    _call("pa_decode_default_workers", _load().pa_decode_default_workers(ctypes.byref(out)))
    return int(out.value)


def pa_set_decode_events(before=None, after=None) -> None:
    """Record two ``torch.cuda.Event`` objects around the attention kernel of
    later pa_decode calls on this thread (``None, None`` stops)."""
    raw = []
    for ev in (before, after):
        if ev is None:
            raw.append(None)
        else:
            if ev.cuda_event == 0:          # torch creates the event on first record
                ev.record()
            raw.append(ctypes.c_void_p(ev.cuda_event))
    _call("pa_set_decode_events", _load().pa_set_decode_events(*raw))


_workspaces = {}


def pa_read_probe(base, tile_ids=None, tile_bytes: int = 4096, nontemporal: bool = False,
                  num_tiles: Optional[int] = None, num_workers: int = 0,
                  stream=None) -> torch.Tensor:
    """Read-bandwidth probe over the bytes of the CUDA tensor ``base``: the
    tiles ``tile_ids`` (int32, in that order) or, with ``tile_ids=None``, the
    first ``num_tiles`` tiles in address order (default: every whole tile).
    Returns the per-worker XOR checksums (int32 tensor on the device)."""
    _need(base.is_cuda and base.is_contiguous(), "base must be a contiguous CUDA tensor")
    nbytes = base.numel() * base.element_size()
    if tile_ids is not None:
        _need(tile_ids.dtype == torch.int32 and tile_ids.dim() == 1 and tile_ids.is_contiguous()
              and tile_ids.get_device() == base.get_device(),
              "tile_ids must be a 1-D int32 tensor on base's device")
        n = tile_ids.numel()
    else:
        n = nbytes // tile_bytes if num_tiles is None else int(num_tiles)
    workers = num_workers if num_workers > 0 else pa_decode_default_workers()
    checksum = torch.empty(workers, dtype=torch.int32, device=base.device)
    _call("pa_read_probe", _load().pa_read_probe(
        _ptr(checksum), _ptr(base), nbytes, _ptr(tile_ids), n, int(tile_bytes),
        1 if nontemporal else 0, workers, _stream(base.device, stream)))
    return checksum


def decode_workspace(device, nbytes: int, stream=None) -> torch.Tensor:
    """A workspace of at least ``nbytes`` for calls on ``stream`` (default:
    the device's current stream), reused by later calls on that same stream.

    A workspace must never serve two calls at once (include/pa.h), so each
    stream has its own: calls on one stream are ordered, calls on two streams
    are not.  The buffer is allocated while ``stream`` is current, so when a
    larger one replaces it, torch's caching allocator hands the old memory
    out again only in that stream's order, after the calls that used it."""
    if not isinstance(device, torch.device):
        device = torch.device(device)
    index = _device_index(device)
    key = (index, _stream(device, stream))   # the stream handle last
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        s = torch.cuda.current_stream(index) if stream is None else stream
        with torch.cuda.stream(s):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=index)
        _workspaces[key] = ws
    return ws


def _check_workspace(workspace: torch.Tensor, ref: torch.Tensor) -> None:
    _need(workspace.is_cuda and workspace.is_contiguous()
          and workspace.get_device() == ref.get_device(),
          "workspace must be a contiguous device tensor on q's device")


def _check_decode_args(q, k_cache, v_cache, block_tables, context_lens, out, k_new, v_new,
                       slot_mapping):
    """Checks pa_decode's tensors; returns the pool shape and ``out`` (made
    when not given)."""
    nb, hkv, bs, d = _check_cache(k_cache, v_cache)
    dev = k_cache.get_device()
    dt = k_cache.dtype
    _need(q.dim() == 3 and q.dtype == dt and q.is_contiguous() and q.get_device() == dev,
          "q must be [num_seqs, num_q_heads, head_dim] like the pools")
    b, hq, qd = q.shape
    _need(qd == d, "q must be [num_seqs, num_q_heads, head_dim] like the pools")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == b and block_tables.is_contiguous()
          and block_tables.get_device() == dev, "block_tables must be int32 [num_seqs, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1
          and context_lens.shape[0] == b and context_lens.is_contiguous()
          and context_lens.get_device() == dev,
          "context_lens must be a contiguous int32 [num_seqs] tensor")
    if k_new is not None and v_new is not None and slot_mapping is not None:
        row = (b, hkv, d)
        for x in (k_new, v_new):
            _need(x.dtype == dt and tuple(x.shape) == row and x.is_contiguous()
                  and x.get_device() == dev,
                  "k_new/v_new must be [num_seqs, num_kv_heads, head_dim]")
        _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1
              and slot_mapping.shape[0] == b and slot_mapping.is_contiguous()
              and slot_mapping.get_device() == dev,
              "slot_mapping must be a contiguous int64 [num_seqs] tensor")
    else:
        _need(k_new is None and v_new is None and slot_mapping is None,
              "k_new, v_new and slot_mapping go together")
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out.dtype == dt and tuple(out.shape) == (b, hq, d) and out.is_contiguous()
              and out.get_device() == dev, "out must match q")
    return (nb, hkv, bs, d), out


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out=None,
              k_new=None, v_new=None, slot_mapping=None, workspace=None, num_workers: int = 0,
              stream=None) -> torch.Tensor:
    """Decode-step paged attention; returns ``out`` [num_seqs, num_q_heads, head_dim]."""
    (nb, hkv, bs, d), out = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                               out, k_new, v_new, slot_mapping)
    b, hq, _ = q.shape
    if workspace is None:
        index = q.get_device()
        need = _decode_need(pa_decode_workspace_size, index, b, hq, hkv, d, num_workers)
        workspace = decode_workspace(q.device, need, stream)
    else:
        _check_workspace(workspace, q)
    _call("pa_decode", _load().pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), b, hq, hkv, d, bs, nb, float(scale),
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(workspace),
        workspace.numel() * workspace.element_size(), int(num_workers), _dtype_code(q),
        _stream(q.device, stream)))
    return out


def pa_decode_shared_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                    head_dim: int, num_workers: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _call("pa_decode_shared_workspace_size", _load().pa_decode_shared_workspace_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, num_workers, ctypes.byref(out)))
    return int(out.value)


def pa_decode_shared(q, k_cache, v_cache, block_tables, context_lens, scale, group_start,
                     prefix_lens, out=None, k_new=None, v_new=None, slot_mapping=None,
                     workspace=None, num_workers: int = 0, stream=None) -> torch.Tensor:
    """Decode-step paged attention over groups of sequences that share a
    prefix: the same result as ``pa_decode``, reading each group's shared
    tokens once.  ``group_start`` int32 [num_groups + 1] (groups are runs of
    consecutive sequences), ``prefix_lens`` int32 [num_seqs] (tokens each
    sequence shares with its group)."""
    (nb, hkv, bs, d), out = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                               out, k_new, v_new, slot_mapping)
    b, hq, _ = q.shape
    _need(group_start.dtype == torch.int32 and group_start.dim() == 1
          and group_start.numel() >= 1 and group_start.is_contiguous()
          and group_start.get_device() == q.get_device(),
          "group_start must be a contiguous int32 [num_groups + 1] tensor on q's device")
    _need(prefix_lens.dtype == torch.int32 and prefix_lens.shape == (b,)
          and prefix_lens.is_contiguous() and prefix_lens.get_device() == q.get_device(),
          "prefix_lens must be a contiguous int32 [num_seqs] tensor on q's device")
    if workspace is None:
        index = q.get_device()
        need = _decode_need(pa_decode_shared_workspace_size, index, b, hq, hkv, d, num_workers)
        workspace = decode_workspace(q.device, need, stream)
    else:
        _check_workspace(workspace, q)
    _call("pa_decode_shared", _load().pa_decode_shared(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), b, hq, hkv, d, bs, nb, float(scale),
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(group_start), group_start.numel() - 1,
        _ptr(prefix_lens), _ptr(workspace), workspace.numel() * workspace.element_size(),
        int(num_workers), _dtype_code(q), _stream(q.device, stream)))
    return out


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out=None,
                      k_new=None, v_new=None, slot_mapping=None, num_workers: int = 0,
                      stream=None) -> torch.Tensor:
    """``pa_decode`` whose workspace is the library's static device scratch
    array: the library call allocates nothing (``out`` is allocated here only
    when not given).  Calls that can overlap on one GPU race (include/pa.h)."""
    (nb, hkv, bs, d), out = _check_decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                               out, k_new, v_new, slot_mapping)
    b, hq, _ = q.shape
    _call("pa_decode_noalloc", _load().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), b, hq, hkv, d, bs, nb, float(scale),
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), int(num_workers), _dtype_code(q),
        _stream(q.device, stream)))
    return out


def pa_prefill_split_plan(num_seqs: int, max_query_len: int, num_query_tokens: int,
                          num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                          max_blocks_per_seq: int, num_splits: int = 0):
    """(splits, workspace bytes) that ``pa_prefill(..., num_splits=...)`` uses
    for these sizes; ``num_splits`` 0 asks for the automatic choice."""
    splits, nbytes = ctypes.c_int(0), ctypes.c_size_t(0)
    _call("pa_prefill_split_plan", _load().pa_prefill_split_plan(
        num_seqs, max_query_len, num_query_tokens, num_q_heads, num_kv_heads, head_dim,
        block_size, max_blocks_per_seq, num_splits, ctypes.byref(splits), ctypes.byref(nbytes)))
    return int(splits.value), int(nbytes.value)


def pa_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
               max_query_len: Optional[int] = None, out=None, stream=None, num_splits: int = 1,
               workspace=None) -> torch.Tensor:
    """Causal attention of each sequence's query chunk (its newest tokens,
    already appended) through the block table; returns ``out``
    [num_query_tokens, num_q_heads, head_dim].  ``max_query_len`` bounds every
    chunk; when omitted it is read from ``query_start`` (a device-to-host
    copy).  ``num_splits`` other than 1 shares each row tile's keys out over
    that many workgroups (0: the library's choice) through ``pa_prefill_split``;
    ``workspace`` (a uint8 device tensor) is then allocated when not given."""
    nb, hkv, bs, d = _check_cache(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == k_cache.dtype and q.is_contiguous()
          and q.get_device() == k_cache.get_device(),
          "q must be [num_query_tokens, num_q_heads, head_dim] like the pools")
    t, hq, _ = q.shape
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.is_contiguous() and block_tables.get_device() == q.get_device(),
          "block_tables must be int32 [num_seqs, max_blocks]")
    b = block_tables.shape[0]
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (b,)
          and context_lens.is_contiguous() and context_lens.get_device() == q.get_device(),
          "context_lens must be int32 [num_seqs]")
    _need(query_start.dtype == torch.int32 and query_start.shape == (b + 1,)
          and query_start.is_contiguous() and query_start.get_device() == q.get_device(),
          "query_start must be int32 [num_seqs + 1]")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if b else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
          and out.get_device() == q.get_device(), "out must match q")
    if num_splits == 1:
        _call("pa_prefill", _load().pa_prefill(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), _ptr(query_start), b, int(max_query_len),
            t, hq, hkv, d, bs, nb, float(scale), _dtype_code(q), _stream(q.device, stream)))
        return out
    if workspace is None:
        _, nbytes = pa_prefill_split_plan(b, int(max_query_len), t, hq, hkv, d, bs,
                                          block_tables.shape[1], int(num_splits))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, q)
    _call("pa_prefill_split", _load().pa_prefill_split(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), _ptr(query_start), b, int(max_query_len), t,
        hq, hkv, d, bs, nb, float(scale), _dtype_code(q), int(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device, stream)))
    return out
