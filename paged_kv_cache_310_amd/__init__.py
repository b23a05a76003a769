"""MI355X-native paged KV cache: decode attention through block tables,
paged KV append and copy-on-write block copy, as hand-written HIP kernels for
gfx950 behind a C ABI (``include/pa.h``), with a thin ctypes binding.

The binding (``pa_append_kv``, ``pa_copy_blocks``, their layer-batched forms
``pa_append_kv_layers`` and ``pa_copy_blocks_layers``, ``pa_decode``,
``pa_decode_noalloc``, ``pa_decode_shared`` (with its workspace size),
``pa_prefill``, ``pa_prefill_split_plan``,
``pa_decode_workspace_size``, and the measurement probe ``pa_read_probe``) is loaded lazily from ``_binding`` so that the
host-only modules (block manager, workload generator) import without a GPU.
"""

__all__ = ["pa_append_kv", "pa_copy_blocks", "pa_append_kv_layers", "pa_copy_blocks_layers",
           "pa_decode", "pa_decode_noalloc", "pa_decode_shared",
           "pa_decode_shared_workspace_size", "pa_prefill", "pa_prefill_split_plan", "pa_decode_workspace_size",
           "pa_decode_default_workers", "decode_workspace", "pa_set_decode_events",
           "pa_status_string", "pa_read_probe", "library_path", "PAError"]


def __getattr__(name):
    if name in __all__:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
