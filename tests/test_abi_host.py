"""The C ABI without a GPU: the library loads into the process torch's HIP
runtime lives in, exports exactly what include/pa.h declares, and rejects bad
scalar arguments before making any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (loads torch's HIP runtime before libpa.so)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_310_amd import _binding, build
    if not os.path.exists(_binding.library_path()):
        build.build()
    return _binding._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_exports_match_header(lib):
    from paged_kv_cache_310_amd import _binding
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == declared_functions()
    for name in exported:
        assert hasattr(lib, name)


def test_single_hip_runtime_in_process(lib):
    maps = open("/proc/self/maps").read()
    hip = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(hip) == 1, hip


def test_status_strings(lib):
    for code in range(6):
        assert lib.pa_status_string(code)
    assert lib.pa_status_string(99) == b"unknown status"


def test_workspace_size_formula(lib):
    sz = ctypes.c_size_t(0)
    rec = lambda w: (w * 48 + 255) // 256 * 256     # one 48-byte merge record per worker
    assert lib.pa_decode_workspace_size(32, 40, 40, 128, 4096, ctypes.byref(sz)) == 0
    assert sz.value == rec(4096) + 4096 * 2 * 1 * 132 * 4
    assert lib.pa_decode_workspace_size(256, 64, 8, 128, 100, ctypes.byref(sz)) == 0
    assert sz.value == rec(100) + 100 * 2 * 8 * 132 * 4
    assert lib.pa_decode_workspace_size(4, 6, 4, 64, 8, ctypes.byref(sz)) == 1   # 6 % 4 != 0


FAKE = 1 << 20   # an aligned address that is never dereferenced: checks fail first


def decode_status(lib, **kw):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, mb=4, lens=FAKE, b=2, hq=8, hkv=8,
                d=128, bs=16, nb=10, scale=0.1, kn=None, vn=None, sm=None, ws=None, wsb=0,
                workers=64, dtype=1)
    args.update(kw)
    return lib.pa_decode(args["out"], args["q"], args["k"], args["v"], args["tab"], args["mb"],
                         args["lens"], args["b"], args["hq"], args["hkv"], args["d"], args["bs"],
                         args["nb"], args["scale"], args["kn"], args["vn"], args["sm"], args["ws"],
                         args["wsb"], args["workers"], args["dtype"], None)


def test_decode_rejects_bad_scalars_before_any_hip_call(lib):
    assert decode_status(lib, d=96) == 2
    assert decode_status(lib, bs=8) == 2
    assert decode_status(lib, dtype=7) == 2
    assert decode_status(lib, hq=6, hkv=4) == 1
    assert decode_status(lib, b=-1) == 1
    assert decode_status(lib, mb=0) == 1
    assert decode_status(lib, scale=float("nan")) == 1
    assert decode_status(lib, kn=FAKE) == 1               # fused arguments go together
    assert decode_status(lib, q=None) == 1
    assert decode_status(lib, q=FAKE + 4) == 1            # not 16-byte aligned
    assert decode_status(lib) == 3                        # no workspace
    assert decode_status(lib, ws=FAKE, wsb=16) == 3       # workspace too small
    assert decode_status(lib, b=0) == 0                   # nothing to do


def shared_status(lib, gs=FAKE, ng=2, plen=FAKE, **kw):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, mb=4, lens=FAKE, b=2, hq=8, hkv=8,
                d=128, bs=16, nb=10, scale=0.1, kn=None, vn=None, sm=None, ws=None, wsb=0,
                workers=64, dtype=1)
    args.update(kw)
    return lib.pa_decode_shared(args["out"], args["q"], args["k"], args["v"], args["tab"],
                                args["mb"], args["lens"], args["b"], args["hq"], args["hkv"],
                                args["d"], args["bs"], args["nb"], args["scale"], args["kn"],
                                args["vn"], args["sm"], gs, ng, plen, args["ws"], args["wsb"],
                                args["workers"], args["dtype"], None)


def test_shared_decode_rejects_bad_arguments_before_any_hip_call(lib):
    assert shared_status(lib, ng=-1) == 1
    assert shared_status(lib, ng=3) == 1                  # more groups than sequences
    assert shared_status(lib, gs=None) == 1
    assert shared_status(lib, plen=None) == 1
    assert shared_status(lib, d=96) == 2
    assert shared_status(lib, hq=6, hkv=4) == 1
    assert shared_status(lib) == 3                        # no workspace
    assert shared_status(lib, ws=FAKE, wsb=4096) == 3     # too small for 64 workers
    assert shared_status(lib, b=0, ng=0) == 0             # nothing to do


def test_shared_workspace_size_covers_both_paths(lib):
    sz = ctypes.c_size_t(0)
    rec = 132 * 4
    r256 = lambda x: (x + 255) // 256 * 256
    assert lib.pa_decode_shared_workspace_size(128, 40, 40, 128, 1024, ctypes.byref(sz)) == 0
    want = (r256(1024 * 48) + r256(1024 * 2 * 16 * rec) + 2 * r256(40 * 128 * 16)
            + 2 * r256(128 * 40 * rec))
    assert sz.value == want
    # fp32 head_dim 64 runs plain decode: the size still covers it
    plain = ctypes.c_size_t(0)
    assert lib.pa_decode_workspace_size(3, 64, 1, 64, 7, ctypes.byref(plain)) == 0
    assert lib.pa_decode_shared_workspace_size(3, 64, 1, 64, 7, ctypes.byref(sz)) == 0
    assert sz.value >= plain.value
    assert lib.pa_decode_shared_workspace_size(4, 6, 4, 64, 8, ctypes.byref(sz)) == 1


def test_noalloc_rejects_a_need_beyond_the_scratch_before_any_hip_call(lib):
    # 200,000 workers of 8 query heads per KV head need 1.7 GB of partials.
    st = lib.pa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 8, 128, 16, 10,
                               0.1, None, None, None, 200000, 1, None)
    assert st == 3
    st = lib.pa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 8, 96, 16, 10,
                               0.1, None, None, None, 8, 1, None)
    assert st == 2


def test_append_and_copy_reject_bad_scalars(lib):
    assert lib.pa_append_kv(None, None, None, None, None, 0, 10, 8, 16, 128, 1, None) == 0
    assert lib.pa_append_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 10, 8, 16, 96, 1, None) == 2
    assert lib.pa_append_kv(None, FAKE, FAKE, FAKE, FAKE, 3, 10, 8, 16, 128, 1, None) == 1
    assert lib.pa_append_kv(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 10, 8, 16, 128, 1, None) == 1
    assert lib.pa_copy_blocks(None, None, None, 0, 10, 8, 16, 128, 1, None) == 0
    assert lib.pa_copy_blocks(FAKE, FAKE, FAKE, 2, 10, 8, 32, 64, 3, None) == 2
    assert lib.pa_copy_blocks(FAKE, FAKE, None, 2, 10, 8, 32, 64, 0, None) == 1


def _ptrs(*values):
    arr = (ctypes.c_void_p * max(len(values), 1))()
    for i, x in enumerate(values):
        arr[i] = x
    return arr


def test_layer_batched_calls_reject_bad_arguments(lib):
    three = _ptrs(FAKE, FAKE + 4096, FAKE + 8192)
    holes = _ptrs(FAKE, None, FAKE)
    skew = _ptrs(FAKE, FAKE + 8, FAKE)
    app = lib.pa_append_kv_layers
    assert app(three, three, three, three, 3, FAKE, 0, 10, 8, 16, 128, 1, None) == 0   # no tokens
    assert app(three, three, three, three, 0, FAKE, 5, 10, 8, 16, 128, 1, None) == 0   # no layers
    assert app(three, three, three, three, -1, FAKE, 5, 10, 8, 16, 128, 1, None) == 1
    assert app(three, three, three, three, 3, FAKE, 5, 10, 8, 16, 96, 1, None) == 2
    assert app(three, holes, three, three, 3, FAKE, 5, 10, 8, 16, 128, 1, None) == 1
    assert app(three, three, three, skew, 3, FAKE, 5, 10, 8, 16, 128, 1, None) == 1
    assert app(None, three, three, three, 3, FAKE, 5, 10, 8, 16, 128, 1, None) == 1
    assert app(three, three, three, three, 3, None, 5, 10, 8, 16, 128, 1, None) == 1
    cp = lib.pa_copy_blocks_layers
    assert cp(three, three, 3, FAKE, 0, 10, 8, 16, 128, 1, None) == 0
    assert cp(three, three, 0, FAKE, 4, 10, 8, 16, 128, 1, None) == 0
    assert cp(three, three, 3, FAKE, -2, 10, 8, 16, 128, 1, None) == 1
    assert cp(three, three, 3, FAKE, 4, 10, 8, 16, 128, 7, None) == 2
    assert cp(three, holes, 3, FAKE, 4, 10, 8, 16, 128, 1, None) == 1
    assert cp(skew, three, 3, FAKE, 4, 10, 8, 16, 128, 1, None) == 1
    assert cp(three, three, 3, None, 4, 10, 8, 16, 128, 1, None) == 1


def prefill_status(lib, **kw):
    args = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, mb=4, lens=FAKE, qs=FAKE, b=2, mq=8,
                t=10, hq=8, hkv=2, d=128, bs=16, nb=10, scale=0.1, dtype=1)
    args.update(kw)
    return lib.pa_prefill(args["out"], args["q"], args["k"], args["v"], args["tab"], args["mb"],
                          args["lens"], args["qs"], args["b"], args["mq"], args["t"], args["hq"],
                          args["hkv"], args["d"], args["bs"], args["nb"], args["scale"],
                          args["dtype"], None)


def test_prefill_rejects_bad_arguments_before_any_hip_call(lib):
    assert prefill_status(lib, dtype=0) == 2              # fp32: no prefill kernel
    assert prefill_status(lib, d=64) == 2
    assert prefill_status(lib, bs=8) == 2
    assert prefill_status(lib, hq=6, hkv=4) == 1
    assert prefill_status(lib, b=-1) == 1
    assert prefill_status(lib, mq=-1) == 1
    assert prefill_status(lib, t=-1) == 1
    assert prefill_status(lib, mb=0) == 1
    assert prefill_status(lib, scale=float("nan")) == 1
    assert prefill_status(lib, qs=None) == 1
    assert prefill_status(lib, out=FAKE + 2) == 1         # not 16-byte aligned
    assert prefill_status(lib, b=0) == 0                  # nothing to do
    assert prefill_status(lib, mq=0) == 0
    assert prefill_status(lib, t=0) == 0


def test_decode_event_hook_arguments(lib):
    assert lib.pa_set_decode_events(FAKE, None) == 1
    assert lib.pa_set_decode_events(None, FAKE) == 1
    assert lib.pa_set_decode_events(None, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from paged_kv_cache_310_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _binding._load()


def test_read_probe_rejects_bad_arguments_before_any_hip_call(lib):
    def st(checksum=FAKE, base=FAKE, base_bytes=1 << 20, ids=None, n=16, tile=4096, nt=0, w=8):
        return lib.pa_read_probe(checksum, base, base_bytes, ids, n, tile, nt, w, None)
    assert st(tile=1024) == 1
    assert st(tile=16384) == 1
    assert st(nt=2) == 1
    assert st(n=-1) == 1
    assert st(w=-1) == 1
    assert st(base_bytes=-1) == 1
    assert st(checksum=None) == 1
    assert st(base=None) == 1
    assert st(base=FAKE + 8) == 1                       # not 16-byte aligned
    assert st(n=(1 << 20) // 4096 + 1) == 1              # more tiles than the buffer holds
    assert st(n=0, checksum=None, base=None) == 0        # nothing to do


def test_prefill_split_rejects_bad_arguments_before_any_hip_call(lib):
    def st(splits, ws=None, ws_bytes=0, **kw):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, mb=4, lens=FAKE, qs=FAKE, b=2, mq=8,
                 t=10, hq=8, hkv=2, d=128, bs=16, nb=10, scale=0.1, dtype=1)
        a.update(kw)
        return lib.pa_prefill_split(a["out"], a["q"], a["k"], a["v"], a["tab"], a["mb"],
                                    a["lens"], a["qs"], a["b"], a["mq"], a["t"], a["hq"],
                                    a["hkv"], a["d"], a["bs"], a["nb"], a["scale"], a["dtype"],
                                    splits, ws, ws_bytes, None)
    need = 3 * 10 * 8 * (128 + 4) * 4
    assert st(-1) == 1
    assert st(33) == 1
    assert st(3, dtype=0) == 2
    assert st(3) == 3                                     # no workspace
    assert st(3, FAKE, need - 1) == 3                     # too small
    assert st(3, FAKE + 8, need) == 3                     # not 16-byte aligned
    assert st(3, b=0) == 0                                # nothing to do


def test_prefill_split_plan(lib):
    splits, nbytes = ctypes.c_int(-7), ctypes.c_size_t(7)

    def plan(s, b=2, mq=8, t=10, hq=8, hkv=2, d=128, bs=16, mb=4):
        return lib.pa_prefill_split_plan(b, mq, t, hq, hkv, d, bs, mb, s, ctypes.byref(splits),
                                         ctypes.byref(nbytes))
    assert plan(3) == 0 and splits.value == 3 and nbytes.value == 3 * 10 * 8 * 132 * 4
    assert plan(16) == 0 and splits.value == 16 and nbytes.value == 16 * 10 * 8 * 132 * 4
    assert plan(1) == 0 and splits.value == 1 and nbytes.value == 0
    assert plan(32) == 0 and splits.value == 32 and nbytes.value == 32 * 10 * 8 * 132 * 4
    assert plan(33) == 1
    assert plan(-1) == 1
    assert plan(3, hq=6, hkv=4) == 1
    assert plan(3, mb=0) == 1
    assert lib.pa_prefill_split_plan(2, 8, 10, 8, 2, 128, 16, 4, 3, None,
                                     ctypes.byref(nbytes)) == 1
