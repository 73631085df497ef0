"""The C ABI library: it loads, exports what the header declares, and rejects bad
arguments on the host before touching the GPU (CPU only: no kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "deltalog.h")
LIB = os.path.join(ROOT, "linear_attention_recurrent_amd", "libdeltalog.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dl_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdeltalog.so is not built: run `python -m linear_attention_recurrent_amd.build`")
    from linear_attention_recurrent_amd import deltalog
    return deltalog.load_library()


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("dl_init_state", "dl_decode_step", "dl_merge", "dl_merge_on", "dl_merge_unit", "dl_eager_step",
              "dl_prefill", "dl_status_string"):
        assert n in names
    assert len(names) == 8, names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {LIB}").read()
    exported = set(re.findall(r"\sT\s+(dl_\w+)$", out, flags=re.M))
    assert exported == set(declared_functions()), exported


def test_side_libraries_export_their_calls():
    """The benchmark's probe library and the tracing build (both outside the ABI) load
    and export what bench.py calls; the tracing build also exports the whole ABI."""
    pkg = os.path.join(ROOT, "linear_attention_recurrent_amd")
    probe = os.path.join(pkg, "libdlprobe.so")
    trace = os.path.join(pkg, "libdeltalog_trace.so")
    for path in (probe, trace):
        if not os.path.exists(path):
            pytest.fail(f"{os.path.basename(path)} is not built: run `python -m linear_attention_recurrent_amd.build --trace`")
    exported = lambda path: set(re.findall(r"\sT\s+(dl_\w+)$", os.popen(f"nm -D --defined-only {path}").read(),
                                           flags=re.M))
    assert exported(probe) == {"dl_probe_tile_read", "dl_probe_tile_read_log", "dl_probe_tile_rw",
                               "dl_probe_tile_stream", "dl_probe_owned_stream", "dl_probe_quarter_split"}
    assert exported(trace) == set(declared_functions()) | {"dl_trace_copy"}
    p = ctypes.CDLL(probe)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    p.dl_probe_owned_stream.argtypes = [vp, ci, ci, vp, ci, vp]
    # argument checks, all rejected before any GPU call: null or misaligned buffers, no
    # tiles or workgroups, an unknown order, the unit order with tiles not a multiple of wgs
    for args in ((None, 512, 0, 0x10000, 256), (0x10000, 512, 0, None, 256), (0x10004, 512, 0, 0x10000, 256),
                 (0x10000, 0, 0, 0x10000, 256), (0x10000, 512, 0, 0x10000, 0), (0x10000, 512, 4, 0x10000, 256),
                 (0x10000, 512, -1, 0x10000, 256),
                 (0x10000, 300, 1, 0x10000, 256)):
        assert p.dl_probe_owned_stream(*args, None) == -1
    p.dl_probe_quarter_split.argtypes = [vp, ci, ci, vp, vp, vp, vp]
    for args in ((None, 512, 0, 0x10000, None, None), (0x10000, 512, 0, None, None, None),
                 (0x10004, 512, 0, 0x10000, None, None), (0x10000, 0, 0, 0x10000, None, None),
                 (0x10000, 512, 1, 0x10000, None, 0x10000), (0x10000, 512, 1, 0x10000, 0x10000, None),
                 (0x10000, 512, 1, 0x10000, 0x10000, 0x10004)):
        assert p.dl_probe_quarter_split(*args, None) == -1
    t = ctypes.CDLL(trace)
    t.dl_trace_copy.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert t.dl_trace_copy(None, -1) == -1  # argument check, no GPU call


def test_status_strings(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    for code, tag in [(dl.DL_OK, "DL_OK"), (dl.DL_EINVAL, "DL_EINVAL"), (dl.DL_EUNSUPPORTED, "DL_EUNSUPPORTED"),
                      (dl.DL_EALIGN, "DL_EALIGN"), (dl.DL_EHIP, "DL_EHIP")]:
        assert dl.status_string(code).startswith(tag)
    assert "unknown" in dl.status_string(12345)


# Fake device addresses: the host checks reject these calls before any HIP call,
# so nothing is dereferenced.
A = 0x10000      # 16-byte aligned
M = 0x10004      # misaligned


def _dims(dl, variant=0, batch=2, heads=2, dk=128, dv=128, L=16, base_dtype=0):
    return dl.Dims(variant, batch, heads, dk, dv, L, base_dtype)


def _pool(dl, base=A):
    return dl.Pool(base, A, A, A, A)


def _io(dl, variant=0, **kw):
    f = dict(q=A, k=A, v=A, decay=A, beta=A if variant != 2 else None,
             bonus=A if variant == 2 else None, out=A)
    f.update(kw)
    return dl.StepIO(f["q"], f["k"], f["v"], f["decay"], f["beta"], f["bonus"], f["out"])


def _decode(lib, dims, pool, io):
    return lib.dl_decode_step(ctypes.byref(dims), ctypes.byref(pool), ctypes.byref(io), None)


def test_dims_errors(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    bad = [(dict(variant=3), dl.DL_EINVAL), (dict(variant=-1), dl.DL_EINVAL), (dict(batch=-1), dl.DL_EINVAL),
           (dict(heads=0), dl.DL_EINVAL), (dict(L=0), dl.DL_EINVAL), (dict(L=129), dl.DL_EINVAL),
           (dict(dk=96), dl.DL_EUNSUPPORTED), (dict(dv=256), dl.DL_EUNSUPPORTED),
           (dict(batch=1 << 20, heads=1 << 12), dl.DL_EINVAL),
           (dict(base_dtype=2), dl.DL_EINVAL), (dict(base_dtype=-1), dl.DL_EINVAL)]
    for kw, code in bad:
        assert _decode(lib, _dims(dl, **kw), _pool(dl), _io(dl)) == code, kw
    assert lib.dl_decode_step(None, ctypes.byref(_pool(dl)), ctypes.byref(_io(dl)), None) == dl.DL_EINVAL


def test_pool_and_io_errors(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    d = _dims(dl)
    assert _decode(lib, d, dl.Pool(A, None, A, A, A), _io(dl)) == dl.DL_EINVAL
    assert _decode(lib, d, _pool(dl, base=M), _io(dl)) == dl.DL_EALIGN
    assert _decode(lib, d, _pool(dl), _io(dl, out=None)) == dl.DL_EINVAL
    assert _decode(lib, d, _pool(dl), _io(dl, q=M)) == dl.DL_EALIGN
    # one-scalar-per-tile arrays need only 4-byte alignment, but not less
    assert _decode(lib, d, _pool(dl), _io(dl, decay=A + 2)) == dl.DL_EALIGN
    assert _decode(lib, d, _pool(dl), _io(dl, out=A + 2)) == dl.DL_EALIGN
    assert _decode(lib, d, dl.Pool(A, A, A, A, A + 2), _io(dl)) == dl.DL_EALIGN
    d1 = _dims(dl, variant=1)
    assert _decode(lib, d1, _pool(dl), _io(dl, variant=1, decay=M)) == dl.DL_EALIGN
    assert _decode(lib, d1, dl.Pool(A, A, A, M, A), _io(dl, variant=1)) == dl.DL_EALIGN
    # variant / pointer mismatches
    assert _decode(lib, d, _pool(dl), _io(dl, beta=None)) == dl.DL_EUNSUPPORTED
    assert _decode(lib, d, _pool(dl), _io(dl, bonus=A)) == dl.DL_EUNSUPPORTED
    d2 = _dims(dl, variant=2, dk=64, dv=64, L=32)
    assert _decode(lib, d2, _pool(dl), _io(dl, variant=2, beta=A)) == dl.DL_EUNSUPPORTED
    assert _decode(lib, d2, _pool(dl), _io(dl, variant=2, bonus=None)) == dl.DL_EUNSUPPORTED
    assert lib.dl_decode_step(ctypes.byref(d), ctypes.byref(_pool(dl)), None, None) == dl.DL_EINVAL


def test_merge_init_eager_errors(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    d = _dims(dl, L=16)
    p = _pool(dl)
    assert lib.dl_merge(ctypes.byref(d), ctypes.byref(p), -1, None) == dl.DL_EINVAL
    assert lib.dl_merge(ctypes.byref(d), ctypes.byref(p), 17, None) == dl.DL_EINVAL
    # DL_MERGE_DUE: nothing is due between calls, so it checks its arguments and launches nothing
    # (the pool's pointers are fake here: a launch would fault)
    assert dl.MERGE_DUE == 0 and dl.MERGE_ALL == 1
    assert lib.dl_merge(ctypes.byref(d), ctypes.byref(p), dl.MERGE_DUE, None) == dl.DL_OK
    assert lib.dl_merge(ctypes.byref(d), None, dl.MERGE_DUE, None) == dl.DL_EINVAL
    assert lib.dl_merge(ctypes.byref(d), ctypes.byref(dl.Pool(M, A, A, A, A)), dl.MERGE_DUE, None) == dl.DL_EALIGN
    assert lib.dl_merge(ctypes.byref(d), None, 1, None) == dl.DL_EINVAL
    for unit in (-1, 3):
        assert lib.dl_merge_on(ctypes.byref(d), ctypes.byref(p), 1, unit, None) == dl.DL_EINVAL
    for unit in (dl.UNIT_AUTO, dl.UNIT_VALU, dl.UNIT_MFMA):
        assert lib.dl_merge_on(ctypes.byref(d), ctypes.byref(p), -1, unit, None) == dl.DL_EINVAL
        assert lib.dl_merge_on(ctypes.byref(d), ctypes.byref(p), dl.MERGE_DUE, unit, None) == dl.DL_OK
        assert lib.dl_merge_on(ctypes.byref(d), None, 1, unit, None) == dl.DL_EINVAL
    fills = (ctypes.c_int32 * 2)(0, 16)
    assert lib.dl_init_state(ctypes.byref(d), ctypes.byref(p), None, fills, None) == dl.DL_EINVAL
    fills = (ctypes.c_int32 * 2)(-1, 0)
    assert lib.dl_init_state(ctypes.byref(d), ctypes.byref(p), None, fills, None) == dl.DL_EINVAL
    assert lib.dl_init_state(ctypes.byref(d), ctypes.byref(p), M, None, None) == dl.DL_EALIGN
    assert lib.dl_eager_step(ctypes.byref(d), None, ctypes.byref(_io(dl)), None) == dl.DL_EINVAL
    assert lib.dl_eager_step(ctypes.byref(d), M, ctypes.byref(_io(dl)), None) == dl.DL_EALIGN
    # the eager comparator keeps an fp32 state only
    dbf = _dims(dl, base_dtype=dl.BASE_BF16)
    assert lib.dl_eager_step(ctypes.byref(dbf), A, ctypes.byref(_io(dl)), None) == dl.DL_EUNSUPPORTED


def test_batch_zero_returns_ok_without_looking_at_pointers(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    d = _dims(dl, batch=0)
    empty = dl.Pool(None, None, None, None, None)
    noio = dl.StepIO(None, None, None, None, None, None, None)
    assert lib.dl_decode_step(ctypes.byref(d), ctypes.byref(empty), ctypes.byref(noio), None) == dl.DL_OK
    assert lib.dl_merge(ctypes.byref(d), ctypes.byref(empty), 1, None) == dl.DL_OK
    assert lib.dl_merge_on(ctypes.byref(d), ctypes.byref(empty), 1, dl.UNIT_MFMA, None) == dl.DL_OK
    assert lib.dl_init_state(ctypes.byref(d), ctypes.byref(empty), None, None, None) == dl.DL_OK
    assert lib.dl_eager_step(ctypes.byref(d), None, ctypes.byref(noio), None) == dl.DL_OK


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "linear_attention_recurrent_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert not re.search(r"(^|[^A-Za-z])_work/", text), f


def _pio(dl, T=8, **kw):
    f = dict(q=A, k=A, v=A, decay=A, beta=A, bonus=None, out=A, eta=None, eps=0.0)
    f.update(kw)
    return dl.PrefillIO(f["q"], f["k"], f["v"], f["decay"], f["beta"], f["bonus"], f["out"], f["eta"], f["eps"], T)


def _prefill(lib, dims, pool, io):
    return lib.dl_prefill(ctypes.byref(dims), ctypes.byref(pool), ctypes.byref(io), None)


def test_prefill_errors(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    d = _dims(dl)
    p = _pool(dl)
    assert _prefill(lib, d, p, _pio(dl, T=-1)) == dl.DL_EINVAL
    assert _prefill(lib, _dims(dl, batch=1, heads=131072), p, _pio(dl)) == dl.DL_EINVAL  # 32-bit chunk offsets
    assert _prefill(lib, _dims(dl, batch=0, heads=131072), p, _pio(dl)) == dl.DL_EINVAL
    assert lib.dl_prefill(ctypes.byref(d), ctypes.byref(p), None, None) == dl.DL_EINVAL
    assert _prefill(lib, _dims(dl, variant=1), p, _pio(dl, decay=A + 4)) == dl.DL_EALIGN  # KDA decay rows: 16 B
    d2 = _dims(dl, variant=2, dk=64, dv=64)
    assert _prefill(lib, d2, p, _pio(dl)) == dl.DL_EUNSUPPORTED                       # beta given, no bonus
    assert _prefill(lib, d2, p, _pio(dl, beta=None)) == dl.DL_EUNSUPPORTED            # no bonus
    assert _prefill(lib, d2, p, _pio(dl, beta=None, bonus=M)) == dl.DL_EALIGN
    assert _prefill(lib, d, p, _pio(dl, bonus=A)) == dl.DL_EUNSUPPORTED               # GDN with a bonus
    assert _prefill(lib, d, p, _pio(dl, q=None)) == dl.DL_EINVAL
    assert _prefill(lib, d, p, _pio(dl, out=None)) == dl.DL_EINVAL
    assert _prefill(lib, d, p, _pio(dl, beta=None)) == dl.DL_EUNSUPPORTED       # neither beta nor eta
    assert _prefill(lib, d, p, _pio(dl, eta=A)) == dl.DL_EUNSUPPORTED           # both
    assert _prefill(lib, d, p, _pio(dl, beta=None, eta=A, eps=-1.0)) == dl.DL_EINVAL
    assert _prefill(lib, d, p, _pio(dl, k=M)) == dl.DL_EALIGN
    assert _prefill(lib, d, p, _pio(dl, decay=A + 2)) == dl.DL_EALIGN
    assert _prefill(lib, d, _pool(dl, base=M), _pio(dl)) == dl.DL_EALIGN
    assert _prefill(lib, d, dl.Pool(A, None, A, A, A), _pio(dl)) == dl.DL_EINVAL
    # an empty prompt needs no prompt pointers (it only folds): checked up to the pool
    assert _prefill(lib, d, dl.Pool(A, None, A, A, A), _pio(dl, T=0, q=None, k=None, v=None, out=None)) == dl.DL_EINVAL
    # batch 0: nothing is looked at
    empty = dl.Pool(None, None, None, None, None)
    assert _prefill(lib, _dims(dl, batch=0), empty, _pio(dl, q=None, k=None, v=None, out=None)) == dl.DL_OK


def test_pool_wrapper_starts_with_empty_logs():
    """The binding's pool allocates its fills as zeros, so a pool used before
    dl_init_state indexes no log slot (host-side allocation check, on the CPU)."""
    import torch

    from linear_attention_recurrent_amd import deltalog as dl
    for variant, dk, dv in ((dl.GDN, 128, 128), (dl.KDA, 128, 64), (dl.RWKV6, 64, 64)):
        p = dl.DeltaLogPool(variant, 3, 2, dk, dv, 8, device="cpu")
        assert p.fill.dtype == torch.int32 and tuple(p.fill.shape) == (3, 2)
        assert int(p.fill.abs().max()) == 0
        assert tuple(p.log_c.shape) == (3, 2, 8, 1 if variant == dl.GDN else dk)


# dl_merge's measured unit table, on both sides of every threshold:
# (variant, dk, dv, bf16 base, the shortest L on matrix cores, or None for never)
MERGE_TABLE = [
    (0, 128, 128, False, 32), (1, 128, 128, False, 32), (2, 128, 128, False, 32),
    (0, 128, 128, True, 32), (1, 128, 128, True, 64), (2, 128, 128, True, 64),
    (0, 128, 64, False, 64), (1, 64, 128, False, 64), (0, 128, 64, True, None), (1, 64, 128, True, None),
    (2, 64, 64, False, None), (2, 64, 64, True, None), (0, 64, 64, False, None),
]


def test_merge_unit_table(lib):
    from linear_attention_recurrent_amd import deltalog as dl
    for variant, dk, dv, bf16, first in MERGE_TABLE:
        base = dl.BASE_BF16 if bf16 else dl.BASE_F32
        for L in (1, 2, 4, 8, 16, 31, 32, 33, 63, 64, 65, 128):
            want = dl.UNIT_MFMA if first is not None and L >= first else dl.UNIT_VALU
            got = dl.dl_merge_unit(dl.Dims(variant, 4, 2, dk, dv, L, base))
            assert got == want, (variant, dk, dv, bf16, L, got)
    assert lib.dl_merge_unit(ctypes.byref(dl.Dims(0, 4, 2, 96, 128, 16, 0))) == dl.DL_EUNSUPPORTED
    assert lib.dl_merge_unit(ctypes.byref(dl.Dims(0, 4, 2, 128, 128, 129, 0))) == dl.DL_EINVAL
    assert lib.dl_merge_unit(None) == dl.DL_EINVAL
