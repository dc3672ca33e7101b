"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* every function include/mk.h declares is exported by libmk.so and bound by the
  Python binding;
* the ctypes structs have the C layout (offsets compiled from the header by gcc);
* argument errors are reported before anything touches the device.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from persistent_megakernel_loop_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mk.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_[a-z_0-9]+)\s*\(", text)))


def header_codes():
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(MK_\w+)\s+(-?\d+)", open(HEADER).read())}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.library_path()):
        pytest.fail("libmk.so is not built: run persistent_megakernel_loop_amd/build.py")
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    declared = header_functions()
    assert len(declared) >= 16
    assert sorted(B.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True, text=True,
                             check=True).stdout
        exported = set(re.findall(r"\bT (mk_\w+)", out))
        assert set(declared) <= exported


def test_struct_layout_matches_header(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    cfg_fields = [f for f, _ in B.MkCfg._fields_]
    w_fields = [f for f, _ in B.MkWeights._fields_]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "mk.h"', "int main(void) {",
           'printf("cfg %zu\\n", sizeof(mk_cfg));', 'printf("weights %zu\\n", sizeof(mk_weights));']
    src += [f'printf("cfg.{f} %zu\\n", offsetof(mk_cfg, {f}));' for f in cfg_fields]
    src += [f'printf("weights.{f} %zu\\n", offsetof(mk_weights, {f}));' for f in w_fields]
    src += ["return 0;", "}"]
    (tmp_path / "layout.c").write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(tmp_path / "layout.c"), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(got["cfg"]) == ctypes.sizeof(B.MkCfg)
    assert int(got["weights"]) == ctypes.sizeof(B.MkWeights)
    for f in cfg_fields:
        assert int(got[f"cfg.{f}"]) == getattr(B.MkCfg, f).offset, f
    for f in w_fields:
        assert int(got[f"weights.{f}"]) == getattr(B.MkWeights, f).offset, f


def test_error_strings(lib):
    codes = header_codes()
    errs = {k: v for k, v in codes.items() if k.startswith("MK_ERR") or k == "MK_OK"}
    assert errs["MK_OK"] == 0 and len(errs) == 12
    seen = set()
    for name, code in errs.items():
        s = lib.mk_strerror(code).decode()
        assert s and s != "unknown error", name
        seen.add(s)
    assert len(seen) == len(errs)
    assert lib.mk_strerror(12345).decode() == "unknown error"


def _cfg(**kw):
    from persistent_megakernel_loop_amd import workload as wl
    c = B.make_cfg(wl.BY_NAME["talker-0.6b"])
    for k, v in kw.items():
        if k == "sections":
            for i in range(3):
                c.sections[i] = v[i] if i < len(v) else 0
            c.n_sections = len(v)
        else:
            setattr(c, k, v)
    return c


def _fake_weights(n_layers, untied=True):
    """Non-null placeholders: mk_create rejects the cfg before it reads any of them."""
    w = B.MkWeights()
    w.embed, w.final_norm = 0x1000, 0x2000
    w.lm_head = 0x3000 if untied else None
    keep = []
    for name in ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down"):
        arr = (ctypes.c_void_p * n_layers)(*([0x4000] * n_layers))
        keep.append(arr)
        setattr(w, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
    return w, keep


def _create(lib, cfg, w):
    h = ctypes.c_void_p(0xdead)
    rc = lib.mk_create(ctypes.byref(w), ctypes.byref(cfg), None, ctypes.byref(h))
    return rc, h.value


@pytest.mark.parametrize("kw,code", [
    (dict(n_layers=0), -1),
    (dict(hidden=-4), -1),
    (dict(n_q_heads=12, n_kv_heads=8), -1),     # heads not a multiple
    (dict(head_dim=127), -1),                   # odd head_dim
    (dict(weight_dtype=7), -1),
    (dict(kv_dtype=-1), -1),
    (dict(sections=(24, 20, 21)), -1),          # pairs do not sum to head_dim/2
    (dict(sections=(64, 0)), -1),               # empty section
    (dict(rope_theta=0.0), -1),
    (dict(rms_eps=float("nan")), -1),
    (dict(max_seq=0), -1),
    (dict(vocab=1 << 18), -2),                  # argmax keys hold 18-bit indices
    (dict(hidden=1536), -2),                    # no body for this shape
    (dict(kv_dtype=0), -2),                     # bf16 body, f32 cache
])
def test_create_rejects_bad_cfg(lib, kw, code):
    cfg = _cfg(**kw)
    w, keep = _fake_weights(max(cfg.n_layers, 1))
    rc, h = _create(lib, cfg, w)
    assert rc == code
    assert h is None  # *out is cleared on failure


def test_create_rejects_missing_pointers(lib):
    cfg = _cfg()
    w, keep = _fake_weights(cfg.n_layers)
    w.lm_head = None  # untied without a head
    assert _create(lib, cfg, w)[0] == -1
    w, keep = _fake_weights(cfg.n_layers)
    keep[3][5] = None  # wv of layer 5
    assert _create(lib, cfg, w)[0] == -1
    assert lib.mk_create(None, ctypes.byref(cfg), None, ctypes.byref(ctypes.c_void_p())) == -1
    assert lib.mk_create(ctypes.byref(w), None, None, ctypes.byref(ctypes.c_void_p())) == -1
    assert lib.mk_create(ctypes.byref(w), ctypes.byref(cfg), None, None) == -1


def test_null_handle_calls(lib):
    i32, i64 = ctypes.c_int32(), ctypes.c_int64()
    info = (ctypes.c_int32 * 5)()
    assert lib.mk_prefill(None, 0x10, None, None, 4, 0x20) == -1
    assert lib.mk_prefill_batched(None, 0x10, None, None, 4, 0x20) == -1
    assert lib.mk_prefill_batched_noalloc(None, 0x10, None, None, 4, 0x20) == -1
    assert lib.mk_read_ids(None, 0, 1, (ctypes.c_int32 * 1)()) == -1
    assert lib.mk_query(None, ctypes.byref(ctypes.c_int32())) == -1
    assert lib.mk_decode(None, 4, None, None, None, 0x20) == -1
    assert lib.mk_decode_phased(None, 4, None, None, None, 0x20) == -1
    assert lib.mk_load_kv(None, 0x10, 4) == -1
    assert lib.mk_reset(None) == -1
    assert lib.mk_position(None, ctypes.byref(i32)) == -1
    assert lib.mk_set_debug(None, None, None) == -1
    assert lib.mk_set_phase_trace(None, None, 0) == -1
    assert lib.mk_set_spin_limit(None, 1) == -1
    assert lib.mk_progress(None, ctypes.byref(i64)) == -1
    assert lib.mk_status(None) == -1
    assert lib.mk_error_info(None, info) == -1
    assert lib.mk_grid_size(None, ctypes.byref(i32)) == -1
    lib.mk_destroy(None)  # no-op


def test_selftest_and_embed_sum_argument_checks(lib):
    # LDS window is 144 KiB; offsets are 16-byte aligned
    assert lib.mk_selftest_lds_dma(None, 0x10, 1, 0, None) == -1
    assert lib.mk_selftest_lds_dma(0x10, 0x20, 0, 0, None) == -1
    assert lib.mk_selftest_lds_dma(0x10, 0x20, 4, 8, None) == -1
    assert lib.mk_selftest_lds_dma(0x10, 0x20, 9217, 0, None) == -1
    assert lib.mk_selftest_lds_dma(0x10, 0x20, 1, 144 * 1024 - 8, None) == -1
    # exchange stress test: positive rounds, a result array
    assert lib.mk_selftest_exchange(0, 0, 0, (ctypes.c_uint32 * 4)(), None) == -1
    assert lib.mk_selftest_exchange(10, 0, 1, None, None) == -1
    # read-stream measurement kernel: non-null buffers, bytes a positive multiple of 16, 1..65536 blocks
    assert lib.mk_bench_stream_read(None, 1024, 0, 0x10, 64, None) == -1
    assert lib.mk_bench_stream_read(0x10, 1000, 0, 0x20, 64, None) == -1
    assert lib.mk_bench_stream_read(0x10, 1024, 0, 0x20, 0, None) == -1
    assert lib.mk_bench_stream_read(0x10, 1024, 0, None, 64, None) == -1
    # product self-test: rows % 32, k % 64, 1 <= n <= 64, non-null buffers
    assert lib.mk_selftest_gemm(None, 32, 64, 0x10, 1, 0x20, None) == -1
    assert lib.mk_selftest_gemm(0x10, 33, 64, 0x20, 1, 0x30, None) == -1
    assert lib.mk_selftest_gemm(0x10, 32, 96, 0x20, 1, 0x30, None) == -1
    assert lib.mk_selftest_gemm(0x10, 32, 64, 0x20, 0, 0x30, None) == -1
    assert lib.mk_selftest_gemm(0x10, 32, 64, 0x20, 65, 0x30, None) == -1
    # embed_sum: null tables, bad sizes, bad dtype
    args = dict(cb=0x10, ncb=16, cbs=2048, tx=0x20, tv=151936, h=1024, dt=1, ids=0x30, n=4, rows=0x40)

    def call(**kw):
        a = dict(args, **kw)
        return lib.mk_embed_sum(a["cb"], a["ncb"], a["cbs"], a["tx"], a["tv"], a["h"], a["dt"], a["ids"], a["n"],
                                a["rows"], None, None)
    for kw in (dict(cb=None), dict(tx=None), dict(ids=None), dict(rows=None), dict(n=-1), dict(ncb=0),
               dict(cbs=0), dict(tv=0), dict(h=0), dict(dt=2)):
        assert call(**kw) == -1, kw
    assert call(n=0) == 0  # nothing to do, nothing launched
    assert call(n=0, cb=None, tx=None, ids=None, rows=None) == 0


def test_stream_rejects_empty_chunks():
    """Decoder.stream checks its chunk size before it enqueues anything."""
    dec = object.__new__(B.Decoder)
    with pytest.raises(ValueError):
        next(dec.stream(4, chunk=0))
