"""ctypes binding of libmk.so (C ABI in include/mk.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  torch provides device memory (tensors) and the stream handle.  When
the library is missing, every entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmk.so"

MK_F32, MK_BF16 = 0, 1
MK_ERR_OVERRUN = -11
PREFILL_AUTO, PREFILL_CHAIN, PREFILL_PERSISTENT = 0, 1, 2  # mk_set_prefill_path

EXPORTS = ("mk_create", "mk_prefill", "mk_prefill_batched", "mk_prefill_batched_noalloc", "mk_decode", "mk_decode_phased", "mk_load_kv", "mk_reset", "mk_position", "mk_set_debug",
           "mk_set_phase_trace", "mk_set_prefill_path", "mk_set_spin_limit", "mk_progress", "mk_read_ids", "mk_query", "mk_status", "mk_error_info", "mk_selftest_lds_dma", "mk_selftest_gemm", "mk_selftest_exchange", "mk_bench_stream_read", "mk_grid_size",
           "mk_embed_sum", "mk_strerror", "mk_destroy")


def library_path() -> str:
    """The in-tree libmk.so, or the file MK_LIBRARY names (an alternative build of the same ABI)."""
    return os.environ.get("MK_LIBRARY") or os.path.join(_PKG, _LIB_NAME)


class MkError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {code} ({_strerror(code)})")


class MkCfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied", ctypes.c_int32), ("weight_dtype", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("n_sections", ctypes.c_int32), ("sections", ctypes.c_int32 * 3), ("max_seq", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class MkWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p)] + [
        (n, _PP) for n in ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up",
                           "w_down")]


_lib = None


def lib():
    """Load libmk.so once; raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m persistent_megakernel_loop_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, pi32 = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    L.mk_create.argtypes = [ctypes.POINTER(MkWeights), ctypes.POINTER(MkCfg), vp, ctypes.POINTER(vp)]
    L.mk_prefill.argtypes = [vp, vp, vp, vp, i32, vp]
    L.mk_prefill_batched.argtypes = [vp, vp, vp, vp, i32, vp]
    L.mk_prefill_batched_noalloc.argtypes = [vp, vp, vp, vp, i32, vp]
    L.mk_decode.argtypes = [vp, i32, vp, vp, vp, vp]
    L.mk_decode_phased.argtypes = [vp, i32, vp, vp, vp, vp]
    L.mk_load_kv.argtypes = [vp, vp, i32]
    L.mk_reset.argtypes = [vp]
    L.mk_position.argtypes = [vp, pi32]
    L.mk_set_debug.argtypes = [vp, vp, vp]
    L.mk_set_phase_trace.argtypes = [vp, vp, i32]
    L.mk_set_spin_limit.argtypes = [vp, ctypes.c_uint32]
    L.mk_set_prefill_path.argtypes = [vp, i32]
    L.mk_progress.argtypes = [vp, ctypes.POINTER(ctypes.c_int64)]
    L.mk_read_ids.argtypes = [vp, i32, i32, pi32]
    L.mk_query.argtypes = [vp, pi32]
    L.mk_status.argtypes = [vp]
    L.mk_error_info.argtypes = [vp, pi32]
    L.mk_selftest_lds_dma.argtypes = [vp, vp, i32, i32, vp]
    L.mk_selftest_gemm.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    L.mk_selftest_exchange.argtypes = [i32, ctypes.c_uint32, i32, ctypes.POINTER(ctypes.c_uint32), vp]
    L.mk_bench_stream_read.argtypes = [vp, ctypes.c_uint64, i32, vp, i32, vp]
    L.mk_grid_size.argtypes = [vp, pi32]
    L.mk_embed_sum.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp, i32, vp, vp, vp]
    L.mk_strerror.argtypes = [ctypes.c_int]
    L.mk_strerror.restype = ctypes.c_char_p
    L.mk_destroy.argtypes = [vp]
    L.mk_destroy.restype = None
    for n in EXPORTS:
        if n not in ("mk_strerror", "mk_destroy"):
            getattr(L, n).restype = ctypes.c_int
    _lib = L
    return L


def _strerror(code: int) -> str:
    try:
        return lib().mk_strerror(code).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(code: int, what: str):
    if code != 0:
        raise MkError(code, what)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def to_device(a: np.ndarray, device="cuda"):
    """numpy array (uint16 bf16 bits or float32) -> torch tensor on the device, same bytes."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def weights_to_device(weights: Dict[str, object], device="cuda") -> Dict[str, object]:
    out = {k: to_device(v, device) for k, v in weights.items() if k != "layers"}
    out["layers"] = [{k: to_device(v, device) for k, v in lw.items()} for lw in weights["layers"]]
    return out


def make_cfg(shape) -> MkCfg:
    c = MkCfg()
    c.n_layers, c.hidden, c.n_q_heads, c.n_kv_heads = shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads
    c.head_dim, c.intermediate, c.vocab = shape.head_dim, shape.intermediate, shape.vocab
    c.tied = 1 if shape.tied else 0
    c.weight_dtype = MK_BF16 if shape.weight_dtype == "bf16" else MK_F32
    c.kv_dtype = MK_BF16 if shape.kv_dtype == "bf16" else MK_F32
    c.rms_eps, c.rope_theta = shape.rms_eps, shape.rope_theta
    c.n_sections = len(shape.sections)
    for k in range(3):
        c.sections[k] = shape.sections[k] if k < len(shape.sections) else 0
    c.max_seq = shape.capacity
    return c


class Decoder:
    """One mk_handle: weights in the library arena, KV cache, position."""

    def __init__(self, shape, dev_weights: Dict[str, object], stream=None, cfg: Optional[MkCfg] = None):
        L = lib()
        self.shape = shape
        self._stream = _stream_handle(stream)
        self.cfg = cfg if cfg is not None else make_cfg(shape)
        nl = self.cfg.n_layers
        w = MkWeights()
        w.embed = _ptr(dev_weights["embed"])
        w.lm_head = _ptr(dev_weights.get("lm_head"))
        w.final_norm = _ptr(dev_weights["final_norm"])
        self._arrays = []
        for n in ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo", "post_norm", "w_gate", "w_up", "w_down"):
            arr = (ctypes.c_void_p * nl)(*[_ptr(dev_weights["layers"][l][n]) for l in range(nl)])
            self._arrays.append(arr)
            setattr(w, n, ctypes.cast(arr, _PP))
        h = ctypes.c_void_p()
        _check(L.mk_create(ctypes.byref(w), ctypes.byref(self.cfg), self._stream, ctypes.byref(h)), "mk_create")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("decoder destroyed")
        return self._h

    def prefill(self, ids, rows=None, pos3=None, out=None, batched: bool = False):
        """Run the prompt; batched=True takes mk_prefill_batched (the whole prompt as a
        batch through per-layer kernels, then the first id's LM head) instead of the
        persistent kernel position by position."""
        n = ids.numel()
        if out is None:
            out = self._empty(1, ids.device)
        fn, name = (lib().mk_prefill_batched, "mk_prefill_batched") if batched else (lib().mk_prefill, "mk_prefill")
        _check(fn(self.handle, _ptr(ids), _ptr(rows), _ptr(pos3), n, _ptr(out)), name)
        return out

    def prefill_batched_noalloc(self, ids, out, rows=None, pos3=None):
        """mk_prefill_batched_noalloc: the batched prefill in the library's fixed scratch
        array; the caller passes the output (a device int32 tensor of at least one
        element), so the call allocates nothing."""
        _check(lib().mk_prefill_batched_noalloc(self.handle, _ptr(ids), _ptr(rows), _ptr(pos3), ids.numel(),
                                                _ptr(out)), "mk_prefill_batched_noalloc")
        return out

    def _empty(self, n: int, device):
        """An int32 device tensor the kernel writes on the handle's stream: allocated from
        torch's cache on that stream, so its block is not handed out again before the
        stream has passed the launch that writes it."""
        import torch
        dev = torch.device(device)
        cur = torch.cuda.current_stream(dev)
        if self._stream in (None, 0, cur.cuda_stream):
            return torch.empty(n, dtype=torch.int32, device=dev)
        with torch.cuda.stream(torch.cuda.ExternalStream(self._stream, device=dev)):
            return torch.empty(n, dtype=torch.int32, device=dev)

    def decode(self, n_steps: int, ids=None, rows=None, pos3=None, out=None, device="cuda"):
        if out is None:
            out = self._empty(n_steps, device if ids is None else ids.device)
        _check(lib().mk_decode(self.handle, n_steps, _ptr(ids), _ptr(rows), _ptr(pos3), _ptr(out)), "mk_decode")
        return out

    def decode_phased(self, n_steps: int, ids=None, rows=None, pos3=None, out=None, device="cuda"):
        """mk_decode_phased: decode's computation, one kernel launch per phase (measurement)."""
        if out is None:
            out = self._empty(n_steps, device if ids is None else ids.device)
        _check(lib().mk_decode_phased(self.handle, n_steps, _ptr(ids), _ptr(rows), _ptr(pos3), _ptr(out)),
               "mk_decode_phased")
        return out

    def load_kv(self, kv, n_pos: int):
        _check(lib().mk_load_kv(self.handle, _ptr(kv), n_pos), "mk_load_kv")

    def reset(self):
        _check(lib().mk_reset(self.handle), "mk_reset")

    @property
    def position(self) -> int:
        p = ctypes.c_int32()
        _check(lib().mk_position(self.handle, ctypes.byref(p)), "mk_position")
        return p.value

    def set_debug(self, hidden=None, trace=None):
        _check(lib().mk_set_debug(self.handle, _ptr(hidden), _ptr(trace)), "mk_set_debug")

    def set_phase_trace(self, phase=None, wg: int = 0):
        _check(lib().mk_set_phase_trace(self.handle, _ptr(phase), wg), "mk_set_phase_trace")

    def set_spin_limit(self, polls: int = 0):
        _check(lib().mk_set_spin_limit(self.handle, polls), "mk_set_spin_limit")

    def set_prefill_path(self, path: int = 0):
        """PREFILL_AUTO, PREFILL_CHAIN or PREFILL_PERSISTENT (mk_set_prefill_path)."""
        _check(lib().mk_set_prefill_path(self.handle, path), "mk_set_prefill_path")

    def progress(self) -> int:
        v = ctypes.c_int64()
        _check(lib().mk_progress(self.handle, ctypes.byref(v)), "mk_progress")
        return v.value

    def read_ids(self, first: int, count: int) -> np.ndarray:
        """Ids [first, first + count) of the last call, from the pinned mirror (no sync)."""
        buf = (ctypes.c_int32 * max(count, 1))()
        _check(lib().mk_read_ids(self.handle, first, count, buf), "mk_read_ids")
        return np.frombuffer(buf, dtype=np.int32, count=count).copy()

    def idle(self) -> bool:
        v = ctypes.c_int32()
        _check(lib().mk_query(self.handle, ctypes.byref(v)), "mk_query")
        return bool(v.value)

    def stream(self, n_steps: int, ids=None, rows=None, pos3=None, chunk: int = 4, out=None):
        """Enqueue one decode launch of n_steps steps and yield its ids as numpy chunks of
        `chunk` (the last may be shorter) while the kernel runs, read from the pinned id
        ring as the progress word advances.  A reader that falls more than the ring's
        4096 ids behind gets the rest from the launch's device output once it ends.
        Raises MkError if the launch ends early with a device error."""
        if chunk < 1:
            raise ValueError("chunk must be at least 1")
        # the launch writes its ids into `out` until it ends: the tensor stays referenced
        # here for the generator's whole life
        out = self.decode(n_steps, ids, rows, pos3, out=out)
        done = 0
        while done < n_steps:
            p = self.progress()
            if p - done >= chunk or p == n_steps or (p > done and self.idle()):
                try:
                    got = self.read_ids(done, p - done)
                except MkError as e:
                    if e.code != MK_ERR_OVERRUN:
                        raise
                    break
                yield got
                done = p
            elif self.idle() and self.progress() == done:
                self.check()
                raise RuntimeError(f"decode ended after {done} of {n_steps} ids")
        if done < n_steps:  # overrun: the rest from the device output
            import torch
            torch.cuda.synchronize(out.device)
            rest = out[done:].cpu().numpy()
            for k in range(0, len(rest), chunk):
                yield rest[k:k + chunk]
        self.check()

    def status(self) -> int:
        return lib().mk_status(self.handle)

    def check(self):
        code = self.status()
        if code != 0:
            info = (ctypes.c_int32 * 5)()
            lib().mk_error_info(self.handle, info)
            raise MkError(code, f"device status (first timeout: recorded={info[0]} wg={info[1]} tag={info[2]} "
                                f"word={info[3]} seen={info[4]})")

    def grid_size(self) -> int:
        n = ctypes.c_int32()
        _check(lib().mk_grid_size(self.handle, ctypes.byref(n)), "mk_grid_size")
        return n.value

    def close(self):
        if getattr(self, "_h", None) is not None:
            lib().mk_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def selftest_lds_dma(src, dst, offset_bytes: int = 0, stream=None):
    """Copy src -> LDS (at offset_bytes) -> dst through the kernel's LDS DMA path (both int32/uint8 device tensors)."""
    n = src.numel() * src.element_size() // 16
    _check(lib().mk_selftest_lds_dma(_ptr(src), _ptr(dst), n, offset_bytes, _stream_handle(stream)), "mk_selftest_lds_dma")


def selftest_gemm(w, x, y=None, stream=None):
    """y[t][r] = sum_k w[r][k] x[t][k] through the batched prefill's product kernels
    (w: [rows][k] bf16 device tensor, x: [n][k] float32 device tensor)."""
    import torch
    rows, k = w.shape
    n = x.shape[0]
    if y is None:
        y = torch.empty((n, rows), dtype=torch.float32, device=x.device)
    _check(lib().mk_selftest_gemm(_ptr(w), rows, k, _ptr(x), n, _ptr(y), _stream_handle(stream)), "mk_selftest_gemm")
    return y


def selftest_exchange(iters: int, spin_limit: int = 0, xcd_local: bool = False, stream=None):
    """Stress test of the exchange protocol: (mismatched words, workgroups that gave up,
    device error word, 1 if XCD-local plain stores were used)."""
    res = (ctypes.c_uint32 * 4)()
    _check(lib().mk_selftest_exchange(iters, spin_limit, int(xcd_local), res, _stream_handle(stream)),
           "mk_selftest_exchange")
    return tuple(int(v) for v in res)


def bench_stream_read(src, nontemporal: bool = False, sink=None, blocks: int = 2048, stream=None):
    """Enqueue one streaming read of the whole device tensor src (measurement kernel)."""
    import torch
    if sink is None:
        sink = torch.zeros(blocks, dtype=torch.int64, device=src.device)
    n = src.numel() * src.element_size() // 16 * 16
    _check(lib().mk_bench_stream_read(_ptr(src), n, int(nontemporal), _ptr(sink), blocks, _stream_handle(stream)),
           "mk_bench_stream_read")
    return sink


def embed_sum(codebooks, text, ids, rows=None, bad=None, stream=None):
    """rows[t] = sum of codebooks[c][ids[t][c]] (c in order) + text[ids[t][-1]], float32, on the device."""
    import torch
    n_cb, cb_size, hidden = codebooks.shape
    n = ids.shape[0]
    dtype = MK_BF16 if codebooks.dtype in (torch.int16, torch.bfloat16) else MK_F32
    if rows is None:
        rows = torch.empty((n, hidden), dtype=torch.float32, device=ids.device)
    _check(lib().mk_embed_sum(_ptr(codebooks), n_cb, cb_size, _ptr(text), text.shape[0], hidden, dtype, _ptr(ids), n,
                              _ptr(rows), _ptr(bad), _stream_handle(stream)), "mk_embed_sum")
    return rows
