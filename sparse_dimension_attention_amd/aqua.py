"""ctypes binding of libaqua (include/aqua.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are passed as raw device
pointers (``tensor.data_ptr()``); shapes are read from the tensors only to fill in the sizes the C
call asks for; the stream is torch's current HIP stream unless one is given.  A non-OK status
raises :class:`AquaError` with the library's message.  There is no fallback: if libaqua.so is
not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libaqua.so")

AQUA_OK, AQUA_ERR_NULL, AQUA_ERR_SHAPE, AQUA_ERR_DTYPE = 0, 1, 2, 3
AQUA_ERR_CAPACITY, AQUA_ERR_ALIGN, AQUA_ERR_WORKSPACE, AQUA_ERR_HIP = 4, 5, 6, 7
AQUA_F32, AQUA_BF16 = 0, 1

_STATUS_NAMES = {0: "AQUA_OK", 1: "AQUA_ERR_NULL", 2: "AQUA_ERR_SHAPE", 3: "AQUA_ERR_DTYPE",
                 4: "AQUA_ERR_CAPACITY", 5: "AQUA_ERR_ALIGN", 6: "AQUA_ERR_WORKSPACE",
                 7: "AQUA_ERR_HIP"}

EXPORTS = ("aqua_version", "aqua_last_error", "aqua_project_keys", "aqua_select_dims",
           "aqua_decode_workspace", "aqua_decode", "aqua_decode_step", "aqua_decode_step_noalloc",
           "aqua_prefill_workspace",
           "aqua_prefill_chunk", "aqua_h2o_init", "aqua_h2o_victim", "aqua_h2o_step",
           "aqua_gram_workspace", "aqua_gram", "aqua_stream_read_probe")


class AquaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class aqua_cache(ctypes.Structure):
    _fields_ = [("kp", ctypes.c_void_p), ("v", ctypes.c_void_p), ("B", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d_head", ctypes.c_int32), ("d_store", ctypes.c_int32),
                ("T_cap", ctypes.c_int32), ("len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libaqua.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cp = ctypes.POINTER(aqua_cache)
    sig = {
        "aqua_version": ([], ctypes.c_char_p),
        "aqua_last_error": ([], ctypes.c_char_p),
        "aqua_project_keys": ([cp, P, P, P, I32, P, P], ctypes.c_int),
        "aqua_select_dims": ([P, I32, I32, I32, P, I32, I32, P, P, P, P], ctypes.c_int),
        "aqua_decode_workspace": ([cp, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "aqua_decode": ([cp, I32, P, P, ctypes.c_float, P, P, P, SZ, P], ctypes.c_int),
        "aqua_decode_step": ([cp, I32, P, P, P, P, I32, I32, ctypes.c_float, P, P, P, P, P, SZ,
                              P], ctypes.c_int),
        "aqua_decode_step_noalloc": ([cp, I32, P, P, P, P, I32, I32, ctypes.c_float, P, P, P, P,
                                      P], ctypes.c_int),
        "aqua_prefill_workspace": ([cp, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "aqua_prefill_chunk": ([cp, I32, P, I32, I32, P, I32, I32, ctypes.c_float, P, P, P, P,
                                SZ, P], ctypes.c_int),
        "aqua_h2o_init": ([cp, P, I32, I32, cp, P, P, P], ctypes.c_int),
        "aqua_h2o_victim": ([P, P, I32, I32, I32, I32, I32, P, P], ctypes.c_int),
        "aqua_stream_read_probe": ([P, SZ, I32, P, P], ctypes.c_int),
        "aqua_gram_workspace": ([I32, ctypes.c_int64, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "aqua_gram": ([I32, P, ctypes.c_int64, I32, P, P, SZ, P], ctypes.c_int),
        "aqua_h2o_step": ([cp, I32, P, P, P, P, I32, I32, ctypes.c_float, P, P, I32, I32, P, P, P,
                           P, P, SZ, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int):
    if status != AQUA_OK:
        raise AquaError(status, load_library().aqua_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        if torch.cuda.is_available():
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        return None
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return AQUA_F32
    if dt == torch.bfloat16:
        return AQUA_BF16
    raise AquaError(AQUA_ERR_DTYPE, f"unsupported dtype {dt}")


def make_cache(kp: torch.Tensor, v: torch.Tensor, length: int = 0) -> aqua_cache:
    """Descriptor of a cache held in kp [B][Hkv][d_store][T_cap] and v [B][Hkv][T_cap][d]."""
    B, Hkv, d_store, T_cap = kp.shape
    return aqua_cache(kp.data_ptr(), v.data_ptr(), B, Hkv, v.shape[-1], d_store, T_cap,
                      int(length), dtype_code(kp.dtype))


def aqua_version() -> str:
    return load_library().aqua_version().decode()


def aqua_last_error() -> str:
    return load_library().aqua_last_error().decode()


def aqua_project_keys(cache: aqua_cache, k_raw, v_raw, P, n: int, slots=None, stream=None):
    _check(load_library().aqua_project_keys(ctypes.byref(cache), _ptr(k_raw), _ptr(v_raw),
                                            _ptr(P), int(n), _ptr(slots), _stream(stream)))


def aqua_select_dims(q, P, d_sel: int, k: int, q_proj, mask, idx=None, stream=None):
    N, d = (q.shape[0], q.shape[1]) if q.dim() == 2 else (q.numel() // q.shape[-1], q.shape[-1])
    _check(load_library().aqua_select_dims(_ptr(q), dtype_code(q.dtype), int(N), int(d), _ptr(P),
                                           int(d_sel), int(k), _ptr(q_proj), _ptr(mask),
                                           _ptr(idx), _stream(stream)))


def aqua_decode_workspace(cache: aqua_cache, Hq: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().aqua_decode_workspace(ctypes.byref(cache), int(Hq), ctypes.byref(n)))
    return n.value


def aqua_decode(cache: aqua_cache, Hq: int, q_proj, mask, scale: float, out, ws, mass=None,
                stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().aqua_decode(ctypes.byref(cache), int(Hq), _ptr(q_proj), _ptr(mask),
                                      float(scale), _ptr(mass), _ptr(out), _ptr(ws), nbytes,
                                      _stream(stream)))


def aqua_decode_step(cache: aqua_cache, Hq: int, q, k_new, v_new, P, d_sel: int, k: int,
                     scale: float, out, ws, mass=None, q_proj_out=None, mask_out=None,
                     stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().aqua_decode_step(ctypes.byref(cache), int(Hq), _ptr(q), _ptr(k_new),
                                           _ptr(v_new), _ptr(P), int(d_sel), int(k),
                                           float(scale), _ptr(mass), _ptr(out),
                                           _ptr(q_proj_out), _ptr(mask_out), _ptr(ws), nbytes,
                                           _stream(stream)))


def aqua_decode_step_noalloc(cache: aqua_cache, Hq: int, q, k_new, v_new, P, d_sel: int, k: int,
                             scale: float, out, mass=None, q_proj_out=None, mask_out=None,
                             stream=None):
    _check(load_library().aqua_decode_step_noalloc(
        ctypes.byref(cache), int(Hq), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(P), int(d_sel),
        int(k), float(scale), _ptr(mass), _ptr(out), _ptr(q_proj_out), _ptr(mask_out),
        _stream(stream)))


def aqua_prefill_workspace(cache: aqua_cache, Hq: int, Lq: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().aqua_prefill_workspace(ctypes.byref(cache), int(Hq), int(Lq),
                                                 ctypes.byref(n)))
    return n.value


def aqua_prefill_chunk(cache: aqua_cache, Hq: int, q, Lq: int, pos0: int, P, d_sel: int, k: int,
                       scale: float, out, ws=None, q_proj_out=None, mask_out=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().aqua_prefill_chunk(ctypes.byref(cache), int(Hq), _ptr(q), int(Lq),
                                             int(pos0), _ptr(P), int(d_sel), int(k), float(scale),
                                             _ptr(out), _ptr(q_proj_out), _ptr(mask_out),
                                             _ptr(ws), nbytes, _stream(stream)))


def aqua_h2o_init(full: aqua_cache, mass_full, heavy: int, recent: int, compact: aqua_cache,
                  mass, slot_pos, stream=None):
    _check(load_library().aqua_h2o_init(ctypes.byref(full), _ptr(mass_full), int(heavy),
                                        int(recent), ctypes.byref(compact), _ptr(mass),
                                        _ptr(slot_pos), _stream(stream)))


def aqua_h2o_victim(mass, slot_pos, t_new: int, recent: int, victim, stream=None):
    B, Hkv, n_slots = mass.shape
    _check(load_library().aqua_h2o_victim(_ptr(mass), _ptr(slot_pos), int(B), int(Hkv),
                                          int(n_slots), int(t_new), int(recent), _ptr(victim),
                                          _stream(stream)))


def aqua_h2o_step(cache: aqua_cache, Hq: int, q, k_new, v_new, P, d_sel: int, k: int,
                  scale: float, mass, slot_pos, t_new: int, recent: int, victim, out, ws,
                  q_proj_out=None, mask_out=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().aqua_h2o_step(ctypes.byref(cache), int(Hq), _ptr(q), _ptr(k_new),
                                        _ptr(v_new), _ptr(P), int(d_sel), int(k), float(scale),
                                        _ptr(mass), _ptr(slot_pos), int(t_new), int(recent),
                                        _ptr(victim), _ptr(out), _ptr(q_proj_out),
                                        _ptr(mask_out), _ptr(ws), nbytes, _stream(stream)))


def aqua_gram_workspace(dtype: int, n: int, d: int) -> int:
    """Bytes of workspace aqua_gram needs for n calibration vectors of d dims."""
    nb = ctypes.c_size_t()
    _check(load_library().aqua_gram_workspace(int(dtype), int(n), int(d), ctypes.byref(nb)))
    return nb.value


def aqua_gram(x, gram, ws, stream=None):
    """gram [d][d] (float64, device) = x^T x for calibration vectors x [n][d] (bf16 or fp32)."""
    n, d = x.shape
    _check(load_library().aqua_gram(dtype_code(x.dtype), _ptr(x), int(n), int(d), _ptr(gram),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def aqua_stream_read_probe(buf, blocks: int, sink, stream=None):
    """One streaming read of the whole tensor buf (a diagnostic for the measured bandwidth)."""
    _check(load_library().aqua_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(),
                                                 int(blocks), _ptr(sink), _stream(stream)))
