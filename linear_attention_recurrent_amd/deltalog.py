"""Python binding of libdeltalog.so: argument marshalling only.

The calls have the C names and meanings declared in include/deltalog.h
(dl_init_state, dl_decode_step, dl_merge, dl_eager_step, dl_prefill).  PyTorch supplies
device memory and the stream; every step of the decode path runs in the HIP
kernels of libdeltalog.so.  There is no CPU fallback: if the library is not
built, or no GPU is present, these calls raise.

One GDN layer, 4 sequences x 8 heads, dk = dv = 128, log length 16:

    import torch
    from linear_attention_recurrent_amd import deltalog as dl

    dev = torch.device("cuda", 0)
    pool = dl.DeltaLogPool(dl.GDN, 4, 8, 128, 128, 16, dev)  # fp32 base; BASE_BF16 for bf16
    dl.dl_init_state(pool)                                   # zero state, empty logs
    out = torch.empty(4, 8, 128, device=dev)
    for q, k, v, alpha, beta in tokens:                      # bf16 [4, 8, 128]; fp32 [4, 8]
        dl.dl_decode_step(pool, pool.step_io(q, k, v, alpha, beta, None, out))
        ...                                                  # out holds this token's outputs
    dl.dl_merge(pool, dl.MERGE_ALL)                          # pool.base: the dense states

A StepIO holds raw device pointers: the tensors it was made from must stay alive
(and unchanged in shape) until the work enqueued with it has run.  Calls enqueue
on torch's current stream of the pool's device unless a stream is passed.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # imported first so the library binds to the HIP runtime torch already loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdeltalog.so")

GDN, KDA, RWKV6 = 0, 1, 2
DL_OK, DL_EINVAL, DL_EUNSUPPORTED, DL_EALIGN, DL_EHIP = 0, -1, -2, -3, -4
BASE_F32, BASE_BF16 = 0, 1
UNIT_AUTO, UNIT_VALU, UNIT_MFMA = 0, 1, 2  # arithmetic unit of a fold (dl_merge_on)
MERGE_DUE, MERGE_ALL = 0, 1                 # the named values of dl_merge's min_fill
MAX_LOG_LEN = 128


class Dims(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("log_len", ctypes.c_int32),
                ("base_dtype", ctypes.c_int32)]


class Pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("log_k", ctypes.c_void_p), ("log_u", ctypes.c_void_p),
                ("log_c", ctypes.c_void_p), ("fill", ctypes.c_void_p)]


class StepIO(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("decay", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("bonus", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("eta", ctypes.c_void_p), ("eps", ctypes.c_float)]


class PrefillIO(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("decay", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("bonus", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("eta", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("tokens", ctypes.c_int32)]


class DeltaLogError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load_library(path: Optional[str] = None, make_default: bool = False) -> ctypes.CDLL:
    """Load libdeltalog.so (once) and declare its signatures.  A `path` loads that build
    of the library instead (the tracing build, say); with make_default it serves every
    later call of this module."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run `python -m linear_attention_recurrent_amd.build`")
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    lib.dl_init_state.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Pool), vp,
                                  ctypes.POINTER(ctypes.c_int32), vp]
    lib.dl_decode_step.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Pool), ctypes.POINTER(StepIO), vp]
    lib.dl_merge.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Pool), ctypes.c_int32, vp]
    lib.dl_merge_on.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Pool), ctypes.c_int32, ctypes.c_int32, vp]
    lib.dl_merge_unit.argtypes = [ctypes.POINTER(Dims)]
    lib.dl_eager_step.argtypes = [ctypes.POINTER(Dims), vp, ctypes.POINTER(StepIO), vp]
    lib.dl_prefill.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Pool), ctypes.POINTER(PrefillIO), vp]
    lib.dl_status_string.argtypes = [ctypes.c_int]
    lib.dl_status_string.restype = ctypes.c_char_p
    for f in (lib.dl_init_state, lib.dl_decode_step, lib.dl_merge, lib.dl_merge_on, lib.dl_merge_unit,
              lib.dl_eager_step, lib.dl_prefill):
        f.restype = ctypes.c_int
    if path is None or make_default:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().dl_status_string(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != DL_OK:
        raise DeltaLogError(rc, what)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device=None) -> int:
    """The hipStream_t to enqueue on: `stream` (a torch stream or a raw handle), else the
    current stream of `device` (read without building a torch Stream object, which
    costs microseconds per call on the step path)."""
    if stream is None:
        if _raw_stream is not None and device is not None:
            return _raw_stream(device.index)
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype, device) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape}, "
                         f"got {t.dtype} {tuple(t.shape)}")


class DeltaLogPool:
    """One layer's state pool: the device tensors of dl_pool plus its dims.

    base  fp32 (base_dtype BASE_F32) or bf16 (BASE_BF16) [B][H][dk][dv]; log_k bf16 [B][H][L][dk];
    log_u fp32 (GDN/KDA) or bf16 (RWKV6) [B][H][L][dv];
    log_c fp32 [B][H][L][1 or dk]; fill int32 [B][H].
    """

    def __init__(self, variant: int, batch: int, heads: int, dk: int, dv: int, log_len: int,
                 device="cuda", base_dtype: int = BASE_F32):
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.variant, self.batch, self.heads = int(variant), int(batch), int(heads)
        self.dk, self.dv, self.log_len = int(dk), int(dv), int(log_len)
        B, H, L = self.batch, self.heads, self.log_len
        g = 1 if variant == GDN else dk
        kw = dict(device=self.device)
        self.base_dtype = int(base_dtype)
        self.base = torch.empty((B, H, dk, dv), dtype=torch.bfloat16 if self.base_dtype == BASE_BF16
                                else torch.float32, **kw)
        self.log_k = torch.empty((B, H, L, dk), dtype=torch.bfloat16, **kw)
        self.log_u = torch.empty((B, H, L, dv), dtype=torch.bfloat16 if variant == RWKV6 else torch.float32,
                                 **kw)
        self.log_c = torch.empty((B, H, L, g), dtype=torch.float32, **kw)
        # zeros: a pool used before dl_init_state holds empty logs, never stray fills
        self.fill = torch.zeros((B, H), dtype=torch.int32, **kw)
        self.c_dims = Dims(self.variant, B, H, self.dk, self.dv, L, self.base_dtype)
        self.c_pool = Pool(self.base.data_ptr(), self.log_k.data_ptr(), self.log_u.data_ptr(),
                           self.log_c.data_ptr(), self.fill.data_ptr())
        # by-reference arguments built once: the decode step is called every token
        self.dims_ref = ctypes.byref(self.c_dims)
        self.pool_ref = ctypes.byref(self.c_pool)

    def tensors(self) -> dict:
        return dict(base=self.base, log_k=self.log_k, log_u=self.log_u, log_c=self.log_c, fill=self.fill)

    def clone(self) -> "DeltaLogPool":
        other = DeltaLogPool(self.variant, self.batch, self.heads, self.dk, self.dv, self.log_len, self.device,
                             self.base_dtype)
        for name, t in self.tensors().items():
            getattr(other, name).copy_(t)
        return other

    def step_io(self, q, k, v, decay, beta, bonus, out, eta=None, eps=0.0) -> StepIO:
        """Check the step tensors against this pool's shape and pack them into a StepIO."""
        return make_step_io(self.variant, self.batch, self.heads, self.dk, self.dv, self.device,
                            q, k, v, decay, beta, bonus, out, eta, eps)


def make_step_io(variant, batch, heads, dk, dv, device, q, k, v, decay, beta, bonus, out,
                 eta=None, eps=0.0) -> StepIO:
    """Pack one step's tensors.  GDN/KDA take either beta (the given step size) or eta
    (the Kaczmarz step size beta = eta / (||k||^2 + eps), computed in the kernel)."""
    B, H = batch, heads
    _need(q, "q", (B, H, dk), torch.bfloat16, device)
    _need(k, "k", (B, H, dk), torch.bfloat16, device)
    _need(v, "v", (B, H, dv), torch.bfloat16, device)
    _need(decay, "decay", (B, H) if variant == GDN else (B, H, dk), torch.float32, device)
    if variant == RWKV6:
        _need(bonus, "bonus", (H, dk), torch.float32, device)
        if beta is not None or eta is not None:
            raise ValueError("beta and eta must be None for RWKV6")
    else:
        if (beta is None) == (eta is None):
            raise ValueError("GDN/KDA take exactly one of beta and eta")
        _need(beta if eta is None else eta, "beta" if eta is None else "eta", (B, H), torch.float32, device)
        if bonus is not None:
            raise ValueError("bonus must be None for GDN/KDA")
    _need(out, "out", (B, H, dv), torch.float32, device)
    return StepIO(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta), _ptr(bonus), _ptr(out), _ptr(eta),
                  float(eps))


# ------------------------------------------------------------- the C calls --
def dl_init_state(pool: DeltaLogPool, init_base: Optional[torch.Tensor] = None,
                  init_fill=None, stream=None) -> None:
    """Start the pool from `init_base` (or zeros) with per-sequence log fills `init_fill`."""
    if init_base is not None:
        _need(init_base, "init_base", tuple(pool.base.shape), torch.float32, pool.device)  # always fp32
    fill_arr = None
    if init_fill is not None:
        vals = [int(x) for x in init_fill]
        if len(vals) != pool.batch:
            raise ValueError(f"init_fill must have {pool.batch} entries")
        fill_arr = (ctypes.c_int32 * max(len(vals), 1))(*vals)
    rc = load_library().dl_init_state(ctypes.byref(pool.c_dims), ctypes.byref(pool.c_pool),
                                      _ptr(init_base), fill_arr, _stream(stream))
    _check(rc, "dl_init_state")


def dl_decode_step(pool: DeltaLogPool, io: StepIO, stream=None) -> None:
    """One decode step (append, or fold on the step that fills the log) for every tile."""
    lib = _lib if _lib is not None else load_library()
    rc = lib.dl_decode_step(pool.dims_ref, pool.pool_ref, ctypes.byref(io), _stream(stream, pool.device))
    if rc != DL_OK:
        raise DeltaLogError(rc, "dl_decode_step")


def dl_merge(pool: DeltaLogPool, min_fill: int = 1, stream=None) -> None:
    """Fold the log of every tile holding >= min_fill entries into its base."""
    rc = load_library().dl_merge(ctypes.byref(pool.c_dims), ctypes.byref(pool.c_pool), int(min_fill),
                                 _stream(stream))
    _check(rc, "dl_merge")


def dl_merge_on(pool: DeltaLogPool, min_fill: int = 1, unit: int = 0, stream=None) -> None:
    """dl_merge with the fold's arithmetic unit given (DL_UNIT_AUTO, DL_UNIT_VALU, DL_UNIT_MFMA)."""
    rc = load_library().dl_merge_on(ctypes.byref(pool.c_dims), ctypes.byref(pool.c_pool), int(min_fill),
                                    int(unit), _stream(stream))
    _check(rc, "dl_merge_on")


def dl_merge_unit(dims: Dims) -> int:
    """The unit dl_merge folds with for pools of these dims (UNIT_VALU or UNIT_MFMA)."""
    rc = load_library().dl_merge_unit(ctypes.byref(dims))
    if rc < 0:
        raise DeltaLogError(rc, "dl_merge_unit")
    return rc


def dl_eager_step(variant: int, state: torch.Tensor, io: StepIO, stream=None) -> None:
    """Eager comparator: read `state` [B][H][dk][dv], update it in place, write io.out."""
    if state.dtype != torch.float32 or state.dim() != 4 or not state.is_contiguous() or not state.is_cuda:
        raise ValueError("state must be a contiguous fp32 cuda tensor [B][H][dk][dv]")
    B, H, dk, dv = state.shape
    dims = Dims(int(variant), B, H, dk, dv, 1, BASE_F32)
    rc = load_library().dl_eager_step(ctypes.byref(dims), state.data_ptr(), ctypes.byref(io), _stream(stream))
    _check(rc, "dl_eager_step")


def make_prefill_io(pool: DeltaLogPool, q, k, v, decay, beta, out, eta=None, eps=0.0, bonus=None) -> PrefillIO:
    """Check a prompt's tensors ([batch][T][heads][...], see dl_prefill_io) against the pool."""
    B, H, dk, dv = pool.batch, pool.heads, pool.dk, pool.dv
    if k is None or k.dim() != 4:
        raise ValueError("k must be a [batch][T][heads][dk] tensor")
    T = int(k.shape[1])
    dev = pool.device
    _need(q, "q", (B, T, H, dk), torch.bfloat16, dev)
    _need(k, "k", (B, T, H, dk), torch.bfloat16, dev)
    _need(v, "v", (B, T, H, dv), torch.bfloat16, dev)
    _need(decay, "decay", (B, T, H) if pool.variant == GDN else (B, T, H, dk), torch.float32, dev)
    if pool.variant == RWKV6:
        _need(bonus, "bonus", (H, dk), torch.float32, dev)
        if beta is not None or eta is not None:
            raise ValueError("beta and eta must be None for RWKV6")
    else:
        if (beta is None) == (eta is None):
            raise ValueError("give exactly one of beta and eta")
        _need(beta if eta is None else eta, "beta" if eta is None else "eta", (B, T, H), torch.float32, dev)
        if bonus is not None:
            raise ValueError("bonus must be None for GDN/KDA")
    _need(out, "out", (B, T, H, dv), torch.float32, dev)
    return PrefillIO(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(beta), _ptr(bonus), _ptr(out), _ptr(eta),
                     float(eps), T)


def dl_prefill(pool: DeltaLogPool, io: PrefillIO, stream=None) -> None:
    """Run a prompt through every tile (chunkwise) and leave the state in the base, log empty."""
    rc = load_library().dl_prefill(ctypes.byref(pool.c_dims), ctypes.byref(pool.c_pool), ctypes.byref(io),
                                   _stream(stream))
    _check(rc, "dl_prefill")
