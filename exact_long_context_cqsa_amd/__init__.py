"""Exact long-context attention for AMD Instinct MI355X: Python binding of ``libcqsa.so``.

Argument marshalling only.  Every step of the computation runs in the HIP library
(``csrc/``); PyTorch provides device memory, pinned host memory and the stream.
If the library is not built, importing this package raises: there is no fallback.

    import exact_long_context_cqsa_amd as cqsa
    out = cqsa.attention(q, k, v, is_causal=True)                 # SDPA semantics, exact
    out, lse = cqsa.attention(q, k, v, is_causal=True, kv_chunk=4096, return_lse=True)

Names follow the C ABI in ``include/cqsa.h``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["attention", "plan", "fwd_partial", "lse_merge", "finalize", "CqsaError", "library_path",
           "fwd_kernel_name", "cqs_assign", "cqs_default_set", "attention_backward", "schedule_trace", "backward_schedule_trace",
           "set_test_controls", "attention_noalloc", "MERGE_AUTO", "MERGE_KERNEL", "MERGE_FUSED"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libcqsa.so")

F16, BF16, F32 = 0, 1, 2
WHERE_DETECT, WHERE_DEVICE, WHERE_HOST = 0, 1, 2
MERGE_AUTO, MERGE_KERNEL, MERGE_FUSED = 0, 1, 2
LSE_NONE, LSE_WITH_OUT, LSE_DEVICE, LSE_HOST = 0, 1, 2, 3
_STATUS = {0: "OK", -1: "INVALID", -2: "UNSUPPORTED", -3: "BUDGET", -4: "OOM", -5: "HIP"}
_DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}


class CqsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("where", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class CqsaOptions(ctypes.Structure):
    _fields_ = [("q_chunk", ctypes.c_int64), ("kv_chunk", ctypes.c_int64), ("kv_splits", ctypes.c_int32),
                ("merge_mode", ctypes.c_int32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
                ("stream", ctypes.c_void_p), ("num_cus", ctypes.c_int32), ("cqs_c", ctypes.c_int32),
                ("cqs_l", ctypes.c_int32), ("precision", ctypes.c_int32), ("cqs_set", ctypes.POINTER(ctypes.c_int32)),
                ("wave_tokens", ctypes.c_int64), ("cqs_itr", ctypes.c_int32)]


class CqsaPlanInfo(ctypes.Structure):
    _fields_ = [("streamed", ctypes.c_int32), ("merge_mode", ctypes.c_int32), ("q_chunk", ctypes.c_int64),
                ("kv_chunk", ctypes.c_int64), ("n_q_chunks", ctypes.c_int64), ("n_kv_chunks", ctypes.c_int64),
                ("kv_splits", ctypes.c_int32), ("block_m", ctypes.c_int32), ("chunk_pairs", ctypes.c_int64),
                ("merges", ctypes.c_int64), ("kernel_launches", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_uint64), ("budget_bytes", ctypes.c_uint64),
                ("h2d_bytes", ctypes.c_uint64), ("d2h_bytes", ctypes.c_uint64), ("h2d_ms", ctypes.c_double),
                ("d2h_ms", ctypes.c_double), ("wall_ms", ctypes.c_double), ("cqs_c", ctypes.c_int32),
                ("cqs_subproblems", ctypes.c_int32), ("cqs_waves", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("wave_tokens", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class CqsaProbeResult(ctypes.Structure):
    _fields_ = [("mfma_f16_flop_per_s", ctypes.c_double), ("mfma_clock_hz", ctypes.c_double),
                ("lds_read_bytes_per_s", ctypes.c_double), ("lds_clock_hz", ctypes.c_double),
                ("hbm_copy_bytes_per_s", ctypes.c_double), ("mfma_seconds", ctypes.c_double),
                ("lds_seconds", ctypes.c_double), ("copy_seconds", ctypes.c_double),
                ("compute_units", ctypes.c_int32), ("wall_clock_khz", ctypes.c_int32)]


class CqsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cqsa {_STATUS.get(status, status)}: {message}")
        self.status = status


def fwd_kernel_name(head_dim: int, precision: int = 0) -> str:
    """The forward kernel (name and shape) a call with this head dim and precision launches."""
    return _lib.cqsa_fwd_kernel_name(int(head_dim), int(precision)).decode()


def probe_device(copy_bytes: int = 1 << 30, repeats: int = 5) -> dict:
    """Rates of the current device measured by cqsa_probe_device: dense fp16 matrix-core FLOP/s,
    LDS read bytes/s and HBM copy bytes/s, with the shader clock of the matrix and LDS runs and the
    per-clock, per-compute-unit figures derived from them."""
    r = CqsaProbeResult()
    _check(_lib.cqsa_probe_device(int(copy_bytes), int(repeats), ctypes.byref(r)))
    d = {name: getattr(r, name) for name, _ in r._fields_}
    cu = max(1, r.compute_units)
    d["mfma_f16_tflops"] = r.mfma_f16_flop_per_s / 1e12
    d["mfma_clock_ghz"] = r.mfma_clock_hz / 1e9
    d["mfma_flop_per_clk_per_cu"] = r.mfma_f16_flop_per_s / (r.mfma_clock_hz * cu) if r.mfma_clock_hz else None
    d["lds_read_tbs"] = r.lds_read_bytes_per_s / 1e12
    d["lds_bytes_per_clk_per_cu"] = r.lds_read_bytes_per_s / (r.lds_clock_hz * cu) if r.lds_clock_hz else None
    d["hbm_copy_gbs"] = r.hbm_copy_bytes_per_s / 1e9
    return d


def library_path() -> str:
    return _LIB_PATH


def set_test_controls(fwd_variant: int = 0, fail_after_launches: int = -1) -> None:
    """Process-wide test and measurement controls (cqsa_set_test_controls): the forward kernel shape
    (0 = the default) and forced launch failures after n launches per call (-1 = off)."""
    _check(_lib.cqsa_set_test_controls(int(fwd_variant), int(fail_after_launches)))


def _load_library():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                          "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(_LIB_PATH)
    T = ctypes.POINTER(CqsaTensor)
    O = ctypes.POINTER(CqsaOptions)
    I = ctypes.POINTER(CqsaPlanInfo)
    fp = ctypes.POINTER(ctypes.c_float)
    lib.cqsa_attention.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, T, fp]
    lib.cqsa_attention.restype = ctypes.c_int
    lib.cqsa_attention_ex.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, T, fp, O, I]
    lib.cqsa_attention_ex.restype = ctypes.c_int
    lib.cqsa_plan.argtypes = [T, T, T, ctypes.c_int, ctypes.c_uint64, T, ctypes.c_int, O, I]
    lib.cqsa_plan.restype = ctypes.c_int
    lib.cqsa_schedule_trace.argtypes = [T, T, T, ctypes.c_int, ctypes.c_uint64, T, ctypes.c_int, O, ctypes.c_char_p,
                                        ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
    lib.cqsa_schedule_trace.restype = ctypes.c_int
    lib.cqsa_backward_schedule_trace.argtypes = [T, T, T, T, T, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int,
                                                 ctypes.c_uint64, T, T, T, O, ctypes.c_char_p, ctypes.c_uint64,
                                                 ctypes.POINTER(ctypes.c_uint64)]
    lib.cqsa_backward_schedule_trace.restype = ctypes.c_int
    lib.cqsa_fwd_partial.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_int64, fp, fp,
                                     ctypes.c_void_p]
    lib.cqsa_fwd_partial.restype = ctypes.c_int
    lib.cqsa_lse_merge.argtypes = [ctypes.POINTER(fp), ctypes.POINTER(fp), ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_int64, fp, fp, ctypes.c_void_p]
    lib.cqsa_lse_merge.restype = ctypes.c_int
    lib.cqsa_finalize.argtypes = [fp, fp, T, fp, ctypes.c_void_p]
    lib.cqsa_finalize.restype = ctypes.c_int
    lib.cqsa_last_error.argtypes = []
    lib.cqsa_last_error.restype = ctypes.c_char_p
    lib.cqsa_version.argtypes = []
    lib.cqsa_version.restype = ctypes.c_int32
    lib.cqsa_struct_size.argtypes = [ctypes.c_int32]
    lib.cqsa_struct_size.restype = ctypes.c_uint64
    lib.cqsa_fwd_kernel_name.argtypes = [ctypes.c_int64, ctypes.c_int32]
    lib.cqsa_fwd_kernel_name.restype = ctypes.c_char_p
    lib.cqsa_attention_backward.argtypes = [T, T, T, T, T, fp, ctypes.c_int, ctypes.c_float, T, T, T, fp,
                                            ctypes.c_void_p]
    lib.cqsa_attention_backward.restype = ctypes.c_int
    lib.cqsa_attention_backward_ex.argtypes = [T, T, T, T, T, fp, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, T, T,
                                               T, O, I]
    lib.cqsa_attention_backward_ex.restype = ctypes.c_int
    lib.cqsa_cqs_assign.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32)]
    lib.cqsa_cqs_assign.restype = ctypes.c_int
    lib.cqsa_cqs_assign_itr.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int32)]
    lib.cqsa_cqs_assign_itr.restype = ctypes.c_int
    lib.cqsa_cqs_default_set.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    lib.cqsa_cqs_default_set.restype = ctypes.c_int32
    lib.cqsa_probe_device.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.POINTER(CqsaProbeResult)]
    lib.cqsa_probe_device.restype = ctypes.c_int
    lib.cqsa_set_test_controls.argtypes = [ctypes.c_int32, ctypes.c_int64]
    lib.cqsa_set_test_controls.restype = ctypes.c_int
    lib.cqsa_attention_noalloc.argtypes = [T, T, T, ctypes.c_int, ctypes.c_float, T, fp, ctypes.c_int32,
                                           ctypes.c_void_p, I]
    lib.cqsa_attention_noalloc.restype = ctypes.c_int
    for which, cls in enumerate((CqsaTensor, CqsaOptions, CqsaPlanInfo, CqsaProbeResult)):
        if lib.cqsa_struct_size(which) != ctypes.sizeof(cls):
            raise ImportError(f"{cls.__name__} layout differs from the built library")
    return lib


_lib = _load_library()


def _check(status: int):
    if status != 0:
        raise CqsaError(status, _lib.cqsa_last_error().decode(errors="replace"))


def _desc(t: torch.Tensor | None, where: int = WHERE_DETECT) -> CqsaTensor:
    d = CqsaTensor()
    if t is None:
        return d
    if t.dim() != 4:
        raise ValueError("tensors are [B, H, N, D]")
    if t.dtype not in _DT:
        raise ValueError(f"dtype {t.dtype} is not fp16/bf16/fp32")
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DT[t.dtype]
    d.where = where
    for i in range(4):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _fptr(t: torch.Tensor | None):
    if t is None:
        return None
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float))


def _device_of(*ts) -> torch.device | None:
    for t in ts:
        if t is not None and t.is_cuda:
            return t.device
    return None


def _int_array(xs):
    return (ctypes.c_int32 * len(xs))(*[int(x) for x in xs])


def cqs_default_set(c: int) -> tuple:
    """The library's built-in interest set for c parts (empty tuple if none)."""
    buf = (ctypes.c_int32 * 64)()
    n = _lib.cqsa_cqs_default_set(int(c), buf, 64)
    return tuple(buf[i] for i in range(n))


def cqs_assign(c: int, interest_set, itr: int = 1) -> list:
    """owner[a][b]: the subproblem of the quorum-set schedule that computes (query part a, key part b);
    with itr > 1, over the c**itr parts of the depth-itr schedule."""
    arr = _int_array(interest_set)
    n = int(c) ** int(itr) if itr >= 1 and c >= 1 else 0
    own = (ctypes.c_int32 * max(1, n * n))()
    if itr == 1:
        _check(_lib.cqsa_cqs_assign(int(c), arr, len(arr), own))
    else:
        _check(_lib.cqsa_cqs_assign_itr(int(c), arr, len(arr), int(itr), own))
    return [[own[a * n + b] for b in range(n)] for a in range(n)]


def _options(q_chunk=None, kv_chunk=None, kv_splits=None, merge=None, stream=None, workspace=None,
             num_cus=None, cqs=None, precision=0, wave_tokens=None, cqs_itr=None) -> CqsaOptions:
    """cqs: None (grid schedule), c (quorum-set schedule with the built-in set) or (c, interest_set);
    cqs_itr: its depth (None or 1: one level; itr > 1: c**itr parts).
    precision: 0 (P rounded to the input dtype) or 1 (split P, hi + lo).
    wave_tokens: packed-row budget of a wave of the quorum-set schedule (None: the default)."""
    o = CqsaOptions()
    o.precision = int(precision or 0)
    o.wave_tokens = int(wave_tokens or 0)
    o.cqs_itr = int(cqs_itr or 0)
    if cqs is not None:
        if isinstance(cqs, int):
            o.cqs_c = cqs
        else:
            c, iset = cqs
            o.cqs_c = int(c)
            arr = _int_array(iset)
            o.cqs_l = len(arr)
            o.cqs_set = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
            o._keep = arr   # the array lives as long as the options
    o.q_chunk = int(q_chunk or 0)
    o.kv_chunk = int(kv_chunk or 0)
    o.kv_splits = int(kv_splits or 0)
    o.merge_mode = int(merge or 0)
    o.stream = stream
    o.num_cus = int(num_cus or 0)
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    return o


def _lse_code(want_lse) -> int:
    """want_lse: False/None (no lse), True (lse where out lives), "device" or "host"."""
    if want_lse in (False, None, 0):
        return LSE_NONE
    if want_lse is True or want_lse == 1:
        return LSE_WITH_OUT
    return {"device": LSE_DEVICE, "host": LSE_HOST}[want_lse]


def plan(q, k, v, is_causal=False, mem_budget=None, *, out=None, want_lse=False, q_chunk=None, kv_chunk=None,
         kv_splits=None, merge=None, where=None, num_cus=None, cqs=None, precision=0, wave_tokens=None,
         cqs_itr=None) -> dict:
    """The plan ``attention`` would run (nothing is allocated or computed).

    ``q``/``k``/``v``/``out`` may be tensors, or ``(shape, dtype)`` pairs with ``where`` = a dict of
    "device"/"host" per name, for a dry run of shapes that do not exist.  ``want_lse``: False, True
    (lse where out lives), "device" or "host"."""
    where = where or {}

    def mk(name, t, default_dtype):
        if isinstance(t, torch.Tensor):
            return _desc(t)
        shape, dtype = t if t is not None else (None, default_dtype)
        d = CqsaTensor()
        d.dtype = _DT[dtype]
        d.where = WHERE_HOST if where.get(name, "device") == "host" else WHERE_DEVICE
        stride = [shape[1] * shape[2] * shape[3], shape[2] * shape[3], shape[3], 1]
        for i in range(4):
            d.shape[i] = shape[i]
            d.stride[i] = stride[i]
        return d

    dq = mk("q", q, None)
    dk = mk("k", k, None)
    dv = mk("v", v, None)
    if out is None:
        qshape = tuple(q.shape) if isinstance(q, torch.Tensor) else tuple(q[0])
        qdt = q.dtype if isinstance(q, torch.Tensor) else q[1]
        out = (qshape, qdt)
    do = mk("out", out, None)
    info = CqsaPlanInfo()
    opt = _options(q_chunk, kv_chunk, kv_splits, merge, num_cus=num_cus, cqs=cqs, precision=precision,
                   wave_tokens=wave_tokens, cqs_itr=cqs_itr)
    _check(_lib.cqsa_plan(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), 1 if is_causal else 0,
                          int(mem_budget or 0), ctypes.byref(do), _lse_code(want_lse), ctypes.byref(opt),
                          ctypes.byref(info)))
    return info.as_dict()


def _trace_desc(t) -> CqsaTensor:
    shape, dtype, where, addr = t[:4]
    stride = t[4] if len(t) > 4 else [shape[1] * shape[2] * shape[3], shape[2] * shape[3], shape[3], 1]
    d = CqsaTensor()
    d.data = int(addr)
    d.dtype = _DT[dtype]
    d.where = {"host": WHERE_HOST, "device": WHERE_DEVICE}.get(where, WHERE_DETECT)
    for i in range(4):
        d.shape[i] = shape[i]
        d.stride[i] = stride[i]
    return d


def backward_schedule_trace(q, k, v, out, dout, lse, dq, dk, dv, is_causal, mem_budget, *, q_chunk=None,
                            kv_chunk=None) -> str:
    """The chunked backward's operations, recorded (see ``cqsa_backward_schedule_trace``).  Tensors are
    ``(shape, dtype, where, address[, strides])`` tuples; lse is ``(where, address)``."""
    ds = [_trace_desc(t) for t in (q, k, v, out, dout)]
    gs = [_trace_desc(t) for t in (dq, dk, dv)]
    opt = _options(q_chunk, kv_chunk, None, None)
    lwhere = WHERE_HOST if lse[0] == "host" else WHERE_DEVICE
    need = ctypes.c_uint64(0)
    args = (*[ctypes.byref(d) for d in ds], ctypes.c_void_p(int(lse[1])), lwhere, 1 if is_causal else 0,
            int(mem_budget), *[ctypes.byref(g) for g in gs], ctypes.byref(opt))
    _check(_lib.cqsa_backward_schedule_trace(*args, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(int(need.value))
    _check(_lib.cqsa_backward_schedule_trace(*args, buf, int(need.value), None))
    return buf.value.decode()


def schedule_trace(q, k, v, is_causal, mem_budget, *, out, want_lse=False, q_chunk=None, kv_chunk=None,
                   kv_splits=None, merge=None, num_cus=256, cqs=None, precision=0, wave_tokens=None,
                   cqs_itr=None) -> str:
    """The operations ``attention`` would issue, recorded instead of run (no GPU needed); see
    ``cqsa_schedule_trace`` in cqsa.h for the line format.  q, k, v and out are
    ``(shape, dtype, where, address)`` tuples ("host" or "device"; the address is a stand-in that is
    never dereferenced), optionally with element strides as a fifth item (default: contiguous).
    ``want_lse``: False, True (lse where out lives), "device" or "host"."""
    def mk(t):
        shape, dtype, where, addr = t[:4]
        stride = t[4] if len(t) > 4 else [shape[1] * shape[2] * shape[3], shape[2] * shape[3], shape[3], 1]
        d = CqsaTensor()
        d.data = int(addr)
        d.dtype = _DT[dtype]
        d.where = {"host": WHERE_HOST, "device": WHERE_DEVICE}.get(where, WHERE_DETECT)
        for i in range(4):
            d.shape[i] = shape[i]
            d.stride[i] = stride[i]
        return d

    dq, dk, dv, do = mk(q), mk(k), mk(v), mk(out)
    opt = _options(q_chunk, kv_chunk, kv_splits, merge, num_cus=num_cus, cqs=cqs, precision=precision,
                   wave_tokens=wave_tokens, cqs_itr=cqs_itr)
    need = ctypes.c_uint64(0)
    args = (ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), 1 if is_causal else 0, int(mem_budget),
            ctypes.byref(do), _lse_code(want_lse), ctypes.byref(opt))
    _check(_lib.cqsa_schedule_trace(*args, None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(int(need.value))
    _check(_lib.cqsa_schedule_trace(*args, buf, int(need.value), None))
    return buf.value.decode()


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, is_causal: bool = False, scale: float | None = None,
              mem_budget: int | None = None, *, q_chunk: int | None = None, kv_chunk: int | None = None,
              kv_splits: int | None = None, merge: int | None = None, out: torch.Tensor | None = None,
              out_dtype: torch.dtype | None = None, return_lse: bool = False, return_info: bool = False,
              stream: torch.cuda.Stream | None = None, cqs=None, precision: int = 0, wave_tokens: int | None = None,
              cqs_itr: int | None = None):
    """Exact ``softmax(scale * q k^T [+ causal mask]) v`` (SDPA semantics; causal is bottom-right
    aligned when Nq < Nk; GQA when k/v have fewer heads).

    q: [B, Hq, Nq, D], k/v: [B, Hkv, Nk, D], fp16 or bf16, D in {64, 128}; each on the GPU or in
    pinned host memory (then streamed in chunks).  ``mem_budget`` caps the device bytes the call
    uses (0/None: the free memory).  ``kv_chunk``/``q_chunk`` force a decomposition; ``merge``
    picks how partials merge (MERGE_KERNEL or MERGE_FUSED).  ``cqs`` runs the cyclic quorum-set
    schedule instead of the chunk grid: c (built-in interest set) or (c, interest_set), ``cqs_itr``
    levels deep (c**cqs_itr parts; default one level); its subproblems run in waves of at most
    ``wave_tokens`` staged rows (one batched launch per wave).
    ``precision=1`` feeds P to the PV product as a hi part plus a lo residual (two accumulator
    chains), for results near fp32 accuracy at about twice the PV work.  Returns out
    (on q's device; pinned host memory when q is on the host), plus lse [B, Hq, Nq] fp32 and the
    plan dict on request.  When q, k or v requires grad (and grad mode is on), the call records an
    autograd node whose backward runs ``attention_backward`` (device-resident inputs only)."""
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v)):
        if out is not None or return_info:
            raise ValueError("out= and return_info are not available on the autograd path")
        res = _AttentionFn.apply(q, k, v, bool(is_causal), scale, dict(
            mem_budget=mem_budget, q_chunk=q_chunk, kv_chunk=kv_chunk, kv_splits=kv_splits, merge=merge,
            out_dtype=out_dtype, stream=stream, cqs=cqs, precision=precision, wave_tokens=wave_tokens,
            cqs_itr=cqs_itr))
        return res if return_lse else res[0]
    dev = _device_of(q, k, v, out)
    if dev is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    B, Hq, Nq, D = q.shape
    if out is None:
        odt = out_dtype or q.dtype
        if q.is_cuda:
            out = torch.empty((B, Hq, Nq, D), dtype=odt, device=q.device)
        else:
            out = torch.empty((B, Hq, Nq, D), dtype=odt, pin_memory=True)
    lse = None
    if return_lse:
        lse = (torch.empty((B, Hq, Nq), dtype=torch.float32, device=out.device) if out.is_cuda
               else torch.empty((B, Hq, Nq), dtype=torch.float32, pin_memory=True))
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        dq, dk, dv, do = _desc(q), _desc(k), _desc(v), _desc(out)
        opt = _options(q_chunk, kv_chunk, kv_splits, merge, stream=st.cuda_stream, cqs=cqs, precision=precision,
                       wave_tokens=wave_tokens, cqs_itr=cqs_itr)
        # the budget is resolved here, once: left to the library, the plan below and the call would each
        # read the free memory, and the workspace allocated in between would change the second reading
        budget = int(mem_budget or 0) or int(torch.cuda.mem_get_info(dev)[0])
        # size the workspace first so that device-resident calls take it from PyTorch's allocator
        # (stream-ordered, no hipMalloc, no synchronisation)
        pinfo = CqsaPlanInfo()
        lse_code = LSE_NONE if lse is None else (LSE_DEVICE if lse.is_cuda else LSE_HOST)
        _check(_lib.cqsa_plan(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), 1 if is_causal else 0, budget,
                              ctypes.byref(do), lse_code, ctypes.byref(opt), ctypes.byref(pinfo)))
        ws = None
        if pinfo.workspace_bytes > 0:
            ws = torch.empty(int(pinfo.workspace_bytes), dtype=torch.uint8, device=dev)
            opt.workspace = ws.data_ptr()
            opt.workspace_bytes = int(pinfo.workspace_bytes)
        info = CqsaPlanInfo()
        sc = float(scale) if scale is not None else 0.0
        _check(_lib.cqsa_attention_ex(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), 1 if is_causal else 0,
                                      sc, budget, ctypes.byref(do), _fptr(lse), ctypes.byref(opt),
                                      ctypes.byref(info)))
        if ws is not None:
            ws.record_stream(st)
    res = (out,)
    if return_lse:
        res += (lse,)
    if return_info:
        res += (info.as_dict(),)
    return res[0] if len(res) == 1 else res


class _AttentionFn(torch.autograd.Function):
    """Autograd node: the forward kernels, then cqsa_attention_backward from the saved out and lse."""

    @staticmethod
    def forward(ctx, q, k, v, is_causal, scale, kw):
        with torch.no_grad():
            out, lse = attention(q.detach(), k.detach(), v.detach(), is_causal, scale, return_lse=True, **kw)
        ctx.save_for_backward(q, k, v, out, lse)
        ctx.is_causal, ctx.scale = is_causal, scale
        ctx.mark_non_differentiable(lse)
        return out, lse

    @staticmethod
    def backward(ctx, dout, _dlse):
        q, k, v, out, lse = ctx.saved_tensors
        g = attention_backward(q, k, v, out, dout.to(q.dtype).contiguous(), lse, ctx.is_causal, ctx.scale)
        return g[0], g[1], g[2], None, None, None


def attention_backward(q, k, v, out, dout, lse, is_causal: bool = False, scale: float | None = None, *,
                       grad_dtype: torch.dtype | None = None, stream: torch.cuda.Stream | None = None,
                       mem_budget: int | None = None, q_chunk: int | None = None, kv_chunk: int | None = None,
                       return_info: bool = False):
    """Gradients (dq, dk, dv) of ``attention`` for the upstream gradient ``dout``, from the forward's
    ``out`` and ``lse``.  dk/dv have k's shape (GQA heads summed).  Every tensor may be on the GPU or
    in pinned host memory; host operands (or a forced ``q_chunk``/``kv_chunk``, or ``mem_budget``) run
    the chunked backward, which streams them under the device-memory budget.  dq is allocated where q
    lives, dk and dv where k lives (pinned when on the host)."""
    gd = grad_dtype or q.dtype
    dev = _device_of(q, k, v, out, dout) or torch.device("cuda", torch.cuda.current_device())

    def like(t, shape):
        return (torch.empty(shape, dtype=gd, device=dev) if t.is_cuda
                else torch.empty(shape, dtype=gd, pin_memory=True))

    dq, dk, dv = like(q, q.shape), like(k, k.shape), like(k, v.shape)
    B, Hq, Nq, _ = q.shape
    chunked = (not all(t.is_cuda for t in (q, k, v, out, dout, lse)) or q_chunk or kv_chunk or mem_budget
               or return_info)
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        sc = float(scale) if scale is not None else 0.0
        if chunked:
            opt = _options(q_chunk, kv_chunk, None, None, stream=st.cuda_stream)
            info = CqsaPlanInfo()
            _check(_lib.cqsa_attention_backward_ex(
                ctypes.byref(_desc(q)), ctypes.byref(_desc(k)), ctypes.byref(_desc(v)), ctypes.byref(_desc(out)),
                ctypes.byref(_desc(dout)), _fptr(lse), 1 if is_causal else 0, sc, int(mem_budget or 0),
                ctypes.byref(_desc(dq)), ctypes.byref(_desc(dk)), ctypes.byref(_desc(dv)), ctypes.byref(opt),
                ctypes.byref(info)))
            return (dq, dk, dv, info.as_dict()) if return_info else (dq, dk, dv)
        stats = torch.empty(max(1, 2 * B * Hq * Nq), dtype=torch.float32, device=dev)
        _check(_lib.cqsa_attention_backward(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)), ctypes.byref(_desc(v)),
                                            ctypes.byref(_desc(out)), ctypes.byref(_desc(dout)), _fptr(lse),
                                            1 if is_causal else 0, sc, ctypes.byref(_desc(dq)),
                                            ctypes.byref(_desc(dk)), ctypes.byref(_desc(dv)), _fptr(stats),
                                            st.cuda_stream))
        stats.record_stream(st)
    return dq, dk, dv


def attention_noalloc(q, k, v, out, lse=None, is_causal: bool = False, scale: float | None = None, *,
                      kv_splits: int = 0, stream: torch.cuda.Stream | None = None) -> dict:
    """cqsa_attention_noalloc: the same attention with every operand on the device and no allocation at
    all (the partials of a split key range live in the library's fixed device array); out and lse
    are the caller's tensors.  Stream-ordered.  Returns the plan that ran."""
    info = CqsaPlanInfo()
    dev = _device_of(q, k, v, out) or torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(dev):
        st = stream if stream is not None else torch.cuda.current_stream(dev)
        sc = float(scale) if scale is not None else 0.0
        _check(_lib.cqsa_attention_noalloc(ctypes.byref(_desc(q)), ctypes.byref(_desc(k)), ctypes.byref(_desc(v)),
                                           1 if is_causal else 0, sc, ctypes.byref(_desc(out)), _fptr(lse),
                                           int(kv_splits), st.cuda_stream, ctypes.byref(info)))
    return info.as_dict()


def fwd_partial(q, k, v, is_causal=False, scale=None, kv_begin=0, kv_end=None, stream=None):
    """Partial triple of one KV chunk: (O unnormalised fp32 [B,Hq,Nq,D], ml fp32 [B,Hq,Nq,2])."""
    B, Hq, Nq, D = q.shape
    kv_end = k.shape[2] if kv_end is None else kv_end
    o = torch.empty((B, Hq, Nq, D), dtype=torch.float32, device=q.device)
    ml = torch.empty((B, Hq, Nq, 2), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        st = stream if stream is not None else torch.cuda.current_stream(q.device)
        dq, dk, dv = _desc(q), _desc(k), _desc(v)
        _check(_lib.cqsa_fwd_partial(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), 1 if is_causal else 0,
                                     float(scale or 0.0), int(kv_begin), int(kv_end), _fptr(o), _fptr(ml),
                                     st.cuda_stream))
    return o, ml


def lse_merge(parts, out=None, stream=None):
    """Merge [(O, ml), ...] partial triples (fp32, [..., D] / [..., 2]) by log-sum-exp."""
    o0, ml0 = parts[0]
    D = o0.shape[-1]
    rows = o0.numel() // D
    o_out, ml_out = out if out is not None else (torch.empty_like(o0), torch.empty_like(ml0))
    FP = ctypes.POINTER(ctypes.c_float)
    op = (FP * len(parts))(*[_fptr(p[0]) for p in parts])
    mp = (FP * len(parts))(*[_fptr(p[1]) for p in parts])
    with torch.cuda.device(o0.device):
        st = stream if stream is not None else torch.cuda.current_stream(o0.device)
        _check(_lib.cqsa_lse_merge(op, mp, len(parts), rows, D, _fptr(o_out), _fptr(ml_out), st.cuda_stream))
    return o_out, ml_out


def finalize(o, ml, out_dtype=torch.float32, return_lse=True, stream=None):
    """out = O / l in ``out_dtype`` and lse = m + ln l from a merged triple [B, Hq, Nq, D] / [..., 2]."""
    B, Hq, Nq, D = o.shape
    out = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=o.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=o.device) if return_lse else None
    with torch.cuda.device(o.device):
        st = stream if stream is not None else torch.cuda.current_stream(o.device)
        do = _desc(out)
        _check(_lib.cqsa_finalize(_fptr(o), _fptr(ml), ctypes.byref(do), _fptr(lse), st.cuda_stream))
    return (out, lse) if return_lse else out
