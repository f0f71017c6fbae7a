"""Python binding of the gfx950 Muon step library (``libmuon.so``).

Argument marshalling only: every step of the optimizer runs in the HIP
kernels behind the C ABI declared in ``include/muon.h``.  PyTorch provides
device memory and streams.  There is no CPU fallback: if the library is not
built, or the device is not gfx950, the calls raise.

The names mirror the C entry points:
``muon_step``, ``muon_step_noalloc``, ``muon_ns``, ``muon_workspace_bytes``,
``muon_ns_workspace_bytes``, ``muon_adamw_step``,
``muon_adamw_workspace_bytes``, ``muon_cayley_step``,
``muon_cayley_workspace_bytes``, ``muon_status_string``,
``muon_last_error_message``, ``muon_profile_enable``, ``muon_profile_read``,
``muon_version``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_UNSUPPORTED = -2
MUON_ERR_WORKSPACE = -3
MUON_ERR_HIP = -4

MUON_F32 = 0
MUON_BF16 = 1

SCALE_RULES = {"naive": 0, "kellerjordan": 1, "mup": 2, "moonlight": 3}
MUON_FLAG_NESTEROV = 1
MUON_KCLASS_COUNT = 9
KERNEL_CLASSES = ("momentum_norm", "norm_finalize", "gram", "poly", "update", "apply", "adamw", "cayley",
                  "update_apply")


class MuonMatrix(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class MuonNsCoeffs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float)]


class MuonHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("eps", ctypes.c_float), ("scale_rule", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
                ("schedule", ctypes.POINTER(MuonNsCoeffs)), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class MuonNsMatrix(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_void_p), ("out", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class MuonAdamwTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
                ("exp_avg_sq", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class MuonAdamwHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class MuonCayleyMatrix(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class MuonCayleyHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta", ctypes.c_float)]


class MuonProfile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * MUON_KCLASS_COUNT), ("launches", ctypes.c_int64 * MUON_KCLASS_COUNT)]


# Every symbol include/muon.h declares, with its ctypes signature.
SIGNATURES = {
    "muon_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MuonMatrix), ctypes.c_int32, ctypes.POINTER(MuonHparams)]),
    "muon_step": (ctypes.c_int32, [ctypes.POINTER(MuonMatrix), ctypes.c_int32, ctypes.POINTER(MuonHparams),
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "muon_step_noalloc": (ctypes.c_int32, [ctypes.POINTER(MuonMatrix), ctypes.c_int32, ctypes.POINTER(MuonHparams),
                                           ctypes.c_void_p]),
    "muon_ns_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MuonNsMatrix), ctypes.c_int32,
                                                  ctypes.POINTER(MuonHparams)]),
    "muon_ns": (ctypes.c_int32, [ctypes.POINTER(MuonNsMatrix), ctypes.c_int32, ctypes.POINTER(MuonHparams),
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "muon_adamw_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MuonAdamwTensor), ctypes.c_int32,
                                                     ctypes.POINTER(MuonAdamwHparams)]),
    "muon_adamw_step": (ctypes.c_int32, [ctypes.POINTER(MuonAdamwTensor), ctypes.c_int32,
                                         ctypes.POINTER(MuonAdamwHparams), ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]),
    "muon_cayley_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MuonCayleyMatrix), ctypes.c_int32,
                                                      ctypes.POINTER(MuonCayleyHparams)]),
    "muon_cayley_step": (ctypes.c_int32, [ctypes.POINTER(MuonCayleyMatrix), ctypes.c_int32,
                                          ctypes.POINTER(MuonCayleyHparams), ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p]),
    "muon_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "muon_last_error_message": (ctypes.c_char_p, []),
    "muon_profile_enable": (ctypes.c_int32, [ctypes.c_int32]),
    "muon_profile_read": (ctypes.c_int32, [ctypes.POINTER(MuonProfile)]),
    "muon_version": (ctypes.c_int32, []),
}

_lib = None


class MuonError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_string(status)} ({detail})")


def load(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                           " or `python matrix_aware_optimizer_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    return load().muon_status_string(int(status)).decode()


def muon_status_string(status: int) -> str:
    return _status_string(status)


def muon_last_error_message() -> str:
    return load().muon_last_error_message().decode()


def muon_version() -> int:
    return int(load().muon_version())


def _check(status: int):
    if status != MUON_OK:
        raise MuonError(status, muon_last_error_message())


# --------------------------------------------------------------------------
# Marshalling helpers
# --------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    raise ValueError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _check_matrix(t, what):
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (row-major)")


def make_hparams(*, lr=0.02, beta=0.95, weight_decay=0.0, eps=1e-7, scale_rule="naive",
                 schedule: Sequence[Sequence[float]] = (), dtype=MUON_BF16, nesterov=False):
    """Build a muon_hparams struct.  Returns (struct, keepalive)."""
    sched = (MuonNsCoeffs * max(1, len(schedule)))()
    for k, (a, b, c) in enumerate(schedule):
        sched[k] = MuonNsCoeffs(a, b, c)
    rule = SCALE_RULES[scale_rule] if isinstance(scale_rule, str) else int(scale_rule)
    hp = MuonHparams(lr, beta, weight_decay, eps, rule, len(schedule),
                     ctypes.cast(sched, ctypes.POINTER(MuonNsCoeffs)), int(dtype),
                     MUON_FLAG_NESTEROV if nesterov else 0)
    return hp, sched


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _workspace_for(need: int, workspace, device, stream):
    """The workspace a call runs with, safe for torch's caching allocator.

    The kernels use the workspace on ``stream``.  A workspace allocated here
    is allocated on that stream, so the allocator orders its reuse after the
    work enqueued there; a caller's workspace used on a stream other than the
    current one is recorded on it (``record_stream``), so dropping it does not
    hand its memory to other work while the call's kernels still read it.
    """
    import torch
    if workspace is None:
        if stream is None:
            return allocate_workspace(need, device)
        with torch.cuda.stream(stream):
            return allocate_workspace(need, device)
    if workspace.numel() * workspace.element_size() < need:
        raise MuonError(MUON_ERR_WORKSPACE, f"workspace has {workspace.numel()} bytes, {need} needed")
    if stream is not None and stream != torch.cuda.current_stream(workspace.device):
        workspace.record_stream(stream)
    return workspace


def _matrices(weights, grads, moms):
    weights, grads, moms = list(weights), list(grads), list(moms)
    if not (len(weights) == len(grads) == len(moms)):
        raise ValueError("weights, grads and momenta must have equal lengths")
    arr = (MuonMatrix * max(1, len(weights)))()
    dtype = None
    for i, (w, g, m) in enumerate(zip(weights, grads, moms)):
        _check_matrix(w, f"weight[{i}]")
        _check_matrix(m, f"momentum[{i}]")
        if g is not None:
            _check_matrix(g, f"grad[{i}]")
            if g.shape != w.shape or g.dtype != w.dtype:
                raise ValueError(f"grad[{i}] must match weight[{i}] in shape and dtype")
        if m.shape != w.shape or m.dtype != w.dtype:
            raise ValueError(f"momentum[{i}] must match weight[{i}] in shape and dtype")
        code = _dtype_code(w)
        if dtype is None:
            dtype = code
        elif code != dtype:
            raise ValueError("all matrices of one call must share a dtype")
        arr[i] = MuonMatrix(w.data_ptr(), g.data_ptr() if g is not None else None, m.data_ptr(),
                            w.shape[0], w.shape[1])
    return arr, len(weights), (MUON_BF16 if dtype is None else dtype)


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------

def muon_workspace_bytes(weights, grads, moms, **hp_kwargs) -> int:
    arr, n, dtype = _matrices(weights, grads, moms)
    hp, keep = make_hparams(dtype=dtype, **hp_kwargs)
    size = load().muon_workspace_bytes(arr, n, ctypes.byref(hp))
    if size == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    return int(size)


def allocate_workspace(nbytes: int, device=None):
    """Device workspace through torch (256-byte aligned by torch's allocator)."""
    import torch
    ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device or "cuda")
    if ws.data_ptr() % 256:
        raise RuntimeError("torch returned a workspace that is not 256-byte aligned")
    return ws


def muon_step(weights: Iterable, grads: Iterable, moms: Iterable, *, lr, beta=0.95, weight_decay=0.0,
              schedule=(), scale_rule="naive", eps=1e-7, nesterov=False, workspace=None, stream=None):
    """One grouped Muon step, in place on ``weights`` and ``moms`` (torch tensors on the GPU).

    A ``None`` gradient skips its matrix.  ``workspace`` is an optional uint8
    device tensor of at least :func:`muon_workspace_bytes` bytes; one is
    allocated through torch otherwise.  Asynchronous on ``stream`` (default:
    torch's current stream).
    """
    weights, grads, moms = list(weights), list(grads), list(moms)
    arr, n, dtype = _matrices(weights, grads, moms)
    hp, keep = make_hparams(lr=lr, beta=beta, weight_decay=weight_decay, eps=eps, scale_rule=scale_rule,
                            schedule=schedule, dtype=dtype, nesterov=nesterov)
    lib = load()
    need = lib.muon_workspace_bytes(arr, n, ctypes.byref(hp))
    if need == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    workspace = _workspace_for(need, workspace, weights[0].device if weights else None, stream)
    _check(lib.muon_step(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                         workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return workspace


NOALLOC_SCRATCH_BYTES = 128 << 20   # MUON_NOALLOC_SCRATCH_BYTES


def muon_step_noalloc(weights: Iterable, grads: Iterable, moms: Iterable, *, lr, beta=0.95, weight_decay=0.0,
                      schedule=(), scale_rule="naive", eps=1e-7, nesterov=False, stream=None):
    """:func:`muon_step` without a workspace and without any allocation: the library
    uses its own per-GPU device array of ``NOALLOC_SCRATCH_BYTES``.  Calls that
    overlap on one GPU race; lists that need more workspace raise MuonError."""
    weights, grads, moms = list(weights), list(grads), list(moms)
    arr, n, dtype = _matrices(weights, grads, moms)
    hp, keep = make_hparams(lr=lr, beta=beta, weight_decay=weight_decay, eps=eps, scale_rule=scale_rule,
                            schedule=schedule, dtype=dtype, nesterov=nesterov)
    _check(load().muon_step_noalloc(arr, n, ctypes.byref(hp), _stream_handle(stream)))


def _ns_matrices(inputs, outputs):
    inputs, outputs = list(inputs), list(outputs)
    if len(inputs) != len(outputs):
        raise ValueError("inputs and outputs must have equal lengths")
    import torch
    arr = (MuonNsMatrix * max(1, len(inputs)))()
    dtype = None
    for i, (x, o) in enumerate(zip(inputs, outputs)):
        _check_matrix(x, f"in[{i}]")
        _check_matrix(o, f"out[{i}]")
        if o.dtype != torch.float32 or o.shape != x.shape:
            raise ValueError(f"out[{i}] must be float32 with the input's shape")
        code = _dtype_code(x)
        if dtype is None:
            dtype = code
        elif code != dtype:
            raise ValueError("all inputs of one call must share a dtype")
        arr[i] = MuonNsMatrix(x.data_ptr(), o.data_ptr(), x.shape[0], x.shape[1])
    return arr, len(inputs), (MUON_BF16 if dtype is None else dtype)


def muon_ns_workspace_bytes(inputs, outputs, *, schedule=(), eps=1e-7) -> int:
    arr, n, dtype = _ns_matrices(inputs, outputs)
    hp, keep = make_hparams(schedule=schedule, eps=eps, dtype=dtype)
    size = load().muon_ns_workspace_bytes(arr, n, ctypes.byref(hp))
    if size == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    return int(size)


def muon_ns(inputs, outputs, *, schedule, eps=1e-7, workspace=None, stream=None):
    """outputs[i] = NS(inputs[i] / (||inputs[i]||_F + eps)), fp32 outputs."""
    inputs, outputs = list(inputs), list(outputs)
    arr, n, dtype = _ns_matrices(inputs, outputs)
    hp, keep = make_hparams(schedule=schedule, eps=eps, dtype=dtype)
    lib = load()
    need = lib.muon_ns_workspace_bytes(arr, n, ctypes.byref(hp))
    if need == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    workspace = _workspace_for(need, workspace, inputs[0].device if inputs else None, stream)
    _check(lib.muon_ns(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                       workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return workspace


def _adamw_tensors(params, grads, exp_avgs, exp_avg_sqs):
    import torch
    params, grads, exp_avgs, exp_avg_sqs = list(params), list(grads), list(exp_avgs), list(exp_avg_sqs)
    if not (len(params) == len(grads) == len(exp_avgs) == len(exp_avg_sqs)):
        raise ValueError("params, grads, exp_avgs and exp_avg_sqs must have equal lengths")
    arr = (MuonAdamwTensor * max(1, len(params)))()
    dtype = None
    for i, (p, g, m, v) in enumerate(zip(params, grads, exp_avgs, exp_avg_sqs)):
        for t, what in ((p, "param"), (m, "exp_avg"), (v, "exp_avg_sq")):
            if not t.is_contiguous():
                raise ValueError(f"{what}[{i}] must be contiguous")
        if g is not None and (not g.is_contiguous() or g.shape != p.shape or g.dtype != p.dtype):
            raise ValueError(f"grad[{i}] must be contiguous and match param[{i}] in shape and dtype")
        for t, what in ((m, "exp_avg"), (v, "exp_avg_sq")):
            if t.dtype != torch.float32 or t.numel() != p.numel():
                raise ValueError(f"{what}[{i}] must be float32 with param[{i}]'s number of elements")
        code = _dtype_code(p)
        if dtype is None:
            dtype = code
        elif code != dtype:
            raise ValueError("all params of one call must share a dtype")
        arr[i] = MuonAdamwTensor(p.data_ptr(), g.data_ptr() if g is not None else None, m.data_ptr(),
                                 v.data_ptr(), p.numel())
    return arr, len(params), (MUON_BF16 if dtype is None else dtype)


def muon_adamw_workspace_bytes(params, grads, exp_avgs, exp_avg_sqs, *, lr=1e-3, betas=(0.9, 0.999),
                               eps=1e-8, weight_decay=0.0, step=1) -> int:
    arr, n, dtype = _adamw_tensors(params, grads, exp_avgs, exp_avg_sqs)
    hp = MuonAdamwHparams(lr, betas[0], betas[1], eps, weight_decay, int(step), dtype)
    size = load().muon_adamw_workspace_bytes(arr, n, ctypes.byref(hp))
    if size == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    return int(size)


def muon_adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr, betas=(0.9, 0.999), eps=1e-8,
                    weight_decay=0.0, step, workspace=None, stream=None):
    """One grouped AdamW step, in place on params and the fp32 moments.

    ``step`` counts calls and starts at 1 (it sets the bias corrections).  A
    ``None`` gradient skips its tensor.  Asynchronous on ``stream``.
    """
    params = list(params)
    arr, n, dtype = _adamw_tensors(params, grads, exp_avgs, exp_avg_sqs)
    hp = MuonAdamwHparams(lr, betas[0], betas[1], eps, weight_decay, int(step), dtype)
    lib = load()
    need = lib.muon_adamw_workspace_bytes(arr, n, ctypes.byref(hp))
    if need == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    workspace = _workspace_for(need, workspace, params[0].device if params else None, stream)
    _check(lib.muon_adamw_step(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                               workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return workspace


def _cayley_matrices(weights, grads, moms):
    import torch
    weights, grads, moms = list(weights), list(grads), list(moms)
    if not (len(weights) == len(grads) == len(moms)):
        raise ValueError("weights, grads and momenta must have equal lengths")
    arr = (MuonCayleyMatrix * max(1, len(weights)))()
    for i, (w, g, m) in enumerate(zip(weights, grads, moms)):
        for t, what in ((w, "weight"), (m, "momentum")) + (((g, "grad"),) if g is not None else ()):
            _check_matrix(t, f"{what}[{i}]")
            if t.dtype != torch.float32 or t.shape != w.shape:
                raise ValueError(f"{what}[{i}] must be float32 with weight[{i}]'s shape")
        arr[i] = MuonCayleyMatrix(w.data_ptr(), g.data_ptr() if g is not None else None, m.data_ptr(),
                                  w.shape[0], w.shape[1])
    return arr, len(weights)


def muon_cayley_workspace_bytes(weights, grads, moms, *, lr=1e-3, beta=0.9) -> int:
    arr, n = _cayley_matrices(weights, grads, moms)
    hp = MuonCayleyHparams(lr, beta)
    size = load().muon_cayley_workspace_bytes(arr, n, ctypes.byref(hp))
    if size == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    return int(size)


def muon_cayley_step(weights, grads, moms, *, lr, beta=0.9, workspace=None, stream=None):
    """One grouped Muon-Cayley step (fp32), in place on ``weights`` and ``moms``.

    Each weight must have orthonormal columns (orthonormal rows when it is wide);
    the update keeps it so.  A ``None`` gradient skips its matrix.
    """
    weights = list(weights)
    arr, n = _cayley_matrices(weights, grads, moms)
    hp = MuonCayleyHparams(lr, beta)
    lib = load()
    need = lib.muon_cayley_workspace_bytes(arr, n, ctypes.byref(hp))
    if need == 0:
        raise MuonError(MUON_ERR_INVALID_ARG, muon_last_error_message())
    workspace = _workspace_for(need, workspace, weights[0].device if weights else None, stream)
    _check(lib.muon_cayley_step(arr, n, ctypes.byref(hp), ctypes.c_void_p(workspace.data_ptr()),
                                workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return workspace


def muon_profile_enable(on: bool = True):
    _check(load().muon_profile_enable(1 if on else 0))


def muon_profile_read() -> dict:
    prof = MuonProfile()
    _check(load().muon_profile_read(ctypes.byref(prof)))
    return {name: {"ms": prof.ms[i], "launches": int(prof.launches[i])} for i, name in enumerate(KERNEL_CLASSES)}
