"""Python binding of libaddrmsnorm_dq (fused (Add)RmsNorm + dynamic quantization).

Argument marshalling only: every step of the operator runs in the HIP
kernels of ``libaddrmsnorm_dq.so``.  torch supplies device memory and
streams.  The C functions are exposed under their own names (without the
``adq_`` prefix); ``add_rms_norm_dynamic_quant_v2`` and
``rms_norm_dynamic_quant`` additionally run both phases on torch tensors
and allocate the outputs.

The shared library is loaded on first use (``lib``); if it has not been
built, that raises ImportError: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libaddrmsnorm_dq.so")

# adq_dtype
F16, BF16, F32, INT8, INT4X2, INT32 = 1, 2, 3, 4, 5, 6
# adq_status
OK, ERR_NULLPTR, ERR_PARAM_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_RUNTIME = range(6)
STATUS_NAMES = {0: "ADQ_OK", 1: "ADQ_ERR_NULLPTR", 2: "ADQ_ERR_PARAM_INVALID",
                3: "ADQ_ERR_UNSUPPORTED", 4: "ADQ_ERR_WORKSPACE", 5: "ADQ_ERR_RUNTIME"}
# adq_path
PATH_AUTO, PATH_ROW, PATH_SPLIT, PATH_GENERIC = 0, 1, 2, 3
PATH_GEMM_TILE128, PATH_GEMM_TILE256, PATH_GEMM_TILE32 = 4, 5, 6
MAX_DIMS = 8

EXPORTED = (
    "adq_add_rms_norm_dynamic_quant_v2_get_workspace_size",
    "adq_add_rms_norm_dynamic_quant_v2",
    "adq_add_rms_norm_dynamic_quant_v2_no_alloc",
    "adq_rms_norm_dynamic_quant_get_workspace_size",
    "adq_rms_norm_dynamic_quant",
    "adq_w8a8_gemm_get_workspace_size",
    "adq_w8a8_gemm",
    "adq_add_lora_get_workspace_size",
    "adq_add_lora",
    "adq_executor_destroy",
    "adq_executor_set_path",
    "adq_executor_set_split",
    "adq_executor_describe",
    "adq_last_error",
)


class Tensor(ctypes.Structure):
    """adq_tensor: a contiguous row-major device tensor."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * MAX_DIMS)]


class SplitConfig(ctypes.Structure):
    """adq_split_config: split-row geometry (tests and tuning)."""
    _fields_ = [("splits", ctypes.c_int32), ("launches", ctypes.c_int32),
                ("wait_us", ctypes.c_int32), ("spread", ctypes.c_int32)]


class AdqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def _load():
    # torch ships its own HIP runtime with the same soname as ROCm's.  Load it
    # first so that this library binds to the runtime torch's tensors and
    # streams belong to; two runtimes in one process do not share devices.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with "
            "`python -m int4_dynamic_quantization_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Tensor)
    vp = ctypes.c_void_p
    u64p = ctypes.POINTER(ctypes.c_uint64)
    exp = ctypes.POINTER(vp)
    lib.adq_add_rms_norm_dynamic_quant_v2_get_workspace_size.argtypes = [
        P, P, P, P, P, P, ctypes.c_double, ctypes.POINTER(ctypes.c_bool), P, P, P, P, P, u64p,
        exp]
    lib.adq_add_rms_norm_dynamic_quant_v2.argtypes = [vp, ctypes.c_uint64, vp, vp]
    lib.adq_add_rms_norm_dynamic_quant_v2_no_alloc.argtypes = [vp, vp]
    lib.adq_rms_norm_dynamic_quant_get_workspace_size.argtypes = [
        P, P, P, P, ctypes.c_double, P, P, u64p, exp]
    lib.adq_rms_norm_dynamic_quant.argtypes = [vp, ctypes.c_uint64, vp, vp]
    lib.adq_w8a8_gemm_get_workspace_size.argtypes = [P, P, P, P, P, P, u64p, exp]
    lib.adq_w8a8_gemm.argtypes = [vp, ctypes.c_uint64, vp, vp]
    i64 = ctypes.c_int64
    lib.adq_add_lora_get_workspace_size.argtypes = [P, P, P, P, P, i64, ctypes.c_double, i64, i64,
                                                    P, u64p, exp]
    lib.adq_add_lora.argtypes = [vp, ctypes.c_uint64, vp, vp]
    lib.adq_executor_destroy.argtypes = [vp]
    lib.adq_executor_destroy.restype = None
    lib.adq_executor_set_path.argtypes = [vp, ctypes.c_int32, u64p]
    lib.adq_executor_set_split.argtypes = [vp, ctypes.POINTER(SplitConfig), u64p]
    lib.adq_executor_describe.argtypes = [vp, ctypes.c_char_p, ctypes.c_uint64]
    lib.adq_executor_describe.restype = ctypes.c_int32
    lib.adq_last_error.argtypes = []
    lib.adq_last_error.restype = ctypes.c_char_p
    for name in ("adq_add_rms_norm_dynamic_quant_v2_get_workspace_size",
                 "adq_add_rms_norm_dynamic_quant_v2",
                 "adq_add_rms_norm_dynamic_quant_v2_no_alloc",
                 "adq_rms_norm_dynamic_quant_get_workspace_size", "adq_rms_norm_dynamic_quant",
                 "adq_w8a8_gemm_get_workspace_size", "adq_w8a8_gemm",
                 "adq_add_lora_get_workspace_size", "adq_add_lora", "adq_executor_set_path",
                 "adq_executor_set_split"):
        getattr(lib, name).restype = ctypes.c_int
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime in this process: {runtimes}")
    return lib


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    # module attribute `lib`: the loaded C-ABI library (loaded on first use)
    if name == "lib":
        return _lib()
    raise AttributeError(name)


def last_error() -> str:
    return _lib().adq_last_error().decode()


def _check(status: int) -> None:
    if status != OK:
        raise AdqError(status, last_error())


# ---- torch <-> adq_tensor marshalling ------------------------------------

def _torch():
    import torch
    return torch


def describe_tensor(t, dtype: int | None = None, shape=None) -> Tensor:
    """adq_tensor for a torch tensor (dtype from torch unless given)."""
    torch = _torch()
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (row-major)")
    if dtype is None:
        dtype = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32,
                 torch.int8: INT8, torch.uint8: INT4X2, torch.int32: INT32}.get(t.dtype)
        if dtype is None:
            raise ValueError(f"unsupported torch dtype {t.dtype}")
    shape = tuple(t.shape) if shape is None else tuple(shape)
    if len(shape) > MAX_DIMS:
        raise ValueError("too many dimensions")
    d = Tensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = dtype
    d.ndim = len(shape)
    for i, s in enumerate(shape):
        d.shape[i] = int(s)
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


class Executor:
    """Owns an adq_executor; keeps the described tensors alive."""

    def __init__(self, handle: ctypes.c_void_p, workspace_size: int, op: str, keep):
        self.handle = handle
        self.workspace_size = int(workspace_size)
        self.op = op
        self._keep = keep
        self.device = None  # torch device of the tensors, when planned from torch tensors

    def set_path(self, path: int) -> int:
        ws = ctypes.c_uint64(0)
        _check(_lib().adq_executor_set_path(self.handle, int(path), ctypes.byref(ws)))
        self.workspace_size = int(ws.value)
        return self.workspace_size

    def set_split(self, splits: int = 0, launches: int = 0, wait_us: int = -1,
                  spread: bool = False) -> int:
        """Split-row path with `splits` chunks per row and the 1-, 2- or
        3-launch form (0 = the planner's choice), the one-launch form's wait
        budget and chunk placement; returns the new workspace size."""
        ws = ctypes.c_uint64(0)
        cfg = SplitConfig(int(splits), int(launches), int(wait_us), int(bool(spread)))
        _check(_lib().adq_executor_set_split(self.handle, ctypes.byref(cfg), ctypes.byref(ws)))
        self.workspace_size = int(ws.value)
        return self.workspace_size

    def describe(self) -> str:
        buf = ctypes.create_string_buffer(512)
        _lib().adq_executor_describe(self.handle, buf, len(buf))
        return buf.value.decode()

    def run(self, workspace=None, stream=None) -> None:
        """Phase 2 on `stream` (a torch.cuda.Stream); by default torch's
        current stream on the executor's device, so the launch is ordered
        with the surrounding torch work (and can be captured in a graph)."""
        ws_ptr = None if workspace is None else workspace.data_ptr()
        ws_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if stream is None:
            stream = _torch().cuda.current_stream(self.device)
        s = stream.cuda_stream
        fn = {"v2": _lib().adq_add_rms_norm_dynamic_quant_v2,
              "rmsnorm": _lib().adq_rms_norm_dynamic_quant,
              "gemm": _lib().adq_w8a8_gemm, "lora": _lib().adq_add_lora}[self.op]
        _check(fn(ws_ptr, ws_size, self.handle, s))

    def run_no_alloc(self, stream=None) -> None:
        """AddRmsNormDynamicQuantV2 phase 2 without a workspace: the library's
        static scratch buffer of the device takes the split-row path's
        partial results (calls on one device must not overlap)."""
        if self.op != "v2":
            raise ValueError("only AddRmsNormDynamicQuantV2 executors run without a workspace")
        if stream is None:
            stream = _torch().cuda.current_stream(self.device)
        _check(_lib().adq_add_rms_norm_dynamic_quant_v2_no_alloc(self.handle, stream.cuda_stream))

    def close(self) -> None:
        if self.handle:
            _lib().adq_executor_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def add_rms_norm_dynamic_quant_v2_get_workspace_size(
        x1, x2, gamma, beta, smooth_scale1, smooth_scale2, epsilon, output_mask, y1_out, y2_out,
        scale1_out, scale2_out, x_out) -> Executor:
    """Phase 1 on adq_tensor descriptors (or None); returns an Executor."""
    mask = None
    if output_mask is not None:
        mask = (ctypes.c_bool * 2)(bool(output_mask[0]), bool(output_mask[1]))
    ws = ctypes.c_uint64(0)
    handle = ctypes.c_void_p(None)
    descs = (x1, x2, gamma, beta, smooth_scale1, smooth_scale2, y1_out, y2_out, scale1_out,
             scale2_out, x_out)
    _check(_lib().adq_add_rms_norm_dynamic_quant_v2_get_workspace_size(
        _ref(x1), _ref(x2), _ref(gamma), _ref(beta), _ref(smooth_scale1), _ref(smooth_scale2),
        float(epsilon), mask, _ref(y1_out), _ref(y2_out), _ref(scale1_out), _ref(scale2_out),
        _ref(x_out), ctypes.byref(ws), ctypes.byref(handle)))
    return Executor(handle, ws.value, "v2", descs)


def rms_norm_dynamic_quant_get_workspace_size(x, gamma, beta, smooth_scales, epsilon, y_out,
                                              scale_out) -> Executor:
    ws = ctypes.c_uint64(0)
    handle = ctypes.c_void_p(None)
    descs = (x, gamma, beta, smooth_scales, y_out, scale_out)
    _check(_lib().adq_rms_norm_dynamic_quant_get_workspace_size(
        _ref(x), _ref(gamma), _ref(beta), _ref(smooth_scales), float(epsilon), _ref(y_out),
        _ref(scale_out), ctypes.byref(ws), ctypes.byref(handle)))
    return Executor(handle, ws.value, "rmsnorm", descs)


# ---- torch-level convenience (allocation + both phases) -------------------

def _quant_out(x, qtype: str):
    torch = _torch()
    lead = tuple(x.shape[:-1])
    n = x.shape[-1]
    if qtype == "int8":
        return torch.empty(lead + (n,), dtype=torch.int8, device=x.device), INT8
    if qtype == "int4":
        return torch.empty(lead + (n // 2,), dtype=torch.uint8, device=x.device), INT4X2
    raise ValueError("quantized output type must be 'int8' or 'int4'")


def plan_add_rms_norm_dynamic_quant_v2(x1, x2, gamma, beta=None, smooth_scale1=None,
                                       smooth_scale2=None, epsilon=1e-6, output_mask=None,
                                       y1_type="int8", y2_type="int8", outputs=None,
                                       path=PATH_AUTO):
    """Allocate outputs (unless given) and run phase 1.

    Returns (executor, outputs dict with x_out, y1, scale1, y2, scale2; an
    output that the call does not produce is None unless passed in)."""
    torch = _torch()
    lead = tuple(x1.shape[:-1])
    outs = dict(outputs or {})
    if "x_out" not in outs:
        outs["x_out"] = torch.empty_like(x1)
    want1 = output_mask[0] if output_mask is not None else True
    want2 = (output_mask[1] if output_mask is not None
             else (smooth_scale1 is not None and smooth_scale2 is not None))
    qd = {}
    for k, want, qt in ((1, want1, y1_type), (2, want2, y2_type)):
        if f"y{k}" not in outs:
            outs[f"y{k}"], qd[k] = _quant_out(x1, qt) if want else (None, None)
        else:
            qd[k] = INT4X2 if qt == "int4" else INT8
        if f"scale{k}" not in outs:
            outs[f"scale{k}"] = (torch.empty(lead, dtype=torch.float32, device=x1.device)
                                 if want else None)
    d = describe_tensor
    ex = add_rms_norm_dynamic_quant_v2_get_workspace_size(
        d(x1), d(x2), d(gamma), d(beta), d(smooth_scale1), d(smooth_scale2), epsilon,
        output_mask, None if outs["y1"] is None else d(outs["y1"], qd[1]),
        None if outs["y2"] is None else d(outs["y2"], qd[2]), d(outs["scale1"]),
        d(outs["scale2"]), d(outs["x_out"]))
    ex._keep = (ex._keep, x1, x2, gamma, beta, smooth_scale1, smooth_scale2, outs)
    ex.device = x1.device
    if path != PATH_AUTO:
        ex.set_path(path)
    return ex, outs


def _workspace(ex, device):
    if ex.workspace_size == 0:
        return None
    torch = _torch()
    return torch.empty(ex.workspace_size, dtype=torch.uint8, device=device)


def _run_once(ex, device, stream, made):
    """Phase 2 with a workspace allocated here.  The workspace and the
    tensors in `made` (allocated here, on torch's current stream) are marked
    as used on the launch stream, so that torch's caching allocator does not
    hand their memory out again before the launched work has finished when
    that stream is not the current one."""
    ws = _workspace(ex, device)
    ex.run(ws, stream)
    if stream is not None:
        for t in [ws] + list(made):
            if t is not None:
                t.record_stream(stream)
    ex.close()


def add_rms_norm_dynamic_quant_v2(x1, x2, gamma, beta=None, smooth_scale1=None,
                                  smooth_scale2=None, epsilon=1e-6, output_mask=None,
                                  y1_type="int8", y2_type="int8", stream=None, path=PATH_AUTO):
    """Both phases on torch tensors; returns (y1, y2, scale1, scale2, x_out)."""
    ex, outs = plan_add_rms_norm_dynamic_quant_v2(
        x1, x2, gamma, beta, smooth_scale1, smooth_scale2, epsilon, output_mask, y1_type,
        y2_type, path=path)
    _run_once(ex, x1.device, stream, outs.values())
    return outs["y1"], outs["y2"], outs["scale1"], outs["scale2"], outs["x_out"]


def plan_rms_norm_dynamic_quant(x, gamma, beta=None, smooth_scales=None, epsilon=1e-6,
                                y_type="int8", outputs=None, path=PATH_AUTO):
    torch = _torch()
    outs = dict(outputs or {})
    if "y" not in outs:
        outs["y"], qd = _quant_out(x, y_type)
    else:
        qd = INT4X2 if y_type == "int4" else INT8
    if "scale" not in outs:
        outs["scale"] = torch.empty(tuple(x.shape[:-1]), dtype=torch.float32, device=x.device)
    d = describe_tensor
    ex = rms_norm_dynamic_quant_get_workspace_size(
        d(x), d(gamma), d(beta), d(smooth_scales), epsilon, d(outs["y"], qd), d(outs["scale"]))
    ex._keep = (ex._keep, x, gamma, beta, smooth_scales, outs)
    ex.device = x.device
    if path != PATH_AUTO:
        ex.set_path(path)
    return ex, outs


def rms_norm_dynamic_quant(x, gamma, beta=None, smooth_scales=None, epsilon=1e-6,
                           y_type="int8", stream=None, path=PATH_AUTO):
    """Both phases on torch tensors; returns (y, scale)."""
    ex, outs = plan_rms_norm_dynamic_quant(x, gamma, beta, smooth_scales, epsilon, y_type,
                                           path=path)
    _run_once(ex, x.device, stream, outs.values())
    return outs["y"], outs["scale"]


def w8a8_gemm_get_workspace_size(a, a_scale, w, w_scale, bias, out) -> Executor:
    """GEMM phase 1 on adq_tensor descriptors (bias may be None)."""
    ws = ctypes.c_uint64(0)
    handle = ctypes.c_void_p(None)
    _check(_lib().adq_w8a8_gemm_get_workspace_size(
        _ref(a), _ref(a_scale), _ref(w), _ref(w_scale), _ref(bias), _ref(out), ctypes.byref(ws),
        ctypes.byref(handle)))
    return Executor(handle, ws.value, "gemm", (a, a_scale, w, w_scale, bias, out))


def plan_w8a8_gemm(a, a_scale, w, w_scale, bias=None, out_dtype=None, out=None,
                   path=PATH_AUTO):
    """Allocate out (unless given) and run GEMM phase 1 on torch tensors:
    a int8 [..., k], a_scale float32 (one per row), w int8 [n, k],
    w_scale float32 [n], bias float32 [n] or None.  `path` may force a tile
    size (PATH_GEMM_TILE128 / PATH_GEMM_TILE256 / PATH_GEMM_TILE32)."""
    torch = _torch()
    if out is None:
        out = torch.empty(tuple(a.shape[:-1]) + (w.shape[0],),
                          dtype=out_dtype or torch.bfloat16, device=a.device)
    d = describe_tensor
    ex = w8a8_gemm_get_workspace_size(d(a, INT8), d(a_scale), d(w, INT8), d(w_scale), d(bias),
                                      d(out))
    ex._keep = (ex._keep, a, a_scale, w, w_scale, bias, out)
    ex.device = a.device
    if path != PATH_AUTO:
        ex.set_path(path)
    return ex, out


def w8a8_gemm(a, a_scale, w, w_scale, bias=None, out_dtype=None, stream=None):
    """Both GEMM phases on torch tensors; returns out."""
    ex, out = plan_w8a8_gemm(a, a_scale, w, w_scale, bias, out_dtype)
    _run_once(ex, a.device, stream, [out])
    return out


def add_lora_get_workspace_size(y, x, weight_b, indices, weight_a, layer_idx, scale, y_offset,
                                y_slice_size, out) -> Executor:
    """AddLora phase 1 on adq_tensor descriptors (weight_a may be None)."""
    ws = ctypes.c_uint64(0)
    handle = ctypes.c_void_p(None)
    _check(_lib().adq_add_lora_get_workspace_size(
        _ref(y), _ref(x), _ref(weight_b), _ref(indices), _ref(weight_a), int(layer_idx),
        float(scale), int(y_offset), int(y_slice_size), _ref(out), ctypes.byref(ws),
        ctypes.byref(handle)))
    return Executor(handle, ws.value, "lora", (y, x, weight_b, indices, weight_a, out))


def plan_add_lora(y, x, weight_b, indices, weight_a=None, layer_idx=0, scale=1.0, y_offset=0,
                  out=None, path=PATH_AUTO):
    """AddLora phase 1 on torch tensors.  out=None allocates a new tensor;
    pass out=y to accumulate in place."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(y)
    d = describe_tensor
    ex = add_lora_get_workspace_size(d(y), d(x), d(weight_b), d(indices), d(weight_a), layer_idx,
                                     scale, y_offset, weight_b.shape[-1], d(out))
    ex._keep = (ex._keep, y, x, weight_b, indices, weight_a, out)
    ex.device = y.device
    if path != PATH_AUTO:
        ex.set_path(path)
    return ex, out


def add_lora(y, x, weight_b, indices, weight_a=None, layer_idx=0, scale=1.0, y_offset=0,
             out=None, stream=None):
    """Both AddLora phases on torch tensors (workspace allocated here); returns out."""
    allocated = out is None
    ex, out = plan_add_lora(y, x, weight_b, indices, weight_a, layer_idx, scale, y_offset, out)
    _run_once(ex, y.device, stream, [out] if allocated else [])
    return out
