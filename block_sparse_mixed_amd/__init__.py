"""Python binding of libda2 (DraftAttention2 hot path on MI355X).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. torch tensors supply device pointers and the current stream. The
functions mirror the C ABI in include/da2.h. The library is loaded on first
use (so that the build step can import this package before it exists); that
first call fails loudly when the library has not been built. There is no
fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libda2.so")

DA2_OK, DA2_ERR_INVALID_ARG, DA2_ERR_UNSUPPORTED, DA2_ERR_WORKSPACE, DA2_ERR_HIP = range(5)
DA2_OUT_BF16, DA2_OUT_FP32 = 0, 1
DA2_FLAG_PACK_EDGES = 1
DA2_SKIP, DA2_LO, DA2_HI = 0, 1, 2
TILE = 128
DPAD = 128


class Da2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {status_string(status)} (status {status})"
        if status == DA2_ERR_HIP:
            name = ctypes.c_char_p()
            code = _lib.da2_last_hip_error(ctypes.byref(name))
            msg += f": {name.value.decode()} ({code})"
        super().__init__(msg)
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("frames", ctypes.c_int32),
        ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("win_h", ctypes.c_int32), ("win_w", ctypes.c_int32),
        ("budget_hi", ctypes.c_double), ("budget_lo", ctypes.c_double), ("softmax_scale", ctypes.c_double),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64),
        ("out_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("out_stride_b", ctypes.c_int64), ("out_stride_h", ctypes.c_int64), ("out_stride_n", ctypes.c_int64),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("n_wy", ctypes.c_int32),
        ("n_wx", ctypes.c_int32), ("n_hi", ctypes.c_int32), ("n_lo", ctypes.c_int32),
        ("tokens", ctypes.c_int64), ("slots", ctypes.c_int64), ("tau", ctypes.c_double),
        ("workspace_bytes", ctypes.c_uint64),
    ] + [(n, ctypes.c_uint64) for n in (
        "off_pool", "off_k8", "off_v8t", "off_e8", "off_q4", "off_k4", "off_v4t",
        "off_sq4", "off_sk4", "off_sv4t", "off_scores", "off_labels", "off_hi", "off_lo", "off_status",
        "off_q8", "off_bias")] + [("n_full", ctypes.c_int32), ("flags", ctypes.c_uint32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


EXPORTS = ("da2_plan", "da2_plan_destroy", "da2_plan_info", "da2_prepare", "da2_attention",
           "da2_set_labels", "da2_forward_scratch", "da2_status_string", "da2_last_hip_error")
SCRATCH_BYTES = 256 << 20      # DA2_SCRATCH_BYTES


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_mixed_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.da2_plan.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(P)]
    lib.da2_plan.restype = ctypes.c_int
    lib.da2_plan_destroy.argtypes = [P]
    lib.da2_plan_destroy.restype = None
    lib.da2_plan_info.argtypes = [P, ctypes.POINTER(PlanInfo)]
    lib.da2_plan_info.restype = ctypes.c_int
    lib.da2_prepare.argtypes = [P, P, P, P, P, ctypes.c_size_t, P]
    lib.da2_prepare.restype = ctypes.c_int
    lib.da2_attention.argtypes = [P, P, ctypes.c_size_t, P, P]
    lib.da2_attention.restype = ctypes.c_int
    lib.da2_set_labels.argtypes = [P, P, ctypes.c_size_t, P, P]
    lib.da2_set_labels.restype = ctypes.c_int
    lib.da2_forward_scratch.argtypes = [P, P, P, P, P, P]
    lib.da2_forward_scratch.restype = ctypes.c_int
    lib.da2_status_string.argtypes = [ctypes.c_int]
    lib.da2_status_string.restype = ctypes.c_char_p
    lib.da2_last_hip_error.argtypes = [ctypes.POINTER(ctypes.c_char_p)]
    lib.da2_last_hip_error.restype = ctypes.c_int
    return lib


class _LazyLib:
    """libda2, opened on first attribute access."""
    _cdll = None

    def __getattr__(self, name):
        if _LazyLib._cdll is None:
            _LazyLib._cdll = _load()
        return getattr(_LazyLib._cdll, name)


_lib = _LazyLib()


def status_string(status: int) -> str:
    return _lib.da2_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != DA2_OK:
        raise Da2Error(status, where)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns a da2_plan_t. Construct with da2_plan(...)."""

    def __init__(self, handle: int, cfg: Config):
        self._h = ctypes.c_void_p(handle)
        self.cfg = cfg
        info = PlanInfo()
        _check(_lib.da2_plan_info(self._h, ctypes.byref(info)), "da2_plan_info")
        self.info = info

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h:
            _lib.da2_plan_destroy(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, device="cuda"):
        """A zeroed uint8 device buffer of workspace_bytes (torch's allocator aligns to >= 256 B)."""
        import torch
        ws = torch.zeros(int(self.info.workspace_bytes), dtype=torch.uint8, device=device)
        assert ws.data_ptr() % 256 == 0
        return ws


def make_config(batch, heads, frames, grid_h, grid_w, head_dim, win_h, win_w, budget_hi, budget_lo,
                softmax_scale=0.0, strides=(0, 0, 0), out_dtype=DA2_OUT_FP32, flags=0,
                out_strides=(0, 0, 0)) -> Config:
    return Config(batch, heads, frames, grid_h, grid_w, head_dim, win_h, win_w, float(budget_hi),
                  float(budget_lo), float(softmax_scale), int(strides[0]), int(strides[1]), int(strides[2]),
                  int(out_dtype), int(flags), int(out_strides[0]), int(out_strides[1]), int(out_strides[2]))


def da2_plan(cfg: Config) -> Plan:
    h = ctypes.c_void_p()
    _check(_lib.da2_plan(ctypes.byref(cfg), ctypes.byref(h)), "da2_plan")
    return Plan(h.value, cfg)


def _strides(plan: Plan, out: bool):
    """Element strides (b, h, n) the kernels use for q/k/v, or for out."""
    c = plan.cfg
    s = (c.stride_b, c.stride_h, c.stride_n)
    if out and (c.out_stride_b or c.out_stride_h or c.out_stride_n):
        s = (c.out_stride_b, c.out_stride_h, c.out_stride_n)
    if not any(s):
        n, d = int(plan.info.tokens), c.head_dim
        s = (c.heads * n * d, n * d, d)
    return s


def _check_tensor(t, what: str, dtypes, need_elems: int):
    """A tensor argument (raw integer pointers are passed on unchecked): its
    dtype, and that its storage holds the need_elems elements the kernels
    touch from its first element on."""
    if t is None or isinstance(t, int):
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{what}: dtype {t.dtype}, expected one of {tuple(str(x) for x in dtypes)}")
    avail = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    if need_elems * t.element_size() > avail:
        raise ValueError(f"{what}: the plan reaches {need_elems} elements from its start, its storage holds "
                         f"{avail // t.element_size()}")


def _check_on_gpu(**tensors):
    for what, t in tensors.items():
        if t is not None and not isinstance(t, int) and t.device.type != "cuda":
            raise ValueError(f"{what} must be on a GPU")


def _qkv_elems(plan: Plan, out: bool) -> int:
    c = plan.cfg
    sb, sh, sn = _strides(plan, out)
    return (c.batch - 1) * sb + (c.heads - 1) * sh + (int(plan.info.tokens) - 1) * sn + c.head_dim


def _check_inputs(plan: Plan, q, k, v):
    import torch
    n = _qkv_elems(plan, False)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name, (torch.bfloat16,), n)


def _check_out(plan: Plan, out):
    import torch
    dt = torch.float32 if plan.cfg.out_dtype == DA2_OUT_FP32 else torch.bfloat16
    _check_tensor(out, "out", (dt,), _qkv_elems(plan, True))


def _check_workspace(workspace):
    import torch
    _check_tensor(workspace, "workspace", (torch.uint8, torch.int8), 0)


# The enqueue calls check their tensor arguments (dtype, extent, device)
# before calling the library, which sees only pointers.
def da2_prepare(plan: Plan, q, k, v, workspace, stream=None):
    _check_inputs(plan, q, k, v)
    _check_workspace(workspace)
    _check_on_gpu(q=q, k=k, v=v, workspace=workspace)
    nbytes = workspace.numel() if hasattr(workspace, "numel") else int(plan.info.workspace_bytes)
    _check(_lib.da2_prepare(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(workspace), nbytes, _stream(stream)),
           "da2_prepare")


def da2_attention(plan: Plan, workspace, out, stream=None):
    _check_workspace(workspace)
    _check_out(plan, out)
    _check_on_gpu(workspace=workspace, out=out)
    nbytes = workspace.numel() if hasattr(workspace, "numel") else int(plan.info.workspace_bytes)
    _check(_lib.da2_attention(plan.handle, _ptr(workspace), nbytes, _ptr(out), _stream(stream)), "da2_attention")


def da2_set_labels(plan: Plan, workspace, labels, stream=None):
    import torch
    nb = int(plan.info.n_blocks)
    _check_workspace(workspace)
    _check_tensor(labels, "labels", (torch.int8,), plan.cfg.batch * plan.cfg.heads * nb * nb)
    _check_on_gpu(workspace=workspace, labels=labels)
    nbytes = workspace.numel() if hasattr(workspace, "numel") else int(plan.info.workspace_bytes)
    _check(_lib.da2_set_labels(plan.handle, _ptr(workspace), nbytes, _ptr(labels), _stream(stream)),
           "da2_set_labels")


def da2_forward_scratch(plan: Plan, q, k, v, out, stream=None):
    """da2_prepare + da2_attention on the library's static workspace (no allocation)."""
    _check_inputs(plan, q, k, v)
    _check_out(plan, out)
    _check_on_gpu(q=q, k=k, v=v, out=out)
    _check(_lib.da2_forward_scratch(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _stream(stream)),
           "da2_forward_scratch")


def workspace_section(plan: Plan, workspace, name: str, dtype, shape):
    """View of one workspace section (see include/da2.h) as a torch tensor."""
    import torch
    off = int(getattr(plan.info, "off_" + name))
    itemsize = torch.tensor([], dtype=dtype).element_size()
    n = 1
    for s in shape:
        n *= s
    return workspace[off:off + n * itemsize].view(dtype).view(*shape)


def attention(q, k, v, frames, grid_h, grid_w, win_h, win_w, budget_hi, budget_lo, softmax_scale=0.0,
              out_dtype=None, workspace=None, stream=None, flags=0):
    """Convenience wrapper: plan, prepare and attend for bf16 [B, H, N, d]
    tensors that share one set of strides with d contiguous (for example
    [B, N, H, d] storage viewed as [B, H, N, d], or slices of a fused QKV
    tensor). The output gets the same strides."""
    import torch
    B, H, N, d = q.shape
    st = tuple(q.stride())
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape")
    if N != frames * grid_h * grid_w:
        raise ValueError(f"q has {N} tokens, but a {frames} x {grid_h} x {grid_w} latent grid has "
                         f"{frames * grid_h * grid_w}")
    if tuple(k.stride()) != st or tuple(v.stride()) != st or st[3] != 1:
        raise ValueError("q, k and v must share their strides, with the last dimension contiguous")
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("q, k and v must be bfloat16")
    if out_dtype is None:
        out_dtype = torch.bfloat16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    if q.device.type != "cuda" or k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one GPU device")
    cfg = make_config(B, H, frames, grid_h, grid_w, d, win_h, win_w, budget_hi, budget_lo, softmax_scale,
                      strides=st[:3], out_dtype=DA2_OUT_FP32 if out_dtype == torch.float32 else DA2_OUT_BF16,
                      flags=flags)
    plan = da2_plan(cfg)
    ws = plan.workspace(q.device) if workspace is None else workspace
    out = torch.empty_strided((B, H, N, d), st, dtype=out_dtype, device=q.device)
    da2_prepare(plan, q, k, v, ws, stream)
    da2_attention(plan, ws, out, stream)
    return out
