"""Python binding of the gfx950 Q4_K SwiGLU MLP library (``include/zinc_mlp.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``_lib/libzinc_mlp.so``.  PyTorch supplies device memory and the
current HIP stream.  If the library has not been built this module raises on
import -- there is no CPU fallback.

Functions carry the C entry points' names and take torch tensors:

* ``zinc_q4k_dequant_f32(blocks, rows, cols)`` -> fp32 ``[rows, cols]``
* ``zinc_mlp_q4k_prefill(w_gate, w_up, w_down, hidden, inter, x, ...)`` -> fp16 y
* ``zinc_mlp_q4k_prefill_block`` / ``zinc_mlp_q4k_decode_block(..., x, norm_weight, eps, mlp_scale, ...)``
  -> fp16 y = x + mlp_scale * MLP(rms_norm(x)) (pre-MLP norm and residual folded in)
* ``zinc_mlp_q4k_prefill_staged(...)`` -> fp16 y (comparison baseline, intermediate in device memory)
* ``zinc_mlp_q4k_decode(...)`` (1 <= M <= 8) -> fp16 y
* ``zinc_moe_q4k_experts(w_gate, w_up, w_down, n_experts, hidden, inter, x, ids, p, ...)`` -> fp16 y
* ``zinc_moe_route_topk(logits, top_k)`` -> (int32 ids, fp32 weights), both on the GPU

Q4_K weights are uint8 tensors holding the raw 144-byte blocks ([rows,
cols/256, 144] or flat); x is fp16 ``[M, hidden]``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libzinc_mlp.so")

ZINC_OK = 0
STATUS_NAMES = {
    0: "ZINC_OK", -1: "ZINC_ERR_NULL", -2: "ZINC_ERR_SHAPE", -3: "ZINC_ERR_ALIGN",
    -4: "ZINC_ERR_WORKSPACE", -5: "ZINC_ERR_ARG", -6: "ZINC_ERR_HIP", -7: "ZINC_ERR_UNSUPPORTED",
}

EXPORTS = (
    "zinc_strerror",
    "zinc_hip_error_string",
    "zinc_q4k_dequant_f32",
    "zinc_q5k_dequant_f32",
    "zinc_q5_1_dequant_f32",
    "zinc_mlp_q4k_prefill_workspace_size",
    "zinc_mlp_q4k_prefill",
    "zinc_mlp_q4k_prefill_block_workspace_size",
    "zinc_mlp_q4k_prefill_block",
    "zinc_mlp_q4k_decode_block_workspace_size",
    "zinc_mlp_q4k_decode_block",
    "zinc_mlp_q4k_prefill_staged_workspace_size",
    "zinc_mlp_q4k_prefill_staged",
    "zinc_mlp_q4k_decode_workspace_size",
    "zinc_mlp_q4k_decode",
    "zinc_mlp_q4k_decode_noalloc_max_bytes",
    "zinc_mlp_q4k_decode_noalloc",
    "zinc_moe_q4k_experts_workspace_size",
    "zinc_moe_q4k_experts",
    "zinc_moe_experts_fmt",
    "zinc_moe_route_topk",
    "zinc_timing_enable",
    "zinc_timing_collect",
    "zinc_timing_disable",
)


class ZincError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS_NAMES.get(status, status)} ({strerror(status)})"
        if status == -6:
            msg += f": {lib.zinc_hip_error_string().decode()}"
        super().__init__(msg)


def _load() -> ctypes.CDLL:
    # torch bundles its own HIP runtime with the same soname as /opt/rocm's.
    # Importing torch first makes the library bind to that already-loaded
    # runtime; otherwise the process would hold two HIP runtimes and torch's
    # streams and allocations would be foreign to the library's launches.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python q4_swiglu_mlp_amd/build.py, or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.zinc_strerror.restype = ctypes.c_char_p
    lib.zinc_strerror.argtypes = [ctypes.c_int]
    lib.zinc_hip_error_string.restype = ctypes.c_char_p
    lib.zinc_hip_error_string.argtypes = []
    lib.zinc_q4k_dequant_f32.restype = ctypes.c_int
    lib.zinc_q4k_dequant_f32.argtypes = [P, I32, I32, P, P]
    for name in ("zinc_q5k_dequant_f32", "zinc_q5_1_dequant_f32"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [P, I32, I32, P, P]
    for name in ("zinc_mlp_q4k_prefill_workspace_size", "zinc_mlp_q4k_prefill_staged_workspace_size",
                 "zinc_mlp_q4k_decode_workspace_size", "zinc_mlp_q4k_prefill_block_workspace_size",
                 "zinc_mlp_q4k_decode_block_workspace_size"):
        fn = getattr(lib, name)
        fn.restype = SZ
        fn.argtypes = [I32, I32, I32]
    for name in ("zinc_mlp_q4k_prefill", "zinc_mlp_q4k_prefill_staged", "zinc_mlp_q4k_decode"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, P, P, I32, I32, P, P, I32, I32, I32, P, SZ, P]
    F32 = ctypes.c_float
    for name in ("zinc_mlp_q4k_prefill_block", "zinc_mlp_q4k_decode_block"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, P, P, I32, I32, P, P, F32, F32, P, I32, I32, I32, P, SZ, P]
    lib.zinc_mlp_q4k_decode_noalloc_max_bytes.restype = SZ
    lib.zinc_mlp_q4k_decode_noalloc_max_bytes.argtypes = []
    lib.zinc_mlp_q4k_decode_noalloc.restype = ctypes.c_int
    lib.zinc_mlp_q4k_decode_noalloc.argtypes = [P, P, P, I32, I32, P, P, I32, I32, I32, P]
    lib.zinc_moe_q4k_experts_workspace_size.restype = SZ
    lib.zinc_moe_q4k_experts_workspace_size.argtypes = [I32, I32, I32, I32, I32]
    lib.zinc_moe_q4k_experts.restype = ctypes.c_int
    lib.zinc_moe_q4k_experts.argtypes = [P, P, P, I32, I32, I32, P, I32, P, P, I32, P, I32, I32, P, SZ, P, P]
    lib.zinc_moe_experts_fmt.restype = ctypes.c_int
    lib.zinc_moe_experts_fmt.argtypes = [P, P, P, I32, I32, I32, I32, P, I32, P, P, I32, P, I32, I32, P, SZ, P, P]
    lib.zinc_moe_route_topk.restype = ctypes.c_int
    lib.zinc_moe_route_topk.argtypes = [P, I32, I32, I32, P, P, P]
    lib.zinc_timing_enable.restype = ctypes.c_int
    lib.zinc_timing_enable.argtypes = [I32]
    lib.zinc_timing_collect.restype = ctypes.c_int
    lib.zinc_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_float), I32, ctypes.POINTER(ctypes.c_int32)]
    lib.zinc_timing_disable.restype = None
    lib.zinc_timing_disable.argtypes = []
    return lib


lib = _load()


def timing_enable(capacity: int) -> None:
    """Record a HIP event pair around the main kernel(s) of each following call."""
    _check(lib.zinc_timing_enable(capacity), "zinc_timing_enable")


def timing_collect(capacity: int) -> list[float]:
    """Wait for the recorded launches; their kernel durations in milliseconds."""
    buf = (ctypes.c_float * capacity)()
    n = ctypes.c_int32(0)
    _check(lib.zinc_timing_collect(buf, capacity, ctypes.byref(n)), "zinc_timing_collect")
    return [float(buf[i]) for i in range(n.value)]


def timing_disable() -> None:
    lib.zinc_timing_disable()


def strerror(status: int) -> str:
    return lib.zinc_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != ZINC_OK:
        raise ZincError(status, where)


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------
# The C ABI sees only pointers, so the wrappers check every tensor's dtype,
# shape and byte size against the sizes the call will read or write before
# handing its pointer over: a mismatch raises ValueError and nothing is
# launched.  Checks on content come first and the device check last, so the
# content checks also run (and are tested) on a machine without a GPU.
# Temporaries (y, the workspace) are allocated on the stream the call is
# enqueued on, so the caching allocator does not hand their memory to other
# work while that stream still uses it.
def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


Q4K_BYTES, Q5K_BYTES, Q51_BYTES = 144, 176, 24


def q4k_matrix_bytes(rows: int, cols: int) -> int:
    """Bytes of a Q4_K matrix [rows x cols]: rows * cols/256 blocks of 144 bytes."""
    return rows * (cols // 256) * Q4K_BYTES


def down_matrix_bytes(fmt: str, rows: int, cols: int) -> int:
    """Bytes of a [rows x cols] W_down in the named block format."""
    if fmt == "q4_k":
        return q4k_matrix_bytes(rows, cols)
    if fmt == "q5_k":
        return rows * (cols // 256) * Q5K_BYTES
    if fmt == "q5_1":
        return rows * (cols // 32) * Q51_BYTES
    raise ValueError(f"unknown down format {fmt!r} (q4_k, q5_k or q5_1)")


def _nbytes(t) -> int:
    return int(t.numel()) * int(t.element_size())


def _need_bytes(t, want: int, what: str) -> None:
    if t is None:
        raise ValueError(f"{what} is required")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if _nbytes(t) != want:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call reads {want}")


def _need(t, dtype, shape, what: str) -> None:
    """t must be a contiguous tensor of `dtype` and exactly `shape`."""
    if t is None:
        raise ValueError(f"{what} is required")
    if t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _activation(x, hidden: int, what: str = "x") -> int:
    torch = _torch()
    if x is None or x.dim() != 2:
        raise ValueError(f"{what} must be a 2-D float16 [M, hidden] tensor")
    _need(x, torch.float16, (int(x.shape[0]), hidden), what)
    return int(x.shape[0])


def _workspace(ws, need: int) -> None:
    if ws is None:
        return
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if _nbytes(ws) < need:
        raise ValueError(f"workspace holds {_nbytes(ws)} bytes, the call needs {need}")


def _on_gpu(*tensors) -> None:
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"all tensors must be on one device ({dev} and {t.device})")


def _resolve_stream(stream, device):
    """The torch stream the call is enqueued on: the current stream of
    `device` by default; an int is taken as a raw hipStream_t handle."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def _empty_on(stream, *args, **kw):
    """torch.empty allocated on `stream` (the allocator then keeps the block
    for that stream's work)."""
    torch = _torch()
    with torch.cuda.stream(stream):
        return torch.empty(*args, **kw)


def zinc_q4k_dequant_f32(blocks, rows: int, cols: int, out=None, stream=None):
    torch = _torch()
    if cols <= 0 or cols % 256 or rows < 0:
        raise ValueError("cols must be a positive multiple of 256 and rows >= 0")
    _need_bytes(blocks, q4k_matrix_bytes(rows, cols), "blocks")
    if out is not None:
        _need(out, torch.float32, (rows, cols), "out")
    _on_gpu(blocks, out)
    s = _resolve_stream(stream, blocks.device)
    if out is None:
        out = _empty_on(s, (rows, cols), dtype=torch.float32, device=blocks.device)
    _check(lib.zinc_q4k_dequant_f32(_ptr(blocks), rows, cols, _ptr(out), s.cuda_stream), "zinc_q4k_dequant_f32")
    return out


def zinc_q5_dequant_f32(fmt: str, blocks, rows: int, cols: int, out=None, stream=None):
    """The fp32 weights of a Q5_K (``fmt="q5_k"``) or Q5_1 (``"q5_1"``) matrix."""
    torch = _torch()
    if fmt not in ("q5_k", "q5_1"):
        raise ValueError(f"unknown format {fmt!r} (q5_k or q5_1)")
    unit = 256 if fmt == "q5_k" else 32
    if cols <= 0 or cols % unit or rows < 0:
        raise ValueError(f"cols must be a positive multiple of {unit} and rows >= 0")
    _need_bytes(blocks, down_matrix_bytes(fmt, rows, cols), "blocks")
    if out is not None:
        _need(out, torch.float32, (rows, cols), "out")
    _on_gpu(blocks, out)
    s = _resolve_stream(stream, blocks.device)
    if out is None:
        out = _empty_on(s, (rows, cols), dtype=torch.float32, device=blocks.device)
    name = {"q5_k": "zinc_q5k_dequant_f32", "q5_1": "zinc_q5_1_dequant_f32"}[fmt]
    _check(getattr(lib, name)(_ptr(blocks), rows, cols, _ptr(out), s.cuda_stream), name)
    return out


def prefill_workspace_size(M: int, hidden: int, inter: int) -> int:
    return int(lib.zinc_mlp_q4k_prefill_workspace_size(M, hidden, inter))


def prefill_staged_workspace_size(M: int, hidden: int, inter: int) -> int:
    return int(lib.zinc_mlp_q4k_prefill_staged_workspace_size(M, hidden, inter))


def decode_workspace_size(M: int, hidden: int, inter: int) -> int:
    return int(lib.zinc_mlp_q4k_decode_workspace_size(M, hidden, inter))


def moe_workspace_size(M: int, top_k: int, n_experts: int, hidden: int, inter: int) -> int:
    return int(lib.zinc_moe_q4k_experts_workspace_size(M, top_k, n_experts, hidden, inter))


def _dense_weights(w_gate, w_up, w_down, hidden: int, inter: int, n_experts: int = 1, down_fmt: str = "q4_k"):
    if hidden <= 0 or hidden % 256 or inter <= 0 or inter % 256:
        raise ValueError("hidden and inter must be positive multiples of 256")
    _need_bytes(w_gate, n_experts * q4k_matrix_bytes(inter, hidden), "w_gate")
    _need_bytes(w_up, n_experts * q4k_matrix_bytes(inter, hidden), "w_up")
    _need_bytes(w_down, n_experts * down_matrix_bytes(down_fmt, hidden, inter), "w_down")


def _dense(fn_name: str, ws_fn, w_gate, w_up, w_down, hidden, inter, x, inter_shift, out_shift, y, workspace,
           stream):
    torch = _torch()
    _dense_weights(w_gate, w_up, w_down, hidden, inter)
    M = _activation(x, hidden)
    if y is not None:
        _need(y, torch.float16, (M, hidden), "y")
    need = int(ws_fn(M, hidden, inter))
    _workspace(workspace, need)
    _on_gpu(w_gate, w_up, w_down, x, y, workspace)
    s = _resolve_stream(stream, x.device)
    if y is None:
        y = _empty_on(s, (M, hidden), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = _empty_on(s, max(need, 16), dtype=torch.uint8, device=x.device)
    st = getattr(lib, fn_name)(_ptr(w_gate), _ptr(w_up), _ptr(w_down), hidden, inter, _ptr(x), _ptr(y), M,
                               inter_shift, out_shift, _ptr(workspace), _nbytes(workspace), s.cuda_stream)
    _check(st, fn_name)
    return y


def zinc_mlp_q4k_prefill(w_gate, w_up, w_down, hidden: int, inter: int, x, inter_shift: int = 0, out_shift: int = 0,
                         y=None, workspace=None, stream=None):
    """y = fp16(MLP(x) * 2^-out_shift) for fp16 x [M, hidden]; fused prefill kernel."""
    return _dense("zinc_mlp_q4k_prefill", prefill_workspace_size, w_gate, w_up, w_down, hidden, inter, x,
                  inter_shift, out_shift, y, workspace, stream)


def _block(fn_name: str, ws_name: str, w_gate, w_up, w_down, hidden, inter, x, norm_weight, norm_eps, mlp_scale,
           inter_shift, out_shift, y, workspace, stream):
    torch = _torch()
    _dense_weights(w_gate, w_up, w_down, hidden, inter)
    M = _activation(x, hidden)
    _need(norm_weight, torch.float16, (hidden,), "norm_weight")
    if y is not None:
        _need(y, torch.float16, (M, hidden), "y")
    need = int(getattr(lib, ws_name)(M, hidden, inter))
    _workspace(workspace, need)
    _on_gpu(w_gate, w_up, w_down, x, norm_weight, y, workspace)
    s = _resolve_stream(stream, x.device)
    if y is None:
        y = _empty_on(s, (M, hidden), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = _empty_on(s, max(need, 16), dtype=torch.uint8, device=x.device)
    st = getattr(lib, fn_name)(_ptr(w_gate), _ptr(w_up), _ptr(w_down), hidden, inter, _ptr(x), _ptr(norm_weight),
                               float(norm_eps), float(mlp_scale), _ptr(y), M, inter_shift, out_shift, _ptr(workspace),
                               _nbytes(workspace), s.cuda_stream)
    _check(st, fn_name)
    return y


def zinc_mlp_q4k_prefill_block(w_gate, w_up, w_down, hidden: int, inter: int, x, norm_weight, norm_eps: float,
                               mlp_scale: float = 1.0, inter_shift: int = 0, out_shift: int = 0, y=None,
                               workspace=None, stream=None):
    """y = fp16((x + mlp_scale * MLP(rms_norm(x) * norm_weight)) * 2^-out_shift); ``y`` may be ``x``."""
    return _block("zinc_mlp_q4k_prefill_block", "zinc_mlp_q4k_prefill_block_workspace_size", w_gate, w_up, w_down,
                  hidden, inter, x, norm_weight, norm_eps, mlp_scale, inter_shift, out_shift, y, workspace, stream)


def zinc_mlp_q4k_decode_block(w_gate, w_up, w_down, hidden: int, inter: int, x, norm_weight, norm_eps: float,
                              mlp_scale: float = 1.0, inter_shift: int = 0, out_shift: int = 0, y=None,
                              workspace=None, stream=None):
    """The decode form (1 <= M <= 8) of zinc_mlp_q4k_prefill_block."""
    return _block("zinc_mlp_q4k_decode_block", "zinc_mlp_q4k_decode_block_workspace_size", w_gate, w_up, w_down,
                  hidden, inter, x, norm_weight, norm_eps, mlp_scale, inter_shift, out_shift, y, workspace, stream)


def zinc_mlp_q4k_prefill_staged(w_gate, w_up, w_down, hidden: int, inter: int, x, inter_shift: int = 0,
                                out_shift: int = 0, y=None, workspace=None, stream=None):
    """The prefill's staged comparison baseline (intermediate in device memory); same y."""
    return _dense("zinc_mlp_q4k_prefill_staged", prefill_staged_workspace_size, w_gate, w_up, w_down, hidden, inter,
                  x, inter_shift, out_shift, y, workspace, stream)


def zinc_mlp_q4k_decode(w_gate, w_up, w_down, hidden: int, inter: int, x, inter_shift: int = 0, out_shift: int = 0,
                        y=None, workspace=None, stream=None):
    """Same result as the prefill entry point for 1 <= M <= 8, via HBM-bound matvecs."""
    return _dense("zinc_mlp_q4k_decode", decode_workspace_size, w_gate, w_up, w_down, hidden, inter, x, inter_shift,
                  out_shift, y, workspace, stream)


def zinc_mlp_q4k_decode_noalloc(w_gate, w_up, w_down, hidden: int, inter: int, x, y, inter_shift: int = 0,
                                out_shift: int = 0, stream=None):
    """zinc_mlp_q4k_decode with the intermediate in the library's own device
    array: nothing is allocated, so ``y`` (fp16 [M, hidden]) is required.
    Calls that overlap in time on one GPU race on that array."""
    torch = _torch()
    _dense_weights(w_gate, w_up, w_down, hidden, inter)
    M = _activation(x, hidden)
    _need(y, torch.float16, (M, hidden), "y")
    _on_gpu(w_gate, w_up, w_down, x, y)
    s = _resolve_stream(stream, x.device)
    st = lib.zinc_mlp_q4k_decode_noalloc(_ptr(w_gate), _ptr(w_up), _ptr(w_down), hidden, inter, _ptr(x), _ptr(y), M,
                                         inter_shift, out_shift, s.cuda_stream)
    _check(st, "zinc_mlp_q4k_decode_noalloc")
    return y


DOWN_FORMATS = {"q4_k": 0, "q5_k": 1, "q5_1": 2}


def _moe_routing(expert_ids, expert_weights, M: int):
    torch = _torch()
    if expert_ids is None or expert_ids.dim() != 2:
        raise ValueError("expert_ids must be a 2-D int32 [M, top_k] tensor")
    top_k = int(expert_ids.shape[1])
    _need(expert_ids, torch.int32, (M, top_k), "expert_ids")
    _need(expert_weights, torch.float32, (M, top_k), "expert_weights")
    return top_k


def zinc_moe_experts_fmt(w_gate, w_up, w_down, down_format: str, n_experts: int, hidden: int, inter: int, x,
                         expert_ids, expert_weights, inter_shift: int = 0, out_shift: int = 0, y=None,
                         workspace=None, dev_error=None, stream=None):
    """The batched-expert call with W_down in ``down_format`` ("q4_k", "q5_k" or "q5_1")."""
    torch = _torch()
    if down_format not in DOWN_FORMATS:
        raise ValueError(f"unknown down format {down_format!r} (q4_k, q5_k or q5_1)")
    if n_experts < 1:
        raise ValueError("n_experts must be >= 1")
    _dense_weights(w_gate, w_up, w_down, hidden, inter, n_experts, down_format)
    M = _activation(x, hidden)
    top_k = _moe_routing(expert_ids, expert_weights, M)
    if y is not None:
        _need(y, torch.float16, (M, hidden), "y")
    if dev_error is not None and (dev_error.dtype != torch.int32 or dev_error.numel() < 1):
        raise ValueError("dev_error must be an int32 tensor of at least one element")
    need = moe_workspace_size(M, top_k, n_experts, hidden, inter)
    _workspace(workspace, need)
    _on_gpu(w_gate, w_up, w_down, x, expert_ids, expert_weights, y, workspace, dev_error)
    s = _resolve_stream(stream, x.device)
    if y is None:
        y = _empty_on(s, (M, hidden), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = _empty_on(s, max(need, 16), dtype=torch.uint8, device=x.device)
    st = lib.zinc_moe_experts_fmt(_ptr(w_gate), _ptr(w_up), _ptr(w_down), DOWN_FORMATS[down_format], n_experts,
                                  hidden, inter, _ptr(x), M, _ptr(expert_ids), _ptr(expert_weights), top_k, _ptr(y),
                                  inter_shift, out_shift, _ptr(workspace), _nbytes(workspace), _ptr(dev_error),
                                  s.cuda_stream)
    _check(st, "zinc_moe_experts_fmt")
    return y


def zinc_moe_q4k_experts(w_gate, w_up, w_down, n_experts: int, hidden: int, inter: int, x, expert_ids,
                         expert_weights, inter_shift: int = 0, out_shift: int = 0, y=None, workspace=None,
                         dev_error=None, stream=None):
    """y[t] = sum_s p[t,s] * MLP_{ids[t,s]}(x[t]) with ids/p read on the GPU.
    ``expert_ids`` int32 [M, top_k] (not torch.topk's int64), ``expert_weights``
    float32 [M, top_k]; this calls the C entry point zinc_moe_q4k_experts."""
    torch = _torch()
    if n_experts < 1:
        raise ValueError("n_experts must be >= 1")
    _dense_weights(w_gate, w_up, w_down, hidden, inter, n_experts)
    M = _activation(x, hidden)
    top_k = _moe_routing(expert_ids, expert_weights, M)
    if y is not None:
        _need(y, torch.float16, (M, hidden), "y")
    if dev_error is not None and (dev_error.dtype != torch.int32 or dev_error.numel() < 1):
        raise ValueError("dev_error must be an int32 tensor of at least one element")
    need = moe_workspace_size(M, top_k, n_experts, hidden, inter)
    _workspace(workspace, need)
    _on_gpu(w_gate, w_up, w_down, x, expert_ids, expert_weights, y, workspace, dev_error)
    s = _resolve_stream(stream, x.device)
    if y is None:
        y = _empty_on(s, (M, hidden), dtype=torch.float16, device=x.device)
    if workspace is None:
        workspace = _empty_on(s, max(need, 16), dtype=torch.uint8, device=x.device)
    st = lib.zinc_moe_q4k_experts(_ptr(w_gate), _ptr(w_up), _ptr(w_down), n_experts, hidden, inter, _ptr(x), M,
                                  _ptr(expert_ids), _ptr(expert_weights), top_k, _ptr(y), inter_shift, out_shift,
                                  _ptr(workspace), _nbytes(workspace), _ptr(dev_error), s.cuda_stream)
    _check(st, "zinc_moe_q4k_experts")
    return y


def zinc_moe_route_topk(logits, top_k: int, expert_ids=None, expert_weights=None, stream=None):
    """Per token the top_k experts by router logit and their softmax weights,
    computed on the GPU.  ``logits`` fp32 ``[M, n_experts]``; returns
    ``(expert_ids int32 [M, top_k], expert_weights fp32 [M, top_k])``."""
    torch = _torch()
    if logits is None or logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous float32 [M, n_experts] tensor")
    M, E = int(logits.shape[0]), int(logits.shape[1])
    if expert_ids is not None:
        _need(expert_ids, torch.int32, (M, top_k), "expert_ids")
    if expert_weights is not None:
        _need(expert_weights, torch.float32, (M, top_k), "expert_weights")
    _on_gpu(logits, expert_ids, expert_weights)
    s = _resolve_stream(stream, logits.device)
    if expert_ids is None:
        expert_ids = _empty_on(s, (M, top_k), dtype=torch.int32, device=logits.device)
    if expert_weights is None:
        expert_weights = _empty_on(s, (M, top_k), dtype=torch.float32, device=logits.device)
    st = lib.zinc_moe_route_topk(_ptr(logits), M, E, top_k, _ptr(expert_ids), _ptr(expert_weights), s.cuda_stream)
    _check(st, "zinc_moe_route_topk")
    return expert_ids, expert_weights
