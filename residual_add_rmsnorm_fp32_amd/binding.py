"""Python binding of ``libfar.so`` (ctypes): argument marshalling only.

Every step of the epilogue runs in the HIP library; this module checks tensor
properties, flattens ``[..., H]`` tensors to ``[T, H]`` (all leading dims are tokens, as
``call_trtllm_fused_allreduce_norm`` does on page "PR #45307 report"), passes raw
device pointers and the current torch stream, and turns status codes into exceptions.
PyTorch is used for device memory and streams only. There is no fallback: if the
library is missing, every call raises.

The functions carry the C names of ``include/far.h``. ``fused_add_rmsnorm`` is the
convenience form that allocates outputs and returns them in the order the pages give:
``(normed_output, new_residual)`` without quantisation (page
"vllm.models.common.ops.fused_allreduce_rms_norm"), ``(result, residual)`` for the static
fp8 epilogue and ``(result, residual, scale)`` for the dynamic per-token one (page
"vllm.compilation.fusion", FusedAddRMSNormStaticQuantPattern /
FusedAddRMSNormDynamicQuantPattern).
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfar.so")

FAR_MAX_PARTIALS = 8
FAR_MAX_WAVES_PER_ROW = 16
FAR_MAX_PACKS_PER_LANE = 5
FAR_DTYPE = {torch.bfloat16: 0, torch.float16: 1}
FAR_QUANT = {None: 0, "none": 0, "static": 1, "dynamic": 2, "group": 3, "tensor": 4}
FAR_FP8_GROUP = 128
FAR_VARIANT = {0: "empty", 1: "vector", 2: "generic"}
FAR_VARIANT_ID = {v: k for k, v in FAR_VARIANT.items()}

FAR_OK = 0
STATUS_NAMES = {
    0: "FAR_OK", 1: "FAR_ERR_NULL_POINTER", 2: "FAR_ERR_BAD_SHAPE", 3: "FAR_ERR_BAD_DTYPE",
    4: "FAR_ERR_BAD_NUM_PARTIALS", 5: "FAR_ERR_BAD_QUANT_ARGS", 6: "FAR_ERR_BAD_ALIAS",
    7: "FAR_ERR_HIP", 8: "FAR_ERR_BAD_PLAN", 9: "FAR_ERR_WORKSPACE", 10: "FAR_ERR_SCRATCH_LIMIT",
}
FAR_NOALLOC_SCRATCH_BYTES = 2 * 1024 * 1024


class FarError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class FarLibraryMissing(RuntimeError):
    pass


class far_plan_t(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32),
        ("waves_per_row", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32),
        ("packs_per_lane", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("grid_blocks", ctypes.c_int64),
    ]

    def as_dict(self) -> dict:
        return {
            "variant": FAR_VARIANT.get(self.variant, self.variant),
            "waves_per_row": self.waves_per_row, "rows_per_block": self.rows_per_block,
            "packs_per_lane": self.packs_per_lane, "block_threads": self.block_threads,
            "grid_blocks": self.grid_blocks,
        }


_vp = ctypes.c_void_p
_MAIN_ARGS = [
    ctypes.POINTER(_vp), ctypes.c_int,            # partials, num_partials
    _vp, _vp,                                     # residual, gamma
    ctypes.c_int64, ctypes.c_int64, ctypes.c_int,  # num_tokens, hidden, dtype
    ctypes.c_float, ctypes.c_float,               # eps, weight_bias
    ctypes.c_int, _vp,                            # quant_mode, scale
    _vp, _vp, _vp, _vp,                           # norm_out, residual_out, quant_out, scale_out
    _vp,                                          # stream
]

_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfar.so once (raises FarLibraryMissing if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise FarLibraryMissing(
            f"{path} is missing: build it with `python -m residual_add_rmsnorm_fp32_amd.build`")
    lib = ctypes.CDLL(path)
    lib.far_fused_add_rmsnorm.argtypes = _MAIN_ARGS
    lib.far_fused_add_rmsnorm.restype = ctypes.c_int
    lib.far_fused_add_rmsnorm_ex.argtypes = _MAIN_ARGS + [ctypes.POINTER(far_plan_t), _vp,
                                                         ctypes.c_int64]
    lib.far_fused_add_rmsnorm_ex.restype = ctypes.c_int
    lib.far_fused_add_rmsnorm_noalloc.argtypes = _MAIN_ARGS
    lib.far_fused_add_rmsnorm_noalloc.restype = ctypes.c_int
    lib.far_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    lib.far_workspace_bytes.restype = ctypes.c_int64
    lib.far_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.POINTER(far_plan_t)]
    lib.far_plan.restype = ctypes.c_int
    lib.far_status_string.argtypes = [ctypes.c_int]
    lib.far_status_string.restype = ctypes.c_char_p
    lib.far_version.argtypes = []
    lib.far_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def far_status_string(status: int) -> str:
    return load_library().far_status_string(int(status)).decode()


def far_version() -> int:
    return int(load_library().far_version())


def far_workspace_bytes(num_tokens: int, hidden: int, quant_mode=None) -> int:
    """Workspace bytes a call needs (0 except for the per-tensor dynamic mode)."""
    return int(load_library().far_workspace_bytes(int(num_tokens), int(hidden), _quant_id(quant_mode)))


def _check(status: int):
    if status != FAR_OK:
        raise FarError(status, far_status_string(status))


def _quant_id(q) -> int:
    if isinstance(q, int):
        return q
    if q not in FAR_QUANT:
        raise ValueError(f"quant must be one of {list(FAR_QUANT)}, got {q!r}")
    return FAR_QUANT[q]


def far_plan(num_tokens: int, hidden: int, num_partials: int, dtype, quant_mode=None) -> dict:
    """The library's automatic launch plan for a shape (pure host logic)."""
    dt = FAR_DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    out = far_plan_t()
    _check(load_library().far_plan(int(num_tokens), int(hidden), int(num_partials), dt,
                                   _quant_id(quant_mode), ctypes.byref(out)))
    return out.as_dict()


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _as_partial_list(partials) -> list:
    if isinstance(partials, torch.Tensor):
        return [partials[i] for i in range(partials.shape[0])]
    return list(partials)


def far_fused_add_rmsnorm(partials, residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                          weight_bias: float, quant_mode, scale, norm_out, residual_out,
                          quant_out, scale_out, stream=None, plan: dict | None = None,
                          workspace: torch.Tensor | None = None) -> None:
    """Call the C entry point on torch device tensors (outputs preallocated).

    ``partials`` is a sequence of P tensors or one ``[P, ...]`` tensor. Every
    ``[..., H]`` tensor is taken as ``[T, H]`` with ``T = numel / H``; all must be
    contiguous and on one GPU. ``quant_out`` may be uint8 or float8_e4m3fn. ``stream``
    defaults to torch's current stream on the tensors' device. ``plan`` (a dict as
    returned by ``far_plan``) forces a launch configuration; ``workspace`` is device
    memory for the per-tensor dynamic mode (``far_workspace_bytes``).
    """
    lib = load_library()
    plist = _as_partial_list(partials)
    P = len(plist)
    if P < 1:
        raise ValueError("at least one partial is needed")
    ref = residual if residual is not None else plist[0]
    if ref.dim() < 1:
        raise ValueError("tensors must have a hidden dimension")
    H = int(ref.shape[-1])
    T = ref.numel() // H if H > 0 else 0
    dev = ref.device
    if dev.type != "cuda":
        raise ValueError("far_fused_add_rmsnorm needs GPU tensors (device memory)")
    dtype = ref.dtype
    if dtype not in FAR_DTYPE:
        raise TypeError(f"storage dtype must be bfloat16 or float16, got {dtype}")

    def check(t, name, numel, dt=None):
        if t is None:
            return
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dt is not None and t.dtype not in dt:
            raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dt}")
        if t.numel() != numel:
            raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")

    for i, p in enumerate(plist):
        check(p, f"partials[{i}]", T * H, (dtype,))
        if p.shape[-1] != H:
            raise ValueError(f"partials[{i}] last dim {p.shape[-1]} != {H}")
    check(residual, "residual", T * H, (dtype,))
    check(gamma, "gamma", H, (dtype,))
    check(norm_out, "norm_out", T * H, (dtype,))
    check(residual_out, "residual_out", T * H, (dtype,))
    check(quant_out, "quant_out", T * H, (torch.uint8, torch.float8_e4m3fn))
    q = _quant_id(quant_mode)
    n_scales = {2: T, 3: T * -(-H // FAR_FP8_GROUP), 4: 1}.get(q, T)
    check(scale_out, "scale_out", n_scales, (torch.float32,))
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be contiguous memory on the tensors' device")
    check(scale, "scale", 1, (torch.float32,))
    if P > FAR_MAX_PARTIALS:
        raise ValueError(f"at most {FAR_MAX_PARTIALS} partials")

    arr = (_vp * max(P, 1))(*[p.data_ptr() for p in plist])
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    args = [arr, P, _ptr(residual), _ptr(gamma), T, H, FAR_DTYPE[dtype], float(eps),
            float(weight_bias), q, _ptr(scale), _ptr(norm_out),
            _ptr(residual_out), _ptr(quant_out), _ptr(scale_out), stream]
    with torch.cuda.device(dev):
        if plan is None and workspace is None:
            st = lib.far_fused_add_rmsnorm(*args)
        else:
            pl = far_plan_t()
            plan_d = plan or {}
            pl.variant = FAR_VARIANT_ID.get(plan_d.get("variant"), plan_d.get("variant", 1))
            pl.waves_per_row = int(plan_d.get("waves_per_row", 0))
            pl.rows_per_block = int(plan_d.get("rows_per_block", 0))
            pl.packs_per_lane = int(plan_d.get("packs_per_lane", 0))
            pl.block_threads = int(plan_d.get("block_threads", 0))
            pl.grid_blocks = int(plan_d.get("grid_blocks", 0))
            ws_ptr = workspace.data_ptr() if workspace is not None else None
            ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
            st = lib.far_fused_add_rmsnorm_ex(*args, ctypes.byref(pl) if plan is not None else None,
                                              ws_ptr, ws_bytes)
    _check(st)


def fused_add_rmsnorm(partials, residual: torch.Tensor | None, gamma: torch.Tensor, eps: float,
                      weight_bias: float = 0.0, quant=None, scale: torch.Tensor | None = None,
                      *, norm_out: torch.Tensor | None = None, want_norm_out: bool = False,
                      residual_out: torch.Tensor | None = None, quant_out=None, scale_out=None,
                      inplace: bool = False, discard_residual: bool = False,
                      plan: dict | None = None):
    """Allocate what is not given, run the epilogue, return the pages' output tuple.

    Returns ``(norm_out, new_residual)`` without quantisation, ``(quant_out,
    new_residual)`` for ``quant="static"`` and ``(quant_out, new_residual, scale_out)``
    for the dynamic modes ``"dynamic"`` (per token), ``"group"`` (per 128 elements of a
    row) and ``"tensor"`` (one scale; a workspace is allocated for the call); with
    quantisation and ``want_norm_out`` the normalised
    output is appended. ``residual=None`` is the form without a residual input (the new
    residual is the sum of the partials). ``inplace=True`` writes the new residual into
    ``residual``; ``discard_residual=True`` does not write it (``None`` is returned in
    its place). Output shapes follow the inputs' (``scale_out`` drops the last dim).
    """
    q = _quant_id(quant)
    plist = _as_partial_list(partials)
    like = residual if residual is not None else plist[0]
    if residual_out is None and not discard_residual:
        if inplace:
            if residual is None:
                raise ValueError("inplace needs a residual tensor")
            residual_out = residual
        else:
            residual_out = torch.empty_like(like)
    if q == 0 or want_norm_out:
        if norm_out is None:
            norm_out = torch.empty_like(like)
    if q != 0 and quant_out is None:
        quant_out = torch.empty(like.shape, dtype=torch.float8_e4m3fn, device=like.device)
    if scale_out is None:
        if q == 2:
            scale_out = torch.empty(like.shape[:-1], dtype=torch.float32, device=like.device)
        elif q == 3:
            groups = -(-like.shape[-1] // FAR_FP8_GROUP)
            scale_out = torch.empty(tuple(like.shape[:-1]) + (groups,), dtype=torch.float32,
                                    device=like.device)
        elif q == 4:
            scale_out = torch.empty(1, dtype=torch.float32, device=like.device)
    workspace = None
    T = like.numel() // like.shape[-1] if like.shape[-1] else 0
    ws_bytes = far_workspace_bytes(T, like.shape[-1], q)
    if ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=like.device)
    far_fused_add_rmsnorm(plist, residual, gamma, eps, weight_bias, q, scale, norm_out,
                          residual_out, quant_out, scale_out, plan=plan, workspace=workspace)
    if q == 0:
        return norm_out, residual_out
    out = (quant_out, residual_out) if q == 1 else (quant_out, residual_out, scale_out)
    return out + ((norm_out,) if want_norm_out else ())
