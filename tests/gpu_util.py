"""Helpers shared by the GPU tests: moving seeded code arrays to the device, running
the HIP path through the binding, running the oracle on the same codes, comparing."""

from __future__ import annotations

import numpy as np
import torch

import compare as cmp
from oracle import far_oracle as orc
from residual_add_rmsnorm_fp32_amd import binding as B

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
QUANT_ID = {"none": 0, "static": 1, "dynamic": 2, "group": 3, "tensor": 4}
DYNAMIC = ("dynamic", "group", "tensor")


def to_dev(codes: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16))
    return t.view(TORCH_DT[dtype]).to(device)


def codes_of(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def run_gpu(inp: dict, dtype: str, eps: float, wb: float, quant: str = "none",
            want_norm: bool = True, plan: dict | None = None, shape=None,
            no_residual: bool = False, discard_residual: bool = False) -> dict:
    """Run the HIP path on freshly uploaded inputs. ``shape`` views every [T, H]
    tensor with that shape (e.g. [B, S, H]) before the call. ``no_residual`` passes no
    residual input; ``discard_residual`` asks for no new residual."""
    partials = [to_dev(p, dtype) for p in inp["partials"]]
    residual = None if no_residual else to_dev(inp["residual"], dtype)
    gamma = to_dev(inp["gamma"], dtype)
    if shape is not None:
        partials = [p.view(shape) for p in partials]
        residual = residual.view(shape) if residual is not None else None
    scale = None
    if quant == "static":
        scale = torch.from_numpy(np.asarray(inp["scale"], np.float32).reshape(1)).cuda()
    outs = B.fused_add_rmsnorm(partials, residual, gamma, eps, wb, quant=quant, scale=scale,
                               want_norm_out=want_norm, plan=plan,
                               discard_residual=discard_residual)
    torch.cuda.synchronize()
    res = {}
    if quant == "none":
        res["norm_out"], res["new_residual"] = codes_of(outs[0]), outs[1]
    else:
        res["quant_out"], res["new_residual"] = codes_of(outs[0]), outs[1]
        if quant in DYNAMIC:
            res["scale_out"] = codes_of(outs[2])
        if want_norm:
            res["norm_out"] = codes_of(outs[-1])
    if res["new_residual"] is None:
        del res["new_residual"]
    else:
        res["new_residual"] = codes_of(res["new_residual"])
    H = inp["gamma"].shape[-1]
    out = {}
    for k, v in res.items():
        if k == "scale_out":
            out[k] = v.reshape(-1, v.shape[-1]) if quant == "group" else v.reshape(-1)
        else:
            out[k] = v.reshape(-1, H)
    return out


def run_oracle(inp: dict, dtype: str, eps: float, wb: float, quant: str = "none",
               rows=None, no_residual: bool = False) -> dict:
    partials, residual = inp["partials"], (None if no_residual else inp["residual"])
    if rows is not None:
        partials = partials[:, rows]
        residual = residual[rows] if residual is not None else None
    return orc.fused_add_rmsnorm(partials, residual, inp["gamma"], dtype, eps, wb,
                                 quant_mode=QUANT_ID[quant], scale=inp.get("scale"))


def abs_terms(inp: dict, dtype: str, rows=None, no_residual: bool = False) -> np.ndarray:
    partials, residual = inp["partials"], inp["residual"]
    if rows is not None:
        partials = partials[:, rows]
        residual = residual[rows]
    s = np.zeros(partials.shape[1:]) if no_residual else np.abs(cmp.decode(residual, dtype))
    for p in partials:
        s = s + np.abs(cmp.decode(p, dtype))
    return s


def compare(gpu: dict, ref: dict, dtype: str, quant: str, inp: dict | None = None,
            rows=None, tag: str = "", no_residual: bool = False) -> dict:
    stats = {}
    at = abs_terms(inp, dtype, rows, no_residual) if inp is not None else None
    g = {k: (v[rows] if rows is not None and not (k == "scale_out" and quant == "tensor") else v)
         for k, v in gpu.items()}
    if "new_residual" in g:
        n_adds = len(inp["partials"]) - (1 if no_residual else 0) if inp is not None else 0
        stats["new_residual"] = cmp.check_storage(g["new_residual"], ref["new_residual"], dtype,
                                                  f"{tag} new_residual", at, n_adds)
    if "norm_out" in g:
        stats["norm_out"] = cmp.check_storage(g["norm_out"], ref["norm_out"], dtype, f"{tag} norm_out")
    if quant != "none":
        stats["quant_out"] = cmp.check_fp8(g["quant_out"], ref["quant_out"], f"{tag} quant_out")
    if quant in DYNAMIC:
        stats["scale_out"] = cmp.check_scales(g["scale_out"], ref["scale_out"], f"{tag} scale_out")
    return stats


def compare_rows_chunked(gpu: dict, inp: dict, dtype: str, eps: float, wb: float,
                         quant: str = "none", chunk: int = 512, tag: str = "") -> list:
    """Every row of a (large) batch against the oracle, in row chunks run by a thread
    pool (the oracle's numpy kernels release the interpreter lock). Per-token modes
    only (per-tensor scales need the whole tensor). Returns the per-chunk statistics."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    T = inp["residual"].shape[0]

    def one(r0):
        rows = np.arange(r0, min(r0 + chunk, T))
        ref = run_oracle(inp, dtype, eps, wb, quant, rows=rows)
        return compare(gpu, ref, dtype, quant, inp, rows=rows, tag=f"{tag} rows {r0}+")

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(one, range(0, T, chunk)))
