"""Helpers for the GPU tests: upload a workload, run the library through
its C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_196_amd as pa
import workload

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
KERNELS = {"valu": pa.PA_KERNEL_VALU, "mfma": pa.PA_KERNEL_MFMA}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


device_tensor = workload.to_device


class Uploaded:
    def __init__(self, w):
        self.w = w
        self.q = device_tensor(w.q, w.dtype)
        self.k = device_tensor(w.k_pool, w.dtype)
        self.v = device_tensor(w.v_pool, w.dtype)
        self.bt = torch.from_numpy(w.block_tables).cuda()
        self.lens = torch.from_numpy(w.seq_lens).cuda()
        self.gs = torch.from_numpy(w.group_start).cuda()
        self.gsh = torch.from_numpy(w.group_shared).cuda()

    def run(self, kernel="auto", out_dtype=torch.float32, cached_prefix_blocks=0):
        k = pa.PA_KERNEL_AUTO if kernel == "auto" else KERNELS[kernel]
        out = pa.decode(self.q, self.k, self.v, self.bt, self.lens, float(self.w.scale),
                        out_dtype=out_dtype, kernel=k, cached_prefix_blocks=cached_prefix_blocks)
        torch.cuda.synchronize()
        return out


def kernels_for(dtype: str):
    return ["valu"] if dtype == "f32" else ["valu", "mfma"]


def max_err(got: torch.Tensor, ref: np.ndarray) -> float:
    g = got.double().cpu().numpy()
    assert g.shape == ref.shape
    assert np.all(np.isfinite(g)), "non-finite output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def desc_of(up, kernel="auto", out_dtype=torch.float32):
    k = pa.PA_KERNEL_AUTO if kernel == "auto" else KERNELS[kernel]
    return pa.make_desc(up.q, up.k, up.bt, out_dtype=out_dtype, kernel=k)


def run_shared(up, kernel="auto", out_dtype=torch.float32, workspace=None, group_start=None,
               group_shared=None):
    """paged_attn_decode_shared on an uploaded workload (its own prefix groups
    unless others are given), after the host check of the groups."""
    w = up.w
    gs = w.group_start if group_start is None else np.asarray(group_start, np.int32)
    gsh = w.group_shared if group_shared is None else np.asarray(group_shared, np.int32)
    desc = desc_of(up, kernel, out_dtype)
    assert pa.pa_validate_shared_host(desc, w.block_tables, w.seq_lens, gs, gsh, gsh.shape[0]) == 0
    k = pa.PA_KERNEL_AUTO if kernel == "auto" else KERNELS[kernel]
    out = torch.full(up.q.shape, float("nan"), dtype=out_dtype, device=up.q.device)
    pa.decode_shared(up.q, up.k, up.v, up.bt, up.lens, torch.from_numpy(gs).cuda(),
                     torch.from_numpy(gsh).cuda(), float(w.scale), out=out, out_dtype=out_dtype,
                     kernel=k, workspace=workspace)
    torch.cuda.synchronize()
    return out
