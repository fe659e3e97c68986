"""Helpers for the GPU tests: upload a workload, run the library through
its C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_196_amd as pa

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
KERNELS = {"valu": pa.PA_KERNEL_VALU, "mfma": pa.PA_KERNEL_MFMA}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def device_tensor(x: np.ndarray, dtype: str, dev="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


class Uploaded:
    def __init__(self, w):
        self.w = w
        self.q = device_tensor(w.q, w.dtype)
        self.k = device_tensor(w.k_pool, w.dtype)
        self.v = device_tensor(w.v_pool, w.dtype)
        self.bt = torch.from_numpy(w.block_tables).cuda()
        self.lens = torch.from_numpy(w.seq_lens).cuda()

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
