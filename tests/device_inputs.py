"""Seeded synthetic inputs on the GPU: the stored bits of one workload uploaded
as torch tensors and wrapped in the library's Cache and Geometry.  Shared by
the GPU tests and bench.py; holds no attention arithmetic and does not touch
the oracle."""

from __future__ import annotations

import numpy as np
import torch

import mla_latent_kv_15_amd as mla
import synth

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def bits_to_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    elif dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == "fp8":
        t = torch.from_numpy(a.astype(np.uint8, copy=False))
    else:
        raise ValueError(dtype)
    return t.to(device)


class DeviceInputs:
    """The stored inputs of one synthetic workload, resident on the GPU."""

    def __init__(self, inp: synth.MLAInputs, device="cuda"):
        wl = inp.wl
        self.inp = inp
        self.wl = wl
        self.q_nope = bits_to_tensor(inp.q_nope, wl.act_dtype, device)
        self.q_rope = bits_to_tensor(inp.q_rope, wl.act_dtype, device)
        self.w_uk = bits_to_tensor(inp.w_uk, wl.act_dtype, device)
        self.w_uv = bits_to_tensor(inp.w_uv, wl.act_dtype, device)
        rows = bits_to_tensor(inp.rows, wl.cache_dtype, device)
        row_scale = (None if inp.row_scale is None
                     else torch.from_numpy(inp.row_scale).to(device))
        bt = (None if inp.block_table is None
              else torch.from_numpy(np.ascontiguousarray(inp.block_table, np.int32)).to(device))
        self.cache = mla.Cache(rows=rows, seq_lens=torch.from_numpy(inp.seq_lens).to(device),
                               max_seq_len=int(inp.max_seq_len), row_scale=row_scale,
                               block_table=bt, seq_stride=int(inp.seq_stride),
                               page_size=int(wl.page_size))
        self.geo = mla.Geometry(heads=wl.heads, d_nope=wl.d_nope, d_rope=wl.d_rope,
                                d_latent=wl.d_latent, d_v=wl.d_v)


def act_torch_dtype(wl) -> torch.dtype:
    return torch.float32 if wl.cache_dtype == "f32" else torch.bfloat16
