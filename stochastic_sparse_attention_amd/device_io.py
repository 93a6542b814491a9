"""Upload synthetic inputs (synth.Inputs) to the GPU and describe them to
libsanta.  Marshalling only: no part of the method is computed here."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import Problem
from .synth import Inputs


@dataclass
class DeviceInputs:
    inp: Inputs
    problem: Problem
    q: object
    k: object
    v: object
    seq_lens: object
    page_table: object

    def u(self, S: int):
        import torch
        return torch.from_numpy(self.inp.u(S)).to(self.q.device)

    def uniforms(self, S: int):
        import torch
        return torch.from_numpy(self.inp.uniforms(S)).to(self.q.device)

    def bernoulli_uniforms(self, draws: int, group_mean: bool):
        import torch
        return torch.from_numpy(self.inp.bernoulli_uniforms(draws, group_mean)).to(self.q.device)

    def k_features(self):
        """K of a contiguous cache transposed per KV head: [B, Hkv, d, n_k]."""
        return self.k.transpose(-1, -2).contiguous()


def _upload(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_device(inp: Inputs, device="cuda", tile_len=None, seq_lens=None) -> DeviceInputs:
    """seq_lens: override of the per-request lengths (host int array)."""
    import torch
    c = inp.cfg
    q = _upload(inp.q, c.q_dtype, device)
    k = _upload(inp.k, c.kv_dtype, device)
    v = _upload(inp.v, c.kv_dtype, device)
    paged = c.page_size > 0
    lens = inp.seq_lens if seq_lens is None else np.asarray(seq_lens, np.int32)
    ragged = paged or not np.all(lens == c.seq_len)
    sl = torch.from_numpy(np.ascontiguousarray(lens, np.int32)).to(device) if ragged else None
    pt = torch.from_numpy(inp.page_table).to(device) if paged else None
    prob = Problem(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.seq_len,
                   dtype=c.q_dtype, kv_dtype=c.kv_dtype, scale=float(inp.scale), tile_len=tile_len or c.tile_len,
                   seq_lens=sl, page_size=c.page_size, page_table=pt)
    return DeviceInputs(inp, prob, q, k, v, sl, pt)
