"""Decode-step stochastic sparse attention (S2ANTA-prop / S2ANTA-flash) for
one MI355X (gfx950).

The computation runs in libsanta.so (hand-written HIP kernels behind the C ABI
of include/santa.h).  This module is the thin Python binding: the functions
below have the names of the C entry points and only marshal arguments -- torch
tensors become device pointers, the current torch stream becomes the
hipStream_t, and a workspace is allocated with torch when none is given.
"""
from __future__ import annotations

import ctypes as C

from . import _lib
from ._lib import SantaError, santa_problem, SANTA_F32, SANTA_BF16, SANTA_FP8_E4M3, VARIANT, SAMPLER

__all__ = [
    "Problem", "santa_workspace_size", "santa_decode_prop", "santa_decode_prop_sampler", "santa_decode_flash",
    "santa_decode_flash_sampler", "santa_decode_prop_bernoulli",
    "exact_decode_ref", "santa_set_timing_events", "SantaError",
]


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


class Problem:
    """santa_problem plus the device tensors it points to (kept alive)."""

    def __init__(self, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, *, dtype,
                 scale, tile_len, seq_lens=None, page_size=0, page_table=None, kv_dtype=None):
        """dtype: storage of q ("f32" or "bf16"); kv_dtype: storage of K and V
        (default: dtype; "fp8" is OCP e4m3 with bf16 q)."""
        codes = {"f32": SANTA_F32, "bf16": SANTA_BF16, "fp8": SANTA_FP8_E4M3}
        dt, kdt = codes[dtype], codes[kv_dtype or dtype]
        self.seq_lens = seq_lens
        self.page_table = page_table
        max_pages = 0 if page_table is None else int(page_table.shape[1])
        self.s = santa_problem(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                               None if seq_lens is None else seq_lens.data_ptr(),
                               dt, kdt, page_size,
                               None if page_table is None else page_table.data_ptr(),
                               max_pages, float(scale), tile_len)

    @property
    def ref(self):
        return C.byref(self.s)


def santa_workspace_size(problem: Problem, variant: str, S: int = 0) -> int:
    n = C.c_size_t()
    _lib._check("santa_workspace_size",
                _lib.load().santa_workspace_size(problem.ref, VARIANT[variant], S, C.byref(n)))
    return n.value


def _workspace(problem, variant, S, workspace, device):
    if workspace is not None:
        return workspace
    import torch
    return torch.empty(max(santa_workspace_size(problem, variant, S), 1), dtype=torch.uint8,
                       device=device)


def santa_decode_prop(problem: Problem, q, k, v, S, u, out, sample_idx=None, tile_budget=None,
                      workspace=None, stream=None):
    ws = _workspace(problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, _ptr(u), _ptr(out),
                                       _ptr(sample_idx), _ptr(tile_budget), _ptr(ws), ws.numel(),
                                       _stream(stream))
    _lib._check("santa_decode_prop", st)
    return ws


def santa_decode_prop_sampler(problem: Problem, q, k, v, S, sampler, u, out, sample_idx=None,
                              tile_budget=None, workspace=None, stream=None):
    """sampler: "sys" (u: [B*Hq] offsets), "strat" or "iid" (u: [B*Hq, S] uniforms)."""
    ws = _workspace(problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop_sampler(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, SAMPLER[sampler],
                                               _ptr(u), _ptr(out), _ptr(sample_idx), _ptr(tile_budget),
                                               _ptr(ws), ws.numel(), _stream(stream))
    _lib._check("santa_decode_prop_sampler", st)
    return ws


def santa_decode_prop_bernoulli(problem: Problem, q, k_features, v, S, u, draws, group_mean, u_bern, out,
                                sample_idx=None, tile_budget=None, features_read=None, workspace=None,
                                stream=None):
    """prop on Bernoulli qK^T scores.  k_features: K transposed per KV head,
    [B, Hkv, d, max_seq_len] bf16; u_bern: [B*Hq (or B*Hkv with group_mean),
    draws, d] uniforms in [0, 1)."""
    ws = _workspace(problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop_bernoulli(problem.ref, _ptr(q), _ptr(k_features), _ptr(v), S, _ptr(u),
                                                 int(draws), int(group_mean), _ptr(u_bern), _ptr(out),
                                                 _ptr(sample_idx), _ptr(tile_budget), _ptr(features_read),
                                                 _ptr(ws), ws.numel(), _stream(stream))
    _lib._check("santa_decode_prop_bernoulli", st)
    return ws


def santa_decode_flash(problem: Problem, q, k, v, S, u, out, sample_idx=None, tile_budget=None,
                       workspace=None, stream=None):
    ws = _workspace(problem, "flash", S, workspace, q.device)
    st = _lib.load().santa_decode_flash(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, _ptr(u), _ptr(out),
                                        _ptr(sample_idx), _ptr(tile_budget), _ptr(ws), ws.numel(),
                                        _stream(stream))
    _lib._check("santa_decode_flash", st)
    return ws


def santa_decode_flash_sampler(problem: Problem, q, k, v, S, sampler, u, out, sample_idx=None,
                               tile_budget=None, workspace=None, stream=None):
    """sampler: "sys" (u: [B*Hq] offsets), "strat" or "iid" (u: [B*Hq, S] uniforms, tile-major)."""
    ws = _workspace(problem, "flash", S, workspace, q.device)
    st = _lib.load().santa_decode_flash_sampler(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, SAMPLER[sampler],
                                                _ptr(u), _ptr(out), _ptr(sample_idx), _ptr(tile_budget),
                                                _ptr(ws), ws.numel(), _stream(stream))
    _lib._check("santa_decode_flash_sampler", st)
    return ws


def exact_decode_ref(problem: Problem, q, k, v, out, workspace=None, stream=None):
    ws = _workspace(problem, "exact", 0, workspace, q.device)
    st = _lib.load().exact_decode_ref(problem.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                      ws.numel(), _stream(stream))
    _lib._check("exact_decode_ref", st)
    return ws


def _event_handle(ev):
    if ev is None:
        return None
    return C.c_void_p(ev.cuda_event if hasattr(ev, "cuda_event") else int(ev))


def santa_set_timing_events(begin=None, end=None):
    """Record `begin`/`end` (torch.cuda.Event, or raw hipEvent_t handles)
    around the dominant kernel of later calls on this thread; None, None turns
    it off."""
    _lib.load().santa_set_timing_events(_event_handle(begin), _event_handle(end))
