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
    "santa_decode_flash_sampler", "santa_decode_prop_bernoulli", "santa_decode_prop_static",
    "santa_decode_prop_fused", "new_workspace",
    "exact_decode_ref", "santa_set_timing_events", "SantaError",
]


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


# ----------------------------------------------------------------------
# Argument checks before any pointer reaches the library: a tensor of the
# wrong type, too short, strided or on another device would make the
# kernels read or write outside it.  Order: dtype, size, layout, device.
# ----------------------------------------------------------------------
def _torch_dtypes(code):
    import torch
    if code == SANTA_F32:
        return (torch.float32,)
    if code == SANTA_BF16:
        return (torch.bfloat16,)
    return (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))   # e4m3 bytes


def _check_tensor(fn, name, t, dtypes, min_numel, exact=False):
    """Raise ValueError unless t has one of `dtypes`, at least (or exactly)
    min_numel elements and is contiguous."""
    if t is None:
        raise ValueError(f"{fn}: {name} is required")
    if not hasattr(t, "data_ptr") or not hasattr(t, "dtype"):
        raise ValueError(f"{fn}: {name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    n = t.numel()
    if (exact and n != min_numel) or n < min_numel:
        raise ValueError(f"{fn}: {name} has {n} elements, "
                         f"{'exactly' if exact else 'at least'} {min_numel} required")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")


def _check_devices(fn, named):
    """Every tensor on the same GPU as the first (q)."""
    dev = named[0][1].device
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError(f"{fn}: {name} is on {t.device}, expected "
                             f"{dev if dev.type == 'cuda' else 'a GPU'}")


def _check_args(fn, problem, q, k, v, out, extra=()):
    """q, K, V, out, the problem's own tensors and the call's other
    arguments (`extra`: (name, tensor or None, dtypes, min_numel)); then all
    on one GPU."""
    P = problem
    B, Hq, Hkv, d, n = P.batch, P.num_q_heads, P.num_kv_heads, P.head_dim, P.max_seq_len
    import torch
    _check_tensor(fn, "q", q, _torch_dtypes(P.q_code), B * Hq * d, exact=True)
    kv = _torch_dtypes(P.kv_code)
    for name, t in (("k", k), ("v", v)):
        if P.page_size:
            page = Hkv * P.page_size * d
            _check_tensor(fn, name, t, kv, page)
            if t.numel() % page:
                raise ValueError(f"{fn}: {name} must hold whole pages of {page} elements")
        else:
            _check_tensor(fn, name, t, kv, B * Hkv * n * d, exact=True)
    _check_tensor(fn, "out", out, (torch.float32,), B * Hq * d)
    if P.seq_lens is not None:
        _check_tensor(fn, "seq_lens", P.seq_lens, (torch.int32,), B, exact=True)
    if P.page_table is not None:
        _check_tensor(fn, "page_table", P.page_table, (torch.int32,), B * P.max_pages, exact=True)
    for name, t, dts, need in extra:
        if t is not None:
            _check_tensor(fn, name, t, dts, need)
    _check_devices(fn, [("q", q), ("k", k), ("v", v), ("out", out), ("seq_lens", P.seq_lens),
                        ("page_table", P.page_table)] + [(name, t) for name, t, _, _ in extra])


def _sampled_extra(fn, problem, S, u, sample_idx, tile_budget, u_per_head):
    import torch
    P = problem
    BH = P.batch * P.num_q_heads
    if u is None:
        raise ValueError(f"{fn}: u is required")
    return [("u", u, (torch.float32,), BH * (u_per_head if u_per_head else 1)),
            ("sample_idx", sample_idx, (torch.int32,), BH * S),
            ("tile_budget", tile_budget, (torch.int32,), BH * P.max_tiles())]


def _ws_bytes(fn, ws, need, device):
    """Bytes of a caller's workspace tensor (any dtype), checked."""
    if not hasattr(ws, "data_ptr"):
        raise ValueError(f"{fn}: workspace must be a torch tensor")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"{fn}: workspace holds {nbytes} bytes, {need} required")
    if not ws.is_contiguous():
        raise ValueError(f"{fn}: workspace must be contiguous")
    if ws.device != device:
        raise ValueError(f"{fn}: workspace is on {ws.device}, expected {device}")
    return nbytes


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
        import torch
        for name, t in (("seq_lens", seq_lens), ("page_table", page_table)):
            if t is not None and (not hasattr(t, "dtype") or t.dtype != torch.int32):
                raise ValueError(f"Problem: {name} must be an int32 tensor")
        if seq_lens is not None and seq_lens.numel() != batch:
            raise ValueError(f"Problem: seq_lens has {seq_lens.numel()} entries, batch is {batch}")
        if page_table is not None and (page_table.dim() != 2 or page_table.shape[0] != batch):
            raise ValueError("Problem: page_table must be [batch, max_pages_per_seq]")
        if (page_size > 0) != (page_table is not None):
            raise ValueError("Problem: a paged cache needs a page table, and only it")
        self.seq_lens = seq_lens
        self.page_table = page_table
        max_pages = 0 if page_table is None else int(page_table.shape[1])
        self.batch, self.num_q_heads, self.num_kv_heads = batch, num_q_heads, num_kv_heads
        self.head_dim, self.max_seq_len, self.tile_len = head_dim, max_seq_len, tile_len
        self.q_code, self.kv_code, self.page_size, self.max_pages = dt, kdt, page_size, max_pages
        self.s = santa_problem(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                               None if seq_lens is None else seq_lens.data_ptr(),
                               dt, kdt, page_size,
                               None if page_table is None else page_table.data_ptr(),
                               max_pages, float(scale), tile_len)

    @property
    def ref(self):
        return C.byref(self.s)

    def max_tiles(self):
        return (self.max_seq_len + self.tile_len - 1) // self.tile_len


def santa_workspace_size(problem: Problem, variant: str, S: int = 0) -> int:
    n = C.c_size_t()
    _lib._check("santa_workspace_size",
                _lib.load().santa_workspace_size(problem.ref, VARIANT[variant], S, C.byref(n)))
    return n.value


def new_workspace(problem, variant, S=0, device="cuda"):
    """A workspace for `variant`, allocated zeroed (the arrival counters that
    santa_decode_prop_fused needs at zero are its first SANTA_SYNC_BYTES)."""
    import torch
    return torch.zeros(max(santa_workspace_size(problem, variant, S), 1), dtype=torch.uint8, device=device)


def _workspace(fn, problem, variant, S, workspace, device):
    """(workspace tensor, its byte count): the caller's, checked, or a new one."""
    need = santa_workspace_size(problem, variant, S)
    if workspace is not None:
        return workspace, _ws_bytes(fn, workspace, need, device)
    ws = new_workspace(problem, variant, S, device)
    return ws, ws.numel()


def santa_decode_prop(problem: Problem, q, k, v, S, u, out, sample_idx=None, tile_budget=None,
                      workspace=None, stream=None):
    fn = "santa_decode_prop"
    _check_args(fn, problem, q, k, v, out, _sampled_extra(fn, problem, S, u, sample_idx, tile_budget, 0))
    ws, nb = _workspace(fn, problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, _ptr(u), _ptr(out),
                                       _ptr(sample_idx), _ptr(tile_budget), _ptr(ws), nb,
                                       _stream(stream))
    _lib._check("santa_decode_prop", st)
    return ws


def santa_decode_prop_fused(problem: Problem, q, k, v, S, u, out, sample_idx=None, tile_budget=None,
                            workspace=None, stream=None):
    """prop in one launch; a caller's workspace must come from
    new_workspace() or otherwise start with SANTA_SYNC_BYTES of zeros."""
    fn = "santa_decode_prop_fused"
    _check_args(fn, problem, q, k, v, out, _sampled_extra(fn, problem, S, u, sample_idx, tile_budget, 0))
    ws, nb = _workspace(fn, problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop_fused(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, _ptr(u), _ptr(out),
                                             _ptr(sample_idx), _ptr(tile_budget), _ptr(ws), nb, _stream(stream))
    _lib._check(fn, st)
    return ws


def santa_decode_prop_sampler(problem: Problem, q, k, v, S, sampler, u, out, sample_idx=None,
                              tile_budget=None, workspace=None, stream=None):
    """sampler: "sys" (u: [B*Hq] offsets), "strat" or "iid" (u: [B*Hq, S] uniforms)."""
    fn = "santa_decode_prop_sampler"
    if sampler not in SAMPLER:
        raise ValueError(f"{fn}: sampler must be one of {sorted(SAMPLER)}")
    _check_args(fn, problem, q, k, v, out,
                _sampled_extra(fn, problem, S, u, sample_idx, tile_budget, 0 if sampler == "sys" else S))
    ws, nb = _workspace(fn, problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop_sampler(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, SAMPLER[sampler],
                                               _ptr(u), _ptr(out), _ptr(sample_idx), _ptr(tile_budget),
                                               _ptr(ws), nb, _stream(stream))
    _lib._check("santa_decode_prop_sampler", st)
    return ws


def santa_decode_prop_bernoulli(problem: Problem, q, k_features, v, S, u, draws, group_mean, u_bern, out,
                                sample_idx=None, tile_budget=None, features_read=None, workspace=None,
                                stream=None):
    """prop on Bernoulli qK^T scores.  k_features: K transposed per KV head,
    [B, Hkv, d, max_seq_len] bf16; u_bern: [B*Hq (or B*Hkv with group_mean),
    draws, d] uniforms in [0, 1)."""
    import torch
    fn = "santa_decode_prop_bernoulli"
    P = problem
    owners = P.batch * (P.num_kv_heads if group_mean else P.num_q_heads)
    if u_bern is None:
        raise ValueError(f"{fn}: u_bern is required")
    extra = _sampled_extra(fn, P, S, u, sample_idx, tile_budget, 0) + [
        ("u_bern", u_bern, (torch.float32,), owners * max(int(draws), 1) * P.head_dim),
        ("features_read", features_read, (torch.int32,), P.batch * P.num_kv_heads)]
    _check_args(fn, P, q, k_features, v, out, extra)
    ws, nb = _workspace(fn, problem, "prop", S, workspace, q.device)
    st = _lib.load().santa_decode_prop_bernoulli(problem.ref, _ptr(q), _ptr(k_features), _ptr(v), S, _ptr(u),
                                                 int(draws), int(group_mean), _ptr(u_bern), _ptr(out),
                                                 _ptr(sample_idx), _ptr(tile_budget), _ptr(features_read),
                                                 _ptr(ws), nb, _stream(stream))
    _lib._check("santa_decode_prop_bernoulli", st)
    return ws


def santa_decode_flash(problem: Problem, q, k, v, S, u, out, sample_idx=None, tile_budget=None,
                       workspace=None, stream=None):
    """tile_budget is ignored by the library (every tile takes S / n_t)."""
    fn = "santa_decode_flash"
    _check_args(fn, problem, q, k, v, out, _sampled_extra(fn, problem, S, u, sample_idx, None, 0))
    ws, nb = _workspace(fn, problem, "flash", S, workspace, q.device)
    st = _lib.load().santa_decode_flash(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, _ptr(u), _ptr(out),
                                        _ptr(sample_idx), None, _ptr(ws), nb, _stream(stream))
    _lib._check("santa_decode_flash", st)
    return ws


def santa_decode_flash_sampler(problem: Problem, q, k, v, S, sampler, u, out, sample_idx=None,
                               tile_budget=None, workspace=None, stream=None):
    """sampler: "sys" (u: [B*Hq] offsets), "strat" or "iid" (u: [B*Hq, S] uniforms, tile-major)."""
    fn = "santa_decode_flash_sampler"
    if sampler not in SAMPLER:
        raise ValueError(f"{fn}: sampler must be one of {sorted(SAMPLER)}")
    _check_args(fn, problem, q, k, v, out,
                _sampled_extra(fn, problem, S, u, sample_idx, None, 0 if sampler == "sys" else S))
    ws, nb = _workspace(fn, problem, "flash", S, workspace, q.device)
    st = _lib.load().santa_decode_flash_sampler(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, SAMPLER[sampler],
                                                _ptr(u), _ptr(out), _ptr(sample_idx), None,
                                                _ptr(ws), nb, _stream(stream))
    _lib._check("santa_decode_flash_sampler", st)
    return ws


def santa_decode_prop_static(problem: Problem, q, k, v, S, u, out, sample_idx=None, tile_budget=None,
                             stream=None):
    """santa_decode_prop with the library's static device workspace: the
    call allocates nothing (for code that cannot allocate)."""
    fn = "santa_decode_prop_static"
    _check_args(fn, problem, q, k, v, out, _sampled_extra(fn, problem, S, u, sample_idx, tile_budget, 0))
    st = _lib.load().santa_decode_prop_static(problem.ref, _ptr(q), _ptr(k), _ptr(v), S, _ptr(u), _ptr(out),
                                              _ptr(sample_idx), _ptr(tile_budget), _stream(stream))
    _lib._check(fn, st)


def exact_decode_ref(problem: Problem, q, k, v, out, workspace=None, stream=None):
    _check_args("exact_decode_ref", problem, q, k, v, out)
    ws, nb = _workspace("exact_decode_ref", problem, "exact", 0, workspace, q.device)
    st = _lib.load().exact_decode_ref(problem.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws),
                                      nb, _stream(stream))
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
