"""CPU oracle for decode-step stochastic sparse attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product library never calls it, and it shares no code with
the GPU path: the C source next to this file restates every step of the
method from the SANTA notes ("Stochastic Sparse Attention for Memory-Bound
Inference", key designs 1-3) in plain fp64 loops.

Functions and their pins (the tests under tests/ hold the checks):
  logits / softmax_weights / exact   pinned to torch's fp64 attention on CPU,
                                      uniform-key closed form
  invert_cdf / sys_thresholds         pinned by hand-derived partitions of U
                                      (tests/golden), one-hot A, S = n_k on a
                                      uniform A, brute-force enumeration
  cell_edges / prop_cells /           pinned by the hand-derived CDFs of the
  flash_cells                         golden partitions (global and per tile);
                                      every oracle threshold lies in its own
                                      token's cell
  santa_prop (= untiled systematic)   E_U[estimate] = AV by exact breakpoint
                                      enumeration; per-tile counts within
                                      {floor, ceil} of S * tile mass
  santa_flash                         n_t = 1 reduces to santa_prop; E_U = AV
  sys_moments / flash_moments         checked against a Monte-Carlo average and
                                      against a brute-force fine U grid
  iid / strat thresholds              i.i.d. variance closed form
  replay                              equals the estimate for the oracle's own
                                      indices
  bernoulli_* / santa_prop_bernoulli  E[score] = <q, K> exactly over a grid of
                                      uniforms; hand-derived coefficients;
                                      |q_i| = max|q| reduces to exact scores
                                      (and prop); read fraction closed form
"""
from __future__ import annotations

import ctypes as C
import os
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB names another build of the same source (the planted-mistake
# test loads altered copies that way); by default the one built here
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


# storage formats of the oracle's problem struct
FORMATS = {"f32": 0, "bf16": 1, "fp8": 2}


class _Problem(C.Structure):
    _fields_ = [
        ("batch", C.c_int), ("num_q_heads", C.c_int), ("num_kv_heads", C.c_int),
        ("head_dim", C.c_int), ("max_seq_len", C.c_int),
        ("seq_lens", C.POINTER(C.c_int)),
        ("q_fmt", C.c_int), ("kv_fmt", C.c_int),
        ("page_size", C.c_int), ("page_table", C.POINTER(C.c_int)),
        ("max_pages", C.c_int), ("scale", C.c_float), ("tile_len", C.c_int),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            if os.environ.get("ORACLE_LIB"):
                raise FileNotFoundError(LIB_PATH)
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        P = C.POINTER(_Problem)
        vp, dp, ip, fp = C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int), C.POINTER(C.c_float)
        L.oracle_logits.argtypes = [P, vp, vp, C.c_int, C.c_int, dp]
        L.oracle_softmax_weights.argtypes = [dp, C.c_int, dp, dp]
        L.oracle_softmax_weights.restype = C.c_double
        L.oracle_invert_cdf.argtypes = [dp, C.c_int, dp, C.c_int, ip, dp]
        L.oracle_cell_edges.argtypes = [dp, C.c_int, ip, C.c_int, dp, dp]
        L.oracle_prop_cells.argtypes = [P, vp, vp, C.c_int, C.c_int, fp, C.c_int, C.c_int, fp, ip,
                                        dp, dp, dp]
        L.oracle_flash_cells.argtypes = [P, vp, vp, C.c_int, C.c_int, fp, ip, dp, dp, dp]
        L.oracle_sys_thresholds.argtypes = [C.c_double, C.c_int, dp]
        L.oracle_strat_thresholds.argtypes = [dp, C.c_int, dp]
        L.oracle_iid_thresholds.argtypes = [dp, C.c_int, dp]
        L.oracle_santa_prop.argtypes = [P, vp, vp, vp, C.c_int, fp, dp, ip, dp, ip]
        L.oracle_santa_prop_sampler.argtypes = [P, vp, vp, vp, C.c_int, C.c_int, fp, dp, ip, dp, ip]
        L.oracle_santa_flash.argtypes = [P, vp, vp, vp, C.c_int, fp, dp, ip, dp, dp]
        L.oracle_santa_flash_sampler.argtypes = [P, vp, vp, vp, C.c_int, C.c_int, fp, dp, ip, dp, dp]
        L.oracle_exact.argtypes = [P, vp, vp, vp, dp]
        L.oracle_replay.argtypes = [P, vp, C.c_int, ip, dp, C.c_int, dp]
        L.oracle_estimate_from_weights.argtypes = [dp, C.c_int, dp, C.c_int, dp, C.c_int, dp]
        L.oracle_sys_moments.argtypes = [dp, C.c_int, dp, C.c_int, C.c_int, dp, dp]
        L.oracle_flash_moments.argtypes = [dp, C.c_int, dp, C.c_int, C.c_int, C.c_int, dp, dp]
        L.oracle_bernoulli_coefs.argtypes = [fp, C.c_int, fp, C.c_int, ip, fp]
        L.oracle_bernoulli_logits.argtypes = [P, vp, vp, C.c_int, C.c_int, fp, C.c_int, C.c_int, dp]
        L.oracle_bernoulli_features.argtypes = [P, vp, C.c_int, C.c_int, fp, ip]
        L.oracle_santa_prop_bernoulli.argtypes = [P, vp, vp, vp, C.c_int, fp, C.c_int, C.c_int, fp,
                                                  dp, ip, dp, ip]
        L.oracle_num_threads.restype = C.c_int
        L.oracle_set_num_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _dptr(a):
    return a.ctypes.data_as(C.POINTER(C.c_double)) if a is not None else None


def _iptr(a):
    return a.ctypes.data_as(C.POINTER(C.c_int)) if a is not None else None


class Problem:
    """Shapes and layout of one decode-attention call, for the oracle.

    Built from the generic fields of an input instance; keeps the host arrays
    it points to alive.
    """

    def __init__(self, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, *,
                 q_dtype, kv_dtype, scale, tile_len, seq_lens=None, page_size=0,
                 page_table=None):
        self._seq = None if seq_lens is None else np.ascontiguousarray(seq_lens, np.int32)
        self._pt = None if page_table is None else np.ascontiguousarray(page_table, np.int32)
        self.s = _Problem(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                          _iptr(self._seq), FORMATS[q_dtype], FORMATS[kv_dtype], page_size,
                          _iptr(self._pt), 0 if self._pt is None else self._pt.shape[1],
                          float(np.float32(scale)), tile_len)
        self.batch, self.num_q_heads, self.head_dim = batch, num_q_heads, head_dim
        self.tile_len = tile_len
        self.max_seq_len = max_seq_len
        self.seq_lens = self._seq

    @classmethod
    def from_inputs(cls, inp, tile_len=None):
        c = inp.cfg
        paged = c.page_size > 0
        ragged = paged or not inp.uniform_len
        return cls(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.seq_len,
                   q_dtype=c.q_dtype, kv_dtype=c.kv_dtype,
                   scale=inp.scale, tile_len=tile_len or c.tile_len,
                   seq_lens=inp.seq_lens if ragged else None, page_size=c.page_size,
                   page_table=inp.page_table if paged else None)

    @property
    def ref(self):
        return C.byref(self.s)

    def max_tiles(self):
        lens = self.seq_lens if self.seq_lens is not None else [self.max_seq_len]
        return max((int(n) + self.tile_len - 1) // self.tile_len for n in lens)


def _vp(a):
    return C.c_void_p(a.ctypes.data)


def logits(prob: Problem, q, k, b, h):
    n = prob.max_seq_len if prob.seq_lens is None else int(prob.seq_lens[b])
    x = np.empty(n, np.float64)
    lib().oracle_logits(prob.ref, _vp(q), _vp(k), b, h, _dptr(x))
    return x


def softmax_weights(x):
    x = np.ascontiguousarray(x, np.float64)
    e = np.empty_like(x)
    m = C.c_double()
    z = lib().oracle_softmax_weights(_dptr(x), x.size, _dptr(e), C.byref(m))
    return e, z, m.value


def invert_cdf(w, t):
    """Indices J_m = min{j : F(j) > t_m} and boundary distances."""
    w = np.ascontiguousarray(w, np.float64)
    t = np.ascontiguousarray(t, np.float64)
    idx = np.empty(t.size, np.int32)
    dl = np.empty(t.size, np.float64)
    rc = lib().oracle_invert_cdf(_dptr(w), w.size, _dptr(t), t.size, _iptr(idx), _dptr(dl))
    if rc:
        raise ValueError(f"oracle_invert_cdf: {rc}")
    return idx, dl


def cell_edges(w, tok):
    """CDF cells [F(j-1), F(j)) of the tokens `tok` for weights w (NaN
    outside [0, n))."""
    w = np.ascontiguousarray(w, np.float64)
    tok = np.ascontiguousarray(tok, np.int32)
    lo = np.empty(tok.size, np.float64)
    hi = np.empty(tok.size, np.float64)
    rc = lib().oracle_cell_edges(_dptr(w), w.size, _iptr(tok), tok.size, _dptr(lo), _dptr(hi))
    if rc:
        raise ValueError(f"oracle_cell_edges: {rc}")
    return lo, hi


def prop_cells(prob: "Problem", q, k, S, u, tok, sampler="sys", draws=0, group_mean=0, ub=None):
    """For each head and threshold position m: the threshold t_m of prop's
    generator and the cell [lo, hi) of token tok[bh, m] in the head's
    (untiled) CDF; on Bernoulli scores when draws > 0.  Returns (thr, lo, hi)
    [B*Hq, S] (NaN for empty requests and for tokens outside the request)."""
    BH = prob.batch * prob.num_q_heads
    u = np.ascontiguousarray(u, np.float32)
    tok = np.ascontiguousarray(tok, np.int32).reshape(BH, S)
    thr, lo, hi = (np.empty((BH, S), np.float64) for _ in range(3))
    ubp = None if ub is None else _fptr(np.ascontiguousarray(ub, np.float32))
    rc = lib().oracle_prop_cells(prob.ref, _vp(q), _vp(k), S, SAMPLERS[sampler], _fptr(u), int(draws),
                                 int(group_mean), ubp, _iptr(tok), _dptr(thr), _dptr(lo), _dptr(hi))
    if rc:
        raise ValueError(f"oracle_prop_cells: {rc}")
    return thr, lo, hi


def flash_cells(prob: "Problem", q, k, S, u, tok, sampler="sys"):
    """As prop_cells for flash: position m belongs to tile m // S_f, and the
    cell is that of tok[bh, m] in the tile's own CDF (NaN outside the tile)."""
    BH = prob.batch * prob.num_q_heads
    u = np.ascontiguousarray(u, np.float32)
    tok = np.ascontiguousarray(tok, np.int32).reshape(BH, S)
    thr, lo, hi = (np.empty((BH, S), np.float64) for _ in range(3))
    rc = lib().oracle_flash_cells(prob.ref, _vp(q), _vp(k), S, SAMPLERS[sampler], _fptr(u), _iptr(tok),
                                  _dptr(thr), _dptr(lo), _dptr(hi))
    if rc:
        raise ValueError(f"oracle_flash_cells: {rc}")
    return thr, lo, hi


def sys_thresholds(U, S):
    t = np.empty(S, np.float64)
    lib().oracle_sys_thresholds(float(U), S, _dptr(t))
    return t


def strat_thresholds(u01):
    u01 = np.ascontiguousarray(u01, np.float64)
    t = np.empty_like(u01)
    lib().oracle_strat_thresholds(_dptr(u01), u01.size, _dptr(t))
    return t


def iid_thresholds(u01):
    u01 = np.ascontiguousarray(u01, np.float64)
    t = np.empty_like(u01)
    lib().oracle_iid_thresholds(_dptr(u01), u01.size, _dptr(t))
    return t


def estimate_from_weights(w, V, t):
    w = np.ascontiguousarray(w, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    t = np.ascontiguousarray(t, np.float64)
    out = np.empty(V.shape[1], np.float64)
    rc = lib().oracle_estimate_from_weights(_dptr(w), w.size, _dptr(V), V.shape[1],
                                            _dptr(t), t.size, _dptr(out))
    if rc:
        raise ValueError(f"oracle_estimate_from_weights: {rc}")
    return out


def sys_moments(w, V, S):
    """Exact E_U and trace Cov_U of the systematic estimator on weights w."""
    w = np.ascontiguousarray(w, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    mean = np.empty(V.shape[1], np.float64)
    var = C.c_double()
    rc = lib().oracle_sys_moments(_dptr(w), w.size, _dptr(V), V.shape[1], S, _dptr(mean), C.byref(var))
    if rc:
        raise ValueError(f"oracle_sys_moments: {rc}")
    return mean, var.value


def flash_moments(w, V, S, T):
    w = np.ascontiguousarray(w, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    mean = np.empty(V.shape[1], np.float64)
    var = C.c_double()
    rc = lib().oracle_flash_moments(_dptr(w), w.size, _dptr(V), V.shape[1], S, T,
                                    _dptr(mean), C.byref(var))
    if rc:
        raise ValueError(f"oracle_flash_moments: {rc}")
    return mean, var.value


def santa_prop(prob: Problem, q, k, v, S, u):
    """S2ANTA-prop (= untiled systematic sampling).  Returns dict of arrays."""
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    u = np.ascontiguousarray(u, np.float32)
    out = np.empty((BH, d), np.float64)
    idx = np.empty((BH, S), np.int32)
    dl = np.empty((BH, S), np.float64)
    mnt = prob.max_tiles()
    tc = np.empty((BH, mnt), np.int32)
    rc = lib().oracle_santa_prop(prob.ref, _vp(q), _vp(k), _vp(v), S,
                                 u.ctypes.data_as(C.POINTER(C.c_float)),
                                 _dptr(out), _iptr(idx), _dptr(dl), _iptr(tc))
    if rc:
        raise ValueError(f"oracle_santa_prop: {rc}")
    return {"out": out, "idx": idx, "delta": dl, "tile_counts": tc}


SAMPLERS = {"sys": 0, "strat": 1, "iid": 2}


def santa_prop_sampler(prob: Problem, q, k, v, S, sampler, u):
    """S2ANTA-prop with the "sys", "strat" or "iid" threshold generator.
    u: [B*Hq] offsets in [0, 1/S) for sys, [B*Hq, S] uniforms in [0,1) else."""
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    u = np.ascontiguousarray(u, np.float32)
    out = np.empty((BH, d), np.float64)
    idx = np.empty((BH, S), np.int32)
    dl = np.empty((BH, S), np.float64)
    mnt = prob.max_tiles()
    tc = np.empty((BH, mnt), np.int32)
    rc = lib().oracle_santa_prop_sampler(prob.ref, _vp(q), _vp(k), _vp(v), S, SAMPLERS[sampler],
                                         u.ctypes.data_as(C.POINTER(C.c_float)),
                                         _dptr(out), _iptr(idx), _dptr(dl), _iptr(tc))
    if rc:
        raise ValueError(f"oracle_santa_prop_sampler: {rc}")
    return {"out": out, "idx": idx, "delta": dl, "tile_counts": tc}


def santa_flash(prob: Problem, q, k, v, S, u):
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    nt = prob.max_tiles()
    u = np.ascontiguousarray(u, np.float32)
    out = np.empty((BH, d), np.float64)
    idx = np.empty((BH, S), np.int32)
    dl = np.empty((BH, S), np.float64)
    pt = np.empty((BH, nt), np.float64)
    rc = lib().oracle_santa_flash(prob.ref, _vp(q), _vp(k), _vp(v), S,
                                  u.ctypes.data_as(C.POINTER(C.c_float)),
                                  _dptr(out), _iptr(idx), _dptr(dl), _dptr(pt))
    if rc:
        raise ValueError(f"oracle_santa_flash: {rc}")
    return {"out": out, "idx": idx, "delta": dl, "ptile": pt}


def santa_flash_sampler(prob: Problem, q, k, v, S, sampler, u):
    """S2ANTA-flash with the "sys", "strat" or "iid" generator per tile.
    u: [B*Hq] offsets for sys; [B*Hq, S] uniforms (tile-major) otherwise."""
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    nt = prob.max_tiles()
    u = np.ascontiguousarray(u, np.float32)
    out = np.empty((BH, d), np.float64)
    idx = np.empty((BH, S), np.int32)
    dl = np.empty((BH, S), np.float64)
    pt = np.empty((BH, nt), np.float64)
    rc = lib().oracle_santa_flash_sampler(prob.ref, _vp(q), _vp(k), _vp(v), S, SAMPLERS[sampler],
                                          u.ctypes.data_as(C.POINTER(C.c_float)),
                                          _dptr(out), _iptr(idx), _dptr(dl), _dptr(pt))
    if rc:
        raise ValueError(f"oracle_santa_flash_sampler: {rc}")
    return {"out": out, "idx": idx, "delta": dl, "ptile": pt}


def exact(prob: Problem, q, k, v):
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    out = np.empty((BH, d), np.float64)
    rc = lib().oracle_exact(prob.ref, _vp(q), _vp(k), _vp(v), _dptr(out))
    if rc:
        raise ValueError(f"oracle_exact: {rc}")
    return out


def replay(prob: Problem, v, S, idx, ptile=None):
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    idx = np.ascontiguousarray(idx, np.int32).reshape(BH, S)
    out = np.empty((BH, d), np.float64)
    nt = 0
    if ptile is not None:
        ptile = np.ascontiguousarray(ptile, np.float64)
        nt = ptile.shape[-1]
    rc = lib().oracle_replay(prob.ref, _vp(v), S, _iptr(idx), _dptr(ptile), nt, _dptr(out))
    if rc:
        raise ValueError(f"oracle_replay: {rc}")
    return out


def _fptr(a):
    return a.ctypes.data_as(C.POINTER(C.c_float))


def bernoulli_coefs(qf, u, draws):
    """Ternary coefficients c [d] (sum of `draws` draws), the scale a and the
    number of nonzero c for one fp32 query qf [d] and uniforms u [draws, d]."""
    qf = np.ascontiguousarray(qf, np.float32)
    u = np.ascontiguousarray(u, np.float32).reshape(draws, qf.size)
    c = np.empty(qf.size, np.int32)
    a = C.c_float()
    nz = lib().oracle_bernoulli_coefs(_fptr(qf), qf.size, _fptr(u), draws, _iptr(c), C.byref(a))
    if nz < 0:
        raise ValueError("oracle_bernoulli_coefs: uniform outside [0, 1)")
    return c, a.value, nz


def bernoulli_logits(prob: Problem, q, k, draws, group_mean, ub, b, h):
    """Bernoulli-estimated scores of head h of request b (fp64)."""
    n = prob.max_seq_len if prob.seq_lens is None else int(prob.seq_lens[b])
    x = np.empty(n, np.float64)
    ub = np.ascontiguousarray(ub, np.float32)
    nz = lib().oracle_bernoulli_logits(prob.ref, _vp(q), _vp(k), draws, int(group_mean), _fptr(ub),
                                       b, h, _dptr(x))
    if nz < 0:
        raise ValueError("oracle_bernoulli_logits: uniform outside [0, 1)")
    return x, nz


def bernoulli_features(prob: Problem, q, draws, group_mean, ub):
    """Features read per KV group [B*Hkv]: the union over its heads."""
    nread = np.empty(prob.batch * prob.s.num_kv_heads, np.int32)
    ub = np.ascontiguousarray(ub, np.float32)
    rc = lib().oracle_bernoulli_features(prob.ref, _vp(q), draws, int(group_mean), _fptr(ub),
                                         _iptr(nread))
    if rc:
        raise ValueError(f"oracle_bernoulli_features: {rc}")
    return nread


def santa_prop_bernoulli(prob: Problem, q, k, v, S, u, draws, group_mean, ub):
    """S2ANTA-prop (systematic) on Bernoulli qK^T scores."""
    BH, d = prob.batch * prob.num_q_heads, prob.head_dim
    u = np.ascontiguousarray(u, np.float32)
    ub = np.ascontiguousarray(ub, np.float32)
    out = np.empty((BH, d), np.float64)
    idx = np.empty((BH, S), np.int32)
    dl = np.empty((BH, S), np.float64)
    tc = np.empty((BH, prob.max_tiles()), np.int32)
    rc = lib().oracle_santa_prop_bernoulli(prob.ref, _vp(q), _vp(k), _vp(v), S, _fptr(u), draws,
                                           int(group_mean), _fptr(ub), _dptr(out), _iptr(idx),
                                           _dptr(dl), _iptr(tc))
    if rc:
        raise ValueError(f"oracle_santa_prop_bernoulli: {rc}")
    return {"out": out, "idx": idx, "delta": dl, "tile_counts": tc}


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    lib().oracle_set_num_threads(int(n))


def timed(fn, *args, reps=1, **kw):
    """Run fn reps times; return (last result, list of wall seconds)."""
    secs = []
    res = None
    for _ in range(reps):
        t0 = time.perf_counter()
        res = fn(*args, **kw)
        secs.append(time.perf_counter() - t0)
    return res, secs
