"""ctypes binding of libsanta.so (the C ABI declared in include/santa.h).

Argument marshalling only: tensors are passed as raw device pointers and the
current torch stream as the hipStream_t; every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library has not
been built, loading it raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SANTA_LIB selects another build of the same ABI (e.g. a comparison build);
# by default the in-tree library is loaded
LIB_PATH = os.environ.get("SANTA_LIB") or os.path.join(HERE, "libsanta.so")

SANTA_OK, SANTA_ERR_INVALID, SANTA_ERR_UNSUPPORTED, SANTA_ERR_WORKSPACE, SANTA_ERR_HIP = 0, -1, -2, -3, -4
SANTA_ERR_TOO_LARGE = -5
SANTA_STATIC_SCRATCH_BYTES = 32 << 20
SANTA_SYNC_BYTES = 64 << 10
SANTA_F32, SANTA_BF16, SANTA_FP8_E4M3 = 0, 1, 2
VARIANT = {"prop": 0, "flash": 1, "exact": 2}
SAMPLER = {"sys": 0, "strat": 1, "iid": 2}

EXPORTS = [
    "santa_workspace_size", "santa_decode_prop", "santa_decode_prop_sampler", "santa_decode_flash",
    "santa_decode_flash_sampler", "santa_decode_prop_bernoulli", "exact_decode_ref", "santa_decode_prop_static",
    "santa_decode_prop_fused",
    "santa_set_timing_events", "santa_status_string", "santa_abi_version",
]


class SantaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class santa_problem(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("max_seq_len", C.c_int32),
        ("seq_lens", C.c_void_p),
        ("q_dtype", C.c_int32), ("kv_dtype", C.c_int32),
        ("page_size", C.c_int32), ("page_table", C.c_void_p),
        ("max_pages_per_seq", C.c_int32), ("scale", C.c_float), ("tile_len", C.c_int32),
    ]


_lib = None


def hip_runtimes_mapped():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def load():
    """Load libsanta.so; raises if it is missing (no fallback path exists).

    The library must run on the HIP runtime that torch uses, since the
    tensors, their device pointers and the stream all come from torch.
    torch ships its own libamdhip64 under the same soname as the system one,
    so torch is imported first: the library's dependency then binds to
    torch's copy.  Opening the library first would map a second runtime,
    and every launch would fail on torch's pointers and streams; if two are
    mapped anyway, loading raises."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m stochastic_sparse_attention_amd.build` "
            "(or __graft_entry__.build()) first")
    import torch  # noqa: F401  (its HIP runtime first)
    L = C.CDLL(LIB_PATH)
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"libsanta: more than one HIP runtime is loaded ({runtimes}); the library must "
                          "share torch's, so import torch before anything opens libsanta.so")
    P = C.POINTER(santa_problem)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    L.santa_workspace_size.argtypes = [P, i32, i32, C.POINTER(sz)]
    L.santa_workspace_size.restype = C.c_int
    sampled = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    L.santa_decode_prop.argtypes = sampled
    L.santa_decode_prop.restype = C.c_int
    L.santa_decode_prop_fused.argtypes = sampled
    L.santa_decode_prop_fused.restype = C.c_int
    L.santa_decode_prop_sampler.argtypes = [P, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.santa_decode_prop_sampler.restype = C.c_int
    L.santa_decode_flash.argtypes = sampled
    L.santa_decode_flash_sampler.argtypes = [P, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.santa_decode_flash_sampler.restype = C.c_int
    L.santa_decode_flash.restype = C.c_int
    L.santa_decode_prop_bernoulli.argtypes = [P, vp, vp, vp, i32, vp, i32, i32, vp, vp, vp, vp, vp,
                                              vp, sz, vp]
    L.santa_decode_prop_bernoulli.restype = C.c_int
    L.santa_decode_prop_static.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp]
    L.santa_decode_prop_static.restype = C.c_int
    L.exact_decode_ref.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    L.exact_decode_ref.restype = C.c_int
    L.santa_set_timing_events.argtypes = [vp, vp]
    L.santa_set_timing_events.restype = C.c_int
    L.santa_status_string.argtypes = [C.c_int]
    L.santa_status_string.restype = C.c_char_p
    L.santa_abi_version.restype = C.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().santa_status_string(status).decode()


def _check(fn, status):
    if status != SANTA_OK:
        raise SantaError(fn, status, status_string(status))
