"""Host-only checks of the C ABI (no GPU needed): every entry point declared
in include/santa.h is exported by libsanta.so, workspace sizing follows the
documented layout, and every validation error returns its status before any
launch (device pointers below are dummies that must never be dereferenced)."""
import ctypes as C
import os
import re

import pytest

from stochastic_sparse_attention_amd import _lib
from stochastic_sparse_attention_amd._lib import santa_problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
PROP, FLASH, EXACT = 0, 1, 2
DUMMY = C.c_void_p(0x100000)          # never dereferenced: validation fails first
OUT = C.c_void_p(0x300000000)         # an output apart from every input


def _header_functions():
    src = open(os.path.join(ROOT, "include", "santa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_exported(lib):
    names = _header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def _problem(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_seq_len=32768,
                seq_lens=None, q_dtype=1, kv_dtype=1, page_size=0, page_table=None,
                max_pages_per_seq=0, scale=128 ** -0.5, tile_len=256)
    base.update(kw)
    return santa_problem(**base)


def _wsize(lib, p, variant, S):
    n = C.c_size_t(0)
    st = lib.santa_workspace_size(C.byref(p), variant, S, C.byref(n))
    return st, n.value


def _prop(lib, p, S=128, ws_bytes=1 << 30, ws=DUMMY, out=OUT, u=DUMMY, q=DUMMY):
    return lib.santa_decode_prop(C.byref(p), q, DUMMY, DUMMY, S, u, out, None, None, ws, ws_bytes, None)


def _flash(lib, p, S=2048, ws_bytes=1 << 30):
    return lib.santa_decode_flash(C.byref(p), DUMMY, DUMMY, DUMMY, S, DUMMY, OUT, None, None, DUMMY,
                                  ws_bytes, None)


def _exact(lib, p, ws_bytes=1 << 30, out=OUT):
    return lib.exact_decode_ref(C.byref(p), DUMMY, DUMMY, DUMMY, out, DUMMY, ws_bytes, None)


def test_workspace_sizes_follow_layout(lib):
    p = _problem()
    st, n = _wsize(lib, p, PROP, 128)
    assert st == OK
    BH, nt = 32, 128
    sync = _lib.SANTA_SYNC_BYTES                           # every variant starts with the counters
    stash = BH * 32768 * 4
    stats = BH * nt * 8
    assert n == sync + stash + stats                       # all 256-byte multiples
    st, n = _wsize(lib, p, EXACT, 0)
    assert st == OK and n == sync + 2 * BH * nt * 4 + BH * nt * 128 * 4
    st, n2 = _wsize(lib, p, FLASH, 2048)
    assert st == OK and n2 == n
    # stash rows are padded to a multiple of the tile length
    st, n = _wsize(lib, _problem(max_seq_len=1000), PROP, 16)
    assert st == OK and n >= 32 * 1024 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=30), INVALID),                     # Hq % Hkv != 0
    (dict(num_q_heads=0), INVALID),
    (dict(max_seq_len=0), INVALID),
    (dict(tile_len=100), INVALID),                       # not a multiple of 64
    (dict(tile_len=192), UNSUPPORTED),                   # multiple of 64, not built
    (dict(head_dim=64), UNSUPPORTED),
    (dict(q_dtype=0), UNSUPPORTED),                      # q and KV dtypes differ
    (dict(q_dtype=0, kv_dtype=2), UNSUPPORTED),          # e4m3 KV needs bf16 q
    (dict(q_dtype=2, kv_dtype=2), INVALID),              # e4m3 is a KV storage only
    (dict(kv_dtype=7), INVALID),
    (dict(num_q_heads=24), UNSUPPORTED),                 # group of 3
    (dict(scale=0.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(page_size=8, page_table=0x1000, max_pages_per_seq=4096), INVALID),
    (dict(page_size=16), INVALID),                       # paged without a table
    (dict(page_size=16, page_table=0x1000, max_pages_per_seq=10), INVALID),
    (dict(max_seq_len=1024 * 256 + 1), UNSUPPORTED),     # more than 1024 tiles
])
def test_problem_validation(lib, kw, code):
    p = _problem(**kw)
    assert _prop(lib, p) == code
    assert _exact(lib, p) == code
    assert _wsize(lib, p, PROP, 128)[0] == code


def test_sample_count_validation(lib):
    p = _problem()
    assert _prop(lib, p, S=0) == INVALID
    assert _prop(lib, p, S=4097) == UNSUPPORTED
    assert _prop(lib, p, S=70000) == INVALID
    assert _flash(lib, p, S=100) == INVALID              # 100 % 128 tiles != 0
    assert _flash(lib, p, S=128 * 300) == UNSUPPORTED    # 300 samples per 256-token tile
    assert _flash(lib, _problem(seq_lens=0x2000)) == INVALID   # ragged flash


def test_fp8_kv_accepted(lib):
    p = _problem(kv_dtype=2)                             # bf16 q, e4m3 K/V
    st, n = _wsize(lib, p, PROP, 128)
    assert st == OK and n == _wsize(lib, _problem(), PROP, 128)[1]
    assert _prop(lib, p, ws_bytes=10) == WORKSPACE        # reaches the workspace check


def test_sampler_validation(lib):
    p = _problem()
    for bad in (-1, 3, 99):
        assert lib.santa_decode_prop_sampler(C.byref(p), DUMMY, DUMMY, DUMMY, 128, bad, DUMMY, OUT, None,
                                             None, DUMMY, 1 << 30, None) == INVALID
    # the sampler call shares the problem and workspace checks of prop
    assert lib.santa_decode_prop_sampler(C.byref(_problem(tile_len=100)), DUMMY, DUMMY, DUMMY, 128, 1, DUMMY,
                                         OUT, None, None, DUMMY, 1 << 30, None) == INVALID
    assert lib.santa_decode_prop_sampler(C.byref(p), DUMMY, DUMMY, DUMMY, 128, 2, DUMMY, OUT, None, None,
                                         DUMMY, 10, None) == WORKSPACE
    assert lib.santa_decode_prop_sampler(C.byref(_problem(batch=0)), DUMMY, DUMMY, DUMMY, 128, 1, DUMMY,
                                         OUT, None, None, DUMMY, 1 << 30, None) == OK


def test_pointer_and_workspace_validation(lib):
    p = _problem()
    need = _wsize(lib, p, PROP, 128)[1]
    assert _prop(lib, p, out=None) == INVALID
    assert _prop(lib, p, u=None) == INVALID
    assert _prop(lib, p, q=None) == INVALID
    assert _prop(lib, p, ws_bytes=need - 1) == WORKSPACE
    assert _prop(lib, p, ws=None) == WORKSPACE
    assert _prop(lib, p, ws=C.c_void_p(0x100010)) == WORKSPACE   # not 256-byte aligned
    assert _exact(lib, p, ws_bytes=10) == WORKSPACE
    assert _exact(lib, p, out=None) == INVALID
    assert lib.santa_decode_prop(None, DUMMY, DUMMY, DUMMY, 128, DUMMY, DUMMY, None, None, DUMMY,
                                 1 << 30, None) == INVALID
    n = C.c_size_t(0)
    assert lib.santa_workspace_size(C.byref(p), 9, 128, C.byref(n)) == INVALID
    assert lib.santa_workspace_size(C.byref(p), PROP, 128, None) == INVALID


def test_output_overlapping_an_input_is_rejected(lib):
    """`out` may not share a byte with q or with the B*Hq offsets of u (prop
    clears output rows while other workgroups still read the query).  The
    workspace is too small throughout, so a call that passed the overlap
    check would stop at WORKSPACE before any launch."""
    p = _problem()                                   # q: 32*128 bf16 = 8 KiB; out: 16 KiB; u: 128 B
    q0 = 0x200000000
    for out in (q0, q0 + 8191, q0 - 16383):          # first byte, last byte, overlap from below
        assert _prop(lib, p, ws_bytes=10, q=C.c_void_p(q0), out=C.c_void_p(out)) == INVALID
        assert _exact(lib, p, ws_bytes=10, out=C.c_void_p(out)) == WORKSPACE   # q is DUMMY there
    for out in (q0 + 8192, q0 - 16384):              # adjacent on either side: allowed
        assert _prop(lib, p, ws_bytes=10, q=C.c_void_p(q0), out=C.c_void_p(out)) == WORKSPACE
    assert _prop(lib, p, ws_bytes=10, u=C.c_void_p(0x400000040), out=C.c_void_p(0x400000000)) == INVALID
    assert _prop(lib, p, ws_bytes=10, u=C.c_void_p(0x400004000), out=C.c_void_p(0x400000000)) == WORKSPACE
    assert lib.exact_decode_ref(C.byref(p), DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 10, None) == INVALID
    assert lib.santa_decode_flash(C.byref(p), DUMMY, DUMMY, DUMMY, 2048, OUT, DUMMY, None, None, DUMMY, 10,
                                  None) == INVALID                    # out == q
    assert lib.santa_decode_prop_fused(C.byref(p), DUMMY, DUMMY, DUMMY, 128, DUMMY, DUMMY, None, None, DUMMY,
                                       10, None) == INVALID
    assert _bern(lib, p, ws_bytes=10) == WORKSPACE
    assert lib.santa_decode_prop_bernoulli(C.byref(p), DUMMY, DUMMY, DUMMY, 128, DUMMY, 4, 0, DUMMY, DUMMY,
                                           None, None, None, DUMMY, 10, None) == INVALID


def test_empty_batch_is_a_noop(lib):
    p = _problem(batch=0)
    # nothing is launched, so dummy pointers are fine
    assert _prop(lib, p) == OK
    assert _flash(lib, p) == OK
    assert _exact(lib, p) == OK


def test_status_strings_and_version(lib):
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, 12):
        assert isinstance(_lib.status_string(code), str) and _lib.status_string(code)
    assert lib.santa_abi_version() >= 3
    assert lib.santa_set_timing_events(None, None) == OK


def test_binding_raises_on_error(lib):
    import stochastic_sparse_attention_amd as sa
    prob = sa.Problem(1, 32, 8, 64, 1024, dtype="bf16", scale=0.125, tile_len=256)
    with pytest.raises(sa.SantaError) as ei:
        sa.santa_workspace_size(prob, "prop", 128)
    assert ei.value.status == UNSUPPORTED


def _bern(lib, p, S=128, draws=4, gm=0, kf=DUMMY, ub=DUMMY, ws_bytes=1 << 30):
    return lib.santa_decode_prop_bernoulli(C.byref(p), DUMMY, kf, DUMMY, S, DUMMY, draws, gm, ub, OUT,
                                           None, None, None, DUMMY, ws_bytes, None)


def test_bernoulli_entry_validates_before_launch(lib):
    """Every case below must fail (or, for B = 0, succeed) before a launch."""
    p = _problem()
    assert _bern(lib, p, draws=0) == INVALID
    assert _bern(lib, p, draws=65) == INVALID
    assert _bern(lib, p, gm=2) == INVALID
    assert _bern(lib, _problem(q_dtype=0, kv_dtype=0)) == UNSUPPORTED      # fp32 not built here
    assert _bern(lib, _problem(kv_dtype=2), kf=C.c_void_p(0x100002)) == INVALID   # e4m3 rows: 4-byte aligned
    assert _bern(lib, _problem(kv_dtype=2, page_size=16, page_table=0x100000,
                               max_pages_per_seq=2048)) == UNSUPPORTED
    assert _bern(lib, _problem(page_size=16, page_table=0x100000, max_pages_per_seq=2048)) == UNSUPPORTED
    assert _bern(lib, _problem(max_seq_len=1022)) == UNSUPPORTED           # rows not 8-byte aligned
    assert _bern(lib, p, kf=C.c_void_p(0x100002)) == INVALID
    assert _bern(lib, p, kf=None) == INVALID
    assert _bern(lib, p, ub=None) == INVALID
    assert _bern(lib, p, ws_bytes=16) == WORKSPACE
    assert _bern(lib, p, S=5000) == UNSUPPORTED
    assert _bern(lib, _problem(batch=0)) == OK


def _prop_fused(lib, p, S=128, ws_bytes=1 << 30):
    return lib.santa_decode_prop_fused(C.byref(p), DUMMY, DUMMY, DUMMY, S, DUMMY, OUT, None, None, DUMMY,
                                       ws_bytes, None)


def test_single_launch_prop_limits(lib):
    """The single-launch prop needs one arrival counter per (request, KV
    group) in the workspace's SANTA_SYNC_BYTES (64 bytes apart); beyond that
    it returns SANTA_ERR_UNSUPPORTED before any launch."""
    groups = _lib.SANTA_SYNC_BYTES // 64
    assert _prop_fused(lib, _problem(batch=groups // 8 + 1)) == UNSUPPORTED      # 8 KV heads per request
    assert _prop_fused(lib, _problem(batch=groups // 8), ws_bytes=16) == WORKSPACE
    assert _prop_fused(lib, _problem(batch=0)) == OK
