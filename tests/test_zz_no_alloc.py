"""santa_decode_prop_static, the allocation-free prop entry point, against
santa_decode_prop (the same kernels with a caller workspace): bitwise equal
outputs, indices and budgets on two calls in a row, the second smaller, so
that the second call runs on scratch the first one filled."""
import ctypes as C

import numpy as np
import pytest

from stochastic_sparse_attention_amd import synth


def _problem_struct(batch, seq_len):
    from stochastic_sparse_attention_amd._lib import santa_problem
    return santa_problem(batch, 32, 8, 128, seq_len, None, 1, 1, 0, None, 0, 128 ** -0.5, 256)


def test_static_rejects_problems_above_its_scratch():
    """32k tokens, 32/8 heads, S = 128: batch 7 fits the 32 MiB scratch,
    batch 8 does not and is refused before anything touches a device."""
    import stochastic_sparse_attention_amd._lib as L
    lib = L.load()
    dummy = C.c_void_p(0x100000)          # never dereferenced: refused on the host
    for batch, want in ((8, L.SANTA_ERR_TOO_LARGE), (64, L.SANTA_ERR_TOO_LARGE)):
        p = _problem_struct(batch, 32768)
        n = C.c_size_t(0)
        assert lib.santa_workspace_size(C.byref(p), 0, 128, C.byref(n)) == 0
        assert n.value > L.SANTA_STATIC_SCRATCH_BYTES
        st = lib.santa_decode_prop_static(C.byref(p), dummy, dummy, dummy, 128, dummy, dummy, None, None, None)
        assert st == want
    p = _problem_struct(7, 32768)
    n = C.c_size_t(0)
    assert lib.santa_workspace_size(C.byref(p), 0, 128, C.byref(n)) == 0
    assert n.value <= L.SANTA_STATIC_SCRATCH_BYTES
    assert L.status_string(L.SANTA_ERR_TOO_LARGE).startswith("problem needs more workspace")


@pytest.mark.gpu
def test_static_matches_prop_on_two_calls():
    import torch
    import stochastic_sparse_attention_amd as sa
    from stochastic_sparse_attention_amd.device_io import to_device
    assert torch.cuda.is_available()
    sa._lib.load()
    gpu = torch.device("cuda:0")
    cases = [("32k layer, batch 2", synth.small_config(2, batch=2, seq_len=32768), 128),
             ("3000 keys, batch 1", synth.small_config(2, batch=1, seq_len=3000), 64)]
    for name, cfg, S in cases:
        print("static entry point:", name, flush=True)
        dev = to_device(synth.make_inputs(cfg, 51), gpu)
        BH = cfg.batch * cfg.num_q_heads
        nt = (cfg.seq_len + cfg.tile_len - 1) // cfg.tile_len
        res = {}
        for which in ("workspace", "static"):
            out = torch.full((BH, cfg.head_dim), float("nan"), dtype=torch.float32, device=gpu)
            idx = torch.full((BH, S), -7, dtype=torch.int32, device=gpu)
            tb = torch.full((BH, nt), -7, dtype=torch.int32, device=gpu)
            if which == "static":
                sa.santa_decode_prop_static(dev.problem, dev.q, dev.k, dev.v, S, dev.u(S), out, idx, tb)
            else:
                sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, dev.u(S), out, idx, tb)
            torch.cuda.synchronize()
            res[which] = (out.cpu().numpy(), idx.cpu().numpy(), tb.cpu().numpy())
        (o1, i1, t1), (o2, i2, t2) = res["workspace"], res["static"]
        assert np.all(np.isfinite(o2)) and np.all(i2 >= 0) and np.all(t2.sum(1) == S)
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), name
        assert np.array_equal(i1, i2) and np.array_equal(t1, t2), name
