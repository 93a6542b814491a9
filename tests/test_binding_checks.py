"""The Python binding rejects malformed tensors before any pointer reaches
the library (CPU tensors only: every check here fires on the host)."""
import pytest
import torch

import stochastic_sparse_attention_amd as sa

B, HQ, HKV, D, N, T, S = 2, 8, 2, 128, 1000, 256, 16
NT = (N + T - 1) // T


def _problem(**kw):
    args = dict(dtype="bf16", scale=D ** -0.5, tile_len=T)
    args.update(kw)
    return sa.Problem(B, HQ, HKV, D, N, **args)


def _ok():
    return dict(q=torch.zeros(B, HQ, D, dtype=torch.bfloat16),
                k=torch.zeros(B, HKV, N, D, dtype=torch.bfloat16),
                v=torch.zeros(B, HKV, N, D, dtype=torch.bfloat16),
                u=torch.zeros(B * HQ, dtype=torch.float32),
                out=torch.zeros(B * HQ, D, dtype=torch.float32),
                sample_idx=torch.zeros(B * HQ, S, dtype=torch.int32),
                tile_budget=torch.zeros(B * HQ, NT, dtype=torch.int32))


def _prop(p, a):
    return sa.santa_decode_prop(p, a["q"], a["k"], a["v"], S, a["u"], a["out"], a["sample_idx"],
                                a["tile_budget"])


@pytest.mark.parametrize("name,bad,msg", [
    ("q", torch.zeros(B, HQ, D, dtype=torch.float32), "dtype"),
    ("q", torch.zeros(B, HQ, D - 1, dtype=torch.bfloat16), "elements"),
    ("k", torch.zeros(B, HKV, N, D, dtype=torch.int16), "dtype"),
    ("v", torch.zeros(B, HKV, N - 1, D, dtype=torch.bfloat16), "elements"),
    ("u", torch.zeros(B * HQ - 1, dtype=torch.float32), "elements"),
    ("u", torch.zeros(B * HQ, dtype=torch.float64), "dtype"),
    ("out", torch.zeros(B * HQ, D, dtype=torch.bfloat16), "dtype"),
    ("out", torch.zeros(B * HQ, D - 1, dtype=torch.float32), "elements"),
    ("out", torch.zeros(D, B * HQ, dtype=torch.float32).t(), "contiguous"),
    ("sample_idx", torch.zeros(B * HQ, S, dtype=torch.int64), "dtype"),
    ("sample_idx", torch.zeros(B * HQ, S - 1, dtype=torch.int32), "elements"),
    ("tile_budget", torch.zeros(B * HQ, NT - 1, dtype=torch.int32), "elements"),
])
def test_prop_rejects_malformed(name, bad, msg):
    a = _ok()
    a[name] = bad
    with pytest.raises(ValueError, match=msg):
        _prop(_problem(), a)


def test_well_formed_cpu_tensors_are_rejected_for_their_device():
    with pytest.raises(ValueError, match="expected a GPU"):
        _prop(_problem(), _ok())


def test_problem_tensors_are_checked():
    with pytest.raises(ValueError, match="int32"):
        _problem(seq_lens=torch.zeros(B, dtype=torch.int64))
    with pytest.raises(ValueError, match="entries"):
        _problem(seq_lens=torch.zeros(B + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        _problem(page_size=16, page_table=torch.zeros(B, 63, dtype=torch.int64))
    with pytest.raises(ValueError, match="page table"):
        _problem(page_size=16)
    # a paged pool must hold whole pages
    p = _problem(page_size=16, page_table=torch.zeros(B, 63, dtype=torch.int32))
    a = _ok()
    a["k"] = torch.zeros(10 * HKV * 16 * D + 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="whole pages"):
        _prop(p, a)


def test_list_samplers_need_S_uniforms_per_head():
    a = _ok()
    with pytest.raises(ValueError, match="elements"):
        sa.santa_decode_prop_sampler(_problem(), a["q"], a["k"], a["v"], S, "strat", a["u"], a["out"])
    with pytest.raises(ValueError, match="sampler"):
        sa.santa_decode_prop_sampler(_problem(), a["q"], a["k"], a["v"], S, "bogus", a["u"], a["out"])


def test_fp8_kv_and_exact_and_bernoulli_checks():
    p = _problem(kv_dtype="fp8")
    a = _ok()
    with pytest.raises(ValueError, match="dtype"):
        sa.exact_decode_ref(p, a["q"], a["k"], a["v"], a["out"])       # bf16 K for an e4m3 cache
    k8 = torch.zeros(B, HKV, N, D, dtype=torch.uint8)
    with pytest.raises(ValueError, match="expected a GPU"):
        sa.exact_decode_ref(p, a["q"], k8, k8, a["out"])
    with pytest.raises(ValueError, match="u_bern"):
        sa.santa_decode_prop_bernoulli(_problem(), a["q"], a["k"], a["v"], S, a["u"], 4, 1,
                                       torch.zeros(B * HKV * 4 * D - 1, dtype=torch.float32), a["out"])
    with pytest.raises(ValueError, match="features_read"):
        sa.santa_decode_prop_bernoulli(_problem(), a["q"], a["k"], a["v"], S, a["u"], 4, 1,
                                       torch.zeros(B * HKV * 4 * D, dtype=torch.float32), a["out"],
                                       features_read=torch.zeros(B * HKV, dtype=torch.int64))


def test_workspace_is_checked():
    a = _ok()
    small = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="expected a GPU"):      # tensors first, then their device
        sa.santa_decode_prop(_problem(), a["q"], a["k"], a["v"], S, a["u"], a["out"], workspace=small)
