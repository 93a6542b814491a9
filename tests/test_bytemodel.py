"""Byte-model pins against the arithmetic the SANTA notes print."""
import numpy as np

from stochastic_sparse_attention_amd import bytemodel as BM
from stochastic_sparse_attention_amd import synth


def test_kv_bytes_llama_32k_is_128_mib():
    """Background: ~128 MB of KV per layer per decode token at 32k (Llama-3.1-8B)."""
    cfg = synth.CONFIGS[2]
    assert 2 * BM.kv_bytes(cfg) == 128 * 2 ** 20
    assert BM.exact_step_bytes(cfg)["partial"] >= 128 * 2 ** 20


def test_budget_fractions():
    """key design 2 / Table 1: S=128 is 0.39% of 32k keys, S=2048 is 6.25%; flash uses 16x."""
    assert round(128 / 32768 * 100, 2) == 0.39
    assert 2048 / 32768 == 0.0625
    assert 2048 // 128 == 16
    # union bound behind the "<1.56%" V-row figure: G*S/n_k for a group of 4
    assert 4 * 128 / 32768 == 0.015625


def test_prop_bytes_cfg2():
    cfg = synth.CONFIGS[2]
    nt = 32768 // 256
    tb = np.zeros((32, nt), np.int32)
    tb[:, :50] = 1                       # 50 visited tiles per head
    tb[:, 0] += 128 - 50
    b = BM.prop_step_bytes(cfg, 128, tb)
    assert b["pass1"] == 64 * 2 ** 20 + 4 * 2 ** 20 + 32 * nt * 8 + 32 * 128 * 2
    assert b["stash_reread"] == 32 * 50 * 256 * 4
    assert b["v_rows"] == 32 * 128 * 256
    assert 72e6 < b["total"] < 77e6


def test_v_row_fraction_counts_distinct_rows():
    cfg = synth.small_config(2, seq_len=1000, num_q_heads=4, num_kv_heads=1)
    idx = np.array([[1, 1, 2], [2, 3, 3], [5, 5, 5], [1, 2, 3]])
    assert BM.v_row_fraction(idx, cfg) == 4 / 1000


def test_bernoulli_pass1_bytes():
    """All features kept: pass 1's bytes plus the uniforms; half kept with the
    mean query: half of K and three quarters of the stash less."""
    from stochastic_sparse_attention_amd import bytemodel as BM
    cfg = synth.CONFIGS[2]
    G, d = 8, cfg.head_dim
    full = BM.bernoulli_pass1_bytes(cfg, np.full(G, d), 4, False)
    assert full == BM.prop_pass1_bytes(cfg) + 32 * 4 * d * 4
    half = BM.bernoulli_pass1_bytes(cfg, np.full(G, d // 2), 4, True)
    stash_saved = 32768 * (32 - 8) * 4          # the mean query writes one stash row per group
    assert half == BM.prop_pass1_bytes(cfg) - BM.kv_bytes(cfg) // 2 + 8 * 4 * d * 4 - stash_saved
