"""Algorithmic HBM bytes of one decode-attention step (what the method must
move), per kernel and per step.

  prop  pass 1:  K (every row once) + stash write (one fp32 per key and q
                 head) + tile stats + q
        reducer: tile stats read + visit records
        pass 2:  stash re-read of the tiles with S_t > 0 + S V rows per q head
                 (counted per sample) + output
  prop on Bernoulli scores, pass 1: the kept features of K only (key
                 design 4), the same stash, stats and q, and the uniforms
  flash tile:    K + S V rows per q head + partials (m, Z, o_t) written
  exact:         K + V (every row once) + partials

The SANTA notes ("Stochastic Sparse Attention for Memory-Bound Inference",
background) put the KV traffic of a Llama-3.1-8B layer at 32k context near
128 MB per decode token; here that is 2 * 8 * 128 * 32768 * 2 B = 128 MiB.
"""
from __future__ import annotations

import numpy as np

F32 = 4


def elem_bytes(dtype: str) -> int:
    return {"bf16": 2, "fp8": 1, "f32": 4}[dtype]


def _lens(cfg, seq_lens=None):
    if seq_lens is not None:
        return np.asarray(seq_lens, np.int64)
    return np.full(cfg.batch, cfg.seq_len, np.int64)


def kv_bytes(cfg, seq_lens=None) -> int:
    """Bytes of one of K or V over the whole batch."""
    return int(_lens(cfg, seq_lens).sum()) * cfg.num_kv_heads * cfg.head_dim * elem_bytes(cfg.kv_dtype)


def num_tiles(n, T):
    return (np.asarray(n, np.int64) + T - 1) // T


def prop_pass1_bytes(cfg, T=None, seq_lens=None) -> int:
    T = T or cfg.tile_len
    n = _lens(cfg, seq_lens)
    H = cfg.num_q_heads
    stash = int(n.sum()) * H * F32
    stats = int(num_tiles(n, T).sum()) * H * 2 * F32
    q = cfg.batch * H * cfg.head_dim * elem_bytes(cfg.q_dtype)
    return kv_bytes(cfg, seq_lens) + stash + stats + q


def bernoulli_pass1_bytes(cfg, features_read, draws, group_mean, T=None, seq_lens=None) -> int:
    """Pass 1 on Bernoulli qK^T scores: of K only the kept features of each
    KV group (features_read [B*Hkv], each a run of n_k values), the stash
    (one row per head, or per group with the mean query, whose G rows are
    equal), the same stats and q as pass 1, and the ternary draws' uniforms."""
    n = _lens(cfg, seq_lens)
    fr = np.asarray(features_read, np.int64).reshape(cfg.batch, cfg.num_kv_heads)
    k = int((fr.sum(axis=1) * n).sum()) * elem_bytes(cfg.kv_dtype)
    owners = cfg.batch * (cfg.num_kv_heads if group_mean else cfg.num_q_heads)
    uniforms = owners * draws * cfg.head_dim * F32
    stash_saved = int(n.sum()) * (cfg.num_q_heads - cfg.num_kv_heads) * F32 if group_mean else 0
    return prop_pass1_bytes(cfg, T, seq_lens) - kv_bytes(cfg, seq_lens) + k + uniforms - stash_saved


def stash_reread_bytes(tile_budget: np.ndarray, cfg, T=None, seq_lens=None) -> int:
    """Stash bytes pass 2 reads: the tiles with S_t > 0 (from the returned budgets)."""
    T = T or cfg.tile_len
    n = _lens(cfg, seq_lens)
    H = cfg.num_q_heads
    tb = np.asarray(tile_budget).reshape(cfg.batch, H, -1)
    total = 0
    for b in range(cfg.batch):
        nt = int(num_tiles(n[b], T))
        lens = np.minimum(T, n[b] - T * np.arange(nt))
        total += int(((tb[b, :, :nt] > 0) * lens[None, :]).sum())
    return total * F32


def prop_step_bytes(cfg, S, tile_budget, T=None, seq_lens=None) -> dict:
    T = T or cfg.tile_len
    n = _lens(cfg, seq_lens)
    BH = cfg.batch * cfg.num_q_heads
    p1 = prop_pass1_bytes(cfg, T, seq_lens)
    stats = int(num_tiles(n, T).sum()) * cfg.num_q_heads * 2 * F32
    reread = stash_reread_bytes(tile_budget, cfg, T, seq_lens)
    vrows = BH * S * cfg.head_dim * elem_bytes(cfg.kv_dtype)
    out = BH * cfg.head_dim * F32
    return {"pass1": p1, "reduce": stats, "pass2": reread + vrows + out,
            "stash_reread": reread, "v_rows": vrows,
            "total": p1 + stats + reread + vrows + out}


def flash_step_bytes(cfg, S, T=None) -> dict:
    T = T or cfg.tile_len
    nt = int(num_tiles(cfg.seq_len, T))
    BH = cfg.batch * cfg.num_q_heads
    k = kv_bytes(cfg)
    vrows = BH * S * cfg.head_dim * elem_bytes(cfg.kv_dtype)
    partials = BH * nt * (cfg.head_dim + 2) * F32
    q = BH * cfg.head_dim * elem_bytes(cfg.q_dtype)
    out = BH * cfg.head_dim * F32
    tile = k + vrows + partials + q
    return {"tile": tile, "merge": partials + out, "total": tile + partials + out}


def exact_step_bytes(cfg, T=None, seq_lens=None) -> dict:
    T = T or cfg.tile_len
    n = _lens(cfg, seq_lens)
    BH = cfg.batch * cfg.num_q_heads
    kv = 2 * kv_bytes(cfg, seq_lens)
    partials = int(num_tiles(n, T).sum()) * cfg.num_q_heads * (cfg.head_dim + 2) * F32
    q = BH * cfg.head_dim * elem_bytes(cfg.q_dtype)
    out = BH * cfg.head_dim * F32
    return {"partial": kv + partials + q, "merge": partials + out, "total": kv + 2 * partials + q + out}


def v_row_fraction(sample_idx: np.ndarray, cfg, seq_lens=None) -> float:
    """Distinct V rows read per KV head over its keys (all requests)."""
    n = _lens(cfg, seq_lens)
    G = cfg.group
    idx = np.asarray(sample_idx).reshape(cfg.batch, cfg.num_kv_heads, G, -1)
    distinct = 0
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            rows = idx[b, g].ravel()
            distinct += np.unique(rows[rows >= 0]).size
    return distinct / float(n.sum() * cfg.num_kv_heads)
