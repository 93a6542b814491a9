"""GPU-vs-oracle comparison helpers (used by the gpu-marked tests, smoke and bench).

The bar (from the target statement of the work):
  * sampled indices identical to the oracle's, except where the oracle's
    threshold lies within 1e-6 of a CDF cell edge; there the GPU's token is
    still correct only if the threshold lies within 1e-6 of that token's
    own cell [F(j-1), F(j)) (prop: the head's CDF; flash: the tile's own
    CDF), i.e. the GPU took a neighbour across the edge, not any token;
  * outputs within 1e-3 max-abs of the oracle's fp64 replay of the GPU's
    own indices (prop: mean of the selected rows; flash: tile means weighed
    by the oracle's tile shares);
  * exact decode within 1e-3 max-abs of the oracle's A.V;
  * tile budgets sum to S and match the GPU's own indices exactly;
  * bitwise identical results on a repeated call.
"""
from __future__ import annotations

import numpy as np

import oracle as O

BOUNDARY_EXEMPT = 1e-6
OUT_TOL = 1e-3


def _torch():
    import torch
    return torch


def run_prop(dev, S, T=None, sampler="sys", uniforms=None, fused=False, workspace=None):
    torch = _torch()
    c = dev.inp.cfg
    BH = c.batch * c.num_q_heads
    T = T or dev.problem.s.tile_len
    max_nt = (c.seq_len + T - 1) // T
    out = torch.full((BH, c.head_dim), float("nan"), dtype=torch.float32, device=dev.q.device)
    idx = torch.full((BH, S), -7, dtype=torch.int32, device=dev.q.device)
    tb = torch.full((BH, max_nt), -7, dtype=torch.int32, device=dev.q.device)
    import stochastic_sparse_attention_amd as sa
    if sampler == "sys":
        uu = dev.u(S) if uniforms is None else torch.from_numpy(uniforms).to(dev.q.device)
        call = sa.santa_decode_prop_fused if fused else sa.santa_decode_prop
        call(dev.problem, dev.q, dev.k, dev.v, S, uu, out, idx, tb, workspace=workspace)
    else:
        assert not fused
        uu = dev.uniforms(S) if uniforms is None else torch.from_numpy(uniforms).to(dev.q.device)
        sa.santa_decode_prop_sampler(dev.problem, dev.q, dev.k, dev.v, S, sampler, uu, out, idx, tb)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), tb.cpu().numpy()


def run_prop_bernoulli(dev, S, draws, group_mean, kf=None):
    torch = _torch()
    c = dev.inp.cfg
    BH = c.batch * c.num_q_heads
    T = dev.problem.s.tile_len
    max_nt = (c.seq_len + T - 1) // T
    out = torch.full((BH, c.head_dim), float("nan"), dtype=torch.float32, device=dev.q.device)
    idx = torch.full((BH, S), -7, dtype=torch.int32, device=dev.q.device)
    tb = torch.full((BH, max_nt), -7, dtype=torch.int32, device=dev.q.device)
    fr = torch.full((c.batch * c.num_kv_heads,), -7, dtype=torch.int32, device=dev.q.device)
    import stochastic_sparse_attention_amd as sa
    kf = dev.k_features() if kf is None else kf
    sa.santa_decode_prop_bernoulli(dev.problem, dev.q, kf, dev.v, S, dev.u(S), draws, group_mean,
                                   dev.bernoulli_uniforms(draws, group_mean), out, idx, tb, fr)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), tb.cpu().numpy(), fr.cpu().numpy()


def run_flash(dev, S, sampler="sys", uniforms=None):
    torch = _torch()
    c = dev.inp.cfg
    BH = c.batch * c.num_q_heads
    out = torch.full((BH, c.head_dim), float("nan"), dtype=torch.float32, device=dev.q.device)
    idx = torch.full((BH, S), -7, dtype=torch.int32, device=dev.q.device)
    import stochastic_sparse_attention_amd as sa
    if sampler == "sys":
        uu = dev.u(S) if uniforms is None else torch.from_numpy(uniforms).to(dev.q.device)
        sa.santa_decode_flash(dev.problem, dev.q, dev.k, dev.v, S, uu, out, idx)
    else:
        sa.santa_decode_flash_sampler(dev.problem, dev.q, dev.k, dev.v, S, sampler, dev.uniforms(S), out, idx)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def run_exact(dev):
    torch = _torch()
    c = dev.inp.cfg
    BH = c.batch * c.num_q_heads
    out = torch.full((BH, c.head_dim), float("nan"), dtype=torch.float32, device=dev.q.device)
    import stochastic_sparse_attention_amd as sa
    sa.exact_decode_ref(dev.problem, dev.q, dev.k, dev.v, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_problem(dev):
    inp = dev.inp
    c = inp.cfg
    seq = None
    if dev.seq_lens is not None:
        seq = dev.seq_lens.cpu().numpy()
    return O.Problem(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, c.seq_len,
                     q_dtype=c.q_dtype, kv_dtype=c.kv_dtype, scale=inp.scale,
                     tile_len=dev.problem.s.tile_len, seq_lens=seq, page_size=c.page_size,
                     page_table=inp.page_table if c.page_size else None)


def cell_distance(thr, lo, hi):
    """Distance from each threshold to the cell [lo, hi) (0 inside it or on
    its upper edge; inf where the cell is undefined: a token outside the
    request or, for flash, outside the threshold's tile)."""
    thr, lo, hi = (np.asarray(a, np.float64) for a in (thr, lo, hi))
    ok = np.isfinite(thr) & np.isfinite(lo) & np.isfinite(hi)
    with np.errstate(invalid="ignore"):
        d = np.maximum(np.maximum(lo - thr, thr - hi), 0.0)
    return np.where(ok, d, np.inf)


def index_report(gpu_idx, ora_idx, delta, cells_of=None):
    """Classify every threshold: match, exempt mismatch or hard mismatch.
    A mismatch is exempt only if the oracle's threshold lies within 1e-6 of
    a cell edge AND within 1e-6 of the GPU token's own cell.  `cells_of(tok)`
    returns (thr, lo, hi) for the given tokens (oracle prop_cells /
    flash_cells); it is called only when there are mismatches."""
    gpu_idx = np.asarray(gpu_idx)
    mism = gpu_idx != ora_idx
    near = delta < BOUNDARY_EXEMPT
    exempt = np.zeros_like(mism)
    worst = 0.0
    if mism.any():
        if cells_of is None:
            raise ValueError("index_report: mismatches need the cells of the GPU's tokens")
        thr, lo, hi = cells_of(gpu_idx)
        dist = cell_distance(thr, lo, hi)
        exempt = mism & near & (dist < BOUNDARY_EXEMPT)
        if exempt.any():
            worst = float(dist[exempt].max())
    hard = mism & ~exempt
    return {"thresholds": int(gpu_idx.size), "mismatch": int(mism.sum()), "hard": int(hard.sum()),
            "exempt": int(exempt.sum()), "near_edges": int(near.sum()),
            "max_exempt_cell_distance": worst}


def check_prop(dev, S, repeat=True, sampler="sys", uniforms=None, oracle_uniforms=None, fused=False,
               workspace=None):
    """Run prop on the GPU (systematic, stratified or i.i.d. thresholds) and
    hold it to the bar; returns a report dict.  `uniforms` replaces the
    seeded offsets [B*Hq] (systematic) or uniforms [B*Hq, S] (list
    generators); the oracle gets `oracle_uniforms` if given (e.g. the same
    values clamped), else the same."""
    inp = dev.inp
    c = inp.cfg
    T = dev.problem.s.tile_len
    out, idx, tb = run_prop(dev, S, sampler=sampler, uniforms=uniforms, fused=fused, workspace=workspace)
    prob = oracle_problem(dev)
    ou = oracle_uniforms if oracle_uniforms is not None else uniforms
    if sampler == "sys":
        ou = inp.u(S) if ou is None else ou
        r = O.santa_prop(prob, inp.q, inp.k, inp.v, S, ou)
    else:
        ou = inp.uniforms(S) if ou is None else ou
        r = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, S, sampler, ou)
    rep = index_report(idx, r["idx"], r["delta"],
                       lambda tok: O.prop_cells(prob, inp.q, inp.k, S, ou, tok, sampler=sampler))
    assert rep["hard"] == 0, rep
    # budgets: sum to S (or 0 for empty requests), match the GPU's own indices
    seq = prob.seq_lens if prob.seq_lens is not None else np.full(c.batch, c.seq_len)
    H = c.num_q_heads
    for bh in range(idx.shape[0]):
        n = int(seq[bh // H])
        if n == 0:
            assert np.all(idx[bh] == -1) and np.all(tb[bh] == 0)
            continue
        assert tb[bh].sum() == S
        own = np.bincount(idx[bh] // T, minlength=tb.shape[1])
        np.testing.assert_array_equal(own, tb[bh])
        assert np.all((idx[bh] >= 0) & (idx[bh] < n))
    # tiles untouched by exempt mismatches carry the oracle's budgets
    clean = ~np.any(idx != r["idx"], axis=1)
    w = r["tile_counts"].shape[1]               # oracle: tiles of the longest request
    assert np.all(tb[:, w:] == 0)
    np.testing.assert_array_equal(tb[clean, :w], r["tile_counts"][clean])
    rp = O.replay(prob, inp.v, S, idx)
    err = float(np.max(np.abs(out - rp))) if out.size else 0.0
    assert err <= OUT_TOL, err
    rep["max_abs_vs_replay"] = err
    rep["max_abs_vs_oracle_estimate"] = float(np.max(np.abs(out - r["out"])))
    if repeat:
        out2, idx2, tb2 = run_prop(dev, S, sampler=sampler, uniforms=uniforms, fused=fused, workspace=workspace)
        assert np.array_equal(idx, idx2) and np.array_equal(tb, tb2)
        assert np.array_equal(out.view(np.uint32), out2.view(np.uint32))
    return rep


def _check_budgets(prob, c, S, T, idx, tb, r):
    seq = prob.seq_lens if prob.seq_lens is not None else np.full(c.batch, c.seq_len)
    H = c.num_q_heads
    for bh in range(idx.shape[0]):
        n = int(seq[bh // H])
        if n == 0:
            assert np.all(idx[bh] == -1) and np.all(tb[bh] == 0)
            continue
        assert tb[bh].sum() == S
        own = np.bincount(idx[bh] // T, minlength=tb.shape[1])
        np.testing.assert_array_equal(own, tb[bh])
        assert np.all((idx[bh] >= 0) & (idx[bh] < n))
    clean = ~np.any(idx != r["idx"], axis=1)
    w = r["tile_counts"].shape[1]
    assert np.all(tb[:, w:] == 0)
    np.testing.assert_array_equal(tb[clean, :w], r["tile_counts"][clean])


def check_prop_bernoulli(dev, S, draws, group_mean, repeat=True):
    """prop on Bernoulli qK^T scores against the oracle: the same bar as
    check_prop, plus the per-group read counts bit-exact."""
    inp = dev.inp
    c = inp.cfg
    T = dev.problem.s.tile_len
    kf = dev.k_features()
    out, idx, tb, fr = run_prop_bernoulli(dev, S, draws, group_mean, kf)
    prob = oracle_problem(dev)
    ub = inp.bernoulli_uniforms(draws, group_mean)
    r = O.santa_prop_bernoulli(prob, inp.q, inp.k, inp.v, S, inp.u(S), draws, group_mean, ub)
    rep = index_report(idx, r["idx"], r["delta"],
                       lambda tok: O.prop_cells(prob, inp.q, inp.k, S, inp.u(S), tok, draws=draws,
                                                group_mean=group_mean, ub=ub))
    assert rep["hard"] == 0, rep
    _check_budgets(prob, c, S, T, idx, tb, r)
    np.testing.assert_array_equal(fr, O.bernoulli_features(prob, inp.q, draws, group_mean, ub))
    rp = O.replay(prob, inp.v, S, idx)
    err = float(np.max(np.abs(out - rp))) if out.size else 0.0
    assert err <= OUT_TOL, err
    rep["max_abs_vs_replay"] = err
    rep["features_read_frac"] = float(fr.mean() / c.head_dim)
    if repeat:
        out2, idx2, tb2, fr2 = run_prop_bernoulli(dev, S, draws, group_mean, kf)
        assert np.array_equal(idx, idx2) and np.array_equal(tb, tb2) and np.array_equal(fr, fr2)
        assert np.array_equal(out.view(np.uint32), out2.view(np.uint32))
    return rep


def check_flash(dev, S, repeat=True, sampler="sys", uniforms=None, oracle_uniforms=None):
    """Flash against the oracle; `uniforms` / `oracle_uniforms` replace the
    systematic offsets as in check_prop."""
    inp = dev.inp
    out, idx = run_flash(dev, S, sampler, uniforms)
    prob = oracle_problem(dev)
    ou = oracle_uniforms if oracle_uniforms is not None else uniforms
    if ou is None:
        ou = inp.u(S) if sampler == "sys" else inp.uniforms(S)
    if sampler == "sys":
        r = O.santa_flash(prob, inp.q, inp.k, inp.v, S, ou)
    else:
        r = O.santa_flash_sampler(prob, inp.q, inp.k, inp.v, S, sampler, ou)
    rep = index_report(idx, r["idx"], r["delta"],
                       lambda tok: O.flash_cells(prob, inp.q, inp.k, S, ou, tok, sampler=sampler))
    assert rep["hard"] == 0, rep
    T = dev.problem.s.tile_len
    nt = r["ptile"].shape[1]
    Sf = S // nt
    assert np.all(idx // T == (np.arange(S) // Sf)[None, :])
    rp = O.replay(prob, inp.v, S, idx, r["ptile"])
    err = float(np.max(np.abs(out - rp)))
    assert err <= OUT_TOL, err
    rep["max_abs_vs_replay"] = err
    if repeat:
        out2, idx2 = run_flash(dev, S, sampler, uniforms)
        assert np.array_equal(idx, idx2)
        assert np.array_equal(out.view(np.uint32), out2.view(np.uint32))
    return rep


def check_exact(dev, repeat=True):
    inp = dev.inp
    out = run_exact(dev)
    prob = oracle_problem(dev)
    ref = O.exact(prob, inp.q, inp.k, inp.v)
    err = float(np.max(np.abs(out - ref)))
    assert err <= OUT_TOL, err
    if repeat:
        out2 = run_exact(dev)
        assert np.array_equal(out.view(np.uint32), out2.view(np.uint32))
    return {"max_abs_vs_oracle": err}
