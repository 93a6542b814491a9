"""Pins of the CPU oracle against what the SANTA notes and the mathematics fix.

Every check here is independent of the oracle's own code path: hand-derived
partitions (tests/golden), closed forms, special cases that reduce to a known
answer, a library routine (torch's fp64 attention on CPU), brute force on tiny
inputs, and exact enumeration against the weighted sum.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from stochastic_sparse_attention_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _golden(name):
    from conftest import GOLDEN
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- sampler
def test_golden_partitions():
    g = _golden("sys_partitions.json")
    for case in g["cases"]:
        S = case["S"]
        for U, want in case["points"]:
            idx, _ = O.invert_cdf(case["w"], O.sys_thresholds(U, S))
            assert idx.tolist() == want, (case["name"], U)


def test_golden_partition_expectation():
    """E_U over the hand-derived intervals equals AV (key design 1: unbiased)."""
    case = _golden("sys_partitions.json")["cases"][0]
    rng = np.random.default_rng(7)
    V = rng.standard_normal((4, 5))
    S = case["S"]
    est = np.zeros(5)
    for a, b, want in case["intervals"]:
        est += (b - a) * S * V[want].mean(axis=0)
    A = np.asarray(case["w"], float) / sum(case["w"])
    np.testing.assert_allclose(est, A @ V, rtol=0, atol=1e-14)
    mean, _ = O.sys_moments(case["w"], V, S)
    np.testing.assert_allclose(mean, A @ V, rtol=0, atol=1e-14)


def test_cell_edges_golden():
    """Token j's cell is [F(j-1), F(j)) of the hand-derived CDF, and every
    hand-derived selection holds its threshold (key design 1: J_m = F^-1(T_m))."""
    g = _golden("sys_partitions.json")
    for case in g["cases"]:
        w, F, S = case["w"], case["F"], case["S"]
        n = len(w)
        lo, hi = O.cell_edges(w, np.arange(n))
        np.testing.assert_allclose(lo, [0.0] + F[:-1], rtol=0, atol=1e-15, err_msg=case["name"])
        np.testing.assert_allclose(hi, F, rtol=0, atol=1e-15, err_msg=case["name"])
        lo, hi = O.cell_edges(w, [-1, n])
        assert np.all(np.isnan(lo)) and np.all(np.isnan(hi))
        for U, want in case["points"]:
            t = U + np.arange(S) / S
            lo, hi = O.cell_edges(w, want)
            assert np.all((lo <= t) & (t < hi)), (case["name"], U)


def _golden_flash_problem():
    g = _golden("flash_small.json")
    w = np.asarray(g["w"], float)
    n, T, S = w.size, g["T"], g["S"]
    q = np.ones((1, 1, 1), np.float32)
    k = np.log(w).astype(np.float32).reshape(1, 1, n, 1)
    prob = O.Problem(1, 1, 1, 1, n, q_dtype="f32", kv_dtype="f32", scale=1.0, tile_len=T)
    return g, q, k, prob


def test_prop_and_flash_cells_golden():
    """The cells the parity check uses: the untiled CDF for prop, each tile's
    own CDF for flash (key designs 2 and 3), on the hand-derived case with
    logits log(w) (so the weights are w up to fp32 rounding of the logs)."""
    g, q, k, prob = _golden_flash_problem()
    S, T = g["S"], g["T"]
    Fg = [0.0] + g["F_global"]
    tok = np.array([[0, 1, 2, 3]], np.int32)
    U = np.array([0.05], np.float32)
    thr, lo, hi = O.prop_cells(prob, q, k, S, U, tok)
    np.testing.assert_allclose(thr[0], float(U[0]) + np.arange(S) / S, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lo[0], Fg[:4], rtol=0, atol=1e-6)
    np.testing.assert_allclose(hi[0], Fg[1:], rtol=0, atol=1e-6)
    # flash: position m belongs to tile m // S_f and sees that tile's CDF
    Sf = S // 2
    U = np.array([0.15], np.float32)
    tok = np.array([[1, 0, 3, 2]], np.int32)
    thr, lo, hi = O.flash_cells(prob, q, k, S, U, tok)
    uf = float(U[0]) * 2
    np.testing.assert_allclose(thr[0], [uf, uf + 1 / Sf, uf, uf + 1 / Sf], rtol=0, atol=1e-15)
    F0, F1 = [0.0] + g["F_tiles"][0], [0.0] + g["F_tiles"][1]
    np.testing.assert_allclose(lo[0], [F0[1], F0[0], F1[1], F1[0]], rtol=0, atol=1e-6)
    np.testing.assert_allclose(hi[0], [F0[2], F0[1], F1[2], F1[1]], rtol=0, atol=1e-6)
    # a token outside its position's tile has no cell there
    thr, lo, hi = O.flash_cells(prob, q, k, S, U, np.array([[2, 1, 0, 3]], np.int32))
    assert np.isnan(lo[0, 0]) and np.isnan(hi[0, 2]) and not np.isnan(lo[0, 1])
    assert T == 2


@pytest.mark.parametrize("sampler", ["sys", "strat", "iid", "bernoulli", "flash"])
def test_oracle_indices_lie_in_their_cells(sampler):
    """Every oracle index's cell holds its threshold, and the boundary
    distance is the distance to the nearer edge of that cell."""
    inp, prob = _small_inputs(2, seq_len=300, batch=2, tile_len=64)
    S = 16
    if sampler == "flash":
        inp, prob = _small_inputs(2, seq_len=320, batch=2, tile_len=64)
        S = 20
        r = O.santa_flash(prob, inp.q, inp.k, inp.v, S, inp.u(S))
        thr, lo, hi = O.flash_cells(prob, inp.q, inp.k, S, inp.u(S), r["idx"])
    elif sampler == "bernoulli":
        ub = inp.bernoulli_uniforms(4, False)
        r = O.santa_prop_bernoulli(prob, inp.q, inp.k, inp.v, S, inp.u(S), 4, 0, ub)
        thr, lo, hi = O.prop_cells(prob, inp.q, inp.k, S, inp.u(S), r["idx"], draws=4, group_mean=0, ub=ub)
    elif sampler == "sys":
        r = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
        thr, lo, hi = O.prop_cells(prob, inp.q, inp.k, S, inp.u(S), r["idx"])
    else:
        uu = inp.uniforms(S)
        r = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, S, sampler, uu)
        thr, lo, hi = O.prop_cells(prob, inp.q, inp.k, S, uu, r["idx"], sampler=sampler)
    assert np.all((lo <= thr) & (thr < hi))
    np.testing.assert_array_equal(r["delta"], np.minimum(thr - lo, hi - thr))


def test_thresholds_closed_form():
    t = O.sys_thresholds(0.03125, 4)
    assert t.tolist() == [0.03125, 0.28125, 0.53125, 0.78125]
    assert O.strat_thresholds([0.0, 0.5, 0.25]).tolist() == [0.0, 0.5, (2 + 0.25) / 3]
    assert O.iid_thresholds([0.7, 0.1, 0.4]).tolist() == [0.1, 0.4, 0.7]


def test_invert_cdf_rejects_bad_thresholds():
    with pytest.raises(ValueError):
        O.invert_cdf([1, 1], [0.5, 0.2])
    with pytest.raises(ValueError):
        O.invert_cdf([1, 1], [1.0])


def _brute_indices(w, t):
    """Count form of the inverse CDF: J = #{j : F(j) <= t} (same cells)."""
    w = np.asarray(w, float)
    F = np.cumsum(w) / w.sum()
    F[-1] = 1.0
    return [int(np.sum(F <= x)) for x in t]


def test_brute_force_tiny():
    rng = np.random.default_rng(11)
    for trial in range(200):
        n = int(rng.integers(1, 7))
        S = int(rng.integers(1, 5))
        w = rng.integers(1, 9, size=n).astype(float)   # positive integer weights
        for U in (rng.random(5) / S):
            t = O.sys_thresholds(U, S)
            idx, dl = O.invert_cdf(w, t)
            assert idx.tolist() == _brute_indices(w, t)
            assert np.all(dl >= 0)


def test_one_hot_weights_any_S():
    rng = np.random.default_rng(3)
    # bf16-valued rows (8 significant bits): S copies sum exactly in fp64,
    # so the mean of S copies is bit-identical to the row
    V = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        rng.standard_normal((9, 4)).astype(np.float32))).astype(np.float64)
    w = np.zeros(9)
    w[5] = 1.0
    for S in (1, 2, 7, 16, 128):
        for U in rng.random(3) / S:
            est = O.estimate_from_weights(w, V, O.sys_thresholds(U, S))
            assert np.array_equal(est, V[5])


def test_S_equals_nk_uniform_is_mean():
    rng = np.random.default_rng(5)
    n = 64
    V = rng.standard_normal((n, 6))
    for U in rng.random(4) / n:
        idx, _ = O.invert_cdf(np.ones(n), O.sys_thresholds(U, n))
        assert idx.tolist() == list(range(n))
        est = O.estimate_from_weights(np.ones(n), V, O.sys_thresholds(U, n))
        np.testing.assert_allclose(est, V.mean(axis=0), rtol=0, atol=1e-15)


def test_moments_match_fine_grid():
    """Exact enumeration vs a brute-force midpoint grid over U."""
    rng = np.random.default_rng(9)
    n, S = 12, 4
    w = rng.random(n)
    V = rng.standard_normal((n, 3))
    mean, var = O.sys_moments(w, V, S)
    N = 20000
    Us = (np.arange(N) + 0.5) / (N * S)
    ests = np.array([O.estimate_from_weights(w, V, O.sys_thresholds(U, S)) for U in Us])
    np.testing.assert_allclose(ests.mean(0), mean, atol=2e-3)
    assert abs(((ests - ests.mean(0)) ** 2).sum(1).mean() - var) < 5e-3


# ------------------------------------------------- variance (key design 1)
def _smooth_weights(n=1024, d=128, seed=1000):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    x = (K @ q) / math.sqrt(d)
    w = np.exp(x - x.max())
    return w, V


def test_iid_variance_closed_form():
    """Eq. (4): Var of the i.i.d. estimator = (sum A_j |V_j|^2 - |AV|^2) / S."""
    w, V = _smooth_weights(n=256, d=8)
    A = w / w.sum()
    S = 8
    closed = (A @ (V ** 2).sum(1) - ((A @ V) ** 2).sum()) / S
    rng = np.random.default_rng(2)
    R = 10000
    ests = np.array([O.estimate_from_weights(w, V, O.iid_thresholds(rng.random(S))) for _ in range(R)])
    emp = ((ests - A @ V) ** 2).sum(1).mean()
    # Monte-Carlo standard error of a mean of R chi-square-like terms
    se = ((ests - A @ V) ** 2).sum(1).std() / math.sqrt(R)
    assert abs(emp - closed) < 4 * se
    np.testing.assert_allclose(ests.mean(0), A @ V, atol=6 * math.sqrt(closed / R))


def test_strat_and_sys_reduce_variance():
    """key design 1 / Table 2: stratified and systematic beat i.i.d. at equal S."""
    w, V = _smooth_weights(n=512, d=16)
    A = w / w.sum()
    S = 16
    iid = (A @ (V ** 2).sum(1) - ((A @ V) ** 2).sum()) / S
    rng = np.random.default_rng(4)
    ests = np.array([O.estimate_from_weights(w, V, O.strat_thresholds(rng.random(S))) for _ in range(3000)])
    strat = ((ests - A @ V) ** 2).sum(1).mean()
    _, sys_var = O.sys_moments(w, V, S)
    assert strat < iid
    assert sys_var < iid


def test_systematic_variance_falls_roughly_as_one_over_S():
    w, V = _smooth_weights()
    Ss = [16, 32, 64, 128, 256]
    var = [O.sys_moments(w, V, S)[1] for S in Ss]
    slope = np.polyfit(np.log(Ss), np.log(var), 1)[0]
    assert slope <= -0.8, (slope, var)


# ------------------------------------------- scores, softmax, exact output
def _small_inputs(cid=1, seed=1, **kw):
    cfg = synth.small_config(cid, **kw)
    inp = synth.make_inputs(cfg, seed)
    return inp, O.Problem.from_inputs(inp)


def test_logits_match_matmul():
    inp, prob = _small_inputs(2, seq_len=300, batch=2, tile_len=64)
    qv = inp.values("q").astype(np.float64)
    kv = inp.values("k").astype(np.float64)
    G = inp.cfg.group
    for b, h in [(0, 0), (1, 31), (1, 13)]:
        x = O.logits(prob, inp.q, inp.k, b, h)
        ref = float(inp.scale) * (kv[b, h // G] @ qv[b, h])
        np.testing.assert_allclose(x, ref, rtol=1e-13, atol=1e-12)


def _torch_sdpa_fp64(inp):
    """torch's attention in fp64 on the CPU (library routine, GQA expanded)."""
    c = inp.cfg
    q = torch.from_numpy(inp.values("q").astype(np.float64))[:, :, None, :]
    k = torch.from_numpy(inp.values("k").astype(np.float64))
    v = torch.from_numpy(inp.values("v").astype(np.float64))
    k = k.repeat_interleave(c.group, dim=1)
    v = v.repeat_interleave(c.group, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(inp.scale))
    return o[:, :, 0, :].reshape(c.batch * c.num_q_heads, c.head_dim).numpy()


@pytest.mark.parametrize("cid,kw", [(1, {}), (2, dict(seq_len=512, batch=2)), (4, dict(seq_len=700, batch=1))])
def test_exact_matches_torch_sdpa(cid, kw):
    inp, prob = _small_inputs(cid, **kw)
    out = O.exact(prob, inp.q, inp.k, inp.v)
    np.testing.assert_allclose(out, _torch_sdpa_fp64(inp), rtol=0, atol=1e-12)


def test_exact_identical_keys_is_mean_of_V():
    inp, prob = _small_inputs(1, hot=0)
    inp.k[...] = inp.k[:, :, :1, :]            # every key the same -> A uniform
    out = O.exact(prob, inp.q, inp.k, inp.v)
    np.testing.assert_allclose(out[0], inp.v[0, 0].astype(np.float64).mean(0), atol=1e-13)


def test_softmax_weights_normalise():
    x = np.array([1000.0, 999.0, -5.0])
    e, z, m = O.softmax_weights(x)
    assert m == 1000.0 and e[0] == 1.0
    np.testing.assert_allclose(e / z, np.exp(x - 1000) / np.exp(x - 1000).sum(), rtol=1e-15)


# ------------------------------------------------ end-to-end S2ANTA-prop
def test_prop_one_hot_end_to_end_is_exact_row():
    """A logit gap > 800 makes A one-hot in fp64: out is exactly that V row."""
    inp, prob = _small_inputs(2, seq_len=512, batch=1, hot=0, sinks=0, tile_len=64)
    G = inp.cfg.group
    kv = inp.values("k").copy()
    qv = inp.values("q")
    for g in range(inp.cfg.num_kv_heads):
        qbar = qv[0, g * G:(g + 1) * G]
        # one key per KV head with a huge score for every head in its group
        kv[0, g] *= 0.0
        j = 37 + 50 * g
        kv[0, g, j] = np.sign(qbar.mean(0)) * 1024.0
    inp.k = synth.f32_to_bf16_bits(kv)
    for h in range(inp.cfg.num_q_heads):
        x = O.logits(prob, inp.q, inp.k, 0, h)
        srt = np.sort(x)
        assert srt[-1] - srt[-2] > 800
    r = O.santa_prop(prob, inp.q, inp.k, inp.v, inp.cfg.S, inp.u(inp.cfg.S))
    vv = inp.values("v")
    for h in range(inp.cfg.num_q_heads):
        g = h // G
        assert np.all(r["idx"][h] == 37 + 50 * g)
        assert np.array_equal(r["out"][h], vv[0, g, 37 + 50 * g].astype(np.float64))


@pytest.mark.parametrize("sampler", ["strat", "iid"])
def test_prop_sampler_one_hot_is_exact_row(sampler):
    """key design 1: whatever the thresholds, a one-hot A selects its token."""
    inp, prob = _small_inputs(2, seq_len=512, batch=1, hot=0, sinks=0, tile_len=64)
    G = inp.cfg.group
    kv = inp.values("k").copy()
    qv = inp.values("q")
    for g in range(inp.cfg.num_kv_heads):
        qbar = qv[0, g * G:(g + 1) * G]
        kv[0, g] *= 0.0
        kv[0, g, 11 + 60 * g] = np.sign(qbar.mean(0)) * 1024.0
    inp.k = synth.f32_to_bf16_bits(kv)
    S = 48
    u = np.random.default_rng(7).random((inp.cfg.num_q_heads, S)).astype(np.float32)
    r = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, S, sampler, u)
    vv = inp.values("v")
    for h in range(inp.cfg.num_q_heads):
        g = h // G
        assert np.all(r["idx"][h] == 11 + 60 * g)
        assert np.array_equal(r["out"][h], vv[0, g, 11 + 60 * g].astype(np.float64))


def _uniform_attention_inputs(n=1024):
    """Identical keys: every logit is equal, A is exactly uniform and
    F_j = (j + 1)/n holds exactly in fp64 for n a power of two."""
    inp, prob = _small_inputs(2, seq_len=n, batch=1, hot=0, sinks=0, tile_len=128,
                              num_q_heads=4, num_kv_heads=1)
    kv = inp.values("k").copy()
    kv[0, 0, :] = kv[0, 0, 0]
    inp.k = synth.f32_to_bf16_bits(kv)
    return inp, prob


def test_prop_strat_with_S_equal_nk_on_uniform_A_is_mean():
    """S2ANTA-strat with one stratum per token on uniform A: threshold m lies in
    [m/n, (m+1)/n), so token m is chosen exactly once and the estimate is
    the mean of V."""
    n = 1024
    inp, prob = _uniform_attention_inputs(n)
    u = np.random.default_rng(3).random((4, n)).astype(np.float32)
    r = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, n, "strat", u)
    V = inp.values("v")[0, 0].astype(np.float64)
    for h in range(4):
        assert np.array_equal(r["idx"][h], np.arange(n))
        np.testing.assert_allclose(r["out"][h], V.mean(0), rtol=0, atol=1e-12)


def test_prop_iid_equal_uniforms_pick_one_token():
    """i.i.d. with every uniform equal to c: all thresholds are c and, on
    uniform A, all select token floor(c n)."""
    n = 1024
    inp, prob = _uniform_attention_inputs(n)
    S = 40
    u = np.full((4, S), 0.3, np.float32)
    r = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, S, "iid", u)
    j = int(np.floor(np.float64(np.float32(0.3)) * n))
    V = inp.values("v")[0, 0].astype(np.float64)
    assert np.all(r["idx"] == j)
    for h in range(4):
        assert np.array_equal(r["out"][h], V[j])


@pytest.mark.parametrize("sampler", ["strat", "iid"])
def test_prop_sampler_invariants(sampler):
    """Indices are nondecreasing in m (sorted thresholds), budgets sum to S,
    and for strat every tile's budget differs from S * p_t by less than 2
    (each stratum holds one threshold; only the two strata cut by the tile's
    CDF edges can go either way)."""
    inp, prob = _small_inputs(2, seq_len=2048, batch=2, tile_len=256)
    S, T = 96, 256
    H = inp.cfg.num_q_heads
    u = np.random.default_rng(11).random((2 * H, S)).astype(np.float32)
    r = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, S, sampler, u)
    assert np.all(np.diff(r["idx"], axis=1) >= 0)
    assert np.all(r["tile_counts"].sum(1) == S)
    if sampler == "strat":
        for bh in range(2 * H):
            b, h = divmod(bh, H)
            e, z, _ = O.softmax_weights(O.logits(prob, inp.q, inp.k, b, h))
            p = np.array([e[t * T:(t + 1) * T].sum() for t in range(e.size // T)]) / z
            assert np.all(np.abs(r["tile_counts"][bh] - S * p) < 2)


def test_prop_sampler_rejects_out_of_range_uniforms():
    inp, prob = _small_inputs(1)
    u = np.zeros((1, 16), np.float32)
    u[0, 3] = 1.0
    with pytest.raises(ValueError):
        O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, 16, "strat", u)


def test_prop_expectation_equals_exact():
    """E_U[S2ANTA-sys] = AV, by exact enumeration on the oracle's own weights."""
    for seed in (1, 2):
        inp, prob = _small_inputs(1, seed=seed)
        x = O.logits(prob, inp.q, inp.k, 0, 0)
        e, _, _ = O.softmax_weights(x)
        V = inp.values("v")[0, 0].astype(np.float64)
        exact = O.exact(prob, inp.q, inp.k, inp.v)[0]
        for S in (4, 16, 64):
            mean, _ = O.sys_moments(e, V, S)
            np.testing.assert_allclose(mean, exact, rtol=0, atol=1e-11)


def test_prop_entry_matches_weight_level_sampler():
    inp, prob = _small_inputs(2, seq_len=640, batch=2, tile_len=128)
    S = inp.cfg.S
    r = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    G = inp.cfg.group
    V = inp.values("v").astype(np.float64)
    for bh in (0, 17, 63):
        b, h = divmod(bh, inp.cfg.num_q_heads)
        e, _, _ = O.softmax_weights(O.logits(prob, inp.q, inp.k, b, h))
        t = O.sys_thresholds(float(inp.u(S)[bh]), S)
        idx, dl = O.invert_cdf(e, t)
        assert np.array_equal(idx, r["idx"][bh])
        np.testing.assert_allclose(r["out"][bh], V[b, h // G][idx].mean(0), rtol=0, atol=1e-14)


def test_prop_tile_counts_are_proportional():
    """key design 2: budget per tile ~ S * Z_tile / Z; here exactly floor or ceil."""
    for cid, kw in [(1, {}), (2, dict(seq_len=2048, batch=1)), (5, dict(batch=3, seq_len=3000, min_seq_len=700))]:
        inp, prob = _small_inputs(cid, **kw)
        S, T = inp.cfg.S, inp.cfg.tile_len
        r = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
        tc = r["tile_counts"]
        assert np.all(tc.sum(1) == S)
        for bh in range(tc.shape[0]):
            b, h = divmod(bh, inp.cfg.num_q_heads)
            e, z, _ = O.softmax_weights(O.logits(prob, inp.q, inp.k, b, h))
            n = e.size
            nt = (n + T - 1) // T
            p = np.array([e[t * T:(t + 1) * T].sum() for t in range(nt)]) / z
            lo, hi = np.floor(S * p - 1e-9), np.ceil(S * p + 1e-9)
            assert np.all(tc[bh, :nt] >= lo) and np.all(tc[bh, :nt] <= hi)
            assert np.all(tc[bh, nt:] == 0)


def test_replay_of_oracle_indices_is_its_estimate():
    inp, prob = _small_inputs(2, seq_len=1024, batch=1)
    S = inp.cfg.S
    r = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    rep = O.replay(prob, inp.v, S, r["idx"])
    np.testing.assert_array_equal(rep, r["out"])


def test_paged_equals_contiguous():
    """The paged layout only changes where rows live, not the result."""
    cfg = synth.small_config(5, batch=3, seq_len=1500, min_seq_len=300)
    inp = synth.make_inputs(cfg, 5)
    prob = O.Problem.from_inputs(inp)
    P = cfg.page_size
    # rebuild a contiguous copy of the same logical rows
    n_max = int(inp.seq_lens.max())
    B, Hkv, d = cfg.batch, cfg.num_kv_heads, cfg.head_dim
    kc = np.zeros((B, Hkv, n_max, d), inp.k.dtype)
    vc = np.zeros_like(kc)
    for b in range(B):
        n = int(inp.seq_lens[b])
        for j in range(n):
            pg = inp.page_table[b, j // P]
            kc[b, :, j] = inp.k[pg, :, j % P]
            vc[b, :, j] = inp.v[pg, :, j % P]
    pc = O.Problem(B, cfg.num_q_heads, Hkv, d, n_max, q_dtype="bf16", kv_dtype="bf16",
                   scale=inp.scale, tile_len=cfg.tile_len, seq_lens=inp.seq_lens)
    S = cfg.S
    a = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    c = O.santa_prop(pc, inp.q, kc, vc, S, inp.u(S))
    assert np.array_equal(a["idx"], c["idx"])
    assert np.array_equal(a["out"], c["out"])
    assert np.all(np.isfinite(a["out"]))      # NaN padding rows never read
    np.testing.assert_array_equal(O.exact(prob, inp.q, inp.k, inp.v), O.exact(pc, inp.q, kc, vc))


# ----------------------------------------------------- S2ANTA-flash
def test_flash_golden():
    g = _golden("flash_small.json")
    w = np.asarray(g["w"], float)
    n, T, S = w.size, g["T"], g["S"]
    q = np.ones((1, 1, 1), np.float32)
    k = np.log(w).astype(np.float32).reshape(1, 1, n, 1)
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 1, n, 1)).astype(np.float32)
    prob = O.Problem(1, 1, 1, 1, n, q_dtype="f32", kv_dtype="f32", scale=1.0, tile_len=T)
    for pt in g["points"]:
        r = O.santa_flash(prob, q, k, v, S, np.array([pt["U"]], np.float32))
        assert r["idx"][0].tolist() == pt["idx"]
        np.testing.assert_allclose(r["ptile"][0], [0.5, 0.5], rtol=1e-6)
    mean, _ = O.flash_moments(np.exp(k.ravel().astype(np.float64)), v.reshape(n, 1).astype(np.float64), S, T)
    A = w / w.sum()
    np.testing.assert_allclose(mean, A @ v.reshape(n, 1), rtol=1e-6)


def test_flash_single_tile_is_systematic():
    inp, prob = _small_inputs(1, tile_len=1024)
    S = inp.cfg.S
    a = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    f = O.santa_flash(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    assert np.array_equal(a["idx"], f["idx"])
    np.testing.assert_allclose(f["out"], a["out"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("sampler", ["strat", "iid"])
def test_flash_sampler_single_tile_is_prop(sampler):
    """One tile holding every token: the tile's S_f = S local thresholds are
    the global ones, so flash selects what prop selects."""
    inp, prob = _small_inputs(1, tile_len=1024)
    S = inp.cfg.S
    u = np.random.default_rng(5).random((1, S)).astype(np.float32)
    a = O.santa_prop_sampler(prob, inp.q, inp.k, inp.v, S, sampler, u)
    f = O.santa_flash_sampler(prob, inp.q, inp.k, inp.v, S, sampler, u)
    assert np.array_equal(a["idx"], f["idx"])
    np.testing.assert_allclose(f["out"], a["out"], rtol=0, atol=1e-15)


def test_flash_strat_uniform_tiles_full_budget_is_exact():
    """Constant logits inside each tile and S_f = T stratified thresholds:
    stratum m of a tile lies in token m's cell, every token is taken once
    and the merged estimate is AV."""
    T, nt, d = 8, 4, 3
    n = T * nt
    rng = np.random.default_rng(9)
    kd = np.zeros((1, 1, n, d), np.float32)
    kd[..., 0] = np.repeat(rng.standard_normal(nt), T).astype(np.float32).reshape(1, 1, n)
    qd = np.zeros((1, 1, d), np.float32)
    qd[..., 0] = 1.0
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    prob = O.Problem(1, 1, 1, d, n, q_dtype="f32", kv_dtype="f32", scale=1.0, tile_len=T)
    u = rng.random((1, n)).astype(np.float32)
    f = O.santa_flash_sampler(prob, qd, kd, v, n, "strat", u)
    assert np.array_equal(f["idx"][0], np.arange(n))
    np.testing.assert_allclose(f["out"], O.exact(prob, qd, kd, v), rtol=0, atol=1e-13)


def test_flash_expectation_equals_exact():
    for seed in (1, 3):
        inp, prob = _small_inputs(1, seed=seed)
        x = O.logits(prob, inp.q, inp.k, 0, 0)
        e, _, _ = O.softmax_weights(x)
        V = inp.values("v")[0, 0].astype(np.float64)
        exact = O.exact(prob, inp.q, inp.k, inp.v)[0]
        for S in (8, 64):
            mean, _ = O.flash_moments(e, V, S, inp.cfg.tile_len)
            np.testing.assert_allclose(mean, exact, rtol=0, atol=1e-11)


def test_flash_uniform_tiles_full_budget_is_exact():
    """Constant logits inside each tile and S_f = T: every token once -> AV."""
    T, nt, d = 8, 4, 3
    n = T * nt
    rng = np.random.default_rng(8)
    tile_logit = rng.standard_normal(nt)
    q = np.ones((1, 1, 1), np.float32)
    k = np.repeat(tile_logit, T).astype(np.float32).reshape(1, 1, n, 1)
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    # head_dim 1 for K but V needs d columns: use d-dim K with only column 0 set
    kd = np.zeros((1, 1, n, d), np.float32)
    kd[..., 0] = k[..., 0]
    qd = np.zeros((1, 1, d), np.float32)
    qd[..., 0] = 1.0
    prob = O.Problem(1, 1, 1, d, n, q_dtype="f32", kv_dtype="f32", scale=1.0, tile_len=T)
    S = T * nt
    f = O.santa_flash(prob, qd, kd, v, S, np.array([0.3 / S], np.float32))
    ex = O.exact(prob, qd, kd, v)
    np.testing.assert_allclose(f["out"], ex, rtol=0, atol=1e-13)


def test_flash_replay_with_oracle_weights():
    inp, prob = _small_inputs(3, seq_len=1024, batch=2, S_flash=64)
    S = inp.cfg.S_flash
    f = O.santa_flash(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    rep = O.replay(prob, inp.v, S, f["idx"], f["ptile"])
    np.testing.assert_allclose(rep, f["out"], rtol=0, atol=1e-14)
    # tile-major layout: tile t's samples lie inside tile t
    T = inp.cfg.tile_len
    Sf = S // (1024 // T)
    tiles = f["idx"] // T
    assert np.all(tiles == (np.arange(S) // Sf)[None, :])


def test_flash_rejects_bad_budget():
    inp, prob = _small_inputs(1)
    with pytest.raises(ValueError):
        O.santa_flash(prob, inp.q, inp.k, inp.v, 12, inp.u(12))   # 12 % 8 != 0


def test_prop_rejects_out_of_range_U():
    inp, prob = _small_inputs(1)
    with pytest.raises(ValueError):
        O.santa_prop(prob, inp.q, inp.k, inp.v, 16, np.array([1.0 / 16], np.float32))


def test_empty_request_reading():
    """R11: a request with no keys gives a zero output and selects nothing."""
    cfg = synth.small_config(5, batch=3, seq_len=600, min_seq_len=100)
    inp = synth.make_inputs(cfg, 2)
    seq = inp.seq_lens.copy()
    seq[1] = 0
    prob = O.Problem(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.seq_len,
                     q_dtype="bf16", kv_dtype="bf16", scale=inp.scale, tile_len=cfg.tile_len,
                     seq_lens=seq, page_size=cfg.page_size, page_table=inp.page_table)
    S = cfg.S
    r = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
    H = cfg.num_q_heads
    assert np.all(r["out"][H:2 * H] == 0) and np.all(r["idx"][H:2 * H] == -1)
    assert np.all(r["tile_counts"][H:2 * H] == 0)
    assert np.all(r["tile_counts"][:H].sum(1) == S)
    ex = O.exact(prob, inp.q, inp.k, inp.v)
    assert np.all(ex[H:2 * H] == 0)
    np.testing.assert_array_equal(O.replay(prob, inp.v, S, r["idx"]), r["out"])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf], np.float32),
                        # exact ties: low half 0x8000 with even and odd upper halves
                        np.array([0x3F808000, 0x3F818000], np.uint32).view(np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(synth.bf16_bits_to_f32(nan))[0]


def test_e4m3_storage_matches_torch():
    """Synthetic e4m3 storage against torch's float8_e4m3fn: every code
    decodes to the same value, and rounding is to nearest with ties to the
    even code (midpoints between neighbouring codes included)."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ours = synth.e4m3_bits_to_f32(codes)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[~np.isnan(ref)], ref[~np.isnan(ref)])
    rng = np.random.default_rng(1)
    fin = ref[np.isfinite(ref)]
    mags = np.unique(np.abs(fin))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)          # exact ties
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 4,
                        rng.uniform(-448, 448, 20000).astype(np.float32),
                        mids, -mids, np.array([0.0, -0.0, 2 ** -9, 2 ** -10, 448.0], np.float32)])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = synth.f32_to_e4m3_bits(x)
    np.testing.assert_array_equal(got, want)
    assert synth.f32_to_e4m3_bits(np.array([1e6], np.float32))[0] == 0x7E     # saturates to 448


def test_oracle_e4m3_widening_through_logits():
    """The oracle widens e4m3 K by its own decoder: with q = e_0 (bf16 1.0)
    and scale 1, the logit of row j is the value of the code stored in it,
    for all 254 finite codes, and NaN for the two NaN codes."""
    codes = np.arange(256, dtype=np.uint8)
    d = 128
    k = np.zeros((1, 1, 256, d), np.uint8)
    k[0, 0, :, 0] = codes
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    qb = synth.f32_to_bf16_bits(q)
    prob = O.Problem(1, 1, 1, d, 256, q_dtype="bf16", kv_dtype="fp8", scale=1.0, tile_len=64)
    x = O.logits(prob, qb, k, 0, 0)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(np.isnan(x), np.isnan(ref))
    np.testing.assert_array_equal(x[~np.isnan(ref)], ref[~np.isnan(ref)])


# ----------------------------------------------------- Bernoulli qK^T
# Key design 4 of the SANTA notes: the query, scaled into [-1, 1], gives the
# Bernoulli probabilities of a ternary query whose score estimate is unbiased.

def _f32_problem(B, Hq, Hkv, d, n, T=64):
    return O.Problem(B, Hq, Hkv, d, n, q_dtype="f32", kv_dtype="f32", scale=1.0, tile_len=T)


def test_bernoulli_hand_derived_coefficients():
    """q = [1, -0.5, 0.25, 0] (a = 1), two draws; uniforms laid out [draw, d].
    Feature 0 (p = 1) is kept by both draws, feature 1 (p = 0.5) only by draw
    0 (0.4 < 0.5, 0.6 > 0.5), feature 2 (p = 0.25) only by draw 1 (0.3, 0.2),
    feature 3 (p = 0) never: c = [2, -1, 1, 0].  A [d, draw] reading of the
    same array would give c_1 = -2."""
    q = np.array([1, -0.5, 0.25, 0], np.float32)
    u = np.array([[0.9, 0.4, 0.3, 0.0], [0.1, 0.6, 0.2, 0.5]], np.float32)
    c, a, nz = O.bernoulli_coefs(q, u, 2)
    assert c.tolist() == [2, -1, 1, 0] and a == 1.0 and nz == 3
    # through the scores: x_j = (a / 2) * (2 K0 - K1 + K2), scale 1
    k = np.array([[[[1.0, 2.0, 4.0, 8.0], [-3.0, 0.5, 0.25, 100.0]]]], np.float32)
    prob = _f32_problem(1, 1, 1, 4, 2)
    x, nz = O.bernoulli_logits(prob, q.reshape(1, 1, 4), k, 2, False, u.reshape(1, 2, 4), 0, 0)
    assert nz == 3
    assert x.tolist() == [0.5 * (2 * 1.0 - 2.0 + 4.0), 0.5 * (2 * -3.0 - 0.5 + 0.25)]


def test_bernoulli_decision_is_strict_and_in_fp32():
    """z is kept iff fl32(u * a) < |q_i|, strictly.  With a = 3 and |q| = 1:
    u = fl32(1/3) gives u * 3 = 1.0 after fp32 rounding, not below 1, so the
    feature is dropped; one fp32 step below, u * 3 rounds under 1 and it is
    kept.  A product exactly equal to |q| (u = 0.5, a = 2) drops it too."""
    q = np.array([3.0, 1.0], np.float32)
    u13 = np.float32(1.0 / 3.0)
    below = np.nextafter(u13, np.float32(0))
    assert np.float32(u13 * np.float32(3)) == 1.0
    assert np.float32(below * np.float32(3)) < 1.0
    c, _, _ = O.bernoulli_coefs(q, np.array([[0.0, u13]], np.float32), 1)
    assert c.tolist() == [1, 0]
    c, _, _ = O.bernoulli_coefs(q, np.array([[0.0, below]], np.float32), 1)
    assert c.tolist() == [1, 1]
    c, _, _ = O.bernoulli_coefs(np.array([2.0, -1.0], np.float32), np.array([[0.5, 0.5]], np.float32), 1)
    assert c.tolist() == [1, 0]          # u * a = 1.0 is not below |q| = 1
    with pytest.raises(ValueError):
        O.bernoulli_coefs(q, np.array([[0.0, 1.0]], np.float32), 1)


@pytest.mark.parametrize("draws", [1, 3])
def test_bernoulli_unbiased_on_exact_grid(draws):
    """E[score] = scale <q, K> (key design 4).  Every |q_i| is a multiple
    a k_i / N of a = 2 with N = 64, and each draw's uniform for feature i
    runs over the N midpoints (m + 1/2)/N once as the run index m goes
    round (shifted per draw and feature).  Exactly k_i of the N midpoints
    fall below k_i / N, so the average over the N runs of each coefficient
    is draws * q_i / a and the average score is the exact one, up to fp64
    rounding."""
    N, d, n, a = 64, 16, 5, 2.0
    rng = np.random.default_rng(3)
    kint = rng.integers(0, N + 1, size=d)
    kint[0] = N                                  # the max, so a = 2
    q = (a * kint / N * rng.choice([-1.0, 1.0], size=d)).astype(np.float32)
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    prob = O.Problem(1, 1, 1, d, n, q_dtype="f32", kv_dtype="f32", scale=0.375, tile_len=64)
    acc = np.zeros(n)
    for m in range(N):
        u = np.empty((draws, d), np.float32)
        for r in range(draws):
            for i in range(d):
                u[r, i] = ((m + 7 * r + 3 * i) % N + 0.5) / N
        x, _ = O.bernoulli_logits(prob, q.reshape(1, 1, d), k, draws, False, u.reshape(1, draws, d), 0, 0)
        acc += x
    want = 0.375 * (k[0, 0].astype(np.float64) @ q.astype(np.float64))
    np.testing.assert_allclose(acc / N, want, rtol=0, atol=1e-12)


def test_bernoulli_full_magnitude_query_is_exact():
    """Every |q_i| equal to a: each draw keeps every feature with its sign,
    c_i = draws * sign(q_i), and the estimate is the exact score for any
    uniforms; prop on these scores selects what prop on exact scores does."""
    cfg = synth.small_config(2, batch=2, seq_len=700, num_q_heads=4, num_kv_heads=2)
    inp = synth.make_inputs(cfg, 11)
    qv = synth.bf16_bits_to_f32(inp.q)
    inp.q = synth.f32_to_bf16_bits(np.where(qv >= 0, 0.5, -0.5).astype(np.float32))
    prob = O.Problem.from_inputs(inp)
    for draws in (1, 4):
        ub = inp.bernoulli_uniforms(draws, False)
        for b, h in [(0, 0), (1, 3)]:
            x, nz = O.bernoulli_logits(prob, inp.q, inp.k, draws, False, ub, b, h)
            assert nz == cfg.head_dim
            np.testing.assert_allclose(x, O.logits(prob, inp.q, inp.k, b, h), rtol=1e-13, atol=1e-13)
        S = cfg.S
        rb = O.santa_prop_bernoulli(prob, inp.q, inp.k, inp.v, S, inp.u(S), draws, False, ub)
        re = O.santa_prop(prob, inp.q, inp.k, inp.v, S, inp.u(S))
        assert np.array_equal(rb["idx"], re["idx"])
        np.testing.assert_allclose(rb["out"], re["out"], rtol=0, atol=1e-12)
        nread = O.bernoulli_features(prob, inp.q, draws, False, ub)
        assert np.all(nread == cfg.head_dim)


def test_bernoulli_zero_query_reads_nothing():
    """q = 0: no feature is kept, every score is 0 and A is uniform."""
    prob = _f32_problem(1, 2, 1, 8, 6)
    q = np.zeros((1, 2, 8), np.float32)
    k = np.random.default_rng(0).standard_normal((1, 1, 6, 8)).astype(np.float32)
    ub = np.full((2, 2, 8), 0.25, np.float32)
    x, nz = O.bernoulli_logits(prob, q, k, 2, False, ub, 0, 1)
    assert nz == 0 and np.all(x == 0.0)
    assert O.bernoulli_features(prob, q, 2, False, ub).tolist() == [0]


def test_bernoulli_read_fraction_closed_form():
    """P(feature i is read) = 1 - (1 - p_i)^draws for independent draws.  With
    p_i = k_i / N and the two draws' uniforms enumerating all N^2 pairs of
    midpoints, the count of runs that read feature i is N^2 - (N - k_i)^2
    exactly; the sum over features is what the per-group counts add to."""
    N, d = 8, 8
    kint = np.array([8, 0, 1, 2, 3, 4, 5, 7])
    q = (kint / N).astype(np.float32).reshape(1, 1, d)
    prob = _f32_problem(1, 1, 1, d, 4)
    mids = (np.arange(N) + 0.5) / N
    total = 0
    for u0 in mids:
        for u1 in mids:
            ub = np.stack([np.full(d, u0), np.full(d, u1)]).astype(np.float32).reshape(1, 2, d)
            total += int(O.bernoulli_features(prob, q, 2, False, ub)[0])
    assert total == int(np.sum(N * N - (N - kint) ** 2))


def test_bernoulli_group_union_and_mean_query():
    """Two heads in one KV group.  Without the mean group query the group
    reads the union of the heads' kept features; with it, the fp32 mean
    query [0.5, -1, 0.5, 0.25] (a = 1) is drawn once and both heads get its
    scores."""
    q = np.array([[[1.0, -1.0, 0.5, 0.0], [0.0, -1.0, 0.5, 0.5]]], np.float32)
    k = np.array([[[[1.0, 2.0, 4.0, 8.0], [0.5, -1.0, 3.0, -2.0]]]], np.float32)
    prob = _f32_problem(1, 2, 1, 4, 2)
    # per head: head 0 keeps {0, 1}, head 1 keeps {1, 3}  -> union of 3
    ub = np.array([[[0.5, 0.5, 0.75, 0.0]], [[0.5, 0.5, 0.75, 0.25]]], np.float32)
    assert O.bernoulli_coefs(q[0, 0], ub[0], 1)[0].tolist() == [1, -1, 0, 0]
    assert O.bernoulli_coefs(q[0, 1], ub[1], 1)[0].tolist() == [0, -1, 0, 1]
    assert O.bernoulli_features(prob, q, 1, False, ub).tolist() == [3]
    # mean query: p = [0.5, 1, 0.5, 0.25]; uniforms [0.25, 0.9, 0.5, 0.2]
    ug = np.array([[[0.25, 0.9, 0.5, 0.2]]], np.float32)
    assert O.bernoulli_coefs(np.array([0.5, -1, 0.5, 0.25], np.float32), ug[0], 1)[0].tolist() == [1, -1, 0, 1]
    assert O.bernoulli_features(prob, q, 1, True, ug).tolist() == [3]
    x0, _ = O.bernoulli_logits(prob, q, k, 1, True, ug, 0, 0)
    x1, _ = O.bernoulli_logits(prob, q, k, 1, True, ug, 0, 1)
    assert x0.tolist() == x1.tolist() == [1.0 - 2.0 + 8.0, 0.5 + 1.0 - 2.0]


def test_bernoulli_mean_query_uses_its_groups_uniforms():
    """Two KV groups of two heads (uniforms [B*Hkv, draws, d]).  Group 1's
    mean query is [0.5, 0.5, -1, 0.25] (a = 1); its own uniforms [0.25, 0.75,
    0.9, 0.1] keep features 0, 2 and 3, c = [1, 0, -1, 1], so both of its
    heads score its keys [1, 2, 4, 8] and [0.5, -1, 3, -2] as 1 - 4 + 8 = 5
    and 0.5 - 3 - 2 = -4.5.  Group 0's uniforms [0.75, 0.25, 0.9, 0.5] would
    give c = [0, 1, -1, 0] instead.  Group 0's mean query [1, 0, 0, 0] keeps
    feature 0 only."""
    q = np.array([[[1, 0, 0, 0], [1, 0, 0, 0], [1, 0.5, -1, 0], [0, 0.5, -1, 0.5]]], np.float32)
    k = np.array([[[[1, 1, 1, 1], [2, 2, 2, 2]], [[1, 2, 4, 8], [0.5, -1, 3, -2]]]], np.float32)
    ug = np.array([[[0.75, 0.25, 0.9, 0.5]], [[0.25, 0.75, 0.9, 0.1]]], np.float32)
    prob = _f32_problem(1, 4, 2, 4, 2)
    assert O.bernoulli_coefs(np.array([0.5, 0.5, -1, 0.25], np.float32), ug[1], 1)[0].tolist() == [1, 0, -1, 1]
    assert O.bernoulli_coefs(np.array([0.5, 0.5, -1, 0.25], np.float32), ug[0], 1)[0].tolist() == [0, 1, -1, 0]
    for h in (2, 3):
        x, nz = O.bernoulli_logits(prob, q, k, 1, True, ug, 0, h)
        assert nz == 3 and x.tolist() == [5.0, -4.5], h
    for h in (0, 1):
        x, nz = O.bernoulli_logits(prob, q, k, 1, True, ug, 0, h)
        assert nz == 1 and x.tolist() == [1.0, 2.0], h
    assert O.bernoulli_features(prob, q, 1, True, ug).tolist() == [1, 3]


@pytest.mark.parametrize("draws", [1, 2])
def test_bernoulli_variance_closed_form(draws):
    """Var of the score estimate = scale^2 (a/draws)^2 sum_i K_i^2 draws p_i (1 - p_i)
    for independent draws.  With q = [a, q_1], feature 0 is always kept and
    all of the variance comes from feature 1 (p = k/N on the midpoint grid);
    enumerating every draw's uniform over the N midpoints gives the exact
    mean and variance: draws times fewer ternary values each of weight a/draws."""
    N, a, k1 = 16, 2.0, 5
    p = k1 / N
    q = np.array([a, -a * p], np.float32).reshape(1, 1, 2)
    K = np.array([[[[0.75, 1.5]]]], np.float32)
    prob = O.Problem(1, 1, 1, 2, 1, q_dtype="f32", kv_dtype="f32", scale=0.5, tile_len=64)
    mids = (np.arange(N) + 0.5) / N
    xs = []
    for combo in np.array(np.meshgrid(*([mids] * draws), indexing="ij")).reshape(draws, -1).T:
        ub = np.zeros((1, draws, 2), np.float32)
        ub[0, :, 1] = combo
        x, _ = O.bernoulli_logits(prob, q, K, draws, False, ub, 0, 0)
        xs.append(x[0])
    xs = np.array(xs)
    exact = 0.5 * (a * 0.75 - a * p * 1.5)
    var = 0.5 ** 2 * (a / draws) ** 2 * 1.5 ** 2 * draws * p * (1 - p)
    np.testing.assert_allclose(xs.mean(), exact, rtol=0, atol=1e-12)
    np.testing.assert_allclose(xs.var(), var, rtol=1e-12, atol=0)
