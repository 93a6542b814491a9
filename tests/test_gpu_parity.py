"""GPU parity: libsanta (through its C ABI) against the fp64 CPU oracle on the
same seeded inputs and the same U.  See tests/parity.py for the bar."""
import sys

import numpy as np
import pytest

from stochastic_sparse_attention_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    assert torch.cuda.is_available(), "gpu-marked tests need a GPU"
    import stochastic_sparse_attention_amd._lib as L
    L.load()                      # raises if libsanta.so is missing: no fallback
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(cfg, seed, gpu, **kw):
    from stochastic_sparse_attention_amd.device_io import to_device
    inp = synth.make_inputs(cfg, seed)
    return to_device(inp, gpu, **kw)


# ----------------------------------------------------------- prop, small
def test_prop_cfg1_many_seeds(gpu):
    """Single fp32 head, n_k=1024, S=16, T=128: 100 seeds, zero hard mismatches."""
    import parity
    tot = {"thresholds": 0, "mismatch": 0, "hard": 0, "exempt": 0}
    for seed in list(range(1, 11)) + list(range(1000, 1090)):
        rep = parity.check_prop(_dev(synth.CONFIGS[1], seed, gpu), 16, repeat=seed < 4)
        for k in tot:
            tot[k] += rep[k]
    _say("cfg1 x100 seeds", tot)
    assert tot["hard"] == 0


@pytest.mark.parametrize("T", [64, 128, 256, 512, 1024])
def test_prop_tiles_ragged_tail(gpu, T):
    import parity
    cfg = synth.small_config(2, batch=2, seq_len=4000)
    rep = parity.check_prop(_dev(cfg, 3, gpu, tile_len=T), 128)
    _say("T", T, rep)


@pytest.mark.parametrize("T,n", [(64, 4000), (64, 12000), (64, 20000), (128, 40000), (64, 65536)])
def test_prop_many_tiles(gpu, T, n):
    """Reducer paths by tiles per lane: n_t = 63, 188, 313, 313 and 1024 (the
    maximum), i.e. 1, 3, 5, 5 and 16 tiles per reducer lane."""
    import parity
    cfg = synth.small_config(2, batch=1, seq_len=n, num_q_heads=8, num_kv_heads=2)
    rep = parity.check_prop(_dev(cfg, 6, gpu, tile_len=T), 256)
    _say("T", T, "n", n, rep)


@pytest.mark.parametrize("sampler", ["strat", "iid"])
@pytest.mark.parametrize("S", [1, 96, 128, 1000, 4096])
def test_prop_samplers(gpu, sampler, S):
    """Stratified and i.i.d. thresholds (key design 1) through the same
    schedule: S = 1, non-powers of two, and S = 4096 (an i.i.d. threshold list
    above 64 KiB of LDS)."""
    import parity
    cfg = synth.small_config(2, batch=2, seq_len=3000, num_q_heads=8, num_kv_heads=2)
    rep = parity.check_prop(_dev(cfg, 8, gpu), S, sampler=sampler)
    _say(sampler, "S", S, rep)


@pytest.mark.parametrize("sampler", ["strat", "iid"])
def test_prop_samplers_ragged_paged_many_tiles(gpu, sampler):
    """Mixed lengths with paged KV, and a long sequence that takes the LDS
    reducer (313 tiles), for both list generators."""
    import parity
    cfg = synth.small_config(5, batch=5, seq_len=4000, min_seq_len=100)
    rep = parity.check_prop(_dev(cfg, 9, gpu), 128, sampler=sampler)
    _say(sampler, "paged ragged", rep)
    cfg = synth.small_config(2, batch=1, seq_len=20000, num_q_heads=8, num_kv_heads=2)
    rep = parity.check_prop(_dev(cfg, 10, gpu, tile_len=64), 256, sampler=sampler)
    _say(sampler, "313 tiles", rep)


@pytest.mark.parametrize("S", [128, 1000, 1024, 1500])
def test_prop_list_ties_and_clamping(gpu, S):
    """i.i.d. thresholds with many equal uniforms (the device sorts by rank
    up to S = 1024, with a bitonic network above), and uniforms outside
    [0, 1) for both list generators: the device clamps them into [0, 1)
    (NaN counts as 0), so its result is the oracle's on the clamped values."""
    import parity
    cfg = synth.small_config(2, batch=1, seq_len=3000, num_q_heads=8, num_kv_heads=2)
    dev = _dev(cfg, 30, gpu)
    rng = np.random.default_rng(S)
    vals = (rng.integers(0, 2 ** 24, 6) * 2.0 ** -24).astype(np.float32)
    u = vals[rng.integers(0, 6, (8, S))]
    _say("iid, 6 distinct uniforms, S", S, parity.check_prop(dev, S, sampler="iid", uniforms=u))
    raw = u.copy()
    raw[:, ::7] = 1.5
    raw[:, 3::11] = -0.25
    raw[:, 5::13] = np.nan
    raw[:, 6::17] = 1.0
    clamped = np.clip(np.nan_to_num(raw, nan=0.0), 0.0, np.float32(1.0 - 2.0 ** -24)).astype(np.float32)
    for smp in ("strat", "iid"):
        _say(smp, "clamped, S", S, parity.check_prop(dev, S, sampler=smp, uniforms=raw, oracle_uniforms=clamped,
                                                     repeat=False))
    # systematic offsets outside [0, 1/S): the device clamps them into
    # [0, u_max], u_max the largest float below 1/S (NaN and -0 as 0)
    Ur, Uc = sys_offsets_out_of_range(8, S)
    _say("sys clamped, S", S, parity.check_prop(dev, S, uniforms=Ur, oracle_uniforms=Uc, repeat=False))


def sys_offsets_out_of_range(BH, S):
    """Raw offsets for BH heads (above 1/S, exactly 1/S, 1, negative, NaN,
    -0, in range) and the values the device is to clamp them to."""
    inv = np.float32(1.0 / S)
    umax = inv if float(inv) < 1.0 / S else np.nextafter(inv, np.float32(0))
    cand = np.array([0.75, inv, 1.0, -0.125, np.nan, -0.0, 0.5 * inv, 2.0 * inv], np.float32)
    raw = cand[np.arange(BH) % cand.size]
    clamped = np.where(np.isnan(raw) | (raw <= 0), np.float32(0), np.minimum(raw, umax)).astype(np.float32)
    return raw, clamped


def test_flash_sys_offset_clamping(gpu):
    """Flash takes the same clamped offset (u_f = U n_t stays below 1/S_f)."""
    import parity
    cfg = synth.small_config(3, batch=1, seq_len=4096, num_q_heads=8, num_kv_heads=2)
    dev = _dev(cfg, 32, gpu)
    for S in (256, 1024):
        Ur, Uc = sys_offsets_out_of_range(8, S)
        _say("flash sys clamped, S", S, parity.check_flash(dev, S, uniforms=Ur, oracle_uniforms=Uc, repeat=False))


def test_sampler_variance_ordering(gpu):
    """key design 1 / Table 2 structure, on the GPU path: over many draws of
    the random inputs, the systematic and stratified estimators have lower
    mean squared error against exact attention than i.i.d. sampling at the
    same S, and all three are unbiased within their standard error."""
    import torch
    import stochastic_sparse_attention_amd as sa
    cfg = synth.small_config(2, batch=1, seq_len=2048, num_q_heads=8, num_kv_heads=2, hot=16)
    dev = _dev(cfg, 12, gpu)
    S, R, BH = 32, 200, 8
    ex = torch.empty((BH, 128), dtype=torch.float32, device=gpu)
    sa.exact_decode_ref(dev.problem, dev.q, dev.k, dev.v, ex)
    out = torch.empty_like(ex)
    rng = np.random.default_rng(99)
    ests = {k: [] for k in ("sys", "strat", "iid")}
    for _ in range(R):
        U = torch.from_numpy((np.floor(rng.random(BH) * 2 ** 24) * 2.0 ** -24 / S).astype(np.float32)).to(gpu)
        uu = torch.from_numpy((np.floor(rng.random((BH, S)) * 2 ** 24) * 2.0 ** -24).astype(np.float32)).to(gpu)
        sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, U, out)
        ests["sys"].append(out.cpu().numpy().copy())
        for smp in ("strat", "iid"):
            sa.santa_decode_prop_sampler(dev.problem, dev.q, dev.k, dev.v, S, smp, uu, out)
            ests[smp].append(out.cpu().numpy().copy())
    exact = ex.cpu().numpy()
    mse = {}
    for k, v in ests.items():
        a = np.stack(v)                                   # [R, BH, d]
        mse[k] = float(((a - exact[None]) ** 2).sum(-1).mean())
        bias = np.abs(a.mean(0) - exact)
        se = a.std(0) / np.sqrt(R)
        assert np.all(bias <= 6 * se + 1e-4), k
    _say("MSE per head at S=32:", mse)
    assert mse["sys"] < mse["iid"] and mse["strat"] < mse["iid"]


@pytest.mark.parametrize("batch", [24, 40])
def test_prop_many_heads(gpu, batch):
    """More than 512 heads: the systematic sampling kernel runs 8 waves per
    head (768 heads), and 4 above 1024 (1280 heads).  Mixed lengths (some
    short requests), paged KV, S = 128 and S = 1000."""
    import parity
    cfg = synth.small_config(5, batch=batch, seq_len=2500, min_seq_len=64)
    dev = _dev(cfg, 19, gpu)
    BH = batch * cfg.num_q_heads
    _say(BH, "heads, S=128", parity.check_prop(dev, 128))
    _say(BH, "heads, S=1000", parity.check_prop(dev, 1000, repeat=False))


@pytest.mark.parametrize("sampler", ["strat", "iid"])
def test_prop_list_many_heads(gpu, sampler):
    """More than 256 heads: the list generators run 8 waves per head (512
    threads: the i.i.d. rank sort up to S = 512, the bitonic network above).
    Mixed lengths, paged KV."""
    import parity
    cfg = synth.small_config(5, batch=24, seq_len=2500, min_seq_len=64)
    dev = _dev(cfg, 21, gpu)
    for S in (128, 1000):
        _say(sampler, "768 heads, S", S, parity.check_prop(dev, S, sampler=sampler, repeat=S == 128))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (32, 8), (16, 2)])
def test_prop_gqa_groups(gpu, hq, hkv):
    import parity
    cfg = synth.small_config(2, batch=1, seq_len=3000, num_q_heads=hq, num_kv_heads=hkv)
    rep = parity.check_prop(_dev(cfg, 4, gpu), 64)
    _say("G", hq // hkv, rep)


@pytest.mark.parametrize("S", [1, 3, 128, 1000, 4096])
def test_prop_budgets(gpu, S):
    """S = 1, non-powers of two, and S far above the number of tiles (multiplicity)."""
    import parity
    cfg = synth.small_config(2, batch=1, seq_len=2500, num_q_heads=8, num_kv_heads=2)
    rep = parity.check_prop(_dev(cfg, 5, gpu), S)
    _say("S", S, rep)


def _offsets_below_tile_edges(dev, S):
    """Per head, the largest fp32 offset U that puts a systematic threshold
    U + m/S just below the oracle's CDF at the end of one tile (a different
    tile per head): the threshold then sits within ~1e-9 of the tile edge,
    where the fp32 count at the tile's last token can fall one short of
    the tile's budget."""
    import oracle as O
    import parity
    inp = dev.inp
    c = inp.cfg
    prob = parity.oracle_problem(dev)
    T = dev.problem.s.tile_len
    u = inp.u(S).astype(np.float32).copy()
    for bh in range(c.batch * c.num_q_heads):
        b, h = divmod(bh, c.num_q_heads)
        e, z, _ = O.softmax_weights(O.logits(prob, inp.q, inp.k, b, h))
        n = e.size
        nt = (n + T - 1) // T
        if nt < 2:
            continue
        t = bh % (nt - 1)                        # not the last tile (its C is 1)
        Ct = float(np.sum(e[: (t + 1) * T], dtype=np.float64) / z)
        m = int(np.floor(Ct * S))
        ustar = Ct - m / S                       # U + m/S = C_t exactly
        uf = np.float32(ustar)
        if float(uf) >= ustar:
            uf = np.nextafter(uf, np.float32(0))
        if float(uf) < 0 or not np.isfinite(uf):
            continue
        u[bh] = uf
    return u


@pytest.mark.parametrize("T", [64, 256, 1024])
def test_prop_thresholds_just_below_tile_edges(gpu, T):
    """Every head has a threshold within ~1e-9 below a tile's upper CDF edge
    (its offset U set from the oracle's CDF), so that the fp32 count at the
    tile's last token lands on either side of the budget: the indices still
    meet the bar (the tile's last token of nonzero weight, or a neighbour
    across the edge within 1e-6)."""
    import parity
    cfg = synth.small_config(2, batch=2, seq_len=3 * T * 4 + 17)
    dev = _dev(cfg, 21, gpu, tile_len=T)
    u = _offsets_below_tile_edges(dev, 128)
    rep = parity.check_prop(dev, 128, uniforms=u)
    _say("T", T, rep)


def test_prop_tiny_sequences(gpu):
    """n_k = 1 and n_k shorter than one tile."""
    import parity
    for n in (1, 2, 63, 65, 255):
        cfg = synth.small_config(2, batch=1, seq_len=n, hot=0, sinks=min(4, n), num_q_heads=8,
                                 num_kv_heads=2)
        rep = parity.check_prop(_dev(cfg, 6, gpu), 16)
        _say("n", n, rep)


def test_output_overlapping_the_query_is_rejected(gpu):
    """Prop clears output rows while other workgroups still read the query,
    so an output that shares memory with q (or with the offsets) is refused
    on the host before anything is launched, and the memory keeps its
    contents."""
    import torch
    import stochastic_sparse_attention_amd as sa
    from stochastic_sparse_attention_amd._lib import SantaError, SANTA_ERR_INVALID
    cfg = synth.small_config(2, batch=1, seq_len=1024)
    dev = _dev(cfg, 3, gpu)
    BH, d, S = cfg.batch * cfg.num_q_heads, cfg.head_dim, cfg.S
    buf = torch.zeros(BH * d, dtype=torch.float32, device=gpu)
    q = buf.view(torch.bfloat16)[:BH * d].view(cfg.batch, cfg.num_q_heads, d)
    q.copy_(dev.q.view(cfg.batch, cfg.num_q_heads, d))
    before = buf.clone()
    for call in (lambda: sa.santa_decode_prop(dev.problem, q, dev.k, dev.v, S, dev.u(S), buf.view(BH, d)),
                 lambda: sa.exact_decode_ref(dev.problem, q, dev.k, dev.v, buf.view(BH, d))):
        with pytest.raises(SantaError) as e:
            call()
        assert e.value.status == SANTA_ERR_INVALID
    u = torch.zeros(BH * d, dtype=torch.float32, device=gpu)
    with pytest.raises(SantaError):
        sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, u[:BH], u.view(BH, d))
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    _say("outputs overlapping q or u are refused")


@pytest.mark.parametrize("cid", [2, 3, 8])
def test_optional_outputs_do_not_change_the_estimate(gpu, cid):
    """The benchmark times the calls without the optional index list and
    budgets (and, on Bernoulli scores, read counts).  At the full workload
    sizes those calls give bitwise the estimate of the calls that write them,
    which the full-size parity tests hold to the oracle: prop with each
    generator, flash where the workload has a flash budget, and prop on
    Bernoulli scores with the mean group query."""
    import torch
    import parity
    import stochastic_sparse_attention_amd as sa
    cfg = synth.CONFIGS[cid]
    _say(f"config {cid}: optional outputs off vs on")
    dev = _dev(cfg, 7, gpu)
    BH, d, S = cfg.batch * cfg.num_q_heads, cfg.head_dim, cfg.S
    out = torch.empty((BH, d), dtype=torch.float32, device=gpu)
    for sampler in ("sys", "strat", "iid"):
        ref, _, _ = parity.run_prop(dev, S, sampler=sampler)
        if sampler == "sys":
            sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, dev.u(S), out)
        else:
            sa.santa_decode_prop_sampler(dev.problem, dev.q, dev.k, dev.v, S, sampler, dev.uniforms(S), out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), sampler
    if cfg.S_flash:
        ref, _ = parity.run_flash(dev, cfg.S_flash)
        sa.santa_decode_flash(dev.problem, dev.q, dev.k, dev.v, cfg.S_flash, dev.u(cfg.S_flash), out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    kf = dev.k_features()
    ref, _, _, _ = parity.run_prop_bernoulli(dev, S, 4, 1, kf)
    sa.santa_decode_prop_bernoulli(dev.problem, dev.q, kf, dev.v, S, dev.u(S), 4, 1,
                                   dev.bernoulli_uniforms(4, 1), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    _say(f"config {cid}: bitwise equal with and without the optional outputs")


def test_prop_one_hot_gives_exact_row(gpu):
    """A logit gap of hundreds makes A one-hot: the output is exactly that V row."""
    import parity
    from stochastic_sparse_attention_amd.device_io import to_device
    cfg = synth.small_config(2, batch=1, seq_len=2048, hot=0, sinks=0)
    inp = synth.make_inputs(cfg, 7)
    G = cfg.group
    kv = inp.values("k").copy()
    qv = inp.values("q")
    kv *= 0.0
    for g in range(cfg.num_kv_heads):
        kv[0, g, 100 + 200 * g] = np.sign(qv[0, g * G:(g + 1) * G].mean(0)) * 1024.0
    inp.k = synth.f32_to_bf16_bits(kv)
    dev = to_device(inp, gpu)
    out, idx, tb = parity.run_prop(dev, 128)
    vv = inp.values("v")
    for h in range(cfg.num_q_heads):
        g = h // G
        assert np.all(idx[h] == 100 + 200 * g)
        assert np.array_equal(out[h], vv[0, g, 100 + 200 * g])
    parity.check_prop(dev, 128)


def test_prop_uniform_S_equals_nk_is_mean(gpu):
    """Identical keys give a uniform A; with S = n_k every token is taken once."""
    import parity
    from stochastic_sparse_attention_amd.device_io import to_device
    cfg = synth.small_config(2, batch=1, seq_len=1024, hot=0, sinks=0, num_q_heads=4, num_kv_heads=1)
    inp = synth.make_inputs(cfg, 8)
    inp.k[...] = inp.k[:, :, :1, :]
    dev = to_device(inp, gpu)
    out, idx, tb = parity.run_prop(dev, 1024)
    # F_j = (j + 1)/1024 exactly, so threshold m = U + m/1024 selects token m:
    # the list must be 0..1023 in threshold order, not only as a set
    U = dev.inp.u(1024)
    assert np.all((U > 1e-6) & (U < 1.0 / 1024 - 1e-6)), U      # no threshold near an edge
    for h in range(4):
        assert np.array_equal(idx[h], np.arange(1024)), h
    np.testing.assert_allclose(out, np.broadcast_to(inp.values("v")[0, 0].mean(0), out.shape), atol=1e-5)


def test_prop_empty_and_ragged_requests(gpu):
    import parity
    cfg = synth.small_config(5, batch=5, seq_len=3000, min_seq_len=100)
    inp = synth.make_inputs(cfg, 9)
    seq = inp.seq_lens.copy()
    seq[2] = 0
    from stochastic_sparse_attention_amd.device_io import to_device
    dev = to_device(inp, gpu, seq_lens=seq)
    rep = parity.check_prop(dev, 128)
    _say("empty+ragged", rep)


def test_prop_paged_small(gpu):
    import parity
    cfg = synth.small_config(5, batch=6, seq_len=5000, min_seq_len=500)
    rep = parity.check_prop(_dev(cfg, 10, gpu), 128)
    _say("paged small", rep)


# ------------------------------------------------------ flash and exact
@pytest.mark.parametrize("T,S", [(256, 256), (256, 2048), (128, 64), (1024, 4)])
def test_flash_small(gpu, T, S):
    import parity
    cfg = synth.small_config(3, batch=2, seq_len=4096)
    rep = parity.check_flash(_dev(cfg, 11, gpu, tile_len=T), S)
    _say("flash", T, S, rep)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_flash_paged_uniform(gpu, kv):
    """Flash over a paged cache: every request has max_seq_len keys, so the
    problem carries a page table but no per-request lengths."""
    import dataclasses
    import parity
    from stochastic_sparse_attention_amd import Problem
    cfg = synth.small_config(5, batch=3, seq_len=4096, min_seq_len=4096, kv_dtype=kv)
    dev = _dev(cfg, 20, gpu)
    prob = Problem(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.seq_len,
                   dtype=cfg.q_dtype, kv_dtype=cfg.kv_dtype, scale=float(dev.inp.scale),
                   tile_len=cfg.tile_len, page_size=cfg.page_size, page_table=dev.page_table)
    dev = dataclasses.replace(dev, problem=prob, seq_lens=None)
    _say("flash paged", kv, parity.check_flash(dev, 512))
    _say("prop paged uniform", kv, parity.check_prop(dev, 128, repeat=False))


@pytest.mark.parametrize("sampler", ["strat", "iid"])
@pytest.mark.parametrize("T,S", [(64, 4096), (256, 256), (256, 4096), (1024, 1024)])
def test_flash_samplers(gpu, sampler, T, S):
    """Stratified and i.i.d. local thresholds per tile: S_f = 64, 16, 256
    (= T) and 256 at n = 4096; and a short last tile."""
    import parity
    cfg = synth.small_config(3, batch=2, seq_len=4096)
    rep = parity.check_flash(_dev(cfg, 22, gpu, tile_len=T), S, sampler=sampler)
    _say("flash", sampler, T, S, rep)
    if T == 256 and S == 256:
        cfg = synth.small_config(3, batch=1, seq_len=1000)      # 4 tiles, the last has 232 rows
        _say("flash ragged", sampler, parity.check_flash(_dev(cfg, 23, gpu), 64, sampler=sampler))


def test_flash_ragged_last_tile(gpu):
    import parity
    cfg = synth.small_config(3, batch=1, seq_len=1000)      # 4 tiles, last has 232 rows
    rep = parity.check_flash(_dev(cfg, 12, gpu), 64)
    _say("flash ragged", rep)


def test_flash_fp32(gpu):
    import parity
    rep = parity.check_flash(_dev(synth.CONFIGS[1], 13, gpu), 64)
    _say("flash fp32", rep)


@pytest.mark.parametrize("cid,kw", [(1, {}), (2, dict(batch=2, seq_len=3000)),
                                    (5, dict(batch=4, seq_len=4000, min_seq_len=300))])
def test_exact_small(gpu, cid, kw):
    import parity
    rep = parity.check_exact(_dev(synth.small_config(cid, **kw), 14, gpu))
    _say("exact", cid, rep)


@pytest.mark.parametrize("cid,kw", [(2, dict(batch=2, seq_len=3000)),
                                    (5, dict(batch=4, seq_len=4000, min_seq_len=300)),
                                    (7, dict(batch=2, seq_len=3000))])
@pytest.mark.parametrize("T", [512, 1024])
def test_exact_larger_splits(gpu, cid, kw, T):
    """The exact baseline at the longer splits the benchmark also times
    (contiguous, paged and e4m3), ragged last tile."""
    import parity
    rep = parity.check_exact(_dev(synth.small_config(cid, **kw), 15, gpu, tile_len=T))
    _say("exact", cid, "T", T, rep)


# ------------------------------------------------- e4m3 KV
@pytest.mark.parametrize("T", [64, 256, 1024])
def test_fp8_prop_small(gpu, T):
    """e4m3 K and V with bf16 queries: prop against the oracle, which widens
    the same bytes with its own decoder."""
    import parity
    cfg = synth.small_config(6, batch=2, seq_len=3000)
    rep = parity.check_prop(_dev(cfg, 15, gpu, tile_len=T), 128)
    _say("fp8 prop T", T, rep)


def test_fp8_prop_samplers_flash_exact(gpu):
    import parity
    cfg = synth.small_config(6, batch=2, seq_len=3000)
    dev = _dev(cfg, 16, gpu)
    for smp in ("strat", "iid"):
        _say("fp8", smp, parity.check_prop(dev, 96, sampler=smp))
    _say("fp8 exact", parity.check_exact(dev))
    cfg = synth.small_config(7, batch=2, seq_len=4096)
    _say("fp8 flash", parity.check_flash(_dev(cfg, 17, gpu), 512))


def test_fp8_paged_ragged(gpu):
    import parity
    cfg = synth.small_config(5, kv_dtype="fp8", batch=5, seq_len=4000, min_seq_len=300)
    dev = _dev(cfg, 18, gpu)
    _say("fp8 paged prop", parity.check_prop(dev, 128))
    _say("fp8 paged exact", parity.check_exact(dev))


# ------------------------------------------------- full-size workloads
@pytest.mark.parametrize("cid", [2, 3, 4, 5, 6, 7])
def test_full_size_prop(gpu, cid):
    import parity
    cfg = synth.CONFIGS[cid]
    _say("generating cfg", cid)
    dev = _dev(cfg, cid, gpu)
    rep = parity.check_prop(dev, cfg.S, repeat=cid == 2)
    _say("full prop cfg", cid, rep)
    if "exact" in cfg.variants:
        _say("full exact cfg", cid, parity.check_exact(dev, repeat=False))
    if "flash" in cfg.variants:
        _say("full flash cfg", cid, parity.check_flash(dev, cfg.S_flash, repeat=False))


def test_full_size_flat_attention(gpu):
    """The 32k batch-1 layer without planted keys or sinks: smooth A, most
    tiles visited.  prop with the three threshold generators, flash at
    S = 2048 and the exact decode, each against the oracle."""
    import parity
    cfg = synth.CONFIGS[8]
    _say("generating flat cfg")
    dev = _dev(cfg, cfg.cid, gpu)
    for smp in ("sys", "strat", "iid"):
        rep = parity.check_prop(dev, cfg.S, sampler=smp, repeat=smp == "sys")
        _say("flat prop", smp, rep)
    out, idx, tb = parity.run_prop(dev, cfg.S)
    visited = (tb > 0).sum(1)
    _say("flat: tiles visited per head", float(visited.mean()), "of", tb.shape[1])
    assert visited.mean() > 0.5 * tb.shape[1]
    _say("flat flash", parity.check_flash(dev, cfg.S_flash, repeat=False))
    _say("flat exact", parity.check_exact(dev, repeat=False))


# ------------------------------------------------- offsets past 2^31 elements
def test_kv_cache_past_2_pow_31_elements(gpu):
    """A KV cache of more than 2^31 elements: 17 requests x 8 KV heads x
    131072 tokens x 128 (4.6 GB each for K and V).  The last request sits at
    the highest offsets; its heads must give bitwise the results of the same
    request run alone (prop, flash and exact decode), which are themselves
    held to the oracle bar."""
    import torch
    import parity
    import stochastic_sparse_attention_amd as sa
    cfg = synth.small_config(4, batch=1, seq_len=131072, num_q_heads=8, num_kv_heads=8)
    dev = _dev(cfg, 31, gpu)
    S, T, B = cfg.S, cfg.tile_len, 17
    nt = cfg.seq_len // T
    SF = 2 * nt
    _say("single request vs oracle, prop", parity.check_prop(dev, S, repeat=False))
    _say("single request vs oracle, flash", parity.check_flash(dev, SF, repeat=False))
    out_s, idx_s, tb_s = parity.run_prop(dev, S)
    outf_s, idxf_s = parity.run_flash(dev, SF)
    oute_s = parity.run_exact(dev)

    H, Hkv, n, d = cfg.num_q_heads, cfg.num_kv_heads, cfg.seq_len, cfg.head_dim
    assert B * Hkv * n * d > 2 ** 31
    g = torch.Generator(device=gpu)
    g.manual_seed(5)
    q = torch.randn((B, H, d), generator=g, device=gpu).to(torch.bfloat16)
    k = torch.randn((B, Hkv, n, d), generator=g, device=gpu, dtype=torch.bfloat16)
    v = torch.randn((B, Hkv, n, d), generator=g, device=gpu, dtype=torch.bfloat16)
    q[B - 1].copy_(dev.q.view(1, H, d)[0])
    k[B - 1].copy_(dev.k.view(1, Hkv, n, d)[0])
    v[B - 1].copy_(dev.v.view(1, Hkv, n, d)[0])
    u = torch.rand(B * H, generator=g, device=gpu) / S
    u[(B - 1) * H:] = dev.u(S)
    uf = torch.rand(B * H, generator=g, device=gpu) / SF
    uf[(B - 1) * H:] = dev.u(SF)
    prob = sa.Problem(B, H, Hkv, d, n, dtype="bf16", scale=dev.inp.scale, tile_len=T)
    out = torch.empty((B * H, d), dtype=torch.float32, device=gpu)
    idx = torch.empty((B * H, S), dtype=torch.int32, device=gpu)
    tb = torch.empty((B * H, nt), dtype=torch.int32, device=gpu)
    sa.santa_decode_prop(prob, q, k, v, S, u, out, idx, tb)
    torch.cuda.synchronize()
    last = slice((B - 1) * H, B * H)
    assert np.array_equal(out[last].cpu().numpy().view(np.uint32), out_s.view(np.uint32))
    assert np.array_equal(idx[last].cpu().numpy(), idx_s) and np.array_equal(tb[last].cpu().numpy(), tb_s)
    outf = torch.empty_like(out)
    idxf = torch.empty((B * H, SF), dtype=torch.int32, device=gpu)
    sa.santa_decode_flash(prob, q, k, v, SF, uf, outf, idxf)
    torch.cuda.synchronize()
    assert np.array_equal(outf[last].cpu().numpy().view(np.uint32), outf_s.view(np.uint32))
    assert np.array_equal(idxf[last].cpu().numpy(), idxf_s)
    oute = torch.empty_like(out)
    sa.exact_decode_ref(prob, q, k, v, oute)
    torch.cuda.synchronize()
    assert np.array_equal(oute[last].cpu().numpy().view(np.uint32), oute_s.view(np.uint32))
    _say("offsets past 2^31 elements: last request bitwise equal (prop, flash, exact)")


@pytest.mark.parametrize("sampler,B", [("sys", 9), ("strat", 5)])
def test_prop_split_heads_match_one_workgroup_per_head(gpu, sampler, B):
    """Up to 256 heads per call (128 with the list generators) each head's
    pass 2 runs on two workgroups whose halves are added onto the output row
    that pass 1 zeroed; above that one workgroup takes the head.  One request
    of flat attention (nearly every tile visited, so both halves add) is run
    alone (split, held to the oracle bar) and repeated B times (more heads
    than the limit): every copy must give the same indices and budgets
    bitwise, and the same output up to its last bits."""
    import torch
    import parity
    import stochastic_sparse_attention_amd as sa
    cfg = synth.small_config(8, seq_len=8192)
    dev = _dev(cfg, 43, gpu)
    S, H, Hkv, n, d = cfg.S, cfg.num_q_heads, cfg.num_kv_heads, cfg.seq_len, cfg.head_dim
    T = dev.problem.s.tile_len
    nt = n // T
    assert H <= 128 < B * H and (sampler != "sys" or B * H > 256)
    _say("split heads, alone vs oracle", sampler, parity.check_prop(dev, S, repeat=False, sampler=sampler))
    out_s, idx_s, tb_s = parity.run_prop(dev, S, sampler=sampler)
    assert (tb_s > 0).sum(axis=1).min() > 4          # more tile groups than one, so both halves add
    q = dev.q.view(1, H, d).repeat(B, 1, 1).contiguous()
    k = dev.k.view(1, Hkv, n, d).repeat(B, 1, 1, 1).contiguous()
    v = dev.v.view(1, Hkv, n, d).repeat(B, 1, 1, 1).contiguous()
    prob = sa.Problem(B, H, Hkv, d, n, dtype="bf16", scale=dev.inp.scale, tile_len=T)
    out = torch.full((B * H, d), float("nan"), dtype=torch.float32, device=gpu)
    idx = torch.full((B * H, S), -7, dtype=torch.int32, device=gpu)
    tb = torch.full((B * H, nt), -7, dtype=torch.int32, device=gpu)
    if sampler == "sys":
        sa.santa_decode_prop(prob, q, k, v, S, dev.u(S).repeat(B), out, idx, tb)
    else:
        sa.santa_decode_prop_sampler(prob, q, k, v, S, sampler, dev.uniforms(S).repeat(B, 1), out, idx, tb)
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(B, H, d)
    ii = idx.cpu().numpy().reshape(B, H, S)
    bb = tb.cpu().numpy().reshape(B, H, nt)
    for r in range(B):
        assert np.array_equal(ii[r], idx_s) and np.array_equal(bb[r], tb_s), r
        assert np.array_equal(o[r].view(np.uint32), o[0].view(np.uint32)), r
    err = float(np.abs(o[0] - out_s).max())
    assert err <= 1e-6 * float(np.abs(out_s).max()) + 1e-7, err
    _say(f"split heads ({sampler}, {B} copies): indices and budgets equal, output max diff {err:.3g}")


def _random_case(i):
    """One seeded draw of a small problem mixing the axes the other tests
    take one at a time: storage type, group size, KV heads, tile length,
    batch, contiguous or paged, ragged (also empty) requests, planted keys or
    flat attention, sample count and threshold generator."""
    rng = np.random.default_rng([0xC0B0, i])
    kv = ["bf16", "fp8", "f32"][int(rng.integers(3))]
    T = int(rng.choice([64, 128, 256, 512, 1024]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if g * Hkv <= 32]))
    B = int(rng.integers(1, 5))
    n = int(rng.integers(1, 6001))
    paged = bool(rng.random() < 0.35)
    hot, sinks = [(0, 0), (8, 0), (64, 4)][int(rng.integers(3))]
    kw = dict(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, seq_len=n, tile_len=T,
              q_dtype="f32" if kv == "f32" else "bf16", kv_dtype=kv)
    if paged:
        cfg = synth.small_config(5, min_seq_len=int(rng.integers(1, n + 1)), **kw)
        lens = None
    else:
        cfg = synth.small_config(2, hot=hot, sinks=sinks, **kw)
        lens = rng.integers(0, n + 1, size=B) if rng.random() < 0.5 else None
    S = int(rng.choice([1, 3, 64, 128, 333, 1024, 4096]))
    sampler = ["sys", "strat", "iid"][int(rng.integers(3))]
    return cfg, lens, S, sampler, int(rng.integers(1 << 30))


@pytest.mark.parametrize("case", range(24))
def test_random_combinations(gpu, case):
    """prop (also in its single launch, with systematic thresholds; and, on
    equal-length contiguous requests, flash) and the exact decode on a
    seeded random mix of shapes and options, each held to the oracle bar."""
    import parity
    cfg, lens, S, sampler, seed = _random_case(case)
    what = (f"case {case}: kv {cfg.kv_dtype}, T {cfg.tile_len}, Hq/Hkv {cfg.num_q_heads}/{cfg.num_kv_heads}, "
            f"B {cfg.batch}, n {cfg.seq_len}, paged {cfg.page_size}, lens {None if lens is None else list(lens)}, "
            f"hot {cfg.hot}+{cfg.sinks}, S {S}, {sampler}")
    _say(what)
    dev = _dev(cfg, seed, gpu, seq_lens=lens)
    _say("  prop", parity.check_prop(dev, S, sampler=sampler))
    if sampler == "sys":
        _say("  single-launch prop", parity.check_prop(dev, S, fused=True))
    _say("  exact", parity.check_exact(dev))
    if not cfg.page_size and lens is None:
        nt = -(-cfg.seq_len // cfg.tile_len)
        Sf = int(np.random.default_rng(case).choice([1, 2, 4]))
        Sf = min(Sf, cfg.tile_len)
        _say("  flash", nt * Sf, parity.check_flash(dev, nt * Sf, sampler=sampler))


# ------------------------------------------------- Bernoulli qK^T + prop
@pytest.mark.parametrize("T", [64, 256, 1024])
@pytest.mark.parametrize("draws,group_mean", [(1, 0), (4, 0), (4, 1), (16, 1)])
def test_bernoulli_prop_small(gpu, T, draws, group_mean):
    """Ragged last tile (3000 keys), two requests, groups of 4."""
    import parity
    cfg = synth.small_config(2, batch=2, seq_len=3000)
    rep = parity.check_prop_bernoulli(_dev(cfg, 41, gpu, tile_len=T), 128, draws, group_mean)
    _say("bernoulli T", T, "draws", draws, "mean", group_mean, rep)


@pytest.mark.parametrize("hq,hkv,T", [(8, 8, 256), (8, 4, 256), (16, 2, 256), (16, 2, 64), (16, 2, 1024)])
@pytest.mark.parametrize("group_mean", [0, 1])
def test_bernoulli_prop_groups(gpu, hq, hkv, T, group_mean):
    """Groups of 1, 2 and 8; G = 8 also at the smallest and largest tiles
    (the most per-slot partial sums in LDS)."""
    import parity
    cfg = synth.small_config(2, batch=2, seq_len=2048, num_q_heads=hq, num_kv_heads=hkv)
    rep = parity.check_prop_bernoulli(_dev(cfg, 42, gpu, tile_len=T), 64, 4, group_mean)
    _say("bernoulli G", hq // hkv, "T", T, "mean", group_mean, rep)


@pytest.mark.parametrize("case", range(12))
def test_bernoulli_random_combinations(gpu, case):
    """Prop on Bernoulli scores over a seeded random mix: bf16 or e4m3 KV,
    group size, KV heads, tile length, batch, ragged (also empty) requests,
    planted keys or none, draws, per-head or mean group query, and S."""
    import parity
    rng = np.random.default_rng([0xBE70, case])
    kv = ["bf16", "fp8"][int(rng.integers(2))]
    T = int(rng.choice([64, 128, 256, 512, 1024]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8) if g * Hkv <= 32]))
    B = int(rng.integers(1, 4))
    n = 4 * int(rng.integers(1, 1501))                 # the feature-major copy takes 4 keys per lane load
    hot, sinks = [(0, 0), (8, 0), (64, 4)][int(rng.integers(3))]
    lens = rng.integers(0, n + 1, size=B) if rng.random() < 0.5 else None
    draws = int(rng.choice([1, 2, 4, 16]))
    gm = int(rng.integers(2))
    S = int(rng.choice([1, 3, 64, 128, 1024]))
    cfg = synth.small_config(2, batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, seq_len=n, tile_len=T,
                             kv_dtype=kv, hot=hot, sinks=sinks)
    _say(f"case {case}: kv {kv}, T {T}, Hq/Hkv {G * Hkv}/{Hkv}, B {B}, n {n}, "
         f"lens {None if lens is None else [int(x) for x in lens]}, hot {hot}+{sinks}, draws {draws}, "
         f"mean {gm}, S {S}")
    dev = _dev(cfg, int(rng.integers(1 << 30)), gpu, seq_lens=lens)
    _say("  bernoulli", parity.check_prop_bernoulli(dev, S, draws, gm))


def test_bernoulli_prop_empty_ragged_and_tiny(gpu):
    """Requests of 0, 4, 300 and 2996 keys in a 3000-key cache, and a cache
    of 4 keys (one partial tile)."""
    import parity
    from stochastic_sparse_attention_amd.device_io import to_device
    cfg = synth.small_config(2, batch=4, seq_len=3000, num_q_heads=8, num_kv_heads=2)
    inp = synth.make_inputs(cfg, 43)
    dev = to_device(inp, gpu, seq_lens=np.array([0, 4, 300, 2996], np.int32))
    for draws, gm in [(4, 0), (4, 1)]:
        _say("bernoulli empty+ragged", gm, parity.check_prop_bernoulli(dev, 128, draws, gm))
    cfg = synth.small_config(2, batch=1, seq_len=4, hot=0, sinks=2, num_q_heads=8, num_kv_heads=2)
    _say("bernoulli 4 keys", parity.check_prop_bernoulli(_dev(cfg, 44, gpu), 16, 2, 0))


@pytest.mark.parametrize("T", [64, 256])
def test_bernoulli_prop_fp8_small(gpu, T):
    """e4m3 K (feature-major) and V with bf16 queries, ragged last tile."""
    import parity
    cfg = synth.small_config(7, batch=2, seq_len=3000)
    dev = _dev(cfg, 45, gpu, tile_len=T)
    for draws, gm in [(4, 0), (4, 1), (1, 1)]:
        _say("bernoulli fp8 T", T, "draws", draws, "mean", gm, parity.check_prop_bernoulli(dev, 128, draws, gm))


@pytest.mark.parametrize("cid", [2, 3, 4, 6, 7])
def test_bernoulli_prop_full_size(gpu, cid):
    import parity
    cfg = synth.CONFIGS[cid]
    dev = _dev(cfg, cid, gpu)
    for draws, gm in [(4, 0), (4, 1)]:
        _say("bernoulli full cfg", cid, "mean", gm,
             parity.check_prop_bernoulli(dev, cfg.S, draws, gm, repeat=cid == 2))


# ------------------------------------------------- single-launch prop
def _fused_vs_two_launch(dev, S, workspace=None):
    """The single-launch prop against the oracle (the parity bar) and against
    the two-launch prop: the same indices and budgets, outputs equal to
    rounding of the summation order."""
    import parity
    rep = parity.check_prop(dev, S, fused=True, workspace=workspace)
    o1, i1, t1 = parity.run_prop(dev, S)
    o2, i2, t2 = parity.run_prop(dev, S, fused=True, workspace=workspace)
    assert np.array_equal(i1, i2) and np.array_equal(t1, t2)
    rep["max_abs_vs_two_launch"] = float(np.max(np.abs(o1 - o2))) if o1.size else 0.0
    assert rep["max_abs_vs_two_launch"] <= 1e-5
    return rep


@pytest.mark.parametrize("T", [64, 256, 1024])
def test_fused_prop_tiles(gpu, T):
    cfg = synth.small_config(2, batch=2, seq_len=4000)
    _say("fused T", T, _fused_vs_two_launch(_dev(cfg, 61, gpu, tile_len=T), 128))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (16, 2)])
def test_fused_prop_groups(gpu, hq, hkv):
    cfg = synth.small_config(2, batch=2, seq_len=3000, num_q_heads=hq, num_kv_heads=hkv)
    _say("fused G", hq // hkv, _fused_vs_two_launch(_dev(cfg, 62, gpu), 64))


def test_fused_prop_paged_ragged_empty(gpu):
    """Paged KV, mixed lengths and an empty request (which counts no tile:
    its tile-0 workgroup writes the empty results)."""
    from stochastic_sparse_attention_amd.device_io import to_device
    cfg = synth.small_config(5, batch=5, seq_len=3000, min_seq_len=100)
    inp = synth.make_inputs(cfg, 63)
    seq = inp.seq_lens.copy()
    seq[1] = 0
    _say("fused paged ragged empty", _fused_vs_two_launch(to_device(inp, gpu, seq_lens=seq), 128))


def test_fused_prop_full_size(gpu):
    cfg = synth.CONFIGS[2]
    _say("fused full size", _fused_vs_two_launch(_dev(cfg, cfg.cid, gpu), cfg.S))


def test_fused_prop_counters_reset(gpu):
    """The arrival counters return to zero after every call: one workspace
    serves repeated calls, and a call on another problem in between (whose
    counters overlap the first problem's), each result still at the bar."""
    import stochastic_sparse_attention_amd as sa
    import torch
    big = _dev(synth.small_config(2, batch=4, seq_len=6000), 64, gpu)
    small = _dev(synth.small_config(2, batch=1, seq_len=1500, num_q_heads=8, num_kv_heads=2), 65, gpu, tile_len=64)
    ws = sa.new_workspace(big.problem, "prop", 128, gpu)
    for rep in range(2):
        _say("fused reuse big", rep, _fused_vs_two_launch(big, 128, workspace=ws))
        _say("fused reuse small", rep, _fused_vs_two_launch(small, 32, workspace=ws))
    torch.cuda.synchronize()
    assert int(ws[:sa._lib.SANTA_SYNC_BYTES].count_nonzero()) == 0


# ------------------------------------------------- HIP graph replay
def test_graph_replays_match_eager(gpu):
    """prop (all three threshold generators, on Bernoulli scores with the
    mean group query, and in one launch), flash (systematic and stratified)
    and exact decode captured in one HIP graph: every replay,
    with eager work and synchronisations in between, gives results bitwise
    equal to the eager calls."""
    import torch
    import stochastic_sparse_attention_amd as sa
    cfg = synth.small_config(2, batch=2, seq_len=3000)
    dev = _dev(cfg, 21, gpu)
    S, BH = 128, cfg.batch * cfg.num_q_heads
    max_nt = (cfg.seq_len + cfg.tile_len - 1) // cfg.tile_len
    U, uu = dev.u(S), dev.uniforms(S)
    ws = torch.empty(sa.santa_workspace_size(dev.problem, "prop", S), dtype=torch.uint8, device=gpu)
    wse = torch.empty(sa.santa_workspace_size(dev.problem, "exact"), dtype=torch.uint8, device=gpu)
    SF = 16 * max_nt                                  # flash: 16 samples per tile
    UF, uuf = dev.u(SF), dev.uniforms(SF)
    wsf = torch.empty(sa.santa_workspace_size(dev.problem, "flash", SF), dtype=torch.uint8, device=gpu)
    outs = {k: torch.empty((BH, 128), dtype=torch.float32, device=gpu)
            for k in ("sys", "strat", "iid", "exact", "flash", "flash_strat", "bernoulli", "fused")}
    wsz = sa.new_workspace(dev.problem, "prop", S, gpu)
    kf, ub = dev.k_features(), dev.bernoulli_uniforms(4, True)
    fr = torch.empty(cfg.batch * cfg.num_kv_heads, dtype=torch.int32, device=gpu)
    idx = torch.empty((BH, S), dtype=torch.int32, device=gpu)
    tb = torch.empty((BH, max_nt), dtype=torch.int32, device=gpu)

    def step():
        sa.santa_decode_prop(dev.problem, dev.q, dev.k, dev.v, S, U, outs["sys"], idx, tb, workspace=ws)
        for smp in ("strat", "iid"):
            sa.santa_decode_prop_sampler(dev.problem, dev.q, dev.k, dev.v, S, smp, uu, outs[smp], workspace=ws)
        sa.exact_decode_ref(dev.problem, dev.q, dev.k, dev.v, outs["exact"], workspace=wse)
        sa.santa_decode_flash(dev.problem, dev.q, dev.k, dev.v, SF, UF, outs["flash"], workspace=wsf)
        sa.santa_decode_flash_sampler(dev.problem, dev.q, dev.k, dev.v, SF, "strat", uuf, outs["flash_strat"],
                                      workspace=wsf)
        sa.santa_decode_prop_bernoulli(dev.problem, dev.q, kf, dev.v, S, U, 4, 1, ub, outs["bernoulli"],
                                       features_read=fr, workspace=ws)
        sa.santa_decode_prop_fused(dev.problem, dev.q, dev.k, dev.v, S, U, outs["fused"], workspace=wsz)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref_idx, ref_tb, ref_fr = idx.clone(), tb.clone(), fr.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=gpu)
    for rep in range(3):
        for v in outs.values():
            v.fill_(float("nan"))
        idx.fill_(-5)
        tb.fill_(-5)
        fr.fill_(-5)
        scratch.mul_(1.0001)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.int32), ref[k].view(torch.int32)), (rep, k)
        assert torch.equal(idx, ref_idx) and torch.equal(tb, ref_tb), rep
        assert torch.equal(fr, ref_fr), rep
    _say("graph replays match eager")
