"""Seeded synthetic decode-attention inputs.

This module only draws inputs: query vectors, KV caches with planted
high-scoring keys, page tables, sequence lengths and the sampling offset U.
It holds none of the method's arithmetic, so both the GPU path and the CPU
oracle take their inputs from here.

Workload shapes follow the pages: a Llama-3.1-8B decode layer (32 query
heads, 8 KV heads, head dim 128, 32k context) from the SANTA notes
("Stochastic Sparse Attention for Memory-Bound Inference", background and
Table 1) and the Double-P review (evaluation setup: LLaMA3.1-8B with GQA group
size 4, Quest's 16-token pages, 4 sink tokens and a 64-token local window).
The pages evaluate on RULER, GSM8K and MMLU; none of those suites is used
here -- these synthetic tensors stand in for their decode-step shape.

Recipe (every config):
  * numpy.random.default_rng(seed); draws in this order: sequence lengths and
    per-(request, KV head) hot density (mixed-batch config only), q, K, V,
    planted positions, planted-key noise, page permutation, U.
  * q, K, V ~ N(0, 1) drawn in fp32, rounded to bf16 (round to nearest even)
    where the config stores bf16.
  * planted keys: k = alpha * qbar/|qbar| * sqrt(d) + N(0, 0.1^2) per element,
    alpha = 3, qbar = mean of the (stored) query heads sharing that KV head.
  * U = floor(r * 2^24) * 2^-24 / S with r ~ Unif[0,1): exact in fp32 and in
    [0, 1/S).  One r per (request, q head), or per request where the config
    says so (replicated over that request's heads).
  * the stratified and i.i.d. threshold generators take S uniforms per
    (request, q head), on the same 2^-24 grid, from their own generator
    seeded by (seed, 0x5A17, S).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ALPHA = 3.0          # planted-key alignment strength
NOISE_STD = 0.1      # per-element noise on planted keys


@dataclass(frozen=True)
class Config:
    """One synthetic workload."""
    cid: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int                  # n_k (contiguous) or the maximum (mixed batch)
    q_dtype: str                  # "f32" | "bf16"
                                  # kv_dtype also "fp8" (OCP e4m3, with bf16 q)
    kv_dtype: str
    S: int                        # samples per q head (prop)
    tile_len: int                 # T, tokens per tile
    hot: int = 0                  # planted keys per KV head (fixed count)
    sinks: int = 0                # tokens 0..sinks-1 planted
    window: int = 0               # last `window` tokens planted
    S_flash: int = 0              # flash budget (0: flash not run on this config)
    u_per_request: bool = False   # one U per request, replicated over heads
    page_size: int = 0            # 0: contiguous KV
    min_seq_len: int = 0          # mixed batch: n_k ~ U{min..seq_len}
    density: tuple = ()           # mixed batch: hot density ~ U[lo, hi]
    variants: tuple = ("prop",)
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    1: Config(1, "single head, n_k=1024, fp32", 1, 1, 1, 128, 1024, "f32", "f32",
              S=16, tile_len=128, hot=8),
    2: Config(2, "Llama-3.1-8B decode layer, 32k context, batch 1", 1, 32, 8, 128, 32768,
              "bf16", "bf16", S=128, tile_len=256, hot=64, sinks=4,
              variants=("prop", "exact")),
    3: Config(3, "Llama-3.1-8B decode layer, 32k context, batch 16", 16, 32, 8, 128, 32768,
              "bf16", "bf16", S=128, tile_len=256, hot=64, sinks=4, S_flash=2048,
              u_per_request=True, variants=("prop", "flash", "exact")),
    4: Config(4, "long context 128k, batch 4", 4, 32, 8, 128, 131072, "bf16", "bf16",
              S=256, tile_len=512, hot=256, sinks=4, window=64,
              variants=("prop", "exact")),
    5: Config(5, "Qwen3-8B-shaped mixed batch of 64, paged 16", 64, 32, 8, 128, 32768,
              "bf16", "bf16", S=128, tile_len=256, page_size=16, min_seq_len=4096,
              density=(0.001, 0.05), variants=("prop", "exact")),
    # e4m3 KV (bf16 queries): the 32k layer shape again, at batch 1 and 16
    6: Config(6, "Llama-3.1-8B decode layer, 32k context, batch 1, fp8 e4m3 KV", 1, 32, 8, 128, 32768,
              "bf16", "fp8", S=128, tile_len=256, hot=64, sinks=4, variants=("prop", "exact")),
    7: Config(7, "Llama-3.1-8B decode layer, 32k context, batch 16, fp8 e4m3 KV", 16, 32, 8, 128, 32768,
              "bf16", "fp8", S=128, tile_len=256, hot=64, sinks=4, S_flash=2048, u_per_request=True,
              variants=("prop", "flash", "exact")),
    # flat attention (no planted keys, no sinks): the logits are ~N(0, 1),
    # so A is smooth, nearly every tile takes a threshold and the visit list
    # runs near its cap (the SANTA notes name flat attention as the case
    # their analysis does not cover)
    8: Config(8, "Llama-3.1-8B decode layer, 32k context, batch 1, flat attention", 1, 32, 8, 128, 32768,
              "bf16", "bf16", S=128, tile_len=256, S_flash=2048, variants=("prop", "flash", "exact")),
}


# --------------------------------------------------------------------------
# bf16 storage helpers (IEEE binary32 with the low 16 bits rounded away)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits.

    Works in uint32 on chunks (finite values cannot overflow: the largest
    finite magnitude plus the rounding bias stays below 2^32); NaN maps to
    the canonical quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.size, np.uint16)
    for s in range(0, flat.size, chunk):
        u = flat[s:s + chunk]
        lsb = (u >> 16) & np.uint32(1)
        r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
        nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = 0x7FC0
        out[s:s + chunk] = r
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# OCP e4m3 storage helpers (1 sign bit, 4 exponent bits with bias 7, 3
# mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; S.1111.111
# is NaN; no infinities; largest finite magnitude 448)
# --------------------------------------------------------------------------
def _e4m3_magnitudes() -> np.ndarray:
    """Values of the codes 0..126 (non-negative, finite), increasing."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round to e4m3: nearest, ties to the even code (even mantissa),
    magnitudes above 448 saturate to 448; NaN maps to 0x7F."""
    x = np.asarray(x, np.float32)
    a = np.abs(x.astype(np.float64)).reshape(-1)
    mags = _e4m3_magnitudes()
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code[a >= 448.0] = 126
    code |= (np.signbit(x.reshape(-1)).astype(np.uint8) << 7)
    code[np.isnan(a)] = 0x7F
    return code.reshape(x.shape)


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, np.uint8)
    table = np.concatenate([_e4m3_magnitudes(), [np.nan]])
    mag = table[b & 0x7F]
    return np.where(b & 0x80, -mag, mag).astype(np.float32)


@dataclass
class Inputs:
    """One drawn problem instance (host arrays)."""
    cfg: Config
    seed: int
    q: np.ndarray              # stored values: float32 array, or uint16 bf16 bits
    k: np.ndarray              # contiguous [B,Hkv,n_k,d] or pool [pages,Hkv,P,d]
    v: np.ndarray
    seq_lens: np.ndarray       # int32 [B]
    page_table: np.ndarray     # int32 [B, max_pages] (empty when contiguous)
    r: np.ndarray              # float64 [B*Hq], on the 2^-24 grid in [0, 1)
    hot_positions: list        # per (b, g): np.ndarray of planted token indices
    scale: np.float32

    def u(self, S: int) -> np.ndarray:
        """Offsets U in [0, 1/S) as fp32 (exact: r is a multiple of 2^-24)."""
        return (self.r / float(S)).astype(np.float32)

    def uniforms(self, S: int) -> np.ndarray:
        """[B*Hq, S] uniforms in [0, 1) on the 2^-24 grid (exact in fp32), for
        the stratified and i.i.d. threshold generators; drawn from their own
        stream, seeded by (seed, S), so the other draws are unchanged."""
        rng = np.random.default_rng([self.seed, 0x5A17, S])
        n = self.cfg.batch * self.cfg.num_q_heads
        return (np.floor(rng.random((n, S)) * 2.0 ** 24) * 2.0 ** -24).astype(np.float32)

    def bernoulli_uniforms(self, draws: int, group_mean: bool) -> np.ndarray:
        """Uniforms in [0, 1) on the 2^-24 grid (exact in fp32) for the
        ternary query draws of Bernoulli scoring: [B*Hq, draws, d] (one set
        per head), or [B*Hkv, draws, d] when a group shares its mean query.
        Their own stream, seeded by (seed, draws, group_mean)."""
        c = self.cfg
        rng = np.random.default_rng([self.seed, 0xBE7, draws, int(group_mean)])
        owners = c.batch * (c.num_kv_heads if group_mean else c.num_q_heads)
        return (np.floor(rng.random((owners, draws, c.head_dim)) * 2.0 ** 24) * 2.0 ** -24).astype(np.float32)

    @property
    def contiguous(self) -> bool:
        return self.cfg.page_size == 0

    @property
    def uniform_len(self) -> bool:
        return bool(np.all(self.seq_lens == self.cfg.seq_len))

    def values(self, name: str) -> np.ndarray:
        """fp32 view of a stored tensor (widens bf16 exactly)."""
        a = getattr(self, name)
        dt = self.cfg.q_dtype if name == "q" else self.cfg.kv_dtype
        return _stored_f32(a, dt)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp8":
        return f32_to_e4m3_bits(x)
    return np.ascontiguousarray(x, np.float32)


def _stored_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "fp8":
        return e4m3_bits_to_f32(x)
    return x


def make_inputs(cfg: Config, seed: int) -> Inputs:
    """Draw one instance of `cfg` from `seed` (deterministic)."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, G = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.group

    # sequence lengths and hot densities (mixed batch only)
    if cfg.min_seq_len:
        seq_lens = rng.integers(cfg.min_seq_len, cfg.seq_len + 1, size=B).astype(np.int32)
        lo, hi = cfg.density
        dens = rng.uniform(lo, hi, size=(B, Hkv))
    else:
        seq_lens = np.full(B, cfg.seq_len, np.int32)
        dens = None

    q32 = rng.standard_normal((B, Hq, d), dtype=np.float32)
    q = _store(q32, cfg.q_dtype)
    qv = _stored_f32(q, cfg.q_dtype).astype(np.float64)

    P = cfg.page_size
    if P:
        pages_per = (seq_lens + P - 1) // P
        num_pages = int(pages_per.sum())
        kshape = (num_pages, Hkv, P, d)
    else:
        kshape = (B, Hkv, cfg.seq_len, d)
    k32 = rng.standard_normal(kshape, dtype=np.float32)
    v32 = rng.standard_normal(kshape, dtype=np.float32)

    # planted positions per (b, g), then their noise
    hot_positions = []
    for b in range(B):
        n = int(seq_lens[b])
        for g in range(Hkv):
            fixed = list(range(min(cfg.sinks, n)))
            if cfg.window:
                fixed += list(range(max(0, n - cfg.window), n))
            fixed = sorted(set(fixed))
            nhot = cfg.hot if dens is None else max(1, int(round(dens[b, g] * n)))
            rest = np.setdiff1d(np.arange(n), np.asarray(fixed, dtype=np.int64))
            nhot = min(nhot, rest.size)
            pick = rng.choice(rest, size=nhot, replace=False) if nhot else np.empty(0, np.int64)
            hot_positions.append(np.sort(np.concatenate([np.asarray(fixed, np.int64), pick])))

    for b in range(B):
        for g in range(Hkv):
            pos = hot_positions[b * Hkv + g]
            if pos.size == 0:
                continue
            qbar = qv[b, g * G:(g + 1) * G].mean(axis=0)
            direction = qbar / np.linalg.norm(qbar)
            noise = rng.normal(0.0, NOISE_STD, size=(pos.size, d))
            rows = (ALPHA * math.sqrt(d) * direction[None, :] + noise).astype(np.float32)
            _plant(k32, rows, b, g, pos, cfg, seq_lens)

    if P:
        # logical page (b, i) -> physical page perm[offset_b + i]
        perm = rng.permutation(num_pages).astype(np.int32)
        # one row per request, wide enough for the longest allowed request
        max_pages = (cfg.seq_len + P - 1) // P
        page_table = np.zeros((B, max_pages), np.int32)
        offs = np.concatenate([[0], np.cumsum(pages_per)])
        for b in range(B):
            page_table[b, :pages_per[b]] = perm[offs[b]:offs[b + 1]]
        # physical pool: page perm[x] holds logical page x
        pool_k = np.empty_like(k32)
        pool_v = np.empty_like(v32)
        pool_k[perm] = k32
        pool_v[perm] = v32
        k32, v32 = pool_k, pool_v
        # slots past the end of each request's last page are never valid keys:
        # fill them with NaN so any read of them shows up in the results
        for b in range(B):
            tail = int(pages_per[b] * P - seq_lens[b])
            if tail:
                last = page_table[b, pages_per[b] - 1]
                k32[last, :, P - tail:, :] = np.nan
                v32[last, :, P - tail:, :] = np.nan
    else:
        page_table = np.zeros((0, 0), np.int32)

    k = _store(k32, cfg.kv_dtype)
    v = _store(v32, cfg.kv_dtype)
    del k32, v32

    nr = B if cfg.u_per_request else B * Hq
    r = np.floor(rng.random(nr) * 2.0 ** 24) * 2.0 ** -24
    if cfg.u_per_request:
        r = np.repeat(r, Hq)
    scale = np.float32(1.0 / math.sqrt(d))
    return Inputs(cfg, seed, q, k, v, seq_lens, page_table, r, hot_positions, scale)


def _plant(k32, rows, b, g, pos, cfg, seq_lens):
    P = cfg.page_size
    if P:
        # before the physical permutation, pages are stored in logical order:
        # request b's logical pages start at sum of earlier requests' pages
        pages_per = (seq_lens + P - 1) // P
        base = int(pages_per[:b].sum())
        k32[base + pos // P, g, pos % P, :] = rows
    else:
        k32[b, g, pos, :] = rows


def small_config(cid: int, **overrides) -> Config:
    """A shrunken copy of config `cid` for fast tests (same structure)."""
    return CONFIGS[cid].scaled(**overrides)
