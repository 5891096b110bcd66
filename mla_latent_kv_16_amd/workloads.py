"""Seeded synthetic inputs for paged latent-KV MLA decode and prefix prefill.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can consume its
output without sharing any of the method's code.

Shapes follow the agent workloads the TokenSpeed pages describe: coding-agent
sessions whose context runs past 50K tokens, speculative decoding at batch
4/8/16 against a long cached prefix, and prefill of a new chunk on top of a
long cached prefix (news article "英伟达力荐，小团队两个月开源一款「光速级」智能体推理引擎",
performance-preview paragraphs).  The trajectories those pages evaluate on are
not available; these seeded tensors stand in for them.

Layout (all little-endian, C-contiguous):
  q_nope      uint16 bf16 bits  [B, Sq, H, 512]   absorbed no-RoPE query part
  q_rope      uint16 bf16 bits  [B, Sq, H, 64]    rotated RoPE query part
  kv_pool     uint16 bf16 bits  [P, 64, 576]      latent rows: 512 c_kv | 64 k_rope
  block_table int32             [B, max_pages]    logical page -> physical page, -1 unused
  seq_lens    int32             [B]               visible rows incl. the Sq new rows

Recipe (numpy PCG64, seed per workload), in this order:
  1. per-request length L_b (fixed, or integers(lo, hi + 1));
  2. perm = permutation(pool_pages) with pool_pages = 2 * sum(ceil(L_b / 64));
     request b takes the next ceil(L_b / 64) entries of perm as its block-table row;
  3. for b in order: standard_normal((L_b, 576), float32) * kv_sigma, rounded to
     bf16 (round-to-nearest-even) and scattered row by row into its pages;
  4. q_nope standard_normal([B, Sq, H, 512]) * q_sigma -> bf16;
  5. q_rope standard_normal([B, Sq, H, 64]) * q_sigma -> bf16.
Pool pages no request uses, and the rows past L_b in each request's last page,
hold bf16 quiet NaN (0x7FC0) so any stray read shows up in the result.

FP8 latent pools (kv_format="e4m3"): the same draws, divided by a per-tensor
scale and rounded to OCP FP8 E4M3 (round-to-nearest-even, saturating at +-448);
kv_pool is then uint8 [P, 64, 576] and stray rows hold the E4M3 NaN code 0x7F.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D_C = 512          # latent (c_kv) width
D_R = 64           # decoupled RoPE key width
D_ROW = D_C + D_R  # one pool row
PAGE = 64          # rows per page
BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0
DEFAULT_KV_SCALE = 2.0 ** -6  # N(0,1) latents / 2^-6 stay inside +-448
DEFAULT_SCALE = np.float32(192.0 ** -0.5)  # (128 nope + 64 rope) ** -0.5


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    seed: int
    B: int
    Sq: int
    H: int
    lens: tuple            # ("fixed", L) or ("uniform", lo, hi) inclusive
    causal: bool = True
    q_sigma: float = 1.0
    kv_sigma: float = 1.0
    description: str = ""


K = 1024
WORKLOADS = {
    "tiny": WorkloadSpec(
        "tiny", 0, B=1, Sq=1, H=16, lens=("fixed", 256),
        description="B=1 Sq=1 H=16, 256-token context in 4 scattered pages of an 8-page pool"),
    "spec4": WorkloadSpec(
        "spec4", 1, B=4, Sq=4, H=16, lens=("fixed", 64 * K + 4),
        description="agent spec-decode B=4 Sq=4 H=16, 65,536-token prefix + 4 draft rows"),
    "spec8": WorkloadSpec(
        "spec8", 2, B=8, Sq=8, H=16, lens=("uniform", 32 * K, 128 * K),
        description="agent spec-decode B=8 Sq=8 H=16, context U[32K,128K]"),
    "spec16": WorkloadSpec(
        "spec16", 3, B=16, Sq=16, H=16, lens=("uniform", 50 * K, 200 * K),
        description="agent spec-decode B=16 Sq=16 H=16, context U[50K,200K]"),
    "sweep": WorkloadSpec(
        "sweep", 4, B=64, Sq=1, H=128, lens=("uniform", 8 * K, 32 * K),
        description="throughput sweep B=64 Sq=1 H=128, context U[8K,32K]"),
    "prefill": WorkloadSpec(
        "prefill", 5, B=1, Sq=4096, H=16, lens=("fixed", 64 * K + 4096),
        description="chunked prefill: 4,096-token chunk on a 65,536-token cached prefix, H=16"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def _e4m3_positive_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, indexed by code 0x00..0x7E."""
    c = np.arange(127)
    e, m = c >> 3, (c & 7).astype(np.float64)
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))


_E4M3_POS = _e4m3_positive_values()


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to OCP FP8 E4M3 codes: nearest value, ties to the
    even code, magnitudes beyond 448 saturated to 448.  Returns uint8 codes.

    Normal results (|x| >= 2^-6) keep 3 mantissa bits: the float32 pattern is rounded
    to nearest-even at bit 20 and re-biased from exponent 127 to 7.  Below 2^-6 the
    codes are the multiples of 2^-9 (subnormals; 8 * 2^-9 is the smallest normal,
    whose code is also 8), so the code is rint(|x| * 512)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(E4M3_MAX))
    bits = a.view(np.uint32)
    r = (bits + np.uint32(0x7FFFF) + ((bits >> np.uint32(20)) & np.uint32(1))) \
        & np.uint32(0xFFF00000)
    exp = ((r >> np.uint32(23)).astype(np.int32) - 127 + 7).clip(0, 15)
    normal = ((exp << 3) | ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32))
    sub = np.rint(a * np.float32(512.0)).astype(np.int32)
    code = np.where(a < np.float32(2.0 ** -6), sub, normal).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    q_nope: np.ndarray       # uint16 [B, Sq, H, 512]
    q_rope: np.ndarray       # uint16 [B, Sq, H, 64]
    kv_pool: np.ndarray      # uint16 bf16 bits, or uint8 E4M3 codes [P, 64, 576]
    block_table: np.ndarray  # int32 [B, max_pages]
    seq_lens: np.ndarray     # int32 [B]
    scale: np.float32
    causal: bool
    kv_format: str = "bf16"  # "bf16" or "e4m3"
    kv_scale: float = 1.0    # per-tensor dequantization scale of an E4M3 pool

    @property
    def B(self):
        return self.q_nope.shape[0]

    @property
    def Sq(self):
        return self.q_nope.shape[1]

    @property
    def H(self):
        return self.q_nope.shape[2]

    @property
    def num_pages(self):
        return self.kv_pool.shape[0]

    @property
    def max_pages(self):
        return self.block_table.shape[1]

    @property
    def row_bytes(self) -> int:
        return self.kv_pool.shape[2] * (1 if self.kv_format == "e4m3" else 2)

    def kv_bytes(self) -> int:
        """Latent bytes a step must read: every visible row once (576 bf16 or E4M3)."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.row_bytes


def _draw_lens(spec: WorkloadSpec, rng: np.random.Generator, B: int) -> np.ndarray:
    kind = spec.lens[0]
    if kind == "fixed":
        return np.full(B, spec.lens[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec.lens[1], spec.lens[2] + 1, size=B).astype(np.int64)
    raise ValueError(kind)


def draw_layout(spec_or_name):
    """Steps 1 and 2 of the recipe alone: (spec, L int64 [B], block_table int32
    [B, max_pages], pool_pages), with the same draws make_workload takes first."""
    spec = WORKLOADS[spec_or_name] if isinstance(spec_or_name, str) else spec_or_name
    rng = np.random.default_rng(spec.seed)
    L = _draw_lens(spec, rng, spec.B)
    pages_per = (L + PAGE - 1) // PAGE
    pool_pages = max(1, 2 * int(pages_per.sum()))
    perm = rng.permutation(pool_pages).astype(np.int32)
    block_table = np.full((spec.B, max(1, int(pages_per.max()))), -1, dtype=np.int32)
    off = 0
    for b in range(spec.B):
        n = int(pages_per[b])
        block_table[b, :n] = perm[off:off + n]
        off += n
    return spec, L, block_table, pool_pages


def make_workload(spec_or_name, *, seed: Optional[int] = None, B: Optional[int] = None,
                  Sq: Optional[int] = None, H: Optional[int] = None,
                  lens=None, causal: Optional[bool] = None,
                  q_sigma: Optional[float] = None, kv_sigma: Optional[float] = None,
                  poison: bool = True, pool_factor: int = 2,
                  scale: Optional[float] = None, kv_format: str = "bf16",
                  kv_scale: Optional[float] = None, rope: bool = True) -> Workload:
    """Build one seeded workload.  Any keyword overrides the named spec.  With
    kv_format="e4m3" the latent rows are the same draws stored as E4M3 codes of
    value / kv_scale."""
    if kv_format not in ("bf16", "e4m3"):
        raise ValueError(kv_format)
    # rope=False: NoPE-MLA, pool rows are the 512-wide latent alone and q_rope is empty
    width = D_ROW if rope else D_C
    kvs = float(DEFAULT_KV_SCALE if kv_scale is None else kv_scale)
    spec = WORKLOADS[spec_or_name] if isinstance(spec_or_name, str) else spec_or_name
    over = {k: v for k, v in dict(seed=seed, B=B, Sq=Sq, H=H, lens=lens, causal=causal,
                                  q_sigma=q_sigma, kv_sigma=kv_sigma).items() if v is not None}
    if over:
        spec = dataclasses.replace(spec, **over)
    rng = np.random.default_rng(spec.seed)
    Bn, Sqn, Hn = spec.B, spec.Sq, spec.H

    L = _draw_lens(spec, rng, Bn)
    if (L < Sqn).any():
        raise ValueError("every request needs at least Sq visible rows")
    pages_per = (L + PAGE - 1) // PAGE
    pool_pages = max(1, pool_factor * int(pages_per.sum()))
    perm = rng.permutation(pool_pages).astype(np.int32)
    max_pages = max(1, int(pages_per.max()))
    block_table = np.full((Bn, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(Bn):
        n = int(pages_per[b])
        block_table[b, :n] = perm[off:off + n]
        off += n

    if kv_format == "e4m3":
        fill = E4M3_NAN if poison else np.uint8(0)
        pool = np.full((pool_pages, PAGE, width), fill, dtype=np.uint8)
    else:
        fill = BF16_NAN if poison else np.uint16(0)
        pool = np.full((pool_pages, PAGE, width), fill, dtype=np.uint16)
    for b in range(Bn):
        Lb = int(L[b])
        draws = rng.standard_normal((Lb, width), dtype=np.float32) * np.float32(spec.kv_sigma)
        if kv_format == "e4m3":
            rows = f32_to_e4m3_bits(draws / np.float32(kvs))
        else:
            rows = f32_to_bf16_bits(draws)
        del draws
        n = int(pages_per[b])
        full = Lb // PAGE
        if full:
            pool[block_table[b, :full]] = rows[:full * PAGE].reshape(full, PAGE, width)
        if n > full:
            tail = Lb - full * PAGE
            pool[block_table[b, full], :tail] = rows[full * PAGE:]
        del rows

    q_nope = f32_to_bf16_bits(rng.standard_normal((Bn, Sqn, Hn, D_C), dtype=np.float32)
                              * np.float32(spec.q_sigma))
    q_rope = f32_to_bf16_bits(rng.standard_normal((Bn, Sqn, Hn, D_R if rope else 0),
                                                  dtype=np.float32)
                              * np.float32(spec.q_sigma))
    sc = DEFAULT_SCALE if scale is None else np.float32(scale)
    return Workload(spec, q_nope, q_rope, pool, block_table, L.astype(np.int32), sc,
                    bool(spec.causal), kv_format, kvs if kv_format == "e4m3" else 1.0)


def kv_bytes_expected(spec: WorkloadSpec) -> float:
    kind = spec.lens[0]
    mean = spec.lens[1] if kind == "fixed" else 0.5 * (spec.lens[1] + spec.lens[2])
    return spec.B * mean * D_ROW * 2


def pages_for(L: int) -> int:
    return int(math.ceil(L / PAGE))


def make_tree_masks(B: int, Sq: int, kind: str = "random", seed: int = 0) -> np.ndarray:
    """Draft trees as ancestor bit masks, uint64 [B, Sq] (Sq <= 64).

    Bit u of mask[b, t] marks draft u as an ancestor of draft t (or t itself).
    Drafts are numbered parents first.  kind: "chain" (draft t's parent is t - 1),
    "star" (every draft hangs off the cached prefix) or "random" (each draft t > 0
    picks its parent uniformly among the prefix and drafts 0 .. t - 1, seeded).
    """
    if not 1 <= Sq <= 64:
        raise ValueError("tree drafts need 1 <= Sq <= 64")
    rng = np.random.default_rng(seed)
    masks = np.zeros((B, Sq), dtype=np.uint64)
    for b in range(B):
        anc = []
        for t in range(Sq):
            if kind == "chain":
                parent = t - 1
            elif kind == "star":
                parent = -1
            elif kind == "random":
                parent = int(rng.integers(-1, t)) if t > 0 else -1
            else:
                raise ValueError(kind)
            m = (1 << t) | (anc[parent] if parent >= 0 else 0)
            anc.append(m)
            masks[b, t] = np.uint64(m)
    return masks
