"""Seeded synthetic inputs for paged MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic. Both the CPU oracle and the GPU path consume what it
produces, so it is the one module the two sides share.

Shapes follow the DeepSeek-V3 dimensions used on the pages: the latent width
d_c = 512 ("DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程", section 2.3),
128 heads of width d_h = 128 (same page, section 2.3; the SC11 note splits the
128 up-projection heads into 32 per card), and a bf16 paged cache with 64-token
blocks (FlashMLA release news, feature list). Each cached token is one 576-wide
row: 512 latent values followed by 64 decoupled-RoPE key values (the pages'
decoupled-RoPE section 3.1 adds a positional key part next to the content part).

All floating-point inputs are stored as bf16 bit patterns (uint16), rounded
from float32 draws to nearest-even. ``f32`` views decode those bits exactly.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 64          # tokens per page
D_LATENT = 512     # d_c: latent width, also the value width dv
D_ROPE = 64        # decoupled RoPE key width
D_ROW = D_LATENT + D_ROPE  # 576 bf16 per cached token
D_NOPE = 128       # d_h: per-head content width of q and of the expanded k/v
SOFTMAX_SCALE = 1.0 / math.sqrt(D_NOPE + D_ROPE)  # 1/sqrt(192)

BF16_NAN = np.uint16(0x7FC0)

# Workloads. ``seqlens`` is a recipe:
#   ("list", [...])                      fixed lengths
#   ("all", L)                           every sequence has length L
#   ("uniform", lo, hi)                  integers uniform on [lo, hi]
#   ("lognormal", median, sigma, lo, hi) rint(lognormal(ln median, sigma)) clipped
CONFIGS: dict[str, dict] = {
    # tiny parity case: batch 2, 16 heads, lengths {37, 100}
    "tiny": dict(b=2, h=16, s_q=1, causal=False, seqlens=("list", [37, 100])),
    # one tensor-parallel share of the SC11 deployment: 32 of 128 heads,
    # batch 128 x sequence 512 (the double-buffer measurement's shape)
    "tp_share": dict(b=128, h=32, s_q=1, causal=False, seqlens=("all", 512)),
    # all 128 heads on one GPU, lengths uniform in [256, 4096]
    "full_heads": dict(b=128, h=128, s_q=1, causal=False, seqlens=("uniform", 256, 4096)),
    # long, variable context: batch 16, lognormal lengths with median 8192
    "long_context": dict(b=16, h=128, s_q=1, causal=False,
                         seqlens=("lognormal", 8192, 1.0, 1, 65536)),
    # two query tokens per sequence under a causal mask (speculative verify)
    "multi_token": dict(b=128, h=128, s_q=2, causal=True, seqlens=("all", 4096)),
    # speculative verify with a longer draft: 8 query tokens per sequence
    # (1024 query rows), causal, lengths uniform in [256, 4096]
    "spec_verify": dict(b=32, h=128, s_q=8, causal=True, seqlens=("uniform", 256, 4096)),
}
CONFIG_ORDER = ["tiny", "tp_share", "full_heads", "long_context", "multi_token", "spec_verify"]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        bias = np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        flat_o[s:s + step] = ((c + bias) >> np.uint32(16)).astype(np.uint16)
    return out


def f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        k = min(step, n - s)
        v = rng.standard_normal(k, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[s:s + k] = bf16_bits(v)
    return out.reshape(shape)


def draw_seqlens(rng: np.random.Generator, b: int, recipe) -> np.ndarray:
    kind = recipe[0]
    if kind == "list":
        L = np.asarray(recipe[1], dtype=np.int64)
        assert L.size == b
    elif kind == "all":
        L = np.full(b, recipe[1], dtype=np.int64)
    elif kind == "uniform":
        L = rng.integers(recipe[1], recipe[2] + 1, size=b, dtype=np.int64)
    elif kind == "lognormal":
        median, sigma, lo, hi = recipe[1:]
        L = np.clip(np.rint(rng.lognormal(math.log(median), sigma, size=b)), lo, hi).astype(np.int64)
    else:
        raise ValueError(f"unknown seqlen recipe {recipe!r}")
    return L.astype(np.int32)


@dataclass
class MLAInputs:
    name: str
    b: int
    h: int
    s_q: int
    causal: bool
    scale: float
    seqlens: np.ndarray        # int32 [b]
    block_table: np.ndarray    # int32 [b, max_blocks]
    kv_cache: np.ndarray       # bf16 bits [num_pages, PAGE, D_ROW]
    q_nope: np.ndarray         # bf16 bits [b, s_q, h, D_NOPE]
    q_pe: np.ndarray           # bf16 bits [b, s_q, h, D_ROPE]
    w_uk: np.ndarray           # bf16 bits [h, D_NOPE, D_LATENT]
    w_uv: np.ndarray           # bf16 bits [h, D_LATENT, D_NOPE]
    trap_pages: list = field(default_factory=list)

    @property
    def num_pages(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def rows(self) -> int:
        """Query rows per sequence that share one KV stream: s_q * h."""
        return self.s_q * self.h


def make_inputs(config, seed: int = 0, *, trap: bool = False, seqlens=None,
                b: int | None = None, h: int | None = None, s_q: int | None = None,
                causal: bool | None = None) -> MLAInputs:
    """Draw one workload.

    ``config`` is a name from CONFIGS or a dict of the same form. The draws use
    one ``np.random.default_rng(seed)`` in this fixed order: sequence lengths,
    page permutation, kv cache, q_nope, q_pe, W_UK, W_UV.

    The block table maps each sequence's logical pages, in order, onto a random
    permutation of all physical pages. With ``trap=True`` two extra physical
    pages filled with NaN are appended, every unused block-table entry points
    at one of them, and the cache slots past each sequence's length in its last
    page are set to NaN: a correct kernel never lets any of these reach a result.
    Without ``trap``, unused entries are 0 and page tails hold ordinary draws.
    """
    if isinstance(config, str):
        name = config
        cfg = dict(CONFIGS[config])
    else:
        cfg = dict(config)
        name = cfg.pop("name", "custom")
    if b is not None:
        cfg["b"] = b
    if h is not None:
        cfg["h"] = h
    if s_q is not None:
        cfg["s_q"] = s_q
    if causal is not None:
        cfg["causal"] = causal
    if seqlens is not None:
        cfg["seqlens"] = ("list", list(seqlens))
        cfg["b"] = len(seqlens)
    B, H, SQ = cfg["b"], cfg["h"], cfg["s_q"]
    rng = np.random.default_rng(seed)
    L = draw_seqlens(rng, B, cfg["seqlens"])
    pages = (L.astype(np.int64) + PAGE - 1) // PAGE
    pages[L <= 0] = 0
    P = int(pages.sum())
    perm = rng.permutation(P).astype(np.int32) if P > 0 else np.zeros(0, np.int32)
    max_blocks = max(1, int(pages.max()) if B > 0 else 1)
    n_trap = 2 if trap else 0
    num_pages = P + n_trap
    trap_ids = list(range(P, P + n_trap))
    fill = trap_ids[0] if trap else 0
    bt = np.full((B, max_blocks), fill, dtype=np.int32)
    off = 0
    for i in range(B):
        n = int(pages[i])
        bt[i, :n] = perm[off:off + n]
        off += n
    if trap and B > 0:
        # alternate the two trap pages over unused entries
        for i in range(B):
            for j in range(int(pages[i]), max_blocks):
                bt[i, j] = trap_ids[(i + j) % 2]
    kv = _normal_bf16(rng, (max(num_pages, 1), PAGE, D_ROW))
    if num_pages == 0:
        kv = kv[:0]
    q_nope = _normal_bf16(rng, (B, SQ, H, D_NOPE))
    q_pe = _normal_bf16(rng, (B, SQ, H, D_ROPE))
    wstd = math.sqrt(1.0 / D_LATENT)  # variance 1/512
    w_uk = _normal_bf16(rng, (H, D_NOPE, D_LATENT), wstd)
    w_uv = _normal_bf16(rng, (H, D_LATENT, D_NOPE), wstd)
    if trap:
        kv[P:] = BF16_NAN
        for i in range(B):
            n = int(pages[i])
            if n > 0:
                tail = int(L[i]) - (n - 1) * PAGE
                if tail < PAGE:
                    kv[bt[i, n - 1], tail:, :] = BF16_NAN
    return MLAInputs(name=name, b=B, h=H, s_q=SQ, causal=bool(cfg.get("causal", False)),
                     scale=SOFTMAX_SCALE, seqlens=L, block_table=bt, kv_cache=kv,
                     q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, trap_pages=trap_ids)


def make_new_rows(inp: MLAInputs, seed: int) -> np.ndarray:
    """The step's new cache rows for ``inp``: bf16 bits [b, s_q, 576], N(0, 1) like the cache
    (latent values then the rotated positional key), from their own generator."""
    rng = np.random.default_rng([seed, 0x6e657752])
    return _normal_bf16(rng, (inp.b, inp.s_q, D_ROW))


def repage(inp: MLAInputs, seed: int) -> MLAInputs:
    """Same logical cache, different physical page placement.

    Physical page p moves to slot perm[p] and every block-table entry follows
    it, so every sequence still reads the same token rows in the same order.
    """
    rng = np.random.default_rng(seed)
    P = inp.num_pages
    perm = rng.permutation(P).astype(np.int32)
    kv = np.empty_like(inp.kv_cache)
    kv[perm] = inp.kv_cache
    bt = perm[inp.block_table]
    return MLAInputs(name=inp.name, b=inp.b, h=inp.h, s_q=inp.s_q, causal=inp.causal,
                     scale=inp.scale, seqlens=inp.seqlens.copy(), block_table=bt, kv_cache=kv,
                     q_nope=inp.q_nope, q_pe=inp.q_pe, w_uk=inp.w_uk, w_uv=inp.w_uv,
                     trap_pages=[int(perm[t]) for t in inp.trap_pages])
