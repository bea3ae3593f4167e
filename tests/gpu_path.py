"""Helpers for the GPU tests: move seeded inputs to the device, run the HIP path
through the Python binding of the C ABI, and compare with the CPU oracle.

Tolerances (the whole-path bar): block-table and page indexing bit-exact;
o_lat and o within max |d| <= 2e-2 and sum|d| / sum|ref| <= 5e-3 of the oracle;
lse within |d| <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

from mla_inputs import f32

MAX_ABS = 2e-2
L1_REL = 5e-3
LSE_ABS = 1e-3


def say(*a):
    print(*a, flush=True)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    return f32(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


class DevInputs:
    def __init__(self, inp):
        self.inp = inp
        self.kv = to_dev_bf16(inp.kv_cache)
        self.bt = to_dev_i32(inp.block_table)
        self.sl = to_dev_i32(inp.seqlens)
        self.q_nope = to_dev_bf16(inp.q_nope)
        self.q_pe = to_dev_bf16(inp.q_pe)
        self.w_uk = to_dev_bf16(inp.w_uk)
        self.w_uv = to_dev_bf16(inp.w_uv)


def run_path(mla, d: DevInputs, slots=None, lo=True, split_overhead=None):
    """metadata -> absorb_q -> decode_paged -> up_v; returns device tensors."""
    inp = d.inp
    kw = {} if split_overhead is None else dict(split_overhead=split_overhead)
    meta, ns = mla.get_metadata(d.sl, slots, s_q=inp.s_q, h=inp.h, **kw)
    q_lat, q_lo = mla.absorb_q(d.q_nope, d.w_uk, lo=lo)
    o_lat, lse = mla.decode_paged(q_lat, d.q_pe, d.kv, d.bt, d.sl, meta, ns, inp.scale, inp.causal,
                                  q_lat_lo=q_lo)
    o = mla.up_v(o_lat, d.w_uv)
    torch.cuda.synchronize()
    return dict(meta=meta, ns=ns, q_lat=q_lat, q_lo=q_lo, o_lat=o_lat, lse=lse, o=o)


def host(res):
    return dict(o_lat=from_dev_bf16(res["o_lat"]), o=from_dev_bf16(res["o"]), lse=res["lse"].cpu().numpy())


def compare(got, ref, seqs, heads, label=""):
    """Check the whole-path bar on the selected sequences and heads; returns the error stats."""
    stats = {}
    for k in ("o_lat", "o"):
        g = got[k][seqs][:, :, heads].astype(np.float64)
        r = ref[k]
        assert np.isfinite(g).all(), f"{label} {k}: non-finite output"
        d = np.abs(g - r)
        stats[k + "_max_abs"] = float(d.max())
        stats[k + "_l1_rel"] = float(d.sum() / max(np.abs(r).sum(), 1e-30))
    g = got["lse"][seqs][:, :, heads].astype(np.float64)
    r = ref["lse"]
    both_inf = np.isneginf(g) & np.isneginf(r)
    assert (np.isneginf(g) == np.isneginf(r)).all(), f"{label} lse: -inf pattern differs"
    d = np.abs(np.where(both_inf, 0.0, g) - np.where(both_inf, 0.0, r))  # rows with no key: both -inf
    stats["lse_max_abs"] = float(d.max())
    say(label, {k: f"{v:.3e}" for k, v in stats.items()})
    assert stats["o_lat_max_abs"] <= MAX_ABS and stats["o_max_abs"] <= MAX_ABS, (label, stats)
    assert stats["o_lat_l1_rel"] <= L1_REL and stats["o_l1_rel"] <= L1_REL, (label, stats)
    assert stats["lse_max_abs"] <= LSE_ABS, (label, stats)
    return stats
