"""Workload constants against the dimensions the pages state (tests/golden/page_facts.txt)."""
import os

import mla_inputs as I


def _facts():
    out = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split()
                out[k] = v
    return out


def test_dimensions_match_pages():
    f = _facts()
    assert I.D_LATENT == int(f["d_c"])
    assert I.D_NOPE == int(f["d_h"])
    assert I.PAGE == int(f["page_tokens"])
    assert I.CONFIGS["full_heads"]["h"] == int(f["heads"])
    assert I.CONFIGS["tp_share"]["h"] == int(f["heads_per_card"])
    assert I.CONFIGS["tp_share"]["b"] == int(f["batch_double_buffer"])
    assert I.CONFIGS["tp_share"]["seqlens"] == ("all", int(f["seq_double_buffer"]))
    assert f["cache_dtype"] == "bf16"


def test_generator_layout():
    inp = I.make_inputs("tiny", seed=0, trap=True)
    assert inp.kv_cache.shape[1:] == (I.PAGE, I.D_ROW) and inp.kv_cache.dtype.name == "uint16"
    assert inp.block_table.dtype.name == "int32" and inp.seqlens.tolist() == [37, 100]
    # unused entries point at trap pages; tails are NaN
    assert set(inp.block_table[0, 1:].tolist()) <= set(inp.trap_pages)
    import numpy as np
    last = inp.block_table[0, 0]
    assert np.isnan(I.f32(inp.kv_cache[last, 37:])).all()
    assert not np.isnan(I.f32(inp.kv_cache[last, :37])).any()
    # bf16 rounding is round-to-nearest-even
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(I.bf16_bits(x), ref)
