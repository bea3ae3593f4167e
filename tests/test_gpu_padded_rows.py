"""Row counts that leave query-row slots of a workgroup empty.

The 128-row decode kernel gives each of its four waves 32 query rows of one
sequence, M = s_q * h rows in all, in ceil(M / 128) row blocks. Where M is not
a multiple of 128 the last row block holds fewer than 128 rows, so some waves
hold only padding rows (for example h = 32 heads with s_q = 3 draft tokens:
96 rows, the fourth wave empty). The speculative-verify usage on the pages
scores several draft tokens per sequence against the same cache
("DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程", section 6.3), and the
FlashMLA usage example plans with s_q * h_q / h_kv rows per KV head, so these
shapes are part of the call's contract. Every output element is compared with
the CPU oracle, with NaN trap pages behind unused block-table entries and NaN
page tails, in one whole piece per slot and in many split pieces.
"""
import pytest

from gpu_path import DevInputs, compare, host, run_path, say
from mla_inputs import make_inputs
from oracle import mla_oracle as O

pytestmark = pytest.mark.gpu

# (h, s_q): M = 96, 80, 112 (one partly empty row block) and 192, 160, 448
# (several row blocks, the last one partly empty)
PADDED = [(32, 3), (16, 5), (16, 7), (64, 3), (32, 5), (64, 7)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("h,s_q", PADDED)
def test_padded_row_blocks(gpu_lib, h, s_q, causal):
    # lengths: shorter than the draft (causal rows with no key), a ragged
    # first page, several pages with a ragged tail, and a longer sequence
    seqlens = [2, 5, 77, 640, 1100]
    inp = make_inputs("tiny", seed=40 + h + s_q, seqlens=seqlens, s_q=s_q, h=h, causal=causal, trap=True)
    ref = O.decode_naive_inputs(inp)
    d = DevInputs(inp)
    for slots in (1, 7, 300):
        say("padded rows: h", h, "s_q", s_q, "M", h * s_q, "causal", causal, "slots", slots)
        res = host(run_path(gpu_lib, d, slots=slots))
        compare(res, ref, list(range(inp.b)), list(range(inp.h)), label=f"h={h} s_q={s_q} slots={slots}")
        assert gpu_lib.take_device_error() == 0
