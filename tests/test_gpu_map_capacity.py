"""GPU parity at the page-map limit. A split of a paged cache (or of a block list) stages its page
(block) ids in LDS: at most 1038 per split on the GQA kernels and 258 on the MLA kernel, plus two
for a split that starts inside a page. Each case below forces splits at that limit, or within a
page of it with split starts inside a page, on each partial kernel form: the vector kernel (8
rows per KV head), the 32-row matrix-core kernel (32 rows), the 16-row kernel (fp8, 4 rows) and
MLA, paged and with block lists. Every result must match the fp64 oracle; the host refuses a
split one page longer (CPU ABI tests)."""
import pytest
import torch

from attention_decode_amd import inputs
from attention_decode_amd.step import DecodeStep
from gpu_util import assert_matches, gpu_available, oracle_of, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def chunk_of(L, S):
    return -(-(-(-L // S)) // 16) * 16


# (id, generator, arguments, forced split count, map limit in pages)
CASES = [
    ("vector_page16_exact", inputs.paged,
     dict(seq_lens=[16 * 1038], num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=16, seed=91), 1, 1038),
    ("vector_page32_inside_pages", inputs.paged,
     dict(seq_lens=[66400, 1000], num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=32, seed=92), 2, 1038),
    ("mfma32_page16_exact", inputs.paged,
     dict(seq_lens=[16 * 1038], num_q_heads=32, num_kv_heads=1, head_dim=128, page_size=16, seed=93), 1, 1038),
    ("mfma16_fp8_page32_inside_pages", inputs.paged,
     dict(seq_lens=[66400], num_q_heads=4, num_kv_heads=1, head_dim=128, page_size=32, seed=94,
          kv_format="fp8"), 2, 1038),
    ("vector_blocklist16_exact", inputs.sparse,
     dict(batch=1, num_q_heads=8, num_kv_heads=1, head_dim=128, kv_len=16 * 2076, q_len=1, block_size=16,
          blocks=list(range(0, 2076, 2)), causal=False, seed=97), 1, 1038),
    ("mfma32_blocklist16_exact", inputs.sparse,
     dict(batch=1, num_q_heads=32, num_kv_heads=1, head_dim=128, kv_len=16 * 2076, q_len=1, block_size=16,
          blocks=list(range(1, 2076, 2)), causal=False, seed=98), 1, 1038),
    ("mla_page16_exact", inputs.mla,
     dict(batch=1, num_heads=16, kv_len=16 * 258, page_size=16, seed=95), 1, 258),
    ("mla_page64_inside_pages", inputs.mla,
     dict(batch=2, num_heads=16, kv_len=32960, seq_lens=[32960, 700], page_size=64, seed=96), 2, 258),
]


@pytest.mark.parametrize("name,gen,kw,S,limit", CASES, ids=[c[0] for c in CASES])
def test_split_at_page_map_limit(orc, name, gen, kw, S, limit):
    w = gen(**kw)
    if w.num_blocks is not None:  # a block list: splits cover listed keys, the map holds block ids
        L, page = int(w.block_idx.shape[-1]) * w.block_size, w.block_size
    else:
        L, page = w.kv_len_max, w.page_size
    chunk = chunk_of(L, S)
    # the most pages any split of this plan touches (a split may start inside a page)
    spans = [((min((s + 1) * chunk, L) - 1) // page) - (s * chunk) // page + 1 for s in range(S) if s * chunk < L]
    say(f"[gpu] {name}: L={L}, S={S}, chunk={chunk}, page={page}, pages per split {spans} (limit {limit} + 2)")
    assert max(spans) >= limit and max(spans) <= limit + 2
    ref_o, ref_l = oracle_of(orc, w)
    step = DecodeStep(w.to("cuda"), num_splits=S)
    assert step.splits == S
    out, lse = step()
    torch.cuda.synchronize()
    assert_matches(out.cpu(), lse.cpu(), ref_o, ref_l, w.dtype, name)
