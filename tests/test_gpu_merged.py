"""GPU: pkv_decode_attention_merged (decode and merge of a whole history in
one call) against pkv_decode_attention followed by pkv_merge_partials, bit
for bit, in its three forms (tiles that are splits; the tile finalize and
the final merge as one launch; more than 64 splits per row, two launches),
and against the float64 oracle."""

import pytest

from paged_kv_cache_10_amd import inputs as I
from gpu_helpers import Case, check_layer, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ragged(gpu):
    w = I.Workload("ragged", seed=11, ctx_lens=[1, 63, 64, 65, 1000, 2049, 0, 4097],
                   num_layers=1, tile_tokens=1024)
    return Case(w, fill=I.BF16_QNAN)


@pytest.fixture(scope="module")
def long_rows(gpu):
    # 9,000 tokens in 64-token splits: 141 splits per row, past one launch's 64
    w = I.Workload("long_rows", seed=12, ctx_lens=[9000, 300], num_layers=1, tile_tokens=128)
    return Case(w, fill=I.BF16_QNAN)


@pytest.mark.parametrize("tile,split", [(1024, 1024), (1024, 256), (4096, 1024), (128, 64)])
def test_merged_equals_decode_then_merge_bitwise(ragged, tile, split):
    sep = ragged.decode(0, tile=tile, split=split)
    got = ragged.decode_merged(0, tile=tile, split=split)
    for x, y in zip(sep, got):
        assert same_bits(x, y)
    check_layer(ragged, 0, got, ragged.oracle_layer(0, tile=tile))


def test_merged_beyond_one_launch_of_tiles(long_rows):
    sep = long_rows.decode(0, tile=128, split=64)
    got = long_rows.decode_merged(0, tile=128, split=64)
    for x, y in zip(sep, got):
        assert same_bits(x, y)
    check_layer(long_rows, 0, got, long_rows.oracle_layer(0, tile=128))
