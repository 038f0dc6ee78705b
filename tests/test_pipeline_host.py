"""Host logic of the pipelined prefill: the chunk schedule (no GPU)."""
import pytest

import sparse_memory_linear_pkm_amd as sdm


@pytest.mark.parametrize("T", [0, 1, 511, 16384, 16385, 100000, 1 << 20, 3_000_001])
def test_prefill_chunks_cover_the_sequence(T):
    c = sdm.prefill_chunks(T)
    assert sum(c) == T
    assert all(n > 0 for n in c)
    # every chunk but the last is a multiple of 512, at most 131,072 tokens,
    # and at most 1.5 times the one before it
    assert all(n % 512 == 0 and n <= 131072 for n in c[:-1])
    assert all(b <= 1.5 * a for a, b in zip(c, c[1:]))
    if T:
        assert c[0] == min(T, 16384)


def test_prefill_chunks_long_context_schedule():
    assert sdm.prefill_chunks(1 << 20) == [16384, 24576, 36864, 55296, 82944, 124416, 131072, 131072, 131072,
                                           131072, 131072, 52736]


def test_prefill_chunks_rejects_bad_parameters():
    with pytest.raises(ValueError):
        sdm.prefill_chunks(-1)
    with pytest.raises(ValueError):
        sdm.prefill_chunks(10, first=100, cap=50)
