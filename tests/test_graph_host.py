"""Host logic of the graph-captured decode step: length buckets."""
from token_level_sparse_hs_amd.graph import length_bucket


def test_length_bucket():
    assert length_bucket(1) == 4096
    assert length_bucket(4096) == 4096
    assert length_bucket(4097) == 8192
    assert length_bucket(65536) == 65536
    assert length_bucket(65537) == 65536 + 8192
    assert length_bucket(262144 + 32) == 262144 + 32768
    for L in [5, 4095, 4097, 30000, 65537, 100000, 262176, 1064976, 1 << 21]:
        b = length_bucket(L)
        assert b >= L
        assert b - L < max(4096, b // 8)  # at most 1/8 of an octave above
