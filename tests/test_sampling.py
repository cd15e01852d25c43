"""Host logic of the GPU parity sampling (CPU): the sampled rows include both
sides of every seam the forward kernel's tiles and waves have."""
import numpy as np
import pytest

from gpu_util import sample_rows, seam_tokens, tile_rows


def test_seam_tokens_cover_tile_edges():
    # 8-wave tiles of 256 rows at G = 4: 64 tokens per tile, 8 per wave
    ts = seam_tokens(65536, 4, 256)
    assert {0, 1, 7, 8, 9, 63, 64, 65, 32767, 32768, 32769, 65471, 65472, 65473, 65535} <= ts
    # G = 3: 85 tokens per tile; the last tile of T = 20000 starts at 19975 (ragged)
    ts = seam_tokens(20000, 3, 256)
    assert {84, 85, 86, 19974, 19975, 19976, 19914, 19915, 19916} <= ts
    assert all(0 <= t < 20000 for t in ts)
    # tiny T: nothing out of range
    assert seam_tokens(3, 8, 128) <= {0, 1, 2}


def test_tile_rows_of_variants():
    assert tile_rows("mfma_bf16_d128_w8") == 256
    assert tile_rows("mfma_bf16_d128_w4") == 128
    assert tile_rows("mfma_bf16_d128_ks") == 128
    assert tile_rows("mfma_f32_d64") == 128
    assert tile_rows("mfma_bf16_d32") == 128
    with pytest.raises(ValueError):
        tile_rows("generic")


def test_sample_rows_per_head():
    cfg = dict(B=2, Hq=8, Hkv=2, T=5000, L=3, d=128)
    rows = sample_rows(cfg, n_random=10, seed=3, rows_per_tile=128)
    seams = seam_tokens(5000, 4, 128)
    for b in range(2):
        for h in range(8):
            got = set(int(t) for t in rows[(rows[:, 0] == b) & (rows[:, 1] == h)][:, 2])
            assert seams <= got
    assert rows.dtype == np.int64 and rows.shape[1] == 3
