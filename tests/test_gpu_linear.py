"""GPU parity of eagle3_linear (the drafter projections' GEMM kernels) against the oracle's
float64 projection, through the C-ABI: the LDS-ring kernel (M <= 32, with and without split-K
partial sums), the wide kernel (33 .. 160 rows, four waves splitting the rows over a shared W
ring; also whole and split k-ranges, ragged rows, a ragged last k-block and a ragged last
n-block), the register-stationary kernel (K not a multiple of 32), and the tiled matrix-core kernel
(M > 160, including ragged M and N, whole and split k-ranges), at fp32 and bf16.  Full-size
shapes are checked on sampled rows."""
import numpy as np
import pytest
import torch

from oracle import eagle3_oracle as O
from speculative_decoding_round_amd import capi, synth
from tests.gpu_util import TOL, need_gpu, np32, rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF, F32 = torch.bfloat16, torch.float32


@pytest.mark.parametrize("M,N,K,dt,rows", [
    (1, 6144, 8192, BF, None),      # ring, one row (QKV shape)
    (10, 4096, 4096, BF, None),     # ring, two waves, split-K partials summed
    (32, 2048, 1024, BF, None),     # ring, two row tiles
    (4, 10240, 16384, BF, None),    # ring, 80 n-blocks: four-wave workgroups, three k-splits
    (40, 4096, 4096, BF, None),     # wide kernel, three row tiles (wave 3 holds none)
    (160, 1024, 4096, BF, None),    # wide kernel, ten row tiles
    (96, 2048, 4096, BF, None),     # wide: six row tiles
    (97, 1000, 1056, BF, None),     # wide: one row past six tiles, ragged n-block, 33 chunks
    (150, 4104, 2080, BF, None),    # wide: ragged rows, n-block and last k-block (65 chunks)
    (33, 1000, 1056, BF, None),     # wide: one row past two tiles, ragged n-block, 33 chunks
    (48, 4096, 8192, BF, None),     # wide: three full row tiles, k split
    (64, 2048, 2304, BF, None),     # wide: four row tiles (one per wave)
    (100, 3072, 4096, BF, None),    # wide: seven row tiles (waves hold 2, 2, 2, 1)
    (128, 4096, 14336, BF, None),   # wide: eight row tiles at the MLP-down shape
    (40, 10240, 16384, BF, 12),     # wide at the 70B-shaped QKV projection
    (40, 128256, 8192, BF, 6),      # wide at the 70B-shaped LM head (one k-range, 501 n-blocks)
    (160, 128256, 4096, BF, 10),    # wide at the batched LM head (ten row tiles)
    (40, 1024, 1000, BF, None),     # register-stationary kernel (K not a multiple of 32)
    (10, 256, 768, F32, None),      # fp32 path
    (256, 1024, 1024, BF, None),    # tiled kernel, one row tile, k split in eight
    (200, 768, 1024, BF, None),     # tiled kernel, fewer rows than one tile
    (300, 1000, 512, BF, None),     # tiled kernel, ragged M and N
    (2048, 6144, 8192, BF, 64),     # tiled kernel at the QKV shape of a 2048-token prompt
    (1024, 6144, 8192, BF, 32),     # the same with 1024 rows: k split in two
    (1024, 4096, 14336, BF, 32),    # tiled kernel at the MLP-down shape
], ids=["ring_m1", "ring_m10_split", "ring_m32", "ring_m4_80_nblocks", "wide_m40", "wide_m160", "wide_m96",
        "wide_m97_ragged", "wide_m150_ragged_split", "wide_m33_ragged",
        "wide_m48_split", "wide_m64", "wide_m100", "wide_m128_down", "wide_qkv_70b", "wide_lm_70b",
        "wide_lm_batch16", "regs_m40_k1000", "fp32_m10", "tile_m256",
        "tile_m200", "tile_ragged", "tile_qkv_2048", "tile_qkv_1024_split", "tile_down_1024"])
def test_linear_matches_oracle(M, N, K, dt, rows):
    need_gpu()
    x = synth.normal((M, K), 1.0, 11 + M, dt, DEV)
    w = synth.normal((N, K), K ** -0.5, 12 + N, dt, DEV)
    y = capi.eagle3_linear(x, w)
    torch.cuda.synchronize()
    sel = np.arange(M) if rows is None else np.random.default_rng(M).choice(M, rows, replace=False)
    ref = O.project(x[torch.as_tensor(sel, device=DEV)].cpu(), w.cpu())
    got = np32(y)[sel]
    assert np.all(np.isfinite(got))
    assert rel_err(got, ref) <= TOL[dt]
    if rows is not None:   # every row written (the sampled check covers values)
        assert torch.isfinite(y).all()


def test_linear_reuses_output_and_strided_rows():
    """X given as every other row of a larger buffer (row stride 2K), two calls into the same
    output: the second overwrites the first completely."""
    need_gpu()
    M, N, K = 300, 512, 256
    big = synth.normal((2 * M, K), 1.0, 3, BF, DEV)
    x = big.view(M, 2 * K)[:, :K]
    w = synth.normal((N, K), K ** -0.5, 4, BF, DEV)
    out = torch.full((M, N), float("nan"), dtype=F32, device=DEV)
    capi.eagle3_linear(x, w, out=out)
    w2 = synth.normal((N, K), K ** -0.5, 5, BF, DEV)
    capi.eagle3_linear(x, w2, out=out)
    torch.cuda.synchronize()
    ref = O.project(x.cpu(), w2.cpu())
    assert rel_err(np32(out), ref) <= TOL[BF]


def test_linear_split_k_is_deterministic():
    """The split-k partial sums are added in split order: two calls agree bit for bit."""
    need_gpu()
    M, N, K = 512, 1024, 2048
    x = synth.normal((M, K), 1.0, 21, BF, DEV)
    w = synth.normal((N, K), K ** -0.5, 22, BF, DEV)
    assert capi.lib().eagle3_linear_workspace_size(M, N, K, capi.EAGLE3_BF16) > 0
    a = capi.eagle3_linear(x, w)
    b = capi.eagle3_linear(x, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("M", [48, 160], ids=["three_tiles", "ten_tiles"])
def test_wide_split_k_is_deterministic(M):
    """The wide kernel's k-split partial sums are added in split order: two calls agree bit for
    bit (48 and 160 rows at the 8B QKV shape, whose plans split the k-range)."""
    need_gpu()
    N, K = 6144, 8192
    assert capi.lib().eagle3_linear_workspace_size(M, N, K, capi.EAGLE3_BF16) > 0
    x = synth.normal((M, K), 1.0, 31, BF, DEV)
    w = synth.normal((N, K), K ** -0.5, 32, BF, DEV)
    a = capi.eagle3_linear(x, w)
    b = capi.eagle3_linear(x, w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    sel = np.array([0, 17, 40, M - 1])
    ref = O.project(x[torch.as_tensor(sel, device=DEV)].cpu(), w.cpu())
    assert rel_err(np32(a)[sel], ref) <= TOL[BF]
