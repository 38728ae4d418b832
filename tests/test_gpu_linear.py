"""GPU parity of eagle3_linear (the drafter projections' GEMM kernels) against the oracle's
float64 projection, through the C-ABI: the LDS-ring kernel (M <= 32, with and without split-K
partial sums), the register-stationary kernel (M up to 160), and the tiled matrix-core kernel
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
    (40, 4096, 4096, BF, None),     # register-stationary kernel
    (160, 1024, 4096, BF, None),    # register-stationary kernel, ten row tiles
    (10, 256, 768, F32, None),      # fp32 path
    (256, 1024, 1024, BF, None),    # tiled kernel, one row tile, k split in eight
    (200, 768, 1024, BF, None),     # tiled kernel, fewer rows than one tile
    (300, 1000, 512, BF, None),     # tiled kernel, ragged M and N
    (2048, 6144, 8192, BF, 64),     # tiled kernel at the QKV shape of a 2048-token prompt
    (1024, 6144, 8192, BF, 32),     # the same with 1024 rows: k split in two
    (1024, 4096, 14336, BF, 32),    # tiled kernel at the MLP-down shape
], ids=["ring_m1", "ring_m10_split", "ring_m32", "regs_m40", "regs_m160", "fp32_m10", "tile_m256",
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
