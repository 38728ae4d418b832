"""Host-side checks of the profile summariser: the LM-head kernel is recognised whatever the
ring's stage count, and only the LM head (role 1, one row tile) is."""
from speculative_decoding_round_amd import profsum


def test_lm_head_pattern_ignores_the_stage_count():
    for nst in (2, 3, 4, 5):
        assert profsum.LM_HEAD_KERNEL.search(f"k_gemm_ring<1, 8, {nst}, false, 1, 1>")
    assert not profsum.LM_HEAD_KERNEL.search("k_gemm_ring<1, 8, 3, false, 2, 4>")    # QKV
    assert not profsum.LM_HEAD_KERNEL.search("k_gemm_ring<1, 8, 3, true, 6, 4>")     # gate/up
    # the wide kernel (33 .. 160 rows): the LM head is role 1 at 16 or 32 tiles per block
    assert profsum.LM_HEAD_KERNEL.search("k_gemm_wide<3, 16, 16, false, 1>")
    assert profsum.LM_HEAD_KERNEL.search("k_gemm_wide<10, 16, 10, false, 1>")
    assert profsum.LM_HEAD_KERNEL.search("k_gemm_wide<3, 32, 17, false, 1>")   # 32 tiles per block
    assert not profsum.LM_HEAD_KERNEL.search("k_gemm_wide<3, 14, 14, true, 6>")
    assert not profsum.LM_HEAD_KERNEL.search("k_gemm_wide<3, 10, 10, false, 0>")


def test_source_hash_tracks_the_sources():
    h = profsum.source_hash(("gemm.hip", "common.h"))
    assert isinstance(h, str) and len(h) == 16
    assert h == profsum.source_hash(("gemm.hip", "common.h"))
    assert h != profsum.source_hash(("attention.hip", "common.h"))
