"""An e4m3 cache with one scale per (layer, block, head) taken from each
appended chunk (FP8_E4M3_BLOCK) against the CPU oracle.

Bars: the scale table and the codes an append writes are bit-exact against
the oracle's rule (oracle.block_scales: fp32 max |x| / 448) and e4m3
quantiser; attention is held to the oracle run on exactly what the cache
holds (the current chunk quantised by the same rule with its own scales),
and to the oracle on the unquantised seeded inputs: at the Matrix-Game size
at 5e-2 (the bar for 8-bit K/V), on small shapes at the quantisation's own error
plus the kernel's bar (bca_harness.assert_fp8).
"""
import math

import numpy as np
import pytest

import oracle
from bca_harness import Sequence, assert_fp8, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def new_cache(L, H, d, n, S, R=False):
    import attention_bca_attend_amd as bca
    return bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype="fp8_block")


def test_block_append_scales_and_codes_exact():
    H, d, n, S = 4, 128, 81, 3
    cache = new_cache(2, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, "fp8_block", seed_layer=41, outlier_frac=0.01)
    appended = []
    _, rk, rv = seq.chunk(70_000)
    seq.append(1, 0, rk, rv, is_ref=True)
    appended.append((S, rk, rv))
    for t in range(5):
        _, k, v = seq.chunk(t)
        if t == 2:
            k = k * np.float32(0.25)  # a block with a smaller range than its neighbours
        seq.append(1, t, k, v)
        appended.append((t % S, k, v))
    torch.cuda.synchronize()
    K, V = cache.blocks(1)
    KS, VS = cache.block_scales(1)
    latest = {}
    for blk, k, v in appended:
        latest[blk] = (k, v)  # later appends overwrite the slot
    for blk, (k, v) in latest.items():
        for x, codes, scales in ((k, K, KS), (v, V, VS)):
            want_s = oracle.block_scales(x)
            got_s = scales[blk].cpu().numpy()
            assert np.array_equal(got_s, want_s), (blk, got_s, want_s)
            got = codes[:, blk].cpu().numpy()  # [H][n][d]
            for h in range(H):
                want = oracle.quant_e4m3(x[:, h, :], float(want_s[h]))
                assert np.array_equal(got[h], want), (blk, h)
    log("fp8 block: scale table and codes bit-exact for every block")


@pytest.mark.parametrize("G,outliers", [(0, True), (1, True), (3, True), (0, False)])
def test_block_sequence(G, outliers):
    H, d, n, S, W = 4, 128, 100, 3, 2
    cache = new_cache(1, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, "fp8_block", seed_layer=42 if outliers else 45,
                   outlier_frac=0.01 if outliers else 0.0)
    _, rk, rv = seq.chunk(80_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(1, 7):
        q, k, v = seq.chunk(t)
        if t == 3:
            k, v = k * np.float32(0.5), v * np.float32(4.0)  # blocks of different ranges
        use_ref = t % 2 == 0
        o, lse, _ = seq.attend(0, t, q, k, v, W, use_ref=use_ref, G=G)
        assert_fp8(seq, o, lse, t, q, k, v, W, use_ref=use_ref, what=f"fp8 block G={G} t={t}")
        seq.append(0, t, k, v)


def test_block_ragged_and_small_chunks():
    # chunks shorter than one key tile and chunks that end mid-tile
    for n in (17, 64, 130):
        H, d, S, W = 2, 128, 2, 2
        cache = new_cache(1, H, d, n, S)
        seq = Sequence(cache, H, d, n, "fp8_block", seed_layer=43 + n, outlier_frac=0.01)
        for t in range(4):
            q, k, v = seq.chunk(t)
            o, lse, _ = seq.attend(0, t, q, k, v, W)
            assert_fp8(seq, o, lse, t, q, k, v, W, what=f"fp8 block n={n} t={t}")
            seq.append(0, t, k, v)


def test_block_full_size_matrix_game_shape():
    # 24 heads x 405 tokens, reference + 20 ring chunks + current, 4 segments,
    # 1% outliers of 8 sigma
    H, d, n, S, W = 24, 128, 405, 20, 20
    cache = new_cache(1, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, "fp8_block", seed_layer=44, outlier_frac=0.01)
    _, rk, rv = seq.chunk(110_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(5, 25):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(25)
    plan = cache.plan(0, cache.spec(25, W, use_ref=True, num_segments=4))
    assert plan["kv_tiles"] == 22 * math.ceil(n / 64), plan  # every block padded to whole tiles
    log("fp8 block full size: oracle ...")
    for G in (4, 0):
        o, lse, _ = seq.attend(0, 25, q, k, v, W, use_ref=True, G=G)
        # Every block's largest value is an 8-sigma outlier, so the per-block
        # scales equal the per-head ones and the codes are those of the e4m3
        # workload; on these seeded inputs e4m3 alone moves O by 6.7e-2
        # against the raw values (4.6e-2 on the e4m3 workload's seeds): the
        # raw bar is that quantisation error plus the kernel's.
        assert_fp8(seq, o, lse, 25, q, k, v, W, use_ref=True, what=f"fp8 block full size G={G}")


def test_block_refused_calls():
    import attention_bca_attend_amd as bca
    cache = new_cache(1, 2, 128, 32, 2)
    with pytest.raises(bca.BcaError) as e:
        cache.set_kv_scales(0, [1.0, 1.0], [1.0, 1.0])
    assert e.value.status == -4
    _, k, v = Sequence(cache, 2, 128, 32, "fp8_block").chunk(0)
    kf, vf = to_dev(k, "fp32"), to_dev(v, "fp32")
    with pytest.raises(bca.BcaError) as e:  # only bf16 inputs are quantised into it
        bca.bca_append_chunk(cache.handle, 0, 0, 0, kf.data_ptr(), vf.data_ptr(), bca.F32, 0)
    assert e.value.status == -4
