"""The INT8-K / FP8-V cache with one scale per (layer, block, head) taken
from each appended chunk (INT8K_FP8V_BLOCK; Matrix-Game 4.0 summary,
technical novelty: each KV interval holds INT8 K and FP8 V and only the
changed interval is re-quantised) against the CPU oracle.

Bars: the scale table and the codes an append writes are bit-exact against
the oracle's rule (oracle.block_scales: fp32 max |x| / 127 for K, / 448 for
V) and its int8 and e4m3 quantisers; attention is held to the oracle run on
exactly what the cache holds (the current chunk quantised by the same rule
with its own scales), and to the oracle on the unquantised seeded inputs: at
the Matrix-Game size at 5e-2 (the bar for 8-bit K/V), on small shapes at the
quantisation's own error plus the kernel's bar (bca_harness.assert_fp8).
"""
import math

import numpy as np
import pytest

import oracle
from bca_harness import TOL, Sequence, assert_fp8, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KIND = "int8k_block"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def new_cache(L, H, d, n, S, R=False):
    import attention_bca_attend_amd as bca
    return bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=KIND)


def test_int8k_append_scales_and_codes_exact():
    H, d, n, S = 4, 128, 81, 3
    cache = new_cache(2, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, KIND, seed_layer=141, outlier_frac=0.01)
    appended = []
    _, rk, rv = seq.chunk(70_000)
    seq.append(1, 0, rk, rv, is_ref=True)
    appended.append((S, rk, rv))
    for t in range(5):
        _, k, v = seq.chunk(t)
        if t == 2:
            k = k * np.float32(0.25)  # a block with a smaller range than its neighbours
        if t == 3:
            k = k.copy()
            k[5, 1, 7] = np.float32(np.nan)  # NaN: code 0, and the head's scale is 1
        seq.append(1, t, k, v)
        appended.append((t % S, k, v))
    torch.cuda.synchronize()
    K, V = cache.blocks(1)
    KS, VS = cache.block_scales(1)
    latest = {}
    for blk, k, v in appended:
        latest[blk] = (k, v)  # later appends overwrite the slot
    for blk, (k, v) in latest.items():
        ks, vs = oracle.block_scales(k, qmax=127.0), oracle.block_scales(v)
        assert np.array_equal(KS[blk].cpu().numpy(), ks), (blk, KS[blk], ks)
        assert np.array_equal(VS[blk].cpu().numpy(), vs), (blk, VS[blk], vs)
        gk = K[:, blk].cpu().numpy().view(np.int8)  # [H][n][d]
        gv = V[:, blk].cpu().numpy()
        for h in range(H):
            assert np.array_equal(gk[h], oracle.quant_int8(k[:, h, :], float(ks[h]))), (blk, h)
            assert np.array_equal(gv[h], oracle.quant_e4m3(v[:, h, :], float(vs[h]))), (blk, h)
    log("int8 K / e4m3 V: scale table and codes bit-exact for every block")


@pytest.mark.parametrize("G,outliers", [(0, True), (1, True), (3, True), (0, False)])
def test_int8k_sequence(G, outliers):
    H, d, n, S, W = 4, 128, 100, 3, 2
    cache = new_cache(1, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, KIND, seed_layer=142 if outliers else 145,
                   outlier_frac=0.01 if outliers else 0.0)
    _, rk, rv = seq.chunk(80_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(1, 7):
        q, k, v = seq.chunk(t)
        if t == 3:
            k, v = k * np.float32(0.5), v * np.float32(4.0)  # blocks of different ranges
        use_ref = t % 2 == 0
        o, lse, _ = seq.attend(0, t, q, k, v, W, use_ref=use_ref, G=G)
        assert_fp8(seq, o, lse, t, q, k, v, W, use_ref=use_ref, what=f"int8k G={G} t={t}")
        seq.append(0, t, k, v)


def test_int8k_ragged_and_small_chunks():
    # chunks shorter than one key tile and chunks that end mid-tile
    for n in (17, 64, 130):
        H, d, S, W = 2, 128, 2, 2
        cache = new_cache(1, H, d, n, S)
        seq = Sequence(cache, H, d, n, KIND, seed_layer=143 + n, outlier_frac=0.01)
        for t in range(4):
            q, k, v = seq.chunk(t)
            o, lse, _ = seq.attend(0, t, q, k, v, W)
            assert_fp8(seq, o, lse, t, q, k, v, W, what=f"int8k n={n} t={t}")
            seq.append(0, t, k, v)


@pytest.mark.parametrize("seed", [4, 44])
def test_int8k_full_size_matrix_game_shape(seed):
    """24 heads x 405 tokens, reference + 20 ring chunks + current, 4 segments
    and the automatic split, 1% outliers of 8 sigma: the seeded inputs of the
    e4m3 workload (seed 4) and of the block-scaled e4m3 test (seed 44), held
    to 5e-2 (the bar for 8-bit K/V) against the unquantised inputs."""
    H, d, n, S, W = 24, 128, 405, 20, 20
    cache = new_cache(1, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, KIND, seed_layer=seed, outlier_frac=0.01)
    _, rk, rv = seq.chunk(100_000 if seed == 4 else 110_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(5, 25):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(25)
    plan = cache.plan(0, cache.spec(25, W, use_ref=True, num_segments=4))
    assert plan["kv_tiles"] == 22 * math.ceil(n / 64), plan
    log(f"int8k full size seed {seed}: oracle ...")
    for G in (4, 0):
        o, lse, _ = seq.attend(0, 25, q, k, v, W, use_ref=True, G=G)
        assert_fp8(seq, o, lse, 25, q, k, v, W, use_ref=True, raw_tol=TOL[KIND],
                   what=f"int8k full size seed {seed} G={G}")


def test_int8k_refused_calls():
    import attention_bca_attend_amd as bca
    cache = new_cache(1, 2, 128, 32, 2)
    with pytest.raises(bca.BcaError) as e:
        cache.set_kv_scales(0, [1.0, 1.0], [1.0, 1.0])
    assert e.value.status == -4
    _, k, v = Sequence(cache, 2, 128, 32, KIND).chunk(0)
    kf, vf = to_dev(k, "fp32"), to_dev(v, "fp32")
    with pytest.raises(bca.BcaError) as e:  # only bf16 inputs are quantised into it
        bca.bca_append_chunk(cache.handle, 0, 0, 0, kf.data_ptr(), vf.data_ptr(), bca.F32, 0)
    assert e.value.status == -4
