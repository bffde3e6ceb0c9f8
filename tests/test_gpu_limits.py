"""The largest configurations the interface accepts, against the CPU oracle:
62 ring slots plus the reference (64 key blocks with the current chunk, the
most a plan holds), 64 segments, and 64 heads on an e4m3 cache."""
import numpy as np
import pytest

from bca_harness import TOL, Sequence, assert_close, log, assert_fp8

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def new_cache(L, H, d, n, S, R=False, dtype="bf16"):
    import attention_bca_attend_amd as bca
    return bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=dtype)


@pytest.mark.parametrize("G", [0, 64])
def test_full_ring_of_62_slots_with_reference(G):
    H, d, n, S, W = 2, 64, 64, 62, 62
    cache = new_cache(1, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=51)
    _, rk, rv = seq.chunk(50_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(70):  # wraps the ring
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(70)
    plan = cache.plan(0, cache.spec(70, W, use_ref=True, num_segments=G))
    assert len(plan["visible_blocks"]) == 64, plan
    o, lse, _ = seq.attend(0, 70, q, k, v, W, use_ref=True, G=G)
    eo, el = seq.expected(70, q, k, v, W, use_ref=True)
    assert_close(o, lse, eo, el, TOL["bf16"], f"62 slots + reference + current, G={G}, "
                                              f"{plan['max_pieces']} pieces per unit")


def test_fp32_full_ring():
    H, d, n, S, W = 2, 64, 16, 62, 40
    cache = new_cache(1, H, d, n, S, R=True, dtype="fp32")
    seq = Sequence(cache, H, d, n, "fp32", seed_layer=52)
    _, rk, rv = seq.chunk(60_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(80):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    for G in (0, 7):
        q, k, v = seq.chunk(80)
        o, lse, _ = seq.attend(0, 80, q, k, v, W, use_ref=True, G=G)
        eo, el = seq.expected(80, q, k, v, W, use_ref=True)
        assert_close(o, lse, eo, el, TOL["fp32"], f"fp32 62-slot ring, window 40, G={G}")


@pytest.mark.parametrize("dtype", ["fp8", "fp8_block", "int8k_block"])
def test_fp8_with_64_heads(dtype):
    H, d, n, S, W = 64, 128, 40, 2, 2
    cache = new_cache(1, H, d, n, S, dtype=dtype)
    scales = None
    if dtype == "fp8":
        scales = ([8.0 / 448.0 * (1 + h / 64) for h in range(H)], [8.0 / 448.0] * H)
    seq = Sequence(cache, H, d, n, dtype, seed_layer=53, outlier_frac=0.01, scales=scales)
    for t in range(4):
        q, k, v = seq.chunk(t)
        o, lse, _ = seq.attend(0, t, q, k, v, W)
        assert_fp8(seq, o, lse, t, q, k, v, W, what=f"{dtype} 64 heads t={t}")
        seq.append(0, t, k, v)
    log(f"{dtype}: 64 heads within the bar")
