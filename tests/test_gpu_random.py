"""Seeded random configurations of the streaming path on every cache type,
against the CPU oracle: chunk sizes (1 token up to several key tiles, on and
off tile boundaries), heads, head dims, ring sizes, windows (0 up to the
whole ring), a reference block used on every other chunk, segment counts,
and enough chunks to wrap the ring. The cases are drawn from fixed seeds, so
a failure names its case and reproduces.

Bars: fp32 1e-5 and bf16 1e-2 against the oracle (max |dO|, |dLSE|); the
8-bit caches as everywhere else (bca_harness.assert_fp8: the kernel bar
against what the cache holds, and the quantisation's own error plus that bar
against the unquantised inputs).
"""
import numpy as np
import pytest

from bca_harness import TOL, Sequence, assert_close, assert_fp8, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CHOICES = [1, 5, 31, 63, 64, 65, 100, 127, 129, 200, 256, 300]
COUNTS = {"bf16": 12, "fp32": 5, "fp8": 5, "fp8_block": 5, "int8k_block": 5}


def draw(kind, count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        d = 128 if kind in ("fp8", "fp8_block", "int8k_block") else int(rng.choice([64, 128]))
        H = int(rng.integers(1, 5))
        n = int(rng.choice(N_CHOICES if kind != "fp32" else N_CHOICES[:8]))
        S = int(rng.integers(1, 7))
        W = int(rng.integers(0, S + 1))
        R = bool(rng.integers(0, 2))
        G = int(rng.choice([0, 0, 1, 2, 3, 5]))
        out.append((kind, i, H, d, n, S, W, R, G))
    return out


CASES = [c for j, (kind, count) in enumerate(COUNTS.items()) for c in draw(kind, count, 9100 + j)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


@pytest.mark.parametrize("kind,i,H,d,n,S,W,R,G", CASES)
def test_random_stream(kind, i, H, d, n, S, W, R, G):
    import attention_bca_attend_amd as bca
    what = f"{kind} case {i}: H {H} d {d} n {n} S {S} W {W} R {R} G {G}"
    log(what)
    cache = bca.Cache(1, H, d, n, S, has_ref=R, kv_dtype=kind)
    scales = ([8.0 / 448.0] * H, [8.0 / 448.0] * H) if kind == "fp8" else None
    seq = Sequence(cache, H, d, n, kind, seed_layer=500 + 37 * i + len(kind), scales=scales)
    if R:
        _, rk, rv = seq.chunk(90_000 + i)
        seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(S + 2):
        q, k, v = seq.chunk(t)
        use_ref = R and t % 2 == 0
        o, lse, _ = seq.attend(0, t, q, k, v, W, use_ref=use_ref, G=G)
        if kind in ("fp32", "bf16"):
            eo, el = seq.expected(t, q, k, v, W, use_ref=use_ref)
            assert_close(o, lse, eo, el, TOL[kind], f"{what} t {t}")
        else:
            assert_fp8(seq, o, lse, t, q, k, v, W, use_ref=use_ref, what=f"{what} t {t}")
        seq.append(0, t, k, v)
