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

from bca_harness import TOL, Sequence, assert_close, assert_fp8, log, to_dev

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


def draw_sequences(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        dtype = "fp32" if i % 4 == 3 else "bf16"
        d = int(rng.choice([64, 128]))
        H = int(rng.integers(1, 5))
        n = int(rng.choice(N_CHOICES if dtype == "bf16" else N_CHOICES[:8]))
        C = int(rng.integers(1, 7))
        W = int(rng.integers(0, C + 1))
        P = int(rng.choice([0, 0, 1, 17, n]))
        G = int(rng.choice([0, 0, 1, 2, 3, 5]))
        out.append((dtype, i, H, d, n, C, P, W, G))
    return out


SEQ_CASES = draw_sequences(16, 9200)


@pytest.mark.parametrize("dtype,i,H,d,n,C,P,W,G", SEQ_CASES)
def test_random_sequence(dtype, i, H, d, n, C, P, W, G):
    """The training form (bca_attend_sequence: every chunk of a clip at once,
    each over the memory prefix, itself and its W predecessors) on random
    shapes against oracle.attend_sequence."""
    import math

    import attention_bca_attend_amd as bca
    import oracle
    import synth
    from bca_harness import to_np
    what = f"sequence {dtype} case {i}: H {H} d {d} n {n} C {C} P {P} W {W} G {G}"
    log(what)
    rows = P + C * n
    seed = 700 + i
    q = synth.tensor((C * n, H, d), synth.TAG_Q, seed, 0, 0, dtype=dtype)
    k = synth.tensor((rows, H, d), synth.TAG_K, seed, 0, 0, dtype=dtype)
    v = synth.tensor((rows, H, d), synth.TAG_V, seed, 0, 0, dtype=dtype)
    o, lse = bca.attend_sequence(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), n, W,
                                 prefix_tokens=P, num_segments=G)
    torch.cuda.synchronize()
    eo, el = oracle.attend_sequence(q, k, v, n, W, P, 1.0 / math.sqrt(d))
    assert_close(to_np(o), to_np(lse), eo, el, TOL[dtype], what)


ROPE_CASES = [c for j, kind in enumerate(("bf16", "fp8", "fp8_block", "int8k_block"))
              for c in draw(kind, 3, 9300 + j)]


@pytest.mark.parametrize("kind,i,H,d,n,S,W,R,G", ROPE_CASES)
def test_random_rope_stream(kind, i, H, d, n, S, W, R, G):
    """The streaming path with rotary embedding fused in (K rotated into the
    ring by bca_append_chunk_rope, Q and the chunk's K by bca_attend_rope; token
    r of chunk t at position t*n + r) against the oracle attending over inputs
    it rotates itself in fp64."""
    import math

    import oracle
    import synth
    import attention_bca_attend_amd as bca
    from bca_harness import (FP8_CACHE_ABS, FP8_CACHE_REL, block_stored, fp8_stored, max_err,
                             to_np)
    base = 10000.0
    what = f"rope {kind} case {i}: H {H} d {d} n {n} S {S} W {W} R {R} G {G}"
    log(what)
    cache = bca.Cache(1, H, d, n, S, has_ref=R, kv_dtype=kind)
    sc = [8.0 / 448.0] * H
    if kind == "fp8":
        cache.set_kv_scales(0, sc, sc)

    def stored(k, v):
        if kind == "fp8":
            return fp8_stored(k, sc), fp8_stored(v, sc)
        if kind in ("fp8_block", "int8k_block"):
            return block_stored(kind, k, v)
        return k.astype(np.float64), v.astype(np.float64)

    seed = 800 + 11 * i + len(kind)
    hist, ref = {}, None
    if R:
        _, rk, rv = synth.qkv(n, H, d, seed, 95_000, 0, dtype="bf16")
        cache.append_chunk(0, 0, to_dev(rk, "bf16"), to_dev(rv, "bf16"), is_ref=True,
                           rope=(base, 0))
        ref = stored(oracle.rope(rk.astype(np.float64), 0, base), rv)
    scale = 1.0 / math.sqrt(d)
    for t in range(S + 2):
        q, k, v = synth.qkv(n, H, d, seed, t, 0, dtype="bf16")
        use_ref = R and t % 2 == 0
        spec = cache.spec(t, W, use_ref=use_ref, num_segments=G)
        o, lse = cache.attend(0, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), spec,
                              rope=(base, t * n))
        qr = oracle.rope(q.astype(np.float64), t * n, base)
        kr = oracle.rope(k.astype(np.float64), t * n, base)
        go, gl = to_np(o), to_np(lse)
        if kind == "bf16":
            eo, el = oracle.attend(qr, kr, v.astype(np.float64), hist, t=t, W=W, scale=scale,
                                   ref=ref, use_ref=use_ref)
            assert_close(go, gl, eo, el, TOL["bf16"], f"{what} t {t}")
        else:
            # the chunk's own K is staged rotated in bf16, then made 8-bit
            ks, vs = stored(synth.round_bf16(kr).astype(np.float64), v)
            eo, el = oracle.attend(qr, ks, vs, hist, t=t, W=W, scale=scale, ref=ref,
                                   use_ref=use_ref)
            assert np.all(np.abs(go - eo) <= FP8_CACHE_ABS + FP8_CACHE_REL * np.abs(eo)), \
                f"{what} t {t}: vs stored {max_err(go, eo)}"
            assert max_err(gl, el) <= FP8_CACHE_ABS, f"{what} t {t}"
        cache.append_chunk(0, t, to_dev(k, "bf16"), to_dev(v, "bf16"), rope=(base, t * n))
        hist[t] = stored(kr, v)
