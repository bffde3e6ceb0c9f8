"""Rotary position embedding fused into the path (bca_append_chunk_rope,
bca_attend_rope) against the CPU oracle's rotation (oracle.rope, fp64).

Bars: the stored K equals the oracle's rotation rounded to the cache dtype,
bf16 within one unit in the last place (plus 2e-6 where a pair's components
cancel), fp32 within 4e-6, 8-bit codes equal or adjacent (on a per-block
cache with the block's K scale taken over the rotated rows, as the oracle's
rule gives it to within the fp32 rotation's rounding); attention as for
bca_attend (1e-5 fp32, 1e-2 bf16, the 8-bit bars of bca_harness.assert_fp8).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from bca_harness import (FP8_CACHE_ABS, FP8_CACHE_REL, TOL, assert_close, block_stored,
                         fp8_stored, log, max_err, to_dev, to_np)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BASE = 10000.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def new_cache(L, H, d, n, S, R=False, dtype="bf16"):
    import attention_bca_attend_amd as bca
    return bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=dtype)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_append_rope_stores_rotated_k(dtype, d):
    H, n, S = 3, 40, 2
    cache = new_cache(1, H, d, n, S, dtype=dtype)
    in_dt = "fp32" if dtype == "fp32" else "bf16"
    for t in (0, 5, 2000):
        _, k, v = synth.qkv(n, H, d, 4, t, 0, dtype=in_dt)
        pos0 = t * n
        cache.append_chunk(0, t, to_dev(k, dtype), to_dev(v, dtype), rope=(BASE, pos0))
        K, V = cache.blocks(0)
        torch.cuda.synchronize()
        kk = K[:, t % S].float().cpu().numpy().astype(np.float64).transpose(1, 0, 2)
        vv = V[:, t % S].float().cpu().numpy().transpose(1, 0, 2)
        want = oracle.rope(k.astype(np.float64), pos0, BASE)
        err = np.abs(kk - want)
        if dtype == "bf16":
            # rounding the fp32 rotation and the exact one can differ by one ulp;
            # where the pair's components cancel, the fp32 rotation's own error
            # (a few 1e-7 absolute) can exceed the ulp of the tiny result
            assert np.all(err <= bf16_ulp(want) + 2e-6), (t, err.max())
            exact = synth.round_bf16(want).reshape(want.shape)
            log(f"append rope bf16 d {d} t {t}: {np.mean(kk == exact):.4%} of K equal to the "
                f"rounded oracle rotation, max |dK| {err.max():.3e}")
        else:
            assert err.max() <= 4e-6, (t, err.max())
        assert np.array_equal(vv, v), "V is stored as given"


def test_append_rope_fp8_codes():
    H, d, n, S = 4, 128, 40, 2
    cache = new_cache(1, H, d, n, S, dtype="fp8")
    ks = [0.011 * (h + 1) for h in range(H)]
    vs = [8.0 / 448.0] * H
    cache.set_kv_scales(0, ks, vs)
    for t in (0, 3, 777):
        _, k, v = synth.qkv(n, H, d, 6, t, 0, dtype="bf16")
        pos0 = t * n
        cache.append_chunk(0, t, to_dev(k, "bf16"), to_dev(v, "bf16"), rope=(BASE, pos0))
        K, V = cache.blocks(0)
        torch.cuda.synchronize()
        kc = K[:, t % S].cpu().numpy()
        vc = V[:, t % S].cpu().numpy()
        rot = oracle.rope(k.astype(np.float64), pos0, BASE).astype(np.float32)
        same = 0
        for h in range(H):
            want = oracle.quant_e4m3(rot[:, h, :], ks[h])
            # same sign bit and magnitude codes at most one apart
            dmag = np.abs((kc[h] & 0x7F).astype(int) - (want & 0x7F).astype(int))
            sign_ok = ((kc[h] ^ want) & 0x80) == 0
            assert np.all((dmag == 0) | ((dmag == 1) & sign_ok)), h
            same += int(np.sum(kc[h] == want))
            assert np.array_equal(vc[h], oracle.quant_e4m3(v[:, h, :], vs[h])), h
        log(f"append rope fp8 t {t}: {same / kc.size:.4%} of K codes equal to the oracle's")
        assert same / kc.size >= 0.99


@pytest.mark.parametrize("kind", ["fp8_block", "int8k_block"])
def test_append_rope_block_scales_and_codes(kind):
    """A rotary append into a per-block cache: the block's K scales are the
    oracle's rule (fp32 max |x| / 448, / 127 for int8 K) over the oracle's
    rotation, to within the fp32 rotation's own rounding (the kernel rotates
    in fp32, the oracle in fp64); the K codes, taken with the stored scale,
    equal the oracle's or differ by one step where the two rotations fall on
    either side of a rounding boundary; V is stored as given, bit for bit."""
    H, d, n, S = 4, 128, 40, 2
    cache = new_cache(1, H, d, n, S, dtype=kind)
    int8 = kind == "int8k_block"
    for t in (0, 3, 777):
        _, k, v = synth.qkv(n, H, d, 6, t, 0, dtype="bf16", outlier_frac=0.01)
        pos0 = t * n
        cache.append_chunk(0, t, to_dev(k, "bf16"), to_dev(v, "bf16"), rope=(BASE, pos0))
        torch.cuda.synchronize()
        K, V = cache.blocks(0)
        KS, VS = cache.block_scales(0)
        blk = t % S
        rot = oracle.rope(k.astype(np.float64), pos0, BASE).astype(np.float32)
        want_ks = oracle.block_scales(rot, qmax=127.0 if int8 else 448.0)
        gks = KS[blk].cpu().numpy()
        assert np.allclose(gks, want_ks, rtol=2.0 ** -20, atol=0.0), (t, gks, want_ks)
        assert np.array_equal(VS[blk].cpu().numpy(), oracle.block_scales(v)), t
        kc = K[:, blk].cpu().numpy()
        vc = V[:, blk].cpu().numpy()
        same = 0
        for h in range(H):
            if int8:
                got = kc[h].view(np.int8).astype(int)
                want = oracle.quant_int8(rot[:, h, :], float(gks[h])).astype(int)
                assert np.all(np.abs(got - want) <= 1), (t, h)
                same += int(np.sum(got == want))
            else:
                want = oracle.quant_e4m3(rot[:, h, :], float(gks[h]))
                dmag = np.abs((kc[h] & 0x7F).astype(int) - (want & 0x7F).astype(int))
                sign_ok = ((kc[h] ^ want) & 0x80) == 0
                assert np.all((dmag == 0) | ((dmag == 1) & sign_ok)), (t, h)
                same += int(np.sum(kc[h] == want))
            assert np.array_equal(vc[h], oracle.quant_e4m3(v[:, h, :], float(VS[blk][h]))), (t, h)
        log(f"append rope {kind} t {t}: {same / kc.size:.4%} of K codes equal to the oracle's")
        assert same / kc.size >= 0.99


CASES = [
    # dtype, H, d, n, S, W, R, G, chunks
    ("bf16", 2, 128, 100, 2, 2, False, 0, 5),
    ("bf16", 3, 64, 130, 3, 2, True, 3, 5),
    ("fp32", 2, 64, 16, 2, 2, False, 2, 6),
    ("fp8", 4, 128, 405 // 5, 4, 3, True, 2, 6),
    ("fp8_block", 4, 128, 405 // 5, 4, 3, True, 2, 6),
    ("int8k_block", 3, 128, 100, 3, 2, True, 0, 5),
]
EIGHT_BIT = ("fp8", "fp8_block", "int8k_block")


@pytest.mark.parametrize("dtype,H,d,n,S,W,R,G,chunks", CASES)
def test_attend_rope_sequence(dtype, H, d, n, S, W, R, G, chunks):
    """Every chunk is appended with K rotated at positions id*n + r, and every
    query chunk attends with Q and its own K rotated the same way; the oracle
    rotates the same inputs in fp64 and attends over the result."""
    cache = new_cache(1, H, d, n, S, R=R, dtype=dtype)
    in_dt = "fp32" if dtype == "fp32" else "bf16"
    scales = None
    if dtype == "fp8":
        scales = ([8.0 / 448.0 * (1 + 0.1 * h) for h in range(H)], [8.0 / 448.0] * H)
        cache.set_kv_scales(0, scales[0], scales[1])

    def stored(k, v):
        if dtype == "fp8":
            return fp8_stored(k, scales[0]), fp8_stored(v, scales[1])
        if dtype in ("fp8_block", "int8k_block"):
            return block_stored(dtype, k, v)
        return k.astype(np.float64), v.astype(np.float64)

    history, history_raw, ref, ref_raw = {}, {}, None, None
    if R:
        _, rk, rv = synth.qkv(n, H, d, 8, 999, 0, dtype=in_dt)
        cache.append_chunk(0, 0, to_dev(rk, dtype), to_dev(rv, dtype), is_ref=True,
                           rope=(BASE, 0))
        rkr = oracle.rope(rk.astype(np.float64), 0, BASE)
        ref = stored(rkr, rv)
        ref_raw = (rkr, rv.astype(np.float64))
    scale = 1.0 / math.sqrt(d)
    for t in range(chunks):
        q, k, v = synth.qkv(n, H, d, 8, t, 0, dtype=in_dt)
        pos0 = t * n
        spec = cache.spec(t, W, use_ref=R, num_segments=G)
        o, lse = cache.attend(0, to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), spec,
                              rope=(BASE, pos0))
        qr = oracle.rope(q.astype(np.float64), pos0, BASE)
        kr = oracle.rope(k.astype(np.float64), pos0, BASE)
        if dtype in EIGHT_BIT:
            # the staging pass writes the rotated K in the qkv dtype (bf16)
            # before the 8-bit copy of the chunk is made from it
            ks, vs = stored(synth.round_bf16(kr).astype(np.float64), v)
        else:
            ks, vs = stored(kr, v)
        eo, el = oracle.attend(qr, ks, vs, history, t=t, W=W, scale=scale, ref=ref, use_ref=R)
        if dtype in EIGHT_BIT:
            # against the cache contents (the kernel's own error), then against
            # the unquantised rotated inputs: within the quantisation's own
            # error plus the kernel's bar (a few hundred keys; see assert_fp8)
            go, gl = to_np(o), to_np(lse)
            log(f"rope {dtype} t={t}: vs stored max|dO| {max_err(go, eo):.3e}, "
                f"max|dLSE| {max_err(gl, el):.3e}")
            assert np.all(np.abs(go - eo) <= FP8_CACHE_ABS + FP8_CACHE_REL * np.abs(eo)), t
            assert max_err(gl, el) <= FP8_CACHE_ABS, t
            ro, rl = oracle.attend(qr, kr, v.astype(np.float64), history_raw, t=t, W=W,
                                   scale=scale, ref=ref_raw, use_ref=R)
            quant = max_err(eo, ro)
            log(f"rope {dtype} t={t}: vs raw max|dO| {max_err(go, ro):.3e}, quantisation alone "
                f"{quant:.3e}")
            assert max_err(go, ro) <= quant + FP8_CACHE_ABS + FP8_CACHE_REL * np.abs(eo).max()
            assert max_err(gl, rl) <= max_err(el, rl) + FP8_CACHE_ABS
        else:
            assert_close(to_np(o), to_np(lse), eo, el, TOL[dtype], f"rope {dtype} t={t}")
        cache.append_chunk(0, t, to_dev(k, dtype), to_dev(v, dtype), rope=(BASE, pos0))
        history[t] = stored(kr, v)
        history_raw[t] = (kr, v.astype(np.float64))


def test_attend_rope_matches_attend_on_rotated_inputs():
    """bca_attend_rope equals bca_attend given inputs rotated by the same kernel
    (the cached chunk rotated by the append, the current chunk's Q and K by the
    staging pass): the two calls differ only in where the rotation happens."""
    H, d, n, S, W = 2, 128, 96, 2, 2
    cache = new_cache(1, H, d, n, S)
    for t in range(2):
        _, k, v = synth.qkv(n, H, d, 12, t, 0, dtype="bf16")
        cache.append_chunk(0, t, to_dev(k, "bf16"), to_dev(v, "bf16"), rope=(BASE, t * n))
    q, k, v = synth.qkv(n, H, d, 12, 2, 0, dtype="bf16")
    spec = cache.spec(2, W, num_segments=1)  # one piece per unit: no partial outputs
    o1, l1 = cache.attend(0, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), spec,
                          rope=(BASE, 2 * n))
    # the staging pass leaves its rotated Q and K at the start of the workspace
    # (the plan needs no region of its own with one piece per unit)
    ws = cache.workspace(spec, rope=True)
    torch.cuda.synchronize()
    nbytes = n * H * d * 2
    qr = ws[:nbytes].view(torch.bfloat16).view(n, H, d).clone()
    kr = ws[((nbytes + 255) // 256) * 256:][:nbytes].view(torch.bfloat16).view(n, H, d).clone()
    want_q = oracle.rope(q.astype(np.float64), 2 * n, BASE)
    assert np.all(np.abs(to_np(qr) - want_q) <= bf16_ulp(want_q) + 2e-6)
    o2, l2 = cache.attend(0, qr, kr, to_dev(v, "bf16"), spec)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_attend_rope_full_size_wan_shape():
    """The Wan-shaped call the benchmark times with the rotation fused in (12
    heads x 1536 tokens, ring of 2 full slots, automatic split), chunk 2 at
    positions 2n .. 3n-1; the oracle on heads 0 and 11 in full."""
    H, d, n, S, W, t = 12, 128, 1536, 2, 2, 2
    cache = new_cache(1, H, d, n, S)
    history = {}
    for c in range(S):
        _, k, v = synth.qkv(n, H, d, 13, c, 0, dtype="bf16")
        cache.append_chunk(0, c, to_dev(k, "bf16"), to_dev(v, "bf16"), rope=(BASE, c * n))
        history[c] = (oracle.rope(k.astype(np.float64), c * n, BASE), v.astype(np.float64))
    q, k, v = synth.qkv(n, H, d, 13, t, 0, dtype="bf16")
    spec = cache.spec(t, W)
    o, lse = cache.attend(0, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), spec,
                          rope=(BASE, t * n))
    o, lse = to_np(o), to_np(lse)
    qr = oracle.rope(q.astype(np.float64), t * n, BASE)
    kr = oracle.rope(k.astype(np.float64), t * n, BASE)
    for h in (0, 11):
        hs = slice(h, h + 1)
        hist = {c: (kv[0][:, hs], kv[1][:, hs]) for c, kv in history.items()}
        eo, el = oracle.attend(qr[:, hs], kr[:, hs], v[:, hs].astype(np.float64), hist, t=t, W=W,
                               scale=1.0 / math.sqrt(d))
        assert_close(o[:, hs], lse[hs], eo, el, TOL["bf16"], f"Wan-shaped rope call head {h}")
