"""GPU path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: mask and ring-slot indexing exact; O and LSE max-abs <= 1e-5 (fp32),
<= 1e-2 (bf16 with fp32 accumulation), <= 5e-2 (fp8 K/V cache).
"""
import math

import numpy as np
import pytest

import synth
from bca_harness import TOL, Sequence, assert_close, assert_fp8, log, max_err, to_dev, to_np

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


# ---------------------------------------------------------------------------
# configuration 0: tiny fp32, H 2, d 64, n 16, W 2, ring of 2 slots, 6 chunks
@pytest.mark.parametrize("G", [0, 1, 2, 4, 7])
def test_cfg0_fp32_sequence(G):
    H, d, n, S, W = 2, 64, 16, 2, 2
    cache = new_cache(1, H, d, n, S, dtype="fp32")
    seq = Sequence(cache, H, d, n, "fp32")
    for t in range(6):
        q, k, v = seq.chunk(t)
        o, lse, spec = seq.attend(0, t, q, k, v, W, G=G)
        eo, el = seq.expected(t, q, k, v, W)
        assert_close(o, lse, eo, el, TOL["fp32"], f"cfg0 G={G} t={t}")
        seq.append(0, t, k, v)
        assert cache.slot_chunk(0, t % S) == t


def test_cfg0_q_zero_lse_counts_visible_keys():
    H, d, n, S, W = 2, 64, 16, 2, 2
    cache = new_cache(1, H, d, n, S, dtype="fp32")
    seq = Sequence(cache, H, d, n, "fp32")
    for t in range(6):
        _, k, v = seq.chunk(t)
        o, lse, _ = seq.attend(0, t, np.zeros((n, H, d), np.float32), k, v, W)
        n_vis = [16, 32, 48, 48, 48, 48][t]
        assert np.abs(lse - math.log(n_vis)).max() <= 1e-6, t
        seq.append(0, t, k, v)


def test_cfg0_one_hot_probe_is_exact():
    # V row of token r of chunk c is e_{16 (c mod 4) + r}; with Q = 0 the output is
    # exactly 1/N_visible on visible columns and exactly 0 elsewhere.
    H, d, n, S, W = 2, 64, 16, 3, 2  # S = W + 1: a stale chunk stays resident
    cache = new_cache(1, H, d, n, S, dtype="fp32")
    seq = Sequence(cache, H, d, n, "fp32")
    for t in range(7):
        _, k, _ = seq.chunk(t)
        v = np.zeros((n, H, d), np.float32)
        for r in range(n):
            v[r, :, 16 * (t % 4) + r] = 1.0
        o, _, _ = seq.attend(0, t, np.zeros((n, H, d), np.float32), k, v, W)
        vis = list(range(max(0, t - W), t)) + [t]
        want = np.zeros(d)
        for c in vis:
            want[16 * (c % 4):16 * (c % 4) + 16] = 1.0 / (n * len(vis))
        for c in range(4):
            cols = slice(16 * c, 16 * c + 16)
            if want[16 * c] == 0.0:
                assert np.all(o[:, :, cols] == 0.0), (t, c)
            else:
                assert np.abs(o[:, :, cols] - want[16 * c]).max() <= 1e-7, (t, c)
        seq.append(0, t, k, v)


# ---------------------------------------------------------------------------
# bf16 shapes: ragged chunks, small chunks, both head dims, segments, reference
BF16_CASES = [
    # H, d, n, S, W, R, G, chunks
    (2, 128, 100, 2, 2, False, 1, 4),
    (3, 128, 200, 3, 2, False, 0, 5),
    (2, 64, 130, 2, 1, False, 3, 4),
    (1, 128, 16, 4, 4, True, 2, 6),
    (2, 128, 1, 3, 3, False, 1, 5),
    (2, 64, 64, 2, 2, True, 7, 4),
    (4, 128, 405, 5, 5, True, 4, 7),
    (2, 128, 257, 1, 0, False, 2, 3),
]


@pytest.mark.parametrize("H,d,n,S,W,R,G,chunks", BF16_CASES)
def test_bf16_sequences(H, d, n, S, W, R, G, chunks):
    cache = new_cache(1, H, d, n, S, R=R, dtype="bf16")
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=H * 1000 + n)
    if R:
        _, rk, rv = seq.chunk(10_000)
        seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(chunks):
        q, k, v = seq.chunk(t)
        o, lse, _ = seq.attend(0, t, q, k, v, W, use_ref=R, G=G)
        eo, el = seq.expected(t, q, k, v, W, use_ref=R)
        assert_close(o, lse, eo, el, TOL["bf16"], f"bf16 H{H} d{d} n{n} S{S} W{W} R{R} G{G} t={t}")
        seq.append(0, t, k, v)


def test_bf16_segments_agree_with_each_other():
    H, d, n, S, W = 2, 128, 300, 3, 3
    cache = new_cache(1, H, d, n, S)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=7)
    for t in range(3):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(3)
    eo, el = seq.expected(3, q, k, v, W)
    outs = {}
    for G in (1, 2, 4, 7, 0):
        o, lse, _ = seq.attend(0, 3, q, k, v, W, G=G)
        assert_close(o, lse, eo, el, TOL["bf16"], f"split G={G}")
        outs[G] = (o, lse)
    # a split only reorders sums: different G differ by rounding only
    for G in (2, 4, 7, 0):
        assert np.abs(outs[G][0] - outs[1][0]).max() <= 4e-3


def test_window_invariance_under_nan_in_stale_slots():
    # S = W + 1 keeps chunk t-W-1 resident; filling it (and the slot of a chunk
    # committed as id t itself) with NaN must leave O and LSE bit-identical.
    H, d, n, S, W = 2, 128, 96, 3, 2
    cache = new_cache(2, H, d, n, S)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=3)
    for t in range(4):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
        seq.append(1, t, k, v)
    q, k, v = seq.chunk(4)
    o1, l1, _ = seq.attend(0, 4, q, k, v, W)
    K, V = cache.blocks(0)
    stale = 1 % S  # chunk 1 = t - W - 1 lives in slot 1
    assert cache.slot_chunk(0, stale) == 1
    K[:, stale].fill_(float("nan"))
    V[:, stale].fill_(float("inf"))
    # layer 1 and other heads do not matter either
    K1, V1 = cache.blocks(1)
    K1.fill_(float("nan"))
    o2, l2, _ = seq.attend(0, 4, q, k, v, W)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o2).all()
    # a visible chunk does change it
    K[:, 3 % S].add_(1.0)
    o3, _, _ = seq.attend(0, 4, q, k, v, W)
    assert not np.array_equal(o1, o3)


def test_deterministic():
    H, d, n, S, W = 3, 128, 333, 2, 2
    cache = new_cache(1, H, d, n, S)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=5)
    for t in range(2):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(2)
    for G in (0, 3):
        a = seq.attend(0, 2, q, k, v, W, G=G)
        b = seq.attend(0, 2, q, k, v, W, G=G)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_merge_ignores_workspace_contents():
    """Whatever the workspace holds before a call (zeros, all ones, random
    bytes, or a previous call's partial outputs) the output and LSE of a
    split window are the same, bit for bit, and match the oracle; so do
    repeated calls on one workspace."""
    H, d, n, S, W = 12, 128, 300, 2, 2
    cache = new_cache(1, H, d, n, S)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=6)
    for t in range(2):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(2)
    eo, el = seq.expected(2, q, k, v, W)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    for G in (3, 0):
        spec = cache.spec(2, W, num_segments=G)
        plan = cache.plan(0, spec)
        assert plan["merge"] == 1, plan
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device="cuda")
        g = torch.Generator(device="cuda").manual_seed(7)
        ref = None
        for fill in ("zero", "ones", "random", "reuse", "reuse"):
            if fill == "zero":
                ws.zero_()
            elif fill == "ones":
                ws.fill_(255)
            elif fill == "random":
                ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device="cuda",
                                       dtype=torch.int32).to(torch.uint8))
            o, lse = cache.attend(0, qd, kd, vd, spec, workspace=ws)
            torch.cuda.synchronize()
            got = (to_np(o), to_np(lse))
            if ref is None:
                ref = got
                assert_close(got[0], got[1], eo, el, TOL["bf16"], f"split G={G}, fresh workspace")
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), (G, fill)
        log(f"split G={G}: same result over zeroed, 0xff, random and reused workspaces")


def test_stream_k_ranges_cross_units():
    """More units than work groups: ranges of tile iterations cross unit
    boundaries, so one work group finishes the end of one unit and starts the
    next, and units are split at uneven points."""
    H, d, n, S, W = 130, 64, 257, 1, 1
    cache = new_cache(1, H, d, n, S)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=8)
    _, k0, v0 = seq.chunk(0)
    seq.append(0, 0, k0, v0)
    q, k, v = seq.chunk(1)
    plan = cache.plan(0, cache.spec(1, W))
    assert plan["units"] > plan["workgroups"] and plan["merge"] == 1, plan
    o, lse, _ = seq.attend(0, 1, q, k, v, W)
    eo, el = seq.expected(1, q, k, v, W)
    assert_close(o, lse, eo, el, TOL["bf16"], f"stream-K {plan['units']} units")


# ---------------------------------------------------------------------------
# append: cache bytes are the input rows, bit for bit (fp8: the oracle's codes)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_append_bytes_exact(dtype):
    H, d, n, S = 3, 64 if dtype == "fp32" else 128, 50, 3
    cache = new_cache(2, H, d, n, S, R=True, dtype=dtype)
    seq = Sequence(cache, H, d, n, dtype, seed_layer=9)
    for t in range(7):
        _, k, v = seq.chunk(t)
        seq.append(1, t, k, v)
        K, V = cache.blocks(1)
        torch.cuda.synchronize()
        kk = K[:, t % S].float().cpu().numpy()  # [H][n][d]
        vv = V[:, t % S].float().cpu().numpy()
        assert np.array_equal(kk, k.transpose(1, 0, 2)) and np.array_equal(vv, v.transpose(1, 0, 2))
        for s in range(S):
            want = max([c for c in range(t + 1) if c % S == s], default=-1)
            assert cache.slot_chunk(1, s) == want
    _, rk, rv = seq.chunk(99)
    seq.append(1, 5, rk, rv, is_ref=True)
    K, _ = cache.blocks(1)
    assert np.array_equal(K[:, S].float().cpu().numpy(), rk.transpose(1, 0, 2))
    assert cache.slot_chunk(1, S) == 5
    # layer 0 untouched (the buffer was never written: only slot ids matter)
    assert all(cache.slot_chunk(0, s) == -1 for s in range(S))


def test_append_fp8_codes_match_oracle_quantiser():
    import oracle
    H, d, n, S = 4, 128, 40, 2
    cache = new_cache(1, H, d, n, S, R=True, dtype="fp8")
    ks = [0.011 * (h + 1) for h in range(H)]
    vs = [8.0 / 448.0 + 0.003 * h for h in range(H)]
    cache.set_kv_scales(0, ks, vs)
    seq = Sequence(cache, H, d, n, "fp8", seed_layer=11, outlier_frac=0.01)
    for t in range(3):
        _, k, v = seq.chunk(t)
        k = k * 3.0  # push some values past the saturation point
        k = synth.round_bf16(k).reshape(k.shape)
        seq.append(0, t, k, v)
        K, V = cache.blocks(0)
        torch.cuda.synchronize()
        kc = K[:, t % S].cpu().numpy()
        vc = V[:, t % S].cpu().numpy()
        for h in range(H):
            assert np.array_equal(kc[h], oracle.quant_e4m3(k[:, h, :], ks[h])), h
            assert np.array_equal(vc[h], oracle.quant_e4m3(v[:, h, :], vs[h])), h


# ---------------------------------------------------------------------------
# fp8 e4m3 K/V cache with per-head scales: the cache holds decode(quant(x/s))*s
# and the chunk attends at that precision, its own keys and values included.
# Every result is held to the oracle twice (bca_harness.assert_fp8): on the
# cache contents (the kernel's own error: Q and P rounded to two e4m3 terms,
# the bf16 output) and on the unquantised seeded inputs. On the second the
# 5e-2 bar for 8-bit K/V is asserted at the Matrix-Game size (8910 keys); on the
# small shapes below (a few hundred keys) e4m3's 3-bit mantissa alone moves
# O by more than that (a row dominated by one key inherits its rounding, up to
# 6 % of an 8-sigma value), so there the bar is the quantisation's own error
# (oracle on cache contents against oracle on raw inputs) plus the kernel's.
def fp8_scales(H, kmax=8.0, vmax=8.0):
    return ([kmax / 448.0 * (1.0 + 0.1 * h) for h in range(H)],
            [vmax / 448.0 * (1.0 + 0.05 * h) for h in range(H)])


@pytest.mark.parametrize("G,outliers", [(0, True), (1, True), (3, True), (0, False), (3, False)])
def test_fp8_sequence(G, outliers):
    H, d, n, S, W = 4, 128, 100, 3, 2
    cache = new_cache(1, H, d, n, S, R=True, dtype="fp8")
    seq = Sequence(cache, H, d, n, "fp8", seed_layer=21 if outliers else 22,
                   outlier_frac=0.01 if outliers else 0.0,
                   scales=fp8_scales(H) if outliers else fp8_scales(H, 6.0, 6.0))
    _, rk, rv = seq.chunk(90_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(1, 7):
        q, k, v = seq.chunk(t)
        use_ref = t % 2 == 0
        o, lse, _ = seq.attend(0, t, q, k, v, W, use_ref=use_ref, G=G)
        assert_fp8(seq, o, lse, t, q, k, v, W, use_ref=use_ref,
                   what=f"fp8 G={G} outliers={outliers} t={t}")
        seq.append(0, t, k, v)


def test_fp8_stream_k_ranges_cross_units():
    """The fp8 kernel with more units than work groups (64 heads x 5 query
    tiles): ranges of tile iterations cross unit boundaries."""
    H, d, n, S, W = 64, 128, 1025, 1, 1
    cache = new_cache(1, H, d, n, S, dtype="fp8")
    seq = Sequence(cache, H, d, n, "fp8", seed_layer=31, outlier_frac=0.01,
                   scales=fp8_scales(H))
    _, k0, v0 = seq.chunk(0)
    seq.append(0, 0, k0, v0)
    q, k, v = seq.chunk(1)
    plan = cache.plan(0, cache.spec(1, W))
    assert plan["units"] > plan["workgroups"] and plan["merge"] == 1, plan
    o, lse, _ = seq.attend(0, 1, q, k, v, W)
    assert_fp8(seq, o, lse, 1, q, k, v, W, what=f"fp8 stream-K {plan['units']} units")


def test_fp8_workspace_holds_the_chunk_copy():
    H, d, n, S = 2, 128, 64, 2
    cache = new_cache(1, H, d, n, S, dtype="fp8")
    spec = cache.spec(0, 2, num_segments=1)
    plan = cache.plan(0, spec)
    # one work group per unit, yet the workspace is needed for the fp8 copy
    assert plan["merge"] == 0 and plan["workspace_bytes"] >= 2 * H * n * d


def test_cfg4_full_size():
    # config-2 shapes over an fp8 cache with 1% outliers of 8 sigma
    H, d, n, S, W = 24, 128, 405, 20, 20
    cache = new_cache(1, H, d, n, S, R=True, dtype="fp8")
    seq = Sequence(cache, H, d, n, "fp8", seed_layer=4, outlier_frac=0.01,
                   scales=([8.0 / 448.0] * H, [8.0 / 448.0] * H))
    _, rk, rv = seq.chunk(100_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    for t in range(5, 25):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(25)
    log("cfg4: oracle ...")
    for G in (4, 0):
        o, lse, _ = seq.attend(0, 25, q, k, v, W, use_ref=True, G=G)
        # the 5e-2 bar for 8-bit K/V, against the unquantised seeded inputs
        assert_fp8(seq, o, lse, 25, q, k, v, W, use_ref=True, raw_tol=TOL["fp8"],
                   what=f"cfg4 full size G={G}")


def test_slot_table_over_64_chunks():
    for S in (2, 20):
        cache = new_cache(1, 1, 64, 8, S)
        seq = Sequence(cache, 1, 64, 8, "bf16", seed_layer=S)
        for t in range(64):
            _, k, v = seq.chunk(t)
            seq.append(0, t, k, v)
            assert cache.slot_chunk(0, t % S) == t
        for s in range(S):
            assert cache.slot_chunk(0, s) == max(c for c in range(64) if c % S == s)


# ---------------------------------------------------------------------------
# full-size configurations (one chunk-layer each, whole output against the oracle)
def test_cfg1_full_size():
    H, d, n, S, W = 12, 128, 1536, 2, 2
    cache = new_cache(1, H, d, n, S)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=0)
    for t in range(2):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(2)
    log("cfg1: oracle ...")
    eo, el = seq.expected(2, q, k, v, W)
    for G in (0, 1):
        o, lse, _ = seq.attend(0, 2, q, k, v, W, G=G)
        assert_close(o, lse, eo, el, TOL["bf16"], f"cfg1 full size G={G}")


def test_cfg2_full_size():
    H, d, n, S, W = 24, 128, 405, 20, 20
    cache = new_cache(1, H, d, n, S, R=True)
    seq = Sequence(cache, H, d, n, "bf16", seed_layer=0)
    _, rk, rv = seq.chunk(100_000)
    seq.append(0, 0, rk, rv, is_ref=True)
    # chunks 5..24 in the ring (slots wrapped), query chunk 25
    for t in range(5, 25):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(25)
    log("cfg2: oracle ...")
    eo, el = seq.expected(25, q, k, v, W, use_ref=True)
    for G in (4, 0):
        o, lse, _ = seq.attend(0, 25, q, k, v, W, use_ref=True, G=G)
        assert_close(o, lse, eo, el, TOL["bf16"], f"cfg2 full size G={G}")


def test_cfg3_64_chunks_first_and_last_layer():
    """Config-1 shapes streamed over 64 chunks through a 30-layer cache: per
    chunk every layer runs 4 denoise-step attends and then appends the
    chunk's K/V into ring slot id mod 2 (31 wraparounds). Layers 0 and 29 are
    held to the oracle at the last step of every chunk: on 49 rows of every
    head for chunks 0 .. 62, on every row for chunk 63. Every row of a chunk
    sees the same keys, so the sampled rows' queries are drawn from the seeded
    generator and the other rows hold arbitrary values."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    H, d, n, S, W, L, C = 12, 128, 1536, 2, 2, 30, 64
    check = (0, L - 1)
    cache = new_cache(L, H, d, n, S)
    rows = list(range(0, n, 32)) + [n - 1]
    scale = 1.0 / math.sqrt(d)

    def committed(l, t):
        return (synth.tensor((n, H, d), synth.TAG_K, l, t, 3),
                synth.tensor((n, H, d), synth.TAG_V, l, t, 3))

    pool = ThreadPoolExecutor(8)
    futs = {(l, t): pool.submit(committed, l, t) for t in range(C) for l in check}
    g = torch.Generator(device="cuda").manual_seed(3)
    filler = [torch.randn((n, H, d), generator=g, device="cuda").to(torch.bfloat16)
              for _ in range(3)]
    hist = {l: {} for l in check}
    worst = 0.0
    for t in range(C):
        spec = cache.spec(t, W, num_segments=0)
        for l in range(L):
            if l in check:
                k, v = futs.pop((l, t)).result()
                kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
            else:
                kd, vd = filler[1], filler[2]
            for step in range(4):
                if l in check and step == 3:
                    if t == C - 1:
                        q = synth.tensor((n, H, d), synth.TAG_Q, l, t, 3)
                        qd, want = to_dev(q, "bf16"), list(range(n))
                    else:
                        q = synth.tensor_rows((n, H, d), rows, synth.TAG_Q, l, t, 3)
                        qd, want = filler[0].clone(), rows
                        qd[rows] = to_dev(q, "bf16")
                    o, lse = cache.attend(l, qd, kd, vd, spec)
                    h = {c: hist[l][c] for c in range(max(0, t - 3), t)}  # t-3: masked
                    eo, el = oracle.attend(q, k, v, h, t=t, W=W, scale=scale,
                                           rows=None if t == C - 1 else list(range(len(rows))))
                    go, gl = to_np(o)[want], to_np(lse)[:, want]
                    assert_close(go, gl, eo, el, TOL["bf16"], f"cfg3 chunk {t} layer {l}"
                                 if t in (0, 1, 2, C - 1) or t % 16 == 0 else None)
                    worst = max(worst, max_err(go, eo), max_err(gl, el))
                else:
                    cache.attend(l, filler[0], kd, vd, spec)
            cache.append_chunk(l, t, kd, vd)
            if l in check:
                hist[l][t] = (k, v)
                hist[l].pop(t - 4, None)
        for l in check:
            assert cache.slot_chunk(l, t % S) == t
    log(f"cfg3: 64 chunks, layers {check}, every chunk within {worst:.3e} of the oracle")
