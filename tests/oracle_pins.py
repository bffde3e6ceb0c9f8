"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises
AssertionError on a mismatch. ``tests/test_oracle_pins.py`` runs them on the
real oracle; ``tests/test_oracle_mutants.py`` runs them on deliberately broken
copies and requires that some pin fails for each.

What pins what:
* hand-computed cases (tests/golden/hand_cases.json): visibility rules, the
  softmax weights, LSE base and the scale;
* Q = 0 closed form: LSE = ln N_visible and O = mean of the visible V rows,
  over the config-0 chunk sequence (N_visible 16, 32, 48, 48, 48, 48);
* one-hot probe: which keys are visible, exactly;
* window invariance under NaN/Inf perturbation of everything invisible;
* split + log-sum-exp merge equals one pass;
* constant and affine V;
* reductions to an independent library routine
  (torch.nn.functional.scaled_dot_product_attention in float64 on the CPU);
* large logits (max subtraction);
* OCP E4M3 codec against torch.float8_e4m3fn and the spec's rounding rules;
* rotary embedding: identity at position 0, lengths, composition, dependence
  on the position difference only, and an independent implementation;
* the whole-sequence (training) form: reductions to library attention (no
  mask, the library's own causal mask, a prefix without mask), agreement with
  the chunk-by-chunk oracle, the Q = 0 closed form and invariance to
  everything outside each chunk's window.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def _arr(x):
    return np.array(x, dtype=np.float64)


def pin_hand_cases(lib):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        hist = {int(i): (_arr(kv["k"]), _arr(kv["v"])) for i, kv in c["history"].items()}
        ref = (_arr(c["ref"]["k"]), _arr(c["ref"]["v"])) if "ref" in c else None
        o, lse = lib.attend(_arr(c["q"]), _arr(c["k_cur"]), _arr(c["v_cur"]), hist, t=c["t"],
                            W=c["W"], scale=c["scale"], ref=ref, use_ref=bool(c["use_ref"]))
        np.testing.assert_allclose(o, _arr(c["expected_o"]), rtol=0, atol=1e-14,
                                   err_msg=c["name"])
        np.testing.assert_allclose(lse, _arr(c["expected_lse"]), rtol=0, atol=1e-14,
                                   err_msg=c["name"])


def _chunks(n, H, d, count, tag_seed, dtype="fp32"):
    out = {}
    for c in range(count):
        k = synth.tensor((n, H, d), synth.TAG_K, tag_seed, c, 0, dtype=dtype)
        v = synth.tensor((n, H, d), synth.TAG_V, tag_seed, c, 0, dtype=dtype)
        out[c] = (k.astype(np.float64), v.astype(np.float64))
    return out


def pin_q_zero_closed_form(lib):
    # config-0 shapes: H 2, d 64, n 16, W 2; six chunk steps, every earlier chunk committed
    H, d, n, W = 2, 64, 16, 2
    chunks = _chunks(n, H, d, 6, 11)
    for t in range(6):
        hist = {c: chunks[c] for c in range(t)}
        q = np.zeros((n, H, d))
        k_cur, v_cur = chunks[t]
        o, lse = lib.attend(q, k_cur, v_cur, hist, t=t, W=W, scale=1 / 8)
        vis = [c for c in range(max(0, t - W), t)] + [t]
        n_vis = n * len(vis)
        assert n_vis == [16, 32, 48, 48, 48, 48][t]
        np.testing.assert_allclose(lse, np.full((H, n), math.log(n_vis)), rtol=0, atol=1e-13)
        vals = np.concatenate([chunks[c][1] for c in vis], axis=0)  # [n_vis][H][d]
        mean = vals.mean(axis=0)
        np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-13)


def pin_one_hot_probe(lib):
    # V row of token r of chunk c is the unit vector e_{16 (c mod 4) + r}; with Q = 0
    # every visible key gets weight exactly 1/N and every other column is exactly 0.
    H, d, n, W = 2, 64, 16, 2
    for t in range(6):
        hist = {}
        for c in range(max(0, t - 3), t):
            k = synth.tensor((n, H, d), synth.TAG_K, 12, c, 0, dtype="fp32").astype(np.float64)
            v = np.zeros((n, H, d))
            for r in range(n):
                v[r, :, 16 * (c % 4) + r] = 1.0
            hist[c] = (k, v)
        k_cur = synth.tensor((n, H, d), synth.TAG_K, 12, t, 0, dtype="fp32").astype(np.float64)
        v_cur = np.zeros((n, H, d))
        for r in range(n):
            v_cur[r, :, 16 * (t % 4) + r] = 1.0
        o, _ = lib.attend(np.zeros((n, H, d)), k_cur, v_cur, hist, t=t, W=W, scale=0.125)
        vis = [c for c in range(max(0, t - W), t)] + [t]
        expect = np.zeros(d)
        for c in vis:
            expect[16 * (c % 4):16 * (c % 4) + 16] = 1.0 / (n * len(vis))
        for i in range(n):
            for h in range(H):
                assert np.array_equal(o[i, h], expect), (t, i, h)


def pin_window_invariance(lib):
    H, d, n, W, t = 2, 16, 8, 2, 5
    chunks = _chunks(n, H, d, 9, 13)
    q = synth.tensor((n, H, d), synth.TAG_Q, 13, t, 0, dtype="fp32")
    k_cur, v_cur = chunks[t]
    base_hist = {c: chunks[c] for c in (1, 2, 3, 4, 5, 7)}  # 1, 2 old; 5 = t; 7 future
    o0, l0 = lib.attend(q, k_cur, v_cur, base_hist, t=t, W=W, scale=0.25)
    bad = dict(base_hist)
    for c, fill in ((1, np.nan), (2, np.inf), (5, -np.inf), (7, 1e300)):
        bad[c] = (np.full((n, H, d), fill), np.full((n, H, d), fill))
    o1, l1 = lib.attend(q, k_cur, v_cur, bad, t=t, W=W, scale=0.25)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # dropping the invisible chunks altogether changes nothing either
    o2, l2 = lib.attend(q, k_cur, v_cur, {3: chunks[3], 4: chunks[4]}, t=t, W=W, scale=0.25)
    assert np.array_equal(o0, o2) and np.array_equal(l0, l2)
    # heads are independent: perturbing head 1 everywhere leaves head 0 bit-identical
    q2 = q.astype(np.float64).copy()
    q2[:, 1] = 7.0
    hist2 = {c: (kv[0].copy(), kv[1].copy()) for c, kv in base_hist.items()}
    for kv in hist2.values():
        kv[0][:, 1] = np.nan
        kv[1][:, 1] = np.nan
    o3, l3 = lib.attend(q2, k_cur, v_cur, hist2, t=t, W=W, scale=0.25)
    assert np.array_equal(o0[:, 0], o3[:, 0]) and np.array_equal(l0[0], l3[0])
    # a window-sized change (a visible chunk) does change the result
    hist4 = dict(base_hist)
    hist4[4] = (chunks[4][0] + 1.0, chunks[4][1])
    o4, _ = lib.attend(q, k_cur, v_cur, hist4, t=t, W=W, scale=0.25)
    assert not np.array_equal(o0, o4)


def pin_split_merge(lib):
    H, d, n = 2, 16, 12
    nk = 5 * n
    rng_k = synth.tensor((nk, H, d), synth.TAG_K, 14, 0, 0, dtype="fp32")
    rng_v = synth.tensor((nk, H, d), synth.TAG_V, 14, 0, 0, dtype="fp32")
    q = synth.tensor((n, H, d), synth.TAG_Q, 14, 0, 0, dtype="fp32")
    mask = np.ones((n, nk), dtype=np.uint8)
    mask[:, n:2 * n] = 0  # one invisible block inside the key list
    o_ref, l_ref = lib.attend_masked(q, rng_k, rng_v, mask, 0.3)
    for G in (1, 2, 4, 7):
        bounds = np.linspace(0, nk, G + 1).round().astype(int)
        ops, lps = [], []
        for g in range(G):
            a, b = bounds[g], bounds[g + 1]
            o_g, l_g = lib.attend_masked(q, rng_k[a:b], rng_v[a:b], mask[:, a:b], 0.3)
            ops.append(o_g.transpose(1, 0, 2).reshape(H * n, d))
            lps.append(l_g.reshape(H * n))
        o_m, l_m = lib.lse_merge(np.stack(ops), np.stack(lps))
        np.testing.assert_allclose(o_m.reshape(H, n, d).transpose(1, 0, 2), o_ref, rtol=0,
                                   atol=1e-12)
        np.testing.assert_allclose(l_m.reshape(H, n), l_ref, rtol=0, atol=1e-12)
    # a piece whose keys are all invisible has LSE -inf and weight 0
    o_e, l_e = lib.attend_masked(q, rng_k[n:2 * n], rng_v[n:2 * n], mask[:, n:2 * n], 0.3)
    assert np.all(l_e == -np.inf) and np.all(o_e == 0.0)


def pin_merge_closed_forms(lib):
    rows, d = 6, 8
    o1 = synth.tensor((rows, d), synth.TAG_MISC, 1, dtype="fp32").astype(np.float64)
    l1 = synth.tensor((rows,), synth.TAG_MISC, 2, dtype="fp32").astype(np.float64)
    # one piece is the identity
    o, l = lib.lse_merge(o1[None], l1[None])
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, l1, rtol=0, atol=1e-15)
    # two identical pieces: same output, LSE + ln 2
    o, l = lib.lse_merge(np.stack([o1, o1]), np.stack([l1, l1]))
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, l1 + math.log(2.0), rtol=0, atol=1e-14)
    # pieces with LSE a and a + ln 3: weights 1/4 and 3/4
    o2 = o1 + 1.0
    o, l = lib.lse_merge(np.stack([o1, o2]), np.stack([l1, l1 + math.log(3.0)]))
    np.testing.assert_allclose(o, 0.25 * o1 + 0.75 * o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, l1 + math.log(4.0), rtol=0, atol=1e-14)
    # an -inf piece contributes nothing
    o, l = lib.lse_merge(np.stack([o1, np.full_like(o1, 5.0)]),
                         np.stack([l1, np.full_like(l1, -np.inf)]))
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, l1, rtol=0, atol=1e-15)


def pin_constant_and_affine_v(lib):
    H, d, n, W, t = 2, 16, 8, 2, 4
    chunks = _chunks(n, H, d, 5, 15)
    q = synth.tensor((n, H, d), synth.TAG_Q, 15, t, 0, dtype="fp32")
    vconst = synth.tensor((H, d), synth.TAG_MISC, 3, dtype="fp32").astype(np.float64)
    hist = {c: (chunks[c][0], np.broadcast_to(vconst, (n, H, d)).copy()) for c in range(t)}
    hist[0] = (chunks[0][0], np.full((n, H, d), np.nan))  # invisible
    o, _ = lib.attend(q, chunks[t][0], np.broadcast_to(vconst, (n, H, d)).copy(), hist, t=t,
                      W=W, scale=0.25)
    np.testing.assert_allclose(o, np.broadcast_to(vconst, o.shape), rtol=1e-14, atol=1e-15)
    # affine: O(a V + b) = a O(V) + b
    hist = {c: chunks[c] for c in range(t)}
    o1, l1 = lib.attend(q, chunks[t][0], chunks[t][1], hist, t=t, W=W, scale=0.25)
    a, b = -2.5, 0.75
    hist_ab = {c: (kv[0], a * kv[1] + b) for c, kv in hist.items()}
    o2, l2 = lib.attend(q, chunks[t][0], a * chunks[t][1] + b, hist_ab, t=t, W=W, scale=0.25)
    np.testing.assert_allclose(o2, a * o1 + b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=0)


def _sdpa(q, k, v, mask_bool, scale):
    """torch SDPA in float64 on the CPU; q [nq][H][d], k/v [nk][H][d], mask [nq][nk]."""
    import torch
    import torch.nn.functional as F
    tq = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(1, 0, 2)
    tk = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).permute(1, 0, 2)
    tv = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).permute(1, 0, 2)
    m = torch.from_numpy(np.ascontiguousarray(mask_bool, dtype=bool))
    o = F.scaled_dot_product_attention(tq.contiguous(), tk.contiguous(), tv.contiguous(),
                                       attn_mask=m, scale=scale)
    s = torch.matmul(tq, tk.transpose(1, 2).contiguous()) * scale
    s = s.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.numpy()


def pin_reduces_to_library_attention(lib):
    H, d, n = 3, 32, 10
    chunks = _chunks(n, H, d, 6, 16)
    q = synth.tensor((n, H, d), synth.TAG_Q, 16, 5, 0, dtype="fp32").astype(np.float64)
    scale = d ** -0.5
    # W = 0, no reference: plain bidirectional attention over the current chunk
    hist = {c: chunks[c] for c in range(5)}
    o, l = lib.attend(q, chunks[5][0], chunks[5][1], hist, t=5, W=0, scale=scale)
    o_s, l_s = _sdpa(q, chunks[5][0], chunks[5][1], np.ones((n, n), bool), scale)
    np.testing.assert_allclose(o, o_s, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_s, rtol=0, atol=1e-12)
    # W >= t: block-causal over the whole prefix; library attention over all keys of
    # chunks 0..5 with an explicit boolean mask (chunk 5's rows see chunks <= 5)
    for W in (2, 5, 6):
        o, l = lib.attend(q, chunks[5][0], chunks[5][1], hist, t=5, W=W, scale=scale)
        K = np.concatenate([chunks[c][0] for c in range(6)])
        V = np.concatenate([chunks[c][1] for c in range(6)])
        cid = np.repeat(np.arange(6), n)
        mask = np.broadcast_to((cid >= 5 - W) & (cid <= 5), (n, 6 * n))
        o_s, l_s = _sdpa(q, K, V, mask, scale)
        np.testing.assert_allclose(o, o_s, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l_s, rtol=0, atol=1e-12)


def pin_token_level_sliding_window(lib):
    # n = 1: every chunk is one token, so block-causal is causal attention with a
    # sliding window of W + 1 tokens; compare the last token of a sequence against
    # library attention with a banded causal mask.
    H, d, T, W = 2, 8, 9, 3
    ks = synth.tensor((T, H, d), synth.TAG_K, 17, 0, 0, dtype="fp32").astype(np.float64)
    vs = synth.tensor((T, H, d), synth.TAG_V, 17, 0, 0, dtype="fp32").astype(np.float64)
    qs = synth.tensor((T, H, d), synth.TAG_Q, 17, 0, 0, dtype="fp32").astype(np.float64)
    idx = np.arange(T)
    band = (idx[None, :] <= idx[:, None]) & (idx[None, :] >= idx[:, None] - W)
    o_s, l_s = _sdpa(qs, ks, vs, band, 0.5)
    for t in range(T):
        hist = {c: (ks[c:c + 1], vs[c:c + 1]) for c in range(t)}
        o, l = lib.attend(qs[t:t + 1], ks[t:t + 1], vs[t:t + 1], hist, t=t, W=W, scale=0.5)
        np.testing.assert_allclose(o[0], o_s[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[:, 0], l_s[:, t], rtol=0, atol=1e-12)


def pin_large_logits(lib):
    # scores near 800 overflow exp() unless the row maximum is subtracted first.
    # Two keys with equal score s: O = mean of their values, LSE = s + ln 2.
    q = np.full((1, 1, 1), 40.0)
    k = np.full((1, 1, 1), 20.0)
    o, l = lib.attend(q, k, np.full((1, 1, 1), 3.0), {0: (k.copy(), np.full((1, 1, 1), 5.0))},
                      t=1, W=1, scale=1.0)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    np.testing.assert_allclose(o, [[[4.0]]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, [[800.0 + math.log(2.0)]], rtol=0, atol=1e-12)
    # the literal form (no subtraction) agrees while scores stay moderate
    H, d, n = 2, 16, 8
    chunks = _chunks(n, H, d, 3, 18)
    q = synth.tensor((n, H, d), synth.TAG_Q, 18, 2, 0, dtype="fp32")
    hist = {c: chunks[c] for c in range(2)}
    a = lib.attend(q, *chunks[2], hist, t=2, W=2, scale=0.25)
    b = lib.attend(q, *chunks[2], hist, t=2, W=2, scale=0.25, literal=True)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)


def pin_e4m3_codec(lib):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    dec = lib.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(dec), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(dec[~nan], ref[~nan])
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9 and dec[0x08] == 2.0 ** -6
    # every finite code round-trips, including the sign of zero
    finite = codes[~nan]
    back = lib.e4m3_encode(dec[~nan].astype(np.float32))
    assert np.array_equal(back, finite)
    # midpoints between neighbours go to the even mantissa
    pos = dec[:0x7F]
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert lib.e4m3_encode(mid) == want, c
        assert lib.e4m3_encode(-mid) == (want | 0x80), c
    # saturation and NaN
    for x, want in ((448.0, 0x7E), (460.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E),
                    (-np.inf, 0xFE), (-500.0, 0xFE)):
        assert lib.e4m3_encode(np.float32(x)) == want, x
    assert lib.e4m3_encode(np.float32(np.nan)) & 0x7F == 0x7F
    # in-range values agree with torch's conversion (round to nearest even)
    x = synth.tensor((4000,), synth.TAG_MISC, 4, dtype="fp32", scale=60.0)
    x = x[np.abs(x) < 440]
    mine = lib.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, theirs)
    # the quantiser divides in single precision and then encodes
    s = np.float32(8.0 / 448.0)
    q = lib.quant_e4m3(x / 60.0, float(s))
    assert np.array_equal(q, lib.e4m3_encode((x / 60.0).astype(np.float32) / s))


def pin_row_subset(lib):
    """Every query row of a chunk sees the same keys, so the oracle on a subset
    of the rows gives exactly those rows of the full result."""
    n, H, d = 12, 2, 8
    hist = _chunks(n, H, d, 3, 60)
    k, v = _chunks(n, H, d, 1, 61)[0]
    q = synth.tensor((n, H, d), synth.TAG_Q, 62, dtype="fp32").astype(np.float64)
    full_o, full_l = lib.attend(q, k, v, hist, t=3, W=2, scale=0.3)
    rows = [0, 5, 11, 7]
    o, l = lib.attend(q, k, v, hist, t=3, W=2, scale=0.3, rows=rows)
    assert np.array_equal(o, full_o[rows]) and np.array_equal(l, full_l[:, rows])


def pin_block_scales(lib):
    """Per-interval scale rule of an 8-bit cache block: per head, the largest
    magnitude over the block's rows and dims divided by the largest code, in
    single precision; 1 for a maximum of 0, infinity or NaN."""
    x = np.zeros((5, 4, 3), dtype=np.float32)
    x[2, 0, 1] = -7.0           # head 0: largest magnitude 7 (negative)
    x[4, 1, 2] = 448.0          # head 1: 448
    x[0, 1, 0] = 100.0
    x[3, 3, 0] = np.inf         # head 3: not finite; head 2 stays all zero
    s = lib.block_scales(x)
    assert s.dtype == np.float32 and s.shape == (4,)
    assert s[0] == np.float32(2.0 ** -6) and s[1] == 1.0 and s[2] == 1.0 and s[3] == 1.0, s
    x[3, 3, 0] = np.nan
    assert lib.block_scales(x)[3] == 1.0
    assert lib.block_scales(x, qmax=127.0)[0] == np.float32(7.0) / np.float32(127.0)
    # one head's maximum never leaks into another head's scale
    y = synth.tensor((16, 3, 8), synth.TAG_MISC, 40, dtype="fp32")
    y[:, 1, :] *= 50.0
    sy = lib.block_scales(y)
    for h in range(3):
        assert sy[h] == np.float32(np.abs(y[:, h, :]).max()) / np.float32(448.0), h
    # exact under powers of two
    for k in (-3, 5):
        assert np.array_equal(lib.block_scales(y * np.float32(2.0 ** k)),
                              sy * np.float32(2.0 ** k))
    # quantising with its own scale puts the largest magnitude on the largest
    # code (448) and nothing beyond
    for h in range(3):
        codes = lib.quant_e4m3(y[:, h, :], float(sy[h]))
        vals = np.abs(lib.e4m3_decode(codes.reshape(-1)))
        assert vals.max() == 448.0 and np.all(vals <= 448.0), h


def pin_int8_codec(lib):
    """Symmetric int8 codes: round to nearest even of fp32(x / scale), clamped
    to [-127, 127]; NaN gives 0."""
    c = np.arange(-127, 128, dtype=np.float32)
    assert np.array_equal(lib.quant_int8(c, 1.0), c.astype(np.int8))  # every code round-trips
    s = np.float32(0.0625)
    assert np.array_equal(lib.quant_int8(c * s, float(s)), c.astype(np.int8))
    # ties go to the even neighbour
    half = np.arange(-128, 127, dtype=np.float32) + np.float32(0.5)
    want = np.where(np.floor(half) % 2 == 0, np.floor(half), np.floor(half) + 1)
    want = np.clip(want, -127, 127)
    assert np.array_equal(lib.quant_int8(half, 1.0), want.astype(np.int8))
    # off-tie values go to the nearest integer
    for x, q in ((0.49, 0), (0.51, 1), (-0.51, -1), (2.4999, 2), (-2.5001, -3)):
        assert lib.quant_int8(np.array([x], np.float32), 1.0)[0] == q, x
    # clamping and NaN
    for x, q in ((127.4, 127), (127.5, 127), (300.0, 127), (-300.0, -127), (np.inf, 127),
                 (-np.inf, -127), (np.nan, 0)):
        assert lib.quant_int8(np.array([x], np.float32), 1.0)[0] == q, x
    # the division is in single precision: 1 / fp32(0.3) = 3.3333333 -> 3
    assert lib.quant_int8(np.array([1.0], np.float32), float(np.float32(0.3)))[0] == 3
    z = synth.tensor((3000,), synth.TAG_MISC, 41, dtype="fp32", scale=3.0)
    sc = np.float32(np.abs(z).max()) / np.float32(127.0)
    q = lib.quant_int8(z, float(sc)).astype(np.float64)
    assert np.abs(q).max() == 127.0
    assert np.all(np.abs(q * float(sc) - z) <= float(sc) / 2 * (1 + 1e-6))


def pin_rope(lib):
    """Rotary embedding: position 0 is the identity, every pair keeps its
    length, rotations compose (position a then b equals a + b), query-key
    products depend only on the position difference, and at base 10000 the
    result equals an independent implementation of the interleaved-pair form
    (transformers' GPT-J rotary helpers, float32 angles)."""
    rng = np.random.default_rng(7)
    H, d = 3, 16
    x = rng.standard_normal((5, H, d))
    y0 = lib.rope(x[:1], 0, 500.0)
    assert np.array_equal(y0, x[:1]), "position 0 must leave x unchanged"
    y = lib.rope(x, 37, 500.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(ny, nx, rtol=1e-12, atol=0), "pairs must keep their length"
    one = x[2:3]
    a, b = 11, 29
    assert np.allclose(lib.rope(lib.rope(one, a, 500.0), b, 500.0), lib.rope(one, a + b, 500.0),
                       rtol=0, atol=1e-12), "rotations must compose"
    q, k = rng.standard_normal((1, H, d)), rng.standard_normal((1, H, d))
    for m, kp, shift in ((5, 2, 40), (0, 9, 123), (300, 300, 7)):
        d0 = np.einsum("nhd,nhd->h", lib.rope(q, m, 500.0), lib.rope(k, kp, 500.0))
        d1 = np.einsum("nhd,nhd->h", lib.rope(q, m + shift, 500.0), lib.rope(k, kp + shift, 500.0))
        assert np.allclose(d0, d1, rtol=0, atol=1e-10), "q.k must depend on m - k only"
    import torch
    from transformers.models.gptj.modeling_gptj import (apply_rotary_pos_emb,
                                                        create_sinusoidal_positions)
    n = 24
    xs = rng.standard_normal((n, H, d)).astype(np.float32)
    table = create_sinusoidal_positions(n, d)  # [n][d]: sin | cos, float32
    sin, cos = table[None, :, : d // 2], table[None, :, d // 2:]
    ref = apply_rotary_pos_emb(torch.from_numpy(xs)[None], sin, cos)[0].double().numpy()
    got = lib.rope(xs.astype(np.float64), 0, 10000.0)
    assert np.abs(got - ref).max() <= 2e-5, "differs from the interleaved-pair rotary form"


def _seq(C, n, H, d, P, seed):
    rows = P + C * n
    q = synth.tensor((C * n, H, d), synth.TAG_Q, seed, 0, 0, dtype="fp32").astype(np.float64)
    k = synth.tensor((rows, H, d), synth.TAG_K, seed, 0, 0, dtype="fp32").astype(np.float64)
    v = synth.tensor((rows, H, d), synth.TAG_V, seed, 0, 0, dtype="fp32").astype(np.float64)
    return q, k, v


def pin_sequence_reduces_to_library_attention(lib):
    """Training form against torch SDPA (float64, CPU) where the block-causal
    mask reduces to something the library does itself."""
    import torch
    import torch.nn.functional as F
    H, d = 2, 16
    scale = d ** -0.5
    # W = 0, no prefix: every chunk attends to itself only, with no mask
    C, n = 4, 6
    q, k, v = _seq(C, n, H, d, 0, 31)
    o, l = lib.attend_sequence(q, k, v, n, 0, 0, scale)
    for c in range(C):
        sl = slice(c * n, (c + 1) * n)
        o_s, l_s = _sdpa(q[sl], k[sl], v[sl], np.ones((n, n), bool), scale)
        np.testing.assert_allclose(o[sl], o_s, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[c], l_s, rtol=0, atol=1e-12)
    # n = 1 and a window covering everything: plain causal attention, with the
    # library's own causal mask (is_causal)
    T = 9
    q, k, v = _seq(T, 1, H, d, 0, 32)
    for W in (T - 1, T + 3):
        o, l = lib.attend_sequence(q, k, v, 1, W, 0, scale)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).permute(1, 0, 2).contiguous()
                      for x in (q, k, v))
        o_s = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
        np.testing.assert_allclose(o, o_s.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # W = 0 with a prefix of P tokens: chunk c attends to [prefix; chunk c], no mask
    C, n, P = 3, 5, 7
    q, k, v = _seq(C, n, H, d, P, 33)
    o, l = lib.attend_sequence(q, k, v, n, 0, P, scale)
    for c in range(C):
        rows = np.r_[0:P, P + c * n:P + (c + 1) * n]
        sl = slice(c * n, (c + 1) * n)
        o_s, l_s = _sdpa(q[sl], k[rows], v[rows], np.ones((n, len(rows)), bool), scale)
        np.testing.assert_allclose(o[sl], o_s, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l[c], l_s, rtol=0, atol=1e-12)


def pin_sequence_matches_chunk_by_chunk(lib):
    """The training form equals the streaming oracle run chunk by chunk (every
    earlier chunk committed, the prefix as the reference chunk when P = n)."""
    H, d, n, C = 2, 8, 5, 6
    scale = 0.4
    for P, W in ((0, 2), (n, 2), (n, 0), (0, 7)):
        q, k, v = _seq(C, n, H, d, P, 34 + P + W)
        o, l = lib.attend_sequence(q, k, v, n, W, P, scale)
        ref = (k[:P], v[:P]) if P else None
        hist = {}
        for c in range(C):
            cur = slice(P + c * n, P + (c + 1) * n)
            sl = slice(c * n, (c + 1) * n)
            o_c, l_c = lib.attend(q[sl], k[cur], v[cur], dict(hist), t=c, W=W, scale=scale,
                                  ref=ref, use_ref=bool(P))
            np.testing.assert_allclose(o[sl], o_c, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l[c], l_c, rtol=0, atol=1e-12)
            hist[c] = (k[cur], v[cur])


def pin_sequence_q_zero_and_invariance(lib):
    """Q = 0: every visible key has weight 1/N, so LSE = ln N with
    N = P + (min(c, W) + 1) n, and O = the mean of the visible V rows. And the
    output of chunk c is bit-identical when every key row outside its window
    (older chunks, later chunks) is replaced by NaN or infinities."""
    H, d, n, C, P, W = 2, 8, 4, 6, 3, 2
    q, k, v = _seq(C, n, H, d, P, 40)
    z = np.zeros_like(q)
    o, l = lib.attend_sequence(z, k, v, n, W, P, 1.0)
    for c in range(C):
        first = max(0, c - W)
        rows = np.r_[0:P, P + first * n:P + (c + 1) * n]
        N = P + (c - first + 1) * n
        assert len(rows) == N
        np.testing.assert_allclose(l[c], np.full((H, n), math.log(N)), rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[c * n:(c + 1) * n],
                                   np.broadcast_to(v[rows].mean(axis=0), (n, H, d)),
                                   rtol=0, atol=1e-13)
    o1, l1 = lib.attend_sequence(q, k, v, n, W, P, 0.5)
    for c in range(C):
        first = max(0, c - W)
        k2, v2 = k.copy(), v.copy()
        outside = np.ones(P + C * n, bool)
        outside[:P] = False
        outside[P + first * n:P + (c + 1) * n] = False
        k2[outside] = np.nan
        v2[outside] = np.inf
        o2, l2 = lib.attend_sequence(q, k2, v2, n, W, P, 0.5)
        sl = slice(c * n, (c + 1) * n)
        assert np.array_equal(o2[sl], o1[sl]) and np.array_equal(l2[c], l1[c]), c


ALL_PINS = [pin_hand_cases, pin_q_zero_closed_form, pin_one_hot_probe, pin_window_invariance,
            pin_split_merge, pin_merge_closed_forms, pin_constant_and_affine_v,
            pin_reduces_to_library_attention, pin_token_level_sliding_window, pin_large_logits,
            pin_e4m3_codec, pin_row_subset, pin_block_scales, pin_int8_codec, pin_rope,
            pin_sequence_reduces_to_library_attention,
            pin_sequence_matches_chunk_by_chunk, pin_sequence_q_zero_and_invariance]
