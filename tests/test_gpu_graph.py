"""The chunk loop captured once in a HIP graph and replayed chunk after chunk
(bca_append_chunk_dev with a device-side chunk id, bca_chunk_counter_advance,
captured bca_attend calls) against the same loop run eagerly on a second
cache with the same contents.

Both run the same kernels with the same plans on the same inputs, so every
replay must give bit-identical outputs, LSE and cache bytes. Two replayed
chunks per case (the first and the last, one layer each end) are also held to
the CPU oracle directly, on the seeded inputs they were computed from. Each
replay is separated from the next by eager work (new inputs copied in, the
eager loop, comparisons) and a synchronisation.
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def _chunk(n, H, d, layer, t, fp8):
    q, k, v = synth.qkv(n, H, d, 70 + layer, t, 0, dtype="bf16",
                        outlier_frac=0.01 if fp8 else 0.0)
    return to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")


def _np_chunk(n, H, d, layer, t, fp8):
    return synth.qkv(n, H, d, 70 + layer, t, 0, dtype="bf16", outlier_frac=0.01 if fp8 else 0.0)


def _oracle_check(kv, H, d, n, layer, t, W, R, o, lse, what):
    """A replayed chunk against the oracle on the seeded inputs it was computed
    from: the chunks t-W .. t-1 (and the reference chunk, id 1000) as the
    history, chunk t as the query chunk. On an 8-bit cache against what the
    cache holds, at the kernel's bar, and against the unquantised inputs within
    the quantisation's own error plus that bar."""
    fp8 = kv in ("fp8", "fp8_block", "int8k_block")

    def stored(k, v):
        if kv == "fp8":
            s = [8.0 / 448.0] * H
            return fp8_stored(k, s), fp8_stored(v, s)
        if kv in ("fp8_block", "int8k_block"):
            return block_stored(kv, k, v)
        return k.astype(np.float64), v.astype(np.float64)

    hist, hraw = {}, {}
    for c in range(max(0, t - W), t):
        _, k, v = _np_chunk(n, H, d, layer, c, fp8)
        hist[c], hraw[c] = stored(k, v), (k.astype(np.float64), v.astype(np.float64))
    ref = ref_raw = None
    if R:
        _, rk, rv = _np_chunk(n, H, d, layer, 1000, fp8)
        ref, ref_raw = stored(rk, rv), (rk.astype(np.float64), rv.astype(np.float64))
    q, k, v = _np_chunk(n, H, d, layer, t, fp8)
    kk, vv = stored(k, v)
    scale = 1.0 / math.sqrt(d)
    eo, el = oracle.attend(q, kk, vv, hist, t=t, W=W, scale=scale, ref=ref, use_ref=R)
    go, gl = to_np(o), to_np(lse)
    if not fp8:
        assert_close(go, gl, eo, el, TOL["bf16"], what)
        return
    ro, rl = oracle.attend(q, k, v, hraw, t=t, W=W, scale=scale, ref=ref_raw, use_ref=R)
    quant = max_err(eo, ro)
    log(f"{what}: vs stored max|dO| {max_err(go, eo):.3e}, vs raw {max_err(go, ro):.3e} "
        f"(quantisation alone {quant:.3e})")
    assert np.all(np.abs(go - eo) <= FP8_CACHE_ABS + FP8_CACHE_REL * np.abs(eo)), what
    assert max_err(gl, el) <= FP8_CACHE_ABS, what
    assert max_err(go, ro) <= quant + FP8_CACHE_ABS + FP8_CACHE_REL * np.abs(eo).max(), what
    assert max_err(gl, rl) <= max_err(el, rl) + FP8_CACHE_ABS, what


CASES = [
    # kv dtype, L, H, d, n, S (= W), reference, segments
    ("bf16", 2, 2, 128, 100, 2, False, 0),
    ("bf16", 2, 3, 64, 64, 3, True, 2),
    ("fp8", 2, 2, 128, 96, 2, True, 0),
    ("fp8_block", 2, 2, 128, 96, 2, True, 0),
    ("int8k_block", 2, 2, 128, 96, 2, True, 0),
]


@pytest.mark.parametrize("kv,L,H,d,n,S,R,G", CASES)
def test_replayed_chunk_step_equals_eager(kv, L, H, d, n, S, R, G):
    import attention_bca_attend_amd as bca
    fp8 = kv in ("fp8", "fp8_block", "int8k_block")
    log(f"graph replay {kv} L {L} H {H} d {d} n {n} S {S} R {R} G {G}")
    A = bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=kv)
    B = bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=kv)
    # the whole memory is compared below, including bytes no call writes (the
    # padding after a block-scaled cache's scale table)
    A.mem.zero_()
    B.mem.zero_()
    for c in (A, B):
        if kv == "fp8":
            for l in range(L):
                c.set_kv_scales(l, [8.0 / 448.0] * H, [8.0 / 448.0] * H)
        for l in range(L):
            if R:
                _, k, v = _chunk(n, H, d, l, 1000, fp8)
                c.append_chunk(l, 0, k, v, is_ref=True)
            for t in range(S):
                _, k, v = _chunk(n, H, d, l, t, fp8)
                c.append_chunk(l, t, k, v)
    # static buffers the graph reads and writes
    Q = [torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    K = [torch.empty_like(Q[0]) for _ in range(L)]
    V = [torch.empty_like(Q[0]) for _ in range(L)]
    O = [torch.empty_like(Q[0]) for _ in range(L)]
    LSE = [torch.empty((H, n), dtype=torch.float32, device="cuda") for _ in range(L)]
    t0 = S
    spec0 = A.spec(t0, S, use_ref=R, num_segments=G)
    ws = A.workspace(spec0)
    d_chunk = torch.full((1,), t0, dtype=torch.int64, device="cuda")
    for l in range(L):
        assert A.replayable(l, spec0)
    # every kernel the graph holds runs once before the capture (code objects
    # load on first launch), on B's spare twin so that A and B stay equal
    scratch = bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=kv)
    if kv == "fp8":
        scratch.set_kv_scales(0, [8.0 / 448.0] * H, [8.0 / 448.0] * H)
    dummy = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    q, k, v = _chunk(n, H, d, 0, 0, fp8)
    scratch.attend(0, q, k, v, scratch.spec(0, S, num_segments=G), workspace=None)
    scratch.append_chunk_dev(0, dummy, k, v)
    bca.Cache.advance_counter(dummy)
    torch.cuda.synchronize()
    assert int(dummy.item()) == 0

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(L):
            A.attend(l, Q[l], K[l], V[l], spec0, out=O[l], lse=LSE[l], workspace=ws)
            A.append_chunk_dev(l, d_chunk, K[l], V[l])
        bca.Cache.advance_counter(d_chunk)
    torch.cuda.synchronize()

    t_end = t0 + 2 * S + 3  # wraps the ring more than twice
    for t in range(t0, t_end):
        for l in range(L):
            q, k, v = _chunk(n, H, d, l, t, fp8)
            Q[l].copy_(q)
            K[l].copy_(k)
            V[l].copy_(v)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            A.set_slot_chunk(l, t % S, t)
        assert int(d_chunk.item()) == t + 1
        if t in (t0, t_end - 1):
            l = 0 if t == t0 else L - 1
            _oracle_check(kv, H, d, n, l, t, S, R, O[l], LSE[l], f"replay {kv} chunk {t} layer {l}")
        spec = B.spec(t, S, use_ref=R, num_segments=G)
        for l in range(L):
            o, lse = B.attend(l, Q[l], K[l], V[l], spec)
            torch.cuda.synchronize()
            assert torch.equal(o, O[l]) and torch.equal(lse, LSE[l]), (t, l)
            B.append_chunk(l, t, K[l], V[l])
        torch.cuda.synchronize()
        assert torch.equal(A.mem, B.mem), f"cache bytes differ after chunk {t}"
        for l in range(L):
            assert A.slot_chunk(l, t % S) == B.slot_chunk(l, t % S) == t
    log(f"graph replay {kv}: chunks {t0}..{t} bit-identical to the eager loop")


def test_device_chunk_id_negative_writes_nothing():
    import attention_bca_attend_amd as bca
    H, d, n, S = 2, 128, 40, 2
    c = bca.Cache(1, H, d, n, S, kv_dtype="bf16")
    c.mem.fill_(7)
    before = c.mem.clone()
    _, k, v = _chunk(n, H, d, 0, 0, False)
    neg = torch.full((1,), -3, dtype=torch.int64, device="cuda")
    c.append_chunk_dev(0, neg, k, v)
    torch.cuda.synchronize()
    assert torch.equal(c.mem, before)
    # a device id of 5 writes slot 1 exactly as bca_append_chunk(5) does
    five = torch.full((1,), 5, dtype=torch.int64, device="cuda")
    c.append_chunk_dev(0, five, k, v)
    ref = bca.Cache(1, H, d, n, S, kv_dtype="bf16")
    ref.mem.fill_(7)
    ref.append_chunk(0, 5, k, v)
    torch.cuda.synchronize()
    assert torch.equal(c.mem, ref.mem)
    assert np.array_equal(c.blocks(0)[0][:, 1].float().cpu().numpy(),
                          k.float().cpu().numpy().transpose(1, 0, 2))


@pytest.mark.parametrize("kv,L,H,d,n,S,W,R,G", [("bf16", 2, 2, 128, 100, 3, 2, False, 0),
                                                ("bf16", 2, 3, 64, 64, 4, 1, True, 2),
                                                ("bf16", 1, 2, 128, 405, 20, 19, True, 4),
                                                ("fp8", 2, 2, 128, 96, 3, 2, True, 0),
                                                ("fp8_block", 2, 2, 128, 96, 3, 2, True, 0),
                                                ("fp8_block", 1, 2, 128, 130, 5, 3, False, 2),
                                                ("int8k_block", 2, 2, 128, 96, 3, 2, True, 0),
                                                ("int8k_block", 1, 3, 128, 64, 4, 1, True, 0)])
def test_replayed_step_with_window_smaller_than_ring(kv, L, H, d, n, S, W, R, G):
    """Windows smaller than the ring see different slots from chunk to chunk:
    the captured attends read the chunk id from the device counter and take
    the visible slots from it (bca_attend_dev; on a block-scaled cache also
    each visible block's scales). Every replay must equal a host-planned
    bca_attend of the same chunk on a twin cache, bit for bit."""
    import attention_bca_attend_amd as bca
    log(f"graph replay, window {W} < ring {S}: {kv} L {L} H {H} d {d} n {n} R {R} G {G}")
    fp8 = kv in ("fp8", "fp8_block", "int8k_block")
    A = bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=kv)
    B = bca.Cache(L, H, d, n, S, has_ref=R, kv_dtype=kv)
    A.mem.zero_()
    B.mem.zero_()
    for c in (A, B):
        for l in range(L):
            if kv == "fp8":
                c.set_kv_scales(l, [8.0 / 448.0] * H, [8.0 / 448.0] * H)
            if R:
                _, k, v = _chunk(n, H, d, l, 1000, fp8)
                c.append_chunk(l, 0, k, v, is_ref=True)
            for t in range(S):
                _, k, v = _chunk(n, H, d, l, t, fp8)
                c.append_chunk(l, t, k, v)
    Q = [torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    K = [torch.empty_like(Q[0]) for _ in range(L)]
    V = [torch.empty_like(Q[0]) for _ in range(L)]
    O = [torch.empty_like(Q[0]) for _ in range(L)]
    LSE = [torch.empty((H, n), dtype=torch.float32, device="cuda") for _ in range(L)]
    t0 = S
    spec0 = A.spec(t0, W, use_ref=R, num_segments=G)
    assert not A.replayable(0, spec0)  # a captured bca_attend would be wrong later
    ws = A.workspace(spec0)
    d_chunk = torch.full((1,), t0, dtype=torch.int64, device="cuda")
    # code objects load on first launch: one eager run on a scratch cache first
    scratch = bca.Cache(1, H, d, n, S, has_ref=R, kv_dtype=kv)
    if kv == "fp8":
        scratch.set_kv_scales(0, [8.0 / 448.0] * H, [8.0 / 448.0] * H)
    for t in range(S):
        _, k, v = _chunk(n, H, d, 0, t, False)
        scratch.append_chunk(0, t, k, v)
    if R:
        scratch.append_chunk(0, 0, k, v, is_ref=True)
    q, k, v = _chunk(n, H, d, 0, S, False)
    scratch.attend_dev(0, d_chunk, q, k, v, spec0, O[0], LSE[0], ws)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(L):
            A.attend_dev(l, d_chunk, Q[l], K[l], V[l], spec0, O[l], LSE[l], ws)
            A.append_chunk_dev(l, d_chunk, K[l], V[l])
        bca.Cache.advance_counter(d_chunk)
    torch.cuda.synchronize()

    t_end = t0 + 2 * S + 3
    for t in range(t0, t_end):
        for l in range(L):
            q, k, v = _chunk(n, H, d, l, t, fp8)
            Q[l].copy_(q)
            K[l].copy_(k)
            V[l].copy_(v)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            A.set_slot_chunk(l, t % S, t)
        assert int(d_chunk.item()) == t + 1
        if t in (t0, t_end - 1):
            # a replay of bca_attend_dev (visible slots from the device-side id)
            l = 0 if t == t0 else L - 1
            _oracle_check(kv, H, d, n, l, t, W, R, O[l], LSE[l],
                          f"replay (device id) {kv} chunk {t} layer {l}")
        spec = B.spec(t, W, use_ref=R, num_segments=G)
        for l in range(L):
            o, lse = B.attend(l, Q[l], K[l], V[l], spec)
            torch.cuda.synchronize()
            assert torch.equal(o, O[l]) and torch.equal(lse, LSE[l]), (t, l)
            B.append_chunk(l, t, K[l], V[l])
        torch.cuda.synchronize()
        assert torch.equal(A.mem, B.mem), f"cache bytes differ after chunk {t}"
    log(f"window {W} < ring {S}: chunks {t0}..{t} bit-identical to host-planned calls")
