"""Training-form block-causal attention over a whole sequence of chunks
(bca_attend_sequence) against the CPU oracle (oracle.attend_sequence, fp64,
explicit dense mask) on the same seeded, rounded inputs.

Bars as for bca_attend: max |dO| and |dLSE| <= 1e-5 for fp32, 1e-2 for bf16
with fp32 accumulation. Invisible key rows poisoned with NaN must leave the
chunks that cannot see them bit-identical.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from bca_harness import TOL, assert_close, log, to_dev, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def seq_inputs(C, n, H, d, P, dtype, seed):
    rows = P + C * n
    q = synth.tensor((C * n, H, d), synth.TAG_Q, seed, 0, 0, dtype=dtype)
    k = synth.tensor((rows, H, d), synth.TAG_K, seed, 0, 0, dtype=dtype)
    v = synth.tensor((rows, H, d), synth.TAG_V, seed, 0, 0, dtype=dtype)
    return q, k, v


def run(q, k, v, n, W, P, G, dtype):
    import attention_bca_attend_amd as bca
    o, lse = bca.attend_sequence(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), n, W,
                                 prefix_tokens=P, num_segments=G)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse)


CASES = [
    # dtype, H, d, n, C, P, W, G
    ("fp32", 2, 64, 16, 6, 0, 2, 0),
    ("fp32", 2, 64, 16, 5, 16, 1, 2),
    ("fp32", 3, 128, 37, 4, 5, 1, 3),
    ("bf16", 2, 128, 100, 5, 0, 2, 0),
    ("bf16", 3, 64, 17, 6, 9, 2, 3),
    ("bf16", 2, 128, 405, 3, 405, 20, 4),
    ("bf16", 2, 128, 64, 4, 0, 0, 1),
    ("bf16", 2, 128, 300, 4, 0, 1, 7),
    ("bf16", 1, 128, 1, 40, 0, 3, 0),
    # steady chunks share one launch: a prefix that stays while the window moves
    ("bf16", 2, 128, 256, 6, 100, 0, 0),
    # 39 steady chunks x 8 heads = 312 units, more than the chip holds: ranges
    # of key tiles cross unit (and chunk) boundaries
    ("bf16", 8, 64, 256, 40, 0, 1, 0),
]


@pytest.mark.parametrize("dtype,H,d,n,C,P,W,G", CASES)
def test_sequence_matches_oracle(dtype, H, d, n, C, P, W, G):
    log(f"sequence {dtype} H {H} d {d} n {n} C {C} P {P} W {W} G {G}")
    q, k, v = seq_inputs(C, n, H, d, P, dtype, 50 + n + C)
    o, lse = run(q, k, v, n, W, P, G, dtype)
    eo, el = oracle.attend_sequence(q, k, v, n, W, P, 1.0 / math.sqrt(d))
    assert_close(o, lse, eo, el, TOL[dtype], f"sequence {dtype} n {n} C {C} P {P} W {W} G {G}")


GROUPED = [
    # H, d, n, C, P, W with the automatic split and at least as many units as
    # the device has CUs: the chunks before the window is full and the steady
    # block run as one launch of groups of different lengths
    (32, 64, 256, 9, 100, 3),  # 5 groups (4 single chunks and the steady block), a prefix
    (16, 64, 128, 16, 0, 9),   # 10 launches' worth: the first 2 chunks alone, 8 groups in one
    (8, 64, 260, 16, 0, 1),    # ragged query tiles (260 = 256 + 4 rows)
]


@pytest.mark.parametrize("H,d,n,C,P,W", GROUPED)
def test_sequence_grouped_launch(H, d, n, C, P, W):
    """Launches of groups against the oracle, every head and row."""
    log(f"grouped sequence H {H} d {d} n {n} C {C} P {P} W {W}")
    q, k, v = seq_inputs(C, n, H, d, P, "bf16", 70 + C + W)
    o, lse = run(q, k, v, n, W, P, 0, "bf16")
    eo, el = oracle.attend_sequence(q, k, v, n, W, P, 1.0 / math.sqrt(d))
    assert_close(o, lse, eo, el, TOL["bf16"], f"grouped sequence n {n} C {C} P {P} W {W}")


def test_sequence_invisible_rows_do_not_leak():
    # NaN in chunk 0's keys and values: chunks c > W never see chunk 0, so their
    # outputs must equal those of an unpoisoned run bit for bit
    H, d, n, C, P, W = 2, 128, 100, 6, 0, 2
    q, k, v = seq_inputs(C, n, H, d, P, "bf16", 61)
    o1, l1 = run(q, k, v, n, W, P, 0, "bf16")
    k2, v2 = k.copy(), v.copy()
    k2[:n] = np.nan
    v2[:n] = np.inf
    o2, l2 = run(q, k2, v2, n, W, P, 0, "bf16")
    for c in range(W + 1, C):
        sl = slice(c * n, (c + 1) * n)
        assert np.array_equal(o1[sl], o2[sl]) and np.array_equal(l1[c], l2[c]), c
    # the poison did reach the chunks that see chunk 0 (what they then hold is
    # not specified: the keys are not numbers)
    assert not np.array_equal(o1[n:2 * n], o2[n:2 * n]), "chunk 1 sees chunk 0"
    log("sequence: NaN in chunk 0 stays out of chunks 3..5")


def test_sequence_equals_streaming_calls():
    # the same clip streamed through a ring cache (bca_attend per chunk, the
    # prefix as the reference chunk) gives the same result within bf16 bars
    import attention_bca_attend_amd as bca
    H, d, n, C, W = 2, 128, 96, 5, 2
    q, k, v = seq_inputs(C, n, H, d, n, "bf16", 62)
    o_seq, l_seq = run(q, k, v, n, W, n, 0, "bf16")
    cache = bca.Cache(1, H, d, n, W, has_ref=True, kv_dtype="bf16")
    cache.append_chunk(0, 0, to_dev(k[:n], "bf16"), to_dev(v[:n], "bf16"), is_ref=True)
    for c in range(C):
        cur = slice(n + c * n, n + (c + 1) * n)
        sl = slice(c * n, (c + 1) * n)
        spec = cache.spec(c, W, use_ref=True)
        o, lse = cache.attend(0, to_dev(q[sl], "bf16"), to_dev(k[cur], "bf16"),
                              to_dev(v[cur], "bf16"), spec)
        assert_close(to_np(o), to_np(lse), o_seq[sl], l_seq[c], TOL["bf16"],
                     f"streamed chunk {c} vs sequence")
        cache.append_chunk(0, c, to_dev(k[cur], "bf16"), to_dev(v[cur], "bf16"))


def test_sequence_full_size_wan_shape():
    # 4 chunks of the Wan-shaped step (12 heads x 1536 tokens, window 2), the
    # launch configuration the benchmark times; the oracle on heads 0 and 11
    H, d, n, C, W = 12, 128, 1536, 4, 2
    q, k, v = seq_inputs(C, n, H, d, 0, "bf16", 63)
    o, lse = run(q, k, v, n, W, 0, 0, "bf16")
    for h in (0, 11):
        hs = slice(h, h + 1)
        eo, el = oracle.attend_sequence(q[:, hs], k[:, hs], v[:, hs], n, W, 0, 1.0 / math.sqrt(d))
        assert_close(o[:, hs], lse[:, hs], eo, el, TOL["bf16"], f"Wan-shaped sequence head {h}")


def test_sequence_unsplit_launch_of_groups():
    """4 Wan-shaped chunks (12 heads x 1536 tokens) with a window of 1: chunk 0
    and chunks 1-3 run as one launch of groups cut on unit boundaries (no unit
    split, no merge, every output row stored whole by the attention kernel);
    the workspace is 0 bytes. The oracle on heads 0 and 11, every row."""
    import attention_bca_attend_amd as bca
    H, d, n, C, W = 12, 128, 1536, 4, 1
    spec = bca.bca_sequence_spec(H, d, n, C, 0, W, 0, 1.0 / math.sqrt(d))
    assert bca.bca_attend_sequence_workspace_bytes(spec, bca.BF16) == 0
    q, k, v = seq_inputs(C, n, H, d, 0, "bf16", 65)
    o, lse = run(q, k, v, n, W, 0, 0, "bf16")
    for h in (0, 11):
        hs = slice(h, h + 1)
        eo, el = oracle.attend_sequence(q[:, hs], k[:, hs], v[:, hs], n, W, 0, 1.0 / math.sqrt(d))
        assert_close(o[:, hs], lse[:, hs], eo, el, TOL["bf16"], f"unsplit launch of groups head {h}")


def test_sequence_wan_clip_of_8_as_benchmarked():
    """The training-form workload in the launch configuration the benchmark
    times: 8 Wan-shaped chunks (12 heads x 1536 tokens), window 2, automatic
    split: one launch of groups over 252 work groups of 144 tiles, no unit
    split, no merge. The oracle on heads 0, 5 and 11, every row."""
    import attention_bca_attend_amd as bca
    H, d, n, C, W = 12, 128, 1536, 8, 2
    spec = bca.bca_sequence_spec(H, d, n, C, 0, W, 0, 1.0 / math.sqrt(d))
    assert bca.bca_attend_sequence_workspace_bytes(spec, bca.BF16) == 0
    q, k, v = seq_inputs(C, n, H, d, 0, "bf16", 66)
    o, lse = run(q, k, v, n, W, 0, 0, "bf16")
    for h in (0, 5, 11):
        hs = slice(h, h + 1)
        eo, el = oracle.attend_sequence(q[:, hs], k[:, hs], v[:, hs], n, W, 0, 1.0 / math.sqrt(d))
        assert_close(o[:, hs], lse[:, hs], eo, el, TOL["bf16"], f"benchmarked 8-chunk clip head {h}")


def test_sequence_64_chunk_wan_clip():
    """A 64-chunk Wan-shaped clip (12 heads x 1536 tokens, window 2) in one
    call: its workspace is bounded by the launches' work groups (below 200 MB;
    here none at all: chunks 0, 1 and 2-63 run as one launch of groups, 4608
    units cut into ranges that all end on unit boundaries, so no unit is split
    and nothing is merged), and chunks 0, 1, 31 and 63 match the oracle on 49
    rows of every head. Only the rows and chunks the oracle sees are seeded
    draws; the rest are device random numbers."""
    import attention_bca_attend_amd as bca
    H, d, n, C, W = 12, 128, 1536, 64, 2
    spec = bca.bca_sequence_spec(H, d, n, C, 0, W, 0, 1.0 / math.sqrt(d))
    need = bca.bca_attend_sequence_workspace_bytes(spec, bca.BF16)
    log(f"64-chunk Wan clip: workspace {need / 1e6:.1f} MB")
    assert need < 200e6
    g = torch.Generator(device="cuda").manual_seed(64)
    qd = torch.randn((C * n, H, d), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((C * n, H, d), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((C * n, H, d), generator=g, device="cuda").to(torch.bfloat16)
    checked = (0, 1, 31, 63)
    kv = {}
    for c in sorted({x for t in checked for x in range(max(0, t - W), t + 1)}):
        kc = synth.tensor((n, H, d), synth.TAG_K, 64, c, 0)
        vc = synth.tensor((n, H, d), synth.TAG_V, 64, c, 0)
        kd[c * n:(c + 1) * n] = to_dev(kc, "bf16")
        vd[c * n:(c + 1) * n] = to_dev(vc, "bf16")
        kv[c] = (kc, vc)
    rows = list(range(0, n, 32)) + [n - 1]
    qs = {}
    for c in checked:
        qs[c] = synth.tensor_rows((n, H, d), rows, synth.TAG_Q, 64, c, 0)
        qd[[c * n + r for r in rows]] = to_dev(qs[c], "bf16")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, lse = bca.attend_sequence(qd, kd, vd, n, W, workspace=ws)
    torch.cuda.synchronize()
    for c in checked:
        hist = {x: kv[x] for x in range(max(0, c - W), c)}
        eo, el = oracle.attend(qs[c], kv[c][0], kv[c][1], hist, t=c, W=W,
                               scale=1.0 / math.sqrt(d), rows=list(range(len(rows))))
        go = to_np(o[c * n:(c + 1) * n])[rows]
        gl = to_np(lse[c])[:, rows]
        assert_close(go, gl, eo, el, TOL["bf16"], f"64-chunk clip, chunk {c}")


def test_sequence_refused_calls():
    import attention_bca_attend_amd as bca
    q = torch.zeros((32, 2, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((32, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bca.BcaError) as e:
        bca.attend_sequence(q, kv, kv, 16, -1)
    assert e.value.status == -1
    with pytest.raises(bca.BcaError) as e:
        bca.attend_sequence(q, kv, kv, 10, 1)  # 32 rows are not chunks of 10
    assert e.value.status == -1
    spec = bca.bca_sequence_spec(2, 64, 16, 2, 0, 1, 4, 0.125)
    need = bca.bca_attend_sequence_workspace_bytes(spec, bca.BF16)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(bca.BcaError) as e:
        bca.bca_attend_sequence(spec, q.data_ptr(), kv.data_ptr(), kv.data_ptr(), bca.BF16,
                                o.data_ptr(), 0, ws.data_ptr(), need - 256)
    assert e.value.status == -3
    with pytest.raises(bca.BcaError) as e:
        bca.bca_attend_sequence(spec, q.data_ptr(), kv.data_ptr(), kv.data_ptr(), bca.FP8_E4M3,
                                o.data_ptr(), 0, ws.data_ptr(), need)
    assert e.value.status == -4
