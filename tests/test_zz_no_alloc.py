"""bca_attend_noalloc (scratch owned by the library, no workspace argument)
against bca_attend with a caller-allocated workspace: the same plan and
kernels on the same inputs, so the outputs must be bit-identical. Two calls
in a row share the GPU's scratch, the second with a smaller input on another
cache (8-bit, so the scratch also holds the e4m3 copy of the chunk); both
are also held to the oracle."""
import math

import numpy as np
import pytest

import oracle
from bca_harness import TOL, Sequence, assert_close, assert_fp8, log, to_dev, to_np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_bca_attend_amd  # noqa: F401  (fails loudly when libbca.so is missing)
    yield


def _noalloc(cache, layer, q, k, v, spec):
    import attention_bca_attend_amd as bca
    o = torch.empty_like(q)
    lse = torch.empty((cache.desc.num_heads, cache.desc.chunk_tokens), dtype=torch.float32,
                      device=q.device)
    bca.bca_attend_noalloc(cache.handle, layer, spec, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           bca.BF16, o.data_ptr(), lse.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    return o, lse


def test_noalloc_equals_attend_on_two_calls():
    import attention_bca_attend_amd as bca
    # call 1: the Wan-shaped chunk (12 heads x 1536 tokens, 4608 keys), split
    # into pieces whose partial outputs live in the scratch
    H, d, n, S, W = 12, 128, 1536, 2, 2
    big = bca.Cache(1, H, d, n, S, kv_dtype="bf16")
    seq = Sequence(big, H, d, n, "bf16", seed_layer=90)
    for t in range(2):
        _, k, v = seq.chunk(t)
        seq.append(0, t, k, v)
    q, k, v = seq.chunk(2)
    spec = big.spec(2, W, num_segments=0)
    plan = big.plan(0, spec)
    assert plan["merge"] == 1 and 0 < plan["workspace_bytes"] <= bca.NOALLOC_SCRATCH_BYTES, plan
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o1, l1 = _noalloc(big, 0, qd, kd, vd, spec)
    o2, l2 = big.attend(0, qd, kd, vd, spec)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rows = list(range(0, n, 64))
    eo, el = oracle.attend(q, k, v, seq.history, t=2, W=W, scale=1 / math.sqrt(d), rows=rows)
    assert_close(to_np(o1)[rows], to_np(l1)[:, rows], eo, el, TOL["bf16"], "noalloc Wan shape")

    # call 2: a smaller chunk on an e4m3 cache with a split window
    H, n, S = 4, 100, 3
    small = bca.Cache(1, H, d, n, S, has_ref=True, kv_dtype="fp8")
    sc = [8.0 / 448.0] * H
    seq2 = Sequence(small, H, d, n, "fp8", seed_layer=91, outlier_frac=0.01, scales=(sc, sc))
    _, rk, rv = seq2.chunk(5000)
    seq2.append(0, 0, rk, rv, is_ref=True)
    for t in range(2):
        _, k, v = seq2.chunk(t)
        seq2.append(0, t, k, v)
    q, k, v = seq2.chunk(2)
    spec = small.spec(2, W, use_ref=True, num_segments=3)
    assert small.plan(0, spec)["workspace_bytes"] < plan["workspace_bytes"]
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o1, l1 = _noalloc(small, 0, qd, kd, vd, spec)
    o2, l2 = small.attend(0, qd, kd, vd, spec)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert_fp8(seq2, to_np(o1), to_np(l1), 2, q, k, v, W, use_ref=True, what="noalloc e4m3")
    log("bca_attend_noalloc: two calls bit-identical to bca_attend")


def test_noalloc_refuses_calls_beyond_the_scratch():
    import attention_bca_attend_amd as bca
    # 64 heads x 4096 tokens, 62-slot window, 64 segments: partials beyond the scratch
    cache = bca.Cache(1, 64, 128, 4096, 2, kv_dtype="bf16")
    spec = cache.spec(2, 2, num_segments=64)
    for t in range(2):
        cache.set_slot_chunk(0, t, t)
    assert cache.plan(0, spec)["workspace_bytes"] > bca.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((4096, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bca.BcaError) as e:
        _noalloc(cache, 0, x, x, x, spec)
    assert e.value.status == -3 and "scratch" in e.value.message
