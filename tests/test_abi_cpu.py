"""The C-ABI library on the host (no GPU): exports, descriptor arithmetic, the
slot table, window resolution, work planning and every error path that is
decided before a kernel is launched."""
import ctypes
import itertools
import os
import re

import pytest

import attention_bca_attend_amd as bca
from attention_bca_attend_amd import BcaError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bca.h")

# a 256-byte aligned stand-in for device memory: creating a cache never touches it
FAKE = 1 << 40


def declared_functions():
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc))
                   if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bca_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    lib = ctypes.CDLL(bca.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def desc(L=2, H=2, d=64, n=16, S=2, R=0, dt=bca.F32):
    return bca.bca_cache_desc(L, H, d, n, S, R, dt)


def make(**kw):
    dsc = desc(**kw)
    nb = bca.bca_cache_bytes(dsc)
    return bca.bca_cache_create(dsc, FAKE, nb), nb


def test_cache_bytes_formula():
    # [L][K|V][H][S+R][n][d]
    assert bca.bca_cache_bytes(desc(L=1, H=2, d=64, n=16, S=2, dt=bca.F32)) == 2 * 2 * 2 * 16 * 64 * 4
    assert bca.bca_cache_bytes(desc(L=30, H=12, d=128, n=1536, S=2, dt=bca.BF16)) == \
        30 * 2 * 12 * 2 * 1536 * 128 * 2
    assert bca.bca_cache_bytes(desc(L=30, H=24, d=128, n=405, S=20, R=1, dt=bca.FP8_E4M3)) == \
        30 * 2 * 24 * 21 * 405 * 128


@pytest.mark.parametrize("field,value", [("num_layers", 0), ("num_heads", 0), ("head_dim", 96),
                                         ("chunk_tokens", 0), ("ring_slots", 0),
                                         ("ring_slots", 63), ("has_ref", 2), ("kv_dtype", 7)])
def test_invalid_descriptor(field, value):
    d = desc()
    setattr(d, field, value)
    assert bca.bca_cache_bytes(d) == 0
    with pytest.raises(BcaError) as e:
        bca.bca_cache_create(d, FAKE, 1 << 30)
    assert e.value.status == -1


def test_fp8_descriptor_limits():
    assert bca.bca_cache_bytes(desc(H=65, d=128, dt=bca.FP8_E4M3)) == 0
    assert bca.bca_cache_bytes(desc(H=8, d=64, dt=bca.FP8_E4M3)) == 0
    assert bca.bca_cache_bytes(desc(H=8, d=128, dt=bca.FP8_E4M3)) > 0


def test_create_checks_memory():
    d = desc()
    nb = bca.bca_cache_bytes(d)
    for ptr, size in ((0, nb), (FAKE + 16, nb), (FAKE, nb - 1)):
        with pytest.raises(BcaError) as e:
            bca.bca_cache_create(d, ptr, size)
        assert e.value.status == -1
    h = bca.bca_cache_create(d, FAKE, nb)
    assert bca.bca_cache_slot_chunk(h, 0, 0) == -1
    bca.bca_cache_destroy(h)


def test_slot_table_hooks_and_plan():
    h, _ = make(S=3, R=1, dt=bca.BF16, d=128, n=100, H=3)
    for s in range(4):
        assert bca.bca_cache_slot_chunk(h, 1, s) == -1
    bca.bca_cache_set_slot_chunk(h, 1, 0, 6)
    bca.bca_cache_set_slot_chunk(h, 1, 1, 7)
    bca.bca_cache_set_slot_chunk(h, 1, 2, 5)
    bca.bca_cache_set_slot_chunk(h, 1, 3, 0)  # reference block
    with pytest.raises(BcaError):
        bca.bca_cache_set_slot_chunk(h, 1, 0, 7)  # 7 mod 3 != 0
    spec = bca.bca_window_spec(8, 2, 1, 1, 0.1)
    p = bca.bca_attend_plan(h, 1, spec)
    assert p["visible_blocks"] == [0, 1, 3, -1]  # slots with 6 and 7, the reference, current
    assert p["visible_chunk_ids"] == [6, 7, 0, -1]
    assert p["visible_keys"] == 400
    assert p["q_tiles"] == 1 and p["units"] == 3
    assert p["workgroups"] == 3 and p["max_pieces"] == 1 and not p["merge"]
    # without the reference
    p = bca.bca_attend_plan(h, 1, bca.bca_window_spec(8, 2, 0, 1, 0.1))
    assert p["visible_blocks"] == [0, 1, -1]
    # other layers are empty
    p = bca.bca_attend_plan(h, 0, bca.bca_window_spec(8, 2, 1, 1, 0.1))
    assert p["visible_blocks"] == [-1]
    bca.bca_cache_destroy(h)


def _ring_model(S, commits):
    """slot -> chunk id after appending `commits` in order (id mod S, newest wins)."""
    ring = {}
    for c in commits:
        ring[c % S] = c
    return ring


def test_window_resolution_brute_force():
    # Every ring of S <= 4 slots, every commit sequence of non-decreasing ids
    # (with repeats) drawn from 0..7 of length <= 4, every W <= S and t <= 10: the
    # visible set equals the committed ids in [t-W, t-1] whenever the window is
    # resident, and the call is refused otherwise.
    checked = 0
    for S in range(1, 5):
        h, _ = make(S=S, n=16, H=1, d=64)
        seqs = [()]
        for length in range(1, 5):
            seqs += [s for s in itertools.combinations_with_replacement(range(8), length)]
        for seq in seqs:
            ring = _ring_model(S, seq)
            for s in range(S):
                bca.bca_cache_set_slot_chunk(h, 0, s, ring.get(s, -1))
            newest = max(seq) if seq else -1
            committed = set(seq)
            for W in range(0, S + 1):
                for t in range(0, 11):
                    spec = bca.bca_window_spec(t, W, 0, 1, 0.125)
                    if newest >= 0 and newest >= t - W + S:
                        with pytest.raises(BcaError) as e:
                            bca.bca_attend_plan(h, 0, spec)
                        assert e.value.status == -2
                        continue
                    p = bca.bca_attend_plan(h, 0, spec)
                    got = sorted(c for c in p["visible_chunk_ids"] if c >= 0)
                    want = sorted(c for c in committed if t - W <= c <= t - 1)
                    assert got == want, (S, seq, W, t)
                    assert p["visible_keys"] == 16 * (len(want) + 1)
                    checked += 1
        bca.bca_cache_destroy(h)
    assert checked > 10000


def test_segment_planning():
    h, _ = make(S=20, R=1, dt=bca.BF16, d=128, n=405, H=24, L=1)
    for c in range(20, 40):
        bca.bca_cache_set_slot_chunk(h, 0, c % 20, c)
    bca.bca_cache_set_slot_chunk(h, 0, 20, 0)
    for G in (1, 2, 4, 7):
        p = bca.bca_attend_plan(h, 0, bca.bca_window_spec(40, 20, 1, G, 0.088))
        assert p["visible_keys"] == 22 * 405
        assert p["kv_tiles"] == -(-21 * 405 // 64) + -(-405 // 64)
        bm = -(-405 // p["q_tiles"])  # rows per query tile (a power of two >= this)
        assert p["q_tiles"] in (1, 2, 4, 7) and p["units"] == 24 * p["q_tiles"]
        assert p["workgroups"] == p["units"] * G
        assert p["max_pieces"] == G and p["merge"] == (G > 1)
        ws = bca.bca_attend_workspace_bytes(h, bca.bca_window_spec(40, 20, 1, G, 0.088))
        assert ws >= p["workspace_bytes"]
        if G > 1:
            assert p["workspace_bytes"] >= p["units"] * G * bm * 129 * 4
    # automatic split: never more work groups than tile iterations
    p = bca.bca_attend_plan(h, 0, bca.bca_window_spec(40, 20, 1, 0, 0.088))
    assert 1 <= p["workgroups"] <= p["units"] * p["kv_tiles"]
    bca.bca_cache_destroy(h)


def test_workspace_covers_every_occupancy():
    h, _ = make(S=2, dt=bca.BF16, d=128, n=1536, H=12, L=1)
    spec = bca.bca_window_spec(5, 2, 0, 0, 0.088)
    ws = bca.bca_attend_workspace_bytes(h, spec)
    for fill in range(3):
        for s in range(2):
            bca.bca_cache_set_slot_chunk(h, 0, s, -1)
        for c in range(5 - fill, 5):
            bca.bca_cache_set_slot_chunk(h, 0, c % 2, c)
        assert bca.bca_attend_plan(h, 0, spec)["workspace_bytes"] <= ws
    bca.bca_cache_destroy(h)


def test_workspace_only_for_split_units():
    """An unsplit bf16 plan needs no workspace; a split one holds the fp32
    partial outputs and LSEs of every piece."""
    h, _ = make(S=2, dt=bca.BF16, d=128, n=1536, H=12, L=1)
    for c in range(3, 5):
        bca.bca_cache_set_slot_chunk(h, 0, c % 2, c)
    p1 = bca.bca_attend_plan(h, 0, bca.bca_window_spec(5, 2, 0, 1, 0.088))
    assert p1["merge"] == 0 and p1["workspace_bytes"] == 0
    p3 = bca.bca_attend_plan(h, 0, bca.bca_window_spec(5, 2, 0, 3, 0.088))
    partial = p3["units"] * 3 * 256 * (128 + 1) * 4
    assert p3["merge"] == 1 and p3["workspace_bytes"] >= partial
    bca.bca_cache_destroy(h)


def test_append_errors_before_launch():
    h, _ = make(S=2, R=0, dt=bca.BF16, d=128, H=2, n=16)
    P = FAKE
    cases = [
        (dict(layer=2), -1), (dict(layer=-1), -1), (dict(chunk_id=-1), -1),
        (dict(is_ref=1), -1), (dict(k=0), -1), (dict(v=P + 8), -1),
        (dict(in_dtype=bca.F32), -4), (dict(in_dtype=9), -1),
    ]
    for over, status in cases:
        args = dict(layer=0, chunk_id=3, is_ref=0, k=P, v=P, in_dtype=bca.BF16)
        args.update(over)
        with pytest.raises(BcaError) as e:
            bca.bca_append_chunk(h, args["layer"], args["chunk_id"], args["is_ref"], args["k"],
                                 args["v"], args["in_dtype"], 0)
        assert e.value.status == status, over
    # out of order: a smaller id than the newest
    bca.bca_cache_set_slot_chunk(h, 0, 1, 5)
    with pytest.raises(BcaError) as e:
        bca.bca_append_chunk(h, 0, 4, 0, P, P, bca.BF16, 0)
    assert e.value.status == -2
    assert bca.bca_cache_slot_chunk(h, 0, 0) == -1 and bca.bca_cache_slot_chunk(h, 0, 1) == 5
    bca.bca_cache_destroy(h)


def test_attend_errors_before_launch():
    h, _ = make(S=2, R=0, dt=bca.BF16, d=128, H=2, n=300)
    P = FAKE

    def call(spec=None, layer=0, q=P, k=P, v=P, dt=bca.BF16, o=P, lse=0, ws=0, wsb=0):
        spec = spec or bca.bca_window_spec(2, 2, 0, 1, 0.1)
        bca.bca_attend(h, layer, spec, q, k, v, dt, o, lse, ws, wsb, 0)

    cases = [
        (dict(layer=3), -1),
        (dict(spec=bca.bca_window_spec(-1, 2, 0, 1, 0.1)), -1),
        (dict(spec=bca.bca_window_spec(2, 3, 0, 1, 0.1)), -1),       # W > S
        (dict(spec=bca.bca_window_spec(2, 2, 1, 1, 0.1)), -1),       # no reference block
        (dict(spec=bca.bca_window_spec(2, 2, 0, 65, 0.1)), -1),
        (dict(spec=bca.bca_window_spec(2, 2, 0, 1, float("nan"))), -1),
        (dict(dt=bca.F32), -4), (dict(dt=bca.FP8_E4M3), -4),
        (dict(q=0), -1), (dict(o=P + 2), -1),
        (dict(spec=bca.bca_window_spec(2, 2, 0, 4, 0.1)), -3),       # needs a workspace
        (dict(spec=bca.bca_window_spec(2, 2, 0, 4, 0.1), ws=P, wsb=16), -3),
    ]
    for over, status in cases:
        with pytest.raises(BcaError) as e:
            call(**over)
        assert e.value.status == status, over
    # residency: newest ring id 9 with S = 2 cannot serve query chunk 5
    bca.bca_cache_set_slot_chunk(h, 0, 1, 9)
    with pytest.raises(BcaError) as e:
        call(spec=bca.bca_window_spec(5, 2, 0, 1, 0.1))
    assert e.value.status == -2
    assert "overwritten" in bca.bca_last_error()
    bca.bca_cache_destroy(h)


def test_fp8_scales_validation_and_reset():
    h, _ = make(S=2, R=1, dt=bca.FP8_E4M3, d=128, H=3)
    bca.bca_cache_set_slot_chunk(h, 0, 0, 4)
    bca.bca_cache_set_slot_chunk(h, 0, 2, 0)
    bca.bca_cache_set_kv_scales(h, 0, [0.5, 1.0, 2.0], [1.0, 1.0, 1.0])
    # new scales empty the layer: stored codes used the old ones
    assert bca.bca_cache_slot_chunk(h, 0, 0) == -1 and bca.bca_cache_slot_chunk(h, 0, 2) == -1
    for bad in ([0.0, 1, 1], [float("inf"), 1, 1], [-1.0, 1, 1]):
        with pytest.raises(BcaError):
            bca.bca_cache_set_kv_scales(h, 0, bad, [1, 1, 1])
    with pytest.raises(BcaError):
        bca.bca_cache_set_kv_scales(h, 5, [1, 1, 1], [1, 1, 1])
    bca.bca_cache_destroy(h)
    h2, _ = make(S=2, dt=bca.BF16, d=128)
    with pytest.raises(BcaError):
        bca.bca_cache_set_kv_scales(h2, 0, [1, 1], [1, 1])
    bca.bca_cache_destroy(h2)


def test_status_strings():
    for code, name in bca.STATUS.items():
        assert bca.bca_status_string(code) == name


def test_one_hip_runtime_per_process():
    """Importing the package before torch must not map a second HIP or HSA
    runtime next to the one torch brings (both drive the same GPU)."""
    import subprocess
    import sys
    code = (
        "import attention_bca_attend_amd, torch, re\n"
        "libs = set()\n"
        "for line in open('/proc/self/maps'):\n"
        "    m = re.search(r'(/\\S*lib(amdhip64|hsa-runtime64)\\S*)', line)\n"
        "    if m: libs.add((m.group(2), m.group(1)))\n"
        "print(sorted(libs))\n"
        "kinds = [k for k, _ in libs]\n"
        "assert kinds.count('amdhip64') == 1 and kinds.count('hsa-runtime64') == 1, libs\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


def test_fp8_cache_plan_needs_the_chunk_copy():
    """An fp8 cache attends over the current chunk quantised into the
    workspace, so even an unsplit plan needs 2 H n d bytes of workspace."""
    H, d, n = 2, 128, 64
    h, _ = make(S=2, dt=bca.FP8_E4M3, d=d, H=H, n=n, L=1)
    spec = bca.bca_window_spec(0, 2, 0, 1, 0.088)
    p = bca.bca_attend_plan(h, 0, spec)
    assert p["merge"] == 0 and p["workspace_bytes"] >= 2 * H * n * d
    assert bca.bca_attend_workspace_bytes(h, spec) >= p["workspace_bytes"]
    with pytest.raises(BcaError) as e:
        bca.bca_attend(h, 0, spec, FAKE, FAKE, FAKE, bca.BF16, FAKE, 0, 0, 0, 0)
    assert e.value.status == -3
    bca.bca_cache_destroy(h)


def test_rope_entry_points_validate_before_launch():
    h, _ = make(S=2, R=0, dt=bca.BF16, d=128, H=2, n=16)
    P = FAKE
    for base, pos0 in ((float("nan"), 0), (float("inf"), 0), (0.0, 0), (-5.0, 0), (1e4, -1)):
        with pytest.raises(BcaError) as e:
            bca.bca_append_chunk_rope(h, 0, 3, 0, P, P, bca.BF16, base, pos0, 0)
        assert e.value.status == -1, (base, pos0)
    # the append checks of bca_append_chunk still apply
    with pytest.raises(BcaError) as e:
        bca.bca_append_chunk_rope(h, 0, 3, 0, P, P, bca.F32, 1e4, 0, 0)
    assert e.value.status == -4
    assert bca.bca_cache_slot_chunk(h, 0, 1) == -1  # nothing recorded
    spec = bca.bca_window_spec(2, 2, 0, 1, 0.1)
    need = bca.bca_attend_rope_workspace_bytes(h, spec)
    # two [n][H][d] bf16 copies on top of what bca_attend needs (none here)
    assert need == bca.bca_attend_workspace_bytes(h, spec) + 2 * 16 * 2 * 128 * 2
    for base, pos0 in ((float("nan"), 0), (0.0, 0), (1e4, -1)):
        with pytest.raises(BcaError) as e:
            bca.bca_attend_rope(h, 0, spec, P, P, P, bca.BF16, base, pos0, P, 0, P, need, 0)
        assert e.value.status == -1, (base, pos0)
    for ws, wsb in ((0, 0), (P, need - 1), (P + 16, need)):
        with pytest.raises(BcaError) as e:
            bca.bca_attend_rope(h, 0, spec, P, P, P, bca.BF16, 1e4, 0, P, 0, ws, wsb, 0)
        assert e.value.status == -3, (ws, wsb)
    bca.bca_cache_destroy(h)


def test_sequence_workspace_bounded_by_work_groups():
    """Partial outputs are indexed by work group (at most two per group), so a
    whole clip's workspace does not grow with its number of chunks: 64 chunks
    of 12 x 1200 tokens need what 8 need, below 200 MB. The Wan-shaped clips
    (12 x 1536) need none: their launch of groups is cut into ranges that all
    end on unit boundaries (252 work groups of 144 tiles for 8 chunks), so no
    unit is split and nothing is merged."""
    S = bca.bca_sequence_spec
    need = {C: bca.bca_attend_sequence_workspace_bytes(S(12, 128, 1200, C, 0, 2, 0, 0.088),
                                                      bca.BF16) for C in (8, 64)}
    assert 0 < need[64] == need[8] < 200e6, need
    # 256 work groups x 2 slots x 256 rows x (128 + 1) fp32
    assert need[64] <= 256 * 2 * 256 * 129 * 4 + 512
    for C in (8, 64):
        assert bca.bca_attend_sequence_workspace_bytes(S(12, 128, 1536, C, 0, 2, 0, 0.088),
                                                       bca.BF16) == 0, C


def test_partial_slots_fit_and_do_not_collide():
    """The kernels' partial-output indexing, checked on the host: work group w
    writes its part of unit u to slot spw*w + (u != first unit of w's range),
    the merge reads piece j of unit u from work group first_wg(u T) + j. Every
    slot written is below spw*P (the workspace holds spw*P slots), no two
    parts share a slot, and the merge reads exactly the slots written."""
    def rb(w, I, P):
        return w * I // P

    def first_wg(x, I, P):
        return ((x + 1) * P + I - 1) // I - 1

    cases = [(72, 72, 216), (48, 140, 192), (4464, 72, 256), (312, 8, 256), (7, 5, 33),
             (100, 3, 256), (1, 9, 9), (3, 4, 5), (256, 1, 256), (30, 7, 64)]
    for units, T, P in cases:
        I = units * T
        assert P <= I
        spw = 1 if (P >= units and P % units == 0) else 2
        written = {}
        for w in range(P):
            a, b = rb(w, I, P), rb(w + 1, I, P)
            u0 = a // T
            it = a
            while it < b:
                u = it // T
                t0 = it - u * T
                t1 = min(T, t0 + (b - it))
                if not (t0 == 0 and t1 == T):
                    slot = spw * w + (1 if u != u0 else 0)
                    assert slot < spw * P, (units, T, P, w, u)
                    assert slot not in written, (units, T, P, w, u)
                    written[slot] = (w, u)
                it += t1 - t0
        read = {}
        for u in range(units):
            w0 = first_wg(u * T, I, P)
            pieces = first_wg((u + 1) * T - 1, I, P) - w0 + 1
            if pieces <= 1:
                continue
            for j in range(pieces):
                slot = (spw * w0 + (1 if u != rb(w0, I, P) // T else 0)) if j == 0 \
                    else spw * (w0 + j)
                read[slot] = (w0 + j, u)
        assert read == written, (units, T, P)



def test_grouped_partial_slots_fit_and_do_not_collide():
    """The same indexing for a launch whose units differ in length (a
    bca_attend_sequence launch of groups: the chunks before the window is full
    and the steady block, units numbered group after group, one range of
    iterations per work group over all of them, two slots per work group).
    The unit of an iteration and the first iteration of a unit come from the
    group table as the kernels compute them; every slot written is below
    2 P, no two parts share one, and the merge reads exactly those."""
    def rb(w, I, P):
        return w * I // P

    def first_wg(x, I, P):
        return ((x + 1) * P + I - 1) // I - 1

    def table(groups):  # [(units, T)] -> [(iter0, units0, T)]
        out, it, u = [], 0, 0
        for units, T in groups:
            out.append((it, u, T))
            it += units * T
            u += units
        return out, it, u

    def unit_of_iter(tab, it):
        g = max(i for i, (i0, _, _) in enumerate(tab) if it >= i0)
        i0, u0, T = tab[g]
        return u0 + (it - i0) // T

    def unit_first_iter(tab, u):
        g = max(i for i, (_, u0, _) in enumerate(tab) if u >= u0)
        i0, u0, T = tab[g]
        return i0 + (u - u0) * T

    cases = [([(72, 24), (72, 48), (432, 72)], 256), ([(12, 3), (12, 5), (60, 7)], 256),
             ([(6, 1), (6, 2), (6, 3), (30, 4)], 17), ([(5, 9), (3, 2)], 7),
             ([(48, 8), (48, 15), (48, 22), (96, 29)], 192)]
    for groups, P in cases:
        tab, I, units = table(groups)
        P = min(P, I)
        spw = 2
        written = {}
        for w in range(P):
            a, b = rb(w, I, P), rb(w + 1, I, P)
            u_first = unit_of_iter(tab, a)
            it = a
            while it < b:
                g = max(i for i, (i0, _, _) in enumerate(tab) if it >= i0)
                i0, u0, T = tab[g]
                u = u0 + (it - i0) // T
                t0 = it - i0 - (u - u0) * T
                t1 = min(T, t0 + (b - it))
                if not (t0 == 0 and t1 == T):
                    slot = spw * w + (1 if u != u_first else 0)
                    assert slot < spw * P, (groups, P, w, u)
                    assert slot not in written, (groups, P, w, u)
                    written[slot] = (w, u)
                it += t1 - t0
        read = {}
        for u in range(units):
            w0 = first_wg(unit_first_iter(tab, u), I, P)
            pieces = first_wg(unit_first_iter(tab, u + 1) - 1, I, P) - w0 + 1
            if pieces <= 1:
                continue
            for j in range(pieces):
                slot = (spw * w0 + (1 if u != unit_of_iter(tab, rb(w0, I, P)) else 0)) if j == 0 \
                    else spw * (w0 + j)
                read[slot] = (w0 + j, u)
        assert read == written, (groups, P)

def test_sequence_entry_point_validates_before_launch():
    P = FAKE
    S = bca.bca_sequence_spec
    good = dict(num_heads=2, head_dim=128, chunk_tokens=300, num_chunks=4, prefix_tokens=0,
                history=1, num_segments=7, scale=0.1)
    spec = S(**good)
    need = bca.bca_attend_sequence_workspace_bytes(spec, bca.BF16)
    # chunks c >= 1 see 600 keys in 7 segments: the largest plan's partials
    # (2 heads x 2 query tiles x 7 pieces x 256 rows x (128 + 1) fp32)
    assert need >= 2 * 2 * 7 * 256 * 129 * 4
    assert bca.bca_attend_sequence_workspace_bytes(spec, bca.FP8_E4M3) == 0
    for field, value in (("num_heads", 0), ("chunk_tokens", 0), ("num_chunks", 0),
                         ("prefix_tokens", -1), ("history", -1), ("num_segments", 65),
                         ("scale", float("nan"))):
        bad = S(**{**good, field: value})
        assert bca.bca_attend_sequence_workspace_bytes(bad, bca.BF16) == 0, field
        with pytest.raises(BcaError) as e:
            bca.bca_attend_sequence(bad, P, P, P, bca.BF16, P, 0, P, need, 0)
        assert e.value.status == -1, field
    for dt, hd in ((bca.FP8_E4M3, 128), (bca.BF16, 96)):
        with pytest.raises(BcaError) as e:
            bca.bca_attend_sequence(S(**{**good, "head_dim": hd}), P, P, P, dt, P, 0, P, need, 0)
        assert e.value.status == -4, (dt, hd)
    with pytest.raises(BcaError) as e:
        bca.bca_attend_sequence(spec, 0, P, P, bca.BF16, P, 0, P, need, 0)
    assert e.value.status == -1
    for ws, wsb in ((0, 0), (P, need - 1), (P + 16, need)):
        with pytest.raises(BcaError) as e:
            bca.bca_attend_sequence(spec, P, P, P, bca.BF16, P, 0, ws, wsb, 0)
        assert e.value.status == -3, (ws, wsb)
    # K/V spans beyond the kernels' 32-bit offsets are refused
    huge = S(**{**good, "chunk_tokens": 1 << 20, "num_chunks": 8})
    with pytest.raises(BcaError) as e:
        bca.bca_attend_sequence(huge, P, P, P, bca.BF16, P, 0, P, 1 << 40, 0)
    assert e.value.status == -1


def test_replay_entry_points_validate_before_launch():
    h, _ = make(S=2, R=0, dt=bca.BF16, d=128, H=2, n=16)
    P = FAKE
    for ptr in (0, P + 4):
        with pytest.raises(BcaError) as e:
            bca.bca_append_chunk_dev(h, 0, ptr, P, P, bca.BF16, 0)
        assert e.value.status == -1
        with pytest.raises(BcaError) as e:
            bca.bca_chunk_counter_advance(ptr, 0)
        assert e.value.status == -1
    with pytest.raises(BcaError) as e:
        bca.bca_append_chunk_dev(h, 2, P, P, P, bca.BF16, 0)  # layer out of range
    assert e.value.status == -1
    with pytest.raises(BcaError) as e:
        bca.bca_append_chunk_dev(h, 0, P, P, P, bca.F32, 0)
    assert e.value.status == -4
    bca.bca_cache_destroy(h)


def test_attend_replayable_rule():
    # host-only: slot contents declared through the restore hook
    h, _ = make(S=2, R=1, dt=bca.BF16, d=128, H=2, n=16)
    spec = lambda t, W, ref=0: bca.bca_window_spec(t, W, ref, 0, 0.1)  # noqa: E731
    assert not bca.bca_attend_replayable(h, 0, spec(2, 2))  # empty ring
    bca.bca_cache_set_slot_chunk(h, 0, 0, 0)
    assert not bca.bca_attend_replayable(h, 0, spec(2, 2))  # slot 1 still empty
    bca.bca_cache_set_slot_chunk(h, 0, 1, 1)
    assert bca.bca_attend_replayable(h, 0, spec(2, 2))      # chunks 0, 1 for t = 2
    assert not bca.bca_attend_replayable(h, 0, spec(2, 1))  # window smaller than the ring
    assert not bca.bca_attend_replayable(h, 0, spec(3, 2))  # chunk 0 is outside t = 3's window
    assert not bca.bca_attend_replayable(h, 0, spec(2, 2, ref=1))  # no reference appended
    bca.bca_cache_set_slot_chunk(h, 0, 2, 0)                # declare the reference
    assert bca.bca_attend_replayable(h, 0, spec(2, 2, ref=1))
    assert not bca.bca_attend_replayable(h, 1, spec(2, 2))  # layer 1 is empty
    with pytest.raises(BcaError):
        bca.bca_attend_replayable(h, 0, spec(2, 3))          # history > ring slots
    bca.bca_cache_destroy(h)


def test_replay_guards_refuse_empty_slots_at_the_stream_start():
    # With t < S the lower bound t - S is negative, so an empty slot (-1) must
    # be refused on its own: a plan captured there would hold fewer blocks
    # than every later chunk sees.
    h, _ = make(S=2, R=0, dt=bca.BF16, d=128, H=2, n=16)
    spec = lambda t, W: bca.bca_window_spec(t, W, 0, 0, 0.1)  # noqa: E731
    assert not bca.bca_attend_replayable(h, 0, spec(0, 2))  # empty ring, t = 0
    assert not bca.bca_attend_replayable(h, 0, spec(1, 2))  # empty ring, t = 1
    bca.bca_cache_set_slot_chunk(h, 0, 0, 0)
    assert not bca.bca_attend_replayable(h, 0, spec(1, 2))  # slot 1 still empty
    bca.bca_cache_set_slot_chunk(h, 0, 1, 1)
    assert bca.bca_attend_replayable(h, 0, spec(2, 2))
    bca.bca_cache_destroy(h)
    P = FAKE
    h, _ = make(S=3, R=0, dt=bca.BF16, d=128, H=2, n=16)
    for t, filled in ((0, 0), (1, 0), (1, 1), (2, 2)):
        for sl in range(3):
            bca.bca_cache_set_slot_chunk(h, 0, sl, sl if sl < filled else -1)
        sp = bca.bca_window_spec(t, 2, 0, 0, 0.1)
        ws = bca.bca_attend_workspace_bytes(h, sp)
        with pytest.raises(BcaError) as e:
            bca.bca_attend_dev(h, 0, sp, P, P, P, P, bca.BF16, P, 0, P, ws, 0)
        assert e.value.status == -1, (t, filled)
    bca.bca_cache_destroy(h)


def test_descriptor_limits_of_32_bit_offsets():
    # one head's cache blocks: (S+R) * n * d * es bytes must stay below 2 GiB
    over = bca.bca_cache_desc(1, 1, 128, 140000, 62, 0, bca.BF16)  # 62 * 140000 * 256 B ≈ 2.22 GB
    assert bca.bca_cache_bytes(over) == 0
    ok = bca.bca_cache_desc(1, 1, 128, 1 << 16, 62, 0, bca.BF16)  # ≈ 1.04 GB
    assert bca.bca_cache_bytes(ok) > 0
    # one chunk's q/k/v rows: n * H * d * 2 bytes (bf16) must stay below 2 GiB
    big = bca.bca_cache_desc(1, 64, 128, 1 << 17, 1, 0, bca.BF16)  # 2^17 * 64 * 256 B = 2 GiB
    assert bca.bca_cache_bytes(big) == 0
    assert bca.bca_cache_bytes(bca.bca_cache_desc(1, 32, 128, 1 << 17, 1, 0, bca.BF16)) > 0


@pytest.mark.parametrize("B", [bca.FP8_E4M3_BLOCK, bca.INT8K_FP8V_BLOCK])
def test_block_scaled_fp8_cache_on_the_host(B):
    d = bca.bca_cache_desc(3, 4, 128, 405, 20, 1, B)
    table = ((3 * 2 * 21 * 4 * 4 + 255) // 256) * 256
    assert bca.bca_cache_bytes(d) == 3 * 2 * 4 * 21 * 405 * 128 + table
    assert bca.bca_cache_bytes(bca.bca_cache_desc(1, 4, 64, 16, 2, 0, B)) == 0  # head_dim 128 only
    h = bca.bca_cache_create(d, FAKE, bca.bca_cache_bytes(d))
    with pytest.raises(BcaError) as e:
        bca.bca_cache_set_kv_scales(h, 0, [1.0] * 4, [1.0] * 4)
    assert e.value.status == -4
    # rotary appends and attends are accepted on these caches (the GPU tests
    # run them); here only checks that fail before any launch
    with pytest.raises(BcaError) as e:
        bca.bca_append_chunk_rope(h, 0, 0, 0, FAKE, FAKE, bca.BF16, float("nan"), 0, 0)
    assert e.value.status == -1
    for sl in range(20):
        bca.bca_cache_set_slot_chunk(h, 0, sl, sl)
    bca.bca_cache_set_slot_chunk(h, 0, 20, 0)
    spec = bca.bca_window_spec(20, 20, 1, 4, 0.1)
    plan = bca.bca_attend_plan(h, 0, spec)
    # every visible block padded to whole 64-key tiles: 21 cache blocks x 7 + 7
    assert plan["kv_tiles"] == 22 * 7 and plan["visible_keys"] == 22 * 405, plan
    need = bca.bca_attend_workspace_bytes(h, spec)
    assert need == plan["workspace_bytes"] and need >= 2 * 4 * 405 * 128 + 2 * 4 * 4
    rneed = bca.bca_attend_rope_workspace_bytes(h, spec)
    assert rneed >= need + 2 * 405 * 4 * 128 * 2  # the rotated Q and K copies on top
    with pytest.raises(BcaError) as e:
        bca.bca_attend_rope(h, 0, spec, FAKE, FAKE, FAKE, bca.BF16, 1e4, 0, FAKE, 0, FAKE,
                            rneed - 1, 0)
    assert e.value.status == -3
    bca.bca_cache_destroy(h)


def test_header_compiles_as_c99_and_links(tmp_path):
    """include/bca.h is plain C: a C99 program using it compiles with warnings
    as errors, links against libbca.so and makes host-only calls."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = os.path.join(tmp_path, "abi_host_calls")
    libdir = os.path.dirname(bca.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(root, "include"), os.path.join(root, "tests", "c", "abi_host_calls.c"),
           "-o", exe, "-L", libdir, "-l:libbca.so", "-Wl,-rpath," + libdir,
           "-Wl,-rpath-link,/opt/rocm/lib", "-Wl,--allow-shlib-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_attend_dev_validates_before_launch():
    P = FAKE
    h, _ = make(S=3, R=0, dt=bca.BF16, d=128, H=2, n=16)
    spec = bca.bca_window_spec(3, 2, 0, 0, 0.1)
    ws = bca.bca_attend_workspace_bytes(h, spec)
    with pytest.raises(BcaError) as e:  # ring not yet holding chunks 0..2
        bca.bca_attend_dev(h, 0, spec, P, P, P, P, bca.BF16, P, 0, P, ws, 0)
    assert e.value.status == -1
    for sl in range(3):
        bca.bca_cache_set_slot_chunk(h, 0, sl, sl)
    for ptr in (0, P + 4):
        with pytest.raises(BcaError) as e:
            bca.bca_attend_dev(h, 0, spec, ptr, P, P, P, bca.BF16, P, 0, P, ws, 0)
        assert e.value.status == -1
    assert ws > 0  # two units spread over the chip: split, so partials need room
    with pytest.raises(BcaError) as e:  # the workspace checks of bca_attend still apply
        bca.bca_attend_dev(h, 0, spec, P, P, P, P, bca.BF16, P, 0, P + 16, ws, 0)
    assert e.value.status == -3
    bca.bca_cache_destroy(h)
    # an fp32 cache is refused; the 8-bit caches (per-head and per-block
    # scales) pass the dtype check and stop at the next one (a misaligned id)
    hf, _ = make(S=3, R=0, dt=bca.F32, d=64, H=2, n=16)
    for sl in range(3):
        bca.bca_cache_set_slot_chunk(hf, 0, sl, sl)
    with pytest.raises(BcaError) as e:
        bca.bca_attend_dev(hf, 0, spec, P, P, P, P, bca.F32, P, 0, P, 1 << 30, 0)
    assert e.value.status == -4
    bca.bca_cache_destroy(hf)
    for dt in (bca.FP8_E4M3, bca.FP8_E4M3_BLOCK, bca.INT8K_FP8V_BLOCK):
        h8, _ = make(S=3, R=0, dt=dt, d=128, H=2, n=16)
        for sl in range(3):
            bca.bca_cache_set_slot_chunk(h8, 0, sl, sl)
        with pytest.raises(BcaError) as e:
            bca.bca_attend_dev(h8, 0, spec, P + 4, P, P, P, bca.BF16, P, 0, P, 1 << 30, 0)
        assert e.value.status == -1, dt
        bca.bca_cache_destroy(h8)
