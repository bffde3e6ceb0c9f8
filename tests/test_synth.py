"""The seeded input generator (no GPU)."""
import numpy as np
import torch

import synth


def test_splitmix64_reference_values():
    # SplitMix64 from state 0: the first outputs published with the generator
    # (Steele, Lea and Flood 2014; also the seeding routine of xoshiro).
    got = synth.raw_u64(0, 0, 3)
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                     0x06C45D188009454F]


def test_counter_based_slices_agree():
    key = synth.stream_key(1, 2, 3)
    whole = synth.raw_u64(key, 0, 100)
    assert np.array_equal(whole[40:60], synth.raw_u64(key, 40, 20))


def test_streams_differ_and_repeat():
    a = synth.tensor((64, 2, 8), synth.TAG_K, 0, 1, 0)
    b = synth.tensor((64, 2, 8), synth.TAG_K, 0, 2, 0)
    c = synth.tensor((64, 2, 8), synth.TAG_K, 0, 1, 0)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_normal_moments():
    z = synth.normal(synth.stream_key(9), 200000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    assert abs((np.abs(z) > 3).mean() - 0.0027) < 0.0008


def test_bf16_rounding_matches_torch():
    x = synth.round_fp32(synth.normal(synth.stream_key(10), 50000) * 3.0)
    mine = synth.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)
    assert np.array_equal(synth.round_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_outliers_fraction_and_value():
    x = synth.tensor((100000,), synth.TAG_K, 5, 0, 0, dtype="fp32", outlier_frac=0.01)
    out = np.abs(x) == 8.0
    assert 0.008 < out.mean() < 0.012
    assert np.abs(x[~out]).max() < 8.0


def test_rows_of_a_tensor_drawn_alone():
    shape = (37, 3, 16)
    full = synth.tensor(shape, synth.TAG_Q, 2, 9, 1)
    rows = [0, 5, 36, 17]
    assert np.array_equal(synth.tensor_rows(shape, rows, synth.TAG_Q, 2, 9, 1), full[rows])
    full32 = synth.tensor(shape, synth.TAG_Q, 2, 9, 1, dtype="fp32")
    assert np.array_equal(synth.tensor_rows(shape, rows, synth.TAG_Q, 2, 9, 1, dtype="fp32"),
                          full32[rows])
