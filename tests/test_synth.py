"""The seeded input generator: reproducible, quantises as documented (CPU only)."""
import numpy as np
import torch

import oracle
import synth


def test_e4m3_encoder_matches_torch_including_ties():
    x = synth.normal(1, 9, 20000) * 60
    grid = oracle.decode_e4m3(np.arange(0x7F))             # positive codes
    mids = (grid[1:] + grid[:-1]) / 2                        # exact ties
    x = np.concatenate([x, mids, -mids, [448.0, -448.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = synth.encode_e4m3(x)
    # signed zeros may differ in sign bit only
    same = (got == ref) | ((got & 0x7F) == 0) & ((ref & 0x7F) == 0)
    assert same.all(), np.nonzero(~same)[0][:10]


def test_e4m3_encoder_saturates():
    assert synth.encode_e4m3(np.array([1e6, -1e6, 470.0])).tolist() == [0x7E, 0xFE, 0x7E]


def test_e2m1_encoder_ties_to_even():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.3, 0.1])
    assert synth.encode_e2m1(x).tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 9, 0]


def test_fp8_rows_scale_is_amax_over_448():
    codes, sc = synth.fp8_normal_rows(0, 1, 50, 128)
    x = synth.normal(0, 1, 50 * 128).reshape(50, 128)
    np.testing.assert_array_equal(sc, (np.abs(x).max(1) / 448).astype(np.float32))
    dec = oracle.decode_e4m3(codes)
    assert (np.abs(dec).max(1) == 448).all()


def test_mxfp4_rows_block_exponent():
    packed, e8 = synth.mxfp4_normal_rows(0, 2, 40, 128)
    x = synth.normal(0, 2, 40 * 128).reshape(40, 128, )
    amax = np.abs(x).reshape(40, 4, 32).max(-1)
    assert np.array_equal(e8.astype(int) - 127, np.floor(np.log2(amax)).astype(int) - 2)


def test_reproducible_and_seed_dependent():
    a = synth.make_problem(8, 300, 4, seed=0)
    b = synth.make_problem(8, 300, 4, seed=0)
    c = synth.make_problem(8, 300, 4, seed=1)
    for f in ("q", "q_scale", "k", "k_scale", "w"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.q, c.q)
    # a draw does not depend on how many values are requested
    assert np.array_equal(synth.normal(3, 4, 10), synth.normal(3, 4, 1000)[:10])
    assert np.array_equal(synth.normal(3, 4, 10, first=500), synth.normal(3, 4, 1000)[500:510])


def test_duplicate_rows_are_byte_copies():
    p = synth.make_problem(4, 1000, 4, k_fmt=synth.K_MXFP4, dup_rows=50)
    dst, src = p.meta["dup_dst"], p.meta["dup_src"]
    assert len(set(dst.tolist())) == 50 and not set(src.tolist()) & set(dst.tolist())
    assert np.array_equal(p.k[dst], p.k[src]) and np.array_equal(p.k_scale[dst], p.k_scale[src])
