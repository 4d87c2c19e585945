"""Pins of the fp64 CPU oracle (oracle/oracle.cpp) against things other than itself:
library decoders, hand-worked fixtures (tests/golden), numpy's fp64 einsum and sort
on small inputs, closed forms, invariants and the pages' key-blocked top-k identity.
CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- decoders
def test_e4m3_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_landmarks():
    d = oracle.decode_e4m3
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x08) == 2.0 ** -6 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x3C) == 1.5 and d(0x40) == 2.0
    pos = d(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()  # positive codes are monotone


def test_e2m1_table():
    # OCP MX v1.0 FP4 E2M1 magnitudes for codes 0..7; code | 8 is the negative.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.decode_e2m1(np.arange(16))
    assert np.array_equal(got[:8], mags)
    assert np.array_equal(got[8:], -np.array(mags))


def test_e8m0_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


# ----------------------------------------------------------------- hand fixtures
def _problem_from_fixture(g):
    T, H, D, L = g["T"], g["H"], g["D"], g["L"]
    q = np.zeros((T, H, D), np.uint8)
    for t, h, d, c in g["q_entries"]:
        q[t, h, d] = c
    if g["k_fmt"] == 0:
        k = np.zeros((L, D), np.uint8)
        for s, d, c in g["k_entries"]:
            k[s, d] = c
        ksc = np.array(g["k_scale"], np.float32)
    else:
        k = np.zeros((L, D // 2), np.uint8)
        for s, b, v in g["k_bytes"]:
            k[s, b] = v
        ksc = np.array(g["k_e8m0"], np.uint8)
    return synth.Problem(q=q, q_scale=np.array(g["q_scale"], np.float32), k=k, k_scale=ksc,
                         k_fmt=g["k_fmt"], w=np.array(g["w"], np.float32),
                         ks=np.array(g["ks"], np.int32), ke=np.array(g["ke"], np.int32),
                         scale=g["scale"])


def test_hand_fp8_fixture():
    g = _load("hand_fp8_logits.json")
    p = _problem_from_fixture(g)
    dq = oracle.Dequantised(p)
    dense = oracle.dense_logits(dq, range(p.T), g["dense_W"])
    assert np.array_equal(dense, np.array(g["dense"]))
    for K, want in g["topk"].items():
        idx, val, _ = oracle.topk(dq, range(p.T), int(K))
        assert idx.tolist() == want, (K, idx)


def test_hand_mxfp4_fixture():
    g = _load("hand_mxfp4_logits.json")
    p = _problem_from_fixture(g)
    dq = oracle.Dequantised(p)
    assert np.array_equal(oracle.dense_logits(dq, [0], 1), np.array(g["dense"]))


def test_hand_candidates_fixture():
    g = _load("hand_candidates.json")
    v = np.array(g["logits"], np.float64)
    assert np.array_equal(oracle.pool_row(v, g["pool"]), g["pooled"])
    for c in g["cases"]:
        mask, blocks = oracle.block_candidates_row(v, g["pool"], c["n_blocks"], g["W"])
        assert blocks.tolist() == c["blocks"]
        assert np.nonzero(mask)[0].tolist() == c["mask_ones"]
    m = g["masked_topk"]
    mask, _ = oracle.block_candidates_row(v, g["pool"], m["n_blocks"], g["W"])
    idx, _ = oracle.topk_row(v, 0, m["K"], mask[:len(v)].astype(bool))
    assert idx.tolist() == m["idx"]


# ----------------------------------------------------------------- closed forms / invariants
def _small(T=5, L=300, H=4, k_fmt=0, seed=3, **kw):
    return synth.make_problem(T, L, H, k_fmt=k_fmt, seed=seed, **kw)


def test_one_hot_closed_form():
    # q[t,h] = a_h e_{d1}, k[s] = b_s e_{d2}: I = sum_h w_h max(0, a_h b_s) if d1 == d2 else 0.
    T, H, D, L = 1, 3, 128, 6
    a_codes = [0x38, 0xB8, 0x44]        # 1, -1, 3
    b_codes = [0x40, 0xC0, 0x30, 0x00, 0x3C, 0xBC]  # 2, -2, .5, 0, 1.5, -1.5
    w = np.array([[0.5, 2.0, 0.25]], np.float32)
    for d1, d2 in [(7, 7), (7, 8)]:
        q = np.zeros((T, H, D), np.uint8)
        q[0, :, d1] = a_codes
        k = np.zeros((L, D), np.uint8)
        k[:, d2] = b_codes
        p = synth.Problem(q=q, q_scale=np.ones((T, H), np.float32), k=k, k_scale=np.ones(L, np.float32),
                          k_fmt=0, w=w, ks=np.array([0], np.int32), ke=np.array([L], np.int32))
        got = oracle.row_logits(oracle.Dequantised(p), 0)
        a = oracle.decode_e4m3(a_codes)
        b = oracle.decode_e4m3(b_codes)
        want = (w[0][:, None] * np.maximum(a[:, None] * b[None, :], 0)).sum(0) if d1 == d2 else np.zeros(L)
        assert np.array_equal(got, want)


def test_nonnegative_inputs_are_linear():
    # With q, k >= 0 every head dot is >= 0, so the ReLU is the identity and
    # I[t, s] = <sum_h w_h qd[t, h], kd[s]>: a different contraction order.
    p = _small(T=3, L=200, H=6)
    p.q = np.where(p.q & 0x80, p.q & 0x7F, p.q).astype(np.uint8)
    p.k = np.where(p.k & 0x80, p.k & 0x7F, p.k).astype(np.uint8)
    dq = oracle.Dequantised(p)
    for t in range(p.T):
        got = oracle.row_logits(dq, t)
        qsum = (dq.w[t][:, None] * dq.qd[t]).sum(0)
        want = dq.kd[dq.ks[t]:dq.ke[t]] @ qsum
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_relu_kills_negated_heads():
    # Negating every q code of one head flips the sign of its dots; the sum of
    # the two variants' contributions equals w_h * |dot| per key.
    p = _small(T=1, L=400, H=2)
    dq = oracle.Dequantised(p)
    base = oracle.row_logits(dq, 0)
    p2 = synth.Problem(**{**p.__dict__})
    p2.q = p.q.copy()
    p2.q[0, 1] ^= 0x80
    p2.q[0, 1][p.q[0, 1] == 0] = 0
    neg = oracle.row_logits(oracle.Dequantised(p2), 0)
    d1 = dq.qd[0, 1] @ dq.kd[:dq.ke[0]].T
    np.testing.assert_allclose(base - neg, dq.w[0, 1] * d1, rtol=1e-12, atol=1e-9)


def test_scale_homogeneity_and_head_permutation():
    p = _small(T=4, L=256, H=8)
    W = oracle.Dequantised(p).W
    base = oracle.dense_logits(oracle.Dequantised(p), range(p.T), W)
    for field in ("w", "k_scale", "q_scale"):
        p2 = synth.Problem(**{**p.__dict__})
        setattr(p2, field, getattr(p, field) * np.float32(2))
        got = oracle.dense_logits(oracle.Dequantised(p2), range(p.T), W)
        assert np.array_equal(got, 2 * base), field
    p2 = synth.Problem(**{**p.__dict__})
    p2.scale = 4.0
    assert np.array_equal(oracle.dense_logits(oracle.Dequantised(p2), range(p.T), W), 4 * base)
    perm = np.random.default_rng(0).permutation(p.H)
    p3 = synth.Problem(**{**p.__dict__})
    p3.q, p3.q_scale, p3.w = p.q[:, perm], p.q_scale[:, perm], p.w[:, perm]
    np.testing.assert_allclose(oracle.dense_logits(oracle.Dequantised(p3), range(p.T), W), base,
                               rtol=1e-12)
    # weights permuted alone must change the result (w is tied to its head)
    p4 = synth.Problem(**{**p.__dict__})
    p4.w = p.w[:, perm]
    assert not np.allclose(oracle.dense_logits(oracle.Dequantised(p4), range(p.T), W), base)


def test_key_permutation_equivariance():
    p = _small(T=1, L=300, H=4, ks=np.array([0], np.int32), ke=np.array([300], np.int32))
    base = oracle.row_logits(oracle.Dequantised(p), 0)
    perm = np.random.default_rng(1).permutation(p.L)
    p2 = synth.Problem(**{**p.__dict__})
    p2.k, p2.k_scale = p.k[perm], p.k_scale[perm]
    got = oracle.row_logits(oracle.Dequantised(p2), 0)
    np.testing.assert_allclose(got, base[perm], rtol=1e-13)


def test_mxfp4_equals_fp8_when_representable():
    # An MXFP4 key whose dequantised values are exactly fp8-representable gives the
    # same logits as the fp8 key holding those values (scales folded into codes).
    p = _small(T=3, L=64, H=4, k_fmt=1, seed=5)
    kd = oracle.dequant_k(p.k, p.k_scale, 1)
    s = np.exp2(np.floor(np.log2(np.abs(kd).max(axis=1) + 1e-300)) - 5)   # per-row power of two
    codes = synth.encode_e4m3(kd / s[:, None])
    assert np.array_equal(oracle.decode_e4m3(codes) * s[:, None], kd)   # exact re-encoding
    p8 = synth.Problem(**{**p.__dict__})
    p8.k, p8.k_scale, p8.k_fmt = codes, s.astype(np.float32), 0
    W = oracle.Dequantised(p).W
    a = oracle.dense_logits(oracle.Dequantised(p), range(p.T), W)
    b = oracle.dense_logits(oracle.Dequantised(p8), range(p.T), W)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_windows_bound_the_row():
    p = _small(T=6, L=500, H=2)
    dq = oracle.Dequantised(p)
    for t in range(p.T):
        v = oracle.row_logits(dq, t)
        assert len(v) == dq.ke[t] - dq.ks[t] == p.L - p.T + t + 1
    # shrinking a window from either side keeps the surviving keys' logits
    full = oracle.row_logits(dq, 5)
    p2 = synth.Problem(**{**p.__dict__})
    p2.ks = dq.ks.astype(np.int32)
    p2.ke = dq.ke.astype(np.int32)
    p2.ks[5], p2.ke[5] = 17, 311
    part = oracle.row_logits(oracle.Dequantised(p2), 5)
    assert np.array_equal(part, full[17:311])


# ----------------------------------------------------------------- top-K
def _is_topk(v32, sel, n):
    """Set characterisation: every selected (v, -j) beats every unselected (v, -j)."""
    s = np.zeros(n, bool)
    s[sel] = True
    if s.all() or not s.any():
        return True
    key_v = v32.astype(np.float64)
    j = np.arange(n)
    # worst selected: smallest value, then largest index; best unselected: largest value, then smallest index
    ws = np.lexsort((-j[s], key_v[s]))[0]
    bu = np.lexsort((j[~s], -key_v[~s]))[0]
    a = (key_v[s][ws], -j[s][ws])
    b = (key_v[~s][bu], -j[~s][bu])
    return a > b


@pytest.mark.parametrize("n,K", [(50, 7), (1000, 64), (33, 33), (10, 40)])
def test_topk_set_characterisation(n, K):
    rng = np.random.default_rng(n * 7 + K)
    v = rng.normal(size=n)
    v[rng.integers(0, n, n // 5)] = 0.5        # exact ties
    idx, val = oracle.topk_row(v, 100, K)
    sel = idx[idx >= 0] - 100
    assert len(sel) == min(n, K)
    assert (np.diff(sel) > 0).all() and (idx[len(sel):] == -1).all()
    assert _is_topk(v.astype(np.float32), sel, n)
    assert np.array_equal(val[:len(sel)], v[sel].astype(np.float32))


def test_topk_all_equal_takes_lowest_indices():
    idx, _ = oracle.topk_row(np.full(100, 3.25), 40, 10)
    assert idx.tolist() == list(range(40, 50))


def test_topk_fp32_decision():
    # Two scores that differ in fp64 but round to the same fp32 tie, and the lower key wins.
    a = 1.0
    b = 1.0 + 2.0 ** -30
    assert np.float32(a) == np.float32(b)
    idx, _ = oracle.topk_row(np.array([a, b, 0.0]), 0, 1)
    assert idx.tolist() == [0]


def test_block_merge_identity():
    # P1 section 2.3: topk(union) == topk(union of per-block topk), for any blocking.
    rng = np.random.default_rng(11)
    for trial in range(20):
        n = int(rng.integers(1, 3000))
        K = int(rng.integers(1, 300))
        v = np.round(rng.normal(size=n), 2)      # many exact ties
        full, _ = oracle.topk_row(v, 0, K)
        bk = int(rng.integers(1, 700))
        cand = []
        for b0 in range(0, n, bk):
            i, _ = oracle.topk_row(v[b0:b0 + bk], b0, K)
            cand.extend(i[i >= 0].tolist())
        cand = np.array(sorted(cand))
        sub, _ = oracle.topk_row(v[cand], 0, K)
        merged = np.full(K, -1, np.int32)
        s = cand[sub[sub >= 0]]
        merged[:len(s)] = s
        assert np.array_equal(merged, full), trial


def test_masked_topk_never_selects_masked_and_pads():
    rng = np.random.default_rng(2)
    v = rng.normal(size=500)
    allowed = rng.random(500) < 0.03
    idx, _ = oracle.topk_row(v, 7, 64, allowed)
    sel = idx[idx >= 0] - 7
    assert allowed[sel].all()
    assert len(sel) == allowed.sum() < 64
    assert (idx[len(sel):] == -1).all()


# ----------------------------------------------------------------- candidates
def test_candidates_counts_and_noop_invariant():
    p = _small(T=6, L=3000, H=4, seed=9)
    dq = oracle.Dequantised(p)
    K = 64
    for t in range(p.T):
        v = oracle.row_logits(dq, t)
        for nb in (16, 64, 1000):
            mask, blocks = oracle.block_candidates_row(v, 8, nb, dq.W)
            assert len(blocks) == min(nb, -(-len(v) // 8))
            assert not mask[len(v):].any()
            assert mask.sum() == sum(min(8, len(v) - 8 * b) for b in blocks)
            if nb >= K:
                # each selected key's block has max >= v_K, so at most K blocks precede or tie it:
                # masking with the candidates of the same logits is a no-op for top-K (K <= n_blocks)
                a, _ = oracle.topk_row(v, dq.ks[t], K, mask[:len(v)].astype(bool))
                b, _ = oracle.topk_row(v, dq.ks[t], K)
                assert np.array_equal(a, b)


def test_partial_last_block_pools_valid_keys_only():
    v = np.array([1.0] * 8 + [5.0, -2.0])  # last block = keys 8, 9
    P = oracle.pool_row(v, 8)
    assert P.tolist() == [1.0, 5.0]
    mask, blocks = oracle.block_candidates_row(v, 8, 1, 16)
    assert blocks.tolist() == [1] and np.nonzero(mask)[0].tolist() == [8, 9]


def test_ratio_windows_hand_example():
    """Worked by hand: request 0 has 10 tokens (3 new), request 1 has 7 (2 new); ratio 2
    gives 5 and 3 keys.  Rows see 8, 9, 10 and 6, 7 tokens: 4, 4, 5 and 3, 3 keys."""
    ks, ke = oracle.ragged_windows([0, 3, 5], [0, 10, 17], [0, 5, 8], ratio=2)
    assert ks.tolist() == [0, 0, 0, 5, 5]
    assert ke.tolist() == [4, 4, 5, 8, 8]


def test_ratio_windows_invariants():
    """Ratio 1 is the plain causal tail; for any ratio the window grows by one key
    exactly when a group completes, and the last row of a request whose length is a
    multiple of the ratio sees all of its keys."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        B = int(rng.integers(1, 6))
        lq = rng.integers(1, 40, B)
        lk = lq + rng.integers(0, 300, B)
        cu_q = np.concatenate([[0], np.cumsum(lq)])
        cu_k = np.concatenate([[0], np.cumsum(lk)])
        ks, ke = oracle.ragged_windows(cu_q, cu_k)
        for i in range(B):
            rows = slice(cu_q[i], cu_q[i + 1])
            assert (ks[rows] == cu_k[i]).all()
            assert ke[cu_q[i + 1] - 1] == cu_k[i + 1]          # the newest row sees every token
            assert (np.diff(ke[rows]) == 1).all()
        for r in (2, 4, 7):
            lk_r = lk - lk % r                                 # whole groups only
            lk_r = np.maximum(lk_r, lq)
            cu_kr = np.concatenate([[0], np.cumsum(lk_r)])
            cu_c = np.concatenate([[0], np.cumsum(lk_r // r)])
            ks, ke = oracle.ragged_windows(cu_q, cu_kr, cu_c, ratio=r)
            for i in range(B):
                rows = np.arange(cu_q[i], cu_q[i + 1])
                seen = lk_r[i] - lq[i] + np.arange(lq[i]) + 1
                steps = np.diff(np.concatenate([[(seen[0] - 1) // r], ke[rows] - cu_c[i]]))
                assert np.array_equal(steps, (seen % r == 0).astype(int))
                if lk_r[i] % r == 0:
                    assert ke[rows[-1]] == cu_c[i + 1]


# ----------------------------------------------------------------- library routines
@pytest.mark.parametrize("k_fmt,H", [(0, 4), (1, 8), (0, 32)])
def test_row_logits_match_numpy_einsum(k_fmt, H):
    """The C++ loops against numpy's fp64 einsum over dequantised arrays that numpy builds
    itself (torch's E4M3 / E8M0 conversions, the E2M1 table): a dropped term, a swapped
    operand, a wrong scale or nibble order fails here."""
    T, L, D = 5, 700, 128
    rng = np.random.default_rng(k_fmt * 10 + H)
    cu_q = np.array([0, 2, 5], np.int32)
    cu_k = np.array([0, 301, 700], np.int32)
    p = synth.make_problem(T, L, H, k_fmt=k_fmt, seed=H + k_fmt, cu_q=cu_q, cu_k=cu_k, w_lo=-1.0, scale=0.625)
    p.q_scale = (p.q_scale * np.exp2(rng.integers(-3, 4, p.q_scale.shape))).astype(np.float32)
    q = torch.from_numpy(p.q).view(torch.float8_e4m3fn).to(torch.float64).numpy() * p.q_scale[..., None]
    if k_fmt == 0:
        k = torch.from_numpy(p.k).view(torch.float8_e4m3fn).to(torch.float64).numpy() * p.k_scale[:, None]
    else:
        table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])
        el = np.stack([table[p.k & 0xF], table[p.k >> 4]], axis=-1).reshape(L, D)
        sc = torch.from_numpy(p.k_scale).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
        k = el * np.repeat(sc, 32, axis=1)
    dq = oracle.Dequantised(p)
    for t in range(T):
        lo, hi = dq.ks[t], dq.ke[t]
        dots = np.einsum("hd,sd->hs", q[t], k[lo:hi]) * p.scale
        want = np.einsum("h,hs->s", p.w[t].astype(np.float64), np.maximum(dots, 0.0))
        np.testing.assert_allclose(oracle.row_logits(dq, t), want, rtol=1e-12, atol=1e-12)


def test_topk_row_matches_numpy_sort():
    """Selection against numpy's lexsort on the fp32-rounded values (value desc, index asc),
    rows with exact ties, signed zeros and masks."""
    rng = np.random.default_rng(23)
    for trial in range(40):
        n = int(rng.integers(1, 600))
        K = int(rng.integers(1, 80))
        v = np.round(rng.normal(size=n), int(rng.integers(0, 4)))
        v[rng.random(n) < 0.1] = -0.0
        allowed = rng.random(n) < 0.7 if trial % 2 else None
        idx, val = oracle.topk_row(v, 9, K, allowed)
        pos = np.arange(n) if allowed is None else np.nonzero(allowed)[0]
        v32 = v[pos].astype(np.float32).astype(np.float64)
        order = np.lexsort((pos, -v32))
        want = np.sort(pos[order[:K]])
        assert idx[:len(want)].tolist() == (want + 9).tolist() and (idx[len(want):] == -1).all()
        assert np.array_equal(val[:len(want)], v[want].astype(np.float32))


def test_ragged_windows_hand_examples():
    """Worked by hand: one request is the chunk at the tail of its prefix (ks = 0,
    ke = L - T + t + 1); a batch of a 3-token request and a 2-new-token request on a
    5-token prefix; an empty request."""
    ks, ke = oracle.ragged_windows([0, 4], [0, 10])
    assert ks.tolist() == [0, 0, 0, 0] and ke.tolist() == [7, 8, 9, 10]
    ks, ke = oracle.ragged_windows([0, 3, 5], [0, 3, 10])
    assert ks.tolist() == [0, 0, 0, 3, 3]
    assert ke.tolist() == [1, 2, 3, 9, 10]
    ks, ke = oracle.ragged_windows([0, 2, 2, 3], [0, 2, 6, 8])
    assert ks.tolist() == [0, 0, 6] and ke.tolist() == [1, 2, 8]
