"""Seeded sweeps of fused-indexer configurations against the oracle.  Each case draws T, L,
H, the key format, K (up to the largest, 2048), B_k, the row chunk, the window layout (causal,
random with empty windows, or a ragged batch of requests on prefixes) and the range of the
head weights (non-negative, or of both signs).  The selected sets must equal the oracle's,
and the selected values too where every head weight is >= 0.  Depending on K and B_k a case
runs block launches only or block and slab launches, one row chunk or several.  Sizes keep
the oracle to a few seconds per case."""
import numpy as np
import pytest
import torch

import mqa_logits_top_amd as idx
import oracle
import synth
from checks import topk_ok

pytestmark = pytest.mark.gpu

N_CASES = 96


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    H = int(rng.choice([32, 64]))
    fmt = int(rng.choice([synth.K_FP8, synth.K_MXFP4]))
    L = int(rng.integers(1, 60001))
    T = int(rng.integers(1, min(96, max(1, 3_000_000 // L)) + 1))   # T * L <= 3e6: the oracle stays quick
    K = int(rng.choice([1, 7, 64, 200, 512, 700, 2048]))
    Bk = int(rng.choice([256, 512, 1024, 2048, 8192, 32768]))
    rc = int(rng.choice([0, 8, 16, 64]))
    layout = str(rng.choice(["causal", "random", "ragged"]))
    w_lo = float(rng.choice([0.0, 0.0, -0.5]))
    kw = {}
    if layout == "causal":
        T = min(T, L)   # a causal chunk's rows are the last T of its L keys
    if layout == "random":
        ks = rng.integers(0, L, T).astype(np.int32)
        ke = np.minimum(ks + rng.integers(0, L + 1, T), L).astype(np.int32)
        ke[::5] = ks[::5]   # some empty windows
        kw = dict(ks=ks, ke=ke)
    elif layout == "ragged":
        B = int(rng.integers(1, 5))
        q_len = rng.multinomial(T, np.ones(B) / B)
        prefix = rng.integers(0, max(1, L // B) + 1, B)
        cu_q = np.concatenate([[0], np.cumsum(q_len)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(q_len + prefix)]).astype(np.int32)
        L = int(cu_k[-1]) if cu_k[-1] > 0 else 1
        kw = dict(cu_q=cu_q, cu_k=cu_k)
    return dict(T=T, L=L, H=H, fmt=fmt, K=K, Bk=Bk, rc=rc, layout=layout, w_lo=w_lo, seed=seed, kw=kw)


def _id(seed):
    c = _draw(seed)
    return (f"s{seed}-T{c['T']}-L{c['L']}-H{c['H']}-f{c['fmt']}-K{c['K']}-B{c['Bk']}-rc{c['rc']}-"
            f"{c['layout']}-w{c['w_lo']}")


@pytest.mark.parametrize("seed", range(N_CASES), ids=_id)
def test_random_fused_config_against_oracle(seed):
    c = _draw(seed)
    p = synth.make_problem(c["T"], c["L"], c["H"], k_fmt=c["fmt"], seed=100 + seed, w_lo=c["w_lo"], **c["kw"])
    d = idx.Inputs.from_host(p)
    dq = oracle.Dequantised(p)
    o = oracle.rows_logits(dq, range(c["T"]))
    gi, gv = idx.idx_logits_topk_fused(d, c["K"], block_k=c["Bk"], row_chunk=c["rc"])
    topk_ok(gi.cpu().numpy(), None if c["w_lo"] < 0 else gv.cpu().numpy(), o, dq.ks, c["K"])


N_CAND_CASES = 48


def _draw_cand(seed):
    c = _draw(500 + seed)
    rng = np.random.default_rng(9000 + seed)
    c["n_blocks"] = int(rng.choice([1, 5, 64, 512, 2048]))
    c["K"] = int(rng.choice([1, 64, 512, 2048]))
    return c


def _id_cand(seed):
    c = _draw_cand(seed)
    return (f"s{seed}-T{c['T']}-L{c['L']}-H{c['H']}-f{c['fmt']}-nb{c['n_blocks']}-K{c['K']}-B{c['Bk']}-"
            f"rc{c['rc']}-{c['layout']}-w{c['w_lo']}")


@pytest.mark.parametrize("seed", range(N_CAND_CASES), ids=_id_cand)
def test_random_candidate_source_and_consumers_against_oracle(seed):
    """The fused candidate source (8-key blocks from each row's ks, top-n_blocks, mask and block
    ids) against the oracle's block selection; then a consumer layer over the same keys
    restricted to the mask (selected sets equal the oracle's on the allowed keys) and the same
    consumer given the block ids (bitwise the mask consumer's result)."""
    from test_gpu_parity import _check_candidates

    c = _draw_cand(seed)
    p = synth.make_problem(c["T"], c["L"], c["H"], k_fmt=c["fmt"], seed=300 + seed, w_lo=c["w_lo"], **c["kw"])
    d = idx.Inputs.from_host(p)
    dq = oracle.Dequantised(p)
    o = oracle.rows_logits(dq, range(c["T"]))
    W = max(d.W, 1)
    nb = c["n_blocks"]
    blocks = torch.empty((c["T"], nb), dtype=torch.int32, device="cuda")
    mask, _ = idx.idx_block_candidates(d, W, n_blocks=nb, block_k=c["Bk"], row_chunk=c["rc"], out_blocks=blocks)
    m = mask.cpu().numpy()
    _check_candidates(dq, o, m, blocks.cpu().numpy(), nb)
    # a later layer over the same keys and windows, restricted to the published candidates
    p2 = synth.consumer_layer(p, seed=300 + seed)
    d2 = idx.Inputs.from_host(p2)
    o2 = oracle.rows_logits(oracle.Dequantised(p2), range(c["T"]))
    K = c["K"]
    mi, mv = idx.idx_logits_topk_fused(d2, K, block_k=c["Bk"], row_chunk=c["rc"], mask=mask)
    allowed = [m[t, :len(o2[t])].astype(bool) for t in range(c["T"])]
    topk_ok(mi.cpu().numpy(), None if c["w_lo"] < 0 else mv.cpu().numpy(), o2, dq.ks, K, allowed=allowed)
    bi, bv = idx.idx_logits_topk_fused_blocks(d2, K, blocks, pool=8, block_k=c["Bk"], row_chunk=c["rc"])
    assert torch.equal(bi, mi) and torch.equal(bv.view(torch.int32), mv.view(torch.int32))


N_DENSE_CASES = 32


def _id_dense(seed):
    return "d" + _id(800 + seed)


@pytest.mark.parametrize("seed", range(N_DENSE_CASES), ids=_id_dense)
def test_random_dense_path_against_oracle(seed):
    """Dense row-relative logits against the oracle to the plain bar (non-negative weights;
    weights of both signs are held to it by a strict xfail elsewhere), the exact top-K of those
    logits against the oracle's selection on the same values, and dense top-(K + 512) plus
    refinement against the fused call: the same index sets bitwise, and the same values where
    every weight is non-negative."""
    from checks import dense_ref, logits_ok
    from test_gpu_parity import _oracle_on

    c = _draw(800 + seed)
    p = synth.make_problem(c["T"], c["L"], c["H"], k_fmt=c["fmt"], seed=600 + seed, w_lo=c["w_lo"], **c["kw"])
    d = idx.Inputs.from_host(p)
    dq = oracle.Dequantised(p)
    o = oracle.rows_logits(dq, range(c["T"]))
    W = max(d.W, 1)
    lg = idx.idx_mqa_logits(d, W)
    if c["w_lo"] >= 0:
        logits_ok(lg.cpu().numpy(), dense_ref(o, W))
    K = c["K"]
    gi, gv = idx.idx_topk(lg, d.ks, d.ke, K, block_k=c["Bk"])
    gi, gv = gi.cpu().numpy(), gv.cpu().numpy()
    for t, win in enumerate(_oracle_on(lg.cpu().numpy(), dq)):
        oi, ov = oracle.topk_row(win, int(dq.ks[t]), K)
        assert np.array_equal(gi[t], oi) and np.array_equal(gv[t], ov), f"row {t}"
    ci, cv = idx.idx_topk(lg, d.ks, d.ke, idx.candidate_capacity(K))
    di, dv = idx.idx_refine_topk(d, ci, cv, K)
    fi, fv = idx.idx_logits_topk_fused(d, K, block_k=c["Bk"], row_chunk=c["rc"])
    assert torch.equal(di, fi)
    if c["w_lo"] >= 0:
        assert torch.equal(dv.view(torch.int32), fv.view(torch.int32))
