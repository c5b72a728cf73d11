"""GPU parity of each C ABI call against the fp64 oracle, on seeded inputs at sizes the
oracle finishes in seconds (several tiles, ragged tails, empty and degenerate cases)."""
import math

import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O
from tests.parity_util import (assert_attn_close, assert_scores_close, np_u16,
                               score_abs_terms)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C(dev):
    from compressed_kv_cache_csa2_amd import csa2
    return csa2


def _i32(x, dev):
    return torch.tensor(x, dtype=torch.int32, device=dev)


def _i64(x, dev):
    return torch.tensor(x, dtype=torch.int64, device=dev)


def _bf16(shape, gen, dev, scale=1.0):
    return (torch.randn(shape, generator=gen) * scale).to(torch.bfloat16).to(dev)


def _e4m3(shape, gen, dev):
    from compressed_kv_cache_csa2_amd.synth import encode_e4m3
    return encode_e4m3(torch.randn(shape, generator=gen)).to(dev)


# --------------------------------------------------------------------------- indexer

def test_indexer_one_hot_reads_every_e4m3_code_in_place(C, dev):
    """Row r, channel c holds code (r + 3c) % 256 (NaN codes replaced); a one-hot indexer
    query on channel c with weight 1 scores ReLU(+-value): every code at every channel."""
    rows = np.arange(256)[:, None]
    chans = np.arange(128)[None, :]
    codes = ((rows + 3 * chans) % 256).astype(np.uint8)
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0
    k_cache = torch.from_numpy(codes).to(dev)
    tests = [(c, h, s) for c, h, s in zip([0, 1, 2, 3, 8, 63, 64, 65, 100, 127] * 2,
                                          list(range(0, 20)), [1.0] * 10 + [-1.0] * 10)]
    n_q = len(tests)
    q = torch.zeros((n_q, 32, 128), dtype=torch.float32)
    w = torch.zeros((n_q, 32), dtype=torch.float32)
    for t, (c, h, s) in enumerate(tests):
        q[t, h, c] = s
        w[t, h] = 1.0
    q = q.to(torch.bfloat16).to(dev)
    w = w.to(dev)
    scores = torch.empty((n_q, 256), dtype=torch.float32, device=dev)
    C.csa2_index_score(C.FULL, q, w, k_cache, _i64([0] * n_q, dev), _i32([256] * n_q, dev), scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for t in range(n_q):
        ref = O.full_scores(np_u16(q[t]), w[t].cpu().numpy(), codes, 0, 256, 256)
        assert np.array_equal(got[t].astype(np.float64), ref), f"query {t} {tests[t]}"


@pytest.mark.parametrize("case", ["tiny", "ragged"])
def test_index_score_full_parity(C, dev, case):
    from compressed_kv_cache_csa2_amd import synth
    if case == "tiny":
        wl = synth.make_workload("tiny_decode_4k").to(dev)
        ld = 4096
    else:
        # ragged: empty, single, sub-block and multi-tile sequences with gaps; the last
        # query's rows run past the end of the cache (absent rows score -inf)
        wl = synth.make_decode("ragged", 6, 0, ("full",), False, 0,
                               n_visible=[0, 1, 7, 4099, 2500, 9000], kv_gap=5, seed=3).to(dev)
        wl.n_visible[5] = 9000 + 37
        ld = 9100
    lay = wl.layers[0]
    scores = torch.empty((wl.n_q, ld), dtype=torch.float32, device=dev)
    bmax = torch.empty((wl.n_q, (ld + 7) // 8), dtype=torch.float32, device=dev)
    C.csa2_index_score(C.FULL, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, scores, bmax)
    torch.cuda.synchronize()
    k_all = wl.k_cache.cpu().numpy()
    got = scores.cpu().numpy()
    for t in range(wl.n_q):
        start, nv = int(wl.kv_start[t]), int(wl.n_visible[t])
        n_rows = max(0, min(nv, k_all.shape[0] - start))
        ref = O.full_scores(np_u16(lay.q_idx[t]), lay.w[t].cpu().numpy(), k_all, start, n_rows, ld)
        terms = np.zeros(ld)
        if n_rows:
            terms[:n_rows] = score_abs_terms(np_u16(lay.q_idx[t]), lay.w[t].cpu().numpy(),
                                             k_all[start:start + n_rows])
        assert_scores_close(got[t], ref, terms, f"query {t}")
    # block maxima are the maxima of the kernel's own scores
    pad = np.full((wl.n_q, bmax.shape[1] * 8), -np.inf, np.float32)
    pad[:, :ld] = got
    assert np.array_equal(bmax.cpu().numpy(), pad.reshape(wl.n_q, -1, 8).max(axis=2))
    # without a score buffer the same pass writes the same block maxima and nothing else
    bmax2 = torch.full_like(bmax, 7.0)
    C.csa2_index_score(C.FULL, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, None,
                       bmax2, ld_scores=ld)
    torch.cuda.synchronize()
    assert torch.equal(bmax2, bmax)


def test_index_score_reindex_parity(C, dev):
    from compressed_kv_cache_csa2_amd import synth
    wl = synth.make_decode("pool", 3, 0, ("full",), False, 0, n_visible=[20000, 777, 16384],
                           kv_gap=11, seed=4).to(dev)
    g = torch.Generator().manual_seed(5)
    pool = torch.full((3, 2048), -1, dtype=torch.int32)
    for t, nv in enumerate([20000, 777, 16384]):
        nb = (nv + 7) // 8
        m = min(2048, nb)
        ids = torch.randperm(nb, generator=g)[:m].sort().values.to(torch.int32)
        pool[t, :m] = ids
    pool[0, 5] = 2600          # beyond n_visible: -inf slots
    pool[2, 2047] = -1
    pool = pool.to(dev)
    q_idx = _bf16((3, 32, 128), g, dev)
    w = torch.rand((3, 32), generator=g).to(dev)
    scores = torch.empty((3, 16384), dtype=torch.float32, device=dev)
    C.csa2_index_score(C.REINDEX, q_idx, w, wl.k_cache, wl.kv_start, wl.n_visible, scores,
                       pool_blocks=pool)
    torch.cuda.synchronize()
    k_all = wl.k_cache.cpu().numpy()
    got = scores.cpu().numpy()
    for t in range(3):
        start, nv = int(wl.kv_start[t]), int(wl.n_visible[t])
        ref = O.reindex_scores(np_u16(q_idx[t]), w[t].cpu().numpy(), k_all, start, nv,
                               pool[t].cpu().numpy())
        pos = O.slots_to_positions(np.arange(16384), pool[t].cpu().numpy())
        ok = np.isfinite(ref)
        terms = np.zeros(16384)
        terms[ok] = score_abs_terms(np_u16(q_idx[t]), w[t].cpu().numpy(), k_all[start + pos[ok]])
        assert_scores_close(got[t], ref, terms, f"query {t}")


@pytest.mark.parametrize("fmt", ["e4m3", "mxfp4"])
def test_full_pass_and_reindex_form_score_bit_identically(C, dev, fmt):
    """The Full pass and the Reindex form give every position the same fp32 score, bit for
    bit: rescoring a pool (or the Full layer's candidate blocks) with the Full layer's own
    query reproduces the values its block maxima came from. Ragged, empty and multi-tile
    sequences; the pool lists every block of each sequence."""
    from compressed_kv_cache_csa2_amd import synth
    nvis = [0, 1, 7, 4099, 2500, 9000, 16384, 8 * 2048 - 3]
    wl = synth.make_decode("fr", len(nvis), 0, ("full",), False, 0, n_visible=nvis, kv_gap=5,
                           seed=6, mxfp4=(fmt == "mxfp4")).to(dev)
    lay = wl.layers[0]
    ld = 16384
    full = torch.empty((wl.n_q, ld), dtype=torch.float32, device=dev)
    pool = torch.full((wl.n_q, 2048), -1, dtype=torch.int32)
    for t, nv in enumerate(nvis):
        nb = (nv + 7) // 8
        pool[t, :nb] = torch.arange(nb, dtype=torch.int32)
    pool = pool.to(dev)
    re = torch.empty((wl.n_q, 16384), dtype=torch.float32, device=dev)
    if fmt == "mxfp4":
        C.csa2_index_score_mxfp4(C.FULL, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                                 wl.n_visible, full)
        C.csa2_index_score_mxfp4(C.REINDEX, lay.q_idx, lay.w, wl.k_codes, wl.k_scales,
                                 wl.kv_start, wl.n_visible, re, pool_blocks=pool)
    else:
        C.csa2_index_score(C.FULL, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, full)
        C.csa2_index_score(C.REINDEX, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible,
                           re, pool_blocks=pool)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int32), re.view(torch.int32))


# --------------------------------------------------------------------------- selection

def _score_rows(kind, n_q, n, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        s = torch.randn((n_q, n), generator=g) * 30 + 70
    elif kind == "signed":                      # both signs: keys on both sides of 2^31
        s = torch.randn((n_q, n), generator=g)
    elif kind == "ties":
        s = torch.randint(-3, 4, (n_q, n), generator=g).float()
    elif kind == "zeros":
        s = torch.zeros((n_q, n))
    else:
        raise ValueError(kind)
    m = torch.rand((n_q, n), generator=g)
    s[m < 0.05] = -math.inf
    s[(m > 0.05) & (m < 0.052)] = math.inf
    return s


def test_index_score_empty_cache(C, dev):
    """No readable entry (n_entries = 0): every score and block maximum is -inf."""
    import ctypes
    n_q, ld = 2, 1000
    q_idx = torch.zeros((n_q, 32, 128), dtype=torch.bfloat16, device=dev)
    w = torch.ones((n_q, 32), dtype=torch.float32, device=dev)
    k_cache = torch.zeros((1, 128), dtype=torch.uint8, device=dev)   # a valid pointer, 0 rows used
    kv_start = torch.zeros(n_q, dtype=torch.int64, device=dev)
    n_vis = torch.full((n_q,), 500, dtype=torch.int32, device=dev)
    scores = torch.zeros((n_q, ld), dtype=torch.float32, device=dev)
    bm = torch.zeros((n_q, (ld + 7) // 8), dtype=torch.float32, device=dev)
    aux = torch.full((n_q, (ld + 7) // 8), 5, dtype=torch.int32, device=dev)
    P = ctypes.c_void_p
    rc = C.lib.csa2_index_score(C.FULL, n_q, 32, 128, P(q_idx.data_ptr()), P(w.data_ptr()),
                                P(k_cache.data_ptr()), 0, P(kv_start.data_ptr()),
                                P(n_vis.data_ptr()), None, 0, 8, P(scores.data_ptr()), ld,
                                P(bm.data_ptr()), bm.shape[1], P(aux.data_ptr()), None)
    assert rc == 0, C.lib.csa2_last_error()
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(scores)) and torch.all(torch.isneginf(bm))
    assert torch.all(aux == 0)   # argmax slot 0, no selectable second score


@pytest.mark.parametrize("kind,n,k,use_bmax", [
    ("normal", 4096, 512, False), ("normal", 5000, 512, True), ("normal", 16384, 2048, False),
    ("normal", 40000, 512, False), ("normal", 40000, 512, True), ("normal", 100003, 512, True),
    ("ties", 3000, 512, False), ("ties", 70000, 512, True), ("ties", 70000, 100, False),
    ("zeros", 50000, 512, True), ("normal", 300, 512, True), ("normal", 1, 512, False),
    ("signed", 20000, 512, True), ("signed", 9000, 700, False), ("signed", 70000, 2048, True),
])
def test_topk_exact(C, dev, kind, n, k, use_bmax):
    n_q = 3
    s = _score_rows(kind, n_q, n, seed=n + k)
    n_valid = torch.tensor([n, max(0, n - 13), n // 2], dtype=torch.int32)
    ld = -(-n // 4) * 4 + 4                       # rows padded to a multiple of 4 (+ spare)
    sd = torch.full((n_q, ld), 7.0)               # padding never read as a score
    sd[:, :n] = s
    sd = sd.to(dev)
    bm = None
    if use_bmax:
        nb = (n + 7) // 8
        pad = torch.full((n_q, nb * 8), -math.inf)
        pad[:, :n] = s
        bmv = torch.full((n_q, -(-nb // 4) * 4), 1e30)
        bmv[:, :nb] = pad.view(n_q, nb, 8).amax(dim=2)
        bm = bmv.to(dev)
    out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    C.csa2_topk(sd, out, k=k, n_cols=n, n_valid=n_valid.to(dev), block_max=bm)
    torch.cuda.synchronize()
    for t in range(n_q):
        nv = int(n_valid[t])
        ref = O.topk_slots(s[t, :nv].double().numpy(), k)
        want = np.full(k, -1, np.int64)
        want[:len(ref)] = ref
        assert np.array_equal(out[t].cpu().numpy(), want), f"row {t}"


@pytest.mark.parametrize("kind,n", [("normal", 300000), ("ties", 70000), ("normal", 9000),
                                    ("signed", 20001), ("zeros", 50000)])
def test_topk_among_pool_candidates_is_exact(C, dev, kind, n):
    """With the pool csa2_block_pool builds from the same scores' block maxima, the Top-K
    restricted to the pool's slots is exactly the unrestricted Top-K (bitwise, ties
    included), also for short and ragged rows."""
    n_q, k = 3, 512
    s = _score_rows(kind, n_q, n, seed=n + 7)
    ld = (n + 3) // 4 * 4 + 4
    sd = torch.full((n_q, ld), 7.0, dtype=torch.float32, device=dev)
    sd[:, :n] = s.to(dev)
    n_valid = torch.tensor([n, n - 5, max(1, n // 3)], dtype=torch.int32, device=dev)
    nb = (ld + 7) // 8
    ld_bm = (nb + 3) // 4 * 4
    bm = torch.full((n_q, ld_bm), 1e30, dtype=torch.float32, device=dev)
    for t in range(n_q):
        nv = int(n_valid[t])
        row = torch.full((((nv + 7) // 8) * 8,), -math.inf, device=dev)
        row[:nv] = sd[t, :nv]
        bm[t, :(nv + 7) // 8] = row.view(-1, 8).amax(dim=1)
    pool = torch.empty((n_q, 2048), dtype=torch.int32, device=dev)
    C.csa2_block_pool(bm, n_valid, pool)
    got = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    ref = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    C.csa2_topk(sd, got, k=k, n_cols=n, n_valid=n_valid, pool_blocks=pool,
                pool_use=C.POOL_CANDIDATES)
    C.csa2_topk(sd, ref, k=k, n_cols=n, n_valid=n_valid)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    for t in range(n_q):   # and against the oracle
        nv = int(n_valid[t])
        want = O.slots_to_positions(O.topk_slots(s[t, :nv].double().numpy(), k), None)
        g = got[t].cpu().numpy()
        assert np.array_equal(np.sort(g[g >= 0]), np.sort(want))


@pytest.mark.parametrize("kind,n", [("normal", 300000), ("ties", 70000), ("normal", 9000),
                                    ("signed", 20001), ("zeros", 50000), ("normal", 7)])
def test_pool_topk_fused_equals_two_calls(C, dev, kind, n):
    """csa2_pool_topk writes the same pool and the same Top-K, bit for bit, as csa2_block_pool
    followed by csa2_topk among the pool's candidates, and the Top-K is the oracle's."""
    n_q, k = 3, 512
    s = _score_rows(kind, n_q, n, seed=n + 11)
    ld = (n + 3) // 4 * 4 + 4
    sd = torch.full((n_q, ld), 7.0, dtype=torch.float32, device=dev)
    sd[:, :n] = s.to(dev)
    n_valid = torch.tensor([n, max(0, n - 5), max(1, n // 3)], dtype=torch.int32, device=dev)
    nb = (ld + 7) // 8
    ld_bm = (nb + 3) // 4 * 4
    bm = torch.full((n_q, ld_bm), 1e30, dtype=torch.float32, device=dev)
    for t in range(n_q):
        nv = int(n_valid[t])
        row = torch.full((((nv + 7) // 8) * 8,), -math.inf, device=dev)
        row[:nv] = sd[t, :nv]
        bm[t, :(nv + 7) // 8] = row.view(-1, 8).amax(dim=1)
    pool_ref = torch.empty((n_q, 2048), dtype=torch.int32, device=dev)
    idx_ref = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    C.csa2_block_pool(bm, n_valid, pool_ref)
    C.csa2_topk(sd, idx_ref, k=k, n_cols=n, n_valid=n_valid, pool_blocks=pool_ref,
                pool_use=C.POOL_CANDIDATES)
    pool = torch.full((n_q, 2048), 12345, dtype=torch.int32, device=dev)
    idx = torch.full((n_q, k), 12345, dtype=torch.int32, device=dev)
    C.csa2_pool_topk(bm, n_valid, pool, sd, idx, k=k, n_cols=n)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool_ref)
    assert torch.equal(idx, idx_ref)
    for t in range(n_q):
        nv = int(n_valid[t])
        want = O.slots_to_positions(O.topk_slots(s[t, :nv].double().numpy(), k), None)
        g = idx[t].cpu().numpy()
        assert np.array_equal(np.sort(g[g >= 0]), np.sort(want)), f"row {t}"


def test_topk_pool_mapping(C, dev):
    n_q, k = 2, 512
    s = _score_rows("normal", n_q, 16384, seed=9)
    pool = torch.full((n_q, 2048), -1, dtype=torch.int32)
    pool[0] = torch.arange(2048, dtype=torch.int32) * 3 + 1
    pool[1, :1000] = torch.arange(1000, dtype=torch.int32) * 7
    s[1, 8000:] = -math.inf
    out = torch.empty((n_q, k), dtype=torch.int32, device=dev)
    C.csa2_topk(s.to(dev), out, k=k, pool_blocks=pool.to(dev))
    torch.cuda.synchronize()
    for t in range(n_q):
        ref = O.slots_to_positions(O.topk_slots(s[t].double().numpy(), k), pool[t].numpy())
        assert np.array_equal(out[t].cpu().numpy(), ref)


@pytest.mark.parametrize("kind,nvis", [("normal", [40000, 16385, 1000, 0, 7]),
                                       ("ties", [200000, 9, 16384 * 8 + 3, 8, 17]),
                                       # more than 32,768 blocks: quads first, then blocks
                                       ("ties", [600000, 262153, 300001, 8, 0]),
                                       ("normal", [1048576, 524289, 262151])])
def test_block_pool_exact(C, dev, kind, nvis):
    n_q = len(nvis)
    width = max(nvis)
    s = _score_rows(kind, n_q, width, seed=width)
    s[s == math.inf] = 1e30
    nb = (width + 7) // 8
    pad = torch.full((n_q, nb * 8), -math.inf)
    for t, nv in enumerate(nvis):
        pad[t, :nv] = s[t, :nv]
    bm = torch.full((n_q, -(-nb // 4) * 4), 1e30)     # padding beyond a row's blocks unused
    bm[:, :nb] = pad.view(n_q, nb, 8).amax(dim=2)
    pool = torch.empty((n_q, 2048), dtype=torch.int32, device=dev)
    C.csa2_block_pool(bm.to(dev), _i32(nvis, dev), pool)
    torch.cuda.synchronize()
    for t, nv in enumerate(nvis):
        ref = O.hsi_pool(s[t, :nv].double().numpy(), nv)
        want = np.full(2048, -1, np.int64)
        want[:len(ref)] = ref
        assert np.array_equal(pool[t].cpu().numpy(), want), f"row {t}"


# --------------------------------------------------------------------------- attention

def _attn_case(n_q, k, n_entries, n_swa, seed, dev, dup=False, holes=True):
    from compressed_kv_cache_csa2_amd import synth
    g = torch.Generator().manual_seed(seed)
    lat = torch.randn((n_entries, 512), generator=g)
    p, s = synth.encode_fp4_rows(lat)
    q = _bf16((n_q, 64, 512), g, dev)
    kv_start = torch.randint(0, max(1, n_entries // 4), (n_q,), generator=g)
    idx = torch.full((n_q, max(k, 1)), -1, dtype=torch.int32)
    for t in range(n_q):
        span = n_entries - int(kv_start[t])
        sel = torch.randint(0, span, (k,), generator=g) if dup else torch.randperm(span, generator=g)[:k]
        idx[t, :len(sel)] = sel.to(torch.int32)
        if holes and k > 4:
            idx[t, 3] = -1
            idx[t, 1] = span + 5     # row past the end of its sequence but maybe in the cache
            idx[t, 2] = n_entries * 4  # row outside the cache: skipped
    win_rows = n_q * 128 + 3
    window = _e4m3((win_rows, 512), g, dev)
    swa_start = torch.arange(n_q, dtype=torch.int64) * 128
    nsw = torch.full((n_q,), n_swa, dtype=torch.int32)
    return dict(q=q, kv_fp4=p.to(dev), kv_scale=s.to(dev), kv_start=kv_start.to(dev), idx=idx,
                window=window, swa_start=swa_start.to(dev), n_swa=nsw.to(dev), k=k)


@pytest.mark.parametrize("n_q,k,n_swa", [(1, 512, 128), (32, 512, 128), (3, 100, 0), (2, 0, 128),
                                         (2, 0, 0), (600, 64, 17), (5, 2048, 128)])
def test_sparse_attn_parity(C, dev, n_q, k, n_swa):
    case = _attn_case(n_q, k, 6000, n_swa, seed=n_q * 1000 + k + n_swa, dev=dev, dup=(n_q == 3))
    idx_d = case["idx"].to(dev)
    out = torch.empty((n_q, 64, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((n_q, 64), dtype=torch.float32, device=dev)
    need = C.workspace_bytes(C.OP_SPARSE_ATTN, n_q, 0, k)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    C.csa2_sparse_attn(case["q"], case["kv_fp4"], case["kv_scale"], case["kv_start"], idx_d,
                       case["window"], case["swa_start"], case["n_swa"], 1 / math.sqrt(512), out,
                       lse, ws, k=k)
    torch.cuda.synchronize()
    p_all, s_all = case["kv_fp4"].cpu().numpy(), case["kv_scale"].cpu().numpy()
    win = case["window"].cpu().numpy()
    n_entries = p_all.shape[0]
    for t in list(range(n_q))[:40]:
        start = int(case["kv_start"][t])
        pos = case["idx"][t, :k].numpy().astype(np.int64)
        pos = pos[(pos >= 0) & (start + pos < n_entries)]
        ents = O.gather_attention_entries(pos, p_all, s_all, start, win,
                                          int(case["swa_start"][t]), n_swa)
        ref, ref_lse = O.sparse_attention(O.bf16_decode(np_u16(case["q"][t])), ents, 1 / math.sqrt(512))
        got = out[t].float().cpu().numpy()
        if ents.shape[0] == 0:
            assert np.all(got == 0) and np.all(np.isneginf(lse[t].cpu().numpy()))
            continue
        assert_attn_close(got, ref, f"query {t}")
        assert np.allclose(lse[t].cpu().numpy(), ref_lse, atol=2e-3, rtol=1e-4)


def test_sparse_attn_single_entry_and_constant_query(C, dev):
    """Closed forms through the kernel: one attended entry is returned exactly (bf16 of an
    exactly representable vector); q = 0 gives the mean of the attended entries."""
    case = _attn_case(2, 16, 500, 0, seed=77, dev=dev, holes=False)
    idx = torch.full((2, 16), -1, dtype=torch.int32)
    idx[0, 7] = 42
    idx[1, :16] = case["idx"][1, :16]
    q = case["q"].clone()
    q[1].zero_()
    out = torch.empty((2, 64, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(1, C.workspace_bytes(C.OP_SPARSE_ATTN, 2, 0, 16)), dtype=torch.uint8, device=dev)
    C.csa2_sparse_attn(q, case["kv_fp4"], case["kv_scale"], case["kv_start"], idx.to(dev),
                       case["window"], case["swa_start"], case["n_swa"], 0.1, out, None, ws)
    torch.cuda.synchronize()
    p_all, s_all = case["kv_fp4"].cpu().numpy(), case["kv_scale"].cpu().numpy()
    row = int(case["kv_start"][0]) + 42
    one = O.fp4_latent_decode(p_all[row], s_all[row])
    assert np.array_equal(out[0].float().cpu().numpy(), np.repeat(one[None], 64, 0))
    start = int(case["kv_start"][1])
    ents = O.fp4_latent_decode(p_all[start + idx[1].numpy()], s_all[start + idx[1].numpy()])
    assert_attn_close(out[1].float().cpu().numpy(), np.repeat(ents.mean(0)[None], 64, 0), "q=0")


# --------------------------------------------------------------------------- MXFP4 keys

def test_mxfp4_indexer_one_hot_reads_every_code_and_scale_in_place(C, dev):
    """Row r, byte b holds (7r + 3b) % 256 (every pair of E2M1 codes) and scale group g of
    row r one of nine E8M0 codes from 2 to 252 (products from 2^-126 to 1.5*2^127); a
    one-hot indexer query on channel c with weight 1 scores ReLU(+-value), exactly."""
    rows = np.arange(256)[:, None]
    codes = ((7 * rows + 3 * np.arange(64)[None, :]) % 256).astype(np.uint8)
    sc_list = np.array([2, 60, 100, 126, 127, 128, 140, 200, 252], np.uint8)
    scales = sc_list[(rows + 2 * np.arange(4)[None, :]) % len(sc_list)].astype(np.uint8)
    k_codes = torch.from_numpy(codes).to(dev)
    k_scales = torch.from_numpy(scales).to(dev)
    chans = [0, 1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 127]
    tests = [(c, h, s) for s in (1.0, -1.0) for h, c in enumerate(chans)]
    n_q = len(tests)
    q = torch.zeros((n_q, 32, 128), dtype=torch.float32)
    w = torch.zeros((n_q, 32), dtype=torch.float32)
    for t, (c, h, s) in enumerate(tests):
        q[t, h, c] = s
        w[t, h] = 1.0
    q = q.to(torch.bfloat16).to(dev)
    w = w.to(dev)
    scores = torch.empty((n_q, 256), dtype=torch.float32, device=dev)
    C.csa2_index_score_mxfp4(C.FULL, q, w, k_codes, k_scales, _i64([0] * n_q, dev),
                             _i32([256] * n_q, dev), scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    for t in range(n_q):
        ref = O.full_scores_mxfp4(np_u16(q[t]), w[t].cpu().numpy(), codes, scales, 0, 256, 256)
        assert np.array_equal(got[t].astype(np.float64), ref), f"query {t} {tests[t]}"


@pytest.mark.parametrize("case", ["tiny", "ragged"])
def test_mxfp4_index_score_full_parity(C, dev, case):
    from compressed_kv_cache_csa2_amd import synth
    if case == "tiny":
        wl = synth.make_workload("tiny_decode_4k_mxfp4").to(dev)
        ld = 4096
    else:
        wl = synth.make_decode("ragged", 6, 0, ("full",), False, 0,
                               n_visible=[0, 1, 7, 4099, 2500, 9000], kv_gap=5, seed=3,
                               mxfp4=True).to(dev)
        wl.n_visible[5] = 9000 + 37   # rows past the end of the cache score -inf
        ld = 9100
    lay = wl.layers[0]
    scores = torch.empty((wl.n_q, ld), dtype=torch.float32, device=dev)
    bmax = torch.empty((wl.n_q, (ld + 7) // 8), dtype=torch.float32, device=dev)
    C.csa2_index_score_mxfp4(C.FULL, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, scores, bmax)
    torch.cuda.synchronize()
    kc, ks = wl.k_codes.cpu().numpy(), wl.k_scales.cpu().numpy()
    got = scores.cpu().numpy()
    for t in range(wl.n_q):
        start, nv = int(wl.kv_start[t]), int(wl.n_visible[t])
        n_rows = max(0, min(nv, kc.shape[0] - start))
        ref = O.full_scores_mxfp4(np_u16(lay.q_idx[t]), lay.w[t].cpu().numpy(), kc, ks, start,
                                  n_rows, ld)
        terms = np.zeros(ld)
        if n_rows:
            terms[:n_rows] = score_abs_terms(np_u16(lay.q_idx[t]), lay.w[t].cpu().numpy(),
                                             kc[start:start + n_rows], ks[start:start + n_rows])
        assert_scores_close(got[t], ref, terms, f"query {t}")
    pad = np.full((wl.n_q, bmax.shape[1] * 8), -np.inf, np.float32)
    pad[:, :ld] = got
    assert np.array_equal(bmax.cpu().numpy(), pad.reshape(wl.n_q, -1, 8).max(axis=2))


def test_mxfp4_index_score_reindex_parity(C, dev):
    from compressed_kv_cache_csa2_amd import synth
    wl = synth.make_decode("pool", 3, 0, ("full",), False, 0, n_visible=[20000, 777, 16384],
                           kv_gap=11, seed=4, mxfp4=True).to(dev)
    g = torch.Generator().manual_seed(5)
    pool = torch.full((3, 2048), -1, dtype=torch.int32)
    for t, nv in enumerate([20000, 777, 16384]):
        nb = (nv + 7) // 8
        m = min(2048, nb)
        pool[t, :m] = torch.randperm(nb, generator=g)[:m].sort().values.to(torch.int32)
    pool[0, 5] = 2600
    pool = pool.to(dev)
    q_idx = _bf16((3, 32, 128), g, dev)
    w = torch.rand((3, 32), generator=g).to(dev)
    scores = torch.empty((3, 16384), dtype=torch.float32, device=dev)
    C.csa2_index_score_mxfp4(C.REINDEX, q_idx, w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, scores, pool_blocks=pool)
    torch.cuda.synchronize()
    kc, ks = wl.k_codes.cpu().numpy(), wl.k_scales.cpu().numpy()
    got = scores.cpu().numpy()
    for t in range(3):
        start, nv = int(wl.kv_start[t]), int(wl.n_visible[t])
        ref = O.reindex_scores_mxfp4(np_u16(q_idx[t]), w[t].cpu().numpy(), kc, ks, start, nv,
                                     pool[t].cpu().numpy())
        pos = O.slots_to_positions(np.arange(16384), pool[t].cpu().numpy())
        ok = np.isfinite(ref)
        terms = np.zeros(16384)
        terms[ok] = score_abs_terms(np_u16(q_idx[t]), w[t].cpu().numpy(), kc[start + pos[ok]],
                                    ks[start + pos[ok]])
        assert_scores_close(got[t], ref, terms, f"query {t}")


# --------------------------------------------------------------------------- cache writes

def _hard_bf16_rows(n, d, seed):
    """bf16 rows that exercise the rounding: normal draws at several magnitudes, exact
    E4M3 and E2M1 midpoints, zeros, subnormal-range values and values past 448."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, d), generator=g) * torch.tensor([0.001, 0.1, 1, 10, 100])[
        torch.randint(0, 5, (n, 1), generator=g)]
    mags = torch.from_numpy(O.E4M3_POS.astype(np.float32))
    mids = (mags[:-1] + mags[1:]) / 2
    k = min(d, mids.numel())
    x[0, :k] = mids[:k]
    x[1, :k] = -mids[:k]
    x[2] = 0.0
    x[3, : d // 2] = 0.0
    x[4] = torch.linspace(-600, 600, d)
    x[5] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, -0.25, -0.75, -5.0, 1e-3,
                         -1e-3, 2.0 ** -8, 2.0 ** -12]).repeat(d // 16)
    return x.to(torch.bfloat16)


def test_write_latent_exact(C, dev):
    n, n_entries = 40, 64
    x = _hard_bf16_rows(n, 512, 31)
    rows = torch.randperm(n_entries, generator=torch.Generator().manual_seed(2))[:n].to(torch.int64)
    rows[7] = -1            # dropped
    rows[9] = n_entries     # out of range: dropped
    kv_fp4 = torch.full((n_entries, 256), 0xAB, dtype=torch.uint8, device=dev)
    kv_scale = torch.full((n_entries, 32), 0xCD, dtype=torch.uint8, device=dev)
    C.csa2_write_latent(x.to(dev), rows.to(dev), kv_fp4, kv_scale)
    torch.cuda.synchronize()
    p, s = O.fp4_latent_quantize(x.float().numpy())
    want_p = np.full((n_entries, 256), 0xAB, np.uint8)
    want_s = np.full((n_entries, 32), 0xCD, np.uint8)
    for r in range(n):
        d = int(rows[r])
        if 0 <= d < n_entries:
            want_p[d], want_s[d] = p[r], s[r]
    assert np.array_equal(kv_fp4.cpu().numpy(), want_p)
    assert np.array_equal(kv_scale.cpu().numpy(), want_s)


@pytest.mark.parametrize("d", [512, 128])
def test_write_e4m3_exact(C, dev, d):
    n, n_rows = 37, 50
    x = _hard_bf16_rows(n, d, 32 + d)
    rows = torch.arange(n, dtype=torch.int64) * 3 % n_rows
    rows[4] = -5
    dst = torch.full((n_rows, d), 0x5A, dtype=torch.uint8, device=dev)
    C.csa2_write_e4m3(x.to(dev), rows.to(dev), dst)
    torch.cuda.synchronize()
    want = np.full((n_rows, d), 0x5A, np.uint8)
    q = O.e4m3_round(x.float().numpy())
    for r in range(n):
        if int(rows[r]) >= 0:
            want[int(rows[r])] = q[r]
    assert np.array_equal(dst.cpu().numpy(), want)


def test_write_mxfp4_key_exact(C, dev):
    n, n_entries = 45, 60
    x = _hard_bf16_rows(n, 128, 33)
    x[6] = x[6] * 2.0 ** 60          # large exponents
    x[8] = x[8] * 2.0 ** -100        # tiny exponents (scale byte clamps at 1)
    rows = torch.arange(n, dtype=torch.int64)
    rows[10] = -1
    k_codes = torch.full((n_entries, 64), 0x11, dtype=torch.uint8, device=dev)
    k_scales = torch.full((n_entries, 4), 0x22, dtype=torch.uint8, device=dev)
    C.csa2_write_mxfp4_key(x.to(dev), rows.to(dev), k_codes, k_scales)
    torch.cuda.synchronize()
    c, s = O.mxfp4_key_quantize(x.float().numpy())
    want_c = np.full((n_entries, 64), 0x11, np.uint8)
    want_s = np.full((n_entries, 4), 0x22, np.uint8)
    for r in range(n):
        if int(rows[r]) >= 0:
            want_c[int(rows[r])], want_s[int(rows[r])] = c[r], s[r]
    assert np.array_equal(k_codes.cpu().numpy(), want_c)
    assert np.array_equal(k_scales.cpu().numpy(), want_s)


def test_written_cache_reads_back_through_the_read_path(C, dev):
    """Rows quantised on the GPU and read back by the indexer (MXFP4 keys) and by the
    attention (FP4 latent, E4M3 window) give the oracle's results on the oracle's own
    quantisation of the same rows."""
    g = torch.Generator().manual_seed(40)
    n = 600
    lat = torch.randn((n, 512), generator=g).to(torch.bfloat16)
    key = torch.randn((n, 128), generator=g).to(torch.bfloat16)
    win = torch.randn((128, 512), generator=g).to(torch.bfloat16)
    rows = torch.arange(n, dtype=torch.int64, device=dev)
    kv_fp4 = torch.zeros((n, 256), dtype=torch.uint8, device=dev)
    kv_scale = torch.zeros((n, 32), dtype=torch.uint8, device=dev)
    k_codes = torch.zeros((n, 64), dtype=torch.uint8, device=dev)
    k_scales = torch.zeros((n, 4), dtype=torch.uint8, device=dev)
    window = torch.zeros((128, 512), dtype=torch.uint8, device=dev)
    C.csa2_write_latent(lat.to(dev), rows, kv_fp4, kv_scale)
    C.csa2_write_mxfp4_key(key.to(dev), rows, k_codes, k_scales)
    C.csa2_write_e4m3(win.to(dev), rows[:128], window)
    q_idx = _bf16((1, 32, 128), g, dev)
    w = torch.rand((1, 32), generator=g).to(dev)
    scores = torch.empty((1, n), dtype=torch.float32, device=dev)
    C.csa2_index_score_mxfp4(C.FULL, q_idx, w, k_codes, k_scales, _i64([0], dev), _i32([n], dev),
                             scores)
    idx = torch.empty((1, 512), dtype=torch.int32, device=dev)
    C.csa2_topk(scores, idx, k=512, n_cols=n)
    q = _bf16((1, 64, 512), g, dev)
    out = torch.empty((1, 64, 512), dtype=torch.bfloat16, device=dev)
    C.csa2_sparse_attn(q, kv_fp4, kv_scale, _i64([0], dev), idx, window, _i64([0], dev),
                       _i32([128], dev), 1.0 / math.sqrt(512), out)
    torch.cuda.synchronize()
    kc, ks = O.mxfp4_key_quantize(key.float().numpy())
    ref_scores = O.full_scores_mxfp4(np_u16(q_idx[0]), w[0].cpu().numpy(), kc, ks, 0, n, n)
    terms = score_abs_terms(np_u16(q_idx[0]), w[0].cpu().numpy(), kc, ks)
    assert_scores_close(scores[0].cpu().numpy(), ref_scores, terms, "rescored keys")
    p, s = O.fp4_latent_quantize(lat.float().numpy())
    wq = O.e4m3_round(win.float().numpy())
    ents = O.gather_attention_entries(idx[0].cpu().numpy(), p, s, 0, wq, 0, 128)
    ref, _ = O.sparse_attention(O.bf16_decode(np_u16(q[0])), ents, 1.0 / math.sqrt(512))
    assert_attn_close(out[0].float().cpu().numpy(), ref, "attention over written rows")


def test_index_score_shared_equals_per_query_and_oracle(C, dev):
    """Queries sharing one sequence (ragged causal n_visible, a batch that is not a multiple
    of the group size, rows past the cache end): the grouped kernel writes the per-query
    kernel's scores and block maxima bit for bit, and both match the oracle."""
    g = torch.Generator().manual_seed(50)
    n_q, n_entries, start, ld = 19, 9000, 300, 8800
    k_cache = _e4m3((n_entries, 128), g, dev)
    q_idx = _bf16((n_q, 32, 128), g, dev)
    w = torch.rand((n_q, 32), generator=g).to(dev)
    nv = [0, 1, 7, 8, 9, 2047, 2048, 2049, 4100, 6000, 8699, 8700, 8701, 8800, 123, 5000, 3,
          8000, 8750]
    n_vis = _i32(nv, dev)
    a = torch.empty((n_q, ld), dtype=torch.float32, device=dev)
    ab = torch.empty((n_q, (ld + 7) // 8), dtype=torch.float32, device=dev)
    b, bb = torch.empty_like(a), torch.empty_like(ab)
    C.csa2_index_score_shared(q_idx, w, k_cache, start, n_vis, a, ab)
    C.csa2_index_score(C.FULL, q_idx, w, k_cache, _i64([start] * n_q, dev), n_vis, b, bb)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ab, bb)
    k_all = k_cache.cpu().numpy()
    got = a.cpu().numpy()
    for t in (0, 1, 5, 7, 11, 12, 13, 18):
        n_rows = max(0, min(nv[t], n_entries - start))
        ref = O.full_scores(np_u16(q_idx[t]), w[t].cpu().numpy(), k_all, start, n_rows, ld)
        terms = np.zeros(ld)
        if n_rows:
            terms[:n_rows] = score_abs_terms(np_u16(q_idx[t]), w[t].cpu().numpy(),
                                             k_all[start:start + n_rows])
        assert_scores_close(got[t], ref, terms, f"query {t}")
