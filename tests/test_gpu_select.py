"""The decoder Full layer's pool and candidate blocks (csa2_pool_candidates) on the GPU: the
pool equals csa2_block_pool's bit for bit, the candidates are a subset of it, and the Top-K
taken among the candidates' rescored slots equals, bit for bit, the Top-K among all pool
slots (the route the chain tests hold to the oracle) and the oracle's whole-row selection.
The one-kernel route (csa2_full_select: pool, rescoring and Top-K on chip) gives the same
pool and Top-K bit for bit."""
import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O
from tests.parity_util import assert_set_band, band_of

pytestmark = pytest.mark.gpu


def _both_routes(wl, k=512):
    from compressed_kv_cache_csa2_amd import csa2 as C
    from compressed_kv_cache_csa2_amd import layers
    buf = layers.alloc_buffers(wl)
    lay = wl.layers[0]
    C.csa2_index_score(C.FULL, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, None,
                       buf.block_max, ld_scores=buf.scores.shape[1])
    dev = wl.k_cache.device
    pool_a = torch.full_like(buf.pool, -5)
    cand = torch.full_like(buf.pool, -5)
    idx_a = torch.full((wl.n_q, k), -5, dtype=torch.int32, device=dev)
    C.csa2_pool_candidates(buf.block_max, wl.n_visible, pool_a, cand, n_keep=2048, k=k)
    sc_a = torch.empty_like(buf.re_scores)
    C.csa2_index_score(C.REINDEX, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, sc_a,
                       pool_blocks=cand)
    C.csa2_topk(sc_a, idx_a, k=k, pool_blocks=cand)
    pool_b = torch.full_like(buf.pool, -5)
    idx_b = torch.full_like(idx_a, -5)
    C.csa2_block_pool(buf.block_max, wl.n_visible, pool_b, n_keep=2048)
    C.csa2_index_score(C.REINDEX, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible,
                       buf.re_scores, pool_blocks=pool_b)
    C.csa2_topk(buf.re_scores, idx_b, k=k, pool_blocks=pool_b)
    # the one-kernel route: a Full pass that also writes the block statistics (its block
    # maxima must equal the plain pass's bit for bit), then csa2_full_select
    bm_c = torch.full_like(buf.block_max, 7.0)
    aux_c = torch.full_like(buf.block_aux, -5)
    C.csa2_index_score(C.FULL, lay.q_idx, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, None,
                       bm_c, ld_scores=buf.scores.shape[1], block_aux=aux_c)
    pool_c = torch.full_like(buf.pool, -5)
    idx_c = torch.full_like(idx_a, -5)
    C.csa2_full_select(bm_c, aux_c, wl.n_visible, pool_c, lay.q_idx, lay.w, wl.k_cache,
                       wl.kv_start, idx_c, n_keep=2048, k=k)
    torch.cuda.synchronize()
    nb = buf.block_max.shape[1]
    for t in range(wl.n_q):
        live = min(nb, (int(wl.n_visible[t]) + 7) // 8)
        assert torch.equal(bm_c[t, :live], buf.block_max[t, :live]), "block maxima differ"
    assert torch.equal(pool_c, pool_b) and torch.equal(idx_c, idx_b), "one-kernel route differs"
    return pool_a, cand, idx_a, pool_b, idx_b


def _check_candidates(pool, cand):
    for p, c in zip(pool.cpu().numpy(), cand.cpu().numpy()):
        n = int((c >= 0).sum())
        assert np.all(c[n:] == -1) and np.all(np.diff(c[:n]) > 0)
        assert np.all(np.isin(c[:n], p[p >= 0]))


@pytest.mark.parametrize("n_visible", [
    [40000, 17000, 3001, 16384 + 8],            # ragged, short, exactly 2048 blocks + 1
    [1, 8, 9, 4104, 4097, 0, 520, 262144],      # tiny, empty, 513 blocks, full 256K
    [300000, 270001],                           # above 32,768 blocks: the quad path
])
def test_candidate_route_equals_pool_route(dev, n_visible):
    from compressed_kv_cache_csa2_amd import synth
    wl = synth.make_decode("fs", len(n_visible), 0, ("full",), True, 32, n_visible=n_visible,
                           kv_gap=5, seed=41).to(dev)
    for k in (512, 100):
        pool_a, cand, idx_a, pool_b, idx_b = _both_routes(wl, k)
        assert torch.equal(pool_a, pool_b), k
        assert torch.equal(idx_a, idx_b), k
        _check_candidates(pool_a, cand)
        # long contexts: the threshold engages and keeps about k + 1 blocks
        for t, nv in enumerate(n_visible):
            if nv > 8 * 2048 * 4:
                assert int((cand[t] >= 0).sum()) <= 2 * (k + 1), (t, k)


def test_candidates_with_ties_everywhere(dev):
    """Keys repeated in runs of 64 rows give equal scores and equal block maxima: ties go to
    the lower position and lower block in both routes, and the result equals the oracle's
    whole-row selection (up to the acceptance band between different runs' values)."""
    from compressed_kv_cache_csa2_amd import synth
    n_visible = [50000, 7777]
    wl = synth.make_decode("fs_ties", 2, 0, ("full",), True, 0, n_visible=n_visible, kv_gap=3,
                           seed=42).to(dev)
    kc = wl.k_cache
    wl.k_cache.copy_(kc[::64].repeat_interleave(64, dim=0)[:kc.shape[0]])
    pool_a, cand, idx_a, pool_b, idx_b = _both_routes(wl)
    assert torch.equal(pool_a, pool_b) and torch.equal(idx_a, idx_b)
    _check_candidates(pool_a, cand)
    lay = wl.layers[0]
    q = lay.q_idx[0:2].view(torch.int16).cpu().numpy().view(np.uint16)
    w = lay.w[0:2].cpu().numpy()
    kch = wl.k_cache.cpu().numpy()
    for t in range(2):
        st = int(wl.kv_start[t])
        s = O.full_scores(q[t], w[t], kch, st, n_visible[t], n_visible[t])
        got = idx_a[t].cpu().numpy()
        kth, band = band_of(s, 512)
        assert_set_band(got[got >= 0], O.topk_slots(s, 512), lambda p: s[p], kth, band,
                        f"query {t}")
        bm = O.block_max(s[:n_visible[t]])
        bm[(n_visible[t] - 1) // 8] = np.inf
        kb, bb = band_of(bm, 2048)
        gp = pool_a[t].cpu().numpy()
        assert_set_band(gp[gp >= 0], O.hsi_pool(s, n_visible[t]), lambda b: bm[b], kb, bb,
                        f"pool {t}")


def _key(v):
    """Selection key of float32 values (0 for -inf): the order-preserving unsigned image."""
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    k = np.where(u & 0x80000000, ~u & 0xFFFFFFFF, u | 0x80000000)
    return np.where(np.isfinite(v) | (v > 0), k, 0).astype(np.uint64)


def test_block_statistics_match_the_pass_scores(dev):
    """One Full pass writing scores, block maxima and block statistics: every block's
    maximum is the largest of its 8 scores, the argmax is the lowest slot holding it, and the
    stored second key is the largest key of the other slots rounded up to a multiple of 8
    (the pass's own scores, bit for bit; ties and partial last blocks included)."""
    from compressed_kv_cache_csa2_amd import csa2 as C
    from compressed_kv_cache_csa2_amd import synth
    n_visible = [40000, 17, 8, 0, 4099]
    wl = synth.make_decode("bs", len(n_visible), 0, ("full",), True, 16, n_visible=n_visible,
                           kv_gap=3, seed=43).to(dev)
    kc = wl.k_cache
    # runs of equal keys in the second query: ties inside blocks
    st = int(wl.kv_start[1])
    kc[st:st + 16] = kc[st:st + 1].expand(16, -1)
    lay = wl.layers[0]
    ld = 40000
    scores = torch.empty((len(n_visible), ld), dtype=torch.float32, device=dev)
    bm = torch.empty((len(n_visible), ld // 8), dtype=torch.float32, device=dev)
    aux = torch.empty((len(n_visible), ld // 8), dtype=torch.int32, device=dev)
    C.csa2_index_score(C.FULL, lay.q_idx, lay.w, kc, wl.kv_start, wl.n_visible, scores, bm,
                       block_aux=aux)
    torch.cuda.synchronize()
    s_all, bm_all = scores.cpu().numpy(), bm.cpu().numpy()
    aux_all = aux.cpu().numpy().view(np.uint32).astype(np.uint64)
    for t, nv in enumerate(n_visible):
        nb = (nv + 7) // 8
        if nb == 0:
            continue
        s = s_all[t, :nb * 8].reshape(nb, 8)
        keys = _key(s)
        arg = np.argmax(keys, axis=1)                       # first (lowest) maximal slot
        assert np.array_equal(bm_all[t, :nb], s[np.arange(nb), arg])
        assert np.array_equal(aux_all[t, :nb] & 7, arg)
        others = keys.copy()
        others[np.arange(nb), arg] = 0
        k2 = others.max(axis=1)
        assert np.array_equal(aux_all[t, :nb] & ~np.uint64(7), (k2 + 7) & ~np.uint64(7)), t


def _mxfp4_routes(wl, k=512):
    """MXFP4 indexer keys: the three-call route (pool_candidates, REINDEX rescoring of the
    candidates, Top-K among their slots), the pool route (block_pool, REINDEX over the whole
    pool, Top-K) and the one-kernel route (csa2_full_select_mxfp4 from a Full pass that also
    writes the block statistics) must give the same pool and Top-K bit for bit."""
    from compressed_kv_cache_csa2_amd import csa2 as C
    from compressed_kv_cache_csa2_amd import layers
    buf = layers.alloc_buffers(wl)
    lay = wl.layers[0]
    ld = buf.scores.shape[1]
    C.csa2_index_score_mxfp4(C.FULL, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, None, buf.block_max, ld_scores=ld)
    dev = wl.k_codes.device
    pool_a = torch.full_like(buf.pool, -5)
    cand = torch.full_like(buf.pool, -5)
    idx_a = torch.full((wl.n_q, k), -5, dtype=torch.int32, device=dev)
    C.csa2_pool_candidates(buf.block_max, wl.n_visible, pool_a, cand, n_keep=2048, k=k)
    sc_a = torch.empty_like(buf.re_scores)
    C.csa2_index_score_mxfp4(C.REINDEX, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, sc_a, pool_blocks=cand)
    C.csa2_topk(sc_a, idx_a, k=k, pool_blocks=cand)
    pool_b = torch.full_like(buf.pool, -5)
    idx_b = torch.full_like(idx_a, -5)
    C.csa2_block_pool(buf.block_max, wl.n_visible, pool_b, n_keep=2048)
    C.csa2_index_score_mxfp4(C.REINDEX, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, buf.re_scores, pool_blocks=pool_b)
    C.csa2_topk(buf.re_scores, idx_b, k=k, pool_blocks=pool_b)
    bm_c = torch.full_like(buf.block_max, 7.0)
    aux_c = torch.full_like(buf.block_aux, -5)
    C.csa2_index_score_mxfp4(C.FULL, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, None, bm_c, ld_scores=ld, block_aux=aux_c)
    pool_c = torch.full_like(buf.pool, -5)
    idx_c = torch.full_like(idx_a, -5)
    C.csa2_full_select_mxfp4(bm_c, aux_c, wl.n_visible, pool_c, lay.q_idx, lay.w, wl.k_codes,
                             wl.k_scales, wl.kv_start, idx_c, n_keep=2048, k=k)
    torch.cuda.synchronize()
    nb = buf.block_max.shape[1]
    for t in range(wl.n_q):
        live = min(nb, (int(wl.n_visible[t]) + 7) // 8)
        assert torch.equal(bm_c[t, :live], buf.block_max[t, :live]), "block maxima differ"
    assert torch.equal(pool_a, pool_b) and torch.equal(idx_a, idx_b), "candidate route differs"
    assert torch.equal(pool_c, pool_b), "one-kernel pool differs"
    assert torch.equal(idx_c, idx_b), "one-kernel Top-K differs"
    return pool_b, idx_b


@pytest.mark.parametrize("n_visible", [
    [40000, 17000, 3001, 16384 + 8],            # ragged, short, exactly 2048 blocks + 1
    [1, 8, 9, 4104, 0, 520, 262144],            # tiny, empty, 513 blocks, full 256K
    [300000],                                   # above 32,768 blocks: the quad path
])
def test_full_select_mxfp4_equals_the_three_calls(dev, n_visible):
    from compressed_kv_cache_csa2_amd import synth
    wl = synth.make_decode("fs4", len(n_visible), 0, ("full",), True, 32, n_visible=n_visible,
                           kv_gap=5, seed=44, mxfp4=True).to(dev)
    for k in (512, 100):
        _mxfp4_routes(wl, k)


def test_full_select_mxfp4_with_ties(dev):
    """MXFP4 key rows repeated in runs of 64 (equal scores and block maxima everywhere):
    every route breaks the ties the same way, and the selection equals the oracle's."""
    from compressed_kv_cache_csa2_amd import synth
    n_visible = [50000, 7777]
    wl = synth.make_decode("fs4_ties", 2, 0, ("full",), True, 0, n_visible=n_visible, kv_gap=3,
                           seed=45, mxfp4=True).to(dev)
    n = wl.k_codes.shape[0]
    wl.k_codes.copy_(wl.k_codes[::64].repeat_interleave(64, dim=0)[:n])
    wl.k_scales.copy_(wl.k_scales[::64].repeat_interleave(64, dim=0)[:n])
    pool, idx = _mxfp4_routes(wl)
    lay = wl.layers[0]
    q = lay.q_idx[0:2].view(torch.int16).cpu().numpy().view(np.uint16)
    w = lay.w[0:2].cpu().numpy()
    codes, scales = wl.k_codes.cpu().numpy(), wl.k_scales.cpu().numpy()
    for t in range(2):
        st = int(wl.kv_start[t])
        s = O.full_scores_mxfp4(q[t], w[t], codes, scales, st, n_visible[t], n_visible[t])
        got = idx[t].cpu().numpy()
        kth, band = band_of(s, 512)
        assert_set_band(got[got >= 0], O.topk_slots(s, 512), lambda p: s[p], kth, band,
                        f"query {t}")


def test_block_statistics_mxfp4(dev):
    """The MXFP4 Full pass's block statistics against its own scores, as for E4M3 keys."""
    from compressed_kv_cache_csa2_amd import csa2 as C
    from compressed_kv_cache_csa2_amd import synth
    n_visible = [40000, 17, 8, 0, 4099]
    wl = synth.make_decode("bs4", len(n_visible), 0, ("full",), True, 16, n_visible=n_visible,
                           kv_gap=3, seed=46, mxfp4=True).to(dev)
    st = int(wl.kv_start[1])
    wl.k_codes[st:st + 16] = wl.k_codes[st:st + 1].expand(16, -1)
    wl.k_scales[st:st + 16] = wl.k_scales[st:st + 1].expand(16, -1)
    lay = wl.layers[0]
    ld = 40000
    scores = torch.empty((len(n_visible), ld), dtype=torch.float32, device=dev)
    bm = torch.empty((len(n_visible), ld // 8), dtype=torch.float32, device=dev)
    aux = torch.empty((len(n_visible), ld // 8), dtype=torch.int32, device=dev)
    C.csa2_index_score_mxfp4(C.FULL, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                             wl.n_visible, scores, bm, block_aux=aux)
    torch.cuda.synchronize()
    s_all, bm_all = scores.cpu().numpy(), bm.cpu().numpy()
    aux_all = aux.cpu().numpy().view(np.uint32).astype(np.uint64)
    for t, nv in enumerate(n_visible):
        nb = (nv + 7) // 8
        if nb == 0:
            continue
        s = s_all[t, :nb * 8].reshape(nb, 8)
        keys = _key(s)
        arg = np.argmax(keys, axis=1)
        assert np.array_equal(bm_all[t, :nb], s[np.arange(nb), arg])
        assert np.array_equal(aux_all[t, :nb] & 7, arg)
        others = keys.copy()
        others[np.arange(nb), arg] = 0
        k2 = others.max(axis=1)
        assert np.array_equal(aux_all[t, :nb] & ~np.uint64(7), (k2 + 7) & ~np.uint64(7)), t
