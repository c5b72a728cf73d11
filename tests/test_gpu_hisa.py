"""The block-mean (HISA-style) two-stage filter on the GPU against the oracle: block-mean
keys bit for bit, bf16 indexer scores, and the pool, Top-K and attention of every indexer
layer of a small decoder stack."""
import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O
from tests.parity_util import assert_scores_close, check_query_hisa, np_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C(dev):
    from compressed_kv_cache_csa2_amd import csa2
    return csa2


def _bf16_abs_terms(q_bits, w, rows_bits):
    qa = np.abs(O.bf16_decode(q_bits))
    ka = np.abs(O.bf16_decode(rows_bits))
    return (ka @ qa.T) @ np.abs(np.asarray(w, np.float64))


def test_block_mean_keys_exact(C, dev):
    from compressed_kv_cache_csa2_amd import layers, synth
    nvis = [20001, 7, 0, 4096 + 3]
    wl = synth.make_decode("bm", 4, 0, ("full",), False, 8, n_visible=nvis, kv_gap=5,
                           seed=41).to(dev)
    means = layers.build_block_means(wl)
    torch.cuda.synchronize()
    k_all = wl.k_cache.cpu().numpy()
    km = np_u16(means.km)
    assert means.n_blocks.cpu().tolist() == [-(-n // 8) for n in nvis]
    for t, nv in enumerate(nvis):
        start, row0 = int(wl.kv_start[t]), int(means.km_start[t])
        nb = -(-nv // 8)
        ref = O.block_mean_keys(k_all[start:start + nv], nv)
        assert np.array_equal(km[row0:row0 + nb], ref), t
        assert not km[row0 + nb:row0 + means.km.shape[0] // 4].any(), t   # rows past nb untouched
    # max_blocks bounds the rows written per query
    km3 = torch.zeros_like(means.km)
    nb3 = torch.full_like(means.n_blocks, -5)
    C.csa2_block_mean_keys(wl.k_cache, wl.kv_start, wl.n_visible, km3, means.km_start, nb3,
                           max_blocks=3)
    torch.cuda.synchronize()
    assert torch.equal(nb3, means.n_blocks)
    for t, nv in enumerate(nvis):
        row0 = int(means.km_start[t])
        m = min(3, -(-nv // 8))
        assert torch.equal(km3[row0:row0 + m], means.km[row0:row0 + m])
        assert not km3[row0 + m:row0 + 3 + 1].view(torch.int16).any()


def test_block_mean_keys_append_updates_the_latest_block(C, dev):
    """After one key is appended per query, recomputing only the latest block gives the same
    means as a full rebuild (completed blocks keep their summary)."""
    from compressed_kv_cache_csa2_amd import synth
    nvis = [1000, 17, 8 * 50, 0]
    wl = synth.make_decode("app", 4, 0, ("full",), False, 0, n_visible=nvis, kv_gap=16,
                           seed=44).to(dev)
    rows_per_q = 200
    km = torch.zeros((4 * rows_per_q, 128), dtype=torch.bfloat16, device=dev)
    km_start = torch.arange(4, dtype=torch.int64, device=dev) * rows_per_q
    nb = torch.zeros(4, dtype=torch.int32, device=dev)
    C.csa2_block_mean_keys(wl.k_cache, wl.kv_start, wl.n_visible, km, km_start, nb,
                           max_blocks=rows_per_q)
    g = torch.Generator().manual_seed(45)
    for t, n in enumerate(nvis):
        new = synth.encode_e4m3(torch.randn((1, 128), generator=g)).to(dev)
        wl.k_cache[int(wl.kv_start[t]) + n] = new[0]
    n_after = wl.n_visible + 1
    C.csa2_block_mean_keys(wl.k_cache, wl.kv_start, n_after, km, km_start, nb,
                           max_blocks=rows_per_q, last_only=True)
    km_full = torch.zeros_like(km)
    nb_full = torch.zeros_like(nb)
    C.csa2_block_mean_keys(wl.k_cache, wl.kv_start, n_after, km_full, km_start, nb_full,
                           max_blocks=rows_per_q)
    torch.cuda.synchronize()
    assert torch.equal(nb, nb_full)
    assert torch.equal(km.view(torch.int16), km_full.view(torch.int16))
    k_all = wl.k_cache.cpu().numpy()
    for t, n in enumerate(nvis):
        start = int(wl.kv_start[t])
        ref = O.block_mean_keys(k_all[start:start + n + 1], n + 1)
        assert np.array_equal(np_u16(km[t * rows_per_q:t * rows_per_q + len(ref)]), ref), t


def test_index_score_bf16_parity(C, dev):
    """Full and Reindex scoring of bf16 key rows against the oracle's indexer score."""
    g = torch.Generator().manual_seed(43)
    nvis = [5000, 33, 2049]
    starts = [0, 5003, 5100]
    n_rows = 7200
    rows = (torch.randn((n_rows, 128), generator=g) * 0.7).to(torch.bfloat16)
    q_idx = torch.randn((3, 32, 128), generator=g).to(torch.bfloat16)
    w = torch.rand((3, 32), generator=g)
    d_rows, d_q, d_w = rows.to(dev), q_idx.to(dev), w.to(dev)
    kv_start = torch.tensor(starts, dtype=torch.int64, device=dev)
    n_visible = torch.tensor(nvis, dtype=torch.int32, device=dev)
    ld = 5024
    scores = torch.empty((3, ld), dtype=torch.float32, device=dev)
    C.csa2_index_score_bf16(C.FULL, d_q, d_w, d_rows, kv_start, n_visible, scores)
    torch.cuda.synchronize()
    rows_bits = np_u16(rows)
    got = scores.cpu().numpy()
    for t in range(3):
        qb, wt = np_u16(q_idx[t]), w[t].numpy()
        k = rows_bits[starts[t]:starts[t] + nvis[t]]
        ref = np.full(ld, -np.inf)
        ref[:nvis[t]] = O.index_score_rows(O.bf16_decode(qb), wt.astype(np.float64),
                                           O.bf16_decode(k))
        terms = np.zeros(ld)
        terms[:nvis[t]] = _bf16_abs_terms(qb, wt, k)
        assert_scores_close(got[t], ref, terms, f"full q{t}")
    # Reindex over a pool of blocks, one beyond the visible range
    pool = torch.full((3, 2048), -1, dtype=torch.int32)
    for t, nv in enumerate(nvis):
        nb = -(-nv // 8)
        ids = torch.randperm(nb, generator=g)[:min(2048, nb)].sort().values
        pool[t, :ids.numel()] = ids.to(torch.int32)
    pool[0, 7] = 700
    d_pool = pool.to(dev)
    re = torch.empty((3, 16384), dtype=torch.float32, device=dev)
    C.csa2_index_score_bf16(C.REINDEX, d_q, d_w, d_rows, kv_start, n_visible, re,
                            pool_blocks=d_pool)
    torch.cuda.synchronize()
    got = re.cpu().numpy()
    for t in range(3):
        qb, wt = np_u16(q_idx[t]), w[t].numpy()
        pos = O.slots_to_positions(np.arange(16384), pool[t].numpy())
        ok = (pos >= 0) & (pos < nvis[t])
        ref = np.full(16384, -np.inf)
        k = rows_bits[starts[t] + pos[ok]]
        ref[ok] = O.index_score_rows(O.bf16_decode(qb), wt.astype(np.float64), O.bf16_decode(k))
        terms = np.zeros(16384)
        terms[ok] = _bf16_abs_terms(qb, wt, k)
        assert_scores_close(got[t], ref, terms, f"reindex q{t}")


def test_hisa_decoder_stack_parity(C, dev):
    """Every indexer layer of a decoder stack selects through the two-stage filter; each
    layer's pool is checked against the oracle's block-mean pool, its Top-K against the
    oracle's rescoring of the GPU's pool, and every layer's attention against the oracle's
    attention over the GPU's indices. The whole stack then reproduces these indices."""
    from compressed_kv_cache_csa2_amd import layers, synth
    nvis = [40000, 17000, 16384 + 8]
    wl = synth.make_decode("hisa", 3, 0, synth.DECODE_LAYERS, True, 32, n_visible=nvis,
                           kv_gap=9, seed=42).to(dev)
    means = layers.build_block_means(wl)
    buf = layers.alloc_buffers(wl)
    pools = {}
    for li, lay in enumerate(wl.layers):
        if lay.mode in ("full", "reindex"):
            layers.hisa_select(wl, lay, buf, means, buf.idx[li])
            pools[li] = buf.pool.clone()
    torch.cuda.synchronize()
    step_idx = buf.idx.clone()
    buf2 = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf2, coarse="hisa", means=means)
    torch.cuda.synchronize()
    assert torch.equal(buf2.idx, step_idx)
    n_cmp = sum(check_query_hisa(wl, step_idx, pools, buf2.out, t) for t in range(wl.n_q))
    assert n_cmp == wl.n_q * len(wl.layers)
