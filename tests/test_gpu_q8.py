"""MXFP8 indexer query over MXFP4 keys on the scaled f8f6f4 MFMA, against the oracle."""
import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O
from tests.parity_util import assert_scores_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C(dev):
    from compressed_kv_cache_csa2_amd import csa2
    return csa2


def test_quantize_mxfp8_exact(C, dev):
    g = torch.Generator().manual_seed(71)
    x = (torch.randn(9, 32, 128, generator=g) * 2).to(torch.bfloat16)
    x[0, 0, :32] = 0.0
    x[1, 5, 32:64] = x[1, 5, 32:64] * 2.0 ** 50
    x[2, 7, 64:96] = x[2, 7, 64:96] * 2.0 ** -70
    x[3, 9, 96:] = -x[3, 9, 96:].abs()
    codes = torch.full((9, 32, 128), 0x5A, dtype=torch.uint8, device=dev)
    scales = torch.full((9, 32, 4), 0x5A, dtype=torch.uint8, device=dev)
    C.csa2_quantize_mxfp8(x.to(dev), codes, scales)
    torch.cuda.synchronize()
    wc, ws = O.mxfp8_quantize(x.float().numpy())
    assert np.array_equal(codes.cpu().numpy(), wc)
    assert np.array_equal(scales.cpu().numpy(), ws)


def _abs_terms(qc, qs, w, kc, ks):
    qa = np.abs(O.mxfp8_decode(qc, qs))
    ka = np.abs(O.mxfp4_key_decode(kc, ks))
    return (ka @ qa.T) @ np.abs(np.asarray(w, np.float64))


@pytest.mark.parametrize("with_scores", [True, False])
def test_index_score_mxfp4_q8_parity(C, dev, with_scores):
    from compressed_kv_cache_csa2_amd import synth
    nvis = [5000, 33, 2049, 0]
    wl = synth.make_decode("q8", 4, 0, ("full",), False, 8, n_visible=nvis, kv_gap=5, seed=72,
                           mxfp4=True).to(dev)
    lay = wl.layers[0]
    qc = torch.empty((4, 32, 128), dtype=torch.uint8, device=dev)
    qs = torch.empty((4, 32, 4), dtype=torch.uint8, device=dev)
    C.csa2_quantize_mxfp8(lay.q_idx, qc, qs)
    ld = 5024
    scores = torch.full((4, ld), 3.0, dtype=torch.float32, device=dev) if with_scores else None
    bmax = torch.full((4, ld // 8), 3.0, dtype=torch.float32, device=dev)
    C.csa2_index_score_mxfp4_q8(C.FULL, qc, qs, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                                wl.n_visible, scores, bmax, ld_scores=ld)
    torch.cuda.synchronize()
    kc_all, ks_all = wl.k_codes.cpu().numpy(), wl.k_scales.cpu().numpy()
    qcn, qsn, w = qc.cpu().numpy(), qs.cpu().numpy(), lay.w.cpu().numpy()
    bm = bmax.cpu().numpy()
    for t, nv in enumerate(nvis):
        start = int(wl.kv_start[t])
        ref = O.full_scores_mxfp4_q8(qcn[t], qsn[t], w[t], kc_all, ks_all, start, nv, ld)
        terms = np.zeros(ld)
        if nv > 0:
            terms[:nv] = _abs_terms(qcn[t], qsn[t], w[t], kc_all[start:start + nv],
                                    ks_all[start:start + nv])
        if with_scores:
            assert_scores_close(scores[t].cpu().numpy(), ref, terms, f"q8 scores q{t}")
        # block maxima: within the same bound of the oracle's block maxima
        refb = ref.reshape(-1, 8).max(axis=1)
        tb = terms.reshape(-1, 8).max(axis=1)
        fin = np.isfinite(refb)
        assert np.array_equal(np.isfinite(bm[t]), fin), t
        assert np.all(np.abs(bm[t][fin] - refb[fin]) <= 1e-5 * tb[fin] + 1e-30), t


def test_small_decode_stack_with_mxfp8_query(dev):
    """A decoder stack (Full with pool, Reindex, Reuse) whose indexer passes quantise their
    query to MXFP8 and score the MXFP4 keys on the scaled MFMA, checked layer by layer."""
    from compressed_kv_cache_csa2_amd import layers, synth
    from tests.parity_util import check_query
    wl = synth.make_decode("q8_stack", 3, 0, synth.DECODE_LAYERS, True, 16,
                           n_visible=[40000, 17000, 16384 + 8], kv_gap=9, seed=73,
                           mxfp4=True).to(dev)
    wl.q8 = True
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    assert sum(check_query(wl, buf, t) for t in range(wl.n_q)) == wl.n_q * len(wl.layers)


def test_small_decode_stack_with_mxfp8_query_over_e4m3_keys(dev):
    """The same stack over E4M3 keys (the matrix core's fp8 B operand, unit key scales)."""
    from compressed_kv_cache_csa2_amd import layers, synth
    from tests.parity_util import check_query
    wl = synth.make_decode("q8_e4m3", 3, 0, synth.DECODE_LAYERS, True, 16,
                           n_visible=[40000, 17000, 16384 + 8], kv_gap=9, seed=74).to(dev)
    wl.q8 = True
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    assert sum(check_query(wl, buf, t) for t in range(wl.n_q)) == wl.n_q * len(wl.layers)


def test_index_score_shared_q8_equals_per_query_and_oracle(dev):
    """Grouped scoring of queries sharing one sequence gives the per-query MXFP8-query
    scores bit for bit, and the oracle's on sampled queries."""
    from compressed_kv_cache_csa2_amd import csa2 as C, synth
    wl = synth.make_prefill("pf_q8", n_q=45, n_entries=9000, device=dev, seed=75)
    lay = wl.layers[0]
    qc = torch.empty((45, 32, 128), dtype=torch.uint8, device=dev)
    qs = torch.empty((45, 32, 4), dtype=torch.uint8, device=dev)
    C.csa2_quantize_mxfp8(lay.q_idx, qc, qs)
    ld = 9024
    s1 = torch.empty((45, ld), dtype=torch.float32, device=dev)
    s2 = torch.empty_like(s1)
    b1 = torch.empty((45, ld // 8), dtype=torch.float32, device=dev)
    b2 = torch.empty_like(b1)
    C.csa2_index_score_shared_q8(qc, qs, lay.w, wl.k_cache, 0, wl.n_visible, s1, b1)
    C.csa2_index_score_q8(C.FULL, qc, qs, lay.w, wl.k_cache, wl.kv_start, wl.n_visible, s2, b2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(b1, b2)
    k_all = wl.k_cache.cpu().numpy()
    for t in (0, 22, 44):
        nv = int(wl.n_visible[t])
        q = (qc[t].cpu().numpy(), qs[t].cpu().numpy())
        ref = O.full_scores_q8(q[0], q[1], lay.w[t].cpu().numpy(), k_all, 0, nv, ld)
        qa = np.abs(O.mxfp8_decode(*q))
        terms = np.zeros(ld)
        terms[:nv] = (np.abs(O.e4m3_decode(k_all[:nv])) @ qa.T) @ np.abs(lay.w[t].cpu().numpy().astype(np.float64))
        assert_scores_close(s1[t].cpu().numpy(), ref, terms, f"shared q8 q{t}")


@pytest.fixture(scope="module")
def decode_256k_q8(dev):
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_workload("decode_256k_q8", device=dev)
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    return wl, buf


@pytest.mark.parametrize("t", [0, 13, 31])
def test_mxfp8_query_selection_departs_only_inside_the_rounding_band(decode_256k_q8, t):
    """decode_256k_q8 at full size: the GPU's MXFP8-query selections (the Full layer's
    Top-512 and pool, then the Reindex layer's Top-512 over that pool) against the bf16-query
    selections the configs specify, computed by the oracle on the same data. With D the
    largest change the query's MXFP8 rounding makes to a score of the row (oracle q8 score
    minus oracle bf16 score), every departure lies within 2D of the bf16 K-th value; the
    overlaps are printed."""
    from compressed_kv_cache_csa2_amd import synth
    from tests.parity_util import assert_set_band, overlap, q8_departure_band
    wl, buf = decode_256k_q8
    seq = synth.sequence_to_host(wl, t)
    nv = seq["n_visible"]
    kc = seq["k_cache"]
    full, re = seq["layers"][0], seq["layers"][1]
    # Full layer over every position
    qc, qs = O.mxfp8_quantize(O.bf16_decode(full["q_idx"]).astype(np.float32))
    s = O.full_scores(full["q_idx"], full["w"], kc, 0, nv, nv)
    s8 = O.full_scores_q8(qc, qs, full["w"], kc, 0, nv, nv)
    tau, band, d = q8_departure_band(s, s8, 512)
    ref_idx = O.topk_slots(s, 512)
    got_idx = buf.idx[0][t].cpu().numpy()
    assert_set_band(got_idx, ref_idx, lambda p: s[p], tau, band, f"q{t} full top-k (q8 vs bf16)")
    # pool: block maxima (the latest block forced in), D bounded by the scores' D
    bm = O.block_max(s[:nv])
    bm8 = O.block_max(s8[:nv])
    bm[(nv - 1) // 8] = bm8[(nv - 1) // 8] = np.inf
    tau_b, band_b, _ = q8_departure_band(bm, bm8, 2048)
    pool_gpu = buf.pool[t].cpu().numpy()
    assert_set_band(pool_gpu, O.topk_slots(bm, 2048), lambda b: bm[b], tau_b, band_b,
                    f"q{t} pool (q8 vs bf16)")
    # Reindex layer over the GPU's pool
    padded = np.full(2048, -1, np.int64)
    kept = pool_gpu[pool_gpu >= 0]
    padded[:len(kept)] = kept
    qc2, qs2 = O.mxfp8_quantize(O.bf16_decode(re["q_idx"]).astype(np.float32))
    r = O.reindex_scores(re["q_idx"], re["w"], kc, 0, nv, padded)
    r8 = O.reindex_scores_q8(qc2, qs2, re["w"], kc, 0, nv, padded)
    tau_r, band_r, d_r = q8_departure_band(r, r8, 512)
    pos_of_slot = O.slots_to_positions(np.arange(len(r)), padded)
    score_at = dict(zip(pos_of_slot.tolist(), r.tolist()))
    ref_re = O.slots_to_positions(O.topk_slots(r, 512), padded)
    got_re = buf.idx[1][t].cpu().numpy()
    assert_set_band(got_re, ref_re, lambda p: score_at[p], tau_r, band_r,
                    f"q{t} reindex top-k (q8 vs bf16)")
    print(f"q{t}: D = {d:.3f} (K-th bf16 score {tau:.2f}), overlaps: full top-k "
          f"{overlap(got_idx, ref_idx):.3f}, pool {overlap(pool_gpu, O.topk_slots(bm, 2048)):.3f}, "
          f"reindex top-k {overlap(got_re, ref_re):.3f} (D = {d_r:.3f})")
