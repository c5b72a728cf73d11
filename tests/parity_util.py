"""Helpers shared by the GPU parity tests: host copies, tolerance and band rules.

Acceptance rules:
  - index sets (Top-K positions, pool blocks) equal the oracle's except for elements whose
    oracle value lies within 1e-3 relative of the K-th oracle value (1e-3 of the largest
    magnitude when the K-th value is 0);
  - attention outputs within max-abs error <= 2e-2 * max|ref|;
  - indexer scores (fp32 MFMA accumulation of exact products) within 1e-5 of the sum of
    the absolute values of their terms;
  - a selection made on MXFP8-query scores s8 against the configs' bf16-query selection
    (scores s): with D the largest |s8 - s| of the row, the two differ only in elements
    whose bf16 value lies within 2D (plus the tie band) of the bf16 K-th value.
"""
import numpy as np
import torch

import oracle.csa2_oracle as O

BAND_REL = 1e-3
ATTN_TOL = 2e-2
SCORE_REL = 1e-5


def np_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def score_abs_terms(q_bits, w, k_codes, k_scales=None):
    """sum_h |w_h| sum_d |q_hd k_d| for every row: the scale of fp32 rounding in a score.
    k_codes are E4M3 rows, or MXFP4 code rows when k_scales is given."""
    qa = np.abs(O.bf16_decode(q_bits))
    if k_scales is None:
        ka = np.abs(O.e4m3_decode(k_codes))
    else:
        ka = np.abs(O.mxfp4_key_decode(k_codes, k_scales))
    return (ka @ qa.T) @ np.abs(np.asarray(w, np.float64))


def assert_scores_close(gpu, ref, abs_terms, what=""):
    gpu = np.asarray(gpu, np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), f"{what}: -inf pattern differs"
    assert np.all(gpu[~fin] == ref[~fin]), what
    err = np.abs(gpu[fin] - ref[fin])
    lim = SCORE_REL * abs_terms[fin] + 1e-30
    bad = np.nonzero(err > lim)[0]
    assert bad.size == 0, f"{what}: {bad.size} scores off, worst {err.max():.3e}"


def band_of(ref_values, k):
    """K-th largest selectable oracle value and the tie band around it."""
    v = np.asarray(ref_values, np.float64)
    sel = O.topk_slots(v, k)
    if sel.size == 0:
        return None, 0.0
    kth = v[sel].min()
    fin = v[np.isfinite(v)]
    scale = abs(kth) if kth != 0 and np.isfinite(kth) else (np.abs(fin).max() if fin.size else 0.0)
    return kth, BAND_REL * scale


def assert_set_band(gpu_items, ref_items, ref_value_of, kth, band, what=""):
    """gpu_items and ref_items may differ only in elements whose oracle value is within the
    band of the K-th value; sizes must agree."""
    g = set(int(x) for x in gpu_items if x >= 0)
    r = set(int(x) for x in ref_items if x >= 0)
    assert len(g) == len([x for x in gpu_items if x >= 0]), f"{what}: duplicate selections"
    assert len(g) == len(r), f"{what}: {len(g)} selected, oracle {len(r)}"
    for x in g ^ r:
        v = ref_value_of(x)
        assert abs(v - kth) <= band, f"{what}: {x} (value {v}) differs outside the band of {kth}"
    return g == r


def q8_departure_band(s_bf16, s_q8, k):
    """K-th largest bf16-query value, and the band outside which a selection on the MXFP8-
    query values may not depart from the bf16 one, with D = max |s_q8 - s_bf16| over the
    finite entries. Any k entries with s >= tau have s_q8 >= tau - D, so the q8 K-th value
    tau8 >= tau - D, and symmetrically tau >= tau8 - D; an entry the q8 selection adds has
    s >= s_q8 - D >= tau8 - D >= tau - 2D, one it drops has s <= s_q8 + D <= tau + 2D.
    The band adds the tie band (the GPU's q8 scores carry fp32 rounding). Returns (tau,
    band, D)."""
    s = np.asarray(s_bf16, np.float64)
    s8 = np.asarray(s_q8, np.float64)
    fin = np.isfinite(s) & np.isfinite(s8)
    assert np.array_equal(np.isfinite(s), np.isfinite(s8)), "finite patterns differ"
    d = float(np.abs(s8[fin] - s[fin]).max()) if fin.any() else 0.0
    kth, tie = band_of(s, k)
    return kth, 2.0 * d + tie, d


def overlap(a, b):
    """|a & b| / |b| over the non-negative entries."""
    a = set(int(x) for x in a if x >= 0)
    b = set(int(x) for x in b if x >= 0)
    return len(a & b) / max(1, len(b))


def assert_attn_close(gpu_out, ref_out, what=""):
    gpu = np.asarray(gpu_out, np.float64)
    ref = np.asarray(ref_out, np.float64)
    scale = np.abs(ref).max()
    err = np.abs(gpu - ref).max()
    assert err <= ATTN_TOL * scale + 1e-30, f"{what}: max-abs err {err:.3e} vs {ATTN_TOL}*{scale:.3e}"
    return err / scale if scale else 0.0


def check_query(wl, buf, t, seq=None, report=None):
    """Compare every layer of query t of a run (buffers `buf`) with the oracle.

    Each step is checked on the GPU's own previous output, so a legitimate swap inside a
    tie band never cascades: the Full Top-K and pool against the oracle's scores, the
    Reindex Top-K against the oracle's rescoring of the GPU's pool, and every attention
    (output and lse) against the oracle's attention over the GPU's published indices.
    Returns the number of attention outputs compared."""
    from compressed_kv_cache_csa2_amd import synth
    seq = seq or synth.sequence_to_host(wl, t)
    nv = seq["n_visible"]
    scale = wl.softmax_scale
    pool_gpu = None
    n_cmp = 0
    for li, lay in enumerate(seq["layers"]):
        k_cache, kv_fp4, kv_scale = lay["k_cache"], lay["kv_fp4"], lay["kv_scale"]
        idx_gpu = buf.published[li][t].cpu().numpy()
        if lay.get("q_idx") is not None and wl.q8:
            qc, qs = O.mxfp8_quantize(O.bf16_decode(lay["q_idx"]).astype(np.float32))
        if lay["mode"] == "swa":
            assert idx_gpu.size == 0, f"q{t} L{li}: an SWA layer attends with no selection"
        elif lay["mode"] == "full":
            if wl.q8 and "k_codes" in seq:
                scores = O.full_scores_mxfp4_q8(qc, qs, lay["w"], seq["k_codes"], seq["k_scales"],
                                                0, nv, nv)
            elif wl.q8:
                scores = O.full_scores_q8(qc, qs, lay["w"], k_cache, 0, nv, nv)
            elif "k_codes" in seq:
                scores = O.full_scores_mxfp4(lay["q_idx"], lay["w"], seq["k_codes"],
                                             seq["k_scales"], 0, nv, nv)
            else:
                scores = O.full_scores(lay["q_idx"], lay["w"], k_cache, 0, nv, nv)
            ref_idx = O.slots_to_positions(O.topk_slots(scores, 512), None)
            kth, band = band_of(scores, 512)
            assert_set_band(idx_gpu, ref_idx, lambda p: scores[p], kth, band,
                            f"q{t} L{li} full top-k")
            if wl.with_pool:
                pool_gpu = buf.pool[t].cpu().numpy()
                ref_pool = O.hsi_pool(scores, nv)
                bm = O.block_max(scores[:nv])
                bm[(nv - 1) // 8] = np.inf
                kb, bb = band_of(bm, 2048)
                assert_set_band(pool_gpu, ref_pool, lambda b: bm[b], kb, bb, f"q{t} pool")
        elif lay["mode"] == "reindex":
            padded = np.full(2048, -1, np.int64)
            kept = pool_gpu[pool_gpu >= 0]
            padded[:len(kept)] = kept
            if wl.q8 and "k_codes" in seq:
                scores = O.reindex_scores_mxfp4_q8(qc, qs, lay["w"], seq["k_codes"],
                                                   seq["k_scales"], 0, nv, padded)
            elif wl.q8:
                scores = O.reindex_scores_q8(qc, qs, lay["w"], k_cache, 0, nv, padded)
            elif "k_codes" in seq:
                scores = O.reindex_scores_mxfp4(lay["q_idx"], lay["w"], seq["k_codes"],
                                                seq["k_scales"], 0, nv, padded)
            else:
                scores = O.reindex_scores(lay["q_idx"], lay["w"], k_cache, 0, nv, padded)
            ref_idx = O.slots_to_positions(O.topk_slots(scores, 512), padded)
            pos_of_slot = O.slots_to_positions(np.arange(len(scores)), padded)
            score_at = dict(zip(pos_of_slot.tolist(), scores.tolist()))
            kth, band = band_of(scores, 512)
            assert_set_band(idx_gpu, ref_idx, lambda p: score_at[p], kth, band,
                            f"q{t} L{li} reindex top-k")
        if lay["mode"] == "swa":
            res = O.swa_layer(lay["q"], lay["window_kv"], 0, lay["n_swa"], scale)
        else:
            res = O.reuse_layer(idx_gpu, lay["q"], kv_fp4, kv_scale, 0, lay["window_kv"], 0,
                                lay["n_swa"], scale)
        rel = assert_attn_close(buf.out[li][t].float().cpu().numpy(), res["out"],
                                f"q{t} L{li} {lay['mode']} attention")
        lse_gpu = buf.lse[li][t].cpu().numpy().astype(np.float64)
        assert np.allclose(lse_gpu, res["lse"], atol=2e-3, rtol=1e-4), f"q{t} L{li} lse"
        n_cmp += 1
        if report is not None:
            report.append((t, li, rel))
    return n_cmp


def check_query_hisa(wl, idx, pools, out, t):
    """Compare query t of a stack run through the block-mean filter with the oracle: each
    indexer layer's pool (pools[li], captured after that layer) against the oracle's
    block-mean pool, its Top-K (idx[li]) against the oracle's rescoring of the GPU's pool,
    and every layer's attention output against the oracle's attention over the GPU's
    indices. Returns the number of attention outputs compared."""
    from compressed_kv_cache_csa2_amd import synth
    seq = synth.sequence_to_host(wl, t)
    nv = seq["n_visible"]
    km = O.block_mean_keys(seq["k_cache"], nv)
    current = None
    n_cmp = 0
    for li, lay in enumerate(seq["layers"]):
        if li in pools:
            bs = O.index_score_rows(O.bf16_decode(lay["q_idx"]), np.asarray(lay["w"], np.float64),
                                    O.bf16_decode(km))
            bs[(nv - 1) // 8] = np.inf
            pool_gpu = pools[li][t].cpu().numpy()
            ref_pool = O.hisa_pool(lay["q_idx"], lay["w"], km, nv)
            kb, bb = band_of(bs, 2048)
            assert_set_band(pool_gpu, ref_pool, lambda b: bs[b], kb, bb, f"q{t} L{li} pool")
            padded = np.full(2048, -1, np.int64)
            kept = pool_gpu[pool_gpu >= 0]
            padded[:len(kept)] = kept
            scores = O.reindex_scores(lay["q_idx"], lay["w"], seq["k_cache"], 0, nv, padded)
            ref_idx = O.slots_to_positions(O.topk_slots(scores, 512), padded)
            pos_of_slot = O.slots_to_positions(np.arange(len(scores)), padded)
            score_at = dict(zip(pos_of_slot.tolist(), scores.tolist()))
            kth, band = band_of(scores, 512)
            current = idx[li][t].cpu().numpy()
            assert_set_band(current, ref_idx, lambda p: score_at[p], kth, band,
                            f"q{t} L{li} top-k")
        res = O.reuse_layer(current, lay["q"], seq["kv_fp4"], seq["kv_scale"], 0,
                            lay["window_kv"], 0, lay["n_swa"], wl.softmax_scale)
        assert_attn_close(out[li][t].float().cpu().numpy(), res["out"], f"q{t} L{li} attention")
        n_cmp += 1
    return n_cmp
