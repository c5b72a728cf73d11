"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test ties one oracle function to something it cannot agree with by construction:
published format tables (tests/golden), library routines (torch casts, scaled dot-product
attention, scipy logsumexp), a literal transcription of the pool construction the blog
page describes in PyTorch terms, brute force with pure-Python loops on tiny inputs,
closed forms and invariants (convex hull, Reuse/Reindex identities, scale invariance).
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------------------------------ codecs

def test_e4m3_exhaustive_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_anchor_codes():
    for code, val in _golden("e4m3_anchors.txt"):
        assert O.e4m3_value(int(code, 16)) == float(val), code
    # monotone over the positive codes, and the negative half mirrors it
    pos = O.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(O.e4m3_decode(np.arange(0x80, 0xFF)), -pos)


def test_e2m1_table_matches_published_magnitudes():
    for code, val in _golden("e2m1_magnitudes.txt"):
        c = int(code)
        assert O.e2m1_value(c) == float(val)
        assert O.e2m1_value(c | 8) == -float(val)
    # largest magnitude of an FP4 value with an E4M3 scale: 6 * 448
    assert O.e2m1_value(7) * O.e4m3_value(0x7E) == 2688.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(4096).astype(np.float32) * 50).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_decode(bits), x.to(torch.float64).numpy())


def test_fp4_latent_nibble_order_and_scale_groups():
    payload = np.zeros((1, 256), np.uint8)
    payload[0, 0] = 0x71          # channel 0 <- code 1 (0.5), channel 1 <- code 7 (6.0)
    payload[0, 8] = 0xA3          # channel 16 <- code 3 (1.5), channel 17 <- code 10 (-1.0)
    scales = np.zeros((1, 32), np.uint8)
    scales[0, 0] = 0x38           # 1.0 for channels 0..15
    scales[0, 1] = 0x40           # 2.0 for channels 16..31
    c = O.fp4_latent_decode(payload, scales)[0]
    assert c[0] == 0.5 and c[1] == 6.0
    assert c[16] == 3.0 and c[17] == -2.0
    assert np.count_nonzero(c) == 4


def test_fp4_roundtrip_with_generator_encoder():
    """Encoder of the input generator and decoder of the oracle invert each other."""
    from compressed_kv_cache_csa2_amd import synth
    # every (code, scale) product that the format can hold is reproduced exactly
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(64, 512))
    codes[:, ::16] = 7            # each group reaches |6| so amax/6 is the scale itself
    scale_codes = rng.integers(0x20, 0x60, size=(64, 32)).astype(np.uint8)
    exact = O.e2m1_decode(codes) * np.repeat(O.e4m3_decode(scale_codes), 16, axis=-1)
    payload, scales = synth.encode_fp4_rows(torch.from_numpy(exact).float())
    back = O.fp4_latent_decode(payload.numpy(), scales.numpy())
    assert np.array_equal(back, exact)
    # random values: error within half an E2M1 step of the group scale (no saturation)
    x = rng.standard_normal((256, 512))
    payload, scales = synth.encode_fp4_rows(torch.from_numpy(x).float())
    back = O.fp4_latent_decode(payload.numpy(), scales.numpy())
    s = np.repeat(O.e4m3_decode(scales.numpy()), 16, axis=-1)
    step = np.where(np.abs(x) / s < 2, 0.5, np.where(np.abs(x) / s < 4, 1.0, 2.0))
    assert np.all(np.abs(back - x) <= 0.5 * step * s + 1e-6 * np.abs(x) + s * 0.02)


# ------------------------------------------------------------------------------ indexer

def _bf16_py(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_index_score_brute_force_loops():
    rng = np.random.default_rng(2)
    q = torch.from_numpy(rng.standard_normal((32, 128)).astype(np.float32)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    w = rng.random(32).astype(np.float32)
    k = rng.integers(0, 256, size=(7, 128)).astype(np.uint8)
    k[k == 0x7F] = 0x7E
    k[k == 0xFF] = 0xFE
    got = O.full_scores(q_bits, w, k, 0, 7, 9)
    for j in range(7):
        s = 0.0
        for h in range(32):
            dot = 0.0
            for d in range(128):
                dot += _bf16_py(q_bits[h, d]) * O.e4m3_value(k[j, d])
            s += float(w[h]) * max(dot, 0.0)
        assert math.isclose(got[j], s, rel_tol=1e-12, abs_tol=1e-12)
    assert got[7] == -np.inf and got[8] == -np.inf


def test_index_score_relu_and_weight_scaling():
    rng = np.random.default_rng(3)
    k = O.e4m3_decode(rng.integers(0, 0x70, size=(5, 128)))       # all positive rows
    q = np.abs(rng.standard_normal((32, 128)))
    w = rng.random(32)
    # every head negative -> every ReLU is zero
    assert np.all(O.index_score_rows(-q, w, k) == 0.0)
    # one head flipped -> it drops out, the others add up
    q2 = q.copy()
    q2[5] = -q2[5]
    w2 = w.copy()
    w2[5] = 0.0
    assert np.allclose(O.index_score_rows(q2, w, k), O.index_score_rows(q, w2, k))
    # positive scale of w scales the scores and leaves the Top-K unchanged
    s1 = O.index_score_rows(q, w, k)
    s2 = O.index_score_rows(q, 3.5 * w, k)
    assert np.allclose(s2, 3.5 * s1)
    assert np.array_equal(O.topk_slots(s1, 3), O.topk_slots(s2, 3))


# ------------------------------------------------------------------------------ Top-K

def _brute_topk(s, k):
    cand = [j for j in range(len(s)) if not math.isnan(s[j]) and s[j] > -math.inf]
    return sorted(sorted(cand, key=lambda j: (-s[j], j))[:k])


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties_and_masks(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    s = rng.integers(-5, 6, size=n).astype(np.float64)    # many ties
    s[rng.random(n) < 0.2] = -np.inf
    s[rng.random(n) < 0.05] = np.inf
    s[rng.random(n) < 0.05] = np.nan
    for k in (1, 7, 64, 512):
        assert O.topk_slots(s, k).tolist() == _brute_topk(s.tolist(), k)


def test_topk_sizes_and_order_property():
    rng = np.random.default_rng(7)
    s = rng.standard_normal(5000)
    s[4000:] = -np.inf
    sel = O.topk_slots(s, 512)
    assert len(sel) == 512 and np.all(np.diff(sel) > 0)
    rest = np.setdiff1d(np.arange(4000), sel)
    assert s[sel].min() >= s[rest].max()
    assert len(O.topk_slots(s[:100], 512)) == 100
    assert len(O.topk_slots(np.full(10, -np.inf), 512)) == 0


# ------------------------------------------------------------------------------ HSI pool

def _pool_bitmap_torch(logits, width, block_size, n_keep):
    """The pool construction as the blog page spells it in PyTorch calls: pad with -inf,
    split into blocks, amax, force the latest block, keep the best blocks, expand."""
    import torch.nn.functional as F
    scores = F.pad(logits, (0, -width % block_size), value=-torch.inf)
    bm = scores.unflatten(-1, (-1, block_size)).amax(dim=-1)
    bm[..., (width - 1) // block_size] = torch.inf
    keep = torch.topk(bm, min(n_keep, bm.shape[-1]), dim=-1).indices
    flags = torch.zeros_like(bm, dtype=torch.bool)
    flags[keep] = True
    return flags.repeat_interleave(block_size, dim=-1)[..., :width]


@pytest.mark.parametrize("width,n_keep", [(21, 2), (64, 3), (1000, 40), (8, 5), (3, 1), (4099, 100)])
def test_pool_matches_pytorch_transcription(width, n_keep):
    rng = np.random.default_rng(width)
    logits = rng.standard_normal(width)           # continuous -> no ties
    ref = _pool_bitmap_torch(torch.from_numpy(logits), width, 8, n_keep).numpy()
    blocks = O.hsi_pool(logits, width, 8, n_keep)
    assert np.array_equal(O.pool_bitmap(blocks, width, 8), ref)
    assert np.all(np.diff(blocks) > 0)


def test_pool_properties():
    rng = np.random.default_rng(11)
    n = 40000
    s = rng.standard_normal(n)
    blocks = O.hsi_pool(s, n)
    assert len(blocks) == 2048 and (n - 1) // 8 in blocks
    bitmap = O.pool_bitmap(blocks, n)
    assert bitmap.sum() == 2048 * 8
    # the Full Top-512 lies inside the pool (each winner's block max beats the rest)
    assert bitmap[O.topk_slots(s, 512)].all()
    # short context: every block is kept
    assert np.array_equal(O.hsi_pool(s[:1000], 1000), np.arange(125))
    assert len(O.hsi_pool(s, 0)) == 0


def test_reindex_with_full_query_reproduces_full_topk():
    rng = np.random.default_rng(12)
    n = 30001
    k_cache = rng.integers(0, 0x7E, size=(n, 128)).astype(np.uint8) ^ (rng.integers(0, 2, size=(n, 128)).astype(np.uint8) << 7)
    q = torch.from_numpy(rng.standard_normal((32, 128)).astype(np.float32)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    w = rng.random(32).astype(np.float32)
    s = O.full_scores(q_bits, w, k_cache, 0, n, n)
    full_idx = O.topk_slots(s, 512)
    pool = O.hsi_pool(s, n)
    padded = np.full(2048, -1)
    padded[:len(pool)] = pool
    rs = O.reindex_scores(q_bits, w, k_cache, 0, n, padded)
    re_idx = O.slots_to_positions(O.topk_slots(rs, 512), padded)
    assert np.array_equal(np.sort(re_idx), full_idx)


# ------------------------------------------------------------------------------ attention

def test_attention_matches_library_sdpa():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((64, 512))
    ents = rng.standard_normal((37, 512))
    out, lse = O.sparse_attention(q, ents, 1 / math.sqrt(512))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(ents)[None, None].expand(1, 64, 37, 512),
        torch.from_numpy(ents)[None, None].expand(1, 64, 37, 512), scale=1 / math.sqrt(512))
    assert np.allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    from scipy.special import logsumexp
    assert np.allclose(lse, logsumexp(q @ ents.T / math.sqrt(512), axis=1), rtol=1e-12)


def test_attention_closed_forms_and_convex_hull():
    rng = np.random.default_rng(14)
    ents = rng.standard_normal((20, 512))
    out, _ = O.sparse_attention(np.zeros((64, 512)), ents, 0.1)
    assert np.allclose(out, ents.mean(axis=0)[None])
    one, lse1 = O.sparse_attention(rng.standard_normal((64, 512)), ents[3:4], 0.1)
    assert np.array_equal(one, np.repeat(ents[3:4], 64, axis=0))
    out, _ = O.sparse_attention(5 * rng.standard_normal((64, 512)), ents, 1.0)
    assert np.all(out <= ents.max(axis=0) + 1e-12) and np.all(out >= ents.min(axis=0) - 1e-12)
    empty, lse0 = O.sparse_attention(np.ones((64, 512)), np.zeros((0, 512)), 1.0)
    assert np.all(empty == 0) and np.all(lse0 == -np.inf)


def _tiny_sequence(seed, n, n_swa=128):
    rng = np.random.default_rng(seed)
    k_cache = rng.integers(0, 0x7E, size=(n, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(n, 128)).astype(np.uint8) << 7)
    from compressed_kv_cache_csa2_amd import synth
    p, s = synth.encode_fp4_rows(torch.from_numpy(rng.standard_normal((n, 512))).float())
    win = synth.encode_e4m3(torch.from_numpy(rng.standard_normal((n_swa, 512))).float()).numpy()
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q_idx = bf(rng.standard_normal((32, 128)))
    w = rng.random(32).astype(np.float32)
    q = bf(rng.standard_normal((64, 512)))
    return k_cache, p.numpy(), s.numpy(), win, q_idx, w, q


def test_full_layer_with_k_covering_context_is_dense_attention():
    n = 300
    k_cache, p, s, win, q_idx, w, q = _tiny_sequence(15, n)
    res = O.full_layer(q_idx, w, k_cache, 0, n, q, p, s, win, 0, 128, 1 / math.sqrt(512), k=512)
    assert np.array_equal(res["idx"], np.arange(n))
    dense = np.concatenate([O.fp4_latent_decode(p, s), O.e4m3_decode(win)], axis=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(O.bf16_decode(q))[None, :, None, :],
        torch.from_numpy(dense)[None, None].expand(1, 64, -1, 512),
        torch.from_numpy(dense)[None, None].expand(1, 64, -1, 512), scale=1 / math.sqrt(512))
    assert np.allclose(res["out"], ref[0, :, 0].numpy(), rtol=1e-11, atol=1e-11)


def test_reuse_with_full_inputs_reproduces_full_layer():
    n = 5000
    k_cache, p, s, win, q_idx, w, q = _tiny_sequence(16, n)
    full = O.full_layer(q_idx, w, k_cache, 0, n, q, p, s, win, 0, 128, 0.05, with_pool=True)
    reuse = O.reuse_layer(full["idx"], q, p, s, 0, win, 0, 128, 0.05)
    assert np.array_equal(reuse["out"], full["out"]) and np.array_equal(reuse["lse"], full["lse"])
    assert len(full["idx"]) == 512 and len(full["pool"]) == 625


def test_model_constants_and_entry_bytes():
    c = {k: int(v) for k, v in _golden("model_constants.txt")}
    assert c["candidate_topk_blocks"] * c["candidate_block_size"] == c["pool_positions"]
    # an FP4 main entry: 512 codes of 4 bits + one scale byte per 16 channels
    main = c["head_dim"] // 2 + c["head_dim"] // 16
    assert main == c["main_entry_bytes"]
    # the pages' 890 B/token: (main entry + MXFP4 indexer entry of 128/2 + 128/32 bytes)
    # times 2.5 entries per token (3 encoder copies at ratio 2, 1 decoder copy at ratio 1)
    idx_mxfp4 = c["idx_dim"] // 2 + c["idx_dim"] // 32
    assert (main + idx_mxfp4) * (3 / 2 + 1) == c["global_kv_bytes_per_token"]
    # the same constants are compiled into the C ABI header
    hdr = open(os.path.join(os.path.dirname(GOLDEN), "..", "include", "csa2.h")).read()
    for key, name in [("n_heads", "CSA2_N_HEADS"), ("head_dim", "CSA2_HEAD_DIM"),
                      ("idx_heads", "CSA2_IDX_HEADS"), ("idx_dim", "CSA2_IDX_DIM"),
                      ("index_topk", "CSA2_INDEX_TOPK"), ("sliding_window", "CSA2_SLIDING_WINDOW"),
                      ("candidate_block_size", "CSA2_CANDIDATE_BLOCK_SIZE"),
                      ("candidate_topk_blocks", "CSA2_CANDIDATE_TOPK_BLOCKS")]:
        assert f"#define {name} {c[key]} " in hdr or f"#define {name} {c[key]}\n" in hdr, name


# --------------------------------------------------------------------------- MXFP4 keys

def test_e8m0_every_code_against_torch():
    """All 256 E8M0 scale codes against torch's float8_e8m0fnu decode (a library
    cross-check of the OCP microscaling scale the pages name for the FP4 indexer cache)."""
    import torch
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([O.e8m0_value(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_mxfp4_unit_scale_is_plain_e2m1_and_scales_are_powers_of_two():
    """Scale code 127 leaves the E2M1 values (pinned by the pages' magnitude set), and one
    step of the scale code doubles every channel of its 32-channel group only."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(7, 64), dtype=np.uint8)
    unit = O.mxfp4_key_decode(codes, np.full((7, 4), 127, np.uint8))
    lo, hi = codes & 0xF, codes >> 4
    plain = np.stack([O.e2m1_decode(lo), O.e2m1_decode(hi)], axis=-1).reshape(7, 128)
    assert np.array_equal(unit, plain)
    for g in range(4):
        sc = np.full((7, 4), 127, np.uint8)
        sc[:, g] = 128
        v = O.mxfp4_key_decode(codes, sc)
        assert np.array_equal(v[:, 32 * g:32 * g + 32], 2 * unit[:, 32 * g:32 * g + 32])
        rest = np.ones(128, bool)
        rest[32 * g:32 * g + 32] = False
        assert np.array_equal(v[:, rest], unit[:, rest])


def test_mxfp4_scores_equal_e4m3_scores_on_shared_values():
    """Keys whose values are exact in both formats (E2M1 x 2^-2..2^1 all lie on the E4M3
    grid) give bit-identical scores through the MXFP4 and the E4M3 oracle paths, pinning
    the nibble order, the channel order and the 32-channel scale groups against the
    pinned E4M3 path."""
    rng = np.random.default_rng(11)
    n = 300
    codes = rng.integers(0, 256, size=(n, 64), dtype=np.uint8)
    scales = rng.integers(125, 129, size=(n, 4), dtype=np.uint8)
    vals = O.mxfp4_key_decode(codes, scales)
    lookup = {v: c for c, v in enumerate(O.E4M3_TABLE) if not np.isnan(v)}
    lookup[0.0] = 0
    e4 = np.vectorize(lambda v: lookup[float(v)])(vals).astype(np.uint8)
    assert np.array_equal(O.e4m3_decode(e4), vals)
    q = (rng.standard_normal((32, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = rng.random(32).astype(np.float32)
    a = O.full_scores(q, w, e4, 0, n - 3, n)
    b = O.full_scores_mxfp4(q, w, codes, scales, 0, n - 3, n)
    assert np.array_equal(a, b)
    pool = np.array([3, 0, -1, 30, 36, 37], np.int64)
    padded = np.full(2048, -1, np.int64)
    padded[:len(pool)] = pool
    assert np.array_equal(O.reindex_scores(q, w, e4, 0, n - 3, padded),
                          O.reindex_scores_mxfp4(q, w, codes, scales, 0, n - 3, padded))


def test_mxfp4_encoder_round_trip():
    """The input generator's MXFP4 encoder against the oracle's decoder: decoding then
    re-encoding a canonical row returns it, and encoding lands within half a grid step of
    the scaled value (one full step of 2 where the top of the range saturates at 6)."""
    import torch
    from compressed_kv_cache_csa2_amd import synth
    x = torch.randn(500, 128, generator=torch.Generator().manual_seed(3)) * 3
    c, s = synth.encode_mxfp4_rows(x)
    d = O.mxfp4_key_decode(c.numpy(), s.numpy())
    step = np.repeat(O.E8M0_TABLE[s.numpy()], 32, axis=-1)
    err = np.abs(d - x.double().numpy()) / step
    assert err.max() <= 2.0 + 1e-12
    assert np.all(err[np.abs(x.double().numpy()) / step <= 6.0] <= 1.0 + 1e-12)
    c2, s2 = synth.encode_mxfp4_rows(torch.from_numpy(d).float())
    assert np.array_equal(O.mxfp4_key_decode(c2.numpy(), s2.numpy()), d)


# --------------------------------------------------------------------------- cache writes

def test_e4m3_round_against_torch_with_ties_and_saturation():
    """The oracle's E4M3 rounding against torch's float8_e4m3fn cast on random values,
    exact midpoints between neighbouring codes and subnormals; above 448 it saturates."""
    import torch
    rng = np.random.default_rng(7)
    vals = [rng.standard_normal(20000).astype(np.float32) * s for s in (1e-3, 0.05, 1, 30, 120)]
    mags = O.E4M3_POS
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (mags[:-1] + mags[1:]) / 2)   # exact in fp32
    x = np.concatenate(vals + [mids, -mids, mags.astype(np.float32), np.float32([0.0, -0.0])])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_round(x), ref)
    assert np.array_equal(O.e4m3_round(np.float32([449, 470, 1e6, -1e6])),
                          np.uint8([0x7E, 0x7E, 0x7E, 0xFE]))


def test_e2m1_round_midpoints_and_saturation():
    """Brute force: every value is mapped to the nearest E2M1 magnitude, exact midpoints go
    to the even code, values past 6 saturate, the sign bit never marks a zero."""
    grid = O.E2M1_POS
    mids = (grid[:-1] + grid[1:]) / 2
    want_mid = [0, 2, 2, 4, 4, 6, 6]      # even code of each neighbouring pair
    assert list(O.e2m1_round(mids.astype(np.float32))) == want_mid
    y = np.linspace(-9, 9, 7201).astype(np.float32)
    got = O.e2m1_round(y)
    mag = O.E2M1_TABLE[got & 7]
    best = np.abs(np.abs(y)[:, None] - grid[None, :]).min(axis=1)
    assert np.all(np.abs(np.abs(y) - mag) == np.where(np.abs(y) > 6, np.abs(y) - 6, best))
    assert not np.any((got == 8))


def test_write_quantisers_equal_the_input_generator():
    """Two independent implementations of readings R16 and R19 agree bit for bit: the
    oracle's numpy quantisers and the input generator's torch encoders."""
    import torch
    from compressed_kv_cache_csa2_amd import synth
    g = torch.Generator().manual_seed(9)
    lat = (torch.randn(400, 512, generator=g) * 2).to(torch.bfloat16).float()
    lat[3] = 0.0
    lat[5, 16:32] = 0.0
    p, s = O.fp4_latent_quantize(lat.numpy())
    p2, s2 = synth.encode_fp4_rows(lat)
    assert np.array_equal(p, p2.numpy()) and np.array_equal(s, s2.numpy())
    key = (torch.randn(400, 128, generator=g) * 3).to(torch.bfloat16).float()
    key[7, :32] = 0.0
    c, sc = O.mxfp4_key_quantize(key.numpy())
    c2, sc2 = synth.encode_mxfp4_rows(key)
    assert np.array_equal(c, c2.numpy()) and np.array_equal(sc, sc2.numpy())
    # and decoding what was written stays within the grid step
    d = O.fp4_latent_decode(p, s)
    step = np.repeat(O.E4M3_TABLE[s], 16, axis=-1)
    assert np.all(np.abs(d - lat.numpy()) <= step * 2.0 + 1e-30)


# ------------------------------------------------------------------ block-mean (HISA) filter

def _e4m3_codes_torch(values):
    """E4M3 codes of values exactly representable in E4M3, through torch's cast."""
    t = torch.as_tensor(np.asarray(values, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_bits_torch(values):
    t = torch.as_tensor(np.asarray(values, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_block_mean_keys_closed_forms():
    rng = np.random.default_rng(31)
    # a block of 8 equal rows has that row as its mean (E4M3 values are exact in bf16; a
    # sum starts from +0, so a block of negative zeros has mean +0)
    row = rng.integers(0, 0x7E, size=128).astype(np.uint8) ^ (rng.integers(0, 2, 128).astype(np.uint8) << 7)
    km = O.block_mean_keys(np.tile(row, (8, 1)), 8)
    assert km.shape == (1, 128)
    want = _bf16_bits_torch(torch.from_numpy(row).view(torch.float8_e4m3fn).float().numpy() + 0.0)
    assert np.array_equal(km[0], want)
    # channel 0 holds 1..8 in block 0 (mean 4.5) and 1, 1, 2 in a 3-row tail (4/3, rounded
    # once to float32 and then to bf16); channel 1 holds -3 everywhere
    vals = np.zeros((11, 128), np.float32)
    vals[:8, 0] = np.arange(1, 9)
    vals[8:, 0] = [1, 1, 2]
    vals[:, 1] = -3
    km = O.block_mean_keys(_e4m3_codes_torch(vals), 11)
    assert km.shape == (2, 128)
    got = torch.from_numpy(km.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert got[0, 0] == 4.5 and got[0, 1] == -3 and got[1, 1] == -3
    assert km[1, 0] == _bf16_bits_torch([np.float32(4) / np.float32(3)])[0]
    assert np.all(got[:, 2:] == 0)


def test_block_mean_keys_within_half_a_bf16_step_of_the_exact_mean():
    rng = np.random.default_rng(32)
    n = 8 * 37 + 5
    codes = rng.integers(0, 0x7E, size=(n, 128)).astype(np.uint8) ^ (rng.integers(0, 2, size=(n, 128)).astype(np.uint8) << 7)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    km = O.block_mean_keys(codes, n)
    assert km.shape == (38, 128)
    got = torch.from_numpy(km.view(np.int16)).view(torch.bfloat16).double().numpy()
    for b in range(38):
        exact = vals[8 * b:min(n, 8 * b + 8)].mean(axis=0)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
        assert np.all(np.abs(got[b] - exact) <= 0.5 * ulp * (1 + 2 ** -16) + 1e-300), b
    # fewer visible positions than rows: the tail is ignored
    assert np.array_equal(O.block_mean_keys(codes, 20), O.block_mean_keys(codes[:20], 20))
    assert O.block_mean_keys(codes, 0).shape == (0, 128)


def test_hisa_pool_reduces_to_the_hsi_pool_on_constant_blocks():
    """When the 8 keys of every block are equal, each block mean is that key, so the
    block-mean scores equal the position scores of the block and the two-stage filter's
    pool is the HSI block-max pool."""
    rng = np.random.default_rng(33)
    n = 8 * 3000 + 5
    nb = -(-n // 8)
    blk = rng.integers(0, 0x7E, size=(nb, 128)).astype(np.uint8) ^ (rng.integers(0, 2, size=(nb, 128)).astype(np.uint8) << 7)
    codes = np.repeat(blk, 8, axis=0)[:n]
    q = torch.from_numpy(rng.standard_normal((32, 128)).astype(np.float32)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    w = rng.random(32).astype(np.float32)
    km = O.block_mean_keys(codes, n)
    pool = O.hisa_pool(q_bits, w, km, n)
    s = O.full_scores(q_bits, w, codes, 0, n, n)
    assert np.array_equal(pool, O.hsi_pool(s, n))
    assert len(pool) == 2048 and nb - 1 in pool and np.all(np.diff(pool) > 0)
    # zero keys in the latest block score 0, the lowest possible: it is still kept
    codes0 = codes.copy()
    codes0[8 * (nb - 1):] = 0
    pool0 = O.hisa_pool(q_bits, w, O.block_mean_keys(codes0, n), n)
    assert nb - 1 in pool0
    # a short context keeps every block; an empty one keeps none
    assert np.array_equal(O.hisa_pool(q_bits, w, O.block_mean_keys(codes, 1000), 1000),
                          np.arange(125))
    assert len(O.hisa_pool(q_bits, w, km[:0], 0)) == 0


def test_block_mean_dilutes_an_isolated_peak():
    """The property the HSI section contrasts with: one strong key among seven weak ones
    keeps its full score under the block max but only a share of it under the block mean."""
    q = np.zeros((32, 128), np.float32)
    q[:, 0] = 1.0
    q_bits = _bf16_bits_torch(q)
    w = np.ones(32, np.float32)
    vals = np.zeros((16, 128), np.float32)
    vals[3, 0] = 8.0                       # block 0: one peak
    vals[8:, 0] = 1.5                      # block 1: uniformly moderate
    codes = _e4m3_codes_torch(vals)
    s = O.full_scores(q_bits, w, codes, 0, 16, 16)
    bm = O.block_max(s)
    assert bm[0] > bm[1]                   # block max ranks the peak first
    km = O.block_mean_keys(codes, 16)
    bs = O.index_score_rows(O.bf16_decode(q_bits), w.astype(np.float64), O.bf16_decode(km))
    assert bs[0] == 32 * 1.0 and bs[1] == 32 * 1.5 and bs[0] < bs[1]


# ------------------------------------------------------------------ encoder schedule

def test_swa_layer_is_dense_attention_over_the_window():
    """An SWA-only layer is softmax attention over the window rows alone: torch's scaled
    dot-product attention over the decoded rows, a Reuse layer with an empty selection,
    and a single window row returned exactly."""
    rng = np.random.default_rng(41)
    win = rng.integers(0, 0x7E, size=(200, 512)).astype(np.uint8) ^ (rng.integers(0, 2, size=(200, 512)).astype(np.uint8) << 7)
    q = torch.from_numpy(rng.standard_normal((64, 512)).astype(np.float32)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    res = O.swa_layer(q_bits, win, 30, 128, 1 / math.sqrt(512))
    rows = torch.from_numpy(win[30:158]).view(torch.float8_e4m3fn).double()
    qd = q.double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        qd[None, :, None, :], rows[None, None].expand(1, 64, 128, 512),
        rows[None, None].expand(1, 64, 128, 512), scale=1 / math.sqrt(512))
    assert np.allclose(res["out"], ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-12)
    empty = np.zeros((0, 256), np.uint8), np.zeros((0, 32), np.uint8)
    reuse = O.reuse_layer(np.zeros(0, np.int64), q_bits, *empty, 0, win, 30, 128,
                          1 / math.sqrt(512))
    assert np.array_equal(res["out"], reuse["out"]) and np.array_equal(res["lse"], reuse["lse"])
    one = O.swa_layer(q_bits, win, 7, 1, 1.0)
    row7 = torch.from_numpy(win[7:8]).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(one["out"], np.repeat(row7, 64, 0))


# ------------------------------------------------------------------ compressor (write side)

def _bf16_bits_of(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_compressor_special_cases():
    rng = np.random.default_rng(51)
    c = _bf16_bits_of(rng.standard_normal((9, 512)))
    z = _bf16_bits_of(rng.standard_normal((9, 512)) * 3)
    cv = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double().numpy()
    # m = 1 is the per-token projection itself
    assert np.array_equal(O.compress_entries(c, z, 1), cv)
    # equal gates give the plain mean of each group; only complete groups give entries
    e = O.compress_entries(c, _bf16_bits_of(np.zeros((9, 512))), 2)
    assert e.shape == (4, 512)
    assert np.allclose(e, (cv[0:8:2] + cv[1:8:2]) / 2, rtol=0, atol=1e-15)
    # a dominant gate selects its token
    zd = np.zeros((9, 512), np.float32)
    zd[1::2, :256] = 80.0
    zd[0::2, 256:] = 80.0
    e = O.compress_entries(c, _bf16_bits_of(zd), 2)
    assert np.allclose(e[:, :256], cv[1:8:2, :256], rtol=1e-30, atol=1e-30)
    assert np.allclose(e[:, 256:], cv[0:8:2, 256:], rtol=1e-30, atol=1e-30)


def test_compressor_matches_torch_softmax_pooling():
    """Against torch's softmax over the group axis, and invariant under a per-channel shift
    of the gates (softmax shift invariance)."""
    rng = np.random.default_rng(52)
    c = _bf16_bits_of(rng.standard_normal((12, 512)))
    z = _bf16_bits_of(rng.standard_normal((12, 512)) * 2)
    cv = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double()
    zv = torch.from_numpy(z.view(np.int16)).view(torch.bfloat16).double()
    for m in (2, 3, 4):
        n = 12 // m
        g = torch.softmax(zv[:n * m].reshape(n, m, 512), dim=1)
        ref = (g * cv[:n * m].reshape(n, m, 512)).sum(dim=1).numpy()
        assert np.allclose(O.compress_entries(c, z, m), ref, rtol=1e-13, atol=1e-14)
    # gates on a 1/8 grid stay exact in bf16 after an integer shift
    zq = rng.integers(-32, 33, size=(12, 512)).astype(np.float32) / 8
    shift = np.tile(rng.integers(-4, 5, size=(1, 512)).astype(np.float32), (12, 1))
    a = O.compress_entries(c, _bf16_bits_of(zq), 2)
    b = O.compress_entries(c, _bf16_bits_of(zq + shift), 2)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_index_key_projection_brute_force():
    rng = np.random.default_rng(53)
    ent = rng.standard_normal((5, 512))
    w = _bf16_bits_of(rng.standard_normal((128, 512)) * 0.05)
    wv = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = O.project_index_keys(ent, w)
    assert got.shape == (5, 128)
    for i in range(5):
        for o in (0, 17, 127):
            assert abs(got[i, o] - sum(ent[i, c] * wv[o, c] for c in range(512))) < 1e-12
    # one-hot weights pick channels
    oh = np.zeros((128, 512), np.float32)
    oh[np.arange(128), 4 * np.arange(128)] = 1.0
    assert np.array_equal(O.project_index_keys(ent, _bf16_bits_of(oh)), ent[:, ::4])


# ------------------------------------------------------------------ MXFP8 indexer query

def test_mxfp8_quantize_against_torch_cast():
    """Per 32-channel group: the exponent from torch's log2, the codes from torch's E4M3
    cast of the clamped quotient (an independent rounding); saturation and zero groups."""
    g = torch.Generator().manual_seed(61)
    x = (torch.randn(40, 32, 128, generator=g) * 3).to(torch.bfloat16).float()
    x[0, 0, :32] = 0.0
    x[1, 2, 32:64] *= 2.0 ** 40
    x[2, 3, 64:96] *= 2.0 ** -60
    codes, scales = O.mxfp8_quantize(x.numpy())
    grp = x.reshape(40, 32, 4, 32)
    amax = grp.abs().amax(-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 8 + 127, torch.full_like(amax, 127.0))
    e = e.clamp(1, 254)
    assert np.array_equal(scales, e.to(torch.uint8).numpy())
    quo = (grp * torch.exp2(127 - e).unsqueeze(-1)).clamp(-448, 448)
    want = quo.to(torch.float8_e4m3fn).view(torch.uint8).reshape(40, 32, 128).numpy()
    # a value that rounds to zero keeps its sign in both; compare the values' bits
    assert np.array_equal(codes, want)


def test_mxfp8_round_trip_and_exact_query_scores():
    rng = np.random.default_rng(62)
    x = torch.from_numpy(rng.standard_normal((6, 32, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    codes, scales = O.mxfp8_quantize(x)
    back = O.mxfp8_decode(codes, scales)
    step = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    # within half an E4M3 step of each value, or the saturation gap at the top
    assert np.all(np.abs(back - x) <= np.maximum(np.abs(x) * 2.0 ** -4, step * 2.0 ** -9) + 64 * step)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -4 + step * 2.0 ** -10 + (np.abs(x) > 448 * step) * 64 * step)
    # a query already on the E4M3 grid with group maxima in [256, 448] quantises exactly
    # (scale byte 127), so its scores equal the bf16-query scores over the same MXFP4 keys
    q = rng.integers(0, 0x7E, size=(32, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(32, 128)).astype(np.uint8) << 7)
    q[:, ::32] = 0x7E                                  # 448 in every group
    qv = O.e4m3_decode(q)
    qc, qs = O.mxfp8_quantize(qv.astype(np.float32))
    assert np.all(qs == 127) and np.array_equal(O.e4m3_decode(qc), qv)
    n = 300
    kc = rng.integers(0, 256, size=(n, 64)).astype(np.uint8)
    ks = rng.integers(120, 135, size=(n, 4)).astype(np.uint8)
    w = rng.random(32)
    q_bits = torch.from_numpy(qv.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = O.full_scores_mxfp4(q_bits, w, kc, ks, 0, n - 7, n)
    got = O.full_scores_mxfp4_q8(qc, qs, w, kc, ks, 0, n - 7, n)
    assert np.array_equal(np.isfinite(got), np.isfinite(ref))
    fin = np.isfinite(ref)
    assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-9)


def test_reindex_q8_over_every_block_equals_full_q8():
    """A pool holding every block (in order) rescored with the MXFP8 query reproduces the
    Full-mode MXFP8 scores slot for slot; absent and out-of-range blocks score -inf."""
    rng = np.random.default_rng(63)
    n = 203
    kc = rng.integers(0, 256, size=(n + 5, 64)).astype(np.uint8)
    ks = rng.integers(118, 136, size=(n + 5, 4)).astype(np.uint8)
    q = torch.from_numpy(rng.standard_normal((32, 128)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    qc, qs = O.mxfp8_quantize(q)
    w = rng.random(32)
    nb = -(-n // 8)
    full = O.full_scores_mxfp4_q8(qc, qs, w, kc, ks, 5, n, nb * 8)
    pool = np.arange(nb)
    re = O.reindex_scores_mxfp4_q8(qc, qs, w, kc, ks, 5, n, pool)
    assert np.array_equal(re, full)
    pool2 = np.array([3, -1, nb + 4])
    re2 = O.reindex_scores_mxfp4_q8(qc, qs, w, kc, ks, 5, n, pool2)
    assert np.array_equal(re2[:8], full[24:32]) and np.all(np.isneginf(re2[8:]))


def test_q8_scores_over_e4m3_keys_exact_query_and_pool_identity():
    """An MXFP8 query that is exact (E4M3 grid, unit scales) scores E4M3 keys exactly as the
    bf16 query does; Reindex over a pool of every block reproduces the Full scores."""
    rng = np.random.default_rng(64)
    q = rng.integers(0, 0x7E, size=(32, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(32, 128)).astype(np.uint8) << 7)
    q[:, ::32] = 0x7E
    qv = O.e4m3_decode(q)
    qc, qs = O.mxfp8_quantize(qv.astype(np.float32))
    n = 150
    k = rng.integers(0, 0x7E, size=(n + 3, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(n + 3, 128)).astype(np.uint8) << 7)
    w = rng.random(32)
    q_bits = torch.from_numpy(qv.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = O.full_scores(q_bits, w, k, 3, n - 5, n)
    got = O.full_scores_q8(qc, qs, w, k, 3, n - 5, n)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)) and np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-9)
    nb = -(-n // 8)
    full = O.full_scores_q8(qc, qs, w, k, 3, n, nb * 8)
    assert np.array_equal(O.reindex_scores_q8(qc, qs, w, k, 3, n, np.arange(nb)), full)


# ------------------------------------------------- quantiser rules against brute force

def _nearest_even_e2m1_mag(a):
    """Brute force: index of the E2M1 magnitude nearest to each a >= 0 (float64), ties to
    the even index, everything past 6 taking the last one. Distances to all eight grid
    values are compared directly (no midpoint table)."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d = np.abs(np.asarray(a, np.float64)[..., None] - grid)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equally near grid points prefer the even index (at most two can tie)
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return np.where(np.asarray(a) >= 6.0, 7, pick)


def _all_bf16_in(lo_exp, hi_exp):
    """Every positive bf16 value 2^lo_exp <= v < 2^hi_exp, as float32."""
    e = np.arange(lo_exp, hi_exp, dtype=np.float64)[:, None]
    m = 1.0 + np.arange(128, dtype=np.float64)[None, :] / 128.0
    return (m * 2.0 ** e).ravel().astype(np.float32)


def test_e2m1_ratio_rounding_is_the_exact_quotient_rounding():
    """Reading R16 ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression",
    2.4.4: E2M1 values under an E4M3 scale): each code is the nearest E2M1 magnitude to the
    exact quotient x / s, ties to the even code. Checked over every signed bf16 in
    [2^-31, 2^17) against every finite positive E4M3 scale (about 1.5M pairs). The fp64
    quotient decides every comparison as the exact one does: x has 8 significant bits and
    a midpoint times s at most 7, so x / s either equals a midpoint exactly or differs
    from it by far more than an fp64 rounding."""
    xs = _all_bf16_in(-31, 17)
    xs = np.concatenate([xs, -xs])
    scales = O.E4M3_POS[1:]                      # 126 finite positive scales
    x = xs[:, None].astype(np.float64)
    s = scales[None, :]
    got = O.e2m1_round_ratio(x, s)
    mag = _nearest_even_e2m1_mag(np.abs(x) / s)
    want = mag | (((x < 0) & (mag > 0)).astype(np.int64) << 3)
    assert np.array_equal(got, want.astype(np.uint8))


def test_fp4_latent_quantize_on_exact_midpoints():
    """Groups whose largest value is 6*s (so the scale is exactly s) and whose other values
    sit exactly on the midpoints between neighbouring E2M1 magnitudes times s: every
    midpoint must go to the even code, and the scale byte must decode to s."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    even_code = np.array([0, 2, 2, 4, 4, 6, 6])
    rows = []
    wants = []
    s_vals = []
    for s in O.E4M3_POS[1:]:
        # 6*s has at most 5 significant bits and a midpoint times s at most 7, so every
        # value is a bf16; (6*s)/6 in float32 is s itself, an E4M3 value
        vals = np.concatenate([[6.0 * s], mids * s, -mids * s, [0.0]])
        code = np.concatenate([[7], even_code, even_code | 8, [0]])
        code = np.where(np.concatenate([[6.0], mids, -mids, [0.0]]) == 0, 0, code)
        # the negative midpoint 0.25 rounds to magnitude 0: no sign bit on a zero code
        code[8] = 0
        rows.append(np.resize(vals, 16))
        wants.append(np.resize(code, 16))
        s_vals.append(s)
    x = np.stack(rows).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), np.stack(rows))   # exact in float32 / bf16
    x = np.concatenate([x] * 32, axis=1)                          # 512 channels per row
    payload, scodes = O.fp4_latent_quantize(x)
    assert np.array_equal(O.E4M3_TABLE[scodes], np.repeat(np.array(s_vals)[:, None], 32, 1))
    lo, hi = payload & 0xF, payload >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(x.shape)
    assert np.array_equal(codes, np.concatenate([np.stack(wants)] * 32, axis=1))


def test_mxfp4_key_exponent_recipe_and_codes():
    """Reading R19 (the OCP microscaling recipe for the MXFP4 indexer cache, "DeepSeek-v4.1
    Flash: Pushing the Limits of KV Cache Compression", 2.4.4 and 3.1): for every nonzero
    32-channel group the shared exponent X puts the group's largest magnitude in [4, 8)
    after scaling by 2^-X, so its largest code is 4 or 6; an all-zero group gets byte 127;
    every code is the nearest-even E2M1 rounding of x * 2^-X (brute force)."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((3000, 128)) * np.exp(rng.uniform(-20, 20, (3000, 1)))).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    x[5, :32] = 0.0
    x[6, 32:64] = -0.0
    # amax exactly on powers of two and just below them
    x[7, 0] = 4.0
    x[8, 0] = np.float32(np.nextafter(np.float32(8.0), np.float32(0)))
    x[8, 0] = torch.tensor(x[8, 0]).to(torch.bfloat16).float().item()
    codes, scales = O.mxfp4_key_quantize(x)
    g = x.reshape(3000, 4, 32).astype(np.float64)
    amax = np.abs(g).max(axis=-1)
    X = scales.astype(np.int64) - 127
    nz = amax > 0
    scaled_max = amax * np.ldexp(1.0, -X)
    assert np.all((scaled_max[nz] >= 4.0) & (scaled_max[nz] < 8.0))
    assert np.all(scales[~nz] == 127)
    assert scales[5, 0] == 127 and scales[6, 1] == 127
    lo, hi = codes & 0xF, codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(3000, 128).reshape(3000, 4, 32)
    mag = _nearest_even_e2m1_mag(np.abs(g) * np.ldexp(1.0, -X)[..., None])
    want = mag | (((g < 0) & (mag > 0)).astype(np.int64) << 3)
    assert np.array_equal(c, want)
    top = (c & 7).max(axis=-1)
    assert set(np.unique(top[nz]).tolist()) <= {6, 7}          # magnitudes 4 and 6


# ------------------------------------------------------------------ Reindex layer as a whole

def test_reindex_layer_composition_and_full_query_identity():
    """reindex_layer is the Reindex mode of "DeepSeek-v4.1 Flash: Pushing the Limits of KV
    Cache Compression" 2.3.2 / 2.3.4: scores over the pool, its own Top-K inside the pool,
    slots mapped through the pool, attention with those indices. (a) With a fresh query it
    equals that chain built from the oracle's pieces; (b) given the Full layer's own
    indexer query, weights, attention query and window it reproduces the Full layer's
    indices and output exactly (every Full winner lies in the pool, and pool slots run in
    ascending position order, so the gather order is the same)."""
    n = 9001
    k_cache, p, s, win, q_idx, w, q = _tiny_sequence(31, n)
    scale = 1 / math.sqrt(512)
    full = O.full_layer(q_idx, w, k_cache, 0, n, q, p, s, win, 0, 128, scale, with_pool=True)
    same = O.reindex_layer(q_idx, w, k_cache, 0, n, full["pool"], q, p, s, win, 0, 128, scale)
    assert np.array_equal(same["idx"], full["idx"])
    assert np.array_equal(same["out"], full["out"]) and np.array_equal(same["lse"], full["lse"])
    _, _, _, win2, q_idx2, w2, q2 = _tiny_sequence(32, 16)
    fresh = O.reindex_layer(q_idx2, w2, k_cache, 0, n, full["pool"], q2, p, s, win2, 0, 100,
                            scale)
    padded = np.full(2048, -1, np.int64)
    padded[:len(full["pool"])] = full["pool"]
    rs = O.reindex_scores(q_idx2, w2, k_cache, 0, n, padded)
    idx = O.slots_to_positions(O.topk_slots(rs, 512), padded)
    ref = O.reuse_layer(idx, q2, p, s, 0, win2, 0, 100, scale)
    assert np.array_equal(fresh["scores"], rs) and np.array_equal(fresh["idx"], idx)
    assert np.array_equal(fresh["out"], ref["out"]) and np.array_equal(fresh["lse"], ref["lse"])
    # every selected position lies in a pool block and is visible
    assert np.all(np.isin(idx // 8, full["pool"])) and np.all(idx < n) and len(idx) == 512
    # a short context (ragged last block): every visible position is selected by both
    m = 301
    short = O.full_layer(q_idx, w, k_cache, 0, m, q, p, s, win, 0, 128, scale, with_pool=True)
    re_short = O.reindex_layer(q_idx, w, k_cache, 0, m, short["pool"], q, p, s, win, 0, 128,
                               scale)
    assert np.array_equal(short["idx"], np.arange(m))
    assert np.array_equal(re_short["idx"], np.arange(m))
    assert np.array_equal(re_short["out"], short["out"])


# ------------------------------------------------------------------ helpers pinned directly

def test_f32_to_bf16_bits_rounds_to_nearest_even():
    """f32_to_bf16_bits against torch's float32 -> bfloat16 conversion (an independent
    implementation of the same rounding) over random finite bit patterns, and the ties by
    hand: a float32 exactly halfway between two bf16 values goes to the one whose last
    mantissa bit is 0."""
    rng = np.random.default_rng(61)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # keep values whose rounding stays finite (the largest bf16 is below float32's maximum)
    x = x[np.abs(x) < np.float32(3.38e38)]
    assert np.array_equal(O.f32_to_bf16_bits(x), _bf16_bits_torch(x))
    one = 0x3F80
    cases = [
        (1.0 + 2.0 ** -8, one),                      # halfway, lower neighbour even
        (1.0 + 2.0 ** -7 + 2.0 ** -8, one + 2),      # halfway, upper neighbour even
        (1.0 + 2.0 ** -8 + 2.0 ** -20, one + 1),     # just above halfway
        (1.0 + 2.0 ** -8 - 2.0 ** -20, one),         # just below halfway
        (-(1.0 + 2.0 ** -8), 0x8000 | one),          # sign carried through
        (2.0 ** -130, 0x0008),                       # a bf16 subnormal, exact
        (2.0 ** -140, 0x0000),                       # below half the smallest bf16 subnormal
    ]
    for v, want in cases:
        got = int(O.f32_to_bf16_bits(np.array([v], np.float32))[0])
        assert got == want, (v, hex(got), hex(want))


def test_gather_attention_entries_brute_force():
    """The attended set of a tiny query, built entry by entry from the scalar decoders:
    main rows at the valid selected positions (in their order, -1 skipped, duplicates kept)
    with c[i] = E2M1(code i) * E4M3(scale[i // 16]), code 2m the low nibble of byte m, then
    the window rows as plain E4M3 values, at most 128 of them."""
    rng = np.random.default_rng(62)
    n_rows, kv_start = 12, 3
    kv_fp4 = rng.integers(0, 256, size=(n_rows + kv_start, 256)).astype(np.uint8)
    kv_scale = rng.integers(0, 0x7F, size=(n_rows + kv_start, 32)).astype(np.uint8)
    window = rng.integers(0, 0x7F, size=(140, 512)).astype(np.uint8)
    window ^= (rng.integers(0, 2, size=window.shape).astype(np.uint8) << 7)
    topk = np.array([4, -1, 0, 11, 4, -1], np.int32)

    def main_row(r):
        out = np.empty(512)
        for i in range(512):
            byte = int(kv_fp4[r, i // 2])
            code = byte & 0xF if i % 2 == 0 else byte >> 4
            out[i] = O.e2m1_value(code) * O.e4m3_value(int(kv_scale[r, i // 16]))
        return out

    for swa_start, n_swa, n_win in ((5, 3, 3), (0, 0, 0), (2, 200, 128)):
        got = O.gather_attention_entries(topk, kv_fp4, kv_scale, kv_start, window, swa_start,
                                         n_swa)
        want = [main_row(kv_start + p) for p in topk if p >= 0]
        want += [np.array([O.e4m3_value(int(b)) for b in window[swa_start + j]])
                 for j in range(n_win)]
        assert got.shape == (4 + n_win, 512)
        assert np.array_equal(got, np.array(want))
