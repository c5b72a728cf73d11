"""Plain fp64 CPU oracle of the CSA2 read path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link this
module: only the test suite, the smoke check of the graft entry point and the CPU
baseline leg of the benchmark do. It shares no code with the HIP library and does not
import the input generator; it receives plain numpy arrays.

Every function is the plain definition of one step, written from the pages:
  [V41F-ARCH] "DeepSeek-V4.1-Flash - Architecture" (reading notes), section 1 (the KV
              and compression-weight projections), section 2 (CSA2 modes,
              layer schedule, main attention settings), section 3 (Hierarchical Sparse
              Indexer), section 4 (KV cache formats and storage).
  [V41F-BLOG] "DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression",
              2.3.1 (indexer, compressor), 2.3.2 (Full / Reindex / Reuse modes),
              2.3.4 (HSI and its block-max pool), 2.4.4 (FP4 main KV cache),
              3.1 (what one cache entry holds), 3.3.1-3.3.2 (the readout of one layer).
Where the pages are silent or garbled, the reading taken is named in the docstring
(R-numbers follow the readings table of the design notes).

Arithmetic is float64. Codes are decoded from their bit definitions; a decode table is
only the closed form evaluated at every code and then indexed. Parity status: every
function below is pinned by a CPU test (exhaustive codec checks, brute force on tiny
inputs, library cross-checks, closed forms and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf

# --------------------------------------------------------------------------------------
# Formats
# --------------------------------------------------------------------------------------


def e4m3_value(code: int) -> float:
    """OCP FP8 E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.

    [V41F-BLOG] 2.4.4 and [V41F-ARCH] 4: the FP4 main KV keeps one E4M3 scale per 16
    channels, and the SWA cache stays in FP8. Exponent field 0 is subnormal
    (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity, so the largest value is 448.
    """
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(code: int) -> float:
    """FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.

    [V41F-BLOG] 2.4.4 and [V41F-ARCH] 4: main-KV values are E2M1 codes. Exponent field 0
    is subnormal (0.5*m); the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    code = int(code) & 0xF
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """OCP microscaling E8M0 scale: an unsigned 8-bit exponent with bias 127, value
    2^(code - 127); 0xFF is NaN.

    [V41F-BLOG] 2.4.4 (the indexer cache is FP4 in the OCP MXFP4 format) and 3.1 (an MXFP4
    indexer K entry is its E2M1 payload plus one scale byte per 32 channels).
    """
    code = int(code) & 0xFF
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E4M3 bytes to float64 (e4m3_value at every element)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of 4-bit E2M1 codes (0..15) to float64."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to float64: they are the top half of a float32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp4_latent_decode(payload: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Main-KV latent rows to float64: c[i] = E2M1(code i) * E4M3(scale[i // 16]).

    [V41F-BLOG] 2.4.4 / [V41F-ARCH] 4: E2M1 values, one E4M3 scale per 16 channels and no
    second-level global scale. Reading R4 (the pages give no packing): channel 2m is the
    low nibble of byte m, channel 2m+1 the high nibble.
    payload [..., 256] uint8, scales [..., 32] uint8 -> [..., 512] float64.
    """
    payload = np.asarray(payload, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = payload & 0xF
    hi = payload >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(payload.shape[:-1] + (payload.shape[-1] * 2,))
    values = e2m1_decode(codes)
    scale_per_channel = np.repeat(e4m3_decode(scales), 16, axis=-1)
    return values * scale_per_channel


def mxfp4_key_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 indexer-key rows to float64: k[c] = E2M1(code c) * E8M0(scale[c // 32]).

    [V41F-BLOG] 2.4.4 and 3.1: 128 channels of E2M1 with one E8M0 scale per 32 channels
    (OCP MXFP4). Reading R4's packing: channel 2m is the low nibble of byte m.
    codes [..., 64] uint8, scales [..., 4] uint8 -> [..., 128] float64.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lo = codes & 0xF
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (codes.shape[-1] * 2,))
    return e2m1_decode(c) * np.repeat(E8M0_TABLE[scales], 32, axis=-1)


# --------------------------------------------------------------------------------------
# Cache writes (quantisers)
# --------------------------------------------------------------------------------------
#
# [V41F-BLOG] 2.4.4: the main KV is stored as E2M1 with one E4M3 scale per 16 channels and
# no global scale, quantised after RoPE; the sliding-window cache stays FP8; the indexer
# cache is OCP MXFP4. The pages give no rounding rule: readings R16 (main KV) and R19
# (MXFP4 keys) take round-to-nearest-even onto each grid, saturating at its largest value.
# Every decision is taken on float32 values (the inputs are bf16, exact in float32, and
# the quotients are float32 divisions), the precision the kernels decide in.

E4M3_POS = E4M3_TABLE[:127]          # codes 0..126: the finite non-negative E4M3 values
E2M1_POS = E2M1_TABLE[:8]            # codes 0..7


def _round_to_grid(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest value of an increasing grid to each a >= 0, ties to the even
    index; values beyond the last grid point take the last index (saturation)."""
    a = np.asarray(a, np.float64)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 1, len(grid) - 1)
    lo = hi - 1
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.where(a >= grid[-1], len(grid) - 1, idx).astype(np.int64)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3 bytes: nearest with ties to the even code, saturating at 448;
    the sign bit is that of x (a negative value that rounds to zero gives 0x80)."""
    x = np.asarray(x, np.float32)
    code = _round_to_grid(np.abs(x).astype(np.float64), E4M3_POS).astype(np.uint8)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def e2m1_round(y: np.ndarray) -> np.ndarray:
    """float32 values -> E2M1 codes: nearest grid magnitude with ties to the even code,
    saturating at 6; the sign bit only on a nonzero code."""
    y = np.asarray(y, np.float32)
    mag = _round_to_grid(np.abs(y).astype(np.float64), E2M1_POS).astype(np.uint8)
    return mag | (((y < 0) & (mag > 0)).astype(np.uint8) << 3)


def e2m1_round_ratio(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E2M1 codes of the exact quotient x / s (s > 0): nearest grid magnitude, ties to the
    even code, saturating at 6. |x| is compared with each midpoint times s, which is exact
    (a midpoint has at most 3 significant bits and an E4M3 scale 4)."""
    a = np.abs(np.asarray(x, np.float64))
    s = np.asarray(s, np.float64)
    mids = (E2M1_POS[:-1] + E2M1_POS[1:]) / 2          # 0.25, 0.75, ..., 5
    mag = np.zeros(np.broadcast(a, s).shape, np.int64)
    for i, m in enumerate(mids):
        t = m * s
        # the midpoint between codes i and i+1 goes to the even one
        mag += (a >= t) if (i + 1) % 2 == 0 else (a > t)
    sign = (np.asarray(x) < 0) & (mag > 0)
    return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Codes [..., 2n] -> bytes [..., n], channel 2m in the low nibble of byte m (R4)."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def fp4_latent_quantize(x: np.ndarray):
    """Main-KV rows (float32 view of bf16) -> (payload [..., 256], scales [..., 32]).

    Reading R16 of [V41F-BLOG] 2.4.4: per 16-channel group the scale is E4M3(amax / 6)
    (amax / 6 as a float32 division) and each value is the E2M1 rounding of the exact
    quotient x / scale; a zero scale gives zero codes.
    """
    x = np.asarray(x, np.float32)
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // 16, 16))
    amax = np.abs(g).max(axis=-1)
    s_code = e4m3_round(amax / np.float32(6.0))
    s = E4M3_TABLE[s_code]
    codes = np.where((s > 0)[..., None], e2m1_round_ratio(g, s[..., None]), 0).astype(np.uint8)
    return _pack_nibbles(codes.reshape(x.shape)), s_code


def mxfp4_key_quantize(x: np.ndarray):
    """Indexer-K rows (float32 view of bf16) -> (codes [..., 64], E8M0 scales [..., 4]).

    Reading R19 (the OCP microscaling recipe for [V41F-BLOG] 2.4.4's MXFP4 indexer cache):
    per 32-channel group the shared exponent is floor(log2 amax) - 2 (2 = E2M1's largest
    exponent), stored as a biased byte kept in 1..254; values are E2M1(x / 2^X). An
    all-zero group gets the unit scale byte 127.
    """
    x = np.asarray(x, np.float32)
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(g).max(axis=-1).astype(np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = m * 2^e, m in [0.5, 1)
    code_s = np.where(amax > 0, np.clip(e - 1 - 2 + 127, 1, 254), 127).astype(np.int64)
    q = (g.astype(np.float64) * np.ldexp(1.0, 127 - code_s)[..., None]).astype(np.float32)
    codes = e2m1_round(q)
    return _pack_nibbles(codes.reshape(x.shape)), code_s.astype(np.uint8)


# --------------------------------------------------------------------------------------
# Indexer
# --------------------------------------------------------------------------------------


def index_score_rows(q_idx: np.ndarray, w: np.ndarray, k_rows: np.ndarray) -> np.ndarray:
    """Lightning-indexer score of some cache rows for one query.

    [V41F-BLOG] 3.3.2 (the indexer query, a per-head weight, and the shared indexer K
    produce the score of every entry) with [V41F-ARCH] 2 (32 indexer heads of dim 128).
    The printed formula is lost; reading R1 takes the DSA lightning indexer form
        s_j = sum_h w_h * ReLU(q_h . k_j)
    with no extra scale (a positive scale changes no selection).
    q_idx [32,128] float64, w [32] float64, k_rows [n,128] float64 -> [n] float64.
    """
    dots = k_rows @ q_idx.T                    # [n, 32]: q_h . k_j
    return np.maximum(dots, 0.0) @ w           # sum_h w_h ReLU(.)


def full_scores(q_idx: np.ndarray, w: np.ndarray, k_cache_codes: np.ndarray,
                kv_start: int, n_visible: int, ld: int) -> np.ndarray:
    """Full mode: score every causally visible position 0 <= j < n_visible of one query.

    [V41F-BLOG] 2.3.4 (a Full layer scores all causally visible main-KV positions) and
    2.3.2 (Full mode runs the indexer itself). Slots at or beyond n_visible are -inf.
    q_idx [32,128] bf16 bits, w [32] float32, k_cache_codes [E,128] E4M3 bytes.
    """
    out = np.full(ld, NEG_INF)
    n = min(int(n_visible), int(ld))
    if n > 0:
        rows = e4m3_decode(k_cache_codes[kv_start:kv_start + n])
        out[:n] = index_score_rows(bf16_decode(q_idx), np.asarray(w, np.float64), rows)
    return out


def reindex_scores(q_idx: np.ndarray, w: np.ndarray, k_cache_codes: np.ndarray,
                   kv_start: int, n_visible: int, pool_blocks: np.ndarray,
                   block_size: int = 8) -> np.ndarray:
    """Reindex mode: score only the positions of the candidate pool.

    [V41F-BLOG] 2.3.2 (Reindex computes its own indexer Q and rescores the reused keys)
    and 2.3.4 (later index layers score only the pool of their query). Slot r stands for
    position pool_blocks[r // 8]*8 + r % 8; a negative block id or a position at or
    beyond n_visible gives -inf.
    """
    pool_blocks = np.asarray(pool_blocks, dtype=np.int64)
    n_slots = pool_blocks.shape[0] * block_size
    out = np.full(n_slots, NEG_INF)
    slot = np.arange(n_slots)
    block = pool_blocks[slot // block_size]
    pos = block * block_size + slot % block_size
    ok = (block >= 0) & (pos < n_visible)
    if ok.any():
        rows = e4m3_decode(k_cache_codes[kv_start + pos[ok]])
        out[ok] = index_score_rows(bf16_decode(q_idx), np.asarray(w, np.float64), rows)
    return out


def full_scores_mxfp4(q_idx: np.ndarray, w: np.ndarray, k_codes: np.ndarray,
                      k_scales: np.ndarray, kv_start: int, n_visible: int, ld: int) -> np.ndarray:
    """full_scores with MXFP4 indexer keys (mxfp4_key_decode rows)."""
    out = np.full(ld, NEG_INF)
    n = min(int(n_visible), int(ld))
    if n > 0:
        rows = mxfp4_key_decode(k_codes[kv_start:kv_start + n], k_scales[kv_start:kv_start + n])
        out[:n] = index_score_rows(bf16_decode(q_idx), np.asarray(w, np.float64), rows)
    return out


def reindex_scores_mxfp4(q_idx: np.ndarray, w: np.ndarray, k_codes: np.ndarray,
                         k_scales: np.ndarray, kv_start: int, n_visible: int,
                         pool_blocks: np.ndarray, block_size: int = 8) -> np.ndarray:
    """reindex_scores with MXFP4 indexer keys."""
    pool_blocks = np.asarray(pool_blocks, dtype=np.int64)
    n_slots = pool_blocks.shape[0] * block_size
    out = np.full(n_slots, NEG_INF)
    slot = np.arange(n_slots)
    block = pool_blocks[slot // block_size]
    pos = block * block_size + slot % block_size
    ok = (block >= 0) & (pos < n_visible)
    if ok.any():
        r = kv_start + pos[ok]
        rows = mxfp4_key_decode(k_codes[r], k_scales[r])
        out[ok] = index_score_rows(bf16_decode(q_idx), np.asarray(w, np.float64), rows)
    return out


# --------------------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------------------


def topk_slots(scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, #candidates) slots with the largest scores, in ascending slot order.

    [V41F-BLOG] 2.3.4 and [V41F-ARCH] 2: keep index_topk = 512 entries per query.
    Readings R9/R10: -inf (not visible) and NaN are never candidates; ties go to the
    lower slot, i.e. the order is (score descending, slot ascending).
    """
    scores = np.asarray(scores, dtype=np.float64)
    cand = np.nonzero(~np.isnan(scores) & (scores > NEG_INF))[0]
    order = np.lexsort((cand, -scores[cand]))          # primary -score, secondary slot
    return np.sort(cand[order[:k]])


def slots_to_positions(slots: np.ndarray, pool_blocks: np.ndarray | None,
                       block_size: int = 8) -> np.ndarray:
    """Map selected slots to cache positions: identity in Full mode, through the pool
    (block id * 8 + offset) in Reindex mode ([V41F-BLOG] 2.3.4)."""
    slots = np.asarray(slots, dtype=np.int64)
    if pool_blocks is None:
        return slots
    pool_blocks = np.asarray(pool_blocks, dtype=np.int64)
    return pool_blocks[slots // block_size] * block_size + slots % block_size


def block_max(scores: np.ndarray, block_size: int = 8) -> np.ndarray:
    """Maximum of each block of 8 consecutive slots, the last block padded with -inf.

    [V41F-BLOG] 2.3.4: the Full layer pads its scores with -inf up to a multiple of the
    block size, splits them into blocks of 8 and takes the max of each block.
    """
    scores = np.asarray(scores, dtype=np.float64)
    nb = -(-scores.shape[0] // block_size)
    padded = np.full(nb * block_size, NEG_INF)
    padded[:scores.shape[0]] = scores
    return padded.reshape(nb, block_size).max(axis=1)


def hsi_pool(scores: np.ndarray, n_visible: int, block_size: int = 8,
             n_keep: int = 2048) -> np.ndarray:
    """HSI candidate pool of one query: the kept block ids in ascending order.

    [V41F-BLOG] 2.3.4 ("How does the Full Mode layer build the candidate pool") and
    [V41F-ARCH] 3: block max over the visible scores, the block holding the latest
    visible position forced to +inf (reading R13) so it always occupies a slot, then the
    top min(2048, #blocks) blocks (ties to the lower block id, reading R10; -inf blocks
    are never kept). The pool's positions are the union of the kept blocks, clipped to
    the visible width.
    """
    n = int(n_visible)
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    bm = block_max(np.asarray(scores, dtype=np.float64)[:n], block_size)
    bm[(n - 1) // block_size] = np.inf
    return topk_slots(bm, n_keep)


def mxfp8_quantize(x: np.ndarray):
    """Rows of bf16 values (as float32) -> MXFP8 (E4M3 codes [..., d], E8M0 scales [..., d/32]).

    The pages' V4 lineage runs the indexer in low precision (FP4 keys, [V41F-BLOG] 2.4.4,
    3.1); reading R24 quantises the indexer query with the OCP microscaling recipe for
    E4M3 elements: per 32-channel group the shared exponent is floor(log2 amax) - 8 (8 =
    E4M3's largest exponent), stored biased and kept in 1..254 (127 for an all-zero group),
    and each value is E4M3(x / 2^X), nearest even, saturating at 448."""
    x = np.asarray(x, np.float32)
    g = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(g).max(axis=-1).astype(np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = m * 2^e, m in [0.5, 1)
    code_s = np.where(amax > 0, np.clip(e - 1 - 8 + 127, 1, 254), 127).astype(np.int64)
    q = (g.astype(np.float64) * np.ldexp(1.0, 127 - code_s)[..., None]).astype(np.float32)
    return e4m3_round(q).reshape(x.shape), code_s.astype(np.uint8)


def mxfp8_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 rows -> float64: E4M3 value of each code times 2^(scale - 127) of its group."""
    v = e4m3_decode(np.asarray(codes, np.uint8))
    sc = np.repeat(np.ldexp(1.0, np.asarray(scales, np.int64) - 127), 32, axis=-1)
    return v * sc


def full_scores_mxfp4_q8(q_codes, q_scales, w, k_codes, k_scales, kv_start, n_visible, width):
    """Full-mode scores with an MXFP8 indexer query over MXFP4 keys (reading R24): the
    index score of [V41F-BLOG] 2.3.1 on the decoded query and keys; slots past n_visible
    are -inf."""
    out = np.full(int(width), NEG_INF)
    n = min(int(n_visible), int(width))
    if n > 0:
        rows = np.arange(int(kv_start), int(kv_start) + n)
        k = mxfp4_key_decode(np.asarray(k_codes)[rows], np.asarray(k_scales)[rows])
        out[:n] = index_score_rows(mxfp8_decode(q_codes, q_scales), np.asarray(w, np.float64), k)
    return out


def reindex_scores_mxfp4_q8(q_codes, q_scales, w, k_codes, k_scales, kv_start, n_visible,
                            pool_blocks, block_size: int = 8) -> np.ndarray:
    """reindex_scores with an MXFP8 query over MXFP4 keys (reading R24): slot s of the pool
    scores position 8 * pool[s / 8] + s % 8 with the decoded query; absent slots -inf."""
    pool_blocks = np.asarray(pool_blocks, dtype=np.int64)
    n_slots = pool_blocks.shape[0] * block_size
    out = np.full(n_slots, NEG_INF)
    slot = np.arange(n_slots)
    block = pool_blocks[slot // block_size]
    pos = block * block_size + slot % block_size
    ok = (block >= 0) & (pos < n_visible)
    if ok.any():
        r = kv_start + pos[ok]
        rows = mxfp4_key_decode(np.asarray(k_codes)[r], np.asarray(k_scales)[r])
        out[ok] = index_score_rows(mxfp8_decode(q_codes, q_scales), np.asarray(w, np.float64), rows)
    return out


def full_scores_q8(q_codes, q_scales, w, k_cache_codes, kv_start, n_visible, width):
    """Full-mode scores with an MXFP8 indexer query over E4M3 keys (reading R24)."""
    out = np.full(int(width), NEG_INF)
    n = min(int(n_visible), int(width))
    if n > 0:
        k = e4m3_decode(np.asarray(k_cache_codes)[int(kv_start):int(kv_start) + n])
        out[:n] = index_score_rows(mxfp8_decode(q_codes, q_scales), np.asarray(w, np.float64), k)
    return out


def reindex_scores_q8(q_codes, q_scales, w, k_cache_codes, kv_start, n_visible, pool_blocks,
                      block_size: int = 8) -> np.ndarray:
    """reindex_scores with an MXFP8 query over E4M3 keys (reading R24)."""
    pool_blocks = np.asarray(pool_blocks, dtype=np.int64)
    n_slots = pool_blocks.shape[0] * block_size
    out = np.full(n_slots, NEG_INF)
    slot = np.arange(n_slots)
    block = pool_blocks[slot // block_size]
    pos = block * block_size + slot % block_size
    ok = (block >= 0) & (pos < n_visible)
    if ok.any():
        rows = e4m3_decode(np.asarray(k_cache_codes)[kv_start + pos[ok]])
        out[ok] = index_score_rows(mxfp8_decode(q_codes, q_scales), np.asarray(w, np.float64), rows)
    return out


# --------------------------------------------------------------------------------------
# Write side: the compressor and the indexer-key projection
# --------------------------------------------------------------------------------------


def compress_entries(c_bits: np.ndarray, z_bits: np.ndarray, m: int) -> np.ndarray:
    """Main-KV entries from m adjacent tokens by gated pooling, fp64 [T // m, d].

    [V41F-ARCH] 1 (the design): per layer the KV content C = H W_KV and the compression
    weights Z = H W_Z are projections of the hidden state; [V41F-BLOG] 3.3.2: the
    compressor is gated pooling that becomes a per-token projection at m = 1; 2.3.1: no
    overlap between the tokens of adjacent entries and no absolute position embedding.
    Reading R22: entry j, channel c = sum over the tokens i of group j (tokens jm .. jm+m-1)
    of softmax_i(Z[., c]) * C[i, c]; only complete groups give an entry. c_bits and z_bits
    are the bf16 projections [T, d]."""
    cv = bf16_decode(np.asarray(c_bits, np.uint16))
    zv = bf16_decode(np.asarray(z_bits, np.uint16))
    n = cv.shape[0] // m
    out = np.zeros((n, cv.shape[1]))
    for j in range(n):
        zg = zv[j * m:(j + 1) * m]
        g = np.exp(zg - zg.max(axis=0))
        g /= g.sum(axis=0)
        out[j] = (g * cv[j * m:(j + 1) * m]).sum(axis=0)
    return out


def project_index_keys(entries: np.ndarray, w_ik_bits: np.ndarray) -> np.ndarray:
    """Indexer keys as a projection of main-KV entries, fp64 [n, 128].

    [V41F-BLOG] 2.3.1: CSA2 obtains the indexer K by projecting the main KV entries instead
    of compressing the hidden state separately. Reading R23: k = entry . W_IK^T with W_IK
    a bf16 [128, d] matrix (output channel major); entries are the bf16 main-KV rows."""
    return np.asarray(entries, np.float64) @ bf16_decode(np.asarray(w_ik_bits, np.uint16)).T


# --------------------------------------------------------------------------------------
# HISA-style block-mean coarse filter (the alternative the pages contrast HSI with)
# --------------------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns, nearest with ties to even (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def block_mean_keys(k_codes: np.ndarray, n_visible: int, block_size: int = 8) -> np.ndarray:
    """Mean indexer key of each block of 8 visible positions, as bf16 bits [nb, 128].

    [V41F-BLOG] 2.3.4 (the HISA paragraphs): the prefix is cut into blocks of consecutive
    positions and each block keeps the mean of its indexer keys, which a first stage
    scores. Reading R20: the mean runs over the block's visible positions (the last block
    may be partial); the sum of E4M3 values is exact in float32, the division by the count
    is a float32 division, and the mean is stored as bf16 (nearest even). The sum starts
    from +0, so a block of negative zeros has mean +0.
    """
    n = int(n_visible)
    nb = -(-n // block_size)
    rows = e4m3_decode(np.asarray(k_codes, np.uint8)[:n])
    out = np.zeros((nb, rows.shape[1]), np.uint16)
    for b in range(nb):
        blk = rows[block_size * b:min(n, block_size * b + block_size)]
        mean32 = np.float32(blk.sum(axis=0)) / np.float32(blk.shape[0])
        out[b] = f32_to_bf16_bits(mean32)
    return out


def hisa_pool(q_idx: np.ndarray, w: np.ndarray, km_bits: np.ndarray, n_visible: int,
              block_size: int = 8, n_keep: int = 2048) -> np.ndarray:
    """First stage of the block-mean filter for one query: score every block's mean key
    with the indexer and keep the top min(n_keep, #blocks) blocks, the block holding the
    latest visible position forced in as in the HSI pool (reading R13), ascending ids."""
    n = int(n_visible)
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    bs = index_score_rows(bf16_decode(q_idx), np.asarray(w, np.float64), bf16_decode(km_bits))
    bs[(n - 1) // block_size] = np.inf
    return topk_slots(bs, n_keep)


def pool_bitmap(blocks: np.ndarray, n_visible: int, block_size: int = 8) -> np.ndarray:
    """The pool as a position bitmap: each kept block's flag repeated 8 times and cut to
    the visible width ([V41F-BLOG] 2.3.4)."""
    nb = -(-int(n_visible) // block_size)
    flags = np.zeros(nb, dtype=bool)
    flags[np.asarray(blocks, dtype=np.int64)] = True
    return np.repeat(flags, block_size)[:int(n_visible)]


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------


def sparse_attention(q: np.ndarray, entries: np.ndarray, softmax_scale: float):
    """Joint softmax attention of all heads of one query over a set of entries.

    [V41F-BLOG] 3.3.1-3.3.2: the selected main-KV entries and the SWA entries are
    concatenated into one attention, and each entry serves as key and as value (the
    output is a convex combination of the attended vectors). [V41F-ARCH] 2: 64 heads of
    dim 512. Reading R6: logits are softmax_scale * q_h . c_j (the pages lose the
    constant; 1/sqrt(512) is passed in by the callers).
    q [64,512] float64, entries [n,512] float64 -> (out [64,512], lse [64]).
    An empty set gives out = 0 and lse = -inf.
    """
    n_heads = q.shape[0]
    if entries.shape[0] == 0:
        return np.zeros((n_heads, entries.shape[1])), np.full(n_heads, NEG_INF)
    logits = softmax_scale * (q @ entries.T)                 # [heads, n]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    out = p @ entries
    lse = (mx + np.log(z))[:, 0]
    return out, lse


def gather_attention_entries(topk_pos: np.ndarray, kv_fp4: np.ndarray, kv_scale: np.ndarray,
                             kv_start: int, window_kv: np.ndarray, swa_start: int,
                             n_swa: int) -> np.ndarray:
    """The attended set of one query: decoded main entries at the selected positions
    (skipping -1 padding) followed by the SWA rows ([V41F-BLOG] 3.3.2; reading R8: the
    window is FP8 without a scale and is not de-duplicated against the selection)."""
    pos = np.asarray(topk_pos, dtype=np.int64)
    pos = pos[pos >= 0]
    rows = kv_start + pos
    main = fp4_latent_decode(kv_fp4[rows], kv_scale[rows]) if rows.size else np.zeros((0, 512))
    n_swa = max(0, min(int(n_swa), 128))
    win = e4m3_decode(window_kv[swa_start:swa_start + n_swa])
    return np.concatenate([main, win.reshape(-1, 512)], axis=0)


# --------------------------------------------------------------------------------------
# One layer of each mode ([V41F-BLOG] 2.3.2, 3.3.3; [V41F-ARCH] 2 "CSA2 modes")
# --------------------------------------------------------------------------------------


def full_layer(q_idx, w, k_cache, kv_start, n_visible, q, kv_fp4, kv_scale, window_kv,
               swa_start, n_swa, softmax_scale, k=512, with_pool=False, k_scales=None):
    """Full mode for one query: score everything visible, take the Top-K, optionally
    build the HSI pool from the same scores, and attend. Returns a dict. With k_scales
    the indexer keys are MXFP4 (k_cache holds their codes)."""
    if k_scales is None:
        scores = full_scores(q_idx, w, k_cache, kv_start, n_visible, n_visible)
    else:
        scores = full_scores_mxfp4(q_idx, w, k_cache, k_scales, kv_start, n_visible, n_visible)
    idx = slots_to_positions(topk_slots(scores, k), None)
    res = {"scores": scores, "idx": idx}
    if with_pool:
        res["pool"] = hsi_pool(scores, n_visible)
    ents = gather_attention_entries(idx, kv_fp4, kv_scale, kv_start, window_kv, swa_start, n_swa)
    res["out"], res["lse"] = sparse_attention(bf16_decode(q), ents, softmax_scale)
    return res


def reindex_layer(q_idx, w, k_cache, kv_start, n_visible, pool, q, kv_fp4, kv_scale,
                  window_kv, swa_start, n_swa, softmax_scale, k=512, k_scales=None):
    """Reindex mode for one query: rescore only the pool with this layer's indexer
    query, take its own Top-K inside the pool, and attend (MXFP4 keys with k_scales)."""
    padded = np.full(2048, -1, dtype=np.int64)
    padded[:len(pool)] = pool
    if k_scales is None:
        scores = reindex_scores(q_idx, w, k_cache, kv_start, n_visible, padded)
    else:
        scores = reindex_scores_mxfp4(q_idx, w, k_cache, k_scales, kv_start, n_visible, padded)
    idx = slots_to_positions(topk_slots(scores, k), padded)
    ents = gather_attention_entries(idx, kv_fp4, kv_scale, kv_start, window_kv, swa_start, n_swa)
    out, lse = sparse_attention(bf16_decode(q), ents, softmax_scale)
    return {"scores": scores, "idx": idx, "out": out, "lse": lse}


def swa_layer(q, window_kv, swa_start, n_swa, softmax_scale):
    """An SWA-only layer for one query (the causal encoder's first two layers,
    [V41F-ARCH] 2 encoder schedule; [V41F-BLOG] 2.3.2): softmax attention over the window
    rows alone, no main-KV entry."""
    ents = e4m3_decode(window_kv[swa_start:swa_start + max(0, min(int(n_swa), 128))])
    out, lse = sparse_attention(bf16_decode(q), ents.reshape(-1, 512), softmax_scale)
    return {"idx": np.zeros(0, np.int64), "out": out, "lse": lse}


def reuse_layer(idx, q, kv_fp4, kv_scale, kv_start, window_kv, swa_start, n_swa,
                softmax_scale):
    """Reuse mode for one query: no scoring and no selection; attend with the latest
    published indices and this layer's own query and window."""
    ents = gather_attention_entries(idx, kv_fp4, kv_scale, kv_start, window_kv, swa_start, n_swa)
    out, lse = sparse_attention(bf16_decode(q), ents, softmax_scale)
    return {"idx": np.asarray(idx), "out": out, "lse": lse}
