"""Mode routing of CSA2 layers over the C ABI (caller side: buffers only, no arithmetic).

Full:    index_score(FULL) -> topk -> sparse_attn; in a decoder stack index_score(FULL, block
         maxima and block statistics) -> full_select (the pool and the Top-K among the
         pool blocks that can hold a Full winner; E4M3 or MXFP4 keys, bf16 query) or, with
         the MXFP8 query, block maxima only -> pool_candidates -> index_score over the
         candidates -> topk among their slots -> sparse_attn
Reindex: index_score(REINDEX, over the pool) -> topk inside the pool -> sparse_attn
Reuse:   sparse_attn with the indices published by the latest Full or Reindex layer
SWA:     sparse_attn over the sliding window alone (the encoder's first two layers)
HISA-style coarse filter (coarse="hisa", the alternative the HSI section contrasts): every
         Full and Reindex layer scores the block-mean keys with its own query, keeps the best
         2,048 blocks (the latest one forced in, as for the HSI pool), rescores their
         positions with the original keys and takes its Top-K there
("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache Compression", 2.3.2 and 3.3.3;
"DeepSeek-V4.1-Flash - Architecture", section 2, mode table and the encoder and decoder
schedules; in the encoder each group's Full layer reads its own cache set and its Reuse
layers read the same one.)
All outputs live in buffers allocated once, so a step allocates nothing.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import csa2 as C
from .synth import POOL_BLOCKS, TOPK, BLOCK


@dataclass
class Buffers:
    scores: torch.Tensor        # f32 [n_q, ld]
    block_max: torch.Tensor     # f32 [n_q, ceil(ld/8)]
    block_aux: torch.Tensor     # i32 [n_q, ceil(ld/8)] block statistics of a Full pass
    pool: torch.Tensor          # i32 [n_q, 2048]
    cand: torch.Tensor          # i32 [n_q, 2048] the Full layer's candidate blocks
    re_scores: torch.Tensor     # f32 [n_q, 16384]
    idx: torch.Tensor           # i32 [n_layers, n_q, 512] (index layers write their slot)
    out: torch.Tensor           # bf16 [n_layers, n_q, 64, 512]
    lse: torch.Tensor           # f32 [n_layers, n_q, 64]
    workspace: torch.Tensor | None
    published: list             # per layer: the index tensor it attended with
    q8_codes: torch.Tensor | None = None    # u8 [n_q, 32, 128] the layer's MXFP8 query
    q8_scales: torch.Tensor | None = None   # u8 [n_q, 32, 4]


@dataclass
class BlockMeans:
    km: torch.Tensor            # bf16 [n_q * max_blocks, 128] block-mean indexer keys
    km_start: torch.Tensor      # i64 [n_q] first km row of each query
    n_blocks: torch.Tensor      # i32 [n_q] ceil(n_visible / 8)


def build_block_means(wl, stream=None) -> BlockMeans:
    """Block-mean keys of every query's visible E4M3 keys. In a decoder these summaries
    are kept up to date as tokens arrive (a new token changes one block), so a decode step
    reads them as resident data."""
    if wl.k_codes is not None:
        raise ValueError("block means are built from E4M3 indexer keys")
    dev = wl.k_cache.device
    max_blocks = -(-max(1, wl.n_ctx) // BLOCK)
    km = torch.zeros((wl.n_q * max_blocks, 128), dtype=torch.bfloat16, device=dev)
    km_start = torch.arange(wl.n_q, dtype=torch.int64, device=dev) * max_blocks
    n_blocks = torch.zeros(wl.n_q, dtype=torch.int32, device=dev)
    C.csa2_block_mean_keys(wl.k_cache, wl.kv_start, wl.n_visible, km, km_start, n_blocks,
                           max_blocks=max_blocks, stream=stream)
    return BlockMeans(km=km, km_start=km_start, n_blocks=n_blocks)


def alloc_buffers(wl, k: int = TOPK) -> Buffers:
    dev = wl.k_cache.device
    n_q, n_l = wl.n_q, len(wl.layers)
    ld = -(-max(8, wl.n_ctx) // 32) * 32          # block-max rows stay a multiple of 4
    ws_bytes = C.workspace_bytes(C.OP_SPARSE_ATTN, n_q, 0, k)
    return Buffers(
        scores=torch.empty((n_q, ld), dtype=torch.float32, device=dev),
        block_max=torch.empty((n_q, (ld + BLOCK - 1) // BLOCK), dtype=torch.float32, device=dev),
        block_aux=torch.empty((n_q, (ld + BLOCK - 1) // BLOCK), dtype=torch.int32, device=dev),
        pool=torch.full((n_q, POOL_BLOCKS), -1, dtype=torch.int32, device=dev),
        cand=torch.full((n_q, POOL_BLOCKS), -1, dtype=torch.int32, device=dev),
        re_scores=torch.empty((n_q, POOL_BLOCKS * BLOCK), dtype=torch.float32, device=dev),
        idx=torch.full((n_l, n_q, k), -1, dtype=torch.int32, device=dev),
        out=torch.empty((n_l, n_q, 64, 512), dtype=torch.bfloat16, device=dev),
        lse=torch.empty((n_l, n_q, 64), dtype=torch.float32, device=dev),
        workspace=torch.zeros(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None,
        published=[None] * n_l,
        q8_codes=torch.empty((n_q, 32, 128), dtype=torch.uint8, device=dev) if wl.q8 else None,
        q8_scales=torch.empty((n_q, 32, 4), dtype=torch.uint8, device=dev) if wl.q8 else None,
    )


# Above this many (query, position) pairs per Full pass the block statistics' extra write
# costs the pass more than the one-kernel selection saves (measured: 32 x 262,144 pairs,
# statistics +5 us against a 12 us faster selection; 64 x 1,048,576 pairs, +51 us against
# 23 us), so larger passes take the three calls.
FUSED_SELECT_MAX_PAIRS = 1 << 24


def fused_full_select(wl) -> bool:
    """Whether a pooled decoder Full layer of this workload takes its pool and Top-K from
    one csa2_full_select (E4M3 keys) or csa2_full_select_mxfp4 call (bf16 indexer query, at
    most FUSED_SELECT_MAX_PAIRS scored pairs)."""
    return wl.with_pool and not wl.q8 and wl.n_q * wl.n_ctx <= FUSED_SELECT_MAX_PAIRS


def full_select(wl, lay, buf: Buffers, out_idx, k: int = TOPK, stream=None):
    """The pool and the Top-K of a pooled decoder Full layer from the block maxima and block
    statistics its Full pass left in buf, over the layer group's key format."""
    if wl.k_codes is not None:
        if lay.group != 0:
            raise ValueError("MXFP4 keys are carried for cache set 0 only")
        C.csa2_full_select_mxfp4(buf.block_max, buf.block_aux, wl.n_visible, buf.pool,
                                 lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                                 out_idx, n_keep=POOL_BLOCKS, k=k, stream=stream)
    else:
        C.csa2_full_select(buf.block_max, buf.block_aux, wl.n_visible, buf.pool, lay.q_idx,
                           lay.w, wl.cache(lay.group)[0], wl.kv_start, out_idx,
                           n_keep=POOL_BLOCKS, k=k, stream=stream)


def index_score(wl, mode, lay, scores, block_max=None, pool_blocks=None, ld_scores=None,
                stream=None, buf=None, block_aux=None):
    """The indexer over the layer group's keys: MXFP4 when the workload carries them (with
    the layer's query in MXFP8, already quantised into buf, when wl.q8), else E4M3; a Full
    pass of queries sharing one sequence scores them in groups per cache tile."""
    k_cache = wl.cache(lay.group)[0]
    if wl.q8 and wl.k_codes is not None:
        C.csa2_index_score_mxfp4_q8(mode, buf.q8_codes, buf.q8_scales, lay.w, wl.k_codes,
                                    wl.k_scales, wl.kv_start, wl.n_visible, scores, block_max,
                                    pool_blocks=pool_blocks, stream=stream, ld_scores=ld_scores)
        return
    if (wl.q8 and mode == C.FULL and wl.shared_start is not None and scores is not None):
        C.csa2_index_score_shared_q8(buf.q8_codes, buf.q8_scales, lay.w, k_cache,
                                     wl.shared_start, wl.n_visible, scores, block_max,
                                     stream=stream)
        return
    if wl.q8:
        C.csa2_index_score_q8(mode, buf.q8_codes, buf.q8_scales, lay.w, k_cache, wl.kv_start,
                              wl.n_visible, scores, block_max, pool_blocks=pool_blocks,
                              stream=stream, ld_scores=ld_scores)
        return
    if (mode == C.FULL and wl.k_codes is None and wl.shared_start is not None
            and scores is not None):
        C.csa2_index_score_shared(lay.q_idx, lay.w, k_cache, wl.shared_start, wl.n_visible,
                                  scores, block_max, stream=stream)
    elif wl.k_codes is not None:
        if lay.group != 0:
            raise ValueError("MXFP4 keys are carried for cache set 0 only")
        C.csa2_index_score_mxfp4(mode, lay.q_idx, lay.w, wl.k_codes, wl.k_scales, wl.kv_start,
                                 wl.n_visible, scores, block_max, pool_blocks=pool_blocks,
                                 stream=stream, ld_scores=ld_scores, block_aux=block_aux)
    else:
        C.csa2_index_score(mode, lay.q_idx, lay.w, k_cache, wl.kv_start, wl.n_visible,
                           scores, block_max, pool_blocks=pool_blocks, stream=stream,
                           ld_scores=ld_scores, block_aux=block_aux)


def hisa_select(wl, lay, buf: Buffers, means: BlockMeans, out_idx, k: int = TOPK,
                stream=None):
    """Two-stage selection from block means: block scores (into buf.block_max) -> the best
    2,048 blocks -> rescoring of their positions with the original keys -> Top-K."""
    C.csa2_index_score_bf16(C.FULL, lay.q_idx, lay.w, means.km, means.km_start, means.n_blocks,
                            buf.block_max, stream=stream)
    C.csa2_block_pool(buf.block_max, wl.n_visible, buf.pool, n_keep=POOL_BLOCKS, stream=stream)
    index_score(wl, C.REINDEX, lay, buf.re_scores, pool_blocks=buf.pool, stream=stream)
    C.csa2_topk(buf.re_scores, out_idx, k=k, pool_blocks=buf.pool, stream=stream)


def run_layers(wl, buf: Buffers, k: int = TOPK, stream=None, coarse: str = "hsi",
               means: BlockMeans | None = None):
    """One pass of the whole layer stack of the workload (one decode or prefill step).
    coarse="hisa" replaces every indexer layer's selection by the block-mean two-stage
    filter over `means` (decoder stacks with a pool only)."""
    if coarse not in ("hsi", "hisa"):
        raise ValueError(f"unknown coarse filter {coarse!r}")
    if coarse == "hisa" and (means is None or not wl.with_pool):
        raise ValueError("coarse='hisa' needs a pooled decoder workload and its block means")
    if wl.q8 and coarse != "hsi":
        raise ValueError("the MXFP8 query is routed with the HSI pool only")
    current = None
    current_group = 0
    for li, lay in enumerate(wl.layers):
        _, kv_fp4, kv_scale = wl.cache(lay.group)
        if lay.mode == "swa":
            buf.published[li] = buf.idx[li][:, :0]
            C.csa2_sparse_attn(lay.q, kv_fp4, kv_scale, wl.kv_start, buf.idx[li], lay.window_kv,
                               lay.swa_start, lay.n_swa, wl.softmax_scale, buf.out[li],
                               buf.lse[li], buf.workspace, k=0, stream=stream)
            continue
        if lay.mode in ("full", "reindex"):
            current_group = lay.group
            if wl.q8:
                C.csa2_quantize_mxfp8(lay.q_idx, buf.q8_codes, buf.q8_scales, stream=stream)
        elif lay.group != current_group:
            raise ValueError("a Reuse layer must read the cache set of the layer whose "
                             "indices it reuses")
        if lay.mode in ("full", "reindex") and coarse == "hisa":
            hisa_select(wl, lay, buf, means, buf.idx[li], k=k, stream=stream)
            current = buf.idx[li]
        elif lay.mode == "full":
            if wl.with_pool:
                # Decoder Full layer: the pass over the whole context writes only the block
                # maxima. The pool holds every Full-layer winner, and so do the pool's
                # candidate blocks (those ranked near the top by maximum, about a quarter of
                # the pool), so the Top-K is taken among the candidates' slots rescored with
                # this layer's own indexer query: the same scores, bit for bit. With E4M3
                # the bf16 query the pass also writes each block's argmax and second score,
                # and one kernel takes the pool and the Top-K from them, rescoring only the
                # few blocks whose second score can win (csa2_full_select, or its MXFP4-key
                # form); the MXFP8 query takes the three calls.
                if fused_full_select(wl):
                    index_score(wl, C.FULL, lay, None, buf.block_max,
                                ld_scores=buf.scores.shape[1], stream=stream, buf=buf,
                                block_aux=buf.block_aux)
                    full_select(wl, lay, buf, buf.idx[li], k=k, stream=stream)
                else:
                    index_score(wl, C.FULL, lay, None, buf.block_max,
                                ld_scores=buf.scores.shape[1], stream=stream, buf=buf)
                    C.csa2_pool_candidates(buf.block_max, wl.n_visible, buf.pool, buf.cand,
                                           n_keep=POOL_BLOCKS, k=k, stream=stream)
                    index_score(wl, C.REINDEX, lay, buf.re_scores, pool_blocks=buf.cand,
                                stream=stream, buf=buf)
                    C.csa2_topk(buf.re_scores, buf.idx[li], k=k, pool_blocks=buf.cand,
                                stream=stream)
            else:
                index_score(wl, C.FULL, lay, buf.scores, buf.block_max, stream=stream, buf=buf)
                C.csa2_topk(buf.scores, buf.idx[li], k=k, n_valid=wl.n_visible,
                            block_max=buf.block_max, stream=stream)
            current = buf.idx[li]
        elif lay.mode == "reindex":
            index_score(wl, C.REINDEX, lay, buf.re_scores, pool_blocks=buf.pool, stream=stream,
                        buf=buf)
            C.csa2_topk(buf.re_scores, buf.idx[li], k=k, pool_blocks=buf.pool, stream=stream)
            current = buf.idx[li]
        elif lay.mode != "reuse":
            raise ValueError(f"unknown mode {lay.mode!r}")
        if current is None:
            raise ValueError("a Reuse layer needs an earlier Full or Reindex layer")
        buf.published[li] = current
        C.csa2_sparse_attn(lay.q, kv_fp4, kv_scale, wl.kv_start, current, lay.window_kv,
                           lay.swa_start, lay.n_swa, wl.softmax_scale, buf.out[li], buf.lse[li],
                           buf.workspace, k=k, stream=stream)
