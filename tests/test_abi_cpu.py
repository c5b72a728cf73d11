"""The C ABI library on the host: it loads, exports every call of include/csa2.h, and
rejects bad arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def C():
    from compressed_kv_cache_csa2_amd import csa2
    return csa2


def test_header_symbols_are_exported(C):
    text = open(HEADER).read()
    names = set(re.findall(r"^(?:int|size_t|const char\*)\s+(csa2_\w+)\(", text, re.M))
    assert names == {"csa2_workspace_bytes", "csa2_index_score", "csa2_index_score_mxfp4",
                     "csa2_block_pool", "csa2_topk", "csa2_pool_topk", "csa2_sparse_attn",
                     "csa2_write_latent", "csa2_write_e4m3", "csa2_write_mxfp4_key",
                     "csa2_index_score_shared", "csa2_index_score_bf16",
                     "csa2_block_mean_keys", "csa2_compress_kv", "csa2_project_index_key",
                     "csa2_quantize_mxfp8", "csa2_index_score_mxfp4_q8", "csa2_index_score_q8",
                     "csa2_index_score_shared_q8", "csa2_pool_candidates", "csa2_full_select",
                     "csa2_full_select_mxfp4", "csa2_version", "csa2_last_error"}
    lib = ctypes.CDLL(C._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert C.version().startswith("csa2-gfx950")


FAKE = 0x10000   # a 64 KiB-aligned address: never dereferenced, validation fails first


def _score(C, **kw):
    a = dict(mode=0, n_q=1, n_heads=32, d_idx=128, q_idx=FAKE, w=FAKE, k_cache=FAKE, n_entries=10,
             kv_start=FAKE, n_visible=FAKE, pool_blocks=None, n_pool=0, block_size=8, scores=FAKE,
             ld=16, block_max=None, ld_bm=0, block_aux=None, stream=None)
    a.update(kw)
    return C.lib.csa2_index_score(*a.values())


def test_index_score_rejections(C):
    assert _score(C, mode=2) == 1 and b"no scoring" in C.lib.csa2_last_error()
    assert _score(C, n_heads=64) == 2
    assert _score(C, d_idx=64) == 2
    assert _score(C, block_size=16) == 2
    assert _score(C, n_q=-1) == 1
    assert _score(C, q_idx=None) == 1
    assert _score(C, q_idx=FAKE + 8) == 1                 # not 16-byte aligned
    assert _score(C, ld=0) == 1
    assert _score(C, mode=1) == 1                         # REINDEX without a pool
    assert _score(C, mode=1, pool_blocks=FAKE, n_pool=2048, ld=100) == 1
    assert _score(C, pool_blocks=FAKE, n_pool=4) == 1     # FULL with a pool
    assert _score(C, block_max=FAKE, ld_bm=1) == 1        # ld_bm < ceil(16/8)
    assert _score(C, scores=None) == 1                    # no scores and no block maxima
    assert b"only in FULL mode with block_max" in C.lib.csa2_last_error()
    assert _score(C, block_aux=FAKE) == 1                 # block statistics need block_max
    assert _score(C, mode=1, pool_blocks=FAKE, n_pool=2, block_max=FAKE, ld_bm=2,
                  block_aux=FAKE) == 1                    # ... and a FULL pass
    assert _score(C, block_max=FAKE, ld_bm=2, block_aux=FAKE + 2) == 1   # misaligned
    assert _score(C, mode=1, pool_blocks=FAKE, n_pool=2, scores=None,
                  block_max=FAKE, ld_bm=2) == 1           # REINDEX always writes scores
    assert _score(C, n_q=0, q_idx=None) == 0              # nothing to do, nothing launched


def test_index_score_mxfp4_rejections(C):
    def call(**kw):
        a = dict(mode=0, n_q=1, n_heads=32, d_idx=128, q_idx=FAKE, w=FAKE, k_codes=FAKE,
                 k_scales=FAKE, n_entries=10, kv_start=FAKE, n_visible=FAKE, pool_blocks=None,
                 n_pool=0, block_size=8, scores=FAKE, ld=16, block_max=None, ld_bm=0,
                 block_aux=None, stream=None)
        a.update(kw)
        return C.lib.csa2_index_score_mxfp4(*a.values())
    assert call(k_scales=None) == 1 and b"null k_scales" in C.lib.csa2_last_error()
    assert call(k_scales=FAKE + 2) == 1 and b"4-byte aligned" in C.lib.csa2_last_error()
    assert call(k_codes=FAKE + 8) == 1                    # codes not 16-byte aligned
    assert call(mode=2) == 1 and b"csa2_index_score_mxfp4" in C.lib.csa2_last_error()
    assert call(n_heads=64) == 2
    assert call(scores=None) == 1
    assert call(block_aux=FAKE) == 1                      # block statistics need block_max
    assert call(mode=1, pool_blocks=FAKE, n_pool=2, block_max=FAKE, ld_bm=2,
                block_aux=FAKE) == 1                      # ... and a FULL pass
    assert call(block_max=FAKE, ld_bm=2, block_aux=FAKE + 2) == 1   # misaligned
    assert call(n_q=0, k_scales=None, q_idx=None) == 0    # nothing to do, nothing launched


def test_index_score_shared_rejections(C):
    L = C.lib
    ok = [1, 32, 128, FAKE, FAKE, FAKE, 10, 0, FAKE, FAKE, 16, None, 0, None]
    def call(**kw):
        a = list(ok)
        names = ["n_q", "n_heads", "d_idx", "q_idx", "w", "k_cache", "n_entries", "kv_start",
                 "n_visible", "scores", "ld", "block_max", "ld_bm", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.csa2_index_score_shared(*a)
    assert call(n_heads=16) == 2
    assert call(scores=None) == 1
    assert call(q_idx=FAKE + 8) == 1
    assert call(ld=0) == 1
    assert call(block_max=FAKE, ld_bm=1) == 1
    assert call(n_q=-1) == 1
    assert call(n_q=0, q_idx=None) == 0


def test_index_score_bf16_rejections(C):
    def call(**kw):
        a = dict(mode=0, n_q=1, n_heads=32, d_idx=128, q_idx=FAKE, w=FAKE, k_rows=FAKE,
                 n_entries=10, kv_start=FAKE, n_visible=FAKE, pool_blocks=None, n_pool=0,
                 block_size=8, scores=FAKE, ld=16, block_max=None, ld_bm=0, stream=None)
        a.update(kw)
        return C.lib.csa2_index_score_bf16(*a.values())
    assert call(mode=2) == 1 and b"csa2_index_score_bf16" in C.lib.csa2_last_error()
    assert call(k_rows=FAKE + 8) == 1                     # rows not 16-byte aligned
    assert call(d_idx=64) == 2
    assert call(mode=1) == 1                              # REINDEX without a pool
    assert call(scores=None) == 1
    assert call(n_q=0, q_idx=None) == 0


def test_block_mean_keys_rejections(C):
    def call(**kw):
        a = dict(n_q=1, d_idx=128, block_size=8, k_cache=FAKE, n_entries=10, kv_start=FAKE,
                 n_visible=FAKE, km=FAKE, km_start=FAKE, n_km_rows=4, max_blocks=2,
                 n_blocks=FAKE, last_only=0, stream=None)
        a.update(kw)
        return C.lib.csa2_block_mean_keys(*a.values())
    assert call(d_idx=64) == 2
    assert call(block_size=16) == 2
    assert call(n_q=-1) == 1
    assert call(km=None) == 1 and b"csa2_block_mean_keys" in C.lib.csa2_last_error()
    assert call(km=FAKE + 8) == 1                         # km not 16-byte aligned
    assert call(max_blocks=0) == 1
    assert call(n_entries=-1) == 1
    assert call(n_q=0, km=None) == 0


def test_compressor_and_projection_rejections(C):
    L = C.lib
    assert L.csa2_compress_kv(2, 10, 256, FAKE, FAKE, 512, FAKE, 512, None) == 2   # d
    assert L.csa2_compress_kv(0, 10, 512, FAKE, FAKE, 512, FAKE, 512, None) == 2   # m
    assert L.csa2_compress_kv(9, 10, 512, FAKE, FAKE, 512, FAKE, 512, None) == 2
    assert L.csa2_compress_kv(2, 10, 512, None, FAKE, 512, FAKE, 512, None) == 1
    assert L.csa2_compress_kv(2, 10, 512, FAKE + 8, FAKE, 512, FAKE, 512, None) == 1
    assert L.csa2_compress_kv(2, 10, 512, FAKE, FAKE, 500, FAKE, 512, None) == 1   # ld_in
    assert L.csa2_compress_kv(2, -1, 512, FAKE, FAKE, 512, FAKE, 512, None) == 1
    assert L.csa2_compress_kv(2, 1, 512, None, None, 0, None, 0, None) == 0        # no entry
    assert L.csa2_project_index_key(4, 512, 64, FAKE, 512, FAKE, FAKE, 128, None) == 2
    assert L.csa2_project_index_key(4, 512, 128, FAKE, 512, None, FAKE, 128, None) == 1
    assert L.csa2_project_index_key(4, 512, 128, FAKE, 256, FAKE, FAKE, 128, None) == 1
    assert L.csa2_project_index_key(4, 512, 128, FAKE + 8, 512, FAKE, FAKE, 128, None) == 1
    assert b"csa2_project_index_key" in L.csa2_last_error()
    assert L.csa2_project_index_key(0, 512, 128, None, 0, None, None, 0, None) == 0


def test_mxfp8_query_rejections(C):
    L = C.lib
    assert L.csa2_quantize_mxfp8(4, 64, FAKE, FAKE, FAKE, None) == 2
    assert L.csa2_quantize_mxfp8(4, 128, None, FAKE, FAKE, None) == 1
    assert L.csa2_quantize_mxfp8(4, 128, FAKE + 8, FAKE, FAKE, None) == 1
    assert L.csa2_quantize_mxfp8(0, 128, None, None, None, None) == 0
    def call(**kw):
        a = dict(mode=0, n_q=1, n_heads=32, d_idx=128, q_codes=FAKE, q_scales=FAKE, w=FAKE,
                 k_codes=FAKE, k_scales=FAKE, n_entries=10, kv_start=FAKE, n_visible=FAKE,
                 pool_blocks=None, n_pool=0, block_size=8, scores=FAKE, ld=16, block_max=None,
                 ld_bm=0, stream=None)
        a.update(kw)
        return L.csa2_index_score_mxfp4_q8(*a.values())
    assert call(mode=2) == 1 and b"no scoring" in L.csa2_last_error()
    assert call(mode=1) == 1                              # REINDEX without a pool
    assert call(pool_blocks=FAKE, n_pool=4) == 1          # FULL with a pool
    assert call(block_size=16) == 2
    assert call(n_heads=16) == 2
    assert call(q_scales=None) == 1
    assert call(q_codes=FAKE + 8) == 1
    assert call(scores=None) == 1
    assert call(block_max=FAKE, ld_bm=1) == 1
    assert call(n_q=0, q_codes=None) == 0


def test_cache_write_rejections(C):
    L = C.lib
    assert L.csa2_write_latent(-1, FAKE, FAKE, FAKE, 256, FAKE, 32, 10, None) == 1
    assert L.csa2_write_latent(1, None, FAKE, FAKE, 256, FAKE, 32, 10, None) == 1
    assert L.csa2_write_latent(1, FAKE, FAKE, FAKE, 255, FAKE, 32, 10, None) == 1   # stride
    assert L.csa2_write_latent(1, FAKE, FAKE, FAKE, 256, FAKE, 31, 10, None) == 1
    assert L.csa2_write_latent(1, FAKE + 8, FAKE, FAKE, 256, FAKE, 32, 10, None) == 1
    assert L.csa2_write_latent(0, None, None, None, 0, None, 0, 0, None) == 0
    assert L.csa2_write_e4m3(1, 64, FAKE, FAKE, FAKE, 64, 10, None) == 2          # d
    assert L.csa2_write_e4m3(1, 512, FAKE, FAKE, FAKE, 256, 10, None) == 1        # stride < d
    assert L.csa2_write_e4m3(1, 128, FAKE, FAKE, FAKE + 4, 128, 10, None) == 1    # dst alignment
    assert L.csa2_write_e4m3(1, 128, FAKE, None, FAKE, 128, 10, None) == 1
    assert L.csa2_write_mxfp4_key(1, FAKE, FAKE, FAKE, None, 10, None) == 1
    assert L.csa2_write_mxfp4_key(1, FAKE, FAKE, FAKE, FAKE, -1, None) == 1
    assert L.csa2_write_mxfp4_key(0, None, None, None, None, 0, None) == 0


def test_topk_and_pool_rejections(C):
    L = C.lib
    ok = dict(n_q=1, scores=FAKE, ld=100, n_cols=100, n_valid=None, bm=None, ld_bm=0, k=512,
              pool_use=0, pool=None, n_pool=0, bs=8, idx=FAKE, ld_idx=512, ws=None, ws_bytes=0,
              stream=None)

    def topk(**kw):
        a = dict(ok)
        a.update(kw)
        return L.csa2_topk(*a.values())
    assert topk(k=0) == 1 and topk(k=4096) == 1
    assert topk(bs=4) == 2
    assert topk(n_cols=101) == 1
    assert topk(ld_idx=100) == 1
    assert topk(bm=FAKE, ld_bm=3) == 1
    assert topk(pool_use=1, pool=FAKE, n_pool=4) == 1    # 4 blocks cannot cover 100 slots
    assert topk(pool_use=3, pool=FAKE, n_pool=16) == 1   # unknown pool use
    assert topk(pool_use=1, pool=None, n_pool=16) == 1   # pool use without a pool
    assert topk(pool_use=0, pool=FAKE, n_pool=16) == 1   # a pool with no use
    assert topk(pool_use=2, pool=FAKE, n_pool=0) == 1
    assert topk(pool_use=2, pool=FAKE, n_pool=4096) == 1
    assert topk(scores=None) == 1
    assert topk(n_q=0, scores=None) == 0
    assert L.csa2_block_pool(1, FAKE, 10, FAKE, 8, 0, FAKE, 2048, None, 0, None) == 1
    assert L.csa2_block_pool(1, FAKE, 10, FAKE, 8, 2049, FAKE, 4096, None, 0, None) == 1
    assert L.csa2_block_pool(1, FAKE, 10, FAKE, 4, 2048, FAKE, 2048, None, 0, None) == 2
    assert L.csa2_block_pool(1, FAKE, 10, FAKE, 8, 2048, FAKE, 100, None, 0, None) == 1
    assert L.csa2_block_pool(0, None, 10, None, 8, 2048, None, 2048, None, 0, None) == 0


def test_pool_topk_rejections(C):
    L = C.lib
    ok = dict(n_q=1, bm=FAKE, ld_bm=4096, nv=FAKE, bs=8, n_keep=2048, pool=FAKE, ld_pool=2048,
              scores=FAKE, ld=32768, n_cols=32768, k=512, idx=FAKE, ld_idx=512, stream=None)

    def pt(**kw):
        a = dict(ok)
        a.update(kw)
        return L.csa2_pool_topk(*a.values())
    assert pt(bs=4) == 2
    assert pt(n_keep=0) == 1 and pt(n_keep=4096) == 1
    assert pt(k=0) == 1 and pt(k=4096) == 1
    assert pt(ld_pool=100) == 1
    assert pt(ld_bm=3) == 1
    assert pt(n_cols=32769) == 1
    assert pt(ld_idx=100) == 1
    assert pt(scores=FAKE + 4) == 1
    assert pt(idx=None) == 1
    assert pt(n_q=0, bm=None) == 0


def test_sparse_attn_rejections_and_workspace(C):
    L = C.lib
    # No call needs scratch memory: the attention's two workgroups per (query, head group)
    # write disjoint channel halves, so nothing is combined through a workspace.
    for op in (C.OP_INDEX_SCORE, C.OP_BLOCK_POOL, C.OP_TOPK, C.OP_SPARSE_ATTN):
        for n_q in (1, 32, 4096):
            assert C.workspace_bytes(op, n_q, 262144, 512) == 0
    ok = dict(n_q=32, heads=64, dim=512, q=FAKE, fp4=FAKE, fs=256, sc=FAKE, ss=32, ne=100,
              kv_start=FAKE, idx=FAKE, ld_idx=512, k=512, win=FAKE, nw=10, swa_start=FAKE,
              n_swa=FAKE, scale=0.04, out=FAKE, lse=None, ws=None, ws_bytes=0, stream=None)

    def attn(**kw):
        a = dict(ok)
        a.update(kw)
        return L.csa2_sparse_attn(*a.values())
    assert attn(heads=32) == 2 and attn(dim=256) == 2
    assert attn(k=-1) == 1 and attn(k=4096) == 1
    assert attn(fs=128) == 1 and attn(fs=264) == 1 and attn(fs=16384) == 1
    assert attn(ss=16) == 1 and attn(ss=16384) == 1
    assert attn(q=FAKE + 4) == 1
    assert attn(out=None) == 1
    assert attn(ld_idx=100) == 1
    assert attn(n_q=0, q=None) == 0


def _pool_cand(C, **kw):
    a = dict(n_q=1, block_max=FAKE, ld_bm=4, n_visible=FAKE, block_size=8, n_keep=2048,
             pool_blocks=FAKE, ld_pool=2048, k=512, cand_blocks=FAKE, ld_cand=2048, stream=None)
    a.update(kw)
    return C.lib.csa2_pool_candidates(*a.values())


def test_pool_candidates_rejections(C):
    assert _pool_cand(C, k=2048) == 1                        # k must stay below n_keep
    assert _pool_cand(C, k=0) == 1
    assert _pool_cand(C, n_keep=4096) == 1
    assert _pool_cand(C, block_size=4) == 2
    assert _pool_cand(C, cand_blocks=None) == 1
    assert _pool_cand(C, block_max=FAKE + 4) == 1           # not 16-byte aligned
    assert _pool_cand(C, ld_bm=6) == 1                      # not a multiple of 4
    assert _pool_cand(C, ld_pool=100) == 1
    assert _pool_cand(C, ld_cand=100) == 1
    assert _pool_cand(C, n_q=0) == 0                        # nothing to do


def _full_select(C, **kw):
    a = dict(n_q=2, block_max=FAKE, ld_bm=8, n_visible=FAKE, block_size=8, n_keep=2048,
             pool_blocks=FAKE, ld_pool=2048, n_heads=32, d_idx=128, q_idx=FAKE, w=FAKE,
             k_cache=FAKE, n_entries=100, kv_start=FAKE, block_aux=FAKE, k=512, topk_idx=FAKE,
             ld_idx=512, stream=None)
    a.update(kw)
    return C.lib.csa2_full_select(*a.values())


def test_full_select_rejections(C):
    assert _full_select(C, k=2048) == 1                      # k must stay below n_keep
    assert _full_select(C, k=0) == 1
    assert _full_select(C, n_keep=4096) == 1
    assert _full_select(C, block_size=4) == 2
    assert _full_select(C, n_heads=64) == 2
    assert _full_select(C, d_idx=64) == 2
    assert _full_select(C, q_idx=None) == 1
    assert _full_select(C, topk_idx=None) == 1
    assert _full_select(C, block_aux=None) == 1
    assert _full_select(C, block_aux=FAKE + 2) == 1         # misaligned
    assert _full_select(C, q_idx=FAKE + 8) == 1             # not 16-byte aligned
    assert _full_select(C, k_cache=FAKE + 4) == 1
    assert _full_select(C, block_max=FAKE + 4) == 1
    assert _full_select(C, ld_bm=6) == 1                    # not a multiple of 4
    assert _full_select(C, ld_pool=100) == 1
    assert _full_select(C, ld_idx=100) == 1
    assert _full_select(C, n_entries=-1) == 1
    assert _full_select(C, n_q=0) == 0                      # nothing to do


def test_full_select_mxfp4_rejections(C):
    def call(**kw):
        a = dict(n_q=2, block_max=FAKE, ld_bm=8, n_visible=FAKE, block_size=8, n_keep=2048,
                 pool_blocks=FAKE, ld_pool=2048, n_heads=32, d_idx=128, q_idx=FAKE, w=FAKE,
                 k_codes=FAKE, k_scales=FAKE, n_entries=100, kv_start=FAKE, block_aux=FAKE,
                 k=512, topk_idx=FAKE, ld_idx=512, stream=None)
        a.update(kw)
        return C.lib.csa2_full_select_mxfp4(*a.values())
    assert call(k_scales=None) == 1 and b"null k_scales" in C.lib.csa2_last_error()
    assert call(k_scales=FAKE + 2) == 1 and b"k_scales" in C.lib.csa2_last_error()
    assert call(k_codes=FAKE + 8) == 1                      # codes not 16-byte aligned
    assert call(k=2048) == 1
    assert call(block_size=4) == 2
    assert call(n_heads=64) == 2
    assert call(block_aux=None) == 1
    assert b"csa2_full_select_mxfp4" in C.lib.csa2_last_error()
    assert call(ld_idx=100) == 1
    assert call(n_q=0, k_scales=None) == 0                  # nothing to do


def test_wrappers_reject_mis_shaped_tensors_before_any_call(C):
    """The Python binding checks every tensor's shape against the query count and the
    compiled sizes before a pointer reaches the library (host tensors: a well-shaped one
    would be refused as not on the device, also before any call)."""
    import torch
    f32, i32, i64, u8, bf = torch.float32, torch.int32, torch.int64, torch.uint8, torch.bfloat16
    n = 4
    q = torch.zeros((n, 32, 128), dtype=bf)
    w = torch.zeros((n, 32), dtype=f32)
    kc = torch.zeros((100, 128), dtype=u8)
    ks = torch.zeros((n,), dtype=i64)
    nv = torch.zeros((n,), dtype=i32)
    sc = torch.zeros((n, 64), dtype=f32)
    bm = torch.zeros((n, 8), dtype=f32)
    cases = [
        lambda: C.csa2_index_score(0, q, w[:3], kc, ks, nv, sc),                   # w rows
        lambda: C.csa2_index_score(0, q, w, kc, ks[:2], nv, sc),                   # kv_start
        lambda: C.csa2_index_score(0, q, w, kc, ks, nv, sc[:3]),                   # score rows
        lambda: C.csa2_index_score(0, q, w, kc, ks, nv, sc, torch.zeros((n, 7))),  # bm width
        lambda: C.csa2_index_score(0, q[:, :, :64], w, kc, ks, nv, sc),            # q width
        lambda: C.csa2_index_score(0, q, w, kc[:, :64], ks, nv, sc),               # key width
        lambda: C.csa2_index_score_q8(0, torch.zeros((n, 32, 128), dtype=u8),
                                      torch.zeros((n, 32, 3), dtype=u8), w, kc, ks, nv, sc),
        lambda: C.csa2_index_score_mxfp4(0, q, w, torch.zeros((100, 64), dtype=u8),
                                         torch.zeros((99, 4), dtype=u8), ks, nv, sc),
        lambda: C.csa2_index_score_shared(q, w, kc, 0, nv[:3], sc),
        lambda: C.csa2_index_score_shared_q8(torch.zeros((n, 32, 128), dtype=u8),
                                             torch.zeros((n, 32, 4), dtype=u8), w[:1], kc, 0,
                                             nv, sc),
        lambda: C.csa2_block_pool(bm, nv[:3], torch.zeros((n, 2048), dtype=i32)),
        lambda: C.csa2_block_pool(bm, nv, torch.zeros((n, 100), dtype=i32)),
        lambda: C.csa2_pool_candidates(bm, nv, torch.zeros((n, 2048), dtype=i32),
                                       torch.zeros((n, 2047), dtype=i32)),
        lambda: C.csa2_full_select(bm, torch.zeros(bm.shape, dtype=i32), nv,
                                   torch.zeros((n, 2048), dtype=i32), q[:3], w, kc, ks,
                                   torch.zeros((n, 512), dtype=i32)),
        lambda: C.csa2_full_select(bm, torch.zeros(bm.shape, dtype=i32), nv,
                                   torch.zeros((n, 2048), dtype=i32), q, w,
                                   torch.zeros((100, 64), dtype=u8), ks,
                                   torch.zeros((n, 512), dtype=i32)),
        lambda: C.csa2_full_select(bm, torch.zeros(bm.shape, dtype=i32), nv,
                                   torch.zeros((n, 2048), dtype=i32), q, w, kc, ks,
                                   torch.zeros((n, 100), dtype=i32)),
        lambda: C.csa2_full_select(bm, torch.zeros((n, 7), dtype=i32), nv,
                                   torch.zeros((n, 2048), dtype=i32), q, w, kc, ks,
                                   torch.zeros((n, 512), dtype=i32)),
        lambda: C.csa2_full_select_mxfp4(bm, torch.zeros(bm.shape, dtype=i32), nv,
                                         torch.zeros((n, 2048), dtype=i32), q, w,
                                         torch.zeros((100, 64), dtype=u8),
                                         torch.zeros((99, 4), dtype=u8), ks,
                                         torch.zeros((n, 512), dtype=i32)),
        lambda: C.csa2_full_select_mxfp4(bm, torch.zeros(bm.shape, dtype=i32), nv,
                                         torch.zeros((n, 2048), dtype=i32), q, w, kc,
                                         torch.zeros((100, 4), dtype=u8), ks,
                                         torch.zeros((n, 512), dtype=i32)),
        lambda: C.csa2_index_score_mxfp4(0, q, w, torch.zeros((100, 64), dtype=u8),
                                         torch.zeros((100, 4), dtype=u8), ks, nv, sc,
                                         block_max=bm, block_aux=torch.zeros((n, 3), dtype=i32)),
        lambda: C.csa2_index_score(0, q, w, kc, ks, nv, sc, block_max=bm,
                                   block_aux=torch.zeros((n, 3), dtype=i32)),
        lambda: C.csa2_topk(sc, torch.zeros((n, 100), dtype=i32), k=512),
        lambda: C.csa2_topk(sc, torch.zeros((3, 512), dtype=i32)),
        lambda: C.csa2_sparse_attn(torch.zeros((n, 64, 512), dtype=bf),
                                   torch.zeros((10, 256), dtype=u8),
                                   torch.zeros((9, 32), dtype=u8), ks,
                                   torch.zeros((n, 512), dtype=i32),
                                   torch.zeros((10, 512), dtype=u8), ks, nv, 0.1,
                                   torch.zeros((n, 64, 512), dtype=bf)),
        lambda: C.csa2_sparse_attn(torch.zeros((n, 64, 512), dtype=bf),
                                   torch.zeros((10, 256), dtype=u8),
                                   torch.zeros((10, 32), dtype=u8), ks,
                                   torch.zeros((n, 100), dtype=i32),
                                   torch.zeros((10, 512), dtype=u8), ks, nv, 0.1,
                                   torch.zeros((n, 64, 512), dtype=bf)),
        lambda: C.csa2_sparse_attn(torch.zeros((n, 64, 512), dtype=bf),
                                   torch.zeros((10, 256), dtype=u8),
                                   torch.zeros((10, 32), dtype=u8), ks,
                                   torch.zeros((n, 512), dtype=i32),
                                   torch.zeros((10, 512), dtype=u8), ks, nv, 0.1,
                                   torch.zeros((n, 64, 256), dtype=bf)),
        lambda: C.csa2_write_mxfp4_key(torch.zeros((5, 128), dtype=bf), torch.zeros(5, dtype=i64),
                                       torch.zeros((10, 32), dtype=u8),
                                       torch.zeros((10, 4), dtype=u8)),
    ]
    for i, case in enumerate(cases):
        with pytest.raises(ValueError) as e:
            case()
        assert "device tensor" not in str(e.value), f"case {i} passed the shape checks"
