"""Python binding of libcsa2.so: the C ABI calls under the same names.

Argument marshalling only: dtype/device/shape checks, raw pointers, the current HIP
stream. Every step of the path runs in the HIP library; if the library is missing the
import fails (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

# CSA2_LIBRARY names another build of the same C ABI (the sanitizer host-check build of the
# CPU tests, whose launchers refuse every launch); by default the in-tree libcsa2.so.
_LIB_PATH = os.environ.get("CSA2_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

FULL, REINDEX, REUSE = 0, 1, 2
POOL_NONE, POOL_SLOTS, POOL_CANDIDATES = 0, 1, 2
OP_INDEX_SCORE, OP_BLOCK_POOL, OP_TOPK, OP_SPARSE_ATTN = 0, 1, 2, 3
CSA2_OK = 0


class Csa2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m compressed_kv_cache_csa2_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, L, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.csa2_index_score.argtypes = [I, I, I, I, P, P, P, L, P, P, P, I, I, P, L, P, L, P, P]
    lib.csa2_index_score_mxfp4.argtypes = [I, I, I, I, P, P, P, P, L, P, P, P, I, I, P, L, P, L, P,
                                           P]
    lib.csa2_index_score_bf16.argtypes = [I, I, I, I, P, P, P, L, P, P, P, I, I, P, L, P, L, P]
    lib.csa2_block_mean_keys.argtypes = [I, I, I, P, L, P, P, P, P, L, L, P, I, P]
    lib.csa2_quantize_mxfp8.argtypes = [I, I, P, P, P, P]
    lib.csa2_index_score_mxfp4_q8.argtypes = [I, I, I, I, P, P, P, P, P, L, P, P, P, I, I, P, L, P,
                                              L, P]
    lib.csa2_index_score_q8.argtypes = [I, I, I, I, P, P, P, P, L, P, P, P, I, I, P, L, P, L, P]
    lib.csa2_index_score_shared_q8.argtypes = [I, I, I, P, P, P, P, L, L, P, P, L, P, L, P]
    lib.csa2_compress_kv.argtypes = [I, I, I, P, P, L, P, L, P]
    lib.csa2_project_index_key.argtypes = [I, I, I, P, L, P, P, L, P]
    lib.csa2_write_latent.argtypes = [I, P, P, P, L, P, L, L, P]
    lib.csa2_write_e4m3.argtypes = [I, I, P, P, P, L, L, P]
    lib.csa2_write_mxfp4_key.argtypes = [I, P, P, P, P, L, P]
    lib.csa2_index_score_shared.argtypes = [I, I, I, P, P, P, L, L, P, P, L, P, L, P]
    lib.csa2_block_pool.argtypes = [I, P, L, P, I, I, P, L, P, Z, P]
    lib.csa2_topk.argtypes = [I, P, L, L, P, P, L, I, I, P, I, I, P, L, P, Z, P]
    lib.csa2_pool_topk.argtypes = [I, P, L, P, I, I, P, L, P, L, L, I, P, L, P]
    lib.csa2_pool_candidates.argtypes = [I, P, L, P, I, I, P, L, I, P, L, P]
    lib.csa2_full_select.argtypes = [I, P, L, P, I, I, P, L, I, I, P, P, P, L, P, P, I, P, L, P]
    lib.csa2_full_select_mxfp4.argtypes = [I, P, L, P, I, I, P, L, I, I, P, P, P, P, L, P, P, I, P,
                                           L, P]
    lib.csa2_sparse_attn.argtypes = [I, I, I, P, P, L, P, L, L, P, P, L, I, P, L, P, P, F, P, P,
                                     P, Z, P]
    for f in ("csa2_index_score_shared", "csa2_write_latent", "csa2_write_e4m3", "csa2_write_mxfp4_key",
              "csa2_index_score", "csa2_index_score_mxfp4", "csa2_block_pool", "csa2_topk", "csa2_pool_topk",
              "csa2_sparse_attn", "csa2_index_score_bf16", "csa2_block_mean_keys",
              "csa2_compress_kv", "csa2_project_index_key", "csa2_quantize_mxfp8",
              "csa2_index_score_mxfp4_q8", "csa2_index_score_q8", "csa2_index_score_shared_q8",
              "csa2_pool_candidates", "csa2_full_select", "csa2_full_select_mxfp4"):
        getattr(lib, f).restype = I
    lib.csa2_workspace_bytes.argtypes = [I, I, L, I]
    lib.csa2_workspace_bytes.restype = Z
    lib.csa2_version.restype = ctypes.c_char_p
    lib.csa2_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status: int):
    if status != CSA2_OK:
        raise Csa2Error(status, lib.csa2_last_error().decode())


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dims(t, name, *dims):
    """Raise ValueError unless tensor t (skipped when None) has len(dims) dimensions, each
    equal to the given int, at least v for a ('>=', v) pair, or anything for None. The C
    ABI receives only pointers and a few sizes, so every other shape is checked here,
    before any pointer is passed on."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dim() != len(dims):
        raise ValueError(f"{name}: expected {len(dims)} dimensions, got shape {tuple(t.shape)}")
    for i, (have, want) in enumerate(zip(t.shape, dims)):
        if want is None:
            continue
        if isinstance(want, tuple):
            if have < want[1]:
                raise ValueError(f"{name}: dimension {i} is {have}, needs >= {want[1]}")
        elif have != want:
            raise ValueError(f"{name}: dimension {i} is {have}, expected {want} "
                             f"(shape {tuple(t.shape)})")


def _index_common(name, n_q, w, kv_start, n_visible, scores, block_max, pool_blocks, ld_scores):
    """Shapes shared by the indexer calls: per-query vectors of n_q, score rows of n_q, block
    maxima covering ceil(ld/8) blocks, a pool of n_q rows."""
    _dims(w, f"{name}: w", n_q, 32)
    _dims(kv_start, f"{name}: kv_start", n_q)
    _dims(n_visible, f"{name}: n_visible", n_q)
    _dims(scores, f"{name}: scores", n_q, None)
    _dims(block_max, f"{name}: block_max", n_q, (">=", (ld_scores + 7) // 8))
    _dims(pool_blocks, f"{name}: pool_blocks", n_q, None)


def version() -> str:
    return lib.csa2_version().decode()


def workspace_bytes(op: int, n_q: int, max_cols: int, k: int) -> int:
    return int(lib.csa2_workspace_bytes(op, n_q, max_cols, k))


def _rows_view(t, width, name):
    if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1 \
            or t.shape[1] < width:
        raise ValueError(f"{name}: expected a device uint8 [rows, >= {width}] view")
    return t.data_ptr(), t.stride(0)


def csa2_quantize_mxfp8(x, codes, scales, stream=None):
    """MXFP8 rows: x bf16 [..., 128] -> codes uint8 [..., 128] (E4M3), scales uint8 [..., 4]."""
    n = x.numel() // 128
    if x.shape[-1] != 128 or codes.numel() != x.numel() or scales.numel() != n * 4:
        raise ValueError("csa2_quantize_mxfp8: x [..., 128], codes like x, scales [..., 4]")
    _check(lib.csa2_quantize_mxfp8(n, 128, _ptr(x, torch.bfloat16, "x"),
                                   _ptr(codes, torch.uint8, "codes"),
                                   _ptr(scales, torch.uint8, "scales"), _stream(stream)))


def csa2_index_score_mxfp4_q8(mode, q_codes, q_scales, w, k_codes, k_scales, kv_start, n_visible,
                              scores, block_max=None, pool_blocks=None, stream=None,
                              ld_scores=None):
    """Scores of an MXFP8 query (q_codes [n_q, 32, 128], q_scales [n_q, 32, 4]) over MXFP4
    keys, FULL or REINDEX (over pool_blocks); FULL scores may be None when block_max is
    given (then ld_scores is needed)."""
    n_q = q_codes.shape[0]
    n_pool = pool_blocks.shape[1] if pool_blocks is not None else 0
    if scores is not None:
        ld_scores = scores.shape[1]
    elif ld_scores is None:
        raise ValueError("csa2_index_score_mxfp4_q8: ld_scores is required when scores is None")
    _dims(q_codes, "csa2_index_score_mxfp4_q8: q_codes", n_q, 32, 128)
    _dims(q_scales, "csa2_index_score_mxfp4_q8: q_scales", n_q, 32, 4)
    _dims(k_codes, "csa2_index_score_mxfp4_q8: k_codes", None, 64)
    _dims(k_scales, "csa2_index_score_mxfp4_q8: k_scales", k_codes.shape[0], 4)
    _index_common("csa2_index_score_mxfp4_q8", n_q, w, kv_start, n_visible, scores, block_max,
                  pool_blocks, ld_scores)
    _check(lib.csa2_index_score_mxfp4_q8(
        mode, n_q, q_codes.shape[1], q_codes.shape[2], _ptr(q_codes, torch.uint8, "q_codes"),
        _ptr(q_scales, torch.uint8, "q_scales"), _ptr(w, torch.float32, "w"),
        _ptr(k_codes, torch.uint8, "k_codes"), _ptr(k_scales, torch.uint8, "k_scales"),
        k_codes.shape[0], _ptr(kv_start, torch.int64, "kv_start"),
        _ptr(n_visible, torch.int32, "n_visible"), _ptr(pool_blocks, torch.int32, "pool_blocks"),
        n_pool, 8, _ptr(scores, torch.float32, "scores"),
        ld_scores, _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0, _stream(stream)))


def csa2_index_score_q8(mode, q_codes, q_scales, w, k_cache, kv_start, n_visible, scores,
                        block_max=None, pool_blocks=None, stream=None, ld_scores=None):
    """csa2_index_score_mxfp4_q8 over E4M3 keys k_cache [E, 128]."""
    n_q = q_codes.shape[0]
    n_pool = pool_blocks.shape[1] if pool_blocks is not None else 0
    if scores is not None:
        ld_scores = scores.shape[1]
    elif ld_scores is None:
        raise ValueError("csa2_index_score_q8: ld_scores is required when scores is None")
    _dims(q_codes, "csa2_index_score_q8: q_codes", n_q, 32, 128)
    _dims(q_scales, "csa2_index_score_q8: q_scales", n_q, 32, 4)
    _dims(k_cache, "csa2_index_score_q8: k_cache", None, 128)
    _index_common("csa2_index_score_q8", n_q, w, kv_start, n_visible, scores, block_max,
                  pool_blocks, ld_scores)
    _check(lib.csa2_index_score_q8(
        mode, n_q, q_codes.shape[1], q_codes.shape[2], _ptr(q_codes, torch.uint8, "q_codes"),
        _ptr(q_scales, torch.uint8, "q_scales"), _ptr(w, torch.float32, "w"),
        _ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
        _ptr(kv_start, torch.int64, "kv_start"), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(pool_blocks, torch.int32, "pool_blocks"), n_pool, 8,
        _ptr(scores, torch.float32, "scores"), ld_scores,
        _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0, _stream(stream)))


def csa2_index_score_shared_q8(q_codes, q_scales, w, k_cache, kv_start: int, n_visible, scores,
                               block_max=None, stream=None):
    """csa2_index_score_shared with an MXFP8 query over E4M3 keys."""
    n_q = q_codes.shape[0]
    _dims(q_codes, "csa2_index_score_shared_q8: q_codes", n_q, 32, 128)
    _dims(q_scales, "csa2_index_score_shared_q8: q_scales", n_q, 32, 4)
    _dims(k_cache, "csa2_index_score_shared_q8: k_cache", None, 128)
    _dims(scores, "csa2_index_score_shared_q8: scores", n_q, None)
    _index_common("csa2_index_score_shared_q8", n_q, w, None, n_visible, scores, block_max,
                  None, scores.shape[1])
    _check(lib.csa2_index_score_shared_q8(
        n_q, q_codes.shape[1], q_codes.shape[2], _ptr(q_codes, torch.uint8, "q_codes"),
        _ptr(q_scales, torch.uint8, "q_scales"), _ptr(w, torch.float32, "w"),
        _ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0], int(kv_start),
        _ptr(n_visible, torch.int32, "n_visible"), _ptr(scores, torch.float32, "scores"),
        scores.shape[1], _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0, _stream(stream)))


def csa2_compress_kv(c, z, out, m, stream=None):
    """Gated pooling of m adjacent tokens: c, z bf16 [T, 512] -> out bf16 [T // m, 512]."""
    if c.shape != z.shape or c.dim() != 2 or c.shape[1] != 512:
        raise ValueError("csa2_compress_kv: c and z must both be [T, 512]")
    if out.dim() != 2 or out.shape[0] < c.shape[0] // m or out.shape[1] != 512:
        raise ValueError("csa2_compress_kv: out must be [>= T // m, 512]")
    _check(lib.csa2_compress_kv(int(m), c.shape[0], 512, _ptr(c, torch.bfloat16, "c"),
                                _ptr(z, torch.bfloat16, "z"), 512,
                                _ptr(out, torch.bfloat16, "out"), 512, _stream(stream)))


def csa2_project_index_key(entries, w_ik, out, stream=None):
    """Indexer keys out bf16 [n, 128] = entries bf16 [n, 512] . w_ik^T, w_ik bf16 [128, 512]."""
    if entries.dim() != 2 or entries.shape[1] != 512 or tuple(w_ik.shape) != (128, 512):
        raise ValueError("csa2_project_index_key: entries [n, 512] and w_ik [128, 512]")
    if out.dim() != 2 or out.shape[0] < entries.shape[0] or out.shape[1] != 128:
        raise ValueError("csa2_project_index_key: out must be [>= n, 128]")
    _check(lib.csa2_project_index_key(entries.shape[0], 512, 128,
                                      _ptr(entries, torch.bfloat16, "entries"), 512,
                                      _ptr(w_ik, torch.bfloat16, "w_ik"),
                                      _ptr(out, torch.bfloat16, "out"), 128, _stream(stream)))


def csa2_write_latent(x, rows, kv_fp4, kv_scale, stream=None):
    """Quantise bf16 latent rows x [n, 512] into kv_fp4 / kv_scale at cache rows `rows`."""
    p_fp4, s_fp4 = _rows_view(kv_fp4, 256, "kv_fp4")
    p_sc, s_sc = _rows_view(kv_scale, 32, "kv_scale")
    if x.dim() != 2 or x.shape[1] != 512 or rows.shape[0] != x.shape[0]:
        raise ValueError("csa2_write_latent: x must be [n, 512] with one row index per row")
    if kv_fp4.shape[0] != kv_scale.shape[0]:
        raise ValueError("csa2_write_latent: kv_fp4 and kv_scale row counts differ")
    _dims(rows, "csa2_write_latent: rows", x.shape[0])
    _check(lib.csa2_write_latent(x.shape[0], _ptr(x, torch.bfloat16, "x"),
                                 _ptr(rows, torch.int64, "rows"), p_fp4, s_fp4, p_sc, s_sc,
                                 kv_fp4.shape[0], _stream(stream)))


def csa2_write_e4m3(x, rows, dst, stream=None):
    """E4M3 rows: window rows (x [n, 512]) or E4M3 indexer keys (x [n, 128]) into dst."""
    d = x.shape[1]
    p, st = _rows_view(dst, d, "dst")
    if x.dim() != 2 or rows.shape[0] != x.shape[0]:
        raise ValueError("csa2_write_e4m3: x must be [n, d] with one row index per row")
    _dims(rows, "csa2_write_e4m3: rows", x.shape[0])
    _check(lib.csa2_write_e4m3(x.shape[0], d, _ptr(x, torch.bfloat16, "x"),
                               _ptr(rows, torch.int64, "rows"), p, st, dst.shape[0],
                               _stream(stream)))


def csa2_write_mxfp4_key(x, rows, k_codes, k_scales, stream=None):
    """MXFP4 indexer keys: x [n, 128] bf16 into k_codes [E, 64] / k_scales [E, 4]."""
    if x.dim() != 2 or x.shape[1] != 128 or rows.shape[0] != x.shape[0]:
        raise ValueError("csa2_write_mxfp4_key: x must be [n, 128] with one row index per row")
    if k_codes.shape[0] != k_scales.shape[0]:
        raise ValueError("csa2_write_mxfp4_key: k_codes and k_scales row counts differ")
    _dims(k_codes, "csa2_write_mxfp4_key: k_codes", None, 64)
    _dims(k_scales, "csa2_write_mxfp4_key: k_scales", None, 4)
    _dims(rows, "csa2_write_mxfp4_key: rows", x.shape[0])
    _check(lib.csa2_write_mxfp4_key(x.shape[0], _ptr(x, torch.bfloat16, "x"),
                                    _ptr(rows, torch.int64, "rows"),
                                    _ptr(k_codes, torch.uint8, "k_codes"),
                                    _ptr(k_scales, torch.uint8, "k_scales"), k_codes.shape[0],
                                    _stream(stream)))


def csa2_index_score(mode, q_idx, w, k_cache, kv_start, n_visible, scores, block_max=None,
                     pool_blocks=None, stream=None, ld_scores=None, block_aux=None):
    """Indexer scores into `scores` [n_q, ld] (and block maxima into `block_max`). With
    scores=None (FULL mode only) just the block maxima of ld_scores slots are written.
    block_aux (FULL, int32 shaped like block_max) receives each block's statistics word for
    csa2_full_select."""
    n_q = q_idx.shape[0]
    n_pool = pool_blocks.shape[1] if pool_blocks is not None else 0
    if scores is not None:
        ld_scores = scores.shape[1]
    elif ld_scores is None:
        raise ValueError("csa2_index_score: ld_scores is required when scores is None")
    _dims(q_idx, "csa2_index_score: q_idx", n_q, 32, 128)
    _dims(k_cache, "csa2_index_score: k_cache", None, 128)
    _index_common("csa2_index_score", n_q, w, kv_start, n_visible, scores, block_max,
                  pool_blocks, ld_scores)
    if block_aux is not None and (block_max is None or block_aux.shape != block_max.shape):
        raise ValueError("csa2_index_score: block_aux needs block_max and its shape")
    _check(lib.csa2_index_score(
        mode, n_q, q_idx.shape[1], q_idx.shape[2], _ptr(q_idx, torch.bfloat16, "q_idx"),
        _ptr(w, torch.float32, "w"), _ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
        _ptr(kv_start, torch.int64, "kv_start"), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(pool_blocks, torch.int32, "pool_blocks"), n_pool, 8,
        _ptr(scores, torch.float32, "scores"), ld_scores,
        _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0,
        _ptr(block_aux, torch.int32, "block_aux"), _stream(stream)))


def csa2_index_score_shared(q_idx, w, k_cache, kv_start: int, n_visible, scores,
                            block_max=None, stream=None):
    """Full-mode scores of queries that all read the cache from row kv_start (a host int),
    each up to its own n_visible."""
    n_q = q_idx.shape[0]
    _dims(q_idx, "csa2_index_score_shared: q_idx", n_q, 32, 128)
    _dims(k_cache, "csa2_index_score_shared: k_cache", None, 128)
    _dims(scores, "csa2_index_score_shared: scores", n_q, None)
    _index_common("csa2_index_score_shared", n_q, w, None, n_visible, scores, block_max, None,
                  scores.shape[1])
    _check(lib.csa2_index_score_shared(
        n_q, q_idx.shape[1], q_idx.shape[2], _ptr(q_idx, torch.bfloat16, "q_idx"),
        _ptr(w, torch.float32, "w"), _ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
        int(kv_start), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(scores, torch.float32, "scores"), scores.shape[1],
        _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0, _stream(stream)))


def csa2_index_score_mxfp4(mode, q_idx, w, k_codes, k_scales, kv_start, n_visible, scores,
                           block_max=None, pool_blocks=None, stream=None, ld_scores=None,
                           block_aux=None):
    """csa2_index_score over MXFP4 indexer keys: k_codes uint8 [E, 64] (two E2M1 codes per
    byte, low nibble first) and k_scales uint8 [E, 4] (E8M0, one per 32 channels). block_aux
    as csa2_index_score's, for csa2_full_select_mxfp4."""
    n_q = q_idx.shape[0]
    n_pool = pool_blocks.shape[1] if pool_blocks is not None else 0
    if scores is not None:
        ld_scores = scores.shape[1]
    elif ld_scores is None:
        raise ValueError("csa2_index_score_mxfp4: ld_scores is required when scores is None")
    if k_codes.shape[0] != k_scales.shape[0]:
        raise ValueError("csa2_index_score_mxfp4: k_codes and k_scales row counts differ")
    _dims(q_idx, "csa2_index_score_mxfp4: q_idx", n_q, 32, 128)
    _dims(k_codes, "csa2_index_score_mxfp4: k_codes", None, 64)
    _dims(k_scales, "csa2_index_score_mxfp4: k_scales", k_codes.shape[0], 4)
    _index_common("csa2_index_score_mxfp4", n_q, w, kv_start, n_visible, scores, block_max,
                  pool_blocks, ld_scores)
    if block_aux is not None and (block_max is None or block_aux.shape != block_max.shape):
        raise ValueError("csa2_index_score_mxfp4: block_aux needs block_max and its shape")
    _check(lib.csa2_index_score_mxfp4(
        mode, n_q, q_idx.shape[1], q_idx.shape[2], _ptr(q_idx, torch.bfloat16, "q_idx"),
        _ptr(w, torch.float32, "w"), _ptr(k_codes, torch.uint8, "k_codes"),
        _ptr(k_scales, torch.uint8, "k_scales"), k_codes.shape[0],
        _ptr(kv_start, torch.int64, "kv_start"), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(pool_blocks, torch.int32, "pool_blocks"), n_pool, 8,
        _ptr(scores, torch.float32, "scores"), ld_scores,
        _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0,
        _ptr(block_aux, torch.int32, "block_aux"), _stream(stream)))


def csa2_block_mean_keys(k_cache, kv_start, n_visible, km, km_start, n_blocks, max_blocks=None,
                         last_only=False, stream=None):
    """Block-mean keys (bf16, one row per 8 visible positions) of each query's E4M3 keys
    into km [R, 128] from row km_start[t]; n_blocks [n_q] int32 receives ceil(n_visible/8).
    max_blocks defaults to what fits in km; last_only recomputes only each query's latest
    block (after an append)."""
    n_q = kv_start.shape[0]
    if km.dim() != 2 or km.shape[1] != 128:
        raise ValueError("csa2_block_mean_keys: km must be [rows, 128]")
    _dims(k_cache, "csa2_block_mean_keys: k_cache", None, 128)
    _dims(n_visible, "csa2_block_mean_keys: n_visible", n_q)
    _dims(km_start, "csa2_block_mean_keys: km_start", n_q)
    _dims(n_blocks, "csa2_block_mean_keys: n_blocks", n_q)
    if max_blocks is None:
        max_blocks = max(1, km.shape[0])
    _check(lib.csa2_block_mean_keys(
        n_q, 128, 8, _ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
        _ptr(kv_start, torch.int64, "kv_start"), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(km, torch.bfloat16, "km"), _ptr(km_start, torch.int64, "km_start"), km.shape[0],
        int(max_blocks), _ptr(n_blocks, torch.int32, "n_blocks"), 1 if last_only else 0,
        _stream(stream)))


def csa2_index_score_bf16(mode, q_idx, w, k_rows, kv_start, n_visible, scores, block_max=None,
                          pool_blocks=None, stream=None, ld_scores=None):
    """csa2_index_score over bf16 key rows k_rows [E, 128] (the block-mean keys)."""
    n_q = q_idx.shape[0]
    n_pool = pool_blocks.shape[1] if pool_blocks is not None else 0
    if scores is not None:
        ld_scores = scores.shape[1]
    elif ld_scores is None:
        raise ValueError("csa2_index_score_bf16: ld_scores is required when scores is None")
    _dims(q_idx, "csa2_index_score_bf16: q_idx", n_q, 32, 128)
    _dims(k_rows, "csa2_index_score_bf16: k_rows", None, 128)
    _index_common("csa2_index_score_bf16", n_q, w, kv_start, n_visible, scores, block_max,
                  pool_blocks, ld_scores)
    _check(lib.csa2_index_score_bf16(
        mode, n_q, q_idx.shape[1], q_idx.shape[2], _ptr(q_idx, torch.bfloat16, "q_idx"),
        _ptr(w, torch.float32, "w"), _ptr(k_rows, torch.bfloat16, "k_rows"), k_rows.shape[0],
        _ptr(kv_start, torch.int64, "kv_start"), _ptr(n_visible, torch.int32, "n_visible"),
        _ptr(pool_blocks, torch.int32, "pool_blocks"), n_pool, 8,
        _ptr(scores, torch.float32, "scores"), ld_scores,
        _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0, _stream(stream)))


def csa2_block_pool(block_max, n_visible, pool_blocks, n_keep=2048, stream=None):
    """HSI pool block ids (ascending, -1 padded) into `pool_blocks` [n_q, >= n_keep]."""
    n_q = block_max.shape[0]
    _dims(block_max, "csa2_block_pool: block_max", n_q, None)
    _dims(n_visible, "csa2_block_pool: n_visible", n_q)
    _dims(pool_blocks, "csa2_block_pool: pool_blocks", n_q, (">=", n_keep))
    _check(lib.csa2_block_pool(
        block_max.shape[0], _ptr(block_max, torch.float32, "block_max"), block_max.shape[1],
        _ptr(n_visible, torch.int32, "n_visible"), 8, n_keep,
        _ptr(pool_blocks, torch.int32, "pool_blocks"), pool_blocks.shape[1], None, 0,
        _stream(stream)))


def csa2_topk(scores, topk_idx, k=512, n_cols=None, n_valid=None, block_max=None,
              pool_blocks=None, pool_use=None, stream=None):
    """Top-k positions (ascending, -1 padded) into `topk_idx` [n_q, >= k]. pool_use defaults
    to POOL_SLOTS when pool_blocks is given (a Reindex layer's scores), else POOL_NONE."""
    n_cols = scores.shape[1] if n_cols is None else n_cols
    if pool_use is None:
        pool_use = POOL_NONE if pool_blocks is None else POOL_SLOTS
    n_q = scores.shape[0]
    _dims(scores, "csa2_topk: scores", n_q, None)
    _dims(topk_idx, "csa2_topk: topk_idx", n_q, (">=", k))
    _dims(n_valid, "csa2_topk: n_valid", n_q)
    _dims(block_max, "csa2_topk: block_max", n_q, (">=", (n_cols + 7) // 8))
    _dims(pool_blocks, "csa2_topk: pool_blocks", n_q, None)
    _check(lib.csa2_topk(
        scores.shape[0], _ptr(scores, torch.float32, "scores"), scores.shape[1], n_cols,
        _ptr(n_valid, torch.int32, "n_valid"), _ptr(block_max, torch.float32, "block_max"),
        block_max.shape[1] if block_max is not None else 0, k, pool_use,
        _ptr(pool_blocks, torch.int32, "pool_blocks"),
        pool_blocks.shape[1] if pool_blocks is not None else 0, 8,
        _ptr(topk_idx, torch.int32, "topk_idx"), topk_idx.shape[1], None, 0, _stream(stream)))


def csa2_pool_topk(block_max, n_visible, pool_blocks, scores, topk_idx, n_keep=2048, k=512,
                   n_cols=None, stream=None):
    """csa2_block_pool then csa2_topk among the pool's candidates, in one kernel: pool ids
    into `pool_blocks` [n_q, >= n_keep] and positions into `topk_idx` [n_q, >= k]."""
    n_cols = scores.shape[1] if n_cols is None else n_cols
    n_q = block_max.shape[0]
    _dims(block_max, "csa2_pool_topk: block_max", n_q, None)
    _dims(n_visible, "csa2_pool_topk: n_visible", n_q)
    _dims(pool_blocks, "csa2_pool_topk: pool_blocks", n_q, (">=", n_keep))
    _dims(scores, "csa2_pool_topk: scores", n_q, None)
    _dims(topk_idx, "csa2_pool_topk: topk_idx", n_q, (">=", k))
    _check(lib.csa2_pool_topk(
        block_max.shape[0], _ptr(block_max, torch.float32, "block_max"), block_max.shape[1],
        _ptr(n_visible, torch.int32, "n_visible"), 8, n_keep,
        _ptr(pool_blocks, torch.int32, "pool_blocks"), pool_blocks.shape[1],
        _ptr(scores, torch.float32, "scores"), scores.shape[1], n_cols, k,
        _ptr(topk_idx, torch.int32, "topk_idx"), topk_idx.shape[1], _stream(stream)))


def csa2_pool_candidates(block_max, n_visible, pool_blocks, cand_blocks, n_keep=2048, k=512,
                         stream=None):
    """The HSI pool into `pool_blocks` [n_q, >= n_keep] and the Full layer's candidate blocks
    (the pool blocks that can hold one of its k best entries) into `cand_blocks`
    [n_q, >= n_keep], both ascending and -1 padded."""
    n_q = block_max.shape[0]
    _dims(block_max, "csa2_pool_candidates: block_max", n_q, None)
    _dims(n_visible, "csa2_pool_candidates: n_visible", n_q)
    _dims(pool_blocks, "csa2_pool_candidates: pool_blocks", n_q, (">=", n_keep))
    _dims(cand_blocks, "csa2_pool_candidates: cand_blocks", n_q, (">=", n_keep))
    _check(lib.csa2_pool_candidates(
        block_max.shape[0], _ptr(block_max, torch.float32, "block_max"), block_max.shape[1],
        _ptr(n_visible, torch.int32, "n_visible"), 8, n_keep,
        _ptr(pool_blocks, torch.int32, "pool_blocks"), pool_blocks.shape[1], k,
        _ptr(cand_blocks, torch.int32, "cand_blocks"), cand_blocks.shape[1], _stream(stream)))


def _full_select_args(fn, block_max, block_aux, n_visible, pool_blocks, q_idx, w, kv_start,
                      topk_idx, n_keep, k):
    n_q = block_max.shape[0]
    _dims(block_max, f"{fn}: block_max", n_q, None)
    if not isinstance(block_aux, torch.Tensor) or block_aux.shape != block_max.shape:
        raise ValueError(f"{fn}: block_aux must have block_max's shape")
    _dims(n_visible, f"{fn}: n_visible", n_q)
    _dims(pool_blocks, f"{fn}: pool_blocks", n_q, (">=", n_keep))
    _dims(q_idx, f"{fn}: q_idx", n_q, 32, 128)
    _dims(w, f"{fn}: w", n_q, 32)
    _dims(kv_start, f"{fn}: kv_start", n_q)
    _dims(topk_idx, f"{fn}: topk_idx", n_q, (">=", k))
    return n_q


def csa2_full_select(block_max, block_aux, n_visible, pool_blocks, q_idx, w, k_cache, kv_start,
                     topk_idx, n_keep=2048, k=512, stream=None):
    """The decoder Full layer's selection in one call (E4M3 keys, bf16 query): the HSI pool
    into `pool_blocks` [n_q, >= n_keep] and the Full Top-K into `topk_idx` [n_q, >= k], from
    the block maxima and statistics (block_aux) of the Full pass of q_idx [n_q, 32, 128] and
    w [n_q, 32] over k_cache [E, 128]."""
    n_q = _full_select_args("csa2_full_select", block_max, block_aux, n_visible, pool_blocks,
                            q_idx, w, kv_start, topk_idx, n_keep, k)
    _dims(k_cache, "csa2_full_select: k_cache", None, 128)
    _check(lib.csa2_full_select(
        n_q, _ptr(block_max, torch.float32, "block_max"), block_max.shape[1],
        _ptr(n_visible, torch.int32, "n_visible"), 8, n_keep,
        _ptr(pool_blocks, torch.int32, "pool_blocks"), pool_blocks.shape[1], 32, 128,
        _ptr(q_idx, torch.bfloat16, "q_idx"), _ptr(w, torch.float32, "w"),
        _ptr(k_cache, torch.uint8, "k_cache"), k_cache.shape[0],
        _ptr(kv_start, torch.int64, "kv_start"), _ptr(block_aux, torch.int32, "block_aux"), k,
        _ptr(topk_idx, torch.int32, "topk_idx"), topk_idx.shape[1], _stream(stream)))


def csa2_full_select_mxfp4(block_max, block_aux, n_visible, pool_blocks, q_idx, w, k_codes,
                           k_scales, kv_start, topk_idx, n_keep=2048, k=512, stream=None):
    """csa2_full_select over MXFP4 indexer keys (k_codes uint8 [E, 64], k_scales uint8
    [E, 4]), from the block maxima and statistics of the csa2_index_score_mxfp4 Full pass."""
    n_q = _full_select_args("csa2_full_select_mxfp4", block_max, block_aux, n_visible,
                            pool_blocks, q_idx, w, kv_start, topk_idx, n_keep, k)
    if k_codes.shape[0] != k_scales.shape[0]:
        raise ValueError("csa2_full_select_mxfp4: k_codes and k_scales row counts differ")
    _dims(k_codes, "csa2_full_select_mxfp4: k_codes", None, 64)
    _dims(k_scales, "csa2_full_select_mxfp4: k_scales", k_codes.shape[0], 4)
    _check(lib.csa2_full_select_mxfp4(
        n_q, _ptr(block_max, torch.float32, "block_max"), block_max.shape[1],
        _ptr(n_visible, torch.int32, "n_visible"), 8, n_keep,
        _ptr(pool_blocks, torch.int32, "pool_blocks"), pool_blocks.shape[1], 32, 128,
        _ptr(q_idx, torch.bfloat16, "q_idx"), _ptr(w, torch.float32, "w"),
        _ptr(k_codes, torch.uint8, "k_codes"), _ptr(k_scales, torch.uint8, "k_scales"),
        k_codes.shape[0], _ptr(kv_start, torch.int64, "kv_start"),
        _ptr(block_aux, torch.int32, "block_aux"), k, _ptr(topk_idx, torch.int32, "topk_idx"),
        topk_idx.shape[1], _stream(stream)))


def csa2_sparse_attn(q, kv_fp4, kv_scale, kv_start, topk_idx, window_kv, swa_start, n_swa,
                     softmax_scale, out, lse=None, workspace=None, k=None, stream=None):
    """Joint sparse attention into `out` [n_q, 64, 512] bf16 (and `lse` [n_q, 64])."""
    n_q = q.shape[0]
    k = topk_idx.shape[1] if k is None else k
    ws = workspace
    need = workspace_bytes(OP_SPARSE_ATTN, n_q, 0, k)
    if need and ws is None:
        raise ValueError(f"csa2_sparse_attn: a workspace of {need} bytes is required")
    for name, t, row in (("kv_fp4", kv_fp4, 256), ("kv_scale", kv_scale, 32)):
        if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1 \
                or t.shape[1] < row:
            raise ValueError(f"{name}: expected a device uint8 [rows, >= {row}] view")
    if kv_scale.shape[0] != kv_fp4.shape[0]:
        raise ValueError("csa2_sparse_attn: kv_fp4 and kv_scale row counts differ")
    _dims(q, "csa2_sparse_attn: q", n_q, 64, 512)
    _dims(kv_start, "csa2_sparse_attn: kv_start", n_q)
    if k > 0:
        _dims(topk_idx, "csa2_sparse_attn: topk_idx", n_q, (">=", k))
    _dims(window_kv, "csa2_sparse_attn: window_kv", None, 512)
    _dims(swa_start, "csa2_sparse_attn: swa_start", n_q)
    _dims(n_swa, "csa2_sparse_attn: n_swa", n_q)
    _dims(out, "csa2_sparse_attn: out", n_q, 64, 512)
    _dims(lse, "csa2_sparse_attn: lse", n_q, 64)
    _check(lib.csa2_sparse_attn(
        n_q, q.shape[1], q.shape[2], _ptr(q, torch.bfloat16, "q"),
        kv_fp4.data_ptr(), kv_fp4.stride(0), kv_scale.data_ptr(), kv_scale.stride(0),
        kv_fp4.shape[0], _ptr(kv_start, torch.int64, "kv_start"),
        _ptr(topk_idx, torch.int32, "topk_idx"), topk_idx.shape[1], k,
        _ptr(window_kv, torch.uint8, "window_kv"), window_kv.shape[0],
        _ptr(swa_start, torch.int64, "swa_start"), _ptr(n_swa, torch.int32, "n_swa"),
        float(softmax_scale), _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(ws, None, "workspace"), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream)))
