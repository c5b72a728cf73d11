"""The named workloads at their full sizes on the GPU, checked against the oracle: every
query of the decodes (32K, 256K, 256K with MXFP4 indexer keys or the block-mean filter, 1M),
and queries spread over the whole batch for the prefill and the encoder. decode_256k runs
exactly as bench.py times it: the layer stack captured in a HIP graph on a side stream and
replayed."""
import sys
import time

import pytest
import torch

from tests.parity_util import check_query

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


def _run(name, dev, graph=False):
    from compressed_kv_cache_csa2_amd import layers, synth
    t0 = time.time()
    wl = synth.make_workload(name, device=dev)
    torch.cuda.synchronize()
    _log(f"{name}: generated {wl.n_q} queries in {time.time() - t0:.1f} s")
    buf = layers.alloc_buffers(wl)
    if graph:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            layers.run_layers(wl, buf, stream=s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            layers.run_layers(wl, buf, stream=s)
        buf.out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for _ in range(2):
                g.replay()
        torch.cuda.synchronize()
    else:
        layers.run_layers(wl, buf)
        torch.cuda.synchronize()
    _log(f"{name}: layer stack ran")
    return wl, buf


def _check(wl, buf, queries):
    n = 0
    for t in queries:
        t0 = time.time()
        n += check_query(wl, buf, t)
        _log(f"{wl.name}: query {t} checked ({time.time() - t0:.1f} s)")
    return n


def test_decode_32k_every_query(dev):
    wl, buf = _run("decode_32k", dev)
    assert _check(wl, buf, range(wl.n_q)) == wl.n_q
    del wl, buf
    torch.cuda.empty_cache()


def test_decode_256k_every_query_as_benched(dev):
    """The headline configuration, every one of its 32 queries through all five layers, run
    exactly as bench.py times it (a HIP graph replayed on a side stream)."""
    wl, buf = _run("decode_256k", dev, graph=True)
    queries = range(wl.n_q)
    assert _check(wl, buf, queries) == wl.n_q * len(wl.layers)
    del wl, buf
    torch.cuda.empty_cache()


def test_decode_256k_mxfp4_every_query(dev):
    wl, buf = _run("decode_256k_mxfp4", dev)
    assert _check(wl, buf, range(wl.n_q)) == wl.n_q * len(wl.layers)
    del wl, buf
    torch.cuda.empty_cache()


def test_decode_256k_block_mean_filter_every_query(dev):
    """decode_256k through the block-mean filter (every indexer layer's pool captured),
    checked on every query; the whole stack then reproduces the same indices."""
    from compressed_kv_cache_csa2_amd import layers, synth
    from tests.parity_util import check_query_hisa
    wl = synth.make_workload("decode_256k", device=dev)
    means = layers.build_block_means(wl)
    buf = layers.alloc_buffers(wl)
    pools = {}
    for li, lay in enumerate(wl.layers):
        if lay.mode in ("full", "reindex"):
            layers.hisa_select(wl, lay, buf, means, buf.idx[li])
            pools[li] = buf.pool.clone()
    torch.cuda.synchronize()
    idx = buf.idx.clone()
    layers.run_layers(wl, buf, coarse="hisa", means=means)
    torch.cuda.synchronize()
    assert torch.equal(buf.idx, idx)
    _log("decode_256k block-mean filter: stack ran")
    n = 0
    queries = range(wl.n_q)
    for t in queries:
        n += check_query_hisa(wl, idx, pools, buf.out, t)
        _log(f"decode_256k block-mean filter: query {t} checked")
    assert n == len(queries) * len(wl.layers)
    del wl, buf, means
    torch.cuda.empty_cache()


def test_prefill_128k_m2_spread(dev):
    """The first two queries, the last, and one in every 32 between (their visible
    contexts grow along the chunk)."""
    wl, buf = _run("prefill_128k_m2", dev)
    queries = sorted({0, 1, wl.n_q - 1} | set(range(31, wl.n_q, 32)))
    assert _check(wl, buf, queries) == len(queries)
    del wl, buf
    torch.cuda.empty_cache()


def test_encoder_128k_m2_spread(dev):
    wl, buf = _run("encoder_128k_m2", dev)
    queries = sorted({wl.n_q - 1} | set(range(0, wl.n_q, 64)))
    assert _check(wl, buf, queries) == len(queries) * len(wl.layers)
    del wl, buf
    torch.cuda.empty_cache()


def test_decode_1m_every_query(dev):
    wl, buf = _run("decode_1m", dev)
    assert _check(wl, buf, range(wl.n_q)) == wl.n_q * len(wl.layers)
    del wl, buf
    torch.cuda.empty_cache()
