"""End-to-end layer stacks (Full -> pool -> Reindex -> Reuse) on the GPU against the
oracle, plus determinism, the Reuse identity and HIP-graph replay."""
import pytest
import torch

from tests.parity_util import check_query

pytestmark = pytest.mark.gpu


def test_tiny_decode_4k_full_layer(dev):
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_workload("tiny_decode_4k").to(dev)
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    assert check_query(wl, buf, 0) == 1


def test_small_decode_stack_with_pool(dev):
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_decode("small_stack", 4, 0, synth.DECODE_LAYERS, True, 32,
                           n_visible=[40000, 17000, 3001, 16384 + 8], kv_gap=9, seed=21).to(dev)
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    compared = sum(check_query(wl, buf, t) for t in range(wl.n_q))
    assert compared == wl.n_q * len(wl.layers)


def test_determinism_and_reuse_identity(dev):
    """Two runs are bitwise identical, and a Reuse layer given the Full layer's own query
    and window reproduces the Full layer's output bitwise."""
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_decode("ident", 3, 30000, synth.DECODE_LAYERS, True, 16, seed=22).to(dev)
    wl.layers[2].q = wl.layers[0].q.clone()
    wl.layers[2].window_kv = wl.layers[0].window_kv.clone()
    wl.layers[1].q_idx = wl.layers[0].q_idx.clone()   # Reindex with the Full query
    wl.layers[1].w = wl.layers[0].w.clone()
    b1 = layers.alloc_buffers(wl)
    b2 = layers.alloc_buffers(wl)
    layers.run_layers(wl, b1)
    layers.run_layers(wl, b2)
    torch.cuda.synchronize()
    assert torch.equal(b1.out.view(torch.int16), b2.out.view(torch.int16))
    assert torch.equal(b1.idx, b2.idx) and torch.equal(b1.pool, b2.pool)
    assert torch.equal(b1.lse, b2.lse)
    # Reuse layer 2 used the Reindex layer's indices; Reindex with the Full query reproduces
    # the Full Top-K (every winner lies in the pool), so layer 2 equals layer 0.
    assert torch.equal(b1.idx[1], b1.idx[0])
    assert torch.equal(b1.out[2].view(torch.int16), b1.out[0].view(torch.int16))


def test_graph_replay_matches_eager(dev):
    """The step captured in a HIP graph and replayed several times (with eager work and
    synchronisations in between) gives the eager result bitwise on every replay."""
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_decode("graph", 4, 20000, synth.DECODE_LAYERS, True, 16, seed=23).to(dev)
    eager = layers.alloc_buffers(wl)
    layers.run_layers(wl, eager)
    torch.cuda.synchronize()
    buf = layers.alloc_buffers(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        layers.run_layers(wl, buf, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layers.run_layers(wl, buf, stream=s)
    for rep in range(3):
        buf.out.zero_()
        buf.idx[:2].fill_(-7)      # the slots the Full and Reindex layers publish
        buf.pool.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf.idx, eager.idx), rep
        assert torch.equal(buf.pool, eager.pool), rep
        assert torch.equal(buf.out.view(torch.int16), eager.out.view(torch.int16)), rep
        layers.run_layers(wl, eager)   # eager work between replays
        torch.cuda.synchronize()


def test_small_decode_stack_with_mxfp4_keys(dev):
    """The decoder stack over MXFP4 indexer keys against the oracle's MXFP4 scoring."""
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_decode("small_stack_mxfp4", 3, 0, synth.DECODE_LAYERS, True, 32,
                           n_visible=[40000, 17000, 3001], kv_gap=9, seed=24,
                           mxfp4=True).to(dev)
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    compared = sum(check_query(wl, buf, t) for t in range(wl.n_q))
    assert compared == wl.n_q * len(wl.layers)


def test_small_encoder_schedule(dev):
    """The encoder's schedule (2 SWA-only layers, then 3 x (Full + 5 Reuse), each group on
    its own cache set) over a small causal chunk: every layer of sampled queries against
    the oracle."""
    from compressed_kv_cache_csa2_amd import layers, synth
    wl = synth.make_encoder("small_encoder", n_q=48, n_entries=3000, seed=24).to(dev)
    assert len(wl.group_caches) == 2
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    compared = sum(check_query(wl, buf, t) for t in (0, 17, wl.n_q - 1))
    assert compared == 3 * len(wl.layers)
    # the groups really read different caches: group 1's Full layer selects differently
    assert not torch.equal(buf.idx[2], buf.idx[8])


@pytest.mark.parametrize("kind", ["prefill", "encoder"])
def test_small_shared_sequence_stacks_with_the_mxfp8_query(dev, kind):
    """The grouped MXFP8-query indexer (queries sharing one sequence) through whole stacks:
    a small chunked prefill and the encoder schedule with the query quantised per layer,
    every layer of sampled queries checked against the oracle's MXFP8-query scores, its
    Top-K and attention over the GPU's indices."""
    from compressed_kv_cache_csa2_amd import layers, synth
    if kind == "prefill":
        wl = synth.make_prefill("small_prefill_q8", n_q=70, n_entries=5000, seed=27).to(dev)
    else:
        wl = synth.make_encoder("small_encoder_q8", n_q=48, n_entries=3000, seed=28).to(dev)
    wl.q8 = True
    buf = layers.alloc_buffers(wl)
    layers.run_layers(wl, buf)
    torch.cuda.synchronize()
    queries = (0, 23, wl.n_q - 1)
    compared = sum(check_query(wl, buf, t) for t in queries)
    assert compared == len(queries) * len(wl.layers)


@pytest.mark.parametrize("kind", ["hisa", "encoder", "encoder_q8"])
def test_graph_replay_of_the_other_stacks(dev, kind):
    """The block-mean filter stack and the encoder schedule (also with the MXFP8 query)
    captured in a HIP graph give the eager result bitwise on every replay (eager work in
    between)."""
    from compressed_kv_cache_csa2_amd import layers, synth
    if kind == "hisa":
        wl = synth.make_decode("g_hisa", 3, 20000, synth.DECODE_LAYERS, True, 16, seed=25).to(dev)
        means = layers.build_block_means(wl)
        kw = dict(coarse="hisa", means=means)
    else:
        wl = synth.make_encoder("g_enc", n_q=40, n_entries=2500, seed=26).to(dev)
        wl.q8 = kind == "encoder_q8"
        kw = {}
    eager = layers.alloc_buffers(wl)
    layers.run_layers(wl, eager, **kw)
    torch.cuda.synchronize()
    buf = layers.alloc_buffers(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        layers.run_layers(wl, buf, stream=s, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layers.run_layers(wl, buf, stream=s, **kw)
    # the slots the indexer layers publish (Reuse and SWA layers publish none of their own)
    rows = [li for li, lay in enumerate(wl.layers) if lay.mode in ("full", "reindex")]
    for rep in range(3):
        buf.out.zero_()
        buf.lse.zero_()
        for li in rows:
            buf.idx[li].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li in rows:
            assert torch.equal(buf.idx[li], eager.idx[li]), (rep, li)
        assert torch.equal(buf.out.view(torch.int16), eager.out.view(torch.int16)), rep
        assert torch.equal(buf.lse, eager.lse), rep
        layers.run_layers(wl, eager, **kw)
