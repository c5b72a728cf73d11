"""End-to-end layer stacks (Full -> pool -> Reindex -> Reuse) on the GPU against the
oracle's own stack, plus determinism and the Reuse identity."""
import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O
from tests.parity_util import (assert_attn_close, assert_set_band, band_of, np_u16)

pytestmark = pytest.mark.gpu


def check_query(wl, buf, t, seq=None, report=None):
    """Compare every layer of query t with the oracle stack run on the same inputs."""
    from compressed_kv_cache_csa2_amd import synth
    seq = seq or synth.sequence_to_host(wl, t)
    nv = seq["n_visible"]
    scale = wl.softmax_scale
    pool_ref = pool_gpu = None
    idx_ref = None
    same_sets = True
    n_cmp = 0
    for li, lay in enumerate(seq["layers"]):
        idx_gpu = buf.published[li][t].cpu().numpy()
        if lay["mode"] == "full":
            res = O.full_layer(lay["q_idx"], lay["w"], seq["k_cache"], 0, nv, lay["q"],
                               seq["kv_fp4"], seq["kv_scale"], lay["window_kv"], 0,
                               lay["n_swa"], scale, with_pool=wl.with_pool)
            kth, band = band_of(res["scores"], 512)
            same_sets = assert_set_band(idx_gpu, res["idx"], lambda p: res["scores"][p], kth, band,
                                        f"q{t} L{li} full top-k")
            if wl.with_pool:
                pool_gpu = buf.pool[t].cpu().numpy()
                bm = O.block_max(res["scores"][:nv])
                bm[(nv - 1) // 8] = np.inf
                kb, bb = band_of(bm, 2048)
                same_pool = assert_set_band(pool_gpu, res["pool"], lambda b: bm[b], kb, bb,
                                            f"q{t} pool")
                pool_ref = res["pool"]
                if not same_pool:
                    same_sets = False
            idx_ref = res["idx"]
        elif lay["mode"] == "reindex":
            res = O.reindex_layer(lay["q_idx"], lay["w"], seq["k_cache"], 0, nv, pool_ref, lay["q"],
                                  seq["kv_fp4"], seq["kv_scale"], lay["window_kv"], 0,
                                  lay["n_swa"], scale)
            if same_sets:
                padded = np.full(2048, -1, np.int64)
                padded[:len(pool_ref)] = pool_ref
                pos_of_slot = O.slots_to_positions(np.arange(16384), padded)
                score_at = dict(zip(pos_of_slot.tolist(), res["scores"].tolist()))
                kth, band = band_of(res["scores"], 512)
                same_sets = assert_set_band(idx_gpu, res["idx"], lambda p: score_at[p], kth, band,
                                            f"q{t} L{li} reindex top-k")
            idx_ref = res["idx"]
        else:
            res = O.reuse_layer(idx_ref, lay["q"], seq["kv_fp4"], seq["kv_scale"], 0,
                                lay["window_kv"], 0, lay["n_swa"], scale)
        if same_sets:
            rel = assert_attn_close(buf.out[li][t].float().cpu().numpy(), res["out"],
                                    f"q{t} L{li} {lay['mode']} attention")
            n_cmp += 1
            if report is not None:
                report.append((t, li, rel))
    return n_cmp


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
    assert compared >= 3 * len(wl.layers)


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
