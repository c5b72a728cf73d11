"""The write side's compressor and indexer-key projection on the GPU against the oracle,
and the chain compressor -> quantising writes."""
import numpy as np
import pytest
import torch

import oracle.csa2_oracle as O
from tests.parity_util import np_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C(dev):
    from compressed_kv_cache_csa2_amd import csa2
    return csa2


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("m,t", [(1, 75), (2, 75), (2, 2048), (3, 50), (8, 64)])
def test_compress_kv_parity(C, dev, m, t):
    c = _bf16((t, 512), 60 + m)
    z = _bf16((t, 512), 70 + m, 2.0)
    n_out = t // m
    out = torch.full((n_out + 2, 512), 7.0, dtype=torch.bfloat16, device=dev)
    C.csa2_compress_kv(c.to(dev), z.to(dev), out, m)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = O.compress_entries(np_u16(c), np_u16(z), m)
    if m == 1:
        assert np.array_equal(np_u16(out[:n_out]), np_u16(c))
    # bf16 rounding (half a step, 2^-9 relative) plus float32 evaluation of the gates
    err = np.abs(got[:n_out] - ref)
    lim = 2.0 ** -8 * np.abs(ref) + 1e-6
    assert np.all(err <= lim), f"m={m}: worst {err.max():.3e}"
    assert np.all(got[n_out:] == 7.0)      # rows past the last entry untouched


def test_compress_kv_dominant_gate_picks_its_token(C, dev):
    c = _bf16((64, 512), 80)
    z = torch.zeros((64, 512), dtype=torch.bfloat16)
    z[1::2, :200] = 90.0
    z[0::2, 200:] = 90.0
    out = torch.empty((32, 512), dtype=torch.bfloat16, device=dev)
    C.csa2_compress_kv(c.to(dev), z.to(dev), out, 2)
    torch.cuda.synchronize()
    o = np_u16(out)
    cb = np_u16(c)
    assert np.array_equal(o[:, :200], cb[1::2, :200])
    assert np.array_equal(o[:, 200:], cb[0::2, 200:])


@pytest.mark.parametrize("n", [1, 32, 100])
def test_project_index_key_parity(C, dev, n):
    e = _bf16((n, 512), 90 + n)
    w = _bf16((128, 512), 91, 0.05)
    out = torch.full((n, 128), 3.0, dtype=torch.bfloat16, device=dev)
    C.csa2_project_index_key(e.to(dev), w.to(dev), out)
    torch.cuda.synchronize()
    ev, wv = O.bf16_decode(np_u16(e)), O.bf16_decode(np_u16(w))
    ref = O.project_index_keys(ev, np_u16(w))
    terms = np.abs(ev) @ np.abs(wv).T
    got = out.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6 * terms + 1e-30), err.max()


def test_compressor_chain_writes_what_the_oracle_quantises(C, dev):
    """Hidden-state projections -> entries (m = 2) -> FP4 latent rows, and entries ->
    indexer keys -> E4M3 rows: every stored byte equals the oracle's quantisation of the
    GPU's own bf16 entries and keys (the rounding decisions are taken on the same values)."""
    t = 1201                                 # one token short of a 601st entry
    c = _bf16((t, 512), 100).to(dev)
    z = _bf16((t, 512), 101, 1.5).to(dev)
    w = _bf16((128, 512), 102, 0.05).to(dev)
    n = t // 2
    ent = torch.empty((n, 512), dtype=torch.bfloat16, device=dev)
    key = torch.empty((n, 128), dtype=torch.bfloat16, device=dev)
    C.csa2_compress_kv(c, z, ent, 2)
    C.csa2_project_index_key(ent, w, key)
    rows = torch.arange(n, dtype=torch.int64, device=dev)
    kv_fp4 = torch.zeros((n, 256), dtype=torch.uint8, device=dev)
    kv_scale = torch.zeros((n, 32), dtype=torch.uint8, device=dev)
    k_cache = torch.zeros((n, 128), dtype=torch.uint8, device=dev)
    C.csa2_write_latent(ent, rows, kv_fp4, kv_scale)
    C.csa2_write_e4m3(key, rows, k_cache)
    torch.cuda.synchronize()
    p, s = O.fp4_latent_quantize(ent.float().cpu().numpy())
    assert np.array_equal(kv_fp4.cpu().numpy(), p) and np.array_equal(kv_scale.cpu().numpy(), s)
    assert np.array_equal(k_cache.cpu().numpy(), O.e4m3_round(key.float().cpu().numpy()))
    ref = O.compress_entries(np_u16(c), np_u16(z), 2)
    got = ent.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
