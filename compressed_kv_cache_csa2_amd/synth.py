"""Seeded synthetic inputs for the CSA2 read path.

This module only makes inputs: random draws, the write-side encoders that store them in
the cache formats (bf16, E4M3, E2M1 with an E4M3 scale per 16 channels), and planted
high-affinity positions. It holds none of the read path's arithmetic (no decoding, no
scoring, no selection, no attention) and is imported by the tests, the benchmark and
users who want the same workloads; the oracle never imports it.

Every draw comes from a torch.Generator seeded from (seed, tensor name, sequence) on the
device that will hold the tensor, so a workload is reproducible on a given device type.
Small workloads are drawn on the host; large ones on the GPU and copied to the host only
for the sequences a check samples.

Workloads (sizes are those of the decode and prefill settings the pages describe:
64 heads x 512 main queries, 32 x 128 indexer queries, Top-512, SWA-128, 8-position
blocks, 2,048 pool blocks):
  tiny_decode_4k    1 query, 4,096 entries, Full only, 16 planted positions.
  decode_32k        16 queries x 32,768 entries, Full only, 64 planted per query.
  decode_256k       32 queries x 262,144 entries; Full (+pool), Reindex, 3 x Reuse.
                    Decoder stacks with a Reindex layer carry a second needle set, planted
                    along that layer's own indexer query (its keys only), so that what the
                    Full layer's pool loses for a later Reindex layer can be measured.
  prefill_128k_m2   4,096 causal queries over one sequence of 131,072 entries at
                    compression ratio 2 (entry e covers source tokens 2e and 2e+1 and is
                    visible from token p when 2e+1 <= p); Full only.
  decode_1m         64 queries x 1,048,576 entries; Full (+pool), Reindex, 3 x Reuse;
                    64 needles per query at evenly spaced positions.
  encoder_128k_m2   the causal encoder's schedule over the prefill_128k_m2 chunk: two
                    SWA-only layers, then three groups of one Full layer (with its own
                    main-KV and indexer-K cache) and five Reuse layers.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import torch

N_HEADS, HEAD_DIM = 64, 512
IDX_HEADS, IDX_DIM = 32, 128
TOPK, WINDOW = 512, 128
BLOCK, POOL_BLOCKS = 8, 2048
SOFTMAX_SCALE = 1.0 / math.sqrt(HEAD_DIM)
PLANT_SHIFT = 3.0

DECODE_LAYERS = ("full", "reindex", "reuse", "reuse", "reuse")
ENCODER_LAYERS = ("swa", "swa") + ("full",) + ("reuse",) * 5 + ("full",) + ("reuse",) * 5 \
    + ("full",) + ("reuse",) * 5


@dataclass
class LayerInputs:
    mode: str                       # "full", "reindex", "reuse" or "swa" (window only)
    q: torch.Tensor                 # bf16 [n_q, 64, 512]
    window_kv: torch.Tensor         # uint8 [rows, 512] E4M3
    swa_start: torch.Tensor         # int64 [n_q]
    n_swa: torch.Tensor             # int32 [n_q]
    q_idx: torch.Tensor | None = None   # bf16 [n_q, 32, 128]
    w: torch.Tensor | None = None       # float32 [n_q, 32]
    group: int = 0                  # which cache set the layer reads (encoder groups)


@dataclass
class Workload:
    name: str
    n_q: int
    n_ctx: int                      # largest visible count
    kv_start: torch.Tensor          # int64 [n_q]
    n_visible: torch.Tensor         # int32 [n_q]
    k_cache: torch.Tensor           # uint8 [E, 128] E4M3
    kv_fp4: torch.Tensor            # uint8 [E, 256] two E2M1 codes per byte
    kv_scale: torch.Tensor          # uint8 [E, 32] E4M3
    layers: list = field(default_factory=list)
    with_pool: bool = False
    planted: torch.Tensor | None = None  # int64 [n_q, n_plant] positions (or None)
    # positions planted along the first Reindex layer's indexer query (or None)
    planted_re: torch.Tensor | None = None
    softmax_scale: float = SOFTMAX_SCALE
    # MXFP4 copy of the indexer keys (the same draws): codes [E, 64], E8M0 scales [E, 4]
    k_codes: torch.Tensor | None = None
    k_scales: torch.Tensor | None = None
    # every query reads the cache from this row (chunked prefill), else None
    shared_start: int | None = None
    # cache sets of groups 1, 2, ... as (k_cache, kv_fp4, kv_scale); group 0 is the above
    group_caches: list = field(default_factory=list)
    # score the MXFP4 keys with the indexer query quantised to MXFP8 (scaled MFMA path)
    q8: bool = False

    def cache(self, group: int = 0):
        """(k_cache, kv_fp4, kv_scale) of a layer group."""
        if group == 0:
            return self.k_cache, self.kv_fp4, self.kv_scale
        return self.group_caches[group - 1]

    @property
    def n_entries(self) -> int:
        return int(self.k_cache.shape[0])

    def to(self, device) -> "Workload":
        """A copy with every tensor on `device` (same bytes)."""
        mv = lambda x: None if x is None else x.to(device)
        layers = [LayerInputs(mode=l.mode, q=mv(l.q), window_kv=mv(l.window_kv),
                              swa_start=mv(l.swa_start), n_swa=mv(l.n_swa), q_idx=mv(l.q_idx),
                              w=mv(l.w), group=l.group) for l in self.layers]
        return Workload(name=self.name, n_q=self.n_q, n_ctx=self.n_ctx, kv_start=mv(self.kv_start),
                        n_visible=mv(self.n_visible), k_cache=mv(self.k_cache),
                        kv_fp4=mv(self.kv_fp4), kv_scale=mv(self.kv_scale), layers=layers,
                        with_pool=self.with_pool, planted=self.planted,
                        planted_re=self.planted_re, softmax_scale=self.softmax_scale,
                        k_codes=mv(self.k_codes), k_scales=mv(self.k_scales), shared_start=self.shared_start,
                        group_caches=[tuple(mv(x) for x in c) for c in self.group_caches],
                        q8=self.q8)


# ----------------------------------------------------------------------------- encoders

def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round to bfloat16 (nearest even)."""
    return x.to(torch.bfloat16)


def encode_e4m3(x: torch.Tensor) -> torch.Tensor:
    """Round to OCP E4M3FN (nearest even, saturating at +-448); returns the bytes."""
    return x.float().clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def _e4m3_bytes_to_float(b: torch.Tensor) -> torch.Tensor:
    return b.view(torch.float8_e4m3fn).float()


def encode_fp4_rows(x: torch.Tensor):
    """Encode rows of 512 values as E2M1 codes with one E4M3 scale per 16 channels.

    Per group of 16: scale = E4M3(amax / 6); each value's exact quotient x/scale is
    rounded to the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6} (nearest, ties to the even code,
    saturating at 6).
    A zero scale gives zero codes. Codes 2m and 2m+1 share byte m, low nibble first.
    Returns (payload uint8 [..., 256], scales uint8 [..., 32]).
    """
    x = x.float()
    g = x.reshape(*x.shape[:-1], x.shape[-1] // 16, 16)
    amax = g.abs().amax(dim=-1)
    s_code = encode_e4m3(amax / 6.0)
    s = _e4m3_bytes_to_float(s_code).unsqueeze(-1)
    # nearest code of the exact quotient g / s: |g| against each grid midpoint times s
    # (exact in float32), a midpoint going to the even code
    a = g.abs()
    code = ((a > 0.25 * s).to(torch.uint8) + (a >= 0.75 * s).to(torch.uint8)
            + (a > 1.25 * s).to(torch.uint8) + (a >= 1.75 * s).to(torch.uint8)
            + (a > 2.5 * s).to(torch.uint8) + (a >= 3.5 * s).to(torch.uint8)
            + (a > 5.0 * s).to(torch.uint8))
    code = code | (((g < 0) & (code > 0)).to(torch.uint8) << 3)
    code = torch.where(s > 0, code, torch.zeros_like(code))
    code = code.reshape(x.shape)
    payload = code[..., 0::2] | (code[..., 1::2] << 4)
    return payload.contiguous(), s_code.contiguous()


def _e2m1_codes(y: torch.Tensor) -> torch.Tensor:
    """E2M1 codes of y: nearest grid magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the
    even code, saturating at 6; the sign bit only on nonzero codes."""
    a = y.abs()
    code = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8) + (a > 1.25).to(torch.uint8)
            + (a >= 1.75).to(torch.uint8) + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
            + (a > 5.0).to(torch.uint8))
    sign = ((y < 0) & (code > 0)).to(torch.uint8) << 3
    return code | sign


def encode_mxfp4_rows(x: torch.Tensor):
    """Encode rows of 128 values in OCP MXFP4: E2M1 codes with one E8M0 scale per 32.

    Per group of 32 (the OCP microscaling recipe): shared exponent X = floor(log2 amax) - 2
    (2 is E2M1's largest exponent), scale byte X + 127 kept in 1..254; each value x / 2^X
    goes to the E2M1 grid (nearest, ties to the even code, saturating at 6). An all-zero
    group gets scale byte 127 and zero codes. Codes 2m and 2m+1 share byte m, low nibble
    first. Returns (codes uint8 [..., 64], scales uint8 [..., 4]).
    """
    x = x.float()
    g = x.reshape(*x.shape[:-1], x.shape[-1] // 32, 32)
    amax = g.abs().amax(dim=-1)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2
    code_s = torch.where(amax > 0, e + 127, torch.full_like(e, 127.0)).clamp(1, 254)
    scale = torch.exp2(code_s - 127)
    code = _e2m1_codes(g / scale.unsqueeze(-1)).reshape(x.shape)
    codes = code[..., 0::2] | (code[..., 1::2] << 4)
    return codes.contiguous(), code_s.to(torch.uint8).contiguous()


# ----------------------------------------------------------------------------- random draws

def _seed(seed: int, *names) -> int:
    h = hashlib.sha256(repr((seed,) + tuple(names)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed, *names) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, *names))
    return g


def _randn(shape, device, seed, *names):
    return torch.randn(shape, generator=_gen(device, seed, *names), device=device,
                       dtype=torch.float32)


def _rand(shape, device, seed, *names):
    return torch.rand(shape, generator=_gen(device, seed, *names), device=device,
                      dtype=torch.float32)


def _unit(v: torch.Tensor) -> torch.Tensor:
    return v / v.norm().clamp_min(1e-30)


def _make_layer(mode, n_q, device, seed, li, window_rows=None, swa_start=None, n_swa=None):
    q = to_bf16(_randn((n_q, N_HEADS, HEAD_DIM), device, seed, "q_main", li))
    if window_rows is None:
        window_rows = n_q * WINDOW
        swa_start = torch.arange(n_q, dtype=torch.int64, device=device) * WINDOW
        n_swa = torch.full((n_q,), WINDOW, dtype=torch.int32, device=device)
    window_kv = encode_e4m3(_randn((window_rows, HEAD_DIM), device, seed, "swa", li))
    layer = LayerInputs(mode=mode, q=q, window_kv=window_kv, swa_start=swa_start, n_swa=n_swa)
    if mode in ("full", "reindex"):
        layer.q_idx = to_bf16(_randn((n_q, IDX_HEADS, IDX_DIM), device, seed, "q_idx", li))
        layer.w = _rand((n_q, IDX_HEADS), device, seed, "w_idx", li)
    return layer


def _fill_sequences(n_q, n_ctx, kv_start, n_visible, n_entries, device, seed, plant_pos,
                    full_layer: LayerInputs, mxfp4=False, tag=(), plant_re=None,
                    reindex_layer: LayerInputs | None = None):
    """Draw the indexer-K and latent rows of every sequence, planting at plant_pos (indexer
    key along the Full layer's weighted indexer query, latent along its summed main query)
    and at plant_re (indexer key only, along the Reindex layer's weighted indexer query).
    With mxfp4 the indexer keys are also encoded in MXFP4 (from the same draws). `tag`
    extends the draw names (a second cache set of the same sequences)."""
    k_cache = torch.zeros((n_entries, IDX_DIM), dtype=torch.uint8, device=device)
    k_codes = torch.zeros((n_entries, IDX_DIM // 2), dtype=torch.uint8, device=device) if mxfp4 else None
    k_scales = torch.full((n_entries, IDX_DIM // 32), 127, dtype=torch.uint8, device=device) if mxfp4 else None
    kv_fp4 = torch.zeros((n_entries, HEAD_DIM // 2), dtype=torch.uint8, device=device)
    kv_scale = torch.zeros((n_entries, HEAD_DIM // 16), dtype=torch.uint8, device=device)
    starts = kv_start.tolist()
    counts = n_visible.tolist()
    shared = len(set(starts)) == 1 and n_q > 1
    seqs = [(0, starts[0], max(counts))] if shared else list(zip(range(n_q), starts, counts))
    for t, start, n in seqs:
        if n <= 0:
            continue
        k = _randn((n, IDX_DIM), device, seed, "k_idx", t, *tag)
        lat = _randn((n, HEAD_DIM), device, seed, "latent", t, *tag)
        if plant_pos is not None and not shared:
            pos = plant_pos[t]
            pos = pos[pos < n]
            qi = full_layer.q_idx[t].float()
            u = _unit((full_layer.w[t].float()[:, None] * qi).sum(0))
            v = _unit(full_layer.q[t].float().sum(0))
            k[pos] += PLANT_SHIFT * u
            lat[pos] += PLANT_SHIFT * v
        if plant_re is not None and not shared:
            pos = plant_re[t]
            pos = pos[pos < n]
            qi = reindex_layer.q_idx[t].float()
            k[pos] += PLANT_SHIFT * _unit((reindex_layer.w[t].float()[:, None] * qi).sum(0))
        k_cache[start:start + n] = encode_e4m3(k)
        if mxfp4:
            kc, ks = encode_mxfp4_rows(k)
            k_codes[start:start + n] = kc
            k_scales[start:start + n] = ks
        p, s = encode_fp4_rows(lat)
        kv_fp4[start:start + n] = p
        kv_scale[start:start + n] = s
    return k_cache, kv_fp4, kv_scale, k_codes, k_scales


def make_decode(name, n_q, n_ctx, layers, with_pool, n_plant, needles="random",
                device="cpu", seed=0, n_visible=None, kv_gap=0, mxfp4=False):
    """Decode batch: every query owns a sequence of n_visible[t] entries (default n_ctx),
    laid out one after the other with kv_gap spare rows between them."""
    if n_visible is None:
        n_visible = [n_ctx] * n_q
    n_visible_t = torch.tensor(n_visible, dtype=torch.int32)
    stride = [int(v) + kv_gap for v in n_visible]
    starts = [0]
    for s in stride[:-1]:
        starts.append(starts[-1] + s)
    n_entries = max(1, starts[-1] + stride[-1]) if n_q else 1
    kv_start_t = torch.tensor(starts[:n_q], dtype=torch.int64)
    lay = [_make_layer(m, n_q, device, seed, li) for li, m in enumerate(layers)]
    planted = None
    planted_re = None
    li_re = next((i for i, m in enumerate(layers) if m == "reindex"), None)
    if n_plant > 0 and n_q > 0 and li_re is not None:
        rows = []
        for t in range(n_q):
            n = max(0, int(n_visible[t]))
            g = _gen("cpu", seed, "plant_re", t)
            r = torch.randperm(max(n, 1), generator=g)[:n_plant].sort().values
            rows.append(torch.cat([r, r.new_full((n_plant - r.numel(),), 0)]) if r.numel() < n_plant else r)
        planted_re = torch.stack(rows)
    if n_plant > 0 and n_q > 0:
        rows = []
        for t in range(n_q):
            n = int(n_visible[t])
            if n <= 0:
                rows.append(torch.zeros(n_plant, dtype=torch.int64))
                continue
            if needles == "even":
                i = torch.arange(n_plant, dtype=torch.float64)
                rows.append(((i + 0.5) * n / n_plant).floor().to(torch.int64))
            else:
                g = _gen("cpu", seed, "plant", t)
                rows.append(torch.randperm(n, generator=g)[:n_plant].sort().values)
        planted = torch.stack([r[:n_plant] if r.numel() >= n_plant else
                               torch.cat([r, r.new_full((n_plant - r.numel(),), 0)]) for r in rows])
    k_cache, kv_fp4, kv_scale, k_codes, k_scales = _fill_sequences(
        n_q, n_ctx, kv_start_t, n_visible_t, n_entries, device, seed,
        None if planted is None else planted.to(device), lay[0], mxfp4=mxfp4,
        plant_re=None if planted_re is None else planted_re.to(device),
        reindex_layer=None if li_re is None else lay[li_re])
    return Workload(name=name, n_q=n_q, n_ctx=max(n_visible) if n_q else 0,
                    kv_start=kv_start_t.to(device), n_visible=n_visible_t.to(device),
                    k_cache=k_cache, kv_fp4=kv_fp4, kv_scale=kv_scale, layers=lay,
                    with_pool=with_pool, planted=planted, planted_re=planted_re,
                    k_codes=k_codes, k_scales=k_scales)


def make_prefill(name="prefill_128k_m2", n_q=4096, n_entries=131072, ratio=2,
                 device="cpu", seed=0):
    """Chunked prefill: the last n_q source tokens of a sequence of ratio*n_entries tokens
    query one shared cache; query i sits at token p = ratio*n_entries - n_q + i and sees
    the entries whose source tokens are all at or before p: n_visible = (p+1)//ratio.
    SWA: a buffer of n_q + 127 rows, query i reads rows i .. i+127."""
    p0 = ratio * n_entries - n_q
    n_visible = [(p0 + i + 1) // ratio for i in range(n_q)]
    n_visible_t = torch.tensor(n_visible, dtype=torch.int32)
    kv_start_t = torch.zeros(n_q, dtype=torch.int64)
    rows = n_q + WINDOW - 1
    swa_start = torch.arange(n_q, dtype=torch.int64, device=device)
    n_swa = torch.full((n_q,), WINDOW, dtype=torch.int32, device=device)
    lay = [_make_layer("full", n_q, device, seed, 0, rows, swa_start, n_swa)]
    k_cache, kv_fp4, kv_scale, _, _ = _fill_sequences(
        n_q, n_entries, kv_start_t, n_visible_t, n_entries, device, seed, None, lay[0])
    return Workload(name=name, n_q=n_q, n_ctx=max(n_visible), kv_start=kv_start_t.to(device),
                    n_visible=n_visible_t.to(device), k_cache=k_cache, kv_fp4=kv_fp4,
                    kv_scale=kv_scale, layers=lay, with_pool=False, planted=None,
                    shared_start=0)


def make_encoder(name="encoder_128k_m2", n_q=4096, n_entries=131072, ratio=2,
                 device="cpu", seed=0):
    """The causal encoder's layer schedule over the same chunk as make_prefill: two SWA-only
    layers, then three groups of (Full, 5 x Reuse). Each group's Full layer computes its
    own main KV and indexer K, so group g reads cache set g (group 0: the workload's own
    tensors, the same cache rows as make_prefill draws); its Reuse layers attend with that
    Full layer's Top-K over the same cache set."""
    p0 = ratio * n_entries - n_q
    n_visible = [(p0 + i + 1) // ratio for i in range(n_q)]
    n_visible_t = torch.tensor(n_visible, dtype=torch.int32)
    kv_start_t = torch.zeros(n_q, dtype=torch.int64)
    rows = n_q + WINDOW - 1
    swa_start = torch.arange(n_q, dtype=torch.int64, device=device)
    n_swa = torch.full((n_q,), WINDOW, dtype=torch.int32, device=device)
    lay = []
    group = -1
    for li, mode in enumerate(ENCODER_LAYERS):
        l = _make_layer(mode, n_q, device, seed, li, rows, swa_start, n_swa)
        if mode == "full":
            group += 1
        l.group = max(group, 0)
        lay.append(l)
    caches = []
    for g in range(group + 1):
        k_cache, kv_fp4, kv_scale, _, _ = _fill_sequences(
            n_q, n_entries, kv_start_t, n_visible_t, n_entries, device, seed, None, lay[0],
            tag=() if g == 0 else ("group", g))
        caches.append((k_cache, kv_fp4, kv_scale))
    k_cache, kv_fp4, kv_scale = caches[0]
    return Workload(name=name, n_q=n_q, n_ctx=max(n_visible), kv_start=kv_start_t.to(device),
                    n_visible=n_visible_t.to(device), k_cache=k_cache, kv_fp4=kv_fp4,
                    kv_scale=kv_scale, layers=lay, with_pool=False, planted=None,
                    shared_start=0, group_caches=caches[1:])


def make_workload(name: str, device="cpu", seed=0, n_q=None) -> Workload:
    """One of the named workloads; n_q (optional) keeps only the first n_q queries. A
    decode workload name with the suffix "_mxfp4" also carries MXFP4 indexer keys, which
    its indexer passes then read instead of the E4M3 ones; a further suffix "_q8" (on a
    decode workload, E4M3 or MXFP4 keys) makes those passes quantise the indexer query to
    MXFP8."""
    if name.endswith("_q8"):
        wl = make_workload(name[:-3], device=device, seed=seed, n_q=n_q)
        wl.name, wl.q8 = name, True
        return wl
    if name.endswith("_mxfp4") and name[:-6] in ("tiny_decode_4k", "decode_32k", "decode_256k",
                                                 "decode_1m"):
        base = name[:-6]
        args = {"tiny_decode_4k": (n_q or 1, 4096, ("full",), False, 16, "random"),
                "decode_32k": (n_q or 16, 32768, ("full",), False, 64, "random"),
                "decode_256k": (n_q or 32, 262144, DECODE_LAYERS, True, 64, "random"),
                "decode_1m": (n_q or 64, 1048576, DECODE_LAYERS, True, 64, "even")}[base]
        return make_decode(name, *args[:5], needles=args[5], device=device, seed=seed,
                           mxfp4=True)
    if name == "tiny_decode_4k":
        return make_decode(name, n_q or 1, 4096, ("full",), False, 16, device=device, seed=seed)
    if name == "decode_32k":
        return make_decode(name, n_q or 16, 32768, ("full",), False, 64, device=device, seed=seed)
    if name == "decode_256k":
        return make_decode(name, n_q or 32, 262144, DECODE_LAYERS, True, 64, device=device,
                           seed=seed)
    if name == "prefill_128k_m2":
        return make_prefill(name, n_q=n_q or 4096, device=device, seed=seed)
    if name == "encoder_128k_m2":
        return make_encoder(name, n_q=n_q or 4096, device=device, seed=seed)
    if name == "decode_1m":
        return make_decode(name, n_q or 64, 1048576, DECODE_LAYERS, True, 64, needles="even",
                           device=device, seed=seed)
    raise ValueError(f"unknown workload {name!r}")


WORKLOADS = ("tiny_decode_4k", "decode_32k", "decode_256k", "prefill_128k_m2", "decode_1m",
             "encoder_128k_m2")


def sequence_to_host(wl: Workload, t: int):
    """Host numpy copies of what query t reads: its rows of the caches (re-based so the
    sequence starts at row 0) and its inputs of every layer."""
    start = int(wl.kv_start[t])
    n = int(wl.n_visible[t])
    sl = slice(start, start + max(n, 0))
    seq = {
        "n_visible": n,
        "k_cache": wl.k_cache[sl].cpu().numpy(),
        "kv_fp4": wl.kv_fp4[sl].cpu().numpy(),
        "kv_scale": wl.kv_scale[sl].cpu().numpy(),
        "layers": [],
    }
    if wl.k_codes is not None:
        seq["k_codes"] = wl.k_codes[sl].cpu().numpy()
        seq["k_scales"] = wl.k_scales[sl].cpu().numpy()
    groups = [(seq["k_cache"], seq["kv_fp4"], seq["kv_scale"])]
    for kc, kf, ks in wl.group_caches:
        groups.append((kc[sl].cpu().numpy(), kf[sl].cpu().numpy(), ks[sl].cpu().numpy()))
    for lay in wl.layers:
        s0 = int(lay.swa_start[t])
        ns = int(lay.n_swa[t])
        kc, kf, ks = groups[lay.group]
        d = {
            "mode": lay.mode,
            "group": lay.group,
            "k_cache": kc,
            "kv_fp4": kf,
            "kv_scale": ks,
            "q": lay.q[t].view(torch.int16).cpu().numpy().view("uint16"),
            "window_kv": lay.window_kv[s0:s0 + max(0, min(ns, WINDOW))].cpu().numpy(),
            "n_swa": ns,
        }
        if lay.q_idx is not None:
            d["q_idx"] = lay.q_idx[t].view(torch.int16).cpu().numpy().view("uint16")
            d["w"] = lay.w[t].cpu().numpy()
        seq["layers"].append(d)
    return seq
