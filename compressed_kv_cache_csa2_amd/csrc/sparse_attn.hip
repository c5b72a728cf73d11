// Joint sparse attention over the selected FP4 latents and the FP8 sliding window, on
// gfx950 MFMA.
//
// For query t and head h over the attended set S (selected main entries, then SWA rows):
//     l_j = scale * q[t,h,:] . c_j,  p = softmax_S(l),  out[t,h,:] = sum_j p_j c_j
// with key = value = c_j ("DeepSeek-v4.1 Flash: Pushing the Limits of KV Cache
// Compression", 3.3.1-3.3.2: one softmax over the concatenation of the window and the
// selected entries; "DeepSeek-V4.1-Flash - Architecture", sections 2 and 4: 64 heads of
// dim 512, FP4 E2M1 main KV with an E4M3 scale per 16 channels, FP8 window).
//
// Work split: a query's selected entries and its window rows are cut into 16-item slices
// (separately, so a slice never mixes the two formats). A workgroup owns one group of 16
// heads and, with at most 32 queries (too few to fill the GPU otherwise), one half (256
// channels) of the output, else all of it; its eight wavefronts (two per SIMD, so one's
// memory waits hide behind the other's arithmetic) each take one of the window's eight
// slices and every eighth slice of the selected entries, and run independently (no
// barrier in the main loop). Both halves of a head group compute the same full-width
// logits and softmax, so each writes its own channels with no merge across workgroups,
// and each wavefront's accumulator is half as large as a full-width one, which leaves the
// registers for a second gather buffer. Per slice a wavefront:
//   - gathers the 16 rows (lane = item x quarter of the 512 channels). The window slice
//     needs no position, so its gather is issued first and it is processed first, while
//     the selected rows are in flight; those are gathered two slices ahead of their use,
//     alternating between two register buffers (one slice ahead, in one buffer, at full
//     width), with the selected positions loaded two slices before the gather. The
//     gathers are indexed buffer loads: an absent item gets an index past the buffer's
//     record count and reads zeros, so every slice of a kind issues the same loads into
//     the same registers and the wait for a slice never includes the loads behind it;
//   - converts them to fp16 with the hardware E2M1/E4M3 -> fp16 conversions and a packed
//     fp16 multiply by the group scale; every value is exact (an E2M1 x E4M3 product has
//     <= 6 significant bits in [2^-10, 2688]). The converted registers are directly the A
//     operand of the logit product S^T (16 items x 16 heads) = C . Q^T
//     (v_mfma_f32_16x16x32_f16, K = 512; B = this group's queries, each head rescaled by a
//     power of two into fp16's range with the inverse folded into the logit scale, held
//     once in LDS in operand order so every read is one contiguous 1 KiB access), and are
//     also stored to the wavefront's own LDS tile;
//   - never rescales its accumulator: the reference max of each head is the largest logit
//     of the first slice with a valid item, and later weights p = 2^(l - ref) may reach
//     2^15 (fp16 holds them); a logit beyond that restarts the wavefront's slices with the
//     raised reference (rare; the result does not depend on the reference);
//   - O^T (the workgroup's channels x 16 heads) += C^T . P^T with v_mfma_f32_16x16x16_f16:
//     P^T is the logits' accumulator layout, A = C^T is read from the tile with LDS
//     transpose reads (ds_read_b64_tr_b16).
// The eight wavefront partials are merged through LDS. Workgroup ids put all workgroups
// of a query on one XCD, so they share its L2 copy of the rows.
#include "csa2_device.h"
#include "csa2_launch.h"

#include <type_traits>

namespace csa2 {

constexpr int AT_WAVES = 8;
constexpr int AT_THREADS = 64 * AT_WAVES;
constexpr int AT_SLICE = 16;                 // items per wavefront step
constexpr int AT_HEADS = 16;                 // heads per workgroup
constexpr int AT_GROUPS = 64 / AT_HEADS;     // head groups per query
// Up to this many queries, a (query, head group) is served by two workgroups, one per
// output channel half (the grid would otherwise leave CUs idle); above it by one.
constexpr int AT_HALVES_MAX_Q = 32;
constexpr int AT_WINDOW = 128;               // largest sliding window
constexpr int AT_WIN_SLICES = AT_WINDOW / AT_SLICE;
constexpr int N_XCD = 8;
constexpr float AT_GAP = 15.f;               // largest log2 weight over the reference
constexpr float AT_LOG2E = 1.4426950408889634f;
constexpr float AT_LN2 = 0.6931471805599453f;

// A wavefront's tile holds 16 rows C[e][0..512) in fp16. Row e starts at element
// TILE_ROW * e and its channel quarter g (128 channels) at + TILE_QUARTER * g: rows are
// 1,120 B apart and quarters 272 B apart, which keeps the transpose reads (16 rows x one
// 32-byte chunk) free of bank conflicts, and every address is a per-lane base plus a
// compile-time offset.
constexpr int TILE_ROW = 560;       // elements
constexpr int TILE_QUARTER = 136;   // elements
constexpr int TILE_ELEMS = AT_SLICE * TILE_ROW;

struct AttnShared {
  union {
    uint16_t tile[AT_WAVES][TILE_ELEMS];   // 140 KiB: per-wave slice tiles
    u32x4 part[AT_WAVES][16][64];          // 128 KiB: merge buffer (half of d), lane order
  };
  u32x4 qop[16][64];                       // 16 KiB: logit B operand per k-step, lane order
  float qpart[AT_WAVES][AT_HEADS];         // per-wave partial |q| maxima
  float wm[AT_WAVES][AT_HEADS];
  float wl[AT_WAVES][AT_HEADS];
};

// Channel assignment: lane (item, g), g = lane / 16, holds channels 128i + 32g .. +31 for
// i = 0..3, and its block j (8 channels) is channels 128(j/4) + 32g + 8(j%4) .. +7. Each
// gather instruction then reads one contiguous 64-byte (FP4) or 128-byte (window) piece
// per row across the item's four lanes, instead of four pieces spread over the row.
//
// One slice's gathered bytes for one lane: 64 B of an FP4 row plus the row's 32 scale
// bytes (RawMain), or 128 B of a window row (RawWin). Absent items read as zeros.
struct RawMain {
  u32x4 v[4];    // v[i]: FP4 bytes 64i + 16g .. +15 = channels 128i + 32g .. +31
  u32x4 sc[2];   // the row's 32 E4M3 group scales
  bool valid;    // the item exists
};
struct RawWin {
  u32x4 v[8];    // v[2i + h]: E4M3 bytes 128i + 32g + 16h .. +15
  bool valid;
};

// Converts the lane's 16 blocks to fp16, stores those of the tile quarters the workgroup
// reads (quarters 0-1 if STORE_LO, 2-3 if STORE_HI) to the lane's place in the tile
// (tile_row + TILE_QUARTER * (j/4) + 8 * (j%4) for block j), and accumulates the logits
// against the query operand held in LDS. Format and stored quarters are template
// parameters: the caller branches once per slice (wavefront-uniform choices), so the 16
// blocks have no branch between them and the operand reads can be issued ahead of the
// products. g is the lane's channel group (lane / 16).
template <bool WINDOW, bool STORE_LO, bool STORE_HI, class R>
__device__ __forceinline__ f32x4 convert_and_score(const R& r, const u32x4 (*qop)[64],
                                                   int lane, int g, uint16_t* tile_row) {
  f16x2 sq[8];   // sq[m]: scale of blocks 2m, 2m+1 (group 8(m/2) + 2g + m%2), in both halves
  if constexpr (!WINDOW) {
    // Groups 8i + 2g and 8i + 2g + 1 are the 16-bit half (g % 2) of scale dword 2i + g/2.
    const int shift = 16 * (g & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (g & 2) ? r.sc[i >> 1][2 * (i & 1) + 1] : r.sc[i >> 1][2 * (i & 1)];
      const f16x2 s2 = e4m3x2_to_f16x2<false>(lo >> shift);
      sq[2 * i] = f16x2{s2.x, s2.x};
      sq[2 * i + 1] = f16x2{s2.y, s2.y};
    }
  }
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
  // The operand of block j + QLEAD is read while block j is converted and multiplied.
  constexpr int QLEAD = 2;
  u32x4 b[QLEAD + 1];
#pragma unroll
  for (int j = 0; j < QLEAD; ++j) b[j] = qop[j][lane];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j + QLEAD < 16) b[(j + QLEAD) % (QLEAD + 1)] = qop[j + QLEAD][lane];
    u32x4 a;
    if constexpr (WINDOW) {
      const u32x4& w = r.v[2 * (j >> 2) + ((j & 3) >> 1)];
      a = fp8x8_to_f16x8(w[2 * (j & 1)], w[2 * (j & 1) + 1]);
    } else {
      a = fp4x8_to_f16x8(r.v[j >> 2][j & 3], sq[j >> 1]);
    }
    if ((j < 8 && STORE_LO) || (j >= 8 && STORE_HI))
      *reinterpret_cast<u32x4*>(tile_row + TILE_QUARTER * (j >> 2) + 8 * (j & 3)) = a;
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b[j % (QLEAD + 1)]), sacc, 0,
        0, 0);
  }
  return sacc;
}

// HALVES = 2: the workgroup owns half of the output channels and keeps two gather buffers
// (its accumulator is half as large); HALVES = 1: all channels, one gather buffer.
template <int HALVES>
__global__ __launch_bounds__(AT_THREADS) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_fp4, int64_t fp4_stride,
    const uint8_t* __restrict__ kv_scale, int64_t sc_stride, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const int32_t* __restrict__ topk_idx, int64_t ld_idx,
    int k, const uint8_t* __restrict__ window_kv, int64_t n_win_rows,
    const int64_t* __restrict__ swa_start, const int32_t* __restrict__ n_swa, float scale,
    int n_q, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ AttnShared sh;

  // id = (g * J + j) * 8 + t % 8 for queries 8g .. 8g+7 and J = 4 head groups x 2 channel
  // halves workgroups per query: every workgroup of query t has id % 8 = t % 8.
  constexpr int DT = 32 / HALVES;     // 16-channel output tiles of this workgroup
  constexpr int NBUF = HALVES;        // gather buffers = slices of lead for a gather
  constexpr int J = AT_GROUPS * HALVES;
  const int id = blockIdx.x;
  const int t = (id / (N_XCD * J)) * N_XCD + id % N_XCD;
  if (t >= n_q) return;
  const int jj = (id / N_XCD) % J;
  const int hg = jj % AT_GROUPS;
  const int dh = jj / AT_GROUPS;   // output channels from 256*dh (0 with one workgroup)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: lets slice indices stay scalar
  const int col = lane & 15;   // head within the group; also the item a lane gathers
  const int gq = lane >> 4;    // lane group 0..3; also the channel quarter a lane gathers
  const int h = hg * AT_HEADS + col;

  // Slices: the selected entries (slice c < n_msl holds entries 16c .. 16c+15), taken by
  // wavefront c % 8, and the window's 8 slices, one per wavefront.
  static_assert(AT_WIN_SLICES == AT_WAVES, "one window slice per wavefront");
  const int n_msl = (k + AT_SLICE - 1) / AT_SLICE;
  const int c0 = wave;

  // Selected positions, through a buffer over this query's k entries: a slot past k (or
  // a slice past the last) reads 0 without touching memory and is marked absent.
  const __amdgpu_buffer_rsrc_t rs_idx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(topk_idx) + (int64_t)t * ld_idx, (short)0, k * 4, 0x00020000);
  // The value is used only when the gather is issued, which re-derives whether the slot
  // exists, so the load is never waited for early.
  auto position = [&](int c) -> int32_t {   // position of this lane's item of slice c
    const int item = AT_SLICE * c + col;
    const bool in = c < n_msl && item < k;
    return __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs_idx, in ? item * 4 : k * 4, 0, 0));
  };
  // p0 is the first slice's position; the next one (p1 with two buffers, else the first
  // look-ahead pX) is loaded up front as well.
  const int32_t p0 = position(c0);
  int32_t p1 = 0, pX = 0;
  if constexpr (NBUF == 2)
    p1 = position(c0 + AT_WAVES);
  else
    pX = position(c0 + AT_WAVES);

  // This wavefront's two k-steps of the logit B operand: Q^T for head h, the channels of
  // blocks j = 2*wave, 2*wave + 1 of channel group gq (the assignment of the gathers).
  const uint16_t* qrow = q + ((int64_t)t * 64 + h) * 512 + 32 * gq + 128 * (wave >> 1) +
                         16 * (wave & 1);
  const u32x4 qr0 = *reinterpret_cast<const u32x4*>(qrow);
  const u32x4 qr1 = *reinterpret_cast<const u32x4*>(qrow + 8);

  // The per-query scalars come through vector loads issued beside the query and position
  // loads, so their latency overlaps with those; as scalar loads they would be waited for
  // at the first barrier, which also drains the scalar-load counter.
  int nsw, base_lo, base_hi, wbase_lo, wbase_hi;
  {
    const __amdgpu_buffer_rsrc_t rs_ks = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int64_t*>(kv_start) + t, (short)0, 8, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_ws = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int64_t*>(swa_start) + t, (short)0, 8, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_ns = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(n_swa) + t, (short)0, 4, 0x00020000);
    base_lo = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(rs_ks, 0, 0, 0));
    base_hi = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(rs_ks, 4, 0, 0));
    wbase_lo = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(rs_ws, 0, 0, 0));
    wbase_hi = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(rs_ws, 4, 0, 0));
    nsw = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(rs_ns, 0, 0, 0));
  }

  // Query scale: per head, the largest |q| over its 512 channels (spread over the eight
  // wavefronts' k-steps), then a power of two that brings it to [2^14, 2^15).
  float qm = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qm = fmaxf(qm, fabsf(__uint_as_float(qr0[i] << 16)));
    qm = fmaxf(qm, fabsf(__uint_as_float(qr0[i] & 0xFFFF0000u)));
    qm = fmaxf(qm, fabsf(__uint_as_float(qr1[i] << 16)));
    qm = fmaxf(qm, fabsf(__uint_as_float(qr1[i] & 0xFFFF0000u)));
  }
  qm = fmaxf(qm, __shfl_xor(qm, 16));
  qm = fmaxf(qm, __shfl_xor(qm, 32));
  if (gq == 0) sh.qpart[wave][col] = qm;
  __syncthreads();
  float qmax = 0.f;
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) qmax = fmaxf(qmax, sh.qpart[w][col]);
  nsw = __builtin_amdgcn_readfirstlane(nsw);
  nsw = nsw < 0 ? 0 : (nsw > AT_WINDOW ? AT_WINDOW : nsw);
  const int64_t base = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(base_hi) << 32) |
                                 (uint32_t)__builtin_amdgcn_readfirstlane(base_lo));
  const int64_t wbase = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(wbase_hi) << 32) |
                                  (uint32_t)__builtin_amdgcn_readfirstlane(wbase_lo));
  // Gather: lane (item col of slice c, quarter gq) -> channels 128*gq .. +127 of that item.
  // The buffers are indexed by row relative to the query's own base, so the 32-bit record
  // index covers any sequence; absent items use an index past every record count.
  constexpr uint32_t ABSENT = 0xFFFFFFFFu;
  const int64_t kv_rows = n_entries - base;
  const int64_t win_rows = n_win_rows - wbase;
  const uint32_t kv_n = kv_rows <= 0 ? 0u : (kv_rows >= (int64_t)ABSENT ? ABSENT - 1u : (uint32_t)kv_rows);
  const uint32_t win_n = win_rows <= 0 ? 0u : (win_rows >= (int64_t)ABSENT ? ABSENT - 1u : (uint32_t)win_rows);
  const __amdgpu_buffer_rsrc_t rs_kv = make_rows_rsrc(kv_fp4 + base * fp4_stride, (int)fp4_stride, kv_n);
  const __amdgpu_buffer_rsrc_t rs_sc = make_rows_rsrc(kv_scale + base * sc_stride, (int)sc_stride, kv_n);
  const __amdgpu_buffer_rsrc_t rs_win = make_rows_rsrc(window_kv + wbase * 512, 512, win_n);
  auto fetch_main = [&](int c, int32_t p, RawMain& raw) {
    const int item = AT_SLICE * c + col;
    const int64_t row = base + p;
    const bool ok = c < n_msl && item < k && p >= 0 && row >= 0 && row < n_entries;
    raw.valid = ok;
    const int ridx = ok ? p : (int)ABSENT;
#pragma unroll
    for (int i = 0; i < 4; ++i) raw.v[i] = sbuf_load_b128(rs_kv, ridx, 64 * i + 16 * gq, 0, 0);
    raw.sc[0] = sbuf_load_b128(rs_sc, ridx, 0, 0, 0);
    raw.sc[1] = sbuf_load_b128(rs_sc, ridx, 16, 0, 0);
  };
  // Window slice w (rows 16w .. 16w+15 of the query's window) belongs to wavefront w.
  auto fetch_win = [&](RawWin& raw) {
    const int wi = AT_SLICE * wave + col;
    const int64_t wr = wbase + wi;
    const bool ok = wi < nsw && wr >= 0 && wr < n_win_rows;
    raw.valid = ok;
    const int ridx = ok ? wi : (int)ABSENT;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      raw.v[i] = sbuf_load_b128(rs_win, ridx, 128 * (i >> 1) + 32 * gq + 16 * (i & 1), 0, 0);
  };

  const int qexp = qmax > 0.f ? (int)((__float_as_uint(qmax) >> 23) & 0xFFu) - 127 : 0;
  int kexp = 14 - qexp;
  kexp = kexp < -126 ? -126 : (kexp > 126 ? 126 : kexp);
  const float up = __uint_as_float((uint32_t)(127 + kexp) << 23);
  // logits in log2 units: l2 = acc * scale * 2^-kexp * log2(e)
  const float lscale = scale * AT_LOG2E * __uint_as_float((uint32_t)(127 - kexp) << 23);
  {
    f16x8 b0, b1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b0[2 * i] = (_Float16)(__uint_as_float(qr0[i] << 16) * up);
      b0[2 * i + 1] = (_Float16)(__uint_as_float(qr0[i] & 0xFFFF0000u) * up);
      b1[2 * i] = (_Float16)(__uint_as_float(qr1[i] << 16) * up);
      b1[2 * i + 1] = (_Float16)(__uint_as_float(qr1[i] & 0xFFFF0000u) * up);
    }
    sh.qop[2 * wave][lane] = __builtin_bit_cast(u32x4, b0);
    sh.qop[2 * wave + 1][lane] = __builtin_bit_cast(u32x4, b1);
  }
  // The window slice is gathered first and processed first: its rows need no position
  // load, so they arrive while the selected rows are still in flight. NBUF main buffers: a
  // slice's rows are requested NBUF steps before their use (with one buffer, the first
  // main gather starts once the window slice is converted). Each gather is followed by
  // the position load of the slice NBUF steps after it, in the same order as in the loop.
  RawWin rw;
  RawMain bufs[NBUF];
  RawMain& bufA = bufs[0];          // buffer of the even steps
  RawMain& bufS = bufs[NBUF - 1];   // buffer of the odd steps
  fetch_win(rw);
  if constexpr (NBUF == 2) {
    fetch_main(c0, p0, bufA);
    pX = position(c0 + 2 * AT_WAVES);
    fetch_main(c0 + AT_WAVES, p1, bufS);
  }
  int32_t pY = position(c0 + (NBUF + 1) * AT_WAVES);
  __syncthreads();   // the query operand is complete

  // Output accumulator: O^T[d = 256*dh + 16*dt + 4*gq + i][h], dt = 0..DT-1.
  f32x4 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();   // reference max of head col (log2 units)
  bool ok_pass = true;               // no logit of this pass overflowed the reference
  float l_run = 0.f;                 // this lane's share of the sum for head col
  uint16_t* const tile = sh.tile[wave];
  uint16_t* const tile_w = tile + TILE_ROW * col + 32 * gq;
  // Transpose reads start at this workgroup's first channel quarter (2*dh).
  const uint16_t* const tile_r =
      tile + TILE_ROW * (4 * gq + (col >> 2)) + 4 * (col & 3) + TILE_QUARTER * (2 * dh);

  // The softmax and PV part of a slice with at least one valid item. A logit exceeding
  // the reference by more than AT_GAP raises the reference and marks the pass for a repeat.
  auto finish = [&](uint64_t valid, f32x4 sacc) {
    // LDS operations of one wavefront complete in order; the fences keep the compiler from
    // moving the tile reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // Logits S^T[e][h]: lane holds items 4*gq + i of head col.
    float lg[4];
    bool over = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lg[i] = ((valid >> (4 * gq + i)) & 1ull) ? sacc[i] * lscale : -__builtin_inff();
      over |= lg[i] > m_ref + AT_GAP;
    }
    if (__ballot(over) != 0ull) {
      float cm = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
      cm = fmaxf(cm, __shfl_xor(cm, 16));
      cm = fmaxf(cm, __shfl_xor(cm, 32));
      // Validity is per item, so every head meets its first valid item in the same slice
      // and the test below is wavefront-uniform.
      const bool first = m_ref == -__builtin_inff();
      m_ref = fmaxf(m_ref, cm);   // finite: the slice has a valid item
      ok_pass = ok_pass && first;
    }
    f16x4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = lg[i] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(lg[i] - m_ref);
      l_run += pe;
      pv[i] = (_Float16)pe;
    }
    // O^T[d][h] += sum_e C^T[d][e] P^T[e][h], K = the slice's 16 items; lane group gq
    // carries items 4*gq .. 4*gq+3 in both operands. A comes from transpose reads: lane i
    // of a 16-lane group addresses channels 16*dt + 4*(i%4) .. +3 of item 4*gq + i/4 and
    // receives channel 16*dt + i of items 4*gq .. 4*gq+3.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x2 a = lds_read_tr16x4(tile_r + TILE_QUARTER * (dt >> 3) + 16 * (dt & 7));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), pv,
                                                       oacc[dt], 0, 0, 0);
    }
  };

  // A main slice (c may lie past the last: its items are all absent); pn is the position
  // of the slice NBUF steps later in this wavefront's sequence (c + NBUF*AT_WAVES), whose
  // gather starts as soon as this slice's registers are free. A slice with no item
  // converts nothing; only its next gather starts.
  // Conversion and logits of a slice, storing only the tile quarters this workgroup reads.
  auto convert_stored = [&](auto window, const auto& raw) -> f32x4 {
    constexpr bool W = decltype(window)::value;
    if constexpr (HALVES == 1)
      return convert_and_score<W, true, true>(raw, sh.qop, lane, gq, tile_w);
    else if (dh == 0)
      return convert_and_score<W, true, false>(raw, sh.qop, lane, gq, tile_w);
    else
      return convert_and_score<W, false, true>(raw, sh.qop, lane, gq, tile_w);
  };
  auto step_main = [&](int c, RawMain& raw, int32_t pn) {
    const uint64_t valid = __ballot(raw.valid);   // bit e: item e of the slice is present
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    if (valid != 0ull) sacc = convert_stored(std::false_type{}, raw);
    fetch_main(c + NBUF * AT_WAVES, pn, raw);
    if (valid != 0ull) finish(valid, sacc);
  };
  auto step_win = [&]() {
    const uint64_t valid = __ballot(rw.valid);
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    if (valid != 0ull) sacc = convert_stored(std::true_type{}, rw);
    if constexpr (NBUF == 1) fetch_main(c0, p0, bufA);
    if (valid != 0ull) finish(valid, sacc);
  };

  // Every step runs unconditionally (a slice past the last is all absent and its loads
  // return zeros without touching memory), so each buffer is written by the same loads on
  // every path and a step waits only for its own slice. With two buffers the steps
  // alternate between them; positions are loaded two steps before their gather, pX and pY
  // alternating so that no register is copied.
  bool again;
#pragma unroll 1
  do {
    ok_pass = true;
    step_win();
#pragma unroll 1
    for (int c = c0; c < n_msl; c += 2 * AT_WAVES) {
      step_main(c, bufA, pX);
      pX = position(c + (NBUF + 2) * AT_WAVES);
      step_main(c + AT_WAVES, bufS, pY);
      pY = position(c + (NBUF + 3) * AT_WAVES);
    }
    again = !ok_pass;
    if (again) {   // a logit overflowed the reference: repeat with the raised one
#pragma unroll
      for (int i = 0; i < DT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run = 0.f;
      fetch_win(rw);
      if constexpr (NBUF == 2) fetch_main(c0, p0, bufA);
      pX = position(c0 + NBUF * AT_WAVES);
      if constexpr (NBUF == 2) fetch_main(c0 + AT_WAVES, p1, bufS);
      pY = position(c0 + (NBUF + 1) * AT_WAVES);
    }
  } while (again);

  // Merge the eight wavefronts: O = sum_w 2^{m_w - M} O_w, L = sum_w 2^{m_w - M} l_w.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (gq == 0) {
    sh.wm[wave][col] = m_ref;
    sh.wl[wave][col] = l_run;
  }
  __syncthreads();   // also ends every wavefront's use of its tile
  // In passes of 16 tiles (one with two halves, two with one workgroup), thread tid
  // reduces the entries (dt = tid/64 and 8 + tid/64, lane l = tid%64) of every wavefront's
  // accumulator: O^T[256*(dh + pass) + 16*dt + 4*(l/16) + i][head l%16], so its head is
  // tid%16 throughout.
  const int oh = tid & 15;
  float fwh[AT_WAVES];
  float Mh = -__builtin_inff();
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) Mh = fmaxf(Mh, sh.wm[w][oh]);
  float Lh = 0.f;
#pragma unroll
  for (int w = 0; w < AT_WAVES; ++w) {
    const float mw = sh.wm[w][oh];
    fwh[w] = mw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mw - Mh);
    Lh += fwh[w] * sh.wl[w][oh];
  }
  const int rl = tid & 63;
  const int rdt = tid >> 6;
  constexpr int NPASS = DT / 16;
  f32x4 acc[NPASS][2];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      sh.part[wave][dt][lane] = __builtin_bit_cast(u32x4, oacc[16 * ps + dt]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 a = __builtin_bit_cast(f32x4, sh.part[0][rdt + 8 * j][rl]) * fwh[0];
#pragma unroll
      for (int w = 1; w < AT_WAVES; ++w)
        a += __builtin_bit_cast(f32x4, sh.part[w][rdt + 8 * j][rl]) * fwh[w];
      acc[ps][j] = a;
    }
    // Before the buffer is written again; also after the last pass, which keeps the
    // compiler from overlapping the passes (that runs the full-width variant out of
    // registers).
    __syncthreads();
  }

  // Two halves compute the same logits, so their maxima and sums agree; each writes its
  // own channels, and the first the log-sum-exp.
  const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
  uint16_t* orow = out + ((int64_t)t * 64 + hg * AT_HEADS + oh) * 512;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 a = acc[ps][j];
      const uint32_t b0 = f32_to_bf16_rne(a[0] * inv), b1 = f32_to_bf16_rne(a[1] * inv);
      const uint32_t b2 = f32_to_bf16_rne(a[2] * inv), b3 = f32_to_bf16_rne(a[3] * inv);
      const int ch = 256 * (dh + ps) + 16 * (rdt + 8 * j) + 4 * (rl >> 4);
      *reinterpret_cast<u32x2*>(orow + ch) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
  if (lse != nullptr && dh == 0 && tid < 16)
    lse[(int64_t)t * 64 + hg * AT_HEADS + oh] =
        Lh > 0.f ? (Mh + __log2f(Lh)) * AT_LN2 : -__builtin_inff();
}

// --------------------------------------------------------------------------------------
// Many queries (chunked prefill, the encoder): one workgroup per query covering all 64 heads,
// so each attended row is gathered and converted once instead of once per head group.
// Items go in slices of 32 (the window's slices first, then the selected entries'); per
// slice:
//   - wavefront w gathers items 4w .. 4w+3 (lane (item, p): channels 32p .. 32p+31) and
//     stores them converted to fp16 (exact, as above) in an LDS tile, one 1,056-byte row
//     per item, its 16-byte pieces permuted (ah_off) so that these stores, the row reads of
//     the logit product and the transposed reads of the value product are free of bank
//     conflicts; barrier;
//   - wavefront (head tile w % 4, item half w / 4) computes S (16 items x 16 heads) with
//     v_mfma_f32_16x16x32_f16 (A = tile rows, B = its heads' queries, held in registers),
//     turns it into weights p = 2^(l - ref) with a per-head reference ref and stores them,
//     already in the value product's B layout, to LDS; barrier;
//   - wavefront w accumulates O^T for output channels 64w .. 64w+63 of all 64 heads over the
//     slice's 32 items with v_mfma_f32_16x16x32_f16 (A = the tile read transposed, B = p),
//     so no partial outputs are merged at the end.
// The reference of a head is the largest logit of the first slice with a valid item (the
// two item halves combine through LDS once); a later logit more than 15 above it (fp16
// weights stay below 2^15) marks the pass, which is repeated with every head's largest
// logit as the reference (rare; the result does not depend on the reference).
constexpr int AH_WAVES = 8;
constexpr int AH_THREADS = 64 * AH_WAVES;
constexpr int AH_SLICE = 32;
constexpr int AH_ROW = 528;        // fp16 elements per tile row (1,056 bytes)
constexpr int AH_MIN_Q = 256;      // from this many queries on, this kernel runs

struct AttnHeadsShared {
  uint16_t tile[2][AH_SLICE * AH_ROW];   // 2 x 33 KiB: converted rows of a slice
  u32x2 pw[2][4][2][64];                 // weights: buffer, head tile, item half, lane
  uint32_t valid[2][AH_SLICE];           // item validity of a slice
  float xch[2][64];                      // per item half and head: maxima or sums
  int flag;                              // a logit overflowed the reference
};

// Element offset of channel ch (a multiple of 4) of tile row r. Rows are 1,056 bytes apart
// (8 dwords past a multiple of 32 banks) and the 16-byte pieces of a row are permuted,
// piece p of row r at p ^ ((p / 8) % 4) ^ ((r / 4) % 2). Then the conversion's stores (16
// lanes of a row write pieces 4g + j, g = 0..15), the logit operand reads (8 rows, one
// piece each) and the transpose reads (two adjacent pieces of 4 rows) each reach 32
// distinct banks per group of lanes served together.
__device__ __forceinline__ int ah_off(int r, int ch) {
  const int p = ch >> 3;
  return r * AH_ROW + ((p ^ ((p >> 3) & 3) ^ ((r >> 2) & 1)) << 3) + (ch & 7);
}

__global__ __launch_bounds__(AH_THREADS) void sparse_attn_heads_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_fp4, int64_t fp4_stride,
    const uint8_t* __restrict__ kv_scale, int64_t sc_stride, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const int32_t* __restrict__ topk_idx, int64_t ld_idx,
    int k, const uint8_t* __restrict__ window_kv, int64_t n_win_rows,
    const int64_t* __restrict__ swa_start, const int32_t* __restrict__ n_swa, float scale,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ AttnHeadsShared sh;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gcol = lane & 15;      // head within a tile (logits); row of an item (tile reads)
  const int grp = lane >> 4;       // lane group
  const int ht = wave & 3;         // logit role: head tile
  const int ih = wave >> 2;        //             item half
  const int h = 16 * ht + gcol;    // this lane's head in the logit role

  // Per-query scalars through buffer loads (issued with the query loads).
  const int64_t base = kv_start[t];
  const int64_t wbase = swa_start[t];
  int nsw = n_swa[t];
  nsw = nsw < 0 ? 0 : (nsw > AT_WINDOW ? AT_WINDOW : nsw);

  // Query operand: head h, k-step ks covers channels 32ks + 8grp .. +7 (16 bytes per lane).
  const uint16_t* qh = q + ((int64_t)t * 64 + h) * 512 + 8 * grp;
  u32x4 qraw[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(qh + 32 * ks);
  float qm = 0.f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qm = fmaxf(qm, fabsf(__uint_as_float(qraw[ks][i] << 16)));
      qm = fmaxf(qm, fabsf(__uint_as_float(qraw[ks][i] & 0xFFFF0000u)));
    }
  qm = fmaxf(qm, __shfl_xor(qm, 16));
  qm = fmaxf(qm, __shfl_xor(qm, 32));
  const int qexp = qm > 0.f ? (int)((__float_as_uint(qm) >> 23) & 0xFFu) - 127 : 0;
  int kexp = 14 - qexp;
  kexp = kexp < -126 ? -126 : (kexp > 126 ? 126 : kexp);
  const float up = __uint_as_float((uint32_t)(127 + kexp) << 23);
  const float lscale = scale * AT_LOG2E * __uint_as_float((uint32_t)(127 - kexp) << 23);
  f16x8 qop[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qop[ks][2 * i] = (_Float16)(__uint_as_float(qraw[ks][i] << 16) * up);
      qop[ks][2 * i + 1] = (_Float16)(__uint_as_float(qraw[ks][i] & 0xFFFF0000u) * up);
    }

  // Slices: n_wsl window slices, then n_msl slices of selected entries.
  const int n_wsl = (nsw + AH_SLICE - 1) / AH_SLICE;
  const int n_msl = (k + AH_SLICE - 1) / AH_SLICE;
  const int n_sl = n_wsl + n_msl;
  // Gather role: item it of a slice, channels 32 * gcol .. +31.
  const int it = 4 * wave + grp;
  constexpr uint32_t ABSENT = 0xFFFFFFFFu;
  const int64_t kv_rows = n_entries - base;
  const int64_t win_rows = n_win_rows - wbase;
  const uint32_t kv_n = kv_rows <= 0 ? 0u : (kv_rows >= (int64_t)ABSENT ? ABSENT - 1u : (uint32_t)kv_rows);
  const uint32_t win_n = win_rows <= 0 ? 0u : (win_rows >= (int64_t)ABSENT ? ABSENT - 1u : (uint32_t)win_rows);
  const __amdgpu_buffer_rsrc_t rs_kv = make_rows_rsrc(kv_fp4 + base * fp4_stride, (int)fp4_stride, kv_n);
  const __amdgpu_buffer_rsrc_t rs_sc = make_rows_rsrc(kv_scale + base * sc_stride, (int)sc_stride, kv_n);
  const __amdgpu_buffer_rsrc_t rs_win = make_rows_rsrc(window_kv + wbase * 512, 512, win_n);
  const __amdgpu_buffer_rsrc_t rs_idx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(topk_idx) + (int64_t)t * ld_idx, (short)0, k * 4, 0x00020000);
  // Position of this lane's item in slice s (main slices only; k reads as absent).
  auto position = [&](int s) -> int32_t {
    const int gi = AH_SLICE * (s - n_wsl) + it;
    const bool in = s >= n_wsl && s < n_sl && gi < k;
    return __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(
                                           rs_idx, in ? gi * 4 : k * 4, 0, 0));
  };
  struct Raw {
    u32x4 v0, v1;      // window: 32 E4M3 bytes; main: v0 = 16 bytes of E2M1 codes
    uint32_t sc;       // main: the scale dword holding groups 2*gcol, 2*gcol + 1
    bool ok;
  };
  auto fetch = [&](int s, int32_t pos, Raw& r) {
    if (s < n_wsl) {
      const int wi = AH_SLICE * s + it;
      r.ok = wi < nsw && wbase + wi >= 0 && wbase + wi < n_win_rows;
      const int idx = r.ok ? wi : (int)ABSENT;
      r.v0 = sbuf_load_b128(rs_win, idx, 32 * gcol, 0, 0);
      r.v1 = sbuf_load_b128(rs_win, idx, 32 * gcol + 16, 0, 0);
      r.sc = 0u;
    } else {
      const int gi = AH_SLICE * (s - n_wsl) + it;
      r.ok = s < n_sl && gi < k && pos >= 0 && base + pos < n_entries && base + pos >= 0;
      const int idx = r.ok ? pos : (int)ABSENT;
      r.v0 = sbuf_load_b128(rs_kv, idx, 16 * gcol, 0, 0);
      r.v1 = u32x4{0u, 0u, 0u, 0u};
      r.sc = sbuf_load_b32(rs_sc, idx, 4 * (gcol >> 1), 0, 0);
    }
  };
  // Converts this lane's 32 channels of slice s to fp16 and stores them to the tile.
  auto convert_store = [&](int s, const Raw& r, uint16_t* tile) {
    u32x4 c[4];
    if (s < n_wsl) {
      c[0] = fp8x8_to_f16x8(r.v0.x, r.v0.y);
      c[1] = fp8x8_to_f16x8(r.v0.z, r.v0.w);
      c[2] = fp8x8_to_f16x8(r.v1.x, r.v1.y);
      c[3] = fp8x8_to_f16x8(r.v1.z, r.v1.w);
    } else {
      // groups 2*gcol (codes of v0.x, v0.y) and 2*gcol + 1 (v0.z, v0.w): the 16-bit half
      // (gcol % 2) of the scale dword
      const uint32_t pair = r.sc >> (16 * (gcol & 1));
      const f16x2 s2 = e4m3x2_to_f16x2<false>(pair);
      const f16x2 sa = f16x2{s2.x, s2.x}, sb = f16x2{s2.y, s2.y};
      c[0] = fp4x8_to_f16x8(r.v0.x, sa);
      c[1] = fp4x8_to_f16x8(r.v0.y, sa);
      c[2] = fp4x8_to_f16x8(r.v0.z, sb);
      c[3] = fp4x8_to_f16x8(r.v0.w, sb);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(tile + ah_off(it, 32 * gcol + 8 * j)) = c[j];
  };

  // Output accumulators: O^T[64 * wave + 16 * ct + 4 * grp + i][16 * hh + gcol].
  f32x4 oacc[4][4];
  float ref = -__builtin_inff();   // reference of head h (log2 units)
  float mx = -__builtin_inff();    // largest logit of head h seen by this lane's items
  float l_run = 0.f;
  bool ref_set = false;
  if (tid == 0) sh.flag = 0;
  bool again;
#pragma unroll 1
  do {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) oacc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    Raw cur;
    int32_t pnext = position(1);
    fetch(0, position(0), cur);
#pragma unroll 1
    for (int s = 0; s < n_sl; ++s) {
      const int buf = s & 1;
      uint16_t* tile = sh.tile[buf];
      convert_store(s, cur, tile);
      if (grp < 4 && gcol == 0) sh.valid[buf][it] = cur.ok ? 1u : 0u;
      const int32_t pn = pnext;
      pnext = position(s + 2);
      fetch(s + 1, pn, cur);     // past the last slice every item is absent: no memory access
      __syncthreads();

      // Logits of items 16 * ih + 4 * grp + i for head h.
      // Operand reads four k-steps at a time into two independent product chains (even and
      // odd k-steps), so LDS latency and the matrix core's result latency overlap.
      const int row = 16 * ih + gcol;
      f32x4 s_even = {0.f, 0.f, 0.f, 0.f}, s_odd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k4 = 0; k4 < 16; k4 += 4) {
        u32x4 av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = *reinterpret_cast<const u32x4*>(tile + ah_off(row, 32 * (k4 + i) + 8 * grp));
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          s_even = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[i]),
                                                          qop[k4 + i], s_even, 0, 0, 0);
          s_odd = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av[i + 1]),
                                                         qop[k4 + i + 1], s_odd, 0, 0, 0);
        }
      }
      const f32x4 sacc = s_even + s_odd;
      float lg[4];
      bool any_valid = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = sh.valid[buf][16 * ih + 4 * grp + i] != 0u;
        lg[i] = v ? sacc[i] * lscale : -__builtin_inff();
        mx = fmaxf(mx, lg[i]);
      }
      if (!ref_set) {
        // uniform: every wavefront reads the same validity words
#pragma unroll
        for (int i = 0; i < AH_SLICE; ++i) any_valid |= sh.valid[buf][i] != 0u;
        if (any_valid) {
          float m = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
          m = fmaxf(m, __shfl_xor(m, 16));
          m = fmaxf(m, __shfl_xor(m, 32));
          if (grp == 0) sh.xch[ih][h] = m;
          __syncthreads();
          ref = fmaxf(sh.xch[0][h], sh.xch[1][h]);
          ref_set = true;
        }
      }
      bool over = false;
      f16x4 pv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        over |= lg[i] > ref + AT_GAP;
        const float pe = lg[i] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(lg[i] - ref);
        l_run += pe;
        pv[i] = (_Float16)pe;
      }
      if (over) sh.flag = 1;
      sh.pw[buf][ht][ih][lane] = __builtin_bit_cast(u32x2, pv);
      __syncthreads();

      // O^T[channels 64 * wave + 16 * ct .. +15][heads] += C^T . P over the slice's 32 items
      // (K = 32): lane group grp carries items 8*grp .. 8*grp+7 in both operands. A is two
      // transpose reads (items 8*grp + r and 8*grp + 4 + r, r = gcol / 4); B is the weights
      // written by the logit lanes of item half grp / 2, lane groups 2*(grp % 2) and
      // 2*(grp % 2) + 1.
      u32x4 at[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int ch = 64 * wave + 16 * ct + 4 * (gcol & 3);
        const u32x2 lo = lds_read_tr16x4(tile + ah_off(8 * grp + (gcol >> 2), ch));
        const u32x2 hi = lds_read_tr16x4(tile + ah_off(8 * grp + 4 + (gcol >> 2), ch));
        at[ct] = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
      const int pl = gcol + 32 * (grp & 1);
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const u32x2 b0 = sh.pw[buf][hh][grp >> 1][pl];
        const u32x2 b1 = sh.pw[buf][hh][grp >> 1][pl + 16];
        const u32x4 bw = u32x4{b0.x, b0.y, b1.x, b1.y};
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          oacc[ct][hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8, at[ct]), __builtin_bit_cast(f16x8, bw), oacc[ct][hh], 0, 0, 0);
      }
    }
    __syncthreads();
    again = sh.flag != 0;   // uniform
    if (again) {
      // repeat with each head's largest logit as its reference (it cannot be exceeded)
      float m = mx;
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (grp == 0) sh.xch[ih][h] = m;
      __syncthreads();
      ref = fmaxf(sh.xch[0][h], sh.xch[1][h]);
      ref_set = true;
      if (tid == 0) sh.flag = 0;
      __syncthreads();
    }
  } while (again);

  // Normalise: L[head] = the sum of both item halves' weights.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (grp == 0) sh.xch[ih][h] = l_run;
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    const int head = 16 * hh + gcol;
    const float L = sh.xch[0][head] + sh.xch[1][head];
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t* orow = out + ((int64_t)t * 64 + head) * 512 + 64 * wave + 4 * grp;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x4 a = oacc[ct][hh];
      const uint32_t b0 = f32_to_bf16_rne(a[0] * inv), b1 = f32_to_bf16_rne(a[1] * inv);
      const uint32_t b2 = f32_to_bf16_rne(a[2] * inv), b3 = f32_to_bf16_rne(a[3] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * ct) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
  }
  if (lse != nullptr && ih == 0 && grp == 0) {
    const float L = sh.xch[0][h] + sh.xch[1][h];
    lse[(int64_t)t * 64 + h] = L > 0.f ? (ref + __log2f(L)) * AT_LN2 : -__builtin_inff();
  }
}

hipError_t launch_sparse_attn(int n_q, const uint16_t* q, const uint8_t* kv_fp4,
                              int64_t fp4_stride, const uint8_t* kv_scale, int64_t scale_stride,
                              int64_t n_entries, const int64_t* kv_start, const int32_t* topk_idx,
                              int64_t ld_idx, int k, const uint8_t* window_kv,
                              int64_t n_window_rows, const int64_t* swa_start,
                              const int32_t* n_swa, float softmax_scale, uint16_t* out,
                              float* lse, hipStream_t stream) {
  if (n_q >= AH_MIN_Q) {
    hipLaunchKernelGGL(sparse_attn_heads_kernel, dim3(n_q), dim3(AH_THREADS), 0, stream, q,
                       kv_fp4, fp4_stride, kv_scale, scale_stride, n_entries, kv_start, topk_idx,
                       ld_idx, k, window_kv, n_window_rows, swa_start, n_swa, softmax_scale, out,
                       lse);
    return hipGetLastError();
  }
  const int groups8 = (n_q + N_XCD - 1) / N_XCD;
  if (n_q <= AT_HALVES_MAX_Q)
    hipLaunchKernelGGL(sparse_attn_kernel<2>, dim3(groups8 * N_XCD * AT_GROUPS * 2),
                       dim3(AT_THREADS), 0, stream, q, kv_fp4, fp4_stride, kv_scale,
                       scale_stride, n_entries, kv_start, topk_idx, ld_idx, k, window_kv,
                       n_window_rows, swa_start, n_swa, softmax_scale, n_q, out, lse);
  else
    hipLaunchKernelGGL(sparse_attn_kernel<1>, dim3(groups8 * N_XCD * AT_GROUPS),
                       dim3(AT_THREADS), 0, stream, q, kv_fp4, fp4_stride, kv_scale,
                       scale_stride, n_entries, kv_start, topk_idx, ld_idx, k, window_kv,
                       n_window_rows, swa_start, n_swa, softmax_scale, n_q, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
