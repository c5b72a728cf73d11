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
// (separately, so a slice never mixes the two formats); a workgroup owns one
// group of 16 heads and one contiguous range of slices (a "split"), and its four
// wavefronts take every fourth slice of that range and run independently (no barrier in
// the main loop). Per slice a wavefront:
//   - gathers the 16 rows (lane = item x quarter of the 512 channels) two slices ahead of
//     their use, so each HBM round trip overlaps two slices of arithmetic. The gathers are
//     indexed buffer loads: an absent item gets an index past the buffer's record count
//     and reads zeros, so every slice issues the same loads into the same registers and
//     the wait for a slice never includes the loads of the slices behind it;
//   - converts them to fp16 with the hardware E2M1/E4M3 -> fp16 conversions and a packed
//     fp16 multiply by the group scale; every value is exact (an E2M1 x E4M3 product has
//     <= 6 significant bits in [2^-10, 2688]). The converted registers are directly the A
//     operand of the logit product S^T (16 items x 16 heads) = C . Q^T
//     (v_mfma_f32_16x16x32_f16, K = 512; B = this group's queries in registers, each head
//     rescaled by a power of two into fp16's range, the inverse folded into the logit
//     scale), and are also stored to the wavefront's own LDS tile;
//   - never rescales its accumulator: the reference max of each head is the largest logit
//     of the first slice with a valid item, and later weights p = 2^(l - ref) may reach
//     2^15 (fp16 holds them); a logit beyond that restarts the wavefront's slices with the
//     raised reference (rare; the result does not depend on the reference);
//   - O^T (512 x 16 heads) += C^T . P^T with v_mfma_f32_16x16x16_f16: P^T is the logits'
//     accumulator layout, A = C^T is read from the tile with LDS transpose reads
//     (ds_read_b64_tr_b16).
// The four wavefront partials are merged through LDS. With more than one split per head
// group, each workgroup stores its (max, sum, O) partial in the workspace and a second
// kernel combines them in split order (no cross-workgroup synchronisation inside a
// kernel). Workgroup ids put all workgroups of a query on one XCD, so they share its L2
// copy of the rows.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int AT_THREADS = 256;
constexpr int AT_WAVES = 4;
constexpr int AT_SLICE = 16;                 // items per wavefront step
constexpr int AT_HEADS = 16;                 // heads per workgroup
constexpr int AT_GROUPS = 64 / AT_HEADS;     // head groups per query
constexpr int AT_MAX_K = 2048;               // largest selection the index staging holds
constexpr int AT_WINDOW = 128;               // largest sliding window
constexpr int AT_MAX_SPLITS = 8;
constexpr int AT_TARGET_WGS = 256;           // one workgroup per compute unit
constexpr int N_XCD = 8;
constexpr float AT_GAP = 15.f;               // largest log2 weight over the reference
constexpr float AT_LOG2E = 1.4426950408889634f;
constexpr float AT_LN2 = 0.6931471805599453f;

int attn_splits(int n_q, int k) {
  const int n_sl = (k + AT_WINDOW + AT_SLICE - 1) / AT_SLICE;
  int s = 1;
  // Double the splits while the grid is below one workgroup per CU and every wavefront
  // would still get at least two slices.
  while (s < AT_MAX_SPLITS && (int64_t)n_q * AT_GROUPS * s < AT_TARGET_WGS &&
         n_sl >= 2 * AT_WAVES * 2 * s)
    s *= 2;
  return s;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace (only with more than one split): [max/sum: float (S x 2 x 16) per (query,
// head group)] [O: float (S x 16 x 512) per group].
size_t attn_workspace_bytes(int n_q, int k) {
  const int s = attn_splits(n_q, k);
  if (s == 1 || n_q <= 0) return 0;
  const size_t groups = (size_t)n_q * AT_GROUPS;
  return align256(groups * s * 2 * AT_HEADS * 4) + groups * s * AT_HEADS * 512 * 4;
}

// A wavefront's tile holds 16 rows C[e][0..512) in fp16. Row e starts at element
// TILE_ROW * e and its channel quarter g (128 channels) at + TILE_QUARTER * g: rows are
// 1,120 B apart and quarters 272 B apart. LDS has 128 four-byte banks; 16-byte accesses are
// served 32 lanes at a time and 8-byte ones 64 at a time. With these strides the
// conversion's stores (16 rows x 2 quarters x one 16-byte block per pass) and the
// transpose reads (16 rows x one 32-byte chunk) each touch every bank exactly once, and
// every address is a per-lane base plus a compile-time offset.
constexpr int TILE_ROW = 560;       // elements
constexpr int TILE_QUARTER = 136;   // elements
constexpr int TILE_ELEMS = AT_SLICE * TILE_ROW;
// Merge buffer rows (one head, 256 channels) are padded to 264 floats so that the stores
// (16 heads x 2 lane groups per pass) and the reads (16 heads x 2 channel groups) are free
// of bank conflicts.
constexpr int PART_ROW = 264;

struct AttnShared {
  union {
    uint16_t tile[AT_WAVES][TILE_ELEMS];         // 70 KiB: per-wave slice tiles
    float part[AT_WAVES][AT_HEADS][PART_ROW];    // 66 KiB: merge buffer, half of d at a time
  };
  int32_t pidx[AT_MAX_K];                        // this split's selected positions
  float wm[AT_WAVES][AT_HEADS];
  float wl[AT_WAVES][AT_HEADS];
};

// One slice's gathered bytes for one lane: 64 B of an FP4 row plus its 8 scale bytes, or
// 128 B of a window row. Absent items read as zeros.
struct Raw {
  u32x4 v[8];
  uint32_t sc0, sc1;
  bool valid;   // the item exists
};

// Converts block j (channels 128*gq + 8j .. +7) of the lane's gathered bytes to fp16.
template <bool WINDOW>
__device__ __forceinline__ u32x4 convert_block(const Raw& r, const f16x2 (&sq)[8], int j) {
  if (WINDOW) return fp8x8_to_f16x8(r.v[j >> 1][2 * (j & 1)], r.v[j >> 1][2 * (j & 1) + 1]);
  return fp4x8_to_f16x8(r.v[j >> 2][j & 3], sq[j >> 1]);
}

// Converts the lane's 16 blocks, stores them to its row quarter of the tile (tile_row)
// and accumulates the logits.
template <bool WINDOW>
__device__ __forceinline__ f32x4 convert_and_score(const Raw& r, const f16x8 (&qb)[16],
                                                   uint16_t* tile_row) {
  f16x2 sq[8];
  if (!WINDOW) {
    const f16x2 s01 = e4m3x2_to_f16x2<false>(r.sc0), s23 = e4m3x2_to_f16x2<true>(r.sc0);
    const f16x2 s45 = e4m3x2_to_f16x2<false>(r.sc1), s67 = e4m3x2_to_f16x2<true>(r.sc1);
    sq[0] = f16x2{s01.x, s01.x}; sq[1] = f16x2{s01.y, s01.y};
    sq[2] = f16x2{s23.x, s23.x}; sq[3] = f16x2{s23.y, s23.y};
    sq[4] = f16x2{s45.x, s45.x}; sq[5] = f16x2{s45.y, s45.y};
    sq[6] = f16x2{s67.x, s67.x}; sq[7] = f16x2{s67.y, s67.y};
  }
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const u32x4 a = convert_block<WINDOW>(r, sq, j);
    *reinterpret_cast<u32x4*>(tile_row + 8 * j) = a;
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), qb[j], sacc, 0,
                                                  0, 0);
  }
  return sacc;
}

__global__ __launch_bounds__(AT_THREADS) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_fp4, int64_t fp4_stride,
    const uint8_t* __restrict__ kv_scale, int64_t sc_stride, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const int32_t* __restrict__ topk_idx, int64_t ld_idx,
    int k, const uint8_t* __restrict__ window_kv, int64_t n_win_rows,
    const int64_t* __restrict__ swa_start, const int32_t* __restrict__ n_swa, float scale,
    int n_q, int n_split, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ AttnShared sh;

  // id = (g * J + j) * 8 + t % 8 for queries 8g .. 8g+7 and J = 4 * n_split workgroups per
  // query: every workgroup of query t has id % 8 = t % 8.
  const int J = AT_GROUPS * n_split;
  const int id = blockIdx.x;
  const int t = (id / (N_XCD * J)) * N_XCD + id % N_XCD;
  if (t >= n_q) return;
  const int jj = (id / N_XCD) % J;
  const int hg = jj % AT_GROUPS;
  const int sp = jj / AT_GROUPS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: lets slice indices stay scalar
  const int col = lane & 15;   // head within the group; also the item a lane gathers
  const int gq = lane >> 4;    // lane group 0..3; also the channel quarter a lane gathers
  const int h = hg * AT_HEADS + col;

  int nsw = n_swa[t];
  nsw = nsw < 0 ? 0 : (nsw > AT_WINDOW ? AT_WINDOW : nsw);
  const int n_msl = (k + AT_SLICE - 1) / AT_SLICE;     // slices of selected entries
  const int n_sl = n_msl + (nsw + AT_SLICE - 1) / AT_SLICE;
  const int lo = (int)((int64_t)sp * n_sl / n_split);
  const int hi = (int)((int64_t)(sp + 1) * n_sl / n_split);
  const int64_t base = kv_start[t];
  const int64_t wbase = swa_start[t];

  // Stage this split's selected positions in LDS (one HBM round trip, overlapped with the
  // query load below).
  const int i_lo = AT_SLICE * lo;
  const int i_hi = min(AT_SLICE * hi, k);
  const int n_idx = i_hi > i_lo ? i_hi - i_lo : 0;
  int32_t pstage[AT_MAX_K / AT_THREADS];
#pragma unroll
  for (int r = 0; r < AT_MAX_K / AT_THREADS; ++r) {
    const int j = tid + AT_THREADS * r;
    pstage[r] = j < n_idx ? topk_idx[(int64_t)t * ld_idx + i_lo + j] : -1;
  }

  // Logit B operand: Q^T for head h, k-step ks, lane group gq = channels 8*ks + 128*gq ..
  // +7 (the conversion below produces the rows with the same channel assignment).
  u32x4 qraw[16];
  const uint16_t* qrow = q + ((int64_t)t * 64 + h) * 512 + 128 * gq;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qraw[ks] = *reinterpret_cast<const u32x4*>(qrow + 8 * ks);

#pragma unroll
  for (int r = 0; r < AT_MAX_K / AT_THREADS; ++r) {
    const int j = tid + AT_THREADS * r;
    if (j < n_idx) sh.pidx[j] = pstage[r];
  }
  __syncthreads();

  // Gather: lane (item col of slice c, quarter gq) -> channels 128*gq .. +127 of that item.
  // Slice c < n_msl holds selected entries 16c .. 16c+15, later slices window rows. The
  // buffers are indexed by row relative to the query's own base, so the 32-bit record
  // index covers any sequence; absent items use an index past every record count.
  constexpr uint32_t ABSENT = 0xFFFFFFFFu;
  const int64_t kv_rows = n_entries - base;
  const int64_t win_rows = n_win_rows - wbase;
  const uint32_t kv_n = kv_rows <= 0 ? 0u : (kv_rows >= (int64_t)ABSENT ? ABSENT - 1u : (uint32_t)kv_rows);
  const uint32_t win_n = win_rows <= 0 ? 0u : (win_rows >= (int64_t)ABSENT ? ABSENT - 1u : (uint32_t)win_rows);
  const __amdgpu_buffer_rsrc_t rs_kv = make_rows_rsrc(kv_fp4 + base * fp4_stride, (int)fp4_stride, kv_n);
  const __amdgpu_buffer_rsrc_t rs_sc = make_rows_rsrc(kv_scale + base * sc_stride, (int)sc_stride, kv_n);
  const __amdgpu_buffer_rsrc_t rs_win = make_rows_rsrc(window_kv + wbase * 512, 512, win_n);
  auto fetch = [&](int c, Raw& raw) {
    const bool main = c < n_msl;   // wavefront-uniform
    uint32_t ridx;
    bool ok;
    if (main) {
      const int item = AT_SLICE * c + col;
      const int li = item - i_lo;
      const int32_t p = sh.pidx[li < 0 ? 0 : (li >= AT_MAX_K ? AT_MAX_K - 1 : li)];
      const int64_t row = base + p;
      ok = c < hi && item < k && p >= 0 && row >= 0 && row < n_entries;
      ridx = (uint32_t)p;
    } else {
      const int wi = AT_SLICE * (c - n_msl) + col;
      const int64_t wr = wbase + wi;
      ok = c < hi && wi < nsw && wr >= 0 && wr < n_win_rows;
      ridx = (uint32_t)wi;
    }
    raw.valid = ok;
    const uint32_t i_main = ok && main ? ridx : ABSENT;
    const uint32_t i_win = ok && !main ? ridx : ABSENT;
    // Blocks 0..3: the FP4 row quarter (64 B) or the first half of the window row quarter;
    // blocks 4..7: the second half of the window row quarter (zeros for FP4 slices).
    const __amdgpu_buffer_rsrc_t r_lo = main ? rs_kv : rs_win;
    const uint32_t i_lo4 = main ? i_main : i_win;
    const int o_lo = main ? 64 * gq : 128 * gq;
#pragma unroll
    for (int i = 0; i < 4; ++i) raw.v[i] = sbuf_load_b128(r_lo, (int)i_lo4, o_lo + 16 * i, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      raw.v[4 + i] = sbuf_load_b128(rs_win, (int)i_win, 128 * gq + 64 + 16 * i, 0, 0);
    const u32x2 s8 = sbuf_load_b64(rs_sc, (int)i_main, 8 * gq, 0, 0);
    raw.sc0 = s8.x;
    raw.sc1 = s8.y;
  };
  Raw buf0, buf1;
  const int c0 = lo + wave;

  float qmax = 0.f;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qmax = fmaxf(qmax, fabsf(__uint_as_float(qraw[ks][i] << 16)));
      qmax = fmaxf(qmax, fabsf(__uint_as_float(qraw[ks][i] & 0xFFFF0000u)));
    }
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
  const int qexp = qmax > 0.f ? (int)((__float_as_uint(qmax) >> 23) & 0xFFu) - 127 : 0;
  int kexp = 14 - qexp;
  kexp = kexp < -126 ? -126 : (kexp > 126 ? 126 : kexp);
  const float up = __uint_as_float((uint32_t)(127 + kexp) << 23);
  // logits in log2 units: l2 = acc * scale * 2^-kexp * log2(e)
  const float lscale = scale * AT_LOG2E * __uint_as_float((uint32_t)(127 - kexp) << 23);
  f16x8 qb[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qb[ks][2 * i] = (_Float16)(__uint_as_float(qraw[ks][i] << 16) * up);
      qb[ks][2 * i + 1] = (_Float16)(__uint_as_float(qraw[ks][i] & 0xFFFF0000u) * up);
    }

  // Output accumulator: O^T[d = 16*dt + 4*gq + i][h], dt = 0..31.
  f32x4 oacc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -__builtin_inff();   // reference max of head col (log2 units)
  float l_run = 0.f;                 // this lane's share of the sum for head col
  uint16_t* tile = sh.tile[wave];
  uint16_t* const tile_w = tile + TILE_ROW * col + TILE_QUARTER * gq;
  const uint16_t* const tile_r = tile + TILE_ROW * (4 * gq + (col >> 2)) + 4 * (col & 3);

  // One slice (c may lie past the split: its items are all absent); returns false when a
  // logit exceeds the reference by more than AT_GAP (the reference is raised, and the
  // caller repeats the pass).
  auto step = [&](int c, Raw& raw) -> bool {
    const uint64_t valid = __ballot(raw.valid);   // bit e: item e of the slice is present
    const f32x4 sacc = c < n_msl ? convert_and_score<false>(raw, qb, tile_w)
                                 : convert_and_score<true>(raw, qb, tile_w);
    // The registers are free again: start the gather two slices ahead.
    fetch(c + 2 * AT_WAVES, raw);
    if (valid == 0ull) return true;
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
      if (!first) return false;
    }
    f16x4 pv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pe = __builtin_amdgcn_exp2f(lg[i] - m_ref);
      l_run += pe;
      pv[i] = (_Float16)pe;
    }
    // O^T[d][h] += sum_e C^T[d][e] P^T[e][h], K = the slice's 16 items; lane group gq
    // carries items 4*gq .. 4*gq+3 in both operands. A comes from transpose reads: lane i
    // of a 16-lane group addresses channels 16*dt + 4*(i%4) .. +3 of item 4*gq + i/4 and
    // receives channel 16*dt + i of items 4*gq .. 4*gq+3.
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const u32x2 a = lds_read_tr16x4(tile_r + TILE_QUARTER * (dt >> 3) + 16 * (dt & 7));
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), pv,
                                                       oacc[dt], 0, 0, 0);
    }
    return true;
  };

  // Every step runs unconditionally (a slice past the split is all absent and its loads
  // return zeros without touching memory), so each buffer is written by the same loads on
  // every path and a step waits only for its own slice.
  bool again;
#pragma unroll 1
  do {
    fetch(c0, buf0);
    fetch(c0 + AT_WAVES, buf1);
    bool ok = true;
#pragma unroll 1
    for (int c = c0; c < hi; c += 2 * AT_WAVES) {
      ok &= step(c, buf0);
      ok &= step(c + AT_WAVES, buf1);
    }
    again = !ok;
    if (again) {   // a logit overflowed the reference: repeat with the raised one
#pragma unroll
      for (int i = 0; i < 32; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run = 0.f;
    }
  } while (again);

  // Merge the four wavefronts: O = sum_w 2^{m_w - M} O_w, L = sum_w 2^{m_w - M} l_w.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (gq == 0) {
    sh.wm[wave][col] = m_ref;
    sh.wl[wave][col] = l_run;
  }
  __syncthreads();   // also ends every wavefront's use of its tile
  // For each half of d, every wave stores its partial [head][d]; then lane (head
  // oh = lane%16, channel group dq = lane/16) of wave w sums channels
  // 64*rep + 16*w + 4*dq .. +3 of the half, each partial weighted by 2^(m_w - M). (The
  // weights are applied by the reader so that the accumulators only ever feed MFMAs and
  // stores.)
  const int oh = lane & 15;
  const int od = 16 * wave + 4 * (lane >> 4);
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
  f32x4 acc[2][4];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int dt = 0; dt < 16; ++dt)
      *reinterpret_cast<f32x4*>(&sh.part[wave][col][16 * dt + 4 * gq]) = oacc[16 * hf + dt];
    __syncthreads();
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int d = od + 64 * rep;
      f32x4 a = *reinterpret_cast<const f32x4*>(&sh.part[0][oh][d]) * fwh[0];
#pragma unroll
      for (int w = 1; w < AT_WAVES; ++w)
        a += *reinterpret_cast<const f32x4*>(&sh.part[w][oh][d]) * fwh[w];
      acc[hf][rep] = a;
    }
    __syncthreads();
  }

  if (n_split > 1) {
    // Partial of this split: O relative to its own max, plus max and sum per head.
    const int64_t g = (int64_t)t * AT_GROUPS + hg;
    float* po = ws_o + (g * n_split + sp) * (AT_HEADS * 512) + oh * 512 + od;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int rep = 0; rep < 4; ++rep)
        *reinterpret_cast<f32x4*>(po + 256 * hf + 64 * rep) = acc[hf][rep];
    if (wave == 0 && lane < 16) {
      ws_ml[(g * n_split + sp) * 32 + oh] = Mh;
      ws_ml[(g * n_split + sp) * 32 + 16 + oh] = Lh;
    }
    return;
  }

  const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
  uint16_t* orow = out + ((int64_t)t * 64 + hg * AT_HEADS + oh) * 512 + od;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const f32x4 a = acc[hf][rep];
      const uint32_t b0 = f32_to_bf16_rne(a[0] * inv), b1 = f32_to_bf16_rne(a[1] * inv);
      const uint32_t b2 = f32_to_bf16_rne(a[2] * inv), b3 = f32_to_bf16_rne(a[3] * inv);
      *reinterpret_cast<u32x2*>(orow + 256 * hf + 64 * rep) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
  if (lse != nullptr && wave == 0 && lane < 16)
    lse[(int64_t)t * 64 + hg * AT_HEADS + oh] =
        Lh > 0.f ? (Mh + __log2f(Lh)) * AT_LN2 : -__builtin_inff();
}

// Combines the split partials of one (query, head group) in split order. Thread (head
// tid/16, channels 32*(tid%16) .. +31).
__global__ __launch_bounds__(AT_THREADS) void attn_merge_kernel(
    int n_split, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int64_t g = blockIdx.x;   // query * 4 + head group
  const int hh = threadIdx.x >> 4;
  const int d0 = 32 * (threadIdx.x & 15);
  float ms[AT_MAX_SPLITS], ls[AT_MAX_SPLITS];
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < AT_MAX_SPLITS; ++s) {
    if (s < n_split) {
      ms[s] = ws_ml[(g * n_split + s) * 32 + hh];
      ls[s] = ws_ml[(g * n_split + s) * 32 + 16 + hh];
      M = fmaxf(M, ms[s]);
    }
  }
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < AT_MAX_SPLITS; ++s) {
    if (s < n_split) {
      const float wgt = ms[s] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
      L += wgt * ls[s];
      const f32x4* src = reinterpret_cast<const f32x4*>(ws_o + (g * n_split + s) * (AT_HEADS * 512) +
                                                        hh * 512 + d0);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += src[i] * wgt;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = out + (g * AT_HEADS + hh) * 512 + d0;   // head = 16 * (g % 4) + hh of query g / 4
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b0 = f32_to_bf16_rne(acc[i][0] * inv), b1 = f32_to_bf16_rne(acc[i][1] * inv);
    const uint32_t b2 = f32_to_bf16_rne(acc[i][2] * inv), b3 = f32_to_bf16_rne(acc[i][3] * inv);
    *reinterpret_cast<u32x2*>(orow + 4 * i) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
  }
  if (lse != nullptr && (threadIdx.x & 15) == 0)
    lse[g * AT_HEADS + hh] = L > 0.f ? (M + __log2f(L)) * AT_LN2 : -__builtin_inff();
}

hipError_t launch_sparse_attn(int n_q, const uint16_t* q, const uint8_t* kv_fp4,
                              int64_t fp4_stride, const uint8_t* kv_scale, int64_t scale_stride,
                              int64_t n_entries, const int64_t* kv_start, const int32_t* topk_idx,
                              int64_t ld_idx, int k, const uint8_t* window_kv,
                              int64_t n_window_rows, const int64_t* swa_start,
                              const int32_t* n_swa, float softmax_scale, uint16_t* out,
                              float* lse, void* workspace, hipStream_t stream) {
  const int splits = attn_splits(n_q, k);
  float* ws_ml = nullptr;
  float* ws_o = nullptr;
  if (splits > 1) {
    const size_t groups = (size_t)n_q * AT_GROUPS;
    uint8_t* w = static_cast<uint8_t*>(workspace);
    ws_ml = reinterpret_cast<float*>(w);
    ws_o = reinterpret_cast<float*>(w + align256(groups * splits * 2 * AT_HEADS * 4));
  }
  const int groups8 = (n_q + N_XCD - 1) / N_XCD;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(groups8 * N_XCD * AT_GROUPS * splits),
                     dim3(AT_THREADS), 0, stream, q, kv_fp4, fp4_stride, kv_scale, scale_stride,
                     n_entries, kv_start, topk_idx, ld_idx, k, window_kv, n_window_rows,
                     swa_start, n_swa, softmax_scale, n_q, splits, ws_ml, ws_o, out, lse);
  if (splits > 1)
    hipLaunchKernelGGL(attn_merge_kernel, dim3(n_q * AT_GROUPS), dim3(AT_THREADS), 0, stream,
                       splits, ws_ml, ws_o, out, lse);
  return hipGetLastError();
}

}  // namespace csa2
