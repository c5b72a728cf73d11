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
// Work split: a workgroup takes one query and one run of the entry list (a "split") and
// all 64 heads; its four wavefronts own 16 heads each. Per chunk of 32 entries:
//   - gather + dequantise: the 256 threads turn 32 rows (FP4 payload + scales, or FP8
//     window rows) into bf16 in LDS, in two layouts: C[e][d] (row-major) and C^T[d][e];
//     the conversion is exact (<= 5 significant bits per value);
//   - logits: S^T (32 entries x 16 heads) = C . Q^T with v_mfma_f32_16x16x32_bf16,
//     A from C[e][d] in LDS, B = this wave's 16 query heads held in registers;
//   - online softmax in fp32 per head (each lane owns one head column);
//   - O^T (512 x 16 heads) += C^T . P^T: A from C^T[d][e] in LDS, B = P^T straight from
//     the logits' accumulator registers (bf16). The 512x16 accumulator stays in
//     registers for the whole split.
// Several splits of one query are merged afterwards with their (max, sum) statistics.
// The workgroup id is arranged so that every split of a query runs on the same XCD and
// the query's 64 KiB of Q is fetched into that XCD's L2 once.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int AT_THREADS = 256;
constexpr int AT_CHUNK = 32;
constexpr int CROW = 512 + 8;   // bf16 per row of C[e][d] (padding spreads LDS banks)
constexpr int CCOL = 32 + 4;    // bf16 per row of C^T[d][e]
constexpr int AT_TARGET_WGS = 512;
constexpr int N_XCD = 8;
constexpr int PART_STRIDE = 512 + 4;  // floats per (query, split, head) partial: o[512], m, l, pad

int attn_splits(int n_q, int k) {
  const int chunks = (k + 128 + AT_CHUNK - 1) / AT_CHUNK;
  if (n_q <= 0) return 1;
  int s = (AT_TARGET_WGS + n_q - 1) / n_q;
  if (s > chunks) s = chunks;
  if (s < 1) s = 1;
  const int per = (chunks + s - 1) / s;
  return (chunks + per - 1) / per;
}

static int attn_chunks_per_split(int k, int splits) {
  const int chunks = (k + 128 + AT_CHUNK - 1) / AT_CHUNK;
  return (chunks + splits - 1) / splits;
}

size_t attn_workspace_bytes(int n_q, int k) {
  const int s = attn_splits(n_q, k);
  if (s <= 1 || n_q <= 0) return 0;
  return (size_t)n_q * s * 64 * PART_STRIDE * sizeof(float);
}

__global__ __launch_bounds__(AT_THREADS, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_fp4, int64_t fp4_stride,
    const uint8_t* __restrict__ kv_scale, int64_t sc_stride, int64_t n_entries,
    const int64_t* __restrict__ kv_start, const int32_t* __restrict__ topk_idx, int64_t ld_idx,
    int k, const uint8_t* __restrict__ window_kv, int64_t n_win_rows,
    const int64_t* __restrict__ swa_start, const int32_t* __restrict__ n_swa, float scale,
    int n_q, int splits, int chunks_per_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part) {
  __shared__ uint16_t crow[AT_CHUNK * CROW];
  __shared__ uint16_t ccol[512 * CCOL];
  __shared__ int valid_e[AT_CHUNK];

  // XCD-aware id: ids g*8*splits .. g*8*splits + 8*splits-1 hold queries 8g..8g+7; id % 8
  // (the XCD the id is dispatched to) equals t % 8 for every split of query t.
  const int id = blockIdx.x;
  const int grp = id / (N_XCD * splits);
  const int r = id % (N_XCD * splits);
  const int s = r / N_XCD;
  const int t = grp * N_XCD + r % N_XCD;
  if (t >= n_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;   // head within the wave's 16
  const int gq = lane >> 4;    // lane group 0..3
  const int h = wave * 16 + col;

  int nsw = n_swa[t];
  nsw = nsw < 0 ? 0 : (nsw > 128 ? 128 : nsw);
  const int n_items = k + nsw;
  const int i_begin = s * chunks_per_split * AT_CHUNK;
  int i_end = i_begin + chunks_per_split * AT_CHUNK;
  if (i_end > n_items) i_end = n_items;
  const int64_t base = kv_start[t];
  const int64_t wbase = swa_start[t];

  // B operand of the logits: Q^T[d][h] for d = 32*ks + 8*gq + (0..7).
  bf16x8 qb[16];
  const uint16_t* qrow = q + ((int64_t)t * 64 + h) * 512 + 8 * gq;
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);

  f32x4 oacc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  // Gather mapping: thread (e = tid % 32, gpart = tid / 32) converts channels
  // 64*gpart .. 64*gpart+63 of entry e of the chunk: 32 payload bytes + 4 scale bytes of a
  // main row, or 64 bytes of a window row. The entry's index is fetched one chunk ahead.
  const int ge = tid & 31;
  const int gpart = tid >> 5;
  auto load_idx = [&](int c0) -> int32_t {
    const int item = c0 + ge;
    return (item < i_end && item < k) ? topk_idx[(int64_t)t * ld_idx + item] : -1;
  };
  int32_t p_next = load_idx(i_begin);

#pragma unroll 1
  for (int c0 = i_begin; c0 < i_end; c0 += AT_CHUNK) {
    const int32_t p = p_next;
    if (c0 + AT_CHUNK < i_end) p_next = load_idx(c0 + AT_CHUNK);
    const int item = c0 + ge;
    u32x4 raw[4] = {};
    uint32_t sc = 0;
    int kind = 0;   // 0 absent, 1 main FP4 row, 2 window FP8 row
    if (item < i_end) {
      if (item < k) {
        const int64_t row = base + p;
        if (p >= 0 && row >= 0 && row < n_entries) {
          const u32x4* src = reinterpret_cast<const u32x4*>(kv_fp4 + row * fp4_stride + 32 * gpart);
          raw[0] = src[0];
          raw[1] = src[1];
          sc = *reinterpret_cast<const uint32_t*>(kv_scale + row * sc_stride + 4 * gpart);
          kind = 1;
        }
      } else {
        const int64_t wr = wbase + (item - k);
        if (wr >= 0 && wr < n_win_rows) {
          const u32x4* src = reinterpret_cast<const u32x4*>(window_kv + wr * 512 + 64 * gpart);
#pragma unroll
          for (int i = 0; i < 4; ++i) raw[i] = src[i];
          kind = 2;
        }
      }
    }
    __syncthreads();   // the previous chunk's LDS tiles are no longer read
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // channels 64*gpart + 8j .. +7
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kind == 1) {
        v = fp4x8_to_bf16x8(raw[j >> 2][j & 3], e4m3_to_f32((sc >> (8 * (j >> 1))) & 0xFFu));
      } else if (kind == 2) {
        const u32x2 lo = e4m3x4_to_bf16x4(raw[(2 * j) >> 2][(2 * j) & 3]);
        const u32x2 hi = e4m3x4_to_bf16x4(raw[(2 * j + 1) >> 2][(2 * j + 1) & 3]);
        v = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
      const int ch = 64 * gpart + 8 * j;
      *reinterpret_cast<u32x4*>(&crow[ge * CROW + ch]) = v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t pair = v[i];
        ccol[(ch + 2 * i) * CCOL + ge] = (uint16_t)(pair & 0xFFFFu);
        ccol[(ch + 2 * i + 1) * CCOL + ge] = (uint16_t)(pair >> 16);
      }
    }
    if (gpart == 0) valid_e[ge] = kind != 0 ? 1 : 0;
    __syncthreads();

    // Logits S^T[e][h] for the chunk's two 16-entry tiles.
    f32x4 sacc[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) {
      sacc[et] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = &crow[(et * 16 + col) * CROW + 8 * gq];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 32 * ks);
        sacc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], sacc[et], 0, 0, 0);
      }
    }
    // This lane holds entries e = 16*et + 4*gq + i of head h.
    float lg[8];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int et = 0; et < 2; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = et * 16 + 4 * gq + i;
        const float x = valid_e[e] ? sacc[et][i] * scale : -__builtin_inff();
        lg[et * 4 + i] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    if (m_new == -__builtin_inff()) continue;  // nothing valid yet (same for every head)
    const float alpha = __expf(m_run - m_new);
    float psum = 0.f;
    uint32_t pb[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = __expf(lg[i] - m_new);
      const float p1 = __expf(lg[i + 1] - m_new);
      psum += p0 + p1;
      pb[i / 2] = f32_to_bf16_rne(p0) | (f32_to_bf16_rne(p1) << 16);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const bf16x8 pv = __builtin_bit_cast(bf16x8, u32x4{pb[0], pb[1], pb[2], pb[3]});
    // O^T[d][h] += sum_e C^T[d][e] P^T[e][h]; the lane's k slots are entries
    // 4*gq .. 4*gq+3 and 16+4*gq .. 16+4*gq+3, matching pv.
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint16_t* crow_t = &ccol[(dt * 16 + col) * CCOL];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(crow_t + 4 * gq);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(crow_t + 16 + 4 * gq);
      const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      oacc[dt] = oacc[dt] * alpha;
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pv, oacc[dt], 0, 0, 0);
    }
  }

  // This lane holds O^T[d = 16*dt + 4*gq + i][h], unnormalised, for every dt.
  if (splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* orow = out + ((int64_t)t * 64 + h) * 512;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const uint32_t b0 = f32_to_bf16_rne(oacc[dt][0] * inv), b1 = f32_to_bf16_rne(oacc[dt][1] * inv);
      const uint32_t b2 = f32_to_bf16_rne(oacc[dt][2] * inv), b3 = f32_to_bf16_rne(oacc[dt][3] * inv);
      *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * gq) = u32x2{b0 | (b1 << 16), b2 | (b3 << 16)};
    }
    if (lse != nullptr && gq == 0)
      lse[(int64_t)t * 64 + h] = l_run > 0.f ? m_run + __logf(l_run) : -__builtin_inff();
  } else {
    float* prow = part + (((int64_t)t * splits + s) * 64 + h) * PART_STRIDE;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt)
      *reinterpret_cast<f32x4*>(prow + 16 * dt + 4 * gq) = oacc[dt];
    if (gq == 0) {
      prow[512] = m_run;
      prow[513] = l_run;
    }
  }
}

// Merge the splits of one (query, head): out = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part,
                                                         int splits, uint16_t* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int th = blockIdx.x;  // t*64 + h
  const int t = th >> 6, h = th & 63;
  const float* p0 = part + ((int64_t)t * splits * 64 + h) * PART_STRIDE;
  const int64_t sstride = 64 * PART_STRIDE;
  float M = -__builtin_inff();
  for (int s = 0; s < splits; ++s) M = fmaxf(M, p0[s * sstride + 512]);
  float L = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int d = threadIdx.x * 2;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < splits; ++s) {
      const float* ps = p0 + s * sstride;
      const float ms = ps[512];
      const float f = ms == -__builtin_inff() ? 0.f : __expf(ms - M);
      L += f * ps[513];
      acc0 += f * ps[d];
      acc1 += f * ps[d + 1];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = out + (int64_t)th * 512;
  *reinterpret_cast<uint32_t*>(orow + d) =
      f32_to_bf16_rne(acc0 * inv) | (f32_to_bf16_rne(acc1 * inv) << 16);
  if (lse != nullptr && threadIdx.x == 0) lse[th] = L > 0.f ? M + __logf(L) : -__builtin_inff();
}

hipError_t launch_sparse_attn(int n_q, const uint16_t* q, const uint8_t* kv_fp4,
                              int64_t fp4_stride, const uint8_t* kv_scale, int64_t scale_stride,
                              int64_t n_entries, const int64_t* kv_start, const int32_t* topk_idx,
                              int64_t ld_idx, int k, const uint8_t* window_kv,
                              int64_t n_window_rows, const int64_t* swa_start,
                              const int32_t* n_swa, float softmax_scale, uint16_t* out,
                              float* lse, void* workspace, hipStream_t stream) {
  const int splits = attn_splits(n_q, k);
  const int cps = attn_chunks_per_split(k, splits);
  const int groups = (n_q + N_XCD - 1) / N_XCD;
  float* part = static_cast<float*>(workspace);
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(groups * N_XCD * splits), dim3(AT_THREADS), 0,
                     stream, q, kv_fp4, fp4_stride, kv_scale, scale_stride, n_entries, kv_start,
                     topk_idx, ld_idx, k, window_kv, n_window_rows, swa_start, n_swa,
                     softmax_scale, n_q, splits, cps, out, lse, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || splits == 1) return err;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(n_q * 64), dim3(256), 0, stream, part, splits, out,
                     lse);
  return hipGetLastError();
}

}  // namespace csa2
