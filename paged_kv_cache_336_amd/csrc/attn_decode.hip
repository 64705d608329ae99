// attn_decode.hip -- paged decode attention for gfx950.
//
// What it computes ("PagedAttention", shubhamtatvamasi.com, section "How
// attention reads paged memory"): for every sequence s and query head q,
// softmax(scale * q . k_j) weighted sum of v_j over the sequence's tokens
// j = 0 .. L_s - 1, where token j lives at offset j % bs of physical block
// block_table[s][j / bs] of a pool [num_blocks, bs, kv_heads, head_dim].  The
// kernel walks the table block by block and keeps a FlashAttention-style
// running maximum / running sum ("online softmax") per query head.
//
// Work unit: (sequence s, kv head h, chunk of <= 16 query heads of the group
// reading h, partition p of the sequence).  One 64-lane wave per unit, so each
// K/V row of a kv head is read once for all query heads that share it.
//
// Per 32-token tile:
//   * K rows go straight from HBM into MFMA A-operand registers as 16-byte
//     loads (lane = token row + 16 * piece group), Q sits in the B operand;
//     S = K . Q^T on v_mfma_f32_16x16x32 (bf16/f16; fp8 keys are decoded to
//     the query's type first) or eight 16x16x4 f32 steps.
//   * Scores are scaled into the log2 domain; the running max uses xor
//     shuffles across the 4 lanes that hold one query head's column.
//   * V rows are loaded as 16-byte pieces, converted to the PV operand type
//     and staged in LDS (XOR-swizzled 16-byte chunks), then read back
//     transposed as the A operand of O^T += V^T . P^T, so P never leaves the
//     registers the QK product left it in.  For bf16/f16 caches P is split
//     into a high and a low part (two MFMAs), which keeps the weights exact
//     to ~2^-16 relative.
//
// Partitions: a sequence longer than one partition writes an unnormalised
// partial (o, running max m, running sum l) per query head to the workspace;
// the wave that completes the last partition of an (s, h, chunk) -- found with
// a device-scope counter -- merges all of them:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// then resets the counter to zero for the next call.  Reduction order depends
// only on logical token positions, so relabelling physical blocks leaves the
// output bit-identical.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <typename QT, typename CT> struct PvOperand { typedef CT type; };
template <> struct PvOperand<BF16, FP8> { typedef F16 type; };
template <> struct PvOperand<F16, FP8> { typedef F16 type; };
template <> struct PvOperand<F32, FP8> { typedef F32 type; };

// Token (within a 32-token tile) that lane group j, operand slot e stands for:
// slots 0-3 are rows 4j..4j+3 of the first 16-token half, slots 4-7 the same
// rows of the second half -- exactly where the QK accumulator left them.
__device__ __forceinline__ int slot_token(int j, int e) {
  return e < 4 ? 4 * j + e : 12 + 4 * j + e;
}

template <int D>
__device__ void merge_partials(const AttnArgs& a, int s, int h, int gc,
                               int gcount, int nparts, float vscale) {
  const int lane = threadIdx.x;
  constexpr int DPL = D / 64;
  for (int g = 0; g < gcount; ++g) {
    const int hq = h * a.group + gc * 16 + g;
    const int64_t base = ((int64_t)s * a.num_q_heads + hq) * a.max_parts;
    float M = -INFINITY;
    for (int q = lane; q < nparts; q += 64) M = fmaxf(M, a.part_m[base + q]);
    M = wave_max(M);
    float den = 0.f;
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
    for (int q = 0; q < nparts; ++q) {
      const float w = fast_exp2(a.part_m[base + q] - M);
      den = fmaf(w, a.part_l[base + q], den);
      const float* src = a.part_o + (base + q) * D + lane * DPL;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, src[k], acc[k]);
    }
    float* dst = a.out + ((int64_t)s * a.num_q_heads + hq) * D + lane * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k) dst[k] = acc[k] / den * vscale;
  }
}

template <typename QT, typename CT, int D, bool UNIFORM>
__global__ __launch_bounds__(64) void attn_decode_kernel(AttnArgs a) {
  typedef typename PvOperand<QT, CT>::type PVT;
  constexpr bool PSPLIT = !is_fp8<CT>::value && CT::bytes == 2;
  constexpr int EP = 16 / CT::bytes;           // cache elements per 16-B piece
  constexpr int KPIECES = D * CT::bytes / 64;  // K pieces per lane per half
  constexpr int KWORDS = KPIECES * 4;
  constexpr int QSTEPS = D / 32;               // k32 steps over head_dim
  constexpr int ROW_BYTES = D * CT::bytes;     // one token's row of one head
  constexpr int PPR = ROW_BYTES / 16;          // pieces per row
  constexpr int NV = PPR / 2;                  // V pieces per lane per tile
  constexpr int TOK_PER_V = 64 / PPR;
  constexpr int PVB = PVT::bytes;
  constexpr int LDS_ROW = D * PVB;
  constexpr int VCH = EP * PVB / 16;           // LDS chunks per V piece
  constexpr int QWORDS = D / 4 * QT::bytes / 4;
  constexpr int NBLK = D / 16;                 // 16-wide output blocks
  static_assert(NV >= 1 && KPIECES >= 1, "head_dim too small");
  static_assert(LDS_ROW / 16 >= 4 * PVB, "swizzle needs 4 distinct spans");

  __shared__ __attribute__((aligned(16))) uint8_t vt[32 * LDS_ROW];

  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int j = lane >> 4;

  int u = blockIdx.x;
  const int part = u % a.max_parts;
  u /= a.max_parts;
  const int gc = u % a.group_chunks;
  u /= a.group_chunks;
  const int h = u % a.num_kv_heads;
  const int s = u / a.num_kv_heads;

  const int L = a.seq_lens[s];
  const int P = a.partition_size;
  const int nparts = L > 0 ? (L + P - 1) / P : 1;
  if (part >= nparts) return;
  const int t_begin = part * P;
  const int t_end = min(t_begin + P, L);
  const int gcount = min(16, a.group - gc * 16);
  const int hq = h * a.group + gc * 16 + c;
  const bool head_live = c < gcount;

  float kscale = 1.f, vscale = 1.f;
  if constexpr (is_fp8<CT>::value) {
    kscale = *a.k_scale;
    vscale = *a.v_scale;
  }
  const float qk_mul = a.qk_scale_log2 * kscale;

  // ---- query: B operand of S = K Q^T, in the same element order as K ----
  uint32_t qw[QWORDS];
  {
    const uint8_t* qrow = static_cast<const uint8_t*>(a.query) +
                          ((int64_t)s * a.num_q_heads + hq) * D * QT::bytes;
    constexpr int QBYTES_PER_R = EP * QT::bytes;
    constexpr int QLOADS = QBYTES_PER_R / 16;
#pragma unroll
    for (int r = 0; r < D / (4 * EP); ++r) {
#pragma unroll
      for (int k = 0; k < QLOADS; ++k) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (head_live)
          v = *reinterpret_cast<const u32x4_t*>(
              qrow + (4 * r + j) * QBYTES_PER_R + 16 * k);
        const int w0 = (r * QBYTES_PER_R + 16 * k) / 4;
        qw[w0 + 0] = v[0];
        qw[w0 + 1] = v[1];
        qw[w0 + 2] = v[2];
        qw[w0 + 3] = v[3];
      }
    }
  }

  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int bs = a.block_size;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) +
                         (int64_t)h * ROW_BYTES;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) +
                         (int64_t)h * ROW_BYTES;
  const int64_t slot_stride = (int64_t)a.num_kv_heads * ROW_BYTES;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4_t oacc[NBLK];
#pragma unroll
  for (int n = 0; n < NBLK; ++n) oacc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = t_begin; t0 < t_end; t0 += 32) {
    // ---------------- slots of the rows this lane loads ----------------
    int kslot[2];
    int vslot[NV];
    if constexpr (UNIFORM) {
      // block_size % 16 == 0: each 16-token half lies in one block, so one
      // (wave-uniform, scalar) table lookup per half.
      int phys[2], off[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tb = t0 + 16 * hh;
        phys[hh] = 0;
        off[hh] = 0;
        if (tb < t_end) {
          const int lb = tb / bs;
          phys[hh] = trow[lb];
          off[hh] = tb - lb * bs;
        }
        kslot[hh] = phys[hh] * bs + off[hh] + c;
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int tv = lane / PPR + v * TOK_PER_V;
        const int hh = (v * TOK_PER_V) >> 4;
        vslot[v] = phys[hh] * bs + off[hh] + (tv & 15);
      }
    } else {
      const int tok = t0 + (lane & 31);
      int myslot = 0;
      if (tok < t_end) {
        const int lb = tok / bs;
        myslot = trow[lb] * bs + (tok - lb * bs);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kslot[hh] = __shfl(myslot, 16 * hh + c, 64);
#pragma unroll
      for (int v = 0; v < NV; ++v)
        vslot[v] = __shfl(myslot, lane / PPR + v * TOK_PER_V, 64);
    }

    // ---------------- loads (masked past the end) ----------------
    uint32_t kw[2][KWORDS];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bool ok = t0 + 16 * hh + c < t_end;
      const uint8_t* row = kbase + (int64_t)kslot[hh] * slot_stride;
#pragma unroll
      for (int r = 0; r < KPIECES; ++r) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (ok) v = *reinterpret_cast<const u32x4_t*>(row + (4 * r + j) * 16);
        kw[hh][4 * r + 0] = v[0];
        kw[hh][4 * r + 1] = v[1];
        kw[hh][4 * r + 2] = v[2];
        kw[hh][4 * r + 3] = v[3];
      }
    }
    u32x4_t vraw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int tv = lane / PPR + v * TOK_PER_V;
      vraw[v] = u32x4_t{0u, 0u, 0u, 0u};
      if (t0 + tv < t_end)
        vraw[v] = *reinterpret_cast<const u32x4_t*>(
            vbase + (int64_t)vslot[v] * slot_stride + (lane % PPR) * 16);
    }

    // ---------------- S = K . Q^T ----------------
    f32x4_t sacc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      sacc[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < QSTEPS; ++st) {
        typename Mma<QT>::operand ka, qb;
        if constexpr (same<QT, CT>::value && QT::bytes == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            ka[w] = kw[hh][4 * st + w];
            qb[w] = qw[4 * st + w];
          }
        } else if constexpr (same<QT, CT>::value) {  // float32
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ka[e] = bitcast<float>(kw[hh][8 * st + e]);
            qb[e] = bitcast<float>(qw[8 * st + e]);
          }
        } else if constexpr (QT::bytes == 2) {  // fp8 keys -> bf16/f16
          const uint32_t w0 = kw[hh][2 * st], w1 = kw[hh][2 * st + 1];
          if constexpr (same<QT, BF16>::value) {
            ka[0] = fp8x2_to_bf16x2(w0, false);
            ka[1] = fp8x2_to_bf16x2(w0, true);
            ka[2] = fp8x2_to_bf16x2(w1, false);
            ka[3] = fp8x2_to_bf16x2(w1, true);
          } else {
            ka[0] = fp8x2_to_f16x2(w0, false);
            ka[1] = fp8x2_to_f16x2(w0, true);
            ka[2] = fp8x2_to_f16x2(w1, false);
            ka[3] = fp8x2_to_f16x2(w1, true);
          }
#pragma unroll
          for (int w = 0; w < 4; ++w) qb[w] = qw[4 * st + w];
        } else {  // fp8 keys -> f32
          const uint32_t w0 = kw[hh][2 * st], w1 = kw[hh][2 * st + 1];
          const f32x2_t p0 = fp8x2_to_f32x2(w0, false), p1 = fp8x2_to_f32x2(w0, true);
          const f32x2_t p2 = fp8x2_to_f32x2(w1, false), p3 = fp8x2_to_f32x2(w1, true);
          ka[0] = p0[0]; ka[1] = p0[1]; ka[2] = p1[0]; ka[3] = p1[1];
          ka[4] = p2[0]; ka[5] = p2[1]; ka[6] = p3[0]; ka[7] = p3[1];
#pragma unroll
          for (int e = 0; e < 8; ++e) qb[e] = bitcast<float>(qw[8 * st + e]);
        }
        sacc[hh] = Mma<QT>::step(ka, qb, sacc[hh]);
      }
    }

    // ---------------- online softmax (log2 domain) ----------------
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float raw = e < 4 ? sacc[0][e] : sacc[1][e - 4];
      sv[e] = (t0 + slot_token(j, e) < t_end) ? raw * qk_mul : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = fast_exp2(sv[e] - m_new);
      psum += pv[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int n = 0; n < NBLK; ++n) oacc[n] *= alpha;

    // ---------------- V -> LDS (PV operand type, swizzled) ----------------
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int tv = lane / PPR + v * TOK_PER_V;
      const int swz = ((tv >> 2) & 3) * PVB;
      uint8_t* rowp = vt + tv * LDS_ROW;
      const int ch0 = (lane % PPR) * VCH;
      if constexpr (same<PVT, CT>::value) {
        *reinterpret_cast<u32x4_t*>(rowp + ((ch0 ^ swz) << 4)) = vraw[v];
      } else if constexpr (PVB == 2) {  // fp8 -> f16, two chunks
        u32x4_t lo, hi;
        lo[0] = fp8x2_to_f16x2(vraw[v][0], false);
        lo[1] = fp8x2_to_f16x2(vraw[v][0], true);
        lo[2] = fp8x2_to_f16x2(vraw[v][1], false);
        lo[3] = fp8x2_to_f16x2(vraw[v][1], true);
        hi[0] = fp8x2_to_f16x2(vraw[v][2], false);
        hi[1] = fp8x2_to_f16x2(vraw[v][2], true);
        hi[2] = fp8x2_to_f16x2(vraw[v][3], false);
        hi[3] = fp8x2_to_f16x2(vraw[v][3], true);
        *reinterpret_cast<u32x4_t*>(rowp + (((ch0 + 0) ^ swz) << 4)) = lo;
        *reinterpret_cast<u32x4_t*>(rowp + (((ch0 + 1) ^ swz) << 4)) = hi;
      } else {  // fp8 -> f32, four chunks
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x2_t p0 = fp8x2_to_f32x2(vraw[v][w], false);
          const f32x2_t p1 = fp8x2_to_f32x2(vraw[v][w], true);
          f32x4_t q = {p0[0], p0[1], p1[0], p1[1]};
          *reinterpret_cast<f32x4_t*>(rowp + (((ch0 + w) ^ swz) << 4)) = q;
        }
      }
    }
    __syncthreads();

    // ---------------- O^T += V^T . P^T ----------------
    typename Mma<PVT>::operand pb_hi, pb_lo;
    if constexpr (PVB == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t h0 = f32_to_bits(pv[2 * w], PVT{});
        const uint32_t h1 = f32_to_bits(pv[2 * w + 1], PVT{});
        pb_hi[w] = h0 | (h1 << 16);
        if constexpr (PSPLIT) {
          const uint32_t l0 = f32_to_bits(pv[2 * w] - bits_to_f32(h0, PVT{}), PVT{});
          const uint32_t l1 = f32_to_bits(pv[2 * w + 1] - bits_to_f32(h1, PVT{}), PVT{});
          pb_lo[w] = l0 | (l1 << 16);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pb_hi[e] = pv[e];
    }
    const int swz_j = j * PVB;
#pragma unroll
    for (int n = 0; n < NBLK; ++n) {
      const int byte = (16 * n + c) * PVB;
      const int col = (((byte >> 4) ^ swz_j) << 4) + (byte & 15);
      typename Mma<PVT>::operand va;
      if constexpr (PVB == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t e0 = *reinterpret_cast<const uint16_t*>(
              vt + slot_token(j, 2 * w) * LDS_ROW + col);
          const uint32_t e1 = *reinterpret_cast<const uint16_t*>(
              vt + slot_token(j, 2 * w + 1) * LDS_ROW + col);
          va[w] = e0 | (e1 << 16);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          va[e] = *reinterpret_cast<const float*>(vt + slot_token(j, e) * LDS_ROW + col);
      }
      oacc[n] = Mma<PVT>::step(va, pb_hi, oacc[n]);
      if constexpr (PSPLIT) oacc[n] = Mma<PVT>::step(va, pb_lo, oacc[n]);
    }
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  float l_tot = xor_sum(l_run, 16);
  l_tot = xor_sum(l_tot, 32);

  if (nparts == 1) {
    if (head_live) {
      const float inv = l_tot > 0.f ? vscale / l_tot : 0.f;
      float* dst = a.out + ((int64_t)s * a.num_q_heads + hq) * D + 4 * j;
#pragma unroll
      for (int n = 0; n < NBLK; ++n) {
        f32x4_t o = oacc[n];
        if (l_tot > 0.f) {
          o[0] = o[0] / l_tot * vscale;
          o[1] = o[1] / l_tot * vscale;
          o[2] = o[2] / l_tot * vscale;
          o[3] = o[3] / l_tot * vscale;
        } else {
          o = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        (void)inv;
        *reinterpret_cast<f32x4_t*>(dst + 16 * n) = o;
      }
    }
    return;
  }

  const int64_t prow = ((int64_t)s * a.num_q_heads + hq) * a.max_parts + part;
  if (head_live) {
    float* dst = a.part_o + prow * D + 4 * j;
#pragma unroll
    for (int n = 0; n < NBLK; ++n) *reinterpret_cast<f32x4_t*>(dst + 16 * n) = oacc[n];
    if (j == 0) {
      a.part_m[prow] = m_run;
      a.part_l[prow] = l_tot;
    }
  }
  __threadfence();
  uint32_t* counter =
      a.counters + ((int64_t)s * a.num_kv_heads + h) * a.group_chunks + gc;
  uint32_t prev = 0;
  if (lane == 0) prev = atomicAdd(counter, 1u);
  prev = __shfl(prev, 0, 64);
  if (prev != (uint32_t)(nparts - 1)) return;
  __threadfence();
  merge_partials<D>(a, s, h, gc, gcount, nparts, vscale);
  if (lane == 0) atomicExch(counter, 0u);
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
static hipError_t launch_d(const AttnArgs& a, int grid, bool uniform,
                           hipStream_t stream) {
  if (uniform)
    hipLaunchKernelGGL((attn_decode_kernel<QT, CT, D, true>), dim3(grid),
                       dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<QT, CT, D, false>), dim3(grid),
                       dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <typename QT, typename CT>
static hipError_t launch_t(const AttnArgs& a, int head_dim, int grid,
                           bool uniform, hipStream_t stream) {
  if (head_dim == 64) return launch_d<QT, CT, 64>(a, grid, uniform, stream);
  return launch_d<QT, CT, 128>(a, grid, uniform, stream);
}

hipError_t launch_attn_decode(const AttnArgs& a, int q_dtype, int cache_dtype,
                              int head_dim, int grid, hipStream_t stream) {
  const bool uniform = (a.block_size % 16) == 0;
  switch (cache_dtype) {
    case PKV_F32: return launch_t<F32, F32>(a, head_dim, grid, uniform, stream);
    case PKV_F16: return launch_t<F16, F16>(a, head_dim, grid, uniform, stream);
    case PKV_BF16: return launch_t<BF16, BF16>(a, head_dim, grid, uniform, stream);
    case PKV_FP8_E4M3:
      if (q_dtype == PKV_BF16) return launch_t<BF16, FP8>(a, head_dim, grid, uniform, stream);
      if (q_dtype == PKV_F16) return launch_t<F16, FP8>(a, head_dim, grid, uniform, stream);
      return launch_t<F32, FP8>(a, head_dim, grid, uniform, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
