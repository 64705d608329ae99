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
// reading h, partition p of the sequence), one 256-thread workgroup (4 waves)
// per unit, so each K/V row of a kv head is read once for all query heads
// that share it.  The partition's 32-token tiles are dealt round-robin to the
// 4 waves; each wave keeps its own online-softmax state and the waves combine
// theirs through LDS at the end.
//
// Per 32-token tile (one wave):
//   * Block-table entries are read with wave-uniform (scalar) loads, one per
//     16-token half-tile when bs % 16 == 0.  The half-tile's base address then
//     lives in SGPRs as a buffer resource whose size covers exactly the live
//     rows, so rows past the end of the sequence are neither fetched nor need
//     a branch, and the next tile's rows are requested before the current one
//     is computed.
//   * K rows go straight from HBM into MFMA A-operand registers as 16-byte
//     loads (lane = token row + 16 * piece group), Q sits in the B operand;
//     S = K . Q^T on v_mfma_f32_16x16x32 (bf16/f16; fp8 keys are decoded to
//     the query's type first) or eight 16x16x4 f32 steps.
//   * Scores are scaled into the log2 domain; the running max uses xor
//     shuffles across the 4 lanes that hold one query head's column.
//   * V rows are loaded as 16-byte pieces, converted to the PV operand type
//     and staged in the wave's own LDS slice (XOR-swizzled 16-byte chunks),
//     then read back transposed as the A operand of O^T += V^T . P^T, so P
//     never leaves the registers the QK product left it in.  For bf16/f16
//     caches P is split into a high and a low part (two MFMAs), which keeps
//     the weights exact to ~2^-16 relative.
//
// Partitions: a sequence longer than one partition writes an unnormalised
// partial (o, running max m, running sum l) per query head to the workspace,
// and a second kernel, one workgroup per (sequence, query head), merges them:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// The kernel boundary is what makes one partition's writes visible to the
// merging workgroup; an in-kernel hand-off would need a device-scope fence in
// every partition's workgroup, which on this part writes back a whole L2 and
// costs far more than the second launch.  Reduction order depends only on
// logical token positions, so relabelling physical blocks leaves the output
// bit-identical.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kRawBufferFlags = 0x00020000;  // dword3: 32-bit data format

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

// Compile-time shape of one (query type, cache type, head_dim) instance.
template <typename QT, typename CT, int D> struct Shape {
  typedef typename PvOperand<QT, CT>::type PVT;
  static constexpr bool PSPLIT = !is_fp8<CT>::value && CT::bytes == 2;
  static constexpr int EP = 16 / CT::bytes;           // elements per piece
  static constexpr int KPIECES = D * CT::bytes / 64;  // K pieces/lane/half
  static constexpr int KWORDS = KPIECES * 4;
  static constexpr int QSTEPS = D / 32;               // k32 steps over D
  static constexpr int ROW_BYTES = D * CT::bytes;     // one token, one head
  static constexpr int PPR = ROW_BYTES / 16;          // pieces per row
  static constexpr int NV = PPR / 2;                  // V pieces/lane/tile
  static constexpr int TOK_PER_V = 64 / PPR;
  static constexpr int PVB = PVT::bytes;
  static constexpr int LDS_ROW = D * PVB;
  static constexpr int VCH = EP * PVB / 16;           // LDS chunks per piece
  static constexpr int QWORDS = D / 4 * QT::bytes / 4;
  static constexpr int NBLK = D / 16;                 // 16-wide output blocks
  static constexpr int STAGE_BYTES = 32 * LDS_ROW;    // V tile, one wave
  static constexpr int ORow = D + 4;                  // padded LDS row (floats)
  static constexpr int COMBINE_BYTES = kWaves * 16 * ORow * 4;
  static constexpr int SMEM_BYTES = kWaves * STAGE_BYTES > COMBINE_BYTES
                                        ? kWaves * STAGE_BYTES
                                        : COMBINE_BYTES;
  static_assert(NV >= 1 && KPIECES >= 1, "head_dim too small");
  static_assert(LDS_ROW / 16 >= 4 * PVB, "swizzle needs 4 distinct spans");
  static_assert(16 % TOK_PER_V == 0, "a V load must not straddle halves");
};

// One tile's raw K and V bytes as loaded from the pool.
template <typename QT, typename CT, int D> struct TileRegs {
  typedef Shape<QT, CT, D> S;
  uint32_t kw[2][S::KWORDS];
  u32x4_t vraw[S::NV];
};

// Online-softmax state of one wave: running max (log2 domain) and this
// lane's share of the running sum for query head column c, and O^T blocks.
template <int NBLK> struct WaveState {
  float m;
  float l;
  f32x4_t o[NBLK];
};

// ---------------------------------------------------------------------------
// Tile loads, block_size % 16 == 0: one table entry per 16-token half, rows
// addressed through a buffer resource spanning the half's live rows only
// (rows past the sequence end read as zero and are never fetched).  tab is
// the partition's window of the block table, staged in LDS, whose entry 0 is
// logical block lb_first; reading it there keeps the table lookups off the
// vector-memory counter, so waiting for one never drains the prefetch.
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
__device__ __forceinline__ void load_tile_uniform(
    TileRegs<QT, CT, D>& tr, const AttnArgs& a, const int32_t* tab,
    int lb_first, const uint8_t* kbase, const uint8_t* vbase, int64_t stride,
    int t0, int t_end, int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int bs = a.block_size;
  // Everything addressing the half-tile is wave-uniform; readfirstlane says
  // so to the compiler, which keeps it in SGPRs (scalar table loads, buffer
  // resources in SGPRs) instead of looping over lanes.
  t0 = __builtin_amdgcn_readfirstlane(t0);
  __amdgpu_buffer_rsrc_t kr[2], vr[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int tb = t0 + 16 * hh;
    int nvalid = t_end - tb;
    nvalid = nvalid < 0 ? 0 : (nvalid > 16 ? 16 : nvalid);
    int64_t row0 = 0;
    if (nvalid > 0) {
      const int lb = tb / bs;
      const int phys = __builtin_amdgcn_readfirstlane(tab[lb - lb_first]);
      row0 = (int64_t)phys * bs + (tb - lb * bs);
    }
    // (the clamp above may be selected as a vector min/max)
    const int nrec = __builtin_amdgcn_readfirstlane(nvalid * (int)stride);
    kr[hh] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kbase + row0 * stride), (short)0, nrec,
        kRawBufferFlags);
    vr[hh] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(vbase + row0 * stride), (short)0, nrec,
        kRawBufferFlags);
  }
  const int kofs = c * (int)stride + j * 16;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int r = 0; r < S::KPIECES; ++r) {
      const u32x4_t v =
          __builtin_amdgcn_raw_buffer_load_b128(kr[hh], kofs + r * 64, 0, 0);
      tr.kw[hh][4 * r + 0] = v[0];
      tr.kw[hh][4 * r + 1] = v[1];
      tr.kw[hh][4 * r + 2] = v[2];
      tr.kw[hh][4 * r + 3] = v[3];
    }
  }
  const int vtok = lane / S::PPR;
  const int vofs = vtok * (int)stride + (lane % S::PPR) * 16;
#pragma unroll
  for (int v = 0; v < S::NV; ++v) {
    const int hh = (v * S::TOK_PER_V) >> 4;
    const int tin = (v * S::TOK_PER_V) & 15;
    // the whole offset goes in the per-lane operand: the range check covers it
    tr.vraw[v] = __builtin_amdgcn_raw_buffer_load_b128(
        vr[hh], vofs + tin * (int)stride, 0, 0);
  }
}

// Tile loads for any block size: one table lookup per token (vector), masked
// lanes skip the load and hold zeros.
template <typename QT, typename CT, int D>
__device__ __forceinline__ void load_tile_any(
    TileRegs<QT, CT, D>& tr, const AttnArgs& a, const int32_t* trow,
    const uint8_t* kbase, const uint8_t* vbase, int64_t stride, int t0,
    int t_end, int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int bs = a.block_size;
  const int tok = t0 + (lane & 31);
  int myslot = 0;
  if (tok < t_end) {
    const int lb = tok / bs;
    myslot = trow[lb] * bs + (tok - lb * bs);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int ks = __shfl(myslot, 16 * hh + c, 64);
    const bool ok = t0 + 16 * hh + c < t_end;
    const uint8_t* row = kbase + (int64_t)ks * stride;
#pragma unroll
    for (int r = 0; r < S::KPIECES; ++r) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4_t*>(row + (4 * r + j) * 16);
      tr.kw[hh][4 * r + 0] = v[0];
      tr.kw[hh][4 * r + 1] = v[1];
      tr.kw[hh][4 * r + 2] = v[2];
      tr.kw[hh][4 * r + 3] = v[3];
    }
  }
#pragma unroll
  for (int v = 0; v < S::NV; ++v) {
    const int tv = lane / S::PPR + v * S::TOK_PER_V;
    const int vs = __shfl(myslot, tv, 64);
    tr.vraw[v] = u32x4_t{0u, 0u, 0u, 0u};
    if (t0 + tv < t_end)
      tr.vraw[v] = *reinterpret_cast<const u32x4_t*>(
          vbase + (int64_t)vs * stride + (lane % S::PPR) * 16);
  }
}

// ---------------------------------------------------------------------------
// One tile: S = K Q^T, online-softmax update, O^T += V^T P^T.
// vt is this wave's LDS slice (32 rows of D PV-operand elements).
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
__device__ __forceinline__ void compute_tile(
    const TileRegs<QT, CT, D>& tr, const uint32_t* qw,
    WaveState<Shape<QT, CT, D>::NBLK>& st, uint8_t* vt, int t0, int t_end,
    float qk_mul, int lane) {
  typedef Shape<QT, CT, D> S;
  typedef typename S::PVT PVT;
  constexpr int PVB = S::PVB;
  const int c = lane & 15;
  const int j = lane >> 4;

  // ---------------- S = K . Q^T ----------------
  f32x4_t sacc[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    sacc[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < S::QSTEPS; ++q) {
      typename Mma<QT>::operand ka, qb;
      if constexpr (same<QT, CT>::value && QT::bytes == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ka[w] = tr.kw[hh][4 * q + w];
          qb[w] = qw[4 * q + w];
        }
      } else if constexpr (same<QT, CT>::value) {  // float32
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ka[e] = bitcast<float>(tr.kw[hh][8 * q + e]);
          qb[e] = bitcast<float>(qw[8 * q + e]);
        }
      } else if constexpr (QT::bytes == 2) {  // fp8 keys -> bf16/f16
        const uint32_t w0 = tr.kw[hh][2 * q], w1 = tr.kw[hh][2 * q + 1];
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
        for (int w = 0; w < 4; ++w) qb[w] = qw[4 * q + w];
      } else {  // fp8 keys -> f32
        const uint32_t w0 = tr.kw[hh][2 * q], w1 = tr.kw[hh][2 * q + 1];
        const f32x2_t p0 = fp8x2_to_f32x2(w0, false), p1 = fp8x2_to_f32x2(w0, true);
        const f32x2_t p2 = fp8x2_to_f32x2(w1, false), p3 = fp8x2_to_f32x2(w1, true);
        ka[0] = p0[0]; ka[1] = p0[1]; ka[2] = p1[0]; ka[3] = p1[1];
        ka[4] = p2[0]; ka[5] = p2[1]; ka[6] = p3[0]; ka[7] = p3[1];
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[e] = bitcast<float>(qw[8 * q + e]);
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
  const float m_new = fmaxf(st.m, mx);
  const float alpha = fast_exp2(st.m - m_new);
  float pv[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = fast_exp2(sv[e] - m_new);
    psum += pv[e];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
#pragma unroll
  for (int n = 0; n < S::NBLK; ++n) st.o[n] *= alpha;

  // ---------------- V -> LDS (PV operand type, swizzled) ----------------
#pragma unroll
  for (int v = 0; v < S::NV; ++v) {
    const int tv = lane / S::PPR + v * S::TOK_PER_V;
    const int swz = ((tv >> 2) & 3) * PVB;
    uint8_t* rowp = vt + tv * S::LDS_ROW;
    const int ch0 = (lane % S::PPR) * S::VCH;
    if constexpr (same<PVT, CT>::value) {
      *reinterpret_cast<u32x4_t*>(rowp + ((ch0 ^ swz) << 4)) = tr.vraw[v];
    } else if constexpr (PVB == 2) {  // fp8 -> f16, two chunks
      u32x4_t lo, hi;
      lo[0] = fp8x2_to_f16x2(tr.vraw[v][0], false);
      lo[1] = fp8x2_to_f16x2(tr.vraw[v][0], true);
      lo[2] = fp8x2_to_f16x2(tr.vraw[v][1], false);
      lo[3] = fp8x2_to_f16x2(tr.vraw[v][1], true);
      hi[0] = fp8x2_to_f16x2(tr.vraw[v][2], false);
      hi[1] = fp8x2_to_f16x2(tr.vraw[v][2], true);
      hi[2] = fp8x2_to_f16x2(tr.vraw[v][3], false);
      hi[3] = fp8x2_to_f16x2(tr.vraw[v][3], true);
      *reinterpret_cast<u32x4_t*>(rowp + (((ch0 + 0) ^ swz) << 4)) = lo;
      *reinterpret_cast<u32x4_t*>(rowp + (((ch0 + 1) ^ swz) << 4)) = hi;
    } else {  // fp8 -> f32, four chunks
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2_t p0 = fp8x2_to_f32x2(tr.vraw[v][w], false);
        const f32x2_t p1 = fp8x2_to_f32x2(tr.vraw[v][w], true);
        f32x4_t q = {p0[0], p0[1], p1[0], p1[1]};
        *reinterpret_cast<f32x4_t*>(rowp + (((ch0 + w) ^ swz) << 4)) = q;
      }
    }
  }
  // The slice is private to this wave and one wave's LDS operations execute
  // in issue order, so the transposed reads below see these stores with no
  // barrier (the compiler keeps the may-alias store -> load order).

  // ---------------- O^T += V^T . P^T ----------------
  typename Mma<PVT>::operand pb_hi, pb_lo;
  if constexpr (PVB == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t h0 = f32_to_bits(pv[2 * w], PVT{});
      const uint32_t h1 = f32_to_bits(pv[2 * w + 1], PVT{});
      pb_hi[w] = h0 | (h1 << 16);
      if constexpr (S::PSPLIT) {
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
  for (int n = 0; n < S::NBLK; ++n) {
    const int byte = (16 * n + c) * PVB;
    const int col = (((byte >> 4) ^ swz_j) << 4) + (byte & 15);
    typename Mma<PVT>::operand va;
    if constexpr (PVB == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t e0 = *reinterpret_cast<const uint16_t*>(
            vt + slot_token(j, 2 * w) * S::LDS_ROW + col);
        const uint32_t e1 = *reinterpret_cast<const uint16_t*>(
            vt + slot_token(j, 2 * w + 1) * S::LDS_ROW + col);
        va[w] = e0 | (e1 << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        va[e] = *reinterpret_cast<const float*>(vt + slot_token(j, e) * S::LDS_ROW + col);
    }
    st.o[n] = Mma<PVT>::step(va, pb_hi, st.o[n]);
    if constexpr (S::PSPLIT) st.o[n] = Mma<PVT>::step(va, pb_lo, st.o[n]);
  }
}

// ---------------------------------------------------------------------------
// Merge of the partitions of one (sequence, query head): one workgroup.
// Threads take 4 output columns each and a strided subset of the partitions
// (D/4 columns x kThreads/(D/4) subsets); subsets are summed through LDS.
// ---------------------------------------------------------------------------
template <int D, bool SCALED>
__global__ __launch_bounds__(kThreads) void attn_merge_kernel(AttnArgs a) {
  constexpr int D4 = D / 4;
  constexpr int NSUB = kThreads / D4;
  __shared__ __attribute__((aligned(16))) float red[NSUB][D];
  __shared__ float sm_red[2][kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hq = blockIdx.x % a.num_q_heads;
  const int s = blockIdx.x / a.num_q_heads;
  const int L = a.seq_lens[s];
  const int nparts = L > 0 ? (L + a.partition_size - 1) / a.partition_size : 1;
  if (nparts <= 1) return;  // written directly by the partition kernel

  const int64_t row = (int64_t)s * a.num_q_heads + hq;
  const auto* pm = as_global(a.part_m + row * a.max_parts);
  const auto* pl = as_global(a.part_l + row * a.max_parts);
  const auto* po = as_global(a.part_o + row * a.max_parts * D);

  // M = max_p m_p
  float M = -INFINITY;
  for (int q = tid; q < nparts; q += kThreads) M = fmaxf(M, pm[q]);
  M = wave_max(M);
  if (lane == 0) sm_red[0][wave] = M;
  __syncthreads();
  M = sm_red[0][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_red[0][w]);

  // den = sum_p 2^(m_p - M) l_p ; acc = sum_p 2^(m_p - M) o_p
  float den = 0.f;
  for (int q = tid; q < nparts; q += kThreads) den += fast_exp2(pm[q] - M) * pl[q];
  den = wave_sum(den);
  if (lane == 0) sm_red[1][wave] = den;

  const int d4 = tid % D4;
  const int sub = tid / D4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int q = sub;
  for (; q + 3 * NSUB < nparts; q += 4 * NSUB) {
    float w[4];
    f32x4_t o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = pm[q + u * NSUB];
      o[u] = *reinterpret_cast<const __attribute__((address_space(1))) f32x4_t*>(
          po + (int64_t)(q + u * NSUB) * D + 4 * d4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += fast_exp2(w[u] - M) * o[u];
  }
  for (; q < nparts; q += NSUB)
    acc += fast_exp2(pm[q] - M) *
           *reinterpret_cast<const __attribute__((address_space(1))) f32x4_t*>(
               po + (int64_t)q * D + 4 * d4);
  *reinterpret_cast<f32x4_t*>(&red[sub][4 * d4]) = acc;
  __syncthreads();

  if (tid < D4) {
    den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) den += sm_red[1][w];
    f32x4_t o = *reinterpret_cast<const f32x4_t*>(&red[0][4 * tid]);
#pragma unroll
    for (int u = 1; u < NSUB; ++u)
      o += *reinterpret_cast<const f32x4_t*>(&red[u][4 * tid]);
    const float vscale = SCALED ? *a.v_scale : 1.f;
    *reinterpret_cast<f32x4_t*>(a.out + row * D + 4 * tid) = o * (vscale / den);
  }
}

template <typename QT, typename CT, int D, bool UNIFORM>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(AttnArgs a) {
  typedef Shape<QT, CT, D> S;
  constexpr int NBLK = S::NBLK;
  constexpr bool PREFETCH = UNIFORM && CT::bytes <= 2;

  __shared__ __attribute__((aligned(16))) uint8_t smem[S::SMEM_BYTES];
  __shared__ float sm_ml[kWaves][2][16];
  __shared__ float sm_stat[32];
  __shared__ int32_t sm_tab[UNIFORM ? kMaxTableWindow : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
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
  const int ntiles = (t_end - t_begin + 31) / 32;
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
  uint32_t qw[S::QWORDS];
  {
    const uint8_t* qrow = static_cast<const uint8_t*>(a.query) +
                          ((int64_t)s * a.num_q_heads + hq) * D * QT::bytes;
    constexpr int QBYTES_PER_R = S::EP * QT::bytes;
    constexpr int QLOADS = QBYTES_PER_R / 16;
#pragma unroll
    for (int r = 0; r < D / (4 * S::EP); ++r) {
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
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) +
                         (int64_t)h * S::ROW_BYTES;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) +
                         (int64_t)h * S::ROW_BYTES;
  const int64_t stride = (int64_t)a.num_kv_heads * S::ROW_BYTES;
  uint8_t* vt = smem + wave * S::STAGE_BYTES;

  int lb_first = 0;
  if constexpr (UNIFORM) {
    // the partition's block-table entries, once per workgroup
    if (t_end > t_begin) {
      lb_first = t_begin / a.block_size;
      const int count = (t_end - 1) / a.block_size - lb_first + 1;
      for (int i = tid; i < count; i += kThreads)
        sm_tab[i] = trow[lb_first + i];
    }
    __syncthreads();
  }

  WaveState<NBLK> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int n = 0; n < NBLK; ++n) st.o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (PREFETCH) {
    // Loads of tile k + kWaves are in flight while tile k is computed; past
    // the last tile the buffer ranges are empty, so those loads fetch
    // nothing and the loop needs no branch around them.
    TileRegs<QT, CT, D> cur, nxt;
    load_tile_uniform<QT, CT, D>(cur, a, sm_tab, lb_first, kbase, vbase,
                                 stride, t_begin + 32 * wave, t_end, lane);
    for (int k = wave; k < ntiles; k += kWaves) {
      load_tile_uniform<QT, CT, D>(nxt, a, sm_tab, lb_first, kbase, vbase,
                                   stride, t_begin + 32 * (k + kWaves), t_end,
                                   lane);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of compute
      compute_tile<QT, CT, D>(cur, qw, st, vt, t_begin + 32 * k, t_end,
                              qk_mul, lane);
      cur = nxt;
    }
  } else {
    for (int k = wave; k < ntiles; k += kWaves) {
      TileRegs<QT, CT, D> cur;
      if constexpr (UNIFORM)
        load_tile_uniform<QT, CT, D>(cur, a, sm_tab, lb_first, kbase, vbase,
                                     stride, t_begin + 32 * k, t_end, lane);
      else
        load_tile_any<QT, CT, D>(cur, a, trow, kbase, vbase, stride,
                                 t_begin + 32 * k, t_end, lane);
      compute_tile<QT, CT, D>(cur, qw, st, vt, t_begin + 32 * k, t_end,
                              qk_mul, lane);
    }
  }

  // ---------------- combine the waves' states ----------------
  float l_w = xor_sum(st.l, 16);
  l_w = xor_sum(l_w, 32);
  if (j == 0) {
    sm_ml[wave][0][c] = st.m;
    sm_ml[wave][1][c] = l_w;
  }
  __syncthreads();  // also: every wave is done with its V slice
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_ml[w][0][c]);
  float Ltot = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      Ltot += fast_exp2(sm_ml[w][0][c] - M) * sm_ml[w][1][c];
  }
  const float f = (st.m == -INFINITY) ? 0.f : fast_exp2(st.m - M);
  float* so = reinterpret_cast<float*>(smem);
  if (head_live) {
    float* dst = so + (wave * 16 + c) * S::ORow + 4 * j;
#pragma unroll
    for (int n = 0; n < NBLK; ++n)
      *reinterpret_cast<f32x4_t*>(dst + 16 * n) = st.o[n] * f;
  }
  if (wave == 0 && j == 0) {  // per-head totals for the output pass
    sm_stat[2 * c] = M;
    sm_stat[2 * c + 1] = Ltot;
  }
  __syncthreads();

  constexpr int D4 = D / 4;
  const int items = gcount * D4;
  const int64_t head0 = (int64_t)s * a.num_q_heads + h * a.group + gc * 16;
  if (nparts == 1) {
    for (int it = tid; it < items; it += kThreads) {
      const int g = it / D4;
      const int d4 = it - g * D4;
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        o += *reinterpret_cast<const f32x4_t*>(so + (w * 16 + g) * S::ORow + 4 * d4);
      const float lt = sm_stat[2 * g + 1];
      o = lt > 0.f ? o * (vscale / lt) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4_t*>(a.out + (head0 + g) * D + 4 * d4) = o;
    }
    return;
  }

  for (int it = tid; it < items; it += kThreads) {
    const int g = it / D4;
    const int d4 = it - g * D4;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      o += *reinterpret_cast<const f32x4_t*>(so + (w * 16 + g) * S::ORow + 4 * d4);
    const int64_t prow = (head0 + g) * a.max_parts + part;
    *reinterpret_cast<f32x4_t*>(a.part_o + prow * D + 4 * d4) = o;
    if (d4 == 0) {
      a.part_m[prow] = sm_stat[2 * g];
      a.part_l[prow] = sm_stat[2 * g + 1];
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
static hipError_t launch_d(const AttnArgs& a, int grid, bool uniform,
                           hipStream_t stream) {
  if (uniform)
    hipLaunchKernelGGL((attn_decode_kernel<QT, CT, D, true>), dim3(grid),
                       dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<QT, CT, D, false>), dim3(grid),
                       dim3(kThreads), 0, stream, a);
  if (a.max_parts > 1)
    hipLaunchKernelGGL((attn_merge_kernel<D, is_fp8<CT>::value>),
                       dim3(a.num_seqs * a.num_q_heads), dim3(kThreads), 0,
                       stream, a);
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
