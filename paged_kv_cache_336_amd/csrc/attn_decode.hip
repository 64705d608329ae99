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
// Work split: a row is (sequence s, kv head h, chunk of <= 16 query heads of
// the group reading h); a row's tiles are 32 consecutive tokens.  All tiles
// of all rows, in row-major order, are divided into equal contiguous ranges,
// one per wave of a grid that fills the GPU once, so every wave streams the
// same number of K/V bytes whatever the mix of sequence lengths.  Each K/V row
// of a kv head is read once, by one wave, for all query heads that share it,
// and waves never wait for one another while streaming.
//
// Per 32-token tile (one wave):
//   * When bs % 16 == 0 each wave holds a 128-entry window of its row's
//     block table in two VGPRs and reads one entry per 16-token half-tile
//     with a wave-uniform readlane.  The half-tile's base address then lives in SGPRs as a
//     buffer resource whose size covers exactly the live rows, so rows past
//     the end of the sequence are neither fetched nor need a branch, and the
//     next tile's rows are requested before the current one is computed.
//   * K rows go straight from HBM into MFMA A-operand registers as 16-byte
//     loads (lane = token row + 16 * piece group), Q sits in the B operand;
//     S = K . Q^T on v_mfma_f32_16x16x32 (bf16/f16; fp8 keys are decoded to
//     the query's type first) or eight 16x16x4 f32 steps.
//   * Scores are scaled into the log2 domain; the running max uses xor
//     shuffles across the 4 lanes that hold one query head's column.
//   * V rows are loaded as 16-byte pieces, converted to the PV operand type
//     and staged in the wave's own LDS slice (32-byte spans permuted per
//     token), then read back with gfx950's transposing LDS read as the A
//     operand of O^T += V^T . P^T, so P never leaves the registers the QK
//     product left it in.  For bf16/f16
//     caches P is split into a high and a low part (two MFMAs), which keeps
//     the weights exact to ~2^-16 relative.
//
// Splits: a row that one wave's range covers entirely is finished by that
// wave.  A row cut by range boundaries gets a partial (o, running max m,
// running sum l) per piece -- a wave holds at most two such pieces, its first
// and its last row -- and a second kernel, one workgroup per cut row, merges
// them:  M = max m_i,  out = sum 2^(m_i - M) o_i / sum 2^(m_i - M) l_i.
// The kernel boundary is what makes the pieces visible to the merging
// workgroup (an in-kernel hand-off would need a device-scope fence per wave,
// which on this part writes back a whole L2).  Reduction order depends only
// on logical token positions and the grid size, so relabelling physical
// blocks leaves the output bit-identical.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kWorkgroupsPerCU = 1;       // default grid: one workgroup per CU
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
  static constexpr int STAGE_BYTES = 32 * LDS_ROW;    // V sub-tile, one wave
  static constexpr int SPANS = LDS_ROW / 32;          // 32-byte spans per row
  // A tile -- the unit of the split and of each load request -- is SUB
  // 32-token sub-tiles (the MFMA tile).  One sub-tile per request measured
  // fastest: larger requests deepen the memory queues and push the loop's
  // registers into spills without adding bandwidth.
  static constexpr int SUB = 1;
  static constexpr int TT = 32 * SUB;                 // tokens per tile
  static_assert(NV >= 1 && KPIECES >= 1, "head_dim too small");
  static_assert(LDS_ROW / 16 >= 4 * PVB, "swizzle needs 4 distinct spans");
  static_assert(16 % TOK_PER_V == 0, "a V load must not straddle halves");
};

// One tile's raw K and V bytes as loaded from the pool, per sub-tile.
template <typename QT, typename CT, int D> struct TileRegs {
  typedef Shape<QT, CT, D> S;
  uint32_t kw[S::SUB][2][S::KWORDS];
  u32x4_t vraw[S::SUB][S::NV];
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
// (rows past the end read as zero and are never fetched, so an empty tile --
// t0 >= t_end -- costs no memory traffic).  The wave's block-table window is
// two VGPRs: lane i of tab_a / tab_b holds the entry of logical block
// wb + i / wb + 64 + i, and a wave-uniform readlane turns it into a scalar.
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
__device__ __forceinline__ void load_tile_uniform(
    TileRegs<QT, CT, D>& tr, int bs, int nblocks, uint32_t tab_a,
    uint32_t tab_b, int wb, const uint8_t* kbase, const uint8_t* vbase,
    int64_t stride, int t0, int t_end, int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
  // Everything addressing a half-tile is wave-uniform; readfirstlane says
  // so to the compiler, which keeps it in SGPRs (buffer resources in SGPRs)
  // instead of looping over lanes.
  t0 = __builtin_amdgcn_readfirstlane(t0);
  const int kofs = c * (int)stride + j * 16;
  const int vtok = lane / S::PPR;
  const int vofs = vtok * (int)stride + (lane % S::PPR) * 16;
#pragma unroll
  for (int sb = 0; sb < S::SUB; ++sb) {
    __amdgpu_buffer_rsrc_t kr[2], vr[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int tb = t0 + 32 * sb + 16 * hh;
      int nvalid = t_end - tb;
      nvalid = nvalid < 0 ? 0 : (nvalid > 16 ? 16 : nvalid);
      int64_t row0 = 0;
      if (nvalid > 0) {
        const int lb = tb / bs;
        const int idx = lb - wb;  // 0 .. 127
        int phys;
        if (idx < 64)  // (tab_b may still be in flight: touch it only if needed)
          phys = __builtin_amdgcn_readlane(tab_a, idx);
        else
          phys = __builtin_amdgcn_readlane(tab_b, idx - 64);
        // an entry outside the pool (the caller's error) is clamped into
        // it: unspecified values, never an access outside the pool
        phys = (uint32_t)phys < (uint32_t)nblocks ? phys : nblocks - 1;
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
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int r = 0; r < S::KPIECES; ++r) {
        const u32x4_t v =
            __builtin_amdgcn_raw_buffer_load_b128(kr[hh], kofs + r * 64, 0, 0);
        tr.kw[sb][hh][4 * r + 0] = v[0];
        tr.kw[sb][hh][4 * r + 1] = v[1];
        tr.kw[sb][hh][4 * r + 2] = v[2];
        tr.kw[sb][hh][4 * r + 3] = v[3];
      }
    }
#pragma unroll
    for (int v = 0; v < S::NV; ++v) {
      const int hh = (v * S::TOK_PER_V) >> 4;
      const int tin = (v * S::TOK_PER_V) & 15;
      // the whole offset goes in the per-lane operand: the range check covers it
      tr.vraw[sb][v] = __builtin_amdgcn_raw_buffer_load_b128(
          vr[hh], vofs + tin * (int)stride, 0, 0);
    }
  }
}

// Tile loads for any block size: one table lookup per token (vector), masked
// lanes skip the load and hold zeros.
template <typename QT, typename CT, int D>
__device__ __forceinline__ void load_tile_any(
    TileRegs<QT, CT, D>& tr, int bs, int nblocks, const int32_t* trow,
    const uint8_t* kbase, const uint8_t* vbase, int64_t stride, int t0,
    int t_end, int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int sb = 0; sb < S::SUB; ++sb) {
    const int ts = t0 + 32 * sb;
    const int tok = ts + (lane & 31);
    int myslot = 0;
    if (tok < t_end) {
      const int lb = tok / bs;
      const int pb = trow[lb];
      myslot = ((uint32_t)pb < (uint32_t)nblocks ? pb : nblocks - 1) * bs +
               (tok - lb * bs);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int ks = __shfl(myslot, 16 * hh + c, 64);
      const bool ok = ts + 16 * hh + c < t_end;
      const uint8_t* row = kbase + (int64_t)ks * stride;
#pragma unroll
      for (int r = 0; r < S::KPIECES; ++r) {
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (ok) v = *reinterpret_cast<const u32x4_t*>(row + (4 * r + j) * 16);
        tr.kw[sb][hh][4 * r + 0] = v[0];
        tr.kw[sb][hh][4 * r + 1] = v[1];
        tr.kw[sb][hh][4 * r + 2] = v[2];
        tr.kw[sb][hh][4 * r + 3] = v[3];
      }
    }
#pragma unroll
    for (int v = 0; v < S::NV; ++v) {
      const int tv = lane / S::PPR + v * S::TOK_PER_V;
      const int vs = __shfl(myslot, tv, 64);
      tr.vraw[sb][v] = u32x4_t{0u, 0u, 0u, 0u};
      if (ts + tv < t_end)
        tr.vraw[sb][v] = *reinterpret_cast<const u32x4_t*>(
            vbase + (int64_t)vs * stride + (lane % S::PPR) * 16);
    }
  }
}

// ---------------------------------------------------------------------------
// A tile's V rows -> the wave's LDS slice, converted to the PV operand type and
// XOR-swizzled in 16-byte chunks so the transposed reads are conflict-free.
// The slice is private to the wave and one wave's LDS operations execute in
// issue order, so no barrier is needed around it.
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
__device__ __forceinline__ void stage_v(const u32x4_t (&vraw)[Shape<QT, CT, D>::NV],
                                        uint8_t* vt, int lane) {
  typedef Shape<QT, CT, D> S;
  typedef typename S::PVT PVT;
  constexpr int PVB = S::PVB;
#pragma unroll
  for (int v = 0; v < S::NV; ++v) {
    const int tv = lane / S::PPR + v * S::TOK_PER_V;
    const int swz = ((tv >> 2) & 3) * PVB;
    uint8_t* rowp = vt + tv * S::LDS_ROW;
    const int ch0 = (lane % S::PPR) * S::VCH;
    if constexpr (PVB == 2) {
      // 16-bit rows: 32-byte spans (16 columns, one output block) permuted
      // by token, so the 8 rows one transposing read touches per pass land
      // on distinct banks
      const int span = (ch0 >> 1) ^ (tv & (S::SPANS - 1));
      uint8_t* dst = rowp + (span << 5) + ((ch0 & 1) << 4);
      if constexpr (same<PVT, CT>::value) {
        *reinterpret_cast<u32x4_t*>(dst) = vraw[v];
      } else {  // fp8 -> f16: the piece's 16 elements fill the whole span
        u32x4_t lo, hi;
        lo[0] = fp8x2_to_f16x2(vraw[v][0], false);
        lo[1] = fp8x2_to_f16x2(vraw[v][0], true);
        lo[2] = fp8x2_to_f16x2(vraw[v][1], false);
        lo[3] = fp8x2_to_f16x2(vraw[v][1], true);
        hi[0] = fp8x2_to_f16x2(vraw[v][2], false);
        hi[1] = fp8x2_to_f16x2(vraw[v][2], true);
        hi[2] = fp8x2_to_f16x2(vraw[v][3], false);
        hi[3] = fp8x2_to_f16x2(vraw[v][3], true);
        *reinterpret_cast<u32x4_t*>(dst) = lo;
        *reinterpret_cast<u32x4_t*>(dst + 16) = hi;
      }
    } else if constexpr (same<PVT, CT>::value) {
      *reinterpret_cast<u32x4_t*>(rowp + ((ch0 ^ swz) << 4)) = vraw[v];
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

}

// ---------------------------------------------------------------------------
// One tile: S = K Q^T, online-softmax update, O^T += V^T P^T.  vt is this
// wave's LDS slice (32 rows of D PV-operand elements), already holding the
// tile's V rows (stage_v).
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
__device__ __forceinline__ void compute_tile(
    const uint32_t (&kw)[2][Shape<QT, CT, D>::KWORDS], const uint32_t* qw,
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
          ka[w] = kw[hh][4 * q + w];
          qb[w] = qw[4 * q + w];
        }
      } else if constexpr (same<QT, CT>::value) {  // float32
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ka[e] = bitcast<float>(kw[hh][8 * q + e]);
          qb[e] = bitcast<float>(qw[8 * q + e]);
        }
      } else if constexpr (QT::bytes == 2) {  // fp8 keys -> bf16/f16
        const uint32_t w0 = kw[hh][2 * q], w1 = kw[hh][2 * q + 1];
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
        const uint32_t w0 = kw[hh][2 * q], w1 = kw[hh][2 * q + 1];
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
#pragma unroll
  for (int n = 0; n < S::NBLK; ++n) {
    typename Mma<PVT>::operand va;
    if constexpr (PVB == 2) {
      // Transposing LDS reads: within each 16-lane group, lane 4k + q
      // addresses 4 columns (4q .. 4q + 3 of output block n) of token
      // 4j + k, and lane c receives column c of the four tokens 4j .. 4j+3
      // -- operand slots 0-3; the same read 16 tokens on gives slots 4-7.
      const int tk = 4 * j + (c >> 2);
      const int off = ((n ^ (tk & (S::SPANS - 1))) << 5) + ((c & 3) << 3);
      const v4i16_t lo = lds_read_tr16(vt + tk * S::LDS_ROW + off);
      const v4i16_t hi = lds_read_tr16(vt + (tk + 16) * S::LDS_ROW + off);
      va[0] = pack_u16x2(lo[0], lo[1]);
      va[1] = pack_u16x2(lo[2], lo[3]);
      va[2] = pack_u16x2(hi[0], hi[1]);
      va[3] = pack_u16x2(hi[2], hi[3]);
    } else {
      const int byte = (16 * n + c) * PVB;
      const int col = (((byte >> 4) ^ (j * PVB)) << 4) + (byte & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        va[e] = *reinterpret_cast<const float*>(vt + slot_token(j, e) * S::LDS_ROW + col);
    }
    st.o[n] = Mma<PVT>::step(va, pb_hi, st.o[n]);
    if constexpr (S::PSPLIT) st.o[n] = Mma<PVT>::step(va, pb_lo, st.o[n]);
  }
}

// ---------------------------------------------------------------------------
// The split of the tile list.  tex[s] (s = 0 .. num_seqs) is the exclusive
// prefix of the per-sequence tile counts ceil(L_s / 32); row (s, u), u =
// kv_head * chunks + chunk, holds tiles [U tex[s] + u T_s, + T_s) of the
// T = U tex[num_seqs] tiles, T_s = tex[s + 1] - tex[s].  With V = min(W, T)
// of the W waves in use, wave w < V owns tiles [ceil(w T / V),
// ceil((w + 1) T / V)) -- at least one -- and the waves from V on own none,
// so the waves holding pieces of one row are consecutive and all hold one.
// Tile t belongs to wave floor(t V / T).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int waves_in_use(int64_t T, int W) {
  return T < W ? (int)T : W;
}
__device__ __forceinline__ int wave_of_tile(int64_t t, int64_t T, int W) {
  return (int)(t * waves_in_use(T, W) / T);
}
__device__ __forceinline__ int64_t first_tile_of_wave(int w, int64_t T, int W) {
  const int V = waves_in_use(T, W);
  return w >= V ? T : ((int64_t)w * T + V - 1) / V;
}

// Partial slot of (wave w, slot q): o [gmax][D], then m [gmax], l [gmax] in
// separate arrays.
__device__ __forceinline__ int64_t slot_index(int w, int q) {
  return (int64_t)w * 2 + q;
}

// ---------------------------------------------------------------------------
// Merge of the pieces of one cut row: one workgroup per row (s, u).  Every
// thread takes 4 output columns of one query head and a strided subset of the
// pieces (nsub threads share an output column), requests the (m, l, o) of up
// to BATCH of its pieces at once, and folds them online:  M = max m_i,
// l = sum 2^(m_i - M) l_i, acc = sum 2^(m_i - M) o_i; the subsets are then
// folded the same way through LDS.  A row of G <= 4 query heads at head_dim
// 128 has 2 threads per column, so with BATCH 16 up to 32 pieces take one
// round of loads.  (Workgroups are kept small: most rows of a large batch
// are not cut, and their workgroups only launch and exit.)
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

// base[byte_off] with a 32-bit offset, so the load can keep the base in
// scalar registers.
template <typename T>
__device__ __forceinline__ T load_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const T*>(static_cast<const uint8_t*>(base) +
                                     byte_off);
}

__device__ __forceinline__ void lse_fold(float& m, float& l, f32x4_t& acc,
                                         float m2, float l2, f32x4_t acc2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both empty
  const float a1 = fast_exp2(m - M), a2 = fast_exp2(m2 - M);
  l = l * a1 + l2 * a2;
  acc = acc * a1 + acc2 * a2;
  m = M;
}

template <int D, bool SCALED, int BATCH>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
  constexpr int D4 = D / 4;
  __shared__ __attribute__((aligned(16))) f32x4_t red_o[kMergeThreads];
  __shared__ float red_m[kMergeThreads], red_l[kMergeThreads];

  const int tid = threadIdx.x;
  const int U = a.num_kv_heads * a.group_chunks;
  const int s = blockIdx.x / U;
  const int u = blockIdx.x - s * U;
  const int* tex = a.tile_prefix;
  const int ts = tex[s + 1] - tex[s];
  if (ts == 0) return;  // zeros written by the partition kernel
  const int64_t T = (int64_t)U * tex[a.num_seqs];
  const int W = a.num_waves;
  const int64_t r0 = (int64_t)U * tex[s] + (int64_t)u * ts;
  const int wf = wave_of_tile(r0, T, W);
  const int wl = wave_of_tile(r0 + ts - 1, T, W);
  if (wf == wl) return;  // finished by one wave
  const int npieces = wl - wf + 1;
  const int q_first = first_tile_of_wave(wf, T, W) < r0 ? 1 : 0;

  const int h = u / a.group_chunks;
  const int gc = u - h * a.group_chunks;
  const int gcount = min(16, a.group - gc * 16);
  const int gmax = a.slot_heads;
  const int64_t head0 = (int64_t)s * a.num_q_heads + h * a.group + gc * 16;

  const int items = gcount * D4;
  const int nsub = items >= kMergeThreads ? 1 : kMergeThreads / items;
  for (int it = tid; it < items * nsub; it += kMergeThreads) {
    const int item = it % items;
    const int sub = it / items;
    const int g = item / D4;
    const int d4 = item - g * D4;
    float m = -INFINITY, l = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // slot of piece i: slot_index(wf + i, i == 0 ? q_first : 0) * gmax + g,
    // as a 32-bit offset (slots * head_dim < 2^24)
    const uint32_t sl0 = (uint32_t)(slot_index(wf, 0) * gmax + g);
    const uint32_t step = 2u * (uint32_t)gmax;
    for (int i0 = sub; i0 < npieces; i0 += BATCH * nsub) {
      float mi[BATCH], li[BATCH];
      f32x4_t oi[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const int i = i0 + k * nsub;
        mi[k] = -INFINITY;
        li[k] = 0.f;
        oi[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (i < npieces) {
          const uint32_t sl = sl0 + step * (uint32_t)i +
                              (i == 0 ? (uint32_t)(q_first * gmax) : 0u);
          mi[k] = load_at<float>(a.part_m, sl * 4u);
          li[k] = load_at<float>(a.part_l, sl * 4u);
          oi[k] = load_at<f32x4_t>(a.part_o, (sl * (uint32_t)D + 4u * d4) * 4u);
        }
      }
#pragma unroll
      for (int k = 0; k < BATCH; ++k) lse_fold(m, l, acc, mi[k], li[k], oi[k]);
    }
    if (nsub == 1) {
      const float f = (SCALED ? *a.v_scale : 1.f) / l;
      *reinterpret_cast<f32x4_t*>(a.out + (head0 + g) * D + 4 * d4) = acc * f;
    } else {
      red_o[it] = acc;
      red_m[it] = m;
      red_l[it] = l;
    }
  }
  if (nsub > 1) {
    __syncthreads();
    for (int item = tid; item < items; item += kMergeThreads) {
      const int g = item / D4;
      const int d4 = item - g * D4;
      float m = red_m[item], l = red_l[item];
      f32x4_t acc = red_o[item];
      for (int sub = 1; sub < nsub; ++sub)
        lse_fold(m, l, acc, red_m[sub * items + item], red_l[sub * items + item],
                 red_o[sub * items + item]);
      const float f = (SCALED ? *a.v_scale : 1.f) / l;
      *reinterpret_cast<f32x4_t*>(a.out + (head0 + g) * D + 4 * d4) = acc * f;
    }
  }
}

// Inclusive scan of one int per thread across the workgroup.
__device__ int block_inclusive_scan(int v, int* sm_wsum) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  if (lane == 63) sm_wsum[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += sm_wsum[w];
  return v + add;
}

// A run of consecutive tiles of one row owned by one wave.
struct Seg {
  int s, h, gc;       // the row
  int t_begin, t_end; // tokens of the sequence it covers
  int ntiles;
  int wb;             // first logical block of its table window
  bool full;          // the whole row: write the final output
  bool valid;
};

// The segment starting at tile t of the wave's range [.., te): the largest s
// with tex[s] <= t / U (binary search in LDS; every lane runs it with the
// same values), then the row and the tile within it.
template <int TT>
__device__ __forceinline__ Seg segment_at(int64_t t, int64_t te, int U,
                                          const int* tex, const int* lens,
                                          const AttnArgs& a) {
  Seg g;
  g.valid = t < te;
  if (!g.valid) {
    g.s = g.h = g.gc = 0;
    g.t_begin = g.t_end = 0;
    g.ntiles = 0;
    g.wb = 0;
    g.full = false;
    return g;
  }
  const int q = (int)(t / U);
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(tex[mid]) <= q) lo = mid;
    else hi = mid - 1;
  }
  const int base_t = __builtin_amdgcn_readfirstlane(tex[lo]);
  const int ts = __builtin_amdgcn_readfirstlane(tex[lo + 1]) - base_t;
  const int L = __builtin_amdgcn_readfirstlane(lens[lo]);
  const int64_t base = (int64_t)U * base_t;
  const int r = (int)(t - base);
  const int u = r / ts;
  const int k0 = r - u * ts;
  const int64_t row_end = base + (int64_t)(u + 1) * ts;
  const int64_t end = te < row_end ? te : row_end;
  g.s = lo;
  g.h = u / a.group_chunks;
  g.gc = u - g.h * a.group_chunks;
  g.ntiles = (int)(end - t);
  g.t_begin = TT * k0;
  g.t_end = min(L, TT * (k0 + g.ntiles));
  g.wb = g.t_begin / a.block_size;
  g.full = k0 == 0 && end == row_end;
  return g;
}

// Entries wb + 64 * half + lane of the segment's table row (0 past the blocks
// the segment can reach; such lanes fetch nothing).
__device__ __forceinline__ uint32_t load_window(const Seg& g, int half,
                                                const AttnArgs& a, int lane) {
  const int nblk = g.valid ? (g.t_end + a.block_size - 1) / a.block_size : 0;
  const int nrec = __builtin_amdgcn_readfirstlane(nblk * 4);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t*>(a.block_tables +
                           (int64_t)g.s * a.max_blocks_per_seq),
      (short)0, nrec, kRawBufferFlags);
  return __builtin_amdgcn_raw_buffer_load_b32(
      r, (g.wb + 64 * half + lane) * 4, 0, 0);
}

// The query rows of a segment's row as the B operand of S = K Q^T (zeros for
// query heads past the chunk's count and for an invalid segment).
template <typename QT, typename CT, int D>
__device__ __forceinline__ void load_query(uint32_t* qw, const Seg& g,
                                           const AttnArgs& a, int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int gcount = min(16, a.group - g.gc * 16);
  const int hq0 = g.h * a.group + g.gc * 16;
  const int nrec = __builtin_amdgcn_readfirstlane(
      g.valid ? gcount * D * QT::bytes : 0);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(static_cast<const uint8_t*>(a.query) +
                           ((int64_t)g.s * a.num_q_heads + hq0) * D * QT::bytes),
      (short)0, nrec, kRawBufferFlags);
  constexpr int QBYTES_PER_R = S::EP * QT::bytes;
  constexpr int QLOADS = QBYTES_PER_R / 16;
#pragma unroll
  for (int rr = 0; rr < D / (4 * S::EP); ++rr) {
#pragma unroll
    for (int k = 0; k < QLOADS; ++k) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          r, c * D * QT::bytes + (4 * rr + j) * QBYTES_PER_R + 16 * k, 0, 0);
      const int w0 = (rr * QBYTES_PER_R + 16 * k) / 4;
      qw[w0 + 0] = v[0];
      qw[w0 + 1] = v[1];
      qw[w0 + 2] = v[2];
      qw[w0 + 3] = v[3];
    }
  }
}

// ---------------------------------------------------------------------------
// Partition kernel: wave w streams tiles [ceil(w T / W), ceil((w+1) T / W))
// of the row-major tile list, one segment (run of one row) after another.
// The next segment's query rows and table window are requested when a
// segment starts and its first tile during the current segment's last tile,
// so a wave's loads run on across segment boundaries.
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D, bool UNIFORM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_decode_kernel(AttnArgs a) {
  typedef Shape<QT, CT, D> S;
  constexpr int NBLK = S::NBLK;
  constexpr bool PREFETCH = UNIFORM && CT::bytes <= 2;

  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * S::STAGE_BYTES];
  __shared__ int sm_wsum[kWaves];
  extern __shared__ int sm_seq[];  // tex[num_seqs + 1] | lens[num_seqs]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int nS = a.num_seqs;
  const int U = a.num_kv_heads * a.group_chunks;
  int* tex = sm_seq;
  int* lens = sm_seq + nS + 1;

  // ---- tile counts of all sequences and their exclusive prefix ----
  {
    const int per = (nS + kThreads - 1) / kThreads;
    const int b0 = min(tid * per, nS);
    const int b1 = min(b0 + per, nS);
    int sum = 0;
    for (int i = b0; i < b1; ++i) {
      // a length beyond the table's reach (the caller's error) is cut to it,
      // so the table reads stay inside the sequence's row
      const int L = min(max(a.seq_lens[i], 0), a.max_seq_tokens);
      lens[i] = L;
      sum += (L + S::TT - 1) / S::TT;
    }
    const int incl = block_inclusive_scan(sum, sm_wsum);
    int run = incl - sum;
    for (int i = b0; i < b1; ++i) {
      tex[i] = run;
      run += (lens[i] + S::TT - 1) / S::TT;
    }
    if (tid == kThreads - 1) tex[nS] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0)  // the merge kernel reads the prefix from here
    for (int i = tid; i <= nS; i += kThreads) a.tile_prefix[i] = tex[i];

  const int W = a.num_waves;
  const int w = blockIdx.x * kWaves + wave;
  const int64_t T = (int64_t)U * tex[nS];
  const int64_t tb = first_tile_of_wave(w, T, W);
  const int64_t te = first_tile_of_wave(w + 1, T, W);

  float vscale = 1.f, kscale = 1.f;
  if constexpr (is_fp8<CT>::value) {
    kscale = *a.k_scale;
    vscale = *a.v_scale;
  }

  // ---- rows of empty sequences sit at tile position U tex[s]; the wave
  // whose range holds that position (the last wave for position T) writes
  // their zeros ----
  {
    int lo = 0, hi = nS;  // first s with U tex[s] >= tb
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)U * __builtin_amdgcn_readfirstlane(tex[mid]) >= tb) hi = mid;
      else lo = mid + 1;
    }
    for (int s = lo; s < nS; ++s) {
      const int64_t pos = (int64_t)U * __builtin_amdgcn_readfirstlane(tex[s]);
      if (pos >= te && !(w == waves_in_use(T, W) - 1 && pos == T) &&
          !(T == 0 && w == 0))
        break;
      if (__builtin_amdgcn_readfirstlane(lens[s]) != 0) continue;
      float* dst = a.out + (int64_t)s * a.num_q_heads * D;
      for (int i = lane; i < a.num_q_heads * D / 4; i += 64)
        reinterpret_cast<f32x4_t*>(dst)[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }

  const float qk_mul = a.qk_scale_log2 * kscale;
  const int64_t stride = (int64_t)a.num_kv_heads * S::ROW_BYTES;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_cache);
  uint8_t* vt = smem + wave * S::STAGE_BYTES;
  const int gmax = a.slot_heads;

  Seg X = segment_at<S::TT>(tb, te, U, tex, lens, a);
  int64_t pos_n = tb + X.ntiles;  // first tile of the next segment
  Seg Xn = segment_at<S::TT>(pos_n, te, U, tex, lens, a);
  bool first_seg = true;
  uint32_t ta = 0, tbw = 0, ta_n = 0, tb_n = 0;
  if constexpr (UNIFORM) {
    ta = load_window(X, 0, a, lane);
    tbw = load_window(X, 1, a, lane);
    ta_n = load_window(Xn, 0, a, lane);
    tb_n = load_window(Xn, 1, a, lane);
  }
  uint32_t qw[S::QWORDS];
  load_query<QT, CT, D>(qw, X, a, lane);
  TileRegs<QT, CT, D> cur;
  if constexpr (PREFETCH)
    load_tile_uniform<QT, CT, D>(cur, a.block_size, a.num_blocks, ta, tbw, X.wb,
                                 kpool + (int64_t)X.h * S::ROW_BYTES,
                                 vpool + (int64_t)X.h * S::ROW_BYTES, stride,
                                 X.t_begin, X.t_end, lane);

  while (X.valid) {
    uint32_t qn[S::QWORDS];
    load_query<QT, CT, D>(qn, Xn, a, lane);

    WaveState<NBLK> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int n = 0; n < NBLK; ++n) st.o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint8_t* kbase = kpool + (int64_t)X.h * S::ROW_BYTES;
    const uint8_t* vbase = vpool + (int64_t)X.h * S::ROW_BYTES;
    if constexpr (PREFETCH) {
      const uint8_t* kbase_n = kpool + (int64_t)Xn.h * S::ROW_BYTES;
      const uint8_t* vbase_n = vpool + (int64_t)Xn.h * S::ROW_BYTES;
      int wb = X.wb;
      for (int k = 0; k < X.ntiles; ++k) {
        const int t0 = X.t_begin + S::TT * k;
        stage_v<QT, CT, D>(cur.vraw[0], vt, lane);
        // the next tile of this wave's stream: tile k + 1 of X, else the
        // first tile of the next segment (an empty range past the end);
        // requested before this tile is computed, which the scheduling
        // barrier keeps (the compiler would otherwise sink the loads to
        // shorten register lifetimes)
        const bool same_seg = k + 1 < X.ntiles;
        const int t_next = t0 + S::TT;
        if (same_seg && t_next / a.block_size - wb >= 64) {
          // the window moves on by 64 blocks; the new upper half is needed
          // only 64 blocks later
          wb += 64;
          ta = tbw;
          Seg shifted = X;
          shifted.wb = wb;
          tbw = load_window(shifted, 1, a, lane);
        }
        TileRegs<QT, CT, D> nxt;
        load_tile_uniform<QT, CT, D>(
            nxt, a.block_size, a.num_blocks, same_seg ? ta : ta_n, same_seg ? tbw : tb_n,
            same_seg ? wb : Xn.wb, same_seg ? kbase : kbase_n,
            same_seg ? vbase : vbase_n, stride,
            same_seg ? t_next : Xn.t_begin, same_seg ? X.t_end : Xn.t_end,
            lane);
        __builtin_amdgcn_sched_barrier(0);
        compute_tile<QT, CT, D>(cur.kw[0], qw, st, vt, t0, X.t_end, qk_mul,
                                lane);
#pragma unroll
        for (int sb = 1; sb < S::SUB; ++sb) {
          if (t0 + 32 * sb < X.t_end) {  // (only the last tile has empty ones)
            stage_v<QT, CT, D>(cur.vraw[sb], vt, lane);
            compute_tile<QT, CT, D>(cur.kw[sb], qw, st, vt, t0 + 32 * sb,
                                    X.t_end, qk_mul, lane);
          }
        }
        cur = nxt;
      }
    } else {
      const int32_t* trow = a.block_tables + (int64_t)X.s * a.max_blocks_per_seq;
      for (int k = 0; k < X.ntiles; ++k) {
        const int t0 = X.t_begin + S::TT * k;
        if constexpr (UNIFORM) {
          const int wb = X.wb + (t0 / a.block_size - X.wb) / 64 * 64;
          Seg shifted = X;
          shifted.wb = wb;
          const uint32_t wa = load_window(shifted, 0, a, lane);
          const uint32_t wbb = load_window(shifted, 1, a, lane);
          load_tile_uniform<QT, CT, D>(cur, a.block_size, a.num_blocks, wa,
                                       wbb, wb, kbase,
                                       vbase, stride, t0, X.t_end, lane);
        } else {
          load_tile_any<QT, CT, D>(cur, a.block_size, a.num_blocks, trow,
                                   kbase, vbase,
                                   stride, t0, X.t_end, lane);
        }
#pragma unroll
        for (int sb = 0; sb < S::SUB; ++sb) {
          if (t0 + 32 * sb < X.t_end) {
            stage_v<QT, CT, D>(cur.vraw[sb], vt, lane);
            compute_tile<QT, CT, D>(cur.kw[sb], qw, st, vt, t0 + 32 * sb,
                                    X.t_end, qk_mul, lane);
          }
        }
      }
    }

    // ---------------- the segment's output (this wave alone) ----------------
    // lane (c + 16 j) holds O^T rows 16 n + 4 j .. + 3 of query head c
    const int gcount = min(16, a.group - X.gc * 16);
    float l_tot = xor_sum(st.l, 16);
    l_tot = xor_sum(l_tot, 32);
    if (c < gcount) {
      if (X.full) {
        const int64_t head = (int64_t)X.s * a.num_q_heads + X.h * a.group +
                             X.gc * 16 + c;
        const float f = l_tot > 0.f ? vscale / l_tot : 0.f;
        float* dst = a.out + head * D + 4 * j;
#pragma unroll
        for (int n = 0; n < NBLK; ++n)
          *reinterpret_cast<f32x4_t*>(dst + 16 * n) = st.o[n] * f;
      } else {
        // first segment of the wave -> slot 0, last -> slot 1
        const int64_t sl = slot_index(w, first_seg ? 0 : 1) * gmax + c;
        float* dst = a.part_o + sl * D + 4 * j;
#pragma unroll
        for (int n = 0; n < NBLK; ++n)
          *reinterpret_cast<f32x4_t*>(dst + 16 * n) = st.o[n];
        if (j == 0) {
          a.part_m[sl] = st.m;
          a.part_l[sl] = l_tot;
        }
      }
    }

    // ---------------- advance to the next segment ----------------
    first_seg = false;
    X = Xn;
    if constexpr (UNIFORM) {
      ta = ta_n;
      tbw = tb_n;
    }
#pragma unroll
    for (int q = 0; q < S::QWORDS; ++q) qw[q] = qn[q];
    pos_n += X.ntiles;
    Xn = segment_at<S::TT>(pos_n, te, U, tex, lens, a);
    if constexpr (UNIFORM) {
      ta_n = load_window(Xn, 0, a, lane);
      tb_n = load_window(Xn, 1, a, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
// Workgroups of the partition kernel: as many as can be resident at once
// (occupancy x CUs), capped by the caller's wave limit and kMaxWaves.
template <typename K>
static int resident_grid(K kernel, size_t dyn_lds, int max_waves) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(kernel), kThreads, dyn_lds) !=
          hipSuccess)
    return -1;
  // One workgroup (one wave per SIMD) per CU measured fastest for the
  // streaming loop: more resident waves deepen the memory queues without
  // adding bandwidth.
  int64_t g = (int64_t)(per_cu < kWorkgroupsPerCU ? per_cu : kWorkgroupsPerCU) * cus;
  if (g < cus) g = cus;
  int64_t cap = kMaxWaves / kWaves;
  if (max_waves > 0 && max_waves / kWaves < cap) cap = max_waves / kWaves;
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

template <typename QT, typename CT, int D, bool UNIFORM>
static hipError_t launch_u(AttnArgs a, int max_waves, hipStream_t stream) {
  auto kernel = attn_decode_kernel<QT, CT, D, UNIFORM>;
  const size_t dyn = ((size_t)2 * a.num_seqs + 1) * sizeof(int);
  const int grid = resident_grid(kernel, dyn, max_waves);
  if (grid < 0) return hipErrorInvalidValue;
  a.num_waves = grid * kWaves;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), dyn, stream, a);
  // Pieces per cut row grow with the wave boundaries per row: fetch them in
  // batches of 16 when there are about 4 or more boundaries per row, else 4
  // (fewer registers, so the mostly idle workgroups of many-row batches
  // launch in one round).
  const int rows = a.num_seqs * a.num_kv_heads * a.group_chunks;
  if (rows > 0 && a.num_waves >= 4 * rows)
    hipLaunchKernelGGL((attn_merge_kernel<D, is_fp8<CT>::value, 16>),
                       dim3(rows), dim3(kMergeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, is_fp8<CT>::value, 4>),
                       dim3(rows), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename QT, typename CT, int D>
static hipError_t launch_d(const AttnArgs& a, int max_waves, bool uniform,
                           hipStream_t stream) {
  if (uniform) return launch_u<QT, CT, D, true>(a, max_waves, stream);
  return launch_u<QT, CT, D, false>(a, max_waves, stream);
}

template <typename QT, typename CT>
static hipError_t launch_t(const AttnArgs& a, int head_dim, int max_waves,
                           bool uniform, hipStream_t stream) {
  if (head_dim == 64) return launch_d<QT, CT, 64>(a, max_waves, uniform, stream);
  return launch_d<QT, CT, 128>(a, max_waves, uniform, stream);
}

hipError_t launch_attn_decode(const AttnArgs& a, int q_dtype, int cache_dtype,
                              int head_dim, int max_waves,
                              hipStream_t stream) {
  const bool uniform = (a.block_size % 16) == 0;
  switch (cache_dtype) {
    case PKV_F32: return launch_t<F32, F32>(a, head_dim, max_waves, uniform, stream);
    case PKV_F16: return launch_t<F16, F16>(a, head_dim, max_waves, uniform, stream);
    case PKV_BF16: return launch_t<BF16, BF16>(a, head_dim, max_waves, uniform, stream);
    case PKV_FP8_E4M3:
      if (q_dtype == PKV_BF16) return launch_t<BF16, FP8>(a, head_dim, max_waves, uniform, stream);
      if (q_dtype == PKV_F16) return launch_t<F16, FP8>(a, head_dim, max_waves, uniform, stream);
      return launch_t<F32, FP8>(a, head_dim, max_waves, uniform, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
