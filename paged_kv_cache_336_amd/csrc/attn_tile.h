// attn_tile.h -- device code shared by the paged attention kernels (one
// query token per sequence in attn_decode.hip, several in attn_multi.hip):
// launch constants, the 32-token tile shapes and loaders, V staging, the
// MFMA tile step with the online softmax, the split of the unit list over
// waves, the segment/window helpers and the fold of a cut row's pieces.
#ifndef PKV_ATTN_TILE_H
#define PKV_ATTN_TILE_H

#include <limits.h>

#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kWorkgroupsPerCU = 1;       // default grid: one workgroup per CU
constexpr int kXcds = 8;                  // dies a grid is dispatched over

// The workgroup number the split uses for workgroup `b` of a grid of `n`.
// Workgroups are handed to the XCDs in turn (b to XCD b % 8), and each XCD
// has its own L2.  When blocks may be shared between sequences (no
// PKV_KV_STREAM hint), the split numbers the workgroups XCD by XCD, so that
// the ranges of one XCD are neighbours in the tile order: sequences that
// share a prompt sit next to each other there, and their shared blocks are
// then served by that XCD's L2 after the first read.  Without sharing the
// dispatch order is kept.  Either way every range is processed exactly
// once, so the result does not depend on it.
__device__ __forceinline__ int split_workgroup(int b, int n, bool shared) {
  if (!shared || n % kXcds != 0) return b;
  return (b % kXcds) * (n / kXcds) + b / kXcds;
}
constexpr uint32_t kRawBufferFlags = 0x00020000;  // dword3: 32-bit data format
// Cache-policy operand of a buffer load: 0 = the default policy; kLoadNT
// sets the non-temporal (streaming) bit.  The tile loaders apply it to the V
// rows, whose loads cover whole 128-byte lines, and to K rows loaded the
// same way for staging through LDS (load_tile_uniform's KL); loaded straight
// into the MFMA operand layout, each K load instruction reads 64 bytes of
// each of 16 rows, so a line is requested by two instructions, and
// streaming those measured slower.
constexpr int kLoadNT = 2;

template <typename QT, typename CT> struct PvOperand { typedef CT type; };
template <> struct PvOperand<BF16, FP8> { typedef F16 type; };
template <> struct PvOperand<F16, FP8> { typedef F16 type; };
template <> struct PvOperand<F32, FP8> { typedef F32 type; };
template <> struct PvOperand<BF16, FP8E5> { typedef F16 type; };
template <> struct PvOperand<F16, FP8E5> { typedef F16 type; };
template <> struct PvOperand<F32, FP8E5> { typedef F32 type; };

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
  static constexpr int KSTAGE_BYTES = 32 * ROW_BYTES;
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

// One tile's raw K and V bytes as loaded from the pool, per sub-tile; with
// per-token fp8 scales also the tile's scales, one per lane: lane c + 16 j
// holds the key (c < 8) or value (c >= 8) scale of the token in score slot
// c % 8 of row group j (slot_token(j, c % 8)), so each 16-lane row holds
// exactly the 16 scales its score slots need (see softmax_tile).
template <typename QT, typename CT, int D> struct TileRegs {
  typedef Shape<QT, CT, D> S;
  uint32_t kw[S::SUB][2][S::KWORDS];
  u32x4_t kraw[S::SUB][S::NV];
  u32x4_t vraw[S::SUB][S::NV];
  float sc[S::SUB];
};

// Per-token fp8 scale arrays [num_blocks, block_size, num_kv_heads], both
// already offset to one kv head (token slot t's scale at [t * hkv]).
struct TokenScales {
  const float* k;
  const float* v;
  int hkv;
};

// Online-softmax state of one wave: running max (log2 domain) and this
// lane's share of the running sum for query head column c, and O^T blocks.
// With per-token value scales O^T is kept in units of 2^mv, mv the running
// maximum of score + log2(value scale) (see softmax_tile).
template <int NBLK> struct WaveState {
  float m;
  float mv;
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
template <typename QT, typename CT, int D, bool PT = false, int AUX = 0,
          bool KL = false>
__device__ __forceinline__ void load_tile_uniform(
    TileRegs<QT, CT, D>& tr, int bs, int nblocks, uint32_t tab_a,
    uint32_t tab_b, int wb, const uint8_t* kbase, const uint8_t* vbase,
    int64_t stride, int t0, int t_end, int lane, TokenScales tsc = {}) {
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
    int64_t first_slot[2];
    int live[2];
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
      first_slot[hh] = row0;
      live[hh] = nvalid;
      // (the clamp above may be selected as a vector min/max)
      const int nrec = __builtin_amdgcn_readfirstlane(nvalid * (int)stride);
      kr[hh] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(kbase + row0 * stride), (short)0, nrec,
          kRawBufferFlags);
      vr[hh] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(vbase + row0 * stride), (short)0, nrec,
          kRawBufferFlags);
    }
    if constexpr (KL) {
#pragma unroll
      for (int v = 0; v < S::NV; ++v) {
        const int hh = (v * S::TOK_PER_V) >> 4;
        const int tin = (v * S::TOK_PER_V) & 15;
        tr.kraw[sb][v] = __builtin_amdgcn_raw_buffer_load_b128(
            kr[hh], vofs + tin * (int)stride, 0, AUX);
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int r = 0; r < S::KPIECES; ++r) {
          const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
              kr[hh], kofs + r * 64, 0, 0);
          tr.kw[sb][hh][4 * r + 0] = v[0];
          tr.kw[sb][hh][4 * r + 1] = v[1];
          tr.kw[sb][hh][4 * r + 2] = v[2];
          tr.kw[sb][hh][4 * r + 3] = v[3];
        }
      }
    }
#pragma unroll
    for (int v = 0; v < S::NV; ++v) {
      const int hh = (v * S::TOK_PER_V) >> 4;
      const int tin = (v * S::TOK_PER_V) & 15;
      // the whole offset goes in the per-lane operand: the range check covers it
      tr.vraw[sb][v] = __builtin_amdgcn_raw_buffer_load_b128(
          vr[hh], vofs + tin * (int)stride, 0, AUX);
    }
    if constexpr (PT) {
      // score slot c % 8: token 4 j + c % 4 of half (c / 4) % 2 (0 past
      // the half's live rows)
      const int hl = (c >> 2) & 1;
      const int t = 4 * j + (c & 3);
      tr.sc[sb] = 0.f;
      if (t < (hl ? live[1] : live[0]))
        tr.sc[sb] = (c < 8 ? tsc.k : tsc.v)[
            ((hl ? first_slot[1] : first_slot[0]) + t) * tsc.hkv];
    }
  }
}

// Tile loads for any block size: one table lookup per token (vector), masked
// lanes skip the load and hold zeros.
template <typename QT, typename CT, int D, bool PT = false>
__device__ __forceinline__ void load_tile_any(
    TileRegs<QT, CT, D>& tr, int bs, int nblocks, const int32_t* trow,
    const uint8_t* kbase, const uint8_t* vbase, int64_t stride, int t0,
    int t_end, int lane, TokenScales tsc = {}) {
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
    if constexpr (PT) {  // score slot c % 8's token (see TileRegs)
      const int t = slot_token(j, c & 7);
      const int st = __shfl(myslot, t, 64);
      tr.sc[sb] = 0.f;
      if (ts + t < t_end)
        tr.sc[sb] = (c < 8 ? tsc.k : tsc.v)[(int64_t)st * tsc.hkv];
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
        lo[0] = fp8x2_to_f16x2<CT>(vraw[v][0], false);
        lo[1] = fp8x2_to_f16x2<CT>(vraw[v][0], true);
        lo[2] = fp8x2_to_f16x2<CT>(vraw[v][1], false);
        lo[3] = fp8x2_to_f16x2<CT>(vraw[v][1], true);
        hi[0] = fp8x2_to_f16x2<CT>(vraw[v][2], false);
        hi[1] = fp8x2_to_f16x2<CT>(vraw[v][2], true);
        hi[2] = fp8x2_to_f16x2<CT>(vraw[v][3], false);
        hi[3] = fp8x2_to_f16x2<CT>(vraw[v][3], true);
        *reinterpret_cast<u32x4_t*>(dst) = lo;
        *reinterpret_cast<u32x4_t*>(dst + 16) = hi;
      }
    } else if constexpr (same<PVT, CT>::value) {
      *reinterpret_cast<u32x4_t*>(rowp + ((ch0 ^ swz) << 4)) = vraw[v];
    } else {  // fp8 -> f32, four chunks
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2_t p0 = fp8x2_to_f32x2<CT>(vraw[v][w], false);
        const f32x2_t p1 = fp8x2_to_f32x2<CT>(vraw[v][w], true);
        f32x4_t q = {p0[0], p0[1], p1[0], p1[1]};
        *reinterpret_cast<f32x4_t*>(rowp + (((ch0 + w) ^ swz) << 4)) = q;
      }
    }
  }

}

template <typename QT, typename CT, int D>
__device__ __forceinline__ int k_lds_at(int t, int x) {
  typedef Shape<QT, CT, D> S;
  constexpr int RPB = S::ROW_BYTES >= 256 ? 1 : 256 / S::ROW_BYTES;
  constexpr int NSW = S::PPR < 16 ? S::PPR : 16;
  return t * S::ROW_BYTES + ((x ^ ((t / RPB) & (NSW - 1))) << 4);
}

template <typename QT, typename CT, int D>
__device__ __forceinline__ void stage_k(
    const u32x4_t (&kraw)[Shape<QT, CT, D>::NV], uint8_t* kt, int lane) {
  typedef Shape<QT, CT, D> S;
#pragma unroll
  for (int v = 0; v < S::NV; ++v) {
    const int tv = lane / S::PPR + v * S::TOK_PER_V;
    *reinterpret_cast<u32x4_t*>(kt + k_lds_at<QT, CT, D>(tv, lane % S::PPR)) =
        kraw[v];
  }
}

template <typename QT, typename CT, int D>
using KWords = uint32_t[2][Shape<QT, CT, D>::KWORDS];

template <typename QT, typename CT, int D>
__device__ __forceinline__ void k_from_lds(KWords<QT, CT, D>& kw,
                                           const uint8_t* kt, int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int r = 0; r < S::KPIECES; ++r) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
          kt + k_lds_at<QT, CT, D>(16 * hh + c, 4 * r + j));
      kw[hh][4 * r + 0] = v[0];
      kw[hh][4 * r + 1] = v[1];
      kw[hh][4 * r + 2] = v[2];
      kw[hh][4 * r + 3] = v[3];
    }
  }
}

// ---------------------------------------------------------------------------
// One tile: S = K Q^T, online-softmax update, O^T += V^T P^T, in three parts
// so that several 16-column query groups can share one tile's K registers
// and V reads (compute_tile_groups).  vt is this wave's LDS slice (32 rows of
// D PV-operand elements), already holding the tile's V rows (stage_v).
// ---------------------------------------------------------------------------

// S = K Q^T of one 16-column group: sacc[hh][e] is the score of token
// 16 hh + 4 j + e against query column c (lane = c + 16 j).
template <typename QT, typename CT, int D>
__device__ __forceinline__ void qk_tile(
    const uint32_t (&kw)[2][Shape<QT, CT, D>::KWORDS], const uint32_t* qw,
    f32x4_t (&sacc)[2]) {
  typedef Shape<QT, CT, D> S;
  sacc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  sacc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the two halves' accumulations are independent: step over D with both
  // in turn, so each MFMA's latency is covered by the other half's
  // (the same order of additions per accumulator)
#pragma unroll
  for (int q = 0; q < S::QSTEPS; ++q) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
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
          ka[0] = fp8x2_to_bf16x2<CT>(w0, false);
          ka[1] = fp8x2_to_bf16x2<CT>(w0, true);
          ka[2] = fp8x2_to_bf16x2<CT>(w1, false);
          ka[3] = fp8x2_to_bf16x2<CT>(w1, true);
        } else {
          ka[0] = fp8x2_to_f16x2<CT>(w0, false);
          ka[1] = fp8x2_to_f16x2<CT>(w0, true);
          ka[2] = fp8x2_to_f16x2<CT>(w1, false);
          ka[3] = fp8x2_to_f16x2<CT>(w1, true);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) qb[w] = qw[4 * q + w];
      } else {  // fp8 keys -> f32
        const uint32_t w0 = kw[hh][2 * q], w1 = kw[hh][2 * q + 1];
        const f32x2_t p0 = fp8x2_to_f32x2<CT>(w0, false), p1 = fp8x2_to_f32x2<CT>(w0, true);
        const f32x2_t p2 = fp8x2_to_f32x2<CT>(w1, false), p3 = fp8x2_to_f32x2<CT>(w1, true);
        ka[0] = p0[0]; ka[1] = p0[1]; ka[2] = p1[0]; ka[3] = p1[1];
        ka[4] = p2[0]; ka[5] = p2[1]; ka[6] = p3[0]; ka[7] = p3[1];
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[e] = bitcast<float>(qw[8 * q + e]);
      }
      sacc[hh] = Mma<QT>::step(ka, qb, sacc[hh]);
    }
  }
}

// Online-softmax update (log2 domain) of one group from its scores; leaves
// P in the PV B-operand layout (for 16-bit caches split hi + lo).  Keys at or
// past t_end -- with CAUSAL, past this lane column's own limit `lim`, which
// the caller folds t_end into -- get weight 0.  With CAUSAL a column may see
// no key of a tile at all; its state then stays empty instead of turning
// into 0 * inf.
//
// PT (per-token fp8 scales; sc as TileRegs::sc): token t's score takes its
// key scale ks_t, and its value row its value scale vs_t, which cannot be
// factored out of the sum.  The PV weight of token t is then 2^(s_t - m)
// vs_t = 2^(u_t - m) with u_t = s_t + log2 vs_t; it is formed as
// 2^(u_t - mv) against a second running maximum mv of u, so the weights fed
// to the PV product stay bounded (by 1, or 2^kLazyMargin under LAZY) whatever
// the scales' range, and O^T is rescaled by 2^(mv_old - mv_new) as the sum l
// is by 2^(m_old - m_new).
// fold_value_scales turns O^T back into units of 2^m at the end.
//
// LAZY: the reference maximum moves only when a tile's maximum exceeds it by
// more than kLazyMargin (log2 units), so weights reach at most
// 2^kLazyMargin and O^T and l are rescaled only on those (rare) steps -- a
// wave-uniform branch skips the multiply of the accumulators otherwise
// (with per-token scales, each of the two maxima follows this rule).  The
// result is the same softmax with another reference point (m is what the
// partials and the merge carry); the PV weights keep the hi + lo split's
// precision relative to their size.
constexpr float kLazyMargin = 8.f;

// FOLD (no per-token scales; qk_mul > 0): the multiplier is applied inside
// each weight's exponent, 2^fma(s, qk_mul, -m), and to the tile's maximum,
// instead of to every score first -- one fused operation per score instead
// of two.  The maximum's own weight is then 2^(its rounding residual), not
// exactly 1, so only callers that promise no bit-exact one-token results
// use it.
template <typename QT, typename CT, int D, bool CAUSAL, bool PT = false,
          bool LAZY = false, bool FOLD = false>
__device__ __forceinline__ void softmax_tile(
    const f32x4_t (&sacc)[2], WaveState<Shape<QT, CT, D>::NBLK>& st, int t0,
    int t_end, int lim, int full_to, float qk_mul, int lane,
    typename Mma<typename Shape<QT, CT, D>::PVT>::operand& pb_hi,
    typename Mma<typename Shape<QT, CT, D>::PVT>::operand& pb_lo,
    float sc = 0.f) {
  typedef Shape<QT, CT, D> S;
  typedef typename S::PVT PVT;
  constexpr int PVB = S::PVB;
  const int j = lane >> 4;
  float sv[8];
  float lvs[8];  // PT: log2 of each token's value scale
  // PT: lanes 8..15 of each row hold value scales: their log2, then lane e
  // (key scale) and 8 + e (log2 value scale) of the row serve slot e
  const float own = PT && (lane & 8) ? __builtin_amdgcn_logf(sc) : sc;
  static_assert(!(FOLD && PT), "folded multiplier: no per-token scales");
  float mul[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mul[e] = FOLD ? 1.f : qk_mul;
    if constexpr (PT) {
      mul[e] *= row_broadcast(own, e);
      lvs[e] = row_broadcast(own, 8 + e);
    }
  }
  // full_to (wave-uniform): every key of a tile below it is live for every
  // column whose output is kept, so such a tile -- most of them -- skips
  // the per-slot mask (columns holding no token compute unmasked scores
  // that are never stored)
  if (t0 + 32 <= full_to) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float raw = e < 4 ? sacc[0][e] : sacc[1][e - 4];
      sv[e] = FOLD ? raw : raw * mul[e];
    }
  } else {
    // slot e of lane group j is key t0 + 4 j + (e < 4 ? e : 12 + e)
    const int bound = (CAUSAL ? lim : t_end) - t0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float raw = e < 4 ? sacc[0][e] : sacc[1][e - 4];
      const bool live = 4 * j < bound - (e < 4 ? e : 12 + e);
      sv[e] = live ? (FOLD ? raw : raw * mul[e]) : -INFINITY;
    }
  }
  float mx = sv[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
  mx = xor_max(mx, 16);
  mx = xor_max(mx, 32);
  if constexpr (FOLD) mx *= qk_mul;  // (-inf stays -inf: qk_mul > 0)
  // (LAZY: keep the old reference unless the tile's maximum passes it by
  // more than the margin; -inf + margin is -inf, so a first finite
  // maximum always moves it)
  const bool grow = !LAZY || mx > st.m + kLazyMargin;
  const float m_new = LAZY ? (grow ? mx : st.m) : fmaxf(st.m, mx);
  const float m_use = CAUSAL && m_new == -INFINITY ? 0.f : m_new;
  // (LAZY: the old sums' factor is needed only in the rare tiles where some
  // column's reference moves; its exponential and the rescale of the
  // accumulators are taken there, in one branch)
  float alpha = 1.f;
  if constexpr (LAZY) {
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      alpha = grow ? fast_exp2(st.m - m_use) : 1.f;
      if constexpr (!PT) {  // (PT: the accumulators have their own reference)
#pragma unroll
        for (int n = 0; n < S::NBLK; ++n) st.o[n] *= alpha;
      }
    }
  } else {
    alpha = fast_exp2(st.m - m_use);
  }
  float pv[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pv[e] = FOLD ? fast_exp2(__builtin_fmaf(sv[e], qk_mul, -m_use))
                 : fast_exp2(sv[e] - m_use);
    psum += pv[e];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  float orescale = alpha;
  if constexpr (PT) {
    float u[8];
    float mxv = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u[e] = sv[e] == -INFINITY ? -INFINITY : sv[e] + lvs[e];
      mxv = fmaxf(mxv, u[e]);
    }
    mxv = xor_max(mxv, 16);
    mxv = xor_max(mxv, 32);
    // the accumulators' reference, lazy as the scores' one: the weights fed
    // to the PV product stay below 2^8
    const bool grow_v = !LAZY || mxv > st.mv + kLazyMargin;
    const float mv_new = LAZY ? (grow_v ? mxv : st.mv) : fmaxf(st.mv, mxv);
    const float mv_use = mv_new == -INFINITY ? 0.f : mv_new;
    if constexpr (LAZY) {
      if (__builtin_amdgcn_ballot_w64(grow_v) != 0) {
        const float f = grow_v ? fast_exp2(st.mv - mv_use) : 1.f;
#pragma unroll
        for (int n = 0; n < S::NBLK; ++n) st.o[n] *= f;
      }
    } else {
      orescale = fast_exp2(st.mv - mv_use);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(u[e] - mv_use);
    st.mv = mv_new;
  }
  if constexpr (!LAZY) {
#pragma unroll
    for (int n = 0; n < S::NBLK; ++n) st.o[n] *= orescale;
  }

  if constexpr (PVB == 2) {
    // pairs of weights rounded to the 16-bit type in one packed conversion;
    // with the split, the residual of each (exact in float32) rounded again
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t h = f32x2_to_bits(pv[2 * w], pv[2 * w + 1], PVT{});
      pb_hi[w] = h;
      if constexpr (S::PSPLIT && FOLD)
        pb_lo[w] = f32x2_to_bits(minus_element<false>(pv[2 * w], h, PVT{}),
                                 minus_element<true>(pv[2 * w + 1], h, PVT{}),
                                 PVT{});
      else if constexpr (S::PSPLIT)
        pb_lo[w] = f32x2_to_bits(pv[2 * w] - lo_bits_to_f32(h, PVT{}),
                                 pv[2 * w + 1] - hi_bits_to_f32(h, PVT{}),
                                 PVT{});
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) pb_hi[e] = pv[e];
  }
}

// V^T of output block n (16 columns of D) in the PV A-operand layout.
template <typename QT, typename CT, int D>
__device__ __forceinline__ void v_operand(
    const uint8_t* vt, int n, int lane,
    typename Mma<typename Shape<QT, CT, D>::PVT>::operand& va) {
  typedef Shape<QT, CT, D> S;
  constexpr int PVB = S::PVB;
  const int c = lane & 15;
  const int j = lane >> 4;
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
}

// One tile for one 16-column group (LAZY: see softmax_tile).
template <typename QT, typename CT, int D, bool CAUSAL = false, bool PT = false,
          bool LAZY = false>
__device__ __forceinline__ void compute_tile(
    const uint32_t (&kw)[2][Shape<QT, CT, D>::KWORDS], const uint32_t* qw,
    WaveState<Shape<QT, CT, D>::NBLK>& st, uint8_t* vt, int t0, int t_end,
    float qk_mul, int lane, int lim = 0, float sc = 0.f) {
  typedef Shape<QT, CT, D> S;
  typedef typename S::PVT PVT;
  f32x4_t sacc[2];
  qk_tile<QT, CT, D>(kw, qw, sacc);
  typename Mma<PVT>::operand pb_hi, pb_lo;
  softmax_tile<QT, CT, D, CAUSAL, PT, LAZY>(sacc, st, t0, t_end, lim,
                                            CAUSAL ? INT_MIN : t_end, qk_mul,
                                            lane, pb_hi, pb_lo, sc);
  // output blocks two at a time, so that a block's lo step does not wait
  // right behind its own hi step (same order per accumulator)
  static_assert(S::NBLK % 2 == 0, "pairs of output blocks");
#pragma unroll
  for (int n = 0; n < S::NBLK; n += 2) {
    typename Mma<PVT>::operand va0, va1;
    v_operand<QT, CT, D>(vt, n, lane, va0);
    v_operand<QT, CT, D>(vt, n + 1, lane, va1);
    st.o[n] = Mma<PVT>::step(va0, pb_hi, st.o[n]);
    st.o[n + 1] = Mma<PVT>::step(va1, pb_hi, st.o[n + 1]);
    if constexpr (S::PSPLIT) {
      st.o[n] = Mma<PVT>::step(va0, pb_lo, st.o[n]);
      st.o[n + 1] = Mma<PVT>::step(va1, pb_lo, st.o[n + 1]);
    }
  }
}

// One tile for NG 16-column groups of query columns (causal limits per
// group, lim_lo[g] the smallest limit among the group's token columns,
// wave-uniform): the tile's K registers and each V^T read serve every group.
template <typename QT, typename CT, int D, int NG, bool PT = false,
          bool LAZY = false, bool FOLD = false>
__device__ __forceinline__ void compute_tile_groups(
    const uint32_t (&kw)[2][Shape<QT, CT, D>::KWORDS],
    const uint32_t (&qw)[NG][Shape<QT, CT, D>::QWORDS],
    WaveState<Shape<QT, CT, D>::NBLK> (&st)[NG], uint8_t* vt, int t0,
    const int (&lim)[NG], const int (&lim_lo)[NG], float qk_mul, int lane,
    float sc = 0.f) {
  typedef Shape<QT, CT, D> S;
  typedef typename S::PVT PVT;
  typename Mma<PVT>::operand pb_hi[NG], pb_lo[NG];
  // (several groups: the QK products and softmax steps run at a raised wave
  // priority, so that while one wave works through them the SIMD's other
  // wave's PV MFMAs fill the matrix unit -- measured 647 -> 632 us on chunked
  // prefill; raising it around the PV MFMAs instead changed nothing)
  if constexpr (NG > 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    f32x4_t sacc[2];
    qk_tile<QT, CT, D>(kw, qw[g], sacc);
    softmax_tile<QT, CT, D, true, PT, LAZY, FOLD>(sacc, st[g], t0, 0, lim[g],
                                                  lim_lo[g], qk_mul, lane,
                                                  pb_hi[g], pb_lo[g], sc);
  }
  if constexpr (NG > 1) __builtin_amdgcn_s_setprio(0);
  if constexpr (NG == 1) {
    // (one group: output blocks two at a time, as compute_tile)
#pragma unroll
    for (int n = 0; n < S::NBLK; n += 2) {
      typename Mma<PVT>::operand va0, va1;
      v_operand<QT, CT, D>(vt, n, lane, va0);
      v_operand<QT, CT, D>(vt, n + 1, lane, va1);
      st[0].o[n] = Mma<PVT>::step(va0, pb_hi[0], st[0].o[n]);
      st[0].o[n + 1] = Mma<PVT>::step(va1, pb_hi[0], st[0].o[n + 1]);
      if constexpr (S::PSPLIT) {
        st[0].o[n] = Mma<PVT>::step(va0, pb_lo[0], st[0].o[n]);
        st[0].o[n + 1] = Mma<PVT>::step(va1, pb_lo[0], st[0].o[n + 1]);
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < S::NBLK; ++n) {
      typename Mma<PVT>::operand va;
      v_operand<QT, CT, D>(vt, n, lane, va);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        st[g].o[n] = Mma<PVT>::step(va, pb_hi[g], st[g].o[n]);
        if constexpr (S::PSPLIT)
          st[g].o[n] = Mma<PVT>::step(va, pb_lo[g], st[g].o[n]);
      }
    }
  }
}

// With per-token value scales: O^T from units of 2^mv back to units of 2^m
// (an empty state stays zero).
template <int NBLK>
__device__ __forceinline__ void fold_value_scales(WaveState<NBLK>& st) {
  const float f = st.mv == -INFINITY ? 0.f : fast_exp2(st.mv - st.m);
#pragma unroll
  for (int n = 0; n < NBLK; ++n) st.o[n] *= f;
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

// (The fused multiply-adds are written out, so that every instance of the
// fold rounds the same way whatever the compiler would contract: a row's
// result then depends only on its pieces, not on the merge's batching.)
__device__ __forceinline__ void lse_fold(float& m, float& l, f32x4_t& acc,
                                         float m2, float l2, f32x4_t acc2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both empty
  const float a1 = fast_exp2(m - M), a2 = fast_exp2(m2 - M);
  l = __builtin_fmaf(l2, a2, l * a1);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(acc2[e], a2, acc[e] * a1);
  m = M;
}

// The fold of one cut row's pieces (all threads of the workgroup call it):
// wf is the row's first wave, npieces its piece count, q_first the slot of
// its first piece in that wave; output column g goes to row row_of(g) of
// ``out`` (head_dim floats each), times vscale (an fp8 cache's value scale
// for the row's kv head, else 1).  THREADS is the workgroup's size (red_*
// hold THREADS entries); each item folds its pieces in the same order
// whatever it is.
template <int D, int BATCH, typename RowOf, int THREADS = kMergeThreads>
__device__ __forceinline__ void merge_row(const AttnArgs& a, int wf,
                                          int npieces, int q_first,
                                          int gcount, RowOf row_of,
                                          float vscale, f32x4_t* red_o,
                                          float* red_m, float* red_l) {
  constexpr int D4 = D / 4;
  const int tid = threadIdx.x;
  const int gmax = a.slot_heads;
  const int items = gcount * D4;
  if (items > THREADS) {
    // More than one item per thread: thread tid folds items it and
    // it + THREADS together (it = tid, tid + 2 THREADS, ...), so
    // the loads of both are in flight at once.  Each item folds its pieces
    // in order, as below.
    constexpr int HB = BATCH / 2 > 0 ? BATCH / 2 : 1;
    const uint32_t step = 2u * (uint32_t)gmax;
    for (int it = tid; it < items; it += 2 * THREADS) {
      const int itb = it + THREADS;
      const bool has_b = itb < items;
      const int ga = it / D4, da = it - ga * D4;
      const int gb = has_b ? itb / D4 : ga, db = has_b ? itb - gb * D4 : da;
      const uint32_t sla = (uint32_t)(slot_index(wf, 0) * gmax + ga);
      const uint32_t slb = (uint32_t)(slot_index(wf, 0) * gmax + gb);
      float ma = -INFINITY, la = 0.f, mb = -INFINITY, lb = 0.f;
      f32x4_t acca = {0.f, 0.f, 0.f, 0.f}, accb = {0.f, 0.f, 0.f, 0.f};
      for (int i0 = 0; i0 < npieces; i0 += HB) {
        float mi[2][HB], li[2][HB];
        f32x4_t oi[2][HB];
#pragma unroll
        for (int k = 0; k < HB; ++k) {
          const int i = i0 + k;
          const uint32_t q = i == 0 ? (uint32_t)(q_first * gmax) : 0u;
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            mi[x][k] = -INFINITY;
            li[x][k] = 0.f;
            oi[x][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (i < npieces && (x == 0 || has_b)) {
              const uint32_t sl = (x ? slb : sla) + step * (uint32_t)i + q;
              mi[x][k] = load_at<float>(a.part_m, sl * 4u);
              li[x][k] = load_at<float>(a.part_l, sl * 4u);
              oi[x][k] = load_at<f32x4_t>(
                  a.part_o, (sl * (uint32_t)D + 4u * (x ? db : da)) * 4u);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < HB; ++k) {
          lse_fold(ma, la, acca, mi[0][k], li[0][k], oi[0][k]);
          lse_fold(mb, lb, accb, mi[1][k], li[1][k], oi[1][k]);
        }
      }
      *reinterpret_cast<f32x4_t*>(a.out + row_of(ga) * D + 4 * da) =
          acca * (vscale / la);
      if (has_b)
        *reinterpret_cast<f32x4_t*>(a.out + row_of(gb) * D + 4 * db) =
            accb * (vscale / lb);
    }
    return;
  }
  // (sub-sums as with kMergeThreads threads whatever THREADS is, so that the
  // fold order, and with it every bit, does not depend on the launch)
  const int nsub = items >= kMergeThreads ? 1 : kMergeThreads / items;
  for (int it = tid; it < items * nsub; it += THREADS) {
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
      const float f = vscale / l;
      *reinterpret_cast<f32x4_t*>(a.out + row_of(g) * D + 4 * d4) = acc * f;
    } else {
      red_o[it] = acc;
      red_m[it] = m;
      red_l[it] = l;
    }
  }
  if (nsub > 1) {
    __syncthreads();
    for (int item = tid; item < items; item += THREADS) {
      const int g = item / D4;
      const int d4 = item - g * D4;
      float m = red_m[item], l = red_l[item];
      f32x4_t acc = red_o[item];
      for (int sub = 1; sub < nsub; ++sub)
        lse_fold(m, l, acc, red_m[sub * items + item], red_l[sub * items + item],
                 red_o[sub * items + item]);
      const float f = vscale / l;
      *reinterpret_cast<f32x4_t*>(a.out + row_of(g) * D + 4 * d4) = acc * f;
    }
  }
}

// An fp8 cache's key / value scale for kv head h (one per tensor, or one per
// kv head when a.scale_per_head).
__device__ __forceinline__ float head_scale(const float* scale,
                                            const AttnArgs& a, int h) {
  return scale[a.scale_per_head ? h : 0];
}

// Inclusive scan of one int per thread across the workgroup.
__device__ __forceinline__ int block_inclusive_scan(int v, int* sm_wsum) {
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

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
// Compute units of the current device and the workgroups of `kernel` one CU
// holds at once with dyn_lds bytes of dynamic LDS.  The answers depend only
// on the device, the kernel and the LDS size, so they are asked of the
// runtime once per (kernel instance, device, LDS size) and kept: later calls
// cost one hipGetDevice and a lookup under a lock.  (The LDS size follows
// the number of sequences, so a serving loop meets a bounded set of them.)
// (Every kernel here has the same type, so the kernel's address is part of
// the key: instances differ in registers and so in occupancy.)
template <typename K>
static bool device_occupancy(K kernel, size_t dyn_lds, int* cus, int* per_cu) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, std::pair<int, int>>
      cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  const auto key =
      std::make_tuple(dev, reinterpret_cast<const void*>(kernel), dyn_lds);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) {
      *cus = it->second.first;
      *per_cu = it->second.second;
      return true;
    }
  }
  int c = 0, p = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &p, reinterpret_cast<const void*>(kernel), kThreads, dyn_lds) !=
          hipSuccess)
    return false;
  {
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = {c, p};
  }
  *cus = c;
  *per_cu = p;
  return true;
}

// Workgroups of the partition kernel: as many as can be resident at once
// (occupancy x CUs), capped by the caller's wave limit and kMaxWaves.
template <typename K>
static int resident_grid(K kernel, size_t dyn_lds, int max_waves,
                         int per_cu_cap = kWorkgroupsPerCU) {
  int cus = 0, per_cu = 0;
  if (!device_occupancy(kernel, dyn_lds, &cus, &per_cu)) return -1;
  // One workgroup (one wave per SIMD) per CU measured fastest for the
  // streaming loop: more resident waves deepen the memory queues without
  // adding bandwidth.
  int64_t g = (int64_t)(per_cu < per_cu_cap ? per_cu : per_cu_cap) * cus;
  if (g < cus) g = cus;
  int64_t cap = kMaxWaves / kWaves;
  if (max_waves > 0 && max_waves / kWaves < cap) cap = max_waves / kWaves;
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

}  // namespace pkv

#endif  // PKV_ATTN_TILE_H
