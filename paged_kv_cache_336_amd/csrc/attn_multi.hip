// attn_multi.hip -- paged attention for several new query tokens per
// sequence (a prompt chunk against a cached prefix, or the draft tokens a
// speculative decoder verifies) on gfx950.
//
// What it computes: the read path of "PagedAttention" (shubhamtatvamasi.com,
// section "How attention reads paged memory") with more than one query per
// sequence.  Sequence s holds L_s tokens; its last q_s are new (their K/V
// already written), and new token j, at position L_s - q_s + j, attends to
// tokens 0 .. L_s - q_s + j: causal within the new tokens, everything before
// them.
//
// Work split: as for one token per sequence (attn_decode.hip), with the
// MFMA's 16 query columns packing (token, head) pairs: a column group holds
// tpr = 16 / G consecutive new tokens of one kv head, their G query heads
// token-major.  A row is (sequence, kv head, NG consecutive groups): the
// wave computing a tile of it runs the tile's K registers and V reads
// through all NG groups, so a sequence's keys and values are read once per
// NG * tpr new tokens (NG = 4 for long query runs such as a prompt chunk,
// 1 for a few drafted tokens).  Every row of a sequence spans the
// sequence's ceil(L_s / 32) tiles in the unit list; tiles past the row's
// last column limit are neither loaded nor computed, and inside the row
// each column masks keys past its own token.  All units of all rows are
// divided evenly among the waves and rows cut between waves are merged by
// log-sum-exp in a second kernel, exactly as in the one-token case.  With
// one new token per sequence this is the one-token kernel's split and
// arithmetic.

#include "attn_tile.h"

namespace pkv {

// A segment of a multi-query row.
struct MSeg : Seg {
  int rr;  // row within its (sequence, kv head): tokens rr * row_tokens ..
  int q0;  // first query row of the sequence
  int nq;  // new tokens of the sequence
  int L;   // its length
};

// Extent of sequence i as the kernels use it.  Values outside the caller's
// contract are clamped so that nothing is addressed outside the buffers: the
// length to [0, max_seq_len], the first query row to [0, num_query_tokens],
// the new-token count to the rows left, the length and max_query_len.
struct MqSeq {
  int L, q0, nq;
};
__device__ __forceinline__ MqSeq mq_seq(const AttnArgs& a, int i) {
  MqSeq m;
  m.L = min(max(a.seq_lens[i], 0), a.max_seq_tokens);
  m.q0 = min(max(a.query_start[i], 0), a.num_query_tokens);
  const int q1 = min(max(a.query_start[i + 1], m.q0), a.num_query_tokens);
  m.nq = min(min(q1 - m.q0, m.L), a.max_query_len);
  return m;
}

// LDS per sequence: tex[num_seqs + 1] (exclusive prefix of the unit counts)
// | lens | first query row | new-token count.
__device__ __forceinline__ MSeg mseg_at(int64_t t, int64_t te, const int* tex,
                                        const int* lens, const int* qs0,
                                        const int* qn, const AttnArgs& a) {
  MSeg g;
  g.valid = t < te;
  g.gc = 0;
  if (!g.valid) {
    g.s = g.h = g.rr = g.q0 = g.nq = g.L = 0;
    g.t_begin = g.t_end = g.ntiles = g.wb = 0;
    g.full = false;
    return g;
  }
  const int ti = (int)t;  // unit indices fit an int32 (checked on the host)
  int lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(tex[mid]) <= ti) lo = mid;
    else hi = mid - 1;
  }
  const int base = __builtin_amdgcn_readfirstlane(tex[lo]);
  const int L = __builtin_amdgcn_readfirstlane(lens[lo]);
  const int nq = __builtin_amdgcn_readfirstlane(qn[lo]);
  const int ts = (L + 31) / 32;
  const int rps = (nq + a.row_tokens - 1) / a.row_tokens;
  const int r = ti - base;
  const int u = r / ts;
  const int k0 = r - u * ts;
  const int64_t row_end = (int64_t)base + (int64_t)(u + 1) * ts;
  const int64_t end = te < row_end ? te : row_end;
  g.s = lo;
  g.h = u / rps;
  g.rr = u - g.h * rps;
  g.q0 = __builtin_amdgcn_readfirstlane(qs0[lo]);
  g.nq = nq;
  g.L = L;
  g.ntiles = (int)(end - t);
  g.t_begin = 32 * k0;
  // the row's last column sees tokens up to L - nq + (its token) + 1
  const int tok_end = L - nq + min(nq, (g.rr + 1) * a.row_tokens);
  g.t_end = min(tok_end, 32 * (k0 + g.ntiles));
  g.wb = g.t_begin / a.block_size;
  g.full = k0 == 0 && end == row_end;
  return g;
}

// Lane column c of group grp of a row: token rr * row_tokens + grp * tpr +
// c / G of the sequence's new ones, query head h * G + c % G; -1 past the
// row's tokens.
__device__ __forceinline__ int mq_token(const MSeg& g, const AttnArgs& a,
                                        int grp, int c) {
  const int tok = g.rr * a.row_tokens + grp * a.tpr + c / a.group;
  return g.valid && c < a.tpr * a.group && tok < g.nq ? tok : -1;
}

// Group grp's query rows as a B operand (zeros for columns past the row's
// tokens).
template <typename QT, typename CT, int D>
__device__ __forceinline__ void load_query_mq(uint32_t* qw, const MSeg& g,
                                              const AttnArgs& a, int grp,
                                              int lane) {
  typedef Shape<QT, CT, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int tok = mq_token(g, a, grp, c);
  // a column past the row's tokens reads beyond the range: zeros, no traffic
  const uint32_t rowoff =
      tok >= 0 ? ((uint32_t)(g.q0 + tok) * (uint32_t)a.num_q_heads +
                  (uint32_t)(g.h * a.group + c % a.group)) *
                     (uint32_t)(D * QT::bytes)
               : 0x80000000u;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.query), (short)0,
      __builtin_amdgcn_readfirstlane((int)a.query_bytes), kRawBufferFlags);
  constexpr int QBYTES_PER_R = S::EP * QT::bytes;
  constexpr int QLOADS = QBYTES_PER_R / 16;
#pragma unroll
  for (int rr = 0; rr < D / (4 * S::EP); ++rr) {
#pragma unroll
    for (int k = 0; k < QLOADS; ++k) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          r, rowoff + (4 * rr + j) * QBYTES_PER_R + 16 * k, 0, 0);
      const int w0 = (rr * QBYTES_PER_R + 16 * k) / 4;
      qw[w0 + 0] = v[0];
      qw[w0 + 1] = v[1];
      qw[w0 + 2] = v[2];
      qw[w0 + 3] = v[3];
    }
  }
}

// Key limit of this lane's column of group grp in segment g (0: the column
// sees nothing).
__device__ __forceinline__ int mq_limit(const MSeg& g, const AttnArgs& a,
                                        int grp, int lane) {
  const int tok = mq_token(g, a, grp, lane & 15);
  return tok >= 0 ? min(g.t_end, g.L - g.nq + tok + 1) : 0;
}

// The smallest key limit among the columns of group grp that hold a token
// (INT_MAX when none does), the same in every lane: a tile whose keys all
// lie below it needs no causal mask.
__device__ __forceinline__ int mq_limit_lo(int lim, const MSeg& g,
                                           const AttnArgs& a, int grp,
                                           int lane) {
  int v = mq_token(g, a, grp, lane & 15) >= 0 ? lim : INT_MAX;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = min(v, __shfl_xor(v, m, 64));
  return __builtin_amdgcn_readfirstlane(v);
}

// NG = 1 keeps the one-token kernel's register budget (two waves per SIMD
// possible); NG = 4 needs up to 512 registers per lane (one wave per SIMD,
// which is what the grid runs anyway).
template <int NG> struct MultiOccupancy { static constexpr int waves = 2; };
template <> struct MultiOccupancy<4> { static constexpr int waves = 1; };

// PT: per-token fp8 scales (a.k_scale / a.v_scale are [num_blocks,
// block_size, num_kv_heads] arrays read beside the rows).
template <typename QT, typename CT, int D, bool UNIFORM, int NG,
          bool PT = false, int AUX = 0>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(MultiOccupancy<NG>::waves)))
void attn_multi_kernel(AttnArgs a) {
  typedef Shape<QT, CT, D> S;
  static_assert(!PT || is_fp8<CT>::value, "per-token scales: fp8 caches");
  static_assert(S::SUB == 1, "one 32-token sub-tile per tile");
  constexpr int NBLK = S::NBLK;
  // (four groups leave no registers for a second tile in flight)
  constexpr bool PREFETCH = UNIFORM && CT::bytes <= 2 && NG == 1;

  __shared__ __attribute__((aligned(16))) uint8_t smem[kWaves * S::STAGE_BYTES];
  __shared__ int sm_wsum[kWaves];
  extern __shared__ int sm_seq[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int nS = a.num_seqs;
  int* tex = sm_seq;
  int* lens = tex + nS + 1;
  int* qs0 = lens + nS;
  int* qn = qs0 + nS;

  // ---- unit counts of all sequences (kv heads x rows x tiles) and their
  // exclusive prefix ----
  {
    const int per = (nS + kThreads - 1) / kThreads;
    const int b0 = min(tid * per, nS);
    const int b1 = min(b0 + per, nS);
    int sum = 0;
    for (int i = b0; i < b1; ++i) {
      const MqSeq m = mq_seq(a, i);
      lens[i] = m.L;
      qs0[i] = m.q0;
      qn[i] = m.nq;
      sum += a.num_kv_heads * ((m.nq + a.row_tokens - 1) / a.row_tokens) *
             ((m.L + 31) / 32);
    }
    const int incl = block_inclusive_scan(sum, sm_wsum);
    int run = incl - sum;
    for (int i = b0; i < b1; ++i) {
      tex[i] = run;
      run += a.num_kv_heads * ((qn[i] + a.row_tokens - 1) / a.row_tokens) *
             ((lens[i] + 31) / 32);
    }
    if (tid == kThreads - 1) tex[nS] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0)  // the merge kernel reads the prefix from here
    for (int i = tid; i <= nS; i += kThreads) a.tile_prefix[i] = tex[i];

  const int W = a.num_waves;
  const int w = split_workgroup(blockIdx.x, gridDim.x, !a.kv_stream) * kWaves +
                wave;
  const int64_t T = tex[nS];
  const int64_t tb = first_tile_of_wave(w, T, W);
  const int64_t te = first_tile_of_wave(w + 1, T, W);

  const int64_t stride = (int64_t)a.num_kv_heads * S::ROW_BYTES;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_cache);
  uint8_t* vt = smem + wave * S::STAGE_BYTES;
  const int gmax = a.slot_heads;

  MSeg X = mseg_at(tb, te, tex, lens, qs0, qn, a);
  int64_t pos_n = tb + X.ntiles;
  MSeg Xn = mseg_at(pos_n, te, tex, lens, qs0, qn, a);
  bool first_seg = true;
  uint32_t ta = 0, tbw = 0, ta_n = 0, tb_n = 0;
  if constexpr (UNIFORM) {
    ta = load_window(X, 0, a, lane);
    tbw = load_window(X, 1, a, lane);
    ta_n = load_window(Xn, 0, a, lane);
    tb_n = load_window(Xn, 1, a, lane);
  }
  // One group: the next segment's query rows are requested when a segment
  // starts (as in the one-token kernel).  Four: there are no registers for a
  // second set, and each segment's are loaded when it starts.
  constexpr bool QPREFETCH = NG == 1;
  uint32_t qw[NG][S::QWORDS];
#pragma unroll
  for (int g = 0; g < NG; ++g) load_query_mq<QT, CT, D>(qw[g], X, a, g, lane);
  auto token_scales = [&](const MSeg& g) {
    return TokenScales{a.k_scale + g.h, a.v_scale + g.h, a.num_kv_heads};
  };
  TileRegs<QT, CT, D> cur;
  if constexpr (PREFETCH)
    load_tile_uniform<QT, CT, D, PT, AUX>(cur, a.block_size, a.num_blocks, ta, tbw,
                                     X.wb, kpool + (int64_t)X.h * S::ROW_BYTES,
                                     vpool + (int64_t)X.h * S::ROW_BYTES,
                                     stride, X.t_begin, X.t_end, lane,
                                     token_scales(X));

  while (X.valid) {
    float kscale = 1.f, vscale = 1.f;  // an fp8 cache's, for this kv head
    if constexpr (is_fp8<CT>::value && !PT) {
      kscale = head_scale(a.k_scale, a, X.h);
      vscale = head_scale(a.v_scale, a, X.h);
    }
    const float qk_mul = a.qk_scale_log2 * kscale;
    const TokenScales tsc = token_scales(X);
    uint32_t qn_w[QPREFETCH ? NG : 1][S::QWORDS];
    int lim[NG], lim_lo[NG];
    WaveState<NBLK> st[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if constexpr (QPREFETCH)
        load_query_mq<QT, CT, D>(qn_w[g], Xn, a, g, lane);
      lim[g] = mq_limit(X, a, g, lane);
      lim_lo[g] = mq_limit_lo(lim[g], X, a, g, lane);
      st[g].m = -INFINITY;
      st[g].mv = -INFINITY;
      st[g].l = 0.f;
#pragma unroll
      for (int n = 0; n < NBLK; ++n) st[g].o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const uint8_t* kbase = kpool + (int64_t)X.h * S::ROW_BYTES;
    const uint8_t* vbase = vpool + (int64_t)X.h * S::ROW_BYTES;
    if constexpr (PREFETCH) {
      const uint8_t* kbase_n = kpool + (int64_t)Xn.h * S::ROW_BYTES;
      const uint8_t* vbase_n = vpool + (int64_t)Xn.h * S::ROW_BYTES;
      int wb = X.wb;
      for (int k = 0; k < X.ntiles; ++k) {
        const int t0 = X.t_begin + 32 * k;
        const bool live = t0 < X.t_end;  // tiles past the row's columns: none
        if (live) stage_v<QT, CT, D>(cur.vraw[0], vt, lane);
        const bool same_seg = k + 1 < X.ntiles;
        const int t_next = t0 + 32;
        if (same_seg && t_next / a.block_size - wb >= 64) {
          wb += 64;
          ta = tbw;
          Seg shifted = X;
          shifted.wb = wb;
          tbw = load_window(shifted, 1, a, lane);
        }
        TileRegs<QT, CT, D> nxt;
        load_tile_uniform<QT, CT, D, PT, AUX>(
            nxt, a.block_size, a.num_blocks, same_seg ? ta : ta_n,
            same_seg ? tbw : tb_n, same_seg ? wb : Xn.wb,
            same_seg ? kbase : kbase_n, same_seg ? vbase : vbase_n, stride,
            same_seg ? t_next : Xn.t_begin, same_seg ? X.t_end : Xn.t_end,
            lane, same_seg ? tsc : token_scales(Xn));
        __builtin_amdgcn_sched_barrier(0);
        if (live)
          compute_tile_groups<QT, CT, D, NG, PT, true>(cur.kw[0], qw, st, vt, t0,
                                                 lim, lim_lo, qk_mul, lane,
                                                 cur.sc[0]);
        cur = nxt;
      }
    } else {
      const int32_t* trow = a.block_tables + (int64_t)X.s * a.max_blocks_per_seq;
      for (int k = 0; k < X.ntiles; ++k) {
        const int t0 = X.t_begin + 32 * k;
        if (t0 >= X.t_end) break;  // the rest of the row is past its columns
        if constexpr (UNIFORM) {
          const int wb = X.wb + (t0 / a.block_size - X.wb) / 64 * 64;
          Seg shifted = X;
          shifted.wb = wb;
          const uint32_t wa = load_window(shifted, 0, a, lane);
          const uint32_t wbb = load_window(shifted, 1, a, lane);
          load_tile_uniform<QT, CT, D, PT, AUX>(cur, a.block_size, a.num_blocks,
                                           wa, wbb, wb, kbase, vbase, stride,
                                           t0, X.t_end, lane, tsc);
        } else {
          load_tile_any<QT, CT, D, PT>(cur, a.block_size, a.num_blocks, trow,
                                       kbase, vbase, stride, t0, X.t_end,
                                       lane, tsc);
        }
        stage_v<QT, CT, D>(cur.vraw[0], vt, lane);
        compute_tile_groups<QT, CT, D, NG, PT, true>(cur.kw[0], qw, st, vt, t0, lim,
                                               lim_lo, qk_mul, lane, cur.sc[0]);
      }
    }
    if constexpr (PT) {
#pragma unroll
      for (int g = 0; g < NG; ++g) fold_value_scales(st[g]);
    }

    // ---------------- the segment's output (this wave alone) ----------------
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float l_tot = xor_sum(st[g].l, 16);
      l_tot = xor_sum(l_tot, 32);
      const int tok = mq_token(X, a, g, c);
      if (tok < 0) continue;
      if (X.full) {
        const int64_t row = (int64_t)(X.q0 + tok) * a.num_q_heads +
                            X.h * a.group + c % a.group;
        const float f = l_tot > 0.f ? vscale / l_tot : 0.f;
        float* dst = a.out + row * D + 4 * j;
#pragma unroll
        for (int n = 0; n < NBLK; ++n)
          *reinterpret_cast<f32x4_t*>(dst + 16 * n) = st[g].o[n] * f;
      } else {
        // slot column: the token's place in the row times G plus the head
        const int64_t sl = slot_index(w, first_seg ? 0 : 1) * gmax +
                           g * a.tpr * a.group + c;
        float* dst = a.part_o + sl * D + 4 * j;
#pragma unroll
        for (int n = 0; n < NBLK; ++n)
          *reinterpret_cast<f32x4_t*>(dst + 16 * n) = st[g].o[n];
        if (j == 0) {
          a.part_m[sl] = st[g].m;
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
    for (int g = 0; g < NG; ++g) {
      if constexpr (QPREFETCH) {
#pragma unroll
        for (int q = 0; q < S::QWORDS; ++q) qw[g][q] = qn_w[g][q];
      } else {
        load_query_mq<QT, CT, D>(qw[g], X, a, g, lane);
      }
    }
    pos_n += X.ntiles;
    Xn = mseg_at(pos_n, te, tex, lens, qs0, qn, a);
    if constexpr (UNIFORM) {
      ta_n = load_window(Xn, 0, a, lane);
      tb_n = load_window(Xn, 1, a, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// Long query runs (a prompt chunk against its cached prefix), 16-bit caches
// with block_size % 16 == 0: rows of kPrefillGroups = 8 column groups, one
// row per workgroup at a time.  The split is over workgroups; the four waves
// walk the same tiles in lockstep, wave w computing groups 2w, 2w + 1, and
// each tile's K and V rows are loaded once per workgroup: every thread
// fetches 1/256 of the tile into registers two tiles ahead, stores it into
// one of two LDS buffers one tile ahead, and all waves read the tile from
// LDS (K rows XOR-swizzled by 16-byte piece for conflict-free operand
// reads, V rows in the span-permuted layout the transposing reads use).  So
// a sequence's K/V is read once per 8 * tpr new tokens (32 at G = 4), and a
// tile's loads are in flight for two tile steps of the whole workgroup.
// Two groups per wave keep a wave under 256 registers, so two workgroups
// share each CU and one wave's softmax overlaps the other's MFMAs (one
// wave per SIMD with four groups each left the matrix cores idle during
// every softmax).
// ---------------------------------------------------------------------------
constexpr int kPrefillGPW = 2;                  // groups per wave
constexpr int kPrefillGroups = kPrefillGPW * kWaves;
constexpr int kPrefillWGsPerCU = 2;             // two waves per SIMD

// One thread's share of a tile's K and V rows (16-byte pieces q = tid + 256 i
// of the tile's 32 x D/8 pieces: token q / (D/8), piece q % (D/8)).
template <int D> struct PrefillStage {
  static constexpr int PPR = D / 8;               // 16-byte pieces per row
  static constexpr int CH = 32 * PPR / kThreads;  // per thread: 2 or 1
  u32x4_t k[CH], v[CH];
};

// Issue the loads of tile t0 of segment X (rows past X.t_end read as zero
// and are not fetched).  Every wave's pieces of one load lie in one 16-token
// half, whose block id a readlane takes from the wave's table window.  The
// tile's first token is token off0 of logical block lb0 (the caller advances
// the pair tile by tile, so no division by block_size is needed here;
// block_size is a multiple of 16, so a half never straddles two blocks).
template <typename ET, int D>
__device__ __forceinline__ void prefill_load(PrefillStage<D>& st,
                                             const MSeg& X, int t0, int lb0,
                                             int off0, uint32_t ta,
                                             uint32_t tb, int wb,
                                             const AttnArgs& a, int tid) {
  constexpr int PPR = PrefillStage<D>::PPR;
  constexpr int ROW = D * ET::bytes;
  const int64_t stride = (int64_t)a.num_kv_heads * ROW;
  const uint8_t* kbase =
      static_cast<const uint8_t*>(a.k_cache) + (int64_t)X.h * ROW;
  const uint8_t* vbase =
      static_cast<const uint8_t*>(a.v_cache) + (int64_t)X.h * ROW;
#pragma unroll
  for (int i = 0; i < PrefillStage<D>::CH; ++i) {
    const int q = tid + kThreads * i;
    const int r = q / PPR;
    const int x = q - r * PPR;
    const int hh = __builtin_amdgcn_readfirstlane(r >> 4);
    const int th = __builtin_amdgcn_readfirstlane(t0 + 16 * hh);
    int nvalid = X.t_end - th;
    nvalid = nvalid < 0 ? 0 : (nvalid > 16 ? 16 : nvalid);
    int64_t row0 = 0;
    if (nvalid > 0) {
      int lb = lb0, off = off0 + 16 * hh;  // token th of the sequence
      if (off >= a.block_size) {
        off -= a.block_size;
        ++lb;
      }
      const int idx = lb - wb;  // 0 .. 127
      int phys = idx < 64 ? __builtin_amdgcn_readlane(ta, idx)
                          : __builtin_amdgcn_readlane(tb, idx - 64);
      phys = (uint32_t)phys < (uint32_t)a.num_blocks ? phys : a.num_blocks - 1;
      row0 = (int64_t)phys * a.block_size + off;
    }
    const int nrec = __builtin_amdgcn_readfirstlane(nvalid * (int)stride);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kbase + row0 * stride), (short)0, nrec,
        kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(vbase + row0 * stride), (short)0, nrec,
        kRawBufferFlags);
    const int off = (r - 16 * hh) * (int)stride + x * 16;
    st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0);
    st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0);
  }
}

// LDS byte offset of piece x of K row r: pieces XOR-permuted by row, so the
// 16 rows one operand read touches fall on distinct banks.
template <int D>
__device__ __forceinline__ int prefill_k_at(int r, int x) {
  constexpr int PPR = D / 8;
  return r * (D * 2) + ((x ^ (r & (PPR - 1))) << 4);
}

template <int D>
__device__ __forceinline__ void prefill_store(const PrefillStage<D>& st,
                                              uint8_t* kb, uint8_t* vb,
                                              int tid) {
  constexpr int PPR = PrefillStage<D>::PPR;
  constexpr int SPANS = D * 2 / 32;
#pragma unroll
  for (int i = 0; i < PrefillStage<D>::CH; ++i) {
    const int q = tid + kThreads * i;
    const int r = q / PPR;
    const int x = q - r * PPR;
    *reinterpret_cast<u32x4_t*>(kb + prefill_k_at<D>(r, x)) = st.k[i];
    // the layout stage_v gives a 16-bit V row (32-byte spans permuted by
    // token), which v_operand's transposing reads expect
    const int span = (x >> 1) ^ (r & (SPANS - 1));
    *reinterpret_cast<u32x4_t*>(vb + r * (D * 2) + (span << 5) +
                                ((x & 1) << 4)) = st.v[i];
  }
}

// The tile's K rows as this lane's MFMA A operand (token 16 hh + c, pieces
// 4 r + j), as load_tile_uniform leaves them in registers.
template <typename ET, int D>
using KRegs = uint32_t[2][Shape<ET, ET, D>::KWORDS];

template <typename ET, int D>
__device__ __forceinline__ void prefill_k_operand(KRegs<ET, D>& kw,
                                                  const uint8_t* kb, int lane) {
  typedef Shape<ET, ET, D> S;
  const int c = lane & 15;
  const int j = lane >> 4;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int r = 0; r < S::KPIECES; ++r) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
          kb + prefill_k_at<D>(16 * hh + c, 4 * r + j));
      kw[hh][4 * r + 0] = v[0];
      kw[hh][4 * r + 1] = v[1];
      kw[hh][4 * r + 2] = v[2];
      kw[hh][4 * r + 3] = v[3];
    }
  }
}

template <typename ET, int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kPrefillWGsPerCU)))
void attn_prefill_kernel(AttnArgs a) {
  typedef Shape<ET, ET, D> S;
  static_assert(ET::bytes == 2, "16-bit caches");
  constexpr int NG = kPrefillGPW;  // groups per wave
  constexpr int TILE = 32 * D * 2;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][TILE];
  __shared__ __attribute__((aligned(16))) uint8_t vbuf[2][TILE];
  __shared__ int sm_wsum[kWaves];
  extern __shared__ int sm_seq[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  const int nS = a.num_seqs;
  int* tex = sm_seq;
  int* lens = tex + nS + 1;
  int* qs0 = lens + nS;
  int* qn = qs0 + nS;

  // ---- unit counts of all sequences and their exclusive prefix (as in
  // attn_multi_kernel) ----
  {
    const int per = (nS + kThreads - 1) / kThreads;
    const int b0 = min(tid * per, nS);
    const int b1 = min(b0 + per, nS);
    int sum = 0;
    for (int i = b0; i < b1; ++i) {
      const MqSeq m = mq_seq(a, i);
      lens[i] = m.L;
      qs0[i] = m.q0;
      qn[i] = m.nq;
      sum += a.num_kv_heads * ((m.nq + a.row_tokens - 1) / a.row_tokens) *
             ((m.L + 31) / 32);
    }
    const int incl = block_inclusive_scan(sum, sm_wsum);
    int run = incl - sum;
    for (int i = b0; i < b1; ++i) {
      tex[i] = run;
      run += a.num_kv_heads * ((qn[i] + a.row_tokens - 1) / a.row_tokens) *
             ((lens[i] + 31) / 32);
    }
    if (tid == kThreads - 1) tex[nS] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0)  // the merge kernel reads the prefix from here
    for (int i = tid; i <= nS; i += kThreads) a.tile_prefix[i] = tex[i];

  const int W = a.num_waves;  // ranges: one per workgroup
  const int w = split_workgroup(blockIdx.x, gridDim.x, !a.kv_stream);
  const int gbase = wave * NG;
  const int64_t T_all = tex[nS];
  const int64_t tb = first_tile_of_wave(w, T_all, W);
  const int64_t te = first_tile_of_wave(w + 1, T_all, W);
  const int64_t n = te - tb;  // tiles of this workgroup (the same in every wave)
  const int gmax = a.slot_heads;

  // ---- the loading side: its segment, tile and table windows, and the
  // next segment's windows ----
  MSeg LX = mseg_at(tb, te, tex, lens, qs0, qn, a);
  int64_t lpos_n = tb + LX.ntiles;
  MSeg LXn = mseg_at(lpos_n, te, tex, lens, qs0, qn, a);
  int lk = 0;
  int lwb = LX.wb;
  // the next tile's first token: token loff of logical block lblk
  int lblk = LX.wb, loff = LX.t_begin - LX.wb * a.block_size;
  uint32_t lta = load_window(LX, 0, a, lane), ltb = load_window(LX, 1, a, lane);
  uint32_t lta_n = load_window(LXn, 0, a, lane);
  uint32_t ltb_n = load_window(LXn, 1, a, lane);
  auto load_next = [&](PrefillStage<D>& st) {
    const int t0 = LX.valid ? LX.t_begin + 32 * lk : 0;
    if (LX.valid && lblk - lwb >= 64) {
      // the window moves on by 64 blocks (at most once per tile)
      lwb += 64;
      lta = ltb;
      Seg shifted = LX;
      shifted.wb = lwb;
      ltb = load_window(shifted, 1, a, lane);
    }
    prefill_load<ET, D>(st, LX, t0, lblk, loff, lta, ltb, lwb, a, tid);
    loff += 32;  // (block_size 16 crosses two blocks per tile)
    if (loff >= a.block_size) {
      loff -= a.block_size;
      ++lblk;
      if (loff >= a.block_size) {
        loff -= a.block_size;
        ++lblk;
      }
    }
    if (LX.valid && ++lk == LX.ntiles) {
      LX = LXn;
      lk = 0;
      lwb = LX.wb;
      lblk = LX.wb;
      loff = LX.t_begin - LX.wb * a.block_size;
      lta = lta_n;
      ltb = ltb_n;
      lpos_n += LX.ntiles;
      LXn = mseg_at(lpos_n, te, tex, lens, qs0, qn, a);
      lta_n = load_window(LXn, 0, a, lane);
      ltb_n = load_window(LXn, 1, a, lane);
    }
  };

  // ---- the computing side ----
  MSeg X = mseg_at(tb, te, tex, lens, qs0, qn, a);
  int64_t pos_n = tb + X.ntiles;
  int k = 0;  // tile within X
  bool first_seg = true;
  uint32_t qw[NG][S::QWORDS];
  int lim[NG], lim_lo[NG];
  WaveState<S::NBLK> st[NG];
  // the score multiplier goes into each weight's exponent (softmax_tile's
  // FOLD), which needs it positive: a negative one becomes its magnitude
  // with the query negated, and zero the smallest normal float (every
  // weight then still rounds to 1)
  const float qk_mul = a.qk_scale_log2 == 0.f ? 1.17549435e-38f
                                              : fabsf(a.qk_scale_log2);
  const uint32_t qflip = a.qk_scale_log2 < 0.f ? 0x80008000u : 0u;
  auto start_segment = [&]() {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      load_query_mq<ET, ET, D>(qw[g], X, a, gbase + g, lane);
#pragma unroll
      for (int q = 0; q < S::QWORDS; ++q) qw[g][q] ^= qflip;
      lim[g] = mq_limit(X, a, gbase + g, lane);
      lim_lo[g] = mq_limit_lo(lim[g], X, a, gbase + g, lane);
      st[g].m = -INFINITY;
      st[g].l = 0.f;
#pragma unroll
      for (int nb = 0; nb < S::NBLK; ++nb)
        st[g].o[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto finish_segment = [&]() {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float l_tot = xor_sum(st[g].l, 16);
      l_tot = xor_sum(l_tot, 32);
      const int tok = mq_token(X, a, gbase + g, c);
      if (tok < 0) continue;
      if (X.full) {
        const int64_t row = (int64_t)(X.q0 + tok) * a.num_q_heads +
                            X.h * a.group + c % a.group;
        const float f = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* dst = a.out + row * D + 4 * j;
#pragma unroll
        for (int nb = 0; nb < S::NBLK; ++nb)
          *reinterpret_cast<f32x4_t*>(dst + 16 * nb) = st[g].o[nb] * f;
      } else {
        // slot column: the token's place in the row times G plus the head
        const int64_t sl = slot_index(w, first_seg ? 0 : 1) * gmax +
                           (gbase + g) * a.tpr * a.group + c;
        float* dst = a.part_o + sl * D + 4 * j;
#pragma unroll
        for (int nb = 0; nb < S::NBLK; ++nb)
          *reinterpret_cast<f32x4_t*>(dst + 16 * nb) = st[g].o[nb];
        if (j == 0) {
          a.part_m[sl] = st[g].m;
          a.part_l[sl] = l_tot;
        }
      }
    }
  };
  // tile p of the range: its loads were issued two steps back and its LDS
  // buffer filled one step back; it fills the other buffer with tile p + 1
  // (held in `next`), reloads `next` with tile p + 3, computes, and the
  // barrier both publishes tile p + 1 and frees buffer b for tile p + 2
  auto tile_step = [&](PrefillStage<D>& next, int b) {
    prefill_store<D>(next, kbuf[b ^ 1], vbuf[b ^ 1], tid);
    load_next(next);
    if (k == 0) start_segment();
    const int t0 = X.t_begin + 32 * k;
    if (t0 < X.t_end) {  // (tiles past the row's columns hold nothing)
      uint32_t kw[2][S::KWORDS];
      prefill_k_operand<ET, D>(kw, kbuf[b], lane);
      compute_tile_groups<ET, ET, D, NG, false, true, true>(kw, qw, st, vbuf[b],
                                                      t0, lim, lim_lo, qk_mul,
                                                      lane);
    }
    __syncthreads();
    if (++k == X.ntiles) {
      finish_segment();
      first_seg = false;
      X = mseg_at(pos_n, te, tex, lens, qs0, qn, a);
      pos_n += X.ntiles;
      k = 0;
    }
  };

  if (n > 0) {
    PrefillStage<D> A, B;
    load_next(A);  // tile 0
    load_next(B);  // tile 1
    prefill_store<D>(A, kbuf[0], vbuf[0], tid);
    load_next(A);  // tile 2
    __syncthreads();
    for (int64_t p = 0; p < n; p += 2) {
      tile_step(B, 0);                  // tile p (buffer 0), B: p+1 -> p+3
      if (p + 1 < n) tile_step(A, 1);   // tile p+1 (buffer 1), A: p+2 -> p+4
    }
  }
}

// Merge of a cut multi-query row: workgroup (s, h, rr) over a grid of
// num_seqs * num_kv_heads * max_rps (rows past a sequence's count exit).
template <int D, bool SCALED, int BATCH, int THREADS = kMergeThreads>
__global__ __launch_bounds__(THREADS) void attn_multi_merge_kernel(
    AttnArgs a) {
  __shared__ __attribute__((aligned(16))) f32x4_t red_o[THREADS];
  __shared__ float red_m[THREADS], red_l[THREADS];
  const int rr = (int)(blockIdx.x % (unsigned)a.max_rps);
  const int sh = (int)(blockIdx.x / (unsigned)a.max_rps);
  const int h = sh % a.num_kv_heads;
  const int s = sh / a.num_kv_heads;
  const MqSeq m = mq_seq(a, s);
  const int rps = (m.nq + a.row_tokens - 1) / a.row_tokens;
  if (rr >= rps) return;
  const int ts = (m.L + 31) / 32;
  const int* tex = a.tile_prefix;
  const int64_t T = tex[a.num_seqs];
  const int W = a.num_waves;
  const int64_t r0 = (int64_t)tex[s] + (int64_t)(h * rps + rr) * ts;
  const int wf = wave_of_tile(r0, T, W);
  const int wl = wave_of_tile(r0 + ts - 1, T, W);
  if (wf == wl) return;  // finished by one wave
  const int npieces = wl - wf + 1;
  const int q_first = first_tile_of_wave(wf, T, W) < r0 ? 1 : 0;
  const int G = a.group;
  const int gcount = min(a.row_tokens, m.nq - rr * a.row_tokens) * G;
  const int64_t tok0 = (int64_t)m.q0 + rr * a.row_tokens;
  auto row_of = [&](int g) {
    return (tok0 + g / G) * a.num_q_heads + h * G + g % G;
  };
  merge_row<D, BATCH, decltype(row_of), THREADS>(
      a, wf, npieces, q_first, gcount, row_of,
      SCALED ? head_scale(a.v_scale, a, h) : 1.f, red_o, red_m, red_l);
}

template <typename QT, typename CT, int D, bool UNIFORM, int NG,
          bool PT = false, int AUX = 0>
static hipError_t launch_mu(AttnArgs a, int max_waves, hipStream_t stream) {
  auto kernel = attn_multi_kernel<QT, CT, D, UNIFORM, NG, PT, AUX>;
  constexpr bool SCALED = is_fp8<CT>::value && !PT;  // merge: output scale
  const size_t dyn = ((size_t)4 * a.num_seqs + 1) * sizeof(int);
  const int cap = max_waves > 0 && max_waves < kMaxWavesMulti ? max_waves
                                                              : kMaxWavesMulti;
  const int grid = resident_grid(kernel, dyn, cap);
  if (grid < 0) return hipErrorInvalidValue;
  a.num_waves = grid * kWaves;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), dyn, stream, a);
  const int64_t rows = (int64_t)a.num_seqs * a.num_kv_heads * a.max_rps;
  if (rows > 0 && a.num_waves >= 4 * rows && a.slot_heads * D / 4 >= 512)
    // (rows of 512 column quads or more: one quad per thread)
    hipLaunchKernelGGL((attn_multi_merge_kernel<D, SCALED, 16, 512>),
                       dim3((unsigned)rows), dim3(512), 0, stream, a);
  else if (rows > 0 && a.num_waves >= 4 * rows)
    hipLaunchKernelGGL((attn_multi_merge_kernel<D, SCALED, 16>),
                       dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, a);
  else if (rows > 0)
    hipLaunchKernelGGL((attn_multi_merge_kernel<D, SCALED, 4>),
                       dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename ET, int D>
static hipError_t launch_prefill(AttnArgs a, int max_waves,
                                 hipStream_t stream) {
  auto kernel = attn_prefill_kernel<ET, D>;
  const size_t dyn = ((size_t)4 * a.num_seqs + 1) * sizeof(int);
  // ranges of kPrefillGroups groups: the workspace's 1024 * 4 group slots
  // per slot pair hold 4096 / kPrefillGroups of them
  constexpr int kMaxRanges = kMaxWavesMulti * kMaxGroupsMulti / kPrefillGroups;
  const int cap = max_waves > 0 && max_waves < kMaxRanges * kWaves
                      ? max_waves : kMaxRanges * kWaves;
  const int grid = resident_grid(kernel, dyn, cap, kPrefillWGsPerCU);
  if (grid < 0) return hipErrorInvalidValue;
  a.num_waves = grid;  // one range per workgroup
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), dyn, stream, a);
  const int64_t rows = (int64_t)a.num_seqs * a.num_kv_heads * a.max_rps;
  if (rows > 0 && a.num_waves >= 4 * rows)
    hipLaunchKernelGGL((attn_multi_merge_kernel<D, false, 16>),
                       dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, a);
  else if (rows > 0)
    hipLaunchKernelGGL((attn_multi_merge_kernel<D, false, 4>),
                       dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename QT, typename CT, int D>
static hipError_t launch_md(const AttnArgs& a, int max_waves, bool uniform,
                            hipStream_t stream) {
  if constexpr (same<QT, CT>::value && QT::bytes == 2) {
    if (uniform && a.row_tokens / a.tpr == kPrefillGroups)
      return launch_prefill<QT, D>(a, max_waves, stream);
  }
  if constexpr (is_fp8<CT>::value) {
    if (a.scale_per_token) {
      if constexpr (!same<QT, F32>::value) {
        if (a.row_tokens / a.tpr == 4) {
          if (uniform)
            return launch_mu<QT, CT, D, true, 4, true>(a, max_waves, stream);
          return launch_mu<QT, CT, D, false, 4, true>(a, max_waves, stream);
        }
      }
      if (uniform)
        return launch_mu<QT, CT, D, true, 1, true>(a, max_waves, stream);
      return launch_mu<QT, CT, D, false, 1, true>(a, max_waves, stream);
    }
  }
  // unshared batches fetch V rows of 128 bytes or more with non-temporal
  // loads, as the decode kernel does (per-token scales excepted)
  if constexpr (!same<QT, F32>::value && D * CT::bytes >= 128) {
    if (uniform && a.kv_stream && !a.scale_per_token) {
      if (a.row_tokens / a.tpr == 4)
        return launch_mu<QT, CT, D, true, 4, false, kLoadNT>(a, max_waves,
                                                             stream);
      return launch_mu<QT, CT, D, true, 1, false, kLoadNT>(a, max_waves,
                                                           stream);
    }
  }
  if constexpr (!same<QT, F32>::value) {
    if (a.row_tokens / a.tpr == 4) {
      if (uniform) return launch_mu<QT, CT, D, true, 4>(a, max_waves, stream);
      return launch_mu<QT, CT, D, false, 4>(a, max_waves, stream);
    }
  }
  if (uniform) return launch_mu<QT, CT, D, true, 1>(a, max_waves, stream);
  return launch_mu<QT, CT, D, false, 1>(a, max_waves, stream);
}

template <typename QT, typename CT>
static hipError_t launch_mt(const AttnArgs& a, int head_dim, int max_waves,
                            bool uniform, hipStream_t stream) {
  if (head_dim == 64) return launch_md<QT, CT, 64>(a, max_waves, uniform, stream);
  return launch_md<QT, CT, 128>(a, max_waves, uniform, stream);
}

int multi_groups_per_row(int q_dtype, int cache_dtype, bool uniform,
                         bool token_scales, int max_query_len, int tpr) {
  const int groups = (max_query_len + tpr - 1) / tpr;
  // workgroup rows of kPrefillGroups groups for long query runs on 16-bit
  // caches with block_size % 16 == 0
  if (q_dtype == cache_dtype && (q_dtype == PKV_BF16 || q_dtype == PKV_F16) &&
      uniform && !token_scales && groups >= 12)
    return kPrefillGroups;
  // four groups once a row would hold three or more (float32 queries keep
  // one: their operands alone fill the registers)
  if (q_dtype == PKV_F32) return 1;
  return groups >= 3 ? 4 : 1;
}

hipError_t launch_attn_multi(const AttnArgs& a, int q_dtype, int cache_dtype,
                             int head_dim, int max_waves, hipStream_t stream) {
  const bool uniform = (a.block_size % 16) == 0;
  switch (cache_dtype) {
    case PKV_F32: return launch_mt<F32, F32>(a, head_dim, max_waves, uniform, stream);
    case PKV_F16: return launch_mt<F16, F16>(a, head_dim, max_waves, uniform, stream);
    case PKV_BF16: return launch_mt<BF16, BF16>(a, head_dim, max_waves, uniform, stream);
    case PKV_FP8_E4M3:
      if (q_dtype == PKV_BF16) return launch_mt<BF16, FP8>(a, head_dim, max_waves, uniform, stream);
      if (q_dtype == PKV_F16) return launch_mt<F16, FP8>(a, head_dim, max_waves, uniform, stream);
      return launch_mt<F32, FP8>(a, head_dim, max_waves, uniform, stream);
    case PKV_FP8_E5M2:
      if (q_dtype == PKV_BF16) return launch_mt<BF16, FP8E5>(a, head_dim, max_waves, uniform, stream);
      if (q_dtype == PKV_F16) return launch_mt<F16, FP8E5>(a, head_dim, max_waves, uniform, stream);
      return launch_mt<F32, FP8E5>(a, head_dim, max_waves, uniform, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
