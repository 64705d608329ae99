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
//   * K rows go from HBM into MFMA A-operand registers as 16-byte loads
//     (lane = token row + 16 * piece group) -- or, with the streaming hint,
//     are loaded as whole 128-byte lines like the V rows (so they can
//     stream), staged in the wave's LDS and read back in that layout --; Q
//     sits in the B operand;
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

#include "attn_tile.h"
#include "kv_encode.h"

namespace pkv {

template <int D, bool SCALED, int BATCH>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) f32x4_t red_o[kMergeThreads];
  __shared__ float red_m[kMergeThreads], red_l[kMergeThreads];

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
  const int64_t head0 = (int64_t)s * a.num_q_heads + h * a.group + gc * 16;

  const float vscale = SCALED ? head_scale(a.v_scale, a, h) : 1.f;
  merge_row<D, BATCH>(a, wf, npieces, q_first, gcount,
                      [&](int g) { return head0 + g; }, vscale, red_o, red_m,
                      red_l);
}

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
// Fused write (paged_attn_decode_fused): the new token of a row's sequence --
// position L - 1, slot slot_mapping[s] -- is written into both pools by the
// wave whose segment reaches the row's end, before that wave loads any tile
// of the segment.  The row is the only reader of that position for its kv
// head (one query-head chunk per kv head), so write-then-read within one wave
// gives exactly the separate write followed by attention.  Lanes 0..PPR-1
// write the K row's 16-byte pieces, lanes 32..32+PPR-1 the V row's; an fp8
// cache stores e4m3(x / scale) as cache_write_slots does.
// ---------------------------------------------------------------------------
template <typename QT, typename CT, int D>
__device__ __forceinline__ void write_new_token(const Seg& g, int L,
                                                const AttnArgs& a, int lane) {
  typedef Shape<QT, CT, D> S;
  if (!g.valid || g.t_end != L || L == 0) return;
  const int slot = a.slot_mapping[g.s];
  if (slot < 0 || (int64_t)slot >= a.num_slots) return;  // no write
  const int half = lane >> 5;  // 0: K, 1: V
  const int pc = lane & 31;
  if (pc >= S::PPR) return;
  uint8_t* dst = static_cast<uint8_t*>(const_cast<void*>(
                     half ? a.v_cache : a.k_cache)) +
                 ((int64_t)slot * a.num_kv_heads + g.h) * S::ROW_BYTES + 16 * pc;
  const uint8_t* src =
      static_cast<const uint8_t*>(half ? a.new_value : a.new_key) +
      ((int64_t)g.s * a.num_kv_heads + g.h) * D * QT::bytes;
  if constexpr (is_fp8<CT>::value) {
    u32x4_t in[QT::bytes];  // the piece's 16 source elements
#pragma unroll
    for (int q = 0; q < QT::bytes; ++q)
      in[q] = *reinterpret_cast<const u32x4_t*>(src + 16 * (QT::bytes * pc + q));
    const float sc = head_scale(half ? a.v_scale : a.k_scale, a, g.h);
    *reinterpret_cast<u32x4_t*>(dst) = encode_piece_fp8<QT, CT>(in, sc);
  } else {
    *reinterpret_cast<u32x4_t*>(dst) =
        *reinterpret_cast<const u32x4_t*>(src + 16 * pc);
  }
}

// Waits until this wave's stores have completed, so its later loads of the
// same bytes see them.
__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt(7), lgkmcnt(15)
}

// ---------------------------------------------------------------------------
// Partition kernel: wave w streams tiles [ceil(w T / W), ceil((w+1) T / W))
// of the row-major tile list, one segment (run of one row) after another.
// The next segment's query rows and table window are requested when a
// segment starts and its first tile during the current segment's last tile,
// so a wave's loads run on across segment boundaries.
// ---------------------------------------------------------------------------
// PT: per-token fp8 scales (a.k_scale / a.v_scale are [num_blocks,
// block_size, num_kv_heads] arrays read beside the rows).
template <typename QT, typename CT, int D, bool UNIFORM, bool WRITE,
          bool PT = false, int AUX = 0>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_decode_kernel(AttnArgs a) {
  typedef Shape<QT, CT, D> S;
  constexpr int NBLK = S::NBLK;
  constexpr bool PREFETCH = UNIFORM && CT::bytes <= 2;
  // K rows through LDS where they stream (AUX: the batch's hint): loaded as
  // whole lines like the V rows, then read back as the MFMA operand
  constexpr bool KL = PREFETCH && AUX != 0;
  constexpr int KST = KL ? S::KSTAGE_BYTES : 0;
  static_assert(!PT || (is_fp8<CT>::value && !WRITE),
                "per-token scales: fp8 caches, separate write");

  __shared__ __attribute__((aligned(16)))
  uint8_t smem[kWaves * (S::STAGE_BYTES + KST)];
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
  const int w = split_workgroup(blockIdx.x, gridDim.x, !a.kv_stream) * kWaves +
                wave;
  const int64_t T = (int64_t)U * tex[nS];
  const int64_t tb = first_tile_of_wave(w, T, W);
  const int64_t te = first_tile_of_wave(w + 1, T, W);


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

  const int64_t stride = (int64_t)a.num_kv_heads * S::ROW_BYTES;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_cache);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_cache);
  uint8_t* vt = smem + wave * S::STAGE_BYTES;
  uint8_t* kt = smem + kWaves * S::STAGE_BYTES + wave * KST;
  const int gmax = a.slot_heads;

  Seg X = segment_at<S::TT>(tb, te, U, tex, lens, a);
  int64_t pos_n = tb + X.ntiles;  // first tile of the next segment
  Seg Xn = segment_at<S::TT>(pos_n, te, U, tex, lens, a);
  bool first_seg = true;
  if constexpr (WRITE) {
    write_new_token<QT, CT, D>(X, lens[X.s], a, lane);
    write_new_token<QT, CT, D>(Xn, lens[Xn.s], a, lane);
    wait_stores();
  }
  uint32_t ta = 0, tbw = 0, ta_n = 0, tb_n = 0;
  if constexpr (UNIFORM) {
    ta = load_window(X, 0, a, lane);
    tbw = load_window(X, 1, a, lane);
    ta_n = load_window(Xn, 0, a, lane);
    tb_n = load_window(Xn, 1, a, lane);
  }
  uint32_t qw[S::QWORDS];
  load_query<QT, CT, D>(qw, X, a, lane);
  // per-token scales of a row's kv head
  auto token_scales = [&](const Seg& g) {
    return TokenScales{a.k_scale + g.h, a.v_scale + g.h, a.num_kv_heads};
  };
  TileRegs<QT, CT, D> cur;
  if constexpr (PREFETCH)
    load_tile_uniform<QT, CT, D, PT, AUX, KL>(cur, a.block_size, a.num_blocks, ta, tbw,
                                     X.wb, kpool + (int64_t)X.h * S::ROW_BYTES,
                                     vpool + (int64_t)X.h * S::ROW_BYTES,
                                     stride, X.t_begin, X.t_end, lane,
                                     token_scales(X));

  while (X.valid) {
    uint32_t qn[S::QWORDS];
    load_query<QT, CT, D>(qn, Xn, a, lane);
    // an fp8 cache's scales for this row's kv head: the key scale folds into
    // the score multiplier, the value scale into the output (per-token
    // scales go into each token's score and PV weight instead)
    float kscale = 1.f, vscale = 1.f;
    if constexpr (is_fp8<CT>::value && !PT) {
      kscale = head_scale(a.k_scale, a, X.h);
      vscale = head_scale(a.v_scale, a, X.h);
    }
    const float qk_mul = a.qk_scale_log2 * kscale;
    const TokenScales tsc = token_scales(X);

    WaveState<NBLK> st;
    st.m = -INFINITY;
    st.mv = -INFINITY;
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
        // the next tile of this wave's stream: tile k + 1 of X, else the
        // first tile of the next segment (an empty range past the end);
        // requested before this tile's V rows are waited for and staged, so
        // that two tiles are in flight during that wait, and kept there by
        // the scheduling barrier (the compiler would otherwise sink the loads
        // to shorten register lifetimes)
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
        load_tile_uniform<QT, CT, D, PT, AUX, KL>(
            nxt, a.block_size, a.num_blocks, same_seg ? ta : ta_n, same_seg ? tbw : tb_n,
            same_seg ? wb : Xn.wb, same_seg ? kbase : kbase_n,
            same_seg ? vbase : vbase_n, stride,
            same_seg ? t_next : Xn.t_begin, same_seg ? X.t_end : Xn.t_end,
            lane, same_seg ? tsc : token_scales(Xn));
        __builtin_amdgcn_sched_barrier(0);
        stage_v<QT, CT, D>(cur.vraw[0], vt, lane);
        if constexpr (KL) {
          stage_k<QT, CT, D>(cur.kraw[0], kt, lane);
          uint32_t kw[2][S::KWORDS];
          k_from_lds<QT, CT, D>(kw, kt, lane);
          compute_tile<QT, CT, D, false, PT, true>(kw, qw, st, vt, t0, X.t_end,
                                             qk_mul, lane, 0, cur.sc[0]);
        } else {
          compute_tile<QT, CT, D, false, PT, true>(cur.kw[0], qw, st, vt, t0,
                                             X.t_end, qk_mul, lane, 0,
                                             cur.sc[0]);
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
          load_tile_uniform<QT, CT, D, PT, AUX>(cur, a.block_size, a.num_blocks,
                                           wa, wbb, wb, kbase, vbase, stride,
                                           t0, X.t_end, lane, tsc);
        } else {
          load_tile_any<QT, CT, D, PT>(cur, a.block_size, a.num_blocks, trow,
                                       kbase, vbase, stride, t0, X.t_end,
                                       lane, tsc);
        }
#pragma unroll
        for (int sb = 0; sb < S::SUB; ++sb) {
          if (t0 + 32 * sb < X.t_end) {
            stage_v<QT, CT, D>(cur.vraw[sb], vt, lane);
            compute_tile<QT, CT, D, false, PT, true>(cur.kw[sb], qw, st, vt,
                                               t0 + 32 * sb, X.t_end, qk_mul,
                                               lane, 0, cur.sc[sb]);
          }
        }
      }
    }
    if constexpr (PT) fold_value_scales(st);

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
    if constexpr (WRITE) {
      write_new_token<QT, CT, D>(Xn, lens[Xn.s], a, lane);
      wait_stores();
    }
    if constexpr (UNIFORM) {
      ta_n = load_window(Xn, 0, a, lane);
      tb_n = load_window(Xn, 1, a, lane);
    }
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <typename T> struct DtypeCode;
template <> struct DtypeCode<F32> { static constexpr int value = PKV_F32; };
template <> struct DtypeCode<F16> { static constexpr int value = PKV_F16; };
template <> struct DtypeCode<BF16> { static constexpr int value = PKV_BF16; };
template <> struct DtypeCode<FP8> { static constexpr int value = PKV_FP8_E4M3; };
template <> struct DtypeCode<FP8E5> { static constexpr int value = PKV_FP8_E5M2; };

template <typename QT, typename CT, int D, bool UNIFORM, bool WRITE,
          bool PT = false, int AUX = 0>
static hipError_t launch_u(AttnArgs a, int max_waves, hipStream_t stream) {
  auto kernel = attn_decode_kernel<QT, CT, D, UNIFORM, WRITE, PT, AUX>;
  constexpr bool SCALED = is_fp8<CT>::value && !PT;  // merge: output scale
  const size_t dyn = ((size_t)2 * a.num_seqs + 1) * sizeof(int);
  const int grid = resident_grid(kernel, dyn, max_waves);
  if (grid < 0) return hipErrorInvalidValue;
  a.num_waves = grid * kWaves;
  if constexpr (WRITE) {
    // With more rows than waves most waves end several rows, and each row
    // end waits for its store before streaming on; the write then goes
    // faster as its own launch ahead of the plain kernel (same result).
    if ((int64_t)a.num_seqs * a.num_kv_heads > a.num_waves) {
      WriteArgs w{};
      w.key = a.new_key;
      w.value = a.new_value;
      w.k_cache = const_cast<void*>(a.k_cache);
      w.v_cache = const_cast<void*>(a.v_cache);
      w.slot_mapping = a.slot_mapping;
      w.k_scale = a.k_scale;
      w.v_scale = a.v_scale;
      w.num_tokens = a.num_seqs;
      w.num_slots = a.num_slots;
      w.block_size = a.block_size;
      w.row_elems = a.num_kv_heads * D;
      w.head_dim = D;
      w.scale_per_head = a.scale_per_head;
      const hipError_t e = launch_cache_write(w, DtypeCode<QT>::value,
                                              DtypeCode<CT>::value, stream);
      if (e != hipSuccess) return e;
      return launch_u<QT, CT, D, UNIFORM, false, false, AUX>(a, max_waves,
                                                             stream);
    }
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), dyn, stream, a);
  // Pieces per cut row grow with the wave boundaries per row: fetch them in
  // batches of 16 when there are about 4 or more boundaries per row, else 4
  // (fewer registers, so the mostly idle workgroups of many-row batches
  // launch in one round).
  const int rows = a.num_seqs * a.num_kv_heads * a.group_chunks;
  if (rows > 0 && a.num_waves >= 4 * rows)
    hipLaunchKernelGGL((attn_merge_kernel<D, SCALED, 16>),
                       dim3(rows), dim3(kMergeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, SCALED, 4>),
                       dim3(rows), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename QT, typename CT, int D>
static hipError_t launch_d(const AttnArgs& a, int max_waves, bool uniform,
                           bool fused, hipStream_t stream) {
  // A batch whose blocks no two sequences share fetches its V rows (of 128
  // bytes or more: whole lines) with non-temporal loads, measured faster;
  // shared prefixes need the caches.
  constexpr bool kLines = D * CT::bytes >= 128;
  if constexpr (is_fp8<CT>::value) {
    if (a.scale_per_token) {  // (never fused: the host rejects it)
      if (fused) return hipErrorInvalidValue;
      if (uniform && a.kv_stream && kLines)
        return launch_u<QT, CT, D, true, false, true, kLoadNT>(a, max_waves,
                                                               stream);
      if (uniform)
        return launch_u<QT, CT, D, true, false, true>(a, max_waves, stream);
      return launch_u<QT, CT, D, false, false, true>(a, max_waves, stream);
    }
  }
  if constexpr (kLines) {
    if (uniform && a.kv_stream) {
      if (fused)
        return launch_u<QT, CT, D, true, true, false, kLoadNT>(a, max_waves,
                                                               stream);
      return launch_u<QT, CT, D, true, false, false, kLoadNT>(a, max_waves,
                                                              stream);
    }
  }
  if (fused) {
    if (uniform) return launch_u<QT, CT, D, true, true>(a, max_waves, stream);
    return launch_u<QT, CT, D, false, true>(a, max_waves, stream);
  }
  if (uniform) return launch_u<QT, CT, D, true, false>(a, max_waves, stream);
  return launch_u<QT, CT, D, false, false>(a, max_waves, stream);
}

template <typename QT, typename CT>
static hipError_t launch_t(const AttnArgs& a, int head_dim, int max_waves,
                           bool uniform, bool fused, hipStream_t stream) {
  if (head_dim == 64)
    return launch_d<QT, CT, 64>(a, max_waves, uniform, fused, stream);
  return launch_d<QT, CT, 128>(a, max_waves, uniform, fused, stream);
}

hipError_t launch_attn_decode(const AttnArgs& a, int q_dtype, int cache_dtype,
                              int head_dim, int max_waves, bool fused,
                              hipStream_t stream) {
  const bool u = (a.block_size % 16) == 0;
  const int hd = head_dim;
  const int mw = max_waves;
  switch (cache_dtype) {
    case PKV_F32: return launch_t<F32, F32>(a, hd, mw, u, fused, stream);
    case PKV_F16: return launch_t<F16, F16>(a, hd, mw, u, fused, stream);
    case PKV_BF16: return launch_t<BF16, BF16>(a, hd, mw, u, fused, stream);
    case PKV_FP8_E4M3:
      if (q_dtype == PKV_BF16) return launch_t<BF16, FP8>(a, hd, mw, u, fused, stream);
      if (q_dtype == PKV_F16) return launch_t<F16, FP8>(a, hd, mw, u, fused, stream);
      return launch_t<F32, FP8>(a, hd, mw, u, fused, stream);
    case PKV_FP8_E5M2:
      if (q_dtype == PKV_BF16) return launch_t<BF16, FP8E5>(a, hd, mw, u, fused, stream);
      if (q_dtype == PKV_F16) return launch_t<F16, FP8E5>(a, hd, mw, u, fused, stream);
      return launch_t<F32, FP8E5>(a, hd, mw, u, fused, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
