// kernels_decode.hip -- block-sparse split-K decode attention and its combine.
//
// Paper: "Elastic Threshold Attention ...".  Attention of the one new query is
// restricted to the admitted blocks and normalised over them (Theoretical
// Foundation, sparse form); inside admitted blocks the logits follow Eq. 3
// (Methodology 2): l_s = S_s * sigmoid(beta (S_s - tau)) except for the
// query's own key s = T-1, which is never gated; only admitted blocks are read
// from HBM and folded into an online softmax (Fig. 6).  Dense mode walks every
// block with raw logits (plain decode attention, the in-house baseline).
//
// Work decomposition.  Sparse decode (decode_flow_kernel): the admitted lists
// of all streams, concatenated, are cut into one equal range per wave; each
// wave walks its range alone and writes a partial per stream it touches, and a
// combine kernel merges each stream's partials (log-sum-exp).  Dense decode,
// and sparse decode over more streams than the balanced kernel holds, cut each
// stream into chunks of `split` blocks, one work-group of 4 waves per chunk
// (wave w takes the chunk's tiles w, w+4, ...), merged the same way.  Either
// way rows are handled in tiles of kRows rows: a key row of D elements is read
// by LPR lanes with one 128-bit load each (bf16, D=128: 16 lanes), so one load
// instruction of a wave covers RPI = 64/LPR rows and a tile is NI = kRows/RPI
// loads of K plus NI loads of V per lane, all issued before any arithmetic,
// the next tile's loads in flight while the current one is folded in.  Each
// lane group keeps its own running (max, sum, weighted V) over its rows; the
// groups are merged at the end of a range or chunk.
#include "eta_internal.h"

namespace eta {

#ifndef ETA_DECODE_ROWS
#define ETA_DECODE_ROWS 16
#endif
constexpr int kRows = ETA_DECODE_ROWS;  // rows per wave tile

__device__ __forceinline__ float fexp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Merge (m2, l2, a2) into (m, l, a); -inf maxima are handled so that empty
// partials contribute nothing.
template <int E>
__device__ __forceinline__ void merge_state(float& m, float& l, float* a, float m2, float l2,
                                            const float* a2) {
  const float mn = fmaxf(m, m2);
  const float ms = (mn == -__builtin_inff()) ? 0.f : mn;
  const float s1 = fexp(m - ms), s2 = fexp(m2 - ms);
  l = l * s1 + l2 * s2;
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = a[e] * s1 + a2[e] * s2;
  m = mn;
}

// Running softmax state of one lane group over the rows it has folded in:
// reference max m, sum l of e^(logit - m), and the e^(logit - m)-weighted sum
// of its EPL value columns.
template <int EPL>
struct RowState {
  float m, l, acc[EPL];
  __device__ __forceinline__ void reset() {
    m = -__builtin_inff();
    l = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  }
};

// Fold one loaded tile into st: NI rows per lane group, row i holding key
// sp[i] (-1: no key) with its K and V chunks kr[i], vr[i].  Logits follow
// Eq. 3 in GATED mode (the query's own key T - 1 ungated), raw otherwise.
template <int D, int DT, int MODE, int NI>
__device__ __forceinline__ void fold_tile(RowState<Elt<DT>::kPer16B>& st, const uint4* kr,
                                          const uint4* vr, const int* sp, const float* qs,
                                          float tau, float beta, int T) {
  constexpr int EPL = Elt<DT>::kPer16B;
  constexpr int LPR = D / EPL;
  float lg[NI];
  float tmax = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float x[EPL];
    widen<DT>(kr[i], x);
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) d = fmaf(qs[e], x[e], d);
    d = group_sum<LPR>(d);
    float lv = d;
    if (MODE == ETA_LOGIT_GATED && sp[i] != T - 1)
      lv = d * __builtin_amdgcn_rcpf(1.f + fexp(-beta * (d - tau)));
    lg[i] = sp[i] >= 0 ? lv : -__builtin_inff();
    tmax = fmaxf(tmax, lg[i]);
  }
  const float mn = fmaxf(st.m, tmax);
  const float ms = (mn == -__builtin_inff()) ? 0.f : mn;
  const float alpha = fexp(st.m - ms);
  st.l *= alpha;
#pragma unroll
  for (int e = 0; e < EPL; ++e) st.acc[e] *= alpha;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float p = fexp(lg[i] - ms);
    st.l += p;
    float y[EPL];
    widen<DT>(vr[i], y);
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[e] = fmaf(p, y[e], st.acc[e]);
  }
  st.m = mn;
}

// Merge the RPI row groups of a wave (xor butterfly: partners end equal).
template <int EPL, int LPR>
__device__ __forceinline__ void merge_groups(RowState<EPL>& st) {
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    const float m2 = __shfl_xor(st.m, off, kWave);
    const float l2 = __shfl_xor(st.l, off, kWave);
    float a2[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(st.acc[e], off, kWave);
    merge_state<EPL>(st.m, st.l, st.acc, m2, l2, a2);
  }
}

// Where a chunk's block indices come from: consecutive blocks first,
// first + 1, ... (dense), or a list the caller staged in LDS (the fused
// screen + decode).
enum ChunkSrc { kChunkDense = 0, kChunkStaged = 2 };

// Attention of one chunk (chunk k of stream u, nblk blocks) by the whole
// work-group.  The chunk's block indices sit in LDS (s_list), so no key or
// value load ever waits on an index load.  Writes the final output when the
// chunk is the stream's only one (single), else the partial (max, sum,
// weighted V) into slot k of the stream.
template <int D, int DT, int MODE, int SRC, int NBUF = 2, int NWV = 4>
__device__ __forceinline__ void chunk_attend(const CacheView& c, const DecodeArgs& a, int u, int k,
                                             int T, int first, int nblk, bool single, float tau,
                                             int* s_list, float (*s_acc)[D], float (*s_ml)[2]) {
  constexpr int EPL = Elt<DT>::kPer16B;
  constexpr int LPR = D / EPL;
  constexpr int RPI = kWave / LPR;
  constexpr int NI = (kRows / RPI) > 0 ? (kRows / RPI) : 1;
  constexpr int RB = D * Elt<DT>::kBytes;
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / LPR, li = lane % LPR;

  float qs[EPL];
  {
    const float* qu = a.q + (size_t)u * D + li * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qs[e] = qu[e] * a.scale;
  }
  const float beta = a.beta;
  const char* kb = static_cast<const char*>(c.k) + (size_t)u * c.cap * RB + li * 16;
  const char* vb = static_cast<const char*>(c.v) + (size_t)u * c.cap * RB + li * 16;
  __syncthreads();

  RowState<EPL> st;
  st.reset();

  const int rows = nblk << c.log2bs;
  const int ntiles = (rows + NI * RPI - 1) / (NI * RPI);

  // Issue the K and V loads of tile t (rows t*NI*RPI ... of the chunk).
  auto fetch = [&](int t, uint4* kr, uint4* vr, int* sp) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = (t * NI + i) * RPI + g;  // row within the chunk
      int s = -1;
      if (rr < rows) {
        const int p = rr >> c.log2bs;
        const int j = SRC == kChunkDense ? first + p : s_list[p];
        s = (j << c.log2bs) + (rr & (c.bs - 1));
        // The list is trusted only as far as it stays inside the stream.
        if ((unsigned)j >= (unsigned)nb || s >= T) s = -1;
      }
      sp[i] = s;
      if (s >= 0) {
        kr[i] = ld16_nt(kb + (size_t)s * RB);
        vr[i] = ld16_nt(vb + (size_t)s * RB);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto consume = [&](const uint4* kr, const uint4* vr, const int* sp) {
    fold_tile<D, DT, MODE, NI>(st, kr, vr, sp, qs, tau, beta, T);
  };

  // NBUF register buffers: the loads of a wave's next NBUF - 1 tiles are in
  // flight while its current tile is folded in.  Tiles are folded in the
  // same order (wave, wave + 4, ...) whatever NBUF, so the result is too.
  uint4 kr[NBUF][NI], vr[NBUF][NI];
  int sp[NBUF][NI];
#pragma unroll
  for (int b = 0; b + 1 < NBUF; ++b)
    if (wave + NWV * b < ntiles) fetch(wave + NWV * b, kr[b], vr[b], sp[b]);
  for (int t0 = wave; t0 < ntiles; t0 += NWV * NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int t = t0 + NWV * b, tp = t + NWV * (NBUF - 1);
      if (tp < ntiles) fetch(tp, kr[(b + NBUF - 1) % NBUF], vr[(b + NBUF - 1) % NBUF],
                             sp[(b + NBUF - 1) % NBUF]);
      if (t < ntiles) consume(kr[b], vr[b], sp[b]);
    }
  }

  merge_groups<EPL, LPR>(st);
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wave][li * EPL + e] = st.acc[e];
    if (li == 0) {
      s_ml[wave][0] = st.m;
      s_ml[wave][1] = st.l;
    }
  }
  __syncthreads();
  // Merge the NWV waves in a fixed order; thread i < D owns output column i.
  const int i = threadIdx.x;
  if (i < D) {
    float mm = s_ml[0][0], ll = s_ml[0][1], aa[1] = {s_acc[0][i]};
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
      const float a2[1] = {s_acc[w][i]};
      merge_state<1>(mm, ll, aa, s_ml[w][0], s_ml[w][1], a2);
    }
    if (single) {
      a.out[(size_t)u * D + i] = aa[0] / ll;  // the stream's only chunk: final output
    } else {
      const size_t slot = (size_t)u * a.max_chunks + k;
      a.part_acc[slot * D + i] = aa[0];
      if (i == 0) {
        a.part_m[slot] = mm;
        a.part_l[slot] = ll;
      }
    }
  }
}

__device__ __forceinline__ int stream_chunks(const CacheView& c, const DecodeArgs& a, int u,
                                             int* T_out, int* cnt_out) {
  const int T = c.seq_len[u / c.H];
  const int nb = T > 0 ? (T + c.bs - 1) >> c.log2bs : 0;
  const int cnt = a.dense ? nb : max(0, min(a.active_cnt[u], nb));
  *T_out = T;
  *cnt_out = cnt;
  return (cnt + a.split - 1) / a.split;
}

// Log-sum-exp merge of the nch partials in slots slot0 .. slot0 + nch - 1 into
// out[u], by the whole work-group of NWV waves: wave w folds chunks w, w+NWV,
// ... into a running (max, sum, weighted V) in one pass with kInflight chunks
// loaded before any is used; lane i owns columns [i*CPL, i*CPL+CPL).  The wave
// states are then merged in a fixed order (deterministic).
// 8 waves per combine work-group: against 16, about 1% faster on the 512K
// and the fused 32K steps, the same elsewhere (4: the same or slower).
constexpr int kInflight = 8;
constexpr int kCombWaves = 8;
template <int D, int NWV = kCombWaves>
__device__ void combine_slots(const DecodeArgs& a, int u, size_t slot0, int nch,
                              float (*s_acc)[D], float (*s_ml)[2]) {
  constexpr int CPL = D / kWave;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const float* pm = a.part_m + slot0;
  const float* pl = a.part_l + slot0;
  const float* pa = a.part_acc + slot0 * D + lane * CPL;
  float m = -__builtin_inff(), l = 0.f, acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
  for (int base = wave; base < nch; base += NWV * kInflight) {
    float mc[kInflight], lc[kInflight], ac[kInflight][CPL];
#pragma unroll
    for (int i = 0; i < kInflight; ++i) {
      const int ch = base + NWV * i;
      const bool ok = ch < nch;
      mc[i] = ok ? pm[ch] : -__builtin_inff();
      lc[i] = ok ? pl[ch] : 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) ac[i][e] = ok ? pa[(size_t)ch * D + e] : 0.f;
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < kInflight; ++i) mx = fmaxf(mx, mc[i]);
    const float ms = (mx == -__builtin_inff()) ? 0.f : mx;
    const float alpha = fexp(m - ms);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < kInflight; ++i) {
      const float wgt = fexp(mc[i] - ms);
      l = fmaf(wgt, lc[i], l);
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[e] = fmaf(wgt, ac[i][e], acc[e]);
    }
    m = mx;
  }
#pragma unroll
  for (int e = 0; e < CPL; ++e) s_acc[wave][lane * CPL + e] = acc[e];
  if (lane == 0) {
    s_ml[wave][0] = m;
    s_ml[wave][1] = l;
  }
  __syncthreads();
  if (t < D) {
    float mm = s_ml[0][0], ll = s_ml[0][1], aa[1] = {s_acc[0][t]};
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
      const float a2[1] = {s_acc[w][t]};
      merge_state<1>(mm, ll, aa, s_ml[w][0], s_ml[w][1], a2);
    }
    a.out[(size_t)u * D + t] = aa[0] / ll;
  }
}

// Dense decode (the baseline): one work-group per possible chunk of `split`
// consecutive blocks, blockIdx.x = u * max_chunks + (k + u % 8) mod max_chunks
// (a stream's chunks are dispatched together, which measured faster than
// chunk-major order, and are rotated so that every XCD gets an even share of
// them); work-groups past a stream's last chunk exit.  RAW logits.
template <int D, int DT>
__global__ __launch_bounds__(256) void decode_grid_kernel(CacheView c, DecodeArgs a) {
  __shared__ float s_acc[4][D];
  __shared__ float s_ml[4][2];
  const int u = blockIdx.x / a.max_chunks;
  const int k = rotated_chunk(blockIdx.x % a.max_chunks, u, a.max_chunks);
  int T, cnt;
  const int nch = stream_chunks(c, a, u, &T, &cnt);
  if (k >= nch) return;
  const int first = k * a.split, nblk = min(a.split, cnt - first);
  chunk_attend<D, DT, ETA_LOGIT_RAW, kChunkDense>(c, a, u, k, T, first, nblk,
                                                  first == 0 && nblk == cnt, 0.f, nullptr,
                                                  s_acc, s_ml);
}

// Combine: one work-group per stream with two or more chunks.
template <int D>
__global__ __launch_bounds__(kCombWaves * kWave) void combine_kernel(CacheView c, DecodeArgs a) {
  __shared__ float s_acc[kCombWaves][D];
  __shared__ float s_ml[kCombWaves][2];
  const int u = blockIdx.x;
  int T, cnt;
  const int nch = stream_chunks(c, a, u, &T, &cnt);
  if (nch == 0) {  // empty stream: zeros
    for (int i = threadIdx.x; i < D; i += blockDim.x) a.out[(size_t)u * D + i] = 0.f;
    return;
  }
  if (nch == 1) return;  // written by the decode kernel
  combine_slots<D>(a, u, (size_t)u * a.max_chunks, nch, s_acc, s_ml);
}

// ---------------------------------------------------------------------------
// Fused threshold + screen + decode, for steps too small to hide the
// separate threshold, screen, compaction and decode launches.  One
// work-group per chunk of a.split <= 32 consecutive blocks, flattened as
// blockIdx.x = k * units + u (the first chunks of every stream are dispatched
// first; chunks past a stream's end exit).  The work-group computes its
// stream's Eq. 1 threshold (tau_of_head: the threshold kernel's order, so the
// same bits), then wave w scores blocks 8 w .. 8 w + 7 of the chunk with the
// screen's Eq. 5 arithmetic (block_score, the same float32 operations in the
// same order, so the admission bits equal eta_screen's), the admitted
// indices go to LDS in ascending order, and the whole work-group attends over
// them (chunk_attend).  Chunk k's partial lands in slot k of the
// stream and the chunked combine merges a stream's ceil(nb / split) slots; a
// chunk that admits nothing leaves the empty partial (max -inf, sum 0), and
// the chunk holding the last block always admits it.
// Register buffers per wave of the fused kernel's attention: four for a
// bfloat16 cache (three tiles in flight while one is folded in; two waves per
// SIMD suffice for the small steps it serves), two for float32 (whose tiles
// take twice the registers).
#ifndef ETA_FUSED_NBUF
#define ETA_FUSED_NBUF 4
#endif
template <int DT>
constexpr int fused_bufs() { return DT == ETA_DT_BF16 ? ETA_FUSED_NBUF : 2; }
// Waves per chunk work-group: waves 0-3 screen the chunk's (up to 32)
// blocks, then all of them share its admitted tiles, so the densest chunks
// (which set the step's time) are spread over eight waves.  Measured at
// 32K x 16 heads, 32-block chunks (one work-group per compute unit): 0.035
// against 0.037 ms per step at 38% density, 0.022 against 0.024 at 10%.
#ifndef ETA_FUSED_WAVES
#define ETA_FUSED_WAVES 8
#endif
constexpr int kFusedWaves = ETA_FUSED_WAVES;  // waves per chunk work-group
template <int D, int DT, int MODE>
__global__ __launch_bounds__(kFusedWaves * kWave, 8 / kFusedWaves) void screen_decode_kernel(
    CacheView c, DecodeArgs a, ScreenDecodeArgs sa) {
  __shared__ int s_list[kMaxFusedChunk];
  __shared__ float s_acc[kFusedWaves][D];
  __shared__ float s_ml[kFusedWaves][2];
  __shared__ uint32_t s_bits[4];
  __shared__ float s_red[kTauThreads / kWave];
  static_assert(4 * kBlocksPerIter == kMaxFusedChunk, "four waves score a whole chunk");
  static_assert(kTauThreads == 256, "the threshold takes the whole work-group");
  const int units = c.B * c.H;
  const int u = blockIdx.x % units, k = blockIdx.x / units;
  const int T = c.seq_len[u / c.H];
  const int nb = T > 0 ? (T + c.bs - 1) >> c.log2bs : 0;
  const int first = k * a.split;
  // Uniform over the work-group.  The first chunk of a stream always runs far
  // enough to report the stream's thresholds, as the threshold kernel does.
  if (first >= nb && k > 0) return;
  const int nbc = T >> c.log2bs;
  const int nblk = first < nb ? min(a.split, nb - first) : 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Waves 0-3 request their blocks' statistics and their query share before
  // the threshold's sum, so those loads overlap it; the score is block_score's
  // arithmetic on the loaded values.
  const bool screener = wave < 4 && kBlocksPerIter * wave < nblk;  // wave-uniform
  const int gi = lane / kLanesPerBlock, li = lane % kLanesPerBlock;
  const int i = kBlocksPerIter * wave + gi;  // block first + i of the stream
  const int j = first + i;
  const bool scored = screener && i < nblk && j < nbc;  // complete blocks of this chunk
  QShare<D> qs;
  uint4 m4[QShare<D>::kLoads], v4[QShare<D>::kLoads];
  float M = 0.f;
  if (screener) {
    load_qshare<D>(a.q + (size_t)u * D, li, qs);
    const size_t row = ((size_t)u * c.cap_blocks + (scored ? j : 0)) * D;
#pragma unroll
    for (int t = 0; t < QShare<D>::kLoads; ++t) {
      m4[t] = scored ? ld16_nt(c.mu + row + 64 * t + 8 * li) : make_uint4(0, 0, 0, 0);
      v4[t] = scored ? ld16_nt(c.var + row + 64 * t + 8 * li) : make_uint4(0, 0, 0, 0);
    }
    M = scored ? c.maxnorm[(size_t)u * c.cap_blocks + j] : 0.f;
  }
  const float tg = tau_of_head(a.q + (size_t)(u / c.H) * c.H * D, sa.W, sa.bias, c.H, c.H * D,
                               u % c.H, s_red);
  const float ts = tg - sa.a;
  if (k == 0 && threadIdx.x == 0) {
    if (sa.tau_gate) sa.tau_gate[u] = tg;
    if (sa.tau_screen) sa.tau_screen[u] = ts;
  }
  if (first >= nb) return;  // an empty stream (T == 0): the combine writes zeros
  if (screener) {
    float dot = 0.f, mom = 0.f;
    score_partials<D>(qs, m4, v4, dot, mom);
    dot = group_sum<kLanesPerBlock>(dot);
    mom = group_sum<kLanesPerBlock>(mom);
    const float geometric = qs.qn * M;
    const float sc = __builtin_isinf(sa.z) ? a.scale * geometric
                                           : a.scale * fminf(fmaf(sa.z, sqrtf(mom), dot), geometric);
    const bool on = i < nblk && (j == nb - 1 || (scored && sc >= ts));
    const uint64_t bal = __ballot(on);
    uint32_t bits = 0;
#pragma unroll
    for (int g = 0; g < kBlocksPerIter; ++g)
      bits |= (uint32_t)((bal >> (g * kLanesPerBlock)) & 1ull) << g;
    if (lane == 0) s_bits[wave] = bits;
  } else if (wave < 4 && lane == 0) {
    s_bits[wave] = 0u;
  }
  __syncthreads();
  const uint32_t word = s_bits[0] | (s_bits[1] << kBlocksPerIter) |
                        (s_bits[2] << (2 * kBlocksPerIter)) | (s_bits[3] << (3 * kBlocksPerIter));
  const int t = threadIdx.x;
  if (t < kMaxFusedChunk && ((word >> t) & 1u)) s_list[__popc(word & ((1u << t) - 1u))] = first + t;
  const int nadm = __popc(word);
  if (t == 0) {
    if (sa.chunk_bits) sa.chunk_bits[(size_t)u * a.max_chunks + k] = word;
    if (sa.ctr && nadm > 0) {
      // Admitted tokens; the stream's last block (always admitted) may be partial.
      const bool last = first + nblk == nb;
      const unsigned long long tokens =
          (unsigned long long)nadm * c.bs - (last ? (unsigned long long)nb * c.bs - T : 0ull);
      atomicAdd(reinterpret_cast<unsigned long long*>(sa.ctr), tokens);
    }
  }
  const int nch = (nb + a.split - 1) / a.split;
  // chunk_attend synchronises the work-group before reading s_list.
  chunk_attend<D, DT, MODE, kChunkStaged, fused_bufs<DT>(), kFusedWaves>(
      c, a, u, k, T, first, nadm, nch == 1, tg, s_list, s_acc, s_ml);
}

// ---------------------------------------------------------------------------
// Balanced sparse decode.  The admitted lists of all streams, concatenated in
// stream order, hold N blocks (exclusive prefix sums start[u]).  Each of
// min(waves, ceil(N / blocks_per_split)) waves takes an equal contiguous range
// of that concatenation (small jobs use fewer waves), walks it with its
// own two-deep load pipeline (no wave waits for another and no work-group
// restarts per chunk), and writes one partial per stream segment it covers
// into slot w + u: along the concatenation the wave index and the stream
// index both only grow and every new segment advances one of them, so the
// slots are distinct.  The combine merges, per stream, the slots of the waves
// that cover it.

// Admitted blocks of stream u, clamped to the blocks the stream holds.
__device__ __forceinline__ int stream_blocks(const CacheView& c, const DecodeArgs& a, int u) {
  const int T = c.seq_len[u / c.H];
  const int nb = T > 0 ? (T + c.bs - 1) >> c.log2bs : 0;
  return max(0, min(a.active_cnt[u], nb));
}

// GS: the stream offsets and each wave's first stream come from global memory
// (flow_scan_kernel, for more streams than LDS holds); otherwise every
// work-group scans the counts into LDS itself.
template <int D, int DT, int MODE, bool GS>
__global__ __launch_bounds__(kFlowThreads, kFlowWGsPerCU) void decode_flow_kernel(CacheView c,
                                                                                  DecodeArgs a) {
  constexpr int EPL = Elt<DT>::kPer16B;
  constexpr int LPR = D / EPL;
  constexpr int RPI = kWave / LPR;
  constexpr int NI = (kRows / RPI) > 0 ? (kRows / RPI) : 1;
  constexpr int RB = D * Elt<DT>::kBytes;
  extern __shared__ int s_start[];  // [units + 1]
  constexpr int NW = kFlowThreads / kWave;  // waves per work-group
  __shared__ int s_wsum[NW];
  const int units = c.B * c.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane / LPR, li = lane % LPR;
  const int waves = gridDim.x * NW;

  // Exclusive prefix sums of the admitted counts, every work-group for itself:
  // thread t sums its run of ceil(units / 256) streams, the runs are scanned
  // across the work-group, then written back as offsets.
  if constexpr (!GS) {
    const int per = (units + kFlowThreads - 1) / kFlowThreads;
    const int u0 = min(units, tid * per), u1 = min(units, u0 + per);
    int sum = 0;
    for (int u = u0; u < u1; ++u) {
      const int n = stream_blocks(c, a, u);
      s_start[u] = n;
      sum += n;
    }
    int incl = sum;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int off = incl - sum;
    for (int w = 0; w < wave; ++w) off += s_wsum[w];
    for (int u = u0; u < u1; ++u) {
      const int n = s_start[u];
      s_start[u] = off;
      off += n;
    }
    if (tid == kFlowThreads - 1) s_start[units] = off;
    __syncthreads();
  }
  auto start_of = [&](int x) { return GS ? a.flow_start[x] : s_start[x]; };
  const FlowPlan plan(start_of(units), waves, a.split);
  if (!GS && blockIdx.x == 0) {  // for the combine
    for (int u = tid; u <= units; u += kFlowThreads) a.flow_start[u] = s_start[u];
    if (tid == 0) a.flow_info[0] = plan.N;
  }
  const int w = blockIdx.x * NW + wave;
  if (w >= plan.wn) return;  // waves are independent from here on

  // Attention of the wave over positions [p, pend) of the concatenation,
  // one partial per stream segment, into slot slot_base + u.
  auto walk = [&](int p, const int pend, const size_t slot_base) {
    int u = 0;  // the last stream with start[u] <= p (so start[u + 1] > p)
    if constexpr (GS) {
      u = a.flow_wave_u[w];
    } else {
      int hi = units - 1;
      while (u < hi) {
        const int mid = (u + hi + 1) >> 1;
        if (s_start[mid] <= p) u = mid; else hi = mid - 1;
      }
    }
    while (p < pend) {
      const int base = start_of(u);
      const int i0 = p - base, i1 = min(pend, start_of(u + 1)) - base;  // local blocks
      const int T = c.seq_len[u / c.H];
      const int nb = (T + c.bs - 1) >> c.log2bs;
      const int32_t* list = a.active_idx + (size_t)u * c.cap_blocks + i0;
      const int nblk = i1 - i0;
      float qs[EPL];
      {
        const float* qu = a.q + (size_t)u * D + li * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) qs[e] = qu[e] * a.scale;
      }
      const float tau = (MODE == ETA_LOGIT_GATED) ? a.tau[u] : 0.f;
      const char* kb = static_cast<const char*>(c.k) + (size_t)u * c.cap * RB + li * 16;
      const char* vb = static_cast<const char*>(c.v) + (size_t)u * c.cap * RB + li * 16;

      // Block indices, 64 per register: lane x holds entry bb + x of lst0 and
      // bb + 64 + x of lst1; the window moves on by 64 once a tile starts past
      // its first half, and the new second half is loaded then, long before use.
      int bb = 0;
      int lst0 = lane < nblk ? list[lane] : -1;
      int lst1 = 64 + lane < nblk ? list[64 + lane] : -1;
      const int rows = nblk << c.log2bs;
      const int ntiles = (rows + kRows - 1) / kRows;

      auto fetch = [&](int t, uint4* kr, uint4* vr, int* sp) {
        const int first_blk = (t * kRows) >> c.log2bs;
        if (first_blk >= bb + 64) {  // wave-uniform
          lst0 = lst1;
          bb += 64;
          lst1 = bb + 64 + lane < nblk ? list[bb + 64 + lane] : -1;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int rr = t * kRows + i * RPI + g;  // row within the segment
          // Every lane takes part in the shuffles (a lane whose own row is past
          // the segment may still hold the entry another lane needs).
          const int o = (rr >> c.log2bs) - bb;  // 0 .. 127
          const int j0 = __shfl(lst0, o & 63, kWave), j1 = __shfl(lst1, o & 63, kWave);
          const int j = o < 64 ? j0 : j1;
          // The list is trusted only as far as it stays inside the stream.
          int s = rr < rows && (unsigned)j < (unsigned)nb ? (j << c.log2bs) + (rr & (c.bs - 1)) : -1;
          if (s >= T) s = -1;
          sp[i] = s;
          if (s >= 0) {
            kr[i] = ld16_nt(kb + (size_t)s * RB);
            vr[i] = ld16_nt(vb + (size_t)s * RB);
          } else {
            kr[i] = make_uint4(0, 0, 0, 0);
            vr[i] = make_uint4(0, 0, 0, 0);
          }
        }
      };

      RowState<EPL> st;
      st.reset();
      uint4 ka[NI], va[NI], kq[NI], vq[NI];
      int sa[NI], sq[NI];
      fetch(0, ka, va, sa);
      for (int t = 0; t < ntiles; t += 2) {
        const bool has_b = t + 1 < ntiles;
        if (has_b) fetch(t + 1, kq, vq, sq);
        fold_tile<D, DT, MODE, NI>(st, ka, va, sa, qs, tau, a.beta, T);
        if (t + 2 < ntiles) fetch(t + 2, ka, va, sa);
        if (has_b) fold_tile<D, DT, MODE, NI>(st, kq, vq, sq, qs, tau, a.beta, T);
      }
      merge_groups<EPL, LPR>(st);
      const size_t slot = slot_base + u;
      if (g == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) a.part_acc[slot * D + li * EPL + e] = st.acc[e];
        if (li == 0) {
          a.part_m[slot] = st.m;
          a.part_l[slot] = st.l;
        }
      }
      p = base + i1;
      if (p < pend)  // next non-empty stream
        do ++u; while (start_of(u + 1) <= p);
    }
  };

  walk(plan.lo(w), plan.lo(w + 1), (size_t)w);
}

// Offsets of the balanced decode for more streams than LDS holds, by one
// work-group: flow_start[u] = admitted blocks of the streams before u (rounds
// of 1024 streams with a running carry), flow_info[0] = N, and flow_wave_u[w]
// = the stream holding position lo(w) of wave w's range (lo(w) =
// floor(w N / wn) >= start[u] exactly when w >= ceil(start[u] wn / N)).
__global__ __launch_bounds__(1024) void flow_scan_kernel(CacheView c, DecodeArgs a, int waves) {
  __shared__ int s_w[1024 / kWave];
  __shared__ int s_carry;
  const int units = c.B * c.H, t = threadIdx.x;
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int r = 0; r < units; r += 1024) {
    const int u = r + t;
    const int cnt = u < units ? stream_blocks(c, a, u) : 0;
    int total;
    const int excl = wg_exclusive_scan<1024 / kWave>(cnt, s_w, &total);
    const int carry = s_carry;
    if (u < units) a.flow_start[u] = carry + excl;
    __syncthreads();  // every thread has read s_carry
    if (t == 0) s_carry = carry + total;
    __syncthreads();
  }
  const int N = s_carry;
  if (t == 0) {
    a.flow_start[units] = N;
    a.flow_info[0] = N;
  }
  __syncthreads();  // flow_start is read back below by other threads
  const FlowPlan plan(N, waves, a.split);
  if (plan.wn == 0) return;
  for (int u = t; u < units; u += 1024) {
    const long long s0 = a.flow_start[u], s1 = a.flow_start[u + 1];
    const int w0 = (int)((s0 * plan.wn + N - 1) / N);
    const int w1 = min(plan.wn, (int)((s1 * plan.wn + N - 1) / N));
    for (int w = w0; w < w1; ++w) a.flow_wave_u[w] = u;
  }
}

// Combine of the balanced decode: one work-group per stream, merging the
// slots of the ranges that cover the stream's positions [p0, p1).
template <int D>
__global__ __launch_bounds__(kCombWaves * kWave) void combine_flow_kernel(CacheView c,
                                                                          DecodeArgs a) {
  __shared__ float s_acc[kCombWaves][D];
  __shared__ float s_ml[kCombWaves][2];
  const int u = blockIdx.x;
  const int p0 = a.flow_start[u], p1 = a.flow_start[u + 1];
  if (p1 <= p0) {  // empty stream: zeros
    for (int i = threadIdx.x; i < D; i += blockDim.x) a.out[(size_t)u * D + i] = 0.f;
    return;
  }
  const FlowPlan plan(a.flow_info[0], a.flow_grid * (kFlowThreads / kWave), a.split);
  const int wf = plan.range_of(p0), wl = plan.range_of(p1 - 1);
  combine_slots<D>(a, u, (size_t)wf + u, wl - wf + 1, s_acc, s_ml);
}

// ---------------------------------------------------------------------------
template <int D, int DT, int MODE, bool DENSE>
static hipError_t decode_t(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  const int units = c.B * c.H;
  hipError_t e;
  if constexpr (!DENSE) {
    // balanced: offsets scanned into LDS, or for more streams written to
    // global memory by the scan kernel first
    if (a.flow_global) {
      hipLaunchKernelGGL(flow_scan_kernel, dim3(1), dim3(1024), 0, s, c, a,
                         a.flow_grid * (kFlowThreads / kWave));
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL((decode_flow_kernel<D, DT, MODE, true>), dim3(a.flow_grid),
                         dim3(kFlowThreads), 0, s, c, a);
    } else {
      hipLaunchKernelGGL((decode_flow_kernel<D, DT, MODE, false>), dim3(a.flow_grid),
                         dim3(kFlowThreads), (size_t)(units + 1) * 4, s, c, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((combine_flow_kernel<D>), dim3(units), dim3(kCombWaves * kWave), 0, s, c,
                       a);
    return hipGetLastError();
  } else {
    const long long grid = (long long)a.max_chunks * units;
    hipLaunchKernelGGL((decode_grid_kernel<D, DT>), dim3((unsigned)grid), dim3(256), 0, s, c, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((combine_kernel<D>), dim3(units), dim3(kCombWaves * kWave), 0, s, c, a);
    return hipGetLastError();
  }
}

template <int D, int DT>
static hipError_t decode_dt(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  if (a.dense) return decode_t<D, DT, ETA_LOGIT_RAW, true>(c, a, s);
  if (a.mode == ETA_LOGIT_RAW) return decode_t<D, DT, ETA_LOGIT_RAW, false>(c, a, s);
  return decode_t<D, DT, ETA_LOGIT_GATED, false>(c, a, s);
}

// Fused threshold + screen + decode, then the chunked combine (a.dense is
// set, so the combine counts ceil(nb / split) chunks per stream).  Merging
// inside the fused kernel (the last chunk of a stream to finish merging the
// others' partials) needs device-scope release and acquire fences around
// every partial, which cost more here than the combine's launch: 0.072 vs
// 0.038 ms per step at 32K x 16 heads, 38%, on MI355X.
template <int D, int DT, int MODE>
static hipError_t screen_decode_t(const CacheView& c, const DecodeArgs& a,
                                  const ScreenDecodeArgs& sa, hipStream_t s) {
  const int units = c.B * c.H;
  const long long grid = (long long)a.max_chunks * units;
  hipLaunchKernelGGL((screen_decode_kernel<D, DT, MODE>), dim3((unsigned)grid),
                     dim3(kFusedWaves * kWave), 0, s, c, a, sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(units), dim3(kCombWaves * kWave), 0, s, c, a);
  return hipGetLastError();
}

template <int D, int DT>
static hipError_t screen_decode_dt(const CacheView& c, const DecodeArgs& a,
                                   const ScreenDecodeArgs& sa, hipStream_t s) {
  if (a.mode == ETA_LOGIT_RAW) return screen_decode_t<D, DT, ETA_LOGIT_RAW>(c, a, sa, s);
  return screen_decode_t<D, DT, ETA_LOGIT_GATED>(c, a, sa, s);
}

hipError_t launch_screen_decode(const CacheView& c, const DecodeArgs& a,
                                const ScreenDecodeArgs& sa, hipStream_t s) {
  if (c.D == 128)
    return c.dtype == ETA_DT_BF16 ? screen_decode_dt<128, ETA_DT_BF16>(c, a, sa, s)
                                  : screen_decode_dt<128, ETA_DT_F32>(c, a, sa, s);
  return c.dtype == ETA_DT_BF16 ? screen_decode_dt<64, ETA_DT_BF16>(c, a, sa, s)
                                : screen_decode_dt<64, ETA_DT_F32>(c, a, sa, s);
}

hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  if (c.D == 128) return c.dtype == ETA_DT_BF16 ? decode_dt<128, ETA_DT_BF16>(c, a, s)
                                                : decode_dt<128, ETA_DT_F32>(c, a, s);
  return c.dtype == ETA_DT_BF16 ? decode_dt<64, ETA_DT_BF16>(c, a, s)
                                : decode_dt<64, ETA_DT_F32>(c, a, s);
}

}  // namespace eta
