// kernels_gqa.hip -- grouped-query screen, compaction and decode.
//
// Paper: "Elastic Threshold Attention ..." (v2 page, Table 5 benchmark shape:
// 32 query heads on 4 KV heads; summary page, Implications: a KV block is
// loaded when any head of its group admits it).  Query head h = kv*G + g
// reads KV head kv.  Every query head is screened with its own query and
// threshold against the KV head's block statistics (Eq. 5) and attends only
// over the blocks it admits itself (Eq. 3 logits); the union of the group's
// admitted blocks is what is read from HBM, once for the whole group.
//
// With G query heads per loaded key row, the scores and the value sums are
// G x b x d contractions, so the decode runs them on the matrix cores
// (v_mfma_f32_16x16x32_bf16; the group is padded to 16).  K and V are bf16 as
// stored; the scaled query and the softmax weights are split into bf16 hi and
// lo parts (x = hi + lo to about 2^-16 relative), so each product is two
// MFMAs and the result keeps float32-level accuracy.
#include "eta_internal.h"

namespace eta {


// ---------------------------------------------------------------------------
// Screen: one work-group per 64-block admission word of KV stream u; wave w
// scores blocks 16 w .. 16 w + 15 of the word in two steps of 8 blocks, 8
// lanes per block.  A block's statistics are loaded once and scored against
// every query head of the group: each lane forms the partial dot products
// q_g . mu and (q_g * q_g) . var over its 8 dims for all NH head slots (NH = 8
// for groups up to 8, 16 up to 16; queries and their squares staged in LDS,
// zero past the group), and an exchange butterfly over the 8 lanes of the
// block (partners l ^ 1, l ^ 2, l ^ 4) leaves lane l with the complete sums
// of NH / 8 heads: at each step a lane keeps half of its values and adds its
// partner's copy of them.  The additions pair the same partial sums as
// group_sum<8> (whose last partner, the half-row mirror l ^ 7, holds the same
// sum as l ^ 4 with its operands commuted), so each head's sums are
// bit-identical to the one-query-per-KV-head screen's.  Each head is then scored once (Eq. 5) instead of
// on all 8 lanes.  Writes the per-block head mask (bit g: query head u*G + g
// admits the block) for every block of the stream, the union admission word,
// and the word's admitted head tokens (for the D_head counter).

// Keep half of the N values of x (the upper half when `upper`), adding the
// copy held by the partner lane: lane ^ 1 or lane ^ 2 by a DPP quad
// permutation (CTRL), lane ^ 4 by ds_swizzle (CTRL = 0: and-mask 31, xor 4).
constexpr int kSwizzleXor4 = 0x101F;
template <int N, int CTRL>
__device__ __forceinline__ void fold_half_dpp(float* x, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float send = upper ? x[i] : x[N / 2 + i];
    const float keep = upper ? x[N / 2 + i] : x[i];
    const float other =
        CTRL ? dpp<CTRL>(send)
             : __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), kSwizzleXor4));
    x[i] = keep + other;
  }
}

// Head slot of the first value lane li (0..7) holds after the butterfly:
// step k keeps the half selected by bit k of li, so bits 0, 1, 2 of li pick
// the head's top three bits in that order.
__device__ __forceinline__ int rev3(int li) {
  return ((li & 1) << 2) | (li & 2) | ((li >> 2) & 1);
}

template <int D, int NH>
__global__ __launch_bounds__(256) void screen_gqa_kernel(CacheView c, int G, const float* q,
                                                         const float* tau_screen, float z,
                                                         float scale, uint32_t* head_mask,
                                                         uint64_t* words, uint32_t* word_tokens,
                                                         int words_per_unit) {
  constexpr int LPB = 8;            // lanes per block
  constexpr int NL = D / 64;        // 128-bit loads (8 bf16) per lane per statistics row
  constexpr int PER = NH / 8;       // heads per lane after the butterfly
  __shared__ __align__(16) float s_q[NH][D];
  __shared__ __align__(16) float s_q2[NH][D];
  __shared__ float s_qn[NH];
  __shared__ float s_ts[NH];
  __shared__ uint32_t s_bits[4];
  __shared__ uint32_t s_tok[4];
  const int units = c.B * c.H;
  const int u = blockIdx.x % units, wd = blockIdx.x / units;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = c.seq_len[u / c.H];
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int nbc = T >> c.log2bs;
  if ((wd << 6) >= nb) return;  // uniform over the work-group
  const int gi = lane / LPB, li = lane % LPB;
  // The word's statistics are requested first, so their latency overlaps the
  // staging of the queries below.
  uint4 m4[2][NL], v4[2][NL];
  float Ms[2];
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (wd << 6) + wave * 16 + it * 8 + gi;
    const bool scored = j < nbc;
    const size_t row = ((size_t)u * c.cap_blocks + j) * D;
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      m4[it][t] = scored ? ld16_nt(c.mu + row + 64 * t + 8 * li) : zero4;
      v4[it][t] = scored ? ld16_nt(c.var + row + 64 * t + 8 * li) : zero4;
    }
    Ms[it] = scored ? c.maxnorm[(size_t)u * c.cap_blocks + j] : 0.f;
  }
  for (int i = threadIdx.x; i < NH * D; i += blockDim.x) {
    const int g = i / D;
    const float x = g < G ? q[(size_t)u * G * D + i] : 0.f;
    s_q[g][i % D] = x;
    s_q2[g][i % D] = x * x;
  }
  if (threadIdx.x < NH) s_ts[threadIdx.x] = threadIdx.x < G ? tau_screen[(size_t)u * G + threadIdx.x] : 0.f;
  __syncthreads();
  // ||q|| per head, 8 lanes per head summing in the same order as the
  // one-head-per-KV-head screen (so G = 1 reproduces it bit for bit).
#pragma unroll
  for (int h8 = 0; h8 < NH; h8 += 32) {
    const int hg = h8 + wave * 8 + gi;
    float qq = 0.f;
    if (hg < NH) {
#pragma unroll
      for (int t = 0; t < NL; ++t) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = s_q[hg][64 * t + 8 * li + e];
          qq = fmaf(x, x, qq);
        }
      }
    }
    qq = group_sum<LPB>(qq);
    if (hg < NH && li == 0) s_qn[hg] = sqrtf(qq);
  }
  __syncthreads();
  const bool z_inf = __builtin_isinf(z);
  const int tail = T - ((nb - 1) << c.log2bs);
  uint32_t bits = 0, tokens = 0;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (wd << 6) + wave * 16 + it * 8 + gi;
    const bool scored = j < nbc;
    // v[2 g] = q_g . mu, v[2 g + 1] = (q_g * q_g) . var over this lane's dims
    float mf[NL][8], vf[NL][8];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      widen<ETA_DT_BF16>(m4[it][t], mf[t]);
      widen<ETA_DT_BF16>(v4[it][t], vf[t]);
    }
    float v[2 * NH];
#pragma unroll
    for (int g = 0; g < NH; ++g) {
      float dot = 0.f, mom = 0.f;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const float4 qa = *reinterpret_cast<const float4*>(&s_q[g][64 * t + 8 * li]);
        const float4 qb = *reinterpret_cast<const float4*>(&s_q[g][64 * t + 8 * li + 4]);
        const float4 ra = *reinterpret_cast<const float4*>(&s_q2[g][64 * t + 8 * li]);
        const float4 rb = *reinterpret_cast<const float4*>(&s_q2[g][64 * t + 8 * li + 4]);
        const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
        const float q2[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qv[e], mf[t][e], dot);
#pragma unroll
        for (int e = 0; e < 8; ++e) mom = fmaf(q2[e], vf[t][e], mom);
      }
      v[2 * g] = dot;
      v[2 * g + 1] = mom;
    }
    fold_half_dpp<2 * NH, kQuadXor1>(v, li & 1);
    fold_half_dpp<NH, kQuadXor2>(v, li & 2);
    fold_half_dpp<NH / 2, 0>(v, li & 4);
    // This lane now holds heads PER * rev3(li) + e, e < PER: (v[2e], v[2e+1]).
    uint32_t mine = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int g = PER * rev3(li) + e;
      const float geometric = s_qn[g] * Ms[it];
      const float sc = z_inf ? scale * geometric
                             : scale * fminf(fmaf(z, sqrtf(v[2 * e + 1]), v[2 * e]), geometric);
      if (g < G && scored && sc >= s_ts[g]) mine |= 1u << g;
    }
    // OR of the block's 8 lanes (disjoint head bits).
    mine |= __shfl_xor(mine, 1, kWave);
    mine |= __shfl_xor(mine, 2, kWave);
    mine |= __shfl_xor(mine, 4, kWave);
    const uint32_t all = (G >= 32) ? 0xffffffffu : ((1u << G) - 1u);
    const uint32_t mask = (j == nb - 1) ? all : mine;  // the last block: every head
    if (li == 0 && j < nb) head_mask[(size_t)u * c.cap_blocks + j] = mask;
    if (li == 0 && j < nb)
      tokens += (uint32_t)__popc(mask) * (uint32_t)(j == nb - 1 ? tail : c.bs);
    const uint64_t bal = __ballot(mask != 0u);
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8)
      bits |= (uint32_t)((bal >> (g8 * LPB)) & 1ull) << (it * 8 + g8);
  }
  // Head tokens of the wave: lanes 0, 8, ..., 56 hold their blocks' counts.
  tokens += __shfl_xor(tokens, 8, kWave);
  tokens += __shfl_xor(tokens, 16, kWave);
  tokens += __shfl_xor(tokens, 32, kWave);
  if (lane == 0) {
    s_bits[wave] = bits;
    s_tok[wave] = tokens;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t word = (uint64_t)s_bits[0] | ((uint64_t)s_bits[1] << 16) |
                          ((uint64_t)s_bits[2] << 32) | ((uint64_t)s_bits[3] << 48);
    words[(size_t)u * words_per_unit + wd] = word;
    word_tokens[(size_t)u * words_per_unit + wd] = s_tok[0] + s_tok[1] + s_tok[2] + s_tok[3];
  }
}

// Compaction of the union words into the ascending union list, plus the
// counters: ctr[0] += admitted tokens summed over the group's query heads
// (the screen's per-word counts), ctr[1] += union tokens.  Thread t takes a
// run of bpt consecutive blocks (bpt a power of two <= 64, so a run lies in
// one word), rounds of 256 runs in ascending order; a work-group scan places
// each run's entries.
__global__ __launch_bounds__(256) void compact_gqa_kernel(CacheView c, const uint64_t* words,
                                                          const uint32_t* word_tokens,
                                                          int words_per_unit,
                                                          int32_t* union_idx, int32_t* union_cnt,
                                                          uint64_t* ctr) {
  __shared__ int s_w[4];
  __shared__ unsigned long long s_tok[4];
  const int u = blockIdx.x, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int T = c.seq_len[u / c.H];
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int nw = (nb + 63) >> 6;
  const uint64_t* wu = words + (size_t)u * words_per_unit;
  int32_t* out = union_idx + (size_t)u * c.cap_blocks;
  const int tail = T - ((nb - 1) << c.log2bs);
  // head tokens: the screen's per-word counts, summed in a fixed order
  unsigned long long head_tokens = 0;
  for (int i = t; i < nw; i += 256) head_tokens += word_tokens[(size_t)u * words_per_unit + i];
  int bpt = 1;
  while (bpt < 64 && bpt * 256 < nb) bpt <<= 1;
  int base_pos = 0;
  for (int r0 = 0; r0 < nb; r0 += 256 * bpt) {
    const int b0 = r0 + t * bpt;  // first block of this thread's run
    uint64_t x = 0;
    if (b0 < nb) {
      x = wu[b0 >> 6] >> (b0 & 63);
      if (bpt < 64) x &= (1ull << bpt) - 1ull;
      const int rem = nb - b0;
      if (rem < 64) x &= (1ull << rem) - 1ull;
    }
    int round_total;
    int pos = base_pos + wg_exclusive_scan<4>(__popcll(x), s_w, &round_total);
    base_pos += round_total;
    while (x) {
      out[pos++] = b0 + __ffsll((unsigned long long)x) - 1;
      x &= x - 1ull;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) head_tokens += __shfl_xor(head_tokens, off, kWave);
  if (lane == 0) s_tok[wave] = head_tokens;
  __syncthreads();
  if (t == 0) {
    const int total = base_pos;
    union_cnt[u] = total;
    if (ctr && total > 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(ctr),
                (s_tok[0] + s_tok[1]) + (s_tok[2] + s_tok[3]));
      const unsigned long long ut =
          (unsigned long long)(total - 1) * c.bs + (unsigned long long)tail;
      atomicAdd(reinterpret_cast<unsigned long long*>(ctr + 1), ut);
    }
  }
}

using GqaArgs = GqaDecode;

// Length T_b of KV stream u's sequence and its block count to decode: every
// block (dense) or the union count, clamped to the blocks the stream holds.
__device__ __forceinline__ void gqa_stream(const CacheView& c, const GqaArgs& a, bool dense, int u,
                                           int* T_out, int* cnt_out) {
  const int T = c.seq_len[u / c.H];
  const int nb = T > 0 ? (T + c.bs - 1) >> c.log2bs : 0;
  *T_out = T;
  *cnt_out = dense ? nb : max(0, min(a.union_cnt[u], nb));
}

// ---------------------------------------------------------------------------
// Grouped decode.  As the per-head balanced decode does with the admitted
// lists, the union lists of all KV streams, concatenated in stream order, are
// cut into equal contiguous ranges, one per wave; a work-group is one wave and
// holds no state shared with others.  The wave walks its range in 32-key
// tiles: coalesced 128-bit loads of whole K and V rows into registers (the
// next tiles' loads in flight while the current one is computed), staged as
// rows in the wave's LDS area (K chunk-swizzled for the score operand, V for
// the transposing read of the value operand).  Keys that are not to be read
// (past the range, the stream, or an out-of-range list entry) load the
// stream's row 0 instead -- finite data -- and are masked out of the softmax,
// so their weights are exactly zero.  Per tile, on v_mfma_f32_16x16x32_bf16
// (the group padded to 16 heads):
//   scores  for each 16-key half st: S[16 keys x 16 heads] = K (A operand:
//           lane l holds key tile_key(st, l % 16), dims 32 kk + 8 (l / 16)
//           .. + 7) times Q^T (B: head l % 16, the same dims; q split hi +
//           lo), so lane l receives head l % 16 and four keys of the half;
//   softmax per head with a lazily moved reference max; weights split hi + lo;
//   values  O[16 heads x 16 dims] += P (A: head l % 16, the lane's 8 score
//           keys as contraction slots) times V (B: dim l % 16, the same
//           slots, by the transposing LDS read).
// The partial of (stream segment, head g) goes to slot (w + u) * G + g.
// Measured on 32 x 128K, 38% head density: about 6% faster than one
// work-group per chunk of union blocks (the kernel it replaced), and on 8192
// KV streams x 4K (offsets in global memory) 0.91 against 1.27 ms.
// Two waves per SIMD at either head dim.  At d = 64 a second tile in flight
// and the uniform tile checks of the WHOLE form together took the 38% call
// (32 x 128K) from 0.40 to 0.38 ms (6.2 to 6.5 TB/s; either alone gave at most
// 3%).  At d = 128 (about 300 registers unconstrained, one wave per SIMD) the bound
// costs a few spilled registers and gains 12% (32 x 128K, 38% head density:
// 0.80 ms against 0.91 ms at one wave per SIMD).
template <int D>
struct GqaFlowShape {
  static constexpr int NK = D / 32;             // 32-dim slabs (score product)
  static constexpr int NV = D / 16;             // 16-dim slabs (value product)
  static constexpr int RB = D * 2;              // bytes per bf16 row
  static constexpr int LPR = D / 8;             // lanes per row of a load
  static constexpr int RPI = 64 / LPR;          // rows per load instruction
  static constexpr int NI = kTileKeys / RPI;    // load instructions per tile and tensor
  static constexpr int TB = kTileKeys * RB;     // one tensor's tile, bytes
  static constexpr int StageBytes = 2 * TB;     // K rows | V rows
  // Tiles in flight per wave beyond the one computed: two at d = 64 (32 more
  // registers, about 222 in all, still two waves per SIMD), one at d = 128.
  static constexpr int Ahead = D == 64 ? 2 : 1;
};

// WHOLE: every 32-key tile lies inside one block (b >= 32), so a tile's
// block index, head mask and position checks are wave-uniform: one lookup per
// tile, scalar base addresses, and per-key tests only in a stream's last tile.
// DENSE: every block of every stream, for every head (the dense baseline,
// RAW logits): the list is the identity and every head mask is full.
// GS: the stream offsets and each wave's first stream come from global memory
// (flow_scan_gqa_kernel, for more streams than LDS holds); otherwise every
// work-group scans the counts into LDS itself.
template <int D, int MODE, bool WHOLE, bool GS, bool DENSE>
__global__ __launch_bounds__(64, 2) void decode_gqa_flow_kernel(CacheView c, GqaArgs a) {
  using Sh = GqaFlowShape<D>;
  constexpr int NK = Sh::NK, NV = Sh::NV, RB = Sh::RB, LPR = Sh::LPR, RPI = Sh::RPI;
  constexpr int NI = Sh::NI, TB = Sh::TB;
  __shared__ __align__(16) char s_stage[Sh::StageBytes];
  extern __shared__ int s_start[];  // [units + 1] (LDS form)
  const int units = c.B * c.H, lane = threadIdx.x, G = a.G;
  // Exclusive prefix sums of the union counts: lane x sums a run of
  // ceil(units / 64) streams, the runs are scanned across the wave.
  if constexpr (!GS) {
    const int per = (units + 63) / 64;
    const int u0 = min(units, lane * per), u1 = min(units, u0 + per);
    int sum = 0;
    for (int u = u0; u < u1; ++u) {
      int T, cnt;
      gqa_stream(c, a, DENSE, u, &T, &cnt);
      s_start[u] = cnt;
      sum += cnt;
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    int off = incl - sum;
    for (int u = u0; u < u1; ++u) {
      const int n = s_start[u];
      s_start[u] = off;
      off += n;
    }
    if (lane == kWave - 1) s_start[units] = off;
    __syncthreads();
  }
  auto start_of = [&](int x) { return GS ? a.flow_start[x] : s_start[x]; };
  const FlowPlan plan(start_of(units), gridDim.x, a.split);
  if (!GS && blockIdx.x == 0) {  // for the combine
    for (int u = lane; u <= units; u += kWave) a.flow_start[u] = s_start[u];
    if (lane == 0) a.flow_info[0] = plan.N;
  }
  const int w = blockIdx.x;
  if (w >= plan.wn) return;
  const int n = lane & 15, grp = lane >> 4;  // operand layout: row/column n, k group grp
  const int ri = lane / LPR, cc = lane % LPR;  // load layout: row ri, 16-byte chunk cc
  const float gk1 = -a.beta * kLog2e;
  // Value-operand rows of the transposing read (as in the prefill kernel).
  const int trow0 = tile_key(0, 4 * grp + ((lane & 15) >> 2));
  const int trow1 = tile_key(1, 4 * grp + ((lane & 15) >> 2));
  const int tr4 = lane & 3;

  // Range bounds and streams are wave-uniform (read into scalar registers).
  int p = __builtin_amdgcn_readfirstlane(plan.lo(w));
  const int pend = __builtin_amdgcn_readfirstlane(plan.lo(w + 1));
  int u = 0;  // the last stream with start[u] <= p (so start[u + 1] > p)
  if constexpr (GS) {
    u = __builtin_amdgcn_readfirstlane(a.flow_wave_u[w]);
  } else {
    int hi = units - 1;
    while (u < hi) {
      const int mid = (u + hi + 1) >> 1;
      if (s_start[mid] <= p) u = mid; else hi = mid - 1;
    }
    u = __builtin_amdgcn_readfirstlane(u);
  }
  while (p < pend) {
    const int base = __builtin_amdgcn_readfirstlane(start_of(u));
    const int i1 = __builtin_amdgcn_readfirstlane(min(pend, start_of(u + 1)) - base);
    const int i0 = p - base;  // local blocks i0 .. i1 - 1 of stream u
    const int nblk = i1 - i0;
    const int T = c.seq_len[u / c.H];
    const int nb = (T + c.bs - 1) >> c.log2bs;
    const int32_t* list = DENSE ? nullptr : a.union_idx + (size_t)u * c.cap_blocks + i0;
    const uint32_t* hmask = DENSE ? nullptr : a.head_mask + (size_t)u * c.cap_blocks;
    const char* kbase = static_cast<const char*>(c.k) + (size_t)u * c.cap * RB;
    const char* vbase = static_cast<const char*>(c.v) + (size_t)u * c.cap * RB;
    // Query operand (head n, dims 32 kk + 8 grp + i), scaled, split hi + lo.
    // Lanes of padding heads (n >= G) load head G-1 and use zeros.
    bf16x8 qhi[NK], qlo[NK];
    {
      const int hn = min(n, G - 1);
      const float4* qn =
          reinterpret_cast<const float4*>(a.q + ((size_t)u * G + hn) * D + 8 * grp);
      const float sc = n < G ? a.scale : 0.f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const float4 x0 = qn[8 * kk], x1 = qn[8 * kk + 1];
        const float x8[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = x8[i] * sc;
          const __bf16 h = (__bf16)x;
          qhi[kk][i] = h;
          qlo[kk][i] = (__bf16)(x - (float)h);
        }
      }
    }
    const float tau_n = MODE == ETA_LOGIT_GATED ? a.tau[(size_t)u * G + min(n, G - 1)] : 0.f;
    // Gate of Eq. 3: sigmoid(beta (S - tau)) = 1 / (1 + 2^(S gk1 + gk0)).
    const float gk0 = a.beta * kLog2e * tau_n;
    // Block indices and head masks, 64 per register: lane x holds entry
    // bb + x in (lst0, hm0) and bb + 64 + x in (lst1, hm1).  The window moves
    // on by 64 when a tile about to be loaded reaches past it (a tile spans at
    // most 8 blocks, so one move suffices); the tiles still to be computed,
    // at most two tiles behind it, then lie inside the new window.
    int bb = 0, lst0, lst1;
    uint32_t hm0, hm1;
    auto load_entry = [&](int x, int& j, uint32_t& hm) {
      if constexpr (DENSE) {
        j = x < nblk ? i0 + x : -1;
        hm = G >= 32 ? 0xffffffffu : (1u << G) - 1u;
      } else {
        j = x < nblk ? list[x] : -1;
        hm = (unsigned)j < (unsigned)nb ? hmask[j] : 0u;
      }
    };
    load_entry(lane, lst0, hm0);
    load_entry(64 + lane, lst1, hm1);
    // (block index, head mask) of segment row rr; every lane takes part.
    auto entry = [&](int rr, int& j, uint32_t& hm) {
      const int o = (rr >> c.log2bs) - bb;
      if constexpr (WHOLE) {  // the same entry for every lane
        const int ou = __builtin_amdgcn_readfirstlane(o);
        const int src0 = ou < 64 ? lst0 : lst1;
        const int src1 = (int)(ou < 64 ? hm0 : hm1);
        j = __builtin_amdgcn_readlane(src0, ou & 63);
        hm = (uint32_t)__builtin_amdgcn_readlane(src1, ou & 63);
      } else {
        const int j0 = __shfl(lst0, o & 63, kWave), j1 = __shfl(lst1, o & 63, kWave);
        const int h0 = __shfl((int)hm0, o & 63, kWave), h1 = __shfl((int)hm1, o & 63, kWave);
        j = o < 64 ? j0 : j1;
        hm = (uint32_t)(o < 64 ? h0 : h1);
      }
    };
    const int rows = nblk << c.log2bs;
    const int ntiles = (rows + kTileKeys - 1) / kTileKeys;
    // Segment row rr -> absolute key position, or -1.
    auto key_pos = [&](int rr, int j) {
      const bool ok = rr < rows && (unsigned)j < (unsigned)nb;
      const int s = ok ? (j << c.log2bs) + (rr & (c.bs - 1)) : -1;
      return s < T ? s : -1;
    };
    // Coalesced loads of tile t: instruction it reads row it*RPI + ri, bytes
    // 16 cc .. 16 cc + 15, of K and of V.  Nothing here waits for the data.
    auto fetch = [&](int t, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
      const int last = min(((t + 1) * kTileKeys - 1) >> c.log2bs, nblk - 1);
      if (last >= bb + 128) {  // wave-uniform; once per 64 blocks
        lst0 = lst1;
        hm0 = hm1;
        bb += 64;
        load_entry(bb + 64 + lane, lst1, hm1);
      }
      if constexpr (WHOLE) {
        int j;
        uint32_t hm;
        entry(t * kTileKeys, j, hm);
        const int s0 = (j << c.log2bs) + ((t * kTileKeys) & (c.bs - 1));  // tile row 0
        if ((unsigned)j < (unsigned)nb && s0 + kTileKeys <= T) {  // every row valid
          const size_t tb = (size_t)s0 * RB;
#pragma unroll
          for (int it = 0; it < NI; ++it) {
            const size_t off = tb + (size_t)((it * RPI + ri) * RB + 16 * cc);
            kr[it] = ld16_nt(kbase + off);
            vr[it] = ld16_nt(vbase + off);
          }
          return;
        }
      }
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int key = it * RPI + ri;
        const int rr = t * kTileKeys + key;
        int j;
        uint32_t hm;
        entry(rr, j, hm);
        const size_t row = (size_t)max(key_pos(rr, j), 0) * RB + 16 * cc;
        kr[it] = ld16_nt(kbase + row);
        vr[it] = ld16_nt(vbase + row);
      }
    };
    // Registers -> LDS rows (chunk slot cc ^ swizzle).
    auto stage = [&](const uint4 (&kr)[NI], const uint4 (&vr)[NI]) {
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int key = it * RPI + ri;
        const int row = tile_row<D>(key) * RB;
        *reinterpret_cast<uint4*>(s_stage + row + 16 * (cc ^ tile_kswz<D>(key))) = kr[it];
        *reinterpret_cast<uint4*>(s_stage + TB + row + 16 * (cc ^ vrow_swz(key))) = vr[it];
      }
    };
    floatx4 O[NV];
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) O[nv] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m = -__builtin_inff(), lsum = 0.f;
    auto compute = [&](int t) {
      const char* sk = s_stage;
      const char* sv = s_stage + TB;
      const int r0 = t * kTileKeys;
      floatx4 S[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int key = tile_key(st, n);
        const char* row = sk + tile_row<D>(key) * RB;
        const int sw = tile_kswz<D>(key);
        S[st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const bf16x8 kv = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(row + 16 * ((4 * kk + grp) ^ sw)));
          S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qhi[kk], S[st], 0, 0, 0);
          S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[kk], S[st], 0, 0, 0);
        }
      }
      // Logits, masks and the running max of head n.  Score i of half st is
      // key 2 grp + st + 8 i of the tile.
      float lg[8];
      float tmax = -__builtin_inff();
      auto gated = [&](float d) {
        return d * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(d, gk1, gk0)));
      };
      bool fast = false;
      if constexpr (WHOLE) {
        int j;
        uint32_t hm;
        entry(r0, j, hm);
        const int s0 = (j << c.log2bs) + (r0 & (c.bs - 1));
        // Every key valid and none of them the own key T - 1.
        fast = (unsigned)j < (unsigned)nb && s0 + kTileKeys < T;
        if (fast) {
          const bool hb = (hm >> n) & 1u;
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float d = S[st][i];
              lg[4 * st + i] = hb ? (MODE == ETA_LOGIT_GATED ? gated(d) : d) : -__builtin_inff();
              tmax = fmaxf(tmax, lg[4 * st + i]);
            }
        }
      }
      if (!fast) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = r0 + 2 * grp + st + 8 * i;
            int j;
            uint32_t hm;
            entry(rr, j, hm);
            const int s = key_pos(rr, j);
            const bool on = (s >= 0) & ((hm >> n) & 1u);
            const float d = S[st][i];
            float lv = d;
            if (MODE == ETA_LOGIT_GATED && s != T - 1) lv = gated(d);
            lg[4 * st + i] = on ? lv : -__builtin_inff();
            tmax = fmaxf(tmax, lg[4 * st + i]);
          }
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      // Lazy rescaling: the reference max m of a head moves only when a tile
      // raises the head's max above m + kLazyRaise (then every head moves to
      // its own max, one wave-uniform branch).  Weights relative to m stay
      // below e^kLazyRaise, well inside float32, and the softmax does not
      // depend on the choice of reference.
      if (__ballot(tmax > m + kLazyRaise) != 0ull) {
        const float mn = fmaxf(m, tmax);
        const float alpha =
            mn == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f((m - mn) * kLog2e);
        lsum *= alpha;
        // O rows are heads 4*grp + i: their factors come from lanes 4*grp + i.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * grp + i, kWave);
#pragma unroll
          for (int nv = 0; nv < NV; ++nv) O[nv][i] *= al;
        }
        m = mn;
      }
      const float ms2 = m == -__builtin_inff() ? 0.f : m * kLog2e;
      float pw[8], psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pw[i] = __builtin_amdgcn_exp2f(fmaf(lg[i], kLog2e, -ms2));
        psum += pw[i];
      }
      lsum += psum;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_hi_lo(pw[2 * i], pw[2 * i + 1], ph[i], pl[i]);
      const bf16x8 phi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
      const bf16x8 plo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
      // Value operand (dim 16 nv + n, slots 8 grp + 4 h + j) by two
      // transposing reads of the staged V rows.
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) {
        const int cidx = 2 * nv + (tr4 >> 1);
        const uint2 v0 = tr_read(sv + tile_row<D>(trow0) * RB + 16 * (cidx ^ vrow_swz(trow0)) +
                                 8 * (tr4 & 1));
        const uint2 v1 = tr_read(sv + tile_row<D>(trow1) * RB + 16 * (cidx ^ vrow_swz(trow1)) +
                                 8 * (tr4 & 1));
        const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
        O[nv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vb, O[nv], 0, 0, 0);
        O[nv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vb, O[nv], 0, 0, 0);
      }
    };
    if constexpr (Sh::Ahead == 2) {
      // Two register sets: tiles t + 1 and t + 2 are in flight during the
      // compute of tile t (tile t + 2 is requested once tile t is staged).
      uint4 ka[NI], va[NI], kb[NI], vb2[NI];
      fetch(0, ka, va);
      if (1 < ntiles) fetch(1, kb, vb2);
      for (int t = 0; t < ntiles; t += 2) {
        stage(ka, va);
        if (t + 2 < ntiles) fetch(t + 2, ka, va);
        wave_lds_sync();
        compute(t);
        wave_lds_sync();
        if (t + 1 >= ntiles) break;
        stage(kb, vb2);
        if (t + 3 < ntiles) fetch(t + 3, kb, vb2);
        wave_lds_sync();
        compute(t + 1);
        wave_lds_sync();
      }
    } else {
      // The next tile's loads are issued once the current one is staged, so
      // they are in flight during its compute.
      uint4 kr[NI], vr[NI];
      fetch(0, kr, vr);
      for (int t = 0; t < ntiles; ++t) {
        stage(kr, vr);
        if (t + 1 < ntiles) fetch(t + 1, kr, vr);
        wave_lds_sync();
        compute(t);
        wave_lds_sync();
      }
    }
    // Head n's sum over the 4 lane groups (they share the reference max).
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    const size_t slot = ((size_t)w + u) * G;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      if (h < G) {
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) a.part_acc[(slot + h) * D + 16 * nv + n] = O[nv][i];
      }
    }
    if (grp == 0 && n < G) {
      a.part_m[slot + n] = m;
      a.part_l[slot + n] = lsum;
    }
    p = base + i1;
    if (p < pend) {  // next non-empty stream
      do ++u; while (start_of(u + 1) <= p);
      u = __builtin_amdgcn_readfirstlane(u);
    }
  }
}

// Offsets of the balanced grouped decode for more KV streams than LDS holds,
// by one work-group: flow_start[u] = union blocks of the streams before u
// (rounds of 1024 streams with a running carry), flow_info[0] = N, and
// flow_wave_u[w] = the stream holding position lo(w) of wave w's range
// (lo(w) = floor(w N / wn) >= start[u] exactly when w >= ceil(start[u] wn / N)).
__global__ __launch_bounds__(1024) void flow_scan_gqa_kernel(CacheView c, GqaArgs a, int waves) {
  __shared__ int s_w[1024 / kWave];
  __shared__ int s_carry;
  const int units = c.B * c.H, t = threadIdx.x;
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int r = 0; r < units; r += 1024) {
    const int u = r + t;
    int T, cnt = 0;
    if (u < units) gqa_stream(c, a, a.dense, u, &T, &cnt);
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

// Combine of the balanced grouped decode: one work-group per query head; its
// partials sit in slots (w + u) * G + g for the ranges w that cover stream u,
// a few tens at most (log-sum-exp in one pass, 4 waves, 4 partials in flight
// per wave, fixed-order wave merge); zeros for empty streams.
template <int D>
__global__ __launch_bounds__(256) void combine_gqa_flow_kernel(CacheView c, GqaArgs a) {
  constexpr int W = 4, INF = 4, CPL = D / kWave;
  __shared__ float s_acc[W][D];
  __shared__ float s_ml[W][2];
  const int uq = blockIdx.x, G = a.G, u = uq / G, g = uq % G;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int p0 = a.flow_start[u], p1 = a.flow_start[u + 1];
  if (p1 <= p0) {
    if (t < D) a.out[(size_t)uq * D + t] = 0.f;
    return;
  }
  const FlowPlan plan(a.flow_info[0], a.flow_grid, a.split);
  const int wf = plan.range_of(p0), wl = plan.range_of(p1 - 1);
  const int nch = wl - wf + 1;
  const size_t slot0 = ((size_t)wf + u) * G + g;
  const float* pm = a.part_m + slot0;
  const float* pl = a.part_l + slot0;
  const float* pa = a.part_acc + slot0 * D + lane * CPL;
  float m = -__builtin_inff(), l = 0.f, acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
  for (int base = wave; base < nch; base += W * INF) {
    float mc[INF], lc[INF], ac[INF][CPL];
#pragma unroll
    for (int i = 0; i < INF; ++i) {
      const int ch = base + W * i;
      const bool ok = ch < nch;
      const size_t o = (size_t)ch * G;
      mc[i] = ok ? pm[o] : -__builtin_inff();
      lc[i] = ok ? pl[o] : 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) ac[i][e] = ok ? pa[o * D + e] : 0.f;
    }
    float mx = m;
#pragma unroll
    for (int i = 0; i < INF; ++i) mx = fmaxf(mx, mc[i]);
    const float ms = (mx == -__builtin_inff()) ? 0.f : mx;
    const float alpha = __builtin_amdgcn_exp2f((m - ms) * kLog2e);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < INF; ++i) {
      const float wgt = __builtin_amdgcn_exp2f((mc[i] - ms) * kLog2e);
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
    float mm = s_ml[0][0], ll = s_ml[0][1], aa = s_acc[0][t];
    for (int w2 = 1; w2 < W; ++w2) {
      const float m2 = s_ml[w2][0], l2 = s_ml[w2][1], a2 = s_acc[w2][t];
      const float mx = fmaxf(mm, m2);
      const float ms = (mx == -__builtin_inff()) ? 0.f : mx;
      const float s1 = __builtin_amdgcn_exp2f((mm - ms) * kLog2e);
      const float s2 = __builtin_amdgcn_exp2f((m2 - ms) * kLog2e);
      ll = ll * s1 + l2 * s2;
      aa = aa * s1 + a2 * s2;
      mm = mx;
    }
    a.out[(size_t)uq * D + t] = aa / ll;
  }
}

// ---------------------------------------------------------------------------
template <int D>
static hipError_t screen_gqa_t(const CacheView& c, int G, const float* q, const float* ts,
                               float z, float scale, int32_t* idx, uint32_t* mask, int32_t* cnt,
                               uint64_t* ctr, uint64_t* words, hipStream_t s) {
  const int units = c.B * c.H;
  const int wpu = ceil_div(c.cap_blocks, 64);
  // per-word head-token counts follow the words in the workspace
  uint32_t* wtok = reinterpret_cast<uint32_t*>(words + (size_t)units * wpu);
  const dim3 grid((unsigned)((long long)wpu * units));
  if (G <= 8)
    hipLaunchKernelGGL((screen_gqa_kernel<D, 8>), grid, dim3(256), 0, s, c, G, q, ts, z, scale,
                       mask, words, wtok, wpu);
  else
    hipLaunchKernelGGL((screen_gqa_kernel<D, 16>), grid, dim3(256), 0, s, c, G, q, ts, z, scale,
                       mask, words, wtok, wpu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_gqa_kernel, dim3(units), dim3(256), 0, s, c, words, wtok, wpu, idx,
                     cnt, ctr);
  return hipGetLastError();
}

hipError_t launch_screen_gqa(const CacheView& c, int G, const float* q, const float* ts, float z,
                             float scale, int32_t* idx, uint32_t* mask, int32_t* cnt,
                             uint64_t* ctr, uint64_t* words, hipStream_t s) {
  return c.D == 128 ? screen_gqa_t<128>(c, G, q, ts, z, scale, idx, mask, cnt, ctr, words, s)
                    : screen_gqa_t<64>(c, G, q, ts, z, scale, idx, mask, cnt, ctr, words, s);
}

// Work-groups of the balanced grouped decode: as many as are resident at once
// (one wave each; registers and LDS set the count).
template <int D, int MODE, bool WHOLE, bool GS, bool DENSE>
static int gqa_flow_grid(int units) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu,
          reinterpret_cast<const void*>(decode_gqa_flow_kernel<D, MODE, WHOLE, GS, DENSE>), 64,
          GS ? 0 : (size_t)(units + 1) * 4) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return device_cus() * min(per_cu, kMaxFlowWavesPerCU);
}

template <int D, int MODE, bool DENSE>
static hipError_t decode_gqa_t(const CacheView& c, const GqaDecode& g, hipStream_t s) {
  const int units = c.B * c.H;
  {
    GqaArgs f = g;
    hipError_t e;
    if (f.flow_global) {
      f.flow_grid = c.bs >= kTileKeys ? gqa_flow_grid<D, MODE, true, true, DENSE>(units)
                                      : gqa_flow_grid<D, MODE, false, true, DENSE>(units);
      hipLaunchKernelGGL(flow_scan_gqa_kernel, dim3(1), dim3(1024), 0, s, c, f, f.flow_grid);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (c.bs >= kTileKeys)
        hipLaunchKernelGGL((decode_gqa_flow_kernel<D, MODE, true, true, DENSE>),
                           dim3(f.flow_grid), dim3(64), 0, s, c, f);
      else
        hipLaunchKernelGGL((decode_gqa_flow_kernel<D, MODE, false, true, DENSE>),
                           dim3(f.flow_grid), dim3(64), 0, s, c, f);
    } else if (c.bs >= kTileKeys) {
      f.flow_grid = gqa_flow_grid<D, MODE, true, false, DENSE>(units);
      hipLaunchKernelGGL((decode_gqa_flow_kernel<D, MODE, true, false, DENSE>),
                         dim3(f.flow_grid), dim3(64), (size_t)(units + 1) * 4, s, c, f);
    } else {
      f.flow_grid = gqa_flow_grid<D, MODE, false, false, DENSE>(units);
      hipLaunchKernelGGL((decode_gqa_flow_kernel<D, MODE, false, false, DENSE>),
                         dim3(f.flow_grid), dim3(64), (size_t)(units + 1) * 4, s, c, f);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((combine_gqa_flow_kernel<D>), dim3(units * g.G), dim3(256), 0, s, c, f);
    return hipGetLastError();
  }
}

template <int D>
static hipError_t decode_gqa_d(const CacheView& c, const GqaDecode& g, hipStream_t s) {
  if (g.dense) return decode_gqa_t<D, ETA_LOGIT_RAW, true>(c, g, s);
  if (g.mode == ETA_LOGIT_RAW) return decode_gqa_t<D, ETA_LOGIT_RAW, false>(c, g, s);
  return decode_gqa_t<D, ETA_LOGIT_GATED, false>(c, g, s);
}

hipError_t launch_decode_gqa(const CacheView& c, const GqaDecode& g, hipStream_t s) {
  return c.D == 128 ? decode_gqa_d<128>(c, g, s) : decode_gqa_d<64>(c, g, s);
}

}  // namespace eta
