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
// scores blocks 16 w .. 16 w + 15 of the word (8 lanes per block).  A block's
// statistics are loaded once and scored against every query head of the
// group (queries, norms and thresholds staged in LDS).  Writes the per-block
// head mask (bit g: query head u*G + g admits the block) for every block of
// the stream and the union admission word.
template <int D>
__global__ __launch_bounds__(256) void screen_gqa_kernel(CacheView c, int G, const float* q,
                                                         const float* tau_screen, float z,
                                                         float scale, uint32_t* head_mask,
                                                         uint64_t* words, int words_per_unit) {
  constexpr int LPB = 8;            // lanes per block
  constexpr int NL = D / 32;        // float4 loads per lane per statistics row
  __shared__ float s_q[kMaxGroup][D];
  __shared__ float s_qn[kMaxGroup];
  __shared__ float s_ts[kMaxGroup];
  __shared__ uint32_t s_bits[4];
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
  float4 m4[2][NL], v4[2][NL];
  float Ms[2];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (wd << 6) + wave * 16 + it * 8 + gi;
    const bool scored = j < nbc;
    const size_t row = ((size_t)u * c.cap_blocks + j) * D;
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      m4[it][t] = scored ? ld16f_nt(c.mu + row + 32 * t + 4 * li) : make_float4(0, 0, 0, 0);
      v4[it][t] = scored ? ld16f_nt(c.var + row + 32 * t + 4 * li) : make_float4(0, 0, 0, 0);
    }
    Ms[it] = scored ? c.maxnorm[(size_t)u * c.cap_blocks + j] : 0.f;
  }
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) s_q[i / D][i % D] = q[(size_t)u * G * D + i];
  if (threadIdx.x < G) s_ts[threadIdx.x] = tau_screen[(size_t)u * G + threadIdx.x];
  __syncthreads();
  // ||q|| per head, 8 lanes per head summing in the same order as the
  // one-head-per-KV-head screen (so G = 1 reproduces it bit for bit).
  {
    const int hg = wave * 8 + gi;
    float qq = 0.f;
    if (hg < G) {
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const float4 v = *reinterpret_cast<const float4*>(&s_q[hg][32 * t + 4 * li]);
        qq = fmaf(v.x, v.x, qq);
        qq = fmaf(v.y, v.y, qq);
        qq = fmaf(v.z, v.z, qq);
        qq = fmaf(v.w, v.w, qq);
      }
    }
    qq = group_sum<LPB>(qq);
    if (hg < G && li == 0) s_qn[hg] = sqrtf(qq);
  }
  __syncthreads();
  const bool z_inf = __builtin_isinf(z);
  const uint32_t all = (G >= 32) ? 0xffffffffu : ((1u << G) - 1u);
  uint32_t bits = 0;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int j = (wd << 6) + wave * 16 + it * 8 + gi;
    const bool scored = j < nbc;
    const float M = Ms[it];
    uint32_t mask = 0;
    for (int g = 0; g < G; ++g) {
      float dot = 0.f, mom = 0.f;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const float4 qv = *reinterpret_cast<const float4*>(&s_q[g][32 * t + 4 * li]);
        dot = fmaf(qv.x, m4[it][t].x, dot);
        dot = fmaf(qv.y, m4[it][t].y, dot);
        dot = fmaf(qv.z, m4[it][t].z, dot);
        dot = fmaf(qv.w, m4[it][t].w, dot);
        mom = fmaf(qv.x * qv.x, v4[it][t].x, mom);
        mom = fmaf(qv.y * qv.y, v4[it][t].y, mom);
        mom = fmaf(qv.z * qv.z, v4[it][t].z, mom);
        mom = fmaf(qv.w * qv.w, v4[it][t].w, mom);
      }
      dot = group_sum<LPB>(dot);
      mom = group_sum<LPB>(mom);
      const float geometric = s_qn[g] * M;
      const float sc = z_inf ? scale * geometric
                             : scale * fminf(fmaf(z, sqrtf(mom), dot), geometric);
      if (scored && sc >= s_ts[g]) mask |= 1u << g;
    }
    if (j == nb - 1) mask = all;  // the last block is admitted for every head
    if (li == 0 && j < nb) head_mask[(size_t)u * c.cap_blocks + j] = mask;
    const uint64_t bal = __ballot(mask != 0u);
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8)
      bits |= (uint32_t)((bal >> (g8 * LPB)) & 1ull) << (it * 8 + g8);
  }
  if (lane == 0) s_bits[wave] = bits;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t word = (uint64_t)s_bits[0] | ((uint64_t)s_bits[1] << 16) |
                          ((uint64_t)s_bits[2] << 32) | ((uint64_t)s_bits[3] << 48);
    words[(size_t)u * words_per_unit + wd] = word;
  }
}

// Compaction of the union words into the ascending union list, plus the
// counters: ctr[0] += admitted tokens summed over the group's query heads,
// ctr[1] += union tokens.  Thread t takes a run of bpt consecutive blocks
// (bpt a power of two <= 64, so a run lies in one word), rounds of 256 runs
// in ascending order; a work-group scan places each run's entries.  The head
// masks of the run's admitted blocks are independent loads.
__global__ __launch_bounds__(256) void compact_gqa_kernel(CacheView c, const uint64_t* words,
                                                          int words_per_unit,
                                                          const uint32_t* head_mask,
                                                          int32_t* union_idx, int32_t* union_cnt,
                                                          uint64_t* ctr) {
  __shared__ int scan[256];
  __shared__ unsigned long long s_tok[256];
  const int u = blockIdx.x, t = threadIdx.x;
  const int T = c.seq_len[u / c.H];
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const uint64_t* wu = words + (size_t)u * words_per_unit;
  const uint32_t* hm = head_mask + (size_t)u * c.cap_blocks;
  int32_t* out = union_idx + (size_t)u * c.cap_blocks;
  const int tail = T - ((nb - 1) << c.log2bs);
  int bpt = 1;
  while (bpt < 64 && bpt * 256 < nb) bpt <<= 1;
  int base_pos = 0;
  unsigned long long head_tokens = 0;
  for (int r0 = 0; r0 < nb; r0 += 256 * bpt) {
    const int b0 = r0 + t * bpt;  // first block of this thread's run
    uint64_t x = 0;
    if (b0 < nb) {
      x = wu[b0 >> 6] >> (b0 & 63);
      if (bpt < 64) x &= (1ull << bpt) - 1ull;
      const int rem = nb - b0;
      if (rem < 64) x &= (1ull << rem) - 1ull;
    }
    const int mine = __popcll(x);
    scan[t] = mine;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = t >= off ? scan[t - off] : 0;
      __syncthreads();
      scan[t] += add;
      __syncthreads();
    }
    int pos = base_pos + scan[t] - mine;
    base_pos += scan[255];
    __syncthreads();  // scan[] is rewritten next round
    while (x) {
      const int j = b0 + __ffsll((unsigned long long)x) - 1;
      out[pos++] = j;
      head_tokens += (unsigned long long)__popc(hm[j]) * (j == nb - 1 ? tail : c.bs);
      x &= x - 1ull;
    }
  }
  s_tok[t] = head_tokens;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (t < st) s_tok[t] += s_tok[t + st];
    __syncthreads();
  }
  if (t == 0) {
    const int total = base_pos;
    union_cnt[u] = total;
    if (ctr && total > 0) {
      atomicAdd(reinterpret_cast<unsigned long long*>(ctr), s_tok[0]);
      const unsigned long long ut =
          (unsigned long long)(total - 1) * c.bs + (unsigned long long)tail;
      atomicAdd(reinterpret_cast<unsigned long long*>(ctr + 1), ut);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode.  One work-group of W waves (4 for d = 64, 2 for d = 128) per chunk
// of `split` union blocks of KV stream u; wave w takes the 32-key tiles w,
// w + W, ...  A tile passes through the wave's own LDS area:
//   load    coalesced 128-bit reads of whole K and V rows (d/8 lanes per row)
//           into registers.  The loads of the wave's next tile are issued as
//           soon as these registers are in LDS, so they overlap the compute of
//           the current tile at no register cost;
//   stage   K rows as stored, each row's 16-byte chunks permuted by an XOR
//           with a function of the key so that the operand reads below hit
//           distinct LDS banks; V transposed, vt[dim][k] with k = 4 (key % 8)
//           + key / 8, rows of 18 words, the 8-byte groups of 4 keys permuted
//           by an XOR with a function of the dim (the same goal, for writes
//           and reads);
//   scores  for each 16-key half st: S[16 keys x 16 heads] = K (A operand:
//           lane l holds key rho(st, l % 16) = 2 ((l%16) / 4) + st +
//           8 ((l%16) % 4), dims 32 kk + 8 (l / 16) .. + 7) times Q^T (B: head
//           l % 16, the same dims; q split hi + lo).  Lane l receives head
//           l % 16 and keys rho(st, 4 (l / 16) + i), i < 4;
//   softmax per head with a lazily moved reference max; weights split hi + lo;
//   values  O[16 heads x 16 dims] += P (A: head l % 16, contraction slots
//           k = 8 (l / 16) + i: by the choice of rho and of the vt order these
//           are exactly the lane's 8 score keys) times V (B: dim l % 16, the
//           same slots, one 16-byte read of vt).
// The W waves' (max, sum, O) are merged through LDS and written as the
// chunk's partial per query head (or the output for single-chunk streams).

template <int D>
struct GqaShape {
  static constexpr int W = D == 64 ? 4 : 2;        // waves per work-group
  // d = 64: at most 168 registers per lane, 3 work-groups (12 waves) per CU.
  // The register budget holds the wave's next tile in flight during the
  // compute of the current one; at 4 per CU (128 registers) it spills.
  // Measured on 32 x 128K at 57% union: 431 us (3 per CU) vs 448 us (4, with
  // spills).
  static constexpr int MinBlocks = D == 64 ? 3 : 1;
  static constexpr int NK = D / 32;                 // 32-dim slabs (score product)
  static constexpr int NV = D / 16;                 // 16-dim slabs (value product)
  static constexpr int RB = D * 2;                  // bytes per bf16 row
  static constexpr int LPR = D / 8;                 // lanes per row in a coalesced load
  static constexpr int RPI = 64 / LPR;              // rows per load instruction
  static constexpr int NI = kTileKeys / RPI;        // load instructions per tile and tensor
  static constexpr int QPL = 8 / RPI;               // vt key groups per lane
  static constexpr int KStride = RB;                // staged K row stride, bytes
  static constexpr int KBytes = kTileKeys * KStride;
  static constexpr int VBytes = D * kVtWords * 4;
  static constexpr int WaveBytes = KBytes + VBytes;  // per-wave LDS area
  static constexpr int MergeBytes = W * 16 * D * 4;
  static_assert(MergeBytes <= W * WaveBytes, "merge area reuses the staging areas");
};

using GqaArgs = GqaDecode;

__device__ __forceinline__ int gqa_stream(const CacheView& c, const GqaArgs& a, bool dense, int u,
                                          int* T_out, int* cnt_out) {
  const int T = c.seq_len[u / c.H];
  const int nb = T > 0 ? (T + c.bs - 1) >> c.log2bs : 0;
  const int cnt = dense ? nb : max(0, min(a.union_cnt[u], nb));
  *T_out = T;
  *cnt_out = cnt;
  return (cnt + a.split - 1) / a.split;
}

template <int D, int MODE, bool DENSE>
__global__ __launch_bounds__(GqaShape<D>::W * 64, GqaShape<D>::MinBlocks) void decode_gqa_kernel(CacheView c, GqaArgs a) {
  using Sh = GqaShape<D>;
  constexpr int W = Sh::W, NK = Sh::NK, NV = Sh::NV, RB = Sh::RB;
  constexpr int LPR = Sh::LPR, RPI = Sh::RPI, NI = Sh::NI, QPL = Sh::QPL;
  extern __shared__ __align__(16) char s_raw[];
  float* s_o = reinterpret_cast<float*>(s_raw);                        // merge: [W][16][D]
  // chunk's block list: (block index, head mask) per slot
  int2* s_blk = reinterpret_cast<int2*>(s_raw + W * Sh::WaveBytes);    // [split]
  __shared__ float s_ml[W][16][2];

  const int u = blockIdx.x / a.max_chunks;
  const int k = rotated_chunk(blockIdx.x % a.max_chunks, u, a.max_chunks);
  int T, cnt;
  const int nch = gqa_stream(c, a, DENSE, u, &T, &cnt);
  if (k >= nch) return;
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int first = k * a.split, nblk = min(a.split, cnt - first);
  const int G = a.G;
  const uint32_t all = (1u << G) - 1u;
  for (int i = threadIdx.x; i < nblk; i += blockDim.x) {
    if constexpr (DENSE) {
      s_blk[i] = make_int2(first + i, (int)all);
    } else {
      const int j = a.union_idx[(size_t)u * c.cap_blocks + first + i];
      const uint32_t hm =
          ((unsigned)j < (unsigned)nb) ? a.head_mask[(size_t)u * c.cap_blocks + j] : 0u;
      s_blk[i] = make_int2(j, (int)hm);
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;  // operand layout: row/column n, k group grp
  char* s_k = s_raw + wave * Sh::WaveBytes;  // staged K tile
  char* s_v = s_k + Sh::KBytes;              // transposed V tile

  // Query operand (head n, dims 32*kk + 8*grp + i), scaled, split hi + lo.
  // Lanes of padding heads (n >= G) load head G-1 and use zeros.
  bf16x8 qhi[NK], qlo[NK];
  {
    const int hn = min(n, G - 1);
    const float4* qn =
        reinterpret_cast<const float4*>(a.q + ((size_t)u * G + hn) * D + 8 * grp);
    float4 qv[NK][2];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      qv[kk][0] = qn[8 * kk];
      qv[kk][1] = qn[8 * kk + 1];
    }
    const float sc = n < G ? a.scale : 0.f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const float x8[8] = {qv[kk][0].x, qv[kk][0].y, qv[kk][0].z, qv[kk][0].w,
                           qv[kk][1].x, qv[kk][1].y, qv[kk][1].z, qv[kk][1].w};
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
  const float gk1 = -a.beta * kLog2e, gk0 = a.beta * kLog2e * tau_n;
  const char* kbase = static_cast<const char*>(c.k) + (size_t)u * c.cap * RB;
  const char* vbase = static_cast<const char*>(c.v) + (size_t)u * c.cap * RB;
  __syncthreads();  // s_blk

  floatx4 O[NV];
#pragma unroll
  for (int nv = 0; nv < NV; ++nv) O[nv] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_inff(), lsum = 0.f;

  const int rows = nblk << c.log2bs;
  const int ntiles = (rows + kTileKeys - 1) / kTileKeys;
  // Chunk row rr -> absolute key position, or -1 past the chunk, past the
  // stream or for an out-of-range list entry.
  auto key_pos = [&](int rr, int j) {
    const int s = (j << c.log2bs) + (rr & (c.bs - 1));
    return (rr < rows && (unsigned)j < (unsigned)nb && s < T) ? s : -1;
  };
  auto slot_of = [&](int rr) { return min(rr >> c.log2bs, nblk - 1); };

  // Coalesced loads of tile t: instruction it reads key it*RPI + lane/LPR,
  // bytes 16 (lane % LPR) .. +15.  Invalid keys read row 0 of the stream
  // (always in bounds) and are zeroed when staged; bit it of `ok` records
  // validity.  Nothing here waits for the data.
  const int ri = lane / LPR, cc = lane % LPR;
  auto fetch = [&](int t, uint4 (&kr)[NI], uint4 (&vr)[NI], uint32_t& ok) {
    int js[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) js[it] = s_blk[slot_of(t * kTileKeys + it * RPI + ri)].x;
    ok = 0;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int s = key_pos(t * kTileKeys + it * RPI + ri, js[it]);
      const size_t off = (size_t)max(s, 0) * RB + 16 * cc;
      kr[it] = ld16_nt(kbase + off);
      vr[it] = ld16_nt(vbase + off);
      ok |= (s >= 0 ? 1u : 0u) << it;
    }
  };
  // Registers -> LDS (zeros for invalid keys).
  auto stage = [&](uint4 (&kr)[NI], uint4 (&vr)[NI], uint32_t ok) {
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      kr[it] = keep(kr[it], (ok >> it) & 1u);
      vr[it] = keep(vr[it], (ok >> it) & 1u);
      const int key = it * RPI + ri;
      const int chunk = cc ^ k_swz(key);
      *reinterpret_cast<uint4*>(s_k + key * Sh::KStride + 16 * chunk) = kr[it];
    }
#pragma unroll
    for (int qi = 0; qi < QPL; ++qi) {
      const int q = ri + RPI * qi;  // keys q + 8 j sit in instructions qi + QPL j
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const int dim = 8 * cc + 2 * w2;
        const uint32_t x0 = word(vr[qi], w2), x1 = word(vr[qi + QPL], w2);
        const uint32_t x2 = word(vr[qi + 2 * QPL], w2), x3 = word(vr[qi + 3 * QPL], w2);
        // dims `dim` (low halves) and dim + 1 (high halves) of keys q + 8 j
        const uint2 lo = make_uint2((x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16));
        const uint2 hi = make_uint2((x0 >> 16) | (x1 & 0xffff0000u),
                                    (x2 >> 16) | (x3 & 0xffff0000u));
        *reinterpret_cast<uint2*>(s_v + (dim * kVtWords + 2 * (q ^ v_swz(dim))) * 4) = lo;
        *reinterpret_cast<uint2*>(s_v + ((dim + 1) * kVtWords + 2 * (q ^ v_swz(dim + 1))) * 4) =
            hi;
      }
    }
  };
  auto compute = [&](int t) {
    const int r0 = t * kTileKeys;
    // Scores.
    floatx4 S[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key = tile_key(st, n);
      const char* row = s_k + key * Sh::KStride;
      const int sw = k_swz(key);
      S[st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const uint4 kx = *reinterpret_cast<const uint4*>(row + 16 * ((4 * kk + grp) ^ sw));
        const bf16x8 kv = __builtin_bit_cast(bf16x8, kx);
        S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qhi[kk], S[st], 0, 0, 0);
        S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qlo[kk], S[st], 0, 0, 0);
      }
    }
    // Logits, masks and the running max of head n.  Score i of half st is
    // key 2 grp + st + 8 i of the tile.
    float lg[8];
    float tmax = -__builtin_inff();
    int2 blk[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) blk[st][i] = s_blk[slot_of(r0 + 2 * grp + st + 8 * i)];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = r0 + 2 * grp + st + 8 * i;
        const int s = key_pos(rr, blk[st][i].x);
        const bool on = (s >= 0) & (((uint32_t)blk[st][i].y >> n) & 1u);
        const float d = S[st][i];
        float lv = d;
        if (MODE == ETA_LOGIT_GATED && s != T - 1)
          lv = d * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(d, gk1, gk0)));
        lg[4 * st + i] = on ? lv : -__builtin_inff();
        tmax = fmaxf(tmax, lg[4 * st + i]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    // Lazy rescaling: the reference max m of a head moves only when a tile
    // raises the head's max above m + kLazyRaise (then every head moves to
    // its own max, one wave-uniform branch).  Weights relative to m stay
    // below e^kLazyRaise, well inside float32, and the softmax is unchanged
    // by the choice of reference.
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
    // Values: B operand = dim 16 nv + n, contraction slots 8 grp .. 8 grp + 7.
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      const int dim = 16 * nv + n;
      const char* vrow = s_v + dim * kVtWords * 4;
      const uint2 v0 = *reinterpret_cast<const uint2*>(vrow + 8 * ((2 * grp) ^ v_swz(dim)));
      const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 8 * ((2 * grp + 1) ^ v_swz(dim)));
      const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
      O[nv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vb, O[nv], 0, 0, 0);
      O[nv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vb, O[nv], 0, 0, 0);
    }
  };

  {
    uint4 kr[NI], vr[NI];
    uint32_t ok = 0;
    int t = wave;
    if (t < ntiles) fetch(t, kr, vr, ok);
    while (t < ntiles) {
      stage(kr, vr, ok);
      if (t + W < ntiles) fetch(t + W, kr, vr, ok);
      wave_lds_sync();
      compute(t);
      wave_lds_sync();
      t += W;
    }
  }
  // Head n's sum over the 4 lane groups (they share the reference max).
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  __syncthreads();  // every wave is done with its staging area
  float* so = s_o + wave * 16 * D;
#pragma unroll
  for (int nv = 0; nv < NV; ++nv)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[(4 * grp + i) * D + 16 * nv + n] = O[nv][i];
  if (grp == 0) {
    s_ml[wave][n][0] = m;
    s_ml[wave][n][1] = lsum;
  }
  __syncthreads();
  // Merge the W waves per (head, dim) in a fixed order.
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, col = e % D;
    float mm = s_ml[0][h][0], ll = s_ml[0][h][1];
    float aa = s_o[h * D + col];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const float m2 = s_ml[w][h][0], l2 = s_ml[w][h][1], a2 = s_o[(w * 16 + h) * D + col];
      const float mx = fmaxf(mm, m2);
      const float ms = (mx == -__builtin_inff()) ? 0.f : mx;
      const float s1 = __builtin_amdgcn_exp2f((mm - ms) * kLog2e);
      const float s2 = __builtin_amdgcn_exp2f((m2 - ms) * kLog2e);
      ll = ll * s1 + l2 * s2;
      aa = aa * s1 + a2 * s2;
      mm = mx;
    }
    const size_t uq = (size_t)u * G + h;
    if (nch == 1) {
      a.out[uq * D + col] = aa / ll;
    } else {
      const size_t slot = uq * a.max_chunks + k;
      a.part_acc[slot * D + col] = aa;
      if (col == 0) {
        a.part_m[slot] = mm;
        a.part_l[slot] = ll;
      }
    }
  }
}

// Combine of the chunk partials of every query head (log-sum-exp, one pass,
// 16 waves, 8 partials in flight per wave, fixed-order wave merge); zero
// output for empty streams.
template <int D>
__global__ __launch_bounds__(1024) void combine_gqa_kernel(CacheView c, GqaArgs a, bool dense) {
  constexpr int W = 16, INF = 8, CPL = D / kWave;
  __shared__ float s_acc[W][D];
  __shared__ float s_ml[W][2];
  const int uq = blockIdx.x, t = threadIdx.x, wave = t >> 6, lane = t & 63;
  int T, cnt;
  const int nch = gqa_stream(c, a, dense, uq / a.G, &T, &cnt);
  if (nch == 0) {
    if (t < D) a.out[(size_t)uq * D + t] = 0.f;
    return;
  }
  if (nch == 1) return;  // written by the decode kernel
  const float* pm = a.part_m + (size_t)uq * a.max_chunks;
  const float* pl = a.part_l + (size_t)uq * a.max_chunks;
  const float* pa = a.part_acc + (size_t)uq * a.max_chunks * D + lane * CPL;
  float m = -__builtin_inff(), l = 0.f, acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) acc[e] = 0.f;
  for (int base = wave; base < nch; base += W * INF) {
    float mc[INF], lc[INF], ac[INF][CPL];
#pragma unroll
    for (int i = 0; i < INF; ++i) {
      const int ch = base + W * i;
      const bool ok = ch < nch;
      mc[i] = ok ? pm[ch] : -__builtin_inff();
      lc[i] = ok ? pl[ch] : 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) ac[i][e] = ok ? pa[(size_t)ch * D + e] : 0.f;
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
    for (int w = 1; w < W; ++w) {
      const float m2 = s_ml[w][0], l2 = s_ml[w][1], a2 = s_acc[w][t];
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
// Balanced grouped decode (d = 64).  As the per-head balanced decode does with
// the admitted lists, the union lists of all KV streams, concatenated in
// stream order, are cut into equal contiguous ranges, one per wave; a
// work-group is one wave and holds no state shared with others.  The wave
// walks its range in 32-key tiles: coalesced 128-bit loads of whole K and V
// rows into registers (the next tile's loads in flight while the current one
// is computed), staged as rows in the wave's LDS area (K chunk-swizzled for
// the score operand, V for the transposing read of the value operand).  Keys
// that are not to be read (past the range, the stream, or an out-of-range
// list entry) load the stream's row 0 instead -- finite data -- and are masked
// out of the softmax, so their weights are exactly zero.  Scores and values of
// all G heads run on the matrix cores as in the chunked kernel; the partial
// of (stream segment, head g) goes to slot (w + u) * G + g.  Measured on
// 32 x 128K, 38% head density: about 6% faster than the chunked kernel.
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
};

template <int D, int MODE>
__global__ __launch_bounds__(64) void decode_gqa_flow_kernel(CacheView c, GqaArgs a) {
  using Sh = GqaFlowShape<D>;
  constexpr int NK = Sh::NK, NV = Sh::NV, RB = Sh::RB, LPR = Sh::LPR, RPI = Sh::RPI;
  constexpr int NI = Sh::NI, TB = Sh::TB;
  __shared__ __align__(16) char s_stage[Sh::StageBytes];
  extern __shared__ int s_start[];  // [units + 1]
  const int units = c.B * c.H, lane = threadIdx.x, G = a.G;
  // Exclusive prefix sums of the union counts: lane x sums a run of
  // ceil(units / 64) streams, the runs are scanned across the wave.
  {
    const int per = (units + 63) / 64;
    const int u0 = min(units, lane * per), u1 = min(units, u0 + per);
    int sum = 0;
    for (int u = u0; u < u1; ++u) {
      int T, cnt;
      gqa_stream(c, a, false, u, &T, &cnt);
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
  const FlowPlan plan(s_start[units], gridDim.x, a.split);
  if (blockIdx.x == 0) {  // for the combine
    for (int u = lane; u <= units; u += kWave) a.flow_start[u] = s_start[u];
    if (lane == 0) a.flow_info[0] = plan.N;
  }
  const int w = blockIdx.x;
  if (w >= plan.wn) return;
  const int n = lane & 15, grp = lane >> 4;  // operand layout: row/column n, k group grp
  const int ri = lane / LPR, cc = lane % LPR;  // load layout: row ri, 16-byte chunk cc
  const bool whole = c.bs >= kTileKeys;      // every tile lies inside one block
  const float gk1 = -a.beta * kLog2e;
  // Value-operand rows of the transposing read (as in the prefill kernel).
  const int trow0 = tile_key(0, 4 * grp + ((lane & 15) >> 2));
  const int trow1 = tile_key(1, 4 * grp + ((lane & 15) >> 2));
  const int tr4 = lane & 3;

  int p = plan.lo(w);
  const int pend = plan.lo(w + 1);
  int u = 0;  // the last stream with start[u] <= p (so start[u + 1] > p)
  {
    int hi = units - 1;
    while (u < hi) {
      const int mid = (u + hi + 1) >> 1;
      if (s_start[mid] <= p) u = mid; else hi = mid - 1;
    }
  }
  while (p < pend) {
    const int base = s_start[u];
    const int i0 = p - base, i1 = min(pend, s_start[u + 1]) - base;  // local blocks
    const int nblk = i1 - i0;
    const int T = c.seq_len[u / c.H];
    const int nb = (T + c.bs - 1) >> c.log2bs;
    const int32_t* list = a.union_idx + (size_t)u * c.cap_blocks + i0;
    const uint32_t* hmask = a.head_mask + (size_t)u * c.cap_blocks;
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
    // on by 64 when a tile about to be loaded reaches past it; the tile still
    // to be computed then lies inside the new window.
    int bb = 0, lst0, lst1;
    uint32_t hm0, hm1;
    auto load_entry = [&](int x, int& j, uint32_t& hm) {
      j = x < nblk ? list[x] : -1;
      hm = (unsigned)j < (unsigned)nb ? hmask[j] : 0u;
    };
    load_entry(lane, lst0, hm0);
    load_entry(64 + lane, lst1, hm1);
    // (block index, head mask) of segment row rr; every lane takes part.
    auto entry = [&](int rr, int& j, uint32_t& hm) {
      const int o = (rr >> c.log2bs) - bb;
      if (whole) {  // the same entry for every lane
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
          if (MODE == ETA_LOGIT_GATED && s != T - 1)
            lv = d * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(d, gk1, gk0)));
          lg[4 * st + i] = on ? lv : -__builtin_inff();
          tmax = fmaxf(tmax, lg[4 * st + i]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      // Lazy rescaling, as in the chunked kernel.
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
    if (p < pend)  // next non-empty stream
      do ++u; while (s_start[u + 1] <= p);
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
  hipLaunchKernelGGL((screen_gqa_kernel<D>), dim3((unsigned)((long long)wpu * units)), dim3(256),
                     0, s, c, G, q, ts, z, scale, mask, words, wpu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_gqa_kernel, dim3(units), dim3(256), 0, s, c, words, wpu, mask, idx,
                     cnt, ctr);
  return hipGetLastError();
}

hipError_t launch_screen_gqa(const CacheView& c, int G, const float* q, const float* ts, float z,
                             float scale, int32_t* idx, uint32_t* mask, int32_t* cnt,
                             uint64_t* ctr, uint64_t* words, hipStream_t s) {
  return c.D == 128 ? screen_gqa_t<128>(c, G, q, ts, z, scale, idx, mask, cnt, ctr, words, s)
                    : screen_gqa_t<64>(c, G, q, ts, z, scale, idx, mask, cnt, ctr, words, s);
}

size_t gqa_decode_lds_bytes(int D, int split) {
  const size_t stage = D == 128 ? (size_t)GqaShape<128>::W * GqaShape<128>::WaveBytes
                                : (size_t)GqaShape<64>::W * GqaShape<64>::WaveBytes;
  return stage + (size_t)split * 8;
}

// Work-groups of the balanced grouped decode: as many as are resident at once
// (one wave each; registers and LDS set the count).
template <int D, int MODE>
static int gqa_flow_grid(int units) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(decode_gqa_flow_kernel<D, MODE>), 64,
          (size_t)(units + 1) * 4) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return device_cus() * min(per_cu, kMaxFlowWavesPerCU);
}

template <int D, int MODE, bool DENSE>
static hipError_t decode_gqa_t(const CacheView& c, const GqaDecode& g, hipStream_t s) {
  const GqaArgs& a = g;
  const int units = c.B * c.H;
  if constexpr (!DENSE && D == 64) {
    if (g.use_flow) {
      GqaArgs f = g;
      f.flow_grid = gqa_flow_grid<D, MODE>(units);
      hipLaunchKernelGGL((decode_gqa_flow_kernel<D, MODE>), dim3(f.flow_grid), dim3(64),
                         (size_t)(units + 1) * 4, s, c, f);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((combine_gqa_flow_kernel<D>), dim3(units * g.G), dim3(256), 0, s, c,
                         f);
      return hipGetLastError();
    }
  }
  const long long grid = (long long)g.max_chunks * c.B * c.H;
  hipLaunchKernelGGL((decode_gqa_kernel<D, MODE, DENSE>), dim3((unsigned)grid),
                     dim3(GqaShape<D>::W * 64),
                     gqa_decode_lds_bytes(D, g.split), s, c, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_gqa_kernel<D>), dim3(c.B * c.H * g.G), dim3(1024), 0, s, c, a,
                     DENSE);
  return hipGetLastError();
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
