// kernels_prefill.hip -- gated causal attention forward over whole sequences.
//
// Paper: "Elastic Threshold Attention ..." (summary page, Methodology 2,
// Eqs. 2-3: the model's own attention, with every off-diagonal score
// multiplied by its soft inclusion gate sigmoid(beta (S - tau_t)) before a
// causal softmax; Methodology 3, Eq. 4: the per-row mean of the gates, whose
// average over heads and positions is the layer's sparsity term).  This is
// the forward pass of prefill and training; decode (one query against a
// cache) is the block-sparse path of the other kernels.
//
// One work-group of 8 waves (d 64) or 4 waves (d 128) takes the query heads
// of one KV head that share its K and V: with hw of them per work-group
// (8 at the pages' group of 8), wave w serves head w % hw at queries
// t0 + 16 (w / hw) .. + 15.  The keys 0 .. t0 + rows - 1 are walked in 32-key
// tiles.  A tile is loaded once for all waves (coalesced 128-bit reads by 256
// threads, the next tile's loads in flight while the current one is
// computed) and staged in LDS as rows (chunk-swizzled), double buffered, one
// barrier per tile; the value product reads V with the transposing LDS read.
// Each wave then computes, on the matrix cores, S^T = K_tile Q_w^T (queries
// as the 16 columns; q is bf16 as given)
// and O += P V with the weights split hi + lo, applying the causal mask, the
// gate and an online softmax per query column in between.
#include "eta_internal.h"

namespace eta {


template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};
template <int I>
struct BufTag {
  static constexpr int value = I;
};

// HPW query heads per wave (2 at d 64 when the group is even: the wave reads
// each staged K/V tile from LDS once for both), 16 query positions each.
template <int D, int HPW>
struct PrefillShape {
  static constexpr int NK = D / 32;                  // 32-dim slabs of the score product
  static constexpr int NV = D / 16;                  // 16-dim slabs of the value product
  static constexpr int RB = D * 2;                   // bytes per bf16 row
  static constexpr int LPR = D / 8;                  // threads per row in a coalesced load
  // (head, 16-query subtile) slots per work-group: 8 at d 64, so each staged
  // K/V tile serves 8 of them; 4 at d 128, whose registers leave room for
  // fewer waves.
  static constexpr int Slots = D == 64 ? 8 : 4;
  static constexpr int NW = Slots / HPW;            // waves per work-group
  static constexpr int Threads = NW * 64;
  static constexpr int KP = kTileKeys * LPR / 256;   // K (and V) loads per loading thread per tile
  static constexpr int KBytes = kTileKeys * RB;
  static constexpr int VBytes = kTileKeys * RB;
  static constexpr int StageBytes = KBytes + VBytes;
  static_assert(KP >= 1, "tile loads");
  static_assert(Threads >= 256, "the first 256 threads load each tile");
};

// Query heads per work-group: the largest power of two up to the slot count
// that divides the group, so that the slots of a work-group are hw query
// heads of one KV head (all reading the same K and V) times slots / hw
// consecutive 16-query subtiles.  Slot s is head s % hw, subtile s / hw.
__host__ __device__ inline int prefill_heads(int slots, int group) {
  int h = slots;
  while (h > 1 && group % h != 0) h >>= 1;
  return h;
}

template <int D, int HPW>
__global__ __launch_bounds__((PrefillShape<D, HPW>::Threads)) void prefill_kernel(PrefillArgs a) {
  using Sh = PrefillShape<D, HPW>;
  constexpr int NK = Sh::NK, NV = Sh::NV, RB = Sh::RB, LPR = Sh::LPR, KP = Sh::KP;
  __shared__ __align__(16) char s_stage[2][Sh::StageBytes];

  const int T = a.T, G = a.G;
  const int hw = prefill_heads(Sh::Slots, G), hblocks = G / hw;
  const int rows = 16 * (Sh::Slots / hw);  // query positions per work-group
  const int units = a.B * a.Hkv * hblocks;
  const int ntq = ceil_div(T, rows);
  const int tq = ntq - 1 - (int)(blockIdx.x / units);  // longest query tiles first
  const int ug = blockIdx.x % units;
  const int b = ug / (a.Hkv * hblocks), kvh = (ug / hblocks) % a.Hkv, hb = ug % hblocks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
  // The wave's slots HPW w .. HPW w + HPW - 1: consecutive heads (hw is a
  // multiple of HPW), one subtile.
  const int slot = HPW * wave;
  const int uq0 = (b * a.Hkv + kvh) * G + hb * hw + slot % hw;  // the wave's first query head
  const int t0 = tq * rows;
  const int n = lane & 15, grp = lane >> 4;
  const int tw = t0 + 16 * (slot / hw);  // the wave's first query
  const int tn = tw + n;                 // this lane's query column
  const char* kbase = static_cast<const char*>(a.k) + ((size_t)b * a.Hkv + kvh) * T * RB;
  const char* vbase = static_cast<const char*>(a.v) + ((size_t)b * a.Hkv + kvh) * T * RB;

  // Query operands: column n = query tn, dims 32 kk + 8 grp .. +7 (rows past
  // the sequence read the last row and are never written).
  // Gate of Eq. 2: sigmoid(beta (scale r - tau)) = 1 / (1 + 2^(r gk1 + gk0)).
  // Scores stay unscaled (raw dot products r) through the softmax: the logit is
  // scale * r * gate, so scale is folded into the exponent constants and the
  // lazy-rescale step (scale > 0 keeps every max and comparison).
  bf16x8 qb[HPW][NK];
  float gk0[HPW];
  const float gk1 = -a.beta * kLog2e * a.scale;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const size_t pos = (size_t)(uq0 + hh) * T + min(tn, T - 1);
    const char* qrow = static_cast<const char*>(a.q) + pos * RB + 16 * grp;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) qb[hh][kk] = __builtin_bit_cast(bf16x8, ld16(qrow + 64 * kk));
    gk0[hh] = a.beta * kLog2e * a.tau[pos];
  }
  const float sl2 = a.scale * kLog2e;
  const float lazy_raw = kLazyRaise / a.scale;

  const int kend = min(T, t0 + rows);  // keys this work-group needs
  const int ntiles = ceil_div(kend, kTileKeys);

  // Cooperative tile loads: K and V as (key, 16-byte chunk) pairs, D/8
  // threads per row, by the first 256 threads.  Keys past the sequence read
  // its last row (finite data; causally masked).  Both are staged as rows;
  // V's value-product operand is taken with the transposing LDS read, so no
  // thread repacks V.
  uint4 kr[KP], vr[KP];
  auto fetch = [&](int j) {
    if (Sh::Threads > 256 && tid >= 256) return;
    const int s0 = j * kTileKeys;
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int e = tid + 256 * p;
      const uint32_t off = (uint32_t)min(s0 + e / LPR, T - 1) * RB + 16 * (e % LPR);
      kr[p] = ld16(kbase + off);
      vr[p] = ld16(vbase + off);
    }
  };
  auto stage = [&](auto buf_tag) {
    if (Sh::Threads > 256 && tid >= 256) return;
    char* sk = s_stage[decltype(buf_tag)::value];
    char* sv = sk + Sh::KBytes;
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      const int e = tid + 256 * p;
      const int key = e / LPR;
      const int row = tile_row<D>(key) * RB;
      *reinterpret_cast<uint4*>(sk + row + 16 * ((e % LPR) ^ tile_kswz<D>(key))) = kr[p];
      *reinterpret_cast<uint4*>(sv + row + 16 * ((e % LPR) ^ vrow_swz(key))) = vr[p];
    }
  };

  // O accumulates P V; L accumulates P 1 (every column of the ones operand),
  // so the softmax denominators of rows 4 grp + i come out of the matrix
  // cores in O's own layout, summed from the same hi + lo weights.
  floatx4 O[HPW][NV], L[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    L[hh] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) O[hh][nv] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                             0x3F803F80u));
  // m: reference max (raw score units) of the lane's query column; ms2 its
  // exponent offset m * scale * log2(e), 0 while the column is empty.
  float m[HPW], ms2[HPW], gsum[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m[hh] = -__builtin_inff();
    ms2[hh] = 0.f;
    gsum[hh] = 0.f;
  }

  // MASK: the tile holds the diagonal or keys past some query (or the wave has
  // queries past the sequence); otherwise every key precedes every query.
  auto compute = [&](int j, auto buf_tag, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int s0 = j * kTileKeys;
    const char* sk = s_stage[decltype(buf_tag)::value];
    const char* sv = sk + Sh::KBytes;
    // Each K operand read serves every head of the wave.
    floatx4 S[HPW][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key = tile_key(st, n);
      const char* row = sk + tile_row<D>(key) * RB;
      const int sw = tile_kswz<D>(key);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) S[hh][st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 kv =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + 16 * ((4 * kk + grp) ^ sw)));
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          S[hh][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[hh][kk], S[hh][st], 0, 0, 0);
      }
    }
    bf16x8 phi[HPW], plo[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      // Score i of half st is key s0 + 2 grp + st + 8 i against query tn.
      float lg[8];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = S[hh][st][i];
          const float g = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(fmaf(d, gk1, gk0[hh])));
          if constexpr (MASK) {
            const int s = s0 + 2 * grp + st + 8 * i;
            const bool on = s <= tn && tn < T;
            gsum[hh] += on ? g : 0.f;
            const float lv = s == tn ? d : d * g;
            lg[4 * st + i] = on ? lv : -__builtin_inff();
          } else {
            gsum[hh] += g;
            lg[4 * st + i] = d * g;
          }
          tmax = fmaxf(tmax, lg[4 * st + i]);
        }
      }
      // Lazy rescaling as in the grouped decode: the reference max of a query
      // moves only when the tile raises it by more than kLazyRaise.  m is the
      // same in the 4 lane groups of a column, so some lane's own max passes
      // m + lazy_raw exactly when some column's max does; the column maxima
      // are formed only then.
      if (__ballot(tmax > m[hh] + lazy_raw) != 0ull) {
        tmax = max_xor32(max_xor16(tmax));
        const float mn = fmaxf(m[hh], tmax);
        const float alpha =
            mn == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f((m[hh] - mn) * sl2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * grp + i, kWave);
          L[hh][i] *= al;
#pragma unroll
          for (int nv = 0; nv < NV; ++nv) O[hh][nv][i] *= al;
        }
        m[hh] = mn;
        ms2[hh] = m[hh] == -__builtin_inff() ? 0.f : m[hh] * sl2;
      }
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        split_hi_lo(__builtin_amdgcn_exp2f(fmaf(lg[2 * i], sl2, -ms2[hh])),
                    __builtin_amdgcn_exp2f(fmaf(lg[2 * i + 1], sl2, -ms2[hh])), ph[i], pl[i]);
      phi[hh] = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
      plo[hh] = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
      L[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[hh], ones, L[hh], 0, 0, 0);
      L[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[hh], ones, L[hh], 0, 0, 0);
    }
    // Value operand (dim 16 nv + n, slots 8 grp + 4 h + j) by two transposing
    // reads, each serving every head of the wave: lane L of group g supplies
    // row tile_key(h, 4 g + (L%16)/4), dims 16 nv + 4 ((L%16) % 4) .. +3, and
    // lane l receives element l % 4 of the rows supplied by lanes
    // 16 g + 4 j + (l%16)/4, j = 0..3.
    const int trow0 = tile_key(0, 4 * grp + ((lane & 15) >> 2));
    const int trow1 = tile_key(1, 4 * grp + ((lane & 15) >> 2));
    const int tr4 = lane & 3;
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      const int c = 2 * nv + (tr4 >> 1);
      const uint2 v0 =
          tr_read(sv + tile_row<D>(trow0) * RB + 16 * (c ^ vrow_swz(trow0)) + 8 * (tr4 & 1));
      const uint2 v1 =
          tr_read(sv + tile_row<D>(trow1) * RB + 16 * (c ^ vrow_swz(trow1)) + 8 * (tr4 & 1));
      const bf16x8 vb = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        O[hh][nv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi[hh], vb, O[hh][nv], 0, 0, 0);
        O[hh][nv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo[hh], vb, O[hh][nv], 0, 0, 0);
      }
    }
  };

  // Tile j sits in buffer j & 1; the loop is unrolled by two so that the
  // buffer, and with it every LDS address, is a per-lane constant plus an
  // immediate offset.
  auto step = [&](int j, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    const bool more = j + 1 < ntiles;
    if (more) fetch(j + 1);
    // keys of tile j all after this wave's queries (or no query left): skip
    if (j * kTileKeys <= tw + 15 && tw < T) {
      if (j * kTileKeys + kTileKeys - 1 < tw && tw + 15 < T)
        compute(j, buf_tag, MaskTag<false>{});
      else
        compute(j, buf_tag, MaskTag<true>{});
    }
    if (more) stage(BufTag<BUF ^ 1>{});
    __syncthreads();
  };
  fetch(0);
  stage(BufTag<0>{});
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    step(j, BufTag<0>{});
    if (j + 1 < ntiles) step(j + 1, BufTag<1>{});
  }

#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int uq = uq0 + hh;
    // Gate sums of a query column over its 4 lane groups.
    const float gs = sum_xor32(sum_xor16(gsum[hh]));
    // O and L rows are queries tw + 4 grp + i.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = L[hh][i];
      const int t = tw + 4 * grp + i;
      if (t < T) {
        float* orow = a.out + ((size_t)uq * T + t) * D;
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) orow[16 * nv + n] = O[hh][nv][i] / li;
      }
    }
    if (a.dens && grp == 0 && tn < T) a.dens[(size_t)uq * T + tn] = gs / (float)(tn + 1);
  }
}

template <int D, int HPW>
static hipError_t prefill_t(const PrefillArgs& a, hipStream_t s) {
  using Sh = PrefillShape<D, HPW>;
  const int hw = prefill_heads(Sh::Slots, a.G);
  const long long grid =
      (long long)ceil_div(a.T, 16 * (Sh::Slots / hw)) * a.B * a.Hkv * (a.G / hw);
  hipLaunchKernelGGL((prefill_kernel<D, HPW>), dim3((unsigned)grid), dim3(Sh::Threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.D == 128) return prefill_t<128, 1>(a, s);
  return a.G % 2 == 0 ? prefill_t<64, 2>(a, s) : prefill_t<64, 1>(a, s);
}

}  // namespace eta
