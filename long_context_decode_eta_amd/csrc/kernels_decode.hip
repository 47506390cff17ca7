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
// Work decomposition: the admitted list of stream u is cut into chunks of
// `split` blocks; one work-group of 4 waves handles one chunk.  The chunk's
// rows are cut into tiles of kRows rows; wave w takes tiles w, w+4, ...  A key
// row of D elements is read by LPR lanes with one 128-bit load each (bf16,
// D=128: 16 lanes), so one load instruction of a wave covers RPI = 64/LPR rows
// and a tile is NI = kRows/RPI loads of K plus NI loads of V per lane, all
// issued before any arithmetic.  Each lane group keeps its own running (max,
// sum, weighted V) over its rows; groups, then waves, are merged at the end.
#include "eta_internal.h"

namespace eta {

constexpr int kRows = 32;  // rows per wave tile

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

template <int D, int DT, int MODE, bool DENSE>
__global__ __launch_bounds__(256) void decode_kernel(CacheView c, DecodeArgs a) {
  constexpr int EPL = Elt<DT>::kPer16B;
  constexpr int LPR = D / EPL;
  constexpr int RPI = kWave / LPR;
  constexpr int NI = (kRows / RPI) > 0 ? (kRows / RPI) : 1;
  constexpr int RB = D * Elt<DT>::kBytes;
  __shared__ float s_acc[4][D];
  __shared__ float s_ml[4][2];

  const int units = c.B * c.H;
  const int u = blockIdx.x % units, k = blockIdx.x / units;
  const int T = c.seq_len[u / c.H];
  if (T <= 0) return;
  const int nb = (T + c.bs - 1) >> c.log2bs;
  // The list is trusted only as far as it stays inside the stream.
  const int cnt = DENSE ? nb : min(a.active_cnt[u], nb);
  const int first = k * a.split;
  if (first >= cnt) return;
  const int nblk = min(a.split, cnt - first);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane / LPR, li = lane % LPR;

  float qs[EPL];
  {
    const float* qu = a.q + (size_t)u * D + li * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qs[e] = qu[e] * a.scale;
  }
  const float tau = (MODE == ETA_LOGIT_GATED) ? a.tau[u] : 0.f;
  const float beta = a.beta;
  const int32_t* list = DENSE ? nullptr : a.active_idx + (size_t)u * c.cap_blocks + first;
  const char* kb = static_cast<const char*>(c.k) + (size_t)u * c.cap * RB + li * 16;
  const char* vb = static_cast<const char*>(c.v) + (size_t)u * c.cap * RB + li * 16;

  float m = -__builtin_inff(), l = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

  const int rows = nblk << c.log2bs;
  const int ntiles = (rows + NI * RPI - 1) / (NI * RPI);
  for (int t = wave; t < ntiles; t += 4) {
    uint4 kr[NI], vr[NI];
    int sp[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int rr = (t * NI + i) * RPI + g;  // row within the chunk
      int s = -1;
      if (rr < rows) {
        const int p = rr >> c.log2bs;
        const int j = DENSE ? first + p : list[p];
        s = (j << c.log2bs) + (rr & (c.bs - 1));
        if ((unsigned)j >= (unsigned)nb || s >= T) s = -1;
      }
      sp[i] = s;
      if (s >= 0) {
        kr[i] = ld16(kb + (size_t)s * RB);
        vr[i] = ld16(vb + (size_t)s * RB);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
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
    const float mn = fmaxf(m, tmax);
    const float ms = (mn == -__builtin_inff()) ? 0.f : mn;
    const float alpha = fexp(m - ms);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float p = fexp(lg[i] - ms);
      l += p;
      float y[EPL];
      widen<DT>(vr[i], y);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, y[e], acc[e]);
    }
    m = mn;
  }

  // Merge the RPI row groups of the wave (xor butterfly: partners end equal).
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float l2 = __shfl_xor(l, off, kWave);
    float a2[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) a2[e] = __shfl_xor(acc[e], off, kWave);
    merge_state<EPL>(m, l, acc, m2, l2, a2);
  }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wave][li * EPL + e] = acc[e];
    if (li == 0) {
      s_ml[wave][0] = m;
      s_ml[wave][1] = l;
    }
  }
  __syncthreads();
  // Merge the 4 waves in a fixed order; thread i < D owns output column i.
  const int i = threadIdx.x;
  if (i < D) {
    float mm = s_ml[0][0], ll = s_ml[0][1], aa[1] = {s_acc[0][i]};
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float a2[1] = {s_acc[w][i]};
      merge_state<1>(mm, ll, aa, s_ml[w][0], s_ml[w][1], a2);
    }
    if (first == 0 && nblk == cnt) {
      a.out[(size_t)u * D + i] = aa[0] / ll;  // single chunk: final output
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

// Log-sum-exp combine of the chunk partials of one stream; also writes the
// zero output of empty streams.  Thread t owns column t % D and the chunks
// t / D, t / D + G, ... (G = 256 / D); the G partial sums are added in a fixed
// order.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CacheView c, DecodeArgs a) {
  __shared__ float s_red[256];
  __shared__ float s_a[256 / D][D];
  __shared__ float s_l[256 / D];
  constexpr int G = 256 / D;
  const int u = blockIdx.x, t = threadIdx.x;
  const int T = c.seq_len[u / c.H];
  if (T <= 0) {
    if (t < D) a.out[(size_t)u * D + t] = 0.f;
    return;
  }
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int cnt = a.dense ? nb : min(a.active_cnt[u], nb);
  if (cnt <= 0) {  // not a list eta_screen produces (it always holds the last block)
    if (t < D) a.out[(size_t)u * D + t] = 0.f;
    return;
  }
  const int nch = (cnt + a.split - 1) / a.split;
  if (nch <= 1) return;  // written by the decode kernel
  const float* pm = a.part_m + (size_t)u * a.max_chunks;
  const float* pl = a.part_l + (size_t)u * a.max_chunks;
  const float* pa = a.part_acc + (size_t)u * a.max_chunks * D;
  float mx = -__builtin_inff();
  for (int ch = t; ch < nch; ch += 256) mx = fmaxf(mx, pm[ch]);
  s_red[t] = mx;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (t < off) s_red[t] = fmaxf(s_red[t], s_red[t + off]);
    __syncthreads();
  }
  const float M = s_red[0];
  const int col = t % D, grp = t / D;
  float A = 0.f, L = 0.f;
  for (int ch = grp; ch < nch; ch += G) {
    const float w = fexp(pm[ch] - M);
    A = fmaf(w, pa[(size_t)ch * D + col], A);
    L = fmaf(w, pl[ch], L);
  }
  s_a[grp][col] = A;
  if (col == 0) s_l[grp] = L;
  __syncthreads();
  if (t < D) {
    float At = 0.f, Lt = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) {
      At += s_a[g2][t];
      Lt += s_l[g2];
    }
    a.out[(size_t)u * D + t] = At / Lt;
  }
}

// ---------------------------------------------------------------------------
template <int D, int DT, int MODE, bool DENSE>
static hipError_t decode_t(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  const long long grid = (long long)a.max_chunks * c.B * c.H;
  hipLaunchKernelGGL((decode_kernel<D, DT, MODE, DENSE>), dim3((unsigned)grid), dim3(256), 0, s, c,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((combine_kernel<D>), dim3(c.B * c.H), dim3(256), 0, s, c, a);
  return hipGetLastError();
}

template <int D, int DT>
static hipError_t decode_dt(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  if (a.dense) return decode_t<D, DT, ETA_LOGIT_RAW, true>(c, a, s);
  if (a.mode == ETA_LOGIT_RAW) return decode_t<D, DT, ETA_LOGIT_RAW, false>(c, a, s);
  return decode_t<D, DT, ETA_LOGIT_GATED, false>(c, a, s);
}

hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t s) {
  if (c.D == 128) return c.dtype == ETA_DT_BF16 ? decode_dt<128, ETA_DT_BF16>(c, a, s)
                                                : decode_dt<128, ETA_DT_F32>(c, a, s);
  return c.dtype == ETA_DT_BF16 ? decode_dt<64, ETA_DT_BF16>(c, a, s)
                                : decode_dt<64, ETA_DT_F32>(c, a, s);
}

}  // namespace eta
