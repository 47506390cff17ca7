// kernels_meta.hip -- KV append, block statistics, threshold predictor.
//
// Block statistics (paper: "Elastic Threshold Attention ...", Methodology 4):
// per complete block of b keys, the centroid mu, the per-coordinate
// population variance var (two passes) and the largest key norm maxnorm.
// Threshold (Methodology 1, Eq. 1): tau = qbar W_tau + b_tau, or frozen
// per-head constants.
#include "eta_internal.h"

namespace eta {

// Statistics of block j of stream u, computed by one wavefront.
// Lane layout: a key row of D elements is read by LPR lanes with one 128-bit
// load each (bf16, D=128: 16 lanes x 8 elements), so one load instruction of
// the wave covers RPI = 64 / LPR rows.  Each lane accumulates its EPL columns
// over rows g, g+RPI, ...; the column sums of the RPI row groups are then
// combined with an xor butterfly.  Row norms are reduced inside the lane group
// with DPP.  When a lane's share of the block is at most NR loads, the rows
// stay in registers between the mean and the variance pass (K is read from
// HBM once); larger blocks re-read them.  `last_row`, when given, replaces row
// b-1 (the append path passes the key it has just written, so the block is
// complete without re-reading).  Both the append and the bulk path call this
// function with the same summation order, so they produce bit-identical
// statistics.
template <int D, int DT, int NR>
__device__ __forceinline__ void block_stats_wave(const CacheView& c, int u, int j,
                                                 const void* last_row, int lane) {
  constexpr int EPL = Elt<DT>::kPer16B;
  constexpr int LPR = D / EPL;
  constexpr int RPI = kWave / LPR;
  constexpr int RB = D * Elt<DT>::kBytes;  // bytes per key row
  const int g = lane / LPR, li = lane % LPR;
  const char* base = static_cast<const char*>(c.k) + ((size_t)u * c.cap + ((size_t)j << c.log2bs)) * RB;
  auto row_ptr = [&](int r) {
    return ((last_row && r == c.bs - 1) ? static_cast<const char*>(last_row)
                                        : base + (size_t)r * RB) + li * 16;
  };
  const int nr = (c.bs + RPI - 1) / RPI;  // loads per lane
  const bool keep = nr <= NR;             // rows fit in registers

  uint4 rows[NR];
  if (keep) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = i * RPI + g;
      rows[i] = (i < nr && r < c.bs) ? ld16_nt(row_ptr(r)) : make_uint4(0, 0, 0, 0);
    }
  }
  float sum[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) sum[e] = 0.f;
  float best = 0.f;  // largest squared row norm
  auto first_pass = [&](int r, const uint4& raw) {
    float n2 = 0.f;
    if (r < c.bs) {
      float x[EPL];
      widen<DT>(raw, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sum[e] += x[e];
        n2 = fmaf(x[e], x[e], n2);
      }
    }
    n2 = group_sum<LPR>(n2);  // every lane of the wave takes part
    best = fmaxf(best, n2);
  };
  if (keep) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (i < nr) first_pass(i * RPI + g, rows[i]);
  } else {
    for (int i = 0; i < nr; ++i) {
      const int r = i * RPI + g;
      first_pass(r, r < c.bs ? ld16(row_ptr(r)) : make_uint4(0, 0, 0, 0));
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) sum[e] += __shfl_xor(sum[e], off, kWave);
    best = fmaxf(best, __shfl_xor(best, off, kWave));
  }
  const float inv_b = 1.0f / (float)c.bs;  // exact: b is a power of two
  float mean[EPL], ss[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    mean[e] = sum[e] * inv_b;
    ss[e] = 0.f;
  }
  auto second_pass = [&](int r, const uint4& raw) {
    if (r < c.bs) {
      float x[EPL];
      widen<DT>(raw, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float dlt = x[e] - mean[e];
        ss[e] = fmaf(dlt, dlt, ss[e]);
      }
    }
  };
  if (keep) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (i < nr) second_pass(i * RPI + g, rows[i]);
  } else {
    for (int i = 0; i < nr; ++i) {
      const int r = i * RPI + g;
      if (r < c.bs) second_pass(r, ld16(row_ptr(r)));
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss[e] += __shfl_xor(ss[e], off, kWave);
  }
  if (g == 0) {
    const size_t row = ((size_t)u * c.cap_blocks + j) * D + li * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      c.mu[row + e] = mean[e];
      c.var[row + e] = ss[e] * inv_b;
    }
    if (lane == 0) c.maxnorm[(size_t)u * c.cap_blocks + j] = sqrtf(best);
  }
}

constexpr int kStatRows = 16;  // loads per lane kept in registers (64 VGPRs)

// ---------------------------------------------------------------------------
// Append: one work-group per sequence b, one wavefront per head (heads h,
// h + waves, ... when there are more heads than waves).  Every wave writes its
// head's k and v at position T_b and computes the statistics of the block the
// token completes; after a barrier one thread advances T_b, so the whole
// append is one launch.
constexpr int kAppendWaves = 8;
template <int D, int DT>
__global__ __launch_bounds__(kAppendWaves * kWave) void append_kernel(CacheView c,
                                                                      const void* k_new,
                                                                      const void* v_new,
                                                                      int32_t* overflow) {
  constexpr int RB = D * Elt<DT>::kBytes;
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int waves = blockDim.x >> 6;
  const int pos = c.seq_len[b];
  if (pos >= c.cap) {  // uniform over the work-group
    if (threadIdx.x == 0) *overflow = 1;
    return;
  }
  for (int h = wave; h < c.H; h += waves) {
    const int u = b * c.H + h;
    const char* kn = static_cast<const char*>(k_new) + (size_t)u * RB;
    const char* vn = static_cast<const char*>(v_new) + (size_t)u * RB;
    const size_t off = ((size_t)u * c.cap + pos) * RB;
    char* kd = static_cast<char*>(const_cast<void*>(c.k)) + off;
    char* vd = static_cast<char*>(const_cast<void*>(c.v)) + off;
    for (int p = lane; p < RB / 16; p += kWave) {
      *reinterpret_cast<uint4*>(kd + p * 16) = ld16(kn + p * 16);
      *reinterpret_cast<uint4*>(vd + p * 16) = ld16(vn + p * 16);
    }
    if (((pos + 1) & (c.bs - 1)) == 0)
      block_stats_wave<D, DT, kStatRows>(c, u, pos >> c.log2bs, kn, lane);
  }
  __syncthreads();  // every wave has read T_b
  if (threadIdx.x == 0) const_cast<int32_t*>(c.seq_len)[b] = pos + 1;
}

// Bulk statistics: 4 wavefronts per work-group, one block each.
// Flattened grid: blockIdx.x = tile * units + u.
template <int D, int DT>
__global__ __launch_bounds__(256) void block_meta_kernel(CacheView c, int first, int nblk) {
  const int units = c.B * c.H;
  const int u = blockIdx.x % units, tile = blockIdx.x / units;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = tile * 4 + wave;
  if (i >= nblk) return;
  const int j = first + i;
  const int T = c.seq_len[u / c.H];
  if (j >= (T >> c.log2bs)) return;
  block_stats_wave<D, DT, kStatRows>(c, u, j, nullptr, lane);
}

// ---------------------------------------------------------------------------
// Threshold (Eq. 1).  Grid (B, ceil(H / 16)), 1024 threads: work-group (b, y)
// computes heads h0 .. h0+15 (h0 = 16 y) of sequence b.  Thread t owns rows
// j = t, t+1024, ... of the H*D-long sum and keeps 16 partial sums, one per
// head; a row's 16 weights are one 64-byte run of W (four 128-bit loads when
// H is a multiple of 16), and a thread's loads of a round are issued before
// its arithmetic.  The partials are then added in a fixed order
// (deterministic): within each wave by an exchange butterfly over lane bits
// 5..2 (at each step a lane keeps half of its heads and adds its partner's
// copy of them, so 15 shuffles leave lane l with one head's sum over 16
// lanes), then over lane bits 1..0, then across the 16 waves by a 4-level
// tree in LDS.
constexpr int kPredHeads = 16;
constexpr int kPredThreads = 1024;
constexpr int kPredRows = 4;  // rows per thread per round (loads in flight)

// Keep half of the N values of x (the upper half when `upper`), adding the
// partner lane's (lane ^ M) copy of the kept half.
template <int N, int M>
__device__ __forceinline__ void fold_half(float* x, bool upper) {
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float send = upper ? x[i] : x[N / 2 + i];
    const float keep = upper ? x[N / 2 + i] : x[i];
    x[i] = keep + __shfl_xor(send, M, kWave);
  }
}

template <bool VEC>
__global__ __launch_bounds__(kPredThreads) void predict_kernel(int H, int D, const float* q,
                                                               const float* W, const float* bias,
                                                               float a, float* tau,
                                                               float* tau_screen) {
  constexpr int NW = kPredThreads / kWave;
  __shared__ float red[NW][kPredHeads];
  const int b = blockIdx.x, h0 = blockIdx.y * kPredHeads, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int hw = min(kPredHeads, H - h0);
  const int n = H * D;
  if (W) {
    float acc[kPredHeads];
#pragma unroll
    for (int e = 0; e < kPredHeads; ++e) acc[e] = 0.f;
    const float* qb = q + (size_t)b * n;
    for (int j0 = t; j0 < n; j0 += kPredThreads * kPredRows) {
      float qj[kPredRows], wv[kPredRows][kPredHeads];
#pragma unroll
      for (int r = 0; r < kPredRows; ++r) {
        const int j = j0 + kPredThreads * r;
        const bool ok = j < n;
        qj[r] = ok ? qb[j] : 0.f;
        const float* wr = W + (size_t)(ok ? j : 0) * H + h0;
        if constexpr (VEC) {
#pragma unroll
          for (int v = 0; v < kPredHeads / 4; ++v) {
            const float4 x = ok ? *reinterpret_cast<const float4*>(wr + 4 * v)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            wv[r][4 * v] = x.x; wv[r][4 * v + 1] = x.y;
            wv[r][4 * v + 2] = x.z; wv[r][4 * v + 3] = x.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < kPredHeads; ++e) wv[r][e] = (ok && e < hw) ? wr[e] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < kPredRows; ++r)
#pragma unroll
        for (int e = 0; e < kPredHeads; ++e) acc[e] = fmaf(qj[r], wv[r][e], acc[e]);
    }
    // Lane l ends with head 8 b5 + 4 b4 + 2 b3 + b2 (b_i: bit i of l).
    fold_half<16, 32>(acc, lane & 32);
    fold_half<8, 16>(acc, lane & 16);
    fold_half<4, 8>(acc, lane & 8);
    fold_half<2, 4>(acc, lane & 4);
    float x = acc[0];
    x += __shfl_xor(x, 2, kWave);
    x += __shfl_xor(x, 1, kWave);
    if ((lane & 3) == 0) {
      const int e = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 +
                    ((lane >> 2) & 1);
      red[wave][e] = x;
    }
    __syncthreads();
  }
  if (t < hw) {
    const int h = h0 + t;
    float v = bias[h];
    if (W) {
      float w8[NW / 2];
#pragma unroll
      for (int i = 0; i < NW / 2; ++i) w8[i] = red[2 * i][t] + red[2 * i + 1][t];
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) w8[i] = w8[2 * i] + w8[2 * i + 1];
#pragma unroll
      for (int i = 0; i < NW / 8; ++i) w8[i] = w8[2 * i] + w8[2 * i + 1];
      v = (w8[0] + w8[1]) + v;
    }
    tau[(size_t)b * H + h] = v;
    tau_screen[(size_t)b * H + h] = v - a;
  }
}

// ---------------------------------------------------------------------------
template <int D, int DT>
static hipError_t append_t(const CacheView& c, const void* kn, const void* vn, int32_t* of,
                           hipStream_t s) {
  const int waves = c.H < kAppendWaves ? c.H : kAppendWaves;
  hipLaunchKernelGGL((append_kernel<D, DT>), dim3(c.B), dim3(waves * kWave), 0, s, c, kn, vn, of);
  return hipGetLastError();
}

hipError_t launch_append(const CacheView& c, const void* kn, const void* vn, int32_t* of,
                         hipStream_t s) {
  if (c.D == 128) return c.dtype == ETA_DT_BF16 ? append_t<128, ETA_DT_BF16>(c, kn, vn, of, s)
                                                : append_t<128, ETA_DT_F32>(c, kn, vn, of, s);
  return c.dtype == ETA_DT_BF16 ? append_t<64, ETA_DT_BF16>(c, kn, vn, of, s)
                                : append_t<64, ETA_DT_F32>(c, kn, vn, of, s);
}

template <int D, int DT>
static hipError_t meta_t(const CacheView& c, int first, int n, hipStream_t s) {
  const long long grid = (long long)ceil_div(n, 4) * c.B * c.H;
  hipLaunchKernelGGL((block_meta_kernel<D, DT>), dim3((unsigned)grid), dim3(256), 0, s, c, first, n);
  return hipGetLastError();
}

hipError_t launch_block_meta(const CacheView& c, int first, int n, hipStream_t s) {
  if (c.D == 128) return c.dtype == ETA_DT_BF16 ? meta_t<128, ETA_DT_BF16>(c, first, n, s)
                                                : meta_t<128, ETA_DT_F32>(c, first, n, s);
  return c.dtype == ETA_DT_BF16 ? meta_t<64, ETA_DT_BF16>(c, first, n, s)
                                : meta_t<64, ETA_DT_F32>(c, first, n, s);
}

hipError_t launch_predict(int B, int H, int D, const float* q, const float* W, const float* bias,
                          float a, float* tau, float* tau_screen, hipStream_t s) {
  const dim3 grid(B, ceil_div(H, kPredHeads));
  if (H % kPredHeads == 0)
    hipLaunchKernelGGL(predict_kernel<true>, grid, dim3(kPredThreads), 0, s, H, D, q, W, bias, a,
                       tau, tau_screen);
  else
    hipLaunchKernelGGL(predict_kernel<false>, grid, dim3(kPredThreads), 0, s, H, D, q, W, bias, a,
                       tau, tau_screen);
  return hipGetLastError();
}

}  // namespace eta
