// kernels_meta.hip -- KV append, block statistics, threshold predictor.
//
// Block statistics (paper: "Elastic Threshold Attention ...", Methodology 4):
// per complete block of b keys, the centroid mu, the per-coordinate
// population variance var (two passes) and the largest key norm maxnorm.
// mu and var are accumulated in float64 and stored as bfloat16 rounded to
// nearest even from the float64 values (half the bytes for the screen to
// read); maxnorm is float32.
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
// x rounded to the nearest bfloat16 (ties to even), as its bit pattern.
// First to float32 rounded to odd (toward zero, the last bit set when
// inexact), then float32 to bfloat16 to nearest even: float32 keeps 16 more
// bits than bfloat16, so the first rounding can neither create nor cross a
// tie of the second (round-to-odd), and the result is the direct rounding of
// x.  For finite x within the float32 range.
__device__ __forceinline__ uint16_t bf16_rne(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  if (fabs((double)f) > fabs(x)) u -= 1u;  // one step back toward zero
  if ((double)__uint_as_float(u) != x) u |= 1u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

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
  double sum[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) sum[e] = 0.0;
  float best = 0.f;  // largest squared row norm
  auto first_pass = [&](int r, const uint4& raw) {
    float n2 = 0.f;
    if (r < c.bs) {
      float x[EPL];
      widen<DT>(raw, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        sum[e] += (double)x[e];
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
  const double inv_b = 1.0 / (double)c.bs;  // exact: b is a power of two
  double mean[EPL], ss[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    mean[e] = sum[e] * inv_b;
    ss[e] = 0.0;
  }
  auto second_pass = [&](int r, const uint4& raw) {
    if (r < c.bs) {
      float x[EPL];
      widen<DT>(raw, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double dlt = (double)x[e] - mean[e];
        ss[e] = fma(dlt, dlt, ss[e]);
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
    uint32_t pm[EPL / 2], pv[EPL / 2];
#pragma unroll
    for (int e = 0; e < EPL; e += 2) {  // two bf16 per 32-bit word
      pm[e / 2] = (uint32_t)bf16_rne(mean[e]) | ((uint32_t)bf16_rne(mean[e + 1]) << 16);
      pv[e / 2] = (uint32_t)bf16_rne(ss[e] * inv_b) |
                  ((uint32_t)bf16_rne(ss[e + 1] * inv_b) << 16);
    }
    if constexpr (EPL == 8) {
      *reinterpret_cast<uint4*>(c.mu + row) = make_uint4(pm[0], pm[1], pm[2], pm[3]);
      *reinterpret_cast<uint4*>(c.var + row) = make_uint4(pv[0], pv[1], pv[2], pv[3]);
    } else {
      *reinterpret_cast<uint2*>(c.mu + row) = make_uint2(pm[0], pm[1]);
      *reinterpret_cast<uint2*>(c.var + row) = make_uint2(pv[0], pv[1]);
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

// Bulk statistics: 4 wavefronts per work-group, meta_blocks(NR) consecutive
// blocks each: 8 for blocks of at most 8 loads per lane (8 x 128K at b = 32,
// with the rows sized to them: 1.07-1.14 -> 0.99 ms), 1 for larger blocks
// (512K at b = 64: no gain, within 4% either way).  Flattened grid:
// blockIdx.x = tile * units + u.
constexpr int meta_blocks(int nr) { return nr <= 8 ? 8 : 1; }
// NR: the register rows of block_stats_wave, the smallest of 4, 8, 16 that
// holds a lane's share of a block (the arithmetic does not depend on it).
template <int D, int DT, int NR>
__global__ __launch_bounds__(256) void block_meta_kernel(CacheView c, int first, int nblk) {
  const int units = c.B * c.H;
  const int u = blockIdx.x % units, tile = blockIdx.x / units;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = c.seq_len[u / c.H];
  constexpr int MB = meta_blocks(NR);
  const int i0 = (tile * 4 + wave) * MB;
  for (int i = i0; i < min(i0 + MB, nblk); ++i) {
    const int j = first + i;
    if (j >= (T >> c.log2bs)) return;
    block_stats_wave<D, DT, NR>(c, u, j, nullptr, lane);
  }
}

// ---------------------------------------------------------------------------
// Threshold (Eq. 1) of up to kTauHeads heads of one sequence per work-group
// of kTauThreads threads, in the summation order of tau_of_head (the fused
// screen + decode computes the same bits): thread t keeps one partial sum per
// head of the residue class j = t, t + 256, ... (fmaf in increasing j, the
// loads of eight j in flight), reading the heads' entries of row j of W, which
// are contiguous (one work-group per (sequence, head) reading column h would
// touch a cache line per entry); then per head the xor
// butterfly over each wave, the four wave sums as (w0 + w1) + (w2 + w3), and
// the bias.  W == NULL (frozen thresholds) gives bias[h] alone.  VEC: W is
// 16-byte aligned and H a multiple of 4, so a lane reads its heads of a row as
// 16-byte loads (a quarter of the cache-line requests of 4-byte loads).
constexpr int kTauHeads = 8;
template <bool VEC>
__global__ __launch_bounds__(kTauThreads) void predict_kernel(int H, int D, const float* q,
                                                              const float* W, const float* bias,
                                                              float a, float* tau,
                                                              float* tau_screen) {
  __shared__ float s_red[kTauThreads / kWave][kTauHeads];
  const int chunks = ceil_div(H, kTauHeads);
  const int b = blockIdx.x / chunks, h0 = (blockIdx.x % chunks) * kTauHeads;
  const int nh = min(kTauHeads, H - h0);
  const int t = threadIdx.x, wave = t / kWave;
  if (W) {
    const int n = H * D;
    const float* qb = q + (size_t)b * n;
    float acc[kTauHeads];
#pragma unroll
    for (int e = 0; e < kTauHeads; ++e) acc[e] = 0.f;
    int j = t;
    for (; j + 7 * kTauThreads < n; j += 8 * kTauThreads) {
      float qv[8], wv[8][kTauHeads];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        qv[r] = qb[j + r * kTauThreads];
        const float* wr = W + (size_t)(j + r * kTauThreads) * H + h0;
        if constexpr (VEC) {
          // nh is a multiple of 4 here (h0 is a multiple of 8 and H of 4)
#pragma unroll
          for (int e4 = 0; e4 < kTauHeads; e4 += 4) {
            const float4 x = e4 < nh ? *reinterpret_cast<const float4*>(wr + e4)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
            wv[r][e4] = x.x;
            wv[r][e4 + 1] = x.y;
            wv[r][e4 + 2] = x.z;
            wv[r][e4 + 3] = x.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < kTauHeads; ++e) wv[r][e] = e < nh ? wr[e] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
#pragma unroll
        for (int e = 0; e < kTauHeads; ++e) acc[e] = fmaf(qv[r], wv[r][e], acc[e]);
      }
    }
    for (; j < n; j += kTauThreads) {
      const float* wr = W + (size_t)j * H + h0;
#pragma unroll
      for (int e = 0; e < kTauHeads; ++e) acc[e] = fmaf(qb[j], e < nh ? wr[e] : 0.f, acc[e]);
    }
#pragma unroll
    for (int e = 0; e < kTauHeads; ++e) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) acc[e] += __shfl_xor(acc[e], m, kWave);
    }
    if ((t & (kWave - 1)) == 0) {
#pragma unroll
      for (int e = 0; e < kTauHeads; ++e) s_red[wave][e] = acc[e];
    }
    __syncthreads();
  }
  if (t < nh) {
    const int h = h0 + t;
    const float v = W ? ((s_red[0][t] + s_red[1][t]) + (s_red[2][t] + s_red[3][t])) + bias[h]
                      : bias[h];
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

template <int D, int DT, int NR>
static hipError_t meta_nr(const CacheView& c, int first, int n, hipStream_t s) {
  const long long grid = (long long)ceil_div(n, 4 * meta_blocks(NR)) * c.B * c.H;
  hipLaunchKernelGGL((block_meta_kernel<D, DT, NR>), dim3((unsigned)grid), dim3(256), 0, s, c,
                     first, n);
  return hipGetLastError();
}

template <int D, int DT>
static hipError_t meta_t(const CacheView& c, int first, int n, hipStream_t s) {
  constexpr int RPI = kWave / (D / Elt<DT>::kPer16B);  // rows per load instruction
  const int nr = ceil_div(c.bs, RPI);                  // loads per lane per block
  if (nr <= 4) return meta_nr<D, DT, 4>(c, first, n, s);
  if (nr <= 8) return meta_nr<D, DT, 8>(c, first, n, s);
  return meta_nr<D, DT, kStatRows>(c, first, n, s);
}

hipError_t launch_block_meta(const CacheView& c, int first, int n, hipStream_t s) {
  if (c.D == 128) return c.dtype == ETA_DT_BF16 ? meta_t<128, ETA_DT_BF16>(c, first, n, s)
                                                : meta_t<128, ETA_DT_F32>(c, first, n, s);
  return c.dtype == ETA_DT_BF16 ? meta_t<64, ETA_DT_BF16>(c, first, n, s)
                                : meta_t<64, ETA_DT_F32>(c, first, n, s);
}

hipError_t launch_predict(int B, int H, int D, const float* q, const float* W, const float* bias,
                          float a, float* tau, float* tau_screen, hipStream_t s) {
  const dim3 grid(B * ceil_div(H, kTauHeads));
  if (H % 4 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0)
    hipLaunchKernelGGL(predict_kernel<true>, grid, dim3(kTauThreads), 0, s, H, D, q, W, bias, a,
                       tau, tau_screen);
  else
    hipLaunchKernelGGL(predict_kernel<false>, grid, dim3(kTauThreads), 0, s, H, D, q, W, bias, a,
                       tau, tau_screen);
  return hipGetLastError();
}

}  // namespace eta
