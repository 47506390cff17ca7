// kernels_screen.hip -- block screen, active-list compaction, calibration.
//
// Screen (paper: "Elastic Threshold Attention ...", Methodology 4, Eq. 5):
//   s_j = scale * min(<q, mu_j> + z sqrt(sum_i q_i^2 var_j,i), ||q|| maxnorm_j)
// A block is skipped iff s_j < threshold; only the statistics (mu and var in
// bfloat16, maxnorm in float32: 4D+4 bytes per block) are read, never the
// keys.  The block holding the newest key is always
// admitted (it holds the query's own, never-gated key of Eq. 3).
#include "eta_internal.h"

namespace eta {

// Calibration values: each wave of a work-group scores 64 consecutive blocks.
constexpr int kBlocksPerWave = 64;
constexpr int kBlocksPerTile = 4 * kBlocksPerWave;

// ---------------------------------------------------------------------------
// Screen: one work-group per 64-block admission word.  Wave w scores blocks
// 16 w .. 16 w + 15 of the word in two steps of 8 blocks whose statistics
// loads are all issued before any reduction, so a wave has its whole share in
// flight at once; the four 16-bit wave masks are merged in LDS and one 64-bit
// word is written.  Flattened grid: blockIdx.x = word * units + u, so the low
// words of every stream are dispatched first and the surplus words of short
// streams exit at once.
constexpr int kScreenSteps = 2;  // steps of 8 blocks per wave
static_assert(4 * kScreenSteps * kBlocksPerIter == 64, "one word per work-group");
template <int D>
__global__ __launch_bounds__(256) void screen_kernel(CacheView c, const float* q,
                                                     const float* tau_screen, float z, float scale,
                                                     uint64_t* words, int words_per_unit) {
  constexpr int NL = QShare<D>::kLoads;
  __shared__ uint32_t s_bits[4];
  const int units = c.B * c.H;
  const int u = blockIdx.x % units, wd = blockIdx.x / units;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = c.seq_len[u / c.H];
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int nbc = T >> c.log2bs;
  if ((wd << 6) >= nb) return;  // uniform over the work-group
  const int gi = lane / kLanesPerBlock, li = lane % kLanesPerBlock;
  QShare<D> qs;
  load_qshare<D>(q + (size_t)u * D, li, qs);
  const float ts = tau_screen[u];
  const bool z_inf = __builtin_isinf(z);
  const int jw = (wd << 6) + wave * (kScreenSteps * kBlocksPerIter) + gi;
  uint4 m4[kScreenSteps][NL], v4[kScreenSteps][NL];
  float M[kScreenSteps];
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int it = 0; it < kScreenSteps; ++it) {
    const int j = jw + it * kBlocksPerIter;
    const size_t row = ((size_t)u * c.cap_blocks + j) * D;
    const bool scored = j < nbc;
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      m4[it][t] = scored ? ld16_nt(c.mu + row + 64 * t + 8 * li) : zero4;
      v4[it][t] = scored ? ld16_nt(c.var + row + 64 * t + 8 * li) : zero4;
    }
    M[it] = scored ? c.maxnorm[(size_t)u * c.cap_blocks + j] : 0.f;
  }
  uint32_t bits = 0;
#pragma unroll
  for (int it = 0; it < kScreenSteps; ++it) {
    const int j = jw + it * kBlocksPerIter;
    float dot = 0.f, mom = 0.f;
    score_partials<D>(qs, m4[it], v4[it], dot, mom);
    dot = group_sum<kLanesPerBlock>(dot);
    mom = group_sum<kLanesPerBlock>(mom);
    const float geometric = qs.qn * M[it];
    const float sc = z_inf ? scale * geometric
                           : scale * fminf(fmaf(z, sqrtf(mom), dot), geometric);
    const bool on = (j == nb - 1) || (j < nbc && sc >= ts);
    const uint64_t bal = __ballot(on);
#pragma unroll
    for (int g = 0; g < kBlocksPerIter; ++g)
      bits |= (uint32_t)((bal >> (g * kLanesPerBlock)) & 1ull) << (it * kBlocksPerIter + g);
  }
  if (lane == 0) s_bits[wave] = bits;
  __syncthreads();
  if (threadIdx.x == 0) {
    constexpr int WB = kScreenSteps * kBlocksPerIter;  // 16 bits per wave
    const uint64_t word = (uint64_t)s_bits[0] | ((uint64_t)s_bits[1] << WB) |
                          ((uint64_t)s_bits[2] << (2 * WB)) | ((uint64_t)s_bits[3] << (3 * WB));
    words[(size_t)u * words_per_unit + wd] = word;
  }
}

// Compaction: one work-group per stream turns the admission words into the
// ascending index list.  Each thread owns a contiguous run of blocks, so an
// exclusive scan of per-thread popcounts gives every thread its output offset
// and the list comes out ascending with no sorting.
__global__ __launch_bounds__(256) void compact_kernel(CacheView c, const uint64_t* words,
                                                      int words_per_unit, int32_t* active_idx,
                                                      int32_t* active_cnt, uint64_t* ctr) {
  __shared__ int s_w[4];
  const int u = blockIdx.x, t = threadIdx.x;
  const int T = c.seq_len[u / c.H];
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const uint64_t* wu = words + (size_t)u * words_per_unit;
  int32_t* out = active_idx + (size_t)u * c.cap_blocks;
  // Thread t takes a run of bpt consecutive blocks (bpt a power of two <= 64,
  // so a run lies in one word); rounds of 256 runs in ascending order.
  int bpt = 1;
  while (bpt < 64 && bpt * 256 < nb) bpt <<= 1;
  int base_pos = 0;
  for (int r0 = 0; r0 < nb; r0 += 256 * bpt) {
    const int b0 = r0 + t * bpt;
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
  if (t == 0) {
    const int total = base_pos;
    active_cnt[u] = total;
    if (ctr && total > 0) {
      const unsigned long long tokens =
          (unsigned long long)(total - 1) * c.bs + (unsigned long long)(T - ((nb - 1) << c.log2bs));
      atomicAdd(reinterpret_cast<unsigned long long*>(ctr), tokens);
    }
  }
}

// ---------------------------------------------------------------------------
// Calibration, step 1: pooled values x = s_j - tau0 for every complete block
// except the last one of its stream; other slots get NaN.  Layout
// values[h][n][b][cap_blocks].  Grid: blockIdx.x = tile * (n_sets*units) + su.
template <int D>
__global__ __launch_bounds__(256) void calib_values_kernel(CacheView c, int n_sets,
                                                           const float* q_sets, const float* tau0,
                                                           float z, float scale, float* values) {
  const int units = c.B * c.H;
  const int su = blockIdx.x % (n_sets * units), tile = blockIdx.x / (n_sets * units);
  const int n = su / units, u = su % units;
  const int b = u / c.H, h = u % c.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j0 = (tile * 4 + wave) * kBlocksPerWave;
  if (j0 >= c.cap_blocks) return;
  const int T = c.seq_len[b];
  const int nb = (T + c.bs - 1) >> c.log2bs;
  const int gi = lane / kLanesPerBlock, li = lane % kLanesPerBlock;
  QShare<D> qs;
  load_qshare<D>(q_sets + (size_t)su * D, li, qs);
  const float t0 = tau0 ? tau0[su] : 0.f;
  const bool z_inf = __builtin_isinf(z);
  float* dst = values + (((size_t)h * n_sets + n) * c.B + b) * c.cap_blocks;
  for (int it = 0; it < kBlocksPerWave / kBlocksPerIter; ++it) {
    const int j = j0 + it * kBlocksPerIter + gi;
    const bool cand = j < nb - 1;  // every block before the last is complete
    const float sc = block_score<D>(c, u, j, cand, qs, li, z, z_inf, scale);
    if (li == 0 && j < c.cap_blocks) dst[j] = cand ? sc - t0 : __builtin_nanf("");
  }
}

// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float funkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// k-th largest (1-based) non-NaN key among x[0..n) by 4 passes of an 8-bit
// MSB-first radix select; all threads of the work-group call it.
__device__ uint32_t radix_select_desc(const float* x, long long n, long long k, uint32_t* hist,
                                      uint32_t* sh) {
  uint32_t prefix = 0, mask = 0;
  long long remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (long long i = threadIdx.x; i < n; i += blockDim.x) {
      const float f = x[i];
      if (f != f) continue;
      const uint32_t key = fkey(f);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int dg = 255;
      for (; dg > 0; --dg) {
        if (remaining <= (long long)hist[dg]) break;
        remaining -= hist[dg];
      }
      sh[0] = (uint32_t)dg;
      sh[1] = (uint32_t)remaining;
    }
    __syncthreads();
    prefix |= sh[0] << shift;
    mask |= 255u << shift;
    remaining = sh[1];
    __syncthreads();
  }
  return prefix;
}

// Calibration, step 2: one work-group per head.
__global__ __launch_bounds__(1024) void calib_select_kernel(CacheView c, int n_sets, float rho,
                                                            const float* values, float* c_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  const int h = blockIdx.x;
  long long N = 0, total = 0, forced = 0;
  for (int b = 0; b < c.B; ++b) {
    const int T = c.seq_len[b];
    if (T <= 0) continue;
    const int nb = (T + c.bs - 1) >> c.log2bs;
    N += (long long)n_sets * (nb - 1);
    total += (long long)n_sets * T;
    forced += (long long)n_sets * (T - ((nb - 1) << c.log2bs));
  }
  const double want = ((double)rho * (double)total - (double)forced) / (double)c.bs;
  long long k = (long long)floor(want + 0.5);
  if (k < 0) k = 0;
  if (k > N) k = N;
  const float* x = values + (size_t)h * n_sets * c.B * c.cap_blocks;
  const long long n = (long long)n_sets * c.B * c.cap_blocks;
  float res;
  if (k == N) {
    res = -__builtin_inff();
  } else if (k == 0) {
    res = __builtin_inff();
  } else {
    const float hi = funkey(radix_select_desc(x, n, k, hist, sh));
    const float lo = funkey(radix_select_desc(x, n, k + 1, hist, sh));
    res = 0.5f * (hi + lo);
  }
  if (threadIdx.x == 0) c_out[h] = res;
}

// ---------------------------------------------------------------------------
template <int D>
static hipError_t screen_t(const CacheView& c, const float* q, const float* ts, float z, float scale,
                           int32_t* idx, int32_t* cnt, uint64_t* ctr, uint64_t* words,
                           hipStream_t s) {
  const int units = c.B * c.H;
  const int wpu = ceil_div(c.cap_blocks, 64);
  const long long grid = (long long)wpu * units;
  hipLaunchKernelGGL((screen_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, c, q, ts, z, scale,
                     words, wpu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, dim3(units), dim3(256), 0, s, c, words, wpu, idx, cnt, ctr);
  return hipGetLastError();
}

hipError_t launch_screen(const CacheView& c, const float* q, const float* ts, float z, float scale,
                         int32_t* idx, int32_t* cnt, uint64_t* ctr, uint64_t* words,
                         hipStream_t s) {
  return c.D == 128 ? screen_t<128>(c, q, ts, z, scale, idx, cnt, ctr, words, s)
                    : screen_t<64>(c, q, ts, z, scale, idx, cnt, ctr, words, s);
}

template <int D>
static hipError_t calib_t(const CacheView& c, int n_sets, const float* q_sets, const float* tau0,
                          float z, float scale, float rho, float* values, float* c_out,
                          hipStream_t s) {
  const long long grid = (long long)ceil_div(c.cap_blocks, kBlocksPerTile) * n_sets * c.B * c.H;
  hipLaunchKernelGGL((calib_values_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, c, n_sets,
                     q_sets, tau0, z, scale, values);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(calib_select_kernel, dim3(c.H), dim3(1024), 0, s, c, n_sets, rho, values,
                     c_out);
  return hipGetLastError();
}

hipError_t launch_calibrate(const CacheView& c, int n_sets, const float* q_sets, const float* tau0,
                            float z, float scale, float rho, float* values, float* c_out,
                            hipStream_t s) {
  return c.D == 128 ? calib_t<128>(c, n_sets, q_sets, tau0, z, scale, rho, values, c_out, s)
                    : calib_t<64>(c, n_sets, q_sets, tau0, z, scale, rho, values, c_out, s);
}

}  // namespace eta
