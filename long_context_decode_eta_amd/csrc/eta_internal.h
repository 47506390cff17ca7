// eta_internal.h -- shared device helpers and launcher declarations of libeta.
//
// Target: gfx950 (CDNA4), wave64.  Everything here is memory-bound GEMV-shaped
// work, so the helpers are about 128-bit loads, lane-group reductions done
// with DPP row permutations (no LDS round trip) and exact bf16 widening.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/eta.h"

namespace eta {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element access.  A bfloat16 is the upper half of an IEEE binary32, so the
// widening below is exact.
template <int DT>
struct Elt;
template <>
struct Elt<ETA_DT_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPer16B = 4;  // elements per 128-bit load
};
template <>
struct Elt<ETA_DT_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Widen one 128-bit load into kPer16B floats.
template <int DT>
__device__ __forceinline__ void widen(const uint4& r, float* x) {
  if constexpr (DT == ETA_DT_F32) {
    x[0] = __uint_as_float(r.x);
    x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z);
    x[3] = __uint_as_float(r.w);
  } else {
    x[0] = bf16lo(r.x); x[1] = bf16hi(r.x);
    x[2] = bf16lo(r.y); x[3] = bf16hi(r.y);
    x[4] = bf16lo(r.z); x[5] = bf16hi(r.z);
    x[6] = bf16lo(r.w); x[7] = bf16hi(r.w);
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 128-bit load with the nontemporal hint: data read once per step
// (K/V rows, block statistics) should not displace reusable lines in L2/MALL.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld16f_nt(const float* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// ---------------------------------------------------------------------------
// Lane-group all-reductions.  Groups are aligned runs of N lanes.  The DPP
// patterns used (quad xor-1, quad xor-2, half-row mirror, row mirror) pair
// every lane with a partner whose partial sum covers the complementary set,
// and a + b == b + a exactly, so every lane of a group ends with the
// bit-identical result.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;  // lane i <-> 15-i within a row of 16
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within each half row

// Split two non-negative floats into bf16 hi + lo pairs (hi rounded to
// nearest, lo the rounded remainder): hi + lo carries 16 significant bits,
// so a product with bf16 operands summed in float32 keeps float32-level
// accuracy.  One packed conversion per pair; the hi halves widen back by a
// shift and a mask.  Element 0 sits in the low 16 bits of each result.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2x __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_hi_lo(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2x){a, b}, bf16x2));
  const float2x rest = {a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2));
}

// Chunk k of stream u in a flat grid of max_chunks work-groups per stream.
// Work-groups are dealt to the 8 XCDs round-robin by blockIdx, so with the
// plain order u * max_chunks + k and max_chunks a multiple of 8, chunk k of
// every stream lands on XCD k % 8 and the XCDs holding the low chunk numbers
// carry the streams' remainders (a stream with 13 chunks puts 2 on XCDs 0-4
// and 1 on XCDs 5-7).  Rotating each stream's chunks by u % 8 spreads the
// remainders over all XCDs; a stream's work-groups stay together.
__device__ __forceinline__ int rotated_chunk(int r, int u, int max_chunks) {
  const int k = r - (u & 7) % max_chunks;
  return k < 0 ? k + max_chunks : k;
}

// Pairs of 16-lane rows on the VALU (gfx950 permlane swaps).  Called with
// the lane's own value as both operands, v_permlane16_swap returns in every
// lane the values of the even and of the odd row of the pair (r, r ^ 1), and
// v_permlane32_swap those of the halves (h, h ^ 1) -- measured lane layout.
// One add or max of the two results then reduces over lanes l and l ^ 16
// (l ^ 32), in the same operand order in both lanes, with no LDS round trip.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  if constexpr (N >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (N == 8) x += dpp<kHalfMirror>(x);
  if constexpr (N >= 16) {
    x += dpp<kRowMirror>(x);
    x += dpp<kHalfMirror>(x);
  }
  if constexpr (N >= 32) x = sum_xor16(x);
  if constexpr (N >= 64) x = sum_xor32(x);
  return x;
}

// Exclusive prefix sum of v over a work-group of NW waves (every thread
// calls it): an inclusive scan within each wave by shuffles, then the wave
// totals from LDS (s_w holds NW ints).  *total receives the sum over the
// work-group.  Two barriers; s_w may be reused after the call.
template <int NW>
__device__ __forceinline__ int wg_exclusive_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = s_w[w];
    base += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------------------
// Matrix-core tiles (grouped-query decode, gated prefill).  A 32-key tile of K
// and V passes through LDS as rows, with their 16-byte chunks permuted, so
// that the v_mfma_f32_16x16x32_bf16 operands (K by 128-bit reads, V by the
// transposing read) are conflict-free LDS reads.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTileKeys = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRaise = 8.f;  // natural-log units

// K chunk permutation of 256-byte rows: chunk c of key r is stored at chunk
// c ^ k_swz(r), conflict-free for the 128-bit operand reads and cheap writes.
__device__ __forceinline__ int k_swz(int key) { return ((key >> 3) & 3) ^ (((key >> 1) & 1) << 2); }

// Orders this wave's LDS writes before its later LDS reads (and vice versa).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Chunk swizzle of staged V rows: the four rows one transposing read takes
// (keys 2 g + h + 8 j, j = 0..3) land their 32 bytes in distinct banks.
__device__ __forceinline__ int vrow_swz(int key) { return 2 * ((key >> 3) & 3); }

// Tiles of 32 rows of D bf16 staged as rows (K with the chunk swizzle
// tile_kswz, V with vrow_swz) and read as MFMA operands (K by 128-bit reads,
// V by the transposing read).  The LDS of gfx950 has 64 four-byte banks and
// serves a 128-bit read 16 lanes at a time and a 64-bit read 32 lanes at a
// time (measured: the bank-conflict counter follows this model exactly).
// With 128-byte rows (D = 64) the row's parity picks the bank half, and the
// rows one pass reads all have the same parity, so row r is stored at
// tile_row(r) = r ^ bit 1 of r, which puts half of each pass in either half;
// the K swizzle then takes bit 2 of the key, so the chunks within a half are
// distinct.  Conflict-free for the staging writes and both operand reads.
// 256-byte rows (D = 128) keep the plain order and k_swz.
template <int D>
__device__ __forceinline__ int tile_row(int key) {
  return D == 64 ? key ^ ((key >> 1) & 1) : key;
}
template <int D>
__device__ __forceinline__ int tile_kswz(int key) {
  return D == 64 ? (((key >> 3) & 3) ^ (((key >> 2) & 1) << 2)) : k_swz(key);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane l receives element
// l % 4 of the 8-byte pieces addressed by lanes 4 j + (l % 16) / 4, j = 0..3
// (measured lane layout on gfx950).  Returned as raw 64 bits.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 tr_read(const char* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Score-tile key of operand row r in 16-key half st of a 32-key tile: with
// this order, the 8 scores a lane receives (keys 2 (l/16) + st + 8 i) are
// exactly its 8 contraction slots of the value product.
__device__ __forceinline__ int tile_key(int st, int r) { return 2 * (r >> 2) + st + 8 * (r & 3); }

// ---------------------------------------------------------------------------
// Device view of the cache (plain values; built on the host per call).
struct CacheView {
  int B, H, D, bs, log2bs, cap, cap_blocks, dtype;
  const void* k;
  const void* v;
  uint16_t* mu;   // bfloat16 bits
  uint16_t* var;  // bfloat16 bits
  float* maxnorm;
  const int32_t* seq_len;
};

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The N admitted (or union) blocks of a balanced decode in wn equal ranges, wn = min(waves, ceil(N / split)),
// range w = [lo(w), lo(w + 1)), all non-empty as wn <= N.
struct FlowPlan {
  int N, wn;
  __device__ FlowPlan(int n, int waves, int split)
      : N(n), wn(n == 0 ? 0 : min(waves, ceil_div(n, split))) {}
  __device__ int lo(int w) const { return (int)((long long)w * N / wn); }
  // The range holding position p < N.
  __device__ int range_of(int p) const {
    int w = (int)((long long)p * wn / N);
    while (w + 1 < wn && lo(w + 1) <= p) ++w;
    return w;
  }
};

// ---------------------------------------------------------------------------
// Eq. 5 block score (paper: "Elastic Threshold Attention ...", Methodology 4),
// shared by the screen, the calibration and the fused screen + decode, so all
// of them take every admission decision with the same float32 arithmetic.
constexpr int kLanesPerBlock = 8;  // lanes that read one block's statistics
constexpr int kBlocksPerIter = kWave / kLanesPerBlock;  // 8 blocks per wave step

// The block statistics mu and var are stored as bfloat16 (8 per 128-bit
// load).  Per-lane share of the query: with 8 lanes per block, load t
// (t < D/64) of lane li reads elements [64 t + 8 li, 64 t + 8 li + 8) of a
// statistics row, so each load instruction covers one full 128-byte line of
// each of 8 blocks; the lane keeps the matching query elements.
template <int D>
struct QShare {
  static constexpr int kLoads = D / 64;
  static constexpr int kElems = 8 * kLoads;
  float q[kElems];
  float q2[kElems];
  float qn;  // ||q||_2
};

template <int D>
__device__ __forceinline__ void load_qshare(const float* qu, int li, QShare<D>& s) {
  float qq = 0.f;
#pragma unroll
  for (int t = 0; t < QShare<D>::kLoads; ++t) {
    const float4 v0 = *reinterpret_cast<const float4*>(qu + 64 * t + 8 * li);
    const float4 v1 = *reinterpret_cast<const float4*>(qu + 64 * t + 8 * li + 4);
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s.q[8 * t + e] = x[e];
      s.q2[8 * t + e] = x[e] * x[e];
      qq = fmaf(x[e], x[e], qq);
    }
  }
  s.qn = sqrtf(group_sum<kLanesPerBlock>(qq));
}

// This lane's partial sums q . mu and (q * q) . var over its elements of one
// block (raw bf16 statistics loads m[t], v[t]), in element order.
template <int D>
__device__ __forceinline__ void score_partials(const QShare<D>& s, const uint4* m,
                                               const uint4* v, float& dot, float& mom) {
#pragma unroll
  for (int t = 0; t < QShare<D>::kLoads; ++t) {
    float mf[8], vf[8];
    widen<ETA_DT_BF16>(m[t], mf);
    widen<ETA_DT_BF16>(v[t], vf);
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(s.q[8 * t + e], mf[e], dot);
#pragma unroll
    for (int e = 0; e < 8; ++e) mom = fmaf(s.q2[8 * t + e], vf[e], mom);
  }
}

// Eq. 5 score of block j of stream u.  All 8 lanes of the block's group must
// call it together (DPP reductions); `valid` false yields garbage that the
// caller ignores.  Every lane of the group returns the identical value.
template <int D>
__device__ __forceinline__ float block_score(const CacheView& c, int u, int j, bool valid,
                                             const QShare<D>& s, int li, float z, bool z_inf,
                                             float scale) {
  float dot = 0.f, mom = 0.f, M = 0.f;
  if (valid) {
    const size_t row = ((size_t)u * c.cap_blocks + j) * D;
    uint4 m[QShare<D>::kLoads], v[QShare<D>::kLoads];
#pragma unroll
    for (int t = 0; t < QShare<D>::kLoads; ++t) {
      m[t] = ld16_nt(c.mu + row + 64 * t + 8 * li);
      v[t] = ld16_nt(c.var + row + 64 * t + 8 * li);
    }
    score_partials<D>(s, m, v, dot, mom);
    M = c.maxnorm[(size_t)u * c.cap_blocks + j];
  }
  dot = group_sum<kLanesPerBlock>(dot);
  mom = group_sum<kLanesPerBlock>(mom);
  const float geometric = s.qn * M;
  if (z_inf) return scale * geometric;
  return scale * fminf(fmaf(z, sqrtf(mom), dot), geometric);
}

// ---------------------------------------------------------------------------
// Eq. 1 threshold of one (sequence, head), tau = sum_j q_j W[j][h] + bias[h]
// over the n = H*D entries of the sequence's query, by the 256 threads of a
// work-group in one fixed order, which the threshold kernel keeps for all the
// heads it sums at once (so the fused screen + decode, which calls this, and
// the threshold kernel produce the same bits): thread t adds q_j W[j][h]
// for j = t, t + 256, ... in that order (fmaf, eight loads in flight), the 64
// lanes of a wave are summed by an xor butterfly (every lane ends with the
// same bits), the four wave sums as (w0 + w1) + (w2 + w3), the bias last.
// W == NULL (frozen thresholds) gives bias[h] alone.  Every thread returns
// the value; with W it contains one barrier (s_red: 4 floats of LDS).  The
// first 256 threads of the work-group do the sum; further threads (a larger
// work-group) take part only in the barrier.
constexpr int kTauThreads = 256;
__device__ __forceinline__ float tau_of_head(const float* qb, const float* W, const float* bias,
                                             int H, int n, int h, float* s_red) {
  if (!W) return bias[h];
  const int t = threadIdx.x;
  if (t < kTauThreads) {
    float acc = 0.f;
    int j = t;
    for (; j + 7 * kTauThreads < n; j += 8 * kTauThreads) {
      float qv[8], wv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        qv[r] = qb[j + r * kTauThreads];
        wv[r] = W[(size_t)(j + r * kTauThreads) * H + h];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) acc = fmaf(qv[r], wv[r], acc);
    }
    for (; j < n; j += kTauThreads) acc = fmaf(qb[j], W[(size_t)j * H + h], acc);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
    if ((t & (kWave - 1)) == 0) s_red[t / kWave] = acc;
  }
  __syncthreads();
  return ((s_red[0] + s_red[1]) + (s_red[2] + s_red[3])) + bias[h];
}

// ---------------------------------------------------------------------------
// Launchers (defined in the kernel translation units).  Each returns the
// hipError_t of its launch; shapes were validated by the caller.
hipError_t launch_append(const CacheView& c, const void* k_new, const void* v_new,
                         int32_t* overflow, hipStream_t s);
hipError_t launch_block_meta(const CacheView& c, int first_block, int n_blocks, hipStream_t s);
hipError_t launch_predict(int B, int H, int D, const float* q, const float* W, const float* bias,
                          float a, float* tau_gate, float* tau_screen, hipStream_t s);
hipError_t launch_screen(const CacheView& c, const float* q, const float* tau_screen, float z,
                         float scale, int32_t* active_idx, int32_t* active_cnt, uint64_t* ctr,
                         uint64_t* words, hipStream_t s);
struct DecodeArgs {
  const float* q;
  const float* tau;
  const int32_t* active_idx;
  const int32_t* active_cnt;
  int mode;  // ETA_LOGIT_GATED / ETA_LOGIT_RAW
  bool dense;
  float beta, scale;
  int split;       // blocks per chunk (dense, fused), least blocks per range (balanced)
  int max_chunks;  // ceil(cap_blocks / split)
  float* part_m;   // partials: [B*H][max_chunks] chunked, slot w + u balanced
  float* part_l;
  float* part_acc; // [...][D]
  float* out;
  int flow_grid;     // work-groups of the balanced decode (kFlowThreads each)
  int* flow_start;   // [B*H + 1] admitted-block offsets of the balanced decode
  int* flow_info;    // [1] total admitted blocks N
  bool flow_global;  // offsets in global memory (flow_scan_kernel), not in LDS
  int* flow_wave_u;  // [waves] first stream of each wave's range (flow_global only)
};
// Work-group size and work-groups per compute unit of the balanced decode
// (2 waves per SIMD, its occupancy: all of them are resident at once) and the
// stream count up to which its work-groups scan the offsets into LDS (above,
// a one-work-group scan kernel writes them to global memory first).  Two
// work-groups per CU leave 256 registers per lane (about 171 used, no spills);
// against three (168 registers, a few spilled) the 38% 128K call went from
// 0.52 to 0.50-0.51 ms, 10% from 0.152 to 0.147, 512K from 0.274 to
// 0.259-0.270; four (128 registers) doubled the time.
constexpr int kFlowThreads = 256;
constexpr int kFlowWGsPerCU = 2;
constexpr int kMaxFlowUnits = 8191;
hipError_t launch_decode(const CacheView& c, const DecodeArgs& a, hipStream_t s);
// Fused threshold + screen + decode: the threshold's and the screen's inputs
// and optional outputs beside the decode arguments (split = blocks per chunk
// <= kMaxFusedChunk, dense set so that the combine counts every chunk of a
// stream).
constexpr int kMaxFusedChunk = 32;
struct ScreenDecodeArgs {
  const float* W;           // [H*D][H] predictor weights, or NULL (frozen constants)
  const float* bias;        // [H]: bias (with W) or the frozen per-head constants
  float a;                  // threshold adjustment: tau_screen = tau - a
  float z;
  float* tau_gate;          // [B*H] written by each stream's first chunk, or NULL
  float* tau_screen;        // [B*H] likewise, or NULL
  uint32_t* chunk_bits;     // [B*H][max_chunks] admission bits of each chunk, or NULL
  uint64_t* ctr;            // += admitted tokens, or NULL
};
hipError_t launch_screen_decode(const CacheView& c, const DecodeArgs& a,
                                const ScreenDecodeArgs& sa, hipStream_t s);
// Grouped-query attention: KV stream u = b*H + kv serves query heads
// u*G .. u*G + G - 1 (G <= 16).
struct GqaDecode {
  int G;
  const float* q;          // [B*H*G][D]
  const float* tau;        // [B*H*G] gate thresholds (GATED)
  const int32_t* union_idx;  // [B*H][cap_blocks] ascending union lists
  const uint32_t* head_mask; // [B*H][cap_blocks] bit g: query head g admits block j
  const int32_t* union_cnt;  // [B*H]
  int mode;
  bool dense;
  float beta, scale;
  int split;        // blocks_per_split: the least union blocks per wave's range
  float* part_m;    // [(waves + B*H) * G] partials, slot (w + u) * G + g
  float* part_l;    // [(waves + B*H) * G]
  float* part_acc;  // [(waves + B*H) * G][D]
  float* out;       // [B*H*G][D]
  int flow_grid;    // one-wave work-groups of the balanced decode (set at launch)
  int* flow_start;  // [B*H + 1] union-block offsets, written by the balanced decode
  int* flow_info;   // [1] total union blocks N
  bool flow_global; // offsets in global memory (flow_scan_gqa_kernel), not in LDS
  int* flow_wave_u; // [waves] first stream of each wave's range (flow_global only)
};
constexpr int kMaxGroup = 16;
// Resident one-wave work-groups per compute unit of the balanced grouped
// decode are at most this many (8 waves per SIMD); it bounds its partial
// slots and the per-wave start table.  Up to kMaxGqaFlowUnits KV streams every
// work-group scans the stream offsets into LDS; above, a one-work-group scan
// kernel writes them (and each wave's first stream) to global memory.
constexpr int kMaxFlowWavesPerCU = 32;
constexpr int kMaxGqaFlowUnits = 6143;
int device_cus();
hipError_t launch_screen_gqa(const CacheView& c, int G, const float* q, const float* tau_screen,
                             float z, float scale, int32_t* union_idx, uint32_t* head_mask,
                             int32_t* union_cnt, uint64_t* ctr, uint64_t* words, hipStream_t s);
hipError_t launch_decode_gqa(const CacheView& c, const GqaDecode& g, hipStream_t s);
// Gated causal attention forward over whole sequences (bf16 q, K, V).
struct PrefillArgs {
  int B, Hkv, G, Hq, T, D;
  const void* q;  // [B][Hq][T][D] bf16
  const void* k;  // [B][Hkv][T][D] bf16
  const void* v;
  const float* tau;  // [B][Hq][T]
  float beta, scale;
  float* out;   // [B][Hq][T][D]
  float* dens;  // [B][Hq][T] or null
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
hipError_t launch_calibrate(const CacheView& c, int n_sets, const float* q_sets,
                            const float* tau0, float z, float scale, float rho, float* values,
                            float* c_out, hipStream_t s);

}  // namespace eta
