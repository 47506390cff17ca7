// eta_api.hip -- host side of the C ABI declared in include/eta.h.
//
// Every entry point validates all of its arguments on the host first, then
// enqueues kernels on the caller's stream.  Nothing is allocated, nothing is
// synchronised and no state survives a call.  Device-side values (sequence
// lengths, admitted counts) are never read back: grids are sized from host
// capacities and surplus work-groups exit at once.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "eta_internal.h"

namespace eta {
// Compute units of the current device (a device property, cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
}  // namespace eta

namespace {
using eta::device_cus;

thread_local char g_err[512] = "";

eta_status fail(eta_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

eta_status ok() {
  g_err[0] = '\0';
  return ETA_OK;
}

bool pow2_block(int b) { return b == 4 || b == 8 || b == 16 || b == 32 || b == 64 || b == 128; }

int ilog2(int b) {
  int r = 0;
  while ((1 << r) < b) ++r;
  return r;
}

// Largest grid we launch is units * ceil(cap_blocks / small) work-groups; keep
// every flattened grid below 2^31.
constexpr long long kMaxGrid = 0x7fffffffLL;

// Validates the cache descriptor; for a non-empty problem every data pointer
// must be set.
eta_status check_cache(const eta_cache* c, eta::CacheView* v) {
  if (!c) return fail(ETA_ERR_NULL_PTR, "cache descriptor is NULL");
  if (c->batch < 0 || c->heads < 0)
    return fail(ETA_ERR_BAD_SHAPE, "batch (%d) and heads (%d) must be >= 0", c->batch, c->heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(ETA_ERR_BAD_SHAPE, "head_dim %d unsupported (64 or 128)", c->head_dim);
  if (!pow2_block(c->block))
    return fail(ETA_ERR_BAD_SHAPE, "block %d unsupported (4, 8, 16, 32, 64 or 128)", c->block);
  if (c->cap_tokens < 1) return fail(ETA_ERR_BAD_SHAPE, "cap_tokens %d must be >= 1", c->cap_tokens);
  if (c->kv_dtype != ETA_DT_F32 && c->kv_dtype != ETA_DT_BF16)
    return fail(ETA_ERR_BAD_ARG, "kv_dtype %d unknown", c->kv_dtype);
  if ((long long)c->batch * c->heads > (1LL << 24))
    return fail(ETA_ERR_BAD_SHAPE, "batch*heads %lld too large", (long long)c->batch * c->heads);
  if (c->batch > 0 && c->heads > 0) {
    if (!c->k || !c->v) return fail(ETA_ERR_NULL_PTR, "cache k/v pointer is NULL");
    if (!c->mu || !c->var || !c->maxnorm)
      return fail(ETA_ERR_NULL_PTR, "cache statistics pointer is NULL");
    if (!c->seq_len) return fail(ETA_ERR_NULL_PTR, "cache seq_len pointer is NULL");
  }
  v->B = c->batch;
  v->H = c->heads;
  v->D = c->head_dim;
  v->bs = c->block;
  v->log2bs = ilog2(c->block);
  v->cap = c->cap_tokens;
  v->cap_blocks = eta::ceil_div(c->cap_tokens, c->block);
  v->dtype = c->kv_dtype;
  v->k = c->k;
  v->v = c->v;
  v->mu = c->mu;
  v->var = c->var;
  v->maxnorm = c->maxnorm;
  v->seq_len = c->seq_len;
  return ETA_OK;
}

bool empty(const eta::CacheView& v) { return v.B == 0 || v.H == 0; }

eta_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ETA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


// Partial slots.  The balanced decode needs one per wave plus one per stream
// (its slots w + u); the flat grid one per possible chunk.
size_t flow_slots(long long units) {
  return (size_t)((long long)(eta::kFlowThreads / 64) * device_cus() * eta::kFlowWGsPerCU + units);
}
size_t grid_slots(long long units, int cap_blocks, int split) {
  return (size_t)(units * ((cap_blocks + split - 1) / split));
}
// Enough for either path (the size query: one workspace serves the sparse and
// the dense decode of a cache).
size_t decode_slots(long long units, int cap_blocks, int split) {
  const size_t f = flow_slots(units), g = grid_slots(units, cap_blocks, split);
  return f > g ? f : g;
}

// Per-wave first streams of the balanced decode's global form.
size_t flow_wave_table_bytes() {
  return align256((size_t)(eta::kFlowThreads / 64) * device_cus() * eta::kFlowWGsPerCU * 4);
}

// Decode workspace: [balanced-decode total at byte 64 | stream offsets
// [units+1] | per-wave first streams | part_m | part_l | part_acc], each
// 256-byte aligned.
size_t decode_ws_slots(long long units, int D, size_t slots) {
  return 256 + align256((size_t)(units + 1) * 4) + flow_wave_table_bytes() +
         align256(slots * 4) * 2 + align256(slots * (size_t)D * 4);
}
size_t decode_ws(long long units, int D, int cap_blocks, int split) {
  return decode_ws_slots(units, D, decode_slots(units, cap_blocks, split));
}


bool bad_float(float x) { return x != x; }

}  // namespace

// ---------------------------------------------------------------------------
// Decode without allocation: the workspace is a file-scope device array of
// kScratchBytes, one copy per device, shared by every such call on it.  Its
// address is looked up once per device (with that device current) and kept;
// the array's name is only a host-side stand-in and is never passed to a
// kernel.  The decode needs no part of it cleared: the kernels of one call
// write every counter and offset before reading it.

namespace {
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

static eta_status static_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ETA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ETA_ERR_HIP, "device %d outside the %d devices with a scratch slot", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ETA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return ETA_OK;
}

extern "C" {

int32_t eta_abi_version(void) { return ETA_ABI_VERSION; }

const char* eta_status_string(eta_status s) {
  switch (s) {
    case ETA_OK: return "ETA_OK";
    case ETA_ERR_NULL_PTR: return "ETA_ERR_NULL_PTR";
    case ETA_ERR_BAD_SHAPE: return "ETA_ERR_BAD_SHAPE";
    case ETA_ERR_BAD_ARG: return "ETA_ERR_BAD_ARG";
    case ETA_ERR_CAPACITY: return "ETA_ERR_CAPACITY";
    case ETA_ERR_WORKSPACE: return "ETA_ERR_WORKSPACE";
    case ETA_ERR_HIP: return "ETA_ERR_HIP";
    default: return "ETA_ERR_UNKNOWN";
  }
}

const char* eta_last_error(void) { return g_err; }

int32_t eta_cache_blocks(const eta_cache* c) {
  if (!c || c->block <= 0 || c->cap_tokens < 0) return -1;
  return eta::ceil_div(c->cap_tokens, c->block);
}

eta_status eta_append_kv(const eta_cache* c, const void* k_new, const void* v_new,
                         int32_t* overflow, void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (empty(v)) return ok();
  if (!k_new || !v_new) return fail(ETA_ERR_NULL_PTR, "k_new/v_new is NULL");
  // T_b lives on the device, so a full sequence can only be reported there:
  // the flag is required, so that a dropped token cannot go unnoticed.
  if (!overflow)
    return fail(ETA_ERR_NULL_PTR, "overflow flag is NULL (required: it reports an append to a "
                                  "full sequence)");
  return hip_status(eta::launch_append(v, k_new, v_new, overflow, (hipStream_t)stream),
                    "eta_append_kv launch");
}

eta_status eta_build_block_meta(const eta_cache* c, int32_t first_block, int32_t n_blocks,
                                void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (first_block < 0) return fail(ETA_ERR_BAD_ARG, "first_block %d < 0", first_block);
  if (n_blocks < -1) return fail(ETA_ERR_BAD_ARG, "n_blocks %d < -1", n_blocks);
  if (n_blocks == -1) n_blocks = first_block < v.cap_blocks ? v.cap_blocks - first_block : 0;
  if ((long long)first_block + n_blocks > v.cap_blocks)
    return fail(ETA_ERR_CAPACITY, "blocks [%d, %lld) exceed cap_blocks %d", first_block,
                (long long)first_block + n_blocks, v.cap_blocks);
  if (empty(v) || n_blocks == 0) return ok();
  if ((long long)eta::ceil_div(n_blocks, 4) * v.B * v.H > kMaxGrid)
    return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  return hip_status(eta::launch_block_meta(v, first_block, n_blocks, (hipStream_t)stream),
                    "eta_build_block_meta launch");
}

eta_status eta_predict_tau(int32_t batch, int32_t heads, int32_t head_dim, const float* q,
                           const float* W, const float* bias_or_c, float a, float* tau_gate,
                           float* tau_screen, void* stream) {
  if (batch < 0 || heads < 0 || head_dim < 1)
    return fail(ETA_ERR_BAD_SHAPE, "batch %d, heads %d, head_dim %d", batch, heads, head_dim);
  if (heads > 256) return fail(ETA_ERR_BAD_SHAPE, "heads %d > 256", heads);
  if (bad_float(a)) return fail(ETA_ERR_BAD_ARG, "a is NaN");
  if (batch == 0 || heads == 0) return ok();
  if (!bias_or_c || !tau_gate || !tau_screen)
    return fail(ETA_ERR_NULL_PTR, "bias_or_c/tau_gate/tau_screen is NULL");
  if (W && !q) return fail(ETA_ERR_NULL_PTR, "q is NULL in dynamic mode");
  return hip_status(eta::launch_predict(batch, heads, head_dim, q, W, bias_or_c, a, tau_gate,
                                        tau_screen, (hipStream_t)stream),
                    "eta_predict_tau launch");
}

size_t eta_screen_workspace_bytes(int32_t batch, int32_t heads, int32_t cap_blocks) {
  if (batch <= 0 || heads <= 0 || cap_blocks <= 0) return 256;
  return align256((size_t)batch * heads * (size_t)eta::ceil_div(cap_blocks, 64) * 8);
}

eta_status eta_screen(const eta_cache* c, const float* q, const float* tau_screen, float z,
                      float scale, int32_t* active_idx, int32_t* active_cnt,
                      uint64_t* density_ctr, void* workspace, size_t workspace_bytes,
                      void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (bad_float(z) || z < 0.f) return fail(ETA_ERR_BAD_ARG, "z must be >= 0 (or +inf)");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (empty(v)) return ok();
  if (!q || !tau_screen || !active_idx || !active_cnt)
    return fail(ETA_ERR_NULL_PTR, "q/tau_screen/active_idx/active_cnt is NULL");
  const size_t need = eta_screen_workspace_bytes(v.B, v.H, v.cap_blocks);
  if (!workspace || workspace_bytes < need)
    return fail(ETA_ERR_WORKSPACE, "screen workspace %zu bytes < %zu", workspace_bytes, need);
  if ((long long)eta::ceil_div(v.cap_blocks, 64) * v.B * v.H > kMaxGrid)
    return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  return hip_status(eta::launch_screen(v, q, tau_screen, z, scale, active_idx, active_cnt,
                                       density_ctr, static_cast<uint64_t*>(workspace),
                                       (hipStream_t)stream),
                    "eta_screen launch");
}

size_t eta_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim,
                                  int32_t cap_blocks, int32_t blocks_per_split) {
  if (batch <= 0 || heads <= 0 || head_dim <= 0 || cap_blocks <= 0 || blocks_per_split <= 0)
    return 256;
  return decode_ws((long long)batch * heads, head_dim, cap_blocks, blocks_per_split);
}

// ws == kStaticScratch: the library's own scratch (eta_decode_noalloc), looked
// up only once the arguments are valid.
static char kStaticScratchTag;
static void* const kStaticScratch = &kStaticScratchTag;

static eta_status decode_common(const eta_cache* c, const float* q, const float* tau_gate,
                                const int32_t* active_idx, const int32_t* active_cnt,
                                int32_t mode, bool dense, float beta, float scale, int32_t split,
                                void* ws, size_t ws_bytes, float* out, void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (mode != ETA_LOGIT_GATED && mode != ETA_LOGIT_RAW)
    return fail(ETA_ERR_BAD_ARG, "logit_mode %d unknown", mode);
  if (mode == ETA_LOGIT_GATED && !dense && (bad_float(beta) || !(beta > 0.f) || isinf(beta)))
    return fail(ETA_ERR_BAD_ARG, "beta must be finite and > 0");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (split < 1 || split > 4096)
    return fail(ETA_ERR_BAD_ARG, "blocks_per_split %d outside [1, 4096]", split);
  if (empty(v)) return ok();
  if (!q || !out) return fail(ETA_ERR_NULL_PTR, "q/out is NULL");
  if (!dense && (!active_idx || !active_cnt))
    return fail(ETA_ERR_NULL_PTR, "active_idx/active_cnt is NULL");
  if (!dense && mode == ETA_LOGIT_GATED && !tau_gate)
    return fail(ETA_ERR_NULL_PTR, "tau_gate is NULL in GATED mode");
  const long long units = (long long)v.B * v.H;
  const int maxc = eta::ceil_div(v.cap_blocks, split);
  if ((long long)maxc * units > kMaxGrid) return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  // Sparse decode runs balanced (equal ranges of all admitted blocks per
  // wave); block positions of all streams together are int32, more than any
  // one device holds (2^31 blocks of at least 4 keys of d >= 64: over 2 TB).
  if (!dense && units * (long long)v.cap_blocks >= 0x7fffffffLL)
    return fail(ETA_ERR_BAD_SHAPE, "B*H*cap_blocks must be below 2^31");
  const bool flow = !dense;
  // A caller's workspace must be as large as the size query says (enough for
  // either path); the static scratch only needs what this call's path uses.
  const size_t slots = flow ? flow_slots(units) : grid_slots(units, v.cap_blocks, split);
  if (ws == kStaticScratch) {
    const size_t need = decode_ws_slots(units, v.D, slots);
    if (need > ws_bytes)
      return fail(ETA_ERR_CAPACITY,
                  "this decode needs %zu bytes of scratch; the static scratch holds %zu "
                  "(use eta_decode with a workspace)", need, ws_bytes);
    if (eta_status s = static_scratch(&ws, &ws_bytes)) return s;
  } else {
    const size_t need = decode_ws(units, v.D, v.cap_blocks, split);
    if (!ws || ws_bytes < need)
      return fail(ETA_ERR_WORKSPACE, "decode workspace %zu bytes < %zu", ws_bytes, need);
  }
  char* w = static_cast<char*>(ws);
  const size_t off_start = 256;
  const size_t off_waves = off_start + align256((size_t)(units + 1) * 4);
  const size_t off_parts = off_waves + flow_wave_table_bytes();
  eta::DecodeArgs a;
  a.q = q;
  a.tau = tau_gate;
  a.active_idx = active_idx;
  a.active_cnt = active_cnt;
  a.mode = dense ? ETA_LOGIT_RAW : mode;
  a.dense = dense;
  a.beta = beta;
  a.scale = scale;
  a.split = split;
  a.max_chunks = maxc;
  a.part_m = reinterpret_cast<float*>(w + off_parts);
  a.part_l = reinterpret_cast<float*>(w + off_parts + align256(slots * 4));
  a.part_acc = reinterpret_cast<float*>(w + off_parts + 2 * align256(slots * 4));
  a.out = out;
  // Dense decode runs on the flat stream-major grid (one work-group per
  // chunk); sparse decode balanced, with its offsets in LDS up to
  // kMaxFlowUnits streams and in global memory above.
  a.flow_grid = device_cus() * eta::kFlowWGsPerCU;
  a.flow_start = reinterpret_cast<int*>(w + off_start);
  a.flow_info = reinterpret_cast<int*>(w + 64);
  a.flow_global = units > eta::kMaxFlowUnits;
  a.flow_wave_u = reinterpret_cast<int*>(w + off_waves);
  return hip_status(eta::launch_decode(v, a, (hipStream_t)stream), "eta_decode launch");
}

eta_status eta_decode(const eta_cache* c, const float* q, const float* tau_gate,
                      const int32_t* active_idx, const int32_t* active_cnt, int32_t logit_mode,
                      float beta, float scale, int32_t blocks_per_split, void* workspace,
                      size_t workspace_bytes, float* out, void* stream) {
  return decode_common(c, q, tau_gate, active_idx, active_cnt, logit_mode, false, beta, scale,
                       blocks_per_split, workspace, workspace_bytes, out, stream);
}

eta_status eta_decode_noalloc(const eta_cache* c, const float* q, const float* tau_gate,
                              const int32_t* active_idx, const int32_t* active_cnt,
                              int32_t logit_mode, float beta, float scale,
                              int32_t blocks_per_split, float* out, void* stream) {
  return decode_common(c, q, tau_gate, active_idx, active_cnt, logit_mode, false, beta, scale,
                       blocks_per_split, kStaticScratch, kScratchBytes, out, stream);
}

eta_status eta_dense_decode(const eta_cache* c, const float* q, float scale,
                            int32_t blocks_per_split, void* workspace, size_t workspace_bytes,
                            float* out, void* stream) {
  return decode_common(c, q, nullptr, nullptr, nullptr, ETA_LOGIT_RAW, true, 1.f, scale,
                       blocks_per_split, workspace, workspace_bytes, out, stream);
}

size_t eta_fused_step_workspace_bytes(int32_t batch, int32_t heads, int32_t head_dim,
                                      int32_t cap_blocks, int32_t blocks_per_chunk) {
  if (batch <= 0 || heads <= 0 || head_dim <= 0 || cap_blocks <= 0 || blocks_per_chunk <= 0)
    return 256;
  const long long units = (long long)batch * heads;
  return decode_ws_slots(units, head_dim, grid_slots(units, cap_blocks, blocks_per_chunk));
}

eta_status eta_fused_step(const eta_cache* c, const float* q, const float* W,
                          const float* bias_or_c, float a, float z, int32_t logit_mode,
                          float beta, float scale, int32_t blocks_per_chunk, float* tau_gate,
                          float* tau_screen, uint32_t* chunk_bits, uint64_t* density_ctr,
                          void* workspace, size_t workspace_bytes, float* out, void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (v.H > 256) return fail(ETA_ERR_BAD_SHAPE, "heads %d > 256", v.H);
  if (logit_mode != ETA_LOGIT_GATED && logit_mode != ETA_LOGIT_RAW)
    return fail(ETA_ERR_BAD_ARG, "logit_mode %d unknown", logit_mode);
  if (logit_mode == ETA_LOGIT_GATED && (bad_float(beta) || !(beta > 0.f) || isinf(beta)))
    return fail(ETA_ERR_BAD_ARG, "beta must be finite and > 0");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (bad_float(z) || z < 0.f) return fail(ETA_ERR_BAD_ARG, "z must be >= 0 (or +inf)");
  if (bad_float(a)) return fail(ETA_ERR_BAD_ARG, "a is NaN");
  if (blocks_per_chunk < 1 || blocks_per_chunk > eta::kMaxFusedChunk)
    return fail(ETA_ERR_BAD_ARG, "blocks_per_chunk %d outside [1, %d]", blocks_per_chunk,
                eta::kMaxFusedChunk);
  if (empty(v)) return ok();
  if (!q || !out || !bias_or_c) return fail(ETA_ERR_NULL_PTR, "q/bias_or_c/out is NULL");
  const long long units = (long long)v.B * v.H;
  if ((long long)v.H * v.D > 0x7fffffffLL / 4) return fail(ETA_ERR_BAD_SHAPE, "heads * head_dim too large");
  const int maxc = eta::ceil_div(v.cap_blocks, blocks_per_chunk);
  if ((long long)maxc * units > kMaxGrid) return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  const size_t slots = grid_slots(units, v.cap_blocks, blocks_per_chunk);
  const size_t need = decode_ws_slots(units, v.D, slots);
  if (!workspace || workspace_bytes < need)
    return fail(ETA_ERR_WORKSPACE, "fused-step workspace %zu bytes < %zu", workspace_bytes, need);
  char* w = static_cast<char*>(workspace);
  const size_t off_parts = 256 + align256((size_t)(units + 1) * 4);
  eta::DecodeArgs d = {};
  d.q = q;
  d.mode = logit_mode;
  d.dense = true;  // the combine merges every chunk of a stream
  d.beta = beta;
  d.scale = scale;
  d.split = blocks_per_chunk;
  d.max_chunks = maxc;
  d.part_m = reinterpret_cast<float*>(w + off_parts);
  d.part_l = reinterpret_cast<float*>(w + off_parts + align256(slots * 4));
  d.part_acc = reinterpret_cast<float*>(w + off_parts + 2 * align256(slots * 4));
  d.out = out;
  eta::ScreenDecodeArgs sa;
  sa.W = W;
  sa.bias = bias_or_c;
  sa.a = a;
  sa.z = z;
  sa.tau_gate = tau_gate;
  sa.tau_screen = tau_screen;
  sa.chunk_bits = chunk_bits;
  sa.ctr = density_ctr;
  return hip_status(eta::launch_screen_decode(v, d, sa, (hipStream_t)stream),
                    "eta_fused_step launch");
}

size_t eta_calibrate_workspace_bytes(int32_t n_sets, int32_t batch, int32_t heads,
                                     int32_t cap_blocks) {
  if (n_sets <= 0 || batch <= 0 || heads <= 0 || cap_blocks <= 0) return 256;
  return align256((size_t)n_sets * batch * heads * (size_t)cap_blocks * 4);
}

eta_status eta_calibrate_threshold(const eta_cache* c, int32_t n_sets, const float* q_sets,
                                   const float* tau0, float z, float scale,
                                   float target_density, void* workspace,
                                   size_t workspace_bytes, float* c_out, void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (n_sets < 1) return fail(ETA_ERR_BAD_SHAPE, "n_sets %d < 1", n_sets);
  if (bad_float(z) || z < 0.f) return fail(ETA_ERR_BAD_ARG, "z must be >= 0 (or +inf)");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (bad_float(target_density) || target_density < 0.f || target_density > 1.f)
    return fail(ETA_ERR_BAD_ARG, "target_density must lie in [0, 1]");
  if (empty(v)) return ok();
  if (!q_sets || !c_out) return fail(ETA_ERR_NULL_PTR, "q_sets/c_out is NULL");
  if ((long long)n_sets * v.B * v.cap_blocks > 0x7fffffffLL)
    return fail(ETA_ERR_CAPACITY, "more than 2^31-1 pooled values per head");
  if ((long long)eta::ceil_div(v.cap_blocks, 256) * n_sets * v.B * v.H > kMaxGrid)
    return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  const size_t need = eta_calibrate_workspace_bytes(n_sets, v.B, v.H, v.cap_blocks);
  if (!workspace || workspace_bytes < need)
    return fail(ETA_ERR_WORKSPACE, "calibrate workspace %zu bytes < %zu", workspace_bytes, need);
  return hip_status(eta::launch_calibrate(v, n_sets, q_sets, tau0, z, scale, target_density,
                                          static_cast<float*>(workspace), c_out,
                                          (hipStream_t)stream),
                    "eta_calibrate_threshold launch");
}

// ---------------------------------------------------------------------------
// Grouped-query attention.

// Grouped screen workspace: the union admission words (8 bytes per 64 blocks)
// followed by each word's admitted head tokens (4 bytes).
size_t eta_screen_gqa_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t cap_blocks) {
  if (batch <= 0 || kv_heads <= 0 || cap_blocks <= 0) return 256;
  return align256((size_t)batch * kv_heads * (size_t)eta::ceil_div(cap_blocks, 64) * 12);
}

eta_status eta_screen_gqa(const eta_cache* c, int32_t group, const float* q,
                          const float* tau_screen, float z, float scale, int32_t* union_idx,
                          uint32_t* head_mask, int32_t* union_cnt, uint64_t* density_ctr,
                          void* workspace, size_t workspace_bytes, void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (group < 1 || group > eta::kMaxGroup)
    return fail(ETA_ERR_BAD_SHAPE, "group %d outside [1, %d]", group, eta::kMaxGroup);
  if (bad_float(z) || z < 0.f) return fail(ETA_ERR_BAD_ARG, "z must be >= 0 (or +inf)");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (empty(v)) return ok();
  if (!q || !tau_screen || !union_idx || !head_mask || !union_cnt)
    return fail(ETA_ERR_NULL_PTR, "q/tau_screen/union_idx/head_mask/union_cnt is NULL");
  const size_t need = eta_screen_gqa_workspace_bytes(v.B, v.H, v.cap_blocks);
  if (!workspace || workspace_bytes < need)
    return fail(ETA_ERR_WORKSPACE, "screen workspace %zu bytes < %zu", workspace_bytes, need);
  if ((long long)eta::ceil_div(v.cap_blocks, 64) * v.B * v.H > kMaxGrid)
    return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  return hip_status(eta::launch_screen_gqa(v, group, q, tau_screen, z, scale, union_idx,
                                           head_mask, union_cnt, density_ctr,
                                           static_cast<uint64_t*>(workspace),
                                           (hipStream_t)stream),
                    "eta_screen_gqa launch");
}

// GQA decode workspace: [balanced-decode total (256 B) | stream offsets
// [units+1] | part_m | part_l | part_acc], each 256-byte aligned.  Partial
// slots: one per query head and chunk of the flat grid; for the balanced
// decode one per query head and (wave, stream) slot, with at most
// kMaxFlowWavesPerCU waves per compute unit.
// Partial slots of the balanced grouped decode: one per (wave, KV stream)
// segment, at most kMaxFlowWavesPerCU waves per compute unit, per query head.
static size_t decode_gqa_slots(long long units, int group) {
  return (size_t)(((long long)eta::kMaxFlowWavesPerCU * device_cus() + units) * group);
}

// Per-wave first streams of the balanced grouped decode's global form.
static size_t gqa_wave_table_bytes() {
  return align256((size_t)eta::kMaxFlowWavesPerCU * device_cus() * 4);
}

static size_t decode_gqa_ws(long long units, int group, int D, int cap_blocks, int split) {
  (void)cap_blocks;
  (void)split;
  const size_t slots = decode_gqa_slots(units, group);
  return 256 + align256((size_t)(units + 1) * 4) + gqa_wave_table_bytes() +
         align256(slots * 4) * 2 + align256(slots * (size_t)D * 4);
}

size_t eta_decode_gqa_workspace_bytes(int32_t batch, int32_t kv_heads, int32_t group,
                                      int32_t head_dim, int32_t cap_blocks,
                                      int32_t blocks_per_split) {
  if (batch <= 0 || kv_heads <= 0 || group <= 0 || head_dim <= 0 || cap_blocks <= 0 ||
      blocks_per_split <= 0)
    return 256;
  return decode_gqa_ws((long long)batch * kv_heads, group, head_dim, cap_blocks,
                       blocks_per_split);
}

static eta_status decode_gqa_common(const eta_cache* c, int32_t group, const float* q,
                                    const float* tau_gate, const int32_t* union_idx,
                                    const uint32_t* head_mask, const int32_t* union_cnt,
                                    int32_t mode, bool dense, float beta, float scale,
                                    int32_t split, void* ws, size_t ws_bytes, float* out,
                                    void* stream) {
  eta::CacheView v;
  if (eta_status s = check_cache(c, &v)) return s;
  if (group < 1 || group > eta::kMaxGroup)
    return fail(ETA_ERR_BAD_SHAPE, "group %d outside [1, %d]", group, eta::kMaxGroup);
  if (v.dtype != ETA_DT_BF16)
    return fail(ETA_ERR_BAD_ARG, "grouped-query decode needs a bf16 cache (kv_dtype %d)",
                v.dtype);
  if (mode != ETA_LOGIT_GATED && mode != ETA_LOGIT_RAW)
    return fail(ETA_ERR_BAD_ARG, "logit_mode %d unknown", mode);
  if (mode == ETA_LOGIT_GATED && !dense && (bad_float(beta) || !(beta > 0.f) || isinf(beta)))
    return fail(ETA_ERR_BAD_ARG, "beta must be finite and > 0");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (split < 1 || split > 2048)
    return fail(ETA_ERR_BAD_ARG, "blocks_per_split %d outside [1, 2048]", split);
  if (empty(v)) return ok();
  if (!q || !out) return fail(ETA_ERR_NULL_PTR, "q/out is NULL");
  if (!dense && (!union_idx || !head_mask || !union_cnt))
    return fail(ETA_ERR_NULL_PTR, "union_idx/head_mask/union_cnt is NULL");
  if (!dense && mode == ETA_LOGIT_GATED && !tau_gate)
    return fail(ETA_ERR_NULL_PTR, "tau_gate is NULL in GATED mode");
  const long long units = (long long)v.B * v.H;
  if (units * group > kMaxGrid) return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  // Block positions of all streams together are int32 (more than any one
  // device holds: 2^31 blocks of at least 4 keys of d >= 64 are over 2 TB).
  if (units * (long long)v.cap_blocks >= 0x7fffffffLL)
    return fail(ETA_ERR_BAD_SHAPE, "B*H_kv*cap_blocks must be below 2^31");
  const size_t need = decode_gqa_ws(units, group, v.D, v.cap_blocks, split);
  if (!ws || ws_bytes < need)
    return fail(ETA_ERR_WORKSPACE, "decode workspace %zu bytes < %zu", ws_bytes, need);
  const size_t slots = decode_gqa_slots(units, group);
  char* w = static_cast<char*>(ws);
  const size_t off_waves = 256 + align256((size_t)(units + 1) * 4);
  const size_t off_parts = off_waves + gqa_wave_table_bytes();
  eta::GqaDecode g;
  g.G = group;
  g.q = q;
  g.tau = tau_gate;
  g.union_idx = union_idx;
  g.head_mask = head_mask;
  g.union_cnt = union_cnt;
  g.mode = dense ? ETA_LOGIT_RAW : mode;
  g.dense = dense;
  g.beta = beta;
  g.scale = scale;
  g.split = split;
  g.part_m = reinterpret_cast<float*>(w + off_parts);
  g.part_l = reinterpret_cast<float*>(w + off_parts + align256(slots * 4));
  g.part_acc = reinterpret_cast<float*>(w + off_parts + 2 * align256(slots * 4));
  g.out = out;
  // The grouped decode, sparse or dense, runs balanced (equal ranges of all
  // union blocks per wave), with its stream offsets in LDS up to
  // kMaxGqaFlowUnits streams and in global memory above.
  g.flow_global = units > eta::kMaxGqaFlowUnits;
  g.flow_grid = 0;
  g.flow_start = reinterpret_cast<int*>(w + 256);
  g.flow_info = reinterpret_cast<int*>(w);
  g.flow_wave_u = reinterpret_cast<int*>(w + off_waves);
  return hip_status(eta::launch_decode_gqa(v, g, (hipStream_t)stream), "eta_decode_gqa launch");
}

eta_status eta_decode_gqa(const eta_cache* c, int32_t group, const float* q,
                          const float* tau_gate, const int32_t* union_idx,
                          const uint32_t* head_mask, const int32_t* union_cnt,
                          int32_t logit_mode, float beta, float scale, int32_t blocks_per_split,
                          void* workspace, size_t workspace_bytes, float* out, void* stream) {
  return decode_gqa_common(c, group, q, tau_gate, union_idx, head_mask, union_cnt, logit_mode,
                           false, beta, scale, blocks_per_split, workspace, workspace_bytes, out,
                           stream);
}

eta_status eta_dense_decode_gqa(const eta_cache* c, int32_t group, const float* q, float scale,
                                int32_t blocks_per_split, void* workspace,
                                size_t workspace_bytes, float* out, void* stream) {
  return decode_gqa_common(c, group, q, nullptr, nullptr, nullptr, nullptr, ETA_LOGIT_RAW, true,
                           1.f, scale, blocks_per_split, workspace, workspace_bytes, out,
                           stream);
}

// ---------------------------------------------------------------------------
// Gated causal attention forward (prefill / training forward).

eta_status eta_gated_prefill(int32_t batch, int32_t kv_heads, int32_t group, int32_t seq_len,
                             int32_t head_dim, const void* q, const void* k, const void* v,
                             const float* tau, float beta, float scale, float* out, float* dens,
                             void* stream) {
  if (batch < 0 || kv_heads < 0 || group < 1 || seq_len < 0)
    return fail(ETA_ERR_BAD_SHAPE, "batch %d, kv_heads %d, group %d, seq_len %d", batch,
                kv_heads, group, seq_len);
  if (head_dim != 64 && head_dim != 128)
    return fail(ETA_ERR_BAD_SHAPE, "head_dim %d unsupported (64 or 128)", head_dim);
  if (bad_float(beta) || !(beta > 0.f) || isinf(beta))
    return fail(ETA_ERR_BAD_ARG, "beta must be finite and > 0");
  if (bad_float(scale) || !(scale > 0.f) || isinf(scale))
    return fail(ETA_ERR_BAD_ARG, "scale must be finite and > 0");
  if (batch == 0 || kv_heads == 0 || seq_len == 0) return ok();
  if (!q || !k || !v || !tau || !out) return fail(ETA_ERR_NULL_PTR, "q/k/v/tau/out is NULL");
  const long long hq = (long long)kv_heads * group;
  if ((long long)batch * hq * seq_len * head_dim > (1LL << 40))
    return fail(ETA_ERR_BAD_SHAPE, "problem too large");
  // The kernel addresses rows within one K/V stream with 32-bit byte offsets.
  if ((long long)seq_len * head_dim * 2 >= (1LL << 32))
    return fail(ETA_ERR_BAD_SHAPE, "seq_len %d too long: one K/V stream must hold < 2^32 bytes",
                seq_len);
  if ((long long)eta::ceil_div(seq_len, 64) * batch * hq > kMaxGrid)
    return fail(ETA_ERR_BAD_SHAPE, "grid too large");
  eta::PrefillArgs a;
  a.B = batch;
  a.Hkv = kv_heads;
  a.G = group;
  a.Hq = (int)hq;
  a.T = seq_len;
  a.D = head_dim;
  a.q = q;
  a.k = k;
  a.v = v;
  a.tau = tau;
  a.beta = beta;
  a.scale = scale;
  a.out = out;
  a.dens = dens;
  return hip_status(eta::launch_prefill(a, (hipStream_t)stream), "eta_gated_prefill launch");
}

}  // extern "C"
