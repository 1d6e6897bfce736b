// Host side of the joint RoPE attention library: the C ABI declared in
// include/flux_attn.h (argument validation, plan lifetime, launches).
//
// Validation runs entirely on the host before any HIP call, so every error
// path can be exercised without a GPU.
#include "flux_attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <mutex>
#include <new>
#include <unordered_set>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return FLUX_ATTN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? FLUX_ATTN_OUT_OF_MEMORY : FLUX_ATTN_DEVICE_ERROR,
              "%s: %s", what, hipGetErrorString(e));
}

size_t elem_bytes(int dtype) { return dtype == FLUX_ATTN_FP8_E4M3 ? 1 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

}  // namespace

struct flux_attn_plan {
  flux_attn_config cfg;
  int device = -1;
  // RoPE table, [max_tokens][head_dim/2], rewritten by each call: packed fp16
  // (cos, sin) for the attention kernels, or fp32 pairs for the tile-mask
  // rule (the allocation is sized for the latter).
  void* rope_table = nullptr;
  flux::RopeFreq freq{};         // per-pair frequencies (host; kernel argument)
  float* part_o = nullptr;       // split-K/V partials: [max_pieces][256][head_dim]
  float2* part_ml = nullptr;     // [max_pieces][256]
  // tile-sparse workspace (bf16 plans): tile means, kept-tile lists
  float* qbar = nullptr;         // [B][H][QT][D]
  float* kbar = nullptr;         // [B][H][KT][D]
  int* kv_list = nullptr;        // [B*H*QT][KT]
  int* kv_count = nullptr;       // [B*H*QT]
  int* tile_order = nullptr;     // [B*H*QT] dispatch order of a tile-sparse launch
  float* dr = nullptr;           // backward: rowsum(dO * O), [B][H][N]
  uint16_t* rq = nullptr;        // backward: bf16 R(q), R(k), [B][N][H][D]
  uint16_t* rk = nullptr;
  int num_cus = 0;
  int max_pieces = 0;
  int sched_mode = 0;  // FLUX_ATTN_SCHEDULE at creation: 0 by cost, 1 'split', 2 'persistent'
  std::vector<hipEvent_t> ev_start, ev_mid, ev_stop;  // kernel timing: attention | merge
  int timing_used = 0;
  unsigned long long* clk = nullptr;  // while timing: shader cycles and wall ticks of the timed kernels
  int wall_khz = 0;                   // rate of the wall-clock counter
};

namespace {

// The RoPE table in the attention kernels' form (packed fp16 pairs).
uint32_t* rope16(flux_attn_plan* p) { return static_cast<uint32_t*>(p->rope_table); }

void release_timing(flux_attn_plan* p) {
  for (auto e : p->ev_start) (void)hipEventDestroy(e);
  for (auto e : p->ev_mid) (void)hipEventDestroy(e);
  for (auto e : p->ev_stop) (void)hipEventDestroy(e);
  p->ev_start.clear();
  p->ev_mid.clear();
  p->ev_stop.clear();
  p->timing_used = 0;
  (void)hipFree(p->clk);
  p->clk = nullptr;
}

}  // namespace

namespace {

// Registry of live plans, so a destroyed or foreign pointer is rejected
// without being dereferenced.
std::mutex g_plans_mu;
std::unordered_set<const flux_attn_plan*> g_plans;

bool plan_live(const flux_attn_plan* p) {
  std::lock_guard<std::mutex> lk(g_plans_mu);
  return p && g_plans.count(p) != 0;
}

}  // namespace

// Scratch memory of the allocation-free forward (flux_attn_forward_noalloc):
// the RoPE table and the split partials of one call.  Every device that loads
// the library holds its own copy until the process ends.  In host code the
// name `scratch` is only a stand-in: kernels get the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) char scratch[FLUX_ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` and compute-unit count, per device ordinal,
// looked up on the first allocation-free call on that device.  A fixed table:
// the lookup itself allocates no host or device memory.
constexpr int kMaxDevices = 64;
struct ScratchDevice {
  bool ready;
  void* ptr;
  int num_cus;
};
std::mutex g_scratch_mu;
ScratchDevice g_scratch[kMaxDevices];

int noalloc_scratch(int dev, ScratchDevice* out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FLUX_ATTN_UNSUPPORTED, "device ordinal %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchDevice& sd = g_scratch[dev];
  if (!sd.ready) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(FLUX_ATTN_DEVICE_ERROR, "scratch has no address on device %d", dev);
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    sd.ptr = ptr;
    sd.num_cus = cus;
    sd.ready = true;
  }
  *out = sd;
  return FLUX_ATTN_OK;
}

}  // namespace

extern "C" {

int flux_attn_abi_version(void) { return FLUX_ATTN_ABI_VERSION; }

const char* flux_attn_status_string(int status) {
  switch (status) {
    case FLUX_ATTN_OK: return "ok";
    case FLUX_ATTN_INVALID_ARGUMENT: return "invalid argument";
    case FLUX_ATTN_UNSUPPORTED: return "unsupported";
    case FLUX_ATTN_DEVICE_ERROR: return "device error";
    case FLUX_ATTN_OUT_OF_MEMORY: return "out of device memory";
    default: return "unknown status";
  }
}

const char* flux_attn_last_error(void) { return g_last_error.c_str(); }

int flux_attn_default_config(flux_attn_config* cfg, int32_t batch, int32_t num_heads, int32_t head_dim,
                             int32_t max_tokens) {
  if (!cfg) return fail(FLUX_ATTN_INVALID_ARGUMENT, "cfg is NULL");
  std::memset(cfg, 0, sizeof *cfg);
  cfg->batch = batch;
  cfg->num_heads = num_heads;
  cfg->head_dim = head_dim;
  cfg->max_tokens = max_tokens;
  cfg->max_segments = 12;
  cfg->rope_axes_dim[0] = head_dim / 4;
  cfg->rope_axes_dim[1] = 3 * head_dim / 8;
  cfg->rope_axes_dim[2] = 3 * head_dim / 8;
  cfg->rope_theta = 10000.0f;
  cfg->softmax_scale = 0.0f;
  cfg->dtype = FLUX_ATTN_BF16;
  return ok();
}

int flux_attn_validate_config(const flux_attn_config* c) {
  if (!c) return fail(FLUX_ATTN_INVALID_ARGUMENT, "config is NULL");
  if (c->batch < 1) return fail(FLUX_ATTN_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", c->batch);
  if (c->num_heads < 1) return fail(FLUX_ATTN_INVALID_ARGUMENT, "num_heads must be >= 1 (got %d)", c->num_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(FLUX_ATTN_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->max_tokens < 1) return fail(FLUX_ATTN_INVALID_ARGUMENT, "max_tokens must be >= 1 (got %d)", c->max_tokens);
  if (c->max_segments < 1)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "max_segments must be >= 1 (got %d)", c->max_segments);
  int sum = 0;
  for (int a = 0; a < 3; ++a) {
    const int d = c->rope_axes_dim[a];
    if (d < 0 || d % 8)
      return fail(FLUX_ATTN_INVALID_ARGUMENT, "rope_axes_dim[%d] = %d must be a non-negative multiple of 8", a, d);
    sum += d;
  }
  if (sum != c->head_dim)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "rope_axes_dim sums to %d, head_dim is %d", sum, c->head_dim);
  if (!(c->rope_theta > 0.0f) || !std::isfinite(c->rope_theta))
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
  if (!std::isfinite(c->softmax_scale)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (c->dtype != FLUX_ATTN_BF16 && c->dtype != FLUX_ATTN_FP8_E4M3)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "unknown dtype %d", c->dtype);
  // Offsets inside one [B][N][H][D] tensor are formed in 64-bit, but the
  // kernels read a batch entry's tokens through buffer resources whose range
  // (num_records) is 32-bit: one batch entry of q, k or v must stay under 4 GiB,
  // or rows past the wrapped range would read as zeros.
  const double elems = (double)c->batch * c->max_tokens * c->num_heads * c->head_dim;
  if (elems > 9.0e15) return fail(FLUX_ATTN_INVALID_ARGUMENT, "tensor too large");
  const double entry_bytes = (double)c->max_tokens * c->num_heads * c->head_dim *
                             (c->dtype == FLUX_ATTN_FP8_E4M3 ? 1.0 : 2.0);
  if (entry_bytes >= 4294967296.0)
    return fail(FLUX_ATTN_UNSUPPORTED,
                "one batch entry of q/k/v is %.0f bytes; the kernels address at most 4 GiB per entry",
                entry_bytes);
  return ok();
}

namespace {

// The forward() checks of everything but the output tensor.
int validate_inputs(const flux_attn_config* c, const void* q, const void* k, const void* v,
                    const float* qkv_scale, const int32_t* segment_tokens, int32_t num_segments,
                    const int32_t* pos_ids, long long* n_out) {
  int st = flux_attn_validate_config(c);
  if (st) return st;
  if (!segment_tokens) return fail(FLUX_ATTN_INVALID_ARGUMENT, "segment_tokens is NULL");
  if (num_segments < 1 || num_segments > c->max_segments)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "num_segments = %d outside [1, %d]", num_segments, c->max_segments);
  long long n = 0;
  for (int i = 0; i < num_segments; ++i) {
    if (segment_tokens[i] < 0)
      return fail(FLUX_ATTN_INVALID_ARGUMENT, "segment_tokens[%d] = %d is negative", i, segment_tokens[i]);
    n += segment_tokens[i];
  }
  if (n < 1) return fail(FLUX_ATTN_INVALID_ARGUMENT, "total token count is 0");
  if (n > c->max_tokens)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "total token count %lld exceeds max_tokens %d", n, c->max_tokens);
  if (!q || !k || !v || !pos_ids) return fail(FLUX_ATTN_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(pos_ids) & 3u) != 0)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "pos_ids must be 4-byte aligned");
  const bool fp8 = c->dtype == FLUX_ATTN_FP8_E4M3;
  if (fp8 && !qkv_scale) return fail(FLUX_ATTN_INVALID_ARGUMENT, "FP8 inputs need qkv_scale");
  if (!fp8 && qkv_scale) return fail(FLUX_ATTN_INVALID_ARGUMENT, "qkv_scale is only used with FP8 inputs");
  *n_out = n;
  return ok();
}

}  // namespace

int flux_attn_validate_forward(const flux_attn_config* c, const void* q, const void* k, const void* v,
                               const float* qkv_scale, const int32_t* segment_tokens, int32_t num_segments,
                               const int32_t* pos_ids, const void* out) {
  long long n = 0;
  int st = validate_inputs(c, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, &n);
  if (st) return st;
  if (!out) return fail(FLUX_ATTN_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (!aligned16(out)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  const size_t in_bytes = (size_t)c->batch * (size_t)n * c->num_heads * c->head_dim * elem_bytes(c->dtype);
  const size_t out_bytes = (size_t)c->batch * (size_t)n * c->num_heads * c->head_dim * 2;
  if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
      overlaps(out, out_bytes, v, in_bytes))
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "out overlaps q, k or v");
  return ok();
}

namespace {

// theta^(-2j/d_a) for pair j of axis slice a, in double.
flux::RopeFreq rope_freq(const flux_attn_config& c) {
  flux::RopeFreq f{};
  int j0 = 0;
  for (int a = 0; a < 3; ++a) {
    const int d = c.rope_axes_dim[a];
    for (int j = 0; j < d / 2; ++j) f.f[j0 + j] = std::pow((double)c.rope_theta, -2.0 * j / d);
    j0 += d / 2;
  }
  return f;
}

}  // namespace

int flux_attn_create(const flux_attn_config* cfg, flux_attn_plan** out) {
  if (!out) return fail(FLUX_ATTN_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  int st = flux_attn_validate_config(cfg);
  if (st) return st;
  auto* p = new (std::nothrow) flux_attn_plan();
  if (!p) return fail(FLUX_ATTN_OUT_OF_MEMORY, "host allocation failed");
  p->cfg = *cfg;
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  const int half = cfg->head_dim / 2;
  p->freq = rope_freq(*cfg);
  e = hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  // Schedule override for tests and measurements (the default is by cost).
  if (const char* sm = std::getenv("FLUX_ATTN_SCHEDULE")) {
    if (std::strcmp(sm, "split") == 0) p->sched_mode = 1;
    if (std::strcmp(sm, "persistent") == 0) p->sched_mode = 2;
  }
  // Split-K/V partials: at most 4 pieces per compute unit, and no more than
  // the launch can produce at max_tokens.
  {
    const long tiles = (long)cfg->batch * cfg->num_heads * ((cfg->max_tokens + 255) / 256);
    const long kv = (cfg->max_tokens + 63) / 64;
    long cap = 4L * p->num_cus;
    const long most = tiles * (kv < 16 ? kv : 16);
    p->max_pieces = (int)(cap < most ? cap : most);
  }
  e = hipMalloc(&p->rope_table, (size_t)cfg->max_tokens * half * sizeof(float2));
  if (e == hipSuccess && p->max_pieces > 0)
    e = hipMalloc(&p->part_o, (size_t)p->max_pieces * 256 * cfg->head_dim * sizeof(float));
  if (e == hipSuccess && p->max_pieces > 0)
    e = hipMalloc(&p->part_ml, (size_t)p->max_pieces * 256 * sizeof(float2));
  if (e == hipSuccess && cfg->dtype == FLUX_ATTN_BF16) {
    const size_t rows = (size_t)cfg->batch * cfg->num_heads;
    const size_t qt = (cfg->max_tokens + 255) / 256, kt = (cfg->max_tokens + 63) / 64;
    e = hipMalloc(&p->qbar, rows * qt * cfg->head_dim * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&p->kbar, rows * kt * cfg->head_dim * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&p->kv_list, rows * qt * kt * sizeof(int));
    if (e == hipSuccess) e = hipMalloc(&p->kv_count, rows * qt * sizeof(int));
    if (e == hipSuccess) e = hipMalloc(&p->tile_order, rows * qt * sizeof(int));
    if (e == hipSuccess) e = hipMalloc(&p->dr, rows * cfg->max_tokens * sizeof(float));
    const size_t elems = rows * cfg->max_tokens * cfg->head_dim;
    if (e == hipSuccess) e = hipMalloc(&p->rq, elems * sizeof(uint16_t));
    if (e == hipSuccess) e = hipMalloc(&p->rk, elems * sizeof(uint16_t));
  }
  if (e != hipSuccess) {
    (void)hipFree(p->rope_table);
    (void)hipFree(p->part_o);
    (void)hipFree(p->part_ml);
    (void)hipFree(p->qbar);
    (void)hipFree(p->kbar);
    (void)hipFree(p->kv_list);
    (void)hipFree(p->kv_count);
    (void)hipFree(p->tile_order);
    (void)hipFree(p->dr);
    (void)hipFree(p->rq);
    (void)hipFree(p->rk);
    delete p;
    return hip_fail(e, "plan workspace");
  }
  {
    std::lock_guard<std::mutex> lk(g_plans_mu);
    g_plans.insert(p);
  }
  *out = p;
  return ok();
}

int flux_attn_get_config(const flux_attn_plan* plan, flux_attn_config* cfg) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  if (!cfg) return fail(FLUX_ATTN_INVALID_ARGUMENT, "cfg is NULL");
  *cfg = plan->cfg;
  return ok();
}

namespace {

// Fills the range table of a bf16 launch with lens[0..n) (token offsets
// tok0s) and returns the launch's tile count.
int set_ranges(flux::AttnArgs& a, const int* tok0s, const int* lens, int n, int batch, int heads) {
  a.nranges = n;
  int tiles = 0;
  for (int r = 0; r < n; ++r) {
    a.rng_tok0[r] = tok0s[r];
    a.rng_len[r] = lens[r];
    a.rng_tile0[r] = tiles;
    tiles += batch * heads * ((lens[r] + 255) / 256);
  }
  a.rng_tile0[n] = tiles;
  return tiles;
}

// Device memory and policy one forward call works with.
struct FwdWorkspace {
  uint32_t* rope;     // packed fp16 RoPE table, at least N x D/2 entries
  float* part_o;      // split partials: [max_pieces][256][D]
  float2* part_ml;    // [max_pieces][256]
  int max_pieces;
  int num_cus;
  int sched_mode;     // 0 by cost, 1 never persistent, 2 persistent where possible
  unsigned long long* clk;  // optional clock measurement of the attention kernels
};

// Optional HIP events bracketing the call: before the attention kernel, after
// it (before the last merge), and at the end.
struct FwdEvents {
  hipEvent_t start, mid, stop;
};

// The launches of one validated forward call: RoPE table, then the attention
// kernel(s) and their merges, on `stream`.
int launch_forward(const flux_attn_config& c, const flux::RopeFreq& freq, const FwdWorkspace& ws, const void* q,
                   const void* k, const void* v, const float* qkv_scale, const int32_t* segment_tokens,
                   int32_t num_segments, const int32_t* pos_ids, void* out, bool joint, float* lse,
                   hipStream_t stream, const FwdEvents* ev) {
  int n = 0;
  for (int i = 0; i < num_segments; ++i) n += segment_tokens[i];
  hipError_t e = flux::launch_rope_table(pos_ids, freq, ws.rope, n, c.head_dim, c.rope_axes_dim[0],
                                         c.rope_axes_dim[1], stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  const float scale = c.softmax_scale > 0.0f ? c.softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
  const float log2e = 1.4426950408889634f;
  // Token ranges attended over: the whole sequence (joint), or each non-empty
  // segment on its own (segment-local).  bf16: one attention launch (+ merge)
  // covers up to kMaxRanges ranges, longest first, so that short segments fill
  // the last round of the long ones; e4m3: one launch per range.  Launches run
  // one after another on the stream and share the partial-state workspace.
  std::vector<int> tok0s, lens;
  {
    int off = 0;
    for (int r = 0; r < (joint ? 1 : num_segments); ++r) {
      const int len = joint ? n : segment_tokens[r];
      if (len > 0) {
        tok0s.push_back(off);
        lens.push_back(len);
      }
      off += len;
    }
  }
  const bool fp8 = c.dtype == FLUX_ATTN_FP8_E4M3;
  std::vector<int> order(lens.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  if (!fp8) std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lens[x] > lens[y]; });
  const int per_launch = fp8 ? 1 : flux::AttnArgs::kMaxRanges;
  const int n_launch = ((int)order.size() + per_launch - 1) / per_launch;
  if (ev) {
    e = hipEventRecord(ev->start, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  const size_t tok = (size_t)c.num_heads * c.head_dim;  // elements per token
  for (int li = 0; li < n_launch; ++li) {
    const int r0 = li * per_launch, r1 = std::min((int)order.size(), r0 + per_launch);
    int gt[flux::AttnArgs::kMaxRanges], gl[flux::AttnArgs::kMaxRanges];
    int max_len = 0;
    for (int r = r0; r < r1; ++r) {
      gt[r - r0] = tok0s[order[r]];
      gl[r - r0] = lens[order[r]];
      max_len = std::max(max_len, gl[r - r0]);
    }
    flux::AttnArgs a{};
    const int tiles = set_ranges(a, gt, gl, r1 - r0, c.batch, c.num_heads);
    const flux::Schedule sch =
        (!fp8 && r1 - r0 == 1)
            ? flux::plan_schedule_dense(tiles, (max_len + 63) / 64, ws.num_cus, ws.max_pieces, c.head_dim,
                                        ws.sched_mode)
            : flux::plan_schedule(tiles, (max_len + 63) / 64, ws.num_cus, ws.max_pieces, c.head_dim);
    a.batch_tokens = n;
    a.heads = c.num_heads;
    a.batch = c.batch;
    a.c = scale * log2e;
    a.part_o = ws.part_o;
    a.part_ml = ws.part_ml;
    a.lse = lse;
    a.clk = ev ? ws.clk : nullptr;
    if (fp8) {
      const size_t off = (size_t)gt[0];
      flux::Fp8Args f{};
      f.q = static_cast<const uint8_t*>(q) + off * tok;
      f.k = static_cast<const uint8_t*>(k) + off * tok;
      f.v = static_cast<const uint8_t*>(v) + off * tok;
      f.scales = qkv_scale;
      f.o = static_cast<uint16_t*>(out) + off * tok;
      f.rope = ws.rope + off * (c.head_dim / 2);
      f.n_tokens = gl[0];
      f.batch_tokens = n;
      f.heads = c.num_heads;
      f.batch = c.batch;
      f.c = a.c;
      f.part_o = a.part_o;
      f.part_ml = a.part_ml;
      f.clk = a.clk;
      e = flux::launch_attn_fp8(f, c.head_dim, sch, stream);
      // the e4m3 merge reads the same fields through AttnArgs: one range at
      // offset 0 of the shifted pointers
      a.o = f.o;
      gt[0] = 0;
      set_ranges(a, gt, gl, 1, c.batch, c.num_heads);
    } else {
      a.q = static_cast<const uint16_t*>(q);
      a.k = static_cast<const uint16_t*>(k);
      a.v = static_cast<const uint16_t*>(v);
      a.o = static_cast<uint16_t*>(out);
      a.rope = ws.rope;
      e = flux::launch_attn_bf16(a, c.head_dim, sch, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    // The joint call's first timing interval brackets its attention kernel
    // alone; in segment-local mode it spans all launches (merges between them
    // included).  The second interval is the last merge.
    if (ev && li == n_launch - 1) {
      e = hipEventRecord(ev->mid, stream);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    e = flux::launch_attn_merge(a, c.head_dim, sch, stream);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  if (ev) {
    e = hipEventRecord(ev->stop, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return ok();
}

int forward_impl(flux_attn_plan* plan, const void* q, const void* k, const void* v, const float* qkv_scale,
                 const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids, void* out,
                 bool joint, float* lse, void* hip_stream) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  const flux_attn_config& c = plan->cfg;
  int st = flux_attn_validate_forward(&c, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, out);
  if (st) return st;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan was created on device %d, current device is %d", plan->device, dev);
  const FwdWorkspace ws{rope16(plan), plan->part_o, plan->part_ml, plan->max_pieces, plan->num_cus,
                        plan->sched_mode, plan->clk};
  const bool timed = plan->timing_used < (int)plan->ev_start.size();
  FwdEvents ev{};
  if (timed) {
    const int i = plan->timing_used;
    ev = FwdEvents{plan->ev_start[i], plan->ev_mid[i], plan->ev_stop[i]};
  }
  st = launch_forward(c, plan->freq, ws, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, out, joint,
                      lse, static_cast<hipStream_t>(hip_stream), timed ? &ev : nullptr);
  if (st) return st;
  if (timed) ++plan->timing_used;
  return ok();
}

}  // namespace

int flux_attn_forward(flux_attn_plan* plan, const void* q, const void* k, const void* v, const float* qkv_scale,
                      const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids, void* out,
                      void* hip_stream) {
  return forward_impl(plan, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, out, true, nullptr,
                      hip_stream);
}

int flux_attn_forward_segment_local(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                                    const float* qkv_scale, const int32_t* segment_tokens, int32_t num_segments,
                                    const int32_t* pos_ids, void* out, void* hip_stream) {
  return forward_impl(plan, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, out, false, nullptr,
                      hip_stream);
}

int flux_attn_forward_noalloc(const flux_attn_config* cfg, const void* q, const void* k, const void* v,
                              const float* qkv_scale, const int32_t* segment_tokens, int32_t num_segments,
                              const int32_t* pos_ids, void* out, void* hip_stream) {
  int st = flux_attn_validate_forward(cfg, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, out);
  if (st) return st;
  const flux_attn_config& c = *cfg;
  long long n = 0;
  for (int i = 0; i < num_segments; ++i) n += segment_tokens[i];
  // Scratch layout: [RoPE table | partial O | partial (m, l)], each 256-byte
  // aligned.  The table must fit; what is left bounds the split pieces.
  const size_t table_bytes = ((size_t)n * (c.head_dim / 2) * 4 + 255) & ~(size_t)255;
  const size_t cap = FLUX_ATTN_NOALLOC_SCRATCH_BYTES;
  if (table_bytes > cap)
    return fail(FLUX_ATTN_UNSUPPORTED,
                "%lld tokens need a %zu-byte RoPE table; the allocation-free scratch holds %zu bytes "
                "(at most %zu tokens at head_dim %d)",
                n, table_bytes, cap, cap / ((size_t)c.head_dim * 2), c.head_dim);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  ScratchDevice sd{};
  st = noalloc_scratch(dev, &sd);
  if (st) return st;
  char* const base = static_cast<char*>(sd.ptr);
  const size_t piece_o = (size_t)256 * c.head_dim * sizeof(float), piece_ml = (size_t)256 * sizeof(float2);
  long pieces = (long)((cap - table_bytes) / (piece_o + piece_ml));
  pieces = std::min(pieces, 4L * sd.num_cus);
  FwdWorkspace ws{};
  ws.rope = reinterpret_cast<uint32_t*>(base);
  ws.part_o = reinterpret_cast<float*>(base + table_bytes);
  ws.part_ml = reinterpret_cast<float2*>(base + table_bytes + (size_t)pieces * piece_o);
  ws.max_pieces = (int)pieces;
  ws.num_cus = sd.num_cus;
  ws.sched_mode = 1;  // whole tiles + split pieces only: the persistent split needs 2 slots per CU
  ws.clk = nullptr;
  return launch_forward(c, rope_freq(c), ws, q, k, v, qkv_scale, segment_tokens, num_segments, pos_ids, out,
                        true, nullptr, static_cast<hipStream_t>(hip_stream), nullptr);
}

int flux_attn_forward_lse(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                          const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids, void* out,
                          float* lse, void* hip_stream) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  if (plan->cfg.dtype != FLUX_ATTN_BF16) return fail(FLUX_ATTN_UNSUPPORTED, "the training forward needs a bf16 plan");
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "lse is NULL or misaligned");
  return forward_impl(plan, q, k, v, nullptr, segment_tokens, num_segments, pos_ids, out, true, lse,
                      hip_stream);
}

int flux_attn_backward(flux_attn_plan* plan, const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, const int32_t* segment_tokens, int32_t num_segments,
                       const int32_t* pos_ids, void* dq, void* dk, void* dv, void* hip_stream) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  const flux_attn_config& c = plan->cfg;
  if (c.dtype != FLUX_ATTN_BF16) return fail(FLUX_ATTN_UNSUPPORTED, "the backward needs a bf16 plan");
  int st = flux_attn_validate_forward(&c, q, k, v, nullptr, segment_tokens, num_segments, pos_ids, out);
  if (st) return st;
  if (!dout || !lse || !dq || !dk || !dv) return fail(FLUX_ATTN_INVALID_ARGUMENT, "a gradient pointer is NULL");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "dout, dq, dk, dv must be 16-byte aligned and lse 4-byte aligned");
  int n = 0;
  for (int i = 0; i < num_segments; ++i) n += segment_tokens[i];
  const size_t bytes = (size_t)c.batch * n * c.num_heads * c.head_dim * 2;
  const void* ins[5] = {q, k, v, out, dout};
  void* grads[3] = {dq, dk, dv};
  for (int gi = 0; gi < 3; ++gi) {
    for (int ii = 0; ii < 5; ++ii)
      if (overlaps(grads[gi], bytes, ins[ii], bytes))
        return fail(FLUX_ATTN_INVALID_ARGUMENT, "a gradient overlaps an input");
    for (int gj = 0; gj < gi; ++gj)
      if (overlaps(grads[gi], bytes, grads[gj], bytes))
        return fail(FLUX_ATTN_INVALID_ARGUMENT, "dq, dk and dv overlap");
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan was created on device %d, current device is %d", plan->device, dev);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  e = flux::launch_rope_table(pos_ids, plan->freq, rope16(plan), n, c.head_dim, c.rope_axes_dim[0],
                              c.rope_axes_dim[1], stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  const float scale = c.softmax_scale > 0.0f ? c.softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
  flux::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dr = plan->dr;
  a.qr = plan->rq;
  a.kr = plan->rk;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.rope = rope16(plan);
  a.n_tokens = n;
  a.heads = c.num_heads;
  a.batch = c.batch;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  const bool timed = plan->timing_used < (int)plan->ev_start.size();
  if (timed) {
    e = hipEventRecord(plan->ev_start[plan->timing_used], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  e = flux::launch_attn_bwd(a, c.head_dim, stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  if (timed) {
    e = hipEventRecord(plan->ev_mid[plan->timing_used], stream);
    if (e == hipSuccess) e = hipEventRecord(plan->ev_stop[plan->timing_used], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    ++plan->timing_used;
  }
  return ok();
}

namespace {

// Checks shared by the tile-sparse entry points: a live bf16 plan on the
// current device and the forward() argument rules (joint mode, no scales).
int sparse_common(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                  const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids, const void* out,
                  const void* mask, int* n_out) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  const flux_attn_config& c = plan->cfg;
  if (c.dtype != FLUX_ATTN_BF16) return fail(FLUX_ATTN_UNSUPPORTED, "tile-sparse attention needs a bf16 plan");
  long long nn = 0;
  int st = out ? flux_attn_validate_forward(&c, q, k, v, nullptr, segment_tokens, num_segments, pos_ids, out)
               : validate_inputs(&c, q, k, v, nullptr, segment_tokens, num_segments, pos_ids, &nn);
  if (st) return st;
  if (!mask) return fail(FLUX_ATTN_INVALID_ARGUMENT, "mask is NULL");
  int n = 0;
  for (int i = 0; i < num_segments; ++i) n += segment_tokens[i];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan was created on device %d, current device is %d", plan->device, dev);
  *n_out = n;
  return ok();
}

float plan_c(const flux_attn_config& c) {
  const float scale = c.softmax_scale > 0.0f ? c.softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
  return scale * 1.4426950408889634f;
}

}  // namespace

int flux_attn_block_mask(flux_attn_plan* plan, const void* q, const void* k, const int32_t* segment_tokens,
                         int32_t num_segments, const int32_t* pos_ids, float tau, uint8_t* mask, void* hip_stream) {
  int n = 0;
  // v and out are not used here (k stands in for v in the shared checks).
  int st = sparse_common(plan, q, k, k, segment_tokens, num_segments, pos_ids, nullptr, mask, &n);
  if (st) return st;
  if (!(tau > 0.0f && tau <= 1.0f)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "tau must be in (0, 1]");
  const flux_attn_config& c = plan->cfg;
  const int KT = (n + 63) / 64;
  if ((size_t)8 * KT * sizeof(float) > flux::kBoundMaxLds)
    return fail(FLUX_ATTN_UNSUPPORTED, "the score-bound tile mask supports at most %zu key tiles (%d tokens); got %d",
                flux::kBoundMaxLds / 32, (int)(flux::kBoundMaxLds / 32) * 64, KT);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = flux::launch_rope_table(pos_ids, plan->freq, rope16(plan), n, c.head_dim, c.rope_axes_dim[0],
                                         c.rope_axes_dim[1], stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  flux::BoundArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.rope = rope16(plan);
  a.mask = mask;
  a.n_tokens = n;
  a.batch_tokens = n;
  a.heads = c.num_heads;
  a.batch = c.batch;
  a.kt = KT;
  a.c = plan_c(c);
  a.log2_tau = std::log2(tau);
  e = flux::launch_tile_bound(a, c.head_dim, plan->num_cus, stream);
  if (e != hipSuccess) return hip_fail(e, "block mask launch");
  return ok();
}

int flux_attn_block_mask_pooled(flux_attn_plan* plan, const void* q, const void* k, const int32_t* segment_tokens,
                                int32_t num_segments, const int32_t* pos_ids, float tau, uint8_t* mask,
                                void* hip_stream) {
  int n = 0;
  int st = sparse_common(plan, q, k, k, segment_tokens, num_segments, pos_ids, nullptr, mask, &n);
  if (st) return st;
  if (!(tau > 0.0f && tau <= 1.0f)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "tau must be in (0, 1]");
  const flux_attn_config& c = plan->cfg;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  float2* const table = static_cast<float2*>(plan->rope_table);
  hipError_t e = flux::launch_rope_table_f32(pos_ids, plan->freq, table, n, c.head_dim, c.rope_axes_dim[0],
                                             c.rope_axes_dim[1], stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  const int QT = (n + 255) / 256, KT = (n + 63) / 64;
  e = flux::launch_tile_means(static_cast<const uint16_t*>(q), table, plan->qbar, n, n, c.num_heads, c.batch,
                              c.head_dim, 256, stream);
  if (e == hipSuccess)
    e = flux::launch_tile_means(static_cast<const uint16_t*>(k), table, plan->kbar, n, n, c.num_heads, c.batch,
                                c.head_dim, 64, stream);
  if (e == hipSuccess)
    e = flux::launch_block_select(plan->qbar, plan->kbar, mask, c.batch * c.num_heads * QT, QT, KT, c.head_dim,
                                  plan_c(c), std::log2(tau), stream);
  if (e != hipSuccess) return hip_fail(e, "block mask launch");
  return ok();
}

int flux_attn_forward_sparse(flux_attn_plan* plan, const void* q, const void* k, const void* v,
                             const int32_t* segment_tokens, int32_t num_segments, const int32_t* pos_ids,
                             const uint8_t* mask, void* out, void* hip_stream) {
  int n = 0;
  int st = sparse_common(plan, q, k, v, segment_tokens, num_segments, pos_ids, out, mask, &n);
  if (st) return st;
  const flux_attn_config& c = plan->cfg;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = flux::launch_rope_table(pos_ids, plan->freq, rope16(plan), n, c.head_dim, c.rope_axes_dim[0],
                                         c.rope_axes_dim[1], stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  const int QT = (n + 255) / 256, KT = (n + 63) / 64;
  const int rows = c.batch * c.num_heads * QT;
  e = flux::launch_mask_to_list(mask, plan->kv_list, plan->kv_count, rows, KT, KT, stream);
  if (e != hipSuccess) return hip_fail(e, "mask compaction launch");
  // Longest lists first: tiles run in order of kept count, so that the last
  // round is made of the shortest ones (and of the split pieces).
  const bool ordered = rows <= 32768;
  if (ordered) {
    e = flux::launch_tile_order(plan->kv_count, plan->tile_order, rows, KT, stream);
    if (e != hipSuccess) return hip_fail(e, "tile order launch");
  }
  const flux::Schedule sch = flux::plan_schedule(rows, KT, plan->num_cus, plan->max_pieces, c.head_dim);
  flux::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(out);
  a.rope = rope16(plan);
  {
    const int t0 = 0;
    set_ranges(a, &t0, &n, 1, c.batch, c.num_heads);
  }
  a.batch_tokens = n;
  a.heads = c.num_heads;
  a.batch = c.batch;
  a.c = plan_c(c);
  a.part_o = plan->part_o;
  a.part_ml = plan->part_ml;
  a.kv_list = plan->kv_list;
  a.kv_count = plan->kv_count;
  a.list_stride = KT;
  a.tile_order = ordered ? plan->tile_order : nullptr;
  const bool timed = plan->timing_used < (int)plan->ev_start.size();
  a.clk = timed ? plan->clk : nullptr;
  if (timed) {
    e = hipEventRecord(plan->ev_start[plan->timing_used], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  e = flux::launch_attn_bf16(a, c.head_dim, sch, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (timed) {
    e = hipEventRecord(plan->ev_mid[plan->timing_used], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  e = flux::launch_attn_merge(a, c.head_dim, sch, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  if (timed) {
    e = hipEventRecord(plan->ev_stop[plan->timing_used], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    ++plan->timing_used;
  }
  return ok();
}

int flux_attn_schedule(int32_t tiles, int32_t kv_tiles, int32_t num_cus, int32_t max_pieces, int32_t head_dim,
                       int32_t* whole_tiles, int32_t* split_tiles, int32_t* split, int32_t* grid) {
  if (!whole_tiles || !split_tiles || !split || !grid) return fail(FLUX_ATTN_INVALID_ARGUMENT, "output is NULL");
  if (tiles < 0 || kv_tiles < 1 || num_cus < 1 || max_pieces < 0 || (head_dim != 64 && head_dim != 128))
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "bad schedule arguments");
  const flux::Schedule s = flux::plan_schedule(tiles, kv_tiles, num_cus, max_pieces, head_dim);
  *whole_tiles = s.whole_tiles;
  *split_tiles = s.split_tiles;
  *split = s.split;
  *grid = s.grid;
  return ok();
}

int flux_attn_timing_enable(flux_attn_plan* plan, int32_t capacity) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  if (capacity < 0 || capacity > 4096)
    return fail(FLUX_ATTN_INVALID_ARGUMENT, "timing capacity %d outside [0, 4096]", capacity);
  release_timing(plan);
  if (capacity > 0) {
    hipError_t e = hipDeviceGetAttribute(&plan->wall_khz, hipDeviceAttributeWallClockRate, plan->device);
    if (e == hipSuccess) e = hipMalloc(&plan->clk, 2 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemset(plan->clk, 0, 2 * sizeof(unsigned long long));
    if (e != hipSuccess) {
      release_timing(plan);
      return hip_fail(e, "timing clock buffer");
    }
  }
  for (int i = 0; i < capacity; ++i) {
    hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
    for (int j = 0; j < 3; ++j) {
      hipError_t e = hipEventCreate(&ev[j]);
      if (e != hipSuccess) {
        for (int jj = 0; jj < j; ++jj) (void)hipEventDestroy(ev[jj]);
        release_timing(plan);
        return hip_fail(e, "hipEventCreate");
      }
    }
    plan->ev_start.push_back(ev[0]);
    plan->ev_mid.push_back(ev[1]);
    plan->ev_stop.push_back(ev[2]);
  }
  return ok();
}

int flux_attn_timing_read(flux_attn_plan* plan, float* attn_ms, float* total_ms, double* clock_mhz,
                          int32_t max_count, int32_t* count) {
  if (!plan_live(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is NULL or destroyed");
  if (!count || (max_count > 0 && !attn_ms)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "output pointer is NULL");
  *count = 0;
  const int n = plan->timing_used;
  if (n > 0) {
    hipError_t e = hipEventSynchronize(plan->ev_stop[n - 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    const int m = n < max_count ? n : max_count;
    for (int i = 0; i < m; ++i) {
      e = hipEventElapsedTime(&attn_ms[i], plan->ev_start[i], plan->ev_mid[i]);
      if (e == hipSuccess && total_ms) e = hipEventElapsedTime(&total_ms[i], plan->ev_start[i], plan->ev_stop[i]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    }
    *count = m;
  }
  if (clock_mhz) *clock_mhz = 0.0;
  if (plan->clk) {
    unsigned long long h[2] = {0, 0};
    hipError_t e = hipMemcpy(h, plan->clk, sizeof h, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemset(plan->clk, 0, sizeof h);
    if (e != hipSuccess) return hip_fail(e, "timing clock read");
    if (clock_mhz && h[1] > 0) *clock_mhz = (double)h[0] / (double)h[1] * plan->wall_khz * 1e-3;
  }
  plan->timing_used = 0;
  return ok();
}

int flux_attn_destroy(flux_attn_plan* plan) {
  if (!plan) return ok();
  {
    std::lock_guard<std::mutex> lk(g_plans_mu);
    if (!g_plans.erase(plan)) return fail(FLUX_ATTN_INVALID_ARGUMENT, "plan is not live (destroyed or foreign)");
  }
  release_timing(plan);
  (void)hipFree(plan->part_o);
  (void)hipFree(plan->part_ml);
  (void)hipFree(plan->qbar);
  (void)hipFree(plan->kbar);
  (void)hipFree(plan->kv_list);
  (void)hipFree(plan->kv_count);
  (void)hipFree(plan->tile_order);
  (void)hipFree(plan->dr);
  (void)hipFree(plan->rq);
  (void)hipFree(plan->rk);
  hipError_t e1 = hipFree(plan->rope_table);
  delete plan;
  if (e1 != hipSuccess) return hip_fail(e1, "hipFree");
  return ok();
}

}  // extern "C"
