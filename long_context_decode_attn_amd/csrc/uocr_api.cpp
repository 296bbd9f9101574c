// C ABI of libuocr.so: host-side validation, launch geometry and status codes.
// Declarations and the meaning of every argument: include/uocr.h.
#include "../../include/uocr.h"
#include "../../include/uocr_calib.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "uocr_internal.h"

// Static workspace of uocr_rswa_decode_static (see static_scratch below).
namespace {
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
}
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return UOCR_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(UOCR_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool overlap(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

constexpr int32_t kMaxPrefix = 1 << 20;
constexpr int32_t kMaxWindow = 1024;
constexpr int64_t kMaxUnits = 1 << 24;

int check_shape(const uocr_shape* sh, const char* fn) {
  if (!sh) return fail(UOCR_ERR_NULL, "%s: shape is NULL", fn);
  if (sh->dtype != UOCR_F32 && sh->dtype != UOCR_BF16)
    return fail(UOCR_ERR_DTYPE, "%s: dtype %d is neither UOCR_F32 nor UOCR_BF16", fn, sh->dtype);
  if (sh->batch < 1 || sh->heads < 1 || (int64_t)sh->batch * sh->heads > kMaxUnits)
    return fail(UOCR_ERR_SHAPE, "%s: batch %d x heads %d must be in [1, 2^24]", fn, sh->batch, sh->heads);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(UOCR_ERR_UNSUPPORTED, "%s: head_dim %d is not 64 or 128", fn, sh->head_dim);
  if (sh->prefix_cap < 0 || sh->prefix_cap > kMaxPrefix)
    return fail(UOCR_ERR_SHAPE, "%s: prefix_cap %d outside [0, 2^20]", fn, sh->prefix_cap);
  if (sh->window < 1 || sh->window > kMaxWindow)
    return fail(UOCR_ERR_SHAPE, "%s: window %d outside [1, 1024]", fn, sh->window);
  if (!std::isfinite(sh->scale)) return fail(UOCR_ERR_SHAPE, "%s: scale is not finite", fn);
  return UOCR_OK;
}

int check_route(const uocr_shape* sh, const uocr_route* r, const char* fn) {
  if (!r) return fail(UOCR_ERR_NULL, "%s: route is NULL", fn);
  if (r->block_size != uocr::kBlock)
    return fail(UOCR_ERR_UNSUPPORTED, "%s: block_size %d (only 32 is implemented)", fn, r->block_size);
  if (r->idx_dim != uocr::kIdxDim)
    return fail(UOCR_ERR_UNSUPPORTED, "%s: idx_dim %d (only 32 is implemented)", fn, r->idx_dim);
  if (r->topk < 1 || r->topk > uocr::kMaxTopk)
    return fail(UOCR_ERR_SHAPE, "%s: topk %d outside [1, 64]", fn, r->topk);
  const int nb_cap = (sh->prefix_cap + uocr::kBlock - 1) / uocr::kBlock;
  if (nb_cap > uocr::kMaxBlocks)
    return fail(UOCR_ERR_UNSUPPORTED, "%s: %d prefix blocks exceed 4096", fn, nb_cap);
  return UOCR_OK;
}

#define CHECK(x)                \
  do {                          \
    const int st_ = (x);        \
    if (st_ != UOCR_OK) return st_; \
  } while (0)

#define NEED(p, name)                                                        \
  do {                                                                       \
    if (!(p)) return fail(UOCR_ERR_NULL, "%s: %s is NULL", fn, name);        \
  } while (0)

#define ALIGN16(p, name)                                                              \
  do {                                                                                \
    if (!aligned16(p)) return fail(UOCR_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, name); \
  } while (0)

#define ALIGN4(p, name)                                                              \
  do {                                                                               \
    if (!aligned4(p)) return fail(UOCR_ERR_ALIGN, "%s: %s is not 4-byte aligned", fn, name); \
  } while (0)

int nb_cap_of(const uocr_shape* sh) { return (sh->prefix_cap + uocr::kBlock - 1) / uocr::kBlock; }
int units_of(const uocr_shape* sh) { return sh->batch * sh->heads; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

size_t ws_bytes_for(int units, int splits, int head_dim) {
  if (splits <= 1) return 0;
  return round256((size_t)units * splits * 2 * 4) + (size_t)units * splits * head_dim * 4;
}

constexpr int kDenseWaves = 4;    // waves per workgroup of the dense decode
constexpr int kSparseWaves = 8;   // waves per workgroup of the sparse decode and step (default)
constexpr int kDefaultCUs = 256;  // compute units of an MI355X, when no device answers
constexpr int kMaxCuDevices = 64;
std::mutex g_cu_mu;
int g_cus[kMaxCuDevices];

// Compute units of the current device (asked once per device); 256 when no
// device can be asked (e.g. argument queries on a host without a GPU).
int device_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxCuDevices) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  std::lock_guard<std::mutex> lock(g_cu_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = kDefaultCUs;
    }
    g_cus[dev] = n;
  }
  return g_cus[dev];
}
constexpr int kMaxPrefillQueries = 1 << 20;  // queries per unit in one prefill routing call

// Dense split geometry: workgroups per unit and keys per workgroup for the
// virtual key sequence of prefix_cap + window keys.
void rswa_geometry(const uocr_shape* sh, int32_t req, int* splits, int* chunk) {
  const int L = sh->prefix_cap + sh->window;
  const int units = units_of(sh);
  const int max_useful = (L + 63) / 64;  // at least 64 keys per workgroup
  int S;
  if (req > 0) {
    S = req;
  } else {
    // The fewest splits (longest chunks, least merging) whose workgroups
    // fill the device's CUs (256 on MI355X) and spread evenly over them: at
    // least one per CU, and the busiest CU holds no more than 1/0.93 of the mean
    // (measured: 480 workgroups stream at 80% of peak, 560 at 69%).  Chunks
    // stay >= 512 keys; failing that, aim at ~2048 workgroups.
    const int cap = (L + 511) / 512;
    const int cus = device_cus();
    S = 0;
    for (int s = 1; s <= cap && S == 0; ++s) {
      const long long n = (long long)units * s;
      const long long slots = (n + cus - 1) / cus * cus;
      if (n >= cus && n * 100 >= slots * 93) S = s;
    }
    if (S == 0) {
      const int want = (2048 + units - 1) / units;
      S = want < cap ? want : cap;
    }
  }
  if (S > max_useful) S = max_useful;
  if (S < 1) S = 1;
  int C = (L + S - 1) / S;
  C = (C + 15) / 16 * 16;
  S = (L + C - 1) / C;
  *splits = S;
  *chunk = C;
}

// Sparse decode geometry: workgroups per unit.  num_splits > 0 is taken as
// given (at most 64); 0 gives one workgroup per unit when there are as many
// units as compute units, otherwise about one workgroup per compute unit in
// all (at most 8 per unit: a unit has at most topk live blocks and the window).
int srswa_splits_of(const uocr_shape* sh, int32_t req) {
  if (req > 0) return req < 64 ? req : 64;
  const int units = units_of(sh);
  const int cus = device_cus();
  if (units >= cus) return 1;
  const int want = (cus + units - 1) / units;
  return want < 8 ? want : 8;
}

// ---------------------------------------------------------------------------
// Static workspace of uocr_rswa_decode_static: a file-scope device array.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` only stands for the array; its address on a device
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int static_scratch(const char* fn, void** ptr);

// page2d RoPE of a fused step: NULL (none) or positions + parameters
int rope_args(const char* fn, const uocr_rope* r, uocr::StepArgs& a) {
  if (!r) return UOCR_OK;
  if (!r->page || !r->offset) return fail(UOCR_ERR_NULL, "%s: rope page / offset is NULL", fn);
  if (!aligned4(r->page) || !aligned4(r->offset))
    return fail(UOCR_ERR_ALIGN, "%s: rope page / offset is not 4-byte aligned", fn);
  if (r->page_mod < 0) return fail(UOCR_ERR_SHAPE, "%s: rope page_mod %d < 0", fn, r->page_mod);
  if (!std::isfinite(r->base) || !(r->base > 0.f))
    return fail(UOCR_ERR_SHAPE, "%s: rope base is not a finite positive number", fn);
  a.rope_page = r->page;
  a.rope_offset = r->offset;
  a.rope_page_mod = r->page_mod;
  a.rope_base = r->base;
  return UOCR_OK;
}

int block_index(const char* fn, const uocr_shape* shape, const uocr_route* route, const void* k_prefix,
                const int32_t* prefix_len, const float* proj, float* kbar_idx, int32_t first_block,
                int32_t last_block, void* stream) {
  CHECK(check_shape(shape, fn));
  CHECK(check_route(shape, route, fn));
  NEED(prefix_len, "prefix_len");
  NEED(proj, "proj");
  ALIGN4(prefix_len, "prefix_len");
  ALIGN16(proj, "proj");
  const int nb_cap = nb_cap_of(shape);
  if (first_block < 0 || last_block < first_block || last_block > nb_cap)
    return fail(UOCR_ERR_SHAPE, "%s: block range [%d, %d) outside [0, %d]", fn, first_block, last_block, nb_cap);
  if (first_block == last_block) return ok();
  NEED(k_prefix, "k_prefix");
  NEED(kbar_idx, "kbar_idx");
  ALIGN16(k_prefix, "k_prefix");
  ALIGN16(kbar_idx, "kbar_idx");
  uocr::IndexArgs a{k_prefix, prefix_len, proj,        kbar_idx,    units_of(shape),
                    shape->heads, shape->prefix_cap, nb_cap, first_block, last_block - first_block};
  return hip_status(uocr::launch_block_index(shape->dtype, shape->head_dim, a,
                                             static_cast<hipStream_t>(stream)), fn);
}

// Dense decode of both entry points: the caller's workspace, or (use_static)
// the library's static one.
int rswa_decode_impl(const char* fn, const uocr_shape* shape, const void* q, const void* k_prefix,
                     const void* v_prefix, const int32_t* prefix_len, const void* k_ring,
                     const void* v_ring, const int32_t* t_gen, void* out, void* workspace,
                     size_t ws_bytes, int32_t num_splits, bool use_static, void* stream) {
  CHECK(check_shape(shape, fn));
  NEED(q, "q");
  NEED(k_ring, "k_ring");
  NEED(v_ring, "v_ring");
  NEED(t_gen, "t_gen");
  NEED(prefix_len, "prefix_len");
  NEED(out, "out");
  if (shape->prefix_cap > 0) {
    NEED(k_prefix, "k_prefix");
    NEED(v_prefix, "v_prefix");
    ALIGN16(k_prefix, "k_prefix");
    ALIGN16(v_prefix, "v_prefix");
  }
  ALIGN16(q, "q");
  ALIGN16(k_ring, "k_ring");
  ALIGN16(v_ring, "v_ring");
  ALIGN16(out, "out");
  ALIGN4(t_gen, "t_gen");
  ALIGN4(prefix_len, "prefix_len");
  if (num_splits < 0) return fail(UOCR_ERR_SHAPE, "%s: num_splits %d < 0", fn, num_splits);
  int S, C;
  rswa_geometry(shape, num_splits, &S, &C);
  const int units = units_of(shape);
  size_t need = ws_bytes_for(units, S, shape->head_dim);
  if (use_static && need > kStaticScratchBytes) {
    if (num_splits > 0)
      return fail(UOCR_ERR_WORKSPACE,
                  "%s: %d splits of %d units need a workspace of %zu bytes, above the static %zu bytes; "
                  "ask for fewer splits (0 picks a count that fits)", fn, S, units, need, kStaticScratchBytes);
    // the chosen geometry does not fit: the most splits whose partials fit
    int s_fit = S;
    while (s_fit > 1 && ws_bytes_for(units, s_fit, shape->head_dim) > kStaticScratchBytes) --s_fit;
    rswa_geometry(shape, s_fit, &S, &C);
    need = ws_bytes_for(units, S, shape->head_dim);
  }
  if (need > 0) {
    if (use_static) {
      CHECK(static_scratch(fn, &workspace));
      ws_bytes = kStaticScratchBytes;
    }
    NEED(workspace, "workspace");
    ALIGN16(workspace, "workspace");
    if (ws_bytes < need)
      return fail(UOCR_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  }
  uocr::DecodeArgs a{};
  a.q = q;
  a.k_prefix = k_prefix;
  a.v_prefix = v_prefix;
  a.prefix_len = prefix_len;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.t_gen = t_gen;
  a.out = out;
  if (need > 0) {
    a.part_ml = static_cast<float*>(workspace);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)units * S * 2 * 4));
  }
  a.units = units;
  a.heads = shape->heads;
  a.prefix_cap = shape->prefix_cap;
  a.window = shape->window;
  a.splits = S;
  a.chunk = C;
  a.waves = kDenseWaves;
  a.qscale = shape->scale * 1.4426950408889634f;
  return hip_status(uocr::launch_rswa_decode(shape->dtype, shape->head_dim, a,
                                             static_cast<hipStream_t>(stream)), fn);
}

// Address of this device's copy of `scratch`, taken on the first call on
// the device (with it current) and kept.
int static_scratch(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(UOCR_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(UOCR_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library keeps addresses for", fn, dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(UOCR_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return UOCR_OK;
}

}  // namespace

extern "C" {

const char* uocr_status_string(int status) {
  switch (status) {
    case UOCR_OK: return "ok";
    case UOCR_ERR_NULL: return "null pointer";
    case UOCR_ERR_SHAPE: return "invalid shape";
    case UOCR_ERR_DTYPE: return "invalid dtype";
    case UOCR_ERR_WORKSPACE: return "workspace missing or too small";
    case UOCR_ERR_ALIGN: return "misaligned pointer";
    case UOCR_ERR_UNSUPPORTED: return "unsupported configuration";
    case UOCR_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* uocr_last_error(void) { return g_last_error.c_str(); }

int uocr_version(void) { return UOCR_VERSION; }

int uocr_ring_append(const uocr_shape* shape, void* k_ring, void* v_ring, const void* k_new,
                     const void* v_new, int32_t* t_gen, void* stream) {
  const char* fn = "uocr_ring_append";
  CHECK(check_shape(shape, fn));
  NEED(k_ring, "k_ring");
  NEED(v_ring, "v_ring");
  NEED(k_new, "k_new");
  NEED(v_new, "v_new");
  NEED(t_gen, "t_gen");
  ALIGN16(k_ring, "k_ring");
  ALIGN16(v_ring, "v_ring");
  ALIGN16(k_new, "k_new");
  ALIGN16(v_new, "v_new");
  ALIGN4(t_gen, "t_gen");
  uocr::AppendArgs a{k_ring, v_ring, k_new, v_new, t_gen, shape->batch, shape->heads, shape->window};
  return hip_status(uocr::launch_ring_append(shape->dtype, shape->head_dim, a,
                                             static_cast<hipStream_t>(stream)), fn);
}

int32_t uocr_rswa_splits(const uocr_shape* shape, int32_t num_splits) {
  if (check_shape(shape, "uocr_rswa_splits") != UOCR_OK) return -1;
  int S, C;
  rswa_geometry(shape, num_splits, &S, &C);
  return S;
}

size_t uocr_rswa_workspace_bytes(const uocr_shape* shape, int32_t num_splits) {
  if (check_shape(shape, "uocr_rswa_workspace_bytes") != UOCR_OK) return 0;
  int S, C;
  rswa_geometry(shape, num_splits, &S, &C);
  return ws_bytes_for(units_of(shape), S, shape->head_dim);
}

int uocr_rswa_decode(const uocr_shape* shape, const void* q, const void* k_prefix,
                     const void* v_prefix, const int32_t* prefix_len, const void* k_ring,
                     const void* v_ring, const int32_t* t_gen, void* out, void* workspace,
                     size_t ws_bytes, int32_t num_splits, void* stream) {
  return rswa_decode_impl("uocr_rswa_decode", shape, q, k_prefix, v_prefix, prefix_len, k_ring, v_ring, t_gen,
                          out, workspace, ws_bytes, num_splits, false, stream);
}

int uocr_rswa_decode_static(const uocr_shape* shape, const void* q, const void* k_prefix,
                            const void* v_prefix, const int32_t* prefix_len, const void* k_ring,
                            const void* v_ring, const int32_t* t_gen, void* out, int32_t num_splits,
                            void* stream) {
  return rswa_decode_impl("uocr_rswa_decode_static", shape, q, k_prefix, v_prefix, prefix_len, k_ring, v_ring,
                          t_gen, out, nullptr, 0, num_splits, true, stream);
}

int uocr_block_index_build(const uocr_shape* shape, const uocr_route* route, const void* k_prefix,
                           const int32_t* prefix_len, const float* proj, float* kbar_idx,
                           void* stream) {
  const char* fn = "uocr_block_index_build";
  if (shape == nullptr) return fail(UOCR_ERR_NULL, "%s: shape is NULL", fn);
  return block_index(fn, shape, route, k_prefix, prefix_len, proj, kbar_idx, 0, nb_cap_of(shape), stream);
}

int uocr_block_index_range(const uocr_shape* shape, const uocr_route* route, const void* k_prefix,
                           const int32_t* prefix_len, const float* proj, float* kbar_idx,
                           int32_t first_block, int32_t last_block, void* stream) {
  return block_index("uocr_block_index_range", shape, route, k_prefix, prefix_len, proj, kbar_idx,
                     first_block, last_block, stream);
}



int uocr_block_score(const uocr_shape* shape, const uocr_route* route, const void* q,
                     const float* proj, const float* kbar_idx, const int32_t* prefix_len,
                     float* scores, void* stream) {
  const char* fn = "uocr_block_score";
  CHECK(check_shape(shape, fn));
  CHECK(check_route(shape, route, fn));
  NEED(q, "q");
  NEED(proj, "proj");
  NEED(prefix_len, "prefix_len");
  ALIGN16(q, "q");
  ALIGN16(proj, "proj");
  ALIGN4(prefix_len, "prefix_len");
  const int nb_cap = nb_cap_of(shape);
  if (nb_cap == 0) return ok();
  NEED(kbar_idx, "kbar_idx");
  NEED(scores, "scores");
  ALIGN16(kbar_idx, "kbar_idx");
  ALIGN4(scores, "scores");
  const int units = units_of(shape);
  // aim at >= 1024 workgroups, at least 64 blocks each
  int parts = (1024 + units - 1) / units;
  const int maxp = (nb_cap + 63) / 64;
  if (parts > maxp) parts = maxp;
  if (parts < 1) parts = 1;
  uocr::ScoreArgs a{q, proj, kbar_idx, prefix_len, scores, units, shape->heads,
                    shape->prefix_cap, nb_cap, parts};
  return hip_status(uocr::launch_block_score(shape->dtype, shape->head_dim, a,
                                             static_cast<hipStream_t>(stream)), fn);
}

int uocr_entmax15_topk(const uocr_shape* shape, const uocr_route* route, const float* scores,
                       const int32_t* prefix_len, int32_t* sel_idx, float* sel_prob,
                       float* sel_bias, void* stream) {
  const char* fn = "uocr_entmax15_topk";
  CHECK(check_shape(shape, fn));
  CHECK(check_route(shape, route, fn));
  NEED(prefix_len, "prefix_len");
  NEED(sel_idx, "sel_idx");
  NEED(sel_bias, "sel_bias");
  ALIGN4(prefix_len, "prefix_len");
  ALIGN4(sel_idx, "sel_idx");
  ALIGN4(sel_bias, "sel_bias");
  if (sel_prob) ALIGN4(sel_prob, "sel_prob");
  if (nb_cap_of(shape) > 0) {
    NEED(scores, "scores");
    ALIGN4(scores, "scores");
  }
  uocr::TopkArgs a{scores, prefix_len, sel_idx, sel_prob, sel_bias, units_of(shape),
                   shape->heads, shape->prefix_cap, nb_cap_of(shape), route->topk};
  return hip_status(uocr::launch_entmax_topk(a, static_cast<hipStream_t>(stream)), fn);
}

int uocr_prefill_route(const uocr_shape* shape, const uocr_route* route, const void* q, int32_t tq,
                       const int32_t* q_pos, const float* proj, const float* kbar_idx,
                       const int32_t* prefix_len, int32_t* sel_idx, float* sel_prob, float* sel_bias,
                       void* stream) {
  const char* fn = "uocr_prefill_route";
  CHECK(check_shape(shape, fn));
  CHECK(check_route(shape, route, fn));
  if (tq < 0 || tq > kMaxPrefillQueries)
    return fail(UOCR_ERR_SHAPE, "%s: tq %d outside [0, %d]", fn, tq, kMaxPrefillQueries);
  if ((long long)units_of(shape) * tq * route->topk > (1ll << 31) - 1)
    return fail(UOCR_ERR_SHAPE, "%s: units x tq x topk exceeds 2^31 - 1", fn);
  if (tq == 0) return ok();
  NEED(q, "q");
  NEED(q_pos, "q_pos");
  NEED(proj, "proj");
  NEED(prefix_len, "prefix_len");
  NEED(sel_idx, "sel_idx");
  NEED(sel_bias, "sel_bias");
  ALIGN16(q, "q");
  ALIGN4(q_pos, "q_pos");
  ALIGN4(proj, "proj");
  ALIGN4(prefix_len, "prefix_len");
  ALIGN4(sel_idx, "sel_idx");
  ALIGN4(sel_bias, "sel_bias");
  if (sel_prob) ALIGN4(sel_prob, "sel_prob");
  const int nb_cap = nb_cap_of(shape);
  if (nb_cap > 0) {
    NEED(kbar_idx, "kbar_idx");
    ALIGN16(kbar_idx, "kbar_idx");
  }
  uocr::PrefillArgs a{q, q_pos, proj, kbar_idx, prefix_len, sel_idx, sel_prob, sel_bias, units_of(shape),
                      shape->heads, shape->prefix_cap, nb_cap, route->topk, tq,
                      uocr::prefill_queries_per_wg(nb_cap)};
  return hip_status(uocr::launch_prefill_route(shape->dtype, shape->head_dim, a,
                                               static_cast<hipStream_t>(stream)), fn);
}

int uocr_ngram_ban(int32_t batch, const int32_t* tokens, int32_t ring_cap, const int32_t* n_gen,
                   const int32_t* page_tokens, int32_t ngram, int32_t window, int32_t page_token,
                   int32_t eos_token, int32_t max_page_tokens, void* logits, int32_t vocab, int32_t dtype,
                   void* stream) {
  const char* fn = "uocr_ngram_ban";
  if (batch < 0) return fail(UOCR_ERR_SHAPE, "%s: batch %d < 0", fn, batch);
  if (dtype != UOCR_F32 && dtype != UOCR_BF16) return fail(UOCR_ERR_DTYPE, "%s: dtype %d", fn, dtype);
  if (ngram < 1) return fail(UOCR_ERR_SHAPE, "%s: ngram %d < 1", fn, ngram);
  if (window < 1 || window > uocr::kMaxNgramWindow)
    return fail(UOCR_ERR_SHAPE, "%s: window %d outside [1, %d]", fn, window, uocr::kMaxNgramWindow);
  if (ring_cap < window) return fail(UOCR_ERR_SHAPE, "%s: ring_cap %d < window %d", fn, ring_cap, window);
  if (vocab < 1) return fail(UOCR_ERR_SHAPE, "%s: vocab %d < 1", fn, vocab);
  if ((long long)batch * vocab > (1ll << 40)) return fail(UOCR_ERR_SHAPE, "%s: batch x vocab too large", fn);
  if (max_page_tokens > 0) {
    NEED(page_tokens, "page_tokens");
    ALIGN4(page_tokens, "page_tokens");
    if (page_token < 0 || page_token >= vocab || eos_token < 0 || eos_token >= vocab)
      return fail(UOCR_ERR_SHAPE, "%s: page_token %d / eos_token %d outside [0, vocab)", fn, page_token,
                  eos_token);
  }
  if (batch == 0) return ok();
  NEED(tokens, "tokens");
  NEED(n_gen, "n_gen");
  NEED(logits, "logits");
  ALIGN4(tokens, "tokens");
  ALIGN4(n_gen, "n_gen");
  if (dtype == UOCR_F32) ALIGN4(logits, "logits");
  uocr::NgramArgs a{tokens, n_gen, max_page_tokens > 0 ? page_tokens : nullptr, logits, batch, ring_cap, ngram,
                    window, page_token, eos_token, max_page_tokens, vocab};
  return hip_status(uocr::launch_ngram_ban(dtype, a, static_cast<hipStream_t>(stream)), fn);
}

int uocr_rope_page2d(const uocr_shape* shape, void* x, void* y, int32_t tokens, const int32_t* page,
                     const int32_t* offset, int32_t page_mod, float base, void* stream) {
  const char* fn = "uocr_rope_page2d";
  CHECK(check_shape(shape, fn));
  if (tokens < 0 || tokens > kMaxPrefix) return fail(UOCR_ERR_SHAPE, "%s: tokens %d outside [0, 2^20]", fn, tokens);
  if (page_mod < 0) return fail(UOCR_ERR_SHAPE, "%s: page_mod %d < 0", fn, page_mod);
  if (!std::isfinite(base) || !(base > 0.f)) return fail(UOCR_ERR_SHAPE, "%s: base must be finite and > 0", fn);
  if ((int64_t)shape->batch * ((tokens + uocr::kRopeTokens - 1) / uocr::kRopeTokens) >= (int64_t(1) << 31))
    return fail(UOCR_ERR_SHAPE, "%s: batch x tokens too large", fn);
  if (tokens == 0) return ok();
  NEED(x, "x");
  NEED(page, "page");
  NEED(offset, "offset");
  ALIGN16(x, "x");
  if (y) ALIGN16(y, "y");
  ALIGN4(page, "page");
  ALIGN4(offset, "offset");
  if (y == x) return fail(UOCR_ERR_SHAPE, "%s: y is x (each tensor would be turned twice)", fn);
  uocr::RopeArgs a{x, y, page, offset, shape->batch, shape->heads, tokens, page_mod, base};
  return hip_status(uocr::launch_rope_page2d(shape->dtype, shape->head_dim, a, static_cast<hipStream_t>(stream)),
                    fn);
}

int32_t uocr_srswa_splits(const uocr_shape* shape, const uocr_route* route, int32_t num_splits) {
  if (check_shape(shape, "uocr_srswa_splits") != UOCR_OK) return -1;
  if (check_route(shape, route, "uocr_srswa_splits") != UOCR_OK) return -1;
  if (num_splits < 0) return -1;
  return srswa_splits_of(shape, num_splits);
}

size_t uocr_srswa_workspace_bytes(const uocr_shape* shape, const uocr_route* route, int32_t num_splits) {
  if (check_shape(shape, "uocr_srswa_workspace_bytes") != UOCR_OK) return 0;
  if (check_route(shape, route, "uocr_srswa_workspace_bytes") != UOCR_OK) return 0;
  if (num_splits < 0) return 0;
  return ws_bytes_for(units_of(shape), srswa_splits_of(shape, num_splits), shape->head_dim);
}

int uocr_srswa_decode(const uocr_shape* shape, const uocr_route* route, const void* q,
                      const void* k_prefix, const void* v_prefix, const int32_t* prefix_len,
                      const int32_t* sel_idx, const float* sel_bias, const void* k_ring,
                      const void* v_ring, const int32_t* t_gen, void* out, void* workspace,
                      size_t ws_bytes, int32_t num_splits, void* stream) {
  const char* fn = "uocr_srswa_decode";
  CHECK(check_shape(shape, fn));
  CHECK(check_route(shape, route, fn));
  NEED(q, "q");
  NEED(prefix_len, "prefix_len");
  NEED(sel_idx, "sel_idx");
  NEED(k_ring, "k_ring");
  NEED(v_ring, "v_ring");
  NEED(t_gen, "t_gen");
  NEED(out, "out");
  if (shape->prefix_cap > 0) {
    NEED(k_prefix, "k_prefix");
    NEED(v_prefix, "v_prefix");
    ALIGN16(k_prefix, "k_prefix");
    ALIGN16(v_prefix, "v_prefix");
  }
  ALIGN16(q, "q");
  ALIGN16(k_ring, "k_ring");
  ALIGN16(v_ring, "v_ring");
  ALIGN16(out, "out");
  ALIGN4(prefix_len, "prefix_len");
  ALIGN4(sel_idx, "sel_idx");
  ALIGN4(t_gen, "t_gen");
  if (sel_bias) ALIGN4(sel_bias, "sel_bias");
  if (num_splits < 0) return fail(UOCR_ERR_SHAPE, "%s: num_splits %d < 0", fn, num_splits);
  const int units = units_of(shape);
  const int S = srswa_splits_of(shape, num_splits);
  const size_t need = ws_bytes_for(units, S, shape->head_dim);
  if (need > 0) {
    NEED(workspace, "workspace");
    ALIGN16(workspace, "workspace");
    if (ws_bytes < need)
      return fail(UOCR_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  }
  uocr::DecodeArgs a{};
  a.q = q;
  a.k_prefix = k_prefix;
  a.v_prefix = v_prefix;
  a.prefix_len = prefix_len;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.t_gen = t_gen;
  a.out = out;
  if (need > 0) {
    a.part_ml = static_cast<float*>(workspace);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)units * S * 2 * 4));
  }
  a.units = units;
  a.heads = shape->heads;
  a.prefix_cap = shape->prefix_cap;
  a.window = shape->window;
  a.splits = S;
  a.waves = kSparseWaves;
  a.qscale = shape->scale * 1.4426950408889634f;
  a.sel_idx = sel_idx;
  a.sel_bias = sel_bias;
  a.topk = route->topk;
  return hip_status(uocr::launch_srswa_decode(shape->dtype, shape->head_dim, a,
                                              static_cast<hipStream_t>(stream)), fn);
}

int uocr_rswa_step(const uocr_shape* shape, const void* q, const void* k_new, const void* v_new,
                   const void* k_prefix, const void* v_prefix, const int32_t* prefix_len, void* k_ring,
                   void* v_ring, const int32_t* t_gen_in, int32_t* t_gen_out, void* out, void* workspace,
                   size_t ws_bytes, int32_t num_splits, const uocr_rope* rope, void* stream) {
  const char* fn = "uocr_rswa_step";
  CHECK(check_shape(shape, fn));
  NEED(q, "q");
  NEED(k_new, "k_new");
  NEED(v_new, "v_new");
  NEED(prefix_len, "prefix_len");
  NEED(k_ring, "k_ring");
  NEED(v_ring, "v_ring");
  NEED(t_gen_in, "t_gen_in");
  NEED(t_gen_out, "t_gen_out");
  NEED(out, "out");
  if (shape->prefix_cap > 0) {
    NEED(k_prefix, "k_prefix");
    NEED(v_prefix, "v_prefix");
    ALIGN16(k_prefix, "k_prefix");
    ALIGN16(v_prefix, "v_prefix");
  }
  ALIGN16(q, "q");
  ALIGN16(k_new, "k_new");
  ALIGN16(v_new, "v_new");
  ALIGN16(k_ring, "k_ring");
  ALIGN16(v_ring, "v_ring");
  ALIGN16(out, "out");
  ALIGN4(prefix_len, "prefix_len");
  ALIGN4(t_gen_in, "t_gen_in");
  ALIGN4(t_gen_out, "t_gen_out");
  if (overlap(t_gen_in, t_gen_out, (size_t)shape->batch * 4))
    return fail(UOCR_ERR_UNSUPPORTED, "%s: t_gen_out overlaps t_gen_in", fn);
  if (num_splits < 0) return fail(UOCR_ERR_SHAPE, "%s: num_splits %d < 0", fn, num_splits);
  int S, C;
  rswa_geometry(shape, num_splits, &S, &C);
  const int units = units_of(shape);
  const size_t need = ws_bytes_for(units, S, shape->head_dim);
  if (need > 0) {
    NEED(workspace, "workspace");
    ALIGN16(workspace, "workspace");
    if (ws_bytes < need)
      return fail(UOCR_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  }
  uocr::StepArgs a{};
  a.d.q = q;
  a.d.k_prefix = k_prefix;
  a.d.v_prefix = v_prefix;
  a.d.prefix_len = prefix_len;
  a.d.k_ring = k_ring;
  a.d.v_ring = v_ring;
  a.d.out = out;
  if (need > 0) {
    a.d.part_ml = static_cast<float*>(workspace);
    a.d.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)units * S * 2 * 4));
  }
  a.d.units = units;
  a.d.heads = shape->heads;
  a.d.prefix_cap = shape->prefix_cap;
  a.d.window = shape->window;
  a.d.splits = S;
  a.d.chunk = C;
  a.d.waves = kDenseWaves;
  a.d.qscale = shape->scale * 1.4426950408889634f;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.t_gen_in = t_gen_in;
  a.t_gen_out = t_gen_out;
  CHECK(rope_args(fn, rope, a));
  return hip_status(uocr::launch_rswa_step(shape->dtype, shape->head_dim, a, static_cast<hipStream_t>(stream)),
                    fn);
}

int uocr_srswa_step(const uocr_shape* shape, const uocr_route* route, const void* q, const void* k_new,
                    const void* v_new, const void* k_prefix, const void* v_prefix, const int32_t* prefix_len,
                    const float* proj, const float* kbar_idx, void* k_ring, void* v_ring,
                    const int32_t* t_gen_in, int32_t* t_gen_out, int32_t* sel_idx, float* sel_prob,
                    float* sel_bias, void* out, int32_t num_splits, const uocr_rope* rope, void* stream) {
  const char* fn = "uocr_srswa_step";
  CHECK(check_shape(shape, fn));
  CHECK(check_route(shape, route, fn));
  NEED(q, "q");
  NEED(k_new, "k_new");
  NEED(v_new, "v_new");
  NEED(prefix_len, "prefix_len");
  NEED(proj, "proj");
  NEED(k_ring, "k_ring");
  NEED(v_ring, "v_ring");
  NEED(t_gen_in, "t_gen_in");
  NEED(t_gen_out, "t_gen_out");
  NEED(sel_idx, "sel_idx");
  NEED(sel_bias, "sel_bias");
  NEED(out, "out");
  if (shape->prefix_cap > 0) {
    NEED(k_prefix, "k_prefix");
    NEED(v_prefix, "v_prefix");
    NEED(kbar_idx, "kbar_idx");
    ALIGN16(k_prefix, "k_prefix");
    ALIGN16(v_prefix, "v_prefix");
    ALIGN16(kbar_idx, "kbar_idx");
  }
  ALIGN16(q, "q");
  ALIGN16(k_new, "k_new");
  ALIGN16(v_new, "v_new");
  ALIGN16(proj, "proj");
  ALIGN16(k_ring, "k_ring");
  ALIGN16(v_ring, "v_ring");
  ALIGN16(out, "out");
  ALIGN4(prefix_len, "prefix_len");
  ALIGN4(t_gen_in, "t_gen_in");
  ALIGN4(t_gen_out, "t_gen_out");
  ALIGN4(sel_idx, "sel_idx");
  ALIGN4(sel_bias, "sel_bias");
  if (sel_prob) ALIGN4(sel_prob, "sel_prob");
  if (overlap(t_gen_in, t_gen_out, (size_t)shape->batch * 4))
    return fail(UOCR_ERR_UNSUPPORTED, "%s: t_gen_out overlaps t_gen_in", fn);
  if (num_splits != 0 && num_splits != 4 && num_splits != 8 && num_splits != 16)
    return fail(UOCR_ERR_SHAPE, "%s: num_splits %d is not 0, 4, 8 or 16", fn, num_splits);
  uocr::StepArgs a{};
  a.d.q = q;
  a.d.k_prefix = k_prefix;
  a.d.v_prefix = v_prefix;
  a.d.prefix_len = prefix_len;
  a.d.k_ring = k_ring;
  a.d.v_ring = v_ring;
  a.d.out = out;
  a.d.units = units_of(shape);
  a.d.heads = shape->heads;
  a.d.prefix_cap = shape->prefix_cap;
  a.d.window = shape->window;
  a.d.splits = 1;
  a.d.waves = num_splits != 0 ? num_splits : kSparseWaves;
  a.d.qscale = shape->scale * 1.4426950408889634f;
  a.d.topk = route->topk;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.t_gen_in = t_gen_in;
  a.t_gen_out = t_gen_out;
  a.proj = proj;
  a.kbar = kbar_idx;
  a.nb_cap = nb_cap_of(shape);
  a.sel_idx = sel_idx;
  a.sel_prob = sel_prob;
  a.sel_bias = sel_bias;
  CHECK(rope_args(fn, rope, a));
  return hip_status(uocr::launch_srswa_step(shape->dtype, shape->head_dim, a, static_cast<hipStream_t>(stream)),
                    fn);
}

int uocr_phase_stamps(uint64_t* dst, int32_t units, void* stream) {
  const char* fn = "uocr_phase_stamps";
  if (!dst) return fail(UOCR_ERR_NULL, "%s: dst is NULL", fn);
  if (units < 1 || units > uocr::kMaxStampUnits)
    return fail(UOCR_ERR_SHAPE, "%s: units %d is not in [1, %d]", fn, units, uocr::kMaxStampUnits);
  const hipError_t e = uocr::read_phase_stamps(dst, (size_t)units * 64 * sizeof(uint64_t),
                                               static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(UOCR_ERR_UNSUPPORTED, "%s: this library records no stamps (libuocr_stamps.so does)", fn);
  if (e != hipSuccess) return fail(UOCR_ERR_HIP, "%s: copy failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // extern "C"
