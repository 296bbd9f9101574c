// Measurement kernels (include/uocr_calib.h): a streaming read of a large
// buffer, an empty launch, a per-workgroup pull, the start times of a grid's
// workgroups and the cost of merging workgroups' partials inside one kernel.  They give the decode
// kernels' denominators on the machine at hand; none of them is part of the
// method.
#include "../../include/uocr_calib.h"

#include <hip/hip_runtime.h>

#include "../../include/uocr.h"

namespace {

constexpr uint32_t kNever = 0x9E3779B9u;  // a hash no buffer of the measurements produces
constexpr int kReadGroups = 4096;
constexpr int kReadThreads = 256;
constexpr int kInFlight = 8;

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ v4u32 load16(const v4u32* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ uint32_t mix(v4u32 v) { return v.x ^ (v.y * 3u) ^ (v.z * 5u) ^ (v.w * 7u); }

// Workgroup g reads the contiguous slice [g * per16, min((g + 1) * per16, n16))
// of 16-byte chunks, kInFlight loads per thread in flight before any is used
// (the access pattern of the dense decode: each workgroup streams its own
// contiguous run).
template <bool NT>
__global__ __launch_bounds__(kReadThreads) void k_calib_read(const v4u32* __restrict__ src, size_t n16,
                                                           size_t per16, uint32_t* sink) {
  const size_t lo = (size_t)blockIdx.x * per16;
  const size_t hi = lo + per16 < n16 ? lo + per16 : n16;
  const size_t stride = blockDim.x;
  size_t i = lo + threadIdx.x;
  uint32_t h = 0;
  for (; i + (kInFlight - 1) * stride < hi; i += kInFlight * stride) {
    v4u32 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = load16<NT>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) h ^= mix(v[u]);
  }
  for (; i < hi; i += stride) h ^= mix(load16<NT>(src + i));
  if (h == kNever) sink[blockIdx.x] = h;
}

__global__ void k_calib_empty() {}

// Workgroup g reads its own run of n16 chunks; each thread keeps kInFlight
// loads in flight.
template <bool NT>
__global__ __launch_bounds__(1024) void k_calib_pull(const v4u32* __restrict__ src, size_t n16, uint32_t* sink) {
  const v4u32* base = src + (size_t)blockIdx.x * n16;
  const size_t stride = blockDim.x;
  size_t i = threadIdx.x;
  uint32_t h = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    v4u32 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = load16<NT>(base + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) h ^= mix(v[u]);
  }
  for (; i < n16; i += stride) h ^= mix(load16<NT>(base + i));
  if (h == kNever) sink[blockIdx.x] = h;
}

// Start time of every workgroup (the constant-rate real-time counter, read
// by thread 0 as the workgroup begins), for the spread of start times across
// the chip.
__global__ void k_calib_start(uint64_t* stamps) {
  if (threadIdx.x == 0) stamps[blockIdx.x] = wall_clock64();
}

// Merging the partial states of `split` workgroups per unit inside one
// kernel: every workgroup writes a partial of kPart floats and adds one to
// its unit's counter; the workgroup that arrives last sums the unit's
// partials, writes out[unit] and clears the counter.  Nothing waits: the
// last to arrive does the merge.  MODE 0: plain stores and loads with a
// device-wide fence (__threadfence) before the count and after it; MODE 1:
// agent-scope relaxed atomic stores and loads of the partials, the count
// after a workgroup-scope fence (which waits for the stores); MODE 2: the
// count alone.
constexpr int kPart = 130;
template <int MODE>
__global__ __launch_bounds__(256) void k_calib_exchange(float* part, int32_t* count, float* out, int split) {
  const int unit = blockIdx.x / split, s = blockIdx.x - unit * split;
  __shared__ int last;
  float* mine = part + ((size_t)unit * split + s) * kPart;
  if constexpr (MODE != 2) {
    for (int t = threadIdx.x; t < kPart; t += blockDim.x) {
      const float v = (float)(s + 1) + (float)t;
      if constexpr (MODE == 1) __hip_atomic_store(mine + t, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else mine[t] = v;
    }
  }
  if constexpr (MODE == 0) __threadfence();
  else __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(count + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == split - 1;
  __syncthreads();
  if (!last) return;
  if constexpr (MODE == 0) __threadfence();
  for (int t = threadIdx.x; t < kPart; t += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < split; ++k) {
      const float* src = part + ((size_t)unit * split + k) * kPart + t;
      if constexpr (MODE == 1) acc += __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if constexpr (MODE == 0) acc += *src;
      else acc += 1.f;
    }
    out[(size_t)unit * kPart + t] = acc;
  }
  if (threadIdx.x == 0) __hip_atomic_store(count + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

bool threads_ok(int32_t t) { return t == 64 || t == 128 || t == 256 || t == 512 || t == 1024; }

}  // namespace

extern "C" {

int uocr_calib_read(const void* src, size_t bytes, int32_t nontemporal, uint32_t* sink, void* stream) {
  if (!src || !sink) return UOCR_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return UOCR_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return UOCR_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const v4u32* p = static_cast<const v4u32*>(src);
  const size_t n16 = bytes / 16, per16 = (n16 + kReadGroups - 1) / kReadGroups;
  if (nontemporal)
    k_calib_read<true><<<kReadGroups, kReadThreads, 0, s>>>(p, n16, per16, sink);
  else
    k_calib_read<false><<<kReadGroups, kReadThreads, 0, s>>>(p, n16, per16, sink);
  return hipGetLastError() == hipSuccess ? UOCR_OK : UOCR_ERR_HIP;
}

int uocr_calib_empty(int32_t groups, int32_t threads, void* stream) {
  if (groups < 1 || groups > (1 << 20) || !threads_ok(threads)) return UOCR_ERR_SHAPE;
  k_calib_empty<<<groups, threads, 0, static_cast<hipStream_t>(stream)>>>();
  return hipGetLastError() == hipSuccess ? UOCR_OK : UOCR_ERR_HIP;
}

int uocr_calib_pull(const void* src, size_t bytes_per_group, int32_t groups, int32_t threads,
                    int32_t nontemporal, uint32_t* sink, void* stream) {
  if (!src || !sink) return UOCR_ERR_NULL;
  if (groups < 1 || groups > (1 << 20) || !threads_ok(threads)) return UOCR_ERR_SHAPE;
  if (bytes_per_group < 16 || bytes_per_group > ((size_t)1 << 26) || bytes_per_group % 16 != 0)
    return UOCR_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return UOCR_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const v4u32* p = static_cast<const v4u32*>(src);
  if (nontemporal)
    k_calib_pull<true><<<groups, threads, 0, s>>>(p, bytes_per_group / 16, sink);
  else
    k_calib_pull<false><<<groups, threads, 0, s>>>(p, bytes_per_group / 16, sink);
  return hipGetLastError() == hipSuccess ? UOCR_OK : UOCR_ERR_HIP;
}

int uocr_calib_start(int32_t groups, int32_t threads, uint64_t* stamps, void* stream) {
  if (!stamps) return UOCR_ERR_NULL;
  if (groups < 1 || groups > (1 << 20) || !threads_ok(threads)) return UOCR_ERR_SHAPE;
  k_calib_start<<<groups, threads, 0, static_cast<hipStream_t>(stream)>>>(stamps);
  return hipGetLastError() == hipSuccess ? UOCR_OK : UOCR_ERR_HIP;
}

int uocr_calib_exchange(int32_t mode, int32_t units, int32_t split, float* part, int32_t* count, float* out,
                        void* stream) {
  if (!part || !count || !out) return UOCR_ERR_NULL;
  if (mode < 0 || mode > 2 || units < 1 || split < 1 || (int64_t)units * split > (1 << 20)) return UOCR_ERR_SHAPE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)(units * split)), b(256);
  if (mode == 0) k_calib_exchange<0><<<g, b, 0, s>>>(part, count, out, split);
  else if (mode == 1) k_calib_exchange<1><<<g, b, 0, s>>>(part, count, out, split);
  else k_calib_exchange<2><<<g, b, 0, s>>>(part, count, out, split);
  return hipGetLastError() == hipSuccess ? UOCR_OK : UOCR_ERR_HIP;
}

}  // extern "C"
