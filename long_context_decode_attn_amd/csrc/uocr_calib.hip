// Measurement kernels (include/uocr_calib.h): a streaming read of a large
// buffer, an empty launch and a per-workgroup pull.  They give the decode
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

}  // extern "C"
