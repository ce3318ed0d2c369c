// Reference streaming kernel for the benchmark (not part of the gather's
// ABI): it moves the bytes of one gather call -- read the shards, write the
// mailbox rows, read mailbox rows back, write the output, rewrite those
// mailbox rows -- with 128-bit accesses and nothing else: no sentinel
// compare, no poll, no dependency between workgroups. Two mailbox-sized
// buffers alternate like the parities: a call writes `box_w` from the shards
// and copies `box_r` (written by the previous call) to the output, then arms
// `box_r`. The benchmark times it beside the gather on the same inputs, as
// the practical ceiling of this read/write mix on the device.
#include <hip/hip_runtime.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

__global__ __launch_bounds__(256) void k_stream_ref(const u32x4 *src, u32x4 *box_w,
                                                    u32x4 *box_r, u32x4 *out, long long n) {
  const u32x4 armed = {0x80000000u, 0x80000000u, 0x80000000u, 0x80000000u};
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  const long long first = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (long long i = first; i < n; i += stride) box_w[i] = __builtin_nontemporal_load(src + i);
  for (long long i = first; i < n; i += stride) {
    __builtin_nontemporal_store(box_r[i], out + i);
    __builtin_nontemporal_store(armed, box_r + i);
  }
}

}  // namespace

// src, box_w, box_r, out: device buffers of `vectors` 16-byte vectors each,
// 16-byte aligned, pairwise disjoint. Returns 0, or -1 for bad arguments, or
// -3 if the launch failed.
extern "C" __attribute__((visibility("default"))) int hgref_stream(
    const void *src, void *box_w, void *box_r, void *out, long long vectors, int grid,
    void *stream) {
  if (!src || !box_w || !box_r || !out || vectors < 0 || grid < 1) return -1;
  if (vectors == 0) return 0;
  hipLaunchKernelGGL(k_stream_ref, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(box_w),
                     static_cast<u32x4 *>(box_r), static_cast<u32x4 *>(out), vectors);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
