// hg_gather_static: the fused logits gather without any allocation, for
// callers that cannot call hipMalloc (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// It runs the same fused kernel as hg_gather, with the parity kept in device
// memory, but its mailbox, parity slots and poll-timeout counter live in the
// file-scope device array `scratch` below instead of a context's allocation.
// Each device holds its own copy of the array from the first call on it until
// the process ends. In host code the name `scratch` does not denote device
// memory: its address on a device comes from hipGetSymbolAddress, taken once
// per device (with that device current) on the first call there, and only that
// address is ever passed to kernels.
//
// Layout of `scratch`: [0, 256) header (word 0: poll-timeout count),
// [256, 256 + 4*16384) the device parity slots, then the mailbox: parity 0 at
// kBoxOffset, parity 1 HG_STATIC_PARITY_BYTES further on. A call of m rows of
// V = tp*shard BF16 uses rows 0..m-1 of one parity, laid out as a context's
// mailbox of that V. Every call re-arms the rows it used, so between calls the
// whole mailbox is all-sentinel whatever V the calls had.

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "hg_internal.h"

#define HG_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kHeaderBytes = 256;
constexpr size_t kBoxOffset = kHeaderBytes + 4 * static_cast<size_t>(hg::kParitySlots);
constexpr size_t kParityBytes = HG_STATIC_PARITY_BYTES;
constexpr size_t kScratchBytes = kBoxOffset + 2 * kParityBytes;
static_assert(kBoxOffset % 256 == 0, "mailbox 256-byte aligned");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr unsigned long long kPollLimit = 1ull << 24;
constexpr int kMaxDevices = 64;

// What the first call on a device sets up.
struct DeviceScratch {
  unsigned char *ptr = nullptr;  // device address of `scratch` on this device
  int cus = 0;
  int per_cu[2] = {0, 0};  // resident fused workgroups per CU at 1 and 2 vectors per lane
  bool ready = false;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

// Resolve the array's address on the current device `dev`, query the launch
// limits and arm the mailbox (with the parity slots zeroed) on `s`. Called
// with g_mu held, once per device.
int set_up(int dev, hipStream_t s, DeviceScratch *d) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &st);
  if (e != hipSuccess) return hg::record_hip_error(e, "hipStreamIsCapturing");
  if (st != hipStreamCaptureStatusNone) {
    hg::record_error("hg_gather_static: the first call on a device arms its scratch mailbox "
                     "and must not be captured");
    return HG_ESTATE;
  }
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) return hg::record_hip_error(e, "hipGetSymbolAddress(scratch)");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hg::record_hip_error(e, "hipDeviceGetAttribute");
  int per_cu[2] = {0, 0};
  for (int v = 1; v <= 2; ++v) {
    const hg::Modes md{v, 0};
    // the 8-entry and 64-entry shard tables give different kernels
    int small = 0, big = 0;
    e = hg::fused_blocks_per_cu(md, 2, hg::kBlock, &small);
    if (e == hipSuccess) e = hg::fused_blocks_per_cu(md, HG_MAX_TP, hg::kBlock, &big);
    if (e != hipSuccess) return hg::record_hip_error(e, "fused_blocks_per_cu");
    per_cu[v - 1] = small < big ? small : big;
  }
  unsigned char *base = static_cast<unsigned char *>(ptr);
  const long long vectors = static_cast<long long>(2 * kParityBytes / 16);
  e = hg::launch_arm(reinterpret_cast<hg::u32x4 *>(base + kBoxOffset), vectors,
                     reinterpret_cast<int *>(base + kHeaderBytes), 8 * cus, 256, s);
  if (e != hipSuccess) return hg::record_hip_error(e, "launch_arm(scratch)");
  d->ptr = base;
  d->cus = cus;
  d->per_cu[0] = per_cu[0];
  d->per_cu[1] = per_cu[1];
  d->ready = true;
  return HG_OK;
}

}  // namespace

HG_API int hg_gather_static(int tp, int shard, const void *const *shards, int m, void *out,
                            void *stream) {
  if (tp < 2 || tp > HG_MAX_TP || shard < 8 || shard % 8 != 0 || m < 0) return HG_EINVAL;
  const size_t row_bytes = static_cast<size_t>(tp) * shard * 2;
  if (static_cast<unsigned long long>(m) * row_bytes > kParityBytes) {
    hg::record_error("hg_gather_static: m * tp * shard * 2 bytes exceed the static mailbox "
                     "parity of HG_STATIC_PARITY_BYTES (8 MiB)");
    return HG_ESIZE;
  }
  if (m == 0) return HG_EDECLINE;
  if (!shards || !out || !aligned16(out)) return HG_EINVAL;
  hg::ShardTable table;
  memset(&table, 0, sizeof table);
  const size_t shard_bytes = static_cast<size_t>(m) * shard * 2;
  const size_t out_bytes = static_cast<size_t>(m) * row_bytes;
  for (int r = 0; r < tp; ++r) {
    const void *p = shards[r];
    if (!p || !aligned16(p) || overlaps(p, shard_bytes, out, out_bytes)) return HG_EINVAL;
    table.p[r] = static_cast<const hg::u32x4 *>(p);
  }

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hg::record_hip_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return HG_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DeviceScratch d;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_dev[dev].ready) {
      const int rc = set_up(dev, s, &g_dev[dev]);
      if (rc != HG_OK) return rc;
    }
    d = g_dev[dev];
  }

  const int vpt = hg::mailbox_vpt(static_cast<long long>(m) * tp * (shard / 8), d.cus);
  const hg::Modes md{vpt, 0};
  const hg::Geometry g = hg::make_geometry(tp, shard, m, vpt);
  const int grid = hg::fused_launch_grid(g.chunks, d.per_cu[vpt - 1], d.cus);
  if (grid < 1) return HG_EINVAL;
  const int waves = hg::kBlock / 64;
  hg::ParityArg pa;
  pa.box = reinterpret_cast<hg::u32x4 *>(d.ptr + kBoxOffset);
  pa.stride = static_cast<long long>(kParityBytes / 16);
  pa.dev = reinterpret_cast<int *>(d.ptr + kHeaderBytes);
  pa.p = 0;
  pa.flip = 1;
  pa.waves = waves;
  pa.per = hg::kParitySlots / (grid * waves);
  pa.last = grid * waves - 1;
  hg::OutRows o;
  o.ptr = static_cast<hg::u32x4 *>(out);
  o.cols = tp * shard;
  o.cvec = o.cols / 8;
  e = hg::launch_fused(table, g, md, pa, static_cast<unsigned>(m * row_bytes), o,
                       reinterpret_cast<unsigned *>(d.ptr), kPollLimit, hg::kPollSkew % grid, grid,
                       hg::kBlock, s);
  if (e != hipSuccess) return hg::record_hip_error(e, "launch_fused(static)");
  return HG_OK;
}
