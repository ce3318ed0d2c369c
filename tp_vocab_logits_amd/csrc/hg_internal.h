// Internal declarations shared by the host API (hg_api.cpp) and the kernels
// (hg_kernels.hip) of libhg.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hg.h"

namespace hg {

// One 16-byte vector: four 32-bit words = eight BF16 elements.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The sentinel word: BF16 +0 in the low half, BF16 -0 in the high half.
constexpr uint32_t kSentinel = 0x80000000u;

// Rank r's shard block: [m][shard] BF16, contiguous rows, 16-byte aligned.
struct ShardTable {
  const u32x4 *p[HG_MAX_TP];
};

// Work geometry of one launch. Work is cut into wave-sized chunks: a chunk is
// 64 * vpt consecutive vectors of one (row, rank) segment, so the rank -- and
// with it the shard pointer -- is the same for every lane of a wave.
struct Geometry {
  int tp;      // ranks
  int sv;      // vectors per shard row   (shard / 8)
  int vv;      // vectors per output row  (tp * sv); also the mailbox row stride
  int cps;     // chunks per segment      (ceil(sv / (64 * vpt)))
  int chunks;  // m * tp * cps
};

// How the push makes its mailbox stores visible to pollers in other
// workgroups of the same kernel.
enum PushMode : int {
  kPushAgentStores = 0,  // relaxed agent-scope atomic stores
  kPushPlainFence = 1,   // plain stores, one agent-scope release fence per wave
};

// Builds the geometry for m rows at `vpt` vectors per lane.
Geometry make_geometry(int tp, int shard, int m, int vpt);

// Kernel launchers. Each returns the launch status (hipGetLastError).
hipError_t launch_arm(u32x4 *box, long long vectors, int grid, int block, hipStream_t s);
hipError_t launch_fused(const ShardTable &sh, const Geometry &g, int vpt, int mode, u32x4 *box,
                        u32x4 *out, unsigned *status, unsigned long long limit, int skew,
                        int grid, int block, hipStream_t s);
hipError_t launch_push(const ShardTable &sh, const Geometry &g, int vpt, u32x4 *box,
                       unsigned long long ranks, int grid, int block, hipStream_t s);
hipError_t launch_collect(const Geometry &g, int vpt, u32x4 *box, u32x4 *out, unsigned *status,
                          unsigned long long limit, int grid, int block, hipStream_t s);
hipError_t launch_stock(const ShardTable &sh, const Geometry &g, int vpt, u32x4 *out, int grid,
                        int block, hipStream_t s);

// Resident workgroups per CU for a kernel instantiation and block size.
hipError_t fused_blocks_per_cu(int vpt, int mode, int block, int *blocks);

}  // namespace hg
