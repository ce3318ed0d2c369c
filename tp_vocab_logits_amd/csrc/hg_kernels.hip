// HIP kernels of the one-shot Lamport-mailbox logits gather, for gfx950.
//
// The method (vLLM API documentation page
// "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather",
// module description and HeadGather class description): every rank's [M, S]
// BF16 shard is pushed into row m of a [cap, V] mailbox of the current parity
// at columns r*S, with the sentinel word (+0, -0) sent as (+0, +0); the
// consumer polls each mailbox word until it is not the sentinel, copies the
// row to the [M, V] output and re-arms the mailbox.
//
// All data movement is in 16-byte vectors (four 32-bit words). The sentinel
// test and rewrite are per 32-bit word, in registers.
//
// Work unit: a chunk = 64 * VPT consecutive vectors of one (row, rank)
// segment; wave w of a workgroup takes chunk `tile * waves + w`. Because the
// rank is uniform over the wave, the shard pointer is read with one scalar load
// from the kernel-argument table.

#include "hg_internal.h"

namespace hg {

namespace {

constexpr int kWave = 64;

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) {
  __builtin_nontemporal_store(v, p);
}

// Agent-coherent read of one vector: two relaxed 64-bit atomic loads at agent
// scope, so a re-read is never served from a stale cache line of this CU or
// this XCD. Each 32-bit word is read atomically; the four words of a vector
// may be read at different moments, which is why every word is tested.
__device__ __forceinline__ u32x4 load_agent(const u32x4 *p) {
  uint64_t *q = reinterpret_cast<uint64_t *>(const_cast<u32x4 *>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32), static_cast<uint32_t>(b),
               static_cast<uint32_t>(b >> 32)};
}

// Agent-coherent write of one vector: two relaxed 64-bit atomic stores at
// agent scope (visible to agent-scope loads of other workgroups without a
// fence).
__device__ __forceinline__ void store_agent(u32x4 *p, u32x4 v) {
  uint64_t *q = reinterpret_cast<uint64_t *>(p);
  __hip_atomic_store(q, static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ u32x4 rewrite_sentinel(u32x4 v) {
  v.x = v.x == kSentinel ? 0u : v.x;
  v.y = v.y == kSentinel ? 0u : v.y;
  v.z = v.z == kSentinel ? 0u : v.z;
  v.w = v.w == kSentinel ? 0u : v.w;
  return v;
}

__device__ __forceinline__ bool has_sentinel(u32x4 v) {
  return (v.x == kSentinel) | (v.y == kSentinel) | (v.z == kSentinel) | (v.w == kSentinel);
}

struct ChunkPos {
  long long base;  // vector offset of the segment in a [m][vv] array
  int row, rank;
  int k0;          // first vector of the chunk inside the segment
};

// Chunk index (wave-uniform) -> its segment and offset.
__device__ __forceinline__ ChunkPos chunk_pos(int c, const Geometry &g, int vpt) {
  const int seg = c / g.cps;
  const int part = c - seg * g.cps;
  const int row = seg / g.tp;
  const int rank = seg - row * g.tp;
  ChunkPos p;
  p.row = row;
  p.rank = rank;
  p.base = static_cast<long long>(row) * g.vv + static_cast<long long>(rank) * g.sv;
  p.k0 = part * kWave * vpt;
  return p;
}

// Store flavours for the push / copy side.
enum Store : int { kStoreAgent = 0, kStorePlain = 1, kStoreStream = 2 };

// Push one chunk: read the shard vectors, rewrite sentinel words (REWRITE),
// store them at the segment's place in `dst` ([m][vv] vectors). A full chunk
// (the wave-uniform common case) runs without per-lane bounds tests, so the
// compiler keeps loads of the next chunk free of waits on this one's stores.
template <int STORE>
__device__ __forceinline__ void store_vec(u32x4 *p, u32x4 w) {
  if (STORE == kStoreAgent) {
    store_agent(p, w);
  } else if (STORE == kStorePlain) {
    *p = w;
  } else {
    store_stream(p, w);
  }
}

template <int VPT, bool REWRITE, int STORE>
__device__ __forceinline__ void push_chunk(const ShardTable &sh, const Geometry &g, int c, int lane,
                                           u32x4 *dst) {
  const ChunkPos p = chunk_pos(c, g, VPT);
  const u32x4 *src = sh.p[p.rank] + static_cast<long long>(p.row) * g.sv + p.k0 + lane;
  u32x4 *d = dst + p.base + p.k0 + lane;
  if (p.k0 + kWave * VPT <= g.sv) {
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = load_stream(src + i * kWave);
#pragma unroll
    for (int i = 0; i < VPT; ++i) store_vec<STORE>(d + i * kWave, REWRITE ? rewrite_sentinel(v[i]) : v[i]);
  } else {
    const int left = g.sv - p.k0 - lane;  // vectors of this segment from this lane on
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (i * kWave < left) {
        const u32x4 v = load_stream(src + i * kWave);
        store_vec<STORE>(d + i * kWave, REWRITE ? rewrite_sentinel(v) : v);
      }
    }
  }
}

// Per-lane poll budget: re-reads left before the lane gives up.
struct PollBudget {
  unsigned long long spins;
  unsigned long long limit;
  bool gave_up;
};

// Re-read one vector until none of its words is the sentinel, within the
// lane's budget.
__device__ __forceinline__ u32x4 await_vec(const u32x4 *p, u32x4 v, unsigned *status,
                                           PollBudget &b) {
  while (!b.gave_up && has_sentinel(v)) {
    if (++b.spins > b.limit) {
      b.gave_up = true;
      __hip_atomic_fetch_add(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    v = load_agent(p);
  }
  return v;
}

// Poll one chunk of the mailbox until no word is the sentinel, copy it to
// `out` and re-arm it.
template <int VPT>
__device__ __forceinline__ void collect_chunk(const Geometry &g, int c, int lane, u32x4 *box,
                                              u32x4 *out, unsigned *status, PollBudget &b) {
  const ChunkPos p = chunk_pos(c, g, VPT);
  u32x4 *bx = box + p.base + p.k0 + lane;
  u32x4 *o = out + p.base + p.k0 + lane;
  const u32x4 armed = {kSentinel, kSentinel, kSentinel, kSentinel};
  if (p.k0 + kWave * VPT <= g.sv) {
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = load_agent(bx + i * kWave);
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = await_vec(bx + i * kWave, v[i], status, b);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      store_stream(o + i * kWave, v[i]);
      bx[i * kWave] = armed;
    }
  } else {
    const int left = g.sv - p.k0 - lane;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (i * kWave < left) {
        const u32x4 v = await_vec(bx + i * kWave, load_agent(bx + i * kWave), status, b);
        store_stream(o + i * kWave, v);
        bx[i * kWave] = armed;
      }
    }
  }
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

__device__ __forceinline__ int waves_per_block() { return static_cast<int>(blockDim.x) / kWave; }

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void k_arm(u32x4 *box, long long vectors) {
  const u32x4 armed = {kSentinel, kSentinel, kSentinel, kSentinel};
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < vectors;
       i += stride)
    box[i] = armed;
}

// One launch does the whole gather. Phase 1: workgroup b pushes tiles
// b, b+G, b+2G, ... Phase 2: it polls, copies and re-arms the tiles pushed by
// workgroup b-skew (its own for b < skew). Every wait is thus on a workgroup
// with a lower index, which the dispatcher started earlier and whose push
// never waits on anything; the grid is also capped at the co-resident limit.
template <int VPT, int MODE>
__global__ __launch_bounds__(1024) void k_fused(ShardTable sh, Geometry g, u32x4 *box, u32x4 *out,
                                                unsigned *status, unsigned long long limit,
                                                int skew) {
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = (g.chunks + waves - 1) / waves;
  const int grid = static_cast<int>(gridDim.x);
  const int me = static_cast<int>(blockIdx.x);

  for (int t = me; t < tiles; t += grid) {
    const int c = t * waves + wave;
    if (c < g.chunks)
      push_chunk<VPT, true, MODE == kPushAgentStores ? kStoreAgent : kStorePlain>(sh, g, c, lane,
                                                                                   box);
  }
  if (MODE == kPushPlainFence) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");

  PollBudget b{0ull, limit, false};
  const int from = me >= skew ? me - skew : me;
  for (int t = from; t < tiles; t += grid) {
    const int c = t * waves + wave;
    if (c < g.chunks) collect_chunk<VPT>(g, c, lane, box, out, status, b);
  }
}

// Split variant, first half: the push alone, by the ranks whose bit is set in
// `ranks` (visible to the next kernel on the stream at kernel end).
template <int VPT>
__global__ __launch_bounds__(1024) void k_push(ShardTable sh, Geometry g, u32x4 *box,
                                               unsigned long long ranks) {
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = (g.chunks + waves - 1) / waves;
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int c = t * waves + wave;
    if (c >= g.chunks) continue;
    const int rank = (c / g.cps) % g.tp;
    if ((ranks >> rank) & 1ull) push_chunk<VPT, true, kStoreStream>(sh, g, c, lane, box);
  }
}

// Split variant, second half: poll, copy, re-arm.
template <int VPT>
__global__ __launch_bounds__(1024) void k_collect(Geometry g, u32x4 *box, u32x4 *out,
                                                  unsigned *status, unsigned long long limit) {
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = (g.chunks + waves - 1) / waves;
  PollBudget b{0ull, limit, false};
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int c = t * waves + wave;
    if (c < g.chunks) collect_chunk<VPT>(g, c, lane, box, out, status, b);
  }
}

// The stock path's single-device share: rank-order concatenation, bytes
// unchanged.
template <int VPT>
__global__ __launch_bounds__(1024) void k_stock(ShardTable sh, Geometry g, u32x4 *out) {
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = (g.chunks + waves - 1) / waves;
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int c = t * waves + wave;
    if (c < g.chunks) push_chunk<VPT, false, kStoreStream>(sh, g, c, lane, out);
  }
}

template <typename F>
hipError_t by_vpt(int vpt, F &&f) {
  switch (vpt) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

Geometry make_geometry(int tp, int shard, int m, int vpt) {
  Geometry g;
  g.tp = tp;
  g.sv = shard / 8;
  g.vv = tp * g.sv;
  const int per_chunk = kWave * vpt;
  g.cps = (g.sv + per_chunk - 1) / per_chunk;
  g.chunks = m * tp * g.cps;
  return g;
}

hipError_t launch_arm(u32x4 *box, long long vectors, int grid, int block, hipStream_t s) {
  hipLaunchKernelGGL(k_arm, dim3(grid), dim3(block), 0, s, box, vectors);
  return hipGetLastError();
}

hipError_t launch_fused(const ShardTable &sh, const Geometry &g, int vpt, int mode, u32x4 *box,
                        u32x4 *out, unsigned *status, unsigned long long limit, int skew,
                        int grid, int block, hipStream_t s) {
  return by_vpt(vpt, [&](auto v) {
    constexpr int V = decltype(v)::value;
    if (mode == kPushPlainFence)
      hipLaunchKernelGGL((k_fused<V, kPushPlainFence>), dim3(grid), dim3(block), 0, s, sh, g, box,
                         out, status, limit, skew);
    else
      hipLaunchKernelGGL((k_fused<V, kPushAgentStores>), dim3(grid), dim3(block), 0, s, sh, g,
                         box, out, status, limit, skew);
    return hipGetLastError();
  });
}

hipError_t launch_push(const ShardTable &sh, const Geometry &g, int vpt, u32x4 *box,
                       unsigned long long ranks, int grid, int block, hipStream_t s) {
  return by_vpt(vpt, [&](auto v) {
    constexpr int V = decltype(v)::value;
    hipLaunchKernelGGL((k_push<V>), dim3(grid), dim3(block), 0, s, sh, g, box, ranks);
    return hipGetLastError();
  });
}

hipError_t launch_collect(const Geometry &g, int vpt, u32x4 *box, u32x4 *out, unsigned *status,
                          unsigned long long limit, int grid, int block, hipStream_t s) {
  return by_vpt(vpt, [&](auto v) {
    constexpr int V = decltype(v)::value;
    hipLaunchKernelGGL((k_collect<V>), dim3(grid), dim3(block), 0, s, g, box, out, status, limit);
    return hipGetLastError();
  });
}

hipError_t launch_stock(const ShardTable &sh, const Geometry &g, int vpt, u32x4 *out, int grid,
                        int block, hipStream_t s) {
  return by_vpt(vpt, [&](auto v) {
    constexpr int V = decltype(v)::value;
    hipLaunchKernelGGL((k_stock<V>), dim3(grid), dim3(block), 0, s, sh, g, out);
    return hipGetLastError();
  });
}

hipError_t fused_blocks_per_cu(int vpt, int mode, int block, int *blocks) {
  return by_vpt(vpt, [&](auto v) {
    constexpr int V = decltype(v)::value;
    const void *fn = mode == kPushPlainFence
                         ? reinterpret_cast<const void *>(&k_fused<V, kPushPlainFence>)
                         : reinterpret_cast<const void *>(&k_fused<V, kPushAgentStores>);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, fn, block, 0);
  });
}

}  // namespace hg
