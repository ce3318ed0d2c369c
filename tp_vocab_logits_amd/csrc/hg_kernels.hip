// HIP kernels of the one-shot Lamport-mailbox logits gather, for gfx950.
//
// The method (vLLM API documentation page
// "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather",
// module description and HeadGather class description): every rank's [M, S]
// BF16 shard is pushed into row m of a [cap, V] mailbox of the current parity
// at columns r*S, with the sentinel word (+0, -0) sent as (+0, +0); the
// consumer polls each mailbox word until it is not the sentinel, copies the
// row to the [M, V] output and re-arms the mailbox. The copy can keep only the
// first `vocab` columns of each row (the padded-vocab slice taken after the
// gather, PR page "[Perf][Kimi-K3] Use the one-shot custom all-gather for TP
// logits", Purpose). The parity is chosen by the host, or read and advanced
// by the kernels themselves (device mode) so that launches replayed from a
// graph alternate it.
//
// All data movement is in 16-byte vectors (four 32-bit words). The sentinel
// test and rewrite are per 32-bit word, in registers.
//
// Work unit: a chunk = 64 * VPT consecutive vectors of one (row, rank)
// segment; wave w of a workgroup takes chunk `tile * waves + w`. Because the
// rank is uniform over the wave, the shard pointer is read with one scalar load
// from the kernel-argument table.
//
// Visibility inside one kernel. The eight XCDs of an MI355X each have their
// own L2, so a mailbox word pushed by one workgroup reaches a poller on another
// XCD only through memory-side caches or HBM. Pushes therefore use 128-bit
// stores carrying the same `sc1` cache-policy bit the compiler gives
// agent-scope atomics, and polls 128-bit `sc1` loads, so a re-read never
// returns a stale line of the poller's own L1 or L2. Calls whose rows span
// 4 GiB or more (past the 32-bit offsets of a buffer resource) use pairs of
// relaxed 64-bit agent-scope atomics instead. Every 32-bit word is written and
// read whole, and the poll tests every word of a vector.

#include "hg_internal.h"

namespace hg {

namespace {

constexpr int kWave = 64;

// Buffer-resource word 3 for raw 32-bit data on the gfx9 family (gfx950).
constexpr int kRawBufferWord3 = 0x00020000;
// Cache-policy operand of the buffer intrinsics on gfx950.
constexpr int kPolicySc1 = 16;
constexpr int kPolicyNt = 2;

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store_stream(u32x4 *p, u32x4 v) {
  __builtin_nontemporal_store(v, p);
}

// Two relaxed 64-bit atomic loads at agent scope. Each 32-bit word is read
// atomically; the four words of a vector may be read at different moments,
// which is why every word is tested.
__device__ __forceinline__ u32x4 load_agent64(const u32x4 *p) {
  uint64_t *q = reinterpret_cast<uint64_t *>(const_cast<u32x4 *>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32), static_cast<uint32_t>(b),
               static_cast<uint32_t>(b >> 32)};
}

// Two relaxed 64-bit atomic stores at agent scope.
__device__ __forceinline__ void store_agent64(u32x4 *p, u32x4 v) {
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

// The mailbox rows of one call, as a pointer and as a buffer resource
// (base = row 0 of the parity, size = the rows in use; used by the 128-bit
// coherent flavours, whose offsets are 32-bit).
struct Box {
  u32x4 *ptr;
  __amdgpu_buffer_rsrc_t rsrc;
};

__device__ __forceinline__ Box make_box(u32x4 *ptr, unsigned bytes) {
  return Box{ptr, __builtin_amdgcn_make_buffer_rsrc(ptr, 0, static_cast<int>(bytes),
                                                    kRawBufferWord3)};
}

// A pointer-only view (stores through `ptr`; the resource is never used).
__device__ __forceinline__ Box pointer_box(u32x4 *ptr) {
  return Box{ptr, __builtin_amdgcn_make_buffer_rsrc(ptr, 0, 0, kRawBufferWord3)};
}

template <int STORE>
__device__ __forceinline__ void box_store(const Box &b, long long idx, u32x4 v) {
  if constexpr (STORE == kPushAgent64) {
    store_agent64(b.ptr + idx, v);
  } else if constexpr (STORE == kPushB128Sc1) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b.rsrc, static_cast<int>(idx * 16), 0, kPolicySc1);
  } else {
    store_stream(b.ptr + idx, v);
  }
}

template <int POLL>
__device__ __forceinline__ u32x4 box_load(const Box &b, long long idx) {
  if constexpr (POLL == kPollAgent64) {
    return load_agent64(b.ptr + idx);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b128(b.rsrc, static_cast<int>(idx * 16), 0,
                                                 kPolicySc1 | kPolicyNt);
  }
}

struct ChunkPos {
  long long base;  // vector offset of the segment in a [m][vv] array
  int row, rank;
  int k0;          // first vector of the chunk inside the segment
};

__device__ __forceinline__ int udiv(int n, Divisor d) {
  return static_cast<int>((__umulhi(static_cast<unsigned>(n), d.mul) + static_cast<unsigned>(n)) >>
                          d.shift);
}

// Chunk index (wave-uniform) -> its segment and offset.
__device__ __forceinline__ ChunkPos chunk_pos(int c, const Geometry &g, int vpt) {
  const int seg = udiv(c, g.by_cps);
  const int part = c - seg * g.cps;
  const int row = udiv(seg, g.by_tp);
  const int rank = seg - row * g.tp;
  ChunkPos p;
  p.row = row;
  p.rank = rank;
  p.base = static_cast<long long>(row) * g.vv + static_cast<long long>(rank) * g.sv;
  p.k0 = part * kWave * vpt;
  return p;
}

// Push one chunk: read the shard vectors, rewrite sentinel words (REWRITE),
// store them at the segment's place in `dst` ([m][vv] vectors). A full chunk
// (the wave-uniform common case) runs without per-lane bounds tests, so the
// compiler keeps loads of the next chunk free of waits on this one's stores.
template <int VPT, bool REWRITE, int STORE, class Table>
__device__ __forceinline__ void push_chunk(const Table &sh, const Geometry &g, int c, int lane,
                                           const Box &dst) {
  const ChunkPos p = chunk_pos(c, g, VPT);
  const u32x4 *src = sh.p[p.rank] + static_cast<long long>(p.row) * g.sv + p.k0 + lane;
  const long long d = p.base + p.k0 + lane;
  if (p.k0 + kWave * VPT <= g.sv) {
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = load_stream(src + i * kWave);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      box_store<STORE>(dst, d + i * kWave, REWRITE ? rewrite_sentinel(v[i]) : v[i]);
  } else {
    const int left = g.sv - p.k0 - lane;  // vectors of this segment from this lane on
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (i * kWave < left) {
        const u32x4 v = load_stream(src + i * kWave);
        box_store<STORE>(dst, d + i * kWave, REWRITE ? rewrite_sentinel(v) : v);
      }
    }
  }
}

// One chunk's push in two halves, for a caller that has not resolved the
// destination yet: load_chunk issues the loads, store_chunk rewrites and
// stores what they returned. Lanes past a ragged segment end load nothing.
template <int VPT>
struct LoadedChunk {
  u32x4 v[VPT];
  long long d;  // mailbox vector index of lane's first vector
  int left;     // vectors of the segment from this lane on
};

template <int VPT, class Table>
__device__ __forceinline__ LoadedChunk<VPT> load_chunk(const Table &sh, const Geometry &g, int c,
                                                       int lane) {
  const ChunkPos p = chunk_pos(c, g, VPT);
  const u32x4 *src = sh.p[p.rank] + static_cast<long long>(p.row) * g.sv + p.k0 + lane;
  LoadedChunk<VPT> L;
  L.d = p.base + p.k0 + lane;
  L.left = g.sv - p.k0 - lane;
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    L.v[i] = i * kWave < L.left ? load_stream(src + i * kWave) : u32x4{0u, 0u, 0u, 0u};
  return L;
}

template <int VPT, int STORE>
__device__ __forceinline__ void store_chunk(const LoadedChunk<VPT> &L, const Box &dst) {
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    if (i * kWave < L.left) box_store<STORE>(dst, L.d + i * kWave, rewrite_sentinel(L.v[i]));
}

// Per-lane poll budget: re-reads left before the lane gives up.
struct PollBudget {
  unsigned long long spins;
  unsigned long long limit;
  bool gave_up;
};

// Re-read one vector until none of its words is the sentinel, within the
// lane's budget.
template <int POLL>
__device__ __forceinline__ u32x4 await_vec(const Box &b, long long idx, u32x4 v, unsigned *status,
                                           PollBudget &bud) {
  while (!bud.gave_up && has_sentinel(v)) {
    if (++bud.spins > bud.limit) {
      bud.gave_up = true;
      __hip_atomic_fetch_add(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    __asm__ __volatile__("" ::: "memory");  // the re-read is a new read
    v = box_load<POLL>(b, idx);
  }
  return v;
}

// Re-arm one mailbox vector with an ordinary (cached, write-back) store. The
// rows are next read by a later call, after the kernel boundary, yet a
// non-temporal re-arm made the M=256 gather about 7 % slower (66.4 against
// 61.9 us, same box, interleaved runs).
__device__ __forceinline__ void rearm_store(const Box &b, long long idx) {
  const u32x4 armed = {kSentinel, kSentinel, kSentinel, kSentinel};
  b.ptr[idx] = armed;
}

// Copy one polled vector (BF16 columns 8*cv .. 8*cv+7 of gathered row `row`)
// to the output, keeping only the columns below o.cols.
__device__ __forceinline__ void out_store(const OutRows &o, int row, int cv, u32x4 v) {
  if (o.cvec) {
    if (cv < o.cvec) store_stream(o.ptr + static_cast<long long>(row) * o.cvec + cv, v);
    return;
  }
  const int left = o.cols - cv * 8;  // columns of the row from this vector on
  if (left <= 0) return;
  unsigned short *e = reinterpret_cast<unsigned short *>(o.ptr) +
                      static_cast<long long>(row) * o.cols + static_cast<long long>(cv) * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < left) e[j] = static_cast<unsigned short>(v[j >> 1] >> (16 * (j & 1)));
}

// Poll one chunk of the mailbox until no word is the sentinel, copy it to
// the output and re-arm it.
template <int VPT, int POLL>
__device__ __forceinline__ void collect_chunk(const Geometry &g, int c, int lane, const Box &box,
                                              const OutRows &out, unsigned *status,
                                              PollBudget &bud) {
  const ChunkPos p = chunk_pos(c, g, VPT);
  const long long d = p.base + p.k0 + lane;
  const int cv = p.rank * g.sv + p.k0 + lane;  // column vector of the output row
  if (p.k0 + kWave * VPT <= g.sv) {
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = box_load<POLL>(box, d + i * kWave);
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = await_vec<POLL>(box, d + i * kWave, v[i], status, bud);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      out_store(out, p.row, cv + i * kWave, v[i]);
      rearm_store(box, d + i * kWave);
    }
  } else {
    const int left = g.sv - p.k0 - lane;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (i * kWave < left) {
        const long long idx = d + i * kWave;
        const u32x4 v = await_vec<POLL>(box, idx, box_load<POLL>(box, idx), status, bud);
        out_store(out, p.row, cv + i * kWave, v);
        rearm_store(box, idx);
      }
    }
  }
}

// A launch that completes a call (one-dimensional grid, at most kParitySlots
// waves) hands the other parity to the next launch in device mode, wave by
// wave: take_parity reads the wave's first slot, and pass_parity writes the
// other parity into the wave's slots (see kParitySlots). No other wave of the
// launch reads those slots, so a wave writes them as soon as it has read its
// own, early in the kernel, where the stores overlap the rest of its work
// (at the wave's end they added a store round trip to every M=1 call: about
// 0.3 us per gather under graph replay). The next launch on the stream, the
// only other reader, starts after this one has ended, so relaxed stores
// suffice and nothing waits on them.
struct NextParity {
  int p;      // this launch's parity
  int next;   // p ^ 1, held in a vector register
  int *slot;  // this lane's first slot, held in vector registers
};

__device__ __forceinline__ NextParity take_parity(const ParityArg &pa) {
  NextParity np;
  np.next = 0;
  np.slot = nullptr;
  if (!pa.dev) {
    np.p = pa.p;
    return np;
  }
  const int slot = pa.flip ? parity_wave(pa) * pa.per : static_cast<int>(blockIdx.x) % kParitySlots;
  np.p = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(pa.dev + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  np.slot = pa.dev + slot + (static_cast<int>(threadIdx.x) & (kWave - 1));
  if (pa.flip) {
    __asm__ __volatile__("v_mov_b32 %0, %1" : "=v"(np.next) : "s"(np.p ^ 1) : "memory");
    __asm__ __volatile__("" : "+v"(np.slot));
  }
  return np;
}

__device__ __forceinline__ void pass_parity(const ParityArg &pa, const NextParity &np) {
  if (!pa.dev || !pa.flip) return;
  const int i = parity_wave(pa);
  const int end = i == pa.last ? kParitySlots : (i + 1) * pa.per;
  // global address space, so the stores stay global rather than flat
  auto *q = (__attribute__((address_space(1))) int *)np.slot;
  for (int s = i * pa.per + (static_cast<int>(threadIdx.x) & (kWave - 1)); s < end;
       s += kWave, q += kWave)
    __hip_atomic_store(q, np.next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

__device__ __forceinline__ int waves_per_block() { return static_cast<int>(blockDim.x) / kWave; }

// Tiles of `waves` chunks (waves per block is a power of two).
__device__ __forceinline__ int tile_count(const Geometry &g, int waves) {
  const int s = __builtin_ctz(static_cast<unsigned>(waves));
  return (g.chunks + waves - 1) >> s;
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void k_arm(u32x4 *box, long long vectors, int *slots) {
  const u32x4 armed = {kSentinel, kSentinel, kSentinel, kSentinel};
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  if (slots)
    for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
         i < kParitySlots; i += stride)
      slots[i] = 0;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < vectors;
       i += stride)
    box[i] = armed;
}

// One launch does the whole gather. Phase 1: workgroup b pushes tiles
// b, b+G, b+2G, ... Phase 2: it polls, copies and re-arms the tiles pushed by
// workgroup (b - skew) mod G, a rotation, so every tile is collected exactly
// once and, with skew 1, by a workgroup on another XCD (workgroups are dealt
// to the XCDs round-robin); skew 0 collects its own tiles. No workgroup waits
// before its own push is done, and the grid is capped at the co-resident
// limit, so every workgroup whose pushes are awaited is running. Beyond that,
// only the first `skew` workgroups wait on a higher-numbered one; every other
// wait is on a workgroup dispatched earlier.
template <int VPT, int PUSH, int POLL, int NT>
__global__ __launch_bounds__(1024) void k_fused(ShardTableN<NT> sh, Geometry g, ParityArg pa,
                                                unsigned box_bytes, OutRows out, unsigned *status,
                                                unsigned long long limit, int skew) {
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = tile_count(g, waves);
  const int grid = static_cast<int>(gridDim.x);
  const int me = static_cast<int>(blockIdx.x);

  // The first chunk's loads go out before the parity is read, so that in
  // device mode the two memory latencies overlap.
  const int c0 = me * waves + wave;
  const bool first = me < tiles && c0 < g.chunks;
  LoadedChunk<VPT> L0;
  if (first) L0 = load_chunk<VPT>(sh, g, c0, lane);
  const NextParity np = take_parity(pa);
  const Box box = make_box(pa.box + np.p * pa.stride, box_bytes);
  if (first) store_chunk<VPT, PUSH>(L0, box);
  pass_parity(pa, np);

  for (int t = me + grid; t < tiles; t += grid) {
    const int c = t * waves + wave;
    if (c < g.chunks) push_chunk<VPT, true, PUSH>(sh, g, c, lane, box);
  }

  PollBudget bud{0ull, limit, false};
  // skew is in [0, grid) (the host reduces it)
  const int from = me >= skew ? me - skew : me - skew + grid;
  for (int t = from; t < tiles; t += grid) {
    const int c = t * waves + wave;
    if (c < g.chunks) collect_chunk<VPT, POLL>(g, c, lane, box, out, status, bud);
  }
}

// Split variant, first half: the push alone, by the ranks whose bit is set in
// `ranks` (visible to the next kernel on the stream at kernel end).
template <int VPT, int NT>
__global__ __launch_bounds__(1024) void k_push(ShardTableN<NT> sh, Geometry g, ParityArg pa,
                                               unsigned long long ranks) {
  u32x4 *box_ptr = pa.box + launch_parity(pa) * pa.stride;
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = tile_count(g, waves);
  const Box box = pointer_box(box_ptr);
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int c = t * waves + wave;
    if (c >= g.chunks) continue;
    const int seg = udiv(c, g.by_cps);
    const int rank = seg - udiv(seg, g.by_tp) * g.tp;
    if ((ranks >> rank) & 1ull) push_chunk<VPT, true, kPushStream>(sh, g, c, lane, box);
  }
}

// Split variant, second half: poll, copy, re-arm.
template <int VPT, int POLL>
__global__ __launch_bounds__(1024) void k_collect(Geometry g, ParityArg pa, unsigned box_bytes,
                                                  OutRows out, unsigned *status,
                                                  unsigned long long limit) {
  const NextParity np = take_parity(pa);
  pass_parity(pa, np);
  u32x4 *box_ptr = pa.box + np.p * pa.stride;
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = tile_count(g, waves);
  const Box box = make_box(box_ptr, box_bytes);
  PollBudget bud{0ull, limit, false};
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int c = t * waves + wave;
    if (c < g.chunks) collect_chunk<VPT, POLL>(g, c, lane, box, out, status, bud);
  }
}

__global__ __launch_bounds__(256) void k_set_slots(int *slots, int value) {
  for (int i = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x); i < kParitySlots;
       i += static_cast<int>(gridDim.x * blockDim.x))
    slots[i] = value;
}

// The stock path's single-device share: rank-order concatenation, bytes
// unchanged, into the first out.cols columns of each output row. Rows kept
// whole (the usual case) take the chunk copy with no per-vector column test.
template <int VPT, int NT>
__global__ __launch_bounds__(1024) void k_stock(ShardTableN<NT> sh, Geometry g, OutRows out) {
  const int waves = waves_per_block();
  const int wave = wave_id();
  const int lane = lane_id();
  const int tiles = tile_count(g, waves);
  if (out.cvec == g.vv) {
    const Box dst = pointer_box(out.ptr);
    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
      const int c = t * waves + wave;
      if (c < g.chunks) push_chunk<VPT, false, kPushStream>(sh, g, c, lane, dst);
    }
    return;
  }
  for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int c = t * waves + wave;
    if (c >= g.chunks) continue;
    const ChunkPos p = chunk_pos(c, g, VPT);
    const u32x4 *src = sh.p[p.rank] + static_cast<long long>(p.row) * g.sv + p.k0 + lane;
    const int cv = p.rank * g.sv + p.k0 + lane;
    const int left = g.sv - p.k0 - lane;
    u32x4 v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] = i * kWave < left ? load_stream(src + i * kWave) : u32x4{};
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (i * kWave < left) out_store(out, p.row, cv + i * kWave, v[i]);
  }
}

// The stock concatenation for rows that are not a whole number of 16-byte
// vectors: one 2-byte element per lane and step, out[i][j] for j < cols.
template <int NT>
__global__ __launch_bounds__(256) void k_stock_elem(ShardTableN<NT> sh, int shard, int m,
                                                    unsigned short *out, int cols) {
  const long long n = static_cast<long long>(m) * cols;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long e = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
       e += stride) {
    const long long row = e / cols;
    const int col = static_cast<int>(e - row * cols);
    const int rank = col / shard;
    const unsigned short *src = reinterpret_cast<const unsigned short *>(sh.p[rank]);
    out[e] = src[row * shard + (col - rank * shard)];
  }
}

template <int N>
using Int = std::integral_constant<int, N>;

// Vectors per lane: 1 or 2 for the mailbox kernels, also 4 for the stock copy.
template <typename F>
hipError_t by_vpt(int vpt, F &&f) {
  switch (vpt) {
    case 1: return f(Int<1>{});
    case 2: return f(Int<2>{});
    default: return hipErrorInvalidValue;
  }
}

template <typename F>
hipError_t by_stock_vpt(int vpt, F &&f) {
  switch (vpt) {
    case 1: return f(Int<1>{});
    case 2: return f(Int<2>{});
    case 4: return f(Int<4>{});
    default: return hipErrorInvalidValue;
  }
}

// Calls f with the shard table in its launch form: an 8-entry copy for up to
// 8 ranks, the full table otherwise.
template <typename F>
hipError_t by_table(const ShardTable &sh, int tp, F &&f) {
  if (tp <= kSmallTable) {
    ShardTableN<kSmallTable> t;
    for (int r = 0; r < kSmallTable; ++r) t.p[r] = sh.p[r];
    return f(t);
  }
  return f(sh);
}

// Calls f with the (push, poll) flavour pair of a launch.
template <typename F>
hipError_t by_flavour(int wide, F &&f) {
  if (wide) return f(Int<kPushAgent64>{}, Int<kPollAgent64>{});
  return f(Int<kPushB128Sc1>{}, Int<kPollB128Sc1Nt>{});
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
  g.by_cps = make_divisor(static_cast<unsigned>(g.cps));
  g.by_tp = make_divisor(static_cast<unsigned>(tp));
  return g;
}

Divisor make_divisor(unsigned d) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  Divisor r;
  r.mul = static_cast<unsigned>(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  r.shift = l;
  return r;
}

hipError_t launch_arm(u32x4 *box, long long vectors, int *slots, int grid, int block,
                      hipStream_t s) {
  hipLaunchKernelGGL(k_arm, dim3(grid), dim3(block), 0, s, box, vectors, slots);
  return hipGetLastError();
}

hipError_t launch_set_slots(int *slots, int value, hipStream_t s) {
  hipLaunchKernelGGL(k_set_slots, dim3(kParitySlots / 256), dim3(256), 0, s, slots, value);
  return hipGetLastError();
}

hipError_t launch_fused(const ShardTable &sh, const Geometry &g, const Modes &md,
                        const ParityArg &pa, unsigned box_bytes, const OutRows &out, unsigned *status,
                        unsigned long long limit, int skew, int grid, int block, hipStream_t s) {
  return by_table(sh, g.tp, [&](const auto &t) {
    constexpr int NT = sizeof(t.p) / sizeof(t.p[0]);
    return by_vpt(md.vpt, [&](auto v) {
      return by_flavour(md.wide, [&](auto pu, auto po) {
        constexpr int V = decltype(v)::value, PU = decltype(pu)::value, PO = decltype(po)::value;
        hipLaunchKernelGGL((k_fused<V, PU, PO, NT>), dim3(grid), dim3(block), 0, s, t, g, pa,
                           box_bytes, out, status, limit, skew);
        return hipGetLastError();
      });
    });
  });
}

hipError_t launch_push(const ShardTable &sh, const Geometry &g, int vpt, const ParityArg &pa,
                       unsigned long long ranks, int grid, int block, hipStream_t s) {
  return by_table(sh, g.tp, [&](const auto &t) {
    constexpr int NT = sizeof(t.p) / sizeof(t.p[0]);
    return by_vpt(vpt, [&](auto v) {
      constexpr int V = decltype(v)::value;
      hipLaunchKernelGGL((k_push<V, NT>), dim3(grid), dim3(block), 0, s, t, g, pa, ranks);
      return hipGetLastError();
    });
  });
}

hipError_t launch_collect(const Geometry &g, const Modes &md, const ParityArg &pa,
                          unsigned box_bytes, const OutRows &out, unsigned *status,
                          unsigned long long limit, int grid, int block, hipStream_t s) {
  return by_vpt(md.vpt, [&](auto v) {
    return by_flavour(md.wide, [&](auto, auto po) {
      constexpr int V = decltype(v)::value, PO = decltype(po)::value;
      hipLaunchKernelGGL((k_collect<V, PO>), dim3(grid), dim3(block), 0, s, g, pa, box_bytes, out,
                         status, limit);
      return hipGetLastError();
    });
  });
}

hipError_t launch_stock(const ShardTable &sh, const Geometry &g, int vpt, const OutRows &out,
                        int grid, int block, hipStream_t s) {
  return by_table(sh, g.tp, [&](const auto &t) {
    constexpr int NT = sizeof(t.p) / sizeof(t.p[0]);
    return by_stock_vpt(vpt, [&](auto v) {
      constexpr int V = decltype(v)::value;
      hipLaunchKernelGGL((k_stock<V, NT>), dim3(grid), dim3(block), 0, s, t, g, out);
      return hipGetLastError();
    });
  });
}

hipError_t launch_stock_elem(const ShardTable &sh, int tp, int shard, int m, unsigned short *out,
                             int cols, int grid, int block, hipStream_t s) {
  return by_table(sh, tp, [&](const auto &t) {
    constexpr int NT = sizeof(t.p) / sizeof(t.p[0]);
    hipLaunchKernelGGL((k_stock_elem<NT>), dim3(grid), dim3(block), 0, s, t, shard, m, out,
                       cols);
    return hipGetLastError();
  });
}

hipError_t fused_blocks_per_cu(const Modes &md, int tp, int block, int *blocks) {
  return by_vpt(md.vpt, [&](auto v) {
    return by_flavour(md.wide, [&](auto pu, auto po) {
      constexpr int V = decltype(v)::value, PU = decltype(pu)::value, PO = decltype(po)::value;
      const void *fn = tp <= kSmallTable
                           ? reinterpret_cast<const void *>(&k_fused<V, PU, PO, kSmallTable>)
                           : reinterpret_cast<const void *>(&k_fused<V, PU, PO, HG_MAX_TP>);
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, fn, block, 0);
    });
  });
}

}  // namespace hg
