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
// Passed by value in the kernel arguments; launches for up to 8 ranks use an
// 8-entry copy, since every kernel-argument byte is written by the host at
// launch (a 64-entry table costs about a microsecond of launch time).
template <int N>
struct ShardTableN {
  const u32x4 *p[N];
};
using ShardTable = ShardTableN<HG_MAX_TP>;
constexpr int kSmallTable = 8;

// Per-rank output blocks as 32-bit words (the lm_head kernel's shard copies).
template <int N>
struct OutTableN {
  uint32_t *p[N];
};
using OutTable = OutTableN<HG_MAX_TP>;

// Work geometry of one launch. Work is cut into wave-sized chunks: a chunk is
// 64 * vpt consecutive vectors of one (row, rank) segment, so the rank -- and
// with it the shard pointer -- is the same for every lane of a wave.
// Division of n < 2^31 by an invariant d >= 1 as (umulhi(n, mul) + n) >> shift
// (Granlund and Montgomery's round-up method; exact for every such n because
// the sum cannot overflow). The multiplier and shift are made on the host.
struct Divisor {
  unsigned mul;
  int shift;
};

struct Geometry {
  int tp;      // ranks
  int sv;      // vectors per shard row   (shard / 8)
  int vv;      // vectors per output row  (tp * sv); also the mailbox row stride
  int cps;     // chunks per segment      (ceil(sv / (64 * vpt)))
  int chunks;  // m * tp * cps
  Divisor by_cps, by_tp;
};

Divisor make_divisor(unsigned d);

// How a launch makes mailbox stores visible to pollers in other workgroups of
// the same kernel, and how a poll reads the mailbox. The 128-bit flavour
// addresses the rows of a call through a buffer resource with 32-bit offsets;
// a call whose rows span 4 GiB or more takes the 64-bit atomic flavour.
enum PushMode : int {
  kPushAgent64 = 0,    // 2 x 64-bit relaxed agent-scope atomic stores
  kPushB128Sc1 = 1,    // 128-bit stores with the agent-coherence (sc1) cache policy
  kPushStream = 2,     // 128-bit non-temporal stores, visible at kernel end (split push)
};

enum PollMode : int {
  kPollAgent64 = 0,    // 2 x 64-bit relaxed agent-scope atomic loads
  kPollB128Sc1Nt = 1,  // 128-bit loads with the sc1 policy and the non-temporal hint
};

// Kernel variant of one launch.
struct Modes {
  int vpt;   // 16-byte vectors per lane per chunk: 1 or 2 (1, 2 or 4 for the stock copy)
  int wide;  // rows span 4 GiB or more: 64-bit atomic push and poll
};

// Where the copy step writes. Row i of the gathered logits goes to
// out + i * cols BF16 elements, and only its columns 0 .. cols-1 are written
// (the padded-vocab slice; cols = tp * shard is the whole row). With
// cols % 8 == 0 the rows are 16-byte aligned and take whole-vector stores
// (cvec = cols / 8); otherwise cvec = 0 and the copy stores element by element.
struct OutRows {
  u32x4 *ptr;
  int cols;
  int cvec;
};

// Device-mode parity slots. All slots hold the same parity between launches.
// In a launch that completes a call (one-dimensional grid of G workgroups of
// W waves, N = G*W at most kParitySlots), wave i = b*W + w owns the slots
// i*K .. i*K + K - 1 with K = kParitySlots / N (the last wave also the
// remainder): it reads slot i*K and then writes the other parity into all of
// its slots -- a contiguous run, so a few cache lines per wave. Every slot is
// written by exactly one wave, and the only slot a wave of that launch reads
// is one it rewrites itself after reading it; no wave waits on another. A
// launch that only reads the parity may read any slot.
constexpr int kParitySlots = 16384;

// Which mailbox parity a launch uses. Host mode (`dev` null): parity `p`,
// chosen by the host. Device mode: the launch reads the parity from the slots
// when it starts and, if `flip`, writes the other parity back at its end.
// Device mode keeps the alternation right when launches are replayed from a
// graph.
struct ParityArg {
  u32x4 *box;        // row 0 of parity 0; parity p starts at box + p * stride
  long long stride;  // 16-byte vectors per parity
  int *dev;          // kParitySlots device parity slots, or null
  int p;             // host-mode parity
  int flip;          // this launch completes a call (fused gather, collect)
  int waves;         // completing launch: waves per workgroup (W)
  int per;           // completing launch: slots per wave (K)
  int last;          // completing launch: index of the last wave (N - 1)
};

// Parity of a launch (device code).
// Index of this wave in a completing launch (the sizes come with the kernel
// arguments, so no dispatch-packet read delays the parity load).
__device__ __forceinline__ int parity_wave(const ParityArg &pa) {
  return static_cast<int>(blockIdx.x) * pa.waves +
         __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / 64);
}

// Parity of a launch that only reads it: every slot holds it.
__device__ __forceinline__ int launch_parity(const ParityArg &pa) {
  if (!pa.dev) return pa.p;
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(
      pa.dev + blockIdx.x % kParitySlots, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Builds the geometry for m rows at `vpt` vectors per lane.
Geometry make_geometry(int tp, int shard, int m, int vpt);

// Kernel launchers. Each returns the launch status (hipGetLastError).
// `box_bytes` is the size of the mailbox rows in use from `box` on (it bounds
// the 128-bit coherent accesses, which use 32-bit offsets).
// launch_arm also zeroes the kParitySlots parity slots at `slots` when
// non-null.
hipError_t launch_arm(u32x4 *box, long long vectors, int *slots, int grid, int block,
                      hipStream_t s);
// Every one of the kParitySlots parity slots := value.
hipError_t launch_set_slots(int *slots, int value, hipStream_t s);
hipError_t launch_fused(const ShardTable &sh, const Geometry &g, const Modes &md,
                        const ParityArg &pa, unsigned box_bytes, const OutRows &out, unsigned *status,
                        unsigned long long limit, int skew, int grid, int block, hipStream_t s);
hipError_t launch_push(const ShardTable &sh, const Geometry &g, int vpt, const ParityArg &pa,
                       unsigned long long ranks, int grid, int block, hipStream_t s);
hipError_t launch_collect(const Geometry &g, const Modes &md, const ParityArg &pa,
                          unsigned box_bytes, const OutRows &out, unsigned *status,
                          unsigned long long limit, int grid, int block, hipStream_t s);
// The stock concatenation into `out` (its columns below out.cols), in 16-byte
// vectors.
hipError_t launch_stock(const ShardTable &sh, const Geometry &g, int vpt, const OutRows &out,
                        int grid, int block, hipStream_t s);
// The same for shards whose rows are not a whole number of 16-byte vectors,
// element by element (2-byte units): out[i][j] for j < cols, row stride cols.
hipError_t launch_stock_elem(const ShardTable &sh, int tp, int shard, int m, unsigned short *out,
                             int cols, int grid, int block, hipStream_t s);

// The lm_head shard product X [m][hidden] @ W_r^T (W_r = w.p[r], [shard][hidden]),
// BF16 in, fp32 accumulate, BF16 out. `box` (mailbox rows of the current
// parity, [m][tp*shard] words) receives the words with the sentinel
// rewritten, when `push`; `shards_out` receives the plain BF16 shards when
// `keep`. Needs shard % 32 == 0 and hidden % 8 == 0.
hipError_t launch_lmhead(const u32x4 *x, const ShardTable &w, const OutTable &shards_out, bool keep,
                         bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                         hipStream_t s);

// Resident workgroups per CU of the fused kernel variant at a block size.
hipError_t fused_blocks_per_cu(const Modes &md, int tp, int block, int *blocks);

// Launch shape of the mailbox kernels: 256-thread workgroups, at most four
// resident per CU, one vector per lane while a phase moves at most four
// vectors per lane slot of the device, two beyond.
constexpr int kBlock = 256;
constexpr int kGridPerCu = 4;
constexpr int kPollSkew = 1;

inline int mailbox_vpt(long long vectors, int cus) {
  const long long lanes = static_cast<long long>(cus) * kBlock;
  return vectors <= 4 * lanes ? 1 : 2;
}

// Workgroups of a fused launch over `chunks` chunks: one per tile of
// kBlock/64 chunks, at most kGridPerCu per CU and never more than can be
// resident at once (every workgroup whose pushes are awaited must be
// running), nor more waves than parity slots. 0 if nothing fits.
inline int fused_launch_grid(long long chunks, int per_cu, int cus) {
  const int waves = kBlock / 64;
  const long long tiles = (chunks + waves - 1) / waves;
  long long lim = static_cast<long long>(per_cu) * cus;
  const long long want = static_cast<long long>(kGridPerCu) * cus;
  if (want < lim) lim = want;
  if (lim > kParitySlots / waves) lim = kParitySlots / waves;  // one slot per wave
  if (lim < 1) return 0;
  return static_cast<int>(tiles < lim ? tiles : lim);
}

// The library's last-error text (hg_last_error_detail): a failed HIP call
// (returns HG_EHIP), or a plain message.
int record_hip_error(hipError_t e, const char *where);
void record_error(const char *what);

}  // namespace hg
