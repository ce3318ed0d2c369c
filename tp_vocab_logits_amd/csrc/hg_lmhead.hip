// The vocab-parallel lm_head shard product that feeds the gather, on gfx950
// matrix cores, with its epilogue pushing straight into the mailbox.
//
// What it computes (vLLM API documentation page
// "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather",
// module description: the lm_head's [M, V/TP] shards are what the gather
// collects; install_logits_gather takes the shard width from the head
// weight's first dimension): for every rank r, shard_r = X @ W_r^T with
// X [M, H] and W_r [S, H] in BF16, accumulated in fp32 and rounded to BF16
// (round to nearest even). The vLLM PR "[Perf][Kimi-K3] Use the one-shot
// custom all-gather for TP logits" (Test Result) has the gather overlap the
// tail of this GEMM; here the GEMM's epilogue performs the push itself.
//
// Variants (selected by the `variant` argument): the default is
// k_lmhead_n320b -- 256 x 320 output tiles, eight waves of 64 x 160,
// buffer loads straight into LDS, and at small M the waves with no row below
// M only load. The others below are the measured alternatives, kept
// selectable: register-staged loads (k_lmhead), direct loads into LDS with
// 256 columns (k_lmhead_dma, k_lmhead_dma2), four waves of 128 x 128
// (k_lmhead_w4) and 320 columns with the global-address loads (k_lmhead_n320).
//
// Work decomposition of the first: a workgroup of 2*NCP waves owns a 256-row x 64*NCP
// column output tile (all of M = 256 at once); wave w computes rows
// 128*(w%2) .. +128 and columns 64*(w/2) .. +64 as 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16. Per 64-wide K step both operand tiles -- X
// [256 x 64] and the weight rows [64*NCP x 64] -- are staged in LDS (two
// stages, rows padded by 16 bytes against bank conflicts). Global loads are
// fully coalesced (eight lanes cover one 128-byte row segment) and run one K
// step ahead of the matrix cores through registers.
//
// K order: lane l supplies 8 consecutive K elements per MFMA. Per 32-wide
// slice of K, the first MFMA takes offsets 0-7 (lanes 0-31) and 16-23 (lanes
// 32-63), the second 8-15 and 24-31; slices follow in order. A and B use the
// same assignment, so every product X[m,k] * W[n,k] is summed exactly once,
// and every variant below performs the same sequence of MFMAs (same bits).

#include "hg_internal.h"

namespace hg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kTM = 256;
// Buffer-resource word 3 for raw 32-bit data on gfx950, and the non-temporal
// cache-policy bit of the buffer intrinsics.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kPolicyNt = 2;
constexpr int kTK = 64;
constexpr int kLdsRow = kTK + 8;  // BF16 per LDS row: 64 + 16-byte pad

__device__ __forceinline__ u32x4 load_stream(const u32x4 *p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

// Swap a 32-bit value with the neighbouring lane (0<->1, 2<->3, ...).
__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF, true));
}

template <int NT, int NCP, bool PUSH, bool KEEP>
__global__ __launch_bounds__(NCP * 128) void k_lmhead(const u32x4 *x, ShardTableN<NT> w,
                                                      OutTableN<NT> shards_out, ParityArg pa,
                                                      int m, int hidden, int shard, int vocab) {
  constexpr int kThreads = NCP * 128;
  constexpr int kTN = 64 * NCP;
  constexpr int kStage = (kTM + kTN) * kLdsRow;      // BF16 per LDS stage
  constexpr int kXLoads = kTM * 8 / kThreads;        // 16-byte loads per thread per step
  constexpr int kWLoads = kTN * 8 / kThreads;
  constexpr int kLoads = kXLoads + kWLoads;
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * kStage];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mh = wave & 1;   // row half of the tile
  const int nq = wave >> 1;  // 64-column group of the tile
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;  // 16-byte vectors per X / W row
  const int steps = (hidden + kTK - 1) / kTK;
  const int seg = tid & 7;     // 16-byte segment of a 128-byte row step

  // Staging loads: load q of thread t covers LDS row (q*kThreads + t)/8 of the
  // stage, segment t%8. Rows 0..255 are X rows, the rest weight rows; the
  // split falls between loads, and a wave's 8 weight rows lie in one rank
  // (shard % 32 == 0), so the rank is uniform per wave and load.
  int xoff[kXLoads];
  bool xok[kXLoads];
#pragma unroll
  for (int q = 0; q < kXLoads; ++q) {
    const int row = (q * kThreads + tid) >> 3;
    xok[q] = m0 + row < m;
    xoff[q] = (xok[q] ? (m0 + row) * hv : 0) + seg;
  }
  const u32x4 *wbase[kWLoads];
  int woff[kWLoads];
  bool wok[kWLoads];
#pragma unroll
  for (int q = 0; q < kWLoads; ++q) {
    const int wrow = ((q * kThreads + tid) >> 3);  // 0 .. kTN-1
    const int n = n0 + wrow;
    const int n_wave = __builtin_amdgcn_readfirstlane(n0 + ((q * kThreads + wave * kWave) >> 3));
    wok[q] = n < vocab;
    const int r = n_wave < vocab ? n_wave / shard : 0;
    wbase[q] = w.p[r];
    woff[q] = (wok[q] ? (n - r * shard) * hv : 0) + seg;
  }

  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 P[kLoads];

  auto load_step = [&](int kb) {
    const int kv = kb * 8;
    const bool kok = kv + seg < hv;
#pragma unroll
    for (int q = 0; q < kXLoads; ++q) {
      const bool ok = kok && xok[q];
      const u32x4 v = x[ok ? xoff[q] + kv : 0];
      P[q] = ok ? v : zero;
    }
#pragma unroll
    for (int q = 0; q < kWLoads; ++q) {
      const bool ok = kok && wok[q];
      const u32x4 v = load_stream(wbase[q] + (ok ? woff[q] + kv : 0));
      P[kXLoads + q] = ok ? v : zero;
    }
  };
  auto store_step = [&](int stage) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int row = (q * kThreads + tid) >> 3;
      *reinterpret_cast<u32x4 *>(&lds[stage * kStage + row * kLdsRow + seg * 8]) = P[q];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[i][cb] = f32x16{};

  // Pipeline: LDS stage kb%2 holds step kb while the registers carry step kb+1.
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int kb = 0; kb < steps; ++kb) {
    const int stage = kb & 1;
    const bool more = kb + 1 < steps;
    if (more) load_step(kb + 1);
    const __bf16 *sa = &lds[stage * kStage];
    const __bf16 *sb = &lds[stage * kStage + kTM * kLdsRow];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // The same K order as the direct-to-LDS variant (two 32-wide halves of
      // the step in turn), so every variant issues the same MFMA sequence.
      const int koff = 32 * (j >> 1) + 16 * half + 8 * (j & 1);
      bf16x8 b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        b[cb] = *reinterpret_cast<const bf16x8 *>(&sb[(64 * nq + 32 * cb + l32) * kLdsRow + koff]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8 *>(&sa[(128 * mh + 32 * i + l32) * kLdsRow + koff]);
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[1], acc[i][1], 0, 0, 0);
      }
    }
    if (more) store_step(stage ^ 1);
    __syncthreads();
  }

  // Epilogue. In a 32x32 accumulator block, lane l holds column l % 32 and
  // rows 8q + 4*(l/32) + t (q, t = 0..3) in element 4q + t. Two neighbouring
  // lanes (columns 2k, 2k+1) exchange halves so that each lane owns whole
  // 32-bit words -- the unit of the sentinel test: the even lane the words of
  // rows t = 0, 2, the odd lane those of rows t = 1, 3.
  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c0 = n0 + 64 * nq + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);  // even column of this lane's word
    const int wcol = s_even >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[i][cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 128 * mh + 32 * i + 8 * q + 4 * half;
        const int row0 = rbase + (even ? 0 : 1);
        const int row1 = rbase + (even ? 2 : 3);
        if (row0 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row0) * words_per_shard_row + wcol] = w0;
          if (PUSH)
            box[static_cast<long long>(row0) * words_per_row + (r * shard >> 1) + wcol] =
                w0 == kSentinel ? 0u : w0;
        }
        if (row1 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row1) * words_per_shard_row + wcol] = w1;
          if (PUSH)
            box[static_cast<long long>(row1) * words_per_row + (r * shard >> 1) + wcol] =
                w1 == kSentinel ? 0u : w1;
        }
      }
    }
  }
}

// Variant with direct global -> LDS loads (gfx950 global_load_lds_dwordx4):
// no register staging, so more K steps can be in flight. K step KS (32 or 64
// elements: 4 or 8 slots of 16 bytes per row), ST LDS stages of [256 X rows +
// 256 weight rows], loads issued ST-1 steps ahead. A wave's load instruction
// fills 1 KB of LDS contiguously, lane-major (1024/(2*KS) rows of 2*KS
// bytes); the lane owning slot s of a row loads the row's K segment
// s ^ swz(row), so the stored layout is XOR-swizzled and the fragment reads (8
// or 16 consecutive rows, one K segment) hit distinct banks. WNT marks the
// weight loads non-temporal (streamed once).
template <int KS>
__device__ __forceinline__ int dswz(int row) {
  // Measured with SQ_LDS_BANK_CONFLICT on the fragment reads: 128-byte rows
  // read in 4 cycles per instruction with no conflicts; 64-byte rows in 6,
  // also with no conflicts (the earlier ((row >> 1) ^ (row >> 3)) & 3 took 8,
  // a quarter of them conflict cycles).
  if constexpr (KS == 32)
    return (row ^ (row >> 2)) & 3;
  else
    return (row ^ (row >> 3)) & 7;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N) (N < 64) without waiting on LDS or export counters
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

template <int NT, int KS, int ST, bool WNT, bool PUSH, bool KEEP>
__global__ __launch_bounds__(512) void k_lmhead_dma(const u32x4 *x, ShardTableN<NT> w,
                                                    OutTableN<NT> shards_out, ParityArg pa, int m,
                                                    int hidden, int shard, int vocab) {
  constexpr int kTN = 256;
  constexpr int kRowBytes = KS * 2;
  constexpr int kSlots = KS / 8;                   // 16-byte slots per row
  constexpr int kRowsPerInst = 1024 / kRowBytes;   // rows one wave instruction fills
  constexpr int kStageBytes = 512 * kRowBytes;
  constexpr int kInst = 512 / (8 * kRowsPerInst);  // instructions per wave per step
  constexpr int kXInst = kInst / 2;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ST * kStageBytes];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mh = wave & 1;
  const int nq = wave >> 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;

  // Instruction q of wave w fills stage rows kRowsPerInst*(8q+w) .. : the
  // first kXInst instructions X rows, the rest weight rows.
  const int lrow = lane / kSlots, lslot = lane % kSlots;
  const u32x4 *src[kInst];
  bool ok[kInst];
  int seg[kInst];
#pragma unroll
  for (int q = 0; q < kInst; ++q) {
    const int srow = kRowsPerInst * (8 * q + wave) + lrow;  // stage row
    seg[q] = lslot ^ dswz<KS>(srow);
    if (q < kXInst) {
      const int row = srow;
      ok[q] = m0 + row < m;
      src[q] = x + static_cast<long long>(ok[q] ? m0 + row : 0) * hv;
    } else {
      const int row = srow - 256;
      const int n = n0 + row;
      const int n_wave = __builtin_amdgcn_readfirstlane(n0 + kRowsPerInst * (8 * q + wave) - 256);
      ok[q] = n < vocab;
      const int r = n_wave < vocab ? n_wave / shard : 0;
      src[q] = w.p[r] + static_cast<long long>(ok[q] ? n - r * shard : 0) * hv;
    }
  }
  // A lane whose row is out of range (or whose K segment is past `hidden`)
  // loads from a valid address; its slot is cleared before use.
  auto issue = [&](int kb) {
    const int stage = kb % ST;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int kv = kb * kSlots + seg[q];
      const u32x4 *p = src[q] + (ok[q] && kv < hv ? kv : 0);
      __attribute__((address_space(3))) void *dst =
          (__attribute__((address_space(3))) void *)(lds + stage * kStageBytes +
                                                     kRowsPerInst * (8 * q + wave) * kRowBytes);
      if (q >= kXInst && WNT)
        __builtin_amdgcn_global_load_lds(p, dst, 16, 0, 2 /* nt */);
      else
        __builtin_amdgcn_global_load_lds(p, dst, 16, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[i][cb] = f32x16{};

  const bool tails = hidden % KS != 0 || m0 + kTM > m;
  for (int p = 0; p < ST - 1 && p < steps; ++p) issue(p);
  for (int kb = 0; kb < steps; ++kb) {
    // Wait for this wave's loads of step kb; later steps stay in flight.
    const int left = steps - 1 - kb;
    if (ST >= 4 && left >= 2)
      wait_vm<(ST >= 4 ? 2 : 0) * kInst>();
    else if (ST >= 3 && left >= 1)
      wait_vm<kInst>();
    else
      wait_vm<0>();
    // Every wave's part of step kb is in LDS once all waves pass the
    // barrier. A plain s_barrier: __syncthreads() would also wait for the
    // later steps' loads still in flight.
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    const int stage = kb % ST;
    unsigned char *sbase = lds + stage * kStageBytes;
    if (tails) {
#pragma unroll
      for (int q = 0; q < kInst; ++q) {
        const int kv = kb * kSlots + seg[q];
        if (!(ok[q] && kv < hv))
          *reinterpret_cast<u32x4 *>(sbase + (kRowsPerInst * (8 * q + wave) + lrow) * kRowBytes +
                                     lslot * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (ST > 1 && kb + ST - 1 < steps) issue(kb + ST - 1);
#pragma unroll
    for (int j = 0; j < KS / 16; ++j) {
      // K segment of this lane for MFMA j: 32-wide slice j/2, half, j%2.
      const int g = 4 * (j >> 1) + 2 * half + (j & 1);
      bf16x8 b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int row = 256 + 64 * nq + 32 * cb + l32;
        b[cb] = *reinterpret_cast<const bf16x8 *>(sbase + row * kRowBytes +
                                                   ((g ^ dswz<KS>(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 128 * mh + 32 * i + l32;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sbase + row * kRowBytes +
                                                            ((g ^ dswz<KS>(row)) << 4));
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[1], acc[i][1], 0, 0, 0);
      }
    }
    if (ST == 1) {
      // single stage: the next step may overwrite only after every wave read
      __syncthreads();
      if (kb + 1 < steps) issue(kb + 1);
    }
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c0 = n0 + 64 * nq + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[i][cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 128 * mh + 32 * i + 8 * q + 4 * half;
        const int row0 = rbase + (even ? 0 : 1);
        const int row1 = rbase + (even ? 2 : 3);
        if (row0 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row0) * words_per_shard_row + wcol] = w0;
          if (PUSH)
            box[static_cast<long long>(row0) * words_per_row + (r * shard >> 1) + wcol] =
                w0 == kSentinel ? 0u : w0;
        }
        if (row1 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row1) * words_per_shard_row + wcol] = w1;
          if (PUSH)
            box[static_cast<long long>(row1) * words_per_row + (r * shard >> 1) + wcol] =
                w1 == kSentinel ? 0u : w1;
        }
      }
    }
  }
}

template <int NT, int NCP>
hipError_t launch_lmhead_nt(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                            bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                            hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  constexpr int kTN = 64 * NCP;
  const dim3 grid((vocab + kTN - 1) / kTN, (m + kTM - 1) / kTM);
  const dim3 block(NCP * 128);
  if (push && keep)
    hipLaunchKernelGGL((k_lmhead<NT, NCP, true, true>), grid, block, 0, s, x, wt, ot, box, m,
                       hidden, shard, vocab);
  else if (push)
    hipLaunchKernelGGL((k_lmhead<NT, NCP, true, false>), grid, block, 0, s, x, wt, ot, box, m,
                       hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead<NT, NCP, false, true>), grid, block, 0, s, x, wt, ot, box, m,
                       hidden, shard, vocab);
  return hipGetLastError();
}

template <int NCP>
hipError_t launch_lmhead_ncp(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                             bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                             hipStream_t s) {
  if (tp <= kSmallTable)
    return launch_lmhead_nt<kSmallTable, NCP>(x, w, so, keep, push, box, m, hidden, shard, tp, s);
  return launch_lmhead_nt<HG_MAX_TP, NCP>(x, w, so, keep, push, box, m, hidden, shard, tp, s);
}

// 64-wide K steps with separate pipeline depths for the two operands: X
// (re-read by every workgroup, served from L2) in XS stages, the weights
// (streamed once from HBM) in WS stages, filling the 160 KB of LDS with
// XS=2, WS=3. X of step kb+XS-1 and weights of step kb+WS-1 are issued after
// the barrier of step kb, X first, so that one wait for "all but the newest
// weight step" covers both operands of step kb.
template <int NT, int XS, int WS, bool PUSH, bool KEEP>
__global__ __launch_bounds__(512) void k_lmhead_dma2(const u32x4 *x, ShardTableN<NT> w,
                                                     OutTableN<NT> shards_out, ParityArg pa, int m,
                                                     int hidden, int shard, int vocab) {
  constexpr int KS = 64;
  constexpr int kTN = 256;
  constexpr int kRowBytes = 128;
  constexpr int kSlots = 8;
  constexpr int kRowsPerInst = 8;
  constexpr int kPart = 256 * kRowBytes;  // one operand tile of one step: 32 KB
  constexpr int kInst = 4;                // per operand, per wave, per step
  __shared__ __attribute__((aligned(1024))) unsigned char lds[(XS + WS) * kPart];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mh = wave & 1;
  const int nq = wave >> 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;

  // Instruction q of wave w fills rows 8*(8q+w) .. +8 of an operand tile.
  const int lrow = lane >> 3, lslot = lane & 7;
  const u32x4 *xsrc[kInst], *wsrc[kInst];
  bool xok[kInst], wok[kInst];
  int seg[kInst];
#pragma unroll
  for (int q = 0; q < kInst; ++q) {
    const int row = kRowsPerInst * (8 * q + wave) + lrow;  // 0..255
    seg[q] = lslot ^ dswz<64>(row);
    xok[q] = m0 + row < m;
    xsrc[q] = x + static_cast<long long>(xok[q] ? m0 + row : 0) * hv;
    const int n = n0 + row;
    const int n_wave = __builtin_amdgcn_readfirstlane(n0 + kRowsPerInst * (8 * q + wave));
    wok[q] = n < vocab;
    const int r = n_wave < vocab ? n_wave / shard : 0;
    wsrc[q] = w.p[r] + static_cast<long long>(wok[q] ? n - r * shard : 0) * hv;
  }
  unsigned char *xbase = lds;
  unsigned char *wbase = lds + XS * kPart;
  auto issue_x = [&](int kb) {
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int kv = kb * kSlots + seg[q];
      __builtin_amdgcn_global_load_lds(
          xsrc[q] + (xok[q] && kv < hv ? kv : 0),
          (__attribute__((address_space(3))) void *)(xbase + (kb % XS) * kPart +
                                                     kRowsPerInst * (8 * q + wave) * kRowBytes),
          16, 0, 0);
    }
  };
  auto issue_w = [&](int kb) {
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int kv = kb * kSlots + seg[q];
      __builtin_amdgcn_global_load_lds(
          wsrc[q] + (wok[q] && kv < hv ? kv : 0),
          (__attribute__((address_space(3))) void *)(wbase + (kb % WS) * kPart +
                                                     kRowsPerInst * (8 * q + wave) * kRowBytes),
          16, 0, 2 /* nt */);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[i][cb] = f32x16{};

  const bool tails = hidden % KS != 0 || m0 + kTM > m;
  // Prologue, in the order the steady state keeps: W(0..WS-2) then X(0..XS-2)
  // interleaved so that X(kb) is always issued before W(kb+WS-2).
  for (int p = 0; p < WS - 1 && p < steps; ++p) {
    if (p < XS - 1) issue_x(p);
    issue_w(p);
  }
  for (int kb = 0; kb < steps; ++kb) {
    // Outstanding, oldest first: ..., X(kb), W(kb+1) [if issued]. Wait until
    // only the newest weight step may remain.
    if (WS >= 3 && kb + 1 < steps)
      wait_vm<kInst>();
    else
      wait_vm<0>();
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    unsigned char *sx = xbase + (kb % XS) * kPart;
    unsigned char *sw = wbase + (kb % WS) * kPart;
    if (tails) {
#pragma unroll
      for (int q = 0; q < kInst; ++q) {
        const int kv = kb * kSlots + seg[q];
        const int off = (kRowsPerInst * (8 * q + wave) + lrow) * kRowBytes + lslot * 16;
        if (!(xok[q] && kv < hv)) *reinterpret_cast<u32x4 *>(sx + off) = u32x4{0u, 0u, 0u, 0u};
        if (!(wok[q] && kv < hv)) *reinterpret_cast<u32x4 *>(sw + off) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kb + XS - 1 < steps) issue_x(kb + XS - 1);
    if (kb + WS - 1 < steps) issue_w(kb + WS - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int g = 4 * (j >> 1) + 2 * half + (j & 1);
      bf16x8 b[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int row = 64 * nq + 32 * cb + l32;
        b[cb] = *reinterpret_cast<const bf16x8 *>(sw + row * kRowBytes + ((g ^ dswz<64>(row)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 128 * mh + 32 * i + l32;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8 *>(sx + row * kRowBytes + ((g ^ dswz<64>(row)) << 4));
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[1], acc[i][1], 0, 0, 0);
      }
    }
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c0 = n0 + 64 * nq + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[i][cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 128 * mh + 32 * i + 8 * q + 4 * half;
        const int row0 = rbase + (even ? 0 : 1);
        const int row1 = rbase + (even ? 2 : 3);
        if (row0 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row0) * words_per_shard_row + wcol] = w0;
          if (PUSH)
            box[static_cast<long long>(row0) * words_per_row + (r * shard >> 1) + wcol] =
                w0 == kSentinel ? 0u : w0;
        }
        if (row1 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row1) * words_per_shard_row + wcol] = w1;
          if (PUSH)
            box[static_cast<long long>(row1) * words_per_row + (r * shard >> 1) + wcol] =
                w1 == kSentinel ? 0u : w1;
        }
      }
    }
  }
}

template <int NT, int XS, int WS>
hipError_t launch_lmhead_dma2_nt(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                                 bool push, const ParityArg &box, int m, int hidden, int shard,
                                 int tp, hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  const dim3 grid((vocab + 255) / 256, (m + kTM - 1) / kTM);
  if (push && keep)
    hipLaunchKernelGGL((k_lmhead_dma2<NT, XS, WS, true, true>), grid, dim3(512), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  else if (push)
    hipLaunchKernelGGL((k_lmhead_dma2<NT, XS, WS, true, false>), grid, dim3(512), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead_dma2<NT, XS, WS, false, true>), grid, dim3(512), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  return hipGetLastError();
}

// Four waves per workgroup, one per SIMD, each computing a 128 x 128 block of
// the 256 x 256 tile (4 x 4 MFMA blocks, 256 accumulator registers): per K
// element a wave reads 256 operand rows from LDS for 16 blocks, where the
// eight-wave layout reads 192 for 8, so LDS traffic per MFMA drops by a
// quarter. 64-wide K steps; X in 2 LDS stages, the weights in 3, direct
// global -> LDS loads into XOR-swizzled rows.
//
// With one wave per SIMD nothing else hides LDS latency, so the wave
// pipelines by hand: the operand fragments of 16-wide K slice j+1 are read
// while the 16 MFMAs of slice j run (two register sets), and the wait and
// barrier for the next K step come before the last slice, so that its first
// fragments load under that slice's MFMAs. Loads of step kb+2 (X) and kb+3
// (weights) are issued right after that barrier, into the stages step kb
// used: every wave has its fragments of step kb in registers by then (it
// waits for its own LDS reads before the barrier).
//
// The MFMAs of every 32 x 32 block run in the same K order as in the other
// variants, so the results are bit-identical to theirs.
template <int NT, bool ONE_RANK, bool PUSH, bool KEEP>
__global__ __launch_bounds__(256) void k_lmhead_w4(const u32x4 *x, ShardTableN<NT> w,
                                                   OutTableN<NT> shards_out, ParityArg pa, int m,
                                                   int hidden, int shard, int vocab) {
  constexpr int XS = 2, WS = 3;
  constexpr int KS = 64;
  constexpr int kTN = 256;
  constexpr int kRowBytes = 128;
  constexpr int kSlots = 8;
  constexpr int kRowsPerInst = 8;
  constexpr int kPart = 256 * kRowBytes;  // one operand tile of one step: 32 KB
  constexpr int kInst = 8;                // per operand, per wave, per step
  __shared__ __attribute__((aligned(1024))) unsigned char lds[(XS + WS) * kPart];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mh = wave & 1;   // 128-row half of the tile
  const int nh = wave >> 1;  // 128-column half of the tile
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;

  // The loads are buffer loads into LDS (buffer_load_dwordx4 ... lds). Their
  // global-address form would make the compiler treat every later LDS read
  // as possibly out of order and wait for all of them at each use. X: one
  // resource from the tile's first row. Weights: instruction q of wave w
  // fills rows 8*(4q+w) .. +8 of the tile, all of one rank, so each gets a
  // wave-uniform resource from its first row -- or, with ONE_RANK (shard a
  // multiple of the 256-row tile, so no tile straddles two ranks), one
  // resource from the tile's first row serves all. A lane whose row is out
  // of range (or whose K segment is past `hidden`) loads offset 0 instead;
  // its slot is cleared before use.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int xrows = m - m0 < kTM ? m - m0 : kTM;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(x + static_cast<long long>(m0) * hv), 0, xrows * hidden * 2,
      kRawBufferWord3);
  // (fixed size: with a size that depends on the template arguments the host
  // compiler silently drops this kernel's launch stub)
  __amdgpu_buffer_rsrc_t wres[kInst];
  int xoff[kInst], woff[kInst], seg[kInst];
  bool xok[kInst], wok[kInst];
  if constexpr (ONE_RANK) {
    const int r = n0 / shard;
    const int trows = vocab - n0 < kTN ? vocab - n0 : kTN;
    wres[0] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(w.p[r] + static_cast<long long>(n0 - r * shard) * hv), 0,
        trows * hidden * 2, kRawBufferWord3);
  }
#pragma unroll
  for (int q = 0; q < kInst; ++q) {
    const int row = kRowsPerInst * (4 * q + wave) + lrow;  // 0..255
    seg[q] = lslot ^ dswz<64>(row);
    xok[q] = row < xrows;
    xoff[q] = row * hv * 16;
    wok[q] = n0 + row < vocab;
    if constexpr (ONE_RANK) {
      woff[q] = row * hv * 16;
    } else {
      const int nfirst = __builtin_amdgcn_readfirstlane(n0 + kRowsPerInst * (4 * q + wave));
      const int r = nfirst < vocab ? nfirst / shard : 0;
      const int s0 = nfirst < vocab ? nfirst - r * shard : 0;
      const int grows =
          nfirst < vocab ? (vocab - nfirst < kRowsPerInst ? vocab - nfirst : kRowsPerInst) : 1;
      wres[q] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<u32x4 *>(w.p[r] + static_cast<long long>(s0) * hv), 0, grows * hidden * 2,
          kRawBufferWord3);
      woff[q] = lrow * hv * 16;
    }
  }
  unsigned char *xbase = lds;
  unsigned char *wbase = lds + XS * kPart;
  auto issue_x = [&](int kb) {
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int kv = kb * kSlots + seg[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres,
          (__attribute__((address_space(3))) void *)(xbase + (kb % XS) * kPart +
                                                     kRowsPerInst * (4 * q + wave) * kRowBytes),
          16, xok[q] && kv < hv ? xoff[q] + kv * 16 : 0, 0, 0, 0);
    }
  };
  auto issue_w = [&](int kb) {
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int kv = kb * kSlots + seg[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wres[ONE_RANK ? 0 : q],
          (__attribute__((address_space(3))) void *)(wbase + (kb % WS) * kPart +
                                                     kRowsPerInst * (4 * q + wave) * kRowBytes),
          16, wok[q] && kv < hv ? woff[q] + kv * 16 : 0, 0, 0, kPolicyNt);
    }
  };
  const bool tails = hidden % KS != 0 || m0 + kTM > m;
  // After the barrier of step kb: clear the slots of this wave's loads that
  // fell outside X's rows, the weight rows or K, before anyone reads them.
  auto clear_tails = [&](int kb) {
    if (!tails) return;
    unsigned char *sx = xbase + (kb % XS) * kPart;
    unsigned char *sw = wbase + (kb % WS) * kPart;
#pragma unroll
    for (int q = 0; q < kInst; ++q) {
      const int kv = kb * kSlots + seg[q];
      const int off = (kRowsPerInst * (4 * q + wave) + lrow) * kRowBytes + lslot * 16;
      if (!(xok[q] && kv < hv)) *reinterpret_cast<u32x4 *>(sx + off) = u32x4{0u, 0u, 0u, 0u};
      if (!(wok[q] && kv < hv)) *reinterpret_cast<u32x4 *>(sw + off) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[i][cb] = f32x16{};

  auto barrier = [] {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
  };
  // Operand fragments of K slice j (0..3) of step kb: weights, then X.
  auto fragments_w = [&](int kb, int j, bf16x8 (&b)[4]) {
    const unsigned char *sw = wbase + (kb % WS) * kPart;
    const int g = 4 * (j >> 1) + 2 * half + (j & 1);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int row = 128 * nh + 32 * cb + l32;
      b[cb] = *reinterpret_cast<const bf16x8 *>(sw + row * kRowBytes + ((g ^ dswz<64>(row)) << 4));
    }
  };
  auto fragments_x = [&](int kb, int j, bf16x8 (&a)[4]) {
    const unsigned char *sx = xbase + (kb % XS) * kPart;
    const int g = 4 * (j >> 1) + 2 * half + (j & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 128 * mh + 32 * i + l32;
      a[i] = *reinterpret_cast<const bf16x8 *>(sx + row * kRowBytes + ((g ^ dswz<64>(row)) << 4));
    }
  };
  auto mfma_rows = [&](int i0, const bf16x8 (&a)[4], const bf16x8 (&b)[4]) {
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[cb], acc[i][cb], 0, 0, 0);
  };

  // Prologue: X0 W0 X1 W1 W2 in that order. Step 0 may start once X0 and W0
  // are in: the newest 3, 2 or 0 instruction groups may still be in flight.
  issue_x(0);
  issue_w(0);
  if (steps > 1) {
    issue_x(1);
    issue_w(1);
  }
  if (steps > 2) issue_w(2);
  if (steps > 2)
    wait_vm<3 * kInst>();
  else if (steps > 1)
    wait_vm<2 * kInst>();
  else
    wait_vm<0>();
  barrier();
  clear_tails(0);

  // The next slice's eight fragment reads go out in two groups of four, one
  // before each half of the current slice's MFMAs: at most 12 LDS reads are
  // then in flight, within what the 4-bit LDS counter can wait on
  // selectively (with 16 the only possible wait would be for all of them).
  // The scheduling barriers keep that order (the scheduler would otherwise
  // trade the overlap for fewer live registers).
  bf16x8 fa[2][4], fb[2][4];
  fragments_w(0, 0, fb[0]);
  fragments_x(0, 0, fa[0]);
  for (int kb = 0; kb < steps; ++kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cur = j & 1, nxt = cur ^ 1;
      if (j < 3) {
        fragments_w(kb, j + 1, fb[nxt]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(0, fa[cur], fb[cur]);
        __builtin_amdgcn_sched_barrier(0);
        fragments_x(kb, j + 1, fa[nxt]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(2, fa[cur], fb[cur]);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        if (kb + 1 < steps) {
          // Step kb+1: X(kb+1) and W(kb+1) must be in; only W(kb+2), issued
          // after X(kb+1), may remain. Own LDS reads of step kb done first.
          if (kb + 2 < steps)
            __builtin_amdgcn_s_waitcnt((kInst & 15) | ((kInst >> 4) << 14) | 0x070);
          else
            __builtin_amdgcn_s_waitcnt(0x070);
          barrier();
          clear_tails(kb + 1);
          if (kb + XS < steps) issue_x(kb + XS);
          if (kb + WS < steps) issue_w(kb + WS);
          fragments_w(kb + 1, 0, fb[nxt]);
          fragments_x(kb + 1, 0, fa[nxt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_rows(0, fa[cur], fb[cur]);
        mfma_rows(2, fa[cur], fb[cur]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int c0 = n0 + 128 * nh + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[i][cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 128 * mh + 32 * i + 8 * q + 4 * half;
        const int row0 = rbase + (even ? 0 : 1);
        const int row1 = rbase + (even ? 2 : 3);
        if (row0 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row0) * words_per_shard_row + wcol] = w0;
          if (PUSH)
            box[static_cast<long long>(row0) * words_per_row + (r * shard >> 1) + wcol] =
                w0 == kSentinel ? 0u : w0;
        }
        if (row1 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row1) * words_per_shard_row + wcol] = w1;
          if (PUSH)
            box[static_cast<long long>(row1) * words_per_row + (r * shard >> 1) + wcol] =
                w1 == kSentinel ? 0u : w1;
        }
      }
    }
  }
}

template <int NT, bool ONE_RANK>
hipError_t launch_lmhead_w4_one(const u32x4 *x, const ShardTableN<NT> &wt, const OutTableN<NT> &ot,
                                bool keep, bool push, const ParityArg &box, int m, int hidden,
                                int shard, int vocab, hipStream_t s) {
  const dim3 grid((vocab + 255) / 256, (m + kTM - 1) / kTM);
  if (push && keep)
    hipLaunchKernelGGL((k_lmhead_w4<NT, ONE_RANK, true, true>), grid, dim3(256), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  else if (push)
    hipLaunchKernelGGL((k_lmhead_w4<NT, ONE_RANK, true, false>), grid, dim3(256), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead_w4<NT, ONE_RANK, false, true>), grid, dim3(256), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_lmhead_w4_nt(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                               bool push, const ParityArg &box, int m, int hidden, int shard,
                               int tp, hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  if (shard % 256 == 0)
    return launch_lmhead_w4_one<NT, true>(x, wt, ot, keep, push, box, m, hidden, shard, vocab, s);
  return launch_lmhead_w4_one<NT, false>(x, wt, ot, keep, push, box, m, hidden, shard, vocab, s);
}

// 256 x 320 output tiles: 163840 columns make 512 tiles, two full rounds on
// 256 CUs, where 256-column tiles make 640 (three rounds, the last half
// empty), and each K step moves 12.5 % more bytes per round trip. Eight waves
// of 64 rows x 160 columns (2 x 5 MFMA blocks, 160 accumulator registers).
// K step KS (64 or 32), ST LDS stages of [256 X rows + 320 weight rows]
// (2 x 72 KB or 4 x 36 KB), loads issued ST-1 steps ahead, direct global ->
// LDS into XOR-swizzled rows as in k_lmhead_dma. A wave's load instruction
// fills 1024 / (2 KS) rows; the weight rows' instructions are dealt to the
// waves in turn, so with KS = 32 (20 of them) waves 0..3 issue one more than
// waves 4..7. Same MFMA sequence per 32 x 32 block as the other variants, so
// the same bits.
template <int NT, int KS, int ST, bool PUSH, bool KEEP>
__global__ __launch_bounds__(512) void k_lmhead_n320(const u32x4 *x, ShardTableN<NT> w,
                                                     OutTableN<NT> shards_out, ParityArg pa, int m,
                                                     int hidden, int shard, int vocab) {
  static_assert((KS == 64 && ST == 2) || (KS == 32 && (ST == 3 || ST == 4)), "stage plan");
  constexpr int kTN = 320;
  constexpr int kRowBytes = 2 * KS;
  constexpr int kSlots = KS / 8;                  // 16-byte slots per row
  constexpr int kRowsPerInst = 1024 / kRowBytes;  // rows one wave instruction fills
  constexpr int kXPart = kTM * kRowBytes;
  constexpr int kStage = (kTM + kTN) * kRowBytes;
  constexpr int kXInst = kTM / kRowsPerInst / 8;  // per wave per step
  constexpr int kWAll = kTN / kRowsPerInst;       // weight instructions per step
  constexpr int kWInst = (kWAll + 7) / 8;         // most per wave
  constexpr int kLong = kXInst + kWInst;          // loads per step, waves 0 .. kWAll%8-1
  constexpr int kShort = kXInst + kWAll / 8;      // loads per step, the other waves
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ST * kStage];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mq = wave & 3;   // 64-row quarter of the tile
  const int nh = wave >> 2;  // 160-column half of the tile
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;
  const bool short_wave = kWAll % 8 != 0 && wave >= kWAll % 8;

  // Instruction q of wave w fills rows kRowsPerInst*(8q+w) .. of an operand.
  const int lrow = lane / kSlots, lslot = lane % kSlots;
  // (arrays of the largest plan's size: with sizes that depend on the
  // template arguments the host compiler silently drops the launch stub)
  static_assert(kXInst <= 4 && kWInst <= 5, "per-wave load arrays");
  const u32x4 *xsrc[4], *wsrc[5];
  bool xok[4], wok[5];
  int xseg[4], wseg[5];
#pragma unroll
  for (int q = 0; q < kXInst; ++q) {
    const int row = kRowsPerInst * (8 * q + wave) + lrow;  // 0..255
    xseg[q] = lslot ^ dswz<KS>(row);
    xok[q] = m0 + row < m;
    xsrc[q] = x + static_cast<long long>(xok[q] ? m0 + row : 0) * hv;
  }
#pragma unroll
  for (int q = 0; q < kWInst; ++q) {
    const int row = kRowsPerInst * (8 * q + wave) + lrow;  // 0..319 when 8q+w < kWAll
    wseg[q] = lslot ^ dswz<KS>(row);
    const int n = n0 + row;
    const int n_wave = __builtin_amdgcn_readfirstlane(n0 + kRowsPerInst * (8 * q + wave));
    wok[q] = 8 * q + wave < kWAll && n < vocab;
    const int r = wok[q] ? n_wave / shard : 0;
    wsrc[q] = w.p[r] + static_cast<long long>(wok[q] ? n - r * shard : 0) * hv;
  }
  // A lane whose row is out of range (or whose K segment is past `hidden`)
  // loads from a valid address; its slot is cleared before use.
  auto issue = [&](int kb) {
    unsigned char *st = lds + (kb % ST) * kStage;
#pragma unroll
    for (int q = 0; q < kXInst; ++q) {
      const int kv = kb * kSlots + xseg[q];
      __builtin_amdgcn_global_load_lds(
          xsrc[q] + (xok[q] && kv < hv ? kv : 0),
          (__attribute__((address_space(3))) void *)(st + kRowsPerInst * (8 * q + wave) * kRowBytes),
          16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < kWInst; ++q) {
      if (8 * q + wave >= kWAll) continue;  // wave-uniform
      const int kv = kb * kSlots + wseg[q];
      __builtin_amdgcn_global_load_lds(
          wsrc[q] + (wok[q] && kv < hv ? kv : 0),
          (__attribute__((address_space(3))) void *)(st + kXPart +
                                                     kRowsPerInst * (8 * q + wave) * kRowBytes),
          16, 0, 2 /* nt */);
    }
  };

  f32x16 acc[2][5];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int cb = 0; cb < 5; ++cb) acc[i][cb] = f32x16{};

  const bool tails = hidden % KS != 0 || m0 + kTM > m || n0 + kTN > vocab;
  for (int p = 0; p < ST - 1 && p < steps; ++p) issue(p);
  for (int kb = 0; kb < steps; ++kb) {
    // Wait for this wave's loads of step kb; the later steps' stay in flight.
    const int ahead = steps - 1 - kb < ST - 2 ? steps - 1 - kb : ST - 2;
    if (ahead >= 2) {
      if (short_wave) wait_vm<2 * kShort>(); else wait_vm<2 * kLong>();
    } else if (ahead == 1) {
      if (short_wave) wait_vm<kShort>(); else wait_vm<kLong>();
    } else {
      wait_vm<0>();
    }
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    unsigned char *sx = lds + (kb % ST) * kStage;
    unsigned char *sw = sx + kXPart;
    if (tails) {
#pragma unroll
      for (int q = 0; q < kXInst; ++q) {
        const int kv = kb * kSlots + xseg[q];
        if (!(xok[q] && kv < hv))
          *reinterpret_cast<u32x4 *>(sx + (kRowsPerInst * (8 * q + wave) + lrow) * kRowBytes +
                                     lslot * 16) = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < kWInst; ++q) {
        const int kv = kb * kSlots + wseg[q];
        if (8 * q + wave < kWAll && !(wok[q] && kv < hv))
          *reinterpret_cast<u32x4 *>(sw + (kRowsPerInst * (8 * q + wave) + lrow) * kRowBytes +
                                     lslot * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kb + ST - 1 < steps) issue(kb + ST - 1);
#pragma unroll
    for (int j = 0; j < KS / 16; ++j) {
      // K segment of this lane for MFMA j: 32-wide slice j/2, half, j%2.
      const int g = 4 * (j >> 1) + 2 * half + (j & 1);
      bf16x8 a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 64 * mq + 32 * i + l32;
        a[i] = *reinterpret_cast<const bf16x8 *>(sx + row * kRowBytes + ((g ^ dswz<KS>(row)) << 4));
      }
#pragma unroll
      for (int cb = 0; cb < 5; ++cb) {
        const int row = 160 * nh + 32 * cb + l32;
        const bf16x8 b =
            *reinterpret_cast<const bf16x8 *>(sw + row * kRowBytes + ((g ^ dswz<KS>(row)) << 4));
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i][cb], 0, 0, 0);
      }
    }
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 5; ++cb) {
    const int c0 = n0 + 160 * nh + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[i][cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 64 * mq + 32 * i + 8 * q + 4 * half;
        const int row0 = rbase + (even ? 0 : 1);
        const int row1 = rbase + (even ? 2 : 3);
        if (row0 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row0) * words_per_shard_row + wcol] = w0;
          if (PUSH)
            box[static_cast<long long>(row0) * words_per_row + (r * shard >> 1) + wcol] =
                w0 == kSentinel ? 0u : w0;
        }
        if (row1 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row1) * words_per_shard_row + wcol] = w1;
          if (PUSH)
            box[static_cast<long long>(row1) * words_per_row + (r * shard >> 1) + wcol] =
                w1 == kSentinel ? 0u : w1;
        }
      }
    }
  }
}

template <int NT, int KS, int ST>
hipError_t launch_lmhead_n320_nt(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                                 bool push, const ParityArg &box, int m, int hidden, int shard,
                                 int tp, hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  const dim3 grid((vocab + 319) / 320, (m + kTM - 1) / kTM);
  if (push && keep)
    hipLaunchKernelGGL((k_lmhead_n320<NT, KS, ST, true, true>), grid, dim3(512), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  else if (push)
    hipLaunchKernelGGL((k_lmhead_n320<NT, KS, ST, true, false>), grid, dim3(512), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead_n320<NT, KS, ST, false, true>), grid, dim3(512), 0, s, x, wt, ot,
                       box, m, hidden, shard, vocab);
  return hipGetLastError();
}

// As k_lmhead_n320 with 64-wide K steps and 2 stages, but the loads are
// buffer loads into LDS (buffer_load_dwordx4 ... lds), as in k_lmhead_w4:
// with the global-address form the compiler waits for every outstanding LDS
// read at each MFMA group, so each pair of MFMAs sits out a whole LDS round
// trip. X: one resource from the tile's first row. Weights: with ONE_RANK
// (shard a multiple of 320, so no tile straddles two ranks) one resource from
// the tile's first row; otherwise one per load instruction, from the first of
// its 8 rows (all of one rank, as shard % 32 == 0).
template <int NT, bool ONE_RANK, bool PUSH, bool KEEP>
__global__ __launch_bounds__(512) void k_lmhead_n320b(const u32x4 *x, ShardTableN<NT> w,
                                                      OutTableN<NT> shards_out, ParityArg pa,
                                                      int m, int hidden, int shard, int vocab) {
  constexpr int KS = 64;
  constexpr int kTN = 320;
  constexpr int kRowBytes = 128;
  constexpr int kSlots = 8;
  constexpr int kXPart = kTM * kRowBytes;           // 32 KB
  constexpr int kStage = (kTM + kTN) * kRowBytes;   // 72 KB
  constexpr int kXInst = 4, kWInst = 5;             // per wave per step
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mq = wave & 3;   // 64-row quarter of the tile
  const int nh = wave >> 2;  // 160-column half of the tile
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;

  // Instruction q of wave w fills rows 8*(8q+w) .. +8 of an operand. A lane
  // whose row is out of range (or whose K segment is past `hidden`) loads
  // offset 0 instead; its slot is cleared before use.
  const int lrow = lane >> 3, lslot = lane & 7;
  const int xrows = m - m0 < kTM ? m - m0 : kTM;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(x + static_cast<long long>(m0) * hv), 0, xrows * hidden * 2,
      kRawBufferWord3);
  __amdgpu_buffer_rsrc_t wres[kWInst];
  int xoff[kXInst], woff[kWInst], xseg[kXInst], wseg[kWInst];
  bool xok[kXInst], wok[kWInst];
#pragma unroll
  for (int q = 0; q < kXInst; ++q) {
    const int row = 8 * (8 * q + wave) + lrow;  // 0..255
    xseg[q] = lslot ^ dswz<64>(row);
    xok[q] = row < xrows;
    xoff[q] = row * hv * 16;
  }
  if constexpr (ONE_RANK) {
    const int r = n0 / shard;
    const int trows = vocab - n0 < kTN ? vocab - n0 : kTN;
    wres[0] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(w.p[r] + static_cast<long long>(n0 - r * shard) * hv), 0,
        trows * hidden * 2, kRawBufferWord3);
  }
#pragma unroll
  for (int q = 0; q < kWInst; ++q) {
    const int row = 8 * (8 * q + wave) + lrow;  // 0..319
    wseg[q] = lslot ^ dswz<64>(row);
    wok[q] = n0 + row < vocab;
    if constexpr (ONE_RANK) {
      woff[q] = row * hv * 16;
    } else {
      const int nfirst = __builtin_amdgcn_readfirstlane(n0 + 8 * (8 * q + wave));
      const int r = nfirst < vocab ? nfirst / shard : 0;
      const int s0 = nfirst < vocab ? nfirst - r * shard : 0;
      const int grows = nfirst < vocab ? (vocab - nfirst < 8 ? vocab - nfirst : 8) : 1;
      wres[q] = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<u32x4 *>(w.p[r] + static_cast<long long>(s0) * hv), 0, grows * hidden * 2,
          kRawBufferWord3);
      woff[q] = lrow * hv * 16;
    }
  }
  // X load instructions whose 8 rows all lie past m are not issued: rows past
  // m only ever reach output rows that are not stored, so their LDS slots may
  // hold anything (likewise weight rows past the vocabulary).
  bool xinst[kXInst];
#pragma unroll
  for (int q = 0; q < kXInst; ++q) xinst[q] = 8 * (8 * q + wave) < xrows;  // wave-uniform
  auto issue = [&](int kb) {
    unsigned char *st = lds + (kb & 1) * kStage;
#pragma unroll
    for (int q = 0; q < kXInst; ++q) {
      if (!xinst[q]) continue;
      const int kv = kb * kSlots + xseg[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void *)(st + 8 * (8 * q + wave) * kRowBytes),
          16, xok[q] && kv < hv ? xoff[q] + kv * 16 : 0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < kWInst; ++q) {
      const int kv = kb * kSlots + wseg[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wres[ONE_RANK ? 0 : q],
          (__attribute__((address_space(3))) void *)(st + kXPart + 8 * (8 * q + wave) * kRowBytes),
          16, wok[q] && kv < hv ? woff[q] + kv * 16 : 0, 0, 0, kPolicyNt);
    }
  };

  f32x16 acc[2][5];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int cb = 0; cb < 5; ++cb) acc[i][cb] = f32x16{};

  // Only a K segment past `hidden` must read as zero: it meets real data in
  // the other operand. Such slots (loaded from offset 0) are cleared.
  const bool ktail = hidden % KS != 0;
  // A wave whose 64 rows all lie at or past m computes nothing (wave-uniform):
  // at small m most waves only stream loads.
  const bool blk0 = m0 + 64 * mq < m;
  issue(0);
  for (int kb = 0; kb < steps; ++kb) {
    wait_vm<0>();  // this wave's loads of step kb (nothing newer is in flight)
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    unsigned char *sx = lds + (kb & 1) * kStage;
    unsigned char *sw = sx + kXPart;
    if (ktail && (kb + 1) * kSlots > hv) {
#pragma unroll
      for (int q = 0; q < kXInst; ++q) {
        const int kv = kb * kSlots + xseg[q];
        if (xinst[q] && kv >= hv)
          *reinterpret_cast<u32x4 *>(sx + (8 * (8 * q + wave) + lrow) * kRowBytes + lslot * 16) =
              u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < kWInst; ++q) {
        const int kv = kb * kSlots + wseg[q];
        if (kv >= hv)
          *reinterpret_cast<u32x4 *>(sw + (8 * (8 * q + wave) + lrow) * kRowBytes + lslot * 16) =
              u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kb + 1 < steps) issue(kb + 1);
    if (!blk0) continue;  // no row of this wave's 64 below m: loads only
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // K segment of this lane for MFMA j: 32-wide slice j/2, half, j%2.
      const int g = 4 * (j >> 1) + 2 * half + (j & 1);
      bf16x8 a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 64 * mq + 32 * i + l32;
        a[i] = *reinterpret_cast<const bf16x8 *>(sx + row * kRowBytes + ((g ^ dswz<64>(row)) << 4));
      }
#pragma unroll
      for (int cb = 0; cb < 5; ++cb) {
        const int row = 160 * nh + 32 * cb + l32;
        const bf16x8 b =
            *reinterpret_cast<const bf16x8 *>(sw + row * kRowBytes + ((g ^ dswz<64>(row)) << 4));
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b, acc[i][cb], 0, 0, 0);
      }
    }
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 5; ++cb) {
    const int c0 = n0 + 160 * nh + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[i][cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 64 * mq + 32 * i + 8 * q + 4 * half;
        const int row0 = rbase + (even ? 0 : 1);
        const int row1 = rbase + (even ? 2 : 3);
        if (row0 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row0) * words_per_shard_row + wcol] = w0;
          if (PUSH)
            box[static_cast<long long>(row0) * words_per_row + (r * shard >> 1) + wcol] =
                w0 == kSentinel ? 0u : w0;
        }
        if (row1 < m) {
          if (KEEP) shards_out.p[r][static_cast<long long>(row1) * words_per_shard_row + wcol] = w1;
          if (PUSH)
            box[static_cast<long long>(row1) * words_per_row + (r * shard >> 1) + wcol] =
                w1 == kSentinel ? 0u : w1;
        }
      }
    }
  }
}

template <int NT, bool ONE_RANK>
hipError_t launch_lmhead_n320b_one(const u32x4 *x, const ShardTableN<NT> &wt,
                                   const OutTableN<NT> &ot, bool keep, bool push,
                                   const ParityArg &box, int m, int hidden, int shard, int vocab,
                                   hipStream_t s) {
  const dim3 grid((vocab + 319) / 320, (m + kTM - 1) / kTM);
  if (push && keep)
    hipLaunchKernelGGL((k_lmhead_n320b<NT, ONE_RANK, true, true>), grid, dim3(512), 0, s, x, wt,
                       ot, box, m, hidden, shard, vocab);
  else if (push)
    hipLaunchKernelGGL((k_lmhead_n320b<NT, ONE_RANK, true, false>), grid, dim3(512), 0, s, x, wt,
                       ot, box, m, hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead_n320b<NT, ONE_RANK, false, true>), grid, dim3(512), 0, s, x, wt,
                       ot, box, m, hidden, shard, vocab);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_lmhead_n320b_nt(const u32x4 *x, const ShardTable &w, const OutTable &so,
                                  bool keep, bool push, const ParityArg &box, int m, int hidden,
                                  int shard, int tp, hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  if (shard % 320 == 0)
    return launch_lmhead_n320b_one<NT, true>(x, wt, ot, keep, push, box, m, hidden, shard, vocab,
                                             s);
  return launch_lmhead_n320b_one<NT, false>(x, wt, ot, keep, push, box, m, hidden, shard, vocab,
                                            s);
}

template <int KS, int ST>
hipError_t launch_lmhead_n320(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                              bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                              hipStream_t s) {
  if (tp <= kSmallTable)
    return launch_lmhead_n320_nt<kSmallTable, KS, ST>(x, w, so, keep, push, box, m, hidden, shard,
                                                      tp, s);
  return launch_lmhead_n320_nt<HG_MAX_TP, KS, ST>(x, w, so, keep, push, box, m, hidden, shard, tp,
                                                  s);
}

template <int NT, int KS, int ST, bool WNT>
hipError_t launch_lmhead_dma_nt(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                                bool push, const ParityArg &box, int m, int hidden, int shard,
                                int tp, hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  const dim3 grid((vocab + 255) / 256, (m + kTM - 1) / kTM);
  if (push && keep)
    hipLaunchKernelGGL((k_lmhead_dma<NT, KS, ST, WNT, true, true>), grid, dim3(512), 0, s, x, wt,
                       ot, box, m, hidden, shard, vocab);
  else if (push)
    hipLaunchKernelGGL((k_lmhead_dma<NT, KS, ST, WNT, true, false>), grid, dim3(512), 0, s, x, wt,
                       ot, box, m, hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead_dma<NT, KS, ST, WNT, false, true>), grid, dim3(512), 0, s, x, wt,
                       ot, box, m, hidden, shard, vocab);
  return hipGetLastError();
}

template <int KS, int ST, bool WNT>
hipError_t launch_lmhead_dma(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                             bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                             hipStream_t s) {
  if (tp <= kSmallTable)
    return launch_lmhead_dma_nt<kSmallTable, KS, ST, WNT>(x, w, so, keep, push, box, m, hidden,
                                                          shard, tp, s);
  return launch_lmhead_dma_nt<HG_MAX_TP, KS, ST, WNT>(x, w, so, keep, push, box, m, hidden, shard,
                                                      tp, s);
}

}  // namespace

hipError_t launch_lmhead(const u32x4 *x, const ShardTable &w, const OutTable &shards_out, bool keep,
                         bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                         int variant, hipStream_t s) {
  switch (variant) {
    case kGemmDirectLds:
      return launch_lmhead_dma<32, 4, false>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmDirectLdsNt:
      return launch_lmhead_dma<32, 4, true>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmDirectLds64:
      return launch_lmhead_dma<64, 2, false>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmDirectLds64Nt:
      return launch_lmhead_dma<64, 2, true>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmDirectLdsDeepW:
      if (tp <= kSmallTable)
        return launch_lmhead_dma2_nt<kSmallTable, 2, 3>(x, w, shards_out, keep, push, box, m,
                                                         hidden, shard, tp, s);
      return launch_lmhead_dma2_nt<HG_MAX_TP, 2, 3>(x, w, shards_out, keep, push, box, m, hidden,
                                                     shard, tp, s);
    case kGemmWave128:
      if (tp <= kSmallTable)
        return launch_lmhead_w4_nt<kSmallTable>(x, w, shards_out, keep, push, box, m, hidden,
                                                       shard, tp, s);
      return launch_lmhead_w4_nt<HG_MAX_TP>(x, w, shards_out, keep, push, box, m, hidden,
                                                   shard, tp, s);
    case kGemmTile320:
      return launch_lmhead_n320<64, 2>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmTile320K32:
      return launch_lmhead_n320<32, 4>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmTile320K32S3:
      return launch_lmhead_n320<32, 3>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmTile320Buf:
      if (tp <= kSmallTable)
        return launch_lmhead_n320b_nt<kSmallTable>(x, w, shards_out, keep, push, box, m, hidden,
                                                   shard, tp, s);
      return launch_lmhead_n320b_nt<HG_MAX_TP>(x, w, shards_out, keep, push, box, m, hidden,
                                               shard, tp, s);
    case kGemmStaged256:
      return launch_lmhead_ncp<4>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    case kGemmStaged128:
      return launch_lmhead_ncp<2>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace hg
