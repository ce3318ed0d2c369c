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
// Work decomposition: a workgroup of 8 waves owns a 256-row x 256-column
// output tile (all of M = 256 at once, 256 consecutive vocab columns); wave w
// computes rows 128*(w%2) .. +128 and columns 64*(w/2) .. +64 as 4 x 2 blocks
// of v_mfma_f32_32x32x16_bf16. Per 64-wide K step the X tile [256 x 64] is
// staged in LDS (double-buffered, rows padded by 16 bytes against bank
// conflicts) and shared by the 8 waves; each wave streams its own 64 weight
// rows straight from HBM into registers, 64 contiguous bytes per lane, one
// step ahead of the matrix cores.
//
// K order inside a step: lane l supplies 8 consecutive K elements per MFMA,
// and lanes 0-31 / 32-63 cover K offsets 0-31 / 32-63 of the step across the
// four MFMAs (sub-step j takes offsets 8j..8j+7 of each half). A and B use the
// same assignment, so every product X[m,k] * W[n,k] is summed exactly once.

#include "hg_internal.h"

namespace hg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kTM = 256;
constexpr int kTN = 256;
constexpr int kTK = 64;
constexpr int kThreads = 512;
constexpr int kLdsRow = kTK + 8;  // BF16 per LDS row: 64 + 16-byte pad
constexpr int kLdsBuf = kTM * kLdsRow;

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

template <int NT, bool PUSH, bool KEEP>
__global__ __launch_bounds__(kThreads) void k_lmhead(const u32x4 *x, ShardTableN<NT> w,
                                                     OutTableN<NT> shards_out, uint32_t *box,
                                                     int m, int hidden, int shard, int vocab) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2][kLdsBuf];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int mh = wave & 1;   // row half of the tile
  const int nq = wave >> 1;  // column quarter of the tile
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;  // 16-byte vectors per X / W row
  const int steps = (hidden + kTK - 1) / kTK;

  // X staging: thread -> (tile row, 32-element half of the K step).
  const int xr = tid >> 1, xh = tid & 1;
  const bool x_ok = m0 + xr < m;
  const u32x4 *xp = x + static_cast<long long>(x_ok ? m0 + xr : 0) * hv + xh * 4;

  // Weight rows of this lane's two 32-column blocks (uniform rank per block).
  const u32x4 *wp[2];
  bool col_ok[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c0 = n0 + 64 * nq + 32 * cb;
    col_ok[cb] = c0 < vocab;
    const int r = col_ok[cb] ? c0 / shard : 0;
    const int s = col_ok[cb] ? c0 - r * shard + l32 : 0;
    wp[cb] = col_ok[cb] ? w.p[r] + static_cast<long long>(s) * hv + half * 4 : nullptr;
  }

  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 xs[4], wc[2][4], wn[2][4];

  auto load_x = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = x_ok && kb * kTK + xh * 32 + 8 * j < hidden;
      xs[j] = ok ? xp[kb * 8 + j] : zero;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4 *>(&lds[buf][xr * kLdsRow + xh * 32 + 8 * j]) = xs[j];
  };
  auto load_w = [&](int kb, u32x4 (&dst)[2][4]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = col_ok[cb] && kb * kTK + half * 32 + 8 * j < hidden;
        dst[cb][j] = ok ? load_stream(wp[cb] + kb * 8 + j) : zero;
      }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) acc[i][cb] = f32x16{};

  load_x(0);
  load_w(0, wc);
  store_x(0);
  __syncthreads();

  for (int kb = 0; kb < steps; ++kb) {
    const int buf = kb & 1;
    const bool more = kb + 1 < steps;
    if (more) {
      load_x(kb + 1);
      load_w(kb + 1, wn);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, wc[0][j]);
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, wc[1][j]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 128 * mh + 32 * i + l32;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8 *>(&lds[buf][row * kLdsRow + 32 * half + 8 * j]);
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[i][1], 0, 0, 0);
      }
    }
    if (more) {
      store_x(buf ^ 1);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) wc[cb][j] = wn[cb][j];
    }
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
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (!col_ok[cb]) continue;
    const int c0 = n0 + 64 * nq + 32 * cb;
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

template <int NT>
hipError_t launch_lmhead_nt(const u32x4 *x, const ShardTable &w, const OutTable &so, bool keep,
                            uint32_t *box, int m, int hidden, int shard, int tp, hipStream_t s) {
  ShardTableN<NT> wt;
  OutTableN<NT> ot;
  for (int r = 0; r < NT; ++r) {
    wt.p[r] = w.p[r];
    ot.p[r] = so.p[r];
  }
  const int vocab = tp * shard;
  const dim3 grid((vocab + kTN - 1) / kTN, (m + kTM - 1) / kTM);
  if (box && keep)
    hipLaunchKernelGGL((k_lmhead<NT, true, true>), grid, dim3(kThreads), 0, s, x, wt, ot, box, m,
                       hidden, shard, vocab);
  else if (box)
    hipLaunchKernelGGL((k_lmhead<NT, true, false>), grid, dim3(kThreads), 0, s, x, wt, ot, box, m,
                       hidden, shard, vocab);
  else
    hipLaunchKernelGGL((k_lmhead<NT, false, true>), grid, dim3(kThreads), 0, s, x, wt, ot, box, m,
                       hidden, shard, vocab);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead(const u32x4 *x, const ShardTable &w, const OutTable &shards_out, bool keep,
                         uint32_t *box, int m, int hidden, int shard, int tp, hipStream_t s) {
  if (tp <= kSmallTable)
    return launch_lmhead_nt<kSmallTable>(x, w, shards_out, keep, box, m, hidden, shard, tp, s);
  return launch_lmhead_nt<HG_MAX_TP>(x, w, shards_out, keep, box, m, hidden, shard, tp, s);
}

}  // namespace hg
