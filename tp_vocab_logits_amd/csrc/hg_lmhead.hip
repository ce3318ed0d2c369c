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
// K order: lane l supplies 8 consecutive K elements per MFMA. Per 32-wide
// slice of K, the first MFMA takes offsets 0-7 (lanes 0-31) and 16-23 (lanes
// 32-63), the second 8-15 and 24-31; slices follow in order. A and B use the
// same assignment, so every product X[m,k] * W[n,k] is summed exactly once,
// and each 32 x 32 output block is one chain of MFMAs over K in increasing
// order: the result bits do not depend on the tiling around it.

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
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

// Swap a 32-bit value with the neighbouring lane (0<->1, 2<->3, ...).
__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF, true));
}

// XOR swizzle of the eight 16-byte K segments of a 128-byte LDS row: the
// fragment reads (16 consecutive rows, one K segment) then hit distinct banks
// (no SQ_LDS_BANK_CONFLICT cycles measured; 4 cycles per 64-lane read).
template <int KS>
__device__ __forceinline__ int dswz(int row) {
  static_assert(KS == 64, "128-byte rows");
  return (row ^ (row >> 3)) & 7;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N) (N < 64) without waiting on LDS or export counters
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// 256 x 320 output tiles: 163840 columns make 512 tiles, two full rounds on
// 256 CUs. Eight waves of 64 rows x 160 columns (2 x 5 MFMA blocks, 160
// accumulator registers). 64-wide K steps, two LDS stages of [256 X rows +
// 320 weight rows] x 128 bytes (72 KB each), filled by buffer loads straight
// into LDS (buffer_load_dwordx4 ... lds) one step ahead; a wave's load
// instruction fills 8 rows, lane-major, each lane loading the K segment that
// the swizzle puts at its slot. X: one buffer resource from the tile's first
// row. Weights: with ONE_RANK (shard a multiple of 320, so no tile straddles
// two ranks) one resource from the tile's first row; otherwise one per load
// instruction, from the first of its 8 rows (all of one rank, as
// shard % 32 == 0).
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


}  // namespace

hipError_t launch_lmhead(const u32x4 *x, const ShardTable &w, const OutTable &shards_out, bool keep,
                         bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                         hipStream_t s) {
  if (tp <= kSmallTable)
    return launch_lmhead_n320b_nt<kSmallTable>(x, w, shards_out, keep, push, box, m, hidden, shard,
                                               tp, s);
  return launch_lmhead_n320b_nt<HG_MAX_TP>(x, w, shards_out, keep, push, box, m, hidden, shard, tp,
                                           s);
}

}  // namespace hg
