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

#include <type_traits>

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
// 256 CUs. Eight waves; wave w owns rows 32w .. 32w+31 of the tile and all
// 320 columns: ten 32 x 32 blocks of v_mfma_f32_32x32x16_bf16, 160
// accumulator registers.
//
// Both operands arrive by buffer loads straight into LDS (buffer_load_dwordx4
// ... lds), each instruction filling 8 rows of 128 bytes (one 64-wide K step)
// lane-major, every lane loading the K segment that the swizzle puts at its
// slot, so the global side is 8 full 128-byte lines per instruction.
//  - Weights (shared by all waves, streamed once from HBM): ST stages of
//    320 rows (40 KB each), loaded ST-1 steps ahead.
//  - X (served from L2: every column tile re-reads it): each wave's 32 rows
//    are private to it, so each wave has its own 4 KB region, loaded one step
//    ahead and read back into registers right after the step's barrier,
//    before the region is refilled.
// Weights: with ONE_RANK (shard a multiple of 320, so no tile straddles two
// ranks) one buffer resource from the tile's first row; otherwise one per
// load instruction, from the first row of its group of 8 (never straddling
// two ranks, as shard % 32 == 0).
//
// Rows past m (X) or past the vocabulary (weights) lie beyond their buffer
// resource's size, so the hardware's range check makes them read as zero.
// K segments past `hidden` (the last step of a hidden size that is not a
// multiple of 64) read the next row's data, or zero past the resource, and
// are cleared before use: in LDS for the weights, in registers for X.
//
// Step kb: wait for X(kb) and the weights of step kb; barrier; read X(kb)
// into registers; issue X(kb+1), then the weights of step kb+ST-1; multiply.
// The loads complete in issue order, so at the top of step kb one wait for
// "all but the newest weight loads" covers X(kb) and W(kb) while ST-2 steps of
// weights stay in flight across it.
template <int NT, bool ONE_RANK, bool PUSH, bool KEEP>
__global__ __launch_bounds__(512) void k_lmhead(const u32x4 *x, ShardTableN<NT> w,
                                                OutTableN<NT> shards_out, ParityArg pa, int m,
                                                int hidden, int shard, int vocab) {
  constexpr int ST = 3;  // weight stages: loaded two steps ahead
  constexpr int NW = 8;
  constexpr int KS = 64;
  constexpr int kTN = 320;
  constexpr int kRowBytes = 128;
  constexpr int kSlots = 8;                   // 16-byte K segments per row and step
  constexpr int kStage = kTN * kRowBytes;     // 40 KB
  constexpr int kXRegion = 32 * kRowBytes;    // 4 KB per wave
  constexpr int kWInst = kTN / 8 / NW;        // weight load instructions per wave and step
  constexpr int kXInst = 4;                   // X load instructions per wave and step
  constexpr int kBlocks = kTN / 32;           // column blocks
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ST * kStage + NW * kXRegion];

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;
  const int lrow = lane >> 3, lslot = lane & 7;
  unsigned char *xreg = lds + ST * kStage + wave * kXRegion;

  // MFMA j of a step takes the lane's K segment 4*(j/2) + 2*half + j%2, of
  // X row 32*wave + l32 and weight row 32*cb + l32. Both are read from rows
  // whose swizzle is (l32 ^ (l32 >> 3)) & 7, with 4 more for odd cb (row
  // 32*cb + l32 has (row >> 3) & 7 = 4*(cb & 1) + (l32 >> 3)): per j one X
  // offset and two weight offsets, the block's 4096*cb an immediate offset.
  const int s0 = (l32 ^ (l32 >> 3)) & 7;
  int xseg[4], xoff[4], boff[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    xseg[j] = 4 * (j >> 1) + 2 * half + (j & 1);
    xoff[j] = l32 * kRowBytes + ((xseg[j] ^ s0) << 4);
#pragma unroll
    for (int p = 0; p < 2; ++p) boff[j][p] = l32 * kRowBytes + ((xseg[j] ^ s0 ^ (4 * p)) << 4);
  }

  // X loads: instruction q fills rows 8q .. 8q+7 of the wave's region; lane
  // (lrow, lslot) loads row 8q + lrow's segment lslot ^ swizzle(8q + lrow) =
  // lslot ^ ((lrow ^ q) & 7). The wave's and the instruction's rows are a
  // uniform part of the offset.
  const int xrows = m - m0 < kTM ? m - m0 : kTM;
  const bool computes = 32 * wave < xrows;  // wave-uniform: a row of this wave is below m
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(x + static_cast<long long>(m0) * hv), 0, xrows * hidden * 2,
      kRawBufferWord3);
  int xvo[kXInst], xslot[kXInst];
#pragma unroll
  for (int q = 0; q < kXInst; ++q) {
    xslot[q] = lslot ^ ((lrow ^ q) & 7);
    xvo[q] = lrow * hv * 16 + xslot[q] * 16;
  }

  // Weight loads: instruction q of wave w fills stage rows 8*g .. 8*g+7,
  // g = 8q + w, so (g & 7) = w and one lane offset serves every instruction;
  // the row group's part of the offset is uniform.
  const int wslot = lslot ^ ((lrow ^ wave) & 7);
  const int wvo = lrow * hv * 16 + wslot * 16;
  __amdgpu_buffer_rsrc_t wres0;
  if constexpr (ONE_RANK) {
    const int r = n0 / shard;
    const int trows = vocab - n0 < kTN ? vocab - n0 : kTN;
    wres0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(w.p[r] + static_cast<long long>(n0 - r * shard) * hv), 0,
        trows * hidden * 2, kRawBufferWord3);
  }
  auto wsrc = [&](int q, int *row_off) __attribute__((always_inline)) {
    const int g = NW * q + wave;
    if constexpr (ONE_RANK) {
      *row_off = 8 * g * hv * 16;
      return wres0;
    } else {
      const int nfirst = n0 + 8 * g;
      const int r = nfirst < vocab ? nfirst / shard : 0;
      const int s0r = nfirst < vocab ? nfirst - r * shard : 0;
      const int grows = nfirst < vocab ? (vocab - nfirst < 8 ? vocab - nfirst : 8) : 0;
      *row_off = 0;
      return __builtin_amdgcn_make_buffer_rsrc(
          const_cast<u32x4 *>(w.p[r] + static_cast<long long>(s0r) * hv), 0, grows * hidden * 2,
          kRawBufferWord3);
    }
  };

  // Loads of step kb (the step's K offset is part of the scalar offset).
  auto issue_w = [&](int kb) __attribute__((always_inline)) {
    unsigned char *st = lds + (kb % ST) * kStage;
#pragma unroll
    for (int q = 0; q < kWInst; ++q) {
      int row_off = 0;
      const __amdgpu_buffer_rsrc_t rs = wsrc(q, &row_off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(st + 8 * (NW * q + wave) * kRowBytes), 16,
          wvo, row_off + kb * kRowBytes, 0, kPolicyNt);
    }
  };
  auto issue_x = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kXInst; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void *)(xreg + 8 * q * kRowBytes), 16, xvo[q],
          (32 * wave + 8 * q) * hv * 16 + kb * kRowBytes, 0, 0);
  };

  f32x16 acc[kBlocks];
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) acc[cb] = f32x16{};

  const bool ktail = hidden % KS != 0;

  // One K step. In the steady state (MAIN) the step always issues X(kb+1)
  // and the weights of step kb+ST-1, so the compiler's wait counts follow one
  // straight path; the last ST-1 steps (and a wave with no row below m) take
  // the general form, which waits for everything outstanding.
  auto step = [&](auto main, auto comp, int kb) __attribute__((always_inline)) {
    constexpr bool MAIN = decltype(main)::value, COMP = decltype(comp)::value;
    if constexpr (MAIN)
      wait_vm<kWInst>();  // X(kb) and every older weight load have landed
    else
      wait_vm<0>();
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    unsigned char *sw = lds + (kb % ST) * kStage;
    bf16x8 xa[4];
    if constexpr (COMP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[j] = *reinterpret_cast<const bf16x8 *>(xreg + xoff[j]);
    }
    if constexpr (!MAIN) {
      if (ktail && kb == steps - 1) {
#pragma unroll
        for (int q = 0; q < kWInst; ++q)
          if (kb * kSlots + wslot >= hv)
            *reinterpret_cast<u32x4 *>(sw + (8 * (NW * q + wave) + lrow) * kRowBytes +
                                       lslot * 16) = u32x4{0u, 0u, 0u, 0u};
        if constexpr (COMP) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kb * kSlots + xseg[j] >= hv) xa[j] = bf16x8{};
        }
        __syncthreads();
      }
    }
    // X(kb+1) may only refill the region once the X reads above have
    // returned (lgkmcnt(0)), and it goes out before the weights so that the
    // next step's single wait covers it.
    auto loads = [&]() __attribute__((always_inline)) {
      if constexpr (COMP) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): X(kb) is in registers
        __asm__ __volatile__("" ::: "memory");
      }
      if constexpr (MAIN) {
        if constexpr (COMP) issue_x(kb + 1);
        issue_w(kb + ST - 1);
      } else {
        if (COMP && kb + 1 < steps) issue_x(kb + 1);
        if (kb + ST - 1 < steps) issue_w(kb + ST - 1);
      }
      __asm__ __volatile__("" ::: "memory");
    };
    if constexpr (COMP) loads();
    if constexpr (COMP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int cb = 0; cb < kBlocks; ++cb) {
          const bf16x8 b = *reinterpret_cast<const bf16x8 *>(sw + boff[j][cb & 1] +
                                                             cb * 32 * kRowBytes);
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[j], b, acc[cb], 0, 0, 0);
        }
      }
    } else {
      loads();
    }
  };

  // Steps 0 .. nmain-1 are steady-state steps, the rest general ones.
  const int nmain = steps > ST - 1 ? steps - (ST - 1) : 0;
  auto run = [&](auto comp) __attribute__((always_inline)) {
    constexpr bool COMP = decltype(comp)::value;
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    if constexpr (COMP) issue_x(0);
#pragma unroll
    for (int s = 0; s < ST - 1; ++s)
      if (s < steps) issue_w(s);
    // (X of step 0 goes out before the weights of steps 0 .. ST-2, so the
    // first wait covers it.)
    int kb = 0;
    for (; kb < nmain; ++kb) step(T{}, comp, kb);
    for (; kb < steps; ++kb) step(F{}, comp, kb);
  };
  if (computes) {
    run(std::integral_constant<bool, true>{});
  } else {
    run(std::integral_constant<bool, false>{});  // no row of this wave below m: loads only
    return;
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < kBlocks; ++cb) {
    const int c0 = n0 + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[cb][4 * q + t]);
      // lanes 2c and 2c+1 hold columns 2c and 2c+1 of rows rbase .. rbase+3;
      // one swap gives each the words (two adjacent columns) of two rows
      const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
      const uint32_t recv = swap_adjacent(send);
      const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
      const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
      const int rbase = m0 + 32 * wave + 8 * q + 4 * half;
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

// ---------------------------------------------------------------------------
// 4 x 2 wave layout: wave w owns rows 64*(w>>1) .. +63 of the 256-row tile
// and columns 160*(w&1) .. +159: 2 x 5 blocks of 32 x 32. K steps of 64,
// 128-byte LDS rows with the same swizzle as above. Weights: 3 stages of
// 320 rows (40 KB), two steps ahead. X of the whole tile: one shared 32 KB
// stage; each wave reads its 64 rows x 64 K into registers (32 VGPRs) right
// after the step's first barrier, and a second barrier (after the first K
// slice of MFMAs) frees the stage for X(kb+1), which goes out before the
// weights of step kb+2 so that the next step's wait leaves those in flight.
template <int NT, bool ONE_RANK, bool PUSH, bool KEEP>
__global__ __launch_bounds__(512) void k_lmhead_4x2(const u32x4 *x, ShardTableN<NT> w,
                                                  OutTableN<NT> shards_out, ParityArg pa, int m,
                                                  int hidden, int shard, int vocab) {
  constexpr int ST = 3;
  constexpr int NW = 8;
  constexpr int KS = 64;
  constexpr int kTN = 320;
  constexpr int kRowBytes = 128;
  constexpr int kSlots = 8;
  constexpr int kWStage = kTN * kRowBytes;  // 40 KB
  constexpr int kXStage = kTM * kRowBytes;  // 32 KB
  constexpr int kInstBytes = 8 * kRowBytes;
  constexpr int kWInst = kTN / 8 / NW;      // 5
  constexpr int kXInst = kTM / 8 / NW;      // 4
  __shared__ __attribute__((aligned(1024))) unsigned char lds[ST * kWStage + kXStage];
  unsigned char *const xlds = lds + ST * kWStage;

  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wr = wave >> 1, wc = wave & 1;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int n0 = static_cast<int>(blockIdx.x) * kTN;
  const int m0 = static_cast<int>(blockIdx.y) * kTM;
  const int hv = hidden >> 3;
  const int steps = (hidden + KS - 1) / KS;
  const int lrow = lane >> 3, lslot = lane & 7;

  // DMA: instruction t = 8q + wave fills rows 8t .. 8t+7 of a stage; lane
  // (lrow, lslot) loads logical segment lslot ^ swizzle(8t + lrow), and
  // swizzle(8t + lrow) = (lrow ^ t) & 7 = (lrow ^ wave) & 7 for every q.
  const int dseg = lslot ^ ((lrow ^ wave) & 7);
  const int dvo = lrow * hv * 16 + dseg * 16;

  // fragment offsets: MFMA j takes logical segment 4*(j>>1) + 2*half + (j&1);
  // rows 32*b + l32 with b even or odd differ by 4 in the swizzle
  const int s0 = (l32 ^ (l32 >> 3)) & 7;
  int fseg[4], foff[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    fseg[j] = 4 * (j >> 1) + 2 * half + (j & 1);
#pragma unroll
    for (int p = 0; p < 2; ++p) foff[j][p] = l32 * kRowBytes + ((fseg[j] ^ s0 ^ (4 * p)) << 4);
  }

  const int xrows = m - m0 < kTM ? m - m0 : kTM;
  const bool computes = 64 * wr < xrows;  // wave-uniform
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(x + static_cast<long long>(m0) * hv), 0, xrows * hidden * 2,
      kRawBufferWord3);

  __amdgpu_buffer_rsrc_t wres0;
  if constexpr (ONE_RANK) {
    const int r = n0 / shard;
    const int trows = vocab - n0 < kTN ? vocab - n0 : kTN;
    wres0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4 *>(w.p[r] + static_cast<long long>(n0 - r * shard) * hv), 0,
        trows * hidden * 2, kRawBufferWord3);
  }
  auto wsrc = [&](int t, int *row_off) __attribute__((always_inline)) {
    if constexpr (ONE_RANK) {
      *row_off = 8 * t * hv * 16;
      return wres0;
    } else {
      const int nfirst = n0 + 8 * t;
      const int r = nfirst < vocab ? nfirst / shard : 0;
      const int s0r = nfirst < vocab ? nfirst - r * shard : 0;
      const int grows = nfirst < vocab ? (vocab - nfirst < 8 ? vocab - nfirst : 8) : 0;
      *row_off = 0;
      return __builtin_amdgcn_make_buffer_rsrc(
          const_cast<u32x4 *>(w.p[r] + static_cast<long long>(s0r) * hv), 0, grows * hidden * 2,
          kRawBufferWord3);
    }
  };
  auto issue_w = [&](int kb, int slot) __attribute__((always_inline)) {
    unsigned char *st = lds + slot * kWStage;
#pragma unroll
    for (int q = 0; q < kWInst; ++q) {
      const int t = NW * q + wave;
      int row_off = 0;
      const __amdgpu_buffer_rsrc_t rs = wsrc(t, &row_off);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(st + t * kInstBytes), 16, dvo,
          row_off + kb * kRowBytes, 0, kPolicyNt);
    }
  };
  auto issue_x = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kXInst; ++q) {
      const int t = NW * q + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void *)(xlds + t * kInstBytes), 16, dvo,
          8 * t * hv * 16 + kb * kRowBytes, 0, 0);
    }
  };

  f32x16 acc[10];
#pragma unroll
  for (int b = 0; b < 10; ++b) acc[b] = f32x16{};

  const bool ktail = hidden % KS != 0;
  const int xbase = 64 * wr * kRowBytes;
  const int wbase = 160 * wc * kRowBytes;

  auto step = [&](auto main, auto comp, int kb, int ws) __attribute__((always_inline)) {
    constexpr bool MAIN = decltype(main)::value, COMP = decltype(comp)::value;
    if constexpr (MAIN)
      wait_vm<kWInst>();  // X(kb) and W(kb) have landed; W(kb+1) may not have
    else
      wait_vm<0>();
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
    unsigned char *sw = lds + ws * kWStage + wbase;
    bf16x8 xa[2][4];
    if constexpr (COMP) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xa[rb][j] =
              *reinterpret_cast<const bf16x8 *>(xlds + xbase + rb * 32 * kRowBytes + foff[j][rb]);
    }
    if constexpr (!MAIN) {
      if (ktail && kb == steps - 1) {
        if (kb * kSlots + dseg >= hv) {
          unsigned char *st = lds + ws * kWStage;
#pragma unroll
          for (int q = 0; q < kWInst; ++q)
            *reinterpret_cast<u32x4 *>(st + (NW * q + wave) * kInstBytes + lane * 16) =
                u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (COMP) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kb * kSlots + fseg[j] >= hv) {
              xa[0][j] = bf16x8{};
              xa[1][j] = bf16x8{};
            }
        }
        __syncthreads();
      }
    }
    // After the second barrier every wave holds X(kb) in registers: X(kb+1)
    // may refill the stage, then the weights of step kb+2 go out (into the
    // stage read in step kb-1).
    auto loads = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's X reads are done
      __asm__ __volatile__("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      __asm__ __volatile__("" ::: "memory");
      const int wnext = ws == 0 ? ST - 1 : ws - 1;
      if constexpr (MAIN) {
        issue_x(kb + 1);
        issue_w(kb + 2, wnext);
      } else {
        if (kb + 1 < steps) issue_x(kb + 1);
        if (kb + 2 < steps) issue_w(kb + 2, wnext);
      }
      __asm__ __volatile__("" ::: "memory");
    };
    if constexpr (COMP) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int cb = 0; cb < 5; ++cb) {
          const bf16x8 b = *reinterpret_cast<const bf16x8 *>(sw + cb * 32 * kRowBytes +
                                                             foff[j][(wc + cb) & 1]);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb * 5 + cb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[rb][j], b, acc[rb * 5 + cb], 0, 0, 0);
        }
        if (j == 0) loads();
      }
    } else {
      loads();
    }
  };

  const int nmain = steps > 2 ? steps - 2 : 0;
  auto run = [&](auto comp) __attribute__((always_inline)) {
    using T = std::integral_constant<bool, true>;
    using F = std::integral_constant<bool, false>;
    issue_x(0);
    issue_w(0, 0);
    if (1 < steps) issue_w(1, 1);
    int kb = 0, ws = 0;
    for (; kb < nmain; ++kb) {
      step(T{}, comp, kb, ws);
      ws = ws == ST - 1 ? 0 : ws + 1;
    }
    for (; kb < steps; ++kb) {
      step(F{}, comp, kb, ws);
      ws = ws == ST - 1 ? 0 : ws + 1;
    }
  };
  if (computes) {
    run(std::integral_constant<bool, true>{});
  } else {
    run(std::integral_constant<bool, false>{});
    return;
  }

  const bool even = (l32 & 1) == 0;
  const int words_per_shard_row = shard >> 1;
  const int words_per_row = vocab >> 1;
  uint32_t *box = PUSH ? reinterpret_cast<uint32_t *>(pa.box + launch_parity(pa) * pa.stride)
                       : nullptr;
#pragma unroll
  for (int cb = 0; cb < 5; ++cb) {
    const int c0 = n0 + 160 * wc + 32 * cb;
    if (c0 >= vocab) continue;
    const int r = c0 / shard;
    const int s_even = c0 - r * shard + (l32 & ~1);
    const int wcol = s_even >> 1;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t b[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = bf16_bits(acc[rb * 5 + cb][4 * q + t]);
        const uint32_t send = even ? (b[1] | (b[3] << 16)) : (b[0] | (b[2] << 16));
        const uint32_t recv = swap_adjacent(send);
        const uint32_t w0 = even ? (b[0] | (recv << 16)) : ((recv & 0xFFFFu) | (b[1] << 16));
        const uint32_t w1 = even ? (b[2] | (recv & 0xFFFF0000u)) : ((recv >> 16) | (b[3] << 16));
        const int rbase = m0 + 64 * wr + 32 * rb + 8 * q + 4 * half;
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

// The 8 x 1 layout streams the weights fastest when few rows compute (one
// wave's MFMAs per tile at M = 1); from 128 rows on, the 4 x 2 layout, with
// 36 % fewer LDS fragment reads per step, is the faster (measured 570 against
// 598 us at M = 256 and 431 against 446 us at M = 128, interleaved runs).
constexpr int k4x2Rows = 128;

template <int NT, bool ONE_RANK>
hipError_t launch_lmhead_one(const u32x4 *x, const ShardTableN<NT> &wt, const OutTableN<NT> &ot,
                             bool keep, bool push, const ParityArg &box, int m, int hidden,
                             int shard, int vocab, hipStream_t s) {
  const dim3 grid((vocab + 319) / 320, (m + kTM - 1) / kTM);
  auto go = [&](auto wide) {
    constexpr bool W = decltype(wide)::value;
    auto launch = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(512), 0, s, x, wt, ot, box, m, hidden, shard, vocab);
    };
    if (push && keep) {
      if constexpr (W) launch(k_lmhead_4x2<NT, ONE_RANK, true, true>);
      else launch(k_lmhead<NT, ONE_RANK, true, true>);
    } else if (push) {
      if constexpr (W) launch(k_lmhead_4x2<NT, ONE_RANK, true, false>);
      else launch(k_lmhead<NT, ONE_RANK, true, false>);
    } else {
      if constexpr (W) launch(k_lmhead_4x2<NT, ONE_RANK, false, true>);
      else launch(k_lmhead<NT, ONE_RANK, false, true>);
    }
  };
  if (m >= k4x2Rows)
    go(std::integral_constant<bool, true>{});
  else
    go(std::integral_constant<bool, false>{});
  return hipGetLastError();
}

template <int NT>
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
  if (shard % 320 == 0)
    return launch_lmhead_one<NT, true>(x, wt, ot, keep, push, box, m, hidden, shard, vocab, s);
  return launch_lmhead_one<NT, false>(x, wt, ot, keep, push, box, m, hidden, shard, vocab, s);
}

}  // namespace

hipError_t launch_lmhead(const u32x4 *x, const ShardTable &w, const OutTable &shards_out, bool keep,
                         bool push, const ParityArg &box, int m, int hidden, int shard, int tp,
                         hipStream_t s) {
  if (tp <= kSmallTable)
    return launch_lmhead_nt<kSmallTable>(x, w, shards_out, keep, push, box, m, hidden, shard, tp,
                                         s);
  return launch_lmhead_nt<HG_MAX_TP>(x, w, shards_out, keep, push, box, m, hidden, shard, tp, s);
}

}  // namespace hg
