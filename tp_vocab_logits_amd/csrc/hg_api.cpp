// Host side of libhg.so: the context, argument checks, parity state and
// launch shapes of the one-shot Lamport-mailbox logits gather. The C ABI is
// declared (and documented) in include/hg.h.
//
// Behaviour follows the vLLM API documentation page
// "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather":
//  - construction allocates the two-parity mailbox, arms it and synchronises
//    the device; the parity starts at 0 (HeadGather.__init__ source);
//  - a call is served only for a served row count and outside graph capture,
//    otherwise the caller takes the stock path and nothing changes; a served
//    call takes the current parity and flips it (HeadGather.__call__ source).
//    On request the parity lives in device memory instead, where the kernels
//    advance it; calls under capture are then served too;
//  - shard widths that are not a multiple of 8 are refused (_install_gather
//    source) and so is a TP of 1 (install_logits_gather source).

#include <stdint.h>
#include <string.h>

#include <new>

#include "hg_internal.h"

#define HG_API extern "C" __attribute__((visibility("default")))

using hg::Geometry;
using hg::ShardTable;
using hg::u32x4;

namespace {

constexpr unsigned long long kDefaultPollLimit = 1ull << 24;
constexpr int kSlotsOffset = 256;
constexpr int kStatusBytes = kSlotsOffset + 4 * hg::kParitySlots;

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char *where) {
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", where, hipGetErrorString(e),
           static_cast<int>(e));
  return HG_EHIP;
}

}  // namespace

namespace hg {

int record_hip_error(hipError_t e, const char *where) { return hip_fail(e, where); }

void record_error(const char *what) { snprintf(g_last_error, sizeof g_last_error, "%s", what); }

}  // namespace hg

namespace {

#define HIP_TRY(expr)                                 \
  do {                                                \
    hipError_t e_ = (expr);                           \
    if (e_ != hipSuccess) return hip_fail(e_, #expr); \
  } while (0)

// Launch shape (hg::kBlock, hg::kGridPerCu, hg::kPollSkew, hg::mailbox_vpt),
// chosen by sweeps on MI355X (TP=8, V=163840, M = 1..256): 128-bit
// agent-coherent pushes and polls move the M=256 gather at about 85 % of HBM
// peak against about 60 % for pairs of 64-bit atomics; four resident
// 256-thread workgroups per CU beat the full co-resident grid; a poll skew of
// 1 keeps every poll on data pushed by a workgroup on another XCD, within
// about 0.1 us per M=1 call of self-polling. One vector per lane while the
// call is small (latency: spread it over many waves), two when it is large
// (more bytes in flight per lane); measured under graph replay (TP=8,
// V=163840): M=4 takes 4.22 us with one against 4.48 with two; M=64 17.1 us
// with two against 18.4 with one and 17.4 with four; M=256 61.8 us with two
// against 63.0 with four.
using hg::kBlock;
using hg::kPollSkew;
using hg::mailbox_vpt;

// The stock concatenation (a plain copy, no polling) keeps its own
// thresholds, up to four vectors per lane.
int stock_vpt(long long vectors, int cus) {
  const long long lanes = static_cast<long long>(cus) * 256;
  if (vectors <= lanes) return 1;
  if (vectors <= 4 * lanes) return 2;
  return 4;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

}  // namespace

struct hg_ctx {
  int tp = 0, shard = 0, cap = 0;
  int device = -1;
  int cus = 0;
  long long vv = 0;             // 16-byte vectors per mailbox row
  int vocab = 0;                // BF16 columns per output row (padded-vocab slice), 1..tp*shard
  u32x4 *box = nullptr;         // [2][cap][vv]
  unsigned *status = nullptr;   // [0] poll timeouts; parity slots from byte kSlotsOffset on
  bool dev_parity = false;      // parity kept in device memory (graph-capturable calls)
  int parity = 0;
  int pending_m = -1;           // split push awaiting its collect
  int pending_parity = 0;
  unsigned long long pending_ranks = 0;  // ranks that pushed into it
  unsigned long long poll_limit = kDefaultPollLimit;
  // resident fused workgroups per CU, [vpt - 1][wide]; -1 unknown
  int fused_per_cu[2][2];

  u32x4 *parity_box(int p) const { return box + static_cast<long long>(p) * cap * vv; }
  int *parity_slots() const { return reinterpret_cast<int *>(status + kSlotsOffset / 4); }
  // Parity selection of a launch: host parity `p` in host mode, the device
  // slots in device mode; `flip` on the launch that completes a call, whose
  // grid and block give the slots' layout (one slot per wave).
  hg::ParityArg parity_arg(int p, bool flip, int grid = 0, int block = 0) const {
    hg::ParityArg pa;
    pa.box = box;
    pa.stride = static_cast<long long>(cap) * vv;
    pa.dev = dev_parity ? parity_slots() : nullptr;
    pa.p = p;
    pa.flip = flip ? 1 : 0;
    const int n = grid * (block / 64);  // waves of the completing launch
    pa.waves = block / 64;
    pa.per = n > 0 ? hg::kParitySlots / n : 0;
    pa.last = n - 1;
    return pa;
  }
  size_t row_bytes() const { return static_cast<size_t>(vv) * 16; }
  size_t out_row_bytes() const { return static_cast<size_t>(vocab) * 2; }
  hg::OutRows out_rows(void *out) const {
    hg::OutRows o;
    o.ptr = static_cast<u32x4 *>(out);
    o.cols = vocab;
    o.cvec = vocab % 8 == 0 ? vocab / 8 : 0;
    return o;
  }
};

namespace {

// Resident fused workgroups per CU for this variant (queried once per
// variant).
int fused_per_cu(hg_ctx *h, const hg::Modes &md, int *n) {
  int &slot = h->fused_per_cu[md.vpt - 1][md.wide];
  if (slot < 0) {
    int v = 0;
    HIP_TRY(hg::fused_blocks_per_cu(md, h->tp, kBlock, &v));
    slot = v;
  }
  *n = slot;
  return HG_OK;
}

int check_device(const hg_ctx *h) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != h->device) return HG_EINVAL;
  return HG_OK;
}

// HG_OK if not capturing, HG_EDECLINE if capturing, HG_EHIP on failure.
int capture_state(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(s, &st);
  if (e == hipErrorStreamCaptureImplicit || e == hipErrorStreamCaptureUnsupported) {
    (void)hipGetLastError();
    return HG_EDECLINE;
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  return st == hipStreamCaptureStatusNone ? HG_OK : HG_EDECLINE;
}

unsigned long long all_ranks(int tp) { return tp >= 64 ? ~0ull : (1ull << tp) - 1; }

// Checks the shard pointers of an m-row call for the ranks in `ranks` and
// fills the kernel table (other entries stay null and are never read).
int load_shards(int tp, int shard, const void *const *shards, int m, unsigned long long ranks,
                ShardTable *t, const void *out, size_t out_bytes, const void *box,
                size_t box_bytes) {
  if (!shards) return HG_EINVAL;
  memset(t, 0, sizeof *t);
  const size_t shard_bytes = static_cast<size_t>(m) * shard * 2;
  for (int r = 0; r < tp; ++r) {
    if (!((ranks >> r) & 1ull)) continue;
    const void *p = shards[r];
    if (!p || !aligned16(p)) return HG_EINVAL;
    if (overlaps(p, shard_bytes, out, out_bytes)) return HG_EINVAL;
    if (box && overlaps(p, shard_bytes, box, box_bytes)) return HG_EINVAL;
    t->p[r] = static_cast<const u32x4 *>(p);
  }
  return HG_OK;
}

int fused_grid(hg_ctx *h, const hg::Modes &md, const Geometry &g, int *grid) {
  int per_cu = 0;
  const int rc = fused_per_cu(h, md, &per_cu);
  if (rc != HG_OK) return rc;
  *grid = hg::fused_launch_grid(g.chunks, per_cu, h->cus);
  return *grid >= 1 ? HG_OK : HG_EINVAL;
}

int split_grid(const hg_ctx *h, const Geometry &g, int block) {
  const int waves = block / 64;
  const long long tiles = (static_cast<long long>(g.chunks) + waves - 1) / waves;
  long long cap = static_cast<long long>(h->cus) * 16;
  if (cap > hg::kParitySlots / waves) cap = hg::kParitySlots / waves;  // one slot per wave
  return static_cast<int>(tiles < cap ? tiles : cap);
}

// The kernel variant for an m-row call. The 128-bit coherent flavours address
// the rows in use through a buffer resource with 32-bit offsets; a call whose
// rows span 4 GiB or more uses the 64-bit atomic flavours instead.
hg::Modes pick_modes(const hg_ctx *h, int m) {
  hg::Modes md;
  md.vpt = mailbox_vpt(static_cast<long long>(m) * h->vv, h->cus);
  md.wide = static_cast<unsigned long long>(m) * h->row_bytes() >= (1ull << 32) ? 1 : 0;
  return md;
}

unsigned used_box_bytes(const hg_ctx *h, int m) {
  const unsigned long long b = static_cast<unsigned long long>(m) * h->row_bytes();
  return b >= (1ull << 32) ? 0u : static_cast<unsigned>(b);
}

// Common checks of hg_gather / hg_push_ranks. Returns HG_OK when the call is
// served. `joining`: a push that may join a pending call of the same m.
int check_call(hg_ctx *h, const void *const *shards, int m, unsigned long long ranks,
               bool joining, const void *out, void *stream, ShardTable *table) {
  if (!h || m < 0) return HG_EINVAL;
  if (ranks == 0 || (ranks & ~all_ranks(h->tp))) return HG_EINVAL;
  if (h->pending_m >= 0) {
    if (!joining || m != h->pending_m || (ranks & h->pending_ranks)) return HG_ESTATE;
  }
  if (m == 0 || m > h->cap) return HG_EDECLINE;
  const int cs = capture_state(static_cast<hipStream_t>(stream));
  if (cs < 0) return cs;
  if (cs == HG_EDECLINE && !h->dev_parity) return HG_EDECLINE;  // host parity cannot be replayed
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  const size_t out_bytes = static_cast<size_t>(m) * h->out_row_bytes();
  const size_t box_bytes = static_cast<size_t>(2) * h->cap * h->row_bytes();
  if (out) {
    if (!aligned16(out) || overlaps(out, out_bytes, h->box, box_bytes)) return HG_EINVAL;
  }
  return load_shards(h->tp, h->shard, shards, m, ranks, table, out, out ? out_bytes : 0, h->box,
                     box_bytes);
}

}  // namespace

HG_API int hg_create(int tp, int shard, int cap, hg_ctx **out) {
  if (!out) return HG_EINVAL;
  *out = nullptr;
  if (tp < 2 || tp > HG_MAX_TP || shard < 8 || shard % 8 != 0 || cap < 1) return HG_EINVAL;
  const long long vv = static_cast<long long>(tp) * (shard / 8);
  if (vv * cap >= (1ll << 31)) return HG_EINVAL;

  hg_ctx *h = new (std::nothrow) hg_ctx;
  if (!h) return HG_ENOMEM;
  h->tp = tp;
  h->shard = shard;
  h->cap = cap;
  h->vv = vv;
  h->vocab = tp * shard;
  auto fail = [&](int rc) {
    if (h->box) (void)hipFree(h->box);
    if (h->status) (void)hipFree(h->status);
    delete h;
    return rc;
  };
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) return fail(hip_fail(e, "hipGetDevice"));
  e = hipDeviceGetAttribute(&h->cus, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess) return fail(hip_fail(e, "hipDeviceGetAttribute"));
  const size_t box_bytes = static_cast<size_t>(2) * cap * vv * 16;
  e = hipMalloc(reinterpret_cast<void **>(&h->box), box_bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(e == hipErrorOutOfMemory ? HG_ENOMEM : hip_fail(e, "hipMalloc(mailbox)"));
  }
  e = hipMalloc(reinterpret_cast<void **>(&h->status), kStatusBytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(e == hipErrorOutOfMemory ? HG_ENOMEM : hip_fail(e, "hipMalloc(status)"));
  }
  e = hipMemset(h->status, 0, kStatusBytes);
  if (e != hipSuccess) return fail(hip_fail(e, "hipMemset(status)"));
  for (auto &a : h->fused_per_cu)
    for (int &c : a) c = -1;
  int rc = hg_arm(h, nullptr);
  if (rc != HG_OK) return fail(rc);
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(hip_fail(e, "hipDeviceSynchronize"));
  *out = h;
  return HG_OK;
}

HG_API int hg_destroy(hg_ctx *h) {
  if (!h) return HG_OK;
  int prev = -1;
  int rc = HG_OK;
  if (hipGetDevice(&prev) == hipSuccess && prev != h->device) (void)hipSetDevice(h->device);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) rc = hip_fail(e, "hipDeviceSynchronize");
  if (h->box) (void)hipFree(h->box);
  if (h->status) (void)hipFree(h->status);
  if (prev >= 0 && prev != h->device) (void)hipSetDevice(prev);
  delete h;
  return rc;
}

HG_API int hg_arm(hg_ctx *h, void *stream) {
  if (!h) return HG_EINVAL;
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  const long long vectors = 2ll * h->cap * h->vv;
  const int block = 256;
  long long grid = (vectors + block - 1) / block;
  if (grid > static_cast<long long>(h->cus) * 8) grid = static_cast<long long>(h->cus) * 8;
  HIP_TRY(hg::launch_arm(h->box, vectors, h->parity_slots(), static_cast<int>(grid), block,
                         static_cast<hipStream_t>(stream)));
  h->parity = 0;
  h->pending_m = -1;
  h->pending_ranks = 0;
  return HG_OK;
}

HG_API int hg_gather(hg_ctx *h, const void *const *shards, int m, void *out, void *stream) {
  ShardTable table;
  int rc = check_call(h, shards, m, h ? all_ranks(h->tp) : 0, false, out, stream, &table);
  if (rc != HG_OK) return rc;
  if (!out) return HG_EINVAL;
  const hg::Modes md = pick_modes(h, m);
  const Geometry g = hg::make_geometry(h->tp, h->shard, m, md.vpt);
  int grid = 0;
  rc = fused_grid(h, md, g, &grid);
  if (rc != HG_OK) return rc;
  const hg::ParityArg pa = h->parity_arg(h->parity, true, grid, kBlock);
  HIP_TRY(hg::launch_fused(table, g, md, pa, used_box_bytes(h, m), h->out_rows(out), h->status,
                           h->poll_limit, kPollSkew % grid, grid, kBlock,
                           static_cast<hipStream_t>(stream)));
  if (!h->dev_parity) h->parity ^= 1;
  return HG_OK;
}

HG_API int hg_push_ranks(hg_ctx *h, const void *const *shards, int m, unsigned long long ranks,
                         void *stream) {
  ShardTable table;
  int rc = check_call(h, shards, m, ranks, true, nullptr, stream, &table);
  if (rc != HG_OK) return rc;
  const int vpt = pick_modes(h, m).vpt;
  const Geometry g = hg::make_geometry(h->tp, h->shard, m, vpt);
  const int p = h->pending_m >= 0 ? h->pending_parity : h->parity;
  HIP_TRY(hg::launch_push(table, g, vpt, h->parity_arg(p, false), ranks, split_grid(h, g, kBlock),
                          kBlock, static_cast<hipStream_t>(stream)));
  h->pending_m = m;
  h->pending_parity = p;
  h->pending_ranks |= ranks;
  return HG_OK;
}

HG_API int hg_push(hg_ctx *h, const void *const *shards, int m, void *stream) {
  if (!h) return HG_EINVAL;
  if (h->pending_m >= 0) return HG_ESTATE;
  return hg_push_ranks(h, shards, m, all_ranks(h->tp), stream);
}

HG_API int hg_collect(hg_ctx *h, int m, void *out, void *stream) {
  if (!h || m < 0) return HG_EINVAL;
  if (h->pending_m < 0 || h->pending_m != m) return HG_ESTATE;
  const int cs = capture_state(static_cast<hipStream_t>(stream));
  if (cs < 0) return cs;
  if (cs == HG_EDECLINE && !h->dev_parity) return HG_EDECLINE;
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  const size_t out_bytes = static_cast<size_t>(m) * h->out_row_bytes();
  const size_t box_bytes = static_cast<size_t>(2) * h->cap * h->row_bytes();
  if (!out || !aligned16(out) || overlaps(out, out_bytes, h->box, box_bytes)) return HG_EINVAL;
  const hg::Modes md = pick_modes(h, m);
  const Geometry g = hg::make_geometry(h->tp, h->shard, m, md.vpt);
  const int grid = split_grid(h, g, kBlock);
  HIP_TRY(hg::launch_collect(g, md, h->parity_arg(h->pending_parity, true, grid, kBlock),
                             used_box_bytes(h, m), h->out_rows(out), h->status, h->poll_limit,
                             grid, kBlock, static_cast<hipStream_t>(stream)));
  h->pending_m = -1;
  h->pending_ranks = 0;
  if (!h->dev_parity) h->parity = h->pending_parity ^ 1;
  return HG_OK;
}

HG_API int hg_stock_gather(int tp, int shard, const void *const *shards, int m, void *out,
                           int vocab, void *stream) {
  if (tp < 1 || tp > HG_MAX_TP || shard < 1 || m < 0) return HG_EINVAL;
  const long long width = static_cast<long long>(tp) * shard;
  if (vocab < 1 || vocab > width) return HG_EINVAL;
  if (m == 0) return HG_OK;
  if (static_cast<long long>(m) * width >= (1ll << 34)) return HG_EINVAL;
  const bool vec = shard % 8 == 0;  // whole 16-byte vectors per shard row
  if (!out || !(vec ? aligned16(out) : aligned2(out))) return HG_EINVAL;
  if (!shards) return HG_EINVAL;
  ShardTable table;
  memset(&table, 0, sizeof table);
  const size_t out_bytes = static_cast<size_t>(m) * vocab * 2;
  const size_t shard_bytes = static_cast<size_t>(m) * shard * 2;
  for (int r = 0; r < tp; ++r) {
    const void *p = shards[r];
    if (!p || !(vec ? aligned16(p) : aligned2(p)) || overlaps(p, shard_bytes, out, out_bytes))
      return HG_EINVAL;
    table.p[r] = static_cast<const u32x4 *>(p);
  }
  int dev = 0, cus = 0;
  HIP_TRY(hipGetDevice(&dev));
  HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!vec) {
    const long long n = static_cast<long long>(m) * vocab;
    long long grid = (n + 255) / 256;
    if (grid > static_cast<long long>(cus) * 8) grid = static_cast<long long>(cus) * 8;
    HIP_TRY(hg::launch_stock_elem(table, tp, shard, m, static_cast<unsigned short *>(out), vocab,
                                  static_cast<int>(grid), 256, s));
    return HG_OK;
  }
  const long long vv = width / 8;
  if (vv * m >= (1ll << 31)) return HG_EINVAL;
  const int vpt = stock_vpt(m * vv, cus);
  const Geometry g = hg::make_geometry(tp, shard, m, vpt);
  const long long tiles = (static_cast<long long>(g.chunks) + 3) / 4;
  const long long cap = static_cast<long long>(cus) * 16;
  hg::OutRows o;
  o.ptr = static_cast<u32x4 *>(out);
  o.cols = vocab;
  o.cvec = vocab % 8 == 0 ? vocab / 8 : 0;
  HIP_TRY(hg::launch_stock(table, g, vpt, o, static_cast<int>(tiles < cap ? tiles : cap), 256, s));
  return HG_OK;
}

namespace {

// Size and pointer rules of the lm_head product; fills the kernel tables.
int check_lmhead(int tp, int shard, const void *x, const void *const *w, int hidden, int m,
                 void *const *shards_out, ShardTable *wt, hg::OutTable *ot) {
  if (tp < 1 || tp > HG_MAX_TP || shard < 32 || shard % 32 != 0 || hidden < 8 || hidden % 8 != 0 ||
      m < 0)
    return HG_EINVAL;
  if (static_cast<long long>(tp) * shard >= (1ll << 31)) return HG_EINVAL;
  if (m == 0) return HG_OK;  // nothing is read or written
  if (!x || !aligned16(x) || !w) return HG_EINVAL;
  memset(wt, 0, sizeof *wt);
  memset(ot, 0, sizeof *ot);
  const size_t x_bytes = static_cast<size_t>(m) * hidden * 2;
  const size_t w_bytes = static_cast<size_t>(shard) * hidden * 2;
  const size_t o_bytes = static_cast<size_t>(m) * shard * 2;
  for (int r = 0; r < tp; ++r) {
    if (!w[r] || !aligned16(w[r])) return HG_EINVAL;
    wt->p[r] = static_cast<const u32x4 *>(w[r]);
    if (shards_out) {
      void *o = shards_out[r];
      if (!o || !aligned16(o)) return HG_EINVAL;
      if (overlaps(o, o_bytes, x, x_bytes) || overlaps(o, o_bytes, w[r], w_bytes)) return HG_EINVAL;
      ot->p[r] = static_cast<uint32_t *>(o);
    }
  }
  return HG_OK;
}

}  // namespace

HG_API int hg_lmhead(int tp, int shard, const void *x, const void *const *w, int hidden, int m,
                     void *const *shards_out, void *stream) {
  if (!shards_out) return HG_EINVAL;
  ShardTable wt;
  hg::OutTable ot;
  const int rc = check_lmhead(tp, shard, x, w, hidden, m, shards_out, &wt, &ot);
  if (rc != HG_OK) return rc;
  if (m == 0) return HG_OK;
  hg::ParityArg none = {};
  HIP_TRY(hg::launch_lmhead(static_cast<const u32x4 *>(x), wt, ot, true, false, none, m, hidden,
                            shard, tp, static_cast<hipStream_t>(stream)));
  return HG_OK;
}

HG_API int hg_gemm_gather(hg_ctx *h, const void *x, const void *const *w, int hidden, int m,
                          void *out, void *const *shards_out, void *stream) {
  if (!h || m < 0) return HG_EINVAL;
  if (h->pending_m >= 0) return HG_ESTATE;
  if (m == 0 || m > h->cap) return HG_EDECLINE;
  const int cs = capture_state(static_cast<hipStream_t>(stream));
  if (cs < 0) return cs;
  if (cs == HG_EDECLINE && !h->dev_parity) return HG_EDECLINE;
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  ShardTable wt;
  hg::OutTable ot;
  rc = check_lmhead(h->tp, h->shard, x, w, hidden, m, shards_out, &wt, &ot);
  if (rc != HG_OK) return rc;
  // out, the mailbox, x, the weights and the shard copies must not overlap
  // one another (the shard copies are already checked against x and w)
  const size_t out_bytes = static_cast<size_t>(m) * h->out_row_bytes();
  const size_t box_bytes = static_cast<size_t>(2) * h->cap * h->row_bytes();
  const size_t w_bytes = static_cast<size_t>(h->shard) * hidden * 2;
  const size_t so_bytes = static_cast<size_t>(m) * h->shard * 2;
  if (!out || !aligned16(out) || overlaps(out, out_bytes, h->box, box_bytes) ||
      overlaps(out, out_bytes, x, static_cast<size_t>(m) * hidden * 2) ||
      overlaps(x, static_cast<size_t>(m) * hidden * 2, h->box, box_bytes))
    return HG_EINVAL;
  for (int r = 0; r < h->tp; ++r) {
    if (overlaps(out, out_bytes, w[r], w_bytes) || overlaps(w[r], w_bytes, h->box, box_bytes))
      return HG_EINVAL;
    if (shards_out && (overlaps(shards_out[r], so_bytes, h->box, box_bytes) ||
                       overlaps(shards_out[r], so_bytes, out, out_bytes)))
      return HG_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(hg::launch_lmhead(static_cast<const u32x4 *>(x), wt, ot, shards_out != nullptr, true,
                            h->parity_arg(h->parity, false), m, hidden, h->shard, h->tp, s));
  const hg::Modes md = pick_modes(h, m);
  const Geometry g = hg::make_geometry(h->tp, h->shard, m, md.vpt);
  const int grid = split_grid(h, g, kBlock);
  HIP_TRY(hg::launch_collect(g, md, h->parity_arg(h->parity, true, grid, kBlock),
                             used_box_bytes(h, m), h->out_rows(out), h->status, h->poll_limit,
                             grid, kBlock, s));
  if (!h->dev_parity) h->parity ^= 1;
  return HG_OK;
}

HG_API int hg_parity(const hg_ctx *h) {
  if (!h) return HG_EINVAL;
  if (!h->dev_parity) return h->parity;
  int v = -1;
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(&v, h->parity_slots(), sizeof v, hipMemcpyDeviceToHost));
  return v;
}

HG_API int hg_set_device_parity(hg_ctx *h, int enable, void *stream) {
  if (!h || (enable != 0 && enable != 1)) return HG_EINVAL;
  if (h->pending_m >= 0) return HG_ESTATE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cs = capture_state(s);
  if (cs == HG_EDECLINE) return HG_EINVAL;  // not while capturing
  if (cs != HG_OK) return cs;
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  if (enable && !h->dev_parity) {
    HIP_TRY(hg::launch_set_slots(h->parity_slots(), h->parity, s));
    h->dev_parity = true;
  } else if (!enable && h->dev_parity) {
    int v = 0;
    HIP_TRY(hipMemcpyAsync(&v, h->parity_slots(), sizeof v, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    h->parity = v & 1;
    h->dev_parity = false;
  }
  return HG_OK;
}

HG_API int hg_set_vocab(hg_ctx *h, int vocab) {
  if (!h || vocab < 1 || vocab > h->tp * h->shard) return HG_EINVAL;
  h->vocab = vocab;
  return HG_OK;
}

HG_API int hg_vocab(const hg_ctx *h) { return h ? h->vocab : HG_EINVAL; }

HG_API int hg_mailbox(const hg_ctx *h, int parity, const void **dev, size_t *bytes) {
  if (!h || (parity != 0 && parity != 1) || !dev || !bytes) return HG_EINVAL;
  *dev = h->parity_box(parity);
  *bytes = static_cast<size_t>(h->cap) * h->row_bytes();
  return HG_OK;
}

HG_API int hg_copy_mailbox(const hg_ctx *h, int parity, void *dst, void *stream) {
  if (!h || (parity != 0 && parity != 1) || !dst) return HG_EINVAL;
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  const size_t bytes = static_cast<size_t>(h->cap) * h->row_bytes();
  if (overlaps(dst, bytes, h->box, 2 * bytes)) return HG_EINVAL;
  HIP_TRY(hipMemcpyAsync(dst, h->parity_box(parity), bytes, hipMemcpyDeviceToDevice,
                         static_cast<hipStream_t>(stream)));
  return HG_OK;
}

HG_API int hg_set_poll_limit(hg_ctx *h, unsigned long long spins) {
  if (!h) return HG_EINVAL;
  h->poll_limit = spins ? spins : kDefaultPollLimit;
  return HG_OK;
}

HG_API int hg_poll_status(hg_ctx *h, void *stream) {
  if (!h) return HG_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int cs = capture_state(s);
  if (cs == HG_EDECLINE) return HG_EINVAL;
  if (cs != HG_OK) return cs;
  int rc = check_device(h);
  if (rc != HG_OK) return rc;
  unsigned count = 0;
  HIP_TRY(hipMemcpyAsync(&count, h->status, sizeof count, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  if (count == 0) return HG_OK;
  HIP_TRY(hipMemsetAsync(h->status, 0, sizeof count, s));
  HIP_TRY(hipStreamSynchronize(s));
  return HG_ETIMEOUT;
}

HG_API int hg_fused_grid_limit(hg_ctx *h, int m) {
  if (!h || m < 1 || m > h->cap) return HG_EINVAL;
  int per_cu = 0;
  const int rc = fused_per_cu(h, pick_modes(h, m), &per_cu);
  if (rc != HG_OK) return rc;
  return per_cu * h->cus;
}

HG_API const char *hg_strerror(int code) {
  switch (code) {
    case HG_OK: return "ok";
    case HG_EDECLINE: return "declined: take the stock gather";
    case HG_EINVAL: return "invalid argument";
    case HG_ENOMEM: return "device memory allocation failed";
    case HG_EHIP: return "HIP runtime error";
    case HG_ETIMEOUT: return "a bounded mailbox poll gave up";
    case HG_ESTATE: return "split push/collect called out of order";
    case HG_ESIZE: return "request exceeds the static scratch buffer";
    default: return "unknown status";
  }
}

HG_API const char *hg_last_error_detail(void) { return g_last_error; }
