/*
 * hg.h -- one-shot Lamport-mailbox gather of vocab-parallel lm_head logits,
 * for AMD MI355X (gfx950). C ABI of libhg.so.
 *
 * The operation (vLLM API documentation page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.logits_gather",
 * module description and HeadGather class description):
 *
 *   Each of TP ranks holds a [M, S] BF16 shard of the vocab-parallel lm_head
 *   logits (S = shard = V / TP). A gather call produces the [M, V] BF16 logits
 *   with rank r at columns r * S -- the layout of NCCL's all-gather -- through
 *   a mailbox of 2 parities x cap rows x V BF16 that is armed with a sentinel.
 *   A word is two adjacent BF16 elements (2k, 2k+1) of a row, read as a
 *   little-endian 32-bit value. The sentinel word is the pair (+0, -0),
 *   0x80000000; a shard word equal to it is written into the mailbox as
 *   (+0, +0), 0x00000000, every other byte moves unchanged. The consumer polls
 *   each mailbox word until it is not the sentinel, copies the row to the
 *   output and re-arms the mailbox. The parity alternates per served call.
 *
 * Here the TP ranks are virtual: every shard and the mailbox sit in the HBM of
 * the one device that was current at hg_create, and one kernel does the push,
 * poll, copy and re-arm for all of them.
 *
 * Conventions for every entry point:
 *  - Return value: HG_OK (0) on success; HG_EDECLINE (1) when the call is not
 *    served -- nothing was enqueued, no state changed, and the caller takes
 *    the stock path (hg_stock_gather, or its own all-gather); a negative
 *    HG_E* code on error (no state changed unless stated).
 *  - `stream` is a hipStream_t passed as void* (NULL: the null stream). Device
 *    work is enqueued on it and the call returns without waiting, unless
 *    stated otherwise.
 *  - Every device pointer must be 16-byte aligned (unless stated otherwise)
 *    and belong to the context's device, which must be the current device at
 *    the call (else HG_EINVAL).
 *  - Ownership: the context owns its mailbox and a status block of 65792
 *    bytes (the poll-timeout counter and 16384 device parity slots); the
 *    caller owns every shard, output and weight buffer.
 *  - Ordering: the library relies on the caller to issue every call on a
 *    context from one host thread at a time and on a single stream, in the
 *    order the calls are made. Stream order is what keeps a kernel from
 *    pushing into mailbox rows that an earlier kernel is still polling or
 *    re-arming; the library does not check it, so calls on two streams, or
 *    two contexts sharing buffers, can race (the pages state the same
 *    one-stream assumption: API page, HeadGather class description).
 */
#ifndef HG_H
#define HG_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of (virtual) ranks a context accepts. */
#define HG_MAX_TP 64

/* Status codes. */
#define HG_OK 0
#define HG_EDECLINE 1  /* not served: take the stock path; nothing enqueued     */
#define HG_EINVAL (-1) /* bad argument (sizes, null or misaligned pointer, ...) */
#define HG_ENOMEM (-2) /* device allocation failed                             */
#define HG_EHIP (-3)   /* a HIP runtime call failed (see hg_last_error_detail)  */
#define HG_ETIMEOUT (-4) /* a bounded poll gave up (reported by hg_poll_status)  */
#define HG_ESTATE (-5) /* split-variant call out of order                       */
#define HG_ESIZE (-6)  /* beyond the static scratch buffer (hg_gather_static)   */

typedef struct hg_ctx hg_ctx;

/*
 * Create a gather context for `tp` virtual ranks of `shard` BF16 columns each
 * and up to `cap` rows per call (API page, HeadGather.__init__ source: the
 * mailbox is allocated with 2 x cap x (shard/2 * tp) 32-bit words and armed;
 * the device is synchronised before returning; the parity starts at 0).
 *
 * Refused with HG_EINVAL: out == NULL; tp < 2 or tp > HG_MAX_TP (a TP of 1 is
 * declined by install_logits_gather); shard < 8 or shard % 8 != 0 (the
 * _install_gather source refuses other shard widths); cap < 1; a mailbox of
 * 2^31 or more 16-byte vectors per parity. HG_ENOMEM / HG_EHIP on device
 * failures. On success *out holds the context; on failure *out is NULL.
 * Served row counts are 1..cap.
 */
int hg_create(int tp, int shard, int cap, hg_ctx **out);

/* Free the mailbox and the context. NULL-safe. Synchronises the device first
 * so no enqueued kernel still uses the mailbox. The pages show no teardown of
 * the mailbox object (API page, HeadGather.__init__ source allocates it for
 * the life of the gather object); this is its end of life. */
int hg_destroy(hg_ctx *h);

/* Re-arm both parities to all-sentinel, reset the parity to 0 and drop any
 * pending split push (stream-ordered on `stream`). Recovery after an error.
 * The pages arm the mailbox only when it is built (API page, HeadGather
 * class description and HeadGather.__init__ source: a fresh mailbox is armed
 * and the parity starts at 0); re-arming later and resetting the parity with
 * it is our reading, so that an armed mailbox always starts at parity 0. */
int hg_arm(hg_ctx *h, void *stream);

/*
 * The gather, fused in one kernel launch (API page, HeadGather.__call__
 * source and module description).
 *
 * shards: host array of tp device pointers; shards[r] is rank r's [m][shard]
 *         BF16 block, row-major, contiguous (row stride = shard elements).
 * m:      rows to gather this call.
 * out:    device [m][vocab] BF16, row-major, 16-byte aligned (vocab =
 *         tp*shard unless hg_set_vocab chose fewer columns); gathered row i,
 *         which holds rank r's row i at columns r*shard .. r*shard+shard-1
 *         with every sentinel word rewritten to zero, is written to row i of
 *         `out` up to column vocab-1. Must not overlap the shards or the
 *         mailbox.
 *
 * HG_EDECLINE (stock path, parity unchanged) when m == 0, m > cap, or the
 * stream is capturing a graph while the parity is kept on the host (it cannot
 * alternate under replay; see hg_set_device_parity). HG_EINVAL for m < 0,
 * NULL / misaligned / overlapping pointers. HG_ESTATE if a split push is
 * pending. On HG_OK the parity flips.
 */
int hg_gather(hg_ctx *h, const void *const *shards, int m, void *out, void *stream);

/*
 * Split variant, first half: push the shards into the current parity's rows
 * 0..m-1 (sentinel words rewritten) and leave the call pending. This is the
 * push half of the one-shot kernel (API page, module description: each rank
 * writes its shard into row m of the mailbox at its column offset, with the
 * sentinel pair sent as (+0, +0)), launched on its own. Same arguments,
 * declines and errors as hg_gather; HG_ESTATE if a push is already pending
 * (the pages have no split call; refusing a second push before the collect
 * is our reading, as a pending call owns its parity's rows). The parity does
 * not change.
 */
int hg_push(hg_ctx *h, const void *const *shards, int m, void *stream);

/*
 * Split variant, partial push: only the ranks whose bit is set in `ranks`
 * (bit r = rank r) push their fragments; shards[r] is read only for those.
 * Each rank of a real TP group pushes its own fragment on its own schedule
 * (API page, module description: every rank pushes into every peer's mailbox
 * and the consumer polls until all fragments have landed); this entry point
 * lets virtual ranks do the same. The pages do not show pushes of separate
 * rank sets; accumulating them into one pending call, and letting a collect
 * with a rank missing give up through the bounded poll, is our reading.
 * Pushes of disjoint rank sets with the same m accumulate into one pending
 * call. HG_ESTATE if a rank already pushed into the pending call or m
 * differs from it; HG_EINVAL if `ranks` is empty or names a rank >= tp. A
 * collect issued while some rank has not pushed polls words that never
 * arrive: its bounded poll gives up (see hg_set_poll_limit /
 * hg_poll_status).
 */
int hg_push_ranks(hg_ctx *h, const void *const *shards, int m, unsigned long long ranks,
                  void *stream);

/*
 * Split variant, second half: poll rows 0..m-1 of the pending parity until no
 * word is the sentinel, copy them to `out` ([m][vocab] BF16, as for
 * hg_gather) and re-arm them; then flip the parity (API page, module
 * description: poll, copy, re-arm; HeadGather.__call__ source: the parity
 * flips once per served call). HG_ESTATE unless a push of the same m is
 * pending (from any set of ranks; not on the pages -- a collect with nothing
 * pushed would only poll until it gives up, so it is refused up front);
 * HG_EDECLINE (nothing changes) if the stream is capturing while the parity
 * is kept on the host.
 */
int hg_collect(hg_ctx *h, int m, void *out, void *stream);

/*
 * The stock gather's single-device share (API page, module description: the
 * all-gather into [TP, M, V/TP] followed by a copy to [M, V]) with the
 * padded-vocab slice applied (PR page, Purpose: the gathered logits keep the
 * real vocabulary's columns): rank-order concatenation, every byte unchanged
 * (no sentinel rewrite), of which the first `vocab` columns of each row are
 * written to out[m][vocab]. Needs no context; tp in [1, HG_MAX_TP],
 * shard >= 1, 1 <= vocab <= tp*shard, m >= 0 (m == 0 does nothing). With
 * shard % 8 == 0 the shards and `out` must be 16-byte aligned and rows move
 * in 16-byte vectors; other widths move element by element and need 2-byte
 * alignment. Only bytes move, so shards of another element type can pass
 * their row width and `vocab` in 2-byte units (bytes / 2). HG_EINVAL on a
 * bad size, a NULL or misaligned pointer, or a shard overlapping `out`.
 */
int hg_stock_gather(int tp, int shard, const void *const *shards, int m, void *out, int vocab,
                    void *stream);

/*
 * The lm_head shard product that feeds the gather (API page, module
 * description: the vocab-parallel lm_head produces the [M, V/TP] shards the
 * gather collects; install_logits_gather takes the shard width from the head
 * weight's first dimension): for every rank r,
 *     shards_out[r] = X @ W_r^T,   BF16 inputs, fp32 accumulation, BF16
 *                                  result rounded to nearest even.
 * x:          device [m][hidden] BF16, row-major.
 * w:          host array of tp device pointers; w[r] = rank r's head-weight
 *             rows [shard][hidden] BF16, row-major.
 * shards_out: host array of tp device pointers; shards_out[r] = [m][shard]
 *             BF16, row-major; must not overlap x or w.
 * HG_EINVAL unless 1 <= tp <= HG_MAX_TP, shard >= 32 and shard % 32 == 0,
 * hidden >= 8 and hidden % 8 == 0, m >= 0, pointers non-NULL and 16-byte
 * aligned. m == 0 does nothing. The result is deterministic (no split-K):
 * each output is one fixed chain of fp32 accumulations over the hidden
 * dimension, so repeated calls, and hg_gemm_gather, give the same bits.
 */
int hg_lmhead(int tp, int shard, const void *x, const void *const *w, int hidden, int m,
              void *const *shards_out, void *stream);

/*
 * Producer and gather: the lm_head product above whose epilogue pushes its
 * words -- sentinel rewritten -- straight into rows 0..m-1 of the current
 * parity (no shard round trip), then the collect kernel polls, copies to
 * `out` ([m][vocab] BF16, vocab as set by hg_set_vocab) and re-arms; the
 * parity flips. Two launches on `stream`. The PR page (Test Result) has the
 * one-shot gather launched early enough to overlap the tail of the LM-head
 * GEMM; here the GEMM's own epilogue is the push. When shards_out is
 * non-NULL the product's BF16 shards are also written there, bytes as
 * computed. Declines and state errors as hg_gather; the size rules of
 * hg_lmhead also apply. HG_EINVAL when `out`, the mailbox, x, any weight
 * block or any shards_out block overlap one another.
 */
int hg_gemm_gather(hg_ctx *h, const void *x, const void *const *w, int hidden, int m, void *out,
                   void *const *shards_out, void *stream);

/* The parity the next served call will use (0 or 1), or HG_EINVAL (API page,
 * HeadGather.__call__ source: a served call uses the current parity, then
 * flips it; a declined call leaves it). With device-side parity on, this
 * synchronises the device and reads it back. */
int hg_parity(const hg_ctx *h);

/*
 * Keep the parity in device memory (enable = 1) or on the host (0, the
 * default). Host-side parity cannot alternate when launches are replayed
 * from a graph, which is why calls under graph capture are otherwise
 * declined (API page, HeadGather class description and HeadGather.__call__
 * source). With device-side parity each launch reads the parity from device
 * memory when it starts and the launch that completes a call (fused gather,
 * collect) writes the other parity back as its workgroups finish, with no
 * wait between workgroups, so calls captured into a graph --
 * hg_gather, hg_push/hg_push_ranks + hg_collect, hg_gemm_gather -- are
 * served and every replay alternates. Switching on copies the host parity to
 * the device (stream-ordered); switching off waits for `stream` and copies it
 * back. HG_ESTATE while a split push is pending; HG_EINVAL while capturing.
 */
int hg_set_device_parity(hg_ctx *h, int enable, void *stream);

/*
 * The padded-vocab slice, folded into the copy step (PR page, Purpose: the
 * gathered logits keep only the real vocabulary's columns after the gather).
 * From the next served call on, hg_gather, hg_collect and hg_gemm_gather
 * write `out` as [m][vocab]: the first `vocab` columns of each gathered row.
 * The mailbox protocol is unchanged -- every word is pushed, polled and
 * re-armed. vocab = tp*shard (the default) writes whole rows; vocab % 8 == 0
 * keeps 16-byte stores, other widths store element by element. HG_EINVAL
 * unless 1 <= vocab <= tp*shard. Calls already enqueued keep their width,
 * and so do calls captured into a graph, on every replay.
 */
int hg_set_vocab(hg_ctx *h, int vocab);

/* Output columns per row of served calls (see hg_set_vocab), or HG_EINVAL. */
int hg_vocab(const hg_ctx *h);

/* Read-only view of one parity of the mailbox, for inspection by tests:
 * *dev = device address of [cap][tp*shard] BF16, *bytes = its size. The
 * mailbox layout is the API page's (HeadGather.__init__ source: 2 parities
 * x cap rows x shard/2*tp words); the pages expose no such view -- it exists
 * so that tests can check that every served call leaves both parities
 * all-sentinel. */
int hg_mailbox(const hg_ctx *h, int parity, const void **dev, size_t *bytes);

/* Enqueue a copy of one parity of the mailbox ([cap][tp*shard] BF16) into the
 * caller's device buffer `dst` (same size, must not overlap the mailbox).
 * An inspection aid like hg_mailbox; not on the pages. */
int hg_copy_mailbox(const hg_ctx *h, int parity, void *dst, void *stream);

/*
 * Bound every poll: a lane that re-reads a sentinel word more than `spins`
 * times gives up, counts a timeout in the context's status block and
 * continues (its output then holds sentinel words). 0 restores the default
 * (2^24 re-reads). Takes effect for calls enqueued afterwards. Not on the
 * pages, whose poll waits without bound (API page, module description); the
 * bound keeps a missing push from hanging the device.
 */
int hg_set_poll_limit(hg_ctx *h, unsigned long long spins);

/* Wait for `stream`, then report and clear the poll-timeout count:
 * HG_OK if no poll gave up since the last check, HG_ETIMEOUT otherwise.
 * HG_EINVAL if the stream is capturing. The reporting side of the bounded
 * poll (hg_set_poll_limit); not on the pages. */
int hg_poll_status(hg_ctx *h, void *stream);

/*
 * The fused gather without allocation, for callers that cannot call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation. It computes what hg_gather computes for a context of
 * (tp, shard, cap >= m) with device-side parity, and writes `out`
 * ([m][tp*shard] BF16, whole rows) exactly as hg_gather does; it needs no
 * context. Its mailbox (two parities of HG_STATIC_PARITY_BYTES each), parity
 * slots and poll-timeout counter live in a static device array of the
 * library, one per device, resolved on the first call on each device (which
 * arms the mailbox on `stream`) and kept until the process ends. No call
 * allocates device or host memory.
 *
 * Limits: m * tp * shard * 2 <= HG_STATIC_PARITY_BYTES (a larger call returns
 * HG_ESIZE and enqueues nothing); tp in [2, HG_MAX_TP], shard >= 8 and
 * shard % 8 == 0 (else HG_EINVAL); m == 0 is declined (HG_EDECLINE), m < 0 is
 * HG_EINVAL; shards and out 16-byte aligned, out overlapping no shard. The
 * first call on a device must not be made under graph capture (HG_ESTATE);
 * later calls may be captured, and replays alternate the parity.
 *
 * Every call on one device shares that device's scratch array, which keeps
 * the previous call's state (the parity, an all-sentinel mailbox): issue all
 * calls on a device from one host thread and on one stream; calls that
 * overlap on one device (two streams, two threads) race. A poll that gives up
 * after 2^24 re-reads is counted in the scratch array and not reported.
 */
#define HG_STATIC_PARITY_BYTES (8u << 20)
int hg_gather_static(int tp, int shard, const void *const *shards, int m, void *out,
                     void *stream);

/* Workgroups the fused kernel of an m-row call may keep resident at once on
 * the context's device (its grid never exceeds this, so every workgroup whose
 * pushes are awaited is running), or a negative code. Not on the pages: the
 * grid sizing of the pages' kernel is not shown (API page, HeadGather.__init__
 * source names only its per-row-count grid table). */
int hg_fused_grid_limit(hg_ctx *h, int m);

/* Static description of a status code. Not on the pages (the pages report
 * a failed build with a logged warning: API page, _install_gather source). */
const char *hg_strerror(int code);

/* The last HIP error seen by this thread inside the library ("" if none).
 * Not on the pages. */
const char *hg_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* HG_H */
