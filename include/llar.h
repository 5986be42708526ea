/*
 * llar.h -- barrier-free small-message AllReduce protocols on one MI355X.
 *
 * The library reduces N tensor-parallel partial outputs into one output,
 * out[i] = sum_r partials[r][i], with the protocols described in "Every
 * Microsecond Matters: Achieving Near Speed-of-Light Latency in GPU
 * Collectives" (agihunt.info summary of arXiv 2607.16100):
 *
 *   LL        -- paragraph "LL (Low-Latency)": an 8-byte flag and 8 bytes of
 *                data leave in one 16-byte store; seeing the flag means the
 *                data is there (no separate signal, 2x staging).
 *   SENTINEL  -- paragraph "Sentinel": the receive buffer is prefilled with a
 *                value data never takes (a negative NaN); the receiver polls
 *                for the value to change and resets the buffer after use.
 *   LL128     -- paragraph "Two-shot LL128 atomic AllReduce": reduce-scatter
 *                by atomic adds into 128-byte lines whose first slot counts
 *                contributions up to N, then all-gather; about D/N staging.
 *   *_PIPELINED -- paragraph "bidirectional communication + double
 *                buffering": the message moves in chunks through two
 *                alternating staging buffers; receiving a chunk from a peer
 *                is the permission to send the next one, so no barrier sits
 *                between iterations.
 *
 * The N ranks are emulated inside one GPU: each rank is a set of workgroups
 * that reads its own partial buffer; ranks exchange data only through the
 * library's staging memory with device-coherent stores, loads and atomics,
 * and every wait is a bounded poll on a flag or a value -- no grid-wide
 * barrier.  The produced value is the AllReduce result seen by one rank.
 *
 * Conventions for every call:
 *   - All functions are plain C, never throw, and return an llar status
 *     (LLAR_OK == 0, negative on error) unless stated otherwise.
 *   - Device pointers are HIP device allocations on the device that was
 *     current when the communicator was created.
 *   - Streams are hipStream_t passed as void* (0 = the null stream).
 *   - A communicator serves one host thread at a time (a call advances its
 *     epoch and reads its options and cached launch limits); different
 *     communicators may be used from different threads at once.
 *   - Workgroups of one call wait on each other, so a call needs all of its
 *     workgroups resident at once: the library checks that its grid fits the
 *     device's occupancy, but kernels from other streams that fill the GPU
 *     at the same time can keep some of them out.  The waits are bounded
 *     ("spin_timeout_us"), so such a call ends with LLAR_ERR_TIMEOUT in the
 *     status word instead of hanging.
 */
#ifndef LLAR_H
#define LLAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct llar_comm llar_comm; /* opaque; owned by the library */

typedef enum {
  LLAR_FP32 = 0, /* IEEE binary32 */
  LLAR_FP16 = 1, /* IEEE binary16 */
  LLAR_BF16 = 2  /* bfloat16 */
} llar_dtype;   /* the pages' "two-shot LL128" paragraph limits the method to these three */

typedef enum {
  LLAR_AUTO = 0,                /* pick per (N, dtype, size) from the tuned table */
  LLAR_LL = 1,                  /* one-shot LL */
  LLAR_SENTINEL = 2,            /* one-shot Sentinel */
  LLAR_LL128 = 3,               /* two-shot LL128 atomic, one round */
  LLAR_LL128_PIPELINED = 4,     /* two-shot LL128 atomic, chunked, double-buffered, implicit credits */
  LLAR_SENTINEL_PIPELINED = 5   /* two-shot Sentinel, chunked, double-buffered, implicit credits */
} llar_protocol;

enum {
  LLAR_OK = 0,
  LLAR_ERR_ARG = -1,          /* bad argument; nothing was launched */
  LLAR_ERR_UNSUPPORTED = -2,  /* valid but not supported (dtype, N, size) */
  LLAR_ERR_NOMEM = -3,        /* device allocation failed */
  LLAR_ERR_HIP = -4,          /* a HIP runtime call failed */
  LLAR_ERR_TIMEOUT = -5,      /* a device-side poll exceeded its time limit */
  LLAR_ERR_DEVICE = -6        /* another device-side protocol error (see the status bits) */
};

/* Create a communicator for n_ranks emulated ranks (1..8) reducing values of
 * `dtype`, with messages up to max_bytes per rank.  Allocates and initialises
 * all staging (two parities per protocol), the device-resident epoch and the
 * status word on the current device, then synchronises.  Returns NULL on
 * failure; llar_last_error() then tells why. */
llar_comm* llar_create(int n_ranks, llar_dtype dtype, size_t max_bytes);

/* out[i] = partials[0][i] + ... + partials[n_ranks-1][i] for i < n_elems.
 *
 * partials: host array of n_ranks device pointers (read during the call only).
 * out:      device pointer to n_elems elements; it may alias one partial.
 * All device pointers must be 16-byte aligned.  dtype must equal the
 * create-time dtype and n_elems * sizeof(dtype) <= max_bytes.  n_elems == 0
 * is a no-op.  The call only enqueues work on `stream` and returns; the
 * caller keeps the buffers alive until the stream reaches that point.
 *
 * Rounding: LL and SENTINEL (one-shot and pipelined) add in binary64 in rank
 * order and round once to dtype (round-to-nearest-even) -- deterministic.
 * LL128 adds with float atomics in an unspecified order (binary32 staging by
 * default) -- non-deterministic, within the staging type's rounding error.
 *
 * Errors: argument errors return at once with nothing enqueued.  Device-side
 * errors (a poll timeout) are latched in the communicator's status word;
 * `out` is then undefined.  One stream at a time per communicator. */
int llar_allreduce(llar_comm* h, const void* const* partials, void* out, size_t n_elems,
                   llar_dtype dtype, llar_protocol protocol, void* stream);

/* The LL one-shot AllReduce of llar_allreduce (out[i] = partials[0][i] + ...
 * + partials[n_ranks-1][i], binary64 in rank order, one rounding; bit for
 * bit the result of llar_allreduce with LLAR_LL) for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It needs no communicator and calls no
 * allocating routine: staging and control state live in one static device
 * array of 2 MiB per GPU, held by each GPU the library runs on until the
 * process ends.
 *
 * n_ranks:  1..8 (above 8: LLAR_ERR_UNSUPPORTED).
 * partials: host array of n_ranks device pointers; out: device pointer; all
 *           16-byte aligned; out may alias a partial.  dtype: any llar_dtype.
 * n_elems:  at most 64 KiB per rank (n_elems * sizeof(dtype) <= 65536),
 *           else LLAR_ERR_UNSUPPORTED with nothing enqueued; 0 is a no-op.
 * The first call on a device sets that device's array up (synchronous
 *   copies; LLAR_ERR_UNSUPPORTED if that call's stream is being captured --
 *   make one eager call first).  Later calls only enqueue one kernel, and
 *   may be captured into graphs (replays number themselves on the device).
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 *   contents: calls on one GPU must be ordered (one stream, or synchronised);
 *   calls that overlap on one GPU race and their results are undefined.
 * Device-side errors (a poll timeout) latch in the array's status word and
 *   are not reported by this call; the communicator's status calls do not
 *   see them. */
int llar_allreduce_noalloc(int n_ranks, const void* const* partials, void* out, size_t n_elems,
                           llar_dtype dtype, void* stream);

/* Point-to-point copy: recv_buf[i] = send_buf[i] for i < n_elems, moved by
 * one sending rank to one receiving rank through the LL or Sentinel staging
 * of this communicator -- the stage-to-stage activation transfer of pipeline
 * parallelism (the pwwt.cn small-message latency article, section 1.1, the
 * PP item, and section 3.3: a 4096 x FP16 hidden state, 8 KB per token).
 * The same one-shot exchange as llar_allreduce with a single producer, and
 * the receiver writes what arrived instead of a sum.
 *
 * send_buf, recv_buf: device pointers to n_elems elements, 16-byte aligned,
 *   not overlapping.  dtype must equal the create-time dtype and
 *   n_elems * sizeof(dtype) <= max_bytes.  n_elems == 0 is a no-op.
 * protocol: LLAR_LL, LLAR_SENTINEL or LLAR_AUTO (LL up to the
 *   "thr_sentinel" size, else Sentinel); any other value is LLAR_ERR_ARG.
 *   Messages above 8 MiB (LL) or 16 MiB (Sentinel) return
 *   LLAR_ERR_UNSUPPORTED.
 * Result: LL delivers every bit pattern unchanged.  The Sentinel cannot carry
 *   its own all-ones pattern: the sender replaces it by the pattern one below
 *   (still a negative NaN of the same payload class), exactly as the
 *   AllReduce's Sentinel producer does; every other pattern arrives
 *   unchanged.
 * Errors, epochs and stream rules are those of llar_allreduce; the call
 *   shares the communicator's staging and epoch with it. */
int llar_send_recv(llar_comm* h, const void* send_buf, void* recv_buf, size_t n_elems,
                   llar_dtype dtype, llar_protocol protocol, void* stream);

/* ReduceScatter: every rank keeps one segment of the element-wise sum (the
 * yololab.net article on network architecture for LLM inference, the table
 * in its All-Reduce / All-Gather / Reduce-Scatter section; the first half of
 * the two-shot AllReduce in the agihunt.info summary's two-shot LL128
 * paragraph).  For every rank j and i < recv_count:
 *
 *   outs[j][i] = partials[0][j*recv_count + i] + ... + partials[N-1][j*recv_count + i]
 *
 * partials: host array of N device pointers, each N * recv_count elements.
 * outs:     host array of N device pointers, each recv_count elements; outs[j]
 *           may be partials[j] + j*recv_count (in place, when that address is
 *           16-byte aligned like every pointer here) but must not overlap any
 *           other block that is read.
 * One launch in which every rank sends its copy of segment j to rank j over
 * the LL or Sentinel wire and rank j sums what arrived with its own copy, in
 * binary64 in rank order with one rounding (deterministic, the same
 * arithmetic as the LL and Sentinel AllReduce).
 * protocol: LLAR_LL, LLAR_SENTINEL or LLAR_AUTO (LL while N * recv_count *
 *   sizeof(dtype) is within the "thr_sentinel" size), or LLAR_LL128: the
 *   reduce-scatter half of the two-shot LL128 AllReduce -- every rank
 *   atomically adds its copy of segment j into rank j's 128-byte lines
 *   (slot 0 counts contributions up to N) and rank j rounds what the lines
 *   hold, in an unspecified order (non-deterministic; binary32 staging, or
 *   16-bit with the "ll128_acc" option).  Others: LLAR_ERR_ARG.
 * Limits: N * recv_count * sizeof(dtype) <= max_bytes (else LLAR_ERR_ARG),
 *   and <= 8 MiB (LL) or 16 MiB (Sentinel, LL128) (else
 *   LLAR_ERR_UNSUPPORTED).
 *   recv_count need not be a multiple of 16 bytes.  recv_count == 0 is a
 *   no-op.  Pointers 16-byte aligned.  Errors, epochs and stream rules are
 *   those of llar_allreduce, whose staging and epoch this call shares. */
int llar_reduce_scatter(llar_comm* h, const void* const* partials, void* const* outs, size_t recv_count,
                        llar_dtype dtype, llar_protocol protocol, void* stream);

/* AllGather: every receiving rank holds every rank's fragment (same table of
 * the yololab.net article; the second half of the two-shot AllReduce).  For
 * every receiving rank j < n_outs, every rank k and i < send_count:
 *
 *   outs[j][k*send_count + i] = inputs[k][i]
 *
 * inputs: host array of N device pointers, each send_count elements.
 * outs:   host array of n_outs device pointers, each N * send_count elements.
 * n_outs: N (every rank's copy -- the replicated result an AllGather leaves
 *         on all ranks) or 1 (rank 0's copy only); others: LLAR_ERR_ARG.
 * Wire: LL moves every bit pattern unchanged.  The Sentinel wire cannot
 *   carry its all-ones pattern, which arrives as the pattern one below (a
 *   negative NaN still); the receiver applies the same to its own fragment,
 *   so every copy is identical.
 * protocol: LLAR_LL, LLAR_SENTINEL or LLAR_AUTO (no LLAR_LL128: nothing is
 *   summed); limits (N * send_count * sizeof(dtype)), errors and streams as
 *   for llar_reduce_scatter. */
int llar_all_gather(llar_comm* h, const void* const* inputs, void* const* outs, int n_outs, size_t send_count,
                    llar_dtype dtype, llar_protocol protocol, void* stream);

/* Free all resources (synchronises the device first).  NULL is a no-op. */
int llar_destroy(llar_comm* h);

/* Status of the last failing host call on this thread (for NULL returns). */
int llar_last_error(void);

/* Human-readable name of a status code (static string). */
const char* llar_status_string(int status);

/* Sticky device-side status: synchronises the device, returns LLAR_OK,
 * LLAR_ERR_TIMEOUT or LLAR_ERR_DEVICE, and writes the raw status bits to
 * *bits when bits is not NULL.  The status stays set until
 * llar_clear_device_status(). */
int llar_get_device_status(llar_comm* h, uint32_t* bits);
int llar_clear_device_status(llar_comm* h);

/* Options (key, value).  Keys:
 *   "spin_timeout_us"  device poll limit in microseconds (default 200000)
 *   "ll128_acc"        LL128 staging type: 0 = binary32 (default), 1 = the I/O type (16-bit packed)
 *   "chunk_bytes"      largest per-rank chunk of the pipelined protocols (0 = tuned default:
 *                      1 MiB for the Sentinel pipeline and the alternating LL128 one, 256 KiB for
 *                      the wave-split LL128 pipeline; clamped to [1 KiB, 4 MiB]); a
 *                      message is cut into the fewest equal chunks of at most this size (whole
 *                      16-byte vectors for the Sentinel), so that every owner gets an even share
 *                      of every chunk
 *   "slices"           workgroups per rank (0 = tuned default); for the pipelined protocols an
 *                      upper bound: every owner slice of a full chunk keeps at least one line
 *                      (LL128) or vector (Sentinel), because the credit is earned by consuming
 *   "threads"          threads per workgroup: 64, 128, 256 or 512, or 1024 for the slot-handshake
 *                      and owner-credit Sentinel pipelines and the wave-split LL128 pipeline (0 =
 *                      tuned default: 1024 for the latter); the pipelined Sentinel splits a
 *                      workgroup into producer and consumer waves and needs at least 128, and the
 *                      LL128 pipeline alternates in one-wave workgroups
 *   "ll128_kernel"     LL128 pipeline: 0 = wave split (default: producer waves and consumer waves
 *                      each take whole chunks in turn, B buffers, a producer adds chunk c once its
 *                      own workgroup's consumers finished chunk c - B/2); 1 = the alternating
 *                      kernel (every wave produces then consumes each chunk, two buffers)
 *   "ll128_buffers"    wave-split LL128 pipeline: staging buffers B, even, 2..64 (0 = 32); fewer
 *                      when they do not fit the region, and a multiple of the consumer waves'
 *                      count (the consumer of chunk c - B is the consumer of chunk c)
 *   "pipeline_buffers" staging buffers of the pipelined Sentinel: 2 to 64 (default 4), as many as
 *                      fit the staging allocated for the largest chunk (a call that needs more
 *                      returns LLAR_ERR_UNSUPPORTED).  Workgroup credit: an even count, and a
 *                      producer runs up to B/2 - 1 chunks ahead of its consumer; owner credit: any
 *                      count, B - 1 chunks ahead; slot handshake: rounded up to a multiple of its
 *                      wave period
 *   "sentinel_credit"  credit of the pipelined Sentinel: 0 = workgroup credit (default: a producer
 *                      stores chunk c once its own workgroup's consumers finished chunk c - B/2);
 *                      1 = slot handshake (a producer stores into a slot once it reads the owner's
 *                      reset there); 2 = owner credit (every owner's consumer waves publish a
 *                      progress word; a producer stores chunk c once every owner finished c - B)
 *   "consumer_waves"   slot handshake, owner credit and the wave-split LL128 pipeline: consumer
 *                      waves per workgroup (0 = default: a quarter of the waves for the handshake
 *                      and the LL128 pipeline, (waves - 1) / 2 for the owner credit, which keeps
 *                      one wave to read the progress words; at most 8 there)
 *   "placement"        0 = auto, 1 = spread (rank r on XCD r mod 8), 2 = local (one slice's ranks share an XCD);
 *                      auto: local for the LL and Sentinel AllReduce and send/recv, spread for LL128, and
 *                      for ReduceScatter / AllGather local from 8 slices per rank up, spread below
 *   "timing"           1 = record device-side start/end wall-clock per call (see llar_get_timing);
 *                      a call whose grid exceeds 4096 workgroups then fails with LLAR_ERR_UNSUPPORTED
 *   "keep_staging"     1 = LL128/Sentinel consumers do not reset staging (tests only; the next call is invalid)
 *   "debug_drop_rank"  tests: the producers of this rank write nothing, so consumers time out (-1 = none)
 *   "trace"            1 = one-shot kernels record per-workgroup phase stamps (see llar_get_trace),
 *                      the pipelined Sentinel per-chunk stamps (see llar_get_pipeline_trace)
 *   "barrier_ablation" 1 = LL and Sentinel AllReduce calls run the same one-shot exchange behind a
 *                      grid-wide memory barrier instead of per-line flags (raw stores, barrier, then
 *                      reads): the synchronisation the pages say earlier implementations pay at every
 *                      step, kept for measurement; same results, up to 8 MiB per rank
 *   "device_epoch"     1 = always read the device-resident epoch; otherwise the host numbers
 *                      stream-ordered calls and the device epoch is used only on a stream that is
 *                      being captured into a graph (replays then never reuse an epoch)
 *                      Epochs (the LL flag, the agihunt.info summary's LL paragraph) run 1 .. 2^31-1
 *                      for host-numbered calls and 2^31 + (1 .. 2^31-1) for device-numbered ones,
 *                      then wrap.  The state that holds epoch values (LL staging, owner-credit
 *                      progress words, per-workgroup epoch words) is cleared at the wrap, so no
 *                      line written a whole cycle earlier can pass for a new one: by fills
 *                      enqueued on the stream of the first host-numbered call after a host wrap,
 *                      and by the wrapping device-numbered call itself on the device (its last
 *                      workgroup waits for the others, clears, then advances the epoch)
 *   "debug_host_epoch", "debug_device_epoch"
 *                      tests: the epoch of the next host-numbered call (1 .. 2^31-1), or the
 *                      device-resident epoch (2^31+1 .. 2^32-1; the per-workgroup epoch words are
 *                      zeroed, staging is left as it is); llar_get_option reads them back
 *   "auto_threshold_sentinel", "auto_threshold_ll128", "auto_threshold_pipelined"
 *                      AUTO size boundaries in bytes per rank: LL up to 64 KiB, one-shot Sentinel
 *                      up to 1.5 MiB, pipelined Sentinel above; LL128 only above its own threshold
 *                      (default: never, its atomics are slower than the Sentinel exchange here)
 *   "auto_protocol"    0 = AUTO follows the thresholds above; 1..5 = AllReduce calls that pass
 *                      LLAR_AUTO run this protocol (send/recv, ReduceScatter and AllGather keep
 *                      their own AUTO rule)
 *   "consumer_groups"  pipelined Sentinel, workgroup credit: deal the chunks to G groups of the
 *                      consumer waves (group g takes chunks g, g + G, ...), so that up to G chunks
 *                      are consumed at once; G must divide the consumer waves (half of the
 *                      workgroup's) and "pipeline_buffers", else LLAR_ERR_ARG.  0 = two groups
 *                      where the consumer waves split evenly, else one
 *   "producer_groups"  the same for the producer waves (group p stores chunks p, p + PG, ...); PG
 *                      must divide the producer waves (half of the workgroup's).  0 = 1
 *   "consumer_split"   one-shot LL / Sentinel under the local placement: rank 0's part of each slice
 *                      on 1 or 2 consumer workgroups (contiguous halves of the slice's units, each
 *                      issuing half the polls); 0 = two from four ranks on, one below
 *   "local_xcds"       one-shot LL / Sentinel (and send/recv) under the local placement: keep the
 *                      slices on XCDs 0 .. k-1 (slice w on XCD w mod k, the workgroups that land on
 *                      the other XCDs idle); 0 = all eight.  XCDs start a launch at different times
 *                      (measured: XCDs 0-2 within 0.16 us, XCD 3 about 0.3 us later, XCDs 4-7 about
 *                      1 us later), so a small exchange can avoid the late ones.  All workgroups
 *                      of a call must be resident at once, so without a "slices" setting the slice
 *                      count shrinks to what k XCDs hold; an explicit one beyond that is
 *                      LLAR_ERR_UNSUPPORTED
 *   "log"              1 = print every call's operation, protocol and launch geometry (kernel,
 *                      grid, threads, chunks, placement, epoch source) on stderr
 * llar_get_option also answers "local_placement_ok" (read-only): 1 when
 * workgroup ids equal mod 8 were seen to share an XCD, which the local
 * placement requires.
 *
 * h == NULL reads or sets the process-wide defaults that every communicator
 * created afterwards starts from (the keys above, same ranges).  They start
 * from the environment, read once (the pwwt.cn small-message latency
 * article closes with NCCL's buffer-size variable as the model of such
 * knobs):
 *   LLAR_SPIN_TIMEOUT_US     "spin_timeout_us"
 *   LLAR_PROTOCOL            "auto_protocol": auto, ll, sentinel, ll128, ll128_pipelined,
 *                            sentinel_pipelined
 *   LLAR_ACCUM               "ll128_acc": fp32 or 16
 *   LLAR_TUNE                path of a file of "key value" (or key=value) lines, any key
 *                            above, '#' comments -- e.g. AUTO thresholds tuned on a machine
 *   LLAR_LOG                 "log"
 *   LLAR_DEBUG_KEEP_STAGING  "keep_staging"
 * A value that does not parse or is out of range is reported on stderr and
 * ignored.
 * Returns LLAR_ERR_ARG for an unknown key or a bad value. */
int llar_set_option(llar_comm* h, const char* key, long long value);
int llar_get_option(llar_comm* h, const char* key, long long* value);

/* Protocol AUTO would run for a message of `bytes` per rank. */
int llar_select_protocol(llar_comm* h, size_t bytes);

/* Copy `bytes` of the staging region of `protocol` to host memory, both
 * parities, in the kernels' layout: LL [parity][sender 1..N-1][vector][two
 * 16-byte lines {d0, epoch, d1, epoch}]; Sentinel [parity][sender][16-byte
 * slot], all-ones when empty; LL128 [parity][128-byte line], slot 0 the
 * count; pipelined Sentinel [buffer][owner][sender][16-byte slot].
 * Synchronises first.  For tests of flags and packing. */
int llar_debug_copy_staging(llar_comm* h, llar_protocol protocol, void* host_dst, size_t bytes);
/* Size in bytes of that staging region (0 if none). */
size_t llar_staging_bytes(llar_comm* h, llar_protocol protocol);

/* Epoch the next call will use (host-numbered, or the device-resident one
 * when the last call read it); synchronises first. */
int llar_get_epoch(llar_comm* h, uint32_t* epoch);

/* Device-side timing of the last `count` timed calls (option "timing"):
 * for each call, the wall-clock ticks (see llar_wallclock_hz) of the first
 * workgroup start and of the last workgroup end (after its final stores were
 * acknowledged).  Writes 2*count uint64 to host_dst, oldest first; returns the
 * number of records written (>= 0) or an error.  Each workgroup stores its
 * own span; this call reduces them (a call that recorded nothing reads as
 * start 2^64-1, end 0). */
int llar_get_timing(llar_comm* h, uint64_t* host_dst, int count);
double llar_wallclock_hz(void);

/* Phase stamps of the last one-shot call made with option "trace": for each
 * workgroup 8 uint64 -- wall ticks at entry, epoch known, first input loaded,
 * first store acknowledged (producer) or all slots ready (consumer), output
 * acknowledged (consumer), exit; then xcc | rank << 8 | slice << 16; spare.
 * Returns the number of workgroup records written (<= max_records). */
int llar_get_trace(llar_comm* h, uint64_t* host_dst, int max_records);

/* Per-chunk stamps of the last pipelined-Sentinel call made with option
 * "trace": for each workgroup 512 uint64 -- wall ticks at which producer wave
 * 0 was granted the credit for chunk c ([c]), issued chunk c's last stores
 * ([128 + c]), consumer wave 0 saw chunk c's slots ready ([256 + c]) and
 * finished chunk c ([384 + c]), for c < 128 (0 = no record).  Returns the
 * number of workgroup records written. */
int llar_get_pipeline_trace(llar_comm* h, uint64_t* host_dst, int max_records);

/* Workgroup geometry the library would launch for this call (for tests and
 * tuning): writes grid size, threads per workgroup, slices and chunks. */
int llar_launch_geometry(llar_comm* h, size_t n_elems, llar_protocol protocol,
                         int* grid, int* threads, int* slices, int* chunks);

/* ---- speed-of-light floor microbenchmarks (same device) ---------------- *
 * "Every Microsecond Matters" (agihunt.info summary), paragraph on the
 * speed-of-light bound: one AllReduce cannot beat two L2 round trips plus one
 * remote write.  On one GPU the analogues are measured here:
 *   kind 0: L2 round trip -- dependent chain of device-coherent 4-byte loads
 *           over a 64-line ring, ns per hop (param: XCD-distance unused)
 *   kind 1: store-to-visibility -- half the round trip of a 16-byte coherent
 *           store / poll ping-pong between workgroups on XCDs a and b,
 *           ns (param = b, a = 0; b = 8 means a second workgroup on XCD 0)
 *   kind 2: empty-kernel launch interval, ns per launch (host timed)
 *   kind 3: device-coherent returning-atomic latency, ns
 *   kind 4: streaming copy bandwidth, GB/s of read+write (param = MiB)
 *   kind 5: L2 round trip to lines another XCD has just written -- a
 *           dependent chain of device-coherent loads over 4096 lines that
 *           workgroup `param` (1..63, on XCD param % 8) wrote, read once
 *           each from XCD 0, ns per hop (param % 8 == 0: the same XCD)
 *   kind 6: empty-kernel launch interval under graph replay (a graph of
 *           param launches, default 100), ns per launch
 *   kind 7: no-return device-scope float atomic throughput with the LL128
 *           lane pattern (each wave instruction adds into two whole 128-byte
 *           lines), G lane operations per second; param bits 0-1: 0 =
 *           binary32, 1 = packed bfloat16 pair, 2 = packed binary16 pair;
 *           bit 2: issued from one XCD only (else all 8); bits 3-4: 1 =
 *           every workgroup adds into one shared 8 KiB window, 2 = each
 *           group of eight consecutive workgroups (one per XCD) shares one
 *           window -- the eight ranks of an LL128 line --, 0 = private windows
 * Results go to *value.  Synchronous. */
int llar_floor_measure(int kind, int param, double* value);

#ifdef __cplusplus
}
#endif
#endif /* LLAR_H */
