// llar_host.hip -- host side of the C ABI declared in include/llar.h:
// communicator lifetime, staging layout, protocol choice, launch geometry,
// options, status and debug exports.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>

#include "llar.h"
#include "llar_device.h"
#include "llar_internal.h"

using namespace llar;

namespace {

thread_local int g_last_error = LLAR_OK;

int fail(int status) {
  g_last_error = status;
  return status;
}

// Per-protocol size caps (bytes per rank) of the single-round protocols; the
// pipelined protocols have no cap (their staging is chunk-sized).
constexpr size_t kCapLL = 8ull << 20;
constexpr size_t kCapSentinel = 16ull << 20;
constexpr size_t kCapLL128 = 16ull << 20;
constexpr size_t kCapChunk = 4ull << 20;  // largest chunk of the pipelined protocols
// default chunk of the wave-split LL128 pipeline; measured on MI355X (1024
// threads, 4 consumer waves, 32 buffers): 16 MiB x 8 fp32 237 us at 256 KiB
// against 258 / 357 us at 128 / 64 KiB; 64 MiB x 8 bf16 1521 us against
// 1680 / 1901 us
constexpr size_t kLL128PipeChunk = 256ull << 10;
constexpr int kTraceMaxWgs = 4096;
constexpr int kSmallSpan = 3;  // XCDs of a one-shot call of 5 to 8 default slices
constexpr int kPipeTraceMaxWgs = 1024;
// The pipelined Sentinel's region holds 8 staging buffers of the largest
// chunk (a call spaces its buffers by its own chunk, so more of a smaller
// chunk fit, up to 64).  With B buffers a producer runs B/2 - 1 chunks ahead
// of its consumer under the workgroup credit (safe with B >= 2 lag + 2), B - 1
// under the owner credit.  Default 4.
constexpr uint32_t kSentinelPipeMaxBuffers = 8;

size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

struct Region {
  uint8_t* ptr = nullptr;
  size_t bytes = 0;
  size_t parity_stride = 0;
  size_t rank_stride = 0;
};

}  // namespace

struct llar_comm {
  int device = 0;
  int n_ranks = 0;
  int kind = 0;
  size_t elem = 0;
  size_t max_bytes = 0;
  int cu_count = 0;
  double wall_hz = 100e6;
  Ctrl* ctrl = nullptr;
  Region ll, sent, ll128, ll128_pipe, sent_pipe;
  bool local_ok = false;  // workgroup b runs on XCD b % 8
  uint64_t* timing_wg = nullptr;  // kTimingRing x kTimingMaxWgs x 2 per-workgroup spans of timed calls
  uint64_t* trace = nullptr;  // kTraceMaxWgs x kTraceWords stamps of the last traced one-shot call
  int trace_grid = 0;
  uint64_t* pipe_trace = nullptr;  // kPipeTraceMaxWgs x kPipeTraceWords stamps of the last traced pipeline call
  uint32_t* credit = nullptr;      // kCreditEntries {count, epoch} progress entries of the pipelined Sentinel's owner credit
  int pipe_trace_grid = 0;
  uint32_t host_epoch = 1;         // epoch of the next host-numbered call
  bool host_wrap_pending = false;  // the host epoch wrapped: clear the epoch-tagged state before the next call
  bool last_call_device = false;   // the last call read the device-resident epoch
  // options
  long long spin_timeout_us = 200000;
  long long ll128_acc = 0;
  long long chunk_bytes = 0;
  long long slices = 0;
  long long threads = 0;
  long long placement = 0;
  long long timing = 0;
  long long keep_staging = 0;
  long long debug_drop_rank = -1;
  long long trace_on = 0;
  long long device_epoch = 0;  // 1: always read the device-resident epoch
  long long pipe_buffers = 4;  // staging buffers of the pipelined Sentinel (2..64, even for the workgroup credit; they must fit the region)
  long long sentinel_credit = 0;  // pipelined Sentinel: 0 = workgroup credit, 1 = slot handshake, 2 = owner credit
  long long cons_waves = 0;       // slot handshake: consumer waves per workgroup (0 = a quarter)
  long long cons_groups = 0;      // pipelined Sentinel, workgroup credit: consumer groups (0 = 2 where they divide)
  long long prod_groups = 0;      // pipelined Sentinel, workgroup credit: producer groups (0 = 1)
  long long cons_split = 0;       // one-shot, local placement: consumer workgroups per slice (0 = 2 from N = 4)
  long long barrier_ablation = 0;  // 1: LL/Sentinel AllReduce behind a grid-wide barrier (measurement)
  long long ll128_kernel = 0;      // pipelined LL128: 0 = producer/consumer waves, B buffers; 1 = alternating, 2 parities
  long long auto_proto = 0;        // 0: AUTO follows the threshold table; 1..5: AUTO AllReduce calls run this protocol
  long long log = 0;               // 1: print every call's protocol and launch geometry to stderr
  long long local_xcds = 0;        // one-shot LL/Sentinel, local placement: slices use XCDs 0 .. n-1 (0 = 8)
  long long ll128_buffers = 0;     // pipelined LL128, wave-split kernel: staging buffers (0 = 8, fewer if they do not fit)
  long long thr_sentinel = 64ll << 10;    // AUTO: LL up to (<=) this many bytes
  long long thr_ll128 = 1ll << 62;        // AUTO: one-shot Sentinel up to here (LL128 one round above)
  // AUTO: pipelined Sentinel above this (measured on MI355X, 8 x bf16 per
  // call: one-shot Sentinel 8.1 / 11.4 / 14.3 us at 1 / 1.5 / 2 MiB, the
  // pipeline 9.9 / 12.7 / 13.5)
  long long thr_pipelined = 3ll << 19;
  // resident workgroups per CU by [ranks - 1][kernel][threads 64 .. 1024],
  // 0 = not asked yet: the occupancy query costs more host time than the
  // rest of a call's set-up
  mutable int occ_cache[8][kKernCount][5] = {};
};

namespace {

int elem_bytes_of(int dtype) { return dtype == LLAR_FP32 ? 4 : 2; }

// Consumer workgroups per slice of a one-shot call under the local placement
// (rank 0's work on a slice split into two parts, so that each consumer
// workgroup issues half the polls; measured on MI355X, N = 8 bf16 LL, device
// span: 8 KiB 1.44-1.49 against 1.51-1.59 us, 16 KiB 1.44-1.50 against
// 1.51-1.61, 64 KiB 1.67-1.70 against 1.75-1.78; fp16 Sentinel 128 KiB
// 2.00-2.03 against 2.14-2.16; N = 4 and N = 2 unchanged).  Option
// "consumer_split": 0 = two from four ranks on, 1 = one, 2 = two.
int oneshot_split(const llar_comm* h, int kernel) {
  if (kernel != kKernOneShotLLLocal && kernel != kKernOneShotSentinelLocal) return 1;
  if (h->cons_split == 0) return h->n_ranks >= 4 ? 2 : 1;
  return (int)h->cons_split;
}

// Workgroups of `kernel` at `threads` that one CU holds at once, for this
// communicator's device and dtype (0 on a failed query, which is asked again
// next time).
int occupancy_of(const llar_comm* h, int n_launch, int kernel, int threads) {
  const int ti = threads == 64 ? 0 : threads == 128 ? 1 : threads == 256 ? 2 : threads == 512 ? 3 : threads == 1024 ? 4 : -1;
  if (ti < 0 || kernel < 0 || kernel >= kKernCount || n_launch < 1 || n_launch > 8)
    return occupancy(h->kind, n_launch, kernel, threads);
  int& slot = h->occ_cache[n_launch - 1][kernel][ti];
  if (slot <= 0) slot = occupancy(h->kind, n_launch, kernel, threads);
  return slot;
}

hipError_t alloc_region(Region& r, size_t bytes, int fill) {
  r.bytes = bytes;
  if (bytes == 0) return hipSuccess;
  hipError_t e = hipMalloc(&r.ptr, bytes);
  if (e != hipSuccess) {
    r.ptr = nullptr;
    return e;
  }
  return hipMemset(r.ptr, fill, bytes);
}

void free_region(Region& r) {
  if (r.ptr) (void)hipFree(r.ptr);
  r.ptr = nullptr;
}

hipError_t init_ctrl(llar_comm* h) {
  Ctrl c;
  memset(&c, 0, sizeof(c));
  c.epoch = 0x80000001u;  // first device-numbered epoch
  c.timing_wg = h->timing_wg;
  c.ll_base = h->ll.ptr;
  c.ll_bytes = h->ll.ptr ? h->ll.bytes : 0u;
  c.credit_base = reinterpret_cast<uint8_t*>(h->credit);
  c.credit_bytes = h->credit ? kCreditBytes : 0u;
  return hipMemcpy(h->ctrl, &c, sizeof(c), hipMemcpyHostToDevice);
}

hipError_t reset_staging(llar_comm* h) {
  hipError_t e = hipSuccess;
  if (h->ll.ptr && (e = hipMemset(h->ll.ptr, 0, h->ll.bytes)) != hipSuccess) return e;
  if (h->sent.ptr && (e = hipMemset(h->sent.ptr, 0xFF, h->sent.bytes)) != hipSuccess) return e;
  if (h->ll128.ptr && (e = hipMemset(h->ll128.ptr, 0, h->ll128.bytes)) != hipSuccess) return e;
  if (h->ll128_pipe.ptr && (e = hipMemset(h->ll128_pipe.ptr, 0, h->ll128_pipe.bytes)) != hipSuccess) return e;
  if (h->sent_pipe.ptr && (e = hipMemset(h->sent_pipe.ptr, 0xFF, h->sent_pipe.bytes)) != hipSuccess) return e;
  // progress words carry the epoch of the call that wrote them, and the
  // device-resident epoch restarts with the control block
  if (h->credit && (e = hipMemset(h->credit, 0, kCreditBytes)) != hipSuccess) return e;
  return hipDeviceSynchronize();
}

void destroy_all(llar_comm* h) {
  if (!h) return;
  (void)hipSetDevice(h->device);
  (void)hipDeviceSynchronize();
  free_region(h->ll);
  free_region(h->sent);
  free_region(h->ll128);
  free_region(h->ll128_pipe);
  free_region(h->sent_pipe);
  if (h->ctrl) (void)hipFree(h->ctrl);
  h->ctrl = nullptr;
  if (h->trace) (void)hipFree(h->trace);
  h->trace = nullptr;
  if (h->timing_wg) (void)hipFree(h->timing_wg);
  h->timing_wg = nullptr;
  if (h->pipe_trace) (void)hipFree(h->pipe_trace);
  h->pipe_trace = nullptr;
  if (h->credit) (void)hipFree(h->credit);
  h->credit = nullptr;
  delete h;
}

// Sentinel two-shot slot size: 16-byte vectors per (owner, sender) slot.
uint32_t sentinel_shard_cap(size_t chunk_bytes, int n_ranks) {
  return (uint32_t)(ceil_div(ceil_div(chunk_bytes, 16), (size_t)n_ranks) + 1);
}

size_t effective_chunk(const llar_comm* h, int proto) {
  size_t c = (size_t)h->chunk_bytes;
  // default: 1 MiB for the Sentinel pipeline and the alternating LL128 one
  // (measured on MI355X for the latter, N = 8: 16 MiB fp32 562 -> 213 us,
  // 64 MiB bf16 2985 -> 1620 us against 128 KiB chunks); 256 KiB for the
  // wave-split LL128 pipeline, whose 32 buffers keep many chunks in flight
  if (c == 0) c = (proto == LLAR_LL128_PIPELINED && h->ll128_kernel == 0) ? kLL128PipeChunk : ((size_t)1 << 20);
  c = std::min(c, kCapChunk);
  c = std::min(c, ceil_div(h->max_bytes, 16) * 16);  // never beyond one whole message
  c = std::max(c, (size_t)1024);
  c = (c / 16) * 16;  // whole 16-byte vectors
  return c;
}

struct Geometry {
  int kernel = 0;
  int threads = 64;
  int slices = 1;       // slices that carry work
  int grid_slices = 1;  // slices the grid covers (local placement pads to 8)
  int chunks = 1;
  uint32_t chunk_elems = 0;
  uint32_t placement = kPlaceSpread;
  int xcd_span = 8;  // local one-shot: XCDs its slices use
};

int clampi(long long v, int lo, int hi) { return (int)std::max<long long>(lo, std::min<long long>(hi, v)); }

// Choose kernel and geometry.  Returns LLAR_OK or an error.
int plan(const llar_comm* h, size_t n_elems, int proto, Geometry& g) {
  const size_t nbytes = n_elems * h->elem;
  const int N = h->n_ranks;
  switch (proto) {
    case LLAR_LL:
    case LLAR_SENTINEL: {
      if (nbytes > (proto == LLAR_LL ? kCapLL : kCapSentinel)) return LLAR_ERR_UNSUPPORTED;
      g.kernel = proto == LLAR_LL ? kKernOneShotLL : kKernOneShotSentinel;
      // the consumer works in 8-byte units: 2 per 16-byte vector
      size_t units = 2 * ceil_div(nbytes, 16);
      // measured on MI355X (graph replay, N = 8): 256 threads below 64
      // slices' worth of units, 512 from there (fp16 Sentinel per call:
      // 128 KiB 4.13 -> 4.01 us, 256 KiB 5.49 -> 5.19, 512 KiB 8.13 -> 7.22;
      // 64 KiB keeps 256: 3.70 against 3.96).  Between 4 and 8 slices the
      // exchange keeps to the first three XCDs under the local placement
      // (below, kSmallSpan)
      g.threads = h->threads ? (int)h->threads : (units >= (size_t)256 * 64 ? 512 : 256);
      g.slices = h->slices ? (int)h->slices : clampi((long long)ceil_div(units, (size_t)g.threads), 1, 64);
      break;
    }
    case LLAR_LL128:
    case LLAR_LL128_PIPELINED: {
      const bool acc16 = (h->ll128_acc == 1) && h->kind != kKindF32;
      const size_t K = acc16 ? 63 : 31;
      size_t chunk_elems;
      if (proto == LLAR_LL128) {
        if (nbytes > kCapLL128) return LLAR_ERR_UNSUPPORTED;
        chunk_elems = std::max<size_t>(n_elems, 1);
      } else {
        // Lines are split among the owners by the chunk, so a message (or
        // last chunk) shorter than the chunk would hand its lines to the
        // first owners alone: the message is cut into equal chunks of at
        // most the configured size.
        const size_t n = std::max<size_t>(n_elems, 1);
        const size_t nch = ceil_div(n, effective_chunk(h, proto) / h->elem);
        chunk_elems = ceil_div(n, nch);
      }
      g.kernel = acc16 ? kKernLL128Acc16 : kKernLL128Acc32;
      g.chunk_elems = (uint32_t)chunk_elems;
      g.chunks = (int)ceil_div(n_elems, chunk_elems);
      size_t lines = ceil_div(std::min(chunk_elems, n_elems), K);
      size_t per_owner = ceil_div(lines, (size_t)N);
      // measured on MI355X, with a producer's owners spread over its waves:
      // one round takes one workgroup per line of an owner's shard, up to 64
      // per rank, of 512 threads once a slice holds 32 lines of every owner
      // and 256 below (16 KiB x 8 bf16: 6.9 against 8.3 us; 2 MiB x 8: 47.9
      // against 54.0); the pipeline takes 512 threads and at most 32 slices
      // (4 MiB x 8 fp32 in 64 KiB chunks: 249 us against 284 at 64 slices)
      const bool piped = (proto == LLAR_LL128_PIPELINED);
      g.slices = h->slices ? (int)h->slices : clampi((long long)per_owner, 1, piped ? 32 : 64);
      const size_t per_slice = ceil_div(per_owner, (size_t)g.slices);
      g.threads = h->threads ? (int)h->threads : ((piped || per_slice >= 32) ? 512 : 256);
      // the pipeline splits a workgroup into producer and consumer waves
      // (two waves at least; a one-wave workgroup alternates).  Measured on
      // MI355X, 4 MiB x 8 fp32 in 64 KiB chunks: 249 us alternating; split
      // 512 threads / 4 consumer waves / 8 buffers 185 us; 1024 / 8 / 16
      // 110 us; 1024 / 4 / 32 74 us (1024 / 2 / 32 81, 1024 / 8 / 32 95)
      if (piped && h->ll128_kernel == 0 && (h->threads == 0 || h->threads >= 128)) {
        g.kernel = acc16 ? kKernLL128WsAcc16 : kKernLL128WsAcc32;
        if (!h->threads) g.threads = 1024;
      }
      if (g.chunks > 1) {
        // the implicit credit reaches a workgroup only through lines of its
        // own: every owner slice of a full chunk must hold at least one line
        size_t min_owner = ceil_div(chunk_elems, K) / (size_t)N;
        if (min_owner == 0) return LLAR_ERR_UNSUPPORTED;
        g.slices = (int)std::min<size_t>((size_t)g.slices, min_owner);
      }
      break;
    }
    case LLAR_SENTINEL_PIPELINED: {
      g.kernel = h->sentinel_credit == 1 ? kKernSentinelHs : h->sentinel_credit == 2 ? kKernSentinelOc : kKernSentinelPipe;
      // Owner shards split the chunk, so the part of a chunk that lies past
      // the message end would be missing from the last owners' shards, and
      // a message shorter than the chunk would go to the first owners'
      // consumers alone.  The message is therefore cut into equal chunks
      // (whole 16-byte vectors) of at most the configured size.
      const size_t nch = std::max<size_t>(ceil_div(nbytes, effective_chunk(h, proto)), 1);
      const size_t cb = std::max<size_t>(ceil_div(ceil_div(nbytes, nch), 16), 1) * 16;
      g.chunk_elems = (uint32_t)(cb / h->elem);
      g.chunks = (int)ceil_div(n_elems, (size_t)g.chunk_elems);
      size_t vecs = ceil_div(std::min(cb, nbytes), 16);
      size_t per_owner = ceil_div(vecs, (size_t)N);
      // half the waves produce, half consume: one owner-slice vector per
      // consumer lane per chunk
      g.threads = h->threads ? (int)h->threads : (h->sentinel_credit != 0 ? 1024 : 512);
      if (g.threads < 128) return LLAR_ERR_ARG;
      // measured on MI355X (64 MiB x 8 bf16): 1 MiB chunks, 512 threads and
      // 32 slices per rank (one workgroup per CU) stream best
      g.slices = h->slices ? (int)h->slices : clampi((long long)ceil_div(per_owner, (size_t)g.threads / 2), 1, 32);
      // owner credit: one 64-vector batch per slice of an owner's shard
      if (g.kernel == kKernSentinelOc && !h->slices) g.slices = clampi((long long)ceil_div(per_owner, 64), 1, 32);
      if (g.chunks > 1) {
        // the credit is earned by consuming: every owner slice of a full
        // chunk must hold at least one vector
        size_t min_owner = (cb / 16) / (size_t)N;
        if (min_owner == 0) return LLAR_ERR_UNSUPPORTED;
        g.slices = (int)std::min<size_t>((size_t)g.slices, min_owner);
      }
      break;
    }
    default:
      return LLAR_ERR_ARG;
  }
  // placement: local (the ranks of a slice share one XCD's L2) for the
  // Sentinel and LL exchanges, spread (rank r on XCD r) for the atomic one
  uint32_t place = kPlaceSpread;
  if (h->placement == 2) place = kPlaceLocal;
  else if (h->placement == 0 && proto != LLAR_LL128 && proto != LLAR_LL128_PIPELINED) place = kPlaceLocal;
  if (place == kPlaceLocal && !h->local_ok) place = kPlaceSpread;
  g.grid_slices = g.slices;
  if (place == kPlaceLocal) {
    // one-shot LL / Sentinel may keep their slices on the first few XCDs
    const bool oneshot = proto == LLAR_LL || proto == LLAR_SENTINEL;
    g.xcd_span = (oneshot && h->local_xcds > 0) ? (int)h->local_xcds : 8;
    // The XCDs start a launch at different times (XCDs 0-2 first, XCD 3
    // about 0.3 us and XCDs 4-7 about 1 us later) and the call waits for its
    // slowest slice.  So a one-shot call of 5 to 8 default 256-thread slices
    // keeps them on XCDs 0-2, two or three per XCD.  Measured on MI355X,
    // 16 KiB x 8 bf16 LL against four 512-thread slices on XCDs 0-3 (five
    // boxes, medians of 60 calls): device span 1.46-1.58 against
    // 1.64-1.81 us; graph replay 2.96-3.51 against 3.25-3.65 us per call.
    // From 32 KiB on, eight XCDs are faster again.
    if (oneshot && h->local_xcds == 0 && !h->threads && !h->slices && g.slices > 4 && g.slices <= 8)
      g.xcd_span = kSmallSpan;
    g.grid_slices = (int)ceil_div((size_t)g.slices, (size_t)g.xcd_span) * 8;
    if (g.kernel == kKernSentinelPipe) g.kernel = kKernSentinelPipeLocal;
    if (g.kernel == kKernSentinelHs) g.kernel = kKernSentinelHsLocal;
    if (g.kernel == kKernSentinelOc) g.kernel = kKernSentinelOcLocal;
    if (g.kernel == kKernOneShotLL) g.kernel = kKernOneShotLLLocal;
    if (g.kernel == kKernOneShotSentinel) g.kernel = kKernOneShotSentinelLocal;
  }
  g.placement = place;
  if (g.threads != 64 && g.threads != 128 && g.threads != 256 && g.threads != 512 && g.threads != 1024)
    return LLAR_ERR_ARG;
  if (g.threads == 1024 && g.kernel != kKernSentinelHs && g.kernel != kKernSentinelHsLocal &&
      g.kernel != kKernSentinelOc && g.kernel != kKernSentinelOcLocal && g.kernel != kKernLL128WsAcc32 &&
      g.kernel != kKernLL128WsAcc16)
    return LLAR_ERR_ARG;
  // a one-shot call kept on the first k XCDs needs all of its workgroups
  // resident there at once: by default its slices shrink to what those
  // XCDs' CUs hold (slice w runs on XCD w mod k with its N ranks, and the
  // second consumer workgroup of a split consumer)
  if (g.placement == kPlaceLocal && g.xcd_span < 8 && !h->slices) {
    const int occ = occupancy_of(h, N, g.kernel, g.threads);
    if (occ <= 0) return LLAR_ERR_HIP;
    const int per_slice = N + oneshot_split(h, g.kernel) - 1;
    const long long fit = (long long)g.xcd_span * ((long long)occ * (h->cu_count / 8) / per_slice);
    g.slices = clampi(std::min<long long>(g.slices, fit), 1, g.slices);
    g.grid_slices = (int)ceil_div((size_t)g.slices, (size_t)g.xcd_span) * 8;
  }
  return LLAR_OK;
}

int auto_protocol(const llar_comm* h, size_t nbytes) {
  if (h->auto_proto > 0) return (int)h->auto_proto;  // forced (option auto_protocol, LLAR_PROTOCOL)
  if ((long long)nbytes <= h->thr_sentinel && nbytes <= kCapLL) return LLAR_LL;
  if ((long long)nbytes > h->thr_pipelined) return LLAR_SENTINEL_PIPELINED;
  if ((long long)nbytes > h->thr_ll128 && nbytes <= kCapLL128) return LLAR_LL128;
  if (nbytes <= kCapSentinel) return LLAR_SENTINEL;
  return LLAR_SENTINEL_PIPELINED;
}

const Region* region_of(const llar_comm* h, int proto) {
  switch (proto) {
    case LLAR_LL: return &h->ll;
    case LLAR_SENTINEL: return &h->sent;
    case LLAR_LL128: return &h->ll128;
    case LLAR_LL128_PIPELINED: return &h->ll128_pipe;
    case LLAR_SENTINEL_PIPELINED: return &h->sent_pipe;
    default: return nullptr;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---- options ------------------------------------------------------------
struct OptionEntry {
  const char* name;
  long long llar_comm::*field;
};
const OptionEntry kOptions[] = {
    {"spin_timeout_us", &llar_comm::spin_timeout_us},
    {"ll128_acc", &llar_comm::ll128_acc},
    {"chunk_bytes", &llar_comm::chunk_bytes},
    {"slices", &llar_comm::slices},
    {"threads", &llar_comm::threads},
    {"placement", &llar_comm::placement},
    {"timing", &llar_comm::timing},
    {"keep_staging", &llar_comm::keep_staging},
    {"debug_drop_rank", &llar_comm::debug_drop_rank},
    {"trace", &llar_comm::trace_on},
    {"device_epoch", &llar_comm::device_epoch},
    {"pipeline_buffers", &llar_comm::pipe_buffers},
    {"sentinel_credit", &llar_comm::sentinel_credit},
    {"consumer_waves", &llar_comm::cons_waves},
    {"barrier_ablation", &llar_comm::barrier_ablation},
    {"ll128_kernel", &llar_comm::ll128_kernel},
    {"ll128_buffers", &llar_comm::ll128_buffers},
    {"auto_protocol", &llar_comm::auto_proto},
    {"log", &llar_comm::log},
    {"local_xcds", &llar_comm::local_xcds},
    {"consumer_groups", &llar_comm::cons_groups},
    {"producer_groups", &llar_comm::prod_groups},
    {"consumer_split", &llar_comm::cons_split},
    {"auto_threshold_sentinel", &llar_comm::thr_sentinel},
    {"auto_threshold_ll128", &llar_comm::thr_ll128},
    {"auto_threshold_pipelined", &llar_comm::thr_pipelined},
};

long long* option_slot(llar_comm* h, const char* key) {
  for (const auto& t : kOptions)
    if (strcmp(t.name, key) == 0) return &(h->*(t.field));
  return nullptr;
}

// Range checks of an option value that need no device (n_ranks: the
// communicator's rank count, or 0 for the process defaults).
bool option_value_ok(const char* key, long long value, int n_ranks) {
  auto is = [&](const char* k) { return strcmp(key, k) == 0; };
  if (is("spin_timeout_us")) return value >= 1;
  if (is("ll128_acc") || is("ll128_kernel")) return value == 0 || value == 1;
  if (is("chunk_bytes")) return value >= 0 && (size_t)value <= kCapChunk;
  if (is("slices")) return value >= 0 && value <= 1024;
  if (is("threads")) return value == 0 || value == 64 || value == 128 || value == 256 || value == 512 || value == 1024;
  if (is("placement")) return value >= 0 && value <= 2;
  if (is("pipeline_buffers")) return value >= 2 && value <= 64;
  if (is("sentinel_credit")) return value >= 0 && value <= 2;
  if (is("consumer_waves")) return value >= 0 && value <= 15;
  if (is("ll128_buffers")) return value == 0 || (value >= 2 && value <= 64 && value % 2 == 0);
  if (is("auto_protocol")) return value >= 0 && value <= LLAR_SENTINEL_PIPELINED;
  if (is("local_xcds")) return value >= 0 && value <= 8;
  if (is("consumer_groups") || is("producer_groups")) return value >= 0 && value <= 8;
  if (is("consumer_split")) return value >= 0 && value <= 2;
  if (is("timing") || is("keep_staging") || is("trace") || is("device_epoch") || is("barrier_ablation") || is("log"))
    return value == 0 || value == 1;
  if (is("debug_drop_rank")) return value >= -1 && (n_ranks == 0 || value < n_ranks);
  if (is("auto_threshold_sentinel") || is("auto_threshold_ll128") || is("auto_threshold_pipelined")) return value >= 0;
  return true;
}

// Process-wide defaults that every communicator starts from: the option
// table's values, then the environment, read once:
//   LLAR_SPIN_TIMEOUT_US  device poll limit (us)
//   LLAR_PROTOCOL         protocol of AllReduce calls that pass LLAR_AUTO:
//                         auto, ll, sentinel, ll128, ll128_pipelined or
//                         sentinel_pipelined
//   LLAR_ACCUM            LL128 staging: fp32 (binary32) or 16 (packed 16-bit)
//   LLAR_TUNE             path of a file of option settings, one "key value"
//                         or "key=value" a line ('#' starts a comment) --
//                         e.g. the AUTO thresholds measured on a machine
//   LLAR_LOG              1: print each call's protocol and launch geometry
//   LLAR_DEBUG_KEEP_STAGING  1: consumers leave staging as it is (tests)
// A value that does not parse or is out of range is reported on stderr and
// ignored.  llar_set_option / llar_get_option with a NULL handle change and
// read these defaults.
std::mutex g_defaults_mu;

void env_warn(const char* var, const char* value, const char* why) {
  fprintf(stderr, "llar: ignoring %s=%s (%s)\n", var, value, why);
}

bool parse_ll(const char* s, long long& v) {
  if (!s || !*s) return false;
  char* end = nullptr;
  v = strtoll(s, &end, 0);
  while (end && (*end == ' ' || *end == '\t' || *end == '\r' || *end == '\n')) ++end;
  return end && *end == '\0';
}

void set_default(llar_comm& d, const char* var, const char* key, const char* text, long long value) {
  long long* slot = option_slot(&d, key);
  if (!slot) return env_warn(var, text, "unknown option");
  if (!option_value_ok(key, value, 0)) return env_warn(var, text, "value out of range");
  *slot = value;
}

void load_env_defaults(llar_comm& d) {
  if (const char* e = getenv("LLAR_SPIN_TIMEOUT_US")) {
    long long v = 0;
    if (parse_ll(e, v)) set_default(d, "LLAR_SPIN_TIMEOUT_US", "spin_timeout_us", e, v);
    else env_warn("LLAR_SPIN_TIMEOUT_US", e, "not a number");
  }
  if (const char* e = getenv("LLAR_PROTOCOL")) {
    static const char* const names[] = {"auto", "ll", "sentinel", "ll128", "ll128_pipelined", "sentinel_pipelined"};
    long long v = -1;
    for (int i = 0; i < 6; ++i)
      if (strcmp(e, names[i]) == 0) v = i;
    if (v < 0 && !parse_ll(e, v)) v = -1;
    if (v >= 0) set_default(d, "LLAR_PROTOCOL", "auto_protocol", e, v);
    else env_warn("LLAR_PROTOCOL", e, "not a protocol name");
  }
  if (const char* e = getenv("LLAR_ACCUM")) {
    if (strcmp(e, "fp32") == 0 || strcmp(e, "binary32") == 0 || strcmp(e, "32") == 0) d.ll128_acc = 0;
    else if (strcmp(e, "16") == 0 || strcmp(e, "packed") == 0 || strcmp(e, "native") == 0) d.ll128_acc = 1;
    else env_warn("LLAR_ACCUM", e, "expected fp32 or 16");
  }
  if (const char* e = getenv("LLAR_LOG")) {
    long long v = 0;
    if (parse_ll(e, v)) set_default(d, "LLAR_LOG", "log", e, v);
    else env_warn("LLAR_LOG", e, "not a number");
  }
  if (const char* e = getenv("LLAR_DEBUG_KEEP_STAGING")) {
    long long v = 0;
    if (parse_ll(e, v)) set_default(d, "LLAR_DEBUG_KEEP_STAGING", "keep_staging", e, v);
    else env_warn("LLAR_DEBUG_KEEP_STAGING", e, "not a number");
  }
  if (const char* e = getenv("LLAR_TUNE")) {
    FILE* f = fopen(e, "r");
    if (!f) return env_warn("LLAR_TUNE", e, "cannot open the file");
    char line[512];
    while (fgets(line, sizeof(line), f)) {
      char* hash = strchr(line, '#');
      if (hash) *hash = '\0';
      for (char* c = line; *c; ++c)
        if (*c == '=' || *c == '\t' || *c == '\r' || *c == '\n') *c = ' ';
      char key[128], val[128];
      if (sscanf(line, "%127s %127s", key, val) != 2) continue;
      long long v = 0;
      if (parse_ll(val, v)) set_default(d, "LLAR_TUNE", key, val, v);
      else env_warn("LLAR_TUNE", val, "not a number");
    }
    fclose(f);
  }
}

llar_comm& defaults_locked() {
  static llar_comm d;
  static bool loaded = false;
  if (!loaded) {
    load_env_defaults(d);
    loaded = true;
  }
  return d;
}

void copy_options(llar_comm* dst, const llar_comm& src) {
  for (const auto& t : kOptions) dst->*(t.field) = src.*(t.field);
}

void log_call(const llar_comm* h, const char* what, int proto, size_t n_elems, const LaunchSpec& ls, uint32_t placement,
              int chunks, bool device_epoch) {
  static const char* const names[] = {"auto", "ll", "sentinel", "ll128", "ll128_pipelined", "sentinel_pipelined"};
  static const char* const dtypes[] = {"fp32", "fp16", "bf16"};
  fprintf(stderr,
          "llar: %s n_ranks=%d dtype=%s elems=%zu bytes=%zu protocol=%s kernel=%d grid=%d threads=%d chunks=%d "
          "placement=%s epoch=%s\n",
          what, h->n_ranks, dtypes[h->kind], n_elems, n_elems * h->elem, (proto >= 0 && proto <= 5) ? names[proto] : "?",
          ls.kernel, ls.grid, ls.threads, chunks, placement == kPlaceLocal ? "local" : "spread",
          device_epoch ? "device" : "host");
}

}  // namespace

extern "C" {

int llar_last_error(void) { return g_last_error; }

const char* llar_status_string(int status) {
  switch (status) {
    case LLAR_OK: return "LLAR_OK";
    case LLAR_ERR_ARG: return "LLAR_ERR_ARG: invalid argument";
    case LLAR_ERR_UNSUPPORTED: return "LLAR_ERR_UNSUPPORTED: unsupported dtype, rank count or size";
    case LLAR_ERR_NOMEM: return "LLAR_ERR_NOMEM: device allocation failed";
    case LLAR_ERR_HIP: return "LLAR_ERR_HIP: HIP runtime error";
    case LLAR_ERR_TIMEOUT: return "LLAR_ERR_TIMEOUT: a device poll exceeded its time limit";
    case LLAR_ERR_DEVICE: return "LLAR_ERR_DEVICE: device-side protocol error";
    default: return "unknown llar status";
  }
}

llar_comm* llar_create(int n_ranks, llar_dtype dtype, size_t max_bytes) {
  if (n_ranks < 1 || (int)dtype < 0 || (int)dtype > 2 || max_bytes == 0) {
    fail(LLAR_ERR_ARG);
    return nullptr;
  }
  if (n_ranks > 8) {
    fail(LLAR_ERR_UNSUPPORTED);
    return nullptr;
  }
  llar_comm* h = new (std::nothrow) llar_comm();
  if (!h) {
    fail(LLAR_ERR_NOMEM);
    return nullptr;
  }
  h->n_ranks = n_ranks;
  h->kind = (int)dtype;
  h->elem = (size_t)elem_bytes_of(dtype);
  h->max_bytes = (max_bytes / h->elem) * h->elem;
  if (h->max_bytes == 0) {
    delete h;
    fail(LLAR_ERR_ARG);
    return nullptr;
  }
  hipError_t e = hipGetDevice(&h->device);
  hipDeviceProp_t prop;
  if (e == hipSuccess) e = hipGetDeviceProperties(&prop, h->device);
  int wc = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wc, hipDeviceAttributeWallClockRate, h->device);
  if (e != hipSuccess) {
    delete h;
    fail(LLAR_ERR_HIP);
    return nullptr;
  }
  h->cu_count = prop.multiProcessorCount;
  h->wall_hz = wc > 0 ? wc * 1000.0 : 100e6;

  const int N = n_ranks;
  const size_t mb = h->max_bytes;
  // LL: [parity][rank 1..N-1][vector][2 x 16 B]
  // (N spare vectors per rank: N blocks of a ReduceScatter or AllGather,
  // each rounded up to whole vectors, fit in (N - 1) rank slots)
  size_t ll_vec = ceil_div(std::min(mb, kCapLL), 16) + (size_t)N;
  h->ll.rank_stride = ll_vec * 32;
  h->ll.parity_stride = h->ll.rank_stride * (size_t)std::max(N - 1, 1);
  // Sentinel one-shot: [parity][rank 1..N-1][vector] 16 B
  size_t s_vec = ceil_div(std::min(mb, kCapSentinel), 16) + (size_t)N;
  h->sent.rank_stride = s_vec * 16;
  h->sent.parity_stride = h->sent.rank_stride * (size_t)std::max(N - 1, 1);
  // LL128 one round: [parity][line] 128 B, binary32 staging needs the most lines
  // (N spare lines: the N segments of a ReduceScatter, each rounded up to
  // whole lines, fit)
  size_t l_one = ceil_div(std::min(mb, kCapLL128) / h->elem, 31) + 1 + (size_t)N;
  h->ll128.parity_stride = l_one * 128;
  // LL128 pipelined: [buffer][line]: two buffers of the largest chunk, or
  // 32 of a chunk up to 256 KiB (the wave-split pipeline's default), which
  // ever is larger
  const size_t chunk_cap = std::max(std::min(ceil_div(mb, 16) * 16, kCapChunk), (size_t)1024);
  size_t l_pipe = ceil_div(chunk_cap / h->elem, 31) + 1;
  size_t l_pipe32 = ceil_div(std::min(chunk_cap, kLL128PipeChunk) / h->elem, 31) + 1;
  h->ll128_pipe.parity_stride = std::max(l_pipe, 16 * l_pipe32) * 128;
  // Sentinel pipelined: [parity][owner][sender][shard vector] 16 B
  size_t cap = sentinel_shard_cap(chunk_cap, N);
  h->sent_pipe.parity_stride = (size_t)N * (size_t)N * cap * 16;

  e = hipMalloc(&h->timing_wg, (size_t)kTimingRing * kTimingMaxWgs * 2 * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMalloc(&h->ctrl, sizeof(Ctrl));
  if (e == hipSuccess) e = hipMalloc(&h->trace, (size_t)kTraceMaxWgs * kTraceWords * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMemset(h->trace, 0, (size_t)kTraceMaxWgs * kTraceWords * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMalloc(&h->pipe_trace, (size_t)kPipeTraceMaxWgs * kPipeTraceWords * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMemset(h->pipe_trace, 0, (size_t)kPipeTraceMaxWgs * kPipeTraceWords * sizeof(uint64_t));
  if (e == hipSuccess) e = hipMalloc(&h->credit, kCreditBytes);
  if (e == hipSuccess) e = hipMemset(h->credit, 0, kCreditBytes);
  if (e == hipSuccess) e = alloc_region(h->ll, 2 * h->ll.parity_stride, 0);
  if (e == hipSuccess) e = alloc_region(h->sent, 2 * h->sent.parity_stride, 0xFF);
  if (e == hipSuccess) e = alloc_region(h->ll128, 2 * h->ll128.parity_stride, 0);
  if (e == hipSuccess) e = alloc_region(h->ll128_pipe, 2 * h->ll128_pipe.parity_stride, 0);
  if (e == hipSuccess) e = alloc_region(h->sent_pipe, kSentinelPipeMaxBuffers * h->sent_pipe.parity_stride, 0xFF);
  // the control block names the regions that a wrap of the epoch clears
  if (e == hipSuccess) e = init_ctrl(h);
  // every region is addressed with 32-bit offsets
  const Region* regs[] = {&h->ll, &h->sent, &h->ll128, &h->ll128_pipe, &h->sent_pipe};
  for (const Region* r : regs)
    if (r->bytes >= (1ull << 32)) {
      destroy_all(h);
      fail(LLAR_ERR_UNSUPPORTED);
      return nullptr;
    }
  // placement check: the local placement needs workgroup b on XCD b % 8
  if (e == hipSuccess) {
    uint32_t* d = nullptr;
    const int G = 64;
    e = hipMalloc(&d, G * sizeof(uint32_t));
    if (e == hipSuccess) e = launch_xcc_probe(d, G, 0);
    std::vector<uint32_t> hx(G, 99u);
    if (e == hipSuccess) e = hipMemcpy(hx.data(), d, G * sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (d) (void)hipFree(d);
    if (e == hipSuccess) {
      // Workgroups are dealt to the 8 XCDs round-robin; the starting XCD may
      // rotate from launch to launch, which the placements tolerate.  What
      // they need: ids equal mod 8 share an XCD, and 8 consecutive ids cover
      // 8 distinct XCDs.
      bool ok = true;
      uint32_t seen = 0;
      for (int i = 0; i < 8; ++i) seen |= 1u << (hx[i] & 31u);
      ok &= (seen == 0xFFu);
      for (int i = 8; i < G; ++i) ok &= (hx[i] == hx[i % 8]);
      h->local_ok = ok;
    }
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    int st = (e == hipErrorOutOfMemory) ? LLAR_ERR_NOMEM : LLAR_ERR_HIP;
    destroy_all(h);
    fail(st);
    return nullptr;
  }
  {
    std::lock_guard<std::mutex> lock(g_defaults_mu);
    copy_options(h, defaults_locked());
  }
  if (h->placement == 2 && !h->local_ok) h->placement = 0;
  if (h->debug_drop_rank >= h->n_ranks) h->debug_drop_rank = -1;
  g_last_error = LLAR_OK;
  return h;
}

int llar_destroy(llar_comm* h) {
  if (!h) return LLAR_OK;
  destroy_all(h);
  return LLAR_OK;
}

int llar_select_protocol(llar_comm* h, size_t bytes) {
  if (!h) return fail(LLAR_ERR_ARG);
  return auto_protocol(h, bytes);
}

int llar_launch_geometry(llar_comm* h, size_t n_elems, llar_protocol protocol, int* grid, int* threads, int* slices,
                         int* chunks) {
  if (!h) return fail(LLAR_ERR_ARG);
  int proto = protocol == LLAR_AUTO ? auto_protocol(h, n_elems * h->elem) : (int)protocol;
  Geometry g;
  int st = plan(h, n_elems, proto, g);
  if (st != LLAR_OK) return fail(st);
  if (grid) *grid = (h->n_ranks + oneshot_split(h, g.kernel) - 1) * g.grid_slices;
  if (threads) *threads = g.threads;
  if (slices) *slices = g.slices;
  if (chunks) *chunks = g.chunks;
  return LLAR_OK;
}

namespace {

uint64_t spin_ticks(const llar_comm* h) { return (uint64_t)((double)h->spin_timeout_us * 1e-6 * h->wall_hz); }

// Epoch source of a call: the host numbers stream-ordered calls; a captured
// call must read the device-resident epoch (its arguments repeat on replay).
bool call_epoch(const llar_comm* h, hipStream_t stream, bool& device_epoch, uint32_t& host_epoch) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return false;
  device_epoch = h->device_epoch || cap != hipStreamCaptureStatusNone;
  host_epoch = device_epoch ? 0u : h->host_epoch;
  return true;
}

void finish_call(llar_comm* h, bool device_epoch) {
  h->last_call_device = device_epoch;
  if (!device_epoch) {
    if (llar_wire::epoch_wraps(h->host_epoch)) h->host_wrap_pending = true;
    h->host_epoch = next_host_epoch(h->host_epoch);
  }
}

// After the host epoch wrapped, every epoch value comes round again: an LL
// line or owner-credit progress word that no call has written for a whole
// cycle of 2^31 - 1 calls would pass for the new call's.  The first
// host-numbered call after the wrap therefore clears both first, ordered on
// its own stream.  (Host-numbered calls are never captured into a graph;
// device-numbered calls clear at their own wrap on the device.)
hipError_t clear_after_host_wrap(llar_comm* h, bool device_epoch, hipStream_t stream) {
  if (device_epoch || !h->host_wrap_pending) return hipSuccess;
  hipError_t e = hipSuccess;
  if (h->ll.ptr) e = hipMemsetAsync(h->ll.ptr, 0, h->ll.bytes, stream);
  if (e == hipSuccess && h->credit) e = hipMemsetAsync(h->credit, 0, kCreditBytes, stream);
  if (e == hipSuccess) h->host_wrap_pending = false;
  return e;
}

// Issue one call of the planned kernel.  `n_launch` ranks take part (the
// communicator's rank count, or two for a point-to-point copy); `parts`
// holds their input pointers.
int issue(llar_comm* h, const void* const* parts, int n_launch, void* out, size_t n_elems, int proto,
          const Geometry& g, hipStream_t stream) {
  const size_t nbytes = n_elems * h->elem;
  // the barrier ablation stages raw vectors in the LL region and leaves what
  // it used zero (invalid LL lines)
  const bool barrier = g.kernel == kKernBarrier || g.kernel == kKernBarrierLocal;
  const Region* reg = barrier ? &h->ll : region_of(h, proto);

  LaunchSpec ls;
  memset(&ls, 0, sizeof(ls));
  ls.kind = h->kind;
  ls.n_ranks = n_launch;
  ls.kernel = g.kernel;
  ls.threads = g.threads;
  ls.oneshot_split = oneshot_split(h, g.kernel);
  ls.grid = (n_launch + ls.oneshot_split - 1) * g.grid_slices;

  // every workgroup must be resident at once: consumers spin on producers
  int occ = occupancy_of(h, n_launch, g.kernel, g.threads);
  if (occ <= 0) return fail(LLAR_ERR_HIP);
  if (ls.grid > occ * h->cu_count) return fail(LLAR_ERR_UNSUPPORTED);
  if (h->timing && ls.grid > kTimingMaxWgs) return fail(LLAR_ERR_UNSUPPORTED);

  const uint64_t spin = spin_ticks(h);
  bool device_epoch = false;
  uint32_t host_epoch = 0;
  if (!call_epoch(h, stream, device_epoch, host_epoch)) return fail(LLAR_ERR_HIP);
  // a device-numbered call records the epoch per workgroup
  if (device_epoch && ls.grid > kTimingMaxWgs) return fail(LLAR_ERR_UNSUPPORTED);
  const bool is_oneshot = g.kernel == kKernOneShotLL || g.kernel == kKernOneShotSentinel ||
                          g.kernel == kKernOneShotLLLocal || g.kernel == kKernOneShotSentinelLocal ||
                          g.kernel == kKernP2PLL || g.kernel == kKernP2PSentinel || g.kernel == kKernP2PLLLocal ||
                          g.kernel == kKernP2PSentinelLocal || g.kernel == kKernBarrier ||
                          g.kernel == kKernBarrierLocal;
  if (is_oneshot) {
    OneShotArgs& a = ls.oneshot;
    for (int r = 0; r < n_launch; ++r) a.part[r] = static_cast<const uint8_t*>(parts[r]);
    a.out = static_cast<uint8_t*>(out);
    a.stage = reg->ptr;
    a.ctrl = h->ctrl;
    a.nbytes = nbytes;
    a.spin_limit = spin;
    a.n_vec = (uint32_t)ceil_div(nbytes, 16);
    a.stage_bytes = (uint32_t)reg->bytes;
    a.parity_stride = (uint32_t)reg->parity_stride;
    a.rank_stride = (uint32_t)reg->rank_stride;
    a.grid = (uint32_t)ls.grid;
    a.slices = (uint32_t)g.slices;
    a.vq = a.n_vec / a.slices;
    a.vr = a.n_vec % a.slices;
    a.placement = g.placement;
    a.timing = h->timing ? 1u : 0u;
    a.keep = h->keep_staging ? 1u : 0u;
    a.drop_rank = h->debug_drop_rank < 0 ? 0xFFFFFFFFu : (uint32_t)h->debug_drop_rank;
    a.trace = (h->trace_on && ls.grid <= kTraceMaxWgs) ? h->trace : nullptr;
    if (a.trace) h->trace_grid = ls.grid;
    a.host_epoch = host_epoch;
    a.xcd_span = (uint32_t)g.xcd_span;
  } else {
    TwoShotArgs& a = ls.twoshot;
    for (int r = 0; r < n_launch; ++r) a.part[r] = static_cast<const uint8_t*>(parts[r]);
    a.out = static_cast<uint8_t*>(out);
    a.stage = reg->ptr;
    a.ctrl = h->ctrl;
    a.n = n_elems;
    a.spin_limit = spin;
    a.chunk_elems = g.chunk_elems;
    a.n_chunks = (uint32_t)g.chunks;
    a.stage_bytes = (uint32_t)reg->bytes;
    a.parity_stride = (uint32_t)reg->parity_stride;
    a.n_buffers = (proto == LLAR_SENTINEL_PIPELINED) ? (uint32_t)h->pipe_buffers : 2u;
    a.shard_cap = (proto == LLAR_SENTINEL_PIPELINED)
                      ? (uint32_t)(reg->parity_stride / ((size_t)h->n_ranks * h->n_ranks * 16))
                      : 0u;
    a.credit = nullptr;
    a.cons_groups = 1u;
    a.prod_groups = 1u;
    if (g.kernel == kKernSentinelPipe || g.kernel == kKernSentinelPipeLocal) {
      // the workgroup credit needs an even buffer count (B >= 2 lag + 2);
      // consumer groups must divide both the consumer waves (half of the
      // workgroup's) and B
      if (a.n_buffers % 2u != 0u) return fail(LLAR_ERR_ARG);
      // Default two groups where the waves split evenly: measured on MI355X,
      // 64 MiB x 8 bf16 in 1 MiB chunks, 4 buffers, two boxes alternating,
      // 284-292 against 296-311 us per call; four one-wave groups, which need
      // two batches per chunk, 455-465 us
      const uint32_t n_cons = (uint32_t)g.threads / 64u - (uint32_t)g.threads / 128u;
      const uint32_t n_prod = (uint32_t)g.threads / 128u;
      const uint32_t G = h->cons_groups > 0 ? (uint32_t)h->cons_groups : (n_cons % 2u == 0u ? 2u : 1u);
      const uint32_t PG = h->prod_groups > 0 ? (uint32_t)h->prod_groups : 1u;
      if (n_cons % G != 0u || a.n_buffers % G != 0u) return fail(LLAR_ERR_ARG);
      if (n_prod % PG != 0u) return fail(LLAR_ERR_ARG);
      a.cons_groups = G;
      a.prod_groups = PG;
      // buffers spaced by this chunk's own stride, so that small chunks can
      // use more of them in the same region
      a.shard_cap = sentinel_shard_cap((size_t)g.chunk_elems * h->elem, h->n_ranks);
      const size_t stride = (size_t)h->n_ranks * h->n_ranks * a.shard_cap * 16;
      if (stride * a.n_buffers > reg->bytes) return fail(LLAR_ERR_UNSUPPORTED);
      a.parity_stride = (uint32_t)stride;
    }
    if (g.kernel == kKernSentinelHs || g.kernel == kKernSentinelHsLocal) {
      // Slot handshake: the chunk-c and chunk-(c - B) uses of a slot are
      // consumer items c*n_bat + b and (c - B)*n_bat + b, taken by consumer
      // wave item % n_cons, and producer items kH times those (plus the
      // owner group), taken by producer wave item % n_prod.  A slot keeps one
      // producer lane and one consumer lane only if n_prod divides
      // B*n_bat*kH and n_cons divides B*n_bat: B is the smallest multiple of
      // the least such period that is at least the requested buffer count.
      const uint32_t nv = (uint32_t)((size_t)g.chunk_elems * h->elem / 16);
      const uint32_t span = (uint32_t)ceil_div(ceil_div(nv, (size_t)h->n_ranks), (size_t)g.slices);
      const uint32_t n_bat = (span + 63u) / 64u;
      const uint32_t n_waves = (uint32_t)g.threads / 64u;
      uint32_t n_cons = n_waves >= 4 ? n_waves / 4 : 1u;
      if (h->cons_waves > 0) n_cons = (uint32_t)h->cons_waves;
      if (n_cons >= n_waves) return fail(LLAR_ERR_ARG);
      const uint32_t n_prod = n_waves - n_cons;
      a.cons_waves = n_cons;
      // producer items split a consumer item into kH owner groups
      const uint32_t kg = (uint32_t)(h->n_ranks + 1) / 2u, kh = ((uint32_t)h->n_ranks + kg - 1u) / kg;
      const uint32_t b_prod = n_prod / std::gcd(n_prod, n_bat * kh);
      const uint32_t b_cons = n_cons / std::gcd(n_cons, n_bat);
      const uint32_t b0 = std::lcm(b_prod, b_cons);
      a.n_buffers = b0 * (uint32_t)ceil_div((size_t)h->pipe_buffers, (size_t)b0);
      a.shard_cap = sentinel_shard_cap((size_t)g.chunk_elems * h->elem, h->n_ranks);
      const size_t stride = (size_t)h->n_ranks * h->n_ranks * a.shard_cap * 16;
      if (stride * a.n_buffers > reg->bytes) return fail(LLAR_ERR_UNSUPPORTED);
      a.parity_stride = (uint32_t)stride;
    }
    if (g.kernel == kKernSentinelOc || g.kernel == kKernSentinelOcLocal) {
      // owner credit: one progress word per (rank, slice, consumer wave);
      // one wave of each workgroup reads them, the rest produce
      const uint32_t n_waves = (uint32_t)g.threads / 64u;
      const uint32_t n_cons = h->cons_waves > 0 ? (uint32_t)h->cons_waves : (n_waves - 1u) / 2u;
      if (n_cons < 1u || n_cons > (uint32_t)kCreditWaves || n_cons + 2u > n_waves) return fail(LLAR_ERR_ARG);
      if (g.slices > kCreditSlices) return fail(LLAR_ERR_UNSUPPORTED);
      // kept staging is never reset, so no buffer may be used twice
      if (h->keep_staging && g.chunks > (int)a.n_buffers) return fail(LLAR_ERR_UNSUPPORTED);
      a.cons_waves = n_cons;
      a.credit = h->credit;
      a.shard_cap = sentinel_shard_cap((size_t)g.chunk_elems * h->elem, h->n_ranks);
      const size_t stride = (size_t)h->n_ranks * h->n_ranks * a.shard_cap * 16;
      if (stride * a.n_buffers > reg->bytes) return fail(LLAR_ERR_UNSUPPORTED);
      a.parity_stride = (uint32_t)stride;
    }
    const bool ll128_ws = g.kernel == kKernLL128WsAcc32 || g.kernel == kKernLL128WsAcc16;
    if (ll128_ws) {
      // producer and consumer waves; B buffers spaced by this chunk's lines.
      // The workgroup credit needs an even B (run-ahead B/2 - 1 chunks) and
      // the consumer of chunk c - B must be the consumer of chunk c
      // (n_cons divides B).  B shrinks to what the region holds.
      const uint32_t n_waves = (uint32_t)g.threads / 64u;
      uint32_t n_cons = h->cons_waves > 0 ? (uint32_t)h->cons_waves : std::max(1u, n_waves / 4u);
      if (n_waves < 2u || n_cons >= n_waves || n_cons > 16u) return fail(LLAR_ERR_ARG);
      const size_t K = g.kernel == kKernLL128WsAcc16 ? 63 : 31;
      const size_t stride = ceil_div((size_t)g.chunk_elems, K) * 128;
      const uint32_t fit = (uint32_t)std::min<size_t>(reg->bytes / stride, 64);
      uint32_t B = std::min<uint32_t>(h->ll128_buffers > 0 ? (uint32_t)h->ll128_buffers : 32u, fit);
      B -= B % 2u;
      if (B < 2u) return fail(LLAR_ERR_UNSUPPORTED);
      if (h->cons_waves > 0) {
        B -= B % std::lcm(2u, n_cons);
        if (B < 2u) return fail(LLAR_ERR_UNSUPPORTED);
      } else {
        n_cons = std::gcd(n_cons, B);  // the default split adapts to the buffers that fit
      }
      // kept staging is never zeroed, so no buffer may be used twice
      if (h->keep_staging && g.chunks > (int)B) return fail(LLAR_ERR_UNSUPPORTED);
      a.n_buffers = B;
      a.cons_waves = n_cons;
      a.parity_stride = (uint32_t)stride;
    }
    a.grid = (uint32_t)ls.grid;
    a.slices = (uint32_t)g.slices;
    a.placement = g.placement;
    a.timing = h->timing ? 1u : 0u;
    a.keep = h->keep_staging ? 1u : 0u;
    a.drop_rank = h->debug_drop_rank < 0 ? 0xFFFFFFFFu : (uint32_t)h->debug_drop_rank;
    a.host_epoch = host_epoch;
    a.trace = nullptr;
    a.threads = (uint32_t)ls.threads;
    a.slices_rcp = 0u;
    const bool pipe_kernel = g.kernel == kKernSentinelPipe || g.kernel == kKernSentinelPipeLocal ||
                             g.kernel == kKernSentinelHs || g.kernel == kKernSentinelHsLocal ||
                             g.kernel == kKernSentinelOc || g.kernel == kKernSentinelOcLocal;
    if (h->trace_on && pipe_kernel && ls.grid <= kPipeTraceMaxWgs) {
      a.trace = h->pipe_trace;
      h->pipe_trace_grid = ls.grid;
    }
    // the chunk must fit the staging that was allocated
    if (proto == LLAR_SENTINEL_PIPELINED) {
      uint32_t need = sentinel_shard_cap((size_t)g.chunk_elems * h->elem, h->n_ranks);
      if (need > a.shard_cap) return fail(LLAR_ERR_UNSUPPORTED);
    } else if (!ll128_ws) {
      size_t K = (g.kernel == kKernLL128Acc16) ? 63 : 31;
      size_t lines = ceil_div((size_t)g.chunk_elems, K);  // the nominal chunk's lines
      if (lines * 128 > reg->parity_stride) return fail(LLAR_ERR_UNSUPPORTED);
      // The line partition divides w x (lines of an owner) by the slice
      // count, w <= slices.  With m = ceil(2^32 / d) and e = m d - 2^32 < d,
      // umulhi(x, m) = floor(x / d) whenever x e < 2^32 (the error term
      // x e / (d 2^32) then stays below 1 / d), so the kernel multiplies
      // instead of dividing when that holds for the largest numerator.
      a.slices_rcp = 0u;
      const uint64_t d = (uint64_t)g.slices;
      if (d >= 2u) {
        const uint64_t m = ((1ull << 32) + d - 1u) / d;
        const uint64_t e = m * d - (1ull << 32);
        const uint64_t x_max = d * ceil_div((uint64_t)lines, (uint64_t)h->n_ranks);
        if (m <= 0xFFFFFFFFull && x_max < (1ull << 32) && x_max * e < (1ull << 32)) a.slices_rcp = (uint32_t)m;
      }
    }
  }
  if (!reg->ptr) return fail(LLAR_ERR_UNSUPPORTED);
  if (clear_after_host_wrap(h, device_epoch, stream) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (h->log) {
    const bool p2p = g.kernel >= kKernP2PLL && g.kernel <= kKernP2PSentinelLocal;
    log_call(h, p2p ? "send_recv" : "allreduce", proto, n_elems, ls, g.placement, g.chunks, device_epoch);
  }
  hipError_t e = launch(ls, stream);
  if (e != hipSuccess) return fail(LLAR_ERR_HIP);
  finish_call(h, device_epoch);
  return LLAR_OK;
}

// ReduceScatter (gather = false) or AllGather (gather = true) of `count`
// elements per block over the LL or Sentinel wire: one launch in which every
// rank sends to and receives from every other rank.  `n_recv` ranks receive
// (N, or 1 for an AllGather seen by rank 0 only).
int run_multi(llar_comm* h, const void* const* ins, void* const* outs, int n_recv, size_t count, llar_dtype dtype,
              llar_protocol protocol, bool gather, hipStream_t stream) {
  if (!h || !ins || !outs) return fail(LLAR_ERR_ARG);
  if ((int)dtype != h->kind) return fail(LLAR_ERR_ARG);
  const int N = h->n_ranks;
  if (n_recv != N && !(gather && n_recv == 1)) return fail(LLAR_ERR_ARG);
  const bool atomic = (protocol == LLAR_LL128 && !gather);  // the reduce-scatter half of the two-shot
  if (protocol != LLAR_AUTO && protocol != LLAR_LL && protocol != LLAR_SENTINEL && !atomic) return fail(LLAR_ERR_ARG);
  if (count == 0) return LLAR_OK;
  if (count > h->max_bytes / h->elem / (size_t)N) return fail(LLAR_ERR_ARG);
  for (int r = 0; r < N; ++r)
    if (!ins[r] || !aligned16(ins[r])) return fail(LLAR_ERR_ARG);
  for (int r = 0; r < n_recv; ++r)
    if (!outs[r] || !aligned16(outs[r])) return fail(LLAR_ERR_ARG);
  const size_t blk = count * h->elem;
  const size_t total = blk * (size_t)N;
  int proto = (int)protocol;
  if (protocol == LLAR_AUTO) proto = ((long long)total <= h->thr_sentinel && total <= kCapLL) ? LLAR_LL : LLAR_SENTINEL;
  if (total > (proto == LLAR_LL ? kCapLL : proto == LLAR_LL128 ? kCapLL128 : kCapSentinel))
    return fail(LLAR_ERR_UNSUPPORTED);
  const Region* reg = region_of(h, proto);
  if (!reg->ptr) return fail(LLAR_ERR_UNSUPPORTED);

  // measured on MI355X: the atomic reduce-scatter issues best from 512-thread
  // workgroups (1 MiB: 28 us against 32 us at 256; equal at 16 KiB)
  const int threads = h->threads ? (int)h->threads : (atomic ? 512 : 256);
  if (threads != 64 && threads != 128 && threads != 256 && threads != 512) return fail(LLAR_ERR_ARG);
  if (atomic) {
    // owner o's segment in lines o*Lo .. o*Lo+Lo-1 of one parity; every
    // owner's lines split into the same slices
    const bool acc16 = (h->ll128_acc == 1) && h->kind != kKindF32;
    const size_t K = acc16 ? 63 : 31;
    const size_t lo_lines = ceil_div(count, K);
    if ((size_t)N * lo_lines * 128 > reg->parity_stride) return fail(LLAR_ERR_UNSUPPORTED);
    // one slice per line of an owner's segment, up to 64 (measured on
    // MI355X: 16 KiB x 8 bf16 4.6 us against 5.7 at one slice per 8 lines)
    const int slices = h->slices ? (int)h->slices : clampi((long long)lo_lines, 1, 64);
    LaunchSpec ls;
    memset(&ls, 0, sizeof(ls));
    ls.kind = h->kind;
    ls.n_ranks = N;
    ls.kernel = acc16 ? kKernRsLL128Acc16 : kKernRsLL128Acc32;
    ls.threads = threads;
    ls.grid = N * slices;
    int occ = occupancy_of(h, N, ls.kernel, threads);
    if (occ <= 0) return fail(LLAR_ERR_HIP);
    if (ls.grid > occ * h->cu_count) return fail(LLAR_ERR_UNSUPPORTED);
    if (h->timing && ls.grid > kTimingMaxWgs) return fail(LLAR_ERR_UNSUPPORTED);
    bool device_epoch = false;
    uint32_t host_epoch = 0;
    if (!call_epoch(h, stream, device_epoch, host_epoch)) return fail(LLAR_ERR_HIP);
    if (device_epoch && ls.grid > kTimingMaxWgs) return fail(LLAR_ERR_UNSUPPORTED);
    MultiArgs& a = ls.multi;
    for (int r = 0; r < N; ++r) {
      a.in[r] = static_cast<const uint8_t*>(ins[r]);
      a.out[r] = static_cast<uint8_t*>(outs[r]);
    }
    a.stage = reg->ptr;
    a.ctrl = h->ctrl;
    a.blk = blk;
    a.spin_limit = spin_ticks(h);
    a.stage_bytes = (uint32_t)reg->bytes;
    a.parity_stride = (uint32_t)reg->parity_stride;
    a.n_recv = (uint32_t)N;
    a.grid = (uint32_t)ls.grid;
    a.slices = (uint32_t)slices;
    a.timing = h->timing ? 1u : 0u;
    a.keep = h->keep_staging ? 1u : 0u;
    a.drop_rank = h->debug_drop_rank < 0 ? 0xFFFFFFFFu : (uint32_t)h->debug_drop_rank;
    a.host_epoch = host_epoch;
    if (clear_after_host_wrap(h, device_epoch, stream) != hipSuccess) return fail(LLAR_ERR_HIP);
    if (h->log) log_call(h, "reduce_scatter", proto, count, ls, kPlaceSpread, 1, device_epoch);
    hipError_t e = launch(ls, stream);
    if (e != hipSuccess) return fail(LLAR_ERR_HIP);
    finish_call(h, device_epoch);
    return LLAR_OK;
  }
  const size_t nv = ceil_div(blk, 16);
  // measured on MI355X (bf16; N = 8 at 1 KiB to 1 MiB in total over every
  // power of two from 1 to 64 slices, N = 2 and 4 at 1 KiB to 1 MiB): from 8
  // slices on the local placement keeps each slice's exchange on one XCD, and
  // 2 to 7 slices, spread over the XCDs, lose to both 1 and 8.  The best
  // count grows as about the square root of a block's 8-byte units (8-16 at
  // 16 to 256 units, 32 at 2048, 64 and more at 16384): N = 8 device time
  // 16 KiB RS 2.74 -> 2.27 us, AG 2.61 -> 2.11; 128 KiB RS 3.42 -> 2.79;
  // 1 MiB RS 6.16 -> 4.65 against the earlier square root / 4.  One slice
  // stays best for an exchange under 2 KiB among fewer than 8 ranks (N = 2
  // and 4 at 1 KiB: 3.1-3.3 against 3.4-3.8 us per call at 8 slices), and
  // blocks of fewer than 8 vectors keep the one slice the earlier rule gave
  // them (not re-measured).
  int slices = (int)h->slices;
  if (!slices)
    slices = (nv < 8 || (N < 8 && total < 2048)) ? 1 : clampi(std::llround(std::sqrt((double)(2 * nv)) / 1.5), 8, 64);
  uint32_t place = kPlaceSpread;
  if (h->local_ok && (h->placement == 2 || (h->placement == 0 && slices >= 8))) place = kPlaceLocal;
  const int grid_slices = place == kPlaceLocal ? (int)ceil_div((size_t)slices, 8) * 8 : slices;
  int kernel;
  if (gather) kernel = proto == LLAR_LL ? kKernAgLL : kKernAgSentinel;
  else kernel = proto == LLAR_LL ? kKernRsLL : kKernRsSentinel;
  if (place == kPlaceLocal) kernel += kKernRsLLLocal - kKernRsLL;

  // staging: N receivers x (N - 1) sender slots per parity
  const size_t slot_stride = nv * (proto == LLAR_LL ? 32 : 16);
  if ((size_t)N * (size_t)std::max(N - 1, 1) * slot_stride > reg->parity_stride) return fail(LLAR_ERR_UNSUPPORTED);

  LaunchSpec ls;
  memset(&ls, 0, sizeof(ls));
  ls.kind = h->kind;
  ls.n_ranks = N;
  ls.kernel = kernel;
  ls.threads = threads;
  ls.grid = N * grid_slices;
  int occ = occupancy_of(h, N, kernel, threads);
  if (occ <= 0) return fail(LLAR_ERR_HIP);
  if (ls.grid > occ * h->cu_count) return fail(LLAR_ERR_UNSUPPORTED);
  if (h->timing && ls.grid > kTimingMaxWgs) return fail(LLAR_ERR_UNSUPPORTED);

  bool device_epoch = false;
  uint32_t host_epoch = 0;
  if (!call_epoch(h, stream, device_epoch, host_epoch)) return fail(LLAR_ERR_HIP);
  // a device-numbered call records the epoch per workgroup
  if (device_epoch && ls.grid > kTimingMaxWgs) return fail(LLAR_ERR_UNSUPPORTED);
  MultiArgs& a = ls.multi;
  for (int r = 0; r < N; ++r) a.in[r] = static_cast<const uint8_t*>(ins[r]);
  for (int r = 0; r < n_recv; ++r) a.out[r] = static_cast<uint8_t*>(outs[r]);
  a.stage = reg->ptr;
  a.ctrl = h->ctrl;
  a.blk = blk;
  a.spin_limit = spin_ticks(h);
  a.vq = (uint32_t)(nv / (size_t)slices);
  a.vr = (uint32_t)(nv % (size_t)slices);
  a.stage_bytes = (uint32_t)reg->bytes;
  a.parity_stride = (uint32_t)reg->parity_stride;
  a.slot_stride = (uint32_t)slot_stride;
  a.n_recv = (uint32_t)n_recv;
  a.aligned = (blk % 16 == 0) ? 1u : 0u;
  a.grid = (uint32_t)ls.grid;
  a.slices = (uint32_t)slices;
  a.timing = h->timing ? 1u : 0u;
  a.keep = h->keep_staging ? 1u : 0u;
  a.drop_rank = h->debug_drop_rank < 0 ? 0xFFFFFFFFu : (uint32_t)h->debug_drop_rank;
  a.host_epoch = host_epoch;
  if (clear_after_host_wrap(h, device_epoch, stream) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (h->log) log_call(h, gather ? "all_gather" : "reduce_scatter", proto, count, ls, place, 1, device_epoch);
  hipError_t e = launch(ls, stream);
  if (e != hipSuccess) return fail(LLAR_ERR_HIP);
  finish_call(h, device_epoch);
  return LLAR_OK;
}

}  // namespace

int llar_allreduce(llar_comm* h, const void* const* partials, void* out, size_t n_elems, llar_dtype dtype,
                   llar_protocol protocol, void* stream) {
  if (!h || !partials) return fail(LLAR_ERR_ARG);
  if ((int)dtype != h->kind) return fail(LLAR_ERR_ARG);
  if (n_elems == 0) return LLAR_OK;
  if (!out || !aligned16(out)) return fail(LLAR_ERR_ARG);
  if (n_elems > h->max_bytes / h->elem) return fail(LLAR_ERR_ARG);
  for (int r = 0; r < h->n_ranks; ++r)
    if (!partials[r] || !aligned16(partials[r])) return fail(LLAR_ERR_ARG);
  if ((int)protocol < 0 || (int)protocol > LLAR_SENTINEL_PIPELINED) return fail(LLAR_ERR_ARG);

  const size_t nbytes = n_elems * h->elem;
  const int proto = protocol == LLAR_AUTO ? auto_protocol(h, nbytes) : (int)protocol;
  Geometry g;
  int st = plan(h, n_elems, proto, g);
  if (st != LLAR_OK) return fail(st);
  if (h->barrier_ablation && (proto == LLAR_LL || proto == LLAR_SENTINEL)) {
    // the same one-shot geometry, synchronised by a grid-wide barrier
    if (nbytes > kCapLL) return fail(LLAR_ERR_UNSUPPORTED);
    g.kernel = g.placement == kPlaceLocal ? kKernBarrierLocal : kKernBarrier;
    if (g.placement == kPlaceLocal && g.xcd_span != 8) {
      g.xcd_span = 8;
      g.grid_slices = (int)ceil_div((size_t)g.slices, 8) * 8;
    }
  }
  return issue(h, partials, h->n_ranks, out, n_elems, proto, g, static_cast<hipStream_t>(stream));
}

int llar_send_recv(llar_comm* h, const void* send_buf, void* recv_buf, size_t n_elems, llar_dtype dtype,
                   llar_protocol protocol, void* stream) {
  if (!h) return fail(LLAR_ERR_ARG);
  if ((int)dtype != h->kind) return fail(LLAR_ERR_ARG);
  if (n_elems == 0) return LLAR_OK;
  if (!send_buf || !recv_buf || !aligned16(send_buf) || !aligned16(recv_buf)) return fail(LLAR_ERR_ARG);
  if (n_elems > h->max_bytes / h->elem) return fail(LLAR_ERR_ARG);
  if (protocol != LLAR_AUTO && protocol != LLAR_LL && protocol != LLAR_SENTINEL) return fail(LLAR_ERR_ARG);
  const size_t nbytes = n_elems * h->elem;
  int proto = (int)protocol;
  if (protocol == LLAR_AUTO) proto = ((long long)nbytes <= h->thr_sentinel && nbytes <= kCapLL) ? LLAR_LL : LLAR_SENTINEL;
  Geometry g;
  int st = plan(h, n_elems, proto, g);
  if (st != LLAR_OK) return fail(st);
  // measured on MI355X (8 KB and 256 KiB fp16): a single sender streams
  // best from 512-thread workgroups, one slice per 1024 8-byte units
  if (!h->threads) g.threads = 512;
  if (!h->local_xcds) g.xcd_span = 8;  // the AllReduce's small-call span is not measured for it
  if (!h->slices) g.slices = clampi((long long)ceil_div(2 * ceil_div(nbytes, 16), (size_t)1024), 2, 64);
  g.grid_slices = g.placement == kPlaceLocal ? (int)ceil_div((size_t)g.slices, (size_t)g.xcd_span) * 8 : g.slices;
  // the one-shot exchange with a single producer, in copy mode
  switch (g.kernel) {
    case kKernOneShotLL: g.kernel = kKernP2PLL; break;
    case kKernOneShotSentinel: g.kernel = kKernP2PSentinel; break;
    case kKernOneShotLLLocal: g.kernel = kKernP2PLLLocal; break;
    case kKernOneShotSentinelLocal: g.kernel = kKernP2PSentinelLocal; break;
    default: return fail(LLAR_ERR_ARG);
  }
  // rank 1 sends; rank 0 receives and reads no input of its own
  const void* parts[2] = {send_buf, send_buf};
  return issue(h, parts, 2, recv_buf, n_elems, proto, g, static_cast<hipStream_t>(stream));
}

int llar_reduce_scatter(llar_comm* h, const void* const* partials, void* const* outs, size_t recv_count,
                        llar_dtype dtype, llar_protocol protocol, void* stream) {
  return run_multi(h, partials, outs, h ? h->n_ranks : 0, recv_count, dtype, protocol, false,
                   static_cast<hipStream_t>(stream));
}

int llar_all_gather(llar_comm* h, const void* const* inputs, void* const* outs, int n_outs, size_t send_count,
                    llar_dtype dtype, llar_protocol protocol, void* stream) {
  return run_multi(h, inputs, outs, n_outs, send_count, dtype, protocol, true, static_cast<hipStream_t>(stream));
}

int llar_get_device_status(llar_comm* h, uint32_t* bits) {
  if (!h) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  uint32_t s = 0;
  if (hipMemcpy(&s, &h->ctrl->status, sizeof(s), hipMemcpyDeviceToHost) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (bits) *bits = s;
  if (s & kStatusTimeout) return LLAR_ERR_TIMEOUT;
  if (s) return LLAR_ERR_DEVICE;
  return LLAR_OK;
}

int llar_clear_device_status(llar_comm* h) {
  if (!h) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  if (init_ctrl(h) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (reset_staging(h) != hipSuccess) return fail(LLAR_ERR_HIP);
  return LLAR_OK;
}

// Tests of the epoch wrap: place the next call's epoch anywhere in its
// range.  "debug_host_epoch" numbers the next stream-ordered call (1 ..
// 2^31 - 1); "debug_device_epoch" sets the device-resident epoch (2^31 + 1 ..
// 2^32 - 1) and zeroes the per-workgroup epoch words, as a fresh control
// block has them.  Neither touches staging: lines written at earlier epochs
// stay, as they would after a real cycle of calls.
static int set_debug_epoch(llar_comm* h, bool device, long long value) {
  if (!device) {
    if (value < 1 || value > (long long)llar_wire::kEpochLast) return fail(LLAR_ERR_ARG);
    h->host_epoch = (uint32_t)value;
    return LLAR_OK;
  }
  if (value <= 0x80000000ll || value > 0xFFFFFFFFll) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  const uint32_t e = (uint32_t)value;
  if (hipMemcpy(&h->ctrl->epoch, &e, sizeof(e), hipMemcpyHostToDevice) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (hipMemset(h->ctrl->read_epoch, 0, sizeof(h->ctrl->read_epoch)) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  return LLAR_OK;
}

int llar_set_option(llar_comm* h, const char* key, long long value) {
  if (!key) return fail(LLAR_ERR_ARG);
  if (!h) {
    // the process-wide defaults of communicators created from now on
    std::lock_guard<std::mutex> lock(g_defaults_mu);
    llar_comm& d = defaults_locked();
    long long* slot = option_slot(&d, key);
    if (!slot || !option_value_ok(key, value, 0)) return fail(LLAR_ERR_ARG);
    *slot = value;
    return LLAR_OK;
  }
  if (strcmp(key, "debug_host_epoch") == 0) return set_debug_epoch(h, false, value);
  if (strcmp(key, "debug_device_epoch") == 0) return set_debug_epoch(h, true, value);
  long long* slot = option_slot(h, key);
  if (!slot) return fail(LLAR_ERR_ARG);
  if (!option_value_ok(key, value, h->n_ranks)) return fail(LLAR_ERR_ARG);
  if (strcmp(key, "placement") == 0 && value == 2 && !h->local_ok) return fail(LLAR_ERR_UNSUPPORTED);
  if (strcmp(key, "timing") == 0 && value == 1 && h->timing == 0) {
    // start from an empty timing ring (the epoch and status words are kept)
    if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
    if (hipMemset(h->ctrl->timing_grid, 0, sizeof(uint32_t) * kTimingRing) != hipSuccess) return fail(LLAR_ERR_HIP);
  }
  *slot = value;
  return LLAR_OK;
}

int llar_get_option(llar_comm* h, const char* key, long long* value) {
  if (!key || !value) return fail(LLAR_ERR_ARG);
  if (!h) {
    std::lock_guard<std::mutex> lock(g_defaults_mu);
    long long* slot = option_slot(&defaults_locked(), key);
    if (!slot) return fail(LLAR_ERR_ARG);
    *value = *slot;
    return LLAR_OK;
  }
  if (strcmp(key, "local_placement_ok") == 0) {
    *value = h->local_ok ? 1 : 0;
    return LLAR_OK;
  }
  if (strcmp(key, "debug_host_epoch") == 0) {
    *value = (long long)h->host_epoch;
    return LLAR_OK;
  }
  if (strcmp(key, "debug_device_epoch") == 0) {
    uint32_t e = 0;
    if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
    if (hipMemcpy(&e, &h->ctrl->epoch, sizeof(e), hipMemcpyDeviceToHost) != hipSuccess) return fail(LLAR_ERR_HIP);
    *value = (long long)e;
    return LLAR_OK;
  }
  long long* slot = option_slot(h, key);
  if (!slot) return fail(LLAR_ERR_ARG);
  *value = *slot;
  return LLAR_OK;
}

size_t llar_staging_bytes(llar_comm* h, llar_protocol protocol) {
  if (!h) return 0;
  const Region* r = region_of(h, (int)protocol);
  return r ? r->bytes : 0;
}

int llar_debug_copy_staging(llar_comm* h, llar_protocol protocol, void* host_dst, size_t bytes) {
  if (!h || !host_dst) return fail(LLAR_ERR_ARG);
  const Region* r = region_of(h, (int)protocol);
  if (!r || !r->ptr || bytes > r->bytes) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  if (hipMemcpy(host_dst, r->ptr, bytes, hipMemcpyDeviceToHost) != hipSuccess) return fail(LLAR_ERR_HIP);
  return LLAR_OK;
}

int llar_get_epoch(llar_comm* h, uint32_t* epoch) {
  if (!h || !epoch) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  if (!h->last_call_device) {
    *epoch = h->host_epoch;
    return LLAR_OK;
  }
  if (hipMemcpy(epoch, &h->ctrl->epoch, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return fail(LLAR_ERR_HIP);
  return LLAR_OK;
}

int llar_get_timing(llar_comm* h, uint64_t* host_dst, int count) {
  if (!h || !host_dst || count < 0) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  Ctrl c;
  if (hipMemcpy(&c, h->ctrl, sizeof(Ctrl), hipMemcpyDeviceToHost) != hipSuccess) return fail(LLAR_ERR_HIP);
  std::vector<uint64_t> wg;
  // the call's span: first start and last end over its workgroups
  auto span = [&](uint32_t slot, uint64_t& t0, uint64_t& t1) -> bool {
    t0 = ~0ull;
    t1 = 0ull;
    const uint32_t g = c.timing_grid[slot];
    if (g == 0u || g > (uint32_t)kTimingMaxWgs) return true;
    wg.resize(2 * (size_t)g);
    if (hipMemcpy(wg.data(), h->timing_wg + (size_t)slot * kTimingMaxWgs * 2, wg.size() * sizeof(uint64_t),
                  hipMemcpyDeviceToHost) != hipSuccess)
      return false;
    for (uint32_t b = 0; b < g; ++b) {
      t0 = std::min(t0, wg[2 * b]);
      t1 = std::max(t1, wg[2 * b + 1]);
    }
    return true;
  };
  int n = std::min(count, kTimingRing - 1);
  // the next call's slot has not run yet; the last n epochs precede it
  const bool dev = h->last_call_device;
  uint32_t e = dev ? c.epoch : h->host_epoch;
  int written = 0;
  for (int i = n; i >= 1; --i) {
    uint32_t ep = e & 0x7FFFFFFFu;
    for (int k = 0; k < i; ++k) ep = (ep == 1u) ? 0x7FFFFFFFu : ep - 1u;
    if (dev) ep |= 0x80000000u;
    if (!span(ep % kTimingRing, host_dst[2 * written], host_dst[2 * written + 1])) return fail(LLAR_ERR_HIP);
    ++written;
  }
  return written;
}

int llar_get_trace(llar_comm* h, uint64_t* host_dst, int max_records) {
  if (!h || !host_dst || max_records < 0) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  int n = std::min(max_records, h->trace_grid);
  if (n > 0 && hipMemcpy(host_dst, h->trace, (size_t)n * kTraceWords * sizeof(uint64_t), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(LLAR_ERR_HIP);
  return n;
}

int llar_get_pipeline_trace(llar_comm* h, uint64_t* host_dst, int max_records) {
  if (!h || !host_dst || max_records < 0) return fail(LLAR_ERR_ARG);
  if (hipDeviceSynchronize() != hipSuccess) return fail(LLAR_ERR_HIP);
  int n = std::min(max_records, h->pipe_trace_grid);
  if (n > 0 && hipMemcpy(host_dst, h->pipe_trace, (size_t)n * kPipeTraceWords * sizeof(uint64_t),
                         hipMemcpyDeviceToHost) != hipSuccess)
    return fail(LLAR_ERR_HIP);
  return n;
}

double llar_wallclock_hz(void) {
  int dev = 0, wc = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0.0;
  if (hipDeviceGetAttribute(&wc, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0.0;
  return wc * 1000.0;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// llar_allreduce_noalloc: the LL one-shot AllReduce for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its staging and control block live in
// one static device array per GPU instead of a communicator's allocations.
// ---------------------------------------------------------------------------
namespace {

// largest message per rank: the AUTO table's LL range
constexpr size_t kNoAllocMaxBytes = 64u << 10;
constexpr int kNoAllocMaxRanks = 8;
constexpr size_t kNoAllocCtrlBytes = (sizeof(Ctrl) + 255u) / 256u * 256u;
// LL region laid out for the largest rank count: [parity 2][sender 1..7][vector][2 lines]
constexpr size_t kNoAllocRankStride = (kNoAllocMaxBytes / 16u + (size_t)kNoAllocMaxRanks) * 32u;
constexpr size_t kNoAllocParityStride = kNoAllocRankStride * (size_t)(kNoAllocMaxRanks - 1);
constexpr size_t kNoAllocLLBytes = 2u * kNoAllocParityStride;
constexpr size_t kNoAllocScratchBytes = 2u << 20;
static_assert(kNoAllocCtrlBytes + kNoAllocLLBytes <= kNoAllocScratchBytes, "no-alloc layout exceeds the scratch array");
constexpr int kNoAllocMaxDevices = 64;

struct NoAllocDevice {
  bool ready = false;
  uint8_t* ptr = nullptr;  // device address of this GPU's copy of `scratch`
  llar_comm comm;          // its regions point into that copy
};
NoAllocDevice g_noalloc[kNoAllocMaxDevices];
std::mutex g_noalloc_mu;

}  // namespace

// Each GPU the library runs on holds one copy of this array until the
// process ends: the control block (epochs, status, per-workgroup epoch
// words) followed by the LL staging.  Host code never names it except to
// look up its device address.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

// Once per device, with that device current and outside stream capture:
// find this GPU's copy of the array, check the placement of workgroups on
// XCDs (the probe writes into the staging, which is then zeroed), and write
// a fresh control block.  No allocation.
int noalloc_setup(NoAllocDevice& d, int dev, hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) return LLAR_ERR_HIP;
  if (cap != hipStreamCaptureStatusNone) return LLAR_ERR_UNSUPPORTED;  // set-up makes synchronous copies
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LLAR_ERR_HIP;
  uint8_t* const base = static_cast<uint8_t*>(p);
  llar_comm& c = d.comm;
  c.device = dev;
  int cus = 0, wc = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return LLAR_ERR_HIP;
  if (hipDeviceGetAttribute(&wc, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return LLAR_ERR_HIP;
  c.cu_count = cus;
  c.wall_hz = wc > 0 ? wc * 1000.0 : 100e6;
  c.max_bytes = kNoAllocMaxBytes;
  c.ctrl = reinterpret_cast<Ctrl*>(base);
  c.ll.ptr = base + kNoAllocCtrlBytes;
  c.ll.bytes = kNoAllocLLBytes;
  c.ll.rank_stride = kNoAllocRankStride;
  c.ll.parity_stride = kNoAllocParityStride;
  // the other protocols' regions, the timing ring, traces and progress
  // words stay absent: this entry point runs the LL exchange only
  const int G = 64;
  uint32_t hx[G];
  uint32_t* probe = reinterpret_cast<uint32_t*>(c.ll.ptr);
  if (launch_xcc_probe(probe, G, 0) != hipSuccess) return LLAR_ERR_HIP;
  if (hipMemcpy(hx, probe, sizeof(hx), hipMemcpyDeviceToHost) != hipSuccess) return LLAR_ERR_HIP;
  bool ok = true;
  uint32_t seen = 0;
  for (int i = 0; i < 8; ++i) seen |= 1u << (hx[i] & 31u);
  ok &= (seen == 0xFFu);
  for (int i = 8; i < G; ++i) ok &= (hx[i] == hx[i % 8]);
  c.local_ok = ok;
  {
    // of the process defaults only these apply here: the other options
    // name regions and modes this entry point does not have
    std::lock_guard<std::mutex> lock(g_defaults_mu);
    c.spin_timeout_us = defaults_locked().spin_timeout_us;
    c.log = defaults_locked().log;
  }
  if (hipMemset(c.ll.ptr, 0, c.ll.bytes) != hipSuccess) return LLAR_ERR_HIP;
  if (init_ctrl(&c) != hipSuccess) return LLAR_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return LLAR_ERR_HIP;
  d.ptr = base;
  d.ready = true;
  return LLAR_OK;
}

}  // namespace

extern "C" int llar_allreduce_noalloc(int n_ranks, const void* const* partials, void* out, size_t n_elems,
                                      llar_dtype dtype, void* stream) {
  if (n_ranks < 1 || !partials || (int)dtype < 0 || (int)dtype > 2) return fail(LLAR_ERR_ARG);
  if (n_ranks > kNoAllocMaxRanks) return fail(LLAR_ERR_UNSUPPORTED);
  if (n_elems == 0) return LLAR_OK;
  const size_t elem = (size_t)elem_bytes_of(dtype);
  if (n_elems > kNoAllocMaxBytes / elem) return fail(LLAR_ERR_UNSUPPORTED);
  if (!out || !aligned16(out)) return fail(LLAR_ERR_ARG);
  for (int r = 0; r < n_ranks; ++r)
    if (!partials[r] || !aligned16(partials[r])) return fail(LLAR_ERR_ARG);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LLAR_ERR_HIP);
  if (dev < 0 || dev >= kNoAllocMaxDevices) return fail(LLAR_ERR_UNSUPPORTED);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoAllocDevice& d = g_noalloc[dev];
  if (!d.ready) {
    const int s = noalloc_setup(d, dev, st);
    if (s != LLAR_OK) return fail(s);
  }
  llar_comm* h = &d.comm;
  h->n_ranks = n_ranks;
  h->kind = (int)dtype;
  h->elem = elem;
  Geometry g;
  const int s = plan(h, n_elems, LLAR_LL, g);
  if (s != LLAR_OK) return fail(s);
  return issue(h, partials, n_ranks, out, n_elems, LLAR_LL, g, st);
}
