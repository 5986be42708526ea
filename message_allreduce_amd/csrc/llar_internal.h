// llar_internal.h -- kernel argument blocks and launch descriptors shared by
// the HIP kernels and the host library (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llar {

struct Ctrl;

// element kinds (same numbering as llar_dtype)
constexpr int kKindF32 = 0;
constexpr int kKindF16 = 1;
constexpr int kKindBF16 = 2;

// wire formats of the one-shot kernel
constexpr int kWireLL = 0;
constexpr int kWireSentinel = 1;

// placements of (rank, slice) onto workgroup ids
constexpr uint32_t kPlaceSpread = 1;
constexpr uint32_t kPlaceLocal = 2;

// kernel variants
enum KernelId : int {
  kKernOneShotLL = 0,
  kKernOneShotSentinel = 1,
  kKernLL128Acc32 = 2,
  kKernLL128Acc16 = 3,
  kKernSentinelPipe = 4,
  kKernSentinelPipeLocal = 5,
  kKernOneShotLLLocal = 6,
  kKernOneShotSentinelLocal = 7,
  kKernSentinelHs = 8,
  kKernSentinelHsLocal = 9,
  // point-to-point: one sender, one receiver (two ranks), copy instead of sum
  kKernP2PLL = 10,
  kKernP2PSentinel = 11,
  kKernP2PLLLocal = 12,
  kKernP2PSentinelLocal = 13,
  // ReduceScatter and AllGather: every rank sends and receives
  kKernRsLL = 14,
  kKernRsSentinel = 15,
  kKernAgLL = 16,
  kKernAgSentinel = 17,
  kKernRsLLLocal = 18,
  kKernRsSentinelLocal = 19,
  kKernAgLLLocal = 20,
  kKernAgSentinelLocal = 21,
  // ReduceScatter over the LL128 atomic wire (binary32 or 16-bit staging)
  kKernRsLL128Acc32 = 22,
  kKernRsLL128Acc16 = 23,
  // ablation: the one-shot reduce with a grid-wide barrier instead of flags
  kKernBarrier = 24,
  kKernBarrierLocal = 25,
  // pipelined Sentinel with the owner credit (llar_kernels.hip)
  kKernSentinelOc = 26,
  kKernSentinelOcLocal = 27,
  // pipelined LL128 with producer and consumer waves and B buffers
  kKernLL128WsAcc32 = 28,
  kKernLL128WsAcc16 = 29,
  kKernCount = 30
};
constexpr int kKernFirstMulti = kKernRsLL;
// kernels that live in llar_multi.hip
constexpr bool is_multi_kernel(int k) { return k >= kKernFirstMulti && k <= kKernBarrierLocal; }

struct OneShotArgs {
  const uint8_t* part[8];
  uint8_t* out;
  uint8_t* stage;        // base of this protocol's staging (both parities)
  Ctrl* ctrl;
  uint64_t nbytes;       // bytes per rank
  uint64_t spin_limit;   // wall-clock ticks
  uint32_t n_vec;        // 16-byte vectors per rank (last one may be partial)
  uint32_t vq, vr;       // slice w holds vq vectors, plus one more when w < vr
  uint32_t stage_bytes;  // size of the staging region (buffer descriptor bound)
  uint32_t parity_stride;
  uint32_t rank_stride;  // bytes per sending rank per parity
  uint32_t grid;
  uint32_t slices;
  uint32_t placement;
  uint32_t timing;
  uint32_t keep;
  uint32_t drop_rank;    // tests: this rank's producers write nothing (0xFFFFFFFF = none)
  uint32_t host_epoch;   // this call's epoch, or 0: read the device-resident epoch
  uint64_t* trace;       // per-workgroup phase stamps (kTraceWords each), or null
  uint32_t xcd_span;     // local placement: slices use XCDs 0 .. xcd_span-1 (8 = all)
};

struct TwoShotArgs {
  const uint8_t* part[8];
  uint8_t* out;
  uint8_t* stage;
  Ctrl* ctrl;
  uint64_t n;            // elements per rank
  uint64_t spin_limit;
  uint32_t chunk_elems;  // elements per rank per chunk
  uint32_t n_chunks;
  uint32_t stage_bytes;
  uint32_t parity_stride;
  uint32_t shard_cap;    // Sentinel: 16-byte vectors per (owner, sender) slot
  uint32_t n_buffers;    // Sentinel pipeline: staging buffers
  uint32_t cons_waves;   // Sentinel slot handshake: consumer waves per workgroup
  uint32_t cons_groups;  // Sentinel pipeline, workgroup credit: consumer groups (chunks dealt round-robin)
  uint32_t prod_groups;  // Sentinel pipeline, workgroup credit: producer groups (chunks dealt round-robin)
  uint32_t grid;
  uint32_t slices;
  uint32_t placement;
  uint32_t timing;
  uint32_t keep;
  uint32_t drop_rank;
  uint32_t host_epoch;
  uint64_t* trace;       // per-workgroup, per-chunk stamps (kPipeTraceWords each), or null
  uint32_t* credit;      // Sentinel pipeline, owner credit: [rank][slice][consumer wave] {count, epoch}, or null
  uint32_t threads;      // workgroup size, read with the other arguments (blockDim.x would be
                         // one more dependent scalar load, from the kernarg line after them)
  uint32_t slices_rcp;   // one-round LL128: ceil(2^32 / slices) when x / slices == umulhi(x, it)
                         // for every numerator of the line partition, else 0 (divide)
};

// ReduceScatter / AllGather over the LL or Sentinel wire.  A block is what
// one sender hands one receiver: RS -- the sender's copy of the receiver's
// segment; AG -- the sender's whole fragment.  Staging per parity:
// [receiver][sender slot 0..N-2][block], sender k at slot k of receiver j
// when k < j, slot k-1 when k > j.
struct MultiArgs {
  const uint8_t* in[8];   // RS: N blocks per rank; AG: one fragment per rank
  uint8_t* out[8];        // RS: one segment per rank; AG: N fragments per receiving rank
  uint8_t* stage;
  Ctrl* ctrl;
  uint64_t blk;           // bytes per block
  uint64_t spin_limit;
  uint32_t vq, vr;        // slice w holds vq 16-byte vectors of a block, plus one when w < vr
  uint32_t stage_bytes;
  uint32_t parity_stride;
  uint32_t slot_stride;   // staging bytes per (receiver, sender) slot
  uint32_t n_recv;        // receiving ranks 0..n_recv-1: N, or 1 for an AllGather seen by rank 0
  uint32_t aligned;       // blk is a multiple of 16 bytes: whole-vector accesses
  uint32_t grid;
  uint32_t slices;
  uint32_t timing;
  uint32_t keep;
  uint32_t drop_rank;
  uint32_t host_epoch;
};

// per-chunk trace of the pipelined Sentinel: per workgroup 4 x kPipeTraceChunks
// stamps (producer credit granted, producer stores issued, consumer slots
// ready, consumer done) of the first kPipeTraceChunks chunks
constexpr int kPipeTraceChunks = 128;
constexpr int kPipeTraceWords = 4 * kPipeTraceChunks;
// owner credit of the pipelined Sentinel: one progress entry per (rank,
// slice, consumer wave), two 32-bit words: chunks finished, and the epoch of
// the call that wrote them
constexpr int kCreditSlices = 64, kCreditWaves = 8;
constexpr size_t kCreditEntries = (size_t)8 * kCreditSlices * kCreditWaves;
constexpr size_t kCreditBytes = kCreditEntries * 2 * sizeof(uint32_t);

// phase trace of the one-shot kernel: per workgroup, thread 0 records
constexpr int kTraceWords = 8;  // start, epoch, input, ready, out-acked, end, id, spare

struct LaunchSpec {
  int kind;
  int n_ranks;
  int kernel;
  int grid;
  int threads;
  int oneshot_split;  // local one-shot: consumer workgroups per slice (1 or 2)
  OneShotArgs oneshot;
  TwoShotArgs twoshot;
  MultiArgs multi;
};

hipError_t launch(const LaunchSpec& ls, hipStream_t stream);
int occupancy(int kind, int n_ranks, int kernel, int threads);
// the ReduceScatter / AllGather kernels (kernel ids from kKernFirstMulti)
hipError_t launch_multi(const LaunchSpec& ls, hipStream_t stream);
int occupancy_multi(int kind, int n_ranks, int kernel, int threads);
hipError_t launch_xcc_probe(uint32_t* out, int grid, hipStream_t stream);

}  // namespace llar
