// llar_device.h -- device-side building blocks of the emulated-rank AllReduce
// protocols on gfx950 (MI355X): coherent 16-byte accesses, the ordering
// primitive, element conversions and rounding, bounded polling.
//
// Memory-ordering scheme (gfx950, one agent, 8 XCDs, one L2 per XCD):
//   * Every access that crosses workgroups goes through device-coherent
//     instructions: buffer loads/stores carrying the sc1 cache-policy bit
//     (what the compiler emits for agent-scope relaxed atomic loads and
//     stores) or agent-scope float/int atomics (which the compiler emits
//     without cache bits).  No staging word is ever read by a plain load.
//   * "Release" is s_waitcnt vmcnt(0): every earlier store/atomic of the wave
//     has been acknowledged at its coherence point before the next one
//     issues.  The agent-scope fences (buffer_wbl2 / buffer_inv) are never
//     used: they walk the whole L2 and cost microseconds.
//   * "Acquire" is the sc1 load itself: loads issued after a flag was seen
//     are coherent and issued later, so they observe what was performed
//     before the flag.
//   * In the XCD-local placement all workgroups that touch a staging range
//     run on one XCD and share its L2, so payload stores there may be plain
//     (write-back) stores; sc1 loads are then served by that L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "llar_wire.h"

namespace llar {

// The staging primitives are those of the public device-side header: the
// kernels below are written with the same building blocks that custom
// kernels use.
using llar_wire::s16x2;
using llar_wire::u32x2;
using llar_wire::u32x4;
using llar_wire::kCpolNone;
using llar_wire::kCpolNt;
using llar_wire::kCpolSc0;
using llar_wire::kCpolSc1;
using llar_wire::ld16_coh;
using llar_wire::ld4_coh;
using llar_wire::ld8_coh;
using llar_wire::make_rsrc;
using llar_wire::sentinel_is_empty;
using llar_wire::st16_coh;
using llar_wire::st16_l2;
using llar_wire::wall_ticks;
template <int kSleep>
using SpinT = llar_wire::PollT<kSleep>;
using Spin = llar_wire::Poll;          // latency-critical polls
using SpinBulk = llar_wire::PollBulk;  // polls of the bandwidth pipeline

// Placement-scoped staging stores: plain stores when every reader shares the
// writer's XCD (local placement), device-coherent ones otherwise.
constexpr llar_wire::Scope scope_of(bool local) { return local ? llar_wire::kXcd : llar_wire::kDevice; }
template <bool kLocal>
__device__ __forceinline__ void st16_stage(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  llar_wire::store16<scope_of(kLocal)>(r, off, v);
}
template <bool kLocal>
__device__ __forceinline__ void st8_stage(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  llar_wire::store8<scope_of(kLocal)>(r, off, v);
}
// Reset of a consumed Sentinel slot in a pipeline that does not read the
// slot again before its producer's next store: under the local placement a
// non-temporal store (sc0 | nt), so that L2 evicts emptied slots before
// staged data (measured on the 64 MiB x 8 reduce: 794 -> 646 MiB written per
// launch, 3 % faster); device-coherent otherwise.
template <bool kLocal>
__device__ __forceinline__ void st16_reset(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 empty = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  if constexpr (kLocal) __builtin_amdgcn_raw_buffer_store_b128(empty, r, off, 0, kCpolSc0 | kCpolNt);
  else st16_stage<false>(r, off, empty);
}
__device__ __forceinline__ void drain_vm() { llar_wire::release(); }

// ---- clocks and ids -------------------------------------------------------------
__device__ __forceinline__ uint32_t xcc_id() {
  // HW register XCC_ID (20), bits 3:0
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;
}

// ---- element decode (exact) ----------------------------------------------------------
__device__ __forceinline__ double dec_f32(uint32_t b) { return (double)__uint_as_float(b); }
__device__ __forceinline__ double dec_bf16(uint32_t h) { return (double)__uint_as_float(h << 16); }
__device__ __forceinline__ double dec_f16(uint32_t h) {
  _Float16 x = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (double)(float)x;
}

// ---- rounding binary64 -> output type ------------------------------------------------
// binary32: the hardware conversion (round to nearest even in the default mode).
__device__ __forceinline__ uint32_t rne_f32(double d) { return __float_as_uint((float)d); }

// binary64 -> binary32 rounded to odd (Boldo & Melquiond): truncate toward zero,
// then force the last bit to 1 when the conversion was inexact.  Rounding that
// value to nearest-even in a format of at most 22 significand bits gives the
// correctly rounded result, because binary32 keeps >= 2 extra bits.
__device__ __forceinline__ float round_odd_f32(double d) {
  float f = (float)d;
  double back = (double)f;
  if (back != d && d == d) {
    uint32_t u = __float_as_uint(f);
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;  // one step toward zero
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f;
}
// binary32 -> bfloat16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t rne_bf16(double d) { return f32_to_bf16_rne(round_odd_f32(d)); }
__device__ __forceinline__ uint32_t rne_f16(double d) {
  _Float16 h = (_Float16)round_odd_f32(d);  // v_cvt_f16_f32: nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// ---- per-type traits ------------------------------------------------------------------
// kind: 0 = binary32, 1 = binary16, 2 = bfloat16 (the ABI's llar_dtype values)
template <int kKind> struct Elem;
template <> struct Elem<0> {
  static constexpr int kBytes = 4, kPerVec = 4;
  static constexpr uint32_t kSentinelWord = 0xFFFFFFFFu;
  __device__ static double dec(uint32_t b) { return dec_f32(b); }
  __device__ static uint32_t enc(double d) { return rne_f32(d); }
  __device__ static float to_f32(uint32_t b) { return __uint_as_float(b); }
  __device__ static uint32_t from_f32(float f) { return __float_as_uint(f); }
};
template <> struct Elem<1> {
  static constexpr int kBytes = 2, kPerVec = 8;
  __device__ static double dec(uint32_t b) { return dec_f16(b); }
  __device__ static uint32_t enc(double d) { return rne_f16(d); }
  __device__ static float to_f32(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }
  __device__ static uint32_t from_f32(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f); }
};
template <> struct Elem<2> {
  static constexpr int kBytes = 2, kPerVec = 8;
  __device__ static double dec(uint32_t b) { return dec_bf16(b); }
  __device__ static uint32_t enc(double d) { return rne_bf16(d); }
  __device__ static float to_f32(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static uint32_t from_f32(float f) { return f32_to_bf16_rne(f); }
};

// Element k (0-based) of a 16-byte vector, as raw bits.
template <int kKind>
__device__ __forceinline__ uint32_t vec_elem(const u32x4& v, int k) {
  if constexpr (Elem<kKind>::kBytes == 4) return v[k];
  else return (v[k >> 1] >> ((k & 1) * 16)) & 0xFFFFu;
}
template <int kKind>
__device__ __forceinline__ void vec_set(u32x4& v, int k, uint32_t bits) {
  if constexpr (Elem<kKind>::kBytes == 4) v[k] = bits;
  else {
    uint32_t sh = (k & 1) * 16;
    v[k >> 1] = (v[k >> 1] & ~(0xFFFFu << sh)) | ((bits & 0xFFFFu) << sh);
  }
}

// Sentinel helpers keyed by element kind (the wire's own are keyed by width).
template <int kKind>
__device__ __forceinline__ u32x4 sentinel_canon(u32x4 v) {
  return llar_wire::sentinel_canon<Elem<kKind>::kBytes>(v);
}
template <int kKind>
__device__ __forceinline__ bool sentinel_ready8(const u32x2& v) {
  return llar_wire::sentinel_ready8<Elem<kKind>::kBytes>(v);
}
template <int kKind>
__device__ __forceinline__ bool sentinel_ready(const u32x4& v) {
  return llar_wire::sentinel_ready<Elem<kKind>::kBytes>(v);
}

// ---- device control block --------------------------------------------------------------
constexpr int kTimingRing = 64;
constexpr int kTimingMaxWgs = 4096;  // largest grid that timing mode records
constexpr uint32_t kStatusTimeout = 1u;
constexpr uint32_t kStatusPlacement = 2u;

// Kernel arguments live in memory; the scalar loads that fetch them miss a
// cold scalar cache at launch.  Loads that the compiler sinks into later
// branches, or chains behind one another, each cost a memory round trip on
// the critical path.  Naming the uniform values a kernel needs in one empty
// asm statement at entry makes them live there, so their loads are issued
// together and waited for once.
#define LLAR_UNIFORM_AT_ENTRY(...) asm volatile("" ::__VA_ARGS__)

struct Ctrl {
  uint32_t epoch;      // current call's epoch, 1..2^32-1 (0 = never written)
  uint32_t pad0[31];
  uint32_t status;     // sticky error bits
  uint32_t pad2[31];
  uint32_t bar_count;  // grid barrier of the barrier-based ablation kernel: arrivals of this call
  uint32_t pad3[31];
  uint32_t bar_gen;    // ... and its generation, advanced by the last arrival
  uint32_t pad4[31];
  uint32_t timing_grid[kTimingRing];  // per epoch slot: workgroups that recorded a span
  uint64_t* timing_wg;  // [kTimingRing][kTimingMaxWgs][2]: each workgroup's start, end (wall ticks)
  // state that carries epoch values, cleared when the device epoch wraps:
  // the LL region (lines {d0, e, d1, e}) and the owner-credit progress words
  uint8_t* ll_base;
  uint64_t ll_bytes;
  uint8_t* credit_base;
  uint64_t credit_bytes;
  uint32_t read_epoch[kTimingMaxWgs];  // device-numbered calls: the epoch workgroup b has read
};

// Epochs: host-numbered calls use 1 .. 2^31-1, device-numbered (graph
// capture) calls use 2^31 + (1 .. 2^31-1); 0 never occurs.  Both sequences
// wrap: the state that holds epoch values is cleared before the first call
// after a wrap (host: stream-ordered fills before that call; device: by the
// wrapping call itself, in wg_end).
__host__ __device__ __forceinline__ uint32_t next_host_epoch(uint32_t e) { return llar_wire::next_epoch(e); }
__host__ __device__ __forceinline__ uint32_t next_device_epoch(uint32_t e) {
  return 0x80000000u | llar_wire::next_epoch(e & llar_wire::kEpochLast);
}
// per-workgroup word written by every workgroup of a device-numbered call
// that wraps the epoch once its staging accesses are done (never an epoch)
constexpr uint32_t kWrapDone = 1u;

__device__ __forceinline__ void raise_status(Ctrl* c, uint32_t bits) {
  __hip_atomic_fetch_or(&c->status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// shared prologue / epilogue: the call's epoch
// ---------------------------------------------------------------------------
// Two epoch sources.  In ordinary stream-ordered use the host numbers the
// calls and passes the epoch in the kernel arguments (host_epoch, bit 31
// clear): nothing to read on the device.  Under graph capture the arguments
// would repeat on every replay, so the kernel reads the device-resident epoch
// (bit 31 set; the two ranges never meet): thread 0 reads it, publishes it
// through LDS and records it in its workgroup's own word of read_epoch.  The
// grid's last workgroup, when it finishes, waits until every word holds this
// epoch -- every workgroup of the call has read it -- and advances it; the
// next call starts after this one.  (One shared arrival counter instead
// serialised an atomic per workgroup on a single address: about 6 us per
// call for a 512-workgroup grid.)
// Timing mode has each workgroup store its own start and end stamps in the
// epoch's ring slot (plain stores, no shared counter); workgroup 0 also
// records the grid so that the reader knows how many entries belong to it.
struct WgState {
  uint32_t epoch;
  bool counted;  // the epoch came from the device (recorded in read_epoch)
  uint64_t t0;
};

__device__ __forceinline__ WgState wg_begin(Ctrl* ctrl, uint32_t host_epoch, bool timing, bool idle) {
  __shared__ uint32_t s_epoch;
  WgState st{host_epoch, false, 0ull};
  if (timing && threadIdx.x == 0) st.t0 = wall_ticks();
  if (host_epoch != 0u) return st;
  if (threadIdx.x == 0) {
    const uint32_t e = __hip_atomic_load(&ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_epoch = e;
    __hip_atomic_store(&ctrl->read_epoch[blockIdx.x], e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  st.epoch = s_epoch;
  st.counted = true;
  return st;
}

// Wait (one wave) until words[0 .. grid) all equal `want`, reading them with
// 16-byte loads, four per lane in flight (a pass costs one memory round trip
// per 1024 workgroups); false when the wall-clock bound expires (every
// workgroup is resident, so the wait ends; the bound is a safeguard).
__device__ __forceinline__ bool wait_words(uint32_t* words, uint32_t grid, uint32_t want) {
  const uint32_t lane = threadIdx.x & 63u;
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(words, grid * 4u);
  llar_wire::Poll poll(100000000ull);  // 1 s
  while (true) {
    bool all = true;
    for (uint32_t w0 = 0; w0 < grid; w0 += 1024u) {
      u32x4 v[4];
#pragma unroll
      for (uint32_t k = 0; k < 4u; ++k) v[k] = ld16_coh(rr, (w0 + (k * 64u + lane) * 4u) * 4u);
#pragma unroll
      for (uint32_t k = 0; k < 4u; ++k)
#pragma unroll
        for (uint32_t t = 0; t < 4u; ++t) all &= (w0 + (k * 64u + lane) * 4u + t >= grid) | (v[k][t] == want);
    }
    if (__all((int)all)) return true;
    if (poll.expired()) return false;
  }
}

// Zero `bytes` (a multiple of 16) at `base` with device-coherent stores,
// every thread of the workgroup taking 16-byte pieces.
__device__ __forceinline__ void clear_region(uint8_t* base, uint64_t bytes) {
  if (base == nullptr || bytes == 0u) return;
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (uint32_t)bytes);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (uint64_t off = (uint64_t)threadIdx.x * 16u; off < bytes; off += (uint64_t)blockDim.x * 16u)
    st16_coh(r, (uint32_t)off, zero);
}

// The last call of the device epoch range (2^32 - 1): the next epoch,
// 2^31 + 1, was used 2^31 - 1 calls ago, and an LL line or progress word
// that no call has written since would pass for a fresh one.  Every
// workgroup of this call, once its own staging accesses are done, records
// kWrapDone; the grid's last workgroup waits for all of them -- nothing of
// this call touches staging any more -- zeroes the LL region, the
// progress words and the per-workgroup epoch words, and only then
// advances the epoch.  (A once-per-cycle clear of a few hundred MiB at most;
// the next call is ordered after this one on the stream.)
__device__ __forceinline__ void wrap_end(Ctrl* ctrl, const WgState& st, uint32_t grid) {
  if (threadIdx.x == 0)
    __hip_atomic_store(&ctrl->read_epoch[blockIdx.x], kWrapDone, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x != grid - 1u) return;
  if (threadIdx.x < 64u) {
    // (an expired wait leaves the status set; the call's output is then
    // undefined anyway, and the epoch still advances)
    const bool ok = wait_words(ctrl->read_epoch, grid, kWrapDone);
    if (threadIdx.x == 0 && !ok) raise_status(ctrl, kStatusTimeout);
  }
  __syncthreads();
  clear_region(ctrl->ll_base, ctrl->ll_bytes);
  clear_region(ctrl->credit_base, ctrl->credit_bytes);
  clear_region(reinterpret_cast<uint8_t*>(ctrl->read_epoch), sizeof(ctrl->read_epoch));
  drain_vm();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&ctrl->epoch, next_device_epoch(st.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wg_end(Ctrl* ctrl, const WgState& st, uint32_t host_epoch, uint32_t grid, bool timing,
                                       bool idle) {
  const bool wrap = st.counted && llar_wire::epoch_wraps(st.epoch);
  if (timing || wrap) {
    drain_vm();
    __syncthreads();
  }
  if (wrap) {
    wrap_end(ctrl, st, grid);
  } else if (st.counted && blockIdx.x == grid - 1u && threadIdx.x < 64u) {
    // every workgroup of the grid has read this call's epoch before it
    // advances
    if (!wait_words(ctrl->read_epoch, grid, st.epoch)) raise_status(ctrl, kStatusTimeout);
    if (threadIdx.x == 0)
      __hip_atomic_store(&ctrl->epoch, next_device_epoch(st.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x != 0) return;
  if (timing) {
    const uint64_t t1 = wall_ticks();
    const uint32_t slot = st.epoch % kTimingRing;
    uint64_t* p = ctrl->timing_wg + ((size_t)slot * kTimingMaxWgs + blockIdx.x) * 2u;
    p[0] = idle ? ~0ull : st.t0;
    p[1] = idle ? 0ull : t1;
    if (blockIdx.x == 0) ctrl->timing_grid[slot] = grid;
  }
}

// Role of workgroup b under a placement known at compile time (no kernel
// argument is needed to find it).
template <bool kLocal, int N>
__device__ __forceinline__ void decode_role_t(uint32_t b, int& r, uint32_t& w) {
  if constexpr (kLocal) {
    const uint32_t x = b & 7u, q = b >> 3;
    r = (int)(q % (uint32_t)N);
    w = (q / (uint32_t)N) * 8u + x;
  } else {
    r = (int)(b % (uint32_t)N);
    w = b / (uint32_t)N;
  }
}

}  // namespace llar
