/*
 * llar_wire.h -- device-side primitives of the LL, Sentinel and LL128 wires,
 * for HIP kernels on gfx950 (MI355X) that move or reduce data between
 * workgroups without a barrier: header-only, the building blocks that the
 * library's own kernels are made of.
 *
 * The packaging follows the low-level buffer API that "Every Microsecond
 * Matters" (agihunt.info summary, the paragraph on the low-level LL buffer
 * API) describes for authors of custom kernels; the wires are its LL,
 * Sentinel and two-shot LL128 paragraphs.  Typical use: a GEMM (or any
 * producer) epilogue puts its tensor-parallel partial tile straight onto a
 * wire, and the owner of the tile waits for the N contributions and reduces
 * them -- no separate AllReduce launch, no grid-wide barrier.
 *
 * Memory model (one agent, 8 XCDs, one L2 per XCD):
 *   - A wire is a device buffer addressed through a buffer descriptor
 *     (make_wire).  Offsets are bytes from its base, 32-bit, and accesses
 *     past its size are dropped by the hardware (loads read 0).
 *   - Every load of a wire is device-coherent (sc1) and re-issued on every
 *     call, so a polling loop sees other workgroups' stores.
 *   - Stores take a Scope: kXcd when every reader runs on the writer's XCD
 *     (workgroups b and b' with b == b' mod 8 share an XCD; plain stores
 *     land in that XCD's L2), kDevice otherwise (sc1 stores).
 *   - release() waits until every earlier store and atomic of the wave has
 *     been acknowledged: call it between data and a separate flag (LL128).
 *     LL and Sentinel need none: the flag travels in the data's own store.
 *   - Waits are bounded: a Poll expires after a wall-clock limit (ticks of
 *     the 100 MHz constant clock, s_memrealtime) and the wait returns false.
 *     A kernel that waits on other workgroups must have them all resident
 *     (grid within occupancy x CUs).
 *
 * Layouts (one 16-byte line or slot per 8 or 16 payload bytes):
 *   LL       line = {data0, epoch, data1, epoch}: each 8-byte half carries
 *            the flag, so either half may land first.  Empty buffer: zero
 *            bytes (epoch 0 never occurs).  No reset between uses: bump the
 *            epoch (next_epoch), and zero the buffer when it wraps.
 *   Sentinel slot = 16 payload bytes; empty = all-ones (a negative NaN in
 *            binary32, binary16 and bfloat16).  The sender replaces a datum
 *            equal to all-ones by the pattern one below (still a negative
 *            NaN); the receiver resets the slot to all-ones after reading.
 *   LL128    line = 128 bytes of the accumulation type A (binary32, or
 *            16-bit packed pairs): slot 0 counts contributions (each sender
 *            adds 1.0 after its data), slots 1..K hold data (K = 31 for
 *            binary32, 63 for 16-bit).  Empty: zero bytes.  The reader
 *            waits for the count N, reads, and zeroes the line.
 */
#ifndef LLAR_WIRE_H
#define LLAR_WIRE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llar_wire {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// gfx950 cache-policy bits of vector memory instructions
constexpr int kCpolNone = 0;
constexpr int kCpolSc0 = 1;
constexpr int kCpolNt = 2;
constexpr int kCpolSc1 = 16;

enum Scope : int { kXcd = 0, kDevice = 1 };

// ---- epochs --------------------------------------------------------------------
// LL epochs are non-zero 31-bit values, a new one for every use of a buffer:
// 1, 2, ..., 2^31 - 1, then 1 again (the library numbers its stream-ordered
// calls in this range and its device-numbered ones in 2^31 + this range, so
// the two never meet).  A wrap brings every value back: a line last written
// at epoch e and left alone for a whole cycle would pass for a fresh line
// when e comes round again, so the buffer must be zeroed before the first
// use after a wrap -- epoch_wraps(e) is true for the last epoch of the range.
constexpr uint32_t kEpochLast = 0x7FFFFFFFu;
__host__ __device__ __forceinline__ uint32_t next_epoch(uint32_t e) {
  const uint32_t n = (e + 1u) & kEpochLast;
  return n == 0u ? 1u : n;
}
__host__ __device__ __forceinline__ bool epoch_wraps(uint32_t e) { return (e & kEpochLast) == kEpochLast; }

// ---- the buffer ------------------------------------------------------------------
// Descriptor of `bytes` bytes at `base` (device memory).  The inputs are
// uniform; after divergent code the compiler can no longer prove it, keeps
// the descriptor in vector registers and turns every access into a
// readfirstlane loop that also hides the memory counters from its wait
// analysis, so uniformity is stated outright.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* const ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  // word3 0x00020000: raw (untyped) 32-bit data format for gfx9-family buffers
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)n, 0x00020000);
}
typedef __amdgpu_buffer_rsrc_t Wire;
__device__ __forceinline__ Wire make_wire(void* base, uint32_t bytes) { return make_rsrc(base, bytes); }

// ---- coherent loads and scoped stores -----------------------------------------------
// The buffer-load builtins count as reads of constant memory: inside a polling
// loop with no store the compiler could hoist them or delete a loop it cannot
// prove finite.  The empty volatile asm with a memory clobber in front of each
// forces a fresh load every time (loads issued back to back still overlap).
__device__ __forceinline__ u32x4 ld16_coh(Wire r, uint32_t off) {
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1);
}
__device__ __forceinline__ u32x2 ld8_coh(Wire r, uint32_t off) {
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolSc1);
}
__device__ __forceinline__ uint32_t ld4_coh(Wire r, uint32_t off) {
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCpolSc1);
}
__device__ __forceinline__ void st16_coh(Wire r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolSc1);
}
__device__ __forceinline__ void st16_l2(Wire r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolNone);
}
template <Scope kScope>
__device__ __forceinline__ void store16(Wire r, uint32_t off, u32x4 v) {
  if constexpr (kScope == kXcd) st16_l2(r, off, v);
  else st16_coh(r, off, v);
}
template <Scope kScope>
__device__ __forceinline__ void store8(Wire r, uint32_t off, u32x2 v) {
  if constexpr (kScope == kXcd) __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpolNone);
  else __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kCpolSc1);
}

// Wait until every vector memory operation of this wave has completed (the
// "release" between data and a separate flag); the signal fences keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void release() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt/lgkmcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- bounded polling ------------------------------------------------------------------
// expired() is called after every failed poll: it backs off kSleep x 64
// cycles (s_sleep) so that waiting waves do not flood the L2 with re-polls
// that the senders' traffic queues behind, and every 16th call checks the
// wall-clock limit.
__device__ __forceinline__ uint64_t wall_ticks() { return (uint64_t)wall_clock64(); }
template <int kSleep>
struct PollT {
  uint64_t t0, limit;
  uint32_t n;
  __device__ __forceinline__ explicit PollT(uint64_t limit_ticks) : t0(wall_ticks()), limit(limit_ticks), n(0) {}
  __device__ __forceinline__ bool expired() {
    if constexpr (kSleep > 0) __builtin_amdgcn_s_sleep(kSleep);
    if ((++n & 15u) != 0u) return false;
    return wall_ticks() - t0 > limit;
  }
};
using Poll = PollT<1>;       // latency-critical waits (about 27 ns back-off)
using PollBulk = PollT<8>;   // waits inside a bandwidth pipeline (about 210 ns)

// ---- LL ----------------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ll_line(u32x2 data, uint32_t epoch) { return u32x4{data[0], epoch, data[1], epoch}; }
__device__ __forceinline__ bool ll_ready(const u32x4& line, uint32_t epoch) {
  return (line[1] == epoch) & (line[3] == epoch);
}
__device__ __forceinline__ u32x2 ll_payload(const u32x4& line) { return u32x2{line[0], line[2]}; }
// 8 payload bytes as one 16-byte line at `off`
template <Scope kScope>
__device__ __forceinline__ void ll_put(Wire w, uint32_t off, u32x2 data, uint32_t epoch) {
  store16<kScope>(w, off, ll_line(data, epoch));
}
// 16 payload bytes as the two lines at off and off + 16
template <Scope kScope>
__device__ __forceinline__ void ll_put16(Wire w, uint32_t off, u32x4 data, uint32_t epoch) {
  store16<kScope>(w, off, u32x4{data[0], epoch, data[1], epoch});
  store16<kScope>(w, off + 16u, u32x4{data[2], epoch, data[3], epoch});
}
// one poll of the line at `off`: true (and the payload) once it carries `epoch`
__device__ __forceinline__ bool ll_try(Wire w, uint32_t off, uint32_t epoch, u32x2& data) {
  const u32x4 line = ld16_coh(w, off);
  data = ll_payload(line);
  return ll_ready(line, epoch);
}
// poll until the line carries `epoch`; false when the Poll expires first
template <int kSleep>
__device__ __forceinline__ bool ll_wait(Wire w, uint32_t off, uint32_t epoch, PollT<kSleep>& poll, u32x2& data) {
  while (!ll_try(w, off, epoch, data))
    if (poll.expired()) return false;
  return true;
}

// ---- Sentinel -------------------------------------------------------------------------------
// kElemBytes: 4 (binary32) or 2 (binary16, bfloat16)
template <int kElemBytes>
__device__ __forceinline__ u32x4 sentinel_canon(u32x4 v) {
  static_assert(kElemBytes == 2 || kElemBytes == 4, "element width");
  if constexpr (kElemBytes == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (v[i] == 0xFFFFFFFFu) ? 0xFFFFFFFEu : v[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x = v[i];
      if ((x & 0xFFFFu) == 0xFFFFu) x -= 1u;
      if ((x >> 16) == 0xFFFFu) x -= 0x10000u;
      v[i] = x;
    }
  }
  return v;
}
// true when no element of the 8-byte unit still holds the sentinel
template <int kElemBytes>
__device__ __forceinline__ bool sentinel_ready8(const u32x2& v) {
  if constexpr (kElemBytes == 4) {
    return (v[0] != 0xFFFFFFFFu) & (v[1] != 0xFFFFFFFFu);
  } else {
    return ((v[0] & 0xFFFFu) != 0xFFFFu) & ((v[0] >> 16) != 0xFFFFu) & ((v[1] & 0xFFFFu) != 0xFFFFu) &
           ((v[1] >> 16) != 0xFFFFu);
  }
}
// true when no element of the 16-byte slot still holds the sentinel
template <int kElemBytes>
__device__ __forceinline__ bool sentinel_ready(const u32x4& v) {
  if constexpr (kElemBytes == 4) {
    return (v[0] != 0xFFFFFFFFu) & (v[1] != 0xFFFFFFFFu) & (v[2] != 0xFFFFFFFFu) & (v[3] != 0xFFFFFFFFu);
  } else {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 4; ++i) ok &= ((v[i] & 0xFFFFu) != 0xFFFFu) & ((v[i] >> 16) != 0xFFFFu);
    return ok;
  }
}
// true when the whole slot holds the sentinel (a reset has fully landed; a
// partly reset slot is not empty yet)
__device__ __forceinline__ bool sentinel_is_empty(const u32x4& v) {
  return (v[0] & v[1] & v[2] & v[3]) == 0xFFFFFFFFu;
}
// 16 payload bytes into the slot at `off` (canonicalised)
template <int kElemBytes, Scope kScope>
__device__ __forceinline__ void sentinel_put(Wire w, uint32_t off, u32x4 data) {
  store16<kScope>(w, off, sentinel_canon<kElemBytes>(data));
}
// one poll of the 8-byte half-slot at `off`
template <int kElemBytes>
__device__ __forceinline__ bool sentinel_try8(Wire w, uint32_t off, u32x2& data) {
  data = ld8_coh(w, off);
  return sentinel_ready8<kElemBytes>(data);
}
template <int kElemBytes>
__device__ __forceinline__ bool sentinel_try(Wire w, uint32_t off, u32x4& data) {
  data = ld16_coh(w, off);
  return sentinel_ready<kElemBytes>(data);
}
template <int kElemBytes, int kSleep>
__device__ __forceinline__ bool sentinel_wait(Wire w, uint32_t off, PollT<kSleep>& poll, u32x4& data) {
  while (!sentinel_try<kElemBytes>(w, off, data))
    if (poll.expired()) return false;
  return true;
}
template <Scope kScope>
__device__ __forceinline__ void sentinel_reset8(Wire w, uint32_t off) {
  store8<kScope>(w, off, u32x2{0xFFFFFFFFu, 0xFFFFFFFFu});
}
template <Scope kScope>
__device__ __forceinline__ void sentinel_reset(Wire w, uint32_t off) {
  store16<kScope>(w, off, u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
}

// ---- LL128 ------------------------------------------------------------------------------------
// Contributions are device-scope float atomics on a flat pointer into the
// line (slot s of the line at byte offset L is at base + L + s * sizeof(A)).
constexpr uint32_t kLL128LineBytes = 128;
__device__ __forceinline__ void ll128_add(float* slot, float v) {
  __hip_atomic_fetch_add(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// two adjacent 16-bit slots (bfloat16 when kBf16, else binary16), packed
template <bool kBf16>
__device__ __forceinline__ void ll128_add2(void* slot_pair, s16x2 v) {
  if constexpr (kBf16) {
    __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<s16x2*>(slot_pair), v);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_global_atomic_fadd_v2f16(reinterpret_cast<h2*>(slot_pair), __builtin_bit_cast(h2, v));
  }
}
// this sender's count: call release() after the sender's data atomics of
// the line, then add 1.0 to slot 0
__device__ __forceinline__ void ll128_flag(float* line) { ll128_add(line, 1.0f); }
template <bool kBf16>
__device__ __forceinline__ void ll128_flag2(void* line, uint32_t one_bits) {
  ll128_add2<kBf16>(line, s16x2{(short)one_bits, (short)0});
}
// poll slot 0 of the line at `off` until it equals `full` (the count N in
// the accumulation type, as raw bits; 16-bit types compare the low half)
template <bool k16, int kSleep>
__device__ __forceinline__ bool ll128_wait(Wire w, uint32_t off, uint32_t full, PollT<kSleep>& poll) {
  while (true) {
    uint32_t f = ld4_coh(w, off);
    if constexpr (k16) f &= 0xFFFFu;
    if (f == full) return true;
    if (poll.expired()) return false;
  }
}
// 16 bytes of a line, after its count is complete; then zero them
__device__ __forceinline__ u32x4 ll128_read16(Wire w, uint32_t off) { return ld16_coh(w, off); }
__device__ __forceinline__ void ll128_reset16(Wire w, uint32_t off) { st16_coh(w, off, u32x4{0u, 0u, 0u, 0u}); }
// The same 16 bytes (at `p`, 8-byte aligned) read and zeroed at once, after
// the line's count is complete: two device-scope 8-byte exchanges with zero,
// which resolve where the line's float atomics did, so no separate zeroing
// store is left to be acknowledged
__device__ __forceinline__ u32x4 ll128_take16(uint8_t* p) {
  uint64_t* const q = reinterpret_cast<uint64_t*>(p);
  const uint64_t lo = __hip_atomic_exchange(q, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_exchange(q + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

}  // namespace llar_wire

#endif  // LLAR_WIRE_H
