// llar_kernels.hip -- HIP kernels (gfx950) of the barrier-free AllReduce
// protocols with N ranks emulated inside one GPU.
//
// Rank emulation: a launch has N * W workgroups; workgroup (rank r, slice w)
// reads only rank r's partial buffer and talks to other ranks only through
// the communicator's staging memory.  No workgroup ever waits on a grid-wide
// barrier: every wait is a bounded poll on a flag or a value written by the
// rank it needs.  Two placements of (r, w) onto workgroup ids (the hardware
// deals workgroup b to XCD b mod 8):
//   spread: b = w*N + r          -- with N = 8, rank r lives on XCD r, so
//                                  every exchange crosses XCDs;
//   local:  b = (w/8*N + r)*8 + w%8 -- all ranks of slice w share XCD w%8 and
//                                  its L2, so staging traffic stays on chip.
//
// Sources (prose of "Every Microsecond Matters", agihunt.info summary):
//   LL paragraph        -> k_oneshot<kWireLL>
//   Sentinel paragraph  -> k_oneshot<kWireSentinel>, k_twoshot_sentinel
//   bidirectional + double buffering paragraph -> the chunk loop of the
//                          two-shot kernels (parity = chunk & 1, implicit credit)
//   Two-shot LL128 paragraph -> k_twoshot_ll128
#include "llar_device.h"
#include "llar_internal.h"

namespace llar {

// ---------------------------------------------------------------------------
// shared prologue / epilogue: the call's epoch
// ---------------------------------------------------------------------------
// Two epoch sources.  In ordinary stream-ordered use the host numbers the
// calls and passes the epoch in the kernel arguments (host_epoch, bit 31
// clear): nothing to read on the device.  Under graph capture the arguments
// would repeat on every replay, so the kernel reads the device-resident epoch
// (bit 31 set; the two ranges never meet): thread 0 reads it, publishes it
// through LDS and takes an arrival ticket; the workgroup that arrives last
// (ticket == G-1) advances it when it finishes -- by then every workgroup of
// the call has read the old value, and the next call starts after this one.
// Timing mode has each workgroup store its own start and end stamps in the
// epoch's ring slot (plain stores, no shared counter); workgroup 0 also
// records the grid so that the reader knows how many entries belong to it.
struct WgState {
  uint32_t epoch;
  uint32_t ticket;
  bool counted;
  uint64_t t0;
};

__device__ __forceinline__ WgState wg_begin(Ctrl* ctrl, uint32_t host_epoch, bool timing, bool idle) {
  __shared__ uint32_t s_epoch;
  WgState st{host_epoch, 0u, false, 0ull};
  if (timing && threadIdx.x == 0) st.t0 = wall_ticks();
  if (host_epoch != 0u) return st;
  if (threadIdx.x == 0) {
    const uint32_t e = __hip_atomic_load(&ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_epoch = e;
    st.ticket = __hip_atomic_fetch_add(&ctrl->arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st.counted = true;
  }
  __syncthreads();
  st.epoch = s_epoch;
  return st;
}

__device__ __forceinline__ void wg_end(Ctrl* ctrl, const WgState& st, uint32_t host_epoch, uint32_t grid, bool timing,
                                       bool idle) {
  if (timing) {
    drain_vm();
    __syncthreads();
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
  if (st.counted && st.ticket == grid - 1u) {
    __hip_atomic_store(&ctrl->arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctrl->epoch, next_device_epoch(st.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void decode_role(uint32_t b, int n_ranks, uint32_t placement, int& r, uint32_t& w) {
  if (placement == kPlaceLocal) {
    uint32_t x = b & 7u, q = b >> 3;
    r = (int)(q % (uint32_t)n_ranks);
    w = (q / (uint32_t)n_ranks) * 8u + x;
  } else {
    r = (int)(b % (uint32_t)n_ranks);
    w = b / (uint32_t)n_ranks;
  }
}

// ---------------------------------------------------------------------------
// tail-safe 16-byte vector access to the caller's buffers
// ---------------------------------------------------------------------------
template <bool kStream = true>
__device__ __forceinline__ u32x4 load_vec(const uint8_t* p, uint64_t v, uint64_t nbytes) {
  uint64_t off = v * 16u;
  if (off + 16u <= nbytes) {
    if constexpr (kStream) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + off));
    else return *reinterpret_cast<const u32x4*>(p + off);
  }
  u32x4 x = {0u, 0u, 0u, 0u};
  for (uint64_t i = off; i < nbytes; i += 2u) {  // element sizes are 2 or 4 bytes
    uint32_t h = *reinterpret_cast<const uint16_t*>(p + i);
    uint32_t k = (uint32_t)(i - off);
    x[k >> 2] |= h << ((k & 2u) * 8u);
  }
  return x;
}
// 8-byte units (the one-shot consumer's granularity)
__device__ __forceinline__ u32x2 load_unit(const uint8_t* p, uint64_t u, uint64_t nbytes) {
  uint64_t off = u * 8u;
  if (off + 8u <= nbytes) return *reinterpret_cast<const u32x2*>(p + off);
  u32x2 x = {0u, 0u};
  for (uint64_t i = off; i < nbytes; i += 2u) {
    uint32_t h = *reinterpret_cast<const uint16_t*>(p + i);
    uint32_t k = (uint32_t)(i - off);
    x[k >> 2] |= h << ((k & 2u) * 8u);
  }
  return x;
}
__device__ __forceinline__ void store_unit(uint8_t* p, uint64_t u, uint64_t nbytes, u32x2 x) {
  uint64_t off = u * 8u;
  if (off + 8u <= nbytes) {
    *reinterpret_cast<u32x2*>(p + off) = x;
    return;
  }
  for (uint64_t i = off; i < nbytes; i += 2u) {
    uint32_t k = (uint32_t)(i - off);
    *reinterpret_cast<uint16_t*>(p + i) = (uint16_t)(x[k >> 2] >> ((k & 2u) * 8u));
  }
}
template <bool kStream = false>
__device__ __forceinline__ void store_vec(uint8_t* p, uint64_t v, uint64_t nbytes, u32x4 x) {
  uint64_t off = v * 16u;
  if (off + 16u <= nbytes) {
    if constexpr (kStream) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p + off));
    else *reinterpret_cast<u32x4*>(p + off) = x;
    return;
  }
  for (uint64_t i = off; i < nbytes; i += 2u) {
    uint32_t k = (uint32_t)(i - off);
    *reinterpret_cast<uint16_t*>(p + i) = (uint16_t)(x[k >> 2] >> ((k & 2u) * 8u));
  }
}

// Reduce one 16-byte vector: own contribution at rank position `own_rank`,
// the others in `d[0..N-2]` ordered by rank; binary64 sum in rank order
// starting from rank 0's value, one rounding to the output type.
// (Array indices stay compile-time -- a runtime index would push the array
// to scratch memory -- and the rank position is chosen with selects.)
template <int kKind, int N>
__device__ __forceinline__ u32x4 reduce_vec(const u32x4& own, int own_rank, const u32x4 (&d)[N > 1 ? N - 1 : 1]) {
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < Elem<kKind>::kPerVec; ++j) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const uint32_t below = (r < N - 1) ? vec_elem<kKind>(d[r < N - 1 ? r : 0], j) : 0u;  // rank r sits at d[r]
      const uint32_t above = (r >= 1) ? vec_elem<kKind>(d[r >= 1 ? r - 1 : 0], j) : 0u;   // rank r sits at d[r-1]
      const uint32_t bits = (r < own_rank) ? below : (r == own_rank) ? vec_elem<kKind>(own, j) : above;
      double x = Elem<kKind>::dec(bits);
      s = (r == 0) ? x : s + x;
    }
    vec_set<kKind>(out, j, Elem<kKind>::enc(s));
  }
  return out;
}

// The same for an 8-byte unit (rank 0's own value first).
template <int kKind, int N>
__device__ __forceinline__ u32x2 reduce_unit(const u32x2& own, const u32x2 (&d)[N > 1 ? N - 1 : 1]) {
  constexpr int kPerUnit = 8 / Elem<kKind>::kBytes;
  u32x2 out = {0u, 0u};
#pragma unroll
  for (int j = 0; j < kPerUnit; ++j) {
    auto elem = [&](const u32x2& v) -> uint32_t {
      if constexpr (Elem<kKind>::kBytes == 4) return v[j];
      else return (v[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
    };
    double s = Elem<kKind>::dec(elem(own));
#pragma unroll
    for (int r = 1; r < N; ++r) s += Elem<kKind>::dec(elem(d[r - 1]));
    uint32_t bits = Elem<kKind>::enc(s);
    if constexpr (Elem<kKind>::kBytes == 4) out[j] = bits;
    else out[j >> 1] |= (bits & 0xFFFFu) << ((j & 1) * 16);
  }
  return out;
}

// ---------------------------------------------------------------------------
// one-shot LL / Sentinel: ranks 1..N-1 push, rank 0 reduces the whole message
// ---------------------------------------------------------------------------
// LL staging: [parity][rank-1][vector][2 lines of 16 B]; a line is
// {data0, epoch, data1, epoch} so each 8-byte half carries its own flag.
// Sentinel staging: [parity][rank-1][vector] 16 B, all-ones when empty.
// Phase trace (debug): thread 0 stamps the wall clock at each step; the
// stamps after stores first wait for the stores to be acknowledged.
__device__ __forceinline__ void trace_at(uint64_t* tr, int slot, bool drain) {
  if (tr && threadIdx.x == 0) {
    if (drain) drain_vm();
    tr[blockIdx.x * kTraceWords + slot] = wall_ticks();
  }
}

template <int kWire, int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(512) k_oneshot(OneShotArgs a) {
  const uint64_t t_entry = wall_ticks();
  int r;
  uint32_t w;
  decode_role(blockIdx.x, N, a.placement, r, w);
  const bool idle = (w >= a.slices);
  // slice w: 16-byte vectors [v0, v1) for producers, 8-byte units [2 v0, 2 v1)
  // for the consumer (one LL line, or half a Sentinel slot, per lane)
  const uint64_t v0 = idle ? 0 : (uint64_t)w * a.n_vec / a.slices;
  const uint64_t v1 = idle ? 0 : (uint64_t)(w + 1) * a.n_vec / a.slices;
  const bool producer = (r != 0) && !idle && (uint32_t)r != a.drop_rank;
  const bool consumer = (r == 0) && !idle;
  // the first input of this thread is requested before anything else
  u32x4 first_vec = {0u, 0u, 0u, 0u};
  u32x2 first_unit = {0u, 0u};
  if (producer && v0 + threadIdx.x < v1) first_vec = load_vec<false>(a.part[r], v0 + threadIdx.x, a.nbytes);
  if (consumer && 2 * v0 + threadIdx.x < 2 * v1) first_unit = load_unit(a.part[0], 2 * v0 + threadIdx.x, a.nbytes);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  if (a.trace && threadIdx.x == 0) a.trace[blockIdx.x * kTraceWords + 0] = t_entry;
  trace_at(a.trace, 1, false);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint32_t e = st.epoch;
  const uint32_t par_off = (e & 1u) * a.parity_stride;
  constexpr uint32_t kVecStage = (kWire == kWireLL) ? 32u : 16u;

  if (producer) {
    const uint8_t* src = a.part[r];
    const uint32_t base = par_off + (uint32_t)(r - 1) * a.rank_stride;
    for (uint64_t v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
      u32x4 x = (v == v0 + threadIdx.x) ? first_vec : load_vec<false>(src, v, a.nbytes);
      if (v == v0) trace_at(a.trace, 2, true);
      uint32_t off = base + (uint32_t)v * kVecStage;
      if constexpr (kWire == kWireLL) {
        st16_stage<kLocal>(rs, off, u32x4{x[0], e, x[1], e});
        st16_stage<kLocal>(rs, off + 16u, u32x4{x[2], e, x[3], e});
      } else {
        st16_stage<kLocal>(rs, off, sentinel_canon<kKind>(x));
      }
      if (v == v0) trace_at(a.trace, 3, true);
    }
  } else if (consumer) {
    const uint8_t* own_src = a.part[0];
    constexpr uint32_t kUnitStage = (kWire == kWireLL) ? 16u : 8u;
    bool dead = false;  // set after a timeout: stop waiting for anything else
    for (uint64_t u = 2 * v0 + threadIdx.x; u < 2 * v1 && !dead; u += blockDim.x) {
      u32x2 own = (u == 2 * v0 + threadIdx.x) ? first_unit : load_unit(own_src, u, a.nbytes);
      if (u == 2 * v0) trace_at(a.trace, 2, true);
      // A slot that is ready stays ready for the rest of the call (LL lines
      // carry this call's epoch; a filled Sentinel slot is only reset by this
      // thread), so reload every slot until one pass sees all of them ready
      // and reduce from that pass.
      u32x2 d[N > 1 ? N - 1 : 1];
      Spin spin(a.spin_limit);
      bool ok = true;
      while (true) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          uint32_t off = par_off + (uint32_t)k * a.rank_stride + (uint32_t)u * kUnitStage;
          if constexpr (kWire == kWireLL) {
            u32x4 line = ld16_coh(rs, off);
            all &= (line[1] == e) & (line[3] == e);
            d[k] = u32x2{line[0], line[2]};
          } else {
            d[k] = ld8_coh(rs, off);
            all &= sentinel_ready8<kKind>(d[k]);
          }
        }
        if (all) break;
        if (spin.expired()) {
          raise_status(a.ctrl, kStatusTimeout);
          ok = false;
          break;
        }
      }
      if (!ok) {
        dead = true;
        continue;
      }
      if (u == 2 * v0) trace_at(a.trace, 3, false);
      store_unit(a.out, u, a.nbytes, reduce_unit<kKind, N>(own, d));
      if (u == 2 * v0) trace_at(a.trace, 4, true);
      if constexpr (kWire == kWireSentinel) {
        if (!a.keep) {
#pragma unroll
          for (int k = 0; k < N - 1; ++k)
            st8_stage<kLocal>(rs, par_off + (uint32_t)k * a.rank_stride + (uint32_t)u * 8u,
                              u32x2{0xFFFFFFFFu, 0xFFFFFFFFu});
        }
      }
    }
  }
  wg_end(a.ctrl, st, a.host_epoch, a.grid, a.timing, idle);
  if (a.trace && threadIdx.x == 0) {
    a.trace[blockIdx.x * kTraceWords + 5] = wall_ticks();
    a.trace[blockIdx.x * kTraceWords + 6] = (uint64_t)xcc_id() | ((uint64_t)r << 8) | ((uint64_t)w << 16);
  }
}

// ---------------------------------------------------------------------------
// two-shot LL128 atomic, chunked and double-buffered
// ---------------------------------------------------------------------------
// Staging: [parity][line] of 128 bytes in the staging type A (binary32, or the
// 16-bit I/O type packed in pairs).  Slot 0 of a line counts contributions
// (each rank adds 1.0); slots 1..K hold elements line*K .. line*K+K-1 of the
// chunk (K = 128/sizeof(A) - 1).  The lines of a chunk are split into N
// contiguous owner ranges; owner s's range is split into W slices.
//
// Workgroup (r, w), for every chunk c (parity c & 1):
//   produce: for every owner s, add rank r's elements of slice (s, w) into
//            the lines, data first; after the wave's data atomics are
//            acknowledged (drain), add 1.0 to each of those lines' slot 0;
//   consume: for each line of slice (r, w), poll slot 0 until it reads N,
//            read the line, round to the I/O type, write `out`, zero the line.
// Implicit credit: finishing consume(c+1) means every rank's slice-w
// workgroup has contributed chunk c+1 to this workgroup's lines (every line
// receives all N contributions), which each did only after all of its waves
// had finished consume(c) and their zeroing stores were acknowledged (drain
// + workgroup barrier between chunks), so the parity of chunk c is free again
// for chunk c+2.  The credit is the workgroup's: a wave may have no line of
// its own to consume while it produces into other owners' lines.  The host
// keeps every owner slice of a full chunk non-empty, so every workgroup
// receives the credit.
template <int kKind, int kAcc16, int N>
__global__ void __launch_bounds__(512) k_twoshot_ll128(TwoShotArgs a) {
  int r;
  uint32_t w;
  decode_role(blockIdx.x, N, a.placement, r, w);
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  constexpr int kSlots = kAcc16 ? 64 : 32;
  constexpr int K = kSlots - 1;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  const uint8_t* src = a.part[r];
  // flag value N in the staging type
  uint32_t flag_full;
  if constexpr (!kAcc16) flag_full = __float_as_uint((float)N);
  else flag_full = E::from_f32((float)N);
  bool dead = idle;  // idle padding workgroup, or a poll timed out

  for (uint32_t c = 0; c < a.n_chunks && !dead; ++c) {
    const uint64_t cbase = (uint64_t)c * a.chunk_elems;
    const uint32_t len = (uint32_t)min((uint64_t)a.chunk_elems, a.n - cbase);
    // Lines are partitioned by the nominal chunk (not this chunk's length):
    // a line must belong to the same (owner, slice) in every chunk, or the
    // implicit credit of one slice would release a line another slice has
    // not consumed yet.  Elements past the message end are masked.
    const uint32_t L = (a.chunk_elems + K - 1) / K;
    // lines that hold data of this chunk: producers flag and consumers poll
    // only these (both sides agree, and a line past them stays zero)
    const uint32_t Lr = (len + K - 1) / K;
    const uint32_t poff = (c & 1u) * a.parity_stride;

    // ---- produce: data atomics for every owner's slice w
    const bool silent = ((uint32_t)r == a.drop_rank);
    for (int s = 0; s < N && !silent; ++s) {
      uint32_t o0 = (uint32_t)((uint64_t)s * L / N), o1 = (uint32_t)((uint64_t)(s + 1) * L / N);
      uint32_t l0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
      uint32_t l1 = min(o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices), Lr);
      for (uint32_t lb = l0 + wave * 8u; lb < l1; lb += n_waves * 8u) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t d = (uint32_t)k * 64u + lane;  // dword of the 8-line block
          uint32_t line = lb + d / 32u;
          uint32_t q = d % 32u;                   // dword within the line
          if (line >= l1) continue;
          uint32_t off = poff + line * 128u + q * 4u;
          if constexpr (!kAcc16) {
            if (q == 0u) continue;  // slot 0 is the flag
            uint32_t e_idx = line * K + q - 1u;
            if (e_idx >= len) continue;
            float val;
            if constexpr (E::kBytes == 4) val = __uint_as_float(reinterpret_cast<const uint32_t*>(src)[cbase + e_idx]);
            else val = E::to_f32(reinterpret_cast<const uint16_t*>(src)[cbase + e_idx]);
            __hip_atomic_fetch_add(reinterpret_cast<float*>(a.stage + off), val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            // two 16-bit slots per dword: slots 2q and 2q+1
            uint32_t lo = 0u, hi = 0u;
            uint32_t s0 = 2u * q, s1 = 2u * q + 1u;
            if (s0 >= 1u) {
              uint32_t e0 = line * K + s0 - 1u;
              if (e0 < len) lo = reinterpret_cast<const uint16_t*>(src)[cbase + e0];
            }
            uint32_t e1 = line * K + s1 - 1u;
            if (e1 < len) hi = reinterpret_cast<const uint16_t*>(src)[cbase + e1];
            if ((lo | hi) == 0u) continue;  // nothing to add (both +0)
            s16x2 v = {(short)lo, (short)hi};
            if constexpr (kKind == kKindBF16)
              __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<s16x2*>(a.stage + off), v);
            else
              __builtin_amdgcn_global_atomic_fadd_v2f16(reinterpret_cast<_Float16 __attribute__((ext_vector_type(2)))*>(a.stage + off),
                                                       __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), v));
          }
        }
      }
    }
    // data of this wave acknowledged before any of its flags
    drain_vm();
    for (int s = 0; s < N && !silent; ++s) {
      uint32_t o0 = (uint32_t)((uint64_t)s * L / N), o1 = (uint32_t)((uint64_t)(s + 1) * L / N);
      uint32_t l0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
      uint32_t l1 = min(o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices), Lr);
      for (uint32_t lb = l0 + wave * 8u; lb < l1; lb += n_waves * 8u) {
        uint32_t line = lb + lane;
        if (lane < 8u && line < l1) {
          uint32_t off = poff + line * 128u;
          if constexpr (!kAcc16) {
            __hip_atomic_fetch_add(reinterpret_cast<float*>(a.stage + off), 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else {
            s16x2 v = {(short)E::from_f32(1.0f), (short)0};
            if constexpr (kKind == kKindBF16)
              __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<s16x2*>(a.stage + off), v);
            else
              __builtin_amdgcn_global_atomic_fadd_v2f16(reinterpret_cast<_Float16 __attribute__((ext_vector_type(2)))*>(a.stage + off),
                                                       __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), v));
          }
        }
      }
    }

    // ---- consume owner r's slice w: 8 lanes per line
    {
      uint32_t o0 = (uint32_t)((uint64_t)r * L / N), o1 = (uint32_t)((uint64_t)(r + 1) * L / N);
      uint32_t l0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
      uint32_t l1 = min(o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices), Lr);
      const uint32_t grp = lane >> 3, j = lane & 7u;
      for (uint32_t lb = l0 + wave * 8u; lb < l1; lb += n_waves * 8u) {
        uint32_t line = lb + grp;
        if (line >= l1) continue;
        uint32_t loff = poff + line * 128u;
        Spin spin(a.spin_limit);
        bool ok = true;
        while (true) {
          uint32_t f = ld4_coh(rs, loff);
          if constexpr (kAcc16) f &= 0xFFFFu;
          if (f == flag_full) break;
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            ok = false;
            break;
          }
        }
        if (!ok) {
          dead = true;
          break;
        }
        u32x4 v = ld16_coh(rs, loff + j * 16u);
        if constexpr (!kAcc16) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            uint32_t q = j * 4u + (uint32_t)t;
            if (q == 0u) continue;
            uint32_t e_idx = line * K + q - 1u;
            if (e_idx >= len) continue;
            if constexpr (E::kBytes == 4) reinterpret_cast<uint32_t*>(a.out)[cbase + e_idx] = v[t];
            else reinterpret_cast<uint16_t*>(a.out)[cbase + e_idx] = (uint16_t)E::from_f32(__uint_as_float(v[t]));
          }
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            uint32_t q = j * 8u + (uint32_t)t;
            if (q == 0u) continue;
            uint32_t e_idx = line * K + q - 1u;
            if (e_idx >= len) continue;
            reinterpret_cast<uint16_t*>(a.out)[cbase + e_idx] = (uint16_t)(v[t >> 1] >> ((t & 1) * 16));
          }
        }
        if (!a.keep) st16_coh(rs, loff + j * 16u, u32x4{0u, 0u, 0u, 0u});
      }
    }
    // every wave's zeroing stores are acknowledged before any wave of this
    // workgroup contributes to the next chunk (a workgroup-uniform exit too)
    drain_vm();
    dead = __syncthreads_or((int)dead) != 0;
  }
  wg_end(a.ctrl, st, a.host_epoch, a.grid, a.timing, idle);
}

// ---------------------------------------------------------------------------
// two-shot Sentinel, chunked and multi-buffered, producer/consumer waves
// ---------------------------------------------------------------------------
// Staging: [buffer][owner s][sender r][vector of s's shard] 16 B, all-ones
// when empty.  Chunk c's vectors are split into N owner shards and each
// shard into W slices; a vector keeps its (owner, slice) in every chunk
// (the partition uses the nominal chunk, the tail of the message is masked).
// Workgroup (r, w) is split in two halves:
//   producer waves: for every chunk c, request rank r's vectors of slice
//            (s, w) for every owner s != r, then -- once this workgroup's
//            consumer waves have finished chunks 0..c-1-lag -- store them,
//            sentinel-canonicalised, into [c % B][s][r].  The loads are
//            issued before the credit wait, so HBM reads overlap it;
//   consumer waves: for each vector of slice (r, w) of chunk c, poll the N-1
//            slots [c % B][r][*], add the own partial (requested one chunk
//            early) and the N-1 staged ones in binary64 in rank order, round,
//            write `out`, reset the slots; drain (the resets are performed),
//            then publish "chunk c done" to the producer waves through LDS.
// The credit: a producer stores chunk c only after this workgroup's
// consumers finished chunk c-1-lag.  They finished it only after every
// peer's producer stored chunk c-1-lag, which each did only after its own
// consumers had finished chunk c-2-2*lag and drained those resets; with
// B >= 2*lag + 2 buffers that covers chunk c-B, the previous user of chunk
// c's buffer.
template <int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(512) k_twoshot_sentinel(TwoShotArgs a) {
  constexpr int kU = 2;   // vectors per producer lane per owner per batch
  constexpr int kUc = 2;  // vectors per consumer lane per batch
  int r;
  uint32_t w;
  decode_role(blockIdx.x, N, a.placement, r, w);
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  __shared__ uint32_t s_done[8];  // per consumer wave: chunks finished
  if (threadIdx.x < 8) s_done[threadIdx.x] = 0u;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint8_t* src = a.part[r];
  const uint64_t nbytes = a.n * (uint64_t)E::kBytes;
  const uint32_t chunk_vecs = (uint32_t)(((uint64_t)a.chunk_elems * E::kBytes + 15u) / 16u);
  const uint64_t total_vecs = (nbytes + 15u) / 16u;
  const uint32_t slot_bytes = a.shard_cap * 16u;
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, n_waves = blockDim.x >> 6;
  const uint32_t n_prod = n_waves / 2, n_cons = n_waves - n_prod;
  const uint32_t n_buf = a.n_buffers;
  const uint32_t lag = n_buf / 2u - 1u;
  // the partition uses the nominal chunk so that a slot keeps its (owner,
  // slice) in every chunk; vectors past the end of the message are masked
  const uint32_t nv = chunk_vecs;
  bool dead = idle;
  uint64_t* tr = (a.trace && !idle) ? a.trace + (uint64_t)blockIdx.x * kPipeTraceWords : nullptr;
  auto stamp = [&](int kind, uint32_t c) {
    if (tr && lane == 0 && c < (uint32_t)kPipeTraceChunks) tr[kind * kPipeTraceChunks + c] = wall_ticks();
  };

  if (wave < n_prod) {
    // ---------------- producer waves
    const uint32_t pl = wave * 64u + lane, PL = n_prod * 64u;
    const bool silent = ((uint32_t)r == a.drop_rank);
    for (uint32_t c = 0; c < a.n_chunks && !dead; ++c) {
      const uint64_t vbase = (uint64_t)c * chunk_vecs;
      // vectors of this chunk that exist; the partition below uses the
      // nominal chunk so that a slot keeps its (owner, slice) in every chunk
      const uint32_t nv_real = (uint32_t)min((uint64_t)chunk_vecs, total_vecs - vbase);
      const uint32_t nv = chunk_vecs;
      const uint32_t poff = (c % n_buf) * a.parity_stride;
      const uint32_t span = (nv / N + 1u) / a.slices + 2u;  // longest (owner, slice) range
      for (uint32_t b0 = 0; b0 < span && !dead; b0 += kU * PL) {
        u32x4 x[N > 1 ? N - 1 : 1][kU];
        uint32_t vo[N > 1 ? N - 1 : 1][kU];  // vector offset inside the owner's shard, or ~0
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          const int s = k < r ? k : k + 1;
          const uint32_t o0 = (uint32_t)((uint64_t)s * nv / N), o1 = (uint32_t)((uint64_t)(s + 1) * nv / N);
          const uint32_t s0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
          const uint32_t s1 = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const uint32_t v = s0 + b0 + pl + (uint32_t)u * PL;
            const bool ok = (v < s1) && (v < nv_real);
            vo[k][u] = ok ? v - o0 : ~0u;
            x[k][u] = ok ? load_vec(src, vbase + v, nbytes) : u32x4{0u, 0u, 0u, 0u};
          }
        }
        if (b0 == 0 && c > lag) {
          // credit: this workgroup's consumers have finished chunks 0..c-1-lag
          Spin spin(a.spin_limit);
          while (true) {
            uint32_t done = ~0u;
            for (uint32_t i = 0; i < n_cons; ++i)
              done = min(done, __hip_atomic_load(&s_done[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (done + lag >= c) break;
            if (spin.expired()) {
              raise_status(a.ctrl, kStatusTimeout);
              dead = true;
              break;
            }
          }
          if (dead) break;
        }
        if (b0 == 0 && wave == 0) stamp(0, c);
        if (silent) continue;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          const int s = k < r ? k : k + 1;
          const uint32_t slot = poff + (uint32_t)(s * N + r) * slot_bytes;
#pragma unroll
          for (int u = 0; u < kU; ++u)
            if (vo[k][u] != ~0u) st16_stage<kLocal>(rs, slot + vo[k][u] * 16u, sentinel_canon<kKind>(x[k][u]));
        }
      }
      if (wave == 0) stamp(1, c);
    }
  } else {
    // ---------------- consumer waves
    const uint32_t cw = wave - n_prod;
    const uint32_t cl = cw * 64u + lane, CL = n_cons * 64u;
    const uint32_t nv = chunk_vecs;
    const uint32_t o0 = (uint32_t)((uint64_t)r * nv / N), o1 = (uint32_t)((uint64_t)(r + 1) * nv / N);
    const uint32_t s0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
    const uint32_t s1n = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
    // own vectors of the first batch of the next chunk, requested early
    u32x4 own_next[kUc];
#pragma unroll
    for (int u = 0; u < kUc; ++u) {
      const uint32_t v = s0 + cl + (uint32_t)u * CL;
      own_next[u] = (!dead && v < s1n && v < total_vecs) ? load_vec(src, v, nbytes) : u32x4{0u, 0u, 0u, 0u};
    }
    for (uint32_t c = 0; c < a.n_chunks && !__any((int)dead); ++c) {
      const uint64_t vbase = (uint64_t)c * chunk_vecs;
      const uint32_t nv_real = (uint32_t)min((uint64_t)chunk_vecs, total_vecs - vbase);
      const uint32_t s1 = min(s1n, max(nv_real, s0));
      const uint32_t my = (c % n_buf) * a.parity_stride + (uint32_t)(r * N) * slot_bytes;
      if (s1 == s0 && cw == 0) stamp(2, c);  // nothing of this chunk here
      for (uint32_t b0 = 0; b0 < s1 - s0 && !dead; b0 += kUc * CL) {
        u32x4 own[kUc];
        bool valid[kUc];
#pragma unroll
        for (int u = 0; u < kUc; ++u) {
          const uint32_t v = s0 + b0 + cl + (uint32_t)u * CL;
          valid[u] = v < s1;
          if (b0 == 0) own[u] = own_next[u];
          else own[u] = valid[u] ? load_vec(src, vbase + v, nbytes) : u32x4{0u, 0u, 0u, 0u};
        }
        u32x4 d[kUc][N > 1 ? N - 1 : 1];
        SpinBulk spin(a.spin_limit);
        while (true) {
          bool all = true;
#pragma unroll
          for (int u = 0; u < kUc; ++u) {
            const uint32_t v = s0 + b0 + cl + (uint32_t)u * CL;
#pragma unroll
            for (int k = 0; k < N - 1; ++k) {
              const int sender = k < r ? k : k + 1;
              d[u][k] = valid[u] ? ld16_coh(rs, my + (uint32_t)sender * slot_bytes + (v - o0) * 16u)
                                 : u32x4{0u, 0u, 0u, 0u};
              all &= sentinel_ready<kKind>(d[u][k]);
            }
          }
          if (all) break;
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            dead = true;
            break;
          }
        }
        if (dead) break;
        if (b0 == 0 && cw == 0) stamp(2, c);
#pragma unroll
        for (int u = 0; u < kUc; ++u) {
          if (!valid[u]) continue;
          const uint32_t v = s0 + b0 + cl + (uint32_t)u * CL;
          store_vec(a.out, vbase + v, nbytes, reduce_vec<kKind, N>(own[u], r, d[u]));
          if (!a.keep) {
#pragma unroll
            for (int k = 0; k < N - 1; ++k) {
              const int sender = k < r ? k : k + 1;
              st16_stage<kLocal>(rs, my + (uint32_t)sender * slot_bytes + (v - o0) * 16u,
                                 u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
            }
          }
        }
      }
      // the resets are performed before the producers may reuse the buffer
      drain_vm();
      if (cw == 0) stamp(3, c);
      if (lane == 0 && !__any((int)dead))
        __hip_atomic_store(&s_done[cw], c + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // request the next chunk's own vectors while the producers fill it
      if (c + 1 < a.n_chunks) {
        const uint64_t nb = (uint64_t)(c + 1) * chunk_vecs;
        const uint32_t nv_next = (uint32_t)min((uint64_t)chunk_vecs, total_vecs - nb);
#pragma unroll
        for (int u = 0; u < kUc; ++u) {
          const uint32_t v = s0 + cl + (uint32_t)u * CL;
          own_next[u] = (v < s1n && v < nv_next) ? load_vec(src, nb + v, nbytes) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  wg_end(a.ctrl, st, a.host_epoch, a.grid, a.timing, idle);
}

// ---------------------------------------------------------------------------
// launchers (host side, one instantiation per (dtype, N))
// ---------------------------------------------------------------------------
template <int kKind, int N>
static hipError_t launch_n(const LaunchSpec& ls, hipStream_t stream) {
  dim3 grid(ls.grid), block(ls.threads);
  switch (ls.kernel) {
    case kKernOneShotLL:
      hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, N, false>), grid, block, 0, stream, ls.oneshot);
      break;
    case kKernOneShotSentinel:
      hipLaunchKernelGGL((k_oneshot<kWireSentinel, kKind, N, false>), grid, block, 0, stream, ls.oneshot);
      break;
    case kKernOneShotLLLocal:
      hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, N, true>), grid, block, 0, stream, ls.oneshot);
      break;
    case kKernOneShotSentinelLocal:
      hipLaunchKernelGGL((k_oneshot<kWireSentinel, kKind, N, true>), grid, block, 0, stream, ls.oneshot);
      break;
    case kKernLL128Acc32:
      hipLaunchKernelGGL((k_twoshot_ll128<kKind, 0, N>), grid, block, 0, stream, ls.twoshot);
      break;
    case kKernLL128Acc16:
      if constexpr (kKind != kKindF32) {
        hipLaunchKernelGGL((k_twoshot_ll128<kKind, 1, N>), grid, block, 0, stream, ls.twoshot);
      } else {
        return hipErrorInvalidValue;
      }
      break;
    case kKernSentinelPipe:
      hipLaunchKernelGGL((k_twoshot_sentinel<kKind, N, false>), grid, block, 0, stream, ls.twoshot);
      break;
    case kKernSentinelPipeLocal:
      hipLaunchKernelGGL((k_twoshot_sentinel<kKind, N, true>), grid, block, 0, stream, ls.twoshot);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kKind>
static hipError_t launch_kind(const LaunchSpec& ls, hipStream_t stream) {
  switch (ls.n_ranks) {
    case 1: return launch_n<kKind, 1>(ls, stream);
    case 2: return launch_n<kKind, 2>(ls, stream);
    case 3: return launch_n<kKind, 3>(ls, stream);
    case 4: return launch_n<kKind, 4>(ls, stream);
    case 5: return launch_n<kKind, 5>(ls, stream);
    case 6: return launch_n<kKind, 6>(ls, stream);
    case 7: return launch_n<kKind, 7>(ls, stream);
    case 8: return launch_n<kKind, 8>(ls, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch(const LaunchSpec& ls, hipStream_t stream) {
  switch (ls.kind) {
    case kKindF32: return launch_kind<kKindF32>(ls, stream);
    case kKindF16: return launch_kind<kKindF16>(ls, stream);
    case kKindBF16: return launch_kind<kKindBF16>(ls, stream);
    default: return hipErrorInvalidValue;
  }
}

// Occupancy of one kernel instance (workgroups per CU at `threads`).
template <int kKind, int N>
static int occupancy_n(int kernel, int threads) {
  int blocks = 0;
  hipError_t err = hipErrorInvalidValue;
  switch (kernel) {
    case kKernOneShotLL: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireLL, kKind, N, false>, threads, 0); break;
    case kKernOneShotSentinel: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireSentinel, kKind, N, false>, threads, 0); break;
    case kKernOneShotLLLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireLL, kKind, N, true>, threads, 0); break;
    case kKernOneShotSentinelLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireSentinel, kKind, N, true>, threads, 0); break;
    case kKernLL128Acc32: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_ll128<kKind, 0, N>, threads, 0); break;
    case kKernLL128Acc16:
      if constexpr (kKind != kKindF32) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_ll128<kKind, 1, N>, threads, 0);
      break;
    case kKernSentinelPipe: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel<kKind, N, false>, threads, 0); break;
    case kKernSentinelPipeLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel<kKind, N, true>, threads, 0); break;
    default: break;
  }
  return err == hipSuccess ? blocks : 0;
}

template <int kKind>
static int occupancy_kind(int n_ranks, int kernel, int threads) {
  switch (n_ranks) {
    case 1: return occupancy_n<kKind, 1>(kernel, threads);
    case 2: return occupancy_n<kKind, 2>(kernel, threads);
    case 3: return occupancy_n<kKind, 3>(kernel, threads);
    case 4: return occupancy_n<kKind, 4>(kernel, threads);
    case 5: return occupancy_n<kKind, 5>(kernel, threads);
    case 6: return occupancy_n<kKind, 6>(kernel, threads);
    case 7: return occupancy_n<kKind, 7>(kernel, threads);
    case 8: return occupancy_n<kKind, 8>(kernel, threads);
    default: return 0;
  }
}

int occupancy(int kind, int n_ranks, int kernel, int threads) {
  switch (kind) {
    case kKindF32: return occupancy_kind<kKindF32>(n_ranks, kernel, threads);
    case kKindF16: return occupancy_kind<kKindF16>(n_ranks, kernel, threads);
    case kKindBF16: return occupancy_kind<kKindBF16>(n_ranks, kernel, threads);
    default: return 0;
  }
}

// Placement probe: every workgroup reports the XCD it runs on.
__global__ void k_xcc_probe(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}
hipError_t launch_xcc_probe(uint32_t* out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(k_xcc_probe, dim3(grid), dim3(64), 0, stream, out);
  return hipGetLastError();
}

}  // namespace llar
