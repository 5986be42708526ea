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
// shared prologue / epilogue: device-resident epoch and the arrival counter
// ---------------------------------------------------------------------------
// Thread 0 reads the epoch, publishes it to the workgroup through LDS and
// takes an arrival ticket.  The workgroup that arrives last (ticket == G-1)
// advances the epoch when it finishes: by then every workgroup of this call
// has read the old value, and the next call starts only after this kernel.
struct WgState {
  uint32_t epoch;
  uint32_t ticket;
};

__device__ __forceinline__ WgState wg_begin(Ctrl* ctrl, bool timing) {
  __shared__ uint32_t s_epoch;
  WgState st{0u, 0u};
  if (threadIdx.x == 0) {
    uint64_t t0 = wall_ticks();
    uint32_t e = __hip_atomic_load(&ctrl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_epoch = e;
    st.ticket = __hip_atomic_fetch_add(&ctrl->arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (timing)
      __hip_atomic_fetch_min(&ctrl->timing[e % kTimingRing][0], t0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  st.epoch = s_epoch;
  return st;
}

__device__ __forceinline__ void wg_end(Ctrl* ctrl, const WgState& st, uint32_t grid, bool timing) {
  if (timing) {
    drain_vm();
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (timing) {
      uint64_t t1 = wall_ticks();
      __hip_atomic_fetch_max(&ctrl->timing[st.epoch % kTimingRing][1], t1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (st.ticket == grid - 1u) {
      uint32_t ne = next_epoch(st.epoch);
      if (timing) {
        __hip_atomic_store(&ctrl->timing[ne % kTimingRing][0], ~0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctrl->timing[ne % kTimingRing][1], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(&ctrl->arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctrl->epoch, ne, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
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
__device__ __forceinline__ u32x4 load_vec(const uint8_t* p, uint64_t v, uint64_t nbytes) {
  uint64_t off = v * 16u;
  if (off + 16u <= nbytes) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + off));
  u32x4 x = {0u, 0u, 0u, 0u};
  for (uint64_t i = off; i < nbytes; i += 2u) {  // element sizes are 2 or 4 bytes
    uint32_t h = *reinterpret_cast<const uint16_t*>(p + i);
    uint32_t k = (uint32_t)(i - off);
    x[k >> 2] |= h << ((k & 2u) * 8u);
  }
  return x;
}
__device__ __forceinline__ void store_vec(uint8_t* p, uint64_t v, uint64_t nbytes, u32x4 x) {
  uint64_t off = v * 16u;
  if (off + 16u <= nbytes) {
    *reinterpret_cast<u32x4*>(p + off) = x;
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
template <int kKind, int N>
__device__ __forceinline__ u32x4 reduce_vec(const u32x4& own, int own_rank, const u32x4 (&d)[N > 1 ? N - 1 : 1]) {
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < Elem<kKind>::kPerVec; ++j) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      uint32_t bits;
      if (r == own_rank) bits = vec_elem<kKind>(own, j);
      else bits = vec_elem<kKind>(d[r < own_rank ? r : r - 1], j);
      double x = Elem<kKind>::dec(bits);
      s = (r == 0) ? x : s + x;
    }
    vec_set<kKind>(out, j, Elem<kKind>::enc(s));
  }
  return out;
}

// ---------------------------------------------------------------------------
// one-shot LL / Sentinel: ranks 1..N-1 push, rank 0 reduces the whole message
// ---------------------------------------------------------------------------
// LL staging: [parity][rank-1][vector][2 lines of 16 B]; a line is
// {data0, epoch, data1, epoch} so each 8-byte half carries its own flag.
// Sentinel staging: [parity][rank-1][vector] 16 B, all-ones when empty.
template <int kWire, int kKind, int N>
__global__ void __launch_bounds__(512) k_oneshot(OneShotArgs a) {
  WgState st = wg_begin(a.ctrl, a.timing);
  int r;
  uint32_t w;
  decode_role(blockIdx.x, N, a.placement, r, w);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint32_t e = st.epoch;
  const uint32_t par_off = (e & 1u) * a.parity_stride;
  const uint64_t v0 = (uint64_t)w * a.n_vec / a.slices, v1 = (uint64_t)(w + 1) * a.n_vec / a.slices;
  constexpr uint32_t kVecStage = (kWire == kWireLL) ? 32u : 16u;

  if (w >= a.slices || (uint32_t)r == a.drop_rank) {
    // idle workgroup (placement padding), or a producer silenced by a test
  } else if (r != 0) {
    // ---- producer of rank r
    const uint8_t* src = a.part[r];
    const uint32_t base = par_off + (uint32_t)(r - 1) * a.rank_stride;
    for (uint64_t v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
      u32x4 x = load_vec(src, v, a.nbytes);
      uint32_t off = base + (uint32_t)v * kVecStage;
      if constexpr (kWire == kWireLL) {
        st16_coh(rs, off, u32x4{x[0], e, x[1], e});
        st16_coh(rs, off + 16u, u32x4{x[2], e, x[3], e});
      } else {
        st16_coh(rs, off, sentinel_canon<kKind>(x));
      }
    }
  } else {
    // ---- consumer (rank 0)
    const uint8_t* own_src = a.part[0];
    bool dead = false;  // set after a timeout: stop waiting for anything else
    for (uint64_t v = v0 + threadIdx.x; v < v1 && !dead; v += blockDim.x) {
      u32x4 own = load_vec(own_src, v, a.nbytes);
      // A slot that is ready stays ready for the rest of the call (LL lines
      // carry this call's epoch; a filled Sentinel slot is only reset by this
      // thread), so reload every slot until one pass sees all of them ready
      // and reduce from that pass.
      u32x4 d[N > 1 ? N - 1 : 1];
      Spin spin(a.spin_limit);
      bool ok = true;
      while (true) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          uint32_t off = par_off + (uint32_t)k * a.rank_stride + (uint32_t)v * kVecStage;
          if constexpr (kWire == kWireLL) {
            u32x4 l0 = ld16_coh(rs, off), l1 = ld16_coh(rs, off + 16u);
            all &= (l0[1] == e) & (l0[3] == e) & (l1[1] == e) & (l1[3] == e);
            d[k] = u32x4{l0[0], l0[2], l1[0], l1[2]};
          } else {
            d[k] = ld16_coh(rs, off);
            all &= sentinel_ready<kKind>(d[k]);
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
      store_vec(a.out, v, a.nbytes, reduce_vec<kKind, N>(own, 0, d));
      if constexpr (kWire == kWireSentinel) {
        if (!a.keep) {
#pragma unroll
          for (int k = 0; k < N - 1; ++k)
            st16_coh(rs, par_off + (uint32_t)k * a.rank_stride + (uint32_t)v * 16u,
                     u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
        }
      }
    }
  }
  wg_end(a.ctrl, st, a.grid, a.timing);
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
// workgroup has contributed chunk c+1, which each did only after finishing
// its own consume(c) (zeroing its chunk-c lines), so the parity of chunk c is
// free again for chunk c+2.
template <int kKind, int kAcc16, int N>
__global__ void __launch_bounds__(512) k_twoshot_ll128(TwoShotArgs a) {
  WgState st = wg_begin(a.ctrl, a.timing);
  int r;
  uint32_t w;
  decode_role(blockIdx.x, N, a.placement, r, w);
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
  bool dead = (w >= a.slices);  // idle padding workgroup, or a poll timed out

  for (uint32_t c = 0; c < a.n_chunks && !__any((int)dead); ++c) {
    const uint64_t cbase = (uint64_t)c * a.chunk_elems;
    const uint32_t len = (uint32_t)min((uint64_t)a.chunk_elems, a.n - cbase);
    const uint32_t L = (len + K - 1) / K;
    const uint32_t poff = (c & 1u) * a.parity_stride;

    // ---- produce: data atomics for every owner's slice w
    const bool silent = ((uint32_t)r == a.drop_rank);
    for (int s = 0; s < N && !silent; ++s) {
      uint32_t o0 = (uint32_t)((uint64_t)s * L / N), o1 = (uint32_t)((uint64_t)(s + 1) * L / N);
      uint32_t l0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
      uint32_t l1 = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
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
      uint32_t l1 = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
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
      uint32_t l1 = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
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
          continue;
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
  }
  wg_end(a.ctrl, st, a.grid, a.timing);
}

// ---------------------------------------------------------------------------
// two-shot Sentinel, chunked and double-buffered
// ---------------------------------------------------------------------------
// Staging: [parity][owner s][sender rank r][vector of s's shard] 16 B,
// all-ones when empty.  Chunk c's vectors are split into N owner shards and
// each shard into W slices.  Workgroup (r, w), per chunk c:
//   produce: for every owner s != r, copy rank r's vectors of slice (s, w)
//            (sentinel-canonicalised) into [c&1][s][r];
//   consume: for each vector of slice (r, w): read its own partial, poll the
//            N-1 slots [c&1][r][*] until no element is the sentinel, add in
//            binary64 in rank order, round, write `out`, reset the slots;
//            then drain, so the resets land before this workgroup's next
//            chunk can be seen by anyone (the credit of the two-shot LL128
//            kernel, with the reset in place of the zeroing).
template <int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(512) k_twoshot_sentinel(TwoShotArgs a) {
  WgState st = wg_begin(a.ctrl, a.timing);
  int r;
  uint32_t w;
  decode_role(blockIdx.x, N, a.placement, r, w);
  using E = Elem<kKind>;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint8_t* src = a.part[r];
  const uint64_t nbytes = a.n * (uint64_t)E::kBytes;
  const uint32_t chunk_vecs = (uint32_t)(((uint64_t)a.chunk_elems * E::kBytes + 15u) / 16u);
  const uint32_t slot_bytes = a.shard_cap * 16u;
  bool dead = (w >= a.slices);  // idle padding workgroup, or a poll timed out

  for (uint32_t c = 0; c < a.n_chunks && !__any((int)dead); ++c) {
    const uint64_t vbase = (uint64_t)c * chunk_vecs;  // first message vector of the chunk
    const uint64_t cbytes = min((uint64_t)a.chunk_elems * E::kBytes, nbytes - (uint64_t)c * a.chunk_elems * E::kBytes);
    const uint32_t nv = (uint32_t)((cbytes + 15u) / 16u);
    const uint32_t poff = (c & 1u) * a.parity_stride;

    // ---- produce
    for (int s = 0; s < N; ++s) {
      if (s == r || (uint32_t)r == a.drop_rank) continue;
      uint32_t o0 = (uint32_t)((uint64_t)s * nv / N), o1 = (uint32_t)((uint64_t)(s + 1) * nv / N);
      uint32_t s0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
      uint32_t s1 = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
      uint32_t slot = poff + (uint32_t)(s * N + r) * slot_bytes;
      for (uint32_t v = s0 + threadIdx.x; v < s1; v += blockDim.x) {
        u32x4 x = load_vec(src, vbase + v, nbytes);
        st16_stage<kLocal>(rs, slot + (v - o0) * 16u, sentinel_canon<kKind>(x));
      }
    }
    // ---- consume
    {
      uint32_t o0 = (uint32_t)((uint64_t)r * nv / N), o1 = (uint32_t)((uint64_t)(r + 1) * nv / N);
      uint32_t s0 = o0 + (uint32_t)((uint64_t)w * (o1 - o0) / a.slices);
      uint32_t s1 = o0 + (uint32_t)((uint64_t)(w + 1) * (o1 - o0) / a.slices);
      const uint32_t my = poff + (uint32_t)(r * N) * slot_bytes;
      for (uint32_t v = s0 + threadIdx.x; v < s1; v += blockDim.x) {
        u32x4 own = load_vec(src, vbase + v, nbytes);
        u32x4 d[N > 1 ? N - 1 : 1];
        Spin spin(a.spin_limit);
        bool ok = true;
        while (true) {
          bool all = true;
#pragma unroll
          for (int k = 0; k < N - 1; ++k) {
            int sender = k < r ? k : k + 1;
            d[k] = ld16_coh(rs, my + (uint32_t)sender * slot_bytes + (v - o0) * 16u);
            all &= sentinel_ready<kKind>(d[k]);
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
          break;
        }
        store_vec(a.out, vbase + v, nbytes, reduce_vec<kKind, N>(own, r, d));
        if (!a.keep) {
#pragma unroll
          for (int k = 0; k < N - 1; ++k) {
            int sender = k < r ? k : k + 1;
            st16_stage<kLocal>(rs, my + (uint32_t)sender * slot_bytes + (v - o0) * 16u,
                               u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu});
          }
        }
      }
    }
    drain_vm();
  }
  wg_end(a.ctrl, st, a.grid, a.timing);
}

// ---------------------------------------------------------------------------
// launchers (host side, one instantiation per (dtype, N))
// ---------------------------------------------------------------------------
template <int kKind, int N>
static hipError_t launch_n(const LaunchSpec& ls, hipStream_t stream) {
  dim3 grid(ls.grid), block(ls.threads);
  switch (ls.kernel) {
    case kKernOneShotLL:
      hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, N>), grid, block, 0, stream, ls.oneshot);
      break;
    case kKernOneShotSentinel:
      hipLaunchKernelGGL((k_oneshot<kWireSentinel, kKind, N>), grid, block, 0, stream, ls.oneshot);
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
    case kKernOneShotLL: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireLL, kKind, N>, threads, 0); break;
    case kKernOneShotSentinel: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireSentinel, kKind, N>, threads, 0); break;
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
