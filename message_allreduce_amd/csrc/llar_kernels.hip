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
//   Sentinel paragraph  -> k_oneshot<kWireSentinel>, k_twoshot_sentinel,
//                          k_twoshot_sentinel_hs, k_twoshot_sentinel_oc
//   bidirectional + double buffering paragraph -> the chunk loops of the
//                          two-shot kernels (LL128: parity = chunk & 1 with an
//                          implicit credit; Sentinel: B rotating buffers with
//                          a workgroup, slot or owner credit)
//   Two-shot LL128 paragraph -> k_twoshot_ll128
// The staging accesses use the primitives of include/llar_wire.h.  The
// ReduceScatter / AllGather kernels and the barrier ablation live in
// llar_multi.hip.
#include "llar_device.h"
#include "llar_internal.h"

namespace llar {

// ---------------------------------------------------------------------------
// tail-safe 16-byte vector access to the caller's buffers
// ---------------------------------------------------------------------------
// Only the last vector of a message can be partial; its elements (2 or 4
// bytes) are moved as halfwords.  Those paths are fully unrolled: a loop of
// loads or stores with a run-time trip count would leave the compiler unable
// to count outstanding memory operations, and every later wait in the
// kernel would then drain all of them (vmcnt(0)) instead of only the ones it
// needs, which serialises the software pipelines.
template <bool kStream = true>
__device__ __forceinline__ u32x4 load_vec(const uint8_t* p, uint64_t v, uint64_t nbytes) {
  const uint64_t off = v * 16u;
  if (off + 16u <= nbytes) {
    if constexpr (kStream) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + off));
    else return *reinterpret_cast<const u32x4*>(p + off);
  }
  u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
  for (uint32_t k = 0; k < 16u; k += 2u) {
    if (off + k < nbytes) x[k >> 2] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + off + k)) << ((k & 2u) * 8u);
  }
  return x;
}
// 8-byte units (the one-shot consumer's granularity)
__device__ __forceinline__ u32x2 load_unit(const uint8_t* p, uint64_t u, uint64_t nbytes) {
  const uint64_t off = u * 8u;
  if (off + 8u <= nbytes) return *reinterpret_cast<const u32x2*>(p + off);
  u32x2 x = {0u, 0u};
#pragma unroll
  for (uint32_t k = 0; k < 8u; k += 2u) {
    if (off + k < nbytes) x[k >> 2] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + off + k)) << ((k & 2u) * 8u);
  }
  return x;
}
__device__ __forceinline__ void store_unit(uint8_t* p, uint64_t u, uint64_t nbytes, u32x2 x) {
  const uint64_t off = u * 8u;
  if (off + 8u <= nbytes) {
    *reinterpret_cast<u32x2*>(p + off) = x;
    return;
  }
#pragma unroll
  for (uint32_t k = 0; k < 8u; k += 2u) {
    if (off + k < nbytes) *reinterpret_cast<uint16_t*>(p + off + k) = (uint16_t)(x[k >> 2] >> ((k & 2u) * 8u));
  }
}
// 4-byte half units (the one-shot consumer's granularity when each lane
// needs only one): the last one of a 16-bit message may hold one element
__device__ __forceinline__ uint32_t load_half(const uint8_t* p, uint64_t h, uint64_t nbytes) {
  const uint64_t off = h * 4u;
  if (off + 4u <= nbytes) return *reinterpret_cast<const uint32_t*>(p + off);
  return off < nbytes ? (uint32_t)*reinterpret_cast<const uint16_t*>(p + off) : 0u;
}
__device__ __forceinline__ void store_half(uint8_t* p, uint64_t h, uint64_t nbytes, uint32_t x) {
  const uint64_t off = h * 4u;
  if (off + 4u <= nbytes) {
    *reinterpret_cast<uint32_t*>(p + off) = x;
    return;
  }
  if (off < nbytes) *reinterpret_cast<uint16_t*>(p + off) = (uint16_t)x;
}
template <bool kStream = false>
__device__ __forceinline__ void store_vec(uint8_t* p, uint64_t v, uint64_t nbytes, u32x4 x) {
  const uint64_t off = v * 16u;
  if (off + 16u <= nbytes) {
    if constexpr (kStream) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p + off));
    else *reinterpret_cast<u32x4*>(p + off) = x;
    return;
  }
#pragma unroll
  for (uint32_t k = 0; k < 16u; k += 2u) {
    if (off + k < nbytes) *reinterpret_cast<uint16_t*>(p + off + k) = (uint16_t)(x[k >> 2] >> ((k & 2u) * 8u));
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

// The same with every rank's value staged: d[0..N-1] in rank order.
template <int kKind, int N>
__device__ __forceinline__ u32x4 reduce_all(const u32x4 (&d)[N]) {
  u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < Elem<kKind>::kPerVec; ++j) {
    double s = Elem<kKind>::dec(vec_elem<kKind>(d[0], j));
#pragma unroll
    for (int r = 1; r < N; ++r) s += Elem<kKind>::dec(vec_elem<kKind>(d[r], j));
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

// The same for a 4-byte half unit (one binary32 or two 16-bit elements).
template <int kKind, int N>
__device__ __forceinline__ uint32_t reduce_half(uint32_t own, const uint32_t (&d)[N > 1 ? N - 1 : 1]) {
  constexpr int kPer = 4 / Elem<kKind>::kBytes;
  uint32_t out = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    auto elem = [&](uint32_t v) -> uint32_t {
      if constexpr (Elem<kKind>::kBytes == 4) return v;
      else return (v >> (j * 16)) & 0xFFFFu;
    };
    double s = Elem<kKind>::dec(elem(own));
#pragma unroll
    for (int r = 1; r < N; ++r) s += Elem<kKind>::dec(elem(d[r - 1]));
    const uint32_t bits = Elem<kKind>::enc(s);
    if constexpr (Elem<kKind>::kBytes == 4) out = bits;
    else out |= (bits & 0xFFFFu) << (j * 16);
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

// kCopy (point-to-point, N = 2): rank 1 sends, rank 0 writes what arrived
// instead of a sum and reads no partial of its own.
// kSplit: rank 0's work on a slice is split over kSplit consumer workgroups
// (contiguous parts of the slice's units), so that fewer polls issue per CU;
// a slice then has N - 1 + kSplit workgroups.
template <int kWire, int kKind, int N, bool kLocal, bool kCopy = false, int kSplit = 1>
__global__ void __launch_bounds__(512) k_oneshot(OneShotArgs a) {
  const uint64_t t_entry = wall_ticks();
  static_assert(kSplit >= 1 && (!kCopy || kSplit == 1), "consumer split");
  constexpr uint32_t NR = (uint32_t)N + kSplit - 1u;  // workgroups per slice
  uint32_t rr, w;  // role in the slice: 0 .. kSplit-1 rank 0's parts, then ranks 1 .. N-1
  // local placement over the first xcd_span XCDs: workgroup b runs on XCD
  // b mod 8; slice w lives on XCD w mod span with its workgroups, and the
  // workgroups on the other XCDs idle (span 8: decode_role_t's placement)
  const uint32_t span = a.xcd_span;
  bool off_span = false;
  if constexpr (kLocal) {
    const uint32_t x = blockIdx.x & 7u, q = blockIdx.x >> 3;
    rr = q % NR;
    w = (q / NR) * span + x;
    off_span = x >= span;
  } else {
    rr = blockIdx.x % NR;
    w = blockIdx.x / NR;
  }
  const int r = rr < (uint32_t)kSplit ? 0 : (int)(rr - kSplit + 1u);
  const uint32_t part = rr < (uint32_t)kSplit ? rr : 0u;
  // every kernel argument used below, requested at entry as one batch
  const uint8_t* const src = a.part[r];
  uint8_t* const out = a.out;
  uint8_t* const stage = a.stage;
  Ctrl* const ctrl = a.ctrl;
  uint64_t* const trace = a.trace;
  const uint64_t nbytes = a.nbytes, spin_limit = a.spin_limit;
  const uint32_t slices = a.slices, vq = a.vq, vr = a.vr, stage_bytes = a.stage_bytes;
  const uint32_t parity_stride = a.parity_stride, rank_stride = a.rank_stride, grid = a.grid;
  const uint32_t timing = a.timing, keep = a.keep, drop_rank = a.drop_rank, host_epoch = a.host_epoch;
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(out), "s"(stage), "s"(ctrl), "s"(trace), "s"(nbytes), "s"(spin_limit),
                        "s"(slices), "s"(vq), "s"(vr), "s"(stage_bytes), "s"(parity_stride), "s"(rank_stride),
                        "s"(grid), "s"(timing), "s"(keep), "s"(drop_rank), "s"(host_epoch));
  const bool idle = off_span || (w >= slices);
  // slice w: 16-byte vectors [v0, v1) for producers, 8-byte units [2 v0, 2 v1)
  // for the consumer (one LL line, or half a Sentinel slot, per lane)
  const uint32_t v0 = idle ? 0u : w * vq + min(w, vr);
  const uint32_t v1 = idle ? 0u : v0 + vq + (w < vr ? 1u : 0u);
  const bool producer = (r != 0) && !idle && (uint32_t)r != drop_rank;
  const bool consumer = (r == 0) && !idle;
  // this consumer workgroup's units: part `part` of the slice's [2 v0, 2 v1)
  const uint32_t ups = (2u * (v1 - v0) + kSplit - 1u) / kSplit;
  const uint32_t u_lo = min(2u * v0 + part * ups, 2u * v1), u_hi = min(u_lo + ups, 2u * v1);
  // LL: when every 4-byte half of this consumer's units has a lane of its
  // own, each lane takes a half (the LL half line {data, epoch}): the same
  // polls spread over twice the lanes, and half the binary64 reduce per lane
  // on the path's critical end (16 KiB x 8 bf16, device span 1.47-1.51 ->
  // 1.39-1.46 us on MI355X).  Sentinel keeps 8-byte units: 4-byte quarter
  // slots measured slower there (128 KiB x 8 fp16, 2.29 -> 2.37 us).
  // Uniform per workgroup.
  const bool halves = kWire == kWireLL && 2u * (u_hi - u_lo) <= blockDim.x;
  // the first input of this thread is requested before anything else
  u32x4 first_vec = {0u, 0u, 0u, 0u};
  u32x2 first_unit = {0u, 0u};
  if (producer && v0 + threadIdx.x < v1) first_vec = load_vec<false>(src, v0 + threadIdx.x, nbytes);
  if (!kCopy && consumer) {
    if (halves) {
      if (2u * u_lo + threadIdx.x < 2u * u_hi) first_unit[0] = load_half(src, 2u * u_lo + threadIdx.x, nbytes);
    } else if (u_lo + threadIdx.x < u_hi) {
      first_unit = load_unit(src, u_lo + threadIdx.x, nbytes);
    }
  }
  WgState st = wg_begin(ctrl, host_epoch, timing, idle);
  if (trace && threadIdx.x == 0) trace[blockIdx.x * kTraceWords + 0] = t_entry;
  trace_at(trace, 1, false);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(stage, stage_bytes);
  const uint32_t e = st.epoch;
  const uint32_t par_off = (e & 1u) * parity_stride;
  constexpr uint32_t kVecStage = (kWire == kWireLL) ? 32u : 16u;
  if (producer) {
    const uint32_t base = par_off + (uint32_t)(r - 1) * rank_stride;
    for (uint32_t v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
      u32x4 x = (v == v0 + threadIdx.x) ? first_vec : load_vec<false>(src, v, nbytes);
      if (v == v0) trace_at(trace, 2, true);
      uint32_t off = base + v * kVecStage;
      if constexpr (kWire == kWireLL) llar_wire::ll_put16<scope_of(kLocal)>(rs, off, x, e);
      else llar_wire::sentinel_put<Elem<kKind>::kBytes, scope_of(kLocal)>(rs, off, x);
      if (v == v0) trace_at(trace, 3, true);
    }
  } else if (consumer && halves) {
    // (LL only) one 4-byte half unit per lane: half h of unit u = h / 2 is
    // the half line {data, epoch} at u * 16 + (h % 2) * 8
    const uint32_t h = 2u * u_lo + threadIdx.x;
    if (h < 2u * u_hi) {
      const uint32_t own = kCopy ? 0u : first_unit[0];
      if (h == 2u * u_lo) trace_at(trace, 2, true);
      const uint32_t off_h = (h >> 1) * 16u + (h & 1u) * 8u;
      // With two ranks, two poll passes in flight, issued half a round trip
      // apart: a pass is re-issued as soon as its answer is checked, so the
      // slot is sampled about every half round trip and an arrival is seen
      // sooner than with one pass at a time (128 B x 2 fp32, device span
      // 0.76 -> 0.64-0.68 us).  With more ranks the doubled poll traffic
      // slows the senders' stores more than it saves (64 KiB x 8 bf16,
      // 2.1 -> 2.4 us), so one pass at a time.  A slot that is ready stays
      // ready for the rest of the call (its line carries this call's epoch),
      // so the pass that first finds every slot ready supplies the data.
      constexpr bool kTwoPass = N <= 2;
      using PT = u32x2;
      PT pa[N > 1 ? N - 1 : 1], pb[N > 1 ? N - 1 : 1];
      auto issue = [&](PT (&q)[N > 1 ? N - 1 : 1]) {
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          q[k] = llar_wire::ld8_coh(rs, par_off + (uint32_t)k * rank_stride + off_h);
        }
      };
      auto ready = [&](const PT (&q)[N > 1 ? N - 1 : 1]) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) all &= q[k][1] == e;
        return all;
      };
      uint32_t d[N > 1 ? N - 1 : 1];
      auto take = [&](const PT (&q)[N > 1 ? N - 1 : 1]) {
#pragma unroll
        for (int k = 0; k < N - 1; ++k) d[k] = q[k][0];
      };
      bool ok = true;
      if constexpr (kTwoPass) {
        llar_wire::PollT<0> spin(spin_limit);
        issue(pa);
        __builtin_amdgcn_s_sleep(2);  // about half an L2 round trip
        while (true) {
          issue(pb);
          if (ready(pa)) {
            take(pa);
            break;
          }
          issue(pa);
          if (ready(pb)) {
            take(pb);
            break;
          }
          if (spin.expired()) {
            raise_status(ctrl, kStatusTimeout);
            ok = false;
            break;
          }
        }
      } else {
        // no back-off between passes: a pass is a lane's N - 1 8-byte loads,
        // and re-issuing it at once sees an arrival sooner (16 KiB x 8 bf16,
        // device span 1.35-1.39 -> 1.31-1.35 us)
        llar_wire::PollT<0> spin(spin_limit);
        while (true) {
          issue(pa);
          if (ready(pa)) {
            take(pa);
            break;
          }
          if (spin.expired()) {
            raise_status(ctrl, kStatusTimeout);
            ok = false;
            break;
          }
        }
      }
      if (ok) {
        if (h == 2u * u_lo) trace_at(trace, 3, false);
        if constexpr (kCopy) store_half(out, h, nbytes, d[0]);
        else store_half(out, h, nbytes, reduce_half<kKind, N>(own, d));
        if (h == 2u * u_lo) trace_at(trace, 4, true);
      }
    }
  } else if (consumer) {
    constexpr uint32_t kUnitStage = (kWire == kWireLL) ? 16u : 8u;
    bool dead = false;  // set after a timeout: stop waiting for anything else
    for (uint32_t u = u_lo + threadIdx.x; u < u_hi && !dead; u += blockDim.x) {
      u32x2 own = {0u, 0u};
      if constexpr (!kCopy) own = (u == u_lo + threadIdx.x) ? first_unit : load_unit(src, u, nbytes);
      if (u == u_lo) trace_at(trace, 2, true);
      // A slot that is ready stays ready for the rest of the call (LL lines
      // carry this call's epoch; a filled Sentinel slot is only reset by this
      // thread), so reload every slot until one pass sees all of them ready
      // and reduce from that pass.
      u32x2 d[N > 1 ? N - 1 : 1];
      Spin spin(spin_limit);
      bool ok = true;
      while (true) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          uint32_t off = par_off + (uint32_t)k * rank_stride + u * kUnitStage;
          if constexpr (kWire == kWireLL) all &= llar_wire::ll_try(rs, off, e, d[k]);
          else all &= llar_wire::sentinel_try8<Elem<kKind>::kBytes>(rs, off, d[k]);
        }
        if (all) break;
        if (spin.expired()) {
          raise_status(ctrl, kStatusTimeout);
          ok = false;
          break;
        }
      }
      if (!ok) {
        dead = true;
        continue;
      }
      if (u == u_lo) trace_at(trace, 3, false);
      if constexpr (kCopy) store_unit(out, u, nbytes, d[0]);
      else store_unit(out, u, nbytes, reduce_unit<kKind, N>(own, d));
      if (u == u_lo) trace_at(trace, 4, true);
      if constexpr (kWire == kWireSentinel) {
        if (!keep) {
#pragma unroll
          for (int k = 0; k < N - 1; ++k)
            llar_wire::sentinel_reset8<scope_of(kLocal)>(rs, par_off + (uint32_t)k * rank_stride + u * 8u);
        }
      }
    }
  }
  wg_end(ctrl, st, host_epoch, grid, timing, idle);
  if (trace && threadIdx.x == 0) {
    trace[blockIdx.x * kTraceWords + 5] = wall_ticks();
    trace[blockIdx.x * kTraceWords + 6] = (uint64_t)xcc_id() | ((uint64_t)r << 8) | ((uint64_t)w << 16);
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
  // every kernel argument, requested at entry as one batch: the partial of
  // this workgroup's rank under both placements, the placement picks one
  int r_l, r_s;
  uint32_t w_l, w_s;
  decode_role_t<true, N>(blockIdx.x, r_l, w_l);
  decode_role_t<false, N>(blockIdx.x, r_s, w_s);
  const uint8_t* const src_l = a.part[r_l];
  const uint8_t* const src_s = a.part[r_s];
  LLAR_UNIFORM_AT_ENTRY("s"(src_l), "s"(src_s), "s"(a.out), "s"(a.stage), "s"(a.ctrl), "s"(a.n), "s"(a.spin_limit),
                        "s"(a.chunk_elems), "s"(a.n_chunks), "s"(a.stage_bytes), "s"(a.parity_stride), "s"(a.grid),
                        "s"(a.slices), "s"(a.placement), "s"(a.timing), "s"(a.keep), "s"(a.drop_rank),
                        "s"(a.host_epoch), "s"(a.threads), "s"(a.slices_rcp));
  const bool local = (a.placement == kPlaceLocal);
  const int r = local ? r_l : r_s;
  const uint32_t w = local ? w_l : w_s;
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  constexpr int kSlots = kAcc16 ? 64 : 32;
  constexpr int K = kSlots - 1;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  // the wave index as a scalar (the same in every lane), and the wave count,
  // a power of two (the host launches 64 to 1024 threads)
  const uint32_t lane = threadIdx.x & 63u, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t n_waves = a.threads >> 6, wave_mask = n_waves - 1u;
  const uint8_t* src = local ? src_l : src_s;
  // flag value N in the staging type
  uint32_t flag_full;
  if constexpr (!kAcc16) flag_full = __float_as_uint((float)N);
  else flag_full = E::from_f32((float)N);
  bool dead = idle;  // idle padding workgroup, or a poll timed out
  // Lines are partitioned by the nominal chunk (not a chunk's length): a
  // line must belong to the same (owner, slice) in every chunk, or the
  // implicit credit of one slice would release a line another slice has not
  // consumed yet.  Elements past the message end are masked.  Owner s holds
  // lines [s L / N, (s+1) L / N), split evenly into the slices; computed once
  // (32-bit: L < 2^19 lines and w < 64).
  const uint32_t L = (a.chunk_elems + K - 1) / K;
  uint32_t sl0[N], sl1[N];
#pragma unroll
  for (int s = 0; s < N; ++s) {
    const uint32_t o0 = (uint32_t)s * L / (uint32_t)N, o1 = ((uint32_t)s + 1u) * L / (uint32_t)N;
    // x / slices as a multiply by the host's reciprocal where it is exact
    // (a software division on this path cost about 0.3 us of issue time)
    auto div_slices = [&](uint32_t x) -> uint32_t { return a.slices_rcp ? __umulhi(x, a.slices_rcp) : x / a.slices; };
    sl0[s] = o0 + div_slices(w * (o1 - o0));
    sl1[s] = o0 + div_slices((w + 1u) * (o1 - o0));
  }

  for (uint32_t c = 0; c < a.n_chunks && !dead; ++c) {
    const uint64_t cbase = (uint64_t)c * a.chunk_elems;
    const uint32_t len = (uint32_t)min((uint64_t)a.chunk_elems, a.n - cbase);
    // lines that hold data of this chunk: producers flag and consumers poll
    // only these (both sides agree, and a line past them stays zero)
    const uint32_t Lr = (len + K - 1) / K;
    const uint32_t poff = (c & 1u) * a.parity_stride;

    // ---- produce: data atomics for every owner's slice w.  An owner's
    // slice is often a single block of 8 lines, so owner s's blocks start at
    // wave (waves - s) mod waves: the waves of the workgroup add into
    // different owners' lines at once instead of all owners falling to wave 0
    const bool silent = ((uint32_t)r == a.drop_rank);
    for (int s = 0; s < N && !silent; ++s) {
      const uint32_t l0 = sl0[s], l1 = min(sl1[s], Lr);
      for (uint32_t lb = l0 + ((wave + (uint32_t)s) & wave_mask) * 8u; lb < l1; lb += n_waves * 8u) {
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
            llar_wire::ll128_add(reinterpret_cast<float*>(a.stage + off), val);
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
            llar_wire::ll128_add2<kKind == kKindBF16>(a.stage + off, s16x2{(short)lo, (short)hi});
          }
        }
      }
    }
    // data of this wave acknowledged before any of its flags; a line is
    // flagged by the wave that added its data (the same block assignment)
    drain_vm();
    for (int s = 0; s < N && !silent; ++s) {
      const uint32_t l0 = sl0[s], l1 = min(sl1[s], Lr);
      for (uint32_t lb = l0 + ((wave + (uint32_t)s) & wave_mask) * 8u; lb < l1; lb += n_waves * 8u) {
        uint32_t line = lb + lane;
        if (lane < 8u && line < l1) {
          uint32_t off = poff + line * 128u;
          if constexpr (!kAcc16) {
            llar_wire::ll128_flag(reinterpret_cast<float*>(a.stage + off));
          } else {
            llar_wire::ll128_flag2<kKind == kKindBF16>(a.stage + off, E::from_f32(1.0f));
          }
        }
      }
    }

    // ---- consume owner r's slice w: 8 lanes per line
    {
      // owner r's slice w (a runtime index into the bounds: selected, not
      // indexed, so that the arrays stay in registers)
      uint32_t l0 = sl0[0], l1 = sl1[0];
#pragma unroll
      for (int s = 1; s < N; ++s) {
        l0 = (s == r) ? sl0[s] : l0;
        l1 = (s == r) ? sl1[s] : l1;
      }
      l1 = min(l1, Lr);
      const uint32_t grp = lane >> 3, j = lane & 7u;
      for (uint32_t lb = l0 + wave * 8u; lb < l1; lb += n_waves * 8u) {
        uint32_t line = lb + grp;
        if (line >= l1) continue;
        uint32_t loff = poff + line * 128u;
        Spin spin(a.spin_limit);
        if (!llar_wire::ll128_wait<kAcc16 != 0>(rs, loff, flag_full, spin)) {
          raise_status(a.ctrl, kStatusTimeout);
          dead = true;
          break;
        }
        // 16-bit staging: read and zero the line's 16 bytes in one exchange
        // (16 KiB x 4 bf16, device 4.54 -> 4.15 us, per call 5.71 -> 5.36 on
        // MI355X); binary32 staging reads, then stores zeros (the exchange
        // measured 0.05-0.15 us slower there); kept staging is only read
        const bool take = kAcc16 && !a.keep;
        const u32x4 v = take ? llar_wire::ll128_take16(a.stage + loff + j * 16u) : llar_wire::ll128_read16(rs, loff + j * 16u);
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
        if (!take && !a.keep) llar_wire::ll128_reset16(rs, loff + j * 16u);
      }
    }
    // every wave's lines are zeroed (its exchanges have returned, its zeroing
    // stores are acknowledged) before any wave of this workgroup contributes
    // to the next chunk (a workgroup-uniform exit too)
    drain_vm();
    dead = __syncthreads_or((int)dead) != 0;
  }
  wg_end(a.ctrl, st, a.host_epoch, a.grid, a.timing, idle);
}

// ---------------------------------------------------------------------------
// two-shot LL128 atomic, chunked, B buffers, producer and consumer waves
// ---------------------------------------------------------------------------
// The same lines, owners, slices and flag counting as k_twoshot_ll128, with
// the work of a workgroup (r, w) split by role so that several chunks are in
// flight at once instead of one chain of atomics, drain, flags, polls and
// zeroing per chunk:
//   producer waves: whole chunks dealt round-robin (wave p takes chunks p,
//            p + n_prod, ...).  For its chunk c a wave adds rank r's elements
//            into slice w of every owner's lines in buffer c % B, drains,
//            then adds 1.0 to each of those lines' slot 0 -- once this
//            workgroup's consumers have finished every chunk below c - lag;
//   consumer waves: whole chunks dealt round-robin as well (wave q takes
//            chunks q, q + n_cons, ...): poll owner r's slice w lines of chunk
//            c until slot 0 reads N, round, write `out`, zero the lines;
//            drain (the zeroing is performed), then count the chunk in LDS.
// Credit (the page's implicit one, as for the pipelined Sentinel): a
// producer adds chunk c after this workgroup's consumers finished chunk
// c - 1 - lag; they finished it only after every rank's slice-w producer
// flagged it, which each did only after its own consumers had finished chunk
// c - 2 - 2 lag and their zeroing was performed.  With B >= 2 lag + 2
// buffers that covers chunk c - B, the previous user of chunk c's buffer.
// The consumer of chunk c - B is the consumer of chunk c (the host makes
// n_cons divide B), so a wave never polls a buffer that still holds the
// previous chunk's full lines: it zeroed them itself and drained before.
// The host keeps every owner slice of a full chunk non-empty (the credit
// travels through lines of this workgroup's own).
template <int kKind, int kAcc16, int N>
__global__ void __launch_bounds__(1024) k_twoshot_ll128_ws(TwoShotArgs a) {
  int r_l, r_s;
  uint32_t w_l, w_s;
  decode_role_t<true, N>(blockIdx.x, r_l, w_l);
  decode_role_t<false, N>(blockIdx.x, r_s, w_s);
  const uint8_t* const src_l = a.part[r_l];
  const uint8_t* const src_s = a.part[r_s];
  LLAR_UNIFORM_AT_ENTRY("s"(src_l), "s"(src_s), "s"(a.out), "s"(a.stage), "s"(a.ctrl), "s"(a.n), "s"(a.spin_limit),
                        "s"(a.chunk_elems), "s"(a.n_chunks), "s"(a.stage_bytes), "s"(a.parity_stride), "s"(a.grid),
                        "s"(a.slices), "s"(a.placement), "s"(a.timing), "s"(a.keep), "s"(a.drop_rank),
                        "s"(a.host_epoch), "s"(a.n_buffers), "s"(a.cons_waves), "s"(a.threads));
  const bool local = (a.placement == kPlaceLocal);
  const int r = local ? r_l : r_s;
  const uint32_t w = local ? w_l : w_s;
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  constexpr int kSlots = kAcc16 ? 64 : 32;
  constexpr int K = kSlots - 1;
  __shared__ uint32_t s_cnt[16];  // per consumer wave: chunks it has finished
  __shared__ uint32_t s_dead;     // some wave's poll expired: everyone stops
  if (threadIdx.x < 16) s_cnt[threadIdx.x] = 0u;
  if (threadIdx.x == 0) s_dead = 0u;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, n_waves = a.threads >> 6;
  const uint32_t n_cons = a.cons_waves, n_prod = n_waves - n_cons;
  const uint32_t n_buf = a.n_buffers, lag = n_buf / 2u - 1u;
  const uint8_t* src = local ? src_l : src_s;
  uint32_t flag_full;
  if constexpr (!kAcc16) flag_full = __float_as_uint((float)N);
  else flag_full = E::from_f32((float)N);
  // lines of the nominal chunk, owners' ranges and this slice of each (as in
  // k_twoshot_ll128: a line keeps its (owner, slice) in every chunk)
  const uint32_t L = (a.chunk_elems + K - 1) / K;
  uint32_t sl0[N], sl1[N];
#pragma unroll
  for (int s = 0; s < N; ++s) {
    const uint32_t o0 = (uint32_t)s * L / (uint32_t)N, o1 = ((uint32_t)s + 1u) * L / (uint32_t)N;
    sl0[s] = o0 + w * (o1 - o0) / a.slices;
    sl1[s] = o0 + (w + 1u) * (o1 - o0) / a.slices;
  }
  auto any_dead = [&]() { return __hip_atomic_load(&s_dead, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0u; };
  auto die = [&]() {
    raise_status(a.ctrl, kStatusTimeout);
    __hip_atomic_store(&s_dead, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // every chunk below the returned one has been finished by this
  // workgroup's consumers (consumer wave q has finished chunks q, q + n_cons,
  // ..., below q + s_cnt[q] * n_cons)
  auto consumed_below = [&]() {
    uint32_t f = ~0u;
    for (uint32_t q = 0; q < n_cons; ++q)
      f = min(f, q + __hip_atomic_load(&s_cnt[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) * n_cons);
    return f;
  };

  if (idle) {
    // padding workgroup of the local placement: nothing to do
  } else if (wave < n_prod) {
    // ---------------- producer waves
    const bool silent = ((uint32_t)r == a.drop_rank);
    // the slice bounds in this rank's owner order r, r + 1, ... (mod N),
    // chosen with selects so that the arrays stay in registers
    uint32_t rsl0[N], rsl1[N];
#pragma unroll
    for (int t = 0; t < N; ++t) {
      rsl0[t] = sl0[0];
      rsl1[t] = sl1[0];
#pragma unroll
      for (int s = 1; s < N; ++s) {
        const bool pick = ((r + t) % N) == s;
        rsl0[t] = pick ? sl0[s] : rsl0[t];
        rsl1[t] = pick ? sl1[s] : rsl1[t];
      }
    }
    for (uint32_t c = wave; c < a.n_chunks && !silent; c += n_prod) {
      const uint64_t cbase = (uint64_t)c * a.chunk_elems;
      const uint32_t len = (uint32_t)min((uint64_t)a.chunk_elems, a.n - cbase);
      const uint32_t Lr = (len + K - 1) / K;
      const uint32_t poff = (c % n_buf) * a.parity_stride;
      if (c > lag) {
        Spin spin(a.spin_limit);
        bool ok = true;
        while (consumed_below() + lag < c) {
          if (any_dead()) {
            ok = false;
            break;
          }
          if (spin.expired()) {
            die();
            ok = false;
            break;
          }
        }
        if (!ok) break;
      }
      // This chunk's lines of slice w, every owner's in turn starting with
      // owner r (so that the N ranks add into different owners' lines at
      // the same moment instead of all into owner 0's, then owner 1's, ...),
      // numbered 0 .. total-1: the t-th owner in that order holds local
      // lines [pre[t], pre[t+1]).  A wave instruction covers two consecutive
      // local lines (64 dwords) whichever owners they belong to, so a slice
      // of a few lines per owner costs a few instructions, not four per
      // owner.
      uint32_t pre[N + 1];
      pre[0] = 0u;
#pragma unroll
      for (int t = 0; t < N; ++t) {
        const uint32_t l1 = min(rsl1[t], Lr);
        pre[t + 1] = pre[t] + (l1 > rsl0[t] ? l1 - rsl0[t] : 0u);
      }
      const uint32_t total = pre[N];
      // line of local line i (i < total): the last owner whose range starts
      // at or before i holds it (empty owners never are the last such)
      auto line_of = [&](uint32_t i) {
        uint32_t line = 0u;
#pragma unroll
        for (int t = 0; t < N; ++t) line = (i >= pre[t]) ? rsl0[t] + (i - pre[t]) : line;
        return line;
      };
      // data: 8 local lines (four wave instructions) at a time, loads first
      for (uint32_t i0 = 0; i0 < total; i0 += 8u) {
        float fv[4];
        s16x2 hv[4];
        bool on[4];
        uint32_t off[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t d = (uint32_t)k * 64u + lane;  // dword of the 8-line block
          const uint32_t i = i0 + d / 32u, q = d % 32u;
          const uint32_t line = line_of(i);
          on[k] = i < total;
          off[k] = poff + line * 128u + q * 4u;
          if constexpr (!kAcc16) {
            const uint32_t e_idx = line * K + q - 1u;
            on[k] = on[k] && q != 0u && e_idx < len;
            if constexpr (E::kBytes == 4) fv[k] = on[k] ? __uint_as_float(reinterpret_cast<const uint32_t*>(src)[cbase + e_idx]) : 0.f;
            else fv[k] = on[k] ? E::to_f32(reinterpret_cast<const uint16_t*>(src)[cbase + e_idx]) : 0.f;
          } else {
            // two 16-bit slots per dword: slots 2q and 2q + 1
            const uint32_t e0 = line * K + 2u * q - 1u, e1 = line * K + 2u * q;
            const uint32_t lo = (on[k] && q != 0u && e0 < len) ? reinterpret_cast<const uint16_t*>(src)[cbase + e0] : 0u;
            const uint32_t hi = (on[k] && e1 < len) ? reinterpret_cast<const uint16_t*>(src)[cbase + e1] : 0u;
            on[k] = on[k] && (lo | hi) != 0u;  // nothing to add (both +0)
            hv[k] = s16x2{(short)lo, (short)hi};
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (!on[k]) continue;
          if constexpr (!kAcc16) llar_wire::ll128_add(reinterpret_cast<float*>(a.stage + off[k]), fv[k]);
          else llar_wire::ll128_add2<kKind == kKindBF16>(a.stage + off[k], hv[k]);
        }
      }
      // the wave's data acknowledged before any of its flags
      drain_vm();
      for (uint32_t i = lane; i < total; i += 64u) {
        const uint32_t off = poff + line_of(i) * 128u;
        if constexpr (!kAcc16) llar_wire::ll128_flag(reinterpret_cast<float*>(a.stage + off));
        else llar_wire::ll128_flag2<kKind == kKindBF16>(a.stage + off, E::from_f32(1.0f));
      }
    }
  } else {
    // ---------------- consumer waves: owner r's slice w, 8 lanes per line
    const uint32_t cw = wave - n_prod;
    uint32_t l0 = sl0[0], l1 = sl1[0];
#pragma unroll
    for (int s = 1; s < N; ++s) {
      l0 = (s == r) ? sl0[s] : l0;
      l1 = (s == r) ? sl1[s] : l1;
    }
    const uint32_t grp = lane >> 3, j = lane & 7u;
    uint32_t done = 0u;
    bool dead = false;
    for (uint32_t c = cw; c < a.n_chunks && !dead; c += n_cons) {
      const uint64_t cbase = (uint64_t)c * a.chunk_elems;
      const uint32_t len = (uint32_t)min((uint64_t)a.chunk_elems, a.n - cbase);
      const uint32_t l1c = min(l1, (len + K - 1) / K);
      const uint32_t poff = (c % n_buf) * a.parity_stride;
      for (uint32_t lb = l0; lb < l1c && !dead; lb += 8u) {
        const uint32_t line = lb + grp;
        const bool mine = line < l1c;
        const uint32_t loff = poff + line * 128u;
        if (mine) {
          Spin spin(a.spin_limit);
          while (true) {
            uint32_t f = ld4_coh(rs, loff);
            if constexpr (kAcc16 != 0) f &= 0xFFFFu;
            if (f == flag_full) break;
            if (any_dead()) {
              dead = true;
              break;
            }
            if (spin.expired()) {
              die();
              dead = true;
              break;
            }
          }
        }
        dead = __any((int)dead) != 0;
        if (dead || !mine) continue;
        u32x4 v = llar_wire::ll128_read16(rs, loff + j * 16u);
        if constexpr (!kAcc16) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t q = j * 4u + (uint32_t)t;
            const uint32_t e_idx = line * K + q - 1u;
            if (q == 0u || e_idx >= len) continue;
            if constexpr (E::kBytes == 4) reinterpret_cast<uint32_t*>(a.out)[cbase + e_idx] = v[t];
            else reinterpret_cast<uint16_t*>(a.out)[cbase + e_idx] = (uint16_t)E::from_f32(__uint_as_float(v[t]));
          }
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t q = j * 8u + (uint32_t)t;
            const uint32_t e_idx = line * K + q - 1u;
            if (q == 0u || e_idx >= len) continue;
            reinterpret_cast<uint16_t*>(a.out)[cbase + e_idx] = (uint16_t)(v[t >> 1] >> ((t & 1) * 16));
          }
        }
        if (!a.keep) llar_wire::ll128_reset16(rs, loff + j * 16u);
      }
      if (dead) break;
      // the zeroing is performed before the producers may count on it
      drain_vm();
      ++done;
      if (lane == 0) __hip_atomic_store(&s_cnt[cw], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
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
//   producer waves, in PG groups (group p takes chunks p, p + PG, ...): for
//            its chunk c, request rank r's vectors of slice (s, w) for every
//            owner s != r, then -- once this workgroup's consumer waves have
//            finished chunks 0..c-1-lag -- store them, sentinel-canonicalised,
//            into [c % B][s][r].  The loads are issued before the credit
//            wait, so HBM reads overlap it;
//   consumer waves, in G groups (group g takes chunks g, g + G, ...): for
//            each vector of slice (r, w) of its chunk c, poll the N-1 slots
//            [c % B][r][*], add the own partial (requested one chunk early)
//            and the N-1 staged ones in binary64 in rank order, round, write
//            `out`, reset the slots; drain (the resets are performed), then
//            count the chunk in LDS for the producer waves.
// The credit: a producer stores chunk c only after this workgroup's
// consumers finished every chunk up to c-1-lag.  They finished it only
// after every peer's producer stored chunk c-1-lag, which each did only
// after its own consumers had finished chunk c-2-2*lag and drained those
// resets; with B >= 2*lag + 2 buffers that covers chunk c-B, the previous
// user of chunk c's buffer.  G divides B, so the group that polls chunk c
// reset chunk c-B's slots itself before (a poll never finds an old chunk's
// full slot).  With G > 1 up to G chunks are consumed at once, each group's
// poll, reduce, reset and drain overlapping the others'; with PG > 1 chunks
// may be stored out of order, which the argument above does not use.
template <int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(512) k_twoshot_sentinel(TwoShotArgs a) {
  constexpr int kU = 2;   // vectors per producer lane per owner per batch
  constexpr int kUc = 2;  // vectors per consumer lane per batch
  int r;
  uint32_t w;
  decode_role_t<kLocal, N>(blockIdx.x, r, w);
  // every kernel argument, requested at entry as one batch
  const uint8_t* src = a.part[r];
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(a.out), "s"(a.stage), "s"(a.ctrl), "s"(a.n), "s"(a.spin_limit),
                        "s"(a.chunk_elems), "s"(a.n_chunks), "s"(a.stage_bytes), "s"(a.parity_stride),
                        "s"(a.shard_cap), "s"(a.n_buffers), "s"(a.grid), "s"(a.slices), "s"(a.timing), "s"(a.keep),
                        "s"(a.drop_rank), "s"(a.host_epoch), "s"(a.trace), "s"(a.cons_groups), "s"(a.prod_groups), "s"(a.threads));
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint64_t nbytes = a.n * (uint64_t)E::kBytes;
  const uint32_t chunk_vecs = (uint32_t)(((uint64_t)a.chunk_elems * E::kBytes + 15u) / 16u);
  const uint64_t total_vecs = (nbytes + 15u) / 16u;
  const uint64_t full_vecs = nbytes / 16u;          // whole vectors of the message
  const bool has_tail = (nbytes % 16u) != 0u;       // vector full_vecs is partial
  const uint32_t slot_bytes = a.shard_cap * 16u;
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, n_waves = a.threads >> 6;
  const uint32_t n_prod = n_waves / 2, n_cons = n_waves - n_prod;
  const uint32_t n_buf = a.n_buffers;
  const uint32_t lag = n_buf / 2u - 1u;
  // consumer groups: G divides both the consumer waves and B; producer
  // groups: PG divides the producer waves (host-checked)
  const uint32_t n_grp = a.cons_groups, gw = n_cons / n_grp;
  const uint32_t n_pgrp = a.prod_groups, pgw = n_prod / n_pgrp;
  // per consumer wave: the next chunk of its group it has not finished (its
  // group's chunks below are done); a group starts at its first chunk
  __shared__ uint32_t s_done[8];
  if (threadIdx.x < n_cons) s_done[threadIdx.x] = threadIdx.x / gw;
  __syncthreads();
  // the partition uses the nominal chunk so that a slot keeps its (owner,
  // slice) in every chunk; vectors past the end of the message are masked
  const uint32_t nv = chunk_vecs;
  bool dead = idle;
  uint64_t* tr = (a.trace && !idle) ? a.trace + (uint64_t)blockIdx.x * kPipeTraceWords : nullptr;
  auto stamp = [&](int kind, uint32_t c) {
    if (tr && lane == 0 && c < (uint32_t)kPipeTraceChunks) tr[kind * kPipeTraceChunks + c] = wall_ticks();
  };

  if (wave < n_prod) {
    // ---------------- producer waves, in PG groups (group p stores chunks
    // p, p + PG, ...: PG chunks' loads in flight at once)
    const uint32_t pg = wave / pgw, pgi = wave % pgw;  // group, and wave within it
    const uint32_t pl = pgi * 64u + lane, PL = pgw * 64u;
    const bool silent = ((uint32_t)r == a.drop_rank);
    // slice w of every other owner's shard, the same in every chunk: owner s
    // holds vectors [s nv / N, (s+1) nv / N) of a chunk, split evenly into
    // the slices (32-bit: nv < 2^18 vectors and w < 64)
    uint32_t own0[N > 1 ? N - 1 : 1], sl0[N > 1 ? N - 1 : 1], sl1[N > 1 ? N - 1 : 1];
#pragma unroll
    for (int k = 0; k < N - 1; ++k) {
      const uint32_t s = (uint32_t)(k < r ? k : k + 1);
      const uint32_t o0 = s * nv / (uint32_t)N, o1 = (s + 1u) * nv / (uint32_t)N;
      own0[k] = o0;
      sl0[k] = o0 + w * (o1 - o0) / a.slices;
      sl1[k] = o0 + (w + 1u) * (o1 - o0) / a.slices;
    }
    for (uint32_t c = pg; c < a.n_chunks && !dead; c += n_pgrp) {
      const uint64_t vbase = (uint64_t)c * chunk_vecs;
      // vectors of this chunk that exist; the partition below uses the
      // nominal chunk so that a slot keeps its (owner, slice) in every chunk
      const uint32_t nv_real = (uint32_t)min((uint64_t)chunk_vecs, total_vecs - vbase);
      // whole vectors of this chunk: the loads below read them through a
      // buffer descriptor; the partial last vector of a message, if any, is
      // staged after the chunk loop
      const uint32_t nv_whole = (uint32_t)min((uint64_t)chunk_vecs, full_vecs > vbase ? full_vecs - vbase : 0u);
      const __amdgpu_buffer_rsrc_t rin = make_rsrc(src + vbase * 16u, nv_whole * 16u);
      const uint32_t nv = chunk_vecs;
      const uint32_t poff = (c % n_buf) * a.parity_stride;
      const uint32_t span = (nv / N + 1u) / a.slices + 2u;  // longest (owner, slice) range
      for (uint32_t b0 = 0; b0 < span && !dead; b0 += kU * PL) {
        u32x4 x[N > 1 ? N - 1 : 1][kU];
        uint32_t vo[N > 1 ? N - 1 : 1][kU];  // vector offset inside the owner's shard, or ~0
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const uint32_t v = sl0[k] + b0 + pl + (uint32_t)u * PL;
            const bool ok = (v < sl1[k]) && (v < nv_whole);
            vo[k][u] = ok ? v - own0[k] : ~0u;
            // non-temporal (sc0 | nt): every input is read once; measured
            // 3 % faster than non-temporal global loads on 64 MiB x 8.  A lane
            // without a vector reads past the descriptor and gets zero.
            x[k][u] = __builtin_amdgcn_raw_buffer_load_b128(rin, ok ? v * 16u : 0x80000000u, 0, kCpolSc0 | kCpolNt);
          }
        }
        if (b0 == 0 && c > lag) {
          // credit: this workgroup's consumers have finished chunks 0..c-1-lag
          // (consumer wave i has finished its group's chunks below s_done[i])
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
        if (b0 == 0 && pgi == 0) stamp(0, c);
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
      if (pgi == 0) stamp(1, c);
    }
    // the partial last vector of the message, by one lane of the group that
    // staged its chunk (that group took the chunk's credit), for the owner
    // whose slice w holds it; the owner's own vector is read by its consumer
    // directly
    const uint32_t tc = (uint32_t)(full_vecs / chunk_vecs), tv = (uint32_t)(full_vecs % chunk_vecs);
    if (has_tail && !dead && !silent && pg == tc % n_pgrp && pgi == 0 && lane == 0) {
#pragma unroll
      for (int k = 0; k < N - 1; ++k) {
        if (tv < sl0[k] || tv >= sl1[k]) continue;
        const int s = k < r ? k : k + 1;
        const uint32_t slot = (tc % n_buf) * a.parity_stride + (uint32_t)(s * N + r) * slot_bytes;
        st16_stage<kLocal>(rs, slot + (tv - own0[k]) * 16u, sentinel_canon<kKind>(load_vec<false>(src, full_vecs, nbytes)));
      }
    }
  } else {
    // ---------------- consumer waves
    const uint32_t cw = wave - n_prod;
    const uint32_t grp = cw / gw, gi = cw % gw;  // group, and wave within it
    const uint32_t cl = gi * 64u + lane, CL = gw * 64u;
    const uint32_t nv = chunk_vecs;
    const uint32_t o0 = (uint32_t)r * nv / (uint32_t)N, o1 = ((uint32_t)r + 1u) * nv / (uint32_t)N;
    const uint32_t s0 = o0 + w * (o1 - o0) / a.slices;
    const uint32_t s1n = o0 + (w + 1u) * (o1 - o0) / a.slices;
    // own vectors of the first batch of the group's next chunk, requested early
    u32x4 own_next[kUc];
    auto request_own = [&](uint32_t cn) {
      const uint64_t nb = (uint64_t)cn * chunk_vecs;
      const uint32_t nv_next = cn < a.n_chunks ? (uint32_t)min((uint64_t)chunk_vecs, total_vecs - nb) : 0u;
#pragma unroll
      for (int u = 0; u < kUc; ++u) {
        const uint32_t v = s0 + cl + (uint32_t)u * CL;
        own_next[u] = (!dead && v < s1n && v < nv_next) ? load_vec(src, nb + v, nbytes) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    request_own(grp);
    for (uint32_t c = grp; c < a.n_chunks && !__any((int)dead); c += n_grp) {
      const uint64_t vbase = (uint64_t)c * chunk_vecs;
      const uint32_t nv_real = (uint32_t)min((uint64_t)chunk_vecs, total_vecs - vbase);
      const uint32_t s1 = min(s1n, max(nv_real, s0));
      const uint32_t my = (c % n_buf) * a.parity_stride + (uint32_t)(r * N) * slot_bytes;
      if (s1 == s0 && gi == 0) stamp(2, c);  // nothing of this chunk here
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
        if (b0 == 0 && gi == 0) stamp(2, c);
#pragma unroll
        for (int u = 0; u < kUc; ++u) {
          if (!valid[u]) continue;
          const uint32_t v = s0 + b0 + cl + (uint32_t)u * CL;
          // non-temporal: the output is not read again, and plain stores would
          // compete with the staging for L2 (measured: 1-2 % faster)
          store_vec<true>(a.out, vbase + v, nbytes, reduce_vec<kKind, N>(own[u], r, d[u]));
          if (!a.keep) {
#pragma unroll
            for (int k = 0; k < N - 1; ++k) {
              const int sender = k < r ? k : k + 1;
              st16_reset<kLocal>(rs, my + (uint32_t)sender * slot_bytes + (v - o0) * 16u);
            }
          }
        }
      }
      // the resets are performed before the producers may reuse the buffer
      drain_vm();
      if (gi == 0) stamp(3, c);
      if (lane == 0 && !__any((int)dead))
        __hip_atomic_store(&s_done[cw], c + n_grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      // request the group's next chunk's own vectors while the producers fill it
      request_own(c + n_grp);
    }
  }
  wg_end(a.ctrl, st, a.host_epoch, a.grid, a.timing, idle);
}

// ---------------------------------------------------------------------------
// two-shot Sentinel, chunked, slot handshake (the reset is the credit)
// ---------------------------------------------------------------------------
// Staging: [buffer][owner s][sender r][vector of s's shard] 16 B, all-ones
// when empty; chunk c uses buffer c % B.  The partition into owner shards
// and slices uses the nominal chunk, so a slot keeps its (owner, slice) in
// every chunk.  Every rank stages its whole slice, its own shard included,
// so consumers never load HBM (a wave's vector memory operations retire in
// order: one HBM load queued before a poll would delay the poll's answer by
// an HBM latency).
// Every slot has one producer lane and one consumer lane, the same in every
// chunk, and alternates empty -> full (data, never all-ones) -> empty:
//   producer lane: stores chunk c's vector into the slot only after reading
//            the slot as empty -- the owner's consumer has taken chunk c - B
//            out of it and reset it (for c < B: unused in this call);
//   consumer lane: polls the N slots of its vector until all are full, adds
//            them in binary64 in rank order, rounds, writes `out` and resets
//            the slots to empty.
// The reset the producer reads is the owner's permission to send the next
// piece through that slot (a per-slot credit): no workgroup waits for a
// whole chunk, and no store is drained before a credit.  Only the slot's own
// producer can fill an empty slot, so a producer may read the slot state as
// early as it likes -- it does so together with the input loads of the work
// item, one item ahead.  A lane's own store to a slot is ordered before its
// own later load of that slot (same lane, same address), so a producer never
// mistakes the empty state it has overwritten for a fresh reset, and a
// consumer never reads data it has consumed.
// Producers keep one work item in flight per wave and rely on the number of
// producer waves (three quarters of a 1024-thread workgroup) for memory
// parallelism.
// The hot loops contain no branch around a memory operation: lanes without
// a vector use an offset past the end of the buffer (loads return zero,
// stores are dropped), and the one partial vector at the end of a message
// is moved after the loops.  The compiler can then wait for exactly the
// operations each step needs instead of draining every outstanding load.
template <int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(1024) k_twoshot_sentinel_hs(TwoShotArgs a) {
  constexpr uint32_t kOff = 0x80000000u;  // an offset past every buffer
  int r;
  uint32_t w;
  decode_role_t<kLocal, N>(blockIdx.x, r, w);
  // every kernel argument, requested at entry as one batch
  const uint8_t* src = a.part[r];
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(a.out), "s"(a.stage), "s"(a.ctrl), "s"(a.n), "s"(a.spin_limit),
                        "s"(a.chunk_elems), "s"(a.n_chunks), "s"(a.stage_bytes), "s"(a.parity_stride),
                        "s"(a.shard_cap), "s"(a.n_buffers), "s"(a.grid), "s"(a.slices), "s"(a.timing), "s"(a.keep),
                        "s"(a.drop_rank), "s"(a.host_epoch), "s"(a.cons_waves), "s"(a.threads));
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint64_t nbytes = a.n * (uint64_t)E::kBytes;
  const uint32_t chunk_vecs = (uint32_t)(((uint64_t)a.chunk_elems * E::kBytes) / 16u);  // chunks are whole vectors
  const uint64_t full_vecs = nbytes / 16u;          // whole vectors of the message
  const bool has_tail = (nbytes % 16u) != 0u;       // vector full_vecs is partial
  const uint64_t total_vecs = full_vecs + (has_tail ? 1u : 0u);
  const uint32_t slot_bytes = a.shard_cap * 16u;
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, n_waves = a.threads >> 6;
  // the host splits the waves: n_cons consume (staging reads only), the
  // rest produce
  const uint32_t n_cons = a.cons_waves, n_prod = n_waves - n_cons;
  const uint32_t n_buf = a.n_buffers;
  const uint32_t nv = chunk_vecs;
  const uint32_t reset_off = a.keep ? kOff : 0u;  // tests: keep the staged data
  const u32x4 kEmpty = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
  // owner s's shard of a chunk is [o0, o1) = [s*nv/N, (s+1)*nv/N); slice w
  // of it is the span-long piece starting at w*span, clamped to the shard
  // (the last slices may be short or empty: this protocol's credit is per
  // slot, nothing waits for a slice)
  const uint32_t span = ((nv + N - 1u) / N + a.slices - 1u) / a.slices;
  auto shard = [&](uint32_t s, uint32_t& o0, uint32_t& s0, uint32_t& s1) {
    o0 = s * nv / (uint32_t)N;
    const uint32_t o1 = (s + 1u) * nv / (uint32_t)N;
    s0 = min(o0 + w * span, o1);
    s1 = min(s0 + span, o1);
  };
  bool dead = idle;

  // Consumer work items are (chunk c, 64-vector batch b of the slice);
  // producer items split each of those into kH groups of kG owners.  A wave
  // takes every n-th item of its role, so different waves work on different
  // chunks at once and a slice that is short per chunk still keeps many
  // waves busy.
  constexpr int kG = (N + 1) / 2, kH = (N + kG - 1) / kG;
  const uint32_t n_bat = (span + 63u) / 64u;
  const uint32_t n_items = dead ? 0u : a.n_chunks * n_bat;  // consumer items
  if (wave < n_prod) {
    // ---------------- producer waves: rank r's slice (s, w) of every owner s
    const bool silent = ((uint32_t)r == a.drop_rank);
    const uint32_t n_pitems = (dead || silent) ? 0u : n_items * kH;
    struct Set {
      u32x4 x[kG];       // input vectors
      u32x4 chk[kG];     // slot state read when the inputs were requested
      uint32_t off[kG];  // slot offsets, or kOff
    };
    auto issue = [&](uint32_t pitem, Set& S) {
      const uint32_t item = pitem / kH, h = pitem % kH;
      const uint32_t c = item / n_bat, b0 = (item % n_bat) * 64u;
      // this chunk's whole vectors of the partial as a buffer view, so a
      // lane past the end reads zero without a branch
      const uint64_t cb = (uint64_t)c * nv * 16u;
      const uint64_t avail = full_vecs * 16u > cb ? full_vecs * 16u - cb : 0u;
      const uint32_t nfull = (uint32_t)min(avail, (uint64_t)nv * 16u);
      const __amdgpu_buffer_rsrc_t rin = make_rsrc(src + cb, nfull);
      const uint32_t boff = (c % n_buf) * a.parity_stride + (uint32_t)r * slot_bytes;
      uint32_t vin[kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const uint32_t s = h * kG + (uint32_t)g;
        uint32_t o0, s0, s1;
        shard(min(s, (uint32_t)N - 1u), o0, s0, s1);
        const uint32_t v = s0 + b0 + lane;
        const bool ok = (s < (uint32_t)N) && (v < s1) && (v * 16u < nfull);
        S.off[g] = ok ? boff + (s * N) * slot_bytes + (v - o0) * 16u : kOff;
        vin[g] = ok ? v * 16u : kOff;
      }
#pragma unroll
      for (int g = 0; g < kG; ++g) S.chk[g] = ld16_coh(rs, S.off[g]);
#pragma unroll
      for (int g = 0; g < kG; ++g) S.x[g] = __builtin_amdgcn_raw_buffer_load_b128(rin, vin[g], 0, kCpolNt);
      // keep these loads here: the compiler would otherwise sink them to
      // their first use and only one item would be in flight
      asm volatile("" ::: "memory");
    };
    auto commit = [&](const Set& S) -> bool {
      uint32_t need = 0u;
#pragma unroll
      for (int g = 0; g < kG; ++g)
        if (S.off[g] != kOff && !sentinel_is_empty(S.chk[g])) need |= 1u << g;
      if (need != 0u) {
        // a slot still held chunk c - B when it was read: read it again
        SpinBulk spin(a.spin_limit);
        while (need != 0u) {
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            return false;
          }
#pragma unroll
          for (int g = 0; g < kG; ++g)
            if ((need >> g) & 1u)
              if (sentinel_is_empty(ld16_coh(rs, S.off[g]))) need &= ~(1u << g);
        }
      }
#pragma unroll
      for (int g = 0; g < kG; ++g) st16_stage<kLocal>(rs, S.off[g], sentinel_canon<kKind>(S.x[g]));
      return true;
    };
    // two items in flight per wave: the next item's loads are issued before
    // this item is stored, so waiting for them never waits for stores
    Set A, B;
    uint32_t item = wave;
    if (item < n_pitems) issue(item, A);
    for (; item < n_pitems; item += 2u * n_prod) {
      if (item + n_prod < n_pitems) issue(item + n_prod, B);
      if (!commit(A)) {
        dead = true;
        break;
      }
      if (item + n_prod >= n_pitems) break;
      if (item + 2u * n_prod < n_pitems) issue(item + 2u * n_prod, A);
      if (!commit(B)) {
        dead = true;
        break;
      }
    }
    // the partial last vector, by the lane that owns its position
    if (has_tail && !dead && !silent) {
      const uint32_t c = (uint32_t)(full_vecs / nv), v = (uint32_t)(full_vecs % nv);
      for (uint32_t s = 0; s < (uint32_t)N; ++s) {
        uint32_t o0, s0, s1;
        shard(s, o0, s0, s1);
        if (v < s0 || v >= s1) continue;
        const uint32_t pitem = (c * n_bat + (v - s0) / 64u) * kH + s / kG;
        if (pitem % n_prod != wave || (v - s0) % 64u != lane) continue;
        const u32x4 x = load_vec<false>(src, full_vecs, nbytes);
        const uint32_t off = (c % n_buf) * a.parity_stride + (uint32_t)(s * N + r) * slot_bytes + (v - o0) * 16u;
        SpinBulk spin(a.spin_limit);
        while (!sentinel_is_empty(ld16_coh(rs, off))) {
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            break;
          }
        }
        st16_stage<kLocal>(rs, off, sentinel_canon<kKind>(x));
      }
    }
  } else {
    // ---------------- consumer waves: owner r's slice w, staging only
    const uint32_t cw = wave - n_prod;
    uint32_t o0, s0, s1n;
    shard((uint32_t)r, o0, s0, s1n);
    for (uint32_t item = cw; item < n_items && !dead; item += n_cons) {
      const uint32_t c = item / n_bat, b0 = (item % n_bat) * 64u;
      const uint64_t vbase = (uint64_t)c * nv;
      // whole vectors of this chunk in the slice; the partial one comes last
      const uint32_t fr = (uint32_t)min((uint64_t)nv, full_vecs > vbase ? full_vecs - vbase : 0u);
      const uint32_t s1 = min(s1n, max(fr, s0));
      if (s0 + b0 >= s1) continue;  // nothing of this item here (wave-uniform)
      const uint32_t my = (c % n_buf) * a.parity_stride + (uint32_t)(r * N) * slot_bytes;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + vbase * 16u, (uint32_t)((uint64_t)fr * 16u));
      const uint32_t v = s0 + b0 + lane;
      const uint32_t so = v < s1 ? my + (v - o0) * 16u : kOff;  // sender 0's slot, or kOff
      const uint32_t oo = v < s1 ? v * 16u : kOff;
      u32x4 d[N];
      SpinBulk spin(a.spin_limit);
      while (true) {
        bool all = true;
#pragma unroll
        for (int s = 0; s < N; ++s) {
          d[s] = ld16_coh(rs, so == kOff ? kOff : so + (uint32_t)s * slot_bytes);
          all &= (so == kOff) | sentinel_ready<kKind>(d[s]);
        }
        if (__all((int)all)) break;
        if (spin.expired()) {
          raise_status(a.ctrl, kStatusTimeout);
          dead = true;
          break;
        }
      }
      if (dead) break;
      __builtin_amdgcn_raw_buffer_store_b128(reduce_all<kKind, N>(d), ro, oo, 0, kCpolNt);
#pragma unroll
      for (int s = 0; s < N; ++s)
        st16_stage<kLocal>(rs, so == kOff ? kOff : so + (uint32_t)s * slot_bytes + reset_off, kEmpty);
    }
    // the partial last vector, by the lane that owns its position
    if (has_tail && !dead) {
      const uint32_t c = (uint32_t)(full_vecs / nv), v = (uint32_t)(full_vecs % nv);
      if (v >= s0 && v < s1n && (c * n_bat + (v - s0) / 64u) % n_cons == cw && (v - s0) % 64u == lane) {
        const uint32_t base = (c % n_buf) * a.parity_stride + (uint32_t)(r * N) * slot_bytes + (v - o0) * 16u;
        u32x4 d[N];
        SpinBulk spin(a.spin_limit);
        while (true) {
          bool all = true;
#pragma unroll
          for (int s = 0; s < N; ++s) {
            d[s] = ld16_coh(rs, base + (uint32_t)s * slot_bytes);
            all &= sentinel_ready<kKind>(d[s]);
          }
          if (all) break;
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            dead = true;
            break;
          }
        }
        if (!dead) {
          store_vec(a.out, full_vecs, nbytes, reduce_all<kKind, N>(d));
#pragma unroll
          for (int s = 0; s < N; ++s) st16_stage<kLocal>(rs, base + (uint32_t)s * slot_bytes + reset_off, kEmpty);
        }
      }
    }
  }
  wg_end(a.ctrl, st, a.host_epoch, a.grid, a.timing, idle);
}

// ---------------------------------------------------------------------------
// two-shot Sentinel, chunked, owner credit (progress words in memory)
// ---------------------------------------------------------------------------
// Staging: [buffer][owner s][sender k][vector of s's shard] 16 B, all-ones
// when empty; chunk c uses buffer c % B.  Every rank stages its whole slice,
// its own shard included, so no wave that polls ever has an HBM load queued
// in front of its polls (a wave's vector memory operations complete in
// order: one HBM load ahead of a poll delays the poll's answer by an HBM
// latency).  Owner shards and slices split the nominal chunk evenly, so a
// slot keeps its (owner, slice) in every chunk.
// A 1024-thread workgroup (r, w) has three roles:
//   producer waves: (chunk, batch) pairs dealt round-robin; a pair loads
//            rank r's vectors of slice w of every owner's shard (one per
//            owner per lane), and stores them into [c % B][s][r] once the
//            chunk is free (below); two pairs in flight per wave;
//   credit wave: reads the progress words of every (owner s, consumer wave)
//            of slice w and publishes in LDS the first chunk that some owner
//            has not consumed yet; chunk c is free once that is > c - B;
//   consumer waves: whole chunks dealt round-robin; for each vector of
//            owner r's slice w, poll the N slots, add them in binary64 in
//            rank order, round, write `out` and reset the slots; after the
//            chunk, drain (the resets are performed) and advance the wave's
//            progress count (a 32-bit word beside a 32-bit word holding the
//            call's epoch, written once the first count is performed).
// Chunk c reuses the buffer of chunk c - B only after every owner has
// consumed chunk c - B and its resets were performed, so B buffers give a
// run-ahead of B - 1 chunks (a credit read from the owners themselves, not
// inferred from this workgroup's own consumers).
template <int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(1024) k_twoshot_sentinel_oc(TwoShotArgs a) {
  constexpr uint32_t kOff = 0x80000000u;  // an offset past every buffer
  int r;
  uint32_t w;
  decode_role_t<kLocal, N>(blockIdx.x, r, w);
  // every kernel argument, requested at entry as one batch
  const uint8_t* src = a.part[r];
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(a.out), "s"(a.stage), "s"(a.ctrl), "s"(a.n), "s"(a.spin_limit),
                        "s"(a.chunk_elems), "s"(a.n_chunks), "s"(a.stage_bytes), "s"(a.parity_stride),
                        "s"(a.shard_cap), "s"(a.n_buffers), "s"(a.grid), "s"(a.slices), "s"(a.timing), "s"(a.keep),
                        "s"(a.drop_rank), "s"(a.host_epoch), "s"(a.cons_waves), "s"(a.credit), "s"(a.threads));
  const bool idle = (w >= a.slices);
  WgState st = wg_begin(a.ctrl, a.host_epoch, a.timing, idle);
  using E = Elem<kKind>;
  __shared__ uint32_t s_free;     // every owner has consumed all chunks below this
  __shared__ uint32_t s_cons[8];  // chunks each consumer wave of this workgroup has finished
  if (threadIdx.x == 0) s_free = 0u;
  if (threadIdx.x < 8) s_cons[threadIdx.x] = 0u;
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stage, a.stage_bytes);
  const uint64_t nbytes = a.n * (uint64_t)E::kBytes;
  const uint32_t nv = (uint32_t)(((uint64_t)a.chunk_elems * E::kBytes) / 16u);  // chunks are whole vectors
  const uint64_t full_vecs = nbytes / 16u;
  const bool has_tail = (nbytes % 16u) != 0u;  // vector full_vecs is partial
  const uint32_t slot_bytes = a.shard_cap * 16u;
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6, n_waves = a.threads >> 6;
  const uint32_t n_cons = a.cons_waves, n_prod = n_waves - n_cons - 1u;
  const uint32_t n_buf = a.n_buffers, n_chunks = a.n_chunks;
  const uint32_t reset_off = a.keep ? kOff : 0u;  // tests: keep the staged data
  // owner s's shard of a chunk is [o0, o1) = [s nv / N, (s+1) nv / N); slice
  // w of it is [o0 + w len / W, o0 + (w+1) len / W), len = o1 - o0 (32-bit:
  // nv < 2^18 vectors, W <= 64)
  const uint32_t span = ((nv + N - 1u) / N + a.slices - 1u) / a.slices;  // longest slice
  auto slice_of = [&](uint32_t s, uint32_t& o0, uint32_t& s0, uint32_t& s1) {
    o0 = s * nv / (uint32_t)N;
    const uint32_t len = (s + 1u) * nv / (uint32_t)N - o0;
    s0 = o0 + w * len / a.slices;
    s1 = o0 + (w + 1u) * len / a.slices;
  };
  // chunk c's whole vectors (the partial last vector is moved on its own)
  auto whole_in = [&](uint32_t c) -> uint32_t {
    const uint64_t vb = (uint64_t)c * nv;
    return (uint32_t)min((uint64_t)nv, full_vecs > vb ? full_vecs - vb : 0u);
  };
  const uint32_t tail_c = (uint32_t)(full_vecs / nv), tail_v = (uint32_t)(full_vecs % nv);
  bool dead = idle;
  uint64_t* tr = (a.trace && !idle) ? a.trace + (uint64_t)blockIdx.x * kPipeTraceWords : nullptr;
  auto stamp = [&](int kind, uint32_t c) {
    if (tr && lane == 0 && c < (uint32_t)kPipeTraceChunks) tr[kind * kPipeTraceChunks + c] = wall_ticks();
  };

  if (wave < n_prod) {
    // ---------------- producer waves
    const bool silent = ((uint32_t)r == a.drop_rank);
    const uint32_t n_bat = (span + 63u) / 64u;  // 64-vector batches of a slice
    const uint32_t n_pairs = (dead || silent) ? 0u : n_chunks * n_bat;
    uint32_t o0s[N], sl0[N], sl1[N];
#pragma unroll
    for (int s = 0; s < N; ++s) slice_of((uint32_t)s, o0s[s], sl0[s], sl1[s]);
    struct Set {
      u32x4 x[N];
      uint32_t off[N];  // slot offsets, or kOff
      uint32_t c, b0;
    };
    auto issue = [&](uint32_t pair, Set& S) {
      const uint32_t c = pair / n_bat, b0 = (pair % n_bat) * 64u;
      S.c = c;
      S.b0 = b0;
      const uint64_t cb = (uint64_t)c * nv * 16u;
      const uint32_t nfull = whole_in(c);
      const __amdgpu_buffer_rsrc_t rin = make_rsrc(src + cb, nfull * 16u);
      const uint32_t boff = (c % n_buf) * a.parity_stride + (uint32_t)r * slot_bytes;
      uint32_t vin[N];
#pragma unroll
      for (int s = 0; s < N; ++s) {
        const uint32_t v = sl0[s] + b0 + lane;
        const bool ok = (v < sl1[s]) && (v < nfull);
        S.off[s] = ok ? boff + (uint32_t)(s * N) * slot_bytes + (v - o0s[s]) * 16u : kOff;
        vin[s] = ok ? v * 16u : kOff;
      }
#pragma unroll
      for (int s = 0; s < N; ++s) S.x[s] = __builtin_amdgcn_raw_buffer_load_b128(rin, vin[s], 0, kCpolNt);
      // keep these loads here: the compiler would otherwise sink them to
      // their first use and only one pair would be in flight
      asm volatile("" ::: "memory");
    };
    // chunk c may be staged once every owner has consumed chunk c - B
    auto wait_free = [&](uint32_t c) -> bool {
      if (c < n_buf) return true;
      SpinBulk spin(a.spin_limit);
      while (__hip_atomic_load(&s_free, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) + n_buf <= c) {
        if (spin.expired()) {
          raise_status(a.ctrl, kStatusTimeout);
          return false;
        }
      }
      return true;
    };
    auto commit = [&](const Set& S) -> bool {
      if (!wait_free(S.c)) return false;
      if (S.b0 == 0u) stamp(0, S.c);
#pragma unroll
      for (int s = 0; s < N; ++s) st16_stage<kLocal>(rs, S.off[s], sentinel_canon<kKind>(S.x[s]));
      if (S.b0 == 0u) stamp(1, S.c);
      return true;
    };
    Set A, B;
    uint32_t pair = wave;
    if (pair < n_pairs) issue(pair, A);
    for (; pair < n_pairs; pair += 2u * n_prod) {
      if (pair + n_prod < n_pairs) issue(pair + n_prod, B);
      if (!commit(A)) {
        dead = true;
        break;
      }
      if (pair + n_prod >= n_pairs) break;
      if (pair + 2u * n_prod < n_pairs) issue(pair + 2u * n_prod, A);
      if (!commit(B)) {
        dead = true;
        break;
      }
    }
    // the partial last vector, by the lane whose pair covers its position
    if (has_tail && !dead && !silent) {
#pragma unroll
      for (int s = 0; s < N; ++s) {
        if (tail_v < sl0[s] || tail_v >= sl1[s]) continue;
        const uint32_t i = tail_v - sl0[s];
        if ((tail_c * n_bat + i / 64u) % n_prod != wave || i % 64u != lane) continue;
        const u32x4 x = load_vec<false>(src, full_vecs, nbytes);
        if (!wait_free(tail_c)) break;
        const uint32_t off =
            (tail_c % n_buf) * a.parity_stride + (uint32_t)(s * N + r) * slot_bytes + (tail_v - o0s[s]) * 16u;
        st16_stage<kLocal>(rs, off, sentinel_canon<kKind>(x));
      }
    }
  } else if (wave == n_prod) {
    // ---------------- credit wave
    // lane l reads owner l / n_cons's consumer wave l % n_cons; that wave
    // has consumed chunks q, q + n_cons, ..., so every chunk below
    // q + count * n_cons that it owns is consumed
    const uint32_t target = n_chunks > n_buf ? n_chunks - n_buf : 0u;  // producers never need more
    const uint32_t q = lane % n_cons;
    // progress entry: [count, epoch] 32-bit words (see the consumer waves)
    uint32_t* const cp =
        lane < (uint32_t)N * n_cons ? a.credit + 2 * (((size_t)(lane / n_cons) * kCreditSlices + w) * kCreditWaves + q)
                                    : nullptr;
    uint32_t have = 0u;
    SpinBulk spin(a.spin_limit);
    while (!dead && have < target) {
      uint32_t f = ~0u;
      if (cp != nullptr) {
        // the count only once its epoch word carries this call's epoch: the
        // writer stored the count first, then the epoch, so a count read
        // after that epoch is this call's (not a stale word of another call)
        uint32_t cnt = 0u;
        if (__hip_atomic_load(cp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == st.epoch)
          cnt = __hip_atomic_load(cp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f = q + cnt * n_cons;
      }
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) f = min(f, (uint32_t)__shfl_xor((int)f, d));
      if (f > have) {
        have = f;
        if (lane == 0) __hip_atomic_store(&s_free, have, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        spin = SpinBulk(a.spin_limit);
      } else if (spin.expired()) {
        raise_status(a.ctrl, kStatusTimeout);
        dead = true;
      }
    }
  } else {
    // ---------------- consumer waves: owner r's slice w, staging only
    const uint32_t cw = wave - n_prod - 1u;
    uint32_t o0, s0, s1n;
    slice_of((uint32_t)r, o0, s0, s1n);
    uint32_t* const my_word = a.credit + 2 * (((size_t)r * kCreditSlices + w) * kCreditWaves + cw);
    uint32_t done = 0u;
    for (uint32_t c = cw; c < n_chunks && !dead; c += n_cons) {
      // chunk c - B, the previous user of these slots, may belong to another
      // consumer wave: its resets must be performed before this wave polls,
      // or it would take chunk c - B's data for chunk c's
      if (c >= n_buf) {
        const uint32_t p = c - n_buf, pq = p % n_cons, need = p / n_cons + 1u;
        SpinBulk spin(a.spin_limit);
        while (__hip_atomic_load(&s_cons[pq], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < need) {
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            dead = true;
            break;
          }
        }
        if (dead) break;
      }
      const uint64_t vbase = (uint64_t)c * nv;
      const uint32_t fr = whole_in(c);
      const uint32_t s1 = min(s1n, max(fr, s0));
      const uint32_t my = (c % n_buf) * a.parity_stride + (uint32_t)(r * N) * slot_bytes;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.out + vbase * 16u, fr * 16u);
      for (uint32_t b0 = 0; s0 + b0 < s1 && !dead; b0 += 64u) {
        const uint32_t v = s0 + b0 + lane;
        const uint32_t so = v < s1 ? my + (v - o0) * 16u : kOff;  // sender 0's slot, or kOff
        const uint32_t oo = v < s1 ? v * 16u : kOff;
        u32x4 d[N];
        SpinBulk spin(a.spin_limit);
        while (true) {
          bool all = true;
#pragma unroll
          for (int k = 0; k < N; ++k) {
            d[k] = ld16_coh(rs, so == kOff ? kOff : so + (uint32_t)k * slot_bytes);
            all &= (so == kOff) | sentinel_ready<kKind>(d[k]);
          }
          if (__all((int)all)) break;
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            dead = true;
            break;
          }
        }
        if (dead) break;
        if (b0 == 0u) stamp(2, c);
        __builtin_amdgcn_raw_buffer_store_b128(reduce_all<kKind, N>(d), ro, oo, 0, kCpolNt);
#pragma unroll
        for (int k = 0; k < N; ++k)
          st16_reset<kLocal>(rs, so == kOff ? kOff : so + (uint32_t)k * slot_bytes + reset_off);
      }
      // the partial last vector, by the lane that owns its position
      if (has_tail && c == tail_c && !dead && tail_v >= s0 && tail_v < s1n && (tail_v - s0) % 64u == lane) {
        const uint32_t base = my + (tail_v - o0) * 16u;
        u32x4 d[N];
        SpinBulk spin(a.spin_limit);
        while (true) {
          bool all = true;
#pragma unroll
          for (int k = 0; k < N; ++k) {
            d[k] = ld16_coh(rs, base + (uint32_t)k * slot_bytes);
            all &= sentinel_ready<kKind>(d[k]);
          }
          if (all) break;
          if (spin.expired()) {
            raise_status(a.ctrl, kStatusTimeout);
            dead = true;
            break;
          }
        }
        if (!dead) {
          store_vec(a.out, full_vecs, nbytes, reduce_all<kKind, N>(d));
#pragma unroll
          for (int k = 0; k < N; ++k) st16_reset<kLocal>(rs, base + (uint32_t)k * slot_bytes + reset_off);
        }
      }
      dead = __any((int)dead) != 0;
      if (dead) break;
      // the resets are performed before the owner's progress advances
      drain_vm();
      ++done;
      if (lane == 0) {
        // 32-bit words like every other polled word: the count, and on the
        // first chunk of the call (after the count is performed) the epoch
        // that makes it this call's
        __hip_atomic_store(my_word, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == 1u) {
          drain_vm();
          __hip_atomic_store(my_word + 1, st.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(&s_cons[cw], done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      stamp(3, c);
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
      if (ls.oneshot_split == 2)
        hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, N, true, false, 2>), grid, block, 0, stream, ls.oneshot);
      else
        hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, N, true>), grid, block, 0, stream, ls.oneshot);
      break;
    case kKernOneShotSentinelLocal:
      if (ls.oneshot_split == 2)
        hipLaunchKernelGGL((k_oneshot<kWireSentinel, kKind, N, true, false, 2>), grid, block, 0, stream, ls.oneshot);
      else
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
    case kKernLL128WsAcc32:
      hipLaunchKernelGGL((k_twoshot_ll128_ws<kKind, 0, N>), grid, block, 0, stream, ls.twoshot);
      break;
    case kKernLL128WsAcc16:
      if constexpr (kKind != kKindF32) {
        hipLaunchKernelGGL((k_twoshot_ll128_ws<kKind, 1, N>), grid, block, 0, stream, ls.twoshot);
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
    case kKernSentinelHs:
      hipLaunchKernelGGL((k_twoshot_sentinel_hs<kKind, N, false>), grid, block, 0, stream, ls.twoshot);
      break;
    case kKernP2PLL:
    case kKernP2PSentinel:
    case kKernP2PLLLocal:
    case kKernP2PSentinelLocal:
      if constexpr (N == 2) {
        if (ls.kernel == kKernP2PLL)
          hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, 2, false, true>), grid, block, 0, stream, ls.oneshot);
        else if (ls.kernel == kKernP2PSentinel)
          hipLaunchKernelGGL((k_oneshot<kWireSentinel, kKind, 2, false, true>), grid, block, 0, stream, ls.oneshot);
        else if (ls.kernel == kKernP2PLLLocal)
          hipLaunchKernelGGL((k_oneshot<kWireLL, kKind, 2, true, true>), grid, block, 0, stream, ls.oneshot);
        else
          hipLaunchKernelGGL((k_oneshot<kWireSentinel, kKind, 2, true, true>), grid, block, 0, stream, ls.oneshot);
      } else {
        return hipErrorInvalidValue;
      }
      break;
    case kKernSentinelHsLocal:
      hipLaunchKernelGGL((k_twoshot_sentinel_hs<kKind, N, true>), grid, block, 0, stream, ls.twoshot);
      break;
    case kKernSentinelOc:
      hipLaunchKernelGGL((k_twoshot_sentinel_oc<kKind, N, false>), grid, block, 0, stream, ls.twoshot);
      break;
    case kKernSentinelOcLocal:
      hipLaunchKernelGGL((k_twoshot_sentinel_oc<kKind, N, true>), grid, block, 0, stream, ls.twoshot);
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
  if (is_multi_kernel(ls.kernel)) return launch_multi(ls, stream);
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
    case kKernLL128WsAcc32: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_ll128_ws<kKind, 0, N>, threads, 0); break;
    case kKernLL128WsAcc16:
      if constexpr (kKind != kKindF32) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_ll128_ws<kKind, 1, N>, threads, 0);
      break;
    case kKernSentinelPipe: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel<kKind, N, false>, threads, 0); break;
    case kKernSentinelPipeLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel<kKind, N, true>, threads, 0); break;
    case kKernSentinelHs: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel_hs<kKind, N, false>, threads, 0); break;
    case kKernP2PLL:
    case kKernP2PSentinel:
    case kKernP2PLLLocal:
    case kKernP2PSentinelLocal:
      // the copy kernels use no more resources than the two-rank one-shot ones
      if constexpr (N == 2) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot<kWireSentinel, kKind, 2, false, true>, threads, 0);
      break;
    case kKernSentinelHsLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel_hs<kKind, N, true>, threads, 0); break;
    case kKernSentinelOc: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel_oc<kKind, N, false>, threads, 0); break;
    case kKernSentinelOcLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_twoshot_sentinel_oc<kKind, N, true>, threads, 0); break;
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
  if (is_multi_kernel(kernel)) return occupancy_multi(kind, n_ranks, kernel, threads);
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
