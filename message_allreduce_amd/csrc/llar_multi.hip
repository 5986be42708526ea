// llar_multi.hip -- ReduceScatter and AllGather over the LL and Sentinel
// wires, N ranks emulated inside one GPU.
//
// Definitions (yololab.net article on network architecture for LLM
// inference, the table of the section on All-Reduce, All-Gather and
// Reduce-Scatter): after a ReduceScatter every rank keeps one segment of the
// element-wise sum; after an AllGather every rank holds every rank's
// fragment.  They are the two halves of the two-shot AllReduce of "Every
// Microsecond Matters" (agihunt.info summary, two-shot LL128 paragraph).
//
// One launch, every rank both sends and receives.  Workgroup (rank r,
// slice w) first puts slice w of its block for each receiving rank into the
// staging slot that rank reads (no wait: producers never block), then polls
// its own N-1 slots for slice w and writes its output.  The wires are those of
// the one-shot AllReduce: LL lines {data0, epoch, data1, epoch} (LL
// paragraph), or a Sentinel-prefilled slot that the receiver resets after
// use (Sentinel paragraph).  Every workgroup of the grid is resident at once
// (the host checks occupancy), so a receiver's poll always ends: the data
// arrives, or the bounded poll expires and latches a timeout.
//
// Blocks need not be a multiple of 16 bytes: then the accesses to the
// caller's buffers (which start at block multiples) move halfwords, and the
// last vector of a block is zero-padded in staging.
#include <stddef.h>

#include "llar_device.h"
#include "llar_internal.h"

namespace llar {
namespace {

// ---- caller-buffer access at a byte offset, clipped at `end` ----------------
// `off` is a multiple of the element size; whole vectors (or units) are moved
// only when the block size keeps them 16-byte aligned.
__device__ __forceinline__ u32x4 load16_at(const uint8_t* p, uint64_t off, uint64_t end, bool aligned) {
  if (aligned && off + 16u <= end) return *reinterpret_cast<const u32x4*>(p + off);
  u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
  for (uint32_t k = 0; k < 16u; k += 2u) {
    if (off + k < end) x[k >> 2] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + off + k)) << ((k & 2u) * 8u);
  }
  return x;
}
__device__ __forceinline__ u32x2 load8_at(const uint8_t* p, uint64_t off, uint64_t end, bool aligned) {
  if (aligned && off + 8u <= end) return *reinterpret_cast<const u32x2*>(p + off);
  u32x2 x = {0u, 0u};
#pragma unroll
  for (uint32_t k = 0; k < 8u; k += 2u) {
    if (off + k < end) x[k >> 2] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + off + k)) << ((k & 2u) * 8u);
  }
  return x;
}
// 4-byte halves of a unit (the LL receiver's granularity when every half of
// its slice has a lane)
__device__ __forceinline__ uint32_t load4_at(const uint8_t* p, uint64_t off, uint64_t end, bool aligned) {
  if (aligned && off + 4u <= end) return *reinterpret_cast<const uint32_t*>(p + off);
  uint32_t x = 0u;
  if (off < end) x = *reinterpret_cast<const uint16_t*>(p + off);
  if (off + 2u < end) x |= (uint32_t)(*reinterpret_cast<const uint16_t*>(p + off + 2u)) << 16;
  return x;
}
__device__ __forceinline__ void store4_at(uint8_t* p, uint64_t off, uint64_t end, bool aligned, uint32_t x) {
  if (aligned && off + 4u <= end) {
    *reinterpret_cast<uint32_t*>(p + off) = x;
    return;
  }
  if (off < end) *reinterpret_cast<uint16_t*>(p + off) = (uint16_t)x;
  if (off + 2u < end) *reinterpret_cast<uint16_t*>(p + off + 2u) = (uint16_t)(x >> 16);
}
__device__ __forceinline__ void store8_at(uint8_t* p, uint64_t off, uint64_t end, bool aligned, u32x2 x) {
  if (aligned && off + 8u <= end) {
    *reinterpret_cast<u32x2*>(p + off) = x;
    return;
  }
#pragma unroll
  for (uint32_t k = 0; k < 8u; k += 2u) {
    if (off + k < end) *reinterpret_cast<uint16_t*>(p + off + k) = (uint16_t)(x[k >> 2] >> ((k & 2u) * 8u));
  }
}

// Reduce an 8-byte unit with the receiver's own value at rank position
// `own_rank` and the senders' values in d[0..N-2] ordered by rank: binary64
// sum in rank order starting from rank 0's value, one rounding.  Indices into
// d stay compile-time; the own position is chosen with selects.
template <int kKind, int N>
__device__ __forceinline__ u32x2 reduce_unit_at(const u32x2& own, int own_rank, const u32x2 (&d)[N > 1 ? N - 1 : 1]) {
  constexpr int kPerUnit = 8 / Elem<kKind>::kBytes;
  u32x2 out = {0u, 0u};
#pragma unroll
  for (int j = 0; j < kPerUnit; ++j) {
    auto elem = [&](const u32x2& v) -> uint32_t {
      if constexpr (Elem<kKind>::kBytes == 4) return v[j];
      else return (v[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
    };
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const uint32_t below = (r < N - 1) ? elem(d[r < N - 1 ? r : 0]) : 0u;  // rank r at d[r]
      const uint32_t above = (r >= 1) ? elem(d[r >= 1 ? r - 1 : 0]) : 0u;   // rank r at d[r-1]
      const uint32_t bits = (r < own_rank) ? below : (r == own_rank) ? elem(own) : above;
      const double x = Elem<kKind>::dec(bits);
      s = (r == 0) ? x : s + x;
    }
    const uint32_t bits = Elem<kKind>::enc(s);
    if constexpr (Elem<kKind>::kBytes == 4) out[j] = bits;
    else out[j >> 1] |= (bits & 0xFFFFu) << ((j & 1) * 16);
  }
  return out;
}

// The same for a 4-byte half (one binary32 or two 16-bit elements).
template <int kKind, int N>
__device__ __forceinline__ uint32_t reduce_half_at(uint32_t own, int own_rank, const uint32_t (&d)[N > 1 ? N - 1 : 1]) {
  constexpr int kPer = 4 / Elem<kKind>::kBytes;
  uint32_t out = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    auto elem = [&](uint32_t v) -> uint32_t {
      if constexpr (Elem<kKind>::kBytes == 4) return v;
      else return (v >> (j * 16)) & 0xFFFFu;
    };
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const uint32_t below = (r < N - 1) ? elem(d[r < N - 1 ? r : 0]) : 0u;  // rank r at d[r]
      const uint32_t above = (r >= 1) ? elem(d[r >= 1 ? r - 1 : 0]) : 0u;   // rank r at d[r-1]
      const uint32_t bits = (r < own_rank) ? below : (r == own_rank) ? elem(own) : above;
      const double x = Elem<kKind>::dec(bits);
      s = (r == 0) ? x : s + x;
    }
    const uint32_t bits = Elem<kKind>::enc(s);
    if constexpr (Elem<kKind>::kBytes == 4) out = bits;
    else out |= (bits & 0xFFFFu) << (j * 16);
  }
  return out;
}

template <int kKind>
__device__ __forceinline__ u32x2 sentinel_canon8(const u32x2& v) {
  const u32x4 c = sentinel_canon<kKind>(u32x4{v[0], v[1], 0u, 0u});
  return u32x2{c[0], c[1]};
}

template <int kWire, int kKind, int N, bool kGather, bool kLocal>
__global__ void __launch_bounds__(512) k_multi(MultiArgs a) {
  int r;
  uint32_t w;
  decode_role_t<kLocal, N>(blockIdx.x, r, w);
  const uint8_t* const src = a.in[r];
  uint8_t* const out = a.out[r];
  uint8_t* const stage = a.stage;
  Ctrl* const ctrl = a.ctrl;
  const uint64_t blk = a.blk, spin_limit = a.spin_limit;
  const uint32_t vq = a.vq, vr = a.vr, stage_bytes = a.stage_bytes, parity_stride = a.parity_stride;
  const uint32_t slot_stride = a.slot_stride, n_recv = a.n_recv, grid = a.grid, slices = a.slices;
  const uint32_t timing = a.timing, keep = a.keep, drop_rank = a.drop_rank, host_epoch = a.host_epoch;
  const bool aligned = a.aligned != 0u;
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(out), "s"(stage), "s"(ctrl), "s"(blk), "s"(spin_limit), "s"(vq), "s"(vr),
                        "s"(stage_bytes), "s"(parity_stride), "s"(slot_stride), "s"(n_recv), "s"(grid), "s"(slices),
                        "s"(timing), "s"(keep), "s"(drop_rank), "s"(host_epoch));
  const bool idle = (w >= slices);
  const uint32_t v0 = idle ? 0u : w * vq + min(w, vr);
  const uint32_t v1 = idle ? 0u : v0 + vq + (w < vr ? 1u : 0u);
  WgState st = wg_begin(ctrl, host_epoch, timing, idle);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(stage, stage_bytes);
  const uint32_t e = st.epoch;
  const uint32_t par_off = (e & 1u) * parity_stride;
  constexpr uint32_t kVecStage = (kWire == kWireLL) ? 32u : 16u;
  constexpr uint32_t kUnitStage = (kWire == kWireLL) ? 16u : 8u;

  // ---- send: slice w of this rank's block for every receiver -----------------
  // Work items are (receiver, vector) pairs, receiver-major, so that a small
  // slice still spreads over the whole workgroup.  The p-th receiver other
  // than this rank is p (p < r) or p + 1.
  if (!idle && (uint32_t)r != drop_rank) {
    const uint32_t span = v1 - v0;
    const uint32_t n_peers = (uint32_t)r < n_recv ? n_recv - 1u : n_recv;
    for (uint32_t it = threadIdx.x; it < n_peers * span; it += blockDim.x) {
      const uint32_t p = it / span, v = v0 + (it - p * span);
      const uint32_t j = p < (uint32_t)r ? p : p + 1u;
      const uint64_t base = kGather ? 0u : (uint64_t)j * blk;
      const u32x4 y = load16_at(src, base + (uint64_t)v * 16u, base + blk, aligned);
      const uint32_t slot = j * (uint32_t)(N - 1) + ((uint32_t)r < j ? (uint32_t)r : (uint32_t)r - 1u);
      const uint32_t off = par_off + slot * slot_stride + v * kVecStage;
      if constexpr (kWire == kWireLL) llar_wire::ll_put16<scope_of(kLocal)>(rs, off, y, e);
      else llar_wire::sentinel_put<Elem<kKind>::kBytes, scope_of(kLocal)>(rs, off, y);
    }
  }

  // ---- receive: slice w from every other rank ---------------------------------
  // LL ReduceScatter: when every 4-byte half of the slice has a lane, each
  // lane takes one half line {data, epoch} (each half carries its own flag):
  // the polls spread over twice the lanes and each lane reduces half as many
  // elements (uniform per workgroup).  Measured on MI355X, bf16, graph-
  // replayed per call: N = 8 16 KiB 3.66 -> 3.34 us (device 2.41 -> 2.02),
  // 4 KiB 3.70 -> 3.43, 128 KiB 4.00 -> 3.78; N = 4 16 KiB 3.37 -> 3.21.  The
  // AllGather, which has nothing to reduce, keeps whole units: halves cost it
  // 0.05-0.1 us there.
  const bool halves = kWire == kWireLL && !kGather && 4u * (v1 - v0) <= blockDim.x;
  if (!idle && (uint32_t)r < n_recv && halves) {
    const uint64_t own_base = (uint64_t)r * blk;
    const uint32_t my_slots = par_off + (uint32_t)r * (uint32_t)(N - 1) * slot_stride;
    const uint32_t h = 4u * v0 + threadIdx.x;  // half h of unit h / 2: staging line h / 2, bytes (h % 2) * 8
    if (h < 4u * v1) {
      const uint32_t own = load4_at(src, own_base + (uint64_t)h * 4u, own_base + blk, aligned);
      const uint32_t off_h = (h >> 1) * 16u + (h & 1u) * 8u;
      uint32_t d[N > 1 ? N - 1 : 1];
      d[0] = 0u;
      Spin spin(spin_limit);
      bool ok = true;
      while (true) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          const u32x2 q = llar_wire::ld8_coh(rs, my_slots + (uint32_t)k * slot_stride + off_h);
          all &= q[1] == e;
          d[k] = q[0];
        }
        if (all) break;
        if (spin.expired()) {
          raise_status(ctrl, kStatusTimeout);
          ok = false;
          break;
        }
      }
      if (ok) store4_at(out, (uint64_t)h * 4u, blk, aligned, reduce_half_at<kKind, N>(own, r, d));
    }
  } else if (!idle && (uint32_t)r < n_recv) {
    const uint64_t own_base = kGather ? 0u : (uint64_t)r * blk;
    const uint32_t my_slots = par_off + (uint32_t)r * (uint32_t)(N - 1) * slot_stride;
    bool dead = false;  // set after a timeout: stop waiting for anything else
    for (uint32_t u = 2u * v0 + threadIdx.x; u < 2u * v1 && !dead; u += blockDim.x) {
      const u32x2 own = load8_at(src, own_base + (uint64_t)u * 8u, own_base + blk, aligned);
      u32x2 d[N > 1 ? N - 1 : 1];
      d[0] = u32x2{0u, 0u};
      Spin spin(spin_limit);
      bool ok = true;
      while (true) {
        bool all = true;
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          const uint32_t off = my_slots + (uint32_t)k * slot_stride + u * kUnitStage;
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
      if constexpr (kGather) {
        // fragment k lands at k * blk: the own one at r, slot k's sender at
        // k (k < r) or k + 1 (k >= r); the Sentinel wire canonicalises every
        // fragment, the own one included, so all receivers agree
        const u32x2 mine = (kWire == kWireSentinel) ? sentinel_canon8<kKind>(own) : own;
        store8_at(out, (uint64_t)r * blk + (uint64_t)u * 8u, (uint64_t)(r + 1) * blk, aligned, mine);
#pragma unroll
        for (int k = 0; k < N - 1; ++k) {
          const uint64_t s = (uint64_t)(k < r ? k : k + 1);
          store8_at(out, s * blk + (uint64_t)u * 8u, (s + 1u) * blk, aligned, d[k]);
        }
      } else {
        store8_at(out, (uint64_t)u * 8u, blk, aligned, reduce_unit_at<kKind, N>(own, r, d));
      }
      if constexpr (kWire == kWireSentinel) {
        if (!keep) {
#pragma unroll
          for (int k = 0; k < N - 1; ++k)
            llar_wire::sentinel_reset8<scope_of(kLocal)>(rs, my_slots + (uint32_t)k * slot_stride + u * 8u);
        }
      }
    }
  }
  wg_end(ctrl, st, host_epoch, grid, timing, idle);
}

// ---- ReduceScatter over the LL128 atomic wire ----------------------------------------
// The reduce-scatter half of the two-shot LL128 AllReduce, with the owners'
// shards equal to the ReduceScatter segments.  Owner o's segment (c
// elements) occupies Lo = ceil(c / K) lines of its own, o*Lo .. o*Lo+Lo-1;
// element i of it sits in line o*Lo + i/K, slot 1 + i%K (K = 31 binary32
// slots, or 63 16-bit ones).  Every owner's lines are split the same way
// into W slices.  Workgroup (rank r, slice w):
//   produce: for every owner o, atomically add rank r's copy of segment o,
//            slice w, into o's lines; once every wave's data atomics are
//            acknowledged (drain + workgroup barrier), add 1.0 to slot 0 of
//            each of those lines;
//   consume: for each line of owner r's slice w, wait for the count N, read
//            it (8 lanes x 16 bytes), round to the output type, zero it.
// No line is shared between slices, so a workgroup only waits for the
// slice-w workgroups of the other ranks, all resident.  The spread placement
// is used: device-scope atomics resolve at the memory side wherever the
// ranks run.
template <int kKind, int kAcc16, int N>
__global__ void __launch_bounds__(512) k_rs_ll128(MultiArgs a) {
  int r;
  uint32_t w;
  decode_role_t<false, N>(blockIdx.x, r, w);
  const uint8_t* const src = a.in[r];
  uint8_t* const out = a.out[r];
  uint8_t* const stage = a.stage;
  Ctrl* const ctrl = a.ctrl;
  const uint64_t blk = a.blk, spin_limit = a.spin_limit;
  const uint32_t stage_bytes = a.stage_bytes, grid = a.grid, slices = a.slices;
  const uint32_t timing = a.timing, keep = a.keep, drop_rank = a.drop_rank, host_epoch = a.host_epoch;
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(out), "s"(stage), "s"(ctrl), "s"(blk), "s"(spin_limit), "s"(stage_bytes),
                        "s"(grid), "s"(slices), "s"(timing), "s"(keep), "s"(drop_rank), "s"(host_epoch));
  using E = Elem<kKind>;
  constexpr uint32_t K = kAcc16 ? 63u : 31u;
  const bool idle = (w >= slices);
  WgState st = wg_begin(ctrl, host_epoch, timing, idle);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(stage, stage_bytes);
  const uint32_t c = (uint32_t)(blk / E::kBytes);  // elements per segment
  const uint32_t Lo = (c + K - 1u) / K;               // lines per owner
  const uint32_t l0 = (uint32_t)((uint64_t)w * Lo / slices), l1 = (uint32_t)((uint64_t)(w + 1u) * Lo / slices);
  const uint32_t nl = idle ? 0u : l1 - l0;
  uint32_t full;
  if constexpr (!kAcc16) full = __float_as_uint((float)N);
  else full = E::from_f32((float)N);

  // ---- produce: data atomics into every owner's lines of slice w, then
  // counts.  The (owner, line, dword) items are spread over all threads at
  // once: a slice holds only a few lines per owner, and walking the owners
  // in turn would leave most waves idle
  if ((uint32_t)r != drop_rank) {
    const uint32_t per_owner = nl * 32u;
    for (uint32_t it = threadIdx.x; it < (uint32_t)N * per_owner; it += blockDim.x) {
      const uint32_t o = it / per_owner, rem = it % per_owner;
      const uint8_t* const seg = src + (uint64_t)o * blk;
      const uint32_t line = l0 + rem / 32u, q = rem % 32u;  // dword q of the line
      uint8_t* const dst = stage + ((uint64_t)o * Lo + line) * llar_wire::kLL128LineBytes + q * 4u;
      if constexpr (!kAcc16) {
        const uint32_t i = line * K + q - 1u;
        if (q == 0u || i >= c) continue;
        float val;
        if constexpr (E::kBytes == 4) val = __uint_as_float(reinterpret_cast<const uint32_t*>(seg)[i]);
        else val = E::to_f32(reinterpret_cast<const uint16_t*>(seg)[i]);
        llar_wire::ll128_add(reinterpret_cast<float*>(dst), val);
      } else {
        // 16-bit slots 2q and 2q+1 hold elements line*K + 2q - 1 and line*K + 2q
        const uint32_t i0 = line * K + 2u * q - 1u, i1 = line * K + 2u * q;
        const uint32_t lo = (q != 0u && i0 < c) ? reinterpret_cast<const uint16_t*>(seg)[i0] : 0u;
        const uint32_t hi = (i1 < c) ? reinterpret_cast<const uint16_t*>(seg)[i1] : 0u;
        if ((lo | hi) == 0u) continue;  // nothing to add (both +0)
        llar_wire::ll128_add2<kKind == kKindBF16>(dst, s16x2{(short)lo, (short)hi});
      }
    }
  }
  // every wave's data atomics acknowledged before any count of this workgroup
  drain_vm();
  __syncthreads();
  if ((uint32_t)r != drop_rank) {
    for (uint32_t it = threadIdx.x; it < (uint32_t)N * nl; it += blockDim.x) {
      const uint32_t o = it / nl, line = l0 + it % nl;
      uint8_t* const dst = stage + ((uint64_t)o * Lo + line) * llar_wire::kLL128LineBytes;
      if constexpr (!kAcc16) llar_wire::ll128_flag(reinterpret_cast<float*>(dst));
      else llar_wire::ll128_flag2<kKind == kKindBF16>(dst, E::from_f32(1.0f));
    }
  }

  // ---- consume owner r's lines of slice w: 8 lanes per line
  for (uint32_t it = threadIdx.x; it < nl * 8u; it += blockDim.x) {
    const uint32_t line = l0 + it / 8u, j = it % 8u;
    const uint32_t loff = ((uint32_t)r * Lo + line) * llar_wire::kLL128LineBytes;
    Spin spin(spin_limit);
    if (!llar_wire::ll128_wait<kAcc16 != 0>(rs, loff, full, spin)) {
      raise_status(ctrl, kStatusTimeout);
      break;
    }
    // 16-bit staging: read and zero the line's 16 bytes in one exchange, as
    // the one-round AllReduce does; binary32 staging reads, then stores zeros
    const bool take = kAcc16 && !keep;
    const u32x4 v = take ? llar_wire::ll128_take16(stage + loff + j * 16u) : llar_wire::ll128_read16(rs, loff + j * 16u);
    if constexpr (!kAcc16) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t s = j * 4u + (uint32_t)t, i = line * K + s - 1u;
        if (s == 0u || i >= c) continue;
        if constexpr (E::kBytes == 4) reinterpret_cast<uint32_t*>(out)[i] = v[t];
        else reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)E::from_f32(__uint_as_float(v[t]));
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t s = j * 8u + (uint32_t)t, i = line * K + s - 1u;
        if (s == 0u || i >= c) continue;
        reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)(v[t >> 1] >> ((t & 1) * 16));
      }
    }
    if (!take && !keep) llar_wire::ll128_reset16(rs, loff + j * 16u);
  }
  wg_end(ctrl, st, host_epoch, grid, timing, idle);
}

// ---- ablation: the one-shot reduce behind a grid-wide barrier ----------------------------
// What the barrier-free protocols replace: "Every Microsecond Matters"
// (agihunt.info summary, the paragraph on where the time goes) locates the
// gap to the speed of light in the global memory barrier that earlier
// implementations place at every synchronisation step.  This kernel is the
// one-shot reduce written that way, for measurement: ranks 1..N-1 store
// their raw vectors into the LL staging region (no flag), every workgroup
// arrives at a grid-wide barrier once its stores are acknowledged, and only
// then do rank 0's workgroups read the staging, reduce (binary64, rank
// order, one rounding: the same result as LL and Sentinel) and zero what
// they read, which leaves those bytes invalid LL lines (epoch 0).  The
// barrier is sense-reversing (arrival count plus generation), so it needs no
// host state between calls and works under graph replay.
template <int kKind, int N, bool kLocal>
__global__ void __launch_bounds__(512) k_oneshot_barrier(OneShotArgs a) {
  int r;
  uint32_t w;
  decode_role_t<kLocal, N>(blockIdx.x, r, w);
  const uint8_t* const src = a.part[r];
  uint8_t* const out = a.out;
  uint8_t* const stage = a.stage;
  Ctrl* const ctrl = a.ctrl;
  const uint64_t nbytes = a.nbytes, spin_limit = a.spin_limit;
  const uint32_t slices = a.slices, vq = a.vq, vr = a.vr, stage_bytes = a.stage_bytes;
  const uint32_t parity_stride = a.parity_stride, rank_stride = a.rank_stride, grid = a.grid;
  const uint32_t timing = a.timing, drop_rank = a.drop_rank, host_epoch = a.host_epoch;
  LLAR_UNIFORM_AT_ENTRY("s"(src), "s"(out), "s"(stage), "s"(ctrl), "s"(nbytes), "s"(spin_limit), "s"(slices),
                        "s"(vq), "s"(vr), "s"(stage_bytes), "s"(parity_stride), "s"(rank_stride), "s"(grid),
                        "s"(timing), "s"(drop_rank), "s"(host_epoch));
  const bool idle = (w >= slices);
  const uint32_t v0 = idle ? 0u : w * vq + min(w, vr);
  const uint32_t v1 = idle ? 0u : v0 + vq + (w < vr ? 1u : 0u);
  WgState st = wg_begin(ctrl, host_epoch, timing, idle);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(stage, stage_bytes);
  const uint32_t par_off = (st.epoch & 1u) * parity_stride;
  // phase 1: ranks 1..N-1 store their raw vectors
  if (!idle && r != 0 && (uint32_t)r != drop_rank) {
    const uint32_t base = par_off + (uint32_t)(r - 1) * rank_stride;
    for (uint32_t v = v0 + threadIdx.x; v < v1; v += blockDim.x) {
      const uint64_t off = (uint64_t)v * 16u;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (off + 16u <= nbytes) {
        x = *reinterpret_cast<const u32x4*>(src + off);
      } else {
#pragma unroll
        for (uint32_t b = 0; b < 16u; b += 2u)
          if (off + b < nbytes) x[b >> 2] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(src + off + b)) << ((b & 2u) * 8u);
      }
      st16_stage<kLocal>(rs, base + v * 16u, x);
    }
  }
  // the grid-wide barrier (sense-reversing): read the generation, arrive;
  // the last arrival resets the count and advances the generation, which
  // releases everybody
  __shared__ uint32_t s_dead;
  drain_vm();
  __syncthreads();
  if (threadIdx.x == 0) {
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(ctrl, (uint32_t)sizeof(Ctrl));
    const uint32_t gen_off = (uint32_t)offsetof(Ctrl, bar_gen);
    const uint32_t gen = ld4_coh(cr, gen_off);
    const uint32_t ticket = __hip_atomic_fetch_add(&ctrl->bar_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t dead = 0u;
    if (ticket == grid - 1u) {
      __hip_atomic_store(&ctrl->bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      drain_vm();  // the reset lands before anybody is released
      __hip_atomic_fetch_add(&ctrl->bar_gen, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      Spin spin(spin_limit);
      while (ld4_coh(cr, gen_off) == gen) {
        if (spin.expired()) {
          raise_status(ctrl, kStatusTimeout);
          dead = 1u;
          break;
        }
      }
    }
    s_dead = dead;
  }
  __syncthreads();
  // phase 2: rank 0 reduces what the barrier guarantees is there
  if (!idle && r == 0 && s_dead == 0u) {
    for (uint32_t u = 2u * v0 + threadIdx.x; u < 2u * v1; u += blockDim.x) {
      const uint64_t off = (uint64_t)u * 8u;
      u32x2 own = {0u, 0u};
      if (off + 8u <= nbytes) {
        own = *reinterpret_cast<const u32x2*>(src + off);
      } else {
#pragma unroll
        for (uint32_t b = 0; b < 8u; b += 2u)
          if (off + b < nbytes) own[b >> 2] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(src + off + b)) << ((b & 2u) * 8u);
      }
      u32x2 d[N > 1 ? N - 1 : 1];
      d[0] = u32x2{0u, 0u};
#pragma unroll
      for (int k = 0; k < N - 1; ++k) d[k] = ld8_coh(rs, par_off + (uint32_t)k * rank_stride + u * 8u);
      const u32x2 s = reduce_unit_at<kKind, N>(own, 0, d);
      if (off + 8u <= nbytes) {
        *reinterpret_cast<u32x2*>(out + off) = s;
      } else {
#pragma unroll
        for (uint32_t b = 0; b < 8u; b += 2u)
          if (off + b < nbytes) *reinterpret_cast<uint16_t*>(out + off + b) = (uint16_t)(s[b >> 2] >> ((b & 2u) * 8u));
      }
#pragma unroll
      for (int k = 0; k < N - 1; ++k) st8_stage<kLocal>(rs, par_off + (uint32_t)k * rank_stride + u * 8u, u32x2{0u, 0u});
    }
  }
  wg_end(ctrl, st, host_epoch, grid, timing, idle);
}

template <int kKind, int N>
hipError_t launch_multi_n(const LaunchSpec& ls, hipStream_t stream) {
  const dim3 grid(ls.grid), block(ls.threads);
  switch (ls.kernel) {
    case kKernRsLL: hipLaunchKernelGGL((k_multi<kWireLL, kKind, N, false, false>), grid, block, 0, stream, ls.multi); break;
    case kKernRsSentinel: hipLaunchKernelGGL((k_multi<kWireSentinel, kKind, N, false, false>), grid, block, 0, stream, ls.multi); break;
    case kKernAgLL: hipLaunchKernelGGL((k_multi<kWireLL, kKind, N, true, false>), grid, block, 0, stream, ls.multi); break;
    case kKernAgSentinel: hipLaunchKernelGGL((k_multi<kWireSentinel, kKind, N, true, false>), grid, block, 0, stream, ls.multi); break;
    case kKernRsLLLocal: hipLaunchKernelGGL((k_multi<kWireLL, kKind, N, false, true>), grid, block, 0, stream, ls.multi); break;
    case kKernRsSentinelLocal: hipLaunchKernelGGL((k_multi<kWireSentinel, kKind, N, false, true>), grid, block, 0, stream, ls.multi); break;
    case kKernAgLLLocal: hipLaunchKernelGGL((k_multi<kWireLL, kKind, N, true, true>), grid, block, 0, stream, ls.multi); break;
    case kKernAgSentinelLocal: hipLaunchKernelGGL((k_multi<kWireSentinel, kKind, N, true, true>), grid, block, 0, stream, ls.multi); break;
    case kKernRsLL128Acc32: hipLaunchKernelGGL((k_rs_ll128<kKind, 0, N>), grid, block, 0, stream, ls.multi); break;
    case kKernBarrier: hipLaunchKernelGGL((k_oneshot_barrier<kKind, N, false>), grid, block, 0, stream, ls.oneshot); break;
    case kKernBarrierLocal: hipLaunchKernelGGL((k_oneshot_barrier<kKind, N, true>), grid, block, 0, stream, ls.oneshot); break;
    case kKernRsLL128Acc16:
      if constexpr (kKind != kKindF32) {
        hipLaunchKernelGGL((k_rs_ll128<kKind, 1, N>), grid, block, 0, stream, ls.multi);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kKind, int N>
int occupancy_multi_n(int kernel, int threads) {
  int blocks = 0;
  hipError_t err = hipErrorInvalidValue;
  switch (kernel) {
    case kKernRsLL: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireLL, kKind, N, false, false>, threads, 0); break;
    case kKernRsSentinel: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireSentinel, kKind, N, false, false>, threads, 0); break;
    case kKernAgLL: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireLL, kKind, N, true, false>, threads, 0); break;
    case kKernAgSentinel: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireSentinel, kKind, N, true, false>, threads, 0); break;
    case kKernRsLLLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireLL, kKind, N, false, true>, threads, 0); break;
    case kKernRsSentinelLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireSentinel, kKind, N, false, true>, threads, 0); break;
    case kKernAgLLLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireLL, kKind, N, true, true>, threads, 0); break;
    case kKernAgSentinelLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_multi<kWireSentinel, kKind, N, true, true>, threads, 0); break;
    case kKernRsLL128Acc32: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_rs_ll128<kKind, 0, N>, threads, 0); break;
    case kKernBarrier: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot_barrier<kKind, N, false>, threads, 0); break;
    case kKernBarrierLocal: err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_oneshot_barrier<kKind, N, true>, threads, 0); break;
    case kKernRsLL128Acc16:
      if constexpr (kKind != kKindF32) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_rs_ll128<kKind, 1, N>, threads, 0);
      break;
    default: break;
  }
  return err == hipSuccess ? blocks : 0;
}

template <int kKind>
hipError_t launch_multi_kind(const LaunchSpec& ls, hipStream_t stream) {
  switch (ls.n_ranks) {
    case 1: return launch_multi_n<kKind, 1>(ls, stream);
    case 2: return launch_multi_n<kKind, 2>(ls, stream);
    case 3: return launch_multi_n<kKind, 3>(ls, stream);
    case 4: return launch_multi_n<kKind, 4>(ls, stream);
    case 5: return launch_multi_n<kKind, 5>(ls, stream);
    case 6: return launch_multi_n<kKind, 6>(ls, stream);
    case 7: return launch_multi_n<kKind, 7>(ls, stream);
    case 8: return launch_multi_n<kKind, 8>(ls, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int kKind>
int occupancy_multi_kind(int n_ranks, int kernel, int threads) {
  switch (n_ranks) {
    case 1: return occupancy_multi_n<kKind, 1>(kernel, threads);
    case 2: return occupancy_multi_n<kKind, 2>(kernel, threads);
    case 3: return occupancy_multi_n<kKind, 3>(kernel, threads);
    case 4: return occupancy_multi_n<kKind, 4>(kernel, threads);
    case 5: return occupancy_multi_n<kKind, 5>(kernel, threads);
    case 6: return occupancy_multi_n<kKind, 6>(kernel, threads);
    case 7: return occupancy_multi_n<kKind, 7>(kernel, threads);
    case 8: return occupancy_multi_n<kKind, 8>(kernel, threads);
    default: return 0;
  }
}

}  // namespace

hipError_t launch_multi(const LaunchSpec& ls, hipStream_t stream) {
  switch (ls.kind) {
    case kKindF32: return launch_multi_kind<kKindF32>(ls, stream);
    case kKindF16: return launch_multi_kind<kKindF16>(ls, stream);
    case kKindBF16: return launch_multi_kind<kKindBF16>(ls, stream);
    default: return hipErrorInvalidValue;
  }
}

int occupancy_multi(int kind, int n_ranks, int kernel, int threads) {
  switch (kind) {
    case kKindF32: return occupancy_multi_kind<kKindF32>(n_ranks, kernel, threads);
    case kKindF16: return occupancy_multi_kind<kKindF16>(n_ranks, kernel, threads);
    case kKindBF16: return occupancy_multi_kind<kKindBF16>(n_ranks, kernel, threads);
    default: return 0;
  }
}

}  // namespace llar
