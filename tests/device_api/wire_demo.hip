// wire_demo.hip -- custom kernels written only against the public device-side
// header llar_wire.h, the way a kernel author would use it: each fuses its
// own arithmetic with a barrier-free exchange between emulated ranks.
//
//   demo_scaled_allreduce_ll   an "epilogue" scales each rank's partial and
//                              puts it on the LL wire; rank 0 waits line by
//                              line and sums in rank order (binary64, one
//                              rounding to binary32).
//   demo_sentinel_chain        rank r waits for rank r-1's running sum on a
//                              Sentinel slot, adds its own value (binary32)
//                              and forwards it; the last rank writes out.
//   demo_ll128_reduce          every rank adds its binary32 values into
//                              LL128 lines and counts itself in slot 0; the
//                              line's owner waits for the count N, writes out
//                              and zeroes the line (a read and a zeroing
//                              store, or with `take` one exchange per 8
//                              bytes that reads and zeroes at once).
//
// Grids: workgroup b is (rank b % N, slice b / N), so ranks sit on different
// XCDs and every store uses the device scope.  Every launch is small enough
// for all its workgroups to be resident at once.  A wait that expires sets
// *status to 1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "llar_wire.h"

namespace {

using namespace llar_wire;

// binary32 product, rounded before any later use: the empty asm makes the
// value opaque, so the compiler cannot contract the multiply into a wider
// fused multiply-add with the sum it feeds
__device__ __forceinline__ float mul_f32(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

struct Parts {
  const float* p[8];
  float scale[8];
};

// ---- LL: scaled partials, rank 0 reduces -------------------------------------------------
template <int N>
__global__ void __launch_bounds__(256) k_scaled_allreduce_ll(Parts in, float* out, uint32_t n, uint8_t* stage,
                                                              uint32_t stage_bytes, uint32_t epoch, uint64_t spin,
                                                              uint32_t* status) {
  const int r = (int)(blockIdx.x % N);
  const uint32_t w = blockIdx.x / N, slices = gridDim.x / N;
  const uint32_t units = (n + 1u) / 2u;            // 8-byte units: 2 binary32 values
  const Wire wire = make_wire(stage, stage_bytes);  // [rank 1..N-1][unit] 16-byte LL lines
  for (uint32_t u = w * blockDim.x + threadIdx.x; u < units; u += slices * blockDim.x) {
    const uint32_t i0 = 2u * u, i1 = 2u * u + 1u;
    auto scaled = [&](int k, uint32_t i) -> float { return i < n ? mul_f32(in.p[k][i], in.scale[k]) : 0.0f; };
    if (r != 0) {
      const u32x2 v = {__float_as_uint(scaled(r, i0)), __float_as_uint(scaled(r, i1))};
      ll_put<kDevice>(wire, ((uint32_t)(r - 1) * units + u) * 16u, v, epoch);
    } else {
      // poll every sender's line in one pass (all loads in flight) until a
      // pass finds them all ready; a ready line stays ready for this epoch
      u32x2 v[N - 1];
      Poll poll(spin);
      while (true) {
        bool all = true;
#pragma unroll
        for (int k = 1; k < N; ++k) all &= ll_try(wire, ((uint32_t)(k - 1) * units + u) * 16u, epoch, v[k - 1]);
        if (all) break;
        if (poll.expired()) {
          atomicOr(status, 1u);
          return;
        }
      }
      double s0 = scaled(0, i0), s1 = scaled(0, i1);
#pragma unroll
      for (int k = 1; k < N; ++k) {
        s0 += (double)__uint_as_float(v[k - 1][0]);
        s1 += (double)__uint_as_float(v[k - 1][1]);
      }
      out[i0] = (float)s0;
      if (i1 < n) out[i1] = (float)s1;
    }
  }
}

// ---- Sentinel: a relay through the ranks --------------------------------------------------
template <int N>
__global__ void __launch_bounds__(256) k_sentinel_chain(Parts in, float* out, uint32_t n, uint8_t* stage,
                                                         uint32_t stage_bytes, uint64_t spin, uint32_t* status) {
  const int r = (int)(blockIdx.x % N);
  const uint32_t w = blockIdx.x / N, slices = gridDim.x / N;
  const uint32_t vecs = (n + 3u) / 4u;              // 16-byte slots: 4 binary32 values
  const Wire wire = make_wire(stage, stage_bytes);  // [link r -> r+1][vector], all-ones when empty
  for (uint32_t v = w * blockDim.x + threadIdx.x; v < vecs; v += slices * blockDim.x) {
    float acc[4];
    if (r == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = (4u * v + t < n) ? in.p[0][4u * v + t] : 0.0f;
    } else {
      u32x4 got;
      Poll poll(spin);
      const uint32_t off = ((uint32_t)(r - 1) * vecs + v) * 16u;
      if (!sentinel_wait<4>(wire, off, poll, got)) {
        atomicOr(status, 1u);
        return;
      }
      sentinel_reset<kDevice>(wire, off);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = __uint_as_float(got[t]) + ((4u * v + t < n) ? in.p[r][4u * v + t] : 0.0f);
    }
    if (r == N - 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (4u * v + t < n) out[4u * v + t] = acc[t];
    } else {
      const u32x4 x = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
      sentinel_put<4, kDevice>(wire, ((uint32_t)r * vecs + v) * 16u, x);
    }
  }
}

// ---- LL128: atomic adds into lines, owner by line ----------------------------------------------
// Line l holds values 31 l .. 31 l + 30 in slots 1..31; slot 0 counts ranks.
// Rank r adds its values of every line, then (after release) counts itself;
// line l belongs to rank l % N, which waits for the count N.  One thread per
// line slot: 32 threads per line, 8 lines per 256-thread workgroup.
template <int N>
__global__ void __launch_bounds__(256) k_ll128_reduce(Parts in, float* out, uint32_t n, uint8_t* stage,
                                                       uint32_t stage_bytes, uint64_t spin, uint32_t* status,
                                                       uint32_t take) {
  const int r = (int)(blockIdx.x % N);
  const uint32_t w = blockIdx.x / N, slices = gridDim.x / N;
  const uint32_t lines = (n + 30u) / 31u;
  const Wire wire = make_wire(stage, stage_bytes);
  const uint32_t q = threadIdx.x & 31u;  // slot of the line
  // adds: every rank, every line
  for (uint32_t l = w * 8u + threadIdx.x / 32u; l < lines; l += slices * 8u) {
    const uint32_t i = 31u * l + q - 1u;
    if (q != 0u && i < n) ll128_add(reinterpret_cast<float*>(stage + l * kLL128LineBytes) + q, in.p[r][i]);
  }
  release();
  for (uint32_t l = w * 8u + threadIdx.x / 32u; l < lines; l += slices * 8u)
    if (q == 0u) ll128_flag(reinterpret_cast<float*>(stage + l * kLL128LineBytes));
  // owner: wait, read, zero
  const uint32_t full = __float_as_uint((float)N);
  for (uint32_t l = w * 8u + threadIdx.x / 32u; l < lines; l += slices * 8u) {
    if (l % N != (uint32_t)r) continue;
    Poll poll(spin);
    if (!ll128_wait<false>(wire, l * kLL128LineBytes, full, poll)) {
      atomicOr(status, 1u);
      return;
    }
    if (q < 8u) {  // 8 lanes read 16 bytes each
      const uint32_t off = l * kLL128LineBytes + q * 16u;
      const u32x4 x = take ? ll128_take16(stage + off) : ll128_read16(wire, off);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t s = 4u * q + t, i = 31u * l + s - 1u;
        if (s != 0u && i < n) out[i] = __uint_as_float(x[t]);
      }
      if (!take) ll128_reset16(wire, off);
    }
  }
}

int grid_for(int n_ranks, uint32_t work, uint32_t per_wg) {
  uint32_t s = (work + per_wg - 1u) / per_wg;
  if (s < 1u) s = 1u;
  if (s > 16u) s = 16u;
  return n_ranks * (int)s;
}

Parts make_parts(const float* const* parts, const float* scales, int n_ranks) {
  Parts p{};
  for (int k = 0; k < n_ranks; ++k) {
    p.p[k] = parts[k];
    p.scale[k] = scales ? scales[k] : 1.0f;
  }
  return p;
}

}  // namespace

#define DEMO_SWITCH_N(n_ranks, CALL) \
  switch (n_ranks) {                 \
    case 2: CALL(2); break;          \
    case 3: CALL(3); break;          \
    case 4: CALL(4); break;          \
    case 5: CALL(5); break;          \
    case 6: CALL(6); break;          \
    case 7: CALL(7); break;          \
    case 8: CALL(8); break;          \
    default: return -1;              \
  }

extern "C" {

// All pointers are device pointers except `parts` and `scales` (host arrays
// of n_ranks entries).  `stage` must hold the documented empty pattern before
// the call and of at least the bytes the kernel addresses:
//   LL:       (n_ranks - 1) * ceil(n / 2) * 16, zero before first use
//   Sentinel: (n_ranks - 1) * ceil(n / 4) * 16, all-ones
//   LL128:    ceil(n / 31) * 128, zero
// Returns 0, or -1 for a bad argument, -2 for a launch error.
int demo_scaled_allreduce_ll(const float* const* parts, const float* scales, float* out, uint32_t n, int n_ranks,
                             void* stage, uint32_t stage_bytes, uint32_t epoch, uint64_t spin_ticks,
                             uint32_t* status, void* stream) {
  if (n == 0 || epoch == 0) return -1;
  const Parts p = make_parts(parts, scales, n_ranks);
  const int grid = grid_for(n_ranks, (n + 1u) / 2u, 256u);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define CALL(N)                                                                                              \
  hipLaunchKernelGGL(k_scaled_allreduce_ll<N>, dim3(grid), dim3(256), 0, s, p, out, n, (uint8_t*)stage, \
                     stage_bytes, epoch, spin_ticks, status)
  DEMO_SWITCH_N(n_ranks, CALL)
#undef CALL
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int demo_sentinel_chain(const float* const* parts, float* out, uint32_t n, int n_ranks, void* stage,
                        uint32_t stage_bytes, uint64_t spin_ticks, uint32_t* status, void* stream) {
  if (n == 0) return -1;
  const Parts p = make_parts(parts, nullptr, n_ranks);
  const int grid = grid_for(n_ranks, (n + 3u) / 4u, 256u);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define CALL(N)                                                                                          \
  hipLaunchKernelGGL(k_sentinel_chain<N>, dim3(grid), dim3(256), 0, s, p, out, n, (uint8_t*)stage, \
                     stage_bytes, spin_ticks, status)
  DEMO_SWITCH_N(n_ranks, CALL)
#undef CALL
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int demo_ll128_reduce(const float* const* parts, float* out, uint32_t n, int n_ranks, void* stage,
                      uint32_t stage_bytes, uint64_t spin_ticks, uint32_t* status, void* stream, int take) {
  if (n == 0) return -1;
  const Parts p = make_parts(parts, nullptr, n_ranks);
  const int grid = grid_for(n_ranks, (n + 30u) / 31u, 8u);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define CALL(N)                                                                                        \
  hipLaunchKernelGGL(k_ll128_reduce<N>, dim3(grid), dim3(256), 0, s, p, out, n, (uint8_t*)stage, \
                     stage_bytes, spin_ticks, status, take ? 1u : 0u)
  DEMO_SWITCH_N(n_ranks, CALL)
#undef CALL
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
