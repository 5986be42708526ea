// llar_floor.hip -- single-GPU analogues of the speed-of-light terms.
//
// "Every Microsecond Matters" (agihunt.info summary), paragraph on the
// speed-of-light bound: an AllReduce needs at least two L2 round trips plus
// one remote write (0.306 us and 0.792 us on GB200, 1.404 us in total).  With
// the ranks emulated on one MI355X the analogues are:
//   L2 round trip   -- one device-coherent (sc1) load of an L2-resident line,
//                      measured as ns per hop of a dependent pointer chase;
//   remote write    -- the time from a 16-byte coherent store on one XCD to
//                      its observation by a poller on another XCD, measured
//                      as half of a store/poll ping-pong round trip.
// Plus the launch interval of an empty kernel, the latency of a returning
// device-scope atomic and the streaming copy bandwidth used as HBM reference.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "llar.h"
#include "llar_device.h"

using namespace llar;

namespace {

__global__ void k_floor_chase(const uint32_t* ring, uint32_t ring_bytes, int hops, uint64_t* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(ring, ring_bytes);
  uint32_t idx = 0;
  for (int i = 0; i < 64; ++i) idx = ld4_coh(rs, idx * 4u);  // warm the lines
  idx = 0;
  uint64_t t0 = wall_ticks();
  for (int i = 0; i < hops; ++i) idx = ld4_coh(rs, idx * 4u);
  uint64_t t1 = wall_ticks();
  out[0] = t1 - t0;
  out[1] = idx;
}

// Workgroups wa and wb play ping-pong with 16-byte coherent stores on two
// separate 256-byte-apart lines; the others return at once.  Each wait is
// bounded by `spin_limit` polls; out[1] / out[3] report success.
__global__ void k_floor_pingpong(uint32_t* flags, int iters, int wa, int wb, long long spin_limit, uint64_t* out) {
  const int b = blockIdx.x;
  if (threadIdx.x != 0 || (b != wa && b != wb)) return;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(flags, 1024);
  const bool ping = (b == wa);
  const uint32_t mine = ping ? 0u : 256u, theirs = ping ? 256u : 0u;
  long long spins = 0;
  int ok = 1;
  uint64_t t0 = wall_ticks();
  for (int i = 1; i <= iters && ok; ++i) {
    const uint32_t u = (uint32_t)i;
    if (ping) st16_coh(rs, mine, u32x4{u, u, u, u});
    while (true) {
      u32x4 v = ld16_coh(rs, theirs);
      if (v[3] == u) break;
      if (++spins > spin_limit) {
        ok = 0;
        break;
      }
    }
    if (!ping && ok) st16_coh(rs, mine, u32x4{u, u, u, u});
  }
  uint64_t t1 = wall_ticks();
  if (ping) {
    out[0] = t1 - t0;
    out[1] = (uint64_t)ok;
  } else {
    out[3] = (uint64_t)ok;
  }
}

__global__ void k_floor_atomic(uint32_t* p, int iters, uint64_t* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  uint32_t v = 0;
  uint64_t t0 = wall_ticks();
  for (int i = 0; i < iters; ++i)
    v = __hip_atomic_fetch_add(p + (v & 1u) * 64u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t t1 = wall_ticks();
  out[0] = t1 - t0;
  out[1] = v;
}

// The L2 round trip to a line another workgroup has just written: workgroup
// wb writes a ring of `lines` 128-byte lines with device-coherent stores
// (word 0 of each line names the next line, a fixed pseudo-random cycle),
// drains and raises a flag; workgroup 0, on XCD 0, waits for the flag
// (bounded) and follows the ring once, so every hop is its first read of a
// line last written from XCD wb % 8.  Out-of-range indices read zero through
// the buffer descriptor, so a wrong chain cannot leave the ring.
__global__ void k_floor_chase_written(uint32_t* ring, uint32_t lines, uint32_t stride, int wb, uint32_t* flag,
                                      long long spin_limit, uint64_t* out) {
  const int b = blockIdx.x;
  const uint32_t ring_bytes = lines * 128u;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(ring, ring_bytes);
  const __amdgpu_buffer_rsrc_t rf = make_rsrc(flag, 64u);
  if (b == wb) {
    for (uint32_t i = threadIdx.x; i < lines; i += blockDim.x) {
      const uint32_t next = ((i + 1u) * stride) % lines;
      const uint32_t here = (i * stride) % lines;
      st16_coh(rs, here * 128u, u32x4{next, 0u, 0u, 0u});
    }
    drain_vm();
    __syncthreads();
    if (threadIdx.x == 0) st16_coh(rf, 0u, u32x4{1u, 1u, 1u, 1u});
    return;
  }
  if (b != 0 || threadIdx.x != 0) return;
  long long spins = 0;
  int ok = 1;
  while (ld4_coh(rf, 0u) != 1u) {
    if (++spins > spin_limit) {
      ok = 0;
      break;
    }
  }
  uint32_t idx = 0;
  uint64_t sum = 0;
  uint64_t t0 = wall_ticks();
  if (ok)
    for (uint32_t i = 0; i < lines; ++i) {
      idx = ld4_coh(rs, idx * 128u);
      sum += idx;
    }
  uint64_t t1 = wall_ticks();
  out[0] = t1 - t0;
  out[1] = (uint64_t)ok;
  out[2] = sum;  // every line visited once: 0 + 1 + ... + (lines - 1)
}

// Throughput of no-return device-scope float atomics with the lane pattern
// of the LL128 producers: every wave instruction adds into 64 consecutive
// dwords (two 128-byte lines).  Active workgroup a of `active` owns a window
// of `window` bytes (private windows, or one window shared by all);
// kType 0: binary32 adds, 1: packed bfloat16 pairs, 2: packed binary16 pairs.
template <int kType>
__global__ void k_floor_atomic_tp(uint8_t* region, uint32_t region_bytes, uint32_t window, int iters,
                                  int one_xcd, int shared) {
  const uint32_t b = blockIdx.x;
  if (one_xcd && (b & 7u) != 0u) return;
  const uint32_t a = one_xcd ? b >> 3 : b;
  // shared 1: one window for all; 2: workgroups 8k .. 8k+7 (one per XCD)
  // share window k, as the eight ranks of an LL128 slice share their lines
  const uint32_t base = shared == 1 ? 0u : ((shared == 2 ? a >> 3 : a) * window) % region_bytes;
  uint32_t off = (threadIdx.x * 4u) % window;
  const uint32_t step = blockDim.x * 4u;
  for (int i = 0; i < iters; ++i) {
    uint8_t* p = region + base + off;
    if constexpr (kType == 0) {
      __hip_atomic_fetch_add(reinterpret_cast<float*>(p), 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (kType == 1) {
      __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<s16x2*>(p), s16x2{(short)0x3F80, (short)0x3F80});
    } else {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_global_atomic_fadd_v2f16(reinterpret_cast<h2*>(p), h2{(_Float16)1.0f, (_Float16)1.0f});
    }
    off += step;
    if (off >= window) off -= window;
  }
}

__global__ void k_floor_empty() {}

__global__ void k_floor_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
}

double wall_hz_now() {
  int dev = 0, wc = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 100e6;
  if (hipDeviceGetAttribute(&wc, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wc <= 0) return 100e6;
  return wc * 1000.0;
}

}  // namespace

extern "C" int llar_floor_measure(int kind, int param, double* value) {
  if (!value || kind < 0 || kind > 7) return LLAR_ERR_ARG;
  const double hz = wall_hz_now();
  uint64_t* d_out = nullptr;
  uint64_t h_out[4] = {0, 0, 0, 0};
  if (hipMalloc(&d_out, 64) != hipSuccess) return LLAR_ERR_NOMEM;
  int status = LLAR_OK;
  hipError_t e = hipSuccess;
  switch (kind) {
    case 0: {  // L2 round trip: 64 lines of 128 B, pseudo-random cyclic order
      const int lines = 64, hops = 4000;
      std::vector<uint32_t> h(lines * 32, 0u);
      std::vector<int> order(lines);
      for (int i = 0; i < lines; ++i) order[i] = (i * 37) % lines;  // 37 is coprime with 64
      for (int i = 0; i < lines; ++i) h[order[i] * 32] = (uint32_t)(order[(i + 1) % lines] * 32);
      uint32_t* d = nullptr;
      e = hipMalloc(&d, h.size() * 4);
      if (e == hipSuccess) e = hipMemcpy(d, h.data(), h.size() * 4, hipMemcpyHostToDevice);
      for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
        hipLaunchKernelGGL(k_floor_chase, dim3(1), dim3(64), 0, 0, d, (uint32_t)(h.size() * 4), hops, d_out);
        e = hipDeviceSynchronize();
      }
      if (e == hipSuccess) e = hipMemcpy(h_out, d_out, 16, hipMemcpyDeviceToHost);
      if (d) (void)hipFree(d);
      *value = (double)h_out[0] / hz * 1e9 / hops;
      break;
    }
    case 1: {  // store -> visibility, half a ping-pong round trip
      if (param < 1 || param > 63) {
        status = LLAR_ERR_ARG;
        break;
      }
      uint32_t* d = nullptr;
      const int iters = 2000;
      e = hipMalloc(&d, 1024);
      for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
        e = hipMemset(d, 0, 1024);
        if (e == hipSuccess) {
          hipLaunchKernelGGL(k_floor_pingpong, dim3(64), dim3(64), 0, 0, d, iters, 0, param, 4000000LL, d_out);
          e = hipDeviceSynchronize();
        }
      }
      if (e == hipSuccess) e = hipMemcpy(h_out, d_out, 32, hipMemcpyDeviceToHost);
      if (d) (void)hipFree(d);
      if (e == hipSuccess && (h_out[1] != 1 || h_out[3] != 1)) status = LLAR_ERR_TIMEOUT;
      *value = (double)h_out[0] / hz * 1e9 / iters / 2.0;
      break;
    }
    case 2: {  // empty launch interval
      hipEvent_t a, b;
      e = hipEventCreate(&a);
      if (e == hipSuccess) e = hipEventCreate(&b);
      const int n = 2000;
      for (int i = 0; i < 100 && e == hipSuccess; ++i) hipLaunchKernelGGL(k_floor_empty, dim3(1), dim3(64), 0, 0);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e == hipSuccess) e = hipEventRecord(a, 0);
      for (int i = 0; i < n && e == hipSuccess; ++i) hipLaunchKernelGGL(k_floor_empty, dim3(1), dim3(64), 0, 0);
      if (e == hipSuccess) e = hipEventRecord(b, 0);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      *value = ms * 1e6 / n;
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
      break;
    }
    case 3: {  // returning atomic latency
      uint32_t* d = nullptr;
      const int iters = 2000;
      e = hipMalloc(&d, 1024);
      if (e == hipSuccess) e = hipMemset(d, 0, 1024);
      for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {
        hipLaunchKernelGGL(k_floor_atomic, dim3(1), dim3(64), 0, 0, d, iters, d_out);
        e = hipDeviceSynchronize();
      }
      if (e == hipSuccess) e = hipMemcpy(h_out, d_out, 16, hipMemcpyDeviceToHost);
      if (d) (void)hipFree(d);
      *value = (double)h_out[0] / hz * 1e9 / iters;
      break;
    }
    case 4: {  // streaming copy, GB/s of read + write
      if (param < 1 || param > 8192) {
        status = LLAR_ERR_ARG;
        break;
      }
      const size_t bytes = (size_t)param << 20;
      const size_t n = bytes / 16;
      u32x4 *s = nullptr, *t = nullptr;
      e = hipMalloc(&s, bytes);
      if (e == hipSuccess) e = hipMalloc(&t, bytes);
      if (e == hipSuccess) e = hipMemset(s, 1, bytes);
      hipEvent_t a, b;
      if (e == hipSuccess) e = hipEventCreate(&a);
      if (e == hipSuccess) e = hipEventCreate(&b);
      const int reps = 10;
      if (e == hipSuccess) {
        hipLaunchKernelGGL(k_floor_copy, dim3(1024), dim3(256), 0, 0, s, t, n);
        e = hipDeviceSynchronize();
      }
      if (e == hipSuccess) e = hipEventRecord(a, 0);
      for (int i = 0; i < reps && e == hipSuccess; ++i) hipLaunchKernelGGL(k_floor_copy, dim3(1024), dim3(256), 0, 0, s, t, n);
      if (e == hipSuccess) e = hipEventRecord(b, 0);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      *value = ms > 0.f ? 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9 : 0.0;
      if (s) (void)hipFree(s);
      if (t) (void)hipFree(t);
      (void)hipEventDestroy(a);
      (void)hipEventDestroy(b);
      break;
    }
    case 5: {  // L2 round trip to lines last written from another workgroup (param = its id)
      if (param < 1 || param > 63) {
        status = LLAR_ERR_ARG;
        break;
      }
      const uint32_t lines = 4096, stride = 1031;  // 512 KiB; 1031 is prime, so the cycle visits every line
      uint32_t *ring = nullptr, *flag = nullptr;
      e = hipMalloc(&ring, (size_t)lines * 128);
      if (e == hipSuccess) e = hipMalloc(&flag, 64);
      double best = 0.0;
      for (int rep = 0; rep < 3 && e == hipSuccess; ++rep) {
        e = hipMemset(ring, 0, (size_t)lines * 128);
        if (e == hipSuccess) e = hipMemset(flag, 0, 64);
        if (e == hipSuccess) {
          hipLaunchKernelGGL(k_floor_chase_written, dim3(64), dim3(256), 0, 0, ring, lines, stride, param, flag,
                             4000000LL, d_out);
          e = hipDeviceSynchronize();
        }
        if (e == hipSuccess) e = hipMemcpy(h_out, d_out, 24, hipMemcpyDeviceToHost);
        if (e == hipSuccess && h_out[1] != 1) status = LLAR_ERR_TIMEOUT;
        // the chain must visit every line once (a stale read would repeat one)
        if (e == hipSuccess && status == LLAR_OK && h_out[2] != (uint64_t)lines * (lines - 1) / 2) status = LLAR_ERR_DEVICE;
        const double ns = (double)h_out[0] / hz * 1e9 / lines;
        if (rep == 0 || ns < best) best = ns;
      }
      if (ring) (void)hipFree(ring);
      if (flag) (void)hipFree(flag);
      *value = best;
      break;
    }
    case 6: {  // empty kernels replayed from a graph of `param` launches, ns per launch
      const int per = param > 0 ? std::min(param, 10000) : 100;
      hipStream_t st = nullptr;
      hipGraph_t g = nullptr;
      hipGraphExec_t ge = nullptr;
      hipEvent_t a = nullptr, b = nullptr;
      e = hipStreamCreate(&st);
      if (e == hipSuccess) e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
      for (int i = 0; i < per && e == hipSuccess; ++i) {
        hipLaunchKernelGGL(k_floor_empty, dim3(1), dim3(64), 0, st);
        e = hipGetLastError();
      }
      if (e == hipSuccess) e = hipStreamEndCapture(st, &g);
      if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
      if (e == hipSuccess) e = hipEventCreate(&a);
      if (e == hipSuccess) e = hipEventCreate(&b);
      const int reps = 20;
      for (int i = 0; i < 2 && e == hipSuccess; ++i) e = hipGraphLaunch(ge, st);
      if (e == hipSuccess) e = hipStreamSynchronize(st);
      if (e == hipSuccess) e = hipEventRecord(a, st);
      for (int i = 0; i < reps && e == hipSuccess; ++i) e = hipGraphLaunch(ge, st);
      if (e == hipSuccess) e = hipEventRecord(b, st);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      *value = ms * 1e6 / ((double)reps * per);
      if (ge) (void)hipGraphExecDestroy(ge);
      if (g) (void)hipGraphDestroy(g);
      if (a) (void)hipEventDestroy(a);
      if (b) (void)hipEventDestroy(b);
      if (st) (void)hipStreamDestroy(st);
      break;
    }
    case 7: {  // atomic throughput, G lane operations per second
      // param: bits 0-1 type (0 binary32, 1 packed bfloat16, 2 packed
      // binary16), bit 2: issue from one XCD only, bits 3-4: 1 = all
      // workgroups share one window, 2 = groups of eight consecutive
      // workgroups share one, 0 = each has its own
      const int type = param & 3, one_xcd = (param >> 2) & 1, shared = (param >> 3) & 3;
      if (type > 2 || param < 0 || param > 31 || shared == 3) {
        status = LLAR_ERR_ARG;
        break;
      }
      const uint32_t region_bytes = 16u << 20, window = 8192u;
      const int grid = 2048, threads = 256, iters = 256;
      uint8_t* region = nullptr;
      e = hipMalloc(&region, region_bytes);
      if (e == hipSuccess) e = hipMemset(region, 0, region_bytes);
      hipEvent_t a = nullptr, b = nullptr;
      if (e == hipSuccess) e = hipEventCreate(&a);
      if (e == hipSuccess) e = hipEventCreate(&b);
      auto run = [&]() {
        if (type == 0)
          hipLaunchKernelGGL(k_floor_atomic_tp<0>, dim3(grid), dim3(threads), 0, 0, region, region_bytes, window, iters,
                             one_xcd, shared);
        else if (type == 1)
          hipLaunchKernelGGL(k_floor_atomic_tp<1>, dim3(grid), dim3(threads), 0, 0, region, region_bytes, window, iters,
                             one_xcd, shared);
        else
          hipLaunchKernelGGL(k_floor_atomic_tp<2>, dim3(grid), dim3(threads), 0, 0, region, region_bytes, window, iters,
                             one_xcd, shared);
      };
      if (e == hipSuccess) {
        run();
        e = hipDeviceSynchronize();
      }
      if (e == hipSuccess) e = hipEventRecord(a, 0);
      if (e == hipSuccess) run();
      if (e == hipSuccess) e = hipEventRecord(b, 0);
      if (e == hipSuccess) e = hipEventSynchronize(b);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
      const double active = one_xcd ? grid / 8.0 : (double)grid;
      *value = ms > 0.f ? active * threads * iters / (ms * 1e-3) / 1e9 : 0.0;
      if (a) (void)hipEventDestroy(a);
      if (b) (void)hipEventDestroy(b);
      if (region) (void)hipFree(region);
      break;
    }
    default:
      status = LLAR_ERR_ARG;
  }
  (void)hipFree(d_out);
  if (status == LLAR_OK && e != hipSuccess) status = LLAR_ERR_HIP;
  return status;
}
