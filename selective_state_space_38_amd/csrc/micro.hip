// Ceiling probes for the roofline figures the benchmark reports: the rate of
// fp32 fused multiply-adds and of the hardware exponential (v_exp_f32) on
// the vector ALUs, their mix in the proportion of a scan step, and streaming
// HBM bandwidth (read, write, copy, in-place read-modify-write) with 16-byte
// accesses.  Each entry point times `reps` launches between two HIP events
// on the caller's stream and returns the average milliseconds per launch.
// Declarations and argument meaning: include/ssm_micro.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm_micro.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// KIND 0: v = v*a + b (one FMA per element-step); 1: v = exp2(-v) (one
// v_exp_f32 with a negated operand); 2: one exp2 and four FMAs per
// element-step, the ratio of transcendentals to multiply-adds in the scan's
// per-state update.  CH independent chains per lane (CH = 1: every
// instruction waits on the one before).  The values stay in [0.5, 1], so no
// denormal or infinite operand occurs.
template <int KIND, int CH>
__global__ __launch_bounds__(256) void valu_probe(const float* __restrict__ seed,
                                                  float* __restrict__ sink, int iters) {
  const float a = seed[0], b = seed[1];
  float v[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) v[k] = seed[2 + (k & 7)] + static_cast<float>(threadIdx.x) * 1e-7f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        if constexpr (KIND == 0) {
          v[k] = fmaf(v[k], a, b);
        } else if constexpr (KIND == 1) {
          v[k] = __builtin_amdgcn_exp2f(-v[k]);
        } else {
          float e = __builtin_amdgcn_exp2f(-v[k]);
          e = fmaf(e, a, b);
          e = fmaf(e, a, b);
          e = fmaf(e, a, b);
          v[k] = fmaf(e, a, b);
        }
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < CH; ++k) s += v[k];
  // keeps every chain live; the seeds never produce this value
  if (s == -1.0f) sink[threadIdx.x] = s;
}

// MODE 0 read, 1 write, 2 copy (src -> dst), 3 read-modify-write in place
// (dst += 1 per word).  Grid-stride over 16-byte vectors, U vectors in
// flight per thread, non-temporal hints (the data is touched once).
template <int MODE, int U>
__global__ __launch_bounds__(256) void stream_probe(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, int64_t n_vec,
                                                    uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const u32x4 one = {1u, 1u, 1u, 1u};
  for (; i + (U - 1) * stride < n_vec; i += U * stride) {
    u32x4 v[U];
    if constexpr (MODE != 1) {
#pragma unroll
      for (int k = 0; k < U; ++k)
        v[k] = __builtin_nontemporal_load((MODE == 3 ? dst : src) + i + k * stride);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      if constexpr (MODE == 0) {
        acc ^= v[k];
      } else if constexpr (MODE == 1) {
        const uint32_t w = static_cast<uint32_t>(i + k * stride);
        const u32x4 o = {w, w, w, w};
        __builtin_nontemporal_store(o, dst + i + k * stride);
      } else if constexpr (MODE == 2) {
        __builtin_nontemporal_store(v[k], dst + i + k * stride);
      } else {
        __builtin_nontemporal_store(v[k] + one, dst + i + k * stride);
      }
    }
  }
  for (; i < n_vec; i += stride) {
    if constexpr (MODE == 0) {
      acc ^= __builtin_nontemporal_load(src + i);
    } else if constexpr (MODE == 1) {
      const uint32_t w = static_cast<uint32_t>(i);
      const u32x4 o = {w, w, w, w};
      __builtin_nontemporal_store(o, dst + i);
    } else if constexpr (MODE == 2) {
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    } else {
      __builtin_nontemporal_store(__builtin_nontemporal_load(dst + i) + one, dst + i);
    }
  }
  if constexpr (MODE == 0) {
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u) sink[0] = x;  // keeps the loads live
  }
}

// Times `reps` launches of `launch` between two events on `st`.
template <typename F>
int time_launches(F launch, int reps, hipStream_t st, float* ms_out) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return SSM_MICRO_ERUNTIME;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return SSM_MICRO_ERUNTIME;
  }
  int rc = SSM_MICRO_OK;
  launch();  // warm-up
  if (hipGetLastError() != hipSuccess) rc = SSM_MICRO_ERUNTIME;
  if (rc == SSM_MICRO_OK && hipEventRecord(e0, st) != hipSuccess) rc = SSM_MICRO_ERUNTIME;
  for (int r = 0; rc == SSM_MICRO_OK && r < reps; ++r) {
    launch();
    if (hipGetLastError() != hipSuccess) rc = SSM_MICRO_ERUNTIME;
  }
  float ms = 0.0f;
  if (rc == SSM_MICRO_OK && (hipEventRecord(e1, st) != hipSuccess ||
                             hipEventSynchronize(e1) != hipSuccess ||
                             hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
    rc = SSM_MICRO_ERUNTIME;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc == SSM_MICRO_OK) *ms_out = ms / static_cast<float>(reps);
  return rc;
}

}  // namespace

extern "C" {

int ssm_micro_valu(int kind, int chains, int blocks, int iters, const float* seed, float* sink,
                   int reps, float* ms_out, void* stream) {
  if (kind < 0 || kind > 2 || (chains != 1 && chains != 8) || blocks <= 0 || iters <= 0 ||
      reps <= 0 || !seed || !sink || !ms_out)
    return SSM_MICRO_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  auto launch = [&]() {
#define SSM_VALU(K, C) hipLaunchKernelGGL((valu_probe<K, C>), grid, block, 0, st, seed, sink, iters)
    if (chains == 1) {
      if (kind == 0) SSM_VALU(0, 1);
      else if (kind == 1) SSM_VALU(1, 1);
      else SSM_VALU(2, 1);
    } else {
      if (kind == 0) SSM_VALU(0, 8);
      else if (kind == 1) SSM_VALU(1, 8);
      else SSM_VALU(2, 8);
    }
#undef SSM_VALU
  };
  return time_launches(launch, reps, st, ms_out);
}

int ssm_micro_stream(int mode, int unroll, int blocks, const void* src, void* dst,
                     int64_t bytes, int slices, void* sink, int reps, float* ms_out,
                     void* stream) {
  if (mode < 0 || mode > 3 || (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) ||
      blocks <= 0 || bytes <= 0 || bytes % 16 != 0 || slices <= 0 || reps <= 0 || !dst ||
      !sink || !ms_out || ((mode == 0 || mode == 2) && !src))
    return SSM_MICRO_EINVAL;
  if (reinterpret_cast<uintptr_t>(dst) % 16 != 0 ||
      (src && reinterpret_cast<uintptr_t>(src) % 16 != 0))
    return SSM_MICRO_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n_vec = bytes / 16;
  uint32_t* k = static_cast<uint32_t*>(sink);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  int launch_no = 0;
  auto launch = [&]() {
    // launch i works on slice i mod slices of the buffers
    const int64_t off = static_cast<int64_t>(launch_no++ % slices) * n_vec;
    const u32x4* s = src ? static_cast<const u32x4*>(src) + off : nullptr;
    u32x4* d = static_cast<u32x4*>(dst) + off;
#define SSM_STREAM(M, U) \
  hipLaunchKernelGGL((stream_probe<M, U>), grid, block, 0, st, s, d, n_vec, k)
#define SSM_STREAM_U(M)                  \
  switch (unroll) {                      \
    case 1: SSM_STREAM(M, 1); break;     \
    case 2: SSM_STREAM(M, 2); break;     \
    case 4: SSM_STREAM(M, 4); break;     \
    default: SSM_STREAM(M, 8); break;    \
  }
    switch (mode) {
      case 0: SSM_STREAM_U(0); break;
      case 1: SSM_STREAM_U(1); break;
      case 2: SSM_STREAM_U(2); break;
      default: SSM_STREAM_U(3); break;
    }
#undef SSM_STREAM_U
#undef SSM_STREAM
  };
  return time_launches(launch, reps, st, ms_out);
}

}  // extern "C"
