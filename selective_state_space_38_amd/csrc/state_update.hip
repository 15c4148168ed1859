// Single-token decode step of the selective scan for gfx950.
//
// One step of the recurrence on a stored state (reading guide FAQ: a fixed
// D x N state per layer, constant time per token, no KV cache), with the same
// discretisation, readout and gate as the forward (reading guide, Method and
// S6; "Mamba / MambaMini" Q&A on Delta*B and SiLU; CSDN "Mamba" 3(1) for D).
// With ZOH the input term is the exact zero-order-hold one of the reading
// guide's Method, (exp(Delta A) - 1) / A * B * x.
//
// The step is a pure read-modify-write stream over the float32 state, so it
// is laid out for HBM (see the kernel comment).  The shuffle partners of a
// lane are always in range: total = B*D*LPC is a multiple of LPC, which
// divides 64.

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One lane owns Q = min(N, 8) consecutive states of one channel (two 16-byte
// vector loads and stores), the N/Q lanes of a channel are neighbours and
// reduce the readout C . h with shuffles.  The state is streamed once, so it
// is read and written with non-temporal hints.  (4 and 16 states per lane
// measured slower: 16 makes the per-instruction accesses of a wave strided.)
// VBC: B and C are aligned for the same vector loads (8 bytes per 4 bfloat16,
// 16 per 4 float32); otherwise they are read element by element.
constexpr int kDecodeStatesPerLane = 8;
template <typename T, int N, bool ZOH, bool VBC>
__global__ __launch_bounds__(256) void state_update_kernel(
    float* __restrict__ state, const T* __restrict__ x, const T* __restrict__ dtp,
    const float* __restrict__ A, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, const T* __restrict__ zp,
    const float* __restrict__ bias, int softplus, T* __restrict__ out,
    int64_t batch, int64_t dim) {
  constexpr int Q = N < kDecodeStatesPerLane ? N : kDecodeStatesPerLane;
  constexpr int LPC = N / Q;               // lanes per channel
  constexpr int NV = Q >= 4 ? Q / 4 : 0;   // 16-byte vectors per lane
  const int64_t total = batch * dim * LPC;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t ic = i < total ? i : total - 1;
  const int64_t bd = ic / LPC;
  const int q = static_cast<int>(ic - bd * LPC);
  const int64_t b = bd / dim;
  const int64_t d = bd - b * dim;

  float h[Q];
  float* hp = state + bd * N + q * Q;
  if constexpr (NV > 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const f32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hp) + v);
      h[4 * v] = hv.x; h[4 * v + 1] = hv.y; h[4 * v + 2] = hv.z; h[4 * v + 3] = hv.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < Q; ++j) h[j] = __builtin_nontemporal_load(hp + j);
  }
  const float s = to_f32(dtp[bd]) + (bias ? bias[d] : 0.0f);
  const float dl = softplus ? softplus_f32(s) : s;
  const float xv = to_f32(x[bd]);
  const float du = dl * xv;
  const float* ap = A + d * N + q * Q;
  const T* bp = Bm + b * N + q * Q;
  const T* cp = Cm + b * N + q * Q;
  float a2[Q], bv[Q], cv[Q];
  if constexpr (NV > 0) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float4 av = reinterpret_cast<const float4*>(ap)[v];
      a2[4 * v] = av.x; a2[4 * v + 1] = av.y; a2[4 * v + 2] = av.z; a2[4 * v + 3] = av.w;
      if constexpr (!VBC) {
#pragma unroll
        for (int j = 4 * v; j < 4 * v + 4; ++j) {
          bv[j] = to_f32(bp[j]);
          cv[j] = to_f32(cp[j]);
        }
      } else if constexpr (sizeof(T) == 2) {
        const uint2 bw = reinterpret_cast<const uint2*>(bp)[v];
        const uint2 cw = reinterpret_cast<const uint2*>(cp)[v];
        bv[4 * v] = __uint_as_float(bw.x << 16); bv[4 * v + 1] = __uint_as_float(bw.x & 0xffff0000u);
        bv[4 * v + 2] = __uint_as_float(bw.y << 16); bv[4 * v + 3] = __uint_as_float(bw.y & 0xffff0000u);
        cv[4 * v] = __uint_as_float(cw.x << 16); cv[4 * v + 1] = __uint_as_float(cw.x & 0xffff0000u);
        cv[4 * v + 2] = __uint_as_float(cw.y << 16); cv[4 * v + 3] = __uint_as_float(cw.y & 0xffff0000u);
      } else {
        const float4 bw = reinterpret_cast<const float4*>(bp)[v];
        const float4 cw = reinterpret_cast<const float4*>(cp)[v];
        bv[4 * v] = bw.x; bv[4 * v + 1] = bw.y; bv[4 * v + 2] = bw.z; bv[4 * v + 3] = bw.w;
        cv[4 * v] = cw.x; cv[4 * v + 1] = cw.y; cv[4 * v + 2] = cw.z; cv[4 * v + 3] = cw.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      a2[j] = ap[j];
      bv[j] = to_f32(bp[j]);
      cv[j] = to_f32(cp[j]);
    }
  }
  float y = 0.0f;
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    const float x2 = dl * (a2[j] * kLog2e);
    const float a = exp2_hw(x2);
    if constexpr (ZOH) {
      h[j] = fmaf(a, h[j], zoh_coef(x2, a, dl, 1.0f / a2[j]) * (xv * bv[j]));
    } else {
      h[j] = fmaf(a, h[j], du * bv[j]);
    }
    y = fmaf(cv[j], h[j], y);
  }
  if (i < total) {
    if constexpr (NV > 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const f32x4 hv = {h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]};
        __builtin_nontemporal_store(hv, reinterpret_cast<f32x4*>(hp) + v);
      }
    } else {
#pragma unroll
      for (int j = 0; j < Q; ++j) __builtin_nontemporal_store(h[j], hp + j);
    }
  }
  // reduce the partial readouts of the channel's LPC neighbouring lanes
#pragma unroll
  for (int off = 1; off < LPC; off <<= 1) y += __shfl_xor(y, off, 64);
  if (i < total && q == 0) {
    y += (Dv ? Dv[d] : 0.0f) * xv;
    if (zp) y = silu_gate(y, to_f32(zp[bd]));
    store_act(out, bd, y);
  }
}

template <typename T>
static hipError_t launch_n(int n, float* state, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* bias, int softplus, int zoh, void* out, int64_t batch,
                           int64_t dim, hipStream_t stream) {
  // B and C rows start at b * N elements: vector loads need the base aligned
  // to 4 elements (N >= 4 keeps every row start aligned with it)
  const uintptr_t vec_bytes = 4 * sizeof(T);
  const bool vbc = reinterpret_cast<uintptr_t>(B) % vec_bytes == 0 &&
                   reinterpret_cast<uintptr_t>(C) % vec_bytes == 0;
  const int q = n < kDecodeStatesPerLane ? n : kDecodeStatesPerLane;
  const int64_t total = batch * dim * (n / q);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const dim3 grid(static_cast<unsigned>(blocks));
#define SSM_LAUNCH_SU_ZV(NN, Z, V)                                                              \
  hipLaunchKernelGGL((state_update_kernel<T, NN, Z, V>), grid, dim3(threads), 0, stream, state, \
                     static_cast<const T*>(x), static_cast<const T*>(dt), A,                    \
                     static_cast<const T*>(B), static_cast<const T*>(C), D,                     \
                     static_cast<const T*>(z), bias, softplus, static_cast<T*>(out), batch, dim)
#define SSM_LAUNCH_SU_Z(NN, Z)          \
  if (vbc) {                            \
    SSM_LAUNCH_SU_ZV(NN, Z, true);      \
  } else {                              \
    SSM_LAUNCH_SU_ZV(NN, Z, false);     \
  }
#define SSM_LAUNCH_SU(NN)         \
  if (zoh) {                      \
    SSM_LAUNCH_SU_Z(NN, true);    \
  } else {                        \
    SSM_LAUNCH_SU_Z(NN, false);   \
  }
  switch (n) {
    case 1: SSM_LAUNCH_SU(1); break;
    case 2: SSM_LAUNCH_SU(2); break;
    case 4: SSM_LAUNCH_SU(4); break;
    case 8: SSM_LAUNCH_SU(8); break;
    case 16: SSM_LAUNCH_SU(16); break;
    case 32: SSM_LAUNCH_SU(32); break;
    case 64: SSM_LAUNCH_SU(64); break;
    default: return hipErrorInvalidValue;
  }
#undef SSM_LAUNCH_SU
#undef SSM_LAUNCH_SU_Z
#undef SSM_LAUNCH_SU_ZV
  return hipGetLastError();
}

hipError_t launch_state_update(int dtype, int dstate, float* state, const void* x,
                               const void* dt, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* dt_bias,
                               int softplus, int zoh, void* out, int64_t batch, int64_t dim,
                               hipStream_t stream) {
  if (dtype == 0)
    return launch_n<float>(dstate, state, x, dt, A, B, C, D, z, dt_bias, softplus, zoh, out,
                           batch, dim, stream);
  return launch_n<bf16_t>(dstate, state, x, dt, A, B, C, D, z, dt_bias, softplus, zoh, out,
                          batch, dim, stream);
}

}  // namespace ssm
