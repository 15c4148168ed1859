// Single-token decode step of the selective scan for gfx950.
//
// One step of the recurrence on a stored state (reading guide FAQ: a fixed
// D x N state per layer, constant time per token, no KV cache), with the same
// discretisation, readout and gate as the forward (reading guide, Method and
// S6; "Mamba / MambaMini" Q&A on Delta*B and SiLU; CSDN "Mamba" 3(1) for D).
//
// The step is a pure read-modify-write stream over the float32 state, so it
// is laid out for HBM: each lane owns Q = min(N, 4) consecutive states of one
// channel (one 16-byte load and store), the N/Q lanes of a channel are
// neighbours, and the readout C . h is reduced across them with shuffles.

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

template <typename T, int N>
__global__ __launch_bounds__(256) void state_update_kernel(
    float* __restrict__ state, const T* __restrict__ x, const T* __restrict__ dtp,
    const float* __restrict__ A, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, const T* __restrict__ zp,
    const float* __restrict__ bias, int softplus, T* __restrict__ out,
    int64_t batch, int64_t dim) {
  constexpr int Q = N < 4 ? N : 4;   // states per lane
  constexpr int LPC = N / Q;         // lanes per channel
  const int64_t total = batch * dim * LPC;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool valid = i < total;
  const int64_t ic = valid ? i : total - 1;
  const int64_t bd = ic / LPC;               // (b, d) flattened
  const int q = static_cast<int>(ic - bd * LPC);
  const int64_t b = bd / dim;
  const int64_t d = bd - b * dim;

  float s = to_f32(dtp[bd]) + (bias ? bias[d] : 0.0f);
  const float dl = softplus ? softplus_f32(s) : s;
  const float xv = to_f32(x[bd]);
  const float du = dl * xv;

  float* hp = state + bd * N + q * Q;
  const float* ap = A + d * N + q * Q;
  const T* bp = Bm + b * N + q * Q;
  const T* cp = Cm + b * N + q * Q;

  float h[Q];
  float a2[Q];
  if constexpr (Q == 4) {
    const float4 hv = *reinterpret_cast<const float4*>(hp);
    const float4 av = *reinterpret_cast<const float4*>(ap);
    h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    a2[0] = av.x; a2[1] = av.y; a2[2] = av.z; a2[3] = av.w;
  } else {
#pragma unroll
    for (int j = 0; j < Q; ++j) { h[j] = hp[j]; a2[j] = ap[j]; }
  }
  float y = 0.0f;
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    const float a = exp2_hw(dl * (a2[j] * kLog2e));
    h[j] = fmaf(a, h[j], du * to_f32(bp[j]));
    y = fmaf(to_f32(cp[j]), h[j], y);
  }
  if (valid) {
    if constexpr (Q == 4) {
      *reinterpret_cast<float4*>(hp) = make_float4(h[0], h[1], h[2], h[3]);
    } else {
#pragma unroll
      for (int j = 0; j < Q; ++j) hp[j] = h[j];
    }
  }
  // reduce the partial readouts of the channel's LPC neighbouring lanes
#pragma unroll
  for (int off = 1; off < LPC; off <<= 1) y += __shfl_xor(y, off, 64);
  if (valid && q == 0) {
    y += (Dv ? Dv[d] : 0.0f) * xv;
    if (zp) y = silu_gate(y, to_f32(zp[bd]));
    store_act(out, bd, y);
  }
}

template <typename T>
static hipError_t launch_n(int n, float* state, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* bias, int softplus, void* out, int64_t batch,
                           int64_t dim, hipStream_t stream) {
  const int lpc = n < 4 ? 1 : n / 4;
  const int64_t total = batch * dim * lpc;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const dim3 grid(static_cast<unsigned>(blocks));
#define SSM_LAUNCH_SU(NN)                                                                       \
  hipLaunchKernelGGL((state_update_kernel<T, NN>), grid, dim3(threads), 0, stream, state,       \
                     static_cast<const T*>(x), static_cast<const T*>(dt), A,                    \
                     static_cast<const T*>(B), static_cast<const T*>(C), D,                     \
                     static_cast<const T*>(z), bias, softplus, static_cast<T*>(out), batch, dim)
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
  return hipGetLastError();
}

hipError_t launch_state_update(int dtype, int dstate, float* state, const void* x,
                               const void* dt, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* dt_bias,
                               int softplus, void* out, int64_t batch, int64_t dim,
                               hipStream_t stream) {
  if (dtype == 0)
    return launch_n<float>(dstate, state, x, dt, A, B, C, D, z, dt_bias, softplus, out, batch,
                           dim, stream);
  return launch_n<bf16_t>(dstate, state, x, dt, A, B, C, D, z, dt_bias, softplus, out, batch,
                          dim, stream);
}

}  // namespace ssm
