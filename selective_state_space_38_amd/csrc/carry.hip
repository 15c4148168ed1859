// Carry combination across consecutive sequence segments, for gfx950.
//
// A segment's steps compose under the pair operator of "Mamba / MambaMini"
// Step 2, (a_j a_i, a_j b_i + b_j), into one transform; with A time-invariant
// its decay is exp(A * sum Delta), so a segment's carry record is its sum of
// Delta per (batch, channel) plus the state it reaches from zero.  Folding the
// records in sequence order from h0 gives every segment's start state (the
// exclusive prefix of Step 4) and the state after the last one.  This is the
// step between a sequence's segments being scanned independently (aggregate
// pass) and their outputs being produced from their true start states.
//
// One thread per (batch, channel, state): the records are walked serially in
// segment order; consecutive threads touch consecutive floats of every
// [batch][dim][n] array, so each access of a wave is one dense run.

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

__global__ __launch_bounds__(256) void carry_combine_kernel(
    const float* __restrict__ sum_delta, const float* __restrict__ agg,
    const float* __restrict__ A, const float* __restrict__ h0, float* __restrict__ h_in,
    float* __restrict__ h_out, int64_t segments, int64_t batch, int64_t dim, int n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t states = batch * dim * n;
  if (i >= states) return;
  const int64_t bd = i / n;  // (batch, channel)
  const int k = static_cast<int>(i - bd * n);
  const int64_t d = bd % dim;
  const float a2 = A[d * n + k] * kLog2e;
  const int64_t cols = batch * dim;
  float h = h0 ? h0[i] : 0.0f;
  for (int64_t s = 0; s < segments; ++s) {
    h_in[s * states + i] = h;
    h = fmaf(exp2_hw(a2 * sum_delta[s * cols + bd]), h, agg[s * states + i]);
  }
  if (h_out) h_out[i] = h;
}

hipError_t launch_carry_combine(const float* sum_delta, const float* agg, const float* A,
                                const float* h0, float* h_in, float* h_out, int64_t segments,
                                int64_t batch, int64_t dim, int n, hipStream_t stream) {
  const int64_t states = batch * dim * n;
  const int threads = 256;
  const int64_t blocks = (states + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(carry_combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                     stream, sum_delta, agg, A, h0, h_in, h_out, segments, batch, dim, n);
  return hipGetLastError();
}

}  // namespace ssm
