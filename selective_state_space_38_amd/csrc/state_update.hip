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
// is laid out for HBM (see the kernel comment).  The exchange partners of a
// lane are always in range: a channel's LPC lanes are aligned neighbours
// within one wave (LPC divides 64).

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Layout.  For N >= 4 a lane holds G = 2 vectors of Q = 4 consecutive
// states; a channel's N states are spread over LPC = N/4 neighbouring lanes,
// which reduce the readout C . h with DPP exchanges.  Vector g of lane l is
// vector g*64 + l of the wave's run of 2*64 vectors, so each state load or
// store instruction of the wave covers one dense 1 KB run (every 64-byte line
// fully used by one instruction), and the two vectors are independent work in
// flight.  The lane's two vectors belong to two channels of the wave's
// 128/LPC.  A workgroup (four waves) owns 512/LPC consecutive channels of a
// run of R batch rows (a lane keeps its channels' A, scaled by log2 e,
// dt_bias and D for all of them).  The state is read once and written once
// (non-temporal).  For N < 4 a lane holds one channel's N states.
// VBC: B and C are aligned for vector loads (8 bytes per 4 bfloat16, 16 per 4
// float32); otherwise they are read element by element.
// (Measured variants that did not pay at the 256 x 5120 x 16 step: four
// vectors per lane, 36-38 us; the two vectors as one channel in two rows,
// 35 us; one lane per channel with its N states as 8-state halves, whose
// 16-byte accesses half-fill every line per instruction, 41-44 us.)
// batch rows per workgroup (software-pipelined, see the kernel); 1, 2, 4
// or 8 are instantiated.  At the 256 x 5120 x 16 step, 1 and 2 rows measured
// 33.7-35 us and 4 or 8 rows 36 us: many short workgroups hide the state's
// latency at least as well as prefetching inside longer ones.  (A persistent
// grid-stride form, 1024 workgroups each prefetching its next tile, measured
// 36.7 us: its registers halve the waves a SIMD holds.)
constexpr int kDecodeRows = 1;

template <int N>
struct DecodeShape {
  static constexpr int Q = N < 4 ? N : 4;        // states per vector
  static constexpr int LPC = N / Q;              // lanes per channel: 1, 2, 4, 8, 16
  static constexpr int G = N < 4 ? 1 : 2;        // vectors (channel groups) per lane
  static constexpr int CPW = G * 64 / LPC;       // channels per wave
  static constexpr int CPB = 4 * CPW;            // channels per workgroup of 256
};

template <typename T, int N, bool ZOH, bool VBC, int R>
__global__ __launch_bounds__(256) void state_update_kernel(
    float* __restrict__ state, const T* __restrict__ x, const T* __restrict__ dtp,
    const float* __restrict__ A, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ Dv, const T* __restrict__ zp,
    const float* __restrict__ bias, int softplus, T* __restrict__ out,
    int64_t batch, int64_t dim, int64_t n_cblk) {
  using S = DecodeShape<N>;
  constexpr int Q = S::Q, LPC = S::LPC, G = S::G;
  constexpr bool kVec = Q == 4;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int wave = static_cast<int>(threadIdx.x) >> 6;
  const int q = lane % LPC;                      // which Q states of the channel
  // workgroup -> (run of R batch rows, block of channels); channel blocks
  // vary fastest, so neighbouring workgroups stream neighbouring state
  const int64_t cb = static_cast<int64_t>(blockIdx.x) % n_cblk;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) / n_cblk * R;
  const int64_t c_wave = cb * S::CPB + wave * S::CPW;
  int64_t dch[G];
  bool dvalid[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t dr = c_wave + g * (64 / LPC) + lane / LPC;
    dvalid[g] = dr < dim;
    dch[g] = dvalid[g] ? dr : dim - 1;           // tail lanes compute, never store
  }

  // the channels' constants
  float a2[G][Q], ia[G][Q], bs[G], dd[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float* ap = A + dch[g] * N + q * Q;
    float av[Q];
    if constexpr (kVec) {
      const float4 w4 = *reinterpret_cast<const float4*>(ap);
      av[0] = w4.x; av[1] = w4.y; av[2] = w4.z; av[3] = w4.w;
    } else {
#pragma unroll
      for (int j = 0; j < Q; ++j) av[j] = ap[j];
    }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      a2[g][j] = av[j] * kLog2e;
      ia[g][j] = ZOH ? 1.0f / av[j] : 0.0f;
    }
    bs[g] = bias ? bias[dch[g]] : 0.0f;
    dd[g] = Dv ? Dv[dch[g]] : 0.0f;
  }

  // One row's inputs.  Row r + 1's loads are issued before row r is computed
  // and stored (two register sets, fully unrolled over the R rows), so a
  // row's memory latency overlaps the previous row's work.  Rows past the
  // batch re-read the last row and store nothing.
  struct RowIn {
    float h[G][Q];
    float bv[Q], cv[Q];
    float dt[G], xv[G], zv[G];
  };
  auto load_row = [&](int r, RowIn& in) {
    const int64_t b = b0 + r < batch ? b0 + r : batch - 1;
    const T* bp = Bm + b * N + q * Q;
    const T* cp = Cm + b * N + q * Q;
    if constexpr (kVec && VBC) {
      if constexpr (sizeof(T) == 2) {
        const uint2 bw = *reinterpret_cast<const uint2*>(bp);
        const uint2 cw = *reinterpret_cast<const uint2*>(cp);
        in.bv[0] = __uint_as_float(bw.x << 16); in.bv[1] = __uint_as_float(bw.x & 0xffff0000u);
        in.bv[2] = __uint_as_float(bw.y << 16); in.bv[3] = __uint_as_float(bw.y & 0xffff0000u);
        in.cv[0] = __uint_as_float(cw.x << 16); in.cv[1] = __uint_as_float(cw.x & 0xffff0000u);
        in.cv[2] = __uint_as_float(cw.y << 16); in.cv[3] = __uint_as_float(cw.y & 0xffff0000u);
      } else {
        const float4 bw = *reinterpret_cast<const float4*>(bp);
        const float4 cw = *reinterpret_cast<const float4*>(cp);
        in.bv[0] = bw.x; in.bv[1] = bw.y; in.bv[2] = bw.z; in.bv[3] = bw.w;
        in.cv[0] = cw.x; in.cv[1] = cw.y; in.cv[2] = cw.z; in.cv[3] = cw.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        in.bv[j] = to_f32(bp[j]);
        in.cv[j] = to_f32(cp[j]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float* hp = state + (b * dim + dch[g]) * N + q * Q;
      if constexpr (kVec) {
        const f32x4 hv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hp));
        in.h[g][0] = hv.x; in.h[g][1] = hv.y; in.h[g][2] = hv.z; in.h[g][3] = hv.w;
      } else {
#pragma unroll
        for (int j = 0; j < Q; ++j) in.h[g][j] = __builtin_nontemporal_load(hp + j);
      }
      const int64_t bd = b * dim + dch[g];
      in.dt[g] = to_f32(dtp[bd]);
      in.xv[g] = to_f32(x[bd]);
      in.zv[g] = zp ? to_f32(zp[bd]) : 0.0f;
    }
  };
  auto finish_row = [&](int r, RowIn& in) {
    const int64_t b = b0 + r;
    const bool live = b < batch;
    float y[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = in.dt[g] + bs[g];
      const float dl = softplus ? softplus_f32(s) : s;
      const float du = dl * in.xv[g];
      float yy = 0.0f;
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        const float x2 = dl * a2[g][j];
        const float a = exp2_hw(x2);
        if constexpr (ZOH) {
          in.h[g][j] = fmaf(a, in.h[g][j], zoh_coef(x2, a, dl, ia[g][j]) * (in.xv[g] * in.bv[j]));
        } else {
          in.h[g][j] = fmaf(a, in.h[g][j], du * in.bv[j]);
        }
        yy = fmaf(in.cv[j], in.h[g][j], yy);
      }
      y[g] = yy;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (dvalid[g] && live) {
        float* hp = state + (b * dim + dch[g]) * N + q * Q;
        if constexpr (kVec) {
          const f32x4 hv = {in.h[g][0], in.h[g][1], in.h[g][2], in.h[g][3]};
          __builtin_nontemporal_store(hv, reinterpret_cast<f32x4*>(hp));
        } else {
#pragma unroll
          for (int j = 0; j < Q; ++j) __builtin_nontemporal_store(in.h[g][j], hp + j);
        }
      }
    }
    // the partial readouts of each channel's LPC neighbouring lanes (every
    // lane of the wave takes part: the rows are uniform over the workgroup)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float v = y[g];
      if constexpr (LPC == 2) {
        v = pair_sum(v);
      } else if constexpr (LPC >= 4) {
        v = quad_sum(v);
        if constexpr (LPC >= 8) v += __shfl_xor(v, 4, 64);
        if constexpr (LPC >= 16) v += __shfl_xor(v, 8, 64);
      }
      y[g] = v;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (dvalid[g] && live && q == 0) {
        float v = y[g] + dd[g] * in.xv[g];
        if (zp) v = silu_gate(v, in.zv[g]);
        store_act(out, b * dim + dch[g], v);
      }
    }
  };

  RowIn in[2];
  load_row(0, in[0]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r + 1 < R) load_row(r + 1, in[(r + 1) & 1]);
    finish_row(r, in[r & 1]);
  }
}

template <typename T>
static hipError_t launch_n(int n, float* state, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* bias, int softplus, int zoh, void* out, int64_t batch,
                           int64_t dim, int decode_rows_override, hipStream_t stream) {
  // B and C rows start at b * N elements: vector loads need the base aligned
  // to 4 elements (N >= 4 keeps every row start aligned with it)
  const uintptr_t vec_bytes = 4 * sizeof(T);
  const bool vbc = reinterpret_cast<uintptr_t>(B) % vec_bytes == 0 &&
                   reinterpret_cast<uintptr_t>(C) % vec_bytes == 0;
  const int q = n < 4 ? n : 4;                          // states per vector
  const int64_t cpb = 4 * (n < 4 ? 1 : 2) * 64 / (n / q);  // channels per workgroup
  const int64_t cblocks = (dim + cpb - 1) / cpb;
  const int rows = (decode_rows_override == 1 || decode_rows_override == 2 ||
                    decode_rows_override == 4 || decode_rows_override == 8)
                       ? decode_rows_override
                       : kDecodeRows;
  const int64_t blocks = cblocks * ((batch + rows - 1) / rows);
  if (blocks > (int64_t{1} << 31) - 1) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
#define SSM_LAUNCH_SU_ZVR(NN, Z, V, RR)                                                         \
  hipLaunchKernelGGL((state_update_kernel<T, NN, Z, V, RR>), grid, block, 0, stream, state,    \
                     static_cast<const T*>(x), static_cast<const T*>(dt), A,                    \
                     static_cast<const T*>(B), static_cast<const T*>(C), D,                     \
                     static_cast<const T*>(z), bias, softplus, static_cast<T*>(out), batch, dim, \
                     cblocks)
#define SSM_LAUNCH_SU_ZV(NN, Z, V)            \
  switch (rows) {                             \
    case 2: SSM_LAUNCH_SU_ZVR(NN, Z, V, 2); break; \
    case 4: SSM_LAUNCH_SU_ZVR(NN, Z, V, 4); break; \
    case 8: SSM_LAUNCH_SU_ZVR(NN, Z, V, 8); break; \
    default: SSM_LAUNCH_SU_ZVR(NN, Z, V, 1); break; \
  }
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
#undef SSM_LAUNCH_SU_ZVR
  return hipGetLastError();
}

hipError_t launch_state_update(int dtype, int dstate, float* state, const void* x,
                               const void* dt, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* dt_bias,
                               int softplus, int zoh, void* out, int64_t batch, int64_t dim,
                               int rows_override, hipStream_t stream) {
  if (dtype == 0)
    return launch_n<float>(dstate, state, x, dt, A, B, C, D, z, dt_bias, softplus, zoh, out,
                           batch, dim, rows_override, stream);
  return launch_n<bf16_t>(dstate, state, x, dt, A, B, C, D, z, dt_bias, softplus, zoh, out,
                          batch, dim, rows_override, stream);
}

}  // namespace ssm
