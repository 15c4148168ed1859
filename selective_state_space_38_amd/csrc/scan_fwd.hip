// Selective-scan (S6) forward for gfx950.
//
// What is computed (pages cited by title and section):
//   Delta_t = softplus(dt_t + dt_bias)          reading guide, Selection mechanism (S6)
//   Abar_t  = exp(Delta_t * A), Bbar_t x_t = Delta_t * B_t * x_t
//                                                reading guide, Method; "Mamba / MambaMini" Q&A
//   h_t = Abar_t * h_{t-1} + Bbar_t x_t          reading guide, Method
//   y_t = C_t . h_t + D * x_t, out = y_t * SiLU(z_t)
//                                                reading guide, Method; CSDN "Mamba" 3(1);
//                                                "Mamba / MambaMini" Q&A on SiLU
// Carries between sequence segments use the pair operator of "Mamba /
// MambaMini" Step 2, (a_j a_i, a_j b_i + b_j), applied to segment aggregates.
//
// Work decomposition.  A workgroup owns one (batch, block of 64 channels,
// sequence segment).  Its NG waves split the N states of every channel into
// groups of G (lane = channel, registers = the group's states), so B_t and C_t
// slices are wave-uniform and come in through scalar loads, and no lane ever
// exchanges data with another lane.  Time is walked serially inside the
// segment in chunks of TC steps:
//   P  (per chunk, steps t = w mod NG): coalesced loads of dt/u, Delta,
//      Delta*u and D*u -> LDS (double buffered);
//   S  (all steps): per state exp2(Delta*A*log2 e), h = a*h + Delta*u*B,
//      y_partial += C*h -> LDS;
//   E  (steps t = w mod NG): sum the NG partials, add D*u, gate with SiLU(z),
//      round and store.
// The expanded state (B, L, D, N) exists only in registers.
//
// Segments of the same channel block are ordered by an atomic ticket
// (segment-major), so a workgroup only ever waits on lower tickets, which are
// already running: no deadlock, whatever order the hardware dispatches in.
//   chained mode    : segment s waits for segment s-1's final state.
//   look-back mode  : segment s first scans its own inputs from a zero state
//                     and publishes that aggregate (sum of Delta, final state);
//                     then walks back over predecessors' aggregates until it
//                     finds a published final state, combines, publishes its
//                     own final state and only then produces its outputs.
// Every wait is bounded; a wait that hits the bound bumps a device error
// counter and continues with the carry gathered so far.

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

__device__ unsigned g_carry_timeouts;

enum : int { kEmpty = 0, kAggregate = 1, kInclusive = 2 };

// Waits until *p >= need (need = kAggregate waits for any publication).
// Returns the observed status, or kEmpty on timeout.
__device__ __forceinline__ int wait_status(const int* p, int need, int limit) {
  int spins = 0;
  int v = load_acquire(p);
  while (v < need) {
    if (++spins > limit) {
      if ((threadIdx.x & 63) == 0) atomicAdd(&g_carry_timeouts, 1u);
      return kEmpty;
    }
    __builtin_amdgcn_s_sleep(2);
    v = load_acquire(p);
  }
  return v;
}

template <typename T, int NG, int G, int TC>
__global__ __launch_bounds__(64 * NG) void scan_fwd_kernel(
    const T* __restrict__ u, const T* __restrict__ dtp,
    const float* __restrict__ A, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dv,
    const T* __restrict__ zp, const float* __restrict__ bias,
    const float* __restrict__ h0, T* __restrict__ out,
    float* __restrict__ last_state, FwdScratch sc, FwdShape sh) {
  constexpr int N = NG * G;
  constexpr int K = TC / NG;  // steps per wave in the P and E phases
  static_assert(TC % NG == 0, "chunk must split evenly over the groups");

  __shared__ float s_delta[2][TC][64];
  __shared__ float s_du[2][TC][64];
  __shared__ float s_skip[2][TC][64];
  __shared__ float s_y[NG][TC][64];
  __shared__ int s_ticket;

  const int lane = threadIdx.x & 63;
  // wave-uniform values go through readfirstlane so the compiler keeps them
  // (and every address built from them, e.g. the B/C slices) in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  if (threadIdx.x == 0) s_ticket = atomicAdd(sc.ticket, 1);
  __syncthreads();
  const int ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  const int seg = ticket / sh.chains;
  const int chain = ticket - seg * sh.chains;
  const int b = chain / sh.n_cblk;
  const int cblk = chain - b * sh.n_cblk;

  const int64_t L = sh.seqlen;
  const int64_t dim = sh.dim;
  const int64_t d = static_cast<int64_t>(cblk) * 64 + lane;
  const bool dvalid = d < dim;
  const int64_t dc = dvalid ? d : dim - 1;  // tail lanes read a valid channel, never store

  float A2[G];
#pragma unroll
  for (int g = 0; g < G; ++g) A2[g] = A[dc * N + w * G + g] * kLog2e;
  const float Dd = sh.has_D ? Dv[dc] : 0.0f;
  const float bs = sh.has_bias ? bias[dc] : 0.0f;
  const bool use_sp = sh.softplus != 0;

  const int64_t t_begin = static_cast<int64_t>(seg) * sh.seg_len;
  const int64_t t_end = (t_begin + sh.seg_len < L) ? t_begin + sh.seg_len : L;
  const int64_t row0 = static_cast<int64_t>(b) * L;  // row of (b, t=0)
  const int rec = chain * sh.n_seg + seg;

  auto act = [&](int64_t t) { return (row0 + t) * dim + dc; };

  // ---- phase P helpers -------------------------------------------------
  auto load_p = [&](int64_t c0, int n, float (&rdt)[K], float (&ru)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int lt = w + k * NG;
      if (lt < n) {
        rdt[k] = to_f32(dtp[act(c0 + lt)]);
        ru[k] = to_f32(u[act(c0 + lt)]);
      }
    }
  };
  auto compute_p = [&](int buf, int n, const float (&rdt)[K], const float (&ru)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int lt = w + k * NG;
      if (lt < n) {
        const float s = rdt[k] + bs;
        const float dl = use_sp ? softplus_f32(s) : s;
        s_delta[buf][lt][lane] = dl;
        s_du[buf][lt][lane] = dl * ru[k];
        s_skip[buf][lt][lane] = Dd * ru[k];
      }
    }
  };

  // ---- aggregate pass: own final state from zero and sum of Delta --------
  auto aggregate_pass = [&](float (&hA)[G], float& sum_delta) {
#pragma unroll
    for (int g = 0; g < G; ++g) hA[g] = 0.0f;
    sum_delta = 0.0f;
    float rdt[K], ru[K];
    int64_t c0 = t_begin;
    int n0 = static_cast<int>((t_end - c0 < TC) ? t_end - c0 : TC);
    load_p(c0, n0, rdt, ru);
    compute_p(0, n0, rdt, ru);
    __syncthreads();
    int buf = 0;
    while (c0 < t_end) {
      const int n = static_cast<int>((t_end - c0 < TC) ? t_end - c0 : TC);
      const int64_t c1 = c0 + n;
      const int n1 = static_cast<int>((t_end - c1 < TC) ? t_end - c1 : TC);
      if (n1 > 0) load_p(c1, n1, rdt, ru);
      for (int lt = 0; lt < n; ++lt) {
        const float dl = s_delta[buf][lt][lane];
        const float du = s_du[buf][lt][lane];
        float bv[G];
        load_slice<G>(Bm + ((row0 + c0 + lt) * N + w * G), bv);
        sum_delta += dl;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float a = exp2_hw(dl * A2[g]);
          hA[g] = fmaf(a, hA[g], du * bv[g]);
        }
      }
      if (n1 > 0) compute_p(buf ^ 1, n1, rdt, ru);
      __syncthreads();
      buf ^= 1;
      c0 = c1;
    }
  };

  // ---- output pass: from carry-in h, produce out and the final state -----
  auto output_pass = [&](float (&h)[G]) {
    float rdt[K], ru[K], rz[K];
    int64_t c0 = t_begin;
    int n0 = static_cast<int>((t_end - c0 < TC) ? t_end - c0 : TC);
    load_p(c0, n0, rdt, ru);
    compute_p(0, n0, rdt, ru);
    __syncthreads();
    int buf = 0;
    while (c0 < t_end) {
      const int n = static_cast<int>((t_end - c0 < TC) ? t_end - c0 : TC);
      const int64_t c1 = c0 + n;
      const int n1 = static_cast<int>((t_end - c1 < TC) ? t_end - c1 : TC);
      if (n1 > 0) load_p(c1, n1, rdt, ru);
      if (sh.has_z) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int lt = w + k * NG;
          if (lt < n) rz[k] = to_f32(zp[act(c0 + lt)]);
        }
      }
      // phase S
      for (int lt = 0; lt < n; ++lt) {
        const float dl = s_delta[buf][lt][lane];
        const float du = s_du[buf][lt][lane];
        const int64_t brow = (row0 + c0 + lt) * N + w * G;
        float bv[G], cv[G];
        load_slice<G>(Bm + brow, bv);
        load_slice<G>(Cm + brow, cv);
        float y = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float a = exp2_hw(dl * A2[g]);
          h[g] = fmaf(a, h[g], du * bv[g]);
          y = fmaf(cv[g], h[g], y);
        }
        s_y[w][lt][lane] = y;
      }
      __syncthreads();
      if (n1 > 0) compute_p(buf ^ 1, n1, rdt, ru);
      // phase E
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int lt = w + k * NG;
        if (lt < n) {
          float y = s_y[0][lt][lane];
#pragma unroll
          for (int q = 1; q < NG; ++q) y += s_y[q][lt][lane];
          y += s_skip[buf][lt][lane];
          if (sh.has_z) y = silu_gate(y, rz[k]);
          if (dvalid) store_act(out, act(c0 + lt), y);
        }
      }
      __syncthreads();
      buf ^= 1;
      c0 = c1;
    }
  };

  // ---- carry-in ------------------------------------------------------------
  float h[G];
  const int gidx = w * G;  // first state of this wave's group
  const int64_t rec_state = static_cast<int64_t>(rec) * N * 64;
  bool published = false;
  if (seg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      h[g] = sh.has_h0 ? h0[(static_cast<int64_t>(b) * dim + dc) * N + gidx + g] : 0.0f;
  } else if (!sh.lookback) {
    const int prev = rec - 1;
    const int st = wait_status(&sc.status[prev * NG + w], kInclusive, sc.spin_limit);
    const int64_t ps = static_cast<int64_t>(prev) * N * 64;
#pragma unroll
    for (int g = 0; g < G; ++g)
      h[g] = (st == kInclusive) ? sc.inc[ps + (gidx + g) * 64 + lane] : 0.0f;
  } else {
    float hA[G];
    float sum_delta;
    aggregate_pass(hA, sum_delta);
#pragma unroll
    for (int g = 0; g < G; ++g) sc.agg_b[rec_state + (gidx + g) * 64 + lane] = hA[g];
    sc.agg_s[(static_cast<int64_t>(rec) * NG + w) * 64 + lane] = sum_delta;
    if (lane == 0) store_release(&sc.status[rec * NG + w], kAggregate);

    // Walk back: acc = (exp2(A2 * acc_s), acc_b) is the combination of the
    // segments between the one being inspected and this one.
    float acc_s = 0.0f;
    float acc_b[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc_b[g] = 0.0f;
    const int rec0 = chain * sh.n_seg;
    for (int j = rec - 1; j >= rec0; --j) {
      const int st = wait_status(&sc.status[j * NG + w], kAggregate, sc.spin_limit);
      const int64_t js = static_cast<int64_t>(j) * N * 64;
      if (st == kInclusive) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float carry = sc.inc[js + (gidx + g) * 64 + lane];
          acc_b[g] = fmaf(exp2_hw(A2[g] * acc_s), carry, acc_b[g]);
        }
        break;
      }
      if (st == kEmpty) break;  // timed out: continue with what was gathered
      const float sj = sc.agg_s[(static_cast<int64_t>(j) * NG + w) * 64 + lane];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float bj = sc.agg_b[js + (gidx + g) * 64 + lane];
        acc_b[g] = fmaf(exp2_hw(A2[g] * acc_s), bj, acc_b[g]);
      }
      acc_s += sj;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) h[g] = acc_b[g];
    if (seg + 1 < sh.n_seg) {
      // this segment's own final state: its aggregate applied after the carry
#pragma unroll
      for (int g = 0; g < G; ++g)
        sc.inc[rec_state + (gidx + g) * 64 + lane] =
            fmaf(exp2_hw(A2[g] * sum_delta), h[g], hA[g]);
      if (lane == 0) store_release(&sc.status[rec * NG + w], kInclusive);
    }
    published = true;
  }

  output_pass(h);

  if (!published && seg + 1 < sh.n_seg) {
#pragma unroll
    for (int g = 0; g < G; ++g) sc.inc[rec_state + (gidx + g) * 64 + lane] = h[g];
    if (lane == 0) store_release(&sc.status[rec * NG + w], kInclusive);
  }
  if (seg + 1 == sh.n_seg && sh.has_last && dvalid) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      last_state[(static_cast<int64_t>(b) * dim + d) * N + gidx + g] = h[g];
  }
}

__global__ void fill_zero_kernel(int* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_fill_zero(int* p, int64_t n, hipStream_t stream) {
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                     stream, p, n);
  return hipGetLastError();
}

template <typename T, int NG, int G>
static hipError_t launch_typed(const FwdPtrs& p, const FwdScratch& s, const FwdShape& sh,
                               int64_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL((scan_fwd_kernel<T, NG, G, kChunk>), dim3(static_cast<unsigned>(workgroups)),
                     dim3(64 * NG), 0, stream, static_cast<const T*>(p.u),
                     static_cast<const T*>(p.delta), p.A, static_cast<const T*>(p.B),
                     static_cast<const T*>(p.C), p.D, static_cast<const T*>(p.z), p.dt_bias,
                     p.h0, static_cast<T*>(p.out), p.last_state, s, sh);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_groups(int groups, int per_group, const FwdPtrs& p,
                                  const FwdScratch& s, const FwdShape& sh, int64_t wg,
                                  hipStream_t st) {
  const int n = groups * per_group;
  switch (n) {
    case 1: return launch_typed<T, 1, 1>(p, s, sh, wg, st);
    case 2: return launch_typed<T, 1, 2>(p, s, sh, wg, st);
    case 4:
      if (groups == 1) return launch_typed<T, 1, 4>(p, s, sh, wg, st);
      break;
    case 8:
      if (groups == 2) return launch_typed<T, 2, 4>(p, s, sh, wg, st);
      if (groups == 1) return launch_typed<T, 1, 8>(p, s, sh, wg, st);
      break;
    case 16:
      if (groups == 4) return launch_typed<T, 4, 4>(p, s, sh, wg, st);
      if (groups == 2) return launch_typed<T, 2, 8>(p, s, sh, wg, st);
      if (groups == 8) return launch_typed<T, 8, 2>(p, s, sh, wg, st);
      if (groups == 1) return launch_typed<T, 1, 16>(p, s, sh, wg, st);
      break;
    case 32:
      if (groups == 8) return launch_typed<T, 8, 4>(p, s, sh, wg, st);
      break;
    case 64:
      if (groups == 16) return launch_typed<T, 16, 4>(p, s, sh, wg, st);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan_fwd(int dtype, int groups, int per_group, const FwdPtrs& p,
                           const FwdScratch& s, const FwdShape& sh, int64_t workgroups,
                           hipStream_t stream) {
  if (dtype == 0) return dispatch_groups<float>(groups, per_group, p, s, sh, workgroups, stream);
  return dispatch_groups<bf16_t>(groups, per_group, p, s, sh, workgroups, stream);
}

hipError_t read_and_clear_errors(hipStream_t stream, unsigned* count) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_carry_timeouts), sizeof(unsigned), 0,
                          hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const unsigned zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_carry_timeouts), &zero, sizeof(unsigned), 0,
                           hipMemcpyHostToDevice);
}

}  // namespace ssm
