// Selective-scan (S6) forward for gfx950.
//
// What is computed (pages cited by title and section):
//   Delta_t = softplus(dt_t + dt_bias)          reading guide, Selection mechanism (S6)
//   Abar_t  = exp(Delta_t * A), Bbar_t x_t = Delta_t * B_t * x_t
//                                                reading guide, Method; "Mamba / MambaMini" Q&A
//             or, with ZOH, the exact zero-order-hold input
//             Bbar_t x_t = (exp(Delta_t A) - 1) / A * B_t * x_t
//                                                reading guide, Method
//   h_t = Abar_t * h_{t-1} + Bbar_t x_t          reading guide, Method
//   y_t = C_t . h_t + D * x_t, out = y_t * SiLU(z_t)
//                                                reading guide, Method; CSDN "Mamba" 3(1);
//                                                "Mamba / MambaMini" Q&A on SiLU
// Carries between sequence segments use the pair operator of "Mamba /
// MambaMini" Step 2, (a_j a_i, a_j b_i + b_j), applied to segment aggregates.
//
// Work decomposition.  A workgroup owns one (batch, block of 64 channels,
// sequence segment).  Its NG scan waves split the N states of every channel
// into groups of G (lane = channel, registers = the group's states), so every
// lane of a wave reads the same B_t / C_t slice (an LDS broadcast) and no
// lane ever exchanges data with another lane.  NP helper waves do the
// rest; each helper thread owns one run of TC / NP channels of one tile row.
// Time is walked serially inside the segment in chunks of TC steps:
//   P  (helpers, one chunk ahead): coalesced loads of the chunk's dt/u/z
//      rows and B/C rows; Delta, Delta*u and float B/C -> LDS (double
//      buffered), D*u and z kept in registers;
//   S  (scan waves, all steps): per state exp2(Delta*A*log2 e),
//      h = a*h + Delta*u*B, y_partial += C*h -> LDS;
//   E  (helpers, one chunk behind): sum the NG partials, add D*u, gate with
//      SiLU(z), round and store.
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
//                     If the predecessor's final state is already published
//                     when the segment starts, it skips straight to its
//                     outputs (and publishes its final state at the end).
// Every wait is bounded; a wait that hits the bound bumps a device error
// counter and continues with the carry gathered so far.
//
// Aggregate-only instances (AGG) stop before the outputs: they return the
// sequence's end state and its sum of Delta, the carry record with which
// independently scanned pieces of a sequence are joined ("Mamba / MambaMini"
// Steps 2-4).  Only u, dt and B are read.  Their scratch then holds every
// split segment's end state (from a zero start) and sum of Delta; FROMREC
// instances take those and an h0 and run every segment's output pass at
// once, none waiting and none running an aggregate pass.

#include "ssm_device.h"
#include "ssm_internal.h"

// This file is compiled once per activation type (-DSSM_FWD_DTYPE=0 for
// float32, 1 for bfloat16) so the two halves build in parallel; each object
// holds its own kernels and error counter in its own namespace.
#if !defined(SSM_FWD_DTYPE)
#error "compile with -DSSM_FWD_DTYPE=0 (float32) or -DSSM_FWD_DTYPE=1 (bfloat16)"
#elif SSM_FWD_DTYPE == 0
#define SSM_FWD_NS fwd_f32
#define SSM_FWD_T float
#else
#define SSM_FWD_NS fwd_bf16
#define SSM_FWD_T bf16_t
#endif

namespace ssm {
namespace SSM_FWD_NS {

__device__ unsigned g_carry_timeouts;

enum : int { kEmpty = 0, kAggregate = 1, kInclusive = 2 };

// Waits until *p >= need (need = kAggregate waits for any publication).
// Polls with plain device-coherent loads and a growing sleep, then issues one
// acquire fence, so waiting waves neither flood memory nor keep invalidating
// the caches the computing waves use.  Returns the observed status, or
// kEmpty when the bound is hit.
__device__ __forceinline__ int wait_status(const int* p, int need, int limit) {
  int spins = 0;
  int v = load_relaxed(p);
  while (v < need) {
    if (++spins > limit) {
      if ((threadIdx.x & 63) == 0) atomicAdd(&g_carry_timeouts, 1u);
      return kEmpty;
    }
    if (spins < 16) {
      __builtin_amdgcn_s_sleep(2);
    } else {
      __builtin_amdgcn_s_sleep(32);
    }
    v = load_relaxed(p);
  }
  acquire_fence();
  return v;
}

template <typename T, int NG, int G, int NP, int TC, bool ZOH, bool VEC, int MODE>
__global__ __launch_bounds__(64 * (NG + NP)) void scan_fwd_kernel(
    const T* __restrict__ u, const T* __restrict__ dtp,
    const float* __restrict__ A, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const float* __restrict__ Dv,
    const T* __restrict__ zp, const float* __restrict__ bias,
    const float* __restrict__ h0, T* __restrict__ out,
    float* __restrict__ last_state, FwdScratch sc, FwdShape sh) {
  constexpr int N = NG * G;
  constexpr int PT = 64 * NP;          // helper threads
  constexpr int EPT = TC / NP;         // tile elements per helper thread (one row run)
  constexpr int TPR = 64 / EPT;        // helper threads per tile row
  static_assert(TC % NP == 0 && 64 % EPT == 0, "chunk must split evenly over the helpers");
  constexpr int ESZ = static_cast<int>(sizeof(T));
  constexpr bool kBCWords = (N * ESZ) % 4 == 0;          // B/C chunk rows are dword granular
  constexpr int BC_UNITS = kBCWords ? TC * N * ESZ / 4 : TC * N;
  constexpr int BCPT = (BC_UNITS + PT - 1) / PT;          // B/C dwords (or elements) per thread
  using TileRun = Run<T, EPT>;

  // Delta and Delta*u (u with ZOH) side by side per channel: one 8-byte
  // read per step
  __shared__ __align__(16) float2 s_dd[2][TC][64];
  __shared__ __align__(16) float s_B[2][TC][N];
  __shared__ __align__(16) float s_C[2][TC][N];
  __shared__ __align__(16) float s_y[2][NG][TC][64];
  __shared__ int s_ticket;
  __shared__ int s_pred_final;

  // MODE: kModeForward, kModeRecord (AGG: the carry record only) or
  // kModeFromRecord (FROMREC: outputs from the carries a record launch kept)
  constexpr bool AGG = MODE == kModeRecord;
  constexpr bool FROMREC = MODE == kModeFromRecord;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values go through readfirstlane so the compiler keeps them
  // (and addresses built from them) in SGPRs
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool scan_wave = w < NG;           // scan waves 0..NG-1, helpers NG..NG+NP-1
  const int gidx = scan_wave ? w * G : 0;  // first state of a scan wave's group

  // Workgroups 0 .. n_full-1 run whole chains (chain = workgroup index; they
  // never wait).  The others are segments of the split chains and take their
  // (segment, chain) from an atomic ticket, segment-major, so a segment only
  // ever waits on lower tickets, which are already running.  Taking the role
  // from the workgroup index keeps it tied to the hardware's placement
  // (workgroups i and i + #CUs share a CU), so each CU gets one whole chain
  // and one segment.
  const bool whole = static_cast<int>(blockIdx.x) < sh.n_full;
  int ticket = 0;
  if constexpr (FROMREC) {
    // no segment waits for another: the order is the workgroup index's
    if (!whole) ticket = static_cast<int>(blockIdx.x) - sh.n_full;
  } else if (!whole) {
    if (tid == 0) s_ticket = atomicAdd(sc.ticket, 1);
    __syncthreads();
    ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  }
  // Issue priority (the wave's own, for the SIMD's arbiter): the scan waves
  // of whole chains are the critical path, their helpers next, the split
  // chains' segments fill the gaps.
  if (whole) {
    if (scan_wave) {
      __builtin_amdgcn_s_setprio(3);
    } else {
      __builtin_amdgcn_s_setprio(2);
    }
  } else if (scan_wave) {
    __builtin_amdgcn_s_setprio(1);
  }
  const int n_split = sh.chains - sh.n_full;
  const int seg = whole ? 0 : ticket / n_split;
  const int chain = whole ? static_cast<int>(blockIdx.x) : sh.n_full + (ticket - seg * n_split);
  const int nseg_c = whole ? 1 : sh.n_seg;       // segments of this chain
  const int b = chain / sh.n_cblk;
  const int cblk = chain - b * sh.n_cblk;

  const int64_t L = sh.seqlen;
  const int64_t dim = sh.dim;
  const int64_t ch0 = static_cast<int64_t>(cblk) * 64;
  const int64_t d = ch0 + lane;                 // scan lane's channel
  const bool dvalid = d < dim;
  const int64_t dc = dvalid ? d : dim - 1;      // tail lanes read a valid channel, never store

  // a split chain's first segment has its own length; the others follow it
  const int64_t t_begin =
      (whole || seg == 0) ? 0 : sh.seg0_len + static_cast<int64_t>(seg - 1) * sh.seg_len;
  const int64_t t_stop = whole ? L : t_begin + (seg == 0 ? sh.seg0_len : sh.seg_len);
  const int64_t t_end = t_stop < L ? t_stop : L;
  const int n_chunks = static_cast<int>((t_end - t_begin + TC - 1) / TC);
  const int64_t row0 = static_cast<int64_t>(b) * L;  // row of (b, t=0)
  // carry records exist for split chains only: rec0 is this chain's first
  // (whole chains never publish or read one)
  const int rec0 = whole ? 0 : (chain - sh.n_full) * sh.n_seg;
  const int rec = rec0 + seg;
  // Barrier-separated iterations of a pass after its prologue: one per chunk,
  // plus one for the last chunk's outputs, rounded up to even (see the
  // helpers' loop); both roles run exactly this many.
  auto pass_iterations = [&](bool out_mode) -> int {
    const int it = out_mode ? n_chunks + 1 : n_chunks;
    return (it + 1) & ~1;
  };
  // rows of chunk c: TC for all but the last chunk (32-bit, so the test stays
  // in scalar registers)
  const int last_rows = static_cast<int>(t_end - t_begin - static_cast<int64_t>(n_chunks - 1) * TC);
  auto chunk_rows = [&](int c) -> int {
    return c < n_chunks - 1 ? TC : (c == n_chunks - 1 ? last_rows : 0);
  };

  // =========================================================================
  // Helper waves: stage the chunk tiles (phase P) and finish the outputs
  // (phase E).  In the iteration where the scan waves run chunk c, the
  // helpers finish chunk c-1, prepare chunk c+1 and issue the loads of chunk
  // c+3 (two register sets, so every load has two chunk times to land).
  // =========================================================================
  struct Prefetch {
    TileRun dt, uu, zz;
    uint32_t bc[2][BCPT];
  };
  auto helper_loop = [&](auto out_c, auto fast_c) {
    // OUT: the output pass (else the aggregate pass of a look-back segment).
    // FAST: softplus on and, in the output pass, a gate: the layer's usual
    // configuration, compiled without per-element selects on the flags.
    constexpr bool OUT = decltype(out_c)::value;
    constexpr bool FAST = decltype(fast_c)::value;
    const int ptid = tid - 64 * NG;
    const int tr = ptid / TPR;
    const int tc = (ptid - tr * TPR) * EPT;
    const int64_t tch = ch0 + tc;                       // first channel of the run
    const bool run_valid = tch < dim;                   // any channel of the run inside
    const int run_last = run_valid ? static_cast<int>((dim - 1 - tch) < (EPT - 1) ? (dim - 1 - tch)
                                                                                  : (EPT - 1))
                                   : 0;
    // VEC: the host guarantees whole aligned runs (dim % EPT == 0, aligned
    // pointers).  Every lane then issues the same vector loads (dead runs past
    // the last channel read the last run and store nothing), so the compiler
    // can count the loads in flight exactly and wait only for the register
    // set being consumed.
    constexpr bool run_vec = VEC && TileRun::kCanVec;
    const int64_t tch_c = run_valid ? tch : (run_vec ? dim - EPT : dim - 1);
    const bool use_sp = FAST || sh.softplus != 0;
    const bool with_z = OUT && (FAST || sh.has_z);
    // without a gate the output pass still loads a z tile (u's, unused) so
    // the loads in flight do not depend on it
    const T* const zsrc = sh.has_z ? zp : u;
    float rD[EPT], rbias[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int64_t ck = tch_c + (k < run_last ? k : run_last);
      rD[k] = sh.has_D ? Dv[ck] : 0.0f;
      rbias[k] = sh.has_bias ? bias[ck] : 0.0f;
    }

    // Addresses: a chunk base that is the same for the whole workgroup (kept
    // in scalar registers) plus this thread's byte offset inside the chunk,
    // computed once.  Rows past the end of a ragged last chunk are clamped to
    // its last row.  The host keeps TC * dim * 4 bytes below 2^31.
    const int cofs = static_cast<int>(tch_c - ch0);
    const int dim32 = static_cast<int>(dim);
    const int r_last = tr < last_rows ? tr : last_rows - 1;
    const uint32_t el_full = static_cast<uint32_t>(tr * dim32 + cofs);
    const uint32_t el_last = static_cast<uint32_t>(r_last * dim32 + cofs);
    const uint32_t ob_full = el_full * ESZ, ob_last = el_last * ESZ;
    auto chunk_el = [&](int c) -> int64_t {       // element (row of chunk c, channel ch0)
      return (row0 + t_begin + static_cast<int64_t>(c) * TC) * dim + ch0;
    };
    // B/C: byte offsets of this thread's words (or elements) in a chunk's rows
    uint32_t bo_full[BCPT], bo_last[BCPT];
    {
      constexpr int kUnit = kBCWords ? 4 : ESZ;
      const int nu_full = kBCWords ? TC * N * ESZ / 4 : TC * N;
      const int nu_last = kBCWords ? last_rows * N * ESZ / 4 : last_rows * N;
#pragma unroll
      for (int k = 0; k < BCPT; ++k) {
        const int e = ptid + k * PT;
        bo_full[k] = static_cast<uint32_t>((e < nu_full ? e : nu_full - 1) * kUnit);
        bo_last[k] = static_cast<uint32_t>((e < nu_last ? e : nu_last - 1) * kUnit);
      }
    }

    // loads of chunk c (clamped to the last chunk, so every iteration loads
    // and consumes the same registers unconditionally)
    auto load_p = [&](int c, Prefetch& pf) {
      const int cc = c < n_chunks ? c : n_chunks - 1;
      const bool lastc = cc == n_chunks - 1;
      const int64_t ce = chunk_el(cc);
      const uint32_t ob = lastc ? ob_last : ob_full;
      if constexpr (run_vec) {
        pf.dt.load_vec(add_bytes(dtp + ce, ob));
        pf.uu.load_vec(add_bytes(u + ce, ob));
        if constexpr (OUT) pf.zz.load_vec(add_bytes(zsrc + ce, ob));
      } else {
        pf.dt.load_elems(add_bytes(dtp + ce, ob), run_last);
        pf.uu.load_elems(add_bytes(u + ce, ob), run_last);
        if constexpr (OUT) pf.zz.load_elems(add_bytes(zsrc + ce, ob), run_last);
      }
      const int64_t base = (row0 + t_begin + static_cast<int64_t>(cc) * TC) * N;  // first B/C element
#pragma unroll
      for (int k = 0; k < BCPT; ++k) {
        const uint32_t o = lastc ? bo_last[k] : bo_full[k];
        if constexpr (kBCWords) {
          pf.bc[0][k] = *add_bytes(reinterpret_cast<const uint32_t*>(Bm + base), o);
          if constexpr (OUT) pf.bc[1][k] = *add_bytes(reinterpret_cast<const uint32_t*>(Cm + base), o);
        } else {
          pf.bc[0][k] = static_cast<uint32_t>(*add_bytes(Bm + base, o));
          if constexpr (OUT) pf.bc[1][k] = static_cast<uint32_t>(*add_bytes(Cm + base, o));
        }
      }
    };
    auto bc_float = [&](uint32_t word, int half) -> float {
      if constexpr (ESZ == 4) {
        return __uint_as_float(word);
      } else {
        return __uint_as_float(half ? (word & 0xffff0000u) : (word << 16));
      }
    };
    // Phase P of chunk c into LDS buffer c % 2: Delta, Delta*u (u with ZOH)
    // and float B/C; D*u and z stay in this thread's registers until phase E.
    // Every prefetched register is consumed unconditionally (only the LDS
    // writes are predicated), so no load can still be counted as in flight
    // when the registers are reloaded.
    auto compute_p = [&](int c, const Prefetch& pf, float (&sk)[EPT], float (&zf)[EPT]) {
      pf.dt.consume_all();
      pf.uu.consume_all();
      if constexpr (OUT) pf.zz.consume_all();
#pragma unroll
      for (int k = 0; k < BCPT; ++k) {
        consume(pf.bc[0][k]);
        if constexpr (OUT) consume(pf.bc[1][k]);
      }
      const int n = chunk_rows(c);
      const int buf = c & 1;
      float dl[EPT], du[EPT];
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        const float uv = pf.uu.get(k);
        const float s = pf.dt.get(k) + rbias[k];
        dl[k] = use_sp ? softplus_f32(s) : s;
        du[k] = ZOH ? uv : dl[k] * uv;
        if constexpr (OUT) {
          sk[k] = rD[k] * uv;
          zf[k] = with_z ? pf.zz.get(k) : 0.0f;
        }
      }
      if (tr < n) {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          s_dd[buf][tr][tc + k] = make_float2(dl[k], du[k]);
        }
      }
      float* sb = &s_B[buf][0][0];
      float* scc = &s_C[buf][0][0];
      if constexpr (kBCWords) {
        const int nw = n * N * ESZ / 4;
#pragma unroll
        for (int k = 0; k < BCPT; ++k) {
          const int e = ptid + k * PT;
          const float b0 = bc_float(pf.bc[0][k], 0), b1 = bc_float(pf.bc[0][k], 1);
          const float c0v = OUT ? bc_float(pf.bc[1][k], 0) : 0.0f;
          const float c1v = OUT ? bc_float(pf.bc[1][k], 1) : 0.0f;
          if (e < nw) {
            if constexpr (ESZ == 4) {
              sb[e] = b0;
              if constexpr (OUT) scc[e] = c0v;
            } else {
              sb[2 * e] = b0;
              sb[2 * e + 1] = b1;
              if constexpr (OUT) {
                scc[2 * e] = c0v;
                scc[2 * e + 1] = c1v;
              }
            }
          }
        }
      } else {
        const int ne = n * N;
#pragma unroll
        for (int k = 0; k < BCPT; ++k) {
          const int e = ptid + k * PT;
          const float bv = to_f32(static_cast<T>(pf.bc[0][k]));
          const float cv = OUT ? to_f32(static_cast<T>(pf.bc[1][k])) : 0.0f;
          if (e < ne) {
            sb[e] = bv;
            if constexpr (OUT) scc[e] = cv;
          }
        }
      }
    };
    // Phase E of chunk c: sum the NG partial readouts, add D*u, gate with
    // SiLU(z), round and store this thread's run.
    const uint32_t ob_f32 = el_full * 4u;
    auto finish_e = [&](int c, const float (&sk)[EPT], const float (&zf)[EPT]) {
      const int n = chunk_rows(c);
      const int buf = c & 1;
      if (tr < n && run_valid) {
        float yv[EPT], yg[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          float y = s_y[buf][0][tr][tc + k];
#pragma unroll
          for (int q = 1; q < NG; ++q) y += s_y[buf][q][tr][tc + k];
          y += sk[k];
          yv[k] = y;
          yg[k] = with_z ? silu_gate(y, zf[k]) : y;
        }
        const int64_t ce = chunk_el(c);
        if (out) store_run<T, EPT>(add_bytes(out + ce, ob_full), yg, run_vec, run_last);
        // training mode: the readout before the gate, for the backward
        if (sc.ysave) store_run<float, EPT>(add_bytes(sc.ysave + ce, ob_f32), yv, run_vec, run_last);
      }
    };

    Prefetch pf0, pf1;
    float sk0[EPT], zf0[EPT], sk1[EPT], zf1[EPT];
    load_p(0, pf0);
    load_p(1, pf1);
    compute_p(0, pf0, sk0, zf0);
    load_p(2, pf0);
    lds_barrier();
    // iteration c (scan waves on chunk c): E(c-1), P(c+1), loads of c+3;
    // chunk k uses register set k % 2.  The count is rounded up to even so
    // both halves of the unrolled loop always run: with a conditional second
    // half the compiler must assume the set consumed next was loaded just
    // before, and waits for every outstanding load and store.
    auto iter = [&](int c, Prefetch& pf, float (&sk)[EPT], float (&zf)[EPT]) {
      if constexpr (OUT) {
        if (c >= 1 && c <= n_chunks) finish_e(c - 1, sk, zf);
      }
      compute_p(c + 1, pf, sk, zf);
      load_p(c + 3, pf);
      lds_barrier();
    };
    const int iters = pass_iterations(OUT);
    for (int c = 0; c < iters; c += 2) {
      iter(c, pf1, sk1, zf1);
      iter(c + 1, pf0, sk0, zf0);
    }
  };

  // =========================================================================
  // Scan waves: the recurrence.  Lane = channel, registers = the wave's G
  // states; B_t / C_t slices are LDS broadcasts.
  // =========================================================================
  float A2[G], iA[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float av = scan_wave ? A[dc * N + gidx + g] : 0.0f;
    A2[g] = av * kLog2e;
    iA[g] = (ZOH && scan_wave) ? 1.0f / av : 0.0f;
  }
  // input term of state g: Delta*u*B (du holds Delta*u), or with ZOH
  // (exp(Delta A) - 1)/A * u*B (du holds u); x2 = Delta*A*log2 e, a = exp2(x2)
  auto input_term = [&](int g, float dl, float x2, float a, float du, float bv) -> float {
    if constexpr (ZOH) {
      return zoh_coef(x2, a, dl, iA[g]) * (du * bv);
    } else {
      return du * bv;
    }
  };

  // aggregate pass: the state reached from hA's initial value (zero for a
  // look-back segment's own aggregate) and the sum of Delta; the helpers
  // stage dt, u and B only
  auto scan_aggregate = [&](float (&hA)[G], float& sum_delta) {
    sum_delta = 0.0f;
    lds_barrier();  // helpers' prologue staged chunk 0
    for (int c = 0; c < n_chunks; ++c) {
      const int n = chunk_rows(c);
      const int buf = c & 1;
      auto step = [&](int lt) {
        const float2 dd = s_dd[buf][lt][lane];
        const float dl = dd.x, du = dd.y;
        float bv[G];
#pragma unroll
        for (int g = 0; g < G; ++g) bv[g] = s_B[buf][lt][gidx + g];
        sum_delta += dl;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float x2 = dl * A2[g];
          const float a = exp2_hw(x2);
          hA[g] = fmaf(a, hA[g], input_term(g, dl, x2, a, du, bv[g]));
        }
      };
      if (n == TC) {
#pragma unroll
        for (int lt = 0; lt < TC; ++lt) step(lt);
      } else {
        for (int lt = 0; lt < n; ++lt) step(lt);
      }
      lds_barrier();
    }
    for (int c = n_chunks; c < pass_iterations(false); ++c) lds_barrier();
  };

  // output pass: from carry-in h, produce the readout partials and the final
  // state; in training mode the state before every kBwdChunk-th step goes to
  // the backward's checkpoint array
  const bool ckpt_on = sc.ckpt != nullptr;
  float* const ckpt_c = ckpt_on ? sc.ckpt + static_cast<int64_t>(chain) * sh.n_ckpt * N * 64 : nullptr;
  auto save_ckpt = [&](int64_t t, const float (&hh)[G]) {
    const int64_t c = t / kBwdChunk;
#pragma unroll
    for (int g = 0; g < G; ++g) ckpt_c[(c * N + gidx + g) * 64 + lane] = hh[g];
  };
  auto scan_output = [&](float (&h)[G]) {
    lds_barrier();  // helpers' prologue staged chunk 0
    for (int c = 0; c < n_chunks; ++c) {
      const int n = chunk_rows(c);
      const int buf = c & 1;
      const int64_t c0 = t_begin + static_cast<int64_t>(c) * TC;
      if (n == TC) {
        // software-pipelined: the LDS operands of step lt + PD are read while
        // step lt computes.  The compiler schedules the unrolled chunk freely
        // (scheduling barriers around each step, which pinned the reads in
        // place, measured 1.3% slower at all three workload shapes with the
        // clocks warm; so did reading 1, 3 or 4 steps ahead)
        constexpr int PD = 2;
        float pdl[PD + 1], pdu[PD + 1], pb[PD + 1][G], pc[PD + 1][G];
        auto rd = [&](int lt, int slot) {
          const float2 dd = s_dd[buf][lt][lane];
          pdl[slot] = dd.x;
          pdu[slot] = dd.y;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            pb[slot][g] = s_B[buf][lt][gidx + g];
            pc[slot][g] = s_C[buf][lt][gidx + g];
          }
        };
#pragma unroll
        for (int k = 0; k < PD; ++k) rd(k, k);
#pragma unroll
        for (int lt = 0; lt < TC; ++lt) {
          if (lt + PD < TC) rd(lt + PD, (lt + PD) % (PD + 1));
          if (lt % kBwdChunk == 0 && ckpt_on) save_ckpt(c0 + lt, h);
          const int slot = lt % (PD + 1);
          float y = 0.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float x2 = pdl[slot] * A2[g];
            const float a = exp2_hw(x2);
            h[g] = fmaf(a, h[g], input_term(g, pdl[slot], x2, a, pdu[slot], pb[slot][g]));
            y = fmaf(pc[slot][g], h[g], y);
          }
          s_y[buf][w][lt][lane] = y;
        }
      } else {
        for (int lt = 0; lt < n; ++lt) {
          if (ckpt_on && (lt % kBwdChunk) == 0) save_ckpt(c0 + lt, h);
          const float2 dd = s_dd[buf][lt][lane];
          const float dl = dd.x, du = dd.y;
          float y = 0.0f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float x2 = dl * A2[g];
            const float a = exp2_hw(x2);
            h[g] = fmaf(a, h[g], input_term(g, dl, x2, a, du, s_B[buf][lt][gidx + g]));
            y = fmaf(s_C[buf][lt][gidx + g], h[g], y);
          }
          s_y[buf][w][lt][lane] = y;
        }
      }
      lds_barrier();
    }
    // the helpers finish the last chunk (and the rounding iteration)
    for (int c = n_chunks; c < pass_iterations(true); ++c) lds_barrier();
  };

  // ---- carry-in ------------------------------------------------------------
  float h[G];
  float own_sum_delta = 0.0f;  // aggregate-only mode: this segment's sum of Delta
  const int64_t rec_state = static_cast<int64_t>(rec) * N * 64;
  bool published = false;
  // Look-back segment: skip the aggregate pass when the predecessor has
  // already published the final state of every state group.  The decision is
  // taken once for the workgroup (the aggregate pass stages tiles with
  // workgroup barriers, so every wave must take the same path).
  bool pred_final = false;
  if (!FROMREC && seg != 0 && sh.lookback) {
    if (tid == 0) {
      int all = 1;
      for (int q = 0; q < NG; ++q) all &= load_relaxed(&sc.status[(rec - 1) * NG + q]) == kInclusive;
      s_pred_final = all;
    }
    lds_barrier();
    pred_final = __builtin_amdgcn_readfirstlane(s_pred_final) != 0;
  }
  const bool run_aggregate = !FROMREC && seg != 0 && sh.lookback && !pred_final;
  // AGG instances compute a sequence's carry record (its sum of Delta and
  // end state) and no outputs: every workgroup runs exactly one aggregate
  // pass, a look-back segment's own (from zero, before its carry is known)
  // or, for the others, the whole work from the carry-in.  Their `out`
  // argument carries the [batch][dim] float32 sums of Delta.
  float* const sum_delta_out = AGG ? reinterpret_cast<float*>(out) : nullptr;

  if (!scan_wave) {
    using kOn = std::integral_constant<bool, true>;
    using kOff = std::integral_constant<bool, false>;
    if constexpr (AGG) {
      if (sh.softplus != 0) {
        helper_loop(kOff{}, kOn{});
      } else {
        helper_loop(kOff{}, kOff{});
      }
    } else {
      if (sh.softplus != 0 && sh.has_z) {
        if (run_aggregate) helper_loop(kOff{}, kOn{});
        helper_loop(kOn{}, kOn{});
      } else {
        if (run_aggregate) helper_loop(kOff{}, kOff{});
        helper_loop(kOn{}, kOff{});
      }
    }
    return;
  }

  if constexpr (FROMREC) {
    // this segment's start from zero (the end state the record launch kept
    // for its predecessor) plus h0 carried over the segments before it:
    // exp(A * their sum of Delta) * h0 (the pair operator, "Mamba /
    // MambaMini" Step 2)
#pragma unroll
    for (int g = 0; g < G; ++g)
      h[g] = sh.has_h0 ? h0[(static_cast<int64_t>(b) * dim + dc) * N + gidx + g] : 0.0f;
    if (seg != 0) {
      float prefix = 0.0f;
      for (int s = 0; s < seg; ++s)
        prefix += sc.agg_s[(static_cast<int64_t>(rec0 + s) * NG + w) * 64 + lane];
      const int64_t ps = static_cast<int64_t>(rec - 1) * N * 64;
#pragma unroll
      for (int g = 0; g < G; ++g)
        h[g] = fmaf(exp2_hw(A2[g] * prefix), h[g], sc.inc[ps + (gidx + g) * 64 + lane]);
    }
  } else if (seg == 0) {
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
  } else if (pred_final) {
    // look-back mode, but the predecessor already published its final state:
    // no aggregate pass needed, behave like a chained segment
    acquire_fence();
    const int64_t ps = static_cast<int64_t>(rec - 1) * N * 64;
#pragma unroll
    for (int g = 0; g < G; ++g) h[g] = sc.inc[ps + (gidx + g) * 64 + lane];
  } else {
    float hA[G];
    float sum_delta;
#pragma unroll
    for (int g = 0; g < G; ++g) hA[g] = 0.0f;
    scan_aggregate(hA, sum_delta);
#pragma unroll
    for (int g = 0; g < G; ++g) sc.agg_b[rec_state + (gidx + g) * 64 + lane] = hA[g];
    sc.agg_s[(static_cast<int64_t>(rec) * NG + w) * 64 + lane] = sum_delta;
    if (lane == 0) store_release(&sc.status[rec * NG + w], kAggregate);

    // Walk back: acc = (exp2(A2 * acc_s), acc_b) is the combination of the
    // segments between the one being inspected and this one.  The walk moves
    // in windows of kWin predecessors: lane i polls the status of record
    // j - i, so one round trip shows which of the nearest kWin records are
    // published, and the records of the ready run (up to and including the
    // first final state) are fetched together before they are combined,
    // nearest first.
    float acc_s = 0.0f;
    float acc_b[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc_b[g] = 0.0f;
    constexpr int kWin = 8;
    int j = rec - 1;
    int spins = 0;
    while (j >= rec0) {
      const int W = (j - rec0 + 1 < kWin) ? j - rec0 + 1 : kWin;
      const int st = lane < W ? load_relaxed(&sc.status[(j - lane) * NG + w]) : kEmpty;
      const uint64_t ready = __ballot(st >= kAggregate);
      const uint64_t incl = __ballot(st == kInclusive);
      // contiguous published run from the nearest record, cut after the first
      // final state in it
      const int run = static_cast<int>(__builtin_ctzll(~ready));  // ready has bit 63 clear
      const uint64_t run_mask = (1ull << run) - 1ull;
      const uint64_t inc_in_run = incl & run_mask;
      const int take = inc_in_run ? static_cast<int>(__builtin_ctzll(inc_in_run)) + 1 : run;
      if (take == 0) {
        if (++spins > sc.spin_limit) {
          if (lane == 0) atomicAdd(&g_carry_timeouts, 1u);
          break;  // timed out: continue with what was gathered
        }
        if (spins < 16) {
          __builtin_amdgcn_s_sleep(2);
        } else {
          __builtin_amdgcn_s_sleep(32);
        }
        continue;
      }
      acquire_fence();
      // the aggregates of the run (slots past it re-read record j), and the
      // final state that ends it, if any
      float rb[kWin][G], rs[kWin], ri[G];
#pragma unroll
      for (int k = 0; k < kWin; ++k) {
        const int jj = j - (k < take ? k : 0);
#pragma unroll
        for (int g = 0; g < G; ++g)
          rb[k][g] = sc.agg_b[(static_cast<int64_t>(jj) * N + gidx + g) * 64 + lane];
        rs[k] = sc.agg_s[(static_cast<int64_t>(jj) * NG + w) * 64 + lane];
      }
      {
        const int ji = j - take + 1;
#pragma unroll
        for (int g = 0; g < G; ++g)
          ri[g] = inc_in_run ? sc.inc[(static_cast<int64_t>(ji) * N + gidx + g) * 64 + lane] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < kWin; ++k) {
        if (k < take) {
          const bool last_inc = inc_in_run && k == take - 1;
#pragma unroll
          for (int g = 0; g < G; ++g)
            acc_b[g] = fmaf(exp2_hw(A2[g] * acc_s), last_inc ? ri[g] : rb[k][g], acc_b[g]);
          acc_s += rs[k];  // unused after a final state
        }
      }
      if (inc_in_run) break;
      j -= take;
      spins = 0;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) h[g] = acc_b[g];
    if (seg + 1 < nseg_c) {
      // this segment's own final state: its aggregate applied after the carry
#pragma unroll
      for (int g = 0; g < G; ++g)
        sc.inc[rec_state + (gidx + g) * 64 + lane] =
            fmaf(exp2_hw(A2[g] * sum_delta), h[g], hA[g]);
      if (lane == 0) store_release(&sc.status[rec * NG + w], kInclusive);
    }
    if constexpr (AGG) {
      // the segment's end state is the result
#pragma unroll
      for (int g = 0; g < G; ++g) h[g] = fmaf(exp2_hw(A2[g] * sum_delta), h[g], hA[g]);
      own_sum_delta = sum_delta;
    }
    published = true;
  }

  if constexpr (AGG) {
    if (!run_aggregate) {
      // one pass from the carry-in found above
      float hA[G];
#pragma unroll
      for (int g = 0; g < G; ++g) hA[g] = h[g];
      scan_aggregate(hA, own_sum_delta);
#pragma unroll
      for (int g = 0; g < G; ++g) h[g] = hA[g];
      // every record of a split chain carries its segment's sum of Delta (a
      // look-back segment stored it with its aggregate), released with the
      // record's status, so that the chain's last segment can add them up
      if (seg + 1 < nseg_c)
        sc.agg_s[(static_cast<int64_t>(rec) * NG + w) * 64 + lane] = own_sum_delta;
    }
  } else {
    scan_output(h);
  }

  if (!FROMREC && !published && seg + 1 < nseg_c) {
#pragma unroll
    for (int g = 0; g < G; ++g) sc.inc[rec_state + (gidx + g) * 64 + lane] = h[g];
    if (lane == 0) store_release(&sc.status[rec * NG + w], kInclusive);
  }
  if (seg + 1 == nseg_c && sh.has_last && dvalid) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      last_state[(static_cast<int64_t>(b) * dim + d) * N + gidx + g] = h[g];
  }
  if (AGG && seg + 1 == nseg_c && w == 0 && dvalid) {
    // the chain's sum of Delta, segment by segment in sequence order (every
    // earlier record was released before this segment acquired its carry)
    float total = 0.0f;
    for (int s = 0; s < seg; ++s) total += sc.agg_s[(static_cast<int64_t>(rec0 + s) * NG) * 64 + lane];
    sum_delta_out[static_cast<int64_t>(b) * dim + d] = total + own_sum_delta;
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
  constexpr int TC = chunk_for_groups(NG);
  constexpr int NP = helper_waves(NG, G);
  const dim3 grid(static_cast<unsigned>(workgroups)), block(64 * (NG + NP));
#define SSM_LAUNCH_FWD(Z, V)                                                                 \
  if (sh.mode == kModeRecord) {                                                              \
    SSM_LAUNCH_FWD_K(Z, V, kModeRecord);                                                     \
  } else if (sh.mode == kModeFromRecord) {                                                   \
    SSM_LAUNCH_FWD_K(Z, V, kModeFromRecord);                                                 \
  } else {                                                                                   \
    SSM_LAUNCH_FWD_K(Z, V, kModeForward);                                                    \
  }
#define SSM_LAUNCH_FWD_K(Z, V, AG)                                                           \
  hipLaunchKernelGGL((scan_fwd_kernel<T, NG, G, NP, TC, Z, V, AG>), grid, block, 0, stream,   \
                     static_cast<const T*>(p.u), static_cast<const T*>(p.delta), p.A,         \
                     static_cast<const T*>(p.B), static_cast<const T*>(p.C), p.D,             \
                     static_cast<const T*>(p.z), p.dt_bias, p.h0,                             \
                     static_cast<T*>(AG == kModeRecord ? static_cast<void*>(p.sum_delta)      \
                                                       : p.out),                              \
                     p.last_state, s, sh)
  if (sh.zoh) {
    if (sh.vec_io) {
      SSM_LAUNCH_FWD(true, true);
    } else {
      SSM_LAUNCH_FWD(true, false);
    }
  } else {
    if (sh.vec_io) {
      SSM_LAUNCH_FWD(false, true);
    } else {
      SSM_LAUNCH_FWD(false, false);
    }
  }
#undef SSM_LAUNCH_FWD
#undef SSM_LAUNCH_FWD_K
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
      if (groups == 8) return launch_typed<T, 8, 8>(p, s, sh, wg, st);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan_fwd(int groups, int per_group, const FwdPtrs& p, const FwdScratch& s,
                           const FwdShape& sh, int64_t workgroups, hipStream_t stream) {
  return dispatch_groups<SSM_FWD_T>(groups, per_group, p, s, sh, workgroups, stream);
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

}  // namespace SSM_FWD_NS
}  // namespace ssm
