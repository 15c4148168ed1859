// Backward of the selective scan (S6) for gfx950.
//
// The gradient of sum(dout * out) + sum(dlast * last_state) with respect to
// every input of the forward (reading guide, Method and Selection mechanism
// (S6) for the forward it differentiates).  The pages fix the memory plan:
// the intermediate states are recomputed on chip during the backward pass
// instead of being stored in HBM (reading guide, Hardware-aware state
// expansion; aigcdaily "Mamba：我们所知的ChatGPT时代的终结者？", Mamba block).
// Here only one state per TC-step chunk is kept (the checkpoint, N floats per
// channel per chunk); the states inside a chunk are recomputed into
// registers.
//
// Chain rule through h_t = Abar_t h_{t-1} + Delta_t u_t B_t, y_t = C_t . h_t
// + D u_t, out_t = y_t SiLU(z_t), with the adjoint lambda_t = dL/dh_t:
//   dy_t      = dout_t SiLU(z_t),   dz_t = dout_t y_t SiLU'(z_t)
//   lambda_t  = dy_t C_t + Abar_{t+1} lambda_{t+1},  lambda_{L-1} += dlast
//   dC_t[n]   = sum_d dy_t h_t[n]            dB_t[n] = sum_d lambda_t[n] Delta_t u_t
//   du_t      = Delta_t sum_n lambda_t B_t + D dy_t
//   dDelta_t  = u_t sum_n lambda_t B_t + sum_n lambda_t Abar_t h_{t-1} A
//   dA[n]     = sum_{b,t} lambda_t Abar_t h_{t-1} Delta_t
//   ddt_t     = dDelta_t softplus'(s_t) = dDelta_t sigmoid(s_t)
//   dh0       = Abar_0 lambda_0
// The adjoint is the forward's linear recurrence run backwards in time with
// decays Abar_{t+1}, the pair operator of "Mamba / MambaMini" Step 2 in
// reverse order.
//
// Work decomposition.  One workgroup per (batch, block of 64 channels); NG
// waves split the N states into groups of G as in the forward (lane =
// channel).  Phase F walks the sequence forwards and stores the state at the
// start of every chunk (checkpoint).  Phase R walks the chunks backwards: it
// reloads the chunk's inputs, recomputes the chunk's states and decays into
// registers from the checkpoint, forms dy and dz, runs the adjoint over the
// chunk, and reduces the per-channel terms:
//   over states (du, dDelta): per-wave partials through LDS, as the forward's
//     readout;
//   over channels (dB, dC): quad sums by DPP, then 16 quads per (t, n) in
//     LDS, written as this channel block's partial; a second kernel adds the
//     channel blocks (deterministic, no atomics);
//   over batch (dA, dD, ddt_bias): per-batch partials, added by the second
//     kernel.
// Rows of a ragged last chunk are padded with Delta = 0, Delta*u = 0, B = C =
// 0 and dy = 0, which makes them identity steps of both recurrences, so
// every chunk runs the same fully unrolled code.

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

__device__ unsigned g_bwd_carry_timeouts;

enum : int { kBwdEmpty = 0, kBwdAggregate = 1, kBwdInclusive = 2 };

template <typename T, int NG, int G, int TC, int TCF>
__global__ __launch_bounds__(64 * NG) void scan_bwd_kernel(BwdPtrs p, BwdShape sh) {
  constexpr int N = NG * G;
  constexpr int NT = 64 * NG;
  constexpr int NQ = 16;                       // quads per wave
  constexpr int EPT = TC / NG;                 // phase R: tile elements per thread
  constexpr int TPR = 64 / EPT;
  constexpr int EPTF = TCF / NG;               // phase F: tile elements per thread
  constexpr int TPRF = 64 / EPTF;
  constexpr int SUB = TCF / TC;                // checkpoints per phase-F chunk
  static_assert(TC % NG == 0 && EPT >= 1 && 64 % EPT == 0, "tile must split over the waves");
  static_assert(TCF % TC == 0 && 64 % EPTF == 0, "phase F chunk must hold whole chunks");
  static_assert(NT % TC == 0 && NT % TCF == 0, "tile rows must split over the threads");
  constexpr int BCE = (TC * N + NT - 1) / NT;   // B/C (or dB/dC) elements per thread, phase R
  constexpr int BCEF = (TCF * N + NT - 1) / NT; // B elements per thread, phase F
  using RunR = Run<T, EPT>;
  using RunF = Run<T, EPTF>;

  // Phase F and phase R use the same LDS.
  struct SmemR {
    float dl[TC][64];
    float du[TC][64];
    float dy[TC][64];
    float B[TC][N];
    float C[TC][N];
    float p1[NG][TC][64];      // partial y, then partial sum_n lambda B
    float p2[NG][TC][64];      // partial sum_n lambda Abar h_{t-1} A
    // quad sums of lambda Delta u and of dy h; rows padded to N + 1 words
    // so the 16 quad leaders of a wave write to 16 different banks
    float rB[TC][NQ][N + 1];
    float rC[TC][NQ][N + 1];
  };
  struct SmemF {
    float dl[2][TCF][64];
    float du[2][TCF][64];
    float B[2][TCF][N];
  };
  union Smem {
    SmemR r;
    SmemF f;
  };
  __shared__ __align__(16) Smem sm;
  __shared__ int s_ticket;
  __shared__ int s_pred_final;

  const T* const xu = static_cast<const T*>(p.u);
  const T* const xdt = static_cast<const T*>(p.delta);
  const T* const xB = static_cast<const T*>(p.B);
  const T* const xC = static_cast<const T*>(p.C);
  const T* const xz = static_cast<const T*>(p.z);
  const T* const xdo = static_cast<const T*>(p.dout);
  T* const gdu = static_cast<T*>(p.du);
  T* const gddl = static_cast<T*>(p.ddelta);
  T* const gdz = static_cast<T*>(p.dz);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups 0 .. n_full-1 run whole chains; the others are segments of
  // the split chains, ordered by an atomic ticket from the LAST segment in
  // time backwards (the adjoint runs backwards), so a segment only waits on
  // lower tickets, which are already running.
  const bool whole = static_cast<int>(blockIdx.x) < sh.n_full;
  int ticket = 0;
  if (!whole) {
    if (tid == 0) s_ticket = atomicAdd(p.ticket, 1);
    __syncthreads();
    ticket = __builtin_amdgcn_readfirstlane(s_ticket);
  }
  const int n_split = sh.chains - sh.n_full;
  const int rseg = whole ? 0 : ticket / n_split;
  const int chain = whole ? static_cast<int>(blockIdx.x) : sh.n_full + (ticket - rseg * n_split);
  const int nseg_c = whole ? 1 : sh.n_seg;
  const int seg = nseg_c - 1 - rseg;              // segment index in time order
  const int b = chain / sh.n_cblk;
  const int cblk = chain - b * sh.n_cblk;
  const int64_t L = sh.seqlen;
  const int64_t dim = sh.dim;
  const int64_t bsz = sh.batch;
  const int64_t ch0 = static_cast<int64_t>(cblk) * 64;
  const int64_t d = ch0 + lane;
  const bool dvalid = d < dim;
  const int64_t dc = dvalid ? d : dim - 1;
  const int gidx = w * G;

  float Af[G], A2[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    Af[g] = p.A[dc * N + gidx + g];
    A2[g] = Af[g] * kLog2e;
  }
  const int64_t row0 = static_cast<int64_t>(b) * L;
  const int64_t nck = sh.nchunks;
  float* ckpt = p.ckpt + (static_cast<int64_t>(chain) * nck) * N * 64;
  // this workgroup's time range and chunks
  const int64_t seg_len_c = whole ? L : sh.seg_len;
  const int64_t t_begin = static_cast<int64_t>(seg) * seg_len_c;
  const int64_t t_end = (t_begin + seg_len_c < L) ? t_begin + seg_len_c : L;
  const int64_t c_lo = t_begin / TC;
  const int64_t c_hi = (t_end - 1) / TC;
  const int rec = whole ? 0 : (chain - sh.n_full) * sh.n_seg + seg;
  const int slot = whole ? 0 : seg;               // partial-sum slot of dA, dD, ddt_bias

  // Tile roles: a thread owns one row of a chunk tile and a run of EPT (phase
  // R) or EPTF (phase F) consecutive channels.  last = index of the run's
  // last channel inside dim, -1 if none.
  auto run_role = [&](int ept, int tpr, int& row, int& col, int& last) {
    row = tid / tpr;
    col = (tid - row * tpr) * ept;
    const int64_t first = ch0 + col;
    last = first < dim ? static_cast<int>((dim - 1 - first) < (ept - 1) ? (dim - 1 - first)
                                                                     : (ept - 1))
                       : -1;
  };
  int tr, tc, run_last, trf, tcf, run_last_f;
  run_role(EPT, TPR, tr, tc, run_last);
  run_role(EPTF, TPRF, trf, tcf, run_last_f);
  const int64_t tch = ch0 + tc, tchf = ch0 + tcf;
  const bool run_valid = run_last >= 0, run_valid_f = run_last_f >= 0;
  const bool run_vec = RunR::kCanVec && sh.vec_io != 0 && run_valid;
  const bool run_vec_f = RunF::kCanVec && sh.vec_io_f != 0 && run_valid_f;
  const int64_t tch_c = run_valid ? tch : dim - 1;
  const int64_t tchf_c = run_valid_f ? tchf : dim - 1;
  const int elem_last = run_last > 0 ? run_last : 0;
  const int elem_last_f = run_last_f > 0 ? run_last_f : 0;

  // ---- phase F: checkpoints, with loads one chunk of TCF steps ahead -------
  // (skipped when the forward's training mode has written them)
  if (!p.ckpt_in) {
    float rbias_f[EPTF];
#pragma unroll
    for (int k = 0; k < EPTF; ++k)
      rbias_f[k] = sh.has_bias ? p.dt_bias[tchf_c + (k < elem_last_f ? k : elem_last_f)] : 0.0f;
    struct RawF {
      RunF dt, u;
      T bb[BCEF];
    };
    auto load_f = [&](int64_t c0, int n, RawF& r) {
      const int rr = trf < n ? trf : n - 1;
      const int64_t off = (row0 + c0 + rr) * dim + tchf_c;
      if (run_vec_f) {
        r.dt.load_vec(xdt + off);
        r.u.load_vec(xu + off);
      } else {
        r.dt.load_elems(xdt + off, elem_last_f);
        r.u.load_elems(xu + off, elem_last_f);
      }
      const int64_t base = (row0 + c0) * N;
#pragma unroll
      for (int k = 0; k < BCEF; ++k) {
        const int e = tid + k * NT;
        r.bb[k] = xB[base + ((e < n * N) ? e : 0)];
      }
    };
    auto stage_f = [&](int buf, int n, const RawF& r) {
      r.dt.consume_all();
      r.u.consume_all();
#pragma unroll
      for (int k = 0; k < EPTF; ++k) {
        const bool ok = trf < n && k <= run_last_f;
        const float s = r.dt.get(k) + rbias_f[k];
        const float dl = sh.softplus ? softplus_f32(s) : s;
        sm.f.dl[buf][trf][tcf + k] = ok ? dl : 0.0f;
        sm.f.du[buf][trf][tcf + k] = ok ? dl * r.u.get(k) : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < BCEF; ++k) {
        const int e = tid + k * NT;
        const float bv = to_f32(r.bb[k]);
        if (e < TCF * N) sm.f.B[buf][e / N][e % N] = e < n * N ? bv : 0.0f;
      }
    };
    float h[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      h[g] = (sh.has_h0 && dvalid) ? p.h0[(static_cast<int64_t>(b) * dim + d) * N + gidx + g]
                                   : 0.0f;
    const int64_t nckf = (L + TCF - 1) / TCF;
    RawF raw;
    load_f(0, static_cast<int>(L < TCF ? L : TCF), raw);
    stage_f(0, static_cast<int>(L < TCF ? L : TCF), raw);
    drain_vmem();
    lds_barrier();
    int buf = 0;
    for (int64_t cf = 0; cf < nckf; ++cf) {
      const int64_t nx = cf + 1 < nckf ? cf + 1 : cf;   // the last chunk reloads itself
      const int64_t nx0 = nx * TCF;
      const int n_nx = static_cast<int>((L - nx0 < TCF) ? L - nx0 : TCF);
      load_f(nx0, n_nx, raw);
#pragma unroll
      for (int sc = 0; sc < SUB; ++sc) {
        const int64_t c = cf * SUB + sc;
        if (c < nck) {
#pragma unroll
          for (int g = 0; g < G; ++g) ckpt[(c * N + gidx + g) * 64 + lane] = h[g];
        }
#pragma unroll
        for (int t = 0; t < TC; ++t) {
          const int row = sc * TC + t;
          const float dl = sm.f.dl[buf][row][lane];
          const float du = sm.f.du[buf][row][lane];
#pragma unroll
          for (int g = 0; g < G; ++g)
            h[g] = fmaf(exp2_hw(dl * A2[g]), h[g], du * sm.f.B[buf][row][gidx + g]);
        }
      }
      stage_f(buf ^ 1, n_nx, raw);
      lds_barrier();
      buf ^= 1;
    }
  }
  __syncthreads();  // phase F's LDS is reused by phase R

  // ---- phase R: chunks of TC steps in reverse, loads one chunk ahead -------
  float rD[EPT], rbias[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int64_t ck = tch_c + (k < elem_last ? k : elem_last);
    rD[k] = sh.has_D ? p.D[ck] : 0.0f;
    rbias[k] = sh.has_bias ? p.dt_bias[ck] : 0.0f;
  }
  struct RawR {
    RunR dt, u, z, dout;
    T bb[BCE], cc[BCE];
    float ck[G];
  };
  // the thread's run of a chunk, converted
  struct RunVals {
    float u[EPT], dl[EPT], sig[EPT], z[EPT], dout[EPT];
  };
  auto load_r = [&](int64_t c, RawR& r) {
    const int64_t c0 = c * TC;
    const int n = static_cast<int>((L - c0 < TC) ? L - c0 : TC);
    const int rr = tr < n ? tr : n - 1;
    const int64_t off = (row0 + c0 + rr) * dim + tch_c;
    if (run_vec) {
      r.dt.load_vec(xdt + off);
      r.u.load_vec(xu + off);
      if (sh.has_z) r.z.load_vec(xz + off);
      r.dout.load_vec(xdo + off);
    } else {
      r.dt.load_elems(xdt + off, elem_last);
      r.u.load_elems(xu + off, elem_last);
      if (sh.has_z) r.z.load_elems(xz + off, elem_last);
      r.dout.load_elems(xdo + off, elem_last);
    }
    const int64_t base = (row0 + c0) * N;
#pragma unroll
    for (int k = 0; k < BCE; ++k) {
      const int e = tid + k * NT;
      const int64_t ec = base + ((e < n * N) ? e : 0);
      r.bb[k] = xB[ec];
      r.cc[k] = xC[ec];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) r.ck[g] = ckpt[(c * N + gidx + g) * 64 + lane];
  };
  auto stage_r = [&](int64_t c, const RawR& r, RunVals& rv, float (&hst)[G]) {
    const int64_t c0 = c * TC;
    const int n = static_cast<int>((L - c0 < TC) ? L - c0 : TC);
    r.dt.consume_all();
    r.u.consume_all();
    if (sh.has_z) r.z.consume_all();
    r.dout.consume_all();
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const bool ok = tr < n && k <= run_last;
      const float s = r.dt.get(k) + rbias[k];
      const float dl = sh.softplus ? softplus_f32(s) : s;
      rv.u[k] = r.u.get(k);
      rv.dl[k] = ok ? dl : 0.0f;
      rv.sig[k] = sh.softplus ? sigmoid_f32(s) : 1.0f;
      rv.z[k] = sh.has_z ? r.z.get(k) : 0.0f;
      rv.dout[k] = r.dout.get(k);
      sm.r.dl[tr][tc + k] = rv.dl[k];
      sm.r.du[tr][tc + k] = ok ? dl * rv.u[k] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < BCE; ++k) {
      const int e = tid + k * NT;
      const float bv = to_f32(r.bb[k]);
      const float cv = to_f32(r.cc[k]);
      if (e < TC * N) {
        sm.r.B[e / N][e % N] = e < n * N ? bv : 0.0f;
        sm.r.C[e / N][e % N] = e < n * N ? cv : 0.0f;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) hst[g] = r.ck[g];
  };

  float lamn[G], dA_acc[G];   // lamn = Abar_{t+1} lambda_{t+1}
#pragma unroll
  for (int g = 0; g < G; ++g) dA_acc[g] = 0.0f;
  bool published = false;
  if (seg == nseg_c - 1) {
    // the last segment in time starts from the final state's gradient
#pragma unroll
    for (int g = 0; g < G; ++g)
      lamn[g] = (sh.has_dlast && dvalid)
                    ? p.dlast[(static_cast<int64_t>(b) * dim + d) * N + gidx + g]
                    : 0.0f;
  } else {
    // A split segment needs the adjoint carried out of the segments after
    // it.  If the next segment has published its inclusive carry for every
    // state group, take it; otherwise compute this segment's aggregate (the
    // adjoint run backwards over the segment from zero, and its sum of
    // Delta), publish it, and walk the later segments' records.  The map
    // carry-in -> carry-out of a segment is lamn_out = exp(A sum Delta)
    // lamn_in + lamn_out(0): the pair operator of "Mamba / MambaMini" Step 2.
    if (tid == 0) {
      int all = 1;
      for (int q = 0; q < NG; ++q)
        all &= __hip_atomic_load(&p.status[(rec + 1) * NG + q], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT) == kBwdInclusive;
      s_pred_final = all;
    }
    lds_barrier();
    const bool next_final = __builtin_amdgcn_readfirstlane(s_pred_final) != 0;
    const int64_t rs_base = static_cast<int64_t>(rec) * N * 64;
    if (next_final) {
      acquire_fence();
      const int64_t ns = static_cast<int64_t>(rec + 1) * N * 64;
#pragma unroll
      for (int g = 0; g < G; ++g) lamn[g] = p.inc[ns + (gidx + g) * 64 + lane];
    } else {
      float lamA[G], sum_delta = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) lamA[g] = 0.0f;
      for (int64_t c = c_hi; c >= c_lo; --c) {
        const int64_t c0 = c * TC;
        const int n = static_cast<int>((L - c0 < TC) ? L - c0 : TC);
        RawR raw;
        RunVals rv;
        float unused[G];
        load_r(c, raw);
        stage_r(c, raw, rv, unused);
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          const bool ok = tr < n && k <= run_last;
          float dyk = rv.dout[k];
          if (sh.has_z) dyk = rv.dout[k] * (rv.z[k] * sigmoid_f32(rv.z[k]));
          sm.r.dy[tr][tc + k] = ok ? dyk : 0.0f;
        }
        lds_barrier();
#pragma unroll
        for (int t = TC - 1; t >= 0; --t) {
          const float dl = sm.r.dl[t][lane];
          const float dyt = sm.r.dy[t][lane];
          sum_delta += dl;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float lam = fmaf(dyt, sm.r.C[t][gidx + g], lamA[g]);
            lamA[g] = exp2_hw(dl * A2[g]) * lam;
          }
        }
        lds_barrier();
      }
#pragma unroll
      for (int g = 0; g < G; ++g) p.agg_b[rs_base + (gidx + g) * 64 + lane] = lamA[g];
      p.agg_s[(static_cast<int64_t>(rec) * NG + w) * 64 + lane] = sum_delta;
      if (lane == 0)
        __hip_atomic_store(&p.status[rec * NG + w], kBwdAggregate, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
      // walk the later segments in windows of kWin: lane i polls record j + i
      float acc_s = 0.0f, acc_b[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc_b[g] = 0.0f;
      const int rec_last = (chain - sh.n_full) * sh.n_seg + sh.n_seg - 1;
      constexpr int kWin = 8;
      int j = rec + 1;
      int spins = 0;
      while (j <= rec_last) {
        const int W = (rec_last - j + 1 < kWin) ? rec_last - j + 1 : kWin;
        const int st = lane < W ? __hip_atomic_load(&p.status[(j + lane) * NG + w],
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : kBwdEmpty;
        const uint64_t ready = __ballot(st >= kBwdAggregate);
        const uint64_t incl = __ballot(st == kBwdInclusive);
        const int run = static_cast<int>(__builtin_ctzll(~ready));
        const uint64_t inc_in_run = incl & ((1ull << run) - 1ull);
        const int take = inc_in_run ? static_cast<int>(__builtin_ctzll(inc_in_run)) + 1 : run;
        if (take == 0) {
          if (++spins > sh.spin_limit) {
            if (lane == 0) atomicAdd(&g_bwd_carry_timeouts, 1u);
            break;
          }
          if (spins < 16) {
            __builtin_amdgcn_s_sleep(2);
          } else {
            __builtin_amdgcn_s_sleep(32);
          }
          continue;
        }
        acquire_fence();
        float rb[kWin][G], rsum[kWin], ri[G];
#pragma unroll
        for (int k = 0; k < kWin; ++k) {
          const int jj = j + (k < take ? k : 0);
#pragma unroll
          for (int g = 0; g < G; ++g)
            rb[k][g] = p.agg_b[(static_cast<int64_t>(jj) * N + gidx + g) * 64 + lane];
          rsum[k] = p.agg_s[(static_cast<int64_t>(jj) * NG + w) * 64 + lane];
        }
        {
          const int ji = j + take - 1;
#pragma unroll
          for (int g = 0; g < G; ++g)
            ri[g] = inc_in_run ? p.inc[(static_cast<int64_t>(ji) * N + gidx + g) * 64 + lane]
                               : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kWin; ++k) {
          if (k < take) {
            const bool last_inc = inc_in_run && k == take - 1;
#pragma unroll
            for (int g = 0; g < G; ++g)
              acc_b[g] = fmaf(exp2_hw(A2[g] * acc_s), last_inc ? ri[g] : rb[k][g], acc_b[g]);
            acc_s += rsum[k];
          }
        }
        if (inc_in_run) break;
        j += take;
        spins = 0;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) lamn[g] = acc_b[g];
      if (seg > 0) {
        // this segment's own carry-out: its aggregate applied after the carry-in
#pragma unroll
        for (int g = 0; g < G; ++g)
          p.inc[rs_base + (gidx + g) * 64 + lane] =
              fmaf(exp2_hw(A2[g] * sum_delta), lamn[g], lamA[g]);
        if (lane == 0)
          __hip_atomic_store(&p.status[rec * NG + w], kBwdInclusive, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      published = true;
    }
  }
  float dD_acc[EPT], dbias_acc[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    dD_acc[k] = 0.0f;
    dbias_acc[k] = 0.0f;
  }
  float* part_bc = p.part_bc + (static_cast<int64_t>(cblk) * bsz + b) * L * (2 * N);

  RawR raw;
  RunVals rv;
  float hstart[G];
  load_r(c_hi, raw);
  stage_r(c_hi, raw, rv, hstart);
  drain_vmem();
  lds_barrier();
  for (int64_t c = c_hi; c >= c_lo; --c) {
    const int64_t c0 = c * TC;
    const int n = static_cast<int>((L - c0 < TC) ? L - c0 : TC);
    const bool row_ok = tr < n;
    const int64_t cn = c > c_lo ? c - 1 : c_lo;   // next chunk to stage (the first reloads itself)
    load_r(cn, raw);

    // recompute the chunk's states and decays from its checkpoint
    float h[G], hs[TC][G], as[TC][G];
#pragma unroll
    for (int g = 0; g < G; ++g) h[g] = hstart[g];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      const float dl = sm.r.dl[t][lane];
      const float du = sm.r.du[t][lane];
      float y = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float a = exp2_hw(dl * A2[g]);
        h[g] = fmaf(a, h[g], du * sm.r.B[t][gidx + g]);
        as[t][g] = a;
        hs[t][g] = h[g];
        y = fmaf(sm.r.C[t][gidx + g], h[g], y);
      }
      sm.r.p1[w][t][lane] = y;
    }
    lds_barrier();

    // dy, dz for this thread's run
    float dy[EPT];
    {
      float dzv[EPT];
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        const bool ok = row_ok && k <= run_last;
        float y = sm.r.p1[0][tr][tc + k];
#pragma unroll
        for (int q = 1; q < NG; ++q) y += sm.r.p1[q][tr][tc + k];
        y += rD[k] * rv.u[k];
        const float go = rv.dout[k];
        float dyk = go;
        dzv[k] = 0.0f;
        if (sh.has_z) {
          const float zv = rv.z[k];
          const float sg = sigmoid_f32(zv);
          dyk = go * (zv * sg);
          dzv[k] = go * y * (sg * fmaf(zv, 1.0f - sg, 1.0f));
        }
        dy[k] = ok ? dyk : 0.0f;
        sm.r.dy[tr][tc + k] = dy[k];
        dD_acc[k] = fmaf(dy[k], rv.u[k], dD_acc[k]);
      }
      if (sh.has_z && gdz && row_ok && run_valid)
        store_run<T, EPT>(gdz + (row0 + c0 + tr) * dim + tch, dzv, run_vec, run_last);
    }
    lds_barrier();

    // adjoint over the chunk, last step first
#pragma unroll
    for (int t = TC - 1; t >= 0; --t) {
      const float dl = sm.r.dl[t][lane];
      const float du = sm.r.du[t][lane];
      const float dyt = sm.r.dy[t][lane];
      float s1 = 0.0f, s2 = 0.0f;
      float pB[G], pC[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float lam = fmaf(dyt, sm.r.C[t][gidx + g], lamn[g]);
        pC[g] = dyt * hs[t][g];
        pB[g] = lam * du;
        s1 = fmaf(lam, sm.r.B[t][gidx + g], s1);
        const float hp = t > 0 ? hs[t > 0 ? t - 1 : 0][g] : hstart[g];
        lamn[g] = as[t][g] * lam;               // Abar_t lambda_t, carried to step t-1
        const float lq = lamn[g] * hp;          // lambda_t Abar_t h_{t-1}
        s2 = fmaf(lq, Af[g], s2);
        dA_acc[g] = fmaf(lq, dl, dA_acc[g]);
      }
      sm.r.p1[w][t][lane] = s1;
      sm.r.p2[w][t][lane] = s2;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        pB[g] = quad_sum(pB[g]);
        pC[g] = quad_sum(pC[g]);
      }
      if ((lane & 3) == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          sm.r.rB[t][lane >> 2][gidx + g] = pB[g];
          sm.r.rC[t][lane >> 2][gidx + g] = pC[g];
        }
      }
    }
    lds_barrier();

    // du, ddelta for this thread's run
    {
      float duv[EPT], ddv[EPT];
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        const bool ok = row_ok && k <= run_last;
        float S1 = sm.r.p1[0][tr][tc + k];
        float S2 = sm.r.p2[0][tr][tc + k];
#pragma unroll
        for (int q = 1; q < NG; ++q) {
          S1 += sm.r.p1[q][tr][tc + k];
          S2 += sm.r.p2[q][tr][tc + k];
        }
        duv[k] = fmaf(rv.dl[k], S1, rD[k] * dy[k]);
        const float ddl = fmaf(rv.u[k], S1, S2);
        ddv[k] = ddl * rv.sig[k];
        dbias_acc[k] += ok ? ddv[k] : 0.0f;
      }
      if (row_ok && run_valid) {
        const int64_t o = (row0 + c0 + tr) * dim + tch;
        store_run<T, EPT>(gdu + o, duv, run_vec, run_last);
        store_run<T, EPT>(gddl + o, ddv, run_vec, run_last);
      }
    }
    // this channel block's dB / dC rows: add the 16 quad sums
#pragma unroll
    for (int k = 0; k < BCE; ++k) {
      const int e = tid + k * NT;
      if (e < TC * N) {
        const int row = e / N;
        const int nn = e - row * N;
        float sb = 0.0f, scv = 0.0f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          sb += sm.r.rB[row][q][nn];
          scv += sm.r.rC[row][q][nn];
        }
        if (row < n) {
          float* pr = part_bc + (c0 + row) * (2 * N);
          pr[nn] = sb;
          pr[N + nn] = scv;
        }
      }
    }
    // the next chunk's inputs (its rows and channels are read only after
    // the barrier; the adjoint that read this chunk's finished before the
    // barrier above)
    stage_r(cn, raw, rv, hstart);
    lds_barrier();
  }

  // a segment that took its carry-in ready-made publishes its carry-out now
  if (!whole && !published && seg > 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      p.inc[static_cast<int64_t>(rec) * N * 64 + (gidx + g) * 64 + lane] = lamn[g];
    if (lane == 0)
      __hip_atomic_store(&p.status[rec * NG + w], kBwdInclusive, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- per-(batch, segment) partials of dA, dD, ddt_bias; dh0 -------------
  const int64_t pslot = static_cast<int64_t>(b) * sh.n_seg + slot;
  if (dvalid) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      p.part_a[(pslot * dim + d) * N + gidx + g] = dA_acc[g];
      if (p.dh0 && seg == 0)
        p.dh0[(static_cast<int64_t>(b) * dim + d) * N + gidx + g] = lamn[g];
    }
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    sm.r.p1[0][tr][tc + k] = dD_acc[k];
    sm.r.p2[0][tr][tc + k] = dbias_acc[k];
  }
  lds_barrier();
  if (tid < 64 && ch0 + tid < dim) {
    float sd = 0.0f, sbias = 0.0f;
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      sd += sm.r.p1[0][t][tid];
      sbias += sm.r.p2[0][t][tid];
    }
    p.part_d[pslot * dim + ch0 + tid] = sd;
    p.part_bias[pslot * dim + ch0 + tid] = sbias;
  }
}

// dB[r][n] = sum_k part[k][r][n], dC[r][n] = sum_k part[k][r][N + n] over the
// channel blocks k, for r = (b, t).
template <typename T>
__global__ __launch_bounds__(256) void reduce_bc_kernel(const float* __restrict__ part,
                                                        T* __restrict__ dB, T* __restrict__ dC,
                                                        int64_t rows, int n, int blocks) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= rows * n) return;
  const int64_t r = i / n;
  const int64_t nn = i - r * n;
  const int64_t stride = rows * 2 * n;
  const float* q = part + r * 2 * n + nn;
  float sb = 0.0f, sc = 0.0f;
  for (int k = 0; k < blocks; ++k) {
    sb += q[k * stride];
    sc += q[k * stride + n];
  }
  store_act(dB, i, sb);
  store_act(dC, i, sc);
}

// out[i] = sum_k part[k * count + i]
__global__ __launch_bounds__(256) void reduce_sum_kernel(const float* __restrict__ part,
                                                         float* __restrict__ out, int64_t count,
                                                         int parts) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.0f;
  for (int k = 0; k < parts; ++k) s += part[k * count + i];
  out[i] = s;
}

static dim3 grid_for(int64_t count) {
  return dim3(static_cast<unsigned>((count + 255) / 256));
}

__global__ void bwd_fill_zero_kernel(int* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <typename T, int NG, int G>
static hipError_t launch_bwd_typed(const BwdPtrs& p, const BwdShape& sh, hipStream_t st) {
  constexpr int TC = kBwdChunk;
  constexpr int TCF = kBwdFwdChunk;
  hipError_t e;
  if (sh.n_seg > 1) {
    // split chains: zero the ticket, the status words and the partial-sum
    // slots that whole chains leave unwritten
    const int64_t n_int = 1 + static_cast<int64_t>(sh.chains - sh.n_full) * sh.n_seg * NG;
    hipLaunchKernelGGL(bwd_fill_zero_kernel, grid_for(n_int), dim3(256), 0, st, p.ticket, n_int);
    const int64_t na = sh.batch * sh.n_seg * sh.dim * (NG * G);
    const int64_t nd = sh.batch * sh.n_seg * sh.dim;
    hipLaunchKernelGGL(bwd_fill_zero_kernel, grid_for(na), dim3(256), 0, st,
                       reinterpret_cast<int*>(p.part_a), na);
    hipLaunchKernelGGL(bwd_fill_zero_kernel, grid_for(nd), dim3(256), 0, st,
                       reinterpret_cast<int*>(p.part_d), nd);
    hipLaunchKernelGGL(bwd_fill_zero_kernel, grid_for(nd), dim3(256), 0, st,
                       reinterpret_cast<int*>(p.part_bias), nd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t workgroups = sh.n_full + static_cast<int64_t>(sh.chains - sh.n_full) * sh.n_seg;
  const dim3 grid(static_cast<unsigned>(workgroups)), block(64 * NG);
  hipLaunchKernelGGL((scan_bwd_kernel<T, NG, G, TC, TCF>), grid, block, 0, st, p, sh);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int N = NG * G;
  const int64_t rows = sh.batch * sh.seqlen;
  hipLaunchKernelGGL(reduce_bc_kernel<T>, grid_for(rows * N), dim3(256), 0, st, p.part_bc,
                     static_cast<T*>(p.dB), static_cast<T*>(p.dC), rows, N, sh.n_cblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int parts = static_cast<int>(sh.batch * sh.n_seg);
  hipLaunchKernelGGL(reduce_sum_kernel, grid_for(sh.dim * N), dim3(256), 0, st, p.part_a, p.dA,
                     sh.dim * N, parts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.dD) {
    hipLaunchKernelGGL(reduce_sum_kernel, grid_for(sh.dim), dim3(256), 0, st, p.part_d, p.dD,
                       sh.dim, parts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.ddt_bias) {
    hipLaunchKernelGGL(reduce_sum_kernel, grid_for(sh.dim), dim3(256), 0, st, p.part_bias,
                       p.ddt_bias, sh.dim, parts);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
static hipError_t dispatch_bwd(int dstate, const BwdPtrs& p, const BwdShape& sh,
                               hipStream_t st) {
  switch (dstate) {
    case 1: return launch_bwd_typed<T, 1, 1>(p, sh, st);
    case 2: return launch_bwd_typed<T, 1, 2>(p, sh, st);
    case 4: return launch_bwd_typed<T, 1, 4>(p, sh, st);
    case 8: return launch_bwd_typed<T, 2, 4>(p, sh, st);
    case 16: return launch_bwd_typed<T, 4, 4>(p, sh, st);
    case 32: return launch_bwd_typed<T, 8, 4>(p, sh, st);
    case 64: return launch_bwd_typed<T, 8, 8>(p, sh, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t read_and_clear_bwd_errors(hipStream_t stream, unsigned* count) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_bwd_carry_timeouts), sizeof(unsigned), 0,
                          hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const unsigned zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_bwd_carry_timeouts), &zero, sizeof(unsigned), 0,
                           hipMemcpyHostToDevice);
}

hipError_t launch_scan_bwd(int dtype, int dstate, const BwdPtrs& p, const BwdShape& sh,
                           hipStream_t stream) {
  if (dtype == 0) return dispatch_bwd<float>(dstate, p, sh, stream);
  return dispatch_bwd<bf16_t>(dstate, p, sh, stream);
}

}  // namespace ssm
