// C ABI of the selective-scan library: validation, launch planning, scratch,
// dispatch.  The operations and conventions are documented in ssm_scan.h.

#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/ssm_scan.h"
#include "ssm_internal.h"

namespace {

constexpr int kDefaultSpinLimit = 1 << 24;
constexpr int64_t kComputeUnits = 256;  // MI355X (gfx950)

// Scratch of the allocation-free forward (selective_scan_fwd_noalloc): the
// ticket, status words and carry records of one call, in an array that every
// device the library runs on holds (its own copy, at its own address) until
// the process ends.  In host code `scratch` is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is passed to
// kernels.  Calls on one device share the array, so calls that overlap on a
// device race on it.
constexpr int64_t kStaticScratchBytes = int64_t{32} << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// This device's address of `scratch` (set-up on the device's first call).
int static_scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSM_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSM_ELAUNCH;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return SSM_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_dstate(int64_t n) {
  return n == 1 || n == 2 || n == 4 || n == 8 || n == 16 || n == 32 || n == 64;
}

int env_int(const char* name, int fallback) {
  const char* v = getenv(name);
  if (!v || !*v) return fallback;
  char* end = nullptr;
  const long x = strtol(v, &end, 10);
  return (end && *end == '\0') ? static_cast<int>(x) : fallback;
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of states each wave keeps per channel.
int states_per_group(int64_t n) {
  int g = env_int("SSM_FORCE_STATES_PER_GROUP", 0);
  if (g > 0 && g <= 16 && n % g == 0) {
    const int64_t groups = n / g;
    // instantiated (groups, per-group) pairs
    if ((n <= 2 && groups == 1) || (n == 4 && groups == 1) || (n == 8 && (groups <= 2)) ||
        (n == 16 && (groups == 1 || groups == 2 || groups == 4 || groups == 8)) ||
        (n == 32 && groups == 8) || (n == 64 && groups == 8))
      return g;
  }
  if (n == 64) return 8;
  return n < 4 ? static_cast<int>(n) : 4;
}

// Chooses state groups, segments and the carry mode for a forward call.
// When the channel blocks alone give at least half the chip's SIMDs a wave,
// each channel block is scanned by one workgroup over the whole sequence (a
// single segment: measured faster than chained segments, whose waiting
// workgroups occupy CU slots).  Otherwise the sequence is cut into segments
// that run concurrently and exchange carries by decoupled look-back; a
// segment whose predecessor has already published its final state skips its
// own aggregate pass.
void plan_forward(const ssm_dims& d, ssm_fwd_plan* p) {
  const int g = states_per_group(d.dstate);
  const int groups = static_cast<int>(d.dstate / g);
  const int chunk = ssm::chunk_for_groups(groups);
  const int64_t cblk = div_up(d.dim, 64);
  const int64_t chains = d.batch * cblk;
  const int64_t waves_per_slice = chains * groups;
  int lookback = waves_per_slice >= 512 ? 0 : 1;
  const int force_mode = env_int("SSM_FORCE_LOOKBACK", -1);
  if (force_mode == 0 || force_mode == 1) lookback = force_mode;

  int64_t seg_len;
  if (!lookback) {
    seg_len = d.seqlen;
  } else {
    // enough segments for ~2048 waves (two per SIMD), each at least 128
    // steps (512 from 16K steps on): the measured best trade of parallelism
    // against the extra aggregate pass, the per-segment start-up and the
    // look-back walk at 256 channels, from 4K to 1M steps
    const int64_t want = div_up(2048, waves_per_slice);
    const int64_t min_seg = d.seqlen >= 16384 ? 512 : 128;
    seg_len = div_up(d.seqlen, want);
    if (seg_len < min_seg) seg_len = min_seg;
  }
  const int force_seg = env_int("SSM_FORCE_SEGMENT", 0);
  if (force_seg > 0) seg_len = force_seg;
  // segments are whole chunks of the kernel instance (16 steps from four
  // state groups on, 32 below), so only a sequence's last segment can end in
  // a partial chunk
  seg_len = div_up(seg_len, chunk) * chunk;
  if (seg_len > d.seqlen) seg_len = div_up(d.seqlen, chunk) * chunk;
  int64_t n_seg = div_up(d.seqlen, seg_len);
  if (n_seg == 1) lookback = 0;
  int64_t whole = n_seg == 1 ? chains : 0;
  int64_t first_len = seg_len;

  // Whole chains beyond a multiple of the CU count would double up on some
  // CUs while the rest idle for the second half.  Those M chains are split
  // into S ~ CUs/M look-back segments instead, so every CU runs one whole
  // chain plus one short segment.
  if (n_seg == 1 && force_mode < 0 && force_seg == 0) {
    const int64_t K = (chains / kComputeUnits) * kComputeUnits;
    const int64_t M = chains - K;
    int64_t S = (K > 0 && M > 0) ? kComputeUnits / M : 1;
    if (S < 3) S = 1;
    const int force_split = env_int("SSM_FORCE_SPLIT", -1);
    if (force_split >= 1 && K > 0 && M > 0) S = force_split;
    if (S > 1) {
      const int64_t sl = div_up(div_up(d.seqlen, S), chunk) * chunk;
      if (div_up(d.seqlen, sl) > 1) {
        seg_len = sl;
        first_len = sl;
        n_seg = div_up(d.seqlen, sl);
        whole = K;
        lookback = 1;
      }
    }
  }
  // A split chain's first segment starts from the initial state and skips
  // the aggregate pass, but its successors' look-back ends only at its final
  // state, published when its output pass ends.  SSM_FORCE_FIRST_SEGMENT
  // sets its length (steps, rounded to the chunk); the other segments then
  // share the rest of the sequence evenly, their count not growing.
  const int force_first = env_int("SSM_FORCE_FIRST_SEGMENT", 0);
  if (n_seg > 1 && force_first > 0) {
    const int64_t fl = div_up(force_first, chunk) * chunk;
    if (fl < d.seqlen) {
      first_len = fl;
      seg_len = div_up(div_up(d.seqlen - fl, n_seg - 1), chunk) * chunk;
      n_seg = 1 + div_up(d.seqlen - fl, seg_len);
    }
  }

  p->state_groups = groups;
  p->states_per_group = g;
  p->segments = static_cast<int32_t>(n_seg);
  p->segment_len = static_cast<int32_t>(seg_len);
  p->lookback = lookback;
  p->chunk = chunk;
  p->workgroups = whole + (chains - whole) * n_seg;
  p->whole_chains = static_cast<int32_t>(whole);
  p->first_segment_len = static_cast<int32_t>(first_len);
  p->helper_waves = ssm::helper_waves(groups, g);
}

int check_dims(const ssm_dims* dims) {
  if (!dims) return SSM_EINVAL;
  if (dims->dtype != SSM_F32 && dims->dtype != SSM_BF16) return SSM_EDTYPE;
  if (dims->batch <= 0 || dims->seqlen <= 0 || dims->dim <= 0 || dims->dstate <= 0)
    return SSM_EINVAL;
  if (!valid_dstate(dims->dstate)) return SSM_EINVAL;
  // 32-bit limits of the launch arithmetic (segment length, channel blocks)
  const int64_t cblk = div_up(dims->dim, 64);
  if (dims->batch * cblk > (1LL << 30)) return SSM_EINVAL;
  if (dims->seqlen > (1LL << 31) - 1024) return SSM_EINVAL;
  // the kernels address a chunk's rows with 32-bit offsets
  if (dims->dim > (1LL << 24)) return SSM_EINVAL;
  return SSM_OK;
}

// Bytes of the training mode's chunk-start states, and the offset of its
// saved readouts (the rest of the checkpoint buffer).
int64_t ckpt_state_bytes(const ssm_dims* dims) {
  return dims->batch * div_up(dims->dim, 64) * div_up(dims->seqlen, ssm::kBwdChunk) *
         dims->dstate * 64 * 4;
}
int64_t ckpt_y_offset(const ssm_dims* dims) { return div_up(ckpt_state_bytes(dims), 256) * 256; }

// The forward's scratch: the ticket and status words, then the split
// segments' carry records (end state; aggregate from zero and sum of Delta
// where the plan walks back; the sums also where they are kept for a record
// or the chain's total), each piece 256-byte aligned.
struct FwdScratchLayout {
  int64_t n_int, off_inc, inc_bytes, aggb_bytes, aggs_bytes, total;
};
FwdScratchLayout fwd_scratch_layout(const ssm_fwd_plan& plan, int64_t recs, int64_t N,
                                    bool keep_sums) {
  auto up256 = [](int64_t bytes) { return div_up(bytes, 256) * 256; };
  const bool need_carry = plan.segments > 1;
  FwdScratchLayout l;
  l.n_int = 1 + (need_carry ? recs * plan.state_groups : 0);
  l.off_inc = up256(l.n_int * 4);
  l.inc_bytes = need_carry ? up256(recs * N * 64 * 4) : 0;
  l.aggb_bytes = plan.lookback ? up256(recs * N * 64 * 4) : 0;
  l.aggs_bytes = (plan.lookback || (keep_sums && need_carry))
                     ? up256(recs * plan.state_groups * 64 * 4)
                     : 0;
  l.total = l.off_inc + l.inc_bytes + l.aggb_bytes + l.aggs_bytes;
  return l;
}

// out may be NULL only for the backward's own forward pass (no_out), which
// keeps just the checkpoint buffer.
int fwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
             const float* D, const void* z, const float* dt_bias, int softplus, const float* h0,
             int bbar, void* out, float* last_state, float* ckpt, const ssm_dims* dims,
             void* stream, bool no_out = false, bool no_alloc = false,
             float* sum_delta_out = nullptr, void* rec = nullptr) {
  int rc = check_dims(dims);
  if (rc != SSM_OK) return rc;
  if (bbar != SSM_BBAR_DELTA && bbar != SSM_BBAR_ZOH) return SSM_EINVAL;
  // aggregate-only mode (the carry record of a segment): no C, readout or outputs
  const bool agg_only = sum_delta_out != nullptr;
  if (agg_only && (!last_state || out || ckpt || C || D || z || no_out)) return SSM_EINVAL;
  // rec: with agg_only, a buffer that keeps every split segment's carry
  // (records from a zero start only); without, the forward starts every
  // segment from those carries
  const bool from_rec = rec != nullptr && !agg_only;
  if (rec && (!aligned(rec, 256) || no_alloc || ckpt || (agg_only && h0))) return SSM_EINVAL;
  if (!u || !delta || !A || !B || (!C && !agg_only) || (!out && !no_out && !agg_only) ||
      (no_out && !ckpt))
    return SSM_EINVAL;
  const void* ptrs[] = {u, delta, A, B, C, D, z, dt_bias, h0, out, last_state, sum_delta_out};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SSM_EALIGN;
  const void* inputs[] = {u, delta, A, B, C, D, z, dt_bias, h0};
  for (const void* p : inputs)
    if (p && (p == out || p == last_state || p == sum_delta_out)) return SSM_EINVAL;
  if (last_state && last_state == out) return SSM_EINVAL;
  if (sum_delta_out && sum_delta_out == last_state) return SSM_EINVAL;
  if (rec) {
    for (const void* p : ptrs)
      if (p && p == rec) return SSM_EINVAL;
  }

  ssm_fwd_plan plan;
  plan_forward(*dims, &plan);
  const int64_t cblk = div_up(dims->dim, 64);
  const int64_t chains = dims->batch * cblk;
  // carry records of the split chains (whole chains need none)
  const int64_t recs = (chains - plan.whole_chains) * plan.segments;
  if (recs * plan.state_groups > (1LL << 30) || plan.workgroups > (1LL << 31) - 1)
    return SSM_EINVAL;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t N = dims->dstate;
  // scratch: ticket + status (ints), then records (floats), 256-byte aligned pieces
  const FwdScratchLayout lay = fwd_scratch_layout(plan, recs, N, agg_only || rec);
  const int64_t n_int = lay.n_int, off_inc = lay.off_inc, inc_bytes = lay.inc_bytes,
                aggb_bytes = lay.aggb_bytes, total = lay.total;

  // a plan of whole chains only takes no ticket and publishes no carry: no
  // scratch, no clearing launch
  const bool need_scratch = plan.whole_chains < chains;
  char* buf = nullptr;
  if (!need_scratch) {
    // nothing to allocate
  } else if (rec) {
    // the caller's record buffer (ssm_fwd_record_bytes): nothing allocated
    buf = static_cast<char*>(rec);
  } else if (no_alloc) {
    // the static array: nothing is allocated or freed by this call
    if (total > kStaticScratchBytes) return SSM_ESCRATCH;
    void* addr = nullptr;
    rc = static_scratch_address(&addr);
    if (rc != SSM_OK) return rc;
    buf = static_cast<char*>(addr);
  } else {
    if (env_int("SSM_TEST_FAIL_ALLOC", 0) == 1) return SSM_ENOMEM;
    if (hipMallocAsync(reinterpret_cast<void**>(&buf), static_cast<size_t>(total), st) !=
            hipSuccess ||
        !buf)
      return SSM_ENOMEM;
  }

  ssm::FwdScratch sc;
  sc.ticket = need_scratch ? reinterpret_cast<int*>(buf) : nullptr;
  sc.status = need_scratch ? sc.ticket + 1 : nullptr;
  sc.inc = need_scratch ? reinterpret_cast<float*>(buf + off_inc) : nullptr;
  sc.agg_b = need_scratch ? reinterpret_cast<float*>(buf + off_inc + inc_bytes) : nullptr;
  sc.agg_s =
      need_scratch ? reinterpret_cast<float*>(buf + off_inc + inc_bytes + aggb_bytes) : nullptr;
  sc.spin_limit = env_int("SSM_TEST_SPIN_LIMIT", kDefaultSpinLimit);
  sc.ckpt = ckpt;
  sc.ysave = ckpt ? reinterpret_cast<float*>(reinterpret_cast<char*>(ckpt) + ckpt_y_offset(dims))
                  : nullptr;

  ssm::FwdShape sh;
  sh.seqlen = dims->seqlen;
  sh.dim = dims->dim;
  sh.chains = static_cast<int32_t>(chains);
  sh.n_cblk = static_cast<int32_t>(cblk);
  sh.n_full = plan.whole_chains;
  sh.n_seg = plan.segments;
  sh.seg_len = plan.segment_len;
  sh.seg0_len = plan.first_segment_len;
  sh.softplus = softplus ? 1 : 0;
  sh.lookback = plan.lookback;
  sh.has_bias = dt_bias != nullptr;
  sh.has_D = D != nullptr;
  sh.has_z = z != nullptr;
  sh.has_h0 = h0 != nullptr;
  sh.has_last = last_state != nullptr;
  sh.zoh = bbar == SSM_BBAR_ZOH ? 1 : 0;
  sh.mode = agg_only ? ssm::kModeRecord : (from_rec ? ssm::kModeFromRecord : ssm::kModeForward);
  sh.n_ckpt = div_up(dims->seqlen, ssm::kBwdChunk);
  {
    // per-thread runs of the chunk tile: chunk / helper waves consecutive channels
    const int64_t ept = plan.chunk / plan.helper_waves;
    const int64_t esz = dims->dtype == SSM_BF16 ? 2 : 4;
    const uintptr_t need = static_cast<uintptr_t>(ept * esz >= 16 ? 16 : ept * esz);
    bool ok = ept * esz >= 4 && dims->dim % ept == 0;
    const void* acts[] = {u, delta, z, out};
    for (const void* a : acts)
      if (a && !aligned(a, need)) ok = false;
    if (sc.ysave && !aligned(sc.ysave, static_cast<uintptr_t>(ept * 4 >= 16 ? 16 : ept * 4)))
      ok = false;
    sh.vec_io = ok ? 1 : 0;
  }

  ssm::FwdPtrs p{u, delta, A, B, C, D, z, dt_bias, h0, out, last_state, sum_delta_out};

  rc = SSM_OK;
  const bool f32 = dims->dtype == SSM_F32;
  if (need_scratch && !from_rec) {
    const hipError_t ez = f32 ? ssm::fwd_f32::launch_fill_zero(sc.ticket, n_int, st)
                              : ssm::fwd_bf16::launch_fill_zero(sc.ticket, n_int, st);
    if (ez != hipSuccess) rc = SSM_ELAUNCH;
  }
  if (rc == SSM_OK) {
    const hipError_t el =
        f32 ? ssm::fwd_f32::launch_scan_fwd(plan.state_groups, plan.states_per_group, p, sc, sh,
                                            plan.workgroups, st)
            : ssm::fwd_bf16::launch_scan_fwd(plan.state_groups, plan.states_per_group, p, sc,
                                             sh, plan.workgroups, st);
    if (el != hipSuccess) rc = SSM_ELAUNCH;
  }
  if (need_scratch && !no_alloc && !rec && hipFreeAsync(buf, st) != hipSuccess && rc == SSM_OK)
    rc = SSM_ELAUNCH;
  return rc;
}

int state_update_impl(float* state, const void* x, const void* dt, const float* A,
                      const void* B, const void* C, const float* D, const void* z,
                      const float* dt_bias, int softplus, int bbar, void* out,
                      const ssm_dims* dims, void* stream) {
  int rc = check_dims(dims);
  if (rc != SSM_OK) return rc;
  if (bbar != SSM_BBAR_DELTA && bbar != SSM_BBAR_ZOH) return SSM_EINVAL;
  if (dims->seqlen != 1) return SSM_EINVAL;
  if (!state || !x || !dt || !A || !B || !C || !out) return SSM_EINVAL;
  const void* ptrs[] = {state, x, dt, A, B, C, D, z, dt_bias, out};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SSM_EALIGN;
  if (dims->dstate >= 4 && (!aligned(state, 16) || !aligned(A, 16))) return SSM_EALIGN;
  const void* inputs[] = {state, x, dt, A, B, C, D, z, dt_bias};
  for (const void* p : inputs)
    if (p == out) return SSM_EINVAL;
  if (dims->batch * dims->dim * dims->dstate > (1LL << 40)) return SSM_EINVAL;
  if (ssm::launch_state_update(dims->dtype, static_cast<int>(dims->dstate), state, x, dt, A, B,
                               C, D, z, dt_bias, softplus ? 1 : 0, bbar == SSM_BBAR_ZOH ? 1 : 0,
                               out, dims->batch, dims->dim,
                               env_int("SSM_FORCE_DECODE_ROWS", 0),
                               static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSM_ELAUNCH;
  return SSM_OK;
}

// waves per workgroup of the backward kernel for N states (as its dispatch)
int bwd_groups(int64_t n) {
  switch (n) {
    case 8: return 2;
    case 16: return 4;
    case 32:
    case 64: return 8;
    default: return 1;
  }
}

int bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
             const float* D, const void* z, const float* dt_bias, int softplus, const float* h0,
             const void* dout, const float* dlast, const float* ckpt_in, void* du, void* ddelta,
             float* dA, void* dB, void* dC, float* dD, void* dz, float* ddt_bias, float* dh0,
             const ssm_dims* dims, void* stream, int bbar = SSM_BBAR_DELTA) {
  int rc = check_dims(dims);
  if (rc != SSM_OK) return rc;
  if (bbar != SSM_BBAR_DELTA && bbar != SSM_BBAR_ZOH) return SSM_EINVAL;
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
    return SSM_EINVAL;
  if (dz && !z) return SSM_EINVAL;  // no gate, no gate gradient
  const void* ins[] = {u, delta, A, B, C, D, z, dt_bias, h0, dout, dlast, ckpt_in};
  const void* outs[] = {du, ddelta, dA, dB, dC, dD, dz, ddt_bias, dh0};
  for (const void* q : ins)
    if (q && !aligned(q, 4)) return SSM_EALIGN;
  for (const void* q : outs)
    if (q && !aligned(q, 4)) return SSM_EALIGN;
  for (const void* o : outs) {
    if (!o) continue;
    for (const void* i : ins)
      if (i == o) return SSM_EINVAL;
    int same = 0;
    for (const void* o2 : outs) same += (o2 == o);
    if (same > 1) return SSM_EINVAL;
  }

  const int64_t N = dims->dstate;
  const int64_t cblk = div_up(dims->dim, 64);
  const int64_t nck = div_up(dims->seqlen, ssm::kBwdChunk);
  auto up256 = [](int64_t bytes) { return div_up(bytes, 256) * 256; };
  // Plan.  The state at any chunk start is known from the checkpoints, so
  // the chains beyond a multiple of the CU count can be split into segments
  // that exchange only the adjoint carry (reverse look-back), as the forward
  // does.  With at most half as many chains as CUs (K = 0) every chain is
  // split, into enough segments for ~4 workgroups per CU (measured best at
  // the million-token shape: 64, 128, 256 segments per chain took 16.4,
  // 10.4, 9.6 ms; with 192 chains, 130M, splitting measured slower);
  // otherwise the remainder chains get ~one segment per CU (4 of 2, 3, 4, 8,
  // 16 measured best at the 2.8B layer).  Segments are at least 512 steps.
  const int64_t chains = dims->batch * cblk;
  int64_t n_full = chains, n_seg = 1, seg_len = dims->seqlen;
  {
    const int64_t K = (chains / kComputeUnits) * kComputeUnits;
    const int64_t M = chains - K;
    int64_t S = M == 0 ? 1
              : (K == 0 ? (M <= kComputeUnits / 2 ? 4 * kComputeUnits / M : 1)
                        : kComputeUnits / M);
    if (S < 3) S = 1;
    int64_t kf = K;
    const int force_split = env_int("SSM_FORCE_BWD_SPLIT", 0);
    const int force_whole = env_int("SSM_FORCE_BWD_WHOLE", -1);
    if (force_split >= 1) {
      S = force_split;
      kf = force_whole >= 0 && force_whole <= chains ? force_whole : K;
    }
    if (S > 1 && kf < chains) {
      int64_t sl = div_up(div_up(dims->seqlen, S), ssm::kBwdSegQuantum) * ssm::kBwdSegQuantum;
      if (force_split < 1 && sl < 512) sl = 512;
      if (div_up(dims->seqlen, sl) > 1) {
        n_full = kf;
        seg_len = sl;
        n_seg = div_up(dims->seqlen, sl);
      }
    }
  }
  const int64_t recs = (chains - n_full) * n_seg;
  const int64_t groups = bwd_groups(N);
  // without the forward's checkpoint buffer, the backward runs the forward's
  // training mode into scratch first
  const int64_t b_ckpt = ckpt_in ? 0 : up256(ssm_ckpt_bytes(dims));
  const int64_t b_bc = up256(cblk * dims->batch * dims->seqlen * 2 * N * 4);
  const int64_t b_a = up256(dims->batch * n_seg * dims->dim * N * 4);
  const int64_t b_d = up256(dims->batch * n_seg * dims->dim * 4);
  const int64_t n_int = 1 + recs * groups;                    // ticket + status words
  const int64_t b_int = up256(n_int * 4);
  const int64_t b_rec = up256(recs * N * 64 * 4);
  const int64_t b_recs = up256(recs * groups * 64 * 4);
  const int64_t total = b_ckpt + b_bc + b_a + 2 * b_d + b_int + 2 * b_rec + b_recs;
  if (total > (1LL << 40)) return SSM_EINVAL;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (env_int("SSM_TEST_FAIL_ALLOC", 0) == 1) return SSM_ENOMEM;
  char* scratch = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&scratch), static_cast<size_t>(total), st) !=
          hipSuccess ||
      !scratch)
    return SSM_ENOMEM;

  const float* ckpt = ckpt_in ? ckpt_in : reinterpret_cast<const float*>(scratch);
  rc = SSM_OK;
  if (!ckpt_in) {
    rc = fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, bbar, nullptr,
                  nullptr, reinterpret_cast<float*>(scratch), dims, stream, /*no_out=*/true);
  }
  const float* ysave =
      reinterpret_cast<const float*>(reinterpret_cast<const char*>(ckpt) + ckpt_y_offset(dims));

  ssm::BwdPtrs p{u, delta, A, B, C, D, z, dt_bias, h0, dout, dlast, ckpt, ysave, du, ddelta,
                 dA, dB, dC, dD, dz, ddt_bias, dh0, nullptr, nullptr, nullptr, nullptr,
                 nullptr, nullptr, nullptr, nullptr, nullptr};
  p.part_bc = reinterpret_cast<float*>(scratch + b_ckpt);
  p.part_a = reinterpret_cast<float*>(scratch + b_ckpt + b_bc);
  p.part_d = reinterpret_cast<float*>(scratch + b_ckpt + b_bc + b_a);
  p.part_bias = reinterpret_cast<float*>(scratch + b_ckpt + b_bc + b_a + b_d);
  {
    char* q = scratch + b_ckpt + b_bc + b_a + 2 * b_d;
    p.ticket = reinterpret_cast<int*>(q);
    p.status = p.ticket + 1;
    p.inc = reinterpret_cast<float*>(q + b_int);
    p.agg_b = reinterpret_cast<float*>(q + b_int + b_rec);
    p.agg_s = reinterpret_cast<float*>(q + b_int + 2 * b_rec);
  }

  ssm::BwdShape sh;
  sh.batch = dims->batch;
  sh.seqlen = dims->seqlen;
  sh.dim = dims->dim;
  sh.n_cblk = static_cast<int32_t>(cblk);
  sh.chains = static_cast<int32_t>(chains);
  sh.n_full = static_cast<int32_t>(n_full);
  sh.n_seg = static_cast<int32_t>(n_seg);
  sh.seg_len = seg_len;
  sh.spin_limit = env_int("SSM_TEST_SPIN_LIMIT", kDefaultSpinLimit);
  sh.nchunks = nck;
  sh.softplus = softplus ? 1 : 0;
  sh.has_D = D != nullptr;
  sh.has_z = z != nullptr;
  sh.has_bias = dt_bias != nullptr;
  sh.has_h0 = h0 != nullptr;
  sh.has_dlast = dlast != nullptr;
  sh.zoh = bbar == SSM_BBAR_ZOH ? 1 : 0;
  {
    // the helpers' runs of ept = kBwdChunk / 4 channels may move as one
    // vector when every run is whole and aligned (the saved readouts are
    // float32 runs)
    const int64_t ept = ssm::kBwdChunk / 4;
    const int64_t esz = dims->dtype == SSM_BF16 ? 2 : 4;
    const uintptr_t need = static_cast<uintptr_t>(ept * esz >= 16 ? 16 : ept * esz);
    bool ok = ept * esz >= 4 && dims->dim % ept == 0 &&
              aligned(ysave, static_cast<uintptr_t>(ept * 4 >= 16 ? 16 : ept * 4));
    const void* acts[] = {u, delta, z, dout, du, ddelta, dz};
    for (const void* a : acts)
      if (a && !aligned(a, need)) ok = false;
    sh.vec_io = ok ? 1 : 0;
  }

  if (rc == SSM_OK && ssm::launch_scan_bwd(dims->dtype, static_cast<int>(N), p, sh, st) !=
                          hipSuccess)
    rc = SSM_ELAUNCH;
  if (hipFreeAsync(scratch, st) != hipSuccess && rc == SSM_OK) rc = SSM_ELAUNCH;
  return rc;
}

int check_conv(const ssm_dims* dims, int width) {
  if (!dims) return SSM_EINVAL;
  if (dims->dtype != SSM_F32 && dims->dtype != SSM_BF16) return SSM_EDTYPE;
  if (dims->batch <= 0 || dims->seqlen <= 0 || dims->dim <= 0) return SSM_EINVAL;
  if (width < 1 || width > 4) return SSM_EINVAL;
  if (dims->batch * dims->seqlen * dims->dim > (1LL << 46)) return SSM_EINVAL;
  return SSM_OK;
}

int conv_fwd_impl(const void* x, const float* weight, const float* bias, const float* state_in,
                  int width, int silu, void* out, float* state_out, const ssm_dims* dims,
                  void* stream) {
  int rc = check_conv(dims, width);
  if (rc != SSM_OK) return rc;
  if (!x || !weight || !out) return SSM_EINVAL;
  const void* ptrs[] = {x, weight, bias, state_in, out, state_out};
  for (const void* q : ptrs)
    if (q && !aligned(q, 4)) return SSM_EALIGN;
  if (out == x || (state_out && (state_out == state_in || state_out == weight)))
    return SSM_EINVAL;
  ssm::ConvPtrs p{x, weight, bias, state_in, out, state_out, nullptr};
  ssm::ConvShape sh{};
  sh.batch = dims->batch;
  sh.seqlen = dims->seqlen;
  sh.dim = dims->dim;
  sh.silu = silu ? 1 : 0;
  // runs of 4 channels, one vector of 16 (float32) or 8 (bfloat16) bytes
  const uintptr_t run_bytes = dims->dtype == SSM_BF16 ? 8 : 16;
  sh.vec_io = (dims->dim % 4 == 0 && aligned(x, run_bytes) && aligned(out, run_bytes)) ? 1 : 0;
  if (ssm::launch_conv1d_fwd(dims->dtype, width, p, sh, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SSM_ELAUNCH;
  return SSM_OK;
}

int conv_update_impl(float* state, const void* x, const float* weight, const float* bias,
                     int width, int silu, void* out, const ssm_dims* dims, void* stream) {
  int rc = check_conv(dims, width);
  if (rc != SSM_OK) return rc;
  if (dims->seqlen != 1) return SSM_EINVAL;
  if (!x || !weight || !out || (width > 1 && !state)) return SSM_EINVAL;
  const void* ptrs[] = {state, x, weight, bias, out};
  for (const void* q : ptrs)
    if (q && !aligned(q, 4)) return SSM_EALIGN;
  if (out == x || (state && (out == state || state == weight))) return SSM_EINVAL;
  ssm::ConvPtrs p{x, weight, bias, nullptr, out, nullptr, state};
  ssm::ConvShape sh{};
  sh.batch = dims->batch;
  sh.seqlen = 1;
  sh.dim = dims->dim;
  sh.silu = silu ? 1 : 0;
  if (ssm::launch_conv1d_update(dims->dtype, width, p, sh, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SSM_ELAUNCH;
  return SSM_OK;
}

int block_impl(const void* x_in, const mamba_block_weights* w, void* out,
               const mamba_block_dims* bd, void* stream) {
  if (!bd || !w || !x_in || !out) return SSM_EINVAL;
  if (bd->dtype != SSM_F32 && bd->dtype != SSM_BF16) return SSM_EDTYPE;
  if (bd->batch <= 0 || bd->seqlen <= 0 || bd->d_model <= 0 || bd->d_inner <= 0 ||
      bd->dt_rank <= 0 || !valid_dstate(bd->d_state) || bd->conv_width < 1 ||
      bd->conv_width > 4)
    return SSM_EINVAL;
  if (!w->in_x || !w->in_z || !w->conv_w || !w->x_dt || !w->x_B || !w->x_C || !w->dt ||
      !w->A || !w->out)
    return SSM_EINVAL;
  const void* ptrs[] = {x_in, out, w->in_x, w->in_z, w->conv_w, w->conv_b, w->x_dt, w->x_B,
                        w->x_C, w->dt, w->dt_bias, w->A, w->D, w->out};
  for (const void* q : ptrs)
    if (q && !aligned(q, 4)) return SSM_EALIGN;
  if (out == x_in) return SSM_EINVAL;
  const int64_t M = bd->batch * bd->seqlen;
  const int64_t di = bd->d_inner, dm = bd->d_model, n = bd->d_state, r = bd->dt_rank;
  // the GEMM library takes 32-bit sizes
  const int64_t lim = (1LL << 31) - 1;
  if (M > lim || di > lim || dm > lim || M * di > (1LL << 46)) return SSM_EINVAL;

  const int64_t esz = bd->dtype == SSM_BF16 ? 2 : 4;
  auto up256 = [](int64_t bytes) { return div_up(bytes, 256) * 256; };
  // u feeds three projections (the low-rank dt, B, C): one GEMM against the
  // stacked weights [x_dt; x_B; x_C] ([dt_rank + 2 d_state][d_inner]) reads u
  // once (each projection is HBM-bound on u); B and C are then copied out as
  // the scan's contiguous [rows][N] operands.  The stack is the caller's
  // memory when the three weights already lie back to back (the rows of one
  // x_proj weight), else a copy.
  const int64_t nx = r + 2 * n;
  const char* wx_dt = static_cast<const char*>(w->x_dt);
  const bool stacked = static_cast<const char*>(w->x_B) == wx_dt + r * di * esz &&
                       static_cast<const char*>(w->x_C) == wx_dt + (r + n) * di * esz;
  const int64_t b_act = up256(M * di * esz);
  const int64_t b_xo = up256(M * nx * esz);
  const int64_t b_bc = up256(M * n * esz);
  const int64_t b_wx = stacked ? 0 : up256(di * nx * esz);
  const int64_t total = 5 * b_act + b_xo + 2 * b_bc + b_wx;  // x, z, u, dt, y; x_proj; B, C
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (env_int("SSM_TEST_FAIL_ALLOC", 0) == 1) return SSM_ENOMEM;
  char* ws = nullptr;
  if (hipMallocAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(total), st) !=
          hipSuccess ||
      !ws)
    return SSM_ENOMEM;
  char* x = ws;
  char* z = x + b_act;
  char* u = z + b_act;
  char* dt = u + b_act;
  char* y = dt + b_act;
  char* xo = y + b_act;
  char* Bm = xo + b_xo;
  char* Cm = Bm + b_bc;
  char* wx_copy = Cm + b_bc;
  const int dtype = bd->dtype;

  int rc = SSM_OK;
  // C[rows][cols] = a[rows][inner] (leading dimension lda) times the [cols][inner]
  // weight transposed
  auto gemm = [&](int64_t rows, int64_t cols, int64_t inner, const void* a, int64_t lda,
                  const void* wt, void* c) {
    if (rc == SSM_OK &&
        ssm::gemm_linear(dtype, rows, cols, inner, a, lda, wt, inner, c, cols, st) !=
            hipSuccess)
      rc = SSM_ELAUNCH;
  };
  gemm(M, di, dm, x_in, dm, w->in_x, x);
  gemm(M, di, dm, x_in, dm, w->in_z, z);
  if (rc == SSM_OK) {
    ssm_dims cd{bd->batch, bd->seqlen, di, 1, dtype};
    rc = conv_fwd_impl(x, w->conv_w, w->conv_b, nullptr, bd->conv_width, 1, u, nullptr, &cd,
                       stream);
  }
  auto copy = [&](void* dst, const void* src, int64_t bytes) {
    if (rc == SSM_OK && hipMemcpyAsync(dst, src, static_cast<size_t>(bytes),
                                       hipMemcpyDeviceToDevice, st) != hipSuccess)
      rc = SSM_ELAUNCH;
  };
  auto copy2d = [&](void* dst, int64_t dpitch, const void* src, int64_t spitch, int64_t width,
                    int64_t height) {
    if (rc == SSM_OK &&
        hipMemcpy2DAsync(dst, static_cast<size_t>(dpitch), src, static_cast<size_t>(spitch),
                         static_cast<size_t>(width), static_cast<size_t>(height),
                         hipMemcpyDeviceToDevice, st) != hipSuccess)
      rc = SSM_ELAUNCH;
  };
  const void* wx = w->x_dt;
  if (!stacked) {
    copy(wx_copy, w->x_dt, r * di * esz);
    copy(wx_copy + r * di * esz, w->x_B, n * di * esz);
    copy(wx_copy + (r + n) * di * esz, w->x_C, n * di * esz);
    wx = wx_copy;
  }
  gemm(M, nx, di, u, di, wx, xo);
  copy2d(Bm, n * esz, xo + r * esz, nx * esz, n * esz, M);
  copy2d(Cm, n * esz, xo + (r + n) * esz, nx * esz, n * esz, M);
  // dt = dt_low dt^T with dt_low the first r columns of the x_proj output
  gemm(M, di, r, xo, nx, w->dt, dt);
  if (rc == SSM_OK) {
    ssm_dims sd{bd->batch, bd->seqlen, di, n, dtype};
    rc = fwd_impl(u, dt, w->A, Bm, Cm, w->D, z, w->dt_bias, 1, nullptr, SSM_BBAR_DELTA, y,
                  nullptr, nullptr, &sd, stream);
  }
  gemm(M, dm, di, y, di, w->out, out);
  if (hipFreeAsync(ws, st) != hipSuccess && rc == SSM_OK) rc = SSM_ELAUNCH;
  return rc;
}

}  // namespace

extern "C" {

int selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* dt_bias,
                       int softplus, void* out, float* last_state, const ssm_dims* dims,
                       void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, nullptr, SSM_BBAR_DELTA, out,
                  last_state, nullptr, dims, stream);
}

int selective_scan_fwd_h0(const void* u, const void* delta, const float* A, const void* B,
                          const void* C, const float* D, const void* z, const float* dt_bias,
                          int softplus, const float* h0, void* out, float* last_state,
                          const ssm_dims* dims, void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, SSM_BBAR_DELTA, out,
                  last_state, nullptr, dims, stream);
}

int selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A,
                               const void* B, const void* C, const float* D, const void* z,
                               const float* dt_bias, int softplus, const float* h0, void* out,
                               float* last_state, const ssm_dims* dims, void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, SSM_BBAR_DELTA, out,
                  last_state, nullptr, dims, stream, /*no_out=*/false, /*no_alloc=*/true);
}

int selective_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                          const void* C, const float* D, const void* z, const float* dt_bias,
                          int softplus, const float* h0, int bbar, void* out,
                          float* last_state, const ssm_dims* dims, void* stream) {
  return fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, bbar, out, last_state,
                  nullptr, dims, stream);
}

int selective_scan_fwd_train_ex(const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* dt_bias, int softplus, const float* h0, int bbar,
                                void* out, float* last_state, float* ckpt,
                                const ssm_dims* dims, void* stream) {
  if (!ckpt) return SSM_EINVAL;
  if (!aligned(ckpt, 4)) return SSM_EALIGN;
  const void* others[] = {u, delta, A, B, C, D, z, dt_bias, h0, out, last_state};
  for (const void* q : others)
    if (q && q == ckpt) return SSM_EINVAL;
  return fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, bbar, out, last_state, ckpt,
                  dims, stream);
}

int selective_scan_fwd_train(const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* dt_bias, int softplus, const float* h0, void* out,
                             float* last_state, float* ckpt, const ssm_dims* dims,
                             void* stream) {
  return selective_scan_fwd_train_ex(u, delta, A, B, C, D, z, dt_bias, softplus, h0,
                                     SSM_BBAR_DELTA, out, last_state, ckpt, dims, stream);
}

int selective_scan_fwd_aggregate(const void* u, const void* delta, const float* A,
                                 const void* B, const float* dt_bias, int softplus,
                                 const float* h0, int bbar, float* sum_delta, float* state,
                                 const ssm_dims* dims, void* stream) {
  if (!sum_delta || !state) return SSM_EINVAL;
  return fwd_impl(u, delta, A, B, nullptr, nullptr, nullptr, dt_bias, softplus, h0, bbar,
                  nullptr, state, nullptr, dims, stream, /*no_out=*/false, /*no_alloc=*/false,
                  sum_delta);
}

int64_t ssm_fwd_record_bytes(const ssm_dims* dims) {
  const int rc = check_dims(dims);
  if (rc != SSM_OK) return rc;
  ssm_fwd_plan plan;
  plan_forward(*dims, &plan);
  const int64_t chains = dims->batch * div_up(dims->dim, 64);
  const int64_t recs = (chains - plan.whole_chains) * plan.segments;
  return fwd_scratch_layout(plan, recs, dims->dstate, true).total;
}

int selective_scan_fwd_aggregate_rec(const void* u, const void* delta, const float* A,
                                     const void* B, const float* dt_bias, int softplus,
                                     int bbar, float* sum_delta, float* state, void* rec,
                                     const ssm_dims* dims, void* stream) {
  if (!sum_delta || !state || !rec) return SSM_EINVAL;
  return fwd_impl(u, delta, A, B, nullptr, nullptr, nullptr, dt_bias, softplus, nullptr, bbar,
                  nullptr, state, nullptr, dims, stream, /*no_out=*/false, /*no_alloc=*/false,
                  sum_delta, rec);
}

int selective_scan_fwd_from_rec(const void* u, const void* delta, const float* A, const void* B,
                                const void* C, const float* D, const void* z,
                                const float* dt_bias, int softplus, const float* h0, int bbar,
                                const void* rec, void* out, float* last_state,
                                const ssm_dims* dims, void* stream) {
  if (!rec) return SSM_EINVAL;
  return fwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, bbar, out, last_state,
                  nullptr, dims, stream, /*no_out=*/false, /*no_alloc=*/false, nullptr,
                  const_cast<void*>(rec));
}

int selective_scan_carry_combine(const float* sum_delta, const float* agg, const float* A,
                                 const float* h0, float* h_in, float* h_out, int64_t segments,
                                 const ssm_dims* dims, void* stream) {
  if (!dims) return SSM_EINVAL;
  ssm_dims d1 = *dims;
  d1.seqlen = 1;  // the sequence length plays no part here
  d1.dtype = SSM_F32;
  const int rc = check_dims(&d1);
  if (rc != SSM_OK) return rc;
  if (segments < 1 || segments > (1LL << 31) - 1) return SSM_EINVAL;
  if (div_up(d1.batch * d1.dim * d1.dstate, 256) > (1LL << 31) - 1) return SSM_EINVAL;
  if (!sum_delta || !agg || !A || !h_in) return SSM_EINVAL;
  const void* ptrs[] = {sum_delta, agg, A, h0, h_in, h_out};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SSM_EALIGN;
  const void* inputs[] = {sum_delta, agg, A, h0};
  for (const void* p : inputs)
    if (p && (p == h_in || p == h_out)) return SSM_EINVAL;
  if (h_out && h_out == h_in) return SSM_EINVAL;
  const hipError_t e = ssm::launch_carry_combine(sum_delta, agg, A, h0, h_in, h_out, segments,
                                                 d1.batch, d1.dim, static_cast<int>(d1.dstate),
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SSM_OK : SSM_ELAUNCH;
}

int64_t ssm_ckpt_bytes(const ssm_dims* dims) {
  const int rc = check_dims(dims);
  if (rc != SSM_OK) return rc;
  return ckpt_y_offset(dims) + dims->batch * dims->seqlen * dims->dim * 4;
}

int selective_state_update(float* state, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* dt_bias, int softplus, void* out, const ssm_dims* dims,
                           void* stream) {
  return state_update_impl(state, x, dt, A, B, C, D, z, dt_bias, softplus, SSM_BBAR_DELTA, out,
                           dims, stream);
}

int selective_state_update_ex(float* state, const void* x, const void* dt, const float* A,
                              const void* B, const void* C, const float* D, const void* z,
                              const float* dt_bias, int softplus, int bbar, void* out,
                              const ssm_dims* dims, void* stream) {
  return state_update_impl(state, x, dt, A, B, C, D, z, dt_bias, softplus, bbar, out, dims,
                           stream);
}

int selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* dt_bias,
                       int softplus, const float* h0, const void* dout, const float* dlast,
                       void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD,
                       void* dz, float* ddt_bias, float* dh0, const ssm_dims* dims,
                       void* stream) {
  return bwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, dout, dlast, nullptr, du,
                  ddelta, dA, dB, dC, dD, dz, ddt_bias, dh0, dims, stream);
}

int selective_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z, const float* dt_bias,
                            int softplus, const float* h0, const void* dout, const float* dlast,
                            const float* ckpt, void* du, void* ddelta, float* dA, void* dB,
                            void* dC, float* dD, void* dz, float* ddt_bias, float* dh0,
                            const ssm_dims* dims, void* stream) {
  if (!ckpt) return SSM_EINVAL;
  return bwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, dout, dlast, ckpt, du, ddelta,
                  dA, dB, dC, dD, dz, ddt_bias, dh0, dims, stream);
}

int selective_scan_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                          const void* C, const float* D, const void* z, const float* dt_bias,
                          int softplus, const float* h0, int bbar, const void* dout,
                          const float* dlast, const float* ckpt, void* du, void* ddelta,
                          float* dA, void* dB, void* dC, float* dD, void* dz, float* ddt_bias,
                          float* dh0, const ssm_dims* dims, void* stream) {
  return bwd_impl(u, delta, A, B, C, D, z, dt_bias, softplus, h0, dout, dlast, ckpt, du, ddelta,
                  dA, dB, dC, dD, dz, ddt_bias, dh0, dims, stream, bbar);
}

int causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                      const float* state_in, int width, int silu, void* out, float* state_out,
                      const ssm_dims* dims, void* stream) {
  return conv_fwd_impl(x, weight, bias, state_in, width, silu, out, state_out, dims, stream);
}

int causal_conv1d_update(float* state, const void* x, const float* weight, const float* bias,
                         int width, int silu, void* out, const ssm_dims* dims, void* stream) {
  return conv_update_impl(state, x, weight, bias, width, silu, out, dims, stream);
}

int mamba_block_fwd(const void* x_in, const mamba_block_weights* weights, void* out,
                    const mamba_block_dims* dims, void* stream) {
  return block_impl(x_in, weights, out, dims, stream);
}

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "SSM_OK: success";
    case SSM_EINVAL: return "SSM_EINVAL: invalid argument (dimension, null pointer or aliasing)";
    case SSM_EDTYPE: return "SSM_EDTYPE: unsupported dtype";
    case SSM_EALIGN: return "SSM_EALIGN: misaligned pointer";
    case SSM_ENOMEM: return "SSM_ENOMEM: scratch allocation failed";
    case SSM_ELAUNCH: return "SSM_ELAUNCH: kernel launch failed";
    case SSM_ETIMEOUT: return "SSM_ETIMEOUT: a segment carry wait hit its bound";
    case SSM_ESCRATCH:
      return "SSM_ESCRATCH: the call needs more carry scratch than the allocation-free "
             "entry point's static array holds (32 MiB)";
    default: return "SSM_UNKNOWN: unknown status code";
  }
}

int ssm_check_device_errors(void* stream) {
  unsigned c32 = 0, c16 = 0, cb = 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (ssm::fwd_f32::read_and_clear_errors(st, &c32) != hipSuccess ||
      ssm::fwd_bf16::read_and_clear_errors(st, &c16) != hipSuccess ||
      ssm::read_and_clear_bwd_errors(st, &cb) != hipSuccess)
    return SSM_ELAUNCH;
  return (c32 || c16 || cb) ? SSM_ETIMEOUT : SSM_OK;
}

int ssm_fwd_plan_for(const ssm_dims* dims, ssm_fwd_plan* plan) {
  const int rc = check_dims(dims);
  if (rc != SSM_OK) return rc;
  if (!plan) return SSM_EINVAL;
  plan_forward(*dims, plan);
  return SSM_OK;
}

}  // extern "C"
