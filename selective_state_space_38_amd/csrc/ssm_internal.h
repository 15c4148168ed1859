// Internal launch interfaces between the C ABI layer (api.hip) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Steps per chunk of the backward's reverse phase: one checkpoint (the state
// before the chunk) per kBwdChunk steps; the chunk's states and decays are
// recomputed into registers.  The forward's training mode writes the same
// checkpoints.
constexpr int kBwdChunk = 8;

// Carry records exchanged between sequence segments of one channel block.
// Only split chains (chain >= n_full) have records: a record is indexed by
// rec = (chain - n_full) * n_seg + seg, and split per state group (one wave
// per group), so every wave publishes and consumes its own part.
struct FwdScratch {
  int* ticket;       // [1] work-order counter (zeroed before launch)
  int* status;       // [recs][groups] 0 empty, 1 aggregate, 2 inclusive
  float* inc;        // [recs][N][64] state at the end of the segment
  float* agg_b;      // [recs][N][64] segment's own final state from zero (look-back only)
  float* agg_s;      // [recs][groups][64] segment's sum of Delta (look-back only)
  int spin_limit;    // bound on each carry wait (iterations of s_sleep)
  float* ckpt;       // nullable: [chains][n_ckpt][N][64] state before every
                     // kBwdChunk-th step, for the backward (training mode)
  float* ysave;      // nullable: [batch][L][D] readout before the gate (y = C.h +
                     // D u), for the backward (training mode)
};

struct FwdShape {
  int64_t seqlen;
  int64_t dim;
  int32_t chains;    // batch * channel blocks
  int32_t n_cblk;    // channel blocks of 64
  int32_t n_full;    // chains 0 .. n_full-1 run whole; the others are split
  int32_t n_seg;     // sequence segments per split chain
  int32_t seg_len;   // timesteps per segment of a split chain (multiple of the chunk)
  int32_t seg0_len;  // timesteps of a split chain's first segment (multiple of the chunk)
  int32_t softplus;
  int32_t lookback;  // 1: decoupled look-back over aggregates, 0: chained
  int32_t has_bias, has_D, has_z, has_h0, has_last;
  int32_t vec_io;    // activation rows may be moved in aligned vector runs
  int32_t zoh;       // 1: exact zero-order-hold input term, 0: Delta * B
  int32_t mode;      // kModeForward, kModeRecord or kModeFromRecord
  int64_t n_ckpt;    // ceil(seqlen / kBwdChunk): checkpoints per chain
};

// Forward launch modes: the forward; the carry record only (sum of Delta
// and end state, no outputs; it also leaves every split segment's carry in
// its scratch); the outputs from the carries a record launch left (every
// segment starts at once, none waits, none runs an aggregate pass).
enum : int { kModeForward = 0, kModeRecord = 1, kModeFromRecord = 2 };
struct FwdPtrs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  const float* h0;
  void* out;
  float* last_state;
  float* sum_delta;  // [batch][dim], written in aggregate-only mode
};

// Forward workgroup shape: `groups` scan waves (one per state group) plus
// helper waves that stage the chunk tiles and finish the outputs.  Chunk
// length (timesteps staged through LDS per iteration): 32 for one or two
// state groups, 16 from four on, where two workgroups must fit a CU's LDS
// (the tiles and the partial readouts of every group are double buffered).
// Segments are a multiple of the instance's chunk.
constexpr int chunk_for_groups(int groups) { return groups >= 4 ? 16 : 32; }
// Helpers: eight where the chunk is 16 and a scan wave holds at most four
// states (each helper thread then owns a run of two channels of one tile
// row), so the helpers' part of every iteration is short; at d_state 16 two
// 12-wave workgroups still fit a CU's registers.  Measured warm: d_state 16
// at 1536 and 5120 channels 2.0% and 0.6% faster than with four, d_state 32
// 0.8%.  Four otherwise: d_state 64 with eight states a wave measured 1.9%
// slower with eight, and a lone 16-state group spills.
constexpr int helper_waves(int groups, int per_group) {
  return groups >= 4 && per_group <= 4 ? 8 : 4;
}

// The forward is built once per activation type; each build lives in its own
// namespace (fwd_f32, fwd_bf16) with the same interface:
//   launch_scan_fwd   the kernel instance for (groups, states/group), or
//                     hipErrorInvalidValue for an unsupported combination;
//   launch_fill_zero  zeroes the ticket/status words before a launch;
//   read_and_clear_errors  reads and clears that build's count of carry
//                     waits that timed out (synchronises the stream first).
#define SSM_DECLARE_FWD(NS)                                                           \
  namespace NS {                                                                      \
  hipError_t launch_scan_fwd(int groups, int per_group, const FwdPtrs& p,             \
                             const FwdScratch& s, const FwdShape& sh,                 \
                             int64_t workgroups, hipStream_t stream);                 \
  hipError_t launch_fill_zero(int* p, int64_t n, hipStream_t stream);                 \
  hipError_t read_and_clear_errors(hipStream_t stream, unsigned* count);              \
  }
SSM_DECLARE_FWD(fwd_f32)
SSM_DECLARE_FWD(fwd_bf16)
#undef SSM_DECLARE_FWD

// Start state of every one of `segments` consecutive sequence segments from
// their carry records (sum of Delta [S][batch][dim], state from zero
// [S][batch][dim][n]), folded in order from h0 (nullable = zeros); h_out
// (nullable) receives the state after the last segment.
hipError_t launch_carry_combine(const float* sum_delta, const float* agg, const float* A,
                                const float* h0, float* h_in, float* h_out, int64_t segments,
                                int64_t batch, int64_t dim, int n, hipStream_t stream);
// rows_override (1, 2, 4 or 8) fixes the batch rows each workgroup walks
// (tuning); otherwise one row per workgroup.
hipError_t launch_state_update(int dtype, int dstate, float* state,
                               const void* x, const void* dt, const float* A,
                               const void* B, const void* C, const float* D,
                               const void* z, const float* dt_bias,
                               int softplus, int zoh, void* out, int64_t batch,
                               int64_t dim, int rows_override, hipStream_t stream);

// Backward: inputs, outputs and scratch of one call.  Activations and their
// gradients (u, delta, z, dout, du, ddelta, dz, B, C, dB, dC) are of the call's
// dtype; everything else is float32.  Nullable: D, z, dt_bias, h0, dlast
// (inputs) and dD, dz, ddt_bias, dh0 (outputs).
struct BwdPtrs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  const float* h0;
  const void* dout;
  const float* dlast;
  // written by the forward's training mode on the same inputs
  const float* ckpt;   // [batch * channel blocks][chunks][N][64] chunk-start states
  const float* ysave;  // [batch][L][D] readout before the gate
  void* du;
  void* ddelta;
  float* dA;
  void* dB;
  void* dC;
  float* dD;
  void* dz;
  float* ddt_bias;
  float* dh0;
  // scratch
  float* part_bc;    // [channel blocks][batch][L][2N] per-block dB | dC rows
  float* part_a;     // [batch][n_seg][dim][N] per-(batch, segment) dA
  float* part_d;     // [batch][n_seg][dim] per-(batch, segment) dD
  float* part_bias;  // [batch][n_seg][dim] per-(batch, segment) ddt_bias
  // adjoint carries between the segments of split chains (reverse look-back)
  int* ticket;       // [1] work-order counter (zeroed before launch)
  int* status;       // [recs][groups] 0 empty, 1 aggregate, 2 inclusive
  float* inc;        // [recs][N][64] adjoint carried out of the segment's start
  float* agg_b;      // [recs][N][64] the same from a zero carry-in
  float* agg_s;      // [recs][groups][64] segment's sum of Delta
};

struct BwdShape {
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int32_t n_cblk;    // channel blocks of 64
  int32_t chains;    // batch * channel blocks
  int32_t n_full;    // chains 0 .. n_full-1 run whole (workgroup = chain)
  int32_t n_seg;     // segments per split chain (1: no split)
  int64_t seg_len;   // steps per segment of a split chain (multiple of kBwdSegQuantum)
  int32_t spin_limit;  // bound on each carry wait
  int64_t nchunks;   // ceil(seqlen / kBwdChunk)
  int32_t softplus;
  int32_t has_D, has_z, has_bias, has_h0, has_dlast;
  int32_t vec_io;    // the helpers' runs (kBwdChunk / 4 channels) may be vector moves
  int32_t zoh;       // 1: the exact zero-order-hold input term, 0: Delta * B
};

// Segment lengths of the backward's split chains are multiples of this.
constexpr int kBwdSegQuantum = 32;

// Launches the backward kernel for (dtype, N) and the reductions over channel
// blocks and batch.  Returns hipErrorInvalidValue for an unsupported N.
hipError_t launch_scan_bwd(int dtype, int dstate, const BwdPtrs& p, const BwdShape& sh,
                           hipStream_t stream);

// Reads and clears the backward's count of adjoint-carry waits that timed
// out (synchronises the stream first).
hipError_t read_and_clear_bwd_errors(hipStream_t stream, unsigned* count);


// Causal depthwise conv1d (+ SiLU): forward over a sequence and the decode
// step.  x and out are of the call's dtype; weight [dim][K], bias [dim] and
// the states [batch][dim][K-1] (oldest input first) are float32.
struct ConvPtrs {
  const void* x;
  const float* weight;
  const float* bias;        // nullable
  const float* state_in;    // forward: inputs before t = 0 (nullable = zeros)
  void* out;
  float* state_out;         // forward: last K-1 inputs (nullable)
  float* state_inout;       // decode: rolling state, updated in place
};

struct ConvShape {
  int64_t batch;
  int64_t seqlen;
  int64_t dim;
  int64_t runs;             // runs of 4 channels (set by the launcher)
  int64_t tiles;            // time tiles of the activation type's tile length (launcher)
  int32_t silu;
  int32_t vec_io;           // rows of x / out may be moved in aligned 4-channel runs
};

hipError_t launch_conv1d_fwd(int dtype, int width, const ConvPtrs& p, const ConvShape& sh,
                             hipStream_t stream);
hipError_t launch_conv1d_update(int dtype, int width, const ConvPtrs& p, const ConvShape& sh,
                                hipStream_t stream);

// Row-major C[M][N] = A[M][K] W^T with W stored [N][K] (a linear layer's
// weight; leading dimensions in elements) on hipBLASLt, float32
// accumulation; dtype 0 = float32, 1 = bfloat16 storage.
hipError_t gemm_linear(int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                       int64_t lda, const void* W, int64_t ldw, void* C, int64_t ldc,
                       hipStream_t stream);

}  // namespace ssm
