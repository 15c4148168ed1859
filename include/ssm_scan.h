/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan library.
 *
 * Operations (pages cited by title and section):
 *   selective_scan_fwd     Selective state-space (S6) forward over a sequence:
 *                          Delta = softplus(dt + dt_bias), Abar = exp(Delta*A),
 *                          Bbar*x = Delta*B*x, h_t = Abar_t*h_{t-1} + Bbar_t*x_t,
 *                          y_t = C_t . h_t + D*x_t, out = y * SiLU(z).
 *                          "Mamba: Linear-Time Sequence Modeling with Selective
 *                          State Spaces" (reading guide), sections Method and
 *                          Selection mechanism (S6); "Mamba / MambaMini" Steps 1-4
 *                          (pair operator, prefix scan, h_{-1} = 0) and Q&A
 *                          (Delta*B, SiLU gate); CSDN "Mamba" section 3(1) (D).
 *   selective_scan_fwd_h0  The same with a caller-given initial state h_{-1}
 *                          ("Mamba / MambaMini" Step 4: h_t = A_cum_t*h_{-1} +
 *                          B_cum_t), so a sequence can be processed in pieces.
 *   selective_state_update One decode step of the same recurrence on a stored
 *                          state (reading guide FAQ: fixed D x N state per
 *                          layer, constant time per token, no KV cache).
 *   selective_scan_fwd_ex, selective_state_update_ex
 *                          The same operations with a choice of input
 *                          discretisation: Delta*B (as above) or the exact
 *                          zero-order hold of the reading guide's Method,
 *                          Bbar = (Delta A)^-1 (exp(Delta A) - 1) Delta B,
 *                          which for the diagonal A is (exp(Delta A) - 1)/A * B
 *                          (limit Delta*B where A = 0).
 *   selective_scan_fwd_aggregate, selective_scan_carry_combine
 *                          A segment's carry record (sum of Delta, state
 *                          reached) and the fold of consecutive segments'
 *                          records into their start states ("Mamba /
 *                          MambaMini" Steps 2-4): a sequence scanned in
 *                          independent pieces (with _aggregate_rec /
 *                          _from_rec, the pieces' inner carries kept).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps none of them after returning.  Calls are asynchronous on `stream`
 *     (a hipStream_t; NULL means the null stream): buffers must stay valid
 *     until the stream's work has finished.
 *   - Layouts are contiguous row-major in the index order written in the
 *     comments; there is no stride support.
 *   - dtype (dims->dtype) is the storage type of the activations u/x, delta/dt,
 *     z, B, C and out: SSM_F32 or SSM_BF16.  A, D, dt_bias, h0, state and
 *     last_state are always float32.  Arithmetic and accumulation are float32;
 *     bfloat16 outputs are rounded to nearest even.
 *   - Nullable arguments: D (treated as 0), z (no gate), dt_bias (0),
 *     h0 (zeros), last_state (not written).
 *   - Errors are reported only through the return value (an ssm_status);
 *     nothing is printed and nothing is thrown.  Argument validation happens
 *     on the host before any HIP call: dims must be > 0, dim at most 2^24
 *     (the kernels address a chunk's rows with 32-bit offsets), dstate must
 *     be one of 1, 2, 4, 8, 16, 32, 64, required pointers non-null, pointers 4-byte
 *     aligned, `out` must not alias an input.  A failed launch returns
 *     SSM_ELAUNCH; faults inside a kernel surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - Entry points that need scratch (carries between sequence segments,
 *     checkpoints, partial sums, the block's intermediates) allocate it
 *     stream-ordered (hipMallocAsync) and free it on the same stream;
 *     failure returns SSM_ENOMEM.  A forward whose launch plan runs every
 *     (batch row, channel block) as one whole chain needs none and
 *     allocates nothing.  The only other state is a per-device count
 *     of timed-out carry waits (read by ssm_check_device_errors) and, for
 *     mamba_block_fwd, one hipBLASLt handle per host thread and device, so
 *     calls on different streams or host threads may run concurrently.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_EINVAL = -1,   /* bad dimension, null required pointer, aliasing */
  SSM_EDTYPE = -2,   /* dims->dtype is not an ssm_dtype */
  SSM_EALIGN = -3,   /* a pointer is not 4-byte aligned */
  SSM_ENOMEM = -4,   /* scratch allocation failed */
  SSM_ELAUNCH = -5,  /* the HIP runtime rejected a launch */
  SSM_ETIMEOUT = -6, /* a carry wait exceeded its bound (see ssm_check_device_errors) */
  SSM_ESCRATCH = -7  /* selective_scan_fwd_noalloc: the call needs more carry scratch than
                        its static array holds */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

/* Input discretisation Bbar of the _ex entry points. */
typedef enum {
  SSM_BBAR_DELTA = 0,  /* Bbar = Delta * B */
  SSM_BBAR_ZOH = 1     /* Bbar = (exp(Delta A) - 1) / A * B, Delta * B where A = 0 */
} ssm_bbar;

typedef struct {
  int64_t batch;   /* B */
  int64_t seqlen;  /* L (must be 1 for selective_state_update) */
  int64_t dim;     /* D, the number of channels (d_inner) */
  int64_t dstate;  /* N, the state size per channel (d_state) */
  int32_t dtype;   /* ssm_dtype of the activations */
} ssm_dims;

/*
 * Forward selective scan.
 *   u, delta, z : [B][L][D] of dtype      (delta holds the raw dt)
 *   A           : [D][N] float32
 *   B, C        : [B][L][N] of dtype
 *   D, dt_bias  : [D] float32 (nullable)
 *   softplus    : nonzero -> Delta = softplus(delta + dt_bias),
 *                 zero    -> Delta = delta + dt_bias
 *   out         : [B][L][D] of dtype, written
 *   last_state  : [B][D][N] float32 (nullable), the state after step L-1
 * Returns an ssm_status.
 */
int selective_scan_fwd(const void* u, const void* delta, const float* A,
                       const void* B, const void* C, const float* D,
                       const void* z, const float* dt_bias, int softplus,
                       void* out, float* last_state, const ssm_dims* dims,
                       void* stream);

/*
 * As selective_scan_fwd, starting from h0 : [B][D][N] float32 (nullable =
 * zeros).  selective_scan_fwd(...) == selective_scan_fwd_h0(..., NULL, ...).
 */
int selective_scan_fwd_h0(const void* u, const void* delta, const float* A,
                          const void* B, const void* C, const float* D,
                          const void* z, const float* dt_bias, int softplus,
                          const float* h0, void* out, float* last_state,
                          const ssm_dims* dims, void* stream);

/*
 * As selective_scan_fwd_h0, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The call allocates and frees nothing (no hipMalloc, hipFree or
 * allocating library routine): its carry scratch (the work-order ticket,
 * status words and segment carry records) lives in a static device array of
 * 32 MiB that each GPU the library runs on holds until the process ends.
 * The first call on a device looks up that device's copy of the array; the
 * array's words that must start at zero are cleared by a fill kernel on
 * `stream` at every call.
 *   - A call whose launch plan needs more than 32 MiB of carry scratch
 *     returns SSM_ESCRATCH before any HIP call (plans with few segment
 *     carries need almost none: the 2.8B-shaped layer ~2.4 MB, the
 *     million-token sequence ~4.5 MB at d_state 16).
 *   - Every call on one GPU shares that GPU's array and the array keeps the
 *     last call's contents: calls that overlap on one GPU (different
 *     streams or host threads without ordering between them) race on it and
 *     give wrong results.  Calls ordered on one stream are safe.
 * Arguments, layouts, results and the other errors as selective_scan_fwd_h0.
 */
int selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A,
                               const void* B, const void* C, const float* D,
                               const void* z, const float* dt_bias, int softplus,
                               const float* h0, void* out, float* last_state,
                               const ssm_dims* dims, void* stream);

/*
 * As selective_scan_fwd_h0 with the input discretisation `bbar` (an
 * ssm_bbar; any other value returns SSM_EINVAL).  With SSM_BBAR_DELTA it is
 * selective_scan_fwd_h0 exactly.  With SSM_BBAR_ZOH the per-state input
 * coefficient (exp(Delta A) - 1)/A is evaluated without cancellation near
 * Delta A = 0 (a series there), at roughly 2.5x the arithmetic of Delta*B.
 */
int selective_scan_fwd_ex(const void* u, const void* delta, const float* A,
                          const void* B, const void* C, const float* D,
                          const void* z, const float* dt_bias, int softplus,
                          const float* h0, int bbar, void* out,
                          float* last_state, const ssm_dims* dims,
                          void* stream);

/*
 * Carry record of a sequence segment: the forward's recurrence over the
 * segment without its readout ("Mamba / MambaMini" Steps 2-4: a segment's
 * steps compose under the pair operator into one transform (A_cum, B_cum);
 * A being time-invariant, A_cum = exp(A * sum_t Delta_t), so the record is the
 * sum of Delta per (batch, channel) plus the state reached).  This is the
 * first pass of a sequence split into segments (or across devices): scan every
 * segment from a zero state, combine the records (selective_scan_carry_combine),
 * then produce each segment's outputs from its true start state
 * (selective_scan_fwd_h0 / _ex with h0).  It reads only u, delta and B.
 *   u, delta, B, A, dt_bias, softplus, bbar : as selective_scan_fwd_ex
 *   h0         : [B][D][N] float32 start state (nullable = zeros, which gives
 *                the segment's B_cum)
 *   sum_delta  : [B][D] float32, written: sum over the L steps of Delta
 *   state      : [B][D][N] float32, written: the state after step L-1
 *                (equal, up to rounding order, to selective_scan_fwd_ex's
 *                last_state on the same inputs)
 * sum_delta and state are required and must not alias each other or an
 * input (SSM_EINVAL).  Scratch, stream ordering and carry-wait bounds as
 * selective_scan_fwd (long sequences are split into concurrently scanned
 * pieces internally).
 */
int selective_scan_fwd_aggregate(const void* u, const void* delta, const float* A,
                                 const void* B, const float* dt_bias, int softplus,
                                 const float* h0, int bbar, float* sum_delta,
                                 float* state, const ssm_dims* dims, void* stream);

/*
 * A piece's carry record that also keeps the carries inside the piece, and
 * the piece's forward from them.  Long pieces are scanned internally as
 * concurrent segments; the forward over a piece then repeats the segments'
 * aggregate passes that the record call already made.  With a record buffer:
 *   ssm_fwd_record_bytes(dims)       bytes of the buffer for dims (a negative
 *                                    ssm_status if dims are invalid)
 *   selective_scan_fwd_aggregate_rec as selective_scan_fwd_aggregate with
 *                                    h0 = NULL, and writes `rec`: every inner
 *                                    segment's end state from a zero start and
 *                                    its sum of Delta
 *   selective_scan_fwd_from_rec      as selective_scan_fwd_ex (from h0,
 *                                    nullable = zeros), reading `rec` from a
 *                                    selective_scan_fwd_aggregate_rec call on
 *                                    the same u, delta, A, B, dt_bias,
 *                                    softplus, bbar and dims: each inner
 *                                    segment starts at exp(A * sum of Delta
 *                                    before it) * h0 + its kept start state,
 *                                    so no segment waits for another or runs
 *                                    an aggregate pass.
 * rec is a device buffer owned by the caller, 256-byte aligned (SSM_EINVAL
 * otherwise), not aliasing any other argument; its layout is internal.  The
 * two calls must see the same launch plan (the same dims).
 */
int64_t ssm_fwd_record_bytes(const ssm_dims* dims);

int selective_scan_fwd_aggregate_rec(const void* u, const void* delta, const float* A,
                                     const void* B, const float* dt_bias, int softplus,
                                     int bbar, float* sum_delta, float* state,
                                     void* rec, const ssm_dims* dims, void* stream);

int selective_scan_fwd_from_rec(const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D,
                                const void* z, const float* dt_bias, int softplus,
                                const float* h0, int bbar, const void* rec,
                                void* out, float* last_state,
                                const ssm_dims* dims, void* stream);

/*
 * Start states of S consecutive sequence segments from their carry records
 * (selective_scan_fwd_aggregate with h0 = NULL on each segment): h_in[0] = h0
 * (zeros when NULL) and h_in[s+1] = exp(A * sum_delta[s]) * h_in[s] + agg[s],
 * the exclusive prefix of the pair operator over the segment index
 * ("Mamba / MambaMini" Steps 2 and 4), folded in segment order.
 *   sum_delta : [S][B][D] float32;  agg : [S][B][D][N] float32
 *   A         : [D][N] float32;     h0  : [B][D][N] float32 (nullable)
 *   h_in      : [S][B][D][N] float32, written (required)
 *   h_out     : [B][D][N] float32, written when non-NULL: the state after
 *               the last segment
 *   segments  : S >= 1.  dims: batch, dim, dstate as for the records;
 *               dims->seqlen and dims->dtype are ignored (all float32).
 * Outputs must not alias inputs or each other (SSM_EINVAL).  Allocates
 * nothing; asynchronous on `stream`.
 */
int selective_scan_carry_combine(const float* sum_delta, const float* agg,
                                 const float* A, const float* h0, float* h_in,
                                 float* h_out, int64_t segments,
                                 const ssm_dims* dims, void* stream);

/*
 * One decode step, in place on `state`.
 *   state       : [B][D][N] float32, read and overwritten with the new state
 *   x, dt, z    : [B][D] of dtype (z nullable)
 *   A           : [D][N] float32;  D, dt_bias : [D] float32 (nullable)
 *   B, C        : [B][N] of dtype
 *   out         : [B][D] of dtype, written
 *   dims->seqlen must be 1.  `out` must not alias an input or `state`.
 *   For dstate >= 4, `state` and A must be 16-byte aligned (SSM_EALIGN
 *   otherwise); B and C are read as vectors when they are aligned to four
 *   elements and element by element when not.
 */
int selective_state_update(float* state, const void* x, const void* dt,
                           const float* A, const void* B, const void* C,
                           const float* D, const void* z,
                           const float* dt_bias, int softplus, void* out,
                           const ssm_dims* dims, void* stream);

/*
 * As selective_state_update with the input discretisation `bbar` (an
 * ssm_bbar; any other value returns SSM_EINVAL).  L successive calls with
 * SSM_BBAR_ZOH reproduce selective_scan_fwd_ex with SSM_BBAR_ZOH.
 */
int selective_state_update_ex(float* state, const void* x, const void* dt,
                              const float* A, const void* B, const void* C,
                              const float* D, const void* z,
                              const float* dt_bias, int softplus, int bbar,
                              void* out, const ssm_dims* dims, void* stream);

/*
 * Backward of selective_scan_fwd_h0 (Delta*B input; selective_scan_bwd_ex
 * below takes either input discretisation): the gradients of
 *   sum(dout * out) + sum(dlast * last_state)
 * with respect to every input, by the chain rule through the recurrence with
 * the adjoint state run backwards in time.  The intermediate states are not
 * stored: the forward's training mode (selective_scan_fwd_train, below) is
 * run first into scratch, keeping one state per 8-step chunk and the readout
 * before the gate, and the states inside a chunk are recomputed on chip
 * (reading guide, Hardware-aware state expansion; aigcdaily "Mamba：我们所知的
 * ChatGPT时代的终结者？", Mamba block).
 *   u, delta, A, B, C, D, z, dt_bias, softplus, h0 : the forward's inputs
 *   dout        : [B][L][D] of dtype, gradient of out
 *   dlast       : [B][D][N] float32 (nullable = zeros), gradient of last_state
 * Outputs (overwritten, never accumulated into):
 *   du, ddelta  : [B][L][D] of dtype (ddelta is the gradient of the raw dt)
 *   dA          : [D][N] float32          dB, dC : [B][L][N] of dtype
 *   dD, ddt_bias: [D] float32 (nullable: not written; a null D or dt_bias
 *                 input still has a gradient, taken at zero)
 *   dz          : [B][L][D] of dtype (nullable; must be NULL when z is NULL)
 *   dh0         : [B][D][N] float32 (nullable), gradient of the initial state
 * Outputs must not alias inputs or each other (SSM_EINVAL).  Scratch of
 * about ssm_ckpt_bytes(dims) + 8*N*ceil(D/64)*B*L bytes is allocated
 * stream-ordered and freed on the stream (SSM_ENOMEM on failure).  Sums over
 * channel blocks and batch rows are done in a fixed order (deterministic).
 */
int selective_scan_bwd(const void* u, const void* delta, const float* A,
                       const void* B, const void* C, const float* D,
                       const void* z, const float* dt_bias, int softplus,
                       const float* h0, const void* dout, const float* dlast,
                       void* du, void* ddelta, float* dA, void* dB, void* dC,
                       float* dD, void* dz, float* ddt_bias, float* dh0,
                       const ssm_dims* dims, void* stream);

/*
 * Causal depthwise conv1d + SiLU over a sequence: the short per-channel
 * convolution a Mamba block applies before the selective SSM ("Mamba /
 * MambaMini" Q&A on the Conv before the SSM; reading guide glossary "Mamba
 * Block"):
 *   out[b][t][d] = act( sum_{k<width} weight[d][k] * x[b][t-(width-1)+k][d] + bias[d] )
 * with x at t < 0 taken from state_in (or zero).
 *   x, out      : [B][L][D] of dims->dtype (dims->dstate is ignored)
 *   weight      : [D][width] float32, width in 1..4;  bias : [D] float32 (nullable)
 *   state_in    : [B][D][width-1] float32 (nullable = zeros): the width-1 inputs
 *                 before t = 0, oldest first
 *   state_out   : [B][D][width-1] float32 (nullable): the last width-1 inputs,
 *                 ready for causal_conv1d_update or the next piece's state_in
 *   silu        : nonzero -> act = SiLU, zero -> identity
 * out must not alias x; state_out must not alias state_in or weight
 * (SSM_EINVAL).  Returns an ssm_status.
 */
int causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                      const float* state_in, int width, int silu, void* out,
                      float* state_out, const ssm_dims* dims, void* stream);

/*
 * One decode step of the same convolution, in place on the rolling state.
 *   state       : [B][D][width-1] float32 (oldest first), read and shifted by
 *                 one input (may be NULL only when width == 1)
 *   x, out      : [B][D] of dims->dtype;  weight, bias, width, silu as above
 *   dims->seqlen must be 1.  L successive calls reproduce causal_conv1d_fwd.
 */
int causal_conv1d_update(float* state, const void* x, const float* weight,
                         const float* bias, int width, int silu, void* out,
                         const ssm_dims* dims, void* stream);

/*
 * Weights of one Mamba block (reading guide glossary "Mamba Block": input
 * projection, 1-D convolution, selective SSM, multiplicative gate; "Mamba /
 * MambaMini" Q&A: d_inner = expand * d_model, the Conv before the SSM, B and
 * C from a linear layer, Delta from a low-rank pair of linear layers).
 * Matrices are row-major [rows][cols]; "dtype" is the block's dims->dtype.
 * A projection's weight is stored [out][in], the layout of a PyTorch linear
 * layer's weight: y = x W^T.  x_dt, x_B and x_C are the row blocks of one
 * [dt_rank + 2 d_state][d_inner] x_proj weight; when they lie back to back
 * in that order the block reads them in place, otherwise it copies them
 * into its scratch.
 */
typedef struct {
  const void* in_x;      /* [d_inner][d_model] dtype: x = x_in in_x^T          */
  const void* in_z;      /* [d_inner][d_model] dtype: z = x_in in_z^T (gate)   */
  const float* conv_w;   /* [d_inner][conv_width] float32                      */
  const float* conv_b;   /* [d_inner] float32 (nullable)                       */
  const void* x_dt;      /* [dt_rank][d_inner] dtype: dt_low = u x_dt^T        */
  const void* x_B;       /* [d_state][d_inner] dtype: B = u x_B^T              */
  const void* x_C;       /* [d_state][d_inner] dtype: C = u x_C^T              */
  const void* dt;        /* [d_inner][dt_rank] dtype: dt = dt_low dt^T         */
  const float* dt_bias;  /* [d_inner] float32 (nullable)                       */
  const float* A;        /* [d_inner][d_state] float32                         */
  const float* D;        /* [d_inner] float32 (nullable)                       */
  const void* out;       /* [d_model][d_inner] dtype: out = y out^T            */
} mamba_block_weights;

typedef struct {
  int64_t batch, seqlen, d_model, d_inner, d_state, dt_rank;
  int32_t conv_width;    /* 1..4 */
  int32_t dtype;         /* ssm_dtype of x_in, out, the projection weights and
                            every intermediate activation */
} mamba_block_dims;

/*
 * Forward of one Mamba block:
 *   x, z  = x_in in_x^T, x_in in_z^T                  (hipBLASLt GEMMs)
 *   u     = SiLU(causal_conv1d(x) + conv_b)            (causal_conv1d_fwd)
 *   dt_low, B, C = u x_dt^T, u x_B^T, u x_C^T;  dt = dt_low dt^T  (GEMMs; the
 *           three projections of u run as one GEMM against the stacked
 *           [x_dt; x_B; x_C])
 *   y     = selective scan of u with Delta = softplus(dt + dt_bias), gated
 *           by SiLU(z)                                 (selective_scan_fwd)
 *   out   = y out^T                                    (GEMM)
 *   x_in, out : [batch][seqlen][d_model] of dtype; out must not alias x_in.
 * GEMMs accumulate in float32; intermediates are stored in dtype.  Scratch
 * for the intermediates (about (5 d_inner + dt_rank + 4 d_state) * batch *
 * seqlen elements of dtype, plus a copy of the stacked x_proj weights
 * unless they are already back to back) is allocated stream-ordered and
 * freed on the stream.  Normalisation and the residual connection are the caller's.
 * Returns an ssm_status (SSM_ELAUNCH if a GEMM fails).
 */
int mamba_block_fwd(const void* x_in, const mamba_block_weights* weights, void* out,
                    const mamba_block_dims* dims, void* stream);

/*
 * Training pair: a forward that also keeps the states the backward needs,
 * and a backward that uses them instead of recomputing its own forward pass.
 *   ckpt : float32 device buffer of ssm_ckpt_bytes(dims) bytes holding the
 *          state before every 8th step of every (batch row, block of 64
 *          channels) -- one state per 8 steps, the backward's recompute
 *          granularity -- and the readout before the gate, y = C.h + D u, of
 *          every (batch row, step, channel) in float32 (the backward forms
 *          dz from it); about (8 N / 8 + 4) bytes per token and channel.  Its
 *          layout is internal to the library; 16-byte alignment lets the
 *          kernels move it in vectors.
 * selective_scan_fwd_train is selective_scan_fwd_h0 (Delta*B input) that
 * also writes ckpt (which must not alias another argument); its out and
 * last_state are identical to selective_scan_fwd_h0's.
 * selective_scan_bwd_ckpt is selective_scan_bwd with ckpt read from a
 * selective_scan_fwd_train call on the same inputs; ckpt NULL -> SSM_EINVAL.
 */
int selective_scan_fwd_train(const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D,
                             const void* z, const float* dt_bias, int softplus,
                             const float* h0, void* out, float* last_state,
                             float* ckpt, const ssm_dims* dims, void* stream);

int selective_scan_bwd_ckpt(const void* u, const void* delta, const float* A,
                            const void* B, const void* C, const float* D,
                            const void* z, const float* dt_bias, int softplus,
                            const float* h0, const void* dout,
                            const float* dlast, const float* ckpt, void* du,
                            void* ddelta, float* dA, void* dB, void* dC,
                            float* dD, void* dz, float* ddt_bias, float* dh0,
                            const ssm_dims* dims, void* stream);

/*
 * The backward and the training forward for either input discretisation
 * `bbar` (an ssm_bbar; another value returns SSM_EINVAL).  With
 * SSM_BBAR_DELTA they are selective_scan_bwd / selective_scan_bwd_ckpt and
 * selective_scan_fwd_train exactly.  With SSM_BBAR_ZOH the forward is
 * selective_scan_fwd_ex's exact zero-order hold, h_t = Abar h_{t-1} + coef u B
 * with coef = (exp(Delta A) - 1)/A (reading guide, Method), and the backward
 * uses d coef/d Delta = exp(Delta A) and d coef/d A = (Delta exp(Delta A) -
 * coef)/A (evaluated by a series where |Delta A| < 1/4, limit Delta^2/2 at
 * A = 0).  selective_scan_bwd_ex takes ckpt NULL (it then runs the training
 * forward itself, as selective_scan_bwd) or the buffer of a
 * selective_scan_fwd_train_ex call with the same inputs and the same bbar.
 */
int selective_scan_fwd_train_ex(const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D,
                                const void* z, const float* dt_bias, int softplus,
                                const float* h0, int bbar, void* out,
                                float* last_state, float* ckpt,
                                const ssm_dims* dims, void* stream);

int selective_scan_bwd_ex(const void* u, const void* delta, const float* A,
                          const void* B, const void* C, const float* D,
                          const void* z, const float* dt_bias, int softplus,
                          const float* h0, int bbar, const void* dout,
                          const float* dlast, const float* ckpt, void* du,
                          void* ddelta, float* dA, void* dB, void* dC,
                          float* dD, void* dz, float* ddt_bias, float* dh0,
                          const ssm_dims* dims, void* stream);

/* Bytes of the ckpt buffer for dims (a negative ssm_status if dims are invalid). */
int64_t ssm_ckpt_bytes(const ssm_dims* dims);

/* Static, human-readable name of a status code (never NULL). */
const char* ssm_status_string(int status);

/*
 * Synchronises `stream`, then reports and clears the current device's count of
 * carry waits that hit their bound (a bounded spin in the forward kernel's
 * segment hand-off; a non-zero count means some outputs are invalid).
 * Returns SSM_OK, SSM_ETIMEOUT, or SSM_ELAUNCH if the runtime call failed.
 */
int ssm_check_device_errors(void* stream);

/*
 * Launch plan the forward would use for `dims` (host only, no GPU call):
 * state_groups = waves sharing one block of 64 channels, each holding
 * states_per_group of the N states of every channel; segments = sequence
 * segments: the first of first_segment_len steps, the others of segment_len
 * steps (the last may be shorter); lookback = 1 if segments exchange partial
 * aggregates (decoupled look-back), 0 if each waits for its predecessor's
 * final state; chunk = steps staged through LDS at a time; workgroups = the
 * launch's grid; whole_chains = how many (batch row, channel block) chains run
 * the whole sequence in one workgroup (the others are split into `segments`);
 * helper_waves = waves per workgroup that stage the inputs and finish the
 * outputs beside the state_groups scan waves (a workgroup has
 * 64 * (state_groups + helper_waves) threads).
 * Returns SSM_OK or a validation error.
 */
typedef struct {
  int32_t state_groups;
  int32_t states_per_group;
  int32_t segments;
  int32_t segment_len;
  int32_t lookback;
  int32_t chunk;
  int64_t workgroups;
  int32_t whole_chains;
  int32_t first_segment_len;
  int32_t helper_waves;
} ssm_fwd_plan;

int ssm_fwd_plan_for(const ssm_dims* dims, ssm_fwd_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
