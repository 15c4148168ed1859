// Causal depthwise conv1d + SiLU for gfx950: the short per-channel
// convolution a Mamba block applies before the selective SSM ("Mamba /
// MambaMini" Q&A on the Conv before the SSM: fuse local context, then a
// nonlinearity; reading guide glossary "Mamba Block"), and its constant-time
// decode step on a rolling state of the last K-1 inputs.
//
//   out[b, t, d] = act( sum_{k<K} w[d, k] x[b, t-(K-1)+k, d] + bias[d] )
//
// The op streams x once and writes out once, so it is HBM-bound and laid out
// for it: a thread owns a run of EPT = 4 consecutive channels (one vector per
// row: 16 bytes of float32, 8 of bfloat16) of a tile of TT time steps; a wave
// reads 64 runs of one row, 1 KB or 512 B contiguous.  The K-1 rows before the
// tile are read once more (the halo, (K-1)/TT extra), or come from the
// caller's initial state at t < 0.  Rows are loaded U at a time ahead of their
// use, kept packed until then, so each thread keeps U vector loads in flight.

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {

typedef uint32_t conv_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t conv_u32x2 __attribute__((ext_vector_type(2)));

// Non-temporal vector load and store of a run of EPT activations (the stream
// is read once and written once; the bfloat16 path measured faster with the
// non-temporal hints, the float32 path without them).
template <typename R>
__device__ __forceinline__ void conv_load_nt(R& r, const void* p) {
  const uint32_t* q = static_cast<const uint32_t*>(p);
  static_assert(R::NW == 1 || R::NW == 2 || R::NW == 4, "runs of 1, 2 or 4 words");
  if constexpr (R::NW == 4) {
    const conv_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const conv_u32x4*>(q));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else if constexpr (R::NW == 2) {
    const conv_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const conv_u32x2*>(q));
    r.w[0] = v.x; r.w[1] = v.y;
  } else {
    r.w[0] = __builtin_nontemporal_load(q);
  }
}

template <typename T, int EPT>
__device__ __forceinline__ void conv_store_nt(T* p, const float (&v)[EPT]) {
  using R = Run<T, EPT>;
  static_assert(R::NW == 1 || R::NW == 2 || R::NW == 4, "runs of 1, 2 or 4 words");
  uint32_t w[R::NW];
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) w[k] = __float_as_uint(v[k]);
  } else {
#pragma unroll
    for (int i = 0; i < R::NW; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  }
  uint32_t* q = reinterpret_cast<uint32_t*>(p);
  if constexpr (R::NW == 4) {
    const conv_u32x4 t = {w[0], w[1], w[2], w[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<conv_u32x4*>(q));
  } else if constexpr (R::NW == 2) {
    const conv_u32x2 t = {w[0], w[1]};
    __builtin_nontemporal_store(t, reinterpret_cast<conv_u32x2*>(q));
  } else {
    __builtin_nontemporal_store(w[0], q);
  }
}

template <typename T, int K, int EPT, int TT, int U, bool NT>
__global__ __launch_bounds__(256) void conv1d_fwd_kernel(ConvPtrs p, ConvShape sh) {
  using R = Run<T, EPT>;
  constexpr int H = K > 1 ? K - 1 : 1;   // window rows (at least 1 for the array)
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t runs = sh.runs;
  const int64_t tiles = sh.tiles;
  if (g >= sh.batch * tiles * runs) return;
  const int64_t run = g % runs;
  const int64_t rest = g / runs;
  const int64_t tile = rest % tiles;
  const int64_t b = rest / tiles;
  const int64_t L = sh.seqlen;
  const int64_t dim = sh.dim;
  const int64_t c0 = run * EPT;
  const int last = static_cast<int>((dim - 1 - c0) < (EPT - 1) ? (dim - 1 - c0) : (EPT - 1));
  const bool vec = R::kCanVec && sh.vec_io != 0;
  const T* x = static_cast<const T*>(p.x) + b * L * dim + c0;
  T* out = static_cast<T*>(p.out) + b * L * dim + c0;

  float w[EPT][K], bias[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int64_t c = c0 + (e < last ? e : last);
#pragma unroll
    for (int k = 0; k < K; ++k) w[e][k] = p.weight[c * K + k];
    bias[e] = p.bias ? p.bias[c] : 0.0f;
  }

  // a row's run as loaded (bfloat16 pairs stay packed until used, so the U
  // rows in flight take half the registers)
  auto load_raw = [&](int64_t t, R& r) {
    if (vec) {
      if constexpr (NT) {
        conv_load_nt(r, x + t * dim);
      } else {
        r.load_vec(x + t * dim);
      }
    } else {
      r.load_elems(x + t * dim, last);
    }
  };
  auto load_row = [&](int64_t t, float (&v)[EPT]) {
    R r;
    load_raw(t, r);
#pragma unroll
    for (int e = 0; e < EPT; ++e) v[e] = r.get(e);
  };

  // window: the K-1 inputs before the current row, oldest first
  const int64_t t0 = tile * TT;
  const int64_t t1 = (t0 + TT < L) ? t0 + TT : L;
  float win[H][EPT];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t t = t0 - (K - 1) + j;
    if (K > 1 && t >= 0) {
      load_row(t, win[j]);
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int64_t c = c0 + (e < last ? e : last);
        win[j][e] = (K > 1 && p.state_in) ? p.state_in[(b * dim + c) * (K - 1) + (K - 1 + t)]
                                          : 0.0f;
      }
    }
  }

  for (int64_t tb = t0; tb < t1; tb += U) {
    const int nr = static_cast<int>((t1 - tb < U) ? t1 - tb : U);
    R raw[U];
#pragma unroll
    for (int i = 0; i < U; ++i) load_raw(tb + (i < nr ? i : nr - 1), raw[i]);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (i < nr) {
        float xi[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) xi[e] = raw[i].get(e);
        float o[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          // oldest input first, the same order as the decode step, so L
          // decode steps reproduce the forward bit for bit
          float acc = bias[e];
#pragma unroll
          for (int k = 0; k < K - 1; ++k) acc = fmaf(w[e][k], win[k][e], acc);
          acc = fmaf(w[e][K - 1], xi[e], acc);
          o[e] = sh.silu ? acc * sigmoid_f32(acc) : acc;
        }
        if (NT && vec) {
          conv_store_nt<T, EPT>(out + (tb + i) * dim, o);
        } else {
          store_run<T, EPT>(out + (tb + i) * dim, o, vec, last);
        }
        if constexpr (K > 1) {
#pragma unroll
          for (int j = 0; j < K - 2; ++j)
#pragma unroll
            for (int e = 0; e < EPT; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
          for (int e = 0; e < EPT; ++e) win[K - 2][e] = xi[e];
        }
      }
    }
  }

  // the tile holding the last row leaves the last K-1 inputs as the state
  if (K > 1 && p.state_out && t1 == L) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (e <= last) {
#pragma unroll
        for (int j = 0; j < K - 1; ++j) p.state_out[(b * dim + c0 + e) * (K - 1) + j] = win[j][e];
      }
    }
  }
}

// One decode step per (batch, channel), in place on the rolling state.
template <typename T, int K>
__global__ __launch_bounds__(256) void conv1d_update_kernel(ConvPtrs p, ConvShape sh) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= sh.batch * sh.dim) return;
  const int64_t d = i % sh.dim;
  float win[K];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) win[j] = p.state_inout[i * (K - 1) + j];
  win[K - 1] = to_f32(static_cast<const T*>(p.x)[i]);
  float acc = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) acc = fmaf(p.weight[d * K + k], win[k], acc);
  store_act(static_cast<T*>(p.out), i, sh.silu ? acc * sigmoid_f32(acc) : acc);
#pragma unroll
  for (int j = 0; j < K - 1; ++j) p.state_inout[i * (K - 1) + j] = win[j + 1];
}

// Per activation type: runs of 4 channels (16 bytes of float32, 8 of
// bfloat16), U rows in flight per thread, tiles of TT steps, non-temporal
// hints.  Measured at the 2.8B layer's activations (bfloat16, 4 x 8192 x
// 5120) and the 130M layer's (float32, 8 x 2048 x 1536): bfloat16 runs of 8
// channels (16 bytes) need 158 registers per lane and hold 3 waves per SIMD,
// 164 us; runs of 4 with 8 rows in flight, 64-step tiles and non-temporal
// hints, 144 us; float32 with 4 rows in flight, 32-step tiles and plain
// accesses, 39 us against 41 us with 8 rows.
template <typename T>
struct ConvConfig {
  static constexpr int EPT = 4;
  static constexpr int U = sizeof(T) == 2 ? 8 : 4;
  static constexpr int TT = sizeof(T) == 2 ? 64 : 32;
  static constexpr bool NT = sizeof(T) == 2;
};

template <typename T, int K>
static hipError_t launch_fwd_k(const ConvPtrs& p, ConvShape sh, hipStream_t st) {
  using CC = ConvConfig<T>;
  sh.runs = (sh.dim + CC::EPT - 1) / CC::EPT;
  sh.tiles = (sh.seqlen + CC::TT - 1) / CC::TT;
  const int64_t threads = sh.batch * sh.tiles * sh.runs;
  if ((threads + 255) / 256 > (int64_t{1} << 31) - 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((conv1d_fwd_kernel<T, K, CC::EPT, CC::TT, CC::U, CC::NT>),
                     dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, st, p, sh);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_fwd(int width, const ConvPtrs& p, const ConvShape& sh,
                               hipStream_t st) {
  switch (width) {
    case 1: return launch_fwd_k<T, 1>(p, sh, st);
    case 2: return launch_fwd_k<T, 2>(p, sh, st);
    case 3: return launch_fwd_k<T, 3>(p, sh, st);
    case 4: return launch_fwd_k<T, 4>(p, sh, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv1d_fwd(int dtype, int width, const ConvPtrs& p, const ConvShape& sh,
                             hipStream_t stream) {
  if (dtype == 0) return dispatch_fwd<float>(width, p, sh, stream);
  return dispatch_fwd<bf16_t>(width, p, sh, stream);
}

template <typename T>
static hipError_t dispatch_update(int width, const ConvPtrs& p, const ConvShape& sh,
                                  hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((sh.batch * sh.dim + 255) / 256));
  switch (width) {
    case 1: hipLaunchKernelGGL((conv1d_update_kernel<T, 1>), grid, dim3(256), 0, st, p, sh); break;
    case 2: hipLaunchKernelGGL((conv1d_update_kernel<T, 2>), grid, dim3(256), 0, st, p, sh); break;
    case 3: hipLaunchKernelGGL((conv1d_update_kernel<T, 3>), grid, dim3(256), 0, st, p, sh); break;
    case 4: hipLaunchKernelGGL((conv1d_update_kernel<T, 4>), grid, dim3(256), 0, st, p, sh); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_conv1d_update(int dtype, int width, const ConvPtrs& p, const ConvShape& sh,
                                hipStream_t stream) {
  if (dtype == 0) return dispatch_update<float>(width, p, sh, stream);
  return dispatch_update<bf16_t>(width, p, sh, stream);
}

}  // namespace ssm
