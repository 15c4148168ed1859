// Device helpers shared by the gfx950 selective-scan kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Activation storage: float, or bfloat16 held as its 16 raw bits.
using bf16_t = uint16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

__device__ __forceinline__ void store_act(float* p, int64_t i, float v) { p[i] = v; }

// Two floats rounded to bfloat16 (nearest even) and packed, lo in bits 0-15:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_vt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_vt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_vt v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_vt));
}
__device__ __forceinline__ void store_act(bf16_t* p, int64_t i, float v) {
  // gfx950 converts with round-to-nearest-even in one instruction.
  const __bf16 r = static_cast<__bf16>(v);
  p[i] = __builtin_bit_cast(bf16_t, r);
}

// p advanced by a byte offset held in 32 bits: with p the same for the whole
// wave, the access can take the scalar-base + 32-bit vector-offset form.
template <typename P>
__device__ __forceinline__ P* add_bytes(P* p, uint32_t bytes) {
  using C = typename std::conditional<std::is_const<P>::value, const char, char>::type;
  return reinterpret_cast<P*>(reinterpret_cast<C*>(p) + bytes);
}

// Hardware transcendentals (v_exp_f32 / v_log_f32 / v_rcp_f32, base 2).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(s) = max(s, 0) + log1p(e) with e = e^-|s| in (0, 1].  With
// w = 1 + e rounded, r = e - (w - 1) is the rounding error exactly (w - 1 is
// exact for w in [1, 2]), and log1p(e) = ln(w) + ln(1 + r/w) = ln(w) + r
// up to r e / w <= 2^-24 e: full relative accuracy for tiny e (where w = 1
// and the result is e itself) without a division.
__device__ __forceinline__ float softplus_f32(float s) {
  const float e = exp2_hw(-fabsf(s) * kLog2e);
  const float w = 1.0f + e;
  const float r = e - (w - 1.0f);
  return fmaxf(s, 0.0f) + fmaf(log2_hw(w), kLn2, r);
}

// softplus(s) and its derivative sigmoid(s) = exp(s - softplus(s)), which
// reuses the softplus value: the difference is exact enough (for large s it
// is -e^-s to within an ulp of s, for very negative s it is s) for a result
// within a few ulp.
__device__ __forceinline__ float softplus_sigmoid(float s, float& sig) {
  const float sp = softplus_f32(s);
  sig = exp2_hw((s - sp) * kLog2e);
  return sp;
}

// Input coefficient of the exact zero-order-hold discretisation for a
// diagonal A: Bbar / B = (exp(Delta A) - 1) / A = Delta * phi(x) with
// x = Delta A and phi(x) = (e^x - 1) / x = sum_k x^k / (k+1)!.  Near x = 0
// the difference a - 1 loses digits, so |x| < 1/4 uses the series up to x^5
// (truncation below 5e-8 relative); elsewhere (a - 1) / A loses at most
// ~4e-7 relative to the rounding of a.  x2 = x log2(e) is the argument the
// hardware exp took, a = exp(x), inv_a = 1 / A.  A = 0 takes the series
// (x = 0) and gives the limit Delta; the other branch is not used there.
__device__ __forceinline__ float zoh_coef(float x2, float a, float delta, float inv_a) {
  // coefficients ln(2)^k / (k+1)! of the series in x2
  float p = 2.2222597e-4f;
  p = fmaf(p, x2, 1.9236258e-3f);
  p = fmaf(p, x2, 1.3876027e-2f);
  p = fmaf(p, x2, 8.0075502e-2f);
  p = fmaf(p, x2, 3.4657359e-1f);
  p = fmaf(p, x2, 1.0f);
  const float series = delta * p;
  const float diff = fmaf(a, inv_a, -inv_a);
  return fabsf(x2) < 0.36067376f ? series : diff;
}

// Derivative in A of the zero-order-hold coefficient: d/dA (exp(Delta A) -
// 1)/A = (Delta a - coef)/A = Delta^2 psi(x), psi(x) = (x e^x - (e^x - 1))/x^2
// = sum_k (k+1) x^k / (k+2)!, x = Delta A.  |x| < 1/4 (where the difference
// cancels) uses the series up to x^5 (truncation below 1e-7 relative), A = 0
// included (limit Delta^2 / 2); elsewhere the difference form, which loses
// about three bits to the cancellation at |x| = 1/4.  Arguments as
// zoh_coef, plus coef, its value.
__device__ __forceinline__ float zoh_coef_dA(float x2, float a, float delta, float coef,
                                             float inv_a) {
  // coefficients (k+1) ln(2)^k / (k+2)! of the series in x2
  float p = 1.9047940e-4f;
  p = fmaf(p, x2, 1.6030215e-3f);
  p = fmaf(p, x2, 1.1100822e-2f);
  p = fmaf(p, x2, 6.0056627e-2f);
  p = fmaf(p, x2, 2.3104906e-1f);
  p = fmaf(p, x2, 0.5f);
  const float series = (delta * delta) * p;
  const float diff = fmaf(delta, a, -coef) * inv_a;
  return fabsf(x2) < 0.36067376f ? series : diff;
}

// y * SiLU(z) = y * z / (1 + e^-z)
__device__ __forceinline__ float silu_gate(float y, float z) {
  return y * (z * rcp_hw(1.0f + exp2_hw(-z * kLog2e)));
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (its fence covers
// global memory), which would stall on the loads prefetched for the next
// chunk; here only LDS operations (lgkmcnt) are drained.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Waits for every outstanding global load of the wave.  Used once before a
// long loop so that values loaded in its set-up are not treated as possibly
// in flight inside every iteration.
__device__ __forceinline__ void drain_vmem() {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0), lgkmcnt/expcnt untouched
}

// Marks a register as used here.  Placed on prefetched values at the point
// where they are consumed, it stops the compiler from sinking the use into a
// predicated block, which would leave the load looking in flight on the other
// path (and force a full memory wait at the top of the next loop iteration).
__device__ __forceinline__ void consume(uint32_t x) { asm volatile("" : : "v"(x)); }

// A run of EPT consecutive activations (one row of a chunk tile) in their
// storage format, packed in dwords.  Vector loads and stores are used when
// the run is aligned (the caller decides); otherwise element by element.
template <typename T, int EPT>
struct Run {
  static constexpr int kBytes = EPT * static_cast<int>(sizeof(T));
  static constexpr int NW = kBytes >= 4 ? kBytes / 4 : 1;
  static constexpr bool kCanVec = kBytes >= 4;
  uint32_t w[NW];

  __device__ __forceinline__ void load_vec(const T* p) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    if constexpr (NW >= 4) {
#pragma unroll
      for (int i = 0; i < NW; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(q + i);
        w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
      }
    } else if constexpr (NW == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(q);
      w[0] = v.x; w[1] = v.y;
    } else {
      w[0] = q[0];
    }
  }
  // element path: element k comes from p[min(k, last)]
  __device__ __forceinline__ void load_elems(const T* p, int last) {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = 0;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const T v = p[k < last ? k : last];
      if constexpr (sizeof(T) == 4) {
        w[k] = __builtin_bit_cast(uint32_t, v);
      } else {
        w[k / 2] |= static_cast<uint32_t>(v) << (16 * (k % 2));
      }
    }
  }
  __device__ __forceinline__ void consume_all() const {
#pragma unroll
    for (int i = 0; i < NW; ++i) consume(w[i]);
  }
  __device__ __forceinline__ float get(int k) const {
    if constexpr (sizeof(T) == 4) {
      return __uint_as_float(w[k]);
    } else {
      const uint32_t word = w[k / 2];
      return __uint_as_float((k % 2) ? (word & 0xffff0000u) : (word << 16));
    }
  }
};

// Stores EPT values (rounded to T) at p[0..EPT): one vector store when vec
// (the caller guarantees alignment and a whole run in range), otherwise
// element by element up to index last.
template <typename T, int EPT>
__device__ __forceinline__ void store_run(T* p, const float (&v)[EPT], bool vec, int last) {
  using R = Run<T, EPT>;
  if constexpr (R::kCanVec) {
    if (vec) {
      R o;
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < EPT; ++k) o.w[k] = __float_as_uint(v[k]);
      } else {
#pragma unroll
        for (int i = 0; i < R::NW; ++i) o.w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
      }
      uint32_t* q = reinterpret_cast<uint32_t*>(p);
      if constexpr (R::NW >= 4) {
#pragma unroll
        for (int i = 0; i < R::NW; i += 4)
          *reinterpret_cast<uint4*>(q + i) = make_uint4(o.w[i], o.w[i + 1], o.w[i + 2], o.w[i + 3]);
      } else if constexpr (R::NW == 2) {
        *reinterpret_cast<uint2*>(q) = make_uint2(o.w[0], o.w[1]);
      } else {
        q[0] = o.w[0];
      }
      return;
    }
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k)
    if (k <= last) store_act(p, k, v[k]);
}

// Sum over the four lanes of a quad (lanes 4i .. 4i+3), returned in all four,
// with two DPP exchanges (quad_perm [1,0,3,2] then [2,3,0,1]).  Contraction is
// off so that a product summed here stays a product plus a DPP add (two
// v_add_f32_dpp); fused into an FMA, the exchange would need its own move.
__device__ __forceinline__ float quad_sum(float v) {
#pragma clang fp contract(off)
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                          0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E,
                                                          0xF, 0xF, true));
  return v;
}

// quad_sum of K values at once: the first exchange for all of them, then the
// second, so no DPP read waits on the add just before it.
template <int K>
__device__ __forceinline__ void quad_sum_all(float (&v)[K]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int i = 0; i < K; ++i)
    v[i] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[i]), 0xB1,
                                                               0xF, 0xF, true));
#pragma unroll
  for (int i = 0; i < K; ++i)
    v[i] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[i]), 0x4E,
                                                               0xF, 0xF, true));
}

// Sum over lane pairs (2i, 2i+1), returned in both: one DPP exchange.
__device__ __forceinline__ float pair_sum(float v) {
#pragma clang fp contract(off)
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1,
                                                          0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float sigmoid_f32(float x) {
  return rcp_hw(1.0f + exp2_hw(-x * kLog2e));
}

// Polling load: coherent at device scope but without the cache invalidation
// an acquire carries; pair with acquire_fence() once the value is seen.
__device__ __forceinline__ int load_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void acquire_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ void store_release(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace ssm
