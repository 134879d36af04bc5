// dp_device.hpp -- gfx950 device helpers shared by the DeltaProduct kernels:
// element conversion, 16-byte vector moves, MFMA fragment traits and small
// lane reductions.  CDNA4 only: 64-lane wavefronts; v_mfma_f32_16x16x32_bf16
// and v_mfma_f32_16x16x32_f16 for the bf16 path, v_mfma_f32_16x16x4_f32 for
// the fp32 path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dp {

using bf16_t = uint16_t;  // bfloat16 storage (raw bits)
using f16_t = _Float16;   // IEEE half

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders LDS only.  Global loads issued before it stay
// in flight (the compiler waits for them where their registers are used), so
// a prefetch of the next chunk overlaps the current chunk's compute.  The
// kernels exchange data between waves through LDS only.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s / d for 0 <= s < 2^31 with a host-computed magic number (see fastdiv_magic).
__device__ __forceinline__ int fastdiv(int s, uint32_t magic, int shift) {
  return (int)(((unsigned long long)(unsigned)s * magic) >> shift);
}

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// fp32 -> fp16, round to nearest even (hardware conversion).
template <>
__device__ __forceinline__ f16_t from_f32<f16_t>(float x) {
  return (f16_t)x;
}

// Elements of type T held in one 16-byte vector.
template <typename T>
struct Vec {
  static constexpr int N = 16 / (int)sizeof(T);
};

// Unpack a 16-byte vector of T into N floats.
__device__ __forceinline__ void unpack16(const u32x4_t& v, float* f, float /*tag*/) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ void unpack16(const u32x4_t& v, float* f, bf16_t /*tag*/) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const u32x4_t& v, float* f, f16_t /*tag*/) {
  f16x8_t h;
  __builtin_memcpy(&h, &v, 16);
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// Store 16 bytes of consecutive elements (fp32 inputs, 16/sizeof(T) of them) as T.
__device__ __forceinline__ void st_vec16(float* p, const float* f) {
  f32x4_t v = {f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4_t*>(p) = v;
}
__device__ __forceinline__ void st_vec16(f16_t* p, const float* f) {
  f16x8_t v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (f16_t)f[i];
  *reinterpret_cast<f16x8_t*>(p) = v;
}

__device__ __forceinline__ void st_vec16(bf16_t* p, const float* f) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (uint32_t)from_f32<bf16_t>(f[2 * i]) | ((uint32_t)from_f32<bf16_t>(f[2 * i + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// Store 4 consecutive elements (fp32 inputs) as T at p.
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  f32x4_t v = {a, b, c, d};
  *reinterpret_cast<f32x4_t*>(p) = v;
}
__device__ __forceinline__ void st4(f16_t* p, float a, float b, float c, float d) {
  f16x4_t v = {(f16_t)a, (f16_t)b, (f16_t)c, (f16_t)d};
  *reinterpret_cast<f16x4_t*>(p) = v;
}
__device__ __forceinline__ void st4(bf16_t* p, float a, float b, float c, float d) {
  u32x2_t v;
  v[0] = (uint32_t)from_f32<bf16_t>(a) | ((uint32_t)from_f32<bf16_t>(b) << 16);
  v[1] = (uint32_t)from_f32<bf16_t>(c) | ((uint32_t)from_f32<bf16_t>(d) << 16);
  *reinterpret_cast<u32x2_t*>(p) = v;
}

// ------------------------------------------------------------ MFMA traits
//
// D(16x16, fp32) += A(16 x KS) * B(KS x 16).  Both operands are read from
// buffers laid out "row by k": A as A[m][k] = base[(row0 + m) * ld + k0 + k],
// B as B[k][n] = base[(row0 + n) * ld + k0 + k] (i.e. the buffer holds B^T).
// Lane l holds row/column (l & 15) and the k slice selected by (l >> 4); the
// same k slice is used for A and B, so the contraction is correct for any
// hardware assignment of k within a lane group.  The accumulator layout is
// D[4 * (l >> 4) + i][l & 15], i = 0..3.
//
// load_t reads the transpose: element (m, k) at base[(k0 + k) * ld + row0 + m].

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  static constexpr int KS = 32;  // k per instruction
  using frag_t = bf16x8_t;

  __device__ __forceinline__ static frag_t load(const bf16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const bf16_t* p = base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4);
    return *reinterpret_cast<const frag_t*>(p);
  }
  __device__ __forceinline__ static frag_t load_t(const bf16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const bf16_t* p = base + (k0 + 8 * (l >> 4)) * ld + row0 + (l & 15);
    u16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e * ld];
    return __builtin_bit_cast(frag_t, v);
  }
  __device__ __forceinline__ static f32x4_t mma(const frag_t& a, const frag_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // 16-deep step (v_mfma_f32_16x16x16_bf16) for a contraction of length 16
  using frag4_t = s16x4_t;
  __device__ __forceinline__ static frag4_t load4(const bf16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const frag4_t*>(base + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  }
  __device__ __forceinline__ static frag4_t load4_t(const bf16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const bf16_t* p = base + (k0 + 4 * (l >> 4)) * ld + row0 + (l & 15);
    frag4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (short)p[e * ld];
    return v;
  }
  __device__ __forceinline__ static f32x4_t mma4(const frag4_t& a, const frag4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<f16_t> {
  static constexpr int KS = 32;
  using frag_t = f16x8_t;

  __device__ __forceinline__ static frag_t load(const f16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const f16_t* p = base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4);
    return *reinterpret_cast<const frag_t*>(p);
  }
  __device__ __forceinline__ static frag_t load_t(const f16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const f16_t* p = base + (k0 + 8 * (l >> 4)) * ld + row0 + (l & 15);
    frag_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e * ld];
    return v;
  }
  __device__ __forceinline__ static f32x4_t mma(const frag_t& a, const frag_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // 16-deep step (v_mfma_f32_16x16x16_f16) for a contraction of length 16
  using frag4_t = f16x4_t;
  __device__ __forceinline__ static frag4_t load4(const f16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    return *reinterpret_cast<const frag4_t*>(base + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  }
  __device__ __forceinline__ static frag4_t load4_t(const f16_t* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    const f16_t* p = base + (k0 + 4 * (l >> 4)) * ld + row0 + (l & 15);
    frag4_t v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = p[e * ld];
    return v;
  }
  __device__ __forceinline__ static f32x4_t mma4(const frag4_t& a, const frag4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KS = 4;
  using frag_t = float;

  __device__ __forceinline__ static frag_t load(const float* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    return base[(row0 + (l & 15)) * ld + k0 + (l >> 4)];
  }
  __device__ __forceinline__ static frag_t load_t(const float* base, int ld, int row0, int k0) {
    const int l = threadIdx.x & 63;
    return base[(k0 + (l >> 4)) * ld + row0 + (l & 15)];
  }
  __device__ __forceinline__ static f32x4_t mma(const frag_t& a, const frag_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  using frag4_t = float;  // unused: every contraction length is a multiple of 4
  __device__ __forceinline__ static frag4_t load4(const float*, int, int, int) { return 0.f; }
  __device__ __forceinline__ static frag4_t load4_t(const float*, int, int, int) { return 0.f; }
  __device__ __forceinline__ static f32x4_t mma4(const frag4_t&, const frag4_t&, const f32x4_t& c) {
    return c;
  }
};

// acc += A[ra.., 0..K) * B[0..K, rb..]  (both "row by k" buffers).  K is a
// multiple of the instruction depth, or of 16 for the 16-bit types (the last
// 16 of the contraction then use the 16-deep instruction).
template <typename T, int K>
__device__ __forceinline__ f32x4_t mm_tile(f32x4_t acc, const T* a, int lda, int ra, const T* b,
                                           int ldb, int rb) {
  using M = Mfma<T>;
  static_assert(K % M::KS == 0 || K % M::KS == 16, "contraction length");
#pragma unroll
  for (int k0 = 0; k0 + M::KS <= K; k0 += M::KS)
    acc = M::mma(M::load(a, lda, ra, k0), M::load(b, ldb, rb, k0), acc);
  if constexpr (K % M::KS == 16)
    acc = M::mma4(M::load4(a, lda, ra, K - 16), M::load4(b, ldb, rb, K - 16), acc);
  return acc;
}

// acc += A^T-read operand (element (m,k) at a[k*lda + ra + m]) times B.
template <typename T, int K>
__device__ __forceinline__ f32x4_t mm_tile_ta(f32x4_t acc, const T* a, int lda, int ra, const T* b,
                                              int ldb, int rb) {
  using M = Mfma<T>;
  static_assert(K % M::KS == 0 || K % M::KS == 16, "contraction length");
#pragma unroll
  for (int k0 = 0; k0 + M::KS <= K; k0 += M::KS)
    acc = M::mma(M::load_t(a, lda, ra, k0), M::load(b, ldb, rb, k0), acc);
  if constexpr (K % M::KS == 16)
    acc = M::mma4(M::load4_t(a, lda, ra, K - 16), M::load4(b, ldb, rb, K - 16), acc);
  return acc;
}

// acc += A * B-transposed-read operand (element (n,k) of B^T at b[k*ldb + rb + n]).
template <typename T, int K>
__device__ __forceinline__ f32x4_t mm_tile_tb(f32x4_t acc, const T* a, int lda, int ra, const T* b,
                                              int ldb, int rb) {
  using M = Mfma<T>;
  static_assert(K % M::KS == 0 || K % M::KS == 16, "contraction length");
#pragma unroll
  for (int k0 = 0; k0 + M::KS <= K; k0 += M::KS)
    acc = M::mma(M::load(a, lda, ra, k0), M::load_t(b, ldb, rb, k0), acc);
  if constexpr (K % M::KS == 16)
    acc = M::mma4(M::load4(a, lda, ra, K - 16), M::load4_t(b, ldb, rb, K - 16), acc);
  return acc;
}

// ------------------------------------------------------------ fp16 register-operand MFMA
//
// The register-resident scan keeps its B operands (state, X, pseudo-values) in
// accumulator layout: lane (g = l >> 4, n = l & 15) of a 16x16 tile holds rows
// 4g..4g+3 of column n.  A 32-deep step over two such tiles t, t+1 uses, for
// lane group g, the k set {16t + 4g + e} U {16t + 16 + 4g + e} (e = 0..3), so
// B comes straight from the two tiles and A is read with the same k set.

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ f16x4_t to_h4(const f32x4_t& t) { return __builtin_convertvector(t, f16x4_t); }
__device__ __forceinline__ f16x8_t cat8(const f16x4_t& a, const f16x4_t& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4_t mfma32h(const f16x8_t& a, const f16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16h(const f16x4_t& a, const f16x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// A rows straight from LDS: row `row`, k set of the step starting at k0.
__device__ __forceinline__ f16x8_t lds_a32(const f16_t* base, int ld, int row, int k0) {
  const f16_t* p = base + row * ld + k0 + 4 * ((threadIdx.x >> 4) & 3);
  return cat8(*reinterpret_cast<const f16x4_t*>(p), *reinterpret_cast<const f16x4_t*>(p + 16));
}
__device__ __forceinline__ f16x4_t lds_a16(const f16_t* base, int ld, int row, int k0) {
  return *reinterpret_cast<const f16x4_t*>(base + row * ld + k0 + 4 * ((threadIdx.x >> 4) & 3));
}
// A = transpose of a row-major LDS tile: element (m, k) = base[k * ld + d0 + m],
// k set {j0 + 4g + e}, via ds_read_b64_tr_b16: in each 16-lane group, source
// lane i (e = i / 4, a = i % 4) points at base[(j0 + 4g + e) * ld + d0 + 4a];
// output lane m then receives element (m, j0 + 4g + e) for e = 0..3.
__device__ __forceinline__ f16x4_t lds_t16(const f16_t* base, int ld, int d0, int j0) {
  const int l = threadIdx.x & 63, i = l & 15, g = l >> 4;
  const f16_t* p = base + (j0 + 4 * g + (i >> 2)) * ld + d0 + 4 * (i & 3);
  return __builtin_bit_cast(f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
}

// acc += A (16 x K: LDS rows `row`) * B (K x 16: register tiles b[0..K/16))
template <int K>
__device__ __forceinline__ f32x4_t mm_ar(f32x4_t acc, const f16_t* a, int lda, int row, const f16x4_t* b) {
  static_assert(K % 16 == 0, "K");
#pragma unroll
  for (int t = 0; t + 1 < K / 16; t += 2) acc = mfma32h(lds_a32(a, lda, row, 16 * t), cat8(b[t], b[t + 1]), acc);
  if constexpr ((K / 16) % 2 == 1) acc = mfma16h(lds_a16(a, lda, row, K - 16), b[K / 16 - 1], acc);
  return acc;
}
// acc += A (16 x K: transpose of LDS rows, element (m,k) = a[k * lda + d0 + m]) * B (register tiles)
template <int K>
__device__ __forceinline__ f32x4_t mm_atr(f32x4_t acc, const f16_t* a, int lda, int d0, const f16x4_t* b) {
  static_assert(K % 16 == 0, "K");
#pragma unroll
  for (int t = 0; t + 1 < K / 16; t += 2)
    acc = mfma32h(cat8(lds_t16(a, lda, d0, 16 * t), lds_t16(a, lda, d0, 16 * t + 16)), cat8(b[t], b[t + 1]),
                  acc);
  if constexpr ((K / 16) % 2 == 1) acc = mfma16h(lds_t16(a, lda, d0, K - 16), b[K / 16 - 1], acc);
  return acc;
}
// acc += A (LDS rows ra) * B (LDS rows rb, the "row by k" buffer of B^T)
template <int K>
__device__ __forceinline__ f32x4_t mm_ll(f32x4_t acc, const f16_t* a, int lda, int ra, const f16_t* b, int ldb,
                                         int rb) {
  static_assert(K % 16 == 0, "K");
#pragma unroll
  for (int t = 0; t + 1 < K / 16; t += 2)
    acc = mfma32h(lds_a32(a, lda, ra, 16 * t), lds_a32(b, ldb, rb, 16 * t), acc);
  if constexpr ((K / 16) % 2 == 1) acc = mfma16h(lds_a16(a, lda, ra, K - 16), lds_a16(b, ldb, rb, K - 16), acc);
  return acc;
}

// ------------------------------------------------------------ lane reductions

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, W);
  return x;
}

// Sum over aligned groups of W consecutive lanes (W = 2, 4, 8 or 16: inside
// one DPP row) by DPP: lane ^ 1, lane ^ 2, the mirrored quad, the mirrored
// half.  Every lane of a group ends with the same value.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float x) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group within a DPP row");
  auto add = [](float v, auto ctrl) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, true));
  };
  x = add(x, std::integral_constant<int, 0xB1>{});                     // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) x = add(x, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) x = add(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (W >= 16) x = add(x, std::integral_constant<int, 0x140>{}); // row_mirror
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    float y = __shfl_up(x, d, 64);
    if (l >= d) x += y;
  }
  return x;
}

// clamp that lets NaN through (comparisons with NaN are false)
__device__ __forceinline__ float clamp_keep_nan(float x, float lo, float hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace dp
