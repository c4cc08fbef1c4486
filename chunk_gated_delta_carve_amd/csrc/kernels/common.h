// Shared device helpers for the CARVE kernels on gfx950 (CDNA4).
//
// MFMA conventions used everywhere (16x16 output tiles, 64-wide wavefronts):
//   lane l, group g = l / 16, column c = l % 16
//   C tile (f32x4):   lane holds C[4g + i][c], i = 0..3
//   A fragment:       lane holds A[c][k-slots of group g]
//   B fragment:       lane holds B[k-slots of group g][c]
// A and B use the same map from (g, slot) to the reduction index k, so any
// permutation of k inside one instruction is allowed as long as both operands
// agree. Two maps are used:
//   natural: slot i of group g is k = K * g + i  (K = slots per lane)
//   c-pair : for bf16 16x16x32, slots 0..3 are k = 4g + i and slots 4..7 are
//            k = 16 + 4g + (i - 4); for f32 16x16x4, step p of a 16-row block
//            uses k = 16 (p / 4) + 4g + (p % 4).
// The c-pair map lets a C tile (rows 4g..4g+3 of a lane) feed the next
// instruction's B operand straight from registers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace carve {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index as a scalar: lets the compiler treat per-wave decisions as
// uniform branches instead of exec-masked divergent code
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename M> __device__ __forceinline__ M from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
constexpr float kLog2e = 1.4426950408889634f;

// Log-decay in log2 units from the decay input: g itself, or, with kLogits,
// g = -softplus(a) from a raw decay logit a, evaluated as
// -(max(a, 0) log2 e + log2(1 + 2^{-|a| log2 e})) so neither end overflows.
template <bool kLogits>
__device__ __forceinline__ float decay_log2(float x) {
  if constexpr (kLogits) return -(fmaxf(x, 0.f) * kLog2e + fast_log2(1.f + fast_exp2(-fabsf(x) * kLog2e)));
  else return x * kLog2e;
}

// logistic(x) = 1 / (1 + e^{-x}); saturates cleanly at both ends
__device__ __forceinline__ float sigmoid_f(float x) {
  return fast_rcp(1.0f + fast_exp2(-x * kLog2e));
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// MFMA policy per operand type.
template <typename M> struct Mma;

// A "unit" is 16 bytes per lane (1 KiB per wave): the operand fragments of one
// 16-row tile over KU consecutive reduction indices (c-pair map), i.e. SPU
// instructions' worth. Units are what the state pass loads and stores.
template <> struct Mma<bf16> {
  static constexpr int KS = 32;  // reduction length of one instruction
  typedef bf16x8 frag;
  typedef bf16x8 unit;
  static constexpr int KU = 32, SPU = 1, UT = 2;   // k per unit, steps per unit, C tiles per unit
  __device__ __forceinline__ static frag step(unit u, int) { return u; }
  // unit from C tiles of a transposed product: t[j] holds k = 16 (UT u + j) + 4g + i
  __device__ __forceinline__ static unit pack(const f32x4* t) {
    return unit{(bf16)t[0][0], (bf16)t[0][1], (bf16)t[0][2], (bf16)t[0][3],
                (bf16)t[1][0], (bf16)t[1][1], (bf16)t[1][2], (bf16)t[1][3]};
  }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // natural map from a row-major tile: row `row`, k = k0 + 8g + i
  __device__ __forceinline__ static frag ld_nat(const bf16* base, int ld, int row, int k0) {
    const int g = lane_id() >> 4;
    return *reinterpret_cast<const bf16x8*>(base + row * ld + k0 + 8 * g);
  }
  __device__ __forceinline__ static frag ld_nat(const float* base, int ld, int row, int k0) {
    const int g = lane_id() >> 4;
    const f32x4* p = reinterpret_cast<const f32x4*>(base + row * ld + k0 + 8 * g);
    f32x4 a = p[0], b = p[1];
    return frag{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
  // c-pair map, reduction step p: k = 32p + 4g + i (i < 4), 32p + 16 + 4g + i - 4
  __device__ __forceinline__ static frag ld_cp(const bf16* base, int ld, int row, int p) {
    const int g = lane_id() >> 4;
    const bf16* r = base + row * ld + 32 * p + 4 * g;
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(r);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(r + 16);
    return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // B operand for reduction step p built from C tiles t[2p], t[2p+1]
  __device__ __forceinline__ static frag from_c(const f32x4* t, int p) {
    f32x4 a = t[2 * p], b = t[2 * p + 1];
    return frag{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
  }
  // number of reduction steps covering `n` rows of C tiles (n multiple of 16)
  __device__ __forceinline__ static constexpr int steps(int n) { return (n + 31) / 32; }
};

template <> struct Mma<float> {
  static constexpr int KS = 4;
  typedef float frag;
  typedef f32x4 unit;
  static constexpr int KU = 16, SPU = 4, UT = 1;
  __device__ __forceinline__ static frag step(unit u, int j) { return u[j]; }
  __device__ __forceinline__ static unit pack(const f32x4* t) { return t[0]; }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag ld_nat(const float* base, int ld, int row, int k0) {
    return base[row * ld + k0 + (lane_id() >> 4)];
  }
  __device__ __forceinline__ static frag ld_cp(const float* base, int ld, int row, int p) {
    const int g = lane_id() >> 4;
    return base[row * ld + 16 * (p >> 2) + 4 * g + (p & 3)];
  }
  __device__ __forceinline__ static frag from_c(const f32x4* t, int p) { return t[p >> 2][p & 3]; }
  __device__ __forceinline__ static constexpr int steps(int n) { return n / 4; }
};

// 16x16x16 product whose B operand is one C tile (bf16: one instruction with
// the natural 4-slot map, which coincides with the C layout; f32: four
// 16x16x4 instructions). The A operand is a lane's 4 values of row c,
// k = 4g + i.
template <typename M> struct Mma16;
template <> struct Mma16<bf16> {
  typedef bf16x4 e4;
  // operands already in bf16: a = A[c][4g + i], b = B[4g + i][c] (a C tile)
  __device__ __forceinline__ static f32x4 mma(e4 a, e4 b, f32x4 c) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b),
                                                      c, 0, 0, 0);
  }
  // a C tile rounded to operand precision
  __device__ __forceinline__ static e4 round(f32x4 x) {
    return e4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  }
};
template <> struct Mma16<float> {
  typedef f32x4 e4;
  __device__ __forceinline__ static f32x4 mma(e4 a, e4 b, f32x4 c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[p], b[p], c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static e4 round(f32x4 x) { return x; }
};

// DPP lane moves (gfx9 encodings): CTRL 0xB1 = quad_perm [1,0,3,2] (lane
// xor 1), 0x4E = quad_perm [2,3,0,1] (lane xor 2), 0x114 = row_shr:4 (lane i
// reads lane i - 4 of its 16-lane row; lanes without a source read 0).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// sum over the four lanes of a quad, in every lane of it
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp_mov<0xB1>(x);
  return x + dpp_mov<0x4E>(x);
}
// sum over the 16 lanes of a DPP row, in every lane of it
__device__ __forceinline__ float sum_row16(float x) {
  x += dpp_mov<0x128>(x);   // row_ror:8
  x += dpp_mov<0x124>(x);   // row_ror:4
  x += dpp_mov<0x122>(x);   // row_ror:2
  return x + dpp_mov<0x121>(x);   // row_ror:1
}
// Sum of the two 16-lane rows of each pair (rows 0 and 1, rows 2 and 3).
__device__ __forceinline__ float sum_row_pairs(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum of the two halves of the wave.
__device__ __forceinline__ float sum_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum over all 64 lanes of the wave, in every lane.
__device__ __forceinline__ float wave_sum(float x) { return sum_halves(sum_row_pairs(sum_row16(x))); }
// 1 / max(sqrt(ss), 1e-12): the inverse L2 norm of a vector whose sum of
// squares is ss, guarded as x / max(|x|, eps) for a zero vector
__device__ __forceinline__ float inv_norm(float ss) { return 1.f / fmaxf(sqrtf(ss), 1e-12f); }

// Sum over the four row groups of a C tile column: lanes c, c+16, c+32, c+48.
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Sum over the 16 columns of a C tile row group: lanes 16g .. 16g+15.
__device__ __forceinline__ f32x4 sum_cols(f32x4 x) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] += __shfl_xor(x[i], m);
  return x;
}

}  // namespace carve
