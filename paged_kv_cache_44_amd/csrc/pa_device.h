// pa_device.h — device-side building blocks shared by the paged KV-cache
// kernels (gfx950 / CDNA4, wave64): storage-type traits, conversions, and
// lane exchanges inside 16-lane DPP rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---------------------------------------------------------------------------
// storage / query types
// ---------------------------------------------------------------------------
enum class Ty : int { F32 = 0, F16 = 1, BF16 = 2, FP8 = 3 };

template <Ty T> struct TyInfo;
template <> struct TyInfo<Ty::F32>  { static constexpr int bytes = 4; };
template <> struct TyInfo<Ty::F16>  { static constexpr int bytes = 2; };
template <> struct TyInfo<Ty::BF16> { static constexpr int bytes = 2; };
template <> struct TyInfo<Ty::FP8>  { static constexpr int bytes = 1; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// Widen one 32-bit word of packed storage codes to floats (exact).
template <Ty T> struct Widen;
template <> struct Widen<Ty::F32> {
  static constexpr int per_word = 1;
  __device__ static __forceinline__ void run(uint32_t w, float* o) { o[0] = u2f(w); }
};
template <> struct Widen<Ty::BF16> {
  static constexpr int per_word = 2;
  __device__ static __forceinline__ void run(uint32_t w, float* o) {
    o[0] = u2f(w << 16);
    o[1] = u2f(w & 0xffff0000u);
  }
};
template <> struct Widen<Ty::F16> {
  static constexpr int per_word = 2;
  __device__ static __forceinline__ void run(uint32_t w, float* o) {
    half2_t h = __builtin_bit_cast(half2_t, w);
    o[0] = (float)h[0];
    o[1] = (float)h[1];
  }
};
template <> struct Widen<Ty::FP8> {
  static constexpr int per_word = 4;
  // OCP E4M3FN codes; the gfx950 conversion is exact and keeps NaN.
  __device__ static __forceinline__ void run(uint32_t w, float* o) {
    auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[0] = lo[0]; o[1] = lo[1]; o[2] = hi[0]; o[3] = hi[1];
  }
};

// fp32 -> 16-bit codes, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t b = f2u(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((b >> 16) | 0x0040u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
  _Float16 h = (_Float16)x;   // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// ---------------------------------------------------------------------------
// lane exchanges inside one 16-lane row (DPP, no LDS traffic)
// ---------------------------------------------------------------------------
// DPP control words (gfx9 encoding)
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <- lane 15-i  (xor 15)
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane i^7 in each half row
constexpr int DPP_ROW_ROR4 = 0x124;     // lane i <- lane (i+4) mod 16
constexpr int DPP_ROW_ROR8 = 0x128;     // lane i <- lane (i+8) mod 16 (xor 8)

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(x), CTRL, 0xF, 0xF, true));
}

// Partner pattern for the reduce-scatter stage that splits on lane bit `bit`
// of the 16-lane row. Stages run from bit 3 down to bit 0; each partner
// differs from the lane in that bit and agrees in every higher bit, which is
// all a reduce-scatter needs (lower bits are not yet split).
template <int BIT> struct StageCtrl;
template <> struct StageCtrl<3> { static constexpr int v = DPP_ROW_MIRROR; };
template <> struct StageCtrl<2> { static constexpr int v = DPP_ROW_HALF_MIRROR; };
template <> struct StageCtrl<1> { static constexpr int v = DPP_QUAD_XOR2; };
template <> struct StageCtrl<0> { static constexpr int v = DPP_QUAD_XOR1; };

// Reduce-scatter of N partial values over the 16 lanes of a row.
// On entry lane c holds v[0..N) (a partial sum over its own dims). After the
// call lane c holds NF = max(1, N/16) complete sums in v[0..NF): value index
// NF * (c >> (4 - H)) + j for j < NF, where H = min(4, log2 N) is the number
// of halving stages; the low 4 - H bits of c then hold duplicates.
template <int BIT, int N>
struct ReduceScatter {
  __device__ static __forceinline__ void run(float* v, int c) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      const bool up = (c >> BIT) & 1;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        float lo = v[j] + dpp<StageCtrl<BIT>::v>(v[j]);
        float hi = v[j + H] + dpp<StageCtrl<BIT>::v>(v[j + H]);
        v[j] = up ? hi : lo;
      }
      if constexpr (BIT > 0) ReduceScatter<BIT - 1, H>::run(v, c);
    } else {
      v[0] += dpp<StageCtrl<BIT>::v>(v[0]);
      if constexpr (BIT > 0) ReduceScatter<BIT - 1, 1>::run(v, c);
    }
  }
};

// Max over lane bits 3 and 2 of the row (lanes c, c^4, c^8, c^12), keeping
// bits 1 and 0 apart.
__device__ __forceinline__ float row_max_bits32(float x) {
  x = fmaxf(x, dpp<DPP_ROW_ROR8>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR4>(x));
  return x;
}

}  // namespace pa
