// pa_write.hip — slot-mapped KV writes ("When KV Capacity Runs Out",
// Figure 2: the KV of a new position is stored in a slot of the sequence's
// current block; "Efficient Memory Management for Large Language Model
// Serving with PagedAttention", block-table paragraph: blocks fill left to
// right). Token i with slot >= 0 goes to block slot / B, offset slot % B.
//
// One thread moves 16 bytes of source (8 fp16/bf16 or 4 fp32 elements of one
// head vector). Same-type writes are byte copies; FP8 pools quantise with an
// IEEE fp32 division by the tensor scale, saturation to +-448 and
// round-to-nearest-even to E4M3FN.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Nearest E4M3FN code of x (ties to even), after clamping to [-448, 448].
// NaN gives the NaN code with x's sign; -0 stays -0.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t bits = f2u(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7fffffffu;
  if (mag > 0x7f800000u) return sign | 0x7fu;                 // NaN
  float a = fminf(u2f(mag), 448.0f);                          // clamp (inf too)
  uint32_t code;
  if (a < 0.015625f) {                                        // below 2^-6: grid 2^-9
    // a * 512 is exact; rint rounds half to even. 8 is the code of 2^-6.
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 mantissa bits of the fp32 encoding, round half to even
    uint32_t b = f2u(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    const uint32_t e = (b >> 23) - 127u + 7u;                 // 1..15
    code = (e << 3) | ((b >> 20) & 7u);
  }
  return sign | code;
}

template <Ty SRC> struct SrcVec {
  static constexpr int elems = 16 / TyInfo<SRC>::bytes;       // per thread
};

template <Ty SRC, Ty DST>
__global__ void __launch_bounds__(256)
write_kernel(const WriteParams a) {
  constexpr int E = SrcVec<SRC>::elems;
  const int per_tok = a.num_kv_heads * a.head_dim / E;        // threads per token
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = gi / per_tok;
  if (tok >= a.num_tokens) return;
  const int rem = (int)(gi - tok * per_tok);
  const int64_t slot = a.slot_mapping[tok];
  if (slot < 0 || slot >= (int64_t)a.num_blocks * a.block_size) return;
  const int64_t blk = slot >> a.log2_block_size;
  const int64_t off = slot & (a.block_size - 1);
  const int epl = a.head_dim / E;                             // threads per head
  const int h = rem / epl;
  const int d0 = (rem - h * epl) * E;
  const int64_t dst = blk * a.block_stride + a.layer_offset +
                      ((int64_t)h * a.block_size + off) * a.head_dim + d0;
  const int64_t src = tok * a.num_kv_heads * a.head_dim + (int64_t)h * a.head_dim + d0;

  const bool is_v = blockIdx.y == 1;
  const char* sp = reinterpret_cast<const char*>(is_v ? a.v_src : a.k_src) + src * TyInfo<SRC>::bytes;
  char* dp = reinterpret_cast<char*>(is_v ? a.v_pool : a.k_pool) + dst * TyInfo<DST>::bytes;
  const uint4 x = *reinterpret_cast<const uint4*>(sp);
  if constexpr (SRC == DST) {
    *reinterpret_cast<uint4*>(dp) = x;
  } else {
    static_assert(DST == Ty::FP8, "only FP8 pools convert");
    const float scale = is_v ? a.v_scale : a.k_scale;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float f[E];
#pragma unroll
    for (int i = 0; i < 4; ++i) Widen<SRC>::run(w[i], f + i * Widen<SRC>::per_word);
    uint32_t codes[E / 4];
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      uint32_t packed = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) packed |= e4m3_rne(__fdiv_rn(f[4 * i + b], scale)) << (8 * b);
      codes[i] = packed;
    }
    if constexpr (E == 8) {
      *reinterpret_cast<uint2*>(dp) = make_uint2(codes[0], codes[1]);
    } else {
      *reinterpret_cast<uint32_t*>(dp) = codes[0];
    }
  }
}

template <Ty SRC, Ty DST>
static hipError_t launch_write_t(const WriteParams& a, hipStream_t st) {
  constexpr int E = SrcVec<SRC>::elems;
  const int64_t threads = (int64_t)a.num_tokens * a.num_kv_heads * a.head_dim / E;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((write_kernel<SRC, DST>), dim3((unsigned)blocks, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_write(const WriteParams& a, int src_ty, int dst_ty, hipStream_t st) {
  const Ty s = (Ty)src_ty, d = (Ty)dst_ty;
  if (s == d) {
    switch (s) {
      case Ty::F32: return launch_write_t<Ty::F32, Ty::F32>(a, st);
      case Ty::F16: return launch_write_t<Ty::F16, Ty::F16>(a, st);
      case Ty::BF16: return launch_write_t<Ty::BF16, Ty::BF16>(a, st);
      case Ty::FP8: return launch_write_t<Ty::FP8, Ty::FP8>(a, st);
    }
  }
  if (d == Ty::FP8) {
    switch (s) {
      case Ty::F32: return launch_write_t<Ty::F32, Ty::FP8>(a, st);
      case Ty::F16: return launch_write_t<Ty::F16, Ty::FP8>(a, st);
      case Ty::BF16: return launch_write_t<Ty::BF16, Ty::FP8>(a, st);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
