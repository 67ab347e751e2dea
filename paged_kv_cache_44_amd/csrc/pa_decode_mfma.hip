// pa_decode_mfma.hip — launch side of the matrix-core decode kernels
// (pa_decode_sk.h) for whole contexts: workgroup count, partial slots,
// team size, and the attend / merge launches.
#include "pa_decode_sk.h"

namespace pa {

bool mfma_supported(int kv_ty, int q_ty, int head_dim, int g, int num_seqs) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  const bool types = (kv == Ty::BF16 && q == Ty::BF16) || (kv == Ty::F16 && q == Ty::F16) ||
                     (kv == Ty::FP8 && (q == Ty::BF16 || q == Ty::F16));
  return types && (head_dim == 64 || head_dim == 128) &&
         (g == 1 || g == 2 || g == 4 || g == 8 || g == 16) && num_seqs <= PA_SK_MAX_SEQS;
}

// Partial slots: one per (team, column segment, head in the group) that can
// hold a piece: (W / T + S * H / T) * T.
size_t sk_slots(int blocks, int num_seqs, int num_kv_heads) {
  return (size_t)blocks * NWM + (size_t)num_seqs * num_kv_heads;
}

// Waves per team: the largest power of two up to 8 that divides the KV heads.
int sk_team(int num_kv_heads) {
  int t = 8;
  while (num_kv_heads % t) t >>= 1;
  return t;
}

int sk_blocks(int kv_ty, int q_ty, int head_dim, int g, int num_seqs) {
  return sk_blocks_mode<M_PLAIN>(kv_ty, q_ty, head_dim, g, num_seqs);
}

hipError_t launch_attend_mfma(const DecodeParams& a, int kv_ty, int q_ty, int g, int blocks,
                              hipStream_t st) {
  return sk_launch_attend<M_PLAIN>(a, kv_ty, q_ty, g, blocks, st);
}

hipError_t launch_merge_mfma(const DecodeParams& a, int q_ty, int g, int blocks, hipStream_t st) {
  return sk_launch_merge<M_PLAIN>(a, q_ty, g, blocks, st);
}

}  // namespace pa
