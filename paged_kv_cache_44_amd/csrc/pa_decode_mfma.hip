// pa_decode_mfma.hip — launch side of the matrix-core decode kernels
// (pa_decode_sk.h) for whole contexts: workgroup count, partial slots,
// team size, and the attend / merge launches.
#include <algorithm>

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

// Workgroups one call launches: all the resident ones, unless the batch has
// so few column chunks (at most num_seqs * ceil(max_ctx / 16) per head
// group) that teams would get under 4 each; then enough teams for about 4
// chunks each, in whole rounds of the 8 XCDs. A small batch's chunks are
// then split over fewer, longer ranges: less to dispatch, and far fewer
// pieces to merge (one sequence of 1,000 tokens: 16 pieces instead of 63
// spread over 256 teams).
int sk_launch_blocks(int blocks_max, int num_seqs, int max_ctx, int num_kv_heads) {
  const int T = sk_team(num_kv_heads);
  const int64_t cols = (int64_t)num_seqs * ((max_ctx + CH - 1) / CH) * (num_kv_heads / T);
  const int64_t teams = std::max<int64_t>(1, (cols + 3) / 4);
  int64_t blocks = (teams * T + NWM - 1) / NWM;
  blocks = (blocks + NXCD - 1) / NXCD * NXCD;
  return (int)std::min<int64_t>(blocks_max, std::max<int64_t>(NXCD, blocks));
}

hipError_t launch_attend_mfma(const DecodeParams& a, int kv_ty, int q_ty, int g, int blocks,
                              hipStream_t st) {
  return sk_launch_attend<M_PLAIN>(a, kv_ty, q_ty, g, blocks, st);
}

hipError_t launch_merge_mfma(const DecodeParams& a, int q_ty, int g, int blocks, hipStream_t st) {
  return sk_launch_merge<M_PLAIN>(a, q_ty, g, blocks, st);
}

}  // namespace pa
