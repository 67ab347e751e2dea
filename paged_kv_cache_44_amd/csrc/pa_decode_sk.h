// pa_decode_sk.h — paged decode attention with the grouped-query tile on
// the gfx950 matrix cores, work split evenly over the resident waves.
//
// Same result as the VALU kernel ("Efficient Memory Management for Large
// Language Model Serving with PagedAttention", kernel paragraph: fetch each
// block through the block table, score the query group against it, combine
// with its values; identical to ordinary attention). With G query heads per
// KV head both products of a 16-token chunk are small dense contractions:
//   S[16 tokens][G heads] = K[16][D] . Q^T[D][G]   (v_mfma_f32_16x16x32)
//   O[G heads][D]        += P[G][16] . V[16][D]    (v_mfma_f32_16x16x16)
// G <= 16 fills the 16 columns of the tile.
//
// Work split ("stream-K"): the W resident waves form teams of T waves (T =
// the largest power of two up to 8 dividing the KV head count). Segments are
// (sequence, head group of T KV heads), sequence-major, each a run of
// ceil(context / 16) column chunks; team t takes columns [t*Cc/Wt,
// (t+1)*Cc/Wt) of the Cc total, wave i of the team the i-th KV head of each
// group. So every team gets the same amount of work whatever the length mix,
// and the T waves of a team read the T head slices of the same KV block (one
// contiguous stretch of the pool) at about the same time, which the memory
// system serves markedly faster than the same number of scattered slices. A
// segment cut by range boundaries leaves one partial (running max m, sum l,
// unnormalised o) per piece and head, stored at slot ((team + segment) * T +
// i); merge_sk_kernel combines them in team order.
//
// Layout facts used (CDNA 16x16xK MFMA, checked on gfx950): lane l holds
// A[row l%16][k in (l/16)*KL ..], B[k in (l/16)*KL ..][col l%16] and
// C[rows 4*(l/16) .. +3][col l%16].
//  * K: lane l loads token l%16, dims 32c + 8(l/16) .. +8 of step c: the A
//    operand of the score MFMA straight from memory.
//  * The score tile comes out as lane l = (tokens 4(l/16)..+3, head l%16),
//    exactly the A-operand layout of the P.V MFMA: probabilities never leave
//    their lane.
//  * V: lane (g, n) loads the slice [VPL*n, +VPL) of tokens 4g..4g+3 (whole
//    256-byte rows per load instruction); P.V MFMA m uses output column n for
//    dim VPL*n + m and takes element m of the four vectors (two byte permutes).
//  * Online softmax with a lazily moved reference maximum per head: it moves
//    (exact cross-lane max, rescale) only when a score exceeds it by more than
//    2^TAU, so probabilities stay <= 2^8 and most chunks need no cross-lane
//    traffic.
//  * Block ids come from a 64-entry window of the block table held in one
//    register (lane i = entry i), read with readlane / a lane shuffle.
//  * Workgroups are dealt to the 8 XCDs round-robin; team ranges are assigned
//    so that each XCD works through one contiguous stretch of sequences.
//  * Each loaded chunk travels with a descriptor (segment, chunk, piece
//    boundaries), so pieces of any length, down to one chunk, are handled
//    while the next chunk is already in flight.
//
// Shared prefixes ("Efficient Memory Management for Large Language Model
// Serving with PagedAttention", sampling paragraph: parallel samples share
// the prompt's blocks; "Continuous Batching and PagedAttention", section
// "Sharing, the part that goes beyond fixing what broke") are read once per
// up to 32/G sequences instead of once per sequence, in two passes of the
// same kernel body that run side by side in one launch
// (attend_sk_dual_kernel):
//  * M_PREFIX: a segment is a slot of up to 32/G consecutive sequences
//    whose tables share the prefix blocks; their queries fill the 32
//    columns of two tiles side by side (column c: sequence first + c/G,
//    head c%G), so each K/V chunk of the prefix is loaded once for all of
//    them (its operands built once, both tiles' products from them). Every
//    piece is left as a partial (m, l, o) per column, and the team range of
//    each prefix segment is recorded.
//  * M_SUFFIX: each sequence's segment starts after its shared prefix (the
//    whole context when it has none). A segment inside one team's range is
//    finished here when its sequence has no prefix, and left as a partial
//    of the sequence's own tokens (pre_m, pre_l, pre_o) when it has one; a
//    cut segment leaves pieces as in the plain decode. Both passes record
//    each segment's team range.
//  * shared_combine_kernel (pa_decode_shared.hip) finishes every other row:
//    the suffix pieces or own partial, plus the prefix pieces.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr int NWM = 4;          // waves per workgroup
constexpr int CH = 16;          // tokens per chunk
constexpr int NXCD = 8;         // XCDs of an MI355X

// Chunks of a sequence: 0 when its context is empty or invalid (those rows
// are written by the merge kernel).
__device__ __forceinline__ int seq_chunks(const DecodeParams& a, int ctx) {
  if (ctx <= 0 || ctx > a.max_context_len) return 0;
  const int64_t nb = ((int64_t)ctx + a.block_size - 1) >> a.log2_block_size;
  if (nb > a.max_blocks_per_seq) return 0;
  return (ctx + CH - 1) / CH;
}

// Tokens of sequence s covered by a shared prefix: the plan's start when it
// is a multiple of 16 inside a valid context, else 0 (no prefix). Every
// kernel of the shared-prefix decode decides "has a prefix" by this.
__device__ __forceinline__ int own_start(const DecodeParams& a, int s, int ctx) {
  if (seq_chunks(a, ctx) == 0) return 0;
  const int st0 = a.share_start[s];
  return (st0 < 0 || st0 > ctx || (st0 & (CH - 1))) ? 0 : st0;
}

// A pass's record of a segment, {first team, last team, column count, teams
// of the pass}, checked against the most teams the launch can have.
__device__ __forceinline__ bool segment_record_ok(const int4 sg, int max_teams) {
  return sg.w > 0 && sg.w <= max_teams && sg.x >= 0 && sg.x <= sg.y && sg.y < sg.w && sg.z > 0;
}

// The prefix-pass segment holding sequence s's prefix for head group hg:
// its index cs, the sequence's first tile column col0, and the teams t0 ..
// t1 (of the pass's teams, and its column count Ccp) whose ranges hold its
// pieces. False when s has no prefix slot or the records do not fit the
// batch (they then are not read).
__device__ __forceinline__ bool prefix_segment(const DecodeParams& a, int s, int hg, int hgs,
                                               int ns, int g, int64_t& cs, int& col0, int& t0,
                                               int& t1, int64_t& ccp, int& teams) {
  const int4 sd = reinterpret_cast<const int4*>(a.share_desc)[s];
  const int p = sd.x;
  if (p < 0 || p > s || s - p >= ns) return false;
  cs = (int64_t)p * hgs + hg;
  const int4 sg = reinterpret_cast<const int4*>(a.share_seg)[cs];
  if (!segment_record_ok(sg, a.pre_teams)) return false;
  t0 = sg.x;
  t1 = sg.y;
  ccp = sg.z;
  teams = sg.w;
  col0 = (s - p) * g;
  return true;
}

// Team ranges. The W resident waves form Wt = W / T teams of T consecutive
// (XCD-contiguous) waves, one KV head of the group per wave; team t takes
// columns [t*Cc/Wt, (t+1)*Cc/Wt) of the Cc total.
__device__ __forceinline__ int64_t team_begin(int64_t t, int64_t Cc, int64_t Wt) {
  return t * Cc / Wt;
}

// Team whose range holds column c (the last team starting at or before c).
__device__ __forceinline__ int64_t team_of(int64_t c, int64_t Cc, int64_t Wt) {
  return ((c + 1) * Wt - 1) / Cc;
}

// Dynamic LDS of the attention kernel: prefix sums, the shared-prefix modes'
// per-segment word, and last-chunk lengths.
inline size_t sk_lds_bytes(int num_seqs, int mode) {
  return (size_t)(num_seqs + 1) * sizeof(int) + (mode ? (size_t)num_seqs * sizeof(uint32_t) : 0) +
         (((size_t)num_seqs + 3) & ~(size_t)3);
}

}  // namespace

// Decode modes (see the head of this file): whole contexts, shared prefixes
// of several sequences side by side, the rest of each context after its
// shared prefix.
constexpr int M_PLAIN = 0, M_PREFIX = 1, M_SUFFIX = 2;

// Occupancy: FP8 pools and D = 64 fit 3 waves per SIMD without spilling;
// 16-bit pools at D = 128 run at 2.
// The prefix pass (16 query columns of several sequences) needs more
// registers and runs at 2 everywhere.
template <Ty KV, int D, int G, int MODE>
constexpr int sk_waves_per_simd() {
  return MODE == M_PREFIX ? 2 : ((KV == Ty::FP8 || D == 64) ? 3 : 2);
}

// The kernel body: a launch of its own (attend_sk_kernel: the workgroup
// index and count are the grid's), or one part of a launch that runs two
// modes side by side (attend_sk_dual_kernel, PART: workgroup part_blk of the
// part's part_nblk).
template <Ty KV, Ty QT, int D, int G, int MODE, bool PART>
__device__ __forceinline__ void attend_sk_body(const DecodeParams& a, const int part_blk,
                                               const int part_nblk) {
  auto blk = [&]() __attribute__((always_inline)) { return PART ? part_blk : (int)blockIdx.x; };
  auto nblk = [&]() __attribute__((always_inline)) { return PART ? part_nblk : (int)gridDim.x; };
  static_assert(QT == Ty::BF16 || QT == Ty::F16, "16-bit queries");
  static_assert(G >= 1 && G <= 16, "group fits the 16-column tile");
  static_assert(MODE == M_PLAIN || MODE == M_PREFIX || MODE == M_SUFFIX, "mode");
  constexpr int GC = MODE == M_PREFIX ? PA_PREFIX_COLS : G;   // columns holding queries
  constexpr int NT = MODE == M_PREFIX ? PA_PREFIX_COLS / 16 : 1;   // 16-column tiles per chunk
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int EB = TyInfo<KV>::bytes;
  constexpr int KS = D / 32;              // score MFMA steps
  constexpr int VPL = D / 16;             // value elements per lane per token = P.V MFMAs
  constexpr int KDW = 8 * EB / 4;         // raw K dwords per lane per step
  constexpr int VDW = VPL * EB / 4;       // raw V dwords per lane per token
  // K loads: whole 128-byte lines where rows have them (see KLayout)
  constexpr bool KFULL = KLayout<D, EB>::FULL;
  constexpr int KR = KLayout<D, EB>::KR;           // K loads per chunk
  constexpr int KW = KLayout<D, EB>::KW;           // dwords per lane per K load
  auto kdim = [](int k, int a) { return kdim_t<D, EB>(k, a); };

  // [num_seqs + 1] chunk prefix sums; in the shared-prefix modes [num_seqs]
  // words (M_PREFIX: first sequence | sequences << 16 of the slot; M_SUFFIX:
  // the first chunk after the shared prefix); then [num_seqs] bytes: tokens
  // in each segment's last chunk (1..16), so a segment spans 16 (chunks - 1)
  // + tail tokens
  extern __shared__ int s_cum[];
  // per wave: the q B-operand of the piece being processed, [tile][step][lane]
  __shared__ uint4 s_q[NWM][NT][KS][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;                // row group
  const int n = lane & 15;                // column: head (scores) / dim slice (values)
  const int S = a.num_seqs;
  const int T = a.team;                   // waves per team = KV heads per head group
  const int HG = a.num_kv_heads / T;      // head groups
  uint32_t* const s_aux = reinterpret_cast<uint32_t*>(s_cum + S + 1);
  uint8_t* const s_tail = reinterpret_cast<uint8_t*>(s_cum + S + 1 + (MODE != M_PLAIN ? S : 0));

  // ---- chunk prefix sums over sequences (every workgroup, in LDS) ---------
  {
    int carry = 0;
    for (int base = 0; base < S; base += NWM * 64) {
      const int s = base + tid;
      int v = 0;
      if (s < S) {
        if constexpr (MODE == M_PREFIX) {
          // slot s: its sequences and the prefix they share (a multiple of
          // 16); a descriptor that does not fit the batch and table is idle
          const int4 sd = reinterpret_cast<const int4*>(a.share_desc)[s];
          const bool fits = sd.y >= 1 && sd.y <= GC / G && sd.x >= 0 && sd.x + sd.y <= S &&
                            sd.z > 0 && seq_chunks(a, sd.z) > 0 && (sd.z & (CH - 1)) == 0;
          v = fits ? sd.z / CH : 0;
          s_aux[s] = fits ? (uint32_t)sd.x | ((uint32_t)sd.y << 16) : 0u;
          s_tail[s] = (uint8_t)(v ? CH : 0);
        } else {
          const int ctx = a.context_lens[s];
          const bool ok = seq_chunks(a, ctx) > 0;
          int st0 = 0;                              // tokens already covered by a prefix
          if constexpr (MODE == M_SUFFIX) {
            st0 = own_start(a, s, ctx);
            s_aux[s] = (uint32_t)(st0 / CH);
          }
          v = ok ? (ctx - st0 + CH - 1) / CH : 0;
          s_tail[s] = (uint8_t)(v ? ctx - st0 - CH * (v - 1) : 0);
        }
      }
      // inclusive scan inside the workgroup: wave scan, then across waves
      int x = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      __shared__ int s_wsum[NWM];
      if (lane == 63) s_wsum[wave] = x;
      __syncthreads();
      int before = carry;
      for (int w = 0; w < wave; ++w) before += s_wsum[w];
      if (s < S) s_cum[s] = before + x - v;                   // exclusive
      int tot = 0;
      for (int w = 0; w < NWM; ++w) tot += s_wsum[w];
      carry += tot;
      __syncthreads();
    }
    if (tid == 0) s_cum[S] = carry;
    __syncthreads();
  }
  // rows of sequences with nothing to attend to: zeros for an empty context,
  // NaN for an invalid one (negative, beyond max_context_len or the table);
  // in M_SUFFIX a context that is all shared prefix is left to
  // shared_combine_kernel
  if constexpr (MODE != M_PREFIX) {
    for (int s = blk(); s < S; s += nblk()) {
      if (s_cum[s + 1] == s_cum[s]) {
        const int64_t base = (int64_t)s * a.num_q_heads * D;
        if (!(MODE == M_SUFFIX && s_aux[s] > 0)) {
          const float fill = a.context_lens[s] == 0 ? 0.f : __builtin_nanf("");
          for (int e = tid; e < a.num_q_heads * D; e += NWM * 64) store_out<QT>(a.out, base + e, fill);
        }
      }
    }
  }
  const int64_t CS = __builtin_amdgcn_readfirstlane(s_cum[S]);   // chunks per KV head
  const int64_t Cc = CS * HG;                                   // column chunks
  // (Cc == 0: every team's range is empty; each still records "nothing to
  // merge" below, so the merge never reads a stale descriptor)
  // XCD-contiguous wave numbering: workgroup b runs on XCD b % 8; give each
  // XCD one contiguous stretch of the column stream (nblk, and the first
  // workgroup of this part of the launch, are multiples of 8, and T divides
  // the 8 waves of a workgroup pair)
  const int per_xcd = nblk() / NXCD;
  const int vb = (blk() % NXCD) * per_xcd + blk() / NXCD;
  const int64_t w = (int64_t)vb * NWM + wave;
  const int64_t Wt = (int64_t)nblk() * NWM / T;                 // teams
  const int64_t team = w / T;
  const int ti = (int)(w - team * T);                           // KV head within the group

  // pools as bytes: element offsets (never negative) scale by EB, with no
  // signed division on the load path
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  auto dw = [](const char* p, int64_t e) __attribute__((always_inline)) {
    return reinterpret_cast<const uint32_t*>(p + e * EB);
  };
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.q);
  const int lg = a.log2_block_size;
  const int bmask = a.block_size - 1;
  const bool big_blocks = a.block_size >= CH;                   // one block per chunk
  const float qk_scale = a.qk_scale_log2;

  // ---- three-stage pipeline over this wave's ranges: the index stage walks
  // the column stream and fetches the block ids of chunk i+2, the load stage
  // issues the K/V loads of chunk i+1, the compute stage processes chunk i.
  // Segment = (sequence, head group), sequence-major; this wave's KV head in
  // it is hg * T + ti.
  struct Seg {
    int seq, hg, nc, ctx;           // ctx: the segment's end, as a token position
    int x;                          // M_PREFIX: slot word; M_SUFFIX: first chunk; else 0
  };
  // flags of a chunk in flight
  constexpr int F_VALID = 1;        // a real chunk (else a placeholder past the wave's last)
  constexpr int F_FIRST = 2;        // first chunk of a piece
  constexpr int F_LAST = 4;         // last chunk of a piece
  constexpr int F_BAD = 8;          // a bad block id was seen in the piece (set at its last chunk)
  struct Desc {
    int seq, hg, nc, ctx, j;        // segment and chunk (j: position / 16)
    int x;                          // Seg::x
    int f;                          // F_* flags
  };
  auto first_chunk = [](int x) { return MODE == M_SUFFIX ? x : 0; };
  auto seg_at = [&](int64_t cg, int& j) __attribute__((always_inline)) -> Seg {     // segment holding column chunk cg
    int lo = 0, hi = S - 1;                          // last s with s_cum[s] * HG <= cg
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)__builtin_amdgcn_readfirstlane(s_cum[mid]) * HG <= cg) lo = mid; else hi = mid - 1;
    }
    Seg sg;
    sg.seq = lo;
    sg.nc = __builtin_amdgcn_readfirstlane(s_cum[lo + 1] - s_cum[lo]);
    const int64_t rel = cg - (int64_t)__builtin_amdgcn_readfirstlane(s_cum[lo]) * HG;
    sg.hg = (int)(rel / sg.nc);
    j = (int)(rel - (int64_t)sg.hg * sg.nc);
    sg.x = MODE != M_PLAIN ? (int)__builtin_amdgcn_readfirstlane(s_aux[lo]) : 0;
    sg.ctx = CH * (first_chunk(sg.x) + sg.nc - 1) + __builtin_amdgcn_readfirstlane(s_tail[lo]);
    return sg;
  };

  // -- index stage state: next column ic of the team's range [.., ie)
  int64_t ic = team_begin(team, Cc, Wt);
  const int64_t ie = team_begin(team + 1, Cc, Wt);
  bool iact = ic < ie;                               // the index stage has chunks left
  if (ti == 0) {
    // merge descriptor of the team: the segment its range ends in, when that
    // segment starts in this range and continues past it: {last team it
    // reaches, sequence, head group, Cc when some team ranges are empty (Cc <
    // Wt) else 0}; else {-1}
    int4 md = make_int4(-1, 0, 0, 0);
    if (iact) {
      int j;
      const Seg sg = seg_at(ie - 1, j);
      const int64_t s0 = ie - 1 - j;                 // the segment's first column
      if (s0 >= ic && s0 + sg.nc > ie)
        md = make_int4((int)team_of(s0 + sg.nc - 1, Cc, Wt), sg.seq, sg.hg, Cc < Wt ? (int)Cc : 0);
    }
    if (lane == 0) reinterpret_cast<int4*>(a.ws_team)[team] = md;
  }
  if (!iact) return;
  int ij = 0;
  Seg is = seg_at(ic, ij);
  bool ifirst = true;                                // next indexed chunk starts a piece

  // Descriptor and block ids of the index stage's chunk; then advance. Lane
  // i fetches the id of the chunk's i-th block (lanes past its last block
  // repeat the last one); out-of-context entries are never read. Once the
  // wave's chunks are exhausted it yields placeholders and repeats its last
  // (in-bounds) id fetch, so every pipeline step issues the same loads.
  const int32_t* irow = a.block_tables;              // table row of the last indexed chunk
  int ifb = 0, ilb = 0;                              // its first and last block
  auto index_chunk = [&](Desc& d, int& idr) __attribute__((always_inline)) {
    // past the range: no flags, no tokens (processing it changes nothing)
    d.f = 0;
    d.x = 0;
    d.seq = d.hg = d.nc = d.ctx = d.j = 0;
    if (iact) {
      const int cb = (first_chunk(is.x) + ij) * CH;
      ifb = cb >> lg;
      ilb = (min(cb + CH, is.ctx) - 1) >> lg;
      // M_PREFIX: the slot's first sequence's table (its sequences share the
      // prefix blocks)
      const int trow = MODE == M_PREFIX ? (is.x & 0xffff) : is.seq;
      irow = a.block_tables + (int64_t)trow * a.max_blocks_per_seq;
      d.seq = is.seq;
      d.hg = is.hg;
      d.nc = is.nc;
      d.ctx = is.ctx;
      d.j = first_chunk(is.x) + ij;
      d.x = is.x;
      if constexpr (MODE != M_PLAIN) {
        // the team range of the segment, for shared_combine_kernel
        if (ij == 0 && ti == 0 && lane == 0)
          reinterpret_cast<int4*>(MODE == M_PREFIX ? a.share_seg : a.suf_seg)[(int64_t)is.seq * HG + is.hg] =
              make_int4((int)team, (int)team_of(ic + is.nc - 1, Cc, Wt), (int)Cc, (int)Wt);
      }
      ++ic;
      ++ij;
      const bool seg_end = ij == is.nc;
      const bool rng_end = ic == ie;
      d.f = F_VALID | (ifirst ? F_FIRST : 0) | ((seg_end || rng_end) ? F_LAST : 0);
      ifirst = seg_end || rng_end;
      if (rng_end) {
        iact = false;
      } else if (seg_end) {
        if (is.hg + 1 < HG) {
          ++is.hg;
        } else {
          is = seg_at(ic, ij);
        }
        ij = 0;
      }
    }
    idr = irow[min(ifb + lane, ilb)];
  };

  // q of this wave's KV head in chunk d's segment as the B operand (lane l:
  // column 16t + l%16 of tile t, dims 32k + 8(l/16) .. +8), fetched into qn
  // with a piece's first chunk and put into LDS at the start of the next
  // pipeline step, after the piece before it has been processed. Columns
  // past the G heads repeat a real head's row: their scores are masked out.
  // M_PREFIX: column c is head c%G of the slot's sequence c/G.
  uint32_t qn[NT][KS][4];
  bool qpend = false;
  auto load_q = [&](const Desc& d) __attribute__((always_inline)) {
    if ((d.f & (F_VALID | F_FIRST)) == (F_VALID | F_FIRST)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int col = 16 * t + n;
        int qseq = d.seq;
        if constexpr (MODE == M_PREFIX) qseq = (d.x & 0xffff) + min(col / G, (d.x >> 16) - 1);
        const int64_t row = ((int64_t)qseq * a.num_q_heads + (int64_t)(d.hg * T + ti) * G + (col % G)) * D;
#pragma unroll
        for (int k = 0; k < KS; ++k) ld<4>(qw + ((row + kdim(k, g)) >> 1), qn[t][k]);
      }
      qpend = true;
    }
  };
  auto flush_q = [&]() __attribute__((always_inline)) {
    if (qpend) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int k = 0; k < KS; ++k)
          s_q[wave][t][k][lane] = make_uint4(qn[t][k][0], qn[t][k][1], qn[t][k][2], qn[t][k][3]);
      qpend = false;
    }
  };

  // -- load stage: issue the K/V loads of chunk d (a placeholder reloads
  // the start of the pool)
  bool lbad = false;                                 // bad block id seen in the load piece
  auto load_chunk = [&](Desc& d, int idr, uint32_t (&kr)[KR][KW],
                        uint32_t (&vr)[4][VDW]) __attribute__((always_inline)) {
    const bool ok = d.f & F_VALID;
    const int ctx = ok ? d.ctx : 1;
    const int cb = ok ? d.j * CH : 0;
    const int fb = cb >> lg;
    const bool badl = idr < 0 || idr >= a.num_blocks;
    const bool bad = __any(badl);
    const int idv = (badl || !ok) ? 0 : idr;
    const int64_t head_off = ok ? a.layer_offset + (int64_t)(d.hg * T + ti) * a.block_size * D : 0;
    auto elem_of = [&](int t) __attribute__((always_inline)) -> int64_t {          // element of token t (< ctx), dim 0
      t = min(t, ctx - 1);
      const int id = big_blocks ? __builtin_amdgcn_readfirstlane(idv) : __shfl(idv, (t >> lg) - fb);
      return (int64_t)id * a.block_stride + head_off + (int64_t)(t & bmask) * D;
    };
    int64_t ek[KFULL ? 2 : 1], ev[4];
    if (big_blocks) {
      const int64_t base = elem_of(cb);                      // one block per chunk
      if constexpr (KFULL) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          ek[hf] = base + (int64_t)min(k_load_row<D, EB>(hf, lane), ctx - 1 - cb) * D + k_load_col<D, EB>(0, lane);
      } else {
        ek[0] = base + (int64_t)min(n, ctx - 1 - cb) * D + 8 * g;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ev[r] = base + (int64_t)min(4 * g + r, ctx - 1 - cb) * D + VPL * n;
    } else {
      if constexpr (KFULL) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) ek[hf] = elem_of(cb + k_load_row<D, EB>(hf, lane)) + k_load_col<D, EB>(0, lane);
      } else {
        ek[0] = elem_of(cb + n) + 8 * g;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ev[r] = elem_of(cb + 4 * g + r) + VPL * n;
    }
    if constexpr (KFULL) {
#pragma unroll
      for (int u = 0; u < KR; ++u) ld_stream<4>(dw(kpool, ek[u & 1] + (u >> 1) * (128 / EB)), kr[u]);
    } else {
#pragma unroll
      for (int k = 0; k < KS; ++k) ld_stream<KDW>(dw(kpool, ek[0] + 32 * k), kr[k]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) ld_stream<VDW>(dw(vpool, ev[r]), vr[r]);
    if (ok) {
      lbad = lbad || bad;
      if (lbad && (d.f & F_LAST)) d.f |= F_BAD;
      if (d.f & F_LAST) lbad = false;
    }
  };

  // ---- compute stage state of the current piece, per column tile
  int pj0 = 0;                                       // first chunk of the piece
  f32x4_t acc[NT][VPL];
  float m_ref[NT], l_sum[NT];                        // reference max of column n (log2 units),
                                                     // this lane's probability sum
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int m = 0; m < VPL; ++m) acc[t][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    m_ref[t] = -__builtin_inff();
    l_sum[t] = 0.f;
  }

  // Write the piece that ends with chunk d (final rows or a partial) and
  // reset the state.
  auto finish_piece = [&](const Desc& d) __attribute__((always_inline)) {
    const bool bad = d.f & F_BAD;
    const int j0 = first_chunk(d.x);
    const bool whole = (pj0 == j0) && (d.j + 1 == j0 + d.nc);
    const int kvh = d.hg * T + ti;
    const int64_t out_row0 = ((int64_t)d.seq * a.num_q_heads + (int64_t)kvh * G) * D;
    const int64_t cseg = (int64_t)d.seq * HG + d.hg;
    const int ncol = MODE == M_PREFIX ? G * (d.x >> 16) : G;   // columns holding queries
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float lt = l_sum[t] + __shfl_xor(l_sum[t], 16);
      lt += __shfl_xor(lt, 32);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * g + r;                    // accumulator row = column of the tile
        const int col = 16 * t + h;
        const float lh = __shfl(lt, h);
        const float mh = __shfl(m_ref[t], h);
        if (col < ncol) {
          if (MODE == M_SUFFIX && whole && d.x > 0) {
            // a sequence with a shared prefix: the partial of its own
            // tokens, to which shared_combine_kernel adds the prefix
            const int64_t prow = (int64_t)d.seq * a.num_q_heads + (int64_t)kvh * G + col;
            float* po = a.pre_o + prow * D + VPL * n;
#pragma unroll
            for (int m = 0; m < VPL; ++m) po[m] = bad ? __builtin_nanf("") : acc[t][m][r];
            if (n == 0) {
              a.pre_m[prow] = bad ? 0.f : mh;
              a.pre_l[prow] = bad ? __builtin_nanf("") : lh;
            }
          } else if (whole && MODE != M_PREFIX) {
            const float norm = bad ? __builtin_nanf("") : a.v_scale / lh;
            const int64_t o = out_row0 + (int64_t)col * D + VPL * n;
#pragma unroll
            for (int m = 0; m < VPL; ++m) store_out<QT>(a.out, o + m, acc[t][m][r] * norm);
          } else {
            const int64_t slot = ((team + cseg) * T + ti) * GC + col;
            float* wo = a.ws_o + slot * D + VPL * n;
#pragma unroll
            for (int m = 0; m < VPL; ++m) wo[m] = bad ? __builtin_nanf("") : acc[t][m][r];
            if (n == 0) {
              a.ws_m[slot] = bad ? 0.f : mh;
              a.ws_l[slot] = bad ? __builtin_nanf("") : lh;
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < VPL; ++m) acc[t][m] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      m_ref[t] = -__builtin_inff();
      l_sum[t] = 0.f;
    }
  };

  auto process_chunk = [&](const uint32_t (&kr)[KR][KW], const uint32_t (&vr)[4][VDW],
                           const Desc& d) __attribute__((always_inline)) {
    if (d.f & F_FIRST) pj0 = d.j;
    const int ctx = d.ctx;
    const int cb = d.j * CH;
    const bool tail = cb + CH > ctx;
    bool live[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) live[r] = !tail || cb + 4 * g + r < ctx;
    const int ncol = MODE == M_PREFIX ? G * (d.x >> 16) : G;
    if constexpr (NT == 1) {
      const f32x4_t s = chunk_scores<KV, QT, D>(kr, [&](int k) { return s_q[wave][0][k][lane]; }, lane);
      float z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = n < ncol && cb + 4 * g + r < ctx;
        z[r] = valid ? s[r] * qk_scale : -__builtin_inff();
      }
      chunk_softmax_pv<KV, QT, D>(z, vr, live, acc[0], m_ref[0], l_sum[0], lane);
    } else {
      // several column tiles: the chunk's K and V operands are built once
      uint32_t kraw[KS][KLayout<D, EB>::KDW];
      k_operand<D, EB>(kr, kraw, lane);
      uint32_t vb[VPL][2];
      if constexpr (KV == Ty::FP8) {
        pv_operands_fp8<D>(vr, live, vb);
      } else {
        uint32_t vw[4][D / 32];
        v_operand<KV, QT, D>(vr, live, vw);
        pv_operands<D>(vw, vb);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const f32x4_t s = chunk_scores_raw<KV, QT, D>(kraw, [&](int k) { return s_q[wave][t][k][lane]; });
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool valid = 16 * t + n < ncol && cb + 4 * g + r < ctx;
          z[r] = valid ? s[r] * qk_scale : -__builtin_inff();
        }
        softmax_pv_b<KV, QT, D>(z, vb, acc[t], m_ref[t], l_sum[t], lane);
      }
    }
    if (d.f & F_LAST) finish_piece(d);
  };

  // ---- the pipeline. Chunks alternate between buffers A and B; a chunk's
  // block ids live in the id register of its buffer from indexing to
  // loading. Each step: q of the previous step's new piece goes to LDS; q of
  // chunk i+1 is fetched if it starts a piece (the only conditional load,
  // issued first so that it cannot shorten the waits that follow); the ids
  // of chunk i+2 and the K/V of chunk i+1 are fetched; chunk i is processed.
  // The waits before processing leave every load of the step in flight.
  // The loop leaves only after a B step: a chunk past the end is processed
  // as a no-op (every score masked, no piece flags). A leave after the A
  // step would reach the loop latch with B's loads unread (the compiler
  // gives a loop with divergent branches a single exit through its latch),
  // and the wait analysis would then drain A's loads at the top of every
  // step before reusing B's registers: one chunk in flight instead of two.
  uint32_t kA[KR][KW], vA[4][VDW], kB[KR][KW], vB[4][VDW];
  Desc dA, dB;                                       // chunk in (or bound for) each buffer
  int iA = 0, iB = 0;
  index_chunk(dA, iA);
  load_q(dA);
  index_chunk(dB, iB);
  load_chunk(dA, iA, kA, vA);
  while (true) {
    Desc dn;
    flush_q();
    load_q(dB);
    index_chunk(dn, iA);
    load_chunk(dB, iB, kB, vB);
    process_chunk(kA, vA, dA);                       // always a chunk of the range
    dA = dn;
    flush_q();
    load_q(dA);
    index_chunk(dn, iB);
    load_chunk(dA, iA, kA, vA);
    process_chunk(kB, vB, dB);                       // past the end: no effect
    if (!(dA.f & F_VALID)) return;                   // (dB past the end implies dA too)
    dB = dn;
  }
}

template <Ty KV, Ty QT, int D, int G, int MODE>
__global__ void __launch_bounds__(NWM * 64)
__attribute__((amdgpu_waves_per_eu(sk_waves_per_simd<KV, D, G, MODE>())))
attend_sk_kernel(const DecodeParams a) {
  attend_sk_body<KV, QT, D, G, MODE, false>(a, 0, 0);
}

// The shared-prefix decode's two passes in one launch: the first pre
// workgroups run the prefix pass (parameters p), the others the suffix pass
// (parameters q), at the same time. Neither reads what the other writes:
// the suffix pass leaves the result of a sequence that has a prefix as a
// partial, and shared_combine_kernel adds the prefix afterwards. The split
// follows the plan's totals: the prefix chunks of the slots (cp) and each
// sequence's own chunks (cs); the prefix pass gets nblk * cp / (cp + 2 cs)
// workgroups (a prefix chunk weighs half an own chunk: it is read once for
// a whole slot, while the short own segments run below streaming speed),
// in whole rounds of the XCDs; none without prefixes, and at least one
// round for each pass otherwise. (32 prompts x 8 samples, 1,024 prompt
// tokens and 64-256 own: about a quarter, which measured best among fixed
// fractions.)
template <Ty KV, Ty QT, int D, int G>
__global__ void __launch_bounds__(NWM * 64)
__attribute__((amdgpu_waves_per_eu(sk_waves_per_simd<KV, D, G, M_PREFIX>())))
attend_sk_dual_kernel(const DecodeParams p, const DecodeParams q) {
  // (totals of a stale plan only steer the split; any split is correct)
  const float tp = (float)max(__builtin_amdgcn_readfirstlane(p.share_tot[0]), 0);
  const float ts = (float)max(__builtin_amdgcn_readfirstlane(p.share_tot[1]), 0);
  const int nb = gridDim.x;                   // a multiple of 8, at least 16
  int pre = 0;
  if (tp > 0.f) {
    const int x = (int)((float)nb * tp / (tp + 2.f * ts)) / NXCD * NXCD;
    pre = min(max(x, NXCD), nb - NXCD);
  }
  pre = __builtin_amdgcn_readfirstlane(pre);   // the same in every lane: keep the parts' indices scalar
  if ((int)blockIdx.x < pre)
    attend_sk_body<KV, QT, D, G, M_PREFIX, true>(p, blockIdx.x, pre);
  else
    attend_sk_body<KV, QT, D, G, M_SUFFIX, true>(q, blockIdx.x - pre, nb - pre);
}

// Merge of segments cut by team range boundaries: M = max_p m_p,
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p. Workgroup (t, i)
// merges KV head i of the group of the segment recorded by team t (if any),
// over its pieces from teams t .. t1 (the last team the segment reaches).
// Threads form PG groups, each covering all GC x D outputs (DPT dims per
// thread) over every PG-th piece with a running (online) combination; the
// groups are combined in LDS. NT threads: 256, or 64 (one group, no LDS
// step, a quarter of the waves to dispatch) when segments average under 4
// pieces, as in batches of many sequences.
// SPLITH: one query head per workgroup (grid z), so a few long segments
// spread over G times the workgroups, each with G times the piece groups.
// (The shared-prefix decode's passes are finished by shared_combine_kernel.)
template <Ty QT, int D, int G, int MODE, int NT = 256, bool BYSEG = false, bool SPLITH = false>
__global__ void __launch_bounds__(NT)
merge_sk_kernel(const DecodeParams a, int64_t W) {
  static_assert(MODE == M_PLAIN, "the shared-prefix passes are finished by shared_combine_kernel");
  static_assert(!SPLITH || BYSEG, "one query head per workgroup: segment-indexed merge only");
  constexpr int GC = SPLITH ? 1 : G;                   // query heads per workgroup
  constexpr int GD = GC * D;
  constexpr int DPT = GD >= 1024 ? 16 : (GD >= 512 ? 8 : 4);   // dims per thread
  constexpr int NV4 = DPT / 4;
  constexpr int TPG = GD / DPT;                        // threads per group
  static_assert(TPG <= NT && NT % TPG == 0, "group size");
  constexpr int PG = NT / TPG;                         // piece groups
  __shared__ float s_m[PG][GC], s_l[PG][GC];
  __shared__ float s_o[PG > 1 ? PG : 1][GD];

  static_assert(!BYSEG || MODE == M_PLAIN, "segment-indexed merge of the plain decode only");
  const int ti = blockIdx.y;
  const int T = a.team;
  const int HG = a.num_kv_heads / T;
  const int64_t Wt = W / T;
  int64_t t0, t1, Cs;
  int seq, hg;
  if constexpr (BYSEG) {
    // workgroup x merges segment x (sequence x / HG, head group x % HG) of
    // a batch of at most 64 sequences: every wave counts the sequences'
    // chunks as the attention kernel does and finds the teams holding the
    // segment's first and last columns (segments lie end to end,
    // sequence-major)
    seq = (int)(blockIdx.x / HG);
    hg = (int)(blockIdx.x - (unsigned)seq * HG);
    const int lane = threadIdx.x & 63;
    const int v = lane < a.num_seqs ? seq_chunks(a, a.context_lens[lane]) : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    const int nc = __shfl(v, seq);
    if (nc == 0) return;                               // nothing to attend to (uniform)
    const int64_t Cc = (int64_t)__shfl(x, 63) * HG;
    const int64_t c0 = (int64_t)(__shfl(x, seq) - nc) * HG + (int64_t)hg * nc;
    t0 = team_of(c0, Cc, Wt);
    t1 = team_of(c0 + nc - 1, Cc, Wt);
    if (t1 <= t0) return;                              // one team: written by the attention kernel
    Cs = Cc < Wt ? Cc : 0;
  } else {
    t0 = blockIdx.x;
    const int4 md = reinterpret_cast<const int4*>(a.ws_team)[t0];
    t1 = md.x;
    if (t1 <= t0) return;                              // no segment to merge here
    seq = md.y;
    hg = md.z;
    Cs = md.w;                                         // nonzero: some team ranges are empty
    // a descriptor the attention launch did not write (a merge launched with
    // other sizes than it) is dropped rather than followed out of range
    if (t1 >= Wt || seq < 0 || seq >= a.num_seqs || hg < 0 || hg >= HG || Cs < 0 || Cs >= Wt)
      return;
  }
  const int kvh = hg * T + ti;
  const int tid = threadIdx.x;
  const int grp = tid / TPG;
  const int t = tid - grp * TPG;
  const int hl = t / (D / DPT);                        // head within the workgroup's
  const int h = hl + (SPLITH ? (int)blockIdx.z : 0);   // head within the KV head's group
  const int d0 = (t - hl * (D / DPT)) * DPT;
  const int64_t orow = ((int64_t)seq * a.num_q_heads + (int64_t)kvh * G + h) * D + d0;
  const int64_t cseg = (int64_t)seq * HG + hg;

  float M = -__builtin_inff(), L = 0.f, O[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) O[e] = 0.f;
  auto combine = [&](float m, float l, const float4* o) {
    const float mn = fmaxf(M, m);
    if (mn == -__builtin_inff()) return;
    const float f1 = __builtin_amdgcn_exp2f(M - mn);   // 0 when M = -inf
    const float f2 = __builtin_amdgcn_exp2f(m - mn);
    L = L * f1 + l * f2;
#pragma unroll
    for (int v = 0; v < NV4; ++v) {
      O[4 * v + 0] = O[4 * v + 0] * f1 + o[v].x * f2;
      O[4 * v + 1] = O[4 * v + 1] * f1 + o[v].y * f2;
      O[4 * v + 2] = O[4 * v + 2] * f1 + o[v].z * f2;
      O[4 * v + 3] = O[4 * v + 3] * f1 + o[v].w * f2;
    }
    M = mn;
  };
  // pieces of teams t0 + grp, t0 + grp + PG, ...; U pieces per round per
  // group (every nonempty team in t0 .. t1 holds a piece: the segment covers
  // it). The 256-thread form, which takes the long segments, issues the next
  // round's loads before this round is combined; every round loads (a lane
  // past the segment's last piece reads team t0's piece, always written, and
  // drops it), so the waits never cover the next round. The 64-thread form's
  // segments have a round or two: it loads and combines round by round.
  constexpr int U = 4;
  const int64_t safe = ((t0 + cseg) * T + ti) * G + h;
  auto fetch = [&](int64_t tb, float (&mv)[U], float (&lv)[U], float4 (&ov)[U][NV4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tm = tb + (int64_t)u * PG;
      const bool ok = tm <= t1 && (Cs == 0 || team_begin(tm, Cs, Wt) != team_begin(tm + 1, Cs, Wt));
      const int64_t slot = ok ? ((tm + cseg) * T + ti) * G + h : safe;
      const float m = a.ws_m[slot], l = a.ws_l[slot];
      mv[u] = ok ? m : -__builtin_inff();
      lv[u] = ok ? l : 0.f;
#pragma unroll
      for (int v = 0; v < NV4; ++v) {
        const float4 o = reinterpret_cast<const float4*>(a.ws_o + slot * D + d0)[v];
        ov[u][v] = ok ? o : make_float4(0, 0, 0, 0);
      }
    }
  };
  if constexpr (NT == 64) {
    for (int64_t tb = t0 + grp; tb <= t1; tb += (int64_t)PG * U) {
      float mv[U], lv[U];
      float4 ov[U][NV4];
      fetch(tb, mv, lv, ov);
#pragma unroll
      for (int u = 0; u < U; ++u) combine(mv[u], lv[u], ov[u]);
    }
  } else {
  float mA[U], lA[U], mB[U], lB[U];
  float4 oA[U][NV4], oB[U][NV4];
  int64_t tb = t0 + grp;
  fetch(tb, mA, lA, oA);
  while (tb <= t1) {
    fetch(tb + (int64_t)PG * U, mB, lB, oB);
#pragma unroll
    for (int u = 0; u < U; ++u) combine(mA[u], lA[u], oA[u]);
    tb += (int64_t)PG * U;
    if (tb > t1) break;
    fetch(tb + (int64_t)PG * U, mA, lA, oA);
#pragma unroll
    for (int u = 0; u < U; ++u) combine(mB[u], lB[u], oB[u]);
    tb += (int64_t)PG * U;
  }
  }
  if constexpr (PG > 1) {
    if (d0 == 0) { s_m[grp][hl] = M; s_l[grp][hl] = L; }
#pragma unroll
    for (int e = 0; e < DPT; ++e) s_o[grp][hl * D + d0 + e] = O[e];
    __syncthreads();
    if (grp != 0) return;
    M = -__builtin_inff(); L = 0.f;
#pragma unroll
    for (int e = 0; e < DPT; ++e) O[e] = 0.f;
#pragma unroll
    for (int q = 0; q < PG; ++q)
      combine(s_m[q][hl], s_l[q][hl], reinterpret_cast<const float4*>(&s_o[q][hl * D + d0]));
  }
  const float norm = a.v_scale / L;
#pragma unroll
  for (int e = 0; e < DPT; ++e) store_out<QT>(a.out, orow + e, O[e] * norm);
}

// ---------------------------------------------------------------------------
// Launch side, templated on the mode. The shared-prefix modes exist for the
// group sizes the C ABI takes (1, 2, 4, 8).
template <Ty KV, Ty QT, int D, int G, int MODE>
static hipError_t sk_launch_t(const DecodeParams& a, int blocks, hipStream_t st) {
  const size_t lds = sk_lds_bytes(a.num_seqs, MODE);
  hipLaunchKernelGGL((attend_sk_kernel<KV, QT, D, G, MODE>), dim3(blocks), dim3(NWM * 64), lds, st, a);
  return hipGetLastError();
}

template <Ty KV, Ty QT, int D, int MODE>
static hipError_t sk_launch_g(const DecodeParams& a, int g, int blocks, hipStream_t st) {
  switch (g) {
    case 1: return sk_launch_t<KV, QT, D, 1, MODE>(a, blocks, st);
    case 2: return sk_launch_t<KV, QT, D, 2, MODE>(a, blocks, st);
    case 4: return sk_launch_t<KV, QT, D, 4, MODE>(a, blocks, st);
    case 8: return sk_launch_t<KV, QT, D, 8, MODE>(a, blocks, st);
    case 16:
      if constexpr (MODE == M_PLAIN) return sk_launch_t<KV, QT, D, 16, MODE>(a, blocks, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <Ty KV, Ty QT, int MODE>
static hipError_t sk_launch_d(const DecodeParams& a, int g, int blocks, hipStream_t st) {
  if (a.head_dim == 64) return sk_launch_g<KV, QT, 64, MODE>(a, g, blocks, st);
  if (a.head_dim == 128) return sk_launch_g<KV, QT, 128, MODE>(a, g, blocks, st);
  return hipErrorInvalidValue;
}

template <int MODE>
static hipError_t sk_launch_attend(const DecodeParams& a, int kv_ty, int q_ty, int g, int blocks,
                                   hipStream_t st) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  if (kv == Ty::BF16 && q == Ty::BF16) return sk_launch_d<Ty::BF16, Ty::BF16, MODE>(a, g, blocks, st);
  if (kv == Ty::F16 && q == Ty::F16) return sk_launch_d<Ty::F16, Ty::F16, MODE>(a, g, blocks, st);
  if (kv == Ty::FP8 && q == Ty::BF16) return sk_launch_d<Ty::FP8, Ty::BF16, MODE>(a, g, blocks, st);
  if (kv == Ty::FP8 && q == Ty::F16) return sk_launch_d<Ty::FP8, Ty::F16, MODE>(a, g, blocks, st);
  return hipErrorInvalidValue;
}

// Workgroups to launch: exactly the number that are resident at once (every
// wave's range is processed concurrently), a multiple of the XCD count.
// More resident workgroups than the compiled target adds no bandwidth (the
// slab reads already keep the memory system full at that occupancy) and only
// shortens each wave's range, raising the merge's share of the work.
static int sk_resident_blocks(const void* kernel, size_t lds, int target) {
  int dev = 0, cus = 256, per_cu = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NWM * 64, lds) != hipSuccess)
      per_cu = 0;
  }
  if (per_cu <= 0 || per_cu > target) per_cu = target;
  const int b = cus * per_cu;
  return b >= NXCD ? b / NXCD * NXCD : NXCD;
}

template <Ty KV, Ty QT, int D, int G, int MODE>
static int sk_blocks_t(int num_seqs) {
  return sk_resident_blocks(reinterpret_cast<const void*>(&attend_sk_kernel<KV, QT, D, G, MODE>),
                            sk_lds_bytes(num_seqs, MODE), sk_waves_per_simd<KV, D, G, MODE>());
}

template <Ty KV, Ty QT, int D, int MODE>
static int sk_blocks_g(int g, int num_seqs) {
  switch (g) {
    case 1: return sk_blocks_t<KV, QT, D, 1, MODE>(num_seqs);
    case 2: return sk_blocks_t<KV, QT, D, 2, MODE>(num_seqs);
    case 4: return sk_blocks_t<KV, QT, D, 4, MODE>(num_seqs);
    case 8: return sk_blocks_t<KV, QT, D, 8, MODE>(num_seqs);
    default:
      if constexpr (MODE == M_PLAIN) return sk_blocks_t<KV, QT, D, 16, MODE>(num_seqs);
      return 0;
  }
}

template <int MODE>
static int sk_blocks_mode(int kv_ty, int q_ty, int head_dim, int g, int num_seqs) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  auto by_d = [&](auto kvt, auto qt) {
    constexpr Ty K = decltype(kvt)::value, Q = decltype(qt)::value;
    return head_dim == 64 ? sk_blocks_g<K, Q, 64, MODE>(g, num_seqs)
                          : sk_blocks_g<K, Q, 128, MODE>(g, num_seqs);
  };
  using BF = std::integral_constant<Ty, Ty::BF16>;
  using HF = std::integral_constant<Ty, Ty::F16>;
  using F8 = std::integral_constant<Ty, Ty::FP8>;
  if (kv == Ty::BF16) return by_d(BF{}, BF{});
  if (kv == Ty::F16) return by_d(HF{}, HF{});
  if (q == Ty::F16) return by_d(F8{}, HF{});
  return by_d(F8{}, BF{});
}

template <Ty QT, int D, int G, int MODE>
static void sk_launch_merge_t(const DecodeParams& a, int64_t W, bool lean, hipStream_t st) {
  const dim3 grid((unsigned)(W / a.team), (unsigned)a.team);
  const int64_t segs = (int64_t)a.num_seqs * (a.num_kv_heads / a.team);
  if constexpr (MODE == M_PLAIN) {
    // few, long segments: one workgroup per (segment, KV head, query head)
    // instead of one per (team, KV head), almost all of which would find
    // nothing
    if (a.num_seqs <= 64 && segs > 0 && W / a.team >= 16 * segs) {
      hipLaunchKernelGGL((merge_sk_kernel<QT, D, G, MODE, 256, true, true>),
                         dim3((unsigned)segs, (unsigned)a.team, G), dim3(256), 0, st, a, W);
      return;
    }
  }
  if (lean)
    hipLaunchKernelGGL((merge_sk_kernel<QT, D, G, MODE, 64>), grid, dim3(64), 0, st, a, W);
  else
    hipLaunchKernelGGL((merge_sk_kernel<QT, D, G, MODE, 256>), grid, dim3(256), 0, st, a, W);
}

template <Ty QT, int D, int MODE>
static hipError_t sk_launch_merge_d(const DecodeParams& a, int64_t W, int g, hipStream_t st) {
  dim3 grid((unsigned)(W / a.team), (unsigned)a.team);
  const int64_t segs = (int64_t)a.num_seqs * (a.num_kv_heads / a.team);
  const bool lean = W / a.team < 4 * segs;            // segments average under 4 pieces
  switch (g) {
    case 1: sk_launch_merge_t<QT, D, 1, MODE>(a, W, lean, st); break;
    case 2: sk_launch_merge_t<QT, D, 2, MODE>(a, W, lean, st); break;
    case 4: sk_launch_merge_t<QT, D, 4, MODE>(a, W, lean, st); break;
    case 8: sk_launch_merge_t<QT, D, 8, MODE>(a, W, lean, st); break;
    case 16:
      if constexpr (MODE == M_PLAIN) {
        hipLaunchKernelGGL((merge_sk_kernel<QT, D, 16, MODE>), grid, dim3(256), 0, st, a, W);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t sk_launch_merge(const DecodeParams& a, int q_ty, int g, int blocks, hipStream_t st) {
  const int64_t W = (int64_t)blocks * NWM;
  auto by_d = [&](auto qt) {
    constexpr Ty Q = decltype(qt)::value;
    if (a.head_dim == 64) return sk_launch_merge_d<Q, 64, MODE>(a, W, g, st);
    if (a.head_dim == 128) return sk_launch_merge_d<Q, 128, MODE>(a, W, g, st);
    return hipErrorInvalidValue;
  };
  switch ((Ty)q_ty) {
    case Ty::BF16: return by_d(std::integral_constant<Ty, Ty::BF16>{});
    case Ty::F16: return by_d(std::integral_constant<Ty, Ty::F16>{});
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
