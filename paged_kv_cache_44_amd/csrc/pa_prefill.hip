// pa_prefill.hip — paged prefill (whole, chunked, or recompute) attention on
// the gfx950 matrix cores: causal attention of each sequence's newest
// positions over the keys and values of all its positions, reached through
// its block table.
//
// A recomputed request runs its prompt and generated tokens again as one
// prefill pass ("When KV Capacity Runs Out", section "Recompute KV from token
// history"); the pass's keys and values are first written to the pool, then
// every position p attends to positions 0 .. p. Query rows are packed
// sequence by sequence (query_start_loc); the n_s rows of sequence s are its
// positions ctx_s - n_s .. ctx_s - 1.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

#include <type_traits>

namespace pa {
namespace {

// ---------------------------------------------------------------------------
// Tiled prefill: each workgroup takes 128 query rows of one (sequence, KV
// head) -- 128 / G consecutive positions x the G query heads -- 32 rows per
// wave, and walks the keys of the causal range in tiles of FKT = 32 or 64
// keys. The four waves stage each tile once in LDS, gathered through the
// block table, double buffered, one barrier per tile. 16-bit pools are
// staged by the memory unit straight into LDS (global_load_lds_dwordx4),
// K and V as key rows, from wave-uniform base addresses when a block holds
// all the rows of one such instruction; FP8 pools go through registers,
// their codes widened exactly to the query's 16-bit type, K as rows and V
// transposed (a row per dim). After the walk the normalised rows pass
// through LDS, so that they leave as whole 16-byte pieces. Both products
// run on the 32x32x16 matrix cores, transposed so that a query row owns a
// lane pair:
//   S^T[FKT keys][32 rows] = K[FKT][D] . Q^T[D][32]    (A = K rows from LDS)
//   O^T[D][32 rows]      += V^T[D][FKT] . P^T[FKT][32] (A = V^T rows from LDS,
//                                                       B = P from registers)
// Lane l holds row l % 32 in the columns of both outputs (the other half of
// each 32 keys, or of the dims, in lane l ^ 32), so the row's softmax state,
// maximum, sum, rescale and normalisation never leave the lane pair. The
// k-slots of P^T's operand follow the score tile's own key order (lane half h
// holds keys 4h + j and 8 + 4h + j of each 16). From key rows, each V^T
// operand is two transposing LDS reads (ds_read_b64_tr_b16: within 16 lanes,
// lane 4j + a reads 4 dims of key j and lane 4a + b receives one dim of 4
// keys); from transposed FP8 staging, V^T is laid out with its keys in that
// order, one 16-byte LDS read per operand.
constexpr int NXCD_PF = 8;        // XCDs of an MI355X
// (sequence, KV head) pairs dealt round-robin over the XCDs: when the KV
// heads are a multiple of the XCDs, so that each XCD gets the same share of
// every sequence
__host__ __device__ inline bool pf_round_robin(int num_kv_heads) {
  return num_kv_heads % NXCD_PF == 0;
}
constexpr int FW = 4;             // waves per workgroup
constexpr int FR = 32;            // query rows per wave
// score of a masked key: finite, so exp2(score * c - m) is exactly 0 without
// a select for any c > 0 and any reference m reached by a real score
constexpr float MASKED = -3.0e38f;

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short tr16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <Op O>
__device__ __forceinline__ f32x16_t mfma32(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x16_t c) {
  const u32x4_t av = {a[0], a[1], a[2], a[3]}, bv = {b[0], b[1], b[2], b[3]};
  if constexpr (O == Op::BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                    __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, av),
                                                   __builtin_bit_cast(f16x8_t, bv), c, 0, 0, 0);
}

// sum of a packed pair of 16-bit values, added to acc
template <Op O>
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
  if constexpr (O == Op::BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w), __builtin_bit_cast(half2_t, 0x3c003c00u),
                                  acc, false);
}

// maximum of x over lanes l and l ^ 32: with both operands equal, the
// half swap leaves each lane its own value in one result and its partner's
// in the other (a VALU exchange, no LDS round trip)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 16 bytes per lane from global memory straight into LDS, lane i's at LDS
// byte offset lds_off + 16 i (the memory unit writes LDS; no registers).
// Issued from asm so that the compiler does not hold every later LDS read
// (of the other buffer) behind it; callers wait for vmcnt to reach 0 before
// the barrier that publishes the tile. No outputs; m0 is set here (one wait
// state before the load reads it).
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_off) : "memory", "m0");
}

// The same from a wave-uniform base address (scalar registers) plus the
// lane's 32-bit byte offset.
__device__ __forceinline__ void lds_dma16_s(const void* base, uint32_t off, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(lds_off) : "memory", "m0");
}

// 16 bytes from LDS byte address addr.
__device__ __forceinline__ uint4 lds_ld16(uint32_t addr) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = *(const __attribute__((address_space(3))) u32x4_t*)(uintptr_t)addr;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Position of key kk (0..15 in a 16-key block) in the staged V^T rows: bits
// 2 and 3 swapped, so that lane half h's 8 keys (4h + j, 8 + 4h + j) are
// contiguous at 8h.
__device__ __forceinline__ int vt_slot(int kk) {
  return (kk & 3) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// LDS of one tile, double buffered. Register-staged (FP8 pools, widened on
// the way): K rows padded by 16 bytes, V transposed (a row per dim).
// Staged straight from memory (16-bit pools): K and V as unpadded key rows,
// their 16-byte chunks permuted per row (see prefill_tiled_kernel).
template <int D, int FKT, bool DIRECT>
struct FaLds {
  static constexpr int PK = DIRECT ? D * 2 : D * 2 + 16;   // bytes per staged K row (a key)
  static constexpr int PV = FKT * 2 + 16;                  // bytes per staged V^T row (a dim)
  static constexpr int KT = FKT * PK;
  static constexpr int VT = DIRECT ? FKT * D * 2 : D * PV;
  static constexpr int BUF = KT + VT;
  static constexpr int BYTES = 2 * BUF;
};

// Keys per tile, and occupancy: 32-key tiles fit 3 waves per SIMD (at most
// 168 registers and 33-37 KB of LDS at D = 128), which hides more latency when
// the grid has many workgroups; 64-key tiles run at 2 and halve the barriers
// and per-tile work of each workgroup, which wins when there are few (a
// single long recompute).
template <int FKT>
constexpr int pf_waves_per_simd() { return FKT == 32 ? 3 : 2; }

// UB (16-bit pools, block_size >= the RPI rows one staging instruction
// moves): each instruction's rows are consecutive keys of one block, so its
// block id and base address are wave-uniform and computed in scalar registers.
template <Ty KV, Ty QT, int D, int G, int FKT, bool UB>
__global__ void __launch_bounds__(FW * 64)
__attribute__((amdgpu_waves_per_eu(pf_waves_per_simd<FKT>())))
prefill_tiled_kernel(const PrefillParams a) {
  static_assert(QT == Ty::BF16 || QT == Ty::F16, "16-bit queries");
  static_assert(G >= 1 && G <= 16 && 16 % G == 0, "group divides the 16-column tile");
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr Op OP = QT == Ty::F16 ? Op::F16 : Op::BF16;   // both products in the query's type
  constexpr int EB = TyInfo<KV>::bytes;
  constexpr int KSTEPS = D / 16;                  // score products per 32 keys
  constexpr int NB = D / 32;                      // output dim blocks = P.V products per 16 keys
  constexpr int TPOS = FW * FR / G;               // positions per workgroup
  constexpr int CD = 16 / EB;                     // dims per 16-byte pool chunk
  constexpr int CPR = D / CD;                     // chunks per key row
  constexpr int NSB = FKT / 32;                   // score blocks of 32 keys per tile
  constexpr int NKB = FKT / 16;                   // key blocks of 16 per tile
  constexpr int JOBS = FKT * CPR;                 // register staging jobs per tile: (key, chunk)
  constexpr int NJ = (JOBS + FW * 64 - 1) / (FW * 64);   // jobs per thread
  static_assert(FKT == 32 || FKT == 64, "keys per tile");
  // 16-bit pools are staged by the memory unit straight into LDS (no
  // registers, no LDS writes): a wave instruction moves 64 x 16 bytes to
  // 1 KiB of consecutive LDS, RPI key rows of ROWB bytes. In row r, LDS
  // chunk position p holds K's 16-byte chunk p ^ (r mod R16) (so the 16
  // rows a score operand read touches hit distinct banks) and V's chunk
  // p ^ 4 (r mod SEGS) (whole 64-byte segments permuted, so the eight rows
  // of a transposing read fall on different banks in pairs at most).
  constexpr bool DIRECT = EB == 2;
  constexpr int ROWB = D * 2;                     // bytes per key row
  constexpr int R16 = ROWB / 16;                  // 16-byte chunks per row
  constexpr int SEGS = ROWB / 64;                 // 64-byte segments per row
  constexpr int RPI = 1024 / ROWB;                // rows per wave instruction
  constexpr int NIW = FKT / (RPI * FW);           // instructions per wave per tile (each of K, V)
  static_assert(!DIRECT || FKT % (RPI * FW) == 0, "tile rows split evenly over the waves");
  static_assert(DIRECT || !UB, "uniform staging bases: 16-bit pools only");
  constexpr int NID = DIRECT ? NIW : NJ;          // block ids a thread fetches per tile
  using L = FaLds<D, FKT, DIRECT>;
  __shared__ __attribute__((aligned(1024))) char lds[L::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;                        // row of the wave (output column)
  const int h = lane >> 5;                        // lane half: keys / dims it holds
  const int H = a.num_kv_heads;
  // Workgroup numbering: workgroup b runs on XCD b % 8, as its (b / 8)-th.
  // An XCD takes every row tile of one (sequence, KV head) pair in turn,
  // longest causal range first, so the tiles that stream the same keys and
  // values run together and share them in that XCD's L2. With a multiple
  // of 8 KV heads the pairs are dealt round-robin over the XCDs (pair p to
  // XCD p % 8: each XCD gets the same heads of every sequence, so the XCDs
  // get equal work whatever the length mix). Otherwise a sequence's heads
  // would not spread evenly, and the (pair, row tile) items go to the XCDs
  // in turn instead (item b on XCD b % 8), so that every XCD gets an even
  // share of every pair.
  const unsigned tiles = (unsigned)a.row_tiles;
  const unsigned pairs = (unsigned)a.num_seqs * (unsigned)H;
  unsigned sh, tl;                                // the pair, and its row tile from the longest
  if (pf_round_robin(H)) {
    const unsigned xi = blockIdx.x / NXCD_PF;     // place on its XCD
    sh = (xi / tiles) * NXCD_PF + blockIdx.x % NXCD_PF;
    tl = xi % tiles;
  } else {
    const unsigned vb = blockIdx.x;
    sh = vb / tiles;
    tl = vb - sh * tiles;
  }
  if (sh >= pairs) return;                        // padding to whole XCD rounds
  const int s = (int)(sh / H);
  const int kvh = (int)(sh - (unsigned)s * H);
  const int tpos0 = (int)(tiles - 1 - tl) * TPOS;  // first query index of the tile
  const int r0 = a.query_start_loc[s];
  const int nq = a.query_start_loc[s + 1] - r0;
  // rows outside the packed query array are never touched
  if (nq <= 0 || tpos0 >= nq || r0 < 0 || (int64_t)r0 + nq > a.num_q_tokens) return;
  const int ctx = a.context_lens[s];
  const int lg = a.log2_block_size;
  const bool ctx_ok = ctx >= nq && ctx <= a.max_context_len &&
                      (((int64_t)ctx + a.block_size - 1) >> lg) <= a.max_blocks_per_seq;

  // this lane's query row: position index qi of the sequence's rows, head hh
  const int R = wave * FR + n;
  const int qi = tpos0 + R / G;
  const int hh = R % G;
  const bool rvalid = qi < nq;
  const int64_t orow = (((int64_t)r0 + min(qi, nq - 1)) * a.num_q_heads + (int64_t)kvh * G + hh) * D;
  // the wave's first and last query index, and the workgroup's last
  const int wq0 = tpos0 + wave * FR / G;
  const int wq1 = min(tpos0 + (wave * FR + FR - 1) / G, nq - 1);
  const bool wave_live = wq0 < nq;
  const int wg_last = min(tpos0 + TPOS - 1, nq - 1);

  auto store_row = [&](const f32x16_t (&o)[NB], float norm) __attribute__((always_inline)) {
    // output block mb, element v: dim 32 mb + 8(v/4) + 4h + v%4
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        store_out<QT>(a.out, orow + 32 * mb + (v >> 2) * 8 + 4 * h + (v & 3), o[mb][v] * norm);
  };
  if (!ctx_ok) {                                  // invalid context or query count: NaN rows
    if (rvalid) {
      f32x16_t o[NB];
#pragma unroll
      for (int m = 0; m < NB; ++m) o[m] = (f32x16_t){};
      store_row(o, __builtin_nanf(""));
    }
    return;
  }
  const int pos_row = rvalid ? ctx - nq + qi : -1;     // this lane's row attends to keys <= it
  const int wmin = ctx - nq + wq0, wmax = ctx - nq + wq1;
  const int nkt = (ctx - nq + wg_last) / FKT + 1;      // key tiles of the workgroup (uniform)

  // scale in log2 units; a negative scale is folded into the query's sign,
  // and a zero one replaced by a tiny positive one (every weight equal, as
  // for zero, while masked keys still get exactly 0)
  float c = a.qk_scale_log2;
  const uint32_t qflip = c < 0.f ? 0x80008000u : 0u;
  c = fmaxf(fabsf(c), 1e-30f);

  // q of this lane's row as the B operand of the score product: dims
  // 16k + 8h .. +8 of step k
  uint32_t qr[KSTEPS][4];
  {
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(a.q);
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      ld<4>(qw + ((orow + 16 * k + 8 * h) >> 1), qr[k]);
#pragma unroll
      for (int x = 0; x < 4; ++x) qr[k][x] ^= qflip;
    }
  }

  // ---- register staging: job j = (key j % FKT, chunk j / FKT): the key's
  // chunk of K and of V. K goes to its row as is. Neighbouring lanes hold
  // the two keys of a pair (same chunk); V^T interleaves them per dim (one
  // dword per dim), the even key's lane writing the chunk's first 8 dims and
  // the odd key's lane the last 8.
  const char* kpool = reinterpret_cast<const char*>(a.k_pool);
  const char* vpool = reinterpret_cast<const char*>(a.v_pool);
  const int bmask = a.block_size - 1;
  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int64_t head_off = a.layer_offset + (int64_t)kvh * a.block_size * D;
  // keys past the context (the last tile's tail) read the last key again:
  // finite values behind masked scores; table entries past the context are
  // never read
  auto key_at = [&](int kt, int jb) __attribute__((always_inline)) {
    return min(kt * FKT + jb % FKT, ctx - 1);
  };
  auto job_of = [&](int i) __attribute__((always_inline)) { return tid + FW * 64 * i; };
  // direct staging: this lane's row of wave instruction j, and its chunk
  // position in that row
  auto drow = [&](int j) __attribute__((always_inline)) { return (wave * NIW + j) * RPI + lane / R16; };
  const int dpos = lane % R16;
  // transposing V reads: lane 16q + 4J + A reads key J's dims from 4A of
  // its 16-dim half vdh = q % 2
  const int vJ = (lane >> 2) & 3, vA = lane & 3, vdh = (lane >> 4) & 1;
  // (UB) lane byte offsets of instruction j's rows from its base, K and V
  uint32_t koff[UB ? NIW : 1], voff[UB ? NIW : 1];
  if constexpr (UB) {
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int r = drow(j);
      koff[j] = (lane / R16) * ROWB + (dpos ^ (r % R16)) * 16;
      voff[j] = (lane / R16) * ROWB + (dpos ^ ((r % SEGS) << 2)) * 16;
    }
  }
  auto fetch_ids = [&](int kt, int (&ids)[NID]) __attribute__((always_inline)) {
    if constexpr (UB) {
#pragma unroll
      for (int j = 0; j < NIW; ++j) ids[j] = trow[min(kt * FKT + (wave * NIW + j) * RPI, ctx - 1) >> lg];
    } else if constexpr (DIRECT) {
#pragma unroll
      for (int j = 0; j < NIW; ++j) ids[j] = trow[min(kt * FKT + drow(j), ctx - 1) >> lg];
    } else {
#pragma unroll
      for (int i = 0; i < NJ; ++i)
        ids[i] = (JOBS % (FW * 64) != 0 && job_of(i) >= JOBS) ? 0 : trow[key_at(kt, job_of(i)) >> lg];
    }
  };
  bool bad = false;                               // a bad block id was staged
  uint32_t stk[DIRECT ? 1 : NJ][4], stv[DIRECT ? 1 : NJ][4];
  auto load_tile = [&](int kt, const int (&ids)[NID]) __attribute__((always_inline)) {
    if constexpr (UB) {
      char* kb = lds + (kt & 1) * L::BUF;
#pragma unroll
      for (int j = 0; j < NIW; ++j) {
        // key0: the instruction's first row; rows past the context read the
        // last key again (then key0 + lane row is clamped per lane)
        const int key0 = min(kt * FKT + (wave * NIW + j) * RPI, ctx - 1);
        const int id = __builtin_amdgcn_readfirstlane(ids[j]);
        const bool ok = id >= 0 && id < a.num_blocks;
        bad = bad || !ok;
        const int64_t e0 = (int64_t)(ok ? id : 0) * a.block_stride + head_off + (int64_t)(key0 & bmask) * D;
        uint32_t lk = koff[j], lv = voff[j];
        if (key0 + RPI > ctx) {
          const int lr = min(lane / R16, ctx - 1 - key0), r = drow(j);
          lk = lr * ROWB + (dpos ^ (r % R16)) * 16;
          lv = lr * ROWB + (dpos ^ ((r % SEGS) << 2)) * 16;
        }
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(kb + (wave * NIW + j) * 1024));
        lds_dma16_s(kpool + e0 * EB, lk, dst);
        lds_dma16_s(vpool + e0 * EB, lv, dst + L::KT);
      }
    } else if constexpr (DIRECT) {
      char* kb = lds + (kt & 1) * L::BUF;
#pragma unroll
      for (int j = 0; j < NIW; ++j) {
        const int r = drow(j);
        const int k = min(kt * FKT + r, ctx - 1);
        const bool ok = ids[j] >= 0 && ids[j] < a.num_blocks;
        bad = bad || !ok;
        const int64_t e = (int64_t)(ok ? ids[j] : 0) * a.block_stride + head_off + (int64_t)(k & bmask) * D;
        const int ck = dpos ^ (r % R16), cv = dpos ^ ((r % SEGS) << 2);
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(kb + (wave * NIW + j) * 1024));
        lds_dma16(kpool + (e + 8 * ck) * EB, dst);
        lds_dma16(vpool + (e + 8 * cv) * EB, dst + L::KT);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NJ; ++i) {
        if (JOBS % (FW * 64) != 0 && job_of(i) >= JOBS) continue;   // (whole waves past the jobs)
        const int jb = job_of(i);
        const int k = key_at(kt, jb);
        const bool ok = ids[i] >= 0 && ids[i] < a.num_blocks;
        bad = bad || !ok;
        const int64_t e = (int64_t)(ok ? ids[i] : 0) * a.block_stride + head_off +
                          (int64_t)(k & bmask) * D + (jb / FKT) * CD;
        ld<4>(reinterpret_cast<const uint32_t*>(kpool + e * EB), stk[i]);
        ld<4>(reinterpret_cast<const uint32_t*>(vpool + e * EB), stv[i]);
      }
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    if constexpr (!DIRECT) {                      // (direct: the memory unit wrote it)
    char* kb = lds + buf * L::BUF;
    char* vb = kb + L::KT;
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
      if (JOBS % (FW * 64) != 0 && job_of(i) >= JOBS) continue;
      const int jb = job_of(i);
      const int key = jb % FKT, ch = jb / FKT;
      static_assert(DIRECT || EB == 1, "register staging: FP8 pools");
      // K: the key's 16 codes widened, into its row
      uint32_t w[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) fp8x4_to<OP>(stk[i][x], w[2 * x], w[2 * x + 1]);
      char* dst = kb + key * L::PK + ch * CD * 2;
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
      // V^T: this lane writes dims 8hv .. 8hv + 7 of the chunk for the pair
      // (hv = key parity); it sends the other half of its own codes to its
      // neighbour (lane ^ 1, the pair's other key) and gets that key's codes
      // of its half back
      const int hv = key & 1;
      uint32_t mine[2], theirs[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t send = hv ? stv[i][x] : stv[i][2 + x];
        theirs[x] = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
        mine[x] = hv ? stv[i][2 + x] : stv[i][x];
      }
      // the pair's even key (wa) and odd key (wb): dims 8hv + 2q, +1 in dword q
      uint32_t wa[4], wb[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        fp8x4_to<OP>(hv ? theirs[x] : mine[x], wa[2 * x], wa[2 * x + 1]);
        fp8x4_to<OP>(hv ? mine[x] : theirs[x], wb[2 * x], wb[2 * x + 1]);
      }
      // dim d's dword holds (even key, odd key) at the pair's slot
      const int kp = key & ~1;
      char* vdst = vb + ((kp & ~15) + vt_slot(kp & 15)) * 2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = ch * CD + 8 * hv + 2 * q;
        *reinterpret_cast<uint32_t*>(vdst + d * L::PV) = __builtin_amdgcn_perm(wb[q], wa[q], 0x05040100u);
        *reinterpret_cast<uint32_t*>(vdst + (d + 1) * L::PV) = __builtin_amdgcn_perm(wb[q], wa[q], 0x07060302u);
      }
    }
    }
  };

  // ---- per-row state: reference max (log2 units), this lane's share of the
  // sum, and O^T (block mb, element v: dim 32 mb + 8(v/4) + 4h + v%4)
  float m_ref = -__builtin_inff();
  float l_sum = 0.f;
  f32x16_t o[NB];
#pragma unroll
  for (int m = 0; m < NB; ++m) o[m] = (f32x16_t){};

  // MASK: the tile may hold keys after some row's position (the causal
  // diagonal, or past the context); tiles wholly at or before the
  // workgroup's first position skip the mask arithmetic
  auto compute = [&](int kt, int buf, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* kb = lds + buf * L::BUF;
    const char* vb = kb + L::KT;
    // scores: sb[b][v] is key 32b + 8(v/4) + 4h + v%4 of the tile, row n
    f32x16_t sb[NSB];
#pragma unroll
    for (int b = 0; b < NSB; ++b) {
      // all of the block's K operands first, then the products
      uint4 kv[KSTEPS];
      if constexpr (DIRECT) {
        // chunk c = 2k + h of row 32b + n sits at c ^ (n mod R16): one lane
        // base (the buffer is 1 KiB aligned), step k flips bits 5 and up of
        // the chunk offset
        const uint32_t kl = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)kb +
                            n * L::PK + ((h ^ (n % R16)) << 4);
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k)
          kv[k] = lds_ld16((kl ^ (k << 5)) + 32 * b * L::PK);
      } else {
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) {
          const int row = 32 * b + n, c = 2 * k + h;          // key row, 16-byte chunk
          kv[k] = *reinterpret_cast<const uint4*>(kb + row * L::PK + c * 16);
        }
      }
      sb[b] = (f32x16_t){};
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        const uint32_t av[4] = {kv[k].x, kv[k].y, kv[k].z, kv[k].w};
        sb[b] = mfma32<OP>(av, qr[k], sb[b]);
      }
      if constexpr (DIRECT) {
        // keep KA operand reads in flight ahead of the dependent products
        // (the scheduler otherwise waits for each read just before its
        // product); more than 3 measured no faster
        constexpr int KA = 3;
        __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);
#pragma unroll
        for (int k = 0; k < KSTEPS - KA; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KA, 0);
      }
    }
    // causal mask: key 32b + 8(v/4) + v%4 + 4h of the tile <= pos_row (a
    // tile wholly before the wave's first position masks nothing)
    if constexpr (MASK) {
      const int thr = kt * FKT + FKT - 1 > wmin ? pos_row - kt * FKT - 4 * h : FKT;
#pragma unroll
      for (int b = 0; b < NSB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * b + (v >> 2) * 8 + (v & 3) > thr) sb[b][v] = MASKED;
    }
    float mx = MASKED;
#pragma unroll
    for (int b = 0; b < NSB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sb[b][v]);
    mx = pair_max(mx);
    // a row with no key here (all masked) leaves its reference alone
    const float zmax = mx <= MASKED ? -__builtin_inff() : mx * c;
    if (__any(zmax > m_ref + SM_TAU)) {
      const float mn = fmaxf(m_ref, zmax);
      const float al = mn == -__builtin_inff() ? 1.f : __builtin_amdgcn_exp2f(m_ref - mn);
      m_ref = mn;
      l_sum *= al;
#pragma unroll
      for (int m = 0; m < NB; ++m) o[m] *= al;
    }
    // probabilities as the B operand of P.V, key block kb (16 keys): k-slot j
    // is key 16kb + 8(j/4) + 4h + j%4, score element v = 8(kb%2) + j; the row
    // sum adds exactly the rounded values the matrix core multiplies
    uint32_t pk[NKB][4];
    const float nm = -m_ref;
#pragma unroll
    for (int b = 0; b < NSB; ++b) {
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(fmaf(sb[b][v], c, nm));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t w = pack2<OP>(p[2 * q], p[2 * q + 1]);
        pk[2 * b + (q >> 2)][q & 3] = w;
        l_sum = add_pair<OP>(w, l_sum);
      }
    }
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; ++kb2) {
      uint4 vv[NB];
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        if constexpr (DIRECT) {
          // V^T operand from key rows by two transposing reads: in each
          // 16-lane group, lane 4J + A reads 4 dims (from 4A) of key J, and
          // lane 4A + B receives dim 4A + B of keys 0..3 (k-slots 4r .. +3:
          // keys 16 kb2 + 8r + 4h + 0..3, as P's operand holds them)
          // key 16 kb2 + 8r + 4h + vJ, chunk c = 4mb + 2vdh + vA/2 at
          // c ^ 4(vJ mod SEGS): a lane base, dim block mb flips bits 6 and up
          const uint32_t vl = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)vb +
                              (4 * h + vJ) * ROWB + (vA & 1) * 8 + (2 * vdh + (vA >> 1)) * 16 +
                              ((vJ % SEGS) << 6);
          uint32_t w4[4];
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const uint32_t src = (vl ^ (mb << 6)) + (16 * kb2 + 8 * r) * ROWB;
            const auto t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) tr16x4_t*)(uintptr_t)src);
            const u32x2_t tw = __builtin_bit_cast(u32x2_t, t);
            w4[2 * r] = tw[0];
            w4[2 * r + 1] = tw[1];
          }
          vv[mb] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        } else {
          vv[mb] = *reinterpret_cast<const uint4*>(vb + (32 * mb + n) * L::PV + (16 * kb2 + 8 * h) * 2);
        }
      }
#pragma unroll
      for (int mb = 0; mb < NB; ++mb) {
        const uint32_t av[4] = {vv[mb].x, vv[mb].y, vv[mb].z, vv[mb].w};
        o[mb] = mfma32<OP>(av, pk[kb2], o[mb]);
      }
    }
  };

  // ---- the tile loop: loads of tile kt+1 and block ids of tile kt+2 in
  // flight while tile kt is processed from LDS; one barrier per tile
  // (direct staging: each wave waits for its own loads into LDS before the
  // barrier that hands the tile to all four)
  int ids_a[NID], ids_b[NID];
  fetch_ids(0, ids_a);
  load_tile(0, ids_a);
  if (nkt > 1) fetch_ids(1, ids_b);
  store_tile(0);
  if constexpr (DIRECT) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto step = [&](int kt, auto mask_tag) __attribute__((always_inline)) {
    const bool more = kt + 1 < nkt;
    if (more) load_tile(kt + 1, ids_b);
    if (kt + 2 < nkt) fetch_ids(kt + 2, ids_a);
    // a wave with no rows, or whose rows all end before this tile, skips it
    if (wave_live && kt * FKT <= wmax) compute(kt, kt & 1, mask_tag);
    if (more) store_tile((kt + 1) & 1);
    if constexpr (DIRECT) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NID; ++i) ids_b[i] = ids_a[i];
  };
  // tiles 0 .. nfull - 1 end at or before the workgroup's first position
  // (every key at or before every row's, none past the context); two loops,
  // each with its own copy of the tile code, so the full tiles carry no mask
  const int nfull = min(nkt, (ctx - nq + tpos0 + 1) / FKT);
  for (int kt = 0; kt < nfull; ++kt) step(kt, std::false_type{});
  for (int kt = nfull; kt < nkt; ++kt) step(kt, std::true_type{});
  bad = __syncthreads_or(bad);
  const float lt = l_sum + __shfl_xor(l_sum, 32);
  const float norm = bad ? __builtin_nanf("") : a.v_scale / lt;
  // Rows leave as whole 16-byte pieces, 16 lanes per row: a lane's O^T
  // elements are 4-dim pieces of one row, so they pass through LDS (free
  // now: every wave is past its last tile). The wave's FR rows are stored
  // row-major with 16-byte chunk c of row r at c ^ (r mod R16), so both the
  // writes and the reads spread over the banks.
  static_assert(FW * FR * ROWB <= L::BYTES, "the output rows fit in the tile buffers");
  char* ob = lds + wave * (FR * ROWB);
  // the lane's row and half again, from the lane counter (rather than
  // values kept in registers through the tile loop)
  int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(ln));
  const int on = ln & 31, oh = ln >> 5;
  auto h16 = [](float x) __attribute__((always_inline)) -> uint32_t {
    return QT == Ty::BF16 ? f32_to_bf16_rne(x) : f32_to_f16_rne(x);
  };
#pragma unroll
  for (int mb = 0; mb < NB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // dims 32 mb + 8q + 4h .. +3: half h of chunk 4 mb + q
      const uint32_t w0 = h16(o[mb][4 * q] * norm) | (h16(o[mb][4 * q + 1] * norm) << 16);
      const uint32_t w1 = h16(o[mb][4 * q + 2] * norm) | (h16(o[mb][4 * q + 3] * norm) << 16);
      const int c = 4 * mb + q;
      *reinterpret_cast<uint2*>(ob + on * ROWB + (c ^ (on % R16)) * 16 + oh * 8) = make_uint2(w0, w1);
    }
  __syncthreads();
  const bool out16 = (reinterpret_cast<uintptr_t>(a.out) & 15) == 0;
#pragma unroll
  for (int i = 0; i < FR / RPI; ++i) {
    const int row = i * RPI + ln / R16, c = ln % R16;
    const uint4 v = *reinterpret_cast<const uint4*>(ob + row * ROWB + (c ^ (row % R16)) * 16);
    const int Rw = wave * FR + row, qw = tpos0 + Rw / G;
    if (qw < nq) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) +
                      (((int64_t)r0 + qw) * a.num_q_heads + (int64_t)kvh * G + Rw % G) * D + 8 * c;
      if (out16) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else {                                    // an output only 4-byte aligned
        uint32_t* d4 = reinterpret_cast<uint32_t*>(dst);
        d4[0] = v.x;
        d4[1] = v.y;
        d4[2] = v.z;
        d4[3] = v.w;
      }
    }
  }
}

template <Ty KV, Ty QT, int D, int FKT, bool UB>
hipError_t launch_g(const PrefillParams& a, int g, dim3 grid, hipStream_t st) {
  switch (g) {
    case 1: hipLaunchKernelGGL((prefill_tiled_kernel<KV, QT, D, 1, FKT, UB>), grid, dim3(FW * 64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_tiled_kernel<KV, QT, D, 2, FKT, UB>), grid, dim3(FW * 64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_tiled_kernel<KV, QT, D, 4, FKT, UB>), grid, dim3(FW * 64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_tiled_kernel<KV, QT, D, 8, FKT, UB>), grid, dim3(FW * 64), 0, st, a); break;
    case 16: hipLaunchKernelGGL((prefill_tiled_kernel<KV, QT, D, 16, FKT, UB>), grid, dim3(FW * 64), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 16-bit pools whose blocks hold at least the rows of one staging
// instruction take the uniform-base form
template <Ty KV, Ty QT, int D, int FKT>
hipError_t launch_u(const PrefillParams& a, int g, dim3 grid, hipStream_t st) {
  if constexpr (TyInfo<KV>::bytes == 2) {
    if (a.block_size >= 1024 / (2 * D)) return launch_g<KV, QT, D, FKT, true>(a, g, grid, st);
  }
  return launch_g<KV, QT, D, FKT, false>(a, g, grid, st);
}

template <Ty KV, Ty QT>
hipError_t launch_d(const PrefillParams& a, int g, dim3 grid, bool wide, hipStream_t st) {
  if (a.head_dim == 64) return wide ? launch_u<KV, QT, 64, 64>(a, g, grid, st) : launch_u<KV, QT, 64, 32>(a, g, grid, st);
  if (a.head_dim == 128) return wide ? launch_u<KV, QT, 128, 64>(a, g, grid, st) : launch_u<KV, QT, 128, 32>(a, g, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int kv_ty, int q_ty, int head_dim, int g) {
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  const bool types = (kv == Ty::BF16 && q == Ty::BF16) || (kv == Ty::F16 && q == Ty::F16) ||
                     (kv == Ty::FP8 && (q == Ty::BF16 || q == Ty::F16));
  return types && (head_dim == 64 || head_dim == 128) &&
         (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
}

// Workgroups along the query rows: each covers 128 / g positions.
int prefill_tiles(int g, int max_query_len) {
  const int64_t per = FW * FR / g;
  return (int)(((int64_t)max_query_len + per - 1) / per);
}

// The launch: the (pair, row tile) items, rounded up to whole rounds of the
// XCDs (with pairs dealt round-robin, their count is already a multiple of 8).
int64_t prefill_grid(int num_seqs, int num_kv_heads, int tiles) {
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  if (pf_round_robin(num_kv_heads)) return pairs * tiles;   // (pairs: a multiple of 8)
  return (pairs * tiles + NXCD_PF - 1) / NXCD_PF * NXCD_PF;
}

hipError_t launch_prefill(const PrefillParams& a0, int kv_ty, int q_ty, int g, int max_query_len,
                          hipStream_t st) {
  PrefillParams a = a0;
  a.row_tiles = prefill_tiles(g, max_query_len);
  const int64_t used = (int64_t)a.num_seqs * a.num_kv_heads * a.row_tiles;
  const int64_t wgs = prefill_grid(a.num_seqs, a.num_kv_heads, a.row_tiles);
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs);
  // 64-key tiles when the grid is at most two rounds of two workgroups per
  // compute unit (few, long workgroups), 32-key tiles otherwise
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  const bool wide = used <= (int64_t)4 * cus;
  const Ty kv = (Ty)kv_ty, q = (Ty)q_ty;
  if (kv == Ty::BF16 && q == Ty::BF16) return launch_d<Ty::BF16, Ty::BF16>(a, g, grid, wide, st);
  if (kv == Ty::F16 && q == Ty::F16) return launch_d<Ty::F16, Ty::F16>(a, g, grid, wide, st);
  if (kv == Ty::FP8 && q == Ty::BF16) return launch_d<Ty::FP8, Ty::BF16>(a, g, grid, wide, st);
  if (kv == Ty::FP8 && q == Ty::F16) return launch_d<Ty::FP8, Ty::F16>(a, g, grid, wide, st);
  return hipErrorInvalidValue;
}

}  // namespace pa
