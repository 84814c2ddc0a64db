// Fused attention forward for gfx950 (one query tile per workgroup).
//
// Page "Stable summary of an attention key block", Definition: each query
// row keeps a summary (m, l, z) of the keys seen so far; the summary of the
// next key block is merged with the page's rule (the larger maximum becomes
// the shift, both sides are rescaled by exp of the old-minus-new maximum);
// at the end z is divided by l.  The empty state (no allowed key seen yet)
// is held as m = -inf, l = 0, z = 0, and the shift used for exponentials is
// forced to 0 while m is -inf, so the empty state merges as the identity.
// Review page "Multi-Head Attention", "The Complete Multi-Head Operation":
// scores are c * q_i . k_j, the mask is applied before the softmax, and the
// head result is written into its column block of the concatenation.
//
// Mapping onto the matrix cores (our design, not the pages'):
// * each wave owns 32 query rows; a workgroup of WAVES waves shares K/V
//   blocks of BN keys staged through two LDS buffers (the next block is
//   written while the current one is read; one barrier per block);
// * the score block is computed transposed, S^T = K Q^T, with a 32x32 MFMA:
//   lane l then holds 16 scores of query (l % 32) per 32-key sub-block, so a
//   row's maximum needs one exchange with the other half-wave only;
// * the value product is computed as O^T = V^T P^T: the transposed score
//   fragment is already in the B-operand layout of the next MFMA.  The
//   A operand needs, per lane, one feature of V for several keys: 2-byte V
//   tiles are stored row-major in LDS and read with the transposing LDS
//   load (ds_read_b64_tr_b16); fp32 V tiles are stored transposed;
// * O^T leaves every lane with one query's output features, so the final
//   division by l and the concatenated store need no cross-lane traffic.
// Base-2 exponentials: scores are carried in units of log2(e) (see the
// query set-up below), so 2^(x - m2) = e^(s - m) and l and z are the page's
// quantities.  Weights feed the value product rounded to T; the normaliser
// sums the same rounded weights (fp32 accumulation), so z / l is an exact
// convex combination of the values the product used.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

namespace mha {

template <typename T, int DH, int DV, int WAVES, int BN_ = 64>
struct AttnCfg {
  static constexpr int VEC = Elem<T>::VEC;
  static constexpr bool TR = sizeof(T) == 2;   // V row-major + transposing reads
  static constexpr int BN = BN_;                // keys per block
  static constexpr int NKB = BN / 32;           // 32-key sub-blocks per block
  static constexpr int NT = 64 * WAVES;         // threads per workgroup
  static constexpr int QT = 32 * WAVES;         // queries per workgroup
  static constexpr int KCH = DH / (2 * VEC);    // k-chunks of the score MFMA
  static constexpr int NDV = DV / 32;           // 32-row blocks of V^T
  static constexpr int KPAD = DH + VEC;         // LDS row stride of K (elements)
  // V: row-major rows of DV (+ pad so the rows one transposing read touches
  // fall in different banks), or transposed rows of BN keys for fp32.
  static constexpr int VROW = TR ? DV + ((DV % 64 == 0) ? 32 : 0) : BN + 4;
  static constexpr int KBUF = BN * KPAD;        // elements per K buffer
  static constexpr int VBUF = TR ? BN * VROW : DV * VROW;
  static constexpr int K_CHUNKS = BN * DH / VEC;
  static constexpr int V_CHUNKS = BN * DV / VEC;
  static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_PER_T = (V_CHUNKS + NT - 1) / NT;
  static constexpr int REG_LDS = 2 * (KBUF + VBUF) * (int)sizeof(T);   // register staging
  // Direct-to-LDS staging (2-byte fast path): unpadded rows of KRB / VRB
  // bytes, three stages of one K tile and one V tile (a kernel may run two),
  // K_WIN / V_WIN 1 KB load instructions per wave per tile.
  static constexpr int KRB = DH * (int)sizeof(T), VRB = DV * (int)sizeof(T);
  static constexpr int KTILE = BN * KRB, VTILE = BN * VRB;
  static constexpr int STAGE = KTILE + VTILE, NS = 3;
  static constexpr int K_WIN = KTILE / 1024 / WAVES, V_WIN = VTILE / 1024 / WAVES;
  static constexpr int DMA_LDS = NS * STAGE;
  static_assert(DH % (2 * VEC) == 0, "DH must be a multiple of a k-chunk");
  static_assert(DV % 32 == 0, "DV must be a multiple of 32");
  static_assert(BN == 32 || BN == 64 || BN == 128, "BN must be 32, 64 or 128");
};

template <typename T>
__device__ __forceinline__ typename Elem<T>::vec negate_chunk(typename Elem<T>::vec v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u ^= (sizeof(T) == 4) ? 0x80000000u : 0x80008000u;
  return __builtin_bit_cast(typename Elem<T>::vec, u);
}

// Sum of eight rounded weights (fp32 accumulation) for the 2-byte types.
__device__ __forceinline__ float sum8(const bf16x8& p, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  #pragma unroll
  for (int t = 0; t < 8; t += 2) {
    const bf16x2 pr = {p[t], p[t + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float sum8(const f16x8& p, float acc) {
  const f16x2 one = {(f16)1.0f, (f16)1.0f};
  #pragma unroll
  for (int t = 0; t < 8; t += 2) {
    const f16x2 pr = {p[t], p[t + 1]};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
  }
  return acc;
}

// XOR permutations of the 16-byte chunks of a K / V row in LDS (direct-to-LDS
// staging), chosen so that the two read patterns hit distinct banks:
// * K rows (RB bytes) are read 16 bytes per lane, 32 consecutive rows at one
//   chunk: chunk c of row r is stored in slot c ^ ((r / (256 / RB)) % (RB / 16)),
//   which gives 16 consecutive rows 16 distinct 16-byte bank groups;
// * V rows are read with the transposing load, 4 rows x 64 bytes per half
//   wave: for RB = 128 or 256, chunk c of row r is stored in slot
//   c ^ 4 ((r / (256 / RB)) % (RB / 64)), putting the 4 rows in distinct 64-byte
//   quarters of the banks; 64- and 192-byte rows are staggered already.
template <int RB>
__device__ __forceinline__ int k_swizzle(int row) {
  constexpr int RPB = RB >= 256 ? 1 : 256 / RB;
  return (row / RPB) % (RB / 16);
}
template <int RB>
__device__ __forceinline__ int v_swizzle(int row) {
  if constexpr (RB == 128 || RB == 256) {
    constexpr int RPB = 256 / RB;
    return 4 * ((row / RPB) % (RB / 64));
  } else {
    return 0;
  }
}

// FAST: every row of Q, K, V is exactly DH / DV wide with 16-byte aligned
// rows, and there is no boolean mask or additive bias (MASKED: there may be,
// with aligned mask rows, p.mask_vec); the host selects it when that holds.
// The general variant predicates every column and reads the masks.
//
// LAZY (deferred shift): the running state of a row is kept as (m, l*, z*)
// with l* = l e^(m - mu), z* = z e^(m - mu) for a reference shift mu <= m
// that is moved up to m only when a block's maximum exceeds mu by more than
// kLazyTau (base-2 units), so weights stay below 2^kLazyTau.  Between moves
// the page's merge of a block at the common shift mu is l* += sum e^(s-mu),
// z* += sum e^(s-mu) v; when mu moves, both sides are rescaled by the
// page's factor.  m itself is tracked exactly, and at the end l = l* e^(mu-m)
// is returned; z*/l* = z/l.  With mu fixed between moves, -mu is fed to the
// score MFMA as its accumulator input, so a weight costs one exponential.
constexpr float kLazyTau = 8.0f;

// Block-sum trigger (deferred shift without row statistics): the row's
// block maximum is not formed.  A weight above 2^kLazyTau makes this lane's
// partial sum of the block's rounded weights exceed 2^kLazyTau, so that sum
// decides when the block is redone at an exact new shift; weights are finite
// and at most 2^kLazyTau whenever it stays below.
constexpr float kLazyLimit = 256.0f;   // 2^kLazyTau
static_assert(kLazyLimit == (float)(1 << (int)kLazyTau), "limit = 2^tau");

// OCC: minimum waves per SIMD the register allocation must allow.
// STATS: the caller wants the final (m, l) per row (deferred-shift variant:
// the exact running maximum is tracked only then).
// SPLIT: one key partition per workgroup; partial summaries are written
// (p.part_m / part_l / part_z) instead of Z.  Uses the exact-shift merge: a
// partition may hold no allowed key for some rows (empty state).
// MASKED (direct-load path, p.mask_vec): 1 = boolean mask and / or additive
// bias read per lane, exact shift; 2 = boolean mask whose tile moves into
// LDS with the K/V tiles; 3 = additive bias alone, its tile moved into LDS
// one block ahead.  2 and 3 may run the deferred shift (no row statistics):
// a row with no allowed key yet keeps mu = -inf, and its first allowed
// block is redone at an exact shift (the +inf scores trip the block-sum
// trigger).
// Key padding without the causal rule: the item of rank k when the items
// are ordered by decreasing key count (ties by index), for B <= 64 (lane i
// holds item i's count; every lane of the wave takes part; the result is
// uniform).
__device__ __forceinline__ int item_of_rank(const AttnParams& p, int k) {
  const int lane = threadIdx.x & 63;
  const int mine = lane < p.B ? max(0, min(p.key_len[lane], p.n_k)) : -1;
  int rank = 0;
  for (int j = 0; j < p.B; ++j) {
    const int other = __builtin_amdgcn_readlane(mine, j);
    rank += (other > mine || (other == mine && j < lane)) ? 1 : 0;
  }
  const unsigned long long hit = __ballot(lane < p.B && rank == k);   // one lane
  return hit ? __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit)) : 0;
}

struct TileId {
  int qt, bh;
};

// Workgroup id -> (query tile, batch*head) of the attention kernels.
// * Default: query tiles outer, heads inner; with round-robin dispatch over
//   the 8 XCDs every tile of one head lands on the same XCD when B*h is a
//   multiple of 8, so its K/V stay in that XCD's L2.  Causal: longest tiles
//   (most keys) first.
// * Key padding without the causal rule (B <= 64), on grids of more than
//   512 workgroups (two per CU; a smaller grid is resident at once and only
//   pays for the ordering): items in decreasing key count, so the longest
//   rows start first and the short ones fill the slots that free up (a
//   longest-first schedule; every tile of an item has the same length).
// * A boolean mask or an additive bias ([B or 1, n_q, n_k], read by every
//   head of an item): the BH / 8 heads an XCD receives are consecutive
//   (b, r) pairs, so an item's heads share its mask rows in that XCD's L2 (a
//   bijection of [0, BH) when BH % 8 == 0).
__device__ __forceinline__ TileId tile_of_workgroup(const AttnParams& p, int id, bool split) {
  const int BH = p.B * p.h;
  if (!split && !p.causal && p.key_len != nullptr && p.B > 1 && p.B <= 64 &&
      p.num_q_tiles * BH > 512) {
    const int per_item = p.num_q_tiles * p.h;
    const int k = id / per_item, within = id - k * per_item;
    const int qt = within / p.h, r = within - qt * p.h;
    return TileId{qt, item_of_rank(p, k) * p.h + r};
  }
  const int qt_rank = id / BH;
  int bh = id - qt_rank * BH;
  if (!split && (p.allowed != nullptr || p.add != nullptr) && BH % 8 == 0)
    bh = (bh % 8) * (BH / 8) + bh / 8;
  return TileId{p.causal ? (p.num_q_tiles - 1 - qt_rank) : qt_rank, bh};
}

template <typename T, int DH, int DV, int WAVES, int BN_, bool FAST, bool LAZY = false, int OCC = 1,
          bool STATS = true, bool SPLIT = false, int MASKED = 0>
__global__ __launch_bounds__(64 * WAVES, OCC) void attn_fwd_kernel(AttnParams p) {
  typedef AttnCfg<T, DH, DV, WAVES, BN_> C;
  static_assert(!(SPLIT && LAZY), "a key partition may hold no allowed key for a row");
  static_assert(STATS || (LAZY && C::TR), "the block-sum trigger is for 2-byte elements");
  static_assert(!(MASKED && !FAST) && !(MASKED == 1 && LAZY),
                "masked fast variants: exact-shift merge, or the deferred shift with the "
                "boolean tile or the bias tile in LDS");
  // MASKED == 3: an additive bias and no boolean mask (its tile staged in LDS
  // as for MASKED == 1): the mask step is one fused multiply-add per score
  // (a forbidden entry, M = -inf, gives -inf by itself) plus the causal /
  // padding threshold on boundary blocks.
  constexpr bool ADDONLY = MASKED == 3;
  // GEN: boolean / additive masks are read (the general variant, or the
  // fast variant with masks whose rows hold aligned groups of four keys)
  constexpr bool GEN = !FAST || MASKED != 0;
  constexpr int NKB = C::NKB;
  typedef typename Elem<T>::vec vec;
  typedef typename Elem<T>::vec4 vec4;
  constexpr int VEC = C::VEC;
  constexpr int BN = C::BN;

  // DMA: K/V tiles move from global memory straight into LDS (NS stages in
  // flight, below); otherwise they are staged through registers (two buffers).
  constexpr bool DMA = C::TR && FAST && BN_ == 64;
  // MASKED == 2: the boolean mask's tile (QT rows x 64 key bytes) is loaded
  // straight into LDS with each block's K/V tiles, after the stages
  constexpr bool MLDS = MASKED == 2;
  static_assert(!MLDS || DMA, "the mask tile travels with the direct loads");
  constexpr int MT = MLDS ? C::QT * BN : 0;
  constexpr int M_WIN = MT / 1024 / WAVES;
  static_assert(M_WIN * 1024 * WAVES == MT, "whole 1 KB mask windows per wave");
  // Stages in flight: three, or two for the boolean tile at three workgroups
  // per CU (at d = 64: 48 KB of LDS instead of 72 KB).  With two, block
  // blk + 1 is issued once every wave is past block blk - 1, so its loads
  // have one block of compute to land instead of two.
  constexpr int NS = (MLDS && OCC >= 3) ? 2 : C::NS;
  constexpr int DMA_LDS = NS * C::STAGE;
  // ALDS (MASKED == 1 or 3, direct-load path): an additive bias tile (QT
  // rows x BN fp32 keys, 32 KB at 64 keys) moves by direct loads into one LDS
  // buffer, each wave its own 32 rows, one block ahead: block blk + 1's rows
  // are issued at the top of block blk (before the K/V loads of block
  // blk + 2) into the buffer the wave has just read block blk's rows from.
  constexpr bool ALDS = (MASKED == 1 || MASKED == 3) && DMA;
  constexpr int AT = ALDS ? C::QT * BN * 4 : 0;
  constexpr int A_WIN = AT / 1024 / WAVES;
  static_assert(!ALDS || A_WIN * 1024 * WAVES == AT, "whole 1 KB bias windows per wave");
  constexpr int LDS_BYTES = DMA ? DMA_LDS + NS * MT + AT : C::REG_LDS;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = Ks + 2 * C::KBUF;
  const unsigned lds_base = (unsigned)(size_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int g = lane >> 5;      // lane half
  const int l32 = lane & 31;

  // Workgroup -> (query tile, batch*head): tile_of_workgroup.
  const int BH = p.B * p.h;
  const int sp = SPLIT ? (int)(blockIdx.x % (unsigned)p.splits) : 0;   // key partition
  const int id = SPLIT ? (int)(blockIdx.x / (unsigned)p.splits) : (int)blockIdx.x;
  const TileId tile = tile_of_workgroup(p, id, SPLIT);
  const int qt = tile.qt, bh = tile.bh;
  const int b = bh / p.h;
  const int r = bh - b * p.h;
  const int q0 = qt * C::QT;
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;

  // Keys any row of this workgroup may use: [0, kend).
  int kvalid = p.n_k;
  if (p.key_len) kvalid = min(kvalid, p.key_len[b]);
  int kend = kvalid;
  if (p.causal) kend = min(kend, q0 + C::QT);
  // Key blocks [blk0, nblk) (absolute indices): all of [0, kend), or this
  // workgroup's partition of it.
  int blk0 = 0;
  if constexpr (SPLIT) {
    const int kbeg = sp * p.split_keys;
    kend = min(kend, kbeg + p.split_keys);
    blk0 = kbeg / BN;
    if (kend < kbeg) kend = kbeg;
  }
  const int nblk = kend > blk0 * BN ? (kend + BN - 1) / BN : blk0;

  const T* Qb = reinterpret_cast<const T*>(p.Q) + (size_t)bh * p.n_q * p.ldq;
  const T* Kb = reinterpret_cast<const T*>(p.K) + (size_t)bh * p.n_k * p.ldk;
  const T* Vb = reinterpret_cast<const T*>(p.V) + (size_t)bh * p.n_k * p.ldv;
  const uint8_t* Gb =
      (GEN && p.allowed) ? p.allowed + (size_t)b * p.allowed_batch_stride : nullptr;
  // additive score bias M (general path only): added to the scaled score
  const float* Ab = (GEN && p.add) ? p.add + (size_t)b * p.add_batch_stride : nullptr;
  const bool vq = FAST || p.vec_q, vk = FAST || p.vec_k, vv = FAST || p.vec_v;
  const int dh = FAST ? DH : p.d_h;
  const int dvh = FAST ? DV : p.d_vh;
  const int ldk = FAST ? DH : p.ldk;
  const int ldv = FAST ? DV : p.ldv;

  // fp32 elements: the query is multiplied by c log2(e) once, in registers,
  // so scores arrive in base-2 units and a weight is 2^(s - m), exactly 1 at
  // the row maximum.  2-byte elements keep the query as given (no second
  // rounding); the scale enters as c' = |c| log2(e) in one fused
  // multiply-add per score, and the sign of c is moved into the query.
  // The deferred-shift variant also scales 2-byte queries once (one extra
  // rounding of q c log2(e) to T), so that the score MFMA alone forms
  // c' s - mu.
  // With an additive bias the mask step forms the scaled score c' s + M log2(e)
  // itself (cs0 = the scale still to apply to the raw product), and later
  // steps see scaled scores (cs = 1).
  constexpr bool PRESCALE = sizeof(T) == 4 || LAZY;
  const float cs0 = PRESCALE ? 1.0f : fabsf(p.scale_log2);
  const float cs = (Ab != nullptr) ? 1.0f : cs0;

  // This lane's query row as the B operand of S^T = K Q^T (registers, whole
  // kernel).
  vec qf[C::KCH];
  #pragma unroll
  for (int c = 0; c < C::KCH; ++c) {
    if constexpr (FAST) {
      // rows past n_q read the last row (their results are never stored)
      const int qc = min(qi, p.n_q - 1);
      qf[c] = *reinterpret_cast<const vec*>(Qb + (size_t)qc * DH + c * 2 * VEC + g * VEC);
    } else {
      qf[c] = (qi < p.n_q) ? load_chunk<T>(Qb + (size_t)qi * p.ldq, c * 2 * VEC + g * VEC, dh, vq)
                           : zero_vec<vec>();
    }
    if constexpr (PRESCALE) {
      #pragma unroll
      for (int e = 0; e < VEC; ++e) qf[c][e] = (T)((float)qf[c][e] * p.scale_log2);
    } else {
      if (p.scale_log2 < 0.f) qf[c] = negate_chunk<T>(qf[c]);
    }
  }

  floatx16 o[C::NDV];
  #pragma unroll
  for (int d = 0; d < C::NDV; ++d)
    #pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m_run = -INFINITY;  // running maximum of the scores (base-2 units)
  float l_run = 0.f;        // this half-wave's part of the running normaliser
  float mu = -INFINITY;     // LAZY: reference shift (l_run, o are kept at mu)
  floatx16 negmu;           // LAZY: -mu in every slot, the score MFMA's C input
  // Masked deferred shift: a row whose blocks so far held no allowed key keeps
  // mu = -inf (negmu = +inf), so its first allowed score comes out +inf and
  // sends that block down the exact redo, which sets mu.
  #pragma unroll
  for (int i = 0; i < 16; ++i) negmu[i] = MASKED ? INFINITY : 0.f;

  // ---- staging of K/V blocks: global -> registers -> LDS ----------------------
  // Thread chunk t of a block covers tile row krow[t] / vrow[t] (a key) and
  // columns kcol[t] / vcol[t]; consecutive threads take consecutive 16-byte
  // chunks of one row (fp32 V: consecutive keys, for the transposed store).
  int krow[C::K_PER_T], kcol[C::K_PER_T], vrow[C::V_PER_T], vcol[C::V_PER_T];
  #pragma unroll
  for (int t = 0; t < C::K_PER_T; ++t) {
    const int ci = tid + t * C::NT;
    krow[t] = ci / (DH / VEC);
    kcol[t] = (ci - krow[t] * (DH / VEC)) * VEC;
  }
  #pragma unroll
  for (int t = 0; t < C::V_PER_T; ++t) {
    const int ci = tid + t * C::NT;
    if constexpr (C::TR) {
      vrow[t] = ci / (DV / VEC);
      vcol[t] = (ci - vrow[t] * (DV / VEC)) * VEC;
    } else {
      const int cc = ci / BN;
      vrow[t] = ci - cc * BN;
      vcol[t] = cc * VEC;
    }
  }
  vec kreg[C::K_PER_T];
  vec vreg[C::V_PER_T];

  auto load_kv = [&](int blk) {
    const int k0 = blk * BN;
    const bool tail = k0 + BN > p.n_k;   // uniform: only the last block can run past n_k
    #pragma unroll
    for (int t = 0; t < C::K_PER_T; ++t) {
      if (C::K_CHUNKS % C::NT != 0 && tid + t * C::NT >= C::K_CHUNKS) continue;
      int key = k0 + krow[t];
      if constexpr (FAST) {
        // keys past n_k read the last key; they are masked out (weight 0)
        if (tail) key = min(key, p.n_k - 1);
        kreg[t] = *reinterpret_cast<const vec*>(Kb + (size_t)key * DH + kcol[t]);
      } else {
        kreg[t] = (key < p.n_k) ? load_chunk<T>(Kb + (size_t)key * ldk, kcol[t], dh, vk)
                                : zero_vec<vec>();
      }
    }
    #pragma unroll
    for (int t = 0; t < C::V_PER_T; ++t) {
      if (C::V_CHUNKS % C::NT != 0 && tid + t * C::NT >= C::V_CHUNKS) continue;
      int key = k0 + vrow[t];
      if constexpr (FAST) {
        if (tail) key = min(key, p.n_k - 1);
        vreg[t] = *reinterpret_cast<const vec*>(Vb + (size_t)key * DV + vcol[t]);
      } else {
        vreg[t] = (key < p.n_k) ? load_chunk<T>(Vb + (size_t)key * ldv, vcol[t], dvh, vv)
                                : zero_vec<vec>();
      }
    }
  };
  auto store_kv = [&](int buf) {
    T* ks = Ks + buf * C::KBUF;
    T* vs = Vs + buf * C::VBUF;
    #pragma unroll
    for (int t = 0; t < C::K_PER_T; ++t) {
      if (C::K_CHUNKS % C::NT != 0 && tid + t * C::NT >= C::K_CHUNKS) continue;
      *reinterpret_cast<vec*>(&ks[krow[t] * C::KPAD + kcol[t]]) = kreg[t];
    }
    #pragma unroll
    for (int t = 0; t < C::V_PER_T; ++t) {
      if (C::V_CHUNKS % C::NT != 0 && tid + t * C::NT >= C::V_CHUNKS) continue;
      if constexpr (C::TR) {
        *reinterpret_cast<vec*>(&vs[vrow[t] * C::VROW + vcol[t]]) = vreg[t];
      } else {
        #pragma unroll
        for (int e = 0; e < VEC; ++e) vs[(vcol[t] + e) * C::VROW + vrow[t]] = vreg[t][e];
      }
    }
  };

  // ---- direct-to-LDS staging -------------------------------------------------
  // Window q of this wave's share of a tile is LDS bytes (wave*WIN + q) KB;
  // lane i fills 16 bytes at 16 i, i.e. tile row t / RB, slot (t % RB) / 16
  // for t = window*1024 + 16 i, from the global chunk the slot holds.
  unsigned koff[DMA ? C::K_WIN : 1], voff[DMA ? C::V_WIN : 1];
  auto tile_row = [&](int win, int rb) { return (win * 1024 + 16 * lane) / rb; };
  auto k_chunk_of = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / C::KRB;
    return ((t % C::KRB) / 16) ^ k_swizzle<C::KRB>(row);
  };
  auto v_chunk_of = [&](int win) {
    const int t = win * 1024 + 16 * lane, row = t / C::VRB;
    return ((t % C::VRB) / 16) ^ v_swizzle<C::VRB>(row);
  };
  if constexpr (DMA) {
    #pragma unroll
    for (int q = 0; q < C::K_WIN; ++q) {
      const int win = wave * C::K_WIN + q;
      koff[q] = tile_row(win, C::KRB) * C::KRB + k_chunk_of(win) * 16;
    }
    #pragma unroll
    for (int q = 0; q < C::V_WIN; ++q) {
      const int win = wave * C::V_WIN + q;
      voff[q] = tile_row(win, C::VRB) * C::VRB + v_chunk_of(win) * 16;
    }
  }
  // Mask tile windows: window w holds tile rows 16 w .. 16 w + 15, 64 bytes
  // each; lane i fills row 16 w + i / 4, slot i % 4, from the row's 16-byte
  // chunk (i % 4) ^ ((row / 4) % 4) (so the reads below, 32 rows at one
  // chunk, spread over the banks).  Rows past n_q read row n_q - 1 and
  // chunks past n_k the last chunk (n_k % 16 == 0): both are never used
  // (rows not stored; keys >= n_k fail the key-count threshold).
  unsigned mrow[MLDS ? M_WIN : 1], mchk[MLDS ? M_WIN : 1];
  if constexpr (MLDS) {
    #pragma unroll
    for (int q = 0; q < M_WIN; ++q) {
      const int t = (wave * M_WIN + q) * 1024 + 16 * lane;
      const int row = t / 64, slot = (t % 64) / 16;
      mrow[q] = (unsigned)min(q0 + row, p.n_q - 1) * (unsigned)p.n_k;
      mchk[q] = (unsigned)((slot ^ ((row >> 2) & 3)) * 16);
    }
  }
  // Bias tile windows (ALDS): window q of wave w holds rows 32 w + 4 q +
  // lane / 16 of the tile, 256 bytes each; lane i fills 16 bytes (slot
  // i % 16) from the row's chunk (i % 16) ^ (row % 16) -- 4 fp32 keys -- so
  // that the reads (16 rows at one chunk per phase) meet distinct bank
  // groups.  With every row of the tile below n_q and every key of the block
  // below n_k, window q's byte offset is 4 (row0 + 4 q) n_k + 4 k0 +
  // 16 (c0 ^ 4 (q % 4)), row0 = q0 + 32 w + lane / 16, c0 = (lane % 16) ^
  // (lane / 16): four per-lane values (abase), the rest scalar.  Otherwise
  // rows past n_q read row n_q - 1 and keys past n_k the last four
  // (n_k % 4 == 0): never used.
  unsigned abase[ALDS ? 4 : 1];
  if constexpr (ALDS) {
    const unsigned row0 = (unsigned)(q0 + wave * 32 + (lane >> 4));
    const unsigned c0 = (unsigned)((lane & 15) ^ (lane >> 4));
    #pragma unroll
    for (int j = 0; j < 4; ++j) abase[j] = 4u * row0 * (unsigned)p.n_k + 16u * (c0 ^ (4u * j));
  }
  const unsigned a_lds = lds_base + (unsigned)(DMA_LDS + NS * MT) + wave * A_WIN * 1024;
  auto issue_bias = [&](int blk) {
    if constexpr (ALDS) {
      const int k0 = blk * BN;
      if (q0 + C::QT <= p.n_q && k0 + BN <= p.n_k) {
        #pragma unroll
        for (int q = 0; q < A_WIN; ++q)
          lds_dma16(Ab + (size_t)k0 + (size_t)(4 * q) * p.n_k, abase[q & 3], a_lds + q * 1024);
      } else {
        #pragma unroll
        for (int q = 0; q < A_WIN; ++q) {
          const int row = wave * 32 + 4 * q + (lane >> 4);
          const int chunk = (lane & 15) ^ (row & 15);
          const unsigned off = 4u * ((unsigned)min(q0 + row, p.n_q - 1) * (unsigned)p.n_k +
                                     (unsigned)min(k0 + 4 * chunk, p.n_k - 4));
          lds_dma16(Ab, off, a_lds + q * 1024);
        }
      }
    }
  };
  // block blk into stage blk % NS; in the last block, rows past n_k read the
  // last key (masked out, weight 0)
  auto issue_kv = [&](int blk) {
    const int k0 = blk * BN;
    const unsigned st = lds_base + (unsigned)((blk % NS) * C::STAGE);
    if constexpr (MLDS) {
      const unsigned mst = lds_base + (unsigned)(DMA_LDS + (blk % NS) * MT);
      #pragma unroll
      for (int q = 0; q < M_WIN; ++q)
        lds_dma16(Gb, mrow[q] + min((unsigned)k0 + mchk[q], (unsigned)(p.n_k - 16)),
                  mst + (wave * M_WIN + q) * 1024);
    }
    const char* kg = reinterpret_cast<const char*>(Kb) + (size_t)k0 * C::KRB;
    const char* vg = reinterpret_cast<const char*>(Vb) + (size_t)k0 * C::VRB;
    if (k0 + BN <= p.n_k) {
      #pragma unroll
      for (int q = 0; q < C::K_WIN; ++q)
        lds_dma16(kg, koff[q], st + (wave * C::K_WIN + q) * 1024);
      #pragma unroll
      for (int q = 0; q < C::V_WIN; ++q)
        lds_dma16(vg, voff[q], st + C::KTILE + (wave * C::V_WIN + q) * 1024);
    } else {
      const int last = p.n_k - 1 - k0;
      #pragma unroll
      for (int q = 0; q < C::K_WIN; ++q) {
        const int win = wave * C::K_WIN + q;
        const unsigned off = min(tile_row(win, C::KRB), last) * C::KRB + k_chunk_of(win) * 16;
        lds_dma16(kg, off, st + win * 1024);
      }
      #pragma unroll
      for (int q = 0; q < C::V_WIN; ++q) {
        const int win = wave * C::V_WIN + q;
        const unsigned off = min(tile_row(win, C::VRB), last) * C::VRB + v_chunk_of(win) * 16;
        lds_dma16(vg, off, st + C::KTILE + win * 1024);
      }
    }
  };
  // Per-lane read offsets within a stage (bytes).  K: row kb*32 + l32, chunk
  // 2c + g; the permutation depends on the row only through l32.  V: the
  // transposing read's row 32 kb + 16 st + 8 h + 4 g + (lane % 16) / 4 and
  // columns 32 d + scol; the permutation depends on the row only through
  // 4 g + (lane % 16) / 4, so kb, st and h are immediates.
  int kro[DMA ? C::KCH : 1], vro[DMA ? C::NDV : 1];
  if constexpr (DMA) {
    #pragma unroll
    for (int c = 0; c < C::KCH; ++c)
      kro[c] = l32 * C::KRB + (((2 * c + g) ^ k_swizzle<C::KRB>(l32)) * 16);
    const int vr = 4 * g + ((lane & 15) >> 2);
    const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d) {
      const int ch = (d * 32 + scol) / 8;
      vro[d] = C::KTILE + vr * C::VRB + ((ch ^ v_swizzle<C::VRB>(vr)) * 16) + (scol % 8) * 2;
    }
  }

  if constexpr (DMA) {
    if constexpr (ALDS) {
      if (Ab != nullptr && nblk > blk0) issue_bias(blk0);
    }
    if (nblk > blk0) issue_kv(blk0);
    if (NS == 3 && nblk > blk0 + 1) issue_kv(blk0 + 1);
  } else {
    if (nblk > blk0) {
      load_kv(blk0);
      store_kv(0);
    }
    __syncthreads();
    if (nblk > blk0 + 1) load_kv(blk0 + 1);
  }

  for (int blk = blk0; blk < nblk; ++blk) {
    floatx4 amv[GEN ? NKB : 1][4];
    if constexpr (DMA) {
      // three stages: block blk has landed once only block blk+1's loads are
      // outstanding; after the barrier no wave reads block blk-1, whose
      // stage is refilled with block blk+2.  Two stages: block blk's loads
      // are the only ones outstanding; after the barrier block blk-1's stage
      // is refilled with block blk+1.
      if (NS == 3 && blk + 1 < nblk) wait_vm_lds<C::K_WIN + C::V_WIN + M_WIN>();
      else wait_vm_lds<0>();
      compiler_fence();
      if constexpr (ALDS) {
        if (Ab != nullptr) {
          // this block's bias rows of this wave (issued one block ago, older
          // than the K/V loads of block blk + 1 that may still be in
          // flight): dword group (kb, a) is chunk 8 kb + 2 a + g of row
          // 32 w + l32, in slot chunk ^ (row % 16)
          const unsigned ab = a_lds + (unsigned)(l32 * 256);
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int a = 0; a < 4; ++a) {
              const int c = 8 * kb + 2 * a + g;
              amv[kb][a] = lds_load_at<floatx4>(ab + (unsigned)((c ^ (l32 & 15)) * 16));
            }
          // the wave's reads of its rows complete before it refills them
          asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        }
      }
      __builtin_amdgcn_s_barrier();
      compiler_fence();
      if constexpr (ALDS) {
        if (Ab != nullptr && blk + 1 < nblk) issue_bias(blk + 1);
      }
      if (blk + NS - 1 < nblk) issue_kv(blk + NS - 1);
    }
    const int cur = (blk - blk0) & 1;   // register staging: buffer of this block
    const T* ks = Ks + cur * C::KBUF;
    const T* vs = Vs + cur * C::VBUF;
    // DMA: this block's stage.  Each read pattern gets one base address per
    // block, made opaque so that the compiler keeps it in one register and
    // folds every other offset into the read instructions (left to itself
    // it kept a separate strength-reduced address per read).
    unsigned kaddr[DMA ? C::KCH : 1], vaddr[DMA ? C::NDV : 1];
    if constexpr (DMA) {
      unsigned st_addr = lds_base + (unsigned)((blk % NS) * C::STAGE);
      asm("" : "+s"(st_addr));
      #pragma unroll
      for (int c = 0; c < C::KCH; ++c) {
        kaddr[c] = st_addr + (unsigned)kro[c];
        asm("" : "+v"(kaddr[c]));
      }
      #pragma unroll
      for (int d = 0; d < C::NDV; ++d) {
        vaddr[d] = st_addr + (unsigned)vro[d];
        asm("" : "+v"(vaddr[d]));
      }
    }
    const int k0 = blk * BN;
    // A wave whose rows all precede this block's first key (causal) sees an
    // empty key set here: its summary is the empty state, a no-op merge.
    bool active = (qw < p.n_q) && !(p.causal && k0 > qw + 31);
    // General path with aligned mask rows: this block's boolean / additive
    // mask entries for this lane's keys, four consecutive keys per load
    // (the keys k0 + 32 kb + 8 a + 4 g + j, j < 4, of score slots
    // (kb, 4 a + j)), issued before the score products so that their
    // latency runs under them.  Rows past n_q read nothing (forbidden,
    // zero bias); groups lie wholly inside or past n_k (n_k % 4 == 0).
    // (ALDS: the bias entries were read from LDS at the top of the block.)
    uint32_t gmv[GEN ? NKB : 1][4];
    // MLDS: the wave's 32 x 64 window of the boolean tile decides the block
    // for the whole wave: no allowed entry -> nothing to add (the empty
    // summary, as for an inactive wave); every entry allowed -> the mask step
    // keeps only the causal / padding thresholds (no per-score byte test).
    bool tile_full = false;
    if constexpr (MLDS) {
      if (active) {
        // this lane's row of the block's mask tile: dword (kb, a) holds keys
        // k0 + 32 kb + 8 a + 4 g .. + 3, in chunk 2 kb + a / 2 of the row
        const int mr = wave * 32 + l32, sw = (mr >> 2) & 3;
        unsigned mb = lds_base + (unsigned)(DMA_LDS + (blk % NS) * MT);
        asm("" : "+s"(mb));
        uint32_t all_and = 0xffffffffu, any_set = 0u;
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          #pragma unroll
          for (int h = 0; h < 2; ++h) {
            // dwords a = 2 h and 2 h + 1: bytes 4 g and 8 + 4 g of chunk c
            const int c = 2 * kb + h;
            const unsigned ca = mb + (unsigned)(mr * 64 + ((c ^ sw) * 16) + 4 * g);
            #pragma unroll
            for (int e = 0; e < 2; ++e) {
              const uint32_t x = lds_load_at<uint32_t>(ca + 8u * (unsigned)e);
              gmv[kb][2 * h + e] = x;
              amv[kb][2 * h + e] = floatx4{0.f, 0.f, 0.f, 0.f};
              all_and &= x;
              any_set |= x;
            }
          }
        // rows past n_q hold a copy of row n_q - 1 (never stored): harmless
        // either way
        if (__all(any_set == 0u)) active = false;
        // every entry allowed if bit 0 is set in every byte: exact for 0 / 1
        // entries; other nonzero bytes may fail it and only take the
        // per-score test below
        tile_full = __all((all_and & 0x01010101u) == 0x01010101u);
      }
    }
    if (active) {
      const bool mvec = GEN && (MLDS || p.mask_vec);
      if constexpr (MLDS) {
      } else if constexpr (GEN) {
        if (mvec) {
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int a = 0; a < 4; ++a) {
              const int key = k0 + kb * 32 + 8 * a + 4 * g;
              const bool in = qi < p.n_q && key < p.n_k;
              const size_t at = (size_t)qi * p.n_k + key;
              gmv[kb][a] = 0xffffffffu;
              if (!ALDS) amv[kb][a] = floatx4{0.f, 0.f, 0.f, 0.f};
              if (Gb != nullptr) gmv[kb][a] = in ? *reinterpret_cast<const uint32_t*>(Gb + at) : 0u;
              if (!ALDS && Ab != nullptr && in)
                amv[kb][a] = *reinterpret_cast<const floatx4*>(Ab + at);
            }
        }
      }
      // ---- raw products S^T (NKB sub-blocks of 32 keys) ----------------------
      floatx16 s[NKB];
      // LAZY: from the second block on every row has a finite mu (the first
      // block always holds key 0, which causal and padding masks allow), so
      // the accumulator starts at -mu; the first block starts at 0.
      const bool shifted = LAZY && blk > 0;
      auto raw_scores = [&](bool at_mu) {
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if (at_mu) {
            s[kb] = negmu;
          } else {
            #pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
          }
          #pragma unroll
          for (int c = 0; c < C::KCH; ++c) {
            vec kf;
            if constexpr (DMA)
              kf = lds_load_at<vec>(kaddr[c] + kb * 32 * C::KRB);
            else
              kf = *reinterpret_cast<const vec*>(
                  &ks[(kb * 32 + l32) * C::KPAD + c * 2 * VEC + g * VEC]);
            mfma_chunk(s[kb], kf, qf[c]);
          }
        }
      };
      raw_scores(shifted);
      // value fragments of this block, read ahead of the weights
      // (not in eight-wave workgroups with value rows of 96+ and heads of 128
      // or the exact-shift merge: there the fragments do not fit the
      // registers of two waves per SIMD)
      // (nor with a staged bias tile and the exact-shift merge: the bias
      // entries hold those registers; nor with the boolean tile at three
      // workgroups per CU, which must fit 168 registers)
      constexpr bool VPRE = DMA && !(ALDS && !(ADDONLY && LAZY)) && !(MLDS && OCC >= 3) &&
                            !(WAVES >= 8 && C::NDV > 2 && (DH >= 128 || !LAZY));
      vec vpre[VPRE ? NKB : 1][2][VPRE ? C::NDV : 1];
      if constexpr (VPRE) {
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          #pragma unroll
          for (int st = 0; st < 2; ++st)
            #pragma unroll
            for (int d = 0; d < C::NDV; ++d) {
              const unsigned v0 = vaddr[d] + (kb * 32 + 16 * st) * C::VRB;
              const vec4 lo = lds_read_tr4_at<T>(v0);
              const vec4 hi = lds_read_tr4_at<T>(v0 + 8 * C::VRB);
              vpre[kb][st][d] = vec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
      }

      // ---- mask: forbidden scores become -inf (weight exactly 0) -------------
      // Score slot (kb, i) of this lane is key k0 + off(kb, i) + 4 g with
      // off = 32 kb + 8 (i / 4) + i % 4.  Causal and key padding allow exactly
      // the keys j <= lim = min(qi, kvalid - 1): one compare per score.
      // causal / padding thresholds bite only on boundary blocks
      const bool need_cp = (k0 + BN > kvalid) || (p.causal && k0 + BN - 1 > qw);
      const bool need_mask =
          need_cp || (GEN && ((Gb != nullptr && !tile_full) || Ab != nullptr));
      auto apply_mask = [&]() {
        const int lim = p.causal ? min(qi, kvalid - 1) : kvalid - 1;
        const int t = lim - k0 - 4 * g;
        if constexpr (ADDONLY) {
          // s' = s c' + M log2(e) (prescaled scores: c' = 1); -inf stays -inf
          auto add_bias = [&](auto cp) {
            constexpr bool CP = decltype(cp)::value;
            #pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
              #pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int a = i >> 2, j = i & 3;
                const int off = kb * 32 + 8 * a + j;
                const float v = PRESCALE ? fmaf(amv[kb][a][j], kLog2e, s[kb][i])
                                         : fmaf(s[kb][i], cs0, amv[kb][a][j] * kLog2e);
                s[kb][i] = (!CP || off <= t) ? v : -INFINITY;
              }
          };
          if (need_cp)
            add_bias(std::true_type());
          else
            add_bias(std::false_type());
          return;
        }
        if constexpr (GEN) {
          if (mvec && !tile_full) {
            auto grouped = [&](auto cp) {
              constexpr bool CP = decltype(cp)::value;   // threshold compare needed
              #pragma unroll
              for (int kb = 0; kb < NKB; ++kb)
                #pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const int a = i >> 2, j = i & 3;
                  const int off = kb * 32 + 8 * a + j;
                  const bool ok = (!CP || off <= t) && ((gmv[kb][a] >> (8 * j)) & 0xffu) != 0u;
                  if (Ab != nullptr)
                    s[kb][i] = ok ? fmaf(s[kb][i], cs0, amv[kb][a][j] * kLog2e) : -INFINITY;
                  else
                    s[kb][i] = ok ? s[kb][i] : -INFINITY;
                }
            };
            if (need_cp)
              grouped(std::true_type());
            else
              grouped(std::false_type());
            return;
          }
        }
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          #pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = kb * 32 + 8 * (i >> 2) + (i & 3);
            bool ok = off <= t;
            if (GEN && Gb != nullptr && !tile_full && ok)
              ok = qi < p.n_q && Gb[(size_t)qi * p.n_k + k0 + off + 4 * g] != 0;
            if (GEN && Ab != nullptr) {
              // an allowed key has index <= lim < n_k, and qi < n_q is checked
              const float mb =
                  (ok && qi < p.n_q) ? Ab[(size_t)qi * p.n_k + k0 + off + 4 * g] : 0.f;
              s[kb][i] = ok ? fmaf(s[kb][i], cs0, mb * kLog2e) : -INFINITY;
            } else {
              s[kb][i] = ok ? s[kb][i] : -INFINITY;
            }
          }
      };
      if (need_mask) apply_mask();
      auto block_max = [&]() {
        float mx = -INFINITY;
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          #pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        return half_max(mx);
      };
      // rescale the running (l, z) by a (a row's shift moved up)
      auto rescale = [&](float a) {
        l_run *= a;
        #pragma unroll
        for (int d = 0; d < C::NDV; ++d)
          #pragma unroll
          for (int i = 0; i < 16; ++i) o[d][i] *= a;
      };

      if constexpr (LAZY && !STATS) {
        if (!shifted) {
          // first block: the exact block maximum becomes mu (masked: -inf
          // stays -inf, see negmu)
          const float mx = block_max();
          const float mu_use = (mx == -INFINITY) ? 0.f : mx;
          mu = MASKED ? mx : mu_use;
          #pragma unroll
          for (int i = 0; i < 16; ++i) negmu[i] = -mu;
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i] - mu_use);
        } else {
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i]);
        }
      } else if constexpr (LAZY) {
        const float mx = block_max();
        if (shifted) {
          // mx = (block maximum) - mu for every row (-inf: no allowed key)
          m_run = fmaxf(m_run, mx + mu);
          if (__any(mx > kLazyTau)) {       // some row ran too far above its shift
            const float dmu = fmaxf(mx, 0.f);  // move mu to max(mu, block max)
            rescale(__builtin_amdgcn_exp2f(-dmu));
            #pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
              #pragma unroll
              for (int i = 0; i < 16; ++i) s[kb][i] -= dmu;
            mu += dmu;
            #pragma unroll
            for (int i = 0; i < 16; ++i) negmu[i] = -mu;
          }
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i]);
        } else {
          // first block: the exact block maximum becomes both m and mu
          m_run = mx;
          mu = (mx == -INFINITY) ? 0.f : mx;
          #pragma unroll
          for (int i = 0; i < 16; ++i) negmu[i] = -mu;
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = __builtin_amdgcn_exp2f(s[kb][i] - mu);
        }
      } else {
        // ---- merge: new shift, rescale the running summary ------------------
        const float mx = block_max();
        const float mblk = (mx == -INFINITY) ? -INFINITY : mx * cs;
        const float m_new = fmaxf(m_run, mblk);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        if (__any(alpha != 1.0f)) rescale(alpha);   // some row's maximum moved
        if (need_mask && !(cs > 0.f)) {
          // a forbidden score is -inf, whose weight 2^(-inf) is 0; with c = 0
          // the product -inf * 0 would be NaN, so there the weight is set to
          // 0 explicitly
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][i], cs, -m_use));
              s[kb][i] = (s[kb][i] == -INFINITY) ? 0.f : e;
            }
        } else {
          #pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            #pragma unroll
            for (int i = 0; i < 16; ++i)
              s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], cs, -m_use));
        }
      }

      // ---- z += P V  (as O^T += V^T P^T), l += sum of the rounded weights --
      if constexpr (C::TR) {
        // weights rounded to T, in the B-operand layout of the value product;
        // slot t of chunk (kb, st) is key kb*32 + 16*st + 4*g + t (t < 4) or
        // kb*32 + 16*st + 8 + 4*g + (t - 4) (t >= 4), as in the score block.
        vec pb[NKB][2];
        float bsum = 0.f;
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          #pragma unroll
          for (int st = 0; st < 2; ++st) {
            floatx8 pf;
            #pragma unroll
            for (int t = 0; t < 8; ++t) pf[t] = s[kb][8 * st + t];
            pb[kb][st] = Cvt<T>::eight(pf);
            bsum = sum8(pb[kb][st], bsum);
          }
        if constexpr (LAZY && !STATS) {
          if (shifted && __any(!(bsum <= kLazyLimit))) {
            // rare: some weight exceeded 2^tau (or overflowed).  Redo the
            // block from its raw scores with mu moved to the exact maximum.
            raw_scores(false);
            if (need_mask) apply_mask();
            const float mx = block_max();
            const float mu_new = fmaxf(mu, mx);
            // masked rows may still have no allowed key (mu_new = -inf):
            // nothing to rescale, weights 0
            const float mu_use = (MASKED && mu_new == -INFINITY) ? 0.f : mu_new;
            rescale((MASKED && mu_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mu - mu_new));
            mu = mu_new;
            #pragma unroll
            for (int i = 0; i < 16; ++i) negmu[i] = -mu;
            bsum = 0.f;
            #pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
              #pragma unroll
              for (int st = 0; st < 2; ++st) {
                floatx8 pf;
                #pragma unroll
                for (int t = 0; t < 8; ++t)
                  pf[t] = __builtin_amdgcn_exp2f(s[kb][8 * st + t] - mu_use);
                pb[kb][st] = Cvt<T>::eight(pf);
                bsum = sum8(pb[kb][st], bsum);
              }
          }
        }
        l_run += bsum;
        const int srow = 4 * g + ((lane & 15) >> 2);
        const int scol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          #pragma unroll
          for (int st = 0; st < 2; ++st)
            #pragma unroll
            for (int d = 0; d < C::NDV; ++d) {
              if constexpr (VPRE) {
                mfma_chunk(o[d], vpre[kb][st][d], pb[kb][st]);
              } else if constexpr (DMA) {
                const unsigned v0 = vaddr[d] + (kb * 32 + 16 * st) * C::VRB;
                const vec4 lo = lds_read_tr4_at<T>(v0);
                const vec4 hi = lds_read_tr4_at<T>(v0 + 8 * C::VRB);
                mfma_chunk(o[d], vec{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]},
                           pb[kb][st]);
              } else {
                const T* v0 = &vs[(kb * 32 + 16 * st + srow) * C::VROW + d * 32 + scol];
                const vec4 lo = lds_read_tr4<T>(v0);
                const vec4 hi = lds_read_tr4<T>(v0 + 8 * C::VROW);
                const vec va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                mfma_chunk(o[d], va, pb[kb][st]);
              }
            }
      } else {
        #pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          #pragma unroll
          for (int a = 0; a < 4; ++a) {
            const floatx4 pf = {s[kb][4 * a], s[kb][4 * a + 1], s[kb][4 * a + 2],
                                s[kb][4 * a + 3]};
            l_run += (pf[0] + pf[1]) + (pf[2] + pf[3]);
            #pragma unroll
            for (int d = 0; d < C::NDV; ++d) {
              const floatx4 va = *reinterpret_cast<const floatx4*>(
                  &vs[(d * 32 + l32) * C::VROW + kb * 32 + 8 * a + 4 * g]);
              mfma_chunk(o[d], va, pf);
            }
          }
        }
      }
    }
    if constexpr (!DMA) {
      if (blk + 1 < nblk) store_kv(cur ^ 1);  // next block into the other buffer
      __syncthreads();
      if (blk + 2 < nblk) load_kv(blk + 2);   // in flight during the next block
    }
  }

  // ---- finalise: z / l, store into the concatenation --------------------------
  float l_tot = half_sum(l_run);
  if constexpr (SPLIT) {
    // this partition's summary of each row: (m, l, z) at shift m, base 2
    if (qi < p.n_q) {
      const size_t pr = ((size_t)sp * BH + bh) * p.n_q + qi;
      #pragma unroll
      for (int d = 0; d < C::NDV; ++d) {
        #pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int e0 = d * 32 + 8 * a + 4 * g;
          store4(p.part_z, kF32, pr * p.d_vh + e0, (p.d_vh % 4) == 0, dvh - e0, o[d][4 * a],
                 o[d][4 * a + 1], o[d][4 * a + 2], o[d][4 * a + 3]);
        }
      }
      if (g == 0) {
        p.part_m[pr] = m_run;
        p.part_l[pr] = l_tot;
      }
    }
    return;
  }
  const float inv = 1.0f / l_tot;
  if constexpr (LAZY && STATS) {
    // l at the exact maximum: l* e^(mu - m)   (z / l is unchanged)
    if (m_run != -INFINITY) l_tot *= __builtin_amdgcn_exp2f(mu - m_run);
  }
  if (qi < p.n_q) {
    const size_t zbase = ((size_t)b * p.n_q + qi) * p.ldz + (size_t)r * p.d_vh;
    #pragma unroll
    for (int d = 0; d < C::NDV; ++d) {
      #pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int e0 = d * 32 + 8 * a + 4 * g;
        store4(p.Z, p.out_dtype, zbase + e0, p.vec_z, dvh - e0, o[d][4 * a] * inv,
               o[d][4 * a + 1] * inv, o[d][4 * a + 2] * inv, o[d][4 * a + 3] * inv);
      }
    }
    if (STATS && g == 0) {
      const size_t ri = (size_t)bh * p.n_q + qi;
      if (p.row_m) p.row_m[ri] = (m_run == -INFINITY) ? -INFINITY : m_run * kLn2;
      if (p.row_l) p.row_l[ri] = l_tot;
    }
  }
}

}  // namespace mha
