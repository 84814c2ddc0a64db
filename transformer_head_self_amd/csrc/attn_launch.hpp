// Head-width dispatch for the fused attention kernel of one element type.
#pragma once

#include "attn.hpp"
#include "attn_decode.hpp"
#include "attn_pipe.hpp"
#include "attn_pipe3.hpp"

namespace mha {

#ifndef MHA_ATTN_WAVES
#define MHA_ATTN_WAVES 4
#endif
#ifndef MHA_ATTN_BN
#define MHA_ATTN_BN 64
#endif
#ifndef MHA_ATTN_PIPE
#define MHA_ATTN_PIPE 1
#endif
#ifndef MHA_PIPE_NS
#define MHA_PIPE_NS 4
#endif
#ifndef MHA_PIPE_OCC
#define MHA_PIPE_OCC 2
#endif
#ifndef MHA_ATTN_PIPE3
#define MHA_ATTN_PIPE3 1
#endif


template <typename T, int DH, int DV>
hipError_t launch_attn_fixed(AttnParams p, hipStream_t stream) {
  constexpr int WAVES = MHA_ATTN_WAVES;
  constexpr int BN = sizeof(T) == 4 ? 64 : MHA_ATTN_BN;  // fp32 tiles stay at 64 keys (LDS)
  typedef AttnCfg<T, DH, DV, WAVES, BN> C;
  p.num_q_tiles = (p.n_q + C::QT - 1) / C::QT;
  const long long grid = (long long)p.num_q_tiles * p.B * p.h;
  if (grid <= 0) return hipSuccess;
  const bool fast = p.d_h == DH && p.d_vh == DV && p.vec_q && p.vec_k && p.vec_v &&
                    p.allowed == nullptr && p.add == nullptr;
  // The deferred-shift variant is used for the fast path (causal / key
  // padding masks only, where every row's first block holds an allowed key)
  // except for bf16, whose extra rounding of the scaled query would cost
  // accuracy.
  constexpr bool lazy = !__is_same(T, bf16);
  // Three waves per SIMD (at most 168 VGPRs) for the fp16 fast path with
  // head widths up to 64: measured 6-8 % faster than two; wider heads need
  // more registers than that.
  constexpr int occ = (__is_same(T, f16) && DH <= 64 && DV <= 64) ? 3 : 1;
  // Without requested row statistics the 2-byte deferred-shift variant
  // skips the running maximum (block-sum trigger).
  const bool stats = p.row_m != nullptr || p.row_l != nullptr;
  // Boolean masks and additive biases on exact-width 2-byte heads with
  // aligned mask rows: the direct-load kernel; the boolean tile (16-byte
  // aligned rows) and the bias alone have variants of their own, which run
  // the deferred shift when no row statistics are requested (a row whose
  // first key blocks allow nothing keeps its shift unset until its first
  // allowed block, which goes down the exact redo); every other combination
  // runs the exact-shift merge.
  if constexpr (sizeof(T) == 2) {
    const bool fast_masked = p.d_h == DH && p.d_vh == DV && p.vec_q && p.vec_k && p.vec_v &&
                             (p.allowed != nullptr || p.add != nullptr) && p.mask_vec;
    if (fast_masked) {
      constexpr int occm = (DH <= 64 && DV <= 64) ? 2 : 1;
      // the boolean tile with the deferred shift at d = 64: three workgroups
      // per CU on two LDS stages (48 KB) and 168 registers, measured against
      // two workgroups on three stages (72 KB) in one process: 176.7-178.1
      // against 190.7-191.5 us at B = 4, T = 4096, h = 16, causal
      constexpr int occb = (DH == 64 && DV == 64) ? 3 : occm;
      // a boolean mask alone with 16-byte aligned rows travels into LDS with
      // the K/V tiles; otherwise each lane loads its mask entries
      // an additive bias alone: the one-FMA mask step, with the deferred
      // shift when no row statistics are requested
      if (p.allowed == nullptr && p.add != nullptr && lazy && !stats)
        hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, true, occm, false, false, 3>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      else if (p.allowed == nullptr && p.add != nullptr)
        hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, false, occm, true, false, 3>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      else if (p.allowed != nullptr && p.add == nullptr && p.mask_g16 && lazy && !stats)
        hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, true, occb, false, false, 2>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      else if (p.allowed != nullptr && p.add == nullptr && p.mask_g16)
        hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, false, occm, true, false, 2>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      else
        hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, false, occm, true, false, 1>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      return hipGetLastError();
    }
  }
  // Eight waves per workgroup (256 query rows) for 2-byte heads of 64 or 128
  // with at least one of the two widths 128: there a four-wave workgroup
  // runs one wave per SIMD (its direct-load stages, 72-128 KB, or its
  // registers leave room for no second one), and two waves per SIMD now
  // share each K/V tile (each 1 KB load window owned by one wave).
  // Measured in one process (causal; d = 128 at B = 1 with 16k tokens, the
  // mixed widths at B = 2 with 8k): d = 128 fp16 heads 1172 -> 968 us
  // without row statistics and 1358 -> 987 us with them, bf16 heads
  // 1575 -> 1093 us; d_h = 64 with d_vh = 128 524 -> 401 us, d_h = 128
  // with d_vh = 64 503 -> 403 us (fp16, no statistics); the other
  // mixed-width cases within 2 % either way.
  constexpr bool wide8 = sizeof(T) == 2 && (DH == 64 || DH == 128) &&
                         (DV == 64 || DV == 128) && (DH == 128 || DV == 128);
  if constexpr (wide8) {
    if (fast) {
      typedef AttnCfg<T, DH, DV, 8, 64> C8;
      p.num_q_tiles = (p.n_q + C8::QT - 1) / C8::QT;
      const long long g8 = (long long)p.num_q_tiles * p.B * p.h;
      if constexpr (lazy) {
        if (!stats) {
          hipLaunchKernelGGL((attn_pipe_kernel<T, DH, DV, 4, 1, 8>), dim3((unsigned)g8),
                             dim3(C8::NT), 0, stream, p);
          return hipGetLastError();
        }
      }
      hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, 8, 64, true, lazy, 1>), dim3((unsigned)g8),
                         dim3(C8::NT), 0, stream, p);
      return hipGetLastError();
    }
  }
#if MHA_ATTN_PIPE3
  // fp16 heads of 64 without row statistics and without the causal rule:
  // the three-stage pipelined kernel (matrix work of the neighbouring blocks
  // interleaved with each block's exponentials).  Measured in one process
  // against attn_fwd_kernel: 49.7 vs 51.7 us (B 16, 12 heads, 512 queries
  // against 2048 padded keys), 14.9 vs 15.5 us (B 2, 8 heads, 1000 tokens,
  // key padding); with the causal rule its pipeline fill and drain per wave
  // cost more than they save (154 vs 146 us at B 4, 16 heads, 4096 tokens).
  if constexpr (__is_same(T, f16) && DH == 64 && DV == 64 && WAVES == 4 && BN == 64) {
    if (fast && !stats && !p.causal) {
      hipLaunchKernelGGL((attn_fwd3_kernel<T, DH, DV, 2>), dim3((unsigned)grid), dim3(C::NT), 0,
                         stream, p);
      return hipGetLastError();
    }
  }
#endif
  if constexpr (lazy && sizeof(T) == 2) {
    if (fast && !stats) {
      // The software-pipelined kernel wins where a block carries more matrix
      // work per weight (value rows of 96: measured 30 % faster, two
      // workgroups per CU); for narrower heads three unpipelined waves per
      // SIMD are faster (measured 7 %).
      if constexpr (MHA_ATTN_PIPE && (DV >= 96 || DH >= 128)) {
        static_assert(WAVES == 4 && BN == 64, "the pipelined kernel's tile");
        hipLaunchKernelGGL((attn_pipe_kernel<T, DH, DV, MHA_PIPE_NS, MHA_PIPE_OCC>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      } else {
        hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, lazy, occ, false>),
                           dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
      }
      return hipGetLastError();
    }
  }
  if (fast)
    hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, lazy, occ>),
                       dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, false>), dim3((unsigned)grid),
                       dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_attn_dv(const AttnParams& p, hipStream_t stream) {
  if (p.d_vh <= 32) return launch_attn_fixed<T, DH, 32>(p, stream);
  if (p.d_vh <= 64) return launch_attn_fixed<T, DH, 64>(p, stream);
  if (p.d_vh <= 96) return launch_attn_fixed<T, DH, 96>(p, stream);
  if (p.d_vh <= 128) return launch_attn_fixed<T, DH, 128>(p, stream);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_attn_typed(const AttnParams& p, hipStream_t stream) {
  if (p.d_h <= 32) return launch_attn_dv<T, 32>(p, stream);
  if (p.d_h <= 64) return launch_attn_dv<T, 64>(p, stream);
  if (p.d_h <= 128) return launch_attn_dv<T, 128>(p, stream);
  return hipErrorInvalidValue;
}

// Key-split form: one workgroup per (query tile, batch*head, key partition),
// writing partial summaries (the merge launch follows in launch_attention_split).
template <typename T, int DH, int DV>
hipError_t launch_attn_split_fixed(AttnParams p, hipStream_t stream) {
  constexpr int WAVES = MHA_ATTN_WAVES;
  constexpr int BN = 64;
  typedef AttnCfg<T, DH, DV, WAVES, BN> C;
  p.num_q_tiles = (p.n_q + C::QT - 1) / C::QT;
  const long long grid = (long long)p.num_q_tiles * p.B * p.h * p.splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 2147483647LL) return hipErrorInvalidValue;
  const bool fast = p.d_h == DH && p.d_vh == DV && p.vec_q && p.vec_k && p.vec_v &&
                    p.allowed == nullptr && p.add == nullptr;
  if (fast)
    hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, true, false, 1, true, true>),
                       dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<T, DH, DV, WAVES, BN, false, false, 1, true, true>),
                       dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t launch_attn_split_dv(const AttnParams& p, hipStream_t stream) {
  if (p.d_vh <= 32) return launch_attn_split_fixed<T, DH, 32>(p, stream);
  if (p.d_vh <= 64) return launch_attn_split_fixed<T, DH, 64>(p, stream);
  if (p.d_vh <= 96) return launch_attn_split_fixed<T, DH, 96>(p, stream);
  if (p.d_vh <= 128) return launch_attn_split_fixed<T, DH, 128>(p, stream);
  return hipErrorInvalidValue;
}

// Decode-shaped partitions: one to four query rows, 2-byte rows of up to 128
// elements in whole 16-byte chunks.
template <typename T, int G, int NQ>
hipError_t launch_attn_decode(const AttnParams& p, hipStream_t stream) {
  const long long grid = (long long)p.B * p.h * p.splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 2147483647LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_decode_kernel<T, G, NQ>), dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int G>
hipError_t launch_attn_decode_nq(const AttnParams& p, hipStream_t stream) {
  if (p.n_q == 1) return launch_attn_decode<T, G, 1>(p, stream);
  if (p.n_q == 2) return launch_attn_decode<T, G, 2>(p, stream);
  return launch_attn_decode<T, G, 4>(p, stream);
}

template <typename T>
bool decode_applies(const AttnParams& p) {
  return sizeof(T) == 2 && p.n_q <= 4 && p.d_h % 8 == 0 && p.d_vh % 8 == 0 && p.d_h <= 128 &&
         p.d_vh <= 128 && p.vec_q && p.vec_k && p.vec_v;
}

template <typename T>
hipError_t launch_attn_split_typed(const AttnParams& p, hipStream_t stream) {
  if constexpr (sizeof(T) == 2) {
    if (decode_applies<T>(p)) {
      const int w = p.d_h > p.d_vh ? p.d_h : p.d_vh;
      if (w <= 32) return launch_attn_decode_nq<T, 4>(p, stream);
      if (w <= 64) return launch_attn_decode_nq<T, 8>(p, stream);
      return launch_attn_decode_nq<T, 16>(p, stream);
    }
  }
  if (p.d_h <= 32) return launch_attn_split_dv<T, 32>(p, stream);
  if (p.d_h <= 64) return launch_attn_split_dv<T, 64>(p, stream);
  if (p.d_h <= 128) return launch_attn_split_dv<T, 128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace mha
