// rfpx_impl.hpp -- internal definitions shared by the librfpx sources:
// format constants, the device image and workspace layouts, the lane
// geometry of the expert kernels, and the register-level block decode.
//
// Block decode on gfx950.  The gate/up products (and prefill's operands)
// run on v_dot2c_f32_bf16 (two bf16 products added into an fp32
// accumulator per lane per issue); the decode kernels' down products use
// the exact-code form further below (CodeGroups).
// A packed code c is turned into a bf16 value by masking it into the
// mantissa of 1.0 (0x3F80): a code whose lowest bit lands at mantissa bit k
// gives 1 + c * 2^(k-7).  One v_and_or_b32 builds a pair word (two codes,
// one per bf16 half) from a shifted copy of the code dword, and one shift
// serves several pairs, so the decode costs 0.6 (FP2) to 1 (FP3) VALU op
// per weight, shared by all columns.  The factor 2^(7-k) of each code and
// the code offset (1.5, 3.5, 7.5) are folded into "prepared" activations,
// computed once per step: the activation of a code at position k is stored
// times 2^(7-k) (exact), and each block's accumulator starts at
// -sum (2^(7-k) + offset) * x, so that
//      sum_j (c_j - offset) x_j  =  start + sum_pairs dot2(v, xpair).
// v and the bf16 activations are exact and each bf16 product is exact in
// fp32, so the only rounding is fp32 accumulation.
//
// Pairings (lo code, hi code) of the 16 pairs of one block (bf16 lo half in
// bits 0..15 of the pair word, hi half in 16..31), with the code's mantissa
// position k:
//   FP2  code dword t (t < 2) holds codes 16t..16t+15; pair 8t+i joins
//        codes 16t+i and 16t+i+8, taken from the dword shifted right by
//        0 (i = 0..2), 6 (i = 3..5) or 12 (i = 6, 7); k = 0, 2, 4, 0, 2, 4,
//        0, 2 for i = 0..7, the same in both halves.
//   FP4  code dword t (t < 4) holds codes 8t..8t+7; pair 4t+i joins codes
//        8t+i and 8t+i+4; i = 0 at k = 0 (no shift), i = 1, 2, 3 at k = 3
//        (shift right 1, 5, 9).
//   FP3  pairs 0..9: codes (lo, lo+5), lo in {0..4, 10..14}; lo at bits
//        4-6 (k = 4), hi at bits 19-21 (k = 3).  Pairs 10..15: codes
//        (lo, lo+6), lo in 20..25; lo at bits 2-4 (k = 2), hi at bits 20-22
//        (k = 4).  Window: bits 3lo-4 (resp. 3lo-2) of the 96-bit code word,
//        taken with one v_alignbit_b32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <utility>

#include "../../include/rfpx.h"

namespace rfpx {

constexpr int kQMax = RFPX_Q_MAX;
constexpr int kKMax = RFPX_K_MAX;
constexpr int kEMax = RFPX_E_MAX;
constexpr int kMaxSlots = kQMax * kKMax + 1;  // routed unique experts + shared
constexpr uint32_t kMagic = 0x58504652u;      // "RFPX"
constexpr uint32_t kVersion = 1;

__host__ __device__ constexpr int code_bytes(int fmt) {
  return fmt == RFPX_FP2 ? 8 : fmt == RFPX_FP3 ? 12 : fmt == RFPX_FP4 ? 16 : 0;
}
__host__ __device__ constexpr int scale_bytes(int fmt) {
  return fmt == RFPX_FP4 ? 1 : (fmt == RFPX_FP2 || fmt == RFPX_FP3) ? 2 : 0;
}
__host__ __device__ constexpr int blk_bytes(int fmt) {
  return code_bytes(fmt) + scale_bytes(fmt);
}
__host__ __device__ constexpr bool valid_fmt(int fmt) {
  return fmt == RFPX_FP2 || fmt == RFPX_FP3 || fmt == RFPX_FP4;
}
// A lane reads one "chunk" per step: two FP2 blocks (16 B of codes), one FP3
// block (12 B) or one FP4 block (16 B).
__host__ __device__ constexpr int chunk_blocks(int fmt) {
  return fmt == RFPX_FP2 ? 2 : 1;
}
// ----------------------------------------------------------------- image

struct ImageHeader {
  uint32_t magic, version;
  int32_t d, f, E, reserved;
  uint64_t total;
  uint64_t pad[4];
};
static_assert(sizeof(ImageHeader) == 64, "header is 64 B");

struct ExpertDesc {
  uint64_t codes[3];   // byte offset of the codes plane of gate, up, down
  uint64_t scales[3];  // byte offset of the scales plane
  int32_t fmt[3];
  int32_t reserved;
};
static_assert(sizeof(ExpertDesc) == 64, "expert entry is 64 B");

constexpr size_t kImgTable = 64;  // table offset

__host__ __device__ __forceinline__ size_t align_up(size_t v, size_t a) {
  return (v + a - 1) / a * a;
}

// ------------------------------------------------------------ lane geometry
// A matrix row of `cols` columns is cpl chunks.  With cpl >= 64 a wave owns
// one row per step and lane l takes chunks l, l+64, ... (tpl of them); with
// cpl < 64 a wave covers rpi = 64/cpl rows per step, cpl lanes per row.
struct Geo {
  int cpl, lpr, rpi, tpl;
};

__host__ __device__ __forceinline__ bool make_geo(int fmt, int cols, Geo *g) {
  if (!valid_fmt(fmt) || cols <= 0 || cols % 32) return false;
  int nb = cols / 32, cb = chunk_blocks(fmt);
  if (nb % cb) return false;
  int cpl = nb / cb;
  if (cpl >= 64) {
    if (cpl % 64) return false;
    g->lpr = 64;
    g->rpi = 1;
    g->tpl = cpl / 64;
  } else {
    if (cpl & (cpl - 1)) return false;
    g->lpr = cpl;
    g->rpi = 64 / cpl;
    g->tpl = 1;
  }
  g->cpl = cpl;
  return true;
}

// ---------------------------------------------------------- workspace
// Route table written by the router kernel, read by the expert kernels.
struct RouteTable {
  int32_t nslots;  // 1 + number of distinct routed experts; slot 0 = shared
  int32_t pad[31];
  int32_t expert[kMaxSlots];
  int32_t ncols[kMaxSlots];
  uint32_t mask[kMaxSlots];
  int32_t cols[kMaxSlots][kQMax];
  float w[kMaxSlots][kQMax];      // gating weight of cols[s][i]
  int32_t ids[kQMax][kKMax];      // top-k per column
  float gw[kQMax][kKMax];         // gating weight per column and rank
  // each slot's down matrix in the image (from the expert table), so that
  // the down kernel needs one dependent read instead of two
  uint64_t dn_codes[kMaxSlots];
  uint64_t dn_scales[kMaxSlots];
  int32_t dn_fmt[kMaxSlots];
  // and its gate and up planes (steps of several columns), so that a gate/up
  // workgroup finds everything it needs in one round of loads
  uint64_t gu_codes[kMaxSlots][2];
  uint64_t gu_scales[kMaxSlots][2];
  int32_t gu_fmt[kMaxSlots];
};

struct WsLayout {
  size_t route;     // RouteTable
  size_t scores;    // fp32 [q][E]
  size_t xp;        // u32  [3 fmts][q][nb_d][vx][16]  prepared activations
  size_t xnc;       // fp32 [3][q][nb_d]               their accumulator starts
  size_t hp;        // fp32 [slots][q][f]              h rows
  size_t total;
  int max_slots;
};

// Rows per wave unit of the expert kernels: one-column passes of FP3/FP4
// take 8 rows (a 64-lane row of FP4 codes is 1 KiB, so 8 rows of gate and
// up keep 17 KiB in flight per wave); everything else takes 4, which keeps
// two-column passes within the register budget of two waves per SIMD.
__host__ __device__ constexpr int unit_rows_for(int fmt, int g) {
  return (g == 1 && fmt != RFPX_FP2) ? 8 : 4;
}
// Gate/up workgroup shape by step width (waves; smallest tile in rows).
#ifndef RFPX_GU_WAVES_Q1
#define RFPX_GU_WAVES_Q1 8
#endif
#ifndef RFPX_GU_ROWS_Q1
#define RFPX_GU_ROWS_Q1 32
#endif
#ifndef RFPX_GU_WAVES_QN
#define RFPX_GU_WAVES_QN 4
#endif
#ifndef RFPX_GU_ROWS_QN
#define RFPX_GU_ROWS_QN 32
#endif
// Down workgroups of steps of several columns: one per CU, 12 waves (three
// per SIMD; 8 measured 2.5% slower at five columns, 16 spills).
#ifndef RFPX_DN_WAVES_QN
#define RFPX_DN_WAVES_QN 12
#endif
#ifndef RFPX_DN_ROWS_QN
#define RFPX_DN_ROWS_QN 16
#endif
constexpr int kGuWavesQ1 = RFPX_GU_WAVES_Q1, kGuRowsQ1 = RFPX_GU_ROWS_Q1;
constexpr int kGuWavesQn = RFPX_GU_WAVES_QN, kGuRowsQn = RFPX_GU_ROWS_QN;
#ifndef RFPX_DN_WAVES_Q1
#define RFPX_DN_WAVES_Q1 8
#endif
#ifndef RFPX_DN_ROWS_Q1
#define RFPX_DN_ROWS_Q1 1
#endif
constexpr int kDnWavesQn = RFPX_DN_WAVES_QN, kDnRowsQn = RFPX_DN_ROWS_QN;
constexpr int kDnWavesQ1 = RFPX_DN_WAVES_Q1, kDnRowsQ1 = RFPX_DN_ROWS_Q1;

// Gate/up units of steps of several columns are 2 rows: a wave keeps the
// next unit's loads in flight while it decodes one (two register sets), and
// 2-row sets keep the kernel at three waves per SIMD (4-row sets measured
// 4% slower at two); one-column steps keep single sets of unit_rows_for
// rows.
__host__ __device__ constexpr int unit_rows_gu(int fmt, int g) {
  return g == 1 ? unit_rows_for(fmt, 1) : 2;
}

// ------------------------------------------------------------ device side
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// One halving step of a multi-value reduction: lanes paired by the DPP
// involution CTRL (which flips lane bit B, and maybe lower bits that no
// earlier step has used) split each pair of values between them: the lane
// with bit B clear keeps the even value plus its partner's even value, the
// other the odd one.
template <int CTRL, int B, int N>
__device__ __forceinline__ void ms_step(const float (&v)[N], float (&w)[N / 2], int lane) {
  const bool odd = (lane >> B) & 1;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const float keep = odd ? v[2 * i + 1] : v[2 * i];
    const float send = odd ? v[2 * i] : v[2 * i + 1];
    w[i] = keep + dpp_f<CTRL>(send);
  }
}

// v[l] + v[l ^ 16] + v[l ^ 32] + v[l ^ 48] in every lane l, without LDS:
// v_permlane16_swap / v_permlane32_swap with both operands v give the two
// halves of each exchange, so one add completes it (fp32 addition is
// commutative, so every lane of a pair gets the same bits).
__device__ __forceinline__ float cross_row_sum(float r) {
  const uint32_t u = __float_as_uint(r);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  r = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const uint32_t w = __float_as_uint(r);
  const auto p32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// Sums of N values (N = 2, 4, 8, 16) over the 64 lanes of a wave, all at
// once: log2(N) halving steps over lane bits 3, 2, 1, 0 (row_mirror,
// row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2], in that order,
// so that each step's partner agrees on every bit used before), plain DPP
// sums over the remaining bits of a 16-lane row, and cross_row_sum across
// the four rows.  Lane l then holds the total of value ms_index<N>(l); the
// lanes ms_writer<N>(l) hold each value once.  About 3N + 8 VALU ops
// instead of 14 per value.
template <int N>
__device__ __forceinline__ float multi_sum(const float (&v)[N], int lane) {
  float r;
  if constexpr (N == 1) {
    r = v[0];
    r += dpp_f<0x140>(r);
    r += dpp_f<0x141>(r);
    r += dpp_f<0x4E>(r);
    r += dpp_f<0xB1>(r);
  } else {
    float a[N / 2];
    ms_step<0x140, 3, N>(v, a, lane);
    if constexpr (N == 2) {
      r = a[0];
      r += dpp_f<0x141>(r);
      r += dpp_f<0x4E>(r);
      r += dpp_f<0xB1>(r);
    } else {
      float b[N / 4];
      ms_step<0x141, 2, N / 2>(a, b, lane);
      if constexpr (N == 4) {
        r = b[0];
        r += dpp_f<0x4E>(r);
        r += dpp_f<0xB1>(r);
      } else {
        float c[N / 8];
        ms_step<0x4E, 1, N / 4>(b, c, lane);
        if constexpr (N == 8) {
          r = c[0] + dpp_f<0xB1>(c[0]);
        } else {
          static_assert(N == 16, "multi_sum: N must be 1, 2, 4, 8 or 16");
          float d[1];
          ms_step<0xB1, 0, 2>(c, d, lane);
          r = d[0];
        }
      }
    }
  }
  return cross_row_sum(r);
}

template <int N>
__device__ __forceinline__ int ms_index(int lane) {
  const int b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1, b0 = lane & 1;
  if (N == 1) return 0;
  if (N == 2) return b3;
  if (N == 4) return b3 + 2 * b2;
  if (N == 8) return b3 + 2 * b2 + 4 * b1;
  return b3 + 2 * b2 + 4 * b1 + 8 * b0;
}

template <int N>
__device__ __forceinline__ bool ms_writer(int lane) {
  if (lane >= 16) return false;
  if (N == 1) return lane == 0;
  if (N == 2) return (lane & 7) == 0;
  if (N == 4) return (lane & 3) == 0;
  if (N == 8) return (lane & 1) == 0;
  return true;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __uint_as_float(b << 16);
}
// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc,
                                         false);
}

// (x & m) | o.  With the OR constant held in a vector register (o from
// one_one_vgpr) the compiler emits one v_and_or_b32 per pair word; with two
// literal constants it emits a separate AND and OR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  return (x & m) | o;
}
// The bf16 pair (1.0, 1.0) in a vector register the compiler cannot fold
// back into a literal.
__device__ __forceinline__ uint32_t one_one_vgpr() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(r));
  return r;
}

// The same constant from an asm statement without side effects: it orders
// no memory access, so wave-uniform loads after it can still be scalar
// loads (an asm volatile counts as a possible store for that analysis).
__device__ __forceinline__ uint32_t one_one_vgpr_pure() {
  uint32_t r;
  asm("v_mov_b32 %0, 0x3f803f80" : "=v"(r));
  return r;
}

// Decode the codes of one block into its 16 bf16 pair words (see the header
// comment for the pairings).  `w` holds the block's code dwords: 2 (FP2),
// 3 (FP3) or 4 (FP4); `one` is one_one_vgpr().
template <int FMT>
__device__ __forceinline__ void decode_pairs(const uint32_t *w, uint32_t *p, uint32_t one);

template <>
__device__ __forceinline__ void decode_pairs<RFPX_FP2>(const uint32_t *w, uint32_t *p,
                                                       uint32_t one) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t v = w[t], v6 = v >> 6, v12 = v >> 12;
    p[8 * t + 0] = and_or(v, 0x00030003u, one);
    p[8 * t + 1] = and_or(v, 0x000C000Cu, one);
    p[8 * t + 2] = and_or(v, 0x00300030u, one);
    p[8 * t + 3] = and_or(v6, 0x00030003u, one);
    p[8 * t + 4] = and_or(v6, 0x000C000Cu, one);
    p[8 * t + 5] = and_or(v6, 0x00300030u, one);
    p[8 * t + 6] = and_or(v12, 0x00030003u, one);
    p[8 * t + 7] = and_or(v12, 0x000C000Cu, one);
  }
}

template <>
__device__ __forceinline__ void decode_pairs<RFPX_FP4>(const uint32_t *w, uint32_t *p,
                                                       uint32_t one) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t v = w[t];
    p[4 * t + 0] = and_or(v, 0x000F000Fu, one);
    p[4 * t + 1] = and_or(v >> 1, 0x00780078u, one);
    p[4 * t + 2] = and_or(v >> 5, 0x00780078u, one);
    p[4 * t + 3] = and_or(v >> 9, 0x00780078u, one);
  }
}

template <>
__device__ __forceinline__ void decode_pairs<RFPX_FP3>(const uint32_t *w, uint32_t *p,
                                                       uint32_t one) {
  constexpr uint32_t MA = 0x00380070u;  // lo bits 4-6, hi bits 19-21
  constexpr uint32_t MB = 0x0070001Cu;  // lo bits 2-4, hi bits 20-22
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
  // type A, window start 3*lo - 4 for lo = 0,1,2,3,4,10,11,12,13,14
  p[0] = and_or(w0 << 4, MA, one);                                 // -4
  p[1] = and_or(w0 << 1, MA, one);                                 // -1
  p[2] = and_or(__builtin_amdgcn_alignbit(w1, w0, 2), MA, one);    // 2
  p[3] = and_or(__builtin_amdgcn_alignbit(w1, w0, 5), MA, one);    // 5
  p[4] = and_or(__builtin_amdgcn_alignbit(w1, w0, 8), MA, one);    // 8
  p[5] = and_or(__builtin_amdgcn_alignbit(w1, w0, 26), MA, one);   // 26
  p[6] = and_or(__builtin_amdgcn_alignbit(w1, w0, 29), MA, one);   // 29
  p[7] = and_or(w1, MA, one);                                      // 32
  p[8] = and_or(__builtin_amdgcn_alignbit(w2, w1, 3), MA, one);    // 35
  p[9] = and_or(__builtin_amdgcn_alignbit(w2, w1, 6), MA, one);    // 38
  // type B, window start 3*lo - 2 for lo = 20..25
  p[10] = and_or(__builtin_amdgcn_alignbit(w2, w1, 26), MB, one);  // 58
  p[11] = and_or(__builtin_amdgcn_alignbit(w2, w1, 29), MB, one);  // 61
  p[12] = and_or(w2, MB, one);                                     // 64
  p[13] = and_or(w2 >> 3, MB, one);                                // 67
  p[14] = and_or(w2 >> 6, MB, one);                                // 70
  p[15] = and_or(w2 >> 9, MB, one);                                // 73
}

// Pair p of a block: the codes (and activations) it joins, and the
// mantissa position k of each code in its bf16 half (the half represents
// 1 + c * 2^(k-7)).
template <int FMT>
__device__ __forceinline__ void pair_def(int p, int &lo, int &hi, int &klo, int &khi) {
  if (FMT == RFPX_FP2) {
    const int i = p & 7;
    lo = 16 * (p >> 3) + i;
    hi = lo + 8;
    klo = khi = 2 * (i % 3);  // 0, 2, 4, 0, 2, 4, 0, 2
  } else if (FMT == RFPX_FP4) {
    const int i = p & 3;
    lo = 8 * (p >> 2) + i;
    hi = lo + 4;
    klo = khi = i == 0 ? 0 : 3;
  } else if (p < 10) {
    lo = p < 5 ? p : p + 5;  // 0..4, 10..14
    hi = lo + 5;
    klo = 4;
    khi = 3;
  } else {
    lo = 20 + (p - 10);  // 20..25
    hi = lo + 6;
    klo = 2;
    khi = 4;
  }
}

// Code offset o in w = (c - o) * scale: 1.5, 3.5, 7.5.
template <int FMT>
__device__ __forceinline__ float code_offset() {
  return FMT == RFPX_FP2 ? 1.5f : FMT == RFPX_FP3 ? 3.5f : 7.5f;
}

// A code at mantissa position k stands for 1 + c * 2^(k-7) = 2^(k-7) *
// (c + 2^(7-k)), so its activation is stored times f = 2^(7-k) (exact) and
// the block's accumulator starts at -sum (f + o) * x; then
//   start + sum_pairs dot2(decoded pair, prepared pair) = sum_j (c_j - o) x_j.
// xl, xh must be bf16 values (their fp32 form); the scaled values are
// exactly bf16 too, so their top 16 bits are the bf16 patterns.
template <int FMT>
__device__ __forceinline__ uint32_t prepared_pair(float xl, float xh, int klo, int khi,
                                                  float *nc) {
  const float flo = (float)(1 << (7 - klo)), fhi = (float)(1 << (7 - khi));
  const float o = code_offset<FMT>();
  *nc -= (flo + o) * xl + (fhi + o) * xh;
  return (__float_as_uint(xl * flo) >> 16) | (__float_as_uint(xh * fhi) & 0xFFFF0000u);
}

// Prepared activations of one block for one virtual column: the 16 pair
// words matching decode_pairs<FMT> and the accumulator start nc.  xb[j] are
// bf16 bit patterns of the block's 32 values.
template <int FMT>
__device__ __forceinline__ void prep_pairs(const uint32_t *xb, uint32_t *pw, float *nc) {
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    int lo, hi, klo, khi;
    pair_def<FMT>(p, lo, hi, klo, khi);
    pw[p] = prepared_pair<FMT>(bf16_bits_to_float(xb[lo]), bf16_bits_to_float(xb[hi]), klo, khi,
                               &acc);
  }
  *nc = acc;
}

// Prefill: one pair word of one block of h (fp32 values, split into bf16 hi + lo)
// for a down matrix of format fmt (a runtime value): writes dst[p] (hi
// parts) and dst[16 + p] (lo parts) and returns the pair's share of the
// block's accumulator start.  A single code path for all formats: three
// inlined template instances of this step behind a runtime format switch
// have been merged by the compiler into one shared block whose FP4 exit lost
// the address of the pair's second value.
__device__ __forceinline__ float prep_h_pair_rt(int fmt, const float *hblk, int p,
                                                uint32_t *dst) {
  int lo, hi, klo, khi;
  float o;
  if (fmt == RFPX_FP2) {
    const int i = p & 7;
    lo = 16 * (p >> 3) + i;
    hi = lo + 8;
    klo = khi = 2 * (i % 3);
    o = 1.5f;
  } else if (fmt == RFPX_FP4) {
    const int i = p & 3;
    lo = 8 * (p >> 2) + i;
    hi = lo + 4;
    klo = khi = i == 0 ? 0 : 3;
    o = 7.5f;
  } else {
    lo = p < 5 ? p : p < 10 ? p + 5 : 20 + (p - 10);
    hi = p < 10 ? lo + 5 : lo + 6;
    klo = p < 10 ? 4 : 2;
    khi = p < 10 ? 3 : 4;
    o = 3.5f;
  }
  const float vl = hblk[lo], vh = hblk[hi];
  const float lh = bf16_bits_to_float(float_to_bf16_rne(vl));
  const float hh = bf16_bits_to_float(float_to_bf16_rne(vh));
  const float ll = bf16_bits_to_float(float_to_bf16_rne(vl - lh));
  const float hl = bf16_bits_to_float(float_to_bf16_rne(vh - hh));
  const float flo = (float)(1 << (7 - klo)), fhi = (float)(1 << (7 - khi));
  dst[p] = (__float_as_uint(lh * flo) >> 16) | (__float_as_uint(hh * fhi) & 0xFFFF0000u);
  dst[16 + p] = (__float_as_uint(ll * flo) >> 16) | (__float_as_uint(hl * fhi) & 0xFFFF0000u);
  return -((flo + o) * (lh + ll) + (fhi + o) * (hh + hl));
}

// ----------------------------------------- exact codes for the down products
//
// The decode kernels' down products take each code as its integer value:
// the block's code dwords are masked so that every byte of a 32-bit window
// holds at most one code, at bit k of the byte; v_cvt_f32_ubyte turns the
// byte into c * 2^k exactly, the prepared h carries the factor 2^-k, and an
// fp32 FMA adds c * h.  The block sum starts at -o * sum(h), so it ends at
// sum_j (c_j - o) h_j.  Per weight and column this is one FMA (plus the
// convert, shared by the columns), where a bf16 hi + lo h costs two bf16
// dot products per pair of weights; on this device an fp32 FMA or byte
// convert issues at twice the rate of a v_dot2.
//
// A group is a 32-bit window of the block's code dwords (dword `src`, or
// alignbit(w[src + 1], w[src], sh) when sh != 0), the mask applied to it,
// and for each byte the code it holds and that code's bit k in the byte (j
// < 0: no code).  Codes sit at bits 2j (FP2), 3j (FP3) or 4j (FP4) of the
// block's little-endian code word.  The products run group by group, byte
// by byte, and the prepared h of a block is stored in that order.
struct CodeByte {
  int8_t j, k;
};
struct CodeGroup {
  int8_t src, sh;
  uint32_t mask;
  CodeByte b[4];
};

template <int FMT>
struct CodeGroups;

// FP2: per dword t, mask 0x03030303 << 2u keeps the codes 16t + 4i + u.
template <>
struct CodeGroups<RFPX_FP2> {
  static constexpr int N = 8;
  static constexpr CodeGroup g[N] = {
      {0, 0, 0x03030303u, {{0, 0}, {4, 0}, {8, 0}, {12, 0}}},
      {0, 0, 0x0C0C0C0Cu, {{1, 2}, {5, 2}, {9, 2}, {13, 2}}},
      {0, 0, 0x30303030u, {{2, 4}, {6, 4}, {10, 4}, {14, 4}}},
      {0, 0, 0xC0C0C0C0u, {{3, 6}, {7, 6}, {11, 6}, {15, 6}}},
      {1, 0, 0x03030303u, {{16, 0}, {20, 0}, {24, 0}, {28, 0}}},
      {1, 0, 0x0C0C0C0Cu, {{17, 2}, {21, 2}, {25, 2}, {29, 2}}},
      {1, 0, 0x30303030u, {{18, 4}, {22, 4}, {26, 4}, {30, 4}}},
      {1, 0, 0xC0C0C0C0u, {{19, 6}, {23, 6}, {27, 6}, {31, 6}}},
  };
};

// FP3: codes 3j never share a byte boundary pattern with the bytes of one
// window, so the 32 codes come from six masks on the three dwords and
// three masks on windows shifted by 2, 34 and 58 bits (twelve integer
// operations per block).
template <>
struct CodeGroups<RFPX_FP3> {
  static constexpr int N = 9;
  static constexpr CodeGroup g[N] = {
      {0, 0, 0x071C0E07u, {{0, 0}, {3, 1}, {6, 2}, {8, 0}}},
      {0, 0, 0x38E07038u, {{1, 3}, {4, 4}, {7, 5}, {9, 3}}},
      {1, 0, 0x0E071C0Eu, {{11, 1}, {14, 2}, {16, 0}, {19, 1}}},
      {1, 0, 0x7038E070u, {{12, 4}, {15, 5}, {17, 3}, {20, 4}}},
      {2, 0, 0x1C0E071Cu, {{22, 2}, {24, 0}, {27, 1}, {30, 2}}},
      {2, 0, 0xE07038E0u, {{23, 5}, {25, 3}, {28, 4}, {31, 5}}},
      {0, 2, 0x7000E070u, {{2, 4}, {5, 5}, {-1, 0}, {10, 4}}},
      {1, 2, 0xE07000E0u, {{13, 5}, {-1, 0}, {18, 4}, {21, 5}}},
      {1, 26, 0xE0700000u, {{-1, 0}, {-1, 0}, {26, 4}, {29, 5}}},
  };
};

// FP4: per dword t, mask 0x0F0F0F0F keeps the codes 8t + 2i, 0xF0F0F0F0
// the codes 8t + 2i + 1.
template <>
struct CodeGroups<RFPX_FP4> {
  static constexpr int N = 8;
  static constexpr CodeGroup g[N] = {
      {0, 0, 0x0F0F0F0Fu, {{0, 0}, {2, 0}, {4, 0}, {6, 0}}},
      {0, 0, 0xF0F0F0F0u, {{1, 4}, {3, 4}, {5, 4}, {7, 4}}},
      {1, 0, 0x0F0F0F0Fu, {{8, 0}, {10, 0}, {12, 0}, {14, 0}}},
      {1, 0, 0xF0F0F0F0u, {{9, 4}, {11, 4}, {13, 4}, {15, 4}}},
      {2, 0, 0x0F0F0F0Fu, {{16, 0}, {18, 0}, {20, 0}, {22, 0}}},
      {2, 0, 0xF0F0F0F0u, {{17, 4}, {19, 4}, {21, 4}, {23, 4}}},
      {3, 0, 0x0F0F0F0Fu, {{24, 0}, {26, 0}, {28, 0}, {30, 0}}},
      {3, 0, 0xF0F0F0F0u, {{25, 4}, {27, 4}, {29, 4}, {31, 4}}},
  };
};

// Every group's mask keeps exactly the listed codes at the listed bits, and
// the groups together list each of the block's 32 codes once.
template <int FMT>
constexpr bool code_groups_valid() {
  constexpr int bits = FMT == RFPX_FP2 ? 2 : FMT == RFPX_FP3 ? 3 : 4;
  bool seen[32] = {};
  int n = 0;
  for (int gi = 0; gi < CodeGroups<FMT>::N; ++gi) {
    const CodeGroup &g = CodeGroups<FMT>::g[gi];
    const int s = 32 * g.src + g.sh;
    for (int b = 0; b < 4; ++b) {
      const uint32_t bm = (g.mask >> (8 * b)) & 0xFFu;
      if (g.b[b].j < 0) {
        if (bm != 0) return false;
        continue;
      }
      const int j = g.b[b].j, k = g.b[b].k;
      if (j >= 32 || seen[j] || bits * j - s - 8 * b != k) return false;
      if (bm != (((1u << bits) - 1u) << k)) return false;
      seen[j] = true;
      ++n;
    }
  }
  return n == 32;
}
static_assert(code_groups_valid<RFPX_FP2>(), "FP2 code groups");
static_assert(code_groups_valid<RFPX_FP3>(), "FP3 code groups");
static_assert(code_groups_valid<RFPX_FP4>(), "FP4 code groups");

// The code and bit of product position q (0..31) of a block.
template <int FMT>
constexpr CodeByte code_at(int q) {
  for (int gi = 0, n = 0; gi < CodeGroups<FMT>::N; ++gi)
    for (int b = 0; b < 4; ++b)
      if (CodeGroups<FMT>::g[gi].b[b].j >= 0 && n++ == q) return CodeGroups<FMT>::g[gi].b[b];
  return CodeByte{-1, 0};
}

// Product position of byte b of group gi (the number of codes before it).
template <int FMT>
constexpr int code_pos(int gi, int b) {
  int n = 0;
  for (int g = 0; g < CodeGroups<FMT>::N; ++g)
    for (int bb = 0; bb < 4; ++bb) {
      if (g == gi && bb == b) return n;
      if (CodeGroups<FMT>::g[g].b[bb].j >= 0) ++n;
    }
  return -1;
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, expanded at compile
// time (so that table entries indexed by I are constants).
template <typename F, int... I>
__host__ __device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__host__ __device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Block scale as an fp32 multiplier: fp16 bits (FP2/FP3) or E8M0 (FP4).
template <int FMT>
__device__ __forceinline__ float block_scale(uint32_t bits) {
  if (FMT == RFPX_FP4) return __builtin_ldexpf(1.0f, (int)(bits & 0xFFu) - 127);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// Wave-uniform values kept in scalar registers: loads the compiler cannot
// prove uniform would otherwise leave bases in VGPRs (64-bit per-lane
// addresses for every load).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
// Buffer resource (V#) over `bytes` bytes at `base` (wave-uniform): loads
// through it take a scalar descriptor, a scalar offset and a 32-bit lane
// offset, and reads past `bytes` return zero instead of faulting.  Word 3 =
// 0x00020000 selects 32-bit raw data on the gfx9 family (gfx950 included).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base,
                                                   uint32_t bytes) {
  void *p = reinterpret_cast<void *>(uniform64(reinterpret_cast<uint64_t>(base)));
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)uniform((int)bytes), 0x00020000);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

#endif  // device side

// ------------------------------------------------------------- host side
// Internal host helpers (abi.hip, codec.hip).
size_t image_layout(int d, int f, int E, const int *fmts, ExpertDesc *desc);
// Host checks of a layer (abi.hip): shapes, limits and the format table;
// the image pointer, its alignment and L->image_bytes against the layout.
rfpx_status check_layer(const moe_layer *L);
rfpx_status check_image(const moe_layer *L);
void set_error(const char *fmt, ...);
rfpx_status fail(rfpx_status st, const char *fmt, ...);

// Launch of a kernel that takes one argument struct.  With an event, the
// launch goes through hipExtLaunchKernel, which stamps t0 with the time the
// kernel starts and t1 with the time it ends (either may be null), so that
// the interval between two stamps holds no launch gap; with neither, it is
// an ordinary launch.
template <typename A>
inline hipError_t launch_k(void (*k)(A), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                           A a, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr) {
  void *args[] = {&a};
  if (!t0 && !t1)
    return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, args, lds, s);
  return hipExtLaunchKernel(reinterpret_cast<const void *>(k), grid, block, args, lds, s, t0,
                            t1, 0);
}

// Launchers (route.hip, expert.hip).
struct ForwardPlan {
  int d, f, E, k, q, xtype;
  float routed_scale;
  const float *router_w;
  const uint8_t *image;
  const void *x;
  float *y;
  int32_t *ids_out;
  float *w_out;
  uint8_t *ws;
  WsLayout wl;
  unsigned gu_fmts;         // bit f set: gate/up format f is present
  unsigned down_fmts;       // bit f set: down format f is present
  Geo geo_gu[5], geo_dn[5];  // indexed by format
  int g;                    // columns per pass of the expert kernels (1, 2)
  int wmax;                 // waves per down workgroup
  int wgu;                  // waves per gate/up workgroup
  int rw_gu, rw_dn;         // rows per workgroup tile
  bool route_only;
  bool pre_route;           // the routing step runs once (k_topk) before the experts
  bool h_early;             // k_down<1>: wave w owns slot w's only unit and loads its
                            // h while the route table is read (no FP2 down matrices)
  hipStream_t stream;
  // optional, 6 hipEvent_t: start and end of the routing kernels, of the
  // gate/up kernel and of the down kernel
  void *const *events;
};
// k_route: router scores and prepared activations; for route_only and
// pre_route also k_topk (the route table; ids and gating weights for
// moe_route_topk).
hipError_t launch_route(const ForwardPlan &p);
// Prefill (prefill.hip): workspace bytes for T tokens (0: unsupported
// shape); with args_out, also the kernel arguments with workspace offsets.
size_t prefill_layout(const moe_layer *L, int T, int xtype, void *args_out);
// events: null, or 6 hipEvent_t as for moe_prefill_forward_timed.
hipError_t launch_prefill(const moe_layer *L, const void *x, int xtype, int T, float *y,
                          uint8_t *ws, size_t image_bytes, hipStream_t stream,
                          void *const *events);
// k_gateup (all slots) and k_down (all slots, with the combine); stamps
// events[2..5] when events are given.
hipError_t launch_experts(const ForwardPlan &p);

}  // namespace rfpx
