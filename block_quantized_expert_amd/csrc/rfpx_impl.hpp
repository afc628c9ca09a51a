// rfpx_impl.hpp -- internal definitions shared by the librfpx sources:
// format constants, the device image and workspace layouts, the lane
// geometry of the expert kernels, and the register-level block decode.
//
// Block decode on gfx950.  The expert products run on v_dot2c_f32_bf16
// (two bf16 products added into an fp32 accumulator per lane per issue).
// A packed code c is turned into the bf16 value 1 + c/2^k by masking it
// into the mantissa of 1.0 (0x3F80): one shift (or funnel shift) and one
// and-or per pair of codes, i.e. about one VALU op per weight, shared by all
// columns.  The constant part of 1 + c/2^k and the code offset (1.5, 3.5,
// 7.5) are folded into a per-block, per-column accumulator start value
// computed once from the activations ("prepared" activations below), so
//      sum_j (c_j - offset) x_j  =  A * (nc + sum_pairs dot2(v, xpair))
// with A = 8 (FP2, FP3) or 16 (FP4).  v and the bf16 activations are exact,
// each bf16 product is exact in fp32, so the only rounding is fp32
// accumulation.
//
// Pairings (lo code, hi code) of the 16 pairs of one block, and where each
// code lands in the 32-bit pair word (bf16 lo in bits 0..15, hi in 16..31):
//   FP2  pair 8t+a (t<2, a<8): codes (16t+a, 16t+a+8) -> bits 4-5 / 20-21,
//        v = 1 + c/8 on both halves.  Window: dword t >> (2a-4).
//   FP4  pair 4t+a (t<4, a<4): codes (8t+a, 8t+a+4)   -> bits 3-6 / 19-22,
//        v = 1 + c/16.  Window: dword t >> (4a-3).
//   FP3  pairs 0..9: codes (lo, lo+5), lo in {0..4, 10..14}; lo at bits 4-6
//        (v = 1 + c/8), hi at bits 19-21 (v = 1 + c/16); the activation of
//        the hi code is stored doubled.  Pairs 10..15: codes (lo, lo+6), lo
//        in 20..25; lo at bits 2-4 (v = 1 + c/32, activation stored x4), hi
//        at bits 20-22 (v = 1 + c/8).  Window: bits 3lo-4 (resp. 3lo-2) of
//        the 96-bit code word, taken with one v_alignbit_b32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rfpx.h"

namespace rfpx {

constexpr int kQMax = RFPX_Q_MAX;
constexpr int kKMax = RFPX_K_MAX;
constexpr int kEMax = RFPX_E_MAX;
constexpr int kMaxSlots = kQMax * kKMax + 1;  // routed unique experts + shared
constexpr uint32_t kMagic = 0x58504652u;      // "RFPX"
constexpr uint32_t kVersion = 1;
constexpr uint32_t kOneOne = 0x3F803F80u;     // bf16 pair (1.0, 1.0)

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
// A in  sum (c - offset) x = A * acc.
__host__ __device__ constexpr float code_gain(int fmt) {
  return fmt == RFPX_FP4 ? 16.f : 8.f;
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
};

struct WsLayout {
  size_t route;     // RouteTable
  size_t scores;    // fp32 [q][E]
  size_t xp;        // u32  [3 fmts][q][nb_d][vx][16]  prepared activations
  size_t xnc;       // fp32 [3][q][nb_d]
  size_t hp;        // u32  [slots][q][nb_f][2][16]    prepared h (hi, lo)
  size_t hnc;       // fp32 [slots][q][nb_f]
  size_t part;      // fp32 [slots][q][d]              weighted partial outputs
  size_t total;
  int max_slots;
};

// ------------------------------------------------------------ device side
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

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

// Decode the codes of one block into its 16 bf16 pair words (see header).
// `w` holds the block's code dwords: 2 (FP2), 3 (FP3) or 4 (FP4).
template <int FMT>
__device__ __forceinline__ void decode_pairs(const uint32_t *w, uint32_t *p);

template <>
__device__ __forceinline__ void decode_pairs<RFPX_FP2>(const uint32_t *w, uint32_t *p) {
  constexpr uint32_t M = 0x00300030u;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t v = w[t];
    p[8 * t + 0] = ((v << 4) & M) | kOneOne;
    p[8 * t + 1] = ((v << 2) & M) | kOneOne;
    p[8 * t + 2] = (v & M) | kOneOne;
    p[8 * t + 3] = ((v >> 2) & M) | kOneOne;
    p[8 * t + 4] = ((v >> 4) & M) | kOneOne;
    p[8 * t + 5] = ((v >> 6) & M) | kOneOne;
    p[8 * t + 6] = ((v >> 8) & M) | kOneOne;
    p[8 * t + 7] = ((v >> 10) & M) | kOneOne;
  }
}

template <>
__device__ __forceinline__ void decode_pairs<RFPX_FP4>(const uint32_t *w, uint32_t *p) {
  constexpr uint32_t M = 0x00780078u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    uint32_t v = w[t];
    p[4 * t + 0] = ((v << 3) & M) | kOneOne;
    p[4 * t + 1] = ((v >> 1) & M) | kOneOne;
    p[4 * t + 2] = ((v >> 5) & M) | kOneOne;
    p[4 * t + 3] = ((v >> 9) & M) | kOneOne;
  }
}

template <>
__device__ __forceinline__ void decode_pairs<RFPX_FP3>(const uint32_t *w, uint32_t *p) {
  constexpr uint32_t MA = 0x00380070u;  // lo bits 4-6, hi bits 19-21
  constexpr uint32_t MB = 0x0070001Cu;  // lo bits 2-4, hi bits 20-22
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
  // type A, window start 3*lo - 4 for lo = 0,1,2,3,4,10,11,12,13,14
  p[0] = ((w0 << 4) & MA) | kOneOne;                                 // -4
  p[1] = ((w0 << 1) & MA) | kOneOne;                                 // -1
  p[2] = (__builtin_amdgcn_alignbit(w1, w0, 2) & MA) | kOneOne;      // 2
  p[3] = (__builtin_amdgcn_alignbit(w1, w0, 5) & MA) | kOneOne;      // 5
  p[4] = (__builtin_amdgcn_alignbit(w1, w0, 8) & MA) | kOneOne;      // 8
  p[5] = (__builtin_amdgcn_alignbit(w1, w0, 26) & MA) | kOneOne;     // 26
  p[6] = (__builtin_amdgcn_alignbit(w1, w0, 29) & MA) | kOneOne;     // 29
  p[7] = (w1 & MA) | kOneOne;                                        // 32
  p[8] = (__builtin_amdgcn_alignbit(w2, w1, 3) & MA) | kOneOne;      // 35
  p[9] = (__builtin_amdgcn_alignbit(w2, w1, 6) & MA) | kOneOne;      // 38
  // type B, window start 3*lo - 2 for lo = 20..25
  p[10] = (__builtin_amdgcn_alignbit(w2, w1, 26) & MB) | kOneOne;    // 58
  p[11] = (__builtin_amdgcn_alignbit(w2, w1, 29) & MB) | kOneOne;    // 61
  p[12] = (w2 & MB) | kOneOne;                                       // 64
  p[13] = ((w2 >> 3) & MB) | kOneOne;                                // 67
  p[14] = ((w2 >> 6) & MB) | kOneOne;                                // 70
  p[15] = ((w2 >> 9) & MB) | kOneOne;                                // 73
}

// Pair p of a block: the codes (and activations) it joins, the factor each
// activation is stored with, and its share of the accumulator start nc.
template <int FMT>
__device__ __forceinline__ void pair_def(int p, int &lo, int &hi, float &slo,
                                         float &shi) {
  if (FMT == RFPX_FP2) {
    lo = 16 * (p >> 3) + (p & 7);
    hi = lo + 8;
    slo = shi = 1.f;
  } else if (FMT == RFPX_FP4) {
    lo = 8 * (p >> 2) + (p & 3);
    hi = lo + 4;
    slo = shi = 1.f;
  } else if (p < 10) {
    lo = p < 5 ? p : p + 5;  // 0..4, 10..14
    hi = lo + 5;
    slo = 1.f;
    shi = 2.f;
  } else {
    lo = 20 + (p - 10);  // 20..25
    hi = lo + 6;
    slo = 4.f;
    shi = 1.f;
  }
}

// nc share of one pair with activations xl, xh (see the header comment):
// FP2 -(1 + 1.5/8)(xl + xh); FP4 -(1 + 7.5/16)(xl + xh);
// FP3 -(slo xl + shi xh) - (3.5/8)(xl + xh).
template <int FMT>
__device__ __forceinline__ float pair_nc(float xl, float xh, float slo, float shi) {
  if (FMT == RFPX_FP2) return -1.1875f * (xl + xh);
  if (FMT == RFPX_FP4) return -1.46875f * (xl + xh);
  return -(slo * xl + shi * xh) - 0.4375f * (xl + xh);
}

// bf16 pair word of pair p from bf16 bit patterns of its two activations
// (the factors 2 and 4 are exact exponent increments).
template <int FMT>
__device__ __forceinline__ uint32_t pair_word(uint32_t bl, uint32_t bh, float slo,
                                              float shi) {
  if (FMT == RFPX_FP3) {
    if (slo != 1.f) bl = float_to_bf16_rne(slo * bf16_bits_to_float(bl));
    if (shi != 1.f) bh = float_to_bf16_rne(shi * bf16_bits_to_float(bh));
  }
  return bl | (bh << 16);
}

// Prepared activations of one block for one virtual column: the 16 bf16
// pair words matching decode_pairs<FMT> and the accumulator start nc.  xb[j]
// are bf16 bit patterns of the block's 32 values.
template <int FMT>
__device__ __forceinline__ void prep_pairs(const uint32_t *xb, uint32_t *pw, float *nc) {
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    int lo, hi;
    float slo, shi;
    pair_def<FMT>(p, lo, hi, slo, shi);
    pw[p] = pair_word<FMT>(xb[lo], xb[hi], slo, shi);
    acc += pair_nc<FMT>(bf16_bits_to_float(xb[lo]), bf16_bits_to_float(xb[hi]), slo, shi);
  }
  *nc = acc;
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
void set_error(const char *fmt, ...);
rfpx_status fail(rfpx_status st, const char *fmt, ...);

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
  unsigned prep_fmts;       // bit f set: gate/up format f is present
  unsigned down_fmts;       // bit f set: down format f is present
  Geo geo_gu[5], geo_dn[5];  // indexed by format
  int g;                    // columns per pass of the expert kernels (1, 2)
  int r;                    // rows per wave
  int wmax;                 // waves per workgroup
  int rw_gu, rw_dn;         // rows per workgroup tile
  bool route_only;
  hipStream_t stream;
  void *const *events;      // optional: 5 hipEvent_t recorded around launches
};
hipError_t launch_route(const ForwardPlan &p);
hipError_t launch_experts(const ForwardPlan &p);

}  // namespace rfpx
