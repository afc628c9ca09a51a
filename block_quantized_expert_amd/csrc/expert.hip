// expert.hip -- the decode step of one routed-MoE layer: router scores, the
// shared and routed experts' dequantize-and-GEMV products with SiLU gating,
// and the weighted combine.
//
// Page "APU 实现 token 自由…" (ainomam.com), section "Lucebox 的优化三板斧":
// in the q-column verify path each packed weight is decoded once and applied
// to every verify column.  Page "Lucebox专攻DeepSeek V4…" (m.mzlw.cn),
// sections "MoE 专家并行" (256 routed experts, top-6, one shared expert) and
// "新手常见疑问" (decode is bound by memory bandwidth).  Page "DeepSeek V4
// Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s" (taozi.news), section
// "ROCmFPX": gate/up in FP2, down in FP3, the shared expert in FP4.
//
// Launches per step (after k_route, route.hip: router scores and prepared
// activations; for steps of several columns also k_topk, which builds the
// route table once):
//   k_gateup  grid (f / RW_GU, slots).  Slot 0 is the shared expert (every
//             column, weight 1): its workgroups need no routing and start
//             streaming at once.  In a one-column step the workgroups of
//             routed slots first run the routing step in LDS (sorted top-k
//             and gating; deterministic, so all workgroups agree;
//             rfpx_route.hpp) and workgroup (0, s) publishes slot s; in a
//             step of several columns they copy their slot's entry of the
//             route table.  Then a gate/up tile of the slot's expert.
//   k_down    grid d / RW_DN.  A workgroup owns RW_DN rows of y for every
//             column and runs the down rows of every slot into them, each
//             row result times the column's gating weight: the combine is
//             its epilogue, and no partial output leaves the workgroup.
//
// A gate/up tile is RW_GU rows of the gate and up matrices (whole 32-row
// blocks of h).  It is cut into units of R rows x one part of 64 chunks per
// row; each wave loads the prepared activations of its chunk once per pass,
// issues every code and scale load of a unit up front (buffer loads: scalar
// descriptor, scalar row offset, 32-bit lane offset), decodes each block in
// registers once for all columns of the pass (v_dot2 on the prepared
// pairs), reduces each row across its lanes (DPP and permlane swaps) and
// writes part sums to LDS.  Then h = silu(g) * u, stored as fp32 rows of the
// slot's h.  k_down loads a lane's blocks of h, puts each block in the
// product order of its down format's exact-code decode (CodeGroups in
// rfpx_impl.hpp) in registers, takes each down code as its integer value
// (v_cvt_f32_ubyte) and adds c * h with fp32 FMAs.
// Lane geometry (Geo): with a row of >= 64 chunks a wave covers one row per
// step and lane l reads chunk l (+ 64 for the second part; fully coalesced
// 1 KiB requests); shorter rows give each wave 64/cpl rows per step.
#include "rfpx_route.hpp"

namespace rfpx {
namespace {

struct ExpArgs {
  const uint8_t *image;
  RouteTable *rt;
  RouteParams rp;
  const uint32_t *xp;   // prepared activations [fmt][q][nb_d][vx][16]
  const float *xnc;     // [fmt][q][nb_d]
  uint32_t *hp;         // h [slot][q][f] (fp32 bits), rows in order
  float *y;
  int d, f, q, nb_d, nb_f;
  int rw_gu, rw_dn;
  Geo geo_gu[5], geo_dn[5];  // by format; all zero for a format not in the host table
  int h_early;               // k_down<1>: see ForwardPlan::h_early
};

// A format read from the device table that the launch was planned for: the
// plan fills the geometry of exactly the formats of the host table (the
// arrays are indexed by constants only, so they stay in scalar registers).
__device__ __forceinline__ bool planned(const Geo (&geo)[5], int fmt) {
  return fmt == RFPX_FP2 ? geo[RFPX_FP2].cpl != 0
       : fmt == RFPX_FP3 ? geo[RFPX_FP3].cpl != 0
       : fmt == RFPX_FP4 ? geo[RFPX_FP4].cpl != 0 : false;
}

// The columns of one slot: expert and count in scalar registers; the column
// list and weights stay in LDS and are read when a pass needs them (indexing
// a register array by a loop counter would put it in scratch memory).  Both
// accessors take a wave-uniform index and return the first lane's value.
struct SlotCols {
  int expert, ncols;
  const int *cols;   // [ncols] global column index of each compact column
  const float *w;    // [ncols] gating weight
  __device__ int col(int i) const { return uniform(cols[i]); }
  __device__ float weight(int i) const {
    return __int_as_float(uniform(__float_as_int(w[i])));
  }
};

template <int FMT>
struct Fmt {
  static constexpr int CB = chunk_blocks(FMT);               // blocks per chunk
  static constexpr int CW = FMT == RFPX_FP3 ? 3 : 4;          // code dwords per chunk
  static constexpr int BW = FMT == RFPX_FP2 ? 2 : CW;         // code dwords per block
  static constexpr int CBYTES = CB * code_bytes(FMT);         // 16, 12, 16
  static constexpr int SBYTES = CB * scale_bytes(FMT);        // 4, 2, 1
};

template <int FMT>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff, uint32_t *w) {
  if (FMT == RFPX_FP3) {
    u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)voff, (int)soff, 0);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
  } else {
    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
}

template <int FMT>
__device__ __forceinline__ uint32_t load_scale(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
  if (FMT == RFPX_FP2) return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
  if (FMT == RFPX_FP3) return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

template <int FMT>
__device__ __forceinline__ uint32_t block_scale_bits(uint32_t sw, int j) {
  return FMT == RFPX_FP2 ? (sw >> (16 * j)) : sw;
}

struct MatPtr {
  __amdgpu_buffer_rsrc_t codes;
  __amdgpu_buffer_rsrc_t scales;
};

// Code and scale loads of one unit: rows row_u + rpi*i (i < R) of NM
// matrices, the lane's own chunk at byte offsets coff (codes) and soff
// (scales) within a row, through the planes' buffer resources.  By default
// a row's offset row * pitch is the scalar operand (no extra registers).
// With LANE_ROW it joins the lane operand instead, which the buffer range
// check covers: a row past the matrix (the "next unit" after a wave's last
// one) then reads as zero with no memory access, so a prefetch of the next
// unit needs no branch -- a branch around it makes the compiler wait for
// the prefetch before computing the current unit.
template <int FMT, int NM, int R, bool LANE_ROW = false>
__device__ __forceinline__ void unit_load(const MatPtr (&mats)[NM], uint32_t cpitch,
                                          uint32_t spitch, int row_u, int rpi, uint32_t coff,
                                          uint32_t soff, uint32_t (&cw)[R][NM][Fmt<FMT>::CW],
                                          uint32_t (&sw)[R][NM]) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t row = (uint32_t)(row_u + rpi * i);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (LANE_ROW) {
        load_chunk<FMT>(mats[m].codes, coff + row * cpitch, 0, cw[i][m]);
        sw[i][m] = load_scale<FMT>(mats[m].scales, soff + row * spitch, 0);
      } else {
        load_chunk<FMT>(mats[m].codes, coff, row * cpitch, cw[i][m]);
        sw[i][m] = load_scale<FMT>(mats[m].scales, soff, row * spitch);
      }
    }
  }
}

// Per-lane partial dot products of the unit's rows with G columns of
// prepared activations: each row's blocks are decoded once and applied to
// every column.  Rows are decoded one at a time (scheduling fences keep the
// decode of one row from being hoisted over the next, which would multiply
// register pressure).
template <int FMT, int G, int VX, int NM, int R>
__device__ __forceinline__ void unit_compute(const uint32_t (&cw)[R][NM][Fmt<FMT>::CW],
                                             const uint32_t (&sw)[R][NM],
                                             const uint32_t (&xr)[G][Fmt<FMT>::CB][VX][16],
                                             const float (&ncr)[G][Fmt<FMT>::CB],
                                             uint32_t one, float (&tot)[R][NM][G]) {
  using F = Fmt<FMT>;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < R; ++i) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < G; ++g) tot[i][m][g] = 0.f;
#pragma unroll
      for (int j = 0; j < F::CB; ++j) {
        uint32_t pr[16];
        decode_pairs<FMT>(&cw[i][m][j * F::BW], pr, one);
        const float s = block_scale<FMT>(block_scale_bits<FMT>(sw[i][m], j));
#pragma unroll
        for (int g = 0; g < G; ++g) {
          // two accumulators halve the chain of dependent dot2 ops
          float acc0 = ncr[g][j], acc1 = 0.f;
#pragma unroll
          for (int v = 0; v < VX; ++v)
#pragma unroll
            for (int p = 0; p < 16; p += 2) {
              acc0 = dot2(pr[p], xr[g][j][v][p], acc0);
              acc1 = dot2(pr[p + 1], xr[g][j][v][p + 1], acc1);
            }
          tot[i][m][g] = fmaf(acc0 + acc1, s, tot[i][m][g]);
        }
      }
    }
  }
}

// The down products of one unit: the unit's rows against GP compact
// columns of h (fp32, put in each block's product order by prep_h, 32 values per
// block and column), one exact-code FMA per weight and column (CodeGroups).
// Rows are decoded one at a time, as in unit_compute.
template <int FMT, int GP, int R>
__device__ __forceinline__ void unit_compute_code(const uint32_t (&cw)[R][1][Fmt<FMT>::CW],
                                                  const uint32_t (&sw)[R][1],
                                                  const uint32_t (&xr)[GP][Fmt<FMT>::CB][2][16],
                                                  const float (&ncr)[GP][Fmt<FMT>::CB],
                                                  float (&tot)[R][1][GP]) {
  using F = Fmt<FMT>;
  using CG = CodeGroups<FMT>;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < GP; ++g) tot[i][0][g] = 0.f;
#pragma unroll
    for (int j = 0; j < F::CB; ++j) {
      const uint32_t *w = &cw[i][0][j * F::BW];
      const float s = block_scale<FMT>(block_scale_bits<FMT>(sw[i][0], j));
      // two accumulators per column halve the chain of dependent FMAs
      float acc[GP][2];
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        acc[g][0] = ncr[g][j];
        acc[g][1] = 0.f;
      }
      static_for<CG::N>([&](auto GI) {
        constexpr int gi = decltype(GI)::value;
        constexpr CodeGroup cg = CG::g[gi];
        uint32_t win;
        if constexpr (cg.sh != 0)
          win = __builtin_amdgcn_alignbit(w[cg.src + 1], w[cg.src], cg.sh);
        else
          win = w[cg.src];
        uint32_t m = win & cg.mask;
        // the masked word stays one value, so that each byte converts with
        // v_cvt_f32_ubyte<b> instead of a byte extract of win plus a convert
        asm("" : "+v"(m));
        static_for<4>([&](auto B) {
          constexpr int b = decltype(B)::value;
          if constexpr (cg.b[b].j >= 0) {
            constexpr int q = code_pos<FMT>(gi, b);
            // v_cvt_f32_ubyte<b>: c * 2^k, exact
            const float c = (float)((m >> (8 * b)) & 0xFFu);
#pragma unroll
            for (int g = 0; g < GP; ++g)
              acc[g][q & 1] = fmaf(c, __uint_as_float(xr[g][j][q >> 4][q & 15]), acc[g][q & 1]);
          }
        });
      });
#pragma unroll
      for (int g = 0; g < GP; ++g) tot[i][0][g] = fmaf(acc[g][0] + acc[g][1], s, tot[i][0][g]);
    }
  }
}

// Prepared activations of the blocks of the lane's chunk `ch` for columns
// colidx[0..G) (format FMT): block b of column c sits at ((c * nb) + b) *
// VX * 16 words, its accumulator start at c * nb + b.
template <int FMT, int G, int VX>
__device__ __forceinline__ void load_prepared_x(const ExpArgs &a, const int (&colidx)[G],
                                                int ch, uint32_t (&xr)[G][Fmt<FMT>::CB][VX][16],
                                                float (&ncr)[G][Fmt<FMT>::CB]) {
  using F = Fmt<FMT>;
  const uint32_t *pw = a.xp + (size_t)(FMT - RFPX_FP2) * a.q * a.nb_d * VX * 16;
  const float *pnc = a.xnc + (size_t)(FMT - RFPX_FP2) * a.q * a.nb_d;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < F::CB; ++j) {
      const size_t item = (size_t)colidx[g] * a.nb_d + ch * F::CB + j;
      const uint4 *src = reinterpret_cast<const uint4 *>(pw + item * VX * 16);
#pragma unroll
      for (int v = 0; v < VX; ++v)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 q4 = src[v * 4 + u];
          xr[g][j][v][4 * u + 0] = q4.x;
          xr[g][j][v][4 * u + 1] = q4.y;
          xr[g][j][v][4 * u + 2] = q4.z;
          xr[g][j][v][4 * u + 3] = q4.w;
        }
      ncr[g][j] = pnc[item];
    }
  }
}

// h of the blocks of chunk `ch` for G compact columns c0.. of a slot, as
// stored by the gate/up kernel: column c's rows are contiguous fp32 (block
// b of column c at ((c * nb) + b) * 32 words), element e of a block in word
// 16 (e / 16) + e % 16 of its register block.
template <int FMT, int G>
__device__ __forceinline__ void load_h(const uint32_t *__restrict__ pw, int nb, int c0, int ch,
                                       uint32_t (&xr)[G][Fmt<FMT>::CB][2][16]) {
  using F = Fmt<FMT>;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < F::CB; ++j) {
      const size_t item = (size_t)(c0 + g) * nb + ch * F::CB + j;
      const uint4 *src = reinterpret_cast<const uint4 *>(pw + item * 32);
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint4 q4 = src[v * 4 + u];
          xr[g][j][v][4 * u + 0] = q4.x;
          xr[g][j][v][4 * u + 1] = q4.y;
          xr[g][j][v][4 * u + 2] = q4.z;
          xr[g][j][v][4 * u + 3] = q4.w;
        }
    }
  }
}

// Blocks of h (as load_h leaves them) into the down products' form, in
// place: position q of a block holds h[code_at(q).j] * 2^-code_at(q).k (the
// exact-code products then need no scaling), and the block's accumulator
// start is -o times the sum of its 32 values (pairwise, in a fixed order).
template <int FMT, int G>
__device__ __forceinline__ void prep_h(uint32_t (&xr)[G][Fmt<FMT>::CB][2][16],
                                       float (&ncr)[G][Fmt<FMT>::CB]) {
  using F = Fmt<FMT>;
  constexpr float o = FMT == RFPX_FP2 ? 1.5f : FMT == RFPX_FP3 ? 3.5f : 7.5f;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < F::CB; ++j) {
      float h[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) h[e] = __uint_as_float(xr[g][j][e >> 4][e & 15]);
      float t[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] = h[2 * e] + h[2 * e + 1];
#pragma unroll
      for (int w = 8; w > 0; w >>= 1)
#pragma unroll
        for (int e = 0; e < w; ++e) t[e] = t[2 * e] + t[2 * e + 1];
      ncr[g][j] = -o * t[0];
      static_for<32>([&](auto Q) {
        constexpr int q = decltype(Q)::value;
        constexpr CodeByte c = code_at<FMT>(q);
        constexpr float sc = 1.0f / (float)(1 << c.k);
        xr[g][j][q >> 4][q & 15] = __float_as_uint(c.k ? h[c.j] * sc : h[c.j]);
      });
    }
  }
}

// The expert's table entry, every field in scalar registers.
__device__ __forceinline__ ExpertDesc load_desc(const uint8_t *image, int e) {
  const ExpertDesc *t = reinterpret_cast<const ExpertDesc *>(image + kImgTable) + e;
  ExpertDesc d;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    d.codes[m] = uniform64(t->codes[m]);
    d.scales[m] = uniform64(t->scales[m]);
    d.fmt[m] = uniform(t->fmt[m]);
  }
  d.reserved = 0;
  return d;
}

// Sum over the lpr lanes of a row group; the result is valid in the group's
// first lane.  A full 64-lane row uses DPP inside each row of 16 lanes
// (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror) and
// v_readlane across the four rows; shorter groups use lane shuffles.
__device__ __forceinline__ float group_sum(float v, int lpr) {
  if (lpr == 64) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
  }
  for (int off = lpr >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Where a unit lies: unit u covers rows [rloc_u, rloc_u + R*rpi) of the tile
// (rows rloc_u + rg + rpi*i for the lane's row group rg) and column part
// u % parts (chunks 64p .. 64p+63 of each row when a row has 128 chunks).
struct UnitPos {
  int rloc_u;   // first row of the unit within the tile (wave-uniform)
  int part;     // column part
};

__device__ __forceinline__ UnitPos unit_pos(int u, int parts, int r, int rpi) {
  UnitPos up;
  up.part = u % parts;
  up.rloc_u = (u / parts) * r * rpi;
  return up;
}

// Dynamic LDS of the product kernels.  Its first blockDim.x words are a
// sink: one word per thread that a reduction's non-writer lanes store to,
// so that the stores of a unit's results need no branch on the lane.  A
// lane-dependent branch inside a unit loop makes the compiler treat the
// loop's exits as divergent, and the extra control-flow path it then adds
// to the loop head makes the next unit's loads wait for every load in
// flight, which undoes the double buffering.
extern __shared__ float dyn_lds[];

__device__ __forceinline__ float *lane_sink() { return dyn_lds + threadIdx.x; }

// ------------------------------------------------------------ gate / up

// Part sums of one computed unit to LDS: gup[m][part][column][row].
template <int FMT, int GP, int R>
__device__ __forceinline__ void gateup_reduce(const float (&tot)[R][2][GP], const Geo &geo,
                                              const UnitPos &up, int c0, int P, int q, int rw,
                                              float *gup) {
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  if (geo.lpr == 64) {  // one row per wave step: reduce all values at once
    constexpr int N = R * 2 * GP;
    // multi_sum takes a power-of-two count: zeros pad the values past N
    constexpr int NP = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16;
    static_assert(N <= 16, "at most 16 values per unit");
    float flat[NP];
#pragma unroll
    for (int n = N; n < NP; ++n) flat[n] = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int g = 0; g < GP; ++g) flat[(i * 2 + m) * GP + g] = tot[i][m][g];
    const float v = multi_sum<NP>(flat, lane);
    const int n = ms_index<NP>(lane);
    const int i = n / (2 * GP), m = (n / GP) % 2, g = n % GP;
    float *dst = ms_writer<NP>(lane) && n < N
                     ? &gup[((m * P + up.part) * q + c0 + g) * rw + up.rloc_u + i]
                     : lane_sink();
    *dst = v;
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          const float v = group_sum(tot[i][m][g], geo.lpr);
          float *dst = li == 0 ? &gup[((m * P + up.part) * q + c0 + g) * rw + up.rloc_u + rg + geo.rpi * i]
                               : lane_sink();
          *dst = v;
        }
  }
}

// One pass of one column over the wave's units u = wave, wave + waves, ...
// (all in part wave % P, since waves is a multiple of P), for one-column
// steps: a tile gives each wave about one unit, so all of a unit's loads go
// out at once and there is no second register set (whose registers would
// halve the waves per SIMD).
template <int FMT, int VX, int R>
__device__ __forceinline__ void gateup_pass1(const ExpArgs &a, const SlotCols &sc, int c0,
                                             const Geo &geo, int units, int wave, int waves,
                                             int tile, const MatPtr (&mats)[2], uint32_t cpitch,
                                             uint32_t spitch, float *gup) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const int P = geo.tpl, rw = a.rw_gu, q = a.q;
  const int colidx[1] = {sc.col(c0)};
  int u = wave;
  UnitPos up = unit_pos(u, P, R, geo.rpi);
  const int ch = li + geo.lpr * up.part;
  const uint32_t coff = (uint32_t)(rg * cpitch + ch * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + ch * F::SBYTES);
  uint32_t cw[R][2][F::CW], sw[R][2];
  unit_load<FMT, 2, R>(mats, cpitch, spitch, tile * rw + up.rloc_u, geo.rpi, coff, soff, cw, sw);
  uint32_t xr[1][F::CB][VX][16];
  float ncr[1][F::CB];
  load_prepared_x<FMT, 1, VX>(a, colidx, ch, xr, ncr);
  const uint32_t one = one_one_vgpr();
  while (true) {
    float tot[R][2][1];
    unit_compute<FMT, 1, VX, 2, R>(cw, sw, xr, ncr, one, tot);
    gateup_reduce<FMT, 1, R>(tot, geo, up, c0, P, q, rw, gup);
    u += waves;
    if (u >= units) break;
    up = unit_pos(u, P, R, geo.rpi);
    unit_load<FMT, 2, R>(mats, cpitch, spitch, tile * rw + up.rloc_u, geo.rpi, coff, soff, cw, sw);
  }
}

// One pass of GP columns (c0 .. c0+GP-1 of the slot) over the wave's units
// u = wave, wave + waves, ... (all in part wave % P, since waves is a
// multiple of P), for steps of several columns.  The prepared activations
// of the wave's chunk are loaded once for all its units; the code and scale
// loads of the next unit are in flight while a unit is decoded (two
// register sets, used in turn), so a wave streams its units without waiting
// a full memory latency for each.
template <int FMT, int GP, int VX, int R>
__device__ __forceinline__ void gateup_pass(const ExpArgs &a, const SlotCols &sc, int c0,
                                            const Geo &geo, int units, int wave, int waves,
                                            int tile, const MatPtr (&mats)[2], uint32_t cpitch,
                                            uint32_t spitch, float *gup /* [2][P][q][rw] */) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const int P = geo.tpl, rw = a.rw_gu, q = a.q;
  int colidx[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) colidx[g] = sc.col(c0 + g);
  int u = wave;
  UnitPos up = unit_pos(u, P, R, geo.rpi);
  const int ch = li + geo.lpr * up.part;
  const uint32_t coff = (uint32_t)(rg * cpitch + ch * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + ch * F::SBYTES);
  uint32_t cwa[R][2][F::CW], swa[R][2], cwb[R][2][F::CW], swb[R][2];
  unit_load<FMT, 2, R, true>(mats, cpitch, spitch, tile * rw + up.rloc_u, geo.rpi, coff, soff, cwa,
                             swa);
  uint32_t xr[GP][F::CB][VX][16];
  float ncr[GP][F::CB];
  load_prepared_x<FMT, GP, VX>(a, colidx, ch, xr, ncr);
  const uint32_t one = one_one_vgpr();
  // the next unit's loads go out unconditionally; past the wave's last unit
  // they address row f, outside the matrix, and read nothing.  Units go in
  // pairs (set a, then set b) with the loop's only exit at its head, and an
  // odd last unit after it: an exit between the two halves would add a path
  // into the loop head on which set b's loads are still in flight, and the
  // compiler would then wait for every load there, each iteration
  const int past = a.f;
  while (u + waves < units) {
    {
      const int un = u + waves;
      const UnitPos upn = unit_pos(un, P, R, geo.rpi);
      unit_load<FMT, 2, R, true>(mats, cpitch, spitch, tile * rw + upn.rloc_u, geo.rpi, coff, soff,
                                 cwb, swb);
      float tot[R][2][GP];
      unit_compute<FMT, GP, VX, 2, R>(cwa, swa, xr, ncr, one, tot);
      gateup_reduce<FMT, GP, R>(tot, geo, up, c0, P, q, rw, gup);
      u = un;
      up = upn;
    }
    {
      const int un = u + waves;
      const UnitPos upn = unit_pos(un, P, R, geo.rpi);
      unit_load<FMT, 2, R, true>(mats, cpitch, spitch, un < units ? tile * rw + upn.rloc_u : past,
                                 geo.rpi, coff, soff, cwa, swa);
      float tot[R][2][GP];
      unit_compute<FMT, GP, VX, 2, R>(cwb, swb, xr, ncr, one, tot);
      gateup_reduce<FMT, GP, R>(tot, geo, up, c0, P, q, rw, gup);
      u = un;
      up = upn;
    }
  }
  if (u < units) {
    float tot[R][2][GP];
    unit_compute<FMT, GP, VX, 2, R>(cwa, swa, xr, ncr, one, tot);
    gateup_reduce<FMT, GP, R>(tot, geo, up, c0, P, q, rw, gup);
  }
}

// h of one gate/up tile of a slot for all of the slot's columns, stored
// as rows of the slot's h: hout[c * f + row] (the down kernel prepares its
// blocks in registers).
template <int FMT, int G, int VX>
__device__ __forceinline__ void gateup_tile(const ExpArgs &a, const SlotCols &sc,
                                            const ExpertDesc &ed, int tile, float *hout,
                                            float *gup) {
  constexpr int R = unit_rows_gu(FMT, G);
  const Geo geo = a.geo_gu[FMT];
  static_assert(G == 2 || R == unit_rows_for(FMT, 1), "one-column steps keep their unit rows");
  const uint32_t cpitch = (uint32_t)(a.d / 32) * code_bytes(FMT);
  const uint32_t spitch = (uint32_t)(a.d / 32) * scale_bytes(FMT);
  const MatPtr mats[2] = {
      {make_rsrc(a.image + ed.codes[0], a.f * cpitch), make_rsrc(a.image + ed.scales[0], a.f * spitch)},
      {make_rsrc(a.image + ed.codes[1], a.f * cpitch), make_rsrc(a.image + ed.scales[1], a.f * spitch)}};
  const int P = geo.tpl, rw = a.rw_gu, q = a.q;
  const int units = rw / (R * geo.rpi) * P;
  const int wave = uniform(threadIdx.x >> 6);
  const int waves = blockDim.x >> 6;
  // columns per pass: 64 registers of prepared activations per lane, i.e.
  // two columns of FP2 chunks (two blocks each) or four of FP3/FP4 chunks
  // (one block), halved for fp32 activations (hi + lo)
  constexpr int GD = G == 1 ? 1 : (FMT == RFPX_FP2 ? 2 : 4) / VX;
  for (int c0 = 0; c0 < sc.ncols; c0 += GD) {
    const int gc = sc.ncols - c0 < GD ? sc.ncols - c0 : GD;
    if (wave < units) {
      if constexpr (G == 1) {
        gateup_pass1<FMT, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
      } else if constexpr (GD == 4) {
        if (gc == 4)
          gateup_pass<FMT, 4, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
        else if (gc == 3)
          gateup_pass<FMT, 3, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
        else if (gc == 2)
          gateup_pass<FMT, 2, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
        else
          gateup_pass<FMT, 1, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
      } else if constexpr (GD == 2) {
        if (gc == 2)
          gateup_pass<FMT, 2, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
        else
          gateup_pass<FMT, 1, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
      } else {
        gateup_pass<FMT, 1, VX, R>(a, sc, c0, geo, units, wave, waves, tile, mats, cpitch, spitch, gup);
      }
    }
    __syncthreads();
    for (int it = threadIdx.x; it < gc * rw; it += blockDim.x) {
      const int c = c0 + it / rw, row = it % rw;
      float g = 0.f, uu = 0.f;
      for (int pp = 0; pp < P; ++pp) {
        g += gup[((0 * P + pp) * q + c) * rw + row];
        uu += gup[((1 * P + pp) * q + c) * rw + row];
      }
      hout[(size_t)c * a.f + row] = silu(g) * uu;
    }
    // the next pass writes gup again
    if (c0 + GD < sc.ncols) __syncthreads();
  }
}

// Gate/up tile `tile` of slot `slot`: its rows of h for every column of the
// slot, into the slot's h in the workspace.  LDS: gup [2][2][q][rw].
template <int G, int VX>
__device__ __forceinline__ void gateup_wg(const ExpArgs &a, const SlotCols &sc, int slot,
                                          int tile, float *lds, const ExpertDesc *pre) {
  float *gup = lds;
  float *hout = reinterpret_cast<float *>(a.hp) + (size_t)slot * a.q * a.f + (size_t)tile * a.rw_gu;
  // the expert's planes: from the route table when given, else the image
  const ExpertDesc ed = pre ? *pre : load_desc(a.image, sc.expert);
  const int fmt = ed.fmt[0];
  if (!planned(a.geo_gu, fmt)) return;  // a table that disagrees with fmts
  if (fmt == RFPX_FP2) gateup_tile<RFPX_FP2, G, VX>(a, sc, ed, tile, hout, gup);
  else if (fmt == RFPX_FP3) gateup_tile<RFPX_FP3, G, VX>(a, sc, ed, tile, hout, gup);
  else gateup_tile<RFPX_FP4, G, VX>(a, sc, ed, tile, hout, gup);
}

// Gate/up tile blockIdx.x of slot blockIdx.y.  Slot 0 is the shared expert
// (every column, weight 1, no routing).  Routed slots of a step of several
// columns (G = 2) read their entry of the route table, which k_topk built
// before the launch; those of a one-column step (G = 1) run the routing
// step in LDS first.
template <int G, int VX>
__global__ __launch_bounds__(512) void k_gateup(ExpArgs a) {
  const int slot = blockIdx.y;
  __shared__ RouteLds rs;
  float *lds = dyn_lds + blockDim.x;  // past the sink
  SlotCols sc;
  if (slot == 0) {
    if (threadIdx.x < kQMax) {
      rs.cols[0][threadIdx.x] = threadIdx.x;
      rs.w[0][threadIdx.x] = 1.f;
    }
    __syncthreads();
    sc.expert = a.rp.E;
    sc.ncols = a.q;
    sc.cols = rs.cols[0];
    sc.w = rs.w[0];
  } else if constexpr (G == 2) {
    // steps of several columns are routed before the launch: the slot's
    // entry of the route table, planes included, every load issued before
    // the slot count is tested (slot < max_slots, so the entry is inside
    // the table); the column list is copied to LDS (it is then read through
    // an LDS pointer on every path; a pointer that may be either LDS or
    // global memory makes every read a slower flat access)
    const int nslots = uniform(a.rt->nslots);
    sc.expert = uniform(a.rt->expert[slot]);
    sc.ncols = uniform(a.rt->ncols[slot]);
    ExpertDesc ed;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      ed.codes[m] = uniform64(a.rt->gu_codes[slot][m]);
      ed.scales[m] = uniform64(a.rt->gu_scales[slot][m]);
      ed.fmt[m] = uniform(a.rt->gu_fmt[slot]);
    }
    ed.codes[2] = uniform64(a.rt->dn_codes[slot]);
    ed.scales[2] = uniform64(a.rt->dn_scales[slot]);
    ed.fmt[2] = uniform(a.rt->dn_fmt[slot]);
    ed.reserved = 0;
    if (threadIdx.x < kQMax) {
      rs.cols[slot][threadIdx.x] = a.rt->cols[slot][threadIdx.x];
      rs.w[slot][threadIdx.x] = a.rt->w[slot][threadIdx.x];
    }
    __syncthreads();
    if (slot >= nslots) return;
    sc.cols = rs.cols[slot];
    sc.w = rs.w[slot];
    gateup_wg<G, VX>(a, sc, slot, blockIdx.x, lds, &ed);
    return;
  } else {
    // one-column step: routing in the workgroup, slot s is rank s - 1
    route_q1(a.rp, &rs, slot);
    if (slot >= uniform(rs.nslots)) return;
    if (blockIdx.x == 0) {
      publish_route(rs, a.q, slot, slot == 1, a.rt);
      if (threadIdx.x == 0) publish_down_desc(a.image, rs.expert[slot], slot, a.rt);
      if (slot == 1 && threadIdx.x == 64) publish_down_desc(a.image, a.rp.E, 0, a.rt);
    }
    sc.expert = uniform(rs.expert[slot]);
    sc.ncols = uniform(rs.ncols[slot]);
    sc.cols = rs.cols[slot];
    sc.w = rs.w[slot];
  }
  gateup_wg<G, VX>(a, sc, slot, blockIdx.x, lds, nullptr);
}

// ----------------------------------------------------------------- down

// *p += v in LDS without waiting for the old value (ds_add_f32): the adds
// of one wave to its own accumulator rows take effect in program order, so
// the sums are the same from run to run.
__device__ __forceinline__ void lds_add(float *p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Weighted row results of one computed down unit into the wave's
// accumulator rows accw[column][row] (LDS, one writer lane per entry).  The
// columns and weights come as separate scalars: a two-entry array indexed
// by a lane value would be placed in scratch memory.
template <int GP, int R>
__device__ __forceinline__ void down_reduce(const float (&to)[R][1][GP], const Geo &geo,
                                            const UnitPos &up, int rw, int col0, int col1,
                                            float wgt0, float wgt1, float *accw) {
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  if (geo.lpr == 64) {
    constexpr int N = R * GP;
    float flat[N];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int g = 0; g < GP; ++g) flat[i * GP + g] = to[i][0][g];
    const float v = multi_sum<N>(flat, lane);
    const int n = ms_index<N>(lane);
    const int i = n / GP, g = n % GP;
    const int cg = (GP == 2 && g) ? col1 : col0;
    const float wg = (GP == 2 && g) ? wgt1 : wgt0;
    lds_add(ms_writer<N>(lane) ? &accw[cg * rw + up.rloc_u + i] : lane_sink(), wg * v);
  } else {
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float v = group_sum(to[i][0][g], geo.lpr);
        lds_add(li == 0 ? &accw[(g ? col1 : col0) * rw + up.rloc_u + rg + geo.rpi * i] : lane_sink(),
                (g ? wgt1 : wgt0) * v);
      }
  }
}

// One unit of one slot's down matrix for GP compact columns c0..: the
// weighted row results are added into the wave's own accumulator rows
// accw[column][row] (LDS, one writer lane per entry).
template <int FMT, int GP, int R>
__device__ __forceinline__ void down_unit(const ExpArgs &a, const SlotCols &sc, int slot, int c0,
                                          const Geo &geo, const UnitPos &up, int r0,
                                          const MatPtr (&mats)[1], uint32_t cpitch,
                                          uint32_t spitch, float *accw) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const int ch = li + geo.lpr * up.part;
  const uint32_t coff = (uint32_t)(rg * cpitch + ch * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + ch * F::SBYTES);
  uint32_t cw[R][1][F::CW], sw[R][1];
  unit_load<FMT, 1, R>(mats, cpitch, spitch, r0 + up.rloc_u, geo.rpi, coff, soff, cw, sw);
  const uint32_t *hps = a.hp + (size_t)slot * a.q * a.nb_f * 32;
  uint32_t xr[GP][F::CB][2][16];
  float ncr[GP][F::CB];
  load_h<FMT, GP>(hps, a.nb_f, c0, ch, xr);
  prep_h<FMT, GP>(xr, ncr);
  float to[R][1][GP];
  unit_compute_code<FMT, GP, R>(cw, sw, xr, ncr, to);
  const int col0 = sc.col(c0), col1 = GP == 2 ? sc.col(c0 + GP - 1) : col0;
  const float wgt0 = sc.weight(c0), wgt1 = GP == 2 ? sc.weight(c0 + GP - 1) : wgt0;
  down_reduce<GP, R>(to, geo, up, a.rw_dn, col0, col1, wgt0, wgt1, accw);
}

// The only unit of a slot's down matrix in a one-column step (rows r0 ..
// r0 + R of the tile, part 0), with the slot's h already in
// registers (FP3/FP4: one block per lane): weights, products, and the
// weighted row results into the wave's accumulator rows.
template <int FMT>
__device__ __forceinline__ void down_unit_h(const ExpArgs &a, uint64_t codes, uint64_t scales,
                                            int r0, int col0, float wgt,
                                            const uint32_t (&hx)[1][1][2][16],
                                            const float (&hn)[1][1], float *accw) {
  using F = Fmt<FMT>;
  static_assert(F::CB == 1, "one block per lane");
  constexpr int R = unit_rows_for(FMT, 1);
  const Geo geo = a.geo_dn[FMT];
  const uint32_t cpitch = (uint32_t)(a.f / 32) * code_bytes(FMT);
  const uint32_t spitch = (uint32_t)(a.f / 32) * scale_bytes(FMT);
  const MatPtr mats[1] = {{make_rsrc(a.image + codes, a.d * cpitch), make_rsrc(a.image + scales, a.d * spitch)}};
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const uint32_t coff = (uint32_t)(rg * cpitch + li * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + li * F::SBYTES);
  uint32_t cw[R][1][F::CW], sw[R][1];
  unit_load<FMT, 1, R>(mats, cpitch, spitch, r0, geo.rpi, coff, soff, cw, sw);
  float to[R][1][1];
  unit_compute_code<FMT, 1, R>(cw, sw, hx, hn, to);
  const UnitPos up = unit_pos(0, 1, R, geo.rpi);
  down_reduce<1, R>(to, geo, up, a.rw_dn, col0, col0, wgt, wgt, accw);
}

// Units [u0, u1) of one slot's down matrix for GP compact columns c0..,
// all in column part 0: the wave loads (and prepares) the slot's h of its chunk
// once and streams the units with the next unit's code and scale loads in
// flight while one is decoded (two register sets, used in turn).
template <int FMT, int GP, int R>
__device__ __forceinline__ void down_run(const ExpArgs &a, const SlotCols &sc, int slot, int c0,
                                         const Geo &geo, int u0, int u1, int r0,
                                         const MatPtr (&mats)[1], uint32_t cpitch,
                                         uint32_t spitch, float *accw) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const int ch = li;
  const uint32_t coff = (uint32_t)(rg * cpitch + ch * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + ch * F::SBYTES);
  const int P = geo.tpl, rw = a.rw_dn;
  uint32_t cwa[R][1][F::CW], swa[R][1], cwb[R][1][F::CW], swb[R][1];
  int u = u0;
  UnitPos up = unit_pos(u, P, R, geo.rpi);
  unit_load<FMT, 1, R, true>(mats, cpitch, spitch, r0 + up.rloc_u, geo.rpi, coff, soff, cwa, swa);
  const uint32_t *hps = a.hp + (size_t)slot * a.q * a.nb_f * 32;
  uint32_t xr[GP][F::CB][2][16];
  float ncr[GP][F::CB];
  load_h<FMT, GP>(hps, a.nb_f, c0, ch, xr);
  prep_h<FMT, GP>(xr, ncr);
  const int col0 = sc.col(c0), col1 = GP == 2 ? sc.col(c0 + GP - 1) : col0;
  const float wgt0 = sc.weight(c0), wgt1 = GP == 2 ? sc.weight(c0 + GP - 1) : wgt0;
  const uint32_t one = one_one_vgpr();
  // as in gateup_pass: the next unit's loads are unconditional (past the
  // run they address row d, outside the matrix, and read nothing), units go
  // in pairs with the loop's only exit at its head, an odd last one after
  const int past = a.d;
  while (u + 1 < u1) {
    {
      const int un = u + 1;
      const UnitPos upn = unit_pos(un, P, R, geo.rpi);
      unit_load<FMT, 1, R, true>(mats, cpitch, spitch, r0 + upn.rloc_u, geo.rpi, coff, soff, cwb, swb);
      float to[R][1][GP];
      unit_compute_code<FMT, GP, R>(cwa, swa, xr, ncr, to);
      down_reduce<GP, R>(to, geo, up, rw, col0, col1, wgt0, wgt1, accw);
      u = un;
      up = upn;
    }
    {
      const int un = u + 1;
      const UnitPos upn = unit_pos(un, P, R, geo.rpi);
      unit_load<FMT, 1, R, true>(mats, cpitch, spitch, un < u1 ? r0 + upn.rloc_u : past, geo.rpi,
                                 coff, soff, cwa, swa);
      float to[R][1][GP];
      unit_compute_code<FMT, GP, R>(cwb, swb, xr, ncr, to);
      down_reduce<GP, R>(to, geo, up, rw, col0, col1, wgt0, wgt1, accw);
      u = un;
      up = upn;
    }
  }
  if (u < u1) {
    float to[R][1][GP];
    unit_compute_code<FMT, GP, R>(cwa, swa, xr, ncr, to);
    down_reduce<GP, R>(to, geo, up, rw, col0, col1, wgt0, wgt1, accw);
  }
}

// Units [u0, u1) of one slot for every column of the slot, in passes of
// up to G columns (FP2 down matrices one column per pass: their chunks hold
// two blocks, so two-column passes would need 128 registers of h).
template <int FMT, int G>
__device__ __forceinline__ void down_slot_run(const ExpArgs &a, const SlotCols &sc, int slot,
                                              const ExpertDesc &ed, int r0, int u0, int u1,
                                              float *accw) {
  constexpr int R = unit_rows_for(FMT, G);
  const Geo geo = a.geo_dn[FMT];
  const uint32_t cpitch = (uint32_t)(a.f / 32) * code_bytes(FMT);
  const uint32_t spitch = (uint32_t)(a.f / 32) * scale_bytes(FMT);
  const MatPtr mats[1] = {
      {make_rsrc(a.image + ed.codes[2], a.d * cpitch), make_rsrc(a.image + ed.scales[2], a.d * spitch)}};
  constexpr int GD = FMT == RFPX_FP2 ? 1 : G;
  for (int c0 = 0; c0 < sc.ncols; c0 += GD) {
    if constexpr (GD == 2) {
      if (sc.ncols - c0 >= 2) down_run<FMT, 2, R>(a, sc, slot, c0, geo, u0, u1, r0, mats, cpitch, spitch, accw);
      else down_run<FMT, 1, R>(a, sc, slot, c0, geo, u0, u1, r0, mats, cpitch, spitch, accw);
    } else {
      down_run<FMT, 1, R>(a, sc, slot, c0, geo, u0, u1, r0, mats, cpitch, spitch, accw);
    }
  }
}

// The units of one slot that fall to this wave: units are dealt to the
// waves round-robin in slot order (`item` counts the units dealt so far).
// Only a wave that owns one of the slot's units builds the slot's buffer
// resources.
template <int FMT, int G>
__device__ __forceinline__ void down_slot(const ExpArgs &a, const SlotCols &sc, int slot,
                                          const ExpertDesc &ed, int r0, int wave, int waves,
                                          int &item, float *accw) {
  constexpr int R = unit_rows_for(FMT, G);
  const Geo geo = a.geo_dn[FMT];
  const int P = geo.tpl;
  const int units = a.rw_dn / (R * geo.rpi) * P;
  // this wave's first unit of the slot: (item + u) % waves == wave
  const int first = (wave - item % waves + waves) % waves;
  item += units;
  if (first >= units) return;
  const uint32_t cpitch = (uint32_t)(a.f / 32) * code_bytes(FMT);
  const uint32_t spitch = (uint32_t)(a.f / 32) * scale_bytes(FMT);
  const MatPtr mats[1] = {
      {make_rsrc(a.image + ed.codes[2], a.d * cpitch), make_rsrc(a.image + ed.scales[2], a.d * spitch)}};
  // FP2 chunks hold two blocks, so two-column passes would need 128
  // registers of h: FP2 down matrices take one column per pass
  constexpr int GD = FMT == RFPX_FP2 ? 1 : G;
  for (int u = first; u < units; u += waves) {
    const UnitPos up = unit_pos(u, P, R, geo.rpi);
    for (int c0 = 0; c0 < sc.ncols; c0 += GD) {
      if constexpr (GD == 2) {
        if (sc.ncols - c0 >= 2)
          down_unit<FMT, 2, R>(a, sc, slot, c0, geo, up, r0, mats, cpitch, spitch, accw);
        else
          down_unit<FMT, 1, R>(a, sc, slot, c0, geo, up, r0, mats, cpitch, spitch, accw);
      } else {
        down_unit<FMT, 1, R>(a, sc, slot, c0, geo, up, r0, mats, cpitch, spitch, accw);
      }
    }
  }
}

// Down rows [r0, r0 + RW_DN) of every slot, combined into y.  The slot table
// is copied to LDS first; each wave accumulates its units into its own LDS
// rows, and the epilogue sums the waves in a fixed order, so y is the same
// bit for bit from run to run.
template <int G>
__global__ __launch_bounds__(G == 1 ? 64 * kDnWavesQ1 : 64 * kDnWavesQn) void k_down(ExpArgs a) {
  __shared__ int32_t t_ncols[kMaxSlots];
  __shared__ int32_t t_cols[kMaxSlots][kQMax];
  __shared__ float t_w[kMaxSlots][kQMax];
  __shared__ uint64_t t_codes[kMaxSlots], t_scales[kMaxSlots];
  __shared__ int32_t t_fmt[kMaxSlots];
  float *acc = dyn_lds + blockDim.x;  // [waves][q][rw], past the sink
  const int rw = a.rw_dn, q = a.q;
  const int waves = blockDim.x >> 6;
  const int wave = uniform(threadIdx.x >> 6);
  // a one-column step always has k + 1 slots (k distinct experts), so its
  // table loads need not wait for the slot count
  const int nslots = G == 1 ? a.rp.k + 1 : uniform(a.rt->nslots);
  for (int i = threadIdx.x; i < waves * q * rw; i += blockDim.x) acc[i] = 0.f;
  // One-column steps with one unit per slot and one wave per slot: wave w's
  // unit is slot w's, and its h (one block per lane, 32 words) does
  // not depend on the route table.  Waves other than the table reader's
  // load it before the table is read, the table reader right after, so
  // that h is not in flight with the weights.
  const bool early = G == 1 && a.h_early;
  uint32_t hx[1][1][2][16];
  float hn[1][1];
  // the lane's block: FP3 and FP4 chunks are one block, so both formats
  // give a row of nb_f chunks <= 64 lanes (one column part), lane l block
  // l mod nb_f
  const int hch = (threadIdx.x & 63) % (a.nb_f < 64 ? a.nb_f : 64);
  if (early && wave != 0 && wave < nslots)
    load_h<RFPX_FP4, 1>(a.hp + (size_t)wave * a.nb_f * 32, a.nb_f, 0, hch, hx);
  // the slot table and each slot's down-matrix entry of the image table,
  // all loads in flight together
  for (int i = threadIdx.x; i < nslots * (kQMax + 1); i += blockDim.x) {
    const int s = i / (kQMax + 1), j = i % (kQMax + 1);
    if (j == kQMax) {
      t_ncols[s] = a.rt->ncols[s];
      t_codes[s] = a.rt->dn_codes[s];
      t_scales[s] = a.rt->dn_scales[s];
      // a format the launch was not planned for (a device table that
      // disagrees with the host table) becomes 0: the slot is skipped
      const int f = a.rt->dn_fmt[s];
      t_fmt[s] = planned(a.geo_dn, f) ? f : 0;
    } else {
      t_cols[s][j] = a.rt->cols[s][j];
      t_w[s][j] = a.rt->w[s][j];
    }
  }
  if (early && wave == 0) load_h<RFPX_FP4, 1>(a.hp, a.nb_f, 0, hch, hx);
  __syncthreads();
  const int r0 = blockIdx.x * rw;
  float *accw = acc + wave * q * rw;
  if (early) {
    if (wave < nslots) {
      const int fmt = uniform(t_fmt[wave]);
      const int col0 = uniform(t_cols[wave][0]);
      const float wgt = __int_as_float(uniform(__float_as_int(t_w[wave][0])));
      const uint64_t codes = uniform64(t_codes[wave]), scales = uniform64(t_scales[wave]);
      if (fmt == RFPX_FP3) {
        prep_h<RFPX_FP3, 1>(hx, hn);
        down_unit_h<RFPX_FP3>(a, codes, scales, r0, col0, wgt, hx, hn, accw);
      } else if (fmt == RFPX_FP4) {
        prep_h<RFPX_FP4, 1>(hx, hn);
        down_unit_h<RFPX_FP4>(a, codes, scales, r0, col0, wgt, hx, hn, accw);
      }
    }
  }
  // Steps of several columns: the units of all slots in slot order, cut
  // into one contiguous run per wave (a run keeps a slot's h in registers
  // across its units); needs every down format in one column part.
  // (units per slot by format, selected: a kernel-argument array indexed
  // at run time would be copied to scratch memory)
  const bool runs = G == 2 && a.geo_dn[RFPX_FP2].tpl <= 1 && a.geo_dn[RFPX_FP3].tpl <= 1 &&
                    a.geo_dn[RFPX_FP4].tpl <= 1;
  const int ups2 = rw / (unit_rows_for(RFPX_FP2, G) * a.geo_dn[RFPX_FP2].rpi);
  const int ups3 = rw / (unit_rows_for(RFPX_FP3, G) * a.geo_dn[RFPX_FP3].rpi);
  const int ups4 = rw / (unit_rows_for(RFPX_FP4, G) * a.geo_dn[RFPX_FP4].rpi);
  auto slot_units = [&](int fmt) {
    return fmt == RFPX_FP2 ? ups2 : fmt == RFPX_FP3 ? ups3 : fmt == RFPX_FP4 ? ups4 : 0;
  };
  if (runs) {
    // The wave finds its run without walking the table slot by slot (one
    // LDS read and wait per slot, before the first weight load): lane l
    // takes slot l's unit count (slot 64, the last possible one, is read
    // apart), a wave scan gives the prefix sums, a ballot the first slot
    // that reaches into the run, and each slot's start and count are then
    // read from the scan's lanes.
    const int l = threadIdx.x & 63;
    const int cl = l < nslots ? slot_units(t_fmt[l]) : 0;
    int inc = cl;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(inc, off, 64);
      inc += l >= off ? v : 0;
    }
    const int c64 = nslots > 64 ? slot_units(uniform(t_fmt[64])) : 0;
    const int tot64 = __builtin_amdgcn_readlane(inc, 63);
    const int total = tot64 + c64;
    const int lo = total * wave / waves, hi = total * (wave + 1) / waves;
    // slots that end at or before the run's start
    int s = __popcll(__ballot(l < nslots && inc <= lo));
    for (; s < nslots; ++s) {
      const int ups = s < 64 ? __builtin_amdgcn_readlane(cl, s) : c64;
      const int start = s < 64 ? __builtin_amdgcn_readlane(inc, s) - ups : tot64;
      if (start >= hi) break;
      const int fmt = uniform(t_fmt[s]);
      const int u0 = lo > start ? lo - start : 0, u1 = hi < start + ups ? hi - start : ups;
      if (u0 < u1) {
        SlotCols sc;
        sc.expert = -1;
        sc.ncols = uniform(t_ncols[s]);
        sc.cols = t_cols[s];
        sc.w = t_w[s];
        ExpertDesc ed{};
        ed.codes[2] = uniform64(t_codes[s]);
        ed.scales[2] = uniform64(t_scales[s]);
        if (fmt == RFPX_FP2) down_slot_run<RFPX_FP2, G>(a, sc, s, ed, r0, u0, u1, accw);
        else if (fmt == RFPX_FP3) down_slot_run<RFPX_FP3, G>(a, sc, s, ed, r0, u0, u1, accw);
        else down_slot_run<RFPX_FP4, G>(a, sc, s, ed, r0, u0, u1, accw);
      }
    }
  }
  int item = 0;
  for (int s = 0; s < nslots && !runs && !early; ++s) {
    SlotCols sc;
    sc.expert = -1;  // not needed: the down entry is in LDS
    sc.ncols = uniform(t_ncols[s]);
    sc.cols = t_cols[s];
    sc.w = t_w[s];
    ExpertDesc ed{};
    ed.codes[2] = uniform64(t_codes[s]);
    ed.scales[2] = uniform64(t_scales[s]);
    const int fmt = uniform(t_fmt[s]);
    if (fmt == RFPX_FP2) down_slot<RFPX_FP2, G>(a, sc, s, ed, r0, wave, waves, item, accw);
    else if (fmt == RFPX_FP3) down_slot<RFPX_FP3, G>(a, sc, s, ed, r0, wave, waves, item, accw);
    else if (fmt == RFPX_FP4) down_slot<RFPX_FP4, G>(a, sc, s, ed, r0, wave, waves, item, accw);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < q * rw; i += blockDim.x) {
    const int c = i / rw, row = i % rw;
    float v = 0.f;
    for (int w = 0; w < waves; ++w) v += acc[(w * q + c) * rw + row];
    a.y[(size_t)c * a.d + r0 + row] = v;
  }
}

ExpArgs make_args(const ForwardPlan &p) {
  ExpArgs a{};
  a.image = p.image;
  a.rt = reinterpret_cast<RouteTable *>(p.ws + p.wl.route);
  a.rp = route_params(p);
  a.xp = reinterpret_cast<const uint32_t *>(p.ws + p.wl.xp);
  a.xnc = reinterpret_cast<const float *>(p.ws + p.wl.xnc);
  a.hp = reinterpret_cast<uint32_t *>(p.ws + p.wl.hp);
  a.y = p.y;
  a.d = p.d;
  a.f = p.f;
  a.q = p.q;
  a.nb_d = p.d / 32;
  a.nb_f = p.f / 32;
  for (int i = 0; i < 5; ++i) {
    a.geo_gu[i] = p.geo_gu[i];
    a.geo_dn[i] = p.geo_dn[i];
  }
  a.rw_gu = p.rw_gu;
  a.rw_dn = p.rw_dn;
  a.h_early = p.h_early ? 1 : 0;
  return a;
}

}  // namespace

hipError_t launch_experts(const ForwardPlan &p) {
  const ExpArgs a = make_args(p);
  const dim3 ggu(p.f / p.rw_gu, p.wl.max_slots), gdn(p.d / p.rw_dn);
  const unsigned nt = 64 * p.wmax, ntg = 64 * p.wgu;
  const size_t lds_gu = ((size_t)ntg + 4 * p.q * p.rw_gu) * sizeof(float);          // sink + gup
  const size_t lds_dn = ((size_t)nt + (size_t)p.wmax * p.q * p.rw_dn) * sizeof(float);  // sink + acc
  const bool bf = p.xtype == RFPX_X_BF16;
  hipEvent_t *ev = (hipEvent_t *)p.events;
  hipEvent_t e0 = ev ? ev[2] : nullptr, e1 = ev ? ev[3] : nullptr;
  void (*gu)(ExpArgs) = p.g == 1 ? (bf ? k_gateup<1, 1> : k_gateup<1, 2>)
                                 : (bf ? k_gateup<2, 1> : k_gateup<2, 2>);
  hipError_t e = launch_k(gu, ggu, dim3(ntg), lds_gu, p.stream, a, e0, e1);
  if (e != hipSuccess) return e;
  e0 = ev ? ev[4] : nullptr;
  e1 = ev ? ev[5] : nullptr;
  return launch_k(p.g == 1 ? k_down<1> : k_down<2>, gdn, dim3(nt), lds_dn, p.stream, a, e0, e1);
}

}  // namespace rfpx
