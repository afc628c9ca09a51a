// expert.hip -- expert-grouped dequantize-and-GEMV for the routed and the
// shared experts, decode path.
//
// Page "APU 实现 token 自由…" (ainomam.com), section "Lucebox 的优化三板斧":
// in the q-column verify path each packed weight is decoded once and applied
// to every verify column.  Page "Lucebox专攻DeepSeek V4…" (m.mzlw.cn),
// section "常见疑问" (FAQ): decode is bound by memory bandwidth.
//
// Three launches after the router (route.hip):
//   k_gateup  grid (f / RW, slots).  Workgroups of routed slots first run
//             the routing step in LDS (rfpx_route.hpp; deterministic, so all
//             agree); workgroup (0, s) publishes slot s for the launches that
//             follow.  Workgroups of slot 0 (the shared expert) need no
//             routing and start streaming at once.  A workgroup owns RW
//             consecutive rows of the gate and up matrices of its slot's
//             expert; each wave owns R rows of both, issues every code and
//             scale load for them up front (buffer loads: scalar descriptor,
//             scalar row offset, 32-bit lane offset), decodes each block in
//             registers once and applies it to all of the slot's columns
//             (v_dot2c_f32_bf16 on the prepared activations), reduces each
//             row across its lanes and forms h = silu(g) * u.  The workgroup
//             then prepares h for the down matrix (bf16 hi + lo pair words,
//             one thread per pair word).
//   k_down    grid (d / RW, slots): the same over the down matrix; each row
//             result times the column's gating weight is stored as a
//             partial.
//   k_combine y[c][i] = sum over slots (in slot order) of the partials:
//             deterministic, no atomics, no device-scope fences.
// Lane geometry (Geo): with a row of >= 64 chunks a wave covers one row per
// step and lane l reads chunks l and l+64 (fully coalesced 1 KiB requests);
// shorter rows give each wave 64/cpl rows per step.
#include "rfpx_route.hpp"

namespace rfpx {
namespace {

struct ExpArgs {
  const uint8_t *image;
  RouteTable *rt;
  RouteParams rp;
  const uint32_t *xp;
  const float *xnc;
  uint32_t *hp;
  float *hnc;
  float *part;
  float *y;
  int d, f, q, nb_d, nb_f;
  int rw_gu, rw_dn;
  Geo geo_gu[5], geo_dn[5];
};

// The columns of one slot: expert and count in scalar registers; the column
// list and weights stay in LDS or the workspace table and are read when a
// pass needs them (indexing a register array by a loop counter would put it
// in scratch memory).
struct SlotCols {
  int expert, ncols;
  const int *cols;   // [ncols] global column index of each compact column
  const float *w;    // [ncols] gating weight
  // i must be wave-uniform (the result is taken from the first lane)
  __device__ int col(int i) const { return uniform(cols[i]); }
  // i may differ between lanes
  __device__ float weight(int i) const { return w[i]; }
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

// Per-lane partial dot products of R rows of NM matrices with G columns for
// one "unit": rows row_u + rpi*i (i < R) of one column part, the lane's own
// chunk at byte offsets coff (codes) and soff (scales) within a row.  Rows
// are read through the matrix planes' buffer resources at scalar offset
// row * pitch (row_u is wave-uniform).  All code and scale loads are issued
// first; then rows are decoded one at a time (scheduling fences keep the
// decode of one row from being hoisted over the next, which would multiply
// register pressure).
template <int FMT, int G, int VX, int NM, int R>
__device__ __forceinline__ void unit_rows(const MatPtr (&mats)[NM], uint32_t cpitch,
                                          uint32_t spitch, int row_u, int rpi,
                                          uint32_t coff, uint32_t soff,
                                          const uint32_t (&xr)[G][Fmt<FMT>::CB][VX][16],
                                          const float (&ncr)[G][Fmt<FMT>::CB],
                                          float (&tot)[R][NM][G]) {
  using F = Fmt<FMT>;
  uint32_t cw[R][NM][F::CW];
  uint32_t sw[R][NM];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t row = (uint32_t)(row_u + rpi * i);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      load_chunk<FMT>(mats[m].codes, coff, row * cpitch, cw[i][m]);
      sw[i][m] = load_scale<FMT>(mats[m].scales, soff, row * spitch);
    }
  }
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
        decode_pairs<FMT>(&cw[i][m][j * F::BW], pr);
        const float s = block_scale<FMT>(block_scale_bits<FMT>(sw[i][m], j));
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = ncr[g][j];
#pragma unroll
          for (int v = 0; v < VX; ++v)
#pragma unroll
            for (int p = 0; p < 16; ++p) acc = dot2(pr[p], xr[g][j][v][p], acc);
          tot[i][m][g] = fmaf(acc, s, tot[i][m][g]);
        }
      }
    }
  }
}

// Prepared activations (or prepared h) of the blocks of chunk `ch` for G
// columns: block b of column c sits at ((c * nb) + b) * VX * 16 words, its
// accumulator start at c * nb + b.
template <int FMT, int G, int VX>
__device__ __forceinline__ void load_prepared(const uint32_t *__restrict__ pw,
                                              const float *__restrict__ pnc, int nb,
                                              const int *colidx, int ch,
                                              uint32_t (&xr)[G][Fmt<FMT>::CB][VX][16],
                                              float (&ncr)[G][Fmt<FMT>::CB]) {
  using F = Fmt<FMT>;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int j = 0; j < F::CB; ++j) {
      const size_t item = (size_t)colidx[g] * nb + ch * F::CB + j;
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

// Where a wave's unit lies: unit u covers rows [rg0, rg0 + R*rpi) of the
// tile (rows rg0 + rg + rpi*i for the lane's row group rg) and column part
// p (chunks 64p .. 64p+63 of each row when a row has 128 chunks).
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

// ------------------------------------------------------------ gate / up

// One unit of GP columns (c0 .. c0+GP-1 of the slot): per-lane partials of
// gate and up rows, reduced across the lanes, written as part sums to LDS.
template <int FMT, int GP, int VX, int R>
__device__ __forceinline__ void gateup_unit(const ExpArgs &a, const SlotCols &sc, int c0,
                                            const Geo &geo, const UnitPos &up, int tile,
                                            const MatPtr (&mats)[2], uint32_t cpitch,
                                            uint32_t spitch, float *gup /* [2][P][kQMax][rw] */) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const int ch = li + geo.lpr * up.part;
  const uint32_t *xpf = a.xp + (size_t)(FMT - RFPX_FP2) * a.q * a.nb_d * VX * 16;
  const float *xncf = a.xnc + (size_t)(FMT - RFPX_FP2) * a.q * a.nb_d;
  int colidx[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) colidx[g] = sc.col(c0 + g);
  uint32_t xr[GP][F::CB][VX][16];
  float ncr[GP][F::CB];
  load_prepared<FMT, GP, VX>(xpf, xncf, a.nb_d, colidx, ch, xr, ncr);
  __builtin_amdgcn_sched_barrier(0);  // activation loads go out before the weights
  const uint32_t coff = (uint32_t)(rg * cpitch + ch * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + ch * F::SBYTES);
  float tot[R][2][GP];
  unit_rows<FMT, GP, VX, 2, R>(mats, cpitch, spitch, tile * a.rw_gu + up.rloc_u, geo.rpi,
                               coff, soff, xr, ncr, tot);
  const int P = geo.tpl, rw = a.rw_gu;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        const float v = group_sum(tot[i][m][g], geo.lpr);
        if (li == 0)
          gup[((m * P + up.part) * kQMax + c0 + g) * rw + up.rloc_u + rg + geo.rpi * i] = v;
      }
}

template <int FMT, int G, int VX, int R>
__device__ __forceinline__ void gateup_tile(const ExpArgs &a, const SlotCols &sc,
                                            const ExpertDesc &ed, float *hs, float *gup) {
  const Geo geo = a.geo_gu[FMT];
  const uint32_t cpitch = (uint32_t)(a.d / 32) * code_bytes(FMT);
  const uint32_t spitch = (uint32_t)(a.d / 32) * scale_bytes(FMT);
  const MatPtr mats[2] = {
      {make_rsrc(a.image + ed.codes[0], a.f * cpitch), make_rsrc(a.image + ed.scales[0], a.f * spitch)},
      {make_rsrc(a.image + ed.codes[1], a.f * cpitch), make_rsrc(a.image + ed.scales[1], a.f * spitch)}};
  const int P = geo.tpl, rw = a.rw_gu;
  const int units = rw / (R * geo.rpi) * P;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int waves = blockDim.x >> 6;
  const float A = code_gain(FMT);
  for (int c0 = 0; c0 < sc.ncols; c0 += G) {
    const int gc = (G == 2 && sc.ncols - c0 >= 2) ? 2 : 1;
    for (int u = wave; u < units; u += waves) {
      const UnitPos up = unit_pos(u, P, R, geo.rpi);
      if (gc == 2)
        gateup_unit<FMT, (G == 2 ? 2 : 1), VX, R>(a, sc, c0, geo, up, blockIdx.x, mats, cpitch, spitch, gup);
      else
        gateup_unit<FMT, 1, VX, R>(a, sc, c0, geo, up, blockIdx.x, mats, cpitch, spitch, gup);
    }
    __syncthreads();
    for (int it = threadIdx.x; it < gc * rw; it += blockDim.x) {
      const int c = c0 + it / rw, row = it % rw;
      float g = 0.f, uu = 0.f;
      for (int pp = 0; pp < P; ++pp) {
        g += gup[((0 * P + pp) * kQMax + c) * rw + row];
        uu += gup[((1 * P + pp) * kQMax + c) * rw + row];
      }
      hs[c * rw + row] = silu(A * g) * (A * uu);
    }
    __syncthreads();
  }
}

// One pair word (hi and lo parts) of one block of h for the down format,
// and its share of the block's accumulator start.
template <int FMT_DN>
__device__ __forceinline__ float prep_h_pair(const float *hblk, int p, uint32_t *dst) {
  int lo, hi;
  float slo, shi;
  pair_def<FMT_DN>(p, lo, hi, slo, shi);
  const float vl = hblk[lo], vh = hblk[hi];
  const uint32_t lh = float_to_bf16_rne(vl), hh = float_to_bf16_rne(vh);
  const uint32_t ll = float_to_bf16_rne(vl - bf16_bits_to_float(lh));
  const uint32_t hl = float_to_bf16_rne(vh - bf16_bits_to_float(hh));
  dst[p] = pair_word<FMT_DN>(lh, hh, slo, shi);
  dst[16 + p] = pair_word<FMT_DN>(ll, hl, slo, shi);
  return pair_nc<FMT_DN>(bf16_bits_to_float(lh), bf16_bits_to_float(hh), slo, shi) +
         pair_nc<FMT_DN>(bf16_bits_to_float(ll), bf16_bits_to_float(hl), slo, shi);
}

template <int G, int VX, int R>
__global__ __launch_bounds__(512) void k_gateup(ExpArgs a) {
  const int slot = blockIdx.y;
  __shared__ RouteLds rs;
  extern __shared__ float lds[];  // hs [kQMax][rw], then gup [2][2][kQMax][rw]
  float *hs = lds;
  float *gup = lds + kQMax * a.rw_gu;
  SlotCols sc;
  if (slot == 0) {  // the shared expert: every column, weight 1, no routing
    if (threadIdx.x < kQMax) {
      rs.cols[0][threadIdx.x] = threadIdx.x;
      rs.w[0][threadIdx.x] = 1.f;
    }
    __syncthreads();
    sc.expert = a.rp.E;
    sc.ncols = a.q;
  } else {
    route_wg(a.rp, &rs);
    if (slot >= uniform(rs.nslots)) return;
    if (blockIdx.x == 0) publish_route(rs, a.q, slot, slot == 1, a.rt);
    sc.expert = uniform(rs.expert[slot]);
    sc.ncols = uniform(rs.ncols[slot]);
  }
  sc.cols = rs.cols[slot];
  sc.w = rs.w[slot];
  const ExpertDesc ed = load_desc(a.image, sc.expert);
  const int fmt = ed.fmt[0];
  if (fmt == RFPX_FP2) gateup_tile<RFPX_FP2, G, VX, R>(a, sc, ed, hs, gup);
  else if (fmt == RFPX_FP3) gateup_tile<RFPX_FP3, G, VX, R>(a, sc, ed, hs, gup);
  else gateup_tile<RFPX_FP4, G, VX, R>(a, sc, ed, hs, gup);
  // prepare h of this tile for the down matrix: 16 threads per (column,
  // block), one pair word each; the block's accumulator start is the sum of
  // the 16 shares (aligned groups of 16 lanes)
  const int nbt = a.rw_gu / 32;
  const int fdn = ed.fmt[2];
  const int nitems = sc.ncols * nbt * 16;
  for (int base = 0; base < nitems; base += blockDim.x) {
    const int it = base + threadIdx.x;
    float share = 0.f;
    size_t item = 0;
    if (it < nitems) {
      const int p = it & 15, cb = it >> 4;
      const int ci = cb / nbt, bt = cb % nbt;
      item = ((size_t)slot * a.q + ci) * a.nb_f + blockIdx.x * nbt + bt;
      const float *hblk = hs + ci * a.rw_gu + 32 * bt;
      uint32_t *dst = a.hp + item * 32;
      if (fdn == RFPX_FP2) share = prep_h_pair<RFPX_FP2>(hblk, p, dst);
      else if (fdn == RFPX_FP3) share = prep_h_pair<RFPX_FP3>(hblk, p, dst);
      else share = prep_h_pair<RFPX_FP4>(hblk, p, dst);
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) share += __shfl_xor(share, off, 64);
    if (it < nitems && (it & 15) == 0) a.hnc[item] = share;
  }
}

// ----------------------------------------------------------------- down

template <int FMT, int GP, int R>
__device__ __forceinline__ void down_unit(const ExpArgs &a, int slot, int c0, const Geo &geo,
                                          const UnitPos &up, int tile, const MatPtr (&mats)[1],
                                          uint32_t cpitch, uint32_t spitch,
                                          float *op /* [P][kQMax][rw] */) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int rg = lane / geo.lpr, li = lane % geo.lpr;
  const int ch = li + geo.lpr * up.part;
  const uint32_t *hps = a.hp + (size_t)slot * a.q * a.nb_f * 32;
  const float *hncs = a.hnc + (size_t)slot * a.q * a.nb_f;
  int colidx[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) colidx[g] = c0 + g;  // compact column index
  uint32_t xr[GP][F::CB][2][16];
  float ncr[GP][F::CB];
  load_prepared<FMT, GP, 2>(hps, hncs, a.nb_f, colidx, ch, xr, ncr);
  __builtin_amdgcn_sched_barrier(0);  // h loads go out before the weights
  const uint32_t coff = (uint32_t)(rg * cpitch + ch * F::CBYTES);
  const uint32_t soff = (uint32_t)(rg * spitch + ch * F::SBYTES);
  float to[R][1][GP];
  unit_rows<FMT, GP, 2, 1, R>(mats, cpitch, spitch, tile * a.rw_dn + up.rloc_u, geo.rpi,
                              coff, soff, xr, ncr, to);
  const int rw = a.rw_dn;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      const float v = group_sum(to[i][0][g], geo.lpr);
      if (li == 0) op[(up.part * kQMax + c0 + g) * rw + up.rloc_u + rg + geo.rpi * i] = v;
    }
}

template <int FMT, int G, int R>
__device__ __forceinline__ void down_tile(const ExpArgs &a, const SlotCols &sc, int slot,
                                          const ExpertDesc &ed, float *op) {
  const Geo geo = a.geo_dn[FMT];
  const uint32_t cpitch = (uint32_t)(a.f / 32) * code_bytes(FMT);
  const uint32_t spitch = (uint32_t)(a.f / 32) * scale_bytes(FMT);
  const MatPtr mats[1] = {
      {make_rsrc(a.image + ed.codes[2], a.d * cpitch), make_rsrc(a.image + ed.scales[2], a.d * spitch)}};
  const int P = geo.tpl, rw = a.rw_dn;
  const int units = rw / (R * geo.rpi) * P;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int waves = blockDim.x >> 6;
  const float A = code_gain(FMT);
  for (int c0 = 0; c0 < sc.ncols; c0 += G) {
    const int gc = (G == 2 && sc.ncols - c0 >= 2) ? 2 : 1;
    for (int u = wave; u < units; u += waves) {
      const UnitPos up = unit_pos(u, P, R, geo.rpi);
      if (gc == 2)
        down_unit<FMT, (G == 2 ? 2 : 1), R>(a, slot, c0, geo, up, blockIdx.x, mats, cpitch, spitch, op);
      else
        down_unit<FMT, 1, R>(a, slot, c0, geo, up, blockIdx.x, mats, cpitch, spitch, op);
    }
    __syncthreads();
    for (int it = threadIdx.x; it < gc * rw; it += blockDim.x) {
      const int ci = c0 + it / rw, row = it % rw;
      float o = 0.f;
      for (int pp = 0; pp < P; ++pp) o += op[(pp * kQMax + ci) * rw + row];
      a.part[((size_t)slot * a.q + ci) * a.d + blockIdx.x * rw + row] = sc.weight(ci) * (A * o);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ SlotCols slot_from_table(const RouteTable *rt, int slot) {
  SlotCols sc;
  sc.expert = uniform(rt->expert[slot]);
  sc.ncols = uniform(rt->ncols[slot]);
  sc.cols = rt->cols[slot];
  sc.w = rt->w[slot];
  return sc;
}

template <int G, int R>
__global__ __launch_bounds__(512) void k_down(ExpArgs a) {
  const int slot = blockIdx.y;
  if (slot >= uniform(a.rt->nslots)) return;
  extern __shared__ float op[];  // [2][kQMax][rw]
  const SlotCols sc = slot_from_table(a.rt, slot);
  const ExpertDesc ed = load_desc(a.image, sc.expert);
  const int fmt = ed.fmt[2];
  if (fmt == RFPX_FP2) down_tile<RFPX_FP2, G, R>(a, sc, slot, ed, op);
  else if (fmt == RFPX_FP3) down_tile<RFPX_FP3, G, R>(a, sc, slot, ed, op);
  else down_tile<RFPX_FP4, G, R>(a, sc, slot, ed, op);
}

// y[c][i] = sum over slots s that hold column c, in slot order, of the
// weighted partials.
__global__ __launch_bounds__(256) void k_combine(ExpArgs a) {
  const int it = blockIdx.x * blockDim.x + threadIdx.x;
  if (it >= a.q * a.d) return;
  const int c = it / a.d, row = it % a.d;
  const RouteTable *rt = a.rt;
  const int nslots = rt->nslots;
  float acc = 0.f;
  for (int s = 0; s < nslots; ++s) {
    const uint32_t m = rt->mask[s];
    if (!((m >> c) & 1u)) continue;
    const int ci = __popc(m & ((1u << c) - 1u));
    acc += a.part[((size_t)s * a.q + ci) * a.d + row];
  }
  a.y[it] = acc;
}

}  // namespace

hipError_t launch_experts(const ForwardPlan &p) {
  ExpArgs a{};
  a.image = p.image;
  a.rt = reinterpret_cast<RouteTable *>(p.ws + p.wl.route);
  a.rp = route_params(p);
  a.xp = reinterpret_cast<const uint32_t *>(p.ws + p.wl.xp);
  a.xnc = reinterpret_cast<const float *>(p.ws + p.wl.xnc);
  a.hp = reinterpret_cast<uint32_t *>(p.ws + p.wl.hp);
  a.hnc = reinterpret_cast<float *>(p.ws + p.wl.hnc);
  a.part = reinterpret_cast<float *>(p.ws + p.wl.part);
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
  const int slots = p.wl.max_slots;
  dim3 ggu(p.f / p.rw_gu, slots), gdn(p.d / p.rw_dn, slots);
  const size_t lds_gu = (size_t)5 * kQMax * p.rw_gu * sizeof(float);  // hs + gup
  const size_t lds_dn = (size_t)2 * kQMax * p.rw_dn * sizeof(float);  // op
  const bool bf = p.xtype == RFPX_X_BF16;
  hipEvent_t *ev = (hipEvent_t *)p.events;
  const unsigned nt = 64 * p.wmax;
  if (p.g == 1) {
    if (bf) k_gateup<1, 1, 4><<<ggu, nt, lds_gu, p.stream>>>(a);
    else k_gateup<1, 2, 4><<<ggu, nt, lds_gu, p.stream>>>(a);
  } else {
    if (bf) k_gateup<2, 1, 4><<<ggu, nt, lds_gu, p.stream>>>(a);
    else k_gateup<2, 2, 4><<<ggu, nt, lds_gu, p.stream>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[2], p.stream);
  if (e != hipSuccess) return e;
  if (p.g == 1) k_down<1, 4><<<gdn, nt, lds_dn, p.stream>>>(a);
  else k_down<2, 4><<<gdn, nt, lds_dn, p.stream>>>(a);
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[3], p.stream);
  if (e != hipSuccess) return e;
  k_combine<<<(p.q * p.d + 255) / 256, 256, 0, p.stream>>>(a);
  e = hipGetLastError();
  if (e == hipSuccess && ev) e = hipEventRecord(ev[4], p.stream);
  return e;
}

}  // namespace rfpx
