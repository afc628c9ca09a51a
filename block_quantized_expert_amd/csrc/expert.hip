// expert.hip -- expert-grouped dequantize-and-GEMV for the routed and the
// shared experts, decode path.
//
// Page "APU 实现 token 自由…" (ainomam.com), section "Lucebox 的优化三板斧":
// in the q-column verify path each packed weight is decoded once and applied
// to every verify column.  Page "Lucebox专攻DeepSeek V4…" (m.mzlw.cn),
// section "常见疑问" (FAQ): decode is bound by memory bandwidth.
//
// Two launches after the router (route.hip):
//   k_gateup  grid (f / RW, slots).  A workgroup owns RW consecutive rows of
//             the gate and up matrices of one slot's expert; each wave owns
//             R rows of both, issues every code and scale load for them up
//             front, decodes each block in registers once and applies it to
//             all of the slot's columns (v_dot2c_f32_bf16 on the prepared
//             activations), reduces each row across its lanes, and forms
//             h = silu(g) * u.  The workgroup then prepares h (bf16 hi + lo
//             pair words for the down matrix's format) for the down kernel.
//   k_down    grid (d / RW, slots).  Same structure over the down matrix;
//             each row result is multiplied by the column's gating weight
//             and stored as a partial; the last workgroup to finish a row
//             tile (device-scope counter) sums the partials of all slots in
//             slot order and writes y -- deterministic, no float atomics.
// Lane geometry (Geo): with a row of >= 64 chunks a wave covers one row per
// step and lane l reads chunks l and l+64 (fully coalesced 1 KiB requests);
// shorter rows give each wave 64/cpl rows per step.
#include "rfpx_impl.hpp"

namespace rfpx {
namespace {

struct ExpArgs {
  const uint8_t *image;
  const RouteTable *rt;
  const uint32_t *xp;
  const float *xnc;
  uint32_t *hp;
  float *hnc;
  float *part;
  float *y;
  int *counters;
  int d, f, q, nb_d, nb_f;
  int rw_gu, rw_dn;
  Geo geo_gu[5], geo_dn[5];
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

// Per-lane partial dot products of R rows of NM matrices with G columns.
// Row i of matrix m is read through the matrix planes' buffer resources at
// scalar offset (row_u + rpi*i) * pitch, row_u wave-uniform, plus the lane's
// own offset (row group and chunk).  All code
// and scale loads are issued first; then rows are decoded and reduced one
// at a time (scheduling fences keep the decode of one row from being
// hoisted over the next, which would multiply register pressure).
struct MatPtr {
  __amdgpu_buffer_rsrc_t codes;
  __amdgpu_buffer_rsrc_t scales;
};

template <int FMT, int TPL, int G, int VX, int NM, int R>
__device__ __forceinline__ void mat_rows(const MatPtr (&mats)[NM], size_t cpitch,
                                size_t spitch, int row_u, int rpi,
                                const uint32_t (&coff)[TPL],
                                const uint32_t (&soff)[TPL],
                                const uint32_t (&xr)[G][TPL * Fmt<FMT>::CB][VX][16],
                                const float (&ncr)[G][TPL * Fmt<FMT>::CB],
                                float (&tot)[R][NM][G]) {
  using F = Fmt<FMT>;
  uint32_t cw[R][NM][TPL][F::CW];
  uint32_t sw[R][NM][TPL];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t row = (uint32_t)(row_u + rpi * i);
    const uint32_t cs = row * (uint32_t)cpitch, ss = row * (uint32_t)spitch;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int t = 0; t < TPL; ++t) {
        load_chunk<FMT>(mats[m].codes, coff[t], cs, cw[i][m][t]);
        sw[i][m][t] = load_scale<FMT>(mats[m].scales, soff[t], ss);
      }
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
      for (int t = 0; t < TPL; ++t) {
#pragma unroll
        for (int j = 0; j < F::CB; ++j) {
          uint32_t pr[16];
          decode_pairs<FMT>(&cw[i][m][t][j * F::BW], pr);
          const float s = block_scale<FMT>(block_scale_bits<FMT>(sw[i][m][t], j));
          const int b = t * F::CB + j;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = ncr[g][b];
#pragma unroll
            for (int v = 0; v < VX; ++v)
#pragma unroll
              for (int p = 0; p < 16; ++p) acc = dot2(pr[p], xr[g][b][v][p], acc);
            tot[i][m][g] = fmaf(acc, s, tot[i][m][g]);
          }
        }
      }
    }
  }
}

// Load prepared activations (or prepared h) of the lane's blocks for the
// columns c0 .. c0+gcount-1 of `base`: block b of column c sits at
// ((c * nb) + b) * VX * 16 words, its accumulator start at c * nb + b.
template <int FMT, int TPL, int G, int VX>
__device__ __forceinline__ void load_prepared(const uint32_t *__restrict__ pw,
                                     const float *__restrict__ pnc, int nb,
                                     const int *colidx, int li, int lpr,
                                     uint32_t (&xr)[G][TPL * Fmt<FMT>::CB][VX][16],
                                     float (&ncr)[G][TPL * Fmt<FMT>::CB]) {
  using F = Fmt<FMT>;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int c = colidx[g];
#pragma unroll
    for (int t = 0; t < TPL; ++t)
#pragma unroll
      for (int j = 0; j < F::CB; ++j) {
        const int blk = (li + lpr * t) * F::CB + j;
        const size_t item = (size_t)c * nb + blk;
        const uint4 *src = reinterpret_cast<const uint4 *>(pw + item * VX * 16);
#pragma unroll
        for (int v = 0; v < VX; ++v)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            uint4 q4 = src[v * 4 + u];
            xr[g][t * F::CB + j][v][4 * u + 0] = q4.x;
            xr[g][t * F::CB + j][v][4 * u + 1] = q4.y;
            xr[g][t * F::CB + j][v][4 * u + 2] = q4.z;
            xr[g][t * F::CB + j][v][4 * u + 3] = q4.w;
          }
        ncr[g][t * F::CB + j] = pnc[item];
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

__device__ __forceinline__ float group_sum(float v, int lpr) {
  for (int off = lpr >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ------------------------------------------------------------ gate / up

template <int FMT_DN>
__device__ __forceinline__ void prep_h_block(const float *hs, uint32_t *dst, float *nc) {
  uint32_t hi[32], lo[32], pw[16];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float v = hs[j];
    hi[j] = float_to_bf16_rne(v);
    lo[j] = float_to_bf16_rne(v - bf16_bits_to_float(hi[j]));
  }
  float nch, ncl;
  prep_pairs<FMT_DN>(hi, pw, &nch);
#pragma unroll
  for (int p = 0; p < 16; ++p) dst[p] = pw[p];
  prep_pairs<FMT_DN>(lo, pw, &ncl);
#pragma unroll
  for (int p = 0; p < 16; ++p) dst[16 + p] = pw[p];
  *nc = nch + ncl;
}

// Lane/row geometry of one wave inside a workgroup tile.
struct WaveRows {
  int rg, li, rloc_u, row_u;
  uint32_t coff[2], soff[2];
};

template <int FMT, int TPL>
__device__ __forceinline__ bool wave_rows(const Geo &geo, int rw, int r, size_t cpitch,
                                 size_t spitch, WaveRows *w) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave >= rw / (geo.rpi * r)) return false;
  w->rg = lane / geo.lpr;
  w->li = lane % geo.lpr;
  w->rloc_u = wave * geo.rpi * r;
  w->row_u = blockIdx.x * rw + w->rloc_u;
#pragma unroll
  for (int t = 0; t < TPL; ++t) {
    w->coff[t] = (uint32_t)(w->rg * cpitch + (size_t)(w->li + geo.lpr * t) * F::CBYTES);
    w->soff[t] = (uint32_t)(w->rg * spitch + (size_t)(w->li + geo.lpr * t) * F::SBYTES);
  }
  return true;
}

// One pass of GP columns (c0 .. c0+GP-1 of the slot) over the wave's rows.
template <int FMT, int TPL, int GP, int VX, int R>
__device__ __forceinline__ void gateup_pass(const ExpArgs &a, int slot, int c0,
                                   const Geo &geo, const WaveRows &wr,
                                   const MatPtr (&mats)[2], size_t cpitch,
                                   size_t spitch, float *hs) {
  using F = Fmt<FMT>;
  const uint32_t *xpf = a.xp + (size_t)(FMT - RFPX_FP2) * a.q * a.nb_d * VX * 16;
  const float *xncf = a.xnc + (size_t)(FMT - RFPX_FP2) * a.q * a.nb_d;
  int colidx[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) colidx[g] = uniform(a.rt->cols[slot][c0 + g]);
  uint32_t xr[GP][TPL * F::CB][VX][16];
  float ncr[GP][TPL * F::CB];
  load_prepared<FMT, TPL, GP, VX>(xpf, xncf, a.nb_d, colidx, wr.li, geo.lpr, xr, ncr);
  __builtin_amdgcn_sched_barrier(0);  // activation loads go out before the weights
  float tot[R][2][GP];
  uint32_t coff[TPL], soff[TPL];
#pragma unroll
  for (int t = 0; t < TPL; ++t) {
    coff[t] = wr.coff[t];
    soff[t] = wr.soff[t];
  }
  mat_rows<FMT, TPL, GP, VX, 2, R>(mats, cpitch, spitch, wr.row_u, geo.rpi, coff, soff,
                                   xr, ncr, tot);
  const float A = code_gain(FMT);
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float gv = A * group_sum(tot[i][0][g], geo.lpr);
      float uv = A * group_sum(tot[i][1][g], geo.lpr);
      if (wr.li == 0)
        hs[(c0 + g) * a.rw_gu + wr.rloc_u + wr.rg + geo.rpi * i] = silu(gv) * uv;
    }
}

template <int FMT, int TPL, int G, int VX, int R>
__device__ __forceinline__ void gateup_body(const ExpArgs &a, int slot, const ExpertDesc &ed,
                            float *hs /* [kQMax][rw] */) {
  const Geo geo = a.geo_gu[FMT];
  const size_t cpitch = (size_t)(a.d / 32) * code_bytes(FMT);
  const size_t spitch = (size_t)(a.d / 32) * scale_bytes(FMT);
  WaveRows wr;
  if (!wave_rows<FMT, TPL>(geo, a.rw_gu, R, cpitch, spitch, &wr)) return;
  const uint32_t cbytes = (uint32_t)(a.f * cpitch), sbytes = (uint32_t)(a.f * spitch);
  const MatPtr mats[2] = {
      {make_rsrc(a.image + ed.codes[0], cbytes), make_rsrc(a.image + ed.scales[0], sbytes)},
      {make_rsrc(a.image + ed.codes[1], cbytes), make_rsrc(a.image + ed.scales[1], sbytes)}};
  const int ncols = uniform(a.rt->ncols[slot]);
  for (int c0 = 0; c0 < ncols; c0 += G) {
    if (G == 2 && ncols - c0 >= 2)
      gateup_pass<FMT, TPL, (G == 2 ? 2 : 1), VX, R>(a, slot, c0, geo, wr, mats, cpitch, spitch, hs);
    else
      gateup_pass<FMT, TPL, 1, VX, R>(a, slot, c0, geo, wr, mats, cpitch, spitch, hs);
  }
}

template <int G, int VX, int R>
__global__ __launch_bounds__(512) void k_gateup(ExpArgs a) {
  const int slot = blockIdx.y;
  const RouteTable *rt = a.rt;
  if (slot >= uniform(rt->nslots)) return;
  const ExpertDesc ed = load_desc(a.image, uniform(rt->expert[slot]));
  extern __shared__ float hs[];  // [kQMax][rw_gu]
  const int fmt = ed.fmt[0];
  const int tpl = a.geo_gu[fmt].tpl;
  if (fmt == RFPX_FP2) {
    if (tpl == 1) gateup_body<RFPX_FP2, 1, G, VX, R>(a, slot, ed, hs);
    else gateup_body<RFPX_FP2, 2, G, VX, R>(a, slot, ed, hs);
  } else if (fmt == RFPX_FP3) {
    if (tpl == 1) gateup_body<RFPX_FP3, 1, G, VX, R>(a, slot, ed, hs);
    else gateup_body<RFPX_FP3, 2, G, VX, R>(a, slot, ed, hs);
  } else {
    if (tpl == 1) gateup_body<RFPX_FP4, 1, G, VX, R>(a, slot, ed, hs);
    else gateup_body<RFPX_FP4, 2, G, VX, R>(a, slot, ed, hs);
  }
  __syncthreads();
  // prepare h of this tile for the down matrix: one item per (column, block)
  const int ncols = rt->ncols[slot];
  const int nbt = a.rw_gu / 32;
  const int fdn = ed.fmt[2];
  for (int it = threadIdx.x; it < ncols * nbt; it += blockDim.x) {
    const int ci = it / nbt, bt = it % nbt;
    const int blk = blockIdx.x * nbt + bt;
    const size_t item = ((size_t)slot * a.q + ci) * a.nb_f + blk;
    const float *src = hs + ci * a.rw_gu + 32 * bt;
    uint32_t *dst = a.hp + item * 32;
    float *nc = a.hnc + item;
    if (fdn == RFPX_FP2) prep_h_block<RFPX_FP2>(src, dst, nc);
    else if (fdn == RFPX_FP3) prep_h_block<RFPX_FP3>(src, dst, nc);
    else prep_h_block<RFPX_FP4>(src, dst, nc);
  }
}

// ----------------------------------------------------------------- down

template <int FMT, int TPL, int GP, int R>
__device__ __forceinline__ void down_pass(const ExpArgs &a, int slot, int c0,
                                 const Geo &geo, const WaveRows &wr,
                                 const MatPtr (&mats)[1], size_t cpitch,
                                 size_t spitch) {
  using F = Fmt<FMT>;
  const uint32_t *hps = a.hp + (size_t)slot * a.q * a.nb_f * 32;
  const float *hncs = a.hnc + (size_t)slot * a.q * a.nb_f;
  int colidx[GP];
#pragma unroll
  for (int g = 0; g < GP; ++g) colidx[g] = c0 + g;  // compact column index
  uint32_t xr[GP][TPL * F::CB][2][16];
  float ncr[GP][TPL * F::CB];
  load_prepared<FMT, TPL, GP, 2>(hps, hncs, a.nb_f, colidx, wr.li, geo.lpr, xr, ncr);
  __builtin_amdgcn_sched_barrier(0);  // h loads go out before the weights
  float to[R][1][GP];
  uint32_t coff[TPL], soff[TPL];
#pragma unroll
  for (int t = 0; t < TPL; ++t) {
    coff[t] = wr.coff[t];
    soff[t] = wr.soff[t];
  }
  mat_rows<FMT, TPL, GP, 2, 1, R>(mats, cpitch, spitch, wr.row_u, geo.rpi, coff, soff,
                                  xr, ncr, to);
  const float A = code_gain(FMT);
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int g = 0; g < GP; ++g) {
      float o = A * group_sum(to[i][0][g], geo.lpr);
      if (wr.li == 0) {
        const int ci = c0 + g;
        a.part[((size_t)slot * a.q + ci) * a.d + wr.row_u + wr.rg + geo.rpi * i] =
            a.rt->w[slot][ci] * o;
      }
    }
}

template <int FMT, int TPL, int G, int R>
__device__ __forceinline__ void down_body(const ExpArgs &a, int slot, const ExpertDesc &ed) {
  const Geo geo = a.geo_dn[FMT];
  const size_t cpitch = (size_t)(a.f / 32) * code_bytes(FMT);
  const size_t spitch = (size_t)(a.f / 32) * scale_bytes(FMT);
  WaveRows wr;
  if (!wave_rows<FMT, TPL>(geo, a.rw_dn, R, cpitch, spitch, &wr)) return;
  const MatPtr mats[1] = {
      {make_rsrc(a.image + ed.codes[2], (uint32_t)(a.d * cpitch)),
       make_rsrc(a.image + ed.scales[2], (uint32_t)(a.d * spitch))}};
  const int ncols = uniform(a.rt->ncols[slot]);
  for (int c0 = 0; c0 < ncols; c0 += G) {
    if (G == 2 && ncols - c0 >= 2)
      down_pass<FMT, TPL, (G == 2 ? 2 : 1), R>(a, slot, c0, geo, wr, mats, cpitch, spitch);
    else
      down_pass<FMT, TPL, 1, R>(a, slot, c0, geo, wr, mats, cpitch, spitch);
  }
}

template <int G, int R>
__global__ __launch_bounds__(512) void k_down(ExpArgs a) {
  const int slot = blockIdx.y;
  const RouteTable *rt = a.rt;
  const int nslots = uniform(rt->nslots);
  if (slot >= nslots) return;
  const ExpertDesc ed = load_desc(a.image, uniform(rt->expert[slot]));
  const int fmt = ed.fmt[2];
  const int tpl = a.geo_dn[fmt].tpl;
  if (fmt == RFPX_FP2) {
    if (tpl == 1) down_body<RFPX_FP2, 1, G, R>(a, slot, ed);
    else down_body<RFPX_FP2, 2, G, R>(a, slot, ed);
  } else if (fmt == RFPX_FP3) {
    if (tpl == 1) down_body<RFPX_FP3, 1, G, R>(a, slot, ed);
    else down_body<RFPX_FP3, 2, G, R>(a, slot, ed);
  } else {
    if (tpl == 1) down_body<RFPX_FP4, 1, G, R>(a, slot, ed);
    else down_body<RFPX_FP4, 2, G, R>(a, slot, ed);
  }
  // ---- last workgroup of this row tile sums the slots in slot order
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = __hip_atomic_fetch_add(&a.counters[1 + blockIdx.x], 1,
                                      __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == nslots - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int it = threadIdx.x; it < a.q * a.rw_dn; it += blockDim.x) {
    const int c = it / a.rw_dn;
    const int row = blockIdx.x * a.rw_dn + it % a.rw_dn;
    float acc = 0.f;
    for (int s = 0; s < nslots; ++s) {
      const uint32_t m = rt->mask[s];
      if (!((m >> c) & 1u)) continue;
      const int ci = __popc(m & ((1u << c) - 1u));
      acc += a.part[((size_t)s * a.q + ci) * a.d + row];
    }
    a.y[(size_t)c * a.d + row] = acc;
  }
}

}  // namespace

hipError_t launch_experts(const ForwardPlan &p) {
  ExpArgs a{};
  a.image = p.image;
  a.rt = reinterpret_cast<const RouteTable *>(p.ws + p.wl.route);
  a.xp = reinterpret_cast<const uint32_t *>(p.ws + p.wl.xp);
  a.xnc = reinterpret_cast<const float *>(p.ws + p.wl.xnc);
  a.hp = reinterpret_cast<uint32_t *>(p.ws + p.wl.hp);
  a.hnc = reinterpret_cast<float *>(p.ws + p.wl.hnc);
  a.part = reinterpret_cast<float *>(p.ws + p.wl.part);
  a.y = p.y;
  a.counters = reinterpret_cast<int *>(p.ws + p.wl.counters);
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
  const size_t lds = (size_t)kQMax * p.rw_gu * sizeof(float);
  const bool bf = p.xtype == RFPX_X_BF16;
  if (p.g == 1) {
    if (bf) k_gateup<1, 1, 4><<<ggu, 64 * p.wmax, lds, p.stream>>>(a);
    else k_gateup<1, 2, 4><<<ggu, 64 * p.wmax, lds, p.stream>>>(a);
    k_down<1, 4><<<gdn, 64 * p.wmax, 0, p.stream>>>(a);
  } else {
    if (bf) k_gateup<2, 1, 4><<<ggu, 64 * p.wmax, lds, p.stream>>>(a);
    else k_gateup<2, 2, 4><<<ggu, 64 * p.wmax, lds, p.stream>>>(a);
    k_down<2, 4><<<gdn, 64 * p.wmax, 0, p.stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace rfpx
