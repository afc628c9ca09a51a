// rfpx_route.hpp -- routing: the router scores of one expert row, and the
// in-workgroup routing step shared by k_topk and the routed gate/up kernel
// (sorted top-k per column, softmax gating, and the slot table of distinct
// experts over the q verify columns, all in LDS).
//
// Routing (page "APU 实现 token 自由…" (ainomam.com), section "Lucebox 的优
// 化三板斧": TOP-K/ARGSORT kernels on the routing path; page "Lucebox专攻
// DeepSeek V4…" (m.mzlw.cn), section "MoE 专家并行": top-6 of 256 plus one
// shared expert): ids = the k largest scores, score descending, ties to the
// lower expert index; w = routed_scale * softmax over the k chosen scores.
#pragma once

#include <math.h>

#include "rfpx_impl.hpp"

namespace rfpx {

struct RouteParams {
  const float *scores;  // [q][E]
  int E, k, q;
  float routed_scale;
};

inline RouteParams route_params(const ForwardPlan &p) {
  RouteParams r;
  r.scores = reinterpret_cast<const float *>(p.ws + p.wl.scores);
  r.E = p.E;
  r.k = p.k;
  r.q = p.q;
  r.routed_scale = p.routed_scale;
  return r;
}

struct RouteLds {
  int32_t ids[kQMax][kKMax];
  float gw[kQMax][kKMax];
  int32_t nslots;
  int32_t expert[kMaxSlots];
  int32_t ncols[kMaxSlots];
  uint32_t mask[kMaxSlots];
  int32_t cols[kMaxSlots][kQMax];
  float w[kMaxSlots][kQMax];
};

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Router scores s[c][e] = sum_i Wr[e][i] x[c][i] of one expert e for the Q
// columns, by one workgroup of NT threads: thread t takes float4 groups t,
// t + NT, ... of the row (d <= 4096), counted from a start that rotates
// with e (every workgroup reads the same x: with one start, all compute
// units of an L2 would ask for the same lines, channel by channel, at the
// same time).  Every load (the row and all Q columns of x) is issued before
// the arithmetic, with clamped indices and zeroed after, so no load waits
// on a branch or on another column's sums; the wave sums meet in LDS.  The
// activation type XT is a template argument: a run-time test around each
// load made the compiler wait for every load before issuing the next.
template <int NT, int Q, int XT>
__device__ __forceinline__ void router_row_q(const float *wr, const void *x, int d, int E,
                                             float *scores, int e) {
  constexpr int NPT = 4096 / 4 / NT;
  const int tid = threadIdx.x;
  const int n4 = d / 4;
  // workgroups e, e + 8, ... share an L2 (the XCDs take workgroups in turn)
  const int rot = (64 * (e >> 3)) % n4;
  int idx[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i4 = min(tid + NT * j, n4 - 1);  // w is zeroed past n4
    idx[j] = i4 + rot < n4 ? i4 + rot : i4 + rot - n4;
  }
  const float4 *wrow = reinterpret_cast<const float4 *>(wr + (size_t)e * d);
  float4 w[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) w[j] = wrow[idx[j]];
  float4 xv[Q][NPT];
#pragma unroll
  for (int c = 0; c < Q; ++c)
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i4 = idx[j];
      if constexpr (XT == RFPX_X_BF16) {
        const uint2 b = reinterpret_cast<const uint2 *>(
            static_cast<const uint16_t *>(x) + (size_t)c * d)[i4];
        xv[c][j] = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                               __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
      } else {
        xv[c][j] = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (size_t)c * d)[i4];
      }
    }
#pragma unroll
  for (int j = 0; j < NPT; ++j)
    if (tid + NT * j >= n4) w[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  float acc[Q];
#pragma unroll
  for (int c = 0; c < Q; ++c) {
    acc[c] = 0.f;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      acc[c] = fmaf(w[j].x, xv[c][j].x, acc[c]);
      acc[c] = fmaf(w[j].y, xv[c][j].y, acc[c]);
      acc[c] = fmaf(w[j].z, xv[c][j].z, acc[c]);
      acc[c] = fmaf(w[j].w, xv[c][j].w, acc[c]);
    }
  }
  __shared__ float part[NT / 64][Q];
  const int lane = tid & 63, wave = tid >> 6;
  // all columns' wave sums at once (DPP halving steps, multi_sum, over a
  // power-of-two count of values: zeros pad the columns past Q)
  constexpr int QP = Q == 1 ? 1 : Q == 2 ? 2 : Q <= 4 ? 4 : 8;
  float accp[QP];
#pragma unroll
  for (int c = 0; c < QP; ++c) accp[c] = c < Q ? acc[c] : 0.f;
  const float r = multi_sum<QP>(accp, lane);
  if (ms_writer<QP>(lane) && ms_index<QP>(lane) < Q) part[wave][ms_index<QP>(lane)] = r;
  __syncthreads();
  if (tid < Q) {
    float s = 0.f;
    for (int wv = 0; wv < NT / 64; ++wv) s += part[wv][tid];
    scores[(size_t)tid * E + e] = s;
  }
}

// router_row_q for a run-time column count q = 1..kQMax and activation type.
template <int NT, int XT>
__device__ __forceinline__ void router_row_x(const float *wr, const void *x, int d, int E, int q,
                                             float *scores, int e) {
  static_assert(kQMax == 8, "one case per column count");
  switch (q) {
    case 1: router_row_q<NT, 1, XT>(wr, x, d, E, scores, e); break;
    case 2: router_row_q<NT, 2, XT>(wr, x, d, E, scores, e); break;
    case 3: router_row_q<NT, 3, XT>(wr, x, d, E, scores, e); break;
    case 4: router_row_q<NT, 4, XT>(wr, x, d, E, scores, e); break;
    case 5: router_row_q<NT, 5, XT>(wr, x, d, E, scores, e); break;
    case 6: router_row_q<NT, 6, XT>(wr, x, d, E, scores, e); break;
    case 7: router_row_q<NT, 7, XT>(wr, x, d, E, scores, e); break;
    default: router_row_q<NT, 8, XT>(wr, x, d, E, scores, e); break;
  }
}

template <int NT>
__device__ __forceinline__ void router_row(const float *wr, const void *x, int xtype, int d,
                                           int E, int q, float *scores, int e) {
  if (xtype == RFPX_X_BF16) router_row_x<NT, RFPX_X_BF16>(wr, x, d, E, q, scores, e);
  else router_row_x<NT, RFPX_X_F32>(wr, x, d, E, q, scores, e);
}

// Order-preserving key of an fp32 score: larger score <=> larger key
// (-0 is folded into +0 first so that the two compare equal, as floats do).
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t dpp_max(uint32_t v, uint32_t w) { return v > w ? v : w; }

// Maximum over the wave, returned in a scalar register: butterfly inside
// each row of 16 lanes with DPP (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror), then the four row results via v_readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = dpp_max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return dpp_max(dpp_max(r0, r1), dpp_max(r2, r3));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
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

// Sorted top-k of column c and its gating weights, by one wave; lane l
// holds experts l, l+64, ... (P of them, E <= 64 P).  Each lane first sorts
// its own keys (score descending, index ascending: a compare-exchange
// network on static indices), so that every round only looks at the lanes'
// heads: the wave maximum of the heads (DPP), the lowest expert index among
// the lanes holding it (one lane in all but exact ties), and that lane
// drops its head.  Lane r < k keeps the r-th expert and score; the softmax
// over the k scores is lane-parallel.  Writes s_ids[0..k) and s_w[0..k).
template <int P>
__device__ __forceinline__ void topk_wave(const RouteParams &rp, int c, int lane,
                                          int32_t *s_ids, float *s_w) {
  uint32_t key[P];
  int idx[P];
  float sv[P];
  // unconditional loads (clamped index) so that all of them are in flight
  // together; entries past E get the key 0, below every real key
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int e = lane + 64 * i;
    sv[i] = rp.scores[(size_t)c * rp.E + (e < rp.E ? e : rp.E - 1)];
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    idx[i] = lane + 64 * i;
    key[i] = idx[i] < rp.E ? score_key(sv[i]) : 0u;
  }
  // insertion network: after it key[0] >= key[1] >= ...; equal keys keep
  // their index order (the swap is strict)
#pragma unroll
  for (int i = 1; i < P; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1];
      const uint32_t ka = key[j - 1], kb = key[j];
      const int ia = idx[j - 1], ib = idx[j];
      key[j - 1] = sw ? kb : ka;
      key[j] = sw ? ka : kb;
      idx[j - 1] = sw ? ib : ia;
      idx[j] = sw ? ia : ib;
    }
  int my_id = 0;
  float my_val = 0.f;
  for (int r = 0; r < rp.k; ++r) {
    const uint32_t kmax = wave_max_u32(key[0]);
    const uint64_t cand = __ballot(key[0] == kmax);
    int best = __builtin_amdgcn_readlane(idx[0], (int)__builtin_ctzll(cand));
    if (cand & (cand - 1ull)) {  // exact tie between lanes: lowest index
      uint64_t m = cand;
      while (m) {
        const int v = __builtin_amdgcn_readlane(idx[0], (int)__builtin_ctzll(m));
        best = v < best ? v : best;
        m &= m - 1ull;
      }
    }
    if (lane == (best & 63)) {  // the winner drops its head
#pragma unroll
      for (int i = 0; i + 1 < P; ++i) {
        key[i] = key[i + 1];
        idx[i] = idx[i + 1];
      }
      key[P - 1] = 0u;
    }
    const uint32_t u = (kmax & 0x80000000u) ? (kmax & 0x7FFFFFFFu) : ~kmax;
    if (lane == r) {
      my_id = best;
      my_val = __uint_as_float(u);
    }
  }
  // softmax over the k chosen scores, relative to the largest (lane 0)
  const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_val), 0));
  const float e = lane < rp.k ? expf(my_val - v0) : 0.f;
  const float z = wave_sum_dpp(e);
  if (lane < rp.k) {
    s_ids[lane] = my_id;
    s_w[lane] = e / z * rp.routed_scale;
  }
}

// Sorted top-k and gating of column c by one wave (dispatch on E).
__device__ __forceinline__ void topk_column(const RouteParams &rp, int c, int lane,
                                            int32_t *s_ids, float *s_w) {
  const int E = rp.E;
  if (E <= 64) topk_wave<1>(rp, c, lane, s_ids, s_w);
  else if (E <= 128) topk_wave<2>(rp, c, lane, s_ids, s_w);
  else if (E <= 256) topk_wave<4>(rp, c, lane, s_ids, s_w);
  else if (E <= 512) topk_wave<8>(rp, c, lane, s_ids, s_w);
  else topk_wave<16>(rp, c, lane, s_ids, s_w);
}

// The routing step of a one-column step, for the workgroup of slot `slot`:
// the k chosen experts are distinct, so slot s (1..k) is rank s - 1 and
// there is nothing to deduplicate.  Fills the header fields, slot 0 and
// the workgroup's own slot of the LDS table, exactly as route_wg would.
// Ends with a barrier.
__device__ __forceinline__ void route_q1(const RouteParams &rp, RouteLds *s, int slot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) topk_column(rp, 0, lane, s->ids[0], s->gw[0]);
  __syncthreads();
  if (threadIdx.x == 0) {
    s->nslots = rp.k + 1;
    s->expert[0] = rp.E;
    s->ncols[0] = 1;
    s->mask[0] = 1u;
    s->cols[0][0] = 0;
    s->w[0][0] = 1.0f;
    if (slot >= 1 && slot <= rp.k) {
      s->expert[slot] = s->ids[0][slot - 1];
      s->ncols[slot] = 1;
      s->mask[slot] = 1u;
      s->cols[slot][0] = 0;
      s->w[slot][0] = s->gw[0][slot - 1];
    }
  }
  __syncthreads();
}

// Whole-workgroup routing into LDS; needs blockDim.x >= 64 * q and LDS
// scratch of 2 E words.  Ends with a barrier, so every thread may read the
// table afterwards.
//
// The q k entries (lane i of wave 0: column i / k, rank i % k) become one
// slot per distinct expert, in order of first appearance, all lanes at
// once: per expert, the lowest lane holding it (LDS atomic minimum) and the
// set of columns that chose it (LDS atomic or).  A lane that is its
// expert's first takes slot 1 + (number of first lanes below it); the
// others read their first lane's slot.  A column picks an expert at most
// once, so an entry's position in its slot is the number of the expert's
// columns below its own, and the slot's columns ascend.
__device__ __forceinline__ void route_wg(const RouteParams &rp, RouteLds *s, uint32_t *scr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < rp.q) topk_column(rp, wave, lane, s->ids[wave], s->gw[wave]);
  __syncthreads();
  if (wave == 0) {
    uint32_t *first = scr, *cmask = scr + rp.E;
    const int n = rp.q * rp.k;
    const bool act = lane < n;
    int e = 0, c = 0;
    float w = 0.f;
    if (act) {
      c = lane / rp.k;
      e = s->ids[c][lane % rp.k];
      w = s->gw[c][lane % rp.k];
      first[e] = 64u;
      cmask[e] = 0u;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    if (act) {
      atomicMin(&first[e], (uint32_t)lane);
      atomicOr(&cmask[e], 1u << c);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    __builtin_amdgcn_wave_barrier();
    int f = lane;
    uint32_t cm = 0;
    if (act) {
      f = (int)first[e];
      cm = cmask[e];
    }
    const uint64_t firsts = __ballot(act && f == lane);
    const int own = 1 + __popcll(firsts & ((1ull << lane) - 1ull));
    const int slot = __shfl(own, f, 64);
    if (act) {
      const int pos = __popc(cm & ((1u << c) - 1u));
      s->cols[slot][pos] = c;
      s->w[slot][pos] = w;
      if (f == lane) {
        s->expert[slot] = e;
        s->ncols[slot] = __popc(cm);
        s->mask[slot] = cm;
      }
    }
    if (lane == 0) {
      s->nslots = 1 + __popcll(firsts);
      s->expert[0] = rp.E;  // the shared expert takes every column
      s->ncols[0] = rp.q;
      s->mask[0] = (1u << rp.q) - 1u;
    }
    if (lane < rp.q) {
      s->cols[0][lane] = lane;
      s->w[0][lane] = 1.0f;
    }
  }
  __syncthreads();
}

// The down-matrix entry of expert e's table row into slot `slot` of the
// workspace table.
__device__ __forceinline__ void publish_down_desc(const uint8_t *image, int e, int slot,
                                                  RouteTable *rt) {
  const ExpertDesc *t = reinterpret_cast<const ExpertDesc *>(image + kImgTable) + e;
  rt->dn_codes[slot] = t->codes[2];
  rt->dn_scales[slot] = t->scales[2];
  rt->dn_fmt[slot] = t->fmt[2];
}

// Copy slot `slot` of the LDS table to the workspace table (slot < 0: all
// slots); with `header`, also the slot count, ids and gating weights.
__device__ __forceinline__ void publish_route(const RouteLds &s, int q, int slot,
                                              bool header, RouteTable *rt) {
  const int tid = threadIdx.x;
  const int s0 = slot < 0 ? 0 : slot, s1 = slot < 0 ? s.nslots : slot + 1;
  for (int i = tid; i < (s1 - s0) * (kQMax + 1); i += blockDim.x) {
    const int sl = s0 + i / (kQMax + 1), j = i % (kQMax + 1);
    if (j == kQMax) {
      rt->expert[sl] = s.expert[sl];
      rt->ncols[sl] = s.ncols[sl];
      rt->mask[sl] = s.mask[sl];
    } else {
      rt->cols[sl][j] = s.cols[sl][j];
      rt->w[sl][j] = s.w[sl][j];
    }
  }
  if (!header) return;
  for (int i = tid; i < kQMax * kKMax; i += blockDim.x) {
    rt->ids[i / kKMax][i % kKMax] = s.ids[i / kKMax][i % kKMax];
    rt->gw[i / kKMax][i % kKMax] = s.gw[i / kKMax][i % kKMax];
  }
  if (tid == 0) rt->nslots = s.nslots;
  if (slot >= 0)  // the shared slot, which no routed workgroup owns
    for (int i = tid; i < kQMax + 1; i += blockDim.x) {
      if (i == kQMax) {
        rt->expert[0] = s.expert[0];
        rt->ncols[0] = s.ncols[0];
        rt->mask[0] = s.mask[0];
      } else {
        rt->cols[0][i] = s.cols[0][i];
        rt->w[0][i] = s.w[0][i];
      }
    }
  (void)q;
}

#endif  // device side

}  // namespace rfpx
