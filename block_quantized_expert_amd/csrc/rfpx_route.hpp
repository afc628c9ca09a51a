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

// Router scores s[c][e] = sum_i Wr[e][i] x[c][i] of one expert e for the q
// columns, by one workgroup of NT threads: thread t takes float4 groups t,
// t + NT, ... of the row (d <= 4096), all loads issued before the
// arithmetic (clamped indices, zeroed after, so no load waits on a branch);
// the wave sums meet in LDS.
template <int NT>
__device__ __forceinline__ void router_row(const float *wr, const void *x, int xtype, int d,
                                           int E, int q, float *scores, int e) {
  constexpr int NPT = 4096 / 4 / NT;
  const int tid = threadIdx.x;
  const int n4 = d / 4;
  const float4 *wrow = reinterpret_cast<const float4 *>(wr + (size_t)e * d);
  float4 w[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i4 = tid + NT * j;
    w[j] = wrow[i4 < n4 ? i4 : n4 - 1];
  }
#pragma unroll
  for (int j = 0; j < NPT; ++j)
    if (tid + NT * j >= n4) w[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  float acc[kQMax];
#pragma unroll
  for (int c = 0; c < kQMax; ++c) {
    acc[c] = 0.f;
    if (c >= q) continue;
    float4 xv[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i4 = min(tid + NT * j, n4 - 1);  // w is zero past n4
      if (xtype == RFPX_X_BF16) {
        const uint2 b = reinterpret_cast<const uint2 *>(
            static_cast<const uint16_t *>(x) + (size_t)c * d)[i4];
        xv[j] = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xFFFF0000u),
                            __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xFFFF0000u));
      } else {
        xv[j] = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + (size_t)c * d)[i4];
      }
    }
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      acc[c] = fmaf(w[j].x, xv[j].x, acc[c]);
      acc[c] = fmaf(w[j].y, xv[j].y, acc[c]);
      acc[c] = fmaf(w[j].z, xv[j].z, acc[c]);
      acc[c] = fmaf(w[j].w, xv[j].w, acc[c]);
    }
  }
  __shared__ float part[NT / 64][kQMax];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int c = 0; c < kQMax; ++c) {
    if (c >= q) break;
    const float s = wave_sum_f32(acc[c]);
    if (lane == 0) part[wave][c] = s;
  }
  __syncthreads();
  if (tid < q) {
    float s = 0.f;
    for (int wv = 0; wv < NT / 64; ++wv) s += part[wv][tid];
    scores[(size_t)tid * E + e] = s;
  }
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

// k rounds of a wave-wide arg-max over (score descending, index ascending)
// for column c; lane l holds experts l, l+64, ...  Each round: every lane
// offers its best untaken expert, the wave maximum of the keys is found
// with DPP, and among the lanes offering it the lowest expert index wins
// (one lane in all but exact ties).
__device__ __forceinline__ void topk_wave(const RouteParams &rp, int c, int lane,
                                          int32_t *ids, float *vals) {
  constexpr int PER = kEMax / 64;
  uint32_t key[PER];
  float sv[PER];
  // unconditional loads (clamped index) so that all of them are in flight
  // together; entries past E get the key 0, below every real key
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    sv[i] = rp.scores[(size_t)c * rp.E + (e < rp.E ? e : rp.E - 1)];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = (lane + 64 * i < rp.E) ? score_key(sv[i]) : 0u;
  for (int r = 0; r < rp.k; ++r) {
    uint32_t kb = 0u;
    int ib = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (64 * i >= rp.E) break;
      if (key[i] > kb) {  // strict: the lower i (lower index) keeps a tie
        kb = key[i];
        ib = lane + 64 * i;
      }
    }
    const uint32_t kmax = wave_max_u32(kb);
    const uint64_t cand = __ballot(kb == kmax);
    int best = __builtin_amdgcn_readlane(ib, (int)__builtin_ctzll(cand));
    if (cand & (cand - 1ull)) {  // exact tie between lanes: lowest index
      uint64_t m = cand;
      while (m) {
        const int l = (int)__builtin_ctzll(m);
        const int v = __builtin_amdgcn_readlane(ib, l);
        best = v < best ? v : best;
        m &= m - 1ull;
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)  // taken (static indices: no scratch)
      if (best == lane + 64 * i) key[i] = 0u;
    const uint32_t u = (kmax & 0x80000000u) ? (kmax & 0x7FFFFFFFu) : ~kmax;
    ids[r] = best;
    vals[r] = __uint_as_float(u);
  }
}

// Whole-workgroup routing into LDS; needs blockDim.x >= 64 * q.  Ends with a
// barrier, so every thread may read the table afterwards.
__device__ __forceinline__ void route_wg(const RouteParams &rp, RouteLds *s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < rp.q) {
    int32_t ids[kKMax];
    float vals[kKMax];
    topk_wave(rp, wave, lane, ids, vals);
    if (lane == 0) {
      float z = 0.f;
      for (int j = 0; j < rp.k; ++j) z += expf(vals[j] - vals[0]);
      for (int j = 0; j < rp.k; ++j) {
        s->ids[wave][j] = ids[j];
        s->gw[wave][j] = expf(vals[j] - vals[0]) / z * rp.routed_scale;
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane i < n holds entry (column i / k, rank i % k); a slot per distinct
    // expert, in order of first appearance
    const int n = rp.q * rp.k;
    int e = -1, c = 0;
    float w = 0.f;
    if (lane < n) {
      c = lane / rp.k;
      e = s->ids[c][lane % rp.k];
      w = s->gw[c][lane % rp.k];
    }
    int first = lane;
    for (int j = 0; j < n; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      if (lane < n && ej == e && j < first) first = j;
    }
    const bool is_first = lane < n && first == lane;
    const uint64_t firsts = __ballot(is_first);
    int slot = 1 + __popcll(firsts & ((1ull << lane) - 1ull));
    slot = __shfl(slot, first, 64);
    int pos = 0, cnt = 0;
    uint32_t mask = 0;
    for (int j = 0; j < n; ++j) {
      const int sj = __builtin_amdgcn_readlane(slot, j), cj = __builtin_amdgcn_readlane(c, j);
      if (sj == slot) {
        ++cnt;
        if (j < lane) ++pos;
        mask |= 1u << cj;
      }
    }
    if (lane < n) {
      s->cols[slot][pos] = c;
      s->w[slot][pos] = w;
      if (is_first) {
        s->expert[slot] = e;
        s->ncols[slot] = cnt;
        s->mask[slot] = mask;
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
