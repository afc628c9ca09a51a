// route.hip -- router scores, top-k, gating and verify-column batching.
//
// Page "APU 实现 token 自由：AMD Ryzen AI MAX+ 395 跑 DeepSeek V4 Flash，284B
// 模型跑出 32 tok/s" (ainomam.com), section "Lucebox 的优化三板斧": the
// routing path runs TOP-K and ARGSORT kernels, and in the q=4 verify path
// each packed weight is decoded once and applied to all 4 columns.  Page
// "Lucebox专攻DeepSeek V4…" (m.mzlw.cn), section "MoE 专家并行": 256 routed
// experts, top-6, plus 1 shared expert per layer.
//
// One launch.  Workgroups 0..E-1 compute router scores, one expert per
// workgroup (the 4 MiB router matrix of d=4096, E=256 is streamed once);
// workgroups E.. prepare the activations for the expert kernels
// (bf16 pair words and per-block accumulator starts, see rfpx_impl.hpp).
// The workgroup that arrives last (device-scope counter) ranks the scores
// of every column -- k rounds of a wave-wide arg-max, ties to the lower
// index -- computes the softmax gating weights, and builds the slot table:
// slot 0 is the shared expert for every column, slots 1.. are the distinct
// routed experts of all q columns with, for each, the columns that chose it
// and their weights.  It also clears the counters the down kernel uses.
#include <math.h>

#include "rfpx_impl.hpp"

namespace rfpx {
namespace {

constexpr int kRouteThreads = 256;

struct RouteArgs {
  int d, E, k, q, xtype, nb_d, vx;
  float routed_scale;
  const float *wr;
  const void *x;
  float *scores;
  RouteTable *rt;
  int *counters;
  int n_counters;
  int n_router_wg;
  int n_prep_items;
  unsigned prep_fmts;
  uint32_t *xp;
  float *xnc;
  int32_t *ids_out;
  float *w_out;
  int route_only;
};

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Router scores of expert e for all q columns, one workgroup per expert:
// thread t takes float4 groups t, t+256, ... of the router row (d <= 4096:
// at most 4 per thread) and the same groups of every column of x, all
// loads issued before any arithmetic; partial sums meet in LDS.
__device__ void router_wg(const RouteArgs &a, int e, int tid) {
  constexpr int NPT = 4;
  const int n4 = a.d / 4;
  const float4 *wrow = reinterpret_cast<const float4 *>(a.wr + (size_t)e * a.d);
  float4 w[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    int i4 = tid + kRouteThreads * j;
    w[j] = i4 < n4 ? wrow[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float acc[kQMax];
#pragma unroll
  for (int c = 0; c < kQMax; ++c) {
    acc[c] = 0.f;
    if (c >= a.q) continue;
    float4 xv[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      int i4 = tid + kRouteThreads * j;
      if (i4 >= n4) {
        xv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      } else if (a.xtype == RFPX_X_BF16) {
        uint2 b = reinterpret_cast<const uint2 *>(
            static_cast<const uint16_t *>(a.x) + (size_t)c * a.d)[i4];
        xv[j] = make_float4(__uint_as_float(b.x << 16),
                            __uint_as_float(b.x & 0xFFFF0000u),
                            __uint_as_float(b.y << 16),
                            __uint_as_float(b.y & 0xFFFF0000u));
      } else {
        xv[j] = reinterpret_cast<const float4 *>(
            static_cast<const float *>(a.x) + (size_t)c * a.d)[i4];
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
  __shared__ float part[kRouteThreads / 64][kQMax];
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int c = 0; c < kQMax; ++c) {
    if (c >= a.q) break;
    float s = wave_sum(acc[c]);
    if (lane == 0) part[wave][c] = s;
  }
  __syncthreads();
  if (tid < a.q) {
    float s = 0.f;
    for (int wv = 0; wv < kRouteThreads / 64; ++wv) s += part[wv][tid];
    a.scores[(size_t)tid * a.E + e] = s;
  }
}

template <int FMT>
__device__ void prep_item(const RouteArgs &a, int c, int b) {
  int fi = FMT - RFPX_FP2;
  size_t item = ((size_t)fi * a.q + c) * a.nb_d + b;
  uint32_t *dst = a.xp + item * (size_t)a.vx * 16;
  uint32_t hi[32], lo[32], pw[16];
  float nc_hi, nc_lo = 0.f;
  if (a.xtype == RFPX_X_BF16) {
    const uint16_t *xs = static_cast<const uint16_t *>(a.x) + (size_t)c * a.d + 32 * b;
#pragma unroll
    for (int j = 0; j < 32; ++j) hi[j] = xs[j];
  } else {
    // fp32 activation = bf16 hi + bf16 lo (relative residual below 2^-16)
    const float *xs = static_cast<const float *>(a.x) + (size_t)c * a.d + 32 * b;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float v = xs[j];
      hi[j] = float_to_bf16_rne(v);
      lo[j] = float_to_bf16_rne(v - bf16_bits_to_float(hi[j]));
    }
  }
  prep_pairs<FMT>(hi, pw, &nc_hi);
#pragma unroll
  for (int p = 0; p < 16; ++p) dst[p] = pw[p];
  if (a.vx == 2) {
    prep_pairs<FMT>(lo, pw, &nc_lo);
#pragma unroll
    for (int p = 0; p < 16; ++p) dst[16 + p] = pw[p];
  }
  a.xnc[item] = nc_hi + nc_lo;
}

// Rank the E scores of one column (one wave): k rounds of arg-max over
// (score descending, index ascending).
__device__ void topk_wave(const RouteArgs &a, int c, int lane, int32_t *ids,
                          float *vals) {
  constexpr int PER = kEMax / 64;
  float sv[PER];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int e = lane + 64 * i;
    sv[i] = e < a.E ? a.scores[(size_t)c * a.E + e] : -INFINITY;
  }
  for (int r = 0; r < a.k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int e = lane + 64 * i;
      bool ok = e < a.E && !((taken >> i) & 1u);
      if (ok && (sv[i] > bv || (sv[i] == bv && e < bi))) {
        bv = sv[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    ids[r] = bi;
    vals[r] = bv;
  }
}

__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  if (bid < a.n_router_wg) {
    router_wg(a, bid, tid);
  } else {
    int item = (bid - a.n_router_wg) * kRouteThreads + tid;
    if (item < a.n_prep_items) {
      // items run over (format present, column, block)
      int per_fmt = a.q * a.nb_d;
      int nth = item / per_fmt, rem = item % per_fmt;
      int c = rem / a.nb_d, b = rem % a.nb_d;
      int fmt = 0;
      for (int f = RFPX_FP2, seen = 0; f <= RFPX_FP4; ++f)
        if ((a.prep_fmts >> f) & 1u) {
          if (seen == nth) fmt = f;
          ++seen;
        }
      if (fmt == RFPX_FP2) prep_item<RFPX_FP2>(a, c, b);
      else if (fmt == RFPX_FP3) prep_item<RFPX_FP3>(a, c, b);
      else if (fmt == RFPX_FP4) prep_item<RFPX_FP4>(a, c, b);
    }
  }

  // ---- last workgroup to arrive ranks, gates and batches
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    int prev = __hip_atomic_fetch_add(&a.counters[0], 1, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (int)gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  __shared__ int32_t s_ids[kQMax][kKMax];
  __shared__ float s_gw[kQMax][kKMax];
  for (int c = wave; c < a.q; c += kRouteThreads / 64) {
    int32_t ids[kKMax];
    float vals[kKMax];
    topk_wave(a, c, lane, ids, vals);
    if (lane == 0) {
      float z = 0.f;
      for (int j = 0; j < a.k; ++j) z += expf(vals[j] - vals[0]);
      for (int j = 0; j < a.k; ++j) {
        float w = expf(vals[j] - vals[0]) / z * a.routed_scale;
        s_ids[c][j] = ids[j];
        s_gw[c][j] = w;
        a.rt->ids[c][j] = ids[j];
        a.rt->gw[c][j] = w;
        if (a.ids_out) a.ids_out[c * a.k + j] = ids[j];
        if (a.w_out) a.w_out[c * a.k + j] = w;
      }
    }
  }
  __syncthreads();
  if (tid == 0) a.counters[0] = 0;  // every other workgroup has arrived
  if (a.route_only) return;
  for (int i = 1 + tid; i < a.n_counters; i += kRouteThreads) a.counters[i] = 0;

  if (wave == 0) {
    // lane i < n holds entry (column i / k, rank i % k)
    const int n = a.q * a.k;
    int e = -1, c = 0;
    float w = 0.f;
    if (lane < n) {
      c = lane / a.k;
      e = s_ids[c][lane % a.k];
      w = s_gw[c][lane % a.k];
    }
    int first = lane;
    for (int j = 0; j < n; ++j) {
      int ej = __shfl(e, j, 64);
      if (lane < n && ej == e && j < first) first = j;
    }
    bool is_first = lane < n && first == lane;
    uint64_t firsts = __ballot(is_first);
    int slot = 1 + __popcll(firsts & ((1ull << lane) - 1ull));
    slot = __shfl(slot, first, 64);
    int pos = 0, cnt = 0;
    uint32_t mask = 0;
    for (int j = 0; j < n; ++j) {
      int sj = __shfl(slot, j, 64), cj = __shfl(c, j, 64);
      if (sj == slot) {
        ++cnt;
        if (j < lane) ++pos;
        mask |= 1u << cj;
      }
    }
    RouteTable *rt = a.rt;
    if (lane < n) {
      rt->cols[slot][pos] = c;
      rt->w[slot][pos] = w;
      if (is_first) {
        rt->expert[slot] = e;
        rt->ncols[slot] = cnt;
        rt->mask[slot] = mask;
      }
    }
    if (lane == 0) {
      rt->nslots = 1 + __popcll(firsts);
      rt->expert[0] = a.E;
      rt->ncols[0] = a.q;
      rt->mask[0] = (1u << a.q) - 1u;
    }
    if (lane < a.q) {
      rt->cols[0][lane] = lane;
      rt->w[0][lane] = 1.0f;
    }
  }
}

}  // namespace

hipError_t launch_route(const ForwardPlan &p) {
  RouteArgs a{};
  a.d = p.d;
  a.E = p.E;
  a.k = p.k;
  a.q = p.q;
  a.xtype = p.xtype;
  a.nb_d = p.d / 32;
  a.vx = p.xtype == RFPX_X_BF16 ? 1 : 2;
  a.routed_scale = p.routed_scale;
  a.wr = p.router_w;
  a.x = p.x;
  a.scores = reinterpret_cast<float *>(p.ws + p.wl.scores);
  a.rt = reinterpret_cast<RouteTable *>(p.ws + p.wl.route);
  a.counters = reinterpret_cast<int *>(p.ws + p.wl.counters);
  a.n_counters = 1 + p.wl.n_tiles_down;
  a.n_router_wg = p.E;
  int nf = __builtin_popcount(p.prep_fmts);
  a.n_prep_items = p.route_only ? 0 : nf * p.q * (p.d / 32);
  a.prep_fmts = p.prep_fmts;
  a.xp = reinterpret_cast<uint32_t *>(p.ws + p.wl.xp);
  a.xnc = reinterpret_cast<float *>(p.ws + p.wl.xnc);
  a.ids_out = p.ids_out;
  a.w_out = p.w_out;
  a.route_only = p.route_only ? 1 : 0;
  int n_prep_wg = (a.n_prep_items + kRouteThreads - 1) / kRouteThreads;
  k_route<<<a.n_router_wg + n_prep_wg, kRouteThreads, 0, p.stream>>>(a);
  return hipGetLastError();
}

}  // namespace rfpx
