// route.hip -- router scores, top-k, gating and verify-column batching.
//
// Page "APU 实现 token 自由：AMD Ryzen AI MAX+ 395 跑 DeepSeek V4 Flash，284B
// 模型跑出 32 tok/s" (ainomam.com), section "Lucebox 的优化三板斧": the
// routing path runs TOP-K and ARGSORT kernels, and in the q=4 verify path
// each packed weight is decoded once and applied to all 4 columns.  Page
// "Lucebox专攻DeepSeek V4…" (m.mzlw.cn), section "MoE 专家并行": 256 routed
// experts, top-6, plus 1 shared expert per layer.
//
// k_route: workgroups 0..E-1 compute the router scores, one expert per
//   workgroup (the 4 MiB router matrix of d=4096, E=256 is streamed once);
//   workgroups E.. prepare the activations for the expert kernels (bf16
//   pair words and per-block accumulator starts, see rfpx_impl.hpp).  No
//   cross-workgroup synchronization: the next launch reads the scores.
// route_wg (device function): ranks the scores of every column -- k rounds
//   of a wave-wide arg-max, ties to the lower index -- computes the softmax
//   gating weights and builds the slot table in LDS: slot 0 is the shared
//   expert for every column, slots 1.. are the distinct routed experts of
//   all q columns in order of first appearance, each with the columns that
//   chose it and their weights.  The computation is deterministic, so every
//   workgroup that runs it gets the same table; the gate/up kernel runs it
//   at its start instead of a separate launch.
// k_topk: one workgroup running route_wg, for moe_route_topk.
#include <math.h>

#include "rfpx_route.hpp"

namespace rfpx {
namespace {

constexpr int kRouteThreads = 256;

struct RouteArgs {
  int d, E, k, q, xtype, nb_d, vx;
  float routed_scale;
  const float *wr;
  const void *x;
  float *scores;
  int n_router_wg;
  int n_prep_items;
  unsigned prep_fmts;
  uint32_t *xp;
  float *xnc;
};

__device__ __forceinline__ float wave_sum(float v) {
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
  // unconditional loads (clamped index, zeroed after) so that every load is
  // in flight before the first use
  float4 w[NPT];
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i4 = tid + kRouteThreads * j;
    w[j] = wrow[i4 < n4 ? i4 : n4 - 1];
  }
#pragma unroll
  for (int j = 0; j < NPT; ++j)
    if (tid + kRouteThreads * j >= n4) w[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  float acc[kQMax];
#pragma unroll
  for (int c = 0; c < kQMax; ++c) {
    acc[c] = 0.f;
    if (c >= a.q) continue;
    float4 xv[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i4c = min(tid + kRouteThreads * j, n4 - 1);  // w is zero past n4
      if (a.xtype == RFPX_X_BF16) {
        uint2 b = reinterpret_cast<const uint2 *>(
            static_cast<const uint16_t *>(a.x) + (size_t)c * a.d)[i4c];
        xv[j] = make_float4(__uint_as_float(b.x << 16),
                            __uint_as_float(b.x & 0xFFFF0000u),
                            __uint_as_float(b.y << 16),
                            __uint_as_float(b.y & 0xFFFF0000u));
      } else {
        xv[j] = reinterpret_cast<const float4 *>(
            static_cast<const float *>(a.x) + (size_t)c * a.d)[i4c];
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

__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a) {
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  if (bid < a.n_router_wg) {
    router_wg(a, bid, tid);
    return;
  }
  int item = (bid - a.n_router_wg) * kRouteThreads + tid;
  if (item >= a.n_prep_items) return;
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

struct TopkArgs {
  RouteParams rp;
  RouteTable *rt;
  int32_t *ids_out;
  float *w_out;
};

__global__ __launch_bounds__(512) void k_topk(TopkArgs a) {
  __shared__ RouteLds s;
  route_wg(a.rp, &s);
  const int tid = threadIdx.x;
  const int q = a.rp.q, k = a.rp.k;
  for (int i = tid; i < q * k; i += blockDim.x) {
    const int c = i / k, j = i % k;
    a.ids_out[i] = s.ids[c][j];
    a.w_out[i] = s.gw[c][j];
  }
  publish_route(s, q, -1, true, a.rt);  // the whole table
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
  a.n_router_wg = p.E;
  int nf = __builtin_popcount(p.prep_fmts);
  a.n_prep_items = p.route_only ? 0 : nf * p.q * (p.d / 32);
  a.prep_fmts = p.prep_fmts;
  a.xp = reinterpret_cast<uint32_t *>(p.ws + p.wl.xp);
  a.xnc = reinterpret_cast<float *>(p.ws + p.wl.xnc);
  int n_prep_wg = (a.n_prep_items + kRouteThreads - 1) / kRouteThreads;
  k_route<<<a.n_router_wg + n_prep_wg, kRouteThreads, 0, p.stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.route_only) return e;
  TopkArgs t{};
  t.rp = route_params(p);
  t.rt = reinterpret_cast<RouteTable *>(p.ws + p.wl.route);
  t.ids_out = p.ids_out;
  t.w_out = p.w_out;
  k_topk<<<1, 512, 0, p.stream>>>(t);
  return hipGetLastError();
}

}  // namespace rfpx
