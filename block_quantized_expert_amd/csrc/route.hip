// route.hip -- router scores and activation preparation (one launch), and
// k_topk for moe_route_topk.
//
// Page "APU 实现 token 自由：AMD Ryzen AI MAX+ 395 跑 DeepSeek V4 Flash，284B
// 模型跑出 32 tok/s" (ainomam.com), section "Lucebox 的优化三板斧": the
// routing path runs TOP-K and ARGSORT kernels, and in the q=4 verify path
// each packed weight is decoded once and applied to all 4 columns.  Page
// "Lucebox专攻DeepSeek V4…" (m.mzlw.cn), section "MoE 专家并行": 256 routed
// experts, top-6, plus one shared expert per layer.
//
// k_route: workgroups 0..E-1 compute the router scores, one expert row per
//   workgroup (the 4 MiB router matrix of d=4096, E=256 is streamed once);
//   workgroups E.. prepare the activations for the gate/up kernel (bf16
//   pair words in each gate/up format's decode order and per-block
//   accumulator starts, rfpx_impl.hpp).  No cross-workgroup
//   synchronization: the next launch reads both.
// k_topk: one workgroup running the routing step (route_wg) into the route
//   table, for moe_route_topk and for layer steps of several columns.  In a
//   one-column step the same step runs at the start of every routed gate/up
//   workgroup instead (it is short there, and overlaps the shared expert).
#include "rfpx_route.hpp"

namespace rfpx {
namespace {

constexpr int kRouteThreads = 256;

struct RouteArgs {
  int d, E, k, q, xtype, nb_d, vx;
  const float *wr;
  const void *x;
  float *scores;
  int n_router_wg;
  int n_prep_items;
  unsigned prep_fmts;
  uint32_t *xp;
  float *xnc;
};

// Prepared activations of block b of column c for gate/up format FMT.
template <int FMT>
__device__ void prep_item(const RouteArgs &a, int c, int b) {
  const int fi = FMT - RFPX_FP2;
  const size_t item = ((size_t)fi * a.q + c) * a.nb_d + b;
  uint32_t *dst = a.xp + item * (size_t)a.vx * 16;
  uint32_t hi[32], lo[32], pw[16];
  float nc_hi, nc_lo = 0.f;
  // the block's 32 activations in 16-byte loads (x is 16-byte aligned and
  // d a multiple of 32, so every block starts on a 64-byte boundary)
  if (a.xtype == RFPX_X_BF16) {
    const uint4 *xs = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) +
                                                      (size_t)c * a.d + 32 * b);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 w = xs[v];
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[8 * v + 2 * i] = wd[i] & 0xFFFFu;
        hi[8 * v + 2 * i + 1] = wd[i] >> 16;
      }
    }
  } else {
    // fp32 activation = bf16 hi + bf16 lo (relative residual below 2^-16)
    const float4 *xs = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) +
                                                        (size_t)c * a.d + 32 * b);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float4 w = xs[v];
      const float wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[4 * v + i] = float_to_bf16_rne(wd[i]);
        lo[4 * v + i] = float_to_bf16_rne(wd[i] - bf16_bits_to_float(hi[4 * v + i]));
      }
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
    router_row<kRouteThreads>(a.wr, a.x, a.xtype, a.d, a.E, a.q, a.scores, bid);
    return;
  }
  const int item = (bid - a.n_router_wg) * kRouteThreads + tid;
  if (item >= a.n_prep_items) return;
  // items run over (format present, column, block)
  const int per_fmt = a.q * a.nb_d;
  const int nth = item / per_fmt, rem = item % per_fmt;
  const int c = rem / a.nb_d, b = rem % a.nb_d;
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
  const uint8_t *image;
  RouteTable *rt;
  int32_t *ids_out;
  float *w_out;
};

constexpr int kTopkThreads = 512;
constexpr int kTopkDescPerThread = (kEMax + 1 + kTopkThreads - 1) / kTopkThreads;

// The image-table fields of one expert that the expert kernels read: every
// plane offset and the gate/up and down formats.
struct SlotPlanes {
  uint64_t codes[3], scales[3];
  int32_t fmt_gu, fmt_dn;
};

__global__ __launch_bounds__(kTopkThreads) void k_topk(TopkArgs a) {
  __shared__ RouteLds s;
  __shared__ SlotPlanes planes[kEMax + 1];
  __shared__ uint32_t scr[2 * kEMax];
  const int tid = threadIdx.x;
  const int q = a.rp.q, k = a.rp.k, E = a.rp.E;
  // the image-table entries (shared expert included), loaded before the
  // routing step so they arrive with the scores
  const ExpertDesc *tab = a.image ? reinterpret_cast<const ExpertDesc *>(a.image + kImgTable) : nullptr;
  SlotPlanes pp[kTopkDescPerThread];
#pragma unroll
  for (int i = 0; i < kTopkDescPerThread; ++i) {
    const int e = tid + kTopkThreads * i;
    if (tab && e <= E) {
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        pp[i].codes[m] = tab[e].codes[m];
        pp[i].scales[m] = tab[e].scales[m];
      }
      pp[i].fmt_gu = tab[e].fmt[0];
      pp[i].fmt_dn = tab[e].fmt[2];
    }
  }
  route_wg(a.rp, &s, scr);
#pragma unroll
  for (int i = 0; i < kTopkDescPerThread; ++i) {
    const int e = tid + kTopkThreads * i;
    if (tab && e <= E) planes[e] = pp[i];
  }
  if (a.ids_out)
    for (int i = tid; i < q * k; i += blockDim.x) {
      const int c = i / k, j = i % k;
      a.ids_out[i] = s.ids[c][j];
      a.w_out[i] = s.gw[c][j];
    }
  publish_route(s, q, -1, true, a.rt);  // the whole table
  __syncthreads();
  if (tab && tid < s.nslots) {
    const SlotPlanes &sp = planes[s.expert[tid]];
    a.rt->dn_codes[tid] = sp.codes[2];
    a.rt->dn_scales[tid] = sp.scales[2];
    a.rt->dn_fmt[tid] = sp.fmt_dn;
    a.rt->gu_codes[tid][0] = sp.codes[0];
    a.rt->gu_codes[tid][1] = sp.codes[1];
    a.rt->gu_scales[tid][0] = sp.scales[0];
    a.rt->gu_scales[tid][1] = sp.scales[1];
    a.rt->gu_fmt[tid] = sp.fmt_gu;
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
  a.wr = p.router_w;
  a.x = p.x;
  a.scores = reinterpret_cast<float *>(p.ws + p.wl.scores);
  a.n_router_wg = p.E;
  const int nf = __builtin_popcount(p.gu_fmts);
  a.n_prep_items = p.route_only ? 0 : nf * p.q * (p.d / 32);
  a.prep_fmts = p.gu_fmts;
  a.xp = reinterpret_cast<uint32_t *>(p.ws + p.wl.xp);
  a.xnc = reinterpret_cast<float *>(p.ws + p.wl.xnc);
  const int n_prep_wg = (a.n_prep_items + kRouteThreads - 1) / kRouteThreads;
  hipEvent_t *ev = (hipEvent_t *)p.events;
  const bool topk = p.route_only || p.pre_route;
  hipError_t e = launch_k(k_route, dim3(a.n_router_wg + n_prep_wg), dim3(kRouteThreads), 0,
                          p.stream, a, ev ? ev[0] : nullptr, ev && !topk ? ev[1] : nullptr);
  if (e != hipSuccess || !topk) return e;
  TopkArgs t{};
  t.rp = route_params(p);
  // moe_route_topk reads the router only: its image is never dereferenced
  t.image = p.route_only ? nullptr : p.image;
  t.rt = reinterpret_cast<RouteTable *>(p.ws + p.wl.route);
  t.ids_out = p.ids_out;
  t.w_out = p.w_out;
  return launch_k(k_topk, dim3(1), dim3(kTopkThreads), 0, p.stream, t, nullptr,
                  ev ? ev[1] : nullptr);
}

}  // namespace rfpx
