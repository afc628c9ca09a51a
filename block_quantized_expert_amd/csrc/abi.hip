// abi.hip -- host side of the C ABI: argument validation, the image and
// workspace layouts, the launch plan of a decode step, status strings.
//
// Layer definition: page "Lucebox专攻DeepSeek V4…" (m.mzlw.cn), section
// "MoE 专家并行" (256 routed experts, top-6, 1 shared); page "APU 实现 token
// 自由…" (ainomam.com), section "Lucebox 的优化三板斧" (TOP-K/ARGSORT routing,
// decode-once for all verify columns).  Everything here runs on the host
// before any launch; nothing here touches device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "rfpx_impl.hpp"

namespace rfpx {

// Device scratch of moe_layer_forward_noalloc: the decode workspace of one
// call, for callers that cannot allocate.  Every GPU the library runs on
// holds its own copy (loaded with the code object, kept until the process
// ends).  In host code `scratch` names a host-side stand-in; the device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

// Device address of `scratch` on the current device (looked up on the first
// call on that device, with the device current).
static rfpx_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RFPX_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RFPX_E_ARG, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RFPX_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RFPX_OK;
}

static thread_local char g_err[512];

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

rfpx_status fail(rfpx_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

size_t image_layout(int d, int f, int E, const int *fmts, ExpertDesc *desc) {
  size_t off = align_up(kImgTable + (size_t)(E + 1) * sizeof(ExpertDesc), 256);
  for (int e = 0; e <= E; ++e) {
    for (int m = 0; m < 3; ++m) {
      int fmt = fmts[3 * e + m];
      size_t rows = m < 2 ? f : d, cols = m < 2 ? d : f;
      size_t nblk = rows * (cols / 32);
      if (desc) {
        desc[e].codes[m] = off;
        desc[e].fmt[m] = fmt;
      }
      off = align_up(off + nblk * code_bytes(fmt), 256);
      if (desc) desc[e].scales[m] = off;
      off = align_up(off + nblk * scale_bytes(fmt), 256);
    }
    if (desc) desc[e].reserved = 0;
  }
  return off;
}

namespace {

bool pow2_in(int v, int lo, int hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

// Rows per workgroup tile.  A unit is R rows (rpi rows per wave step) of one
// column part; R depends on the format and the pass width (unit_rows_for).
// Gate/up tiles hold whole 32-row blocks of h (the down matrix's blocks).
bool pick_tile_gateup(const Geo *geo, unsigned fmts, int g, int rows, int min_rows, int *rw) {
  int t = 32 > min_rows ? 32 : min_rows;
  for (int f = RFPX_FP2; f <= RFPX_FP4; ++f)
    if ((fmts >> f) & 1u) {
      const int unit = geo[f].rpi * unit_rows_gu(f, g);
      t = t > unit ? t : unit;
    }
  if (t > rows || rows % t) return false;
  *rw = t;
  return true;
}

// Down tiles: about 512 workgroups over the d rows (two per compute unit),
// and at least one unit of every present format.
bool pick_tile_down(const Geo *geo, unsigned fmts, int g, int rows, int min_rows, int *rw) {
  int t = rows / 512 > 1 ? rows / 512 : 1;
  t = t > min_rows ? t : min_rows;
  for (int f = RFPX_FP2; f <= RFPX_FP4; ++f)
    if ((fmts >> f) & 1u) {
      const int unit = geo[f].rpi * unit_rows_for(f, g);
      t = t > unit ? t : unit;
    }
  if (t > rows || rows % t) return false;
  *rw = t;
  return true;
}

}  // namespace

rfpx_status check_layer(const moe_layer *L) {
  if (!L) return fail(RFPX_E_ARG, "layer is null");
  if (!L->fmts) return fail(RFPX_E_ARG, "layer format table is null");
  if (!pow2_in(L->d, 256, 4096))
    return fail(RFPX_E_SHAPE, "d=%d: must be a power of two in [256, 4096]", L->d);
  if (!pow2_in(L->f, 64, 4096))
    return fail(RFPX_E_SHAPE, "f=%d: must be a power of two in [64, 4096]", L->f);
  if (L->n_experts < 1 || L->n_experts > kEMax)
    return fail(RFPX_E_SHAPE, "n_experts=%d: must be in [1, %d]", L->n_experts, kEMax);
  if (L->top_k < 1 || L->top_k > kKMax || L->top_k > L->n_experts)
    return fail(RFPX_E_SHAPE, "top_k=%d: must be in [1, min(E, %d)]", L->top_k, kKMax);
  for (int i = 0; i < 3 * (L->n_experts + 1); ++i)
    if (!valid_fmt(L->fmts[i]))
      return fail(RFPX_E_FORMAT, "format table entry %d is %d", i, L->fmts[i]);
  for (int e = 0; e <= L->n_experts; ++e)
    if (L->fmts[3 * e] != L->fmts[3 * e + 1])
      return fail(RFPX_E_FORMAT, "expert %d: gate and up formats differ", e);
  return RFPX_OK;
}

rfpx_status check_image(const moe_layer *L) {
  if (!L->image) return fail(RFPX_E_ARG, "layer image is null");
  if ((uintptr_t)L->image % 256) return fail(RFPX_E_ALIGN, "image not 256-byte aligned");
  const size_t need = image_layout(L->d, L->f, L->n_experts, L->fmts, nullptr);
  if (L->image_bytes != need)
    return fail(RFPX_E_FORMAT, "image_bytes is %zu, the format table lays out %zu", L->image_bytes,
                need);
  return RFPX_OK;
}

namespace {

// Everything a decode step needs that depends only on shapes and formats.
rfpx_status make_plan(const moe_layer *L, int q, int xtype, ForwardPlan *p) {
  rfpx_status st = check_layer(L);
  if (st) return st;
  if (q < 1 || q > kQMax) return fail(RFPX_E_SHAPE, "q=%d: must be in [1, %d]", q, kQMax);
  if (xtype != RFPX_X_F32 && xtype != RFPX_X_BF16)
    return fail(RFPX_E_ARG, "xtype=%d", xtype);
  memset(p, 0, sizeof *p);
  p->d = L->d;
  p->f = L->f;
  p->E = L->n_experts;
  p->k = L->top_k;
  p->q = q;
  p->xtype = xtype;
  p->routed_scale = L->routed_scale;
  p->router_w = L->router_w;
  p->image = L->image;
  for (int e = 0; e <= L->n_experts; ++e) {
    p->gu_fmts |= 1u << L->fmts[3 * e];
    p->down_fmts |= 1u << L->fmts[3 * e + 2];
  }
  for (int f = RFPX_FP2; f <= RFPX_FP4; ++f) {
    if ((p->gu_fmts >> f) & 1u) {
      if (!make_geo(f, L->d, &p->geo_gu[f]) || p->geo_gu[f].tpl > 2)
        return fail(RFPX_E_SHAPE, "d=%d does not tile for gate/up format %d", L->d, f);
    }
    if ((p->down_fmts >> f) & 1u) {
      if (!make_geo(f, L->f, &p->geo_dn[f]) || p->geo_dn[f].tpl > 2)
        return fail(RFPX_E_SHAPE, "f=%d does not tile for down format %d", L->f, f);
    }
  }
  p->g = q == 1 ? 1 : 2;
  // with several columns the routing step costs more and every routed
  // gate/up workgroup would repeat it: run it once before the experts
  p->pre_route = q > 1;  // exactly the steps of two-column passes (g = 2)
  // waves per down workgroup (a multiple of the column parts, 1 or 2)
  p->wmax = q == 1 ? kDnWavesQ1 : kDnWavesQn;
  // gate/up workgroups: waves and the smallest tile; a wave streams
  // rw_gu / (4 rpi) * parts / waves units with the next one in flight
  p->wgu = q == 1 ? kGuWavesQ1 : kGuWavesQn;
  const int gu_min = q == 1 ? kGuRowsQ1 : kGuRowsQn;
  if (!pick_tile_gateup(p->geo_gu, p->gu_fmts, p->g, L->f, gu_min < L->f ? gu_min : L->f,
                        &p->rw_gu))
    return fail(RFPX_E_SHAPE, "f=%d: no gate/up tile for this format mix", L->f);
  const int dn_min = q == 1 ? kDnRowsQ1 : kDnRowsQn;
  if (!pick_tile_down(p->geo_dn, p->down_fmts, p->g, L->d, dn_min < L->d ? dn_min : L->d,
                      &p->rw_dn))
    return fail(RFPX_E_SHAPE, "d=%d: no down tile for this format mix", L->d);
  // per-wave accumulators of the down tile in LDS: fewer waves when a wide
  // tile (short rows make long units) and many columns would not fit
  if (q == 1) {
    // one-column steps deal the units of the k + 1 slots round-robin: no
    // more waves than the most units a tile can hold (7 at k = 6 with one
    // unit per slot), kept a multiple of the column parts
    int per_slot = 1, parts = 1;
    for (int f = RFPX_FP2; f <= RFPX_FP4; ++f)
      if ((p->down_fmts >> f) & 1u) {
        const int u = p->rw_dn / (unit_rows_for(f, 1) * p->geo_dn[f].rpi) * p->geo_dn[f].tpl;
        per_slot = per_slot > u ? per_slot : u;
        parts = parts > p->geo_dn[f].tpl ? parts : p->geo_dn[f].tpl;
      }
    const int units = (L->top_k + 1) * per_slot;
    if (units < p->wmax) p->wmax = (units + parts - 1) / parts * parts;
    // one unit per slot and one wave per slot: a wave knows its slot (and,
    // with one block per lane, its h) before the route table arrives
    p->h_early = per_slot == 1 && parts == 1 && p->wmax == L->top_k + 1 &&
                 !((p->down_fmts >> RFPX_FP2) & 1u);
  }
  // per wave: its accumulator rows and 64 sink words
  while (p->wmax > 2 && (size_t)p->wmax * (q * p->rw_dn + 64) * sizeof(float) > 48 * 1024) p->wmax /= 2;
  if ((size_t)p->wmax * (q * p->rw_dn + 64) * sizeof(float) > 48 * 1024)
    return fail(RFPX_E_SHAPE, "f=%d, q=%d: down tile of %d rows needs too much LDS", L->f, q,
                p->rw_dn);

  WsLayout &w = p->wl;
  const int nb_f = L->f / 32;
  w.max_slots = 1 + (q * L->top_k < L->n_experts ? q * L->top_k : L->n_experts);
  size_t off = 0;
  w.route = off;
  off = align_up(off + sizeof(RouteTable), 256);
  w.scores = off;
  off = align_up(off + (size_t)q * L->n_experts * 4, 256);
  const int vx = xtype == RFPX_X_BF16 ? 1 : 2;
  const int nb_d = L->d / 32;
  w.xp = off;
  off = align_up(off + (size_t)3 * q * nb_d * vx * 16 * 4, 256);
  w.xnc = off;
  off = align_up(off + (size_t)3 * q * nb_d * 4, 256);
  w.hp = off;
  off = align_up(off + (size_t)w.max_slots * q * nb_f * 32 * 4, 256);
  w.total = off;
  return RFPX_OK;
}

// Router, image and activations of a decode call; the image is checked only
// when the call reads it (moe_route_topk does not).
rfpx_status check_inputs(const moe_layer *L, const void *x, bool reads_image) {
  if (!L->router_w) return fail(RFPX_E_ARG, "layer router is null");
  rfpx_status st = reads_image ? check_image(L) : RFPX_OK;
  if (st) return st;
  if (!x) return fail(RFPX_E_ARG, "x is null");
  if ((uintptr_t)L->router_w % 16 || (uintptr_t)x % 16)
    return fail(RFPX_E_ALIGN, "router weights and x must be 16-byte aligned");
  return RFPX_OK;
}

// ... and the workspace.
rfpx_status check_run(const moe_layer *L, const ForwardPlan &p, const void *x,
                      void *ws, size_t ws_bytes, bool reads_image) {
  rfpx_status st = check_inputs(L, x, reads_image);
  if (st) return st;
  if (!ws) return fail(RFPX_E_ARG, "workspace is null");
  if ((uintptr_t)ws % 256) return fail(RFPX_E_ALIGN, "workspace not 256-byte aligned");
  if (ws_bytes < p.wl.total)
    return fail(RFPX_E_WORKSPACE, "workspace holds %zu bytes, needs %zu", ws_bytes, p.wl.total);
  return RFPX_OK;
}

}  // namespace
}  // namespace rfpx

using namespace rfpx;

extern "C" {

const char *rfpx_status_str(int st) {
  switch (st) {
    case RFPX_OK: return "ok";
    case RFPX_E_ARG: return "bad argument";
    case RFPX_E_SHAPE: return "unsupported shape";
    case RFPX_E_ALIGN: return "misaligned pointer";
    case RFPX_E_FORMAT: return "bad format table or image";
    case RFPX_E_WORKSPACE: return "workspace or output too small";
    case RFPX_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *rfpx_last_error(void) { return g_err; }

size_t moe_workspace_bytes(const moe_layer *L, int q_or_T, int prefill) {
  ForwardPlan p;
  if (prefill) {
    if (check_layer(L)) return 0;
    return prefill_layout(L, q_or_T, RFPX_X_F32, nullptr);  // fp32 x needs the most
  }
  if (make_plan(L, q_or_T, RFPX_X_F32, &p)) return 0;  // fp32 x needs the most
  return p.wl.total;
}

rfpx_status moe_route_topk(const moe_layer *L, const void *x, int xtype, int q,
                           int32_t *ids, float *w, void *ws, size_t ws_bytes,
                           void *stream) {
  ForwardPlan p;
  rfpx_status st = make_plan(L, q, xtype, &p);
  if (st) return st;
  if ((st = check_run(L, p, x, ws, ws_bytes, false))) return st;
  if (!ids || !w) return fail(RFPX_E_ARG, "ids or w is null");
  p.x = x;
  p.ids_out = ids;
  p.w_out = w;
  p.ws = static_cast<uint8_t *>(ws);
  p.route_only = true;
  p.stream = (hipStream_t)stream;
  hipError_t e = launch_route(p);
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "moe_route_topk: %s", hipGetErrorString(e));
}

rfpx_status moe_layer_forward(const moe_layer *L, const void *x, int xtype, int q,
                              float *y, void *ws, size_t ws_bytes, void *stream) {
  return moe_layer_forward_timed(L, x, xtype, q, y, ws, ws_bytes, stream, nullptr);
}

rfpx_status moe_layer_forward_timed(const moe_layer *L, const void *x, int xtype,
                                    int q, float *y, void *ws, size_t ws_bytes,
                                    void *stream, void *const *events) {
  ForwardPlan p;
  rfpx_status st = make_plan(L, q, xtype, &p);
  if (st) return st;
  if ((st = check_run(L, p, x, ws, ws_bytes, true))) return st;
  if (!y) return fail(RFPX_E_ARG, "y is null");
  p.x = x;
  p.y = y;
  p.ws = static_cast<uint8_t *>(ws);
  p.stream = (hipStream_t)stream;
  p.events = events;
  hipError_t e = launch_route(p);
  if (e == hipSuccess) e = launch_experts(p);
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "moe_layer_forward: %s", hipGetErrorString(e));
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

rfpx_status moe_layer_forward_noalloc(const moe_layer *L, const void *x, int xtype, int q,
                                      float *y, void *stream) {
  ForwardPlan p;
  rfpx_status st = make_plan(L, q, xtype, &p);
  if (st) return st;
  if ((st = check_inputs(L, x, true))) return st;
  if (!y) return fail(RFPX_E_ARG, "y is null");
  if (p.wl.total > kScratchBytes)
    return fail(RFPX_E_WORKSPACE,
                "moe_layer_forward_noalloc: this shape needs %zu bytes of workspace, the "
                "library's scratch holds %zu; use moe_layer_forward with a workspace",
                p.wl.total, kScratchBytes);
  void *ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return moe_layer_forward(L, x, xtype, q, y, ws, kScratchBytes, stream);
}

rfpx_status moe_prefill_forward(const moe_layer *L, const void *x, int xtype, int T,
                                float *y, void *ws, size_t ws_bytes, void *stream) {
  return moe_prefill_forward_timed(L, x, xtype, T, y, ws, ws_bytes, stream, nullptr);
}

rfpx_status moe_prefill_forward_timed(const moe_layer *L, const void *x, int xtype, int T,
                                      float *y, void *ws, size_t ws_bytes, void *stream,
                                      void *const *events) {
  rfpx_status st = check_layer(L);
  if (st) return st;
  if (xtype != RFPX_X_F32 && xtype != RFPX_X_BF16) return fail(RFPX_E_ARG, "xtype=%d", xtype);
  if (T < 1 || T > 65536) return fail(RFPX_E_SHAPE, "T=%d: must be in [1, 65536]", T);
  if (L->d % 128 || L->f % 64)
    return fail(RFPX_E_SHAPE, "prefill needs d a multiple of 128 and f of 64 (d=%d, f=%d)",
                L->d, L->f);
  const size_t need = prefill_layout(L, T, xtype, nullptr);
  if (!need) return fail(RFPX_E_SHAPE, "prefill: unsupported shape (T=%d)", T);
  if (!L->router_w) return fail(RFPX_E_ARG, "layer router is null");
  if ((st = check_image(L))) return st;
  if (!x || !y || !ws) return fail(RFPX_E_ARG, "x, y or workspace is null");
  if ((uintptr_t)ws % 256) return fail(RFPX_E_ALIGN, "workspace not 256-byte aligned");
  if ((uintptr_t)L->router_w % 16 || (uintptr_t)x % 16 || (uintptr_t)y % 16)
    return fail(RFPX_E_ALIGN, "router weights, x and y must be 16-byte aligned");
  if (ws_bytes < need)
    return fail(RFPX_E_WORKSPACE, "workspace holds %zu bytes, needs %zu", ws_bytes, need);
  const size_t image_bytes = L->image_bytes;
  if (image_bytes > 0xFFFFFFFFull)
    return fail(RFPX_E_SHAPE, "prefill: image of %zu bytes exceeds 4 GiB", image_bytes);
  hipError_t e = launch_prefill(L, x, xtype, T, y, static_cast<uint8_t *>(ws), image_bytes,
                                (hipStream_t)stream, events);
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "moe_prefill_forward: %s", hipGetErrorString(e));
}

}  // extern "C"
