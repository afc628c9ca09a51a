// prefill.hip -- prefill chunk through one layer (tokens grouped per expert,
// grouped products on the matrix cores).  Page "DeepSeek V4 Flash 在 128GB
// 锐龙 AI MAX+ 上跑到 32 tok/s" (taozi.news), section "稀疏预填充：约 250
// tok/s": prefill is batched per layer.
#include "rfpx_impl.hpp"

using namespace rfpx;

extern "C" rfpx_status moe_prefill_forward(const moe_layer *L, const void *x,
                                           int xtype, int T, float *y,
                                           void *ws, size_t ws_bytes,
                                           void *stream) {
  (void)L; (void)x; (void)xtype; (void)T; (void)y; (void)ws; (void)ws_bytes;
  (void)stream;
  return fail(RFPX_E_SHAPE, "moe_prefill_forward: not available in this build");
}
