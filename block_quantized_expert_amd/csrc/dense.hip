// dense.hip -- a dense block-quantized projection applied to q verify
// columns: y[c] = W x_c for c < q, each packed block read and decoded once
// and applied to every column.
//
// Page "APU 实现 token 自由…" (ainomam.com), section "Lucebox 的优化三板斧":
// in the q=4 verify path each packed dense weight is decoded once for all 4
// columns.  Page "DeepSeek V4 Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s"
// (taozi.news), section "ROCmFPX": dense and sensitive projections stay in
// ROCmFP4 or wider; any of FP2/FP3/FP4 is accepted here.
//
// Dense image (a permutation of the canonical blocks): rows are cut into
// tiles of 64; within a tile, chunk k (one block, two for FP2) of its 64
// rows sits contiguously, row r of the tile at lane r:
//   codes  [tile][chunk][64 rows][chunk code bytes: 16 | 12 | 16]
//   scales [tile][chunk][64 rows][chunk scale bytes: 4 | 2 | 1]
// (the scales plane starts on a 256-byte boundary).  A wave then owns 64
// rows, lane l row l: every code load is one fully coalesced 1 KiB (FP3:
// 768 B) request, the activations of a block are the same for all lanes
// (scalar loads, held in scalar registers), and each lane accumulates its
// own row for every column, so no cross-lane reduction is needed.
//
// Launches: k_dense (grid tiles x splits; the waves of a workgroup split
// the tile's chunks, their sums meet in LDS in a fixed order) and, when a
// tile's chunks are split over several workgroups (fewer than 256 tiles),
// k_dense_sum (the splits' partial sums in split order).  A workgroup first
// issues all its weight loads, then, while they are in flight, prepares the
// activations of its blocks (bf16 pair words in the format's decode order
// and each block's accumulator start, as for the expert kernels) into LDS,
// where every lane of a wave reads the same words (broadcast reads).  y is
// the same bit for bit from run to run.
#include "rfpx_impl.hpp"

namespace rfpx {
namespace {

constexpr int kDenseWavesMax = 8;
constexpr int kDenseCpwMax = 16;  // blocks in flight per wave (16 KiB of FP4 codes)
constexpr size_t kDenseLdsMax = 64 * 1024;  // dynamic LDS of one workgroup

struct DenseArgs {
  const uint8_t *codes;    // codes plane
  const uint8_t *scales;   // scales plane
  const void *x;
  float *y;                // [q][rows]
  float *part;             // [splits][q][rows] (splits > 1)
  int rows, cols, nb, nch, q, xtype, vx;
  int waves, cpw, splits;  // chunks per wave; workgroups per tile
};

template <int FMT>
struct DFmt {
  static constexpr int CB = chunk_blocks(FMT);           // blocks per chunk
  static constexpr int CW = FMT == RFPX_FP3 ? 3 : 4;      // code dwords per chunk
  static constexpr int BW = FMT == RFPX_FP2 ? 2 : CW;     // code dwords per block
  static constexpr int CBYTES = CB * code_bytes(FMT);
  static constexpr int SBYTES = CB * scale_bytes(FMT);
};

// Prepared activations of block b of column c into dst (vx * 16 words) and
// its accumulator start into *nc.
template <int FMT>
__device__ void dense_prep_item(const DenseArgs &a, int c, int b, uint32_t *dst, float *nc) {
  uint32_t hi[32], lo[32], pw[16];
  float nc_hi, nc_lo = 0.f;
  if (a.xtype == RFPX_X_BF16) {
    const uint4 *xs = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) +
                                                      (size_t)c * a.cols + 32 * b);
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
                                                        (size_t)c * a.cols + 32 * b);
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
  for (int p = 0; p < 16; p += 4)
    *reinterpret_cast<uint4 *>(dst + p) = make_uint4(pw[p], pw[p + 1], pw[p + 2], pw[p + 3]);
  if (a.vx == 2) {
    prep_pairs<FMT>(lo, pw, &nc_lo);
#pragma unroll
    for (int p = 0; p < 16; p += 4)
      *reinterpret_cast<uint4 *>(dst + 16 + p) = make_uint4(pw[p], pw[p + 1], pw[p + 2], pw[p + 3]);
  }
  *nc = nc_hi + nc_lo;
}

template <int FMT>
__device__ __forceinline__ void dense_load(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                           uint32_t coff, uint32_t soff, uint32_t *cw,
                                           uint32_t &sw) {
  using F = DFmt<FMT>;
  if (FMT == RFPX_FP3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, (int)coff, 0, 0);
    cw[0] = v.x;
    cw[1] = v.y;
    cw[2] = v.z;
    sw = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)soff, 0, 0);
  } else {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)coff, 0, 0);
    cw[0] = v.x;
    cw[1] = v.y;
    cw[2] = v.z;
    cw[3] = v.w;
    if (FMT == RFPX_FP2) sw = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)soff, 0, 0);
    else sw = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)soff, 0, 0);
  }
  (void)F::CB;
}

// Tile blockIdx.x, split blockIdx.y: wave w takes chunks
// (split * waves + w) * cpw .. + cpw of the tile's rows, all loads issued
// first; the workgroup's prepared activations go to LDS meanwhile; each lane
// then accumulates its row for the Q columns.  LDS: the prepared words
// [Q][blocks][VX * 16], their starts [Q][blocks], the wave sums [waves][Q][64].
template <int FMT, int Q, int VX>
__global__ __launch_bounds__(64 * kDenseWavesMax) void k_dense(DenseArgs a) {
  using F = DFmt<FMT>;
  constexpr int CPW_MAX = kDenseCpwMax / F::CB;  // 16 blocks in flight per wave
  extern __shared__ __align__(16) uint32_t lds[];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int tile = blockIdx.x, split = blockIdx.y;
  const int k0 = (split * a.waves + wave) * a.cpw;
  const uint64_t tile_chunks = (uint64_t)tile * a.nch;
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc(a.codes + (tile_chunks + k0) * 64 * F::CBYTES, (uint32_t)(a.cpw * 64 * F::CBYTES));
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(a.scales + (tile_chunks + k0) * 64 * F::SBYTES, (uint32_t)(a.cpw * 64 * F::SBYTES));
  // every load unconditional: chunks past cpw lie past the buffer
  // resources' ranges and read as zero without a memory access (a guard
  // per load would make the compiler wait for each load before the next)
  uint32_t cw[CPW_MAX][F::CW], sw[CPW_MAX];
#pragma unroll
  for (int i = 0; i < CPW_MAX; ++i)
    dense_load<FMT>(rc, rs, (uint32_t)((i * 64 + lane) * F::CBYTES),
                    (uint32_t)((i * 64 + lane) * F::SBYTES), cw[i], sw[i]);
  // the workgroup's blocks b0 .. b0 + nbw of every column, prepared into LDS
  const int nbw = a.waves * a.cpw * F::CB, b0 = split * nbw;
  uint32_t *xw_lds = lds;                                            // [Q][nbw][VX*16]
  float *nc_lds = reinterpret_cast<float *>(lds + (size_t)Q * nbw * VX * 16);  // [Q][nbw]
  float *red = nc_lds + Q * nbw;                                      // [waves][Q][64]
  for (int it = threadIdx.x; it < Q * nbw; it += blockDim.x) {
    const int c = it / nbw, bl = it % nbw;
    dense_prep_item<FMT>(a, c, b0 + bl, xw_lds + (size_t)it * VX * 16, nc_lds + it);
  }
  __syncthreads();
  float acc[Q];
#pragma unroll
  for (int c = 0; c < Q; ++c) acc[c] = 0.f;
  const uint32_t one = one_one_vgpr_pure();
#pragma unroll
  for (int i = 0; i < CPW_MAX; ++i) {
    if (i < a.cpw) {
#pragma unroll
    for (int j = 0; j < F::CB; ++j) {
      const int bl = (wave * a.cpw + i) * F::CB + j;  // block within the workgroup
      uint32_t pr[16];
      decode_pairs<FMT>(&cw[i][j * F::BW], pr, one);
      const float s = block_scale<FMT>(FMT == RFPX_FP2 ? (sw[i] >> (16 * j)) : sw[i]);
#pragma unroll
      for (int c = 0; c < Q; ++c) {
        // every lane reads the same words: broadcast LDS reads
        const uint4 *xv = reinterpret_cast<const uint4 *>(xw_lds + ((size_t)c * nbw + bl) * VX * 16);
        float t0 = nc_lds[c * nbw + bl], t1 = 0.f;
#pragma unroll
        for (int v = 0; v < VX; ++v)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint4 w4 = xv[4 * v + u];
            t0 = dot2(w4.x, pr[4 * u + 0], t0);
            t1 = dot2(w4.y, pr[4 * u + 1], t1);
            t0 = dot2(w4.z, pr[4 * u + 2], t0);
            t1 = dot2(w4.w, pr[4 * u + 3], t1);
          }
        acc[c] = fmaf(t0 + t1, s, acc[c]);
      }
    }
    }
  }
#pragma unroll
  for (int c = 0; c < Q; ++c) red[(wave * Q + c) * 64 + lane] = acc[c];
  __syncthreads();
  for (int i = threadIdx.x; i < Q * 64; i += blockDim.x) {
    const int c = i / 64, l = i % 64;
    float v = 0.f;
    for (int w = 0; w < a.waves; ++w) v += red[(w * Q + c) * 64 + l];
    const size_t row = (size_t)tile * 64 + l;
    if (a.splits == 1) a.y[(size_t)c * a.rows + row] = v;
    else a.part[((size_t)split * Q + c) * a.rows + row] = v;
  }
}

// y[c][r] = sum over splits, in split order, of the partial sums.
__global__ __launch_bounds__(256) void k_dense_sum(DenseArgs a) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n = (size_t)a.q * a.rows;
  if (i >= n) return;
  float v = 0.f;
  for (int s = 0; s < a.splits; ++s) v += a.part[(size_t)s * n + i];
  a.y[i] = v;
}

// Canonical blocks -> dense image (one thread per block).
__global__ __launch_bounds__(256) void k_dense_image(int fmt, const uint8_t *__restrict__ src,
                                                    int rows, int nb, uint8_t *__restrict__ codes,
                                                    uint8_t *__restrict__ scales, int to_image,
                                                    float *__restrict__ w) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows * nb) return;
  const int r = (int)(i / nb), b = (int)(i % nb);
  const int cb = code_bytes(fmt), sb = scale_bytes(fmt), bb = cb + sb;
  const int CB = chunk_blocks(fmt), nch = nb / CB;
  const int k = b / CB, jb = b % CB;
  const size_t slot = ((size_t)(r / 64) * nch + k) * 64 + (r % 64);
  uint8_t *c = codes + slot * (CB * cb) + jb * cb;
  uint8_t *s = scales + slot * (CB * sb) + jb * sb;
  if (to_image) {
    const uint8_t *blk = src + (size_t)i * bb;
    for (int t = 0; t < cb; ++t) c[t] = blk[t];
    for (int t = 0; t < sb; ++t) s[t] = blk[cb + t];
    return;
  }
  // dequantize straight from the image, for checking its layout
  const float o = fmt == RFPX_FP2 ? 1.5f : fmt == RFPX_FP3 ? 3.5f : 7.5f;
  const float sc = fmt == RFPX_FP4 ? __builtin_ldexpf(1.0f, (int)s[0] - 127)
                                   : half_bits_to_float((uint32_t)(s[0] | (s[1] << 8)));
  float *dst = w + (size_t)r * nb * 32 + 32 * b;
  for (int j = 0; j < 32; ++j) {
    const int pos = fmt * j;
    const uint32_t two = (uint32_t)c[pos >> 3] | ((pos >> 3) + 1 < cb ? (uint32_t)c[(pos >> 3) + 1] << 8 : 0u);
    const int code = (int)((two >> (pos & 7)) & ((1u << fmt) - 1u));
    dst[j] = ((float)code - o) * sc;
  }
}

struct DensePlan {
  int nb, nch, waves, cpw, splits, vx;
  size_t codes_bytes, scales_off, image_bytes, lds, ws_total;
};

// LDS of one k_dense workgroup: prepared words, starts and wave sums.
size_t dense_lds(int q, int vx, int nbw, int waves) {
  return (size_t)q * nbw * vx * 64 + (size_t)q * nbw * 4 + (size_t)waves * q * 64 * 4;
}

rfpx_status dense_plan(int fmt, int rows, int cols, int q, int xtype, DensePlan *p) {
  if (!valid_fmt(fmt)) return fail(RFPX_E_FORMAT, "unknown format %d", fmt);
  if (rows < 64 || rows % 64 || cols < 32 || cols % 32 || cols > (1 << 16))
    return fail(RFPX_E_SHAPE, "dense %dx%d: rows a multiple of 64, cols a multiple of 32 "
                "(at most 65536)", rows, cols);
  const int nb = cols / 32, CB = chunk_blocks(fmt);
  if (nb % CB) return fail(RFPX_E_SHAPE, "dense FP2 needs cols a multiple of 64");
  if (q < 1 || q > kQMax) return fail(RFPX_E_SHAPE, "q=%d: must be in [1, %d]", q, kQMax);
  if (xtype != RFPX_X_F32 && xtype != RFPX_X_BF16) return fail(RFPX_E_ARG, "xtype=%d", xtype);
  p->nb = nb;
  p->nch = nb / CB;
  p->vx = xtype == RFPX_X_BF16 ? 1 : 2;
  const size_t nblk = (size_t)rows * nb;
  p->codes_bytes = nblk * code_bytes(fmt);
  p->scales_off = align_up(p->codes_bytes, 256);
  p->image_bytes = p->scales_off + nblk * scale_bytes(fmt);
  // waves per workgroup: at most 8 and a power of two dividing the chunks
  int waves = kDenseWavesMax;
  while (waves > 1 && p->nch % waves) waves /= 2;
  const int per_tile = p->nch / waves;  // chunk runs per wave over all splits
  const int tiles = rows / 64;
  // chunks per wave: a power of two dividing per_tile, at most
  // kDenseCpwMax, small enough that the launch has a workgroup per compute
  // unit (256) and that the workgroup's prepared activations fit in LDS;
  // the rest of a tile goes to further workgroups (splits)
  long long want = (long long)per_tile * tiles / 256;
  int cpw = kDenseCpwMax / CB;
  while (cpw > 1 && (per_tile % cpw || cpw > want ||
                     dense_lds(q, p->vx, waves * cpw * CB, waves) > kDenseLdsMax))
    cpw /= 2;
  p->waves = waves;
  p->cpw = cpw;
  p->splits = per_tile / cpw;
  p->lds = dense_lds(q, p->vx, waves * cpw * CB, waves);
  if (p->lds > kDenseLdsMax)
    return fail(RFPX_E_SHAPE, "dense %dx%d at q=%d: one chunk per wave needs %zu bytes of LDS",
                rows, cols, q, p->lds);
  p->ws_total = align_up(p->splits > 1 ? (size_t)p->splits * q * rows * 4 : 0, 256);
  return RFPX_OK;
}

template <int FMT, int VX>
void *dense_kernel(int q) {
  switch (q) {
    case 1: return reinterpret_cast<void *>(k_dense<FMT, 1, VX>);
    case 2: return reinterpret_cast<void *>(k_dense<FMT, 2, VX>);
    case 3: return reinterpret_cast<void *>(k_dense<FMT, 3, VX>);
    case 4: return reinterpret_cast<void *>(k_dense<FMT, 4, VX>);
    case 5: return reinterpret_cast<void *>(k_dense<FMT, 5, VX>);
    case 6: return reinterpret_cast<void *>(k_dense<FMT, 6, VX>);
    case 7: return reinterpret_cast<void *>(k_dense<FMT, 7, VX>);
    default: return reinterpret_cast<void *>(k_dense<FMT, 8, VX>);
  }
}

}  // namespace
}  // namespace rfpx

using namespace rfpx;

extern "C" {

size_t rfpx_dense_image_bytes(int fmt, int rows, int cols) {
  DensePlan p;
  if (dense_plan(fmt, rows, cols, 1, RFPX_X_BF16, &p)) return 0;
  return p.image_bytes;
}

static rfpx_status dense_image_kernel(const char *fn, int fmt, const uint8_t *src, int rows,
                                      int cols, uint8_t *image, int to_image, float *w,
                                      void *stream) {
  DensePlan p;
  rfpx_status st = dense_plan(fmt, rows, cols, 1, RFPX_X_BF16, &p);
  if (st) return st;
  if ((uintptr_t)image % 256) return fail(RFPX_E_ALIGN, "%s: image not 256-byte aligned", fn);
  const long long n = (long long)rows * p.nb;
  k_dense_image<<<(unsigned)((n + 255) / 256), 256, 0, (hipStream_t)stream>>>(
      fmt, src, rows, p.nb, image, image + p.scales_off, to_image, w);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "%s: %s", fn, hipGetErrorString(e));
}

rfpx_status rfpx_dense_image_build(int fmt, const uint8_t *canonical, int rows, int cols,
                                   uint8_t *image, size_t cap, void *stream) {
  if (!canonical || !image) return fail(RFPX_E_ARG, "rfpx_dense_image_build: null pointer");
  const size_t need = rfpx_dense_image_bytes(fmt, rows, cols);
  if (!need) return fail(RFPX_E_SHAPE, "rfpx_dense_image_build: unsupported %d x %d (format %d)",
                         rows, cols, fmt);
  if (cap < need)
    return fail(RFPX_E_WORKSPACE, "rfpx_dense_image_build: image holds %zu bytes, needs %zu", cap,
                need);
  return dense_image_kernel("rfpx_dense_image_build", fmt, canonical, rows, cols, image, 1,
                            nullptr, stream);
}

rfpx_status rfpx_dense_image_unpack(int fmt, const uint8_t *image, int rows, int cols, float *w,
                                    void *stream) {
  if (!image || !w) return fail(RFPX_E_ARG, "rfpx_dense_image_unpack: null pointer");
  return dense_image_kernel("rfpx_dense_image_unpack", fmt, nullptr, rows, cols,
                            const_cast<uint8_t *>(image), 0, w, stream);
}

size_t rfpx_dense_workspace_bytes(int fmt, int rows, int cols, int q) {
  DensePlan p16, p32;
  if (dense_plan(fmt, rows, cols, q, RFPX_X_BF16, &p16) ||
      dense_plan(fmt, rows, cols, q, RFPX_X_F32, &p32))
    return 0;
  // at least 256 bytes, so that a valid shape never reads as "unsupported"
  const size_t n = p16.ws_total > p32.ws_total ? p16.ws_total : p32.ws_total;
  return n > 256 ? n : 256;
}

rfpx_status rfpx_dense_forward(int fmt, const uint8_t *image, int rows, int cols, const void *x,
                               int xtype, int q, float *y, void *ws, size_t ws_bytes,
                               void *stream) {
  DensePlan p;
  rfpx_status st = dense_plan(fmt, rows, cols, q, xtype, &p);
  if (st) return st;
  if (q < 1) return fail(RFPX_E_SHAPE, "q=%d: must be in [1, %d]", q, kQMax);
  if (!image || !x || !y || !ws) return fail(RFPX_E_ARG, "rfpx_dense_forward: null pointer");
  if ((uintptr_t)image % 256 || (uintptr_t)ws % 256)
    return fail(RFPX_E_ALIGN, "rfpx_dense_forward: image and workspace must be 256-byte aligned");
  if ((uintptr_t)x % 16) return fail(RFPX_E_ALIGN, "rfpx_dense_forward: x must be 16-byte aligned");
  if (ws_bytes < p.ws_total)
    return fail(RFPX_E_WORKSPACE, "workspace holds %zu bytes, needs %zu", ws_bytes, p.ws_total);
  DenseArgs a{};
  a.codes = image;
  a.scales = image + p.scales_off;
  a.x = x;
  a.part = reinterpret_cast<float *>(ws);
  a.y = y;
  a.rows = rows;
  a.cols = cols;
  a.nb = p.nb;
  a.nch = p.nch;
  a.q = q;
  a.xtype = xtype;
  a.vx = p.vx;
  a.waves = p.waves;
  a.cpw = p.cpw;
  a.splits = p.splits;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p.vx == 1;
  void *k = fmt == RFPX_FP2 ? (bf ? dense_kernel<RFPX_FP2, 1>(q) : dense_kernel<RFPX_FP2, 2>(q))
          : fmt == RFPX_FP3 ? (bf ? dense_kernel<RFPX_FP3, 1>(q) : dense_kernel<RFPX_FP3, 2>(q))
                            : (bf ? dense_kernel<RFPX_FP4, 1>(q) : dense_kernel<RFPX_FP4, 2>(q));
  void *args[] = {&a};
  hipError_t e = hipLaunchKernel(k, dim3(rows / 64, p.splits), dim3(64 * p.waves), args, p.lds, s);
  if (e == hipSuccess && p.splits > 1) {
    const size_t n = (size_t)q * rows;
    e = launch_k(k_dense_sum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "rfpx_dense_forward: %s", hipGetErrorString(e));
}

}  // extern "C"
