// codec.hip -- ROCmFP2/FP3/FP4 block codec on the GPU and the device image
// of a layer's experts.
//
// Formats: page "DeepSeek V4 Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s"
// (taozi.news), section "ROCmFPX：把 284B 权重压进 128 GB": 32 weights per
// block, FP2 10 bytes (2.50 bit/weight), FP3 ~3.50, FP4 ~4.25.  Bit layout,
// quantizer rule and image layout are the ones fixed in include/rfpx.h.
//
// All kernels here run once per model load (packing, image build) or in
// checks (unpack); one thread handles one 32-weight block.
#include <math.h>

#include "rfpx_impl.hpp"

namespace rfpx {
namespace {

constexpr int kThreads = 256;

// Code j of a block (FP2/FP3/FP4) from its little-endian code bytes.
__device__ inline int get_code(int fmt, const uint8_t *b, int j) {
  int nbit = fmt;  // 2, 3, 4 bits per code
  int pos = nbit * j;
  uint32_t two = (uint32_t)b[pos >> 3] | ((uint32_t)b[(pos >> 3) + 1] << 8);
  return (int)((two >> (pos & 7)) & ((1u << nbit) - 1u));
}

__device__ inline float code_offset_f(int fmt) {
  return fmt == RFPX_FP2 ? 1.5f : fmt == RFPX_FP3 ? 3.5f : 7.5f;
}

// double -> IEEE half bits, round to nearest even, by integer manipulation
// of the binary64 encoding.
__device__ inline uint16_t dbl_to_half_rne(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  u &= 0x7FFFFFFFFFFFFFFFull;
  int ex = (int)(u >> 52);
  uint64_t frac = u & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7FF) return (uint16_t)(sign | (frac ? 0x7E00u : 0x7C00u));
  if (ex == 0) return sign;  // zero, or a double subnormal far below 2^-25
  int E = ex - 1023;
  if (E > 15) return (uint16_t)(sign | 0x7C00u);
  uint64_t m = frac | (1ull << 52);  // value = m * 2^(E-52)
  int shift = E >= -14 ? 42 : 42 + (-14 - E);
  if (shift > 63) return sign;
  uint64_t q = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1ull);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1ull))) ++q;
  if (E >= -14) {
    if (q == 2048) {
      q = 1024;
      if (++E > 15) return (uint16_t)(sign | 0x7C00u);
    }
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024));
  }
  return (uint16_t)(sign | (uint16_t)q);  // 1024 is the smallest normal
}

// ceil(log2(v)) for a positive normal double, from its exponent and fraction.
__device__ inline int ceil_log2_pos(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  int e = (int)((u >> 52) & 0x7FF) - 1023;
  return (u & 0xFFFFFFFFFFFFFull) ? e + 1 : e;
}

template <int FMT>
__device__ inline void write_block(uint8_t *dst, const int *codes,
                                   uint32_t scale_bits) {
  constexpr int NB = FMT;
  constexpr int CB = code_bytes(FMT);
  uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    int pos = NB * j;
    uint64_t v = (uint64_t)(uint32_t)codes[j] << (pos & 31);
    words[pos >> 5] |= (uint32_t)v;
    if ((pos & 31) + NB > 32) words[(pos >> 5) + 1] |= (uint32_t)(v >> 32);
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) dst[i] = (uint8_t)(words[i >> 2] >> (8 * (i & 3)));
  if (FMT == RFPX_FP4) {
    dst[16] = (uint8_t)scale_bits;
  } else {
    dst[CB] = (uint8_t)(scale_bits & 0xFF);
    dst[CB + 1] = (uint8_t)(scale_bits >> 8);
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_pack(const float *__restrict__ w,
                                                   long long nblk,
                                                   uint8_t *__restrict__ out) {
  long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= nblk) return;
  constexpr int BB = blk_bytes(FMT);
  constexpr double O = FMT == RFPX_FP2 ? 1.5 : FMT == RFPX_FP3 ? 3.5 : 7.5;
  constexpr double CMAX = (double)((1 << FMT) - 1);
  const float *src = w + i * 32;
  float v[32];
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    v[j] = src[j];
    a = fmaxf(a, fabsf(v[j]));
  }
  uint8_t *dst = out + i * BB;
  int c[32];
  if (a == 0.f) {
#pragma unroll
    for (int j = 0; j < BB; ++j) dst[j] = 0;
    return;
  }
  if (FMT == RFPX_FP4) {
    int e = 127 + ceil_log2_pos((double)a / O);
    e = e < 1 ? 1 : (e > 254 ? 254 : e);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      double t = rint(ldexp((double)v[j], 127 - e) + O);
      c[j] = (int)fmin(fmax(t, 0.0), CMAX);
    }
    write_block<FMT>(dst, c, (uint32_t)e);
    return;
  }
  uint16_t s16 = dbl_to_half_rne((double)a / O);
  if ((s16 & 0x7FFFu) == 0x7C00u) s16 = 0x7BFF;  // clamp to 65504
  double s = (double)half_bits_to_float(s16);
  if (s == 0.0) {
#pragma unroll
    for (int j = 0; j < BB; ++j) dst[j] = 0;
    return;
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    double t = rint((double)v[j] / s + O);
    c[j] = (int)fmin(fmax(t, 0.0), CMAX);
  }
  write_block<FMT>(dst, c, s16);
}

// Importance-weighted quantizer (page "DeepSeek V4 Flash 在 128GB 锐龙 AI
// MAX+ 上跑到 32 tok/s", section "ROCmFPX": weights are quantized with an
// importance matrix).  Per block: candidate scales around the absmax one
// (FP2/FP3: fp16 of a / (o t), t = 1, 1 + 1/16, 1 - 1/16, ..., 1 +- 8/16;
// FP4: exponents e0, e0 - 1, e0 + 1), nearest codes from each stored scale,
// and the candidate of least sum_j imp_j (w_j - (c_j - o) s)^2 is kept (the
// first listed on a tie).  The error is a decision: it is evaluated in
// double with every operation rounded on its own (no fused multiply-add),
// in column order, so that the choice is reproducible bit for bit.
#pragma clang fp contract(off)
template <int FMT>
__device__ inline double wblock_error(const float *v, const float *imp, const int *c,
                                      double s) {
  constexpr double O = FMT == RFPX_FP2 ? 1.5 : FMT == RFPX_FP3 ? 3.5 : 7.5;
  double err = 0.0;
  for (int j = 0; j < 32; ++j) {
    const double d = (double)v[j] - ((double)c[j] - O) * s;
    err = err + (double)imp[j] * (d * d);
  }
  return err;
}

template <int FMT>
__device__ inline void wblock_codes(const float *v, double s, int *c) {
  constexpr double O = FMT == RFPX_FP2 ? 1.5 : FMT == RFPX_FP3 ? 3.5 : 7.5;
  constexpr double CMAX = (double)((1 << FMT) - 1);
  for (int j = 0; j < 32; ++j) c[j] = (int)fmin(fmax(rint((double)v[j] / s + O), 0.0), CMAX);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_pack_weighted(const float *__restrict__ w,
                                                            const float *__restrict__ imp,
                                                            int nb, long long nblk,
                                                            uint8_t *__restrict__ out) {
  long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= nblk) return;
  constexpr int BB = blk_bytes(FMT);
  constexpr double O = FMT == RFPX_FP2 ? 1.5 : FMT == RFPX_FP3 ? 3.5 : 7.5;
  const float *src = w + i * 32;
  const float *im = imp + (i % nb) * 32;  // the block's 32 input columns
  float v[32], a = 0.f;
  for (int j = 0; j < 32; ++j) {
    v[j] = src[j];
    a = fmaxf(a, fabsf(v[j]));
  }
  uint8_t *dst = out + i * BB;
  int c[32], best_c[32];
  double best = 0.0;
  bool have = false;
  uint32_t best_bits = 0;
  if (a != 0.f) {
    if (FMT == RFPX_FP4) {
      const int e0 = 127 + ceil_log2_pos((double)a / O);
      int seen[3], nseen = 0;
      for (int k = 0; k < 3; ++k) {
        int e = k == 0 ? e0 : k == 1 ? e0 - 1 : e0 + 1;
        e = e < 1 ? 1 : (e > 254 ? 254 : e);
        bool dup = false;
        for (int n = 0; n < nseen; ++n) dup |= seen[n] == e;
        if (dup) continue;
        seen[nseen++] = e;
        const double sc = ldexp(1.0, e - 127);
        wblock_codes<FMT>(v, sc, c);
        const double err = wblock_error<FMT>(v, im, c, sc);
        if (!have || err < best) {
          have = true;
          best = err;
          best_bits = (uint32_t)e;
          for (int j = 0; j < 32; ++j) best_c[j] = c[j];
        }
      }
    } else {
      uint16_t seen[17];
      int nseen = 0;
      for (int k = 0; k < 17; ++k) {
        const int t = (k + 1) / 2 * ((k & 1) ? 1 : -1);  // 0, 1, -1, 2, -2, ...
        uint16_t s16 = dbl_to_half_rne((double)a / (O * (1.0 + (double)t / 16.0)));
        if ((s16 & 0x7FFFu) == 0x7C00u) s16 = 0x7BFF;
        const double sc = (double)half_bits_to_float(s16);
        if (sc == 0.0) continue;
        bool dup = false;
        for (int n = 0; n < nseen; ++n) dup |= seen[n] == s16;
        if (dup) continue;
        seen[nseen++] = s16;
        wblock_codes<FMT>(v, sc, c);
        const double err = wblock_error<FMT>(v, im, c, sc);
        if (!have || err < best) {
          have = true;
          best = err;
          best_bits = s16;
          for (int j = 0; j < 32; ++j) best_c[j] = c[j];
        }
      }
    }
  }
  if (!have) {
    for (int j = 0; j < BB; ++j) dst[j] = 0;
    return;
  }
  write_block<FMT>(dst, best_c, best_bits);
}
#pragma clang fp contract(fast)

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_pack_codes(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ sbits,
    long long nblk, uint8_t *__restrict__ out) {
  long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= nblk) return;
  int c[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) c[j] = codes[i * 32 + j] & ((1 << FMT) - 1);
  uint32_t sb = sbits[i];
  if (FMT == RFPX_FP4) sb &= 0xFFu;
  write_block<FMT>(out + i * blk_bytes(FMT), c, sb);
}

// Decode blocks whose code bytes sit every code_stride bytes and whose
// scale bytes sit every scale_stride bytes: canonical blocks (both strides
// the block size) or the two planes of the device image.
__global__ __launch_bounds__(kThreads) void k_unpack(
    int fmt, const uint8_t *__restrict__ codes, int code_stride,
    const uint8_t *__restrict__ scales, int scale_stride, long long nblk,
    float *__restrict__ w) {
  long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= nblk) return;
  int cb = code_bytes(fmt);
  uint8_t cbytes[17];
  for (int j = 0; j < cb; ++j) cbytes[j] = codes[i * code_stride + j];
  cbytes[cb] = 0;
  const uint8_t *sp = scales + i * scale_stride;
  double s;
  if (fmt == RFPX_FP4)
    s = ldexp(1.0, (int)sp[0] - 127);
  else
    s = (double)half_bits_to_float((uint32_t)(sp[0] | (sp[1] << 8)));
  double o = (double)code_offset_f(fmt);
  float *dst = w + i * 32;
  for (int j = 0; j < 32; ++j)
    dst[j] = (float)(((double)get_code(fmt, cbytes, j) - o) * s);
}

// Canonical blocks of one matrix -> its codes plane and scales plane.  The
// first thread of the gate matrix of each expert also writes the expert's
// table entry; expert 0 writes the image header.
__global__ __launch_bounds__(kThreads) void k_image_matrix(
    int fmt, const uint8_t *__restrict__ src, long long nblk,
    uint8_t *__restrict__ image, uint64_t codes_off, uint64_t scales_off,
    int write_desc, int expert, ExpertDesc desc, ImageHeader hdr) {
  long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i == 0 && write_desc) {
    ExpertDesc *t = reinterpret_cast<ExpertDesc *>(image + kImgTable) + expert;
    *t = desc;
    if (expert == 0) *reinterpret_cast<ImageHeader *>(image) = hdr;
  }
  if (i >= nblk) return;
  int cb = code_bytes(fmt), sb = scale_bytes(fmt), bb = cb + sb;
  const uint8_t *s = src + i * bb;
  uint8_t *c = image + codes_off + i * cb;
  uint8_t *sc = image + scales_off + i * sb;
  for (int j = 0; j < cb; ++j) c[j] = s[j];
  for (int j = 0; j < sb; ++j) sc[j] = s[cb + j];
}

// ------------------------------------------------------------ validation
// The host format table travels in the kernel arguments, two bits per
// matrix (format - 2): 3 (E + 1) <= 3075 entries fit in 193 words.
constexpr int kFmtWords = (3 * (kEMax + 1) * 2 + 31) / 32;

struct ValArgs {
  const uint8_t *image;
  uint32_t *report;
  size_t image_bytes;
  int d, f, E;
  uint32_t fmt_bits[kFmtWords];
};

__device__ __forceinline__ int val_fmt(const ValArgs &a, int i) {
  return RFPX_FP2 + (int)((a.fmt_bits[i >> 4] >> (2 * (i & 15))) & 3u);
}

// Bytes entry i = 3 e + m of the layout occupies: its codes plane and its
// scales plane, each rounded up to 256 bytes (the layout of image_layout).
__device__ __forceinline__ uint64_t val_entry_bytes(const ValArgs &a, int i) {
  const int fmt = val_fmt(a, i), m = i % 3;
  const uint64_t rows = m < 2 ? a.f : a.d, cols = m < 2 ? a.d : a.f;
  const uint64_t nblk = rows * (cols / 32);
  return align_up(nblk * code_bytes(fmt), 256) + align_up(nblk * scale_bytes(fmt), 256);
}

// Start of entry i (its codes plane) in the layout of the host table: the
// table's aligned end plus the bytes of entries 0..i-1, summed by the
// workgroup.  All threads must call it; it ends with a barrier.
__device__ uint64_t val_entry_start(const ValArgs &a, int i, uint64_t *red) {
  uint64_t part = 0;
  for (int j = threadIdx.x; j < i; j += blockDim.x) part += val_entry_bytes(a, j);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  uint64_t tot = align_up(kImgTable + (uint64_t)(a.E + 1) * sizeof(ExpertDesc), 256);
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) tot += red[w];
  __syncthreads();
  return tot;
}

// Header and expert table (one workgroup): report[0] header faults,
// report[1] mismatching table entries; clears report[2], report[3] for the
// scale scan that follows on the same stream.  Each thread walks a
// contiguous run of entries, starting from the sum of the runs below it.
__global__ __launch_bounds__(kThreads) void k_validate_head(ValArgs a) {
  __shared__ uint64_t run_bytes[kThreads];
  __shared__ uint32_t bad;
  const int tid = threadIdx.x, n = 3 * (a.E + 1);
  const int per = (n + kThreads - 1) / kThreads, i0 = tid * per, i1 = min(n, i0 + per);
  uint64_t mine = 0;
  for (int i = i0; i < i1; ++i) mine += val_entry_bytes(a, i);
  run_bytes[tid] = mine;
  if (tid == 0) bad = 0;
  __syncthreads();
  uint64_t off = align_up(kImgTable + (uint64_t)(a.E + 1) * sizeof(ExpertDesc), 256);
  for (int t = 0; t < tid; ++t) off += run_bytes[t];
  const ExpertDesc *tab = reinterpret_cast<const ExpertDesc *>(a.image + kImgTable);
  uint32_t mis = 0;
  for (int i = i0; i < i1; ++i) {
    const int e = i / 3, m = i % 3, fmt = val_fmt(a, i);
    const uint64_t rows = m < 2 ? a.f : a.d, cols = m < 2 ? a.d : a.f;
    const uint64_t codes = off, scales = align_up(off + rows * (cols / 32) * code_bytes(fmt), 256);
    if (tab[e].fmt[m] != fmt || tab[e].codes[m] != codes || tab[e].scales[m] != scales) ++mis;
    off += val_entry_bytes(a, i);
  }
  if (mis) atomicAdd(&bad, mis);
  __syncthreads();
  if (tid == 0) {
    const ImageHeader *h = reinterpret_cast<const ImageHeader *>(a.image);
    uint32_t hf = 0;
    if (h->magic != kMagic) hf |= 1u;
    if (h->version != kVersion) hf |= 2u;
    if (h->d != a.d || h->f != a.f || h->E != a.E) hf |= 4u;
    if (h->total != a.image_bytes) hf |= 8u;
    a.report[0] = hf;
    a.report[1] = bad;
    a.report[2] = 0;
    a.report[3] = 0;
  }
}

// Scales of entry blockIdx.y (at the offset the host table implies), part
// blockIdx.x of gridDim.x: counts fp16 Inf/NaN (FP2/FP3) or E8M0 = 255
// (FP4) into report[2].  Planes are 256-byte aligned and read as words;
// the tail past the last whole word is read bytewise.
__global__ __launch_bounds__(kThreads) void k_validate_scales(ValArgs a) {
  __shared__ uint64_t red[kThreads / 64];
  const int i = blockIdx.y, fmt = val_fmt(a, i), m = i % 3;
  const uint64_t rows = m < 2 ? a.f : a.d, cols = m < 2 ? a.d : a.f;
  const uint64_t nblk = rows * (cols / 32);
  const uint64_t start = val_entry_start(a, i, red);
  const uint8_t *sp = a.image + align_up(start + nblk * code_bytes(fmt), 256);
  const uint64_t nbytes = nblk * scale_bytes(fmt), nwords = nbytes / 4;
  const uint32_t *w = reinterpret_cast<const uint32_t *>(sp);
  uint32_t cnt = 0;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t j = (uint64_t)blockIdx.x * kThreads + threadIdx.x; j < nwords; j += stride) {
    const uint32_t v = w[j];
    if (fmt == RFPX_FP4) {
#pragma unroll
      for (int b = 0; b < 4; ++b) cnt += ((v >> (8 * b)) & 0xFFu) == 0xFFu;
    } else {
      cnt += (v & 0x7C00u) == 0x7C00u;
      cnt += (v & 0x7C000000u) == 0x7C000000u;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (uint64_t b = nwords * 4; b < nbytes; b += scale_bytes(fmt)) {
      if (fmt == RFPX_FP4) cnt += sp[b] == 0xFFu;
      else cnt += ((sp[b] | (sp[b + 1] << 8)) & 0x7C00) == 0x7C00;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
  if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(&a.report[2], cnt);
}

unsigned grid_for(long long n) { return (unsigned)((n + kThreads - 1) / kThreads); }

rfpx_status check_matrix(int fmt, int rows, int cols) {
  if (!valid_fmt(fmt)) return fail(RFPX_E_FORMAT, "unknown format %d", fmt);
  if (rows < 0 || cols < 0 || cols % 32)
    return fail(RFPX_E_SHAPE, "matrix %dx%d: cols must be a multiple of 32",
                rows, cols);
  return RFPX_OK;
}

}  // namespace
}  // namespace rfpx

using namespace rfpx;

extern "C" {

size_t rfpx_block_bytes(int fmt) {
  return valid_fmt(fmt) ? (size_t)blk_bytes(fmt) : 0;
}

size_t rfpx_matrix_bytes(int fmt, int rows, int cols) {
  if (!valid_fmt(fmt) || rows < 0 || cols < 0 || cols % 32) return 0;
  return (size_t)rows * (size_t)(cols / 32) * (size_t)blk_bytes(fmt);
}

rfpx_status rfpx_pack(int fmt, const float *w, int rows, int cols, uint8_t *out,
                      size_t cap, void *stream) {
  rfpx_status st = check_matrix(fmt, rows, cols);
  if (st) return st;
  long long nblk = (long long)rows * (cols / 32);
  if (nblk == 0) return RFPX_OK;
  if (!w || !out) return fail(RFPX_E_ARG, "rfpx_pack: null pointer");
  if (cap < rfpx_matrix_bytes(fmt, rows, cols))
    return fail(RFPX_E_WORKSPACE, "rfpx_pack: output holds %zu bytes, needs %zu",
                cap, rfpx_matrix_bytes(fmt, rows, cols));
  hipStream_t s = (hipStream_t)stream;
  switch (fmt) {
    case RFPX_FP2: k_pack<RFPX_FP2><<<grid_for(nblk), kThreads, 0, s>>>(w, nblk, out); break;
    case RFPX_FP3: k_pack<RFPX_FP3><<<grid_for(nblk), kThreads, 0, s>>>(w, nblk, out); break;
    default: k_pack<RFPX_FP4><<<grid_for(nblk), kThreads, 0, s>>>(w, nblk, out); break;
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "rfpx_pack: %s", hipGetErrorString(e));
}

rfpx_status rfpx_pack_weighted(int fmt, const float *w, const float *imp, int rows, int cols,
                               uint8_t *out, size_t cap, void *stream) {
  rfpx_status st = check_matrix(fmt, rows, cols);
  if (st) return st;
  long long nblk = (long long)rows * (cols / 32);
  if (nblk == 0) return RFPX_OK;
  if (!w || !imp || !out) return fail(RFPX_E_ARG, "rfpx_pack_weighted: null pointer");
  if (cap < rfpx_matrix_bytes(fmt, rows, cols))
    return fail(RFPX_E_WORKSPACE, "rfpx_pack_weighted: output holds %zu bytes, needs %zu", cap,
                rfpx_matrix_bytes(fmt, rows, cols));
  hipStream_t s = (hipStream_t)stream;
  const int nb = cols / 32;
  switch (fmt) {
    case RFPX_FP2: k_pack_weighted<RFPX_FP2><<<grid_for(nblk), kThreads, 0, s>>>(w, imp, nb, nblk, out); break;
    case RFPX_FP3: k_pack_weighted<RFPX_FP3><<<grid_for(nblk), kThreads, 0, s>>>(w, imp, nb, nblk, out); break;
    default: k_pack_weighted<RFPX_FP4><<<grid_for(nblk), kThreads, 0, s>>>(w, imp, nb, nblk, out); break;
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "rfpx_pack_weighted: %s", hipGetErrorString(e));
}

rfpx_status rfpx_pack_codes(int fmt, const uint8_t *codes, const uint16_t *sbits,
                            int rows, int cols, uint8_t *out, size_t cap,
                            void *stream) {
  rfpx_status st = check_matrix(fmt, rows, cols);
  if (st) return st;
  long long nblk = (long long)rows * (cols / 32);
  if (nblk == 0) return RFPX_OK;
  if (!codes || !sbits || !out) return fail(RFPX_E_ARG, "rfpx_pack_codes: null pointer");
  if (cap < rfpx_matrix_bytes(fmt, rows, cols))
    return fail(RFPX_E_WORKSPACE, "rfpx_pack_codes: output too small");
  hipStream_t s = (hipStream_t)stream;
  switch (fmt) {
    case RFPX_FP2: k_pack_codes<RFPX_FP2><<<grid_for(nblk), kThreads, 0, s>>>(codes, sbits, nblk, out); break;
    case RFPX_FP3: k_pack_codes<RFPX_FP3><<<grid_for(nblk), kThreads, 0, s>>>(codes, sbits, nblk, out); break;
    default: k_pack_codes<RFPX_FP4><<<grid_for(nblk), kThreads, 0, s>>>(codes, sbits, nblk, out); break;
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "rfpx_pack_codes: %s", hipGetErrorString(e));
}

rfpx_status rfpx_unpack(int fmt, const uint8_t *in, int rows, int cols, float *w,
                        void *stream) {
  rfpx_status st = check_matrix(fmt, rows, cols);
  if (st) return st;
  long long nblk = (long long)rows * (cols / 32);
  if (nblk == 0) return RFPX_OK;
  if (!in || !w) return fail(RFPX_E_ARG, "rfpx_unpack: null pointer");
  int bb = blk_bytes(fmt), cb = code_bytes(fmt);
  k_unpack<<<grid_for(nblk), kThreads, 0, (hipStream_t)stream>>>(fmt, in, bb, in + cb, bb,
                                                                 nblk, w);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "rfpx_unpack: %s", hipGetErrorString(e));
}

size_t moe_image_bytes(int d, int f, int n_experts, const int *fmts) {
  if (!fmts || d <= 0 || f <= 0 || d % 32 || f % 32 || n_experts < 1 ||
      n_experts > kEMax)
    return 0;
  for (int i = 0; i < 3 * (n_experts + 1); ++i)
    if (!valid_fmt(fmts[i])) return 0;
  return image_layout(d, f, n_experts, fmts, nullptr);
}

rfpx_status moe_image_build(int d, int f, int n_experts, const int *fmts,
                            const uint8_t *const *canonical, uint8_t *image,
                            size_t cap, void *stream) {
  if (!fmts || !canonical || !image) return fail(RFPX_E_ARG, "moe_image_build: null pointer");
  size_t need = moe_image_bytes(d, f, n_experts, fmts);
  if (!need) return fail(RFPX_E_SHAPE, "moe_image_build: bad d=%d f=%d E=%d or format table", d, f, n_experts);
  if ((uintptr_t)image % 256) return fail(RFPX_E_ALIGN, "moe_image_build: image not 256-byte aligned");
  if (cap < need) return fail(RFPX_E_WORKSPACE, "moe_image_build: image holds %zu bytes, needs %zu", cap, need);
  for (int e = 0; e <= n_experts; ++e)
    if (fmts[3 * e] != fmts[3 * e + 1])
      return fail(RFPX_E_FORMAT, "moe_image_build: expert %d gate/up formats differ", e);
  for (int i = 0; i < 3 * (n_experts + 1); ++i)
    if (!canonical[i]) return fail(RFPX_E_ARG, "moe_image_build: canonical[%d] is null", i);
  ExpertDesc *desc = new ExpertDesc[n_experts + 1];
  image_layout(d, f, n_experts, fmts, desc);
  ImageHeader hdr{};
  hdr.magic = kMagic;
  hdr.version = kVersion;
  hdr.d = d;
  hdr.f = f;
  hdr.E = n_experts;
  hdr.total = need;
  hipStream_t s = (hipStream_t)stream;
  hipError_t err = hipSuccess;
  for (int e = 0; e <= n_experts && err == hipSuccess; ++e) {
    for (int m = 0; m < 3; ++m) {
      int fmt = fmts[3 * e + m];
      int rows = m < 2 ? f : d, cols = m < 2 ? d : f;
      long long nblk = (long long)rows * (cols / 32);
      k_image_matrix<<<grid_for(nblk), kThreads, 0, s>>>(
          fmt, canonical[3 * e + m], nblk, image, desc[e].codes[m],
          desc[e].scales[m], m == 0, e, desc[e], hdr);
      err = hipGetLastError();
      if (err != hipSuccess) break;
    }
  }
  delete[] desc;
  return err == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "moe_image_build: %s", hipGetErrorString(err));
}

rfpx_status moe_image_validate(const moe_layer *L, uint32_t *report, void *stream) {
  rfpx_status st = check_layer(L);
  if (st) return st;
  if ((st = check_image(L))) return st;
  if (!report) return fail(RFPX_E_ARG, "moe_image_validate: report is null");
  if ((uintptr_t)report % 4) return fail(RFPX_E_ALIGN, "moe_image_validate: report not 4-byte aligned");
  ValArgs a{};
  a.image = L->image;
  a.report = report;
  a.image_bytes = L->image_bytes;
  a.d = L->d;
  a.f = L->f;
  a.E = L->n_experts;
  const int n = 3 * (L->n_experts + 1);
  for (int i = 0; i < n; ++i)
    a.fmt_bits[i >> 4] |= (uint32_t)(L->fmts[i] - RFPX_FP2) << (2 * (i & 15));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_k(k_validate_head, dim3(1), dim3(kThreads), 0, s, a);
  // enough parts per plane that the scan spreads over the device
  const int parts = n >= 512 ? 4 : n >= 64 ? 16 : 64;
  if (e == hipSuccess)
    e = launch_k(k_validate_scales, dim3(parts, n), dim3(kThreads), 0, s, a);
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "moe_image_validate: %s", hipGetErrorString(e));
}

rfpx_status moe_image_unpack(const moe_layer *L, int expert, int matrix, float *w,
                             void *stream) {
  rfpx_status st = check_layer(L);
  if (st) return st;
  if ((st = check_image(L))) return st;
  if (!w) return fail(RFPX_E_ARG, "moe_image_unpack: null pointer");
  if (expert < 0 || expert > L->n_experts || matrix < 0 || matrix > 2)
    return fail(RFPX_E_ARG, "moe_image_unpack: expert %d matrix %d out of range", expert, matrix);
  ExpertDesc *desc = new ExpertDesc[L->n_experts + 1];
  image_layout(L->d, L->f, L->n_experts, L->fmts, desc);
  int fmt = L->fmts[3 * expert + matrix];
  int rows = matrix < 2 ? L->f : L->d, cols = matrix < 2 ? L->d : L->f;
  long long nblk = (long long)rows * (cols / 32);
  k_unpack<<<grid_for(nblk), kThreads, 0, (hipStream_t)stream>>>(
      fmt, L->image + desc[expert].codes[matrix], code_bytes(fmt),
      L->image + desc[expert].scales[matrix], scale_bytes(fmt), nblk, w);
  delete[] desc;
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "moe_image_unpack: %s", hipGetErrorString(e));
}

}  // extern "C"
