// measure.hip -- a plain streaming read, the achievable HBM ceiling that the
// layer kernels are compared with (page "Lucebox专攻DeepSeek V4…"
// (m.mzlw.cn), section "新手常见疑问": decode is bound by memory bandwidth).
//
// k_stream_read: every thread reads 16-byte pieces at a grid stride, eight
// loads in flight before any use, and folds them with XOR; the lanes of a
// wave and the waves of a workgroup fold their words too, and workgroup w
// writes its word to sink[w] (so the read cannot be optimized away, and the
// result is checkable: the XOR of the sink words is the XOR of every 32-bit
// word of the buffer).  Loads go through a buffer resource per batch, so the
// pieces past the end of the buffer read as zero.
#include "rfpx_impl.hpp"

namespace rfpx {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int kReadSinkWords = 2048;  // at most one word per workgroup

__global__ __launch_bounds__(kReadThreads) void k_stream_read(const uint8_t *src, uint64_t bytes,
                                                             uint32_t *sink) {
  const uint64_t pieces = bytes / 16;
  const uint64_t nthreads = (uint64_t)gridDim.x * kReadThreads;
  const uint64_t t = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  // pieces t, t + n, t + 2n, ...: eight at a time, each batch relative to
  // its own buffer resource (byte offsets below 4 GiB within a batch)
  for (uint64_t base = 0; base < pieces; base += kReadUnroll * nthreads) {
    const uint64_t first = base * 16;
    const uint64_t span = bytes - first;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(src + first, (uint32_t)(span < 0xFFFFFFF0ull ? span : 0xFFFFFFF0ull));
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int i = 0; i < kReadUnroll; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((t + i * nthreads) * 16), 0, 0);
#pragma unroll
    for (int i = 0; i < kReadUnroll; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
    for (int i = 0; i < kReadThreads / 64; ++i) w ^= part[i];
    sink[blockIdx.x] = w;
  }
}

}  // namespace
}  // namespace rfpx

using namespace rfpx;

extern "C" {

size_t rfpx_stream_read_sink_words(void) { return kReadSinkWords; }

rfpx_status rfpx_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink) return fail(RFPX_E_ARG, "rfpx_stream_read: null pointer");
  if (bytes == 0 || bytes % 16 || (uintptr_t)src % 16)
    return fail(RFPX_E_ALIGN, "rfpx_stream_read: bytes and src must be non-zero multiples of 16");
  if ((uintptr_t)sink % 4) return fail(RFPX_E_ALIGN, "rfpx_stream_read: sink not 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  // enough workgroups to keep eight loads in flight per thread over the
  // device (at most 2048 workgroups of 256 threads: 64 MiB per batch of
  // eight); sink words past the workgroup count are left as they are
  const uint64_t pieces = bytes / 16;
  uint64_t wg = (pieces + kReadThreads * kReadUnroll - 1) / (kReadThreads * kReadUnroll);
  if (wg > kReadSinkWords) wg = kReadSinkWords;
  k_stream_read<<<(unsigned)wg, kReadThreads, 0, s>>>(static_cast<const uint8_t *>(src), bytes,
                                                     sink);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? RFPX_OK : fail(RFPX_E_HIP, "rfpx_stream_read: %s", hipGetErrorString(e));
}

}  // extern "C"
