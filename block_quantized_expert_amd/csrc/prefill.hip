// prefill.hip -- a prefill chunk of T tokens through one routed-MoE layer:
// tokens grouped by expert, each expert's gate/up and down products as
// dense tiles on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Page "DeepSeek V4 Flash 在 128GB 锐龙 AI MAX+ 上跑到 32 tok/s" (taozi.news),
// section "稀疏预填充": prefill is batched per layer; section "ROCmFPX":
// gate/up FP2, down FP3, the shared expert FP4.  Page "Lucebox专攻DeepSeek
// V4…" (m.mzlw.cn), section "MoE 专家并行": 256 routed experts, top-6, one
// shared expert.
//
// The per-token result is the decode path's (moe_layer_forward with one
// column per token); only the order of fp32 sums differs.  Launches:
//   k_pf_scores  router scores S = X Wr^T, fp32 products on the matrix cores.
//   k_pf_prep    prepared activations of every token and block for each
//                gate/up format present (the decode path's pair words and
//                accumulator starts, rfpx_impl.hpp).
//   k_pf_topk    sorted top-k and gating weights, one wave per token.
//   k_pf_group   one workgroup per expert: the (token, rank, weight) entries
//                that chose it, in token order (stable); the shared expert
//                takes every token at rank k with weight 1.
//   k_pf_plan    row offsets of each expert's rows of h, and the task list:
//                (expert, first row, rows) chunks of at most 128 rows, full
//                chunks first, then the rest by size (largest first).
//   k_pf_gateup  grid (f/64, tasks): a task's tokens x 64 rows of gate and
//                up.  Each wave owns 16 rows and every 16-token tile of the
//                task.  Per 32-weight block the B operand is the block's
//                decoded pair words (the same v_and_or decode as the decode
//                path; four per lane), the A operand the prepared
//                activations and the C operand the block's accumulator start,
//                so the MFMA result is sum_j (c_j - o) x_j exactly up to fp32
//                rounding; the block scale is applied in fp32 to that
//                result.  h = silu(g) * u, then prepared (bf16 hi + lo pair
//                words for the expert's down format) as rows of hp.
//   k_pf_down    grid (d/64, tasks): the down product of the task's rows of
//                h (two MFMAs per block, hi and lo), times the gating
//                weight, into out[token][rank][d].
//   k_pf_combine y[t] = sum over ranks 0..k (the shared expert last).
#include <type_traits>

#include "rfpx_route.hpp"

namespace rfpx {
namespace {

constexpr int kChunk = 64;      // rows (tokens) per task
constexpr int kPfWaves = 4;     // waves per product workgroup
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kTileGU = 64;     // gate/up rows per workgroup: 4 waves x 16 (of gate and of up)
constexpr int kTileDN = 128;    // down rows per workgroup: 4 waves x 2 x 16
constexpr int kMT = kChunk / 16;
constexpr int kXcds = 8;        // accelerator complex dies of the chip

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct PfTask {
  int expert, m0, rows, pad;
};

struct PfArgs {
  const uint8_t *image;
  size_t image_bytes;
  const float *wr;
  const void *x;
  float *y;
  int d, f, E, k, T, xtype, vx, nb_d, nb_f;
  float routed_scale;
  int rows_max, max_tasks;
  unsigned gu_fmts, dn_fmts;  // bit f: format f appears in the host table
  int fmt_slot[5];
  // workspace
  float *scores;       // [T][E]
  int32_t *ids;        // [T][k]
  float *gw;           // [T][k]
  int32_t *counts;     // [E+1]
  int32_t *ltok;       // [E+1][T]
  int32_t *lrank;      // [E+1][T]
  float *lw;           // [E+1][T]
  int32_t *offs;       // [E+2]
  int32_t *ntasks;     // [1]
  PfTask *tasks;       // [max_tasks]
  uint32_t *xp;        // [fmt slot][T][nb_d][vx][16]
  float *xnc;          // [fmt slot][nb_d][T]
  uint32_t *hp;        // [rows_max + 16][nb_f][32]
  float *hnc;          // [nb_f][rows_max + 16]
  float *out;          // [T][k+1][d]
};

// ---------------------------------------------------------------- scores

// S[t][e] = sum_i x[t][i] Wr[e][i] on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32: fp32 products, fp32 sums).  A wave owns 16
// tokens x 32 experts (two 16 x 16 tiles); a workgroup of four waves 32
// tokens x 64 experts, so its waves share each x and Wr fragment through
// L1.  The order of the k terms inside a step of 32 is free: lane (kq, col)
// takes k = 8 kq .. 8 kq + 7, i.e. 8 contiguous elements of its row, which
// it loads in one or two 16-byte reads; the next step is loaded while the
// current one runs.
template <int XT>
__device__ __forceinline__ void scores_load(const PfArgs &a, int t, int k, float *xv) {
  if (XT == RFPX_X_BF16) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.x) +
                                                      (size_t)t * a.d + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      xv[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  } else {
    const float *p = static_cast<const float *>(a.x) + (size_t)t * a.d + k;
    const floatx4 v0 = *reinterpret_cast<const floatx4 *>(p);
    const floatx4 v1 = *reinterpret_cast<const floatx4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = v0[i];
      xv[4 + i] = v1[i];
    }
  }
}

template <int XT>
__global__ __launch_bounds__(256) void k_pf_scores(PfArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kq = lane >> 4, col = lane & 15;
  const int t0 = blockIdx.y * 32 + 16 * (wave & 1), e0 = blockIdx.x * 64 + 32 * (wave >> 1);
  const int t = min(t0 + col, a.T - 1);
  const int er[2] = {min(e0 + col, a.E - 1), min(e0 + 16 + col, a.E - 1)};
  floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  // a ring of NS steps of 32: the loads of step s + NS - 1 go out while step
  // s is multiplied, so about NS - 1 steps of loads are in flight (one wave
  // per SIMD: there is no other wave to cover the latency).  d is a multiple
  // of 32 NS, and the ring index of every step is a compile-time constant.
  constexpr int NS = 4;
  float xn[NS][8], wn[NS][2][8];
  auto load = [&](int k0, float (&xb)[8], float (&wb)[2][8]) __attribute__((always_inline)) {
    const int k = k0 + 8 * kq;
    scores_load<XT>(a, t, k, xb);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const float *p = a.wr + (size_t)er[n] * a.d + k;
      const floatx4 v0 = *reinterpret_cast<const floatx4 *>(p);
      const floatx4 v1 = *reinterpret_cast<const floatx4 *>(p + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wb[n][i] = v0[i];
        wb[n][4 + i] = v1[i];
      }
    }
  };
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) load(32 * st, xn[st], wn[st]);
  for (int k0 = 0; k0 < a.d; k0 += 32 * NS) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int kn = k0 + 32 * (st + NS - 1);
      if (kn < a.d) load(kn, xn[(st + NS - 1) % NS], wn[(st + NS - 1) % NS]);
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(xn[st][s], wn[st][n][s], acc[n], 0, 0, 0);
    }
  }
  // D[4 kq + i][col]: token t0 + 4 kq + i, expert e0 + 16 n + col
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = t0 + 4 * kq + i, e = e0 + 16 * n + col;
      if (tt < a.T && e < a.E) a.scores[(size_t)tt * a.E + e] = acc[n][i];
    }
}

// ------------------------------------------------- prepared activations

// (x is 16-byte aligned and d a multiple of 128, so a block of x starts on
// a 64-byte boundary and its prepared words on a 64-byte boundary too.)
template <int FMT>
__device__ void pf_prep_item(const PfArgs &a, int slot, int t, int b) {
  uint32_t hi[32], lo[32], pw[16];
  float nc_hi, nc_lo = 0.f;
  if (a.xtype == RFPX_X_BF16) {
    const uint4 *xs = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.x) +
                                                      (size_t)t * a.d + 32 * b);
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
    const float4 *xs = reinterpret_cast<const float4 *>(static_cast<const float *>(a.x) +
                                                        (size_t)t * a.d + 32 * b);
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
  uint4 *dst = reinterpret_cast<uint4 *>(a.xp + (((size_t)slot * a.T + t) * a.nb_d + b) * a.vx * 16);
  prep_pairs<FMT>(hi, pw, &nc_hi);
#pragma unroll
  for (int v = 0; v < 4; ++v) dst[v] = uint4{pw[4 * v], pw[4 * v + 1], pw[4 * v + 2], pw[4 * v + 3]};
  if (a.vx == 2) {
    prep_pairs<FMT>(lo, pw, &nc_lo);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      dst[4 + v] = uint4{pw[4 * v], pw[4 * v + 1], pw[4 * v + 2], pw[4 * v + 3]};
  }
  a.xnc[((size_t)slot * a.nb_d + b) * a.T + t] = nc_hi + nc_lo;
}

__global__ __launch_bounds__(256) void k_pf_prep(PfArgs a) {
  const int item = blockIdx.x * 256 + threadIdx.x;
  const int per_fmt = a.T * a.nb_d;
  const int nf = __builtin_popcount(a.gu_fmts);
  if (item >= nf * per_fmt) return;
  // tokens fastest: the accumulator starts of neighbouring threads are
  // neighbours ([slot][block][token])
  const int slot = item / per_fmt, rem = item % per_fmt;
  const int b = rem / a.T, t = rem % a.T;
  int fmt = 0;
  for (int f = RFPX_FP2; f <= RFPX_FP4; ++f)
    if (((a.gu_fmts >> f) & 1u) && a.fmt_slot[f] == slot) fmt = f;
  if (fmt == RFPX_FP2) pf_prep_item<RFPX_FP2>(a, slot, t, b);
  else if (fmt == RFPX_FP3) pf_prep_item<RFPX_FP3>(a, slot, t, b);
  else if (fmt == RFPX_FP4) pf_prep_item<RFPX_FP4>(a, slot, t, b);
}

// ----------------------------------------------------------------- top-k

__global__ __launch_bounds__(512) void k_pf_topk(PfArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 8 + wave;
  if (t >= a.T) return;
  RouteParams rp;
  rp.scores = a.scores;
  rp.E = a.E;
  rp.k = a.k;
  rp.q = 1;
  rp.routed_scale = a.routed_scale;
  int32_t *ids = a.ids + (size_t)t * a.k;
  float *w = a.gw + (size_t)t * a.k;
  if (a.E <= 64) topk_wave<1>(rp, t, lane, ids, w);
  else if (a.E <= 128) topk_wave<2>(rp, t, lane, ids, w);
  else if (a.E <= 256) topk_wave<4>(rp, t, lane, ids, w);
  else if (a.E <= 512) topk_wave<8>(rp, t, lane, ids, w);
  else topk_wave<16>(rp, t, lane, ids, w);
}

// -------------------------------------------------------------- grouping

// Entries (token, rank, weight) of expert blockIdx.x in token order: chunks
// of kGroupThreads (token, rank) entries, compacted with a ballot per wave
// and the wave counts through LDS (two count buffers, one barrier per
// chunk); the ids of the next chunk are loaded while one is compacted.
constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;

__global__ __launch_bounds__(kGroupThreads) void k_pf_group(PfArgs a) {
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t *ltok = a.ltok + (size_t)e * a.T;
  int32_t *lrank = a.lrank + (size_t)e * a.T;
  float *lw = a.lw + (size_t)e * a.T;
  if (e == a.E) {  // the shared expert: every token, rank k, weight 1
    for (int t = tid; t < a.T; t += kGroupThreads) {
      ltok[t] = t;
      lrank[t] = a.k;
      lw[t] = 1.f;
    }
    if (tid == 0) a.counts[e] = a.T;
    return;
  }
  __shared__ int wcount[2][kGroupWaves];
  int base = 0;
  const int n = a.T * a.k;
  int idn = tid < n ? a.ids[tid] : -1;
  for (int j0 = 0, it = 0; j0 < n; j0 += kGroupThreads, ++it) {
    const int j = j0 + tid;
    const bool hit = idn == e;
    const int jn = j + kGroupThreads;
    idn = jn < n ? a.ids[jn] : -1;
    const uint64_t m = __ballot(hit);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    int *wc = wcount[it & 1];
    if (lane == 0) wc[wave] = __popcll(m);
    __syncthreads();
    int woff = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kGroupWaves; ++w) {
      const int c = wc[w];
      woff += w < wave ? c : 0;
      total += c;
    }
    if (hit) {
      const int pos = base + woff + before;
      ltok[pos] = j / a.k;
      lrank[pos] = j % a.k;
      lw[pos] = a.gw[j];
    }
    base += total;
  }
  if (tid == 0) a.counts[e] = base;
}

// Row offsets (exclusive scan of the counts) and the task list.  One
// workgroup of 1024 threads; experts e = tid, tid + 1024.
__global__ __launch_bounds__(1024) void k_pf_plan(PfArgs a) {
  __shared__ int cnt[1025], scan[1025], wsum[2][16], tot[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ne = a.E + 1;
  for (int e = tid; e < ne; e += 1024) cnt[e] = a.counts[e];
  __syncthreads();
  // exclusive scans of rows and of full chunks over the experts: thread i
  // holds experts 2i and 2i + 1 (ne <= 1025 <= 2048); wave scans by lane
  // shuffles, then the 16 wave totals
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  const int c0 = e0 < ne ? cnt[e0] : 0, c1 = e1 < ne ? cnt[e1] : 0;
  const int own_r = c0 + c1, own_f = c0 / kChunk + c1 / kChunk;
  int r = own_r, f = own_f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int rr = __shfl_up(r, off, 64), ff = __shfl_up(f, off, 64);
    if (lane >= off) {
      r += rr;
      f += ff;
    }
  }
  if (lane == 63) {
    wsum[0][wave] = r;
    wsum[1][wave] = f;
  }
  __syncthreads();
  if (tid == 0) {
    int sr = 0, sf = 0;
    for (int w = 0; w < 16; ++w) {
      const int vr = wsum[0][w], vf = wsum[1][w];
      wsum[0][w] = sr;
      wsum[1][w] = sf;
      sr += vr;
      sf += vf;
    }
    tot[0] = sr;
    tot[1] = sf;
  }
  __syncthreads();
  const int rex = r - own_r + wsum[0][wave], fex = f - own_f + wsum[1][wave];
  if (e0 < ne) {
    a.offs[e0] = rex;
    scan[e0] = fex;
  }
  if (e1 < ne) {
    a.offs[e1] = rex + c0;
    scan[e1] = fex + c0 / kChunk;
  }
  if (tid == 0) a.offs[ne] = tot[0];
  __syncthreads();
  const int nfull = tot[1];
  int nrem = 0;
  for (int e = 0; e < ne; ++e) nrem += (cnt[e] % kChunk) != 0;
  for (int e = tid; e < ne; e += 1024) {
    const int c = cnt[e], fc = c / kChunk, r = c % kChunk;
    for (int i = 0; i < fc; ++i) {
      PfTask t;
      t.expert = e;
      t.m0 = i * kChunk;
      t.rows = kChunk;
      t.pad = 0;
      a.tasks[scan[e] + i] = t;
    }
    if (r) {
      // rank among the remainder chunks: larger first, then lower expert
      int rank = 0;
      for (int e2 = 0; e2 < ne; ++e2) {
        const int r2 = cnt[e2] % kChunk;
        rank += r2 > r || (r2 == r && e2 < e);
      }
      PfTask t;
      t.expert = e;
      t.m0 = fc * kChunk;
      t.rows = r;
      t.pad = 0;
      a.tasks[nfull + rank] = t;
    }
  }
  if (tid == 0) a.ntasks[0] = nfull + nrem;
}

// ------------------------------------------------------ MFMA operands

// Per-lane decode of pairs 4kq..4kq+3 of one block (the B operand of a
// 16x16x32 MFMA: lane l holds k = 8(l/16) .. +7 of column l%16, i.e. pair
// words 4kq .. 4kq+3 with kq = l/16).  The shifts and masks per lane put
// each code at the mantissa position its pair has in the full-block decode
// (decode_pairs), so the prepared activations match.
template <int FMT>
struct QuadDecode {
  uint32_t sh[4], mk[4];
  uint32_t bsh;  // FP3: first bit of the lane's 64-bit window
  int word;      // code dword (FP2, FP4) or first dword - 1 (FP3) of the lane
  __device__ void init(int kq) {
    if (FMT == RFPX_FP2) {
      const bool odd = kq & 1;
      const uint32_t M0 = 0x00030003u, M1 = 0x000C000Cu, M2 = 0x00300030u;
      sh[0] = odd ? 6 : 0;
      sh[1] = odd ? 6 : 0;
      sh[2] = odd ? 12 : 0;
      sh[3] = odd ? 12 : 6;
      mk[0] = odd ? M1 : M0;
      mk[1] = odd ? M2 : M1;
      mk[2] = odd ? M0 : M2;
      mk[3] = odd ? M1 : M0;
      word = kq >> 1;
      bsh = 0;
    } else if (FMT == RFPX_FP4) {
      sh[0] = 0;
      sh[1] = 1;
      sh[2] = 5;
      sh[3] = 9;
      mk[0] = 0x000F000Fu;
      mk[1] = mk[2] = mk[3] = 0x00780078u;
      word = kq;
      bsh = 0;
    } else {
      // the lane's 64-bit window starts at bit -4, 8, 35, 64 of the block's
      // 96-bit code word (kq = 0..3); pairs 4kq..4kq+3 sit at these offsets
      // into it (selects, not a table: a per-lane table index would go to
      // scratch memory)
      const uint32_t MA = 0x00380070u, MB = 0x0070001Cu;
      sh[0] = 0;
      sh[1] = kq == 1 ? 18 : 3;
      sh[2] = kq == 1 ? 21 : kq == 2 ? 23 : 6;
      sh[3] = kq == 1 ? 24 : kq == 2 ? 26 : 9;
      mk[0] = kq == 3 ? MB : MA;
      mk[1] = kq == 3 ? MB : MA;
      mk[2] = kq >= 2 ? MB : MA;
      mk[3] = kq >= 2 ? MB : MA;
      word = kq - 1;
      bsh = kq == 0 ? 28 : kq == 1 ? 8 : kq == 2 ? 3 : 0;
    }
  }
};

// Decoded pair words of one lane from its code dwords q (1 for FP2/FP4, 3
// for FP3: the dwords at word-1 .. word+1 of the block).
template <int FMT>
__device__ __forceinline__ void decode_quad(const QuadDecode<FMT> &qd, const uint32_t *q,
                                            uint32_t one, uint32_t *pw) {
  if (FMT == RFPX_FP3) {
    const uint32_t u0 = __builtin_amdgcn_alignbit(q[1], q[0], qd.bsh);
    const uint32_t u1 = __builtin_amdgcn_alignbit(q[2], q[1], qd.bsh);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pw[j] = and_or(__builtin_amdgcn_alignbit(u1, u0, qd.sh[j]), qd.mk[j], one);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) pw[j] = and_or(q[0] >> qd.sh[j], qd.mk[j], one);
  }
}

template <int FMT>
__device__ __forceinline__ void load_quad(__amdgpu_buffer_rsrc_t r, uint32_t block_off,
                                          const QuadDecode<FMT> &qd, uint32_t *q) {
  if (FMT == RFPX_FP3) {
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)(block_off + 4 * qd.word), 0, 0);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
  } else {
    q[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(block_off + 4 * qd.word), 0, 0);
  }
}

template <int FMT>
__device__ __forceinline__ float load_block_scale(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if (FMT == RFPX_FP4) return block_scale<RFPX_FP4>(__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0));
  return block_scale<FMT>(__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t *w) {
  u32x4 v;
  v.x = w[0];
  v.y = w[1];
  v.z = w[2];
  v.w = w[3];
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ floatx4 mfma(const bf16x8 &a, const bf16x8 &b, const floatx4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------- gate / up

// Where each of a task's (at most kChunk) rows keeps its A operand and its
// accumulator starts: byte offsets of block 0 (block b adds b times the
// stride), and rows past the task's count alias a valid row.
struct PfRows {
  uint32_t a_row[kChunk];
  uint32_t nc_row[kChunk];
};

// Weight rows staged in LDS.  Every wave owns kRowsPerWave rows of B (16
// rows x NT tiles x NM matrices) and a private LDS region holding a span of
// SB consecutive blocks of each of them: the codes, then the scales, each
// loaded as whole 16-byte pieces starting at the 16-byte boundary at or
// below the span (so a row's cache lines are consumed whole, not a few
// bytes per block as in a per-lane read of the MFMA operand layout).  A row
// of the region: 16 bytes of slack (an FP3 lane reads from 4 bytes before
// its block), then the pieces; the pitch is an odd multiple of 16 bytes,
// which spreads the 16 rows one read touches over the LDS banks.
constexpr int kRowsPerWave = 32;

template <int FMT>
struct BStage {
  static constexpr int CB = FMT == RFPX_FP2 ? 8 : FMT == RFPX_FP3 ? 12 : 16;  // code bytes
  static constexpr int SBY = FMT == RFPX_FP4 ? 1 : 2;                          // scale bytes
  static constexpr int SB = FMT == RFPX_FP4 ? 8 : 16;                          // blocks per span
  static constexpr int NPC = (15 + SB * CB + 15) / 16;                        // code pieces
  static constexpr int NPS = (15 + SB * SBY + 15) / 16;                       // scale pieces
  static constexpr int P = NPC + NPS;
  static constexpr int PITCH0 = 16 + 16 * P;
  static constexpr int PITCH = (PITCH0 / 16) % 2 ? PITCH0 : PITCH0 + 16;     // bytes
  static constexpr int NB = (kRowsPerWave * P + 63) / 64;                     // b128 per lane
};
constexpr int kBRegionBytes =
    kRowsPerWave * (BStage<RFPX_FP3>::PITCH > BStage<RFPX_FP2>::PITCH
                        ? (BStage<RFPX_FP3>::PITCH > BStage<RFPX_FP4>::PITCH ? BStage<RFPX_FP3>::PITCH
                                                                             : BStage<RFPX_FP4>::PITCH)
                        : (BStage<RFPX_FP2>::PITCH > BStage<RFPX_FP4>::PITCH ? BStage<RFPX_FP2>::PITCH
                                                                             : BStage<RFPX_FP4>::PITCH));

// A staging: two buffers of chunk x rows x (words of a block + 4 of padding).
constexpr int kLdsAWords = 2 * 4 * kChunk * 20;

// Blocks per chunk of the A staging for NMT tiles of 16 rows and NA terms:
// as many as one LDS buffer holds (a power of two, at most the B span), so
// that a task of few tokens passes fewer barriers.
template <int FMT, int NA, int NMT>
struct AChunk {
  static constexpr int AWP = NA * 16 + 4;  // words per row and block (padded)
  static constexpr int CAP = kLdsAWords / 2 / (16 * NMT * AWP);
  static constexpr int KC0 = CAP >= 16 ? 16 : CAP >= 8 ? 8 : CAP >= 4 ? 4 : CAP >= 2 ? 2 : 1;
  static constexpr int KC = KC0 < BStage<FMT>::SB ? KC0 : BStage<FMT>::SB;
};

// Output tile of a grouped product over nblocks blocks of 32: the task's
// rows (16 NMT, at most kChunk) x NT 16-row tiles of NM matrices per wave.
// Software-pipelined in chunks of KC blocks: while chunk c is multiplied,
// the A words (and accumulator starts) of chunk c+1 are in flight to
// registers, to be stored to the other LDS buffer.  The B span of the
// wave's rows is refilled from registers every SB/KC chunks, and the next
// span is then requested.  NA = number of A terms per block (1, or 2 for
// bf16 hi + lo), chained through the MFMA accumulator.  NMT = number of
// 16-row tiles of A in use (a compile-time count, so that the products of a
// block issue back to back).
template <int FMT, int NM, int NT, int NA, int NMT>
__device__ __forceinline__ void pf_gemm(const PfArgs &a, int nblocks,
                                        __amdgpu_buffer_rsrc_t ar, uint32_t a_stride,
                                        __amdgpu_buffer_rsrc_t ncr, uint32_t nc_stride,
                                        const PfRows &rows, const ExpertDesc &ed, int mat0,
                                        int row0 /* first B row of this wave */, int nbB,
                                        uint32_t *lds_a, float *lds_nc, uint8_t *lds_b,
                                        floatx4 (&acc)[kMT][NT][NM]) {
  using BS = BStage<FMT>;
  static_assert(16 * NT * NM == kRowsPerWave, "a wave owns kRowsPerWave rows of B");
  static_assert(NM <= 2, "plane offsets are selected for at most two matrices");
  constexpr int KC = AChunk<FMT, NA, NMT>::KC;
  static_assert(BS::SB % KC == 0, "a B span holds whole chunks");
  constexpr int AW = NA * 16, AWP = AW + 4, V4 = AW / 4;
  constexpr int ROWS = 16 * NMT;  // A rows staged
  constexpr int PPR = KC * V4;    // 16-byte pieces of one A row per chunk (contiguous)
  constexpr int NLD = ROWS * PPR / kPfThreads;
  static_assert(NLD * kPfThreads == ROWS * PPR, "A loads must split evenly");
  static_assert(KC * ROWS <= kPfThreads, "one accumulator start per thread");
  constexpr int CPS = BS::SB / KC;  // chunks per B span
  const int tid = threadIdx.x, lane = tid & 63, kq = lane >> 4, col = lane & 15;
  QuadDecode<FMT> qd;
  qd.init(kq);
  const __amdgpu_buffer_rsrc_t img = make_rsrc(a.image, (uint32_t)a.image_bytes);
  const uint32_t rstride_c = (uint32_t)nbB * BS::CB, rstride_s = (uint32_t)nbB * BS::SBY;
  // this lane's LDS read addresses (bytes) of each (tile, matrix)
  uint32_t lc[NT][NM], ls[NT][NM];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t row = (uint32_t)(row0 + 16 * nt + col);
      const uint32_t rr = (uint32_t)(m * 16 * NT + 16 * nt + col);
      lc[nt][m] = rr * BS::PITCH + 16 + (row * rstride_c) % 16 + 4 * qd.word;
      ls[nt][m] = rr * BS::PITCH + 16 + 16 * BS::NPC + (row * rstride_s) % 16;
      // (a span of codes is a whole number of 16-byte pieces, so a row's
      // code offset in its first piece is the same for every span; the
      // scale offset of an FP4 span of 8 bytes alternates, see below)
    }
  const int nchunks = (nblocks + KC - 1) / KC;
  const int nspans = (nblocks + BS::SB - 1) / BS::SB;
  // A words (and accumulator starts) in flight two chunks ahead, in two
  // register sets: a chunk's loads go out two chunks before their LDS store,
  // so that they have two chunks of products to arrive in
  u32x4 ra0[NLD], ra1[NLD];
  float rnc0 = 0.f, rnc1 = 0.f;
  u32x4 rb[BS::NB];

  auto issue_b = [&](int sp) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < BS::NB; ++q) {
      const int item = lane + 64 * q;
      const int rr = min(item / BS::P, kRowsPerWave - 1), p = item % BS::P;
      const int row = row0 + rr % (16 * NT);
      // plane offsets of the row's matrix (selects: no indexed register array)
      const bool m1 = NM > 1 && rr >= 16 * NT;
      const uint32_t cbase = (uint32_t)(m1 ? ed.codes[mat0 + 1] : ed.codes[mat0]);
      const uint32_t sbase = (uint32_t)(m1 ? ed.scales[mat0 + 1] : ed.scales[mat0]);
      uint32_t off, span;
      int pp;
      if (p < BS::NPC) {
        off = cbase + row * rstride_c + sp * (BS::SB * BS::CB);
        span = BS::SB * BS::CB;
        pp = p;
      } else {
        off = sbase + row * rstride_s + sp * (BS::SB * BS::SBY);
        span = BS::SB * BS::SBY;
        pp = p - BS::NPC;
      }
      const bool need = item < kRowsPerWave * BS::P && 16u * pp < (off & 15u) + span;
      rb[q] = need ? __builtin_amdgcn_raw_buffer_load_b128(img, (int)((off & ~15u) + 16 * pp), 0, 0)
                   : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_b = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < BS::NB; ++q) {
      const int item = lane + 64 * q;
      const int rr = item / BS::P, p = item % BS::P;
      if (item < kRowsPerWave * BS::P)
        *reinterpret_cast<u32x4 *>(lds_b + rr * BS::PITCH + 16 + 16 * p) = rb[q];
    }
  };
  // chunk c's A loads (and accumulator starts), every load unconditional: a
  // chunk past the last re-reads the last block, and a thread without an
  // accumulator start re-reads one.  Every store of a loaded value is
  // unconditional too (a thread without an accumulator start stores it to
  // its LDS sink word): a load or a use behind a branch leaves the load
  // pending on the other path, and the compiler then waits for every load
  // in flight before the next write to its registers.
  auto issue_a = [&](int c, u32x4 (&ra)[NLD], float &rnc) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int item = tid + kPfThreads * q;
      const int r = item / PPR, pc = item % PPR;
      const int j = pc / V4, w4 = pc % V4;
      const int blk = min(c * KC + j, nblocks - 1);
      ra[q] = __builtin_amdgcn_raw_buffer_load_b128(
          ar, (int)(rows.a_row[r] + blk * a_stride + 16 * w4), 0, 0);
    }
    {
      const int t = min(tid, KC * ROWS - 1);
      const int r = t % ROWS, j = t / ROWS;
      const int blk = min(c * KC + j, nblocks - 1);
      rnc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          ncr, (int)(rows.nc_row[r] + blk * nc_stride), 0, 0));
    }
  };
  auto store_a = [&](int buf, const u32x4 (&ra)[NLD], float rnc) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int item = tid + kPfThreads * q;
      const int r = item / PPR, pc = item % PPR;
      const int j = pc / V4, w4 = pc % V4;
      *reinterpret_cast<u32x4 *>(lds_a + ((buf * KC + j) * ROWS + r) * AWP + 4 * w4) = ra[q];
    }
    // (a thread past the starts writes past both buffers' starts, inside
    // the 2 x 4 x kChunk words of the region: KC x ROWS <= kPfThreads)
    lds_nc[tid < KC * ROWS ? buf * KC * ROWS + tid : KC * ROWS + tid] = rnc;
  };

  issue_b(0);
  issue_a(0, ra0, rnc0);
  issue_a(1, ra1, rnc1);
  store_b();
  if (nspans > 1) issue_b(1);
  store_a(0, ra0, rnc0);
  __syncthreads();
  const uint32_t one = one_one_vgpr();
  // chunk c: its A words are in LDS buffer c & 1; chunk c + 1's are in
  // flight in `rnext`; chunk c + 2's loads go out into `rfree` (the set
  // chunk c came from)
  auto chunk = [&](int c, u32x4 (&rfree)[NLD], float &ncfree, const u32x4 (&rnext)[NLD],
                   const float &ncnext) __attribute__((always_inline)) {
    issue_a(c + 2, rfree, ncfree);
    const int buf = c & 1;
    const int jb0 = (c % CPS) * KC;
    // shift of this span's scales within their first piece
    const uint32_t sadd = (BS::SB * BS::SBY) % 16 ? (uint32_t)((c / CPS) * BS::SB * BS::SBY) % 16 : 0u;
    // one block: decode the B words of the wave's rows from LDS and run
    // the products of every 16-row tile of A
    auto block = [&](int j) __attribute__((always_inline)) {
      const uint32_t *la = lds_a + (buf * KC + j) * ROWS * AWP;
      const float *ln = lds_nc + (buf * KC + j) * ROWS;
      const int jb = jb0 + j;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 bop[NM];
        float bs[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const uint8_t *cp = lds_b + lc[nt][m] + jb * BS::CB;
          uint32_t q[3], pw[4];
          q[0] = *reinterpret_cast<const uint32_t *>(cp);
          if (FMT == RFPX_FP3) {
            q[1] = *reinterpret_cast<const uint32_t *>(cp + 4);
            q[2] = *reinterpret_cast<const uint32_t *>(cp + 8);
          }
          decode_quad<FMT>(qd, q, one, pw);
          bop[m] = as_bf16x8(pw);
          const uint32_t lsr = ls[nt][m] - (ls[nt][m] & 15u) + (((ls[nt][m] & 15u) + sadd) & 15u);
          const uint8_t *sp = lds_b + lsr + jb * BS::SBY;
          bs[m] = FMT == RFPX_FP4 ? block_scale<RFPX_FP4>(*sp)
                                  : block_scale<FMT>(*reinterpret_cast<const uint16_t *>(sp));
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          {
            bf16x8 av[NA];
#pragma unroll
            for (int v = 0; v < NA; ++v)
              av[v] = __builtin_bit_cast(
                  bf16x8, *reinterpret_cast<const u32x4 *>(la + (mt * 16 + col) * AWP + v * 16 + 4 * kq));
            const floatx4 cin = *reinterpret_cast<const floatx4 *>(ln + mt * 16 + 4 * kq);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              floatx4 pr = mfma(av[0], bop[m], cin);
#pragma unroll
              for (int v = 1; v < NA; ++v) pr = mfma(av[v], bop[m], pr);
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mt][nt][m][i] = fmaf(bs[m], pr[i], acc[mt][nt][m][i]);
            }
          }
        }
      }
    };
    // one loop with the chunk's block count as its trip count: a separate
    // loop for a partial last chunk made the compiler copy every
    // accumulator register into and out of the full-chunk loop at each
    // chunk (unrolling further raises the registers past two waves per SIMD
    // and measures slower)
    const int jn = min(KC, nblocks - c * KC);
#pragma unroll 1
    for (int j = 0; j < jn; ++j) block(j);
    // (stored also after the last chunk, where nobody reads that buffer: an
    // unconditional use keeps the compiler's waits for the next set exact)
    store_a((c + 1) & 1, rnext, ncnext);
    if (c + 1 < nchunks) {
      if ((c + 1) % CPS == 0) {
        // this wave has finished with its span: refill it, ask for the next
        const int sp = (c + 1) / CPS;
        store_b();
        if (sp + 1 < nspans) issue_b(sp + 1);
      }
    }
    __syncthreads();
  };
  // chunks in pairs with no test between them: for an odd chunk count (one
  // chunk: d and f are powers of two, so a count above one is even) the
  // last pair's second chunk has no blocks (its loads re-read the last
  // block and nobody reads what it stores), so that every load of a set is
  // used on every path and the compiler's waits stay exact
  for (int c = 0; c < nchunks; c += 2) {
    chunk(c, ra0, rnc0, ra1, rnc1);
    chunk(c + 1, ra1, rnc1, ra0, rnc0);
  }
}

// LDS of the prefill products: the A staging buffers (also the h tile of
// the gate/up epilogue), the accumulator starts, the B regions of the
// waves and the row table.
static_assert(kChunk * kTileGU <= kLdsAWords, "h tile fits");

struct PfLds {
  uint32_t a[kLdsAWords];
  float nc[2 * 4 * kChunk];
  uint8_t b[kPfWaves][kBRegionBytes];
  PfRows rows;
};

__device__ __forceinline__ ExpertDesc pf_desc(const PfArgs &a, int e) {
  const ExpertDesc *tab = reinterpret_cast<const ExpertDesc *>(a.image + kImgTable);
  ExpertDesc ed;
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    ed.codes[m] = uniform64(tab[e].codes[m]);
    ed.scales[m] = uniform64(tab[e].scales[m]);
    ed.fmt[m] = uniform(tab[e].fmt[m]);
  }
  ed.reserved = 0;
  return ed;
}

// Workgroup -> (task, column slice).  Workgroups are handed to the XCDs in
// turn (workgroup n to XCD n mod 8), so the slices of task t are numbered
// to land on XCD t mod 8 together: the task's A rows are then fetched into
// one L2 only.
__device__ __forceinline__ bool pf_work(const PfArgs &a, int nslices, int *task, int *slice) {
  const int n = blockIdx.x, xcd = n % kXcds, local = n / kXcds;
  const int t = xcd + kXcds * (local / nslices);
  *slice = local % nslices;
  *task = t;
  return t < a.ntasks[0];
}

// ------------------------------------------------------------- gate / up

// A workgroup covers kTileGU rows of gate and of up: each wave one 16-row
// tile of both.  After the products the h tile goes through LDS, and the
// workgroup prepares its kTileGU / 32 blocks of h for the down matrix.
template <int FMT, int VX>
__device__ __forceinline__ void pf_gateup_task(const PfArgs &a, const PfTask &tk, const ExpertDesc &ed, int slice,
                               PfLds &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kq = lane >> 4, col = lane & 15;
  const int e = tk.expert, m0 = tk.m0, cnt = tk.rows;
  const int nmt = (cnt + 15) >> 4;
  const int slot = a.fmt_slot[FMT];
  const int n0 = slice * kTileGU;
  for (int r = tid; r < kChunk; r += kPfThreads) {
    const int tok = a.ltok[(size_t)e * a.T + m0 + (r < cnt ? r : 0)];
    sm.rows.a_row[r] = (uint32_t)(((size_t)slot * a.T + tok) * a.nb_d * VX * 64);
    sm.rows.nc_row[r] = (uint32_t)(((size_t)slot * a.nb_d * a.T + tok) * 4);
  }
  __syncthreads();
  const size_t nf = __builtin_popcount(a.gu_fmts);
  const __amdgpu_buffer_rsrc_t xpr = make_rsrc(a.xp, (uint32_t)(nf * a.T * a.nb_d * VX * 64));
  const __amdgpu_buffer_rsrc_t ncr = make_rsrc(a.xnc, (uint32_t)(nf * a.nb_d * a.T * 4));
  floatx4 acc[kMT][1][2];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[mt][0][m] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int row0 = n0 + 16 * wave;
#define PF_GU(n)                                                                          \
  pf_gemm<FMT, 2, 1, VX, n>(a, a.nb_d, xpr, VX * 64, ncr, a.T * 4, sm.rows, ed, 0, row0, \
                            a.nb_d, sm.a, sm.nc, sm.b[wave], acc)
  switch (nmt) {
    case 1: PF_GU(1); break;
    case 2: PF_GU(2); break;
    case 3: PF_GU(3); break;
    default: PF_GU(4); break;
  }
#undef PF_GU
  // h tile [kChunk][kTileGU] in LDS, then h prepared for the down matrix:
  // 16 lanes per (row, block of 32)
  float *hs = reinterpret_cast<float *>(sm.a);
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
    if (mt < nmt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hs[(mt * 16 + 4 * kq + i) * kTileGU + 16 * wave + col] =
            silu(acc[mt][0][0][i]) * acc[mt][0][1][i];
  __syncthreads();
  const int fdn = ed.fmt[2];
  const int rowbase = a.offs[e] + m0;
  constexpr int kHB = kTileGU / 32;  // h blocks per workgroup
  const int p = lane & 15;
  for (int it = tid >> 4; it < cnt * kHB; it += kPfThreads / 16) {
    const int r = it / kHB, hb = it % kHB;
    const size_t hrow = (size_t)rowbase + r;
    const int fbg = n0 / 32 + hb;
    uint32_t *dst = a.hp + (hrow * a.nb_f + fbg) * 32;
    float share = prep_h_pair_rt(fdn, hs + r * kTileGU + 32 * hb, p, dst);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) share += __shfl_xor(share, off, 64);
    if (p == 0) a.hnc[(size_t)fbg * (a.rows_max + 16) + hrow] = share;
  }
}

template <int VX>
__global__ __launch_bounds__(kPfThreads) void k_pf_gateup(PfArgs a) {
  int t, slice;
  if (!pf_work(a, a.f / kTileGU, &t, &slice)) return;
  const PfTask tk = a.tasks[t];
  __shared__ __align__(16) PfLds sm;
  const ExpertDesc ed = pf_desc(a, tk.expert);
  const int fmt = ed.fmt[0];
  // a device table that disagrees with the host table: no activations were
  // prepared for an unplanned format
  if (fmt < 0 || fmt > 4 || !((a.gu_fmts >> fmt) & 1u)) return;
  if (fmt == RFPX_FP2) pf_gateup_task<RFPX_FP2, VX>(a, tk, ed, slice, sm);
  else if (fmt == RFPX_FP3) pf_gateup_task<RFPX_FP3, VX>(a, tk, ed, slice, sm);
  else pf_gateup_task<RFPX_FP4, VX>(a, tk, ed, slice, sm);
}

// ------------------------------------------------------------------- down

// A workgroup covers kTileDN rows of the down matrix: two 16-row tiles per
// wave.
template <int FMT>
__device__ __forceinline__ void pf_down_task(const PfArgs &a, const PfTask &tk, const ExpertDesc &ed, int slice,
                             PfLds &sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kq = lane >> 4, col = lane & 15;
  const int e = tk.expert, m0 = tk.m0, cnt = tk.rows;
  const int nmt = (cnt + 15) >> 4;
  const int row0 = slice * kTileDN + 32 * wave;
  const int rowbase = a.offs[e] + m0;
  for (int r = tid; r < kChunk; r += kPfThreads) {
    const size_t row = (size_t)rowbase + (r < cnt ? r : 0);
    sm.rows.a_row[r] = (uint32_t)(row * a.nb_f * 128);
    sm.rows.nc_row[r] = (uint32_t)(row * 4);
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t hpr =
      make_rsrc(a.hp, (uint32_t)((size_t)(a.rows_max + 16) * a.nb_f * 128));
  const __amdgpu_buffer_rsrc_t ncr =
      make_rsrc(a.hnc, (uint32_t)((size_t)a.nb_f * (a.rows_max + 16) * 4));
  floatx4 acc[kMT][2][1];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt][0] = floatx4{0.f, 0.f, 0.f, 0.f};
#define PF_DN(n)                                                                          \
  pf_gemm<FMT, 1, 2, 2, n>(a, a.nb_f, hpr, 128, ncr, (a.rows_max + 16) * 4, sm.rows, ed, 2, \
                           row0, a.nb_f, sm.a, sm.nc, sm.b[wave], acc)
  switch (nmt) {
    case 1: PF_DN(1); break;
    case 2: PF_DN(2); break;
    case 3: PF_DN(3); break;
    default: PF_DN(4); break;
  }
#undef PF_DN
  const int *ltok = a.ltok + (size_t)e * a.T + m0;
  const int *lrank = a.lrank + (size_t)e * a.T + m0;
  const float *lw = a.lw + (size_t)e * a.T + m0;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
    if (mt < nmt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * kq + i;
        if (r < cnt) {
          const int t = ltok[r];
          float *o = a.out + ((size_t)t * (a.k + 1) + lrank[r]) * a.d + row0 + col;
          const float w = lw[r];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) o[16 * nt] = w * acc[mt][nt][0][i];
        }
      }
}

__global__ __launch_bounds__(kPfThreads) void k_pf_down(PfArgs a) {
  int t, slice;
  if (!pf_work(a, a.d / kTileDN, &t, &slice)) return;
  const PfTask tk = a.tasks[t];
  __shared__ __align__(16) PfLds sm;
  const ExpertDesc ed = pf_desc(a, tk.expert);
  const int fmt = ed.fmt[2];
  if (fmt < 0 || fmt > 4 || !((a.dn_fmts >> fmt) & 1u)) return;
  if (fmt == RFPX_FP2) pf_down_task<RFPX_FP2>(a, tk, ed, slice, sm);
  else if (fmt == RFPX_FP3) pf_down_task<RFPX_FP3>(a, tk, ed, slice, sm);
  else pf_down_task<RFPX_FP4>(a, tk, ed, slice, sm);
}

// ---------------------------------------------------------------- combine

// Four outputs per thread (d is a multiple of 4): the loads of every rank
// are issued before the sums, which run in rank order.
__global__ __launch_bounds__(256) void k_pf_combine(PfArgs a) {
  const size_t i4 = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i4 >= (size_t)a.T * a.d / 4) return;
  const size_t t = i4 * 4 / a.d, n = i4 * 4 % a.d;
  const floatx4 *src = reinterpret_cast<const floatx4 *>(a.out + t * (a.k + 1) * a.d + n);
  const size_t rstride = (size_t)a.d / 4;
  floatx4 o[kKMax + 1];
#pragma unroll
  for (int r = 0; r <= kKMax; ++r)
    if (r <= a.k) o[r] = src[r * rstride];
  floatx4 v = o[0];
#pragma unroll
  for (int r = 1; r <= kKMax; ++r)
    if (r <= a.k)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += o[r][j];
  *reinterpret_cast<floatx4 *>(a.y + i4 * 4) = v;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

// Workspace plan of the prefill path; returns 0 for an unsupported shape.
size_t prefill_layout(const moe_layer *L, int T, int xtype, void *args_out) {
  if (T < 1 || T > 65536) return 0;
  PfArgs a{};
  a.d = L->d;
  a.f = L->f;
  a.E = L->n_experts;
  a.k = L->top_k;
  a.T = T;
  a.xtype = xtype;
  a.vx = xtype == RFPX_X_BF16 ? 1 : 2;
  a.nb_d = L->d / 32;
  a.nb_f = L->f / 32;
  a.routed_scale = L->routed_scale;
  a.rows_max = T * (L->top_k + 1);
  a.max_tasks = (L->n_experts + 1) + (a.rows_max + kChunk - 1) / kChunk;
  int nf = 0;
  for (int f = 0; f < 5; ++f) a.fmt_slot[f] = -1;
  for (int e = 0; e <= L->n_experts; ++e) {
    a.gu_fmts |= 1u << L->fmts[3 * e];
    a.dn_fmts |= 1u << L->fmts[3 * e + 2];
  }
  for (int f = RFPX_FP2; f <= RFPX_FP4; ++f)
    if ((a.gu_fmts >> f) & 1u) a.fmt_slot[f] = nf++;
  if (L->d % kTileDN || L->f % kTileGU) return 0;
  const size_t E1 = L->n_experts + 1;
  size_t off = 0;
  struct Item {
    size_t *dst;
    size_t bytes;
  };
  size_t o_scores, o_ids, o_gw, o_counts, o_ltok, o_lrank, o_lw, o_offs, o_ntasks, o_tasks,
      o_xp, o_xnc, o_hp, o_hnc, o_out;
  const Item items[] = {
      {&o_scores, (size_t)T * L->n_experts * 4},
      {&o_ids, (size_t)T * L->top_k * 4},
      {&o_gw, (size_t)T * L->top_k * 4},
      {&o_counts, E1 * 4},
      {&o_ltok, E1 * T * 4},
      {&o_lrank, E1 * T * 4},
      {&o_lw, E1 * T * 4},
      {&o_offs, (E1 + 1) * 4},
      {&o_ntasks, 4},
      {&o_tasks, (size_t)a.max_tasks * sizeof(PfTask)},
      {&o_xp, (size_t)nf * T * a.nb_d * a.vx * 64},
      {&o_xnc, (size_t)nf * a.nb_d * T * 4},
      {&o_hp, (size_t)(a.rows_max + 16) * a.nb_f * 128},
      {&o_hnc, (size_t)a.nb_f * (a.rows_max + 16) * 4},
      {&o_out, (size_t)T * (L->top_k + 1) * L->d * 4},
  };
  for (const Item &it : items) {
    *it.dst = off;
    off = align256(off + it.bytes);
  }
  // buffer resources address hp and xp with 32-bit offsets
  if ((size_t)(a.rows_max + 16) * a.nb_f * 128 > 0xFFFFFFFFull) return 0;
  if (args_out) {
    a.scores = reinterpret_cast<float *>(o_scores);
    a.ids = reinterpret_cast<int32_t *>(o_ids);
    a.gw = reinterpret_cast<float *>(o_gw);
    a.counts = reinterpret_cast<int32_t *>(o_counts);
    a.ltok = reinterpret_cast<int32_t *>(o_ltok);
    a.lrank = reinterpret_cast<int32_t *>(o_lrank);
    a.lw = reinterpret_cast<float *>(o_lw);
    a.offs = reinterpret_cast<int32_t *>(o_offs);
    a.ntasks = reinterpret_cast<int32_t *>(o_ntasks);
    a.tasks = reinterpret_cast<PfTask *>(o_tasks);
    a.xp = reinterpret_cast<uint32_t *>(o_xp);
    a.xnc = reinterpret_cast<float *>(o_xnc);
    a.hp = reinterpret_cast<uint32_t *>(o_hp);
    a.hnc = reinterpret_cast<float *>(o_hnc);
    a.out = reinterpret_cast<float *>(o_out);
    *static_cast<PfArgs *>(args_out) = a;
  }
  return off;
}

hipError_t launch_prefill(const moe_layer *L, const void *x, int xtype, int T, float *y,
                          uint8_t *ws, size_t image_bytes, hipStream_t stream,
                          void *const *events) {
  PfArgs a;
  if (!prefill_layout(L, T, xtype, &a)) return hipErrorInvalidValue;
  // turn workspace offsets into pointers
  auto rel = [ws](auto *&p) { p = reinterpret_cast<std::remove_reference_t<decltype(p)>>(ws + reinterpret_cast<uintptr_t>(p)); };
  rel(a.scores);
  rel(a.ids);
  rel(a.gw);
  rel(a.counts);
  rel(a.ltok);
  rel(a.lrank);
  rel(a.lw);
  rel(a.offs);
  rel(a.ntasks);
  rel(a.tasks);
  rel(a.xp);
  rel(a.xnc);
  rel(a.hp);
  rel(a.hnc);
  rel(a.out);
  a.image = L->image;
  a.image_bytes = image_bytes;
  a.wr = L->router_w;
  a.x = x;
  a.y = y;
  hipEvent_t *ev = (hipEvent_t *)events;
  auto evt = [ev](int i) { return ev ? ev[i] : nullptr; };
  const dim3 gsc((a.E + 63) / 64, (T + 31) / 32);
  hipError_t e = launch_k(xtype == RFPX_X_BF16 ? k_pf_scores<RFPX_X_BF16> : k_pf_scores<RFPX_X_F32>,
                          gsc, dim3(256), 0, stream, a, evt(0));
  if (e != hipSuccess) return e;
  const int nf = __builtin_popcount(a.gu_fmts);
  const size_t nprep = (size_t)nf * T * a.nb_d;
  if ((e = launch_k(k_pf_prep, dim3((unsigned)((nprep + 255) / 256)), dim3(256), 0, stream,
                    a)) != hipSuccess ||
      (e = launch_k(k_pf_topk, dim3((T + 7) / 8), dim3(512), 0, stream, a)) != hipSuccess ||
      (e = launch_k(k_pf_group, dim3(a.E + 1), dim3(kGroupThreads), 0, stream, a)) !=
          hipSuccess ||
      (e = launch_k(k_pf_plan, dim3(1), dim3(1024), 0, stream, a, nullptr, evt(1))) !=
          hipSuccess)
    return e;
  // workgroups: every task's slices, the tasks padded to a multiple of kXcds
  const int tpad = (a.max_tasks + kXcds - 1) / kXcds * kXcds;
  const int ggu = tpad * (a.f / kTileGU), gdn = tpad * (a.d / kTileDN);
  if ((e = launch_k(a.vx == 1 ? k_pf_gateup<1> : k_pf_gateup<2>, dim3(ggu), dim3(kPfThreads), 0,
                    stream, a, evt(2), evt(3))) != hipSuccess ||
      (e = launch_k(k_pf_down, dim3(gdn), dim3(kPfThreads), 0, stream, a, evt(4))) !=
          hipSuccess)
    return e;
  return launch_k(k_pf_combine, dim3((unsigned)(((size_t)T * a.d / 4 + 255) / 256)), dim3(256),
                  0, stream, a, nullptr, evt(5));
}

}  // namespace rfpx
