// The small kernels around the split-KV decode: query absorption, LSE
// combine, W_UV up-projection, YaRN RoPE and the cache append.
//
// Pages cited: "mHC+MLA+MTP 是什么？拆开给 Agent 用的百亿 MoE", MLA section
// (kv_b_proj: latent -> per-head [k_nope | v]; kv_a_proj_with_mqa output
// cached as latent + rope; YaRN rope) and "256K 长上下文真能本地用", §一
// (rope_scaling fields, attention_bias false).
#include "mla_internal.h"

#include <algorithm>

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 in one rounding, to nearest, ties to even (finite, normal range).
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x00000FFFFFFFFFFFull + lsb;              // (1 << 44) - 1 + lsb
  u &= ~0x00001FFFFFFFFFFFull;                   // keep 7 fraction bits
  const float f = (float)__longlong_as_double((long long)u);   // exact
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// ---------------------------------------------------------------------------
// Query absorption: Q_abs[r][0:512] = bf16(W_UK[h]^T q_nope[r]),
// Q_abs[r][512:576] = q_pe[r], for rows r = (b, j, h).  The fp32 residual
// q_lat - bf16(q_lat) is kept for the first-order LSE correction in the
// up-projection kernel.
// W_UK[h] = w_kv_b rows [h*256, h*256 + 128).  A workgroup covers (head,
// 64-column block, 4 query rows): thread (ng, c8) loads the 4 x 8 weights
// W_UK[h][4ng .. 4ng+3][c8*8 .. c8*8+7] as four 16-byte loads, forms the
// partial dot products of its 4 rows over those 4 nope dims, and the 32
// partials of each output are summed through LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kAbsorbRows = 4;

__global__ void __launch_bounds__(256) absorb_query(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ q_pe,
                                                     const uint16_t* __restrict__ w_kv_b,
                                                     uint16_t* __restrict__ qabs,
                                                     float* __restrict__ qres,
                                                     uint8_t* __restrict__ zero_row, int rows_bs) {
  __shared__ float red[kAbsorbRows][32][64];
  const int cblk = blockIdx.x;          // 8 blocks of 64 latent columns
  const int h = blockIdx.y;
  const int r0 = blockIdx.z * kAbsorbRows;
  const int t = threadIdx.x;
  if (cblk == 0 && h == 0 && r0 == 0 && t < kChunksPerRow)   // the decode kernel's zero row
    ((uint4*)zero_row)[t] = make_uint4(0, 0, 0, 0);
  const int c8 = t & 7, ng = t >> 3;
  const uint16_t* wk = w_kv_b + ((size_t)h * kWRowsPerHead + 4 * ng) * kLatent + cblk * 64 + c8 * 8;
  uint4 w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = *(const uint4*)(wk + (size_t)k * kLatent);
  uint2 q[kAbsorbRows];
#pragma unroll
  for (int rr = 0; rr < kAbsorbRows; ++rr) {
    const int r = min(r0 + rr, rows_bs - 1);
    q[rr] = *(const uint2*)(q_nope + ((size_t)r * kHeads + h) * kNope + 4 * ng);
  }
#pragma unroll
  for (int rr = 0; rr < kAbsorbRows; ++rr) {
    const float qv[4] = {__uint_as_float(q[rr].x << 16), __uint_as_float(q[rr].x & 0xFFFF0000u),
                         __uint_as_float(q[rr].y << 16), __uint_as_float(q[rr].y & 0xFFFF0000u)};
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t wd[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(qv[k], __uint_as_float(wd[e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(qv[k], __uint_as_float(wd[e] & 0xFFFF0000u), acc[2 * e + 1]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rr][ng][c8 * 8 + e] = acc[e];
  }
  __syncthreads();
  const int rr = t >> 6, col = t & 63;
  const int r = r0 + rr;
  if (r >= rows_bs) return;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) acc += red[rr][k][col];
  const size_t row = (size_t)r * kHeads + h;
  uint16_t* dst = qabs + row * kRow;
  const uint16_t qb = f32_to_bf16(acc);
  dst[cblk * 64 + col] = qb;
  qres[row * kLatent + cblk * 64 + col] = acc - bf16_to_f32(qb);
  if (cblk == 0) dst[kLatent + col] = q_pe[row * kRope + col];   // the rope part, copied
}

// ---------------------------------------------------------------------------
// LSE combine of the split partials.  One workgroup per (sequence b, row
// group of 16 rows, 16-column block); its waves take every W-th split
// (W = waves in the workgroup), reading the partials in their own layout
// (lane holds rows 4g..4g+3 of column n16) eight splits at a time, and keep
// a running max per row.  The waves' results are merged in a fixed order,
// so the combine is deterministic.
//   o_lat[row] = sum_i 2^(lse_i - M) O_i / sum_i 2^(lse_i - M)
//   lse2[row]  = M + log2 sum_i 2^(lse_i - M)   (log2 units)
// A split whose rows see no token has lse_i = -inf and weight 0.
// ---------------------------------------------------------------------------
constexpr int kCombineMaxWaves = 16;
constexpr int kCombineBatch = 8;

__global__ void __launch_bounds__(1024) lse_combine(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    const int32_t* __restrict__ ctx_lens, int Sq,
                                                    int splits, int kv_chunk, float* __restrict__ o_lat,
                                                    float* __restrict__ lse2_out) {
  __shared__ f32x4 red_o[kCombineMaxWaves][64];
  __shared__ f32x4 red_m[kCombineMaxWaves][4];
  __shared__ f32x4 red_w[kCombineMaxWaves][4];
  const int cbm = blockIdx.x;           // 32 column blocks of 16
  const int rgg = blockIdx.y;           // row group in [0, 2*Sq)
  const int b = blockIdx.z;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, n16 = lane & 15;
  const int RGT = 2 * Sq;
  const int L = ctx_lens[b];
  const int nsplit = min(splits, (L + kv_chunk - 1) / kv_chunk);
  const size_t lse_stride = (size_t)Sq * 32;
  const float* lse_base = part_lse + (size_t)b * splits * lse_stride + rgg * 16 + 4 * g;
  const float* o_base = part_o + (((size_t)b * splits * RGT + rgg) * 32 + cbm) * 256 + lane * 4;
  const size_t o_stride = (size_t)RGT * 32 * 256;

  f32x4 m = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
  f32x4 wsum = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < nsplit; s0 += nw * kCombineBatch) {
    f32x4 l4[kCombineBatch], o4[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int s = min(s0 + k * nw, nsplit - 1);   // past the end: re-read, weight 0 below
      l4[k] = *(const f32x4*)(lse_base + s * lse_stride);
      o4[k] = *(const f32x4*)(o_base + s * o_stride);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch in flight before the first use
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
      if (s0 + k * nw >= nsplit) l4[k] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bm = m[i];
#pragma unroll
      for (int k = 0; k < kCombineBatch; ++k) bm = fmaxf(bm, l4[k][i]);
      const float sc = (m[i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m[i] - bm);
      wsum[i] *= sc;
      acc[i] *= sc;
      m[i] = bm;
#pragma unroll
      for (int k = 0; k < kCombineBatch; ++k) {
        const float wt = (l4[k][i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(l4[k][i] - bm);
        wsum[i] += wt;
        acc[i] = fmaf(wt, o4[k][i], acc[i]);
      }
    }
  }
  red_o[wave][lane] = acc;
  if (n16 == 0) {
    red_m[wave][g] = m;
    red_w[wave][g] = wsum;
  }
  __syncthreads();
  if (wave != 0) return;
  f32x4 M = red_m[0][g];
  for (int w = 1; w < nw; ++w) {
    const f32x4 t = red_m[w][g];
#pragma unroll
    for (int i = 0; i < 4; ++i) M[i] = fmaxf(M[i], t[i]);
  }
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f}, ws = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < nw; ++w) {
    const f32x4 tm = red_m[w][g], tw = red_w[w][g], to = red_o[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sc = (tm[i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(tm[i] - M[i]);
      ws[i] = fmaf(tw[i], sc, ws[i]);
      o[i] = fmaf(to[i], sc, o[i]);
    }
  }
  const int j = rgg >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const int h = (rgg & 1) * 16 + r;
    const size_t row = ((size_t)b * Sq + j) * kHeads + h;
    o_lat[row * kLatent + cbm * 16 + n16] = (ws[i] > 0.f) ? o[i] / ws[i] : 0.f;
    if (cbm == 0 && n16 == 0) lse2_out[row] = (ws[i] > 0.f) ? M[i] + __log2f(ws[i]) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// W_UV up-projection: out[r][v] = bf16(sum_c W_UV[h][v][c] o_lat[r][c]),
// W_UV[h] = w_kv_b rows [h*256 + 128, h*256 + 256).  A workgroup covers
// (head, 16 output dims, 4 query rows); 16 lanes split each 512-long dot
// product, and every load of the workgroup is issued before the first FMA.
//
// The workgroup of output block 0 also writes the natural-log LSE.  Scores
// were taken with the bf16-rounded absorbed query; the exact score differs
// by scale * (q_lat - bf16(q_lat)) . c_t, so to first order the LSE moves by
// the softmax mean of that difference, scale * qres . o_lat.
// ---------------------------------------------------------------------------
constexpr int kUpRows = 4;

__global__ void __launch_bounds__(256) upproject(const float* __restrict__ o_lat,
                                                 const uint16_t* __restrict__ w_kv_b,
                                                 const float* __restrict__ qres,
                                                 const float* __restrict__ lse2, float scale_log2,
                                                 uint16_t* __restrict__ out, float* __restrict__ lse,
                                                 int rows_bs) {
  const int vblk = blockIdx.x;          // 8 blocks of 16 output dims
  const int h = blockIdx.y;
  const int r0 = blockIdx.z * kUpRows;
  const int vl = threadIdx.x >> 4;
  const int v = vblk * 16 + vl;
  const int part = threadIdx.x & 15;    // columns [part*32, part*32 + 32)
  const uint16_t* wrow = w_kv_b + ((size_t)h * kWRowsPerHead + kNope + v) * kLatent + part * 32;
  // workgroups of output block 0 also finish the LSE: lanes of output dim vl
  // take row r0 + (vl & 3)
  const bool lse_wg = (lse != nullptr) && vblk == 0;
  const int rc = r0 + (vl & (kUpRows - 1));
  const size_t crow = (size_t)min(rc, rows_bs - 1) * kHeads + h;

  uint4 wu[4];
  float4 x[kUpRows][8];
  float4 qr[8];
  float l2 = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) wu[k] = *(const uint4*)(wrow + 8 * k);
#pragma unroll
  for (int rr = 0; rr < kUpRows; ++rr) {
    const size_t row = (size_t)min(r0 + rr, rows_bs - 1) * kHeads + h;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[rr][k] = *(const float4*)(o_lat + row * kLatent + part * 32 + 4 * k);
  }
  if (lse_wg) {
#pragma unroll
    for (int k = 0; k < 8; ++k) qr[k] = *(const float4*)(qres + crow * kLatent + part * 32 + 4 * k);
    l2 = lse2[crow];
  }
  __builtin_amdgcn_sched_barrier(0);   // every load in flight before the first use

  float w[32];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t wd[4] = {wu[k].x, wu[k].y, wu[k].z, wu[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[8 * k + 2 * e] = __uint_as_float(wd[e] << 16);
      w[8 * k + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int rr = 0; rr < kUpRows; ++rr) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc = fmaf(w[4 * k], x[rr][k].x, acc);
      acc = fmaf(w[4 * k + 1], x[rr][k].y, acc);
      acc = fmaf(w[4 * k + 2], x[rr][k].z, acc);
      acc = fmaf(w[4 * k + 3], x[rr][k].w, acc);
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 16);
    const int r = r0 + rr;
    if (part == 0 && r < rows_bs) out[((size_t)r * kHeads + h) * kVDim + v] = f32_to_bf16(acc);
  }
  if (lse_wg) {
    float corr = 0.f;
#pragma unroll
    for (int rr = 0; rr < kUpRows; ++rr) {
      float c = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        c = fmaf(qr[k].x, x[rr][k].x, c);
        c = fmaf(qr[k].y, x[rr][k].y, c);
        c = fmaf(qr[k].z, x[rr][k].z, c);
        c = fmaf(qr[k].w, x[rr][k].w, c);
      }
      corr = ((vl & (kUpRows - 1)) == rr) ? c : corr;
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) corr += __shfl_xor(corr, d, 16);
    if (part == 0 && vl < kUpRows && rc < rows_bs)
      lse[crow] = (l2 == kNegInf) ? kNegInf : (l2 + scale_log2 * corr) * 0.69314718055994530942f;
  }
}

// ---------------------------------------------------------------------------
// YaRN RoPE: pair (i, i + rope_dim/2) of row r rotated by
// positions[r] * inv_freq[i], in fp64, rounded once to bf16.  Each thread
// reads and writes only its own pair, so dst may equal src.
// ---------------------------------------------------------------------------
struct InvFreq {
  double v[32];
};

__global__ void __launch_bounds__(256) rope_rotate(const uint16_t* src, int64_t ld_src,
                                                   uint16_t* dst, int64_t ld_dst,
                                                   const int32_t* __restrict__ positions, int64_t n,
                                                   InvFreq inv, int half) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * half) return;
  const int64_t r = idx / half;
  const int i = (int)(idx - r * half);
  const uint16_t* in = src + r * ld_src;
  uint16_t* o = dst + r * ld_dst;
  const double ang = (double)positions[r] * inv.v[i];
  double s, c;
  sincos(ang, &s, &c);
  const double lo = (double)bf16_to_f32(in[i]);
  const double hi = (double)bf16_to_f32(in[i + half]);
  const uint16_t out_lo = f64_to_bf16(lo * c - hi * s);
  const uint16_t out_hi = f64_to_bf16(hi * c + lo * s);
  o[i] = out_lo;
  o[i + half] = out_hi;
}

// ---------------------------------------------------------------------------
// Cache append: cache[slot] = [c_kv row | k_pe row], 72 sixteen-byte chunks.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) cache_append(uint8_t* __restrict__ cache,
                                                    const uint16_t* __restrict__ c_kv, int64_t ld_c,
                                                    const uint16_t* __restrict__ k_pe, int64_t ld_k,
                                                    const int64_t* __restrict__ slots, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * kChunksPerRow) return;
  const int64_t t = idx / kChunksPerRow;
  const int c = (int)(idx - t * kChunksPerRow);
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const uint4 v = (c < 64) ? *(const uint4*)(c_kv + t * ld_c + c * 8)
                           : *(const uint4*)(k_pe + t * ld_k + (c - 64) * 8);
  *(uint4*)(cache + slot * kRowBytes + c * 16) = v;
}

}  // namespace

hipError_t launch_absorb(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_kv_b,
                         uint16_t* qabs, float* qres, uint8_t* zero_row, int rows, hipStream_t stream) {
  const unsigned rb = (unsigned)((rows + kAbsorbRows - 1) / kAbsorbRows);
  hipLaunchKernelGGL(absorb_query, dim3(kLatent / 64, kHeads, rb), dim3(256), 0, stream, q_nope, q_pe,
                     w_kv_b, qabs, qres, zero_row, rows);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_lse, const int32_t* ctx_lens,
                          int B, int Sq, int splits, int kv_chunk, float* o_lat, float* lse2,
                          hipStream_t stream) {
  // enough waves that each takes about a batch of splits, at most 16
  const int waves = std::min(kCombineMaxWaves, std::max(1, (splits + kCombineBatch - 1) / kCombineBatch));
  hipLaunchKernelGGL(lse_combine, dim3(32, 2 * Sq, B), dim3(64 * waves), 0, stream, part_o, part_lse,
                     ctx_lens, Sq, splits, kv_chunk, o_lat, lse2);
  return hipGetLastError();
}

hipError_t launch_upproj(const float* o_lat, const uint16_t* w_kv_b, const float* qres,
                         const float* lse2, float scale_log2, uint16_t* out, float* lse, int rows,
                         hipStream_t stream) {
  const unsigned rb = (unsigned)((rows + kUpRows - 1) / kUpRows);
  hipLaunchKernelGGL(upproject, dim3(kVDim / 16, kHeads, rb), dim3(256), 0, stream, o_lat, w_kv_b,
                     qres, lse2, scale_log2, out, lse, rows);
  return hipGetLastError();
}

hipError_t launch_rope(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst,
                       const int32_t* positions, int64_t n, const double* inv_freq, int rope_dim,
                       hipStream_t stream) {
  InvFreq inv;
  const int half = rope_dim / 2;
  for (int i = 0; i < 32; ++i) inv.v[i] = i < half ? inv_freq[i] : 0.0;
  const int64_t total = n * half;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(rope_rotate, dim3(blocks), dim3(256), 0, stream, src, ld_src, dst, ld_dst,
                     positions, n, inv, half);
  return hipGetLastError();
}

hipError_t launch_append(uint8_t* cache, int64_t num_slots, const uint16_t* c_kv, int64_t ld_c,
                         const uint16_t* k_pe, int64_t ld_k, const int64_t* slots, int64_t n,
                         hipStream_t stream) {
  (void)num_slots;
  const int64_t total = n * kChunksPerRow;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(cache_append, dim3(blocks), dim3(256), 0, stream, cache, c_kv, ld_c, k_pe, ld_k,
                     slots, n);
  return hipGetLastError();
}

}  // namespace mla
