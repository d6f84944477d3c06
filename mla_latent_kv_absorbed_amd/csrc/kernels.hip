// The small kernels around the split-KV decode: query absorption, LSE
// combine, W_UV up-projection, YaRN RoPE and the cache append.
//
// Pages cited: "mHC+MLA+MTP 是什么？拆开给 Agent 用的百亿 MoE", MLA section
// (kv_b_proj: latent -> per-head [k_nope | v]; kv_a_proj_with_mqa output
// cached as latent + rope; YaRN rope) and "256K 长上下文真能本地用", §一
// (rope_scaling fields, attention_bias false).
#include "mla_internal.h"

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
// W_UK[h] = w_kv_b rows [h*256, h*256 + 128).  One workgroup per (head,
// 64-column block) keeps its 128 x 64 slice of W_UK in registers (each
// thread one column) and sweeps every query row of that head.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) absorb_query(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ q_pe,
                                                     const uint16_t* __restrict__ w_kv_b,
                                                     uint16_t* __restrict__ qabs,
                                                     float* __restrict__ qres,
                                                     uint8_t* __restrict__ zero_row, int rows_bs) {
  const int cblk = blockIdx.x;          // 8 blocks of 64 latent columns
  const int h = blockIdx.y;
  if (cblk == 0 && h == 0 && threadIdx.x < kChunksPerRow)   // the decode kernel's zero row
    ((uint4*)zero_row)[threadIdx.x] = make_uint4(0, 0, 0, 0);
  const int col = cblk * 64 + (threadIdx.x & 63);
  const int rsub = threadIdx.x >> 6;    // 4 query-row lanes
  float w[kNope];
  const uint16_t* wk = w_kv_b + (size_t)h * kWRowsPerHead * kLatent + col;
#pragma unroll
  for (int n = 0; n < kNope; ++n) w[n] = bf16_to_f32(wk[(size_t)n * kLatent]);

  for (int r = rsub; r < rows_bs; r += 4) {
    const uint16_t* qn = q_nope + ((size_t)r * kHeads + h) * kNope;
    float acc = 0.f;
#pragma unroll
    for (int n8 = 0; n8 < kNope; n8 += 8) {
      const uint4 v = *(const uint4*)(qn + n8);   // same address across the wave: one fetch
      const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc = fmaf(__uint_as_float(wd[k] << 16), w[n8 + 2 * k], acc);
        acc = fmaf(__uint_as_float(wd[k] & 0xFFFF0000u), w[n8 + 2 * k + 1], acc);
      }
    }
    uint16_t* dst = qabs + ((size_t)r * kHeads + h) * kRow;
    const uint16_t qb = f32_to_bf16(acc);
    dst[col] = qb;
    qres[((size_t)r * kHeads + h) * kLatent + col] = acc - bf16_to_f32(qb);
    if (cblk == 0) {   // the 64 threads of this row's lane group copy its rope part
      const int e = threadIdx.x & 63;
      dst[kLatent + e] = q_pe[((size_t)r * kHeads + h) * kRope + e];
    }
  }
}

// ---------------------------------------------------------------------------
// LSE combine of the split partials.  One workgroup per (sequence b, row
// group of 16 rows, 16-column block); each of its 4 waves sums a quarter of
// the splits, in the partials' own layout (lane holds rows 4g..4g+3 of
// column n16), and the quarters are added in a fixed order.
//   o_lat[row] = sum_i 2^(lse_i - M) O_i / sum_i 2^(lse_i - M)
//   lse2[row]  = M + log2 sum_i 2^(lse_i - M)   (log2 units)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) lse_combine(const float* __restrict__ part_o,
                                                   const float* __restrict__ part_lse,
                                                   const int32_t* __restrict__ ctx_lens, int Sq,
                                                   int splits, int kv_chunk, float* __restrict__ o_lat,
                                                   float* __restrict__ lse2_out) {
  __shared__ float red_m[4][16];
  __shared__ float red_w[4][16];
  __shared__ f32x4 red_o[4][64];
  const int cbm = blockIdx.x;           // 32 column blocks of 16
  const int rgg = blockIdx.y;           // row group in [0, 2*Sq)
  const int b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, n16 = lane & 15;
  const int RGT = 2 * Sq;
  const int L = ctx_lens[b];
  const int nsplit = min(splits, (L + kv_chunk - 1) / kv_chunk);

  // 1. row maxima of the split LSEs (rows 4g..4g+3 of the group)
  f32x4 m4 = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
  for (int s = wave; s < nsplit; s += 4) {
    const f32x4 l4 = *(const f32x4*)(part_lse + ((size_t)b * splits + s) * (Sq * 32) + rgg * 16 + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) m4[i] = fmaxf(m4[i], l4[i]);
  }
  if (n16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red_m[wave][4 * g + i] = m4[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    m4[i] = fmaxf(fmaxf(red_m[0][r], red_m[1][r]), fmaxf(red_m[2][r], red_m[3][r]));
  }

  // 2. weighted sums
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 wsum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = wave; s < nsplit; s += 4) {
    const size_t unit = (size_t)b * splits + s;
    const f32x4 l4 = *(const f32x4*)(part_lse + unit * (Sq * 32) + rgg * 16 + 4 * g);
    const f32x4 o4 = *(const f32x4*)(part_o + ((unit * RGT + rgg) * 32 + cbm) * 256 + lane * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wt = (l4[i] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(l4[i] - m4[i]);
      wsum[i] += wt;
      acc[i] = fmaf(wt, o4[i], acc[i]);
    }
  }
  red_o[wave][lane] = acc;
  if (n16 == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red_w[wave][4 * g + i] = wsum[i];
  }
  __syncthreads();
  if (wave != 0) return;
  f32x4 o = red_o[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const f32x4 t = red_o[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] += t[i];
  }
  const int j = rgg >> 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const float ws = red_w[0][r] + red_w[1][r] + red_w[2][r] + red_w[3][r];
    const int h = (rgg & 1) * 16 + r;
    const size_t row = ((size_t)b * Sq + j) * kHeads + h;
    o_lat[row * kLatent + cbm * 16 + n16] = (ws > 0.f) ? o[i] / ws : 0.f;
    if (cbm == 0 && n16 == 0) lse2_out[row] = (ws > 0.f) ? m4[i] + __log2f(ws) : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// W_UV up-projection: out[r][v] = bf16(sum_c W_UV[h][v][c] o_lat[r][c]),
// W_UV[h] = w_kv_b rows [h*256 + 128, h*256 + 256).  One workgroup per
// (head, 16 output dims); 16 lanes split each 512-long dot product.
//
// The workgroup of output block 0 also writes the natural-log LSE.  Scores
// were taken with the bf16-rounded absorbed query; the exact score differs
// by scale * (q_lat - bf16(q_lat)) . c_t, so to first order the LSE moves by
// the softmax mean of that difference, scale * qres . o_lat.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) upproject(const float* __restrict__ o_lat,
                                                 const uint16_t* __restrict__ w_kv_b,
                                                 const float* __restrict__ qres,
                                                 const float* __restrict__ lse2, float scale_log2,
                                                 uint16_t* __restrict__ out, float* __restrict__ lse,
                                                 int rows_bs) {
  const int vblk = blockIdx.x;          // 8 blocks of 16 output dims
  const int h = blockIdx.y;
  const int vl = threadIdx.x >> 4;
  const int v = vblk * 16 + vl;
  const int part = threadIdx.x & 15;    // columns [part*32, part*32 + 32)
  const uint16_t* wrow = w_kv_b + ((size_t)h * kWRowsPerHead + kNope + v) * kLatent + part * 32;
  const bool lse_lane = (lse != nullptr) && vblk == 0 && vl == 0;
  float w[32];
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const uint4 u = *(const uint4*)(wrow + k);
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[k + 2 * e] = __uint_as_float(wd[e] << 16);
      w[k + 2 * e + 1] = __uint_as_float(wd[e] & 0xFFFF0000u);
    }
  }
  for (int r = 0; r < rows_bs; ++r) {
    const size_t row = (size_t)r * kHeads + h;
    const float* ol = o_lat + row * kLatent + part * 32;
    float acc = 0.f, corr = 0.f;
#pragma unroll
    for (int k = 0; k < 32; k += 4) {
      const float4 x = *(const float4*)(ol + k);
      acc = fmaf(w[k], x.x, acc);
      acc = fmaf(w[k + 1], x.y, acc);
      acc = fmaf(w[k + 2], x.z, acc);
      acc = fmaf(w[k + 3], x.w, acc);
      if (lse_lane) {
        const float4 d = *(const float4*)(qres + row * kLatent + part * 32 + k);
        corr = fmaf(d.x, x.x, corr);
        corr = fmaf(d.y, x.y, corr);
        corr = fmaf(d.z, x.z, corr);
        corr = fmaf(d.w, x.w, corr);
      }
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) {
      acc += __shfl_xor(acc, d, 16);
      corr += __shfl_xor(corr, d, 16);
    }
    if (part == 0) {
      out[row * kVDim + v] = f32_to_bf16(acc);
      if (lse_lane) {
        const float l2 = lse2[row];
        lse[row] = (l2 == kNegInf) ? kNegInf : (l2 + scale_log2 * corr) * 0.69314718055994530942f;
      }
    }
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
  hipLaunchKernelGGL(absorb_query, dim3(kLatent / 64, kHeads), dim3(256), 0, stream, q_nope, q_pe,
                     w_kv_b, qabs, qres, zero_row, rows);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part_o, const float* part_lse, const int32_t* ctx_lens,
                          int B, int Sq, int splits, int kv_chunk, float* o_lat, float* lse2,
                          hipStream_t stream) {
  hipLaunchKernelGGL(lse_combine, dim3(32, 2 * Sq, B), dim3(256), 0, stream, part_o, part_lse,
                     ctx_lens, Sq, splits, kv_chunk, o_lat, lse2);
  return hipGetLastError();
}

hipError_t launch_upproj(const float* o_lat, const uint16_t* w_kv_b, const float* qres,
                         const float* lse2, float scale_log2, uint16_t* out, float* lse, int rows,
                         hipStream_t stream) {
  hipLaunchKernelGGL(upproject, dim3(kVDim / 16, kHeads), dim3(256), 0, stream, o_lat, w_kv_b,
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
