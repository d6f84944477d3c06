// The kernels around the split-KV decode: the per-call preparation (query
// absorption, query RoPE, cache rows of the new tokens), the fused LSE
// combine + W_UV up-projection, and the stand-alone YaRN RoPE and cache
// append.
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

// YaRN RoPE of one rotation pair (x_i, x_{i+half}) at angle pos * inv_freq_i:
// cos/sin and the rotation in fp64, each result rounded once to bf16.
__device__ __forceinline__ void rope_pair(uint16_t lo, uint16_t hi, double ang, uint16_t* out_lo,
                                          uint16_t* out_hi) {
#pragma clang fp contract(off)   // products and differences rounded separately, as written
  double s, c;
  sincos(ang, &s, &c);
  const double a = (double)bf16_to_f32(lo), b = (double)bf16_to_f32(hi);
  *out_lo = f64_to_bf16(a * c - b * s);
  *out_hi = f64_to_bf16(b * c + a * s);
}

// Sum over a 256-thread workgroup (every thread gets the total).
__device__ __forceinline__ int block_sum256(int v, int* red4) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if (lane == 0) red4[wv] = v;
  __syncthreads();
  const int r = red4[0] + red4[1] + red4[2] + red4[3];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_max256(int v, int* red4) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, 64));
  if (lane == 0) red4[wv] = v;
  __syncthreads();
  const int r = max(max(red4[0], red4[1]), max(red4[2], red4[3]));
  __syncthreads();
  return r;
}

// Inclusive prefix sum over a 256-thread workgroup; *total gets the sum.
__device__ __forceinline__ int block_scan256(int v, int* red4, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(v, d, 64);
    if (lane >= d) v += y;
  }
  if (lane == 63) red4[wv] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += red4[w];
  *total = red4[0] + red4[1] + red4[2] + red4[3];
  __syncthreads();
  return v + before;
}

// The split schedule of one call, built by one 256-thread workgroup: splits
// of c tiles, c fixed or chosen here so that the segments of all sequences
// number at most target_segs where the lengths allow; then the first
// segment of every sequence and the segment descriptors {b, first token, end
// token, L_b} in sequence order.  Up to kSchedLds sequences, the lengths and
// segment starts stay in LDS (`lds`, 2 * kSchedLds + 1 ints) and each
// descriptor is found by binary search; larger batches take a serial path.
constexpr int kSchedLds = 2048;

__device__ void build_schedule(const PrepParams& p, int* lds) {
  __shared__ int red4[4];
  const int t = threadIdx.x;
  const bool in_lds = p.B <= kSchedLds;
  int* lens = lds;                    // [kSchedLds]
  int* starts = lds + kSchedLds;      // [kSchedLds + 1]
  auto len_of = [&](int b) { return in_lds ? lens[b] : p.ctx_lens[b]; };
  if (in_lds) {
    for (int b = t; b < p.B; b += 256) lens[b] = p.ctx_lens[b];
    __syncthreads();
  }
  int c = p.fixed_tiles;
  if (c <= 0) {
    int tsum = 0, tmax = 1;
    for (int b = t; b < p.B; b += 256) {
      const int tb = (len_of(b) + kPage - 1) / kPage;
      tsum += tb;
      tmax = max(tmax, tb);
    }
    const int T = block_sum256(tsum, red4);
    tmax = max(kMinTilesPerSplit, block_max256(tmax, red4));
    // c never exceeds the longest sequence's tiles: from there on every
    // sequence is a single split, and more sequences than the target cannot
    // be helped by longer splits
    c = min(tmax, max(kMinTilesPerSplit, (T + p.target_segs - 1) / p.target_segs));
    for (int it = 0; it < 8; ++it) {   // the last split of each sequence is short: grow c until it fits
      int n = 0;
      for (int b = t; b < p.B; b += 256) n += ((len_of(b) + kPage - 1) / kPage + c - 1) / c;
      n = block_sum256(n, red4);
      if (n <= p.target_segs || c >= tmax) break;
      c = min(tmax, max(c + 1, (int)(((long long)c * n + p.target_segs - 1) / p.target_segs)));
    }
  }
  const int chunk = c * kPage;
  int carry = 0;
  for (int base = 0; base < p.B; base += 256) {
    const int b = base + t;
    const int L = (b < p.B) ? len_of(b) : 0;
    const int n = (b < p.B) ? ((L + kPage - 1) / kPage + c - 1) / c : 0;
    int total;
    const int first = carry + block_scan256(n, red4, &total) - n;
    if (b < p.B) {
      p.seg_start[b] = min(first, p.max_segs);
      if (in_lds) {
        starts[b] = first;
      } else {
        for (int k = 0; k < n && first + k < p.max_segs; ++k)
          p.seg_desc[first + k] = make_int4(b, k * chunk, min(L, (k + 1) * chunk), L);
      }
    }
    carry += total;
  }
  if (t == 0) p.seg_start[p.B] = min(carry, p.max_segs);
  if (in_lds) {
    __syncthreads();
    for (int w = t; w < min(carry, p.max_segs); w += 256) {
      int lo = 0, hi = p.B - 1;          // last b with starts[b] <= w
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (starts[mid] <= w) lo = mid;
        else hi = mid - 1;
      }
      const int k = w - starts[lo], L = lens[lo];
      p.seg_desc[w] = make_int4(lo, k * chunk, min(L, (k + 1) * chunk), L);
    }
  }
  for (int w = carry + t; w < p.max_segs; w += 256) p.seg_desc[w] = make_int4(-1, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Preparation of one decode call.  Grid (8 latent blocks of 64 + 1, 32
// heads, query-row blocks of 4); row r = b*Sq + j.
//  * Absorption: Q_abs[r][h][0:512] = bf16(W_UK[h]^T q_nope[r][h]) and the
//    fp32 residual q_lat - bf16(q_lat) (for the first-order LSE correction).
//    W_UK[h] = w_kv_b rows [h*256, h*256 + 128).  Thread (ng, c8) loads
//    W_UK[h][4ng .. 4ng+3][c8*8 .. c8*8+7] as four 16-byte loads, forms the
//    partial dot products of the block's 4 rows over those 4 nope dims, and
//    the 32 partials of each output are summed through LDS in a fixed order.
//  * Rope part: Q_abs[r][h][512:576] = q_pe[r][h], rotated at the query's
//    position p = L_b - Sq + j when `rotate` is set (latent block 0).
//  * New tokens (when c_new is given): cache row of token p of sequence b =
//    [c_new[r] | rot(k_new[r], p)] (head 0 writes the latent, head 1 of
//    latent block 0 the rope part).
//  * Workgroup (8, 0, 0) zeroes the decode kernel's zero row and builds the
//    split schedule (the other workgroups of that column exit at once).
// ---------------------------------------------------------------------------
constexpr int kPrepRows = 4;

__global__ void __launch_bounds__(256) prep_query(PrepParams p) {
  __shared__ float red[kPrepRows][32][64];
  static_assert(sizeof(red) >= (2 * kSchedLds + 1) * sizeof(int), "schedule scratch");
  const int cblk = blockIdx.x;
  const int h = blockIdx.y;
  const int r0 = blockIdx.z * kPrepRows;
  const int t = threadIdx.x;
  if (cblk == kLatent / 64) {           // the extra column: schedule and zero row
    if (h == 0 && r0 == 0) {
      if (t < kChunksPerRow) ((uint4*)p.zero_row)[t] = make_uint4(0, 0, 0, 0);
      build_schedule(p, (int*)&red[0][0][0]);
    }
    return;
  }
  const int c8 = t & 7, ng = t >> 3;
  const uint16_t* wk = p.w_kv_b + ((size_t)h * kWRowsPerHead + 4 * ng) * kLatent + cblk * 64 + c8 * 8;
  uint4 w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = *(const uint4*)(wk + (size_t)k * kLatent);
  uint2 q[kPrepRows];
#pragma unroll
  for (int rr = 0; rr < kPrepRows; ++rr) {
    const int r = min(r0 + rr, p.rows - 1);
    q[rr] = *(const uint2*)(p.q_nope + ((size_t)r * kHeads + h) * kNope + 4 * ng);
  }
#pragma unroll
  for (int rr = 0; rr < kPrepRows; ++rr) {
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
  if (r >= p.rows) return;
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < 32; ++k) acc += red[rr][k][col];
  const size_t hrow = (size_t)r * kHeads + h;
  uint16_t* dst = p.qabs + hrow * kRow;
  const uint16_t qb = f32_to_bf16(acc);
  dst[cblk * 64 + col] = qb;
  p.qres[hrow * kLatent + cblk * 64 + col] = acc - bf16_to_f32(qb);

  const int b = r / p.Sq;
  const int pos = p.ctx_lens[b] - p.Sq + (r - b * p.Sq);
  const int half = kRope / 2;
  if (cblk == 0) {
    const uint16_t* src = p.q_pe + hrow * kRope;
    if (!p.rotate) {
      dst[kLatent + col] = src[col];
    } else if (col < half) {
      uint16_t lo, hi;
      rope_pair(src[col], src[col + half], (double)pos * p.inv.v[col], &lo, &hi);
      dst[kLatent + col] = lo;
      dst[kLatent + col + half] = hi;
    }
  }
  if (p.c_new != nullptr && p.fp8 && pos >= 0 && ((h == 0 && cblk < 4) || (h == 1 && cblk == 0))) {
    // 8-bit row: latent group cblk (128 values, 2 per lane of this row's wave)
    // quantised with its own scale; the rope key rotated into bf16 at byte 528
    int64_t slot;
    if (p.paged) slot = (int64_t)p.block_table[(size_t)b * p.max_pages + pos / kPage] * kPage + pos % kPage;
    else slot = (int64_t)b * p.stride_tokens + pos;
    uint8_t* row = p.cache + slot * kF8Row;
    if (h == 0) {
      const uint32_t two = *(const uint32_t*)(p.c_new + r * p.ld_c + cblk * kF8Group + 2 * col);
      const float x0 = __uint_as_float(two << 16), x1 = __uint_as_float(two & 0xFFFF0000u);
      float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
      const float scale = amax / kE4M3Max;
      const uint32_t q0 = scale > 0.f ? f32_to_e4m3(x0 / scale) : 0u;
      const uint32_t q1 = scale > 0.f ? f32_to_e4m3(x1 / scale) : 0u;
      *(uint16_t*)(row + cblk * kF8Group + 2 * col) = (uint16_t)(q0 | (q1 << 8));
      if (col == 0) *(float*)(row + kF8ScaleOff + 4 * cblk) = scale;
    } else {
      uint16_t* rope = (uint16_t*)(row + kF8RopeOff);
      const uint16_t* src = p.k_new + r * p.ld_k;
      if (!p.rotate) {
        rope[col] = src[col];
      } else if (col < half) {
        uint16_t lo, hi;
        rope_pair(src[col], src[col + half], (double)pos * p.inv.v[col], &lo, &hi);
        rope[col] = lo;
        rope[col + half] = hi;
      }
    }
  }
  if (p.c_new != nullptr && !p.fp8 && pos >= 0 && (h == 0 || (h == 1 && cblk == 0))) {
    int64_t slot;
    if (p.paged) slot = (int64_t)p.block_table[(size_t)b * p.max_pages + pos / kPage] * kPage + pos % kPage;
    else slot = (int64_t)b * p.stride_tokens + pos;
    uint16_t* crow = (uint16_t*)(p.cache + slot * kRowBytes);
    if (h == 0) {
      crow[cblk * 64 + col] = p.c_new[r * p.ld_c + cblk * 64 + col];
    } else {
      const uint16_t* src = p.k_new + r * p.ld_k;
      if (!p.rotate) {
        crow[kLatent + col] = src[col];
      } else if (col < half) {
        uint16_t lo, hi;
        rope_pair(src[col], src[col + half], (double)pos * p.inv.v[col], &lo, &hi);
        crow[kLatent + col] = lo;
        crow[kLatent + col + half] = hi;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LSE combine of the segment partials with this column block's share of the
// W_UV up-projection.  Grid (8 latent blocks of 64 columns, 32 heads, rows);
// a workgroup of 256 threads handles head row (r, h) on columns
// [64 cb, 64 cb + 64):
//  1. its 16 groups of 16 lanes take every 16th of the sequence's segments,
//     16 per batch with every load in flight, each lane 4 columns, and keep
//     a running max; the groups are merged in a fixed order:
//       o_lat = sum_i 2^(lse_i - M) O_i / W,   W = sum_i 2^(lse_i - M)
//     (a segment whose row saw no token has lse_i = -inf and weight 0);
//  2. share[v] = sum over the block's columns of W_UV[h][v][c] o_lat[c]
//     (W_UV[h] = w_kv_b rows [h*256 + 128, h*256 + 256)) and the block's share
//     of qres . o_lat go to the workspace; block 0 also stores (M, W).
// finalize_out then adds the 8 shares in block order.
// ---------------------------------------------------------------------------
constexpr int kCombGroups = 16;
constexpr int kCombBatch = 16;

__global__ void __launch_bounds__(256) combine_blocks(CombineParams p) {
  __shared__ f32x4 red_acc[kCombGroups][16];
  __shared__ float red_m[kCombGroups], red_w[kCombGroups];
  __shared__ float olat[64];
  const int cb = blockIdx.x;
  const int h = blockIdx.y;
  const int r = blockIdx.z;
  const int b = r / p.Sq;
  const int j = r - b * p.Sq;
  const size_t hrow = (size_t)r * kHeads + h;
  const int t = threadIdx.x;
  const int grp = t >> 4, c4 = t & 15;

  // W_UV[h][v][64 cb + 32 half .. + 32): thread (v, half), requested first
  const int v = t >> 1, half = t & 1;
  const uint16_t* wrow = p.w_kv_b + ((size_t)h * kWRowsPerHead + kNope + v) * kLatent + cb * 64 + 32 * half;
  uint4 wu[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) wu[k] = *(const uint4*)(wrow + 8 * k);
  float4 qr = make_float4(0.f, 0.f, 0.f, 0.f);
  if (t < 16) qr = *(const float4*)(p.qres + hrow * kLatent + cb * 64 + 4 * t);

  const int seg0 = p.seg_start[b];
  const int nseg = min(p.seg_start[b + 1], p.max_segs) - seg0;
  const size_t unit_rows = (size_t)p.Sq * kHeads;
  const uint16_t* obase = p.part_o + ((size_t)seg0 * unit_rows + j * kHeads + h) * kLatent + cb * 64 + 4 * c4;
  const float* lbase = p.part_lse + (size_t)seg0 * unit_rows + j * kHeads + h;
  const size_t ostride = unit_rows * kLatent;

  float m = kNegInf, wsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = grp; s0 < nseg; s0 += kCombGroups * kCombBatch) {
    float l[kCombBatch];
    uint2 o4[kCombBatch];   // 4 bf16 values
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const int s = min(s0 + k * kCombGroups, nseg - 1);   // past the end: re-read, weight 0 below
      l[k] = lbase[s * unit_rows];
      o4[k] = *(const uint2*)(obase + s * ostride);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch in flight before the first use
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k)
      if (s0 + k * kCombGroups >= nseg) l[k] = kNegInf;
    float bm = m;
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) bm = fmaxf(bm, l[k]);
    const float sc = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - bm);
    wsum *= sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= sc;
    m = bm;
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const float wt = (l[k] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(l[k] - bm);
      wsum += wt;
      const float ov[4] = {__uint_as_float(o4[k].x << 16), __uint_as_float(o4[k].x & 0xFFFF0000u),
                           __uint_as_float(o4[k].y << 16), __uint_as_float(o4[k].y & 0xFFFF0000u)};
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(wt, ov[i], acc[i]);
    }
  }
  red_acc[grp][c4] = acc;
  if (c4 == 0) {
    red_m[grp] = m;
    red_w[grp] = wsum;
  }
  __syncthreads();
  if (t < 64) {   // wave 0: merge the groups, this block's o_lat and share of qres . o_lat
    float M = red_m[0];
#pragma unroll
    for (int g2 = 1; g2 < kCombGroups; ++g2) M = fmaxf(M, red_m[g2]);
    float W = 0.f;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g2 = 0; g2 < kCombGroups; ++g2) {
      const float sc = (red_m[g2] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(red_m[g2] - M);
      W = fmaf(red_w[g2], sc, W);
      const f32x4 a = red_acc[g2][t & 15];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(a[i], sc, o[i]);
    }
    const float inv = (W > 0.f) ? 1.f / W : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= inv;
    float c = 0.f;
    if (t < 16) {
      *(f32x4*)(olat + 4 * t) = o;
      c = qr.x * o[0];
      c = fmaf(qr.y, o[1], c);
      c = fmaf(qr.z, o[2], c);
      c = fmaf(qr.w, o[3], c);
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) c += __shfl_xor(c, d, 16);
    if (t == 0) {
      p.corr_part[hrow * 8 + cb] = c;
      if (cb == 0) {
        p.stat[2 * hrow] = M;
        p.stat[2 * hrow + 1] = W;
      }
    }
  }
  __syncthreads();

  float up = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t wd[4] = {wu[k].x, wu[k].y, wu[k].z, wu[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 32 * half + 8 * k + 2 * e;
      up = fmaf(__uint_as_float(wd[e] << 16), olat[c], up);
      up = fmaf(__uint_as_float(wd[e] & 0xFFFF0000u), olat[c + 1], up);
    }
  }
  up += __shfl_xor(up, 1, 2);
  if (half == 0) p.up_part[(hrow * 8 + cb) * kVDim + v] = up;
}

// ---------------------------------------------------------------------------
// out[r][h][v] = bf16(sum over the 8 latent blocks of their W_UV shares), in
// block order; lse = ln 2 * (M + log2 W + scale_log2 * sum of the blocks'
// qres . o_lat).  Scores were taken with the bf16-rounded absorbed query; the
// exact score differs by scale * (q_lat - bf16(q_lat)) . c_t, so to first
// order the LSE moves by the softmax mean of that difference,
// scale * qres . o_lat.  Two head rows per 256-thread workgroup.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) finalize_out(CombineParams p) {
  const size_t hrow = (size_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int v = threadIdx.x & 127;
  if (hrow >= (size_t)p.hrows) return;
  const float* u = p.up_part + hrow * 8 * kVDim + v;
  float sum = 0.f;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) sum += u[cb * kVDim];
  p.out[hrow * kVDim + v] = f32_to_bf16(sum);
  if (v == 0 && p.lse != nullptr) {
    float corr = 0.f;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) corr += p.corr_part[hrow * 8 + cb];
    const float M = p.stat[2 * hrow], W = p.stat[2 * hrow + 1];
    p.lse[hrow] = (W > 0.f) ? (M + __log2f(W) + p.scale_log2 * corr) * 0.69314718055994530942f : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// YaRN RoPE: pair (i, i + rope_dim/2) of row r rotated by
// positions[r] * inv_freq[i].  Each thread reads and writes only its own
// pair, so dst may equal src.
// ---------------------------------------------------------------------------
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
  uint16_t lo, hi;
  rope_pair(in[i], in[i + half], (double)positions[r] * inv.v[i], &lo, &hi);
  o[i] = lo;
  o[i + half] = hi;
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

// ---------------------------------------------------------------------------
// 8-bit cache append: one wave per row.  Lane l holds latent values
// [8l, 8l + 8) of group l / 16; the 16 lanes of a group agree on
// amax = max |x|, scale = amax / 448 (fp32), codes e4m3(x / scale) (a group of
// zeros: scale 0, codes 0); lanes 0..7 copy the bf16 rope key (16 bytes each).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) cache_append_fp8(uint8_t* __restrict__ cache,
                                                        const uint16_t* __restrict__ c_kv, int64_t ld_c,
                                                        const uint16_t* __restrict__ k_pe, int64_t ld_k,
                                                        const int64_t* __restrict__ slots, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= n) return;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const uint4 v = *(const uint4*)(c_kv + t * ld_c + 8 * lane);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 16));
  const float scale = amax / kE4M3Max;
  uint32_t q[2] = {0u, 0u};
  if (scale > 0.f) {
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k >> 2] |= f32_to_e4m3(x[k] / scale) << (8 * (k & 3));
  }
  uint8_t* row = cache + slot * kF8Row;
  *(uint2*)(row + 8 * lane) = make_uint2(q[0], q[1]);
  if ((lane & 15) == 0) *(float*)(row + kF8ScaleOff + 4 * (lane >> 4)) = scale;
  if (lane < 8) *(uint4*)(row + kF8RopeOff + 16 * lane) = *(const uint4*)(k_pe + t * ld_k + 8 * lane);
}

}  // namespace

hipError_t launch_append_fp8(uint8_t* cache, const uint16_t* c_kv, int64_t ld_c, const uint16_t* k_pe,
                             int64_t ld_k, const int64_t* slots, int64_t n, hipStream_t stream) {
  const unsigned blocks = (unsigned)((n + 3) / 4);
  hipLaunchKernelGGL(cache_append_fp8, dim3(blocks), dim3(256), 0, stream, cache, c_kv, ld_c, k_pe, ld_k, slots, n);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  const unsigned rb = (unsigned)((p.rows + kPrepRows - 1) / kPrepRows);
  hipLaunchKernelGGL(prep_query, dim3(kLatent / 64 + 1, kHeads, rb), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine_upproject(const CombineParams& p, hipStream_t stream) {
  const unsigned rows = (unsigned)(p.hrows / kHeads);
  hipLaunchKernelGGL(combine_blocks, dim3(kLatent / 64, kHeads, rows), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(finalize_out, dim3((unsigned)((p.hrows + 1) / 2)), dim3(256), 0, stream, p);
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
