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
// of c tiles, c fixed (and sub-split when the chunks leave compute units
// idle) or chosen here so that the segments of all sequences number at most
// target_segs where the lengths allow; then the first
// segment of every sequence and the segment descriptors (SegDesc: sequence,
// first tile, tile stride, tiles, length) in sequence order.  Up to kSchedLds sequences, the lengths and
// segment starts stay in LDS (`lds`, 2 * kSchedLds + 1 ints) and each
// descriptor is found by binary search; larger batches take a serial path.
constexpr int kSchedLds = 2048;

__device__ void build_schedule(const PrepParams& p, int* lds) {
  __shared__ int red4[4];
  const int t = threadIdx.x;
  const bool in_lds = p.B <= kSchedLds;
  int* lens = lds;                    // [kSchedLds]
  int* starts = lds + kSchedLds;      // [kSchedLds + 1]
  // lengths clamped into [Sq, max_ctx_len]; a clamped length raises the fault
  // bit once (the first thread that meets one in this workgroup's pass)
  bool bad_len = false;
  auto read_len = [&](int b) {
    bool bad;
    const int L = clamp_ctx_len(p.ctx_lens[b], p.Sq, p.max_ctx_len, &bad);
    bad_len |= bad;
    return L;
  };
  auto len_of = [&](int b) { return in_lds ? lens[b] : read_len(b); };
  if (in_lds) {
    for (int b = t; b < p.B; b += 256) lens[b] = read_len(b);
    __syncthreads();
  }
  int c = p.fixed_tiles;
  if (c > 0) {
    // A fixed chunk that leaves compute units idle (fewer chunks than the
    // target) has every chunk cut into k equal sub-splits, k a power of two
    // dividing c, each of at least kMinTilesPerSplit tiles, while the
    // segments stay within the target.  The sub-split boundaries include
    // every chunk boundary, and the combine's LSE merge over the sub-splits
    // equals merging each chunk's sub-splits first and then the chunks.
    int n = 0;
    for (int b = t; b < p.B; b += 256) n += ((len_of(b) + kPage - 1) / kPage + c - 1) / c;
    n = block_sum256(n, red4);
    while (c % 2 == 0 && c / 2 >= kMinTilesPerSplit && 2LL * n <= p.target_segs) {
      c /= 2;
      n *= 2;   // an upper bound of the segments with the halved split
    }
  } else {
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
  // segment k of the n of a sequence: a contiguous run of c tiles, or with
  // the balanced schedule and at least kDealMinSplits splits, every n-th tile
  // from tile k
  auto desc = [&](int b, int k, int n, int L) {
    const int tiles = (L + kPage - 1) / kPage;
    const bool dealt = p.fixed_tiles == 0 && n >= kDealMinSplits;
    SegDesc d;
    d.b = b;
    d.first = dealt ? k : k * c;
    d.stride = dealt ? n : 1;
    d.ntiles = dealt ? (tiles - k + n - 1) / n : min(c, tiles - k * c);
    d.L = L;
    d.pad[0] = d.pad[1] = d.pad[2] = 0;
    return d;
  };
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
        for (int k = 0; k < n && first + k < p.max_segs; ++k) p.seg_desc[first + k] = desc(b, k, n, L);
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
      const int L = lens[lo];
      p.seg_desc[w] = desc(lo, w - starts[lo], ((L + kPage - 1) / kPage + c - 1) / c, L);
    }
  }
  for (int w = carry + t; w < p.max_segs; w += 256) {
    SegDesc d = {};
    d.b = -1;
    p.seg_desc[w] = d;
  }
  if (bad_len) raise_fault(p.faults, kFaultCtxLen);
}

// ---------------------------------------------------------------------------
// Preparation of one decode call.  Grid (8 latent blocks of 64 + 4 + 1, 32
// heads, blocks of 16 query rows); row r = b*Sq + j.
//  * Absorption (x < 8): Q_abs[r][h][64x .. 64x + 64) = bf16(W_UK[h]^T
//    q_nope[r][h]) on those columns and the fp32 residual q_lat - bf16(q_lat)
//    (for the first-order LSE correction).  W_UK[h] = w_kv_b rows [h*256,
//    h*256 + 128).  On the matrix cores: the block's W_UK columns go to LDS
//    transposed (each column's 128 nope dims contiguous), and wave w forms
//    columns [64x + 16w, 64x + 16w + 16) of the 16 rows with four steps of
//    v_mfma_f32_16x16x32_bf16 (fp32 sums of exact bf16 products), the
//    columns as A, the query rows as B.
//  * Rope part and new tokens (x = 8 .. 11, head h, a quarter of the block's
//    rows each): Q_abs[r][h][512:576] = q_pe[r][h],
//    rotated at the query's position p = L_b - Sq + j when `rotate` is set;
//    with c_new given, head 0 writes the new tokens' latent into their cache
//    rows (a bit copy, or quantised for the 8-bit format) and head 1 their
//    rope keys (rotated at p).  These run beside the absorption instead of
//    after it, since the fp64 angle arithmetic is long.
//  * Workgroup (12, 0, 0) zeroes the decode kernel's zero row and builds the
//    split schedule (the other workgroups of that column exit at once).
// ---------------------------------------------------------------------------
constexpr int kWtStride = kNope + 8;   // bf16 per transposed W_UK column in LDS (272 bytes)
constexpr int kPrepLds = 64 * kWtStride * 2;
static_assert(kPrepLds >= (2 * kSchedLds + 1) * (int)sizeof(int), "schedule scratch");
constexpr int kPrepRopeCol = kLatent / 64;       // first grid column of the rope part and new tokens
constexpr int kPrepRopeCols = 4;                 // rope columns: 4 of the block's 16 rows each
constexpr int kPrepSchedCol = kPrepRopeCol + kPrepRopeCols;   // grid column of the schedule

// Position of query row r (clamped length) and its sequence.
__device__ __forceinline__ int query_pos(const PrepParams& p, int r, int* b) {
  *b = r / p.Sq;
  bool bad;   // raised by the schedule
  return clamp_ctx_len(p.ctx_lens[*b], p.Sq, p.max_ctx_len, &bad) - p.Sq + (r - *b * p.Sq);
}

// Cache slot of the new token at position pos of sequence b, or -1 when its
// page lies outside the pool (the fault is raised when `flag`).
__device__ __forceinline__ int64_t new_token_slot(const PrepParams& p, int b, int pos, bool flag) {
  if (p.paged) {
    const int page = p.block_table[(size_t)b * p.max_pages + pos / kPage];
    if (!page_ok(page, p.num_pages)) {
      if (flag) raise_fault(p.faults, kFaultPage);
      return -1;
    }
    return (int64_t)page * kPage + pos % kPage;
  }
  return (int64_t)b * p.stride_tokens + pos;
}

// Rope part of Q_abs for head h and (heads 0 and 1) the new tokens' cache
// rows, query rows [r0, r1).  Waves 0-1 rotate the query rope parts, waves
// 2-3 write the cache rows at the same time (two independent chains of a
// length load, rotations or a slot lookup, and stores).
__device__ void prep_rope_and_rows(const PrepParams& p, int h, int r0, int r1) {
  const int t = threadIdx.x;
  constexpr int half = kRope / 2;
  if (t < 128) {
    for (int i = t; i < (r1 - r0) * half; i += 128) {
      const int r = r0 + i / half, k = i % half;
      const size_t hrow = (size_t)r * kHeads + h;
      const uint16_t* src = p.q_pe + hrow * kRope;
      uint16_t lo = src[k], hi = src[k + half];
      if (p.rotate) {
        int b;
        const int pos = query_pos(p, r, &b);
        rope_pair(lo, hi, (double)pos * p.inv.v[k], &lo, &hi);
      }
      uint16_t* dst = p.fp8 ? (uint16_t*)((uint8_t*)p.qabs + hrow * kQRecBytes + kQRecRope) : p.qabs + hrow * kRow + kLatent;
      dst[k] = lo;
      dst[k + half] = hi;
    }
    return;
  }
  if (p.c_new == nullptr || h > 1) return;
  // waves 2 and 3: one new token's row at a time, its values requested
  // before the slot lookup
  const int wave = (t >> 6) - 2, lane = t & 63;
  for (int r = r0 + wave; r < r1; r += 2) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    uint16_t klo = 0, khi = 0;
    if (h == 0) {
      v = *(const uint4*)(p.c_new + r * p.ld_c + 8 * lane);
    } else if (lane < half) {
      klo = p.k_new[r * p.ld_k + lane];
      khi = p.k_new[r * p.ld_k + lane + half];
    }
    int b;
    const int pos = query_pos(p, r, &b);
    const int64_t slot = new_token_slot(p, b, pos, lane == 0);
    if (slot < 0) continue;   // wave-uniform
    if (h == 0) {
      if (!p.fp8) {
        *(uint4*)(p.cache + slot * kRowBytes + 16 * lane) = v;
      } else {
        // lane l holds latent values [8l, 8l + 8) of group l / 16; the 16
        // lanes of a group agree on amax, scale = amax / 448 and the codes
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
        uint8_t* row = p.cache + slot * kF8Row;
        *(uint2*)(row + 8 * lane) = make_uint2(q[0], q[1]);
        if ((lane & 15) == 0) *(float*)(row + kF8ScaleOff + 4 * (lane >> 4)) = scale;
      }
    } else if (lane < half) {
      uint16_t* rope = p.fp8 ? (uint16_t*)(p.cache + slot * kF8Row + kF8RopeOff)
                             : (uint16_t*)(p.cache + slot * kRowBytes) + kLatent;
      if (!p.rotate) {
        rope[lane] = klo;
        rope[lane + half] = khi;
      } else {
        uint16_t lo, hi;
        rope_pair(klo, khi, (double)pos * p.inv.v[lane], &lo, &hi);
        rope[lane] = lo;
        rope[lane + half] = hi;
      }
    }
  }
}

__global__ void __launch_bounds__(256) prep_query(PrepParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kPrepLds];
  __shared__ float bmax[4][16];   // 8-bit records: each wave's 16-column row maxima
  const int cblk = blockIdx.x;
  const int h = blockIdx.y;
  const int r0 = blockIdx.z * p.rows_per_wg;
  const int r1 = min(r0 + p.rows_per_wg, p.rows);
  const int t = threadIdx.x;
  if (cblk == kPrepSchedCol) {
    if (h == 0 && r0 == 0) {
      if (t < kChunksPerRow) ((uint4*)p.zero_row)[t] = make_uint4(0, 0, 0, 0);
      build_schedule(p, (int*)smem);
    }
    return;
  }
  if (cblk >= kPrepRopeCol) {
    const int part = (p.rows_per_wg + kPrepRopeCols - 1) / kPrepRopeCols;
    const int a = r0 + (cblk - kPrepRopeCol) * part;
    prep_rope_and_rows(p, h, a, min(a + part, r1));
    return;
  }
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, n16 = lane & 15;
  // B operand: query row r0 + n16 (zero past the last row), nope dims
  // 32 ks + 8 g .. + 8 of step ks
  const int rq = r0 + n16;
  bf16x8 qb[kNope / 32];
#pragma unroll
  for (int ks = 0; ks < kNope / 32; ++ks) qb[ks] = bf16x8{};
  if (rq < p.rows) {
    const uint16_t* qs = p.q_nope + ((size_t)rq * kHeads + h) * kNope + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kNope / 32; ++ks) qb[ks] = *(const bf16x8*)(qs + 32 * ks);
  }
  // W_UK[h] rows 2 kp and 2 kp + 1 (kp = t % 64), the block's columns
  // [16 cg, 16 cg + 16) (cg = t / 64), written transposed: LDS dword
  // c * kWtStride / 2 + kp holds (W[2kp][c], W[2kp + 1][c])
  {
    const int kp = t & 63, cg = t >> 6;
    const uint16_t* w0 = p.w_kv_b + ((size_t)h * kWRowsPerHead + 2 * kp) * kLatent + cblk * 64 + 16 * cg;
    const uint4 a0 = *(const uint4*)w0, a1 = *(const uint4*)(w0 + 8);
    const uint4 b0 = *(const uint4*)(w0 + kLatent), b1 = *(const uint4*)(w0 + kLatent + 8);
    const uint32_t ra[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const uint32_t rb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    uint32_t* wt = (uint32_t*)smem + (16 * cg) * (kWtStride / 2) + kp;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wt[(2 * i) * (kWtStride / 2)] = (ra[i] & 0xFFFFu) | (rb[i] << 16);
      wt[(2 * i + 1) * (kWtStride / 2)] = (ra[i] >> 16) | (rb[i] & 0xFFFF0000u);
    }
  }
  __syncthreads();
  // D^T[col][row] = sum_k W[k][col] q[row][k]: wave w the 16 columns
  // [16 w, 16 w + 16) of the block; A operand = column 16 w + n16, dims
  // 32 ks + 8 g .. + 8 (16 bytes of LDS)
  f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* arow = smem + ((16 * wave + n16) * kWtStride + 8 * g) * 2;
#pragma unroll
  for (int ks = 0; ks < kNope / 32; ++ks)
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(arow + 64 * ks), qb[ks], d, 0, 0, 0);
  // lane (g, n16) holds row r0 + n16, columns 64 cblk + 16 w + 4 g + i
  const size_t hrow = (size_t)rq * kHeads + h;
  const int col = cblk * 64 + 16 * wave + 4 * g;
  s16x4 qv;
  f32x4 res, qf;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t qbits = f32_to_bf16(d[i]);
    qv[i] = (short)qbits;
    qf[i] = bf16_to_f32(qbits);
    res[i] = d[i] - qf[i];
  }
  if (!p.fp8) {
    if (rq < p.rows) {
      *(s16x4*)(p.qabs + hrow * kRow + col) = qv;
      *(f32x4*)(p.qres + hrow * kLatent + col) = res;
    }
    return;
  }
  // The 8-bit cache kernel's record: bf16(q) = (hi + lo / 16) * 2^-e for the
  // 32-column block of waves 2m, 2m + 1, with e = 7 - exponent(block max), so
  // |q| * 2^e < 256; hi is q * 2^e rounded to E4M3, lo the remainder times 16
  // rounded to E4M3 (exact for every value above 2^-13 of the block max).
  float m = fmaxf(fmaxf(fabsf(qf[0]), fabsf(qf[1])), fmaxf(fabsf(qf[2]), fabsf(qf[3])));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  if (g == 0) bmax[wave][n16] = m;
  __syncthreads();
  const float bm = fmaxf(bmax[wave & ~1][n16], bmax[wave | 1][n16]);
  const int E = (int)((__float_as_uint(bm) >> 23) & 0xFFu) - 127;
  const bool zero = !(bm >= 1.17549435e-38f) || E < -116;   // zero, subnormal or below 2^-116: all zero codes
  const int e = 7 - E;
  const float f = zero ? 0.f : __uint_as_float((uint32_t)(127 + e) << 23);
  uint32_t hw = 0u, lw = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = qf[i] * f;   // exact: a power of two
    const uint32_t hc = f32_to_e4m3(x);
    const uint32_t lc = f32_to_e4m3((x - e4m3_to_f32(hc)) * 16.0f);
    hw |= hc << (8 * i);
    lw |= lc << (8 * i);
  }
  if (rq < p.rows) {
    uint8_t* rec = (uint8_t*)p.qabs + hrow * kQRecBytes;
    *(uint32_t*)(rec + kQRecHi + col) = hw;
    *(uint32_t*)(rec + kQRecLo + col) = lw;
    *(f32x4*)(p.qres + hrow * kLatent + col) = res;
    if (g == 0 && (wave & 1) == 0) {
      const int bi = col / 32;
      rec[kQRecScaleOff + 4 * (bi % 4) + bi / 4] = (uint8_t)(zero ? 127 : 127 - e);
    }
  }
}

// ---------------------------------------------------------------------------
// LSE combine of the segment partials with this column block's share of the
// W_UV up-projection.  Grid (8 latent blocks of 64 columns, 32 heads, blocks
// of RB query rows); a workgroup of 256 threads handles head h of rows
// r0 .. r0 + RB - 1 on columns [64 cb, 64 cb + 64), RB = rows_per_wg (16, the
// one instantiation; calls with one row per workgroup take combine_one_row
// below), so that the block's W_UV share is read once for RB rows:
//  1. 16 groups of 16 lanes, 16 / RB groups per row; the groups of a row take
//     every (16 / RB)-th of its sequence's segments, 16 per batch with every
//     load in flight, each lane 4 columns, keeping a running max; a row's
//     groups are then merged in a fixed order:
//       o_lat = sum_i 2^(lse_i - M) O_i / W,   W = sum_i 2^(lse_i - M)
//     (a segment whose row saw no token has lse_i = -inf and weight 0);
//  2. for every row, share[v] = sum over the block's columns of
//     W_UV[h][v][c] o_lat[c] (W_UV[h] = w_kv_b rows [h*256 + 128, h*256 + 256))
//     and the block's share of qres . o_lat go to the workspace; block 0
//     also stores (M, W).  The shares of the RB rows are one matrix-core
//     product (W_UV as A, the rows as B, each fp32 o_lat split into bf16
//     hi + lo); on the vector units this product bounded the kernel.
// finalize_out then adds the 8 shares in block order.
// ---------------------------------------------------------------------------
constexpr int kCombGroups = 16;
constexpr int kCombBatch = 16;
constexpr int kCombRowsMax = 16;

template <int RB>
__global__ void __launch_bounds__(256) combine_blocks(CombineParams p) {
  static_assert(RB >= 2 && RB <= kCombRowsMax && (RB & (RB - 1)) == 0, "rows per workgroup");
  __shared__ f32x4 red_acc[kCombGroups][16];
  __shared__ float red_m[kCombGroups], red_w[kCombGroups];
  __shared__ float olat[RB][64];
  const int cb = blockIdx.x;
  const int h = blockIdx.y;
  const int r0 = blockIdx.z * RB;
  const int rows = p.hrows / kHeads;
  const int t = threadIdx.x;
  const int grp = t >> 4, c4 = t & 15;
  constexpr int gpr = kCombGroups / RB; // lane groups per row
  const int rr = grp / gpr, gi = grp - rr * gpr;
  const int r = r0 + rr;

  // A operands of the up-projection, requested first: wave w takes the 32
  // values v = 32 w + 16 vt + n16 (vt = 0, 1), lane (g, n16) the columns
  // 64 cb + 32 ks + 8 g .. + 8 of W_UV[h][v] (ks = 0, 1)
  const int lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, n16 = lane & 15;
  bf16x8 wa[2][2];
#pragma unroll
  for (int vt = 0; vt < 2; ++vt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      wa[vt][ks] = *(const bf16x8*)(p.w_kv_b + ((size_t)h * kWRowsPerHead + kNope + 32 * wave + 16 * vt + n16) * kLatent +
                                    cb * 64 + 32 * ks + 8 * g);
  // qres of row t / 16 of the block, 4 columns
  float4 qr = make_float4(0.f, 0.f, 0.f, 0.f);
  if (t < 16 * RB && r0 + (t >> 4) < rows)
    qr = *(const float4*)(p.qres + ((size_t)(r0 + (t >> 4)) * kHeads + h) * kLatent + cb * 64 + 4 * (t & 15));

  float m = kNegInf, wsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (r < rows) {
    const int b = r / p.Sq;
    const int j = r - b * p.Sq;
    const int seg0 = p.seg_start[b];
    const int nseg = min(p.seg_start[b + 1], p.max_segs) - seg0;
    const size_t unit_rows = (size_t)p.Sq * kHeads;
    const uint16_t* obase = p.part_o + ((size_t)seg0 * unit_rows + j * kHeads + h) * kLatent + cb * 64 + 4 * c4;
    const float* lbase = p.part_lse + (size_t)seg0 * unit_rows + j * kHeads + h;
    const size_t ostride = unit_rows * kLatent;
    for (int s0 = gi; s0 < nseg; s0 += gpr * kCombBatch) {
      float l[kCombBatch];
      uint2 o4[kCombBatch];   // 4 bf16 values
#pragma unroll
      for (int k = 0; k < kCombBatch; ++k) {
        const int s = min(s0 + k * gpr, nseg - 1);   // past the end: re-read, weight 0 below
        l[k] = lbase[s * unit_rows];
        o4[k] = *(const uint2*)(obase + s * ostride);
      }
      __builtin_amdgcn_sched_barrier(0);   // every load of the batch in flight before the first use
#pragma unroll
      for (int k = 0; k < kCombBatch; ++k)
        if (s0 + k * gpr >= nseg) l[k] = kNegInf;
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
  }
  red_acc[grp][c4] = acc;
  if (c4 == 0) {
    red_m[grp] = m;
    red_w[grp] = wsum;
  }
  __syncthreads();
  if (t < 16 * RB) {   // row t / 16 of the block: merge its groups; o_lat and the share of qres . o_lat
    const int rr2 = t >> 4, g0 = rr2 * gpr, lane16 = t & 15;
    float M = red_m[g0];
    for (int g2 = 1; g2 < gpr; ++g2) M = fmaxf(M, red_m[g0 + g2]);
    float W = 0.f;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g2 = 0; g2 < gpr; ++g2) {
      const float sc = (red_m[g0 + g2] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(red_m[g0 + g2] - M);
      W = fmaf(red_w[g0 + g2], sc, W);
      const f32x4 a = red_acc[g0 + g2][lane16];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = fmaf(a[i], sc, o[i]);
    }
    const float inv = (W > 0.f) ? 1.f / W : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= inv;
    *(f32x4*)(&olat[rr2][4 * lane16]) = o;
    float c = qr.x * o[0];
    c = fmaf(qr.y, o[1], c);
    c = fmaf(qr.z, o[2], c);
    c = fmaf(qr.w, o[3], c);
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) c += __shfl_xor(c, d, 16);
    const int r2 = r0 + rr2;
    if (lane16 == 0 && r2 < rows) {
      const size_t hrow = (size_t)r2 * kHeads + h;
      p.corr_part[hrow * 8 + cb] = c;
      if (cb == 0) {
        p.stat[2 * hrow] = M;
        p.stat[2 * hrow + 1] = W;
      }
    }
  }
  __syncthreads();

  // share^T[v][row] = sum over the block's columns of W_UV[h][v][c] o_lat[row][c]
  // on the matrix cores: B = the block's rows (row n16, zero past RB), each
  // fp32 value split into bf16 hi + lo (hi + lo equals it to 16 significant
  // bits), one product for each, fp32 sums
  bf16x8 bhi[2], blo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (n16 < RB) ? olat[n16 < RB ? n16 : 0][32 * ks + 8 * g + e] : 0.f;
      const uint16_t hb = f32_to_bf16(x);
      bhi[ks][e] = __builtin_bit_cast(__bf16, hb);
      blo[ks][e] = __builtin_bit_cast(__bf16, f32_to_bf16(x - bf16_to_f32(hb)));
    }
  }
  const int r2 = r0 + n16;
#pragma unroll
  for (int vt = 0; vt < 2; ++vt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[vt][ks], bhi[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[vt][ks], blo[ks], acc, 0, 0, 0);
    }
    // lane (g, n16): row r0 + n16, values 32 w + 16 vt + 4 g .. + 4
    if (n16 < RB && r2 < rows)
      *(f32x4*)(p.up_part + (((size_t)r2 * kHeads + h) * 8 + cb) * kVDim + 32 * wave + 16 * vt + 4 * g) = acc;
  }
}

// The same for one query row per workgroup (calls with fewer than 16 query
// rows, e.g. a single sequence decoding one token), written for that case:
// wave 0 merges the 16 groups, and the share goes straight to the workspace.
// At one row it measured 0.5 us per call faster than combine_blocks<1>.
__global__ void __launch_bounds__(256) combine_one_row(CombineParams p) {
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
                                                    const int64_t* __restrict__ slots, int64_t n,
                                                    int64_t num_slots, uint32_t* faults) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * kChunksPerRow) return;
  const int64_t t = idx / kChunksPerRow;
  const int c = (int)(idx - t * kChunksPerRow);
  const int64_t slot = slots[t];
  if (slot < 0) return;
  if (slot_fault(slot, num_slots)) {   // outside the cache: the row is skipped
    if (c == 0) raise_fault(faults, kFaultSlot);
    return;
  }
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
                                                        const int64_t* __restrict__ slots, int64_t n,
                                                        int64_t num_slots, uint32_t* faults) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= n) return;
  const int64_t slot = slots[t];
  if (slot < 0) return;
  if (slot_fault(slot, num_slots)) {   // outside the cache: the row is skipped
    if (lane == 0) raise_fault(faults, kFaultSlot);
    return;
  }
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

hipError_t launch_append_fp8(uint8_t* cache, int64_t num_slots, const uint16_t* c_kv, int64_t ld_c,
                             const uint16_t* k_pe, int64_t ld_k, const int64_t* slots, int64_t n,
                             uint32_t* faults, hipStream_t stream) {
  const unsigned blocks = (unsigned)((n + 3) / 4);
  hipLaunchKernelGGL(cache_append_fp8, dim3(blocks), dim3(256), 0, stream, cache, c_kv, ld_c, k_pe, ld_k, slots, n,
                     num_slots, faults);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepParams& p, hipStream_t stream) {
  const unsigned rb = (unsigned)((p.rows + p.rows_per_wg - 1) / p.rows_per_wg);
  hipLaunchKernelGGL(prep_query, dim3(kPrepSchedCol + 1, kHeads, rb), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine_upproject(const CombineParams& p, hipStream_t stream) {
  const unsigned rows = (unsigned)(p.hrows / kHeads);
  const unsigned rblocks = (rows + p.rows_per_wg - 1) / p.rows_per_wg;
  const dim3 grid(kLatent / 64, kHeads, rblocks);
  if (p.rows_per_wg == 1) hipLaunchKernelGGL(combine_one_row, grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(combine_blocks<kCombRowsMax>, grid, dim3(256), 0, stream, p);
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
                         uint32_t* faults, hipStream_t stream) {
  const int64_t total = n * kChunksPerRow;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(cache_append, dim3(blocks), dim3(256), 0, stream, cache, c_kv, ld_c, k_pe, ld_k,
                     slots, n, num_slots, faults);
  return hipGetLastError();
}

}  // namespace mla
