// Split-KV flash decoding over the latent cache on gfx950 (bf16 MFMA).
//
// What is computed (per sequence b, split of kv_chunk tokens, query token j,
// head h): the online-softmax partial of
//     s_t = scale * ([q_lat | q_pe] . [c_t | k_pe_t])
// over the split's visible tokens, i.e. (O = sum_t p_t c_t / sum_t p_t,
// lse = log2 sum_t 2^(s_t log2 e)).  The cache row [c_t | k_pe_t] is what
// kv_a_proj_with_mqa writes ("mHC+MLA+MTP 是什么", MLA section); scoring
// against the latent directly is the W_UK absorption, and the LSE combine and
// W_UV up-projection of the partials follow in combine.hip.
//
// Work decomposition (one workgroup of 4 waves per (sequence, split)):
//  * A 64-token tile (one page, 72 KiB) is staged in LDS by direct
//    global->LDS loads, double buffered, so a tile streams in while the
//    previous one is consumed.  Tile rows are swizzled at 16-byte granularity
//    (latent chunk c of token t sits at c ^ (t & 15), rope chunk 64+k at
//    64 + (k ^ ((t >> 1) & 7))) so that both read patterns below are free of
//    LDS bank conflicts.
//  * The 32*QG query rows (query token, head) are cut into row groups of 16.
//    Each wave owns one row group and a share of every tile's tokens and
//    keeps its own running max, sum and 16 x 512 fp32 accumulator: no wave
//    waits on another inside the tile loop.  With one query token two waves
//    share a row group (each takes 32 tokens of a tile) and merge at the end.
//  * Scores: S^T[token][row] = C_tile . Q^T on v_mfma_f32_16x16x32_bf16, the
//    cache tile as the A operand (ds_read_b128 of 8 latent values per lane)
//    and the wave's 16 query rows held in registers as the B operand.
//  * The S^T accumulator layout (lane = row, 4 tokens per lane) is exactly the
//    A-operand layout P[row][token] of the value product, with the token order
//    (4g + e, 16 + 4g + e); the value operand C[token][col] is fetched in that
//    token order with ds_read_b64_tr_b16 (transposing 4 x 16 blocks), so P
//    never leaves registers.
//  * The running max moves only when a row's tile max exceeds it by more
//    than 8 (log2 units); until then p <= 256 and no rescale is needed.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 8.0f;

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_vm_18() { asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); }
__device__ __forceinline__ void wait_vm_0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Chunk <-> slot swizzle of a tile row (an involution within each group).
__device__ __forceinline__ int tile_slot(int tok, int c) {
  return c < 64 ? (c ^ (tok & 15)) : (64 + ((c - 64) ^ ((tok >> 1) & 7)));
}

__device__ __forceinline__ float bcast_row(float v, int src_lane) { return __shfl(v, src_lane, 64); }

// Row scaling of a 16x16 accumulator block on the matrix cores:
// returns c + diag(f) . x, where f[row] is held by the lanes with n16 == row
// and x is in the accumulator layout (lane holds rows 4g+i, column n16).
// Four v_mfma_f32_16x16x4f32 with A[m][k] = f[m] if m == 4k + i, else 0, and
// B[k][n] = x[4k + i][n]; each output is one exact fp32 product plus zeros.
// Keeping this off the vector ALU lets the accumulators live in AGPRs.
struct RowScale {
  float a[4];
};
__device__ __forceinline__ RowScale make_row_scale(float f, int g, int n16) {
  RowScale r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.a[i] = (n16 == 4 * g + i) ? f : 0.f;
  return r;
}
__device__ __forceinline__ f32x4 scale_rows(const RowScale& r, f32x4 x, f32x4 c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(r.a[i], x[i], c, 0, 0, 0);
  return c;
}

template <int QG, bool PAGED>
__global__ void __launch_bounds__(256, 1) splitkv_decode(DecodeParams p) {
  constexpr int RG = 2 * QG;        // row groups of 16 rows
  constexpr int TP = 4 / RG;        // waves per row group
  constexpr int TOKW = 64 / TP;     // tokens of each tile one wave scores
  constexpr int NBLK = TOKW / 16;   // 16-token score blocks per tile
  constexpr int NKV = TOKW / 32;    // 32-token k-steps of the value product

  // Two tile buffers as separate objects so that reads of one are known not
  // to alias the direct-to-LDS loads in flight into the other.
  __shared__ __attribute__((aligned(1024))) uint8_t tile_a[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t tile_b[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  const int rg = wave % RG, tp = wave / RG;

  const int unit = blockIdx.x;
  const int b = unit / p.splits;
  const int split = unit - b * p.splits;
  const int L = p.ctx_lens[b];
  const int t_begin = split * p.kv_chunk;
  const int t_end = min(L, t_begin + p.kv_chunk);
  if (t_begin >= t_end) return;     // split past the end: the combine never reads it

  const int j = p.j0 + (rg >> 1);
  const int limit = min(t_end, L - p.Sq + j + 1);   // rows of this wave see tokens < limit
  const int rg_glob = 2 * p.j0 + rg;
  float* out_o = p.part_o + ((size_t)unit * (2 * p.Sq) + rg_glob) * (32 * 64 * 4);
  float* out_lse = p.part_lse + (size_t)unit * (p.Sq * 32) + rg_glob * 16;

  // The wave's 16 query rows, as MFMA B operands: lane holds row n16, 8 dims.
  bf16x8 q[18];
  {
    const uint16_t* qrow = p.qabs + (((size_t)b * p.Sq + j) * 32 + (rg & 1) * 16 + n16) * kRow + g * 8;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) q[ks] = *(const bf16x8*)(qrow + ks * 32);
  }

  // Byte offset inside a tile of each 16-byte chunk this lane loads: LDS slot
  // P = (wave*18 + i)*64 + lane holds chunk (tok = P / 72, tile_slot(tok, P % 72)).
  int off[18];
#pragma unroll
  for (int i = 0; i < 18; ++i) {
    const int P = (wave * 18 + i) * 64 + lane;
    const int tok = P / kChunksPerRow;
    const int c = tile_slot(tok, P - tok * kChunksPerRow);
    off[i] = tok * kRowBytes + c * 16;
  }

  // LDS read offsets.  Score reads: token tok_w + 16*blk + n16, chunk
  // 4*ks + g, slot (4ks + g) ^ n16 = 16*(ks/4) + ((4*(ks%4)) ^ (g ^ n16)); the
  // 16*(ks/4) and 16*blk parts become instruction immediates.
  const int tok_w = tp * TOKW;
  const int qk_row = (tok_w + n16) * kRowBytes;
  int qk_off[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) qk_off[bb] = qk_row + (((4 * bb) ^ (g ^ n16)) << 4);
  int rope_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) rope_off[kk] = qk_row + ((64 + ((4 * kk + g) ^ (n16 >> 1))) << 4);
  // Value reads (transposed, 8 bytes): token tok_w + 32*kk + 4g + (n16 >> 2)
  // (+16 for the upper half), columns 16*cb + 4*(n16 & 3); the chunk
  // 2cb + ((n16 >> 1) & 1) sits at slot 16*(cb/8) + ((2*(cb%8)) ^ v).
  const int pv_tok = tok_w + 4 * g + (n16 >> 2);
  const int pv_v = ((n16 >> 1) & 1) ^ (pv_tok & 15);
  const int pv_row = pv_tok * kRowBytes + (n16 & 1) * 8;
  int pv_off[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) pv_off[bb] = pv_row + (((2 * bb) ^ pv_v) << 4);

  const int tile0 = t_begin >> 6;
  const int ntiles = (t_end - t_begin + 63) >> 6;

  auto tile_src = [&](int tile) -> const uint8_t* {
    if constexpr (PAGED) {
      const int page = p.block_table[(size_t)b * p.max_pages + tile];
      return p.cache + (size_t)page * kTileBytes;
    } else {
      return p.cache + ((size_t)b * p.stride_tokens + (size_t)tile * kPage) * kRowBytes;
    }
  };

  // Enqueue tile `tile` into `buf`; returns whether it was a full tile.
  auto issue_tile = [&](int tile, uint8_t* buf) -> bool {
    const uint8_t* src = tile_src(tile);
    const int nval = min(kPage, t_end - tile * kPage);
    uint8_t* dst = buf + wave * 18 * 1024;
    if (nval == kPage) {
#pragma unroll
      for (int i = 0; i < 18; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(src + off[i]), (lds_void_t*)(dst + i * 1024), 16, 0, 0);
      return true;
    }
    // Ragged last tile: rows past the end are never read from memory; their
    // LDS slots get zeros so that masked tokens multiply zeros, not garbage.
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      if (off[i] / kRowBytes < nval)
        __builtin_amdgcn_global_load_lds((const void*)(src + off[i]), (lds_void_t*)(dst + i * 1024), 16, 0, 0);
      else
        *(int4*)(dst + i * 1024 + lane * 16) = make_int4(0, 0, 0, 0);
    }
    return false;
  };

  f32x4 o[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // reference max of row n16 (log2 units)
  float l_part = 0.f;      // this lane's share of the row sum

  auto process = [&](const uint8_t* T, int tile) {
    const int abs_w = tile * kPage + tok_w;   // absolute position of the wave's first token

    // ---- scores S^T = C . Q^T, 16 tokens per block
    f32x4 s[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const uint8_t* base = T + blk * 16 * kRowBytes;
      // all 18 operand reads of the block are issued before the MFMA chain
      bf16x8 a[18];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) a[ks] = *(const bf16x8*)(base + qk_off[ks & 3] + (ks >> 2) * 256);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) a[16 + kk] = *(const bf16x8*)(base + rope_off[kk]);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], q[ks], acc, 0, 0, 0);
      s[blk] = acc;
    }

    // ---- scale, mask, tile max of row n16
    float mt = kNegInf;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = abs_w + blk * 16 + 4 * g + i;
        const float v = (t < limit) ? s[blk][i] * p.scale_log2 : kNegInf;
        s[blk][i] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));

    // ---- move the reference max only when a row outgrows it by kTau
    const bool grow = mt > m_ref + kTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.f;
      m_ref = grow ? mt : m_ref;
      l_part *= alpha;
      const RowScale rs = make_row_scale(alpha, g, n16);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) o[cb] = scale_rows(rs, o[cb], f32x4{0.f, 0.f, 0.f, 0.f});
    }

    // ---- P = 2^(s - m_ref) in bf16, as the A operand of the value product
    const float mref = (m_ref == kNegInf) ? 0.f : m_ref;
    bf16x8 pa[NKV];
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 e = (__bf16)__builtin_amdgcn_exp2f(s[2 * kk + half][i] - mref);
          l_part += (float)e;
          pa[kk][half * 4 + i] = e;
        }

    // ---- O += P . C[:, 0:512]; B operand by transposed LDS reads
#pragma unroll
    for (int kk = 0; kk < NKV; ++kk) {
      const uint8_t* base = T + kk * 32 * kRowBytes;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        const uint8_t* a = base + pv_off[cb & 7] + (cb >> 3) * 256;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a + 16 * kRowBytes));
        const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[kk], __builtin_bit_cast(bf16x8, both), o[cb], 0, 0, 0);
      }
    }
  };

  // Double-buffered tile loop, unrolled by two so each buffer is named statically.
  bool full = issue_tile(tile0, tile_a);
  (void)full;
  for (int it = 0; it < ntiles; it += 2) {
    bool next_full = false;
    if (it + 1 < ntiles) next_full = issue_tile(tile0 + it + 1, tile_b);
    if (next_full) wait_vm_18(); else wait_vm_0();
    lds_barrier();
    process(tile_a, tile0 + it);
    lds_barrier();
    if (it + 1 >= ntiles) break;
    next_full = false;
    if (it + 2 < ntiles) next_full = issue_tile(tile0 + it + 2, tile_a);
    if (next_full) wait_vm_18(); else wait_vm_0();
    lds_barrier();
    process(tile_b, tile0 + it + 1);
    lds_barrier();
  }

  // ---- finalize: row sums, merge the two token halves, normalise, write
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);

  if constexpr (TP == 2) {
    float* xo = (float*)tile_a + rg * (32 * 64 * 4 + 32);
    float* xm = xo + 32 * 64 * 4;
    float* xl = xm + 16;
    if (tp == 1) {
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) *(f32x4*)(xo + (cb * 64 + lane) * 4) = o[cb];
      if (lane < 16) { xm[lane] = m_ref; xl[lane] = l_row; }
    }
    lds_barrier();
    if (tp == 1) return;
    const float m1 = xm[n16], l1 = xl[n16];
    const float mm = fmaxf(m_ref, m1);
    const float a0 = (m_ref == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
    const float a1 = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_row = l_row * a0 + l1 * a1;
    m_ref = mm;
    // o = diag(a0/l) o + diag(a1/l) o1, normalised in the same step
    const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
    const RowScale r0 = make_row_scale(a0 * inv, g, n16);
    const RowScale r1 = make_row_scale(a1 * inv, g, n16);
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const f32x4 o1 = *(const f32x4*)(xo + (cb * 64 + lane) * 4);
      o[cb] = scale_rows(r1, o1, scale_rows(r0, o[cb], f32x4{0.f, 0.f, 0.f, 0.f}));
    }
  } else {
    const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
    const RowScale r0 = make_row_scale(inv, g, n16);
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) o[cb] = scale_rows(r0, o[cb], f32x4{0.f, 0.f, 0.f, 0.f});
  }

#pragma unroll
  for (int cb = 0; cb < 32; ++cb) *(f32x4*)(out_o + (cb * 64 + lane) * 4) = o[cb];
  if (lane < 16) out_lse[lane] = (l_row > 0.f) ? m_ref + __log2f(l_row) : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int B, int query_group, bool paged, hipStream_t stream) {
  const dim3 grid((unsigned)B * (unsigned)p.splits), block(256);
  if (query_group == 1) {
    if (paged) hipLaunchKernelGGL((splitkv_decode<1, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((splitkv_decode<1, false>), grid, block, 0, stream, p);
  } else {
    if (paged) hipLaunchKernelGGL((splitkv_decode<2, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((splitkv_decode<2, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
