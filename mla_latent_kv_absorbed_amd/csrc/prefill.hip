// Chunked prefill of MLA attention on gfx950: the un-absorbed form.
//
// A chunk of Tq new tokens (positions L - Tq .. L - 1 of one sequence, their
// cache rows already written) attends causally to the sequence's L cached
// tokens.  With many query tokens the keys and values are worth expanding:
// kv_b_proj turns each cached latent c_t into per-head K_nope[h] = W_UK[h] c_t
// and V[h] = W_UV[h] c_t ("mHC+MLA+MTP 是什么", MLA section), after which the
// attention is plain multi-head attention with a 192-wide key
// [K_nope | k_pe_t] (the rope key shared by all heads) and a 128-wide value:
//     s_jt = scale * (q_nope[j,h] . K_nope[t,h] + q_pe[j,h] . k_pe[t]),  t <= L - Tq + j
//     out[j,h] = sum_t softmax_t(s_jt) V[t,h]
// per query token 2*32*(192 + 128) flops per visible token, against
// 2*32*(576 + 512) for the absorbed form: above a few hundred query tokens
// the expansion (2*512*8192 flops per cached token, once) pays for itself.
//
// Two kernels:
//  * expand_kv: KV[t][o] = fp16(sum_k W[o][k] c_t[k]) for the 8192 rows o of
//    kv_b_proj (per head [k_nope 128 | v 128]); 256 persistent workgroups of
//    8 waves walk 256 x 256 output tiles with one pipeline of 64-wide k stages
//    (double-buffered in LDS through direct global->LDS loads), on
//    v_mfma_f32_16x16x32_bf16.  The expanded values are kept in fp16, whose
//    11-bit significand rounds a key 8 times more finely than bf16 at the same
//    matrix-core rate: a row that sees one or two tokens has no other tokens
//    to average that rounding out of its log-sum-exp.
//  * prefill_attention: flash attention (rescaling only when a row's maximum
//    outgrows its reference by 2^8); a workgroup of 8 waves takes 256 query
//    rows of one head, each wave 32 rows (two row groups of 16, so every LDS
//    read of a key or value tile feeds two MFMAs); 64-token tiles of
//    [K_nope | k_pe] and V stream through a three-tile LDS ring.
//    S^T = K . Q^T with the keys as the A operand (fp16 products over the
//    128 nope dims, bf16 over the 64 rope dims, one fp32 accumulator); the
//    S^T accumulator layout is the B-operand layout of P in O^T += V^T P^T
//    (fp16), with V^T fetched by ds_read_b64_tr_b16, so P stays in registers.  The query tiles of a head
//    are placed on one XCD (workgroups x, x + 8, ...), where they read the
//    head's key and value tiles from the same L2.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kKvRow = kHeads * kWRowsPerHead;   // 8192 expanded values per token
constexpr int kKvStride = kKvRow + kRope;         // workspace row: [8192 expanded (fp16) | 64 rope key (bf16)]
constexpr float kF16Max = 65504.0f;              // largest finite fp16

typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((address_space(3))) const f16x8 lds_f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) const uint8_t lds_cu8;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gaddr)
               : "memory", "m0");
}

// One 16-byte direct global->LDS load from a wave-uniform base plus a
// per-lane 32-bit offset (LDS byte lds + 16 * lane).
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ lds_cu8* lds_base(uint32_t lds) {
  asm volatile("" : "+s"(lds));
  return (lds_cu8*)lds;
}

// ---------------------------------------------------------------------------
// expand_kv.  KV[t][o] = fp16(W[o][:] . c_t) for the 8192 rows o of kv_b_proj.
// Output tiles of 256 rows x 256 tokens; one workgroup of 8 waves per compute
// unit walks its tiles with one pipeline of 64-wide k stages across tile
// boundaries (the next tile's first stages load while the current tile
// finishes and is written).  W rows are the A operand, cache rows B (both read
// k-contiguous, 16 bytes per lane); wave (wo, wt) owns rows o0 + 128 wo ..
// and tokens t0 + 64 wt .., i.e. 8 x 4 blocks of 16 x 16, so every 16-byte
// read feeds 4 or 8 products.  LDS stage: W tile [256][64] and C tile
// [256][64] bf16, rows of 8 chunks of 16 bytes; chunk c of row r sits at
// position c ^ ((r >> 1) & 7), which keeps the reads free of bank conflicts.
// Tile placement: workgroup x runs on XCD x % 8 and takes the 4 row tiles
// [4 (x % 8), 4 (x % 8) + 4) of kv_b_proj (1 MiB of W, resident in that
// XCD's L2) for token tiles x / 32, x / 32 + 8, ...
// ---------------------------------------------------------------------------
constexpr int kExpTile = 256;
constexpr int kExpStageK = 64;
constexpr int kExpStageBytes = 2 * kExpTile * kExpStageK * 2;   // 64 KiB: W tile then C tile
constexpr int kExpStages = kLatent / kExpStageK;                // 8 per tile
constexpr int kExpLoads = kExpStageBytes / 16 / 512;             // 8 per lane per stage
constexpr int kExpGrid = 256;                                    // persistent workgroups
constexpr int kExpOTiles = kKvRow / kExpTile;                    // 32
static_assert(kExpOTiles == 4 * kXcds && kExpGrid == kExpOTiles * kXcds, "tile placement");

__global__ void __launch_bounds__(512, 2) expand_kv(const uint16_t* __restrict__ w, const uint8_t* __restrict__ cache,
                                                 int32_t L, uint16_t* __restrict__ kv, uint32_t* faults) {
  __shared__ __attribute__((aligned(1024))) uint8_t st[2 * kExpStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  const int x = blockIdx.x;
  const int ot = 4 * (x % kXcds) + ((x / kXcds) & 3);
  const int o0 = ot * kExpTile;
  const int tt0 = x / (4 * kXcds);                 // first token tile; then every 8th
  const int ntt = (L + kExpTile - 1) / kExpTile;
  const int ntiles = tt0 < ntt ? (ntt - tt0 + kXcds - 1) / kXcds : 0;
  if (ntiles == 0) return;
  const int nst = ntiles * kExpStages;
  const uint32_t st_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)st);

  // load i of this lane: LDS position P = (wave * 8 + i) * 64 + lane
  // (16-byte units); waves 0-3 fill the W tile, waves 4-7 the C tile.  The
  // in-tile byte offsets are fixed; the tile and stage enter through the
  // wave-uniform base.
  const bool wpart = wave < 4;
  uint32_t off[kExpLoads];
#pragma unroll
  for (int i = 0; i < kExpLoads; ++i) {
    const int Q = ((wave & 3) * kExpLoads + i) * 64 + lane;
    const int row = Q >> 3, c = (Q & 7) ^ ((row >> 1) & 7);
    off[i] = (uint32_t)((wpart ? row * kLatent : row * kRow) + c * 8) * 2u;
  }
  auto issue = [&](int s, int buf) {
    const int kst = s & (kExpStages - 1);
    const int t0 = (tt0 + kXcds * (s / kExpStages)) * kExpTile;
    const uint32_t dst = st_lds + buf * kExpStageBytes + wave * kExpLoads * 1024;
    if (wpart) {
      const uint8_t* src = (const uint8_t*)w + ((size_t)o0 * kLatent + kst * kExpStageK) * 2;
#pragma unroll
      for (int i = 0; i < kExpLoads; ++i) dma16s(src, off[i], dst + i * 1024);
    } else if (t0 + kExpTile <= L) {
      const uint8_t* src = cache + ((size_t)t0 * kRow + kst * kExpStageK) * 2;
#pragma unroll
      for (int i = 0; i < kExpLoads; ++i) dma16s(src, off[i], dst + i * 1024);
    } else {   // last token tile: rows past L repeat row L - 1
#pragma unroll
      for (int i = 0; i < kExpLoads; ++i) {
        const int row = off[i] / (kRow * 2);
        const uint32_t inrow = off[i] - row * (kRow * 2);
        dma16(cache + ((size_t)min(t0 + row, L - 1) * kRow + kst * kExpStageK) * 2 + inrow, dst + i * 1024);
      }
    }
  };

  const int wo = wave & 1, wt = wave >> 1;
  f32x4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // read offsets within a tile: row r, chunk 4 ks + g
  auto rd = [&](int row, int ks) -> int { return row * 128 + (((4 * ks + g) ^ ((row >> 1) & 7)) << 4); };

  issue(0, 0);
  if (nst > 1) issue(1, 1);
  for (int s = 0; s < nst; ++s) {
    // stage s has landed; stage s + 1 may still load, and after a tile's
    // stores (issued between the loads of stages s and s + 1) those may
    // still drain
    if (s + 1 < nst) {
      if (s > 0 && (s & (kExpStages - 1)) == 0) vm_wait<kExpLoads + 16>();
      else vm_wait<kExpLoads>();
    } else {
      vm_wait<0>();
    }
    lds_barrier();
    lds_cu8* W = lds_base(st_lds + (s & 1) * kExpStageBytes);
    lds_cu8* C = W + kExpTile * kExpStageK * 2;
#pragma unroll
    for (int ks = 0; ks < kExpStageK / 32; ++ks) {
      bf16x8 a[8], bb[4];
#pragma unroll
      for (int ob = 0; ob < 8; ++ob) a[ob] = *(lds_bf16x8_t*)(W + rd(128 * wo + 16 * ob + n16, ks));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) bb[tb] = *(lds_bf16x8_t*)(C + rd(64 * wt + 16 * tb + n16, ks));
#pragma unroll
      for (int ob = 0; ob < 8; ++ob)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[ob][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ob], bb[tb], acc[ob][tb], 0, 0, 0);
    }
    lds_barrier();   // every wave is done with this buffer before it is refilled
    if ((s & (kExpStages - 1)) == kExpStages - 1) {
      // tile done: lane (g, n16) of block (ob, tb) holds rows
      // o0 + 128 wo + 16 ob + 4 g .. + 3 of token t0 + 64 wt + 16 tb + n16.
      // For each pair of blocks (2p, 2p + 1) one lane-row swap
      // (v_permlane16_swap: rows [A0 B0 A2 B2], [A1 B1 A3 B3]) gives lane row
      // g the 8 consecutive rows 16 (2p + (g & 1)) + 8 (g >> 1) .. + 7 of its
      // token, stored as 16 bytes (64 contiguous bytes per token and pair).
      // Every row of the tile is written (rows past L repeat row L - 1), so
      // that the attention's last tile reads defined values.
      const int t0 = (tt0 + kXcds * (s / kExpStages)) * kExpTile;
      float amax = 0.f;   // largest magnitude in this lane's share (fp16 range check)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int t = t0 + 64 * wt + 16 * tb + n16;
        uint16_t* krow = kv + (size_t)t * kKvStride + o0 + 128 * wo + 16 * (g & 1) + 8 * (g >> 1);
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            amax = fmaxf(amax, fmaxf(fabsf(acc[2 * pr][tb][i]), fabsf(acc[2 * pr + 1][tb][i])));
          const u32x2 a = __builtin_bit_cast(u32x2, __builtin_convertvector(acc[2 * pr][tb], f16x4));
          const u32x2 b = __builtin_bit_cast(u32x2, __builtin_convertvector(acc[2 * pr + 1][tb], f16x4));
          const auto lo = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
          const auto hi = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
          *(uint4*)(krow + 32 * pr) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
          acc[2 * pr][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
          acc[2 * pr + 1][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      // values past the largest finite fp16 (65504) or not finite: flagged
      if (__builtin_amdgcn_ballot_w64(!(amax <= kF16Max)) != 0 && lane == 0) raise_fault(faults, kFaultFp16Range);
    }
    if (s + 2 < nst) issue(s + 2, s & 1);
  }
  if (ot == 0) {   // the tiles' rope keys, copied next to the expanded rows (after the pipeline)
    for (int k = 0; k < ntiles; ++k) {
      const int t0 = (tt0 + kXcds * k) * kExpTile;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = j * 512 + tid, tk = e >> 3, c = e & 7;
        const uint4 r = *(const uint4*)(cache + (size_t)min(t0 + tk, L - 1) * kRowBytes + (kLatent + 8 * c) * 2);
        *(uint4*)(kv + (size_t)(t0 + tk) * kKvStride + kKvRow + 8 * c) = r;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// prefill_attention.  A key/value tile of 64 tokens sits in LDS as padded
// rows: key rows of 416 bytes ([K_nope 16 chunks | k_pe 8 chunks | pad 2],
// chunk = 16 bytes) and value rows of 288 bytes ([V 16 chunks | pad 2]).
// Both the 16-byte key reads (lanes: tokens t..t+15 x 4 chunks) and the
// 8-byte transposed value reads (8 tokens x 4 column quarters per 32 lanes)
// are then free of bank conflicts (measured with the LDS bank-conflict
// counter: a 400-byte key row or a 272-byte value row conflicts two-way),
// and every read of a tile is one per-lane base plus an immediate offset.
// ---------------------------------------------------------------------------
constexpr int kPfTile = 64;                          // tokens per key/value tile
constexpr int kPfKRow = 416;                         // LDS bytes per key row
constexpr int kPfVRow = 288;                         // LDS bytes per value row
constexpr int kPfKBytes = kPfTile * kPfKRow;         // 26624
constexpr int kPfTileBytes = kPfKBytes + kPfTile * kPfVRow;   // 45056
constexpr int kPfInstr = kPfTileBytes / 1024;        // 44 wave-wide direct loads per tile
constexpr int kPfWaves = 8;                          // waves per workgroup (32 query rows each)
constexpr int kPfSlots = 3;                          // tiles in the LDS ring
constexpr int kPfWide = kPfInstr - 5 * kPfWaves;     // waves 0..3 issue 6 loads per tile, the rest 5
constexpr float kPfTau = 8.0f;                       // log2 headroom of p above the row's reference
static_assert(kPfInstr * 1024 == kPfTileBytes && kPfWide == 4, "tile split");

struct PrefillParams {
  const uint16_t* q_nope;   // bf16 [Tq][32][128]
  const uint16_t* q_pe;     // bf16 [Tq][32][64], rotated
  const uint16_t* kv;       // bf16 [L rounded up to 256][8256]: expanded rows and rope keys
  int32_t L, Tq, qtiles;
  float scale_log2;
  uint16_t* out;            // bf16 [Tq][32][128]
  float* lse;               // fp32 [Tq][32] or null
  uint32_t* faults;         // the device's fault word
};

// Maxima of finite or infinite scores (no NaN handling needed; written as
// the plain instructions so that no quieting of the MFMA results is added).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float fmax2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Maximum over lanes n, n + 16, n + 32, n + 48 (the four 16-lane rows of a
// wave), by two lane-half swaps instead of LDS permutes.
__device__ __forceinline__ float max_rows4(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__builtin_bit_cast(float, a[0]), __builtin_bit_cast(float, a[1]));
  const unsigned w = __builtin_bit_cast(unsigned, v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, b[0]), __builtin_bit_cast(float, b[1]));
}

// Eight waves of 32 query rows (two row groups of 16; two waves per SIMD)
// take 256 consecutive query rows of one head, so every key and value byte
// brought into LDS feeds 256 rows.  Three tiles rotate through the LDS ring:
// two are loading while one is consumed.
__global__ void __launch_bounds__(kPfWaves * 64, 2) prefill_attention(PrefillParams p) {
  constexpr int RG = 2;                       // row groups of 16 query rows per wave
  constexpr int kRowsW = 16 * RG;             // query rows per wave
  constexpr int kQRows = kPfWaves * kRowsW;   // query rows per workgroup (one head)
  constexpr int SLOTS = kPfSlots;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[SLOTS * kPfTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  // workgroup x on XCD x % 8 takes head (k8 / qtiles) * 8 + x % 8: a head's
  // query tiles share one XCD's L2; the longest (last) query tiles go first
  const int x = blockIdx.x;
  const int k8 = x / kXcds;
  const int h = (k8 / p.qtiles) * kXcds + x % kXcds;
  const int qt = p.qtiles - 1 - k8 % p.qtiles;
  const int q0 = qt * kQRows;
  const int base = p.L - p.Tq;                     // position of query row 0
  const uint32_t ring_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)ring);

  // this wave's rows: q0 + kRowsW wave + 16 rg + n16 (rows past Tq repeat Tq - 1, never stored).
  // The nope part meets the fp16 keys, so it is widened to fp16 (exact for
  // bf16 values of magnitude 2^-14 .. 65504; smaller ones round to the fp16
  // subnormal grid, an absolute error below 2^-25); the rope part stays bf16.
  f16x8 qn16[RG][4];
  bf16x8 qr[RG][2];
  float qmax = 0.f;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int j = min(q0 + kRowsW * wave + 16 * rg + n16, p.Tq - 1);
    const uint16_t* qn = p.q_nope + ((size_t)j * kHeads + h) * kNope + 8 * g;
    const uint16_t* qp = p.q_pe + ((size_t)j * kHeads + h) * kRope + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 v = *(const bf16x8*)(qn + 32 * ks);
      const f32x8 w = __builtin_convertvector(v, f32x8);
#pragma unroll
      for (int i = 0; i < 8; ++i) qmax = fmaxf(qmax, fabsf(w[i]));
      qn16[rg][ks] = __builtin_convertvector(w, f16x8);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qr[rg][ks] = *(const bf16x8*)(qp + 32 * ks);
  }
  if (__builtin_amdgcn_ballot_w64(!(qmax <= kF16Max)) != 0 && lane == 0) raise_fault(p.faults, kFaultFp16Range);
  // settle the query loads before the direct loads start (a wait placed at
  // their first use would also drain the tiles in flight)
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(qn16[rg][ks]));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) asm volatile("" ::"v"(qr[rg][ks]));
  }

  // key/value tiles of tokens [0, last visible of the workgroup's rows]
  const int last_row = min(q0 + kQRows, p.Tq) - 1;
  const int ntiles = (base + last_row) / kPfTile + 1;

  // direct loads: wave-wide load I of a tile fills LDS bytes [1024 I,
  // 1024 (I + 1)); waves 0..3 issue loads 6w .. 6w + 5, waves 4..7 loads
  // 24 + 5 (w - 4) .. + 4.  Lane position P = 64 I + lane (16-byte units):
  // P < 1664 is chunk P % 26 of key row P / 26, else chunk Q % 18 of value
  // row Q / 18 (Q = P - 1664); pad chunks repeat the row's first chunk.  The
  // byte offsets within a tile are the same for every tile.
  const bool wide = wave < kPfWide;
  const int i0 = wide ? 6 * wave : kPfWide + 5 * wave;
  uint32_t off[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int P = (i0 + i) * 64 + lane;
    int e;
    if (P < kPfTile * 26) {
      const int t = P / 26, c = P - 26 * t;
      e = t * kKvStride + (c < 16 ? h * kWRowsPerHead + 8 * c : (c < 24 ? kKvRow + 8 * (c - 16) : h * kWRowsPerHead));
    } else {
      const int Q = P - kPfTile * 26, t = Q / 18, c = Q - 18 * t;
      e = t * kKvStride + h * kWRowsPerHead + kNope + (c < 16 ? 8 * c : 0);
    }
    off[i] = (uint32_t)e * 2u;
  }
  auto issue = [&](int tile, int slot) {
    const uint8_t* src = (const uint8_t*)p.kv + (size_t)tile * (kPfTile * kKvStride * 2);
    const uint32_t dst = ring_lds + slot * kPfTileBytes + i0 * 1024;
#pragma unroll
    for (int i = 0; i < 5; ++i) dma16s(src, off[i], dst + i * 1024);
    if (wide) dma16s(src, off[5], dst + 5 * 1024);
  };

  // score reads: token 16 tb + n16 of the step, chunk 4 ks + g
  const int k_lane = n16 * kPfKRow + 16 * g;
  // value reads (transposed, 8 bytes): token 4g + (n16 >> 2) (+16) of the
  // step, columns 16 vb + 4 (n16 & 3) .. + 3 (bytes 32 vb + 8 (n16 & 3))
  const int v_lane = kPfKBytes + (4 * g + (n16 >> 2)) * kPfVRow + 8 * (n16 & 3);

  f32x4 o[RG][8];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int vb = 0; vb < 8; ++vb) o[rg][vb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per row: m, the reference maximum of scale * s (log2 units); nsub = -m
  // (0 while the row has seen nothing); thr = (m + kPfTau) / scale, the raw
  // score above which the reference has to move; l, this lane's share of the sum
  float m[RG], nsub[RG], thr[RG], l[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m[rg] = kNegInf;
    nsub[rg] = 0.f;
    thr[rg] = kNegInf;
    l[rg] = 0.f;
  }
  const float inv_scale = 1.f / p.scale_log2;
  // visibility: row r sees tokens <= base + r; lim_wave is the wave's smallest
  int lim[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) lim[rg] = base + q0 + kRowsW * wave + 16 * rg + n16;
  const int lim_wave = base + q0 + kRowsW * wave;

#pragma unroll
  for (int k = 0; k < SLOTS - 1; ++k)
    if (k < ntiles) issue(k, k);
  for (int it = 0; it < ntiles; ++it) {
    // tile it has landed (tile it + 1 may still be loading), and every wave
    // is done with the slot that tile it + SLOTS - 1 refills
    if (it + 1 < ntiles) {
      if (wide) vm_wait<6>();
      else vm_wait<5>();
    } else {
      vm_wait<0>();
    }
    lds_barrier();
    if (it + SLOTS - 1 < ntiles) issue(it + SLOTS - 1, (it + SLOTS - 1) % SLOTS);
    lds_cu8* T = lds_base(ring_lds + (it % SLOTS) * kPfTileBytes);

    // two 32-token steps, each: scores, online softmax, value product (kept
    // as a loop: unrolled, the rescale branch costs register copies)
#pragma unroll 1
    for (int hb = 0; hb < 2; ++hb) {
      const int tk0 = it * kPfTile + 32 * hb;
      // ---- S^T = K . Q^T for 2 token blocks x 2 row groups
      f32x4 s[RG][2];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) s[rg][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {   // nope dims: fp16 keys
        f16x8 a[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) a[tb] = *(lds_f16x8_t*)(T + k_lane + (32 * hb + 16 * tb) * kPfKRow + 64 * ks);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            s[rg][tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tb], qn16[rg][ks], s[rg][tb], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {   // rope dims: bf16 keys
        bf16x8 a[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          a[tb] = *(lds_bf16x8_t*)(T + k_lane + (32 * hb + 16 * tb) * kPfKRow + 16 * (16 + 4 * ks));
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            s[rg][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tb], qr[rg][ks], s[rg][tb], 0, 0, 0);
      }
      // causal mask, only on steps that reach past the wave's first row
      // (a wave-uniform branch; the empty asm keeps it a branch)
      if (tk0 + 31 > lim_wave) {
        asm volatile("");
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              s[rg][tb][i] = (tk0 + 16 * tb + 4 * g + i <= lim[rg]) ? s[rg][tb][i] : kNegInf;
      }

      // ---- softmax per row (lane n16 of each row group; 8 tokens per lane)
      // with a lazily moved reference: p = 2^(scale s - m) may reach
      // 2^kPfTau.  Each lane compares its own scores with the row's raw
      // threshold; only when one exceeds it (or at the row's first visible
      // token) is the row maximum formed across the four lanes of the row,
      // m moved and O and l rescaled.  The scale is positive, so maxima are
      // taken on the raw scores.
      float lm[RG];
      bool over = false;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        lm[rg] = max3f(max3f(s[rg][0][0], s[rg][0][1], s[rg][0][2]), max3f(s[rg][0][3], s[rg][1][0], s[rg][1][1]),
                       fmax2f(s[rg][1][2], s[rg][1][3]));
        over |= lm[rg] > thr[rg];
      }
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const float mt = max_rows4(lm[rg]) * p.scale_log2;
          const bool move = mt > m[rg] + kPfTau;
          const float alpha = move ? (m[rg] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[rg] - mt)) : 1.f;
          m[rg] = move ? mt : m[rg];
          if (m[rg] != kNegInf) {
            nsub[rg] = -m[rg];
            thr[rg] = (m[rg] + kPfTau) * inv_scale;
          }
          l[rg] *= alpha;
#pragma unroll
          for (int vb = 0; vb < 8; ++vb)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[rg][vb][i] *= alpha;
        }
      }
      f16x8 pa[RG];   // p <= 2^kPfTau: inside the fp16 range
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        // k order of the 32-token step: tokens 4g+i of block 0, then of block 1
        f32x8 e;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) e[4 * tb + i] = __builtin_amdgcn_exp2f(fmaf(s[rg][tb][i], p.scale_log2, nsub[rg]));
        l[rg] += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
        pa[rg] = __builtin_convertvector(e, f16x8);
      }

      // ---- O^T += V^T . P^T: 8 value blocks of 16 columns, this 32-token step
#pragma unroll
      for (int vb = 0; vb < 8; ++vb) {
        lds_cu8* a = T + v_lane + 32 * hb * kPfVRow + 32 * vb;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a + 16 * kPfVRow));
        const f16x8 av = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          o[rg][vb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, pa[rg], o[rg][vb], 0, 0, 0);
      }
    }
  }

  // ---- output: lane (g, n16) holds columns 16 vb + 4g .. + 3 of row n16
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    float lr = l[rg];
    lr += __shfl_xor(lr, 16, 64);
    lr += __shfl_xor(lr, 32, 64);
    const int j = q0 + kRowsW * wave + 16 * rg + n16;
    if (j >= p.Tq) continue;
    const float inv = (lr > 0.f) ? 1.f / lr : 0.f;
    uint16_t* orow = p.out + ((size_t)j * kHeads + h) * kVDim + 4 * g;
#pragma unroll
    for (int vb = 0; vb < 8; ++vb) {
      s16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(short, (__bf16)(o[rg][vb][i] * inv));
      *(s16x4*)(orow + 16 * vb) = v;
    }
    if (p.lse != nullptr && g == 0)
      p.lse[(size_t)j * kHeads + h] = (lr > 0.f) ? (m[rg] + __log2f(lr)) * 0.69314718055994530942f : kNegInf;
  }
}

}  // namespace

hipError_t launch_prefill(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_kv_b, const uint8_t* cache,
                          int32_t L, int32_t Tq, float scale_log2, uint16_t* kv, uint16_t* out, float* lse,
                          uint32_t* faults, hipStream_t stream) {
  hipLaunchKernelGGL(expand_kv, dim3(kExpGrid), dim3(512), 0, stream, w_kv_b, cache, L, kv, faults);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  PrefillParams pp;
  pp.q_nope = q_nope;
  pp.q_pe = q_pe;
  pp.kv = kv;
  pp.L = L;
  pp.Tq = Tq;
  pp.scale_log2 = scale_log2;
  pp.out = out;
  pp.lse = lse;
  pp.faults = faults;
  constexpr int kRows = 32 * kPfWaves;
  pp.qtiles = (Tq + kRows - 1) / kRows;
  hipLaunchKernelGGL(prefill_attention, dim3((unsigned)(pp.qtiles * kHeads)),
                     dim3(64 * kPfWaves), 0, stream, pp);
  return hipGetLastError();
}

size_t prefill_workspace_bytes(int32_t L) {
  return (size_t)((L + kExpTile - 1) / kExpTile) * kExpTile * kKvStride * 2;
}

}  // namespace mla
