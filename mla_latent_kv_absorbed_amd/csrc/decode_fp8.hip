// Split-KV flash decoding over the 8-bit latent cache on gfx950.
//
// The cache row of a token is [512 E4M3 codes | 4 fp32 scales | 64 bf16 rope
// key] (656 bytes): the 8-bit KV cache of "256K 长上下文真能本地用", §三
// (plan A), in the gfx950 8-bit float format with one scale per 128 latent
// values.  What is computed is the attention of the bf16 kernel (decode.hip)
// on the dequantised latent c = code * scale:
//     s_t = scale_softmax * (sum_g scale_{t,g} (q_lat,g . code_{t,g}) + q_pe . k_pe_t)
//     O   = sum_t p_t sum_g scale_{t,g} code_{t,g} / sum_t p_t
// The work is split as in the bf16 kernel (8 waves, two per SIMD; scores by
// row group and token share, the value product by latent columns, P through
// LDS):
//  * scores: the codes of a 128-column group are read as 32 bytes per lane
//    (two ds_read_b128) and multiplied on the 8-bit matrix path
//    (v_mfma_scale_f32_16x16x128_f8f6f4) by the absorbed query, which the
//    preparation kernel split exactly into two E4M3 pieces with a
//    power-of-two scale per 32 columns (the instruction's block scales);
//    each group has its own score accumulator, and the four are combined
//    with the tokens' scales (the rope part has its own bf16 accumulator);
//  * values: O^T = C^T P'^T with P'_g = bf16(p * scale_{t,g}) for the
//    columns of group g: the score waves write P'_g of all four groups to
//    LDS, and each value wave (its 64 columns lie in one group) reads its
//    group's; the codes are fetched column-wise with the 8-bit transposing
//    read ds_read_b64_tr_b8
//    (lanes 2r, 2r+1 of a 16-lane group supply the two halves of row r's 16
//    bytes; lane i receives byte i of rows 0..7), which gives each lane 8
//    tokens of one column in the MFMA k order, and widened to bf16 exactly
//    (E4M3 values are exact in bf16) for v_mfma_f32_16x16x32_bf16.
// Slots of 64 tokens (41,984 bytes, 43,008 in LDS) stream through a three-slot LDS ring, so
// two slots are in flight while one is consumed; waves 0-3 issue the direct
// loads.  The query records arrive the same way ahead of the first slot.  A
// workgroup serves QG query tokens of 32 rows each (QG = 1 when Sq = 1, else
// 2: two tokens' P' buffers and the ring fill LDS to within 480 bytes);
// further query groups of a split are served by workgroups that read the
// split together (work_item).
#include "mla_internal.h"

#include <hip/hip_ext.h>

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 64.0f;                              // log2 headroom above the reference max
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kDmaLanes = 256;                             // waves 0-3 issue the direct loads
constexpr int kSlotTok = 64;
constexpr int kSlotBytes = kSlotTok * kF8Row;              // 41984
constexpr int kChunks = kSlotBytes / 16;                   // 2624 sixteen-byte chunks
constexpr int kF8ChunksPerRow = kF8Row / 16;               // 41
constexpr int kRowLds = kF8Row + 16;                       // 672: a row in LDS and a 16-byte pad
constexpr int kRowChunksLds = kRowLds / 16;                // 42
constexpr int kSlotWaveLoads = kSlotTok * kRowChunksLds / 64;   // 42 wave-wide 16-byte loads per slot
constexpr int kLoadsPerLane = (kSlotWaveLoads + 3) / 4;    // 11: waves 0-2
constexpr int kLoadsLastWave = kSlotWaveLoads - 3 * kLoadsPerLane;   // 9: wave 3
constexpr int kSlotLds = kSlotWaveLoads * 1024;            // 43008: the slot's 64 rows of 672 bytes
constexpr int kSlots = 3;
constexpr int kCbPerWave = kLatent / 16 / kWaves;          // 4 column blocks of 16 per wave

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4_t;
typedef __attribute__((address_space(3))) const uint8_t lds_cu8;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4_t;
typedef __attribute__((address_space(3))) const float lds_f32_t;

// LDS address of a ring position, opaque to the compiler: all reads of a
// slot then share one base register and use immediate offsets, instead of
// addresses precomputed for every ring position.
__device__ __forceinline__ lds_cu8* slot_base(uint32_t lds) {
  asm volatile("" : "+s"(lds));
  return (lds_cu8*)lds;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most `ahead` slots' worth of direct loads (N per slot) are
// outstanding.
template <int N>
__device__ __forceinline__ void wait_loads_ahead(int ahead) {
  if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * N) : "memory");
  else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// The same for this wave: waves 0-2 issue kLoadsPerLane loads per slot,
// wave 3 kLoadsLastWave (waves that issue none pass at once).
__device__ __forceinline__ void wait_slots_ahead(int ahead, bool last_dma_wave) {
  if (last_dma_wave) wait_loads_ahead<kLoadsLastWave>(ahead);
  else wait_loads_ahead<kLoadsPerLane>(ahead);
}

// One 16-byte direct global->LDS load from a wave-uniform base plus a
// per-lane 32-bit offset (LDS byte lds + 16 * lane).
// The base must be wave-uniform; it is moved to scalar registers explicitly.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t su = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"((const void*)(uintptr_t)su)
               : "memory", "m0");
}

// One 16-byte direct global->LDS load (LDS byte lds + 16 * lane).
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gaddr)
               : "memory", "m0");
}

// Eight E4M3 codes (bytes 0..7 of two dwords) -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(i32x2 w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}


// One latent group's scores on the 8-bit matrix path: codes (unit scale) times
// the query's hi and lo pieces, whose block scales are byte K of sh and sl.
template <int K>
__device__ __forceinline__ f32x4 mfma_q8(const i32x8& a, const i32x8& qh, const i32x8& ql, uint32_t sh, uint32_t sl,
                                         f32x4 c) {
  c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qh, c, 0, 0, 0, 127, K, (int)sh);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, ql, c, 0, 0, 0, 127, K, (int)sl);
}

template <int QG, bool PAGED>
__global__ void __launch_bounds__(kThreads, 1) splitkv_decode_fp8(DecodeParams p) {
  constexpr int RG = 2 * QG;           // row groups of 16 query rows
  constexpr int ROWS = 16 * RG;
  constexpr int TPW = kWaves / RG;     // score waves per row group
  constexpr int TOKW = kSlotTok / TPW; // tokens of each slot one score wave handles
  constexpr int NBLK = TOKW / 16;      // 16-token score blocks per slot and wave
  constexpr int NQ = ROWS * (kQRecBytes / 16) / kDmaLanes;   // query-record loads per DMA lane
  static_assert(NQ * kDmaLanes * 16 == ROWS * kQRecBytes, "query records split");
  static_assert(ROWS * kQRecBytes <= (kSlots - 1) * kSlotLds, "query records fit in ring positions 1..2");

  __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlots * kSlotLds];
  // P'_G = bf16(p * scale_G) for the four latent groups G, [G][row group]
  // [32-token step][row][32 tokens in MFMA k order]; 16-byte granule q of row
  // r is stored at granule q ^ ((r >> 1) & 3) (conflict-free 16-byte reads
  // of 8 consecutive rows, as in decode.hip)
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[4 * RG * 2 * 16 * 64];
  __shared__ float stat[3][TPW][ROWS];   // per score wave and row: slot max, sum, true max
  __shared__ int flags[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  const int rg = wave % RG, tq = wave / RG;   // score role: row group, token share
  const bool dma_wave = wave < kDmaLanes / 64;
  const bool last_dma_wave = wave == kDmaLanes / 64 - 1;

  int unit, grp;   // segment and query group
  work_item(p.groups, unit, grp);
  if (unit >= p.segments) return;
  const SegDesc seg = p.seg_desc[unit];   // slots first + i * stride (i < ntiles) of sequence b
  const int b = seg.b, L = seg.L;
  if (b < 0 || seg.ntiles < 1) return;   // no segment: the combine never reads it

  // Query token of the score role's rows; a repeat of token Sq - 1 (computed,
  // never written) fills the second half of the last group when Sq is odd.
  const int j_grp = QG * grp + (rg >> 1);
  const int j = j_grp < p.Sq ? j_grp : p.Sq - 1;
  const int limit = L - p.Sq + j + 1;   // rows of this wave see tokens < limit

  const uint32_t ring_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)ring);
  const int nslot = seg.ntiles;
  auto slot_at = [&](int i) { return seg.first + i * seg.stride; };   // absolute slot index

  // A slot is copied by waves 0-3 into 672-byte LDS rows: LDS chunk
  // P = (wave * kLoadsPerLane + i) * 64 + lane is chunk c = P % 42 of token
  // P / 42, i.e. slot chunk P - P / 42 (the row pad c = 41 repeats the row's
  // chunk 0); the 42 wave-wide loads are loads 0..10 of waves 0-2 and 0..8
  // of wave 3.
  // With 672-byte rows (mod 256 the same as the bf16 kernel's 1,184-byte
  // rows) the 16-byte score reads of 16 consecutive rows are free of bank
  // conflicts, which the bank-conflict counter showed for 656-byte rows.
  // dma_off: the slot byte offsets of this lane's loads, two per register.
  uint32_t dma_off[(kLoadsPerLane + 1) / 2];
#pragma unroll
  for (int i = 0; i < (kLoadsPerLane + 1) / 2; ++i) dma_off[i] = 0u;
#pragma unroll
  for (int i = 0; i < kLoadsPerLane; ++i) {
    const int P = (wave * kLoadsPerLane + i) * 64 + lane;
    const int tok = (P * 3121) >> 17;   // P / 42 for P < 4096
    const int c = P - kRowChunksLds * tok;
    int chunk = P - tok - (c == kF8ChunksPerRow ? kF8ChunksPerRow : 0);
    if (tok >= kSlotTok) chunk -= kChunks;
    dma_off[i >> 1] |= (uint32_t)(16 * chunk) << (16 * (i & 1));
  }
  auto issue = [&](int ts, int r) {
    if (!dma_wave) return;
    const uint8_t* src;
    int nval = min(kSlotTok, L - ts * kSlotTok);
    if constexpr (PAGED) {
      const int page = p.block_table[(size_t)b * p.max_pages + ts];
      src = p.cache + (size_t)page * kF8Tile;
      if (!page_ok(page, p.num_pages)) {   // a page outside the pool: its rows are read as zeros
        if (tid == 0) raise_fault(p.faults, kFaultPage);
        src = p.cache;
        nval = 0;
      }
    } else {
      src = p.cache + ((size_t)b * p.stride_tokens + (size_t)ts * kSlotTok) * kF8Row;
    }
    const uint32_t dst = ring_lds + r * kSlotLds + wave * kLoadsPerLane * 1024;
    if (nval == kSlotTok) {
#pragma unroll
      for (int i = 0; i < kLoadsPerLane; ++i) {
        if (i >= kLoadsLastWave && last_dma_wave) break;
        dma16s(src, (dma_off[i >> 1] >> (16 * (i & 1))) & 0xFFFFu, dst + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerLane; ++i) {
        if (i >= kLoadsLastWave && last_dma_wave) break;
        const int P = (wave * kLoadsPerLane + i) * 64 + lane;
        const int tok = (P * 3121) >> 17;
        const int c = P - kRowChunksLds * tok;
        const int cc = c < kF8ChunksPerRow ? c : 0;
        const uint8_t* a = (tok < nval) ? src + (tok * kF8ChunksPerRow + cc) * 16 : p.zero_row + cc * 16;
        dma16(a, dst + i * 1024);
      }
    }
  };


  // ---- prologue: the ROWS query records of the group (token by token, head
  // order, kQRecBytes each, contiguous in the workspace) into ring positions
  // 1..2, copied linearly (the records of a token past Sq - 1, in the last
  // group of an odd Sq, repeat those of token Sq - 1), the first slot into
  // position 0
  if (dma_wave) {
    const uint32_t dst = ring_lds + kSlotLds + wave * NQ * 1024;
    const uint8_t* src = (const uint8_t*)p.qabs + ((size_t)b * p.Sq + QG * grp) * 32 * kQRecBytes;
    const int tokens_here = p.Sq - QG * grp;   // query tokens of this group present (>= 1)
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      int off = ((wave * NQ + i) * 64 + lane) * 16;
      if (QG > 1 && off >= tokens_here * 32 * kQRecBytes) off -= 32 * kQRecBytes;
      dma16(src + off, dst + i * 1024);
    }
  }
  issue(slot_at(0), 0);
  wait_slots_ahead(1, last_dma_wave);   // the query rows (older than the first slot) have landed
  lds_barrier();
  // This wave's 16 query rows as MFMA B operands, lane (g, n16) holding row
  // n16: for latent group k the E4M3 pieces of columns 128k + 16g .. + 16 and
  // 128k + 64 + 16g .. + 16 (the columns of the cache codes the lane reads;
  // the matrix instruction pairs element i of A and B lanes of one group, and
  // takes the scale of the 32 columns 128k + 32b .. of row n from lane
  // (b, n)), the scale bytes of blocks 4k + g for k = 0..3 in one register,
  // and the bf16 rope part (dims 8 (4kk + g) .. + 8).
  i32x8 qh[4], ql[4];
  bf16x8 qrope[2];
  uint32_t qsh, qsl;
  {
    const uint8_t* qb = ring + kSlotLds + (rg * 16 + n16) * kQRecBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const i32x4 h0 = *(const i32x4*)(qb + kQRecHi + 128 * k + 16 * g);
      const i32x4 h1 = *(const i32x4*)(qb + kQRecHi + 128 * k + 64 + 16 * g);
      const i32x4 l0 = *(const i32x4*)(qb + kQRecLo + 128 * k + 16 * g);
      const i32x4 l1 = *(const i32x4*)(qb + kQRecLo + 128 * k + 64 + 16 * g);
      qh[k] = i32x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      ql[k] = i32x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qrope[kk] = *(const bf16x8*)(qb + kQRecRope + (4 * kk + g) * 16);
    qsh = *(const uint32_t*)(qb + kQRecScaleOff + 4 * g);
    qsl = qsh - 0x04040404u;   // lo pieces carry a factor 16 (scale bytes are at least 4)
  }
  lds_barrier();   // every wave has its query rows before slots 1..2 overwrite them
  const int pro = min(kSlots, nslot);
  for (int k = 1; k < pro; ++k) issue(slot_at(k), k);

  // value reads: lanes 2r, 2r+1 of the 16-lane group g fetch token
  // t(g, r) = 4g + r (r < 4) or 16 + 4g + r - 4 (+32 for the second step),
  // bytes 8 (lane & 1) of each 16-column block; this wave's blocks are
  // cb = 4*wave + c, all in latent group wave / 2.
  const int r8 = (lane & 15) >> 1;
  const int vtok = (r8 < 4) ? 4 * g + r8 : 12 + 4 * g + r8;
  const int v_off = vtok * kRowLds + (lane & 1) * 8 + kCbPerWave * wave * 16;
  const int pgrp = wave >> 1;
  // lane (n16, g) of a value wave reads granule g of P' row n16 of its group
  const int pb_rd = pgrp * (RG * 2 * 16 * 64) + n16 * 64 + ((g ^ ((n16 >> 1) & 3)) * 16);

  f32x4 o[kCbPerWave][RG];
#pragma unroll
  for (int c = 0; c < kCbPerWave; ++c)
#pragma unroll
    for (int r2 = 0; r2 < RG; ++r2) o[c][r2] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // reference max of row rg*16 + n16 (log2 units), fixed once set
  float m_true = kNegInf;  // running true max of that row over this wave's tokens
  float l_part = 0.f;      // this lane's share of the row sum
  bool overflow = false;   // some score exceeded m_ref + kTau (wave-uniform)
  int pass = 0;

  auto process = [&](lds_cu8* T, int ts, bool first) __attribute__((always_inline)) {
    const int tok0 = tq * TOKW;                // first token of this wave's share
    const int abs_w = ts * kSlotTok + tok0;

    // ---- scores, per 16-token block: four latent groups and the rope part;
    // the reads of one group are in flight while the previous one is widened
    // and multiplied
    float s[NBLK][4];
    float mt = kNegInf;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      __builtin_amdgcn_sched_barrier(0);
      lds_cu8* rowb = T + (tok0 + 16 * blk + n16) * kRowLds + g * 16;
      f32x4 sg[5];
#pragma unroll
      for (int k = 0; k < 5; ++k) sg[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      i32x4 cur[2], nxt[2];   // 64-column blocks 2k, 2k + 1 of group k
#pragma unroll
      for (int i = 0; i < 2; ++i) cur[i] = *(const lds_i32x4_t*)(rowb + i * 64);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < 3) {
#pragma unroll
          for (int i = 0; i < 2; ++i) nxt[i] = *(const lds_i32x4_t*)(rowb + (2 * (k + 1) + i) * 64);
        }
        __builtin_amdgcn_sched_barrier(0);
        {
          // codes x (hi + lo / 16) * 2^-e on the 8-bit matrix path: the codes
          // with unit scale (127), the query pieces with their block scales
          const i32x8 a = i32x8{cur[0][0], cur[0][1], cur[0][2], cur[0][3], cur[1][0], cur[1][1], cur[1][2], cur[1][3]};
          sg[k] = k == 0 ? mfma_q8<0>(a, qh[k], ql[k], qsh, qsl, sg[k])
                  : k == 1 ? mfma_q8<1>(a, qh[k], ql[k], qsh, qsl, sg[k])
                  : k == 2 ? mfma_q8<2>(a, qh[k], ql[k], qsh, qsl, sg[k])
                           : mfma_q8<3>(a, qh[k], ql[k], qsh, qsl, sg[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (k < 3) {
#pragma unroll
          for (int i = 0; i < 2; ++i) cur[i] = nxt[i];
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 rp = *(lds_bf16x8_t*)(rowb + kF8RopeOff + kk * 64);
        sg[4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rp, qrope[kk], sg[4], 0, 0, 0);
      }
      // combine the groups with the tokens' scales, scale, mask
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 sc = *(lds_f32x4_t*)(T + (tok0 + 16 * blk + 4 * g + i) * kRowLds + kF8ScaleOff);
        float v = sg[4][i];
#pragma unroll
        for (int k = 0; k < 4; ++k) v = fmaf(sc[k], sg[k][i], v);
        const int t = abs_w + 16 * blk + 4 * g + i;
        v = (t < limit) ? v * p.scale_log2 : kNegInf;
        s[blk][i] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    m_true = fmaxf(m_true, mt);

    // ---- reference max: the row's maximum over the split's first slot, the
    // same for every wave of the row group
    if (first && pass == 0) {
      if (g == 0) stat[0][tq][rg * 16 + n16] = mt;
      lds_barrier();
      float m = stat[0][0][rg * 16 + n16];
#pragma unroll
      for (int k = 1; k < TPW; ++k) m = fmaxf(m, stat[0][k][rg * 16 + n16]);
      m_ref = m;
    }
    overflow = overflow || (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0);

    // ---- p = 2^(s - m_ref), and P'_G = bf16(p * scale_G) of every group into
    // LDS in the value product's B-operand layout: token t of the slot is step
    // t/32, k = 8*((t%16)/4) + 4*((t/16)%2) + t%4
    const float mref = (m_ref == kNegInf) ? 0.f : m_ref;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      f32x4 pf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = __builtin_amdgcn_exp2f(s[blk][i] - mref);
        l_part += (float)(__bf16)pf[i];
      }
      const int t16 = tok0 + blk * 16;
      const int ks = t16 >> 5, bb = (t16 >> 4) & 1;
      f32x4 sc[4];   // the four group scales of token 4g + i of the block
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = *(lds_f32x4_t*)(T + (t16 + 4 * g + i) * kRowLds + kF8ScaleOff);
      uint8_t* pw = pbuf + ((rg * 2 + ks) * 16 + n16) * 64 + ((g ^ ((n16 >> 1) & 3)) * 16) + bb * 8;
#pragma unroll
      for (int G = 0; G < 4; ++G) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)(pf[i] * sc[i][G]);
        *(bf16x4*)(pw + G * (RG * 2 * 16 * 64)) = v;
      }
    }
    lds_barrier();

    // ---- O^T += C^T . P'^T over this wave's 4 column blocks and all rows,
    // with P' of this wave's latent group
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      i32x2 cv[kCbPerWave];
#pragma unroll
      for (int c = 0; c < kCbPerWave; ++c)
        cv[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(T + ks * 32 * kRowLds + v_off + c * 16));
      bf16x8 pb[RG];
#pragma unroll
      for (int r2 = 0; r2 < RG; ++r2) pb[r2] = *(const bf16x8*)(pbuf + pb_rd + (r2 * 2 + ks) * (16 * 64));
#pragma unroll
      for (int c = 0; c < kCbPerWave; ++c) {
        const bf16x8 av = e4m3x8_to_bf16(cv[c]);
#pragma unroll
        for (int r2 = 0; r2 < RG; ++r2)
          o[c][r2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[r2], o[c][r2], 0, 0, 0);
      }
    }
  };

  // Slot loop.  Iteration it: wait for slot it (everyone's loads, via the
  // barrier, which also frees the ring position of slot it - 1), request slot
  // it + 2 into that position (slots 0..2 came with the prologue), consume
  // slot it.  A second pass runs only if some row outgrew its reference.
  for (;;) {
    for (int it = 0; it < nslot; ++it) {
      wait_slots_ahead(it == 0 ? pro - 1 : min(nslot, it + 2) - it - 1, last_dma_wave);
      lds_barrier();
      if (it >= 1 && it + 2 < nslot) issue(slot_at(it + 2), (it + 2) % kSlots);
      process(slot_base(ring_lds + (it % kSlots) * kSlotLds), slot_at(it), it == 0);
    }
    // row sums and true maxima of each score wave's token share
    float lsum = l_part;
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (g == 0) {
      stat[1][tq][rg * 16 + n16] = lsum;
      stat[2][tq][rg * 16 + n16] = m_true;
    }
    if (lane == 0) flags[wave] = overflow ? 1 : 0;
    lds_barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) any |= flags[w];
    if (any == 0 || pass == 1) break;
    pass = 1;
    float m = stat[2][0][rg * 16 + n16];
#pragma unroll
    for (int k = 1; k < TPW; ++k) m = fmaxf(m, stat[2][k][rg * 16 + n16]);
    m_ref = m;
    overflow = false;
    l_part = 0.f;
#pragma unroll
    for (int c = 0; c < kCbPerWave; ++c)
#pragma unroll
      for (int r2 = 0; r2 < RG; ++r2) o[c][r2] = f32x4{0.f, 0.f, 0.f, 0.f};
    lds_barrier();   // flags and stat read by everyone before they are written again
    for (int k = 0; k < pro; ++k) issue(slot_at(k), k);
  }

  // ---- finalize: row r = r2*16 + n16 of the group is query token
  // QG*grp + r/32, head r%32; partial rows [unit][j*32 + h][512] bf16
  const size_t unit_rows = (size_t)unit * p.Sq * 32;
#pragma unroll
  for (int r2 = 0; r2 < RG; ++r2) {
    const int jr = QG * grp + (r2 >> 1);
    if (jr >= p.Sq) continue;
    const int r = r2 * 16 + n16;
    float lrow = stat[1][0][r];
#pragma unroll
    for (int k = 1; k < TPW; ++k) lrow += stat[1][k][r];
    const float inv = (lrow > 0.f) ? 1.f / lrow : 0.f;
    uint16_t* orow = p.part_o + (unit_rows + (size_t)jr * 32 + (r & 31)) * kLatent + 4 * g;
#pragma unroll
    for (int c = 0; c < kCbPerWave; ++c) {
      s16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(short, (__bf16)(o[c][r2][i] * inv));
      *(s16x4*)(orow + (kCbPerWave * wave + c) * 16) = v;
    }
    if (tq == 0 && r2 == rg && g == 0)
      p.part_lse[unit_rows + (size_t)jr * 32 + (r & 31)] = (lrow > 0.f) ? m_ref + __log2f(lrow) : kNegInf;
  }
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeParams& p, int segments, int qg, bool paged, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(decode_grid(segments, p.groups)), block(kThreads);
  if (qg == 2) {
    if (paged) hipExtLaunchKernelGGL((splitkv_decode_fp8<2, true>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
    else hipExtLaunchKernelGGL((splitkv_decode_fp8<2, false>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
  } else {
    if (paged) hipExtLaunchKernelGGL((splitkv_decode_fp8<1, true>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
    else hipExtLaunchKernelGGL((splitkv_decode_fp8<1, false>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
  }
  return hipGetLastError();
}

}  // namespace mla
