// Split-KV flash decoding over the latent cache on gfx950 (bf16 MFMA).
//
// What is computed (per sequence b, split of its tokens, query token j,
// head h): the online-softmax partial of
//     s_t = scale * ([q_lat | q_pe] . [c_t | k_pe_t])
// over the split's visible tokens, i.e. (O = sum_t p_t c_t / sum_t p_t,
// lse = log2 sum_t 2^(s_t log2 e)).  The cache row [c_t | k_pe_t] is what
// kv_a_proj_with_mqa writes ("mHC+MLA+MTP 是什么", MLA section); scoring
// against the latent directly is the W_UK absorption, and the LSE combine and
// W_UV up-projection of the partials follow in kernels.hip.
//
// Work decomposition (one workgroup of 8 waves, two per SIMD, per split and
// query group; a segment record of the call's schedule names the split's
// sequence, its 64-token tiles (first + i * stride) and the sequence length):
//  * The split streams through LDS in 64-token slots (one page) of a
//    two-slot ring, filled by direct global->LDS 16-byte loads (9 or 10 per
//    lane per slot): while the waves consume one slot the next is in flight.
//    A slot row in LDS is the token's 1,152 bytes followed by 32 pad bytes
//    (1,184-byte rows): with that stride both read patterns below are free of
//    LDS bank conflicts (measured with the bank-conflict counter; the
//    XOR-swizzled 1,152-byte rows used before conflicted two-way on the
//    score reads), and every read of a slot is one per-lane base plus an
//    immediate offset.
//  * The query rows come ahead of the first slot into the second ring
//    position (1,152-byte rows, latent chunk c of row r at c ^ (r & 15), rope
//    chunk 64+k at 64 + (k ^ ((r >> 1) & 7))), from where each wave takes its
//    16 rows into registers; only then is the second slot requested.  The
//    first slot is thus awaited on its own, not behind later slots.
//  * The 32*QG query rows (query token, head) are cut into row groups of 16.
//    Scores: wave w takes row group w % RG and a 64/TPW-token share of each
//    slot (TPW = 8 / RG waves per row group) and forms S^T[token][row] =
//    C_slot . Q^T on v_mfma_f32_16x16x32_bf16: cache rows as the A operand
//    (ds_read_b128, several in flight), its query rows in registers as B.
//  * Softmax without rescaling: a row's reference max m_ref is the maximum of
//    its scores in the split's first slot (taken across the row group's score
//    waves through LDS), fixed afterwards; p = 2^(s - m_ref) may grow to 2^64
//    (sums stay far inside fp32).  The score waves also track the true
//    maxima; if any score exceeds its reference by more than 64 (log2 units),
//    the workgroup streams the split a second time with the references set to
//    the true maxima, where p <= 1.
//  * P (bf16) goes to a small LDS buffer in the B-operand layout of the value
//    product; after one barrier, wave w accumulates O^T[col][row] = C^T . P^T
//    for latent columns [64w, 64w + 64) and every query row, the latent
//    values C^T fetched with ds_read_b64_tr_b16 (transposing 4 x 16 blocks).
//    Each cached value is thus read once by the value product, and a wave's
//    accumulators hold complete sums over the split: after the loop they are
//    scaled by 1 / sum_t p_t and written as row-major bf16 partial rows.
#include "mla_internal.h"

#include <hip/hip_ext.h>

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 64.0f;          // log2 headroom of p above the reference max
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kSlotTok = 64;           // tokens per ring slot (one page)
constexpr int kRowLds = kRowBytes + 32;                     // 1184: LDS bytes per slot row
constexpr int kSlotLds = kSlotTok * kRowLds;                // 75776
constexpr int kSlotInstr = kSlotLds / 1024;                 // 74 wave-wide direct loads per slot
constexpr int kWide = kSlotInstr - 9 * kWaves;              // waves 0..1 issue 10 loads per slot, the rest 9
constexpr int kSlots = 2;              // ring slots: one in flight while one is consumed
constexpr int kQLoads = 9;             // query-row loads per lane of a wave that has query rows
constexpr int kCbPerWave = kLatent / 16 / kWaves;           // 4 column blocks of 16 per wave
static_assert(kSlotInstr * 1024 == kSlotLds && kWide == 2, "slot split");

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef __attribute__((address_space(3))) const uint8_t lds_cu8;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;

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

// Wait until at most `ahead` (0 or 1) slots' worth of this wave's direct
// loads (10 per slot for the wide waves, else 9) are still outstanding.
__device__ __forceinline__ void wait_slots_ahead(bool wide, int ahead) {
  if (ahead >= 1) {
    if (wide) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// One 16-byte direct global->LDS load: LDS byte lds + 16 * lane receives the
// 16 bytes at this lane's gaddr (M0 holds the wave-uniform LDS address).
// Written out so that the compiler does not order later LDS reads of other
// slots behind it; completion is awaited explicitly with wait_slots_ahead.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gaddr)
               : "memory", "m0");
}

// The same from a wave-uniform base (moved to scalar registers) plus a
// per-lane 32-bit offset.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  const uint64_t su = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"((const void*)(uintptr_t)su)
               : "memory", "m0");
}

// Chunk <-> query-row position swizzle (an involution within each group).
__device__ __forceinline__ int tile_slot(int tok, int c) {
  return c < 64 ? (c ^ (tok & 15)) : (64 + ((c - 64) ^ ((tok >> 1) & 7)));
}

// The work of one workgroup: query tokens j0 .. j0 + QG - 1 (QG = 1 or 2)
// against segment `unit`.  The LDS buffers are the kernel's (sized for
// QG = 2), so that both instantiations called from one kernel share them.
template <int QG, bool PAGED>
__device__ __forceinline__ void splitkv_body(const DecodeParams& p, int unit, int j0, uint8_t* ring, uint8_t* pbuf,
                                             float* stat_lds, int* flags) {
  constexpr int RG = 2 * QG;           // row groups of 16 query rows
  constexpr int ROWS = 16 * RG;
  constexpr int TPW = kWaves / RG;     // score waves per row group
  constexpr int TOKW = kSlotTok / TPW; // tokens of each slot one score wave handles
  constexpr int NBLK = TOKW / 16;      // 16-token score blocks per slot and wave
  constexpr int kQkRing = QG == 1 ? 8 : 6;   // score operand reads in flight per wave
  static_assert((ROWS * kChunksPerRow) % (kQLoads * 64) == 0, "query rows fill whole waves' loads");
  static_assert(ROWS * kRowBytes <= kSlotLds, "query rows fit in a ring position");

  // per score wave and row: slot max, sum, true max
  float (*stat)[TPW][ROWS] = reinterpret_cast<float (*)[TPW][ROWS]>(stat_lds);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  const int rg = wave % RG, tq = wave / RG;   // score role: row group, token share

  const SegDesc seg = p.seg_desc[unit];   // slots first + i * stride (i < ntiles) of sequence b
  const int b = seg.b, L = seg.L;
  if (b < 0 || seg.ntiles < 1) return;   // no segment: the combine never reads it

  // Query token of the score role's rows (j0 + QG <= Sq: a last group with
  // fewer tokens runs as QG = 1).
  const int j_grp = j0 + (rg >> 1);
  const int j = j_grp < p.Sq ? j_grp : p.Sq - 1;
  const int limit = L - p.Sq + j + 1;   // rows of this wave see tokens < limit

  // Slot loads: wave-wide load I of a slot fills LDS bytes [1024 I,
  // 1024 (I + 1)) of the ring position; waves 0..1 issue loads 10w .. 10w + 9,
  // waves 2..7 loads 2 + 9w .. + 8.  Lane position P = 64 I + lane (16-byte
  // units) is chunk P % 74 of the slot's token P / 74; chunks 72 and 73 are
  // the row's pad and repeat chunks 0 and 1.  off[i]: the chunk's byte offset
  // in the slot's cache rows (the same for every slot).
  const bool wide = wave < kWide;
  const int i0 = wide ? 10 * wave : kWide + 9 * wave;
  uint32_t off[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int P = (i0 + i) * 64 + lane;
    const int tok = P / (kRowLds / 16);
    const int c = P - tok * (kRowLds / 16);
    off[i] = (uint32_t)(tok * kRowBytes + (c < kChunksPerRow ? c : c - kChunksPerRow) * 16);
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)ring);

  const int nslot = seg.ntiles;
  auto slot_at = [&](int i) { return seg.first + i * seg.stride; };   // absolute slot index

  // Enqueue slot `ts` (absolute slot index) of the sequence into ring slot
  // `r`; rows at or past L come from the zero row, so masked tokens
  // multiply zeros.
  auto issue = [&](int ts, int r) {
    const uint8_t* src;
    int nval = min(kSlotTok, L - ts * kSlotTok);
    if constexpr (PAGED) {
      const int page = p.block_table[(size_t)b * p.max_pages + ts];
      src = p.cache + (size_t)page * kTileBytes;
      if (!page_ok(page, p.num_pages)) {   // a page outside the pool: its rows are read as zeros
        if (tid == 0) raise_fault(p.faults, kFaultPage);
        src = p.cache;
        nval = 0;
      }
    } else {
      src = p.cache + ((size_t)b * p.stride_tokens + (size_t)ts * kSlotTok) * kRowBytes;
    }
    const uint32_t dst = ring_lds + r * kSlotLds + i0 * 1024;
    if (nval == kSlotTok) {
#pragma unroll
      for (int i = 0; i < 9; ++i) dma16s(src, off[i], dst + i * 1024);
      if (wide) dma16s(src, off[9], dst + 9 * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        if (i == 9 && !wide) break;
        const int tok = off[i] / kRowBytes;
        const uint8_t* a = (tok < nval) ? src + off[i] : p.zero_row + (off[i] - tok * kRowBytes);
        dma16(a, dst + i * 1024);
      }
    }
  };

  // ---- prologue: the query rows (row r of the group as "token" r, 1,152-byte
  // rows, chunk c at tile_slot(r, c)) into the second ring position, by the
  // waves 0 .. ROWS * 72 / 576 - 1 (9 loads each), the first slot into the first
  if (wave * kQLoads * 64 < ROWS * kChunksPerRow) {
    const uint32_t dst = ring_lds + kSlotLds + wave * kQLoads * 1024;
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int P = (wave * kQLoads + i) * 64 + lane;
      const int r = P / kChunksPerRow;
      const int c = tile_slot(r, P - r * kChunksPerRow);
      const int jj = min(j0 + (r >> 5), p.Sq - 1);
      const uint8_t* src = (const uint8_t*)p.qabs + (((size_t)b * p.Sq + jj) * 32 + (r & 31)) * kRowBytes + c * 16;
      dma16(src, dst + i * 1024);
    }
  }
  issue(slot_at(0), 0);
  wait_slots_ahead(wide, 1);   // the query rows (older than the first slot) have landed
  lds_barrier();
  bf16x8 q[18];   // this wave's 16 query rows as MFMA B operands: lane holds row n16, 8 dims
  {
    // row n16, chunk 4*ks + g at position (4ks + g) ^ n16 = 16*(ks/4) +
    // ((4*(ks%4)) ^ (g ^ n16)); rope chunks 64 + ((4kk + g) ^ (n16 >> 1))
    const uint8_t* qb = ring + kSlotLds + (rg * 16 + n16) * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int pos = ks < 16 ? 16 * (ks >> 2) + ((4 * (ks & 3)) ^ (g ^ n16)) : 64 + ((4 * (ks - 16) + g) ^ (n16 >> 1));
      q[ks] = *(const bf16x8*)(qb + pos * 16);
    }
  }
  lds_barrier();   // every wave has its query rows before the second slot overwrites them
  if (nslot > 1) issue(slot_at(1), 1);

  // Score reads of a slot: token n16 of a 16-token block, chunk 4*ks + g
  // (rope chunks 64 + 4kk + g follow the latent ones): one base per lane.
  const int qk_lane = n16 * kRowLds + g * 16;
  // Value reads (transposed, 8 bytes): token 4g + (n16 >> 2) (+16 for the
  // upper half of a 32-token step, +32 for the second step), columns
  // 16*cb + 4*(n16 & 3) (chunk 2cb + ((n16 >> 1) & 1), bytes 8 (n16 & 1)).
  // This wave's blocks: cb = 4*wave + c.
  const int pv_lane = (4 * g + (n16 >> 2)) * kRowLds + (n16 & 1) * 8 + ((n16 >> 1) & 1) * 16 +
                      kCbPerWave * wave * 32;
  // P reads: row n16 of a row group, one 32-token step: 16 bytes at k = 8g
  // (granule g, swizzled).
  const int pb_rd = n16 * 64 + ((g ^ ((n16 >> 1) & 3)) * 16);

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
    const int abs_w = ts * kSlotTok + tok0;    // its absolute position

    // ---- scores S^T = C . Q^T, 16 tokens per block; reads run kQkRing ahead
    constexpr int NQK = NBLK * 18;
    auto qk_src = [&](int i) -> lds_bf16x8_t* {
      const int blk = i % NBLK, ks = i / NBLK;
      return (lds_bf16x8_t*)(T + (tok0 + blk * 16) * kRowLds + qk_lane + ks * 64);
    };
    f32x4 s[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 rq[kQkRing];
#pragma unroll
    for (int i = 0; i < kQkRing; ++i) rq[i] = *qk_src(i);
    __builtin_amdgcn_sched_group_barrier(0x100, kQkRing, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int blk = i % NBLK, ks = i / NBLK;
      s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rq[i % kQkRing], q[ks], s[blk], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kQkRing < NQK) {
        rq[i % kQkRing] = *qk_src(i + kQkRing);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }

    // ---- scale, mask, slot max of row n16 over this wave's tokens
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

    // ---- P = 2^(s - m_ref) in bf16 into the value product's B-operand
    // layout: token t of the slot is step t/32, k = 8*((t%16)/4) + 4*((t/16)%2) + t%4
    const float mref = (m_ref == kNegInf) ? 0.f : m_ref;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      s16x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 e = (__bf16)__builtin_amdgcn_exp2f(s[blk][i] - mref);
        l_part += (float)e;
        pk[i] = __builtin_bit_cast(short, e);
      }
      const int t16 = tok0 + blk * 16;   // first token of the block (a multiple of 16)
      const int ks = t16 >> 5, bb = (t16 >> 4) & 1;
      *(s16x4*)(pbuf + ((rg * 2 + ks) * 16 + n16) * 64 + ((g ^ ((n16 >> 1) & 3)) * 16) + bb * 8) = pk;
    }
    lds_barrier();

    // ---- O^T += C^T . P^T over this wave's 4 column blocks and all rows
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb[RG];
#pragma unroll
      for (int r2 = 0; r2 < RG; ++r2) pb[r2] = *(const bf16x8*)(pbuf + (r2 * 2 + ks) * 1024 + pb_rd);
      s16x4 lo[kCbPerWave], hi[kCbPerWave];
#pragma unroll
      for (int c = 0; c < kCbPerWave; ++c) {
        lds_cu8* a = T + pv_lane + c * 32 + ks * 32 * kRowLds;
        lo[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)a);
        hi[c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(a + 16 * kRowLds));
      }
#pragma unroll
      for (int c = 0; c < kCbPerWave; ++c) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[c], hi[c], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int r2 = 0; r2 < RG; ++r2)
          o[c][r2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[r2], o[c][r2], 0, 0, 0);
      }
    }
  };

  // Slot loop.  Iteration it: wait for slot it (its loads and everyone
  // else's, via the barrier, which also frees the slot consumed at it - 1),
  // request slot it + 1 into that freed ring position (slot 1 came with the
  // prologue), consume slot it.  A second pass runs only if some row outgrew
  // its reference by kTau.
  for (;;) {
    for (int it = 0; it < nslot; ++it) {
      wait_slots_ahead(wide, (it == 0 && nslot > 1) ? 1 : 0);
      lds_barrier();
      if (it >= 1 && it + 1 < nslot) issue(slot_at(it + 1), (it + 1) % kSlots);
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
    for (int k = 0; k < min(kSlots, nslot); ++k) issue(slot_at(k), k);
  }

  // ---- finalize: row r = r2*16 + n16 of the group is query token
  // j0 + r/32, head r%32; partial rows [unit][j*32 + h][512] bf16
  const size_t unit_rows = (size_t)unit * p.Sq * 32;
#pragma unroll
  for (int r2 = 0; r2 < RG; ++r2) {
    const int jr = j0 + (r2 >> 1);
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

template <int QG, bool PAGED>
__global__ void __launch_bounds__(kThreads, 1) splitkv_decode(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlots * kSlotLds];
  // P in bf16, [row group][32-token step][row][32 tokens in MFMA k order];
  // 16-byte granule q of row r is stored at granule q ^ ((r >> 1) & 3), so
  // that the value product's 16-byte reads of rows 0..7 (and 8..15) fall on
  // distinct banks (with q ^ ((r % 16) >> 2) rows r and r + 2 collided: the
  // bank-conflict counter read 5.8 million cycles per verify 32x2 launch, now
  // 0.13 million)
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2 * QG * 2 * 16 * 64];
  __shared__ float stat[3 * kWaves * 16];   // [3][score waves per row group][rows of the group]
  __shared__ int flags[kWaves];
  int unit, grp;   // segment and query group
  work_item(p.groups, unit, grp);
  if (unit >= p.segments) return;
  const int j0 = QG * grp;
  if constexpr (QG > 1) {
    // the last group of an odd Sq holds one token: its workgroups run the
    // one-token body, instead of computing a repeat of the token beside it
    if (j0 + 1 == p.Sq) {
      splitkv_body<1, PAGED>(p, unit, j0, ring, pbuf, stat, flags);
      return;
    }
  }
  splitkv_body<QG, PAGED>(p, unit, j0, ring, pbuf, stat, flags);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int segments, int query_group, bool paged, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(decode_grid(segments, p.groups)), block(kThreads);
  // with events, the dispatch itself records them at kernel start and end
  if (query_group == 1) {
    if (paged) hipExtLaunchKernelGGL((splitkv_decode<1, true>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
    else hipExtLaunchKernelGGL((splitkv_decode<1, false>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
  } else {
    if (paged) hipExtLaunchKernelGGL((splitkv_decode<2, true>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
    else hipExtLaunchKernelGGL((splitkv_decode<2, false>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
  }
  return hipGetLastError();
}

}  // namespace mla
