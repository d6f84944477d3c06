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
// Work decomposition (one workgroup of 4 waves per split, described by a
// segment record {b, first token, end token, L_b} of the call's schedule):
//  * The split streams through LDS in 64-token slots (one page, 72 KiB) of a
//    two-slot ring, filled by direct global->LDS 16-byte loads: while the
//    waves consume one slot the next is in flight, and the first two slots
//    are requested before anything else.  Slot rows are swizzled at 16-byte
//    granularity (latent chunk c of token t sits at c ^ (t & 15), rope chunk
//    64+k at 64 + (k ^ ((t >> 1) & 7))) so that both read patterns below are
//    free of LDS bank conflicts.
//  * The 32*QG query rows (query token, head) are cut into row groups of 16.
//    Each wave owns one row group and a share of every slot's tokens and
//    keeps its own running max, sum and 16 x 512 fp32 accumulator (AGPRs); no
//    wave waits on another inside the loop apart from one barrier per slot.
//    With one query token two waves share a row group (32 tokens of each slot
//    apiece) and merge at the end.
//  * Scores: S^T[token][row] = C_slot . Q^T on v_mfma_f32_16x16x32_bf16, the
//    cache rows as the A operand (ds_read_b128 of 8 latent values per lane,
//    eight reads in flight) and the wave's 16 query rows held in registers as
//    the B operand.
//  * The S^T accumulator layout (lane = row, 4 tokens per lane) is exactly the
//    operand layout of P[row][token] in the value product; the latent values
//    C[token][col] are fetched in that token order with ds_read_b64_tr_b16
//    (transposing 4 x 16 blocks), so P never leaves registers.  The product
//    is taken as O^T = C^T . P^T (latent values as the A operand), so that a
//    lane's accumulator holds 4 consecutive latent columns of one row and the
//    partials leave the kernel as plain row-major fp32 rows.
//  * No rescaling inside the loop: a row's reference max is fixed at its
//    first visible slot, and p = 2^(s - m_ref) may grow to 2^64 (sums stay far
//    inside fp32).  Each wave also tracks the rows' true maxima; if any score
//    ever exceeds its reference by more than 64 (log2 units), the workgroup
//    streams the split a second time with the references set to the true
//    maxima, where p <= 1.  The accumulators are therefore only ever
//    accumulated by MFMAs, zeroed, or written to LDS after the loop.
#include "mla_internal.h"

#include <hip/hip_ext.h>

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 64.0f;          // log2 headroom of p above the reference max
constexpr int kQkRing = 8;             // score operand reads in flight per wave
constexpr int kPvRing = 6;             // value operand column blocks in flight per wave
constexpr int kSlotTok = 64;           // tokens per ring slot (one page)
constexpr int kSlotBytes = kSlotTok * kRowBytes;   // 73728
constexpr int kSlots = 2;              // ring slots: kSlots - 1 in flight while one is consumed
constexpr int kLoadsPerLane = kSlotBytes / 16 / 256;   // 18

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most `ahead` slots' worth of direct loads (kLoadsPerLane per
// lane per slot) are still outstanding.
template <int PER_SLOT>
__device__ __forceinline__ void wait_slots_ahead(int ahead) {
  if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER_SLOT) : "memory");
  else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER_SLOT) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

// Chunk <-> slot-row position swizzle (an involution within each group).
__device__ __forceinline__ int tile_slot(int tok, int c) {
  return c < 64 ? (c ^ (tok & 15)) : (64 + ((c - 64) ^ ((tok >> 1) & 7)));
}

template <int QG, bool PAGED>
__global__ void __launch_bounds__(256, 1) splitkv_decode(DecodeParams p) {
  constexpr int RG = 2 * QG;          // row groups of 16 rows
  constexpr int TP = 4 / RG;          // waves per row group
  constexpr int TOKW = kSlotTok / TP; // tokens of each slot one wave handles
  constexpr int NBLK = TOKW / 16;     // 16-token score blocks per slot

  __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlots * kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n16 = lane & 15;
  const int rg = wave % RG, tp = wave / RG;

  int unit, grp;   // segment (tokens [t_begin, t_end) of sequence b) and query group
  work_item(p.groups, unit, grp);
  if (unit >= p.segments) return;
  const int4 seg = p.seg_desc[unit];
  const int b = seg.x, t_begin = seg.y, t_end = seg.z, L = seg.w;
  if (b < 0 || t_begin >= t_end) return;   // no segment: the combine never reads it

  // Query token of this wave's rows; a repeat of token Sq - 1 (computed, never
  // written) fills the second half of the last group when Sq is odd.
  const int j_grp = QG * grp + (rg >> 1);
  const bool real = j_grp < p.Sq;
  const int j = real ? j_grp : p.Sq - 1;
  const int limit = min(t_end, L - p.Sq + j + 1);   // rows of this wave see tokens < limit
  // partial rows of this wave's row group: [unit][j*32 + h][512] fp32
  const int rg_glob = 2 * QG * grp + rg;
  float* out_o = p.part_o + ((size_t)unit * (2 * p.Sq) + rg_glob) * (16 * kLatent);
  float* out_lse = p.part_lse + (size_t)unit * (p.Sq * 32) + rg_glob * 16;

  // Byte offset inside a slot of each 16-byte chunk this lane loads: LDS
  // position P = (wave*kLoadsPerLane + i)*64 + lane holds chunk (tok = P / 72,
  // tile_slot(tok, P % 72)) of the slot's token tok.
  int off[kLoadsPerLane];
#pragma unroll
  for (int i = 0; i < kLoadsPerLane; ++i) {
    const int P = (wave * kLoadsPerLane + i) * 64 + lane;
    const int tok = P / kChunksPerRow;
    const int c = tile_slot(tok, P - tok * kChunksPerRow);
    off[i] = tok * kRowBytes + c * 16;
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)ring);

  const int s0 = t_begin / kSlotTok;                    // first slot index of the split
  const int nslot = (t_end - t_begin + kSlotTok - 1) / kSlotTok;

  // Enqueue the split's slot `ts` (absolute slot index) into ring slot
  // `r`.  Every lane issues exactly kLoadsPerLane loads; rows past the end of
  // the split come from the zero row, so masked tokens multiply zeros.
  auto issue = [&](int ts, int r) {
    const uint8_t* src;
    if constexpr (PAGED) {
      constexpr int kSlotsPerPage = kPage / kSlotTok;
      const int page = p.block_table[(size_t)b * p.max_pages + ts / kSlotsPerPage];
      src = p.cache + (size_t)page * kTileBytes + (ts % kSlotsPerPage) * kSlotBytes;
    } else {
      src = p.cache + ((size_t)b * p.stride_tokens + (size_t)ts * kSlotTok) * kRowBytes;
    }
    const int nval = min(kSlotTok, t_end - ts * kSlotTok);
    const uint32_t dst = ring_lds + r * kSlotBytes + wave * kLoadsPerLane * 1024;
    if (nval == kSlotTok) {
#pragma unroll
      for (int i = 0; i < kLoadsPerLane; ++i) dma16(src + off[i], dst + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < kLoadsPerLane; ++i) {
        const int tok = off[i] / kRowBytes;
        const uint8_t* a = (tok < nval) ? src + off[i] : p.zero_row + (off[i] - tok * kRowBytes);
        dma16(a, dst + i * 1024);
      }
    }
  };

  // The first two slots (both ring positions) are requested before the query
  // rows are read.
  const int pro = min(kSlots, nslot);
  for (int k = 0; k < pro; ++k) issue(s0 + k, k);

  // The wave's 16 query rows, as MFMA B operands: lane holds row n16, 8 dims.
  bf16x8 q[18];
  {
    const uint16_t* qrow = p.qabs + (((size_t)b * p.Sq + j) * 32 + (rg & 1) * 16 + n16) * kRow + g * 8;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) q[ks] = *(const bf16x8*)(qrow + ks * 32);
  }
  // Settle the query loads here, once: a wait the compiler placed at their
  // first use inside the slot loop would count only its own loads and so
  // also drain the cache slots requested ahead of every iteration.
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) asm volatile("" ::"v"(q[ks]));

  // LDS read offsets within a slot.  Score reads: token tok_w + 16*blk + n16,
  // chunk 4*ks + g, position (4ks + g) ^ n16 = 16*(ks/4) + ((4*(ks%4)) ^ (g ^ n16));
  // the 16*(ks/4) and 16*blk parts become instruction immediates.
  const int tok_w = tp * TOKW;
  const int qk_row = (tok_w + n16) * kRowBytes;
  int qk_off[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) qk_off[bb] = qk_row + (((4 * bb) ^ (g ^ n16)) << 4);
  int rope_off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) rope_off[kk] = qk_row + ((64 + ((4 * kk + g) ^ (n16 >> 1))) << 4);
  // Value reads (transposed, 8 bytes): token tok_w + 4g + (n16 >> 2) (+16 for
  // the upper half of a 32-token step), columns 16*cb + 4*(n16 & 3); chunk
  // 2cb + ((n16 >> 1) & 1) sits at position 16*(cb/8) + ((2*(cb%8)) ^ v).
  const int pv_tok = tok_w + 4 * g + (n16 >> 2);
  const int pv_v = ((n16 >> 1) & 1) ^ (pv_tok & 15);
  const int pv_row = pv_tok * kRowBytes + (n16 & 1) * 8;
  int pv_off[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) pv_off[bb] = pv_row + (((2 * bb) ^ pv_v) << 4);

  f32x4 o[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // reference max of row n16 (log2 units), fixed once set
  float m_true = kNegInf;  // running true max of row n16
  float l_part = 0.f;      // this lane's share of the row sum
  bool overflow = false;   // some score exceeded m_ref + kTau (wave-uniform)

  auto process = [&](const uint8_t* T, int ts) __attribute__((always_inline)) {
    const int abs_w = ts * kSlotTok + tok_w;   // absolute position of the wave's first token

    // ---- scores S^T = C . Q^T, 16 tokens per block; reads run kQkRing ahead
    constexpr int NQK = NBLK * 18;
    auto qk_src = [&](int i) -> const bf16x8* {
      const int blk = i % NBLK, ks = i / NBLK;
      const uint8_t* base = T + blk * 16 * kRowBytes;
      return (const bf16x8*)(ks < 16 ? base + qk_off[ks & 3] + (ks >> 2) * 256 : base + rope_off[ks - 16]);
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

    // ---- scale, mask, slot max of row n16
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

    // ---- reference max: set at the row's first visible slot (its
    // accumulator is still zero then), never moved afterwards
    m_true = fmaxf(m_true, mt);
    m_ref = (m_ref == kNegInf) ? mt : m_ref;
    overflow = overflow || (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0);

    // ---- P = 2^(s - m_ref) in bf16, in the A-operand layout of P . C
    const float mref = (m_ref == kNegInf) ? 0.f : m_ref;
    __bf16 pe[NBLK][4];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pe[blk][i] = (__bf16)__builtin_amdgcn_exp2f(s[blk][i] - mref);
        l_part += (float)pe[blk][i];
      }

    // ---- O += P . C[:, 0:512]; value operand by transposed LDS reads
    auto pv_src = [&](int cb) -> const uint8_t* { return T + pv_off[cb & 7] + (cb >> 3) * 256; };
    if constexpr (NBLK == 1) {
      // 16 tokens: v_mfma_f32_16x16x16_bf16, one 4-token transposed read per block
      s16x4 pa;
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = __builtin_bit_cast(short, pe[0][i]);
      s16x4 rv[kPvRing];
#pragma unroll
      for (int i = 0; i < kPvRing; ++i) rv[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)pv_src(i));
      __builtin_amdgcn_sched_group_barrier(0x100, kPvRing, 1);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) {
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(rv[cb % kPvRing], pa, o[cb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (cb + kPvRing < 32) {
          rv[cb % kPvRing] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)pv_src(cb + kPvRing));
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
      }
    } else {
      // 32-token k-steps: v_mfma_f32_16x16x32_bf16, two transposed reads per
      // block (tokens 4g+e and 16+4g+e, the order of the score accumulator)
      constexpr int NKV = NBLK / 2;
      constexpr int NPV = NKV * 32;
      bf16x8 pa[NKV];
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) { pa[kk][i] = pe[2 * kk][i]; pa[kk][4 + i] = pe[2 * kk + 1][i]; }
      auto pv_at = [&](int i) -> const uint8_t* { return pv_src(i % 32) + (i / 32) * 32 * kRowBytes; };
      s16x4 lo[kPvRing], hi[kPvRing];
#pragma unroll
      for (int i = 0; i < kPvRing; ++i) {
        lo[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)pv_at(i));
        hi[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(pv_at(i) + 16 * kRowBytes));
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvRing, 1);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int kk = i / 32, cb = i % 32, r = i % kPvRing;
        const s16x8 both = __builtin_shufflevector(lo[r], hi[r], 0, 1, 2, 3, 4, 5, 6, 7);
        o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, both), pa[kk], o[cb], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (i + kPvRing < NPV) {
          lo[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)pv_at(i + kPvRing));
          hi[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(pv_at(i + kPvRing) + 16 * kRowBytes));
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
      }
    }
  };

  // Slot loop.  Iteration it: wait for slot it (its loads and everyone
  // else's, via the barrier, which also frees the slot consumed at it - 1),
  // request slot it + 1 into that freed ring position (slot 1 came with the
  // prologue), consume slot it.  Only while slot 0 is awaited can a later
  // slot's loads be outstanding.
  // A second pass runs only if some row outgrew its reference by kTau.
  int pass = 0;
  for (;;) {
    for (int it = 0; it < nslot; ++it) {
      wait_slots_ahead<kLoadsPerLane>((it == 0 && nslot > 1) ? 1 : 0);
      lds_barrier();
      if (it >= 1 && it + 1 < nslot) issue(s0 + it + 1, (it + 1) % kSlots);
      process(ring + (it % kSlots) * kSlotBytes, s0 + it);
    }
    lds_barrier();   // every wave is done with the last slot
    int* flag = (int*)ring;
    if (lane == 0) flag[wave] = overflow ? 1 : 0;
    lds_barrier();
    const bool again = (flag[0] | flag[1] | flag[2] | flag[3]) != 0;
    lds_barrier();
    if (!again || pass == 1) break;
    pass = 1;
    m_ref = m_true;
    overflow = false;
    l_part = 0.f;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < pro; ++k) issue(s0 + k, k);
  }

  // ---- finalize.  The accumulators go to LDS straight from AGPRs; each
  // wave then reads them back four values at a time, merges the two token
  // halves of its row group (one query token) and normalises.  Keeping every
  // use of the accumulators out of the vector ALU lets them stay in AGPRs.
  float l_row = l_part;
  l_row += __shfl_xor(l_row, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);

  constexpr int kRegion = 32 * 64 * 4 + 32;   // floats: accumulators + m + l
  float* mine = (float*)ring + wave * kRegion;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) *(f32x4*)(mine + (cb * 64 + lane) * 4) = o[cb];
  if (lane < 16) {
    mine[32 * 64 * 4 + lane] = m_ref;
    mine[32 * 64 * 4 + 16 + lane] = l_row;
  }
  lds_barrier();

  float a_own = 1.f, a_other = 0.f;
  const float* other = nullptr;
  if constexpr (TP == 2) {
    if (tp == 1) return;
    other = (const float*)ring + (wave + RG) * kRegion;   // the wave sharing these rows
    const float m1 = other[32 * 64 * 4 + n16], l1 = other[32 * 64 * 4 + 16 + n16];
    const float mm = fmaxf(m_ref, m1);
    a_own = (m_ref == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
    a_other = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_row = l_row * a_own + l1 * a_other;
    m_ref = mm;
  }
  // lane (g, n16) holds row n16, columns 16*cb + 4g .. 16*cb + 4g + 3
  if (!real) return;
  const float inv = (l_row > 0.f) ? 1.f / l_row : 0.f;
  const float s_own = a_own * inv, s_other = a_other * inv;
  float* orow = out_o + n16 * kLatent + 4 * g;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) {
    f32x4 v = *(const f32x4*)(mine + (cb * 64 + lane) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= s_own;
    if constexpr (TP == 2) {
      const f32x4 w = *(const f32x4*)(other + (cb * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fmaf(w[i], s_other, v[i]);
    }
    *(f32x4*)(orow + cb * 16) = v;
  }
  if (lane < 16) out_lse[lane] = (l_row > 0.f) ? m_ref + __log2f(l_row) : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int segments, int query_group, bool paged, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(decode_grid(segments, p.groups)), block(256);
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
