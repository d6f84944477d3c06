// Split-KV flash decoding over the 8-bit latent cache on gfx950.
//
// The cache row of a token is [512 E4M3 codes | 4 fp32 scales | 64 bf16 rope
// key] (656 bytes): the 8-bit KV cache of "256K 长上下文真能本地用", §三
// (plan A), in the gfx950 8-bit float format with one scale per 128 latent
// values.  What is computed is the attention of the bf16 kernel (decode.hip)
// on the dequantised latent c = code * scale:
//     s_t = scale_softmax * (sum_g scale_{t,g} (q_lat,g . code_{t,g}) + q_pe . k_pe_t)
//     O   = sum_t p_t sum_g scale_{t,g} code_{t,g} / sum_t p_t
// E4M3 values are exact in bf16, so both products stay on bf16 MFMA:
//  * scores: the codes of 32 latent columns are read as 8 bytes per lane
//    (ds_read_b64) and widened to bf16 exactly; each 128-column group has its
//    own score accumulator, and the four are combined with the tokens'
//    scales (the rope part has its own accumulator, unscaled);
//  * values: O^T = C^T P'^T with P'_g = bf16(p * scale_{t,g}) for the
//    columns of group g; the codes are fetched column-wise with the 8-bit
//    transposing read ds_read_b64_tr_b8 (lanes 2r, 2r+1 of a 16-lane group
//    supply the two halves of row r's 16 bytes; lane i receives byte i of
//    rows 0..7), which gives each lane 8 tokens of one column in the order
//    of the score accumulator, and widened to bf16 exactly.
// Slots of 64 tokens (41,984 bytes) stream through a three-slot LDS ring, so
// two slots are in flight while one is consumed.  Everything else (segment
// records, reference max with a second pass, finalisation) is as in the bf16
// kernel.
#include "mla_internal.h"

#include <hip/hip_ext.h>

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 64.0f;                              // log2 headroom above the reference max
constexpr int kSlotTok = 64;
constexpr int kSlotBytes = kSlotTok * kF8Row;              // 41984
constexpr int kChunks = kSlotBytes / 16;                   // 2624 sixteen-byte chunks
constexpr int kChunksPerRow = kF8Row / 16;                 // 41
constexpr int kLoadsPerLane = (kChunks + 255) / 256;       // 11
constexpr int kSlotLds = kLoadsPerLane * 256 * 16;         // 45056: the slot and a pad
constexpr int kSlots = 3;
constexpr int kBatch = 8;                                // LDS reads per pipeline stage

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most `ahead` slots' worth of direct loads are outstanding.
__device__ __forceinline__ void wait_slots_ahead(int ahead) {
  if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLoadsPerLane) : "memory");
  else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsPerLane) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Wait until at most N LDS operations of this wave are outstanding (they
// complete in issue order).
template <int N>
__device__ __forceinline__ void lds_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
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

template <int QG, bool PAGED>
__global__ void __launch_bounds__(256, 1) splitkv_decode_fp8(DecodeParams p) {
  constexpr int RG = 2 * QG;          // row groups of 16 rows
  constexpr int TP = 4 / RG;          // waves per row group
  constexpr int TOKW = kSlotTok / TP; // tokens of each slot one wave handles
  constexpr int NSUB = TOKW / 32;     // 32-token steps per slot

  __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlots * kSlotLds];

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

  // A slot is copied linearly: LDS byte 16 P <- slot byte 16 P for the
  // kLoadsPerLane chunks P = (wave * kLoadsPerLane + i) * 64 + lane; chunks
  // past the slot fill a pad from the zero row.
  int ptok[kLoadsPerLane];
#pragma unroll
  for (int i = 0; i < kLoadsPerLane; ++i) {
    const int P = (wave * kLoadsPerLane + i) * 64 + lane;
    ptok[i] = (P < kChunks) ? P / kChunksPerRow : kSlotTok;
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)ring);

  const int s0 = t_begin / kSlotTok;
  const int nslot = (t_end - t_begin + kSlotTok - 1) / kSlotTok;

  auto issue = [&](int ts, int r) {
    const uint8_t* src;
    if constexpr (PAGED) {
      const int page = p.block_table[(size_t)b * p.max_pages + ts];
      src = p.cache + (size_t)page * kF8Tile;
    } else {
      src = p.cache + ((size_t)b * p.stride_tokens + (size_t)ts * kSlotTok) * kF8Row;
    }
    const int nval = min(kSlotTok, t_end - ts * kSlotTok);
    const uint32_t dst = ring_lds + r * kSlotLds + wave * kLoadsPerLane * 1024;
#pragma unroll
    for (int i = 0; i < kLoadsPerLane; ++i) {
      const int P = (wave * kLoadsPerLane + i) * 64 + lane;
      const uint8_t* a = (ptok[i] < nval) ? src + P * 16
                                          : p.zero_row + (P - ptok[i] * kChunksPerRow) % kChunksPerRow * 16;
      dma16(a, dst + i * 1024);
    }
  };

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

  const int tok_w = tp * TOKW;
  // value reads: lanes 2r, 2r+1 of the 16-lane group g fetch token
  // t(g, r) = 4g + r (r < 4) or 16 + 4g + r - 4, bytes 8 (lane & 1) of each
  // 16-column block
  const int r8 = (lane & 15) >> 1;
  const int vtok = (r8 < 4) ? 4 * g + r8 : 12 + 4 * g + r8;
  const int v_off = vtok * kF8Row + (lane & 1) * 8;

  f32x4 o[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf;   // reference max of row n16 (log2 units), fixed once set
  float m_true = kNegInf;  // running true max of row n16
  float l_part = 0.f;      // this lane's share of the row sum
  bool overflow = false;   // some score exceeded m_ref + kTau (wave-uniform)

  auto process = [&](const uint8_t* T, int ts) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int tok0 = tok_w + 32 * sub;          // first token of this step within the slot
      const int abs0 = ts * kSlotTok + tok0;

      // ---- scores, per 16-token block: four latent groups and the rope part.
      // The block scales are requested first.
      const uint8_t* rowb = T + (tok0 + n16) * kF8Row + g * 8;   // block 0; block 1 is 16 rows on
      f32x4 sc[2][4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[blk][i] = *(const lds_f32x4_t*)(T + (tok0 + 16 * blk + 4 * g + i) * kF8Row + kF8ScaleOff);
      f32x4 sg[2][5];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int k = 0; k < 5; ++k) sg[blk][k] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto lat = [&](int i) -> i32x2 {   // read i: block i % 2, k-step i / 2
        return *(const lds_i32x2_t*)(rowb + (i & 1) * 16 * kF8Row + (i >> 1) * 32);
      };
      // two-stage pipeline in batches of kBatch reads: the next batch is in
      // flight while the current one is widened and multiplied
      i32x2 rq[2][kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) rq[0][i] = lat(i);
#pragma unroll
      for (int bt = 0; bt < 32 / kBatch; ++bt) {
        const int cur = bt & 1;
        if (bt + 1 < 32 / kBatch) {
#pragma unroll
          for (int i = 0; i < kBatch; ++i) rq[cur ^ 1][i] = lat((bt + 1) * kBatch + i);
          lds_wait<kBatch>();
        } else {
          lds_wait<0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 a[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) a[i] = e4m3x8_to_bf16(rq[cur][i]);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int ii = bt * kBatch + i, blk = ii & 1, ks = ii >> 1;
          sg[blk][ks >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], q[ks], sg[blk][ks >> 2], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const uint8_t* a = T + (tok0 + 16 * blk + n16) * kF8Row + kF8RopeOff + kk * 64 + g * 16;
          sg[blk][4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const lds_bf16x8_t*)a, q[16 + kk], sg[blk][4], 0, 0, 0);
        }

      // ---- combine the groups, scale, mask, step max of row n16
      float s[2][4];
      float mt = kNegInf;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sg[blk][4][i];
#pragma unroll
          for (int k = 0; k < 4; ++k) v = fmaf(sc[blk][i][k], sg[blk][k][i], v);
          const int t = abs0 + 16 * blk + 4 * g + i;
          v = (t < limit) ? v * p.scale_log2 : kNegInf;
          s[blk][i] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      m_true = fmaxf(m_true, mt);
      m_ref = (m_ref == kNegInf) ? mt : m_ref;
      overflow = overflow || (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0);

      // ---- P'_k = bf16(p * scale_k) in the operand layout of the value product
      const float mref = (m_ref == kNegInf) ? 0.f : m_ref;
      float pf[2][4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[blk][i] = __builtin_amdgcn_exp2f(s[blk][i] - mref);
          l_part += (float)(__bf16)pf[blk][i];
        }
      bf16x8 pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[k][i] = (__bf16)(pf[0][i] * sc[0][i][k]);
          pk[k][4 + i] = (__bf16)(pf[1][i] * sc[1][i][k]);
        }

      // ---- O^T += C^T P'^T over 32 column blocks of 16 (transposed reads in
      // the same two-stage pipeline)
      const uint8_t* vb = T + tok0 * kF8Row + v_off;
      auto val = [&](int cb) -> i32x2 {
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(vb + cb * 16));
      };
      i32x2 rv[2][kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) rv[0][i] = val(i);
#pragma unroll
      for (int bt = 0; bt < 32 / kBatch; ++bt) {
        const int cur = bt & 1;
        if (bt + 1 < 32 / kBatch) {
#pragma unroll
          for (int i = 0; i < kBatch; ++i) rv[cur ^ 1][i] = val((bt + 1) * kBatch + i);
          lds_wait<kBatch>();
        } else {
          lds_wait<0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 a[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) a[i] = e4m3x8_to_bf16(rv[cur][i]);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int cb = bt * kBatch + i;
          o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], pk[cb >> 3], o[cb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Slot loop.  Iteration it: wait for slot it (everyone's loads, via the
  // barrier, which also frees the ring position of slot it - 1), request slot
  // it + 2 into that position (slots 0..2 came with the prologue), consume
  // slot it.  A second pass runs only if some row outgrew its reference.
  int pass = 0;
  for (;;) {
    for (int it = 0; it < nslot; ++it) {
      wait_slots_ahead(it == 0 ? pro - 1 : min(nslot, it + 2) - it - 1);
      lds_barrier();
      if (it >= 1 && it + 2 < nslot) issue(s0 + it + 2, (it + 2) % kSlots);
      process(ring + (it % kSlots) * kSlotLds, s0 + it);
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

  // ---- finalize, as in the bf16 kernel: accumulators to LDS, the two token
  // halves of a row group merged (one query token), normalised, written as
  // row-major fp32 partial rows.
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
    other = (const float*)ring + (wave + RG) * kRegion;
    const float m1 = other[32 * 64 * 4 + n16], l1 = other[32 * 64 * 4 + 16 + n16];
    const float mm = fmaxf(m_ref, m1);
    a_own = (m_ref == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
    a_other = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
    l_row = l_row * a_own + l1 * a_other;
    m_ref = mm;
  }
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

hipError_t launch_decode_fp8(const DecodeParams& p, int segments, int query_group, bool paged,
                             hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(decode_grid(segments, p.groups)), block(256);
  if (query_group == 1) {
    if (paged) hipExtLaunchKernelGGL((splitkv_decode_fp8<1, true>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
    else hipExtLaunchKernelGGL((splitkv_decode_fp8<1, false>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
  } else {
    if (paged) hipExtLaunchKernelGGL((splitkv_decode_fp8<2, true>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
    else hipExtLaunchKernelGGL((splitkv_decode_fp8<2, false>), grid, block, 0, stream, ev_start, ev_stop, 0, p);
  }
  return hipGetLastError();
}

}  // namespace mla
