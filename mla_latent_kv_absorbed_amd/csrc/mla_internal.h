// Internal definitions shared by the library's translation units.
//
// Shape (Xing4.0-29B-A4B attention; "256K 长上下文真能本地用", §一 config.json
// and "mHC+MLA+MTP 是什么", MLA section): 32 heads, latent 512, rope 64,
// nope 128, v 128.  A cache row is [latent 512 | rope key 64] bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kHeads = 32;
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kNope = 128;
constexpr int kVDim = 128;
constexpr int kRow = kLatent + kRope;           // 576 cached values per token
constexpr int kRowBytes = kRow * 2;             // 1152
constexpr int kPage = 64;                       // tokens per page = tokens per tile
constexpr int kTileBytes = kPage * kRowBytes;   // 73728
constexpr int kChunksPerRow = kRowBytes / 16;   // 72 sixteen-byte chunks
constexpr int kWRowsPerHead = kNope + kVDim;    // 256 kv_b_proj rows per head
constexpr int kMaxQueryGroup = 2;               // query tokens one decode pass handles

// 8-bit latent cache rows: [512 E4M3 codes | 4 fp32 scales (one per 128
// latent values) | 64 bf16 rope key] = 656 bytes.
constexpr int kF8Row = 656;
constexpr int kF8ScaleOff = 512;
constexpr int kF8RopeOff = 528;
constexpr int kF8Group = 128;
constexpr int kF8Tile = kPage * kF8Row;         // 41984 bytes per page
constexpr float kE4M3Max = 448.0f;

// The absorbed query row of one (query token, head) as the 8-bit cache kernel
// takes it (kQRecBytes per head row): the bf16 latent part q split exactly
// into two E4M3 pieces with a power-of-two scale per 32 columns,
//     q[c] = (hi[c] + lo[c] / 16) * 2^(s_b - 127),   b = c / 32,
// then the rope part in bf16 and the 16 scale bytes s_b (E8M0), stored at
// kQRecScaleOff + 4 (b % 4) + b / 4.  The bf16 kernel takes the same region
// as bf16 rows of kRow values.
constexpr int kQRecHi = 0;
constexpr int kQRecLo = kLatent;                       // 512
constexpr int kQRecRope = 2 * kLatent;                 // 1024: bf16 [64]
constexpr int kQRecScaleOff = kQRecRope + 2 * kRope;   // 1152
constexpr int kQRecBytes = 1280;                       // 80 sixteen-byte chunks
static_assert(kQRecScaleOff + 16 <= kQRecBytes && kQRecBytes >= kRowBytes, "query record");

// Fault bits of the per-device fault word (values as MLA_FAULT_* in mla.h).
// A kernel that meets an index outside its documented range skips or clamps
// that item, so that every access stays inside the caller's buffers, and ORs
// the bit into the word.
constexpr uint32_t kFaultSlot = 1u;        // append: slot >= num_slots (row skipped)
constexpr uint32_t kFaultPage = 2u;        // block-table page outside [0, num_pages)
constexpr uint32_t kFaultCtxLen = 4u;      // ctx_lens[b] outside [Sq, max_ctx_len] (clamped)
constexpr uint32_t kFaultFp16Range = 8u;   // prefill: a value beyond the fp16 range

// The range rules, shared by the kernels and the host-side validator.
// A context length is clamped into [Sq, max_ctx_len]; a page must lie in
// [0, num_pages); a slot below 0 means "skip" (no fault), one at or above
// num_slots is a fault.
__host__ __device__ inline int clamp_ctx_len(int L, int Sq, int max_ctx_len, bool* bad) {
  const bool lo = L < Sq, hi = L > max_ctx_len;
  *bad = lo || hi;
  return lo ? Sq : (hi ? max_ctx_len : L);
}
__host__ __device__ inline bool page_ok(int64_t page, int64_t num_pages) { return page >= 0 && page < num_pages; }
__host__ __device__ inline bool slot_fault(int64_t slot, int64_t num_slots) { return slot >= num_slots; }

__device__ __forceinline__ void raise_fault(uint32_t* faults, uint32_t bit) {
  if (faults != nullptr) __hip_atomic_fetch_or(faults, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Split schedule.  A sequence's tiles (64 tokens each) are dealt out to
// splits of about `c` tiles; every split is one segment, processed by one
// workgroup of the split-KV kernel.  Segments are numbered sequence by
// sequence; seg_start[b] is the first segment of sequence b and
// seg_start[B] the count.  With a fixed kv_chunk, c = kv_chunk / 64 and each
// split is a contiguous run of c tiles (a chunk, or an equal part of one);
// with kv_chunk = 0 the preparation kernel chooses c on the device from the
// actual context lengths so that all sequences together give about one
// segment per compute unit (never below kMinTilesPerSplit tiles), and when a
// sequence gets n = ceil(tiles / c) >= kDealMinSplits splits, they take its
// tiles in turn: split k holds tiles k, k + n, k + 2n, ...  Dealt out this
// way, the workgroups of a long sequence read neighbouring tiles at any
// moment instead of regions a split apart, which streams a contiguous cache
// faster (the LSE combine does not depend on which tokens a split holds).
// With a few splits per sequence the contiguous runs measured slightly
// faster.
constexpr int kMinTilesPerSplit = 2;
constexpr int kDealMinSplits = 16;

// One segment: tiles first + i * stride (i < ntiles) of sequence b, whose
// clamped length is L (tokens at or past L are masked; the tile that holds
// token L - 1 is the only partial one).
struct alignas(16) SegDesc {
  int32_t b;        // sequence; -1: no segment (its workgroup returns, the combine never reads it)
  int32_t first;    // first tile of the segment
  int32_t stride;   // tile step: 1 for a contiguous run
  int32_t ntiles;   // tiles of the segment, at least 1
  int32_t L;        // clamped length of sequence b
  int32_t pad[3];
};

// Workspace layout of one decode call (byte offsets, each 256-aligned).
// rows = B * Sq query tokens; a "head row" is one (query token, head).
struct WorkspaceLayout {
  size_t qabs;      // [rows][32] query rows of kQRecBytes: bf16 [W_UK^T q_nope | rotated q_pe]
                    // at a kRow stride (bf16 cache), or the 8-bit kernel's records
  size_t qres;      // fp32 [rows][32][512]: W_UK^T q_nope - bf16(W_UK^T q_nope)
  size_t part_o;    // bf16 [max_segs][Sq*32][512]: normalised segment partials
  size_t part_lse;  // fp32 [max_segs][Sq*32], log2 domain
  size_t seg_desc;  // SegDesc [max_segs]
  size_t seg_start; // int32 [B + 1]
  size_t up_part;   // fp32 [rows*32][8][128]: W_UV shares of the 8 latent blocks
  size_t corr_part; // fp32 [rows*32][8]
  size_t stat;      // fp32 [rows*32][2]
  size_t zero_row;  // 1152 zero bytes: stand-in source for cache rows past a split's end
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(int B, int Sq, int max_segs) {
  WorkspaceLayout w;
  const size_t seq_rows = size_t(Sq) * kHeads;
  const size_t hrows = size_t(B) * seq_rows;
  size_t off = 0;
  w.qabs = off;      off = align256(off + hrows * kQRecBytes);
  w.qres = off;      off = align256(off + hrows * kLatent * 4);
  w.part_o = off;    off = align256(off + size_t(max_segs) * seq_rows * kLatent * 2);
  w.part_lse = off;  off = align256(off + size_t(max_segs) * seq_rows * 4);
  w.seg_desc = off;  off = align256(off + size_t(max_segs) * sizeof(SegDesc));
  w.seg_start = off; off = align256(off + (size_t(B) + 1) * 4);
  w.up_part = off;   off = align256(off + hrows * 8 * kVDim * 4);
  w.corr_part = off; off = align256(off + hrows * 8 * 4);
  w.stat = off;      off = align256(off + hrows * 2 * 4);
  w.zero_row = off;  off = align256(off + kRowBytes);
  w.total = off;
  return w;
}

// YaRN inverse frequencies of the 32 rotation pairs, passed by value.
struct InvFreq {
  double v[32];
};

struct DecodeParams {
  const uint16_t* qabs;         // bf16 [B][Sq][32][576]
  const uint8_t* cache;         // bf16 rows of 576
  int64_t stride_tokens;        // contiguous layout: tokens per sequence block
  const int32_t* block_table;   // paged layout: [B][max_pages]
  int32_t max_pages;
  const SegDesc* seg_desc;      // [segments]
  int32_t segments;             // segment records (grid capacity)
  int32_t groups;               // query groups per segment (see work_item)
  int32_t Sq;                   // query tokens per sequence
  float scale_log2;             // softmax_scale * log2(e)
  uint16_t* part_o;             // bf16 normalised partial rows
  float* part_lse;
  const uint8_t* zero_row;      // kRowBytes zero bytes
  int64_t num_pages;            // paged layout: pages of the pool (block-table entries are checked)
  uint32_t* faults;             // the device's fault word
};

// Query tokens per split-KV workgroup, and the number of such query groups
// that cover Sq tokens.  A group of two keeps 64 query rows (4 row groups of
// 16); a single query token uses 32 rows.  For odd Sq > 1 the last group
// holds one token: the bf16 kernel's workgroups of that group run as
// one-token workgroups, the 8-bit kernel's compute a repeat of token Sq - 1
// in the second half (never written).
inline int query_group(int Sq, bool) { return Sq == 1 ? 1 : kMaxQueryGroup; }
inline int query_groups(int Sq, bool fp8) { return (Sq + query_group(Sq, fp8) - 1) / query_group(Sq, fp8); }

// Workgroups of one split-KV launch: every (segment, query group) pair.
// The device hands consecutive workgroups to its 8 XCDs in turn (workgroup
// x runs on XCD x % 8), and each XCD has its own L2.  With several query
// groups, the groups of a segment therefore get numbers x, x + 8, x + 16, ...:
// the same XCD, dispatched one after the other, so they stream the same
// cache rows at about the same time and only the first read of a row goes
// to HBM.  The mapping is a locality choice only; any placement is correct.
constexpr int kXcds = 8;
inline unsigned decode_grid(int segments, int groups) {
  return groups == 1 ? (unsigned)segments : (unsigned)(((segments + kXcds - 1) / kXcds) * kXcds * groups);
}
__device__ __forceinline__ void work_item(int groups, int& unit, int& grp) {
  const int x = blockIdx.x;
  if (groups == 1) {
    unit = x;
    grp = 0;
    return;
  }
  const int k = x / kXcds;
  unit = (k / groups) * kXcds + x % kXcds;
  grp = k % groups;
}

// Encoding of an fp32 value |y| <= 448 as an OCP FP8 E4M3 code, nearest,
// ties to the even code (sign bit from y).  Below 2^-6 the codes step by
// 2^-9 (subnormals); above, the fp32 significand is rounded to 3 bits.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);     // exact scaling; rint: nearest, ties to even
  } else {
    uint32_t ua = __float_as_uint(a);
    ua += 0x7FFFFu + ((ua >> 20) & 1u);              // round the significand to 3 bits
    code = ((((ua >> 23) - 120u) << 3) | ((ua >> 20) & 7u));
    code = code > 0x7Eu ? 0x7Eu : code;              // 448 is the largest finite code
  }
  return code | sign;
}

// The value of an OCP FP8 E4M3 code (finite codes).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t e = (code >> 3) & 15u, m = code & 7u;
  const float a = e == 0 ? (float)m * 0.001953125f                        // m * 2^-9
                         : __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e - 7)
  return (code & 0x80u) ? -a : a;
}

// Everything that precedes the split-KV pass: the absorbed query rows, the
// rope part of the query (copied, or rotated at p = L_b - Sq + j), the cache
// rows of the new tokens (optional), the split schedule and the decode
// kernel's zero row.
struct PrepParams {
  const uint16_t* q_nope;       // bf16 [rows][32][128]
  const uint16_t* q_pe;         // bf16 [rows][32][64]
  const uint16_t* w_kv_b;       // bf16 [8192][512]
  uint16_t* qabs;
  float* qres;
  uint8_t* zero_row;
  int32_t rows;                 // B * Sq
  int32_t B;
  int32_t Sq;
  const int32_t* ctx_lens;      // read clamped into [Sq, max_ctx_len]
  int32_t max_ctx_len;
  int64_t num_pages;
  uint32_t* faults;
  int32_t rows_per_wg;          // query rows per workgroup (prep_rows_per_wg)
  int32_t rotate;               // q_pe and k_new are rotated here when non-zero
  InvFreq inv;
  const uint16_t* c_new;        // bf16 [rows][ld_c] latent rows of the new tokens, or null
  int64_t ld_c;
  const uint16_t* k_new;        // bf16 [rows][ld_k] rope rows of the new tokens
  int64_t ld_k;
  uint8_t* cache;
  int64_t stride_tokens;
  const int32_t* block_table;
  int32_t max_pages;
  int32_t paged;
  int32_t fp8;                  // cache rows are 8-bit (kF8Row bytes)
  // split schedule
  int32_t fixed_tiles;          // tiles per split, or 0: balance on the device
  int32_t target_segs;          // balanced: aim at no more segments than this
  int32_t max_segs;             // capacity of seg_desc / part_o
  SegDesc* seg_desc;
  int32_t* seg_start;
};

struct CombineParams {
  const uint16_t* part_o;
  const float* part_lse;
  const int32_t* seg_start;
  int32_t max_segs;
  int32_t Sq;
  int32_t hrows;                // rows * 32
  int32_t rows_per_wg;          // query rows per workgroup (combine_rows_per_wg)
  const uint16_t* w_kv_b;
  const float* qres;
  float scale_log2;
  uint16_t* out;                // bf16 [rows][32][128]
  float* lse;                   // fp32 [rows][32] or null
  float* up_part;               // fp32 [rows*32][8][128]: W_UV shares of the 8 latent blocks
  float* corr_part;             // fp32 [rows*32][8]: qres . o_lat shares
  float* stat;                  // fp32 [rows*32][2]: combined (M, W), log2 domain
};

// Query rows per workgroup of the preparation kernel: one 16-row tile of
// its matrix-core absorption.  Query rows per workgroup of the combine: 16
// from 16 rows on (one matrix-core tile of the up-projection, W_UV read once
// per 16 rows; 4 rows per workgroup measured 1.3% slower per paged 16x64K
// layer), else one (combine_one_row, which spreads a few rows over more
// compute units).
inline int prep_rows_per_wg(int) { return 16; }
inline int combine_rows_per_wg(int rows) { return rows >= 16 ? 16 : 1; }

// Launchers (each enqueues on `stream`; return hipError_t of the launch).
// ev_start / ev_stop (may be null): recorded by the dispatches themselves at
// the start of the first and the end of the last split-KV launch.
hipError_t launch_decode(const DecodeParams& p, int segments, int query_group, bool paged, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop);
hipError_t launch_prep(const PrepParams& p, hipStream_t stream);
hipError_t launch_combine_upproject(const CombineParams& p, hipStream_t stream);
hipError_t launch_rope(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst,
                       const int32_t* positions, int64_t n, const double* inv_freq, int rope_dim,
                       hipStream_t stream);
hipError_t launch_append(uint8_t* cache, int64_t num_slots, const uint16_t* c_kv, int64_t ld_c,
                         const uint16_t* k_pe, int64_t ld_k, const int64_t* slots, int64_t n,
                         uint32_t* faults, hipStream_t stream);
hipError_t launch_append_fp8(uint8_t* cache, int64_t num_slots, const uint16_t* c_kv, int64_t ld_c,
                             const uint16_t* k_pe, int64_t ld_k, const int64_t* slots, int64_t n,
                             uint32_t* faults, hipStream_t stream);
// Chunked prefill (prefill.hip): expand the L context rows through kv_b_proj
// into kv (rows [8192 expanded values, fp16 | 64 rope key, bf16], L rounded
// up to 256 rows, prefill_workspace_bytes), then causal attention of the Tq
// chunk tokens.
hipError_t launch_prefill(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_kv_b, const uint8_t* cache,
                          int32_t L, int32_t Tq, float scale_log2, uint16_t* kv, uint16_t* out, float* lse,
                          uint32_t* faults, hipStream_t stream);
size_t prefill_workspace_bytes(int32_t L);
hipError_t launch_decode_fp8(const DecodeParams& p, int segments, int qg, bool paged, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop);

}  // namespace mla
