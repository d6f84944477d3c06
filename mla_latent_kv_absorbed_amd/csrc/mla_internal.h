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

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// Workspace layout of one decode call (byte offsets, each 256-aligned).
struct WorkspaceLayout {
  size_t qabs;      // bf16 [B][Sq][32][576]: [W_UK^T q_nope | q_pe]
  size_t qres;      // fp32 [B][Sq][32][512]: W_UK^T q_nope - bf16(W_UK^T q_nope)
  size_t part_o;    // fp32 [B][splits][2*Sq][32 col blocks][64 lanes][4]
  size_t part_lse;  // fp32 [B][splits][Sq*32], log2 domain
  size_t o_lat;     // fp32 [B][Sq][32][512]
  size_t lse2;      // fp32 [B][Sq][32], combined LSE in log2 units before correction
  size_t zero_row;  // 1152 zero bytes: stand-in source for cache rows past a split's end
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(int B, int Sq, int splits) {
  WorkspaceLayout w;
  size_t off = 0;
  w.qabs = off;     off = align256(off + size_t(B) * Sq * kHeads * kRow * 2);
  w.qres = off;     off = align256(off + size_t(B) * Sq * kHeads * kLatent * 4);
  w.part_o = off;   off = align256(off + size_t(B) * splits * Sq * kHeads * kLatent * 4);
  w.part_lse = off; off = align256(off + size_t(B) * splits * Sq * kHeads * 4);
  w.o_lat = off;    off = align256(off + size_t(B) * Sq * kHeads * kLatent * 4);
  w.lse2 = off;     off = align256(off + size_t(B) * Sq * kHeads * 4);
  w.zero_row = off; off = align256(off + kRowBytes);
  w.total = off;
  return w;
}

struct DecodeParams {
  const uint16_t* qabs;         // bf16 [B][Sq][32][576]
  const uint8_t* cache;         // bf16 rows of 576
  int64_t stride_tokens;        // contiguous layout: tokens per sequence block
  const int32_t* block_table;   // paged layout: [B][max_pages]
  int32_t max_pages;
  const int32_t* ctx_lens;      // [B]
  int32_t Sq;                   // query tokens per sequence
  int32_t j0;                   // first query token of this pass
  int32_t kv_chunk;             // tokens per split (multiple of 64)
  int32_t splits;               // splits per sequence (grid.x / B)
  float scale_log2;             // softmax_scale * log2(e)
  float* part_o;
  float* part_lse;
  const uint8_t* zero_row;      // kRowBytes zero bytes
};

// Launchers (each enqueues on `stream`; return hipError_t of the launch).
hipError_t launch_decode(const DecodeParams& p, int B, int query_group, bool paged, hipStream_t stream);
hipError_t launch_absorb(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_kv_b,
                         uint16_t* qabs, float* qres, uint8_t* zero_row, int rows, hipStream_t stream);
hipError_t launch_combine(const float* part_o, const float* part_lse, const int32_t* ctx_lens,
                          int B, int Sq, int splits, int kv_chunk, float* o_lat, float* lse2,
                          hipStream_t stream);
hipError_t launch_upproj(const float* o_lat, const uint16_t* w_kv_b, const float* qres,
                         const float* lse2, float scale_log2, uint16_t* out, float* lse, int rows,
                         hipStream_t stream);
hipError_t launch_rope(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst,
                       const int32_t* positions, int64_t n, const double* inv_freq, int rope_dim,
                       hipStream_t stream);
hipError_t launch_append(uint8_t* cache, int64_t num_slots, const uint16_t* c_kv, int64_t ld_c,
                         const uint16_t* k_pe, int64_t ld_k, const int64_t* slots, int64_t n,
                         hipStream_t stream);

}  // namespace mla
