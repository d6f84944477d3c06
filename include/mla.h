/*
 * mla.h - C ABI of the MI355X (gfx950) MLA latent-KV decode library.
 *
 * Multi-head Latent Attention decode over a compressed KV cache in the
 * Xing4.0-29B-A4B attention shape: 32 heads, kv_lora_rank 512, qk_nope 128,
 * qk_rope 64, v_head 128, YaRN rope (factor 64, 4096 -> 262144).
 *
 * Pages cited:
 *  [KV-ledger] "256K 长上下文真能本地用？Xing4.0 原生长上下文的工程代价拆解",
 *              §一 (config.json: kv_lora_rank, v_head_dim, rope_scaling,
 *              attention_bias) and §二 (what the cache holds per token).
 *  [MLA-arch]  "mHC+MLA+MTP 是什么？拆开给 Agent 用的百亿 MoE", section
 *              "MLA：256K 上下文的内存革命" (kv_a_proj_with_mqa writes a 512-wide
 *              latent plus a 64-wide rope component per token into the cache;
 *              kv_b_proj expands per-head keys and values from the latent at
 *              attention time; YaRN rope with yarn_get_mscale).
 *
 * General conventions
 *  - Every pointer argument is a DEVICE pointer unless marked "host".
 *  - bf16 is bfloat16 (1-8-7), passed as raw 16-bit values.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no
 *    pointer after a call returns and holds no state between calls, except
 *    two static device arrays per device (the fault word below and the
 *    scratch of mla_decode_step_paged_noalloc) and the opt-in kernel timing
 *    at the end of this header.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream).  MLA_OK means "enqueued"; device faults show up at the
 *    caller's next synchronisation.  No call synchronises the host.
 *  - Arguments are validated on the host before anything is enqueued; a bad
 *    argument returns an error code and enqueues nothing.  Contents of device
 *    arrays (block tables, context lengths, slot mappings) are not read by
 *    the host; the kernels check them instead: a slot at or beyond num_slots
 *    is skipped, a block-table page outside [0, num_pages) is read as zero
 *    rows (and not written by the fused step), a context length outside
 *    [Sq, max_ctx_len] is clamped into it, so every access stays inside the
 *    caller's buffers.  Each such event sets a bit of the device's sticky
 *    fault word (MLA_FAULT_*), which mla_device_faults() reads after the work
 *    has finished; mla_check_decode_inputs() and mla_check_slot_mapping()
 *    apply the same rules to host copies of those arrays (a debug check
 *    before enqueueing).
 *  - The library is reentrant; concurrent calls on different streams must
 *    use different workspaces.
 */
#ifndef MLA_LATENT_KV_ABSORBED_MLA_H
#define MLA_LATENT_KV_ABSORBED_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mla_status;
#define MLA_OK               0
#define MLA_ERR_NULL         1   /* a required pointer is NULL                       */
#define MLA_ERR_SHAPE        2   /* shape constants or sizes are not supported       */
#define MLA_ERR_RANGE        3   /* a size is out of range (e.g. Sq > max_ctx_len)   */
#define MLA_ERR_ALIGN        4   /* a pointer or leading dimension is misaligned     */
#define MLA_ERR_WORKSPACE    5   /* workspace too small                              */
#define MLA_ERR_DEVICE       6   /* a HIP runtime call failed                        */
#define MLA_ERR_UNSUPPORTED  7   /* a valid request this library does not implement  */
#define MLA_ERR_SCRATCH      8   /* the no-allocation entry point needs more than its
                                    static scratch (MLA_STATIC_SCRATCH_BYTES)          */

/* Bits of the per-device fault word (mla_device_faults). */
#define MLA_FAULT_SLOT        1u /* a slot >= num_slots: the row was not written          */
#define MLA_FAULT_PAGE        2u /* a block-table page outside [0, num_pages): its rows
                                    were read as zeros and not written                   */
#define MLA_FAULT_CTX_LEN     4u /* a context length outside [Sq, max_ctx_len]: clamped  */
#define MLA_FAULT_FP16_RANGE  8u /* mla_prefill: a query or an expanded key/value beyond
                                    the fp16 range (|x| > 65504); results not reliable  */

/* Cache row formats (mla_shape.kv_cache_dtype).
 *  MLA_CACHE_BF16      576 bf16 = 1152 bytes: [latent (512) | rope key (64)]
 *  MLA_CACHE_FP8_E4M3  656 bytes: [512 OCP FP8 E4M3 codes | 4 fp32 scales |
 *                      64 bf16 rope key]; latent value = code * scale of its
 *                      group of 128 (scale = group max |x| / 448, fp32; codes
 *                      round to nearest, ties to even; a group of zeros has
 *                      scale 0).  The 8-bit cache of [KV-ledger §三] (plan A),
 *                      which halves the cache bytes of bf16.
 * A page holds 64 rows of the chosen format. */
#define MLA_CACHE_BF16      0
#define MLA_CACHE_FP8_E4M3  1

/* Attention shape.  The library implements exactly num_heads 32,
 * kv_lora_rank 512, qk_nope_head_dim 128, qk_rope_head_dim 64, v_head_dim 128
 * and page_size 64 ([KV-ledger §一]; [MLA-arch]); anything else returns
 * MLA_ERR_SHAPE.  softmax_scale multiplies q.k; for this model it is
 * (qk_nope + qk_rope)^-1/2 * mscale^2 with mscale = 0.1 ln(64) + 1
 * (YaRN's attention-logit correction named by [MLA-arch]); see
 * mla_default_shape().  kv_cache_dtype selects the cache row format of every
 * call that takes a cache (MLA_CACHE_BF16 or MLA_CACHE_FP8_E4M3). */
typedef struct {
    int32_t num_heads;
    int32_t kv_lora_rank;
    int32_t qk_nope_head_dim;
    int32_t qk_rope_head_dim;
    int32_t v_head_dim;
    int32_t page_size;
    float   softmax_scale;
    int32_t kv_cache_dtype;
} mla_shape;

/* YaRN rope parameters ([KV-ledger §一] rope_scaling; base not printed for
 * this model, 10000 is the customary value).  Rotation pairs element i with
 * element i + rope_dim/2 of each rope vector. */
typedef struct {
    double  base;                 /* rope theta                        */
    double  factor;               /* 64                                */
    double  original_max_position;/* 4096                              */
    double  beta_fast;            /* 32                                */
    double  beta_slow;            /* 1                                 */
    int32_t rope_dim;             /* 64                                */
} mla_rope_params;

/* Fills *shape with the model's shape, its softmax scale and the bf16 cache
 * format (host). */
mla_status mla_default_shape(mla_shape* shape /* host */);

/* Fills *params with the model's YaRN parameters, base 10000 (host). */
mla_status mla_default_rope(mla_rope_params* params /* host */);

/* Human-readable name of a status code (static string). */
const char* mla_status_string(mla_status status);

/* Apply YaRN rotary position embedding: dst row r = rot(src row r, positions[r]).
 * [MLA-arch]: the rope component uses YaRN scaling (factor 64 from 4096
 * positions); [KV-ledger §一] prints the rope_scaling fields.
 *   src, ld_src  bf16 rows; row r's rope vector is src[r*ld_src .. + rope_dim)
 *   dst, ld_dst  bf16 rows receiving the rotated vectors (dst == src with
 *                ld_dst == ld_src rotates in place; other elements of a dst
 *                row are not touched)
 *   positions    int32 [n] position of each row (0 <= pos < 2^24)
 *   n            rows (0 is a no-op)
 * Element i pairs with element i + rope_dim/2.  Angles pos * inv_freq and
 * their cos/sin are formed in fp64; each rotated value is rounded once from
 * fp64 to bf16 (nearest, ties to even).  src and dst must be 16-byte
 * aligned with leading dimensions >= rope_dim and multiples of 8; src and dst
 * rows must not partially overlap. */
mla_status mla_rope_yarn(const mla_rope_params* params /* host */, const void* src, int64_t ld_src,
                         void* dst, int64_t ld_dst, const int32_t* positions, int64_t n, void* stream);

/* Write cache rows: cache[slot] = [c_kv row (512) | k_pe row (64)], a bit
 * copy for the bf16 format; for the fp8 format the latent row is quantised
 * (see the cache row formats above) and the rope key copied.
 * [MLA-arch]: only the compressed latent and the rope component are cached
 * per token, no per-head K or V.
 *   cache         [num_slots] rows of the shape's format; for the paged layout slot =
 *                 page * page_size + offset, for the contiguous layout slot =
 *                 b * stride + t
 *   c_kv, ld_c    bf16 latent rows [n][ld_c] (ld_c >= 512)
 *   k_pe, ld_k    bf16 rope rows [n][ld_k] (ld_k >= 64), already rotated
 *   num_slots     rows the cache holds; a slot >= num_slots is skipped and
 *                 sets MLA_FAULT_SLOT
 *   slot_mapping  int64 [n]; a negative slot skips the row
 * Requires 16-byte aligned cache, c_kv and k_pe and ld_c, ld_k multiples
 * of 8 (MLA_ERR_ALIGN otherwise). */
mla_status mla_cache_append(const mla_shape* shape /* host */, void* cache, int64_t num_slots,
                            const void* c_kv, int64_t ld_c, const void* k_pe, int64_t ld_k,
                            const int64_t* slot_mapping, int64_t n, void* stream);

/* Decode attention against a contiguous cache.
 * For query token j of sequence b (position p = L_b - Sq + j, whose own row
 * is already in the cache) and head h:
 *   q_lat = W_UK[h]^T q_nope            (W_UK folded into the query)
 *   s_t   = softmax_scale * (q_lat . c_t + q_pe . k_pe_t),  t = 0..p
 *   o     = W_UV[h] * sum_t softmax(s)_t c_t
 * which equals attention with keys [W_UK c_t ; k_pe_t] and values W_UV c_t
 * expanded by kv_b_proj ([MLA-arch]).  W_UK[h] and W_UV[h] are rows
 * [h*256, h*256+128) and [h*256+128, h*256+256) of w_kv_b.
 *   q_nope       bf16 [B][Sq][32][128]
 *   q_pe         bf16 [B][Sq][32][64], already rotated
 *   w_kv_b       bf16 [8192][512] (nn.Linear storage: out x in)
 *   cache        [B][stride_tokens] rows of the shape's format
 *   ctx_lens     int32 [B], Sq <= L_b <= max_ctx_len (a value outside is
 *                clamped into that range and sets MLA_FAULT_CTX_LEN)
 *   max_ctx_len  host upper bound of ctx_lens, <= stride_tokens
 *   kv_chunk     tokens per split, a multiple of 64, or 0 to let the
 *                library choose (splits sized from the actual ctx_lens on the
 *                device, about one workgroup per compute unit; a sequence
 *                with 16 or more such splits deals its 64-token tiles out to
 *                them in turn, so a split is then not a contiguous range; the
 *                result differs only by rounding).  When the
 *                chunks of a call are fewer than the device's compute units
 *                (per query group), each chunk is cut into 2^k equal
 *                sub-splits of at least 128 tokens, within that count; the
 *                LSE combine over the sub-splits equals combining each
 *                chunk's sub-splits and then the chunks.
 *   out          bf16 [B][Sq][32][128]
 *   lse          fp32 [B][Sq][32] natural-log sum of exp(s_t), or NULL
 *   workspace    device scratch of mla_decode_workspace_size() bytes,
 *                256-byte aligned
 * Supports 1 <= Sq <= 16 and B * Sq <= 65535.  B = 0 is a no-op.  All Sq
 * query tokens are served by one pass over the cache: the workgroups of the
 * query groups (two tokens each) of one split read the same rows together.
 * MLA_ERR_RANGE also when the splits times the ceil(Sq/2) query groups exceed
 * 2^24 workgroups. */
mla_status mla_decode(const mla_shape* shape /* host */, const void* q_nope, const void* q_pe,
                      const void* w_kv_b, const void* cache, int64_t stride_tokens,
                      const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                      int32_t kv_chunk, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Decode attention against a paged cache: as mla_decode, but token t of
 * sequence b lives in slot block_table[b][t / 64] * 64 + t % 64 of
 *   cache        [num_pages][64] rows of the shape's format
 *   block_table  int32 [B][max_pages_per_seq], max_pages_per_seq >=
 *                ceil(max_ctx_len / 64)
 * Every page a sequence uses must be in [0, num_pages); a page outside is
 * read as 64 zero rows and sets MLA_FAULT_PAGE. */
mla_status mla_decode_paged(const mla_shape* shape /* host */, const void* q_nope, const void* q_pe,
                            const void* w_kv_b, const void* cache, int64_t num_pages,
                            const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                            int32_t kv_chunk, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* One decode step of a layer for Sq new tokens per sequence, fused: the
 * whole path of [MLA-arch] from the new tokens' projections to the attention
 * output.  For token j of sequence b, at position p = L_b - Sq + j
 * (ctx_lens already count the new tokens):
 *   1. k_pe_new row (b*Sq + j) is rotated by YaRN RoPE at p and, with
 *      c_kv_new row (b*Sq + j), written into the cache slot of token p (the
 *      cache write of mla_cache_append; [MLA-arch], [KV-ledger §二]);
 *   2. q_pe[b][j] is rotated at p (as mla_rope_yarn);
 *   3. the decode of mla_decode / mla_decode_paged runs on the result.
 * The results are bitwise those of mla_rope_yarn + mla_cache_append +
 * mla_decode with the same arguments; the rotated q_pe is not written back.
 *   rope          host YaRN parameters (as mla_rope_yarn)
 *   q_pe          bf16 [B][Sq][32][64], NOT rotated
 *   c_kv_new      bf16 [B*Sq][ld_c] latent rows of the new tokens (ld_c >= 512)
 *   k_pe_new      bf16 [B*Sq][ld_k] rope rows, NOT rotated (ld_k >= 64)
 *   cache         written at the new tokens' slots, read by the decode
 * Every other argument as in mla_decode.  c_kv_new and k_pe_new must be
 * 16-byte aligned with ld_c, ld_k multiples of 8.  In the paged form a new
 * token whose page lies outside [0, num_pages) is not written
 * (MLA_FAULT_PAGE). */
mla_status mla_decode_step(const mla_shape* shape /* host */, const mla_rope_params* rope /* host */,
                           const void* q_nope, const void* q_pe, const void* c_kv_new, int64_t ld_c,
                           const void* k_pe_new, int64_t ld_k, const void* w_kv_b, void* cache,
                           int64_t stride_tokens, const int32_t* ctx_lens, int32_t max_ctx_len,
                           int32_t B, int32_t Sq, int32_t kv_chunk, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* mla_decode_step against a paged cache (arguments as mla_decode_paged). */
mla_status mla_decode_step_paged(const mla_shape* shape /* host */, const mla_rope_params* rope /* host */,
                                 const void* q_nope, const void* q_pe, const void* c_kv_new, int64_t ld_c,
                                 const void* k_pe_new, int64_t ld_k, const void* w_kv_b, void* cache,
                                 int64_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                                 int32_t kv_chunk, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Workspace bytes mla_decode, mla_decode_paged and the mla_decode_step calls
 * need for these sizes (host).
 * kv_chunk as in mla_decode (0 = the library's choice). */
mla_status mla_decode_workspace_size(const mla_shape* shape /* host */, int32_t B, int32_t Sq,
                                     int32_t max_ctx_len, int32_t kv_chunk,
                                     size_t* bytes /* host */);

/* The kv_chunk the library would use for kv_chunk = 0 when all B sequences
 * hold max_ctx_len tokens, for the bf16 cache format (host).  (The 8-bit
 * format serves each query token with its own workgroups, so for Sq > 1 it
 * aims at fewer, longer splits.) */
mla_status mla_decode_auto_chunk(int32_t B, int32_t Sq, int32_t max_ctx_len, int32_t* kv_chunk /* host */);

/* Workspace bytes mla_prefill needs for a context of ctx_len tokens (host):
 * the expanded rows, 16,512 B per token (ctx_len rounded up to 256).
 * MLA_ERR_UNSUPPORTED for the 8-bit cache format. */
mla_status mla_prefill_workspace_size(const mla_shape* shape /* host */, int32_t ctx_len,
                                      size_t* bytes /* host */);

/* Chunked prefill of one sequence, in the un-absorbed form.  The chunk's Tq
 * query tokens sit at positions p = L - Tq + j (L = ctx_len; their cache rows
 * are already written, e.g. by mla_rope_yarn + mla_cache_append) and each sees
 * tokens 0..p.  kv_b_proj expands every cached latent into per-head keys and
 * values ([MLA-arch]: "实时展开"):
 *   K_nope[t][h] = W_UK[h] c_t,  V[t][h] = W_UV[h] c_t   (fp16, fp32 sums)
 *   s_jt = softmax_scale * (q_nope[j][h] . K_nope[t][h] + q_pe[j][h] . k_pe_t)
 *   out[j][h] = sum_t softmax(s)_t V[t][h],  lse[j][h] = ln sum_t exp(s_jt)
 * which for many query tokens costs fewer flops than the absorbed form of
 * mla_decode (2*32*(192+128) per query and visible token, plus 2*512*8192 per
 * cached token for the expansion, against 2*32*(576+512)).
 *   q_nope       bf16 [Tq][32][128]
 *   q_pe         bf16 [Tq][32][64], already rotated
 *   w_kv_b       bf16 [8192][512]
 *   cache        bf16 rows [ctx_len][576] of the sequence (contiguous; a paged
 *                sequence is gathered first)
 *   out          bf16 [Tq][32][128];  lse  fp32 [Tq][32] or NULL
 *   workspace    device scratch of mla_prefill_workspace_size() bytes,
 *                16-byte aligned
 * Supports 1 <= Tq <= ctx_len <= 2^20 and the bf16 cache format only
 * (MLA_ERR_UNSUPPORTED for the 8-bit format).  The expanded keys and values
 * and q_nope are held in fp16 on the matrix cores: magnitudes up to 65504;
 * a larger one sets MLA_FAULT_FP16_RANGE. */
mla_status mla_prefill(const mla_shape* shape /* host */, const void* q_nope, const void* q_pe,
                       const void* w_kv_b, const void* cache, int32_t ctx_len, int32_t Tq, void* out,
                       float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* mla_decode_step_paged for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that forbid allocation): the same
 * arguments without the workspace, which is taken from a static device
 * array of MLA_STATIC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends.  The call allocates nothing.  A request
 * whose workspace (mla_decode_workspace_size) exceeds that size returns
 * MLA_ERR_SCRATCH and enqueues nothing.  All calls on one device share its
 * array: calls that may overlap on one device (different streams, or other
 * host threads) race and must be serialised by the caller.  The first call on
 * a device (or any other call of this library there) looks up the array's
 * device address, so it must not be the first library call inside a capture. */
#define MLA_STATIC_SCRATCH_BYTES (64u << 20)
mla_status mla_decode_step_paged_noalloc(const mla_shape* shape /* host */, const mla_rope_params* rope /* host */,
                                         const void* q_nope, const void* q_pe, const void* c_kv_new, int64_t ld_c,
                                         const void* k_pe_new, int64_t ld_k, const void* w_kv_b, void* cache,
                                         int64_t num_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                                         const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                                         int32_t kv_chunk, void* out, float* lse, void* stream);

/* Reads the fault word of the current device (MLA_FAULT_* bits set by any
 * kernel of this library since the word was last cleared) into *faults
 * (host), after waiting for all work on the device; clear != 0 then resets
 * it to zero.  A debugging aid: it synchronises the device, so it must not
 * be called during graph capture. */
mla_status mla_device_faults(uint32_t* faults /* host */, int32_t clear);

/* Host-side debug check of decode inputs (host copies of the device
 * arrays): *faults (host) receives the MLA_FAULT_* bits the kernels would
 * set: MLA_FAULT_CTX_LEN for a length outside [Sq, max_ctx_len],
 * MLA_FAULT_PAGE for a page outside [0, num_pages) among the first
 * ceil(L_b / 64) entries of a row (L_b after clamping).  block_table may be
 * NULL (contiguous layout). */
mla_status mla_check_decode_inputs(int32_t B, int32_t Sq, int32_t max_ctx_len, const int32_t* ctx_lens /* host */,
                                   const int32_t* block_table /* host */, int32_t max_pages_per_seq,
                                   int64_t num_pages, uint32_t* faults /* host */);

/* Host-side debug check of an append's slot mapping (host copy):
 * MLA_FAULT_SLOT if any slot is >= num_slots (negative slots are skips). */
mla_status mla_check_slot_mapping(const int64_t* slot_mapping /* host */, int64_t n, int64_t num_slots,
                                  uint32_t* faults /* host */);

/* Kernel timing, a profiling aid (not needed to compute anything).
 * After mla_timing_enable(n), each of the next n decode calls has its
 * split-KV attention kernel(s) record a HIP event pair themselves, at the
 * start of the first and the end of the last launch; calls beyond n are not
 * timed.  mla_timing_collect() waits for the recorded
 * events and returns the summed kernel time in milliseconds and the number
 * of timed kernel launches; mla_timing_disable() releases the events.  This
 * is the library's only global state: enable it outside HIP graph capture,
 * from one host thread. */
mla_status mla_timing_enable(int32_t max_calls);
mla_status mla_timing_collect(double* total_ms /* host */, int32_t* launches /* host */);
mla_status mla_timing_disable(void);

/* Streaming-read ceiling, a measurement aid (not needed to compute anything):
 * one launch reads all `bytes` of device buffer `buf` once (2048 workgroups,
 * each a contiguous share, streamed with 16-byte direct global->LDS loads as
 * the decode kernels stream the cache) and stores one XOR digest per wave to
 * `sink`, device int32 [MLA_READ_PROBE_SINK_INTS]; the XOR of the digests is
 * the XOR of the buffer's 32-bit words.  Timed by the caller (events on `stream`),
 * it gives the HBM read rate a plain streaming kernel reaches on this device,
 * against which the decode kernels' rates can be read.  `buf` 16-byte
 * aligned, bytes a non-zero multiple of 16 (MLA_ERR_ALIGN / MLA_ERR_RANGE
 * otherwise); the caller owns both buffers. */
#define MLA_READ_PROBE_SINK_INTS 8192
mla_status mla_read_probe(const void* buf, size_t bytes, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_LATENT_KV_ABSORBED_MLA_H */
