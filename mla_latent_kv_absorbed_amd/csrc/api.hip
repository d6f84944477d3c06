// C ABI of the MLA latent-KV decode library (declarations and contracts in
// include/mla.h).  Host side only: argument checks, split selection,
// workspace carving and kernel launches on the caller's stream.
#include <math.h>
#include <algorithm>
#include <mutex>
#include <string.h>

#include "mla.h"   // include/mla.h (on the include path)
#include "mla_internal.h"

using namespace mla;

// Per-device fault word: the kernels OR MLA_FAULT_* bits into it when they
// meet an index outside its range (mla_device_faults reads and clears it).
__device__ uint32_t g_fault_word = 0;

// Scratch of mla_decode_step_paged_noalloc, in place of a caller's workspace:
// each device the library runs on holds its own copy until the process ends.
constexpr size_t kStaticScratchBytes = (size_t)MLA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

// Device addresses of the two arrays above, looked up once per device (with
// that device current) by hipGetSymbolAddress: in host code the arrays' names
// are host-side stand-ins, never device addresses.
constexpr int kMaxDevices = 64;
struct DeviceSymbols {
  std::once_flag once;
  hipError_t err = hipSuccess;
  uint32_t* faults = nullptr;
  uint8_t* scratch = nullptr;
};
DeviceSymbols g_symbols[kMaxDevices];

const DeviceSymbols* device_symbols() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceSymbols& d = g_symbols[dev];
  std::call_once(d.once, [&d] {
    d.err = hipGetSymbolAddress((void**)&d.faults, HIP_SYMBOL(g_fault_word));
    if (d.err == hipSuccess) d.err = hipGetSymbolAddress((void**)&d.scratch, HIP_SYMBOL(scratch));
  });
  return d.err == hipSuccess ? &d : nullptr;
}

constexpr int kMaxSq = 16;
constexpr int64_t kMaxRows = 65535;   // B * Sq: the supported range of query rows per call

// Opt-in kernel timing (mla_timing_*): event pairs around split-KV launches.
struct Timing {
  bool on = false;
  int capacity = 0;       // event pairs
  int used = 0;
  hipEvent_t* ev = nullptr;   // 2 * capacity events
} g_timing;

void timing_free() {
  if (g_timing.ev != nullptr) {
    for (int i = 0; i < 2 * g_timing.capacity; ++i) (void)hipEventDestroy(g_timing.ev[i]);
    delete[] g_timing.ev;
  }
  g_timing = Timing();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Longest context of one prefill call (32-bit byte offsets inside a tile of
// expanded rows stay far inside range; the workspace is 16.5 KiB per token).
constexpr int32_t kMaxPrefillCtx = 1 << 20;

mla_status check_shape(const mla_shape* s) {
  if (s == nullptr) return MLA_ERR_NULL;
  if (s->num_heads != kHeads || s->kv_lora_rank != kLatent || s->qk_nope_head_dim != kNope ||
      s->qk_rope_head_dim != kRope || s->v_head_dim != kVDim || s->page_size != kPage ||
      (s->kv_cache_dtype != MLA_CACHE_BF16 && s->kv_cache_dtype != MLA_CACHE_FP8_E4M3))
    return MLA_ERR_SHAPE;
  if (!(s->softmax_scale > 0.f) || !isfinite(s->softmax_scale)) return MLA_ERR_RANGE;
  return MLA_OK;
}

// Compute units of the current device (the balanced schedule aims at one
// split-KV workgroup per unit).
int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

// Upper bound of the number of segments (splits) of a call: with a fixed
// kv_chunk every sequence has at most ceil(max_ctx_len / kv_chunk) chunks,
// and chunks are sub-split only while the segments stay within the target;
// the balanced schedule (kv_chunk = 0) chooses c >= ceil(T / target) tiles,
// so sum_b ceil(tiles_b / c) <= T / c + B <= target + B, or else c = the
// longest sequence's tiles, which makes every sequence one split (B segments).
int64_t max_segments(int B, int max_ctx, int kv_chunk, int target) {
  if (kv_chunk > 0) return std::max<int64_t>((int64_t)B * ((max_ctx + kv_chunk - 1) / kv_chunk), target);
  return (int64_t)target + B;
}

// Tokens per split the balanced schedule picks when all B sequences hold
// max_ctx tokens (the device decides from the actual lengths).
int balanced_chunk(int B, int max_ctx, int target) {
  const int64_t tiles = (max_ctx + kPage - 1) / kPage;
  const int64_t T = tiles * B;
  // never more than one sequence's tiles: from there on each sequence is one split
  const int64_t cmax = std::max<int64_t>(kMinTilesPerSplit, tiles);
  int64_t c = std::min(cmax, std::max<int64_t>(kMinTilesPerSplit, (T + target - 1) / target));
  for (int it = 0; it < 8; ++it) {
    const int64_t n = B * ((tiles + c - 1) / c);
    if (n <= target || c >= cmax) break;
    c = std::min(cmax, std::max<int64_t>(c + 1, (c * n + target - 1) / target));
  }
  return (int)(c * kPage);
}

// YaRN NTK-by-parts frequencies (Peng et al., 2023): pairs turning more than
// beta_fast times over the original context keep base^(-2i/d); pairs turning
// fewer than beta_slow times are divided by the factor; a linear ramp over
// the pair index joins the two.
void yarn_frequencies(const mla_rope_params& p, double* out) {
  const int half = p.rope_dim / 2;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < half; ++i) {
    const double f = pow(p.base, -2.0 * i / p.rope_dim);
    out[i] = f;
  }
  if (p.factor <= 1.0) return;
  auto index_of_turns = [&](double turns) {
    return p.rope_dim * log(p.original_max_position / (two_pi * turns)) / (2.0 * log(p.base));
  };
  double lo = floor(index_of_turns(p.beta_fast));
  double hi = ceil(index_of_turns(p.beta_slow));
  if (lo < 0) lo = 0;
  if (hi > p.rope_dim - 1) hi = p.rope_dim - 1;
  if (hi == lo) hi = lo + 1e-3;
  for (int i = 0; i < half; ++i) {
    double ramp = (i - lo) / (hi - lo);
    ramp = ramp < 0 ? 0 : (ramp > 1 ? 1 : ramp);
    out[i] = out[i] * (1.0 - ramp) + (out[i] / p.factor) * ramp;
  }
}

// Workspace argument meaning "use the device's static scratch" (the
// no-allocation entry point); never a valid device address.
void* const kUseStaticScratch = (void*)(uintptr_t)1;

// Optional fused front end of a decode call: rotate q_pe (and the new
// tokens' rope rows) at p = L_b - Sq + j and write the new tokens' cache rows.
struct StepInputs {
  const mla_rope_params* rope;  // null: q_pe is already rotated, nothing appended
  const void* c_new;
  int64_t ld_c;
  const void* k_new;
  int64_t ld_k;
};

mla_status check_rope(const mla_rope_params* params) {
  if (params == nullptr) return MLA_ERR_NULL;
  if (params->rope_dim != kRope || !(params->base > 1.0) || !(params->factor >= 1.0) ||
      !(params->original_max_position > 0) || !(params->beta_fast > params->beta_slow) ||
      !(params->beta_slow > 0))
    return MLA_ERR_SHAPE;
  return MLA_OK;
}

mla_status decode_common(const mla_shape* shape, const StepInputs& step, const void* q_nope,
                         const void* q_pe, const void* w_kv_b, const void* cache, int64_t stride_tokens,
                         int64_t num_pages, const int32_t* block_table, int32_t max_pages,
                         const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                         int32_t kv_chunk, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, bool paged) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (step.rope != nullptr && (st = check_rope(step.rope)) != MLA_OK) return st;
  if (B < 0 || Sq < 1 || Sq > kMaxSq || max_ctx_len < Sq) return MLA_ERR_RANGE;
  if ((int64_t)B * Sq > kMaxRows) return MLA_ERR_RANGE;
  if (B == 0) return MLA_OK;
  if (!q_nope || !q_pe || !w_kv_b || !cache || !ctx_lens || !out || !workspace) return MLA_ERR_NULL;
  if (paged) {
    if (!block_table) return MLA_ERR_NULL;
    if (num_pages < 1 || max_pages < (max_ctx_len + kPage - 1) / kPage) return MLA_ERR_RANGE;
  } else {
    if (stride_tokens < max_ctx_len) return MLA_ERR_RANGE;
  }
  if (kv_chunk < 0 || kv_chunk % kPage != 0) return MLA_ERR_RANGE;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(w_kv_b) || !aligned16(cache) || !aligned16(out) ||
      (workspace != kUseStaticScratch && ((uintptr_t)workspace & 255u) != 0))
    return MLA_ERR_ALIGN;
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return MLA_ERR_ALIGN;
  if (step.rope != nullptr) {
    if (!step.c_new || !step.k_new) return MLA_ERR_NULL;
    if (step.ld_c < kLatent || step.ld_k < kRope) return MLA_ERR_RANGE;
    if (!aligned16(step.c_new) || !aligned16(step.k_new) || step.ld_c % 8 != 0 || step.ld_k % 8 != 0)
      return MLA_ERR_ALIGN;
  }
  const int target = compute_units();
  const bool fp8 = shape->kv_cache_dtype == MLA_CACHE_FP8_E4M3;
  const int groups = query_groups(Sq, fp8);
  const int64_t segs = max_segments(B, max_ctx_len, kv_chunk, target);
  // one split-KV launch covers every (segment, query group) pair; its
  // workgroups times 256 threads must fit in 32 bits
  if (((segs + kXcds - 1) / kXcds) * kXcds * groups > (int64_t)(0xFFFFFFFFu / 256)) return MLA_ERR_RANGE;
  const WorkspaceLayout wl = workspace_layout(B, Sq, (int)segs);
  const bool use_static = workspace == kUseStaticScratch;
  if (use_static) {
    if (wl.total > kStaticScratchBytes) return MLA_ERR_SCRATCH;
  } else if (workspace_bytes < wl.total) {
    return MLA_ERR_WORKSPACE;
  }
  const DeviceSymbols* sym = device_symbols();
  if (sym == nullptr) return MLA_ERR_DEVICE;
  if (use_static) workspace = sym->scratch;

  uint8_t* ws = (uint8_t*)workspace;
  uint16_t* qabs = (uint16_t*)(ws + wl.qabs);
  float* qres = (float*)(ws + wl.qres);
  uint8_t* zero_row = ws + wl.zero_row;
  hipStream_t s = (hipStream_t)stream;
  const int rows = B * Sq;
  const float scale_log2 = shape->softmax_scale * 1.44269504088896340736f;

  PrepParams pp;
  pp.q_nope = (const uint16_t*)q_nope;
  pp.q_pe = (const uint16_t*)q_pe;
  pp.w_kv_b = (const uint16_t*)w_kv_b;
  pp.qabs = qabs;
  pp.qres = qres;
  pp.zero_row = zero_row;
  pp.rows = rows;
  pp.rows_per_wg = prep_rows_per_wg(rows);
  pp.Sq = Sq;
  pp.ctx_lens = ctx_lens;
  pp.max_ctx_len = max_ctx_len;
  pp.num_pages = num_pages;
  pp.faults = sym->faults;
  pp.rotate = step.rope != nullptr;
  memset(&pp.inv, 0, sizeof(pp.inv));
  if (step.rope != nullptr) yarn_frequencies(*step.rope, pp.inv.v);
  pp.c_new = (const uint16_t*)step.c_new;
  pp.ld_c = step.ld_c;
  pp.k_new = (const uint16_t*)step.k_new;
  pp.ld_k = step.ld_k;
  pp.cache = (uint8_t*)cache;
  pp.stride_tokens = stride_tokens;
  pp.block_table = block_table;
  pp.max_pages = max_pages;
  pp.paged = paged ? 1 : 0;
  pp.fp8 = fp8 ? 1 : 0;
  pp.B = B;
  pp.fixed_tiles = kv_chunk / kPage;
  pp.target_segs = std::max(1, target / groups);   // about one workgroup per compute unit
  pp.max_segs = (int)segs;
  pp.seg_desc = (SegDesc*)(ws + wl.seg_desc);
  pp.seg_start = (int32_t*)(ws + wl.seg_start);
  if (launch_prep(pp, s) != hipSuccess) return MLA_ERR_DEVICE;

  DecodeParams p;
  p.qabs = qabs;
  p.cache = (const uint8_t*)cache;
  p.stride_tokens = stride_tokens;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.seg_desc = pp.seg_desc;
  p.Sq = Sq;
  p.segments = (int)segs;
  p.groups = groups;
  p.scale_log2 = scale_log2;
  p.part_o = (uint16_t*)(ws + wl.part_o);
  p.part_lse = (float*)(ws + wl.part_lse);
  p.zero_row = zero_row;
  p.num_pages = num_pages;
  p.faults = sym->faults;
  const bool timed = g_timing.on && g_timing.used < g_timing.capacity;
  {
    hipEvent_t ev0 = timed ? g_timing.ev[2 * g_timing.used] : nullptr;
    hipEvent_t ev1 = timed ? g_timing.ev[2 * g_timing.used + 1] : nullptr;
    const hipError_t e = fp8 ? launch_decode_fp8(p, (int)segs, query_group(Sq, true), paged, s, ev0, ev1)
                             : launch_decode(p, (int)segs, query_group(Sq, false), paged, s, ev0, ev1);
    if (e != hipSuccess) return MLA_ERR_DEVICE;
  }
  if (timed) ++g_timing.used;

  CombineParams cp;
  cp.part_o = p.part_o;
  cp.part_lse = p.part_lse;
  cp.seg_start = pp.seg_start;
  cp.max_segs = (int)segs;
  cp.Sq = Sq;
  cp.hrows = rows * kHeads;
  cp.rows_per_wg = combine_rows_per_wg(rows);
  cp.w_kv_b = (const uint16_t*)w_kv_b;
  cp.qres = qres;
  cp.scale_log2 = scale_log2;
  cp.out = (uint16_t*)out;
  cp.lse = lse;
  cp.up_part = (float*)(ws + wl.up_part);
  cp.corr_part = (float*)(ws + wl.corr_part);
  cp.stat = (float*)(ws + wl.stat);
  if (launch_combine_upproject(cp, s) != hipSuccess) return MLA_ERR_DEVICE;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_default_shape(mla_shape* shape) {
  if (shape == nullptr) return MLA_ERR_NULL;
  shape->num_heads = kHeads;
  shape->kv_lora_rank = kLatent;
  shape->qk_nope_head_dim = kNope;
  shape->qk_rope_head_dim = kRope;
  shape->v_head_dim = kVDim;
  shape->page_size = kPage;
  shape->kv_cache_dtype = MLA_CACHE_BF16;
  const double mscale = 0.1 * 1.0 * log(64.0) + 1.0;      // mscale_all_dim 1.0, factor 64
  shape->softmax_scale = (float)(mscale * mscale / sqrt((double)(kNope + kRope)));
  return MLA_OK;
}

mla_status mla_default_rope(mla_rope_params* p) {
  if (p == nullptr) return MLA_ERR_NULL;
  p->base = 10000.0;
  p->factor = 64.0;
  p->original_max_position = 4096.0;
  p->beta_fast = 32.0;
  p->beta_slow = 1.0;
  p->rope_dim = kRope;
  return MLA_OK;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: unsupported shape";
    case MLA_ERR_RANGE: return "MLA_ERR_RANGE: a size is out of range";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: misaligned pointer or leading dimension";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: a HIP runtime call failed";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: not implemented";
    case MLA_ERR_SCRATCH:
      return "MLA_ERR_SCRATCH: the call needs more scratch than the static buffer of the no-allocation entry point";
    default: return "MLA_ERR_UNKNOWN";
  }
}

mla_status mla_rope_yarn(const mla_rope_params* params, const void* src, int64_t ld_src, void* dst,
                         int64_t ld_dst, const int32_t* positions, int64_t n, void* stream) {
  const mla_status st = check_rope(params);
  if (st != MLA_OK) return st;
  if (n < 0 || ld_src < params->rope_dim || ld_dst < params->rope_dim) return MLA_ERR_RANGE;
  if (n == 0) return MLA_OK;
  if (!src || !dst || !positions) return MLA_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst) || ld_src % 8 != 0 || ld_dst % 8 != 0) return MLA_ERR_ALIGN;
  if (n > (int64_t)1 << 40) return MLA_ERR_RANGE;
  double inv[32];
  yarn_frequencies(*params, inv);
  return launch_rope((const uint16_t*)src, ld_src, (uint16_t*)dst, ld_dst, positions, n, inv,
                     params->rope_dim, (hipStream_t)stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_DEVICE;
}

mla_status mla_cache_append(const mla_shape* shape, void* cache, int64_t num_slots, const void* c_kv,
                            int64_t ld_c, const void* k_pe, int64_t ld_k, const int64_t* slot_mapping,
                            int64_t n, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (n < 0 || num_slots < 0 || ld_c < kLatent || ld_k < kRope) return MLA_ERR_RANGE;
  if (n == 0) return MLA_OK;
  if (!cache || !c_kv || !k_pe || !slot_mapping) return MLA_ERR_NULL;
  if (!aligned16(cache) || !aligned16(c_kv) || !aligned16(k_pe) || ld_c % 8 != 0 || ld_k % 8 != 0 ||
      ((uintptr_t)slot_mapping & 7u) != 0)
    return MLA_ERR_ALIGN;
  if (n > (int64_t)1 << 40) return MLA_ERR_RANGE;
  const DeviceSymbols* sym = device_symbols();
  if (sym == nullptr) return MLA_ERR_DEVICE;
  if (shape->kv_cache_dtype == MLA_CACHE_FP8_E4M3)
    return launch_append_fp8((uint8_t*)cache, num_slots, (const uint16_t*)c_kv, ld_c, (const uint16_t*)k_pe, ld_k,
                             slot_mapping, n, sym->faults, (hipStream_t)stream) == hipSuccess
               ? MLA_OK
               : MLA_ERR_DEVICE;
  return launch_append((uint8_t*)cache, num_slots, (const uint16_t*)c_kv, ld_c, (const uint16_t*)k_pe,
                       ld_k, slot_mapping, n, sym->faults, (hipStream_t)stream) == hipSuccess
             ? MLA_OK
             : MLA_ERR_DEVICE;
}

mla_status mla_decode(const mla_shape* shape, const void* q_nope, const void* q_pe, const void* w_kv_b,
                      const void* cache, int64_t stride_tokens, const int32_t* ctx_lens,
                      int32_t max_ctx_len, int32_t B, int32_t Sq, int32_t kv_chunk, void* out,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(shape, StepInputs{}, q_nope, q_pe, w_kv_b, cache, stride_tokens, 0, nullptr, 0,
                       ctx_lens, max_ctx_len, B, Sq, kv_chunk, out, lse, workspace, workspace_bytes, stream,
                       false);
}

mla_status mla_decode_paged(const mla_shape* shape, const void* q_nope, const void* q_pe,
                            const void* w_kv_b, const void* cache, int64_t num_pages,
                            const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                            int32_t kv_chunk, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return decode_common(shape, StepInputs{}, q_nope, q_pe, w_kv_b, cache, 0, num_pages, block_table,
                       max_pages_per_seq, ctx_lens, max_ctx_len, B, Sq, kv_chunk, out, lse, workspace,
                       workspace_bytes, stream, true);
}

mla_status mla_decode_step(const mla_shape* shape, const mla_rope_params* rope, const void* q_nope,
                           const void* q_pe, const void* c_kv_new, int64_t ld_c, const void* k_pe_new,
                           int64_t ld_k, const void* w_kv_b, void* cache, int64_t stride_tokens,
                           const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                           int32_t kv_chunk, void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (rope == nullptr) return MLA_ERR_NULL;
  return decode_common(shape, StepInputs{rope, c_kv_new, ld_c, k_pe_new, ld_k}, q_nope, q_pe, w_kv_b, cache,
                       stride_tokens, 0, nullptr, 0, ctx_lens, max_ctx_len, B, Sq, kv_chunk, out, lse,
                       workspace, workspace_bytes, stream, false);
}

mla_status mla_decode_step_paged(const mla_shape* shape, const mla_rope_params* rope, const void* q_nope,
                                 const void* q_pe, const void* c_kv_new, int64_t ld_c, const void* k_pe_new,
                                 int64_t ld_k, const void* w_kv_b, void* cache, int64_t num_pages,
                                 const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                                 int32_t kv_chunk, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (rope == nullptr) return MLA_ERR_NULL;
  return decode_common(shape, StepInputs{rope, c_kv_new, ld_c, k_pe_new, ld_k}, q_nope, q_pe, w_kv_b, cache,
                       0, num_pages, block_table, max_pages_per_seq, ctx_lens, max_ctx_len, B, Sq, kv_chunk,
                       out, lse, workspace, workspace_bytes, stream, true);
}

mla_status mla_prefill_workspace_size(const mla_shape* shape, int32_t ctx_len, size_t* bytes) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (shape->kv_cache_dtype != MLA_CACHE_BF16) return MLA_ERR_UNSUPPORTED;
  if (bytes == nullptr) return MLA_ERR_NULL;
  if (ctx_len < 1 || ctx_len > kMaxPrefillCtx) return MLA_ERR_RANGE;
  *bytes = prefill_workspace_bytes(ctx_len);
  return MLA_OK;
}

mla_status mla_prefill(const mla_shape* shape, const void* q_nope, const void* q_pe, const void* w_kv_b,
                       const void* cache, int32_t ctx_len, int32_t Tq, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (shape->kv_cache_dtype != MLA_CACHE_BF16) return MLA_ERR_UNSUPPORTED;
  if (ctx_len < 1 || ctx_len > kMaxPrefillCtx || Tq < 1 || Tq > ctx_len) return MLA_ERR_RANGE;
  if (!q_nope || !q_pe || !w_kv_b || !cache || !out || !workspace) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(w_kv_b) || !aligned16(cache) || !aligned16(out) ||
      !aligned16(workspace))
    return MLA_ERR_ALIGN;
  if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return MLA_ERR_ALIGN;
  if (workspace_bytes < prefill_workspace_bytes(ctx_len)) return MLA_ERR_WORKSPACE;
  const DeviceSymbols* sym = device_symbols();
  if (sym == nullptr) return MLA_ERR_DEVICE;
  const float scale_log2 = shape->softmax_scale * 1.44269504088896340736f;
  if (launch_prefill((const uint16_t*)q_nope, (const uint16_t*)q_pe, (const uint16_t*)w_kv_b, (const uint8_t*)cache,
                     ctx_len, Tq, scale_log2, (uint16_t*)workspace, (uint16_t*)out, lse, sym->faults,
                     (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_DEVICE;
  return MLA_OK;
}

mla_status mla_decode_workspace_size(const mla_shape* shape, int32_t B, int32_t Sq, int32_t max_ctx_len,
                                     int32_t kv_chunk, size_t* bytes) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (bytes == nullptr) return MLA_ERR_NULL;
  if (B < 0 || Sq < 1 || Sq > kMaxSq || max_ctx_len < Sq) return MLA_ERR_RANGE;
  if ((int64_t)B * Sq > kMaxRows) return MLA_ERR_RANGE;
  if (kv_chunk < 0 || kv_chunk % kPage != 0) return MLA_ERR_RANGE;
  if (B == 0) {
    *bytes = 0;
    return MLA_OK;
  }
  const int64_t segs = max_segments(B, max_ctx_len, kv_chunk, compute_units());
  if (segs > 0x7FFFFFFF) return MLA_ERR_RANGE;
  *bytes = workspace_layout(B, Sq, (int)segs).total;
  return MLA_OK;
}

mla_status mla_decode_step_paged_noalloc(const mla_shape* shape, const mla_rope_params* rope, const void* q_nope,
                                         const void* q_pe, const void* c_kv_new, int64_t ld_c, const void* k_pe_new,
                                         int64_t ld_k, const void* w_kv_b, void* cache, int64_t num_pages,
                                         const int32_t* block_table, int32_t max_pages_per_seq,
                                         const int32_t* ctx_lens, int32_t max_ctx_len, int32_t B, int32_t Sq,
                                         int32_t kv_chunk, void* out, float* lse, void* stream) {
  if (rope == nullptr) return MLA_ERR_NULL;
  return decode_common(shape, StepInputs{rope, c_kv_new, ld_c, k_pe_new, ld_k}, q_nope, q_pe, w_kv_b, cache,
                       0, num_pages, block_table, max_pages_per_seq, ctx_lens, max_ctx_len, B, Sq, kv_chunk,
                       out, lse, kUseStaticScratch, 0, stream, true);
}

mla_status mla_device_faults(uint32_t* faults, int32_t clear) {
  if (faults == nullptr) return MLA_ERR_NULL;
  const DeviceSymbols* sym = device_symbols();
  if (sym == nullptr) return MLA_ERR_DEVICE;
  if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_DEVICE;
  if (hipMemcpy(faults, sym->faults, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_DEVICE;
  if (clear) {
    if (hipMemset(sym->faults, 0, sizeof(uint32_t)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
      return MLA_ERR_DEVICE;
  }
  return MLA_OK;
}

mla_status mla_check_decode_inputs(int32_t B, int32_t Sq, int32_t max_ctx_len, const int32_t* ctx_lens,
                                   const int32_t* block_table, int32_t max_pages_per_seq, int64_t num_pages,
                                   uint32_t* faults) {
  if (faults == nullptr || (B > 0 && ctx_lens == nullptr)) return MLA_ERR_NULL;
  if (B < 0 || Sq < 1 || Sq > kMaxSq || max_ctx_len < Sq) return MLA_ERR_RANGE;
  if (block_table != nullptr && (num_pages < 1 || max_pages_per_seq < (max_ctx_len + kPage - 1) / kPage))
    return MLA_ERR_RANGE;
  uint32_t f = 0;
  for (int b = 0; b < B; ++b) {
    bool bad;
    const int L = clamp_ctx_len(ctx_lens[b], Sq, max_ctx_len, &bad);
    if (bad) f |= kFaultCtxLen;
    if (block_table != nullptr) {
      const int32_t* row = block_table + (size_t)b * max_pages_per_seq;
      for (int k = 0; k < (L + kPage - 1) / kPage; ++k)
        if (!page_ok(row[k], num_pages)) f |= kFaultPage;
    }
  }
  *faults = f;
  return MLA_OK;
}

mla_status mla_check_slot_mapping(const int64_t* slot_mapping, int64_t n, int64_t num_slots, uint32_t* faults) {
  if (faults == nullptr || (n > 0 && slot_mapping == nullptr)) return MLA_ERR_NULL;
  if (n < 0 || num_slots < 0) return MLA_ERR_RANGE;
  uint32_t f = 0;
  for (int64_t i = 0; i < n; ++i)
    if (slot_fault(slot_mapping[i], num_slots)) f |= kFaultSlot;
  *faults = f;
  return MLA_OK;
}

mla_status mla_timing_enable(int32_t max_calls) {
  if (max_calls < 1 || max_calls > (1 << 20)) return MLA_ERR_RANGE;
  timing_free();
  g_timing.ev = new hipEvent_t[2 * (size_t)max_calls];
  for (int i = 0; i < 2 * max_calls; ++i) {
    if (hipEventCreate(&g_timing.ev[i]) != hipSuccess) {
      g_timing.capacity = i / 2;
      for (int k = 2 * g_timing.capacity; k < i; ++k) (void)hipEventDestroy(g_timing.ev[k]);
      timing_free();
      return MLA_ERR_DEVICE;
    }
  }
  g_timing.capacity = max_calls;
  g_timing.used = 0;
  g_timing.on = true;
  return MLA_OK;
}

mla_status mla_timing_collect(double* total_ms, int32_t* launches) {
  if (total_ms == nullptr || launches == nullptr) return MLA_ERR_NULL;
  double sum = 0.0;
  for (int i = 0; i < g_timing.used; ++i) {
    if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) return MLA_ERR_DEVICE;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess)
      return MLA_ERR_DEVICE;
    sum += ms;
  }
  *total_ms = sum;
  *launches = g_timing.used;
  return MLA_OK;
}

mla_status mla_timing_disable(void) {
  timing_free();
  return MLA_OK;
}

mla_status mla_decode_auto_chunk(int32_t B, int32_t Sq, int32_t max_ctx_len, int32_t* kv_chunk) {
  if (kv_chunk == nullptr) return MLA_ERR_NULL;
  if (B < 0 || Sq < 1 || Sq > kMaxSq || max_ctx_len < Sq) return MLA_ERR_RANGE;
  *kv_chunk = balanced_chunk(B < 1 ? 1 : B, max_ctx_len, std::max(1, compute_units() / query_groups(Sq, false)));
  return MLA_OK;
}

}  // extern "C"
