// C ABI of libgqla: argument validation on the host, then kernel dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and never touches the device.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/gqla.h"
#include "common.hip.h"
#include "params.hip.h"

namespace gqla {
hipError_t gqa_dispatch(int hpg, int sq, int dn, int dv, int dr, const DecodeParams& p,
                        hipStream_t stream, bool* supported);
hipError_t absorb_dispatch(int hpg, int sq, int r, int dn, int dv, int dr, const DecodeParams& p,
                           hipStream_t stream, bool* supported, bool merge_only);
hipError_t expand_dispatch(int r, int dn, int dv, int dr, const ExpandParams& p, hipStream_t stream,
                           bool* supported);
hipError_t combine_dispatch(int dv, const CombineParams& p, hipStream_t stream, bool* supported);
hipError_t append_launch(const AppendParams& p, int r, int dn, int dv, int dr, hipStream_t stream, bool* supported);
hipError_t sparse_codes_launch(const SparseCodeParams& p, hipStream_t stream);
}  // namespace gqla

// Workspace of gqla_decode_mqa_absorb_noalloc: one copy per GPU, kept until
// the process ends.  Host code never uses the name itself (on the host it is a
// stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GQLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];                 // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up on the first call with
// that device current.
hipError_t scratch_of_current_device(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if ((int)sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// The shapes compiled into this library.
bool shape_supported(const gqla_dims* d) {
  const int hpg = d->num_heads / d->num_groups;
  if (d->block_size != 64 || (d->s_q != 1 && d->s_q != 2)) return false;
  if (d->d_latent == 512 && d->d_rope == 64 && d->d_nope == 128 && d->d_v == 128)
    return hpg == 16 || hpg == 4 || hpg == 32;
  if (d->d_latent == 64 && d->d_rope == 16 && d->d_nope == 32 && d->d_v == 32) return hpg == 8;
  return false;
}

int check_dims(const gqla_dims* d) {
  if (!d) return GQLA_ERR_INVALID_ARG;
  if (d->num_heads <= 0 || d->num_groups <= 0 || d->d_latent <= 0 || d->d_rope < 0 ||
      d->d_nope <= 0 || d->d_v <= 0 || d->s_q <= 0 || d->block_size <= 0)
    return GQLA_ERR_INVALID_ARG;
  if (d->num_heads % d->num_groups != 0) return GQLA_ERR_INVALID_ARG;
  if (!(isfinite(d->softmax_scale)) || d->softmax_scale < 0.f) return GQLA_ERR_INVALID_ARG;
  if (!shape_supported(d)) return GQLA_ERR_UNSUPPORTED_SHAPE;
  return GQLA_OK;
}

float scale_of(const gqla_dims* d) {
  return d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)(d->d_nope + d->d_rope));
}

// Shared checks of the two decode entry points.  cache/w_uk/w_uv are checked
// by the caller (the GQA path has no weights).  `partials`: the split plan
// writes caller-provided part_out / part_lse (GQA path); otherwise `out` is
// always required (the absorb path merges its splits itself).
int check_decode(const gqla_dims* d, int32_t batch, const void* q_nope, const void* q_rope,
                 const void* cache, const int32_t* block_table, int32_t max_blocks,
                 const int32_t* seqlens, const int32_t* split_offsets, int32_t split_tokens,
                 int32_t total_splits, const void* out, const float* lse, const float* part_out,
                 const float* part_lse, bool partials) {
  int st = check_dims(d);
  if (st != GQLA_OK) return st;
  if (batch < 0 || max_blocks <= 0) return GQLA_ERR_INVALID_ARG;
  if (!q_nope || !q_rope || !cache || !block_table || !seqlens) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(cache) || !aligned4(block_table) ||
      !aligned4(seqlens))
    return GQLA_ERR_MISALIGNED;
  if (split_offsets) {
    if (split_tokens <= 0 || split_tokens % d->block_size != 0 || total_splits < batch)
      return GQLA_ERR_BAD_SPLIT_PLAN;
    if (!aligned4(split_offsets)) return GQLA_ERR_MISALIGNED;
    if (partials) {
      if (!part_out || !part_lse) return GQLA_ERR_INVALID_ARG;
      if (!aligned16(part_out) || !aligned4(part_lse)) return GQLA_ERR_MISALIGNED;
    } else if (!out) {
      return GQLA_ERR_INVALID_ARG;
    }
  } else {
    if (!out) return GQLA_ERR_INVALID_ARG;
  }
  if (out && !aligned16(out)) return GQLA_ERR_MISALIGNED;
  if (lse && !aligned4(lse)) return GQLA_ERR_MISALIGNED;
  return GQLA_OK;
}

gqla::DecodeParams make_params(const gqla_dims* d, int32_t batch, const void* q_nope,
                               const void* q_rope, const void* cache, const int32_t* block_table,
                               int32_t max_blocks, const int32_t* seqlens, const void* w_uk,
                               const void* w_uv, const int32_t* split_offsets,
                               int32_t split_tokens, int32_t total_splits, void* out, float* lse,
                               float* part_out, float* part_lse) {
  gqla::DecodeParams p;
  p.q_nope = (const uint16_t*)q_nope;
  p.q_rope = (const uint16_t*)q_rope;
  p.cache = (const uint16_t*)cache;
  p.block_table = block_table;
  p.seqlens = seqlens;
  p.w_uk = (const uint16_t*)w_uk;
  p.w_uv = (const uint16_t*)w_uv;
  p.split_offsets = split_offsets;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.part_out = part_out;
  p.part_lse = part_lse;
  p.batch = batch;
  p.max_blocks = max_blocks;
  p.num_groups = d->num_groups;
  p.split_tokens = split_offsets ? split_tokens : 0;
  p.num_units = split_offsets ? total_splits : batch;
  p.scale_log2 = scale_of(d) * gqla::kLog2e;
  p.qcat = nullptr;
  p.wuvT = nullptr;
  p.olat = nullptr;
  p.olse = nullptr;
  p.codes = nullptr;
  p.topk_pad = 0;
  return p;
}

int finish(hipError_t e, bool supported) {
  if (!supported) return GQLA_ERR_UNSUPPORTED_SHAPE;
  return e == hipSuccess ? GQLA_OK : GQLA_ERR_HIP;
}

int enqueue_combine(const gqla_dims* d, int32_t batch, const int32_t* split_offsets,
                    const float* part_out, const float* part_lse, void* out, float* lse,
                    hipStream_t stream) {
  gqla::CombineParams c;
  c.part_out = part_out;
  c.part_lse = part_lse;
  c.split_offsets = split_offsets;
  c.out = (uint16_t*)out;
  c.lse = lse;
  c.batch = batch;
  c.rows = d->s_q * d->num_heads;
  bool ok = true;
  hipError_t e = gqla::combine_dispatch(d->d_v, c, stream, &ok);
  return finish(e, ok);
}

}  // namespace

extern "C" {

int gqla_abi_version(void) { return 201; }

const char* gqla_status_string(int status) {
  switch (status) {
    case GQLA_OK: return "GQLA_OK";
    case GQLA_ERR_INVALID_ARG: return "GQLA_ERR_INVALID_ARG: null pointer, bad dimension or inconsistent argument";
    case GQLA_ERR_UNSUPPORTED_SHAPE: return "GQLA_ERR_UNSUPPORTED_SHAPE: no kernel instantiated for these dimensions";
    case GQLA_ERR_MISALIGNED: return "GQLA_ERR_MISALIGNED: tensor pointers must be 16-byte aligned (index arrays 4-byte)";
    case GQLA_ERR_BAD_SPLIT_PLAN: return "GQLA_ERR_BAD_SPLIT_PLAN: split_tokens must be a positive multiple of block_size and total_splits >= batch";
    case GQLA_ERR_HIP: return "GQLA_ERR_HIP: kernel launch failed";
    case GQLA_ERR_SCRATCH_LIMIT: return "GQLA_ERR_SCRATCH_LIMIT: the call needs more workspace than the library's fixed scratch array (GQLA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown gqla status";
  }
}

int64_t gqla_latent_page_elems(const gqla_dims* d) {
  if (!d) return -1;
  return (int64_t)d->block_size * (d->d_latent + d->d_rope);
}

int64_t gqla_expanded_page_elems(const gqla_dims* d) {
  if (!d) return -1;
  return (int64_t)d->block_size * ((int64_t)d->num_groups * (d->d_nope + d->d_v) + d->d_rope);
}

// Workspace of the absorb path, four regions each starting on a 256-byte
// boundary: the absorbed query rows [batch][s_q][h_q][r + d_rope] (bf16),
// W_UV transposed [g][d_v][r] (bf16), the split partials o_lat
// [units][s_q][h_q][r] (bf16) and their lse [units][s_q][h_q] (fp32), with
// units = total_splits under a split plan, else batch.
static bool absorb_ws_dims_ok(const gqla_dims* d, int32_t batch, int32_t total_splits) {
  return d && batch > 0 && total_splits >= 0 && d->s_q > 0 && d->num_heads > 0 && d->d_latent > 0 &&
         d->d_rope >= 0 && d->num_groups > 0 && d->d_v > 0;
}

static void absorb_ws_layout(const gqla_dims* d, int32_t batch, int32_t total_splits, uint64_t off[5]) {
  auto up = [](uint64_t n) { return (n + 255u) & ~(uint64_t)255u; };
  const uint64_t rows = (uint64_t)d->s_q * d->num_heads;
  const uint64_t units = total_splits > 0 ? (uint64_t)total_splits : (uint64_t)batch;
  off[0] = 0;
  off[1] = off[0] + up((uint64_t)batch * rows * (uint64_t)(d->d_latent + d->d_rope) * 2u);
  off[2] = off[1] + up((uint64_t)d->num_groups * d->d_v * (uint64_t)d->d_latent * 2u);
  off[3] = off[2] + up(units * rows * (uint64_t)d->d_latent * 2u);
  off[4] = off[3] + up(units * rows * 4u);
}

uint64_t gqla_mqa_absorb_workspace_bytes(const gqla_dims* d, int32_t batch, int32_t total_splits) {
  if (!absorb_ws_dims_ok(d, batch, total_splits)) return 0;
  uint64_t off[5];
  absorb_ws_layout(d, batch, total_splits, off);
  return off[4];
}

int gqla_mqa_absorb_workspace_offsets(const gqla_dims* d, int32_t batch, int32_t total_splits,
                                      uint64_t* offsets) {
  if (!absorb_ws_dims_ok(d, batch, total_splits) || !offsets) return GQLA_ERR_INVALID_ARG;
  uint64_t off[5];
  absorb_ws_layout(d, batch, total_splits, off);
  for (int i = 0; i < 4; ++i) offsets[i] = off[i];
  return GQLA_OK;
}

int gqla_expand_cache(const gqla_dims* d, const void* latent_pages, const void* w_uk,
                      const void* w_uv, int64_t num_pages, const int32_t* page_ids,
                      int64_t num_pages_to_expand, void* expanded_pages, void* stream) {
  int st = check_dims(d);
  if (st != GQLA_OK) return st;
  if (num_pages < 0 || num_pages_to_expand < 0) return GQLA_ERR_INVALID_ARG;
  if (!page_ids && num_pages_to_expand > num_pages) return GQLA_ERR_INVALID_ARG;
  if (num_pages_to_expand == 0) return GQLA_OK;
  if (!latent_pages || !w_uk || !w_uv || !expanded_pages) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(latent_pages) || !aligned16(w_uk) || !aligned16(w_uv) ||
      !aligned16(expanded_pages) || (page_ids && !aligned4(page_ids)))
    return GQLA_ERR_MISALIGNED;
  gqla::ExpandParams p;
  p.latent = (const uint16_t*)latent_pages;
  p.w_uk = (const uint16_t*)w_uk;
  p.w_uv = (const uint16_t*)w_uv;
  p.page_ids = page_ids;
  p.expanded = (uint16_t*)expanded_pages;
  p.n_expand = num_pages_to_expand;
  p.num_groups = d->num_groups;
  p.whole_quads = 0;                               // (set by the launcher)
  p.pieces = 1;
  bool ok = true;
  hipError_t e = gqla::expand_dispatch(d->d_latent, d->d_nope, d->d_v, d->d_rope, p,
                                       (hipStream_t)stream, &ok);
  return finish(e, ok);
}

int gqla_append_tokens(const gqla_dims* d, int32_t batch, int32_t n_new, const void* new_rows,
                       void* latent_pages, int64_t num_pages, const int32_t* block_table,
                       int32_t max_blocks, const int32_t* cache_seqlens, const void* w_uk,
                       const void* w_uv, void* expanded_pages, void* stream) {
  int st = check_dims(d);
  if (st != GQLA_OK) return st;
  if (batch < 1 || n_new < 1 || n_new > d->block_size || num_pages < 1 || max_blocks < 1)
    return GQLA_ERR_INVALID_ARG;
  if (!new_rows || !latent_pages || !block_table || !cache_seqlens) return GQLA_ERR_INVALID_ARG;
  if (expanded_pages && (!w_uk || !w_uv)) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(new_rows) || !aligned16(latent_pages) || !aligned4(block_table) ||
      !aligned4(cache_seqlens) ||
      (expanded_pages && (!aligned16(expanded_pages) || !aligned16(w_uk) || !aligned16(w_uv))))
    return GQLA_ERR_MISALIGNED;
  gqla::AppendParams a;
  a.new_rows = (const uint16_t*)new_rows;
  a.latent = (uint16_t*)latent_pages;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.w_uk = (const uint16_t*)w_uk;
  a.w_uv = (const uint16_t*)w_uv;
  a.expanded = (uint16_t*)expanded_pages;
  a.row_elems = (int64_t)d->d_latent + d->d_rope;
  a.num_groups = d->num_groups;
  a.batch = batch;
  a.n_new = n_new;
  a.max_blocks = max_blocks;
  a.bs = d->block_size;
  (void)num_pages;
  bool ok = true;
  hipError_t e = gqla::append_launch(a, d->d_latent, d->d_nope, d->d_v, d->d_rope, (hipStream_t)stream, &ok);
  return finish(e, ok);
}

int gqla_decode_mqa_absorb(const gqla_dims* d, int32_t batch, const void* q_nope,
                           const void* q_rope, const void* latent_pages,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* cache_seqlens, const void* w_uk, const void* w_uv,
                           const int32_t* split_offsets, int32_t split_tokens,
                           int32_t total_splits, void* out, float* lse, void* workspace,
                           uint64_t workspace_bytes, void* stream) {
  int st = check_decode(d, batch, q_nope, q_rope, latent_pages, block_table, max_blocks,
                        cache_seqlens, split_offsets, split_tokens, total_splits, out, lse,
                        nullptr, nullptr, false);
  if (st != GQLA_OK) return st;
  if (!w_uk || !w_uv) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(w_uk) || !aligned16(w_uv)) return GQLA_ERR_MISALIGNED;
  if (batch == 0) return GQLA_OK;
  const int32_t ws_splits = split_offsets ? total_splits : 0;
  if (!workspace || workspace_bytes < gqla_mqa_absorb_workspace_bytes(d, batch, ws_splits))
    return GQLA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return GQLA_ERR_MISALIGNED;
  gqla::DecodeParams p = make_params(d, batch, q_nope, q_rope, latent_pages, block_table,
                                     max_blocks, cache_seqlens, w_uk, w_uv, split_offsets,
                                     split_tokens, total_splits, out, lse, nullptr, nullptr);
  uint64_t off[5];
  absorb_ws_layout(d, batch, ws_splits, off);
  p.qcat = (uint16_t*)((char*)workspace + off[0]);
  p.wuvT = (uint16_t*)((char*)workspace + off[1]);
  p.olat = (uint16_t*)((char*)workspace + off[2]);
  p.olse = (float*)((char*)workspace + off[3]);
  bool ok = true;
  hipError_t e = gqla::absorb_dispatch(d->num_heads / d->num_groups, d->s_q, d->d_latent,
                                       d->d_nope, d->d_v, d->d_rope, p, (hipStream_t)stream, &ok, false);
  return finish(e, ok);
}

int gqla_decode_mqa_absorb_noalloc(const gqla_dims* d, int32_t batch, const void* q_nope,
                                   const void* q_rope, const void* latent_pages,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* cache_seqlens, const void* w_uk, const void* w_uv,
                                   const int32_t* split_offsets, int32_t split_tokens,
                                   int32_t total_splits, void* out, float* lse, void* stream) {
  int st = check_decode(d, batch, q_nope, q_rope, latent_pages, block_table, max_blocks,
                        cache_seqlens, split_offsets, split_tokens, total_splits, out, lse,
                        nullptr, nullptr, false);
  if (st != GQLA_OK) return st;
  if (!w_uk || !w_uv) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(w_uk) || !aligned16(w_uv)) return GQLA_ERR_MISALIGNED;
  if (batch == 0) return GQLA_OK;
  const uint64_t need = gqla_mqa_absorb_workspace_bytes(d, batch, split_offsets ? total_splits : 0);
  if (need == 0) return GQLA_ERR_INVALID_ARG;
  if (need > GQLA_NOALLOC_SCRATCH_BYTES) return GQLA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (scratch_of_current_device((hipStream_t)stream, &ws) != hipSuccess) return GQLA_ERR_HIP;
  return gqla_decode_mqa_absorb(d, batch, q_nope, q_rope, latent_pages, block_table, max_blocks,
                                cache_seqlens, w_uk, w_uv, split_offsets, split_tokens, total_splits, out,
                                lse, ws, need, stream);
}

uint64_t gqla_mqa_absorb_merge_workspace_bytes(const gqla_dims* d) {
  if (!d || d->num_groups <= 0 || d->d_v <= 0 || d->d_latent <= 0) return 0;
  return ((uint64_t)d->num_groups * d->d_v * (uint64_t)d->d_latent * 2u + 255u) & ~(uint64_t)255u;
}

int gqla_mqa_absorb_merge(const gqla_dims* d, int32_t batch, const void* part_lat, const float* part_lse,
                          const int32_t* split_offsets, int32_t total_splits, const void* w_uv, void* out,
                          float* lse, void* workspace, uint64_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st != GQLA_OK) return st;
  if (batch < 0) return GQLA_ERR_INVALID_ARG;
  if (split_offsets && total_splits < batch) return GQLA_ERR_BAD_SPLIT_PLAN;
  if (!part_lat || !part_lse || !w_uv || !out) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(part_lat) || !aligned4(part_lse) || !aligned16(w_uv) || !aligned16(out) ||
      (lse && !aligned4(lse)) || (split_offsets && !aligned4(split_offsets)))
    return GQLA_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < gqla_mqa_absorb_merge_workspace_bytes(d)) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return GQLA_ERR_MISALIGNED;
  if (batch == 0) return GQLA_OK;
  gqla::DecodeParams p = make_params(d, batch, nullptr, nullptr, nullptr, nullptr, 1, nullptr, nullptr, w_uv,
                                     split_offsets, 0, split_offsets ? total_splits : batch, out, lse, nullptr,
                                     nullptr);
  p.wuvT = (uint16_t*)workspace;
  p.olat = (uint16_t*)part_lat;
  p.olse = (float*)part_lse;
  bool ok = true;
  hipError_t e = gqla::absorb_dispatch(d->num_heads / d->num_groups, d->s_q, d->d_latent, d->d_nope, d->d_v,
                                       d->d_rope, p, (hipStream_t)stream, &ok, true);
  return finish(e, ok);
}

int gqla_decode_gqa(const gqla_dims* d, int32_t batch, const void* q_nope, const void* q_rope,
                    const void* expanded_pages, const int32_t* block_table, int32_t max_blocks,
                    const int32_t* cache_seqlens, const int32_t* split_offsets,
                    int32_t split_tokens, int32_t total_splits, void* out, float* lse,
                    float* part_out, float* part_lse, void* stream) {
  int st = check_decode(d, batch, q_nope, q_rope, expanded_pages, block_table, max_blocks,
                        cache_seqlens, split_offsets, split_tokens, total_splits, out, lse,
                        part_out, part_lse, true);
  if (st != GQLA_OK) return st;
  if (batch == 0) return GQLA_OK;
  gqla::DecodeParams p = make_params(d, batch, q_nope, q_rope, expanded_pages, block_table,
                                     max_blocks, cache_seqlens, nullptr, nullptr, split_offsets,
                                     split_tokens, total_splits, out, lse, part_out, part_lse);
  bool ok = true;
  hipError_t e = gqla::gqa_dispatch(d->num_heads / d->num_groups, d->s_q, d->d_nope, d->d_v,
                                    d->d_rope, p, (hipStream_t)stream, &ok);
  st = finish(e, ok);
  if (st != GQLA_OK || !split_offsets || !out) return st;
  return enqueue_combine(d, batch, split_offsets, part_out, part_lse, out, lse, (hipStream_t)stream);
}

int gqla_sparse_workspace_offsets(const gqla_dims* d, int32_t batch, int32_t topk,
                                  int32_t split_entries, uint64_t* offsets) {
  if (!d || !offsets || d->num_groups <= 0 || d->num_heads <= 0 || d->s_q <= 0 || d->d_v <= 0 ||
      batch <= 0 || topk <= 0 || topk > INT32_MAX - 31 || split_entries < 0)
    return GQLA_ERR_INVALID_ARG;
  const uint64_t pad = ((uint64_t)topk + 31) / 32 * 32;
  auto up = [](uint64_t x) { return (x + 255) / 256 * 256; };
  const uint64_t codes = (uint64_t)batch * (uint64_t)d->num_groups * pad * 4u;
  uint64_t o = up(codes);
  offsets[0] = 0;
  if (split_entries == 0) {
    offsets[1] = offsets[2] = offsets[3] = offsets[4] = codes;
    return GQLA_OK;
  }
  const uint64_t units = (uint64_t)batch * ((pad + (uint64_t)split_entries - 1) / (uint64_t)split_entries);
  const uint64_t rows = units * (uint64_t)d->s_q * (uint64_t)d->num_heads;
  offsets[1] = o;                                   // split plan, int32 [batch + 1]
  o = up(o + ((uint64_t)batch + 1) * 4u);
  offsets[2] = o;                                   // partial outputs, fp32 [units][s_q][h_q][d_v]
  o = up(o + rows * (uint64_t)d->d_v * 4u);
  offsets[3] = o;                                   // partial lse, fp32 [units][s_q][h_q]
  offsets[4] = o + rows * 4u;                       // end
  return GQLA_OK;
}

uint64_t gqla_sparse_workspace_bytes(const gqla_dims* d, int32_t batch, int32_t topk, int32_t split_entries) {
  uint64_t off[5];
  if (gqla_sparse_workspace_offsets(d, batch, topk, split_entries, off) != GQLA_OK) return 0;
  return off[4];
}

int gqla_decode_gqa_sparse(const gqla_dims* d, int32_t batch, const void* q_nope, const void* q_rope,
                           const void* expanded_pages, int64_t num_pages, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* cache_seqlens, const int32_t* indices,
                           int32_t topk, int32_t split_entries, void* out, float* lse,
                           void* workspace, uint64_t workspace_bytes, void* stream) {
  int st = check_decode(d, batch, q_nope, q_rope, expanded_pages, block_table, max_blocks,
                        cache_seqlens, nullptr, 0, 0, out, lse, nullptr, nullptr, true);
  if (st != GQLA_OK) return st;
  if (!indices || topk <= 0 || topk > INT32_MAX - 31 || num_pages <= 0) return GQLA_ERR_INVALID_ARG;
  if (num_pages > ((int64_t)1 << 28) / d->block_size) return GQLA_ERR_INVALID_ARG;   // 28-bit row codes
  if (split_entries < 0 || split_entries % 32 != 0) return GQLA_ERR_BAD_SPLIT_PLAN;
  if (!aligned4(indices)) return GQLA_ERR_MISALIGNED;
  if (batch == 0) return GQLA_OK;
  uint64_t off[5];
  if (gqla_sparse_workspace_offsets(d, batch, topk, split_entries, off) != GQLA_OK) return GQLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < off[4]) return GQLA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return GQLA_ERR_MISALIGNED;
  const int32_t topk_pad = (topk + 31) / 32 * 32;
  const int32_t n_split = split_entries ? (topk_pad + split_entries - 1) / split_entries : 0;
  if (split_entries && (int64_t)batch * n_split > INT32_MAX) return GQLA_ERR_BAD_SPLIT_PLAN;
  unsigned char* ws = (unsigned char*)workspace;
  int32_t* plan = split_entries ? (int32_t*)(ws + off[1]) : nullptr;
  float* part_out = split_entries ? (float*)(ws + off[2]) : nullptr;
  float* part_lse = split_entries ? (float*)(ws + off[3]) : nullptr;
  gqla::SparseCodeParams cp;
  cp.indices = indices;
  cp.block_table = block_table;
  cp.seqlens = cache_seqlens;
  cp.codes = (uint32_t*)workspace;
  cp.num_pages = num_pages;
  cp.batch = batch;
  cp.num_groups = d->num_groups;
  cp.topk = topk;
  cp.topk_pad = topk_pad;
  cp.max_blocks = max_blocks;
  cp.block_size = d->block_size;
  cp.s_q = d->s_q;
  cp.split_offsets = plan;
  cp.splits_per_seq = n_split;
  if (gqla::sparse_codes_launch(cp, (hipStream_t)stream) != hipSuccess) return GQLA_ERR_HIP;
  gqla::DecodeParams p = make_params(d, batch, q_nope, q_rope, expanded_pages, block_table,
                                     max_blocks, cache_seqlens, nullptr, nullptr, plan, split_entries,
                                     batch * n_split, out, lse, part_out, part_lse);
  p.codes = (const uint32_t*)workspace;
  p.topk_pad = topk_pad;
  bool ok = true;
  hipError_t e = gqla::gqa_dispatch(d->num_heads / d->num_groups, d->s_q, d->d_nope, d->d_v,
                                    d->d_rope, p, (hipStream_t)stream, &ok);
  st = finish(e, ok);
  if (st != GQLA_OK || !split_entries) return st;
  return enqueue_combine(d, batch, plan, part_out, part_lse, out, lse, (hipStream_t)stream);
}

int gqla_splitkv_combine(const gqla_dims* d, int32_t batch, const int32_t* split_offsets,
                         int32_t total_splits, const float* part_out, const float* part_lse,
                         void* out, float* lse, void* stream) {
  int st = check_dims(d);
  if (st != GQLA_OK) return st;
  if (batch < 0 || total_splits < 0) return GQLA_ERR_INVALID_ARG;
  if (batch == 0) return GQLA_OK;
  if (!split_offsets || !part_out || !part_lse || !out) return GQLA_ERR_INVALID_ARG;
  if (!aligned4(split_offsets) || !aligned16(part_out) || !aligned4(part_lse) || !aligned16(out) ||
      (lse && !aligned4(lse)))
    return GQLA_ERR_MISALIGNED;
  return enqueue_combine(d, batch, split_offsets, part_out, part_lse, out, lse, (hipStream_t)stream);
}

}  // extern "C"
