// flk_api.cpp -- the C ABI declared in include/flk.h: host-side validation, then launches.
//
// Every check that can fail runs before the first HIP call, so a rejected call enqueues
// nothing and writes nothing (the FlashLoop RFC, vllm-rlt #156, section 4: incompatible
// explicit choices fail clearly rather than silently changing the algorithm).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "../../include/flk.h"
#include "flk_internal.h"
#include "flk_readers.h"
#include "flk_fp4.h"
#include "flk_select.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

flk_status check_stream_ptrs(const void* codes, const void* params) {
  if (!codes || !params) return FLK_E_NULL;
  if (!aligned(codes, 16) || !aligned(params, 16)) return FLK_E_ALIGN;
  return FLK_OK;
}

bool k_tiles(const flk_desc* d) { return d->kind == FLK_KIND_K && d->k_grouping == FLK_KGROUP_TILE; }

// Groups of a stream of n compact rows over T positions: K has one parameter row per 64
// compact rows, or per 64-position tile with tile groups; V one per (row, head, 64 channels).
size_t n_groups(const flk_desc* d, int64_t n, int64_t T) {
  const size_t W = size_t(d->n_heads) * size_t(d->head_dim);
  if (k_tiles(d)) return T < 1 ? 0 : size_t((T + FLK_GROUP - 1) / FLK_GROUP) * W;
  if (d->kind == FLK_KIND_K) return size_t((n + FLK_GROUP - 1) / FLK_GROUP) * W;
  return size_t(n) * size_t(d->n_heads) * size_t((d->head_dim + FLK_GROUP - 1) / FLK_GROUP);
}

// The window part of a stream's buffers: codes and params of the rows (and, for tile-grouped
// K, tiles) before position p0, which hold rows_before compact rows.
size_t codes_offset(const flk_desc* d, int64_t rows_before) {
  return size_t(rows_before) * size_t(d->n_heads) * size_t(d->head_dim) / 2;
}
size_t params_offset(const flk_desc* d, int64_t rows_before, int64_t p0) {
  const size_t W = size_t(d->n_heads) * size_t(d->head_dim);
  if (d->kind == FLK_KIND_K) return k_tiles(d) ? size_t(p0 / FLK_GROUP) * W : size_t(rows_before / FLK_GROUP) * W;
  return size_t(rows_before) * size_t(d->n_heads) * size_t((d->head_dim + FLK_GROUP - 1) / FLK_GROUP);
}

flk::EncArgs enc_args(const flk_desc* d, const void* x, const int32_t* rows, int32_t n, int32_t T, void* recon,
                      uint8_t* codes, uint32_t* params, int32_t* tile_start, uint32_t* status) {
  return flk::EncArgs{static_cast<const uint16_t*>(x), rows, static_cast<uint16_t*>(recon), codes, params,
                      rows ? tile_start : nullptr, status, n, T, d->n_heads * d->head_dim, 0, 0,
                      k_tiles(d) ? 1 : 0};
}

// Every BF16 tensor of a call stays below 4 GiB (n*H*D < 2^31 elements): the kernels address
// rows through buffer descriptors with 32-bit byte offsets.
bool rows_fit(const flk_desc* d, int64_t n) {
  return n * int64_t(d->n_heads) * int64_t(d->head_dim) < (int64_t(1) << 31);
}

flk_status to_status(hipError_t e) { return e == hipSuccess ? FLK_OK : FLK_E_LAUNCH; }

bool is_fp4(const flk_desc* d) { return d->format == FLK_FMT_NVFP4 || d->format == FLK_FMT_MXFP4; }
bool is_mx(const flk_desc* d) { return d->format == FLK_FMT_MXFP4; }

// The check of the entry points that implement INT4 streams only: a well-formed FP4
// descriptor is a valid request they do not implement.
flk_status int4_desc(const flk_desc* d) {
  const flk_status st = flk_desc_check(d);
  if (st != FLK_OK) return st;
  return is_fp4(d) ? FLK_E_UNSUPPORTED : FLK_OK;
}

flk_status load_chain(const flk_desc* d, int32_t T, const flk_stream* chain, int32_t n_loops,
                      flk::ChainArgs* out) {
  if (!chain) return FLK_E_NULL;
  if (n_loops < 1 || n_loops > FLK_MAX_LOOPS) return FLK_E_SHAPE;
  std::memset(out, 0, sizeof(*out));
  int kept = 0;
  for (int l = 0; l < n_loops; ++l) {
    const flk_stream& s = chain[l];
    if (s.reserved != 0) return FLK_E_DESC;
    if (l == 0 && (s.rows != nullptr || s.n_rows != T)) return FLK_E_SHAPE;   // dense base
    if (s.n_rows < 0 || s.n_rows > T) return FLK_E_SHAPE;
    if (s.n_rows == 0) continue;          // an empty loop: every position inherits
    if (s.rows == nullptr && s.n_rows != T) return FLK_E_SHAPE;
    flk_status st = check_stream_ptrs(s.codes, s.params);
    if (st != FLK_OK) return st;
    if (s.rows && !s.tile_start) return FLK_E_NULL;      // compact loops carry their index
    if (s.rows && (!aligned(s.rows, 4) || !aligned(s.tile_start, 4))) return FLK_E_ALIGN;
    out->s[kept].rows = s.rows;
    out->s[kept].tile_start = s.rows ? s.tile_start : nullptr;
    out->s[kept].codes = s.codes;
    out->s[kept].params = s.params;
    out->s[kept].n = s.n_rows;
    ++kept;
  }
  out->n_loops = kept;
  out->ktile = k_tiles(d) ? 1 : 0;
  return FLK_OK;
}

}  // namespace

extern "C" {

void flk_desc_init(flk_desc* d, int kind, int32_t n_heads, int32_t head_dim) {
  if (!d) return;
  std::memset(d, 0, sizeof(*d));
  d->abi_version = FLK_ABI_VERSION;
  d->format = FLK_FMT_INT4_AFFINE;
  d->kind = uint8_t(kind);
  d->group = FLK_GROUP;
  d->param_dtype = FLK_PARAM_FP16_MIN_SCALE;
  d->nibble_order = FLK_NIBBLE_LOW_EVEN;
  d->n_heads = n_heads;
  d->head_dim = head_dim;
  d->k_grouping = FLK_KGROUP_ROWS;
}

void flk_desc_init_nvfp4(flk_desc* d, int kind, int32_t n_heads, int32_t head_dim) {
  flk_desc_init(d, kind, n_heads, head_dim);
  if (!d) return;
  d->format = FLK_FMT_NVFP4;
  d->group = FLK_FP4_BLOCK;
  d->param_dtype = FLK_PARAM_E4M3_BLOCK_F32_STREAM;
}

void flk_desc_init_mxfp4(flk_desc* d, int kind, int32_t n_heads, int32_t head_dim) {
  flk_desc_init(d, kind, n_heads, head_dim);
  if (!d) return;
  d->format = FLK_FMT_MXFP4;
  d->group = FLK_MX_BLOCK;
  d->param_dtype = FLK_PARAM_E8M0_BLOCK;
}

flk_status flk_desc_check(const flk_desc* d) {
  if (!d) return FLK_E_NULL;
  const bool int4 = d->format == FLK_FMT_INT4_AFFINE && d->group == FLK_GROUP &&
                    d->param_dtype == FLK_PARAM_FP16_MIN_SCALE &&
                    (d->k_grouping == FLK_KGROUP_ROWS || d->k_grouping == FLK_KGROUP_TILE);
  const bool nv = d->format == FLK_FMT_NVFP4 && d->group == FLK_FP4_BLOCK &&
                  d->param_dtype == FLK_PARAM_E4M3_BLOCK_F32_STREAM && d->k_grouping == FLK_KGROUP_ROWS;
  const bool mx = d->format == FLK_FMT_MXFP4 && d->group == FLK_MX_BLOCK && d->param_dtype == FLK_PARAM_E8M0_BLOCK &&
                  d->k_grouping == FLK_KGROUP_ROWS;
  if (d->abi_version != FLK_ABI_VERSION || !(int4 || nv || mx) || (d->kind != FLK_KIND_K && d->kind != FLK_KIND_V) ||
      d->nibble_order != FLK_NIBBLE_LOW_EVEN || d->reserved[0] != 0 || d->reserved[1] != 0 || d->reserved[2] != 0)
    return FLK_E_DESC;
  if (d->n_heads < 1 || d->head_dim < 8 || d->head_dim > FLK_MAX_HEAD_DIM || d->head_dim % 8 != 0)
    return FLK_E_SHAPE;
  if (nv && d->head_dim % FLK_FP4_BLOCK != 0) return FLK_E_SHAPE;
  if (mx && d->head_dim % FLK_MX_BLOCK != 0) return FLK_E_SHAPE;
  if (int64_t(d->n_heads) * d->head_dim > (int64_t(1) << 20)) return FLK_E_SHAPE;
  return FLK_OK;
}

size_t flk_codes_bytes(const flk_desc* d, int32_t n_rows) {
  if (flk_desc_check(d) != FLK_OK || n_rows < 0) return 0;
  return size_t(n_rows) * size_t(d->n_heads) * size_t(d->head_dim) / 2;
}

size_t flk_params_bytes(const flk_desc* d, int32_t n_rows, int32_t T) {
  if (flk_desc_check(d) != FLK_OK || n_rows < 0) return 0;
  if (is_mx(d))                                   // one E8M0 byte per 32 elements
    return size_t(n_rows) * size_t(d->n_heads) * size_t(d->head_dim) / FLK_MX_BLOCK;
  if (is_fp4(d))                                  // header, then one E4M3 byte per 16 elements
    return 16 + size_t(n_rows) * size_t(d->n_heads) * size_t(d->head_dim) / FLK_FP4_BLOCK;
  return 4 * n_groups(d, n_rows, T);
}

size_t flk_rows_bytes(int32_t n_rows, int sparse) {
  if (n_rows < 0) return 0;
  return sparse ? 4 * size_t(n_rows) : 0;
}

size_t flk_tile_index_bytes(int32_t T) {
  if (T < 1) return 0;
  return 4 * (size_t((T + FLK_GROUP - 1) / FLK_GROUP) + 1);
}

size_t flk_stream_bytes(const flk_desc* d, int32_t n_rows, int32_t T, int sparse) {
  if (flk_desc_check(d) != FLK_OK || n_rows < 0 || T < 1 || n_rows > T) return 0;
  return flk_codes_bytes(d, n_rows) + flk_params_bytes(d, n_rows, T) +
         (sparse ? flk_rows_bytes(n_rows, 1) + flk_tile_index_bytes(T) : 0);
}

int32_t flk_rolling_prefix(int32_t n_tokens) {
  if (n_tokens < 2 * FLK_GROUP) return 0;
  return ((n_tokens - FLK_GROUP) / FLK_GROUP) * FLK_GROUP;
}

size_t flk_attn_workspace_bytes(const flk_desc* k_desc, int32_t T, int32_t n_q_heads) {
  if (int4_desc(k_desc) != FLK_OK || T < 0 || n_q_heads < 1) return 0;
  return flk::attn_workspace_bytes(T, k_desc->n_heads, n_q_heads);
}

const char* flk_status_string(flk_status s) {
  switch (s) {
    case FLK_OK: return "ok";
    case FLK_E_NULL: return "required pointer is NULL";
    case FLK_E_SHAPE: return "size out of range";
    case FLK_E_ALIGN: return "pointer misaligned";
    case FLK_E_DESC: return "descriptor not recognised";
    case FLK_E_UNSUPPORTED: return "unsupported request";
    case FLK_E_WORKSPACE: return "workspace missing or too small";
    case FLK_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int flk_abi_version(void) { return FLK_ABI_VERSION; }

flk_status flk_encode_base(const flk_desc* d, const void* x, int32_t T, uint8_t* codes,
                           uint32_t* params, void* recon, uint32_t* dev_status, void* stream) {
  flk_status st = flk_desc_check(d);
  if (st != FLK_OK) return st;
  if (!x || !recon) return FLK_E_NULL;
  if (T < 1 || !rows_fit(d, T)) return FLK_E_SHAPE;
  st = check_stream_ptrs(codes, params);
  if (st != FLK_OK) return st;
  if (!aligned(x, 16) || !aligned(recon, 16) || (dev_status && !aligned(dev_status, 4))) return FLK_E_ALIGN;
  if (is_fp4(d))
    return to_status(flk::launch_fp4_encode(false, is_mx(d), x, nullptr, T, T, d->n_heads, d->head_dim, recon, codes,
                                            params, nullptr, dev_status, static_cast<hipStream_t>(stream)));
  return to_status(flk::launch_encode(d->kind, false,
                                      enc_args(d, x, nullptr, T, T, recon, codes, params, nullptr, dev_status),
                                      d->n_heads, d->head_dim, static_cast<hipStream_t>(stream)));
}

flk_status flk_encode_residual(const flk_desc* d, const void* x_rows, const int32_t* rows,
                               int32_t n_rows, int32_t T, void* recon, uint8_t* codes,
                               uint32_t* params, int32_t* tile_start, uint32_t* dev_status,
                               void* stream) {
  flk_status st = flk_desc_check(d);
  if (st != FLK_OK) return st;
  if (!recon) return FLK_E_NULL;
  if (T < 1 || n_rows < 0 || n_rows > T || !rows_fit(d, T)) return FLK_E_SHAPE;
  if (!aligned(recon, 16) || (dev_status && !aligned(dev_status, 4))) return FLK_E_ALIGN;
  if (n_rows == 0) return FLK_OK;                 // an empty loop: every position inherits
  if (rows == nullptr && n_rows != T) return FLK_E_SHAPE;
  if (!x_rows) return FLK_E_NULL;
  st = check_stream_ptrs(codes, params);
  if (st != FLK_OK) return st;
  if (rows && !tile_start) return FLK_E_NULL;
  if (!aligned(x_rows, 16) || (rows && (!aligned(rows, 4) || !aligned(tile_start, 4))))
    return FLK_E_ALIGN;
  if (is_fp4(d))
    return to_status(flk::launch_fp4_encode(true, is_mx(d), x_rows, rows, n_rows, T, d->n_heads, d->head_dim, recon,
                                            codes, params, rows ? tile_start : nullptr, dev_status,
                                            static_cast<hipStream_t>(stream)));
  return to_status(flk::launch_encode(d->kind, true,
                                      enc_args(d, x_rows, rows, n_rows, T, recon, codes, params, tile_start,
                                               dev_status),
                                      d->n_heads, d->head_dim, static_cast<hipStream_t>(stream)));
}

flk_status flk_reconstruct(const flk_desc* d, int32_t T, const flk_stream* chain, int32_t n_loops,
                           void* out, void* stream) {
  flk_status st = flk_desc_check(d);
  if (st != FLK_OK) return st;
  if (!out) return FLK_E_NULL;
  if (T < 1 || !rows_fit(d, T)) return FLK_E_SHAPE;
  flk::ChainArgs ca;
  st = load_chain(d, T, chain, n_loops, &ca);
  if (st != FLK_OK) return st;
  if (!aligned(out, 16)) return FLK_E_ALIGN;
  if (is_fp4(d))
    return to_status(flk::launch_fp4_reconstruct(ca, true, is_mx(d), d->kind, T, d->n_heads, d->head_dim, out,
                                                 static_cast<hipStream_t>(stream)));
  return to_status(flk::launch_reconstruct(d->kind, T, d->n_heads, d->head_dim, ca, out,
                                           static_cast<hipStream_t>(stream)));
}

flk_status flk_reconstruct_mixed(const flk_desc* bd, const flk_desc* rd, int32_t T, const flk_stream* chain,
                                 int32_t n_loops, void* out, void* stream) {
  flk_status st = flk_desc_check(bd);
  if (st != FLK_OK) return st;
  if ((st = flk_desc_check(rd)) != FLK_OK) return st;
  if (bd->kind != rd->kind || bd->n_heads != rd->n_heads || bd->head_dim != rd->head_dim) return FLK_E_DESC;
  if (!is_fp4(rd)) {
    if (is_fp4(bd)) return FLK_E_UNSUPPORTED;                 // FP4 base, INT4 residuals
    return flk_reconstruct(bd, T, chain, n_loops, out, stream);
  }
  if (is_fp4(bd) && bd->format != rd->format) return FLK_E_UNSUPPORTED;   // NVFP4 with MXFP4
  if (!out) return FLK_E_NULL;
  if (T < 1 || !rows_fit(bd, T)) return FLK_E_SHAPE;
  flk::ChainArgs ca;
  st = load_chain(bd, T, chain, n_loops, &ca);
  if (st != FLK_OK) return st;
  if (!aligned(out, 16)) return FLK_E_ALIGN;
  return to_status(flk::launch_fp4_reconstruct(ca, is_fp4(bd), is_mx(rd), bd->kind, T, bd->n_heads, bd->head_dim, out,
                                               static_cast<hipStream_t>(stream)));
}

namespace {

// The checks flk_decode_attn_packed and flk_decode_attn_packed_noalloc share (all but the
// workspace); on FLK_OK the chains are loaded into kc and vc.
flk_status check_decode_attn(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q, int32_t n_q_heads,
                             const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops, const void* out,
                             flk::ChainArgs* kc, flk::ChainArgs* vc) {
  flk_status st = int4_desc(kd);
  if (st != FLK_OK) return st;
  st = int4_desc(vd);
  if (st != FLK_OK) return st;
  if (kd->kind != FLK_KIND_K || vd->kind != FLK_KIND_V) return FLK_E_DESC;
  if (kd->n_heads != vd->n_heads || kd->head_dim != vd->head_dim) return FLK_E_SHAPE;
  if (!q || !out) return FLK_E_NULL;
  if (T < 1 || !rows_fit(kd, T) || n_q_heads < 1 || n_q_heads % kd->n_heads != 0) return FLK_E_SHAPE;
  if (kd->head_dim != 128 || n_q_heads / kd->n_heads > 16) return FLK_E_UNSUPPORTED;
  st = load_chain(kd, T, k_chain, n_loops, kc);
  if (st != FLK_OK) return st;
  st = load_chain(vd, T, v_chain, n_loops, vc);
  if (st != FLK_OK) return st;
  if (!aligned(q, 16) || !aligned(out, 16)) return FLK_E_ALIGN;
  return FLK_OK;
}

}  // namespace

flk_status flk_decode_attn_packed(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q,
                                  int32_t n_q_heads, const flk_stream* k_chain,
                                  const flk_stream* v_chain, int32_t n_loops, float softmax_scale,
                                  void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  flk::ChainArgs kc, vc;
  const flk_status st = check_decode_attn(kd, vd, T, q, n_q_heads, k_chain, v_chain, n_loops, out, &kc, &vc);
  if (st != FLK_OK) return st;
  // the exact need of this launch (flk_attn_workspace_bytes is a bound on it)
  const size_t need = flk::attn_workspace_need(T, 0, kd->n_heads, n_q_heads);
  if (!workspace || workspace_bytes < need) return FLK_E_WORKSPACE;
  if (!aligned(workspace, 16)) return FLK_E_ALIGN;
  return to_status(flk::launch_decode_attn(T, kd->n_heads, kd->head_dim, n_q_heads, q, kc, vc, nullptr,
                                           nullptr, 0, softmax_scale, out, workspace, workspace_bytes,
                                           static_cast<hipStream_t>(stream)));
}

flk_status flk_decode_attn_packed_noalloc(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q,
                                          int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain,
                                          int32_t n_loops, float softmax_scale, void* out, void* stream) {
  flk::ChainArgs kc, vc;
  const flk_status st = check_decode_attn(kd, vd, T, q, n_q_heads, k_chain, v_chain, n_loops, out, &kc, &vc);
  if (st != FLK_OK) return st;
  if (flk::attn_workspace_need(T, 0, kd->n_heads, n_q_heads) > size_t(FLK_NOALLOC_SCRATCH_BYTES))
    return FLK_E_WORKSPACE;
  return to_status(flk::launch_decode_attn_noalloc(T, kd->n_heads, kd->head_dim, n_q_heads, q, kc, vc,
                                                   softmax_scale, out, static_cast<hipStream_t>(stream)));
}

namespace {

// The readers' format code of a K and a V chain, each described by its base loop's and its
// residual loops' descriptors: INT4 throughout (0), INT4 base + NVFP4 residuals (1), NVFP4
// throughout (2), INT4 base + MXFP4 residuals (3), MXFP4 throughout (4), the same for K and V.
// An FP4 base with INT4 residuals, NVFP4 with MXFP4, and tile-grouped K with FP4 residuals are
// FLK_E_UNSUPPORTED.
flk_status chain_fmt(const flk_desc* kd_base, const flk_desc* kd_resid, const flk_desc* vd_base,
                     const flk_desc* vd_resid, int* fmt) {
  flk_status st;
  for (const flk_desc* d : {kd_base, kd_resid, vd_base, vd_resid})
    if ((st = flk_desc_check(d)) != FLK_OK) return st;
  if (kd_base->kind != FLK_KIND_K || kd_resid->kind != FLK_KIND_K || vd_base->kind != FLK_KIND_V ||
      vd_resid->kind != FLK_KIND_V)
    return FLK_E_DESC;
  for (const flk_desc* d : {kd_resid, vd_base, vd_resid})
    if (d->n_heads != kd_base->n_heads || d->head_dim != kd_base->head_dim) return FLK_E_SHAPE;
  const auto fmt_of = [](const flk_desc* b, const flk_desc* r) {
    if (!is_fp4(r)) return is_fp4(b) ? -1 : 0;
    if (is_fp4(b) && b->format != r->format) return -1;
    return (is_mx(r) ? 3 : 1) + (is_fp4(b) ? 1 : 0);
  };
  const int fk = fmt_of(kd_base, kd_resid), fv = fmt_of(vd_base, vd_resid);
  if (fk < 0 || fk != fv) return FLK_E_UNSUPPORTED;
  if (fk != 0 && kd_base->k_grouping != FLK_KGROUP_ROWS) return FLK_E_UNSUPPORTED;
  *fmt = fk;
  return FLK_OK;
}

}  // namespace

flk_status flk_decode_attn_mixed(const flk_desc* kd_base, const flk_desc* kd_resid, const flk_desc* vd_base,
                                 const flk_desc* vd_resid, int32_t T, const void* q, int32_t n_q_heads,
                                 const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops,
                                 float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  int fk = 0;
  flk_status st = chain_fmt(kd_base, kd_resid, vd_base, vd_resid, &fk);
  if (st != FLK_OK) return st;
  if (fk == 0)
    return flk_decode_attn_packed(kd_base, vd_base, T, q, n_q_heads, k_chain, v_chain, n_loops, softmax_scale, out,
                                  workspace, workspace_bytes, stream);
  if (!q || !out) return FLK_E_NULL;
  if (T < 1 || !rows_fit(kd_base, T) || n_q_heads < 1 || n_q_heads % kd_base->n_heads != 0) return FLK_E_SHAPE;
  if (kd_base->head_dim != 128 || n_q_heads / kd_base->n_heads > 16) return FLK_E_UNSUPPORTED;
  flk::ChainArgs kc, vc;
  if ((st = load_chain(kd_base, T, k_chain, n_loops, &kc)) != FLK_OK) return st;
  if ((st = load_chain(vd_base, T, v_chain, n_loops, &vc)) != FLK_OK) return st;
  if (!aligned(q, 16) || !aligned(out, 16)) return FLK_E_ALIGN;
  const size_t need = flk::attn_workspace_need(T, 0, kd_base->n_heads, n_q_heads);
  if (!workspace || workspace_bytes < need) return FLK_E_WORKSPACE;
  if (!aligned(workspace, 16)) return FLK_E_ALIGN;
  return to_status(flk::launch_decode_attn_fmt(fk, T, kd_base->n_heads, n_q_heads, q, kc, vc, softmax_scale, out,
                                               workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

// ---- sparse decode attention ----------------------------------------------------------------

namespace {

// The shape and pointer checks shared by the sparse calls (those of flk_decode_attn_packed); kd
// and vd describe the chains' base loops and are well formed.
flk_status check_sparse(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q, int32_t n_q_heads,
                        const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops, int32_t k,
                        const void* out, const int32_t* sel, const float* mass, const float* o_ref,
                        const float* c_ref, flk::ChainArgs* kc, flk::ChainArgs* vc) {
  flk_status st;
  if (kd->kind != FLK_KIND_K || vd->kind != FLK_KIND_V) return FLK_E_DESC;
  if (kd->n_heads != vd->n_heads || kd->head_dim != vd->head_dim) return FLK_E_SHAPE;
  if (!q || !out || !sel || !mass || !o_ref || !c_ref) return FLK_E_NULL;
  if (T < 1 || !rows_fit(kd, T) || n_q_heads < 1 || n_q_heads % kd->n_heads != 0) return FLK_E_SHAPE;
  if (int64_t(T) * n_q_heads >= (int64_t(1) << 31)) return FLK_E_SHAPE;   // the scores of one call
  if (k < 1 || k > T) return FLK_E_SHAPE;
  if (kd->head_dim != 128 || n_q_heads / kd->n_heads > 16) return FLK_E_UNSUPPORTED;
  st = load_chain(kd, T, k_chain, n_loops, kc);
  if (st != FLK_OK) return st;
  st = load_chain(vd, T, v_chain, n_loops, vc);
  if (st != FLK_OK) return st;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(sel, 4) || !aligned(mass, 4) || !aligned(o_ref, 16) ||
      !aligned(c_ref, 16))
    return FLK_E_ALIGN;
  return FLK_OK;
}

}  // namespace

size_t flk_sparse_workspace_bytes(const flk_desc* k_desc, int32_t T, int32_t n_q_heads, int32_t k, int32_t n_loops) {
  if (int4_desc(k_desc) != FLK_OK || T < 1 || n_q_heads < 1 || k < 1 || k > T || n_loops < 1 ||
      n_loops > FLK_MAX_LOOPS)
    return 0;
  return flk::sparse_workspace_bytes(T, k_desc->n_heads, n_q_heads, k, n_loops);
}

namespace {

flk_status sparse_reference(int fmt, const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q,
                            int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops,
                            int32_t k, float softmax_scale, void* out, int32_t* sel, float* mass, float* o_ref,
                            float* c_ref, void* workspace, size_t workspace_bytes, void* stream) {
  flk::ChainArgs kc, vc;
  flk_status st = check_sparse(kd, vd, T, q, n_q_heads, k_chain, v_chain, n_loops, k, out, sel, mass, o_ref, c_ref,
                               &kc, &vc);
  if (st != FLK_OK) return st;
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  if (!workspace || workspace_bytes < flk::sparse_workspace_bytes(T, kd->n_heads, n_q_heads, k, nl))
    return FLK_E_WORKSPACE;
  if (!aligned(workspace, 256)) return FLK_E_ALIGN;
  return to_status(flk::launch_sparse_reference(fmt, T, kd->n_heads, n_q_heads, k, q, kc, vc, softmax_scale, out,
                                                sel, mass, o_ref, c_ref, workspace, workspace_bytes,
                                                static_cast<hipStream_t>(stream)));
}

flk_status sparse_loop(int fmt, const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q, int32_t n_q_heads,
                       const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops, int32_t k,
                       float softmax_scale, const int32_t* sel, const float* mass, const float* o_ref,
                       const float* c_ref, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  flk::ChainArgs kc, vc;
  flk_status st = check_sparse(kd, vd, T, q, n_q_heads, k_chain, v_chain, n_loops, k, out, sel, mass, o_ref, c_ref,
                               &kc, &vc);
  if (st != FLK_OK) return st;
  const int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  if (!workspace || workspace_bytes < flk::sparse_workspace_bytes(T, kd->n_heads, n_q_heads, k, nl))
    return FLK_E_WORKSPACE;
  if (!aligned(workspace, 256)) return FLK_E_ALIGN;
  return to_status(flk::launch_sparse_loop(fmt, T, kd->n_heads, n_q_heads, k, q, kc, vc, softmax_scale, sel, mass,
                                           o_ref, c_ref, out, workspace, workspace_bytes,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

flk_status flk_sparse_attn_reference(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q,
                                     int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain,
                                     int32_t n_loops, int32_t k, float softmax_scale, void* out, int32_t* sel,
                                     float* mass, float* o_ref, float* c_ref, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  flk_status st;
  if ((st = int4_desc(kd)) != FLK_OK || (st = int4_desc(vd)) != FLK_OK) return st;
  return sparse_reference(0, kd, vd, T, q, n_q_heads, k_chain, v_chain, n_loops, k, softmax_scale, out, sel, mass,
                          o_ref, c_ref, workspace, workspace_bytes, stream);
}

flk_status flk_sparse_attn_loop(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q, int32_t n_q_heads,
                                const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops, int32_t k,
                                float softmax_scale, const int32_t* sel, const float* mass, const float* o_ref,
                                const float* c_ref, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  flk_status st;
  if ((st = int4_desc(kd)) != FLK_OK || (st = int4_desc(vd)) != FLK_OK) return st;
  return sparse_loop(0, kd, vd, T, q, n_q_heads, k_chain, v_chain, n_loops, k, softmax_scale, sel, mass, o_ref, c_ref,
                     out, workspace, workspace_bytes, stream);
}

flk_status flk_sparse_attn_reference_mixed(const flk_desc* kd_base, const flk_desc* kd_resid,
                                           const flk_desc* vd_base, const flk_desc* vd_resid, int32_t T,
                                           const void* q, int32_t n_q_heads, const flk_stream* k_chain,
                                           const flk_stream* v_chain, int32_t n_loops, int32_t k,
                                           float softmax_scale, void* out, int32_t* sel, float* mass, float* o_ref,
                                           float* c_ref, void* workspace, size_t workspace_bytes, void* stream) {
  int fmt = 0;
  flk_status st = chain_fmt(kd_base, kd_resid, vd_base, vd_resid, &fmt);
  if (st != FLK_OK) return st;
  return sparse_reference(fmt, kd_base, vd_base, T, q, n_q_heads, k_chain, v_chain, n_loops, k, softmax_scale, out,
                          sel, mass, o_ref, c_ref, workspace, workspace_bytes, stream);
}

flk_status flk_sparse_attn_loop_mixed(const flk_desc* kd_base, const flk_desc* kd_resid, const flk_desc* vd_base,
                                      const flk_desc* vd_resid, int32_t T, const void* q, int32_t n_q_heads,
                                      const flk_stream* k_chain, const flk_stream* v_chain, int32_t n_loops,
                                      int32_t k, float softmax_scale, const int32_t* sel, const float* mass,
                                      const float* o_ref, const float* c_ref, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  int fmt = 0;
  flk_status st = chain_fmt(kd_base, kd_resid, vd_base, vd_resid, &fmt);
  if (st != FLK_OK) return st;
  return sparse_loop(fmt, kd_base, vd_base, T, q, n_q_heads, k_chain, v_chain, n_loops, k, softmax_scale, sel, mass,
                     o_ref, c_ref, out, workspace, workspace_bytes, stream);
}

// ---- token selection and row partition -----------------------------------------------------

int32_t flk_select_count(int32_t T, int32_t window, const int32_t* pct, int32_t n_budgets) {
  if (T < 0 || window < 1 || n_budgets < 0 || (n_budgets > 0 && !pct)) return -1;
  for (int32_t i = 0; i < n_budgets; ++i)
    if (pct[i] < 0 || pct[i] > 100) return -1;
  int64_t total = 0;
  for (int64_t w0 = 0; w0 < T; w0 += window) {
    const int64_t len = std::min<int64_t>(window, T - w0);
    int64_t n = len;
    for (int32_t i = 0; i < n_budgets; ++i) n = std::min<int64_t>(n, (int64_t(pct[i]) * len + 99) / 100);
    total += n;
  }
  return int32_t(total);
}

size_t flk_select_workspace_bytes(int32_t T, int32_t window) {
  if (T < 1 || window < 1) return 0;
  return flk::select_workspace_bytes(T, window);
}

flk_status flk_select_rows(const void* h_prev, const void* h_prev2, int32_t T, int32_t d, const int32_t* rows_prev,
                           int32_t n_prev, int32_t window, int32_t pct, float eps, float* scores,
                           int32_t* rows_out, int32_t n_out, int32_t* slot, void* workspace,
                           size_t workspace_bytes, uint32_t* dev_status, void* stream) {
  if (!h_prev || !h_prev2 || (n_out > 0 && !rows_out)) return FLK_E_NULL;
  if (T < 1 || d < 8 || d % 8 != 0 || d > 16384 || int64_t(T) * d >= (int64_t(1) << 31)) return FLK_E_SHAPE;
  if (n_prev < 0 || n_prev > T || (!rows_prev && n_prev != T && n_prev != 0)) return FLK_E_SHAPE;
  if (window < 1 || pct < 0 || pct > 100 || n_out < 0 || n_out > n_prev) return FLK_E_SHAPE;
  if (!(eps > 0.0f) || !(eps <= 3.4028234663852886e38f)) return FLK_E_SHAPE;
  if (h_prev == h_prev2) return FLK_E_SHAPE;
  if (pct > 0 && pct < 100 && n_prev > 0 && !scores) return FLK_E_NULL;
  if (!aligned(h_prev, 16) || !aligned(h_prev2, 16) || (rows_prev && !aligned(rows_prev, 4)) ||
      (scores && !aligned(scores, 4)) || !aligned(rows_out, 4) || (slot && !aligned(slot, 4)) ||
      (dev_status && !aligned(dev_status, 4)))
    return FLK_E_ALIGN;
  if (!workspace || workspace_bytes < flk::select_workspace_bytes(T, window)) return FLK_E_WORKSPACE;
  if (!aligned(workspace, 4)) return FLK_E_ALIGN;
  // An empty previous set: the kernels see a list of zero positions, which they never read.
  if (n_prev == 0) rows_prev = static_cast<const int32_t*>(workspace);
  return to_status(flk::launch_select_rows(h_prev, h_prev2, T, d, rows_prev, n_prev, window, pct, eps, scores,
                                           rows_out, n_out, slot, workspace, workspace_bytes, dev_status,
                                           static_cast<hipStream_t>(stream)));
}

flk_status flk_partition_rows(const uint8_t* cls, int32_t n, int32_t* gather, int32_t* scatter, int32_t* counts,
                              uint32_t* dev_status, void* stream) {
  if (!counts || (n > 0 && (!cls || !gather || !scatter))) return FLK_E_NULL;
  if (n < 0) return FLK_E_SHAPE;
  if ((gather && !aligned(gather, 4)) || (scatter && !aligned(scatter, 4)) || !aligned(counts, 4) ||
      (dev_status && !aligned(dev_status, 4)))
    return FLK_E_ALIGN;
  return to_status(flk::launch_partition_rows(cls, n, gather, scatter, counts, dev_status,
                                              static_cast<hipStream_t>(stream)));
}

// ---- appending whole tiles (rolling-tail flush) --------------------------------------------

namespace {

// The checks of flk_append_base / flk_append_residual for one window.  On FLK_OK, *a is the
// window's encode (pointers offset into the streams) or, when *empty is set, an empty compact
// window whose tile index entries (and zero K tile params) still have to be written.
flk_status check_append(const flk_desc* d, bool resid, const flk_append_unit& u, flk::EncArgs* a, bool* empty) {
  *empty = false;
  if (u.reserved != 0) return FLK_E_DESC;
  if (!u.recon) return FLK_E_NULL;
  if (u.p0 < 0 || u.n_pos < FLK_GROUP || u.p0 % FLK_GROUP != 0 || u.n_pos % FLK_GROUP != 0) return FLK_E_SHAPE;
  if (!rows_fit(d, int64_t(u.p0) + u.n_pos)) return FLK_E_SHAPE;
  if (u.n_rows < 0 || u.n_rows > u.n_pos || u.rows_before < 0 || u.rows_before > u.p0) return FLK_E_SHAPE;
  const bool dense = u.rows == nullptr && u.n_rows > 0;
  if (!resid && !dense) return FLK_E_SHAPE;                       // loop 1 covers every position
  if (dense && (u.n_rows != u.n_pos || u.rows_before != u.p0)) return FLK_E_SHAPE;
  if (!dense && d->kind == FLK_KIND_K && !k_tiles(d)) return FLK_E_UNSUPPORTED;
  if (u.n_rows > 0 && !u.x) return FLK_E_NULL;
  if (!dense && !u.tile_start) return FLK_E_NULL;
  if (u.n_rows > 0 || k_tiles(d)) {
    const flk_status st = check_stream_ptrs(u.codes, u.params);
    if (st != FLK_OK) return st;
  }
  if (!aligned(u.recon, 16) || (u.x && !aligned(u.x, 16)) || (u.rows && !aligned(u.rows, 4)) ||
      (u.tile_start && !aligned(u.tile_start, 4)))
    return FLK_E_ALIGN;
  // an empty V window may come without stream buffers: no offset is added to a NULL pointer
  *a = enc_args(d, u.x, u.rows, u.n_rows, u.n_pos, u.recon,
                u.codes ? u.codes + codes_offset(d, u.rows_before) : nullptr,
                u.params ? u.params + params_offset(d, u.rows_before, u.p0) : nullptr, nullptr, nullptr);
  // a compact window writes its tile index entries, also when it has no rows (and so may come
  // with rows == NULL): enc_args keeps the index only for a non-NULL rows pointer
  a->tile_start = dense ? nullptr : u.tile_start + u.p0 / FLK_GROUP;
  a->pos0 = u.rows ? u.p0 : 0;
  a->row0 = u.rows_before;
  *empty = u.n_rows == 0;
  return FLK_OK;
}

// An empty compact window: tile_start[p0/64 .. (p0+n_pos)/64] = rows_before, and zero params
// for the window's tiles of a tile-grouped K stream.
hipError_t fill_empty_window(const flk_desc* d, const flk::EncArgs& a, hipStream_t s) {
  if (!a.tile_start || (k_tiles(d) && !a.params)) return hipErrorInvalidValue;   // V writes no params
  const int32_t nt = a.T / FLK_GROUP;
  hipError_t e = flk::launch_fill_u32(reinterpret_cast<uint32_t*>(a.tile_start), nt + 1, uint32_t(a.row0), s);
  if (e == hipSuccess && k_tiles(d)) e = flk::launch_fill_u32(a.params, int64_t(nt) * a.W, 0u, s);
  return e;
}

}  // namespace

flk_status flk_append_base(const flk_desc* d, const void* x, int32_t p0, int32_t n_pos, uint8_t* codes,
                           uint32_t* params, void* recon, uint32_t* dev_status, void* stream) {
  flk_status st = int4_desc(d);
  if (st != FLK_OK) return st;
  if (!x) return FLK_E_NULL;
  if (dev_status && !aligned(dev_status, 4)) return FLK_E_ALIGN;
  const flk_append_unit u{x, nullptr, recon, codes, params, nullptr, n_pos, p0, n_pos, p0, d->kind, 0};
  flk::EncArgs a;
  bool empty;
  st = check_append(d, false, u, &a, &empty);
  if (st != FLK_OK) return st;
  a.status = dev_status;
  return to_status(flk::launch_encode(d->kind, false, a, d->n_heads, d->head_dim, static_cast<hipStream_t>(stream)));
}

flk_status flk_append_residual(const flk_desc* d, const void* x_rows, const int32_t* rows, int32_t n_rows,
                               int32_t p0, int32_t n_pos, int32_t rows_before, void* recon, uint8_t* codes,
                               uint32_t* params, int32_t* tile_start, uint32_t* dev_status, void* stream) {
  flk_status st = int4_desc(d);
  if (st != FLK_OK) return st;
  if (dev_status && !aligned(dev_status, 4)) return FLK_E_ALIGN;
  const flk_append_unit u{x_rows, rows, recon, codes, params, tile_start, n_rows, p0, n_pos, rows_before, d->kind, 0};
  flk::EncArgs a;
  bool empty;
  st = check_append(d, true, u, &a, &empty);
  if (st != FLK_OK) return st;
  a.status = dev_status;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (empty) return to_status(fill_empty_window(d, a, s));
  return to_status(flk::launch_encode(d->kind, true, a, d->n_heads, d->head_dim, s));
}

flk_status flk_decode_attn_rolling(const flk_desc* kd, const flk_desc* vd, int32_t T, const void* q,
                                   int32_t n_q_heads, const flk_stream* k_chain, const flk_stream* v_chain,
                                   int32_t n_loops, const void* k_tail, const void* v_tail, int32_t tail_len,
                                   float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  flk_status st = int4_desc(kd);
  if (st != FLK_OK) return st;
  st = int4_desc(vd);
  if (st != FLK_OK) return st;
  if (kd->kind != FLK_KIND_K || vd->kind != FLK_KIND_V) return FLK_E_DESC;
  if (kd->n_heads != vd->n_heads || kd->head_dim != vd->head_dim) return FLK_E_SHAPE;
  if (!q || !out) return FLK_E_NULL;
  if (T < 0 || tail_len < 0 || int64_t(T) + tail_len < 1 || !rows_fit(kd, T) || !rows_fit(kd, tail_len) ||
      n_q_heads < 1 || n_q_heads % kd->n_heads != 0)
    return FLK_E_SHAPE;
  if (kd->head_dim != 128 || n_q_heads / kd->n_heads > 16) return FLK_E_UNSUPPORTED;
  if (tail_len > 0 && (!k_tail || !v_tail)) return FLK_E_NULL;
  flk::ChainArgs kc{}, vc{};
  if (T > 0) {
    st = load_chain(kd, T, k_chain, n_loops, &kc);
    if (st != FLK_OK) return st;
    st = load_chain(vd, T, v_chain, n_loops, &vc);
    if (st != FLK_OK) return st;
  }
  if (!aligned(q, 16) || !aligned(out, 16) || (tail_len > 0 && (!aligned(k_tail, 16) || !aligned(v_tail, 16))))
    return FLK_E_ALIGN;
  // the exact need of this launch (flk_attn_workspace_bytes is a bound on it)
  const size_t need = flk::attn_workspace_need(T, tail_len, kd->n_heads, n_q_heads);
  if (!workspace || workspace_bytes < need) return FLK_E_WORKSPACE;
  if (!aligned(workspace, 16)) return FLK_E_ALIGN;
  return to_status(flk::launch_decode_attn(T, kd->n_heads, kd->head_dim, n_q_heads, q, kc, vc, k_tail, v_tail,
                                           tail_len, softmax_scale, out, workspace, workspace_bytes,
                                           static_cast<hipStream_t>(stream)));
}

namespace {

const flk_desc* unit_desc(const flk_desc* kd, const flk_desc* vd, int32_t kind) {
  return kind == FLK_KIND_K ? kd : kind == FLK_KIND_V ? vd : nullptr;
}

flk_status check_pair(const flk_desc* kd, const flk_desc* vd) {
  if (kd) {
    const flk_status st = int4_desc(kd);
    if (st != FLK_OK) return st;
    if (kd->kind != FLK_KIND_K) return FLK_E_DESC;
  }
  if (vd) {
    const flk_status st = int4_desc(vd);
    if (st != FLK_OK) return st;
    if (vd->kind != FLK_KIND_V) return FLK_E_DESC;
  }
  return FLK_OK;
}

// The checks of flk_encode_base / flk_encode_residual for one unit; *skip marks an empty loop.
flk_status check_encode_unit(const flk_desc* d, bool resid, const flk_unit& u, flk::EncArgs* a, bool* skip) {
  *skip = false;
  if (u.reserved != 0) return FLK_E_DESC;
  if (!u.recon) return FLK_E_NULL;
  if (u.T < 1 || u.n_rows < 0 || u.n_rows > u.T || !rows_fit(d, u.T)) return FLK_E_SHAPE;
  if (!aligned(u.recon, 16)) return FLK_E_ALIGN;
  if (!resid && (u.rows != nullptr || u.n_rows != u.T)) return FLK_E_SHAPE;
  if (u.n_rows == 0) {
    *skip = true;
    return FLK_OK;
  }
  if (u.rows == nullptr && u.n_rows != u.T) return FLK_E_SHAPE;
  if (!u.x) return FLK_E_NULL;
  const flk_status st = check_stream_ptrs(u.codes, u.params);
  if (st != FLK_OK) return st;
  if (u.rows && !u.tile_start) return FLK_E_NULL;
  if (!aligned(u.x, 16) || (u.rows && (!aligned(u.rows, 4) || !aligned(u.tile_start, 4)))) return FLK_E_ALIGN;
  *a = enc_args(d, u.x, u.rows, u.n_rows, u.T, u.recon, u.codes, u.params, u.tile_start, nullptr);
  return FLK_OK;
}

flk_status encode_batch(bool resid, const flk_desc* kd, const flk_desc* vd, const flk_unit* units, int32_t n_units,
                        uint32_t* dev_status, void* stream) {
  if (n_units < 0) return FLK_E_SHAPE;
  if (n_units == 0) return FLK_OK;
  if (!units) return FLK_E_NULL;
  flk_status st = check_pair(kd, vd);
  if (st != FLK_OK) return st;
  if (dev_status && !aligned(dev_status, 4)) return FLK_E_ALIGN;
  std::vector<flk::EncArgs> batch[2];       // [0] dense (or base), [1] compact
  std::vector<int> kinds[2];
  std::vector<std::pair<int, flk::EncArgs>> singles;
  for (int32_t i = 0; i < n_units; ++i) {
    const flk_unit& u = units[i];
    const flk_desc* d = unit_desc(kd, vd, u.kind);
    if (u.kind != FLK_KIND_K && u.kind != FLK_KIND_V) return FLK_E_DESC;
    if (!d) return FLK_E_NULL;
    flk::EncArgs a;
    bool skip;
    st = check_encode_unit(d, resid, u, &a, &skip);
    if (st != FLK_OK) return st;
    if (skip) continue;
    a.status = dev_status;
    if (flk::encode_batchable(u.kind, d->n_heads, d->head_dim)) {
      batch[u.rows ? 1 : 0].push_back(a);
      kinds[u.rows ? 1 : 0].push_back(u.kind);
    } else {
      singles.emplace_back(i, a);
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int g = 0; g < 2; ++g) {
    if (batch[g].empty()) continue;
    const hipError_t e = flk::launch_encode_batch(resid, g == 1, batch[g].data(), kinds[g].data(),
                                                  int(batch[g].size()), s);
    if (e != hipSuccess) return FLK_E_LAUNCH;
  }
  for (const auto& [i, a] : singles) {
    const flk_desc* d = unit_desc(kd, vd, units[i].kind);
    const hipError_t e = flk::launch_encode(units[i].kind, resid, a, d->n_heads, d->head_dim, s);
    if (e != hipSuccess) return FLK_E_LAUNCH;
  }
  return FLK_OK;
}

uint32_t pattern_key(const flk::ChainArgs& c) {
  uint32_t m = uint32_t(c.n_loops) << 16;
  for (int l = 0; l < c.n_loops; ++l) m |= (c.s[l].rows ? 1u : 0u) << l;
  return m;
}

}  // namespace

flk_status flk_encode_base_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_unit* units,
                                 int32_t n_units, uint32_t* dev_status, void* stream) {
  return encode_batch(false, k_desc, v_desc, units, n_units, dev_status, stream);
}

flk_status flk_encode_residual_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_unit* units,
                                     int32_t n_units, uint32_t* dev_status, void* stream) {
  return encode_batch(true, k_desc, v_desc, units, n_units, dev_status, stream);
}

namespace {

flk_status append_batch(bool resid, const flk_desc* kd, const flk_desc* vd, const flk_append_unit* units,
                        int32_t n_units, uint32_t* dev_status, void* stream) {
  if (n_units < 0) return FLK_E_SHAPE;
  if (n_units == 0) return FLK_OK;
  if (!units) return FLK_E_NULL;
  flk_status st = check_pair(kd, vd);
  if (st != FLK_OK) return st;
  if (dev_status && !aligned(dev_status, 4)) return FLK_E_ALIGN;
  std::vector<flk::EncArgs> batch[2];       // [0] dense (or loop 1), [1] compact
  std::vector<int> kinds[2];
  std::vector<std::pair<int, flk::EncArgs>> singles, empties;
  for (int32_t i = 0; i < n_units; ++i) {
    const flk_append_unit& u = units[i];
    if (u.kind != FLK_KIND_K && u.kind != FLK_KIND_V) return FLK_E_DESC;
    const flk_desc* d = unit_desc(kd, vd, u.kind);
    if (!d) return FLK_E_NULL;
    flk::EncArgs a;
    bool empty;
    st = check_append(d, resid, u, &a, &empty);
    if (st != FLK_OK) return st;
    a.status = dev_status;
    if (empty) {
      empties.emplace_back(i, a);
    } else if (flk::encode_batchable(u.kind, d->n_heads, d->head_dim)) {
      batch[u.rows ? 1 : 0].push_back(a);
      kinds[u.rows ? 1 : 0].push_back(u.kind);
    } else {
      singles.emplace_back(i, a);
    }
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int g = 0; g < 2; ++g) {
    if (batch[g].empty()) continue;
    if (flk::launch_encode_batch(resid, g == 1, batch[g].data(), kinds[g].data(), int(batch[g].size()), s) !=
        hipSuccess)
      return FLK_E_LAUNCH;
  }
  for (const auto& [i, a] : singles) {
    const flk_desc* d = unit_desc(kd, vd, units[i].kind);
    if (flk::launch_encode(units[i].kind, resid, a, d->n_heads, d->head_dim, s) != hipSuccess) return FLK_E_LAUNCH;
  }
  for (const auto& [i, a] : empties)
    if (fill_empty_window(unit_desc(kd, vd, units[i].kind), a, s) != hipSuccess) return FLK_E_LAUNCH;
  return FLK_OK;
}

}  // namespace

flk_status flk_append_base_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_append_unit* units,
                                 int32_t n_units, uint32_t* dev_status, void* stream) {
  return append_batch(false, k_desc, v_desc, units, n_units, dev_status, stream);
}

flk_status flk_append_residual_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_append_unit* units,
                                     int32_t n_units, uint32_t* dev_status, void* stream) {
  return append_batch(true, k_desc, v_desc, units, n_units, dev_status, stream);
}

flk_status flk_reconstruct_batch(const flk_desc* k_desc, const flk_desc* v_desc, const flk_recon_unit* units,
                                 int32_t n_units, void* stream) {
  if (n_units < 0) return FLK_E_SHAPE;
  if (n_units == 0) return FLK_OK;
  if (!units) return FLK_E_NULL;
  flk_status st = check_pair(k_desc, v_desc);
  if (st != FLK_OK) return st;
  std::vector<flk::RecArgs> batch;
  std::vector<flk::RecArgs> singles;
  for (int32_t i = 0; i < n_units; ++i) {
    const flk_recon_unit& u = units[i];
    if (u.kind != FLK_KIND_K && u.kind != FLK_KIND_V) return FLK_E_DESC;
    if (u.reserved != 0) return FLK_E_DESC;
    const flk_desc* d = unit_desc(k_desc, v_desc, u.kind);
    if (!d) return FLK_E_NULL;
    if (!u.out) return FLK_E_NULL;
    if (u.T < 1 || !rows_fit(d, u.T)) return FLK_E_SHAPE;
    flk::RecArgs a;
    st = load_chain(d, u.T, u.chain, u.n_loops, &a.chain);
    if (st != FLK_OK) return st;
    if (!aligned(u.out, 16)) return FLK_E_ALIGN;
    a.out = u.out;
    a.T = u.T;
    a.H = d->n_heads;
    a.D = d->head_dim;
    a.kind = u.kind;
    (flk::reconstruct_batchable(a.H, a.D) ? batch : singles).push_back(a);
  }
  // units with the same loop count and compact pattern share launches
  std::stable_sort(batch.begin(), batch.end(), [](const flk::RecArgs& a, const flk::RecArgs& b) {
    return pattern_key(a.chain) < pattern_key(b.chain);
  });
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!batch.empty() && flk::launch_reconstruct_batch(batch.data(), int(batch.size()), s) != hipSuccess)
    return FLK_E_LAUNCH;
  for (const auto& a : singles)
    if (flk::launch_reconstruct(a.kind, a.T, a.H, a.D, a.chain, a.out, s) != hipSuccess) return FLK_E_LAUNCH;
  return FLK_OK;
}

}  // extern "C"
