// C ABI of liblynx: argument validation, parameter blocks and kernel launches.
// Every argument error is detected here, on the host, before any launch.  The
// library allocates no device memory; the only state kept between calls is the
// per-GPU address of the no-allocation attention's buffer (lynx_attn.hip).
//
// Sources, cited by page title and section:
//   [Review] "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
//            LLM Inference" (technical review of arXiv 2607.01831).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/lynx.h"
#include "lynx_common.hpp"
#include "lynx_kernels.hpp"

using namespace lynx;

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }


bool pow2_chunk(int c) { return c == 8 || c == 16 || c == 32 || c == 64 || c == 128 || c == 256; }

// Shared validation of the page geometry; fills `g` on success.
int check_geometry(int n_pages, int P, int Hkv, int D, int C, float alpha, Geometry* g) {
  if (n_pages < 0 || P <= 0 || Hkv <= 0 || D <= 0 || C <= 0) return LYNX_EINVAL;
  if (P % C != 0) return LYNX_EINVAL;
  if (!std::isfinite(alpha) || !(alpha > 0.0f)) return LYNX_EINVAL;
  if (D != kHeadDim) return LYNX_EUNSUPPORTED;
  if (!pow2_chunk(C)) return LYNX_EUNSUPPORTED;
  if ((long long)P * Hkv * kHeadDim / 2 > 0x7fffffffll) return LYNX_EUNSUPPORTED;   // page byte counts in int
  if ((long long)n_pages * Hkv * ((P + kDecTile - 1) / kDecTile) > 0x7fffffffll ||
      (long long)n_pages * Hkv * (kHeadDim / kSlab) * ((P + kTileTokens - 1) / kTileTokens) > 0x7fffffffll)
    return LYNX_EUNSUPPORTED;
  g->n_pages = n_pages;
  g->P = P;
  g->Hkv = Hkv;
  g->C = C;
  g->nck = P / C;
  g->H = Hkv * D;
  g->codes = (long long)P * g->H / 2;
  g->res_seg = g->codes;
  g->anc_seg = g->codes + 4ll * g->H * (2 + 2ll * (P / C));
  return LYNX_OK;
}

// |x_hat| = ((1+alpha)^(I/127) - 1)/alpha  ([Review] Mechanism 1, Stage 3, Eq. 8 as
// normalised in the Worked Example, Eq. 14-15).
double alaw_mag(int I, double alpha) { return std::expm1((double)I / kCodeMax * std::log1p(alpha)) / alpha; }

// Signed anchor value of a nibble: Q_anc = nibble as 4-bit two's complement;
// S = -1 iff Q_anc < 0; V_mag = Q_anc or -Q_anc - 1 (Eq. 9 inverted).
void anchor_fields(int nib, int* S, int* vmag) {
  const int q = nib >= 8 ? nib - 16 : nib;
  *S = q < 0 ? -1 : 1;
  *vmag = q < 0 ? -q - 1 : q;
}

// The encoder for chunk C: pages of one tile take Stage 1 in the same kernel, longer
// pages read the gamma stored by the two Stage 1 kernels.
template <int C>
const void* encode_kernel(bool page_stored) {
  return page_stored ? reinterpret_cast<const void*>(&k_encode<C, true>)
                     : reinterpret_cast<const void*>(&k_encode<C, false>);
}

int launch(const void* fn, dim3 grid, void* args_struct, hipStream_t stream) {
  void* kargs[] = {args_struct};
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(kThreads), kargs, 0, stream);
  return e == hipSuccess ? LYNX_OK : LYNX_ELAUNCH;
}

}  // namespace

extern "C" {

const char* lynx_strerror(int status) {
  switch (status) {
    case LYNX_OK: return "ok";
    case LYNX_EINVAL: return "invalid argument (size, count, chunk, alpha, selector or dtype)";
    case LYNX_EALIGN: return "null or misaligned pointer (16-byte for data, 4-byte for index tables)";
    case LYNX_EUNSUPPORTED: return "shape not supported by this library";
    case LYNX_ENOSPACE: return "workspace too small";
    case LYNX_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int lynx_stream_sizes(int page_tokens, int kv_heads, int head_dim, int chunk, size_t* anchor_seg_bytes,
                      size_t* residual_seg_bytes) {
  if (page_tokens <= 0 || kv_heads <= 0 || head_dim <= 0 || chunk <= 0) return LYNX_EINVAL;
  if (page_tokens % chunk != 0) return LYNX_EINVAL;
  const long long H = (long long)kv_heads * head_dim;
  if ((page_tokens * H) % 2 != 0) return LYNX_EINVAL;
  const long long codes = page_tokens * H / 2;
  if (anchor_seg_bytes) *anchor_seg_bytes = (size_t)(codes + 4ll * H * (2 + 2ll * (page_tokens / chunk)));
  if (residual_seg_bytes) *residual_seg_bytes = (size_t)codes;
  return LYNX_OK;
}

int lynx_encode(const void* kv_dev, int n_pages, int page_tokens, int kv_heads, int head_dim, int chunk,
                float alpha, unsigned sel, void* anchor_dev, void* residual_dev, void* hip_stream) {
  EncodeArgs a;
  std::memset(&a, 0, sizeof(a));
  int st = check_geometry(n_pages, page_tokens, kv_heads, head_dim, chunk, alpha, &a.g);
  if (st != LYNX_OK) return st;
  if ((sel & ~(LYNX_SEL_ANCHOR | LYNX_SEL_RESIDUAL)) != 0 || !(sel & LYNX_SEL_ANCHOR)) return LYNX_EINVAL;
  if (n_pages == 0) return LYNX_OK;
  if (!aligned16(kv_dev) || !aligned16(anchor_dev)) return LYNX_EALIGN;
  if ((sel & LYNX_SEL_RESIDUAL) && !aligned16(residual_dev)) return LYNX_EALIGN;
  a.kv = static_cast<const uint16_t*>(kv_dev);
  a.anchor = static_cast<uint8_t*>(anchor_dev);
  a.residual = (sel & LYNX_SEL_RESIDUAL) ? static_cast<uint8_t*>(residual_dev) : nullptr;
  a.alpha = alpha;
  const double al = (double)alpha, L = std::log1p(al);
  a.ylog2k = (float)((double)kCodeMax / std::log2(1.0 + al));
  // Band half-width around a rounding boundary of Y inside which the float32
  // estimate is not trusted and the element is decided in float64: 7 units of 2^-16
  // (1.07e-4).  The float32 evaluation's error stays below 3.1e-5 (bound derived in
  // the design notes), so the margin is 3.4x.
  a.zband = 7;
  a.bnd[0] = 0.0;
  for (int j = 1; j <= kCodeMax; ++j) a.bnd[j] = std::expm1(((double)j - 0.5) * L / kCodeMax) / al;
  a.bnd[128] = INFINITY;
  // one workgroup per (page, head, 64-channel slab, 256-token tile)
  const long long ntiles = (page_tokens + kTileTokens - 1) / kTileTokens;
  const long long n_wg = (long long)n_pages * kv_heads * (kHeadDim / kSlab) * ntiles;
  const bool stored = ntiles > 1;
  const void* fn = nullptr;
  switch (chunk) {
    case 8: fn = encode_kernel<8>(stored); break;
    case 16: fn = encode_kernel<16>(stored); break;
    case 32: fn = encode_kernel<32>(stored); break;
    case 64: fn = encode_kernel<64>(stored); break;
    case 128: fn = encode_kernel<128>(stored); break;
    default: fn = encode_kernel<256>(stored); break;
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (ntiles > 1) {
    // Stage 1 of a page longer than one tile: per-tile extremes, then gamma per (page, channel)
    st = launch(reinterpret_cast<const void*>(&k_page_extremes), dim3((unsigned)n_wg), &a, stream);
    if (st != LYNX_OK) return st;
    const long long n_ch = (long long)n_pages * a.g.H;
    st = launch(reinterpret_cast<const void*>(&k_page_finish), dim3((unsigned)((n_ch + kThreads - 1) / kThreads)), &a,
                stream);
    if (st != LYNX_OK) return st;
  }
  return launch(fn, dim3((unsigned)n_wg), &a, stream);
}

size_t lynx_encode_to_host_staging_bytes(int group_pages, int page_tokens, int kv_heads, int head_dim, int chunk) {
  Geometry g;
  if (group_pages <= 0 || check_geometry(group_pages, page_tokens, kv_heads, head_dim, chunk, 1.0f, &g) != LYNX_OK)
    return 0;
  return 2 * (size_t)group_pages * (size_t)(g.anc_seg + g.res_seg);
}

int lynx_encode_to_host(const void* kv_dev, int n_pages, int page_tokens, int kv_heads, int head_dim, int chunk,
                        float alpha, int group_pages, void* staging_dev, size_t staging_bytes, void* anchor_host,
                        void* residual_host, void* compute_stream, void* copy_stream) {
  Geometry g;
  int st = check_geometry(n_pages, page_tokens, kv_heads, head_dim, chunk, alpha, &g);
  if (st != LYNX_OK) return st;
  if (group_pages <= 0) return LYNX_EINVAL;
  if (n_pages == 0) return LYNX_OK;
  if (anchor_host == nullptr || residual_host == nullptr) return LYNX_EINVAL;
  if (!aligned16(kv_dev) || !aligned16(staging_dev)) return LYNX_EALIGN;
  const int gp = group_pages < n_pages ? group_pages : n_pages;
  const size_t a_sz = (size_t)g.anc_seg, r_sz = (size_t)g.res_seg;
  if (staging_bytes < 2 * (size_t)gp * (a_sz + r_sz)) return LYNX_ENOSPACE;
  hipStream_t cs = static_cast<hipStream_t>(compute_stream), xs = static_cast<hipStream_t>(copy_stream);
  // enc[b]: group in staging buffer b encoded; cpy[b]: its copies done, buffer b free again
  hipEvent_t enc[2] = {nullptr, nullptr}, cpy[2] = {nullptr, nullptr};
  int rc = LYNX_OK;
  for (int b = 0; b < 2 && rc == LYNX_OK; ++b)
    if (hipEventCreateWithFlags(&enc[b], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&cpy[b], hipEventDisableTiming) != hipSuccess)
      rc = LYNX_ELAUNCH;
  // copies still queued on copy_stream (an earlier call's) may read the staging buffers:
  // the first encodes wait for them
  for (int b = 0; b < 2 && rc == LYNX_OK; ++b)
    if (hipEventRecord(cpy[b], xs) != hipSuccess) rc = LYNX_ELAUNCH;
  const size_t kv_page_elems = (size_t)page_tokens * g.H;
  uint8_t* stage = static_cast<uint8_t*>(staging_dev);
  for (int g0 = 0, grp = 0; g0 < n_pages && rc == LYNX_OK; g0 += gp, ++grp) {
    const int n = n_pages - g0 < gp ? n_pages - g0 : gp;
    const int b = grp & 1;
    uint8_t* anc = stage + (size_t)b * gp * (a_sz + r_sz);
    uint8_t* res = anc + (size_t)gp * a_sz;
    if (hipStreamWaitEvent(cs, cpy[b], 0) != hipSuccess) { rc = LYNX_ELAUNCH; break; }
    rc = lynx_encode(static_cast<const uint16_t*>(kv_dev) + (size_t)g0 * kv_page_elems, n, page_tokens, kv_heads,
                     head_dim, chunk, alpha, LYNX_SEL_ANCHOR | LYNX_SEL_RESIDUAL, anc, res, cs);
    if (rc != LYNX_OK) break;
    // the anchor segments leave first, then the residual ones
    if (hipEventRecord(enc[b], cs) != hipSuccess || hipStreamWaitEvent(xs, enc[b], 0) != hipSuccess ||
        hipMemcpyAsync(static_cast<uint8_t*>(anchor_host) + (size_t)g0 * a_sz, anc, (size_t)n * a_sz,
                       hipMemcpyDeviceToHost, xs) != hipSuccess ||
        hipMemcpyAsync(static_cast<uint8_t*>(residual_host) + (size_t)g0 * r_sz, res, (size_t)n * r_sz,
                       hipMemcpyDeviceToHost, xs) != hipSuccess ||
        hipEventRecord(cpy[b], xs) != hipSuccess)
      rc = LYNX_ELAUNCH;
  }
  for (int b = 0; b < 2; ++b) {          // released by the runtime once the recorded work is done
    if (enc[b]) (void)hipEventDestroy(enc[b]);
    if (cpy[b]) (void)hipEventDestroy(cpy[b]);
  }
  return rc;
}

static int decode_common(bool full, const void* anchor_dev, const void* residual_dev, int n_pages,
                         int page_tokens, int kv_heads, int head_dim, int chunk, float alpha, int out_dtype,
                         void* out_dev, void* hip_stream) {
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  int st = check_geometry(n_pages, page_tokens, kv_heads, head_dim, chunk, alpha, &a.g);
  if (st != LYNX_OK) return st;
  if (out_dtype != LYNX_OUT_BF16 && out_dtype != LYNX_OUT_F32) return LYNX_EINVAL;
  if (n_pages == 0) return LYNX_OK;
  if (!aligned16(anchor_dev) || !aligned16(out_dev)) return LYNX_EALIGN;
  if (full && !aligned16(residual_dev)) return LYNX_EALIGN;
  a.anchor = static_cast<const uint8_t*>(anchor_dev);
  a.residual = full ? static_cast<const uint8_t*>(residual_dev) : nullptr;
  a.out = out_dev;
  const double al = (double)alpha;
  if (full) {
    // index = anchor nibble | residual nibble << 4; I = V_recon - V_res ([Review] Eq. 15)
    for (int idx = 0; idx < 256; ++idx) {
      int S, vmag;
      anchor_fields(idx & 15, &S, &vmag);
      const int rn = idx >> 4;
      const int vres = rn >= 8 ? rn - 16 : rn;
      int I = 16 * vmag + 7 - vres;
      a.lut[idx] = (float)(S * alaw_mag(I, al));
    }
  } else {
    // anchor only: I = 16*V_mag + 7 (the residual taken as 0)
    for (int nib = 0; nib < 16; ++nib) {
      int S, vmag;
      anchor_fields(nib, &S, &vmag);
      a.lut[nib] = (float)(S * alaw_mag(16 * vmag + 7, al));
    }
  }
  const int ntiles = (page_tokens + kDecTile - 1) / kDecTile;
  const long long n_units = (long long)n_pages * kv_heads * ntiles;    // (page, head, 128-token tile)
  // one workgroup per unit: measured 8-11% faster than 2048 workgroups walking ranges of
  // units, whose loads wait behind their previous unit's stores
  const dim3 grid((unsigned)n_units);
  const void* fn;
  if (full) fn = out_dtype == LYNX_OUT_F32 ? reinterpret_cast<const void*>(&k_decode<true, true>)
                                           : reinterpret_cast<const void*>(&k_decode<true, false>);
  else fn = out_dtype == LYNX_OUT_F32 ? reinterpret_cast<const void*>(&k_decode<false, true>)
                                      : reinterpret_cast<const void*>(&k_decode<false, false>);
  return launch(fn, grid, &a, static_cast<hipStream_t>(hip_stream));
}

int lynx_decode_anchor(const void* anchor_dev, int n_pages, int page_tokens, int kv_heads, int head_dim,
                       int chunk, float alpha, int out_dtype, void* out_dev, void* hip_stream) {
  return decode_common(false, anchor_dev, nullptr, n_pages, page_tokens, kv_heads, head_dim, chunk, alpha,
                       out_dtype, out_dev, hip_stream);
}

int lynx_decode_full(const void* anchor_dev, const void* residual_dev, int n_pages, int page_tokens,
                     int kv_heads, int head_dim, int chunk, float alpha, int out_dtype, void* out_dev,
                     void* hip_stream) {
  return decode_common(true, anchor_dev, residual_dev, n_pages, page_tokens, kv_heads, head_dim, chunk, alpha,
                       out_dtype, out_dev, hip_stream);
}

size_t lynx_attn_workspace_bytes(int batch, int ctx_tokens, int q_heads, int kv_heads, int head_dim,
                                 int page_tokens, int chunk) {
  return attn_workspace_bytes(batch, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk);
}

int lynx_attn_anchor(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch,
                     int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                     float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype,
                     void* out_dev, void* hip_stream) {
  return attn_anchor_launch(q_dev, k_anchor_dev, v_anchor_dev, batch, ctx_tokens, q_heads, kv_heads, head_dim,
                            page_tokens, chunk, alpha, sm_scale, workspace_dev, ws_bytes, out_dtype, out_dev,
                            static_cast<hipStream_t>(hip_stream));
}

int lynx_attn_anchor_noalloc(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch,
                             int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                             float alpha, float sm_scale, int out_dtype, void* out_dev, void* hip_stream) {
  return attn_anchor_noalloc_launch(q_dev, k_anchor_dev, v_anchor_dev, batch, ctx_tokens, q_heads, kv_heads,
                                    head_dim, page_tokens, chunk, alpha, sm_scale, out_dtype, out_dev,
                                    static_cast<hipStream_t>(hip_stream));
}

int lynx_attn_anchor_paged(const void* q_dev, const void* k_anchor_pool_dev, const void* v_anchor_pool_dev,
                           int n_pool_pages, const int32_t* block_table_dev, const int32_t* seq_lens_dev, int batch,
                           int max_pages_per_seq, int q_heads, int kv_heads, int head_dim, int page_tokens,
                           int chunk, float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes,
                           int out_dtype, void* out_dev, void* hip_stream) {
  return attn_anchor_paged_launch(q_dev, k_anchor_pool_dev, v_anchor_pool_dev, n_pool_pages, block_table_dev,
                                  seq_lens_dev, batch, max_pages_per_seq, q_heads, kv_heads, head_dim, page_tokens,
                                  chunk, alpha, sm_scale, workspace_dev, ws_bytes, out_dtype, out_dev,
                                  static_cast<hipStream_t>(hip_stream));
}

size_t lynx_attn_verify_workspace_bytes(int batch, int n_query, int ctx_tokens, int q_heads, int kv_heads,
                                        int head_dim, int page_tokens, int chunk) {
  return verify_workspace_bytes(batch, n_query, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk);
}

int lynx_attn_verify(const void* q_dev, const void* k_anchor_dev, const void* k_residual_dev,
                     const void* v_anchor_dev, const void* v_residual_dev, int batch, int n_query, int ctx_tokens,
                     int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk, float alpha,
                     float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype, void* out_dev,
                     float* lse_dev, void* hip_stream) {
  return verify_launch(q_dev, k_anchor_dev, k_residual_dev, v_anchor_dev, v_residual_dev, batch, n_query,
                       ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk, alpha, sm_scale, workspace_dev,
                       ws_bytes, out_dtype, out_dev, lse_dev, static_cast<hipStream_t>(hip_stream));
}

int lynx_attn_verify_paged(const void* q_dev, const void* k_anchor_pool_dev, const void* k_residual_pool_dev,
                           const void* v_anchor_pool_dev, const void* v_residual_pool_dev, int n_pool_pages,
                           const int32_t* block_table_dev, const int32_t* seq_lens_dev, int batch, int n_query,
                           int max_pages_per_seq, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                           float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype,
                           void* out_dev, float* lse_dev, void* hip_stream) {
  return verify_paged_launch(q_dev, k_anchor_pool_dev, k_residual_pool_dev, v_anchor_pool_dev, v_residual_pool_dev,
                             n_pool_pages, block_table_dev, seq_lens_dev, batch, n_query, max_pages_per_seq, q_heads,
                             kv_heads, head_dim, page_tokens, chunk, alpha, sm_scale, workspace_dev, ws_bytes,
                             out_dtype, out_dev, lse_dev, static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
