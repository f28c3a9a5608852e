// Kernel and launcher declarations shared between the C ABI shim and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "lynx_common.hpp"

namespace lynx {

template <int C, bool PAGE_STORED>
__global__ void k_encode(EncodeArgs a);
__global__ void k_page_extremes(EncodeArgs a);
__global__ void k_page_finish(EncodeArgs a);
template <bool FULL, bool F32OUT>
__global__ void k_decode(DecodeArgs a);

// Anchor-only decode attention (lynx_attn.hip).
size_t attn_workspace_bytes(int batch, int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens,
                            int chunk);
int attn_anchor_launch(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch,
                       int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                       float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype,
                       void* out_dev, hipStream_t stream);
int attn_anchor_noalloc_launch(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch,
                               int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                               float alpha, float sm_scale, int out_dtype, void* out_dev, hipStream_t stream);
int attn_anchor_paged_launch(const void* q_dev, const void* k_anchor_pool, const void* v_anchor_pool, int n_pool,
                             const int32_t* block_table, const int32_t* seq_lens, int batch, int max_pages,
                             int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk, float alpha,
                             float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype, void* out_dev,
                             hipStream_t stream);

// Verification-pass attention over full codes (lynx_verify.hip).
size_t verify_workspace_bytes(int batch, int n_query, int ctx_tokens, int q_heads, int kv_heads, int head_dim,
                              int page_tokens, int chunk);
int verify_launch(const void* q_dev, const void* k_anchor_dev, const void* k_residual_dev, const void* v_anchor_dev,
                  const void* v_residual_dev, int batch, int n_query, int ctx_tokens, int q_heads, int kv_heads,
                  int head_dim, int page_tokens, int chunk, float alpha, float sm_scale, void* workspace_dev,
                  size_t ws_bytes, int out_dtype, void* out_dev, float* lse_dev, hipStream_t stream);
int verify_paged_launch(const void* q_dev, const void* k_anchor_pool, const void* k_residual_pool,
                        const void* v_anchor_pool, const void* v_residual_pool, int n_pool, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int n_query, int max_pages, int q_heads, int kv_heads,
                        int head_dim, int page_tokens, int chunk, float alpha, float sm_scale, void* workspace_dev,
                        size_t ws_bytes, int out_dtype, void* out_dev, float* lse_dev, hipStream_t stream);

}  // namespace lynx
