// Verification-pass attention over full (anchor + residual) codes, for gfx950.
//
// Sources, cited by page title and section:
//   [Review] "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
//            LLM Inference" (technical review of arXiv 2607.01831):
//            Mechanism 3, single parallel verification pass (all draft tokens in
//            one forward pass once Q_full is available); Mechanism 2, residual
//            phase (Q_full = dequant(Q_anc + Q_res)); Prerequisites §1, Eq. 1.
//
// Every one of the M draft tokens of a sequence attends, per query head, to the
// sequence's context tokens, whose keys and values are the full decode
//     x_hat[t,d] = A[c,d] L[n_td] + B[c,d],   A = (gamma_scale+eps)(sigma+eps),
//                                             B = gamma_min + mu (gamma_scale+eps),
// with L[n] the signed alpha-law value of the 8-bit full code n (anchor nibble |
// residual nibble << 4) and c the chunk of token t.
//
// Decomposition: one workgroup (8 waves) per (sequence, kv head, block of 128 query
// rows, context split); query row r = m*G + h (draft token m, query head h of the
// group).  Per 64-token tile the workgroup first decodes the tile once into LDS:
//   * keys as K_hat = A*L + B in float32, stored as BF16 high and low parts
//     (K_hat ~ hi + lo to ~16 bits), row-major [token][channel];
//   * values as the raw table values L (float16), transposed [channel][token];
// then each wave takes 16 query rows:
//   scores  S^T[token, row] = K_hi q + K_lo q on MFMA 16x16x32 bf16 (the BF16 query
//           is exact in this format);
//   online softmax in base 2 per row;
//   values  T^T[d, row] = sum_t L_V[d, t] p[t, row] on MFMA 16x16x32 f16, and
//           O += A_V T + B_V sum(p) (the value map applied after the product).
// Each wave writes a partial (m, l, o[128]) per row and split; k_verify_combine
// merges the splits with the log-sum-exp rule and returns O and the natural-log
// LSE of each row's scaled scores.
#include "../../include/lynx.h"
#include "lynx_kernels.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace lynx {

namespace {

typedef _Float16 vh8 __attribute__((ext_vector_type(8)));
typedef __bf16 vb8 __attribute__((ext_vector_type(8)));
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu4 __attribute__((ext_vector_type(4)));

constexpr int kVWaves = 8;                 // waves per workgroup
constexpr int kVThreads = kVWaves * 64;
constexpr int kVRows = 16 * kVWaves;       // query rows per workgroup (16 per wave)
constexpr int kVTile = 64;                 // context tokens per step
constexpr int kLutCopies = 16;             // copies of each table entry (lane l reads copy l % 16)
constexpr int kRec = kHeadDim + 4;         // floats per partial record (o 16-byte aligned)

struct VerifyArgs {
  const uint16_t* q;                       // [B][M][Hq][128] BF16
  const uint8_t* kanc;
  const uint8_t* kres;
  const uint8_t* vanc;
  const uint8_t* vres;
  float* ws;                               // [B*M*Hq][splits][kRec] partials: m, l, 0, 0, o[128]
  void* out;                               // [B][M][Hq][128]
  float* lse;                              // [B][M][Hq] or nullptr
  int B, M, Hq, Hkv, G, P, C, npages, nck, H, R, rowblocks;
  long long anc_seg, codes;                // residual segment = codes bytes
  int splits, tiles_per_split, ntiles;
  float qscale;                            // sm_scale * log2(e): scores kept in base 2
  int out_f32;
  float lut32[256];                        // S|x| of the full code n = anchor | residual << 4
  uint16_t lut16[256];                     // the same, float16 (round to nearest even)
};

// Reductions over the 4 lane groups (l / 16) with the gfx950 lane-swap instructions.
__device__ __forceinline__ float group_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// BF16 of a float, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One tile's raw inputs for this thread.
struct VerifyIn {
  uint2 ka, kr;          // key codes: token t/8, channels 16*(t%8) .. +15
  uint32_t va[2], vr[2]; // value codes: tokens 2*(t/16), +1; channels 8*(t%16) .. +7
  float meta[4];         // threads < 256: gamma_min, gamma_scale, mu, sigma of one channel
};

__device__ __forceinline__ void verify_load(const VerifyArgs& a, int b, int kvh, int tile, int tid, VerifyIn& in) {
  const int tok = tile * kVTile;
  const int page = tok / a.P;
  const int tin = tok - page * a.P;
  const int kc = tin / a.C;
  const size_t pg = (size_t)b * a.npages + page;
  const size_t row0 = ((size_t)kvh * a.P + tin) * (kHeadDim / 2);
  {
    const int t = tid >> 3, e8 = tid & 7;
    const size_t off = row0 + (size_t)t * (kHeadDim / 2) + 8 * e8;
    in.ka = *reinterpret_cast<const uint2*>(a.kanc + pg * a.anc_seg + off);
    in.kr = *reinterpret_cast<const uint2*>(a.kres + pg * a.codes + off);
  }
  {
    const int c8 = tid & 15, tq = tid >> 4;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const size_t off = row0 + (size_t)(2 * tq + r) * (kHeadDim / 2) + 4 * c8;
      in.va[r] = *reinterpret_cast<const uint32_t*>(a.vanc + pg * a.anc_seg + off);
      in.vr[r] = *reinterpret_cast<const uint32_t*>(a.vres + pg * a.codes + off);
    }
  }
  if (tid < 2 * kHeadDim) {
    const int c = tid & (kHeadDim - 1);
    const uint8_t* seg = (tid < kHeadDim ? a.kanc : a.vanc) + pg * a.anc_seg + a.codes;
    const float* meta = reinterpret_cast<const float*>(seg) + kvh * kHeadDim + c;
    in.meta[0] = meta[0];
    in.meta[1] = meta[a.H];
    in.meta[2] = meta[2 * (size_t)a.H + (size_t)kc * a.H];
    in.meta[3] = meta[2 * (size_t)a.H + (size_t)(a.nck + kc) * a.H];
  }
}

}  // namespace

__global__ __launch_bounds__(kVThreads) void k_verify(VerifyArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int b = blockIdx.z / a.rowblocks, rb = blockIdx.z - b * a.rowblocks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  __shared__ float s_lut[256 * kLutCopies];          // float32 table, entry e copy c at e*16 + c
  __shared__ uint16_t s_lut16[256 * kLutCopies];     // float16 table
  __shared__ uint32_t s_kh[kVTile * 64];             // K_hat BF16 high parts, [token][channel pair]
  __shared__ uint32_t s_kl[kVTile * 64];             // K_hat BF16 low parts
  __shared__ uint32_t s_lv[kHeadDim * (kVTile / 2)]; // L_V float16, [channel][token pair]
  __shared__ float2 s_abk[kHeadDim];                 // (A_K, B_K) per channel
  __shared__ float2 s_abv[kHeadDim];                 // (A_V, B_V) per channel

  for (int i = tid; i < 256 * kLutCopies; i += kVThreads) {
    s_lut[i] = a.lut32[i / kLutCopies];
    s_lut16[i] = a.lut16[i / kLutCopies];
  }
  const int lcopy = tid & (kLutCopies - 1);

  // this lane's query row (column n of the wave's MFMA tiles) and its BF16 operand:
  // channels 32kk + 8g .. +7 for k-step kk
  const int row = rb * kVRows + wave * 16 + n;
  const bool row_live = row < a.R;
  vb8 qop[4];
  {
    const int m = row_live ? row / a.G : 0, hh = row_live ? row - (row / a.G) * a.G : 0;
    const uint16_t* qp = a.q + ((size_t)(b * a.M + m) * a.Hq + kvh * a.G + hh) * kHeadDim + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * kk);
      if (!row_live) w = make_uint4(0u, 0u, 0u, 0u);
      const vu4 wv = {w.x, w.y, w.z, w.w};
      qop[kk] = __builtin_bit_cast(vb8, wv);
    }
  }
  const float qscale = a.qscale;

  float m_run = -INFINITY, l_run = 0.0f;
  vf4 o_acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o_acc[j] = vf4{0.f, 0.f, 0.f, 0.f};

  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(a.ntiles, t_begin + a.tiles_per_split);
  VerifyIn in;
  if (t_begin < t_end) verify_load(a, b, kvh, t_begin, tid, in);

  for (int tile = t_begin; tile < t_end; ++tile) {
    __syncthreads();   // the previous tile's LDS tables are no longer read (and the lookup tables are filled)

    // ---- the chunk's affine maps, one channel of K or V per thread
    if (tid < 2 * kHeadDim) {
      const float d1 = in.meta[1] + (float)kEps, d2 = in.meta[3] + (float)kEps;
      const float2 ab = make_float2(d1 * d2, fmaf(in.meta[2], d1, in.meta[0]));
      if (tid < kHeadDim) s_abk[tid] = ab;
      else s_abv[tid - kHeadDim] = ab;
    }
    __syncthreads();

    // ---- decode the tile into LDS
    {
      // keys: token t = tid/8, channels 16*(tid%8) + k; K_hat = A*L + B, split into BF16 hi + lo
      const int t = tid >> 3, e8 = tid & 7;
      const uint32_t kw[2] = {in.ka.x, in.ka.y}, rw[2] = {in.kr.x, in.kr.y};
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          float kh[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int sh = 4 * (k + e);
            const uint32_t idx = ((kw[w] >> sh) & 0xFu) | (((rw[w] >> sh) & 0xFu) << 4);
            const float2 ab = s_abk[16 * e8 + 8 * w + k + e];
            kh[e] = fmaf(ab.x, s_lut[idx * kLutCopies + lcopy], ab.y);
          }
          const uint32_t h0 = bf16_bits(kh[0]), h1 = bf16_bits(kh[1]);
          const uint32_t l0 = bf16_bits(kh[0] - __uint_as_float(h0 << 16));
          const uint32_t l1 = bf16_bits(kh[1] - __uint_as_float(h1 << 16));
          hi[4 * w + k / 2] = h0 | (h1 << 16);
          lo[4 * w + k / 2] = l0 | (l1 << 16);
        }
      }
      // row t holds 64 channel pairs = 16 columns of 16 B; column c16 at c16 ^ (t & 15)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c16 = (2 * e8 + h) ^ (t & 15);
        *reinterpret_cast<uint4*>(&s_kh[t * 64 + 4 * c16]) = make_uint4(hi[4 * h], hi[4 * h + 1], hi[4 * h + 2], hi[4 * h + 3]);
        *reinterpret_cast<uint4*>(&s_kl[t * 64 + 4 * c16]) = make_uint4(lo[4 * h], lo[4 * h + 1], lo[4 * h + 2], lo[4 * h + 3]);
      }
    }
    {
      // values: channels 8*(tid%16) + j, tokens 2*(tid/16), +1; L as float16 pairs, transposed.
      // Row d holds 16 units of 8 B (4 tokens each); unit u at u ^ (d & 15).
      const int c8 = tid & 15, tq = tid >> 4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t i0 = ((in.va[0] >> (4 * j)) & 0xFu) | (((in.vr[0] >> (4 * j)) & 0xFu) << 4);
        const uint32_t i1 = ((in.va[1] >> (4 * j)) & 0xFu) | (((in.vr[1] >> (4 * j)) & 0xFu) << 4);
        const uint32_t v = (uint32_t)s_lut16[i0 * kLutCopies + lcopy] | ((uint32_t)s_lut16[i1 * kLutCopies + lcopy] << 16);
        const int d = 8 * c8 + j;
        const int unit = (tq >> 1) ^ (d & 15);
        s_lv[d * (kVTile / 2) + 2 * unit + (tq & 1)] = v;
      }
    }
    // the next tile's raw inputs are loaded while this one is used
    if (tile + 1 < t_end) verify_load(a, b, kvh, tile + 1, tid, in);
    __syncthreads();

    // ---- scores for this wave's 16 rows: S^T[token, row], tokens 16mb + 4g + i
    float s[16];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      vf4 acc = vf4{0.f, 0.f, 0.f, 0.f};
      const int t = 16 * mb + n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c16 = (4 * kk + g) ^ n;          // (t & 15) == n
        const uint4 wh = *reinterpret_cast<const uint4*>(&s_kh[t * 64 + 4 * c16]);
        const uint4 wl = *reinterpret_cast<const uint4*>(&s_kl[t * 64 + 4 * c16]);
        const vu4 vh = {wh.x, wh.y, wh.z, wh.w}, vl = {wl.x, wl.y, wl.z, wl.w};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vb8, vh), qop[kk], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vb8, vl), qop[kk], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[4 * mb + i] = acc[i] * qscale;
    }

    // ---- online softmax (base 2) for row n over the tile's 64 tokens
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = group_max(mt);
    const float m_new = fmaxf(m_run, mt);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    float lsum = 0.0f;
    vh8 pt[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(s[i] - m_new);
      lsum += p;
      pt[i >> 3][i & 7] = (_Float16)p;
    }
    l_run = fmaf(l_run, corr, lsum);
    if (__builtin_amdgcn_ballot_w64(corr != 1.0f) != 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) o_acc[j] *= corr;
    }
    m_run = m_new;
    const float lt = group_sum(lsum);

    // ---- values: T^T[d, row] = sum_t L_V[d, t] p[t, row], d = 16j + 4g + i of the output block j.
    // The k index of step ks runs over tokens 32ks + 4g + 0..3 then 32ks + 16 + 4g + 0..3 (the
    // layout of the probabilities in pt[ks]); the table values are read in the same order.
    vf4 tacc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) tacc[j] = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 16 * j + n;
        const int u0 = (8 * ks + g) ^ (d & 15), u1 = (8 * ks + 4 + g) ^ (d & 15);
        const uint2 w0 = *reinterpret_cast<const uint2*>(&s_lv[d * (kVTile / 2) + 2 * u0]);
        const uint2 w1 = *reinterpret_cast<const uint2*>(&s_lv[d * (kVTile / 2) + 2 * u1]);
        const vu4 va4 = {w0.x, w0.y, w1.x, w1.y};
        tacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vh8, va4), pt[ks], tacc[j], 0, 0, 0);
      }
    }
    // ---- undo the value map: o += A_V * T + B_V * sum(p)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 ab01 = *reinterpret_cast<const float4*>(&s_abv[16 * j + 4 * g]);
      const float4 ab23 = *reinterpret_cast<const float4*>(&s_abv[16 * j + 4 * g + 2]);
      o_acc[j][0] = fmaf(ab01.x, tacc[j][0], fmaf(ab01.y, lt, o_acc[j][0]));
      o_acc[j][1] = fmaf(ab01.z, tacc[j][1], fmaf(ab01.w, lt, o_acc[j][1]));
      o_acc[j][2] = fmaf(ab23.x, tacc[j][2], fmaf(ab23.y, lt, o_acc[j][2]));
      o_acc[j][3] = fmaf(ab23.z, tacc[j][3], fmaf(ab23.w, lt, o_acc[j][3]));
    }
  }

  // ---- this split's partial record for the lane's row: (m, l, o[d]) with d = 16j + 4g + i
  l_run = group_sum(l_run);
  if (row_live) {
    const int m = row / a.G, hh = row - m * a.G;
    float* rec = a.ws + ((size_t)((b * a.M + m) * a.Hq + kvh * a.G + hh) * a.splits + split) * kRec;
    if (g == 0) *reinterpret_cast<float4*>(rec) = make_float4(m_run, l_run, 0.0f, 0.0f);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<float4*>(rec + 4 + 16 * j + 4 * g) = make_float4(o_acc[j][0], o_acc[j][1], o_acc[j][2], o_acc[j][3]);
  }
}

// log-sum-exp merge of the context splits: one workgroup per (sequence, draft token, query head)
__global__ __launch_bounds__(kHeadDim) void k_verify_combine(VerifyArgs a) {
  const int row = blockIdx.x;          // (b * M + m) * Hq + hq
  const int d = threadIdx.x;
  const float* rec = a.ws + (size_t)row * a.splits * kRec;
  float M2 = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M2 = fmaxf(M2, rec[(size_t)s * kRec]);
  float o = 0.0f, l = 0.0f;
  for (int s = 0; s < a.splits; ++s) {
    const float* r = rec + (size_t)s * kRec;
    const float f = (r[0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(r[0] - M2);
    o = fmaf(r[4 + d], f, o);
    l = fmaf(r[1], f, l);
  }
  const float res = o / l;
  if (a.out_f32) static_cast<float*>(a.out)[(size_t)row * kHeadDim + d] = res;
  else {
    const uint32_t u = __float_as_uint(res);
    static_cast<uint16_t*>(a.out)[(size_t)row * kHeadDim + d] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  // natural-log LSE of the scaled scores: the partials are in base 2
  if (a.lse && d == 0) a.lse[row] = (M2 + __log2f(l)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

struct VerifyPlan {
  int rowblocks, splits, tiles_per_split, ntiles;
};

bool verify_plan(int batch, int n_query, int ctx, int Hq, int Hkv, int D, int P, int C, VerifyPlan* pl) {
  if (batch <= 0 || n_query <= 0 || ctx <= 0 || Hq <= 0 || Hkv <= 0 || P <= 0 || C <= 0) return false;
  if (ctx % P != 0 || P % C != 0 || Hq % Hkv != 0) return false;
  if (D != kHeadDim || C % kVTile != 0) return false;
  const long long R = (long long)n_query * (Hq / Hkv);
  pl->rowblocks = (int)((R + kVRows - 1) / kVRows);
  pl->ntiles = ctx / kVTile;
  const long long units = (long long)batch * Hkv * pl->rowblocks;
  int want = (int)((1024 + units - 1) / units);               // aim for ~1024 workgroups
  want = std::max(1, std::min(want, pl->ntiles));
  pl->tiles_per_split = (pl->ntiles + want - 1) / want;
  pl->splits = (pl->ntiles + pl->tiles_per_split - 1) / pl->tiles_per_split;
  return true;
}

}  // namespace

size_t verify_workspace_bytes(int batch, int n_query, int ctx, int Hq, int Hkv, int D, int P, int C) {
  VerifyPlan pl;
  if (!verify_plan(batch, n_query, ctx, Hq, Hkv, D, P, C, &pl)) return 0;
  return (size_t)batch * n_query * Hq * pl.splits * kRec * sizeof(float);
}

int verify_launch(const void* q_dev, const void* k_anchor_dev, const void* k_residual_dev, const void* v_anchor_dev,
                  const void* v_residual_dev, int batch, int n_query, int ctx_tokens, int q_heads, int kv_heads,
                  int head_dim, int page_tokens, int chunk, float alpha, float sm_scale, void* workspace_dev,
                  size_t ws_bytes, int out_dtype, void* out_dev, float* lse_dev, hipStream_t stream) {
  if (batch < 0 || n_query <= 0 || ctx_tokens <= 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 ||
      page_tokens <= 0 || chunk <= 0)
    return LYNX_EINVAL;
  if (ctx_tokens % page_tokens != 0 || page_tokens % chunk != 0 || q_heads % kv_heads != 0) return LYNX_EINVAL;
  if (!std::isfinite(alpha) || !(alpha > 0.0f) || !std::isfinite(sm_scale)) return LYNX_EINVAL;
  if (out_dtype != LYNX_OUT_BF16 && out_dtype != LYNX_OUT_F32) return LYNX_EINVAL;
  if (head_dim != kHeadDim || chunk % kVTile != 0 || batch > 65535 || kv_heads > 65535) return LYNX_EUNSUPPORTED;
  if (batch == 0) return LYNX_OK;
  VerifyPlan pl;
  if (!verify_plan(batch, n_query, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk, &pl))
    return LYNX_EINVAL;
  if ((long long)batch * pl.rowblocks > 65535 || (long long)batch * n_query * q_heads > 0x7fffffffll)
    return LYNX_EUNSUPPORTED;
  const size_t need = (size_t)batch * n_query * q_heads * pl.splits * kRec * sizeof(float);
  auto al16 = [](const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!al16(q_dev) || !al16(k_anchor_dev) || !al16(k_residual_dev) || !al16(v_anchor_dev) ||
      !al16(v_residual_dev) || !al16(out_dev) || !al16(workspace_dev) ||
      (lse_dev != nullptr && (reinterpret_cast<uintptr_t>(lse_dev) & 3u) != 0))
    return LYNX_EALIGN;
  if (ws_bytes < need) return LYNX_ENOSPACE;

  VerifyArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q_dev);
  a.kanc = static_cast<const uint8_t*>(k_anchor_dev);
  a.kres = static_cast<const uint8_t*>(k_residual_dev);
  a.vanc = static_cast<const uint8_t*>(v_anchor_dev);
  a.vres = static_cast<const uint8_t*>(v_residual_dev);
  a.ws = static_cast<float*>(workspace_dev);
  a.out = out_dev;
  a.lse = lse_dev;
  a.B = batch;
  a.M = n_query;
  a.Hq = q_heads;
  a.Hkv = kv_heads;
  a.G = q_heads / kv_heads;
  a.P = page_tokens;
  a.C = chunk;
  a.npages = ctx_tokens / page_tokens;
  a.nck = page_tokens / chunk;
  a.H = kv_heads * head_dim;
  a.R = n_query * a.G;
  a.rowblocks = pl.rowblocks;
  a.codes = (long long)page_tokens * a.H / 2;
  a.anc_seg = a.codes + 4ll * a.H * (2 + 2ll * a.nck);
  a.splits = pl.splits;
  a.tiles_per_split = pl.tiles_per_split;
  a.ntiles = pl.ntiles;
  const double scale = sm_scale > 0.0f ? (double)sm_scale : 1.0 / std::sqrt((double)head_dim);
  a.qscale = (float)(scale * 1.4426950408889634);   // log2(e)
  a.out_f32 = out_dtype == LYNX_OUT_F32;
  // full-code table: index = anchor nibble | residual nibble << 4, I = V_recon - V_res
  // ([Review] Eq. 9 inverted and Eq. 15), |x| = ((1+alpha)^(I/127) - 1)/alpha
  const double al = (double)alpha, L = std::log1p(al);
  for (int idx = 0; idx < 256; ++idx) {
    const int an = idx & 15, rn = idx >> 4;
    const int qa = an >= 8 ? an - 16 : an;
    const int S = qa < 0 ? -1 : 1, vmag = qa < 0 ? -qa - 1 : qa;
    const int vres = rn >= 8 ? rn - 16 : rn;
    const int I = 16 * vmag + 7 - vres;
    const double v = S * std::expm1((double)I / kCodeMax * L) / al;
    a.lut32[idx] = (float)v;
    const _Float16 h = (_Float16)v;
    a.lut16[idx] = __builtin_bit_cast(uint16_t, h);
  }
  void* kargs[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&k_verify),
                                 dim3((unsigned)pl.splits, (unsigned)kv_heads, (unsigned)(batch * pl.rowblocks)),
                                 dim3(kVThreads), kargs, 0, stream);
  if (e != hipSuccess) return LYNX_ELAUNCH;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&k_verify_combine), dim3((unsigned)(batch * n_query * q_heads)),
                      dim3(kHeadDim), kargs, 0, stream);
  return e == hipSuccess ? LYNX_OK : LYNX_ELAUNCH;
}

}  // namespace lynx
