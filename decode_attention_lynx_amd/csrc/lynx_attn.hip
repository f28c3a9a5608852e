// Single-token decode attention over anchor-only codes (the speculative draft
// path), fused with the anchor decode, for gfx950.
//
// Sources, cited by page title and section:
//   [Review] "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
//            LLM Inference" (technical review of arXiv 2607.01831):
//            Prerequisites §1, Eq. 1 (O = softmax(Q K^T / sqrt(d_k)) V);
//            Mechanism 2, decode-side anchor phase (drafting runs on
//            Q_approx = dequant(Q_anc, gamma, mu, sigma)); Mechanism 1, Eq. 8-9.
//
// The anchor decode of a key is k_hat[t,d] = A[c,d] L[n_td] + B[c,d] with
// A = (gamma_scale+eps)(sigma+eps), B = gamma_min + mu(gamma_scale+eps) for the
// chunk c of token t, and L[n] = S|x| of the anchor nibble n.  Folding the
// per-chunk affine map into the query turns the score into
//     q . k_hat_t = sum_d (q_d A[c,d]) L[n_td] + sum_d q_d B[c,d],
// a dense contraction over the raw nibble table values, which runs on MFMA.
// Likewise sum_t p_t v_hat[t,d] = A_V[c,d] sum_t p_t L[n_td] + B_V[c,d] sum_t p_t.
//
// Decomposition: one workgroup (12 or 8 waves) per (sequence, kv head, context split);
// each wave walks tiles of 64 tokens (32 for pages of an odd number of 32-token chunks, or
// chunks of 8) with an online softmax; a tile holds one chunk of 64 or more, or 2 or 4
// whole chunks, each folded with its own map.  The waves merge in LDS and write one partial
// (m, l, o[128]) per query head; k_attn_combine merges the splits with the log-sum-exp rule.
//
// MFMA v_mfma_f32_16x16x32_f16 (A 16x32, B 32x16, C 16x16; lane l supplies row /
// column l % 16 and the k-block l / 16; C rows 4*(l/16)..+3, column l % 16):
//   scores  S^T[token, col] = sum_d L[token, d] * qt[d, col]: A = nibble-table values of
//           16 tokens, B = the folded query in float16 hi + lo parts (~22 bits): for groups
//           of up to 8 heads columns 0..7 hold the high parts and 8..15 the remainders (one
//           MFMA, the halves added after); for groups of 9..16 heads column h is head h and
//           the two parts take two MFMAs.  The key map carries a per-tile power-of-two
//           exponent that keeps every folded |q| inside float16, undone in float32.
//   values  O^T[d, col] += sum_t L_V[t, d] * p[t, col]: A = table values of 16
//           channels over 32 tokens, B = float16 probabilities.
#include "../../include/lynx.h"
#include "lynx_kernels.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

namespace lynx {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kAttnWorkgroups = 256;   // workgroups the context splits aim for
constexpr int kMaxGroup = 16;        // query heads per kv head handled by one workgroup

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* kanc;
  const uint8_t* vanc;
  float* ws;
  void* out;
  int B, T, Hq, Hkv, G, P, C, npages, nck, H;
  long long anc_seg, codes;
  int splits, tiles_per_split, ntiles;
  float qscale;        // sm_scale * log2(e): scores are kept in base 2
  int out_f32;
  // paged form: sequence b's page p is pool segment block_table[b * max_pages + p] (clamped
  // into [0, n_pool)), and only its first seq_lens[b] tokens (clamped into [0, T]) count.
  // Contiguous form: block_table and seq_lens are null, segment b * npages + p, T tokens.
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_pages, n_pool;
  uint32_t pair[256];  // float16 pair table: entry b = L[b & 15] | L[b >> 4] << 16 (L = S|x| of a nibble)
};

// Segment of sequence b's page `page` (uniform: a scalar load in the paged form).
__device__ __forceinline__ size_t segment_of(const AttnArgs& a, int b, int page) {
  if (a.block_table == nullptr) return (size_t)b * a.npages + page;
  const int s = a.block_table[(size_t)b * a.max_pages + page];
  return (size_t)min(max(s, 0), a.n_pool - 1);
}

__device__ __forceinline__ float dpp_row_ror8(float v) {
  // rotate right by 8 lanes inside each row of 16: column n reads column n ^ 8
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}

// Reductions over the 4 lane groups (l / 16) with the gfx950 lane-swap instructions:
// v_permlane32_swap of a value with itself yields, in every lane, the value of lane
// l and of lane l ^ 32 in its two outputs; v_permlane16_swap does the same for l ^ 16.
// No LDS round trip, and every lane of a group ends with the same result.
__device__ __forceinline__ float xor32_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max_g(float v) {
  v = xor32_pair_max(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_g(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// The pair table (256 dwords) is held in 64 copies, entry e of copy r at byte
// e*256 + 4r, and lane l reads copy l: no two lanes ever meet in a bank.  The byte
// address (e << 8) | 4l is assembled by one v_perm from the code word (byte k = e)
// and a register holding 4l in its low byte.
__device__ __forceinline__ uint32_t pair_at(const uint32_t* s_pair, uint32_t lane4, uint32_t w, int k) {
  const uint32_t addr = __builtin_amdgcn_perm(lane4, w, 0x0c0c0004u | ((uint32_t)k << 8));
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(s_pair) + addr);
}

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// 8 consecutive channels of one token (one dword of nibbles) -> MFMA operand
__device__ __forceinline__ h8 lookup_row(uint32_t w, const uint32_t* s_pair, uint32_t lane4) {
  const u32x4v r = {pair_at(s_pair, lane4, w, 0), pair_at(s_pair, lane4, w, 1), pair_at(s_pair, lane4, w, 2),
                    pair_at(s_pair, lane4, w, 3)};
  return __builtin_bit_cast(h8, r);
}

// one wave's raw inputs for one 64-token tile
// CPT: chunks per tile (1, or 2 for a chunk of 32 in a 64-token tile)
template <int TILE, int CPT>
struct TileIn {
  uint4 kw[TILE / 16];      // K code rows tin + 16mb + n, bytes 16g .. 16g+15
  uint32_t vw[TILE / 4];    // V code dword n of the rows this lane feeds to the value MFMAs
  // gamma_min, gamma_scale, then mu and sigma of each chunk of the tile, for channels
  // 2*lane, 2*lane+1: [0..1] gamma_min, [2..3] gamma_scale, [4+4k..5+4k] mu, [6+4k..7+4k] sigma
  float km[4 + 4 * CPT], vm[4 + 4 * CPT];
};

// Per-lane byte offsets of one wave's tile loads; they do not depend on the tile, whose
// (wave-uniform) base addresses are added to them.  Code rows are 32 bytes per token in
// each of the head's two 64-channel code blocks (block b at b * P * 32 from the head's
// first row).
struct TileOffsets {
  uint32_t kcode;   // K code rows: channels 32g .. +31 of token n, i.e. block g/2, bytes 16(g%2) .. +15
  uint32_t vcode;   // V code rows: channels 8(n%16) .. +7 (block n/8, dword n%8) of row 4g
  uint32_t meta;    // float32 metadata of channels 2*lane, 2*lane + 1: 8*lane
};

__device__ __forceinline__ TileOffsets tile_offsets(int lane, int P) {
  const int n = lane & 15, g = lane >> 4;
  TileOffsets o;
  o.kcode = (uint32_t)((g >> 1) * P * kCodeRow + n * kCodeRow + 16 * (g & 1));
  o.vcode = (uint32_t)((n >> 3) * P * kCodeRow + 4 * (n & 7) + 4 * g * kCodeRow);
  o.meta = (uint32_t)(8 * lane);
  return o;
}

// `tile` is wave-uniform: the page, chunk and segment addresses are scalar arithmetic.
template <int TILE, int CPT>
__device__ __forceinline__ void load_tile(const AttnArgs& a, int b, int kvh, int tile, const TileOffsets& lo,
                                          TileIn<TILE, CPT>& t) {
  const int tok = tile * TILE;
  const int page = tok / a.P;
  const int tin = tok - page * a.P;
  const int kc = tin / a.C;
  const size_t seg = segment_of(a, b, page) * (size_t)a.anc_seg;
  const size_t row0 = code_offset(a.P, kvh, 0, tin);   // block 0 of the head, token tin
  const uint8_t* kcb = a.kanc + seg + row0;
  const uint8_t* vcb = a.vanc + seg + row0;
  // every code byte is read once.  Key rows are read as 16-byte pieces that tile whole 512 B
  // runs of each code block: streaming loads, which keep the caches for the metadata (the page
  // statistics are shared by all tiles of a page).  Value rows are read as 4-byte words, one
  // 32 B run of a code row per 8 lanes: plain (cached) loads, so the other half of each line
  // the memory returns is still in L2 when the next row's load asks for it (with streaming
  // loads these 32 B runs cost ~10% of the kernel time).
#pragma unroll
  for (int mb = 0; mb < TILE / 16; ++mb) t.kw[mb] = ld_stream(kcb + lo.kcode + 16 * mb * kCodeRow);
#pragma unroll
  for (int ks = 0; ks < TILE / 32; ++ks)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 32 * ks + (r < 4 ? r : 12 + r);     // + 4g (in the lane offset)
      t.vw[8 * ks + r] = *reinterpret_cast<const uint32_t*>(vcb + lo.vcode + row * kCodeRow);
    }
  const uint8_t* kmb = a.kanc + seg + a.codes + (size_t)kvh * kHeadDim * 4;
  const uint8_t* vmb = a.vanc + seg + a.codes + (size_t)kvh * kHeadDim * 4;
  size_t offs[2 + 2 * CPT];
  offs[0] = 0;
  offs[1] = (size_t)a.H;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    offs[2 + 2 * k] = 2 * (size_t)a.H + (size_t)(kc + k) * a.H;
    offs[3 + 2 * k] = 2 * (size_t)a.H + (size_t)(a.nck + kc + k) * a.H;
  }
#pragma unroll
  for (int f = 0; f < 2 + 2 * CPT; ++f) {
    const float2 k2 = *reinterpret_cast<const float2*>(kmb + offs[f] * 4 + lo.meta);
    const float2 v2 = *reinterpret_cast<const float2*>(vmb + offs[f] * 4 + lo.meta);
    t.km[2 * f] = k2.x;
    t.km[2 * f + 1] = k2.y;
    t.vm[2 * f] = v2.x;
    t.vm[2 * f + 1] = v2.y;
  }
}

// Maximum over all 64 lanes (every lane ends with it).
__device__ __forceinline__ float wave_max_all(float v) {
  v = wave_max_g(v);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
}

// TILE tokens per wave step holding CPT chunks of CT = TILE / CPT tokens (8 .. 64).
// GW = 8: the 16 MFMA columns are 8 query heads twice, the first 8 carrying the float16 high
//         part of the folded query and the second 8 its remainder (groups of up to 8 heads);
// GW = 16: the 16 columns are 16 query heads, the two parts of the folded query in two MFMAs.
// WAVES waves per workgroup: 12 (three per SIMD) or 8 (two per SIMD, for the register use of
// four chunks per tile).
template <int TILE, int CPT, int GW, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES / 4))) void k_attn_anchor(AttnArgs a) {
  constexpr int CT = TILE / CPT;       // tokens per chunk
  static_assert(CT >= 8 && (CT >= 16 || TILE == 32), "chunks of 8 tokens use 32-token tiles");
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: tile addressing stays scalar
  const int n = lane & 15, g = lane >> 4;
  const int hh = n & (GW - 1);          // query head (within the group) of this column
  const bool lo_col = GW == 8 && n >= 8;

  // LDS: the replicated pair table during the loop, reused for the wave merge after it
  constexpr int kPairWords = 256 * 64;
  // merge records of 8 heads at a time: o of head h at word h*kMergeRow + d + d/32 (one pad
  // word per 32 channels: the writes of the 8 heads x 4 lane groups then fall in 32 banks)
  constexpr int kMergeRow = kHeadDim + 4;
  constexpr int kMergeWords = 2 * WAVES * kMaxGroup + WAVES * 8 * kMergeRow;
  __shared__ uint32_t s_big[kPairWords > kMergeWords ? kPairWords : kMergeWords];
  // per wave: (A_K, B_K) of the chunk being folded, and (A_V, B_V) of every chunk of the tile,
  // for channels 2i, 2i+1 at slot swz(i), where swz(16g + t) = 4t + g puts the 4 lane groups'
  // simultaneous reads in different banks
  __shared__ float4 s_kab[WAVES][kHeadDim / 2];
  __shared__ float4 s_vab[WAVES][CPT][kHeadDim / 2];
  uint32_t* s_pair = s_big;

#pragma unroll 8
  for (int w = tid; w < kPairWords; w += WAVES * 64) s_pair[w] = a.pair[w >> 6];   // word 64e + r: entry e, copy r
  const uint32_t lane4 = 4u * (uint32_t)lane;

  // this lane's query slice (head hh, channels 32g .. 32g+31), kept as BF16 pairs, and the
  // largest |q| of the workgroup's heads (range of the folded query, below)
  uint32_t qw[16];
  float qmax = 0.0f;
  {
    const bool live = hh < a.G;
    const uint16_t* qp = a.q + ((size_t)(b * a.Hq + kvh * a.G + (live ? hh : 0))) * kHeadDim + 32 * g;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + 8 * v4);
      qw[4 * v4 + 0] = live ? w.x : 0u;
      qw[4 * v4 + 1] = live ? w.y : 0u;
      qw[4 * v4 + 2] = live ? w.z : 0u;
      qw[4 * v4 + 3] = live ? w.w : 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(qw[i])), fabsf(bf16_hi(qw[i]))));
    qmax = wave_max_all(qmax);
  }
  const float qscale = a.qscale;
  // |q_d A_d| * qscale <= qmax * (gamma_scale + eps) * (1 + eps) * qscale, since sigma <= 1
  const float qbound = qmax * (1.0f + (float)kEps) * qscale;
  const float lo_w = lo_col ? 1.0f : 0.0f;
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.0f;
  f4 o_acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o_acc[j] = f4{0.f, 0.f, 0.f, 0.f};

  // this sequence's context: T tokens, or its own length in the paged form
  const int seq_len = a.seq_lens == nullptr ? a.T : min(max(a.seq_lens[b], 0), a.T);
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min((seq_len + TILE - 1) / TILE, t_begin + a.tiles_per_split);   // may be empty
  float4* kab = s_kab[wave];
  float4 (*vab)[kHeadDim / 2] = s_vab[wave];
  const int slot = 4 * (lane & 15) + (lane >> 4);

  const TileOffsets toff = tile_offsets(lane, a.P);

  // one tile of this wave: scores, online softmax, values
  auto process = [&](const TileIn<TILE, CPT>& cur, int tile) {
    // ---- range of the folded query.  A key channel of range gamma_scale folds into
    //      |q~_d| <= |q_d| (gamma_scale + eps)(sigma + eps) qscale, which must stay inside
    //      float16.  The key map carries 2^-E, E >= 0 the smallest exponent that keeps every
    //      |q~| of the tile below 2^15 (from the tile's largest channel range), and the scores
    //      are scaled back by 2^E in float32 before the softmax.  Ordinary KV has E = 0.  (The
    //      reduction is done every tile: a branch around it, taken only when some lane's bound
    //      is large, measured ~5% slower than the unconditional ~12 instructions.)
    float sd, su;
    {
      const float mb_all = wave_max_all((fmaxf(cur.km[2], cur.km[3]) + (float)kEps) * qbound);
      const int e = (int)((__float_as_uint(mb_all) >> 23) & 0xFFu) - 127;   // floor(log2)
      const int E = max(0, e - 14);                                        // mb_all * 2^-E < 2^15
      sd = __uint_as_float((uint32_t)(127 - E) << 23);
      su = __uint_as_float((uint32_t)(127 + E) << 23);
    }
    const float qs = qscale * sd;

    // ---- the value maps of the tile's chunks, A = (gamma_scale+eps)(sigma+eps),
    //      B = gamma_min + mu (gamma_scale+eps), for channels 2*lane, 2*lane+1
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      float av[2], bv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float d1v = cur.vm[2 + e] + (float)kEps, d2v = cur.vm[6 + 4 * k + e] + (float)kEps;
        av[e] = d1v * d2v;
        bv[e] = fmaf(cur.vm[4 + 4 * k + e], d1v, cur.vm[e]);
      }
      vab[k][slot] = make_float4(av[0], av[1], bv[0], bv[1]);
    }

    // ---- per chunk: its key map (with the softmax scale, base 2, and 2^-E) folded into the
    //      query, qt = q*A_K as float16 high / low parts and beta = q.B_K, then the scores of
    //      its tokens: S^T = L_K (tokens x 128) * qt (128 x 16 columns)
    constexpr int NS = TILE / 4;         // scores per lane: TILE/16 row blocks x 4
    float s[NS];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      {
        float ak[2], bk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float d1k = cur.km[2 + e] + (float)kEps, d2k = cur.km[6 + 4 * k + e] + (float)kEps;
          ak[e] = d1k * d2k * qs;
          bk[e] = fmaf(cur.km[4 + 4 * k + e], d1k, cur.km[e]) * qs;
        }
        if (k > 0) __builtin_amdgcn_wave_barrier();   // the previous chunk's fold has read the slot
        kab[slot] = make_float4(ak[0], ak[1], bk[0], bk[1]);
        __builtin_amdgcn_wave_barrier();
      }
      h8 bq[4], bql[4];
      float beta = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t bw[4], bwl[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float4 ab = kab[4 * (4 * kk + e2) + g];   // channels 32g + 8kk + 2e2, +1
          const uint32_t w = qw[4 * kk + e2];
          const float x0 = bf16_lo(w), x1 = bf16_hi(w);
          beta = fmaf(x0, ab.z, fmaf(x1, ab.w, beta));
          const float q0 = x0 * ab.x, q1 = x1 * ab.y;
          // float16 split of the folded query: hi = rtz(q), lo = rtz(q - hi); hi + lo carries
          // ~22 bits of q
          const auto hi = __builtin_amdgcn_cvt_pkrtz(q0, q1);
          if constexpr (GW == 8) {          // columns 0..7 take hi, 8..15 take lo
            const float r0 = fmaf(-(float)hi[0], lo_w, q0), r1 = fmaf(-(float)hi[1], lo_w, q1);
            bw[e2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
          } else {
            bw[e2] = __builtin_bit_cast(uint32_t, hi);
            bwl[e2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(q0 - (float)hi[0], q1 - (float)hi[1]));
          }
        }
        const u32x4v bv4 = {bw[0], bw[1], bw[2], bw[3]};
        bq[kk] = __builtin_bit_cast(h8, bv4);
        if constexpr (GW == 16) {
          const u32x4v bl4 = {bwl[0], bwl[1], bwl[2], bwl[3]};
          bql[kk] = __builtin_bit_cast(h8, bl4);
        }
      }
      beta = wave_sum_g(beta);
      const float hb = GW == 8 ? 0.5f * beta : beta;   // GW 8: each of the two column halves carries half
      // row blocks of 16 tokens of this chunk (a row block holds two chunks of 8 tokens: the
      // lanes of rows 0..7, g < 2, take the first, g >= 2 the second)
      constexpr int MB0 = CT >= 16 ? CT / 16 : 1;
#pragma unroll
      for (int mi = 0; mi < MB0; ++mi) {
        const int mb = CT >= 16 ? k * (CT / 16) + mi : k / 2;
        f4 acc = f4{hb, hb, hb, hb};
        const uint32_t w4[4] = {cur.kw[mb].x, cur.kw[mb].y, cur.kw[mb].z, cur.kw[mb].w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const h8 lk = lookup_row(w4[kk], s_pair, lane4);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lk, bq[kk], acc, 0, 0, 0);
          if constexpr (GW == 16) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lk, bql[kk], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = GW == 8 ? acc[i] + dpp_row_ror8(acc[i]) : acc[i];
          if (CT >= 16) s[4 * mb + i] = v;
          else if ((g >> 1) == (k & 1)) s[4 * mb + i] = v;
        }
      }
    }
    if ((tile + 1) * TILE > seq_len) {   // the sequence ends inside this tile: mask the tail
#pragma unroll
      for (int mb = 0; mb < TILE / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tile * TILE + 16 * mb + 4 * g + i >= seq_len) s[4 * mb + i] = -INFINITY;
    }

    // ---- online softmax (base 2) for the column's head over this tile's tokens; the scores
    //      are in units of 2^-E
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < NS; ++i) mt = fmaxf(mt, s[i]);
    mt = wave_max_g(mt) * su;
    const float m_new = fmaxf(m_run, mt);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    float lrb[TILE / 16];                // per row block: this lane's rows' p
    h8 pt[TILE / 32];
#pragma unroll
    for (int mb = 0; mb < TILE / 16; ++mb) lrb[mb] = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[i], su, -m_new));
      lrb[i >> 2] += p;
      pt[i >> 3][i & 7] = (_Float16)p;
    }
    float lsum_all = 0.0f;
#pragma unroll
    for (int mb = 0; mb < TILE / 16; ++mb) lsum_all += lrb[mb];
    l_run = fmaf(l_run, corr, lsum_all);
    if (__builtin_amdgcn_ballot_w64(corr != 1.0f) != 0) {   // the running max moved for some head
#pragma unroll
      for (int j = 0; j < 8; ++j) o_acc[j] *= corr;
    }
    m_run = m_new;

    // ---- values, per chunk: T^T = L_V (128 x its tokens) * p (its tokens x 16 columns),
    // block j holds d = 8*row + j.  Token pairs (2i, 2i+1) of a k-step are interleaved into
    // pair-table indices per channel.  Then the chunk's value map is undone:
    // o += A_V * T + B_V * sum(p), channel d = 32g + 8i + j.
    // The B operand of k-step ks holds, in lane group g, tokens 32ks + 4g + r (dwords 0, 1) and
    // 32ks + 16 + 4g + r (dwords 2, 3), r = 0..3.
    auto apply_map = [&](int k, const f4 (&tacc)[8], float lt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          const float4 ab = vab[k][4 * (4 * i + j2) + g];   // channels 32g + 8i + 2j2, +1
          o_acc[2 * j2][i] = fmaf(ab.x, tacc[2 * j2][i], fmaf(ab.z, lt, o_acc[2 * j2][i]));
          o_acc[2 * j2 + 1][i] = fmaf(ab.y, tacc[2 * j2 + 1][i], fmaf(ab.w, lt, o_acc[2 * j2 + 1][i]));
        }
      }
    };
    auto value_operands = [&](int ks, h8 (&av)[8]) {
      uint32_t ev[4], od[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w0 = cur.vw[8 * ks + 2 * i], w1 = cur.vw[8 * ks + 2 * i + 1];
        ev[i] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);   // byte k: channel 2k of tokens 2i, 2i+1
        od[i] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);  // byte k: channel 2k+1
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t* src = (j & 1) ? od : ev;
        const u32x4v r = {pair_at(s_pair, lane4, src[0], j >> 1), pair_at(s_pair, lane4, src[1], j >> 1),
                          pair_at(s_pair, lane4, src[2], j >> 1), pair_at(s_pair, lane4, src[3], j >> 1)};
        av[j] = __builtin_bit_cast(h8, r);
      }
    };
    if constexpr (CT >= 32) {
      constexpr int KSC = CT / 32;       // k-steps of 32 tokens per chunk
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        float lk = 0.0f;
#pragma unroll
        for (int mb = k * (CT / 16); mb < (k + 1) * (CT / 16); ++mb) lk += lrb[mb];
        const float lt = wave_sum_g(lk);
        f4 tacc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) tacc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = KSC * k; ks < KSC * (k + 1); ++ks) {
          uint32_t ev[4], od[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = cur.vw[8 * ks + 2 * i], w1 = cur.vw[8 * ks + 2 * i + 1];
            ev[i] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);
            od[i] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t* src = (j & 1) ? od : ev;
            const u32x4v r = {pair_at(s_pair, lane4, src[0], j >> 1), pair_at(s_pair, lane4, src[1], j >> 1),
                              pair_at(s_pair, lane4, src[2], j >> 1), pair_at(s_pair, lane4, src[3], j >> 1)};
            tacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, r), pt[ks], tacc[j], 0, 0, 0);
          }
        }
        apply_map(k, tacc, lt);
      }
    } else {
      // chunks of 16 or 8 tokens: each k-step holds 32 / CT chunks; the table operands of the
      // k-step are formed once and the products run once per chunk, on the probabilities of
      // that chunk's tokens only (the others zeroed: whole dword pairs for a chunk of 16, and
      // for a chunk of 8 also the lane groups of the other half)
      constexpr int CK = 32 / CT;
#pragma unroll
      for (int ks = 0; ks < TILE / 32; ++ks) {
        h8 av[8];
        value_operands(ks, av);
        const u32x4v pw = __builtin_bit_cast(u32x4v, pt[ks]);
#pragma unroll
        for (int c = 0; c < CK; ++c) {
          const int hf = CT == 16 ? c : c >> 1;           // dword pair holding the chunk's tokens
          const bool mine = CT == 16 ? true : (g >> 1) == (c & 1);
          const uint32_t d0 = hf == 0 && mine ? pw[0] : 0u, d1 = hf == 0 && mine ? pw[1] : 0u;
          const uint32_t d2 = hf == 1 && mine ? pw[2] : 0u, d3 = hf == 1 && mine ? pw[3] : 0u;
          const u32x4v pm = {d0, d1, d2, d3};
          const h8 pc = __builtin_bit_cast(h8, pm);
          // this lane's p of the chunk's tokens: row block 2ks + hf, all its rows (CT = 16) or
          // the rows of lane groups (c & 1)*2, +1 (CT = 8)
          const float lt = wave_sum_g(mine ? lrb[2 * ks + hf] : 0.0f);
          f4 tacc[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            tacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[j], pc, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          apply_map(ks * CK + c, tacc, lt);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();   // the next tile rewrites this wave's (A, B) tables
  };

  // tiles t_begin + wave, + WAVES, ...: one tile buffer per wave; the other waves of the SIMD
  // hide each other's load latency (a second buffer would cost a wave's registers)
  TileIn<TILE, CPT> cur;
  for (int tile = t_begin + wave; tile < t_end; tile += WAVES) {
    load_tile(a, b, kvh, tile, toff, cur);
    process(cur, tile);
  }

  // ---- merge the waves, 8 heads at a time (GW 8: columns 0..G-1 hold the result, 8..15
  //      duplicate them; GW 16: column h holds head h)
  l_run = wave_sum_g(l_run);
  __syncthreads();                      // every wave is done with the pair table: reuse its LDS
  float (*s_m)[kMaxGroup] = reinterpret_cast<float (*)[kMaxGroup]>(s_big);
  float (*s_l)[kMaxGroup] = reinterpret_cast<float (*)[kMaxGroup]>(s_big + WAVES * kMaxGroup);
  float (*s_o)[8][kMergeRow] = reinterpret_cast<float (*)[8][kMergeRow]>(s_big + 2 * WAVES * kMaxGroup);
  if (g == 0 && n < GW) { s_m[wave][n] = m_run; s_l[wave][n] = l_run; }
  for (int h0 = 0; h0 < a.G; h0 += 8) {
    if (n >= h0 && n < h0 + 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][n - h0][8 * (4 * g + i) + j + g] = o_acc[j][i];   // d = 32g + 8i + j
    }
    __syncthreads();
    const int nh = min(8, a.G - h0);
    for (int idx = tid; idx < nh * kHeadDim; idx += WAVES * 64) {
      const int hl = idx / kHeadDim, d = idx - hl * kHeadDim, h = h0 + hl;
      float M = s_m[0][h];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) M = fmaxf(M, s_m[w][h]);
      float o = 0.0f, l = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = (s_m[w][h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
        o = fmaf(s_o[w][hl][d + (d >> 5)], f, o);
        l = fmaf(s_l[w][h], f, l);
      }
      float* rec = a.ws + ((size_t)((b * a.Hq + kvh * a.G + h) * a.splits + split)) * (kHeadDim + 2);
      rec[2 + d] = o;
      if (d == 0) { rec[0] = M; rec[1] = l; }
    }
    __syncthreads();                    // the records of these heads are read before the next heads overwrite them
  }
}

// log-sum-exp merge of the context splits: one workgroup per (sequence, query head)
__global__ __launch_bounds__(kHeadDim) void k_attn_combine(AttnArgs a) {
  const int bh = blockIdx.x;       // b * Hq + hq
  const int d = threadIdx.x;
  const float* rec = a.ws + (size_t)bh * a.splits * (kHeadDim + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, rec[(size_t)s * (kHeadDim + 2)]);
  float o = 0.0f, l = 0.0f;
#pragma unroll 8
  for (int s = 0; s < a.splits; ++s) {
    const float* r = rec + (size_t)s * (kHeadDim + 2);
    const float f = (r[0] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(r[0] - M);
    o = fmaf(r[2 + d], f, o);
    l = fmaf(r[1], f, l);
  }
  const float res = l > 0.0f ? o / l : 0.0f;   // an empty context gives 0
  if (a.out_f32) static_cast<float*>(a.out)[(size_t)bh * kHeadDim + d] = res;
  else {
    const uint32_t u = __float_as_uint(res);
    static_cast<uint16_t*>(a.out)[(size_t)bh * kHeadDim + d] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

struct AttnPlan {
  int tile, cpt, splits, tiles_per_split, ntiles;
};

// Tile of the context (a tile lies inside one page): 64 tokens inside one chunk of 64 or
// more; for a chunk of 32, two chunks when the pages hold whole 64-token tiles, else 32 tokens
// of one chunk; for a chunk of 16, four chunks in pages of whole 64-token tiles; for a chunk
// of 8, four chunks of a 32-token tile in pages of whole 32-token tiles; 0 for the shapes the
// kernel does not take.  *cpt = chunks per tile.
int attn_tile(int C, int P, int* cpt) {
  *cpt = 1;
  if (C % 64 == 0) return 64;
  if (C == 32) {
    if (P % 64 == 0) { *cpt = 2; return 64; }
    return 32;
  }
  if (C == 16 && P % 64 == 0) { *cpt = 4; return 64; }
  if (C == 8 && P % 32 == 0) { *cpt = 4; return 32; }
  return 0;
}

// Waves per workgroup for chunks-per-tile cpt and group width gw: 12 (three per SIMD) where
// the registers allow it, 8 where four chunks per tile, or two chunks with 16 heads, need more.
int attn_waves(int cpt, int gw) { return cpt >= 4 || (cpt == 2 && gw == 16) ? 8 : 12; }

template <int GW>
const void* attn_kernel(int tile, int cpt) {
  if (tile == 32) return cpt == 4 ? reinterpret_cast<const void*>(&k_attn_anchor<32, 4, GW, 8>)
                                  : reinterpret_cast<const void*>(&k_attn_anchor<32, 1, GW, 12>);
  if (cpt == 4) return reinterpret_cast<const void*>(&k_attn_anchor<64, 4, GW, 8>);
  if (cpt == 2) return reinterpret_cast<const void*>(&k_attn_anchor<64, 2, GW, GW == 16 ? 8 : 12>);
  return reinterpret_cast<const void*>(&k_attn_anchor<64, 1, GW, 12>);
}

bool attn_plan(int batch, int ctx, int Hq, int Hkv, int D, int P, int C, AttnPlan* pl) {
  if (batch <= 0 || ctx <= 0 || Hq <= 0 || Hkv <= 0 || P <= 0 || C <= 0) return false;
  if (ctx % P != 0 || P % C != 0 || Hq % Hkv != 0) return false;
  pl->tile = attn_tile(C, P, &pl->cpt);
  if (D != kHeadDim || pl->tile == 0 || Hq / Hkv > kMaxGroup) return false;
  pl->ntiles = ctx / pl->tile;
  // One workgroup per compute unit of the 256-CU gfx950 parts (12 or 8 waves fill a CU at
  // this kernel's register use): long-lived workgroups, one table fill and one merge each.
  // The split count minimises rounds of workgroups x tiles per split (ties: fewer splits).
  const long long units = (long long)batch * Hkv;
  long long best_cost = -1;
  for (int want = 1; want <= pl->ntiles && want <= 4096; ++want) {
    const int tps = (pl->ntiles + want - 1) / want;
    const int splits = (pl->ntiles + tps - 1) / tps;            // no empty split
    const long long rounds = (units * splits + kAttnWorkgroups - 1) / kAttnWorkgroups;
    const long long cost = rounds * tps;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      pl->tiles_per_split = tps;
      pl->splits = splits;
    }
  }
  return true;
}

uint16_t f64_to_f16_bits(double x) {
  const _Float16 h = (_Float16)x;     // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace

size_t attn_workspace_bytes(int batch, int ctx, int Hq, int Hkv, int D, int P, int C) {
  AttnPlan pl;
  if (!attn_plan(batch, ctx, Hq, Hkv, D, P, C, &pl)) return 0;
  return (size_t)batch * Hq * pl.splits * (kHeadDim + 2) * sizeof(float);
}

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Every argument check of the anchor attention except those of the workspace: LYNX_OK with
// *need the workspace bytes (0 for an empty batch, which has nothing to do).
int attn_check(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch, int ctx_tokens,
               int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk, float alpha, float sm_scale,
               int out_dtype, const void* out_dev, size_t* need) {
  *need = 0;
  if (batch < 0 || ctx_tokens <= 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 || page_tokens <= 0 ||
      chunk <= 0)
    return LYNX_EINVAL;
  if (ctx_tokens % page_tokens != 0 || page_tokens % chunk != 0 || q_heads % kv_heads != 0) return LYNX_EINVAL;
  if (!std::isfinite(alpha) || !(alpha > 0.0f) || !std::isfinite(sm_scale)) return LYNX_EINVAL;
  if (out_dtype != LYNX_OUT_BF16 && out_dtype != LYNX_OUT_F32) return LYNX_EINVAL;
  int cpt_unused = 0;
  if (head_dim != kHeadDim || attn_tile(chunk, page_tokens, &cpt_unused) == 0 || q_heads / kv_heads > kMaxGroup ||
      batch > 65535 ||
      kv_heads > 65535)
    return LYNX_EUNSUPPORTED;
  if (batch == 0) return LYNX_OK;
  AttnPlan pl;
  if (!attn_plan(batch, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk, &pl)) return LYNX_EINVAL;
  if (!aligned16(q_dev) || !aligned16(k_anchor_dev) || !aligned16(v_anchor_dev) || !aligned16(out_dev))
    return LYNX_EALIGN;
  *need = (size_t)batch * q_heads * pl.splits * (kHeadDim + 2) * sizeof(float);
  return LYNX_OK;
}

// Shared by the contiguous and the paged entry points (block_table == nullptr: contiguous).
int attn_launch(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch, int ctx_tokens,
                int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk, float alpha, float sm_scale,
                void* workspace_dev, size_t ws_bytes, int out_dtype, void* out_dev, const int32_t* block_table,
                const int32_t* seq_lens, int max_pages, int n_pool, hipStream_t stream) {
  size_t need = 0;
  const int st = attn_check(q_dev, k_anchor_dev, v_anchor_dev, batch, ctx_tokens, q_heads, kv_heads, head_dim,
                            page_tokens, chunk, alpha, sm_scale, out_dtype, out_dev, &need);
  if (st != LYNX_OK || batch == 0) return st;
  AttnPlan pl;
  attn_plan(batch, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk, &pl);
  if (!aligned16(workspace_dev)) return LYNX_EALIGN;
  if (ws_bytes < need) return LYNX_ENOSPACE;

  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q_dev);
  a.kanc = static_cast<const uint8_t*>(k_anchor_dev);
  a.vanc = static_cast<const uint8_t*>(v_anchor_dev);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.max_pages = max_pages;
  a.n_pool = n_pool;
  a.ws = static_cast<float*>(workspace_dev);
  a.out = out_dev;
  a.B = batch;
  a.T = ctx_tokens;
  a.Hq = q_heads;
  a.Hkv = kv_heads;
  a.G = q_heads / kv_heads;
  a.P = page_tokens;
  a.C = chunk;
  a.npages = ctx_tokens / page_tokens;
  a.nck = page_tokens / chunk;
  a.H = kv_heads * head_dim;
  a.codes = (long long)page_tokens * a.H / 2;
  a.anc_seg = a.codes + 4ll * a.H * (2 + 2ll * a.nck);
  a.splits = pl.splits;
  a.tiles_per_split = pl.tiles_per_split;
  a.ntiles = pl.ntiles;
  const double scale = sm_scale > 0.0f ? (double)sm_scale : 1.0 / std::sqrt((double)head_dim);
  a.qscale = (float)(scale * 1.4426950408889634);   // log2(e)
  a.out_f32 = out_dtype == LYNX_OUT_F32;
  const double al = (double)alpha, L = std::log1p(al);
  uint16_t lut[16];
  for (int nib = 0; nib < 16; ++nib) {
    const int qv = nib >= 8 ? nib - 16 : nib;                 // Q_anc
    const int S = qv < 0 ? -1 : 1, vmag = qv < 0 ? -qv - 1 : qv;
    const double mag = std::expm1((double)(16 * vmag + 7) / kCodeMax * L) / al;
    lut[nib] = f64_to_f16_bits(S * mag);
  }
  for (int bt = 0; bt < 256; ++bt) a.pair[bt] = (uint32_t)lut[bt & 15] | ((uint32_t)lut[bt >> 4] << 16);
  void* kargs[] = {&a};
  // query groups of up to 8 heads: two MFMA columns per head (float16 high / low parts of the
  // folded query); up to 16: one column per head
  const void* fn = a.G <= 8 ? attn_kernel<8>(pl.tile, pl.cpt) : attn_kernel<16>(pl.tile, pl.cpt);
  hipError_t e = hipLaunchKernel(fn,
                                 dim3((unsigned)pl.splits, (unsigned)kv_heads, (unsigned)batch),
                                 dim3(attn_waves(pl.cpt, a.G <= 8 ? 8 : 16) * 64), kargs, 0, stream);
  if (e != hipSuccess) return LYNX_ELAUNCH;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&k_attn_combine), dim3((unsigned)(batch * q_heads)),
                      dim3(kHeadDim), kargs, 0, stream);
  return e == hipSuccess ? LYNX_OK : LYNX_ELAUNCH;
}

}  // namespace

int attn_anchor_launch(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch,
                       int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                       float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype,
                       void* out_dev, hipStream_t stream) {
  return attn_launch(q_dev, k_anchor_dev, v_anchor_dev, batch, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens,
                     chunk, alpha, sm_scale, workspace_dev, ws_bytes, out_dtype, out_dev, nullptr, nullptr, 0, 0,
                     stream);
}

int attn_anchor_paged_launch(const void* q_dev, const void* k_anchor_pool, const void* v_anchor_pool, int n_pool,
                             const int32_t* block_table, const int32_t* seq_lens, int batch, int max_pages,
                             int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk, float alpha,
                             float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype, void* out_dev,
                             hipStream_t stream) {
  if (n_pool <= 0 || max_pages <= 0 || page_tokens <= 0) return LYNX_EINVAL;
  if ((long long)max_pages * page_tokens > 0x7fffffffll) return LYNX_EUNSUPPORTED;
  auto al4 = [](const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (!al4(block_table) || !al4(seq_lens)) return LYNX_EALIGN;
  return attn_launch(q_dev, k_anchor_pool, v_anchor_pool, batch, max_pages * page_tokens, q_heads, kv_heads,
                     head_dim, page_tokens, chunk, alpha, sm_scale, workspace_dev, ws_bytes, out_dtype, out_dev,
                     block_table, seq_lens, max_pages, n_pool, stream);
}

// ---------------------------------------------------------------------------
// The anchor attention without caller workspace: its split-context partial records go to
// `scratch`, a device array of LYNX_ATTN_SCRATCH_BYTES that every GPU the library runs on holds
// for the life of the process.  In host code `scratch` names a host-side stand-in, not the
// device memory: its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to the kernels.  No allocation happens.
// Every record the combine pass reads is written by the attention kernel of the same call, so
// nothing needs clearing; calls that overlap on one GPU (on different streams) share the array
// and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[LYNX_ATTN_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of the current device's `scratch`, looked up on the first call on that device.
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return LYNX_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LYNX_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return LYNX_OK;
}

}  // namespace

int attn_anchor_noalloc_launch(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev, int batch,
                               int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                               float alpha, float sm_scale, int out_dtype, void* out_dev, hipStream_t stream) {
  // every argument error first, on the host; then the records this shape needs against the buffer
  size_t need = 0;
  int st = attn_check(q_dev, k_anchor_dev, v_anchor_dev, batch, ctx_tokens, q_heads, kv_heads, head_dim,
                      page_tokens, chunk, alpha, sm_scale, out_dtype, out_dev, &need);
  if (st != LYNX_OK || batch == 0) return st;
  if (need > (size_t)LYNX_ATTN_SCRATCH_BYTES) return LYNX_ENOSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != LYNX_OK) return st;
  return attn_launch(q_dev, k_anchor_dev, v_anchor_dev, batch, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens,
                     chunk, alpha, sm_scale, ws, need, out_dtype, out_dev, nullptr, nullptr, 0, 0, stream);
}

}  // namespace lynx
