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
// Decomposition: one workgroup (8 waves) per (sequence, kv head, block of 256 query
// rows, context split); query row r = m*G + h (draft token m, query head h of the
// group); each wave owns 32 rows as two MFMA column groups of 16.  The context is
// walked in 64-token tiles (a tile lies inside one page and holds one chunk of 64 or
// more, or 2 or 4 whole chunks of 32 or 16 tokens, each token decoded with the map of its
// own chunk).  Each tile is decoded once into LDS for all rows:
//   * keys as K_hat * scale * log2(e) in float32, stored as BF16 high and low parts
//     (K_hat ~ hi + lo to 16 bits), row-major [token][channel];
//   * values as V_hat * 2^-E in float16 (E a power-of-two range exponent, 0 for ordinary
//     KV), transposed [channel][token] in the k order of the value MFMA's operand;
// the decode of tile i+1 runs in the same step as the products over tile i (two LDS
// buffers, one barrier per tile).  Per tile and wave:
//   scores  S^T[token, row] = K_hi q + K_lo q on MFMA 16x16x32 bf16 (the BF16 query
//           is exact in this format); each key fragment read feeds both groups;
//   online softmax in base 2 per row, the running maximum moved only when a tile
//           raises it by more than 8 or a lane's sum of its 16 probabilities of the tile
//           reaches 2^12 (so probabilities stay below 2^12, exact in range);
//   values  O^T[d, row] += sum_t V_hat[d, t] p[t, row] on MFMA 16x16x32 f16, o held in
//           units of 2^E.
// LDS traffic bounds this loop: per 64-token tile a workgroup reads 48 KB of key and
// value operands per wave (384 KB) and moves ~176 KB in the decode, against ~128 B per
// clock; the layout keeps every product operand one 16-byte read and the key buffers
// within the 64 KB reach of an LDS instruction's immediate offset.
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
typedef __bf16 vb2 __attribute__((ext_vector_type(2)));
typedef _Float16 vh2 __attribute__((ext_vector_type(2)));
typedef float vf2 __attribute__((ext_vector_type(2)));
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef uint32_t vu4 __attribute__((ext_vector_type(4)));

constexpr int kVWaves = 8;                 // waves per workgroup
constexpr int kVThreads = kVWaves * 64;
constexpr int kVGroups = 2;                // MFMA column groups (16 rows each) per wave
constexpr int kVRows = 16 * kVGroups * kVWaves;   // query rows per workgroup (256)
static_assert(kVThreads == 512, "the tile decode maps 512 threads onto 64 tokens x 128 channels");
constexpr int kVTile = 64;                 // context tokens per step
constexpr int kLutCopies = 32;             // copies of each table entry (lane l reads copy l % 32)
constexpr int kRec = kHeadDim + 4;         // floats per partial record (o 16-byte aligned)
constexpr int kVWorkgroups = 256;          // workgroups the context splits aim for (one per CU)
constexpr float kLazyMax = 8.0f;           // the running maximum moves only beyond this (base 2)
constexpr float kLazySumBound = 4096.0f;   // bound on a lane's sum of its 16 probabilities of a tile
constexpr float kF16Safe = 60000.0f;       // largest |value| stored as float16 (maximum 65504)

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
  // paged form: sequence b's page p is pool segment block_table[b * max_pages + p] (clamped
  // into [0, n_pool)) of both streams, and only its first seq_lens[b] tokens (clamped into
  // [0, npages * P]) count.  Contiguous form: both null, segment b * npages + p.
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_pages, n_pool;
  float lut32[256];                        // S|x| of the full code n = anchor | residual << 4
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

// BF16 pair (round to nearest even, one v_cvt_pk_bf16_f32) of two floats, lo = a
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  const vf2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, vb2));
}


// One tile's raw codes for this thread.
struct CodeIn {
  uint32_t ka[2], kr[2]; // key codes: tokens tid/16 and tid/16 + 32, channels 8*(tid%16) .. +7
  uint32_t va[2], vr[2]; // value codes: tokens 2*(tid%32), +1; channels 8*(tid/32) .. +7
};

struct TileAddr {
  size_t seg;     // segment index of the tile's page
  size_t row0;    // byte offset of the tile's first code row in block 0 of this kv head
  int kc;         // chunk of the tile within its page
};

// Block-table entry of `tile`'s page (paged form; 0 otherwise), fetched a step ahead of its use
// as a vector load: fetched at its use, the wait for it would also wait for every load issued
// before it (the loads of a wave complete in order).
__device__ __forceinline__ int fetch_segment(const VerifyArgs& a, int b, int tile) {
  if (a.block_table == nullptr) return 0;
  return __builtin_nontemporal_load(a.block_table + (size_t)b * a.max_pages + tile * kVTile / a.P);
}

__device__ __forceinline__ TileAddr tile_addr(const VerifyArgs& a, int b, int kvh, int tile, int fetched) {
  const int tok = tile * kVTile;
  const int page = tok / a.P;
  const int tin = tok - page * a.P;
  TileAddr t;
  if (a.block_table == nullptr) {
    t.seg = (size_t)b * a.npages + page;
  } else {
    t.seg = (size_t)min(max(__builtin_amdgcn_readfirstlane(fetched), 0), a.n_pool - 1);
  }
  t.row0 = code_offset(a.P, kvh, 0, tin);
  t.kc = tin / a.C;
  return t;
}

__device__ __forceinline__ void load_codes(const VerifyArgs& a, int b, int kvh, int tile, int fetched, int tid,
                                           CodeIn& in) {
  const TileAddr ta = tile_addr(a, b, kvh, tile, fetched);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    // channels 8*(tid%16) .. +7: code block (tid%16)/8, dword tid%8 of the row of token tid/16 + 32r
    const size_t off = ta.row0 + (size_t)((tid & 15) >> 3) * a.P * kCodeRow + (size_t)((tid >> 4) + 32 * r) * kCodeRow +
                       4 * (tid & 7);
    in.ka[r] = *reinterpret_cast<const uint32_t*>(a.kanc + ta.seg * a.anc_seg + off);
    in.kr[r] = *reinterpret_cast<const uint32_t*>(a.kres + ta.seg * a.codes + off);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    // channels 8*(tid/32) .. +7: code block tid/256, dword (tid/32)%8 of its row
    const size_t off = ta.row0 + (size_t)(tid >> 8) * a.P * kCodeRow + (size_t)(2 * (tid & 31) + r) * kCodeRow +
                       4 * ((tid >> 5) & 7);
    in.va[r] = *reinterpret_cast<const uint32_t*>(a.vanc + ta.seg * a.anc_seg + off);
    in.vr[r] = *reinterpret_cast<const uint32_t*>(a.vres + ta.seg * a.codes + off);
  }
}

// gamma_min, gamma_scale, mu and sigma of channels 2l, 2l+1 of the tile's CPT chunks, for
// lane l of wave 0 (keys) or wave 1 (values)
// (each channel pair held as one 64-bit value, so that its two halves stay one register pair
// from the load to the use: split, a copy of one half made the wave wait for the load right
// after issuing it)
template <int CPT>
struct MetaIn {
  uint64_t gmin, gscale, mu[CPT], sigma[CPT];
};
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

template <int CPT>
__device__ __forceinline__ MetaIn<CPT> load_meta(const VerifyArgs& a, int b, int kvh, int tile, int fetched,
                                                 int wave, int lane) {
  const TileAddr ta = tile_addr(a, b, kvh, tile, fetched);
  const uint8_t* seg = (wave == 0 ? a.kanc : a.vanc) + ta.seg * a.anc_seg + a.codes;
  const float* meta = reinterpret_cast<const float*>(seg) + kvh * kHeadDim + 2 * lane;
  MetaIn<CPT> m;
  m.gmin = *reinterpret_cast<const uint64_t*>(meta);
  m.gscale = *reinterpret_cast<const uint64_t*>(meta + a.H);
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    m.mu[k] = *reinterpret_cast<const uint64_t*>(meta + 2 * (size_t)a.H + (size_t)(ta.kc + k) * a.H);
    m.sigma[k] = *reinterpret_cast<const uint64_t*>(meta + 2 * (size_t)a.H + (size_t)(a.nck + ta.kc + k) * a.H);
  }
  return m;
}

// (A, B) of one channel; the key map carries the softmax scale
__device__ __forceinline__ float2 affine(float gmin, float gscale, float mu, float sigma, float scale) {
  const float d1 = gscale + (float)kEps, d2 = sigma + (float)kEps;
  return make_float2(d1 * d2 * scale, fmaf(mu, d1, gmin) * scale);
}

// CPT = chunks per 64-token tile (1 for a chunk of 64 or more, 2 / 4 for chunks of 32 / 16)
template <int CPT>
struct alignas(16) VerifyLds {
  // the key parts first: the products' reads of both buffers then sit within the 64 KB reach of
  // an LDS instruction's immediate offset
  uint32_t kh[2][kVTile * 64];             // K_hat BF16 high parts, [token][channel pair], per buffer
  uint32_t kl[2][kVTile * 64];             // K_hat BF16 low parts
  uint32_t lv[2][kHeadDim * (kVTile / 2)]; // V_hat * 2^-E as float16, [channel][token slot]
  float lut[256 * kLutCopies];             // float32 table, entry e copy c at e*32 + c
  float2 abk[2][CPT][kHeadDim + kHeadDim / 16];  // (A_K, B_K) of channel c at c + c/16, scaled
  float2 abv[2][CPT][kHeadDim];            // (A_V, B_V) 2^-E per channel
  int vexp[2];                             // E of the tile in each slot
};

// Value rows: row d holds the 64 tokens of channel d in eight 16-byte slots.  Slot 4ks + g holds
// tokens 32ks + 4g + 0..3 then 32ks + 16 + 4g + 0..3, the k order of one lane's f16 MFMA operand
// (the layout of the probabilities), so that the operand is one 16-byte read; slot s sits at
// s ^ ((d >> 1) & 7), which puts the 16 rows one read spans on distinct banks.  Word of the
// token pair 2tp, 2tp + 1 of channel d:
__device__ __forceinline__ int lv_word(int d, int tp) {
  const int slot = 4 * (tp >> 4) + ((tp >> 1) & 3);
  return d * (kVTile / 2) + 4 * (slot ^ ((d >> 1) & 7)) + 2 * ((tp >> 3) & 1) + (tp & 1);
}

// Smallest e >= 0 with (|A| + |B|) 2^-e <= kF16Safe: a bound on |V_hat| 2^-e over the chunk,
// since |L| <= 1.
__device__ __forceinline__ int value_exponent(float2 ab) {
  const float bound = fabsf(ab.x) + fabsf(ab.y);
  if (bound <= kF16Safe) return 0;
  if (!(bound < INFINITY)) return 126;
  // bound = m 2^x with m in [0.5, 1), kF16Safe = ms 2^16 (ms = 60000 / 65536, exact): e = x - 16
  // when m <= ms, else x - 15
  int x;
  const float m = frexpf(bound, &x);
  return x - 16 + (m > kF16Safe / 65536.0f ? 1 : 0);
}

// Maps of one tile into slot `buf`: wave 0 writes the key maps of channels 2l, 2l+1, wave 1
// the value maps, scaled by 2^-E with E the running maximum of the tiles' range exponents
// (held in E_map by wave 1).
template <int CPT>
__device__ __forceinline__ void write_maps(VerifyLds<CPT>& L, int buf, const MetaIn<CPT>& m, float qscale,
                                           int wave, int l, int& E_map) {
  if (wave == 0) {
    const int c = 2 * l + (l >> 3);       // channel 2l at 2l + 2l/16
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      L.abk[buf][k][c] = affine(lo_f(m.gmin), lo_f(m.gscale), lo_f(m.mu[k]), lo_f(m.sigma[k]), qscale);
      L.abk[buf][k][c + 1] = affine(hi_f(m.gmin), hi_f(m.gscale), hi_f(m.mu[k]), hi_f(m.sigma[k]), qscale);
    }
  } else {
    float2 ab0[CPT], ab1[CPT];
    int e = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      ab0[k] = affine(lo_f(m.gmin), lo_f(m.gscale), lo_f(m.mu[k]), lo_f(m.sigma[k]), 1.0f);
      ab1[k] = affine(hi_f(m.gmin), hi_f(m.gscale), hi_f(m.mu[k]), hi_f(m.sigma[k]), 1.0f);
      e = max(e, max(value_exponent(ab0[k]), value_exponent(ab1[k])));
    }
    if (__builtin_amdgcn_ballot_w64(e > E_map) != 0) {   // values beyond the range so far: rare
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) e = max(e, __shfl_xor(e, sh));
      E_map = max(E_map, e);
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (E_map != 0) {
        ab0[k] = make_float2(ldexpf(ab0[k].x, -E_map), ldexpf(ab0[k].y, -E_map));
        ab1[k] = make_float2(ldexpf(ab1[k].x, -E_map), ldexpf(ab1[k].y, -E_map));
      }
      *reinterpret_cast<float4*>(&L.abv[buf][k][2 * l]) = make_float4(ab0[k].x, ab0[k].y, ab1[k].x, ab1[k].y);
    }
    if (l == 0) L.vexp[buf] = E_map;
  }
}

// Decode this thread's part of one tile into buffer `buf` (maps of slot `buf`; a tile of CPT
// chunks takes the map of each token's chunk).
template <int CPT>
__device__ __forceinline__ void decode_tile(VerifyLds<CPT>& L, int buf, const CodeIn& in, int tid, int lcopy) {
  {
    // keys: tokens tid/16 and tid/16 + 32, channels 8*(tid%16) + k, K_hat = A*L + B split into
    // BF16 hi + lo; row t holds 16 columns of 16 B (8 channels each), column c16 at c16 ^ (t & 15),
    // so the 16 lanes of one token write its whole row.  A thread reads the maps of its 8 channels
    // once for both tokens (twice when they fall in different chunks).
    const int cu = tid & 15, t0 = tid >> 4;
    // the BF16 pairs (-1, 0) and (0, -1) from registers (an inline constant of a packed BF16
    // operand is not read as such a pair)
    uint32_t nlo = 0x0000BF80u, nhi = 0xBF800000u;
    asm volatile("" : "+v"(nlo), "+v"(nhi));
    const vb2 neg_lo = __builtin_bit_cast(vb2, nlo), neg_hi = __builtin_bit_cast(vb2, nhi);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t = t0 + 32 * r;
      // the padding spreads the 16 channel units' maps over distinct banks
      const float2* abk = L.abk[buf][CPT == 1 ? 0 : t / (kVTile / CPT)];
      // byte k of ev / od: full code of channel 8cu + 2k / 2k+1
      const uint32_t ev = (in.ka[r] & 0x0F0F0F0Fu) | ((in.kr[r] << 4) & 0xF0F0F0F0u);
      const uint32_t od = ((in.ka[r] >> 4) & 0x0F0F0F0Fu) | (in.kr[r] & 0xF0F0F0F0u);
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ch = 8 * cu + 2 * k;
        const float2 ab0 = abk[ch + (ch >> 4)], ab1 = abk[ch + 1 + (ch >> 4)];
        const float x0 = fmaf(ab0.x, L.lut[((ev >> (8 * k)) & 0xFFu) * kLutCopies + lcopy], ab0.y);
        const float x1 = fmaf(ab1.x, L.lut[((od >> (8 * k)) & 0xFFu) * kLutCopies + lcopy], ab1.y);
        const uint32_t h = bf16x2(x0, x1);
        hi[k] = h;
        // x - hi, exact in float32, as a dot product of the BF16 pair with (-1, 0) / (0, -1)
        const vb2 hv = __builtin_bit_cast(vb2, h);
        lo[k] = bf16x2(__builtin_amdgcn_fdot2_f32_bf16(hv, neg_lo, x0, false),
                       __builtin_amdgcn_fdot2_f32_bf16(hv, neg_hi, x1, false));
      }
      const int c16 = cu ^ (t & 15);
      *reinterpret_cast<uint4*>(&L.kh[buf][t * 64 + 4 * c16]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      *reinterpret_cast<uint4*>(&L.kl[buf][t * 64 + 4 * c16]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  {
    // values: channels 8*(tid/32) + j, tokens 2*(tid%32), +1: V_hat = A*L + B (times 2^-E)
    // as float16 pairs, transposed into the slots of lv_word.
    const int c8 = tid >> 5, tq = tid & 31;
    const uint32_t ev0 = (in.va[0] & 0x0F0F0F0Fu) | ((in.vr[0] << 4) & 0xF0F0F0F0u);
    const uint32_t od0 = ((in.va[0] >> 4) & 0x0F0F0F0Fu) | (in.vr[0] & 0xF0F0F0F0u);
    const uint32_t ev1 = (in.va[1] & 0x0F0F0F0Fu) | ((in.vr[1] << 4) & 0xF0F0F0F0u);
    const uint32_t od1 = ((in.va[1] >> 4) & 0x0F0F0F0Fu) | (in.vr[1] & 0xF0F0F0F0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sh = 8 * (j >> 1);
      const uint32_t i0 = (((j & 1) ? od0 : ev0) >> sh) & 0xFFu;
      const uint32_t i1 = (((j & 1) ? od1 : ev1) >> sh) & 0xFFu;
      const int d = 8 * c8 + j;
      const float2 ab = L.abv[buf][CPT == 1 ? 0 : tq / (kVTile / 2 / CPT)][d];   // the tokens' chunk
      const vf2 x = {fmaf(ab.x, L.lut[i0 * kLutCopies + lcopy], ab.y), fmaf(ab.x, L.lut[i1 * kLutCopies + lcopy], ab.y)};
      L.lv[buf][lv_word(d, tq)] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, vh2));
    }
  }
}

}  // namespace

template <int CPT>
__global__ __launch_bounds__(kVThreads) void k_verify(VerifyArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int b = blockIdx.z / a.rowblocks, rb = blockIdx.z - b * a.rowblocks;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  __shared__ VerifyLds<CPT> L;

  for (int i = tid; i < 256 * kLutCopies; i += kVThreads) L.lut[i] = a.lut32[i / kLutCopies];
  const int lcopy = tid & (kLutCopies - 1);

  // this wave's query rows: group gq of the wave, column n; BF16 operand channels 32kk + 8g .. +7
  const int row_base = rb * kVRows + wave * (16 * kVGroups);
  const bool wave_live = row_base < a.R;                  // wave-uniform
  vb8 qop[kVGroups][4];
#pragma unroll
  for (int gq = 0; gq < kVGroups; ++gq) {
    const int row = row_base + 16 * gq + n;
    const bool live = row < a.R;
    const int m = live ? row / a.G : 0, hh = live ? row - m * a.G : 0;
    const uint16_t* qp = a.q + ((size_t)(b * a.M + m) * a.Hq + kvh * a.G + hh) * kHeadDim + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + 32 * kk);
      if (!live) w = make_uint4(0u, 0u, 0u, 0u);
      const vu4 wv = {w.x, w.y, w.z, w.w};
      qop[gq][kk] = __builtin_bit_cast(vb8, wv);
    }
  }

  // Online softmax state per row (base 2).  The key products start from -m_run, so they
  // yield s - m_run directly; m_run moves only when a tile exceeds it by more than
  // kLazyMax or a lane's probabilities of a tile sum to kLazySumBound or more.  o_acc is held
  // in units of 2^E_acc (the values' range exponent).
  float m_run[kVGroups], l_run[kVGroups];
  vf4 cinit[kVGroups];
  vf4 o_acc[kVGroups][8];
#pragma unroll
  for (int gq = 0; gq < kVGroups; ++gq) {
    m_run[gq] = -INFINITY;
    l_run[gq] = 0.0f;
    cinit[gq] = vf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) o_acc[gq][j] = vf4{0.f, 0.f, 0.f, 0.f};
  }
  int E_acc = 0;

  // this sequence's context: all tiles, or its own length in the paged form
  const int seq_len = a.seq_lens == nullptr ? a.ntiles * kVTile : min(max(a.seq_lens[b], 0), a.ntiles * kVTile);
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min((seq_len + kVTile - 1) / kVTile, t_begin + a.tiles_per_split);
  const int t_last = t_end - 1;         // loads past the split's end re-read its last tile (unused)
  const int nt = t_end - t_begin;       // workgroup-uniform; <= 0 past a short sequence: no tiles
  if (nt > 0) {

  // prologue: maps of tiles 0 and 1, codes of tiles 0 and 1, tile 0 decoded into buffer 0
  const bool mapper = wave < 2;          // wave-uniform: wave 0 keys, wave 1 values
  int E_map = 0;
  const int f0 = fetch_segment(a, b, t_begin), f1 = fetch_segment(a, b, min(t_begin + 1, t_last));
  int f_cur = fetch_segment(a, b, min(t_begin + 2, t_last));   // the tile whose codes step i loads: i + 2
  if (mapper) {
    write_maps(L, 0, load_meta<CPT>(a, b, kvh, t_begin, f0, wave, lane), a.qscale, wave, lane, E_map);
    write_maps(L, 1, load_meta<CPT>(a, b, kvh, min(t_begin + 1, t_last), f1, wave, lane), a.qscale, wave, lane,
               E_map);
  }
  CodeIn cin;
  load_codes(a, b, kvh, t_begin, f0, tid, cin);
  __syncthreads();                       // the table and the maps of tiles 0 and 1 are in LDS
  E_acc = L.vexp[0];
  decode_tile(L, 0, cin, tid, lcopy);
  load_codes(a, b, kvh, min(t_begin + 1, t_last), f1, tid, cin);

  // step i (buffer par = i & 1): decode tile i+1 into the other buffer, products over tile i,
  // maps of tile i+2 into slot par
  auto step = [&](int i, int par) {
    __syncthreads();   // buffer par is decoded; buffer 1-par and maps slot par are free
    const int f_next = fetch_segment(a, b, min(t_begin + i + 3, t_last));
    decode_tile(L, 1 - par, cin, tid, lcopy);
    // the metadata of tile i+2 (written as maps at the end of this step: loaded and used within one
    // step, so that no copy of it crosses the loop) ahead of its codes
    MetaIn<CPT> meta;
    if (mapper) meta = load_meta<CPT>(a, b, kvh, min(t_begin + i + 2, t_last), f_cur, wave, lane);
    load_codes(a, b, kvh, min(t_begin + i + 2, t_last), f_cur, tid, cin);

    if (wave_live) {
      // ---- scores minus m_run, S^T[token, row] of both groups: tokens 16mb + 4g + e, row n
      float s[kVGroups][16];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        vf4 acc[kVGroups];
#pragma unroll
        for (int gq = 0; gq < kVGroups; ++gq) acc[gq] = cinit[gq];
        const int t = 16 * mb + n;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int c16 = (4 * kk + g) ^ n;          // (t & 15) == n
          const uint4 wh = *reinterpret_cast<const uint4*>(&L.kh[par][t * 64 + 4 * c16]);
          const uint4 wl = *reinterpret_cast<const uint4*>(&L.kl[par][t * 64 + 4 * c16]);
          const vu4 vh = {wh.x, wh.y, wh.z, wh.w}, vl = {wl.x, wl.y, wl.z, wl.w};
#pragma unroll
          for (int gq = 0; gq < kVGroups; ++gq) {
            acc[gq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vb8, vh), qop[gq][kk], acc[gq], 0, 0, 0);
            acc[gq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(vb8, vl), qop[gq][kk], acc[gq], 0, 0, 0);
          }
        }
#pragma unroll
        for (int gq = 0; gq < kVGroups; ++gq)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[gq][4 * mb + e] = acc[gq][e];
        __builtin_amdgcn_sched_barrier(0);   // bound the key fragments held in registers
      }
      if ((t_begin + i + 1) * kVTile > seq_len) {   // the sequence ends inside this tile: mask the tail
        const int tok0 = (t_begin + i) * kVTile;
#pragma unroll
        for (int gq = 0; gq < kVGroups; ++gq)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (tok0 + 16 * (e >> 2) + 4 * g + (e & 3) >= seq_len) s[gq][e] = -INFINITY;
      }

      // ---- the value operands of the tile, read ahead of the softmax (which hides their latency):
      //      lane (n, g) of step ks takes channel 16j + n, slot 4ks + g
      //      ((d >> 1) & 7 == (n >> 1) & 7, so block j is a constant offset from two lane bases)
      const uint32_t* vbase0 = &L.lv[par][n * (kVTile / 2) + 4 * (g ^ ((n >> 1) & 7))];
      const uint32_t* vbase1 = &L.lv[par][n * (kVTile / 2) + 4 * ((4 + g) ^ ((n >> 1) & 7))];
      auto vread = [&](int j, int ks) {
        const uint4 w = *reinterpret_cast<const uint4*>((ks ? vbase1 : vbase0) + 16 * (kVTile / 2) * j);
        return vu4{w.x, w.y, w.z, w.w};
      };

      // ---- online softmax: p = 2^(s - m_run) as is while every lane's sum of its 16 p stays
      //      below kLazySumBound (so every p does), with no tile maximum taken; otherwise (rare,
      //      and on the first tile) the row's maximum moves to the tile's where the tile exceeds
      //      it by more than kLazyMax or a lane sum reached the bound, o and l are rescaled and p
      //      is taken again
      vh8 pt[kVGroups][2];
#pragma unroll
      for (int gq = 0; gq < kVGroups; ++gq) {
        float p[16];
        float lsum = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = __builtin_amdgcn_exp2f(s[gq][e]);
          lsum += p[e];
        }
        const bool ok = lsum < kLazySumBound && m_run[gq] != -INFINITY;
        if (__builtin_amdgcn_ballot_w64(!ok) != 0) {
          float mt = s[gq][0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[gq][e]);
          mt = group_max(mt);                               // tile maximum minus m_run (or itself)
          const bool big = group_max(ok ? 0.0f : 1.0f) != 0.0f;   // some lane of the row failed
          const float base = m_run[gq] == -INFINITY ? 0.0f : m_run[gq];
          const bool up = mt + base > m_run[gq] + kLazyMax || (big && mt != -INFINITY);
          if (up) {
            const float corr = __builtin_amdgcn_exp2f(m_run[gq] - (mt + base));
            m_run[gq] = mt + base;
            cinit[gq] = vf4{-m_run[gq], -m_run[gq], -m_run[gq], -m_run[gq]};
            l_run[gq] *= corr;
#pragma unroll
            for (int j = 0; j < 8; ++j) o_acc[gq][j] *= corr;
            lsum = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              p[e] = __builtin_amdgcn_exp2f(s[gq][e] - mt);
              lsum += p[e];
            }
          }
        }
        l_run[gq] += lsum;
#pragma unroll
        for (int e = 0; e < 16; ++e) pt[gq][e >> 3][e & 7] = (_Float16)p[e];
      }

      // ---- values: O^T[d, row] += sum_t V_hat[d, t] p[t, row], d = 16j + 4g + e of block j.
      // The k index of step ks runs over tokens 32ks + 4g + 0..3 then 32ks + 16 + 4g + 0..3
      // (the layout of the probabilities); the values are read in the same order.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const vu4 v0 = vread(j, 0), v1 = vread(j, 1);
#pragma unroll
        for (int gq = 0; gq < kVGroups; ++gq)
          o_acc[gq][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vh8, v0), pt[gq][0], o_acc[gq][j], 0, 0, 0);
#pragma unroll
        for (int gq = 0; gq < kVGroups; ++gq)
          o_acc[gq][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(vh8, v1), pt[gq][1], o_acc[gq][j], 0, 0, 0);
        if (j % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // bound the value operands held in registers
      }
    }

    // ---- o in the units of tile i+1 (rare: the values' range grew)
    const int E_nxt = L.vexp[1 - par];
    if (E_nxt > E_acc) {
#pragma unroll
      for (int gq = 0; gq < kVGroups; ++gq)
#pragma unroll
        for (int j = 0; j < 8; ++j) o_acc[gq][j] *= ldexpf(1.0f, E_acc - E_nxt);
      E_acc = E_nxt;
    }
    // ---- maps of tile i+2 into slot par (read by the decode in step i+1)
    if (mapper) {
      write_maps(L, par, meta, a.qscale, wave, lane, E_map);
    }
    f_cur = f_next;
  };

  for (int i = 0; i < nt; i += 2) {
    step(i, 0);
    if (i + 1 < nt) step(i + 1, 1);
  }
  }   // nt > 0

  // ---- this split's partial records for the lane's rows: (m, l, o[d]) with d = 16j + 4g + e
  const float oscale = ldexpf(1.0f, E_acc);
#pragma unroll
  for (int gq = 0; gq < kVGroups; ++gq) {
    const float l = group_sum(l_run[gq]);
    const int row = row_base + 16 * gq + n;
    if (row < a.R) {
      const int m = row / a.G, hh = row - m * a.G;
      float* rec = a.ws + ((size_t)((b * a.M + m) * a.Hq + kvh * a.G + hh) * a.splits + split) * kRec;
      if (g == 0) *reinterpret_cast<float4*>(rec) = make_float4(m_run[gq], l, 0.0f, 0.0f);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4*>(rec + 4 + 16 * j + 4 * g) =
            make_float4(o_acc[gq][j][0] * oscale, o_acc[gq][j][1] * oscale, o_acc[gq][j][2] * oscale,
                        o_acc[gq][j][3] * oscale);
    }
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
  const float res = l > 0.0f ? o / l : 0.0f;   // an empty context gives 0 (and LSE -inf)
  if (a.out_f32) static_cast<float*>(a.out)[(size_t)row * kHeadDim + d] = res;
  else {
    const uint32_t u = __float_as_uint(res);
    static_cast<uint16_t*>(a.out)[(size_t)row * kHeadDim + d] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
  // natural-log LSE of the scaled scores: the partials are in base 2
  if (a.lse && d == 0) a.lse[row] = l > 0.0f ? (M2 + __log2f(l)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

// Chunks per 64-token tile: 1 for a chunk that is a multiple of 64, 2 for a chunk of 32 in
// pages of a multiple of 64 tokens (a tile then holds two whole chunks of one page); 0 otherwise.
int verify_cpt(int C, int P) {
  if (C > 0 && C % kVTile == 0) return 1;
  if (P % kVTile != 0) return 0;
  if (C == kVTile / 2) return 2;
  if (C == kVTile / 4) return 4;     // chunks of 8 would need 34 KB of maps: beyond the LDS
  return 0;
}

struct VerifyPlan {
  int rowblocks, splits, tiles_per_split, ntiles;
};

bool verify_plan(int batch, int n_query, int ctx, int Hq, int Hkv, int D, int P, int C, VerifyPlan* pl) {
  if (batch <= 0 || n_query <= 0 || ctx <= 0 || Hq <= 0 || Hkv <= 0 || P <= 0 || C <= 0) return false;
  if (ctx % P != 0 || P % C != 0 || Hq % Hkv != 0) return false;
  if (D != kHeadDim || verify_cpt(C, P) == 0) return false;
  const long long R = (long long)n_query * (Hq / Hkv);
  pl->rowblocks = (int)((R + kVRows - 1) / kVRows);
  pl->ntiles = ctx / kVTile;
  // Split the context so that rounds of kVWorkgroups workgroups x tiles per split is least
  // (ties: fewer splits, less merging).
  const long long units = (long long)batch * Hkv * pl->rowblocks;
  long long best_cost = -1;
  for (int want = 1; want <= pl->ntiles && want <= 4096; ++want) {
    const int tps = (pl->ntiles + want - 1) / want;
    const int splits = (pl->ntiles + tps - 1) / tps;
    const long long rounds = (units * splits + kVWorkgroups - 1) / kVWorkgroups;
    const long long cost = rounds * tps;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      pl->tiles_per_split = tps;
      pl->splits = splits;
    }
  }
  return true;
}

}  // namespace

size_t verify_workspace_bytes(int batch, int n_query, int ctx, int Hq, int Hkv, int D, int P, int C) {
  VerifyPlan pl;
  if (!verify_plan(batch, n_query, ctx, Hq, Hkv, D, P, C, &pl)) return 0;
  return (size_t)batch * n_query * Hq * pl.splits * kRec * sizeof(float);
}

namespace {

int verify_launch_common(const void* q_dev, const void* k_anchor_dev, const void* k_residual_dev,
                         const void* v_anchor_dev, const void* v_residual_dev, int batch, int n_query, int ctx_tokens,
                         int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk, float alpha,
                         float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype, void* out_dev,
                         float* lse_dev, const int32_t* block_table, const int32_t* seq_lens, int max_pages,
                         int n_pool, hipStream_t stream) {
  if (batch < 0 || n_query <= 0 || ctx_tokens <= 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 ||
      page_tokens <= 0 || chunk <= 0)
    return LYNX_EINVAL;
  if (ctx_tokens % page_tokens != 0 || page_tokens % chunk != 0 || q_heads % kv_heads != 0) return LYNX_EINVAL;
  if (!std::isfinite(alpha) || !(alpha > 0.0f) || !std::isfinite(sm_scale)) return LYNX_EINVAL;
  if (out_dtype != LYNX_OUT_BF16 && out_dtype != LYNX_OUT_F32) return LYNX_EINVAL;
  if (head_dim != kHeadDim || verify_cpt(chunk, page_tokens) == 0 || batch > 65535 || kv_heads > 65535)
    return LYNX_EUNSUPPORTED;
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
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.max_pages = max_pages;
  a.n_pool = n_pool;
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
  }
  void* kargs[] = {&a};
  const int cpt = verify_cpt(chunk, page_tokens);
  const void* fn = cpt == 1   ? reinterpret_cast<const void*>(&k_verify<1>)
                   : cpt == 2 ? reinterpret_cast<const void*>(&k_verify<2>)
                              : reinterpret_cast<const void*>(&k_verify<4>);
  hipError_t e = hipLaunchKernel(fn,
                                 dim3((unsigned)pl.splits, (unsigned)kv_heads, (unsigned)(batch * pl.rowblocks)),
                                 dim3(kVThreads), kargs, 0, stream);
  if (e != hipSuccess) return LYNX_ELAUNCH;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&k_verify_combine), dim3((unsigned)(batch * n_query * q_heads)),
                      dim3(kHeadDim), kargs, 0, stream);
  return e == hipSuccess ? LYNX_OK : LYNX_ELAUNCH;
}

}  // namespace

int verify_launch(const void* q_dev, const void* k_anchor_dev, const void* k_residual_dev, const void* v_anchor_dev,
                  const void* v_residual_dev, int batch, int n_query, int ctx_tokens, int q_heads, int kv_heads,
                  int head_dim, int page_tokens, int chunk, float alpha, float sm_scale, void* workspace_dev,
                  size_t ws_bytes, int out_dtype, void* out_dev, float* lse_dev, hipStream_t stream) {
  return verify_launch_common(q_dev, k_anchor_dev, k_residual_dev, v_anchor_dev, v_residual_dev, batch, n_query,
                              ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk, alpha, sm_scale,
                              workspace_dev, ws_bytes, out_dtype, out_dev, lse_dev, nullptr, nullptr, 0, 0, stream);
}

int verify_paged_launch(const void* q_dev, const void* k_anchor_pool, const void* k_residual_pool,
                        const void* v_anchor_pool, const void* v_residual_pool, int n_pool, const int32_t* block_table,
                        const int32_t* seq_lens, int batch, int n_query, int max_pages, int q_heads, int kv_heads,
                        int head_dim, int page_tokens, int chunk, float alpha, float sm_scale, void* workspace_dev,
                        size_t ws_bytes, int out_dtype, void* out_dev, float* lse_dev, hipStream_t stream) {
  if (n_pool <= 0 || max_pages <= 0 || page_tokens <= 0) return LYNX_EINVAL;
  if ((long long)max_pages * page_tokens > 0x7fffffffll) return LYNX_EUNSUPPORTED;
  auto al4 = [](const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (!al4(block_table) || !al4(seq_lens)) return LYNX_EALIGN;
  return verify_launch_common(q_dev, k_anchor_pool, k_residual_pool, v_anchor_pool, v_residual_pool, batch, n_query,
                              max_pages * page_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk, alpha,
                              sm_scale, workspace_dev, ws_bytes, out_dtype, out_dev, lse_dev, block_table, seq_lens,
                              max_pages, n_pool, stream);
}

}  // namespace lynx
