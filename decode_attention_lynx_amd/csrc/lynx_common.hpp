// Shared device helpers and launch-parameter blocks for liblynx (gfx950).
//
// Sources, cited by page title and section:
//   [Review] "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
//            LLM Inference" (technical review of arXiv 2607.01831).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lynx {

constexpr int kHeadDim = 128;        // head_dim supported by this library
constexpr int kThreads = 256;        // workgroup size of the codec kernels
constexpr int kSlab = 64;            // channels of one kv head handled by one codec workgroup
constexpr int kDG = kSlab / 8;       // channel groups of 8 per slab (8)
constexpr int kTG = kThreads / kDG;  // token groups per tile (32)
constexpr int kTokPerThread = 8;     // consecutive tokens owned by one codec thread
constexpr int kTileTokens = kTG * kTokPerThread;   // 256 tokens per encode tile
constexpr int kDecDG = kHeadDim / 8;                // decode: channel groups of 8 per kv head (16)
constexpr int kDecTG = kThreads / kDecDG;           // decode: token groups per tile (16)
constexpr int kDecTile = kDecTG * kTokPerThread;    // decode: 128 tokens per tile
constexpr double kEps = 1e-6;        // epsilon of both normalisation stages (not given on the pages)
constexpr int kCodeMax = 127;        // 2^7 - 1 ([Review] Mechanism 1, Stage 3, Eq. 7)

// Geometry of one encode/decode call.  Channel c = h*128 + d; a page row (one token)
// holds H = kv_heads*128 BF16 values.  Codes are nibbles ordered
// [kv_head][channel block][token][channel in block], blocks of kCodeBlock channels: the
// 32-byte code row of (head, block, token) lies at code_offset(P, h, d, t).
constexpr int kCodeBlock = 64;                      // channels per code block
constexpr int kCodeRow = kCodeBlock / 2;            // bytes of one token's code row in a block
__host__ __device__ constexpr size_t code_offset(int P, int h, int d, int t) {
  return ((size_t)(h * (kHeadDim / kCodeBlock) + d / kCodeBlock) * P + t) * kCodeRow + (d % kCodeBlock) / 2;
}
struct Geometry {
  int n_pages;
  int P;            // tokens per page
  int Hkv;          // kv heads
  int C;            // chunk tokens (power of two in [8, 256], divides P)
  int nck;          // P / C
  int H;            // Hkv * 128
  long long anc_seg;  // bytes per anchor segment
  long long res_seg;  // bytes per residual segment
  long long codes;    // P*H/2: nibble bytes per stream per page
};

struct EncodeArgs {
  const uint16_t* kv;
  uint8_t* anchor;
  uint8_t* residual;     // nullptr: residual not selected
  Geometry g;
  float alpha;           // alpha of Eq. 7
  float ylog2k;          // 127 / log2(1 + alpha), rounded to float
  uint32_t zband;        // half-width, in units of 2^-16 of Y, of the band around a rounding
                         // boundary whose elements are decided in float64
  float pad0;
  // bnd[j] = |X_f| at which Y = j - 1/2 (j = 1..127): expm1((j - 1/2) ln(1+alpha)/127)/alpha.
  // bnd[0] = 0, bnd[128] = +inf.  Used by the float64 path to decide Round(Y).
  double bnd[129];
};

struct DecodeArgs {
  const uint8_t* anchor;
  const uint8_t* residual;   // full decode only
  void* out;
  Geometry g;
  // Signed reconstruction table S*|x_hat| in float:
  //  anchor decode: index = anchor nibble (16 entries)
  //  full decode  : index = anchor nibble | residual nibble << 4 (256 entries)
  float lut[256];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming (non-temporal) load / store: data touched once is not kept in the caches.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(void* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4*>(p));
}

// The hardware hands workgroup i to XCD (i mod 8), and each XCD has its own L2.
// Renumber so that every XCD works through one contiguous range of logical units:
// neighbouring units (which share cache lines of the code streams) meet in one L2.
constexpr int kXCDs = 8;
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int q = n / kXCDs, r = n % kXCDs, x = i % kXCDs, k = i / kXCDs;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> BF16 of two values, packed (lo = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  ua = (ua + 0x7fffu + ((ua >> 16) & 1u)) >> 16;
  ub = (ub + 0x7fffu + ((ub >> 16) & 1u)) & 0xffff0000u;
  return ua | ub;
}

}  // namespace lynx
