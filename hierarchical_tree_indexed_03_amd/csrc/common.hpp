// Shared definitions of the ZHA HIP library (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zha {

constexpr int MAXL = 16;        // max summary levels
constexpr int GMAX = 8;         // max query heads per KV head (group size)
constexpr int NB1 = 512;        // coarse top-p bins over delta = max score - score
constexpr float BINS_PER_UNIT = 16.f;   // coarse bins per unit of score (covers delta < 32)
constexpr int NB2 = 512;        // fine sub-bins inside the boundary coarse bin
constexpr float MASS_SCALE = 1099511627776.0f;  // 2^40: fixed-point unit of probability mass
constexpr int CAND_PAIRWISE = 256;  // boundary ties resolved pairwise in LDS up to this many
constexpr int EXPAND_CHUNK = 1024;  // union-list entries per expand workgroup
constexpr int MAX_SPLITS = 512;     // attention splits per KV head
constexpr int SEL_P = 64;           // top-p histogram / classify workgroups per KV head (max)
constexpr int TD_MAX = 33792;       // nodes of a level selected top-down (32768 + room for appends)
constexpr int TD_WORDS = TD_MAX / 32;
// Every level scored from the keys (block-4 trees with key-form level 1, at least 4 levels):
// a score workgroup covers one level-4 node; the top-down selection takes level 1 from
// global memory up to AK_N1 nodes, and keeps the dot products of the levels above level 4
// in LDS (at most AK_DUP floats).
constexpr int AK_B = 4;
constexpr int AK_LC = 4;
constexpr int AK_N1 = 131072;
constexpr int AK_DUP = 12288;
// the append's sibling aggregates: per level R x (D + 2) floats rounded to a multiple of 4
// (16-byte aligned levels), (MAXL + 1) levels per KV head
#define SIB_LEVEL(R, D) ((((R) * ((D) + 2)) + 3) & ~3)
#define SIB_STRIDE(R, D) ((int64_t)(MAXL + 1) * SIB_LEVEL(R, D))

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// 16 bytes as a native vector (loads and stores of it stay register values, where a copy of
// the uint4 struct can become a memcpy that keeps an array of them in scratch memory)
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

struct bf16_t { uint16_t bits; };   // storage type of bfloat16 tensors

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
// nearest bfloat16 (ties to even) of a finite float, as its 16 bits
__device__ __forceinline__ uint32_t f2bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// OCP MX FP4 of 32 consecutive elements: scale X = 2^(floor(log2 amax) - 2), stored as the
// biased exponent byte E8M0 = floor(log2 amax) - 2 + 127 (0 for an all-zero block); each
// element the nearest of X*{0,.5,1,1.5,2,3,4,6} (ties to the even code, clamped at 6X).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);   // biased exponent of amax
  return amax > 0.f ? (uint32_t)(e >= 2 ? e - 2 : 0) : 0u;
}
__device__ __forceinline__ uint32_t e2m1_code(float x, uint32_t scale_byte) {
  // x / X exactly: a power-of-two scaling
  const float a = fabsf(x) * __uint_as_float((uint32_t)(254 - (int)scale_byte) << 23);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.f);
  return m | (x < 0.f ? 8u : 0u);
}

// Device invariant checks, compiled in with -DZHA_DEBUG: a failed check sets its bit in the
// handle's check word (read and cleared by zha_debug_check); nothing traps.
enum CheckBit {
  CHK_LIST_SIZE = 0,     // a union list longer than its level's node capacity
  CHK_NODE_RANGE = 1,    // a union-list node id outside the level
  CHK_CAND_RANGE = 2,    // a boundary-bin candidate past its list's capacity
  CHK_EXPAND_RANGE = 3,  // an expanded list past the next level's capacity
  CHK_TOKEN_RANGE = 4,   // an attended token at or past N
  CHK_SPLITS = 5,        // attention splits past MAX_SPLITS
  CHK_TD_SIZE = 6,       // a top-down level larger than TD_MAX
};
#ifdef ZHA_DEBUG
#define ZHA_CHECK(devref, cond, bit) \
  do { if (!(cond)) atomicOr((devref).err, 1u << (bit)); } while (0)
#else
#define ZHA_CHECK(devref, cond, bit) do { } while (0)
#endif

// Order-preserving map float -> uint32 (a < b  <=>  key(a) < key(b)).
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Top-p binning of one score relative to the head's max: everything that decides a node's
// fate goes through these functions so every kernel takes the same decision.
struct BinSub { uint32_t bin, sub; };
__device__ __forceinline__ BinSub bin_of(float score, float maxs) {
  BinSub r;
  const float delta = maxs - score;                 // >= 0
  const float u = delta * BINS_PER_UNIT;
  r.bin = u < (float)(NB1 - 1) ? (uint32_t)u : (uint32_t)(NB1 - 1);
  const float frac = u - (float)r.bin;              // in [0, 1) unless clamped
  r.sub = 0;
  if (r.bin < (uint32_t)(NB1 - 1)) {
    const float f = frac * (float)NB2;
    r.sub = f < (float)(NB2 - 1) ? (uint32_t)f : (uint32_t)(NB2 - 1);
  }
  return r;
}
__device__ __forceinline__ uint64_t mass_of(float score, float maxs) {
  return (uint64_t)(expf(-(maxs - score)) * MASS_SCALE);   // in (0, 2^40]
}
struct BinMass { uint32_t bin, sub; uint64_t mass; };
__device__ __forceinline__ BinMass bin_mass(float score, float maxs) {
  const BinSub bs = bin_of(score, maxs);
  BinMass r;
  r.bin = bs.bin;
  r.sub = bs.sub;
  r.mass = mass_of(score, maxs);
  return r;
}

// Per (level, query head) routing state.
struct QState {
  uint32_t maxkey;    // ordered key of the max score over the head's frontier
  uint32_t b1;        // boundary coarse bin; NB1 => keep every frontier node
  uint32_t b2;        // boundary fine sub-bin inside b1
  uint32_t ncand;     // frontier nodes of this head that fell into bin b1 (candidate list length)
  uint64_t total;     // sum of fixed-point masses (Z)
  uint64_t target;    // ceil(p * Z): the kept prefix must reach this mass
  uint64_t above1;    // mass of bins < b1
  uint64_t above2;    // mass of bins < b1 and sub-bins < b2 of b1
  uint32_t nties;     // nodes in (b1, b2)
  uint32_t flags;     // bit 0: resolved through the radix path
  uint32_t pad[2];
};
static_assert(sizeof(QState) == 64, "QState layout");

// Device pointers of one handle's workspace (computed on the host).
struct Dev {
  // tree
  float* s[MAXL + 1];       // level l: [Hkv][ncap[l]][R][D]
  float* c[MAXL + 1];       // level l: [Hkv][ncap[l]][R]
  float* lse[MAXL + 1];     // level l: [Hkv][ncap[l]][R] log mass at r_j (build/append only)
  bf16_t* sq[MAXL + 1];     // level l: [Hkv][ncap[l]][R][D] the router's bf16 copy of s (bf16
                            // router planes only; null at a level the router reads no planes of)
  uint8_t* s4[MAXL + 1];    // level l: [Hkv][ncap[l]][R][D/2] the router's FP4 copy of s (MX FP4
                            // router planes only): E2M1 codes, element 2i in the low nibble of byte i
  uint8_t* s4x[MAXL + 1];   // level l: [Hkv][ncap[l]][R][D/32] E8M0 scale of each 32 elements
  float* w1;                // [Hkv][ncap[1]][R][b] token weights of the level-1 planes
                            // (key-form scoring only; null otherwise)
  int64_t ncap[MAXL + 1];   // node capacity per level (index 0: gather list = ncap[1])
  // router, per level l = 0..L (0 = kept level-1 blocks)
  int32_t* node[MAXL + 1];  // [Hkv][ncap[l]]
  uint32_t* mask[MAXL + 1]; // [Hkv][ncap[l]]
  uint32_t* keep[MAXL + 1]; // [Hkv][ncap[l]]           (l >= 1)
  float* score[MAXL + 1];   // [Hkv][GMAX][ncap[l]]     (l >= 1)
  int32_t* part[MAXL + 1];  // [Hkv][nchunks(l)]        expand partial counts
  int32_t* cnt;             // [MAXL + 1][Hkv] entries of each union list
  int32_t* ucnt;            // [MAXL + 1][Hkv] entries some head's frontier holds (a dense list
                            // may hold nodes of no head's frontier, with mask 0)
  QState* qs;               // [MAXL + 1][Hq]
  uint64_t* hpart;          // [Hkv][SEL_P][GMAX][NB1] per-workgroup coarse mass histograms
  uint32_t* tdbits;         // [MAXL + 1][Hq][2][TD_WORDS] top-down frontier / kept bitmaps
  uint32_t* kb1;            // [Hq][2][ncap[1] / 32] level-1 frontier / kept bitmaps when every level is
                            // scored from the keys (level 1 selected top-down); null otherwise
  float* kdots;             // [Hkv][ncap[4]][GMAX][R] level-4 dot products q.s_j / sqrt(d) of that path
  uint32_t* tick;           // [Hkv] workgroups of each KV head done with that path's top-down selection
                            // (zeroed by the prep kernel; the last one writes the gather list)
  float* sib;               // [Hkv][SIB_STRIDE] = [MAXL + 1][R][D + 2] per level: aggregate (LSE, A, s) of the
                            // rightmost node's complete children (append)
  int64_t* sibkey;          // [Hkv][MAXL + 1] first child * 256 + count it was built from; -1 none
  int32_t* cand;            // [Hq][ncap[1]]
  float* qf;                // [Hq][D] sigma * q in fp32
  float* apart;             // [Hq][MAX_SPLITS][D + 2] attention partials (m, l, o)
  uint32_t* err;            // invariant-check bits (debug builds)
};

}  // namespace zha
