// Device helpers of the fused denoising step (gfx950).
//
//  * Philox4x32-10 counter-based generator, written from Salmon, Moraes,
//    Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
//  * The Gumbel transform of a Philox word, in base-2 units.
//  * The per-slice partial record of one position's tempered distribution
//    and its associative merge.
//
// Units.  The epilogue works on x2 = z * log2(e) / T (tempered logits in
// bits), so every exponential is a native v_exp_f32 (2^x) and every
// logarithm a native v_log_f32 (log2).  For a set of logits with running
// maximum m (bits) the record keeps
//     S = sum 2^(x2 - m),   A = sum (x2 - m) 2^(x2 - m)
// from which the entropy in nats is H = ln2 * (log2 S - A / S): with
// p = 2^(x2 - m) / S and ln p = ln2 (x2 - m - log2 S),
// -sum p ln p = ln2 (log2 S - A / S).
// Gumbel-max in bits: with g = -ln(-ln u) and G2 = -log2(-log2 u),
// g log2(e) = G2 - log2(ln 2), so y2 = x2 + G2 = (x + g) log2(e) + log2(ln 2):
// the argmax of y2 is the argmax of x + g, and natural-unit gaps are bit gaps
// times ln 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgd {

constexpr float kNeg = -1.0e30f;           // "no logit" sentinel (finite on purpose)
constexpr int kNoIndex = 0x7fffffff;

// ---------------------------------------------------------------------------
// Philox4x32-10
// ---------------------------------------------------------------------------
struct Philox4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {  // Weyl key schedule between rounds
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t prod0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t prod1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(prod1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(prod0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)prod1;
    c3 = (uint32_t)prod0;
    c0 = n0;
    c2 = n2;
  }
  return {c0, c1, c2, c3};
}

// The same generator for a wave-uniform key (held in scalar registers): each
// round's two three-way XORs are single v_bitop3_b32 instructions (truth
// table 0x96 = a ^ b ^ c) with the round key as the scalar operand.
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

__device__ __forceinline__ Philox4 philox4x32_10_uniform_key(uint32_t c0, uint32_t c1, uint32_t c2,
                                                             uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t prod0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t prod1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3_key((uint32_t)(prod1 >> 32), c1, k0);
    const uint32_t n2 = xor3_key((uint32_t)(prod0 >> 32), c3, k1);
    c1 = (uint32_t)prod1;
    c3 = (uint32_t)prod0;
    c0 = n0;
    c2 = n2;
  }
  return {c0, c1, c2, c3};
}

// Uniform token in [0, V) from a word: the high half of w * V.
__device__ __forceinline__ int32_t word_to_token(uint32_t w, uint32_t V) {
  return (int32_t)(((uint64_t)w * V) >> 32);
}

// -log2(-log2 u) with u = ((w >> 9) + 1/2) 2^-23 (exact in fp32): the word's
// top 23 bits under the exponent of 1.0 give 1 + (w >> 9) 2^-23 (one
// v_alignbit_b32), and subtracting 1 - 2^-24 from it is exact.
__device__ __forceinline__ float gumbel_bits(uint32_t w) {
  const float u = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u)) - 0x1.fffffep-1f;
  const float nl = -__builtin_amdgcn_logf(u);      // -log2 u > 0
  return -__builtin_amdgcn_logf(nl);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Partial record of one position over a slice of the vocabulary.
// ---------------------------------------------------------------------------
struct Rec {
  float m;      // max tempered logit (bits)
  float S;      // sum 2^(x2 - m)
  float A;      // sum (x2 - m) 2^(x2 - m)
  int32_t am;   // first index attaining m
  float y1;     // largest Gumbel-perturbed logit (bits)
  int32_t i1;   // first index attaining y1
  float y2;     // second largest (another index)
  float pad;
};
static_assert(sizeof(Rec) == 32, "record is 32 bytes");

__device__ __forceinline__ Rec rec_empty() {
  Rec r;
  r.m = kNeg; r.S = 0.f; r.A = 0.f; r.am = kNoIndex;
  r.y1 = kNeg; r.i1 = kNoIndex; r.y2 = kNeg; r.pad = 0.f;
  return r;
}

// Merge of two records over disjoint slices; `a` is the record of the slice
// merged first (the result does not depend on slice order except through
// rounding, and callers always merge in a fixed order).
__device__ __forceinline__ Rec rec_merge(const Rec& a, const Rec& b) {
  Rec r;
  r.m = fmaxf(a.m, b.m);
  const float da = a.m - r.m, db = b.m - r.m;
  const float sa = fexp2(da), sb = fexp2(db);
  r.S = a.S * sa + b.S * sb;
  r.A = (a.A + da * a.S) * sa + (b.A + db * b.S) * sb;
  const int am_tie = min(a.am, b.am);
  r.am = b.m > a.m ? b.am : (b.m < a.m ? a.am : am_tie);
  const bool b_first = b.y1 > a.y1 || (b.y1 == a.y1 && b.i1 < a.i1);
  r.y1 = b_first ? b.y1 : a.y1;
  r.i1 = b_first ? b.i1 : a.i1;
  r.y2 = b_first ? fmaxf(b.y2, a.y1) : fmaxf(a.y2, b.y1);
  r.pad = 0.f;
  return r;
}

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t rec_u32x4_t;

// Records move through memory as two 16-byte vectors.
__device__ __forceinline__ Rec rec_load(const Rec* p) {
  const rec_u32x4_t lo = *reinterpret_cast<const rec_u32x4_t*>(p);
  const rec_u32x4_t hi = *(reinterpret_cast<const rec_u32x4_t*>(p) + 1);
  Rec r;
  r.m = __uint_as_float(lo[0]); r.S = __uint_as_float(lo[1]); r.A = __uint_as_float(lo[2]);
  r.am = (int32_t)lo[3];
  r.y1 = __uint_as_float(hi[0]); r.i1 = (int32_t)hi[1]; r.y2 = __uint_as_float(hi[2]);
  r.pad = 0.f;
  return r;
}

__device__ __forceinline__ void rec_store(Rec* p, const Rec& r) {
  const rec_u32x4_t lo = {__float_as_uint(r.m), __float_as_uint(r.S), __float_as_uint(r.A),
                          (uint32_t)r.am};
  const rec_u32x4_t hi = {__float_as_uint(r.y1), (uint32_t)r.i1, __float_as_uint(r.y2), 0u};
  *reinterpret_cast<rec_u32x4_t*>(p) = lo;
  *(reinterpret_cast<rec_u32x4_t*>(p) + 1) = hi;
}

// Field-wise select (a select of whole structs would be lowered through scratch).
__device__ __forceinline__ Rec rec_pick(bool take_a, const Rec& a, const Rec& b) {
  Rec r;
  r.m = take_a ? a.m : b.m;
  r.S = take_a ? a.S : b.S;
  r.A = take_a ? a.A : b.A;
  r.am = take_a ? a.am : b.am;
  r.y1 = take_a ? a.y1 : b.y1;
  r.i1 = take_a ? a.i1 : b.i1;
  r.y2 = take_a ? a.y2 : b.y2;
  r.pad = 0.f;
  return r;
}

__device__ __forceinline__ Rec rec_shfl_xor(const Rec& a, int mask) {
  Rec r;
  r.m = __shfl_xor(a.m, mask);
  r.S = __shfl_xor(a.S, mask);
  r.A = __shfl_xor(a.A, mask);
  r.am = __shfl_xor(a.am, mask);
  r.y1 = __shfl_xor(a.y1, mask);
  r.i1 = __shfl_xor(a.i1, mask);
  r.y2 = __shfl_xor(a.y2, mask);
  r.pad = 0.f;
  return r;
}

}  // namespace dgd
