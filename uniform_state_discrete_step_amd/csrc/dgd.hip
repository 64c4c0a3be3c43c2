// libdgd: the per-step denoising update of uniform-state discrete diffusion
// on AMD Instinct MI355X (gfx950, CDNA4).
//
// Per step, three kernels:
//   k_project_packed (or k_project for a row-major table)
//                   bf16 MFMA projection z = H W^T (W streamed once from HBM,
//                   H chunks staged through LDS) fused with the tempered
//                   softmax-entropy, argmax and Gumbel-max reductions in its
//                   epilogue; writes one 32-byte partial record per
//                   (position, vocabulary group).  Logits stay in registers.
//   k_merge         merges the partial records of each position;
//   k_commit        one workgroup per canvas applies the early-stop rule,
//                   sorts the open positions by entropy, applies the entropy
//                   bound, writes samples and re-noises the rest.
// plus k_init_block at the start of each block, and, when the caller asks for
// them:
//   k_rmsnorm       the output norm of H, before the projection (the logit
//                   softcap is applied inside the projection's epilogue);
//   k_sc_topk       the self-conditioning top-K of every position, from
//                   candidate lists the projection's epilogue keeps;
//   k_sc_embed      the next forward's self-conditioning input from a top-K;
//   k_label         the sparse label read for typed decisions.
// Tables: k_pack_vocab (bf16, streaming order) and k_pack_vocab_q4 (4-bit).
// Validation and measurement: k_debug_gumbel, k_debug_philox, k_ceiling_hbm,
// k_ceiling_mfma.
//
// The method follows "The Annotated DiffusionGemma" walkthrough, section
// "Sampling" (temperature, entropy, low-entropy prefix, early stop), with the
// knob semantics of the ComfyUI "DiffusionGemma Denoise (KV Cache)" node page
// (Inputs table) and the TensorSharp DiffusionGemma doc ("3. Sampler
// contract").  The C ABI is declared and documented in include/dgd.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/dgd.h"
#include "dgd_device.h"

using namespace dgd;

namespace {

// ---------------------------------------------------------------------------
// tiling constants of the projection
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;           // merge/commit and init kernels: 4 waves of 64

// Blocks of 32 positions per epilogue loop body of the packed projection
// (four: the accumulator rotation between bodies then moves 256 instead of
// 1792 registers per tile, 14 us less at 256 x 262144 x 2816; the variant
// that also keeps top-K lists fits four as well, without spills)
#ifndef DGD_EPI_UNROLL
#define DGD_EPI_UNROLL 4
#endif
#ifndef DGD_EPI_UNROLL_TOPK
#define DGD_EPI_UNROLL_TOPK 4
#endif

// Phase timing (a measurement build, DGD_PHASE_TIMING defined): the packed
// projection records, per workgroup (0..1023) and wave, the 100 MHz wall
// clock at kernel start, at the start, K-loop end and epilogue end of its
// first four tiles, and at kernel end, plus the shader clock at start and
// end.  Lane 0 of each wave writes its slots with vector stores; the last
// launch overwrites the previous one.  dgd_phase_times() reads them.
constexpr int kPhaseWorkgroups = 1024, kPhaseSlots = 16;
#ifdef DGD_PHASE_TIMING
__device__ unsigned long long g_phase[kPhaseWorkgroups * 4 * kPhaseSlots];
#define PHASE_AT(slot, clk)                                                                    \
  do {                                                                                         \
    if ((threadIdx.x & 63) == 0 && blockIdx.x < kPhaseWorkgroups)                              \
      g_phase[(blockIdx.x * 4 + ((threadIdx.x >> 6) & 3)) * kPhaseSlots + (slot)] = (clk);     \
  } while (0)
#else
#define PHASE_AT(slot, clk) \
  do {                      \
  } while (0)
#endif
constexpr int kWaves = kThreads / 64;
constexpr int kPThreads = 512;          // projection: 8 waves, two per SIMD
constexpr int kVGroups = 4;             // projection waves along the vocabulary ...
constexpr int kPGroups = 2;             // ... and along the positions
constexpr int kVB = 2;                  // 32-row vocabulary blocks per wave (A fragments)
constexpr int kVocabPerWave = 32 * kVB; // 64 vocabulary rows per wave
constexpr int kVocabTile = kVGroups * kVocabPerWave;   // 256 vocabulary rows per tile
constexpr int kKChunk = 64;             // hidden elements per LDS stage
constexpr int kMaxGroups = 256;         // vocabulary groups (partials per position)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr double kLn2 = 0.693147180559945309417232121458176568;
constexpr float kMasked = -2.0e30f;      // logit (bits) of vocabulary ids past V
constexpr double kMinTemperature = 1e-4;  // keeps tempered fp32 logits finite
constexpr double kLog2e = 1.442695040888963407359924681001892137;

// Words per canvas in the state block after prev_argmax: stable_count, done,
// steps_used, converged, n_committed, mean_entropy, new_commits, status and
// the three band counters.
constexpr int kStateWordsPerCanvas = 11;

// Per-position flags the merge leaves for the commit kernel.
constexpr int32_t kRowNonFinite = 1;    // the position's logits were not all finite
constexpr int32_t kRowNearSample = 2;   // top-two Gumbel gap below the sample band

// Tie bands of the step's float decisions (nats), counted per canvas.
constexpr double kBandSample = 1e-4;
constexpr double kBandCommit = 1e-5;
constexpr double kBandConv = 1e-5;

struct ProjArgs {
  const uint16_t* H;      // [M][d]
  const uint16_t* W;      // [V][d]
  Rec* part;              // [M][P]
  float* logits;          // [M][V] (validation) or null
  const int32_t* done;    // [B]
  int32_t M, V, d, L, B;
  int32_t P, n_vtiles, n_mtiles;
  int32_t block, gstep;
  float c2;               // log2(e) / T_s
  float cap_in, cap_out;  // softcap: 2 log2(e) / c and c * c2 (used only when the cap is on)
  struct ScEnt* cand;     // [M][P][kScCand] self-conditioning candidates, or null
  uint32_t key[DGD_MAX_CANVASES][2];
};

struct CommitArgs {
  const Rec* part;
  int32_t P;
  float* rowM;            // merged max (bits) and sum 2^(x2 - m) of each position
  float* rowS;
  float* rowH;
  int32_t* rowA;
  int32_t* rowTok;
  int32_t* rowF;          // per-position flags (kRowNonFinite, kRowNearSample)
  float* out_entropy;
  int32_t* out_argmax;
  int32_t* out_token;
  float* out_gap;
  int16_t* commit_step;
  int32_t* canvas;
  uint8_t* committed;
  int32_t* st_prev;
  int32_t* st_stable;
  int32_t* st_done;
  int32_t* st_steps;
  int32_t* st_conv;
  int32_t* st_ncomm;
  float* st_mean;
  int32_t* st_new;
  int32_t* st_status;
  int32_t* st_bsample;
  int32_t* st_bcommit;
  int32_t* st_bconv;
  int32_t B, L, G, V, N, block, step, gstep, freeze, final_emit, stab;
  float conf;
  float bound[DGD_MAX_CANVASES];
  uint32_t key[DGD_MAX_CANVASES][2];
};

struct InitArgs {
  int32_t* canvas;
  uint8_t* committed;
  int32_t* st_prev;
  int32_t* st_stable;
  int32_t* st_done;
  int32_t* st_steps;
  int32_t* st_conv;
  int32_t* st_ncomm;
  float* st_mean;
  int32_t* st_new;
  int32_t* st_status;
  int32_t* st_bsample;
  int32_t* st_bcommit;
  int32_t* st_bconv;
  int32_t B, L, G, V, block;
  uint32_t key[DGD_MAX_CANVASES][2];
};

// Vocabulary groups: tiles vt = g, g + P, g + 2P, ... belong to group g.  The
// count depends on V only, so a position's merge order never depends on how
// many canvases are batched together.
__host__ __device__ inline int num_vtiles(int V) { return (V + kVocabTile - 1) / kVocabTile; }
__host__ __device__ inline int num_groups(int V) {
  const int t = num_vtiles(V);
  return t < kMaxGroups ? t : kMaxGroups;
}

// Block id -> (M tile, vocabulary group).  Consecutive ids go to different
// XCDs (round-robin); the ids one XCD receives walk the M tiles of one group
// before the next group, so tiles that share W rows run on one L2.
__device__ inline void tile_of_block(int id, int n_mtiles, int P, int& mt, int& g) {
  if ((P & 7) == 0) {
    const int xcd = id & 7, j = id >> 3;
    mt = j % n_mtiles;
    g = (j / n_mtiles) * 8 + xcd;
  } else {
    mt = id % n_mtiles;
    g = id / n_mtiles;
  }
}

__device__ inline bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS rows are 128 bytes (eight 16-byte segments); segment e of row r is
// stored in slot e ^ swz(r).  swz differs for the 8 rows of any aligned
// group of 8, and for the 8 even (and the 8 odd) rows of any aligned group of
// 16, so 128-bit accesses by consecutive lanes to consecutive rows are
// conflict-free whether the LDS serves 8 or 16 such lanes per cycle.
__device__ inline int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Raw buffer resources: word 3 selects 32-bit untyped access on gfx9-family
// parts; kOOB is an offset beyond any num_records (the load returns zero).
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kNonTemporal = 2;   // streaming (nt) cache policy for W

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector-memory
// and `lgkm` LDS/scalar operations of this wave are outstanding.
constexpr int waitcnt_enc(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

// Softcapped logit in bits: c * tanh(z / c) * log2(e) / T, given
// cin = 2 log2(e) / c and cout = c * log2(e) / T.  tanh(t) = 1 - 2 / (e + 1)
// with e = 2^(2 log2(e) t) = e^(2t): for large t, e = inf and the result is
// exactly cout; for very negative t, e = 0 and it is exactly -cout.  Absolute
// error a few 2^-24 of the tanh (the cancellation in 1 - 2 / (e + 1) near
// t = 0 is absolute, not relative), then scaled by cout.
__device__ __forceinline__ float softcap_bits(float z, float cin, float cout) {
  const float e = fexp2(z * cin);
  const float r = __builtin_amdgcn_rcpf(e + 1.f);
  return fmaf(-2.f * cout, r, cout);
}

// Record of one position over the 64 vocabulary ids held by a lane pair:
// z[vb][4q + e] (lane half h) is the logit of id vbase + 32 vb + 8 q + 4 h + e.
// The two halves' records are merged; both lanes return the merged record.
// kCap: the logits pass through the softcap first (c2 is then unused).
// kInPlace: z is left holding the tempered logits in bits (the top-K lists
// read them); otherwise z keeps the raw logits and the scale by c2 is fused
// into the operations that use it (one rounding instead of two).
template <bool kUniformKey, bool kCap, bool kInPlace>
__device__ __forceinline__ Rec tile_record(f32x16_t (&z)[kVB], int vbase, int half, int V, float c2,
                                           float cin, float cout, uint32_t pabs, uint32_t gstep,
                                           uint32_t key0, uint32_t key1) {
  static_assert(!kCap || kInPlace, "the capped logits are computed in place");
  // value index i = vb*16 + 4q + e  <->  vocabulary id vbase + vb*32 + 8q + 4h + e
  if constexpr (kCap) {
#pragma unroll
    for (int i = 0; i < kVB * 16; ++i) {
      z[i >> 4][i & 15] = softcap_bits(z[i >> 4][i & 15], cin, cout);
      if ((i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (kInPlace) {
#pragma unroll
    for (int i = 0; i < kVB * 16; ++i) z[i >> 4][i & 15] = __fmul_rn(z[i >> 4][i & 15], c2);
  }
  const float sc = kInPlace ? 1.f : c2;   // from the values in z to bits
  // In a ragged last tile, ids past V get kMasked (raw or in bits: c2 > 1
  // keeps it below kNeg either way): they add exact zeros to S and A and
  // never win the argmax or the sample.
  if (vbase + kVocabPerWave > V) {
#pragma unroll
    for (int i = 0; i < kVB * 16; ++i) {
      const int v = vbase + (i >> 4) * 32 + 8 * ((i >> 2) & 3) + 4 * half + (i & 3);
      z[i >> 4][i & 15] = v < V ? z[i >> 4][i & 15] : kMasked;
    }
  }
  auto off = [](int i) { return (i >> 4) * 32 + 8 * ((i >> 2) & 3) + (i & 3); };
  // Largest value (max3 chains); its tempered value round(mr * sc) is the
  // largest tempered logit, rounding being monotone.
  float mr = kNeg;
#pragma unroll
  for (int i = 0; i < kVB * 16; ++i) mr = fmaxf(mr, z[i >> 4][i & 15]);
  const float m = fmaxf(__fmul_rn(mr, sc), kNeg);
  __builtin_amdgcn_sched_barrier(0);
  // Sums and the first index of the maximum, last value first (so the
  // final assignment is the smallest id).
  float S = 0.f, A = 0.f;
  int ao = -1;
#pragma unroll
  for (int i = kVB * 16 - 1; i >= 0; --i) {
    const float zi = z[i >> 4][i & 15];
    const float dx = fmaf(zi, sc, -m);
    const float e = fexp2(dx);
    S += e;
    A = fmaf(dx, e, A);
    ao = zi == mr ? off(i) : ao;
    if ((i & 7) == 0) __builtin_amdgcn_sched_barrier(0);
  }
  float y1 = kNeg, y2 = kNeg;
  int io = -1;
#pragma unroll
  for (int grp = 0; grp < kVB * 4; ++grp) {
    const int v0 = vbase + (grp >> 2) * 32 + 8 * (grp & 3) + 4 * half;
    Philox4 pw;
    if constexpr (kUniformKey)
      pw = philox4x32_10_uniform_key((uint32_t)v0 >> 2, pabs, gstep, 0u, key0, key1);
    else
      pw = philox4x32_10((uint32_t)v0 >> 2, pabs, gstep, 0u, key0, key1);
    const uint32_t words[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // top two, first index on ties
      const int i = 4 * grp + e;
      const float y = fmaf(z[i >> 4][i & 15], sc, gumbel_bits(words[e]));
      y2 = __builtin_amdgcn_fmed3f(y, y1, y2);   // y2 <= y1: max(y2, min(y, y1))
      const bool gt = y > y1;
      io = gt ? off(i) : io;
      y1 = gt ? y : y1;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const int vlane = vbase + 4 * half;
  Rec loc;
  loc.m = m; loc.S = S; loc.A = A; loc.am = ao < 0 ? kNoIndex : vlane + ao;
  loc.y1 = y1; loc.i1 = io < 0 ? kNoIndex : vlane + io; loc.y2 = y2; loc.pad = 0.f;
  const Rec oth = rec_shfl_xor(loc, 32);
  return rec_merge(rec_pick(half == 0, loc, oth), rec_pick(half == 0, oth, loc));
}

// ---------------------------------------------------------------------------
// Self-conditioning top-K: candidate lists built in the projection's epilogue
// ---------------------------------------------------------------------------
// For every position and every vocabulary band of its group (the 64 rows of
// each of the group's tiles that one wave owns), the epilogue keeps a list of
// the kScWave largest tempered logits seen over the group's tiles, with their
// ids.  Each lane first takes the top kScLane values of its own 32 ids in the
// tile; the two lanes of a position then merge theirs into the band list in
// LDS.  Lists order by value only (equal values in any order): every value a
// list dropped is at most its last entry, which is tagged.  k_sc_topk
// recomputes a list's part of the vocabulary exactly whenever a tagged value
// reaches the K-th selected value, so its result is exact, ties included.
constexpr int kScLane = 3;                     // per-lane list: one tile, 32 ids
constexpr int kScWave = 4;                     // per-(band, position) list over the tiles
constexpr int kScCand = kVGroups * kScWave;    // candidates per (position, group)
constexpr uint32_t kScLaneTag = 0x80000000u;   // last entry of a lane list
constexpr uint32_t kScWaveTag = 0x40000000u;   // last entry of a band list
constexpr uint32_t kScIdBits = 0x3FFFFFFFu;
constexpr uint32_t kScNoId = kScIdBits;        // empty slot: never a valid id

struct ScEnt {
  float x;       // tempered logit in bits (x2 = z * log2(e) / T, or the capped value)
  uint32_t id;   // vocabulary id | tags
};
static_assert(sizeof(ScEnt) == 8, "candidate is 8 bytes");

// Insert (x, i) into a list sorted by value, largest first, dropping its last
// entry (an equal value goes after the entries already there).
template <int N>
__device__ __forceinline__ void sc_insert(float (&lx)[N], uint32_t (&li)[N], float x, uint32_t i) {
  bool b[N];
#pragma unroll
  for (int k = 0; k < N; ++k) b[k] = x > lx[k];
  // values: entry k becomes the median of (x, entry k-1, entry k), the list
  // being sorted; ids follow the comparisons
#pragma unroll
  for (int k = N - 1; k >= 1; --k) {
    lx[k] = __builtin_amdgcn_fmed3f(x, lx[k - 1], lx[k]);
    li[k] = b[k - 1] ? li[k - 1] : (b[k] ? i : li[k]);
  }
  lx[0] = fmaxf(lx[0], x);
  li[0] = b[0] ? i : li[0];
}

__device__ __forceinline__ void sc_list_clear(ScEnt* slot) {
  const u32x4_t e = {__float_as_uint(kNeg), kScNoId, __float_as_uint(kNeg), kScNoId};
  reinterpret_cast<u32x4_t*>(slot)[0] = e;
  reinterpret_cast<u32x4_t*>(slot)[1] = e;
}

// One tile of one position: z holds the lane's 32 tempered logits (after
// tile_record, ids past V already masked); slot is the position's band list
// in LDS, updated by the lane of half 0.
__device__ __forceinline__ void sc_tile_update(const f32x16_t (&z)[kVB], int vbase, int half,
                                               ScEnt* slot) {
  // top kScLane values of the lane's 32 ids, by sorted insertion
  static_assert(kScLane == 3 && kScWave == 4, "list sizes");
  float t0 = -INFINITY, t1 = -INFINITY, t2 = -INFINITY;
  int o0 = 0, o1 = 0, o2 = 0;
#pragma unroll
  for (int i = 0; i < kVB * 16; ++i) {
    const float x = z[i >> 4][i & 15];
    const int off = (i >> 4) * 32 + 8 * ((i >> 2) & 3) + (i & 3);
    const bool c0 = x > t0, c1 = x > t1, c2 = x > t2;
    // t0 >= t1 >= t2: each new value is a median of three (or the maximum)
    t2 = __builtin_amdgcn_fmed3f(x, t1, t2);
    o2 = c1 ? o1 : (c2 ? off : o2);
    t1 = __builtin_amdgcn_fmed3f(x, t0, t1);
    o1 = c0 ? o0 : (c1 ? off : o1);
    t0 = fmaxf(t0, x);
    o0 = c0 ? off : o0;
    if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t base = (uint32_t)(vbase + 4 * half);
  const uint32_t i0 = base + o0, i1 = base + o1, i2 = (base + o2) | kScLaneTag;
  const float u0 = __shfl_xor(t0, 32), u1 = __shfl_xor(t1, 32), u2 = __shfl_xor(t2, 32);
  const uint32_t j0 = __shfl_xor(i0, 32), j1 = __shfl_xor(i1, 32), j2 = __shfl_xor(i2, 32);
  if (half == 0) {
    const u32x4_t a = reinterpret_cast<const u32x4_t*>(slot)[0];
    const u32x4_t b = reinterpret_cast<const u32x4_t*>(slot)[1];
    float lx[kScWave] = {__uint_as_float(a[0]), __uint_as_float(a[2]), __uint_as_float(b[0]),
                         __uint_as_float(b[2])};
    uint32_t li[kScWave] = {a[1], a[3], b[1], b[3]};
    sc_insert(lx, li, t0, i0);
    sc_insert(lx, li, t1, i1);
    sc_insert(lx, li, t2, i2);
    sc_insert(lx, li, u0, j0);
    sc_insert(lx, li, u1, j1);
    sc_insert(lx, li, u2, j2);
    const u32x4_t na = {__float_as_uint(lx[0]), li[0], __float_as_uint(lx[1]), li[1]};
    const u32x4_t nb = {__float_as_uint(lx[2]), li[2], __float_as_uint(lx[3]), li[3]};
    reinterpret_cast<u32x4_t*>(slot)[0] = na;
    reinterpret_cast<u32x4_t*>(slot)[1] = nb;
  }
}

// ---------------------------------------------------------------------------
// k_project: fused projection + tempered softmax-entropy / argmax / Gumbel-max
// ---------------------------------------------------------------------------
// Workgroup = 8 waves, two per SIMD (one wave per SIMD cannot stream 128-bit
// LDS reads at the rate the MFMAs consume them).  Tile = 256 vocabulary rows x
// MROWS = 32*MB positions; wave w covers vocabulary rows 64*(w%4) .. +63 (two
// 32-row blocks) and positions (w/4)*MROWS/2 .. +MROWS/2-1.
//
// MFMA v_mfma_f32_32x32x16_bf16 with A = W (vocabulary along the MFMA rows)
// and B = H (positions along the MFMA columns): lane l holds, per 32-position
// block and vocabulary block, 16 logits of ONE position (column l%32) at
// vocabulary rows 8q + 4(l/32) + e (q, e = 0..3), i.e. groups of four
// consecutive ids: exactly the four words of one Philox call.
//
// K loop, per 64-element hidden chunk: the workgroup reads the W chunk
// [256 x 64] eight lanes per 128-byte line (two chunks in flight, in
// registers) and the H chunk [MROWS x 64] (L2-resident, one chunk ahead), and
// stages both in double-buffered, swizzled LDS, from which the MFMA fragments
// are read.  MFMA sub-step s (0..3) uses hidden elements 32h + 8s .. +7 for
// lane half h in both operands: the same permutation of k on A and B, so the
// products summed are exactly those of the plain dot product.
//
// kUniformKey: every 32-row block lies inside one canvas (L % 32 == 0), so the
// Philox key is wave-uniform and lives in scalar registers.  kCap: the logit
// softcap is applied before the temperature.
template <int MB, bool kLogits, bool kUniformKey, bool kCap>
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
k_project(const ProjArgs a) {
  static_assert(MB == 2 || MB == 4 || MB == 8, "MB");
  constexpr int MROWS = 32 * MB;
  constexpr int MBW = MB / kPGroups;                      // position blocks per wave
  constexpr int PPW = MROWS / kPGroups;                   // positions per wave
  constexpr int HSEG = MROWS * (kKChunk / 8) / kPThreads; // 16-byte H segments per thread
  constexpr int WSEG = kVocabTile * (kKChunk / 8) / kPThreads;  // 16-byte W segments per thread
  constexpr int HBUF = MROWS * kKChunk * 2;
  constexpr int WBUF = kVocabTile * kKChunk * 2;
  static_assert(HSEG >= 1 && WSEG == 4, "tiling");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * HBUF + 2 * WBUF];
  // running record of every (wave, position of its group) over the tiles seen
  __shared__ __attribute__((aligned(16))) Rec recs[8 * PPW];
  uint8_t* const hbuf0 = smem;
  uint8_t* const wbuf0 = smem + 2 * HBUF;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int wv = wave & (kVGroups - 1), wp = wave / kVGroups;

  int mt, g;
  tile_of_block(blockIdx.x, a.n_mtiles, a.P, mt, g);
  const int row0 = mt * MROWS;
  {
    const int last_row = min(row0 + MROWS, a.M) - 1;
    bool all_done = true;
    for (int c = row0 / a.L; c <= last_row / a.L; ++c) all_done &= (a.done[c] != 0);
    if (all_done) return;
  }

  for (int i = tid; i < 8 * PPW; i += kPThreads) rec_store(recs + i, rec_empty());
  // (the first __syncthreads of the tile loop orders these writes)

  const int nk = (a.d + kKChunk - 1) / kKChunk;
  const size_t d = (size_t)a.d;

  for (int vt = g; vt < a.n_vtiles; vt += a.P) {
    const int vbase = vt * kVocabTile + wv * kVocabPerWave;
    // Buffer resources for this tile: rows past the end of W (or of the
    // M tile) lie beyond num_records and read as zero without a memory
    // access; so does any offset with bit 31 set.  All offsets are in the
    // 32-bit VGPR offset so the range check covers them.
    const int vrows = min(kVocabTile, a.V - vt * kVocabTile);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (size_t)vt * kVocabTile * d), (short)0, (int)((size_t)vrows * d * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.H + (size_t)row0 * d), (short)0, (int)((size_t)min(MROWS, a.M - row0) * d * 2),
        kRsrcWord3);
    // Wave w loads tile rows 32w .. 32w+31 of W, instruction j covering rows
    // 32w + 8j .. +7 with lane l reading 16 bytes at segment l%8 of row l/8
    // (eight lanes per 128-byte line).
    const uint32_t woff = (uint32_t)((32 * wave + (lane >> 3)) * d * 2 + (lane & 7) * 16);
    const uint32_t wstride = (uint32_t)(8 * d * 2);                     // 8 rows
    const uint32_t hoff = (uint32_t)((tid >> 3) * d * 2 + (tid & 7) * 16);
    const uint32_t hstride = (uint32_t)((kPThreads / 8) * d * 2);      // 64 rows

    // Loads of hidden elements past d (including whole chunks past the end)
    // get bit 31 set in their offset: beyond num_records, they read zeros
    // without a memory access.  Built with bit operations, not a select, so
    // the loop body stays straight-line code.
    auto load_w = [&](int c, u32x4_t (&dst)[WSEG]) {
      const uint32_t oob = (uint32_t)(c * kKChunk + (lane & 7) * 8 >= a.d) << 31;
#pragma unroll
      for (int j = 0; j < WSEG; ++j) {
        const uint32_t off = (woff + (uint32_t)j * wstride + (uint32_t)(c * kKChunk * 2)) | oob;
        dst[j] = __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, kNonTemporal);
      }
    };
    auto store_w = [&](int buf, const u32x4_t (&src)[WSEG]) {
      uint8_t* base = wbuf0 + buf * WBUF;
#pragma unroll
      for (int j = 0; j < WSEG; ++j) {
        const int r = 32 * wave + 8 * j + (lane >> 3);
        *(u32x4_t*)(base + r * 128 + (((lane & 7) ^ swz(r)) << 4)) = src[j];
      }
    };
    auto load_h = [&](int c, u32x4_t (&dst)[HSEG]) {
      const uint32_t oob = (uint32_t)(c * kKChunk + (tid & 7) * 8 >= a.d) << 31;
#pragma unroll
      for (int i = 0; i < HSEG; ++i) {
        const uint32_t off = (hoff + (uint32_t)i * hstride + (uint32_t)(c * kKChunk * 2)) | oob;
        dst[i] = __builtin_amdgcn_raw_buffer_load_b128(hres, off, 0, 0);
      }
    };
    auto store_h = [&](int buf, const u32x4_t (&src)[HSEG]) {
      uint8_t* base = hbuf0 + buf * HBUF;
#pragma unroll
      for (int i = 0; i < HSEG; ++i) {
        const int idx = i * kPThreads + tid;
        const int r = idx >> 3, e = idx & 7;
        *(u32x4_t*)(base + r * 128 + ((e ^ swz(r)) << 4)) = src[i];
      }
    };

    f32x16_t acc[kVB][MBW];
#pragma unroll
    for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
      for (int pb = 0; pb < MBW; ++pb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[vb][pb][i] = 0.f;

    // One chunk: MFMAs on the W and H chunks in LDS buffer c&1 while H(c+1)
    // (L2-resident) and W(c+2) (HBM) are in flight; W(c+1), loaded one chunk
    // earlier, is written to LDS at the end.  The issue order is pinned
    // (vmcnt retires loads in order): H(c+1) strictly before W(c+2), so the
    // wait for H at the end of the chunk leaves the W prefetch in flight.
    // Chunks past the end read zeros and add exact zeros, so the loop runs
    // whole pairs of chunks and the register ring index stays static.
    auto chunk = [&](int c, u32x4_t (&wload)[WSEG], const u32x4_t (&wstore)[WSEG],
                     u32x4_t (&hs)[HSEG]) {
      __builtin_amdgcn_sched_barrier(0);
      load_h(c + 1, hs);
      __builtin_amdgcn_sched_barrier(0);
      load_w(c + 2, wload);
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* hb = hbuf0 + (c & 1) * HBUF;
      const uint8_t* wb = wbuf0 + (c & 1) * WBUF;
      // Fragments of one sub-step are read from LDS, then its MFMAs issue
      // (the other wave on the SIMD covers the read latency).
      auto load_frags = [&](int s, bf16x8_t (&av)[kVB], bf16x8_t (&bv)[MBW]) {
        const int e = (4 * half + s) ^ swz(col);
#pragma unroll
        for (int vb = 0; vb < kVB; ++vb)
          av[vb] = as_bf16x8(*(const u32x4_t*)(wb + (wv * kVocabPerWave + vb * 32 + col) * 128 + (e << 4)));
#pragma unroll
        for (int pb = 0; pb < MBW; ++pb)
          bv[pb] = as_bf16x8(*(const u32x4_t*)(hb + (wp * PPW + pb * 32 + col) * 128 + (e << 4)));
      };
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t af[kVB], bf[MBW];
        load_frags(s, af, bf);
#pragma unroll
        for (int pb = 0; pb < MBW; ++pb)
#pragma unroll
          for (int vb = 0; vb < kVB; ++vb)
            acc[vb][pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[vb], bf[pb], acc[vb][pb], 0, 0, 0);
      }
      store_h((c + 1) & 1, hs);
      store_w((c + 1) & 1, wstore);
      __syncthreads();
    };

    u32x4_t wx[WSEG], wy[WSEG], hs[HSEG];
    __syncthreads();   // previous tile's readers of smem are done
    load_w(0, wx);
    load_w(1, wy);
    load_h(0, hs);
    store_w(0, wx);
    store_h(0, hs);
    __syncthreads();
    for (int c = 0; c < nk; c += 2) {
      chunk(c, wx, wy, hs);       // loads W(c+2) into wx, stores W(c+1) from wy
      chunk(c + 1, wy, wx, hs);   // loads W(c+3) into wy, stores W(c+2) from wx
    }

    // ---------------- epilogue: one position per lane per block ----------
    // One loop body for all blocks (not unrolled: it is long).  Block pb is
    // always taken from acc[.][0] and the accumulators are rotated down one
    // block at the end of the body, so every register index stays static.
#pragma unroll 1
    for (int pb = 0; pb < MBW; ++pb) {
      f32x16_t z[kVB];
#pragma unroll
      for (int vb = 0; vb < kVB; ++vb) z[vb] = acc[vb][0];
      const int r = row0 + wp * PPW + pb * 32 + col;
      const bool rvalid = r < a.M;
      int cv = rvalid ? r / a.L : 0;
      if constexpr (kUniformKey) cv = __builtin_amdgcn_readfirstlane(cv);
      const int p = r - cv * a.L;
      const uint32_t pabs = (uint32_t)(a.block * a.L + p);
      const uint32_t key0 = a.key[cv][0], key1 = a.key[cv][1];

      if constexpr (kLogits) {
        if (rvalid) {
#pragma unroll
          for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int v0 = vbase + vb * 32 + 8 * q + 4 * half;
              float* dst = a.logits + (size_t)r * a.V + v0;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (v0 + e < a.V) dst[e] = z[vb][4 * q + e];
            }
        }
      }

      const Rec wrec = tile_record<kUniformKey, kCap, kCap>(z, vbase, half, a.V, a.c2, a.cap_in, a.cap_out, pabs,
                                                      (uint32_t)a.gstep, key0, key1);
      if (half == 0) {
        Rec* slot = recs + wave * PPW + pb * 32 + col;
        rec_store(slot, rec_merge(rec_load(slot), wrec));
      }
#pragma unroll
      for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
        for (int k = 0; k + 1 < MBW; ++k) acc[vb][k] = acc[vb][k + 1];
    }
  }

  // ------- merge the four vocabulary waves of each position (fixed order) -------
  __syncthreads();
  for (int t = tid; t < MROWS; t += kPThreads) {
    const int gp = t / PPW, lp = t % PPW;
    Rec r = rec_load(recs + (gp * kVGroups) * PPW + lp);
#pragma unroll
    for (int w = 1; w < kVGroups; ++w) r = rec_merge(r, rec_load(recs + (gp * kVGroups + w) * PPW + lp));
    const int row = row0 + t;
    if (row < a.M) rec_store(a.part + (size_t)row * a.P + g, r);
  }
}

// ---------------------------------------------------------------------------
// Packed vocabulary table and the projection kernel that streams it
// ---------------------------------------------------------------------------
// dgd_pack_vocab() rewrites W [V][d] once into MFMA fragment order, so that
// every 128-bit load of the projection reads 1 KB of contiguous memory and
// lands directly in the A-operand registers (no LDS staging of W):
//   64-row group rg, 64-element hidden chunk c, MFMA step s (0..3),
//   32-row fragment f (0..1), lane l (0..63), element j (0..7)  ->
//   W[64 rg + 32 f + l%32][64 c + 32 (l/32) + 8 s + j]
// (the hidden-index permutation 32h + 8s + j is the one the H fragments use,
// so the summed products are exactly those of the plain dot product).  Rows
// past V and hidden elements past d are stored as zeros.
constexpr int kPackRows = 64;
constexpr uint32_t kPackChunkBytes = 8192;   // 4 steps x 2 fragments x 1 KB

__host__ __device__ inline int packed_chunks(int d) { return (d + kKChunk - 1) / kKChunk; }
__host__ __device__ inline int packed_groups(int V) { return (V + kPackRows - 1) / kPackRows; }

// 4-bit table in streaming order.  Per 64-row group rg and 64-element hidden
// chunk c, 2560 bytes:
//   [0, 1024)     fragment f = 0: lane l, 16 bytes = four 32-bit words, word s
//                 holding the codes of row 64 rg + l%32, hidden 64 c + 32 (l/32)
//                 + 8 s + j in nibble j (j = 0..7)
//   [1024, 2048)  the same for f = 1 (rows 64 rg + 32 + l%32)
//   [2048, 2560)  lane l, 8 bytes: bf16 scale and minimum of (f = 0 row, group
//                 2c + l/32), then of (f = 1 row, same group)
// Rows past V and groups past d hold zero codes, scales and minima (value 0).
constexpr uint32_t kQ4ChunkBytes = 2560;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

__global__ void __launch_bounds__(kThreads) k_pack_vocab_q4(const uint8_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ mins,
                                                            uint8_t* __restrict__ out, int V, int d,
                                                            int nk, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;   // (rg, c, lane)
  if (u >= units) return;
  const int lane = (int)(u & 63);
  const int64_t q = u >> 6;
  const int c = (int)(q % nk);
  const int64_t rg = q / nk;
  const int h = lane >> 5, ngroups = d / 32;
  const int grp = 2 * c + h;
  uint8_t* blk = out + q * kQ4ChunkBytes;
  uint32_t sm[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int64_t v = rg * kPackRows + 32 * f + (lane & 31);
    const bool ok = v < V && grp < ngroups;
    u32x4_t w = {0u, 0u, 0u, 0u};
    if (ok) {
      const uint32_t* src = (const uint32_t*)(codes + v * (d / 2) + grp * 16);
#pragma unroll
      for (int s = 0; s < 4; ++s) w[s] = src[s];
    }
    *(u32x4_t*)(blk + f * 1024 + lane * 16) = w;
    sm[f] = ok ? ((uint32_t)scales[v * ngroups + grp] | ((uint32_t)mins[v * ngroups + grp] << 16)) : 0u;
  }
  *(u32x2_t*)(blk + 2048 + lane * 8) = u32x2_t{sm[0], sm[1]};
}

// One 32-bit word of a dequantized A fragment: elements 2e and 2e+1 of the
// eight codes in `codes` (nibble j = element j), as bf16(fp32(s) q + fp32(m)).
__device__ __forceinline__ uint32_t q4_pair(uint32_t codes, int e, float sc, float mn) {
  // even elements in the low nibble of each byte, odd ones in the high: split
  // once into two byte vectors (shared by the four words of a fragment) and
  // convert byte e of each
  uint32_t lo = codes & 0x0F0F0F0Fu, hi = (codes >> 4) & 0x0F0F0F0Fu;
  // opaque to the combiner, so the byte conversions stay v_cvt_f32_ubyteN of
  // the split words (the same asm on the same code word merges across the
  // four calls) instead of a bit-field extract each
  asm("" : "+v"(lo), "+v"(hi));
  const float q0 = (float)((lo >> (8 * e)) & 0xFFu);
  const float q1 = (float)((hi >> (8 * e)) & 0xFFu);
  const float w0 = fmaf(sc, q0, mn), w1 = fmaf(sc, q1, mn);
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t p = {(__bf16)w0, (__bf16)w1};
  return __builtin_bit_cast(uint32_t, p);
}

__global__ void __launch_bounds__(kThreads) k_pack_vocab(const uint16_t* __restrict__ W,
                                                         uint16_t* __restrict__ Wp, int V, int d,
                                                         int nk, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (u >= units) return;
  const int lane = (int)(u & 63);
  const int f = (int)((u >> 6) & 1);
  const int s = (int)((u >> 7) & 3);
  const int64_t q = u >> 9;                      // rg * nk + c
  const int c = (int)(q % nk);
  const int64_t v = (q / nk) * kPackRows + 32 * f + (lane & 31);
  const int k = c * kKChunk + 32 * (lane >> 5) + 8 * s;
  u32x4_t val = {0u, 0u, 0u, 0u};
  if (v < V && k < d) val = *(const u32x4_t*)(W + v * d + k);
  *(u32x4_t*)(Wp + u * 8) = val;
}

// k_project_packed: the projection over a packed table.  Tile = 256
// vocabulary rows x MROWS = 32*NB positions, one workgroup per CU, 4*PW
// waves (PW per SIMD).  Wave w owns vocabulary rows 64*(w%4) .. +63 of the
// tile against positions (w/4)*PPW .. +PPW-1 (PPW = MROWS/PW): 2 x NBW MFMA
// fragments, 32*NBW fp32 accumulators in AGPRs.  PW = 1 keeps one wave per
// SIMD with 512 registers (each W fragment loaded once); PW = 2 runs two
// waves per SIMD with 256 registers each (the two waves of a vocabulary group
// load the same W fragments, the second from cache).
//
// K loop, per 64-element hidden chunk c:
//   * W: fragments go straight from memory into a ring of RING chunks of
//     registers; the loads of chunk c+RING are issued as chunk c's MFMAs free
//     their registers.  Chunks at or past nk read zeros without a memory
//     access (the loop is padded to whole rings).
//   * H: chunk c+HB reaches LDS by DMA (buffer_load ... lds) into the buffer
//     chunk c has just finished with; HB buffers, swizzled rows.
//   * one barrier per chunk, inside MFMA step 3 (see chunk()).
// The H stream is cyclic over the chunks, so a tile finds the first HB chunks
// of H already in LDS.
template <int NB, bool kLogits, bool kUniformKey, bool kCap, bool kTopK, bool kQ4, int PW, int RING,
          int HB>
__global__ void __launch_bounds__(256 * PW) __attribute__((amdgpu_waves_per_eu(PW, PW)))
k_project_packed(const ProjArgs a) {
  static_assert(NB == 1 || NB == 2 || NB == 4 || NB == 8, "NB");
  static_assert(PW == 1 || PW == 2, "PW");
  constexpr int THREADS = 256 * PW;
  constexpr int WAVES = 4 * PW;
  constexpr int NBW = (NB >= PW) ? NB / PW : 1;      // B fragments per wave
  constexpr int PPW = 32 * NBW;                       // positions per wave
  constexpr int MROWS = PPW * PW;                     // positions per tile
  constexpr int HSEG = MROWS * (kKChunk / 8) / THREADS;   // DMA loads per thread per chunk
  constexpr int HBUF = MROWS * kKChunk * 2;
  static_assert(HSEG >= 1 && HSEG * THREADS == MROWS * (kKChunk / 8), "tiling");
  static_assert(RING % HB == 0, "the H buffer of a chunk must be static in the unrolled ring");
  // VMEM operations a wave issues after its DMA of H(c+1) (step 3 of chunk
  // c+1-HB, after the barrier) before it waits for it (step 3 of chunk c):
  // the two W loads of that step 3, HB-2 whole chunks (8 W loads and HSEG
  // DMA loads each) and the six W loads of steps 0-2 of chunk c.  Tile
  // prologues only add loads after it, which keeps the wait sufficient.
  // With the 4-bit table a chunk has three W loads, all issued at the end of
  // step 3, so only those of that step 3 and of the HB-2 chunks between stay
  // in flight.
  constexpr int kDmaLag = kQ4 ? 3 + (HB - 2) * (3 + HSEG) : 2 + (HB - 2) * (8 + HSEG) + 6;
  static_assert(kDmaLag <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t hsm[HB][HBUF];
  __shared__ __attribute__((aligned(16))) Rec recs[WAVES * PPW];
  // self-conditioning band lists, kScWave entries per (wave, position)
  __shared__ __attribute__((aligned(16))) ScEnt slist[kTopK ? WAVES * PPW * kScWave : 1];

  const int tid = threadIdx.x;
  // wave indices are uniform: keep them (and the buffer resources built from
  // them) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 3, wp = wave >> 2;
  const int lane = tid & 63, half = lane >> 5, col = lane & 31;
  PHASE_AT(0, wall_clock64());
  PHASE_AT(1, clock64());
  int phase_tile = 0;

  int mt, g;
  tile_of_block(blockIdx.x, a.n_mtiles, a.P, mt, g);
  const int row0 = mt * MROWS;
  {
    const int last_row = min(row0 + MROWS, a.M) - 1;
    bool all_done = true;
    for (int c = row0 / a.L; c <= last_row / a.L; ++c) all_done &= (a.done[c] != 0);
    if (all_done) return;
  }
  for (int i = tid; i < WAVES * PPW; i += THREADS) rec_store(recs + i, rec_empty());
  if constexpr (kTopK)
    for (int i = tid; i < WAVES * PPW; i += THREADS) sc_list_clear(slist + i * kScWave);

  const int nk = packed_chunks(a.d);
  const int nkr = (nk + RING - 1) / RING * RING;   // chunk loop padded to whole rings
  const size_t d = (size_t)a.d;
  constexpr uint32_t kChunkBytes = kQ4 ? kQ4ChunkBytes : kPackChunkBytes;
  const uint32_t rg_bytes = (uint32_t)nk * kChunkBytes;
  const int n_rg = packed_groups(a.V);

  // W fragments of the wave's 64-row group in tile vt (empty past the end)
  auto wres_of = [&](int vt) {
    const int rg = vt * 4 + wv;
    const bool ok = vt < a.n_vtiles && rg < n_rg;
    return __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.W + (ok ? (size_t)rg * (rg_bytes / 2) : 0)), (short)0, ok ? (int)rg_bytes : 0,
        kRsrcWord3);
  };
  const __amdgpu_buffer_rsrc_t hres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.H + (size_t)row0 * d), (short)0, (int)((size_t)min(MROWS, a.M - row0) * d * 2),
      kRsrcWord3);
  const uint32_t lane_off = (uint32_t)lane * 16;

  // H chunks reach LDS by DMA: instruction i of wave w fills rows
  // (i*WAVES + w)*8 .. +7 of an H buffer, lane l writing slot l%8 of row l/8,
  // so that slot holds hidden segment (l%8) ^ swz(row).  Rows past M re-read
  // row M-1 and segments past d re-read segment 0 of their row: no access
  // leaves H, and the packed W is zero at those hidden indices, so they add
  // exact zeros (their rows are never stored).
  //
  // The DMA is written as inline assembly on purpose: the compiler's wait
  // insertion treats a pending LDS DMA as making the vector-memory counter
  // unordered and then waits for every load in flight (vmcnt(0)) before the
  // next use of a W register, which drains the W prefetch.  The waits the
  // DMA needs are explicit in the K loop instead (vmcnt before each barrier).
  const int hseg = (lane & 7) ^ swz((lane >> 3) + 8 * (wave & 1));
  const int last_rel = a.M - 1 - row0;
  const uint32_t d2 = (uint32_t)(d * 2);
  // loads i0 .. i1-1 of the chunk's HSEG (all by default)
  auto dma_h = [&](int c, uint8_t* hbuf, int i0 = 0, int i1 = -1) {
    if (i1 < 0) i1 = HSEG;
    const uint32_t koff = c * kKChunk + hseg * 8 < a.d ? (uint32_t)(c * kKChunk * 2) : 0u - (uint32_t)hseg * 16;
    const uint32_t lbase =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)hbuf + (uint32_t)wave * 1024u;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int r = min((i * WAVES + wave) * 8 + (lane >> 3), last_rel);
      const uint32_t off = (uint32_t)r * d2 + (uint32_t)hseg * 16 + koff;
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(off), "s"(hres), "{m0}"(lbase + (uint32_t)(i * WAVES * 1024)));
    }
  };
  // B fragment pb (of this wave's positions) of MFMA step s from an H buffer
  auto read_b = [&](const uint8_t* hb, int s, int pb) {
    const int e = (4 * half + s) ^ swz(col);
    return as_bf16x8(*(const u32x4_t*)(hb + (wp * PPW + pb * 32 + col) * 128 + (e << 4)));
  };

  bf16x8_t bfr[NBW];   // B fragments of the step in progress
  // prologue: H chunks 0 .. HB-1 (later tiles find them already in place)
#pragma unroll
  for (int b = 0; b < HB; ++b) dma_h(b < nk ? b : 0, hsm[b]);
  __builtin_amdgcn_s_waitcnt(waitcnt_enc(0, 0));
  __syncthreads();

  for (int vt = g; vt < a.n_vtiles; vt += a.P) {
    const int vbase = vt * kVocabTile + wv * kVocabPerWave;
    const __amdgpu_buffer_rsrc_t wr = wres_of(vt);
    if (phase_tile < 4) PHASE_AT(2 + 3 * phase_tile, wall_clock64());

    f32x16_t acc[kVB][NBW];
    auto zero_acc = [&]() {
#pragma unroll
      for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
        for (int pb = 0; pb < NBW; ++pb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[vb][pb][i] = 0.f;
    };
    if constexpr (kQ4) {
      // 4-bit table: a chunk is two code vectors and the scales (three loads),
      // so the ring is deeper for the same registers.  A fragments are
      // dequantized one 32-bit word at a time between the MFMAs of the step
      // before (two A buffers alternate by step parity), so the VALU work
      // runs while the matrix pipe is busy.
      u32x4_t qring[RING][2];
      u32x2_t sring[RING];
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        const uint32_t oob = (uint32_t)(r >= nk) << 31;
        const uint32_t base = (uint32_t)r * kQ4ChunkBytes;
        __builtin_amdgcn_sched_barrier(0);
        qring[r][0] = __builtin_amdgcn_raw_buffer_load_b128(wr, (base + lane_off) | oob, 0, kNonTemporal);
        __builtin_amdgcn_sched_barrier(0);
        qring[r][1] = __builtin_amdgcn_raw_buffer_load_b128(wr, (base + 1024u + lane_off) | oob, 0,
                                                            kNonTemporal);
        __builtin_amdgcn_sched_barrier(0);
        sring[r] = __builtin_amdgcn_raw_buffer_load_b64(wr, (base + 2048u + (uint32_t)lane * 8u) | oob, 0,
                                                        kNonTemporal);
      }
      __builtin_amdgcn_sched_barrier(0);
      zero_acc();
      u32x4_t abuf[2][2];   // [step parity][fragment f]: 8 bf16 each
      // word k (0..7) of the A fragments of step s: fragment k / 4, word k % 4
      auto deq_word = [&](const u32x4_t (&q)[2], const u32x2_t& sc, int s, int k, u32x4_t (&dst)[2]) {
        const int f = k / 4, e = k % 4;
        const uint32_t smw = sc[f];
        dst[f][e] = q4_pair(q[f][s], e, __uint_as_float(smw << 16), __uint_as_float(smw & 0xffff0000u));
      };
#pragma unroll
      for (int k = 0; k < 8; ++k) deq_word(qring[0], sring[0], 0, k, abuf[0]);

      auto chunk_q4 = [&](int c, u32x4_t (&qcur)[2], u32x2_t& scur, const u32x4_t (&qnext)[2],
                          const u32x2_t& snext, uint8_t* hcur, const uint8_t* hnext) {
        const uint32_t woob = (uint32_t)(c + RING >= nk) << 31;
        const uint32_t wbase = (uint32_t)(c + RING) * kQ4ChunkBytes;
        const int h2 = c + HB < nkr ? c + HB : c + HB - nkr;
        const int hc2 = h2 < nk ? h2 : 0;
        // the A word (pb) of the step after s: this chunk's codes, or the next
        // chunk's step 0 during step 3
        auto deq_next = [&](int s, int pb) {
          if (pb >= 8) return;
          if (s < 3) deq_word(qcur, scur, s + 1, pb, abuf[(s + 1) & 1]);
          else deq_word(qnext, snext, 0, pb, abuf[0]);
        };
        // One MFMA, the dequantized word(s) owed after this fragment pair,
        // the other MFMA, then the LDS read into the B register both have
        // issued from: the VALU work fills the matrix pipe's time of the
        // first MFMA as well (a wave waits at the issue of the second until
        // the pipe takes it).
        auto mfma1 = [&](int s, int pb, int f) {
          const bf16x8_t af = as_bf16x8(abuf[s & 1][f]);
          acc[f][pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[pb], acc[f][pb], 0, 0, 0);
        };
        auto deq_owed = [&](int s, int pb) {
          deq_next(s, pb);
          if constexpr (NBW < 8)
            if (pb == NBW - 1)
#pragma unroll
              for (int k = NBW; k < 8; ++k) deq_next(s, k);
        };
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
          for (int pb = 0; pb < NBW; ++pb) {
            __builtin_amdgcn_sched_barrier(0);
            mfma1(s, pb, 0);
            __builtin_amdgcn_sched_barrier(0);
            deq_owed(s, pb);
            __builtin_amdgcn_sched_barrier(0);
            mfma1(s, pb, 1);
            __builtin_amdgcn_sched_barrier(0);
            bfr[pb] = read_b(hcur, s + 1, pb);
          }
        }
#pragma unroll
        for (int pb = 0; pb < NBW / 2; ++pb) {
          __builtin_amdgcn_sched_barrier(0);
          mfma1(3, pb, 0);
          __builtin_amdgcn_sched_barrier(0);
          deq_owed(3, pb);
          __builtin_amdgcn_sched_barrier(0);
          mfma1(3, pb, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_enc(kDmaLag, 0));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < NBW / 2; ++pb) bfr[pb] = read_b(hnext, 0, pb);
        __builtin_amdgcn_sched_barrier(0);
        // the DMA of H(c+HB) spread over the MFMA windows of the second half
        {
          constexpr int NH = NBW - NBW / 2, PER = (HSEG + 2 * NH - 1) / (2 * NH);
#pragma unroll
          for (int j = 0; j < NH; ++j) {
            const int pb = NBW / 2 + j;
            __builtin_amdgcn_sched_barrier(0);
            mfma1(3, pb, 0);
            __builtin_amdgcn_sched_barrier(0);
            dma_h(hc2, hcur, min(HSEG, 2 * j * PER), min(HSEG, (2 * j + 1) * PER));
            deq_owed(3, pb);
            __builtin_amdgcn_sched_barrier(0);
            mfma1(3, pb, 1);
            __builtin_amdgcn_sched_barrier(0);
            dma_h(hc2, hcur, min(HSEG, (2 * j + 1) * PER), min(HSEG, (2 * j + 2) * PER));
            bfr[pb] = read_b(hnext, 0, pb);
          }
        }

        __builtin_amdgcn_sched_barrier(0);
        qcur[0] = __builtin_amdgcn_raw_buffer_load_b128(wr, (wbase + lane_off) | woob, 0, kNonTemporal);
        __builtin_amdgcn_sched_barrier(0);
        qcur[1] = __builtin_amdgcn_raw_buffer_load_b128(wr, (wbase + 1024u + lane_off) | woob, 0,
                                                        kNonTemporal);
        __builtin_amdgcn_sched_barrier(0);
        scur = __builtin_amdgcn_raw_buffer_load_b64(wr, (wbase + 2048u + (uint32_t)lane * 8u) | woob, 0,
                                                    kNonTemporal);
        __builtin_amdgcn_sched_barrier(0);
      };
#pragma unroll
      for (int pb = 0; pb < NBW; ++pb) bfr[pb] = read_b(hsm[0], 0, pb);
      for (int c = 0; c < nkr; c += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r)
          chunk_q4(c + r, qring[r], sring[r], qring[(r + 1) % RING], sring[(r + 1) % RING],
                   hsm[r % HB], hsm[(r + 1) % HB]);
      }
    } else {
      // W ring, first RING chunks of the tile, issued in chunk order (pinned:
      // vmcnt retires in order, so waits for the first chunks need not drain
      // the later ones)
      u32x4_t ring[RING][8];
#pragma unroll
      for (int r = 0; r < RING; ++r) {
        const uint32_t oob = (uint32_t)(r >= nk) << 31;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          __builtin_amdgcn_sched_barrier(0);
          ring[r][j] = __builtin_amdgcn_raw_buffer_load_b128(
              wr, ((uint32_t)r * kPackChunkBytes + lane_off + (uint32_t)j * 1024u) | oob, 0, kNonTemporal);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      zero_acc();

      // One chunk c (LDS buffer hcur, W registers wreg).  Per MFMA step s the
      // issue order is pinned by scheduling barriers: for each B fragment, its
      // two MFMAs and then the LDS read of the same fragment of step s+1 into
      // the register just consumed; then the two W loads of chunk c+RING into
      // the W registers of step s.  Step 3 is split around the chunk's only
      // barrier: the first half of its MFMAs, a wait for this wave's DMA of
      // H(c+1) (kDmaLag later loads may stay in flight) and for its LDS reads,
      // the barrier, then the reads of step 0 of chunk c+1 from hnext for the
      // first half, then the rest of the MFMAs with the DMA of H(c+HB) into
      // hcur spread over their issue windows, one or two loads after each
      // MFMA (every wave has read its last fragment of chunk c before the
      // barrier; the DMA loads are still all issued before the step's W
      // loads, so the count kDmaLag is unchanged).
      auto chunk = [&](int c, u32x4_t (&wreg)[8], uint8_t* hcur, const uint8_t* hnext) {
        const uint32_t woob = (uint32_t)(c + RING >= nk) << 31;
        const uint32_t wbase = (uint32_t)(c + RING) * kPackChunkBytes + lane_off;
        const int h2 = c + HB < nkr ? c + HB : c + HB - nkr;
        const int hc2 = h2 < nk ? h2 : 0;   // any valid chunk for a padding one
        auto mfma2 = [&](int s, int pb) {
          const bf16x8_t a0 = as_bf16x8(wreg[2 * s]), a1 = as_bf16x8(wreg[2 * s + 1]);
          acc[0][pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bfr[pb], acc[0][pb], 0, 0, 0);
          acc[1][pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bfr[pb], acc[1][pb], 0, 0, 0);
        };
        auto wload = [&](int s) {
          wreg[2 * s] = __builtin_amdgcn_raw_buffer_load_b128(
              wr, (wbase + (uint32_t)(2 * s) * 1024u) | woob, 0, kNonTemporal);
          wreg[2 * s + 1] = __builtin_amdgcn_raw_buffer_load_b128(
              wr, (wbase + (uint32_t)(2 * s + 1) * 1024u) | woob, 0, kNonTemporal);
        };
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
          for (int pb = 0; pb < NBW; ++pb) {
            __builtin_amdgcn_sched_barrier(0);
            mfma2(s, pb);
            __builtin_amdgcn_sched_barrier(0);
            bfr[pb] = read_b(hcur, s + 1, pb);
          }
          __builtin_amdgcn_sched_barrier(0);
          wload(s);
        }
#pragma unroll
        for (int pb = 0; pb < NBW / 2; ++pb) {
          __builtin_amdgcn_sched_barrier(0);
          mfma2(3, pb);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_enc(kDmaLag, 0));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < NBW / 2; ++pb) bfr[pb] = read_b(hnext, 0, pb);
        __builtin_amdgcn_sched_barrier(0);
        // the DMA of H(c+HB) spread over the MFMA windows of the second half
        {
          auto mfma1 = [&](int pb, int f) {
            acc[f][pb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wreg[6 + f]), bfr[pb], acc[f][pb],
                                                                 0, 0, 0);
          };
          constexpr int NH = NBW - NBW / 2, PER = (HSEG + 2 * NH - 1) / (2 * NH);
#pragma unroll
          for (int j = 0; j < NH; ++j) {
            const int pb = NBW / 2 + j;
            __builtin_amdgcn_sched_barrier(0);
            mfma1(pb, 0);
            __builtin_amdgcn_sched_barrier(0);
            dma_h(hc2, hcur, min(HSEG, 2 * j * PER), min(HSEG, (2 * j + 1) * PER));
            __builtin_amdgcn_sched_barrier(0);
            mfma1(pb, 1);
            __builtin_amdgcn_sched_barrier(0);
            dma_h(hc2, hcur, min(HSEG, (2 * j + 1) * PER), min(HSEG, (2 * j + 2) * PER));
            bfr[pb] = read_b(hnext, 0, pb);
          }
        }

        __builtin_amdgcn_sched_barrier(0);
        wload(3);
        __builtin_amdgcn_sched_barrier(0);
      };
      // step-0 fragments of chunk 0 (H chunk 0 is in hsm[0]: loaded in the
      // prologue or by the previous tile's stream, which waited for it)
#pragma unroll
      for (int pb = 0; pb < NBW; ++pb) bfr[pb] = read_b(hsm[0], 0, pb);
      for (int c = 0; c < nkr; c += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r) chunk(c + r, ring[r], hsm[r % HB], hsm[(r + 1) % HB]);
      }

    }

    if (phase_tile < 4) PHASE_AT(3 + 3 * phase_tile, wall_clock64());
    // ---------------- epilogue: one position per lane per block ----------
    // One loop body for EU blocks at a time (the body is long, so the loop
    // is not unrolled further).  Body block u is always taken from acc[.][u]
    // and the accumulators are rotated down EU blocks at the end of the body,
    // so every register index stays static and the accumulators never leave
    // AGPRs.
    constexpr int EU0 = kTopK ? DGD_EPI_UNROLL_TOPK : DGD_EPI_UNROLL;
    constexpr int EU = NBW < EU0 ? NBW : EU0;
    static_assert(NBW % EU == 0, "epilogue unroll");
#pragma unroll 1
    for (int pb0 = 0; pb0 < NBW; pb0 += EU) {
#pragma unroll
      for (int u = 0; u < EU; ++u) {
        const int pb = pb0 + u;
        f32x16_t z[kVB];
#pragma unroll
        for (int vb = 0; vb < kVB; ++vb) z[vb] = acc[vb][u];
        const int r = row0 + wp * PPW + pb * 32 + col;
        const bool rvalid = r < a.M;
        int cv = rvalid ? r / a.L : 0;
        if constexpr (kUniformKey) cv = __builtin_amdgcn_readfirstlane(cv);
        const int p = r - cv * a.L;
        const uint32_t pabs = (uint32_t)(a.block * a.L + p);
        const uint32_t key0 = a.key[cv][0], key1 = a.key[cv][1];

        if constexpr (kLogits) {
          if (rvalid) {
#pragma unroll
            for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int v0 = vbase + vb * 32 + 8 * q + 4 * half;
                float* dst = a.logits + (size_t)r * a.V + v0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (v0 + e < a.V) dst[e] = z[vb][4 * q + e];
              }
          }
        }
        const Rec wrec = tile_record<kUniformKey, kCap, kCap || kTopK>(z, vbase, half, a.V, a.c2, a.cap_in,
                                                                       a.cap_out,
                                                        pabs, (uint32_t)a.gstep, key0, key1);
        if (half == 0) {
          Rec* slot = recs + wave * PPW + pb * 32 + col;
          rec_store(slot, rec_merge(rec_load(slot), wrec));
        }
        if constexpr (kTopK) sc_tile_update(z, vbase, half, slist + (wave * PPW + pb * 32 + col) * kScWave);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
        for (int k = 0; k + EU < NBW; ++k) acc[vb][k] = acc[vb][k + EU];
    }
    if (phase_tile < 4) PHASE_AT(4 + 3 * phase_tile, wall_clock64());
    ++phase_tile;
  }

  // ------- merge the four vocabulary waves of each position (fixed order) -------
  __syncthreads();
  for (int t = tid; t < MROWS; t += THREADS) {
    const int tp = t / PPW, lp = t % PPW;
    Rec r = rec_load(recs + (tp * 4) * PPW + lp);
#pragma unroll
    for (int w = 1; w < 4; ++w) r = rec_merge(r, rec_load(recs + (tp * 4 + w) * PPW + lp));
    const int row = row0 + t;
    if (row < a.M) rec_store(a.part + (size_t)row * a.P + g, r);
  }
  PHASE_AT(14, wall_clock64());
  PHASE_AT(15, clock64());
  // ------- self-conditioning candidates: the four band lists of each position -------
  if constexpr (kTopK) {
    for (int t = tid; t < MROWS * kScCand; t += THREADS) {
      const int pos = t / kScCand, k = t % kScCand, band = k / kScWave, e = k % kScWave;
      const int w = (pos / PPW) * 4 + band;
      ScEnt ent = slist[(w * PPW + pos % PPW) * kScWave + e];
      if (e == kScWave - 1) ent.id |= kScWaveTag;
      const int row = row0 + pos;
      if (row < a.M) a.cand[((size_t)row * a.P + g) * kScCand + k] = ent;
    }
  }
}

// ---------------------------------------------------------------------------
// k_merge, k_commit
// ---------------------------------------------------------------------------
// Sum of one int per thread over the workgroup (wave butterflies, then LDS).
__device__ inline int block_sum_i32(int v, int* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int out = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) out += red[w];
  __syncthreads();
  return out;
}

// Block-wide sums of one double and four ints in a fixed order: each wave
// adds its lanes by an xor butterfly (every lane pairs the same values, so
// all lanes hold the same sum), then the wave sums are added in wave order.
// The double result therefore never depends on timing.
struct BlockSums {
  double d;
  int i[4];
};
__device__ inline BlockSums block_sums(double d, int i0, int i1, int i2, int i3, double* dred,
                                       int* ired) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int v[4] = {i0, i1, i2, i3};
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    d += __shfl_xor(d, off);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] += __shfl_xor(v[k], off);
  }
  if (lane == 0) {
    dred[wave] = d;
#pragma unroll
    for (int k = 0; k < 4; ++k) ired[4 * wave + k] = v[k];
  }
  __syncthreads();
  BlockSums o{0.0, {0, 0, 0, 0}};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    o.d += dred[w];
#pragma unroll
    for (int k = 0; k < 4; ++k) o.i[k] += ired[4 * w + k];
  }
  __syncthreads();
  return o;
}

typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));

// Commit phase of one canvas, run by one workgroup.  Every per-position
// input is read from memory once, into LDS, before the canvas's done flag is
// tested, so all of these loads are in flight together.  The mean entropy is
// a float64 sum in a fixed pairwise order (block_sums); the exclusive prefix
// over the ranked entropies is added by one lane in rank order.  Both are the
// same doubles whatever the timing.
__device__ void commit_canvas(const CommitArgs& a, int c) {
  // (entropy bits, position) of each eligible position, ~0 otherwise; two
  // padding keys (~0) after the last let the ranking read keys in pairs
  __shared__ __attribute__((aligned(16))) unsigned long long keys[DGD_MAX_CANVAS_LEN + 2];
  __shared__ unsigned long long ranked[DGD_MAX_CANVAS_LEN];  // eligible keys in rank order
  __shared__ int32_t stok[DGD_MAX_CANVAS_LEN];               // sampled token
  __shared__ int32_t sam[DGD_MAX_CANVAS_LEN];                // argmax
  __shared__ uint8_t sopen[DGD_MAX_CANVAS_LEN];              // not committed before this step
  __shared__ double dred[kWaves];
  __shared__ int ired[4 * kWaves];
  __shared__ int s_acc;
  __shared__ double s_edge_sum[2];   // running sums before ranks n_acc - 1 and n_acc
  const int tid = threadIdx.x;
  const int L = a.L;
  const size_t rbase = (size_t)c * L;
  const size_t cbase = (size_t)c * a.G + (size_t)a.block * L;

  double hs = 0.0;   // this thread's positions, in order
  int moved = 0, elig = 0, bad = 0, near_sample = 0;
  for (int p = tid; p < L; p += kThreads) {
    const float h = a.rowH[rbase + p];
    const int am = a.rowA[rbase + p];
    const int tk = a.rowTok[rbase + p];
    const int fl = a.rowF[rbase + p];
    const int prev = a.st_prev[rbase + p];
    const bool open = a.committed[cbase + p] == 0;
    sam[p] = am;
    stok[p] = tk;
    sopen[p] = open;
    moved += (am != prev);
    bad += (fl & kRowNonFinite) != 0;
    near_sample += (fl & kRowNearSample) != 0;
    const bool e = a.freeze == 0 || open;
    keys[p] = e ? (((unsigned long long)__float_as_uint(h) << 32) | (unsigned)p) : ~0ull;
    elig += e;
    hs += (double)h;
  }
  if (tid < 2) keys[L + tid] = ~0ull;
  if (a.st_done[c]) return;   // uniform: the whole workgroup leaves before any barrier
  const BlockSums sums = block_sums(hs, moved, elig, bad, near_sample, dred, ired);
  if (sums.i[2] > 0) {
    // a position without a distribution (non-finite logits): the canvas
    // stops with an error status; canvas, mask and argmax reference stay as
    // they were
    if (tid == 0) {
      a.st_status[c] = DGD_STATUS_NONFINITE;
      a.st_done[c] = 1;
      a.st_conv[c] = 0;
      a.st_steps[c] = a.step + 1;
      a.st_mean[c] = __builtin_nanf("");
      a.st_new[c] = 0;
      a.st_bsample[c] = sums.i[3];
      a.st_bcommit[c] = 0;
      a.st_bconv[c] = 0;
    }
    return;
  }
  const bool stable = sums.i[0] == 0;
  const int n_elig = sums.i[1];
  const double mean = sums.d / (double)L;
  const int sc = stable ? a.st_stable[c] + 1 : 0;
  const bool converged = mean < (double)a.conf && sc >= a.stab;
  const bool final_step = converged || a.step == a.N - 1;

  int new_commits = 0, near_commit = 0;
  if (final_step) {
    for (int p = tid; p < L; p += kThreads) {
      const size_t idx = cbase + p;
      const bool open = sopen[p];
      if (a.freeze == 0 || open) {
        a.canvas[idx] = a.final_emit ? sam[p] : stok[p];
        a.committed[idx] = 1;
        if (a.commit_step) a.commit_step[idx] = (int16_t)a.step;
        new_commits += open;
      }
    }
    new_commits = block_sum_i32(new_commits, ired);
    if (tid == 0) {
      a.st_done[c] = 1;
      a.st_conv[c] = converged ? 1 : 0;
      a.st_ncomm[c] = L;
    }
  } else {
    // rank the eligible keys, ascending (entropy bits order entropies >= 0;
    // positions break ties; keys are distinct)
    if (L <= 512) {
      // rank by counting: every thread compares its keys with all others
      for (int p = tid; p < L; p += kThreads) {
        const unsigned long long k = keys[p];
        if (k == ~0ull) continue;
        int rank = 0;
#pragma unroll 8
        for (int j = 0; j < L; j += 2) {
          const u64x2_t kk = *reinterpret_cast<const u64x2_t*>(keys + j);
          rank += (kk.x < k) + (kk.y < k);
        }
        ranked[rank] = k;
      }
    } else {
      int n2 = 1;
      while (n2 < L) n2 <<= 1;
      for (int i = tid; i < n2; i += kThreads) ranked[i] = i < L ? keys[i] : ~0ull;
      __syncthreads();
      for (int k = 2; k <= n2; k <<= 1) {   // bitonic sort
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int i = tid; i < n2; i += kThreads) {
            const int ixj = i ^ j;
            if (ixj > i) {
              const unsigned long long ki = ranked[i], kj = ranked[ixj];
              const bool up = (i & k) == 0;
              if ((ki > kj) == up) { ranked[i] = kj; ranked[ixj] = ki; }
            }
          }
          __syncthreads();
        }
      }
    }
    __syncthreads();
    // Exclusive float64 running sum over the ranks, in rank order.  Entropies
    // are >= 0 and rounding is monotone, so the sums never decrease: the
    // accepted ranks are the prefix before the first sum above the bound,
    // and the scan stops there.
    const double bound = (double)a.bound[c];
    if (tid == 0) {
      double run = 0.0, before_last = 0.0;
      int n_acc = n_elig;
      for (int r0 = 0; r0 < n_elig && n_acc == n_elig; r0 += 16) {   // 16 ranks per batch: the LDS reads overlap
        const int nb = min(16, n_elig - r0);
        double h[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          h[j] = j < nb ? (double)__uint_as_float((unsigned)(ranked[r0 + j] >> 32)) : 0.0;
        for (int j = 0; j < nb; ++j) {
          if (run > bound) {
            n_acc = r0 + j;
            break;
          }
          before_last = run;
          run += h[j];
        }
      }
      s_acc = n_acc;
      s_edge_sum[0] = before_last;   // before rank n_acc - 1 (the last accepted)
      s_edge_sum[1] = run;           // before rank n_acc (the first rejected, if any)
    }
    __syncthreads();
    const int n_acc = s_acc;
    // commit band: positions whose entropy is within kBandCommit of the last
    // accepted or the first rejected one, and those two ranks when the
    // running sum before them is within kBandCommit of the bound
    {
      const int e0 = n_acc - 1, e1 = n_acc;
      const bool has0 = e0 >= 0 && e0 < n_elig, has1 = e1 < n_elig;
      const double h0 = has0 ? (double)__uint_as_float((unsigned)(ranked[e0] >> 32)) : 0.0;
      const double h1 = has1 ? (double)__uint_as_float((unsigned)(ranked[e1] >> 32)) : 0.0;
      for (int rk = tid; rk < n_elig; rk += kThreads) {
        const double h = (double)__uint_as_float((unsigned)(ranked[rk] >> 32));
        bool nb = (has0 && fabs(h - h0) <= kBandCommit) || (has1 && fabs(h - h1) <= kBandCommit);
        nb |= (rk == e0 && has0 && fabs(s_edge_sum[0] - bound) <= kBandCommit);
        nb |= (rk == e1 && has1 && fabs(s_edge_sum[1] - bound) <= kBandCommit);
        near_commit += nb;
      }
    }
    const uint32_t k0 = a.key[c][0], k1 = a.key[c][1];
    for (int rk = tid; rk < n_elig; rk += kThreads) {
      const int p = (int)(ranked[rk] & 0xffffffffu);
      const size_t idx = cbase + p;
      if (rk < n_acc) {
        a.canvas[idx] = stok[p];
        a.committed[idx] = 1;
        if (a.commit_step) a.commit_step[idx] = (int16_t)a.step;
        ++new_commits;
      } else {
        const uint32_t pabs = (uint32_t)(a.block * L + p);
        const Philox4 w = philox4x32_10(0u, pabs, (uint32_t)a.gstep, 1u, k0, k1);
        a.canvas[idx] = word_to_token(w.x, (uint32_t)a.V);
        a.committed[idx] = 0;
      }
    }
    new_commits = block_sum_i32(new_commits, ired);
    near_commit = block_sum_i32(near_commit, ired);
    if (tid == 0) {
      a.st_conv[c] = 0;
      a.st_ncomm[c] = (a.freeze ? (L - n_elig) : 0) + new_commits;
    }
  }
  if (tid == 0) {
    a.st_stable[c] = sc;
    a.st_steps[c] = a.step + 1;
    a.st_mean[c] = (float)mean;
    a.st_new[c] = new_commits;
    a.st_status[c] = 0;
    a.st_bsample[c] = sums.i[3];
    a.st_bcommit[c] = near_commit;
    a.st_bconv[c] = fabs(mean - (double)a.conf) < kBandConv ? 1 : 0;
  }
  // the argmax canvas of this step becomes the reference of the next one
  for (int p = tid; p < L; p += kThreads) a.st_prev[rbase + p] = sam[p];
}

// ---------------------------------------------------------------------------
// k_rmsnorm: the output norm of the final hidden states
// ---------------------------------------------------------------------------
// float64 -> bfloat16 bits, one rounding to nearest with ties to even.  In
// bfloat16's normal range the double is rounded at its 45th fraction bit
// (keeping bfloat16's 7) with an integer add on its bit pattern; the result
// has 8 significant bits and converts to float exactly.  Below 2^-126 the
// spacing is bfloat16's subnormal step 2^-133: scale, round to an integer
// (rint: ties to even), scale back, all exact in double.
__device__ inline uint16_t f64_to_bf16_rne(double v) {
  if (fabs(v) < 0x1p-126) {
    const double q = rint(v * 0x1p133) * 0x1p-133;
    return (uint16_t)(__float_as_uint((float)q) >> 16);
  }
  uint64_t u = (uint64_t)__double_as_longlong(v);
  u += ((1ull << 44) - 1) + ((u >> 45) & 1);
  u &= ~((1ull << 45) - 1);
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

__device__ inline double bf16_f64(uint32_t bits16) {
  return (double)__uint_as_float(bits16 << 16);
}

// One workgroup per row of H: h = w * x * sqrt(d) / (||x|| + eps), with the
// squared norm summed in double (16-byte loads, per-lane partial sums, then a
// butterfly and an LDS pass over the four waves), every product and the
// quotient in double in that order, and one rounding to bfloat16.  The row is
// read twice; the second read comes from cache.
__global__ void __launch_bounds__(kThreads) k_rmsnorm(const uint16_t* __restrict__ H,
                                                      const uint16_t* __restrict__ w,
                                                      uint16_t* __restrict__ out, int d,
                                                      double sqrt_d, double eps) {
  __shared__ double red[kWaves];
  const size_t row = blockIdx.x;
  const u32x4_t* x4 = (const u32x4_t*)(H + row * d);
  const u32x4_t* w4 = (const u32x4_t*)w;
  u32x4_t* o4 = (u32x4_t*)(out + row * d);
  const int n8 = d >> 3;
  double ss = 0.0;
  for (int k = threadIdx.x; k < n8; k += kThreads) {
    const u32x4_t v = x4[k];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double lo = bf16_f64(v[j] & 0xffffu), hi = bf16_f64(v[j] >> 16);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) tot += red[i];
  const double den = sqrt(tot) + eps;
  for (int k = threadIdx.x; k < n8; k += kThreads) {
    const u32x4_t v = x4[k], g = w4[k];
    u32x4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double xl = bf16_f64(v[j] & 0xffffu), xh = bf16_f64(v[j] >> 16);
      const double wl = bf16_f64(g[j] & 0xffffu), wh = bf16_f64(g[j] >> 16);
      const uint32_t bl = f64_to_bf16_rne(wl * xl * sqrt_d / den);
      const uint32_t bh = f64_to_bf16_rne(wh * xh * sqrt_d / den);
      r[j] = bl | (bh << 16);
    }
    o4[k] = r;
  }
}

// Grid (ceil(L/4), B); one wave per position merges that position's partial
// records (fixed order: lanes over the groups, then a butterfly).
__global__ void __launch_bounds__(kThreads) k_merge(const CommitArgs a) {
  constexpr int kPerLane = kMaxGroups / 64;   // records per lane (P <= kMaxGroups)
  const int c = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int p = blockIdx.x * kWaves + wave;
  if (p >= a.L) return;
  const size_t r = (size_t)c * a.L + p;
  const Rec* pr = a.part + r * a.P;
  // Every record load is issued before the first is used and before the done
  // flag is tested (the records lie in the workspace either way), so the
  // loads overlap instead of queueing behind one another.
  Rec part[kPerLane];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j)
    part[j] = lane + 64 * j < a.P ? rec_load(pr + lane + 64 * j) : rec_empty();
  if (a.st_done[c]) return;
  Rec rec = rec_empty();
#pragma unroll
  for (int j = 0; j < kPerLane; ++j)
    if (lane + 64 * j < a.P) rec = rec_merge(rec, part[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Rec o = rec_shfl_xor(rec, off);
    const bool upper = (lane & off) != 0;
    rec = rec_merge(rec_pick(upper, o, rec), rec_pick(upper, rec, o));
  }
  if (lane == 0) {
    const double S = (double)rec.S, A = (double)rec.A;
    // A NaN or +inf logit leaves a non-finite maximum, sum or moment (NaN
    // never wins a comparison, so it cannot hide in them); logits that are
    // all -inf leave no argmax.  Such a position has no distribution: it is
    // flagged, its entropy is NaN and its ids -1, and the commit kernel stops
    // the canvas instead of ranking or sampling it.
    const bool finite = isfinite(rec.m) && isfinite(rec.S) && isfinite(rec.A) &&
                        isfinite(rec.y1) && rec.S > 0.f && rec.am != kNoIndex &&
                        rec.i1 != kNoIndex;
    double Hn = kLn2 * (log2(S) - A / S);
    if (Hn < 0.0) Hn = 0.0;   // rounding below the exact minimum (0, a one-hot row)
    const float H = finite ? (float)Hn : __builtin_nanf("");
    const float gap = finite ? (float)(((double)rec.y1 - (double)rec.y2) * kLn2) : __builtin_nanf("");
    const int32_t am = finite ? rec.am : -1, tok = finite ? rec.i1 : -1;
    a.rowM[r] = rec.m;
    a.rowS[r] = rec.S;
    a.rowH[r] = H;
    a.rowA[r] = am;
    a.rowTok[r] = tok;
    a.rowF[r] = (finite ? 0 : kRowNonFinite) | ((double)gap < kBandSample ? kRowNearSample : 0);
    if (a.out_entropy) a.out_entropy[r] = H;
    if (a.out_argmax) a.out_argmax[r] = am;
    if (a.out_token) a.out_token[r] = tok;
    if (a.out_gap) a.out_gap[r] = gap;
  }
}

// ---------------------------------------------------------------------------
// k_sc_topk: the K most probable tokens of each position
// ---------------------------------------------------------------------------
// One workgroup per position.  The candidate pool starts as the position's
// band lists of every group; keys order candidates by (logit desc, id asc):
//   key = ord(x) << 32 | (0xFFFFFF - id) << 8 | tags,   0 = no candidate.
// Selection: the K-th largest of the per-thread maxima bounds the K-th key
// from below; the keys above that bound (at most 32 K) are sorted in LDS.
// While a tagged candidate's value reaches the K-th selected value, the part
// of the vocabulary its list covered (the lane's 32 ids in one tile, or the
// whole band of the group) is recomputed exactly with fp32 dot products, its
// old candidates leave the pool, the recomputed ones join it, and the
// selection runs again.
constexpr int kScMaxK = DGD_SC_MAX_TOPK;
constexpr int kScPoolExtra = 4096;          // recomputed candidates per position
constexpr int kScSortMax = 32 * kScMaxK;    // keys above the bound

struct ScArgs {
  const ScEnt* cand;      // [M][P][kScCand]
  const float* rowM;
  const float* rowS;
  const uint16_t* H;      // rows the projection read
  const uint16_t* W;      // packed table
  const int32_t* done;
  float* out_prob;        // [M][K]
  int32_t* out_id;        // [M][K]
  int32_t* out_status;    // [M] or null
  int32_t M, V, d, L, P, K, n_vtiles;
  float c2, cap_in, cap_out;
  int32_t cap;
};

__device__ __forceinline__ uint64_t sc_key(float x, uint32_t idtag) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  const uint32_t id = idtag & kScIdBits;
  return ((uint64_t)ord << 32) | ((uint64_t)(0xFFFFFFu - id) << 8) | (idtag >> 30);
}
__device__ __forceinline__ float sc_key_x(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ __forceinline__ uint32_t sc_key_id(uint64_t k) {
  return 0xFFFFFFu - (uint32_t)((k >> 8) & 0xFFFFFFu);
}

// Descending bitonic sort of buf[0..n), n a power of two <= 2 * kThreads * 8.
__device__ void sc_sort_desc(uint64_t* buf, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = buf[i], y = buf[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            buf[i] = y;
            buf[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Descending bitonic sort of the 64 R keys one wave holds, key i = lane R + r
// in v[r]: compare-exchanges inside a lane for distances below R, across
// lanes (by shuffle) above.  No barriers.
template <int R>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&v)[R]) {
  const int lane = threadIdx.x & 63;
  constexpr int N = 64 * R;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if ((r ^ j) > r) {
            const int i = lane * R + r;
            const bool desc = (i & k) == 0;
            const uint64_t x = v[r], y = v[r ^ j];
            const bool swap = desc ? (x < y) : (x > y);
            v[r] = swap ? y : x;
            v[r ^ j] = swap ? x : y;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int i = lane * R + r;
          const uint64_t o = __shfl_xor(v[r], j / R);
          const bool keep_max = ((i & j) == 0) == ((i & k) == 0);
          v[r] = keep_max ? max(v[r], o) : min(v[r], o);
        }
      }
    }
  }
}

// Tempered logit of vocabulary id v for one position, recomputed from the
// packed table: an fp32 dot product in hidden order, then the same
// temperature (or softcap) transform as the projection's epilogue.
__device__ float sc_logit(const ScArgs& a, const uint16_t* hrow, int v) {
  const int nk = packed_chunks(a.d);
  const int rg = v / kPackRows, f = (v % kPackRows) / 32, lv = v % 32;
  float acc = 0.f;
  // two chunks per round, their 16 table pieces and 16 hidden pieces loaded
  // before any product (pieces past d are skipped; sums stay in hidden order)
  for (int c0 = 0; c0 < nk; c0 += 2) {
    u32x4_t w[16], x[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int c = c0 + q / 8, h = (q / 4) % 2, s = q % 4;
      const int k0 = c * kKChunk + 32 * h + 8 * s;
      if (c < nk && k0 < a.d) {
        const size_t u = ((((size_t)rg * nk + c) * 4 + s) * 2 + f) * 64 + lv + 32 * h;
        w[q] = *(const u32x4_t*)(a.W + u * 8);
        x[q] = *(const u32x4_t*)(hrow + k0);
      } else {
        w[q] = u32x4_t{0u, 0u, 0u, 0u};
        x[q] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(__uint_as_float(x[q][j] << 16), __uint_as_float(w[q][j] << 16), acc);
        acc = fmaf(__uint_as_float(x[q][j] & 0xffff0000u), __uint_as_float(w[q][j] & 0xffff0000u), acc);
      }
  }
  return a.cap ? softcap_bits(acc, a.cap_in, a.cap_out) : __fmul_rn(acc, a.c2);
}

__global__ void __launch_bounds__(kThreads) k_sc_topk(const ScArgs a) {
  __shared__ uint64_t pool[kMaxGroups * kScCand + kScPoolExtra];
  __shared__ uint64_t sbuf[kScSortMax];
  __shared__ uint64_t tmax[kThreads];
  __shared__ int s_cnt;
  __shared__ uint64_t s_bound;
  __shared__ uint64_t s_tagged;
  const int row = blockIdx.x;
  if (a.done[row / a.L]) return;
  const int tid = threadIdx.x;
  {
    // a position without a distribution (non-finite logits; its canvas
    // stops in k_commit): no ids, NaN probabilities, status -2
    const float m = a.rowM[row], S = a.rowS[row];
    if (!(isfinite(m) && isfinite(S) && S > 0.f)) {
      if (tid < a.K) {
        a.out_prob[(size_t)row * a.K + tid] = __builtin_nanf("");
        a.out_id[(size_t)row * a.K + tid] = -1;
      }
      if (tid == 0 && a.out_status) a.out_status[row] = -2;
      return;
    }
  }
  const int n0 = a.P * kScCand;
  {
    // all loads first (independent), then the keys
    constexpr int kPer = kMaxGroups * kScCand / kThreads;
    ScEnt e[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * kThreads;
      if (i < n0) e[j] = a.cand[(size_t)row * n0 + i];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + j * kThreads;
      if (i < n0) pool[i] = (e[j].id & kScIdBits) < (uint32_t)a.V ? sc_key(e[j].x, e[j].id) : 0ull;
    }
  }
  int npool = n0;
  int status = 0;
  const uint16_t* hrow = a.H + (size_t)row * a.d;
  __syncthreads();
  for (;;) {
    // ---- select: bound from the per-thread maxima (sorted by wave 0), then
    // sort what is above it (one wave when it fits, else the whole block)
    uint64_t mx = 0;
    for (int i = tid; i < npool; i += kThreads) mx = max(mx, pool[i]);
    tmax[tid] = mx;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    if (tid < 64) {
      uint64_t v[kThreads / 64];
#pragma unroll
      for (int r = 0; r < kThreads / 64; ++r) v[r] = tmax[tid * (kThreads / 64) + r];
      wave_sort_desc(v);
#pragma unroll
      for (int r = 0; r < kThreads / 64; ++r)
        if (tid * (kThreads / 64) + r == a.K - 1) s_bound = v[r];
    }
    __syncthreads();
    const uint64_t bound = s_bound;
    for (int i = tid; i < npool; i += kThreads) {
      const uint64_t k = pool[i];
      if (k != 0 && k >= bound) sbuf[atomicAdd(&s_cnt, 1)] = k;
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (cnt <= 64) {
      if (tid < 64) {
        uint64_t v[1] = {tid < cnt ? sbuf[tid] : 0ull};
        wave_sort_desc(v);
        sbuf[tid] = v[0];
      }
      __syncthreads();
    } else {
      int n = 128;
      while (n < cnt) n <<= 1;
      for (int i = cnt + tid; i < n; i += kThreads) sbuf[i] = 0;
      __syncthreads();
      sc_sort_desc(sbuf, n);
    }
    // ---- a tagged candidate whose value reaches the K-th selected value:
    // its list may have dropped values as large as its own (the largest such
    // key is taken; none, and the selection is exact)
    const uint64_t kth = sbuf[a.K - 1];
    const uint32_t kth_ord = (uint32_t)(kth >> 32);     // 0 when fewer than K
    if (tid == 0) s_tagged = 0;
    __syncthreads();
    {
      uint64_t best = 0;
      for (int i = tid; i < npool; i += kThreads) {
        const uint64_t k = pool[i];
        if ((k & 3ull) && (uint32_t)(k >> 32) >= kth_ord) best = max(best, k);
      }
      if (best) atomicMax((unsigned long long*)&s_tagged, (unsigned long long)best);
    }
    __syncthreads();
    const uint64_t tagged = s_tagged;
    if (tagged == 0) break;
    // ---- recompute the part of the vocabulary the tagged list covered
    const uint32_t tid_v = sc_key_id(tagged);
    const int vt = (int)(tid_v / kVocabTile), band = (int)(tid_v % kVocabTile) / kVocabPerWave;
    const int g = vt % a.P;
    const bool whole_band = (tagged & 1ull) != 0;     // band list tag (id bit 30)
    const int tiles = whole_band ? (a.n_vtiles - g + a.P - 1) / a.P : 1;
    const int seg = whole_band ? tiles * kVocabPerWave : 32;
    if (npool + seg > n0 + kScPoolExtra) { status = -1; break; }
    // drop the part's candidates
    const int half = (int)(tid_v % 8) / 4;
    for (int i = tid; i < npool; i += kThreads) {
      const uint64_t k = pool[i];
      if (k == 0) continue;
      const uint32_t v = sc_key_id(k);
      const int kvt = (int)(v / kVocabTile), kband = (int)(v % kVocabTile) / kVocabPerWave;
      const bool in = whole_band ? (kvt % a.P == g && kband == band)
                                 : (kvt == vt && kband == band && (int)(v % 8) / 4 == half);
      if (in) pool[i] = 0;
    }
    // recompute it: one id per thread
    for (int i = tid; i < seg; i += kThreads) {
      int v;
      if (whole_band) {
        v = (g + (i / kVocabPerWave) * a.P) * kVocabTile + band * kVocabPerWave + i % kVocabPerWave;
      } else {
        v = vt * kVocabTile + band * kVocabPerWave + (i / 16) * 32 + 8 * ((i / 4) % 4) + 4 * half + i % 4;
      }
      pool[npool + i] = v < a.V ? sc_key(sc_logit(a, hrow, v), (uint32_t)v) : 0ull;
    }
    npool += seg;
    ++status;
    __syncthreads();
  }
  // ---- outputs: probabilities 2^(x - m) / S, best first
  if (tid < a.K) {
    // (a key of 0 is left only when the recomputation budget ran out)
    const uint64_t k = sbuf[tid];
    const float p = k ? fexp2(sc_key_x(k) - a.rowM[row]) / a.rowS[row] : 0.f;
    a.out_prob[(size_t)row * a.K + tid] = p;
    a.out_id[(size_t)row * a.K + tid] = k ? (int32_t)sc_key_id(k) : -1;
  }
  if (tid == 0 && a.out_status) a.out_status[row] = status;
}

// ---------------------------------------------------------------------------
// k_sc_embed: the self-conditioning input, scale * sum_j bf16(p_j) E[id_j]
// ---------------------------------------------------------------------------
// One workgroup per row.  The row's K (probability, id) pairs go to LDS
// first; each thread then owns 8 consecutive hidden elements (16 bytes of
// every table row) and adds the K scaled pieces in order, in fp32, with the
// loads of 8 pieces in flight at a time, and rounds once to bf16 (nearest,
// ties to even).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ void __launch_bounds__(kThreads) k_sc_embed(const float* __restrict__ prob,
                                                       const int32_t* __restrict__ ids, int K,
                                                       const uint16_t* __restrict__ W, int packed,
                                                       int V, int d, float scale,
                                                       uint16_t* __restrict__ out) {
  __shared__ float sp[kScMaxK];
  __shared__ int32_t sid[kScMaxK];
  const int row = blockIdx.x;
  if (threadIdx.x < K) {
    // bf16(p); ids outside [0, V) contribute nothing (weight 0, row 0)
    const int v = ids[(size_t)row * K + threadIdx.x];
    const bool ok = v >= 0 && v < V;
    sp[threadIdx.x] = ok ? __uint_as_float(f32_to_bf16_rne(prob[(size_t)row * K + threadIdx.x]) << 16) : 0.f;
    sid[threadIdx.x] = ok ? v : 0;
  }
  __syncthreads();
  const int nk = packed_chunks(d);
  for (int k0 = threadIdx.x * 8; k0 < d; k0 += kThreads * 8) {
    const int c = k0 / kKChunk, h = (k0 % kKChunk) / 32, s = (k0 % 32) / 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < K; j0 += 8) {
      u32x4_t w[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int j = j0 + jj < K ? j0 + jj : K - 1;
        const int v = sid[j];
        size_t off;
        if (packed) {
          const int rg = v / kPackRows, f = (v % kPackRows) / 32, lv = v % 32;
          off = (((((size_t)rg * nk + c) * 4 + s) * 2 + f) * 64 + lv + 32 * h) * 8;
        } else {
          off = (size_t)v * d + k0;
        }
        w[jj] = *(const u32x4_t*)(W + off);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj >= K) break;
        const float pj = sp[j0 + jj];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(pj, __uint_as_float(w[jj][e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(pj, __uint_as_float(w[jj][e] & 0xffff0000u), acc[2 * e + 1]);
        }
      }
    }
    u32x4_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = f32_to_bf16_rne(acc[2 * e] * scale) | (f32_to_bf16_rne(acc[2 * e + 1] * scale) << 16);
    *(u32x4_t*)(out + (size_t)row * d + k0) = r;
  }
}

// ---------------------------------------------------------------------------
// k_label: the sparse label read
// ---------------------------------------------------------------------------
// One workgroup per row.  Wave w takes labels w, w + 4, ...: its lanes take
// 16-byte pieces of the hidden dimension (consecutive pieces on consecutive
// lanes), add 8 fp32 products each, and a butterfly sums the lanes.  The
// logits (capped when asked) go to LDS; the block then forms the tempered
// softmax over the labels in bits: p = 2^(x2 - m) / S with x2 = z * log2(e) / T.
struct LabelArgs {
  const uint16_t* H;      // [rows][d]
  const uint16_t* W;      // table, row-major or packed
  float* logits;          // [rows][n] or null
  float* probs;           // [rows][n]
  int32_t rows, V, d, n, packed;
  float c2, cap_in, cap;  // cap: c (0 = off)
  int32_t labels[DGD_MAX_LABELS];
};

__device__ __forceinline__ float block_max_f32(float v, float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float out = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) out = fmaxf(out, red[w]);
  __syncthreads();
  return out;
}

__device__ __forceinline__ float block_sum_f32(float v, float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float out = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) out += red[w];
  __syncthreads();
  return out;
}

__global__ void __launch_bounds__(kThreads) k_label(const LabelArgs a) {
  __shared__ float zs[DGD_MAX_LABELS];
  __shared__ float red[kWaves];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint16_t* hrow = a.H + (size_t)row * a.d;
  const int nk = packed_chunks(a.d), n8 = a.d / 8;
  for (int l = wave; l < a.n; l += kWaves) {
    const int v = a.labels[l];
    const int rg = v / kPackRows, f = (v % kPackRows) / 32, lv = v % 32;
    float acc = 0.f;
    for (int q = lane; q < n8; q += 64) {
      const int k0 = q * 8;
      size_t off;
      if (a.packed) {
        const int c = k0 / kKChunk, h = (k0 % kKChunk) / 32, sidx = (k0 % 32) / 8;
        off = (((((size_t)rg * nk + c) * 4 + sidx) * 2 + f) * 64 + lv + 32 * h) * 8;
      } else {
        off = (size_t)v * a.d + k0;
      }
      const u32x4_t w = *(const u32x4_t*)(a.W + off);
      const u32x4_t x = *(const u32x4_t*)(hrow + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(__uint_as_float(x[j] << 16), __uint_as_float(w[j] << 16), acc);
        acc = fmaf(__uint_as_float(x[j] & 0xffff0000u), __uint_as_float(w[j] & 0xffff0000u), acc);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) zs[l] = a.cap != 0.f ? softcap_bits(acc, a.cap_in, a.cap) : acc;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int l = tid; l < a.n; l += kThreads) m = fmaxf(m, zs[l] * a.c2);
  m = block_max_f32(m, red);
  float sum = 0.f;
  for (int l = tid; l < a.n; l += kThreads) sum += fexp2(zs[l] * a.c2 - m);
  sum = block_sum_f32(sum, red);
  for (int l = tid; l < a.n; l += kThreads) {
    a.probs[(size_t)row * a.n + l] = fexp2(zs[l] * a.c2 - m) / sum;
    if (a.logits) a.logits[(size_t)row * a.n + l] = zs[l];
  }
}

// Grid (B): the commit of every canvas that is not done, one workgroup each
// (the kernel boundary after k_merge publishes the per-position results).
__global__ void __launch_bounds__(kThreads) k_commit(const CommitArgs a) {
  commit_canvas(a, blockIdx.x);
}

// Grid (ceil(L/256), B).
__global__ void __launch_bounds__(kThreads) k_init_block(const InitArgs a) {
  const int c = blockIdx.y;
  const int p = blockIdx.x * kThreads + threadIdx.x;
  if (p < a.L) {
    const uint32_t pabs = (uint32_t)(a.block * a.L + p);
    const size_t idx = (size_t)c * a.G + pabs;
    const Philox4 w = philox4x32_10(0u, pabs, (uint32_t)a.block, 2u, a.key[c][0], a.key[c][1]);
    a.canvas[idx] = word_to_token(w.x, (uint32_t)a.V);
    a.committed[idx] = 0;
    a.st_prev[(size_t)c * a.L + p] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.st_stable[c] = 0;
    a.st_done[c] = 0;
    a.st_steps[c] = 0;
    a.st_conv[c] = 0;
    a.st_ncomm[c] = 0;
    a.st_mean[c] = 0.f;
    a.st_new[c] = 0;
    a.st_status[c] = 0;
    a.st_bsample[c] = 0;
    a.st_bcommit[c] = 0;
    a.st_bconv[c] = 0;
  }
}

__global__ void k_debug_gumbel(const uint32_t* words, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = gumbel_bits(words[i]);
}

// The generator the kernels use, for validation: per-call keys (the
// general form) or one key for all calls (the form whose key lives in scalar
// registers, as the fused step uses it when a 32-row block is in one canvas).
__global__ void k_debug_philox(const u32x4_t* ctr, const u32x2_t* key, uint32_t k0, uint32_t k1,
                               u32x4_t* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const u32x4_t c = ctr[i];
  Philox4 p;
  if (key) {
    const u32x2_t k = key[i];
    p = philox4x32_10(c[0], c[1], c[2], c[3], k[0], k[1]);
  } else {
    p = philox4x32_10_uniform_key(c[0], c[1], c[2], c[3], k0, k1);
  }
  out[i] = u32x4_t{p.x, p.y, p.z, p.w};
}

// ---------------------------------------------------------------------------
// Ceilings: what this GPU sustains on the projection's two resources
// ---------------------------------------------------------------------------
// HBM: every thread streams 16-byte non-temporal loads over the buffer, four
// in flight, and folds them with XOR into one word per workgroup.
__global__ void __launch_bounds__(256) k_ceiling_hbm(const u32x4_t* __restrict__ buf, int64_t n16,
                                                     uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(buf + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x % 1024, x);
}

// MFMA: one wave per SIMD, eight A and eight B fragments of real data in
// registers (from `ops`), every (A, B) pair per round into eight
// accumulators: 64 independent v_mfma_f32_32x32x16_bf16 per round.
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_ceiling_mfma(const u32x4_t* __restrict__ ops, int64_t n16, int64_t rounds, float* sink) {
  const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
  bf16x8_t a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = as_bf16x8(ops[(base + k) % n16]);
    b[k] = as_bf16x8(ops[(base + 8 + k) % n16]);
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int64_t r = 0; r < rounds; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += acc[j][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DGD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t part, rowM, rowS, rowH, rowA, rowTok, rowF, cand, total;
  int P;
};

WsLayout ws_layout(int B, int L, int V) {
  WsLayout w{};
  const size_t M = (size_t)B * L;
  w.P = num_groups(V);
  size_t off = 0;
  w.part = off;     off = align256(off + M * (size_t)w.P * sizeof(Rec));
  w.rowM = off;     off = align256(off + M * sizeof(float));
  w.rowS = off;     off = align256(off + M * sizeof(float));
  w.rowH = off;     off = align256(off + M * sizeof(float));
  w.rowA = off;     off = align256(off + M * sizeof(int32_t));
  w.rowTok = off;   off = align256(off + M * sizeof(int32_t));
  w.rowF = off;     off = align256(off + M * sizeof(int32_t));
  w.cand = off;     off = align256(off + M * (size_t)w.P * kScCand * sizeof(ScEnt));
  w.total = off;
  return w;
}

struct StateView {
  int32_t *prev, *stable, *done, *steps, *conv, *ncomm, *newc, *status, *bsample, *bcommit, *bconv;
  float* mean;
};

StateView state_view(void* state, int B, int L) {
  int32_t* s = (int32_t*)state;
  const size_t BL = (size_t)B * L;
  StateView v;
  v.prev = s;
  v.stable = s + BL;
  v.done = s + BL + B;
  v.steps = s + BL + 2 * (size_t)B;
  v.conv = s + BL + 3 * (size_t)B;
  v.ncomm = s + BL + 4 * (size_t)B;
  v.mean = (float*)(s + BL + 5 * (size_t)B);
  v.newc = s + BL + 6 * (size_t)B;
  v.status = s + BL + 7 * (size_t)B;
  v.bsample = s + BL + 8 * (size_t)B;
  v.bcommit = s + BL + 9 * (size_t)B;
  v.bconv = s + BL + 10 * (size_t)B;
  return v;
}

bool finite01(float x) { return std::isfinite(x) && x >= 0.f && x <= 1.f; }

int check_shape(const dgd_ctx* ctx) {
  if (!ctx) return fail(DGD_EINVAL, "ctx is NULL");
  if (ctx->B < 1 || ctx->B > DGD_MAX_CANVASES)
    return fail(DGD_EUNSUPPORTED, "B=%d outside [1, %d]", ctx->B, DGD_MAX_CANVASES);
  if (ctx->L < 1 || ctx->L > DGD_MAX_CANVAS_LEN)
    return fail(DGD_EUNSUPPORTED, "L=%d outside [1, %d]", ctx->L, DGD_MAX_CANVAS_LEN);
  if (ctx->G < ctx->L || ctx->G > DGD_MAX_GEN_LENGTH || ctx->G % ctx->L != 0)
    return fail(DGD_EINVAL, "G=%d must be a multiple of L=%d in [L, %d]", ctx->G, ctx->L,
                DGD_MAX_GEN_LENGTH);
  if (ctx->V < 1 || ctx->V > DGD_MAX_VOCAB)
    return fail(DGD_EUNSUPPORTED, "V=%d outside [1, 2^24]", ctx->V);
  if (ctx->d < 8 || ctx->d > DGD_MAX_HIDDEN || ctx->d % 8 != 0)
    return fail(DGD_EUNSUPPORTED, "d=%d must be a multiple of 8 in [8, %d]", ctx->d,
                DGD_MAX_HIDDEN);
  if (!ctx->state) return fail(DGD_EINVAL, "ctx->state is NULL");
  if (ctx->vocab_layout != DGD_VOCAB_ROWS && ctx->vocab_layout != DGD_VOCAB_PACKED &&
      ctx->vocab_layout != DGD_VOCAB_Q4)
    return fail(DGD_EINVAL, "vocab_layout=%d is not DGD_VOCAB_ROWS, DGD_VOCAB_PACKED or DGD_VOCAB_Q4",
                ctx->vocab_layout);
  if (ctx->vocab_layout == DGD_VOCAB_Q4 && ctx->d % 32 != 0)
    return fail(DGD_EUNSUPPORTED, "d=%d: the 4-bit table needs a multiple of 32", ctx->d);
  return DGD_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The optional self-conditioning outputs.
int check_sc(const dgd_ctx* ctx) {
  const int K = ctx->sc_topk;
  if (K == 0) return DGD_OK;
  if (K < 0 || K > DGD_SC_MAX_TOPK) return fail(DGD_EINVAL, "sc_topk=%d outside [0, %d]", K, DGD_SC_MAX_TOPK);
  if (K > ctx->V) return fail(DGD_EINVAL, "sc_topk=%d exceeds V=%d", K, ctx->V);
  if (ctx->vocab_layout != DGD_VOCAB_PACKED)
    return fail(DGD_EUNSUPPORTED, "sc_topk needs the packed vocabulary layout");
  if (!ctx->sc_prob || !ctx->sc_id) return fail(DGD_EINVAL, "sc_topk is set but sc_prob/sc_id is NULL");
  return DGD_OK;
}

// The optional lm-head tail; H_bytes is the extent of H (all steps for dgd_run).
int check_tail(const dgd_ctx* ctx, const void* H, size_t H_bytes) {
  const float c = ctx->softcap;
  if (!std::isfinite(c) || (c != 0.f && (c < 0.01f || c > 10000.f)))
    return fail(DGD_EINVAL, "softcap=%g must be 0 or in [0.01, 10000]", c);
  if (!ctx->norm_weight) return DGD_OK;
  if (!ctx->norm_h) return fail(DGD_EINVAL, "norm_weight is set but norm_h is NULL");
  if (!aligned16(ctx->norm_weight) || !aligned16(ctx->norm_h))
    return fail(DGD_EINVAL, "norm_weight/norm_h is not 16-byte aligned");
  if (!finite01(ctx->norm_eps)) return fail(DGD_EINVAL, "norm_eps=%g outside [0, 1]", ctx->norm_eps);
  const uintptr_t h0 = (uintptr_t)H, h1 = h0 + H_bytes;
  const uintptr_t n0 = (uintptr_t)ctx->norm_h, n1 = n0 + (size_t)ctx->B * ctx->L * ctx->d * 2;
  if (h0 < n1 && n0 < h1) return fail(DGD_EINVAL, "norm_h overlaps H");
  return DGD_OK;
}

int check_params(const dgd_params* prm) {
  if (!prm) return fail(DGD_EINVAL, "params is NULL");
  const int N = prm->num_inference_steps;
  if (N < 1 || N > DGD_MAX_STEPS) return fail(DGD_EINVAL, "num_inference_steps=%d outside [1, 1024]", N);
  if (!finite01(prm->t_min) || !finite01(prm->t_max))
    return fail(DGD_EINVAL, "t_min=%g / t_max=%g must be finite and in [0, 1]", prm->t_min, prm->t_max);
  const double tlast = (double)prm->t_max + ((double)(N - 1) / N) * ((double)prm->t_min - prm->t_max);
  if (!(prm->t_max >= kMinTemperature) || !(tlast >= kMinTemperature))
    return fail(DGD_EINVAL, "temperature schedule goes below %g (t_min=%g, t_max=%g)",
                kMinTemperature, prm->t_min, prm->t_max);
  if (!finite01(prm->confidence)) return fail(DGD_EINVAL, "confidence=%g outside [0, 1]", prm->confidence);
  if (prm->stability_threshold < 0 || prm->stability_threshold > DGD_MAX_STEPS)
    return fail(DGD_EINVAL, "stability_threshold=%d outside [0, 1024]", prm->stability_threshold);
  if (prm->freeze != 0 && prm->freeze != 1) return fail(DGD_EINVAL, "freeze must be 0 or 1");
  if (prm->final_emit != 0 && prm->final_emit != 1) return fail(DGD_EINVAL, "final_emit must be 0 or 1");
  return DGD_OK;
}

int check_knobs(const dgd_ctx* ctx, const uint64_t* seed, bool need_bounds) {
  if (!seed) return fail(DGD_EINVAL, "seed is NULL");
  if (need_bounds) {
    if (!ctx->entropy_bound) return fail(DGD_EINVAL, "ctx->entropy_bound is NULL");
    for (int c = 0; c < ctx->B; ++c)
      if (!finite01(ctx->entropy_bound[c]))
        return fail(DGD_EINVAL, "entropy_bound[%d]=%g outside [0, 1]", c, ctx->entropy_bound[c]);
  }
  return DGD_OK;
}

// Checks shared by the step entry points (own_workspace: the caller's
// ctx->workspace must be there and large enough).
int check_step(const dgd_bf16* H, const dgd_bf16* W_vocab, int32_t* canvas, uint8_t* committed,
               int32_t block, int32_t step, const dgd_params* params, const uint64_t* seed,
               const dgd_ctx* ctx, bool own_workspace);

int check_workspace(const dgd_ctx* ctx) {
  const WsLayout w = ws_layout(ctx->B, ctx->L, ctx->V);
  if (!ctx->workspace) return fail(DGD_EINVAL, "ctx->workspace is NULL");
  if (((uintptr_t)ctx->workspace & 255) != 0) return fail(DGD_EINVAL, "workspace is not 256-byte aligned");
  if (ctx->workspace_bytes < w.total)
    return fail(DGD_EWORKSPACE, "workspace has %zu bytes, needs %zu", ctx->workspace_bytes, w.total);
  return DGD_OK;
}

int check_step(const dgd_bf16* H, const dgd_bf16* W_vocab, int32_t* canvas, uint8_t* committed,
               int32_t block, int32_t step, const dgd_params* params, const uint64_t* seed,
               const dgd_ctx* ctx, bool own_workspace) {
  int rc = check_shape(ctx);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if ((rc = check_knobs(ctx, seed, true))) return rc;
  if (own_workspace && (rc = check_workspace(ctx))) return rc;
  if (!H || !W_vocab || !canvas || !committed) return fail(DGD_EINVAL, "H/W_vocab/canvas/committed is NULL");
  if (!aligned16(H) || !aligned16(W_vocab)) return fail(DGD_EINVAL, "H/W_vocab is not 16-byte aligned");
  if ((rc = check_tail(ctx, H, (size_t)ctx->B * ctx->L * ctx->d * 2))) return rc;
  if ((rc = check_sc(ctx))) return rc;
  if (block < 0 || block >= ctx->G / ctx->L)
    return fail(DGD_EINVAL, "block=%d outside [0, %d)", block, ctx->G / ctx->L);
  if (step < 0 || step >= params->num_inference_steps)
    return fail(DGD_EINVAL, "step=%d outside [0, %d)", step, params->num_inference_steps);
  return DGD_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation step
// ---------------------------------------------------------------------------
// A workspace per GPU in a file-scope device array, for callers that cannot
// allocate (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Every GPU the library runs on holds its own copy until
// the process ends.  The array's name in host code is a host-side stand-in,
// not a device address: its address on a device comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that pointer reaches kernels.  The step carries no data in it from one
// call to the next (every byte a step reads, the same step wrote first), so
// nothing needs clearing; calls that overlap on one GPU race on it.
constexpr size_t kScratchBytes = 32u << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, or null

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DGD_EUNSUPPORTED, "device %d: the no-allocation step serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255) != 0) return fail(DGD_EHIP, "scratch address %p is unusable", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DGD_OK;
}

void fill_keys(uint32_t (*key)[2], const uint64_t* seed, int B) {
  for (int c = 0; c < B; ++c) {
    key[c][0] = (uint32_t)(seed[c] & 0xffffffffu);
    key[c][1] = (uint32_t)(seed[c] >> 32);
  }
}

int launch_init(int32_t* canvas, uint8_t* committed, int block, const uint64_t* seed,
                const dgd_ctx* ctx) {
  InitArgs a{};
  a.canvas = canvas;
  a.committed = committed;
  const StateView sv = state_view(ctx->state, ctx->B, ctx->L);
  a.st_prev = sv.prev; a.st_stable = sv.stable; a.st_done = sv.done; a.st_steps = sv.steps;
  a.st_conv = sv.conv; a.st_ncomm = sv.ncomm; a.st_mean = sv.mean; a.st_new = sv.newc;
  a.st_status = sv.status; a.st_bsample = sv.bsample; a.st_bcommit = sv.bcommit;
  a.st_bconv = sv.bconv;
  a.B = ctx->B; a.L = ctx->L; a.G = ctx->G; a.V = ctx->V; a.block = block;
  fill_keys(a.key, seed, ctx->B);
  const dim3 grid((ctx->L + kThreads - 1) / kThreads, ctx->B);
  hipLaunchKernelGGL(k_init_block, grid, dim3(kThreads), 0, (hipStream_t)ctx->stream, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_init_block launch");
}

struct Timer {
  std::vector<hipEvent_t> ev;
  bool on = false;
  int begin(hipStream_t s) {
    if (!on) return DGD_OK;
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return hip_fail(r, "hipEventCreate");
    ev.push_back(e);
    r = hipEventRecord(e, s);
    return r == hipSuccess ? DGD_OK : hip_fail(r, "hipEventRecord");
  }
  // Events come in threes per step: before the projection, after it, and
  // after the step's last kernel.
  int finish(const dgd_ctx* ctx) {
    if (!on) return DGD_OK;
    double total = 0.0, tail = 0.0;
    int n = 0;
    int rc = DGD_OK;
    if (!ev.empty()) {
      hipError_t r = hipEventSynchronize(ev.back());
      if (r != hipSuccess) rc = hip_fail(r, "hipEventSynchronize");
      for (size_t i = 0; rc == DGD_OK && i + 2 < ev.size(); i += 3) {
        float ms = 0.f, ms2 = 0.f;
        r = hipEventElapsedTime(&ms, ev[i], ev[i + 1]);
        if (r == hipSuccess) r = hipEventElapsedTime(&ms2, ev[i + 1], ev[i + 2]);
        if (r != hipSuccess) { rc = hip_fail(r, "hipEventElapsedTime"); break; }
        total += ms;
        tail += ms2;
        ++n;
      }
    }
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    if (rc == DGD_OK) {
      *ctx->k1_ms = total;
      if (ctx->k1_launches) *ctx->k1_launches = n;
      if (ctx->tail_ms) *ctx->tail_ms = tail;
    }
    return rc;
  }
};

// Calls f(std::integral_constant<bool, b>...) for run-time flags b...: one
// kernel instantiation per combination.
template <bool... Bs, typename F>
void with_flags(F&& f) { f(std::integral_constant<bool, Bs>{}...); }
template <bool... Bs, typename F, typename... Rest>
void with_flags(F&& f, bool b, Rest... rest) {
  if (b) with_flags<Bs..., true>(f, rest...);
  else with_flags<Bs..., false>(f, rest...);
}

struct Flags {
  bool logits, uniform, cap, topk, q4;
};

template <int MB>
void launch_project_mb(const ProjArgs& a, dim3 grid, hipStream_t s, Flags fl) {
  with_flags([&](auto lg, auto uni, auto cap) {
    hipLaunchKernelGGL((k_project<MB, decltype(lg)::value, decltype(uni)::value, decltype(cap)::value>),
                       grid, dim3(kPThreads), 0, s, a);
  }, fl.logits, fl.uniform, fl.cap);
}

// Launch shape of the packed projection: one wave per SIMD, a two-chunk W
// register ring, two H buffers.  (Measured on the 256 x 262144 x 2816 step:
// two waves per SIMD with 256 registers each ran 12% slower, since both waves
// of a vocabulary group load the same W fragments; deeper W rings and H DMA
// leads changed nothing or ran slower.)
constexpr int kPackedPW = 1, kPackedRing = 2, kPackedHB = 2;

// The 4-bit table keeps four chunks in its register ring (10 registers per
// chunk against 32 for bf16 fragments).
constexpr int kQ4Ring = 4;

// Workgroups that fill MI355X's 256 compute units once (the packed
// projection runs one workgroup per CU).
constexpr int kFillWorkgroups = 256;

template <int NB>
void launch_packed_nb(const ProjArgs& a, dim3 grid, hipStream_t s, Flags fl) {
  constexpr int PW = kPackedPW, HB = kPackedHB;
  with_flags([&](auto lg, auto uni, auto cap, auto topk, auto q4) {
    constexpr bool kQ4 = decltype(q4)::value, kTopK = decltype(topk)::value;
    constexpr int R = kQ4 ? kQ4Ring : kPackedRing;
    // (the top-K recomputation reads bf16 fragments: never with a 4-bit table)
    if constexpr (!(kQ4 && kTopK))
      hipLaunchKernelGGL((k_project_packed<NB, decltype(lg)::value, decltype(uni)::value,
                                           decltype(cap)::value, kTopK, kQ4, PW, R, HB>),
                         grid, dim3(256 * PW), 0, s, a);
  }, fl.logits, fl.uniform, fl.cap, fl.topk, fl.q4);
}

int launch_step(const dgd_bf16* H, const dgd_bf16* W, int32_t* canvas, uint8_t* committed,
                int block, int step, const dgd_params* prm, const uint64_t* seed,
                const dgd_ctx* ctx, Timer& timer) {
  const int B = ctx->B, L = ctx->L, V = ctx->V, dd = ctx->d;
  const int M = B * L;
  const int N = prm->num_inference_steps;
  const WsLayout wl = ws_layout(B, L, V);
  uint8_t* ws = (uint8_t*)ctx->workspace;
  const StateView sv = state_view(ctx->state, B, L);
  hipStream_t stream = (hipStream_t)ctx->stream;
  const int gstep = block * N + step;
  const double T = (double)prm->t_max + ((double)step / N) * ((double)prm->t_min - prm->t_max);

  if (ctx->norm_weight) {
    hipLaunchKernelGGL(k_rmsnorm, dim3(M), dim3(kThreads), 0, stream, H, ctx->norm_weight,
                       ctx->norm_h, dd, std::sqrt((double)dd), (double)ctx->norm_eps);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return hip_fail(e0, "k_rmsnorm launch");
    H = ctx->norm_h;
  }

  ProjArgs pa{};
  pa.H = H; pa.W = W;
  pa.part = (Rec*)(ws + wl.part);
  pa.logits = ctx->logits;
  pa.done = sv.done;
  pa.M = M; pa.V = V; pa.d = dd; pa.L = L; pa.B = B;
  pa.P = wl.P;
  pa.n_vtiles = num_vtiles(V);
  pa.block = block; pa.gstep = gstep;
  pa.c2 = (float)(kLog2e / T);
  const bool cap = ctx->softcap != 0.f;
  if (cap) {
    pa.cap_in = (float)(2.0 * kLog2e / ctx->softcap);
    pa.cap_out = (float)(ctx->softcap * kLog2e / T);
  }
  fill_keys(pa.key, seed, B);
  const bool topk = ctx->sc_topk > 0;
  if (topk) pa.cand = (ScEnt*)(ws + wl.cand);
  const bool q4 = ctx->vocab_layout == DGD_VOCAB_Q4;
  const Flags fl{ctx->logits != nullptr, (L % 32) == 0, cap, topk, q4};
  int rc;
  if (ctx->vocab_layout == DGD_VOCAB_PACKED || ctx->vocab_layout == DGD_VOCAB_Q4) {
    int NB = M <= 32 ? 1 : M <= 64 ? 2 : M <= 128 ? 4 : 8;
    // A small vocabulary leaves CUs idle (one workgroup per tile and group):
    // split the positions into more tiles until the grid covers every CU.
    // Each (position, group) record is computed the same way in any tiling.
    while (NB > 1 && ((M + 32 * NB - 1) / (32 * NB)) * wl.P < kFillWorkgroups) NB >>= 1;
    pa.n_mtiles = (M + 32 * NB - 1) / (32 * NB);
    const dim3 grid1(pa.n_mtiles * pa.P);
    if ((rc = timer.begin(stream))) return rc;
    switch (NB) {
      case 1: launch_packed_nb<1>(pa, grid1, stream, fl); break;
      case 2: launch_packed_nb<2>(pa, grid1, stream, fl); break;
      case 4: launch_packed_nb<4>(pa, grid1, stream, fl); break;
      default: launch_packed_nb<8>(pa, grid1, stream, fl); break;
    }
  } else {
    const int MB = M <= 64 ? 2 : M <= 128 ? 4 : 8;
    pa.n_mtiles = (M + 32 * MB - 1) / (32 * MB);
    const dim3 grid1(pa.n_mtiles * pa.P);
    if ((rc = timer.begin(stream))) return rc;
    switch (MB) {
      case 2: launch_project_mb<2>(pa, grid1, stream, fl); break;
      case 4: launch_project_mb<4>(pa, grid1, stream, fl); break;
      default: launch_project_mb<8>(pa, grid1, stream, fl); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "k_project launch");
  rc = timer.begin(stream);
  if (rc) return rc;

  CommitArgs ca{};
  ca.part = pa.part; ca.P = wl.P;
  ca.rowM = (float*)(ws + wl.rowM);
  ca.rowS = (float*)(ws + wl.rowS);
  ca.rowH = (float*)(ws + wl.rowH);
  ca.rowA = (int32_t*)(ws + wl.rowA);
  ca.rowTok = (int32_t*)(ws + wl.rowTok);
  ca.rowF = (int32_t*)(ws + wl.rowF);
  ca.out_entropy = ctx->entropy; ca.out_argmax = ctx->argmax;
  ca.out_token = ctx->token; ca.out_gap = ctx->gap;
  ca.commit_step = ctx->commit_step;
  ca.canvas = canvas; ca.committed = committed;
  ca.st_prev = sv.prev; ca.st_stable = sv.stable; ca.st_done = sv.done; ca.st_steps = sv.steps;
  ca.st_conv = sv.conv; ca.st_ncomm = sv.ncomm; ca.st_mean = sv.mean; ca.st_new = sv.newc;
  ca.st_status = sv.status; ca.st_bsample = sv.bsample; ca.st_bcommit = sv.bcommit;
  ca.st_bconv = sv.bconv;
  ca.B = B; ca.L = L; ca.G = ctx->G; ca.V = V; ca.N = N;
  ca.block = block; ca.step = step; ca.gstep = gstep;
  ca.freeze = prm->freeze; ca.final_emit = prm->final_emit; ca.stab = prm->stability_threshold;
  ca.conf = prm->confidence;
  for (int c = 0; c < B; ++c) ca.bound[c] = ctx->entropy_bound[c];
  fill_keys(ca.key, seed, B);
  const dim3 grid2((L + kWaves - 1) / kWaves, B);
  hipLaunchKernelGGL(k_merge, grid2, dim3(kThreads), 0, stream, ca);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "k_merge launch");
  if (topk) {
    // before k_commit: a canvas this step finishes still gets its distribution
    ScArgs sa{};
    sa.cand = pa.cand; sa.rowM = ca.rowM; sa.rowS = ca.rowS;
    sa.H = pa.H; sa.W = pa.W; sa.done = sv.done;
    sa.out_prob = ctx->sc_prob; sa.out_id = ctx->sc_id; sa.out_status = ctx->sc_status;
    sa.M = M; sa.V = V; sa.d = dd; sa.L = L; sa.P = wl.P; sa.K = ctx->sc_topk;
    sa.n_vtiles = pa.n_vtiles;
    sa.c2 = pa.c2; sa.cap_in = pa.cap_in; sa.cap_out = pa.cap_out; sa.cap = cap ? 1 : 0;
    hipLaunchKernelGGL(k_sc_topk, dim3(M), dim3(kThreads), 0, stream, sa);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "k_sc_topk launch");
  }
  hipLaunchKernelGGL(k_commit, dim3(B), dim3(kThreads), 0, stream, ca);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "k_commit launch");
  return timer.begin(stream);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* dgd_last_error(void) { return g_err.c_str(); }

int dgd_phase_times(uint64_t* dst, size_t n) {
  g_err.clear();
  if (!dst) return fail(DGD_EINVAL, "dst is NULL");
  if (n > (size_t)kPhaseWorkgroups * 4 * kPhaseSlots)
    return fail(DGD_EINVAL, "n=%zu exceeds %d entries", n, kPhaseWorkgroups * 4 * kPhaseSlots);
#ifdef DGD_PHASE_TIMING
  const hipError_t e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_phase), n * sizeof(uint64_t));
  return e == hipSuccess ? DGD_OK : hip_fail(e, "hipMemcpyFromSymbol(phase times)");
#else
  return fail(DGD_EUNSUPPORTED, "phase timing is recorded only by a library built with "
                                "DGD_PHASE_TIMING (build.py --phase-timing)");
#endif
}

size_t dgd_state_bytes(int32_t B, int32_t L) {
  if (B < 1 || L < 1) return 0;
  return ((size_t)B * L + kStateWordsPerCanvas * (size_t)B) * 4;
}

size_t dgd_workspace_bytes(int32_t B, int32_t L, int32_t V, int32_t d) {
  if (B < 1 || B > DGD_MAX_CANVASES || L < 1 || L > DGD_MAX_CANVAS_LEN || V < 1 ||
      V > DGD_MAX_VOCAB || d < 8 || d > DGD_MAX_HIDDEN || d % 8 != 0)
    return 0;
  return ws_layout(B, L, V).total;
}

int dgd_init_block(int32_t* canvas, uint8_t* committed, int32_t block, const dgd_params* params,
                   const uint64_t* seed, const dgd_ctx* ctx) {
  g_err.clear();
  int rc = check_shape(ctx);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if ((rc = check_knobs(ctx, seed, false))) return rc;
  if (!canvas || !committed) return fail(DGD_EINVAL, "canvas/committed is NULL");
  if (block < 0 || block >= ctx->G / ctx->L)
    return fail(DGD_EINVAL, "block=%d outside [0, %d)", block, ctx->G / ctx->L);
  return launch_init(canvas, committed, block, seed, ctx);
}

int dgd_step(const dgd_bf16* H, const dgd_bf16* W_vocab, int32_t* canvas, uint8_t* committed,
             int32_t block, int32_t step, const dgd_params* params, const uint64_t* seed,
             const dgd_ctx* ctx) {
  g_err.clear();
  int rc = check_step(H, W_vocab, canvas, committed, block, step, params, seed, ctx, true);
  if (rc) return rc;
  Timer timer;
  timer.on = ctx->k1_ms != nullptr;
  rc = launch_step(H, W_vocab, canvas, committed, block, step, params, seed, ctx, timer);
  const int rt = timer.finish(ctx);
  return rc ? rc : rt;
}

int dgd_step_noalloc(const dgd_bf16* H, const dgd_bf16* W_vocab, int32_t* canvas,
                     uint8_t* committed, int32_t block, int32_t step, const dgd_params* params,
                     const uint64_t* seed, const dgd_ctx* ctx) {
  g_err.clear();
  int rc = check_step(H, W_vocab, canvas, committed, block, step, params, seed, ctx, false);
  if (rc) return rc;
  if (ctx->k1_ms)
    return fail(DGD_EINVAL, "kernel timing (k1_ms) creates HIP events: not offered by the "
                            "no-allocation step");
  const WsLayout w = ws_layout(ctx->B, ctx->L, ctx->V);
  const size_t need = ctx->sc_topk > 0 ? w.total : w.cand;   // candidates only with a top-K
  if (need > kScratchBytes)
    return fail(DGD_EUNSUPPORTED, "this shape needs %zu bytes of scratch; the no-allocation step "
                                  "has %zu", need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  dgd_ctx c = *ctx;
  c.workspace = ws;
  c.workspace_bytes = kScratchBytes;
  Timer timer;   // off: no events
  return launch_step(H, W_vocab, canvas, committed, block, step, params, seed, &c, timer);
}

int dgd_run_steps(const dgd_bf16* H_steps, const dgd_bf16* W_vocab, int32_t* canvas,
                  uint8_t* committed, int32_t first_step, int32_t n_steps,
                  const dgd_params* params, const uint64_t* seed, const dgd_ctx* ctx) {
  g_err.clear();
  int rc = check_shape(ctx);
  if (rc) return rc;
  if ((rc = check_params(params))) return rc;
  if ((rc = check_knobs(ctx, seed, true))) return rc;
  if ((rc = check_workspace(ctx))) return rc;
  if (!H_steps || !W_vocab || !canvas || !committed)
    return fail(DGD_EINVAL, "H_steps/W_vocab/canvas/committed is NULL");
  if (!aligned16(H_steps) || !aligned16(W_vocab))
    return fail(DGD_EINVAL, "H_steps/W_vocab is not 16-byte aligned");
  const int N = params->num_inference_steps;
  const int blocks = ctx->G / ctx->L;
  const int64_t total = (int64_t)blocks * N;
  if (first_step < 0 || n_steps < 0 || (int64_t)first_step + n_steps > total)
    return fail(DGD_EINVAL, "steps [%d, %d + %d) outside the run's %lld steps", first_step,
                first_step, n_steps, (long long)total);
  const size_t step_elems = (size_t)ctx->B * ctx->L * ctx->d;
  if ((rc = check_tail(ctx, H_steps, (size_t)blocks * N * step_elems * 2))) return rc;
  if ((rc = check_sc(ctx))) return rc;
  Timer timer;
  timer.on = ctx->k1_ms != nullptr;
  for (int g = first_step; g < first_step + n_steps && rc == DGD_OK; ++g) {
    const int b = g / N, s = g % N;
    if (s == 0) rc = launch_init(canvas, committed, b, seed, ctx);
    if (rc == DGD_OK)
      rc = launch_step(H_steps + (size_t)g * step_elems, W_vocab, canvas, committed, b, s, params,
                       seed, ctx, timer);
  }
  const int rt = timer.finish(ctx);
  return rc ? rc : rt;
}

int dgd_run(const dgd_bf16* H_steps, const dgd_bf16* W_vocab, int32_t* canvas, uint8_t* committed,
            const dgd_params* params, const uint64_t* seed, const dgd_ctx* ctx) {
  if (!ctx || !params) {
    g_err.clear();
    return fail(DGD_EINVAL, "ctx/params is NULL");
  }
  const int64_t total = ctx->L > 0 ? (int64_t)(ctx->G / ctx->L) * params->num_inference_steps : 0;
  if (total > INT32_MAX) {
    g_err.clear();
    return fail(DGD_EINVAL, "too many steps");
  }
  return dgd_run_steps(H_steps, W_vocab, canvas, committed, 0, (int32_t)total, params, seed, ctx);
}

size_t dgd_packed_vocab_bytes(int32_t V, int32_t d) {
  if (V < 1 || V > DGD_MAX_VOCAB || d < 8 || d > DGD_MAX_HIDDEN || d % 8 != 0) return 0;
  return (size_t)packed_groups(V) * kPackRows * (size_t)packed_chunks(d) * kKChunk * 2;
}

size_t dgd_q4_vocab_bytes(int32_t V, int32_t d) {
  if (V < 1 || V > DGD_MAX_VOCAB || d < 32 || d > DGD_MAX_HIDDEN || d % 32 != 0) return 0;
  return (size_t)packed_groups(V) * (size_t)packed_chunks(d) * kQ4ChunkBytes;
}

int dgd_pack_vocab_q4(const uint8_t* codes, const dgd_bf16* scales, const dgd_bf16* mins, void* W_q4,
                      int32_t V, int32_t d, void* stream) {
  g_err.clear();
  if (!codes || !scales || !mins || !W_q4) return fail(DGD_EINVAL, "codes/scales/mins/W_q4 is NULL");
  if (V < 1 || V > DGD_MAX_VOCAB) return fail(DGD_EUNSUPPORTED, "V=%d outside [1, 2^24]", V);
  if (d < 32 || d > DGD_MAX_HIDDEN || d % 32 != 0)
    return fail(DGD_EUNSUPPORTED, "d=%d must be a multiple of 32 in [32, %d]", d, DGD_MAX_HIDDEN);
  if (((uintptr_t)codes & 15) || ((uintptr_t)scales & 1) || ((uintptr_t)mins & 1) || !aligned16(W_q4))
    return fail(DGD_EINVAL, "codes/W_q4 must be 16-byte and scales/mins 2-byte aligned");
  const size_t bytes = dgd_q4_vocab_bytes(V, d);
  const uintptr_t o0 = (uintptr_t)W_q4, o1 = o0 + bytes;
  const uintptr_t ranges[3][2] = {{(uintptr_t)codes, (uintptr_t)codes + (size_t)V * d / 2},
                                  {(uintptr_t)scales, (uintptr_t)scales + (size_t)V * (d / 32) * 2},
                                  {(uintptr_t)mins, (uintptr_t)mins + (size_t)V * (d / 32) * 2}};
  for (const auto& r : ranges)
    if (r[0] < o1 && o0 < r[1]) return fail(DGD_EINVAL, "W_q4 overlaps an input");
  const int nk = packed_chunks(d);
  const int64_t units = (int64_t)packed_groups(V) * nk * 64;
  const int64_t blocks = (units + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_pack_vocab_q4, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     codes, scales, mins, (uint8_t*)W_q4, V, d, nk, units);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_pack_vocab_q4 launch");
}

int dgd_pack_vocab(const dgd_bf16* W_vocab, dgd_bf16* W_packed, int32_t V, int32_t d, void* stream) {
  g_err.clear();
  if (!W_vocab || !W_packed) return fail(DGD_EINVAL, "W_vocab/W_packed is NULL");
  if (V < 1 || V > DGD_MAX_VOCAB) return fail(DGD_EUNSUPPORTED, "V=%d outside [1, 2^24]", V);
  if (d < 8 || d > DGD_MAX_HIDDEN || d % 8 != 0)
    return fail(DGD_EUNSUPPORTED, "d=%d must be a multiple of 8 in [8, %d]", d, DGD_MAX_HIDDEN);
  if (!aligned16(W_vocab) || !aligned16(W_packed))
    return fail(DGD_EINVAL, "W_vocab/W_packed is not 16-byte aligned");
  const size_t bytes = dgd_packed_vocab_bytes(V, d);
  const uintptr_t s0 = (uintptr_t)W_vocab, s1 = s0 + (size_t)V * d * 2;
  const uintptr_t d0 = (uintptr_t)W_packed, d1 = d0 + bytes;
  if (s0 < d1 && d0 < s1) return fail(DGD_EINVAL, "W_vocab and W_packed overlap");
  const int64_t units = (int64_t)(bytes / 16);
  const int64_t blocks = (units + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_pack_vocab, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     W_vocab, W_packed, V, d, packed_chunks(d), units);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_pack_vocab launch");
}

int dgd_sc_embed(const float* sc_prob, const int32_t* sc_id, int32_t rows, int32_t K,
                 const dgd_bf16* W_vocab, int32_t vocab_layout, int32_t V, int32_t d, float scale,
                 dgd_bf16* out, void* stream) {
  g_err.clear();
  if (!sc_prob || !sc_id || !W_vocab || !out) return fail(DGD_EINVAL, "sc_prob/sc_id/W_vocab/out is NULL");
  if (rows < 0) return fail(DGD_EINVAL, "rows=%d < 0", rows);
  if (K < 1 || K > DGD_SC_MAX_TOPK) return fail(DGD_EINVAL, "K=%d outside [1, %d]", K, DGD_SC_MAX_TOPK);
  if (V < 1 || V > DGD_MAX_VOCAB) return fail(DGD_EUNSUPPORTED, "V=%d outside [1, 2^24]", V);
  if (d < 8 || d > DGD_MAX_HIDDEN || d % 8 != 0)
    return fail(DGD_EUNSUPPORTED, "d=%d must be a multiple of 8 in [8, %d]", d, DGD_MAX_HIDDEN);
  if (vocab_layout != DGD_VOCAB_ROWS && vocab_layout != DGD_VOCAB_PACKED)
    return fail(DGD_EINVAL, "vocab_layout=%d is neither DGD_VOCAB_ROWS nor DGD_VOCAB_PACKED", vocab_layout);
  if (!std::isfinite(scale)) return fail(DGD_EINVAL, "scale is not finite");
  if (!aligned16(W_vocab) || !aligned16(out)) return fail(DGD_EINVAL, "W_vocab/out is not 16-byte aligned");
  if (rows == 0) return DGD_OK;
  hipLaunchKernelGGL(k_sc_embed, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, sc_prob, sc_id, K,
                     W_vocab, vocab_layout == DGD_VOCAB_PACKED ? 1 : 0, V, d, scale, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_sc_embed launch");
}

int dgd_label_probs(const dgd_bf16* H, int32_t rows, const dgd_bf16* W_vocab, int32_t vocab_layout,
                    int32_t V, int32_t d, const int32_t* labels, int32_t n_labels, float temperature,
                    float softcap, float* logits, float* probs, void* stream) {
  g_err.clear();
  if (!H || !W_vocab || !labels || !probs) return fail(DGD_EINVAL, "H/W_vocab/labels/probs is NULL");
  if (rows < 0) return fail(DGD_EINVAL, "rows=%d < 0", rows);
  if (V < 1 || V > DGD_MAX_VOCAB) return fail(DGD_EUNSUPPORTED, "V=%d outside [1, 2^24]", V);
  if (d < 8 || d > DGD_MAX_HIDDEN || d % 8 != 0)
    return fail(DGD_EUNSUPPORTED, "d=%d must be a multiple of 8 in [8, %d]", d, DGD_MAX_HIDDEN);
  if (vocab_layout != DGD_VOCAB_ROWS && vocab_layout != DGD_VOCAB_PACKED)
    return fail(DGD_EINVAL, "vocab_layout=%d is neither DGD_VOCAB_ROWS nor DGD_VOCAB_PACKED", vocab_layout);
  if (n_labels < 1 || n_labels > DGD_MAX_LABELS)
    return fail(DGD_EINVAL, "n_labels=%d outside [1, %d]", n_labels, DGD_MAX_LABELS);
  for (int i = 0; i < n_labels; ++i)
    if (labels[i] < 0 || labels[i] >= V) return fail(DGD_EINVAL, "labels[%d]=%d outside [0, V)", i, labels[i]);
  if (!std::isfinite(temperature) || temperature < kMinTemperature)
    return fail(DGD_EINVAL, "temperature=%g must be finite and >= %g", temperature, kMinTemperature);
  if (!std::isfinite(softcap) || (softcap != 0.f && (softcap < 0.01f || softcap > 10000.f)))
    return fail(DGD_EINVAL, "softcap=%g must be 0 or in [0.01, 10000]", softcap);
  if (!aligned16(H) || !aligned16(W_vocab)) return fail(DGD_EINVAL, "H/W_vocab is not 16-byte aligned");
  if (rows == 0) return DGD_OK;
  LabelArgs la{};
  la.H = H; la.W = W_vocab; la.logits = logits; la.probs = probs;
  la.rows = rows; la.V = V; la.d = d; la.n = n_labels;
  la.packed = vocab_layout == DGD_VOCAB_PACKED ? 1 : 0;
  la.c2 = (float)(kLog2e / (double)temperature);
  la.cap = softcap;
  la.cap_in = softcap != 0.f ? (float)(2.0 * kLog2e / softcap) : 0.f;
  for (int i = 0; i < n_labels; ++i) la.labels[i] = labels[i];
  hipLaunchKernelGGL(k_label, dim3((unsigned)rows), dim3(kThreads), 0, (hipStream_t)stream, la);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_label launch");
}

int dgd_debug_philox(const uint32_t* ctr, const uint32_t* key, uint64_t uniform_key, uint32_t* out,
                     int64_t n, void* stream) {
  g_err.clear();
  if (!ctr || !out) return fail(DGD_EINVAL, "ctr/out is NULL");
  if (n < 0) return fail(DGD_EINVAL, "n < 0");
  if (((uintptr_t)ctr & 15) || ((uintptr_t)out & 15) || ((uintptr_t)key & 7))
    return fail(DGD_EINVAL, "ctr/out must be 16-byte and key 8-byte aligned");
  if (n == 0) return DGD_OK;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return fail(DGD_EUNSUPPORTED, "n too large");
  hipLaunchKernelGGL(k_debug_philox, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4_t*)ctr, (const u32x2_t*)key, (uint32_t)(uniform_key & 0xffffffffu),
                     (uint32_t)(uniform_key >> 32), (u32x4_t*)out, n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_debug_philox launch");
}

int dgd_ceiling_hbm_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  g_err.clear();
  if (!buf || !sink) return fail(DGD_EINVAL, "buf/sink is NULL");
  if (!aligned16(buf) || bytes % 16 != 0) return fail(DGD_EINVAL, "buf must be 16-byte aligned, bytes a multiple of 16");
  if (bytes == 0) return DGD_OK;
  hipLaunchKernelGGL(k_ceiling_hbm, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const u32x4_t*)buf,
                     (int64_t)(bytes / 16), sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_ceiling_hbm launch");
}

int dgd_ceiling_mfma_bf16(const void* ops, size_t bytes, int64_t rounds, int32_t workgroups, float* sink,
                          void* stream) {
  g_err.clear();
  if (!ops || !sink) return fail(DGD_EINVAL, "ops/sink is NULL");
  if (!aligned16(ops) || bytes < 256 || bytes % 16 != 0)
    return fail(DGD_EINVAL, "ops must be 16-byte aligned, bytes >= 256 and a multiple of 16");
  if (rounds < 1 || workgroups < 1 || workgroups > (1 << 20))
    return fail(DGD_EINVAL, "rounds >= 1 and workgroups in [1, 2^20] required");
  hipLaunchKernelGGL(k_ceiling_mfma, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4_t*)ops, (int64_t)(bytes / 16), rounds, sink);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_ceiling_mfma launch");
}

int dgd_debug_gumbel(const uint32_t* words, float* out, int64_t n, void* stream) {
  g_err.clear();
  if (!words || !out) return fail(DGD_EINVAL, "words/out is NULL");
  if (n < 0) return fail(DGD_EINVAL, "n < 0");
  if (n == 0) return DGD_OK;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return fail(DGD_EUNSUPPORTED, "n too large");
  hipLaunchKernelGGL(k_debug_gumbel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     words, out, n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? DGD_OK : hip_fail(e, "k_debug_gumbel launch");
}

}  // extern "C"
