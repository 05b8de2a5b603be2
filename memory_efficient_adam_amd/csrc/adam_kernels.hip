// Fused compressed-moment Adam/AdamW step for gfx950 (MI355X).
//
// One 256-thread workgroup (4 wave64s) owns one 2048-element block: it
// reads the block's params, grads, stored moments and old scales once,
// keeps the updated moments in registers, reduces the block statistic
// (DPP cross-lane steps + one cross-wave LDS step; for the percentile
// statistic, walks down the top values (of the lanes' top-4 lists, or of
// per-wave lists when v is the only 8-bit moment) or an LDS radix select;
// skipped for a moment whose static scale is already set), requantizes and
// writes params, moments and the new scales once.  With AMSGrad the running
// maximum of v travels the same way as v.  The step is a streaming map over
// HBM (14-20 bytes per parameter, ~1.5 flop/byte), so there is no MFMA work; what matters is
// coalesced 16-byte loads, enough bytes in flight per CU and a VALU budget
// of roughly 100 instructions per element at the bandwidth target.
//
// Method sources: "feat: add 8-bit Adam optimizer for memory efficiency"
// (AiDotNet PR #814) -- key-features list and walkthrough sequence diagram
// (dequantize -> bias-corrected Adam -> quantize, block-wise, signed m /
// unsigned v, dynamic scales, optional fp32 m, stochastic rounding,
// percentile scaling); "perf(training): make BF16-Adam fused-compatible"
// (AiDotNet PR #1745) -- bf16 moment buffers in one fused Adam/AdamW kernel,
// and AMSGrad named there as a variant still without one (built after
// Reddi, Kale & Kumar, "On the Convergence of Adam and Beyond", ICLR 2018).
// Philox4x32-10 follows Salmon et al., "Parallel Random Numbers: As Easy as
// 1, 2, 3" (SC'11).
//
// Thread -> element map: thread t handles elements 4t..4t+3 and
// 1024+4t..1024+4t+3 of its block, so every vector load of a wave covers one
// contiguous span (1 KiB of fp32 per wave per instruction).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "adam_internal.h"

namespace adam_mi355x {
namespace {

constexpr int kWaves = kThreads / 64;
constexpr int kGroups = kBlock / (kThreads * 4);  // 4-element groups per thread (2)
constexpr int kItems = kGroups * 4;               // elements per thread (8)
constexpr float kTiny = 0x1p-112f;                // smallest block statistic encoded

// ---------------------------------------------------------------- streaming access
// Every byte of params, grads and state is touched exactly once per step, so
// all data accesses are non-temporal (the "nt" cache policy): measured on
// MI355X this raises the mixed read/write stream rate by 5-10% over the
// default policy, and only when loads and stores both use it.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 ld_f32x4(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ u32x2 ld_u32x2(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ uint32_t ld_u32(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
template <class T>
__device__ __forceinline__ T ld_one(const T *p) {
    return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ void st_f32x4(float *p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void st_u32x2(void *p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}
__device__ __forceinline__ void st_u32(void *p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(p));
}
__device__ __forceinline__ void st_one(float *p, float v) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even, on the upper 16 bits; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    if (x != x) return 0x7FC0u;
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- Philox4x32-10
// kFreshKeys: the round keys are formed in the call, two scalar adds a round
// (an empty asm keeps the compiler from precomputing all twenty once per
// kernel into scalar registers).  The percentile variants take it: there
// the twenty registers were spilled to vector lanes (GPT-1.3B set with
// stochastic rounding, 100 steps: percentile 99.9 +1.6%, 99.0 +2.9%); the
// block-maximum ones keep them (-1.2% with fresh keys).
template <bool kFreshKeys>
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
    if constexpr (kFreshKeys) asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // one 32x32->64 multiply each (v_mad_u64_u32) instead of separate hi/lo
        const uint64_t prod0 = (uint64_t)0xD2511F53u * c[0];
        const uint64_t prod1 = (uint64_t)0xCD9E8D57u * c[2];
        // three-input XOR in one v_bitop3_b32 (truth table 0x96)
        c[0] = __builtin_amdgcn_bitop3_b32((uint32_t)(prod1 >> 32), c[1], k0, 0x96);
        c[1] = (uint32_t)prod1;
        c[2] = __builtin_amdgcn_bitop3_b32((uint32_t)(prod0 >> 32), c[3], k1, 0x96);
        c[3] = (uint32_t)prod0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// ---------------------------------------------------------------- reductions
// Cross-lane steps use DPP (data-parallel primitives: a VALU operand taken
// from another lane of the same row, or broadcast between rows), a few cycles
// each, instead of LDS-routed lane shuffles.  Lanes a DPP step does not
// write read 0, the identity of both the max of non-negative values and the
// sum below.
template <int kCtrl, int kRowMask = 0xF, int kBankMask = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, kBankMask, false);
}
constexpr int kQuadPerm1032 = 0xB1;  // lanes 1,0,3,2 of each quad
constexpr int kQuadPerm2301 = 0x4E;  // lanes 2,3,0,1 of each quad
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr3 = 0x113, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Max over the wave of unsigned values, as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = max(x, dpp<kQuadPerm1032>(x));
    x = max(x, dpp<kQuadPerm2301>(x));
    x = max(x, dpp<kRowRor4>(x));
    x = max(x, dpp<kRowRor8>(x));
    x = max(x, dpp<kRowBcast15, 0xA>(x));
    x = max(x, dpp<kRowBcast31, 0xC>(x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    uint32_t v = x + dpp<kRowShr1>(x);
    v += dpp<kRowShr2>(x);
    v += dpp<kRowShr3>(x);              // v = sum of lanes i-3..i of the row
    v += dpp<kRowShr4, 0xF, 0xE>(v);    // lanes 4..15: i-7..i
    v += dpp<kRowShr8, 0xF, 0xC>(v);    // lanes 8..15: whole row prefix
    v += dpp<kRowBcast15, 0xA>(v);      // rows 1, 3 add the previous row's total
    v += dpp<kRowBcast31, 0xC>(v);      // rows 2, 3 add the total of rows 0..1
    return v;
}

// threadIdx.x as a value computed here: LDS addresses derived from it are
// then formed where they are used instead of being hoisted out of the block
// loop and held in vector registers through the whole step.
__device__ __forceinline__ int local_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// A zero 16-byte vector made where it is stored (a constant one is hoisted
// out of the block loop, where its four registers get spilled).
__device__ __forceinline__ uint4 zero4() {
    uint32_t z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return uint4{z, z, z, z};
}

// Block-wide max of N non-negative values per thread (one barrier).  The
// values are never NaN (each is an fmaxf over |m|, v or the AMSGrad maximum
// from 0, which drops NaN), so the order of their bit patterns, with the sign
// bit cleared (-0 -> +0), is the float order: one DPP integer max per step
// (a float max would add a quieting max to each DPP move).
template <int N>
__device__ __forceinline__ void block_max(float (&x)[N], float (*red)[kWaves]) {
    const int t = local_tid(), lane = t & 63, wave = t >> 6;
    uint32_t u[N];
#pragma unroll
    for (int i = 0; i < N; ++i) u[i] = wave_max_u32(__float_as_uint(x[i]) & 0x7FFFFFFFu);
    static_assert(kWaves == 4, "four partial maxima");
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) red[i][wave] = __uint_as_float(u[i]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint4 q = *reinterpret_cast<const uint4 *>(red[i]);
        x[i] = __uint_as_float(max(max(q.x, q.y), max(q.z, q.w)));
    }
}

// Per-moment LDS scratch row of the select: [0, kWaves) the waves' partial
// maxima of the end pick, and the coarse pass's result as published by its
// scanning wave: [kWaves] the chosen bin, [kWaves + 1] the rank within it,
// [kWaves + 2] the bin's count; 8 words, so that each half is one 16-byte
// access.
constexpr int kSelRow = 8;
constexpr int kFineBins = 256;
static_assert(kWaves == 4, "a row's first half holds the four waves' partials");

// Histogram counting of one pass: moment k's keys with take(k, key) add 1 at
// byte offset digit(k, key) of hist[k] (LDS atomics; the caller's barrier
// completes them).  Keys are |x| as bit patterns (the order of non-negative
// floats).
template <int N, int kRow, class Digit, class Take>
__device__ __forceinline__ void hist_count(const float *const (&x)[N], const bool (&act)[N], Digit digit,
                                           Take take, uint32_t (*hist)[kRow]) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
        if (!act[k]) continue;
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const uint32_t key = __float_as_uint(x[k][i]) & 0x7FFFFFFFu;
            if (take(k, key))
                atomicAdd(reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(hist[k]) + digit(k, key)), 1u);
        }
    }
}

// One wave finds the bin of a 2048-bin histogram holding the rank-th
// smallest counted key: lane L sums bins [32 L, 32 L + 32), a wave prefix
// sum and a ballot find the lane whose range holds the rank, then lanes
// 0..31 take one bin each of that range and a second prefix sum and ballot
// find the bin.  Returns (bin, rank within it, its count), wave-uniform.  If
// no bin holds the rank (possible only when NaN keys upset the counts) the
// answer is some bin of the histogram.
__device__ __forceinline__ uint4 wave_pick_2048(const uint32_t *hist, uint32_t rank) {
    const int lane = local_tid() & 63;
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist + 32 * lane);
    uint32_t sum = 0u;
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
        // four 16-byte reads in flight at a time (all eight would hold 32
        // registers at once); lane L starts at its chunk L mod 8, so that the
        // lanes of one read (128 bytes apart) spread over the LDS banks
        const uint4 q0 = h4[(i + lane) & 7], q1 = h4[(i + 1 + lane) & 7], q2 = h4[(i + 2 + lane) & 7],
                    q3 = h4[(i + 3 + lane) & 7];
        sum += (q0.x + q0.y + q0.z + q0.w) + (q1.x + q1.y + q1.z + q1.w) + (q2.x + q2.y + q2.z + q2.w) +
               (q3.x + q3.y + q3.z + q3.w);
        asm volatile("" ::: "memory");
    }
    const uint32_t incl = wave_inclusive_sum(sum);
    const uint64_t hit = __ballot(incl - sum <= rank && rank < incl);
    const int L = hit ? __builtin_ctzll(hit) : 0;
    const uint32_t below = (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
    const uint32_t hb = lane < 32 ? hist[32 * L + lane] : 0u;
    const uint32_t incl2 = below + wave_inclusive_sum(hb);
    const uint64_t hit2 = __ballot(lane < 32 && incl2 - hb <= rank && rank < incl2);
    const int j = hit2 ? __builtin_ctzll(hit2) : 0;
    const uint32_t below2 = (uint32_t)__builtin_amdgcn_readlane((int)(incl2 - hb), j);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)hb, j);
    return uint4{(uint32_t)(32 * L + j), rank - below2, cnt, 0u};
}

// The same for a 256-bin histogram, by every wave for itself (no barrier
// after it): lane L holds bins [4 L, 4 L + 4); the four bins of the lane
// whose range holds the rank are settled in scalar registers.
__device__ __forceinline__ void wave_pick_256(const uint32_t *hist, uint32_t rank, uint32_t &bin, uint32_t &rank_in,
                                              uint32_t &count) {
    const int lane = local_tid() & 63;
    const uint4 q = reinterpret_cast<const uint4 *>(hist)[lane];
    const uint32_t sum = q.x + q.y + q.z + q.w;
    const uint32_t incl = wave_inclusive_sum(sum);
    const uint64_t hit = __ballot(incl - sum <= rank && rank < incl);
    const int L = hit ? __builtin_ctzll(hit) : 0;
    uint32_t r = rank - (uint32_t)__builtin_amdgcn_readlane((int)(incl - sum), L);
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)q.x, L);
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane((int)q.y, L);
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_readlane((int)q.z, L);
    const uint32_t b3 = (uint32_t)__builtin_amdgcn_readlane((int)q.w, L);
    uint32_t b = 4u * (uint32_t)L, c = b0;
    if (r >= b0) { r -= b0; ++b; c = b1;
        if (r >= b1) { r -= b1; ++b; c = b2;
            if (r >= b2) { r -= b2; ++b; c = b3; } } }
    bin = b;
    rank_in = r;
    count = c;
}

// The answer when it is the largest or the smallest key of its bin (the
// rank within the bin is count - 1, or 0), in one barrier.  A bin is a key
// range [lo, hi) (its prefix, then every lower bit), and the bins below it
// and above it hold the other keys, so
//   largest of the bin  = largest key below hi: the largest u = key - hi
//                         (unsigned, mod 2^32; keys below hi give u >= 2^31,
//                         the others u < 2^31);
//   smallest of the bin = smallest key at or above lo: the largest
//                         u = lo - 1 - key = ~key + lo (keys >= lo give
//                         u >= 2^31).
// Both are u = (key ^ s) + c (one v_xad_u32), and a block maximum of u with
// identity 0 finds it; key = (u - c) ^ s.
template <int N>
__device__ __forceinline__ void block_end_pick(const float *const (&x)[N], const bool (&end)[N],
                                               const uint32_t (&lo)[N], const uint32_t (&width)[N],
                                               const uint32_t (&rank)[N], const uint32_t (&count)[N],
                                               uint32_t (&out)[N], uint32_t (*scratch)[kSelRow]) {
    const int t = local_tid(), lane = t & 63, wave = t >> 6;
    uint32_t sx[N], c[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const bool largest = rank[k] + 1u == count[k];
        sx[k] = largest ? 0u : 0xFFFFFFFFu;
        c[k] = largest ? 0u - (lo[k] + width[k]) : lo[k];
        if (!end[k]) continue;
        uint32_t u[kItems];
#pragma unroll
        for (int i = 0; i < kItems; ++i) u[i] = ((__float_as_uint(x[k][i]) & 0x7FFFFFFFu) ^ sx[k]) + c[k];
        uint32_t best = max(max(max(u[0], u[1]), max(u[2], u[3])), max(max(u[4], u[5]), max(u[6], u[7])));
        best = wave_max_u32(best);
        if (lane == 0) scratch[k][wave] = best;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        if (!end[k]) continue;
        const uint4 part = *reinterpret_cast<const uint4 *>(&scratch[k][0]);
        const uint32_t m = max(max(part.x, part.y), max(part.z, part.w));
        out[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)((m - c[k]) ^ sx[k]));
    }
}

// rank-th smallest of one moment's 2048 keys by bisection on the key value:
// the answer is the largest v with at most `rank` keys below v, built bit by
// bit from the top (31 rounds, each a block-wide count: a compare per key, a
// DPP wave sum and one barrier, the rounds alternating between two LDS slot
// rows so that one barrier per round orders them).
__device__ __forceinline__ uint32_t block_bisect(const float *x, uint32_t rank, uint32_t (*slots)[kWaves]) {
    const int t = local_tid(), lane = t & 63, wave = t >> 6;
    uint32_t lo = 0u;
#pragma unroll 1
    for (int bit = 30; bit >= 0; --bit) {
        const uint32_t cand = lo | (1u << bit);
        uint32_t c = 0u;
#pragma unroll
        for (int i = 0; i < kItems; ++i) c += (__float_as_uint(x[i]) & 0x7FFFFFFFu) < cand ? 1u : 0u;
        c = wave_inclusive_sum(c);
        if (lane == 63) slots[bit & 1][wave] = c;
        __syncthreads();
        uint32_t total = 0u;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) total += slots[bit & 1][w];
        if (total <= rank) lo = cand;
    }
    return lo;
}

// Before the block maximum's barrier: the select's histograms start at zero
// (that barrier orders these stores before the select's counting).
template <int N>
__device__ __forceinline__ void select_clear(const bool (&act)[N], uint32_t (*hist)[kBlock],
                                             uint32_t (*fine)[kFineBins]) {
    const int tid = local_tid();
    static_assert(kBlock == 2 * 4 * kThreads && kFineBins == 4 * 64, "clear in 16-byte stores");
#pragma unroll
    for (int k = 0; k < N; ++k) {
        if (!act[k]) continue;
        uint4 *h4 = reinterpret_cast<uint4 *>(hist[k]);
        h4[tid] = zero4();
        h4[tid + kThreads] = zero4();
        if (N <= 2 && tid < 64) reinterpret_cast<uint4 *>(fine[k])[tid] = zero4();
    }
}

// rank-th smallest (0-based) of the block's 2048 keys (8 per thread) of each
// of N moments, by LDS radix select (select_clear ran before the block
// maximum's barrier).  top[k] is moment k's largest key (the block maximum),
// E its exponent field.
//   coarse pass: the digit is the key's binade below E (0..14) and its top 7
//           mantissa bits: bin = (key >> 16) - ((E - 15) << 7), i.e. 128 +
//           128 (14 - d) + mantissa for a key d binades below E, clamped to
//           [127, 2047], so that every key 15 or more binades below E lands
//           in bin 127 (three instructions per key: extract, one shift-add
//           to the byte offset, clamp).  Moments cluster in a
//           few binades under the block maximum, so 128 bins per binade keep
//           few keys per bin and few lanes of a wave's atomic add meet on one
//           LDS word (a digit of the top 11 key bits puts ~80 keys of the
//           densest binade in one of its 8 bins).  A bin >= 128 fixes the
//           key's bits 30..16.  After the counting barrier wave k alone scans
//           moment k's histogram (wave_pick_2048) and publishes the bin; a
//           second barrier hands it to every wave;
//   fine passes: bits 15..8, then 7..0, of the keys in that bin, 256 bins,
//           each wave scanning the small histogram for itself (one barrier
//           per pass).
// After the coarse pass and after the first fine pass, a moment whose answer
// is the largest or the smallest key of its bin (rank count - 1 or 0: a bin
// holding one or two keys, or the end of a longer one) skips the rest and
// takes it by block_end_pick; the moments still undecided run the next pass
// (the first fine pass in its own pre-cleared histogram, or with three
// moments in the coarse histogram's words 0..255; the rare second in its
// words 256..511; both of the latter cleared behind a barrier).  When
// the answer lies in bin 127 (15 binades or more below the maximum: zeros and
// tiny values, e.g. a low percentile of a block with exact zeros), that
// moment's statistic comes from block_bisect over all its keys instead.
template <int N>
__device__ void block_select_n(const float *const (&x)[N], const bool (&act)[N], const uint32_t (&top)[N],
                               uint32_t rank0, uint32_t (&out)[N], uint32_t (*hist)[kBlock],
                               uint32_t (*fine)[kFineBins], uint32_t (*scratch)[kSelRow]) {
    static_assert(N <= kWaves, "one scanning wave per moment");
    const int wave = local_tid() >> 6;
    // stage of each moment (block-uniform): 0 done or inactive, 1 bisection,
    // 2 end pick, 3 next counting pass
    int32_t base[N], nbase4[N];
    uint32_t rank[N], bin[N], count[N], pfx[N], mask[N], stage[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
        base[k] = ((int32_t)(top[k] >> 23) - 15) * 128;
        nbase4[k] = -4 * base[k];
        out[k] = 0u;
    }
    hist_count<N, kBlock>(
        x, act,
        [&](int k, uint32_t key) {
            // 4 (key >> 16) - 4 base in one shift-add (left to itself the
            // compiler subtracts first and shifts after), clamped in bytes
            int32_t off;
            asm("v_lshl_add_u32 %0, %1, 2, %2" : "=v"(off) : "v"(__builtin_amdgcn_ubfe(key, 16, 15)), "s"(nbase4[k]));
            return (uint32_t)min(max(off, 4 * 127), 4 * (kBlock - 1));
        },
        [](int, uint32_t) { return true; }, hist);
    __syncthreads();
    bool scans = false;  // wave-uniform: this wave scans moment `wave`
#pragma unroll
    for (int k = 0; k < N; ++k) scans = scans || (wave == k && act[k]);
    if (scans) {
        const uint4 res = wave_pick_2048(hist[wave], rank0);
        if ((local_tid() & 63) == 0) *reinterpret_cast<uint4 *>(&scratch[wave][kWaves]) = res;
    }
    __syncthreads();
    bool more[N], any = false;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        // block-uniform: scalar registers (as vector values they crowd the
        // kernel's vector registers into spills)
        const uint4 res = *reinterpret_cast<const uint4 *>(&scratch[k][kWaves]);
        bin[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)res.x);
        rank[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)res.y);
        count[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)res.z);
        pfx[k] = (uint32_t)((int32_t)bin[k] + base[k]) << 16;  // bits 30..16 of the bin's keys
        mask[k] = 0x7FFF0000u;
        stage[k] = !act[k] ? 0u : bin[k] == 127u ? 1u : (rank[k] == 0u || rank[k] + 1u == count[k]) ? 2u : 3u;
        more[k] = stage[k] == 3u;
        any = any || more[k];
    }
    if (any) {  // block-uniform
        // N = 3: in the coarse histogram's first 256 words, free after the
        // publishing barrier, cleared behind one more barrier
        uint32_t *fh[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
            if constexpr (N <= 2) fh[k] = fine[k];
            else fh[k] = hist[k];
        }
        if constexpr (N > 2) {
#pragma unroll
            for (int k = 0; k < N; ++k)
                if (more[k] && local_tid() < kFineBins / 4)
                    reinterpret_cast<uint4 *>(hist[k])[local_tid()] = zero4();
            __syncthreads();
        }
        const auto fine_digit = [](int, uint32_t key) { return (key >> 6) & (255u << 2); };
        const auto fine_take = [&](int k, uint32_t key) { return (key & mask[k]) == pfx[k]; };
        if constexpr (N <= 2)
            hist_count<N, kFineBins>(x, more, fine_digit, fine_take, fine);
        else
            hist_count<N, kBlock>(x, more, fine_digit, fine_take, hist);
        __syncthreads();
        any = false;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            if (more[k]) {
                wave_pick_256(fh[k], rank[k], bin[k], rank[k], count[k]);
                pfx[k] |= bin[k] << 8;  // bits 30..8
                mask[k] = 0x7FFFFF00u;
                stage[k] = (rank[k] == 0u || rank[k] + 1u == count[k]) ? 2u : 3u;
            }
            more[k] = stage[k] == 3u;
            any = any || more[k];
        }
        if (any) {  // block-uniform
            // words 256..511 of the coarse histogram: no wave reads them after
            // the publishing barrier (the first fine pass of three moments
            // uses words 0..255, which slower waves may still be scanning)
#pragma unroll
            for (int k = 0; k < N; ++k)
                if (more[k] && local_tid() < kFineBins / 4)
                    reinterpret_cast<uint4 *>(hist[k] + kFineBins)[local_tid()] = zero4();
            __syncthreads();
            hist_count<N, kBlock>(
                x, more, [](int, uint32_t key) { return (key << 2) & (255u << 2); },
                [&](int k, uint32_t key) { return (key & mask[k]) == pfx[k]; },
                reinterpret_cast<uint32_t (*)[kBlock]>(hist[0] + kFineBins));
            __syncthreads();
#pragma unroll
            for (int k = 0; k < N; ++k) {
                if (more[k]) {
                    wave_pick_256(hist[k] + kFineBins, rank[k], bin[k], rank[k], count[k]);
                    out[k] = pfx[k] | bin[k];
                }
            }
        }
    }
    // the end pick's partial maxima use words of the scratch rows that no
    // pass reads
    bool end[N];
    any = false;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        end[k] = stage[k] == 2u;
        any = any || end[k];
    }
    if (any) {
        uint32_t width[N];
#pragma unroll
        for (int k = 0; k < N; ++k) width[k] = (~mask[k] & 0x7FFFFFFFu) + 1u;  // keys of one bin
        block_end_pick<N>(x, end, pfx, width, rank, count, out, scratch);
    }
    // a moment left for the bisection has its own coarse histogram, which no
    // wave reads after the publishing barrier
#pragma unroll
    for (int k = 0; k < N; ++k)
        if (stage[k] == 1u) out[k] = block_bisect(x[k], rank0, reinterpret_cast<uint32_t (*)[kWaves]>(hist[k]));
}

// The same statistic when it lies near the top: the rank-th smallest of the
// 2048 keys is the need-th largest, need = 2048 - rank, counted with
// multiplicity.  A high percentile (99.9 of a full block: need 4) makes
// need small, and then walks down the distinct values replace the radix
// passes (the launch picks one path or the other for the whole step, see
// walk_covers).  With two or three moments (8-bit m and v, or AMSGrad) each
// lane writes its top-4 keys of each moment to LDS and, after one barrier,
// wave k walks moment k's 1024 keys alone (lane_top4 / top_select below):
// one walk per moment instead of one per wave and moment plus a merge (one
// box, interleaved 100-step runs: ViT-Base 8-bit at 99.9 +4.3%, GPT-1.3B SR
// +5.4%, with AMSGrad +6.2%).  With v alone (fp32 m) the four waves walk
// their own keys; the lane lists gained nothing there (-1.4%, within the
// run-to-run spread of that set):
//   wave_top:  each wave takes its own keys' largest value, counts it,
//              drops it, and repeats until at least `need` keys are counted;
//              the (value, count) list goes to LDS.  No barrier.
//   top_merge: after one barrier, the same walk over the union of the four
//              lists (64 entries, one per lane), stopping at `need`; wave k
//              merges moment k and publishes it through LDS (one more
//              barrier), so the merges cost one wave each.
// The union walk is exact: each wave's list holds every key of that wave
// down to its last value L_w, with counts, and the answer s has at least
// `need` keys at or above it in the block, so s >= max_w L_w; at and above
// that point the union counts every key, and s is in its own wave's list
// (fewer than `need` keys of the block lie above it).
// A key is the value's bit pattern shifted up one place with the low bit set
// (one v_lshl_or: the sign drops out, the order of magnitudes stays, no key
// is 0), so 0 marks "dropped" / "empty" and the unsigned max with its
// identity 0 serves both walks.
constexpr uint32_t kTopCap = 16;  // entries of a wave's list (the union: one per lane)
static_assert(kWaves * kTopCap == 64, "one union entry per lane");


__device__ __forceinline__ uint32_t top_key(float x) { return (__float_as_uint(x) << 1) | 1u; }

// top values of |x| over the wave's 512 keys; writes kTopCap (value+1,
// count) entries at val[wave * kTopCap ...], unused entries (0, 0).
// need in [1, kTopCap], wave-uniform.
__device__ __forceinline__ void wave_top(const float (&x)[kItems], uint32_t need, uint32_t *val,
                                         uint32_t *cnt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t key[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) key[i] = top_key(x[i]);
    uint32_t my_val = 0u, my_cnt = 0u, acc = 0u;
    // each round counts at least one key (the wave holds 512 > kTopCap), so
    // kTopCap rounds always reach need
    for (uint32_t it = 0; it < kTopCap; ++it) {
        uint32_t lm = key[0];
#pragma unroll
        for (int i = 1; i < kItems; ++i) lm = max(lm, key[i]);
        const uint32_t M = wave_max_u32(lm);
        uint32_t C = 0u;
#pragma unroll
        for (int i = 0; i < kItems; ++i) {
            const bool hit = key[i] == M;
            C += (uint32_t)__popcll(__ballot(hit));
            key[i] = hit ? 0u : key[i];
        }
        // lane `it` of the list: one v_writelane each (it, M and C are uniform;
        // the lane select goes through M0, the one scalar source besides the
        // value that the instruction may read on this architecture)
        asm("v_writelane_b32 %0, %1, m0" : "+v"(my_val) : "s"(M), "{m0}"(it));
        asm("v_writelane_b32 %0, %1, m0" : "+v"(my_cnt) : "s"(C), "{m0}"(it));
        acc += C;
        if (acc >= need) break;
    }
    if (lane < (int)kTopCap) {
        val[wave * kTopCap + lane] = my_val;
        cnt[wave * kTopCap + lane] = my_cnt;
    }
}

// The same walk with less work per round: each lane first keeps only its two
// largest keys, sorted (k0 >= k1), and a round looks at the lanes' heads k0
// only: M = the largest head, counted over the heads equal to it, and those
// lanes shift their lists up by one.  While every lane still holds a known
// key, M is the wave's largest remaining key; a value repeated within a lane
// comes back as M in the next round, so it may appear in the list more than
// once (the merge sums such entries).  A lane whose list runs empty may hide
// more keys at or above the next value: if need is not reached by then, the
// wave returns false and takes the full walk (a wave falls back when one
// lane holds two of its three largest keys: ~4% of waves for distinct keys).
// The round that reaches need may miss such hidden copies of M in its count;
// the merge stays exact, since that count is still at least need, and only
// the counts above the last value enter its sums below the answer.
// The walks serve need <= 4 (percentiles of 99.85 and above for a full
// block, the pages' default 99.9 among them); from need 5 on, the radix
// select is faster (8-bit ViT-Base set, percentile 99.5 (need 12): 317
// against 288 Gparams/s for per-wave walks over per-lane top-4 lists, 342
// against 322 for one selecting wave per moment over the union of the lane
// lists, whose serial rounds grow with need: 338 against 285 at 99.0).
constexpr uint32_t kWalkNeed = 4;

__device__ __forceinline__ bool wave_top_lanes(const float (&x)[kItems], uint32_t need, uint32_t *val,
                                               uint32_t *cnt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t k0 = top_key(x[0]), k1 = top_key(x[1]);
    {
        const uint32_t hi = max(k0, k1);
        k1 = min(k0, k1);
        k0 = hi;
    }
#pragma unroll
    for (int i = 2; i < kItems; ++i) {
        const uint32_t y = top_key(x[i]);
        // with k0 >= k1 the second largest of (k0, k1, y) is their median:
        // one v_med3 in place of a min and a max
        asm("v_med3_u32 %0, %1, %2, %3" : "=v"(k1) : "v"(k0), "v"(k1), "v"(y));
        k0 = max(k0, y);
    }
    uint32_t my_val = 0u, my_cnt = 0u, acc = 0u;
    // each round counts at least one key, so kWalkNeed rounds always reach need
    for (uint32_t it = 0; it < kWalkNeed; ++it) {
        const uint32_t M = wave_max_u32(k0);
        const bool hit = k0 == M;
        const uint32_t C = (uint32_t)__popcll(__ballot(hit));
        // lane `it` of the list: one v_writelane each (it, M and C are uniform;
        // the lane select goes through M0, the one scalar source besides the
        // value that the instruction may read on this architecture)
        asm("v_writelane_b32 %0, %1, m0" : "+v"(my_val) : "s"(M), "{m0}"(it));
        asm("v_writelane_b32 %0, %1, m0" : "+v"(my_cnt) : "s"(C), "{m0}"(it));
        acc += C;
        if (acc >= need) break;
        k0 = hit ? k1 : k0;
        k1 = hit ? 0u : k1;
        if (__ballot(k0 == 0u) != 0) return false;  // a lane without a known key
    }
    if (lane < (int)kTopCap) {
        val[wave * kTopCap + lane] = my_val;
        cnt[wave * kTopCap + lane] = my_cnt;
    }
    return true;
}

__device__ __forceinline__ void wave_top_any(const float (&x)[kItems], uint32_t need, uint32_t *val,
                                             uint32_t *cnt) {
    if (!wave_top_lanes(x, need, val, cnt)) wave_top(x, need, val, cnt);
}

// Lane top-4: the four largest keys of the lane's 8 (with multiplicity),
// sorted.  The union of every lane's top-4 holds the block's need-th largest
// key s for need <= 4 and counts it right: a lane's keys above s are fewer
// than need, so all of them are in its top-4, and a lane contributes either
// all its keys at s or four keys at or above s.
__device__ __forceinline__ uint4 lane_top4(const float (&x)[kItems]) {
    uint32_t k0 = top_key(x[0]), k1 = top_key(x[1]), k2 = 0u, k3 = 0u;
    {
        const uint32_t hi = max(k0, k1);
        k1 = min(k0, k1);
        k0 = hi;
    }
#pragma unroll
    for (int i = 2; i < kItems; ++i) {
        const uint32_t y = top_key(x[i]);
        asm("v_med3_u32 %0, %1, %2, %3" : "=v"(k3) : "v"(k2), "v"(k3), "v"(y));
        asm("v_med3_u32 %0, %1, %2, %3" : "=v"(k2) : "v"(k1), "v"(k2), "v"(y));
        asm("v_med3_u32 %0, %1, %2, %3" : "=v"(k1) : "v"(k0), "v"(k1), "v"(y));
        k0 = max(k0, y);
    }
    return uint4{k0, k1, k2, k3};
}

// need-th largest key (and the largest) over the 256 lanes' top-4 lists,
// by one wave: lane L takes the lists of threads L, L + 64, L + 128, L + 192
// (16 keys), keeps its two largest, and walks down the lanes' heads as
// wave_top_lanes does; if a lane's list runs empty first, the walk over all
// 16 keys per lane.  Returned as magnitude bit patterns {need-th, maximum}.
__device__ __forceinline__ uint2 top_select(const uint32_t *cand, uint32_t need) {
    const int lane = threadIdx.x & 63;
    uint32_t key[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 q = reinterpret_cast<const uint4 *>(cand)[lane + 64 * j];
        key[4 * j] = q.x; key[4 * j + 1] = q.y; key[4 * j + 2] = q.z; key[4 * j + 3] = q.w;
    }
    uint32_t k0 = max(key[0], key[4]), k1 = min(key[0], key[4]);
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        if (i == 4) continue;
        asm("v_med3_u32 %0, %1, %2, %3" : "=v"(k1) : "v"(k0), "v"(k1), "v"(key[i]));
        k0 = max(k0, key[i]);
    }
    const uint32_t top = wave_max_u32(k0);
    uint32_t M = top, acc = 0u;
    bool ok = true;
    for (uint32_t it = 0; it < kWalkNeed; ++it) {
        const bool hit = k0 == M;
        acc += (uint32_t)__popcll(__ballot(hit));
        if (acc >= need) break;
        k0 = hit ? k1 : k0;
        k1 = hit ? 0u : k1;
        if (__ballot(k0 == 0u) != 0) { ok = false; break; }
        M = wave_max_u32(k0);
    }
    if (!ok) {  // a lane held three or more of the top keys: walk all 16 per lane
        M = top;
        acc = 0u;
        for (uint32_t it = 0; it < kWalkNeed; ++it) {
            uint32_t c = 0u;  // this lane's keys at M, summed over the wave below
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const bool hit = key[i] == M;
                c += hit ? 1u : 0u;
                key[i] = hit ? 0u : key[i];
            }
            acc += (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(c), 63);
            if (acc >= need) break;
            uint32_t lm = key[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) lm = max(lm, key[i]);
            M = wave_max_u32(lm);
        }
    }
    return make_uint2(M >> 1, top >> 1);
}

// need-th largest key over the union of the wave lists (after a barrier
// that follows every wave_top), computed by one wave, with the largest key
// of the union, which is the block maximum (each list starts at its wave's
// largest key).  Returned as magnitude bit patterns {need-th, maximum}.
// Each round consumes at least one entry of count >= 1, and the entries hold
// at least need counts in total, so the walk stops within 64 rounds.
__device__ __forceinline__ uint2 top_merge(const uint32_t *val, const uint32_t *cnt, uint32_t need) {
    const int lane = threadIdx.x & 63;
    uint32_t v = val[lane];
    const uint32_t n = cnt[lane];
    const uint32_t top = wave_max_u32(v);  // every list starts at its wave's largest key
    uint32_t acc = 0u, M = top;
    if (__ballot(n > 1u) == 0) {  // every entry one key (distinct values): a ballot counts a round
        for (int it = 0; it < 64; ++it) {
            const bool hit = v == M;
            acc += (uint32_t)__popcll(__ballot(hit));
            if (acc >= need) break;
            v = hit ? 0u : v;
            M = wave_max_u32(v);
        }
    } else {
        for (int it = 0; it < 64; ++it) {
            const uint32_t s = wave_inclusive_sum(v == M ? n : 0u);
            acc += (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
            if (acc >= need) break;
            v = v == M ? 0u : v;
            M = wave_max_u32(v);
        }
    }
    return make_uint2(M >> 1, top >> 1);
}

// ---------------------------------------------------------------- quantizer
// Code magnitude for |x| = a with statistic A and r = fl(qmax/A) (A >= kTiny).
// For a < A, a <= A(1 - 2^-24) and r <= (qmax/A)(1 + 2^-24), so y = fl(a*r) <=
// qmax: neither rounding can pass qmax (at y = qmax the fraction is 0), and
// only a >= A -- possible with the percentile statistic or a kept scale, or
// at the block maximum, where y may fall just below qmax -- needs the end
// pin.  kEnd selects how it is applied:
//   kPinEnd:   k = qmax wherever a >= A (a compare and a select);
//   kClampEnd: y clamped to qmax before rounding (one min) -- the same codes
//              when qmax = 127: at a >= A, y >= fl(A*r) >= 127 - 2^-17 (A*r
//              is within 127 * 2^-24 < 2^-17 of 127, the spacing below 127
//              being 2^-17), and both roundings take any y in
//              [127 - 2^-17, 127] to 127 (for stochastic rounding ceil(y *
//              2^16) = 127 * 2^16 there).  Not for qmax = 255: the spacing
//              below 255 is 2^-16, and y = 255 - 2^-16 rounds stochastically
//              to 254 for the draw 65535.
//   kNoEnd:    nothing (only a = A reaches y near qmax, and nearest-even
//              rounding takes it to qmax).
// Stochastic rounding: floor(y) + [u16 * 2^-16 < frac(y)] is computed as
// (ceil(y * 2^16) + 65535 - u16) >> 16.  With Y = y * 2^16 (exact, Y < 2^24)
// = 2^16 floor(y) + F, u16 < F holds iff u16 < ceil(F), iff the low 16 bits of
// ceil(Y) + 65535 - u16 carry into bit 16.  Callers pass nu16 = 65535 - u16,
// taken from the complement of the draw word: one NOT serves both halves.
enum EndRule { kNoEnd, kPinEnd, kClampEnd };

// floor(x) converted to int32 in one instruction (the compiler emits a floor
// and a separate convert for (int)floorf(x)); exact for |x| < 2^31, checked
// against floorf on the hardware over 2^25 values in [-2^24, 2^24].
__device__ __forceinline__ int32_t cvt_floor(float x) {
    int32_t r;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

template <bool kSR, EndRule kEnd>
__device__ __forceinline__ uint32_t code_magnitude(float a, float A, float r, uint32_t qmax, uint32_t nu16) {
    float y = a * r;
    if constexpr (kEnd == kClampEnd) y = fminf(y, (float)qmax);
    uint32_t k;
    if constexpr (kSR) {
        // ceil(Y) = -floor(-Y): one convert and one subtract
        k = (nu16 - (uint32_t)cvt_floor(y * -65536.0f)) >> 16;
    } else {
        k = (uint32_t)rintf(y);
    }
    if constexpr (kEnd == kPinEnd) k = a >= A ? qmax : k;
    return k;
}

// ---------------------------------------------------------------- one block
// Scalars of one block: where its data lives and its stored scales.
struct BlockCtx {
    uint64_t gidx;   // flat state index of the block's first element
    uint64_t didx;   // stochastic-rounding draw index of the block's first element
    float *p;        // the block's params
    const void *g;   // the block's grads
    uint32_t n;      // live elements (1..2048)
    uint32_t npad;   // n rounded up to 16 (state entries owned by the block)
    uint32_t slot;   // scale slot
};

// The descriptor, pointer and draw-index tables do not change during a launch: reading
// them through the constant address space lets them be scalar loads even
// after the kernel's own stores (a generic load there would be a vector load
// whose wait also drains every prefetched data load).
typedef const __attribute__((address_space(4))) BlockDesc *ConstDescPtr;
typedef const __attribute__((address_space(4))) TensorRef *ConstTensorPtr;
typedef const __attribute__((address_space(4))) uint64_t *ConstU64Ptr;

template <bool kGradBf16>
__device__ __forceinline__ BlockCtx load_ctx(const StepArgs &a, uint32_t idx) {
    const ConstDescPtr d = (ConstDescPtr)a.desc + idx;
    const uint32_t lb_n = d->lb_n;
    const ConstTensorPtr tr = (ConstTensorPtr)a.tensors + d->tensor;
    const size_t local = (size_t)(lb_n >> kBlockBits) * kBlock;
    BlockCtx c;
    c.gidx = (uint64_t)d->gidx16 * 16u;
    c.didx = ((ConstU64Ptr)a.draw_first)[d->tensor] + local;
    c.p = tr->p + local;
    c.g = kGradBf16 ? (const void *)(reinterpret_cast<const uint16_t *>(tr->g) + local)
                    : (const void *)(reinterpret_cast<const float *>(tr->g) + local);
    c.n = (lb_n & (kBlock - 1)) + 1u;
    c.npad = (c.n + 15u) & ~15u;
    c.slot = d->slot;
    return c;
}

// Raw (undecoded) per-thread data of one block, as loaded.  w: the AMSGrad
// running maximum of v, stored as v is (unused without kAms).
template <int kStore, bool kGradBf16, bool kAms>
struct BlockRegs {
    float p[kItems];
    uint32_t g[kGradBf16 ? kItems / 2 : kItems];  // fp32 bits, or bf16 pairs
    uint32_t m[kStore == kStoreBf16 ? kItems / 2 : (kStore == kStoreQ8 ? kGroups : kItems)];
    uint32_t v[kStore == kStoreBf16 ? kItems / 2 : kGroups];
    uint32_t w[!kAms ? 1 : (kStore == kStoreBf16 ? kItems / 2 : kGroups)];
    float Am, Av, Aw;  // stored scales of the 8-bit moments
};

// Issues every load of one block.  kFull: the block has 2048 live elements,
// so all loads are unconditional 16/8/4-byte vector loads (no branches: the
// compiler's wait counts then let the loads stay in flight across the
// previous block's compute).  Otherwise the ragged last group uses element
// loads and state slots past the tensor's padded segment are not touched.
template <int kStore, bool kGradBf16, bool kAms, bool kFull>
__device__ __forceinline__ void load_data(const StepArgs &a, const BlockCtx &c,
                                          BlockRegs<kStore, kGradBf16, kAms> &r) {
    const int tid = kFull ? (int)threadIdx.x : local_tid();  // the ragged path: see local_tid
    r.Am = kStore == kStoreQ8 ? a.m_scale[c.slot] : 0.0f;
    r.Av = kStore != kStoreBf16 ? a.v_scale[c.slot] : 0.0f;
    r.Aw = kAms && kStore != kStoreBf16 ? a.w_scale[c.slot] : 0.0f;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
        if (kFull || e0 + 4 <= c.n) {
            const f32x4 x = ld_f32x4(c.p + e0);
            r.p[4 * j + 0] = x.x; r.p[4 * j + 1] = x.y; r.p[4 * j + 2] = x.z; r.p[4 * j + 3] = x.w;
            if constexpr (kGradBf16) {
                const u32x2 h = ld_u32x2(reinterpret_cast<const uint16_t *>(c.g) + e0);
                r.g[2 * j] = h.x;
                r.g[2 * j + 1] = h.y;
            } else {
                const f32x4 y = ld_f32x4(reinterpret_cast<const float *>(c.g) + e0);
                r.g[4 * j + 0] = __float_as_uint(y.x); r.g[4 * j + 1] = __float_as_uint(y.y);
                r.g[4 * j + 2] = __float_as_uint(y.z); r.g[4 * j + 3] = __float_as_uint(y.w);
            }
        } else {
            // ragged last group: element loads, zeros past the tensor's end
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool in = e0 + k < c.n;
                r.p[4 * j + k] = in ? ld_one(c.p + e0 + k) : 0.0f;
                if constexpr (kGradBf16) {
                    const uint32_t h = in ? ld_one(reinterpret_cast<const uint16_t *>(c.g) + e0 + k) : 0u;
                    if (k & 1) r.g[2 * j + k / 2] |= h << 16;
                    else r.g[2 * j + k / 2] = h;
                } else {
                    r.g[4 * j + k] = in ? __float_as_uint(ld_one(reinterpret_cast<const float *>(c.g) + e0 + k)) : 0u;
                }
            }
        }
        // state: entries past the tensor's end (its 16-element padding) take
        // no part in the step, whatever a written or loaded state holds
        // there: in a ragged block they are masked to zero as they arrive
        // (integer masks, element k of the group kept iff k < live), so
        // they decode as zero and are stored back as zero
        const size_t s = c.gidx + e0;
        const bool in = kFull || e0 < c.npad;
        int32_t live = 4;
        uint32_t keep8 = ~0u, keep16lo = ~0u, keep16hi = ~0u;
        if constexpr (!kFull) {
            live = min(max((int32_t)c.n - (int32_t)e0, 0), 4);
            keep8 = (uint32_t)(0xFFFFFFFFull >> (32 - 8 * live));
            keep16lo = (uint32_t)(0xFFFFFFFFull >> (32 - 16 * min(live, 2)));
            keep16hi = (uint32_t)(0xFFFFFFFFull >> (32 - 16 * max(live - 2, 0)));
        }
        if constexpr (kStore == kStoreBf16) {
            u32x2 hm = {0u, 0u}, hv = {0u, 0u};
            if (in) {
                hm = ld_u32x2(reinterpret_cast<const uint16_t *>(a.m_state) + s);
                hv = ld_u32x2(reinterpret_cast<const uint16_t *>(a.v_state) + s);
            }
            r.m[2 * j] = hm.x & keep16lo; r.m[2 * j + 1] = hm.y & keep16hi;
            r.v[2 * j] = hv.x & keep16lo; r.v[2 * j + 1] = hv.y & keep16hi;
            if constexpr (kAms) {
                u32x2 hw = {0u, 0u};
                if (in) hw = ld_u32x2(reinterpret_cast<const uint16_t *>(a.w_state) + s);
                r.w[2 * j] = hw.x & keep16lo; r.w[2 * j + 1] = hw.y & keep16hi;
            }
        } else {
            r.v[j] = in ? ld_u32(reinterpret_cast<const uint8_t *>(a.v_state) + s) & keep8 : 0u;
            if constexpr (kAms) r.w[j] = in ? ld_u32(reinterpret_cast<const uint8_t *>(a.w_state) + s) & keep8 : 0u;
            if constexpr (kStore == kStoreQ8) {
                r.m[j] = in ? ld_u32(reinterpret_cast<const int8_t *>(a.m_state) + s) & keep8 : 0u;
            } else {
                f32x4 mf = {0.f, 0.f, 0.f, 0.f};
                if (in) mf = ld_f32x4(reinterpret_cast<const float *>(a.m_state) + s);
                r.m[4 * j + 0] = __float_as_uint(mf.x); r.m[4 * j + 1] = __float_as_uint(mf.y);
                r.m[4 * j + 2] = __float_as_uint(mf.z); r.m[4 * j + 3] = __float_as_uint(mf.w);
                if constexpr (!kFull) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) r.m[4 * j + k] &= (uint32_t)((int32_t)(k - live) >> 31);
                }
            }
        }
    }
}

// LDS of one block's max reduction (m, v and the AMSGrad maximum).
struct BlockLds {
    alignas(16) float red[3][kWaves];  // rows read as one 16-byte word
};

// Block statistic of a step: the block maximum, or the percentile taken by
// the top walks or by the radix select.
enum PctMode { kPctNone = 0, kPctTop = 1, kPctRadix = 2 };

// LDS of the percentile statistic (kN: moments with a statistic, 2 or 3).
template <int kPct, int kN>
struct SelectLds {};
template <int kN>
struct SelectLds<kPctTop, kN> {
    union {
        alignas(16) uint32_t cand[kN][4 * kThreads];  // lanes' top-4 keys (two or three moments)
        struct {
            uint32_t val[3][kWaves * kTopCap];
            uint32_t cnt[3][kWaves * kTopCap];
        } w;  // wave lists of the walks (v alone)
    };
    uint32_t res[3];  // statistic of each moment
    uint32_t top[3];  // and its block maximum
};
template <int kN>
struct SelectLds<kPctRadix, kN> {  // histograms + scratch row per moment
    alignas(16) uint32_t h[kN][kBlock];      // coarse pass (16-byte aligned rows: cleared in 16-byte stores)
    // first fine pass; with three moments it shares the coarse histograms
    // instead (27 KiB of LDS per workgroup would leave room for 5 per CU, 24
    // KiB leaves room for the 6 their registers allow)
    alignas(16) uint32_t f[kN <= 2 ? kN : 1][kFineBins];
    alignas(16) uint32_t s[kN][kSelRow];
};

// ---------------------------------------------------------------- exact sqrt / divide
// Correctly rounded square root and quotient for operands in a normal range,
// without the range handling of the general sequences (which scale tiny or
// huge operands and patch zeros, infinities and NaNs).  Where they apply
// they perform the same operations as the general correctly rounded
// sequences, so the results are the same bits.
//
// sqrt_rn: x in [2^-96, 2^128).  The hardware square root is within one ulp
// of sqrt(x), so the rounded root is it or a neighbour; the sign of the
// exact residual x - s' * s (one fma) tells which: x <= s_- * s means sqrt(x)
// lies below the midpoint of s_- and s, x > s_+ * s that it lies above the
// midpoint of s and s_+ (x, s_- * s and s * s_+ sit on a grid too coarse for
// x to fall strictly between a product and its midpoint square).
__device__ __forceinline__ float sqrt_rn(float x) {
    const float s = __builtin_amdgcn_sqrtf(x);
    const float sm = __uint_as_float(__float_as_uint(s) - 1u);
    const float sp = __uint_as_float(__float_as_uint(s) + 1u);
    float r = fmaf(-sm, s, x) <= 0.0f ? sm : s;
    return fmaf(-sp, s, x) > 0.0f ? sp : r;
}

// div_rn: d in [2^-40, 2^77], |n| in [2^-40, 2^40] (quotient and reciprocal
// normal, no intermediate over- or underflow): the hardware reciprocal, one
// Newton step, and two quotient corrections whose remainders n - d*q are
// exact (fma).
__device__ __forceinline__ float div_rn(float n, float d) {
    float r = __builtin_amdgcn_rcpf(d);
    r = fmaf(fmaf(-d, r, 1.0f), r, r);
    float q = n * r;
    q = fmaf(fmaf(-d, q, n), r, q);
    return fmaf(fmaf(-d, q, n), r, q);
}

// Codes of four unsigned values x[b..b+3] (v, or the AMSGrad maximum) packed
// into the bytes of one word; nu: the complements of the group's four Philox
// words, of which the 16 bits at `shift` are the complemented draws.
template <bool kSR>
__device__ __forceinline__ uint32_t pack_u8(const float (&x)[kItems], int b, float pin, float r,
                                            const uint32_t (&nu)[4], int shift) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float ax = fabsf(x[b + k]);
        if constexpr (kSR) {
            c |= code_magnitude<true, kPinEnd>(ax, pin, r, 255u, (nu[k] >> shift) & 0xFFFFu) << (8 * k);
        } else {
            // nearest-even rounding, clamped to [0, 255], packed into byte k: the
            // clamp is the end pin (|x| >= A gives y >= 254.99998)
            c = __builtin_amdgcn_cvt_pk_u8_f32(ax * r, k, c);
        }
    }
    return c;
}

__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Decode, update, store params; block statistic; requantize and store state.
// kStatic: a moment whose stored scale is already set (>= kTiny) keeps it and
// skips its statistic; values at or beyond it saturate through the end rule.
// kAms: AMSGrad -- the running maximum w of v is decoded, updated to
// max(w, v), used in the denominator and stored as v is, with its own scale.
template <int kStore, bool kGradBf16, bool kSR, int kPct, bool kStatic, bool kAms, bool kFull>
__device__ __forceinline__ void process_block(const StepArgs &a, const BlockCtx &c,
                                              const BlockRegs<kStore, kGradBf16, kAms> &r,
                                              BlockLds &lds, SelectLds<kPct, kAms ? 3 : 2> &sel) {
    constexpr bool kQuantM = (kStore == kStoreQ8);
    const int tid = threadIdx.x;
    float p[kItems], g[kItems], mo[kItems], vo[kItems], wo[kItems];  // wo: AMSGrad only

    // ---- decode
    constexpr float Rm = 1.0f / 127.0f;
    constexpr float Rv = 1.0f / 255.0f;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        p[i] = r.p[i];
        if constexpr (kGradBf16) g[i] = bf16_to_f32((r.g[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
        else g[i] = __uint_as_float(r.g[i]);
        if constexpr (kStore == kStoreBf16) {
            mo[i] = bf16_to_f32((r.m[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
            vo[i] = bf16_to_f32((r.v[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
            if constexpr (kAms) wo[i] = bf16_to_f32((r.w[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
        } else {
            vo[i] = ((float)((r.v[i / 4] >> (8 * (i & 3))) & 0xFFu) * Rv) * r.Av;
            if constexpr (kAms) wo[i] = ((float)((r.w[i / 4] >> (8 * (i & 3))) & 0xFFu) * Rv) * r.Aw;
            if constexpr (kQuantM) {
                const int32_t q = ((int32_t)(r.m[i / 4] << (24 - 8 * (i & 3)))) >> 24;
                mo[i] = ((float)q * Rm) * r.Am;
            } else {
                mo[i] = __uint_as_float(r.m[i]);
            }
        }
    }

    // ---- the Adam/AdamW element update (moments stay in registers)
    if (a.l2) {  // Adam with L2-coupled weight decay (uniform branch)
#pragma unroll
        for (int i = 0; i < kItems; ++i) g[i] = fmaf(a.wd, p[i], g[i]);
    }
    float mmax = 0.0f, vmax = 0.0f, wmax = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        // moments of the 4-element group
        float m_lo = __builtin_inff(), m_hi = 0.0f, v_lo = __builtin_inff();  // min, max |m|; min v
#pragma unroll
        for (int i = 4 * j; i < 4 * j + 4; ++i) {
            const float gi = g[i];
            const float m = fmaf(a.beta1, mo[i], a.omb1 * gi);
            const float v = fmaf(a.beta2, vo[i], a.omb2 * (gi * gi));
            if constexpr (kAms) {
                wo[i] = fmaxf(wo[i], v);  // the second moment the denominator uses
                wmax = fmaxf(wmax, wo[i]);
            }
            mo[i] = m;
            vo[i] = v;
            vmax = fmaxf(vmax, v);
            m_hi = fmaxf(m_hi, fabsf(m));
            m_lo = fminf(m_lo, fabsf(m));
            v_lo = fminf(v_lo, kAms ? wo[i] : v);
        }
        mmax = fmaxf(mmax, m_hi);
        // p = p*decay - step * m / (sqrt(v) * ibc2 + eps).  When every lane's
        // group lies in the normal range (v at least 2^-96 for sqrt_rn; |m|
        // in [2^-40, 2^40] for div_rn, whose divisor sqrt(v) * ibc2 + eps is
        // in [2^-40, 2^77] given ibc2 <= 2^12 and eps in [2^-40, 2^20]) the
        // wave takes the short sequences, otherwise the general ones.  Same
        // bits either way; one decision per group lets a group's update start
        // while the next group's loads are still in flight.
        const float(&vden)[kItems] = kAms ? wo : vo;
        const bool in_range = a.fast_ok && v_lo >= 0x1p-96f && m_lo >= 0x1p-40f && m_hi <= 0x1p40f;
        if (__all(in_range)) {
#pragma unroll
            for (int i = 4 * j; i < 4 * j + 4; ++i) {
                const float den = fmaf(sqrt_rn(vden[i]), a.ibc2, a.eps);
                p[i] = fmaf(-a.step, div_rn(mo[i], den), p[i] * a.decay);
            }
        } else {
#pragma unroll
            for (int i = 4 * j; i < 4 * j + 4; ++i) {
                const float den = fmaf(sqrtf(vden[i]), a.ibc2, a.eps);
                p[i] = fmaf(-a.step, mo[i] / den, p[i] * a.decay);
            }
        }
    }

    // ---- store params
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
        if (kFull || e0 + 4 <= c.n) {
            st_f32x4(c.p + e0, f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]});
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (e0 + k < c.n) st_one(c.p + e0 + k, p[4 * j + k]);
        }
    }

    if constexpr (kStore == kStoreBf16) {
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
            if (kFull || e0 < c.npad) {
                const size_t s = c.gidx + e0;
                const u32x2 hm = {f32_to_bf16(mo[4 * j]) | (f32_to_bf16(mo[4 * j + 1]) << 16),
                                  f32_to_bf16(mo[4 * j + 2]) | (f32_to_bf16(mo[4 * j + 3]) << 16)};
                const u32x2 hv = {f32_to_bf16(vo[4 * j]) | (f32_to_bf16(vo[4 * j + 1]) << 16),
                                  f32_to_bf16(vo[4 * j + 2]) | (f32_to_bf16(vo[4 * j + 3]) << 16)};
                st_u32x2(reinterpret_cast<uint16_t *>(a.m_state) + s, hm);
                st_u32x2(reinterpret_cast<uint16_t *>(a.v_state) + s, hv);
                if constexpr (kAms) {
                    const u32x2 hw = {f32_to_bf16(wo[4 * j]) | (f32_to_bf16(wo[4 * j + 1]) << 16),
                                      f32_to_bf16(wo[4 * j + 2]) | (f32_to_bf16(wo[4 * j + 3]) << 16)};
                    st_u32x2(reinterpret_cast<uint16_t *>(a.w_state) + s, hw);
                }
            }
        }
    } else {
        // ---- block statistic (the old scales are block-uniform: every lane
        // read the same word, so readfirstlane makes the branches scalar)
        bool keep_m = false, keep_v = false, keep_w = false;
        float Am_old = 0.0f, Av_old = 0.0f, Aw_old = 0.0f;
        if constexpr (kStatic) {
            Av_old = uniform(r.Av);
            keep_v = Av_old >= kTiny;
            if constexpr (kQuantM) {
                Am_old = uniform(r.Am);
                keep_m = Am_old >= kTiny;
            }
            if constexpr (kAms) {
                Aw_old = uniform(r.Aw);
                keep_w = Aw_old >= kTiny;
            }
        }
        const bool need_m = kQuantM && !keep_m, need_v = !keep_v, need_w = kAms && !keep_w;
        // percentile: rank-th smallest of the block's 2048 keys (the padding
        // adds zeros below the n values), i.e. the need-th largest
        uint32_t rank = 0, need = 0;
        if constexpr (kPct != kPctNone) {
            // (full blocks: the same double arithmetic, done once on the host)
            if constexpr (kFull) rank = a.rank_full;
            else rank = (uint32_t)floor(a.pfrac * (double)(c.n - 1)) + (kBlock - c.n);
            need = kBlock - rank;  // in [1, kWalkNeed] for kPctTop (walk_covers)
        }
        constexpr bool kLaneLists = kQuantM || kAms;  // two or three moments walked
        if constexpr (kPct == kPctTop) {  // lists of the walks; the barrier below publishes them
            if constexpr (kLaneLists) {
                uint4 *c4[3];
#pragma unroll
                for (int k = 0; k < (kAms ? 3 : 2); ++k) c4[k] = reinterpret_cast<uint4 *>(sel.cand[k]);
                if (need_m) c4[0][tid] = lane_top4(mo);
                if (need_v) c4[1][tid] = lane_top4(vo);
                if constexpr (kAms)
                    if (need_w) c4[2][tid] = lane_top4(wo);
            } else {
                if (need_v) wave_top_any(vo, need, sel.w.val[1], sel.w.cnt[1]);
            }
        }
        if constexpr (kPct == kPctTop) {
            // the walks' lists hold each wave's largest key: the merge finds
            // the block maximum too, and this barrier only publishes them
            if (need_m || need_v || need_w) __syncthreads();
        } else if (need_m || need_v || need_w) {
            if constexpr (kPct == kPctRadix) {
                if constexpr (kAms) {
                    const bool act[3] = {need_m, need_v, need_w};
                    select_clear<3>(act, sel.h, sel.f);
                } else {
                    const bool act[2] = {need_m, need_v};
                    select_clear<2>(act, sel.h, sel.f);
                }
            }
            if constexpr (kAms) {
                float x[3] = {mmax, vmax, wmax};
                block_max<3>(x, lds.red);
                mmax = x[0]; vmax = x[1]; wmax = x[2];
            } else {
                float x[2] = {mmax, vmax};
                block_max<2>(x, lds.red);
                mmax = x[0]; vmax = x[1];
            }
        }
        float Amn = keep_m ? Am_old : mmax, Avn = keep_v ? Av_old : vmax, Awn = keep_w ? Aw_old : wmax;
        if constexpr (kPct == kPctTop) {
            // wave k walks or merges moment k's lists and publishes the statistic
            const int wave = threadIdx.x >> 6;
            const bool need_k[3] = {need_m, need_v, need_w};
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (wave == k && need_k[k]) {
                    uint2 st;
                    if constexpr (kLaneLists) st = top_select(sel.cand[k], need);
                    else st = top_merge(sel.w.val[k], sel.w.cnt[k], need);
                    if ((threadIdx.x & 63) == 0) {
                        sel.res[k] = st.x;
                        sel.top[k] = st.y;
                    }
                }
            }
            __syncthreads();
            mmax = __uint_as_float(sel.top[0]);
            vmax = __uint_as_float(sel.top[1]);
            wmax = __uint_as_float(sel.top[2]);
        }
        if constexpr (kPct != kPctNone) {
            float st[3] = {0.0f, 0.0f, 0.0f};
            if constexpr (kPct == kPctTop) {
                st[0] = __uint_as_float(sel.res[0]);
                st[1] = __uint_as_float(sel.res[1]);
                st[2] = __uint_as_float(sel.res[2]);
            } else {
                if constexpr (kAms) {
                    const float *const xs[3] = {mo, vo, wo};
                    const bool act[3] = {need_m, need_v, need_w};
                    const uint32_t top[3] = {__float_as_uint(mmax), __float_as_uint(vmax), __float_as_uint(wmax)};
                    uint32_t res[3];
                    block_select_n<3>(xs, act, top, rank, res, sel.h, sel.f, sel.s);
                    st[0] = __uint_as_float(res[0]);
                    st[1] = __uint_as_float(res[1]);
                    st[2] = __uint_as_float(res[2]);
                } else {
                    const float *const xs[2] = {mo, vo};
                    const bool act[2] = {need_m, need_v};
                    const uint32_t top[2] = {__float_as_uint(mmax), __float_as_uint(vmax)};
                    uint32_t res[2];
                    block_select_n<2>(xs, act, top, rank, res, sel.h, sel.f, sel.s);
                    st[0] = __uint_as_float(res[0]);
                    st[1] = __uint_as_float(res[1]);
                }
            }
            if (need_m) Amn = st[0] < kTiny ? mmax : st[0];
            if (need_v) Avn = st[1] < kTiny ? vmax : st[1];
            if constexpr (kAms)
                if (need_w) Awn = st[2] < kTiny ? wmax : st[2];
        }
        constexpr bool kPin = kSR || kPct != kPctNone || kStatic;
        const bool mzero = !(Amn >= kTiny), vzero = !(Avn >= kTiny), wzero = !(Awn >= kTiny);
        const float rm = mzero ? 0.0f : 127.0f / Amn;
        const float rv = vzero ? 0.0f : 255.0f / Avn;
        const float rw = (!kAms || wzero) ? 0.0f : 255.0f / Awn;
        // a zero block has r = 0, so y = 0 and every code is 0; its pin
        // threshold is +inf so that the end pin never fires
        const float pin_v = vzero ? __builtin_inff() : Avn;
        const float pin_w = wzero ? __builtin_inff() : Awn;

        // ---- the AMSGrad maximum's draws (stochastic rounding): one Philox
        // call per 8 elements, on the counter stream with bit 63 set; element
        // i takes half i mod 2 of word (i / 2) mod 4 at counter i / 8.  The
        // lanes of a pair (2m, 2m + 1) hold the two halves of one 8-element
        // group of each of their 4-element groups: the even lane computes
        // the call of their first group, the odd lane that of their second,
        // and one DPP swap hands each lane the two words it lacks.  Every
        // lane takes part (the swap reads its partner): an 8-element group
        // lies wholly inside or wholly past a tensor's 16-padded segment.
        static_assert(kGroups == 2, "a lane pair's two 4-element groups");
        uint32_t wdraw[kGroups][2] = {};
        if constexpr (kSR && kAms) {
            const bool odd = (tid & 1) != 0;
            const uint64_t g8 = (c.didx >> 3) + (odd ? (uint64_t)(kThreads * 4 / 8) : 0u) + (uint64_t)(tid >> 1);
            uint32_t ctr[4] = {(uint32_t)g8, (uint32_t)(g8 >> 32) | 0x80000000u, a.t_lo, a.t_hi};
            philox4x32_10<kPct != kPctNone>(ctr, a.seed_lo, a.seed_hi);
            // the even lane lacks words 0, 1 of the second group's call, the
            // odd lane words 2, 3 of the first group's
            const uint32_t got0 = dpp<kQuadPerm1032>(odd ? ctr[0] : ctr[2]);
            const uint32_t got1 = dpp<kQuadPerm1032>(odd ? ctr[1] : ctr[3]);
            wdraw[0][0] = odd ? got0 : ctr[0];
            wdraw[0][1] = odd ? got1 : ctr[1];
            wdraw[1][0] = odd ? ctr[2] : got0;
            wdraw[1][1] = odd ? ctr[3] : got1;
        }

        // ---- requantize and store codes
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
            if (!kFull && e0 >= c.npad) continue;
            const size_t s = c.gidx + e0;
            uint32_t rnd[4] = {0u, 0u, 0u, 0u}, rnd_w[4] = {0u, 0u, 0u, 0u};
            if constexpr (kSR) {
                const uint64_t grp = (c.didx + e0) >> 2;  // draw index / 4
                uint32_t ctr[4] = {(uint32_t)grp, (uint32_t)(grp >> 32), a.t_lo, a.t_hi};
                philox4x32_10<kPct != kPctNone>(ctr, a.seed_lo, a.seed_hi);
                // complemented draws (65535 - u16 in each half); the empty asm
                // keeps each complement in a register, where both halves'
                // subtractions read it (left visible, the compiler re-derives
                // the low half's complement from the word: one more op)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    rnd[k] = ~ctr[k];
                    asm("" : "+v"(rnd[k]));
                }
                if constexpr (kAms) {
                    rnd_w[0] = ~wdraw[j][0];
                    rnd_w[1] = ~wdraw[j][0] >> 16;
                    rnd_w[2] = ~wdraw[j][1];
                    rnd_w[3] = ~wdraw[j][1] >> 16;
                }
            }
            st_u32(reinterpret_cast<uint8_t *>(a.v_state) + s, pack_u8<kSR>(vo, 4 * j, pin_v, rv, rnd, 16));
            if constexpr (kAms)
                st_u32(reinterpret_cast<uint8_t *>(a.w_state) + s, pack_u8<kSR>(wo, 4 * j, pin_w, rw, rnd_w, 0));
            if constexpr (kQuantM) {
                uint32_t cm = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float x = mo[4 * j + k];
                    const uint32_t q = code_magnitude<kSR, kPin ? kClampEnd : kNoEnd>(fabsf(x), Amn, rm, 127u,
                                                                                      rnd[k] & 0xFFFFu);
                    const uint32_t qs = x < 0.0f ? 0u - q : q;  // -0 gives 0
                    cm |= (qs & 0xFFu) << (8 * k);
                }
                st_u32(reinterpret_cast<int8_t *>(a.m_state) + s, cm);
            } else {
                st_f32x4(reinterpret_cast<float *>(a.m_state) + s,
                         f32x4{mo[4 * j], mo[4 * j + 1], mo[4 * j + 2], mo[4 * j + 3]});
            }
        }
        // a kept scale is not rewritten: with no statistic there is no
        // barrier between the waves' reads of it and this store
        if (tid == 0) {
            if (need_m) a.m_scale[c.slot] = mzero ? 0.0f : Amn;
            if (need_v) a.v_scale[c.slot] = vzero ? 0.0f : Avn;
            if (need_w) a.w_scale[c.slot] = wzero ? 0.0f : Awn;
        }
    }
}

// ---------------------------------------------------------------- kernel
// Waves per SIMD the radix-select variants are compiled for.  Left to
// itself the compiler spends registers freely there (the select's passes and
// its bisection fallback) and lands at 4-7 waves per SIMD; asking for one
// or two more gets them by moving a few scalar registers into vector lanes,
// with no memory spills (checked per variant; the stochastic-rounding
// AMSGrad variants would spill and keep the compiler's choice).  8-bit
// ViT-Base set at percentile 99.0: 317 Gparams/s at 8 waves against 309 at
// 7.  The static-scale 8-bit variants carry the kept scales besides and take
// one wave fewer (at 8 they spill a register to memory).
constexpr int select_waves(int store, bool sr, int pct, bool ams, bool stat) {
    if (pct != 2 || (sr && ams)) return 1;
    if (store == kStoreQ8) return (!sr && !ams ? 8 : (sr ? 7 : 6)) - (stat ? 1 : 0);
    return !sr && !ams ? 7 : 6;
}

// One workgroup per block; workgroups beyond the grid limit loop (stride =
// grid size).  Descriptors [0, n_full) are full blocks, whose path has no
// tail checks; the rest are the tensors' ragged last blocks.
template <int kStore, bool kGradBf16, bool kSR, int kPct, bool kStatic, bool kAms>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(select_waves(kStore, kSR, kPct, kAms, kStatic))))
adam_step_kernel(StepArgs a) {
    __shared__ BlockLds lds;
    __shared__ SelectLds<kPct, kAms ? 3 : 2> sel;
    for (uint32_t i0 = blockIdx.x; i0 < a.n_all; i0 += gridDim.x) {
        // XCD-aware order: workgroup i0 runs on XCD i0 mod 8, and here each
        // XCD takes runs of 16 consecutive blocks, the runs dealt round-robin
        // (a bijection on the first n - n mod 128 blocks; the rest keep their
        // order).  Measured +2% for the 8-bit nearest-rounding step and ~+1%
        // for the percentile one; with stochastic rounding +2.9% on the
        // ViT-Base 8-bit set (fp32 grads), +1.1% on the fp32-m + 8-bit-v
        // shard set, level on the GPT-1.3B set.  Stochastic rounding with
        // AMSGrad keeps plain order (GPT-1.3B shaped set: -3.1% with it).
        uint32_t i = i0;
        if (!(kSR && kAms) && gridDim.x == a.n_all && i0 < a.n_all - a.n_all % 128u) {
            const uint32_t x = i0 & 7u, k = i0 >> 3;
            i = ((k >> 4) << 7) + (x << 4) + (k & 15u);
        }
        BlockRegs<kStore, kGradBf16, kAms> r;
        const BlockCtx c = load_ctx<kGradBf16>(a, i);
        if (i < a.n_full) {
            load_data<kStore, kGradBf16, kAms, true>(a, c, r);
            process_block<kStore, kGradBf16, kSR, kPct, kStatic, kAms, true>(a, c, r, lds, sel);
        } else {
            load_data<kStore, kGradBf16, kAms, false>(a, c, r);
            process_block<kStore, kGradBf16, kSR, kPct, kStatic, kAms, false>(a, c, r, lds, sel);
        }
        if (i0 + gridDim.x < a.n_all) __syncthreads();  // LDS reused by the next block
    }
}

// Occupancy cap.  Too many outstanding requests thrash the HBM pages, so the
// variants with little compute per block stream fastest with few workgroups
// resident per CU; their launch reserves LDS it does not use (CU LDS is 160
// KiB).  Measured per variant: bf16 moments (no block statistic) at most 3;
// 8-bit with the block maximum and nearest rounding at most 4 (GPT-1.3B
// shaped set with bf16 gradients +7% over uncapped, ViT-Base with fp32
// gradients unchanged); fp32 m + 8-bit v with the percentile walk and
// nearest rounding (one walk per block) at most 4 (Llama-7B shaped set
// +2.6%).  Stochastic rounding with the block maximum and bf16 gradients
// (no AMSGrad) at most 5 (GPT-1.3B shaped set, three boxes: +0.4%, +0.8%,
// +2.4%; 4 per CU -6%; with fp32 gradients 5 per CU cost 1.7%, with AMSGrad
// 1.1%; the fp32-m storage takes the same cap, not measured there).  The other stochastic-rounding variants, the radix select and the
// walks over two or three moments spend longer per block and need every
// resident workgroup to keep enough bytes in flight (a cap of 4 cost them
// 5-9%), so they are not capped.
constexpr int kCuLdsBytes = 160 * 1024;
#ifndef ADAM_BF16_RESIDENT_PER_CU
#define ADAM_BF16_RESIDENT_PER_CU 3
#endif
#ifndef ADAM_Q8_NEAREST_RESIDENT_PER_CU
#define ADAM_Q8_NEAREST_RESIDENT_PER_CU 4
#endif
#ifndef ADAM_Q8_RESIDENT_PER_CU
#define ADAM_Q8_RESIDENT_PER_CU 8
#endif
#ifndef ADAM_Q8_SR_BF16G_RESIDENT_PER_CU
#define ADAM_Q8_SR_BF16G_RESIDENT_PER_CU 5
#endif
constexpr size_t reserve_lds(int resident) { return resident >= 8 ? 0 : kCuLdsBytes / (resident + 1) + 1024; }
constexpr uint32_t kMaxGrid = (1u << 24) - 1;  // grid.x * 256 work-items < 2^32

template <int kStore, bool kGradBf16, bool kSR, int kPct, bool kStatic, bool kAms>
hipError_t launch_one(const StepArgs &a, hipStream_t stream) {
    const uint32_t grid = std::min<uint32_t>(a.n_all, kMaxGrid);
    if (grid == 0) return hipSuccess;
    constexpr bool kLight = !kSR && (kPct == kPctNone || (kPct == kPctTop && kStore == kStoreQ8VOnly && !kAms));
    constexpr bool kSrBf16g = kSR && kGradBf16 && !kAms && kPct == kPctNone;
    constexpr int kResident = kStore == kStoreBf16 ? ADAM_BF16_RESIDENT_PER_CU
                              : kLight             ? ADAM_Q8_NEAREST_RESIDENT_PER_CU
                              : kSrBf16g           ? ADAM_Q8_SR_BF16G_RESIDENT_PER_CU
                                                   : ADAM_Q8_RESIDENT_PER_CU;
    constexpr size_t kStaticLds = sizeof(BlockLds) + sizeof(SelectLds<kPct, kAms ? 3 : 2>);
    constexpr size_t kDyn = reserve_lds(kResident) > kStaticLds ? reserve_lds(kResident) - kStaticLds : 0;
    hipLaunchKernelGGL((adam_step_kernel<kStore, kGradBf16, kSR, kPct, kStatic, kAms>), dim3(grid), dim3(kThreads),
                       kDyn, stream, a);
    return hipGetLastError();
}

// The walks serve a step when every block's need is at most kWalkNeed.  need =
// n - floor(p (n - 1)) for a block of n values never falls as n grows (n + 1
// raises the floor by 0 or 1), so the full block's need decides; the double
// arithmetic is the kernel's own, so both sides agree on it.
bool walk_covers(double pfrac) {
    return (uint32_t)kBlock - (uint32_t)floor(pfrac * (double)(kBlock - 1)) <= kWalkNeed;
}

template <int kStore, bool kGradBf16, bool kSR, bool kStatic, bool kAms>
hipError_t launch_stat(const Variant &v, const StepArgs &a, hipStream_t stream) {
    if (!v.percentile) return launch_one<kStore, kGradBf16, kSR, kPctNone, kStatic, kAms>(a, stream);
    return walk_covers(a.pfrac) ? launch_one<kStore, kGradBf16, kSR, kPctTop, kStatic, kAms>(a, stream)
                                : launch_one<kStore, kGradBf16, kSR, kPctRadix, kStatic, kAms>(a, stream);
}

template <int kStore, bool kGradBf16, bool kStatic, bool kAms>
hipError_t launch_rounding(const Variant &v, const StepArgs &a, hipStream_t stream) {
    return v.stochastic ? launch_stat<kStore, kGradBf16, true, kStatic, kAms>(v, a, stream)
                        : launch_stat<kStore, kGradBf16, false, kStatic, kAms>(v, a, stream);
}

template <int kStore, bool kGradBf16, bool kAms>
hipError_t launch_q(const Variant &v, const StepArgs &a, hipStream_t stream) {
    return v.static_scales ? launch_rounding<kStore, kGradBf16, true, kAms>(v, a, stream)
                           : launch_rounding<kStore, kGradBf16, false, kAms>(v, a, stream);
}

template <bool kAms>
hipError_t launch_storage(const Variant &v, const StepArgs &a, hipStream_t stream) {
    switch (v.storage) {
    case kStoreBf16:
        return v.grad_bf16 ? launch_one<kStoreBf16, true, false, kPctNone, false, kAms>(a, stream)
                           : launch_one<kStoreBf16, false, false, kPctNone, false, kAms>(a, stream);
    case kStoreQ8:
        return v.grad_bf16 ? launch_q<kStoreQ8, true, kAms>(v, a, stream)
                           : launch_q<kStoreQ8, false, kAms>(v, a, stream);
    case kStoreQ8VOnly:
        return v.grad_bf16 ? launch_q<kStoreQ8VOnly, true, kAms>(v, a, stream)
                           : launch_q<kStoreQ8VOnly, false, kAms>(v, a, stream);
    default:
        return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- allocation-free step tables
// The tables of the allocation-free entry point: block descriptors, then
// per-tensor pointer pairs, then per-tensor draw indices.  One copy per GPU,
// held until the process ends (17.5 MiB); every call on a GPU rewrites the
// parts it uses before its step kernel reads them.
constexpr size_t kScratchDescBytes = (size_t)kScratchMaxBlocks * sizeof(BlockDesc);
constexpr size_t kScratchTensorBytes = (size_t)kScratchMaxTensors * sizeof(TensorRef);
constexpr size_t kScratchBytes = kScratchDescBytes + kScratchTensorBytes + (size_t)kScratchMaxTensors * 8;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// One workgroup row per tensor of the chunk (blockIdx.x), the tensor's blocks
// spread over blockIdx.y and the threads.  Ordinary vector stores.
__global__ void __launch_bounds__(kThreads) fill_tables_kernel(FillArgs f) {
    const FillTensor &t = f.t[blockIdx.x];
    const uint32_t nblk = (t.n + kBlock - 1) / kBlock, full = t.n / kBlock;
    for (uint32_t b = blockIdx.y * kThreads + threadIdx.x; b < nblk; b += gridDim.y * kThreads) {
        const uint32_t len = b < full ? (uint32_t)kBlock : t.n - full * kBlock;
        f.desc[b < full ? t.first_full + b : t.tail] =
            BlockDesc{t.gidx16 + b * (kBlock / 16), t.index, (b << kBlockBits) | (len - 1u), t.first_slot + b};
    }
    if (blockIdx.y == 0 && threadIdx.x == 0) {
        f.tensors[t.index] = TensorRef{t.p, t.g};
        f.draw[t.index] = t.draw;
    }
}

}  // namespace

hipError_t launch_step(const Variant &v, const StepArgs &a, hipStream_t stream) {
    return v.amsgrad ? launch_storage<true>(v, a, stream) : launch_storage<false>(v, a, stream);
}

hipError_t scratch_tables(int device, BlockDesc **desc, TensorRef **tensors, uint64_t **draw) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *base[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!base[device]) {
        // the array's name is a host-side stand-in: its device address on the
        // current device comes from the runtime, once per device
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        base[device] = p;
    }
    unsigned char *b = static_cast<unsigned char *>(base[device]);
    *desc = reinterpret_cast<BlockDesc *>(b);
    *tensors = reinterpret_cast<TensorRef *>(b + kScratchDescBytes);
    *draw = reinterpret_cast<uint64_t *>(b + kScratchDescBytes + kScratchTensorBytes);
    return hipSuccess;
}

hipError_t launch_fill(const FillArgs &f, hipStream_t stream) {
    if (f.count == 0 || f.count > (uint32_t)kFillChunk) return hipErrorInvalidValue;
    uint32_t most = 1;
    for (uint32_t k = 0; k < f.count; ++k) most = std::max(most, (f.t[k].n + kBlock - 1) / kBlock);
    const uint32_t rows = std::min<uint32_t>((most + kThreads - 1) / kThreads, 256u);
    hipLaunchKernelGGL(fill_tables_kernel, dim3(f.count, rows), dim3(kThreads), 0, stream, f);
    return hipGetLastError();
}

}  // namespace adam_mi355x
