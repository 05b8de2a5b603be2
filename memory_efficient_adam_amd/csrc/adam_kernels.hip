// Fused compressed-moment Adam/AdamW step for gfx950 (MI355X).
//
// One 256-thread workgroup (4 wave64s) owns one 2048-element block: it
// reads the block's params, grads, stored moments and old scales once,
// keeps the updated moments in registers, reduces the block statistic
// (wave shuffles + a cross-wave LDS step; an LDS radix select for the
// percentile statistic), requantizes and writes params, moments and the new
// scales once.  The step is a streaming map over HBM (14-20 bytes per
// parameter, ~1.5 flop/byte), so there is no MFMA work; what matters is
// coalesced 16-byte loads, enough bytes in flight per CU and a VALU budget
// of roughly 100 instructions per element at the bandwidth target.
//
// Method sources: "feat: add 8-bit Adam optimizer for memory efficiency"
// (AiDotNet PR #814) -- key-features list and walkthrough sequence diagram
// (dequantize -> bias-corrected Adam -> quantize, block-wise, signed m /
// unsigned v, dynamic scales, optional fp32 m, stochastic rounding,
// percentile scaling); "perf(training): make BF16-Adam fused-compatible"
// (AiDotNet PR #1745) -- bf16 moment buffers in one fused Adam/AdamW kernel.
// Philox4x32-10 follows Salmon et al., "Parallel Random Numbers: As Easy as
// 1, 2, 3" (SC'11).
//
// Thread -> element map: thread t handles elements 4t..4t+3 and
// 1024+4t..1024+4t+3 of its block, so every vector load of a wave covers one
// contiguous span (1 KiB of fp32 per wave per instruction).
#include <hip/hip_runtime.h>
#include <stdint.h>

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
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c[0];
        const uint32_t hi0 = __umulhi(0xD2511F53u, c[0]);
        const uint32_t lo1 = 0xCD9E8D57u * c[2];
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c[2]);
        c[0] = hi1 ^ c[1] ^ k0;
        c[1] = lo1;
        c[2] = hi0 ^ c[3] ^ k1;
        c[3] = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Block-wide max of two non-negative values (one barrier).
__device__ __forceinline__ void block_max2(float &a, float &b, float (*red)[kWaves]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    a = wave_max(a);
    b = wave_max(b);
    if (lane == 0) {
        red[0][wave] = a;
        red[1][wave] = b;
    }
    __syncthreads();
    a = red[0][0];
    b = red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        a = fmaxf(a, red[0][w]);
        b = fmaxf(b, red[1][w]);
    }
}

// rank-th smallest (0-based) of the block's 2048 keys (8 per thread): LDS
// radix select over the 31 magnitude bits in digits of 11, 11 and 9 bits.
// Keys are bit patterns of non-negative floats, whose order they preserve.
__device__ uint32_t block_select(const uint32_t (&key)[kItems], uint32_t rank, uint32_t *hist,
                                 uint32_t *scratch) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t prefix = 0, pmask = 0;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 20 : (pass == 1 ? 9 : 0);
        const int bits = pass == 2 ? 9 : 11;
        const int nb = 1 << bits;
        const int per = nb / kThreads;
        for (int i = tid; i < nb; i += kThreads) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kItems; ++i)
            if ((key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & (nb - 1)], 1u);
        __syncthreads();
        uint32_t mine = 0;
        for (int i = 0; i < per; ++i) mine += hist[tid * per + i];
        uint32_t incl = wave_inclusive_sum(mine, lane);
        if (lane == 63) scratch[wave] = incl;
        __syncthreads();
        for (int w = 0; w < wave; ++w) incl += scratch[w];
        const uint32_t excl = incl - mine;
        if (excl <= rank && rank < incl) {
            uint32_t cum = excl;
            int b = tid * per;
            while (cum + hist[b] <= rank) cum += hist[b++];
            scratch[kWaves] = (uint32_t)b;
            scratch[kWaves + 1] = rank - cum;
        }
        __syncthreads();
        const uint32_t digit = scratch[kWaves];
        rank = scratch[kWaves + 1];
        prefix |= digit << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
    }
    return prefix;
}

// ---------------------------------------------------------------- quantizer
// Code magnitude for |x| = a with statistic A and r = fl(qmax/A) (A >= kTiny).
template <bool kSR>
__device__ __forceinline__ float code_magnitude(float a, float A, float r, float qmax, uint32_t u16) {
    if (a >= A) return qmax;
    const float y = a * r;
    float k;
    if constexpr (kSR) {
        const float down = floorf(y);
        const float frac = y - down;
        const float u = (float)u16 * 0x1p-16f;
        k = down + (u < frac ? 1.0f : 0.0f);
    } else {
        k = rintf(y);
    }
    return fminf(k, qmax);
}

template <int kStore, bool kGradBf16, bool kSR, bool kPct>
__global__ void __launch_bounds__(kThreads) adam_step_kernel(StepArgs a) {
    constexpr bool kQuantM = (kStore == kStoreQ8);
    constexpr bool kQuantV = (kStore != kStoreBf16);

    const uint32_t blk = a.blk0 + blockIdx.x;
    const BlockDesc d = a.desc[blk];
    const TensorRef tr = a.tensors[d.tensor];
    const uint32_t n = (d.lb_n & (kBlock - 1)) + 1u;
    const uint32_t npad = (n + 15u) & ~15u;
    const size_t local = (size_t)(d.lb_n >> kBlockBits) * kBlock;
    const int tid = threadIdx.x;

    float *__restrict__ pp = tr.p + local;

    float p[kItems], g[kItems], mo[kItems], vo[kItems];

    // ---- load params and grads (vector loads; element loads in a ragged tail group)
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
        if (e0 + 4 <= n) {
            const f32x4 x = ld_f32x4(pp + e0);
            p[4 * j + 0] = x.x; p[4 * j + 1] = x.y; p[4 * j + 2] = x.z; p[4 * j + 3] = x.w;
            if constexpr (kGradBf16) {
                const u32x2 h = ld_u32x2(reinterpret_cast<const uint16_t *>(tr.g) + local + e0);
                g[4 * j + 0] = bf16_to_f32(h.x & 0xFFFFu);
                g[4 * j + 1] = bf16_to_f32(h.x >> 16);
                g[4 * j + 2] = bf16_to_f32(h.y & 0xFFFFu);
                g[4 * j + 3] = bf16_to_f32(h.y >> 16);
            } else {
                const f32x4 y = ld_f32x4(reinterpret_cast<const float *>(tr.g) + local + e0);
                g[4 * j + 0] = y.x; g[4 * j + 1] = y.y; g[4 * j + 2] = y.z; g[4 * j + 3] = y.w;
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool in = e0 + c < n;
                p[4 * j + c] = in ? ld_one(pp + e0 + c) : 0.0f;
                if constexpr (kGradBf16)
                    g[4 * j + c] = in ? bf16_to_f32(ld_one(reinterpret_cast<const uint16_t *>(tr.g) + local + e0 + c)) : 0.0f;
                else
                    g[4 * j + c] = in ? ld_one(reinterpret_cast<const float *>(tr.g) + local + e0 + c) : 0.0f;
            }
        }
    }

    // ---- load and decode the stored moments (padding entries hold zeros)
    float Am = 0.0f, Av = 0.0f;
    if constexpr (kQuantM) Am = a.m_scale[blk];
    if constexpr (kQuantV) Av = a.v_scale[blk];
    constexpr float Rm = 1.0f / 127.0f;
    constexpr float Rv = 1.0f / 255.0f;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
        const size_t s = d.gidx + e0;
        const bool in = e0 < npad;
        if constexpr (kStore == kStoreBf16) {
            u32x2 hm = {0u, 0u}, hv = {0u, 0u};
            if (in) {
                hm = ld_u32x2(reinterpret_cast<const uint16_t *>(a.m_state) + s);
                hv = ld_u32x2(reinterpret_cast<const uint16_t *>(a.v_state) + s);
            }
            mo[4 * j + 0] = bf16_to_f32(hm.x & 0xFFFFu); mo[4 * j + 1] = bf16_to_f32(hm.x >> 16);
            mo[4 * j + 2] = bf16_to_f32(hm.y & 0xFFFFu); mo[4 * j + 3] = bf16_to_f32(hm.y >> 16);
            vo[4 * j + 0] = bf16_to_f32(hv.x & 0xFFFFu); vo[4 * j + 1] = bf16_to_f32(hv.x >> 16);
            vo[4 * j + 2] = bf16_to_f32(hv.y & 0xFFFFu); vo[4 * j + 3] = bf16_to_f32(hv.y >> 16);
        } else {
            uint32_t cv = 0;
            if (in) cv = ld_u32(reinterpret_cast<const uint8_t *>(a.v_state) + s);
#pragma unroll
            for (int c = 0; c < 4; ++c) vo[4 * j + c] = ((float)((cv >> (8 * c)) & 0xFFu) * Rv) * Av;
            if constexpr (kQuantM) {
                uint32_t cm = 0;
                if (in) cm = ld_u32(reinterpret_cast<const int8_t *>(a.m_state) + s);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int32_t q = ((int32_t)(cm << (24 - 8 * c))) >> 24;
                    mo[4 * j + c] = ((float)q * Rm) * Am;
                }
            } else {
                f32x4 mf = {0.f, 0.f, 0.f, 0.f};
                if (in) mf = ld_f32x4(reinterpret_cast<const float *>(a.m_state) + s);
                mo[4 * j + 0] = mf.x; mo[4 * j + 1] = mf.y; mo[4 * j + 2] = mf.z; mo[4 * j + 3] = mf.w;
            }
        }
    }

    // ---- the Adam/AdamW element update (moments stay in registers)
    float mmax = 0.0f, vmax = 0.0f;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
        float gi = g[i];
        if (a.l2) gi = fmaf(a.wd, p[i], gi);
        const float m = fmaf(a.beta1, mo[i], a.omb1 * gi);
        const float v = fmaf(a.beta2, vo[i], a.omb2 * (gi * gi));
        const float den = fmaf(sqrtf(v), a.ibc2, a.eps);
        p[i] = fmaf(-a.step, m / den, p[i] * a.decay);
        mo[i] = m;
        vo[i] = v;
        mmax = fmaxf(mmax, fabsf(m));
        vmax = fmaxf(vmax, v);
    }

    // ---- store params
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
        if (e0 + 4 <= n) {
            st_f32x4(pp + e0, f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]});
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (e0 + c < n) st_one(pp + e0 + c, p[4 * j + c]);
        }
    }

    if constexpr (kStore == kStoreBf16) {
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
            if (e0 < npad) {
                const size_t s = d.gidx + e0;
                const u32x2 hm = {f32_to_bf16(mo[4 * j]) | (f32_to_bf16(mo[4 * j + 1]) << 16),
                                  f32_to_bf16(mo[4 * j + 2]) | (f32_to_bf16(mo[4 * j + 3]) << 16)};
                const u32x2 hv = {f32_to_bf16(vo[4 * j]) | (f32_to_bf16(vo[4 * j + 1]) << 16),
                                  f32_to_bf16(vo[4 * j + 2]) | (f32_to_bf16(vo[4 * j + 3]) << 16)};
                st_u32x2(reinterpret_cast<uint16_t *>(a.m_state) + s, hm);
                st_u32x2(reinterpret_cast<uint16_t *>(a.v_state) + s, hv);
            }
        }
        return;
    } else {
        // ---- block statistic
        __shared__ float red[2][kWaves];
        block_max2(mmax, vmax, red);
        float Amn = mmax, Avn = vmax;
        if constexpr (kPct) {
            __shared__ uint32_t hist[kBlock];
            __shared__ uint32_t scratch[kWaves + 2];
            const uint32_t rank = (uint32_t)floor(a.pfrac * (double)(n - 1)) + (kBlock - n);
            uint32_t key[kItems];
            if constexpr (kQuantM) {
#pragma unroll
                for (int i = 0; i < kItems; ++i) key[i] = __float_as_uint(mo[i]) & 0x7FFFFFFFu;
                const float sel = __uint_as_float(block_select(key, rank, hist, scratch));
                Amn = sel < kTiny ? mmax : sel;
                __syncthreads();  // hist/scratch reused below
            }
#pragma unroll
            for (int i = 0; i < kItems; ++i) key[i] = __float_as_uint(vo[i]) & 0x7FFFFFFFu;
            const float sel = __uint_as_float(block_select(key, rank, hist, scratch));
            Avn = sel < kTiny ? vmax : sel;
        }
        const bool mzero = !(Amn >= kTiny), vzero = !(Avn >= kTiny);
        const float rm = mzero ? 0.0f : 127.0f / Amn;
        const float rv = vzero ? 0.0f : 255.0f / Avn;

        // ---- requantize and store codes
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const uint32_t e0 = j * (kThreads * 4) + 4 * tid;
            if (e0 >= npad) continue;
            const size_t s = d.gidx + e0;
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if constexpr (kSR) {
                const uint64_t grp = s >> 2;
                uint32_t c[4] = {(uint32_t)grp, (uint32_t)(grp >> 32), a.t_lo, a.t_hi};
                philox4x32_10(c, a.seed_lo, a.seed_hi);
                w[0] = c[0]; w[1] = c[1]; w[2] = c[2]; w[3] = c[3];
            }
            uint32_t cv = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float k = vzero ? 0.0f
                                      : code_magnitude<kSR>(fabsf(vo[4 * j + c]), Avn, rv, 255.0f, w[c] >> 16);
                cv |= ((uint32_t)k) << (8 * c);
            }
            st_u32(reinterpret_cast<uint8_t *>(a.v_state) + s, cv);
            if constexpr (kQuantM) {
                uint32_t cm = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float x = mo[4 * j + c];
                    const float k = mzero ? 0.0f
                                          : code_magnitude<kSR>(fabsf(x), Amn, rm, 127.0f, w[c] & 0xFFFFu);
                    const int32_t q = x < 0.0f ? -(int32_t)k : (int32_t)k;
                    cm |= ((uint32_t)q & 0xFFu) << (8 * c);
                }
                st_u32(reinterpret_cast<int8_t *>(a.m_state) + s, cm);
            } else {
                st_f32x4(reinterpret_cast<float *>(a.m_state) + s,
                         f32x4{mo[4 * j], mo[4 * j + 1], mo[4 * j + 2], mo[4 * j + 3]});
            }
        }
        if (tid == 0) {
            if constexpr (kQuantM) a.m_scale[blk] = mzero ? 0.0f : Amn;
            a.v_scale[blk] = vzero ? 0.0f : Avn;
        }
    }
}

template <int kStore, bool kGradBf16, bool kSR, bool kPct>
hipError_t launch_one(const StepArgs &a, uint32_t nblk, hipStream_t stream) {
    hipLaunchKernelGGL((adam_step_kernel<kStore, kGradBf16, kSR, kPct>), dim3(nblk), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int kStore, bool kGradBf16>
hipError_t launch_q(const Variant &v, const StepArgs &a, uint32_t nblk, hipStream_t stream) {
    if (v.stochastic)
        return v.percentile ? launch_one<kStore, kGradBf16, true, true>(a, nblk, stream)
                            : launch_one<kStore, kGradBf16, true, false>(a, nblk, stream);
    return v.percentile ? launch_one<kStore, kGradBf16, false, true>(a, nblk, stream)
                        : launch_one<kStore, kGradBf16, false, false>(a, nblk, stream);
}

}  // namespace

hipError_t launch_step(const Variant &v, const StepArgs &a, uint32_t nblk, hipStream_t stream) {
    switch (v.storage) {
    case kStoreBf16:
        return v.grad_bf16 ? launch_one<kStoreBf16, true, false, false>(a, nblk, stream)
                           : launch_one<kStoreBf16, false, false, false>(a, nblk, stream);
    case kStoreQ8:
        return v.grad_bf16 ? launch_q<kStoreQ8, true>(v, a, nblk, stream)
                           : launch_q<kStoreQ8, false>(v, a, nblk, stream);
    case kStoreQ8VOnly:
        return v.grad_bf16 ? launch_q<kStoreQ8VOnly, true>(v, a, nblk, stream)
                           : launch_q<kStoreQ8VOnly, false>(v, a, nblk, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace adam_mi355x
