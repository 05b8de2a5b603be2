// Stream probe: the Adam step's loads and stores with no arithmetic (the
// interface and the pattern are described in adam_stream_probe.h).  It is a
// measurement kernel, built as its own library; the step does not use it.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "adam_stream_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlock = 2048;
constexpr uint32_t kPattern = 0x01010101u;
constexpr int kCuLdsBytes = 160 * 1024;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// four elements of B bytes each, as one load / store
template <int B>
struct Quad;
template <>
struct Quad<1> {
    typedef uint32_t T;
};
template <>
struct Quad<2> {
    typedef u32x2 T;
};
template <>
struct Quad<4> {
    typedef u32x4 T;
};

template <int B>
__device__ __forceinline__ typename Quad<B>::T ld_quad(const void *base, size_t e) {
    return __builtin_nontemporal_load(reinterpret_cast<const typename Quad<B>::T *>(
        static_cast<const char *>(base) + e * B));
}
template <int B>
__device__ __forceinline__ void st_quad(void *base, size_t e, typename Quad<B>::T x) {
    __builtin_nontemporal_store(x, reinterpret_cast<typename Quad<B>::T *>(static_cast<char *>(base) + e * B));
}

struct ProbeArgs {
    float *p;
    const void *g;
    void *m;
    void *v;
    void *w;
    float *scales;
    uint32_t n_blocks;
};

// kG: grad bytes (4 or 2); kM, kV, kW: moment bytes per element (kW = 0: no
// third moment); kS: scales per block (0..3); 8-bit moments (kS > 0) put a
// barrier between the block's loads and its stores.
template <int kG, int kM, int kV, int kW, int kS>
__global__ void __launch_bounds__(kThreads) stream_probe_kernel(ProbeArgs a) {
    const uint32_t i0 = blockIdx.x, n = a.n_blocks;
    // the step's XCD order: workgroup i0 runs on XCD i0 mod 8, each XCD takes
    // runs of 16 consecutive blocks (a bijection on the first n - n mod 128)
    uint32_t blk = i0;
    if (i0 < n - n % 128u) {
        const uint32_t x = i0 & 7u, k = i0 >> 3;
        blk = ((k >> 4) << 7) + (x << 4) + (k & 15u);
    }
    const int tid = threadIdx.x;
    const size_t base = (size_t)blk * kBlock;

    f32x4 p[2];
    typename Quad<kG>::T g[2];
    typename Quad<kM>::T m[2];
    typename Quad<kV>::T v[2];
    typename Quad<(kW > 0 ? kW : 1)>::T w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const size_t e = base + (size_t)j * (kThreads * 4) + 4 * tid;
        p[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.p + e));
        g[j] = ld_quad<kG>(a.g, e);
        m[j] = ld_quad<kM>(a.m, e);
        v[j] = ld_quad<kV>(a.v, e);
        if constexpr (kW > 0) w[j] = ld_quad<kW>(a.w, e);
    }
    // the block's scales, read by every thread as the step reads them
    // (block-uniform addresses)
    uint32_t sc[3] = {0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kS; ++k) sc[k] = reinterpret_cast<const uint32_t *>(a.scales)[(size_t)k * n + blk];
    if constexpr (kS > 0) {
        // the step's block statistic needs every loaded value before its
        // barrier: wait for all of this thread's loads, then the barrier
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const size_t e = base + (size_t)j * (kThreads * 4) + 4 * tid;
        f32x4 gf;
        if constexpr (kG == 4) {
            gf = __builtin_bit_cast(f32x4, g[j]);
        } else {
            gf = f32x4{__uint_as_float(g[j].x << 16), __uint_as_float(g[j].x & 0xFFFF0000u),
                       __uint_as_float(g[j].y << 16), __uint_as_float(g[j].y & 0xFFFF0000u)};
        }
        __builtin_nontemporal_store(p[j] + gf, reinterpret_cast<f32x4 *>(a.p + e));
        st_quad<kM>(a.m, e, m[j] ^ kPattern);
        st_quad<kV>(a.v, e, v[j] ^ kPattern);
        if constexpr (kW > 0) st_quad<kW>(a.w, e, w[j] ^ kPattern);
    }
    if (kS > 0 && tid == 0) {
#pragma unroll
        for (int k = 0; k < kS; ++k)
            __builtin_nontemporal_store(sc[k] + 1u, reinterpret_cast<uint32_t *>(a.scales) + (size_t)k * n + blk);
    }
}

// per-storage layout: moment bytes per element and scales per block
struct Layout {
    int m, v, w, s;
};

bool layout_of(int32_t storage, int32_t amsgrad, Layout &l) {
    const bool ams = amsgrad != 0;
    switch (storage) {
    case 1:  // bf16 m, v (and w)
        l = Layout{2, 2, ams ? 2 : 0, 0};
        return true;
    case 2:  // 8-bit m, v (and w), a scale each
        l = Layout{1, 1, ams ? 1 : 0, ams ? 3 : 2};
        return true;
    case 3:  // fp32 m, 8-bit v (and w), a scale per 8-bit moment
        l = Layout{4, 1, ams ? 1 : 0, ams ? 2 : 1};
        return true;
    default:
        return false;
    }
}

template <int kG, int kM, int kV, int kW, int kS>
hipError_t launch(const ProbeArgs &a, size_t lds, hipStream_t stream) {
    hipLaunchKernelGGL((stream_probe_kernel<kG, kM, kV, kW, kS>), dim3(a.n_blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <int kG>
hipError_t launch_layout(const Layout &l, const ProbeArgs &a, size_t lds, hipStream_t stream) {
    if (l.m == 2) return l.w ? launch<kG, 2, 2, 2, 0>(a, lds, stream) : launch<kG, 2, 2, 0, 0>(a, lds, stream);
    if (l.m == 1) return l.w ? launch<kG, 1, 1, 1, 3>(a, lds, stream) : launch<kG, 1, 1, 0, 2>(a, lds, stream);
    return l.w ? launch<kG, 4, 1, 1, 2>(a, lds, stream) : launch<kG, 4, 1, 0, 1>(a, lds, stream);
}

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" uint64_t adam_stream_probe_bytes(uint32_t n_blocks, int32_t grad_bytes, int32_t storage,
                                            int32_t amsgrad) {
    Layout l;
    if (!layout_of(storage, amsgrad, l) || (grad_bytes != 2 && grad_bytes != 4)) return 0;
    const uint64_t n = (uint64_t)n_blocks * kBlock;
    return n * (uint64_t)(4 + 4 + grad_bytes + 2 * (l.m + l.v + l.w)) + (uint64_t)n_blocks * 8u * (uint64_t)l.s;
}

extern "C" int adam_stream_probe(void *param, const void *grad, void *m, void *v, void *w, float *scales,
                                 uint32_t n_blocks, int32_t grad_bytes, int32_t storage, int32_t amsgrad,
                                 int32_t resident_per_cu, void *stream) {
    Layout l;
    if (!layout_of(storage, amsgrad, l) || (grad_bytes != 2 && grad_bytes != 4)) return -1;
    if (n_blocks == 0 || n_blocks >= (1u << 24) || resident_per_cu < 2 || resident_per_cu > 8) return -1;
    if (!aligned16(param) || !aligned16(grad) || !aligned16(m) || !aligned16(v)) return -1;
    if (l.w && !aligned16(w)) return -1;
    if (l.s && !aligned16(scales)) return -1;
    const ProbeArgs a{static_cast<float *>(param), grad, m, v, w, scales, n_blocks};
    // LDS the kernel does not use, reserved so that at most resident_per_cu
    // workgroups fit on a CU (at 2: 54.6 KiB of the CU's 160)
    const size_t lds = resident_per_cu >= 8 ? 0 : (size_t)kCuLdsBytes / (size_t)(resident_per_cu + 1) + 1024;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = grad_bytes == 4 ? launch_layout<4>(l, a, lds, s) : launch_layout<2>(l, a, lds, s);
    return e == hipSuccess ? 0 : -5;
}
