// Host runtime behind the C ABI declared in include/adam_mi355x.h:
// argument validation, the padded state layout and per-block descriptor
// table, state allocation, the per-step host scalars (fp64, rounded once --
// the 8-bit Adam page's review comment forms the bias corrections with
// Math.Pow on doubles) and the kernel launch on the caller's stream.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "adam_internal.h"
#include "adam_mi355x.h"

using namespace adam_mi355x;

namespace {
constexpr int kTableSlots = 4;  // resident pointer tables per state
constexpr int kStageSlots = 8;  // pinned staging buffers per state

struct TableSlot {
    TensorRef *dev = nullptr;
    std::vector<TensorRef> ptrs;  // the pointer set this table holds
    uint64_t last_use = 0;
    bool valid = false;
};
}  // namespace

struct adam_state {
    int device = -1;
    adam_layout layout{};
    int32_t n_tensors = 0;
    std::vector<int64_t> numels;
    int64_t padded = 0;   // sum of pad16(numel)
    int64_t nblocks = 0;
    int64_t n_full = 0;   // blocks of 2048 elements (listed first)
    BlockDesc *d_desc = nullptr;
    // per tensor: the stochastic-rounding draw index of element 0 (default:
    // the tensor's own segment start in this state)
    std::vector<int64_t> draw_first;
    uint64_t *d_draw = nullptr;
    // Device copies of the caller's per-tensor {param, grad} pointer pairs.
    // A few recently used pointer sets stay resident, so a caller that
    // alternates between gradient buffers uploads nothing; a new set is
    // staged through a ring of pinned buffers so the host does not wait for
    // earlier uploads unless the ring wraps onto one still queued.
    TableSlot tables[kTableSlots];
    uint64_t table_clock = 0;
    TensorRef *stage[kStageSlots] = {};
    hipEvent_t stage_done[kStageSlots] = {};
    bool stage_pending[kStageSlots] = {};
    int next_stage = 0;
    void *m = nullptr;                   // bf16 / int8 / fp32 first moment
    void *v = nullptr;                   // bf16 / uint8 second moment
    float *m_scale = nullptr;
    float *v_scale = nullptr;
    void *w = nullptr;                   // AMSGrad running max of v: bf16 / uint8
    float *w_scale = nullptr;
};

namespace {

thread_local std::string g_error;

int fail(int code, const std::string &msg) {
    g_error = msg;
    return code;
}

// Runs an entry point's body: a host allocation failure inside it comes back
// as ADAM_ENOMEM instead of escaping through the C ABI.
template <class F>
auto guarded(F &&body) noexcept -> decltype(body()) {
    try {
        return body();
    } catch (const std::bad_alloc &) {
        try { g_error = "host allocation failed"; } catch (...) { g_error.clear(); }
        return ADAM_ENOMEM;
    } catch (...) {
        try { g_error = "unexpected host exception"; } catch (...) { g_error.clear(); }
        return ADAM_EDEVICE;
    }
}

int64_t pad16(int64_t n) { return (n + 15) / 16 * 16; }

int64_t blocks_of(int64_t n) { return (n + kBlock - 1) / kBlock; }

int check_layout(const adam_layout *l) {
    if (!l) return fail(ADAM_EINVAL, "layout is NULL");
    if (l->storage != ADAM_STORE_BF16 && l->storage != ADAM_STORE_Q8 && l->storage != ADAM_STORE_Q8_V_ONLY)
        return fail(ADAM_EINVAL, "unknown storage mode " + std::to_string(l->storage));
    if (l->grad_dtype != ADAM_GRAD_F32 && l->grad_dtype != ADAM_GRAD_BF16)
        return fail(ADAM_EINVAL, "unknown grad dtype " + std::to_string(l->grad_dtype));
    if (l->block_size != ADAM_BLOCK_SIZE)
        return fail(ADAM_EINVAL, "block_size must be " + std::to_string(ADAM_BLOCK_SIZE) + ", got " +
                                     std::to_string(l->block_size));
    if (l->options & ~(uint32_t)ADAM_OPT_AMSGRAD) return fail(ADAM_EINVAL, "unknown layout option bits");
    return ADAM_OK;
}

int check_numels(int32_t n_tensors, const int64_t *numels) {
    if (n_tensors < 0) return fail(ADAM_EINVAL, "n_tensors < 0");
    if (n_tensors > 0 && !numels) return fail(ADAM_EINVAL, "numels is NULL");
    for (int32_t k = 0; k < n_tensors; ++k)
        if (numels[k] < 0 || numels[k] >= (int64_t(1) << 32))
            return fail(ADAM_EINVAL, "numel of tensor " + std::to_string(k) + " outside [0, 2^32)");
    return ADAM_OK;
}

bool amsgrad(const adam_layout &l) { return (l.options & ADAM_OPT_AMSGRAD) != 0; }

// (bytes per padded element, bytes per block) of a layout's state
void storage_costs(const adam_layout &l, int64_t &per_elem, int64_t &per_block) {
    switch (l.storage) {
    case ADAM_STORE_BF16: per_elem = 4; per_block = 0; break;
    case ADAM_STORE_Q8: per_elem = 2; per_block = 8; break;
    default: per_elem = 5; per_block = 4; break;
    }
    if (amsgrad(l)) {  // the running maximum is stored as v is
        per_elem += l.storage == ADAM_STORE_BF16 ? 2 : 1;
        per_block += l.storage == ADAM_STORE_BF16 ? 0 : 4;
    }
}

bool is_finite(float x) { return std::isfinite(x); }

int check_hparams(const adam_hparams *hp, int32_t storage) {
    if (!hp) return fail(ADAM_EINVAL, "hparams is NULL");
    if (hp->t < 1) return fail(ADAM_EINVAL, "t must be >= 1");
    if (!(hp->lr >= 0.0f) || !is_finite(hp->lr)) return fail(ADAM_EINVAL, "lr must be finite and >= 0");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f)) return fail(ADAM_EINVAL, "beta1 must be in [0, 1)");
    if (!(hp->beta2 >= 0.0f && hp->beta2 < 1.0f)) return fail(ADAM_EINVAL, "beta2 must be in [0, 1)");
    if (!(hp->eps > 0.0f) || !is_finite(hp->eps)) return fail(ADAM_EINVAL, "eps must be finite and > 0");
    if (!(hp->weight_decay >= 0.0f) || !is_finite(hp->weight_decay))
        return fail(ADAM_EINVAL, "weight_decay must be finite and >= 0");
    const uint32_t known = ADAM_F_DECOUPLED_WD | ADAM_F_STOCHASTIC | ADAM_F_PERCENTILE | ADAM_F_STATIC_SCALES;
    if (hp->flags & ~known) return fail(ADAM_EINVAL, "unknown flag bits");
    if (hp->reserved != 0) return fail(ADAM_EINVAL, "reserved must be 0");
    if ((hp->flags & ADAM_F_PERCENTILE) && !(hp->percentile >= 0.0f && hp->percentile <= 100.0f))
        return fail(ADAM_EINVAL, "percentile must be in [0, 100]");
    if (storage == ADAM_STORE_BF16 && (hp->flags & (ADAM_F_STOCHASTIC | ADAM_F_PERCENTILE | ADAM_F_STATIC_SCALES)))
        return fail(ADAM_EINVAL, "stochastic rounding, percentile and static scales apply to 8-bit storage only");
    return ADAM_OK;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(ADAM_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

// draw indices stay below 2^62, so index / 4 never reaches bit 63 of the Philox
// group counter, which the AMSGrad maximum's draws set
constexpr int64_t kDrawIndexLimit = int64_t(1) << 62;

// Draw indices must be multiples of 16 (a 4-element draw group never straddles
// two tensors) and keep every element's index below 2^62.
int check_draw_first(int32_t n_tensors, const int64_t *numels, const int64_t *first) {
    if (n_tensors > 0 && !first) return fail(ADAM_EINVAL, "draw index array is NULL");
    for (int32_t k = 0; k < n_tensors; ++k)
        if (first[k] < 0 || first[k] % 16 != 0 || first[k] > kDrawIndexLimit - pad16(numels[k]))
            return fail(ADAM_EINVAL, "draw index of tensor " + std::to_string(k) +
                                         " must be a multiple of 16 in [0, 2^62 - padded size]");
    return ADAM_OK;
}

void release(adam_state *s) {
    if (!s) return;
    if (s->device >= 0) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        if (cur != s->device) (void)hipSetDevice(s->device);
        (void)hipDeviceSynchronize();
        for (int i = 0; i < kStageSlots; ++i) {
            if (s->stage_done[i]) (void)hipEventDestroy(s->stage_done[i]);
            (void)hipHostFree(s->stage[i]);
        }
        for (int i = 0; i < kTableSlots; ++i) (void)hipFree(s->tables[i].dev);
        (void)hipFree(s->d_desc);
        (void)hipFree(s->d_draw);
        (void)hipFree(s->m);
        (void)hipFree(s->v);
        (void)hipFree(s->m_scale);
        (void)hipFree(s->v_scale);
        (void)hipFree(s->w);
        (void)hipFree(s->w_scale);
        if (cur >= 0 && cur != s->device) (void)hipSetDevice(cur);
    }
    delete s;
}

int alloc_zeroed(void **p, int64_t bytes, hipStream_t stream) {
    if (bytes == 0) return ADAM_OK;
    if (hipMalloc(p, (size_t)bytes) != hipSuccess) {
        (void)hipGetLastError();
        *p = nullptr;
        return fail(ADAM_ENOMEM, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
    }
    hipError_t e = hipMemsetAsync(*p, 0, (size_t)bytes, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync");
    return ADAM_OK;
}

struct BufferView {
    void *ptr;
    int64_t bytes;
};

BufferView buffer_of(const adam_state *s, int32_t which) {
    const int32_t st = s->layout.storage;
    const bool ams = amsgrad(s->layout);
    switch (which) {
    case ADAM_BUF_M_CODES: return st == ADAM_STORE_Q8 ? BufferView{s->m, s->padded} : BufferView{nullptr, -1};
    case ADAM_BUF_V_CODES: return st != ADAM_STORE_BF16 ? BufferView{s->v, s->padded} : BufferView{nullptr, -1};
    case ADAM_BUF_M_SCALE:
        return st == ADAM_STORE_Q8 ? BufferView{s->m_scale, 4 * s->nblocks} : BufferView{nullptr, -1};
    case ADAM_BUF_V_SCALE:
        return st != ADAM_STORE_BF16 ? BufferView{s->v_scale, 4 * s->nblocks} : BufferView{nullptr, -1};
    case ADAM_BUF_M_BF16: return st == ADAM_STORE_BF16 ? BufferView{s->m, 2 * s->padded} : BufferView{nullptr, -1};
    case ADAM_BUF_V_BF16: return st == ADAM_STORE_BF16 ? BufferView{s->v, 2 * s->padded} : BufferView{nullptr, -1};
    case ADAM_BUF_M_F32:
        return st == ADAM_STORE_Q8_V_ONLY ? BufferView{s->m, 4 * s->padded} : BufferView{nullptr, -1};
    case ADAM_BUF_VMAX_CODES:
        return ams && st != ADAM_STORE_BF16 ? BufferView{s->w, s->padded} : BufferView{nullptr, -1};
    case ADAM_BUF_VMAX_SCALE:
        return ams && st != ADAM_STORE_BF16 ? BufferView{s->w_scale, 4 * s->nblocks} : BufferView{nullptr, -1};
    case ADAM_BUF_VMAX_BF16:
        return ams && st == ADAM_STORE_BF16 ? BufferView{s->w, 2 * s->padded} : BufferView{nullptr, -1};
    default: return BufferView{nullptr, -1};
    }
}

// The per-step arguments of the kernel from hyperparameters (fp64 host
// scalars, each rounded once), shared by both step entry points.
void fill_scalars(StepArgs &a, const adam_hparams *hp) {
    const double b1 = hp->beta1, b2 = hp->beta2;
    const double bc1 = 1.0 - std::pow(b1, (double)hp->t);
    const double bc2 = 1.0 - std::pow(b2, (double)hp->t);
    const bool decoupled = (hp->flags & ADAM_F_DECOUPLED_WD) != 0;
    a.step = (float)((double)hp->lr / bc1);
    a.ibc2 = (float)(1.0 / std::sqrt(bc2));
    a.decay = decoupled ? (float)(1.0 - (double)hp->lr * (double)hp->weight_decay) : 1.0f;
    a.omb1 = (float)(1.0 - b1);
    a.omb2 = (float)(1.0 - b2);
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.eps = hp->eps;
    a.wd = hp->weight_decay;
    a.l2 = decoupled ? 0u : 1u;
    a.fast_ok = (hp->eps >= 0x1p-40f && hp->eps <= 0x1p20f) ? 1u : 0u;
    a.pfrac = (double)hp->percentile / 100.0;
    a.rank_full = (uint32_t)floor(a.pfrac * (double)(kBlock - 1));  // the kernel's own arithmetic
    a.seed_lo = (uint32_t)hp->seed;
    a.seed_hi = (uint32_t)(hp->seed >> 32);
    a.t_lo = (uint32_t)(uint64_t)hp->t;
    a.t_hi = (uint32_t)((uint64_t)hp->t >> 32);
}

}  // namespace

extern "C" {

const char *adam_last_error(void) { return g_error.c_str(); }

int64_t adam_state_bytes(int32_t n_tensors, const int64_t *numels, const adam_layout *layout) {
    int rc = check_numels(n_tensors, numels);
    if (rc) return rc;
    if ((rc = check_layout(layout))) return rc;
    int64_t per_elem, per_block;
    storage_costs(*layout, per_elem, per_block);
    int64_t total = 0;
    for (int32_t k = 0; k < n_tensors; ++k) total += pad16(numels[k]) * per_elem + blocks_of(numels[k]) * per_block;
    return total;
}

int adam_state_create(adam_state **out, int32_t n_tensors, const int64_t *numels, const adam_layout *layout,
                      void *hip_stream) {
    return guarded([&]() -> int {
        if (!out) return fail(ADAM_EINVAL, "out is NULL");
        *out = nullptr;
        int rc = check_numels(n_tensors, numels);
        if (rc) return rc;
        if ((rc = check_layout(layout))) return rc;

        int64_t total_blocks = 0, total_padded = 0;
        for (int32_t k = 0; k < n_tensors; ++k) {
            total_blocks += blocks_of(numels[k]);
            total_padded += pad16(numels[k]);
        }
        if (total_blocks >= (int64_t(1) << 32) || total_padded / 16 >= (int64_t(1) << 32))
            return fail(ADAM_EINVAL, "state too large: more than 2^32 - 1 blocks or 2^36 elements");

        adam_state *s = new (std::nothrow) adam_state();
        if (!s) return fail(ADAM_ENOMEM, "host allocation failed");
        hipError_t e = hipGetDevice(&s->device);
        if (e != hipSuccess) {
            s->device = -1;
            release(s);
            return hip_fail(e, "hipGetDevice");
        }
        s->layout = *layout;
        s->n_tensors = n_tensors;
        // descriptors: full blocks first, then each tensor's ragged last block;
        // scale slots keep the tensor-major block numbering
        std::vector<BlockDesc> desc, tails;
        try {
            s->numels.assign(numels, numels + n_tensors);
            s->draw_first.resize(n_tensors);
            desc.reserve((size_t)total_blocks);
            int64_t slot = 0;
            for (int32_t k = 0; k < n_tensors; ++k) {
                const int64_t n = numels[k];
                for (int64_t b = 0; b * kBlock < n; ++b, ++slot) {
                    const int64_t len = std::min<int64_t>(kBlock, n - b * kBlock);
                    const BlockDesc d{(uint32_t)((s->padded + b * kBlock) / 16), (uint32_t)k,
                                      (uint32_t)((b << kBlockBits) | (len - 1)), (uint32_t)slot};
                    (len == kBlock ? desc : tails).push_back(d);
                }
                s->draw_first[k] = s->padded;
                s->padded += pad16(n);
            }
            s->n_full = (int64_t)desc.size();
            desc.insert(desc.end(), tails.begin(), tails.end());
        } catch (const std::bad_alloc &) {
            release(s);
            return fail(ADAM_ENOMEM, "host allocation of the descriptor table failed");
        }
        s->nblocks = (int64_t)desc.size();

        hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
        const int32_t st = layout->storage;
        const int64_t m_bytes = st == ADAM_STORE_BF16 ? 2 * s->padded : (st == ADAM_STORE_Q8 ? s->padded : 4 * s->padded);
        const int64_t v_bytes = st == ADAM_STORE_BF16 ? 2 * s->padded : s->padded;
        if ((rc = alloc_zeroed(&s->m, m_bytes, stream)) || (rc = alloc_zeroed(&s->v, v_bytes, stream))) {
            release(s);
            return rc;
        }
        if (st == ADAM_STORE_Q8 && (rc = alloc_zeroed((void **)&s->m_scale, 4 * s->nblocks, stream))) {
            release(s);
            return rc;
        }
        if (st != ADAM_STORE_BF16 && (rc = alloc_zeroed((void **)&s->v_scale, 4 * s->nblocks, stream))) {
            release(s);
            return rc;
        }
        if (amsgrad(*layout) &&
            ((rc = alloc_zeroed(&s->w, st == ADAM_STORE_BF16 ? 2 * s->padded : s->padded, stream)) ||
             (st != ADAM_STORE_BF16 && (rc = alloc_zeroed((void **)&s->w_scale, 4 * s->nblocks, stream))))) {
            release(s);
            return rc;
        }
        if (s->nblocks > 0) {
            if (hipMalloc((void **)&s->d_desc, desc.size() * sizeof(BlockDesc)) != hipSuccess) {
                (void)hipGetLastError();
                release(s);
                return fail(ADAM_ENOMEM, "hipMalloc of the descriptor table failed");
            }
            e = hipMemcpyAsync(s->d_desc, desc.data(), desc.size() * sizeof(BlockDesc), hipMemcpyHostToDevice, stream);
            if (e != hipSuccess) {
                release(s);
                return hip_fail(e, "descriptor upload");
            }
        }
        if (n_tensors > 0) {
            if (hipMalloc((void **)&s->d_draw, (size_t)n_tensors * 8) != hipSuccess) {
                (void)hipGetLastError();
                release(s);
                return fail(ADAM_ENOMEM, "hipMalloc of the draw-index table failed");
            }
            e = hipMemcpyAsync(s->d_draw, s->draw_first.data(), (size_t)n_tensors * 8, hipMemcpyHostToDevice,
                               stream);
            if (e != hipSuccess) {
                release(s);
                return hip_fail(e, "draw-index upload");
            }
            const size_t tbytes = (size_t)n_tensors * sizeof(TensorRef);
            for (int i = 0; i < kTableSlots; ++i) {
                if (hipMalloc((void **)&s->tables[i].dev, tbytes) != hipSuccess) {
                    (void)hipGetLastError();
                    release(s);
                    return fail(ADAM_ENOMEM, "pointer table allocation failed");
                }
            }
            for (int i = 0; i < kStageSlots; ++i) {
                if (hipHostMalloc((void **)&s->stage[i], tbytes, hipHostMallocDefault) != hipSuccess) {
                    (void)hipGetLastError();
                    release(s);
                    return fail(ADAM_ENOMEM, "pinned staging allocation failed");
                }
                if ((e = hipEventCreateWithFlags(&s->stage_done[i], hipEventDisableTiming)) != hipSuccess) {
                    release(s);
                    return hip_fail(e, "hipEventCreate");
                }
            }
        }
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) {
            release(s);
            return hip_fail(e, "hipStreamSynchronize");
        }
        *out = s;
        return ADAM_OK;
    });
}

void adam_state_destroy(adam_state *s) { release(s); }

}  // extern "C"

// ---------------------------------------------------------------- checkpoint
namespace {
constexpr char kMagic[8] = {'M', 'E', 'A', 'M', 'S', 'T', 'A', 'T'};
constexpr uint32_t kFormatVersion = 2;
constexpr uint32_t kEndMarker = 0xFFFFFFFFu;

int64_t align8(int64_t n) { return (n + 7) / 8 * 8; }

// 64-bit multiply-xor hash over whole 8-byte words (little-endian), then the
// remaining bytes one at a time.
uint64_t stream_hash(const uint8_t *p, int64_t n) {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ (uint64_t)n;
    int64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t w;
        std::memcpy(&w, p + i, 8);
        h = (h ^ w) * 0x100000001B3ull;
        h ^= h >> 29;
    }
    for (; i < n; ++i) h = (h ^ p[i]) * 0x100000001B3ull;
    return h ^ (h >> 32);
}

// The state buffers a layout has, in enum adam_buffer order.
std::vector<int32_t> buffers_of(const adam_layout &l) {
    std::vector<int32_t> b;
    switch (l.storage) {
    case ADAM_STORE_BF16: b = {ADAM_BUF_M_BF16, ADAM_BUF_V_BF16}; break;
    case ADAM_STORE_Q8: b = {ADAM_BUF_M_CODES, ADAM_BUF_V_CODES, ADAM_BUF_M_SCALE, ADAM_BUF_V_SCALE}; break;
    default: b = {ADAM_BUF_V_CODES, ADAM_BUF_V_SCALE, ADAM_BUF_M_F32}; break;
    }
    if (amsgrad(l)) {
        if (l.storage == ADAM_STORE_BF16) {
            b.push_back(ADAM_BUF_VMAX_BF16);
        } else {
            b.push_back(ADAM_BUF_VMAX_CODES);
            b.push_back(ADAM_BUF_VMAX_SCALE);
        }
    }
    return b;
}

int64_t header_bytes(int32_t n_tensors) { return 40 + 16 * (int64_t)n_tensors; }

template <class T>
void put(uint8_t *base, int64_t &off, T v) {
    std::memcpy(base + off, &v, sizeof(T));
    off += sizeof(T);
}
template <class T>
bool get(const uint8_t *base, int64_t n, int64_t &off, T &v) {
    if (off + (int64_t)sizeof(T) > n) return false;
    std::memcpy(&v, base + off, sizeof(T));
    off += sizeof(T);
    return true;
}
}  // namespace

extern "C" {

int64_t adam_state_serialized_bytes(const adam_state *s) {
    return guarded([&]() -> int64_t {
        if (!s) return fail(ADAM_EINVAL, "state is NULL");
        int64_t n = header_bytes(s->n_tensors);
        for (int32_t b : buffers_of(s->layout)) n += 16 + align8(buffer_of(s, b).bytes);
        return n + 16;
    });
}

int adam_state_save(adam_state *s, void *dst, int64_t nbytes, void *hip_stream) {
    return guarded([&]() -> int {
        if (!s || !dst) return fail(ADAM_EINVAL, "state or destination is NULL");
        const int64_t need = adam_state_serialized_bytes(s);
        if (nbytes != need)
            return fail(ADAM_EINVAL, "nbytes " + std::to_string(nbytes) + " != serialized size " + std::to_string(need));
        uint8_t *out = static_cast<uint8_t *>(dst);
        hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
        int64_t off = 0;
        std::memcpy(out, kMagic, 8);
        off = 8;
        put<uint32_t>(out, off, kFormatVersion);
        put<uint32_t>(out, off, (uint32_t)header_bytes(s->n_tensors));
        put<int32_t>(out, off, s->layout.storage);
        put<int32_t>(out, off, s->layout.grad_dtype);
        put<int32_t>(out, off, s->layout.block_size);
        put<uint32_t>(out, off, s->layout.options);
        put<int32_t>(out, off, s->n_tensors);
        put<uint32_t>(out, off, 0u);
        for (int32_t k = 0; k < s->n_tensors; ++k) put<int64_t>(out, off, s->numels[k]);
        for (int32_t k = 0; k < s->n_tensors; ++k) put<int64_t>(out, off, s->draw_first[k]);
        const std::vector<int32_t> bufs = buffers_of(s->layout);
        hipError_t e;
        for (int32_t b : bufs) {
            const BufferView v = buffer_of(s, b);
            put<uint32_t>(out, off, (uint32_t)b);
            put<uint32_t>(out, off, 0u);
            put<uint64_t>(out, off, (uint64_t)v.bytes);
            if (v.bytes > 0 &&
                (e = hipMemcpyAsync(out + off, v.ptr, (size_t)v.bytes, hipMemcpyDeviceToHost, stream)) != hipSuccess)
                return hip_fail(e, "state copy to host");
            std::memset(out + off + v.bytes, 0, (size_t)(align8(v.bytes) - v.bytes));
            off += align8(v.bytes);
        }
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
        put<uint32_t>(out, off, kEndMarker);
        put<uint32_t>(out, off, (uint32_t)bufs.size());
        const uint64_t h = stream_hash(out, off);
        put<uint64_t>(out, off, h);
        return ADAM_OK;
    });
}

int adam_state_load(adam_state **out, const void *src, int64_t nbytes, void *hip_stream) {
    return guarded([&]() -> int {
        if (!out || !src) return fail(ADAM_EINVAL, "out or source is NULL");
        *out = nullptr;
        const uint8_t *in = static_cast<const uint8_t *>(src);
        int64_t off = 0;
        if (nbytes < header_bytes(0) + 16 || std::memcmp(in, kMagic, 8) != 0)
            return fail(ADAM_EINVAL, "not a serialized Adam state");
        off = 8;
        uint32_t version = 0, hbytes = 0, hzero = 1;
        adam_layout lay{};
        int32_t n_tensors = 0;
        get(in, nbytes, off, version);
        if (version != kFormatVersion) return fail(ADAM_EINVAL, "unsupported state format version " + std::to_string(version));
        get(in, nbytes, off, hbytes);
        get(in, nbytes, off, lay.storage);
        get(in, nbytes, off, lay.grad_dtype);
        get(in, nbytes, off, lay.block_size);
        get(in, nbytes, off, lay.options);
        get(in, nbytes, off, n_tensors);
        get(in, nbytes, off, hzero);
        if (n_tensors < 0 || hzero != 0 || (int64_t)hbytes != header_bytes(n_tensors) || (int64_t)hbytes > nbytes - 16)
            return fail(ADAM_EINVAL, "corrupt state header");
        int rc = check_layout(&lay);
        if (rc) return rc;
        std::vector<int64_t> numels(n_tensors);
        for (int32_t k = 0; k < n_tensors; ++k) get(in, nbytes, off, numels[k]);
        if ((rc = check_numels(n_tensors, numels.data()))) return rc;
        std::vector<int64_t> draw_first(n_tensors);
        for (int32_t k = 0; k < n_tensors; ++k) get(in, nbytes, off, draw_first[k]);
        if ((rc = check_draw_first(n_tensors, numels.data(), draw_first.data()))) return rc;
        // the trailer and checksum cover everything before the checksum itself
        if (nbytes % 8 != 0) return fail(ADAM_EINVAL, "serialized state size is not a multiple of 8");
        uint64_t want_hash = 0;
        std::memcpy(&want_hash, in + nbytes - 8, 8);
        if (stream_hash(in, nbytes - 8) != want_hash) return fail(ADAM_EINVAL, "serialized state checksum mismatch");
        // records: exactly the layout's buffers, in order, with the sizes it implies
        const std::vector<int32_t> bufs = buffers_of(lay);
        int64_t padded = 0, nblocks = 0;
        for (int64_t n : numels) {
            padded += pad16(n);
            nblocks += blocks_of(n);
        }
        std::vector<std::pair<int64_t, int64_t>> payload;  // (offset, bytes) per record
        for (int32_t b : bufs) {
            uint32_t id = 0, zero = 1;
            uint64_t len = 0;
            if (!get(in, nbytes, off, id) || !get(in, nbytes, off, zero) || !get(in, nbytes, off, len))
                return fail(ADAM_EINVAL, "truncated serialized state");
            int64_t expect = 0;
            switch (b) {
            case ADAM_BUF_M_CODES: case ADAM_BUF_V_CODES: case ADAM_BUF_VMAX_CODES: expect = padded; break;
            case ADAM_BUF_M_SCALE: case ADAM_BUF_V_SCALE: case ADAM_BUF_VMAX_SCALE: expect = 4 * nblocks; break;
            case ADAM_BUF_M_BF16: case ADAM_BUF_V_BF16: case ADAM_BUF_VMAX_BF16: expect = 2 * padded; break;
            default: expect = 4 * padded; break;
            }
            if ((int32_t)id != b || zero != 0 || (int64_t)len != expect)
                return fail(ADAM_EINVAL, "state record " + std::to_string(b) + " missing, out of order or of the wrong size");
            if (off + align8((int64_t)len) > nbytes - 16) return fail(ADAM_EINVAL, "truncated serialized state");
            payload.emplace_back(off, (int64_t)len);
            off += align8((int64_t)len);
        }
        uint32_t end = 0, count = 0;
        get(in, nbytes, off, end);
        get(in, nbytes, off, count);
        if (end != kEndMarker || count != bufs.size() || off != nbytes - 8)
            return fail(ADAM_EINVAL, "corrupt serialized state trailer");

        adam_state *s = nullptr;
        if ((rc = adam_state_create(&s, n_tensors, numels.data(), &lay, hip_stream))) return rc;
        if ((rc = adam_state_set_draw_index(s, draw_first.data(), hip_stream))) {
            release(s);
            return rc;
        }
        hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
        hipError_t e;
        for (size_t i = 0; i < bufs.size(); ++i) {
            const BufferView v = buffer_of(s, bufs[i]);
            if (v.bytes > 0 && (e = hipMemcpyAsync(v.ptr, in + payload[i].first, (size_t)v.bytes,
                                                   hipMemcpyHostToDevice, stream)) != hipSuccess) {
                release(s);
                return hip_fail(e, "state copy to device");
            }
        }
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) {
            release(s);
            return hip_fail(e, "hipStreamSynchronize");
        }
        *out = s;
        return ADAM_OK;
    });
}

int32_t adam_state_describe(const adam_state *s, adam_layout *layout, int64_t *numels, int32_t max_tensors) {
    if (!s || !layout) return fail(ADAM_EINVAL, "state or layout is NULL");
    if (max_tensors > 0 && !numels) return fail(ADAM_EINVAL, "numels is NULL");
    *layout = s->layout;
    for (int32_t k = 0; k < s->n_tensors && k < max_tensors; ++k) numels[k] = s->numels[k];
    return s->n_tensors;
}

int adam_state_set_draw_index(adam_state *s, const int64_t *first_index, void *hip_stream) {
    return guarded([&]() -> int {
        if (!s) return fail(ADAM_EINVAL, "state is NULL");
        int rc = check_draw_first(s->n_tensors, s->numels.data(), first_index);
        if (rc) return rc;
        if (s->n_tensors == 0) return ADAM_OK;
        hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
        std::copy(first_index, first_index + s->n_tensors, s->draw_first.begin());
        // stream order puts the copy after every earlier step that read the table
        hipError_t e = hipMemcpyAsync(s->d_draw, s->draw_first.data(), (size_t)s->n_tensors * 8,
                                      hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "draw-index upload");
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
        return ADAM_OK;
    });
}

int32_t adam_state_get_draw_index(const adam_state *s, int64_t *first_index, int32_t max_tensors) {
    if (!s) return fail(ADAM_EINVAL, "state is NULL");
    if (max_tensors > 0 && !first_index) return fail(ADAM_EINVAL, "first_index is NULL");
    for (int32_t k = 0; k < s->n_tensors && k < max_tensors; ++k) first_index[k] = s->draw_first[k];
    return s->n_tensors;
}

int64_t adam_state_buffer_bytes(const adam_state *s, int32_t which) {
    if (!s) return fail(ADAM_EINVAL, "state is NULL");
    const BufferView b = buffer_of(s, which);
    if (b.bytes < 0) return fail(ADAM_EINVAL, "buffer " + std::to_string(which) + " absent in this storage mode");
    return b.bytes;
}

static int copy_buffer(adam_state *s, int32_t which, void *dst, const void *src, int64_t nbytes,
                       void *hip_stream, bool read) {
    if (!s) return fail(ADAM_EINVAL, "state is NULL");
    const BufferView b = buffer_of(s, which);
    if (b.bytes < 0) return fail(ADAM_EINVAL, "buffer " + std::to_string(which) + " absent in this storage mode");
    if (nbytes != b.bytes)
        return fail(ADAM_EINVAL, "nbytes " + std::to_string(nbytes) + " != buffer size " + std::to_string(b.bytes));
    if (nbytes == 0) return ADAM_OK;
    if (read ? !dst : !src) return fail(ADAM_EINVAL, "NULL buffer pointer");
    hipError_t e = hipMemcpyAsync(read ? dst : b.ptr, read ? b.ptr : src, (size_t)nbytes, hipMemcpyDefault,
                                  reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
    return ADAM_OK;
}

int adam_state_read(adam_state *s, int32_t which, void *dst, int64_t nbytes, void *hip_stream) {
    return copy_buffer(s, which, dst, nullptr, nbytes, hip_stream, true);
}

int adam_state_write(adam_state *s, int32_t which, const void *src, int64_t nbytes, void *hip_stream) {
    return copy_buffer(s, which, nullptr, src, nbytes, hip_stream, false);
}

int adam_step(adam_state *s, float *const *params, const void *const *grads, const adam_hparams *hp,
              const adam_layout *expect, void *hip_stream) {
    return guarded([&]() -> int {
        if (!s) return fail(ADAM_EINVAL, "state is NULL");
        if (!expect) return fail(ADAM_EINVAL, "expected layout is NULL");
        if (expect->storage != s->layout.storage || expect->grad_dtype != s->layout.grad_dtype ||
            expect->block_size != s->layout.block_size || expect->options != s->layout.options)
            return fail(ADAM_EMODE, "layout differs from the one the state was created with");
        int rc = check_hparams(hp, s->layout.storage);
        if (rc) return rc;
        if (s->n_tensors > 0 && (!params || !grads)) return fail(ADAM_EINVAL, "params or grads is NULL");
        for (int32_t k = 0; k < s->n_tensors; ++k) {
            if (s->numels[k] == 0) continue;
            if (!params[k] || !grads[k]) return fail(ADAM_EINVAL, "NULL pointer for tensor " + std::to_string(k));
            if ((reinterpret_cast<uintptr_t>(params[k]) | reinterpret_cast<uintptr_t>(grads[k])) & 15u)
                return fail(ADAM_EALIGN, "tensor " + std::to_string(k) + " is not 16-byte aligned");
        }
        if (s->nblocks == 0) return ADAM_OK;
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        if (dev != s->device)
            return fail(ADAM_EINVAL, "state lives on device " + std::to_string(s->device) + ", current is " +
                                         std::to_string(dev));
        hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
        // A graph would replay this call's t and hyperparameters, and the
        // pointer table it names may be re-used by later calls (and a new
        // one's upload would read a recycled host staging slot at replay):
        // refuse before recording anything.
        hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(stream, &capture)) != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (capture != hipStreamCaptureStatusNone)
            return fail(ADAM_EINVAL, "adam_step cannot be recorded into a graph: the stream is capturing");

        // the device pointer table holding these pointers (uploading it if new)
        int slot = -1;
        for (int i = 0; i < kTableSlots && slot < 0; ++i) {
            const TableSlot &ts = s->tables[i];
            if (!ts.valid) continue;
            bool same = true;
            for (int32_t k = 0; k < s->n_tensors && same; ++k)
                same = ts.ptrs[k].p == params[k] && ts.ptrs[k].g == grads[k];
            if (same) slot = i;
        }
        if (slot < 0) {
            slot = 0;  // least recently used (or never used) table
            for (int i = 1; i < kTableSlots; ++i)
                if (!s->tables[i].valid || (s->tables[slot].valid && s->tables[i].last_use < s->tables[slot].last_use))
                    slot = i;
            TableSlot &ts = s->tables[slot];
            const int st = s->next_stage;
            s->next_stage = (st + 1) % kStageSlots;
            if (s->stage_pending[st]) {  // the ring wrapped onto a copy still queued
                if ((e = hipEventSynchronize(s->stage_done[st])) != hipSuccess) return hip_fail(e, "hipEventSynchronize");
                s->stage_pending[st] = false;
            }
            ts.valid = false;
            ts.ptrs.resize(s->n_tensors);
            for (int32_t k = 0; k < s->n_tensors; ++k) ts.ptrs[k] = TensorRef{params[k], grads[k]};
            std::memcpy(s->stage[st], ts.ptrs.data(), s->n_tensors * sizeof(TensorRef));
            // stream order puts this copy after every earlier kernel that reads ts.dev
            e = hipMemcpyAsync(ts.dev, s->stage[st], s->n_tensors * sizeof(TensorRef), hipMemcpyHostToDevice, stream);
            if (e != hipSuccess) return hip_fail(e, "pointer table upload");
            if ((e = hipEventRecord(s->stage_done[st], stream)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            s->stage_pending[st] = true;
            ts.valid = true;
        }
        s->tables[slot].last_use = ++s->table_clock;

        StepArgs a{};
        a.desc = s->d_desc;
        a.tensors = s->tables[slot].dev;
        a.m_state = s->m;
        a.v_state = s->v;
        a.m_scale = s->m_scale;
        a.v_scale = s->v_scale;
        a.draw_first = s->d_draw;
        a.w_state = s->w;
        a.w_scale = s->w_scale;
        fill_scalars(a, hp);  // host scalars: fp64, each rounded once to fp32

        a.n_full = (uint32_t)s->n_full;
        a.n_all = (uint32_t)s->nblocks;
        Variant v{s->layout.storage, s->layout.grad_dtype == ADAM_GRAD_BF16, (hp->flags & ADAM_F_STOCHASTIC) != 0,
                  (hp->flags & ADAM_F_PERCENTILE) != 0, (hp->flags & ADAM_F_STATIC_SCALES) != 0,
                  amsgrad(s->layout)};
        if ((e = launch_step(v, a, stream)) != hipSuccess) return hip_fail(e, "kernel launch");
        return ADAM_OK;
    });
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free step

extern "C" {

int adam_step_noalloc(int32_t n_tensors, const int64_t *numels, const adam_layout *layout, float *const *params,
                      const void *const *grads, void *const *state, const int64_t *draw_index,
                      const adam_hparams *hp, void *hip_stream) {
    return guarded([&]() -> int {
        int rc = check_numels(n_tensors, numels);
        if (rc) return rc;
        if ((rc = check_layout(layout))) return rc;
        if ((rc = check_hparams(hp, layout->storage))) return rc;
        if (n_tensors > (int32_t)kScratchMaxTensors)
            return fail(ADAM_EINVAL, "adam_step_noalloc takes at most " + std::to_string(kScratchMaxTensors) +
                                         " tensors, got " + std::to_string(n_tensors));
        int64_t nblocks = 0, padded = 0;
        for (int32_t k = 0; k < n_tensors; ++k) {
            nblocks += blocks_of(numels[k]);
            padded += pad16(numels[k]);
        }
        if (nblocks > (int64_t)kScratchMaxBlocks)
            return fail(ADAM_EINVAL, "adam_step_noalloc takes at most " + std::to_string(kScratchMaxBlocks) +
                                         " blocks of 2048 elements (its fixed table space), got " +
                                         std::to_string(nblocks));
        if (n_tensors > 0 && (!params || !grads)) return fail(ADAM_EINVAL, "params or grads is NULL");
        for (int32_t k = 0; k < n_tensors; ++k) {
            if (numels[k] == 0) continue;
            if (!params[k] || !grads[k]) return fail(ADAM_EINVAL, "NULL pointer for tensor " + std::to_string(k));
            if ((reinterpret_cast<uintptr_t>(params[k]) | reinterpret_cast<uintptr_t>(grads[k])) & 15u)
                return fail(ADAM_EALIGN, "tensor " + std::to_string(k) + " is not 16-byte aligned");
        }
        if (!state) return fail(ADAM_EINVAL, "state buffer array is NULL");
        for (int32_t b : buffers_of(*layout)) {
            if (padded == 0) break;
            if (!state[b]) return fail(ADAM_EINVAL, "state buffer " + std::to_string(b) + " is NULL");
            if (reinterpret_cast<uintptr_t>(state[b]) & 15u)
                return fail(ADAM_EALIGN, "state buffer " + std::to_string(b) + " is not 16-byte aligned");
        }
        if (draw_index && (rc = check_draw_first(n_tensors, numels, draw_index))) return rc;
        if (nblocks == 0) return ADAM_OK;

        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
        BlockDesc *desc = nullptr;
        TensorRef *tensors = nullptr;
        uint64_t *draw = nullptr;
        if ((e = scratch_tables(dev, &desc, &tensors, &draw)) != hipSuccess)
            return hip_fail(e, "scratch table address (hipGetSymbolAddress)");
        hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);

        // the tables, written on the device from kernel arguments (no host
        // staging buffer, no copy): full blocks first, then the ragged ones
        int64_t n_full = 0;
        for (int32_t k = 0; k < n_tensors; ++k) n_full += numels[k] / kBlock;
        FillArgs f{};
        f.desc = desc;
        f.tensors = tensors;
        f.draw = draw;
        int64_t full_at = 0, tail_at = n_full, slot = 0, seg = 0;
        for (int32_t k = 0; k < n_tensors; ++k) {
            const int64_t n = numels[k];
            if (n > 0) {
                FillTensor &t = f.t[f.count++];
                t.p = params[k];
                t.g = grads[k];
                t.draw = draw_index ? (uint64_t)draw_index[k] : (uint64_t)seg;
                t.n = (uint32_t)n;
                t.gidx16 = (uint32_t)(seg / 16);
                t.first_full = (uint32_t)full_at;
                t.tail = (uint32_t)tail_at;
                t.first_slot = (uint32_t)slot;
                t.index = (uint32_t)k;
                if (f.count == (uint32_t)kFillChunk) {
                    if ((e = launch_fill(f, stream)) != hipSuccess) return hip_fail(e, "table fill launch");
                    f.count = 0;
                }
            }
            full_at += n / kBlock;
            tail_at += (n % kBlock) != 0;
            slot += blocks_of(n);
            seg += pad16(n);
        }
        if (f.count > 0 && (e = launch_fill(f, stream)) != hipSuccess) return hip_fail(e, "table fill launch");

        StepArgs a{};
        a.desc = desc;
        a.tensors = tensors;
        a.draw_first = draw;
        const int32_t st = layout->storage;
        const bool ams = amsgrad(*layout);
        a.m_state = state[st == ADAM_STORE_BF16 ? ADAM_BUF_M_BF16 : (st == ADAM_STORE_Q8 ? ADAM_BUF_M_CODES : ADAM_BUF_M_F32)];
        a.v_state = state[st == ADAM_STORE_BF16 ? ADAM_BUF_V_BF16 : ADAM_BUF_V_CODES];
        a.m_scale = st == ADAM_STORE_Q8 ? static_cast<float *>(state[ADAM_BUF_M_SCALE]) : nullptr;
        a.v_scale = st != ADAM_STORE_BF16 ? static_cast<float *>(state[ADAM_BUF_V_SCALE]) : nullptr;
        a.w_state = ams ? state[st == ADAM_STORE_BF16 ? ADAM_BUF_VMAX_BF16 : ADAM_BUF_VMAX_CODES] : nullptr;
        a.w_scale = ams && st != ADAM_STORE_BF16 ? static_cast<float *>(state[ADAM_BUF_VMAX_SCALE]) : nullptr;
        fill_scalars(a, hp);
        a.n_full = (uint32_t)n_full;
        a.n_all = (uint32_t)nblocks;
        Variant v{st, layout->grad_dtype == ADAM_GRAD_BF16, (hp->flags & ADAM_F_STOCHASTIC) != 0,
                  (hp->flags & ADAM_F_PERCENTILE) != 0, (hp->flags & ADAM_F_STATIC_SCALES) != 0, ams};
        if ((e = launch_step(v, a, stream)) != hipSuccess) return hip_fail(e, "kernel launch");
        return ADAM_OK;
    });
}

}  // extern "C"
