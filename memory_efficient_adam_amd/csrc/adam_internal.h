// Internal interface between the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace adam_mi355x {

constexpr int kBlock = 2048;     // elements per quantization block (8-bit Adam page default)
constexpr int kThreads = 256;    // one workgroup per block: 4 wave64s
constexpr int kBlockBits = 11;   // log2(kBlock)

// One entry per 2048-element block, built once at create.  The table lists
// the full (2048-element) blocks first and the ragged last blocks of the
// tensors after them, so the hot loop over full blocks has no tail checks.
//   gidx16: flat (16-padded) state index of the block's first element / 16
//   tensor: index into the per-tensor pointer table
//   lb_n:   (block index within its tensor) << 11 | (elements in block - 1)
//   slot:   the block's scale slot (blocks numbered tensor-major)
struct BlockDesc {
    uint32_t gidx16;
    uint32_t tensor;
    uint32_t lb_n;
    uint32_t slot;
};
static_assert(sizeof(BlockDesc) == 16, "descriptor is one 16-byte load");

// Per-tensor device pointers, refreshed when the caller's pointers change.
struct TensorRef {
    float *p;
    const void *g;
};
static_assert(sizeof(TensorRef) == 16, "pointer pair is one 16-byte load");

enum Storage : int { kStoreBf16 = 1, kStoreQ8 = 2, kStoreQ8VOnly = 3 };

// Kernel arguments for one step (passed by value in the kernarg segment).
struct StepArgs {
    const BlockDesc *desc;
    const TensorRef *tensors;
    void *m_state;   // bf16 / int8 codes / fp32, per storage mode
    void *v_state;   // bf16 / uint8 codes
    float *m_scale;  // per block (Q8)
    float *v_scale;  // per block (Q8, Q8_V_ONLY)
    const uint64_t *draw_first;  // per tensor: stochastic-rounding draw index of element 0
    void *w_state;   // AMSGrad running max of v: bf16 / uint8 codes (else NULL)
    float *w_scale;  // its per-block scale (8-bit storage with AMSGrad)
    float step;      // lr / (1 - beta1^t)
    float ibc2;      // 1 / sqrt(1 - beta2^t)
    float decay;     // 1 - lr*wd (AdamW) or 1 (Adam)
    float omb1;      // 1 - beta1
    float omb2;      // 1 - beta2
    float beta1, beta2, eps, wd;
    uint32_t l2;     // 1: Adam with L2-coupled decay (g += wd*p)
    uint32_t fast_ok;  // 1: eps in [2^-40, 2^20], so the short exact sqrt/divide may apply
    double pfrac;    // percentile / 100 (percentile statistic)
    uint32_t rank_full;  // floor(pfrac * 2047): the percentile's rank in a full block
    uint32_t seed_lo, seed_hi, t_lo, t_hi;
    uint32_t n_full;   // descriptors [0, n_full) are full blocks
    uint32_t n_all;    // descriptors [n_full, n_all) are ragged last blocks
};

struct Variant {
    int storage;     // Storage
    bool grad_bf16;
    bool stochastic;
    bool percentile;
    bool static_scales;  // keep a block's scale once set (8-bit storage)
    bool amsgrad;        // the state holds the running max of v
};

// Enqueues the step kernel over every descriptor.
hipError_t launch_step(const Variant &v, const StepArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- allocation-free step
// The allocation-free entry point keeps the tables a state would own (block
// descriptors, per-tensor pointer pairs and draw indices) in one file-scope
// device array of the kernel module, so it allocates nothing.  Its limits:
constexpr uint32_t kScratchMaxTensors = 65536;
constexpr uint32_t kScratchMaxBlocks = 1u << 20;  // 2^31 elements in 2048-blocks

// The device address of the scratch tables on `device` (which must be the
// current device): taken once per device with hipGetSymbolAddress, then
// cached.  desc[kScratchMaxBlocks], tensors[kScratchMaxTensors],
// draw[kScratchMaxTensors].
hipError_t scratch_tables(int device, BlockDesc **desc, TensorRef **tensors, uint64_t **draw);

// One tensor's entries of the scratch tables, written on the device by a
// fill kernel (48 bytes, passed in the kernel arguments).
struct FillTensor {
    float *p;
    const void *g;
    uint64_t draw;        // draw index of element 0
    uint32_t n;           // numel (>= 1)
    uint32_t gidx16;      // flat index of element 0 / 16
    uint32_t first_full;  // descriptor index of its first full block
    uint32_t tail;        // descriptor index of its ragged last block (if n % 2048)
    uint32_t first_slot;  // scale slot of its first block
    uint32_t index;       // tensor index
};
static_assert(sizeof(FillTensor) == 48, "fill entry layout");

constexpr int kFillChunk = 64;  // tensors per fill launch (kernel arguments < 4 KiB)
struct FillArgs {
    BlockDesc *desc;
    TensorRef *tensors;
    uint64_t *draw;
    uint32_t count;  // entries of t[] used
    uint32_t pad;
    FillTensor t[kFillChunk];
};

hipError_t launch_fill(const FillArgs &f, hipStream_t stream);

}  // namespace adam_mi355x
