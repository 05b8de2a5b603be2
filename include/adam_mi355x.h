/*
 * adam_mi355x.h -- C ABI of the compressed-moment Adam/AdamW step for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the Adam parameter update whose optimizer state is kept
 * compressed, as two pages describe it:
 *   - "feat: add 8-bit Adam optimizer for memory efficiency" (AiDotNet PR
 *     #814): block-wise 8-bit state, one scale per block (default block
 *     2048), signed first moment / unsigned second moment, scales recomputed
 *     every step ("dynamic"), optional fp32 first moment
 *     (CompressBothMoments=false), optional stochastic rounding, optional
 *     percentile-based scale (default 99.9); each step dequantizes, applies
 *     the bias-corrected Adam update and requantizes (walkthrough sequence
 *     diagram); memory accounting (GetMemoryUsage); option validation
 *     (BlockSize > 0, percentile within 0..100: review comments).
 *   - "perf(training): make BF16-Adam fused-compatible (proper bf16 moment
 *     kernel, not a gate)" (AiDotNet PR #1745): first and second moments in
 *     half-size bf16 buffers updated by one fused Adam/AdamW kernel; the
 *     optimizer configuration that a compiled step was set up with is checked
 *     on every step so that a changed moment-storage flag is not missed
 *     (review comment on the drift-detection tuple).  The same page names
 *     AMSGrad as a variant still lacking a fused kernel; it is built here
 *     (layout option ADAM_OPT_AMSGRAD) after Reddi, Kale & Kumar, "On the
 *     Convergence of Adam and Beyond" (ICLR 2018), in PyTorch's convention.
 *
 * Numerics of one element (fp32, each operation rounded once; g widened
 * exactly from bf16 when grads are bf16):
 *   [Adam, L2-coupled:  g = fma(wd, p, g)]
 *   m = fma(beta1, m_old, (1-beta1)*g)
 *   v = fma(beta2, v_old, (1-beta2)*(g*g))
 *   [AMSGrad: w = max(w_old, v), the running maximum; w replaces v below]
 *   p = fma(-lr/(1-beta1^t), m / fma(sqrt(v), 1/sqrt(1-beta2^t), eps), p*decay)
 * with decay = 1 - lr*wd for AdamW and 1 for Adam, the bias-correction
 * scalars formed in fp64 on the host and rounded once to fp32.  bf16
 * storage rounds to nearest, ties to even.  8-bit storage: per block the
 * statistic A (max |x|, or the percentile entry of |x| -- falling back to
 * the max when that entry is below 2^-112) is stored as the fp32 scale; a
 * code q decodes to (q * fl(1/qmax)) * A with qmax = 127 (m, int8, -128
 * never produced) or 255 (v, uint8); encoding rounds |x| * fl(qmax/A) to
 * nearest-even (or stochastically: up iff u < frac with u a 16-bit draw of
 * Philox4x32-10, key = seed, counter = (draw index / 4, t), word = draw
 * index mod 4 -- the draw index being the flat index unless set otherwise
 * (adam_state_set_draw_index) -- low half for m and high half for v; the
 * AMSGrad maximum draws one Philox call per 8 elements: half (i mod 2) of
 * word (i / 2) mod 4 at counter (i / 8 + 2^63, t) for draw index i) and
 * pins |x| >= A to qmax; a block with A < 2^-112 stores zero codes and
 * scale 0.  The AMSGrad maximum is stored as v is: bf16, or uint8 codes
 * with their own per-block scale.
 *
 * State layout (device memory owned by the library): tensor k's segment has
 * pad16(numel_k) entries and starts at the sum of the earlier segments (its
 * "flat index" range); blocks of 2048 elements are numbered tensor-major,
 * one fp32 scale per block per quantized moment.  Padding entries take no
 * part in a step (whatever they hold decodes as zero) and a step stores
 * them back as zero.
 *
 * Threading: calls on one state must not run concurrently from several host
 * threads (they share its host-side table cache) and must be ordered on the
 * device (same stream, or the caller synchronizes); different states are
 * independent, from any threads and streams.  All device work is
 * enqueued on the caller's HIP stream (hipStream_t passed as void*; NULL is
 * the null stream); argument errors are reported synchronously before any
 * device work.  adam_last_error() returns a thread-local message for the
 * last failing call on the calling thread.  A host memory allocation that
 * fails inside any call returns ADAM_ENOMEM (no C++ exception crosses the
 * interface).
 */
#ifndef ADAM_MI355X_H
#define ADAM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct adam_state adam_state; /* opaque; owns all optimizer-state memory */

enum adam_status {
    ADAM_OK = 0,
    ADAM_EINVAL = -1,  /* bad argument or hyperparameter (see each call) */
    ADAM_EMODE = -2,   /* layout passed to adam_step differs from the one at create */
    ADAM_EALIGN = -3,  /* a param/grad pointer is not 16-byte aligned */
    ADAM_ENOMEM = -4,  /* device or pinned-host allocation failed */
    ADAM_EDEVICE = -5  /* a HIP call failed (includes launch errors) */
};

enum adam_storage {
    ADAM_STORE_BF16 = 1,     /* m, v: bf16 (round to nearest even) */
    ADAM_STORE_Q8 = 2,       /* m: int8 [-127,127], v: uint8, fp32 scale per block each */
    ADAM_STORE_Q8_V_ONLY = 3 /* m: fp32, v: uint8 + fp32 scale per block */
};

enum adam_grad_dtype { ADAM_GRAD_F32 = 0, ADAM_GRAD_BF16 = 1 };

enum adam_flags {
    ADAM_F_DECOUPLED_WD = 1u, /* AdamW (p *= 1 - lr*wd); else Adam with L2 (g += wd*p) */
    ADAM_F_STOCHASTIC = 2u,   /* 8-bit storage only: Philox stochastic rounding; else nearest-even */
    ADAM_F_PERCENTILE = 4u,   /* 8-bit storage only: percentile block statistic; else absmax */
    /* 8-bit storage only: static scales.  The 8-bit Adam page's options class
     * turns dynamic quantization (scales that follow the moments, the default)
     * on or off; off is read as: a block's scale is set by the first step that
     * quantizes it with a statistic >= 2^-112 (its stored scale still 0) and
     * is kept from then on; moment values at or beyond a kept scale take the
     * end code (+-127, 255).  Such blocks skip the block statistic.  Steps
     * with and without this flag may be mixed on one state. */
    ADAM_F_STATIC_SCALES = 8u
};

enum adam_buffer {
    ADAM_BUF_M_CODES = 0, /* int8[padded elements]     (Q8) */
    ADAM_BUF_V_CODES = 1, /* uint8[padded elements]    (Q8, Q8_V_ONLY) */
    ADAM_BUF_M_SCALE = 2, /* float[blocks]             (Q8) */
    ADAM_BUF_V_SCALE = 3, /* float[blocks]             (Q8, Q8_V_ONLY) */
    ADAM_BUF_M_BF16 = 4,  /* uint16[padded elements]   (BF16) */
    ADAM_BUF_V_BF16 = 5,  /* uint16[padded elements]   (BF16) */
    ADAM_BUF_M_F32 = 6,   /* float[padded elements]    (Q8_V_ONLY) */
    ADAM_BUF_VMAX_CODES = 7, /* uint8[padded elements] (Q8, Q8_V_ONLY with AMSGRAD) */
    ADAM_BUF_VMAX_SCALE = 8, /* float[blocks]          (Q8, Q8_V_ONLY with AMSGRAD) */
    ADAM_BUF_VMAX_BF16 = 9,  /* uint16[padded elements] (BF16 with AMSGRAD) */
    ADAM_BUF_COUNT = 10      /* number of buffer ids */
};

enum adam_options {
    ADAM_OPT_AMSGRAD = 1u /* keep the running maximum of v (AMSGrad) */
};

#define ADAM_BLOCK_SIZE 2048 /* the only block size the gfx950 kernels take */

typedef struct {
    int32_t storage;    /* enum adam_storage */
    int32_t grad_dtype; /* enum adam_grad_dtype */
    int32_t block_size; /* must be ADAM_BLOCK_SIZE */
    uint32_t options;   /* enum adam_options bits; unknown bits are EINVAL */
} adam_layout;

typedef struct {
    float lr;           /* >= 0, finite */
    float beta1;        /* in [0, 1) */
    float beta2;        /* in [0, 1) */
    float eps;          /* > 0, finite */
    float weight_decay; /* >= 0, finite */
    float percentile;   /* in [0, 100]; read only with ADAM_F_PERCENTILE */
    int64_t t;          /* 1-based step number (bias correction, SR counter) */
    uint32_t flags;     /* enum adam_flags */
    uint32_t reserved;  /* must be 0 */
    uint64_t seed;      /* Philox key for stochastic rounding */
} adam_hparams;

/*
 * Bytes of optimizer state for a tensor list, without allocating:
 *   sum_k pad16(numel_k) * e + blocks * s, with (e, s) = (4, 0) for BF16,
 *   (2, 8) for Q8 and (5, 4) for Q8_V_ONLY; ADAM_OPT_AMSGRAD adds (2, 0)
 *   for BF16 and (1, 4) for the 8-bit modes.
 * The per-block descriptor table (16 bytes per block) and the per-tensor
 * pointer table (16 bytes per tensor) are bookkeeping, not counted.
 * Memory accounting follows the 8-bit Adam page (GetMemoryUsage).
 * Pure host function.  Returns < 0 (an adam_status) on bad arguments:
 * n_tensors < 0, numels NULL with n_tensors > 0, numel < 0 or >= 2^32,
 * layout NULL or invalid.
 */
int64_t adam_state_bytes(int32_t n_tensors, const int64_t *numels, const adam_layout *layout);

/*
 * Creates a state for n_tensors tensors of the given element counts (zero
 * counts allowed; n_tensors may be 0) on the current HIP device: allocates
 * the moment buffers, scales and block-descriptor table and zero-fills them
 * (m = v = 0, scales 0: the initial state of the 8-bit Adam page).  Work is
 * enqueued on hip_stream and the call returns after it completes.
 * On success *out owns the state (free with adam_state_destroy).
 * Errors: EINVAL (as adam_state_bytes, or out NULL), ENOMEM, EDEVICE.
 */
int adam_state_create(adam_state **out, int32_t n_tensors, const int64_t *numels,
                      const adam_layout *layout, void *hip_stream);

/*
 * One Adam/AdamW step over every tensor of the state, enqueued on
 * hip_stream as a single kernel launch (one 256-thread workgroup per
 * 2048-element block).  The operation is the loop body of the 8-bit Adam
 * page's walkthrough sequence diagram (dequantize m and v, the Adam update
 * with bias correction, quantize m and v), fused into one pass over memory
 * as the BF16-Adam page's "The real fix" section asks for the bf16-moment
 * step; the layout check is that page's drift-detection review comment.
 *   params[k]: device float[numel_k], updated in place;
 *   grads[k]:  device float[numel_k] or bf16 (uint16)[numel_k] per the
 *              layout's grad_dtype, read only;
 *   both arrays are host arrays of n_tensors device pointers, each 16-byte
 *   aligned (NULL allowed only for zero-size tensors), owned by the caller
 *   and left untouched by the library beyond the kernel's accesses.
 *   expect: the layout the caller believes the state has; any difference
 *   from the layout given at create returns EMODE (no work enqueued).
 * Errors (no work enqueued): EINVAL (NULL state/params/grads/hp/expect,
 * hyperparameter outside its domain, unknown flag bits, reserved != 0,
 * STOCHASTIC, PERCENTILE or STATIC_SCALES with BF16 storage, call from a
 * device other than the one the state was created on, hip_stream in HIP
 * graph capture: a captured launch would replay this call's t and
 * hyperparameters with a pointer table that later calls may re-use), EMODE,
 * EALIGN; EDEVICE if the launch fails.  Device faults surface on the
 * caller's next synchronization.
 */
int adam_step(adam_state *s, float *const *params, const void *const *grads,
              const adam_hparams *hp, const adam_layout *expect, void *hip_stream);

/* Size in bytes of one state buffer (enum adam_buffer), or < 0 if the
   state's storage mode has no such buffer. */
int64_t adam_state_buffer_bytes(const adam_state *s, int32_t which);

/*
 * Copies a whole state buffer to dst (device or host memory, caller-owned),
 * or overwrites it from src, asynchronously on hip_stream; nbytes must equal
 * adam_state_buffer_bytes(s, which).  Used for inspection, checkpoints and
 * tests: the 8-bit Adam page's PR description lists full serialization
 * support among its key features, beside block-wise quantization with a
 * scale per block; these calls expose the state's buffers (codes, scales or
 * moments) one at a time.  Errors: EINVAL (unknown/absent buffer, size mismatch, NULL
 * pointer), EDEVICE.
 */
int adam_state_read(adam_state *s, int32_t which, void *dst, int64_t nbytes, void *hip_stream);
int adam_state_write(adam_state *s, int32_t which, const void *src, int64_t nbytes,
                     void *hip_stream);

/*
 * Checkpoint / resume of the whole optimizer state: the 8-bit Adam page
 * lists full serialization support, and its follow-up fix writes a presence
 * marker per moment so that a reader never assumes a buffer the writer did
 * not store.  The serialized form is a self-describing little-endian byte
 * stream in host memory:
 *   header   "MEAMSTAT", u32 version (2), u32 header bytes (40 + 16*n),
 *            i32 storage, i32 grad_dtype, i32 block_size, u32 options,
 *            i32 n_tensors, u32 0, i64 numels[n_tensors],
 *            i64 draw_index[n_tensors] (adam_state_set_draw_index)
 *   records  one per state buffer the layout has (enum adam_buffer order):
 *            u32 buffer id, u32 0, u64 byte count, the bytes, zero padding
 *            to a multiple of 8
 *   trailer  u32 0xFFFFFFFF, u32 record count, u64 checksum (a 64-bit
 *            multiply-xor hash over every preceding byte, 8 bytes at a time)
 * adam_state_serialized_bytes: the stream's size for this state (< 0 on a
 * NULL state).
 * adam_state_save: writes the stream to dst (host memory, nbytes exactly
 * the serialized size); the device copies are ordered on hip_stream after
 * earlier work on the state, and the call returns once dst is complete.
 * adam_state_load: validates the whole stream on the host (magic, version,
 * layout, numels, draw indices, the exact set and sizes of the records,
 * trailer and checksum) before any device call, then creates a state on the current
 * device holding exactly the saved contents (free with adam_state_destroy).
 * A resumed run is bit-identical to an uninterrupted one.
 * Errors: EINVAL (NULL pointers, size mismatch, any validation failure),
 * ENOMEM, EDEVICE.
 */
int64_t adam_state_serialized_bytes(const adam_state *s);
int adam_state_save(adam_state *s, void *dst, int64_t nbytes, void *hip_stream);
int adam_state_load(adam_state **out, const void *src, int64_t nbytes, void *hip_stream);

/*
 * Stochastic-rounding draw index of each tensor's element 0.  The draws of
 * an element come from the Philox counter of its draw index (see the
 * numerics above); by default that is the element's flat index in this
 * state.  A state that holds a shard of a larger parameter set (ZeRO-1:
 * block-aligned slices of tensors on several GPUs) sets, for each slice,
 * the flat index its first element has in the unsharded state, so that the
 * shards together draw exactly the unsharded state's stream.  The indices
 * are part of the state and of its checkpoint.
 * adam_state_set_draw_index: first_index[k] for k < n_tensors, each a
 * multiple of 16 with first_index[k] + pad16(numel_k) <= 2^62; uploaded on
 * hip_stream, ordered after earlier steps on it, and the call returns once
 * done.  Errors: EINVAL (NULL state, NULL array with tensors, an index out
 * of range), EDEVICE.
 * adam_state_get_draw_index (pure host): the first min(n_tensors,
 * max_tensors) indices into first_index; returns the tensor count, or < 0
 * on a NULL state (or NULL array with max_tensors > 0).
 */
int adam_state_set_draw_index(adam_state *s, const int64_t *first_index, void *hip_stream);
int32_t adam_state_get_draw_index(const adam_state *s, int64_t *first_index, int32_t max_tensors);

/* Describes a state (pure host): its layout and tensor count, and the
   first min(n_tensors, max_tensors) element counts into numels (which may
   be NULL when max_tensors is 0).  Returns the tensor count, or < 0 on a
   NULL state or layout pointer. */
int32_t adam_state_describe(const adam_state *s, adam_layout *layout, int64_t *numels,
                            int32_t max_tensors);

/* Frees every buffer of the state (after synchronizing the device).
   NULL is ignored. */
void adam_state_destroy(adam_state *s);

/*
 * adam_step_noalloc -- for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same step as adam_step (same kernels, same results bit for
 * bit) over state buffers the caller owns, with no state object, no
 * allocation and no host-to-device copy: the block-descriptor, pointer and
 * draw-index tables that adam_state_create would allocate live in one fixed
 * device array of the library (17.5 MiB per GPU, held until the process
 * ends) and are written by small fill kernels from kernel arguments, on
 * hip_stream, before the step kernel.
 *   numels, layout: the tensor list and layout, as for adam_state_create.
 *   params, grads: as for adam_step.
 *   state: ADAM_BUF_COUNT device pointers indexed by enum adam_buffer; the
 *     entries of the buffers the layout has (see adam_state_read) must point
 *     at caller-owned device memory of exactly the sizes a state of this
 *     tensor list would have (padded elements = sum of pad16(numel); blocks =
 *     sum of ceil(numel / 2048); scales in tensor-major block order), each
 *     16-byte aligned; the others are ignored.  A new state is all zeros.
 *   draw_index: per tensor, the stochastic-rounding draw index of element 0
 *     (see adam_state_set_draw_index), or NULL for the flat index.
 * Limits: at most 65536 tensors and 2^20 blocks (2^31 elements) per call;
 * larger lists return EINVAL with a message naming the limit.
 * Every call on a GPU shares that GPU's table array, and a call's tables
 * stay there until the next call rewrites them: calls that overlap on one
 * GPU (two streams, or two host threads, without ordering between them)
 * race on the tables and must not be issued.  Calls ordered on one stream
 * are safe.  A graph capture records the fill kernels with the step, so a
 * replay rewrites its own tables; it repeats the call as recorded (same t,
 * hyperparameters and pointers).
 * Errors (no work enqueued): EINVAL (as adam_state_bytes and adam_step, a
 * NULL state array or needed buffer, the limits above), EALIGN; EDEVICE if
 * a launch fails.
 */
int adam_step_noalloc(int32_t n_tensors, const int64_t *numels, const adam_layout *layout,
                      float *const *params, const void *const *grads, void *const *state,
                      const int64_t *draw_index, const adam_hparams *hp, void *hip_stream);

/* Thread-local description of the last error on this thread ("" if none). */
const char *adam_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ADAM_MI355X_H */
