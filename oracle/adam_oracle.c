/*
 * adam_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of the Adam/AdamW parameter step whose
 * moment state is stored compressed (bf16 moments, or block-wise 8-bit codes
 * with one fp32 scale per block).  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load this library; the product path
 * never does.  It shares no source, header, table or constant generator with
 * the HIP implementation.
 *
 * Sources (web pages; cited by title and section):
 *   [P814]  "feat: add 8-bit Adam optimizer for memory efficiency" (AiDotNet
 *           PR #814): the PR description's key-features list, the walkthrough's
 *           sequence diagram (Dequantize -> Adam update with bias correction ->
 *           Quantize), the review comments on Adam8BitOptimizerOptions and on
 *           UpdateParameters, the follow-up commit message, and the PR body's
 *           "Motivation" and "Implementation Details" sections.
 *   [P1745] "perf(training): make BF16-Adam fused-compatible (proper bf16
 *           moment kernel, not a gate)" (AiDotNet PR #1745): the PR description
 *           and the "The real fix" section (half-size ushort m/v buffers, fused
 *           Adam/AdamW).
 *   [SMDS11] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *           1, 2, 3", SC'11 -- definition of the Philox4x32 bijection.
 *   [KB15]  Kingma & Ba, "Adam: A Method for Stochastic Optimization",
 *           Algorithm 1 (the pages name the update but never print it).
 *   [RKK18] Reddi, Kale & Kumar, "On the Convergence of Adam and Beyond",
 *           ICLR 2018 -- AMSGrad, which [P1745] names (the PR description and
 *           "The real fix": still without a fused kernel) but never prints.
 *
 * Precision: the pages store params and per-block scales as 32-bit floats and
 * moments as bf16 or bytes; every code is an integer decided by fp32
 * arithmetic, so this oracle computes in fp32 with each operation written
 * out once (explicit fmaf, correctly rounded / and sqrtf, no contraction:
 * build with -O2 -ffp-contract=off, no fast-math).  Host scalars are formed in
 * fp64 and rounded once.
 *
 * Pins (tests/test_oracle_*.py check each against something other than this
 * file): t=1 closed form, g=0 decay-only, textbook fp64 Adam and
 * torch.optim.AdamW, exhaustive round-trip / fixed-point / constant-block
 * properties of the codebook, brute-force nearest-code search, exhaustive
 * stochastic-rounding draw counts, numpy.percentile(method="lower"), the
 * PyTorch bf16 cast, and PyTorch's header-only Philox engine.  Static scales:
 * first step equal to the dynamic one, scales unchanged once set, later codes
 * nearest in the codebook of the kept scale (brute force).  AMSGrad:
 * torch.optim.AdamW/Adam(amsgrad=True) in the fp32 mode, the running
 * maximum's draws against PyTorch's Philox engine, every 8-bit step of a
 * 6-step run composed from pinned parts.
 * Multi-step trajectories: every step of 8-step runs checked from the state
 * the oracle holds before it (decoded, one torch.optim.AdamW step, the
 * result re-encoded by the pinned rules), in the bf16, 8-bit and fp32-m
 * modes with nearest and stochastic rounding.  The pages print no worked
 * multi-step example to compare a trajectory with as a whole.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Bit views                                                            */
/* ------------------------------------------------------------------ */
static uint32_t bits_of(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float float_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* ------------------------------------------------------------------ */
/* bf16 storage [P1745, "The real fix": m/v kept as half-size ushort    */
/* buffers]. Reading: the stored 16 bits are the upper half of the fp32 */
/* pattern rounded to nearest, ties to even; NaN -> 0x7FC0; widening    */
/* back is exact (append 16 zero bits).                                 */
/* ------------------------------------------------------------------ */
uint16_t orc_bf16_from_f32(float x)
{
    if (isnan(x))
        return 0x7FC0u;
    uint32_t u = bits_of(x);
    uint32_t upper = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    /* round up when the dropped half is above one half, or exactly one
       half and the kept part is odd */
    if (dropped > 0x8000u || (dropped == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

float orc_f32_from_bf16(uint16_t h)
{
    return float_of(((uint32_t)h) << 16);
}

void orc_bf16_from_f32_array(const float *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_bf16_from_f32(x[i]);
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 [SMDS11]: ten rounds of the 4x32 S-box, key bumped by  */
/* the Weyl constants between rounds.                                   */
/* ------------------------------------------------------------------ */
static void philox_round(uint32_t c[4], const uint32_t k[2])
{
    const uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    const uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    const uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    const uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t out[4];
    out[0] = hi1 ^ c[1] ^ k[0];
    out[1] = lo1;
    out[2] = hi0 ^ c[3] ^ k[1];
    out[3] = lo0;
    memcpy(c, out, sizeof out);
}

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; r++) {
        if (r > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        philox_round(c, k);
    }
    memcpy(out, c, sizeof c);
}

/* Stochastic-rounding draws [P814, key features: "stochastic rounding
   option"].  Reading: element with padded flat index i at step t takes
   word (i mod 4) of Philox4x32-10 with key = (lo32 seed, hi32 seed) and
   counter = (lo32(c), hi32(c), lo32 t, hi32 t), c = i/4.  The first moment
   (which 0) uses the low 16 bits of that word, the second moment (which 1)
   the high 16 bits.  The running maximum of the second moment (AMSGrad,
   which 2) draws from a second stream, one Philox call per 8 elements:
   element i takes half (i mod 2) -- the low 16 bits for even i, the high 16
   for odd i -- of word ((i/2) mod 4) at counter c = i/8 + 2^63 (flat
   indices stay below 2^62, so these counters never meet the first
   stream's). */
void orc_sr_draws(uint64_t seed, int64_t t, int64_t gidx0, int64_t n,
                  int32_t which, uint16_t *out)
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int64_t j = 0; j < n; j++) {
        const uint64_t i = (uint64_t)(gidx0 + j);
        const uint64_t grp = which == 2 ? ((i >> 3) | (1ull << 63)) : (i >> 2);
        const uint32_t ctr[4] = {(uint32_t)grp, (uint32_t)(grp >> 32),
                                 (uint32_t)(uint64_t)t, (uint32_t)((uint64_t)t >> 32)};
        uint32_t w[4];
        orc_philox4x32_10(ctr, key, w);
        uint32_t half_hi;
        uint32_t word;
        if (which == 2) {
            word = w[(i >> 1) & 3u];
            half_hi = (uint32_t)(i & 1u);
        } else {
            word = w[i & 3u];
            half_hi = which == 1;
        }
        out[j] = (uint16_t)(half_hi ? (word >> 16) : (word & 0xFFFFu));
    }
}

/* ------------------------------------------------------------------ */
/* Block statistic [P814, key features: "block-wise quantization",     */
/* "percentile-based scaling for outlier robustness"; review comment on */
/* QuantizationPercentile: values outside 0..100 break the index].      */
/* a[] holds non-negative magnitudes.  Absmax mode: the exact maximum.  */
/* Percentile mode: entry floor(p/100*(n-1)) (p/100 formed in fp64) of  */
/* the ascending order; if that entry is below TINY, the maximum.       */
/* ------------------------------------------------------------------ */
#define ORC_TINY 0x1p-112f

static int cmp_float_asc(const void *pa, const void *pb)
{
    const float a = *(const float *)pa, b = *(const float *)pb;
    return (a > b) - (a < b);
}

int64_t orc_percentile_rank(float p, int64_t n)
{
    const double frac = (double)p / 100.0;
    return (int64_t)floor(frac * (double)(n - 1));
}

float orc_block_stat(const float *a, int64_t n, int32_t use_pct, float p)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++)
        if (a[i] > amax)
            amax = a[i];
    if (!use_pct || n == 0)
        return amax;
    float *sorted = (float *)malloc((size_t)n * sizeof(float));
    memcpy(sorted, a, (size_t)n * sizeof(float));
    qsort(sorted, (size_t)n, sizeof(float), cmp_float_asc);
    float stat = sorted[orc_percentile_rank(p, n)];
    free(sorted);
    if (stat < ORC_TINY)
        stat = amax;
    return stat;
}

/* ------------------------------------------------------------------ */
/* Codebook and quantizer [P814, key features: signed first moment,     */
/* unsigned second moment; follow-up commit: symmetric [-127,127]       */
/* alphabet with one byte value unused].  Reading: the stored scale is  */
/* the block statistic A itself; code q decodes to fl(fl(q*R)*A) with   */
/* R = fl(1/qmax); qmax = 127 (signed) or 255 (unsigned).               */
/* ------------------------------------------------------------------ */
float orc_dequantize(int32_t q, float A, int32_t is_signed)
{
    const float qmax = is_signed ? 127.0f : 255.0f;
    const float R = 1.0f / qmax;
    const float unit = (float)q * R;
    return unit * A;
}

void orc_dequantize_block(const int32_t *codes, int64_t n, int32_t is_signed,
                          float A, float *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_dequantize(codes[i], A, is_signed);
}

/* Quantize one block given its statistic A (already chosen).  draws == NULL
   selects round-to-nearest-even; otherwise draws[i] (16 bits) selects
   stochastic rounding: round up iff draws[i]/2^16 < fractional part.
   Returns the scale to store (0 for a block whose statistic is below TINY). */
float orc_quantize_with_stat(const float *x, int64_t n, int32_t is_signed, float A,
                             const uint16_t *draws, int32_t *codes)
{
    const int32_t qmax = is_signed ? 127 : 255;
    if (!(A >= ORC_TINY)) {
        for (int64_t i = 0; i < n; i++)
            codes[i] = 0;
        return 0.0f;
    }
    const float r = (float)qmax / A;
    for (int64_t i = 0; i < n; i++) {
        const float a = fabsf(x[i]);
        int32_t k;
        if (a >= A) {
            k = qmax; /* at or beyond the statistic: the end of the alphabet */
        } else {
            const float y = a * r;
            if (draws == NULL) {
                k = (int32_t)rintf(y); /* ties to even (default rounding mode) */
            } else {
                const float down = floorf(y);
                const float frac = y - down;           /* exact */
                const float u = (float)draws[i] * 0x1p-16f; /* exact */
                k = (int32_t)down + (u < frac ? 1 : 0);
            }
            if (k > qmax)
                k = qmax;
        }
        codes[i] = (is_signed && x[i] < 0.0f) ? -k : k;
    }
    return A;
}

/* Statistic + quantization of one block of raw moment values. */
float orc_quantize_block(const float *x, int64_t n, int32_t is_signed, int32_t use_pct,
                         float p, const uint16_t *draws, int32_t *codes)
{
    float *mag = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; i++)
        mag[i] = fabsf(x[i]);
    const float A = orc_block_stat(mag, n, use_pct, p);
    free(mag);
    return orc_quantize_with_stat(x, n, is_signed, A, draws, codes);
}

/* ------------------------------------------------------------------ */
/* Host scalars [P814 review comment on UpdateParameters: bias          */
/* corrections via Math.Pow on doubles].  bc1 = 1-b1^t, bc2 = 1-b2^t in */
/* fp64; out = {step = lr/bc1, ibc2 = 1/sqrt(bc2), decay, 1-b1, 1-b2},  */
/* each rounded once to fp32.  decay = 1 - lr*wd for decoupled weight   */
/* decay (AdamW), 1 for L2-coupled Adam [P1745: plain Adam/AdamW].      */
/* ------------------------------------------------------------------ */
void orc_host_scalars(float lr, float beta1, float beta2, float wd, int64_t t,
                      int32_t decoupled, float out[5])
{
    const double b1 = (double)beta1, b2 = (double)beta2;
    const double bc1 = 1.0 - pow(b1, (double)t);
    const double bc2 = 1.0 - pow(b2, (double)t);
    out[0] = (float)((double)lr / bc1);
    out[1] = (float)(1.0 / sqrt(bc2));
    out[2] = decoupled ? (float)(1.0 - (double)lr * (double)wd) : 1.0f;
    out[3] = (float)(1.0 - b1);
    out[4] = (float)(1.0 - b2);
}

/* ------------------------------------------------------------------ */
/* The step [P814 sequence diagram: dequantize m, dequantize v, Adam    */
/* update with bias correction, quantize m, quantize v; KB15 Alg. 1].   */
/* ------------------------------------------------------------------ */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q8 = 2, ORC_Q8_V_ONLY = 3 };

typedef struct {
    float lr, beta1, beta2, eps, wd, pct;
    int64_t t;
    int32_t decoupled, stochastic, use_pct, static_scales, amsgrad;
    uint64_t seed;
} orc_hparams;

/* Scale of one quantized moment of a block [P814, walkthrough, the options
   class: UseDynamicQuantization, on by default, chooses scales that follow
   the moments through training].  Dynamic: the statistic of the new values,
   every step.  Static (our reading of the option switched off): the scale
   found the first time the block is quantized (stored scale still 0) is
   kept; later values at or beyond it saturate to the end of the alphabet. */
static float quantize_moment(const float *x, int64_t n, int32_t is_signed, const orc_hparams *h,
                             float stored, const uint16_t *draws, int32_t *codes)
{
    if (h->static_scales && stored >= ORC_TINY)
        return orc_quantize_with_stat(x, n, is_signed, stored, draws, codes);
    return orc_quantize_block(x, n, is_signed, h->use_pct, h->pct, draws, codes);
}

/* One element of the update; m_old/v_old/w_old are already dequantized.
   AMSGrad [RKK18, Algorithm 2, in PyTorch's convention: the running maximum
   w of the uncorrected second moment replaces v in the denominator, and the
   bias correction of v is applied to it]: w = max(w_old, v). */
static void adam_element(float p, float g, float m_old, float v_old, float w_old,
                         const orc_hparams *h, const float s[5], float *p_new, float *m_new,
                         float *v_new, float *w_new)
{
    const float step = s[0], ibc2 = s[1], decay = s[2], omb1 = s[3], omb2 = s[4];
    if (!h->decoupled)
        g = fmaf(h->wd, p, g); /* L2-coupled Adam: gradient += wd * p */
    const float m = fmaf(h->beta1, m_old, omb1 * g);
    const float gg = g * g;
    const float v = fmaf(h->beta2, v_old, omb2 * gg);
    const float w = h->amsgrad ? fmaxf(w_old, v) : v;
    const float denom = fmaf(sqrtf(w), ibc2, h->eps);  /* sqrt(v_hat) + eps */
    const float ratio = m / denom;                      /* m_hat/(...) * bc1 */
    *p_new = fmaf(-step, ratio, p * decay);
    *m_new = m;
    *v_new = v;
    *w_new = w;
}

static int64_t pad16(int64_t n) { return (n + 15) / 16 * 16; }

/* State of the elements a step works on: each pointer, if not NULL,
   points at the first element (scales: the first scale slot) of the range.
   w* hold the running maximum of the second moment (AMSGrad), stored like v:
   wf fp32 (F32 mode), wh bf16 (BF16 mode), wq + ws codes and scale (8-bit
   modes). */
typedef struct {
    int8_t *mq;
    uint8_t *vq, *wq;
    float *ms, *vs, *ws;
    uint16_t *mh, *vh, *wh;
    float *mf, *vf, *wf;
} orc_ptrs;

/* Per-block worker: n elements of one block whose first padded flat index
   is gidx; q points at the block's state.  m/v/w_new_out, if not NULL,
   receive the unquantized new moments. */
static void step_block(float *p, const float *g32, const uint16_t *g16, int64_t n,
                       int64_t gidx, int32_t storage, const orc_hparams *h,
                       const float s[5], const orc_ptrs *q,
                       float *m_new_out, float *v_new_out, float *w_new_out)
{
    float *m_new = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    float *v_new = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    float *w_new = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t j = 0; j < n; j++) {
        const float gj = g32 ? g32[j] : orc_f32_from_bf16(g16[j]);
        float m_old, v_old, w_old = 0.0f;
        switch (storage) {
        case ORC_F32:
            m_old = q->mf[j];
            v_old = q->vf[j];
            if (h->amsgrad)
                w_old = q->wf[j];
            break;
        case ORC_BF16:
            m_old = orc_f32_from_bf16(q->mh[j]);
            v_old = orc_f32_from_bf16(q->vh[j]);
            if (h->amsgrad)
                w_old = orc_f32_from_bf16(q->wh[j]);
            break;
        case ORC_Q8:
            m_old = orc_dequantize(q->mq[j], q->ms[0], 1);
            v_old = orc_dequantize(q->vq[j], q->vs[0], 0);
            if (h->amsgrad)
                w_old = orc_dequantize(q->wq[j], q->ws[0], 0);
            break;
        default: /* ORC_Q8_V_ONLY */
            m_old = q->mf[j];
            v_old = orc_dequantize(q->vq[j], q->vs[0], 0);
            if (h->amsgrad)
                w_old = orc_dequantize(q->wq[j], q->ws[0], 0);
            break;
        }
        adam_element(p[j], gj, m_old, v_old, w_old, h, s, &p[j], &m_new[j], &v_new[j],
                     &w_new[j]);
        if (m_new_out)
            m_new_out[j] = m_new[j];
        if (v_new_out)
            v_new_out[j] = v_new[j];
        if (w_new_out)
            w_new_out[j] = w_new[j];
    }

    if (storage == ORC_F32) {
        for (int64_t j = 0; j < n; j++) {
            q->mf[j] = m_new[j];
            q->vf[j] = v_new[j];
            if (h->amsgrad)
                q->wf[j] = w_new[j];
        }
    } else if (storage == ORC_BF16) {
        for (int64_t j = 0; j < n; j++) {
            q->mh[j] = orc_bf16_from_f32(m_new[j]);
            q->vh[j] = orc_bf16_from_f32(v_new[j]);
            if (h->amsgrad)
                q->wh[j] = orc_bf16_from_f32(w_new[j]);
        }
    } else {
        int32_t *codes = (int32_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int32_t));
        uint16_t *draws = NULL;
        if (h->stochastic)
            draws = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
        if (storage == ORC_Q8) {
            if (draws)
                orc_sr_draws(h->seed, h->t, gidx, n, 0, draws);
            q->ms[0] = quantize_moment(m_new, n, 1, h, q->ms[0], draws, codes);
            for (int64_t j = 0; j < n; j++)
                q->mq[j] = (int8_t)codes[j];
        } else {
            for (int64_t j = 0; j < n; j++)
                q->mf[j] = m_new[j];
        }
        if (draws)
            orc_sr_draws(h->seed, h->t, gidx, n, 1, draws);
        q->vs[0] = quantize_moment(v_new, n, 0, h, q->vs[0], draws, codes);
        for (int64_t j = 0; j < n; j++)
            q->vq[j] = (uint8_t)codes[j];
        if (h->amsgrad) {
            /* the running maximum: same alphabet, statistic and rounding as v,
               its own scale per block and its own draws */
            if (draws)
                orc_sr_draws(h->seed, h->t, gidx, n, 2, draws);
            q->ws[0] = quantize_moment(w_new, n, 0, h, q->ws[0], draws, codes);
            for (int64_t j = 0; j < n; j++)
                q->wq[j] = (uint8_t)codes[j];
        }
        free(codes);
        free(draws);
    }
    free(m_new);
    free(v_new);
    free(w_new);
}

/* q advanced to element i0 and scale slot blk (NULL entries stay NULL). */
static orc_ptrs advance(const orc_ptrs *q, int64_t i0, int64_t blk)
{
    orc_ptrs r;
    r.mq = q->mq ? q->mq + i0 : NULL;
    r.vq = q->vq ? q->vq + i0 : NULL;
    r.wq = q->wq ? q->wq + i0 : NULL;
    r.ms = q->ms ? q->ms + blk : NULL;
    r.vs = q->vs ? q->vs + blk : NULL;
    r.ws = q->ws ? q->ws + blk : NULL;
    r.mh = q->mh ? q->mh + i0 : NULL;
    r.vh = q->vh ? q->vh + i0 : NULL;
    r.wh = q->wh ? q->wh + i0 : NULL;
    r.mf = q->mf ? q->mf + i0 : NULL;
    r.vf = q->vf ? q->vf + i0 : NULL;
    r.wf = q->wf ? q->wf + i0 : NULL;
    return r;
}

/* The buffers a storage mode needs are all present. */
static int has_buffers(const orc_ptrs *q, int32_t storage, int32_t amsgrad)
{
    switch (storage) {
    case ORC_F32: return q->mf && q->vf && (!amsgrad || q->wf);
    case ORC_BF16: return q->mh && q->vh && (!amsgrad || q->wh);
    case ORC_Q8: return q->mq && q->vq && q->ms && q->vs && (!amsgrad || (q->wq && q->ws));
    case ORC_Q8_V_ONLY: return q->mf && q->vq && q->vs && (!amsgrad || (q->wq && q->ws));
    default: return 0;
    }
}

/*
 * Multi-tensor step.  Layout [P814 key features: block-wise, block size
 * default 2048]: tensor k's state occupies a segment of pad16(numel_k)
 * entries starting at the sum of the earlier segments; its blocks cover
 * local [b*block, min(numel, (b+1)*block)), numbered tensor-major.
 * grads[k] points at fp32 (grad_bf16 == 0) or bf16 bit patterns.
 * m/v/w_new_out, if not NULL, receive the unquantized new moments (flat,
 * padded).  Returns 0, or -1 on an argument the step does not define.
 */
int orc_adam_step(int32_t n_tensors, const int64_t *numels, int32_t block,
                  int32_t storage, int32_t grad_bf16, float *const *params,
                  const void *const *grads, const orc_ptrs *state, float lr, float beta1,
                  float beta2, float eps, float wd, float pct, int64_t t, int32_t decoupled,
                  int32_t stochastic, int32_t use_pct, int32_t static_scales, int32_t amsgrad,
                  uint64_t seed, float *m_new_out, float *v_new_out, float *w_new_out)
{
    if (n_tensors < 0 || block <= 0 || t < 1 || storage < ORC_F32 || storage > ORC_Q8_V_ONLY)
        return -1;
    if (!(pct >= 0.0f && pct <= 100.0f) || !state || !has_buffers(state, storage, amsgrad))
        return -1;
    const orc_hparams h = {lr, beta1, beta2, eps, wd, pct, t, decoupled, stochastic, use_pct,
                           static_scales, amsgrad, seed};
    float s[5];
    orc_host_scalars(lr, beta1, beta2, wd, t, decoupled, s);

    int64_t seg = 0, blk = 0;
    for (int32_t k = 0; k < n_tensors; k++) {
        const int64_t n = numels[k];
        if (n < 0)
            return -1;
        for (int64_t b0 = 0; b0 < n; b0 += block) {
            const int64_t nb = (n - b0 < block) ? (n - b0) : block;
            const float *g32 = grad_bf16 ? NULL : (const float *)grads[k] + b0;
            const uint16_t *g16 = grad_bf16 ? (const uint16_t *)grads[k] + b0 : NULL;
            const int64_t i0 = seg + b0;
            const orc_ptrs q = advance(state, i0, blk);
            step_block(params[k] + b0, g32, g16, nb, i0, storage, &h, s, &q,
                       m_new_out ? m_new_out + i0 : NULL, v_new_out ? v_new_out + i0 : NULL,
                       w_new_out ? w_new_out + i0 : NULL);
            blk++;
        }
        seg += pad16(n);
    }
    return 0;
}

/*
 * Blocks one at a time, for full-size workloads checked on a sample of
 * blocks (blocks are independent of one another).  Block i has n[i]
 * elements, first padded flat index gidx[i]; p[i]/g[i] point at its params
 * and grads; its state lives at offset off[i] of the given arrays (one
 * scale slot per block, slot i).  Same arithmetic as orc_adam_step.
 */
int orc_adam_step_blocks(int64_t n_blocks, const int64_t *n, const int64_t *gidx,
                         const int64_t *off, int32_t storage, int32_t grad_bf16,
                         float *const *p, const void *const *g, const orc_ptrs *state,
                         float lr, float beta1, float beta2, float eps, float wd, float pct,
                         int64_t t, int32_t decoupled, int32_t stochastic, int32_t use_pct,
                         int32_t static_scales, int32_t amsgrad, uint64_t seed)
{
    if (n_blocks < 0 || t < 1 || storage < ORC_F32 || storage > ORC_Q8_V_ONLY)
        return -1;
    if (!(pct >= 0.0f && pct <= 100.0f) || !state || !has_buffers(state, storage, amsgrad))
        return -1;
    const orc_hparams h = {lr, beta1, beta2, eps, wd, pct, t, decoupled, stochastic, use_pct,
                           static_scales, amsgrad, seed};
    float s[5];
    orc_host_scalars(lr, beta1, beta2, wd, t, decoupled, s);
    for (int64_t i = 0; i < n_blocks; i++) {
        const orc_ptrs q = advance(state, off[i], i);
        step_block(p[i], grad_bf16 ? NULL : (const float *)g[i],
                   grad_bf16 ? (const uint16_t *)g[i] : NULL, n[i], gidx[i], storage,
                   &h, s, &q, NULL, NULL, NULL);
    }
    return 0;
}

void orc_f32_from_bf16_array(const uint16_t *h, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_f32_from_bf16(h[i]);
}
