/*
 * CPU oracle for the ZeRO-DP partitioned optimizer step (one rank's shard).
 *
 * TEST INFRASTRUCTURE. This file is the slow, obviously-correct reference the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header, table or
 * helper with the HIP library, and the library never calls it.
 *
 * Build: gcc -O2 -fno-tree-vectorize -ffp-contract=off -shared -fPIC
 *        (scalar loops, every float operation rounded on its own, no FMA).
 *
 * Sources (web pages on ZeRO, cited by title and section):
 *   [DS12]  "DeepSpeed ZeRO stage 1/2" walkthrough, chapter "01 · ZeRO 的显存数学与
 *           Stage 1/2": §3 flatten / partition / own-one-segment, §4 ② the
 *           base + remainder split, §6 the six actions of step().
 *   [NOTES] "ZeRO: Memory Optimizations Toward Training Trillion Parameter
 *           Models" reading notes, second part §3 (per-coordinate Adam update)
 *           and §4 (all-reduce = reduce-scatter then all-gather; the averaged
 *           shard formula).
 *   [ZERO-ZH] Chinese translation of the ZeRO paper, §3.1 (mixed-precision
 *           Adam: fp16 params/grads, fp32 master, momentum, variance).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - remainder elements go one each to the first (numel mod N_d) ranks;
 *   - the average accumulates in fp32, in replica order, then divides by N_d;
 *   - overflow = any non-finite value in the fp32 average, before unscaling;
 *   - bias correction m/(1-b1^t), v/(1-b2^t) with t = applied steps from 1,
 *     eps added after the square root;
 *   - AdamW = decoupled decay theta*(1 - lr*wd) before the Adam update;
 *   - every elementwise op in fp32 round-to-nearest-even, scalars formed in
 *     fp64 and rounded once, b^t by successive fp64 multiplication;
 *   - skip on overflow leaves master, m, v and params untouched and t unchanged,
 *     and halves the loss scale (floor min_scale).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-3)

#define OR_F16 1
#define OR_BF16 2

/* ------------------------------------------------------------------------- */
/* 16-bit floating-point encodings, written from the IEEE 754 definitions.    */
/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.                   */
/* bfloat16: the upper 16 bits of binary32 (1 sign, 8 exponent, 7 fraction).   */
/* ------------------------------------------------------------------------- */

float oracle_f16_decode(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    float mag;
    if (e == 0)
        mag = ldexpf((float)frac, -24); /* subnormal: frac * 2^-24 */
    else if (e == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexpf((float)(frac + 1024), e - 25); /* 1.frac * 2^(e-15) */
    return sign ? -mag : mag;
}

float oracle_bf16_decode(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* Round |x| to a multiple of 2^q, ties to even, exactly (|x| has <= 24
 * significant bits, so the scaled value and its rounding are exact in fp64). */
static double round_to_quantum(double ax, int q)
{
    double s = ldexp(ax, -q);
    double fl = floor(s);
    double frac = s - fl;
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    return ldexp(r, q);
}

uint16_t oracle_f16_encode(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7e00; /* canonical quiet NaN */
    double ax = fabs((double)x);
    if (isinf(ax))
        return sign | 0x7c00;
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);      /* ax = f * 2^e, f in [0.5, 1) */
    int q = e - 11;     /* 11 significant bits */
    if (q < -24)
        q = -24;        /* subnormal spacing */
    double v = round_to_quantum(ax, q);
    if (v >= 65536.0)   /* beyond the largest finite value after rounding */
        return sign | 0x7c00;
    if (v < ldexp(1.0, -14))
        return sign | (uint16_t)ldexp(v, 24); /* subnormal (or zero) */
    int ev;
    double f = frexp(v, &ev);                 /* v = f * 2^ev */
    int field = ev - 1 + 15;
    uint16_t frac = (uint16_t)(ldexp(f, 11) - 1024.0);
    return sign | (uint16_t)(field << 10) | frac;
}

uint16_t oracle_bf16_encode(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7fc0;
    double ax = fabs((double)x);
    if (isinf(ax))
        return sign | 0x7f80;
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);
    int q = e - 8;      /* 8 significant bits */
    if (q < -133)
        q = -133;       /* bf16 subnormal spacing */
    double v = round_to_quantum(ax, q);
    if (v >= ldexp(1.0, 128))
        return sign | 0x7f80;
    float fv = (float)v; /* exact: v has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &fv, sizeof bits);
    return sign | (uint16_t)(bits >> 16);
}

static float decode16(int dt, uint16_t h)
{
    return dt == OR_BF16 ? oracle_bf16_decode(h) : oracle_f16_decode(h);
}

void oracle_decode16(const uint16_t *bits, int64_t n, int32_t dt, float *out)
{
    for (int64_t j = 0; j < n; ++j)
        out[j] = decode16(dt, bits[j]);
}

static uint16_t encode16(int dt, float x)
{
    return dt == OR_BF16 ? oracle_bf16_encode(x) : oracle_f16_encode(x);
}

/* ------------------------------------------------------------------------- */
/* Partition [DS12 §4 ②]: base = numel / N_d, rem = numel % N_d; the first    */
/* rem ranks get one element more. Optional padding of the flat length to a   */
/* multiple of align_elems [DS12 §4 ① and §7, alignment padding].           */
/* ------------------------------------------------------------------------- */

int oracle_partition(int64_t numel, int32_t n_d, int64_t align_elems,
                     int64_t *offsets, int64_t *sizes, int64_t *padded_out)
{
    if (numel < 0 || n_d < 1 || align_elems < 1 || !offsets || !sizes)
        return OR_EINVAL;
    int64_t padded = numel;
    if (align_elems > 1) {
        int64_t r = numel % align_elems;
        if (r != 0) {
            if (numel > INT64_MAX - (align_elems - r))
                return OR_EINVAL;
            padded = numel + (align_elems - r);
        }
    }
    int64_t base = padded / n_d;
    int64_t rem = padded % n_d;
    int64_t off = 0;
    for (int32_t r = 0; r < n_d; ++r) {
        int64_t size = base + (r < rem ? 1 : 0);
        offsets[r] = off;
        sizes[r] = size;
        off += size;
    }
    if (padded_out)
        *padded_out = padded;
    return OR_OK;
}

/* Which pieces of which tensors fall inside rank `rank`'s segment: the flat
 * vector is the tensors laid end to end in order [DS12 §3 ①], and a tensor may
 * straddle two segments [DS12 §4 ④, §7]. For each overlap the oracle reports
 * the tensor index, the position inside the shard, the position inside the
 * tensor and the length. Returns the number of slices, or a negative error. */
int oracle_tensor_slices(const int64_t *numels, int32_t n_tensors, int32_t n_d,
                         int32_t rank, int64_t align_elems, int32_t cap,
                         int32_t *tensor, int64_t *shard_begin,
                         int64_t *tensor_begin, int64_t *length)
{
    if (!numels || n_tensors < 0 || n_d < 1 || rank < 0 || rank >= n_d)
        return OR_EINVAL;
    int64_t total = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (numels[i] < 0)
            return OR_EINVAL;
        total += numels[i];
    }
    int64_t *offs = malloc(sizeof(int64_t) * (size_t)n_d);
    int64_t *sizes = malloc(sizeof(int64_t) * (size_t)n_d);
    if (!offs || !sizes) {
        free(offs);
        free(sizes);
        return OR_ENOMEM;
    }
    int rc = oracle_partition(total, n_d, align_elems, offs, sizes, NULL);
    int64_t lo = offs[rank], hi = offs[rank] + sizes[rank];
    free(offs);
    free(sizes);
    if (rc)
        return rc;
    int32_t count = 0;
    int64_t start = 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        int64_t b = start, e = start + numels[i];
        start = e;
        int64_t ob = b > lo ? b : lo;
        int64_t oe = e < hi ? e : hi;
        if (ob >= oe)
            continue;
        if (count >= cap)
            return OR_EINVAL;
        tensor[count] = i;
        shard_begin[count] = ob - lo;
        tensor_begin[count] = ob - b;
        length[count] = oe - ob;
        ++count;
    }
    return count;
}

/* ------------------------------------------------------------------------- */
/* Average of this rank's segment over the N_d gradient copies:               */
/*   avg^(k) = (1/N_d) * sum_r g_r^(k)    [NOTES §4]                           */
/* accumulated in fp32 in replica order, then divided by N_d.                  */
/* ------------------------------------------------------------------------- */

void oracle_average(const uint16_t *const *replicas, int32_t n_d, int32_t grad_dt,
                    int64_t n, float *out)
{
    float nd = (float)n_d;
    for (int64_t j = 0; j < n; ++j) {
        float acc = 0.0f;
        for (int32_t r = 0; r < n_d; ++r)
            acc = acc + decode16(grad_dt, replicas[r][j]);
        out[j] = acc / nd;
    }
}

/* Overflow scan and squared L2 norm of the unscaled gradient [DS12 §6 steps
 * 1-3]: flag = any non-finite a[j]; norm2 += g*g in fp64, in index order, with
 * g = a[j] * inv_scale rounded to fp32. Accumulates into *norm2 and *flag so a
 * long vector can be fed in order, chunk after chunk. */
void oracle_norm_overflow(const float *a, int64_t n, float inv_scale,
                          double *norm2, int32_t *flag)
{
    double acc = *norm2;
    int32_t f = *flag;
    for (int64_t j = 0; j < n; ++j) {
        if (!isfinite(a[j]))
            f = 1;
        float g = a[j] * inv_scale;
        acc += (double)g * (double)g;
    }
    *norm2 = acc;
    *flag = f;
}

/* b^t by t successive fp64 multiplications. */
static double beta_pow(double beta, int64_t t)
{
    double p = 1.0;
    for (int64_t i = 0; i < t; ++i)
        p = p * beta;
    return p;
}

/* One Adam/AdamW update of n coordinates for applied step t (t >= 1), on the
 * rank's fp32 master/m/v shard, followed by the fp32 -> 16-bit copy into the
 * rank's slice of the flat parameter vector [NOTES §3 update equations;
 * DS12 §6 steps 3-5; ZERO-ZH §3.1 for the fp32 state]. `param` points at the
 * first element of the rank's slice (NULL: no writeback). `clip` multiplies
 * the unscaled gradient (DS12 §6 step 3 unscales and clips; 1 = no clip). */
void oracle_adam_update(int64_t n, const float *a, float inv_scale, float clip,
                        float *master, float *m, float *v,
                        uint16_t *param, int32_t param_dt, int64_t t,
                        double lr, double beta1, double beta2, double eps,
                        double weight_decay)
{
    const float b1 = (float)(1.0 - beta_pow(beta1, t)); /* 1 - beta1^t */
    const float b2 = (float)(1.0 - beta_pow(beta2, t)); /* 1 - beta2^t */
    const float c1 = (float)(1.0 - beta1);
    const float c2 = (float)(1.0 - beta2);
    const float decay = (float)(1.0 - lr * weight_decay);
    const float beta1f = (float)beta1, beta2f = (float)beta2;
    const float epsf = (float)eps, lrf = (float)lr;
    for (int64_t j = 0; j < n; ++j) {
        float g = a[j] * inv_scale;              /* unscale */
        g = g * clip;                            /* clip (1 = none) */
        float theta = master[j];
        if (weight_decay != 0.0)
            theta = theta * decay;               /* decoupled decay */
        float mt = beta1f * m[j] + c1 * g;       /* first moment */
        float vt = beta2f * v[j] + c2 * (g * g); /* second moment */
        float mhat = mt / b1;
        float vhat = vt / b2;
        float denom = sqrtf(vhat) + epsf;
        float upd = mhat / denom;
        float next = theta - lrf * upd;
        master[j] = next;
        m[j] = mt;
        v[j] = vt;
        if (param)
            param[j] = encode16(param_dt, next);
    }
}

/* fp32 master -> 16-bit parameter slice [DS12 §6 step 5]. */
void oracle_cast(const float *master, int64_t n, uint16_t *param, int32_t param_dt)
{
    for (int64_t j = 0; j < n; ++j)
        param[j] = encode16(param_dt, master[j]);
}

/* ------------------------------------------------------------------------- */
/* The whole step over a list of parameter groups, in the order of [DS12 §6]:  */
/* overflow check (skip + lower the loss scale on overflow), global norm,      */
/* unscale, Adam on the shard, write back. The all-gather that follows is      */
/* another rank's business and is not part of a one-rank step.                 */
/* ------------------------------------------------------------------------- */

typedef struct {
    int64_t n;                        /* shard length S */
    int32_t n_d;                      /* gradient copies to average */
    int32_t grad_dt;                  /* OR_F16 / OR_BF16 */
    const uint16_t *const *replicas;  /* n_d host arrays of n elements */
    float *master, *m, *v;            /* fp32 [n], updated in place */
    uint16_t *param;                  /* rank's slice of the flat vector, or NULL */
    int32_t param_dt;
    int32_t pad_;
    double lr, beta1, beta2, eps, weight_decay;
} oracle_group;

typedef struct {
    int32_t skip_on_overflow;  /* 1: dynamic loss scale with skip; 0: static scale */
    int32_t growth_interval;   /* applied steps between doublings (0 = never)     */
    double backoff;            /* scale factor on overflow, e.g. 0.5               */
    double growth;             /* scale factor after growth_interval good steps    */
    double min_scale;          /* floor of the scale                               */
    double max_grad_norm;      /* clip the gradient to this global norm (0 = off)  */
} oracle_policy;

typedef struct {
    int64_t step;        /* applied steps t */
    double norm2;        /* last sum of squares of the unscaled gradient */
    float loss_scale;    /* S_l */
    int32_t overflow;    /* last flag */
    int32_t skipped;     /* last call skipped */
    int32_t good_steps;  /* consecutive applied steps since the last scale change */
    float clip;          /* last clip multiplier (1 = none) */
    int32_t pad_;
} oracle_state;

/* Clip multiplier for a global norm: min(1, max_norm / (norm + 1e-6)) in
 * fp64, rounded once to fp32; 1 when clipping is off or the norm is not
 * finite. The pages name clipping (DS12 §6 step 3) without its formula; this
 * is the usual global-norm rule with torch's 1e-6 guard. */
static float clip_multiplier(double norm2, double max_norm)
{
    if (!(max_norm > 0.0) || !isfinite(norm2))
        return 1.0f;
    double c = max_norm / (sqrt(norm2) + 1e-6);
    return (float)(c < 1.0 ? c : 1.0);
}

/* The verdict and the update of DS12 §6, given the groups' averaged
 * gradients avg[g] (as oracle_average computes them), the overflow flag and
 * the squared norm of the unscaled gradient: record norm and flag, the clip
 * multiplier; on overflow with skip, back the scale off and change nothing
 * else; otherwise Adam on every group with the unscale multiplier 1/S of the
 * scale in force, t + 1, and the growth bookkeeping. */
static void apply_verdict(const oracle_group *groups, int32_t n_groups, float *const *avg,
                          const oracle_policy *policy, oracle_state *st,
                          double norm2, int32_t flag)
{
    const float inv_scale = (float)(1.0 / (double)st->loss_scale);
    st->norm2 = norm2;
    st->overflow = flag;
    st->clip = clip_multiplier(norm2, policy->max_grad_norm);
    if (flag && policy->skip_on_overflow) {
        double s = (double)st->loss_scale * policy->backoff;
        if (s < policy->min_scale)
            s = policy->min_scale;
        st->loss_scale = (float)s;
        st->good_steps = 0;
        st->skipped = 1;
        return;
    }
    int64_t t = st->step + 1;
    for (int32_t g = 0; g < n_groups; ++g) {
        const oracle_group *G = &groups[g];
        oracle_adam_update(G->n, avg[g], inv_scale, st->clip, G->master, G->m, G->v,
                           G->param, G->param_dt, t, G->lr, G->beta1,
                           G->beta2, G->eps, G->weight_decay);
    }
    st->step = t;
    st->skipped = 0;
    if (policy->skip_on_overflow) {
        st->good_steps += 1;
        if (policy->growth_interval > 0 &&
            st->good_steps == policy->growth_interval) {
            st->loss_scale = (float)((double)st->loss_scale * policy->growth);
            st->good_steps = 0;
        }
    }
}

/* The step of DS12 §6 over `groups`. The overflow flag and the norm come from
 * these groups' averaged gradients, or, when `given` is set, are the caller's
 * (given_norm2, given_flag): the flag and norm² of a whole shard of which the
 * groups hold a sample of coordinates. Everything else is the same. */
static int step_core(const oracle_group *groups, int32_t n_groups,
                     const oracle_policy *policy, oracle_state *st,
                     int given, double given_norm2, int32_t given_flag)
{
    if (!groups || n_groups < 1 || !policy || !st)
        return OR_EINVAL;
    float **avg = calloc((size_t)n_groups, sizeof(float *));
    if (!avg)
        return OR_ENOMEM;
    int rc = OR_OK;
    const float inv_scale = (float)(1.0 / (double)st->loss_scale);
    double norm2 = 0.0;
    int32_t flag = 0;
    for (int32_t g = 0; g < n_groups && rc == OR_OK; ++g) {
        avg[g] = malloc(sizeof(float) * (size_t)(groups[g].n > 0 ? groups[g].n : 1));
        if (!avg[g]) {
            rc = OR_ENOMEM;
            break;
        }
        oracle_average(groups[g].replicas, groups[g].n_d, groups[g].grad_dt,
                       groups[g].n, avg[g]);
        oracle_norm_overflow(avg[g], groups[g].n, inv_scale, &norm2, &flag);
    }
    if (rc == OR_OK) {
        if (given) {
            norm2 = given_norm2;
            flag = given_flag;
        }
        apply_verdict(groups, n_groups, avg, policy, st, norm2, flag);
    }
    for (int32_t g = 0; g < n_groups; ++g)
        free(avg[g]);
    free(avg);
    return rc;
}

int oracle_step(const oracle_group *groups, int32_t n_groups,
                const oracle_policy *policy, oracle_state *st)
{
    return step_core(groups, n_groups, policy, st, 0, 0.0, 0);
}

int oracle_step_given_norm(const oracle_group *groups, int32_t n_groups,
                           const oracle_policy *policy, oracle_state *st,
                           double norm2, int32_t flag)
{
    return step_core(groups, n_groups, policy, st, 1, norm2, flag != 0);
}

/* The step from averaged gradients: avg[g] holds group g's average (the
 * output of oracle_average on its copies; the groups' replica fields are not
 * read), norm2 and flag the squared norm and overflow flag of the whole shard
 * (oracle_norm_overflow over every group, in order, or over a shard of which
 * the groups hold a part). Lets a caller average a large shard once, chunk by
 * chunk, and then step each chunk. */
int oracle_step_from_average(const oracle_group *groups, int32_t n_groups,
                             float *const *avg, const oracle_policy *policy,
                             oracle_state *st, double norm2, int32_t flag)
{
    if (!groups || n_groups < 1 || !avg || !policy || !st)
        return OR_EINVAL;
    for (int32_t g = 0; g < n_groups; ++g)
        if (!avg[g] && groups[g].n > 0)
            return OR_EINVAL;
    apply_verdict(groups, n_groups, avg, policy, st, norm2, flag != 0);
    return OR_OK;
}
