/*
 * CPU oracle: the arithmetic of one DP rank's sharded Adam step.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and bench.py's CPU
 * baseline may load this library. It shares no code with the HIP path.
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math), so every float
 * operation below is one IEEE-754 binary32 operation rounded to nearest-even,
 * subnormals kept, in exactly the order written.
 *
 * What it computes, per owned element (page "04 · 分布式优化器"):
 *   - §5: the gradient scaling factor is applied to the grad buffer in place,
 *     before the collective. Reading: the in-place multiply of a bf16 buffer
 *     rounds its fp32 product back to bf16.
 *   - §4.2: the reduce-scatter leaves the rank the sum of the D ranks'
 *     contributions over its range, in the bf16 grad buffer. Reading: summed
 *     in fp32 in fixed rank order 0..D-1 starting from rank 0's term, rounded
 *     to bf16 once.
 *   - §4.3: that bf16 slice is copied into the fp32 main grad of the shard,
 *     Adam runs on the fp32 master/m/v shard only, and the updated master is
 *     written back (as bf16) into the parameter buffer's owned range.
 * The page names Adam but not its arithmetic. Reading: Adam with bias
 * correction (Kingma & Ba, "Adam: A Method for Stochastic Optimization",
 * Algorithm 1) with weight decay decoupled from the gradient and scaled by
 * the learning rate (Loshchilov & Hutter, "Decoupled Weight Decay
 * Regularization"), evaluated in this fixed fp32 order:
 *   m' = b1*m + (1-b1)*g            v' = b2*v + (1-b2)*(g*g)
 *   u  = (m'/bc1) / (sqrt(v'/bc2) + eps)
 *   p' = p - lr*(u + wd*p)
 * with 1-b1 and 1-b2 formed in fp32 and bc_i = 1 - b_i^t formed in double
 * by t repeated products and rounded once to fp32.
 *
 * Global-norm clipping (the distributed-training notes, §8.3: the squared
 * sums of every rank's gradient shard are summed across ranks, the square
 * root is the global norm, and clipping happens before the update).
 * Reading: the norm is over the reduced bf16 gradient g of the owned
 * parameter elements, squares summed in fp64; the clipping coefficient is
 * min(1, max_norm / (norm + 1e-6)) in fp64, rounded to fp32 (the convention
 * of PyTorch's clip_grad_norm_), and multiplies the fp32 main grad before
 * Adam; a norm that is not finite means a skipped step (found-inf).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 <-> fp32 ------------------------------------------------------ */

/* A bf16 value is the top half of the binary32 with the same sign, exponent
 * and leading 7 mantissa bits, so widening is exact. */
static float widen(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* The bf16 nearest to x, ties to the even neighbour. Finite values beyond
 * the largest bf16 round to +-Inf; subnormals are kept; a NaN stays a NaN
 * (quiet bit set, sign kept). */
static uint16_t narrow(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    /* The two bf16 neighbours of x are `toward` (the top 16 bits: x with its
     * low mantissa bits dropped, i.e. rounded toward zero) and the next bf16
     * away from zero, toward + 1 (the carry walks into the exponent, which
     * also gives the right answer at a binade edge and at the largest
     * finite value, where the next pattern is Inf). The dropped 16 bits
     * say where x sits between them; 0x8000 is the exact midpoint. */
    uint16_t toward = (uint16_t)(u >> 16);
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (toward & 1u)))
        toward = (uint16_t)(toward + 1u);
    return toward;
}

/* ---- one element --------------------------------------------------------- */

typedef struct {
    float lr, beta1, beta2, eps, weight_decay, bc1, bc2;
} oracle_hp;

/* The scaled, reduced gradient of one element, as the bf16 the reduce-scatter
 * leaves in the grad buffer. */
static uint16_t reduce_one(int32_t n_rep, const uint16_t *const *rep, int64_t i, float scale)
{
    float acc = widen(narrow(widen(rep[0][i]) * scale));
    for (int32_t j = 1; j < n_rep; ++j) {
        float term = widen(narrow(widen(rep[j][i]) * scale));
        acc = acc + term;
    }
    return narrow(acc);
}

/* One Adam update of one fp32 element, in the order stated at the top. */
static void adam_one(const oracle_hp *hp, float g, float *p, float *m, float *v)
{
    const float omb1 = 1.0f - hp->beta1;
    const float omb2 = 1.0f - hp->beta2;

    float m1 = hp->beta1 * *m;
    float m2 = omb1 * g;
    float mn = m1 + m2;

    float gg = g * g;
    float v1 = hp->beta2 * *v;
    float v2 = omb2 * gg;
    float vn = v1 + v2;

    float mh = mn / hp->bc1;
    float vh = vn / hp->bc2;
    float den = sqrtf(vh) + hp->eps;
    float u = mh / den;

    float wdp = hp->weight_decay * *p;
    float u2 = u + wdp;
    float st = hp->lr * u2;
    float pn = *p - st;

    *m = mn;
    *v = vn;
    *p = pn;
}

/* ---- exported ------------------------------------------------------------- */

/* 1 - beta^t: the double 1.0 multiplied t times by (double)beta, rounded once. */
float oracle_bias_correction(float beta, int64_t t)
{
    double pw = 1.0;
    for (int64_t i = 0; i < t; ++i)
        pw *= (double)beta;
    return (float)(1.0 - pw);
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the element loops that follow (n >= 1); each element is
 * independent, so results do not depend on it. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

void oracle_narrow(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = narrow(x[i]);
}

void oracle_widen(const uint16_t *h, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = widen(h[i]);
}

/* out[i] = bf16( sum_j bf16(rep[j][i] * scale) ), j = 0..n_rep-1 in order. */
void oracle_reduce(int32_t n_rep, const uint16_t *const *rep, float scale, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = reduce_one(n_rep, rep, i, scale);
}

/* Adam on n fp32 elements whose gradient is the bf16 `grad`; writes bf16(p')
 * to param_out when it is not NULL. hp = {lr, b1, b2, eps, wd, bc1, bc2}. */
void oracle_adam(int64_t n, const uint16_t *grad, float *master, float *m, float *v,
                 uint16_t *param_out, const float *hp_in)
{
    oracle_hp hp = {hp_in[0], hp_in[1], hp_in[2], hp_in[3], hp_in[4], hp_in[5], hp_in[6]};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        adam_one(&hp, widen(grad[i]), &master[i], &m[i], &v[i]);
        if (param_out)
            param_out[i] = narrow(master[i]);
    }
}

/* Sum over i of g_i^2 in double, i = 0..n-1 in order, where g is the reduced
 * gradient of reduce_one. Sequential, so the order is the element order. */
double oracle_norm_sq(int32_t n_rep, const uint16_t *const *rep, float scale, int64_t n)
{
    double total = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double g = (double)widen(reduce_one(n_rep, rep, i, scale));
        total = total + g * g;
    }
    return total;
}

/* Clipping coefficient from the ranks' squared norms, summed in index order.
 * A NaN result means: skip the step (the norm is not finite). */
float oracle_clip_coefficient(const double *parts, int32_t n, float max_norm, double *norm_out)
{
    double total = 0.0;
    for (int32_t i = 0; i < n; ++i)
        total = total + parts[i];
    double norm = sqrt(total);
    if (norm_out)
        *norm_out = norm;
    if (!isfinite(norm))
        return NAN;
    double c = (double)max_norm / (norm + 1e-6);
    return (float)(c < 1.0 ? c : 1.0);
}

/* The whole step for n contiguous owned elements: reduce the n_rep
 * contributions, copy into the fp32 main grad and multiply it by grad_coeff
 * (1 without clipping; the product is also stored to main_grad_out when not
 * NULL), Adam, bf16 write-back to param_out when not NULL. */
void oracle_step(int32_t n_rep, const uint16_t *const *rep, float scale, int64_t n,
                 float *master, float *m, float *v, uint16_t *param_out,
                 float *main_grad_out, const float *hp_in, float grad_coeff)
{
    oracle_hp hp = {hp_in[0], hp_in[1], hp_in[2], hp_in[3], hp_in[4], hp_in[5], hp_in[6]};
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float g = widen(reduce_one(n_rep, rep, i, scale)) * grad_coeff;
        if (main_grad_out)
            main_grad_out[i] = g;
        adam_one(&hp, g, &master[i], &m[i], &v[i]);
        if (param_out)
            param_out[i] = narrow(master[i]);
    }
}
