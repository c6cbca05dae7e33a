/*
 * csa_oracle.c -- plain, slow, obviously-correct CPU oracle for the CSA/HCA
 * Compressor (THD-packed gated-softmax pooling), forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library; the two agree because each follows the same statement of the
 * method.
 *
 * Sources (web pages; the part cited follows the colon):
 *   [PR5984]  NVIDIA/Megatron-LM pull request 5984 page, which carries the
 *             squashed commit log of cudnn-frontend PR #427.
 *   [PR710]   cudnn-frontend pull request 710 page (ratio=2 envelope).
 *
 * What is computed ([PR5984: fused forward+backward commit] lists the fused
 * steps: collect the window rows, add the positional bias to the score, form
 * the overlapping window, softmax in fp32, weight kv by it and sum, round the
 * sum to bf16; [PR5984: coff in {1,2} commit] gives the coff=1 window;
 * [PR5984: zero-init folding commit] gives the backward's store contract and
 * the never-consumed slot classes):
 *
 *   Segments s = 0..S-1 are rows [cu[s], cu[s+1]) of kv/score ([T_cap, W],
 *   W = coff*d, bf16).  Segment s has nb_s = floor(L_s / r) output blocks;
 *   output row n = off_s + b, off = exclusive prefix sum of nb.
 *   Window of block (s, b) for output column j in [0, d), in this order:
 *     coff == 2 and b >= 1: rows cu[s]+(b-1)r+i, column j,       position i
 *                           (previous block, first-half columns)
 *     always:               rows cu[s]+b*r+i,   column (coff-1)d+j, position i
 *                           (own block; second half when coff == 2)
 *   For b == 0 at coff == 2 the previous half does not exist and is excluded.
 *   x_k = score + ape[position, column], p = softmax(x) over the window,
 *   out[n, j] = bf16(sum_k p_k kv_k).
 *   Backward with g = dOut[n, j]:  dKV = p g,  dScore = p g (kv - out_fp),
 *   dAPE[position, column] += p g (kv - out_fp).  Every slot of dKV/dScore
 *   that lies in no window is +0.0.
 *
 * Two oracles live here:
 *   *_f64 : the plain definition in double precision (exp, division).
 *   *_f32 : the same quantities under a fixed fp32 evaluation order (the
 *           pages require fp32 softmax intermediates but do not fix an order;
 *           this file fixes one so that results are reproducible bit for bit):
 *             x_k = f32(score_k) + ape_k                   (one fp32 add)
 *             m   = max_k x_k
 *             e_k = EXP(x_k - m)                           (EXP below)
 *             Z   = ((e_0 + e_1) + e_2) + ...              (window order)
 *             R   = 1 / Z                                  (correctly rounded)
 *             acc = fma(e_{K-1}, v_{K-1}, ... fma(e_0, v_0, 0))
 *           Every window, of any length (ratio 128 gives 128 or 256
 *           entries), is summed this way in one chain: the pages fix fp32
 *           intermediates but no chunking, so the plain single-chain order is
 *           the reference.  A kernel that sums in chunks and merges the
 *           chunk sums ([PR5984: ratio=128 commit]) is compared with it
 *           within the rounding such a reordering can cause, not bit for bit.
 *             o   = acc * R,  out = bf16_rne(o)
 *             G   = R * f32(dOut),  a_k = e_k * G
 *             dKV_k = bf16_rne(a_k),  ds_k = a_k * (v_k - o),
 *             dScore_k = bf16_rne(ds_k)
 *             dAPE = sum of the fp32 ds_k, accumulated here in double.
 *   EXP(y) (for the y <= 0 the softmax produces):
 *             y  = max(y, -104)      (below this e^y is under half the
 *                                      smallest fp32 subnormal)
 *             k  = rint(y * L2E)
 *             r  = fma(-k, LN2_LO, fma(-k, LN2_HI, y))     (Cody-Waite)
 *             q  = Taylor polynomial of e^r, degree 7, Horner with fma,
 *                  coefficients fp32(1/n!)
 *             EXP = ldexp(q, k)
 *   Built with -ffp-contract=off: every fma above is explicit, nothing else
 *   is fused.  IEEE subnormals are kept (no flush to zero).
 *
 * Pins (tests/test_oracle_pins.py): EXP against the exact exponential over
 * its domain; the constants against their exact rational definitions; bf16
 * rounding against the round-to-nearest-even definition; a one-hot window
 * reproduces kv bit for bit; a uniform window reproduces the arithmetic mean;
 * a brute-force double evaluation with an independently written window
 * membership test; central finite differences and PyTorch double autograd for
 * the backward; the zero set of dKV equals the never-consumed slot set;
 * sum_k ds_k = 0 per window; f32 vs f64 agreement within bf16 rounding.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_NO_MEMORY (-2)

/* ---------------------------------------------------------------------- */
/* bf16 <-> fp32                                                           */
/* ---------------------------------------------------------------------- */

/* A bf16 value is the upper half of an fp32 bit pattern. */
float oracle_f32_from_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round-to-nearest, ties-to-even, on the bit pattern (finite inputs).  The
 * pages fix bf16 outputs but not the rounding; nearest-even is the IEEE
 * default and the plainest reading. */
uint16_t oracle_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------------- */
/* EXP: the fixed fp32 exponential used by the *_f32 oracle                */
/* ---------------------------------------------------------------------- */

static const float L2E = 0x1.715476p+0f;     /* fp32 nearest to log2(e)        */
static const float LN2_HI = 0x1.62e430p-1f;  /* fp32 nearest to ln(2)          */
static const float LN2_LO = -0x1.05c610p-29f;/* fp32 nearest to ln(2) - LN2_HI */
static const float EXP_C[8] = {              /* fp32 nearest to 1/n!, n=0..7   */
    0x1.000000p+0f, 0x1.000000p+0f, 0x1.000000p-1f, 0x1.555556p-3f,
    0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f};
static const float EXP_Y_MIN = -104.0f;

float oracle_exp_f32(float y)
{
    if (y < EXP_Y_MIN) y = EXP_Y_MIN;
    float t = y * L2E;
    float k = rintf(t);
    float r = fmaf(-k, LN2_HI, y);
    r = fmaf(-k, LN2_LO, r);
    float q = EXP_C[7];
    for (int n = 6; n >= 0; --n) q = fmaf(q, r, EXP_C[n]);
    return ldexpf(q, (int)k);
}

/* EXP over an array (for the accuracy pin). */
void oracle_exp_f32_array(const float* y, float* out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp_f32(y[i]);
}

/* Expose the constants so the pin tests can check them against their exact
 * definitions.  out[0]=L2E, out[1]=LN2_HI, out[2]=LN2_LO, out[3]=y_min,
 * out[4..11]=EXP_C[0..7]. */
void oracle_exp_constants(float* out)
{
    out[0] = L2E;
    out[1] = LN2_HI;
    out[2] = LN2_LO;
    out[3] = EXP_Y_MIN;
    for (int n = 0; n < 8; ++n) out[4 + n] = EXP_C[n];
}

/* OpenMP threads used by the parallel window loops (reported with timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Set the number of OpenMP threads of later calls (for the one-thread
 * timings of the CPU baseline). */
void oracle_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* ---------------------------------------------------------------------- */
/* Pack bookkeeping                                                        */
/* ---------------------------------------------------------------------- */

/* Output block count N = sum_s floor(L_s / r).  [PR5984: zero-init folding
 * commit] calls this total_comp; the output has one row per block. */
int oracle_total_comp(const int32_t* cu, int32_t S, int32_t r, int64_t* N)
{
    if (!cu || !N || S < 0 || r < 1) return ORACLE_BAD_ARGS;
    int64_t total = 0;
    for (int32_t s = 0; s < S; ++s) {
        int64_t L = (int64_t)cu[s + 1] - (int64_t)cu[s];
        if (L < 0) return ORACLE_BAD_ARGS;
        total += L / r;
    }
    *N = total;
    return ORACLE_OK;
}

/* The window of one output block, listed in the order given in the header.
 * rows[k], colbase[k] (0 for the first half, (coff-1)*d for the own half) and
 * pos[k] (APE row = position inside the block).  Returns the entry count. */
static int window_of(const int32_t* cu, int32_t s, int64_t b, int32_t r,
                     int32_t coff, int32_t d, int64_t* rows, int32_t* colbase,
                     int32_t* pos)
{
    int K = 0;
    int64_t own = (int64_t)cu[s] + b * r;
    if (coff == 2 && b >= 1) {
        for (int32_t i = 0; i < r; ++i) {
            rows[K] = own - r + i;
            colbase[K] = 0;
            pos[K] = i;
            ++K;
        }
    }
    for (int32_t i = 0; i < r; ++i) {
        rows[K] = own + i;
        colbase[K] = (coff - 1) * d;
        pos[K] = i;
        ++K;
    }
    return K;
}

typedef struct {
    int64_t N;
    int32_t* seg; /* segment of output row n */
    int64_t* blk; /* block index of output row n inside its segment */
} blocks_t;

static int check_pack(const int32_t* cu, int32_t S, int64_t T_cap, int32_t r,
                      int32_t coff, int32_t d)
{
    if (!cu || S < 0 || T_cap < 0 || r < 1 || d < 1) return ORACLE_BAD_ARGS;
    if (coff != 1 && coff != 2) return ORACLE_BAD_ARGS;
    if (cu[0] != 0) return ORACLE_BAD_ARGS;
    for (int32_t s = 0; s < S; ++s)
        if (cu[s + 1] < cu[s]) return ORACLE_BAD_ARGS;
    if ((int64_t)cu[S] > T_cap) return ORACLE_BAD_ARGS;
    return ORACLE_OK;
}

static int list_blocks(const int32_t* cu, int32_t S, int32_t r, blocks_t* bl)
{
    int64_t N;
    int rc = oracle_total_comp(cu, S, r, &N);
    if (rc) return rc;
    bl->N = N;
    bl->seg = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N ? N : 1));
    bl->blk = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N ? N : 1));
    if (!bl->seg || !bl->blk) {
        free(bl->seg);
        free(bl->blk);
        return ORACLE_NO_MEMORY;
    }
    int64_t n = 0;
    for (int32_t s = 0; s < S; ++s) {
        int64_t nb = ((int64_t)cu[s + 1] - cu[s]) / r;
        for (int64_t b = 0; b < nb; ++b, ++n) {
            bl->seg[n] = s;
            bl->blk[n] = b;
        }
    }
    return ORACLE_OK;
}

static void free_blocks(blocks_t* bl)
{
    free(bl->seg);
    free(bl->blk);
}

/* ---------------------------------------------------------------------- */
/* fp32 oracle (fixed evaluation order, see header)                        */
/* ---------------------------------------------------------------------- */

/* Shared body of the fp32 forward and backward: one (block, column) window.
 * Fills e[], v[], returns R and o. */
static void window_f32(const uint16_t* kv, const uint16_t* score,
                       const float* ape, int64_t W, int K, const int64_t* rows,
                       const int32_t* colbase, const int32_t* pos, int32_t j,
                       float* e, float* v, float* R_out, float* o_out)
{
    float x[K];
    for (int k = 0; k < K; ++k) {
        int64_t col = colbase[k] + j;
        x[k] = oracle_f32_from_bf16(score[rows[k] * W + col]) + ape[(int64_t)pos[k] * W + col];
        v[k] = oracle_f32_from_bf16(kv[rows[k] * W + col]);
    }
    float m = x[0];
    for (int k = 1; k < K; ++k) m = fmaxf(m, x[k]);
    for (int k = 0; k < K; ++k) e[k] = oracle_exp_f32(x[k] - m);
    float Z = e[0];
    for (int k = 1; k < K; ++k) Z = Z + e[k];
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) acc = fmaf(e[k], v[k], acc);
    float R = 1.0f / Z;
    *R_out = R;
    *o_out = acc * R;
}

/* Forward.  kv, score: bf16 bits [T_cap, coff*d]; ape fp32 [r, coff*d];
 * cu int32 [S+1]; out bf16 bits [N, d] with N = oracle_total_comp(). */
int oracle_fwd_f32(const uint16_t* kv, const uint16_t* score, const float* ape,
                   const int32_t* cu, int32_t S, int64_t T_cap, int32_t r,
                   int32_t coff, int32_t d, uint16_t* out, int64_t N_expected)
{
    int rc = check_pack(cu, S, T_cap, r, coff, d);
    if (rc) return rc;
    blocks_t bl;
    rc = list_blocks(cu, S, r, &bl);
    if (rc) return rc;
    if (bl.N != N_expected) {
        free_blocks(&bl);
        return ORACLE_BAD_ARGS;
    }
    const int64_t W = (int64_t)coff * d;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < bl.N; ++n) {
        int64_t rows[2 * r];
        int32_t colbase[2 * r], pos[2 * r];
        float e[2 * r], v[2 * r];
        int K = window_of(cu, bl.seg[n], bl.blk[n], r, coff, d, rows, colbase, pos);
        for (int32_t j = 0; j < d; ++j) {
            float R, o;
            window_f32(kv, score, ape, W, K, rows, colbase, pos, j, e, v, &R, &o);
            out[n * d + j] = oracle_bf16_from_f32(o);
        }
    }
    free_blocks(&bl);
    return ORACLE_OK;
}

/* Backward.  dout bf16 bits [N, d]; dkv, dscore bf16 bits [T_cap, coff*d]
 * (fully written: never-consumed slots are +0.0); dape double [r, coff*d]
 * (the exact-order double sum of the fp32 ds values, window by window in
 * output-row order); ds32 (optional, may be NULL) fp32 [T_cap, coff*d] gets
 * the unrounded ds (0 where not consumed); o32 (optional) fp32 [N, d] gets
 * the recomputed fp32 forward value. */
int oracle_bwd_f32(const uint16_t* kv, const uint16_t* score, const float* ape,
                   const int32_t* cu, int32_t S, int64_t T_cap, int32_t r,
                   int32_t coff, int32_t d, const uint16_t* dout,
                   int64_t N_expected, uint16_t* dkv, uint16_t* dscore,
                   double* dape, float* ds32, float* o32)
{
    int rc = check_pack(cu, S, T_cap, r, coff, d);
    if (rc) return rc;
    blocks_t bl;
    rc = list_blocks(cu, S, r, &bl);
    if (rc) return rc;
    if (bl.N != N_expected) {
        free_blocks(&bl);
        return ORACLE_BAD_ARGS;
    }
    const int64_t W = (int64_t)coff * d;
    float* ds = ds32;
    if (!ds) {
        ds = (float*)malloc(sizeof(float) * (size_t)(T_cap * W ? T_cap * W : 1));
        if (!ds) {
            free_blocks(&bl);
            return ORACLE_NO_MEMORY;
        }
    }
    /* Every slot starts as +0.0; consumed slots are overwritten below. */
    memset(dkv, 0, sizeof(uint16_t) * (size_t)(T_cap * W));
    memset(dscore, 0, sizeof(uint16_t) * (size_t)(T_cap * W));
    memset(ds, 0, sizeof(float) * (size_t)(T_cap * W));

#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < bl.N; ++n) {
        int64_t rows[2 * r];
        int32_t colbase[2 * r], pos[2 * r];
        float e[2 * r], v[2 * r];
        int K = window_of(cu, bl.seg[n], bl.blk[n], r, coff, d, rows, colbase, pos);
        for (int32_t j = 0; j < d; ++j) {
            float R, o;
            window_f32(kv, score, ape, W, K, rows, colbase, pos, j, e, v, &R, &o);
            if (o32) o32[n * d + j] = o;
            float G = R * oracle_f32_from_bf16(dout[n * d + j]);
            for (int k = 0; k < K; ++k) {
                int64_t slot = rows[k] * W + colbase[k] + j;
                float a = e[k] * G;
                float dsk = a * (v[k] - o);
                dkv[slot] = oracle_bf16_from_f32(a);
                dscore[slot] = oracle_bf16_from_f32(dsk);
                ds[slot] = dsk;
            }
        }
    }

    /* dAPE: plain serial sum in double, in output-row then window order. */
    for (int64_t i = 0; i < (int64_t)r * W; ++i) dape[i] = 0.0;
    for (int64_t n = 0; n < bl.N; ++n) {
        int64_t rows[2 * r];
        int32_t colbase[2 * r], pos[2 * r];
        int K = window_of(cu, bl.seg[n], bl.blk[n], r, coff, d, rows, colbase, pos);
        for (int k = 0; k < K; ++k)
            for (int32_t j = 0; j < d; ++j) {
                int64_t col = colbase[k] + j;
                dape[(int64_t)pos[k] * W + col] += (double)ds[rows[k] * W + col];
            }
    }
    if (!ds32) free(ds);
    free_blocks(&bl);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------- */
/* fp64 oracle: the plain definition                                       */
/* ---------------------------------------------------------------------- */

static void window_f64(const double* kv, const double* score,
                       const double* ape, int64_t W, int K, const int64_t* rows,
                       const int32_t* colbase, const int32_t* pos, int32_t j,
                       double* p, double* v, double* o_out)
{
    double x[K];
    for (int k = 0; k < K; ++k) {
        int64_t col = colbase[k] + j;
        x[k] = score[rows[k] * W + col] + ape[(int64_t)pos[k] * W + col];
        v[k] = kv[rows[k] * W + col];
    }
    double m = x[0];
    for (int k = 1; k < K; ++k) m = fmax(m, x[k]);
    double Z = 0.0;
    for (int k = 0; k < K; ++k) {
        p[k] = exp(x[k] - m);
        Z += p[k];
    }
    double o = 0.0;
    for (int k = 0; k < K; ++k) {
        p[k] = p[k] / Z;
        o += p[k] * v[k];
    }
    *o_out = o;
}

/* Forward in double.  kv, score and ape are given as double values (the
 * tests pass the bf16/fp32 inputs widened exactly, or perturbed copies for
 * finite differences); out double [N, d] is not rounded to bf16. */
int oracle_fwd_f64(const double* kv, const double* score, const double* ape,
                   const int32_t* cu, int32_t S, int64_t T_cap, int32_t r,
                   int32_t coff, int32_t d, double* out, int64_t N_expected)
{
    int rc = check_pack(cu, S, T_cap, r, coff, d);
    if (rc) return rc;
    blocks_t bl;
    rc = list_blocks(cu, S, r, &bl);
    if (rc) return rc;
    if (bl.N != N_expected) {
        free_blocks(&bl);
        return ORACLE_BAD_ARGS;
    }
    const int64_t W = (int64_t)coff * d;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < bl.N; ++n) {
        int64_t rows[2 * r];
        int32_t colbase[2 * r], pos[2 * r];
        double p[2 * r], v[2 * r];
        int K = window_of(cu, bl.seg[n], bl.blk[n], r, coff, d, rows, colbase, pos);
        for (int32_t j = 0; j < d; ++j) {
            double o;
            window_f64(kv, score, ape, W, K, rows, colbase, pos, j, p, v, &o);
            out[n * d + j] = o;
        }
    }
    free_blocks(&bl);
    return ORACLE_OK;
}

/* Backward in double: dkv, dscore double [T_cap, coff*d] (0 where not
 * consumed), dape double [r, coff*d].  dout double [N, d] is the upstream
 * gradient. */
int oracle_bwd_f64(const double* kv, const double* score, const double* ape,
                   const int32_t* cu, int32_t S, int64_t T_cap, int32_t r,
                   int32_t coff, int32_t d, const double* dout,
                   int64_t N_expected, double* dkv, double* dscore, double* dape)
{
    int rc = check_pack(cu, S, T_cap, r, coff, d);
    if (rc) return rc;
    blocks_t bl;
    rc = list_blocks(cu, S, r, &bl);
    if (rc) return rc;
    if (bl.N != N_expected) {
        free_blocks(&bl);
        return ORACLE_BAD_ARGS;
    }
    const int64_t W = (int64_t)coff * d;
    for (int64_t i = 0; i < T_cap * W; ++i) dkv[i] = dscore[i] = 0.0;
    for (int64_t i = 0; i < (int64_t)r * W; ++i) dape[i] = 0.0;
    for (int64_t n = 0; n < bl.N; ++n) {
        int64_t rows[2 * r];
        int32_t colbase[2 * r], pos[2 * r];
        double p[2 * r], v[2 * r];
        int K = window_of(cu, bl.seg[n], bl.blk[n], r, coff, d, rows, colbase, pos);
        for (int32_t j = 0; j < d; ++j) {
            double o;
            window_f64(kv, score, ape, W, K, rows, colbase, pos, j, p, v, &o);
            double g = dout[n * d + j];
            for (int k = 0; k < K; ++k) {
                int64_t col = colbase[k] + j;
                double a = p[k] * g;
                double dsk = a * (v[k] - o);
                dkv[rows[k] * W + col] = a;
                dscore[rows[k] * W + col] = dsk;
                dape[(int64_t)pos[k] * W + col] += dsk;
            }
        }
    }
    free_blocks(&bl);
    return ORACLE_OK;
}
