/*
 * sq_oracle.c -- CPU oracle for the quantized gated delta-rule decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * model that the GPU path is checked against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * Sources (cited by title and section throughout):
 *   [P1] "K1 論文詳解" (k1-news, paper of 2026-10-09), STEPQuant article,
 *        sections 背景 (background), 方法 (method), 實驗結果 (results).
 *   [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
 *        sections 直接量化为什么会翻车 (why direct quantization fails),
 *        时间维度 (temporal dimension), 空间维度 (spatial dimension),
 *        工程落地 (deployment).
 *
 * Arithmetic is fp64 throughout.  The only places where a lower precision
 * appears are the ones where the stored state itself has that precision:
 *   - a quantized code is decided by rounding an fp32 quotient (the same
 *     precision the GPU path decides it in), ties to even, then clamped;
 *   - an FP16 pivot value is rounded fp64 -> fp32 -> binary16 (ties to even);
 *   - an FP32-state value is rounded fp64 -> fp32;
 *   - the readout o is returned as fp32.
 *
 * Every function below is a direct transcription of a definition; there is no
 * blocking, fusion or reordering.  Bit fields are read and written one bit at
 * a time on purpose.
 *
 * Besides the scalar-gate step, the file holds the per-key-channel-gate step
 * (the reading of the KDA gate named in [P5] 直接量化为什么会翻车), in the
 * same style, with a dense brute-force recurrence of its own.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32, written from the format definition.       */
/* Pivot heads keep their state as FP16 ([P1] 方法; [P5] 时间维度).           */
/* ------------------------------------------------------------------------ */

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24); /* zero or subnormal: m * 2^-24 */
    } else if (e == 31) {
        if (m != 0) return nanf("");
        v = INFINITY;
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1.m) * 2^(e-15) */
    }
    return (float)(sign ? -v : v);
}

/* round-half-to-even of a non-negative double that is an exact multiple of
 * 2^-k for some k (so frac is exact) */
static double rne_nonneg(double x)
{
    double fl = floor(x);
    double frac = x - fl;
    if (frac > 0.5) return fl + 1.0;
    if (frac < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    double a = fabs((double)x);
    /* 65520 = 65504 + half an ulp: at and above it RNE goes to infinity */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; n == 1024 lands on the smallest
         * normal, whose encoding is exactly 1024 */
        double n = rne_nonneg(a / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int E;
    frexp(a, &E); /* a in [2^(E-1), 2^E) */
    int ex = E - 1; /* unbiased exponent */
    double ulp = ldexp(1.0, ex - 10);
    double n = rne_nonneg(a / ulp); /* in [1024, 2048] */
    /* n == 2048 carries into the exponent field by plain addition */
    uint32_t bits = ((uint32_t)(ex + 15) << 10) + (uint32_t)n - 1024u;
    return (uint16_t)(sign | bits);
}

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> binary32.  A bfloat16 is the upper half of a binary32 (sign, */
/* 8 exponent bits, 7 mantissa bits).  Used by the BF16-state format, an     */
/* unquantized 16-bit baseline beside the FP32 state (not a format of the    */
/* pages: a comparison point, as the FP32 state is [P1] 實驗結果).           */
/* ------------------------------------------------------------------------ */

#define ORC_BITS_BF16 144 /* head_bits value of a bfloat16 state */

float orc_bf16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -133); /* zero or subnormal: m * 2^-126 * 2^-7 */
    } else if (e == 255) {
        if (m != 0) return nanf("");
        v = INFINITY;
    } else {
        v = ldexp((double)(128 + m), e - 134); /* (1.m) * 2^(e-127) */
    }
    return (float)(sign ? -v : v);
}

uint16_t orc_f32_to_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0);
    double a = fabs((double)x);
    if (isinf(x)) return (uint16_t)(sign | 0x7f80);
    /* largest finite bfloat16 is (2 - 2^-7) 2^127; half an ulp above it RNE
     * goes to infinity */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7f80);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: quantum 2^-133; n == 128 is the smallest normal */
        double n = rne_nonneg(a / ldexp(1.0, -133));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int E;
    frexp(a, &E);
    int ex = E - 1;
    double ulp = ldexp(1.0, ex - 7);
    double n = rne_nonneg(a / ulp); /* in [128, 256] */
    uint32_t bits = ((uint32_t)(ex + 127) << 7) + (uint32_t)n - 128u;
    return (uint16_t)(sign | bits);
}

/* ------------------------------------------------------------------------ */
/* Tile layout.                                                              */
/*                                                                            */
/* A tile is one head's d_k x d_v state for one request slot; rows i are key */
/* dimensions and columns j are value dimensions ([P5] 空间维度).  Elements   */
/* are numbered in 4x4 blocks: block (i/4, j/4) has index                    */
/*     B = (i/4) * (d_v/4) + (j/4)                                           */
/* (block rows in order, blocks left to right inside a block row), and       */
/* inside a block the four rows of a column are consecutive:                 */
/*     n = 16*B + 4*(j%4) + (i%4).                                           */
/* Field n occupies bits [n*w, n*w + w) of the tile read as a little-endian  */
/* bit stream, w being the field width: 4, 6 or 8 for codes, 16 for an FP16 */
/* pivot or a bfloat16 state, 32 for an FP32 state.  So 4-bit codes sit two */
/* per byte (even n in                                                        */
/* the low nibble) and 6-bit codes four per three bytes (a 24-bit little-    */
/* endian group holds fields 4g..4g+3 at bit offsets 0, 6, 12, 18).          */
/* ------------------------------------------------------------------------ */

long orc_elem_index(int i, int j, int dv)
{
    long B = (long)(i / 4) * (long)(dv / 4) + (long)(j / 4);
    return 16 * B + 4 * (j % 4) + (i % 4);
}

int orc_field_width(int bits)
{
    if (bits == 4 || bits == 6 || bits == 8 || bits == 16 || bits == 32) return bits;
    if (bits == ORC_BITS_BF16) return 16;
    return 0;
}

long orc_tile_bytes(int bits, int dk, int dv)
{
    return (long)dk * (long)dv * (long)orc_field_width(bits) / 8;
}

uint32_t orc_field_get(const uint8_t *tile, int w, long n)
{
    uint32_t v = 0;
    for (int b = 0; b < w; b++) {
        long pos = n * (long)w + b;
        if ((tile[pos >> 3] >> (pos & 7)) & 1) v |= (uint32_t)1 << b;
    }
    return v;
}

void orc_field_put(uint8_t *tile, int w, long n, uint32_t v)
{
    for (int b = 0; b < w; b++) {
        long pos = n * (long)w + b;
        uint8_t mask = (uint8_t)(1u << (pos & 7));
        if ((v >> b) & 1)
            tile[pos >> 3] |= mask;
        else
            tile[pos >> 3] &= (uint8_t)~mask;
    }
}

/* Pool layout: each slot owns a slab; a slab holds the tiles of heads
 * 0..H-1 in order, each tile starting on a 256-byte boundary.  There is one
 * resident state per request slot ([P1] 背景; [P5] opening). */
static long align256(long x) { return (x + 255) / 256 * 256; }

long orc_pool_layout(int n_heads, const uint8_t *head_bits, int dk, int dv, int64_t *off)
{
    long o = 0;
    for (int h = 0; h < n_heads; h++) {
        if (off) off[h] = o;
        o += align256(orc_tile_bytes(head_bits[h], dk, dv));
    }
    return o; /* slab bytes */
}

/* ------------------------------------------------------------------------ */
/* Quantizer.                                                                */
/*                                                                            */
/* Codes are b-bit integers, b in {4,6,8} ([P5] 直接量化为什么会翻车), in the  */
/* symmetric range [-Q, Q], Q = 2^(b-1) - 1, stored excess-2^(b-1): the     */
/* field holds q + 2^(b-1).  The step of element (i,j) is the product of a  */
/* per-key-row factor r_i and a per-value-column factor c_j ([P5] 空间维度; */
/* [P1] 方法), rounded once to fp32: s_ij = fl32(r_i * c_j).                 */
/*   dequantize:  x = q * s_ij                                               */
/*   quantize:    q = clamp(rne(fl32(x / s_ij)), -Q, Q); NaN -> 0            */
/* ------------------------------------------------------------------------ */

double orc_step_size(float r, float c)
{
    return (double)(float)((double)r * (double)c); /* exact product, one fp32 rounding */
}

double orc_decode_field(int bits, uint32_t f, double s)
{
    if (bits == 4 || bits == 6 || bits == 8) {
        int q = (int)f - (1 << (bits - 1));
        return (double)q * s;
    }
    if (bits == 16) return (double)orc_f16_to_f32((uint16_t)f);
    if (bits == ORC_BITS_BF16) return (double)orc_bf16_to_f32((uint16_t)f);
    float x;
    memcpy(&x, &f, 4);
    return (double)x;
}

int orc_quantize(int bits, double x, double s)
{
    int Q = (1 << (bits - 1)) - 1;
    float z = (float)(x / s); /* the decision is taken on an fp32 quotient */
    if (isnan(z)) return 0;
    double r;
    if (z >= 0)
        r = rne_nonneg((double)z);
    else
        r = -rne_nonneg(-(double)z);
    if (r > Q) r = Q;
    if (r < -Q) r = -Q;
    return (int)r;
}

uint32_t orc_encode_field(int bits, double x, double s)
{
    if (bits == 4 || bits == 6 || bits == 8)
        return (uint32_t)(orc_quantize(bits, x, s) + (1 << (bits - 1)));
    if (bits == 16) return orc_f32_to_f16((float)x);
    if (bits == ORC_BITS_BF16) return orc_f32_to_bf16((float)x);
    float y = (float)x;
    uint32_t u;
    memcpy(&u, &y, 4);
    return u;
}

/* Decode a whole tile to fp64 (row-major S[i*dv + j]). */
void orc_decode_tile(int bits, int dk, int dv, const uint8_t *tile, const float *r, const float *c,
                     double *S)
{
    int w = orc_field_width(bits);
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) {
            double s = (bits <= 8) ? orc_step_size(r[i], c[j]) : 1.0;
            uint32_t f = orc_field_get(tile, w, orc_elem_index(i, j, dv));
            S[(long)i * dv + j] = orc_decode_field(bits, f, s);
        }
}

/* Is the value an element is stored from not finite?  For a code that value
 * is the fp32 quotient fl32(x / s) the code is decided on; for an FP16, BF16
 * or FP32 element it is fl32(x).  (The pages are silent on non-finite values;
 * the reading taken is that the store reports them, see orc_encode_tile.) */
int orc_nonfinite_field(int bits, double x, double s)
{
    float y = (bits == 4 || bits == 6 || bits == 8) ? (float)(x / s) : (float)x;
    return !isfinite(y);
}

/* Encode an fp64 tile (row-major) into packed fields.  Returns 1 if any
 * element's stored-from value is not finite (orc_nonfinite_field), else 0:
 * the tile's contribution to the pool's sticky flag.  Such an element is still
 * stored by the rule of orc_quantize / the float conversions. */
int orc_encode_tile(int bits, int dk, int dv, const double *S, const float *r, const float *c,
                    uint8_t *tile)
{
    int w = orc_field_width(bits);
    int bad = 0;
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) {
            double s = (bits <= 8) ? orc_step_size(r[i], c[j]) : 1.0;
            double x = S[(long)i * dv + j];
            bad |= orc_nonfinite_field(bits, x, s);
            orc_field_put(tile, w, orc_elem_index(i, j, dv), orc_encode_field(bits, x, s));
        }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* One decode step on one tile.                                              */
/*                                                                            */
/* Each step reads the stored state, updates it, requantizes it and stores  */
/* it back ([P5] 直接量化为什么会翻车).  The update is the gated delta rule   */
/* ([P5] opening): decay by the gate alpha plus a correction along the       */
/* current key ([P5] 时间维度), i.e.                                          */
/*     S' = alpha (I - beta k k^T) S + beta k v^T.                           */
/* Expanding (I - beta k k^T) S = S - beta k (k^T S) with u = S^T k gives    */
/*     S'_ij = alpha S_ij + beta k_i (v_j - alpha u_j),                       */
/* which is what is evaluated (the dense form is evaluated separately by     */
/* orc_bruteforce and the two are compared in the tests).  The query readout */
/* o = S'^T q ([P5] 空间维度: output error is a key/query/gate-weighted sum  */
/* over rows) is taken from the updated state before requantization.         */
/* ------------------------------------------------------------------------ */

int orc_step_tile(int bits, int dk, int dv, uint8_t *tile, const float *r, const float *c,
                  const float *q, const float *k, const float *v, float alpha, float beta,
                  float *o)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    orc_decode_tile(bits, dk, dv, tile, r, c, S);
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++) acc += (double)k[i] * S[(long)i * dv + j];
        u[j] = acc;
    }
    double a = alpha, b = beta;
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++)
            S[(long)i * dv + j] = a * S[(long)i * dv + j] + b * (double)k[i] * ((double)v[j] - a * u[j]);
    if (o) {
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += (double)q[i] * S[(long)i * dv + j];
            o[j] = (float)acc;
        }
    }
    int bad = orc_encode_tile(bits, dk, dv, S, r, c, tile);
    free(u);
    free(S);
    return bad;
}

/* Readout without update: o = S^T q from the stored (dequantized) state. */
void orc_readout_tile(int bits, int dk, int dv, const uint8_t *tile, const float *r,
                      const float *c, const float *q, float *o)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    orc_decode_tile(bits, dk, dv, tile, r, c, S);
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++) acc += (double)q[i] * S[(long)i * dv + j];
        o[j] = (float)acc;
    }
    free(S);
}

/* ------------------------------------------------------------------------ */
/* Pool-level step: the batch of requests n = 0..n_req-1, request n owning  */
/* slot slot_ids[n].  Inputs are row-major [n_req][H][d]; alpha, beta are    */
/* [n_req][H].  The factors of slot p, head h are r + (p*S + h)*d_k and      */
/* c + (p*S + h)*d_v: with the scale stride S = 0 one set [H][d] is shared   */
/* by every slot, with S >= H every slot has its own ([P5] 空间维度 gives     */
/* each row and each column of a state matrix its own factor).  The          */
/* (request, head) tiles are independent; they are split over n_threads     */
/* plain threads in contiguous chunks.  The step returns how many tiles     */
/* stored a value from a non-finite one (orc_encode_tile): the pool's       */
/* sticky flag is set iff that count is non-zero.                            */
/* ------------------------------------------------------------------------ */

typedef struct {
    uint8_t *pool;
    long slab;
    const int64_t *off;
    int n_heads, dk, dv;
    const uint8_t *bits;
    const float *r, *c;
    long sstride; /* scale slot stride S */
    const int32_t *slot_ids;
    const float *q, *k, *v, *alpha, *beta;
    float *o;
    long t0, t1;
    int readout_only;
    int channel_gate; /* alpha is [n_req][H][d_k] (orc_step_tile_kda) */
    long flagged;     /* out: tiles whose step met a non-finite value */
} orc_job;

static const float *orc_factors(const float *base, long stride, int32_t slot, int h, int d)
{
    return base + ((long)slot * stride + h) * (long)d;
}

int orc_step_tile_kda(int bits, int dk, int dv, uint8_t *tile, const float *r, const float *c,
                      const float *q, const float *k, const float *v, const float *alpha,
                      float beta, float *o);

static void *orc_worker(void *arg)
{
    orc_job *J = (orc_job *)arg;
    for (long t = J->t0; t < J->t1; t++) {
        long n = t / J->n_heads;
        int h = (int)(t % J->n_heads);
        uint8_t *tile = J->pool + (long)J->slot_ids[n] * J->slab + J->off[h];
        const float *r = orc_factors(J->r, J->sstride, J->slot_ids[n], h, J->dk);
        const float *c = orc_factors(J->c, J->sstride, J->slot_ids[n], h, J->dv);
        const float *q = J->q + t * J->dk;
        float *o = J->o ? J->o + t * J->dv : NULL;
        if (J->readout_only) {
            orc_readout_tile(J->bits[h], J->dk, J->dv, tile, r, c, q, o);
        } else if (J->channel_gate) {
            J->flagged += orc_step_tile_kda(J->bits[h], J->dk, J->dv, tile, r, c, q,
                                            J->k + t * J->dk, J->v + t * J->dv,
                                            J->alpha + t * J->dk, J->beta[t], o);
        } else {
            J->flagged += orc_step_tile(J->bits[h], J->dk, J->dv, tile, r, c, q, J->k + t * J->dk,
                                        J->v + t * J->dv, J->alpha[t], J->beta[t], o);
        }
    }
    return NULL;
}

static long orc_run(orc_job *base, long n_tiles, int n_threads)
{
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    orc_job jobs[256];
    long chunk = (n_tiles + n_threads - 1) / n_threads;
    int started = 0, n_jobs = 0;
    for (int w = 0; w < n_threads; w++) {
        jobs[w] = *base;
        jobs[w].t0 = (long)w * chunk;
        jobs[w].t1 = jobs[w].t0 + chunk < n_tiles ? jobs[w].t0 + chunk : n_tiles;
        if (jobs[w].t0 >= jobs[w].t1) break;
        n_jobs++;
        if (n_threads == 1) {
            orc_worker(&jobs[w]);
        } else {
            pthread_create(&th[w], NULL, orc_worker, &jobs[w]);
            started++;
        }
    }
    for (int w = 0; w < started; w++) pthread_join(th[w], NULL);
    long flagged = 0;
    for (int w = 0; w < n_jobs; w++) flagged += jobs[w].flagged;
    return flagged;
}

long orc_step_pool(uint8_t *pool, int n_heads, int dk, int dv, const uint8_t *head_bits,
                   const float *r, const float *c, long scale_stride, const int32_t *slot_ids,
                   int n_req, const float *q, const float *k, const float *v, const float *alpha,
                   const float *beta, float *o, int n_threads)
{
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_heads > 0 ? n_heads : 1));
    orc_job J;
    memset(&J, 0, sizeof(J));
    J.pool = pool;
    J.slab = orc_pool_layout(n_heads, head_bits, dk, dv, off);
    J.off = off;
    J.n_heads = n_heads;
    J.dk = dk;
    J.dv = dv;
    J.bits = head_bits;
    J.r = r;
    J.c = c;
    J.sstride = scale_stride;
    J.slot_ids = slot_ids;
    J.q = q;
    J.k = k;
    J.v = v;
    J.alpha = alpha;
    J.beta = beta;
    J.o = o;
    long flagged = orc_run(&J, (long)n_req * n_heads, n_threads);
    free(off);
    return flagged;
}

void orc_readout_pool(const uint8_t *pool, int n_heads, int dk, int dv, const uint8_t *head_bits,
                      const float *r, const float *c, long scale_stride, const int32_t *slot_ids,
                      int n_req, const float *q, float *o, int n_threads)
{
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_heads > 0 ? n_heads : 1));
    orc_job J;
    memset(&J, 0, sizeof(J));
    J.pool = (uint8_t *)pool;
    J.slab = orc_pool_layout(n_heads, head_bits, dk, dv, off);
    J.off = off;
    J.n_heads = n_heads;
    J.dk = dk;
    J.dv = dv;
    J.bits = head_bits;
    J.r = r;
    J.c = c;
    J.sstride = scale_stride;
    J.slot_ids = slot_ids;
    J.q = q;
    J.o = o;
    J.readout_only = 1;
    orc_run(&J, (long)n_req * n_heads, n_threads);
    free(off);
}

/* Quantize-and-store: encode fp32 states S[n_req][H][d_k][d_v] (row-major)
 * into the tiles of slots slot_ids[n], factors as orc_step_pool.  Returns the
 * number of tiles that stored a value from a non-finite one. */
long orc_store_pool(uint8_t *pool, int n_heads, int dk, int dv, const uint8_t *head_bits,
                    const float *r, const float *c, long scale_stride, const int32_t *slot_ids,
                    int n_req, const float *S)
{
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_heads > 0 ? n_heads : 1));
    long slab = orc_pool_layout(n_heads, head_bits, dk, dv, off);
    double *D = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    long flagged = 0;
    for (int n = 0; n < n_req; n++)
        for (int h = 0; h < n_heads; h++) {
            const float *src = S + ((long)n * n_heads + h) * (long)dk * dv;
            for (long e = 0; e < (long)dk * dv; e++) D[e] = (double)src[e];
            flagged += orc_encode_tile(head_bits[h], dk, dv, D,
                                       orc_factors(r, scale_stride, slot_ids[n], h, dk),
                                       orc_factors(c, scale_stride, slot_ids[n], h, dv),
                                       pool + (long)slot_ids[n] * slab + off[h]);
        }
    free(D);
    free(off);
    return flagged;
}

/* ------------------------------------------------------------------------ */
/* Brute-force recurrence (unquantized, fp64), an independent formulation    */
/* used only to pin orc_step_tile's expanded form.                           */
/*                                                                            */
/* With A_t = alpha_t (I - beta_t k_t k_t^T) formed as a dense d_k x d_k     */
/* matrix and Phi(t, s) = A_t A_(t-1) ... A_s (Phi(t, t+1) = I),             */
/*     S_t = Phi(t,1) S_0 + sum_{s=1..t} Phi(t, s+1) beta_s k_s v_s^T,       */
/*     o_t = S_t^T q_t.                                                      */
/* Inputs are [T][d]; S0 and S_T are row-major d_k x d_v; o is [T][d_v].     */
/* ------------------------------------------------------------------------ */

static void matmul(int n, int m, int p, const double *A, const double *B, double *C)
{
    for (int i = 0; i < n; i++)
        for (int j = 0; j < p; j++) {
            double acc = 0.0;
            for (int l = 0; l < m; l++) acc += A[(long)i * m + l] * B[(long)l * p + j];
            C[(long)i * p + j] = acc;
        }
}

void orc_bruteforce(int dk, int dv, int T, const double *S0, const double *q, const double *k,
                    const double *v, const double *alpha, const double *beta, double *ST,
                    double *o)
{
    size_t kk = (size_t)dk * dk, kv = (size_t)dk * dv;
    double *A = (double *)malloc(sizeof(double) * kk * (size_t)T);
    double *Phi = (double *)malloc(sizeof(double) * kk);
    double *tmp = (double *)malloc(sizeof(double) * kk);
    double *St = (double *)malloc(sizeof(double) * kv);
    double *term = (double *)malloc(sizeof(double) * kv);
    double *outer = (double *)malloc(sizeof(double) * kv);
    for (int t = 0; t < T; t++)
        for (int i = 0; i < dk; i++)
            for (int l = 0; l < dk; l++)
                A[t * kk + (size_t)i * dk + l] =
                    alpha[t] * ((i == l ? 1.0 : 0.0) - beta[t] * k[(long)t * dk + i] * k[(long)t * dk + l]);
    memcpy(St, S0, sizeof(double) * kv); /* T == 0 leaves S_T = S_0 */
    for (int t = 0; t < T; t++) { /* S_(t+1) in 1-based terms */
        /* Phi(t..0) applied to S0 */
        for (size_t e = 0; e < kk; e++) Phi[e] = ((e / dk) == (e % dk)) ? 1.0 : 0.0;
        for (int s = 0; s <= t; s++) { /* Phi = A_t ... A_0 */
            matmul(dk, dk, dk, A + (size_t)s * kk, Phi, tmp);
            memcpy(Phi, tmp, sizeof(double) * kk);
        }
        matmul(dk, dk, dv, Phi, S0, St);
        for (int s = 0; s <= t; s++) {
            /* Phi(t, s+1) = A_t ... A_(s+1) */
            for (size_t e = 0; e < kk; e++) Phi[e] = ((e / dk) == (e % dk)) ? 1.0 : 0.0;
            for (int m = s + 1; m <= t; m++) {
                matmul(dk, dk, dk, A + (size_t)m * kk, Phi, tmp);
                memcpy(Phi, tmp, sizeof(double) * kk);
            }
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++)
                    outer[(long)i * dv + j] = beta[s] * k[(long)s * dk + i] * v[(long)s * dv + j];
            matmul(dk, dk, dv, Phi, outer, term);
            for (size_t e = 0; e < kv; e++) St[e] += term[e];
        }
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += q[(long)t * dk + i] * St[(long)i * dv + j];
            o[(long)t * dv + j] = acc;
        }
    }
    memcpy(ST, St, sizeof(double) * kv);
    free(outer);
    free(term);
    free(St);
    free(tmp);
    free(Phi);
    free(A);
}

/* Array forms of the binary16 conversions (for the tests). */
void orc_f32_to_f16_array(const float *x, uint16_t *h, long n)
{
    for (long e = 0; e < n; e++) h[e] = orc_f32_to_f16(x[e]);
}

void orc_f32_to_bf16_array(const float *x, uint16_t *h, long n)
{
    for (long i = 0; i < n; i++) h[i] = orc_f32_to_bf16(x[i]);
}

void orc_bf16_to_f32_array(const uint16_t *h, float *x, long n)
{
    for (long i = 0; i < n; i++) x[i] = orc_bf16_to_f32(h[i]);
}

void orc_f16_to_f32_array(const uint16_t *h, float *x, long n)
{
    for (long e = 0; e < n; e++) x[e] = orc_f16_to_f32(h[e]);
}

/* Load-and-dequantize: write the states of slots slot_ids[n] as fp32
 * S[n_req][H][d_k][d_v] (row-major), each element the decoded value rounded
 * once to fp32 (codes: fl32(q * s_ij); pivots: the binary16 value; FP32: the
 * stored value). */
void orc_load_pool(const uint8_t *pool, int n_heads, int dk, int dv, const uint8_t *head_bits,
                   const float *r, const float *c, long scale_stride, const int32_t *slot_ids,
                   int n_req, float *S)
{
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_heads > 0 ? n_heads : 1));
    long slab = orc_pool_layout(n_heads, head_bits, dk, dv, off);
    double *D = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    for (int n = 0; n < n_req; n++)
        for (int h = 0; h < n_heads; h++) {
            orc_decode_tile(head_bits[h], dk, dv, pool + (long)slot_ids[n] * slab + off[h],
                            orc_factors(r, scale_stride, slot_ids[n], h, dk),
                            orc_factors(c, scale_stride, slot_ids[n], h, dv), D);
            float *dst = S + ((long)n * n_heads + h) * (long)dk * dv;
            for (long e = 0; e < (long)dk * dv; e++) dst[e] = (float)D[e];
        }
    free(D);
    free(off);
}

/* ------------------------------------------------------------------------ */
/* Per-channel gate (the gating of the second model family, Kimi-Linear,     */
/* named in [P5] 直接量化为什么会翻车 as KDA; the pages give no formula).      */
/* Reading: the gate is a vector alpha in R^{d_k} that decays each key row,  */
/*     S' = (I - beta k k^T) diag(alpha) S + beta k v^T.                      */
/* With T = diag(alpha) S and u = T^T k:  S'_ij = alpha_i S_ij               */
/*     + beta k_i (v_j - u_j),  o = S'^T q.                                  */
/* ------------------------------------------------------------------------ */

int orc_step_tile_kda(int bits, int dk, int dv, uint8_t *tile, const float *r, const float *c,
                      const float *q, const float *k, const float *v, const float *alpha,
                      float beta, float *o)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    orc_decode_tile(bits, dk, dv, tile, r, c, S);
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) S[(long)i * dv + j] *= (double)alpha[i]; /* T */
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++) acc += (double)k[i] * S[(long)i * dv + j];
        u[j] = acc;
    }
    double b = beta;
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) S[(long)i * dv + j] += b * (double)k[i] * ((double)v[j] - u[j]);
    if (o) {
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += (double)q[i] * S[(long)i * dv + j];
            o[j] = (float)acc;
        }
    }
    int bad = orc_encode_tile(bits, dk, dv, S, r, c, tile);
    free(u);
    free(S);
    return bad;
}

/* Pool-level per-channel-gate step; alpha is [n_req][H][d_k], the rest as
 * orc_step_pool. */
long orc_step_pool_kda(uint8_t *pool, int n_heads, int dk, int dv, const uint8_t *head_bits,
                       const float *r, const float *c, long scale_stride, const int32_t *slot_ids,
                       int n_req, const float *q, const float *k, const float *v,
                       const float *alpha, const float *beta, float *o, int n_threads)
{
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_heads > 0 ? n_heads : 1));
    orc_job J;
    memset(&J, 0, sizeof(J));
    J.pool = pool;
    J.slab = orc_pool_layout(n_heads, head_bits, dk, dv, off);
    J.off = off;
    J.n_heads = n_heads;
    J.dk = dk;
    J.dv = dv;
    J.bits = head_bits;
    J.r = r;
    J.c = c;
    J.sstride = scale_stride;
    J.slot_ids = slot_ids;
    J.q = q;
    J.k = k;
    J.v = v;
    J.alpha = alpha;
    J.beta = beta;
    J.o = o;
    J.channel_gate = 1;
    long flagged = orc_run(&J, (long)n_req * n_heads, n_threads);
    free(off);
    return flagged;
}

/* Dense fp64 recurrence with A_t = (I - beta_t k_t k_t^T) diag(alpha_t);
 * alpha is [T][d_k].  Same conventions as orc_bruteforce. */
void orc_bruteforce_kda(int dk, int dv, int T, const double *S0, const double *q, const double *k,
                        const double *v, const double *alpha, const double *beta, double *ST,
                        double *o)
{
    size_t kk = (size_t)dk * dk, kv = (size_t)dk * dv;
    double *A = (double *)malloc(sizeof(double) * kk);
    double *St = (double *)malloc(sizeof(double) * kv);
    double *nx = (double *)malloc(sizeof(double) * kv);
    memcpy(St, S0, sizeof(double) * kv);
    for (int t = 0; t < T; t++) {
        for (int i = 0; i < dk; i++)
            for (int l = 0; l < dk; l++)
                A[(size_t)i * dk + l] = ((i == l ? 1.0 : 0.0) - beta[t] * k[(long)t * dk + i] *
                                         k[(long)t * dk + l]) * alpha[(long)t * dk + l];
        matmul(dk, dk, dv, A, St, nx);
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++)
                nx[(long)i * dv + j] += beta[t] * k[(long)t * dk + i] * v[(long)t * dv + j];
        memcpy(St, nx, sizeof(double) * kv);
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += q[(long)t * dk + i] * St[(long)i * dv + j];
            o[(long)t * dv + j] = acc;
        }
    }
    memcpy(ST, St, sizeof(double) * kv);
    free(nx);
    free(St);
    free(A);
}
