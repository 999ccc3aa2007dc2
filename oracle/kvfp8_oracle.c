/*
 * kvfp8 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar C implementation of what the FP8-E4M3 scaled paged
 * KV cache computes.  It exists to check the HIP library; it is never part of
 * the product path.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -std=c11 -shared -fPIC (no fast-math), so
 * every float/double operation below rounds exactly as written.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "llama : Add FP8 KV-cache support (#28392)", llama.cpp commit
 *        202c1a229 (gitnews mirror): src/llama-graph.cpp
 *        build_attn_scale_kv_inputs / build_attn_scale_kv_output (scale
 *        folding); tests/test-fp8.cpp check_fp8_attention (double-precision
 *        brute-force attention) and check_fp8_context_shift (dequantize ->
 *        rope -> requantize K-shift).
 *   [P2] git.wylab.me compare view, branch osimons/ocp_fp8_kv: ggml
 *        ggml_f8_e4m3_to_fp32, ggml_round_to_nearest_even,
 *        ggml_fp32_to_f8_e4m3 (the E4M3 codec).
 *   [P3] vllm.cpp PR #1641 "feat(KV-FP8): W3 -- half-sized KV blocks ...":
 *        KVBytesPerBlock halving; the store rounding envelope.
 *
 * Cache layout (a choice of this library; the pages fix none).  Per layer a
 * K pool and a V pool, each [num_blocks][num_kv_heads][block_size*head_dim]
 * bytes.  Slot s lives in block s / BS at in-block token t = s % BS.  Inside
 * one (block, kv-head) tile of BS*D bytes:
 *   K byte of (t, d) at  ((d / (D/4)) * BS + t) * (D/4) + d % (D/4)
 *   V byte of (t, d) at  ((t / 4) * D + d) * 4 + t % 4
 * i.e. K is split into four column quarters, each [BS][D/4]; V is stored
 * d-major inside groups of four consecutive tokens.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* bf16 widening: a bf16 value is the top 16 bits of an fp32 value.    */
/* ------------------------------------------------------------------ */
static float orc_bf16_to_f32(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

float orc_bf16_bits_to_f32(uint16_t bits) { return orc_bf16_to_f32(bits); }

/* ------------------------------------------------------------------ */
/* E4M3 decode [P2, ggml_f8_e4m3_to_fp32]: 1 sign bit, 4 exponent bits  */
/* (bias 7), 3 mantissa bits; magnitude 0x7F is NaN; exponent field 0   */
/* is the subnormal range m * 2^-9.                                     */
/* ------------------------------------------------------------------ */
float orc_e4m3_decode(uint8_t code)
{
    const uint8_t mag = code & 0x7F;
    if (mag == 0x7F)
        return NAN;
    const int e = mag >> 3;
    const int m = mag & 0x7;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -9);
    else
        v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (code & 0x80) ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Round a non-negative float to the nearest integer, ties to even      */
/* [P2, ggml_round_to_nearest_even].  Inputs here are below 2^4, so     */
/* floor and the subtraction are exact.                                 */
/* ------------------------------------------------------------------ */
static int orc_round_half_even(float x)
{
    const float fl = floorf(x);
    const int i = (int)fl;
    const float frac = x - fl;
    if (frac > 0.5f)
        return i + 1;
    if (frac < 0.5f)
        return i;
    return (i & 1) ? i + 1 : i;
}

/* ------------------------------------------------------------------ */
/* E4M3 encode, saturating [P2, ggml_fp32_to_f8_e4m3], in the pages'    */
/* order: sign; NaN; zero; saturation of Inf and |x| >= 448 to the      */
/* largest finite code; subnormal range |x| < 2^-6 on the 2^-9 grid;    */
/* otherwise exponent from frexp and a 3-bit mantissa rounded half-even */
/* with carry into the exponent, saturating again at the top.           */
/* ------------------------------------------------------------------ */
uint8_t orc_e4m3_encode(float x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;
    const float a = fabsf(x);

    if (isnan(a))
        return sign | 0x7F;
    if (a == 0.0f)
        return sign;
    if (isinf(a) || a >= 448.0f)
        return sign | 0x7E;
    if (a < 0.015625f)
        return sign | (uint8_t)orc_round_half_even(a * 512.0f);

    int ex;
    const float frac = frexpf(a, &ex);   /* a = frac * 2^ex, frac in [0.5, 1) */
    const float sig = frac * 2.0f;        /* a = sig * 2^(ex-1), sig in [1, 2) */
    int biased = ex + 6;                  /* (ex - 1) + 7 */
    int mant = orc_round_half_even((sig - 1.0f) * 8.0f);
    if (mant == 8) {
        mant = 0;
        biased += 1;
    }
    if (biased > 15 || (biased == 15 && mant > 6))
        return sign | 0x7E;
    return sign | (uint8_t)((biased << 3) | mant);
}

void orc_e4m3_decode_n(const uint8_t *codes, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(codes[i]);
}

void orc_e4m3_encode_n(const float *x, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(x[i]);
}

/* ------------------------------------------------------------------ */
/* Scale intake.  A scale must be finite and nonzero [P1,               */
/* llama_init_from_model]; the store multiplies by the fp32 reciprocal, */
/* so that reciprocal must be finite too.  Returns 1 when usable.       */
/* ------------------------------------------------------------------ */
int orc_scale_ok(float s)
{
    if (!isfinite(s) || s == 0.0f)
        return 0;
    const float inv = 1.0f / s;
    return isfinite(inv) && inv != 0.0f;
}

float orc_scale_inverse(float s) { return 1.0f / s; }

/* ------------------------------------------------------------------ */
/* Tile layout (see the header comment).                                */
/* ------------------------------------------------------------------ */
int64_t orc_k_tile_offset(int t, int d, int BS, int D)
{
    const int quarter = D / 4;
    return ((int64_t)(d / quarter) * BS + t) * quarter + d % quarter;
}

int64_t orc_v_tile_offset(int t, int d, int BS, int D)
{
    (void)BS;
    return ((int64_t)(t / 4) * D + d) * 4 + t % 4;
}

static int64_t orc_tile_base(int64_t block, int h, int Hkv, int BS, int D)
{
    return (block * Hkv + h) * (int64_t)BS * D;
}

/* ------------------------------------------------------------------ */
/* Store [P1, build_attn_scale_kv_inputs: the cache holds K/s_k and     */
/* V/s_v; P2, quantize_row_f8_e4m3_ref].  x is the bf16 input widened   */
/* to fp32, y = fl32(x * fl32(1/s)), code = encode(y).  IEEE 754 leaves */
/* the sign of a NaN produced by a multiply unspecified, so a NaN input */
/* keeps its own sign.  A negative slot, or one at or past the pool's   */
/* NB * BS slots, means "skip this token".                              */
/* k, v: [T][Hkv][D] bf16 bits with a token stride in elements.         */
/* ------------------------------------------------------------------ */
void orc_store_typed(const uint16_t *k, const uint16_t *v,
                     int64_t k_tok_stride, int64_t v_tok_stride,
                     const int64_t *slots, int64_t T,
                     int Hkv, int D, int BS, int64_t NB, int k_eb, int v_eb,
                     float k_scale, float v_scale, void *k_pool, void *v_pool)
{
    const float k_inv = 1.0f / k_scale;
    const float v_inv = 1.0f / v_scale;
    for (int64_t i = 0; i < T; ++i) {
        const int64_t slot = slots[i];
        if (slot < 0 || slot >= NB * BS)
            continue;
        const int64_t block = slot / BS;
        const int t = (int)(slot % BS);
        for (int h = 0; h < Hkv; ++h) {
            const int64_t base = orc_tile_base(block, h, Hkv, BS, D);
            for (int d = 0; d < D; ++d) {
                const uint16_t bk = k[i * k_tok_stride + (int64_t)h * D + d];
                const uint16_t bv = v[i * v_tok_stride + (int64_t)h * D + d];
                const int64_t ek = base + orc_k_tile_offset(t, d, BS, D);
                const int64_t ev = base + orc_v_tile_offset(t, d, BS, D);
                if (k_eb == 2) {
                    ((uint16_t *)k_pool)[ek] = bk;
                } else {
                    const float xk = orc_bf16_to_f32(bk);
                    ((uint8_t *)k_pool)[ek] = orc_e4m3_encode(isnan(xk) ? xk : xk * k_inv);
                }
                if (v_eb == 2) {
                    ((uint16_t *)v_pool)[ev] = bv;
                } else {
                    const float xv = orc_bf16_to_f32(bv);
                    ((uint8_t *)v_pool)[ev] = orc_e4m3_encode(isnan(xv) ? xv : xv * v_inv);
                }
            }
        }
    }
}

void orc_store(const uint16_t *k, const uint16_t *v,
               int64_t k_tok_stride, int64_t v_tok_stride,
               const int64_t *slots, int64_t T,
               int Hkv, int D, int BS, int64_t NB, float k_scale, float v_scale,
               uint8_t *k_pool, uint8_t *v_pool)
{
    orc_store_typed(k, v, k_tok_stride, v_tok_stride, slots, T, Hkv, D, BS, NB, 1, 1,
                    k_scale, v_scale, k_pool, v_pool);
}

/* ------------------------------------------------------------------ */
/* Gather the dequantized fp32 K and V rows of one sequence and one     */
/* kv-head, in position order, following the block table:               */
/* Kd = fl32(decode(code) * s_k), Vd = fl32(decode(code) * s_v).  A     */
/* bf16 pool (element bytes 2) holds the values themselves: Kd = the    */
/* bf16 value times its scale (1 for such a pool).                      */
/* ------------------------------------------------------------------ */
static float orc_element(const void *pool, int eb, int64_t e)
{
    if (eb == 2)
        return orc_bf16_to_f32(((const uint16_t *)pool)[e]);
    return orc_e4m3_decode(((const uint8_t *)pool)[e]);
}

void orc_gather_typed(const void *k_pool, const void *v_pool,
                      int Hkv, int D, int BS, int k_eb, int v_eb,
                      const int32_t *table, int L, int h,
                      float k_scale, float v_scale,
                      float *kd, float *vd)
{
    for (int p = 0; p < L; ++p) {
        const int64_t block = table[p / BS];
        const int t = p % BS;
        const int64_t base = orc_tile_base(block, h, Hkv, BS, D);
        for (int d = 0; d < D; ++d) {
            kd[(int64_t)p * D + d] = orc_element(k_pool, k_eb, base + orc_k_tile_offset(t, d, BS, D)) * k_scale;
            vd[(int64_t)p * D + d] = orc_element(v_pool, v_eb, base + orc_v_tile_offset(t, d, BS, D)) * v_scale;
        }
    }
}

void orc_gather_dequant(const uint8_t *k_pool, const uint8_t *v_pool,
                        int Hkv, int D, int BS,
                        const int32_t *table, int L, int h,
                        float k_scale, float v_scale,
                        float *kd, float *vd)
{
    orc_gather_typed(k_pool, v_pool, Hkv, D, BS, 1, 1, table, L, h, k_scale, v_scale, kd, vd);
}

/* ------------------------------------------------------------------ */
/* Attention of one query row over the first n keys, by definition, in  */
/* fp64 [P1, check_fp8_attention]: score_t = (q . Kd_t) * sm_scale,     */
/* p = softmax(score) with the maximum subtracted, o = sum_t p_t Vd_t.  */
/* n == 0 gives zeros.                                                  */
/* ------------------------------------------------------------------ */
static void orc_attend_row(const uint16_t *q, const float *kd, const float *vd,
                           int n, int D, double sm_scale, double *scores, double *o)
{
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (n == 0)
        return;
    double mx = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += (double)orc_bf16_to_f32(q[d]) * (double)kd[(int64_t)t * D + d];
        scores[t] = dot * sm_scale;
        if (scores[t] > mx)
            mx = scores[t];
    }
    double sum = 0.0;
    for (int t = 0; t < n; ++t) {
        scores[t] = exp(scores[t] - mx);
        sum += scores[t];
    }
    for (int t = 0; t < n; ++t) {
        const double p = scores[t] / sum;
        for (int d = 0; d < D; ++d)
            o[d] += p * (double)vd[(int64_t)t * D + d];
    }
}

/* ------------------------------------------------------------------ */
/* Paged decode attention.  Query head h of sequence b reads kv-head    */
/* h / (Hq / Hkv) (grouped-query attention) over seq_lens[b] cached     */
/* tokens.  q: [B][Hq][D] bf16 bits; out: [B][Hq][D] fp64.              */
/* heads: optional list of n_sel (b, h) pairs to compute (others are    */
/* left untouched); NULL computes every (b, h).                         */
/* Returns 0, or -1 when scratch memory cannot be allocated.            */
/* ------------------------------------------------------------------ */
int orc_decode_attn_typed(const uint16_t *q, int Hq,
                          const void *k_pool, const void *v_pool,
                          int Hkv, int D, int BS, int k_eb, int v_eb,
                          const int32_t *block_tables, int max_blocks,
                          const int32_t *seq_lens, int B,
                          float k_scale, float v_scale, double sm_scale,
                          const int32_t *sel, int64_t n_sel, double *out)
{
    const int g = Hq / Hkv;
    int maxL = 0;
    for (int b = 0; b < B; ++b)
        if (seq_lens[b] > maxL)
            maxL = seq_lens[b];
    float *kd = (float *)malloc(sizeof(float) * ((size_t)maxL * D + 1));
    float *vd = (float *)malloc(sizeof(float) * ((size_t)maxL * D + 1));
    double *scores = (double *)malloc(sizeof(double) * ((size_t)maxL + 1));
    if (!kd || !vd || !scores) {
        free(kd); free(vd); free(scores);
        return -1;
    }
    const int64_t total = sel ? n_sel : (int64_t)B * Hq;
    for (int64_t i = 0; i < total; ++i) {
        const int b = sel ? sel[2 * i] : (int)(i / Hq);
        const int h = sel ? sel[2 * i + 1] : (int)(i % Hq);
        const int L = seq_lens[b];
        const int kvh = h / g;
        orc_gather_typed(k_pool, v_pool, Hkv, D, BS, k_eb, v_eb, block_tables + (int64_t)b * max_blocks,
                         L, kvh, k_scale, v_scale, kd, vd);
        orc_attend_row(q + ((int64_t)b * Hq + h) * D, kd, vd, L, D, sm_scale, scores,
                       out + ((int64_t)b * Hq + h) * D);
    }
    free(kd); free(vd); free(scores);
    return 0;
}

int orc_decode_attn(const uint16_t *q, int Hq,
                    const uint8_t *k_pool, const uint8_t *v_pool,
                    int Hkv, int D, int BS,
                    const int32_t *block_tables, int max_blocks,
                    const int32_t *seq_lens, int B,
                    float k_scale, float v_scale, double sm_scale,
                    const int32_t *sel, int64_t n_sel, double *out)
{
    return orc_decode_attn_typed(q, Hq, k_pool, v_pool, Hkv, D, BS, 1, 1, block_tables, max_blocks,
                                 seq_lens, B, k_scale, v_scale, sm_scale, sel, n_sel, out);
}

/* ------------------------------------------------------------------ */
/* Chunked-prefill attention.  Sequence b has context_lens[b] tokens    */
/* cached before its chunk of cu_q_lens[b+1]-cu_q_lens[b] query tokens; */
/* the chunk's own K/V are already in the cache after the context.      */
/* Query token i of the chunk sits at position ctx_b + i and attends    */
/* causally to positions 0 .. ctx_b + i [P1, check_fp8_attention: past */
/* <= token].  q, out: [total_q][Hq][D].                                */
/* sel: optional list of n_sel (global query index, head) pairs.        */
/* ------------------------------------------------------------------ */
int orc_prefill_attn_typed(const uint16_t *q, int Hq,
                           const void *k_pool, const void *v_pool,
                           int Hkv, int D, int BS, int k_eb, int v_eb,
                           const int32_t *cu_q_lens, const int32_t *context_lens,
                           const int32_t *block_tables, int max_blocks, int B,
                           float k_scale, float v_scale, double sm_scale,
                           const int64_t *sel, int64_t n_sel, double *out)
{
    const int g = Hq / Hkv;
    int maxL = 0;
    for (int b = 0; b < B; ++b) {
        const int L = context_lens[b] + cu_q_lens[b + 1] - cu_q_lens[b];
        if (L > maxL)
            maxL = L;
    }
    float *kd = (float *)malloc(sizeof(float) * ((size_t)maxL * D + 1));
    float *vd = (float *)malloc(sizeof(float) * ((size_t)maxL * D + 1));
    double *scores = (double *)malloc(sizeof(double) * ((size_t)maxL + 1));
    if (!kd || !vd || !scores) {
        free(kd); free(vd); free(scores);
        return -1;
    }
    const int64_t total_q = cu_q_lens[B];
    const int64_t total = sel ? n_sel : total_q * Hq;
    int cached_b = -1, cached_h = -1;
    for (int64_t i = 0; i < total; ++i) {
        const int64_t qi = sel ? sel[2 * i] : i / Hq;
        const int h = sel ? (int)sel[2 * i + 1] : (int)(i % Hq);
        int b = 0;
        while (b + 1 < B && cu_q_lens[b + 1] <= qi)
            ++b;
        const int pos = context_lens[b] + (int)(qi - cu_q_lens[b]);
        const int L = context_lens[b] + cu_q_lens[b + 1] - cu_q_lens[b];
        const int kvh = h / g;
        if (b != cached_b || kvh != cached_h) {
            orc_gather_typed(k_pool, v_pool, Hkv, D, BS, k_eb, v_eb, block_tables + (int64_t)b * max_blocks,
                             L, kvh, k_scale, v_scale, kd, vd);
            cached_b = b;
            cached_h = kvh;
        }
        orc_attend_row(q + (qi * Hq + h) * D, kd, vd, pos + 1, D, sm_scale, scores,
                       out + (qi * Hq + h) * D);
    }
    free(kd); free(vd); free(scores);
    return 0;
}

int orc_prefill_attn(const uint16_t *q, int Hq,
                     const uint8_t *k_pool, const uint8_t *v_pool,
                     int Hkv, int D, int BS,
                     const int32_t *cu_q_lens, const int32_t *context_lens,
                     const int32_t *block_tables, int max_blocks, int B,
                     float k_scale, float v_scale, double sm_scale,
                     const int64_t *sel, int64_t n_sel, double *out)
{
    return orc_prefill_attn_typed(q, Hq, k_pool, v_pool, Hkv, D, BS, 1, 1, cu_q_lens, context_lens,
                                  block_tables, max_blocks, B, k_scale, v_scale, sm_scale, sel, n_sel, out);
}

/* ------------------------------------------------------------------ */
/* K-shift [P1, build_rope_shift excludes F8_E4M3 from the in-place     */
/* rope; check_fp8_context_shift: expected bytes are                    */
/* quantize(rope(to_float(bytes), shift)) with no scale applied].       */
/* Rotary pair i (0 <= i < rot/2) turns by angle delta * theta^(-2i/rot),*/
/* with cos and sin taken in double and rounded to fp32.  Pairs are     */
/* (i, i + rot/2) for the NEOX style (style 1) and (2i, 2i+1) for the   */
/* NORM style (style 0).  The rotation is done in fp64 on the decoded   */
/* values and rounded to fp32 before encoding.  A pair holding a NaN    */
/* code becomes the NaN code 0x7F in both places (the sign of an        */
/* arithmetic NaN is not defined by IEEE 754).  Dims >= rot untouched.  */
/* Slots < 0 or at or past the pool's NB * BS slots are skipped.        */
/* ------------------------------------------------------------------ */
void orc_rope_table(int rot_dim, int delta, float theta, float *cos_out, float *sin_out)
{
    for (int i = 0; i < rot_dim / 2; ++i) {
        const double omega = pow((double)theta, -2.0 * (double)i / (double)rot_dim);
        const double angle = (double)delta * omega;
        cos_out[i] = (float)cos(angle);
        sin_out[i] = (float)sin(angle);
    }
}

uint16_t orc_f32_to_bf16_rne(float x);

/* Rotate every rotary pair of one slot's K rows (all kv-heads) by the
 * angles whose fp32 cos/sin are cs[p], sn[p].  eb = 1: E4M3 codes (a pair
 * holding a NaN code becomes the NaN code in both places); eb = 2: bf16
 * values [P3, "What turning it on costs": the bf16 twin of the cache],
 * rotated the same way and rounded to fp32 then to the nearest bf16 (a pair
 * holding a NaN becomes the quiet NaN 0x7FC0 in both places). */
static void orc_kshift_slot(void *pool, int eb, int Hkv, int D, int BS, int64_t slot,
                            const float *cs, const float *sn, int rot_dim, int style)
{
    const int64_t block = slot / BS;
    const int t = (int)(slot % BS);
    for (int h = 0; h < Hkv; ++h) {
        const int64_t base = orc_tile_base(block, h, Hkv, BS, D);
        for (int p = 0; p < rot_dim / 2; ++p) {
            const int d0 = style == 1 ? p : 2 * p;
            const int d1 = style == 1 ? p + rot_dim / 2 : 2 * p + 1;
            const int64_t e0 = base + orc_k_tile_offset(t, d0, BS, D);
            const int64_t e1 = base + orc_k_tile_offset(t, d1, BS, D);
            float x0, x1;
            if (eb == 1) {
                x0 = orc_e4m3_decode(((uint8_t *)pool)[e0]);
                x1 = orc_e4m3_decode(((uint8_t *)pool)[e1]);
            } else {
                x0 = orc_bf16_to_f32(((uint16_t *)pool)[e0]);
                x1 = orc_bf16_to_f32(((uint16_t *)pool)[e1]);
            }
            if (isnan(x0) || isnan(x1)) {
                if (eb == 1) {
                    ((uint8_t *)pool)[e0] = 0x7F;
                    ((uint8_t *)pool)[e1] = 0x7F;
                } else {
                    ((uint16_t *)pool)[e0] = 0x7FC0;
                    ((uint16_t *)pool)[e1] = 0x7FC0;
                }
                continue;
            }
            const double c = cs[p], s = sn[p];
            const double r0 = (double)x0 * c - (double)x1 * s;
            const double r1 = (double)x0 * s + (double)x1 * c;
            if (eb == 1) {
                ((uint8_t *)pool)[e0] = orc_e4m3_encode((float)r0);
                ((uint8_t *)pool)[e1] = orc_e4m3_encode((float)r1);
            } else {
                ((uint16_t *)pool)[e0] = orc_f32_to_bf16_rne((float)r0);
                ((uint16_t *)pool)[e1] = orc_f32_to_bf16_rne((float)r1);
            }
        }
    }
}

int orc_kshift_typed(void *k_pool, int eb, int Hkv, int D, int BS, int64_t NB,
                     const int64_t *slots, int64_t n_slots,
                     int delta, float theta, int rot_dim, int style)
{
    float *cs = (float *)malloc(sizeof(float) * (size_t)(rot_dim / 2 + 1));
    float *sn = (float *)malloc(sizeof(float) * (size_t)(rot_dim / 2 + 1));
    if (!cs || !sn) {
        free(cs); free(sn);
        return -1;
    }
    orc_rope_table(rot_dim, delta, theta, cs, sn);
    for (int64_t i = 0; i < n_slots; ++i) {
        const int64_t slot = slots[i];
        if (slot < 0 || slot >= NB * BS)
            continue;
        orc_kshift_slot(k_pool, eb, Hkv, D, BS, slot, cs, sn, rot_dim, style);
    }
    free(cs); free(sn);
    return 0;
}

int orc_kshift(uint8_t *k_pool, int Hkv, int D, int BS, int64_t NB,
               const int64_t *slots, int64_t n_slots,
               int delta, float theta, int rot_dim, int style)
{
    return orc_kshift_typed(k_pool, 1, Hkv, D, BS, NB, slots, n_slots, delta, theta, rot_dim, style);
}

/* Per-slot deltas [P1, tests/test-fp8.cpp check_fp8_context_shift: the
 * shift tensor holds one position offset per cache cell, so cells move by
 * different amounts in one pass]: slot slots[i] turns by deltas[i], each
 * exactly as orc_kshift would turn it alone.  The angle table is rebuilt
 * whenever the delta changes from the previous slot's. */
int orc_kshift_per_slot_typed(void *k_pool, int eb, int Hkv, int D, int BS, int64_t NB,
                              const int64_t *slots, const int32_t *deltas, int64_t n_slots,
                              float theta, int rot_dim, int style)
{
    float *cs = (float *)malloc(sizeof(float) * (size_t)(rot_dim / 2 + 1));
    float *sn = (float *)malloc(sizeof(float) * (size_t)(rot_dim / 2 + 1));
    if (!cs || !sn) {
        free(cs); free(sn);
        return -1;
    }
    int have = 0;
    int32_t current = 0;
    for (int64_t i = 0; i < n_slots; ++i) {
        const int64_t slot = slots[i];
        if (slot < 0 || slot >= NB * BS)
            continue;
        if (!have || deltas[i] != current) {
            current = deltas[i];
            orc_rope_table(rot_dim, current, theta, cs, sn);
            have = 1;
        }
        orc_kshift_slot(k_pool, eb, Hkv, D, BS, slot, cs, sn, rot_dim, style);
    }
    free(cs); free(sn);
    return 0;
}

int orc_kshift_per_slot(uint8_t *k_pool, int Hkv, int D, int BS, int64_t NB,
                        const int64_t *slots, const int32_t *deltas, int64_t n_slots,
                        float theta, int rot_dim, int style)
{
    return orc_kshift_per_slot_typed(k_pool, 1, Hkv, D, BS, NB, slots, deltas, n_slots, theta, rot_dim,
                                     style);
}

/* ------------------------------------------------------------------ */
/* Scale calibration.  [P3, "Unreached and owed"] names runtime KV-scale */
/* calibration as not built there; its benchmark configuration sets a    */
/* per-tensor scale of amax / 448, which maps the tensor's largest        */
/* magnitude onto E4M3's largest finite value (448, [P2]                  */
/* ggml_fp32_to_f8_e4m3 saturation bound).  This oracle follows that      */
/* rule: amax is the largest |x| over the bf16 elements seen so far (any  */
/* NaN makes it NaN), the fp32 scale is the correctly rounded quotient    */
/* amax / 448, and a bf16 scale is that fp32 value rounded to the nearest */
/* bf16, ties to even.                                                    */
/* ------------------------------------------------------------------ */

/* Running amax over rows [rows][row_elems] with a row stride, starting
 * from `amax` (0 for a fresh tensor).  NaN is returned as quiet NaN. */
float orc_amax_bf16(const uint16_t *x, int64_t rows, int64_t row_elems, int64_t stride, float amax)
{
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t e = 0; e < row_elems; ++e) {
            const float a = fabsf(orc_bf16_to_f32(x[r * stride + e]));
            if (isnan(a) || isnan(amax))
                amax = NAN;
            else if (a > amax)
                amax = a;
        }
    }
    return amax;
}

/* fp32 scale from amax: one IEEE division (NaN in, NaN out). */
float orc_scale_from_amax(float amax) { return amax / 448.0f; }

/* Nearest bf16 to an fp32 value, ties to the even significand; values at
 * or past the midpoint between the largest finite bf16 and 2^128 go to
 * infinity; NaN gives the quiet NaN 0x7FC0.  Written from the definition:
 * the two bf16 neighbours of x (truncation and the next value away from
 * zero) are compared by their distance to x in fp64, which holds all of
 * them exactly. */
uint16_t orc_f32_to_bf16_rne(float x)
{
    if (isnan(x))
        return 0x7FC0;
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0)
        return lo;
    const uint16_t hi = (uint16_t)(lo + 1);
    const double vx = (double)x;
    const double vlo = (double)orc_bf16_to_f32(lo);
    double vhi;
    if ((hi & 0x7FFFu) == 0x7F80u)
        vhi = copysign(ldexp(1.0, 128), vx);   /* the step past the largest finite value */
    else
        vhi = (double)orc_bf16_to_f32(hi);
    const double dlo = fabs(vx - vlo), dhi = fabs(vhi - vx);
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1u) ? hi : lo;
}

/* ------------------------------------------------------------------ */
/* Bytes of one block for one layer, K and V together [P3, W3 summary:  */
/* KVBytesPerBlock is exactly halved for one-byte elements].            */
/* ------------------------------------------------------------------ */
int64_t orc_kv_bytes_per_block(int BS, int Hkv, int D, int elem_bytes)
{
    return 2 * (int64_t)BS * Hkv * D * elem_bytes;
}
