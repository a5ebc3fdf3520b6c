/*
 * ra_oracle.c -- plain CPU oracle for the RotateAttention INT4 attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant generator with the HIP library; the two are written
 * independently from the same method description.
 *
 * Source pages (cited by title and section):
 *  [RA]  "RotateAttention: RoPE-Aware Rotation and Range Rectification for INT4
 *        Quantized Attention in Video Generation" -- pith.science review page:
 *        abstract, Sec. 3 / Fig. 2 (3D RoPE segments), Sec. 4.1 / Fig. 3
 *        (Interleaved and Half rotations, H2 blocks, orthogonality argument),
 *        Sec. 4.2 (range-optimized P: scale 15, zero-point -8; the symmetric
 *        P quantization it replaces, which leaves half of the INT4 codes
 *        unused, as the ablation mode), Sec. 5.1
 *        (FP16 step/block fallback), free-parameter ledger.
 *  [PARO] "PAROAttention" review page -- 64-token blocks aligned with the
 *        FlashAttention tile (precedent for the Q/K quantization block).
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * Every float operation below is IEEE binary32 (or binary64 where stated) in
 * the order written; -ffp-contract=off keeps a*b+c from being fused.
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function that implements it.  Integer quantities (codes, scores, P codes,
 * PV sums) are exact; the final normalisation is carried in binary64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { ORA_ROT_NONE = 0, ORA_ROT_INTERLEAVED = 1, ORA_ROT_HALF = 2, ORA_ROT_FULL = 3 };
enum { ORA_BLOCK = 64 };      /* tokens per Q/K scale block and per key step */
enum { ORA_CODE_MAX = 7 };    /* symmetric INT4 codes in [-7, 7] */
enum { ORA_MAX_D = 256 };

int ora_block(void) { return ORA_BLOCK; }

void ora_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }
int ora_get_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* 3D RoPE tables ([RA] Sec. 3, Fig. 2: head dims split into frame / height /
 * width segments, each rotated by its own axis coordinate).
 * Reading: adjacent pairs (2j, 2j+1) inside a segment of even length L;
 * frequency theta^(-2j/L); positions start at 0.  With the Interleaved
 * rotation folded into the RoPE angles ([RA] Sec. 4.1), each pair angle
 * gains +pi/4, i.e. the 2x2 block R(pi/4) is composed with R(pos*freq).
 * Angles in binary64, cos/sin rounded once to binary32.                     */
static void seg_table(int npos, int L, double theta, int interleaved,
                      float *cs, float *sn)
{
    int half = L / 2;
    for (int p = 0; p < npos; ++p) {
        for (int j = 0; j < half; ++j) {
            double expo = (double)(-2 * j) / (double)L;
            double freq = pow(theta, expo);
            double ang = (double)p * freq;
            if (interleaved) {
                double quarter = M_PI / 4.0;
                ang = ang + quarter;
            }
            cs[p * half + j] = (float)cos(ang);
            sn[p * half + j] = (float)sin(ang);
        }
    }
}

/* Exported for table-equality tests: cos/sin of segment s (0 frame, 1 height,
 * 2 width) laid out [pos][pair]. */
int ora_rope_table(int npos, int L, double theta, int rot, float *cs, float *sn)
{
    if (npos < 1 || L < 2 || (L & 1)) return -1;
    seg_table(npos, L, theta, rot == ORA_ROT_INTERLEAVED, cs, sn);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Orthonormal Walsh-Hadamard transform of one row v[D] (D a power of two) in
 * binary32, in this order: butterfly stages h = 1, 2, 4, ..., D/2, each pair
 * (i, i + h) with bit h of i clear becoming (v_i + v_{i+h}, v_i - v_{i+h});
 * then one multiply of every element by f32(1/sqrt(D)).  Used for the full
 * rotation of Q/K and the V-side Hadamard.                                  */
static void fwht_f32(float *v, int D)
{
    const float sc = (float)(1.0 / sqrt((double)D));
    for (int h = 1; h < D; h <<= 1)
        for (int i = 0; i < D; ++i)
            if (!(i & h)) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    for (int i = 0; i < D; ++i) v[i] = v[i] * sc;
}

/* ------------------------------------------------------------------------ */
/* RoPE + RoPE-aware rotation of one token row x[D] -> y[D] (binary32).
 * Pair rotation (a, b) -> (a c - b s, a s + b c), each product rounded, then
 * the sum/difference rounded.
 * Half rotation ([RA] Sec. 4.1 / Fig. 3: dim i of a segment of length L
 * meets dim i + L/2 of the same segment; block H2 = (1/sqrt2)[[1,1],[1,-1]] by the
 * free-parameter ledger) is applied after RoPE:
 *   u' = (u + w) r,  w' = (u - w) r,  r = binary32(1/sqrt2).
 * Full rotation (the dense comparator of [RA] Figs. 4-6, which rotates all D
 * dimensions of the head at once; reading: the orthonormal Walsh-Hadamard
 * matrix) is applied to the whole RoPE'd row: y = fwht(RoPE(x)).             */
static void rotate_row(const float *x, float *y, int D, const int *seg,
                       const int *pos, float *const *cs, float *const *sn,
                       int rot)
{
    float tmp[ORA_MAX_D];
    const float r = (float)M_SQRT1_2;
    int off = 0;
    for (int s = 0; s < 3; ++s) {
        int L = seg[s], half = L / 2;
        const float *c = cs[s] + (size_t)pos[s] * half;
        const float *sv = sn[s] + (size_t)pos[s] * half;
        for (int j = 0; j < half; ++j) {
            float a = x[off + 2 * j], b = x[off + 2 * j + 1];
            float ac = a * c[j], bs = b * sv[j];
            float as = a * sv[j], bc = b * c[j];
            tmp[off + 2 * j] = ac - bs;
            tmp[off + 2 * j + 1] = as + bc;
        }
        if (rot == ORA_ROT_HALF) {
            for (int i = 0; i < half; ++i) {
                float u = tmp[off + i], w = tmp[off + i + half];
                float sum = u + w, dif = u - w;
                y[off + i] = sum * r;
                y[off + i + half] = dif * r;
            }
        } else {
            for (int i = 0; i < L; ++i) y[off + i] = tmp[off + i];
        }
        off += L;
    }
    if (rot == ORA_ROT_FULL) fwht_f32(y, D);
}

/* x, y: [B, N, H, D] binary32.  Token n -> (f, h, w) in row-major order with
 * w fastest (N = F*Hh*W).  rot: 0 none, 1 interleaved (merged), 2 half,
 * 3 full (D must be a power of two). */
int ora_rope_rotate(const float *x, float *y, int B, int H, int D,
                    int F, int Hh, int W, const int *seg, double theta, int rot)
{
    if (D > ORA_MAX_D || seg[0] + seg[1] + seg[2] != D) return -1;
    for (int s = 0; s < 3; ++s) if (seg[s] < 2 || (seg[s] & 1)) return -1;
    if (rot < 0 || rot > 3 || (rot == ORA_ROT_FULL && (D & (D - 1)))) return -1;
    int dims[3] = {F, Hh, W};
    float *cs[3], *sn[3];
    for (int s = 0; s < 3; ++s) {
        size_t n = (size_t)dims[s] * (seg[s] / 2);
        cs[s] = (float *)malloc(n * sizeof(float));
        sn[s] = (float *)malloc(n * sizeof(float));
        seg_table(dims[s], seg[s], theta, rot == ORA_ROT_INTERLEAVED, cs[s], sn[s]);
    }
    long N = (long)F * Hh * W;
    #pragma omp parallel for schedule(static)
    for (long bn = 0; bn < (long)B * N; ++bn) {
        long n = bn % N;
        int pos[3];
        pos[0] = (int)(n / ((long)Hh * W));
        pos[1] = (int)((n / W) % Hh);
        pos[2] = (int)(n % W);
        for (int h = 0; h < H; ++h) {
            size_t o = ((size_t)bn * H + h) * D;
            rotate_row(x + o, y + o, D, seg, pos, cs, sn, rot);
        }
    }
    for (int s = 0; s < 3; ++s) { free(cs[s]); free(sn[s]); }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Symmetric INT4 quantizer of one group ([RA] abstract: INT4 Q and K).
 * Reading: codes in [-7, 7]; scale = amax / 7; code = RNE(x * (7 / amax)),
 * clamped; an all-zero group gets scale 0 and codes 0.                     */
static float group_scale(float amax, float *inv)
{
    if (amax == 0.0f) { *inv = 0.0f; return 0.0f; }
    *inv = 7.0f / amax;
    return amax / 7.0f;
}

static int8_t quant_one(float x, float inv)
{
    float t = x * inv;
    float q = rintf(t);
    if (q > (float)ORA_CODE_MAX) q = (float)ORA_CODE_MAX;
    if (q < -(float)ORA_CODE_MAX) q = -(float)ORA_CODE_MAX;
    return (int8_t)q;
}

/* Q/K: one scale per (b, h, 64-token block) over the valid tokens x all D
 * channels (reading of the per-(head, 64-token block) granularity; [PARO]
 * uses the same 64-block tile).  y: [B, N, H, D]; codes: [B, H, N, D];
 * scales: [B, H, ceil(N/64)]. */
int ora_quant_qk(const float *y, int B, int N, int H, int D,
                 int8_t *codes, float *scales)
{
    int nblk = (N + ORA_BLOCK - 1) / ORA_BLOCK;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            for (int blk = 0; blk < nblk; ++blk) {
                int n0 = blk * ORA_BLOCK;
                int n1 = n0 + ORA_BLOCK < N ? n0 + ORA_BLOCK : N;
                float amax = 0.0f;
                for (int n = n0; n < n1; ++n)
                    for (int d = 0; d < D; ++d) {
                        float a = fabsf(y[(((size_t)b * N + n) * H + h) * D + d]);
                        if (a > amax) amax = a;
                    }
                float inv;
                float s = group_scale(amax, &inv);
                scales[((size_t)b * H + h) * nblk + blk] = s;
                for (int n = n0; n < n1; ++n)
                    for (int d = 0; d < D; ++d) {
                        float v = y[(((size_t)b * N + n) * H + h) * D + d];
                        codes[(((size_t)b * H + h) * N + n) * D + d] =
                            (s == 0.0f) ? 0 : quant_one(v, inv);
                    }
            }
        }
    return 0;
}

/* V: one scale per (b, h, channel) over all N tokens (per-channel symmetric
 * INT4).  v: [B, N, H, D]; codes: [B, H, N, D]; scales: [B, H, D]. */
int ora_quant_v(const float *v, int B, int N, int H, int D,
                int8_t *codes, float *scales)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            for (int d = 0; d < D; ++d) {
                float amax = 0.0f;
                for (int n = 0; n < N; ++n) {
                    float a = fabsf(v[(((size_t)b * N + n) * H + h) * D + d]);
                    if (a > amax) amax = a;
                }
                float inv;
                float s = group_scale(amax, &inv);
                scales[((size_t)b * H + h) * D + d] = s;
                for (int n = 0; n < N; ++n) {
                    float x = v[(((size_t)b * N + n) * H + h) * D + d];
                    codes[(((size_t)b * H + h) * N + n) * D + d] =
                        (s == 0.0f) ? 0 : quant_one(x, inv);
                }
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* V-side Hadamard ([RA] summary and reproducibility notes: a standard
 * Hadamard transform fused offline into V).  Reading: each V row is
 * multiplied by the orthonormal Walsh-Hadamard matrix H = H_D / sqrt(D)
 * (Sylvester order) before the per-channel quantization, and the attention
 * output row by the same matrix (symmetric and its own inverse), so the
 * operator still returns attention(Q, K, V); in a model the second product
 * would be folded into the output projection.  Binary32, in this order:
 * butterfly stages h = 1, 2, 4, ..., D/2, each pair (i, i + h) with bit h of
 * i clear becoming (x_i + x_{i+h}, x_i - x_{i+h}); then one multiply of every
 * element by f32(1/sqrt(D)).                                               */
int ora_fwht_rows(float *x, int64_t rows, int D)
{
    if (D < 1 || (D & (D - 1))) return -1;
    for (int64_t r = 0; r < rows; ++r) fwht_f32(x + r * D, D);
    return 0;
}

/* The same transform in binary64 (the output side of the float path). */
static void fwht_f64(double *v, int D)
{
    for (int h = 1; h < D; h <<= 1)
        for (int i = 0; i < D; ++i)
            if (!(i & h)) {
                double a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    const double sc = 1.0 / sqrt((double)D);
    for (int i = 0; i < D; ++i) v[i] *= sc;
}

/* ------------------------------------------------------------------------ */
/* Range-optimized P map ([RA] Sec. 4.2 and the free-parameter ledger: fixed
 * scale 15 and zero-point -8, so p in [0, 1] covers the whole signed INT4
 * range [-8, 7]; abstract: p = exp(QK - max QK)).
 *
 * With the exponent d = log2 p (a binary32 value <= 0 in the attention
 * below), code = round(15 * 2^d) - 8, rounding half up; u = code + 8 is in
 * [0, 15].  The rounding is decided exactly by counting thresholds:
 *   u = #{k in 0..14 : d >= T_k},
 * where T_k is the smallest binary32 value with 15 * 2^T_k >= k + 1/2 in
 * exact arithmetic (15 * 2^d >= k + 1/2 holds exactly for the d >= T_k).
 *
 * Symmetric P quantization (the baseline [RA] Sec. 4.2 replaces: P >= 0 on
 * a symmetric INT4 grid reaches only the codes 0..7): code = u = round(7 p)
 * in [0, 7], zero-point 0; thresholds as above with 7 in place of 15.
 * pmap_scale(mode) is the scale: 15 for mode 0, 7 for mode 1.
 *
 * The thresholds start from the binary64 logarithm and are moved one
 * binary32 step at a time until P * 2^d >= k + 1/2 holds at T_k and fails
 * one step below; the test uses exp2l (64-bit significand), far finer than
 * the distance of any binary32 value from the exact boundary.               */
static int pmap_scale(int p_mode) { return p_mode ? 7 : 15; }

static int meets(float d, int P, int k)
{
    return (long double)P * exp2l((long double)d) >= (long double)k + 0.5L;
}

int ora_pmap_thresholds_p(int p_mode, float *T)
{
    if (p_mode != 0 && p_mode != 1) return -1;
    const int P = pmap_scale(p_mode);
    for (int k = 0; k < P; ++k) {
        float d = (float)log2((double)(2 * k + 1) / (2.0 * P));
        while (!meets(d, P, k)) d = nextafterf(d, INFINITY);
        while (meets(nextafterf(d, -INFINITY), P, k)) d = nextafterf(d, -INFINITY);
        T[k] = d;
    }
    return 0;
}

static int pmap_u(float d, const float *T, int P)
{
    int u = 0;
    for (int k = 0; k < P; ++k)
        if (d >= T[k]) ++u;
    return u;
}

/* Vectorised form for tests: u[i] = map(d[i]) (u = code + zero-point). */
int ora_pmap_p(const float *d, int64_t n, int p_mode, uint8_t *u)
{
    float T[15];
    if (ora_pmap_thresholds_p(p_mode, T)) return -1;
    const int P = pmap_scale(p_mode);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) u[i] = (uint8_t)pmap_u(d[i], T, P);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* INT4 attention for one (b, h) slice, on selected query rows.
 *
 * Online softmax over key steps of 64 keys in ascending order (reading of
 * p = exp(QK - max(QK)) [RA abstract] inside a FlashAttention loop: the max
 * is the running max, updated once per 64-key step).  Exponents are in log2
 * units, so p = 2^d.
 *   scores     S = sum_d qhat kc                               (exact int)
 *   c          = f32(f32(s_q s_k) * alpha),
 *              alpha = f32(log2(e) * softmax_scale)
 *   step max   m_t = max over the step's keys of f32(S_j c);  m = max(m, m_t)
 *              (m starts at -inf)
 *   exponent   d_j = f32(S_j c - m): the exact value S_j c - m rounded once
 *              to binary32 (d_j <= 0 up to half an ulp of m)
 *   P code     u_j = round(15 * 2^d_j) by the thresholds above; code = u - 8
 *              (p_mode 1, symmetric: u_j = round(7 * 2^d_j), code = u)
 *   sums       U = sum_j u_j;  num_c = sum_j u_j vhat_jc;
 *              PV_c = sum_j code_j vhat_jc = num_c - 8 sum_j vhat_jc
 *   float path (binary64):  beta = 2^(m_old - m),
 *              A = A beta + num,  L = L beta + U,  o = A s_v / L,
 *              times H when the V codes are of V H (v_hadamard).
 * The dequantized P is u/15 (u/7), so the scale cancels in A/L: the row is
 * normalised by the sum of its quantized probabilities.
 *
 * qc, kc, vc: [N, D] int8 codes of this (b, h); sq, sk: [ceil(N/64)];
 * sv: [D].  rows: nrows query indices; o: [nrows, D] binary64.
 * m_out (optional): final running max per selected row (binary32).
 * Tile dump (optional, dbg_kb >= 0): for selected rows, after key step dbg_kb,
 * s_int[r*64 + j], p_code[r*64 + j] (-zero-point for keys >= N),
 * d_val[r*64 + j] (the exponent d, -inf for keys >= N), pv_int[r*D + c],
 * m_after[r], indexed by r = position of the row in `rows`.                 */
int ora_attention_head(const int8_t *qc, const float *sq,
                       const int8_t *kc, const float *sk,
                       const int8_t *vc, const float *sv,
                       int N, int D, double softmax_scale, int p_mode, int v_hadamard,
                       const int32_t *rows, int nrows, double *o, float *m_out,
                       int dbg_kb, int32_t *s_int, int8_t *p_code, float *d_val,
                       int32_t *pv_int, float *m_after)
{
    if (D > ORA_MAX_D || N < 1) return -1;
    float T[15];
    if (ora_pmap_thresholds_p(p_mode, T)) return -1;
    const int P = pmap_scale(p_mode), zp = p_mode ? 0 : 8;
    const float alpha = (float)(M_LOG2E * softmax_scale);
    int nkb = (N + ORA_BLOCK - 1) / ORA_BLOCK;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int i = rows[r];
        int qb = i / ORA_BLOCK;
        const int8_t *qi = qc + (size_t)i * D;
        float m = -INFINITY;
        double A[ORA_MAX_D], L = 0.0;
        int32_t S[ORA_BLOCK], u[ORA_BLOCK];
        float dv[ORA_BLOCK];
        int64_t num[ORA_MAX_D];
        for (int c = 0; c < D; ++c) A[c] = 0.0;

        for (int kb = 0; kb < nkb; ++kb) {
            int j0 = kb * ORA_BLOCK;
            int nj = (j0 + ORA_BLOCK < N ? ORA_BLOCK : N - j0);
            float sqk = sq[qb] * sk[kb];
            float c = sqk * alpha;

            float mnew = m;
            for (int j = 0; j < nj; ++j) {
                const int8_t *kj = kc + (size_t)(j0 + j) * D;
                int64_t acc = 0;
                for (int d = 0; d < D; ++d) acc += (int64_t)qi[d] * kj[d];
                S[j] = (int32_t)acc;
                float t = (float)((double)S[j] * (double)c);   /* exact product, one rounding */
                if (t > mnew) mnew = t;
            }

            int64_t U = 0;
            for (int c2 = 0; c2 < D; ++c2) num[c2] = 0;
            for (int j = 0; j < nj; ++j) {
                dv[j] = fmaf((float)S[j], c, -mnew);           /* S c - m, one rounding */
                u[j] = pmap_u(dv[j], T, P);
                U += u[j];
                const int8_t *vj = vc + (size_t)(j0 + j) * D;
                for (int c2 = 0; c2 < D; ++c2) num[c2] += (int64_t)u[j] * vj[c2];
            }
            double beta = exp2((double)m - (double)mnew);
            for (int c2 = 0; c2 < D; ++c2) A[c2] = A[c2] * beta + (double)num[c2];
            L = L * beta + (double)U;
            m = mnew;

            if (kb == dbg_kb) {
                for (int j = 0; j < ORA_BLOCK; ++j) {
                    if (s_int) s_int[(size_t)r * ORA_BLOCK + j] = j < nj ? S[j] : 0;
                    if (p_code) p_code[(size_t)r * ORA_BLOCK + j] =
                        (int8_t)(j < nj ? u[j] - zp : -zp);
                    if (d_val) d_val[(size_t)r * ORA_BLOCK + j] = j < nj ? dv[j] : -INFINITY;
                }
                if (pv_int)
                    for (int c2 = 0; c2 < D; ++c2) {
                        int64_t acc = 0;
                        for (int j = 0; j < nj; ++j)
                            acc += (int64_t)(u[j] - zp) * vc[(size_t)(j0 + j) * D + c2];
                        pv_int[(size_t)r * D + c2] = (int32_t)acc;
                    }
                if (m_after) m_after[r] = m;
            }
        }
        for (int c2 = 0; c2 < D; ++c2)
            o[(size_t)r * D + c2] = A[c2] * (double)sv[c2] / L;
        if (v_hadamard) fwht_f64(o + (size_t)r * D, D);   /* back from the rotated V basis */
        if (m_out) m_out[r] = m;
    }
    return 0;
}

/* Integer digests of every P code of selected rows over all key steps:
 * dig_sum[r] = sum_j u_j and dig_hash[r] = sum_j u_j * h(j) mod 2^32 with
 * h(j) = (2654435761 * (j + 1)) mod 2^32, j the key index, u = code +
 * zero-point.  A compact fingerprint of a whole row of codes for comparing
 * long rows.  Same arithmetic as ora_attention_head; m_out as there.       */
int ora_code_digests(const int8_t *qc, const float *sq, const int8_t *kc, const float *sk,
                     int N, int D, double softmax_scale, int p_mode,
                     const int32_t *rows, int nrows, uint32_t *dig_sum, uint32_t *dig_hash,
                     float *m_out)
{
    if (D > ORA_MAX_D || N < 1) return -1;
    float T[15];
    if (ora_pmap_thresholds_p(p_mode, T)) return -1;
    const int P = pmap_scale(p_mode);
    const float alpha = (float)(M_LOG2E * softmax_scale);
    int nkb = (N + ORA_BLOCK - 1) / ORA_BLOCK;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
        int i = rows[r];
        int qb = i / ORA_BLOCK;
        const int8_t *qi = qc + (size_t)i * D;
        float m = -INFINITY;
        int32_t S[ORA_BLOCK];
        uint32_t ds = 0, dh = 0;
        for (int kb = 0; kb < nkb; ++kb) {
            int j0 = kb * ORA_BLOCK;
            int nj = (j0 + ORA_BLOCK < N ? ORA_BLOCK : N - j0);
            float c = (sq[qb] * sk[kb]) * alpha;
            float mnew = m;
            for (int j = 0; j < nj; ++j) {
                const int8_t *kj = kc + (size_t)(j0 + j) * D;
                int64_t acc = 0;
                for (int d = 0; d < D; ++d) acc += (int64_t)qi[d] * kj[d];
                S[j] = (int32_t)acc;
                float t = (float)((double)S[j] * (double)c);
                if (t > mnew) mnew = t;
            }
            for (int j = 0; j < nj; ++j) {
                uint32_t u = (uint32_t)pmap_u(fmaf((float)S[j], c, -mnew), T, P);
                ds += u;
                dh += u * (2654435761u * (uint32_t)(j0 + j + 1));
            }
            m = mnew;
        }
        dig_sum[r] = ds;
        dig_hash[r] = dh;
        if (m_out) m_out[r] = m;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Mixed-precision schedule ([RA] Sec. 5.1: FP16 on the first/last sampling
 * steps and the first/last DiT blocks, INT4 elsewhere).  Reading: a call runs
 * at full precision when its step OR its block is in a head/tail set.
 * Returns 1 for the full-precision path, 0 for INT4.                       */
int ora_schedule_full_precision(int steps_head, int steps_tail,
                                int blocks_head, int blocks_tail,
                                int step, int n_steps, int block, int n_blocks)
{
    int step_fp = step < steps_head || step >= n_steps - steps_tail;
    int block_fp = block < blocks_head || block >= n_blocks - blocks_tail;
    return step_fp || block_fp;
}
