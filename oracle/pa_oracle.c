/*
 * Paged-attention decode oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU product path never
 * links, loads or calls it, and it shares no code, header, table or constant
 * with the GPU path.
 *
 * What it computes (ROCm/aiter PR #7092 "pa_decode: zero V rows past the
 * context before PV", section "Root cause"; ROCm/aiter PR #7056 "pa_decode:
 * MXFP4 K/V in the shared PA tile kernel", section "Summary"):
 *
 *   for every sequence b, query token i < qlen and query head h:
 *     kvh   = h / q_per_kv                      (heads grouped contiguously)
 *     for t < L_b:  page = block_tables[b][t / page_size], slot = t % page_size
 *                   s_t  = softmax_scale * dot(qhat, deq_K(page, kvh, slot))
 *     pi_t  = exp(s_t - max s) / sum_u exp(s_u - max s)
 *     o[d]  = sum_t pi_t * deq_V(page, kvh, slot)[d]
 *   L_b = 0 gives o = 0.
 *
 * Tokens t >= L_b and block-table columns >= ceil(L_b / page_size) are never
 * read, so whatever bytes sit in rows no sequence owns cannot reach o.
 * All arithmetic is fp64. Each format decoder below is written from the
 * format's own definition (OCP 8-bit floating point e4m3fn; OCP Microscaling
 * e2m1 elements with e8m0 block scales, one per 32 elements along head_dim;
 * bfloat16 as the top half of an IEEE binary32).
 *
 * Readings where the pages leave a step open are listed in the design notes
 * of the repository; the ones that change arithmetic here are:
 *   - softmax_scale defaults to 1/sqrt(head_dim) when the caller passes 0;
 *   - for an MXFP4 cache with a bf16 query, every (b, i, h) query row is
 *     quantized to e4m3 with a power-of-two scale 2^e, e the smallest integer
 *     with max|q| <= 448 * 2^e (e = 0 for an all-zero row), round to nearest
 *     even with saturation to +-448, and the logits are multiplied by 2^e;
 *   - an e4m3 query is used as stored, with unit scale;
 *   - with qlen > 1 every query row attends to all of [0, L_b) unless the
 *     problem asks for causal attention;
 *   - causal attention (query tokens are the last qlen positions of the
 *     sequence, their K/V already in the cache): query token i attends to
 *     t < e_i = L_b - qlen + i + 1; otherwise e_i = L_b;
 *   - a sliding window of W > 0 tokens keeps t >= e_i - W as well, so query
 *     token i attends to [max(0, e_i - W), e_i); an empty range gives o = 0.
 *
 * The MXFP4 cache write (oracle_write_kv_mxfp4) encodes each 32-element
 * block with the OCP Microscaling conversion; its readings are stated there.
 *
 * Parity pins live in the test suite: brute-force dense attention, softmax
 * normalisation, context_len = 1, split/merge invariance, page-permutation
 * invariance, decoder tables checked against library casts, and for the
 * encoder a hand-derived rounding table, exact round trips of representable
 * blocks and the scale range the conversion guarantees.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- problem description (the oracle's own; not shared with the GPU path) ---- */
typedef struct {
    int32_t num_seqs, qlen, num_kv_heads, q_per_kv, head_dim, page_size;
    int32_t num_blocks, max_blocks_per_seq;
    int32_t kv_dtype;   /* 0 bf16, 1 fp8 e4m3fn, 2 mxfp4 (e2m1 + e8m0 per 32) */
    int32_t scale_mode; /* 0 none, 1 per-tensor fp32[1], 2 per-token fp32 [blocks][kvh][page] */
    int32_t v_layout;   /* 0 plain [blocks][kvh][page][D], 1 transposed [blocks][kvh][D][page] */
    int32_t q_dtype;    /* 0 bf16, 1 e4m3fn */
    double softmax_scale;
    int32_t causal;     /* 1: query token i attends to t < L - qlen + i + 1 */
    int32_t window;     /* > 0: and to t >= (that end) - window; 0: no window */
} oracle_problem;

enum { OR_OK = 0, OR_EINVAL = 1 };

/* ---------------------------------------------------------------- decoders */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; exponent field 0 encodes subnormals m * 2^-9. */
double oracle_e4m3_to_f64(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int m = b & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* OCP MX e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; all 16 codes finite.
 * exponent field 0: subnormal 0.5 * m. */
double oracle_e2m1_to_f64(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 0x3;
    int m = nibble & 0x1;
    double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return sign ? -v : v;
}

/* OCP MX e8m0 scale: 2^(byte - 127); byte 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* ----------------------------------------------------------------- encoders */

/* Round an fp64 value to bfloat16, round-to-nearest-even (NaN -> 0x7FC0).
 * Obvious form: binary-search the two non-negative codes whose values bracket
 * |x| (codes are monotone in value), take the nearer, ties to the even code.
 * Above the largest finite value the upper neighbour is infinity, which counts
 * as 2^128 for the distance, as IEEE-754 rounding does. */
uint16_t oracle_f64_to_bf16_rne(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (isinf(ax))
        return (uint16_t)(sign | 0x7F80);
    uint16_t lo = 0, hi = 0x7F80;
    while (hi - lo > 1) {
        uint16_t mid = (uint16_t)((lo + hi) / 2);
        if (oracle_bf16_to_f64(mid) <= ax)
            lo = mid;
        else
            hi = mid;
    }
    double vlo = oracle_bf16_to_f64(lo);
    double vhi = (hi == 0x7F80) ? ldexp(1.0, 128) : oracle_bf16_to_f64(hi);
    double dlo = ax - vlo, dhi = vhi - ax;
    uint16_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo & 1) ? hi : lo;
    return (uint16_t)(sign | pick);
}

/* Round an fp64 value to OCP e4m3fn, nearest with ties to the even code,
 * saturating to +-448 (no NaN output for finite input). Brute force over the
 * 127 non-negative finite codes. */
uint8_t oracle_f64_to_e4m3_rne_sat(double x)
{
    uint8_t sign = (x < 0) ? 0x80 : 0;
    double ax = fabs(x);
    int best = 0;
    double bestd = INFINITY;
    if (isnan(x))
        return 0x7F;
    if (ax >= 448.0)
        return (uint8_t)(sign | 0x7E);
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(oracle_e4m3_to_f64((uint8_t)c) - ax);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/* Power-of-two exponent for one query row: the smallest e with amax <= 448 * 2^e
 * (0 for an all-zero row). */
int oracle_q_row_exponent(double amax)
{
    if (!(amax > 0.0))
        return 0;
    int e = -160;
    while (amax > ldexp(448.0, e))
        e++;
    return e;
}

/* Round an fp64 value to OCP MX e2m1, nearest with ties to the even code,
 * saturating to +-6: every magnitude at or above 6 gives the largest code.
 * Below that, brute force over the 8 non-negative codes. The sign bit is the
 * sign of x (so small negative values give the code of -0). */
uint8_t oracle_f64_to_e2m1_rne_sat(double x)
{
    uint8_t sign = signbit(x) ? 0x8 : 0;
    double ax = fabs(x);
    int best = 0;
    double bestd = INFINITY;
    if (ax >= 6.0)
        return (uint8_t)(sign | 7);
    for (int c = 0; c <= 7; c++) {
        double d = fabs(oracle_e2m1_to_f64((uint8_t)c) - ax);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/*
 * oracle_mxfp4_encode_block: one 32-element block to MXFP4, following the OCP
 * Microscaling (MX) v1.0 conversion from scalars to an MX block:
 *   shared exponent E = floor(log2(max_i |v_i|)) - 2   (2 = largest e2m1 exponent);
 *   scale byte = E + 127;
 *   element i = e2m1_rne_sat(v_i / 2^E), packed two per byte, element 2k in
 *   the low nibble of byte k.
 * Readings taken where neither the pages nor the format fix the case:
 *   E is clamped to [-126, 127], not the format's [-127, 127]: the MXFP4
 *   decode supports scale bytes 1..254 in the rows it reads (ROCm/aiter PR
 *   #7056, "Summary"), so a finite block never gets byte 0; an all-zero block
 *   (log2 0 = -inf) gets the bottom of the range, byte 1, and zero elements;
 *   a block holding NaN or an infinity gets scale byte 0xFF (the e8m0 NaN)
 *   and zero elements, so every element decodes to NaN.
 */
void oracle_mxfp4_encode_block(const double v[32], uint8_t data[16], uint8_t* scale)
{
    double amax = 0.0;
    int finite = 1;
    for (int i = 0; i < 32; i++) {
        if (!isfinite(v[i]))
            finite = 0;
        else if (fabs(v[i]) > amax)
            amax = fabs(v[i]);
    }
    memset(data, 0, 16);
    if (!finite) {
        *scale = 0xFF;
        return;
    }
    int E = -126;
    if (amax > 0.0) {
        int e2;
        frexp(amax, &e2); /* amax = f * 2^e2 with f in [0.5, 1): floor(log2 amax) = e2 - 1 */
        E = (e2 - 1) - 2;
        if (E < -126)
            E = -126;
        if (E > 127)
            E = 127;
    }
    *scale = (uint8_t)(E + 127);
    for (int i = 0; i < 32; i++) {
        uint8_t c = oracle_f64_to_e2m1_rne_sat(ldexp(v[i], -E));
        data[i / 2] |= (uint8_t)((i & 1) ? (c << 4) : c);
    }
}

/*
 * oracle_write_kv_mxfp4: store new K and V rows into MXFP4 paged caches (the
 * cache write that produces the pages the MXFP4 decode reads; ROCm/aiter PR
 * #7056, "Summary": K/V pages of e2m1 data [blocks][Hkv][page][D/2] with e8m0
 * scales [blocks][Hkv][page][D/32], written by a separate KV-write kernel).
 *   key, value: bf16 bits [N][Hkv][D];  slots: int32 [N];
 *   token n with 0 <= slots[n] < num_blocks * page_size goes to page
 *   slots[n] / page_size, row slots[n] % page_size, for every KV head; other
 *   slot values (the usual -1 for padding) write nothing.
 *   Every 32-element block of a row is encoded by oracle_mxfp4_encode_block.
 * Bytes of rows no token maps to are left as they were. If two tokens map to
 * one slot the later token wins. Returns 0, or 1 for an invalid description.
 */
int oracle_write_kv_mxfp4(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          int32_t num_blocks, const uint16_t* key, const uint16_t* value, const int32_t* slots,
                          uint8_t* key_cache, uint8_t* value_cache, uint8_t* key_scale, uint8_t* value_scale)
{
    if (num_tokens < 0 || num_kv_heads < 1 || head_dim < 32 || head_dim % 32 != 0 || page_size < 1 ||
        num_blocks < 1)
        return OR_EINVAL;
    const int64_t nslots = (int64_t)num_blocks * page_size;
    const int nblk = head_dim / 32;
    for (int64_t n = 0; n < num_tokens; n++) {
        const int64_t s = slots[n];
        if (s < 0 || s >= nslots)
            continue;
        const int64_t page = s / page_size, row = s % page_size;
        for (int h = 0; h < num_kv_heads; h++) {
            const int64_t src = (n * num_kv_heads + h) * (int64_t)head_dim;
            const int64_t dst_row = (page * num_kv_heads + h) * (int64_t)page_size + row;
            for (int j = 0; j < nblk; j++) {
                double v[32];
                for (int t = 0; t < 2; t++) {
                    const uint16_t* in = t == 0 ? key : value;
                    uint8_t* cache = t == 0 ? key_cache : value_cache;
                    uint8_t* sc = t == 0 ? key_scale : value_scale;
                    for (int i = 0; i < 32; i++)
                        v[i] = oracle_bf16_to_f64(in[src + 32 * j + i]);
                    oracle_mxfp4_encode_block(v, cache + dst_row * (head_dim / 2) + 16 * j, sc + dst_row * nblk + j);
                }
            }
        }
    }
    return OR_OK;
}

/*
 * oracle_mqa_logits_mxfp4: the sparse indexer's per-token scores over a paged
 * MXFP4 index-K cache (ROCm/aiter PR #5761, "Unify gfx950+gfx1250 MXFP4 paged
 * MQA-logits": per query row, logits over the positions of its own window
 * [local_start, local_end) of the sequence row_to_batch names, K read through
 * that sequence's block table; one K head shared by all query heads; q and
 * per-head weights per row; nothing outside the window is written, and a row
 * of no live sequence writes nothing).
 * Reading taken where the pages do not print the formula (the published sparse
 * indexer score, whose per-head weights only make sense with a nonlinearity):
 *   out[r][t] = sum_h weights[r][h] * relu( sum_d qhat[r][h][d] * khat[t][d] )
 * with qhat, khat the MXFP4 values (e2m1 times the e8m0 scale of their 32-element
 * block) and relu(x) = (x < 0 ? 0 : x), so a NaN score (e.g. from an e8m0 NaN
 * scale) stays NaN.
 *   q        u8 [R][H][D/2]   q_scale u8 [R][H][D/32]   weights fp32 [R][H]
 *   k_cache  u8 [NB][PG][D/2] k_scale u8 [NB][PG][D/32]
 *   block_tables int32 [B][W]; row_to_batch, local_starts, local_ends int32 [R]
 *   out, mag fp64 [R][out_stride]: for every row r with 0 <= row_to_batch[r] < B,
 *   positions t in [max(start, 0), min(end, W * PG, out_stride)) get the score,
 *   and mag (nullable) gets sum_h |weights[r][h]| * sum_d |qhat * khat|, the
 *   magnitude the rounding error of a finite-precision sum scales with.
 *   Everything else is left as the caller filled it.
 * Returns 0, or 1 for an invalid description or a window position whose block
 * table entry is outside [0, NB).
 */
int oracle_mqa_logits_mxfp4(int32_t num_rows, int32_t num_heads, int32_t head_dim, int32_t page_size,
                            int32_t num_blocks, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t out_stride,
                            const uint8_t* q, const uint8_t* q_scale, const float* weights, const uint8_t* k_cache,
                            const uint8_t* k_scale, const int32_t* block_tables, const int32_t* row_to_batch,
                            const int32_t* local_starts, const int32_t* local_ends, double* out, double* mag)
{
    if (num_rows < 0 || num_heads < 1 || head_dim < 32 || head_dim > 512 || head_dim % 32 != 0 ||
        page_size < 1 || num_blocks < 1 || num_seqs < 0 || max_blocks_per_seq < 0 || out_stride < 0)
        return OR_EINVAL;
    const int D = head_dim, nb = head_dim / 32;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < num_rows; r++) {
        const int b = row_to_batch[r];
        if (b < 0 || b >= num_seqs)
            continue;
        int64_t t0 = local_starts[r] < 0 ? 0 : local_starts[r];
        int64_t t1 = local_ends[r];
        if (t1 > (int64_t)max_blocks_per_seq * page_size)
            t1 = (int64_t)max_blocks_per_seq * page_size;
        if (t1 > out_stride)
            t1 = out_stride;
        double* qh = (double*)malloc(sizeof(double) * (size_t)num_heads * D);
        for (int h = 0; h < num_heads; h++)
            for (int d = 0; d < D; d++) {
                const int64_t e = ((int64_t)r * num_heads + h) * D + d;
                const uint8_t byte = q[e / 2];
                qh[h * D + d] = oracle_e2m1_to_f64((uint8_t)((d & 1) ? byte >> 4 : byte & 0xF)) *
                                oracle_e8m0_to_f64(q_scale[((int64_t)r * num_heads + h) * nb + d / 32]);
            }
        double kh[512];
        for (int64_t t = t0; t < t1; t++) {
            const int32_t page = block_tables[(int64_t)b * max_blocks_per_seq + t / page_size];
            if (page < 0 || page >= num_blocks) {
                bad = 1;
                continue;
            }
            const int64_t row = (int64_t)page * page_size + t % page_size;
            for (int d = 0; d < D; d++) {
                const uint8_t byte = k_cache[row * (D / 2) + d / 2];
                kh[d] = oracle_e2m1_to_f64((uint8_t)((d & 1) ? byte >> 4 : byte & 0xF)) *
                        oracle_e8m0_to_f64(k_scale[row * nb + d / 32]);
            }
            double acc = 0.0, m = 0.0;
            for (int h = 0; h < num_heads; h++) {
                double s = 0.0, sa = 0.0;
                for (int d = 0; d < D; d++) {
                    s += qh[h * D + d] * kh[d];
                    sa += fabs(qh[h * D + d] * kh[d]);
                }
                const double w = weights[(int64_t)r * num_heads + h];
                acc += w * (s < 0.0 ? 0.0 : s);
                m += fabs(w) * sa;
            }
            out[(int64_t)r * out_stride + t] = acc;
            if (mag)
                mag[(int64_t)r * out_stride + t] = m;
        }
        free(qh);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/* ------------------------------------------------------------- cache reads */

static double kv_elem(const oracle_problem* p, const void* cache, const void* scale_mx, int64_t page, int kvh,
                      int slot, int d, int transposed)
{
    const int64_t PG = p->page_size, D = p->head_dim, H = p->num_kv_heads;
    if (p->kv_dtype == 2) {
        const uint8_t* data = (const uint8_t*)cache;
        const uint8_t* sc = (const uint8_t*)scale_mx;
        int64_t row = (page * H + kvh) * PG + slot;
        uint8_t byte = data[row * (D / 2) + d / 2];
        uint8_t nib = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        return oracle_e2m1_to_f64(nib) * oracle_e8m0_to_f64(sc[row * (D / 32) + d / 32]);
    }
    int64_t idx;
    if (transposed)
        idx = ((page * H + kvh) * D + d) * PG + slot;
    else
        idx = ((page * H + kvh) * PG + slot) * D + d;
    if (p->kv_dtype == 0)
        return oracle_bf16_to_f64(((const uint16_t*)cache)[idx]);
    return oracle_e4m3_to_f64(((const uint8_t*)cache)[idx]);
}

static double token_scale(const oracle_problem* p, const void* scale, int64_t page, int kvh, int slot)
{
    if (p->kv_dtype == 2 || p->scale_mode == 0)
        return 1.0;
    const float* s = (const float*)scale;
    if (p->scale_mode == 1)
        return (double)s[0];
    return (double)s[(page * p->num_kv_heads + kvh) * p->page_size + slot];
}

/* ------------------------------------------------------------------ decode */

/*
 * oracle_pa_decode: attention of every selected sequence over its tokens
 * [t_begin, min(t_end, L_b)), intersected for query token i with its causal /
 * sliding-window range [s_i, e_i). With t_begin = 0 and t_end < 0 the range is
 * the whole context. out: fp64 [num_seqs][qlen][Hq][D], normalised over the range
 * (0 for an empty range). lse (nullable): fp64 [num_seqs][qlen][Hq], the
 * natural log of sum_t exp(s_t) over the range (-inf for an empty range).
 * seqs (nullable): the sequence indices to compute; rows of other sequences
 * are left untouched. Returns 0, or 1 for an invalid description.
 */
int oracle_pa_decode(const oracle_problem* p, const void* query, const void* key_cache, const void* value_cache,
                     const void* k_scale, const void* v_scale, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* seqs, int32_t n_seqs, int32_t t_begin,
                     int32_t t_end, double* out, double* lse, int32_t nthreads)
{
    if (!p || p->num_seqs < 0 || p->qlen < 1 || p->num_kv_heads < 1 || p->q_per_kv < 1 || p->head_dim < 1 ||
        p->page_size < 1 || p->max_blocks_per_seq < 0 || p->num_blocks < 1 || p->window < 0 ||
        (p->causal != 0 && p->causal != 1))
        return OR_EINVAL;
    if (p->kv_dtype == 2 && (p->head_dim % 32) != 0)
        return OR_EINVAL;
    const int B = p->num_seqs, QL = p->qlen, H = p->num_kv_heads, G = p->q_per_kv, D = p->head_dim;
    const int Hq = H * G;
    const double sigma = (p->softmax_scale != 0.0) ? p->softmax_scale : 1.0 / sqrt((double)D);
    const int nsel = seqs ? n_seqs : B;
    const int transposed = (p->v_layout == 1);
    const void* k_mx = (p->kv_dtype == 2) ? k_scale : NULL;
    const void* v_mx = (p->kv_dtype == 2) ? v_scale : NULL;
    int npairs = nsel * H;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int pair = 0; pair < npairs; pair++) {
        int b = seqs ? seqs[pair / H] : pair / H;
        int kvh = pair % H;
        int L = context_lens[b];
        int r0 = t_begin < 0 ? 0 : t_begin;
        int r1 = (t_end < 0 || t_end > L) ? L : t_end;
        double* qhat = (double*)malloc(sizeof(double) * (size_t)D);
        double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        for (int i = 0; i < QL; i++) {
            /* this query token's tokens: [s_i, e_i) within [r0, r1) */
            int e_i = p->causal ? L - QL + i + 1 : L;
            int s_i = p->window > 0 ? e_i - p->window : 0;
            int t0 = s_i > r0 ? s_i : r0;
            int t1 = e_i < r1 ? e_i : r1;
            int n = t1 > t0 ? t1 - t0 : 0;
            for (int hg = 0; hg < G; hg++) {
                int h = kvh * G + hg;
                int64_t row = ((int64_t)b * QL + i) * Hq + h;
                double* o = out + row * D;
                /* query row */
                double qscale = 1.0;
                if (p->q_dtype == 1) {
                    const uint8_t* q8 = (const uint8_t*)query + row * D;
                    for (int d = 0; d < D; d++)
                        qhat[d] = oracle_e4m3_to_f64(q8[d]);
                } else {
                    const uint16_t* q16 = (const uint16_t*)query + row * D;
                    for (int d = 0; d < D; d++)
                        qhat[d] = oracle_bf16_to_f64(q16[d]);
                    if (p->kv_dtype == 2) {
                        double amax = 0.0;
                        for (int d = 0; d < D; d++)
                            if (fabs(qhat[d]) > amax)
                                amax = fabs(qhat[d]);
                        int e = oracle_q_row_exponent(amax);
                        for (int d = 0; d < D; d++)
                            qhat[d] = oracle_e4m3_to_f64(oracle_f64_to_e4m3_rne_sat(ldexp(qhat[d], -e)));
                        qscale = ldexp(1.0, e);
                    }
                }
                /* scores */
                double mx = -INFINITY;
                for (int j = 0; j < n; j++) {
                    int t = t0 + j;
                    int64_t page = block_tables[(int64_t)b * p->max_blocks_per_seq + t / p->page_size];
                    int slot = t % p->page_size;
                    double dot = 0.0;
                    for (int d = 0; d < D; d++)
                        dot += qhat[d] * kv_elem(p, key_cache, k_mx, page, kvh, slot, d, 0);
                    s[j] = sigma * qscale * token_scale(p, k_scale, page, kvh, slot) * dot;
                    if (s[j] > mx)
                        mx = s[j];
                }
                /* softmax and weighted sum of V rows */
                double den = 0.0;
                for (int d = 0; d < D; d++)
                    acc[d] = 0.0;
                for (int j = 0; j < n; j++) {
                    int t = t0 + j;
                    int64_t page = block_tables[(int64_t)b * p->max_blocks_per_seq + t / p->page_size];
                    int slot = t % p->page_size;
                    double w = exp(s[j] - mx);
                    double vs = token_scale(p, v_scale, page, kvh, slot);
                    den += w;
                    for (int d = 0; d < D; d++)
                        acc[d] += w * vs * kv_elem(p, value_cache, v_mx, page, kvh, slot, d, transposed);
                }
                for (int d = 0; d < D; d++)
                    o[d] = (n > 0) ? acc[d] / den : 0.0;
                if (lse)
                    lse[row] = (n > 0) ? mx + log(den) : -INFINITY;
            }
        }
        free(qhat);
        free(s);
        free(acc);
    }
    return OR_OK;
}

/*
 * oracle_lse_merge: combine attention results over disjoint token ranges.
 * o_parts: [nparts][D] each normalised over its range, lse_parts: [nparts].
 * Result: sum_p exp(lse_p - LSE) o_p with LSE = log sum_p exp(lse_p); parts
 * with lse = -inf contribute nothing; all-empty gives 0.
 */
void oracle_lse_merge(int32_t nparts, int32_t D, const double* o_parts, const double* lse_parts, double* out,
                      double* lse_out)
{
    double mx = -INFINITY;
    for (int p = 0; p < nparts; p++)
        if (lse_parts[p] > mx)
            mx = lse_parts[p];
    for (int d = 0; d < D; d++)
        out[d] = 0.0;
    if (mx == -INFINITY) {
        if (lse_out)
            *lse_out = -INFINITY;
        return;
    }
    double den = 0.0;
    for (int p = 0; p < nparts; p++)
        den += exp(lse_parts[p] - mx);
    for (int p = 0; p < nparts; p++) {
        double w = exp(lse_parts[p] - mx) / den;
        for (int d = 0; d < D; d++)
            out[d] += w * o_parts[(int64_t)p * D + d];
    }
    if (lse_out)
        *lse_out = mx + log(den);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
