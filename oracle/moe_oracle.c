/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference of the routed NVFP4 mixture-of-experts FFN. Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg load this library; the GPU
 * library shares no code, header, table or helper with it.
 *
 * What it computes, and where each step comes from:
 *  - NVFP4 weights: 64 weights in a 36-byte block, four UE4M3 sub-scales (one per 16 weights)
 *    followed by 32 code bytes of E2M1 nibbles (moe_sel_census.rs, the NVFP4 block constants;
 *    moe_union_probe.rs, the per-expert byte arithmetic: half a byte of code per weight plus one
 *    scale byte per 16 weights). Inside a block: byte j (j<4) is the scale of weights 16j..16j+15; byte 4+i holds
 *    weight 2i in its low nibble and weight 2i+1 in its high nibble (the plainest reading; the
 *    pages give no nibble order). A row is out-row o, contiguous along the input features.
 *  - E2M1 and UE4M3 values: the OCP Microscaling (MX) FP4 E2M1 element type and the OCP FP8
 *    E4M3 ("fn": bias 7, no infinities, 0x7F NaN) type with its sign bit required to be 0.
 *  - Routing buckets: pairs p = t*k + j are pushed into per-expert lists in ascending p, the
 *    non-empty lists are concatenated in ascending expert id, and the offsets are the running
 *    totals (moe_sk_repro.rs, the host bucketing in main before the grouped calls). Ids outside
 *    [expert_base, expert_base+E) are not routed here and are counted instead.
 *  - The FFN per routed pair: gate and up projections of the token's activation row, SiLU of
 *    the gate times the up value, the down projection, and the router-weighted sum over the
 *    token's k slots taken in ascending slot order (moe_union_probe.rs: the fused
 *    sel_gu_silu and sel_v3 kernels it names; moe_sk_repro.rs: gate, up and down grouped
 *    calls). Everything is fp64; the intermediate h is not rounded (a diagnostic switch,
 *    orc_set_h_round, rounds it to bf16 or to a bf16 hi + lo pair instead).
 *
 *  - Second-level scales (the ModelOpt NVFP4 form the Rocket post's banks use): optionally one
 *    fp32 factor per expert and bank multiplies every weight of that expert's bank, so a weight
 *    is code value * UE4M3 scale * s2[e]. Absent (NULL), the factor is 1.
 *
 * Two forms of the FFN are provided. The per-slot form walks the pairs of each token and decodes
 * each needed weight row as it goes. The union form decodes every distinct active expert once
 * and then walks that expert's bucket (moe_union_probe.rs: the union-of-experts gather). Both
 * perform the same fp64 operations in the same order and must agree bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK_WEIGHTS 64
#define ORC_BLOCK_BYTES 36

/* OCP MX FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa. */
double orc_e2m1(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* OCP FP8 E4M3 (fn) with the sign bit fixed at 0: bits 6..3 exponent (bias 7), bits 2..0
 * mantissa; exponent 0 is subnormal (m * 2^-9); 0x7F is NaN. Bytes with bit 7 set are not
 * UE4M3 values and also return NaN. */
double orc_ue4m3(int byte)
{
    if (byte < 0 || byte > 0x7E) return NAN;
    int e = (byte >> 3) & 15, m = byte & 7;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* bfloat16 bit pattern to its exact value. */
double orc_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Weight i of one NVFP4 row. */
double orc_nvfp4_weight(const uint8_t *row, int64_t i)
{
    const uint8_t *blk = row + (i / ORC_BLOCK_WEIGHTS) * ORC_BLOCK_BYTES;
    int w = (int)(i % ORC_BLOCK_WEIGHTS);
    int scale_byte = blk[w / 16];
    int code_byte = blk[4 + w / 2];
    int code = (w & 1) ? (code_byte >> 4) : (code_byte & 15);
    return orc_e2m1(code) * orc_ue4m3(scale_byte);
}

int64_t orc_row_bytes(int64_t in_f) { return in_f / ORC_BLOCK_WEIGHTS * ORC_BLOCK_BYTES; }

/* Decode n_rows consecutive rows of in_f weights into out[n_rows][in_f]. */
void orc_dequant_rows(const uint8_t *rows, int64_t n_rows, int64_t in_f, double *out)
{
    int64_t rb = orc_row_bytes(in_f);
    for (int64_t r = 0; r < n_rows; r++)
        for (int64_t i = 0; i < in_f; i++) out[r * in_f + i] = orc_nvfp4_weight(rows + r * rb, i);
}

/*
 * Expert-first bucketing. ids[T*k] (pair p = t*k + j). Local expert = id - expert_base.
 * Writes offsets[E+1] (exclusive running totals over all E local experts), pair_ids[0 ..
 * offsets[E]) (pairs grouped by expert, ascending p inside a bucket), active[0 .. n_active)
 * (non-empty local experts, ascending), counts[0] = n_active, counts[1] = n_nonlocal.
 * Returns 0, or -1 on bad arguments.
 */
int orc_route_bucket(const int32_t *ids, int64_t T, int32_t k, int32_t E, int32_t expert_base,
                     int32_t *offsets, int32_t *pair_ids, int32_t *active, int32_t *counts)
{
    if (T < 0 || k < 1 || E < 1) return -1;
    int64_t P = T * k;
    int64_t *count = calloc((size_t)E, sizeof *count);
    int64_t *cursor = calloc((size_t)E, sizeof *cursor);
    if (!count || !cursor) { free(count); free(cursor); return -1; }
    int64_t nonlocal = 0;
    for (int64_t p = 0; p < P; p++) {
        int64_t e = (int64_t)ids[p] - expert_base;
        if (e < 0 || e >= E) nonlocal++;
        else count[e]++;
    }
    int64_t run = 0, n_active = 0;
    for (int32_t e = 0; e < E; e++) {
        offsets[e] = (int32_t)run;
        cursor[e] = run;
        run += count[e];
        if (count[e] > 0) active[n_active++] = e;
    }
    offsets[E] = (int32_t)run;
    for (int64_t p = 0; p < P; p++) {
        int64_t e = (int64_t)ids[p] - expert_base;
        if (e < 0 || e >= E) continue;
        pair_ids[cursor[e]++] = (int32_t)p;
    }
    counts[0] = (int32_t)n_active;
    counts[1] = (int32_t)nonlocal;
    free(count);
    free(cursor);
    return 0;
}

static double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Diagnostic rounding of the intermediate h (a reading the pages leave open: how precisely the
 * gate/up result is carried into the down projection). The canonical oracle keeps h unrounded
 * (mode 0). Mode 1 rounds h to fp32 and then to bf16 (nearest, ties to even), as a pipeline
 * storing h as one bf16 value would; mode 2 keeps the fp32 value as hi + lo, hi its bf16
 * rounding and lo the bf16 rounding of the remainder. Process-wide; tests set and reset it. */
static int g_h_round = 0;
void orc_set_h_round(int32_t mode) { g_h_round = mode; }

static double bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double round_h(double h)
{
    if (g_h_round == 0) return h;
    const float f = (float)h;
    const double hi = bf16_round(f);
    if (g_h_round == 1) return hi;
    /* f - hi is exact in fp32: both are fp32 values and hi agrees with f in its top 8 bits */
    return hi + bf16_round((float)((double)f - hi));
}

/* One pair through one expert, from dense decoded matrices:
 * g = Wg x, u = Wu x, h = silu(g) * u, d = Wd h. Sums run in ascending index. */
static void pair_ffn_dense(const double *x, const double *Wg, const double *Wu, const double *Wd,
                           int32_t H, int32_t F, double *h, double *d)
{
    for (int32_t o = 0; o < F; o++) {
        double g = 0.0, u = 0.0;
        for (int32_t i = 0; i < H; i++) g += Wg[(int64_t)o * H + i] * x[i];
        for (int32_t i = 0; i < H; i++) u += Wu[(int64_t)o * H + i] * x[i];
        h[o] = round_h(orc_silu(g) * u);
    }
    for (int32_t r = 0; r < H; r++) {
        double s = 0.0;
        for (int32_t o = 0; o < F; o++) s += Wd[(int64_t)r * F + o] * h[o];
        d[r] = s;
    }
}

/* Multiply n decoded weights by a bank's second-level scale (s = 1: unchanged). */
static void scale_weights(double *w, int64_t n, double s)
{
    if (s != 1.0)
        for (int64_t i = 0; i < n; i++) w[i] *= s;
}

/* The second-level scale of expert e in a bank (1 when the bank has none). */
static double s2_of(const float *s2, int64_t e) { return s2 ? (double)s2[e] : 1.0; }

/* The same arithmetic, decoding each weight row just before it is used; sg, su, sd are the
 * expert's second-level scales of the three banks. */
static void pair_ffn_rowwise(const double *x, const uint8_t *gate, const uint8_t *up,
                             const uint8_t *down, int32_t H, int32_t F, double sg, double su,
                             double sd, double *row, double *h, double *d)
{
    int64_t rbh = orc_row_bytes(H), rbf = orc_row_bytes(F);
    for (int32_t o = 0; o < F; o++) {
        double g = 0.0, u = 0.0;
        orc_dequant_rows(gate + o * rbh, 1, H, row);
        scale_weights(row, H, sg);
        for (int32_t i = 0; i < H; i++) g += row[i] * x[i];
        orc_dequant_rows(up + o * rbh, 1, H, row);
        scale_weights(row, H, su);
        for (int32_t i = 0; i < H; i++) u += row[i] * x[i];
        h[o] = round_h(orc_silu(g) * u);
    }
    for (int32_t r = 0; r < H; r++) {
        double s = 0.0;
        orc_dequant_rows(down + r * rbf, 1, F, row);
        scale_weights(row, F, sd);
        for (int32_t o = 0; o < F; o++) s += row[o] * h[o];
        d[r] = s;
    }
}

static void set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Per-slot form. Computes y for the n_tokens token indices in tokens[] (all T tokens if tokens
 * is NULL; then n_tokens must equal T) into y[n_tokens][H], fp64.
 * Banks: expert e's gate rows start at gate + e*gate_stride (bytes), likewise up and down;
 * gate/up rows have H inputs, down rows F inputs.
 */
int orc_ffn_per_slot_s2(const uint16_t *x_bf16, const float *topk_w, const int32_t *ids,
                        int64_t T, int32_t k, int32_t E, int32_t expert_base, int32_t H,
                        int32_t F, const uint8_t *gate, int64_t gate_stride, const uint8_t *up,
                        int64_t up_stride, const uint8_t *down, int64_t down_stride,
                        const float *gate_s2, const float *up_s2, const float *down_s2,
                        const int64_t *tokens, int64_t n_tokens, double *y, int32_t n_threads)
{
    if (T < 0 || k < 1 || E < 1 || H % 64 || F % 64 || H < 64 || F < 64) return -1;
    if (!tokens && n_tokens != T) return -1;
    set_threads(n_threads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t n = 0; n < n_tokens; n++) {
        int64_t t = tokens ? tokens[n] : n;
        if (t < 0 || t >= T) { bad = 1; continue; }
        double *xr = malloc(sizeof(double) * (size_t)H);
        double *row = malloc(sizeof(double) * (size_t)(H > F ? H : F));
        double *h = malloc(sizeof(double) * (size_t)F);
        double *d = malloc(sizeof(double) * (size_t)H);
        double *yr = y + n * H;
        for (int32_t i = 0; i < H; i++) xr[i] = orc_bf16(x_bf16[t * H + i]);
        for (int32_t r = 0; r < H; r++) yr[r] = 0.0;
        for (int32_t j = 0; j < k; j++) {
            int64_t e = (int64_t)ids[t * k + j] - expert_base;
            if (e < 0 || e >= E) continue;
            pair_ffn_rowwise(xr, gate + e * gate_stride, up + e * up_stride,
                             down + e * down_stride, H, F, s2_of(gate_s2, e), s2_of(up_s2, e),
                             s2_of(down_s2, e), row, h, d);
            double wt = (double)topk_w[t * k + j];
            for (int32_t r = 0; r < H; r++) yr[r] += wt * d[r];
        }
        free(xr); free(row); free(h); free(d);
    }
    return bad ? -1 : 0;
}

/* Without second-level scales. */
int orc_ffn_per_slot(const uint16_t *x_bf16, const float *topk_w, const int32_t *ids, int64_t T,
                     int32_t k, int32_t E, int32_t expert_base, int32_t H, int32_t F,
                     const uint8_t *gate, int64_t gate_stride, const uint8_t *up,
                     int64_t up_stride, const uint8_t *down, int64_t down_stride,
                     const int64_t *tokens, int64_t n_tokens, double *y, int32_t n_threads)
{
    return orc_ffn_per_slot_s2(x_bf16, topk_w, ids, T, k, E, expert_base, H, F, gate,
                               gate_stride, up, up_stride, down, down_stride, NULL, NULL, NULL,
                               tokens, n_tokens, y, n_threads);
}

/*
 * Union form: bucket the pairs, decode each active expert once, run every pair of its bucket,
 * then combine each token's slots in ascending slot order.
 * tokens (NULL: all T tokens, n_tokens must equal T) selects the tokens whose y rows are wanted;
 * only the pairs of those tokens are computed, each exactly as in the full layer, and
 * y[n][H] (fp64) receives token tokens[n]. If h_out is not NULL it receives h[p][F] for every
 * computed local pair p (other rows are left untouched).
 * The active experts are shared out over the threads, each decoding its experts into buffers of
 * its own; a pair's arithmetic (and so every bit of y) does not depend on the thread count.
 */
int orc_ffn_union_sel_s2(const uint16_t *x_bf16, const float *topk_w, const int32_t *ids,
                         int64_t T, int32_t k, int32_t E, int32_t expert_base, int32_t H,
                         int32_t F, const uint8_t *gate, int64_t gate_stride, const uint8_t *up,
                         int64_t up_stride, const uint8_t *down, int64_t down_stride,
                         const float *gate_s2, const float *up_s2, const float *down_s2,
                         const int64_t *tokens, int64_t n_tokens, double *y, double *h_out,
                         int32_t n_threads)
{
    if (T < 0 || k < 1 || E < 1 || H % 64 || F % 64 || H < 64 || F < 64) return -1;
    if (!tokens && n_tokens != T) return -1;
    set_threads(n_threads);
    int64_t P = T * k;
    int32_t *offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *pair_ids = malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    int32_t *active = malloc(sizeof(int32_t) * (size_t)E);
    int32_t counts[2];
    char *want = calloc((size_t)(T > 0 ? T : 1), 1);        /* token t's y row is wanted */
    int64_t *row_of = malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));  /* its D row block */
    double *D = NULL;
    char *has = calloc((size_t)(P > 0 ? P : 1), 1);
    int rc = -1, bad = 0;
    if (!offsets || !pair_ids || !active || !want || !row_of || !has) goto out;
    for (int64_t n = 0; n < n_tokens; n++) {
        int64_t t = tokens ? tokens[n] : n;
        if (t < 0 || t >= T) goto out;
        if (!want[t]) row_of[t] = n;   /* a token listed twice takes its first row */
        want[t] = 1;
    }
    /* D[(row_of[t]) * k + j][H]: the down output of slot j of a wanted token */
    D = calloc((size_t)(n_tokens > 0 ? n_tokens : 1) * (size_t)k * (size_t)H, sizeof(double));
    if (!D) goto out;
    if (orc_route_bucket(ids, T, k, E, expert_base, offsets, pair_ids, active, counts)) goto out;
#pragma omp parallel reduction(| : bad)
    {
        double *Wg = malloc(sizeof(double) * (size_t)F * H);
        double *Wu = malloc(sizeof(double) * (size_t)F * H);
        double *Wd = malloc(sizeof(double) * (size_t)H * F);
        double *xr = malloc(sizeof(double) * (size_t)H);
        double *h = malloc(sizeof(double) * (size_t)F);
        if (!Wg || !Wu || !Wd || !xr || !h) bad = 1;
#pragma omp for schedule(dynamic, 1)
        for (int32_t a = 0; a < counts[0]; a++) {
            if (!Wg || !Wu || !Wd || !xr || !h) continue;
            int32_t e = active[a];
            int32_t b0 = offsets[e], b1 = offsets[e + 1], needed = 0;
            for (int32_t q = b0; q < b1; q++) needed |= want[pair_ids[q] / k];
            if (!needed) continue;
            orc_dequant_rows(gate + e * gate_stride, F, H, Wg);
            orc_dequant_rows(up + e * up_stride, F, H, Wu);
            orc_dequant_rows(down + e * down_stride, H, F, Wd);
            scale_weights(Wg, (int64_t)F * H, s2_of(gate_s2, e));
            scale_weights(Wu, (int64_t)F * H, s2_of(up_s2, e));
            scale_weights(Wd, (int64_t)H * F, s2_of(down_s2, e));
            for (int32_t q = b0; q < b1; q++) {
                int64_t p = pair_ids[q], t = p / k;
                if (!want[t]) continue;
                for (int32_t i = 0; i < H; i++) xr[i] = orc_bf16(x_bf16[t * H + i]);
                pair_ffn_dense(xr, Wg, Wu, Wd, H, F, h, D + (row_of[t] * k + p % k) * H);
                if (h_out) memcpy(h_out + p * F, h, sizeof(double) * (size_t)F);
                has[p] = 1;
            }
        }
        free(Wg); free(Wu); free(Wd); free(xr); free(h);
    }
    if (bad) goto out;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < n_tokens; n++) {
        int64_t t = tokens ? tokens[n] : n;
        double *yr = y + n * H;
        for (int32_t r = 0; r < H; r++) yr[r] = 0.0;
        for (int32_t j = 0; j < k; j++) {
            int64_t p = t * k + j;
            if (!has[p]) continue;
            double wt = (double)topk_w[p];
            const double *d = D + (row_of[t] * k + j) * H;
            for (int32_t r = 0; r < H; r++) yr[r] += wt * d[r];
        }
    }
    rc = 0;
out:
    free(offsets); free(pair_ids); free(active); free(want); free(row_of); free(D); free(has);
    return rc;
}

/* All T tokens. */
int orc_ffn_union_s2(const uint16_t *x_bf16, const float *topk_w, const int32_t *ids, int64_t T,
                     int32_t k, int32_t E, int32_t expert_base, int32_t H, int32_t F,
                     const uint8_t *gate, int64_t gate_stride, const uint8_t *up,
                     int64_t up_stride, const uint8_t *down, int64_t down_stride,
                     const float *gate_s2, const float *up_s2, const float *down_s2, double *y,
                     double *h_out, int32_t n_threads)
{
    return orc_ffn_union_sel_s2(x_bf16, topk_w, ids, T, k, E, expert_base, H, F, gate,
                                gate_stride, up, up_stride, down, down_stride, gate_s2, up_s2,
                                down_s2, NULL, T, y, h_out, n_threads);
}

/* Without second-level scales. */
int orc_ffn_union(const uint16_t *x_bf16, const float *topk_w, const int32_t *ids, int64_t T,
                  int32_t k, int32_t E, int32_t expert_base, int32_t H, int32_t F,
                  const uint8_t *gate, int64_t gate_stride, const uint8_t *up, int64_t up_stride,
                  const uint8_t *down, int64_t down_stride, double *y, double *h_out,
                  int32_t n_threads)
{
    return orc_ffn_union_s2(x_bf16, topk_w, ids, T, k, E, expert_base, H, F, gate, gate_stride,
                            up, up_stride, down, down_stride, NULL, NULL, NULL, y, h_out,
                            n_threads);
}

/*
 * Router: top-k selection plus softmax weights, per token (the step that produces the routed
 * pairs the rest of this file consumes). The pages name a router without spelling it out; the
 * reading taken here is the plainest one consistent with their workloads (k distinct experts per
 * token, weights a softmax over the selected experts' logits):
 *  - slot j of token t holds the j-th largest logit of row t, with equal logits taken in
 *    ascending expert id, and no expert taken twice;
 *  - w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected logits (l_0 the largest),
 *    in fp64 from the fp32 logits.
 * Selection compares the fp32 logits exactly (as doubles, which order them identically).
 * Returns 0, or -1 on bad arguments (k < 1 or k > E).
 */
int orc_router_topk(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *ids, double *w)
{
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
    unsigned char *taken = malloc((size_t)E);
    if (!taken) return -1;
    for (int64_t t = 0; t < T; t++) {
        const float *l = logits + t * E;
        memset(taken, 0, (size_t)E);
        for (int32_t j = 0; j < k; j++) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || (double)l[e] > (double)l[best]) best = e;   /* first max wins */
            }
            taken[best] = 1;
            ids[t * k + j] = best;
        }
        double top = (double)l[ids[t * k]], sum = 0.0;
        for (int32_t j = 0; j < k; j++) sum += exp((double)l[ids[t * k + j]] - top);
        for (int32_t j = 0; j < k; j++) w[t * k + j] = exp((double)l[ids[t * k + j]] - top) / sum;
    }
    free(taken);
    return 0;
}
