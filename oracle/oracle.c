/*
 * CPU oracle for the Ulysses 4D all-to-all relayout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no header, helper, table
 * or constant with the GPU library; the two are written independently from
 * the pages and compared element by element.
 *
 * Sources (fast-ulysses 0.1.0 PyPI page; fast-ulysses 0.2.1 README;
 * FastVideo "Ulysses performance on GB200"):
 *   - mode 0 trades a sequence shard for a head shard, mode 1 trades it back
 *     (both fast-ulysses pages, introduction; 0.2.1 Quick start);
 *   - per-rank uneven seq_splits / head_splits, even splits being a special
 *     case (0.1.0 "What it does"; 0.2.1 "Key features");
 *   - the result equals torch.distributed permute + all_to_all_single +
 *     permute (0.1.0 "Results"; 0.2.1 "Performance"), which fixes rank order:
 *     sequence pieces are concatenated in source-rank order and rank r owns
 *     the contiguous head block [head_off_r, head_off_r + H_r);
 *   - per-plane window bytes for the plane-at-a-time exchange (FastVideo
 *     page, first two paragraphs);
 *   - QK RMSNorm + RoPE fused into the scatter (0.1.0 "What it does", last
 *     paragraph).  The pages give no formula; the reading written out in
 *     oracle_qknorm_rope_mode0 below is the one this project fixes, and
 *     oracle_row_sum_of_squares exposes its first step for the tests.
 *
 * Everything is plain index loops over (rank, batch, sequence, head,
 * element).  The relayout copies raw element bytes and never converts, so
 * NaN payloads, -0 and fp8 encodings are preserved.  Built with -O2
 * -ffp-contract=off and no fast-math: every float operation below is one
 * IEEE single-precision operation in the written order.
 *
 * The *_threads entry points run the very same loops with an OpenMP pragma
 * that hands whole destination rows to `threads` threads: each row is
 * computed by one thread exactly as in the single-threaded form, so the
 * results are identical; the threads only shorten the wall time (the
 * benchmark's all-cores baseline and the full-size checks use them).
 *
 * Return codes: 0 on success, -1 on invalid arguments (nothing written).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_MAX_WORLD 64

/* ------------------------------------------------------------------ */
/* Geometry                                                            */
/* ------------------------------------------------------------------ */

typedef struct {
    int world;
    int64_t b, d, esz;
    int64_t S[ORACLE_MAX_WORLD];      /* seq_splits  */
    int64_t H[ORACLE_MAX_WORLD];      /* head_splits */
    int64_t seq_off[ORACLE_MAX_WORLD + 1];
    int64_t head_off[ORACLE_MAX_WORLD + 1];
    int64_t s_global, n_global;
} geom_t;

static int geom_init(geom_t *g, int world, int64_t b, int64_t d, int64_t esz,
                     const int64_t *seq_splits, const int64_t *head_splits)
{
    int j;
    if (world < 1 || world > ORACLE_MAX_WORLD || b < 0 || d < 1 || esz < 1)
        return -1;
    g->world = world;
    g->b = b;
    g->d = d;
    g->esz = esz;
    g->seq_off[0] = 0;
    g->head_off[0] = 0;
    for (j = 0; j < world; ++j) {
        if (seq_splits[j] < 0 || head_splits[j] < 0)
            return -1;
        g->S[j] = seq_splits[j];
        g->H[j] = head_splits[j];
        g->seq_off[j + 1] = g->seq_off[j] + seq_splits[j];
        g->head_off[j + 1] = g->head_off[j] + head_splits[j];
    }
    g->s_global = g->seq_off[world];
    g->n_global = g->head_off[world];
    return 0;
}

/* The source rank whose sequence range [seq_off_j, seq_off_{j+1}) holds S. */
static int seq_owner(const geom_t *g, int64_t S)
{
    int j;
    for (j = 0; j < g->world; ++j)
        if (g->seq_off[j] <= S && S < g->seq_off[j + 1])
            return j;
    return -1;
}

/* The source rank whose head range [head_off_j, head_off_{j+1}) holds H. */
static int head_owner(const geom_t *g, int64_t H)
{
    int j;
    for (j = 0; j < g->world; ++j)
        if (g->head_off[j] <= H && H < g->head_off[j + 1])
            return j;
    return -1;
}

/* Shape of rank `rank`'s shard: the input (is_dst = 0) or output (is_dst = 1)
 * of `mode`.  Mode-0 input and mode-1 output are (b, S_r, n_global, d); mode-0
 * output and mode-1 input are (b, s_global, H_r, d). */
int oracle_shape(int mode, int world, int64_t b, int64_t d,
                 const int64_t *seq_splits, const int64_t *head_splits,
                 int rank, int is_dst, int64_t shape[4])
{
    geom_t g;
    int seq_sharded;
    if (mode != 0 && mode != 1)
        return -1;
    if (geom_init(&g, world, b, d, 1, seq_splits, head_splits) != 0)
        return -1;
    if (rank < 0 || rank >= world)
        return -1;
    /* sequence-sharded side: mode-0 source or mode-1 destination */
    seq_sharded = (mode == 0) ? !is_dst : is_dst;
    shape[0] = b;
    shape[1] = seq_sharded ? g.S[rank] : g.s_global;
    shape[2] = seq_sharded ? g.n_global : g.H[rank];
    shape[3] = d;
    return 0;
}

/* Bytes one rank's window must hold for ONE batch plane of the exchange:
 * the largest per-rank destination plane, max_r s_global*H_r*d*esz (mode 0)
 * or max_r S_r*n_global*d*esz (mode 1).  The FastVideo page prints this
 * figure for 250,000 tokens, 56 heads, d = 128, bf16, four ranks. */
int64_t oracle_window_bytes(int mode, int world, int64_t d, int64_t esz,
                            const int64_t *seq_splits, const int64_t *head_splits)
{
    geom_t g;
    int64_t best = 0, bytes;
    int r;
    if (mode != 0 && mode != 1)
        return -1;
    if (geom_init(&g, world, 1, d, esz, seq_splits, head_splits) != 0)
        return -1;
    for (r = 0; r < world; ++r) {
        if (mode == 0)
            bytes = g.s_global * g.H[r] * d * esz;
        else
            bytes = g.S[r] * g.n_global * d * esz;
        if (bytes > best)
            best = bytes;
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* Pure relayout                                                       */
/* ------------------------------------------------------------------ */

/* Source byte address of destination element (r, bi, s, h, e).
 *   mode 0: out_r[bi][S][h][e] = in_j[bi][S - seq_off_j][head_off_r + h][e],
 *           j the owner of global position S;
 *   mode 1: out_r[bi][s][H][e] = in_j[bi][seq_off_r + s][H - head_off_j][e],
 *           j the owner of global head H. */
static const unsigned char *source_of(const geom_t *g, int mode,
                                      const void *const *src, int r,
                                      int64_t bi, int64_t s, int64_t h, int64_t e)
{
    int j;
    int64_t elem;
    if (mode == 0) {
        j = seq_owner(g, s);
        elem = ((bi * g->S[j] + (s - g->seq_off[j])) * g->n_global
                + (g->head_off[r] + h)) * g->d + e;
    } else {
        j = head_owner(g, h);
        elem = ((bi * g->s_global + (g->seq_off[r] + s)) * g->H[j]
                + (h - g->head_off[j])) * g->d + e;
    }
    return (const unsigned char *)src[j] + elem * g->esz;
}

/* Full relayout.  src[j] and dst[r] are host buffers laid out contiguously,
 * row-major, d innermost, with the shapes oracle_shape() reports. */
static int a2a_4d(int mode, int world, int64_t b, int64_t d, int64_t esz,
                  const int64_t *seq_splits, const int64_t *head_splits,
                  const void *const *src, void *const *dst, int threads)
{
    geom_t g;
    int r;
    if (mode != 0 && mode != 1)
        return -1;
    if (geom_init(&g, world, b, d, esz, seq_splits, head_splits) != 0)
        return -1;
    for (r = 0; r < world; ++r) {
        unsigned char *out = (unsigned char *)dst[r];
        const int64_t rows = (mode == 0) ? g.s_global : g.S[r];
        const int64_t heads = (mode == 0) ? g.H[r] : g.n_global;
        int64_t bi, s;
#pragma omp parallel for collapse(2) schedule(static) if (threads > 1) num_threads(threads)
        for (bi = 0; bi < b; ++bi)
            for (s = 0; s < rows; ++s) {
                int64_t h, e;
                for (h = 0; h < heads; ++h)
                    for (e = 0; e < d; ++e) {
                        int64_t at = (((bi * rows + s) * heads + h) * d + e) * esz;
                        memcpy(out + at, source_of(&g, mode, src, r, bi, s, h, e),
                               (size_t)esz);
                    }
            }
    }
    return 0;
}

int oracle_a2a_4d(int mode, int world, int64_t b, int64_t d, int64_t esz,
                  const int64_t *seq_splits, const int64_t *head_splits,
                  const void *const *src, void *const *dst)
{
    return a2a_4d(mode, world, b, d, esz, seq_splits, head_splits, src, dst, 1);
}

int oracle_a2a_4d_threads(int mode, int world, int64_t b, int64_t d, int64_t esz,
                          const int64_t *seq_splits, const int64_t *head_splits,
                          const void *const *src, void *const *dst, int threads)
{
    if (threads < 1)
        return -1;
    return a2a_4d(mode, world, b, d, esz, seq_splits, head_splits, src, dst, threads);
}

/* The same definition evaluated at n chosen destination coordinates.
 * coords is n x 5 int64: (rank, bi, s, h, e) in the destination shard's
 * own index space; out receives n * esz bytes.  Used to check outputs too
 * large for a full CPU pass. */
int oracle_a2a_4d_sample(int mode, int world, int64_t b, int64_t d, int64_t esz,
                         const int64_t *seq_splits, const int64_t *head_splits,
                         const void *const *src, int64_t n,
                         const int64_t *coords, void *out)
{
    geom_t g;
    int64_t i;
    if (mode != 0 && mode != 1)
        return -1;
    if (geom_init(&g, world, b, d, esz, seq_splits, head_splits) != 0)
        return -1;
    for (i = 0; i < n; ++i) {
        const int64_t *c = coords + 5 * i;
        int r = (int)c[0];
        int64_t rows, heads;
        if (r < 0 || r >= world)
            return -1;
        rows = (mode == 0) ? g.s_global : g.S[r];
        heads = (mode == 0) ? g.H[r] : g.n_global;
        if (c[1] < 0 || c[1] >= b || c[2] < 0 || c[2] >= rows || c[3] < 0
            || c[3] >= heads || c[4] < 0 || c[4] >= d)
            return -1;
        memcpy((unsigned char *)out + i * esz,
               source_of(&g, mode, src, r, c[1], c[2], c[3], c[4]), (size_t)esz);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Fused QK RMSNorm + RoPE on the mode-0 relayout                       */
/* ------------------------------------------------------------------ */

/* bfloat16 <-> float.  bf16 is the top half of an IEEE binary32; rounding
 * to it is round-to-nearest, ties to even, on the 16 dropped bits. */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t float_to_bf16_rne(float f)
{
    uint32_t u, lsb;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays NaN (quiet) */
    lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Array helpers, exposed so the tests can pin the rounding on its own. */
void oracle_f32_to_bf16(const float *in, uint16_t *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = float_to_bf16_rne(in[i]);
}

void oracle_bf16_to_f32(const uint16_t *in, float *out, int64_t n)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = bf16_to_float(in[i]);
}

/* RoPE table: cos_tab[S][p] = (float)cos(S * w_p), sin_tab likewise, with
 * w_p = theta^(-2p/d), all in double precision and rounded to float once.
 * Shape [s_global][d/2].  RoFormer's rotary position embedding. */
int oracle_rope_table(double theta, int64_t s_global, int64_t d,
                      float *cos_out, float *sin_out)
{
    int64_t S, p, half;
    if (s_global < 0 || d < 2 || d % 2 != 0 || !(theta > 0.0))
        return -1;
    half = d / 2;
    for (S = 0; S < s_global; ++S)
        for (p = 0; p < half; ++p) {
            double w = pow(theta, -2.0 * (double)p / (double)d);
            double angle = (double)S * w;
            cos_out[S * half + p] = (float)cos(angle);
            sin_out[S * half + p] = (float)sin(angle);
        }
    return 0;
}

/* One row of d elements at global sequence position S:
 *   1. xf[i] = x[i] widened to float (exact);
 *   2. one partial sum of squares per group of 8 consecutive elements, in
 *      ascending order, each step one fused multiply-add: p = fmaf(x, x, p);
 *   3. those d/8 partials summed as a pairwise tree with adjacent pairing
 *      ((p0+p1), (p2+p3), ...; then pairs of those; ...);
 *   4. ms = ss / d;  inv = 1 / sqrt(ms + eps), both correctly rounded;
 *   5. y[i] = (xf[i] * inv) * gamma[i];
 *   6. rotate each interleaved pair (2p, 2p+1) by the angle S * w_p:
 *        o[2p]   = y[2p]*cos - y[2p+1]*sin,
 *        o[2p+1] = y[2p]*sin + y[2p+1]*cos,
 *      each product rounded before the add / subtract;
 *   7. round each o[i] to bf16, nearest-even. */
/* Sum of squares of one row in the fixed fp32 order: one fused
 * multiply-add chain per group of 8 consecutive elements (ascending), then
 * the pairwise tree over the d/8 partial sums with adjacent pairing. */
static float row_sum_of_squares(const float *xf, int64_t d)
{
    float part[512];
    int64_t i, l, k, n;
    for (l = 0; l < d / 8; ++l) {
        part[l] = 0.0f;
        for (i = 8 * l; i < 8 * l + 8; ++i)
            part[l] = fmaf(xf[i], xf[i], part[l]);
    }
    for (n = d / 8; n > 1; n /= 2)
        for (k = 0; k < n / 2; ++k)
            part[k] = part[2 * k] + part[2 * k + 1];
    return part[0];
}

static void norm_rope_row(const uint16_t *x, uint16_t *o, int64_t d,
                          const float *gamma, float eps,
                          const float *cos_row, const float *sin_row)
{
    float xf[4096], y[4096];
    float ss, ms, inv;
    int64_t i, p;
    for (i = 0; i < d; ++i)
        xf[i] = bf16_to_float(x[i]);
    ss = row_sum_of_squares(xf, d);
    ms = ss / (float)d;
    inv = 1.0f / sqrtf(ms + eps);
    for (i = 0; i < d; ++i)
        y[i] = (xf[i] * inv) * gamma[i];
    for (p = 0; p < d / 2; ++p) {
        float c = cos_row[p], s = sin_row[p];
        float a = y[2 * p] * c;
        float bb = y[2 * p + 1] * s;
        float cc = y[2 * p] * s;
        float dd = y[2 * p + 1] * c;
        o[2 * p] = float_to_bf16_rne(a - bb);
        o[2 * p + 1] = float_to_bf16_rne(cc + dd);
    }
}

static int fused_d_ok(int64_t d)
{
    int64_t n;
    if (d < 8 || d > 4096 || d % 8 != 0)
        return 0;
    for (n = d / 8; n > 1; n /= 2)
        if (n % 2 != 0)
            return 0; /* the adjacent-pairing tree needs a power of two */
    return 1;
}

/* The fixed-order sum of squares of one bf16 row of d elements (the first
 * step of the fused row operation), exposed so that tests can pin the order
 * on rows whose partial sums round differently under other orders. */
int oracle_row_sum_of_squares(int64_t d, const uint16_t *x, float *ss)
{
    float xf[4096];
    int64_t i;
    if (!fused_d_ok(d) || !x || !ss)
        return -1;
    for (i = 0; i < d; ++i)
        xf[i] = bf16_to_float(x[i]);
    *ss = row_sum_of_squares(xf, d);
    return 0;
}

/* Mode-0 relayout of one bf16 tensor (q or k) with RMSNorm over d and RoPE
 * at the GLOBAL sequence position of each destination row.  Tables are
 * [s_global][d/2] floats (oracle_rope_table), gamma has d floats. */
static int qknorm_rope_mode0(int world, int64_t b, int64_t d,
                             const int64_t *seq_splits, const int64_t *head_splits,
                             const uint16_t *const *src, uint16_t *const *dst,
                             const float *gamma, float eps,
                             const float *cos_tab, const float *sin_tab, int threads)
{
    geom_t g;
    int r;
    if (!fused_d_ok(d))
        return -1;
    if (geom_init(&g, world, b, d, 2, seq_splits, head_splits) != 0)
        return -1;
    for (r = 0; r < world; ++r) {
        int64_t bi, S;
#pragma omp parallel for collapse(2) schedule(static) if (threads > 1) num_threads(threads)
        for (bi = 0; bi < b; ++bi)
            for (S = 0; S < g.s_global; ++S) {
                int j = seq_owner(&g, S);
                int64_t h;
                for (h = 0; h < g.H[r]; ++h) {
                    const uint16_t *x = src[j]
                        + ((bi * g.S[j] + (S - g.seq_off[j])) * g.n_global
                           + g.head_off[r] + h) * d;
                    uint16_t *o = dst[r] + ((bi * g.s_global + S) * g.H[r] + h) * d;
                    norm_rope_row(x, o, d, gamma, eps,
                                  cos_tab + S * (d / 2), sin_tab + S * (d / 2));
                }
            }
    }
    return 0;
}

int oracle_qknorm_rope_mode0(int world, int64_t b, int64_t d,
                             const int64_t *seq_splits, const int64_t *head_splits,
                             const uint16_t *const *src, uint16_t *const *dst,
                             const float *gamma, float eps,
                             const float *cos_tab, const float *sin_tab)
{
    return qknorm_rope_mode0(world, b, d, seq_splits, head_splits, src, dst, gamma, eps,
                             cos_tab, sin_tab, 1);
}

int oracle_qknorm_rope_mode0_threads(int world, int64_t b, int64_t d,
                                     const int64_t *seq_splits, const int64_t *head_splits,
                                     const uint16_t *const *src, uint16_t *const *dst,
                                     const float *gamma, float eps,
                                     const float *cos_tab, const float *sin_tab, int threads)
{
    if (threads < 1)
        return -1;
    return qknorm_rope_mode0(world, b, d, seq_splits, head_splits, src, dst, gamma, eps,
                             cos_tab, sin_tab, threads);
}

/* The fused definition evaluated on n chosen destination rows.  rows is
 * n x 4 int64: (rank, bi, S, h); out receives n * d bf16 values. */
int oracle_qknorm_rope_mode0_sample(int world, int64_t b, int64_t d,
                                    const int64_t *seq_splits,
                                    const int64_t *head_splits,
                                    const uint16_t *const *src, const float *gamma,
                                    float eps, const float *cos_tab,
                                    const float *sin_tab, int64_t n,
                                    const int64_t *rows, uint16_t *out)
{
    geom_t g;
    int64_t i;
    if (!fused_d_ok(d))
        return -1;
    if (geom_init(&g, world, b, d, 2, seq_splits, head_splits) != 0)
        return -1;
    for (i = 0; i < n; ++i) {
        const int64_t *c = rows + 4 * i;
        int r = (int)c[0], j;
        int64_t bi = c[1], S = c[2], h = c[3];
        const uint16_t *x;
        if (r < 0 || r >= world || bi < 0 || bi >= b || S < 0 || S >= g.s_global
            || h < 0 || h >= g.H[r])
            return -1;
        j = seq_owner(&g, S);
        x = src[j] + ((bi * g.S[j] + (S - g.seq_off[j])) * g.n_global
                      + g.head_off[r] + h) * d;
        norm_rope_row(x, out + i * d, d, gamma, eps, cos_tab + S * (d / 2),
                      sin_tab + S * (d / 2));
    }
    return 0;
}
