/*
 * iir_oracle.c -- plain, single-threaded CPU oracle for the integer motion and PSNR sums.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg use it. It shares no code, header,
 * table or constant with the GPU library: the filter taps are derived here from their definition.
 *
 * What it computes (each step cites the page passage it follows):
 *
 *  - SSE per plane ("ADR-1392: CUDA motion, PSNR and moment kernels add one atomic per block ...",
 *    Context and Decision 2): the sum over the plane of (ref - dist)^2, an exact 64-bit integer.
 *    The page states the sum is integer-exact and order-independent, so the plain definition is
 *    the oracle.
 *
 *  - Blurred luma ("ADR-1392", Decision 4; "Research-0735: CUDA motion kernel ncu hotpath analysis
 *    (576x324)", Key observations 2 and the shared-memory section): a 5x5 separable Gaussian,
 *    radius 2 (a 20-wide tile serves 16 outputs). The vertical pass is rounded with a shift by the
 *    bit depth, the horizontal pass with a shift by 16. Readings where the pages are silent:
 *      taps   g = round(65536 * exp(-k^2/2) / sum_{k=-2..2} exp(-k^2/2)), k = -2..2
 *               (sigma = 1 sampled Gaussian; the sum must be exactly 2^16 so a flat image stays flat)
 *      round  add half of the divisor before each shift (all operands are non-negative)
 *      mirror whole-sample reflection: -1 -> 1, -2 -> 2, n -> n-2, n+1 -> n-3 (needs n >= 3)
 *      V[i][j]  = (sum_k g_k x[m(i+k-2, H)][j] + 2^(bpc-1)) >> bpc
 *      Bl[i][j] = (sum_l g_l V[i][m(j+l-2, W)] + 2^15) >> 16
 *
 *  - SAD ("ADR-1392", Context: motion sums one integer per pixel into one 64-bit accumulator):
 *    sum of |Bl_t - Bl_(t-1)| over the luma plane of the reference video, for every frame that has
 *    a previous frame; the first frame of a clip without a previous frame has no SAD (0, flagged).
 *
 *  - Motion v2, difference first ("ADR-1392", Decision 4: the kernel stages prev - cur and runs
 *    the separable filter on it, vertical pass rounded by the bit depth, horizontal by 16;
 *    "Larger motion tiles ..." alternative: the horizontal sum needs 33 bits): the same taps and
 *    mirror on the signed difference D = prev - cur of consecutive reference luma frames. The
 *    shifts of negative sums are read as floor (arithmetic shifts), with the same half-divisor
 *    added first; SAD2 = sum of |F| over the plane.
 *      V2[i][j] = floor((sum_k g_k D[m(i+k-2, H)][j] + 2^(bpc-1)) / 2^bpc)
 *      F[i][j]  = floor((sum_l g_l V2[i][m(j+l-2, W)] + 2^15) / 2^16)
 *
 *  - Derived scores (host doubles; "ADR-1392", Consequences lists psnr_*, mse_* and the motion
 *    scores): motion = SAD / (256 W H); mse_c = SSE_c / (W_c H_c); psnr_c = 10 log10(peak^2 / mse_c)
 *    with peak = 2^bpc - 1, +inf when SSE_c = 0. Build with -ffp-contract=off.
 *
 * Pins (tests/oracle_pins.py, run without a GPU): brute-force 25-term evaluation per output with
 * numpy's own edge reflection, scipy.ndimage.correlate1d, hand-derived impulse and step responses,
 * flat-plane and bit-depth closed forms, flip/translation invariance, the +-1 error bound against
 * the exact real filter, brute-force SSE/SAD, clip composition and split; planted-mistake copies of
 * this file must each fail one of them (tests/test_oracle_mutants.py). The three readings above
 * (tap values, rounding, mirror) are not fixed by the pages: agreement with the pages on those is
 * parity unpinned; the pins fix that this file computes exactly what the readings say.
 *
 * Planes: 4:2:0, luma W x H, chroma ceil(W/2) x ceil(H/2). 8-bit samples are uint8; 9- to 16-bit
 * samples are little-endian uint16 in [0, 2^bpc - 1] ("ADR-1392", Consequences checks the outputs
 * at 8, 10 and 16 bits). Every function returns 0 on success and a negative value on bad
 * arguments or on a sample outside [0, 2^bpc - 1].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IIRO_OK 0
#define IIRO_EINVAL (-1)
#define IIRO_ERANGE (-2)
#define IIRO_ENOMEM (-3)

/* sigma = 1 sampled Gaussian, 5 taps, scaled to 2^16 and rounded to nearest. */
int iiro_taps(int32_t g[5])
{
    double w[5], s = 0.0;
    for (int k = -2; k <= 2; ++k) {
        w[k + 2] = exp(-0.5 * (double)(k * k));
        s += w[k + 2];
    }
    int64_t total = 0;
    for (int k = 0; k < 5; ++k) {
        g[k] = (int32_t)floor(65536.0 * w[k] / s + 0.5);
        total += g[k];
    }
    return total == 65536 ? IIRO_OK : IIRO_EINVAL;
}

/* Whole-sample mirror of index i into [0, n); only ever called with -2 <= i <= n + 1. */
static int64_t mirror(int64_t i, int64_t n)
{
    if (i < 0)
        i = -i;
    if (i >= n)
        i = 2 * n - 2 - i;
    return i;
}

static int64_t sample(const void *plane, int64_t pitch, int64_t i, int64_t j, int bpc)
{
    const uint8_t *row = (const uint8_t *)plane + i * pitch;
    if (bpc == 8)
        return row[j];
    uint16_t v;
    memcpy(&v, row + 2 * j, 2);
    return v;
}

static int check_range(const void *plane, int64_t pitch, int32_t w, int32_t h, int bpc)
{
    int64_t maxv = ((int64_t)1 << bpc) - 1;
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j)
            if (sample(plane, pitch, i, j, bpc) > maxv)
                return IIRO_ERANGE;
    return IIRO_OK;
}

static int bad_dims(int32_t w, int32_t h, int32_t bpc)
{
    return bpc < 8 || bpc > 16 || w < 1 || h < 1;
}

/* Sum of squared differences of one plane. */
int iiro_sse(const void *ref, int64_t ref_pitch, const void *dist, int64_t dist_pitch, int32_t w,
             int32_t h, int32_t bpc, uint64_t *out)
{
    if (!ref || !dist || !out || bad_dims(w, h, bpc))
        return IIRO_EINVAL;
    if (check_range(ref, ref_pitch, w, h, bpc) || check_range(dist, dist_pitch, w, h, bpc))
        return IIRO_ERANGE;
    uint64_t s = 0;
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j) {
            int64_t d = sample(ref, ref_pitch, i, j, bpc) - sample(dist, dist_pitch, i, j, bpc);
            s += (uint64_t)(d * d);
        }
    *out = s;
    return IIRO_OK;
}

/* Separable blur of one luma plane into out (w x h uint16, row pitch out_pitch elements). */
int iiro_blur(const void *plane, int64_t pitch, int32_t w, int32_t h, int32_t bpc, uint16_t *out,
              int64_t out_pitch)
{
    if (!plane || !out || bad_dims(w, h, bpc) || w < 3 || h < 3 || out_pitch < w)
        return IIRO_EINVAL;
    if (check_range(plane, pitch, w, h, bpc))
        return IIRO_ERANGE;
    int32_t g[5];
    if (iiro_taps(g))
        return IIRO_EINVAL;
    int64_t *v = (int64_t *)malloc(sizeof(int64_t) * (size_t)w * (size_t)h);
    if (!v)
        return IIRO_ENOMEM;
    /* vertical pass, rounded by the bit depth */
    const int64_t vround = (int64_t)1 << (bpc - 1);
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j) {
            int64_t acc = 0;
            for (int k = 0; k < 5; ++k)
                acc += (int64_t)g[k] * sample(plane, pitch, mirror(i + k - 2, h), j, bpc);
            v[i * w + j] = (acc + vround) >> bpc;
        }
    /* horizontal pass, rounded by 16 */
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j) {
            int64_t acc = 0;
            for (int l = 0; l < 5; ++l)
                acc += (int64_t)g[l] * v[i * w + mirror(j + l - 2, w)];
            out[i * out_pitch + j] = (uint16_t)((acc + 32768) >> 16);
        }
    free(v);
    return IIRO_OK;
}

/* Sum of absolute differences of two contiguous w x h uint16 planes. */
int iiro_sad(const uint16_t *a, const uint16_t *b, int32_t w, int32_t h, uint64_t *out)
{
    if (!a || !b || !out || w < 1 || h < 1)
        return IIRO_EINVAL;
    uint64_t s = 0;
    for (int64_t n = 0; n < (int64_t)w * h; ++n)
        s += (uint64_t)(a[n] > b[n] ? a[n] - b[n] : b[n] - a[n]);
    *out = s;
    return IIRO_OK;
}

/*
 * A clip of nframes frame pairs. Every plane array is contiguous: frame t of a plane starts at
 * t * (plane bytes). prev_blur, when not NULL, is the blurred reference luma of the frame before
 * the clip (w x h uint16), so frame 0 also gets a SAD. out receives nframes x 4 sums
 * {SAD, SSE_Y, SSE_U, SSE_V}; has_motion receives 1 where the SAD is defined. last_blur, when not
 * NULL, receives the blurred reference luma of the last frame.
 */
int iiro_clip(const void *ry, const void *ru, const void *rv, const void *dy, const void *du,
              const void *dv, int32_t nframes, int32_t w, int32_t h, int32_t bpc,
              const uint16_t *prev_blur, uint64_t *out, int32_t *has_motion, uint16_t *last_blur)
{
    if (!ry || !ru || !rv || !dy || !du || !dv || !out || !has_motion || nframes < 1 ||
        bad_dims(w, h, bpc) || w < 3 || h < 3)
        return IIRO_EINVAL;
    const int64_t bps = bpc == 8 ? 1 : 2;
    const int32_t wc = (w + 1) / 2, hc = (h + 1) / 2;
    const int64_t ybytes = (int64_t)w * h * bps, cbytes = (int64_t)wc * hc * bps;
    const int64_t n = (int64_t)w * h;
    uint16_t *prev = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n);
    uint16_t *cur = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n);
    if (!prev || !cur) {
        free(prev);
        free(cur);
        return IIRO_ENOMEM;
    }
    int have_prev = prev_blur != NULL;
    if (have_prev)
        memcpy(prev, prev_blur, sizeof(uint16_t) * (size_t)n);
    int rc = IIRO_OK;
    for (int64_t t = 0; t < nframes && rc == IIRO_OK; ++t) {
        const uint8_t *fy = (const uint8_t *)ry + t * ybytes, *gy = (const uint8_t *)dy + t * ybytes;
        const uint8_t *fu = (const uint8_t *)ru + t * cbytes, *gu = (const uint8_t *)du + t * cbytes;
        const uint8_t *fv = (const uint8_t *)rv + t * cbytes, *gv = (const uint8_t *)dv + t * cbytes;
        uint64_t *o = out + 4 * t;
        rc = iiro_sse(fy, w * bps, gy, w * bps, w, h, bpc, &o[1]);
        if (!rc)
            rc = iiro_sse(fu, wc * bps, gu, wc * bps, wc, hc, bpc, &o[2]);
        if (!rc)
            rc = iiro_sse(fv, wc * bps, gv, wc * bps, wc, hc, bpc, &o[3]);
        if (!rc)
            rc = iiro_blur(fy, w * bps, w, h, bpc, cur, w);
        if (rc)
            break;
        o[0] = 0;
        has_motion[t] = have_prev;
        if (have_prev)
            rc = iiro_sad(cur, prev, w, h, &o[0]);
        uint16_t *tmp = prev;
        prev = cur;
        cur = tmp;
        have_prev = 1;
    }
    if (rc == IIRO_OK && last_blur)
        memcpy(last_blur, prev, sizeof(uint16_t) * (size_t)n);
    free(prev);
    free(cur);
    return rc;
}

/* floor(x / 2^s) for any sign of x, written out rather than left to the shift of a negative */
static int64_t floor_shift(int64_t x, int s)
{
    const int64_t d = (int64_t)1 << s;
    return x >= 0 ? x / d : -((-x + d - 1) / d);
}

/*
 * Motion v2 filter of one frame pair: out (w x h int32, row pitch out_pitch elements) receives F,
 * the separable filter of prev - cur with floor rounding. prev and cur share `pitch`.
 */
int iiro_diff_blur(const void *prev, const void *cur, int64_t pitch, int32_t w, int32_t h,
                   int32_t bpc, int32_t *out, int64_t out_pitch)
{
    if (!prev || !cur || !out || bad_dims(w, h, bpc) || w < 3 || h < 3 || out_pitch < w)
        return IIRO_EINVAL;
    if (check_range(prev, pitch, w, h, bpc) || check_range(cur, pitch, w, h, bpc))
        return IIRO_ERANGE;
    int32_t g[5];
    if (iiro_taps(g))
        return IIRO_EINVAL;
    int64_t *v = (int64_t *)malloc(sizeof(int64_t) * (size_t)w * (size_t)h);
    if (!v)
        return IIRO_ENOMEM;
    /* vertical pass on the difference, floor after adding half of 2^bpc */
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j) {
            int64_t acc = 0;
            for (int k = 0; k < 5; ++k) {
                const int64_t r = mirror(i + k - 2, h);
                acc += (int64_t)g[k] * (sample(prev, pitch, r, j, bpc) - sample(cur, pitch, r, j, bpc));
            }
            v[i * w + j] = floor_shift(acc + ((int64_t)1 << (bpc - 1)), bpc);
        }
    /* horizontal pass, floor after adding 2^15 */
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j) {
            int64_t acc = 0;
            for (int l = 0; l < 5; ++l)
                acc += (int64_t)g[l] * v[i * w + mirror(j + l - 2, w)];
            out[i * out_pitch + j] = (int32_t)floor_shift(acc + 32768, 16);
        }
    free(v);
    return IIRO_OK;
}

/*
 * A clip with motion v2: like iiro_clip, but out[4 t] is SAD2 of frames t - 1 and t (sum |F|).
 * prev_luma, when not NULL, is the reference luma of the frame before the clip (w x h samples,
 * contiguous), so frame 0 also has a SAD2.
 */
int iiro_clip_v2(const void *ry, const void *ru, const void *rv, const void *dy, const void *du,
                 const void *dv, int32_t nframes, int32_t w, int32_t h, int32_t bpc,
                 const void *prev_luma, uint64_t *out, int32_t *has_motion)
{
    if (!ry || !ru || !rv || !dy || !du || !dv || !out || !has_motion || nframes < 1 ||
        bad_dims(w, h, bpc) || w < 3 || h < 3)
        return IIRO_EINVAL;
    const int64_t bps = bpc == 8 ? 1 : 2;
    const int32_t wc = (w + 1) / 2, hc = (h + 1) / 2;
    const int64_t ybytes = (int64_t)w * h * bps, cbytes = (int64_t)wc * hc * bps;
    int32_t *f = (int32_t *)malloc(sizeof(int32_t) * (size_t)w * (size_t)h);
    if (!f)
        return IIRO_ENOMEM;
    int rc = IIRO_OK;
    for (int64_t t = 0; t < nframes && rc == IIRO_OK; ++t) {
        const uint8_t *fy = (const uint8_t *)ry + t * ybytes, *gy = (const uint8_t *)dy + t * ybytes;
        const uint8_t *fu = (const uint8_t *)ru + t * cbytes, *gu = (const uint8_t *)du + t * cbytes;
        const uint8_t *fv = (const uint8_t *)rv + t * cbytes, *gv = (const uint8_t *)dv + t * cbytes;
        const void *before = t > 0 ? (const void *)(fy - ybytes) : prev_luma;
        uint64_t *o = out + 4 * t;
        rc = iiro_sse(fy, w * bps, gy, w * bps, w, h, bpc, &o[1]);
        if (!rc)
            rc = iiro_sse(fu, wc * bps, gu, wc * bps, wc, hc, bpc, &o[2]);
        if (!rc)
            rc = iiro_sse(fv, wc * bps, gv, wc * bps, wc, hc, bpc, &o[3]);
        o[0] = 0;
        has_motion[t] = before != NULL;
        if (!rc && before) {
            rc = iiro_diff_blur(before, fy, w * bps, w, h, bpc, f, w);
            for (int64_t n = 0; !rc && n < (int64_t)w * h; ++n)
                o[0] += (uint64_t)(f[n] < 0 ? -(int64_t)f[n] : (int64_t)f[n]);
        }
    }
    free(f);
    return rc;
}

/*
 * Derived scores of one frame: out = {motion, mse_y, mse_u, mse_v, psnr_y, psnr_u, psnr_v}.
 * sums = {SAD, SSE_Y, SSE_U, SSE_V}. motion is 0 when has_motion is 0.
 */
int iiro_scores(int32_t w, int32_t h, int32_t bpc, const uint64_t sums[4], int32_t has_motion,
                double out[7])
{
    if (!sums || !out || bad_dims(w, h, bpc))
        return IIRO_EINVAL;
    const double npx[3] = {(double)w * (double)h, (double)((w + 1) / 2) * (double)((h + 1) / 2),
                           (double)((w + 1) / 2) * (double)((h + 1) / 2)};
    const double peak = (double)(((int64_t)1 << bpc) - 1);
    out[0] = has_motion ? (double)sums[0] / (256.0 * npx[0]) : 0.0;
    for (int c = 0; c < 3; ++c) {
        double mse = (double)sums[1 + c] / npx[c];
        out[1 + c] = mse;
        out[4 + c] = sums[1 + c] == 0 ? INFINITY : 10.0 * log10(peak * peak / mse);
    }
    return IIRO_OK;
}

/*
 * Luma moments of one plane ("ADR-1392: CUDA motion, PSNR and moment kernels add one atomic per
 * block ...", Decision 6 and Consequences: the moment kernel sums the reference and distorted
 * luma and their squares into four accumulators; float_moment reports their means). out receives
 * {sum x, sum x^2} over the plane, exact 64-bit integers.
 */
int iiro_moments(const void *plane, int64_t pitch, int32_t w, int32_t h, int32_t bpc,
                 uint64_t out[2])
{
    if (!plane || !out || bad_dims(w, h, bpc))
        return IIRO_EINVAL;
    if (check_range(plane, pitch, w, h, bpc))
        return IIRO_ERANGE;
    uint64_t s1 = 0, s2 = 0;
    for (int64_t i = 0; i < h; ++i)
        for (int64_t j = 0; j < w; ++j) {
            const uint64_t x = (uint64_t)sample(plane, pitch, i, j, bpc);
            s1 += x;
            s2 += x * x;
        }
    out[0] = s1;
    out[1] = s2;
    return IIRO_OK;
}

/*
 * Second motion score of each frame of a clip ("ADR-1392", Consequences lists the motion2
 * output; the pages give no formula, so this is the reading): frame t's motion2 is the smaller
 * of its own motion and the next frame's, and the clip's last frame keeps its own motion.
 */
int iiro_motion2(const double *motion, int32_t n, double *out)
{
    if (!motion || !out || n < 1)
        return IIRO_EINVAL;
    for (int32_t t = 0; t < n; ++t) {
        const double a = motion[t];
        const double b = t + 1 < n ? motion[t + 1] : a;
        out[t] = b < a ? b : a;
    }
    return IIRO_OK;
}

/*
 * Clip aggregates (reading; the pages name aggregate PSNR outputs without a formula): for plane c
 * the aggregate PSNR is 10 log10(peak^2 / MSE_c) with MSE_c the clip's total squared error over
 * its total sample count (+infinity when the total is 0); the mean motion and mean motion2 are
 * the plain averages of the per-frame scores (frame 0 of a clip without a previous frame scores
 * 0). sums holds n x 4 {SAD, SSE_Y, SSE_U, SSE_V}; out = {apsnr_y, apsnr_u, apsnr_v,
 * mean_motion, mean_motion2}.
 */
int iiro_aggregate(int32_t w, int32_t h, int32_t bpc, const uint64_t *sums,
                   const int32_t *has_motion, int32_t n, double out[5])
{
    if (!sums || !has_motion || !out || n < 1 || bad_dims(w, h, bpc))
        return IIRO_EINVAL;
    double *motion = (double *)malloc(sizeof(double) * (size_t)n);
    double *motion2 = (double *)malloc(sizeof(double) * (size_t)n);
    if (!motion || !motion2) {
        free(motion);
        free(motion2);
        return IIRO_ENOMEM;
    }
    uint64_t total[3] = {0, 0, 0};
    for (int32_t t = 0; t < n; ++t) {
        double s[7];
        int rc = iiro_scores(w, h, bpc, sums + 4 * (int64_t)t, has_motion[t], s);
        if (rc) {
            free(motion);
            free(motion2);
            return rc;
        }
        motion[t] = s[0];
        for (int c = 0; c < 3; ++c)
            total[c] += sums[4 * (int64_t)t + 1 + c];
    }
    iiro_motion2(motion, n, motion2);
    const double npx[3] = {(double)w * (double)h, (double)((w + 1) / 2) * (double)((h + 1) / 2),
                           (double)((w + 1) / 2) * (double)((h + 1) / 2)};
    const double peak = (double)(((int64_t)1 << bpc) - 1);
    const double peak_sq = peak * peak;
    for (int c = 0; c < 3; ++c) {
        const double mse = (double)total[c] / ((double)n * npx[c]);
        out[c] = total[c] == 0 ? INFINITY : 10.0 * log10(peak_sq / mse);
    }
    double m1 = 0.0, m2 = 0.0;
    for (int32_t t = 0; t < n; ++t) {
        m1 += motion[t];
        m2 += motion2[t];
    }
    out[3] = m1 / (double)n;
    out[4] = m2 / (double)n;
    free(motion);
    free(motion2);
    return IIRO_OK;
}
