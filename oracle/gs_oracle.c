/*
 * CPU oracle for the forward tile-based 3D Gaussian-splatting rasterizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant table with the HIP
 * library: every formula below is written out again from the lesson
 * "3D Gaussian Splatting from scratch" (aiengineeringfromscratch.com).
 *
 * Precision.  Every quantity that decides an integer (visibility, depth bits,
 * screen position, radius, tile rectangle, tile count) is computed in IEEE
 * binary32 with no FMA contraction (build with -ffp-contract=off), sums taken
 * left to right, and exp evaluated in binary64 then rounded to binary32.
 * Colour and compositing are computed in binary64.
 *
 * Plain and slow on purpose: the image is a per-pixel loop over every
 * visible Gaussian in global (depth, index) order, keeping those whose tile
 * rectangle contains the pixel's 16x16 tile.
 *
 * Parity unpinned: a few conventions that the lesson does not fix are taken
 * as stated and pinned only by self-consistency -- the sign convention of the
 * degree-3 SH terms, the quaternion component order (w, x, y, z) and
 * handedness, the camera axes (x right, y down, z forward), the pixel (i, j)
 * sampled at (x = j, y = i), and the near-plane value.  Every formula built
 * on them is pinned (tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TILE 16
#define ALPHA_MAX 0.99

/* ------------------------------------------------------------------------ */
/* Per-Gaussian record produced by the projection stage.                   */
/* ------------------------------------------------------------------------ */
typedef struct {
    float R[9], t[3];          /* world -> camera, row-major */
    float fx, fy, cx, cy, znear;
    int32_t width, height;
} oracle_camera;

/* Tile membership rules (option GS_OPT_TILE_TEST of the library). */
#define TILE_TEST_SQUARE 0   /* every tile of [u-r, u+r] x [v-r, v+r] (the pages' rule)              */
#define TILE_TEST_ELLIPSE 1  /* those of them whose pixel-centre box meets the 3-sigma ellipse q <= 9 */

/* Outputs are planes of length n (index g). */
typedef struct {
    float *depth;              /* camera-space z                                 */
    float *mean2d;             /* [2][n]  (u, v) pixel coordinates                */
    float *cov2d;              /* [3][n]  (a, b, c) of the projected covariance   */
    float *conic;              /* [3][n]  (c, -b, a) / det                        */
    float *radius;             /* [n]     ceil(3 sqrt(lambda_max))                */
    float *cov3d;              /* [6][n]  Sigma00,01,02,11,12,22                  */
    int32_t *rect;             /* [4][n]  x0, x1, y0, y1 in tiles, [x0,x1)x[y0,y1) */
    uint32_t *tile_count;      /* [n]                                             */
    double *rgb;               /* [3][n]  SH colour in binary64                   */
    float *ellipse;            /* [5][n]  ymax, dyr, b/c, det/c, c (see oracle_row_span); may be NULL */
} oracle_projected;

/* Clamp that sends NaN to the lower bound (so the int conversion is defined). */
static float clampf_lo(float x, float lo, float hi) {
    if (!(x > lo)) x = lo;
    if (x > hi) x = hi;
    return x;
}

/*
 * Real spherical-harmonic basis up to degree 3 at unit direction (x, y, z).
 * Lesson, section "Étape 6: Évaluation des harmoniques sphériques": the
 * constants and signs of degrees 0-2 are the ones printed there (degree 1
 * enters as -y, +z, -x; degree 2 as +xy, +yz, +(2z^2-x^2-y^2), +xz, +(x^2-y^2)).
 * Degree 3 is not printed; it is the real-SH closed form with normalisation
 * sqrt((2l+1)/(4 pi) (l-|m|)!/(l+|m|)!) * sqrt(2) for m != 0, ordered m=-3..3,
 * and odd m entering with a minus sign like the printed degree-1 band.
 */
static void sh_basis(double x, double y, double z, double Y[16]) {
    const double pi = 3.14159265358979323846;
    const double k00 = 0.5 / sqrt(pi);
    const double k1 = sqrt(3.0 / (4.0 * pi));
    const double k2a = sqrt(15.0 / (4.0 * pi));   /* xy, yz, xz */
    const double k20 = sqrt(5.0 / (16.0 * pi));   /* 2z^2 - x^2 - y^2 */
    const double k22 = sqrt(15.0 / (16.0 * pi));  /* x^2 - y^2 */
    const double k33 = sqrt(35.0 / (32.0 * pi));
    const double k32 = sqrt(105.0 / (4.0 * pi));
    const double k31 = sqrt(21.0 / (32.0 * pi));
    const double k30 = sqrt(7.0 / (16.0 * pi));
    const double k32b = sqrt(105.0 / (16.0 * pi));
    double xx = x * x, yy = y * y, zz = z * z;
    Y[0] = k00;
    Y[1] = -k1 * y;
    Y[2] = k1 * z;
    Y[3] = -k1 * x;
    Y[4] = k2a * x * y;
    Y[5] = k2a * y * z;
    Y[6] = k20 * (2.0 * zz - xx - yy);
    Y[7] = k2a * x * z;
    Y[8] = k22 * (xx - yy);
    Y[9] = -k33 * y * (3.0 * xx - yy);
    Y[10] = k32 * x * y * z;
    Y[11] = -k31 * y * (4.0 * zz - xx - yy);
    Y[12] = k30 * z * (2.0 * zz - 3.0 * xx - 3.0 * yy);
    Y[13] = -k31 * x * (4.0 * zz - xx - yy);
    Y[14] = k32b * z * (xx - yy);
    Y[15] = -k33 * x * (xx - 3.0 * yy);
}

void oracle_sh_basis(double x, double y, double z, double *out16) { sh_basis(x, y, z, out16); }

/*
 * Scale activation (lesson, "Ce qu'un Gaussien porte": log-scales exponentiated
 * at render time): the binary64 exp of the binary32 log-scale, rounded to
 * binary32.  oracle_scale_activation applies it to an array (OpenMP).
 */
static float scale_activation(float log_scale) { return (float)exp((double)log_scale); }

void oracle_scale_activation(int64_t n, const float *log_scale, float *scale) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) scale[i] = scale_activation(log_scale[i]);
}

/*
 * 3D covariance Sigma = R S S^T R^T with R from the normalised quaternion
 * (w, x, y, z) and S = diag(exp(log_scale)).  Lesson, sections "Ce qu'un
 * Gaussien porte" and "Étape 5: De la 2D à la 3D".  binary32, no contraction.
 * Writes Sigma00, 01, 02, 11, 12, 22.
 */
void oracle_cov3d(const float q_in[4], const float ls[3], float out6[6]) {
    float qw = q_in[0], qx = q_in[1], qy = q_in[2], qz = q_in[3];
    float nrm = sqrtf(((qw * qw + qx * qx) + qy * qy) + qz * qz);
    float w = qw / nrm, x = qx / nrm, y = qy / nrm, z = qz / nrm;
    float r[3][3];
    r[0][0] = 1.0f - 2.0f * (y * y + z * z);
    r[0][1] = 2.0f * (x * y - w * z);
    r[0][2] = 2.0f * (x * z + w * y);
    r[1][0] = 2.0f * (x * y + w * z);
    r[1][1] = 1.0f - 2.0f * (x * x + z * z);
    r[1][2] = 2.0f * (y * z - w * x);
    r[2][0] = 2.0f * (x * z - w * y);
    r[2][1] = 2.0f * (y * z + w * x);
    r[2][2] = 1.0f - 2.0f * (x * x + y * y);
    float s[3];
    for (int i = 0; i < 3; ++i) s[i] = scale_activation(ls[i]);
    float m[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) m[i][j] = r[i][j] * s[j];
    float S[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) S[i][j] = (m[i][0] * m[j][0] + m[i][1] * m[j][1]) + m[i][2] * m[j][2];
    out6[0] = S[0][0]; out6[1] = S[0][1]; out6[2] = S[0][2];
    out6[3] = S[1][1]; out6[4] = S[1][2]; out6[5] = S[2][2];
}

/*
 * Projection of one Gaussian.  Lesson, section "L'étape de projection":
 * mu' = project(mu), Sigma' = J W Sigma W^T J^T, with W the camera's
 * world->camera rotation and J the Jacobian of the perspective map taken at
 * the camera-space mean t = W mu + t_cw.  Culled when t_z <= znear or the 2D
 * covariance is not positive definite.  The screen radius is three standard
 * deviations along the major eigen-axis, r = ceil(3 sqrt(lambda_max)).
 * Tile assignment (flowchart "Assign to tiles (16x16 screen-space)") takes
 * every 16x16 tile met by the square [u-r, u+r] x [v-r, v+r].
 */
/*
 * Exact 3-sigma footprint per tile row (tile test ELLIPSE; an integer rule that
 * the library's GS_TILE_ELLIPSE option states the same way).  With the 2D
 * covariance [[a, b], [b, c]], the ellipse q <= 9 cut at height dy is centred at
 * (b/c) dy with half-width sqrt((det/c) (9 - dy^2/c)), |dy| <= 3 sqrt(c); its right
 * end is largest at dy = 3b/sqrt(a) and its left end smallest at -3b/sqrt(a).  For
 * tile row ty (pixel-centre rows 16 ty .. 16 ty + 15) those heights are clamped to
 * the row's band, giving the x-extent [u + xl, u + xr]; the kept tiles are the tx of
 * the rectangle [x0, x1) whose pixel-centre columns 16 tx .. 16 tx + 15 meet it.
 * binary32 in this order, no contraction; E = (ymax, dyr, bc, kc, c).  Writes the
 * half-open span [*a, *b) (empty: *a == *b).
 */
void oracle_row_span(float u, float v, const float E[5], int32_t x0, int32_t x1, int32_t ty, int32_t *pa,
                     int32_t *pb) {
    const float ymax = E[0], dyr = E[1], bc = E[2], kc = E[3], c = E[4];
    *pa = *pb = x0;
    const float p = (float)(16 * ty) - v;
    const float q = (float)(16 * ty + 15) - v;
    const float lo = fmaxf(p, -ymax), hi = fminf(q, ymax);
    if (!(lo <= hi)) return;
    const float dr = fminf(fmaxf(dyr, lo), hi);
    const float dl = fminf(fmaxf(-dyr, lo), hi);
    const float tr = fmaxf(9.0f - (dr * dr) / c, 0.0f);
    const float tl = fmaxf(9.0f - (dl * dl) / c, 0.0f);
    const float xr = bc * dr + sqrtf(kc * tr);
    const float xl = bc * dl - sqrtf(kc * tl);
    float fa = ceilf(((u + xl) - 15.0f) * 0.0625f);
    float fb = floorf((u + xr) * 0.0625f) + 1.0f;
    fa = fmaxf(fa, (float)x0);
    fb = fminf(fb, (float)x1);
    if (!(fa < fb)) return;
    *pa = (int32_t)fa;
    *pb = (int32_t)fb;
}

/* Ellipse parameters of oracle_row_span from the 2D covariance (binary32, this order). */
static void ellipse_params(float a, float b, float c, float det, float E[5]) {
    E[0] = 3.0f * sqrtf(c);
    E[1] = (3.0f * b) / sqrtf(a);
    E[2] = b / c;
    E[3] = det / c;
    E[4] = c;
}

/* Whether tile (tx, ty) of Gaussian g's rectangle is one of its pairs. */
int32_t oracle_tile_kept(int64_t n, int64_t g, const float *mean2d, const float *ellipse, const int32_t *rect,
                         int32_t tile_test, int32_t tx, int32_t ty) {
    if (tx < rect[g] || tx >= rect[n + g] || ty < rect[2 * n + g] || ty >= rect[3 * n + g]) return 0;
    if (tile_test != TILE_TEST_ELLIPSE) return 1;
    float E[5];
    for (int k = 0; k < 5; ++k) E[k] = ellipse[k * n + g];
    if (!(E[4] > 0.0f) || !(E[0] > 0.0f)) return 1;   /* degenerate covariance: the whole rectangle */
    int32_t a, b;
    oracle_row_span(mean2d[g], mean2d[n + g], E, rect[g], rect[n + g], ty, &a, &b);
    return tx >= a && tx < b;
}

void oracle_preprocess_ex(int64_t n, int32_t sh_degree, const float *mean, const float *quat,
                          const float *log_scale, const float *opacity, const float *sh,
                          const oracle_camera *cam, int32_t tile_test, oracle_projected *out);

void oracle_preprocess(int64_t n, int32_t sh_degree, const float *mean, const float *quat,
                       const float *log_scale, const float *opacity, const float *sh,
                       const oracle_camera *cam, oracle_projected *out) {
    oracle_preprocess_ex(n, sh_degree, mean, quat, log_scale, opacity, sh, cam, TILE_TEST_SQUARE, out);
}

void oracle_preprocess_ex(int64_t n, int32_t sh_degree, const float *mean, const float *quat,
                          const float *log_scale, const float *opacity, const float *sh,
                          const oracle_camera *cam, int32_t tile_test, oracle_projected *out) {
    (void)opacity;
    const int32_t tiles_x = (cam->width + TILE - 1) / TILE;
    const int32_t tiles_y = (cam->height + TILE - 1) / TILE;
    const float *W = cam->R;
    const int K = (sh_degree + 1) * (sh_degree + 1);
    /* camera centre C = -R^T t, binary64 (colour path only) */
    double C[3];
    for (int i = 0; i < 3; ++i)
        C[i] = -((double)W[0 * 3 + i] * cam->t[0] + (double)W[1 * 3 + i] * cam->t[1] +
                 (double)W[2 * 3 + i] * cam->t[2]);

    for (int64_t g = 0; g < n; ++g) {
        float mx = mean[g], my = mean[n + g], mz = mean[2 * n + g];
        float tx = ((W[0] * mx + W[1] * my) + W[2] * mz) + cam->t[0];
        float ty = ((W[3] * mx + W[4] * my) + W[5] * mz) + cam->t[1];
        float tz = ((W[6] * mx + W[7] * my) + W[8] * mz) + cam->t[2];
        out->depth[g] = tz;
        out->tile_count[g] = 0;
        for (int k = 0; k < 4; ++k) out->rect[k * n + g] = 0;

        float q[4] = {quat[g], quat[n + g], quat[2 * n + g], quat[3 * n + g]};
        float ls[3] = {log_scale[g], log_scale[n + g], log_scale[2 * n + g]};
        float S6[6];
        oracle_cov3d(q, ls, S6);
        for (int k = 0; k < 6; ++k) out->cov3d[k * n + g] = S6[k];
        float S[3][3] = {{S6[0], S6[1], S6[2]}, {S6[1], S6[3], S6[4]}, {S6[2], S6[4], S6[5]}};

        float j00 = cam->fx / tz;
        float j02 = -(cam->fx * tx) / (tz * tz);
        float j11 = cam->fy / tz;
        float j12 = -(cam->fy * ty) / (tz * tz);
        float T[2][3];
        for (int k = 0; k < 3; ++k) {
            T[0][k] = j00 * W[0 * 3 + k] + j02 * W[2 * 3 + k];
            T[1][k] = j11 * W[1 * 3 + k] + j12 * W[2 * 3 + k];
        }
        float U[2][3];
        for (int i = 0; i < 2; ++i)
            for (int k = 0; k < 3; ++k) U[i][k] = (T[i][0] * S[0][k] + T[i][1] * S[1][k]) + T[i][2] * S[2][k];
        float a = (U[0][0] * T[0][0] + U[0][1] * T[0][1]) + U[0][2] * T[0][2];
        float b = (U[0][0] * T[1][0] + U[0][1] * T[1][1]) + U[0][2] * T[1][2];
        float c = (U[1][0] * T[1][0] + U[1][1] * T[1][1]) + U[1][2] * T[1][2];
        float det = a * c - b * b;
        float mid = 0.5f * (a + c);
        float hd = 0.5f * (a - c);
        float lam = mid + sqrtf(hd * hd + b * b);
        float r = ceilf(3.0f * sqrtf(lam));
        float u = cam->fx * (tx / tz) + cam->cx;
        float v = cam->fy * (ty / tz) + cam->cy;
        out->mean2d[g] = u;
        out->mean2d[n + g] = v;
        out->cov2d[g] = a;
        out->cov2d[n + g] = b;
        out->cov2d[2 * n + g] = c;
        out->conic[g] = c / det;
        out->conic[n + g] = -b / det;
        out->conic[2 * n + g] = a / det;
        out->radius[g] = r;

        /* SH colour in the direction from the camera centre to the mean. */
        double dx = (double)mx - C[0], dy = (double)my - C[1], dz = (double)mz - C[2];
        double dn = sqrt(dx * dx + dy * dy + dz * dz);
        double Y[16];
        sh_basis(dx / dn, dy / dn, dz / dn, Y);
        for (int ch = 0; ch < 3; ++ch) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += Y[k] * (double)sh[(int64_t)(k * 3 + ch) * n + g];
            out->rgb[ch * n + g] = acc;
        }

        if (!(tz > cam->znear)) continue;
        if (!(det > 0.0f)) continue;
        int32_t x0 = (int32_t)clampf_lo(floorf((u - r) * 0.0625f), 0.0f, (float)tiles_x);
        int32_t x1 = (int32_t)clampf_lo(floorf((u + r) * 0.0625f) + 1.0f, 0.0f, (float)tiles_x);
        int32_t y0 = (int32_t)clampf_lo(floorf((v - r) * 0.0625f), 0.0f, (float)tiles_y);
        int32_t y1 = (int32_t)clampf_lo(floorf((v + r) * 0.0625f) + 1.0f, 0.0f, (float)tiles_y);
        if (x1 <= x0 || y1 <= y0) continue;
        out->rect[g] = x0;
        out->rect[n + g] = x1;
        out->rect[2 * n + g] = y0;
        out->rect[3 * n + g] = y1;
        float E[5];
        ellipse_params(a, b, c, det, E);
        if (out->ellipse)
            for (int k = 0; k < 5; ++k) out->ellipse[k * n + g] = E[k];
        if (tile_test == TILE_TEST_ELLIPSE && E[4] > 0.0f && E[0] > 0.0f) {
            uint32_t count = 0;
            for (int32_t ty = y0; ty < y1; ++ty) {
                int32_t sa, sb;
                oracle_row_span(u, v, E, x0, x1, ty, &sa, &sb);
                count += (uint32_t)(sb - sa);
            }
            out->tile_count[g] = count;
        } else {
            out->tile_count[g] = (uint32_t)((x1 - x0) * (y1 - y0));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Binning: (tile, depth) keys of every (Gaussian, tile) pair, sorted.      */
/* ------------------------------------------------------------------------ */
static uint32_t float_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

typedef struct {
    uint64_t key;
    uint32_t val;
} kv_pair;

static int cmp_kv(const void *pa, const void *pb) {
    const kv_pair *a = (const kv_pair *)pa, *b = (const kv_pair *)pb;
    if (a->key != b->key) return a->key < b->key ? -1 : 1;
    if (a->val != b->val) return a->val < b->val ? -1 : 1;
    return 0;
}

int64_t oracle_total_pairs(int64_t n, const uint32_t *tile_count) {
    int64_t m = 0;
    for (int64_t g = 0; g < n; ++g) m += tile_count[g];
    return m;
}

/*
 * Lists every (Gaussian, tile) pair in Gaussian order, tiles row-major over
 * the rectangle, keyed (tile_id << 32) | bits(depth) with the Gaussian index
 * as value; then orders the pairs by (key, index) and records for each tile
 * the half-open range of its entries ((0,0) for an empty tile).  Flowchart
 * "Assign to tiles" then "Depth-sort per tile"; camera-space z is the sort
 * depth (section "Étape 5").  Equal depths keep ascending Gaussian index.
 * Any output pointer may be NULL.
 */
void oracle_bin_ex(int64_t n, const float *depth, const int32_t *rect, const uint32_t *tile_count,
                   int32_t tiles_x, int32_t tiles_y, const float *mean2d, const float *ellipse, int32_t tile_test,
                   uint64_t *keys_unsorted, uint32_t *vals_unsorted, uint64_t *keys_sorted, uint32_t *vals_sorted,
                   uint32_t *ranges);

void oracle_bin(int64_t n, const float *depth, const int32_t *rect, const uint32_t *tile_count,
                int32_t tiles_x, int32_t tiles_y, uint64_t *keys_unsorted, uint32_t *vals_unsorted,
                uint64_t *keys_sorted, uint32_t *vals_sorted, uint32_t *ranges) {
    oracle_bin_ex(n, depth, rect, tile_count, tiles_x, tiles_y, NULL, NULL, TILE_TEST_SQUARE, keys_unsorted,
                  vals_unsorted, keys_sorted, vals_sorted, ranges);
}

/* As oracle_bin; with tile_test ELLIPSE only the kept tiles of each rectangle are
 * listed (still row-major), which needs mean2d and ellipse. */
void oracle_bin_ex(int64_t n, const float *depth, const int32_t *rect, const uint32_t *tile_count,
                   int32_t tiles_x, int32_t tiles_y, const float *mean2d, const float *ellipse, int32_t tile_test,
                   uint64_t *keys_unsorted, uint32_t *vals_unsorted, uint64_t *keys_sorted, uint32_t *vals_sorted,
                   uint32_t *ranges) {
    int64_t m = oracle_total_pairs(n, tile_count);
    kv_pair *pairs = (kv_pair *)malloc(sizeof(kv_pair) * (size_t)(m > 0 ? m : 1));
    int64_t e = 0;
    for (int64_t g = 0; g < n; ++g) {
        if (tile_count[g] == 0) continue;
        int32_t x0 = rect[g], x1 = rect[n + g], y0 = rect[2 * n + g], y1 = rect[3 * n + g];
        for (int32_t ty = y0; ty < y1; ++ty)
            for (int32_t tx = x0; tx < x1; ++tx) {
                if (tile_test == TILE_TEST_ELLIPSE &&
                    !oracle_tile_kept(n, g, mean2d, ellipse, rect, tile_test, tx, ty))
                    continue;
                uint64_t tile = (uint64_t)(ty * tiles_x + tx);
                pairs[e].key = (tile << 32) | float_bits(depth[g]);
                pairs[e].val = (uint32_t)g;
                ++e;
            }
    }
    if (keys_unsorted)
        for (int64_t i = 0; i < m; ++i) keys_unsorted[i] = pairs[i].key;
    if (vals_unsorted)
        for (int64_t i = 0; i < m; ++i) vals_unsorted[i] = pairs[i].val;
    qsort(pairs, (size_t)m, sizeof(kv_pair), cmp_kv);
    if (keys_sorted)
        for (int64_t i = 0; i < m; ++i) keys_sorted[i] = pairs[i].key;
    if (vals_sorted)
        for (int64_t i = 0; i < m; ++i) vals_sorted[i] = pairs[i].val;
    if (ranges) {
        int64_t tiles = (int64_t)tiles_x * tiles_y;
        for (int64_t t = 0; t < 2 * tiles; ++t) ranges[t] = 0;
        for (int64_t i = 0; i < m; ++i) {
            int64_t t = (int64_t)(pairs[i].key >> 32);
            if (i == 0 || (int64_t)(pairs[i - 1].key >> 32) != t) ranges[2 * t] = (uint32_t)i;
            ranges[2 * t + 1] = (uint32_t)(i + 1);
        }
    }
    free(pairs);
}

/* ------------------------------------------------------------------------ */
/* Compositing (binary64).                                                 */
/* ------------------------------------------------------------------------ */
typedef struct {
    float depth;
    uint32_t g;
} depth_order;

static int cmp_depth(const void *pa, const void *pb) {
    const depth_order *a = (const depth_order *)pa, *b = (const depth_order *)pb;
    if (a->depth != b->depth) return a->depth < b->depth ? -1 : 1;
    return a->g < b->g ? -1 : (a->g > b->g ? 1 : 0);
}

/*
 * Front-to-back alpha compositing.  Lesson, section "La règle de composition
 * alpha": C = sum_i alpha_i T_i c_i, T_i = prod_{j<i} (1 - alpha_j),
 * alpha_i = o_i exp(-0.5 d^T Sigma'^-1 d); the 2D rasteriser of "Étape 2"
 * clamps alpha to at most 0.99 and samples pixel (i, j) at x = j, y = i.
 *
 * For each requested pixel, walks every Gaussian with tile_count > 0 in
 * ascending (depth, index) and blends those whose tile rectangle holds the
 * pixel's tile (all of them when support_all != 0).  When t_eps > 0 the pixel
 * stops right after the blend that brings T below t_eps.  The background
 * enters as C + T_final * bg.
 *
 * pixels: NULL for the whole image (row-major), else n_pix flat indices y*W+x.
 * out_rgb[n_pix*3], out_T[n_pix], out_count[n_pix] (blended pairs); out_T and
 * out_count may be NULL.
 */
void oracle_composite_ex(int64_t n, const float *mean2d, const float *conic, const float *opacity,
                         const double *rgb, const float *depth, const int32_t *rect,
                         const uint32_t *tile_count, const float *ellipse, int32_t tile_test, int32_t width,
                         int32_t height, const double bg[3], int32_t support_all, double t_eps,
                         const int64_t *pixels, int64_t n_pix, double *out_rgb, double *out_T, int64_t *out_count);

void oracle_composite(int64_t n, const float *mean2d, const float *conic, const float *opacity,
                      const double *rgb, const float *depth, const int32_t *rect,
                      const uint32_t *tile_count, int32_t width, int32_t height, const double bg[3],
                      int32_t support_all, double t_eps, const int64_t *pixels, int64_t n_pix,
                      double *out_rgb, double *out_T, int64_t *out_count) {
    oracle_composite_ex(n, mean2d, conic, opacity, rgb, depth, rect, tile_count, NULL, TILE_TEST_SQUARE, width,
                        height, bg, support_all, t_eps, pixels, n_pix, out_rgb, out_T, out_count);
}

/* As oracle_composite; with tile_test ELLIPSE a Gaussian reaches a pixel only when the
 * pixel's tile is one of its kept tiles (oracle_tile_kept). */
void oracle_composite_ex(int64_t n, const float *mean2d, const float *conic, const float *opacity,
                         const double *rgb, const float *depth, const int32_t *rect,
                         const uint32_t *tile_count, const float *ellipse, int32_t tile_test, int32_t width,
                         int32_t height, const double bg[3], int32_t support_all, double t_eps,
                         const int64_t *pixels, int64_t n_pix, double *out_rgb, double *out_T, int64_t *out_count) {
    depth_order *order = (depth_order *)malloc(sizeof(depth_order) * (size_t)(n > 0 ? n : 1));
    int64_t nv = 0;
    for (int64_t g = 0; g < n; ++g)
        if (tile_count[g] > 0) {
            order[nv].depth = depth[g];
            order[nv].g = (uint32_t)g;
            ++nv;
        }
    qsort(order, (size_t)nv, sizeof(depth_order), cmp_depth);
    if (!pixels) n_pix = (int64_t)width * height;

#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t p = 0; p < n_pix; ++p) {
        int64_t flat = pixels ? pixels[p] : p;
        int32_t px = (int32_t)(flat % width), py = (int32_t)(flat / width);
        int32_t tx = px / TILE, ty = py / TILE;
        double T = 1.0, C[3] = {0.0, 0.0, 0.0};
        int64_t cnt = 0;
        for (int64_t k = 0; k < nv; ++k) {
            int64_t g = order[k].g;
            if (!support_all) {
                if (tx < rect[g] || tx >= rect[n + g] || ty < rect[2 * n + g] || ty >= rect[3 * n + g])
                    continue;
                if (tile_test == TILE_TEST_ELLIPSE &&
                    !oracle_tile_kept(n, g, mean2d, ellipse, rect, tile_test, tx, ty))
                    continue;
            }
            double dx = (double)px - (double)mean2d[g];
            double dy = (double)py - (double)mean2d[n + g];
            double q = (double)conic[g] * dx * dx + 2.0 * (double)conic[n + g] * dx * dy +
                       (double)conic[2 * n + g] * dy * dy;
            double alpha = (double)opacity[g] * exp(-0.5 * q);
            if (alpha > ALPHA_MAX) alpha = ALPHA_MAX;
            for (int ch = 0; ch < 3; ++ch) C[ch] += T * alpha * rgb[ch * n + g];
            T *= (1.0 - alpha);
            ++cnt;
            if (t_eps > 0.0 && T < t_eps) break;
        }
        for (int ch = 0; ch < 3; ++ch) out_rgb[p * 3 + ch] = C[ch] + T * bg[ch];
        if (out_T) out_T[p] = T;
        if (out_count) out_count[p] = cnt;
    }
    free(order);
}
