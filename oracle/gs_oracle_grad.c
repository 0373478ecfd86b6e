/*
 * CPU oracle for the gradients of the Gaussian-splatting rasterizer.
 *
 * TEST INFRASTRUCTURE ONLY, like gs_oracle.c: nothing on the product path may
 * call, link or load it.  It shares no code with the HIP library.
 *
 * The lesson "3D Gaussian Splatting from scratch" (aiengineeringfromscratch.com),
 * section "Pourquoi est-ce différenciable", states that projection, tile
 * assignment, alpha compositing and the SH evaluation are differentiable in
 * the Gaussian parameters (mu, q, s, opacity, SH coefficients).  This file
 * writes that derivative out by hand, in binary64:
 *
 *   oracle_project64          the projection of gs_oracle.c (sections
 *                             "L'étape de projection", "Étape 5", "Étape 6")
 *                             in binary64, with no integer decision;
 *   oracle_project_backward   its vector-Jacobian product;
 *   oracle_composite_fixed    front-to-back compositing (section "La règle de
 *                             composition alpha") over FIXED per-pixel lists:
 *                             the Gaussians one of whose tiles (the rectangle,
 *                             or its exact-footprint part) is the pixel's, in a
 *                             given depth order, cut after a given count per
 *                             pixel (or at T < t_eps);
 *   oracle_composite_backward its vector-Jacobian product.
 *
 * With the lists held fixed the image is a smooth function of the screen
 * quantities, so every routine here is checked against central finite
 * differences of its forward partner (tests/test_oracle_grad.py).  The tile
 * rectangles, the depth order and the per-pixel cut are integer decisions: the
 * gradient treats them as constants, as the lesson's training loop does.
 *
 * Camera array cam[16]: R[9] (world->camera, row-major), t[3], fx, fy, cx, cy.
 * Planes are [component][n] as in gs_oracle.c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TILE 16
#define ALPHA_MAX 0.99

void oracle_sh_basis(double x, double y, double z, double *out16);

/* Gradient of the 16 real SH basis polynomials (gs_oracle.c, sh_basis) with
 * respect to (x, y, z), taken as polynomials before any normalisation. */
static void sh_basis_grad(double x, double y, double z, double G[16][3]) {
    const double pi = 3.14159265358979323846;
    const double k1 = sqrt(3.0 / (4.0 * pi));
    const double k2a = sqrt(15.0 / (4.0 * pi));
    const double k20 = sqrt(5.0 / (16.0 * pi));
    const double k22 = sqrt(15.0 / (16.0 * pi));
    const double k33 = sqrt(35.0 / (32.0 * pi));
    const double k32 = sqrt(105.0 / (4.0 * pi));
    const double k31 = sqrt(21.0 / (32.0 * pi));
    const double k30 = sqrt(7.0 / (16.0 * pi));
    const double k32b = sqrt(105.0 / (16.0 * pi));
    const double xx = x * x, yy = y * y, zz = z * z;
    memset(G, 0, sizeof(double) * 48);
    /* degree 1: -k1 y, k1 z, -k1 x */
    G[1][1] = -k1;
    G[2][2] = k1;
    G[3][0] = -k1;
    /* degree 2 */
    G[4][0] = k2a * y; G[4][1] = k2a * x;                        /* k2a x y */
    G[5][1] = k2a * z; G[5][2] = k2a * y;                        /* k2a y z */
    G[6][0] = -2.0 * k20 * x; G[6][1] = -2.0 * k20 * y; G[6][2] = 4.0 * k20 * z;  /* k20 (2zz-xx-yy) */
    G[7][0] = k2a * z; G[7][2] = k2a * x;                        /* k2a x z */
    G[8][0] = 2.0 * k22 * x; G[8][1] = -2.0 * k22 * y;           /* k22 (xx-yy) */
    /* degree 3 */
    G[9][0] = -k33 * 6.0 * x * y;                                /* -k33 y (3xx - yy) */
    G[9][1] = -k33 * (3.0 * xx - 3.0 * yy);
    G[10][0] = k32 * y * z; G[10][1] = k32 * x * z; G[10][2] = k32 * x * y;   /* k32 x y z */
    G[11][0] = 2.0 * k31 * x * y;                                /* -k31 y (4zz - xx - yy) */
    G[11][1] = -k31 * (4.0 * zz - xx - 3.0 * yy);
    G[11][2] = -8.0 * k31 * y * z;
    G[12][0] = -6.0 * k30 * x * z;                               /* k30 z (2zz - 3xx - 3yy) */
    G[12][1] = -6.0 * k30 * y * z;
    G[12][2] = k30 * (6.0 * zz - 3.0 * xx - 3.0 * yy);
    G[13][0] = -k31 * (4.0 * zz - 3.0 * xx - yy);                /* -k31 x (4zz - xx - yy) */
    G[13][1] = 2.0 * k31 * x * y;
    G[13][2] = -8.0 * k31 * x * z;
    G[14][0] = 2.0 * k32b * x * z;                               /* k32b z (xx - yy) */
    G[14][1] = -2.0 * k32b * y * z;
    G[14][2] = k32b * (xx - yy);
    G[15][0] = -k33 * (3.0 * xx - 3.0 * yy);                     /* -k33 x (xx - 3yy) */
    G[15][1] = 6.0 * k33 * x * y;
}

/* Per-Gaussian intermediate values of the binary64 projection. */
typedef struct {
    double qn, w, x, y, z;     /* quaternion norm and unit quaternion */
    double R[3][3], s[3], M[3][3], S[3][3];
    double t[3];               /* camera-space mean */
    double T0[3], T1[3];       /* rows of J W */
    double a, b, c, det;       /* 2D covariance [[a, b], [b, c]] */
    double u, v, A, B, C;      /* mean2d, conic */
    double dir[3], dn, d[3];   /* camera centre -> mean, its length, unit direction */
} proj64;

static void camera_centre(const double cam[16], double Cc[3]) {
    for (int i = 0; i < 3; ++i)
        Cc[i] = -(cam[0 * 3 + i] * cam[9] + cam[1 * 3 + i] * cam[10] + cam[2 * 3 + i] * cam[11]);
}

static void project_one(int64_t n, int64_t g, const double *mean, const double *quat, const double *log_scale,
                        const double cam[16], proj64 *P) {
    const double *W = cam;
    const double fx = cam[12], fy = cam[13], cx = cam[14], cy = cam[15];
    double mu[3] = {mean[g], mean[n + g], mean[2 * n + g]};
    double q[4] = {quat[g], quat[n + g], quat[2 * n + g], quat[3 * n + g]};
    P->qn = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
    double w = q[0] / P->qn, x = q[1] / P->qn, y = q[2] / P->qn, z = q[3] / P->qn;
    P->w = w; P->x = x; P->y = y; P->z = z;
    double (*R)[3] = P->R;
    R[0][0] = 1.0 - 2.0 * (y * y + z * z);
    R[0][1] = 2.0 * (x * y - w * z);
    R[0][2] = 2.0 * (x * z + w * y);
    R[1][0] = 2.0 * (x * y + w * z);
    R[1][1] = 1.0 - 2.0 * (x * x + z * z);
    R[1][2] = 2.0 * (y * z - w * x);
    R[2][0] = 2.0 * (x * z - w * y);
    R[2][1] = 2.0 * (y * z + w * x);
    R[2][2] = 1.0 - 2.0 * (x * x + y * y);
    for (int j = 0; j < 3; ++j) P->s[j] = exp(log_scale[j * n + g]);
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) P->M[i][j] = R[i][j] * P->s[j];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            P->S[i][j] = P->M[i][0] * P->M[j][0] + P->M[i][1] * P->M[j][1] + P->M[i][2] * P->M[j][2];
    for (int i = 0; i < 3; ++i) P->t[i] = W[i * 3] * mu[0] + W[i * 3 + 1] * mu[1] + W[i * 3 + 2] * mu[2] + cam[9 + i];
    const double tx = P->t[0], ty = P->t[1], tz = P->t[2];
    const double j00 = fx / tz, j02 = -fx * tx / (tz * tz), j11 = fy / tz, j12 = -fy * ty / (tz * tz);
    for (int k = 0; k < 3; ++k) {
        P->T0[k] = j00 * W[k] + j02 * W[6 + k];
        P->T1[k] = j11 * W[3 + k] + j12 * W[6 + k];
    }
    double U0[3], U1[3];
    for (int k = 0; k < 3; ++k) {
        U0[k] = P->T0[0] * P->S[0][k] + P->T0[1] * P->S[1][k] + P->T0[2] * P->S[2][k];
        U1[k] = P->T1[0] * P->S[0][k] + P->T1[1] * P->S[1][k] + P->T1[2] * P->S[2][k];
    }
    P->a = U0[0] * P->T0[0] + U0[1] * P->T0[1] + U0[2] * P->T0[2];
    P->b = U0[0] * P->T1[0] + U0[1] * P->T1[1] + U0[2] * P->T1[2];
    P->c = U1[0] * P->T1[0] + U1[1] * P->T1[1] + U1[2] * P->T1[2];
    P->det = P->a * P->c - P->b * P->b;
    P->u = fx * tx / tz + cx;
    P->v = fy * ty / tz + cy;
    P->A = P->c / P->det;
    P->B = -P->b / P->det;
    P->C = P->a / P->det;
    double Cc[3];
    camera_centre(cam, Cc);
    for (int i = 0; i < 3; ++i) P->dir[i] = mu[i] - Cc[i];
    P->dn = sqrt(P->dir[0] * P->dir[0] + P->dir[1] * P->dir[1] + P->dir[2] * P->dir[2]);
    for (int i = 0; i < 3; ++i) P->d[i] = P->dir[i] / P->dn;
}

/*
 * binary64 projection: mean2d [2][n], conic [3][n] (A, B, C with
 * q = A dx^2 + 2 B dx dy + C dy^2), rgb [3][n] = sum_k Y_k(d) sh[k], cov2d
 * [3][n] (a, b, c) and depth [n] (camera-space z).  No culling: every
 * Gaussian in front of the camera gets values.  Any output may be NULL.
 */
void oracle_project64(int64_t n, int32_t K, const double *mean, const double *quat, const double *log_scale,
                      const double *sh, const double cam[16], double *mean2d, double *conic, double *rgb,
                      double *cov2d, double *depth) {
    for (int64_t g = 0; g < n; ++g) {
        proj64 P;
        project_one(n, g, mean, quat, log_scale, cam, &P);
        if (mean2d) { mean2d[g] = P.u; mean2d[n + g] = P.v; }
        if (conic) { conic[g] = P.A; conic[n + g] = P.B; conic[2 * n + g] = P.C; }
        if (cov2d) { cov2d[g] = P.a; cov2d[n + g] = P.b; cov2d[2 * n + g] = P.c; }
        if (depth) depth[g] = P.t[2];
        if (rgb) {
            double Y[16];
            oracle_sh_basis(P.d[0], P.d[1], P.d[2], Y);
            for (int ch = 0; ch < 3; ++ch) {
                double acc = 0.0;
                for (int k = 0; k < K; ++k) acc += Y[k] * sh[(int64_t)(k * 3 + ch) * n + g];
                rgb[(int64_t)ch * n + g] = acc;
            }
        }
    }
}

/*
 * Vector-Jacobian product of oracle_project64 (chain rule written out step
 * by step, in the reverse order of the forward):
 *   conic = adj(cov2d) / det           -> d cov2d
 *   cov2d = T Sigma T^T, T = J(t) W    -> d Sigma, d T -> d J -> d t
 *   mean2d = (fx tx/tz + cx, fy ty/tz + cy) -> d t;  d mean += W^T d t
 *   Sigma = M M^T, M = R(q/|q|) diag(exp(log_scale)) -> d q, d log_scale
 *   rgb = sum_k Y_k(d) sh[k], d = (mean - C)/|mean - C| -> d sh, d mean
 * Inputs g_mean2d [2][n], g_conic [3][n], g_rgb [3][n] (any may be NULL =
 * zero).  Outputs (overwritten): g_mean [3][n], g_quat [4][n],
 * g_log_scale [3][n], g_sh [K*3][n].
 */
void oracle_project_backward(int64_t n, int32_t K, const double *mean, const double *quat,
                             const double *log_scale, const double *sh, const double cam[16],
                             const double *g_mean2d, const double *g_conic, const double *g_rgb,
                             double *g_mean, double *g_quat, double *g_log_scale, double *g_sh) {
    const double *W = cam;
    const double fx = cam[12], fy = cam[13];
    for (int64_t g = 0; g < n; ++g) {
        proj64 P;
        project_one(n, g, mean, quat, log_scale, cam, &P);
        const double du = g_mean2d ? g_mean2d[g] : 0.0, dv = g_mean2d ? g_mean2d[n + g] : 0.0;
        const double dA = g_conic ? g_conic[g] : 0.0, dB = g_conic ? g_conic[n + g] : 0.0;
        const double dC = g_conic ? g_conic[2 * n + g] : 0.0;
        const double a = P.a, b = P.b, c = P.c, det2 = P.det * P.det;
        /* conic -> 2D covariance */
        const double da = (-c * c * dA + b * c * dB - b * b * dC) / det2;
        const double db = (2.0 * b * c * dA - (a * c + b * b) * dB + 2.0 * a * b * dC) / det2;
        const double dc = (-b * b * dA + a * b * dB - a * a * dC) / det2;
        /* cov2d = (T0 S T0, T0 S T1, T1 S T1): gradient for Sigma (symmetric) and for T0, T1 */
        double GS[3][3];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j)
                GS[i][j] = da * P.T0[i] * P.T0[j] + 0.5 * db * (P.T0[i] * P.T1[j] + P.T1[i] * P.T0[j]) +
                           dc * P.T1[i] * P.T1[j];
        double ST0[3], ST1[3], dT0[3], dT1[3];
        for (int i = 0; i < 3; ++i) {
            ST0[i] = P.S[i][0] * P.T0[0] + P.S[i][1] * P.T0[1] + P.S[i][2] * P.T0[2];
            ST1[i] = P.S[i][0] * P.T1[0] + P.S[i][1] * P.T1[1] + P.S[i][2] * P.T1[2];
        }
        for (int i = 0; i < 3; ++i) {
            dT0[i] = 2.0 * da * ST0[i] + db * ST1[i];
            dT1[i] = db * ST0[i] + 2.0 * dc * ST1[i];
        }
        /* T0 = j00 W_row0 + j02 W_row2, T1 = j11 W_row1 + j12 W_row2 */
        double dj00 = 0, dj02 = 0, dj11 = 0, dj12 = 0;
        for (int k = 0; k < 3; ++k) {
            dj00 += dT0[k] * W[k];
            dj02 += dT0[k] * W[6 + k];
            dj11 += dT1[k] * W[3 + k];
            dj12 += dT1[k] * W[6 + k];
        }
        const double tx = P.t[0], ty = P.t[1], tz = P.t[2];
        const double tz2 = tz * tz, tz3 = tz2 * tz;
        double dt[3];
        dt[0] = dj02 * (-fx / tz2) + du * fx / tz;
        dt[1] = dj12 * (-fy / tz2) + dv * fy / tz;
        dt[2] = dj00 * (-fx / tz2) + dj02 * (2.0 * fx * tx / tz3) + dj11 * (-fy / tz2) +
                dj12 * (2.0 * fy * ty / tz3) - du * fx * tx / tz2 - dv * fy * ty / tz2;
        double gm[3];
        for (int i = 0; i < 3; ++i) gm[i] = W[i] * dt[0] + W[3 + i] * dt[1] + W[6 + i] * dt[2];
        /* Sigma = M M^T -> dM = 2 GS M */
        double dM[3][3];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j)
                dM[i][j] = 2.0 * (GS[i][0] * P.M[0][j] + GS[i][1] * P.M[1][j] + GS[i][2] * P.M[2][j]);
        /* M = R diag(s) */
        double dR[3][3], ds[3] = {0, 0, 0};
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) {
                dR[i][j] = dM[i][j] * P.s[j];
                ds[j] += dM[i][j] * P.R[i][j];
            }
        for (int j = 0; j < 3; ++j) g_log_scale[j * n + g] = ds[j] * P.s[j];
        /* R(w, x, y, z) of the unit quaternion */
        const double w = P.w, x = P.x, y = P.y, z = P.z;
        double dq[4];
        dq[0] = 2.0 * (-z * dR[0][1] + y * dR[0][2] + z * dR[1][0] - x * dR[1][2] - y * dR[2][0] + x * dR[2][1]);
        dq[1] = 2.0 * (y * dR[0][1] + z * dR[0][2] + y * dR[1][0] - 2.0 * x * dR[1][1] - w * dR[1][2] +
                       z * dR[2][0] + w * dR[2][1] - 2.0 * x * dR[2][2]);
        dq[2] = 2.0 * (-2.0 * y * dR[0][0] + x * dR[0][1] + w * dR[0][2] + x * dR[1][0] + z * dR[1][2] -
                       w * dR[2][0] + z * dR[2][1] - 2.0 * y * dR[2][2]);
        dq[3] = 2.0 * (-2.0 * z * dR[0][0] - w * dR[0][1] + x * dR[0][2] + w * dR[1][0] - 2.0 * z * dR[1][1] +
                       y * dR[1][2] + x * dR[2][0] + y * dR[2][1]);
        /* q_hat = q / |q| */
        const double qh[4] = {w, x, y, z};
        const double dot = qh[0] * dq[0] + qh[1] * dq[1] + qh[2] * dq[2] + qh[3] * dq[3];
        for (int i = 0; i < 4; ++i) g_quat[i * n + g] = (dq[i] - qh[i] * dot) / P.qn;
        /* colour */
        double Y[16], GY[16][3];
        oracle_sh_basis(P.d[0], P.d[1], P.d[2], Y);
        sh_basis_grad(P.d[0], P.d[1], P.d[2], GY);
        double gd[3] = {0, 0, 0};
        for (int k = 0; k < K; ++k) {
            double wk = 0.0;
            for (int ch = 0; ch < 3; ++ch) {
                const double gr = g_rgb ? g_rgb[(int64_t)ch * n + g] : 0.0;
                g_sh[(int64_t)(k * 3 + ch) * n + g] = Y[k] * gr;
                wk += sh[(int64_t)(k * 3 + ch) * n + g] * gr;
            }
            for (int i = 0; i < 3; ++i) gd[i] += GY[k][i] * wk;
        }
        const double dd = gd[0] * P.d[0] + gd[1] * P.d[1] + gd[2] * P.d[2];
        for (int i = 0; i < 3; ++i) gm[i] += (gd[i] - P.d[i] * dd) / P.dn;
        for (int i = 0; i < 3; ++i) g_mean[i * n + g] = gm[i];
    }
}

int32_t oracle_tile_kept(int64_t n, int64_t g, const float *mean2d, const float *ellipse, const int32_t *rect,
                         int32_t tile_test, int32_t tx, int32_t ty);

/* Tile membership of the lists: the rectangle, and with tile_test 1 the exact 3-sigma
 * footprint of gs_oracle.c (binary32 mean2d32 and ellipse from its projection). */
typedef struct {
    const float *mean2d32, *ellipse;
    int32_t tile_test;
} list_rule;

/* The list of pixel (px, py): Gaussians of order[] one of whose tiles is the pixel's. */
static int64_t pixel_list(int64_t n, const int32_t *rect, const list_rule *rule, const int64_t *order, int64_t nv,
                          int32_t px, int32_t py, int64_t *list) {
    const int32_t tx = px / TILE, ty = py / TILE;
    int64_t len = 0;
    for (int64_t k = 0; k < nv; ++k) {
        const int64_t g = order[k];
        if (oracle_tile_kept(n, g, rule->mean2d32, rule->ellipse, rect, rule->tile_test, tx, ty)) list[len++] = g;
    }
    return len;
}

static double pixel_alpha(int64_t n, int64_t g, double px, double py, const double *mean2d, const double *conic,
                          const double *opacity, double *G_out, double *dx_out, double *dy_out) {
    const double dx = px - mean2d[g], dy = py - mean2d[n + g];
    const double q = conic[g] * dx * dx + 2.0 * conic[n + g] * dx * dy + conic[2 * n + g] * dy * dy;
    const double G = exp(-0.5 * q);
    *G_out = G;
    *dx_out = dx;
    *dy_out = dy;
    double alpha = opacity[g] * G;
    return alpha > ALPHA_MAX ? ALPHA_MAX : alpha;
}

/*
 * Front-to-back compositing over fixed lists, binary64.  order[nv]: the
 * Gaussians in compositing order.  Pixel p blends the first n_limit[p]
 * entries of its list when n_limit is given (the count a forward pass found),
 * else stops right after the blend that brings T below t_eps (t_eps <= 0:
 * never).  out_rgb [W*H*3] = C + T bg, out_T [W*H], out_count [W*H] (blended
 * entries); out_T and out_count may be NULL.
 */
void oracle_composite_fixed(int64_t n, const double *mean2d, const double *conic, const double *opacity,
                            const double *rgb, const int32_t *rect, const float *mean2d32, const float *ellipse,
                            int32_t tile_test, const int64_t *order, int64_t nv,
                            int32_t width, int32_t height, const double bg[3], const int64_t *n_limit, double t_eps,
                            double *out_rgb, double *out_T, int64_t *out_count) {
    const list_rule rule = {mean2d32, ellipse, tile_test};
    int64_t *list = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nv > 0 ? nv : 1));
    for (int32_t py = 0; py < height; ++py)
        for (int32_t px = 0; px < width; ++px) {
            const int64_t p = (int64_t)py * width + px;
            int64_t len = pixel_list(n, rect, &rule, order, nv, px, py, list);
            if (n_limit && n_limit[p] < len) len = n_limit[p];
            double T = 1.0, C[3] = {0.0, 0.0, 0.0};
            int64_t cnt = 0;
            for (int64_t i = 0; i < len; ++i) {
                const int64_t g = list[i];
                double G, dx, dy;
                const double alpha = pixel_alpha(n, g, px, py, mean2d, conic, opacity, &G, &dx, &dy);
                for (int ch = 0; ch < 3; ++ch) C[ch] += T * alpha * rgb[(int64_t)ch * n + g];
                T *= 1.0 - alpha;
                ++cnt;
                if (!n_limit && t_eps > 0.0 && T < t_eps) break;
            }
            for (int ch = 0; ch < 3; ++ch) out_rgb[p * 3 + ch] = C[ch] + T * bg[ch];
            if (out_T) out_T[p] = T;
            if (out_count) out_count[p] = cnt;
        }
    free(list);
}

/*
 * Vector-Jacobian product of oracle_composite_fixed for the cotangent
 * g_image [W*H*3] (dL/d out_rgb).  For each pixel the forward list is walked
 * once to record alpha_i and T_i = prod_{j<i} (1 - alpha_i), then backwards:
 *   dL/dc_i     = alpha_i T_i dL/dC
 *   dL/dalpha_i = T_i (c_i - B_i) . dL/dC - T_final (bg . dL/dC) / (1 - alpha_i)
 * with B_i = sum_{j>i} c_j alpha_j prod_{i<k<j} (1 - alpha_k) the colour
 * behind entry i (B_{i-1} = alpha_i c_i + (1 - alpha_i) B_i).  alpha =
 * min(0.99, o G) has no derivative in o and G where the clamp is active;
 * elsewhere dL/do = G dL/dalpha and, with G = exp(-q/2),
 *   dL/du = o G dL/dalpha (A dx + B dy),  dL/dv = o G dL/dalpha (B dx + C dy),
 *   dL/dA = -dx^2/2 o G dL/dalpha,  dL/dB = -dx dy o G dL/dalpha,
 *   dL/dC = -dy^2/2 o G dL/dalpha.
 * Outputs (overwritten): g_mean2d [2][n], g_conic [3][n], g_opacity [n],
 * g_rgb [3][n].  pixels: NULL for every pixel, else n_pix flat indices y*W+x,
 * the only pixels whose cotangent is taken (the others count as zero).
 */
void oracle_composite_backward(int64_t n, const double *mean2d, const double *conic, const double *opacity,
                               const double *rgb, const int32_t *rect, const float *mean2d32, const float *ellipse,
                               int32_t tile_test, const int64_t *order, int64_t nv,
                               int32_t width, int32_t height, const double bg[3], const int64_t *n_limit,
                               double t_eps, const double *g_image, const int64_t *pixels, int64_t n_pix,
                               double *g_mean2d, double *g_conic, double *g_opacity, double *g_rgb) {
    memset(g_mean2d, 0, sizeof(double) * 2 * (size_t)n);
    memset(g_conic, 0, sizeof(double) * 3 * (size_t)n);
    memset(g_opacity, 0, sizeof(double) * (size_t)n);
    memset(g_rgb, 0, sizeof(double) * 3 * (size_t)n);
    const size_t cap = (size_t)(nv > 0 ? nv : 1);
    int64_t *list = (int64_t *)malloc(sizeof(int64_t) * cap);
    double *al = (double *)malloc(sizeof(double) * cap);
    double *Ts = (double *)malloc(sizeof(double) * cap);
    const list_rule rule = {mean2d32, ellipse, tile_test};
    if (!pixels) n_pix = (int64_t)width * height;
    for (int64_t pi = 0; pi < n_pix; ++pi) {
        const int64_t p = pixels ? pixels[pi] : pi;
        const int32_t px = (int32_t)(p % width), py = (int32_t)(p / width);
        int64_t len = pixel_list(n, rect, &rule, order, nv, px, py, list);
        if (n_limit && n_limit[p] < len) len = n_limit[p];
        double T = 1.0;
        int64_t cnt = 0;
        for (int64_t i = 0; i < len; ++i) {
            double G, dx, dy;
            al[i] = pixel_alpha(n, list[i], px, py, mean2d, conic, opacity, &G, &dx, &dy);
            Ts[i] = T;
            T *= 1.0 - al[i];
            ++cnt;
            if (!n_limit && t_eps > 0.0 && T < t_eps) break;
        }
        const double *gC = g_image + p * 3;
        const double bg_term = T * (bg[0] * gC[0] + bg[1] * gC[1] + bg[2] * gC[2]);
        double Bk[3] = {0.0, 0.0, 0.0};
        for (int64_t i = cnt - 1; i >= 0; --i) {
            const int64_t g = list[i];
            double G, dx, dy;
            const double alpha = pixel_alpha(n, g, px, py, mean2d, conic, opacity, &G, &dx, &dy);
            double d_alpha = -bg_term / (1.0 - alpha);
            for (int ch = 0; ch < 3; ++ch) {
                const double c = rgb[(int64_t)ch * n + g];
                g_rgb[(int64_t)ch * n + g] += alpha * Ts[i] * gC[ch];
                d_alpha += Ts[i] * (c - Bk[ch]) * gC[ch];
                Bk[ch] = alpha * c + (1.0 - alpha) * Bk[ch];
            }
            if (opacity[g] * G < ALPHA_MAX) {
                g_opacity[g] += G * d_alpha;
                const double dq = opacity[g] * G * d_alpha;   /* dL/d(-q/2) */
                const double A = conic[g], B = conic[n + g], Cc = conic[2 * n + g];
                g_mean2d[g] += dq * (A * dx + B * dy);
                g_mean2d[n + g] += dq * (B * dx + Cc * dy);
                g_conic[g] += -0.5 * dx * dx * dq;
                g_conic[n + g] += -dx * dy * dq;
                g_conic[2 * n + g] += -0.5 * dy * dy * dq;
            }
        }
    }
    free(list);
    free(al);
    free(Ts);
}
