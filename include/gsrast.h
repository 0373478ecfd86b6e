/*
 * gsrast — tile-based differentiable 3D Gaussian-splatting rasterizer for AMD
 * Instinct MI355X (gfx950), C ABI.
 *
 * The method: the lesson "3D Gaussian Splatting from scratch"
 * (aiengineeringfromscratch.com).  A Gaussian carries a world position, a
 * unit quaternion, per-axis log-scales, an opacity in [0,1] and
 * spherical-harmonic colour coefficients (section "Ce qu'un Gaussien porte").
 * Rendering projects each Gaussian with the camera extrinsics and intrinsics,
 * assigns it to 16x16 screen tiles, depth-sorts per tile and alpha-composites
 * front to back (flowchart under "Rastérisation, non rayée"; sections
 * "L'étape de projection" and "La règle de composition alpha").
 *
 * Conventions shared by every entry point
 *  - All array pointers inside gs_gaussians, and the output image, are DEVICE
 *    pointers on the context's device.  The caller owns them; the library never
 *    frees or retains them past the call.
 *  - Every call returns a gs_status and never aborts or throws across the ABI.
 *    Arguments are validated on the host before any HIP call, so
 *    GS_ERR_INVALID_ARGUMENT leaves the device untouched.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    gs_bin_and_sort and gs_render wait, once per call, for the number of
 *    (Gaussian, tile) pairs: the prefix-sum kernel stores it into host memory
 *    and the call waits for that kernel (not for the whole stream).  The pair
 *    kernels are enqueued before that wait on buffers sized from earlier calls,
 *    so the GPU does not idle; when the count exceeds that capacity the buffers
 *    grow and the pair kernels run again before the call returns.  All other
 *    calls are asynchronous.
 *  - One context per host thread / stream at a time; a context is not
 *    thread-safe.  Views returned in gs_projected / gs_binning point into
 *    context-owned device memory and stay valid until the next call on the
 *    same context or gs_context_destroy.
 */
#ifndef GSRAST_H
#define GSRAST_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, degree or camera; nothing was enqueued */
    GS_ERR_OUT_OF_MEMORY = 2,    /* device workspace could not grow (or would pass GS_OPT_MAX_WORKSPACE_BYTES) */
    GS_ERR_CAPACITY = 3,         /* pair count above 2^32-1 or above GS_OPT_MAX_DUPS */
    GS_ERR_DEVICE = 4            /* a HIP call failed; gs_last_error() has the HIP message */
} gs_status;

/* Tile edge in pixels (flowchart: "Assign to tiles (16x16 screen-space)"). */
#define GS_TILE 16
/* Largest alpha a single Gaussian may take (section "Étape 2": clamp to 0.99). */
#define GS_ALPHA_MAX 0.99f
/* A pixel stops after the blend that brings its transmittance below this. */
#define GS_T_EPS 1e-4f
/* Floats per projected-splat record (see gs_projected.splat). */
#define GS_SPLAT_STRIDE 16
/* Bytes of the static device array gs_render_noalloc takes its buffers from (per device). */
#define GS_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * Gaussian parameters, structure of arrays, fp32, device memory, index g in
 * [0, n) fastest (section "Ce qu'un Gaussien porte" lists the fields):
 *   mean      [3][n]  world position
 *   quat      [4][n]  rotation quaternion (w, x, y, z); normalised in-kernel
 *   log_scale [3][n]  per-axis log-scales, exponentiated at render time
 *   opacity   [n]     already in [0, 1] (post-sigmoid)
 *   sh        [K*3][n] with K = (sh_degree+1)^2; plane k*3+c is coefficient k of
 *                     colour channel c
 * n may be 0 (the image is then the background).  n < 2^31.
 */
typedef struct {
    int64_t n;
    int32_t sh_degree; /* 0..3 (section "Étape 6": up to 16 terms per channel) */
    int32_t reserved;
    const float *mean;
    const float *quat;
    const float *log_scale;
    const float *opacity;
    const float *sh;
} gs_gaussians;

/*
 * Pinhole camera (host memory, passed by pointer).  R, t map world to camera
 * coordinates, x right, y down, z forward: p_cam = R p_world + t, R row-major.
 * Pixel (row i, column j) is sampled at x = j, y = i (integer positions).
 * Requirements: width, height in [1, 32768]; fx, fy > 0; znear > 0; all
 * finite.  Gaussians with camera-space z <= znear are culled.
 */
typedef struct {
    float R[9];
    float t[3];
    float fx, fy, cx, cy;
    float znear;
    int32_t width, height;
} gs_camera;

/*
 * Output of gs_preprocess (views into context memory, device pointers).
 *   splat [n][GS_SPLAT_STRIDE] fp32 records (64 bytes):
 *          0 u, 1 v            projected mean in pixels
 *          2 opacity
 *          3, 4, 5             -log2(e)/2 * (A, 2B, C): alpha = opacity * 2^(f3 dx^2 + f4 dx dy + f5 dy^2)
 *          6 r, 7 g, 8 b       SH colour in the view direction
 *          9 radius            ceil(3 sqrt(largest eigenvalue of the 2D covariance))
 *          10 A, 11 B, 12 C    conic = inverse 2D covariance: q = A dx^2 + 2 B dx dy + C dy^2
 *          13 depth            camera-space z (same as depth[g])
 *          14, 15              unused
 *   depth      [n] camera-space z
 *   rect       [n][4] uint16: x0, x1, y0, y1 tile rectangle, half-open
 *   tile_count [n] (x1-x0)*(y1-y0) for a visible Gaussian, else 0
 * Fields other than tile_count and rect are unspecified when tile_count is 0.
 */
typedef struct {
    int64_t n;
    int32_t tiles_x, tiles_y;
    const float *splat;
    const float *depth;
    const uint16_t *rect;
    const uint32_t *tile_count;
} gs_projected;

/*
 * Output of gs_bin_and_sort (views into context memory, device pointers).
 * One entry per (visible Gaussian, tile of its rectangle); num_dups entries.
 *   keys        [num_dups] (tile_id << 32) | bit pattern of the fp32 depth,
 *               tile_id = ty * tiles_x + tx; ascending, equal keys ordered by
 *               ascending Gaussian index.  NULL in GS_SORT_DEPTH_FIRST mode when
 *               GS_OPT_EMIT_KEYS is 0.
 *   values      [num_dups] Gaussian index of each sorted entry
 *   tile_ranges [tiles_x*tiles_y][2] half-open [start, end) into keys/values;
 *               (0, 0) for a tile no Gaussian touches
 *   keys_unsorted / values_unsorted: the pairs before sorting, listed by
 *               Gaussian index then row-major over the rectangle; only filled in
 *               GS_SORT_KEY64 mode with GS_OPT_EMIT_KEYS set, else NULL.
 *   super_entries  entries of the super-tile list (one per visible Gaussian and 8 x 8-tile
 *               super-tile its rectangle meets) when the lists were built by super-tile
 *               binning, else 0 (informational: the traffic of the binning stage)
 *   depth_buckets  number of depth buckets when GS_DEPTH_ORDER_BUCKETS ordered the
 *               Gaussians of this frame, 0 when the radix sort did (GS_DEPTH_ORDER_RADIX,
 *               a fallback from too large a bucket or one whose kernel the frame left out,
 *               GS_SORT_KEY64, or fewer than 2 Gaussians)
 */
typedef struct {
    int64_t num_dups;
    int32_t tiles_x, tiles_y;
    const uint64_t *keys;
    const uint32_t *values;
    const uint32_t *tile_ranges;
    const uint64_t *keys_unsorted;
    const uint32_t *values_unsorted;
    int64_t super_entries;
    int64_t depth_buckets;
} gs_binning;

/* Sorting strategies; both give identical keys, values and ranges. */
typedef enum {
    /* depth-sort the Gaussians once (32-bit keys), then build the per-tile lists in that
       order (GS_OPT_BINNING says how; the default) */
    GS_SORT_DEPTH_FIRST = 0,
    /* duplicate 64-bit (tile << 32 | depth) keys in Gaussian order, then a
       stable LSD radix sort over the significant key bits */
    GS_SORT_KEY64 = 1
} gs_sort_mode;

/* Which tiles a Gaussian is listed in. */
typedef enum {
    /* every tile of the square [u-r, u+r] x [v-r, v+r], r the 3-sigma radius along the major
       axis (flowchart "Assign to tiles (16x16 screen-space)"; the default) */
    GS_TILE_SQUARE = 0,
    /* those tiles of the square whose pixel-centre box [16tx, 16tx+15] x [16ty, 16ty+15]
       meets the 3-sigma ellipse d^T cov2d^-1 d <= 9 (fewer pairs; drops contributions
       below o exp(-9/2) per pixel).  Per tile row the kept tiles are one span: the
       ellipse cut at height dy is centred at (b/c) dy with half-width
       sqrt((det/c)(9 - dy^2/c)); its ends peak at dy = +-3b/sqrt(a) clamped to the
       row's band.  Evaluated in binary32 in a fixed order, so counts and keys are exact.
       The pair listing checks on the device that each Gaussian's spans add up to its tile
       count and stays inside its rectangle either way; a mismatch (never seen) raises a
       flag that the next gs_bin_and_sort / gs_render on the context returns as
       GS_ERR_DEVICE. */
    GS_TILE_ELLIPSE = 1
} gs_tile_test;

/* How GS_SORT_DEPTH_FIRST turns the depth-ordered Gaussians into per-tile lists; all give
   identical values and ranges (and keys, when emitted). */
typedef enum {
    /* GS_BINNING_SUPER_TILE for scenes of at least 65536 Gaussians, else GS_BINNING_RADIX
       (below that the super-tile path's extra kernels cost more than they save; the default) */
    GS_BINNING_AUTO = 0,
    /* group the tiles 8 x 8 into super-tiles, sort the Gaussians stably by super-tile (one
       8-bit radix pass over about two entries per Gaussian), then expand each super-tile's
       list into its 64 tiles, ranking a Gaussian within a tile by ballots in list order
       (used when the image has at most 256 super-tiles and 65536 tiles, and more than one
       Gaussian, else GS_BINNING_RADIX) */
    GS_BINNING_SUPER_TILE = 1,
    /* list every (Gaussian, tile) pair, then a stable radix sort on the tile id */
    GS_BINNING_RADIX = 2
} gs_binning_mode;

/* How GS_SORT_DEPTH_FIRST orders the Gaussians by (depth, index); both give the same order
   (flowchart step "Depth-sort per tile"). */
typedef enum {
    /* B buckets linear in depth between the smallest and largest depth of the Gaussians with
       tiles (B = 256 .. 8192 with the scene), one distribution pass, then each bucket sorted
       by (depth bits, index) in LDS.  If a bucket holds more than 4096 Gaussians (depths
       crowded into a sliver of the range) the frame falls back to GS_DEPTH_ORDER_RADIX.
       Buckets of 2049 to 4096 Gaussians have a kernel of their own, which a context launches
       only while its last bucketed frame met such a bucket; a frame that meets one without it
       falls back the same way (and the next frame launches it).  Results are the same bits on
       every path.  The default. */
    GS_DEPTH_ORDER_BUCKETS = 0,
    /* stable LSD radix sort of the 32 depth bits, four 8-bit passes */
    GS_DEPTH_ORDER_RADIX = 1
} gs_depth_order;

typedef enum {
    GS_OPT_SORT_MODE = 0,            /* gs_sort_mode, default GS_SORT_DEPTH_FIRST */
    GS_OPT_EMIT_KEYS = 1,            /* 1: gs_bin_and_sort materialises keys (default 1); gs_render never does */
    GS_OPT_MAX_DUPS = 2,             /* cap on pairs per frame, at most and by default 2^32-1 -> GS_ERR_CAPACITY */
    GS_OPT_MAX_WORKSPACE_BYTES = 3,  /* cap on context device memory (default: none) -> GS_ERR_OUT_OF_MEMORY */
    GS_OPT_PROFILE = 4,              /* 1: bracket every kernel with HIP events (see gs_profile_read) */
    GS_OPT_TILE_TEST = 5,            /* gs_tile_test, default GS_TILE_SQUARE; read by gs_preprocess, and the
                                        binning, compositing and backward of that projection follow it */
    GS_OPT_BINNING = 6,              /* gs_binning_mode, default GS_BINNING_AUTO (depth-first mode) */
    GS_OPT_DEPTH_ORDER = 7           /* gs_depth_order, default GS_DEPTH_ORDER_BUCKETS (depth-first mode); read
                                        by gs_preprocess and the binning of that projection */
} gs_option;

/* Per-stage timing collected while GS_OPT_PROFILE is 1. */
typedef enum {
    GS_STAGE_PREPROCESS = 0,
    GS_STAGE_DEPTH_SORT = 1,   /* depth-first mode: the depth order (buckets or radix passes) */
    GS_STAGE_SCAN = 2,         /* prefix sum of tile counts */
    GS_STAGE_DUPLICATE = 3,    /* pair listing, or the super-tile listing */
    GS_STAGE_TILE_SORT = 4,    /* radix passes over the pair list; or super-tile sort, expansion into
                                  tiles, ranges and the heaviest-first tile launch order */
    GS_STAGE_RANGES = 5,       /* radix binning: tile ranges (+ key emission), heaviest-first tile
                                  launch order; not recorded under super-tile binning */
    GS_STAGE_COMPOSITE = 6,
    GS_STAGE_READBACK = 7,     /* not recorded: the pair count reaches the host with no stream operation */
    GS_STAGE_BACKWARD_COMPOSITE = 8,   /* gs_backward: per-tile reverse walk */
    GS_STAGE_BACKWARD_SETUP = 9,       /* gs_backward: tile launch order; pair offsets in Gaussian order (depth-first mode) */
    GS_STAGE_BACKWARD_GAUSSIAN = 10,   /* gs_backward: per-Gaussian sums + projection and colour chain rule */
    GS_STAGE_COUNT = 11
} gs_stage;

typedef struct {
    double ms[GS_STAGE_COUNT];        /* summed kernel time per stage, milliseconds */
    int64_t launches[GS_STAGE_COUNT]; /* kernels (or copies) timed per stage */
} gs_profile;

typedef struct gs_context gs_context;

/* Creates a context on HIP device `device`.  GS_ERR_DEVICE if the device
 * cannot be selected.  *out is set to NULL on failure. */
gs_status gs_context_create(gs_context **out, int device);
/* Frees all context memory.  NULL is accepted. */
void gs_context_destroy(gs_context *ctx);
/* Sets an option (gs_option).  GS_ERR_INVALID_ARGUMENT on an unknown option or value. */
gs_status gs_context_set_option(gs_context *ctx, int option, int64_t value);

/*
 * Host-only argument check used by every entry point (no HIP call).  On error
 * writes a NUL-terminated reason into msg (if msg_len > 0).  `camera` may be
 * NULL when only the Gaussians are checked; `gaussians` may be NULL likewise.
 */
gs_status gs_check_arguments(const gs_gaussians *gaussians, const gs_camera *camera, char *msg,
                             size_t msg_len);

/*
 * Projection + SH colour + tile rectangle per Gaussian (sections "Ce qu'un
 * Gaussien porte", "L'étape de projection", "Étape 5: De la 2D à la 3D",
 * "Étape 6").  Sigma = R S S^T R^T; Sigma' = J W Sigma W^T J^T with J taken
 * at the camera-space mean; radius 3 sigma along the major axis; colour from
 * the SH expansion in the direction camera centre -> mean.
 */
gs_status gs_preprocess(gs_context *ctx, const gs_gaussians *gaussians, const gs_camera *camera,
                        gs_projected *out, hipStream_t stream);

/*
 * Caches the view-independent part of the projection: the 3D covariance
 * Sigma = R S S^T R^T of every Gaussian (section "Ce qu'un Gaussien porte"), six
 * floats per Gaussian in context memory.  While the cache is held, gs_preprocess
 * (and gs_render) on the same context reads it instead of quat and log_scale
 * whenever its gaussians have the same n, quat and log_scale pointers: several
 * views of one scene then compute Sigma once.  The result is bit-identical to the
 * uncached preprocess.  The library cannot see writes to caller memory: after
 * changing quat or log_scale in place, call again (or drop the cache).
 * `gaussians` NULL drops the cache.  gs_render_noalloc never uses it.
 * Asynchronous on `stream`; errors as gs_preprocess (invalid arguments are
 * checked with gs_check_arguments).
 */
gs_status gs_cache_covariance(gs_context *ctx, const gs_gaussians *gaussians, hipStream_t stream);

/*
 * Tile binning of the last gs_preprocess output: prefix sum of tile counts,
 * (tile, depth) pair listing, stable sort, and per-tile ranges (flowchart
 * steps "Assign to tiles" and "Depth-sort per tile").  `projected` must be the
 * view returned by the last gs_preprocess on this context.  Waits once for
 * the pair count (see the conventions above).
 */
gs_status gs_bin_and_sort(gs_context *ctx, const gs_projected *projected, const gs_camera *camera,
                          gs_binning *out, hipStream_t stream);

/*
 * Front-to-back alpha compositing per 16x16 tile (section "La règle de
 * composition alpha"): alpha = min(0.99, o exp(-q/2)), C += T alpha c,
 * T *= (1 - alpha); a pixel stops after the blend that brings T below
 * GS_T_EPS; out = C + T bg.  bg_rgb: 3 host floats.  image_hwc: device
 * [height][width][3] fp32, fully overwritten.
 */
gs_status gs_composite(gs_context *ctx, const gs_projected *projected, const gs_binning *binning,
                       const gs_camera *camera, const float bg_rgb[3], float *image_hwc,
                       hipStream_t stream);

/*
 * As gs_composite, and also writes per-pixel diagnostics when non-NULL:
 * final_T [height][width] final transmittance, n_blend [height][width] number
 * of Gaussians blended into the pixel.  If blend_total is non-NULL (a device
 * uint64), the sum of n_blend over the image is added to it.
 */
gs_status gs_composite_ex(gs_context *ctx, const gs_projected *projected, const gs_binning *binning,
                          const gs_camera *camera, const float bg_rgb[3], float *image_hwc,
                          float *final_T, uint32_t *n_blend, unsigned long long *blend_total,
                          hipStream_t stream);

/* gs_preprocess + gs_bin_and_sort + gs_composite on one stream (keys are not
 * materialised).  Waits once for the pair count (see the conventions above). */
gs_status gs_render(gs_context *ctx, const gs_gaussians *gaussians, const gs_camera *camera,
                    const float bg_rgb[3], float *image_hwc, hipStream_t stream);

/*
 * gs_render for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, stages, kernels
 * and result (bit for bit) as gs_render, but no intermediate buffer comes from the context's
 * workspace: every one is carved from one static device array of GS_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that each device the library runs on holds until the process ends, and the call
 * makes no allocation (no hipMalloc, hipFree or event creation; profiling is off for it).
 * The context must exist (created beforehand: it holds the host-visible pair-count word).
 * Limits: the Gaussians and tiles may take at most half the array (132 bytes per Gaussian,
 * up to 8 MiB of depth-bucket counts, 12 bytes per tile: about 250 k Gaussians at 1080p),
 * the frame as a whole with its pairs
 * (4 to 12 bytes each, counted on the device) the full array; beyond either the call returns
 * GS_ERR_CAPACITY (the pair case after waiting for the count, with nothing composited).
 * Every call on one device shares that device's array and leaves its contents behind:
 * calls that overlap on one device (other streams, threads or contexts) race, and the
 * caller must order them.  Afterwards the context holds no projection or binning (the
 * staged entry points need a new gs_preprocess); its own workspace is untouched.
 */
gs_status gs_render_noalloc(gs_context *ctx, const gs_gaussians *gaussians, const gs_camera *camera,
                            const float bg_rgb[3], float *image_hwc, hipStream_t stream);

/*
 * Gradients of a scalar loss L with respect to the Gaussian parameters, device
 * fp32 planes with the layout of gs_gaussians ([component][n], index g fastest).
 * The five parameter planes are required; the screen-space planes are optional
 * (NULL = not written).  Every plane is overwritten, not accumulated into.
 *   mean [3][n], quat [4][n], log_scale [3][n], opacity [n], sh [K*3][n]
 *   mean2d [2][n]   dL/d(u, v) of the projected mean
 *   conic  [3][n]   dL/d(A, B, C), q = A dx^2 + 2 B dx dy + C dy^2
 *   rgb    [3][n]   dL/d(r, g, b) of the SH colour
 * A Gaussian in no tile list gets zeros.
 */
typedef struct {
    float *mean;
    float *quat;
    float *log_scale;
    float *opacity;
    float *sh;
    float *mean2d;
    float *conic;
    float *rgb;
} gs_gradients;

/*
 * Backward pass of gs_preprocess + gs_bin_and_sort + gs_composite_ex (section
 * "Pourquoi est-ce différenciable": projection, alpha compositing and the SH
 * colour are differentiable in mean, quaternion, log-scales, opacity and SH
 * coefficients).  `gaussians`, `projected` and `binning` must be the inputs
 * and outputs of the last forward on this context; final_T and n_blend are the
 * per-pixel outputs of that forward's gs_composite_ex (device [height][width]);
 * grad_image is dL/d(image), device [height][width][3]; bg_rgb the forward's 3
 * host floats.  Tile rectangles, per-tile order and each pixel's stopping point
 * are held fixed (they are integer decisions).  Gradients are deterministic:
 * per-(Gaussian, tile) partial sums are written to context memory and summed
 * per Gaussian in a fixed order (no floating-point atomics).  Asynchronous.
 */
gs_status gs_backward(gs_context *ctx, const gs_gaussians *gaussians, const gs_camera *camera,
                      const gs_projected *projected, const gs_binning *binning, const float bg_rgb[3],
                      const float *final_T, const uint32_t *n_blend, const float *grad_image,
                      const gs_gradients *grads, hipStream_t stream);

/*
 * The lesson's dense 2D splat rasteriser (sections "Étape 1: Un gaussien 2D",
 * "Étape 2: Rasteriser à éclaboussure en 2D"): every splat at every pixel
 * (x = column, y = row), alpha = clamp(o exp(-d^T cov^-1 d / 2), 0, 0.99),
 * splats in ascending (depth, index) order, front-to-back compositing with no
 * early stop, out = C + T bg (bg_rgb: 3 host floats, NULL = black).  All
 * arrays are device fp32, row-major: means [n][2] (x, y in pixels),
 * covs [n][2][2], colours [n][3], opacities [n], depths [n] (order only),
 * image [height][width][3].  n in [0, 2^31); the ranking is quadratic in n,
 * sized for the lesson's hundreds to thousands of splats.  Context memory:
 * 4 bytes per (splat, pixel) for the transmittance the backward reads.
 */
gs_status gs_splat2d_forward(gs_context *ctx, int64_t n, const float *means, const float *covs,
                             const float *colours, const float *opacities, const float *depths, int32_t height,
                             int32_t width, const float bg_rgb[3], float *image, hipStream_t stream);

/*
 * Gradient of sum(grad_image * image) for the last gs_splat2d_forward on this
 * context, called with the same arguments (section "Étape 4" trains the splats
 * by gradient descent): grad_means [n][2], grad_covs [n][2][2] (full-matrix
 * gradient, as for a general inverse), grad_colours [n][3], grad_opacities [n],
 * all overwritten.  The depth order is held fixed.  Deterministic (fixed
 * summation order, no floating-point atomics).  Asynchronous.
 */
gs_status gs_splat2d_backward(gs_context *ctx, int64_t n, const float *means, const float *covs,
                              const float *colours, const float *opacities, const float *depths, int32_t height,
                              int32_t width, const float bg_rgb[3], const float *grad_image, float *grad_means,
                              float *grad_covs, float *grad_colours, float *grad_opacities, hipStream_t stream);

/*
 * The scale activation of gs_preprocess (lesson, sections "Ce qu'un Gaussien
 * porte" and "Étape 5": S = diag(exp(log_scale))), elementwise:
 * scale[i] = binary32 rounding of the binary64 exp of log_scale[i].  Device
 * arrays of n >= 0 floats (may not overlap).  Tile counts and keys depend on
 * these bits, so the call exists to check the device's exp against a host's
 * for every input of a range.  Asynchronous.
 */
gs_status gs_scale_activation(gs_context *ctx, const float *log_scale, float *scale, int64_t n,
                              hipStream_t stream);

/* Reads (and resets) the accumulated per-stage times; waits for the timed work. */
gs_status gs_profile_read(gs_context *ctx, gs_profile *out);

/* Static description of a status code. */
const char *gs_status_string(gs_status status);
/* Message of the last failure on this context ("" if none).  NULL ctx -> "". */
const char *gs_last_error(const gs_context *ctx);

#ifdef __cplusplus
}
#endif

#endif /* GSRAST_H */
