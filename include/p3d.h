/*
 * p3d.h -- C ABI of libp3d: pixel-aligned projection conditioning on AMD
 * Instinct MI355X (gfx950).
 *
 * For every token (a cell of a dense 3-D grid or a sparse voxel) the library
 * projects the cell centre through a fixed frontal pinhole camera, samples a
 * channels-last image feature map there with grid_sample semantics, emits an
 * in-image mask, and applies the per-token linear layer proj_linear; the
 * classifier-free-guidance null branch is filled on the device.
 *
 * Sources (web pages, cited by title and section):
 *   pixal3d_mrp_mlx, history of tests/, commit landing the pixel-aligned head
 *     -- project_points, bilinear_sample, ProjGrid and distance_from_fov; the
 *     grid_sample conventions (align_corners=False half-texel mapping, border
 *     padding that clamps the source index before the corners are taken) and
 *     a camera that looks down -Z.
 *   trellis.cpp PR #38 "Initial support for Pixal3D":
 *     commit adding pixal3d.cpp -- tokens are grid cells projected by a fixed
 *       frontal camera whose only free parameter is the FOV; closed-form
 *       distance;
 *     commit exposing extend_pixel -- worked example of that distance;
 *     commit introducing FlowCond -- proj_linear maps the per-token
 *       view-aligned feature into model space; the null proj of the CFG
 *       negative branch is zeroed on the device instead of materialised;
 *     commit wiring the stages -- proj_in_channels is read off the weight and
 *       a mismatch fails with a message;
 *     commit checking widths in lin() -- errors name the tensor and both
 *       shapes;
 *     commit adding per-request camera fields -- every image has its own FOV;
 *     commit on the cascade requantization -- the projection grid is the
 *       endpoint-inclusive linspace(-1, 1, grid), and a high-resolution token
 *       maps to the nearest node, round(u * (grid - 1)), where TRELLIS.2
 *       floors u * grid;
 *     commit adding the NAF upsampler -- the shape and texture stages sample
 *       the DINOv3 map and its NAF-upsampled version (another size) at the
 *       same points and concatenate them, hence proj_in_channels = 2048;
 *     commit adding proj mode to the DiT -- every block has its own
 *       proj_linear whose output is added into that block's residual, over a
 *       projection that stays fixed for the stage.
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or retains them past the call.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without synchronising. Results are ready when the
 *     stream reaches that point.
 *   - Every call returns a p3d_status. On any status other than P3D_OK
 *     nothing was enqueued (P3D_ERR_HIP: the launch itself failed), and
 *     p3d_last_error() -- a per-thread string, valid until that thread's next
 *     call -- names the offending argument with the expected and actual
 *     values or shapes.
 *   - Camera arrays are HOST arrays, read during the call only.
 *   - Floating-point decisions that produce integers (pixel indices, masks)
 *     are taken in binary32 with one rounding per operation in the order
 *     documented below (no contraction), so they are reproducible bit for
 *     bit by any IEEE binary32 implementation of the same steps.
 */
#ifndef P3D_H
#define P3D_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum p3d_status {
    P3D_OK = 0,
    P3D_ERR_INVALID_ARG = 1,  /* value outside its documented range */
    P3D_ERR_SHAPE = 2,        /* sizes that must agree do not */
    P3D_ERR_DTYPE = 3,        /* element type (combination) not supported */
    P3D_ERR_UNSUPPORTED = 4,  /* valid, but outside what the kernels handle */
    P3D_ERR_HIP = 5           /* the HIP runtime rejected a launch */
} p3d_status;

typedef enum p3d_dtype {
    P3D_F32 = 0,              /* IEEE binary32 */
    P3D_BF16 = 1              /* bfloat16 (upper half of a binary32) */
} p3d_dtype;

/* A per-image pinhole camera on the +Z axis looking down -Z at the origin.
 * focal = 1 / tan(fov / 2) in normalised image units (full-angle FOV);
 * distance = camera-to-origin distance in world units (the unit cube spans
 * [-1/2, 1/2]^3). Both finite and > 0. A distance of 0.5 or less is
 * accepted and defined: cells at or behind the camera plane (depth <= 0) get
 * mask 0; at depth exactly 0, gx and gy are +-inf (NaN for a cell on the
 * axis), and the sampling index clamp maps them to the edge texel (NaN to
 * texel 0), the same as for any other out-of-range coordinate. */
typedef struct p3d_camera {
    float focal;
    float distance;
} p3d_camera;

/* Largest batch (number of images / cameras) one call accepts. Cameras
 * travel to the device inside the kernel arguments. */
#define P3D_MAX_BATCH 256
/* Most blocks one p3d_proj_linear_grouped call applies. */
#define P3D_MAX_GROUPS 64

/* ------------------------------------------------------------------------
 * Host helpers (no device work, no stream).
 * --------------------------------------------------------------------- */

/* Library version string, e.g. "p3d 1.0.0 gfx950". Static storage. */
const char* p3d_version(void);

/* Name of a status code. Static storage. */
const char* p3d_status_string(p3d_status s);

/* Message of this thread's last failed call ("" if none). */
const char* p3d_last_error(void);

/* p3d_stream_copy -- copy `bytes` from src to dst on the device with
 * 16-byte non-temporal loads and stores: the achievable HBM rate (read plus
 * write) that measurements set beside the datasheet bandwidth. Not a step of
 * the method.
 *   src, dst  DEVICE pointers, 16-byte aligned, not overlapping
 *   bytes     a multiple of 16 (0 enqueues nothing)
 *   stream    hipStream_t, NULL = default stream
 * P3D_ERR_INVALID_ARG for NULL pointers with bytes > 0, P3D_ERR_UNSUPPORTED
 * for misalignment or a size that is not a multiple of 16. */
p3d_status p3d_stream_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Closed-form camera distance (pixal3d.cpp camera solve; extend_pixel worked
 * example: 49.13 deg on a 512 px frame gives 1.094 / 0.875 / 0.729 for
 * extend_px = 0 / 64 / 128). The distance puts the corner of the unit cube's
 * z = 0 square on the frame border, pushed extend_px pixels beyond it:
 *     d = 0.5 / tan(fov/2) * (S/2) / (S/2 + extend_px),   S = image_size.
 * Computed in binary64 with the C library tan. fov_deg must lie in (0, 180),
 * image_size >= 1 and S/2 + extend_px > 0; otherwise returns NaN and sets
 * the last error. */
double p3d_distance_from_fov(double fov_deg, int32_t image_size, int32_t extend_px);

/* Camera for a full-angle FOV (degrees, in (0, 180)) and a distance (> 0,
 * finite): focal = (float)(1 / tan(fov/2)) computed in binary64 and rounded
 * once; distance rounded once to binary32. */
p3d_status p3d_make_camera(double fov_deg, double distance, p3d_camera* out);

/* ------------------------------------------------------------------------
 * p3d_project_points -- project_points / ProjGrid (pixel-aligned head
 * commit; pixal3d.cpp commit).
 *
 * Token n has the integer cell (b, x, y, z): coords[4n .. 4n+3], or, when
 * coords is NULL, the dense enumeration n = ((b*R + x)*R + y)*R + z (then n
 * must equal batch * R^3, or be 0). For each token, in binary32:
 *   p_a   = ((float)c_a + 0.5f) / (float)R - 0.5f      (a = x, y, z)
 *   depth = distance_b - p_z
 *   gx    = (focal_b * p_x) / depth
 *   gy    = -((focal_b * p_y) / depth)                 (image rows go down)
 *   mask  = b in [0, batch) && depth > 0 && -1 <= gx <= 1 && -1 <= gy <= 1
 *   ix    = min(max(((gx + 1) * W - 1) / 2, 0), W - 1)  (NaN -> 0)
 *   x0    = floor(ix), tx = ix - x0; likewise iy, y0, ty with H.
 * A batch column outside [0, batch) is clamped into range to pick the camera
 * and gets mask 0. Cells outside [0, R) are projected by the same formulas.
 *
 *   coords  [n, 4] int32 device, or NULL (dense grid)
 *   n       tokens (>= 0; 0 enqueues nothing)
 *   resolution  R >= 1
 *   cams    host array [batch]; 1 <= batch <= P3D_MAX_BATCH
 *   height, width  H, W >= 1 of the feature map the pixels index
 *   outputs (device, any may be NULL = not written):
 *     grid  [n, 2] float (gx, gy)     pixel [n, 2] int32 (x0, y0)
 *     frac  [n, 2] float (tx, ty)     depth [n] float    mask [n] uint8 0/1
 * --------------------------------------------------------------------- */
p3d_status p3d_project_points(const int32_t* coords, int64_t n, int32_t resolution,
                              const p3d_camera* cams, int32_t batch,
                              int32_t height, int32_t width,
                              float* grid, int32_t* pixel, float* frac,
                              float* depth, uint8_t* mask, void* stream);

/* ------------------------------------------------------------------------
 * p3d_bilinear_sample -- bilinear_sample == grid_sample(mode='bilinear',
 * align_corners=False, padding_mode='border') (pixel-aligned head commit).
 *
 * feat is channels-last [batch, H, W, C] (row (b, y, x) holds C contiguous
 * channels). For point n with normalised (gx, gy) = grid[2n], grid[2n+1] and
 * item b = batch_index[n] (0 when batch_index is NULL; clamped into range):
 * the source indices, corners and fractions follow p3d_project_points, the
 * far corners are x1 = min(x0 + 1, W - 1), y1 = min(y0 + 1, H - 1), and
 *   out[n, c] = (1-tx)(1-ty) F[y0,x0,c] + tx(1-ty) F[y0,x1,c]
 *             + (1-tx)ty F[y1,x0,c] + tx ty F[y1,x1,c]
 * with binary32 weights and binary32 arithmetic. Points outside the image
 * keep their border-clamped value (only the mask of p3d_project_points
 * flags them).
 *
 *   feat, feat_dtype   device map; F32 or BF16
 *   batch, height, width, channels   map shape; C % 8 == 0 (BF16) or
 *                      C % 4 == 0 (F32); batch*H*W < 2^31
 *   grid [n, 2] float, batch_index [n] int32 or NULL   (device)
 *   out [n, C] device, out_dtype: F32 (any map) or BF16 (BF16 map only;
 *                      round to nearest even)
 *   Alignment: feat and out 16-byte aligned.
 * --------------------------------------------------------------------- */
p3d_status p3d_bilinear_sample(const void* feat, p3d_dtype feat_dtype,
                               int32_t batch, int32_t height, int32_t width,
                               int32_t channels,
                               const float* grid, const int32_t* batch_index, int64_t n,
                               void* out, p3d_dtype out_dtype, void* stream);

/* p3d_bilinear_sample_ordered -- p3d_bilinear_sample processing the points in
 * the order `order` (DEVICE int32 [n], 4-byte aligned: p3d_token_order's
 * output when the points are projected tokens, or any permutation of
 * [0, n); NULL = the natural order). Row p of out still belongs to point p,
 * so the call writes the same bytes as p3d_bilinear_sample; points that
 * share corner rows are sampled together. An entry outside [0, n) breaks the
 * contract: it is clamped into [0, n), so nothing outside the arrays is
 * touched, and which rows are written is unspecified. */
p3d_status p3d_bilinear_sample_ordered(const void* feat, p3d_dtype feat_dtype,
                                       int32_t batch, int32_t height, int32_t width,
                                       int32_t channels, const float* grid,
                                       const int32_t* batch_index, int64_t n,
                                       const int32_t* order, void* out, p3d_dtype out_dtype,
                                       void* stream);

/* ------------------------------------------------------------------------
 * p3d_proj_cond -- the whole path, fused (pixal3d.cpp commit: grid
 * projection and ProjCond; FlowCond commit: proj_linear and the null proj
 * zeroed on the device).
 *
 * out has n + n_null rows of out_dim values, in `dtype`:
 *   rows [0, n):            Y[n,:] = W * S[n,:] + bias, where S is the
 *                           p3d_bilinear_sample of the p3d_project_points
 *                           point of token n; for BF16 the sample is rounded
 *                           to bf16 (nearest even) before the product, which
 *                           accumulates in binary32 (matrix cores).
 *   rows [n, n + n_null):   the CFG null branch: the proj input is zero, so
 *                           the row is proj_linear(0) = bias (+0 with no
 *                           bias). Neither the map nor the weight is read.
 * Sampled features exist only on chip; they are never written to memory.
 *
 *   coords, n, resolution, cams, batch   as p3d_project_points
 *   feat, dtype, height, width, channels  map as p3d_bilinear_sample; map,
 *                           weight, bias and out all have `dtype`
 *   weight [out_dim, weight_in] row-major (a torch Linear weight), device;
 *                           weight_in must equal channels (the weight's input
 *                           width is checked against the map's channels; a
 *                           mismatch is P3D_ERR_SHAPE naming both shapes)
 *   bias [out_dim] device, or NULL
 *   out_dim                 1 <= D <= 2^20; D % 8 == 0 (BF16) or D % 4 == 0 (F32);
 *                           the tile count ceil(n / 128) * ceil(D / 512) (BF16) or
 *                           ceil(n / 128) * ceil(D / 128) (F32) must stay below
 *                           2^31 (P3D_ERR_UNSUPPORTED)
 *   n_null                  >= 0 null rows appended after the n token rows
 *   out [(n + n_null), D] device; mask [n] uint8 device or NULL
 *   Alignment: feat, weight, bias and out 16-byte aligned.
 * --------------------------------------------------------------------- */
p3d_status p3d_proj_cond(const int32_t* coords, int64_t n, int32_t resolution,
                         const p3d_camera* cams, int32_t batch,
                         const void* feat, p3d_dtype dtype,
                         int32_t height, int32_t width, int32_t channels,
                         const void* weight, int32_t out_dim, int32_t weight_in,
                         const void* bias, int64_t n_null,
                         void* out, uint8_t* mask, void* stream);

/* ------------------------------------------------------------------------
 * Point modes and cascade requantization (PR #38, cascade requantization
 * commit; pixel-aligned head commit: ProjGrid).
 *
 * P3D_POINTS_CELL_CENTRES: integer position c on a grid of R is the cell
 *   centre (c + 1/2)/R - 1/2 (binary32, in that order); the default of
 *   p3d_project_points and p3d_proj_cond.
 * P3D_POINTS_GRID_NODES: c is node c of the endpoint-inclusive projection
 *   grid linspace(-1, 1, R) at half scale: c/(R - 1) - 1/2 (binary32, in
 *   that order); R >= 2. The end nodes lie on the faces of the unit cube.
 * --------------------------------------------------------------------- */
typedef enum p3d_points {
    P3D_POINTS_CELL_CENTRES = 0,
    P3D_POINTS_GRID_NODES = 1
} p3d_points;

typedef enum p3d_requant {
    P3D_REQUANT_ROUND_NODES = 0,  /* Pixal3D: nearest node, round(u (G - 1)) */
    P3D_REQUANT_FLOOR_CELLS = 1   /* TRELLIS.2: cell floor(u G) */
} p3d_requant;

/* p3d_requantize_coords -- map sparse coords of a source grid of
 * src_resolution cells onto a grid of `grid` positions (the cascade step
 * from the upsampled res-512 coords to the high-resolution token grid).
 *
 * For each token (b, x, y, z) and each axis, u = (c + 1/2)/src_resolution
 * (the source cell centre in [0, 1]); the output position is
 *   P3D_REQUANT_ROUND_NODES: round(u (grid - 1)), nearest integer, ties to
 *     even -- the node whose projection-grid point is nearest, which keeps
 *     the pixel-aligned sample registered (use P3D_POINTS_GRID_NODES next);
 *   P3D_REQUANT_FLOOR_CELLS: floor(u grid) -- the cell containing u.
 * Both are evaluated exactly in integer arithmetic (no rounding error).
 * Coordinates outside [0, src_resolution) are clamped into it first; the
 * batch column is copied unchanged.
 *
 *   src [n,4] int32 device, 16-byte aligned; dst [n,4] int32 device,
 *   16-byte aligned (may equal src); 1 <= src_resolution, 1 <= grid, both
 *   <= 2^20; grid >= 2 for P3D_REQUANT_ROUND_NODES.
 * --------------------------------------------------------------------- */
p3d_status p3d_requantize_coords(const int32_t* src, int64_t n, int32_t src_resolution,
                                 int32_t grid, p3d_requant mode, int32_t* dst, void* stream);

/* p3d_project_points_ex -- p3d_project_points with a point mode. */
p3d_status p3d_project_points_ex(const int32_t* coords, int64_t n, int32_t resolution,
                                 p3d_points points, const p3d_camera* cams, int32_t batch,
                                 int32_t height, int32_t width,
                                 float* grid, int32_t* pixel, float* frac,
                                 float* depth, uint8_t* mask, void* stream);

/* One channels-last feature map [batch, height, width, channels] on the
 * device (the batch count is the call's). */
typedef struct p3d_map {
    const void* feat;
    int32_t height;
    int32_t width;
    int32_t channels;
} p3d_map;

/* p3d_proj_cond_ex -- p3d_proj_cond with a point mode and one or two maps.
 *
 * With two maps (the NAF commit's 2048 proj channels: the DINOv3 map and its
 * upsampled version) every token is projected once; the normalised point is
 * sampled on each map at that map's own height and width, and the sample is
 * map 0's channels followed by map 1's:
 *   S[n] = [ sample(maps[0], g_n) , sample(maps[1], g_n) ]     (C0 + C1)
 *   Y[n] = W S[n] + bias,   W [out_dim, C0 + C1].
 * Everything else is as p3d_proj_cond (null rows, mask, rounding).
 *
 *   maps    host array [n_maps] of p3d_map, 1 <= n_maps <= 2; every map has
 *           `dtype`, the call's batch count, batch*height*width < 2^31 and
 *           channels % 8 == 0 (BF16) or % 4 == 0 (F32); with two maps,
 *           maps[0].channels % 64 == 0
 *   weight_in must equal the summed channels (P3D_ERR_SHAPE otherwise)
 * --------------------------------------------------------------------- */
p3d_status p3d_proj_cond_ex(const int32_t* coords, int64_t n, int32_t resolution,
                            p3d_points points, const p3d_camera* cams, int32_t batch,
                            p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                            const void* weight, int32_t out_dim, int32_t weight_in,
                            const void* bias, int64_t n_null,
                            void* out, uint8_t* mask, void* stream);

/* ------------------------------------------------------------------------
 * p3d_proj_cond_ws -- p3d_proj_cond_ex with the tokens taken in image-space
 * order, through a caller-owned workspace. Same arguments, results and
 * errors as p3d_proj_cond_ex, plus:
 *
 *   workspace        DEVICE buffer of at least workspace_bytes, 256-byte
 *                    aligned, owned by the caller; its contents on entry do
 *                    not matter and on return are undefined. Calls that
 *                    share one workspace must not overlap (they would race
 *                    on it); the library keeps no pointer to it.
 *   workspace_bytes  >= p3d_proj_cond_workspace_size(n, batch, maps, n_maps),
 *                    else P3D_ERR_INVALID_ARG with both sizes.
 *
 * For BF16 and n > 0 the call first sorts the tokens by the texel block
 * their top-left bilinear corner falls in (batch item, then the Morton index
 * of 4 x 4-texel blocks on the map with the most texels) with a counting
 * sort in the workspace, then runs p3d_proj_cond_ex's fused kernel over the
 * tokens in that order, writing each token's row and mask byte at the
 * token's own index. Tokens that share corner rows are then processed
 * together, so the rows are fetched fewer times. Each output row depends on
 * its own token only, and the arithmetic per row is unchanged, so `out` and
 * `mask` are identical bit for bit to p3d_proj_cond_ex's (pixel-aligned
 * head commit of pixal3d_mrp_mlx; FlowCond commit of trellis.cpp PR #38).
 * F32 calls and null-only calls run p3d_proj_cond_ex unchanged and do not
 * touch the workspace. The sort costs 20-30 us on 100k tokens; a launch
 * whose tiles (128 tokens x 512 features) fit one round on the device gains
 * less than that (7000 tokens on 256 compute units: 5 us), and is better
 * served by p3d_proj_cond_ex.
 * --------------------------------------------------------------------- */
size_t p3d_proj_cond_workspace_size(int64_t n, int32_t batch, const p3d_map* maps,
                                    int32_t n_maps);
                                    /* 0 on invalid sizes (p3d_last_error says why) */
p3d_status p3d_proj_cond_ws(const int32_t* coords, int64_t n, int32_t resolution,
                            p3d_points points, const p3d_camera* cams, int32_t batch,
                            p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                            const void* weight, int32_t out_dim, int32_t weight_in,
                            const void* bias, int64_t n_null,
                            void* out, uint8_t* mask,
                            void* workspace, size_t workspace_bytes, void* stream);

/* p3d_proj_cond_noalloc -- p3d_proj_cond_ws without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The scratch lives in
 * a static device array of the library, P3D_NOALLOC_MAX_TOKENS tokens' worth
 * (8.25 MB per GPU, held until the process ends); the call allocates
 * nothing itself. Same arguments, results and errors as p3d_proj_cond_ex,
 * plus P3D_ERR_UNSUPPORTED when n > P3D_NOALLOC_MAX_TOKENS (nothing is
 * enqueued). The array is shared by every call on a GPU and keeps the last
 * call's contents: calls that overlap on one GPU (several streams or host
 * threads) race on it and must be serialised by the caller. */
#define P3D_NOALLOC_MAX_TOKENS 1048576
p3d_status p3d_proj_cond_noalloc(const int32_t* coords, int64_t n, int32_t resolution,
                                 p3d_points points, const p3d_camera* cams, int32_t batch,
                                 p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                 const void* weight, int32_t out_dim, int32_t weight_in,
                                 const void* bias, int64_t n_null,
                                 void* out, uint8_t* mask, void* stream);

/* ------------------------------------------------------------------------
 * p3d_projection_stats -- projection diagnostics (PR #38, commits adding the
 * per-stage projection statistics and the cross-resolution agreement). The
 * conditioning has no run-time failure mode: a wrong camera, grid or map
 * layout still yields finite features. These figures expose it:
 *   coverage             tokens inside the frame / tokens (a ratio: the
 *                        cube's near corners leave the frame legitimately);
 *   per-half mean, std   of the samples of each map (as fed to proj_linear:
 *                        bf16-rounded for BF16 maps) over all tokens and
 *                        that map's channels -- halves that describe the
 *                        same points must share a scale;
 *   cosine               per token, cos(S0, S1) between the two maps'
 *                        samples (equal channel counts), averaged over the
 *                        tokens where both are non-zero -- the halves, or a
 *                        512 and a 1024 map of one image, must correlate.
 * The same projection and sampling as p3d_proj_cond_ex; nothing is written
 * but the sums below, from which the figures follow:
 *   coverage = inside / tokens
 *   mean_h   = sum[h] / (tokens * C_h)
 *   std_h    = sqrt(sum_sq[h] / (tokens * C_h) - mean_h^2)
 *   cosine   = cos_sum / cos_count
 * Sums are carried in binary64 and accumulated with device atomics (their
 * order, and so the last bits, varies between runs). For BF16 maps each
 * token's partial sums over a lane's share of its channels (C / 16 products
 * of bf16 samples per map) are binary32 first; FP32 maps are binary64
 * throughout. The non-zero test of the cosine is exact. With one map, or two
 * of unequal channels, cos_sum = cos_count = 0.
 *
 *   coords .. batch      as p3d_project_points_ex
 *   dtype, maps, n_maps  as p3d_proj_cond_ex (any channel split)
 *   stats                DEVICE pointer to one p3d_proj_stats, 8-byte
 *                        aligned; overwritten (zeroed on the stream first)
 * --------------------------------------------------------------------- */
typedef struct p3d_proj_stats {
    double tokens;
    double inside;
    double sum[2];
    double sum_sq[2];
    double cos_sum;
    double cos_count;
} p3d_proj_stats;

p3d_status p3d_projection_stats(const int32_t* coords, int64_t n, int32_t resolution,
                                p3d_points points, const p3d_camera* cams, int32_t batch,
                                p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                p3d_proj_stats* stats, void* stream);

/* ------------------------------------------------------------------------
 * p3d_token_order -- an image-space order of the tokens, to be passed to the
 * *_ordered calls (and computed inside p3d_proj_cond_ws). The sampling calls
 * take tokens in runs (tiles, windows); tokens whose bilinear corners share
 * map rows should share a run, so each row is fetched once instead of once
 * per token (pixel-aligned head commit of pixal3d_mrp_mlx: every token reads
 * the four texels around its projection).
 *
 * order[i] receives the token at sorted position i, a permutation of
 * [0, n): tokens sorted by batch item, then by the Morton index of the 4 x
 * 4-texel block (coarser for large maps or batches, so that there are at
 * most 16384 blocks) that contains their top-left corner texel on a
 * key_height x key_width map -- the largest map the tokens will sample. The
 * projection is p3d_project_points_ex's. The order among tokens of one block
 * is unspecified and may change from call to call; results of the *_ordered
 * calls do not depend on it beyond the order of their floating-point sums.
 *
 *   coords .. batch        as p3d_project_points_ex
 *   key_height, key_width  the key map's size, >= 1
 *   order                  DEVICE int32 [n], 4-byte aligned, written
 *   workspace              DEVICE scratch of at least
 *                          p3d_token_order_workspace_size(n, batch,
 *                          key_height, key_width) bytes, 256-byte aligned,
 *                          caller-owned, contents undefined on return;
 *                          calls sharing one workspace must not overlap
 * --------------------------------------------------------------------- */
size_t p3d_token_order_workspace_size(int64_t n, int32_t batch, int32_t key_height,
                                      int32_t key_width);
                                      /* 0 on invalid sizes (p3d_last_error says why) */
p3d_status p3d_token_order(const int32_t* coords, int64_t n, int32_t resolution,
                           p3d_points points, const p3d_camera* cams, int32_t batch,
                           int32_t key_height, int32_t key_width, int32_t* order,
                           void* workspace, size_t workspace_bytes, void* stream);

/* p3d_projection_stats_ordered -- p3d_projection_stats processing the tokens
 * in the order `order` (DEVICE int32 [n] from p3d_token_order, or any
 * permutation of [0, n); NULL = the natural order); the sums change only in
 * the order of their additions. An entry outside [0, n) breaks the
 * contract: it is clamped into [0, n), so nothing outside the arrays is
 * touched, and the sums are unspecified. */
p3d_status p3d_projection_stats_ordered(const int32_t* coords, int64_t n, int32_t resolution,
                                        p3d_points points, const p3d_camera* cams, int32_t batch,
                                        p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                        const int32_t* order, p3d_proj_stats* stats,
                                        void* stream);

/* p3d_stats_figures -- the figures the commit adding the per-stage projection
 * statistics prints, from the sums of p3d_projection_stats (a HOST copy of
 * the p3d_proj_stats, read after the stream has finished it):
 *   coverage = inside / tokens
 *   mean[h]  = sum[h] / (tokens * channels[h])
 *   std[h]   = sqrt(max(sum_sq[h] / (tokens * channels[h]) - mean[h]^2, 0)),
 *              the population standard deviation of map h's samples
 *   cosine   = cos_sum / cos_count
 * A figure whose denominator is 0 (no tokens, h >= n_maps, no token with
 * both samples non-zero) is NaN. Host-only, binary64.
 *   channels  host array [n_maps] of each map's channel count, >= 1 */
typedef struct p3d_stats_fig {
    double coverage;
    double mean[2];
    double std[2];
    double cosine;
} p3d_stats_fig;

p3d_status p3d_stats_figures(const p3d_proj_stats* stats, const int32_t* channels,
                             int32_t n_maps, p3d_stats_fig* out);

/* ------------------------------------------------------------------------
 * Gather once per stage, apply every block's proj_linear every step (PR #38,
 * proj-mode commit): the samples do not change within a stage, so they are
 * gathered once (p3d_proj_sample) and each denoising step runs all blocks'
 * linears over them in one launch (p3d_proj_linear_grouped).
 *
 * p3d_proj_sample -- the gather half of p3d_proj_cond_ex: project every token
 * and write its samples S[n, C0 + C1] (map 0's channels, then map 1's) in
 * `dtype`; BF16 samples are rounded to nearest even exactly as the fused path
 * rounds them before proj_linear. mask [n] uint8 or NULL.
 *   coords .. maps, n_maps   as p3d_proj_cond_ex (two maps: maps[0].channels
 *                            need only be a multiple of 8 (BF16) / 4 (F32))
 *   S        [n, C0 + C1] device, 16-byte aligned
 * --------------------------------------------------------------------- */
p3d_status p3d_proj_sample(const int32_t* coords, int64_t n, int32_t resolution,
                           p3d_points points, const p3d_camera* cams, int32_t batch,
                           p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                           void* S, uint8_t* mask, void* stream);

/* p3d_proj_sample_ordered -- p3d_proj_sample processing the tokens in the
 * order `order` (as p3d_projection_stats_ordered); row t of S and mask byte
 * t still belong to token t, so the call writes the same bytes as
 * p3d_proj_sample. */
p3d_status p3d_proj_sample_ordered(const int32_t* coords, int64_t n, int32_t resolution,
                                   p3d_points points, const p3d_camera* cams, int32_t batch,
                                   p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                   const int32_t* order, void* S, uint8_t* mask, void* stream);

/* p3d_proj_cond_ordered -- p3d_proj_cond_ex over the tokens in the order
 * `order` (DEVICE int32 [n], 4-byte aligned: p3d_token_order's output for
 * the map with the most texels, or any permutation of [0, n); required when
 * n > 0). Row t of `out` and mask byte t still belong to token t, so `out`
 * and `mask` are identical bit for bit to p3d_proj_cond_ex's. It is
 * p3d_proj_cond_ws split in two, for callers that compute one order per
 * stage and share it with p3d_projection_stats_ordered and
 * p3d_proj_sample_ordered. F32 calls ignore the order. An entry outside
 * [0, n) breaks the contract: it is clamped into [0, n), so nothing outside
 * the arrays is touched, and which rows are written is unspecified. */
p3d_status p3d_proj_cond_ordered(const int32_t* coords, int64_t n, int32_t resolution,
                                 p3d_points points, const p3d_camera* cams, int32_t batch,
                                 p3d_dtype dtype, const p3d_map* maps, int32_t n_maps,
                                 const void* weight, int32_t out_dim, int32_t weight_in,
                                 const void* bias, int64_t n_null, void* out, uint8_t* mask,
                                 const int32_t* order, void* stream);

/* p3d_proj_cond_plan -- how a BF16 fused call (p3d_proj_cond, _ex, _ws,
 * _noalloc, _ordered) of n tokens and out_dim features is cut into
 * workgroup tiles on a device of compute_units CUs; one workgroup fills a
 * CU, so the tiles run in rounds of compute_units. Host-only, no device
 * call; the launches use the same rule:
 *   - whole tiles are 128 tokens x 512 features, numbered token tile major;
 *   - when the R tiles past the last full round fit one round four times
 *     over (4 R <= compute_units), each runs as four 32-token parts, else
 *     when they fit twice over as two 64-token parts (parts follow the
 *     whole tiles; a part covers rows part * part_rows of its tile);
 *   - a launch of fewer tiles than CUs that neither split fits runs as
 *     96-token tiles throughout when those still fit one round.
 * The CFG null rows go with the token tiles: token tile q writes the
 * tile_rows-row null blocks q, q + token_tiles, ...
 *   n              tokens, 0 <= n <= 2^30 (0: no tiles)
 *   out_dim        1 <= D <= 2^20
 *   compute_units  >= 1
 * P3D_ERR_INVALID_ARG for a NULL plan or a value out of range,
 * P3D_ERR_UNSUPPORTED when ceil(n / 128) * ceil(out_dim / 512) >= 2^31 (the
 * fused calls refuse such sizes too). */
typedef struct p3d_tile_plan {
    int32_t tile_rows;      /* tokens per whole tile: 128, or 96 */
    int32_t token_tiles;    /* ceil(n / tile_rows) */
    int32_t feature_tiles;  /* ceil(out_dim / 512) */
    int32_t whole_tiles;    /* tiles that run whole */
    int32_t part_rows;      /* tokens per tail part: 32, 64, or 0 (no parts) */
    int32_t parts;          /* tail parts (4 or 2 per split tile) */
} p3d_tile_plan;

p3d_status p3d_proj_cond_plan(int64_t n, int32_t out_dim, int32_t compute_units,
                              p3d_tile_plan* plan);

/* p3d_proj_linear_grouped -- for each block g in [0, groups):
 *   accumulate == 0:  outs[g][t] = W_g S[t] + b_g
 *   accumulate != 0:  outs[g][t] = outs[g][t] + W_g S[t] + b_g
 * with binary32 accumulation on the matrix cores and one rounding to bf16 at
 * the end (the residual add included). BF16 only.
 *   S        [n, K] bf16 device (from p3d_proj_sample), 16-byte aligned
 *   weights  HOST array [groups] of device [out_dim, K] bf16 pointers
 *   biases   HOST array [groups] of device [out_dim] bf16 pointers (entries
 *            may be NULL), or NULL for none
 *   outs     HOST array [groups] of device [n, out_dim] bf16 pointers
 *            (distinct, not overlapping S)
 *   1 <= groups <= P3D_MAX_GROUPS; K % 8 == 0; out_dim % 8 == 0
 * --------------------------------------------------------------------- */
p3d_status p3d_proj_linear_grouped(const void* S, int64_t n, int32_t K, p3d_dtype dtype,
                                   int32_t groups, const void* const* weights,
                                   const void* const* biases, int32_t out_dim,
                                   void* const* outs, int32_t accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* P3D_H */
