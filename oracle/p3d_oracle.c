/*
 * p3d_oracle.c -- plain CPU oracle for pixel-aligned projection conditioning.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The product (libp3d) never links,
 * calls or reads it, and it shares no source with the product: every step
 * below is written out again here from the pages' description.
 *
 * Sources (web pages; cited by title and section):
 *   [MLX-head]  pixal3d_mrp_mlx, history of tests/, the commit that lands the
 *               pixel-aligned head (proj.py: ProjGrid, project_points,
 *               bilinear_sample, distance_from_fov) and its list of checks
 *               against grid_sample.
 *   [PR38-cam]  trellis.cpp pull request #38 "Initial support for Pixal3D",
 *               commit adding pixal3d.cpp (camera solve, grid projection,
 *               per-stage ProjCond).
 *   [PR38-ext]  same PR, commit exposing extend_pixel (worked example of the
 *               camera distance at 49.13 deg on a 512 px frame).
 *   [PR38-flow] same PR, commit introducing FlowCond / proj_linear (null proj
 *               zeroed on the device).
 *   [PR38-quant] same PR, commit on the cascade requantization: the
 *               projection grid is the endpoint-inclusive linspace(-1, 1,
 *               grid), and Pixal3D maps a high-resolution coordinate to the
 *               NEAREST node, round(u * (grid - 1)), where TRELLIS.2 takes
 *               floor(u * grid).
 *   [PR38-naf]  same PR, commit adding the NAF upsampler: the shape and
 *               texture stages sample two maps (the DINOv3 map and its
 *               NAF-upsampled version) and feed the concatenation, hence
 *               proj_in_channels = 2048.
 *   [PR38-diag] same PR, commits adding projection diagnostics (coverage;
 *               per-half mean/std and the halves' cosine similarity) and the
 *               cross-resolution agreement of samples at the same points.
 *   [PR38-proj] same PR, commit adding proj mode to the DiT: every block
 *               carries its own proj_linear whose output is added into that
 *               block's residual, over a projection that is fixed for the
 *               stage.
 *
 * Precision. Whatever decides an integer (pixel index, in-image mask) is
 * computed in binary32 with one IEEE rounding per operation, in the order
 * written, with no contraction (build with -ffp-contract=off), because the
 * GPU path decides the same integers in binary32. Sums of products (the
 * bilinear blend, the linear layer) accumulate in binary64.
 *
 * Readings taken where the pages are silent:
 *   - token point = cell centre (c + 1/2)/R - 1/2 per axis, world extent +-1/2;
 *     in grid-node mode the point is node c of linspace(-1, 1, R) scaled to
 *     the same extent: c/(R - 1) - 1/2;
 *   - requantization: u = (c + 1/2)/R_src (the source cell centre in [0, 1]);
 *     "round" is to the nearest integer, ties to even, and is evaluated
 *     exactly in integers (no ties occur at the pages' sizes);
 *   - two maps: the sample is map 0's channels followed by map 1's, each map
 *     sampled at the same normalised point on its own height and width;
 *   - per-block linears: the stage's samples S are gathered once and every
 *     block applies Y_g = W_g S + b_g; with a residual, the block's running
 *     value R_g becomes round(R_g + W_g S + b_g), one rounding;
 *   - diagnostics: coverage = tokens with mask 1 / tokens; the per-half
 *     mean/std run over every token and channel of that half's samples as
 *     fed to proj_linear (bf16-rounded for bf16 maps); the cosine is taken
 *     per token between the two halves (equal channel counts) and averaged
 *     over the tokens where both halves are non-zero;
 *   - camera at (0, 0, +d) looking down -Z: depth = d - z;
 *   - FOV is the full angle: focal = 1/tan(fov/2) in normalised image units;
 *   - image y grows downwards: gy = -(f*y)/depth;
 *   - mask = depth > 0 and |gx| <= 1 and |gy| <= 1 (NaN gives 0);
 *   - out-of-image samples keep their border-clamped value (mask only);
 *   - the null (CFG negative) branch zeroes the INPUT of proj_linear, so its
 *     rows equal the bias (or +0 with no bias);
 *   - a batch column outside [0, batch) is clamped for addressing and gets
 *     mask 0.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_VERSION 1

int orc_version(void) { return ORC_VERSION; }

/* Threads used by the row-parallel loops (each output row is computed by one
 * thread on its own, so the thread count never changes a result). */
int orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* ---------------------------------------------------------------- bf16 ---
 * bfloat16 is the upper half of an IEEE binary32: sign, 8 exponent bits,
 * 7 stored mantissa bits. Widening is exact. Narrowing rounds to nearest,
 * ties to even; NaN stays NaN (quiet bit set), infinities stay infinite. */

float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          /* quiet NaN */
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;                                        /* may carry into
                                                              the exponent:
                                                              that is the
                                                              correct result */
    return (uint16_t)kept;
}

/* binary64 -> bf16, correctly rounded (nearest, ties to even) in one step.
 * Rounding first to binary32 with round-to-odd keeps enough information
 * (binary32 carries 16 more significant bits than bf16) for the second
 * rounding to equal the direct one. */
uint16_t orc_f64_to_bf16(double x)
{
    if (isnan(x)) return orc_f32_to_bf16((float)x);
    float t = (float)x;
    if (isfinite(x) && (double)t != x) {
        if (fabs((double)t) > fabs(x))
            t = nextafterf(t, 0.0f);                       /* truncate */
        uint32_t u;
        memcpy(&u, &t, sizeof u);
        u |= 1u;                                           /* sticky bit */
        memcpy(&t, &u, sizeof u);
    }
    return orc_f32_to_bf16(t);
}

void orc_quantize_bf16(const double* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(x[i]);
}

/* -------------------------------------------------------------- camera ---
 * [PR38-cam], [PR38-ext]: only the FOV is free; the distance is the closed
 * form that puts the unit cube's registered corner on the frame border:
 *   d = (1/2) / tan(fov/2) * (S/2) / (S/2 + e)
 * with S the frame size in pixels and e = extend_pixel (pixels the corner is
 * pushed beyond the border). Computed in binary64 with the C library tan. */
double orc_distance_from_fov(double fov_deg, int32_t image_size, int32_t extend_px)
{
    const double pi = 3.14159265358979323846;
    double half_angle = fov_deg * pi / 360.0;
    double half_size = 0.5 * (double)image_size;
    return 0.5 / tan(half_angle) * half_size / (half_size + (double)extend_px);
}

/* The per-image camera handed to the projection: focal = 1/tan(fov/2) and the
 * distance, each rounded once to binary32. */
void orc_camera(double fov_deg, double distance, float* focal, float* dist)
{
    const double pi = 3.14159265358979323846;
    *focal = (float)(1.0 / tan(fov_deg * pi / 360.0));
    *dist = (float)distance;
}

/* ---------------------------------------------------------- projection ---
 * [MLX-head] project_points / ProjGrid; [PR38-cam]: every denoiser token is
 * one cell of a 3-D grid, and that cell is projected into the conditioning
 * image by a fixed camera facing the object. */

static float cell_centre(int32_t c, int32_t R)
{
    return ((float)c + 0.5f) / (float)R - 0.5f;
}

/* [PR38-quant]: node c of the endpoint-inclusive grid linspace(-1, 1, R), in
 * world units (half of the normalised value): c/(R-1) - 1/2. R >= 2. */
static float grid_node(int32_t c, int32_t R)
{
    return (float)c / (float)(R - 1) - 0.5f;
}

/* The world coordinate of integer position c on a grid of R: the cell centre
 * (points == 0) or the grid node (points == 1). */
static float token_point(int32_t c, int32_t R, int32_t points)
{
    return points ? grid_node(c, R) : cell_centre(c, R);
}

/* ---------------------------------------------------- requantization ---
 * [PR38-quant]: a coordinate c on the source grid of R_src cells has the
 * normalised position u = (c + 1/2)/R_src. Mode 0 (Pixal3D) maps it to the
 * nearest node of a grid of G nodes, round(u (G - 1)); mode 1 (TRELLIS.2)
 * to the cell floor(u G). Both are ratios of integers:
 *   u (G - 1) = (2c + 1)(G - 1) / (2 R_src),   u G = (2c + 1) G / (2 R_src),
 * so they are evaluated exactly. Coordinates are clamped to [0, R_src - 1]
 * first; the batch column is copied. */
static int32_t requant_axis(int32_t c, int32_t src_res, int32_t grid, int32_t mode)
{
    if (c < 0) c = 0;
    if (c > src_res - 1) c = src_res - 1;
    int64_t den = 2 * (int64_t)src_res;
    if (mode == 1) return (int32_t)(((2 * (int64_t)c + 1) * grid) / den);
    int64_t num = (2 * (int64_t)c + 1) * (int64_t)(grid - 1);
    int64_t q = num / den, rem = num - q * den;
    if (2 * rem > den || (2 * rem == den && (q & 1))) q += 1;
    return (int32_t)q;
}

void orc_requantize(const int32_t* src, int64_t n, int32_t src_res, int32_t grid,
                    int32_t mode, int32_t* dst)
{
    for (int64_t i = 0; i < n; ++i) {
        dst[4 * i] = src[4 * i];
        for (int k = 1; k < 4; ++k)
            dst[4 * i + k] = requant_axis(src[4 * i + k], src_res, grid, mode);
    }
}

/* grid_sample, align_corners=False, padding_mode='border' ([MLX-head]): a
 * normalised coordinate g maps to the source index ((g+1)*size - 1)/2, the
 * SOURCE INDEX is clamped to [0, size-1], and only then are the two
 * neighbouring texels taken. */
static void source_index(float g, int32_t size, int32_t* i0, int32_t* i1, float* t)
{
    float ix = ((g + 1.0f) * (float)size - 1.0f) / 2.0f;
    ix = fminf(fmaxf(ix, 0.0f), (float)(size - 1));
    float fl = floorf(ix);
    *i0 = (int32_t)fl;
    *t = ix - fl;
    *i1 = (*i0 + 1 < size) ? *i0 + 1 : size - 1;
}

/* The source index mapping alone, for a normalised coordinate g. */
void orc_source_index(float g, int32_t size, int32_t* i0, int32_t* i1, float* t)
{
    source_index(g, size, i0, i1, t);
}

/* Token n's integer cell (b, x, y, z): from coords[n] = (b, x, y, z), or
 * (coords == NULL) from the dense enumeration n = ((b*R + x)*R + y)*R + z. */
static void token_cell(const int32_t* coords, int64_t n, int32_t R, int32_t cell[4])
{
    if (coords) {
        for (int k = 0; k < 4; ++k) cell[k] = coords[4 * n + k];
    } else {
        int64_t r = R;
        cell[3] = (int32_t)(n % r);
        cell[2] = (int32_t)((n / r) % r);
        cell[1] = (int32_t)((n / (r * r)) % r);
        cell[0] = (int32_t)(n / (r * r * r));
    }
}

/* One token: normalised image coordinates, depth, mask, corner indices and
 * fractions. cams: focal[b], dist[b]. */
static void project_one(const int32_t cell[4], int32_t R, int32_t points,
                        const float* focal, const float* dist, int32_t batch,
                        float* gx_out, float* gy_out, float* depth_out,
                        uint8_t* mask_out, int32_t* bsel)
{
    int32_t b = cell[0];
    int valid = (b >= 0 && b < batch);
    if (b < 0) b = 0;
    if (b >= batch) b = batch - 1;
    float px = token_point(cell[1], R, points);
    float py = token_point(cell[2], R, points);
    float pz = token_point(cell[3], R, points);
    float f = focal[b];
    float depth = dist[b] - pz;                 /* camera at +d, looks down -Z */
    float gx = (f * px) / depth;
    float gy = -((f * py) / depth);             /* image rows grow downwards */
    uint8_t m = (uint8_t)(valid && depth > 0.0f && gx >= -1.0f && gx <= 1.0f &&
                          gy >= -1.0f && gy <= 1.0f);
    *gx_out = gx;
    *gy_out = gy;
    *depth_out = depth;
    *mask_out = m;
    *bsel = b;
}

/* Project tokens [0, n). Any output pointer may be NULL.
 *   grid  [n,2] (gx, gy)      pixel [n,2] (x0, y0) after the border clamp
 *   frac  [n,2] (tx, ty)      depth [n]             mask [n] (0/1)       */
void orc_project_ex(const int32_t* coords, int64_t n, int32_t R, int32_t points,
                    const float* focal, const float* dist, int32_t batch,
                    int32_t H, int32_t W,
                    float* grid, int32_t* pixel, float* frac, float* depth,
                    uint8_t* mask)
{
    for (int64_t i = 0; i < n; ++i) {
        int32_t cell[4];
        token_cell(coords, i, R, cell);
        float gx, gy, d;
        uint8_t m;
        int32_t b;
        project_one(cell, R, points, focal, dist, batch, &gx, &gy, &d, &m, &b);
        int32_t x0, x1, y0, y1;
        float tx, ty;
        source_index(gx, W, &x0, &x1, &tx);
        source_index(gy, H, &y0, &y1, &ty);
        if (grid) { grid[2 * i] = gx; grid[2 * i + 1] = gy; }
        if (pixel) { pixel[2 * i] = x0; pixel[2 * i + 1] = y0; }
        if (frac) { frac[2 * i] = tx; frac[2 * i + 1] = ty; }
        if (depth) depth[i] = d;
        if (mask) mask[i] = m;
    }
}

/* Cell-centre projection (the default point mode). */
void orc_project(const int32_t* coords, int64_t n, int32_t R,
                 const float* focal, const float* dist, int32_t batch,
                 int32_t H, int32_t W,
                 float* grid, int32_t* pixel, float* frac, float* depth,
                 uint8_t* mask)
{
    orc_project_ex(coords, n, R, 0, focal, dist, batch, H, W, grid, pixel, frac, depth, mask);
}

/* ------------------------------------------------------ bilinear sample ---
 * [MLX-head] bilinear_sample == grid_sample(bilinear, align_corners=False,
 * padding_mode='border') on a channels-last map feat[b][y][x][c].
 * S[c] = sum over the four corners of weight * F, weights
 * (1-tx)(1-ty), tx(1-ty), (1-tx)ty, tx*ty computed in binary32, the sum in
 * binary64. */

static double feat_at(const void* feat, int32_t is_bf16, int64_t row, int32_t C, int32_t c)
{
    int64_t idx = row * (int64_t)C + c;
    if (is_bf16) return (double)orc_bf16_to_f32(((const uint16_t*)feat)[idx]);
    return (double)((const float*)feat)[idx];
}

static void sample_one(const void* feat, int32_t is_bf16, int32_t b, int32_t H,
                       int32_t W, int32_t C, float gx, float gy, double* out)
{
    int32_t x0, x1, y0, y1;
    float tx, ty;
    source_index(gx, W, &x0, &x1, &tx);
    source_index(gy, H, &y0, &y1, &ty);
    float w00 = (1.0f - tx) * (1.0f - ty);
    float w01 = tx * (1.0f - ty);
    float w10 = (1.0f - tx) * ty;
    float w11 = tx * ty;
    int64_t base = (int64_t)b * H;
    int64_t r00 = (base + y0) * W + x0, r01 = (base + y0) * W + x1;
    int64_t r10 = (base + y1) * W + x0, r11 = (base + y1) * W + x1;
    for (int32_t c = 0; c < C; ++c) {
        out[c] = (double)w00 * feat_at(feat, is_bf16, r00, C, c) +
                 (double)w01 * feat_at(feat, is_bf16, r01, C, c) +
                 (double)w10 * feat_at(feat, is_bf16, r10, C, c) +
                 (double)w11 * feat_at(feat, is_bf16, r11, C, c);
    }
}

/* Sample n points. grid [n,2] normalised (gx, gy); bidx [n] batch item or
 * NULL (item 0; out-of-range items are clamped); out [n,C] binary64. */
void orc_sample(const void* feat, int32_t is_bf16, int32_t batch, int32_t H,
                int32_t W, int32_t C, const float* grid, const int32_t* bidx,
                int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) {
        int32_t b = bidx ? bidx[i] : 0;
        if (b < 0) b = 0;
        if (b >= batch) b = batch - 1;
        sample_one(feat, is_bf16, b, H, W, C, grid[2 * i], grid[2 * i + 1],
                   out + i * (int64_t)C);
    }
}

/* ------------------------------------------------------------- linear ---
 * [PR38-flow] proj_linear: Y[n][d] = sum_c W[d][c] * S[n][c] + bias[d],
 * W row-major [D][C] (a torch Linear weight), accumulated in binary64.
 * bias may be NULL. */
static double param_at(const void* p, int32_t is_bf16, int64_t idx)
{
    if (is_bf16) return (double)orc_bf16_to_f32(((const uint16_t*)p)[idx]);
    return (double)((const float*)p)[idx];
}

void orc_linear(const double* S, int64_t n, int32_t C, const void* weight,
                const void* bias, int32_t is_bf16, int32_t D, double* Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        for (int32_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int32_t c = 0; c < C; ++c)
                acc += param_at(weight, is_bf16, (int64_t)d * C + c) * S[i * (int64_t)C + c];
            if (bias) acc += param_at(bias, is_bf16, d);
            Y[i * (int64_t)D + d] = acc;
        }
    }
}

/* ---------------------------------------------------------- whole path ---
 * Projection conditioning for a chosen subset of output rows.
 * rows[k] in [0, n + n_null): rows below n are tokens (project -> sample ->
 * [bf16 rounding of the sample when the maps are bf16, as a bf16 grid_sample
 * feeding a bf16 Linear would do] -> proj_linear); rows at or above n are the
 * CFG null branch, whose proj input is zero ([PR38-flow]), i.e. the bias.
 * The sample is the concatenation over the n_maps maps ([PR38-naf]): map m
 * is feats[m], [batch, Hs[m], Ws[m], Cs[m]], and the weight is
 * [D, sum of Cs]. Y [nrows, D] binary64 (not yet rounded to the output
 * type), mask [nrows] (null rows: 0). S_scratch holds nrows * sum(Cs). */
void orc_proj_cond_rows_ex(const int32_t* coords, int64_t n, int32_t R, int32_t points,
                           const float* focal, const float* dist, int32_t batch,
                           int32_t n_maps, const void* const* feats, const int32_t* Hs,
                           const int32_t* Ws, const int32_t* Cs, int32_t is_bf16,
                           const void* weight, const void* bias, int32_t D, int64_t n_null,
                           const int64_t* rows, int64_t nrows,
                           double* Y, uint8_t* mask, double* S_scratch)
{
    (void)n_null;
    int32_t C = 0;
    for (int32_t m = 0; m < n_maps; ++m) C += Cs[m];
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t r = rows[k];
        double* y = Y + k * (int64_t)D;
        if (r >= n) {
            for (int32_t d = 0; d < D; ++d) y[d] = bias ? param_at(bias, is_bf16, d) : 0.0;
            if (mask) mask[k] = 0;
            continue;
        }
        int32_t cell[4];
        token_cell(coords, r, R, cell);
        float gx, gy, dep;
        uint8_t msk;
        int32_t b;
        project_one(cell, R, points, focal, dist, batch, &gx, &gy, &dep, &msk, &b);
        double* s = S_scratch + k * (int64_t)C;
        int32_t off = 0;
        for (int32_t m = 0; m < n_maps; ++m) {
            sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy, s + off);
            off += Cs[m];
        }
        if (is_bf16)
            for (int32_t c = 0; c < C; ++c) s[c] = (double)orc_bf16_to_f32(orc_f64_to_bf16(s[c]));
        for (int32_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int32_t c = 0; c < C; ++c)
                acc += param_at(weight, is_bf16, (int64_t)d * C + c) * s[c];
            if (bias) acc += param_at(bias, is_bf16, d);
            y[d] = acc;
        }
        if (mask) mask[k] = msk;
    }
}

/* One map, cell centres. */
void orc_proj_cond_rows(const int32_t* coords, int64_t n, int32_t R,
                        const float* focal, const float* dist,
                        const void* feat, int32_t is_bf16, int32_t batch,
                        int32_t H, int32_t W, int32_t C, const void* weight,
                        const void* bias, int32_t D, int64_t n_null,
                        const int64_t* rows, int64_t nrows,
                        double* Y, uint8_t* mask, double* S_scratch)
{
    const void* feats[1] = {feat};
    orc_proj_cond_rows_ex(coords, n, R, 0, focal, dist, batch, 1, feats, &H, &W, &C, is_bf16,
                          weight, bias, D, n_null, rows, nrows, Y, mask, S_scratch);
}

/* --------------------------------------------------------- diagnostics ---
 * [PR38-diag]: figures that expose a wrong camera, grid or map layout, none
 * of which fails at run time. Over tokens [0, n) (samples as in the whole
 * path, before proj_linear):
 *   out[0] tokens n          out[1] tokens with mask 1
 *   out[2+h] sum of the samples of map h over all tokens and its channels
 *   out[4+h] sum of their squares
 *   out[6]   sum over tokens of cos(S0, S1) = <S0, S1> / (|S0| |S1|), for
 *            two maps with equal channels, over tokens with |S0|, |S1| > 0
 *   out[7]   the number of tokens in out[6]
 * Accumulated in binary64 in token order. */
void orc_projection_stats(const int32_t* coords, int64_t n, int32_t R, int32_t points,
                          const float* focal, const float* dist, int32_t batch,
                          int32_t n_maps, const void* const* feats, const int32_t* Hs,
                          const int32_t* Ws, const int32_t* Cs, int32_t is_bf16,
                          double* out, double* S_scratch)
{
    for (int k = 0; k < 8; ++k) out[k] = 0.0;
    int32_t C = 0;
    for (int32_t m = 0; m < n_maps; ++m) C += Cs[m];
    const int cosine = (n_maps == 2 && Cs[0] == Cs[1]);
    for (int64_t t = 0; t < n; ++t) {
        int32_t cell[4];
        token_cell(coords, t, R, cell);
        float gx, gy, dep;
        uint8_t msk;
        int32_t b;
        project_one(cell, R, points, focal, dist, batch, &gx, &gy, &dep, &msk, &b);
        double* s = S_scratch;
        int32_t off = 0;
        for (int32_t m = 0; m < n_maps; ++m) {
            sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy, &s[off]);
            off += Cs[m];
        }
        if (is_bf16)
            for (int32_t c = 0; c < C; ++c) s[c] = (double)orc_bf16_to_f32(orc_f64_to_bf16(s[c]));
        out[0] += 1.0;
        out[1] += (double)msk;
        off = 0;
        for (int32_t m = 0; m < n_maps; ++m) {
            for (int32_t c = 0; c < Cs[m]; ++c) {
                out[2 + m] += s[off + c];
                out[4 + m] += s[off + c] * s[off + c];
            }
            off += Cs[m];
        }
        if (cosine) {
            double dot = 0.0, n0 = 0.0, n1 = 0.0;
            for (int32_t c = 0; c < Cs[0]; ++c) {
                dot += s[c] * s[Cs[0] + c];
                n0 += s[c] * s[c];
                n1 += s[Cs[0] + c] * s[Cs[0] + c];
            }
            if (n0 > 0.0 && n1 > 0.0) {
                out[6] += dot / (sqrt(n0) * sqrt(n1));
                out[7] += 1.0;
            }
        }
    }
}

/* -------------------------------------------------- diagnostic figures ---
 * [PR38-diag]: the figures printed per stage, from the sums of
 * orc_projection_stats (raw[8] in that layout), written out from their
 * definitions over the N = tokens * C_h samples x of map h:
 *   coverage  = inside / tokens
 *   mean_h    = (1/N) sum x
 *   std_h     = population standard deviation, sqrt((1/N) sum (x - mean)^2),
 *               which the sums give as sqrt((sum x^2 - N mean^2) / N);
 *               rounding can take the radicand a hair below 0 for a constant
 *               map, where the deviation is 0
 *   cosine    = cos_sum / cos_count (mean cosine over the counted tokens)
 * out[6] = {coverage, mean_0, std_0, mean_1, std_1, cosine}; a figure with an
 * empty denominator (no tokens, no map h, no counted token) is NaN. */
void orc_stats_figures(const double* raw, const int32_t* channels, int32_t n_maps,
                       double* out)
{
    const double tokens = raw[0];
    out[0] = tokens > 0.0 ? raw[1] / tokens : NAN;
    for (int32_t h = 0; h < 2; ++h) {
        out[1 + 2 * h] = NAN;
        out[2 + 2 * h] = NAN;
        if (h >= n_maps) continue;
        const double N = tokens * (double)channels[h];
        if (!(N > 0.0)) continue;
        const double mean = raw[2 + h] / N;
        double var = (raw[4 + h] - N * mean * mean) / N;
        if (var < 0.0) var = 0.0;
        out[1 + 2 * h] = mean;
        out[2 + 2 * h] = sqrt(var);
    }
    out[5] = raw[7] > 0.0 ? raw[6] / raw[7] : NAN;
}

/* ------------------------------------------------------ gather once ---
 * The samples S of tokens rows[k] (the whole path before proj_linear):
 * S_out [nrows, sum Cs] binary64, bf16-rounded values for bf16 maps. */
void orc_proj_sample_rows(const int32_t* coords, int64_t n, int32_t R, int32_t points,
                          const float* focal, const float* dist, int32_t batch,
                          int32_t n_maps, const void* const* feats, const int32_t* Hs,
                          const int32_t* Ws, const int32_t* Cs, int32_t is_bf16,
                          const int64_t* rows, int64_t nrows, double* S_out, uint8_t* mask)
{
    int32_t C = 0;
    for (int32_t m = 0; m < n_maps; ++m) C += Cs[m];
    (void)n;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nrows; ++k) {
        int32_t cell[4];
        token_cell(coords, rows[k], R, cell);
        float gx, gy, dep;
        uint8_t msk;
        int32_t b;
        project_one(cell, R, points, focal, dist, batch, &gx, &gy, &dep, &msk, &b);
        double* s = S_out + k * (int64_t)C;
        int32_t off = 0;
        for (int32_t m = 0; m < n_maps; ++m) {
            sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy,
                       S_out + k * (int64_t)C + off);
            off += Cs[m];
        }
        if (is_bf16)
            for (int32_t c = 0; c < C; ++c) s[c] = (double)orc_bf16_to_f32(orc_f64_to_bf16(s[c]));
        if (mask) mask[k] = msk;
    }
}

/* ------------------------------------------------- per-block linears ---
 * [PR38-proj]: for each block g, Y_g[k][d] = sum_c W_g[d][c] S[k][c] + b_g[d]
 * over the given S rows (binary64); with a residual (res_g != NULL, the
 * block's running values at the same rows, binary64), the result is
 * res_g + that. weights / biases: arrays of G parameter pointers (bias
 * entries may be NULL), each [D][K] / [D], f32 or bf16 bits.
 * Y [G][nrows][D]. */
void orc_linear_grouped(const double* S, int64_t nrows, int32_t K, int32_t G,
                        const void* const* weights, const void* const* biases,
                        int32_t is_bf16, int32_t D, const double* const* res, double* Y)
{
    for (int32_t g = 0; g < G; ++g) {
        double* y = Y + (int64_t)g * nrows * D;
        orc_linear(S, nrows, K, weights[g], biases ? biases[g] : NULL, is_bf16, D, y);
        if (res && res[g])
            for (int64_t i = 0; i < nrows * (int64_t)D; ++i) y[i] += res[g][i];
    }
}
