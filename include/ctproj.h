/*
 * ctproj.h -- C ABI of the MI355X (gfx950) ray-driven projector pair.
 *
 * The library computes, for an arbitrary per-view acquisition geometry,
 *
 *   A    : the cell-constant Siddon forward projector.  Entry a_ij is the
 *          length of ray i inside voxel j, so (A x)_i is the line integral of
 *          the piecewise-constant volume along ray i (diffct documentation,
 *          "Differentiable analytical reconstruction"; one ray per detector
 *          pixel, no detector-area integration: "Trajectories and Geometry" >
 *          "Parameterized detector surfaces").
 *   A^T  : its matched adjoint (backprojection), the exact transpose of A
 *          (diffct documentation: Projector.backproject applies the matched
 *          adjoint; the Quickstart pairs A with it and notes that it does not
 *          invert A).
 *   SIRT : x <- x + relax * C A^T R (y - A x) with R = 1/(A 1) per ray and
 *          C = 1/(A^T 1) per voxel, each 0 where the sum is 0 (the pages name
 *          a SIRT solver -- diffct "API Reference" > "Numerical Solvers",
 *          ASTRA SIRT3D_CUDA in the electron-tomography article -- without
 *          printing its formula; this is the standard form).
 *
 * Conventions (diffct documentation, "Trajectories and Geometry" >
 * "Trajectory format"):
 *   - Cartesian (x, y, z) coordinates, origin at the volume centre, one length
 *     unit for positions and spacings.
 *   - Volume: float32, C-contiguous (D, H, W), i.e. index ((z*H)+y)*W+x.
 *     2D beams use D = 1 (dz is then ignored).
 *   - Sinogram: float32, C-contiguous (views, U, V), V fastest.  2D: V = 1.
 *   - Flat-detector pixel (u, v) centre:
 *       det_center + (u - (U-1)/2) du det_u + (v - (V-1)/2) dv det_v.
 *   - fan/cone rays are the segment from the source to the pixel centre;
 *     parallel and parallel3d rays are infinite lines through the pixel
 *     (the Projector class reference describes parallel3d rays as unbounded
 *     lines through the detector pixels).
 *   - Voxels are half-open boxes [lo + k s, lo + (k+1) s): a ray lying exactly
 *     on a lattice plane belongs to the higher-index cell.  On an axis a ray
 *     never crosses (its direction component is 0, or below 2^-40 of the
 *     largest), its coordinate comes from one float64 evaluation of the pixel
 *     origin and counts as on a plane when within 2^-30 cell of it, in the
 *     forward, both adjoints and the intersection count alike, so A and A^T
 *     agree on such rays (pixel centres on planes arise, e.g., from an odd
 *     detector over an even volume at equal pitch).
 *
 * Ownership and threading:
 *   - Every float* argument of the compute calls is a DEVICE pointer owned by
 *     the caller (e.g. a torch tensor's data_ptr()).  The library never frees
 *     or retains them.
 *   - A geometry handle is owned by the library from ct_geom_create until
 *     ct_geom_destroy.  Besides its per-view tables it may hold up to two
 *     volume-sized float32 buffers: copies of the volume in y- or z-fastest
 *     order that the forward projector reads for views whose detector axes run
 *     along y or z (ct_geom_create allocates only those some view needs).  The
 *     forward calls (ct_project, ct_project_region, ct_sirt_residual,
 *     ct_sirt_step*, ct_cgls_*) write these copies, so such calls on one handle
 *     must not overlap in time: they are serialised conveniences.  For
 *     concurrent forward projections with one handle, ct_project_ws takes the
 *     copies in caller workspace and only reads the handle, as every other
 *     call does.
 *   - When the volume fits one buffer, the detector sides are below 2^16 and
 *     the table fits 4 GiB, the handle also holds the adjoint's record table:
 *     64 bytes per (brick, view) pair (bricks of 16 x 16 x 32 voxels, 16 x 16
 *     in 2D), the footprint of the brick on that view's detector and its anchor
 *     ray, built at creation and only read afterwards (512^3 with 720 views:
 *     755 MB).  Adjoint calls over the whole volume read it; region calls
 *     whose boxes are not the whole volume, and handles without the table,
 *     compute the same values in the kernel (the same bits).
 *   - Every compute call is asynchronous and ordered on the caller's stream
 *     (a hipStream_t passed as void*; NULL is the legacy default stream).
 *   - Compute calls allocate nothing: all device memory they touch is the
 *     caller's buffers plus the handle's own buffers.  Two exceptions, both for
 *     problems larger than one buffer: on a lattice of >= 2^30 voxels the
 *     volume copies are allocated by the first ct_project_region at that
 *     region's size (and grown when a later region is larger), and the
 *     host-streaming calls allocate and free their own device staging.
 *
 * Errors: every call returns a ct_status_t.  Host-side validation happens
 * before anything is enqueued; on error nothing was launched.  A launch
 * failure reported by the HIP runtime is returned as CT_E_HIP.  No C++
 * exception crosses this interface.  ct_last_error() gives a message for the
 * most recent failing call on the calling thread.
 */
#ifndef CTPROJ_H
#define CTPROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ct_geom_s *ct_geom_t;     /* opaque, library-owned */
typedef void *ct_stream_t;               /* a hipStream_t; NULL = default stream */

typedef enum {
    CT_PARALLEL2D = 0,   /* rows: ray_dir, det_origin (= detector centre), det_u   */
    CT_FAN2D = 1,        /* rows: src_pos, det_center, det_u                       */
    CT_CONE = 2,         /* rows: src_pos, det_center, det_u, det_v                */
    CT_PARALLEL3D = 3    /* rows: ray_dir, det_center, det_u, det_v                */
} ct_beam_t;

typedef enum {
    CT_OK = 0,
    CT_E_NULL = 1,       /* a required pointer is NULL                              */
    CT_E_SHAPE = 2,      /* a size is zero/negative or inconsistent with the beam  */
    CT_E_NONFINITE = 3,  /* a frame value or spacing is NaN or infinite            */
    CT_E_FRAME = 4,      /* axes not unit / not orthogonal, ray tangent to the
                            detector, source on the detector plane or at its centre */
    CT_E_RANGE = 5,      /* geometry too far from the volume, or sizes beyond the
                            library's limits                                        */
    CT_E_ALIAS = 6,      /* an output buffer overlaps another buffer of the call    */
    CT_E_NOMEM = 7,      /* device allocation of the handle's tables failed         */
    CT_E_HIP = 8,        /* the HIP runtime reported an error                       */
    CT_E_ARG = 9         /* invalid enum value, handle, spacing or scalar argument  */
} ct_status_t;

typedef struct {
    int32_t beam;               /* ct_beam_t */
    int32_t reserved;           /* must be 0 */
    int64_t n_views;            /* >= 1 */
    int64_t vol_shape[3];       /* (D, H, W); 2D beams: D = 1 */
    double voxel_spacing[3];    /* (dz, dy, dx) > 0; 2D: dz ignored */
    int64_t det_shape[2];       /* (U, V); 2D beams: V = 1 */
    double det_spacing[2];      /* (du, dv) > 0; 2D: dv ignored */
    const double *frames;       /* HOST pointer, n_views x 12 float64, row-major:
                                   a(3) c(3) e_u(3) e_v(3) in (x, y, z) order, with
                                   a = src_pos (fan, cone) or ray_dir (parallel,
                                   parallel3d), c = detector centre.  2D beams: all
                                   z components 0, e_v ignored.  Copied at create. */
} ct_geom_desc_t;

/*
 * Frame validation only (host, float64, no device work).  Rules follow diffct
 * "Trajectories and Geometry" > "Custom acquisition example": finite values,
 * the same nonzero view count, unit direction axes, ray_dir orthogonal to
 * det_u (2D parallel), det_u orthogonal to det_v (3D), parallel3d rays not
 * tangent to the detector plane, fan/cone source not at the detector centre
 * and not viewing the detector edge-on, the nearer of source and detector
 * centre within 1e6 voxel spacings of the origin and both within 1e15.
 * Tolerances: |norm - 1| <= 1e-6, |dot| <= 1e-6, |ray . normal| > 1e-6.
 * Library limits: each extent < 2^20, voxel spacings in [1e-10, 1e10] within a
 * ratio of 1e6 of each other.  Calls that take the whole volume or sinogram as
 * one device buffer further need D*H*W < 2^30 and views*U*V < 2^31 (else
 * CT_E_RANGE); larger problems go through the region and host-streaming calls,
 * whose device buffers obey the same two bounds.
 */
ct_status_t ct_geom_validate(const ct_geom_desc_t *desc);

/* Validate, precompute the per-view float64 ray table, allocate and upload it
 * to the current HIP device, and build the adjoint's record table there when it
 * fits (synchronous).  *out receives the handle. */
ct_status_t ct_geom_create(const ct_geom_desc_t *desc, ct_geom_t *out);

/* Create a geometry whose detector is a parameterized surface (diffct
 * documentation, "Trajectories and Geometry" > "Parameterized detector
 * surfaces"): pixel (u, v) of view k sits at the world point
 *   c + o_u e_u + o_v e_v + o_n n,   n = e_u x e_v  (2D: (e_u_y, -e_u_x, 0)),
 * with (c, e_u, e_v) the view's frame and (o_u, o_v, o_n) the pixel's local
 * offsets in physical units.  offsets: HOST float64, row-major (U, V, 3), shared
 * by every view (per_view = 0), or (n_views, U, V, 3) (per_view != 0); 2D beams
 * use V = 1 and need o_v = 0.  Rays are built exactly as for the flat detector
 * with the surface point in place of the flat pixel centre (fan/cone: from the
 * source to the point; parallel: through the point along the ray direction),
 * so project/backproject keep the matched Siddon model, one ray per pixel.
 * The flat-detector frame checks of ct_geom_create apply; in addition offsets
 * must be finite and every fan/cone pixel must lie in front of the source
 * (CT_E_FRAME).  The handle also keeps the offsets (float64) and per-view
 * footprint bounds on the device.  Synchronous, like ct_geom_create. */
ct_status_t ct_geom_create_surface(const ct_geom_desc_t *desc, const double *offsets, int per_view,
                                   ct_geom_t *out);

/* Free the handle and its device tables.  NULL is accepted.  The caller must
 * make sure no work using the handle is still pending. */
ct_status_t ct_geom_destroy(ct_geom_t g);

/* Host copy of the per-view ray table (n_views x CT_VIEW_TABLE_STRIDE doubles),
 * for inspection.  Works without a device: it may be called on a handle made by
 * ct_geom_create, or with desc != NULL and g == NULL to compute it on the host. */
#define CT_VIEW_TABLE_STRIDE 48
ct_status_t ct_geom_view_table(ct_geom_t g, const ct_geom_desc_t *desc, double *out);

/* Range of the adjoint's fixed-point accumulation, for inspection (host only,
 * no device work; with g == NULL it is computed from desc, surface != 0 for a
 * parameterized detector).  *rays_bound receives a bound on the (ray, voxel)
 * pairs one voxel can collect over all views: per view, the pixel centres in
 * the voxel's image on a flat detector, (e_u + 1)(e_v + 1) for an image of
 * e_u x e_v pixels (fan/cone: magnified at the volume corner nearest the
 * source plane; a volume reaching that plane, or a surface detector: U V).
 * Each pair adds less than 2^46 units, and the 64-bit sums are kept below
 * 2^62: *shift receives the right shift applied to every term, 0 unless
 * *rays_bound >= 2^16 (then ceil(log2(*rays_bound)) - 16).  Each ray still
 * keeps its own 24 significant bits, so the shift costs no precision beyond
 * one accumulator unit per term. */
ct_status_t ct_geom_adjoint_range(ct_geom_t g, const ct_geom_desc_t *desc, int surface, double *rays_bound,
                                  int32_t *shift);

/* Which adjoint a geometry takes (host only when desc is given, no device work;
 * or from a handle g, then desc is ignored).  surface: the geometry has a
 * parameterized detector (always the brick walk).
 *   CT_ADJOINT_BRICK: rays binned per 16 x 16 x 32 brick and walked through it,
 *     exact 64-bit integer sums in LDS.
 *   CT_ADJOINT_LINE: a separable tilt series -- parallel3d, every view's rays
 *     inside planes of one volume axis d, one detector axis running along d at
 *     exactly one pixel per voxel (|pixel step| = voxel spacing along d) and the
 *     other detector axis without a d component.  Then the rays of one pixel
 *     column lie in one voxel plane and each plane is a 2D parallel projection
 *     (the electron-tomography article's dual-axis tilt series about x and y is
 *     such a geometry).  The adjoint
 *     forms each ray's chord through a voxel once per line of 32 voxels along d
 *     (16 when some views' planes are z planes, or a view's rows are too dense
 *     for a 32 x 32 x 16 brick to stage them), from the ray's offset to the
 *     voxel's centre (the chord of a line through a square), and sums chord *
 *     value in float32 over 32 views, then in the brick's float32 accumulator:
 *     per voxel the error is within about (2 * rays per voxel and 32 views +
 *     views / 32) * 2^-24 of sum_i |a_ij y_i|.  A ray lying on a voxel plane
 *     belongs to the higher voxel, as in the walks. */
enum { CT_ADJOINT_BRICK = 0, CT_ADJOINT_LINE = 1 };
ct_status_t ct_geom_adjoint_kind(ct_geom_t g, const ct_geom_desc_t *desc, int surface, int32_t *kind);

/* Forward projection A: sino[view][u][v] = sum_j a_ij vol[j].
 * vol: device (D,H,W) float32; sino: device (views,U,V) float32.
 * Every ray is written, missed rays as 0 (diffct "Large Volumes and Chunked
 * Execution" > "Resident layouts and accumulation": forward kernels overwrite
 * each ray, including missed rays).  vol and sino must not overlap; vol must
 * hold finite values (a non-finite voxel may spread to rays that pass near it). */
ct_status_t ct_project(ct_geom_t g, const float *vol, float *sino, ct_stream_t stream);

/* The same forward projection with the volume copies in caller memory, so the
 * handle is only read: calls with one handle may run concurrently on
 * different streams as long as each has its own work buffer (the handle is
 * then immutable after create, as the library's other read-only calls treat
 * it).  ct_project is the serialised convenience that keeps the copies in the
 * handle.  work: DEVICE memory of at least ct_forward_workspace_size bytes,
 * 256-byte aligned, caller-owned scratch (overwritten; it may be NULL when
 * that size is 0, i.e. every view gathers from the caller's x-fastest
 * volume); it must not overlap vol or sino.  Same results as ct_project, bit
 * for bit. */
ct_status_t ct_project_ws(ct_geom_t g, const float *vol, float *sino, void *work, size_t work_bytes,
                          ct_stream_t stream);

/* Bytes of ct_project_ws workspace: one volume-sized float32 copy, rounded up
 * to 256 bytes, per axis order other than x-fastest that some view's gathers
 * use (y- and/or z-fastest; 0 for 2D beams and for geometries whose views all
 * gather along x).  From a handle, or with g == NULL computed on the host from
 * desc (no device work). */
ct_status_t ct_forward_workspace_size(ct_geom_t g, const ct_geom_desc_t *desc, size_t *bytes);

/* Matched adjoint A^T: vol[j] = sum_i a_ij sino[i]; every voxel is overwritten.
 * Volume bricks accumulate their rays in on-chip memory (LDS) and are each
 * written once, with no global atomics.  Each term is a product of a
 * fixed-point piece length (2^-23 of a voxel diagonal) and the ray value in
 * fixed point, summed in 64-bit integers, so the result is bit-for-bit the
 * same on every run (unlike an adjoint built on float atomics: the diffct
 * documentation notes run-to-run differences of its atomic adjoint in
 * "Example results").  Range: each ray value keeps 24 significant bits
 * whatever the other rays of its brick hold (rays far below the brick's
 * largest are stored as a mantissa whose products are shifted down), so per
 * voxel the error stays near float32's 2^-24 of sum_i |a_ij y_i|; rays below
 * 2^-46 of the largest ray crossing the same 16 x 16 x 32 brick add nothing.
 * The sums cannot overflow (ct_geom_adjoint_range).  sino must hold finite
 * values; sino and vol must not overlap. */
ct_status_t ct_backproject(ct_geom_t g, const float *sino, float *vol, ct_stream_t stream);

/* The same A^T by one lane per ray with global float atomics (a measured
 * baseline; float32 summation order varies between runs, as the diffct
 * documentation notes for its atomic adjoint in "Example results"). */
ct_status_t ct_backproject_atomic(ct_geom_t g, const float *sino, float *vol, ct_stream_t stream);

/* ---- Ordered subsets (SART) ----
 * The ASTRA guide lists SART with MinConstraint / MaxConstraint /
 * ReconstructionMask.  Read here as ordered-subset SIRT: the views are taken in
 * subsets [view_begin, view_end) one after another, and each subset applies the
 * bounded, masked SIRT step of its own rays,
 *   x <- clip(x + relax * C_s * A_s^T R_s (y_s - A_s x), lo, hi) where mask != 0,
 * with R_s = 1 / (A_s 1) (the subset's rows of R) and C_s = 1 / (A_s^T 1) (0 where
 * the sums are 0).  One view per subset is SART; the whole range is SIRT.
 * ct_sirt_weights_views: row_inv_batch (view_end - view_begin, U, V) and
 * col_inv (D, H, W) for the subset.  ct_sirt_step_views: y_batch, row_inv_batch
 * and work_batch hold the subset's views; lo = -inf, hi = +inf and mask = NULL
 * give the plain step.  Device buffers, asynchronous on stream.  Errors as for
 * ct_sirt_step_bounded, plus CT_E_SHAPE for an empty or out-of-range view range
 * (checked first). */
ct_status_t ct_sirt_weights_views(ct_geom_t g, int64_t view_begin, int64_t view_end,
                                  float *row_inv_batch, float *col_inv, ct_stream_t stream);
ct_status_t ct_sirt_step_views(ct_geom_t g, int64_t view_begin, int64_t view_end, float *x,
                               const float *y_batch, const float *row_inv_batch,
                               const float *col_inv, float relax, float lo, float hi,
                               const uint8_t *mask, float *work_batch, ct_stream_t stream);

/* ---- Regions and view batches (chunked execution) ----
 * The diffct documentation ("Large Volumes and Chunked Execution" > "Resident
 * layouts and accumulation") splits large problems into volume tiles and view
 * batches: projection adds the disjoint tile integrals, the adjoint accumulates
 * each tile over the view batches, tiles keep the global lattice so cells on
 * internal boundaries keep their owner.  These two calls are those building
 * blocks.  A region is a box of voxel indices inside the volume; its buffer is a
 * contiguous (nz, ny, nx) float32 array holding just that box.  A view batch is
 * the views [view_begin, view_end) of the handle; its sinogram buffer is
 * (view_end - view_begin, U, V).  Summing ct_project_region over disjoint regions
 * that cover the volume gives ct_project (up to float32 summation order), and
 * ct_backproject_region over view batches, accumulated, gives the region of
 * ct_backproject.
 * Errors: CT_E_SHAPE if the box is empty or leaves the volume or the view range is
 * empty or leaves [0, n_views) (checked first, so empty buffers may be NULL);
 * CT_E_NULL for a NULL buffer; CT_E_ALIAS if the two buffers overlap. */
typedef struct {
    int64_t z0, y0, x0;   /* first voxel of the box (z, y, x) */
    int64_t nz, ny, nx;   /* its extents, >= 1, inside the volume */
} ct_region_t;

/* sino_batch (+)= A restricted to the region's voxels, for the batch's views.
 * accumulate = 0 overwrites every ray of the batch (rays missing the region get
 * 0); accumulate != 0 adds to what sino_batch holds.  Device buffers; they must
 * not overlap.  Forward calls on one handle must not overlap in time. */
ct_status_t ct_project_region(ct_geom_t g, const float *vol_region, ct_region_t region,
                              int64_t view_begin, int64_t view_end, float *sino_batch, int accumulate,
                              ct_stream_t stream);

/* vol_region (+)= A^T of the batch's rays, restricted to the region.
 * accumulate = 0 overwrites every voxel of the region; != 0 adds (the brick
 * adjoint, bit-reproducible per call). */
ct_status_t ct_backproject_region(ct_geom_t g, const float *sino_batch, int64_t view_begin,
                                  int64_t view_end, ct_region_t region, float *vol_region,
                                  int accumulate, ct_stream_t stream);

/* ---- Host streaming (volumes and sinograms in host memory) ----
 * The out-of-core pattern of the diffct documentation ("Large Volumes and
 * Chunked Execution"): the data stay in host memory and pass through the
 * device in slabs of the volume and batches of views, built on the region
 * calls above, with uploads, kernels and downloads on three streams of their
 * own so transfers overlap the kernels.  A^T runs slabs outer, batches inner
 * (each slab accumulates every batch on the device, then is downloaded); A
 * runs batches outer, slabs inner.  With one batch (batch_views >= n_views)
 * the sinogram is uploaded once; with one slab the volume is.
 * Slab axis: z slabs are contiguous in host memory; y and x slabs are copied
 * as pitched 2D blocks.  The forward is slow on slabs whose faces are normal
 * to the detector rows' direction e_v (the rays of one wave enter such a face
 * at widely spread points): with axis = -1 the forward slabs along z unless
 * e_v leans mostly on z (e.g. a circular cone orbit about z), else along the
 * one of y and x that e_v leans on least; the adjoint slabs along z (y in 2D).
 *
 * sino_host: (n_views, U, V) float32, vol_host: (D, H, W) float32, both HOST
 * memory owned by the caller; allocated with hipHostMalloc the copies run
 * asynchronously, pageable memory works with staged copies.  The calls are
 * synchronous: they first wait for the work queued on `stream`, and return
 * when the output is in host memory.  Device memory allocated and freed per
 * call: A^T: (1 or 2) x slab voxels + (1 or 2) x batch_views*U*V floats (two
 * buffers only when there is more than one slab / batch); A likewise.  The
 * handle's forward volume copies are grown to the slab size if smaller.
 * The A^T result is bit-reproducible for a given plan.
 *
 * Errors: CT_E_ARG if a plan size is < 1; CT_E_RANGE if a slab has >= 2^30
 * voxels or a batch >= 2^31 rays; CT_E_ALIAS if the host buffers overlap;
 * CT_E_NOMEM if staging cannot be allocated; CT_E_HIP for copy or launch
 * failures (the output is then incomplete). */
typedef struct {
    int64_t slab;          /* planes per device slab along `axis` (>= 1; clamped to the extent) */
    int64_t batch_views;   /* views per device batch (>= 1; clamped to n_views) */
    int32_t axis;          /* slab normal: 0 = z, 1 = y, 2 = x, -1 = chosen by the library */
    int32_t reserved;      /* must be 0 */
} ct_stream_plan_t;

ct_status_t ct_backproject_host(ct_geom_t g, const float *sino_host, float *vol_host,
                                ct_stream_plan_t plan, ct_stream_t stream);
ct_status_t ct_project_host(ct_geom_t g, const float *vol_host, float *sino_host,
                            ct_stream_plan_t plan, ct_stream_t stream);

/* ---- Analytical FBP / FDK (a second operator, not the Siddon pair) ----
 * diffct documentation, "Differentiable analytical reconstruction" and the API
 * reference's "Analytical Reconstruction Helpers" and "Ramp Filter Options":
 * FBP (parallel2d, fan2d) and FDK (cone) on a flat detector run
 *   1. pre-weights: the fan/cone cosine weight |(p - a).n| / |p - a| of each
 *      pixel, and Parker's short-scan weights when short_scan is set;
 *   2. a ramp filter along u, zero-padded to pad_factor * U samples and applied
 *      as a real multiplier: the band-limited Ram-Lak ramp (Ramachandran and
 *      Lakshminarayanan; Kak and Slaney ch. 3) times the chosen window of
 *      f = k / P (Shepp-Logan sin(pi f)/(pi f), cosine cos(pi f), Hamming
 *      0.54 + 0.46 cos(2 pi f), Hann 0.5 + 0.5 cos(2 pi f));
 *   3. angular weights: half the gap to the neighbouring views, periodic over
 *      2 pi (fan/cone) or pi (parallel), one-sided at the ends for short scans,
 *      times 1/2 for full fan/cone turns; or the caller's own;
 *   4. the voxel-driven interpolating weighted backprojection: each voxel
 *      centre x gathers, per view, the bilinearly interpolated filtered value
 *      where it projects, times R D / U(x)^2 (fan/cone: U(x) = (x - a).n,
 *      D = (c - a).n, R = (iso - a).n) or 1 (parallel); samples outside the
 *      detector are 0, and a voxel at or behind the source (U(x) <= 0) lies
 *      on no ray of that view and gathers nothing from it.  Its transpose
 *      scatters the same coefficients.
 * It is not the ct_backproject adjoint.  ct_fbp_filter does 1-3,
 * ct_fbp_backproject does 4, ct_fbp_run does both. */
typedef struct ct_fbp_s *ct_fbp_t;       /* opaque, library-owned */

typedef enum {
    CT_WINDOW_RAMLAK = 0,
    CT_WINDOW_SHEPP_LOGAN = 1,
    CT_WINDOW_COSINE = 2,
    CT_WINDOW_HAMMING = 3,
    CT_WINDOW_HANN = 4
} ct_window_t;

typedef struct {
    int32_t window;       /* ct_window_t */
    int32_t pad_factor;   /* zero padding of each row to pad_factor * U samples, 1..16 */
    int32_t short_scan;   /* fan/cone: Parker weights; the angles must span pi + 2 x half fan angle */
    int32_t iso_given;    /* iso[] holds the isocentre; else the least-squares point nearest the
                             lines through each source along its detector normal */
    double iso[3];        /* world (x, y, z) */
    int64_t reserved;     /* must be 0 */
} ct_fbp_opts_t;

/* Builds a plan on the current device (synchronous): validates desc (same
 * rules as ct_geom_validate; beams parallel2d, fan2d, cone; flat detector;
 * U <= 4096, pad_factor * U <= 16384, U >= 2 and for cone V >= 2), computes the
 * filter, the angular and Parker weights and the per-view backprojection
 * tables in float64, and uploads them.  angles: HOST, n_views radians (needed
 * unless angular_weights is given, and always for short scans);
 * angular_weights: HOST, n_views, or NULL for the rule above.
 * A cone-beam plan also owns device staging for the backprojection: the
 * filtered sinogram of one batch of nb <= 128 views in pair-interleaved form
 * with a border of zeros (8 nb (U + 1)(V + 2) bytes, at most 4 GiB unless one
 * view alone needs more; the views are split into equal batches).  Backprojections
 * with one plan therefore share it: calls of ct_fbp_backproject or ct_fbp_run
 * with the same plan on different streams must not overlap in time.
 * Errors: CT_E_NULL, CT_E_ARG (beam, window, pad, short scan on parallel, a
 * span too short, an isocentre that cannot be estimated), CT_E_SHAPE,
 * CT_E_RANGE (also a cone detector with (U + 1)(V + 2) >= 2^29, whose one-view
 * staging would pass 32-bit byte offsets, or with V + 2 >= 2^20, whose row
 * stride would pass the gather's 24-bit offset arithmetic), CT_E_NONFINITE,
 * CT_E_NOMEM, CT_E_HIP. */
ct_status_t ct_fbp_create(const ct_geom_desc_t *desc, const double *angles,
                          const double *angular_weights, const ct_fbp_opts_t *opts, ct_fbp_t *out);
ct_status_t ct_fbp_destroy(ct_fbp_t f);
/* The plan's isocentre (3 doubles) and angular weights (n_views doubles); either may be NULL. */
ct_status_t ct_fbp_info(ct_fbp_t f, double *iso, double *angular_weights);

/* Overrides of the filter stage and per-slice view weights (diffct
 * documentation, "Differentiable analytical reconstruction": the paragraph on
 * the complete APIs, and "Helical approximation").  Every pointer is HOST
 * memory read during ct_fbp_create_ext only; NULL keeps the default.
 *   filter_response: pad_factor * U / 2 + 1 real multipliers M_k (k = 0..P/2,
 *     P = pad_factor * U) in physical units, used in place of the windowed
 *     Ram-Lak multiplier of step 2 (opts->window is then ignored);
 *   projection_weights: pre-weights used in place of the cosine weight of
 *     step 1 (Parker's weights, when short_scan is set, still multiply);
 *     U * V values (index u * V + v) shared by every view, or, when
 *     projection_weights_per_view is 1, n_views * U * V values (view-major);
 *   slice_weights (cone only): D * n_views values, w[s * n_views + i] the
 *     weight of view i for the voxels of axial slice s (z index s).  Step 3
 *     then applies no angular weight and step 4 multiplies view i's
 *     contribution to a voxel of slice s by w[s][i]; the transpose scatters
 *     with the same factors.  ct_helical_view_weights computes the helical
 *     approximation's weights; any others may be passed.  Not combinable
 *     with angular_weights or short_scan.  Views whose weights are 0 for a
 *     whole band of 64 slices are skipped there.
 * reserved fields must be 0. */
typedef struct {
    const double *filter_response;
    const double *projection_weights;
    const double *slice_weights;
    int32_t projection_weights_per_view;   /* 0: U * V shared values; 1: n_views * U * V */
    int32_t direct_filter;    /* 1: step 2 always by direct circular convolution with the
                                 P-periodic kernel; 0: through FFTs when P is a power of
                                 two in [64, 4096] (the same filter either way) */
    int64_t reserved[4];
} ct_fbp_ext_t;

/* ct_fbp_create with the overrides above (ext NULL: exactly ct_fbp_create).
 * With slice_weights, angles may be NULL, and ct_fbp_info reports angular
 * weights of 1.  Errors: those of ct_fbp_create, and CT_E_ARG (slice weights
 * on a non-cone beam or with angular_weights / short_scan, a per-view or
 * direct-filter flag other than 0 or 1, nonzero reserved fields), CT_E_NONFINITE (a non-finite
 * override value). */
ct_status_t ct_fbp_create_ext(const ct_geom_desc_t *desc, const double *angles,
                              const double *angular_weights, const ct_fbp_opts_t *opts,
                              const ct_fbp_ext_t *ext, ct_fbp_t *out);

/* Per-slice view weights of the helical approximation (same page, "Helical
 * approximation"): the rows are filtered once, and each axial slice is
 * reconstructed from the full turn of views centred where the source crosses
 * it, with the half redundancy factor.  Computed on the host in float64:
 *   theta_c(s) = the unwrapped angle at which the source z (frames' a_z)
 *     reaches the slice centre z_s (voxel-centre z), by linear interpolation
 *     between the two samples around it;
 *   w[s][i] = 1/2 * integral over [theta_c - pi, theta_c + pi] of the hat
 *     function of view i (the piecewise-linear interpolation basis on the
 *     angles), so that each slice's weights sum to pi.
 * desc: a cone geometry (validated as by ct_geom_validate) with n_views >= 2;
 * angles: HOST, n_views unwrapped radians, strictly monotone; the source z
 * must be strictly monotone too.  weights: HOST, D * n_views doubles
 * (slice-major), written on success only.
 * Errors: CT_E_NULL, CT_E_ARG (beam not cone, fewer than 2 views, angles or
 * source z not strictly monotone), CT_E_NONFINITE, CT_E_RANGE (a slice centre
 * outside the source's z range, or a slice whose full turn leaves the
 * scanned angles: incomplete windows are rejected). */
ct_status_t ct_helical_view_weights(const ct_geom_desc_t *desc, const double *angles, double *weights);

/* filtered = steps 1-3 of sino; (views, U, V) device buffers that must not overlap. */
ct_status_t ct_fbp_filter(ct_fbp_t f, const float *sino, float *filtered, ct_stream_t stream);
/* vol = step 4 of filtered (overwrites every voxel).  Cone: per batch of views,
 * the plan's staging receives the batch pair-interleaved, (q[u][v], q[u+1][v])
 * per pixel inside a border of zeros, so that one 16-byte load fetches the four
 * bilinear taps; the first batch writes vol, the later ones add to it. */
ct_status_t ct_fbp_backproject(ct_fbp_t f, const float *filtered, float *vol, ct_stream_t stream);
/* sino = transpose of step 4 applied to vol (overwrites; float atomics, so the
 * order of additions, and the last bits, vary between runs). */
ct_status_t ct_fbp_backproject_transpose(ct_fbp_t f, const float *vol, float *sino, ct_stream_t stream);
/* vol = FBP/FDK of sino, with work (sinogram-sized) holding the filtered data. */
ct_status_t ct_fbp_run(ct_fbp_t f, const float *sino, float *work, float *vol, ct_stream_t stream);

/* SIRT weights (once per geometry): row_inv[i] = 1/(A 1)_i, col_inv[j] =
 * 1/(A^T 1)_j, each 0 where the sum is 0.  row_inv: (views,U,V); col_inv:
 * (D,H,W); device float32, non-overlapping. */
ct_status_t ct_sirt_weights(ct_geom_t g, float *row_inv, float *col_inv, ct_stream_t stream);

/* First half of a SIRT iteration: work_sino = row_inv * (y - A x). */
ct_status_t ct_sirt_residual(ct_geom_t g, const float *x, const float *y, const float *row_inv,
                             float *work_sino, ct_stream_t stream);

/* Second half: x += relax * col_inv * A^T work_sino (x read and written in place). */
ct_status_t ct_sirt_update(ct_geom_t g, const float *work_sino, const float *col_inv, float relax,
                           float *x, ct_stream_t stream);

/* One SIRT iteration = ct_sirt_residual then ct_sirt_update, stream-ordered.
 * work_sino is caller scratch of sinogram size; relax must be finite. */
ct_status_t ct_sirt_step(ct_geom_t g, float *x, const float *y, const float *row_inv,
                         const float *col_inv, float relax, float *work_sino, ct_stream_t stream);

/* Bounded and masked SIRT (the box constraints and reconstruction mask of the
 * ASTRA SART/SIRT options printed in the ASTRA guide: MinConstraint,
 * MaxConstraint, ReconstructionMask).  The update becomes
 *   x_j <- min(max(x_j + relax * col_inv_j * (A^T work_sino)_j, lo), hi)
 * for voxels with mask[j] != 0, while voxels with mask[j] == 0 keep their value
 * (mask: device uint8, volume-shaped, or NULL for all voxels).  lo <= hi; either
 * may be infinite.  A brick with no masked voxel is skipped entirely. */
ct_status_t ct_sirt_update_bounded(ct_geom_t g, const float *work_sino, const float *col_inv,
                                   float relax, float lo, float hi, const uint8_t *mask, float *x,
                                   ct_stream_t stream);

/* One bounded/masked SIRT iteration: ct_sirt_residual then
 * ct_sirt_update_bounded, stream-ordered. */
ct_status_t ct_sirt_step_bounded(ct_geom_t g, float *x, const float *y, const float *row_inv,
                                 const float *col_inv, float relax, float lo, float hi,
                                 const uint8_t *mask, float *work_sino, ct_stream_t stream);

/* ---- CGLS: conjugate gradients on the least-squares problem min ||A x - y||_2 ----
 * The solver the diffct documentation benchmarks ("Performance": time per CGLS
 * iteration at 512^3) and ships ("API Reference" > "Numerical Solvers": cgls);
 * its state is x, s, p (volume-shaped) and r, q (sinogram-shaped) with float64
 * norms ("Large Volumes and Chunked Execution" > "Runnable iterative
 * reconstruction").  The pages give no formula; the standard recurrence is:
 *   start:  r = y - A x,  s = A^T r,  p = s,  gamma = ||s||^2
 *   step:   q = A p,  alpha = gamma / ||q||^2,  x += alpha p,  r -= alpha q,
 *           s = A^T r,  beta = ||s||^2 / gamma,  gamma = ||s||^2,  p = s + beta p
 * (alpha = 0 when ||q|| = 0 and beta = 0 when gamma = 0, so a converged state
 * stays put).  Vectors are float32; the norms are float64 sums in a fixed order
 * and the scalars stay in the caller's workspace on the device, so a step
 * needs no host round trip and its result is the same on every run.  Every
 * buffer is device memory; none may overlap another of the call. */

/* Bytes of device workspace (8-byte aligned) that ct_cgls_init/ct_cgls_step
 * need for this geometry: 256 bytes of scalars plus one float64 per block of
 * the largest launch. */
ct_status_t ct_cgls_workspace_size(ct_geom_t g, size_t *bytes);

/* Start: r = y - A x (x is the caller's initial volume, e.g. zeros), s = A^T r,
 * p = s, and the scalars in work.  y, r: (views,U,V); x, s, p: (D,H,W). */
ct_status_t ct_cgls_init(ct_geom_t g, const float *y, const float *x, float *r, float *s, float *p,
                         void *work, ct_stream_t stream);

/* One iteration, updating x, r, s, p, q and the scalars in work in place. */
ct_status_t ct_cgls_step(ct_geom_t g, float *x, float *r, float *s, float *p, float *q, void *work,
                         ct_stream_t stream);

/* One CGLS iteration that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The same kernels and results as ct_cgls_step, bit
 * for bit; the per-block partial sums live in a fixed 32 MiB array in the
 * library's device memory (one per GPU, held until the process ends) instead
 * of the caller's workspace.  state: the first 256 bytes of a workspace that
 * ct_cgls_init filled (the scalars), device memory, 8-byte aligned, read and
 * updated in place.  Geometries whose largest launch has more than 2^22
 * blocks (see ct_cgls_workspace_size: its bytes / 8 - 32) are rejected with
 * CT_E_RANGE before any launch.  All calls on one GPU share the array, so
 * calls that overlap in time on one GPU (different streams or threads) race;
 * the first call on a device looks the array up there. */
ct_status_t ct_cgls_step_noalloc(ct_geom_t g, float *x, float *r, float *s, float *p, float *q, double *state,
                                 ct_stream_t stream);

/* Copy the scalars to the host (synchronises the stream): out[0] = gamma =
 * ||A^T r||^2, out[1] = alpha and out[2] = beta of the last step, out[3] =
 * ||q||^2 of the last step, out[4] = ||r||^2. */
ct_status_t ct_cgls_scalars(ct_geom_t g, const void *work, double out[5], ct_stream_t stream);

/* Ray-voxel intersections: the number of (ray, voxel) pairs the traversal
 * visits, i.e. per ray the number of lattice-plane crossings inside the volume
 * plus one, from the float64 entry and exit cells.  This equals the number of
 * pairs with positive length except where a ray crosses two planes at exactly
 * the same point.  per_ray (device uint32, sinogram-shaped) may be NULL; if
 * non-NULL it receives each ray's count.  *total (host) receives the sum; this
 * call synchronises the stream. */
ct_status_t ct_count_intersections(ct_geom_t g, uint32_t *per_ray, uint64_t *total,
                                   ct_stream_t stream);

/* Message of the most recent failing call on this thread ("" if none). */
const char *ct_last_error(void);

/* Library version string. */
const char *ct_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CTPROJ_H */
