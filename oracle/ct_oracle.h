/*
 * ct_oracle.h -- float64 CPU reference for the ray-driven projector pair.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the oracle that the HIP library is checked
 * against.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load it.  It shares no code, header, table or helper with the
 * HIP library and must never be used on the product path.
 *
 * What it computes (diffct documentation, "Differentiable analytical
 * reconstruction": the projector is the cell-constant Siddon forward operator
 * with a matched adjoint; "Trajectories and Geometry" > "Parameterized detector
 * surfaces": one ray per pixel, no detector-area integration):
 *
 *   a_ij = length of (ray_i  intersected with  cell_j)
 *   (A x)_i  = sum_j a_ij x_j        (line integral of the cell-constant volume)
 *   (A^T y)_j = sum_i a_ij y_i       (the literal transpose)
 *
 * Cells are half-open boxes [lo + k s, lo + (k+1) s) of the lattice centred on
 * the origin, so a ray lying exactly on a lattice plane belongs to the cell on
 * the higher-index side and zero-length touches contribute nothing.
 */
#ifndef CT_ORACLE_H
#define CT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORA_PARALLEL2D = 0, ORA_FAN2D = 1, ORA_CONE = 2, ORA_PARALLEL3D = 3 };

typedef struct {
    int beam;
    int64_t n_views;
    int64_t nz, ny, nx;      /* volume (D, H, W); 2D: nz = 1 */
    double sz, sy, sx;       /* voxel spacing (dz, dy, dx); 2D: sz = 1 */
    int64_t nu, nv;          /* detector (U, V); 2D: nv = 1 */
    double su, sv;           /* detector spacing (du, dv) */
    const double *frames;    /* n_views x 12: a(3) c(3) e_u(3) e_v(3), x,y,z order */
    /* Parameterized detector surface (NULL: flat detector).  Per pixel the local
     * offsets (o_u, o_v, o_n), shape (U, V, 3), or (views, U, V, 3) when
     * offsets_per_view != 0; the pixel's world point is
     *   c + o_u e_u + o_v e_v + o_n n,  n = e_u x e_v (3D), (e_u_y, -e_u_x, 0) (2D)
     * (diffct documentation, "Trajectories and Geometry" > "Parameterized
     * detector surfaces"). */
    const double *offsets;
    int offsets_per_view;
} ora_geom;

typedef struct {
    double o[3];             /* origin (x, y, z) */
    double d[3];             /* direction */
    double tmin, tmax;       /* parameter range of the ray */
} ora_ray;

/* Ray through pixel (u, v) of a view: flat-detector pixel-centre formula, or
 * the surface point of the pixel when the geometry has surface offsets. */
void ora_ray_of(const ora_geom *g, int64_t view, int64_t u, int64_t v, ora_ray *r);

/* Length of the ray inside the half-open box [lo, hi) (slab method). */
double ora_box_chord(const ora_ray *r, const double lo[3], const double hi[3]);

/* Forward value of one ray by incremental cell traversal; optional nnz/tie counts. */
double ora_trace(const ora_geom *g, const ora_ray *r, const double *vol,
                 int64_t *nnz, int64_t *ties);

/* Whole forward projection: sino[(view * nu + u) * nv + v]. Returns 0. */
int ora_project(const ora_geom *g, const double *vol, double *sino, int nthreads,
                int64_t *nnz_total, int64_t *ties_total);

/* Forward values of selected rays (flat ray ids); optional per-ray nnz. */
int ora_project_rays(const ora_geom *g, const double *vol, const int64_t *ray_ids,
                     int64_t n, double *out, int64_t *nnz_per_ray, int nthreads);

/* Adjoint by Siddon's merged plane-crossing lists (coded separately from
 * ora_trace).  vol is overwritten.  Rays with y_i == 0 add nothing and are
 * skipped. */
int ora_backproject(const ora_geom *g, const double *sino, double *vol, int nthreads);

/* Row sums of A in closed form: for every ray, the length of its chord through
 * the whole volume box (slab method), out[(view * nu + u) * nv + v].  Equals
 * A 1 up to rounding, without walking the cells.  Returns 0. */
int ora_row_chords(const ora_geom *g, double *out, int nthreads);

/* Dense matrix A (n_rays x n_voxels) by per-cell chords: tiny grids only. */
int ora_brute_matrix(const ora_geom *g, double *A);

/* (A^T y)_j for one voxel j by per-cell chords over every ray. */
double ora_column_dot(const ora_geom *g, int64_t j, const double *sino, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
