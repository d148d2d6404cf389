/*
 * ct_oracle.c -- plain, slow, float64 reference of the Siddon projector pair.
 *
 * TEST INFRASTRUCTURE ONLY (see ct_oracle.h).  Written for readability: every
 * quantity is computed in physical coordinates exactly as the definitions
 * read, with no blocking, tiling or reordering beyond splitting work across
 * threads.
 *
 * Sources:
 *  - diffct documentation, "Trajectories and Geometry" > "Trajectory format":
 *    Cartesian (x, y[, z]) coordinates, volume indexed [z, y, x], origin at the
 *    volume centre, one length unit, flat-detector pixel centre
 *      det_center + (u - (U-1)/2) du det_u + (v - (V-1)/2) dv det_v,
 *    parallel3d rays are infinite lines through the pixels.
 *  - diffct documentation, "Differentiable analytical reconstruction": the
 *    projector is the cell-constant Siddon forward operator and its adjoint is
 *    the matched transpose.
 *  - diffct documentation, "Large Volumes and Chunked Execution" > "Resident
 *    layouts and accumulation": forward kernels overwrite every ray, missed
 *    rays included (a missed ray is 0).
 *  - Siddon's method: the ray's parameter interval inside the volume is cut at
 *    every lattice-plane crossing; each piece lies in one cell and contributes
 *    its length times that cell's value.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - fan/cone rays are the segment from the source to the pixel centre
 *    (parameter t in [0, 1]); parallel rays are infinite lines.
 *  - the 2D parallel "det_origin" is the detector centre.
 *  - 2D is 3D with one z slab of thickness dz = 1 centred on z = 0.
 *  - lengths are physical (voxel spacing applies), in the frames' unit.
 */
#include "ct_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* geometry                                                            */
/* ------------------------------------------------------------------ */

static int is_parallel(int beam) { return beam == ORA_PARALLEL2D || beam == ORA_PARALLEL3D; }

static void lattice(const ora_geom *g, int64_t n[3], double s[3], double lo[3], double hi[3])
{
    n[0] = g->nx; n[1] = g->ny; n[2] = g->nz;
    s[0] = g->sx; s[1] = g->sy; s[2] = g->sz;
    for (int a = 0; a < 3; ++a) {
        lo[a] = -0.5 * (double)n[a] * s[a];
        hi[a] = 0.5 * (double)n[a] * s[a];
    }
}

void ora_ray_of(const ora_geom *g, int64_t view, int64_t u, int64_t v, ora_ray *r)
{
    const double *f = g->frames + 12 * view;
    const double *a = f, *c = f + 3, *eu = f + 6, *ev = f + 9;
    int three_d = (g->beam == ORA_CONE || g->beam == ORA_PARALLEL3D);
    double p[3];
    if (g->offsets) {
        /* surface point: c + o_u e_u + o_v e_v + o_n n */
        const double *o = g->offsets + 3 * ((g->offsets_per_view ? view * g->nu * g->nv : 0)
                                            + u * g->nv + v);
        double n[3];
        if (three_d) {
            n[0] = eu[1] * ev[2] - eu[2] * ev[1];
            n[1] = eu[2] * ev[0] - eu[0] * ev[2];
            n[2] = eu[0] * ev[1] - eu[1] * ev[0];
        } else {
            n[0] = eu[1];
            n[1] = -eu[0];
            n[2] = 0.0;
        }
        for (int k = 0; k < 3; ++k)
            p[k] = c[k] + o[0] * eu[k] + (three_d ? o[1] * ev[k] : 0.0) + o[2] * n[k];
    } else {
        double ou = ((double)u - 0.5 * (double)(g->nu - 1)) * g->su;
        double ov = three_d ? ((double)v - 0.5 * (double)(g->nv - 1)) * g->sv : 0.0;
        for (int k = 0; k < 3; ++k)
            p[k] = c[k] + ou * eu[k] + (three_d ? ov * ev[k] : 0.0);
    }
    if (is_parallel(g->beam)) {
        for (int k = 0; k < 3; ++k) { r->o[k] = p[k]; r->d[k] = a[k]; }
        r->tmin = -INFINITY;
        r->tmax = INFINITY;
    } else {
        for (int k = 0; k < 3; ++k) { r->o[k] = a[k]; r->d[k] = p[k] - a[k]; }
        r->tmin = 0.0;
        r->tmax = 1.0;
    }
}

static double norm3(const double d[3]) { return sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]); }

/* Parameter interval of the ray inside the half-open box [lo, hi).
 * Returns 0 if the intersection is empty or has zero length. */
static int clip_box(const ora_ray *r, const double lo[3], const double hi[3],
                    double *tin, double *tout)
{
    double a = r->tmin, b = r->tmax;
    for (int k = 0; k < 3; ++k) {
        if (r->d[k] == 0.0) {
            /* parallel to the planes of this axis: inside iff lo <= o < hi */
            if (!(r->o[k] >= lo[k] && r->o[k] < hi[k])) return 0;
        } else {
            double t0 = (lo[k] - r->o[k]) / r->d[k];
            double t1 = (hi[k] - r->o[k]) / r->d[k];
            if (t0 > t1) { double tt = t0; t0 = t1; t1 = tt; }
            if (t0 > a) a = t0;
            if (t1 < b) b = t1;
        }
    }
    if (!(b > a)) return 0;
    *tin = a;
    *tout = b;
    return 1;
}

double ora_box_chord(const ora_ray *r, const double lo[3], const double hi[3])
{
    double a, b;
    if (!clip_box(r, lo, hi, &a, &b)) return 0.0;
    return (b - a) * norm3(r->d);
}

/* ------------------------------------------------------------------ */
/* forward: incremental traversal                                      */
/* ------------------------------------------------------------------ */

double ora_trace(const ora_geom *g, const ora_ray *r, const double *vol,
                 int64_t *nnz, int64_t *ties)
{
    int64_t n[3];
    double s[3], lo[3], hi[3];
    lattice(g, n, s, lo, hi);
    double tin, tout;
    int64_t local_nnz = 0, local_ties = 0;

    /* a ray lying exactly in a lattice plane is a tie event */
    for (int k = 0; k < 3; ++k) {
        if (r->d[k] == 0.0) {
            double q = (r->o[k] - lo[k]) / s[k];
            if (q == floor(q) && q >= 0 && q <= (double)n[k]) local_ties++;
        }
    }
    if (!clip_box(r, lo, hi, &tin, &tout)) {
        if (ties) *ties += local_ties;
        return 0.0;
    }
    double L = norm3(r->d);

    /* first cell: the one holding the points just after t_in */
    int64_t i[3], step[3];
    double next[3];
    for (int k = 0; k < 3; ++k) {
        double q = (r->o[k] + tin * r->d[k] - lo[k]) / s[k];
        int64_t c;
        if (r->d[k] > 0)      { c = (int64_t)floor(q); step[k] = 1; }
        else if (r->d[k] < 0) { c = (int64_t)ceil(q) - 1; step[k] = -1; }
        else                  { c = (int64_t)floor(q); step[k] = 0; }
        if (c < 0) c = 0;
        if (c > n[k] - 1) c = n[k] - 1;
        i[k] = c;
        /* parameter of the next plane crossed along this axis */
        if (r->d[k] > 0)      next[k] = (lo[k] + (double)(c + 1) * s[k] - r->o[k]) / r->d[k];
        else if (r->d[k] < 0) next[k] = (lo[k] + (double)c * s[k] - r->o[k]) / r->d[k];
        else                  next[k] = INFINITY;
    }

    double sum = 0.0, t = tin;
    for (;;) {
        double tn = tout;
        for (int k = 0; k < 3; ++k) if (next[k] < tn) tn = next[k];
        double len = (tn - t) * L;
        if (len > 0.0) {
            sum += len * vol[(i[2] * n[1] + i[1]) * n[0] + i[0]];
            local_nnz++;
        }
        if (tn >= tout) break;
        int crossing = 0;
        for (int k = 0; k < 3; ++k) if (next[k] == tn) crossing++;
        if (crossing > 1) local_ties++;
        int left = 0;
        for (int k = 0; k < 3; ++k) {
            if (next[k] == tn) {
                i[k] += step[k];
                if (i[k] < 0 || i[k] >= n[k]) { left = 1; break; }
                if (step[k] > 0) next[k] = (lo[k] + (double)(i[k] + 1) * s[k] - r->o[k]) / r->d[k];
                else             next[k] = (lo[k] + (double)i[k] * s[k] - r->o[k]) / r->d[k];
            }
        }
        if (left) break;
        t = tn;
    }
    if (nnz) *nnz += local_nnz;
    if (ties) *ties += local_ties;
    return sum;
}

/* ------------------------------------------------------------------ */
/* threading helper                                                     */
/* ------------------------------------------------------------------ */

typedef struct {
    void (*fn)(void *ctx, int64_t begin, int64_t end, int tid);
    void *ctx;
    int64_t begin, end;
    int tid;
} job_t;

static void *job_main(void *p)
{
    job_t *j = (job_t *)p;
    j->fn(j->ctx, j->begin, j->end, j->tid);
    return NULL;
}

static int clamp_threads(int nthreads, int64_t count)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (count < nthreads) nthreads = (int)(count > 0 ? count : 1);
    return nthreads;
}

/* Split [0, count) into contiguous ranges, one per thread. */
static void run_parallel(int nthreads, int64_t count,
                         void (*fn)(void *, int64_t, int64_t, int), void *ctx)
{
    nthreads = clamp_threads(nthreads, count);
    pthread_t th[256];
    job_t jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = count * t / nthreads;
        jobs[t].end = count * (t + 1) / nthreads;
        jobs[t].tid = t;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, job_main, &jobs[t]);
    job_main(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* whole projection                                                     */
/* ------------------------------------------------------------------ */

typedef struct {
    const ora_geom *g;
    const double *vol;
    double *sino;
    const int64_t *ids;
    int64_t *nnz_per;
    int64_t nnz[256], ties[256];
} proj_ctx;

static void proj_views(void *p, int64_t v0, int64_t v1, int tid)
{
    proj_ctx *c = (proj_ctx *)p;
    const ora_geom *g = c->g;
    int64_t nnz = 0, ties = 0;
    for (int64_t view = v0; view < v1; ++view)
        for (int64_t u = 0; u < g->nu; ++u)
            for (int64_t v = 0; v < g->nv; ++v) {
                ora_ray r;
                ora_ray_of(g, view, u, v, &r);
                c->sino[(view * g->nu + u) * g->nv + v] = ora_trace(g, &r, c->vol, &nnz, &ties);
            }
    c->nnz[tid] = nnz;
    c->ties[tid] = ties;
}

int ora_project(const ora_geom *g, const double *vol, double *sino, int nthreads,
                int64_t *nnz_total, int64_t *ties_total)
{
    proj_ctx c;
    memset(&c, 0, sizeof c);
    c.g = g; c.vol = vol; c.sino = sino;
    run_parallel(nthreads, g->n_views, proj_views, &c);
    int64_t nnz = 0, ties = 0;
    for (int t = 0; t < 256; ++t) { nnz += c.nnz[t]; ties += c.ties[t]; }
    if (nnz_total) *nnz_total = nnz;
    if (ties_total) *ties_total = ties;
    return 0;
}

static void proj_rays(void *p, int64_t b, int64_t e, int tid)
{
    proj_ctx *c = (proj_ctx *)p;
    const ora_geom *g = c->g;
    (void)tid;
    for (int64_t k = b; k < e; ++k) {
        int64_t id = c->ids[k];
        int64_t v = id % g->nv;
        int64_t u = (id / g->nv) % g->nu;
        int64_t view = id / (g->nv * g->nu);
        ora_ray r;
        ora_ray_of(g, view, u, v, &r);
        int64_t nnz = 0;
        c->sino[k] = ora_trace(g, &r, c->vol, &nnz, NULL);
        if (c->nnz_per) c->nnz_per[k] = nnz;
    }
}

int ora_project_rays(const ora_geom *g, const double *vol, const int64_t *ray_ids,
                     int64_t n, double *out, int64_t *nnz_per_ray, int nthreads)
{
    proj_ctx c;
    memset(&c, 0, sizeof c);
    c.g = g; c.vol = vol; c.sino = out; c.ids = ray_ids; c.nnz_per = nnz_per_ray;
    run_parallel(nthreads, n, proj_rays, &c);
    return 0;
}

typedef struct {
    const ora_geom *g;
    double *out;
} chord_ctx;

static void chord_views(void *p, int64_t v0, int64_t v1, int tid)
{
    chord_ctx *c = (chord_ctx *)p;
    const ora_geom *g = c->g;
    int64_t n[3];
    double s[3], lo[3], hi[3];
    (void)tid;
    lattice(g, n, s, lo, hi);
    for (int64_t view = v0; view < v1; ++view)
        for (int64_t u = 0; u < g->nu; ++u)
            for (int64_t v = 0; v < g->nv; ++v) {
                ora_ray r;
                ora_ray_of(g, view, u, v, &r);
                c->out[(view * g->nu + u) * g->nv + v] = ora_box_chord(&r, lo, hi);
            }
}

int ora_row_chords(const ora_geom *g, double *out, int nthreads)
{
    chord_ctx c;
    c.g = g; c.out = out;
    run_parallel(nthreads, g->n_views, chord_views, &c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* adjoint: merged plane-crossing lists (Siddon's alpha sets)           */
/* ------------------------------------------------------------------ */

/* Append to buf the parameters of every plane of axis k crossed strictly
 * inside (ta, tb), in increasing order. */
static int64_t axis_crossings(const ora_ray *r, int k, double lo, double s, int64_t n,
                              double ta, double tb, double *buf)
{
    if (r->d[k] == 0.0) return 0;
    double qa = (r->o[k] + ta * r->d[k] - lo) / s;
    double qb = (r->o[k] + tb * r->d[k] - lo) / s;
    double qmin = qa < qb ? qa : qb, qmax = qa < qb ? qb : qa;
    int64_t k0 = (int64_t)floor(qmin) - 1, k1 = (int64_t)ceil(qmax) + 1;
    if (k0 < 0) k0 = 0;
    if (k1 > n) k1 = n;
    int64_t m = 0;
    if (r->d[k] > 0) {
        for (int64_t p = k0; p <= k1; ++p) {
            double t = (lo + (double)p * s - r->o[k]) / r->d[k];
            if (t > ta && t < tb) buf[m++] = t;
        }
    } else {
        for (int64_t p = k1; p >= k0; --p) {
            double t = (lo + (double)p * s - r->o[k]) / r->d[k];
            if (t > ta && t < tb) buf[m++] = t;
        }
    }
    return m;
}

typedef struct {
    const ora_geom *g;
    const double *sino;
    double *vol;
    int slab_axis;           /* 2 = z slabs, 1 = y slabs */
    int64_t slab_n;
    int nthreads;
} bp_ctx;

static void bp_slabs(void *p, int64_t s0, int64_t s1, int tid)
{
    bp_ctx *c = (bp_ctx *)p;
    const ora_geom *g = c->g;
    (void)tid;
    int64_t n[3];
    double s[3], lo[3], hi[3];
    lattice(g, n, s, lo, hi);
    int ax = c->slab_axis;
    /* the thread owns cells with index along ax in [s0, s1) */
    double slab_lo[3], slab_hi[3];
    for (int k = 0; k < 3; ++k) { slab_lo[k] = lo[k]; slab_hi[k] = hi[k]; }
    slab_lo[ax] = lo[ax] + (double)s0 * s[ax];
    slab_hi[ax] = lo[ax] + (double)s1 * s[ax];

    int64_t cap = n[0] + n[1] + n[2] + 16;
    double *lists[3];
    for (int k = 0; k < 3; ++k) lists[k] = (double *)malloc(sizeof(double) * (size_t)cap);
    double *merged = (double *)malloc(sizeof(double) * (size_t)(3 * cap + 2));

    for (int64_t view = 0; view < g->n_views; ++view)
        for (int64_t u = 0; u < g->nu; ++u)
            for (int64_t v = 0; v < g->nv; ++v) {
                double y = c->sino[(view * g->nu + u) * g->nv + v];
                if (y == 0.0) continue;
                ora_ray r;
                ora_ray_of(g, view, u, v, &r);
                double ta, tb;
                if (!clip_box(&r, slab_lo, slab_hi, &ta, &tb)) continue;
                double L = norm3(r.d);
                int64_t m[3];
                for (int k = 0; k < 3; ++k)
                    m[k] = axis_crossings(&r, k, lo[k], s[k], n[k], ta, tb, lists[k]);
                /* merge the three sorted lists between the end points */
                int64_t nm = 0, p0 = 0, p1 = 0, p2 = 0;
                merged[nm++] = ta;
                while (p0 < m[0] || p1 < m[1] || p2 < m[2]) {
                    double best = INFINITY;
                    int which = -1;
                    if (p0 < m[0] && lists[0][p0] < best) { best = lists[0][p0]; which = 0; }
                    if (p1 < m[1] && lists[1][p1] < best) { best = lists[1][p1]; which = 1; }
                    if (p2 < m[2] && lists[2][p2] < best) { best = lists[2][p2]; which = 2; }
                    if (which == 0) p0++; else if (which == 1) p1++; else p2++;
                    merged[nm++] = best;
                }
                merged[nm++] = tb;
                for (int64_t q = 0; q + 1 < nm; ++q) {
                    double gap = merged[q + 1] - merged[q];
                    if (!(gap > 0.0)) continue;
                    double tm = 0.5 * (merged[q] + merged[q + 1]);
                    int64_t cell[3];
                    for (int k = 0; k < 3; ++k) {
                        int64_t ck = (int64_t)floor((r.o[k] + tm * r.d[k] - lo[k]) / s[k]);
                        int64_t lo_c = (k == ax) ? s0 : 0, hi_c = (k == ax) ? s1 - 1 : n[k] - 1;
                        if (ck < lo_c) ck = lo_c;
                        if (ck > hi_c) ck = hi_c;
                        cell[k] = ck;
                    }
                    c->vol[(cell[2] * n[1] + cell[1]) * n[0] + cell[0]] += gap * L * y;
                }
            }
    for (int k = 0; k < 3; ++k) free(lists[k]);
    free(merged);
}

int ora_backproject(const ora_geom *g, const double *sino, double *vol, int nthreads)
{
    int64_t nvox = g->nx * g->ny * g->nz;
    memset(vol, 0, sizeof(double) * (size_t)nvox);
    bp_ctx c;
    c.g = g; c.sino = sino; c.vol = vol;
    c.slab_axis = g->nz > 1 ? 2 : 1;
    c.slab_n = g->nz > 1 ? g->nz : g->ny;
    c.nthreads = nthreads;
    run_parallel(nthreads, c.slab_n, bp_slabs, &c);
    return 0;
}

/* ------------------------------------------------------------------ */
/* brute force: every (ray, cell) pair                                  */
/* ------------------------------------------------------------------ */

static void cell_box(const ora_geom *g, int64_t j, double blo[3], double bhi[3])
{
    int64_t n[3];
    double s[3], lo[3], hi[3];
    lattice(g, n, s, lo, hi);
    int64_t ix = j % n[0], iy = (j / n[0]) % n[1], iz = j / (n[0] * n[1]);
    int64_t idx[3] = {ix, iy, iz};
    for (int k = 0; k < 3; ++k) {
        blo[k] = lo[k] + (double)idx[k] * s[k];
        bhi[k] = lo[k] + (double)(idx[k] + 1) * s[k];
    }
}

int ora_brute_matrix(const ora_geom *g, double *A)
{
    int64_t nvox = g->nx * g->ny * g->nz;
    int64_t i = 0;
    for (int64_t view = 0; view < g->n_views; ++view)
        for (int64_t u = 0; u < g->nu; ++u)
            for (int64_t v = 0; v < g->nv; ++v, ++i) {
                ora_ray r;
                ora_ray_of(g, view, u, v, &r);
                for (int64_t j = 0; j < nvox; ++j) {
                    double blo[3], bhi[3];
                    cell_box(g, j, blo, bhi);
                    A[i * nvox + j] = ora_box_chord(&r, blo, bhi);
                }
            }
    return 0;
}

typedef struct {
    const ora_geom *g;
    const double *sino;
    double blo[3], bhi[3];
    double part[256];
} col_ctx;

static void col_views(void *p, int64_t v0, int64_t v1, int tid)
{
    col_ctx *c = (col_ctx *)p;
    const ora_geom *g = c->g;
    double acc = 0.0;
    for (int64_t view = v0; view < v1; ++view)
        for (int64_t u = 0; u < g->nu; ++u)
            for (int64_t v = 0; v < g->nv; ++v) {
                double y = c->sino[(view * g->nu + u) * g->nv + v];
                if (y == 0.0) continue;
                ora_ray r;
                ora_ray_of(g, view, u, v, &r);
                acc += ora_box_chord(&r, c->blo, c->bhi) * y;
            }
    c->part[tid] = acc;
}

double ora_column_dot(const ora_geom *g, int64_t j, const double *sino, int nthreads)
{
    col_ctx c;
    memset(&c, 0, sizeof c);
    c.g = g; c.sino = sino;
    cell_box(g, j, c.blo, c.bhi);
    run_parallel(nthreads, g->n_views, col_views, &c);
    double s = 0.0;
    for (int t = 0; t < 256; ++t) s += c.part[t];
    return s;
}
