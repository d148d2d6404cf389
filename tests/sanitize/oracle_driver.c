/*
 * Sanitizer driver for the float64 oracle (oracle/ct_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py.
 * Exercises every oracle entry point on small geometries of all four beams,
 * including a detector surface, rays that miss, rays along lattice planes and
 * a cone source inside the volume, and checks two identities so a silently
 * wrong build also fails: the adjoint identity <A x, y> = <x, A^T y> and the
 * brute-force matrix against the traversal.  Exit status 0 means clean.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ct_oracle.h"

static unsigned long long rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

/* frames for n views: fan/cone sources on a circle (radius sid) with the
 * detector opposite (at sdd), parallel rays tilted out of the xy plane */
static void make_frames(int beam, int n, double sid, double sdd, double *fr)
{
    for (int k = 0; k < n; ++k) {
        double th = 6.283185307179586 * k / n + 0.1, c = cos(th), s = sin(th);
        double *f = fr + 12 * k;
        memset(f, 0, 12 * sizeof(double));
        if (beam == ORA_FAN2D || beam == ORA_CONE) {
            f[0] = sid * c; f[1] = sid * s; f[2] = beam == ORA_CONE ? 0.3 : 0.0;
            f[3] = -(sdd - sid) * c; f[4] = -(sdd - sid) * s;
        } else {
            double tilt = beam == ORA_PARALLEL3D ? 0.2 : 0.0;
            f[0] = -c * cos(tilt); f[1] = -s * cos(tilt); f[2] = sin(tilt);
        }
        f[6] = s; f[7] = -c; f[8] = 0.0;                         /* e_u */
        if (beam == ORA_CONE || beam == ORA_PARALLEL3D) {         /* e_v = n x e_u */
            if (beam == ORA_PARALLEL3D) {
                double a[3] = {f[0], f[1], f[2]};
                f[9] = a[1] * f[8] - a[2] * f[7];
                f[10] = a[2] * f[6] - a[0] * f[8];
                f[11] = a[0] * f[7] - a[1] * f[6];
                double nv = sqrt(f[9] * f[9] + f[10] * f[10] + f[11] * f[11]);
                f[9] /= nv; f[10] /= nv; f[11] /= nv;
            } else {
                f[11] = 1.0;
            }
        }
    }
}

static int check(int beam, int nz, int ny, int nx, int nu, int nv, int views, double sid, double sdd,
                 int surface)
{
    ora_geom g;
    memset(&g, 0, sizeof g);
    g.beam = beam; g.n_views = views;
    g.nz = nz; g.ny = ny; g.nx = nx;
    g.sz = 1.0; g.sy = 0.9; g.sx = 1.1;
    g.nu = nu; g.nv = nv; g.su = 0.8; g.sv = 0.7;
    double *fr = malloc(sizeof(double) * 12 * views);
    make_frames(beam, views, sid, sdd, fr);
    g.frames = fr;
    double *off = NULL;
    if (surface) {
        off = malloc(sizeof(double) * 3 * nu * nv);
        for (int u = 0; u < nu; ++u)
            for (int v = 0; v < nv; ++v) {
                double *o = off + 3 * (u * nv + v);
                o[0] = (u - 0.5 * (nu - 1)) * g.su;
                o[1] = (beam == ORA_CONE || beam == ORA_PARALLEL3D) ? (v - 0.5 * (nv - 1)) * g.sv : 0.0;
                o[2] = -0.01 * o[0] * o[0];
            }
        g.offsets = off;
    }
    const long nvox = (long)nz * ny * nx, nray = (long)views * nu * nv;
    double *x = malloc(sizeof(double) * nvox), *y = malloc(sizeof(double) * nray);
    double *ax = malloc(sizeof(double) * nray), *aty = malloc(sizeof(double) * nvox);
    double *rc = malloc(sizeof(double) * nray), *A = malloc(sizeof(double) * nray * nvox);
    for (long j = 0; j < nvox; ++j) x[j] = urand();
    for (long i = 0; i < nray; ++i) y[i] = urand() < 0.1 ? 0.0 : urand();
    int64_t nnz = 0, ties = 0;
    ora_project(&g, x, ax, 3, &nnz, &ties);
    ora_backproject(&g, y, aty, 3);
    ora_row_chords(&g, rc, 2);
    ora_brute_matrix(&g, A);
    double lhs = 0.0, rhs = 0.0;
    for (long i = 0; i < nray; ++i) lhs += ax[i] * y[i];
    for (long j = 0; j < nvox; ++j) rhs += x[j] * aty[j];
    int bad = fabs(lhs - rhs) > 1e-12 * fabs(lhs);
    long brute_nnz = 0;
    for (long i = 0; i < nray; ++i) {
        double s = 0.0, row = 0.0;
        for (long j = 0; j < nvox; ++j) {
            s += A[i * nvox + j] * x[j];
            row += A[i * nvox + j];
            brute_nnz += A[i * nvox + j] > 0.0;
        }
        if (fabs(s - ax[i]) > 1e-11 * (1.0 + fabs(s)) || fabs(row - rc[i]) > 1e-11 * (1.0 + row)) bad = 1;
    }
    if (ties == 0 && brute_nnz != nnz) bad = 1;
    int64_t ids[7] = {0, nray - 1, nray / 2, nray / 3, 1, nray / 5, nray / 7};
    double sel[7];
    int64_t cnt[7];
    ora_project_rays(&g, x, ids, 7, sel, cnt, 2);
    for (int k = 0; k < 7; ++k)
        if (sel[k] != ax[ids[k]]) bad = 1;
    double cd = ora_column_dot(&g, nvox / 2, y, 2);
    if (fabs(cd - aty[nvox / 2]) > 1e-11 * (1.0 + fabs(cd))) bad = 1;
    ora_ray r;
    ora_ray_of(&g, views - 1, nu - 1, nv - 1, &r);
    ora_trace(&g, &r, x, NULL, NULL);
    printf("beam %d %dx%dx%d det %dx%d views %d surface %d: nnz %lld ties %lld identity %.2e %s\n", beam, nz,
           ny, nx, nu, nv, views, surface, (long long)nnz, (long long)ties, fabs(lhs - rhs) / fabs(lhs),
           bad ? "FAIL" : "ok");
    free(fr); free(off); free(x); free(y); free(ax); free(aty); free(rc); free(A);
    return bad;
}

int main(void)
{
    int bad = 0;
    bad |= check(ORA_PARALLEL2D, 1, 9, 11, 17, 1, 6, 0, 0, 0);
    bad |= check(ORA_FAN2D, 1, 10, 8, 19, 1, 7, 25.0, 40.0, 0);
    bad |= check(ORA_FAN2D, 1, 10, 8, 19, 1, 5, 25.0, 40.0, 1);
    bad |= check(ORA_CONE, 5, 6, 7, 13, 9, 5, 20.0, 35.0, 0);
    bad |= check(ORA_CONE, 5, 6, 7, 13, 9, 4, 20.0, 35.0, 1);
    bad |= check(ORA_CONE, 6, 6, 6, 11, 9, 4, 1.5, 30.0, 0);     /* source inside the volume */
    bad |= check(ORA_PARALLEL3D, 5, 6, 7, 12, 10, 6, 0, 0, 0);
    bad |= check(ORA_PARALLEL3D, 4, 4, 4, 8, 8, 2, 0, 0, 1);
    return bad;
}
