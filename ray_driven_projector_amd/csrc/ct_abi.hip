// ct_abi.hip -- the extern "C" entry points declared in include/ctproj.h.
//
// Each call validates its arguments on the host (null pointers, handle,
// overlapping buffers) before anything is enqueued, then launches on the
// caller's stream.  Buffer aliasing is rejected as the diffct Projector class
// reference describes for project_into ("Known overlapping/read-only outputs
// are rejected before execution").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "ct_internal.h"
#include "ct_launch.h"

namespace ctp {

namespace {
thread_local char g_err[512] = "";
}

void set_error(const char *msg) {
    std::snprintf(g_err, sizeof g_err, "%s", msg ? msg : "");
}

}  // namespace ctp

using namespace ctp;

struct ct_geom_s {
    uint64_t magic;
    GeomHost host;
    std::vector<double> table;          // host copy of the view table
    double *d_views = nullptr;          // device view table
    unsigned long long *d_total = nullptr;  // device counter for ct_count_intersections
    int device = 0;
    int brick_shape = 5;                // adjoint bricks of 16 x 16 x 32
    int fwd_order = 5;                  // forward block order: 2 x 2 tile groups, views inside
    float *d_vol_yf = nullptr;          // y-fastest volume copy read by some views' gathers
    float *d_vol_zf = nullptr;          // z-fastest volume copy read by some views' gathers
    double *d_off = nullptr;            // detector surface offsets (float64), or null: flat
    int surf_per_view = 0;
    float *d_env = nullptr;             // per-view footprint envelopes of the surface
};

namespace {

constexpr uint64_t kMagic = 0x43545052'4F4A3031ull;  // "CTPROJ01"

ct_status_t fail(ct_status_t st, const char *msg) {
    set_error(msg);
    return st;
}

ct_status_t hip_fail(hipError_t e, const char *where) {
    char buf[400];
    std::snprintf(buf, sizeof buf, "%s: %s", where, hipGetErrorString(e));
    set_error(buf);
    return CT_E_HIP;
}

bool valid(ct_geom_t g) { return g && g->magic == kMagic; }

LaunchGeom lg(ct_geom_t g) {
    LaunchGeom l{};
    l.views = g->d_views;
    l.W = (int)g->host.W;
    l.H = (int)g->host.H;
    l.D = (int)g->host.D;
    l.U = (int)g->host.U;
    l.V = (int)g->host.V;
    l.n_views = (int)g->host.n_views;
    l.spx = g->host.sx;
    l.spy = g->host.sy;
    l.spz = g->host.sz;
    l.two_d = g->host.is2d;
    l.brick_shape = g->brick_shape;
    l.fwd_order = g->fwd_order;
    l.vol_yf = g->d_vol_yf;
    l.vol_zf = g->d_vol_zf;
    l.surf_off = g->d_off;
    l.surf_per_view = g->surf_per_view;
    l.surf_env = g->d_env;
    return l;
}

// Launch geometry for a region of the volume and a batch of views: the buffer
// holds the region only, the sinogram buffer the batch only.
LaunchGeom lg_region(ct_geom_t g, const ct_region_t &r, int64_t vb, int64_t ve, bool accumulate) {
    LaunchGeom l = lg(g);
    l.W = (int)r.nx;
    l.H = (int)r.ny;
    l.D = (int)r.nz;
    l.offx = (int)r.x0;
    l.offy = (int)r.y0;
    l.offz = (int)r.z0;
    l.accumulate = accumulate ? 1 : 0;
    l.views = g->d_views + (size_t)vb * CT_VIEW_TABLE_STRIDE;
    l.n_views = (int)(ve - vb);
    if (g->d_off && g->surf_per_view) l.surf_off = g->d_off + (size_t)vb * g->host.U * g->host.V * 3;
    if (g->d_env) l.surf_env = g->d_env + (size_t)vb * surface_env_floats((int)g->host.U, (int)g->host.V);
    return l;
}

ct_status_t check_region(ct_geom_t g, const ct_region_t &r, int64_t vb, int64_t ve) {
    const GeomHost &h = g->host;
    if (r.nz < 1 || r.ny < 1 || r.nx < 1 || r.z0 < 0 || r.y0 < 0 || r.x0 < 0 || r.z0 + r.nz > h.D ||
        r.y0 + r.ny > h.H || r.x0 + r.nx > h.W)
        return fail(CT_E_SHAPE, "region is empty or not inside the volume");
    if (vb < 0 || ve > h.n_views || vb >= ve) return fail(CT_E_SHAPE, "view range is empty or out of range");
    return CT_OK;
}

size_t vol_bytes(ct_geom_t g) { return (size_t)g->host.D * g->host.H * g->host.W * sizeof(float); }
size_t sino_bytes(ct_geom_t g) {
    return (size_t)g->host.n_views * g->host.U * g->host.V * sizeof(float);
}

struct Span {
    const void *p;
    size_t n;
};
bool overlap(Span a, Span b) {
    const char *a0 = (const char *)a.p, *b0 = (const char *)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

struct Arg {
    Span span;
    bool output;
};

// Every output must overlap no other buffer of the call (inputs may share memory).
ct_status_t check_alias(std::initializer_list<Arg> args) {
    const Arg *v = args.begin();
    const size_t n = args.size();
    for (size_t i = 0; i < n; ++i)
        for (size_t j = i + 1; j < n; ++j)
            if ((v[i].output || v[j].output) && overlap(v[i].span, v[j].span))
                return fail(CT_E_ALIAS, "an output buffer overlaps another buffer of the call");
    return CT_OK;
}

// Launch shapes.  CTPROJ_BRICK (0..6) overrides the adjoint brick shape,
// CTPROJ_FWD_ORDER (0..7) the forward block order, and
// CTPROJ_FWD_LAYOUT=x keeps every forward gather on the caller's x-fastest volume;
// both only change the work decomposition (used for tuning comparisons).
// Defaults measured on 512^3 cone and parallel3d workloads: 16 x 16 x 32 bricks,
// forward order 5 (groups of 2 x 2 pixel tiles, every view of a group in turn).
void choose_tiles(ct_geom_s *g) {
    g->brick_shape = 5;
    if (const char *e = std::getenv("CTPROJ_BRICK")) {
        const int v = std::atoi(e);
        if (v >= 0 && v <= 6) g->brick_shape = v;
    }
    g->fwd_order = 5;
    if (const char *e = std::getenv("CTPROJ_FWD_ORDER")) {
        const int v = std::atoi(e);
        if (v >= 0 && v <= 7) g->fwd_order = v;
    }
    const char *lay = std::getenv("CTPROJ_FWD_LAYOUT");
    if (lay && lay[0] == 'x') {
        for (int64_t k = 0; k < g->host.n_views; ++k) {
            double *t = g->table.data() + k * CT_VIEW_TABLE_STRIDE;
            const double su[3] = {t[VT_OU] + t[VT_DU], t[VT_OU + 1] + t[VT_DU + 1], t[VT_OU + 2] + t[VT_DU + 2]};
            const double sv[3] = {t[VT_OV] + t[VT_DV], t[VT_OV + 1] + t[VT_DV + 1], t[VT_OV + 2] + t[VT_DV + 2]};
            const double nu = std::sqrt(su[0] * su[0] + su[1] * su[1] + su[2] * su[2]);
            const double nv = std::sqrt(sv[0] * sv[0] + sv[1] * sv[1] + sv[2] * sv[2]);
            const double au = nu > 0 ? std::fabs(su[0]) / nu : 0.0, av = nv > 0 ? std::fabs(sv[0]) / nv : 0.0;
            t[VT_LAYOUT] = 0.0;
            t[VT_PATCH] = (g->host.is2d || au >= av) ? 0.0 : 1.0;
        }
    }
}

ct_status_t launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return hip_fail(e, what);
    set_error("");
    return CT_OK;
}

ct_status_t ensure_device(ct_geom_t g) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != g->device) return fail(CT_E_ARG, "current HIP device differs from the handle's device");
    return CT_OK;
}

}  // namespace

extern "C" {

const char *ct_last_error(void) { return g_err; }

const char *ct_version(void) { return "ctproj 0.1 gfx950"; }

ct_status_t ct_geom_validate(const ct_geom_desc_t *desc) {
    const char *why = "";
    ct_status_t st = validate_desc(desc, nullptr, &why);
    if (st != CT_OK) return fail(st, why);
    set_error("");
    return CT_OK;
}

ct_status_t ct_geom_view_table(ct_geom_t g, const ct_geom_desc_t *desc, double *out) {
    if (!out) return fail(CT_E_NULL, "output pointer is NULL");
    if (g) {
        if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
        std::memcpy(out, g->table.data(), g->table.size() * sizeof(double));
        set_error("");
        return CT_OK;
    }
    GeomHost h;
    const char *why = "";
    ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return fail(st, why);
    build_view_table(desc, h, out);
    set_error("");
    return CT_OK;
}

static void free_handle(ct_geom_s *g) {
    if (g->d_views) (void)hipFree(g->d_views);
    if (g->d_total) (void)hipFree(g->d_total);
    if (g->d_vol_yf) (void)hipFree(g->d_vol_yf);
    if (g->d_vol_zf) (void)hipFree(g->d_vol_zf);
    if (g->d_off) (void)hipFree(g->d_off);
    if (g->d_env) (void)hipFree(g->d_env);
    delete g;
}

static ct_status_t create_impl(const ct_geom_desc_t *desc, const double *offsets, int per_view,
                               ct_geom_t *out) {
    if (!out) return fail(CT_E_NULL, "output handle pointer is NULL");
    *out = nullptr;
    GeomHost h;
    const char *why = "";
    ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return fail(st, why);
    const size_t n_off = offsets ? (size_t)(per_view ? h.n_views : 1) * h.U * h.V * 3 : 0;
    for (size_t i = 0; i < n_off; ++i) {
        if (!std::isfinite(offsets[i])) return fail(CT_E_NONFINITE, "surface offset not finite");
        if (h.is2d && i % 3 == 1 && offsets[i] != 0.0)
            return fail(CT_E_ARG, "2D surface offsets need o_v = 0");
    }
    ct_geom_s *g = new (std::nothrow) ct_geom_s();
    if (!g) return fail(CT_E_NOMEM, "host allocation failed");
    g->magic = kMagic;
    g->host = h;
    try {
        g->table.assign((size_t)h.n_views * CT_VIEW_TABLE_STRIDE, 0.0);
    } catch (...) {
        delete g;
        return fail(CT_E_NOMEM, "host allocation failed");
    }
    build_view_table(desc, h, g->table.data());
    choose_tiles(g);
    hipError_t e = hipGetDevice(&g->device);
    if (e != hipSuccess) {
        delete g;
        return hip_fail(e, "hipGetDevice");
    }
    size_t nb = g->table.size() * sizeof(double);
    e = hipMalloc((void **)&g->d_views, nb);
    if (e != hipSuccess) {
        delete g;
        (void)hipGetLastError();
        return fail(CT_E_NOMEM, "hipMalloc of the view table failed");
    }
    e = hipMalloc((void **)&g->d_total, sizeof(unsigned long long));
    if (e != hipSuccess) {
        (void)hipFree(g->d_views);
        delete g;
        (void)hipGetLastError();
        return fail(CT_E_NOMEM, "hipMalloc of the counter failed");
    }
    e = hipMemcpy(g->d_views, g->table.data(), nb, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(g->d_views);
        (void)hipFree(g->d_total);
        delete g;
        return hip_fail(e, "hipMemcpy of the view table");
    }
    // volume copies in other axis orders, for the views whose gathers read them
    bool need_y = false, need_z = false;
    for (int64_t k = 0; k < h.n_views; ++k) {
        const double lay = g->table[(size_t)k * CT_VIEW_TABLE_STRIDE + VT_LAYOUT];
        need_y = need_y || lay == 1.0;
        need_z = need_z || lay == 2.0;
    }
    const size_t vbytes = (size_t)h.D * h.H * h.W * sizeof(float);
    if ((need_y && hipMalloc((void **)&g->d_vol_yf, vbytes) != hipSuccess) ||
        (need_z && hipMalloc((void **)&g->d_vol_zf, vbytes) != hipSuccess)) {
        (void)hipGetLastError();
        free_handle(g);
        return fail(CT_E_NOMEM, "hipMalloc of a volume layout copy failed");
    }
    if (offsets) {
        // surface offsets, then the per-view footprint envelopes (synchronous)
        g->surf_per_view = per_view ? 1 : 0;
        const size_t env_bytes =
            (size_t)h.n_views * surface_env_floats((int)h.U, (int)h.V) * sizeof(float);
        if (hipMalloc((void **)&g->d_off, n_off * sizeof(double)) != hipSuccess ||
            hipMalloc((void **)&g->d_env, env_bytes) != hipSuccess) {
            (void)hipGetLastError();
            free_handle(g);
            return fail(CT_E_NOMEM, "hipMalloc of the detector surface failed");
        }
        e = hipMemcpy(g->d_off, offsets, n_off * sizeof(double), hipMemcpyHostToDevice);
        if (e == hipSuccess) e = launch_surface_env(lg(g), g->d_total, nullptr);
        unsigned long long bad = 0;
        if (e == hipSuccess) e = hipMemcpy(&bad, g->d_total, sizeof bad, hipMemcpyDeviceToHost);
        if (e != hipSuccess) {
            free_handle(g);
            return hip_fail(e, "detector surface set-up");
        }
        if (bad) {
            free_handle(g);
            return fail(CT_E_FRAME, "a surface pixel is not in front of the source");
        }
    }
    *out = g;
    set_error("");
    return CT_OK;
}

ct_status_t ct_geom_create(const ct_geom_desc_t *desc, ct_geom_t *out) {
    return create_impl(desc, nullptr, 0, out);
}

ct_status_t ct_geom_create_surface(const ct_geom_desc_t *desc, const double *offsets, int per_view,
                                   ct_geom_t *out) {
    if (!offsets) return fail(CT_E_NULL, "offsets must be non-NULL");
    return create_impl(desc, offsets, per_view, out);
}

ct_status_t ct_geom_destroy(ct_geom_t g) {
    if (!g) return CT_OK;
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    g->magic = 0;
    free_handle(g);
    set_error("");
    return CT_OK;
}

ct_status_t ct_project(ct_geom_t g, const float *vol, float *sino, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!vol || !sino) return fail(CT_E_NULL, "vol and sino must be non-NULL");
    Span V{vol, vol_bytes(g)}, S{sino, sino_bytes(g)};
    ct_status_t st = check_alias({{V, false}, {S, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_project(lg(g), vol, sino, (hipStream_t)stream), "ct_project launch");
}

ct_status_t ct_backproject(ct_geom_t g, const float *sino, float *vol, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!vol || !sino) return fail(CT_E_NULL, "vol and sino must be non-NULL");
    Span V{vol, vol_bytes(g)}, S{sino, sino_bytes(g)};
    ct_status_t st = check_alias({{V, true}, {S, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_backproject(lg(g), sino, vol, (hipStream_t)stream), "ct_backproject launch");
}

ct_status_t ct_project_region(ct_geom_t g, const float *vol_region, ct_region_t region,
                              int64_t view_begin, int64_t view_end, float *sino_batch, int accumulate,
                              ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    ct_status_t st = check_region(g, region, view_begin, view_end);
    if (st != CT_OK) return st;
    if (!vol_region || !sino_batch) return fail(CT_E_NULL, "buffers must be non-NULL");
    const size_t vb = (size_t)region.nz * region.ny * region.nx * sizeof(float);
    const size_t sb = (size_t)(view_end - view_begin) * g->host.U * g->host.V * sizeof(float);
    st = check_alias({{Span{vol_region, vb}, false}, {Span{sino_batch, sb}, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_project(lg_region(g, region, view_begin, view_end, accumulate != 0),
                                   vol_region, sino_batch, (hipStream_t)stream),
                    "ct_project_region launch");
}

ct_status_t ct_backproject_region(ct_geom_t g, const float *sino_batch, int64_t view_begin,
                                  int64_t view_end, ct_region_t region, float *vol_region,
                                  int accumulate, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    ct_status_t st = check_region(g, region, view_begin, view_end);
    if (st != CT_OK) return st;
    if (!vol_region || !sino_batch) return fail(CT_E_NULL, "buffers must be non-NULL");
    const size_t vb = (size_t)region.nz * region.ny * region.nx * sizeof(float);
    const size_t sb = (size_t)(view_end - view_begin) * g->host.U * g->host.V * sizeof(float);
    st = check_alias({{Span{vol_region, vb}, true}, {Span{sino_batch, sb}, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_backproject(lg_region(g, region, view_begin, view_end, accumulate != 0),
                                       sino_batch, vol_region, (hipStream_t)stream),
                    "ct_backproject_region launch");
}

ct_status_t ct_backproject_atomic(ct_geom_t g, const float *sino, float *vol, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!vol || !sino) return fail(CT_E_NULL, "vol and sino must be non-NULL");
    Span V{vol, vol_bytes(g)}, S{sino, sino_bytes(g)};
    ct_status_t st = check_alias({{V, true}, {S, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_backproject_atomic(lg(g), sino, vol, (hipStream_t)stream),
                    "ct_backproject_atomic launch");
}

ct_status_t ct_sirt_weights(ct_geom_t g, float *row_inv, float *col_inv, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!row_inv || !col_inv) return fail(CT_E_NULL, "row_inv and col_inv must be non-NULL");
    Span R{row_inv, sino_bytes(g)}, C{col_inv, vol_bytes(g)};
    ct_status_t st = check_alias({{R, true}, {C, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    hipError_t e = launch_rowinv(lg(g), row_inv, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ct_sirt_weights row launch");
    return launched(launch_colinv(lg(g), col_inv, (hipStream_t)stream), "ct_sirt_weights column launch");
}

ct_status_t ct_sirt_residual(ct_geom_t g, const float *x, const float *y, const float *row_inv,
                             float *work_sino, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !y || !row_inv || !work_sino) return fail(CT_E_NULL, "a buffer pointer is NULL");
    Span X{x, vol_bytes(g)}, Y{y, sino_bytes(g)}, R{row_inv, sino_bytes(g)}, E{work_sino, sino_bytes(g)};
    ct_status_t st = check_alias({{X, false}, {Y, false}, {R, false}, {E, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_residual(lg(g), x, y, row_inv, work_sino, (hipStream_t)stream),
                    "ct_sirt_residual launch");
}

ct_status_t ct_sirt_update(ct_geom_t g, const float *work_sino, const float *col_inv, float relax,
                           float *x, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !work_sino || !col_inv) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (!std::isfinite(relax)) return fail(CT_E_ARG, "relax must be finite");
    Span X{x, vol_bytes(g)}, E{work_sino, sino_bytes(g)}, C{col_inv, vol_bytes(g)};
    ct_status_t st = check_alias({{X, true}, {E, false}, {C, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_sirt_update(lg(g), work_sino, col_inv, relax, x, (hipStream_t)stream),
                    "ct_sirt_update launch");
}

ct_status_t ct_sirt_update_bounded(ct_geom_t g, const float *work_sino, const float *col_inv,
                                  float relax, float lo, float hi, const uint8_t *mask, float *x,
                                  ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !work_sino || !col_inv) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (!std::isfinite(relax)) return fail(CT_E_ARG, "relax must be finite");
    if (std::isnan(lo) || std::isnan(hi) || !(lo <= hi)) return fail(CT_E_ARG, "bounds must satisfy lo <= hi");
    const size_t nvox = vol_bytes(g) / sizeof(float);
    Span X{x, vol_bytes(g)}, E{work_sino, sino_bytes(g)}, C{col_inv, vol_bytes(g)}, M{mask, nvox};
    ct_status_t st = check_alias({{X, true}, {E, false}, {C, false}});
    if (st == CT_OK && mask) st = check_alias({{X, true}, {M, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    return launched(launch_sirt_update_bounded(lg(g), work_sino, col_inv, relax, lo, hi, mask, x,
                                               (hipStream_t)stream),
                    "ct_sirt_update_bounded launch");
}

ct_status_t ct_sirt_step_bounded(ct_geom_t g, float *x, const float *y, const float *row_inv,
                                 const float *col_inv, float relax, float lo, float hi,
                                 const uint8_t *mask, float *work_sino, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !y || !row_inv || !col_inv || !work_sino) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (!std::isfinite(relax)) return fail(CT_E_ARG, "relax must be finite");
    if (std::isnan(lo) || std::isnan(hi) || !(lo <= hi)) return fail(CT_E_ARG, "bounds must satisfy lo <= hi");
    const size_t nvox = vol_bytes(g) / sizeof(float);
    Span X{x, vol_bytes(g)}, Y{y, sino_bytes(g)}, R{row_inv, sino_bytes(g)}, C{col_inv, vol_bytes(g)},
        E{work_sino, sino_bytes(g)};
    Span M{mask, nvox};
    ct_status_t st = check_alias({{X, true}, {Y, false}, {R, false}, {C, false}, {E, true}});
    if (st == CT_OK && mask) st = check_alias({{X, true}, {E, true}, {M, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    hipError_t e = launch_residual(lg(g), x, y, row_inv, work_sino, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ct_sirt_step_bounded residual launch");
    return launched(launch_sirt_update_bounded(lg(g), work_sino, col_inv, relax, lo, hi, mask, x,
                                               (hipStream_t)stream),
                    "ct_sirt_step_bounded update launch");
}

ct_status_t ct_sirt_step(ct_geom_t g, float *x, const float *y, const float *row_inv,
                         const float *col_inv, float relax, float *work_sino, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !y || !row_inv || !col_inv || !work_sino) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (!std::isfinite(relax)) return fail(CT_E_ARG, "relax must be finite");
    Span X{x, vol_bytes(g)}, Y{y, sino_bytes(g)}, R{row_inv, sino_bytes(g)}, C{col_inv, vol_bytes(g)},
        E{work_sino, sino_bytes(g)};
    ct_status_t st = check_alias({{X, true}, {Y, false}, {R, false}, {C, false}, {E, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    hipError_t e = launch_residual(lg(g), x, y, row_inv, work_sino, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ct_sirt_step residual launch");
    return launched(launch_sirt_update(lg(g), work_sino, col_inv, relax, x, (hipStream_t)stream),
                    "ct_sirt_step update launch");
}

// ---- CGLS ----

static size_t cgls_partials(ct_geom_t g) {
    const LaunchGeom l = lg(g);
    size_t n = cgls_ray_blocks(l);
    n = std::max(n, cgls_brick_blocks(l));
    n = std::max(n, (size_t)kCglsVecBlocks);
    return n;
}

ct_status_t ct_cgls_workspace_size(ct_geom_t g, size_t *bytes) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!bytes) return fail(CT_E_NULL, "bytes must be non-NULL");
    *bytes = sizeof(double) * (kCglsStateDoubles + cgls_partials(g));
    set_error("");
    return CT_OK;
}

ct_status_t ct_cgls_init(ct_geom_t g, const float *y, const float *x, float *r, float *s, float *p,
                         void *work, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!y || !x || !r || !s || !p || !work) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (((uintptr_t)work & 7u) != 0) return fail(CT_E_ARG, "work must be 8-byte aligned");
    size_t wb = 0;
    ct_cgls_workspace_size(g, &wb);
    Span Y{y, sino_bytes(g)}, X{x, vol_bytes(g)}, R{r, sino_bytes(g)}, S{s, vol_bytes(g)},
        P{p, vol_bytes(g)}, Wk{work, wb};
    ct_status_t st = check_alias({{Y, false}, {X, false}, {R, true}, {S, true}, {P, true}, {Wk, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    double *state = (double *)work;
    return launched(launch_cgls_init(lg(g), y, x, r, s, p, state, state + kCglsStateDoubles,
                                     (hipStream_t)stream),
                    "ct_cgls_init launch");
}

ct_status_t ct_cgls_step(ct_geom_t g, float *x, float *r, float *s, float *p, float *q, void *work,
                         ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !r || !s || !p || !q || !work) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (((uintptr_t)work & 7u) != 0) return fail(CT_E_ARG, "work must be 8-byte aligned");
    size_t wb = 0;
    ct_cgls_workspace_size(g, &wb);
    Span X{x, vol_bytes(g)}, R{r, sino_bytes(g)}, S{s, vol_bytes(g)}, P{p, vol_bytes(g)},
        Q{q, sino_bytes(g)}, Wk{work, wb};
    ct_status_t st = check_alias({{X, true}, {R, true}, {S, true}, {P, true}, {Q, true}, {Wk, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    double *state = (double *)work;
    return launched(launch_cgls_step(lg(g), x, r, s, p, q, state, state + kCglsStateDoubles,
                                     (hipStream_t)stream),
                    "ct_cgls_step launch");
}

ct_status_t ct_cgls_scalars(ct_geom_t g, const void *work, double *out, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!work || !out) return fail(CT_E_NULL, "work and out must be non-NULL");
    ct_status_t st = ensure_device(g);
    if (st != CT_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    double host[kCglsStateDoubles];
    hipError_t e = hipMemcpyAsync(host, work, sizeof host, hipMemcpyDeviceToHost, hs);
    if (e != hipSuccess) return hip_fail(e, "ct_cgls_scalars copy");
    e = hipStreamSynchronize(hs);
    if (e != hipSuccess) return hip_fail(e, "ct_cgls_scalars sync");
    out[0] = host[CS_GAMMA];
    out[1] = host[CS_ALPHA];
    out[2] = host[CS_BETA];
    out[3] = host[CS_QQ];
    out[4] = host[CS_RR];
    set_error("");
    return CT_OK;
}

ct_status_t ct_count_intersections(ct_geom_t g, uint32_t *per_ray, uint64_t *total, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!total) return fail(CT_E_NULL, "total must be non-NULL");
    ct_status_t st = ensure_device(g);
    if (st != CT_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_count(lg(g), per_ray, g->d_total, s);
    if (e != hipSuccess) return hip_fail(e, "ct_count_intersections launch");
    unsigned long long host = 0;
    e = hipMemcpyAsync(&host, g->d_total, sizeof host, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "ct_count_intersections copy");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "ct_count_intersections sync");
    *total = (uint64_t)host;
    set_error("");
    return CT_OK;
}

}  // extern "C"
