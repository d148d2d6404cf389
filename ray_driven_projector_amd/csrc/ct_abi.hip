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
#include <mutex>
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
    double rays_bound = 0.0;            // brick adjoint: (ray, voxel) pairs a voxel can collect
    int yshift = 0;                     // brick adjoint: right shift of every term (range bound)
    float *d_vol_yf = nullptr;          // y-fastest volume copy read by some views' gathers
    float *d_vol_zf = nullptr;          // z-fastest volume copy read by some views' gathers
    bool need_yf = false, need_zf = false;  // some view reads that copy
    bool packet = false;                // every view has a packet axis (flat detector)
    size_t layout_cap = 0;              // voxels the copies hold (allocated on first use)
    double *d_off = nullptr;            // detector surface offsets (float64), or null: flat
    int surf_per_view = 0;
    float *d_env = nullptr;             // per-view footprint envelopes of the surface
    void *d_brick_rec = nullptr;        // brick adjoint: per-(brick, view) footprints and anchors of
                                        // the whole volume (read-only after creation), or null
    LineView *d_line = nullptr;         // separable tilt series: per-view line table (the adjoint
                                        // runs the line kernel), or null
    int line_shape = -1;                // its brick shape (kLineShapes)
};

namespace {

constexpr uint64_t kMagic = 0x43545052'4F4A3031ull;  // "CTPROJ01"

// Whole-volume calls address the volume and the sinogram as single buffers:
// fewer than 2^30 voxels (32-bit byte offsets in the gathers) and 2^31 rays.
// Larger lattices are reached through the region and host-streaming calls.
constexpr int64_t kMaxBufferVoxels = int64_t(1) << 30;
constexpr int64_t kMaxBufferRays = int64_t(1) << 31;
// The brick adjoint's record table (64 bytes per brick and view) is built at
// creation when it fits this budget and the detector sides fit 16 bits; else the
// kernel computes footprints and anchors itself.
constexpr size_t kMaxBrickRecordBytes = size_t(4) << 30;

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
    l.persp = g->host.beam == CT_FAN2D || g->host.beam == CT_CONE;
    l.yshift = g->yshift;
    l.vol_yf = g->d_vol_yf;
    l.vol_zf = g->d_vol_zf;
    l.need_yf = g->need_yf;
    l.need_zf = g->need_zf;
    l.packet = g->packet && !g->d_off;
    l.surf_off = g->d_off;
    l.surf_per_view = g->surf_per_view;
    l.surf_env = g->d_env;
    l.brick_rec = g->d_brick_rec;
    l.rec_stride = (int)g->host.n_views;
    l.rec_view0 = 0;
    l.line_tab = g->d_line;
    l.line_shape = g->line_shape;
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
    // the record table holds the whole volume's bricks: regions compute their own
    const bool whole = r.x0 == 0 && r.y0 == 0 && r.z0 == 0 && r.nx == g->host.W && r.ny == g->host.H &&
                       r.nz == g->host.D;
    if (whole) l.rec_view0 = (int)vb;
    else l.brick_rec = nullptr;
    if (g->d_line) l.line_tab = g->d_line + vb;
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
    if (r.nz * r.ny * r.nx >= kMaxBufferVoxels) return fail(CT_E_RANGE, "region has >= 2^30 voxels");
    if ((ve - vb) * h.U * h.V >= kMaxBufferRays) return fail(CT_E_RANGE, "view batch has >= 2^31 rays");
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

ct_status_t launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return hip_fail(e, what);
    set_error("");
    return CT_OK;
}

ct_status_t device_ok(ct_geom_t g) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != g->device) return fail(CT_E_ARG, "current HIP device differs from the handle's device");
    return CT_OK;
}

ct_status_t ensure_device(ct_geom_t g) {
    const GeomHost &h = g->host;
    if (h.D * h.H * h.W >= kMaxBufferVoxels)
        return fail(CT_E_RANGE, "whole-volume calls need fewer than 2^30 voxels; use regions");
    if (h.n_views * h.U * h.V >= kMaxBufferRays)
        return fail(CT_E_RANGE, "whole-sinogram calls need fewer than 2^31 rays; use view batches");
    return device_ok(g);
}

// The forward's volume copies in other axis orders, for a volume buffer of
// nvox voxels: allocated at the first forward call, grown when a later call
// needs more (hipFree waits for the device, so no queued launch still reads
// the old copies).
ct_status_t ensure_layouts(ct_geom_t g, size_t nvox) {
    if ((!g->need_yf && !g->need_zf) || nvox <= g->layout_cap) return CT_OK;
    if (g->d_vol_yf) (void)hipFree(g->d_vol_yf);
    if (g->d_vol_zf) (void)hipFree(g->d_vol_zf);
    g->d_vol_yf = g->d_vol_zf = nullptr;
    g->layout_cap = 0;
    const size_t bytes = nvox * sizeof(float);
    if ((g->need_yf && hipMalloc((void **)&g->d_vol_yf, bytes) != hipSuccess) ||
        (g->need_zf && hipMalloc((void **)&g->d_vol_zf, bytes) != hipSuccess)) {
        (void)hipGetLastError();
        if (g->d_vol_yf) (void)hipFree(g->d_vol_yf);
        g->d_vol_yf = nullptr;
        return fail(CT_E_NOMEM, "hipMalloc of a volume layout copy failed");
    }
    g->layout_cap = nvox;
    return CT_OK;
}

size_t full_voxels(ct_geom_t g) { return (size_t)g->host.D * g->host.H * g->host.W; }

// ---- host streaming: device staging, streams and events of one call ----
struct Staging {
    hipStream_t cs = nullptr, up = nullptr, down = nullptr;   // compute, host->device, device->host
    hipEvent_t h2d[2] = {}, used[2] = {}, done[2] = {}, d2h[2] = {};
    std::vector<void *> bufs;

    hipError_t init() {
        hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&up, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipStreamCreateWithFlags(&down, hipStreamNonBlocking);
        for (int i = 0; i < 2 && e == hipSuccess; ++i) {
            e = hipEventCreateWithFlags(&h2d[i], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&used[i], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&done[i], hipEventDisableTiming);
            if (e == hipSuccess) e = hipEventCreateWithFlags(&d2h[i], hipEventDisableTiming);
        }
        return e;
    }
    float *alloc(size_t n) {
        void *p = nullptr;
        if (hipMalloc(&p, n * sizeof(float)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        bufs.push_back(p);
        return (float *)p;
    }
    // every stream drained, then everything released
    hipError_t finish() {
        hipError_t e = hipSuccess, f;
        for (hipStream_t st : {cs, up, down})
            if (st && (f = hipStreamSynchronize(st)) != hipSuccess && e == hipSuccess) e = f;
        return e;
    }
    ~Staging() {
        (void)finish();
        for (void *p : bufs) (void)hipFree(p);
        for (int i = 0; i < 2; ++i)
            for (hipEvent_t ev : {h2d[i], used[i], done[i], d2h[i]})
                if (ev) (void)hipEventDestroy(ev);
        for (hipStream_t st : {cs, up, down})
            if (st) (void)hipStreamDestroy(st);
    }
};

// The slab axis the forward prefers: a slab face whose normal runs along the
// detector rows' direction e_v (e_u in 2D) is crossed by the rays of one wave
// at widely different points, which desynchronises the wave's gathers; so the
// forward slabs along z unless e_v leans mostly on z, else along whichever of
// y and x e_v leans on least.  The adjoint's bricks do not care: it slabs along
// z (contiguous host copies), or y for 2D.
int auto_axis(ct_geom_t g, bool forward) {
    const GeomHost &h = g->host;
    if (!forward) return h.is2d ? 1 : 0;
    double sc[3] = {0, 0, 0};   // mean |e . axis| for z, y, x
    for (int64_t k = 0; k < h.n_views; ++k) {
        const double *t = g->table.data() + (size_t)k * CT_VIEW_TABLE_STRIDE + (h.is2d ? VT_EU : VT_EV);
        const double ex = t[0] * h.sx, ey = t[1] * h.sy, ez = t[2] * h.sz;   // back to world units
        const double n = std::sqrt(ex * ex + ey * ey + ez * ez);
        if (n > 0) {
            sc[0] += std::fabs(ez) / n;
            sc[1] += std::fabs(ey) / n;
            sc[2] += std::fabs(ex) / n;
        }
    }
    for (double &v : sc) v /= (double)h.n_views;
    if (!h.is2d && sc[0] <= 0.5) return 0;
    return sc[2] < sc[1] ? 2 : 1;
}

// Validates a host-streaming call; returns the slab axis, thickness and batch size.
ct_status_t check_plan(ct_geom_t g, const void *vol, const void *sino, ct_stream_plan_t plan,
                       bool forward, int &axis, int64_t &ns, int64_t &nb) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!vol || !sino) return fail(CT_E_NULL, "vol and sino must be non-NULL");
    if (plan.slab < 1 || plan.batch_views < 1) return fail(CT_E_ARG, "plan sizes must be >= 1");
    if (plan.axis < -1 || plan.axis > 2 || plan.reserved != 0)
        return fail(CT_E_ARG, "plan axis must be -1, 0, 1 or 2 and reserved 0");
    const GeomHost &h = g->host;
    axis = plan.axis < 0 ? auto_axis(g, forward) : plan.axis;
    const int64_t ext[3] = {h.D, h.H, h.W};
    ns = std::min<int64_t>(plan.slab, ext[axis]);
    nb = std::min<int64_t>(plan.batch_views, h.n_views);
    const int64_t slab_vox = h.D * h.H * h.W / ext[axis] * ns;
    if (slab_vox >= kMaxBufferVoxels) return fail(CT_E_RANGE, "slab has >= 2^30 voxels");
    if (nb * h.U * h.V >= kMaxBufferRays) return fail(CT_E_RANGE, "view batch has >= 2^31 rays");
    ct_status_t st = check_alias({{Span{vol, vol_bytes(g)}, true}, {Span{sino, sino_bytes(g)}, true}});
    if (st != CT_OK) return st;
    return device_ok(g);
}

// Slab k of thickness ns along axis (0 = z, 1 = y, 2 = x), clipped to the volume.
ct_region_t slab_region(ct_geom_t g, int axis, int64_t k, int64_t ns) {
    const GeomHost &h = g->host;
    ct_region_t r{0, 0, 0, h.D, h.H, h.W};
    int64_t *lo = axis == 0 ? &r.z0 : (axis == 1 ? &r.y0 : &r.x0);
    int64_t *n = axis == 0 ? &r.nz : (axis == 1 ? &r.ny : &r.nx);
    *lo = k * ns;
    *n = std::min<int64_t>(ns, *n - *lo);
    return r;
}

// Copies a slab between the host volume (D, H, W) and its packed device buffer.
hipError_t copy_slab(ct_geom_t g, const ct_region_t &r, float *host_vol, float *dev, bool to_device,
                     hipStream_t s) {
    const size_t W = (size_t)g->host.W, H = (size_t)g->host.H;
    float *hp = host_vol + ((size_t)r.z0 * H + r.y0) * W + r.x0;
    const size_t f = sizeof(float);
    size_t width, rows, hpitch;
    if (r.ny == (int64_t)H && r.nx == (int64_t)W) {   // z slab: one contiguous block
        const size_t bytes = (size_t)r.nz * H * W * f;
        return to_device ? hipMemcpyAsync(dev, hp, bytes, hipMemcpyHostToDevice, s)
                         : hipMemcpyAsync(hp, dev, bytes, hipMemcpyDeviceToHost, s);
    }
    if (r.nx == (int64_t)W) {   // y slab: one row of ny*W per z plane
        width = (size_t)r.ny * W * f;
        rows = (size_t)r.nz;
        hpitch = H * W * f;
    } else {                    // x slab: one row of nx per (z, y)
        width = (size_t)r.nx * f;
        rows = (size_t)r.nz * r.ny;
        hpitch = W * f;
    }
    return to_device ? hipMemcpy2DAsync(dev, width, hp, hpitch, width, rows, hipMemcpyHostToDevice, s)
                     : hipMemcpy2DAsync(hp, hpitch, dev, width, width, rows, hipMemcpyDeviceToHost, s);
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

ct_status_t ct_geom_adjoint_range(ct_geom_t g, const ct_geom_desc_t *desc, int surface, double *rays_bound,
                                  int32_t *shift) {
    if (!rays_bound || !shift) return fail(CT_E_NULL, "output pointer is NULL");
    if (g) {
        if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
        *rays_bound = g->rays_bound;
        *shift = g->yshift;
        set_error("");
        return CT_OK;
    }
    GeomHost h;
    const char *why = "";
    ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return fail(st, why);
    std::vector<double> table;
    try {
        table.assign((size_t)h.n_views * CT_VIEW_TABLE_STRIDE, 0.0);
    } catch (...) {
        return fail(CT_E_NOMEM, "host allocation failed");
    }
    build_view_table(desc, h, table.data());
    *rays_bound = adjoint_rays_bound(h, table.data(), surface != 0);
    *shift = adjoint_term_shift(*rays_bound);
    set_error("");
    return CT_OK;
}

ct_status_t ct_geom_adjoint_kind(ct_geom_t g, const ct_geom_desc_t *desc, int surface, int32_t *kind) {
    if (!kind) return fail(CT_E_NULL, "output pointer is NULL");
    if (g) {
        if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
        *kind = g->d_line ? CT_ADJOINT_LINE : CT_ADJOINT_BRICK;
        set_error("");
        return CT_OK;
    }
    GeomHost h;
    const char *why = "";
    ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return fail(st, why);
    std::vector<double> table;
    std::vector<LineView> lines;
    try {
        table.assign((size_t)h.n_views * CT_VIEW_TABLE_STRIDE, 0.0);
        lines.resize((size_t)h.n_views);
    } catch (...) {
        return fail(CT_E_NOMEM, "host allocation failed");
    }
    build_view_table(desc, h, table.data());
    *kind = !surface && build_line_table(h, table.data(), lines.data()) >= 0 ? CT_ADJOINT_LINE : CT_ADJOINT_BRICK;
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
    if (g->d_brick_rec) (void)hipFree(g->d_brick_rec);
    if (g->d_line) (void)hipFree(g->d_line);
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
    g->rays_bound = adjoint_rays_bound(h, g->table.data(), offsets != nullptr);
    g->yshift = adjoint_term_shift(g->rays_bound);
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
    // volume copies in other axis orders, for the views whose gathers read them:
    // whole-volume size here when the volume fits one buffer, else allocated by
    // the first region forward at its region's size
    g->packet = !offsets;
    for (int64_t k = 0; k < h.n_views; ++k) {
        const double lay = g->table[(size_t)k * CT_VIEW_TABLE_STRIDE + VT_LAYOUT];
        g->need_yf = g->need_yf || lay == 1.0;
        g->need_zf = g->need_zf || lay == 2.0;
        g->packet = g->packet && g->table[(size_t)k * CT_VIEW_TABLE_STRIDE + VT_PACKET] >= 0.0;
    }
    if (h.D * h.H * h.W < kMaxBufferVoxels) {
        st = ensure_layouts(g, full_voxels(g));
        if (st != CT_OK) {
            free_handle(g);
            return st;
        }
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
    // a separable tilt series takes the line adjoint (per-view table, synchronous)
    if (!offsets) {
        std::vector<LineView> lines((size_t)h.n_views);
        g->line_shape = build_line_table(h, g->table.data(), lines.data());
        if (g->line_shape >= 0) {
            const size_t bytes = lines.size() * sizeof(LineView);
            if (hipMalloc((void **)&g->d_line, bytes) != hipSuccess) {
                (void)hipGetLastError();
                free_handle(g);
                return fail(CT_E_NOMEM, "hipMalloc of the line table failed");
            }
            e = hipMemcpy(g->d_line, lines.data(), bytes, hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                free_handle(g);
                return hip_fail(e, "hipMemcpy of the line table");
            }
        }
    }
    // the brick adjoint's record table (synchronous); without it the kernel
    // computes the same footprints and anchors itself
    if (!g->d_line && h.D * h.H * h.W < kMaxBufferVoxels && h.U < 65536 && h.V < 65536) {
        const LaunchGeom l = lg(g);
        const size_t bytes = brick_record_count(l) * brick_record_bytes();
        if (bytes <= kMaxBrickRecordBytes) {
            if (hipMalloc(&g->d_brick_rec, bytes) != hipSuccess) {
                (void)hipGetLastError();
                g->d_brick_rec = nullptr;   // the kernel computes them
            } else {
                e = launch_brick_records(l, g->d_brick_rec, nullptr);
                if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
                if (e != hipSuccess) {
                    free_handle(g);
                    return hip_fail(e, "brick record table");
                }
            }
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
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
    return launched(launch_project(lg(g), vol, sino, (hipStream_t)stream), "ct_project launch");
}

// Workspace of ct_project_ws: the y-fastest copy (if a view gathers from it)
// then the z-fastest one, each volume-sized and 256-byte aligned.
static size_t layout_copy_bytes(size_t nvox) { return (nvox * sizeof(float) + 255) & ~size_t(255); }

static size_t forward_workspace(bool yf, bool zf, size_t nvox) {
    return (size_t)(yf ? 1 : 0) * layout_copy_bytes(nvox) + (size_t)(zf ? 1 : 0) * layout_copy_bytes(nvox);
}

ct_status_t ct_forward_workspace_size(ct_geom_t g, const ct_geom_desc_t *desc, size_t *bytes) {
    if (!bytes) return fail(CT_E_NULL, "bytes must be non-NULL");
    if (g) {
        if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
        *bytes = forward_workspace(g->need_yf, g->need_zf, full_voxels(g));
        set_error("");
        return CT_OK;
    }
    GeomHost h;
    const char *why = "";
    ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return fail(st, why);
    std::vector<double> table;
    try {
        table.assign((size_t)h.n_views * CT_VIEW_TABLE_STRIDE, 0.0);
    } catch (...) {
        return fail(CT_E_NOMEM, "host allocation failed");
    }
    build_view_table(desc, h, table.data());
    bool yf = false, zf = false;
    for (int64_t k = 0; k < h.n_views; ++k) {
        const double lay = table[(size_t)k * CT_VIEW_TABLE_STRIDE + VT_LAYOUT];
        yf = yf || lay == 1.0;
        zf = zf || lay == 2.0;
    }
    *bytes = forward_workspace(yf, zf, (size_t)h.D * h.H * h.W);
    set_error("");
    return CT_OK;
}

ct_status_t ct_project_ws(ct_geom_t g, const float *vol, float *sino, void *work, size_t work_bytes,
                          ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!vol || !sino) return fail(CT_E_NULL, "vol and sino must be non-NULL");
    const size_t need = forward_workspace(g->need_yf, g->need_zf, full_voxels(g));
    if (need > 0 && !work) return fail(CT_E_NULL, "work must be non-NULL (ct_forward_workspace_size > 0)");
    if (work_bytes < need) return fail(CT_E_ARG, "work_bytes is below ct_forward_workspace_size");
    if (((uintptr_t)work & 255u) != 0) return fail(CT_E_ARG, "work must be 256-byte aligned");
    Span V{vol, vol_bytes(g)}, S{sino, sino_bytes(g)}, Wk{work, need};
    ct_status_t st = need > 0 ? check_alias({{V, false}, {S, true}, {Wk, true}})
                              : check_alias({{V, false}, {S, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    LaunchGeom l = lg(g);
    char *w = (char *)work;
    l.vol_yf = g->need_yf ? (float *)w : nullptr;
    l.vol_zf = g->need_zf ? (float *)(w + (g->need_yf ? layout_copy_bytes(full_voxels(g)) : 0)) : nullptr;
    return launched(launch_project(l, vol, sino, (hipStream_t)stream), "ct_project_ws launch");
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
    if ((st = device_ok(g)) != CT_OK) return st;
    if ((st = ensure_layouts(g, vb / sizeof(float))) != CT_OK) return st;
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
    if ((st = device_ok(g)) != CT_OK) return st;
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
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
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

// ---- ordered subsets (SART): the SIRT weights and step on a range of views ----

ct_status_t ct_sirt_weights_views(ct_geom_t g, int64_t view_begin, int64_t view_end, float *row_inv,
                                  float *col_inv, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    const GeomHost &h = g->host;
    const ct_region_t all{0, 0, 0, h.D, h.H, h.W};
    ct_status_t st = check_region(g, all, view_begin, view_end);
    if (st != CT_OK) return st;
    if (!row_inv || !col_inv) return fail(CT_E_NULL, "row_inv and col_inv must be non-NULL");
    const size_t sb = (size_t)(view_end - view_begin) * h.U * h.V * sizeof(float);
    st = check_alias({{Span{row_inv, sb}, true}, {Span{col_inv, vol_bytes(g)}, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    const LaunchGeom l = lg_region(g, all, view_begin, view_end, false);
    hipError_t e = launch_rowinv(l, row_inv, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ct_sirt_weights_views row launch");
    return launched(launch_colinv(l, col_inv, (hipStream_t)stream), "ct_sirt_weights_views column launch");
}

ct_status_t ct_sirt_step_views(ct_geom_t g, int64_t view_begin, int64_t view_end, float *x, const float *y,
                               const float *row_inv, const float *col_inv, float relax, float lo, float hi,
                               const uint8_t *mask, float *work, ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    const GeomHost &h = g->host;
    const ct_region_t all{0, 0, 0, h.D, h.H, h.W};
    ct_status_t st = check_region(g, all, view_begin, view_end);
    if (st != CT_OK) return st;
    if (!x || !y || !row_inv || !col_inv || !work) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (!std::isfinite(relax)) return fail(CT_E_ARG, "relax must be finite");
    if (std::isnan(lo) || std::isnan(hi) || !(lo <= hi)) return fail(CT_E_ARG, "bounds must satisfy lo <= hi");
    const size_t sb = (size_t)(view_end - view_begin) * h.U * h.V * sizeof(float);
    const size_t nvox = vol_bytes(g) / sizeof(float);
    Span X{x, vol_bytes(g)}, Y{y, sb}, R{row_inv, sb}, C{col_inv, vol_bytes(g)}, E{work, sb}, M{mask, nvox};
    st = check_alias({{X, true}, {Y, false}, {R, false}, {C, false}, {E, true}});
    if (st == CT_OK && mask) st = check_alias({{X, true}, {E, true}, {M, false}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
    const LaunchGeom l = lg_region(g, all, view_begin, view_end, false);
    hipError_t e = launch_residual(l, x, y, row_inv, work, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ct_sirt_step_views residual launch");
    return launched(launch_sirt_update_bounded(l, work, col_inv, relax, lo, hi, mask, x, (hipStream_t)stream),
                    "ct_sirt_step_views update launch");
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
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
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
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
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
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
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
    if ((st = ensure_layouts(g, full_voxels(g))) != CT_OK) return st;
    double *state = (double *)work;
    return launched(launch_cgls_step(lg(g), x, r, s, p, q, state, state + kCglsStateDoubles,
                                     (hipStream_t)stream),
                    "ct_cgls_step launch");
}

// ---- CGLS step without device allocation ----
// The per-block float64 partial sums of a CGLS step held in a fixed array of
// the library's own device memory, for callers that cannot allocate (graph
// capture, serving loops).  Each GPU the library runs on holds its own copy
// until the process ends; its address on a device comes from
// hipGetSymbolAddress on that device (the array's name is only a host-side
// stand-in).  Every partial a finalize reads is written by the launch before
// it, so nothing needs clearing between calls.
constexpr size_t kStaticPartials = size_t(1) << 22;   // 4 Mi doubles, 32 MiB per device
static __device__ __align__(256) double scratch[kStaticPartials];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on `device` (the current device).
ct_status_t static_scratch(int device, double **out) {
    if (device < 0 || device >= kMaxDevices) return fail(CT_E_RANGE, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the CGLS scratch");
        g_scratch_ptr[device] = (double *)ptr;
    }
    *out = g_scratch_ptr[device];
    return CT_OK;
}
}  // namespace

ct_status_t ct_cgls_step_noalloc(ct_geom_t g, float *x, float *r, float *s, float *p, float *q, double *state,
                                 ct_stream_t stream) {
    if (!valid(g)) return fail(CT_E_ARG, "invalid geometry handle");
    if (!x || !r || !s || !p || !q || !state) return fail(CT_E_NULL, "a buffer pointer is NULL");
    if (((uintptr_t)state & 7u) != 0) return fail(CT_E_ARG, "state must be 8-byte aligned");
    Span X{x, vol_bytes(g)}, R{r, sino_bytes(g)}, S{s, vol_bytes(g)}, P{p, vol_bytes(g)},
        Q{q, sino_bytes(g)}, St{state, kCglsStateDoubles * sizeof(double)};
    ct_status_t st = check_alias({{X, true}, {R, true}, {S, true}, {P, true}, {Q, true}, {St, true}});
    if (st != CT_OK) return st;
    if ((st = ensure_device(g)) != CT_OK) return st;
    const size_t need = cgls_partials(g);
    if (need > kStaticPartials)
        return fail(CT_E_RANGE, "geometry needs more CGLS partial sums than the 4 Mi-double static scratch "
                                "holds; use ct_cgls_step with a workspace");
    if ((g->need_yf || g->need_zf) && g->layout_cap < full_voxels(g))
        return fail(CT_E_RANGE, "the handle holds no whole-volume layout copies");
    double *partial = nullptr;
    if ((st = static_scratch(g->device, &partial)) != CT_OK) return st;
    return launched(launch_cgls_step(lg(g), x, r, s, p, q, state, partial, (hipStream_t)stream),
                    "ct_cgls_step_noalloc launch");
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

// ---- host-streaming A^T and A ----

// A^T: slabs outer, view batches inner.  Each slab accumulates the batches'
// adjoints on the device, then goes back to the host while the next slab runs.
// Batch k's upload waits for the kernel that last read its buffer (batch k-2);
// slab s's first kernel waits for the download of slab s-2.
ct_status_t ct_backproject_host(ct_geom_t g, const float *sino_host, float *vol_host,
                                ct_stream_plan_t plan, ct_stream_t stream) {
    int axis = 0;
    int64_t ns = 0, nb = 0;
    ct_status_t st = check_plan(g, vol_host, sino_host, plan, false, axis, ns, nb);
    if (st != CT_OK) return st;
    const GeomHost &h = g->host;
    const int64_t ext = axis == 0 ? h.D : (axis == 1 ? h.H : h.W);
    const int64_t n_slabs = (ext + ns - 1) / ns, n_batches = (h.n_views + nb - 1) / nb;
    const size_t ray_per_view = (size_t)h.U * h.V;
    const size_t slab_vox = (size_t)(h.D * h.H * h.W / ext) * ns;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);   // after the caller's queued work
    if (e != hipSuccess) return hip_fail(e, "ct_backproject_host: caller stream");
    Staging k;
    if ((e = k.init()) != hipSuccess) return hip_fail(e, "ct_backproject_host: streams");
    float *vbuf[2] = {k.alloc(slab_vox), n_slabs > 1 ? k.alloc(slab_vox) : nullptr};
    float *sbuf[2] = {k.alloc(nb * ray_per_view), n_batches > 1 ? k.alloc(nb * ray_per_view) : nullptr};
    if (!vbuf[0] || !sbuf[0] || (n_slabs > 1 && !vbuf[1]) || (n_batches > 1 && !sbuf[1]))
        return fail(CT_E_NOMEM, "ct_backproject_host: device staging allocation failed");
    auto ok = [&](hipError_t r) { if (e == hipSuccess) e = r; return e == hipSuccess; };
    if (n_batches == 1) {   // one batch: the sinogram is uploaded once and stays
        ok(hipMemcpyAsync(sbuf[0], sino_host, h.n_views * ray_per_view * sizeof(float),
                          hipMemcpyHostToDevice, k.up));
        ok(hipEventRecord(k.h2d[0], k.up));
        ok(hipStreamWaitEvent(k.cs, k.h2d[0], 0));
    }
    int64_t kb = 0;
    for (int64_t s = 0; s < n_slabs && e == hipSuccess; ++s) {
        const ct_region_t r = slab_region(g, axis, s, ns);
        const int vs = (int)(s & 1);
        if (s >= 2) ok(hipStreamWaitEvent(k.cs, k.d2h[vs], 0));
        for (int64_t b = 0; b < n_batches && e == hipSuccess; ++b, ++kb) {
            const int64_t vb = b * nb, ve = std::min<int64_t>(h.n_views, vb + nb);
            const int bs = n_batches == 1 ? 0 : (int)(kb & 1);
            if (n_batches > 1) {
                if (kb >= 2) ok(hipStreamWaitEvent(k.up, k.used[bs], 0));
                ok(hipMemcpyAsync(sbuf[bs], sino_host + vb * ray_per_view,
                                  (ve - vb) * ray_per_view * sizeof(float), hipMemcpyHostToDevice, k.up));
                ok(hipEventRecord(k.h2d[bs], k.up));
                ok(hipStreamWaitEvent(k.cs, k.h2d[bs], 0));
            }
            ok(launch_backproject(lg_region(g, r, vb, ve, b > 0), sbuf[bs], vbuf[vs], k.cs));
            if (n_batches > 1) ok(hipEventRecord(k.used[bs], k.cs));
        }
        ok(hipEventRecord(k.done[vs], k.cs));
        ok(hipStreamWaitEvent(k.down, k.done[vs], 0));
        ok(copy_slab(g, r, vol_host, vbuf[vs], false, k.down));
        ok(hipEventRecord(k.d2h[vs], k.down));
    }
    const hipError_t f = k.finish();
    if (e == hipSuccess) e = f;
    return launched(e, "ct_backproject_host");
}

// A: view batches outer, slabs inner.  Each batch accumulates the slabs'
// projections on the device, then goes back to the host.
ct_status_t ct_project_host(ct_geom_t g, const float *vol_host, float *sino_host, ct_stream_plan_t plan,
                            ct_stream_t stream) {
    int axis = 0;
    int64_t ns = 0, nb = 0;
    ct_status_t st = check_plan(g, vol_host, sino_host, plan, true, axis, ns, nb);
    if (st != CT_OK) return st;
    const GeomHost &h = g->host;
    const int64_t ext = axis == 0 ? h.D : (axis == 1 ? h.H : h.W);
    const int64_t n_slabs = (ext + ns - 1) / ns, n_batches = (h.n_views + nb - 1) / nb;
    const size_t ray_per_view = (size_t)h.U * h.V;
    const size_t slab_vox = (size_t)(h.D * h.H * h.W / ext) * ns;
    if ((st = ensure_layouts(g, slab_vox)) != CT_OK) return st;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "ct_project_host: caller stream");
    Staging k;
    if ((e = k.init()) != hipSuccess) return hip_fail(e, "ct_project_host: streams");
    float *vbuf[2] = {k.alloc(slab_vox), n_slabs > 1 ? k.alloc(slab_vox) : nullptr};
    float *sbuf[2] = {k.alloc(nb * ray_per_view), n_batches > 1 ? k.alloc(nb * ray_per_view) : nullptr};
    if (!vbuf[0] || !sbuf[0] || (n_slabs > 1 && !vbuf[1]) || (n_batches > 1 && !sbuf[1]))
        return fail(CT_E_NOMEM, "ct_project_host: device staging allocation failed");
    auto ok = [&](hipError_t r) { if (e == hipSuccess) e = r; return e == hipSuccess; };
    float *vol_src = const_cast<float *>(vol_host);   // only read: copies go host -> device
    if (n_slabs == 1) {   // one slab: the volume is uploaded once and stays
        ok(copy_slab(g, slab_region(g, axis, 0, ns), vol_src, vbuf[0], true, k.up));
        ok(hipEventRecord(k.h2d[0], k.up));
        ok(hipStreamWaitEvent(k.cs, k.h2d[0], 0));
    }
    int64_t ks = 0;
    for (int64_t b = 0; b < n_batches && e == hipSuccess; ++b) {
        const int64_t vb = b * nb, ve = std::min<int64_t>(h.n_views, vb + nb);
        const int bs = (int)(b & 1);
        if (b >= 2) ok(hipStreamWaitEvent(k.cs, k.d2h[bs], 0));
        for (int64_t s = 0; s < n_slabs && e == hipSuccess; ++s, ++ks) {
            const ct_region_t r = slab_region(g, axis, s, ns);
            const int vs = n_slabs == 1 ? 0 : (int)(ks & 1);
            if (n_slabs > 1) {
                if (ks >= 2) ok(hipStreamWaitEvent(k.up, k.used[vs], 0));
                ok(copy_slab(g, r, vol_src, vbuf[vs], true, k.up));
                ok(hipEventRecord(k.h2d[vs], k.up));
                ok(hipStreamWaitEvent(k.cs, k.h2d[vs], 0));
            }
            ok(launch_project(lg_region(g, r, vb, ve, s > 0), vbuf[vs], sbuf[bs], k.cs));
            if (n_slabs > 1) ok(hipEventRecord(k.used[vs], k.cs));
        }
        ok(hipEventRecord(k.done[bs], k.cs));
        ok(hipStreamWaitEvent(k.down, k.done[bs], 0));
        ok(hipMemcpyAsync(sino_host + vb * ray_per_view, sbuf[bs], (ve - vb) * ray_per_view * sizeof(float),
                          hipMemcpyDeviceToHost, k.down));
        ok(hipEventRecord(k.d2h[bs], k.down));
    }
    const hipError_t f = k.finish();
    if (e == hipSuccess) e = f;
    return launched(e, "ct_project_host");
}

}  // extern "C"
