// ct_geometry.cpp -- host-side frame validation and per-view ray tables.
//
// Validation rules: diffct documentation, "Trajectories and Geometry" >
// "Custom acquisition example" (finite frames with a common nonzero view count;
// ray_dir orthogonal to det_u for 2D parallel beams, det_u orthogonal to det_v
// for 3D beams; parallel3d rays must not be tangent to the detector plane;
// fan/cone sources must not coincide with the detector centre nor view the
// detector edge-on; the nearer of source and detector centre within 1e6 voxel
// spacings of the origin, both endpoints within 1e15) and the Projector class
// reference ("Direction axes are unit vectors").  The pages give no numeric
// tolerances; 1e-6 is used for unit length, orthogonality and tangency.
//
// Pixel centres: "Trajectories and Geometry" > "Trajectory format",
//   det_center + (u - (U-1)/2) du det_u + (v - (V-1)/2) dv det_v.
#include <cmath>
#include <cstring>

#include "ct_internal.h"

namespace ctp {

namespace {

struct V3 {
    double x, y, z;
};
inline V3 v3(const double *p) { return {p[0], p[1], p[2]}; }
inline V3 operator+(V3 a, V3 b) { return {a.x + b.x, a.y + b.y, a.z + b.z}; }
inline V3 operator-(V3 a, V3 b) { return {a.x - b.x, a.y - b.y, a.z - b.z}; }
inline V3 operator*(double s, V3 a) { return {s * a.x, s * a.y, s * a.z}; }
inline double dot(V3 a, V3 b) { return a.x * b.x + a.y * b.y + a.z * b.z; }
inline double norm(V3 a) { return std::sqrt(dot(a, a)); }
inline V3 cross(V3 a, V3 b) { return {a.y * b.z - a.z * b.y, a.z * b.x - a.x * b.z, a.x * b.y - a.y * b.x}; }

constexpr double kTolUnit = 1e-6;
constexpr double kTolOrtho = 1e-6;
constexpr double kTolTangent = 1e-6;

// Detector normal: 3D e_u x e_v, 2D the in-plane normal (e_u.y, -e_u.x, 0).
V3 detector_normal(bool is2d, V3 eu, V3 ev) {
    if (is2d) return {eu.y, -eu.x, 0.0};
    return cross(eu, ev);
}

bool finite_all(const double *p, int n) {
    for (int i = 0; i < n; ++i)
        if (!std::isfinite(p[i])) return false;
    return true;
}

}  // namespace

ct_status_t validate_desc(const ct_geom_desc_t *desc, GeomHost *out, const char **why) {
    static const char *none = "";
    *why = none;
    if (!desc) { *why = "descriptor is NULL"; return CT_E_NULL; }
    if (!desc->frames) { *why = "frames pointer is NULL"; return CT_E_NULL; }
    if (desc->beam < 0 || desc->beam > 3) { *why = "unknown beam type"; return CT_E_ARG; }
    if (desc->reserved != 0) { *why = "reserved field must be 0"; return CT_E_ARG; }
    GeomHost g;
    g.beam = desc->beam;
    g.is2d = (desc->beam == CT_PARALLEL2D || desc->beam == CT_FAN2D);
    g.n_views = desc->n_views;
    g.D = desc->vol_shape[0];
    g.H = desc->vol_shape[1];
    g.W = desc->vol_shape[2];
    g.U = desc->det_shape[0];
    g.V = desc->det_shape[1];
    if (g.n_views < 1) { *why = "n_views must be >= 1"; return CT_E_SHAPE; }
    if (g.D < 1 || g.H < 1 || g.W < 1) { *why = "volume extents must be >= 1"; return CT_E_SHAPE; }
    if (g.U < 1 || g.V < 1) { *why = "detector extents must be >= 1"; return CT_E_SHAPE; }
    if (g.is2d && (g.D != 1 || g.V != 1)) { *why = "2D beams need D = 1 and V = 1"; return CT_E_SHAPE; }
    const int64_t lim = int64_t(1) << 20;
    if (g.D >= lim || g.H >= lim || g.W >= lim || g.U >= lim || g.V >= lim || g.n_views >= lim) {
        *why = "an extent is >= 2^20";
        return CT_E_RANGE;
    }

    for (int k = 0; k < 3; ++k)
        if (!std::isfinite(desc->voxel_spacing[k])) { *why = "voxel spacing not finite"; return CT_E_NONFINITE; }
    for (int k = 0; k < 2; ++k)
        if (!std::isfinite(desc->det_spacing[k])) { *why = "detector spacing not finite"; return CT_E_NONFINITE; }
    g.sz = g.is2d ? 1.0 : desc->voxel_spacing[0];
    g.sy = desc->voxel_spacing[1];
    g.sx = desc->voxel_spacing[2];
    g.du = desc->det_spacing[0];
    g.dv = g.is2d ? 1.0 : desc->det_spacing[1];
    if (!(g.sz > 0 && g.sy > 0 && g.sx > 0)) { *why = "voxel spacing must be > 0"; return CT_E_ARG; }
    if (!(g.du > 0 && g.dv > 0)) { *why = "detector spacing must be > 0"; return CT_E_ARG; }
    {
        // keep per-voxel step lengths representable in float32
        const double smax = std::fmax(g.sx, std::fmax(g.sy, g.sz));
        const double smn = std::fmin(g.sx, std::fmin(g.sy, g.sz));
        if (smn < 1e-10 || smax > 1e10 || smax > 1e6 * smn) {
            *why = "voxel spacings must lie in [1e-10, 1e10] within a ratio of 1e6";
            return CT_E_RANGE;
        }
    }

    const double smin = std::fmin(g.sx, std::fmin(g.sy, g.is2d ? g.sy : g.sz));
    const bool parallel = (g.beam == CT_PARALLEL2D || g.beam == CT_PARALLEL3D);
    for (int64_t k = 0; k < g.n_views; ++k) {
        const double *f = desc->frames + 12 * k;
        if (!finite_all(f, g.is2d ? 9 : 12)) { *why = "frame value not finite"; return CT_E_NONFINITE; }
        V3 a = v3(f), c = v3(f + 3), eu = v3(f + 6), ev = g.is2d ? V3{0, 0, 0} : v3(f + 9);
        if (g.is2d && (a.z != 0.0 || c.z != 0.0 || eu.z != 0.0)) {
            *why = "2D frames must have zero z components";
            return CT_E_FRAME;
        }
        if (std::fabs(norm(eu) - 1.0) > kTolUnit) { *why = "det_u is not a unit vector"; return CT_E_FRAME; }
        if (!g.is2d) {
            if (std::fabs(norm(ev) - 1.0) > kTolUnit) { *why = "det_v is not a unit vector"; return CT_E_FRAME; }
            if (std::fabs(dot(eu, ev)) > kTolOrtho) { *why = "det_u and det_v are not orthogonal"; return CT_E_FRAME; }
        }
        V3 n = detector_normal(g.is2d, eu, ev);
        if (parallel) {
            if (std::fabs(norm(a) - 1.0) > kTolUnit) { *why = "ray_dir is not a unit vector"; return CT_E_FRAME; }
            if (g.beam == CT_PARALLEL2D && std::fabs(dot(a, eu)) > kTolOrtho) {
                *why = "ray_dir and det_u are not orthogonal";
                return CT_E_FRAME;
            }
            if (std::fabs(dot(a, n)) <= kTolTangent) { *why = "ray_dir is tangent to the detector plane"; return CT_E_FRAME; }
            if (norm(c) > 1e6 * smin) { *why = "detector centre beyond 1e6 voxel spacings"; return CT_E_RANGE; }
        } else {
            V3 sc = c - a;
            double dist = norm(sc);
            if (!(dist > 0.0)) { *why = "source coincides with the detector centre"; return CT_E_FRAME; }
            if (std::fabs(dot(sc, n)) <= kTolTangent * dist) { *why = "source views the detector edge-on"; return CT_E_FRAME; }
            double near = std::fmin(norm(a), norm(c)), far = std::fmax(norm(a), norm(c));
            if (near > 1e6 * smin) { *why = "nearer endpoint beyond 1e6 voxel spacings"; return CT_E_RANGE; }
            if (far > 1e15 * smin) { *why = "endpoint beyond 1e15 voxel spacings"; return CT_E_RANGE; }
        }
    }
    if (out) *out = g;
    return CT_OK;
}

namespace {

bool invert3(const double m[9], double inv[9]) {
    double a = m[0], b = m[1], c = m[2], d = m[3], e = m[4], f = m[5], g = m[6], h = m[7], i = m[8];
    double A = e * i - f * h, B = -(d * i - f * g), C = d * h - e * g;
    double det = a * A + b * B + c * C;
    if (det == 0.0 || !std::isfinite(det)) return false;
    double r = 1.0 / det;
    inv[0] = A * r;
    inv[1] = -(b * i - c * h) * r;
    inv[2] = (b * f - c * e) * r;
    inv[3] = B * r;
    inv[4] = (a * i - c * g) * r;
    inv[5] = -(a * f - c * d) * r;
    inv[6] = C * r;
    inv[7] = -(a * h - b * g) * r;
    inv[8] = (a * e - b * d) * r;
    return true;
}

}  // namespace

// Forward gather layout per view.  The 16-wide side of a wave's pixel patch runs
// along one detector axis; the gather reads the volume copy whose contiguous axis
// carries the largest share of that axis's pixel step, so neighbouring lanes read
// neighbouring words.  score[a][p] = |step_p . e_a| / |step_p|.  A copy that only
// a few views would use (each needs its own transposed volume) is given up for the
// best copy already in use when that is at least 95% as well aligned.  2D beams
// have one detector axis and keep the caller's x-fastest layout.
static void choose_layouts(const GeomHost &g, double *table) {
    if (g.is2d) return;
    const int64_t n = g.n_views;
    auto score = [&](const double *t, int a, int p) {
        const double *o = t + (p == 0 ? VT_OU : VT_OV), *d = t + (p == 0 ? VT_DU : VT_DV);
        const double st[3] = {o[0] + d[0], o[1] + d[1], o[2] + d[2]};
        const double nn = std::sqrt(st[0] * st[0] + st[1] * st[1] + st[2] * st[2]);
        return nn > 0 ? std::fabs(st[a]) / nn : 0.0;
    };
    int64_t use[3] = {0, 0, 0};
    for (int64_t k = 0; k < n; ++k) {
        double *t = table + k * CT_VIEW_TABLE_STRIDE;
        double best = -1.0;
        int la = 0, pa = 0;
        for (int p = 0; p < 2; ++p)
            for (int a = 0; a < 3; ++a)
                if (score(t, a, p) > best + 1e-9) { best = score(t, a, p); la = a; pa = p; }
        t[VT_LAYOUT] = la;
        t[VT_PATCH] = pa;
        use[la]++;
    }
    for (int64_t k = 0; k < n; ++k) {
        double *t = table + k * CT_VIEW_TABLE_STRIDE;
        const int la = (int)t[VT_LAYOUT];
        if (use[la] * 16 >= n) continue;
        const double own = score(t, la, (int)t[VT_PATCH]);
        double best = -1.0;
        int ba = -1, bp = 0;
        for (int a = 0; a < 3; ++a) {
            if (a == la || use[a] * 16 < n) continue;
            for (int p = 0; p < 2; ++p)
                if (score(t, a, p) > best) { best = score(t, a, p); ba = a; bp = p; }
        }
        if (ba >= 0 && best >= 0.95 * own) {
            t[VT_LAYOUT] = ba;
            t[VT_PATCH] = bp;
        }
    }
}

void build_view_table(const ct_geom_desc_t *desc, const GeomHost &g, double *table) {
    const bool parallel = (g.beam == CT_PARALLEL2D || g.beam == CT_PARALLEL3D);
    const V3 s = {g.sx, g.sy, g.sz};
    const V3 n3 = {double(g.W), double(g.H), double(g.D)};
    const V3 lo = {-0.5 * n3.x * s.x, -0.5 * n3.y * s.y, -0.5 * n3.z * s.z};
    auto to_vox_point = [&](V3 p) { return V3{(p.x - lo.x) / s.x, (p.y - lo.y) / s.y, (p.z - lo.z) / s.z}; };
    auto to_vox_vec = [&](V3 p) { return V3{p.x / s.x, p.y / s.y, p.z / s.z}; };
    auto put = [](double *dst, V3 v) { dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; };

    for (int64_t k = 0; k < g.n_views; ++k) {
        const double *f = desc->frames + 12 * k;
        double *t = table + k * CT_VIEW_TABLE_STRIDE;
        std::memset(t, 0, sizeof(double) * CT_VIEW_TABLE_STRIDE);
        V3 a = v3(f), c = v3(f + 3), eu = v3(f + 6), ev = g.is2d ? V3{0, 0, 0} : v3(f + 9);
        V3 step_u = g.du * eu;
        V3 step_v = g.is2d ? V3{0, 0, 0} : g.dv * ev;
        V3 p00 = c - (0.5 * double(g.U - 1)) * step_u - (0.5 * double(g.V - 1)) * step_v;
        if (g.is2d) p00 = c - (0.5 * double(g.U - 1)) * step_u;
        V3 P00 = to_vox_point(p00), SU = to_vox_vec(step_u), SV = to_vox_vec(step_v);
        V3 n = detector_normal(g.is2d, eu, ev);
        V3 O00, OU{0, 0, 0}, OV{0, 0, 0}, D00, DU{0, 0, 0}, DV{0, 0, 0};
        if (parallel) {
            O00 = P00;
            OU = SU;
            OV = SV;
            D00 = to_vox_vec(a);
            t[VT_TMIN] = -kTBig;
            t[VT_TMAX] = kTBig;
            t[VT_PERSP] = 0.0;
        } else {
            O00 = to_vox_point(a);
            D00 = P00 - O00;
            DU = SU;
            DV = SV;
            t[VT_TMIN] = 0.0;
            t[VT_TMAX] = 1.0;
            t[VT_PERSP] = 1.0;
        }
        put(t + VT_O00, O00);
        put(t + VT_OU, OU);
        put(t + VT_OV, OV);
        put(t + VT_D00, D00);
        put(t + VT_DU, DU);
        put(t + VT_DV, DV);
        put(t + VT_N, V3{n.x * s.x, n.y * s.y, n.z * s.z});
        // columns of M: D00, DU + OU, DV + OV (2D: the normal stands in for v)
        V3 c1 = DU + OU;
        V3 c2 = g.is2d ? to_vox_vec(V3{0, 0, 1}) : DV + OV;
        double m[9] = {D00.x, c1.x, c2.x, D00.y, c1.y, c2.y, D00.z, c1.z, c2.z};
        double inv[9];
        if (!invert3(m, inv)) std::memset(inv, 0, sizeof inv);  // unreachable after validation
        for (int q = 0; q < 9; ++q) t[VT_MINV + q] = inv[q];
        // Forward gather layout: chosen for all views by choose_layouts.
        t[VT_LAYOUT] = 0.0;
        t[VT_PATCH] = 0.0;
        // detector frame for parameterized surfaces
        put(t + VT_C, to_vox_point(c));
        put(t + VT_EU, to_vox_vec(eu));
        put(t + VT_EV, to_vox_vec(ev));
        put(t + VT_EN, to_vox_vec(n));
        // packets: u's (or v's) pixel step runs along one axis alone, whose
        // direction component is below 2^-40 of the largest (the gathers take
        // it as 0): rays one step apart along that detector axis differ only in
        // a coordinate they never cross
        t[VT_PACKET] = -1.0;
        if (parallel && !g.is2d) {
            const double dd[3] = {D00.x, D00.y, D00.z};
            const double dm = std::max(std::fabs(dd[0]), std::max(std::fabs(dd[1]), std::fabs(dd[2]))) * 0x1p-40;
            const double su[3] = {OU.x, OU.y, OU.z}, sv[3] = {OV.x, OV.y, OV.z};
            // the pixel step runs along one axis alone, which the rays do not cross
            auto along = [&](const double *st) {
                int k = -1, n = 0;
                for (int i = 0; i < 3; ++i)
                    if (st[i] != 0.0) {
                        k = i;
                        ++n;
                    }
                return n == 1 && std::fabs(dd[k]) < dm;
            };
            if (along(su)) t[VT_PACKET] = 0.0;
            else if (along(sv)) t[VT_PACKET] = 1.0;
        }
    }
    choose_layouts(g, table);
}

// A pixel's coordinate on an axis its ray never crosses, settled on a lattice
// plane when within 2^-30 cell of it: a ray in a plane belongs to the cell above
// (the kernels decide these cells the same way).
static double settle_on_plane(double o) {
    const double r = std::nearbyint(o);
    return std::fabs(o - r) < 0x1p-30 ? r : o;
}

int build_line_table(const GeomHost &g, const double *table, LineView *out) {
    if (g.is2d || g.beam != CT_PARALLEL3D) return -1;
    // one view's pixels are read through a buffer of 32-bit byte offsets, where a
    // negative offset (a pixel before the detector) must fall outside the view
    if ((double)g.U * (double)g.V * 4.0 >= 2147483648.0) return -1;
    const double sp[3] = {g.sx, g.sy, g.sz};
    bool fits[2] = {true, true};   // every view's rows fit each shape's stage
    for (int64_t k = 0; k < g.n_views; ++k) {
        const double *t = table + (size_t)k * CT_VIEW_TABLE_STRIDE;
        if (t[VT_PACKET] < 0.0) return -1;
        LineView &L = out[k];
        std::memset(&L, 0, sizeof L);
        L.P = t[VT_PACKET] == 0.0 ? 0 : 1;
        const double *OP = t + (L.P == 0 ? VT_OU : VT_OV), *OQ = t + (L.P == 0 ? VT_OV : VT_OU);
        const double *O = t + VT_O00, *D = t + VT_D00;
        int d = -1;
        for (int i = 0; i < 3; ++i)
            if (OP[i] != 0.0) d = i;
        // one voxel plane per pixel column, the other detector axis in the plane
        if (d < 0 || std::fabs(OP[d]) != 1.0 || OQ[d] != 0.0) return -1;
        L.d = d;
        L.g = OP[d] > 0.0 ? 1 : -1;
        const double kc = std::floor(settle_on_plane(O[d]));
        if (std::fabs(kc) > 1e9) return -1;
        L.kc = (int)kc;
        const int a = d == 0 ? 1 : 0, b = d == 2 ? 1 : 2;
        // in-plane direction in voxel coordinates; a component below 2^-40 of the
        // largest counts as zero, as in the walks
        const double dm = std::max(std::fabs(D[0]), std::max(std::fabs(D[1]), std::fabs(D[2]))) * 0x1p-40;
        double ea = std::fabs(D[a]) < dm ? 0.0 : D[a], eb = std::fabs(D[b]) < dm ? 0.0 : D[b];
        const double len = std::sqrt(ea * ea + eb * eb);
        if (!(len > 0.0)) return -1;
        ea /= len;
        eb /= len;
        const double na = -eb, nb = ea;
        // physical length per voxel-coordinate length along the ray
        const double kap = std::sqrt((D[a] * sp[a]) * (D[a] * sp[a]) + (D[b] * sp[b]) * (D[b] * sp[b])) /
                           std::sqrt(D[a] * D[a] + D[b] * D[b]);
        L.na = na;
        L.nb = nb;
        L.naf = (float)na;
        L.nbf = (float)nb;
        L.E0 = na * O[a] + nb * O[b];
        L.dq = na * OQ[a] + nb * OQ[b];
        if (!(std::fabs(L.dq) > 1e-9)) return -1;
        L.inv_dq = 1.0 / L.dq;
        L.inv_dqf = (float)L.inv_dq;
        const double A = std::fabs(ea), B = std::fabs(eb);
        L.H = (float)(0.5 * (A + B));
        L.Lmax = (float)(kap / std::max(A, B));
        if (A == 0.0 || B == 0.0) {
            L.aligned = A == 0.0 ? 1 : 2;
            const int c = A == 0.0 ? a : b;
            L.X0 = O[c];
            L.Xq = OQ[c];
            if (L.Xq == 0.0) return -1;
        } else {
            L.R = (float)(kap / (A * B));
        }
        // rows one brick stages for this view: its cross-section's shadow along n
        for (int k2 = 0; k2 < 2; ++k2) {
            const LineShape &sh = kLineShapes[k2];
            const int ext[3] = {sh.bx, sh.by, sh.bz};
            const double w = 0.5 * (std::fabs(na) * ext[a] + std::fabs(nb) * ext[b]);
            if (2.0 * (0.5 * (A + B) + w) / std::fabs(L.dq) + 4.0 > (double)sh.rows) fits[k2] = false;
        }
        if (d == 2) fits[1] = false;   // shape 1's lines run along x or y only
    }
    // each view's distance to the next view of its family (0: the last one)
    int last[3] = {-1, -1, -1};
    for (int64_t k = 0; k < g.n_views; ++k) {
        const int d = out[k].d;
        if (last[d] >= 0) out[last[d]].next = (int)(k - last[d]);
        last[d] = (int)k;
    }
    return fits[1] ? 1 : (fits[0] ? 0 : -1);
}

// Range of the brick adjoint's 64-bit accumulator.  Each (ray, voxel) pair adds
// at most one voxel chord times the largest ray value: below 2^46 in the
// accumulator's units (both factors are under 2^23).  The rays of one view that
// cross one voxel are those whose pixel centres fall in the voxel's image on
// the detector: at most (e_u + 1)(e_v + 1) for an image of extent e_u x e_v
// pixels.  Parallel beams: e_u = sum_a |d beta / d X_a| (the second row of
// MINV; voxel-coordinate axes are one voxel long).  Fan/cone: u = beta/alpha,
// d u / d X_a = (MINV1_a - u MINV0_a) / alpha with 0 <= u <= U - 1 wherever a
// pixel centre lies, and alpha is smallest at a corner of the volume box (it
// is affine in X); a box reaching the source plane (alpha <= 0) may be
// crossed by every ray of the view.  A detector surface has no such image
// bound: every pixel counts.  The sum over the views times 2^46 must stay
// below 2^62 (one bit of margin under the sign); each doubling beyond that
// costs one bit of right shift on every term.
double adjoint_rays_bound(const GeomHost &g, const double *table, bool surface) {
    const double all = double(g.U) * double(g.V);
    double total = 0.0;
    for (int64_t k = 0; k < g.n_views; ++k) {
        const double *t = table + k * CT_VIEW_TABLE_STRIDE;
        const double *M = t + VT_MINV;
        double count = all;
        if (!surface) {
            double eu = 0.0, ev = 0.0;
            bool bounded = true;
            if (t[VT_PERSP] != 0.0) {
                double amin = INFINITY;
                for (int c = 0; c < 8; ++c) {
                    const double X[3] = {(c & 1) ? double(g.W) : 0.0, (c & 2) ? double(g.H) : 0.0,
                                         (c & 4) ? double(g.D) : 0.0};
                    double al = 0.0;
                    for (int a = 0; a < 3; ++a) al += M[a] * (X[a] - t[VT_O00 + a]);
                    amin = std::fmin(amin, al);
                }
                bounded = amin > 1e-9;
                if (bounded) {
                    for (int a = 0; a < 3; ++a) {
                        eu += std::fabs(M[3 + a]) + double(g.U - 1) * std::fabs(M[a]);
                        ev += std::fabs(M[6 + a]) + double(g.V - 1) * std::fabs(M[a]);
                    }
                    eu /= amin;
                    ev /= amin;
                }
            } else {
                for (int a = 0; a < 3; ++a) {
                    eu += std::fabs(M[3 + a]);
                    ev += std::fabs(M[6 + a]);
                }
            }
            if (bounded) {
                const double nu = std::fmin(double(g.U), eu + 1.0);
                const double nv = g.is2d ? 1.0 : std::fmin(double(g.V), ev + 1.0);
                count = nu * nv;
            }
        }
        total += count;
    }
    return total;
}

int adjoint_term_shift(double rays_bound) {
    int h = 0;
    while (h < 40 && rays_bound >= std::ldexp(1.0, 16 + h)) ++h;
    return h;
}

}  // namespace ctp
