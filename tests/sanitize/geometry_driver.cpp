// Sanitizer driver for the host side of the HIP library: the frame validation,
// the per-view ray table and the adjoint's range bound
// (ray_driven_projector_amd/csrc/ct_geometry.cpp, no HIP code), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitize.py.
// Runs valid descriptors of all four beams and every validation error path;
// exit status 0 means clean and every status as expected.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "ct_internal.h"

namespace ctp {
void set_error(const char *) {}
}

using namespace ctp;

static std::vector<double> frames(int beam, int n) {
    std::vector<double> f(12 * n, 0.0);
    for (int k = 0; k < n; ++k) {
        const double th = 2.0 * M_PI * k / n, c = std::cos(th), s = std::sin(th);
        double *r = &f[12 * k];
        if (beam == CT_FAN2D || beam == CT_CONE) {
            r[0] = 50 * c; r[1] = 50 * s;
            r[3] = -30 * c; r[4] = -30 * s;
        } else {
            r[0] = -c; r[1] = -s;
        }
        r[6] = s; r[7] = -c;
        if (beam == CT_CONE || beam == CT_PARALLEL3D) r[11] = 1.0;
    }
    return f;
}

static ct_geom_desc_t desc(int beam, const std::vector<double> &f, int n) {
    ct_geom_desc_t d{};
    d.beam = beam;
    d.n_views = n;
    const bool two_d = beam == CT_PARALLEL2D || beam == CT_FAN2D;
    d.vol_shape[0] = two_d ? 1 : 7; d.vol_shape[1] = 9; d.vol_shape[2] = 11;
    d.voxel_spacing[0] = 1.0; d.voxel_spacing[1] = 0.9; d.voxel_spacing[2] = 1.1;
    d.det_shape[0] = 21; d.det_shape[1] = two_d ? 1 : 13;
    d.det_spacing[0] = 0.8; d.det_spacing[1] = 0.7;
    d.frames = f.data();
    return d;
}

static int expect(const char *what, ct_status_t got, ct_status_t want) {
    if (got != want) {
        std::printf("%s: status %d, expected %d\n", what, (int)got, (int)want);
        return 1;
    }
    return 0;
}

int main() {
    int bad = 0;
    for (int beam = 0; beam < 4; ++beam) {
        const int n = 9;
        std::vector<double> f = frames(beam, n);
        ct_geom_desc_t d = desc(beam, f, n);
        GeomHost h;
        const char *why = "";
        bad |= expect("valid", validate_desc(&d, &h, &why), CT_OK);
        std::vector<double> table((size_t)n * CT_VIEW_TABLE_STRIDE);
        build_view_table(&d, h, table.data());
        for (double v : table)
            if (!std::isfinite(v) && std::fabs(v) != 1e30) bad |= 1;
        const double b0 = adjoint_rays_bound(h, table.data(), false);
        const double b1 = adjoint_rays_bound(h, table.data(), true);
        if (!(b0 > 0 && b0 <= b1) || adjoint_term_shift(b0) != 0 || adjoint_term_shift(1e9) != 14) bad |= 1;
        std::printf("beam %d: table ok, rays bound %.1f (surface %.0f)\n", beam, b0, b1);

        // error paths, each on a copy of the valid frames
        const double nan = std::numeric_limits<double>::quiet_NaN();
        struct Case { const char *what; int idx; double val; ct_status_t want; };
        const Case cases[] = {
            {"NaN frame", 4, nan, CT_E_NONFINITE},
            {"non-unit e_u", 6, 2.0, CT_E_FRAME},
            {"far away", 0, 1e17, beam == CT_FAN2D || beam == CT_CONE ? CT_E_RANGE : CT_E_FRAME},
        };
        for (const Case &c : cases) {
            std::vector<double> g = f;
            g[c.idx] = c.val;
            ct_geom_desc_t e = desc(beam, g, n);
            const ct_status_t st = validate_desc(&e, &h, &why);
            if (st == CT_OK) bad |= expect(c.what, st, c.want);
        }
        ct_geom_desc_t e = d;
        e.n_views = 0;
        bad |= expect("no views", validate_desc(&e, &h, &why), CT_E_SHAPE);
        e = d;
        e.voxel_spacing[1] = -1.0;
        bad |= (validate_desc(&e, &h, &why) == CT_OK);
        e = d;
        e.frames = nullptr;
        bad |= expect("null frames", validate_desc(&e, &h, &why), CT_E_NULL);
        e = d;
        e.reserved = 3;
        bad |= expect("reserved", validate_desc(&e, &h, &why), CT_E_ARG);
        e = d;
        e.beam = 7;
        bad |= expect("beam", validate_desc(&e, &h, &why), CT_E_ARG);
    }
    {
        GeomHost h;
        const char *why = "";
        bad |= expect("null descriptor", validate_desc(nullptr, &h, &why), CT_E_NULL);
    }
    return bad;
}
