// ct_internal.h -- data shared by the host side and the kernels of libctproj.
//
// Per-view ray table (float64, CT_VIEW_TABLE_STRIDE doubles per view).  All
// vectors are in VOXEL coordinates: X_a = (x_a - lo_a) / s_a with lo_a = -n_a s_a / 2,
// so voxel (i_x, i_y, i_z) is the unit cube [i, i+1) on each axis and the volume
// box is [0, W) x [0, H) x [0, D).
//
// The ray of pixel (u, v) is X(t) = O(u, v) + t Dir(u, v), t in [tmin, tmax], with
//   O   = O00 + u OU + v OV
//   Dir = D00 + u DU + v DV
// fan/cone : O = source (OU = OV = 0), Dir = pixel centre - source, t in [0, 1]
// parallel : O = pixel centre,         Dir = ray_dir (DU = DV = 0), t unbounded
// The physical length of dt is |dt| * || Dir (.) spacing ||.
//
// N: detector normal scaled by the voxel spacing (n_a s_a), so that a plane
// parallel to the detector through a voxel-space point C is {X : (X - C).N = 0}.
// MINV: inverse of the 3x3 matrix [D00 | DU+OU | DV+OV] (columns); for a point X
// it gives (alpha, beta, gamma) = MINV (X - O00) with
//   perspective (fan/cone): u = beta / alpha, v = gamma / alpha (alpha > 0 in front
//                           of the source)
//   parallel              : u = beta, v = gamma
// 2D geometries put the detector normal in the third column so MINV exists; the
// v coordinate is then meaningless and ignored.
//
// C / EU / EV / EN: the detector frame, for parameterized detector surfaces.
//
// LAYOUT / PATCH: the forward projector gathers from the volume copy whose
// contiguous axis lies closest to the detector direction along which a wave's
// 16-wide pixel patch runs, so neighbouring lanes read neighbouring words.
#pragma once

#include <cstdint>

#include "ctproj.h"

namespace ctp {

enum ViewSlot : int {
    VT_O00 = 0,
    VT_OU = 3,
    VT_OV = 6,
    VT_D00 = 9,
    VT_DU = 12,
    VT_DV = 15,
    VT_TMIN = 18,
    VT_TMAX = 19,
    VT_N = 20,
    VT_PERSP = 23,
    VT_MINV = 24,   // 9 values, row-major
    VT_LAYOUT = 33, // volume copy the forward gathers from: 0 x-, 1 y-, 2 z-fastest
    VT_PATCH = 34,  // forward wave patch: 0 = 16 u x 4 v, 1 = 4 u x 16 v
    VT_C = 35,      // detector centre (point)
    VT_EU = 38,     // e_u, e_v and the normal n as voxel-coordinate vectors (e / s):
    VT_EV = 41,     // a surface pixel with local offsets (o_u, o_v, o_n) sits at
    VT_EN = 44,     // C + o_u EU + o_v EV + o_n EN
    VT_END = 47
};
static_assert(VT_END <= CT_VIEW_TABLE_STRIDE, "view table overflow");

// finite stand-in for an unbounded parameter range (keeps arithmetic NaN-free)
constexpr double kTBig = 1e30;

struct GeomHost {
    int beam = 0;
    bool is2d = false;
    int64_t n_views = 0;
    int64_t D = 0, H = 0, W = 0;
    double sz = 1, sy = 1, sx = 1;
    int64_t U = 0, V = 0;
    double du = 1, dv = 1;
};

// Validation and table precompute (host only, no HIP calls): ct_geometry.cpp
ct_status_t validate_desc(const ct_geom_desc_t *desc, GeomHost *out, const char **why);
void build_view_table(const ct_geom_desc_t *desc, const GeomHost &g, double *table);

void set_error(const char *msg);

}  // namespace ctp
