// ct_launch.h -- launchers implemented in ct_kernels.hip, used by ct_abi.hip.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

namespace ctp {

struct LaunchGeom {
    const double *views;  // device view table
    int W, H, D, U, V, n_views;
    double spx, spy, spz;  // voxel spacing (x, y, z)
    bool two_d;
    bool persp;            // fan/cone beam (rays from a source), else parallel
    int yshift;            // brick adjoint: every fixed-point term is shifted right by
                           // this many bits (0 unless the geometry's term bound needs it)
    int offx, offy, offz;  // region launches: voxel index of the buffer's first voxel
    int accumulate;        // region launches: add to the output instead of writing it
    const double *surf_off; // detector surface offsets (device float64), or null: flat
    int surf_per_view;      // offsets given per view
    float *surf_env;        // per-view footprint envelopes of the surface (device)
    float *vol_yf;         // handle-owned y-fastest volume copy, or null if no view reads it
    float *vol_zf;         // handle-owned z-fastest volume copy, or null if no view reads it
    bool need_yf, need_zf; // some view's gathers read that copy
    bool packet;           // flat detector and every view has a packet axis (VT_PACKET >= 0):
                           // the forward takes rays in packets
    const void *brick_rec; // brick adjoint: the handle's per-(brick, view) record table, or null
                           // (launches whose bricks are not the whole volume's compute them)
    int rec_stride;        // views per brick in the table
    int rec_view0;         // table view of the launch's first view
    const void *line_tab;  // separable tilt series: the line table (LineView) from the launch's
                           // first view; the adjoint then runs the line kernel (else null)
    int line_shape;        // its brick shape (an index into kLineShapes)
};

hipError_t launch_fill(float *p, size_t n, float v, hipStream_t s);
hipError_t launch_project(const LaunchGeom &g, const float *vol, float *sino, hipStream_t s);
hipError_t launch_residual(const LaunchGeom &g, const float *x, const float *y, const float *rinv,
                           float *e, hipStream_t s);
hipError_t launch_rowinv(const LaunchGeom &g, float *rinv, hipStream_t s);
hipError_t launch_count(const LaunchGeom &g, uint32_t *per_ray, unsigned long long *total,
                        hipStream_t s);
hipError_t launch_backproject_atomic(const LaunchGeom &g, const float *sino, float *vol,
                                     hipStream_t s);
hipError_t launch_backproject(const LaunchGeom &g, const float *sino, float *vol, hipStream_t s);
hipError_t launch_sirt_update(const LaunchGeom &g, const float *e, const float *cinv, float relax,
                              float *x, hipStream_t s);
hipError_t launch_colinv(const LaunchGeom &g, float *cinv, hipStream_t s);
// The brick adjoint's per-(brick, view) record table of a whole-volume launch:
// brick_record_count(g) records of brick_record_bytes() each (footprint and
// anchor of every pair), built once at geometry creation.
size_t brick_record_count(const LaunchGeom &g);
size_t brick_record_bytes();
hipError_t launch_brick_records(const LaunchGeom &g, void *out, hipStream_t s);
// Per-view footprint envelopes of a detector surface (once, at geometry creation).
// bad (device) receives nonzero if a fan/cone surface pixel is not in front of
// the source.
hipError_t launch_surface_env(const LaunchGeom &g, unsigned long long *bad, hipStream_t s);
size_t surface_env_floats(int U, int V);   // per view
hipError_t launch_sirt_update_bounded(const LaunchGeom &g, const float *e, const float *cinv,
                                      float relax, float lo, float hi, const uint8_t *mask, float *x,
                                      hipStream_t s);

// CGLS.  Workspace: kCglsStateDoubles scalars, then one float64 partial per
// block of the largest launch (forward blocks, bricks or kCglsVecBlocks).
enum CglsSlot : int { CS_GAMMA = 0, CS_ALPHA = 1, CS_BETA = 2, CS_QQ = 3, CS_RR = 4 };
enum CglsOp : int { CO_RR = 0, CO_INIT = 1, CO_ALPHA = 2, CO_BETA = 3 };
constexpr int kCglsStateDoubles = 32;   // 256 bytes
constexpr unsigned kCglsVecBlocks = 4096;
size_t cgls_ray_blocks(const LaunchGeom &g);
size_t cgls_brick_blocks(const LaunchGeom &g);
hipError_t launch_cgls_init(const LaunchGeom &g, const float *y, const float *x, float *r, float *s,
                            float *p, double *state, double *partial, hipStream_t st);
hipError_t launch_cgls_step(const LaunchGeom &g, float *x, float *r, float *s, float *p, float *q,
                            double *state, double *partial, hipStream_t st);

}  // namespace ctp
