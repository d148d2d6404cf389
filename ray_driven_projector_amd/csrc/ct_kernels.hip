// ct_kernels.hip -- gfx950 kernels of the ray-driven projector pair.
//
// Operator (diffct documentation, "Differentiable analytical reconstruction"):
// the cell-constant Siddon forward projector A, a_ij = length of ray i inside
// voxel j, and its matched adjoint A^T.  Siddon's observation is used in both
// directions: along a ray the cell boundaries are the planes of the three lattice
// axes, so the ray's parameter interval inside the volume is cut at each plane
// crossing and each piece lies in exactly one cell.
//
// Numerics.  Per ray, the clip against the box, the first and last cell and the
// number of plane crossings per axis are computed in float64.  The walk itself
// runs in float32 on the physical distance measured from the ray's entry point:
// the m-th crossing of axis a sits at fma(m, q_a, l0_a) (q_a = length per cell
// along a, l0_a = distance to the first crossing), recomputed rather than
// accumulated so its error stays at one rounding.  The walk ends at
//   l_end = min(chord, min_a fma(N_a, q_a, l0_a)),
// evaluated with the same float32 expression as the crossings; since that
// expression is monotone in m, any crossing taken before l_end is one of the
// N_a real crossings of its axis, so cell indices never leave the volume.
//
// Layout.  Volume (D,H,W) float32, sinogram (views,U,V) float32, V fastest.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "ct_internal.h"
#include "ct_launch.h"

namespace ctp {

#define CT_INF __builtin_huge_valf()

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs of the chip; this maps
// the hardware block id to a logical tile id so that each XCD walks a
// contiguous range of tiles (neighbouring tiles share volume cache lines in that
// XCD's L2).  Bijective for any block count.
__device__ __forceinline__ int xcd_remap(int hw, int nblocks) {
    constexpr int kXcd = 8;
    int q = nblocks / kXcd, r = nblocks % kXcd;
    int x = hw % kXcd, k = hw / kXcd;
    return x * q + min(x, r) + k;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// One axis of the slab clip in voxel coordinates: box [0, n) on this axis.
__device__ __forceinline__ void clip_axis(double o, double d, double n, double &tin, double &tout,
                                          bool &hit) {
    if (d == 0.0) {
        hit = hit && (o >= 0.0) && (o < n);
    } else {
        double inv = 1.0 / d;
        double t0 = -o * inv, t1 = (n - o) * inv;
        tin = fmax(tin, fmin(t0, t1));
        tout = fmin(tout, fmax(t0, t1));
    }
}

// First cell, crossing count and distance (in cells) to the first crossing on
// one axis, for the interval [tin, tout].  The first cell holds the points just
// after tin, the last cell those just before tout.
__device__ __forceinline__ void axis_cells(double o, double d, double tin, double tout, int n,
                                           int &c0, int &ncross, double &dist) {
    double e = fma(tin, d, o);
    double x = fma(tout, d, o);
    int ce, cx;
    if (d > 0.0) {
        ce = (int)floor(e);
        cx = (int)ceil(x) - 1;
    } else if (d < 0.0) {
        ce = (int)ceil(e) - 1;
        cx = (int)floor(x);
    } else {
        ce = (int)floor(e);
        cx = ce;
    }
    ce = min(max(ce, 0), n - 1);
    cx = min(max(cx, 0), n - 1);
    c0 = ce;
    ncross = d > 0.0 ? max(cx - ce, 0) : (d < 0.0 ? max(ce - cx, 0) : 0);
    dist = d > 0.0 ? (double)(ce + 1) - e : (d < 0.0 ? e - (double)ce : 0.0);
}

// Walk state of one ray (T = float for the gathers, double where every single
// piece length must be exact to float64 rounding).
template <class T>
struct Walk {
    int idx;            // element index of the current cell
    int stx, sty, stz;  // signed element strides
    int ncross;         // plane crossings inside the interval (all axes)
    T l0x, l0y, l0z;
    T qx, qy, qz;
    T lend;
};

__device__ __forceinline__ float t_fma(float a, float b, float c) { return fmaf(a, b, c); }
__device__ __forceinline__ double t_fma(double a, double b, double c) { return fma(a, b, c); }
__device__ __forceinline__ float t_min(float a, float b) { return fminf(a, b); }
__device__ __forceinline__ double t_min(double a, double b) { return fmin(a, b); }
template <class T> __device__ __forceinline__ T t_inf();
template <> __device__ __forceinline__ float t_inf<float>() { return __builtin_huge_valf(); }
template <> __device__ __forceinline__ double t_inf<double>() { return __builtin_huge_val(); }

// Build the walk of the ray o + t d (voxel coordinates) through the box
// [0,nx) x [0,ny) x [0,nz), t in [tmin, tmax]; element strides (1, sy, sz).
// Returns false if the ray misses the box.  chord receives the physical length.
template <class T>
__device__ __forceinline__ bool make_walk(double ox, double oy, double oz, double dx, double dy,
                                          double dz, double tmin, double tmax, int nx, int ny,
                                          int nz, int sy, int sz, double spx, double spy,
                                          double spz, Walk<T> &w, float &chord) {
    // A component below 2^-40 of the largest moves the ray by less than 1e-12 of
    // its length along that axis: treat the ray as parallel to those planes, which
    // keeps every per-axis step length finite in float32.
    {
        const double dm = fmax(fabs(dx), fmax(fabs(dy), fabs(dz))) * 0x1p-40;
        if (fabs(dx) < dm) dx = 0.0;
        if (fabs(dy) < dm) dy = 0.0;
        if (fabs(dz) < dm) dz = 0.0;
    }
    double tin = tmin, tout = tmax;
    bool hit = true;
    clip_axis(ox, dx, (double)nx, tin, tout, hit);
    clip_axis(oy, dy, (double)ny, tin, tout, hit);
    clip_axis(oz, dz, (double)nz, tin, tout, hit);
    hit = hit && (tout > tin);
    if (!hit) return false;
    int cx, cy, cz, nxc, nyc, nzc;
    double ddx, ddy, ddz;
    axis_cells(ox, dx, tin, tout, nx, cx, nxc, ddx);
    axis_cells(oy, dy, tin, tout, ny, cy, nyc, ddy);
    axis_cells(oz, dz, tin, tout, nz, cz, nzc, ddz);
    double px = dx * spx, py = dy * spy, pz = dz * spz;
    double L = sqrt(px * px + py * py + pz * pz);
    w.idx = (cz * ny + cy) * nx + cx;
    w.ncross = nxc + nyc + nzc;
    w.stx = dx > 0.0 ? 1 : -1;
    w.sty = dy > 0.0 ? sy : -sy;
    w.stz = dz > 0.0 ? sz : -sz;
    const T ch = (T)((tout - tin) * L);
    T lend = ch;
    if (dx != 0.0) {
        double q = L / fabs(dx);
        w.qx = (T)q;
        w.l0x = (T)(ddx * q);
        lend = t_min(lend, t_fma((T)nxc, w.qx, w.l0x));
    } else {
        w.qx = (T)0;
        w.l0x = t_inf<T>();
    }
    if (dy != 0.0) {
        double q = L / fabs(dy);
        w.qy = (T)q;
        w.l0y = (T)(ddy * q);
        lend = t_min(lend, t_fma((T)nyc, w.qy, w.l0y));
    } else {
        w.qy = (T)0;
        w.l0y = t_inf<T>();
    }
    if (dz != 0.0) {
        double q = L / fabs(dz);
        w.qz = (T)q;
        w.l0z = (T)(ddz * q);
        lend = t_min(lend, t_fma((T)nzc, w.qz, w.l0z));
    } else {
        w.qz = (T)0;
        w.l0z = t_inf<T>();
    }
    w.lend = lend;
    chord = (float)ch;
    return true;
}

// Visit every (cell, length) piece of the walk in order; f(idx, len).
template <class T, class F>
__device__ __forceinline__ void walk(const Walk<T> &w, F &&f) {
    int idx = w.idx;
    T lc = (T)0;
    T mx = (T)0, my = (T)0, mz = (T)0;
    T lx = w.l0x, ly = w.l0y, lz = w.l0z;
    const T lend = w.lend;
    for (;;) {
        const T tmin = t_min(t_min(lx, ly), lz);
        const T tn = t_min(tmin, lend);
        f(idx, tn - lc);
        if (!(tmin < lend)) break;  // also leaves on NaN
        lc = tn;
        if (lx == tmin) {
            idx += w.stx;
            mx += (T)1;
            lx = t_fma(mx, w.qx, w.l0x);
        }
        if (ly == tmin) {
            idx += w.sty;
            my += (T)1;
            ly = t_fma(my, w.qy, w.l0y);
        }
        if (lz == tmin) {
            idx += w.stz;
            mz += (T)1;
            lz = t_fma(mz, w.qz, w.l0z);
        }
    }
}

// Ray set-up shared by the gathers: drop negligible direction components, clip
// to the volume box in float64.  Returns false on a miss.
__device__ __forceinline__ bool clip_ray(double ox, double oy, double oz, double &dx, double &dy,
                                         double &dz, double tmin, double tmax, int nx, int ny,
                                         int nz, double &tin, double &tout) {
    const double dm = fmax(fabs(dx), fmax(fabs(dy), fabs(dz))) * 0x1p-40;
    if (fabs(dx) < dm) dx = 0.0;
    if (fabs(dy) < dm) dy = 0.0;
    if (fabs(dz) < dm) dz = 0.0;
    tin = tmin;
    tout = tmax;
    bool hit = true;
    clip_axis(ox, dx, (double)nx, tin, tout, hit);
    clip_axis(oy, dy, (double)ny, tin, tout, hit);
    clip_axis(oz, dz, (double)nz, tin, tout, hit);
    return hit && (tout > tin);
}

// Cells of one axis for a chunk of the ray.  On the major axis the chunk's first
// cell and cell count are known exactly; a chunk after the first starts on a
// plane of that axis, one full cell before its next crossing.
__device__ __forceinline__ void chunk_axis(double o, double d, double ta, double tb, int n,
                                           bool major, int first, int cells, bool first_chunk,
                                           int &c0, int &ncr, double &dist) {
    if (major) {
        c0 = first;
        ncr = cells - 1;
        if (first_chunk) {
            const double e = fma(ta, d, o);
            dist = d > 0.0 ? (double)(first + 1) - e : e - (double)first;
        } else {
            dist = 1.0;
        }
    } else {
        axis_cells(o, d, ta, tb, n, c0, ncr, dist);
    }
}

// Cells of the major axis covered by one chunk of the float32 walk.  Positions
// inside a chunk stay below 64 * sqrt(3) cell lengths, where float32 resolves
// better than 1e-5 of a cell.
constexpr int kChunk = 64;

// Visit the pieces of the ray o + t d, t in [tin, tout] (inside the box), with
// the float32 walk re-based at every kChunk cells of the major axis.
template <class F>
__device__ __forceinline__ void walk_chunked(double ox, double oy, double oz, double dx, double dy,
                                             double dz, double tin, double tout, int nx, int ny,
                                             int nz, int sy, int sz, double spx, double spy,
                                             double spz, F &&f) {
    const double px = dx * spx, py = dy * spy, pz = dz * spz;
    const double L = sqrt(px * px + py * py + pz * pz);
    const double ax = fabs(dx), ay = fabs(dy), az = fabs(dz);
    const int M = (ax >= ay && ax >= az) ? 0 : (ay >= az ? 1 : 2);
    const double oM = M == 0 ? ox : (M == 1 ? oy : oz);
    const double dM = M == 0 ? dx : (M == 1 ? dy : dz);
    const int nM = M == 0 ? nx : (M == 1 ? ny : nz);
    const double eM = fma(tin, dM, oM), xM = fma(tout, dM, oM);
    const int sgn = dM > 0.0 ? 1 : -1;
    int cin = sgn > 0 ? (int)floor(eM) : (int)ceil(eM) - 1;
    int cout = sgn > 0 ? (int)ceil(xM) - 1 : (int)floor(xM);
    cin = min(max(cin, 0), nM - 1);
    cout = min(max(cout, 0), nM - 1);
    const int ncell = max((cout - cin) * sgn, 0) + 1;
    const int nch = (ncell + kChunk - 1) / kChunk;
    const float qx = dx != 0.0 ? (float)(L / ax) : 0.f;
    const float qy = dy != 0.0 ? (float)(L / ay) : 0.f;
    const float qz = dz != 0.0 ? (float)(L / az) : 0.f;
    double ta = tin;
    for (int ch = 0; ch < nch; ++ch) {
        const int first = cin + sgn * ch * kChunk;
        const int cells = min(kChunk, ncell - ch * kChunk);
        double tb = tout;
        if (ch != nch - 1) {
            const int P = sgn > 0 ? first + cells : first - cells + 1;
            tb = ((double)P - oM) / dM;
        }
        int cx, cy, cz, nxc, nyc, nzc;
        double ddx, ddy, ddz;
        chunk_axis(ox, dx, ta, tb, nx, M == 0, first, cells, ch == 0, cx, nxc, ddx);
        chunk_axis(oy, dy, ta, tb, ny, M == 1, first, cells, ch == 0, cy, nyc, ddy);
        chunk_axis(oz, dz, ta, tb, nz, M == 2, first, cells, ch == 0, cz, nzc, ddz);
        Walk<float> w;
        w.idx = (cz * ny + cy) * nx + cx;
        w.ncross = nxc + nyc + nzc;
        w.stx = dx > 0.0 ? 1 : -1;
        w.sty = dy > 0.0 ? sy : -sy;
        w.stz = dz > 0.0 ? sz : -sz;
        float lend = (float)((tb - ta) * L);
        w.qx = qx;
        w.qy = qy;
        w.qz = qz;
        w.l0x = dx != 0.0 ? (float)(ddx * (L / ax)) : CT_INF;
        w.l0y = dy != 0.0 ? (float)(ddy * (L / ay)) : CT_INF;
        w.l0z = dz != 0.0 ? (float)(ddz * (L / az)) : CT_INF;
        if (dx != 0.0) lend = fminf(lend, fmaf((float)nxc, qx, w.l0x));
        if (dy != 0.0) lend = fminf(lend, fmaf((float)nyc, qy, w.l0y));
        if (dz != 0.0) lend = fminf(lend, fmaf((float)nzc, qz, w.l0z));
        w.lend = lend;
        walk(w, f);
        ta = tb;
    }
}

// ---------------------------------------------------------------------------
// ray-driven kernels (forward, SIRT residual, row sums, counting, atomic A^T)
// ---------------------------------------------------------------------------

enum RayMode : int { RM_PROJECT = 0, RM_RESIDUAL = 1, RM_ROWINV = 2, RM_COUNT = 3, RM_ATOMIC_BP = 4 };

struct RayArgs {
    const double *views;
    const float *vol;          // RM_PROJECT, RM_RESIDUAL
    float *out;                // sinogram-shaped output; RM_ATOMIC_BP: the volume
    const float *sino;         // RM_RESIDUAL: y; RM_ATOMIC_BP: the sinogram
    const float *rinv;         // RM_RESIDUAL
    uint32_t *counts;          // RM_COUNT (nullable)
    unsigned long long *total; // RM_COUNT
    int W, H, D, U, V, n_views;
    double spx, spy, spz;
    int n_utiles, n_vtiles, n_blocks;
    uint32_t vol_bytes;
};

// Tiles: 3D 16(u) x 16(v) per 256-thread block, each wave an 8 x 8 patch, so
// the 64 rays of a wave form a tight bundle that touches few cache lines per
// step.  2D: 256 consecutive u per block.  Block order: v-band outermost, then
// view, then u tile, so all views of one detector band (one slab of the volume
// for cone/parallel3d orbits) run together while that slab is cache-resident.
template <int MODE, bool TWO_D>
__global__ __launch_bounds__(256) void ray_kernel(RayArgs a) {
    const int blk = xcd_remap(blockIdx.x, a.n_blocks);
    const int ut = blk % a.n_utiles;
    const int rest = blk / a.n_utiles;
    const int view = rest % a.n_views;
    const int band = rest / a.n_views;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int u, v;
    if (TWO_D) {
        u = ut * 256 + threadIdx.x;
        v = 0;
    } else {
        u = ut * 16 + (wv & 1) * 8 + (lane >> 3);
        v = band * 16 + (wv >> 1) * 8 + (lane & 7);
    }
    const bool active = (u < a.U) && (v < a.V);
    uint32_t my_count = 0;
    if (active) {
        const double *vw = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
        const double fu = (double)u, fv = (double)v;
        double ox = vw[VT_O00 + 0] + fu * vw[VT_OU + 0] + fv * vw[VT_OV + 0];
        double oy = vw[VT_O00 + 1] + fu * vw[VT_OU + 1] + fv * vw[VT_OV + 1];
        double oz = vw[VT_O00 + 2] + fu * vw[VT_OU + 2] + fv * vw[VT_OV + 2];
        double dx = vw[VT_D00 + 0] + fu * vw[VT_DU + 0] + fv * vw[VT_DV + 0];
        double dy = vw[VT_D00 + 1] + fu * vw[VT_DU + 1] + fv * vw[VT_DV + 1];
        double dz = vw[VT_D00 + 2] + fu * vw[VT_DU + 2] + fv * vw[VT_DV + 2];
        const size_t ray = ((size_t)view * a.U + u) * a.V + v;
        using WT = typename std::conditional<MODE == RM_ATOMIC_BP, double, float>::type;
        Walk<WT> w;
        float chord = 0.f;
        bool hit = false;
        if (MODE != RM_PROJECT && MODE != RM_RESIDUAL)
            hit = make_walk<WT>(ox, oy, oz, dx, dy, dz, vw[VT_TMIN], vw[VT_TMAX], a.W, a.H, a.D, a.W,
                                a.W * a.H, a.spx, a.spy, a.spz, w, chord);
        if (MODE == RM_PROJECT || MODE == RM_RESIDUAL) {
            float acc = 0.f;
            double tin, tout;
            if (clip_ray(ox, oy, oz, dx, dy, dz, vw[VT_TMIN], vw[VT_TMAX], a.W, a.H, a.D, tin, tout)) {
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.vol, a.vol_bytes);
                walk_chunked(ox, oy, oz, dx, dy, dz, tin, tout, a.W, a.H, a.D, a.W, a.W * a.H, a.spx,
                             a.spy, a.spz,
                             [&](int idx, float len) { acc = fmaf(len, load_f32(rs, idx * 4), acc); });
            }
            if (MODE == RM_PROJECT) {
                a.out[ray] = acc;
            } else {
                a.out[ray] = a.rinv[ray] * (a.sino[ray] - acc);
            }
        } else if (MODE == RM_ROWINV) {
            // (A 1)_i is the ray's chord through the whole volume
            float r = (hit && chord > 0.f) ? 1.0f / chord : 0.f;
            a.out[ray] = isfinite(r) ? r : 0.f;
        } else if (MODE == RM_COUNT) {
            // cells visited = plane crossings + 1, from the float64 entry and exit
            // cells (each crossing starts a new cell; exact ties would add empty ones)
            const uint32_t c = hit ? (uint32_t)(w.ncross + 1) : 0u;
            if (a.counts) a.counts[ray] = c;
            my_count = c;
        } else if (MODE == RM_ATOMIC_BP) {
            const float y = a.sino[ray];
            if (hit && y != 0.f) {
                float *vol = a.out;
                walk(w, [&](int idx, WT len) {
                    if (len > (WT)0) atomicAdd(vol + idx, (float)len * y);
                });
            }
        }
    }
    if (MODE == RM_COUNT) {
        // wave reduction then one 64-bit atomic per wave
        unsigned long long c = my_count;
        for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
        if (lane == 0 && c) atomicAdd(a.total, c);
    }
}

// ---------------------------------------------------------------------------
// brick-binned adjoint
// ---------------------------------------------------------------------------
//
// One workgroup owns one brick of BX x BY x BZ voxels and keeps its partial
// sums in LDS.  The waves of the workgroup take the views in turn; for its view a
// wave projects the brick's 8 corners onto the detector (their bounding box holds
// every pixel whose ray meets the brick), then walks each of those rays through the
// brick only, adding length * y into LDS.  After all views the brick is written
// once: no global atomics (the order of the LDS adds still varies between runs).
//
// Each ray is re-expressed per (view, brick) around the plane through the brick
// centre parallel to the detector: for a flat detector the point where pixel
// (u, v)'s ray meets that plane is affine in (u, v), so it is formed in float32
// from a float64 anchor at the footprint's first pixel plus small integer offsets;
// positions inside the walk then stay within tens of voxels of the brick and keep
// float32 resolution near 1e-6 voxel.

enum BrickMode : int { BM_BACKPROJECT = 0, BM_SIRT_UPDATE = 1, BM_COLINV = 2 };

struct BrickArgs {
    const double *views;
    const float *sino;        // BM_BACKPROJECT, BM_SIRT_UPDATE
    float *vol;               // output (BM_SIRT_UPDATE: x, read-modify-write; BM_COLINV: col_inv)
    const float *cinv;        // BM_SIRT_UPDATE
    float relax;
    int W, H, D, U, V, n_views;
    double spx, spy, spz;
    int nbx, nby, nbz, n_blocks;
};

template <int BX, int BY, int BZ, int NT, int MODE>
__global__ __launch_bounds__(NT) void brick_kernel(BrickArgs a) {
    constexpr int LSY = BX + 1;           // padded LDS strides: rays of a wave that
    constexpr int LSZ = LSY * BY + 1;     // differ only in y or z hit different banks
    constexpr int LN = LSZ * BZ;
    constexpr int NWAVES = NT / 64;
    __shared__ float acc[LN];
    for (int i = threadIdx.x; i < LN; i += NT) acc[i] = 0.f;
    __syncthreads();

    const int blk = xcd_remap(blockIdx.x, a.n_blocks);
    const int bxi = blk % a.nbx;
    const int byi = (blk / a.nbx) % a.nby;
    const int bzi = blk / (a.nbx * a.nby);
    const int x0 = bxi * BX, y0 = byi * BY, z0 = bzi * BZ;
    const int ex = min(BX, a.W - x0), ey = min(BY, a.H - y0), ez = min(BZ, a.D - z0);
    const double cbx = x0 + 0.5 * ex, cby = y0 + 0.5 * ey, cbz = z0 + 0.5 * ez;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const bool two_d = (a.D == 1 && a.V == 1);

    for (int view = wv; view < a.n_views; view += NWAVES) {
        const double *vw = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
        // ---- footprint: project corner (lane & 7) of the brick ----
        const int c = lane & 7;
        const double X = (c & 1) ? x0 + ex : x0;
        const double Y = (c & 2) ? y0 + ey : y0;
        const double Z = (c & 4) ? z0 + ez : z0;
        const double rx = X - vw[VT_O00 + 0], ry = Y - vw[VT_O00 + 1], rz = Z - vw[VT_O00 + 2];
        const double al = vw[VT_MINV + 0] * rx + vw[VT_MINV + 1] * ry + vw[VT_MINV + 2] * rz;
        const double be = vw[VT_MINV + 3] * rx + vw[VT_MINV + 4] * ry + vw[VT_MINV + 5] * rz;
        const double ga = vw[VT_MINV + 6] * rx + vw[VT_MINV + 7] * ry + vw[VT_MINV + 8] * rz;
        const bool persp = vw[VT_PERSP] != 0.0;
        float cu, cvv;
        int bad = 0;
        if (persp) {
            bad = !(al > 1e-9);
            cu = bad ? 0.f : (float)(be / al);
            cvv = bad ? 0.f : (float)(ga / al);
        } else {
            cu = (float)be;
            cvv = (float)ga;
        }
        float umin = cu, umax = cu, vmin = cvv, vmax = cvv;
        for (int off = 1; off < 8; off <<= 1) {
            umin = fminf(umin, __shfl_xor(umin, off));
            umax = fmaxf(umax, __shfl_xor(umax, off));
            vmin = fminf(vmin, __shfl_xor(vmin, off));
            vmax = fmaxf(vmax, __shfl_xor(vmax, off));
            bad |= __shfl_xor(bad, off);
        }
        int u0, u1, v0, v1;
        if (bad) {
            u0 = 0; u1 = a.U - 1; v0 = 0; v1 = a.V - 1;
        } else {
            // guard the float conversions against far-away projections
            umin = fmaxf(umin, -1.f); umax = fminf(umax, (float)a.U);
            vmin = fmaxf(vmin, -1.f); vmax = fminf(vmax, (float)a.V);
            u0 = max(0, (int)ceilf(umin - 1e-3f));
            u1 = min(a.U - 1, (int)floorf(umax + 1e-3f));
            v0 = max(0, (int)ceilf(vmin - 1e-3f));
            v1 = min(a.V - 1, (int)floorf(vmax + 1e-3f));
        }
        if (two_d) { v0 = 0; v1 = 0; }
        if (u0 > u1 || v0 > v1) continue;
        const int nfu = u1 - u0 + 1, nfv = v1 - v0 + 1;
        const int nrays = nfu * nfv;
        const float inv_nfv = 1.0f / (float)nfv;

        // ---- per (view, brick) ray parametrisation, anchored at (u0, v0) ----
        const double nx_ = vw[VT_N + 0], ny_ = vw[VT_N + 1], nz_ = vw[VT_N + 2];
        const double fu0 = u0, fv0 = v0;
        // origin and direction of the anchor pixel's ray
        const double aox = vw[VT_O00 + 0] + fu0 * vw[VT_OU + 0] + fv0 * vw[VT_OV + 0];
        const double aoy = vw[VT_O00 + 1] + fu0 * vw[VT_OU + 1] + fv0 * vw[VT_OV + 1];
        const double aoz = vw[VT_O00 + 2] + fu0 * vw[VT_OU + 2] + fv0 * vw[VT_OV + 2];
        const double adx = vw[VT_D00 + 0] + fu0 * vw[VT_DU + 0] + fv0 * vw[VT_DV + 0];
        const double ady = vw[VT_D00 + 1] + fu0 * vw[VT_DU + 1] + fv0 * vw[VT_DV + 1];
        const double adz = vw[VT_D00 + 2] + fu0 * vw[VT_DU + 2] + fv0 * vw[VT_DV + 2];
        // Dir . N is the same for every pixel of a flat detector
        const double tb = ((cbx - aox) * nx_ + (cby - aoy) * ny_ + (cbz - aoz) * nz_) /
                          (adx * nx_ + ady * ny_ + adz * nz_);
        const float A0x = (float)(aox + tb * adx - x0);
        const float A0y = (float)(aoy + tb * ady - y0);
        const float A0z = (float)(aoz + tb * adz - z0);
        const float Aux = (float)(vw[VT_OU + 0] + tb * vw[VT_DU + 0]);
        const float Auy = (float)(vw[VT_OU + 1] + tb * vw[VT_DU + 1]);
        const float Auz = (float)(vw[VT_OU + 2] + tb * vw[VT_DU + 2]);
        const float Avx = (float)(vw[VT_OV + 0] + tb * vw[VT_DV + 0]);
        const float Avy = (float)(vw[VT_OV + 1] + tb * vw[VT_DV + 1]);
        const float Avz = (float)(vw[VT_OV + 2] + tb * vw[VT_DV + 2]);
        const float Dx = (float)adx, Dy = (float)ady, Dz = (float)adz;
        const float DUx = (float)vw[VT_DU + 0], DUy = (float)vw[VT_DU + 1], DUz = (float)vw[VT_DU + 2];
        const float DVx = (float)vw[VT_DV + 0], DVy = (float)vw[VT_DV + 1], DVz = (float)vw[VT_DV + 2];
        const float t0 = (float)(vw[VT_TMIN] - tb), t1 = (float)(vw[VT_TMAX] - tb);
        const float spx = (float)a.spx, spy = (float)a.spy, spz = (float)a.spz;
        const float fex = (float)ex, fey = (float)ey, fez = (float)ez;
        const float *ysrc = a.sino + ((size_t)view * a.U + u0) * a.V + v0;

        for (int r = lane; r < nrays; r += 64) {
            int iu = (int)(((float)r + 0.5f) * inv_nfv);
            int iv = r - iu * nfv;
            if (iv < 0) { iu -= 1; iv += nfv; } else if (iv >= nfv) { iu += 1; iv -= nfv; }
            float yv;
            if (MODE == BM_COLINV) {
                yv = 1.f;
            } else {
                yv = ysrc[(size_t)iu * a.V + iv];
                if (yv == 0.f) continue;
            }
            const float fu = (float)iu, fv = (float)iv;
            const float ox = fmaf(fv, Avx, fmaf(fu, Aux, A0x));
            const float oy = fmaf(fv, Avy, fmaf(fu, Auy, A0y));
            const float oz = fmaf(fv, Avz, fmaf(fu, Auz, A0z));
            float dx = fmaf(fv, DVx, fmaf(fu, DUx, Dx));
            float dy = fmaf(fv, DVy, fmaf(fu, DUy, Dy));
            float dz = fmaf(fv, DVz, fmaf(fu, DUz, Dz));
            {
                const float dm = fmaxf(fabsf(dx), fmaxf(fabsf(dy), fabsf(dz))) * 0x1p-40f;
                if (fabsf(dx) < dm) dx = 0.f;
                if (fabsf(dy) < dm) dy = 0.f;
                if (fabsf(dz) < dm) dz = 0.f;
            }
            // clip to the brick [0,ex) x [0,ey) x [0,ez) and to [t0, t1]
            float tin = t0, tout = t1;
            bool hit = true;
            float ix_ = 0.f, iy_ = 0.f, iz_ = 0.f;
            if (dx != 0.f) {
                ix_ = 1.0f / dx;
                float a0 = -ox * ix_, a1 = (fex - ox) * ix_;
                tin = fmaxf(tin, fminf(a0, a1));
                tout = fminf(tout, fmaxf(a0, a1));
            } else {
                hit = hit && ox >= 0.f && ox < fex;
            }
            if (dy != 0.f) {
                iy_ = 1.0f / dy;
                float a0 = -oy * iy_, a1 = (fey - oy) * iy_;
                tin = fmaxf(tin, fminf(a0, a1));
                tout = fminf(tout, fmaxf(a0, a1));
            } else {
                hit = hit && oy >= 0.f && oy < fey;
            }
            if (dz != 0.f) {
                iz_ = 1.0f / dz;
                float a0 = -oz * iz_, a1 = (fez - oz) * iz_;
                tin = fmaxf(tin, fminf(a0, a1));
                tout = fminf(tout, fmaxf(a0, a1));
            } else {
                hit = hit && oz >= 0.f && oz < fez;
            }
            if (!(hit && tout > tin)) continue;
            // entry / exit cells and crossing counts per axis
            const float px = dx * spx, py = dy * spy, pz = dz * spz;
            const float L = sqrtf(px * px + py * py + pz * pz);
            int cx, cy, cz, nxc, nyc, nzc;
            float l0x, l0y, l0z, qx, qy, qz;
            float lend = (tout - tin) * L;
            auto axis = [&](float o, float d, float inv, int n, int &c0, int &ncr, float &l0,
                            float &q) {
                const float e = fmaf(tin, d, o), xx = fmaf(tout, d, o);
                int ce, ce2;
                if (d > 0.f) { ce = (int)floorf(e); ce2 = (int)ceilf(xx) - 1; }
                else if (d < 0.f) { ce = (int)ceilf(e) - 1; ce2 = (int)floorf(xx); }
                else { ce = (int)floorf(e); ce2 = ce; }
                ce = min(max(ce, 0), n - 1);
                ce2 = min(max(ce2, 0), n - 1);
                c0 = ce;
                if (d != 0.f) {
                    ncr = d > 0.f ? max(ce2 - ce, 0) : max(ce - ce2, 0);
                    q = L * fabsf(inv);
                    const float dist = d > 0.f ? (float)(ce + 1) - e : e - (float)ce;
                    l0 = dist * q;
                    lend = fminf(lend, fmaf((float)ncr, q, l0));
                } else {
                    ncr = 0;
                    q = 0.f;
                    l0 = CT_INF;
                }
            };
            axis(ox, dx, ix_, ex, cx, nxc, l0x, qx);
            axis(oy, dy, iy_, ey, cy, nyc, l0y, qy);
            axis(oz, dz, iz_, ez, cz, nzc, l0z, qz);
            Walk<float> w;
            w.idx = cz * LSZ + cy * LSY + cx;
            w.stx = dx > 0.f ? 1 : -1;
            w.sty = dy > 0.f ? LSY : -LSY;
            w.stz = dz > 0.f ? LSZ : -LSZ;
            w.l0x = l0x; w.l0y = l0y; w.l0z = l0z;
            w.qx = qx; w.qy = qy; w.qz = qz;
            w.lend = lend;
            walk(w, [&](int idx, float len) {
                if (len > 0.f) atomicAdd(&acc[idx], len * yv);
            });
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BX * BY * BZ; i += NT) {
        const int lx = i % BX, ly = (i / BX) % BY, lz = i / (BX * BY);
        if (lx < ex && ly < ey && lz < ez) {
            const size_t g = ((size_t)(z0 + lz) * a.H + (y0 + ly)) * a.W + (x0 + lx);
            const float val = acc[lz * LSZ + ly * LSY + lx];
            if (MODE == BM_BACKPROJECT) {
                a.vol[g] = val;
            } else if (MODE == BM_SIRT_UPDATE) {
                a.vol[g] = fmaf(a.relax * a.cinv[g], val, a.vol[g]);
            } else {
                const float r = val > 0.f ? 1.0f / val : 0.f;
                a.vol[g] = isfinite(r) ? r : 0.f;
            }
        }
    }
}

__global__ void fill_kernel(float *p, size_t n, float v) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

__global__ void zero_u64_kernel(unsigned long long *p) { *p = 0ull; }

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static RayArgs ray_args(const LaunchGeom &g) {
    RayArgs a{};
    a.views = g.views;
    a.W = g.W; a.H = g.H; a.D = g.D; a.U = g.U; a.V = g.V; a.n_views = g.n_views;
    a.spx = g.spx; a.spy = g.spy; a.spz = g.spz;
    if (g.two_d) {
        a.n_utiles = (g.U + 255) / 256;
        a.n_vtiles = 1;
    } else {
        a.n_utiles = (g.U + 15) / 16;
        a.n_vtiles = (g.V + 15) / 16;
    }
    a.n_blocks = a.n_utiles * a.n_vtiles * g.n_views;
    a.vol_bytes = (uint32_t)((size_t)g.W * g.H * g.D * 4);
    return a;
}

template <int MODE>
static hipError_t launch_ray(const LaunchGeom &g, RayArgs a, hipStream_t s) {
    if (g.two_d)
        hipLaunchKernelGGL((ray_kernel<MODE, true>), dim3(a.n_blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((ray_kernel<MODE, false>), dim3(a.n_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill(float *p, size_t n, float v, hipStream_t s) {
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

hipError_t launch_project(const LaunchGeom &g, const float *vol, float *sino, hipStream_t s) {
    RayArgs a = ray_args(g);
    a.vol = vol;
    a.out = sino;
    return launch_ray<RM_PROJECT>(g, a, s);
}

hipError_t launch_residual(const LaunchGeom &g, const float *x, const float *y, const float *rinv,
                           float *e, hipStream_t s) {
    RayArgs a = ray_args(g);
    a.vol = x;
    a.sino = y;
    a.rinv = rinv;
    a.out = e;
    return launch_ray<RM_RESIDUAL>(g, a, s);
}

hipError_t launch_rowinv(const LaunchGeom &g, float *rinv, hipStream_t s) {
    RayArgs a = ray_args(g);
    a.out = rinv;
    return launch_ray<RM_ROWINV>(g, a, s);
}

hipError_t launch_count(const LaunchGeom &g, uint32_t *per_ray, unsigned long long *total,
                        hipStream_t s) {
    hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    RayArgs a = ray_args(g);
    a.counts = per_ray;
    a.total = total;
    return launch_ray<RM_COUNT>(g, a, s);
}

hipError_t launch_backproject_atomic(const LaunchGeom &g, const float *sino, float *vol,
                                     hipStream_t s) {
    hipError_t e = launch_fill(vol, (size_t)g.W * g.H * g.D, 0.f, s);
    if (e != hipSuccess) return e;
    RayArgs a = ray_args(g);
    a.sino = sino;
    a.out = vol;
    return launch_ray<RM_ATOMIC_BP>(g, a, s);
}

// Brick shapes: 3D 16 x 16 x 16 voxels with 4 waves; 2D 64 x 64 pixels with 4 waves.
template <int MODE>
static hipError_t launch_brick(const LaunchGeom &g, const float *sino, float *vol,
                               const float *cinv, float relax, hipStream_t s) {
    BrickArgs a{};
    a.views = g.views;
    a.sino = sino;
    a.vol = vol;
    a.cinv = cinv;
    a.relax = relax;
    a.W = g.W; a.H = g.H; a.D = g.D; a.U = g.U; a.V = g.V; a.n_views = g.n_views;
    a.spx = g.spx; a.spy = g.spy; a.spz = g.spz;
    if (g.two_d) {
        constexpr int BX = 64, BY = 64, BZ = 1, NT = 256;
        a.nbx = (g.W + BX - 1) / BX; a.nby = (g.H + BY - 1) / BY; a.nbz = 1;
        a.n_blocks = a.nbx * a.nby * a.nbz;
        hipLaunchKernelGGL((brick_kernel<BX, BY, BZ, NT, MODE>), dim3(a.n_blocks), dim3(NT), 0, s, a);
    } else {
        constexpr int BX = 16, BY = 16, BZ = 16, NT = 256;
        a.nbx = (g.W + BX - 1) / BX; a.nby = (g.H + BY - 1) / BY; a.nbz = (g.D + BZ - 1) / BZ;
        a.n_blocks = a.nbx * a.nby * a.nbz;
        hipLaunchKernelGGL((brick_kernel<BX, BY, BZ, NT, MODE>), dim3(a.n_blocks), dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_backproject(const LaunchGeom &g, const float *sino, float *vol, hipStream_t s) {
    return launch_brick<BM_BACKPROJECT>(g, sino, vol, nullptr, 0.f, s);
}

hipError_t launch_sirt_update(const LaunchGeom &g, const float *e, const float *cinv, float relax,
                              float *x, hipStream_t s) {
    return launch_brick<BM_SIRT_UPDATE>(g, e, x, cinv, relax, s);
}

hipError_t launch_colinv(const LaunchGeom &g, float *cinv, hipStream_t s) {
    return launch_brick<BM_COLINV>(g, nullptr, cinv, nullptr, 0.f, s);
}

}  // namespace ctp
