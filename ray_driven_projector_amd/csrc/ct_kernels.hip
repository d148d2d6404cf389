// ct_kernels.hip -- gfx950 kernels of the ray-driven projector pair.
//
// Operator (diffct documentation, "Differentiable analytical reconstruction"):
// the cell-constant Siddon forward projector A, a_ij = length of ray i inside
// voxel j, and its matched adjoint A^T.  Siddon's observation is used in both
// directions: along a ray the cell boundaries are the planes of the three lattice
// axes, so the ray's parameter interval inside the volume is cut at each plane
// crossing and each piece lies in exactly one cell.
//
// Walk.  The pieces of a ray are enumerated by an integer fixed-point walk: the
// positions of the next crossing on each axis are unsigned 32-bit multiples of a
// walk unit (forward: about 1e-9 of the walk's length; brick adjoint: just under
// 2^-23 of a voxel diagonal).  The m-th crossing of axis a is
// l0_a + m q_a, formed by exact (saturating) integer adds, so nothing drifts; the
// walk ends at
//   l_end = min(chord, min_a (l0_a + N_a q_a)),
// N_a being the number of planes of axis a crossed inside the interval (from
// float64 or float32 entry/exit cells).  Any crossing taken before l_end is
// therefore one of the N_a real crossings of its axis, so cell indices never leave
// the volume or the brick, whatever the rounding of the set-up.
//
// Precision.  The forward gather sets each ray up in float64 and re-bases the walk
// every 64 (fan/cone) or 128 (parallel) cells of the major axis, so every piece
// length is resolved to better than 1e-5 of a cell.  The brick adjoint sets each ray up in float32 in
// brick-local coordinates (positions within tens of voxels) and sums exact
// integer products, so its result does not depend on the order of the adds.
// The atomic adjoint keeps a float64 walk.
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

// Out-of-range offsets (including negative ones, seen as huge unsigned values)
// read 0 through a buffer resource.
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}

__device__ __forceinline__ uint32_t umin3(uint32_t a, uint32_t b, uint32_t c) { return min(min(a, b), c); }

// Wave-uniform values: keep them in scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ double uni(double x) {
    const long long b = __builtin_bit_cast(long long, x);
    const int lo = __builtin_amdgcn_readfirstlane((int)(b & 0xFFFFFFFFll)), hi = __builtin_amdgcn_readfirstlane((int)(b >> 32));
    return __builtin_bit_cast(double, (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
// The opposite: hold a value in a vector register.  A loop that selects among
// wave-uniform operands with a per-lane mask needs them in vector registers
// (one scalar operand per instruction); held there, the copies stay out of the loop.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
    asm("" : "+v"(x));
    return x;
}

// Non-negative float64 to fixed point, saturating.
__device__ __forceinline__ uint32_t fix64(double x) {
    return (uint32_t)fmin(x + 0.5, 4294967295.0);
}

// Non-negative float32 to fixed point, saturating (INF -> 0xFFFFFFFF).
__device__ __forceinline__ uint32_t fix32(float x) { return (uint32_t)fminf(x, 4294967040.f); }

// l0 + n q, saturating at 0xFFFFFFFF.
__device__ __forceinline__ uint32_t last_plus_one(uint32_t l0, uint32_t n, uint32_t q) {
    const unsigned long long t = (unsigned long long)n * q + l0;
    return (t >> 32) ? 0xFFFFFFFFu : (uint32_t)t;
}

// ---------------------------------------------------------------------------
// float64 ray set-up
// ---------------------------------------------------------------------------

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

// The coordinate (in cells) of a ray on an axis it never crosses.  A ray lying
// in a lattice plane belongs to the cell above it; the frames' arithmetic puts
// such a ray a few ulps either side of the plane, so a coordinate within 2^-30
// cell of a plane is taken to lie on it.  Every path (forward, packets, both
// adjoints, counts) decides these cells from this value, so A and A^T agree on
// such rays.
__device__ __forceinline__ double on_plane(double o) {
    const double r = rint(o);
    return fabs(o - r) < 0x1p-30 ? r : o;
}

// Drop direction components below 2^-40 of the largest (they move the ray by
// less than 1e-12 of its length along that axis: the ray is then parallel to
// those planes), settle the origin on those axes (on_plane), and clip to the
// volume box.  Returns false on a miss.
__device__ __forceinline__ bool clip_ray(double &ox, double &oy, double &oz, double &dx, double &dy,
                                         double &dz, double tmin, double tmax, int nx, int ny,
                                         int nz, double &tin, double &tout) {
    const double dm = fmax(fabs(dx), fmax(fabs(dy), fabs(dz))) * 0x1p-40;
    if (fabs(dx) < dm) { dx = 0.0; ox = on_plane(ox); }
    if (fabs(dy) < dm) { dy = 0.0; oy = on_plane(oy); }
    if (fabs(dz) < dm) { dz = 0.0; oz = on_plane(oz); }
    tin = tmin;
    tout = tmax;
    bool hit = true;
    clip_axis(ox, dx, (double)nx, tin, tout, hit);
    clip_axis(oy, dy, (double)ny, tin, tout, hit);
    clip_axis(oz, dz, (double)nz, tin, tout, hit);
    return hit && (tout > tin);
}

// ---------------------------------------------------------------------------
// float64 walk (atomic adjoint) -- same plan as the integer walk, in doubles
// ---------------------------------------------------------------------------

struct DWalk {
    int idx;            // element index of the current cell
    int stx, sty, stz;  // signed element strides
    int ncross;         // plane crossings inside the interval (all axes)
    double l0x, l0y, l0z, qx, qy, qz, lend;
};

__device__ __forceinline__ void daxis(double d, double L, int n, double dist, double &q,
                                      double &l0, double &lend) {
    if (d != 0.0) {
        q = L / fabs(d);
        l0 = dist * q;
        lend = fmin(lend, fma((double)n, q, l0));
    } else {
        q = 0.0;
        l0 = __builtin_huge_val();
    }
}

__device__ __forceinline__ bool make_dwalk(double ox, double oy, double oz, double dx, double dy,
                                           double dz, double tmin, double tmax, int nx, int ny,
                                           int nz, double spx, double spy, double spz, DWalk &w,
                                           double &chord) {
    double tin, tout;
    if (!clip_ray(ox, oy, oz, dx, dy, dz, tmin, tmax, nx, ny, nz, tin, tout)) return false;
    int cx, cy, cz, nxc, nyc, nzc;
    double ddx, ddy, ddz;
    axis_cells(ox, dx, tin, tout, nx, cx, nxc, ddx);
    axis_cells(oy, dy, tin, tout, ny, cy, nyc, ddy);
    axis_cells(oz, dz, tin, tout, nz, cz, nzc, ddz);
    const double px = dx * spx, py = dy * spy, pz = dz * spz;
    const double L = sqrt(px * px + py * py + pz * pz);
    w.idx = (cz * ny + cy) * nx + cx;
    w.ncross = nxc + nyc + nzc;
    w.stx = dx > 0.0 ? 1 : -1;
    w.sty = dy > 0.0 ? nx : -nx;
    w.stz = dz > 0.0 ? nx * ny : -nx * ny;
    chord = (tout - tin) * L;
    w.lend = chord;
    daxis(dx, L, nxc, ddx, w.qx, w.l0x, w.lend);
    daxis(dy, L, nyc, ddy, w.qy, w.l0y, w.lend);
    daxis(dz, L, nzc, ddz, w.qz, w.l0z, w.lend);
    return true;
}

template <class F>
__device__ __forceinline__ void dwalk(const DWalk &w, F &&f) {
    int idx = w.idx;
    double lc = 0.0, mx = 0.0, my = 0.0, mz = 0.0;
    double lx = w.l0x, ly = w.l0y, lz = w.l0z;
    for (;;) {
        const double tmin = fmin(fmin(lx, ly), lz);
        const double tn = fmin(tmin, w.lend);
        f(idx, tn - lc);
        if (!(tmin < w.lend)) break;  // also leaves on NaN
        lc = tn;
        if (lx == tmin) { idx += w.stx; mx += 1.0; lx = fma(mx, w.qx, w.l0x); }
        if (ly == tmin) { idx += w.sty; my += 1.0; ly = fma(my, w.qy, w.l0y); }
        if (lz == tmin) { idx += w.stz; mz += 1.0; lz = fma(mz, w.qz, w.l0z); }
    }
}

// ---------------------------------------------------------------------------
// parameterized detector surfaces
// ---------------------------------------------------------------------------

// Per-pixel local offsets (o_u, o_v, o_n) of a detector surface, shared by the
// views (U, V, 3) or per view (views, U, V, 3), float64.
struct Surface {
    const double *off;   // null: flat detector
    int per_view;
};

// Voxel-coordinate point of pixel (u, v) on the surface of a view:
// C + o_u EU + o_v EV + o_n EN.
__device__ __forceinline__ void surface_point(const double *vw, const Surface &sf, int view, int u,
                                              int v, int U, int V, double &px, double &py,
                                              double &pz) {
    const double *o = sf.off + 3 * ((sf.per_view ? (size_t)view * U * V : 0) + (size_t)u * V + v);
    const double ou = o[0], ov = o[1], on = o[2];
    px = vw[VT_C + 0] + ou * vw[VT_EU + 0] + ov * vw[VT_EV + 0] + on * vw[VT_EN + 0];
    py = vw[VT_C + 1] + ou * vw[VT_EU + 1] + ov * vw[VT_EV + 1] + on * vw[VT_EN + 1];
    pz = vw[VT_C + 2] + ou * vw[VT_EU + 2] + ov * vw[VT_EV + 2] + on * vw[VT_EN + 2];
}

// Coordinate k of the origin of flat-detector pixel (u, v), in voxel
// coordinates: one fixed sequence of two fused multiply-adds, so every kernel
// that needs it gets the same bits.
__device__ __forceinline__ double pixel_origin(const double *vw, int k, int u, int v) {
    return fma((double)v, vw[VT_OV + k], fma((double)u, vw[VT_OU + k], vw[VT_O00 + k]));
}

// Ray of pixel (u, v): origin and direction in voxel coordinates (flat detector:
// the affine table; surface: the source or the pixel's surface point).
__device__ __forceinline__ void pixel_ray(const double *vw, const Surface &sf, int view, int u, int v,
                                          int U, int V, double &ox, double &oy, double &oz,
                                          double &dx, double &dy, double &dz) {
    if (!sf.off) {
        const double fu = (double)u, fv = (double)v;
        ox = pixel_origin(vw, 0, u, v);
        oy = pixel_origin(vw, 1, u, v);
        oz = pixel_origin(vw, 2, u, v);
        dx = vw[VT_D00 + 0] + fu * vw[VT_DU + 0] + fv * vw[VT_DV + 0];
        dy = vw[VT_D00 + 1] + fu * vw[VT_DU + 1] + fv * vw[VT_DV + 1];
        dz = vw[VT_D00 + 2] + fu * vw[VT_DU + 2] + fv * vw[VT_DV + 2];
        return;
    }
    double px, py, pz;
    surface_point(vw, sf, view, u, v, U, V, px, py, pz);
    if (vw[VT_PERSP] != 0.0) {   // from the source to the surface point
        ox = vw[VT_O00 + 0]; oy = vw[VT_O00 + 1]; oz = vw[VT_O00 + 2];
        dx = px - ox; dy = py - oy; dz = pz - oz;
    } else {                     // through the surface point along the ray direction
        ox = px; oy = py; oz = pz;
        dx = vw[VT_D00 + 0]; dy = vw[VT_D00 + 1]; dz = vw[VT_D00 + 2];
    }
}

// Where each surface pixel's ray crosses the flat detector plane, in flat pixel
// units (the coordinates the brick footprints are computed in), reduced per view
// to monotone envelopes.  Per view, env_size(U, V) floats:
//   colmin[U], colmax[U]               over all v, for each column u
//   then per tile of kEnvTile columns:  rowmin[V], rowmax[V] over the tile's columns
// with the max arrays made running maxima and the min arrays running minima from
// the right.  A brick whose flat footprint is [a, b] x [c, d] can only be seen by
// columns u with colmax[u] >= a and colmin[u] <= b, and, within a column tile,
// by rows v with rowmax[v] >= c and rowmin[v] <= d: index ranges found by binary
// search.  Per-tile rows keep the v range tight where the surface's flat v
// depends on u (a cylinder's does, by 1 / cos of the fan angle).
constexpr int kEnvTile = 16;
__host__ __device__ inline size_t env_size(int U, int V) {
    return 2 * (size_t)U + (size_t)((U + kEnvTile - 1) / kEnvTile) * 2 * V;
}
__global__ __launch_bounds__(256) void surface_env_kernel(const double *views, Surface sf, int U,
                                                          int V, float *env,
                                                          unsigned long long *bad) {
    const int view = blockIdx.x;
    const double *vw = views + (size_t)view * CT_VIEW_TABLE_STRIDE;
    float *e = env + (size_t)view * env_size(U, V);
    const int nt = (U + kEnvTile - 1) / kEnvTile;
    const bool persp = vw[VT_PERSP] != 0.0;
    auto flat = [&](int u, int v, float &fu, float &fv) {
        double px, py, pz;
        surface_point(vw, sf, view, u, v, U, V, px, py, pz);
        const double rx = px - vw[VT_O00 + 0], ry = py - vw[VT_O00 + 1], rz = pz - vw[VT_O00 + 2];
        const double al = vw[VT_MINV + 0] * rx + vw[VT_MINV + 1] * ry + vw[VT_MINV + 2] * rz;
        const double be = vw[VT_MINV + 3] * rx + vw[VT_MINV + 4] * ry + vw[VT_MINV + 5] * rz;
        const double ga = vw[VT_MINV + 6] * rx + vw[VT_MINV + 7] * ry + vw[VT_MINV + 8] * rz;
        // a fan/cone pixel must lie in front of the source (its ray crosses the
        // flat detector plane at a positive parameter)
        if (persp && !(al > 1e-9)) atomicOr(bad, 1ull);
        fu = (float)(persp ? be / al : be);
        fv = (float)(persp ? ga / al : ga);
    };
    for (int u = threadIdx.x; u < U; u += 256) {
        float lo = 3e38f, hi = -3e38f;
        for (int v = 0; v < V; ++v) {
            float fu, fv;
            flat(u, v, fu, fv);
            lo = fminf(lo, fu);
            hi = fmaxf(hi, fu);
        }
        e[u] = lo;
        e[U + u] = hi;
    }
    for (int k = threadIdx.x; k < nt * V; k += 256) {
        const int t = k / V, v = k - t * V;
        float lo = 3e38f, hi = -3e38f;
        for (int u = t * kEnvTile; u < min(U, (t + 1) * kEnvTile); ++u) {
            float fu, fv;
            flat(u, v, fu, fv);
            lo = fminf(lo, fv);
            hi = fmaxf(hi, fv);
        }
        float *r = e + 2 * U + (size_t)t * 2 * V;
        r[v] = lo;
        r[V + v] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int u = 1; u < U; ++u) e[U + u] = fmaxf(e[U + u], e[U + u - 1]);
        for (int u = U - 2; u >= 0; --u) e[u] = fminf(e[u], e[u + 1]);
    }
    for (int t = threadIdx.x; t < nt; t += 256) {
        float *r = e + 2 * U + (size_t)t * 2 * V;
        for (int v = 1; v < V; ++v) r[V + v] = fmaxf(r[V + v], r[V + v - 1]);
        for (int v = V - 2; v >= 0; --v) r[v] = fminf(r[v], r[v + 1]);
    }
}

// First index i in [0, n) with a[i] >= x (GT: a[i] > x), n if none; a
// non-decreasing, wave-uniform arguments, called by the whole wave.  A 64-way
// search: every lane probes the start of one of 64 chunks and a ballot picks
// the chunk holding the first hit, so n <= 4096 takes two rounds of loads
// (a binary search would take twelve dependent ones).
template <bool GT>
__device__ __forceinline__ int first_hit(const float *a, int n, float x, int lane) {
    int lo = 0, len = n;   // the first hit lies in [lo, lo + len], lo + len meaning none
    while (len > 64) {
        const int step = (len + 63) >> 6;
        const int i = lo + lane * step;
        const bool in = i < lo + len;
        const float ai = a[in ? i : 0];   // n >= 1: index 0 is always there
        const uint64_t hit = __ballot(in && (GT ? ai > x : ai >= x));
        const int nprobe = (len + step - 1) / step;   // lanes that probed
        if (hit == 0ull) {
            const int last = lo + (nprobe - 1) * step;   // every probe missed
            len = lo + len - (last + 1);
            lo = last + 1;
        } else {
            const int L = __ffsll((unsigned long long)hit) - 1;
            const int hi = lo + L * step;                // a hit; the one before missed
            const int nlo = L == 0 ? lo : lo + (L - 1) * step + 1;
            len = hi - nlo;
            lo = nlo;
            if (len == 0) return lo;
        }
    }
    const int i = lo + lane;
    const bool in = lane < len;
    const float ai = a[in ? i : 0];
    const uint64_t hit = __ballot(in && (GT ? ai > x : ai >= x));
    return hit == 0ull ? lo + len : lo + __ffsll((unsigned long long)hit) - 1;
}

// ---------------------------------------------------------------------------
// integer walk
// ---------------------------------------------------------------------------

struct IWalk {
    uint32_t idx;           // byte offset of the current cell
    uint32_t stx, sty, stz; // byte strides (two's complement for negative steps)
    uint32_t lx, ly, lz;    // next crossing per axis (0xFFFFFFFF: none)
    uint32_t qx, qy, qz;    // crossing spacing per axis
    uint32_t lend;          // end of the walk
};

// One step of the gather walk: advance past the current piece, returning its
// length and the byte offset of the next cell.
struct GStep {
    uint32_t seg;
    bool last;
};
// Exactly one axis steps per call, the first of x, y, z whose next crossing is
// the minimum; where planes are crossed at the same point the next call takes
// the other axis after a piece of length 0.
__device__ __forceinline__ GStep gstep(const IWalk &w, uint32_t &idx, uint32_t &lc, uint32_t &lx,
                                       uint32_t &ly, uint32_t &lz) {
    const uint32_t qx = w.qx, qy = w.qy, qz = w.qz, sx = w.stx, sy = w.sty, sz = w.stz;
    const uint32_t tmin = umin3(lx, ly, lz);
    const uint32_t tn = min(tmin, w.lend);
    // the step masks are combined as wave masks, on the scalar unit
    const uint64_t mx = __builtin_amdgcn_ballot_w64(lx == tmin);
    const uint64_t my = __builtin_amdgcn_ballot_w64(ly == tmin) & ~mx;
    const bool bx = __builtin_amdgcn_inverse_ballot_w64(mx);
    const bool by = __builtin_amdgcn_inverse_ballot_w64(my);
    const bool bxy = __builtin_amdgcn_inverse_ballot_w64(mx | my);
    const uint32_t nx = __builtin_elementwise_add_sat(lx, qx);
    const uint32_t ny = __builtin_elementwise_add_sat(ly, qy);
    const uint32_t nz = __builtin_elementwise_add_sat(lz, qz);
    const uint32_t syz = by ? sy : sz;
    lx = bx ? nx : lx;
    ly = by ? ny : ly;
    lz = bxy ? lz : nz;
    idx += bx ? sx : syz;
    GStep g{tn - lc, tmin >= w.lend};
    lc = tn;
    return g;
}

// The same walk for a ray that never crosses the planes of one axis (that
// direction component is 0: the third axis's next crossing stays at 0xFFFFFFFF
// and never is the minimum): the two live axes a and b, in x, y, z order, so
// ties step a first as the three-axis step does, and the pieces and cells are
// the same.
struct IWalk2 {
    uint32_t idx, sa, sb, la, lb, qa, qb, lend;
};
__device__ __forceinline__ IWalk2 live_axes(const IWalk &w, int dead) {
    IWalk2 v;
    v.idx = w.idx;
    v.lend = w.lend;
    v.la = dead == 0 ? w.ly : w.lx;
    v.qa = dead == 0 ? w.qy : w.qx;
    v.sa = dead == 0 ? w.sty : w.stx;
    v.lb = dead == 2 ? w.ly : w.lz;
    v.qb = dead == 2 ? w.qy : w.qz;
    v.sb = dead == 2 ? w.sty : w.stz;
    return v;
}
__device__ __forceinline__ GStep gstep2(const IWalk2 &w, uint32_t &idx, uint32_t &lc, uint32_t &la,
                                        uint32_t &lb) {
    const uint32_t tmin = min(la, lb);
    const uint32_t tn = min(tmin, w.lend);
    const bool ba = la == tmin;
    const uint32_t na = __builtin_elementwise_add_sat(la, w.qa);
    const uint32_t nb = __builtin_elementwise_add_sat(lb, w.qb);
    la = ba ? na : la;
    lb = ba ? lb : nb;
    idx += ba ? w.sa : w.sb;
    GStep g{tn - lc, tmin >= w.lend};
    lc = tn;
    return g;
}

constexpr int kPacket = 4;   // rays per packet (forward and brick adjoint)
// Forward packet blocks (measured on the 512^3 dual-axis SIRT residual):
// 8 waves, each 8 packets along P (one 128-byte line of the volume copy's
// contiguous axis) x 8 rows, so a block takes a tile of 32 x 64 pixels, and
// one tile runs through every view in turn.  8.57 ms; 8.81 with 1024-thread
// blocks of 32 x 128 (one block per CU at 96 VGPRs), 10.6 with 256-thread
// 32 x 32; earlier shapes 12.1 ms with 256-thread 64 x 16, 9.1 with 1024-thread
// 64 x 64, 20.3 with 16 x 256 (half lines); grouping 2 / 4 tiles per view
// 10.7 / 12.9.
constexpr int kPacketTileGroup = 1;
constexpr int kPacketWaves = 8;
constexpr int kPacketLanesP = 8;
constexpr int kPacketTP = kPacketLanesP * kPacket, kPacketTQ = (64 / kPacketLanesP) * kPacketWaves;   // tile

// Sum of length * value over the walk, in walk units.  The cell offsets do not
// depend on the loaded values, so the walk runs ahead of the arithmetic: each
// iteration generates four pieces and has their four gathers in flight before
// the first product is formed.  Steps generated past the end of the walk have
// zero length (their cells may lie outside the volume; the buffer resource reads
// 0 there, and in-volume values are finite, so they add nothing).
__device__ __forceinline__ float iwalk_gather(const IWalk &w, __amdgpu_buffer_rsrc_t rs) {
    uint32_t idx = w.idx;
    uint32_t lc = 0, lx = w.lx, ly = w.ly, lz = w.lz;
    float acc = 0.f;
    float v0 = load_f32(rs, idx);
    for (;;) {
        const GStep s0 = gstep(w, idx, lc, lx, ly, lz);
        const float v1 = load_f32(rs, idx);
        const GStep s1 = gstep(w, idx, lc, lx, ly, lz);
        const float v2 = load_f32(rs, idx);
        const GStep s2 = gstep(w, idx, lc, lx, ly, lz);
        const float v3 = load_f32(rs, idx);
        const GStep s3 = gstep(w, idx, lc, lx, ly, lz);
        acc = fmaf((float)s0.seg, v0, acc);
        acc = fmaf((float)s1.seg, v1, acc);
        acc = fmaf((float)s2.seg, v2, acc);
        v0 = load_f32(rs, idx);
        acc = fmaf((float)s3.seg, v3, acc);
        // the next crossing never moves backwards, so once one step has reached
        // the end every later one has: the fourth step's test covers all four
        if (s3.last) break;
    }
    return acc;
}
__device__ __forceinline__ float iwalk_gather2(const IWalk2 &w, __amdgpu_buffer_rsrc_t rs) {
    uint32_t idx = w.idx;
    uint32_t lc = 0, la = w.la, lb = w.lb;
    float acc = 0.f;
    float v0 = load_f32(rs, idx);
    for (;;) {
        const GStep s0 = gstep2(w, idx, lc, la, lb);
        const float v1 = load_f32(rs, idx);
        const GStep s1 = gstep2(w, idx, lc, la, lb);
        const float v2 = load_f32(rs, idx);
        const GStep s2 = gstep2(w, idx, lc, la, lb);
        const float v3 = load_f32(rs, idx);
        const GStep s3 = gstep2(w, idx, lc, la, lb);
        acc = fmaf((float)s0.seg, v0, acc);
        acc = fmaf((float)s1.seg, v1, acc);
        acc = fmaf((float)s2.seg, v2, acc);
        v0 = load_f32(rs, idx);
        acc = fmaf((float)s3.seg, v3, acc);
        if (s3.last) break;
    }
    return acc;
}

// The two-axis gather for a packet of K rays that share the walk: at every
// piece one gather per ray (ray j's cell is off[j] bytes from the walk's) and
// one sum per ray, each formed exactly as iwalk_gather2 forms it.  CONSEC:
// the rays' cells are consecutive words (off[j] = 4 j), read by one
// K-word load.
template <int K, bool CONSEC>
__device__ __forceinline__ void iwalk_gather2_packet(const IWalk2 &w, __amdgpu_buffer_rsrc_t rs,
                                                     const uint32_t (&off)[K], float (&acc)[K]) {
    uint32_t idx = w.idx;
    uint32_t lc = 0, la = w.la, lb = w.lb;
    float v0[K], v1[K], v2[K], v3[K];
    const auto gather = [&](float (&v)[K]) {
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = load_f32(rs, idx + (CONSEC ? 4u * j : off[j]));
    };
#pragma unroll
    for (int j = 0; j < K; ++j) acc[j] = 0.f;
    gather(v0);
    for (;;) {
        const GStep s0 = gstep2(w, idx, lc, la, lb);
        gather(v1);
        const GStep s1 = gstep2(w, idx, lc, la, lb);
        gather(v2);
        const GStep s2 = gstep2(w, idx, lc, la, lb);
        gather(v3);
        const GStep s3 = gstep2(w, idx, lc, la, lb);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            acc[j] = fmaf((float)s0.seg, v0[j], acc[j]);
            acc[j] = fmaf((float)s1.seg, v1[j], acc[j]);
            acc[j] = fmaf((float)s2.seg, v2[j], acc[j]);
        }
        gather(v0);
#pragma unroll
        for (int j = 0; j < K; ++j) acc[j] = fmaf((float)s3.seg, v3[j], acc[j]);
        if (s3.last) break;
    }
}

// ---------------------------------------------------------------------------
// forward: float64 set-up, integer walk re-based per chunk
// ---------------------------------------------------------------------------

// Cells of the major axis covered by one chunk of the walk.
// 128 for parallel rays; fan/cone rays of one wave differ more in length, and
// their last chunks leave more lanes idle when a chunk is long, so they take 64.
constexpr int kChunkLog2Parallel = 7, kChunkLog2Persp = 6;

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

__device__ __forceinline__ void fix_axis(double d, double L, double S, int ncr, double dist,
                                         uint32_t &l0, uint32_t &q, uint32_t &lend) {
    if (d != 0.0) {
        const double qS = (L / fabs(d)) * S;
        q = fix64(qS);
        l0 = fix64(dist * qS);
        lend = min(lend, last_plus_one(l0, (uint32_t)ncr, q));
    } else {
        q = 0u;
        l0 = 0xFFFFFFFFu;
    }
}

// Line integral of the ray o + t d, t in [tin, tout] (inside the box), with the
// walk re-based every 2^clog2 cells of the major axis (2^31 walk units per chunk).
// nparts > 1: only chunks part, part + nparts, ...; a chunk's start is then its
// first plane's parameter, the same expression that ends the chunk before it, so
// every chunk's pieces are those of the whole walk.
__device__ __forceinline__ float project_ray(double ox, double oy, double oz, double dx, double dy,
                                             double dz, double tin, double tout, int nx, int ny,
                                             int nz, double spx, double spy, double spz,
                                             uint32_t ex, uint32_t ey, uint32_t ez,
                                             __amdgpu_buffer_rsrc_t rs, int clog2, int part = 0,
                                             int nparts = 1) {
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
    const int chunk = 1 << clog2;
    const int nch = (ncell + chunk - 1) >> clog2;
    // (ex, ey, ez): element strides of x, y, z in the volume copy being read
    const uint32_t sx = ex * 4u, sy = ey * 4u, sz = ez * 4u;
    // an axis the ray never crosses (parallel tilt series, 2D beams): when every
    // ray of the wave has the same one, the two-axis walk
    const int dead = dx == 0.0 ? 0 : (dy == 0.0 ? 1 : (dz == 0.0 ? 2 : 3));
    const int dead0 = __builtin_amdgcn_readfirstlane(dead);
    const bool two_axis = dead0 < 3 && __builtin_amdgcn_ballot_w64(dead != dead0) == 0;
    float total = 0.f;
    double ta = tin;
    for (int ch = part; ch < nch; ch += nparts) {
        const int first = cin + sgn * (ch << clog2);
        if (nparts > 1 && ch != 0) ta = ((double)(sgn > 0 ? first : first + 1) - oM) / dM;
        const int cells = min(chunk, ncell - (ch << clog2));
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
        const double chord = (tb - ta) * L;
        const double S = 0x1p31 / chord;   // walk units per length unit
        IWalk w;
        w.idx = (uint32_t)cx * sx + (uint32_t)cy * sy + (uint32_t)cz * sz;
        w.stx = dx > 0.0 ? sx : 0u - sx;
        w.sty = dy > 0.0 ? sy : 0u - sy;
        w.stz = dz > 0.0 ? sz : 0u - sz;
        w.lend = 1u << 31;
        fix_axis(dx, L, S, nxc, ddx, w.lx, w.qx, w.lend);
        fix_axis(dy, L, S, nyc, ddy, w.ly, w.qy, w.lend);
        fix_axis(dz, L, S, nzc, ddz, w.lz, w.qz, w.lend);
        const float sum = two_axis ? iwalk_gather2(live_axes(w, dead0), rs) : iwalk_gather(w, rs);
        total = fmaf(sum, (float)(chord * 0x1p-31), total);
        ta = tb;
    }
    return total;
}

// ---------------------------------------------------------------------------
// ray-driven kernels (forward, SIRT residual, row sums, counting, atomic A^T)
// ---------------------------------------------------------------------------

// RM_PROJECT_SQ: A p plus per-block sums of squares; RM_CGLS_R0: y - A x plus
// per-block sums of squares (the CGLS start).
enum RayMode : int {
    RM_PROJECT = 0, RM_RESIDUAL = 1, RM_ROWINV = 2, RM_COUNT = 3, RM_ATOMIC_BP = 4,
    RM_PROJECT_SQ = 5, RM_CGLS_R0 = 6
};

struct RayArgs {
    const double *views;
    const float *vol;          // RM_PROJECT, RM_RESIDUAL: the caller's x-fastest volume
    const float *vol_yf;       // y-fastest copy ((z*W + x)*H + y), if a view reads it
    const float *vol_zf;       // z-fastest copy ((x*H + y)*D + z), if a view reads it
    float *out;                // sinogram-shaped output; RM_ATOMIC_BP: the volume
    const float *sino;         // RM_RESIDUAL: y; RM_ATOMIC_BP: the sinogram
    const float *rinv;         // RM_RESIDUAL
    uint32_t *counts;          // RM_COUNT (nullable)
    unsigned long long *total; // RM_COUNT
    double *partial;           // RM_PROJECT_SQ, RM_CGLS_R0: one sum of squares per block
    Surface surf;              // detector surface (off == null: flat)
    int offx, offy, offz;      // voxel index of the volume buffer's first voxel (a region)
    int accumulate;            // RM_PROJECT: add to the sinogram instead of writing it
    int W, H, D, U, V, n_views;
    double spx, spy, spz;
    int n_utiles, n_vtiles, n_blocks;
    uint32_t vol_bytes;
};

// Tiles: a 256-thread block takes 16 x 16 pixels of one view; each wave takes a
// 16 x 4 (or 4 x 16) patch whose 16-wide side runs along the detector axis that
// the view's volume copy stores contiguously, so the 64 rays of a wave read few
// cache lines per step.  2D: 64 consecutive u per block; the forward modes give
// each ray four lanes, which take every fourth chunk of its walk and sum their
// parts in a fixed order (a 2D sinogram has too few rays to keep the SIMDs busy
// with one lane each: the gathers' latency went unhidden), and the other modes
// use the first wave only.  Block order: groups
// of 2 v-bands x 2 u-tiles, and inside a group every view in turn, so
// the blocks an XCD runs together trace the same few pixel tiles through
// neighbouring views; their rays cross the same voxels at nearly the same time
// and the gathers hit in L2 (this order cut the 512^3 forward times by a
// quarter against v-band, view, u-tile).
// SURF: parameterized detector surface (rays from the offsets table).
template <int MODE, bool TWO_D, bool SURF>
__global__ __launch_bounds__(256) void ray_kernel(RayArgs a) {
    const int blk = xcd_remap(blockIdx.x, a.n_blocks);
    // groups of 2 v-bands x 2 u-tiles; within a group: view, then band, then
    // u-tile (the last group of each kind may be short)
    constexpr int TU = 2, TB = 2;
    const int bg = blk / (a.n_views * a.n_utiles * TB);
    int r = blk - bg * (a.n_views * a.n_utiles * TB);
    const int tb = min(TB, a.n_vtiles - bg * TB);
    const int ug = r / (a.n_views * TU * tb);
    r -= ug * (a.n_views * TU * tb);
    const int tu = min(TU, a.n_utiles - ug * TU);
    const int view = r / (tu * tb);
    r -= view * (tu * tb);
    const int band = bg * TB + r / tu;
    const int ut = ug * TU + r % tu;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    constexpr bool kFwd = MODE == RM_PROJECT || MODE == RM_RESIDUAL || MODE == RM_PROJECT_SQ ||
                          MODE == RM_CGLS_R0;
    constexpr bool SPLIT = TWO_D && kFwd;   // four lanes per ray
    int u, v;
    if (SPLIT) {
        u = ut * 64 + (threadIdx.x >> 2);
        v = 0;
    } else if (TWO_D) {
        u = threadIdx.x < 64 ? ut * 64 + threadIdx.x : a.U;   // first wave only
        v = 0;
    } else {
        const double *vw0 = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
        if (vw0[VT_PATCH] == 0.0) {   // 16 u x 4 v per wave
            u = ut * 16 + (lane & 15);
            v = band * 16 + wv * 4 + (lane >> 4);
        } else {                      // 4 u x 16 v per wave
            u = ut * 16 + wv * 4 + (lane >> 4);
            v = band * 16 + (lane & 15);
        }
    }
    const bool active = (u < a.U) && (v < a.V);
    // the lane that writes a ray's result (the whole group agrees on active and on
    // the clip, so the exchanges below stay inside active lanes)
    const bool writer = !SPLIT || (threadIdx.x & 3) == 0;
    uint32_t my_count = 0;
    double my_sq = 0.0;
    if (active) {
        const double *vw = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
        double ox, oy, oz, dx, dy, dz;
        pixel_ray(vw, SURF ? a.surf : Surface{nullptr, 0}, view, u, v, a.U, a.V, ox, oy, oz, dx, dy,
                  dz);
        ox -= a.offx;   // into the coordinates of the volume buffer (a region of the lattice)
        oy -= a.offy;
        oz -= a.offz;
        const size_t ray = ((size_t)view * a.U + u) * a.V + v;
        if (kFwd) {
            float acc = 0.f;
            double tin, tout;
            if (clip_ray(ox, oy, oz, dx, dy, dz, vw[VT_TMIN], vw[VT_TMAX], a.W, a.H, a.D, tin, tout)) {
                const int layout = TWO_D ? 0 : (int)vw[VT_LAYOUT];
                const uint32_t W = a.W, H = a.H, D = a.D;
                const float *src = layout == 0 ? a.vol : (layout == 1 ? a.vol_yf : a.vol_zf);
                const uint32_t ex = layout == 0 ? 1u : (layout == 1 ? H : H * D);
                const uint32_t ey = layout == 0 ? W : (layout == 1 ? 1u : D);
                const uint32_t ez = layout == 0 ? W * H : (layout == 1 ? W * H : 1u);
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, a.vol_bytes);
                acc = project_ray(ox, oy, oz, dx, dy, dz, tin, tout, a.W, a.H, a.D, a.spx, a.spy,
                                  a.spz, ex, ey, ez, rs,
                                  vw[VT_PERSP] != 0.0 ? kChunkLog2Persp : kChunkLog2Parallel,
                                  SPLIT ? (int)(threadIdx.x & 3) : 0, SPLIT ? 4 : 1);
            }
            if (SPLIT) {   // (part 0 + part 1) + (part 2 + part 3), the same on every lane
                acc += __shfl_xor(acc, 1);
                acc += __shfl_xor(acc, 2);
            }
            if (writer) {
                if (MODE == RM_PROJECT || MODE == RM_PROJECT_SQ) {
                    if (MODE == RM_PROJECT && a.accumulate) acc += a.out[ray];
                    a.out[ray] = acc;
                    if (MODE == RM_PROJECT_SQ) my_sq = (double)acc * acc;
                } else if (MODE == RM_CGLS_R0) {
                    const float r = a.sino[ray] - acc;
                    a.out[ray] = r;
                    my_sq = (double)r * r;
                } else {
                    a.out[ray] = a.rinv[ray] * (a.sino[ray] - acc);
                }
            }
        } else {
            DWalk w;
            double chord = 0.0;
            const bool hit = make_dwalk(ox, oy, oz, dx, dy, dz, vw[VT_TMIN], vw[VT_TMAX], a.W, a.H,
                                        a.D, a.spx, a.spy, a.spz, w, chord);
            if (MODE == RM_ROWINV) {
                // (A 1)_i is the ray's chord through the whole volume
                const float ch = (float)chord;
                const float r = (hit && ch > 0.f) ? 1.0f / ch : 0.f;
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
                    dwalk(w, [&](int idx, double len) {
                        if (len > 0.0) atomicAdd(vol + idx, (float)len * y);
                    });
                }
            }
        }
    }
    if (MODE == RM_COUNT) {
        // wave reduction then one 64-bit atomic per wave
        unsigned long long c = my_count;
        for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
        if (lane == 0 && c) atomicAdd(a.total, c);
    }
    if (MODE == RM_PROJECT_SQ || MODE == RM_CGLS_R0) {
        // fixed-order block sum (float64), one partial per block
        __shared__ double wsum[4];
        double q = my_sq;
        for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
        if (lane == 0) wsum[wv] = q;
        __syncthreads();
        if (threadIdx.x == 0) a.partial[blockIdx.x] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    }
}

// Forward in packets (flat detector; every view parallel with a packet axis P,
// VT_PACKET): the rays of one row along P differ only in their coordinate on
// the axis d they never cross, so they walk the same cells of the other two
// axes.  A thread takes kPacket consecutive pixels along P: one clip and one
// walk, and at every piece one gather per ray from its own cell of d.  Each
// ray's sum is formed exactly as ray_kernel forms it (same clip, chunks,
// pieces and order of additions).  Tiles: a block takes kPacketTP pixels
// along P x kPacketTQ across; blocks run tile by tile, each tile through every
// view in turn.  RM_PROJECT, RM_RESIDUAL, and the CGLS forms RM_PROJECT_SQ and
// RM_CGLS_R0 with their fixed-order block sums of squares (one partial per block).
template <int MODE>
__global__ __launch_bounds__(64 * kPacketWaves) void ray_packet_kernel(RayArgs a) {
    constexpr int K = kPacket;
    const int blk = xcd_remap(blockIdx.x, a.n_blocks);
    // groups of kPacketTileGroup consecutive tiles; inside a group every view
    // in turn, the group's tiles innermost
    constexpr int G = kPacketTileGroup;
    const int grp = blk / (a.n_views * G), rg = blk - grp * (a.n_views * G);
    const int view = rg / G, tile = grp * G + (rg - (rg / G) * G);
    const double *vw = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
    const bool pu = vw[VT_PACKET] == 0.0;   // packets along u (else v)
    constexpr int TP = kPacketTP, TQ = kPacketTQ, RQ = 64 / kPacketLanesP;
    const int NP = pu ? a.U : a.V, NQ = pu ? a.V : a.U;
    const int ntp = (NP + TP - 1) / TP, ntq = (NQ + TQ - 1) / TQ;
    const bool tile_ok = tile < ntp * ntq;   // (a block past the last tile only writes its partial)
    const int tp = tile % ntp, tq = tile / ntp;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int p0 = tp * TP + (lane % kPacketLanesP) * K, q = tq * TQ + wv * RQ + lane / kPacketLanesP;
    constexpr bool SQ = MODE == RM_PROJECT_SQ || MODE == RM_CGLS_R0;
    double my_sq = 0.0;
    if (tile_ok && p0 < NP && q < NQ) {
    const int kk = min(K, NP - p0);
    const int u0 = pu ? p0 : q, v0 = pu ? q : p0;
    double ox, oy, oz, dx, dy, dz;
    pixel_ray(vw, Surface{nullptr, 0}, view, u0, v0, a.U, a.V, ox, oy, oz, dx, dy, dz);
    ox -= a.offx;
    oy -= a.offy;
    oz -= a.offz;
    // the clip of clip_ray, without the untraversed axis (tested per ray)
    const double dm = fmax(fabs(dx), fmax(fabs(dy), fabs(dz))) * 0x1p-40;
    if (fabs(dx) < dm) { dx = 0.0; ox = on_plane(ox); }
    if (fabs(dy) < dm) { dy = 0.0; oy = on_plane(oy); }
    if (fabs(dz) < dm) { dz = 0.0; oz = on_plane(oz); }
    // d: the axis the packet's pixel step runs along (the rays do not cross it)
    const int ps = pu ? VT_OU : VT_OV;
    const int d = vw[ps + 0] != 0.0 ? 0 : (vw[ps + 1] != 0.0 ? 1 : 2);
    double tin = vw[VT_TMIN], tout = vw[VT_TMAX];
    bool hit = true;
    if (d != 0) clip_axis(ox, dx, (double)a.W, tin, tout, hit);
    if (d != 1) clip_axis(oy, dy, (double)a.H, tin, tout, hit);
    if (d != 2) clip_axis(oz, dz, (double)a.D, tin, tout, hit);
    hit = hit && tout > tin;
    // per ray: its coordinate on d (as pixel_ray forms it), slab test and cell
    const int layout = (int)vw[VT_LAYOUT];
    const uint32_t W = a.W, H = a.H, D = a.D;
    const uint32_t ex = layout == 0 ? 1u : (layout == 1 ? H : H * D);
    const uint32_t ey = layout == 0 ? W : (layout == 1 ? 1u : D);
    const uint32_t ez = layout == 0 ? W * H : (layout == 1 ? W * H : 1u);
    const uint32_t sd = 4u * (d == 0 ? ex : (d == 1 ? ey : ez));
    const int nd = d == 0 ? a.W : (d == 1 ? a.H : a.D);
    bool in[K];
    int cd[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        double rx = ox, ry = oy, rz = oz, qx, qy, qz;
        if (j > 0) {
            pixel_ray(vw, Surface{nullptr, 0}, view, u0 + (pu ? j : 0), v0 + (pu ? 0 : j), a.U, a.V, rx, ry, rz, qx,
                      qy, qz);
            rx -= a.offx;
            ry -= a.offy;
            rz -= a.offz;
        }
        const double od = on_plane(d == 0 ? rx : (d == 1 ? ry : rz));
        in[j] = j < kk && od >= 0.0 && od < (double)nd;
        cd[j] = min(max((int)floor(od), 0), nd - 1);
    }
    float tot[K];
#pragma unroll
    for (int j = 0; j < K; ++j) tot[j] = 0.f;
    if (hit) {
        const float *src = layout == 0 ? a.vol : (layout == 1 ? a.vol_yf : a.vol_zf);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, a.vol_bytes);
        uint32_t off[K];
        bool consec = sd == 4u;   // the rays' cells are consecutive words
#pragma unroll
        for (int j = 0; j < K; ++j) {
            off[j] = (uint32_t)(cd[j] - cd[0]) * sd;
            consec = consec && (!in[j] || cd[j] == cd[0] + j);
        }
        const bool vec = __builtin_amdgcn_ballot_w64(!consec) == 0;
        // project_ray's chunked walk for the live axes; the untraversed axis
        // only places the cells
        const double px = dx * a.spx, py = dy * a.spy, pz = dz * a.spz;
        const double L = sqrt(px * px + py * py + pz * pz);
        const double ax_ = fabs(dx), ay_ = fabs(dy), az_ = fabs(dz);
        const int M = (ax_ >= ay_ && ax_ >= az_) ? 0 : (ay_ >= az_ ? 1 : 2);
        const double oM = M == 0 ? ox : (M == 1 ? oy : oz);
        const double dM = M == 0 ? dx : (M == 1 ? dy : dz);
        const int nM = M == 0 ? a.W : (M == 1 ? a.H : a.D);
        const double eM = fma(tin, dM, oM), xM = fma(tout, dM, oM);
        const int sgn = dM > 0.0 ? 1 : -1;
        int cin = sgn > 0 ? (int)floor(eM) : (int)ceil(eM) - 1;
        int cout = sgn > 0 ? (int)ceil(xM) - 1 : (int)floor(xM);
        cin = min(max(cin, 0), nM - 1);
        cout = min(max(cout, 0), nM - 1);
        const int ncell = max((cout - cin) * sgn, 0) + 1;
        constexpr int clog2 = kChunkLog2Parallel;
        const int chunk = 1 << clog2;
        const int nch = (ncell + chunk - 1) >> clog2;
        const uint32_t sx = ex * 4u, sy = ey * 4u, sz = ez * 4u;
        double ta = tin;
        for (int ch = 0; ch < nch; ++ch) {
            const int first = cin + sgn * (ch << clog2);
            const int cells = min(chunk, ncell - (ch << clog2));
            double tb = tout;
            if (ch != nch - 1) {
                const int P = sgn > 0 ? first + cells : first - cells + 1;
                tb = ((double)P - oM) / dM;
            }
            int cx, cy, cz, nxc, nyc, nzc;
            double ddx, ddy, ddz;
            chunk_axis(ox, dx, ta, tb, a.W, M == 0, first, cells, ch == 0, cx, nxc, ddx);
            chunk_axis(oy, dy, ta, tb, a.H, M == 1, first, cells, ch == 0, cy, nyc, ddy);
            chunk_axis(oz, dz, ta, tb, a.D, M == 2, first, cells, ch == 0, cz, nzc, ddz);
            if (d == 0) cx = cd[0];
            else if (d == 1) cy = cd[0];
            else cz = cd[0];
            const double chord = (tb - ta) * L;
            const double S = 0x1p31 / chord;
            IWalk w;
            w.idx = (uint32_t)cx * sx + (uint32_t)cy * sy + (uint32_t)cz * sz;
            w.stx = dx > 0.0 ? sx : 0u - sx;
            w.sty = dy > 0.0 ? sy : 0u - sy;
            w.stz = dz > 0.0 ? sz : 0u - sz;
            w.lend = 1u << 31;
            fix_axis(dx, L, S, nxc, ddx, w.lx, w.qx, w.lend);
            fix_axis(dy, L, S, nyc, ddy, w.ly, w.qy, w.lend);
            fix_axis(dz, L, S, nzc, ddz, w.lz, w.qz, w.lend);
            float sum[K];
            if (vec) iwalk_gather2_packet<K, true>(live_axes(w, d), rs, off, sum);
            else iwalk_gather2_packet<K, false>(live_axes(w, d), rs, off, sum);
            const float cs = (float)(chord * 0x1p-31);
#pragma unroll
            for (int j = 0; j < K; ++j) tot[j] = fmaf(sum[j], cs, tot[j]);
            ta = tb;
        }
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
        if (j >= kk) break;
        const int u = u0 + (pu ? j : 0), v = v0 + (pu ? 0 : j);
        const size_t ray = ((size_t)view * a.U + u) * a.V + v;
        const float acc = in[j] ? tot[j] : 0.f;
        if (MODE == RM_PROJECT) {
            a.out[ray] = a.accumulate ? acc + a.out[ray] : acc;
        } else if (MODE == RM_PROJECT_SQ) {
            a.out[ray] = acc;
            my_sq += (double)acc * acc;
        } else if (MODE == RM_CGLS_R0) {
            const float r = a.sino[ray] - acc;
            a.out[ray] = r;
            my_sq += (double)r * r;
        } else {
            a.out[ray] = a.rinv[ray] * (a.sino[ray] - acc);
        }
    }
    }
    if constexpr (SQ) {
        // fixed-order block sum (float64), one partial per block
        __shared__ double wsum[kPacketWaves];
        double t = my_sq;
        for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
        if (lane == 0) wsum[wv] = t;
        __syncthreads();
        if (threadIdx.x == 0) {
            double b = 0.0;
            for (int k = 0; k < kPacketWaves; ++k) b += wsum[k];
            a.partial[blockIdx.x] = b;
        }
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
// once: no global atomics, and the integer LDS sums do not depend on the order of
// the adds.
//
// Each ray is re-expressed per (view, brick) around the plane through the brick
// centre parallel to the detector: for a flat detector the point where pixel
// (u, v)'s ray meets that plane is affine in (u, v), so it is formed in float32
// from a float64 anchor at the footprint's centre pixel plus small integer
// offsets; positions are taken relative to the brick centre, so they stay within
// about half a brick diagonal and keep float32 resolution near 1e-6 voxel.
// Negative directions are mirrored about the brick centre so every axis is
// walked upwards in the set-up arithmetic.

// BM_CGLS: s = A^T r written out, per-brick sums of s^2, and optionally
// x += alpha p (alpha read from the CGLS state) and p = s (the start).
enum BrickMode : int { BM_BACKPROJECT = 0, BM_SIRT_UPDATE = 1, BM_COLINV = 2, BM_CGLS = 3 };

struct BrickRec;
struct BrickArgs {
    const double *views;
    const float *sino;        // BM_BACKPROJECT, BM_SIRT_UPDATE
    float *vol;               // output (BM_SIRT_UPDATE: x, read-modify-write; BM_COLINV: col_inv)
    const float *cinv;        // BM_SIRT_UPDATE
    float relax;
    bool bounded;             // BM_SIRT_UPDATE: clamp the updated x to [lo, hi]
    float lo, hi;
    const uint8_t *mask;      // BM_SIRT_UPDATE: update only voxels with mask != 0 (nullable)
    float *x_upd;             // BM_CGLS: x += alpha p_old (nullable)
    const float *p_old;       // BM_CGLS, with x_upd
    float *p_copy;            // BM_CGLS: p = s (nullable)
    const double *state;      // BM_CGLS: CGLS scalars (alpha)
    double *partial;          // BM_CGLS: one sum of s^2 per brick
    Surface surf;             // detector surface (off == null: flat)
    const float *env;         // surface: per-view footprint envelopes
    int offx, offy, offz;     // voxel index of the volume buffer's first voxel (a region)
    const BrickRec *rec;      // per-(brick, view) records of this launch's bricks, or null:
                              // record of brick b, view k at rec[b * rec_stride + k]
    int rec_stride;
    int y_vec4;               // the sinogram's rows are 16-byte aligned (V % 4 == 0, aligned base):
                              // pass 1 reads them four values at a time
    int accumulate;           // BM_BACKPROJECT: add to the volume instead of writing it
    int yshift;               // every term shifted right by this many bits (range bound)
    int W, H, D, U, V, n_views;
    double spx, spy, spz;
    int nbx, nby, nbz, n_blocks;
};

// Non-negative float32 to fixed point with the convert's own saturation
// (values from 2^32 up and INF give 0xFFFFFFFF, negative values 0).
__device__ __forceinline__ uint32_t sat_u32(float x) {
    uint32_t r;
    asm("v_cvt_u32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Crossing plan of one mirrored (non-negative direction) axis of extent e =
// 2h, in brick-centred coordinates, for a walk entering at tin: entry cell fe
// (float), the fixed-point position l0 of the first crossing, and far = the
// position of the crossing of the brick's far face, l0 + (e - 1 - fe) q,
// saturating.  A walk that ends at or before far takes at most e - 1 - fe
// crossings of this axis, so it never leaves the brick.
__device__ __forceinline__ void baxis(float o, float a, float tin, float h, float em1, float qf,
                                      uint32_t q, float &fe, uint32_t &l0, uint32_t &far) {
    const float E = fmaf(tin, a, o);   // entry coordinate, centred
    fe = __builtin_amdgcn_fmed3f(floorf(E + h), 0.f, em1);
    l0 = sat_u32(((fe + 1.f - h) - E) * qf);
    far = last_plus_one(l0, sat_u32(em1 - fe), q);
}

// Block sum of one float64 per thread in a fixed order; the result is valid in
// thread 0.  wsum: one slot per wave.
template <int NT>
__device__ __forceinline__ double block_sum(double v, double *wsum) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 0) wsum[wv] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int k = 0; k < NT / 64; ++k) t += wsum[k];
    return t;
}

// Footprint of the brick [x0, x0+ex) x [y0, y0+ey) x [z0, z0+ez) on the detector of
// one view: the bounding box of its 8 projected corners.  Returns false if no pixel
// can see it.  Two forms give the same box: the wave form (lane & 7 projects
// corner lane & 7, lanes reduce in groups of 8; the surface envelopes are searched
// by the whole wave) and the lane form (one lane projects all 8 corners and
// searches alone), which builds the per-(brick, view) record table.
struct Footprint {
    int u0, u1, v0, v1;
};
// View-table reads through the constant address space: wave-uniform reads
// become scalar loads (the table is never written while a kernel runs).
typedef const __attribute__((address_space(4))) double *ConstViewPtr;
__device__ __forceinline__ double vt(const double *vw, int i) { return ((ConstViewPtr)vw)[i]; }
// Corner c (bit 0: x, bit 1: y, bit 2: z far side) on the detector, in pixel units;
// bad: the corner lies at or behind the source.
__device__ __forceinline__ void corner_uv(const double *vw, int c, int x0, int y0, int z0, int ex, int ey,
                                          int ez, bool persp, float &cu, float &cvv, int &bad) {
    const double X = (c & 1) ? x0 + ex : x0;
    const double Y = (c & 2) ? y0 + ey : y0;
    const double Z = (c & 4) ? z0 + ez : z0;
    const double rx = X - vt(vw, VT_O00 + 0), ry = Y - vt(vw, VT_O00 + 1), rz = Z - vt(vw, VT_O00 + 2);
    const double al = vt(vw, VT_MINV + 0) * rx + vt(vw, VT_MINV + 1) * ry + vt(vw, VT_MINV + 2) * rz;
    const double be = vt(vw, VT_MINV + 3) * rx + vt(vw, VT_MINV + 4) * ry + vt(vw, VT_MINV + 5) * rz;
    const double ga = vt(vw, VT_MINV + 6) * rx + vt(vw, VT_MINV + 7) * ry + vt(vw, VT_MINV + 8) * rz;
    bad = 0;
    if (persp) {
        // a corner at or behind the source: every pixel may see the brick
        bad = !(al > 1e-9);
        cu = bad ? 0.f : (float)(be / al);
        cvv = bad ? 0.f : (float)(ga / al);
    } else {
        cu = (float)be;
        cvv = (float)ga;
    }
}
// First index i in [0, n) with a[i] >= x (GT: a[i] > x), n if none; a
// non-decreasing.  One lane alone (binary search): the same index as first_hit.
template <bool GT>
__device__ __forceinline__ int first_hit_lane(const float *a, int n, float x) {
    int lo = 0, hi = n;   // the first hit lies in [lo, hi]
    while (lo < hi) {
        const int mid = lo + ((hi - lo) >> 1);
        const bool hit = GT ? a[mid] > x : a[mid] >= x;
        hi = hit ? mid : hi;
        lo = hit ? lo : mid + 1;
    }
    return lo;
}
// The pixel box from the corners' extremes (wave-uniform in the wave form).
template <bool WAVE>
__device__ __forceinline__ bool footprint_box(float umin, float umax, float vmin, float vmax, int bad, int U,
                                              int V, bool two_d, const float *env, int lane, Footprint &f) {
    const auto hit_lo = [&](const float *a, int n, float x) {
        if constexpr (WAVE) return first_hit<false>(a, n, x, lane);
        else return first_hit_lane<false>(a, n, x);
    };
    const auto hit_hi = [&](const float *a, int n, float x) {
        if constexpr (WAVE) return first_hit<true>(a, n, x, lane);
        else return first_hit_lane<true>(a, n, x);
    };
    if (bad) {
        f.u0 = 0; f.u1 = U - 1; f.v0 = 0; f.v1 = V - 1;
    } else if (env) {
        // detector surface: the pixel ranges whose flat-plane crossings can fall in
        // the box (monotone envelopes; a margin for their float32 rounding)
        const float m = 1e-2f;
        f.u0 = hit_lo(env + U, U, umin - m);
        f.u1 = hit_hi(env, U, umax + m) - 1;
        f.v0 = V;
        f.v1 = -1;
        if (f.u0 <= f.u1) {
            for (int t = f.u0 / kEnvTile; t <= f.u1 / kEnvTile; ++t) {
                const float *r = env + 2 * U + (size_t)t * 2 * V;
                f.v0 = min(f.v0, hit_lo(r + V, V, vmin - m));
                f.v1 = max(f.v1, hit_hi(r, V, vmax + m) - 1);
            }
        }
    } else {
        // guard the float conversions against far-away projections
        umin = fmaxf(umin, -1.f); umax = fminf(umax, (float)U);
        vmin = fmaxf(vmin, -1.f); vmax = fminf(vmax, (float)V);
        f.u0 = max(0, (int)ceilf(umin - 1e-3f));
        f.u1 = min(U - 1, (int)floorf(umax + 1e-3f));
        f.v0 = max(0, (int)ceilf(vmin - 1e-3f));
        f.v1 = min(V - 1, (int)floorf(vmax + 1e-3f));
    }
    if (two_d) { f.v0 = 0; f.v1 = 0; }
    return f.u0 <= f.u1 && f.v0 <= f.v1;
}
__device__ __forceinline__ bool brick_footprint(const double *vw, int lane, int x0, int y0, int z0,
                                                int ex, int ey, int ez, int U, int V, bool two_d,
                                                const float *env, Footprint &f) {
    const bool persp = vt(vw, VT_PERSP) != 0.0;
    float cu, cvv;
    int bad;
    corner_uv(vw, lane & 7, x0, y0, z0, ex, ey, ez, persp, cu, cvv, bad);
    float umin = cu, umax = cu, vmin = cvv, vmax = cvv;
    for (int off = 1; off < 8; off <<= 1) {
        umin = fminf(umin, __shfl_xor(umin, off));
        umax = fmaxf(umax, __shfl_xor(umax, off));
        vmin = fminf(vmin, __shfl_xor(vmin, off));
        vmax = fmaxf(vmax, __shfl_xor(vmax, off));
        bad |= __shfl_xor(bad, off);
    }
    umin = uni(umin); umax = uni(umax); vmin = uni(vmin); vmax = uni(vmax);
    bad = uni(bad);
    return footprint_box<true>(umin, umax, vmin, vmax, bad, U, V, two_d, env, lane, f);
}
__device__ __forceinline__ bool brick_footprint_lane(const double *vw, int x0, int y0, int z0, int ex, int ey,
                                                     int ez, int U, int V, bool two_d, const float *env,
                                                     Footprint &f) {
    const bool persp = vw[VT_PERSP] != 0.0;
    float umin = 3e38f, umax = -3e38f, vmin = 3e38f, vmax = -3e38f;
    int bad = 0;
    for (int c = 0; c < 8; ++c) {
        float cu, cvv;
        int b;
        corner_uv(vw, c, x0, y0, z0, ex, ey, ez, persp, cu, cvv, b);
        umin = fminf(umin, cu); umax = fmaxf(umax, cu);
        vmin = fminf(vmin, cvv); vmax = fmaxf(vmax, cvv);
        bad |= b;
    }
    return footprint_box<false>(umin, umax, vmin, vmax, bad, U, V, two_d, env, 0, f);
}

// The ray of a footprint's centre pixel (u0 + nfu/2, v0 + nfv/2), re-expressed
// around the plane through the brick centre parallel to the detector: for a flat
// detector, the point where pixel (u, v) meets that plane is affine in (u, v), so
// per ray it is formed in float32 from this anchor plus small integer offsets and
// positions stay within tens of voxels.  Positions are relative to the brick
// centre; "fast" is the footprint's fast pixel axis (u when the view's wave patch
// runs along u).  Computed in float64, rounded once.
struct Anchor {
    float A0x, A0y, A0z;   // anchor point on the plane, relative to the brick centre
    float Afx, Afy, Afz;   // its step per fast pixel
    float Asx, Asy, Asz;   // its step per slow pixel
    float Dx, Dy, Dz;      // direction of the centre pixel's ray
    float tv0, tv1;        // the ray's parameter range, relative to the plane crossing
};
__device__ __forceinline__ Anchor make_anchor(const double *vw, const Footprint &f, double cbx, double cby,
                                              double cbz, bool ufast) {
    const int nfu = f.u1 - f.u0 + 1, nfv = f.v1 - f.v0 + 1;
    const double fu0 = f.u0 + nfu / 2, fv0 = f.v0 + nfv / 2;
    const double nx_ = vt(vw, VT_N + 0), ny_ = vt(vw, VT_N + 1), nz_ = vt(vw, VT_N + 2);
    const double aox = vt(vw, VT_O00 + 0) + fu0 * vt(vw, VT_OU + 0) + fv0 * vt(vw, VT_OV + 0);
    const double aoy = vt(vw, VT_O00 + 1) + fu0 * vt(vw, VT_OU + 1) + fv0 * vt(vw, VT_OV + 1);
    const double aoz = vt(vw, VT_O00 + 2) + fu0 * vt(vw, VT_OU + 2) + fv0 * vt(vw, VT_OV + 2);
    const double adx = vt(vw, VT_D00 + 0) + fu0 * vt(vw, VT_DU + 0) + fv0 * vt(vw, VT_DV + 0);
    const double ady = vt(vw, VT_D00 + 1) + fu0 * vt(vw, VT_DU + 1) + fv0 * vt(vw, VT_DV + 1);
    const double adz = vt(vw, VT_D00 + 2) + fu0 * vt(vw, VT_DU + 2) + fv0 * vt(vw, VT_DV + 2);
    // Dir . N is the same for every pixel of a flat detector
    const double tb = ((cbx - aox) * nx_ + (cby - aoy) * ny_ + (cbz - aoz) * nz_) /
                      (adx * nx_ + ady * ny_ + adz * nz_);
    const int pf = ufast ? VT_OU : VT_OV, ps = ufast ? VT_OV : VT_OU;
    const int qf_ = ufast ? VT_DU : VT_DV, qs_ = ufast ? VT_DV : VT_DU;
    Anchor an;
    an.A0x = (float)(aox + tb * adx - cbx);
    an.A0y = (float)(aoy + tb * ady - cby);
    an.A0z = (float)(aoz + tb * adz - cbz);
    an.Afx = (float)(vt(vw, pf + 0) + tb * vt(vw, qf_ + 0));
    an.Afy = (float)(vt(vw, pf + 1) + tb * vt(vw, qf_ + 1));
    an.Afz = (float)(vt(vw, pf + 2) + tb * vt(vw, qf_ + 2));
    an.Asx = (float)(vt(vw, ps + 0) + tb * vt(vw, qs_ + 0));
    an.Asy = (float)(vt(vw, ps + 1) + tb * vt(vw, qs_ + 1));
    an.Asz = (float)(vt(vw, ps + 2) + tb * vt(vw, qs_ + 2));
    an.Dx = (float)adx;
    an.Dy = (float)ady;
    an.Dz = (float)adz;
    an.tv0 = (float)(vt(vw, VT_TMIN) - tb);
    an.tv1 = (float)(vt(vw, VT_TMAX) - tb);
    return an;
}

// One (brick, view) pair of the record table: the footprint (u1 < u0: the view
// does not see the brick) and the anchor.  64 bytes, read by scalar loads.
struct BrickRec {
    uint32_t fu;   // u0 | u1 << 16
    uint32_t fv;   // v0 | v1 << 16
    Anchor an;
};
static_assert(sizeof(BrickRec) == 64, "brick record layout");
typedef const __attribute__((address_space(4))) BrickRec *ConstRecPtr;
// a record's anchor, field by field (scalar loads)
__device__ __forceinline__ Anchor rec_anchor(ConstRecPtr r) {
    Anchor an;
    an.A0x = r->an.A0x; an.A0y = r->an.A0y; an.A0z = r->an.A0z;
    an.Afx = r->an.Afx; an.Afy = r->an.Afy; an.Afz = r->an.Afz;
    an.Asx = r->an.Asx; an.Asy = r->an.Asy; an.Asz = r->an.Asz;
    an.Dx = r->an.Dx; an.Dy = r->an.Dy; an.Dz = r->an.Dz;
    an.tv0 = r->an.tv0; an.tv1 = r->an.tv1;
    return an;
}

// LDS scatter into 64-bit fixed point: lds[cell] += length * Y for every piece,
// length in walk units and Y the ray's value in fixed point, both below 2^23 in
// magnitude, so the product is formed exactly by the 24-bit multiplier
// (v_mul_i32_i24 / v_mul_hi_i32_i24) and the integer sums do not depend on the
// order of the adds.  Float atomic adds in LDS run some 30x slower than integer
// ones on this chip, hence the integer accumulator.
//
// Range.  The accumulator's unit is set per brick by its largest |y|.  A ray
// far below that keeps its own 24 significant bits: Y is its mantissa scaled
// up by 2^k and each product is shifted right by k before the add (SHIFT
// walks), so its terms carry float32-like relative precision (the shift drops
// less than one accumulator unit, about 2^-45 of the brick's largest term).
// Rays within 2^6 of the largest use the plain walk (at least 17 bits).  A
// geometry whose per-voxel sum could pass 2^63 (many views of voxels much
// larger than the pixels, or a source near the volume) shifts every term by
// the host-computed a.yshift as well.
constexpr float kPieceUnits = 8323072.f;   // 2^23 - 2^16
constexpr int kFpCache = 1024;             // brick kernel: views whose footprints LDS keeps
__device__ __forceinline__ unsigned long long mul24_64(uint32_t len, int y) {
    const int a = (int)(len << 8) >> 8, b = (y << 8) >> 8;   // 24-bit operands
    return (unsigned long long)((long long)a * (long long)b);
}
__device__ __forceinline__ void lds_add(unsigned long long *lds, uint32_t byte_off,
                                        unsigned long long v) {
    atomicAdd((unsigned long long *)((char *)lds + byte_off), v);
}
// Move past the crossing at t = min(lx, ly, lz): exactly one axis steps, the
// first of x, y, z whose next crossing is t.  Where two planes are crossed at
// the same point the other axis steps on the next call, after a piece of
// length 0 (it adds nothing; its cell, one step along the first axis, lies in
// the brick because that crossing was a real one).
__device__ __forceinline__ void sadvance(uint32_t qx, uint32_t qy, uint32_t qz, uint32_t sx,
                                         uint32_t sy, uint32_t sz, uint32_t t, uint32_t &idx,
                                         uint32_t &lx, uint32_t &ly, uint32_t &lz) {
    // the step masks are combined as wave masks, on the scalar unit
    const uint64_t mx = __builtin_amdgcn_ballot_w64(lx == t);
    const uint64_t my = __builtin_amdgcn_ballot_w64(ly == t) & ~mx;
    const bool bx = __builtin_amdgcn_inverse_ballot_w64(mx);
    const bool by = __builtin_amdgcn_inverse_ballot_w64(my);
    const bool bxy = __builtin_amdgcn_inverse_ballot_w64(mx | my);
    const uint32_t nx = __builtin_elementwise_add_sat(lx, qx);
    const uint32_t ny = __builtin_elementwise_add_sat(ly, qy);
    const uint32_t nz = __builtin_elementwise_add_sat(lz, qz);
    const uint32_t syz = by ? sy : sz;   // values, not field addresses: no table in memory
    lx = bx ? nx : lx;
    ly = by ? ny : ly;
    lz = bxy ? lz : nz;
    idx += bx ? sx : syz;
}
// Two pieces per iteration with one exit test: the loop is entered only while the
// next event t lies before l_end, so the first piece of an iteration is whole;
// the second is cut at l_end.  A cell is only written before a crossing at or
// past l_end has been taken, so every offset stays inside the brick.
template <bool SHIFT>
__device__ __forceinline__ unsigned long long term(uint32_t len, int Y, int sh) {
    const unsigned long long p = mul24_64(len, Y);
    return SHIFT ? (unsigned long long)((long long)p >> sh) : p;
}
template <bool SHIFT>
__device__ __forceinline__ void iwalk_scatter_fix(const IWalk &w, unsigned long long *lds, int Y, int sh) {
    const uint32_t qx = w.qx, qy = w.qy, qz = w.qz, sx = w.stx, sy = w.sty, sz = w.stz;
    const uint32_t lend = w.lend;
    uint32_t idx = w.idx;
    uint32_t lx = w.lx, ly = w.ly, lz = w.lz;
    uint32_t lc = 0, t = umin3(lx, ly, lz);
    while (t < lend) {
        lds_add(lds, idx, term<SHIFT>(t - lc, Y, sh));
        sadvance(qx, qy, qz, sx, sy, sz, t, idx, lx, ly, lz);
        lc = t;
        t = umin3(lx, ly, lz);
        const uint32_t tn = min(t, lend);
        lds_add(lds, idx, term<SHIFT>(tn - lc, Y, sh));
        sadvance(qx, qy, qz, sx, sy, sz, t, idx, lx, ly, lz);
        lc = tn;
        t = umin3(lx, ly, lz);
    }
    if (lc < lend) lds_add(lds, idx, term<SHIFT>(lend - lc, Y, sh));
}

// The two-axis walk (one direction component 0; see live_axes): the same
// pieces and cells as the three-axis walk.
template <bool SHIFT>
__device__ __forceinline__ void iwalk2_scatter_fix(const IWalk2 &w, unsigned long long *lds, int Y, int sh) {
    const uint32_t qa = w.qa, qb = w.qb, sa = w.sa, sb = w.sb, lend = w.lend;
    uint32_t idx = w.idx, la = w.la, lb = w.lb;
    uint32_t lc = 0, t = min(la, lb);
    const auto advance = [&]() {
        const bool ba = la == t;
        const uint32_t na = __builtin_elementwise_add_sat(la, qa);
        const uint32_t nb = __builtin_elementwise_add_sat(lb, qb);
        la = ba ? na : la;
        lb = ba ? lb : nb;
        idx += ba ? sa : sb;
    };
    while (t < lend) {
        lds_add(lds, idx, term<SHIFT>(t - lc, Y, sh));
        advance();
        lc = t;
        t = min(la, lb);
        const uint32_t tn = min(t, lend);
        lds_add(lds, idx, term<SHIFT>(tn - lc, Y, sh));
        advance();
        lc = tn;
        t = min(la, lb);
    }
    if (lc < lend) lds_add(lds, idx, term<SHIFT>(lend - lc, Y, sh));
}

// A packet of K rays that share their walk (parallel rays one detector step
// apart along the axis none of them crosses): the live-axis walk once, and at
// every piece one term per ray into its own cell of the untraversed axis
// (off[j], from the walk's cell).  A ray without a value there has Y = 0.
// SD > 0: the rays' cells are consecutive along the untraversed axis, whose
// LDS byte stride is SD: off[j] = j SD, an immediate offset of the add.
template <bool SHIFT, int K, uint32_t SD>
__device__ __forceinline__ void iwalk2_scatter_packet(const IWalk2 &w, unsigned long long *lds, const int (&Y)[K],
                                                      const int (&sh)[K], const uint32_t (&off)[K]) {
    const uint32_t qa = w.qa, qb = w.qb, sa = w.sa, sb = w.sb, lend = w.lend;
    uint32_t idx = w.idx, la = w.la, lb = w.lb;
    uint32_t lc = 0, t = min(la, lb);
    const auto put = [&](uint32_t len) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if constexpr (SD > 0) {
                unsigned long long *cell = (unsigned long long *)((char *)lds + idx) + j * (SD / 8);
                atomicAdd(cell, term<SHIFT>(len, Y[j], sh[j]));
            } else {
                lds_add(lds, idx + off[j], term<SHIFT>(len, Y[j], sh[j]));
            }
        }
    };
    const auto advance = [&]() {
        const bool ba = la == t;
        const uint32_t na = __builtin_elementwise_add_sat(la, qa);
        const uint32_t nb = __builtin_elementwise_add_sat(lb, qb);
        la = ba ? na : la;
        lb = ba ? lb : nb;
        idx += ba ? sa : sb;
    };
    while (t < lend) {
        put(t - lc);
        advance();
        lc = t;
        t = min(la, lb);
        const uint32_t tn = min(t, lend);
        put(tn - lc);
        advance();
        lc = tn;
        t = min(la, lb);
    }
    if (lc < lend) put(lend - lc);
}

// Everything of a brick walk that depends on the ray direction alone (for
// parallel rays: once per view and brick).  Components below 2^-40 of the
// largest count as zero; the test is taken over the wave, so waves without any
// such component (nearly all of them) skip the special clip.  Negative
// directions are mirrored about the brick centre, so every axis walks upwards.
struct DirPlan {
    float axx, ayy, azz;      // |direction|
    float ix, iy, iz;         // 1 / |direction| (approximate reciprocal)
    float LS;                 // walk units per unit of the ray parameter
    float qfx, qfy, qfz;      // crossing spacing per axis, in walk units
    uint32_t qx, qy, qz;      // the same in fixed point, saturating
    uint32_t stx, sty, stz;   // LDS byte strides of a step along each axis
    bool nx, ny, nz;          // mirrored axes
    bool slow;                // some lane of the wave has a zero component
};

template <int LSY, int LSZ, bool TWO_D>
__device__ __forceinline__ DirPlan dir_plan(float dx, float dy, float dz, float spx, float spy, float spz,
                                            float S) {
    DirPlan p;
    if (TWO_D) dz = 0.f;
    const float dm = fmaxf(fabsf(dx), fmaxf(fabsf(dy), fabsf(dz))) * 0x1p-40f;
    const float amin = TWO_D ? fminf(fabsf(dx), fabsf(dy)) : fminf(fabsf(dx), fminf(fabsf(dy), fabsf(dz)));
    p.slow = __builtin_amdgcn_ballot_w64(amin < dm) != 0;   // wave-uniform
    if (p.slow) {
        if (fabsf(dx) < dm) dx = 0.f;
        if (fabsf(dy) < dm) dy = 0.f;
        if (!TWO_D && fabsf(dz) < dm) dz = 0.f;
    }
    p.nx = dx < 0.f;
    p.ny = dy < 0.f;
    p.nz = dz < 0.f;
    p.axx = fabsf(dx);
    p.ayy = fabsf(dy);
    p.azz = fabsf(dz);
    p.ix = __builtin_amdgcn_rcpf(p.axx);
    p.iy = __builtin_amdgcn_rcpf(p.ayy);
    p.iz = TWO_D ? 0.f : __builtin_amdgcn_rcpf(p.azz);
    const float px = dx * spx, py = dy * spy, pz = dz * spz;
    p.LS = __builtin_amdgcn_sqrtf(px * px + py * py + pz * pz) * S;
    p.qfx = p.LS * p.ix;
    p.qfy = p.LS * p.iy;
    p.qfz = p.LS * p.iz;
    p.qx = sat_u32(p.qfx);
    p.qy = sat_u32(p.qfy);
    p.qz = TWO_D ? 0xFFFFFFFFu : sat_u32(p.qfz);
    p.stx = p.nx ? (uint32_t)-8 : 8u;
    p.sty = p.ny ? (uint32_t)(-8 * LSY) : (uint32_t)(8 * LSY);
    p.stz = TWO_D ? 0u : (p.nz ? (uint32_t)(-8 * LSZ) : (uint32_t)(8 * LSZ));
    return p;
}

// The same for a direction already mirrored to positive components, none of
// them near zero (the caller has shown both for every ray of the footprint);
// signs and strides are then the caller's, once per footprint.
template <bool TWO_D>
__device__ __forceinline__ DirPlan dir_plan_pos(float ax, float ay, float az, float spx, float spy,
                                                float spz, float S) {
    DirPlan p;
    if (TWO_D) az = 0.f;
    p.slow = false;
    p.nx = p.ny = p.nz = false;
    p.axx = ax;
    p.ayy = ay;
    p.azz = az;
    p.ix = __builtin_amdgcn_rcpf(ax);
    p.iy = __builtin_amdgcn_rcpf(ay);
    p.iz = TWO_D ? 0.f : __builtin_amdgcn_rcpf(az);
    const float px = ax * spx, py = ay * spy, pz = az * spz;
    p.LS = __builtin_amdgcn_sqrtf(px * px + py * py + pz * pz) * S;
    p.qfx = p.LS * p.ix;
    p.qfy = p.LS * p.iy;
    p.qfz = p.LS * p.iz;
    p.qx = sat_u32(p.qfx);
    p.qy = sat_u32(p.qfy);
    p.qz = TWO_D ? 0xFFFFFFFFu : sat_u32(p.qfz);
    p.stx = p.sty = p.stz = 0u;
    return p;
}

// Walk every ray of one view's footprint through the brick.  PERSP: fan/cone
// rays (direction per ray); otherwise parallel rays, whose direction and all
// that is derived from it are the same for the whole footprint and computed
// once, outside the ray loop.  TWO_D: single-slice bricks of a 2D geometry,
// whose rays lie in the slice (z is neither clipped nor walked).  S = walk units
// per length unit; yscale = power-of-two fixed-point scale of the ray values.
template <int LSY, int LSZ, int MODE, bool PERSP, bool TWO_D, bool SURF>
__device__ __forceinline__ void brick_rays(const BrickArgs &a, const double *vw, int view,
                                           const Footprint &f, const Anchor &an, int lane, int x0, int y0,
                                           int z0, int ex, int ey, int ez, double cbx, double cby,
                                           double cbz, float S, float yscale,
                                           unsigned long long *acc) {
    const float fex = (float)ex, fey = (float)ey, fez = (float)ez;
    const float hx = 0.5f * fex, hy = 0.5f * fey, hz = 0.5f * fez;
    const float spx = (float)a.spx, spy = (float)a.spy, spz = (float)a.spz;
    const int u0 = f.u0, v0 = f.v0;
    const int gx0 = x0 + a.offx, gy0 = y0 + a.offy, gz0 = z0 + a.offz;   // the brick's first cell on the lattice
    const int nfu = f.u1 - f.u0 + 1, nfv = f.v1 - f.v0 + 1, nrays = nfu * nfv;
    const bool ufast = !TWO_D && vt(vw, VT_PATCH) == 0.0;
    const int nf = ufast ? nfu : nfv;

    // ---- the footprint's anchor (centre pixel u0 + cu, v0 + cv; pixel offsets
    // stay within half the footprint) and the per-pixel direction steps ----
    const int cu = nfu / 2, cv = nfv / 2;
    const float fnx = (float)vt(vw, VT_N + 0), fny = (float)vt(vw, VT_N + 1), fnz = (float)vt(vw, VT_N + 2);
    const int qf_ = ufast ? VT_DU : VT_DV, qs_ = ufast ? VT_DV : VT_DU;
    const float A0x = uni(an.A0x), A0y = uni(an.A0y), A0z = uni(an.A0z);
    const float Afx = uni(an.Afx), Afy = uni(an.Afy), Afz = uni(an.Afz);
    const float Asx = uni(an.Asx), Asy = uni(an.Asy), Asz = uni(an.Asz);
    const float Dx = uni(an.Dx), Dy = uni(an.Dy), Dz = uni(an.Dz);
    const float DFx = uni((float)vt(vw, qf_ + 0)), DFy = uni((float)vt(vw, qf_ + 1));
    const float DFz = uni((float)vt(vw, qf_ + 2));
    const float DSx = uni((float)vt(vw, qs_ + 0)), DSy = uni((float)vt(vw, qs_ + 1));
    const float DSz = uni((float)vt(vw, qs_ + 2));
    const float tv0 = uni(an.tv0), tv1 = uni(an.tv1);
    // parallel rays: one direction plan for the footprint, and the anchor
    // coefficients of the origin mirrored with it (a sign change is exact)
    constexpr bool SHARED_DIR = !PERSP && !SURF;
    DirPlan dp0{};
    int dead = TWO_D ? 2 : 3;   // an axis no ray of the footprint crosses (3: none)
    float mA0x = A0x, mA0y = A0y, mA0z = A0z, mAfx = Afx, mAfy = Afy, mAfz = Afz, mAsx = Asx, mAsy = Asy,
          mAsz = Asz;
    if (SHARED_DIR) {
        dp0 = dir_plan<LSY, LSZ, TWO_D>(Dx, Dy, Dz, spx, spy, spz, S);
        // wave-uniform: keep the plan in scalar registers
        dp0.axx = uni(dp0.axx); dp0.ayy = uni(dp0.ayy); dp0.azz = uni(dp0.azz);
        dp0.ix = uni(dp0.ix); dp0.iy = uni(dp0.iy); dp0.iz = uni(dp0.iz);
        dp0.LS = uni(dp0.LS);
        dp0.qfx = uni(dp0.qfx); dp0.qfy = uni(dp0.qfy); dp0.qfz = uni(dp0.qfz);
        dp0.qx = (uint32_t)uni((int)dp0.qx); dp0.qy = (uint32_t)uni((int)dp0.qy);
        dp0.qz = (uint32_t)uni((int)dp0.qz);
        if (dp0.nx) { mA0x = -A0x; mAfx = -Afx; mAsx = -Asx; }
        if (dp0.ny) { mA0y = -A0y; mAfy = -Afy; mAsy = -Asy; }
        if (dp0.nz) { mA0z = -A0z; mAfz = -Afz; mAsz = -Asz; }
        if (!TWO_D) dead = uni(dp0.axx == 0.f ? 0 : (dp0.ayy == 0.f ? 1 : (dp0.azz == 0.f ? 2 : 3)));
    }
    const float *ysrc = a.sino + ((size_t)view * a.U + u0) * a.V + v0;
    const uint32_t yfs = ufast ? a.V : 1, yss = ufast ? 1 : a.V;   // sinogram strides, fast / slow

    // Ray r of the footprint is pixel lf = r mod nf of slow row srow(r / nf).
    // Parallel rays take the rows from the centre outwards, so the 64 rays of a
    // round lie at similar distances from the brick's projected centre and walk
    // similar lengths through it (fewer idle lanes than in row order; for
    // fan/cone footprints the gain does not pay for the index arithmetic).
    // (lk, lf) advance by 64 rays per round; yo is the sinogram offset of the
    // ray from (u0, v0).
    const int step_slow = 64 / nf, step_fast = 64 - step_slow * nf;
    const int hs = (nrays / nf) >> 1;
    const auto srow = [hs](int k) {
        return PERSP ? k : hs + ((k & 1) ? -((k + 1) >> 1) : (k >> 1));
    };
    const float af = (float)(ufast ? cu : cv), as_ = (float)(ufast ? cv : cu);
    // Fan/cone rays on a flat detector: each direction component is affine in
    // the ray's (fast, slow) pixel offsets, so over the footprint it takes its
    // extremes at the four corners.  Where every component keeps one sign at
    // the corners with a margin (2^-20 of the largest sum of term magnitudes,
    // far above the rounding of the per-ray sums, about 2^-23 of it, and above
    // the direction plan's near-zero threshold), the footprint is walked with
    // its coefficients mirrored once to positive directions: the signs, the
    // mirroring and the strides are then settled per footprint, not per ray.
    // Mirroring negates operands, which is exact, so the walks are unchanged.
    bool fsign = false;
    float mDx = Dx, mDy = Dy, mDz = Dz, mDFx = DFx, mDFy = DFy, mDFz = DFz, mDSx = DSx, mDSy = DSy,
          mDSz = DSz;
    float kx = 8.f, ky = (float)(8 * LSY), kz = (float)(8 * LSZ), k0 = 0.f;
    uint32_t fstx = 0, fsty = 0, fstz = 0;
    if (PERSP && !SURF && nrays > 0) {
        const int nrow = nrays / nf;
        const float f0 = -af, f1 = (float)(nf - 1) - af, s0 = -as_, s1 = (float)(nrow - 1) - as_;
        const float fm = fmaxf(fabsf(f0), fabsf(f1)), sm = fmaxf(fabsf(s0), fabsf(s1));
        const float Tx = fabsf(Dx) + fm * fabsf(DFx) + sm * fabsf(DSx);
        const float Ty = fabsf(Dy) + fm * fabsf(DFy) + sm * fabsf(DSy);
        const float Tz = TWO_D ? 0.f : fabsf(Dz) + fm * fabsf(DFz) + sm * fabsf(DSz);
        const float thr = 0x1p-20f * fmaxf(Tx, fmaxf(Ty, Tz));
        const auto sgn = [&](float D, float DF, float DS) {
            const float c00 = fmaf(s0, DS, fmaf(f0, DF, D)), c10 = fmaf(s0, DS, fmaf(f1, DF, D));
            const float c01 = fmaf(s1, DS, fmaf(f0, DF, D)), c11 = fmaf(s1, DS, fmaf(f1, DF, D));
            const float lo = fminf(fminf(c00, c10), fminf(c01, c11));
            const float hi = fmaxf(fmaxf(c00, c10), fmaxf(c01, c11));
            return lo > thr ? 1.f : (hi < -thr ? -1.f : 0.f);
        };
        const float sgx = sgn(Dx, DFx, DSx), sgy = sgn(Dy, DFy, DSy);
        const float sgz = TWO_D ? 1.f : sgn(Dz, DFz, DSz);
        fsign = sgx != 0.f && sgy != 0.f && sgz != 0.f;
        if (fsign) {
            mDx = sgx * Dx; mDFx = sgx * DFx; mDSx = sgx * DSx;
            mDy = sgy * Dy; mDFy = sgy * DFy; mDSy = sgy * DSy;
            mDz = sgz * Dz; mDFz = sgz * DFz; mDSz = sgz * DSz;
            mA0x = sgx * A0x; mAfx = sgx * Afx; mAsx = sgx * Asx;
            mA0y = sgy * A0y; mAfy = sgy * Afy; mAsy = sgy * Asy;
            mA0z = sgz * A0z; mAfz = sgz * Afz; mAsz = sgz * Asz;
            // cell offset from the mirrored cell indices: c for a positive
            // axis, e - 1 - c for a mirrored one
            kx = 8.f * sgx;
            ky = (float)(8 * LSY) * sgy;
            kz = (float)(8 * LSZ) * sgz;
            k0 = (sgx < 0.f ? 8.f * (fex - 1.f) : 0.f) + (sgy < 0.f ? (float)(8 * LSY) * (fey - 1.f) : 0.f) +
                 (sgz < 0.f ? (float)(8 * LSZ) * (fez - 1.f) : 0.f);
            fstx = in_vgpr(sgx < 0.f ? (uint32_t)-8 : 8u);
            fsty = in_vgpr(sgy < 0.f ? (uint32_t)(-8 * LSY) : (uint32_t)(8 * LSY));
            fstz = in_vgpr(TWO_D ? 0u : (sgz < 0.f ? (uint32_t)(-8 * LSZ) : (uint32_t)(8 * LSZ)));
        }
    }
    int lk = lane / nf, lf = lane - lk * nf;
    uint32_t yo = __umul24(lf, yfs) + __umul24(srow(lk), yss);   // offsets < 2^24, products < 2^31
    float ynext = 1.f;
    if (MODE != BM_COLINV && lane < nrays) ynext = ysrc[yo];
    // surface: the frame in registers, and each ray's offsets fetched one round
    // ahead like its value (a surface pixel shares the sinogram's pixel index)
    double sCx = 0, sCy = 0, sCz = 0, sUx = 0, sUy = 0, sUz = 0, sVx = 0, sVy = 0, sVz = 0;
    double sNx = 0, sNy = 0, sNz = 0, sDx = 0, sDy = 0, sDz = 0;
    const double *ob = nullptr;
    double o0n = 0, o1n = 0, o2n = 0;
    if (SURF) {
        sCx = vt(vw, VT_C + 0); sCy = vt(vw, VT_C + 1); sCz = vt(vw, VT_C + 2);
        sUx = vt(vw, VT_EU + 0); sUy = vt(vw, VT_EU + 1); sUz = vt(vw, VT_EU + 2);
        sVx = vt(vw, VT_EV + 0); sVy = vt(vw, VT_EV + 1); sVz = vt(vw, VT_EV + 2);
        sNx = vt(vw, VT_EN + 0); sNy = vt(vw, VT_EN + 1); sNz = vt(vw, VT_EN + 2);
        sDx = vt(vw, VT_D00 + 0); sDy = vt(vw, VT_D00 + 1); sDz = vt(vw, VT_D00 + 2);
        if (PERSP) {   // offsets relative to the source: P - S = (C - S) + o . E
            sCx -= vt(vw, VT_O00 + 0); sCy -= vt(vw, VT_O00 + 1); sCz -= vt(vw, VT_O00 + 2);
        }
        ob = a.surf.off + 3 * ((a.surf.per_view ? (size_t)view * a.U * a.V : 0) +
                               (size_t)u0 * a.V + v0);
        if (lane < nrays) { o0n = ob[3 * yo]; o1n = ob[3 * yo + 1]; o2n = ob[3 * yo + 2]; }
    }
    const auto walk_rays = [&](auto fs_tag) __attribute__((always_inline)) {
    constexpr bool FS = decltype(fs_tag)::value;   // mirrored fan/cone footprint
    for (int r = lane; r < nrays; r += 64) {
        const float cf = (float)lf - af, cs = (float)srow(lk) - as_;
        const int pu = ufast ? u0 + lf : u0 + srow(lk), pv = ufast ? v0 + srow(lk) : v0 + lf;   // its pixel
        lf += step_fast;
        lk += step_slow;
        if (lf >= nf) { lf -= nf; lk += 1; }
        yo = __umul24(lf, yfs) + __umul24(srow(lk), yss);
        // take this ray's prefetched values before issuing the next ray's loads, so
        // the wait covers only loads issued a round earlier
        const float yv = ynext;
        const double o0 = o0n, o1 = o1n, o2 = o2n;
        if (r + 64 < nrays) {
            if (MODE != BM_COLINV) ynext = ysrc[yo];
            if (SURF) { o0n = ob[3 * yo]; o1n = ob[3 * yo + 1]; o2n = ob[3 * yo + 2]; }
        }
        if (yv == 0.f) continue;
        float mx, my, mz, t0, t1;   // origin relative to the brick centre, mirrored
        DirPlan dp;
        if (SHARED_DIR) {
            dp = dp0;
            mx = fmaf(cs, mAsx, fmaf(cf, mAfx, mA0x));
            my = fmaf(cs, mAsy, fmaf(cf, mAfy, mA0y));
            mz = TWO_D ? mA0z : fmaf(cs, mAsz, fmaf(cf, mAfz, mA0z));
            t0 = tv0;
            t1 = tv1;
        } else if (FS) {
            mx = fmaf(cs, mAsx, fmaf(cf, mAfx, mA0x));
            my = fmaf(cs, mAsy, fmaf(cf, mAfy, mA0y));
            mz = TWO_D ? mA0z : fmaf(cs, mAsz, fmaf(cf, mAfz, mA0z));
            dp = dir_plan_pos<TWO_D>(fmaf(cs, mDSx, fmaf(cf, mDFx, mDx)), fmaf(cs, mDSy, fmaf(cf, mDFy, mDy)),
                                     fmaf(cs, mDSz, fmaf(cf, mDFz, mDz)), spx, spy, spz, S);
            t0 = tv0;
            t1 = tv1;
        } else {
            float ox, oy, oz, dx, dy, dz;
            if (SURF) {
                // surface pixel: the ray from the table, re-expressed in float64 around
                // the plane through the brick centre parallel to the flat detector
                // (any parameter near the plane will do: the origin is then formed in
                // float64 exactly on the ray for that parameter, so the crossing
                // parameter itself is computed in float32)
                const double px = sCx + o0 * sUx + o1 * sVx + o2 * sNx;
                const double py = sCy + o0 * sUy + o1 * sVy + o2 * sNy;
                const double pz = sCz + o0 * sUz + o1 * sVz + o2 * sNz;
                double rdx, rdy, rdz, bx_, by_, bz_;   // direction; origin relative to the brick centre
                if (PERSP) {
                    rdx = px; rdy = py; rdz = pz;
                    bx_ = vt(vw, VT_O00 + 0) - cbx; by_ = vt(vw, VT_O00 + 1) - cby; bz_ = vt(vw, VT_O00 + 2) - cbz;
                } else {
                    rdx = sDx; rdy = sDy; rdz = sDz;
                    bx_ = px - cbx; by_ = py - cby; bz_ = pz - cbz;
                }
                const float num = -((float)bx_ * fnx + (float)by_ * fny + (float)bz_ * fnz);
                const float den = (float)rdx * fnx + (float)rdy * fny + (float)rdz * fnz;
                const double tr = (double)(num * __builtin_amdgcn_rcpf(den));
                ox = (float)fma(tr, rdx, bx_);
                oy = (float)fma(tr, rdy, by_);
                oz = TWO_D ? A0z : (float)fma(tr, rdz, bz_);
                dx = (float)rdx;
                dy = (float)rdy;
                dz = TWO_D ? 0.f : (float)rdz;
                t0 = (float)(vt(vw, VT_TMIN) - tr);
                t1 = (float)(vt(vw, VT_TMAX) - tr);
            } else {
                ox = fmaf(cs, Asx, fmaf(cf, Afx, A0x));
                oy = fmaf(cs, Asy, fmaf(cf, Afy, A0y));
                oz = TWO_D ? A0z : fmaf(cs, Asz, fmaf(cf, Afz, A0z));
                dx = fmaf(cs, DSx, fmaf(cf, DFx, Dx));
                dy = fmaf(cs, DSy, fmaf(cf, DFy, Dy));
                dz = TWO_D ? 0.f : fmaf(cs, DSz, fmaf(cf, DFz, Dz));
                t0 = tv0;
                t1 = tv1;
            }
            dp = dir_plan<LSY, LSZ, TWO_D>(dx, dy, dz, spx, spy, spz, S);
            mx = dp.nx ? -ox : ox;
            my = dp.ny ? -oy : oy;
            mz = dp.nz ? -oz : oz;
        }
        // slab clip: lo = (-h - m) / a, hi = (h - m) / a; an axis the ray does
        // not move along holds it for every t iff -h <= m < h
        float cx = -hx - mx, cy = -hy - my, cz = -hz - mz, cix = dp.ix, ciy = dp.iy, ciz = dp.iz;
        if (!FS && dp.slow) {
            // On an axis the ray does not move along, its cell comes from its
            // float64 origin as the forward forms it (pixel_origin / pixel_ray,
            // on_plane), so both sides agree on rays that lie in a lattice plane;
            // the ray's float32 coordinate there is moved to that cell's centre.
            const auto zero_axis = [&](int k, float ad, int g0, int e, float h, float &m, float &c,
                                       float &ci) __attribute__((always_inline)) {
                if (ad == 0.f) {
                    double o;
                    if constexpr (SURF) {
                        double p[3], q[3];
                        pixel_ray(vw, a.surf, view, pu, pv, a.U, a.V, p[0], p[1], p[2], q[0], q[1], q[2]);
                        o = p[k];
                    } else if constexpr (PERSP) {
                        o = vt(vw, VT_O00 + k);   // the source (pixel_origin of every pixel)
                    } else {
                        o = pixel_origin(vw, k, pu, pv);
                    }
                    const double l = on_plane(o) - (double)g0;
                    const bool in = l >= 0.0 && l < (double)e;
                    m = in ? (float)floor(l) + 0.5f - h : 0.f;
                    c = in ? -h : 1.f;   // lo -> -inf / +inf
                    ci = 1e35f;
                }
            };
            zero_axis(0, dp.axx, gx0, ex, hx, mx, cx, cix);
            zero_axis(1, dp.ayy, gy0, ey, hy, my, cy, ciy);
            if (!TWO_D) zero_axis(2, dp.azz, gz0, ez, hz, mz, cz, ciz);
        }
        const float lox = cx * cix, hix = fmaf(fex, cix, lox);
        const float loy = cy * ciy, hiy = fmaf(fey, ciy, loy);
        const float loz = TWO_D ? -3e38f : cz * ciz;
        const float hiz = TWO_D ? 3e38f : fmaf(fez, ciz, loz);
        const float tin = fmaxf(fmaxf(fmaxf(lox, loy), loz), t0);
        const float tout = fminf(fminf(fminf(hix, hiy), hiz), t1);
        if (!(tin < tout)) continue;
        IWalk w;
        w.qx = dp.qx;
        w.qy = dp.qy;
        w.qz = dp.qz;
        float fcx, fcy, fcz = 0.f;
        uint32_t farx, fary, farz = 0xFFFFFFFFu;
        baxis(mx, dp.axx, tin, hx, fex - 1.f, dp.qfx, w.qx, fcx, w.lx, farx);
        baxis(my, dp.ayy, tin, hy, fey - 1.f, dp.qfy, w.qy, fcy, w.ly, fary);
        if (!TWO_D) baxis(mz, dp.azz, tin, hz, fez - 1.f, dp.qfz, w.qz, fcz, w.lz, farz);
        else w.lz = 0xFFFFFFFFu;
        // the walk ends at the ray's own end (a segment may stop inside the
        // brick) or at the first far-face crossing, whichever comes first
        w.lend = min(sat_u32((tout - tin) * dp.LS), min(min(farx, fary), farz));
        // back to real cell indices (exact small integers in float) and strides
        if (FS) {
            w.idx = (uint32_t)fmaf(fcz, kz, fmaf(fcy, ky, fmaf(fcx, kx, k0)));
            w.stx = fstx;
            w.sty = fsty;
            w.stz = fstz;
        } else {
            const float rcx = dp.nx ? fex - 1.f - fcx : fcx;
            const float rcy = dp.ny ? fey - 1.f - fcy : fcy;
            const float rcz = dp.nz ? fez - 1.f - fcz : fcz;
            w.idx = (uint32_t)fmaf(rcz, (float)(8 * LSZ), fmaf(rcy, (float)(8 * LSY), rcx * 8.f));
            w.stx = in_vgpr(dp.stx);
            w.sty = in_vgpr(dp.sty);
            w.stz = in_vgpr(dp.stz);
        }
        // the ray value in fixed point: rays within 2^6 of the brick's largest as
        // they are (|Y| >= 2^17), smaller ones (and all rays when the geometry
        // asks for a shift) as a 24-bit mantissa with the product shifted back
        const float Yf = yv * yscale;   // |Yf| < 2^23
        const bool mant = a.yshift != 0 || fabsf(Yf) < 0x1p17f;
        if (__builtin_amdgcn_ballot_w64(mant)) {
            const int up = mant ? 23 - __builtin_amdgcn_frexp_expf(Yf) : 0;
            const int sh = up + a.yshift;
            const int Y = (int)rintf(__builtin_amdgcn_fmed3f(ldexpf(Yf, up), -8388607.f, 8388607.f));
            if (sh <= 46) {   // else every term is below one unit
                if (dead < 3) iwalk2_scatter_fix<true>(live_axes(w, dead), acc, Y, sh);
                else iwalk_scatter_fix<true>(w, acc, Y, sh);
            }
        } else {
            const int Y = (int)rintf(__builtin_amdgcn_fmed3f(Yf, -8388607.f, 8388607.f));
            if (dead < 3) iwalk2_scatter_fix<false>(live_axes(w, dead), acc, Y, 0);
            else iwalk_scatter_fix<false>(w, acc, Y, 0);
        }
    }
    };
    // Parallel rays with an untraversed axis d whose footprint's fast pixel
    // step runs along d alone: the rays of a row differ only in their d
    // coordinate, so they have the same walk through the other two axes.  A
    // lane then takes a packet of kPacket consecutive rays of a row: one
    // set-up and one walk, one term per ray (a ray outside the brick's d slab,
    // or past the row's end, gets Y = 0).  The arithmetic is that of the ray
    // path above, term by term, so the sums are the same.
    const auto walk_packets = [&]() __attribute__((always_inline)) {
        constexpr int K = kPacket;
        // slots: live axes a < b (x, y, z order), untraversed axis d (values
        // picked by value, so no reference is selected)
        const int d = dead;
        const auto A = [d](auto x, auto y, auto z) { return d == 0 ? y : x; };
        const auto B = [d](auto x, auto y, auto z) { return d == 2 ? y : z; };
        const auto Dd = [d](auto x, auto y, auto z) { return d == 0 ? x : (d == 1 ? y : z); };
        const float ha = A(hx, hy, hz), hb = B(hx, hy, hz);
        const float ea = A(fex, fey, fez), eb = B(fex, fey, fez), ed = Dd(fex, fey, fez);
        const int ied = Dd(ex, ey, ez), gd0 = Dd(gx0, gy0, gz0);
        const float A0a = A(mA0x, mA0y, mA0z), A0b = B(mA0x, mA0y, mA0z);
        const float Asa = A(mAsx, mAsy, mAsz), Asb = B(mAsx, mAsy, mAsz);
        const float ia = A(dp0.ix, dp0.iy, dp0.iz), ib = B(dp0.ix, dp0.iy, dp0.iz);
        const float aa = A(dp0.axx, dp0.ayy, dp0.azz), ab = B(dp0.axx, dp0.ayy, dp0.azz);
        const float qfa = A(dp0.qfx, dp0.qfy, dp0.qfz), qfb = B(dp0.qfx, dp0.qfy, dp0.qfz);
        const uint32_t qa = A(dp0.qx, dp0.qy, dp0.qz), qb = B(dp0.qx, dp0.qy, dp0.qz);
        const bool na = A(dp0.nx, dp0.ny, dp0.nz), nb = B(dp0.nx, dp0.ny, dp0.nz), nd = Dd(dp0.nx, dp0.ny, dp0.nz);
        constexpr uint32_t SX = 8u, SY = 8u * LSY, SZ = 8u * LSZ;   // LDS byte strides
        const uint32_t Sa = A(SX, SY, SZ), Sb = B(SX, SY, SZ), Sd = Dd(SX, SY, SZ);
        const uint32_t sta = in_vgpr(na ? 0u - Sa : Sa), stb = in_vgpr(nb ? 0u - Sb : Sb);
        const float LS = dp0.LS;
        const int nrow = nrays / nf, np = (nf + K - 1) / K, npk = nrow * np;
        const int pstep_slow = 64 / np, pstep_fast = 64 - pstep_slow * np;
        int prow = lane / np, pp = lane - prow * np;
        for (int r = lane; r < npk; r += 64) {
            const int lf0 = pp * K, row = srow(prow);
            const int kk = min(K, nf - lf0);
            pp += pstep_fast;
            prow += pstep_slow;
            if (pp >= np) { pp -= np; prow += 1; }
            const float cs = (float)row - as_, cf0 = (float)lf0 - af;
            const uint32_t yo = __umul24(lf0, yfs) + __umul24(row, yss);
            float yv[K];
#pragma unroll
            for (int j = 0; j < K; ++j)
                yv[j] = j < kk ? (MODE == BM_COLINV ? 1.f : ysrc[yo + j * yfs]) : 0.f;
            // the live axes: shared by the packet (their fast-step terms are 0)
            const float ma = fmaf(cs, Asa, A0a), mb = fmaf(cs, Asb, A0b);
            const float loa = (-ha - ma) * ia, hia = fmaf(ea, ia, loa);
            const float lob = (-hb - mb) * ib, hib = fmaf(eb, ib, lob);
            const float tin = fmaxf(fmaxf(loa, lob), tv0);
            const float tout = fminf(fminf(hia, hib), tv1);
            if (!(tin < tout)) continue;
            IWalk2 w;
            float fca, fcb;
            uint32_t fara, farb;
            baxis(ma, aa, tin, ha, ea - 1.f, qfa, qa, fca, w.la, fara);
            baxis(mb, ab, tin, hb, eb - 1.f, qfb, qb, fcb, w.lb, farb);
            w.qa = qa;
            w.qb = qb;
            w.sa = sta;
            w.sb = stb;
            w.lend = min(sat_u32((tout - tin) * LS), min(fara, farb));
            const float rca = na ? ea - 1.f - fca : fca, rcb = nb ? eb - 1.f - fcb : fcb;
            w.idx = (uint32_t)rca * Sa + (uint32_t)rcb * Sb;
            // per ray: its cell of the untraversed axis and its fixed-point value
            float Yf[K];
            uint32_t off[K];
            bool mant_any = false;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                // the cell on d from the ray's float64 origin as the forward forms it
                // (pixel_origin, on_plane), so both sides agree on rays in a lattice plane
                const int pf = lf0 + j;
                const double ld = on_plane(pixel_origin(vw, d, ufast ? u0 + pf : u0 + row, ufast ? v0 + row : v0 + pf)) -
                                  (double)gd0;
                const bool in = ld >= 0.0 && ld < (double)ied;
                const float fcd = in ? (float)floor(ld) : 0.f;
                off[j] = (uint32_t)(nd ? ed - 1.f - fcd : fcd) * Sd;
                Yf[j] = in ? yv[j] * yscale : 0.f;   // |Yf| < 2^23
                mant_any = mant_any || (Yf[j] != 0.f && (a.yshift != 0 || fabsf(Yf[j]) < 0x1p17f));
            }
            bool some = false, consec = true;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                some = some || Yf[j] != 0.f;
                consec = consec && off[j] == off[0] + j * Sd;
            }
            if (!some) continue;
            // consecutive cells (every ray's, also those without a value):
            // the walk's cell takes ray 0's, the others are immediate offsets
            const bool cw = __builtin_amdgcn_ballot_w64(!consec) == 0;
            if (cw) {
                w.idx += off[0];
#pragma unroll
                for (int j = 0; j < K; ++j) off[j] = 0u;
            }
            const auto walk = [&](auto shift_tag, const int(&Y)[K], const int(&sh)[K]) {
                constexpr bool SH = decltype(shift_tag)::value;
                if (cw && d == 0) iwalk2_scatter_packet<SH, K, SX>(w, acc, Y, sh, off);
                else if (cw && d == 1) iwalk2_scatter_packet<SH, K, SY>(w, acc, Y, sh, off);
                else if (cw) iwalk2_scatter_packet<SH, K, SZ>(w, acc, Y, sh, off);
                else iwalk2_scatter_packet<SH, K, 0>(w, acc, Y, sh, off);
            };
            int Y[K], sh[K];
            if (__builtin_amdgcn_ballot_w64(mant_any)) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    const bool mant = a.yshift != 0 || fabsf(Yf[j]) < 0x1p17f;
                    const int up = mant ? 23 - __builtin_amdgcn_frexp_expf(Yf[j]) : 0;
                    sh[j] = up + a.yshift;
                    const int Yv = (int)rintf(__builtin_amdgcn_fmed3f(ldexpf(Yf[j], up), -8388607.f, 8388607.f));
                    Y[j] = sh[j] <= 46 ? Yv : 0;   // else every term is below one unit
                    sh[j] = min(sh[j], 46);
                }
                walk(std::true_type{}, Y, sh);
            } else {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    Y[j] = (int)rintf(__builtin_amdgcn_fmed3f(Yf[j], -8388607.f, 8388607.f));
                    sh[j] = 0;
                }
                walk(std::false_type{}, Y, sh);
            }
        }
    };
    if constexpr (PERSP && !SURF) {
        if (fsign) walk_rays(std::true_type{});
        else walk_rays(std::false_type{});
    } else if constexpr (SHARED_DIR && !TWO_D) {
        // exactly one untraversed axis, and the fast pixel step along it alone
        const bool pk = dead == 0   ? (mAfy == 0.f && mAfz == 0.f && dp0.ayy != 0.f && dp0.azz != 0.f)
                        : dead == 1 ? (mAfx == 0.f && mAfz == 0.f && dp0.axx != 0.f && dp0.azz != 0.f)
                        : dead == 2 ? (mAfx == 0.f && mAfy == 0.f && dp0.axx != 0.f && dp0.ayy != 0.f)
                                    : false;
        if (pk) walk_packets();
        else walk_rays(std::false_type{});
    } else {
        walk_rays(std::false_type{});
    }
}

// Write-out of one brick: each voxel's adjoint value val(lx, ly, lz) (local
// indices) goes once to the volume through the mode's epilogue: A^T (written or
// added), the SIRT update x += relax C A^T e (optionally masked and clamped), the
// CGLS adjoint with its fused vector updates and the brick's sum of squares, or
// the column weights 1 / (A^T 1).
template <int BX, int BY, int BZ, int NT, int MODE, class F>
__device__ __forceinline__ void brick_writeout(const BrickArgs &a, int x0, int y0, int z0, int ex, int ey,
                                               int ez, F &&val_of) {
    const float alpha = (MODE == BM_CGLS && a.x_upd) ? (float)a.state[CS_ALPHA] : 0.f;
    double sq = 0.0;
    for (int i = threadIdx.x; i < BX * BY * BZ; i += NT) {
        const int lx = i % BX, ly = (i / BX) % BY, lz = i / (BX * BY);
        if (lx < ex && ly < ey && lz < ez) {
            const size_t g = ((size_t)(z0 + lz) * a.H + (y0 + ly)) * a.W + (x0 + lx);
            const float val = val_of(lx, ly, lz);
            if (MODE == BM_BACKPROJECT) {
                a.vol[g] = a.accumulate ? a.vol[g] + val : val;
            } else if (MODE == BM_SIRT_UPDATE) {
                if (!a.mask || a.mask[g]) {
                    float v = fmaf(a.relax * a.cinv[g], val, a.vol[g]);
                    if (a.bounded) v = fminf(fmaxf(v, a.lo), a.hi);
                    a.vol[g] = v;
                }
            } else if (MODE == BM_CGLS) {
                a.vol[g] = val;
                sq += (double)val * val;
                if (a.p_copy) a.p_copy[g] = val;
                if (a.x_upd) a.x_upd[g] = fmaf(alpha, a.p_old[g], a.x_upd[g]);
            } else {
                const float r = val > 0.f ? 1.0f / val : 0.f;
                a.vol[g] = isfinite(r) ? r : 0.f;
            }
        }
    }
    if (MODE == BM_CGLS) {
        // fixed-order block sum (float64), one partial per brick
        __shared__ double wsq[NT / 64];
        const double t = block_sum<NT>(sq, wsq);
        if (threadIdx.x == 0) a.partial[blockIdx.x] = t;
    }
}

// Two 512-thread workgroups (or four of 256, one of 1024) share a CU through
// their LDS, i.e. 4 waves per SIMD; the register budget is held to that.
// SURF: parameterized detector surface (per-pixel rays from the offsets table).
// REC: footprints and anchors come from the launch's record table (a.rec).
template <int BX, int BY, int BZ, int NT, int MODE, bool SURF, bool PERSP, bool REC>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void brick_kernel(
    BrickArgs a) {
    constexpr int LSY = BX + 1;           // padded LDS strides (elements): rays of a
    constexpr int LSZ = LSY * BY + 1;     // wave that differ only in y or z hit
    constexpr int LN = LSZ * BZ;          // different banks
    constexpr int NWAVES = NT / 64;
    __shared__ unsigned long long acc[LN];
    __shared__ float wave_max[NWAVES];
    // footprints found in pass 1, reused by pass 2 (u1 < u0: the view misses
    // the brick); for up to kFpCache views on detectors below 2^16 pixels a
    // side, and only where the LDS still holds the workgroups of 4 waves per SIMD
    constexpr bool FPC = !REC && (LN * 8 + kFpCache * 8 + 1024) * (1024 / NT) <= 160 * 1024;
    __shared__ ushort4 fpc[FPC ? kFpCache : 1];
    for (int i = threadIdx.x; i < LN; i += NT) acc[i] = 0ull;

    const int blk = xcd_remap(blockIdx.x, a.n_blocks);
    const int bxi = blk % a.nbx;
    const int byi = (blk / a.nbx) % a.nby;
    const int bzi = blk / (a.nbx * a.nby);
    const int x0 = bxi * BX, y0 = byi * BY, z0 = bzi * BZ;   // within the volume buffer
    const int ex = min(BX, a.W - x0), ey = min(BY, a.H - y0), ez = min(BZ, a.D - z0);
    const int gx0 = x0 + a.offx, gy0 = y0 + a.offy, gz0 = z0 + a.offz;   // on the lattice
    const double cbx = gx0 + 0.5 * ex, cby = gy0 + 0.5 * ey, cbz = gz0 + 0.5 * ez;
    const int lane = threadIdx.x & 63, wv = uni((int)(threadIdx.x >> 6));
    constexpr bool TWO_D = BZ == 1;   // single-slice bricks serve the 2D beams only
    if (MODE == BM_SIRT_UPDATE && a.mask) {
        // a brick with no voxel to update does no work at all
        int any = 0;
        for (int i = threadIdx.x; i < BX * BY * BZ; i += NT) {
            const int lx = i % BX, ly = (i / BX) % BY, lz = i / (BX * BY);
            if (lx < ex && ly < ey && lz < ez)
                any |= a.mask[((size_t)(z0 + lz) * a.H + (y0 + ly)) * a.W + (x0 + lx)] != 0;
        }
        if (!__syncthreads_or(any)) return;
    }
    const bool two_d = TWO_D;
    const float spx = (float)a.spx, spy = (float)a.spy, spz = (float)a.spz;

    // ---- pass 1: largest |y| over the rays that can meet this brick ----
    // Footprints come from the record table when the launch has one, else they
    // are computed here and kept in LDS for pass 2.
    const ConstRecPtr rec = REC ? (ConstRecPtr)a.rec + (size_t)blk * a.rec_stride : nullptr;
    float ymax = 1.f;
    const bool cache = !REC && FPC && MODE != BM_COLINV && a.n_views <= kFpCache && a.U < 65536 && a.V < 65536;
    const auto rec_footprint = [&](int view, Footprint &f) {
        const uint32_t fu = rec[view].fu, fv = rec[view].fv;
        f.u0 = uni((int)(fu & 0xFFFFu));
        f.u1 = uni((int)(fu >> 16));
        f.v0 = uni((int)(fv & 0xFFFFu));
        f.v1 = uni((int)(fv >> 16));
        return f.u0 <= f.u1;
    };
    if (MODE != BM_COLINV) {
        float m = 0.f;
        // the next view's footprint words are fetched one view ahead
        uint32_t nxu = 1u, nxv = 0u;
        if (REC && wv < a.n_views) { nxu = rec[wv].fu; nxv = rec[wv].fv; }
        for (int view = wv; view < a.n_views; view += NWAVES) {
            const double *vw = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
            Footprint f;
            bool seen;
            if constexpr (REC) {
                const uint32_t fu = nxu, fv = nxv;
                if (view + NWAVES < a.n_views) { nxu = rec[view + NWAVES].fu; nxv = rec[view + NWAVES].fv; }
                f.u0 = uni((int)(fu & 0xFFFFu));
                f.u1 = uni((int)(fu >> 16));
                f.v0 = uni((int)(fv & 0xFFFFu));
                f.v1 = uni((int)(fv >> 16));
                seen = f.u0 <= f.u1;
            } else {
                seen = brick_footprint(vw, lane, gx0, gy0, gz0, ex, ey, ez, a.U, a.V, two_d,
                                       a.env ? a.env + (size_t)view * env_size(a.U, a.V) : nullptr, f);
                if (cache && lane == 0)
                    fpc[view] = seen ? make_ushort4((unsigned short)f.u0, (unsigned short)f.u1,
                                                    (unsigned short)f.v0, (unsigned short)f.v1)
                                     : make_ushort4(1, 0, 0, 0);
            }
            if (!seen) continue;
            const int nfu = f.u1 - f.u0 + 1;
            if (a.y_vec4) {
                // aligned groups of four pixels of each footprint row: the groups at
                // the row's ends may hold pixels beyond the footprint, which only
                // raise the maximum (the scale stays valid, a little coarser)
                const int g0 = f.v0 >> 2, ng = (f.v1 >> 2) - g0 + 1, n = nfu * ng;
                const float4 *ysrc = (const float4 *)(a.sino + ((size_t)view * a.U + f.u0) * a.V) + g0;
                const int rowg = a.V >> 2;
                const int step_slow = 64 / ng, step_fast = 64 - step_slow * ng;
                int iu = lane / ng, ig = lane - (lane / ng) * ng;
                // four independent loads in flight per round; a lane past the end
                // reloads the footprint's first group, which leaves the maximum as is
                for (int r = lane; r < n; r += 256) {
                    float4 q[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        q[k] = ysrc[r + 64 * k < n ? iu * rowg + ig : 0];
                        ig += step_fast;
                        iu += step_slow;
                        if (ig >= ng) { ig -= ng; iu += 1; }
                    }
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        m = fmaxf(m, fmaxf(fmaxf(fabsf(q[k].x), fabsf(q[k].y)), fmaxf(fabsf(q[k].z), fabsf(q[k].w))));
                }
            } else {
                const int nfv = f.v1 - f.v0 + 1, nrays = nfu * nfv;
                const float *ysrc = a.sino + ((size_t)view * a.U + f.u0) * a.V + f.v0;
                const int step_slow = 64 / nfv, step_fast = 64 - step_slow * nfv;
                int iu = lane / nfv, iv = lane - (lane / nfv) * nfv;
                for (int r = lane; r < nrays; r += 64) {
                    m = fmaxf(m, fabsf(ysrc[(size_t)iu * a.V + iv]));
                    iv += step_fast;
                    iu += step_slow;
                    if (iv >= nfv) { iv -= nfv; iu += 1; }
                }
            }
        }
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        if (lane == 0) wave_max[wv] = m;
        __syncthreads();
        ymax = 0.f;
        for (int k = 0; k < NWAVES; ++k) ymax = fmaxf(ymax, wave_max[k]);
    } else {
        __syncthreads();
    }
    // Ray values in fixed point: |y| * yscale < 2^23 for every ray of the brick.
    const float yscale = ymax > 0.f ? ldexpf(1.f, 22 - ilogbf(ymax)) : 1.f;

    // ---- pass 2: walk every footprint ray through the brick ----
    // Walk units: just under 2^23 per voxel diagonal.  A piece never exceeds the
    // ray's crossing length of one cell along its major axis, which is at most
    // the voxel diagonal, so piece lengths fit the 24-bit multiplier.
    const float vdiag = two_d ? sqrtf(spx * spx + spy * spy) : sqrtf(spx * spx + spy * spy + spz * spz);
    const float S = kPieceUnits / vdiag;
    for (int view = wv; view < a.n_views; view += NWAVES) {
        const double *vw = a.views + (size_t)view * CT_VIEW_TABLE_STRIDE;
        Footprint f;
        Anchor an;
        if constexpr (REC) {
            if (!rec_footprint(view, f)) continue;
            an = rec_anchor(rec + view);
        } else {
            if (cache) {
                const ushort4 c = fpc[view];   // written by this wave in pass 1
                f.u0 = uni((int)c.x);
                f.u1 = uni((int)c.y);
                f.v0 = uni((int)c.z);
                f.v1 = uni((int)c.w);
                if (f.u1 < f.u0) continue;
            } else if (!brick_footprint(vw, lane, gx0, gy0, gz0, ex, ey, ez, a.U, a.V, two_d,
                                        a.env ? a.env + (size_t)view * env_size(a.U, a.V) : nullptr, f)) {
                continue;
            }
            an = make_anchor(vw, f, cbx, cby, cbz, !TWO_D && vt(vw, VT_PATCH) == 0.0);
        }
        // PERSP: every view of the geometry is fan/cone (else parallel)
        brick_rays<LSY, LSZ, MODE, PERSP, TWO_D, SURF>(a, vw, view, f, an, lane, x0, y0, z0, ex, ey, ez, cbx,
                                                       cby, cbz, S, yscale, acc);
    }
    __syncthreads();
    const double inv_scale = ldexp(1.0, a.yshift) / ((double)S * (double)yscale);
    brick_writeout<BX, BY, BZ, NT, MODE>(a, x0, y0, z0, ex, ey, ez, [&](int lx, int ly, int lz) {
        return (float)((double)(long long)acc[lz * LSZ + ly * LSY + lx] * inv_scale);
    });
}

// ---------------------------------------------------------------------------
// line adjoint: separable parallel views (LineView)
// ---------------------------------------------------------------------------
//
// Every view of the geometry lies in planes of one volume axis d (a tilt series
// about a volume axis with one detector column per voxel plane).  One 512-thread
// workgroup owns a brick (kLineShapes: 32 x 32 x 16 voxels with lines of 32 when
// no view's planes are z planes, else 16 x 16 x 32 with lines of 16).  Views are
// taken family by family (d = x, y, z); within a family every thread owns a
// segment (line) of voxels along d at one in-plane cell.  Per view the workgroup
// stages in LDS the rows of the view that can meet its brick, for the pixel
// columns whose planes hold its voxels; each thread then finds the rows meeting
// its cell (one or two), forms each ray's chord through the cell once, from the
// ray's offset to the cell centre (the trapezoid of a unit square), and adds
// chord * value to the voxels of its line.  No ray is walked and nothing is
// added atomically: sums run in float32 registers over 32 views, then into the
// brick's float32 accumulator in LDS (each voxel belongs to one line per family),
// which is written once.
constexpr int kLinePitch = 36;   // floats per staged row: up to 32 pixel columns, padded
typedef const __attribute__((address_space(4))) LineView *ConstLinePtr;
// a view's entry, field by field (scalar loads)
__device__ __forceinline__ LineView load_line(ConstLinePtr p) {
    LineView L;
    L.E0 = p->E0; L.dq = p->dq; L.X0 = p->X0; L.Xq = p->Xq; L.na = p->na; L.nb = p->nb;
    L.inv_dq = p->inv_dq; L.naf = p->naf; L.nbf = p->nbf; L.H = p->H; L.R = p->R; L.Lmax = p->Lmax;
    L.inv_dqf = p->inv_dqf; L.d = p->d; L.P = p->P; L.g = p->g; L.kc = p->kc; L.aligned = p->aligned;
    L.next = p->next;
    return L;
}

// One family of views (untraversed axis D) of one brick: sums into acc.
template <int MODE, int D, int SHAPE, int LSY, int LSZ>
__device__ __forceinline__ void line_family(const BrickArgs &a, ConstLinePtr lv, float *acc,
                                            float (&stage)[2][kLineShapes[SHAPE].rows * kLinePitch], int &buf,
                                            int x0, int y0, int z0, int ex, int ey, int ez) {
    constexpr int NT = 512;
    constexpr LineShape SH = kLineShapes[SHAPE];
    constexpr int SEG = SH.seg, ROWS = SH.rows;
    constexpr int AX = D == 0 ? 1 : 0, BXS = D == 2 ? 1 : 2;   // in-plane axes a < b
    constexpr int EXT[3] = {SH.bx, SH.by, SH.bz};
    constexpr int EA = EXT[AX], EB = EXT[BXS];
    constexpr int W = EXT[D];                                  // staged pixel columns (the brick along D)
    static_assert(EA * EB * (W / SEG) == NT, "one segment per thread");
    static_assert(W <= kLinePitch - 4, "staged row pitch");
    // staged values per thread: 64 rows (at most) of W columns, whichever way the
    // threads run over them (rows past the view's count are not loaded)
    static_assert(ROWS <= 64, "staged rows");
    constexpr int NSLOT = W * 64 / NT;
    const int tid = threadIdx.x;
    // this thread's segment: cell (la, lb), voxels s0 .. s0 + SEG - 1 along D
    const int la = tid % EA, lb = (tid / EA) % EB, s0 = (tid / (EA * EB)) * SEG;
    const int gd = D == 0 ? x0 + a.offx : (D == 1 ? y0 + a.offy : z0 + a.offz);   // on the lattice
    const int ga = AX == 0 ? x0 + a.offx : y0 + a.offy, gb = BXS == 1 ? y0 + a.offy : z0 + a.offz;
    const int ea = AX == 0 ? ex : ey, eb = BXS == 1 ? ey : ez, ed = D == 0 ? ex : (D == 1 ? ey : ez);
    const bool live = la < ea && lb < eb && s0 < ed;
    // the cell centre relative to the cross-section's centre (exact in float64)
    const double ca = la + 0.5 - 0.5 * ea, cb = lb + 0.5 - 0.5 * eb;
    int view = 0;
    while (view < a.n_views && lv[view].d != D) ++view;
    if (view >= a.n_views) return;
    float part[SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) part[j] = 0.f;
    int batch = 0;
    // the thread's slots of the staged block: slot m holds row i0 + m di, column
    // j0 + m dj; along its slots the pixel's v stays fixed and u steps
    const auto slot0 = [&](int P, int &i0, int &j0, int &di, int &dj) {
        if (P == 0) {   // p = u, q = v: threads along the rows (memory order), NSLOT
                        // consecutive columns each
            i0 = tid & 63;
            j0 = (tid >> 6) * NSLOT;
            di = 0;
            dj = 1;
        } else {        // p = v, q = u: threads along the columns (memory order)
            j0 = tid & (W - 1);
            i0 = tid / W;
            di = NT / W;
            dj = 0;
        }
    };
    // A view's per-brick quantities (wave-uniform): the rows of the view that can
    // meet the brick, referred to the row nearest the centre of the brick's
    // cross-section, so the per-cell arithmetic meets small numbers.
    struct Head {
        LineView L;
        double qr, C0d;
        int qref, rlo, nrows;
    };
    const auto head = [&](int v, Head &h) __attribute__((always_inline)) {
        h.L = load_line(lv + v);
        const double Eref = h.L.E0 - h.L.na * (ga + 0.5 * ea) - h.L.nb * (gb + 0.5 * eb);
        h.qr = rint(-Eref * h.L.inv_dq);
        h.qref = uni((int)h.qr);
        h.C0d = uni(fma(h.qr, h.L.dq, Eref));
        const float w = 0.5f * (fabsf(h.L.naf) * (float)ea + fabsf(h.L.nbf) * (float)eb);
        const float C0 = (float)h.C0d;
        const float r1 = (-h.L.H - w - C0) * h.L.inv_dqf, r2 = (h.L.H + w - C0) * h.L.inv_dqf;
        h.rlo = uni((int)floorf(fminf(r1, r2)) - 1);
        h.nrows = uni(min(ROWS, (int)ceilf(fmaxf(r1, r2)) + 2 - h.rlo));
    };
    // This thread's values of a view's staged block (rows q = qref + rlo + i, pixel
    // columns p = g (gd + j - kc), zero off the detector), loaded along the
    // sinogram's contiguous v.  Columns past the brick are loaded too (they only
    // reach voxels that are never written out), and so are rows past the view's
    // count (never stored); a row off the detector in v reads nothing, through an
    // offset past the buffer.
    const auto fetch = [&](int v, const Head &h, float (&ld)[NSLOT]) __attribute__((always_inline)) {
        int i0, j0, di, dj;
        slot0(h.L.P, i0, j0, di, dj);
        const int q0 = h.qref + h.rlo + i0, p0 = h.L.g * (gd + j0 - h.L.kc);
        const int u0 = h.L.P == 0 ? p0 : q0, vv = h.L.P == 0 ? q0 : p0;
        const int du = h.L.P == 0 ? h.L.g * dj : di;
        const bool vok = vv >= 0 && vv < a.V;
        // the view's pixels as one buffer: offsets of pixels off the detector in u
        // fall outside it (a negative one wraps high) and read 0
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(a.sino + (size_t)v * a.U * a.V, (uint32_t)(a.U * a.V) * 4u);
        // (24-bit products: validated detector sides are under 2^20 pixels)
        const uint32_t off0 = (uint32_t)(__mul24(u0, a.V) + vv) * 4u;
        const uint32_t dstep = (uint32_t)uni(du * a.V * 4);
#pragma unroll
        for (int m = 0; m < NSLOT; ++m) {
            const int u = u0 + m * du;
            if (MODE == BM_COLINV)
                ld[m] = (vok && u >= 0 && u < a.U) ? 1.f : 0.f;
            else
                ld[m] = load_f32(rs, vok ? off0 + m * dstep : 0x80000000u);
        }
    };
    const auto stash = [&](const Head &h, const float (&ld)[NSLOT], float *st) __attribute__((always_inline)) {
        int i0, j0, di, dj;
        slot0(h.L.P, i0, j0, di, dj);
        if (h.L.P == 0) {   // a row's NSLOT consecutive columns: one store
            if (i0 < h.nrows) {
                float *dst = st + i0 * kLinePitch + j0;
                if constexpr (NSLOT == 4)
                    *(float4 *)dst = make_float4(ld[0], ld[1], ld[2], ld[3]);
                else
                    *(float2 *)dst = make_float2(ld[0], ld[1]);
            }
        } else {
#pragma unroll
            for (int m = 0; m < NSLOT; ++m) {
                const int i = i0 + m * di;
                if (i < h.nrows) st[i * kLinePitch + j0] = ld[m];
            }
        }
    };
    // Software pipeline: a view's block is loaded into registers while the
    // workgroup sums the view before it, and stored to the other staging buffer
    // at the top of its own turn; one barrier per view.
    Head h;
    float ld[NSLOT];
    head(view, h);
    fetch(view, h, ld);
    for (;;) {
        stash(h, ld, stage[buf]);
        const bool last = h.L.next == 0 || view + h.L.next >= a.n_views;
        const int nview = view + h.L.next;
        Head hn;
        float ldn[NSLOT];
        if (!last) {
            head(nview, hn);
            fetch(nview, hn, ldn);
        }
        __syncthreads();
        const float *st = stage[buf];
        const LineView &L = h.L;
        const int rlo = h.rlo, nrows = h.nrows;
        const double qr = h.qr, C0d = h.C0d;
        // the rows meeting this cell, each with its chord, summed into the segment
        if (live) {
            // offset of row qref + r from this cell's centre: C + r dq, formed in
            // float64 for the first candidate (offsets of tens of voxels cancel to
            // under one, and near-axis rays have chord ramps as steep as 1 / sin of
            // their angle to the axis), then stepped by dq
            const double Cd = C0d - L.na * ca - L.nb * cb;
            const float C = (float)Cd;
            // rows strictly inside the window |offset| < H meet the cell; oblique rays
            // at its edge have zero chord, aligned ones there are decided below
            const float t1 = (-L.H - C) * L.inv_dqf, t2 = (L.H - C) * L.inv_dqf;
            const int edge = L.aligned ? 0 : 1;
            const int rA = max((int)floorf(fminf(t1, t2)) + edge, rlo);
            const int rB = min((int)ceilf(fmaxf(t1, t2)) - edge, rlo + nrows - 1);
            float dl = 0.f, step = 0.f;
            const double cell = L.aligned == 1 ? ga + la : gb + lb;
            if (!L.aligned) {
                dl = (float)fma((double)rA, L.dq, Cd);
                step = (float)L.dq;
            }
            const float *row = st + (rA - rlo) * kLinePitch + s0;
            for (int r = rA; r <= rB; ++r, row += kLinePitch) {
                float Lc;
                if (L.aligned) {
                    // the rays' constant coordinate relative to this cell, per row in
                    // float64 and settled on the lattice planes (on_plane): a ray in a
                    // cell's lower plane belongs to that cell
                    const double x = on_plane(fma(qr + r, L.Xq, L.X0)) - cell;
                    Lc = (x >= 0.0 && x < 1.0) ? L.Lmax : 0.f;
                } else {
                    Lc = fminf(fmaxf((L.H - fabsf(dl)) * L.R, 0.f), L.Lmax);
                    dl += step;
                }
                // (a zero chord, an aligned ray on the cell's far edge, adds nothing)
                const float4 *row4 = (const float4 *)row;
#pragma unroll
                for (int k = 0; k < SEG / 4; ++k) {
                    const float4 q = row4[k];
                    part[4 * k + 0] = fmaf(Lc, q.x, part[4 * k + 0]);
                    part[4 * k + 1] = fmaf(Lc, q.y, part[4 * k + 1]);
                    part[4 * k + 2] = fmaf(Lc, q.z, part[4 * k + 2]);
                    part[4 * k + 3] = fmaf(Lc, q.w, part[4 * k + 3]);
                }
            }
        }
        buf ^= 1;
        if (++batch == 32 || last) {
            // into the brick's accumulator: each voxel belongs to one segment here
            if (live) {
                constexpr int STEP = D == 0 ? 1 : (D == 1 ? LSY : LSZ);
                const int base = D == 0 ? lb * LSZ + la * LSY : (D == 1 ? lb * LSZ + la : lb * LSY + la);
#pragma unroll
                for (int j = 0; j < SEG; ++j) {
                    acc[base + (s0 + j) * STEP] += part[j];
                    part[j] = 0.f;
                }
            }
            batch = 0;
        }
        if (last) break;
        view = nview;
        h = hn;
#pragma unroll
        for (int m = 0; m < NSLOT; ++m) ld[m] = ldn[m];
    }
    __syncthreads();   // the next family's segments own other voxels
}

template <int MODE, int SHAPE>
__global__ __launch_bounds__(512) void line_kernel(BrickArgs a, const LineView *lines) {
    constexpr LineShape SH = kLineShapes[SHAPE];
    constexpr int BX = SH.bx, BY = SH.by, BZ = SH.bz, NT = 512;
    constexpr int LSY = BX + 1, LSZ = LSY * BY + 1, LN = LSZ * BZ;
    __shared__ float acc[LN];
    __shared__ float stage[2][SH.rows * kLinePitch];
    const int tid = threadIdx.x;
    for (int i = tid; i < LN; i += NT) acc[i] = 0.f;

    const int blk = xcd_remap(blockIdx.x, a.n_blocks);
    const int bxi = blk % a.nbx;
    const int byi = (blk / a.nbx) % a.nby;
    const int bzi = blk / (a.nbx * a.nby);
    const int x0 = bxi * BX, y0 = byi * BY, z0 = bzi * BZ;   // within the volume buffer
    const int ex = min(BX, a.W - x0), ey = min(BY, a.H - y0), ez = min(BZ, a.D - z0);
    if (MODE == BM_SIRT_UPDATE && a.mask) {
        // a brick with no voxel to update does no work at all
        int any = 0;
        for (int i = tid; i < BX * BY * BZ; i += NT) {
            const int lx = i % BX, ly = (i / BX) % BY, lz = i / (BX * BY);
            if (lx < ex && ly < ey && lz < ez)
                any |= a.mask[((size_t)(z0 + lz) * a.H + (y0 + ly)) * a.W + (x0 + lx)] != 0;
        }
        if (!__syncthreads_or(any)) return;
    }
    const ConstLinePtr lv = (ConstLinePtr)lines;
    int buf = 0;
    line_family<MODE, 0, SHAPE, LSY, LSZ>(a, lv, acc, stage, buf, x0, y0, z0, ex, ey, ez);
    line_family<MODE, 1, SHAPE, LSY, LSZ>(a, lv, acc, stage, buf, x0, y0, z0, ex, ey, ez);
    if constexpr (SHAPE == 0) line_family<MODE, 2, SHAPE, LSY, LSZ>(a, lv, acc, stage, buf, x0, y0, z0, ex, ey, ez);
    __syncthreads();
    brick_writeout<BX, BY, BZ, NT, MODE>(a, x0, y0, z0, ex, ey, ez, [&](int lx, int ly, int lz) {
        return acc[lz * LSZ + ly * LSY + lx];
    });
}

// The record table of a whole-volume brick launch: for every (brick, view) pair,
// one lane computes the footprint (lane form) and the anchor exactly as the brick
// kernel would, so launches that read the table give the same bits as launches
// that compute them.  Pairs are brick-major (all views of brick 0 first).
template <int BX, int BY, int BZ>
__global__ __launch_bounds__(256) void brick_rec_kernel(const double *views, int n_views, int W, int H, int D,
                                                        int U, int V, const float *env, int nbx, int nby,
                                                        size_t n_pairs, BrickRec *out) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n_pairs) return;
    const int b = (int)(i / (size_t)n_views), view = (int)(i - (size_t)b * n_views);
    const int bxi = b % nbx, byi = (b / nbx) % nby, bzi = b / (nbx * nby);
    const int x0 = bxi * BX, y0 = byi * BY, z0 = bzi * BZ;
    const int ex = min(BX, W - x0), ey = min(BY, H - y0), ez = min(BZ, D - z0);
    const double cbx = x0 + 0.5 * ex, cby = y0 + 0.5 * ey, cbz = z0 + 0.5 * ez;
    const double *vw = views + (size_t)view * CT_VIEW_TABLE_STRIDE;
    constexpr bool TWO_D = BZ == 1;
    Footprint f;
    BrickRec r{};
    if (brick_footprint_lane(vw, x0, y0, z0, ex, ey, ez, U, V, TWO_D,
                             env ? env + (size_t)view * env_size(U, V) : nullptr, f)) {
        r.fu = (uint32_t)f.u0 | (uint32_t)f.u1 << 16;
        r.fv = (uint32_t)f.v0 | (uint32_t)f.v1 << 16;
        r.an = make_anchor(vw, f, cbx, cby, cbz, !TWO_D && vt(vw, VT_PATCH) == 0.0);
    } else {
        r.fu = 1u;   // u0 = 1 > u1 = 0: unseen
        r.fv = 0u;
    }
    out[i] = r;
}

// out[a + b*tb + o*to] = in[a*sa + b + o*so]: one 32 x 32 tile of a 2D transpose
// per block (reads contiguous along b, writes contiguous along a) for each outer
// index o.  Builds the y- and z-fastest volume copies.
__global__ __launch_bounds__(256) void transpose_kernel(const float *__restrict__ in,
                                                        float *__restrict__ out, int A, int B,
                                                        size_t sa, size_t so, size_t tb, size_t to) {
    __shared__ float tile[32][33];
    const int b0 = blockIdx.x * 32, a0 = blockIdx.y * 32;
    const size_t o = blockIdx.z;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int k = ty; k < 32; k += 8) {
        const int aa = a0 + k, bb = b0 + tx;
        if (aa < A && bb < B) tile[k][tx] = in[(size_t)aa * sa + bb + o * so];
    }
    __syncthreads();
    for (int k = ty; k < 32; k += 8) {
        const int bb = b0 + k, aa = a0 + tx;
        if (aa < A && bb < B) out[aa + (size_t)bb * tb + o * to] = tile[tx][k];
    }
}

__global__ void fill_kernel(float *p, size_t n, float v) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

__global__ void zero_u64_kernel(unsigned long long *p) { *p = 0ull; }

// ---------------------------------------------------------------------------
// CGLS vector steps (diffct docs, "Large Volumes and Chunked Execution" >
// "Runnable iterative reconstruction": state x, s, p and r, q, float64 norms).
// Scalars live in device memory, so an iteration needs no host round trip.
// ---------------------------------------------------------------------------

// Sum the per-block partials (fixed order) and derive the scalars of one step:
//   CO_RR    rr = ||r||^2
//   CO_INIT  gamma = ||s||^2
//   CO_ALPHA qq = ||q||^2, alpha = gamma / qq (0 if qq = 0)
//   CO_BETA  beta = ||s||^2 / gamma (0 if gamma = 0), then gamma = ||s||^2
__global__ __launch_bounds__(1024) void cgls_finalize_kernel(const double *__restrict__ partial, int n,
                                                             double *state, int op) {
    __shared__ double wsum[16];
    double v = 0.0;
    for (int i = threadIdx.x; i < n; i += 1024) v += partial[i];
    const double t = block_sum<1024>(v, wsum);
    if (threadIdx.x == 0) {
        if (op == CO_RR) {
            state[CS_RR] = t;
        } else if (op == CO_INIT) {
            state[CS_GAMMA] = t;
            state[CS_ALPHA] = 0.0;
            state[CS_BETA] = 0.0;
        } else if (op == CO_ALPHA) {
            state[CS_QQ] = t;
            state[CS_ALPHA] = t > 0.0 ? state[CS_GAMMA] / t : 0.0;
        } else {
            const double g = state[CS_GAMMA];
            state[CS_BETA] = g > 0.0 ? t / g : 0.0;
            state[CS_GAMMA] = t;
        }
    }
}

// r -= alpha q, with per-block sums of the new r^2.
__global__ __launch_bounds__(256) void cgls_update_r_kernel(float *__restrict__ r,
                                                            const float *__restrict__ q, size_t n,
                                                            bool vec, const double *state,
                                                            double *partial) {
    __shared__ double wsum[4];
    const float alpha = (float)state[CS_ALPHA];
    const size_t n4 = vec ? n / 4 : 0;   // vec: both buffers 16-byte aligned
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    double sq = 0.0;
    float4 *r4 = reinterpret_cast<float4 *>(r);
    const float4 *q4 = reinterpret_cast<const float4 *>(q);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 a = r4[i];
        const float4 b = q4[i];
        a.x = fmaf(-alpha, b.x, a.x);
        a.y = fmaf(-alpha, b.y, a.y);
        a.z = fmaf(-alpha, b.z, a.z);
        a.w = fmaf(-alpha, b.w, a.w);
        r4[i] = a;
        sq += ((double)a.x * a.x + (double)a.y * a.y) + ((double)a.z * a.z + (double)a.w * a.w);
    }
    for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float v = fmaf(-alpha, q[i], r[i]);
        r[i] = v;
        sq += (double)v * v;
    }
    const double t = block_sum<256>(sq, wsum);
    if (threadIdx.x == 0) partial[blockIdx.x] = t;
}

// p = s + beta p.
__global__ __launch_bounds__(256) void cgls_update_p_kernel(float *__restrict__ p,
                                                            const float *__restrict__ s, size_t n,
                                                            bool vec, const double *state) {
    const float beta = (float)state[CS_BETA];
    const size_t n4 = vec ? n / 4 : 0;   // vec: both buffers 16-byte aligned
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    float4 *p4 = reinterpret_cast<float4 *>(p);
    const float4 *s4 = reinterpret_cast<const float4 *>(s);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 a = p4[i];
        const float4 b = s4[i];
        a.x = fmaf(beta, a.x, b.x);
        a.y = fmaf(beta, a.y, b.y);
        a.z = fmaf(beta, a.z, b.z);
        a.w = fmaf(beta, a.w, b.w);
        p4[i] = a;
    }
    for (size_t i = n4 * 4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = fmaf(beta, p[i], s[i]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static RayArgs ray_args(const LaunchGeom &g) {
    RayArgs a{};
    a.offx = g.offx; a.offy = g.offy; a.offz = g.offz;
    a.accumulate = g.accumulate;
    a.surf = Surface{g.surf_off, g.surf_per_view};
    a.views = g.views;
    a.W = g.W; a.H = g.H; a.D = g.D; a.U = g.U; a.V = g.V; a.n_views = g.n_views;
    a.spx = g.spx; a.spy = g.spy; a.spz = g.spz;
    if (g.two_d) {
        a.n_utiles = (g.U + 63) / 64;
        a.n_vtiles = 1;
    } else {
        a.n_utiles = (g.U + 15) / 16;
        a.n_vtiles = (g.V + 15) / 16;
    }
    a.n_blocks = a.n_utiles * a.n_vtiles * g.n_views;
    a.vol_bytes = (uint32_t)((size_t)g.W * g.H * g.D * 4);
    return a;
}

// The forward kinds the packet kernel serves, and the geometries it serves them on.
constexpr bool packet_mode(int mode) {
    return mode == RM_PROJECT || mode == RM_RESIDUAL || mode == RM_PROJECT_SQ || mode == RM_CGLS_R0;
}
static bool packet_geom(const LaunchGeom &g) { return g.packet && !g.two_d && !g.surf_off; }
// Blocks of a packet launch: tiles of kPacketTP x kPacketTQ pixels, the first
// along each view's packet axis, for every view.
static int packet_blocks(const LaunchGeom &g) {
    constexpr int TP = kPacketTP, TQ = kPacketTQ;
    const int tu = ((g.U + TP - 1) / TP) * ((g.V + TQ - 1) / TQ), tv = ((g.V + TP - 1) / TP) * ((g.U + TQ - 1) / TQ);
    const int G = kPacketTileGroup;
    return g.n_views * ((std::max(tu, tv) + G - 1) / G) * G;
}

template <int MODE>
static hipError_t launch_ray(const LaunchGeom &g, RayArgs a, hipStream_t s) {
    if (packet_mode(MODE) && packet_geom(g)) {
        a.n_blocks = packet_blocks(g);
        hipLaunchKernelGGL((ray_packet_kernel<packet_mode(MODE) ? MODE : RM_PROJECT>), dim3(a.n_blocks),
                           dim3(64 * kPacketWaves), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid(a.n_blocks), block(256);
    if (g.two_d) {
        if (a.surf.off) hipLaunchKernelGGL((ray_kernel<MODE, true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((ray_kernel<MODE, true, false>), grid, block, 0, s, a);
    } else {
        if (a.surf.off) hipLaunchKernelGGL((ray_kernel<MODE, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((ray_kernel<MODE, false, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_fill(float *p, size_t n, float v, hipStream_t s) {
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

// Build the y- and z-fastest copies of the volume that the views' gathers use.
static hipError_t stage_layouts(const LaunchGeom &g, const float *vol, RayArgs &a, hipStream_t s) {
    a.vol_yf = g.vol_yf;
    a.vol_zf = g.vol_zf;
    if ((g.need_yf && !g.vol_yf) || (g.need_zf && !g.vol_zf)) return hipErrorInvalidValue;
    const size_t W = g.W, H = g.H, D = g.D;
    if (g.vol_yf) {   // (z, x, y): per z slice, transpose (y, x) -> (x, y)
        dim3 grid((unsigned)((W + 31) / 32), (unsigned)((H + 31) / 32), (unsigned)D);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, vol, g.vol_yf, (int)H, (int)W,
                           W, W * H, H, W * H);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (g.vol_zf) {   // (x, y, z): per y row, transpose (z, x) -> (x, z)
        dim3 grid((unsigned)((W + 31) / 32), (unsigned)((D + 31) / 32), (unsigned)H);
        hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, vol, g.vol_zf, (int)D, (int)W,
                           W * H, W, H * D, D);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_project(const LaunchGeom &g, const float *vol, float *sino, hipStream_t s) {
    RayArgs a = ray_args(g);
    a.vol = vol;
    a.out = sino;
    const hipError_t e = stage_layouts(g, vol, a, s);
    if (e != hipSuccess) return e;
    return launch_ray<RM_PROJECT>(g, a, s);
}

hipError_t launch_residual(const LaunchGeom &g, const float *x, const float *y, const float *rinv,
                           float *e, hipStream_t s) {
    RayArgs a = ray_args(g);
    const hipError_t er = stage_layouts(g, x, a, s);
    if (er != hipSuccess) return er;
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

template <int BX, int BY, int BZ, int NT, int MODE>
static void launch_brick_shape(BrickArgs &a, const LaunchGeom &g, hipStream_t s) {
    a.nbx = (g.W + BX - 1) / BX;
    a.nby = (g.H + BY - 1) / BY;
    a.nbz = (g.D + BZ - 1) / BZ;
    a.n_blocks = a.nbx * a.nby * a.nbz;
    const dim3 grid(a.n_blocks), block(NT);
    const auto go = [&](auto surf, auto persp) {
        constexpr bool SF = decltype(surf)::value, PS = decltype(persp)::value;
        if (a.rec) hipLaunchKernelGGL((brick_kernel<BX, BY, BZ, NT, MODE, SF, PS, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((brick_kernel<BX, BY, BZ, NT, MODE, SF, PS, false>), grid, block, 0, s, a);
    };
    if (a.surf.off) {
        if (g.persp) go(std::true_type{}, std::true_type{});
        else go(std::true_type{}, std::false_type{});
    } else {
        if (g.persp) go(std::false_type{}, std::true_type{});
        else go(std::false_type{}, std::false_type{});
    }
}

static void brick_shape(const LaunchGeom &g, int &bx, int &by, int &bz) {
    bx = 16;
    by = 16;
    bz = g.two_d ? 1 : 32;
}

size_t brick_record_count(const LaunchGeom &g) {
    int bx, by, bz;
    brick_shape(g, bx, by, bz);
    return (size_t)((g.W + bx - 1) / bx) * ((g.H + by - 1) / by) * ((g.D + bz - 1) / bz) * (size_t)g.n_views;
}
size_t brick_record_bytes() { return sizeof(BrickRec); }

hipError_t launch_brick_records(const LaunchGeom &g, void *out, hipStream_t s) {
    int bx, by, bz;
    brick_shape(g, bx, by, bz);
    const size_t n = brick_record_count(g);
    const int nbx = (g.W + bx - 1) / bx, nby = (g.H + by - 1) / by;
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (g.two_d)
        hipLaunchKernelGGL((brick_rec_kernel<16, 16, 1>), grid, block, 0, s, g.views, g.n_views, g.W, g.H, g.D,
                           g.U, g.V, g.surf_env, nbx, nby, n, (BrickRec *)out);
    else
        hipLaunchKernelGGL((brick_rec_kernel<16, 16, 32>), grid, block, 0, s, g.views, g.n_views, g.W, g.H,
                           g.D, g.U, g.V, g.surf_env, nbx, nby, n, (BrickRec *)out);
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_brick_args(const LaunchGeom &g, BrickArgs a, hipStream_t s) {
    a.views = g.views;
    a.rec = g.brick_rec ? (const BrickRec *)g.brick_rec + g.rec_view0 : nullptr;
    a.rec_stride = g.rec_stride;
    a.y_vec4 = (g.V % 4 == 0 && ((uintptr_t)a.sino & 15u) == 0) ? 1 : 0;
    a.offx = g.offx; a.offy = g.offy; a.offz = g.offz;
    a.accumulate = g.accumulate;
    a.surf = Surface{g.surf_off, g.surf_per_view};
    a.env = g.surf_env;
    a.W = g.W; a.H = g.H; a.D = g.D; a.U = g.U; a.V = g.V; a.n_views = g.n_views;
    a.spx = g.spx; a.spy = g.spy; a.spz = g.spz;
    a.yshift = g.yshift;
    // 3D: bricks of 16 x 16 x 32 voxels, 512 threads; 2D: 16 x 16, 256 threads;
    // separable tilt series: the line adjoint on the same bricks
    if (g.line_tab && !g.two_d) {
        const LineShape &sh = kLineShapes[g.line_shape];
        a.nbx = (g.W + sh.bx - 1) / sh.bx;
        a.nby = (g.H + sh.by - 1) / sh.by;
        a.nbz = (g.D + sh.bz - 1) / sh.bz;
        a.n_blocks = a.nbx * a.nby * a.nbz;
        if (g.line_shape == 1)
            hipLaunchKernelGGL((line_kernel<MODE, 1>), dim3(a.n_blocks), dim3(512), 0, s, a,
                               (const LineView *)g.line_tab);
        else
            hipLaunchKernelGGL((line_kernel<MODE, 0>), dim3(a.n_blocks), dim3(512), 0, s, a,
                               (const LineView *)g.line_tab);
    } else if (g.two_d) {
        launch_brick_shape<16, 16, 1, 256, MODE>(a, g, s);
    } else {
        launch_brick_shape<16, 16, 32, 512, MODE>(a, g, s);
    }
    return hipGetLastError();
}

template <int MODE>
static hipError_t launch_brick(const LaunchGeom &g, const float *sino, float *vol,
                               const float *cinv, float relax, hipStream_t s) {
    BrickArgs a{};
    a.sino = sino;
    a.vol = vol;
    a.cinv = cinv;
    a.relax = relax;
    return launch_brick_args<MODE>(g, a, s);
}

hipError_t launch_backproject(const LaunchGeom &g, const float *sino, float *vol, hipStream_t s) {
    return launch_brick<BM_BACKPROJECT>(g, sino, vol, nullptr, 0.f, s);
}

hipError_t launch_sirt_update(const LaunchGeom &g, const float *e, const float *cinv, float relax,
                              float *x, hipStream_t s) {
    return launch_brick<BM_SIRT_UPDATE>(g, e, x, cinv, relax, s);
}

hipError_t launch_sirt_update_bounded(const LaunchGeom &g, const float *e, const float *cinv,
                                      float relax, float lo, float hi, const uint8_t *mask, float *x,
                                      hipStream_t s) {
    BrickArgs a{};
    a.sino = e;
    a.vol = x;
    a.cinv = cinv;
    a.relax = relax;
    a.bounded = true;
    a.lo = lo;
    a.hi = hi;
    a.mask = mask;
    return launch_brick_args<BM_SIRT_UPDATE>(g, a, s);
}

hipError_t launch_colinv(const LaunchGeom &g, float *cinv, hipStream_t s) {
    return launch_brick<BM_COLINV>(g, nullptr, cinv, nullptr, 0.f, s);
}

size_t surface_env_floats(int U, int V) { return env_size(U, V); }

hipError_t launch_surface_env(const LaunchGeom &g, unsigned long long *bad, hipStream_t s) {
    hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, bad);
    hipLaunchKernelGGL(surface_env_kernel, dim3(g.n_views), dim3(256), 0, s, g.views,
                       Surface{g.surf_off, g.surf_per_view}, g.U, g.V, g.surf_env, bad);
    return hipGetLastError();
}

// ---- CGLS ----

// partials of the CGLS forward (RM_PROJECT_SQ, RM_CGLS_R0): one per block of the launch
size_t cgls_ray_blocks(const LaunchGeom &g) {
    return packet_geom(g) ? (size_t)packet_blocks(g) : (size_t)ray_args(g).n_blocks;
}

size_t cgls_brick_blocks(const LaunchGeom &g) {
    int bx, by, bz;
    brick_shape(g, bx, by, bz);
    if (g.line_tab && !g.two_d) {   // the line adjoint's bricks
        bx = kLineShapes[g.line_shape].bx;
        by = kLineShapes[g.line_shape].by;
        bz = kLineShapes[g.line_shape].bz;
    }
    return (size_t)((g.W + bx - 1) / bx) * ((g.H + by - 1) / by) * ((g.D + bz - 1) / bz);
}

static hipError_t cgls_finalize(const double *partial, size_t n, double *state, int op, hipStream_t s) {
    hipLaunchKernelGGL(cgls_finalize_kernel, dim3(1), dim3(1024), 0, s, partial, (int)n, state, op);
    return hipGetLastError();
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

hipError_t launch_cgls_init(const LaunchGeom &g, const float *y, const float *x, float *r, float *sv,
                            float *p, double *state, double *partial, hipStream_t s) {
    // r = y - A x, rr = ||r||^2
    RayArgs ra = ray_args(g);
    hipError_t e = stage_layouts(g, x, ra, s);
    if (e != hipSuccess) return e;
    ra.vol = x;
    ra.sino = y;
    ra.out = r;
    ra.partial = partial;
    if ((e = launch_ray<RM_CGLS_R0>(g, ra, s)) != hipSuccess) return e;
    if ((e = cgls_finalize(partial, cgls_ray_blocks(g), state, CO_RR, s)) != hipSuccess) return e;
    // s = A^T r, p = s, gamma = ||s||^2
    BrickArgs b{};
    b.sino = r;
    b.vol = sv;
    b.p_copy = p;
    b.state = state;
    b.partial = partial;
    if ((e = launch_brick_args<BM_CGLS>(g, b, s)) != hipSuccess) return e;
    return cgls_finalize(partial, cgls_brick_blocks(g), state, CO_INIT, s);
}

hipError_t launch_cgls_step(const LaunchGeom &g, float *x, float *r, float *sv, float *p, float *q,
                            double *state, double *partial, hipStream_t s) {
    // q = A p, alpha = gamma / ||q||^2
    RayArgs ra = ray_args(g);
    hipError_t e = stage_layouts(g, p, ra, s);
    if (e != hipSuccess) return e;
    ra.vol = p;
    ra.out = q;
    ra.partial = partial;
    if ((e = launch_ray<RM_PROJECT_SQ>(g, ra, s)) != hipSuccess) return e;
    if ((e = cgls_finalize(partial, cgls_ray_blocks(g), state, CO_ALPHA, s)) != hipSuccess) return e;
    // r -= alpha q, rr = ||r||^2
    const size_t m = (size_t)g.n_views * g.U * g.V;
    const bool vr = aligned16(r) && aligned16(q);
    hipLaunchKernelGGL(cgls_update_r_kernel, dim3(kCglsVecBlocks), dim3(256), 0, s, r, q, m, vr,
                       (const double *)state, partial);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = cgls_finalize(partial, kCglsVecBlocks, state, CO_RR, s)) != hipSuccess) return e;
    // s = A^T r and x += alpha p (old p) in the brick write-out; beta, gamma
    BrickArgs b{};
    b.sino = r;
    b.vol = sv;
    b.x_upd = x;
    b.p_old = p;
    b.state = state;
    b.partial = partial;
    if ((e = launch_brick_args<BM_CGLS>(g, b, s)) != hipSuccess) return e;
    if ((e = cgls_finalize(partial, cgls_brick_blocks(g), state, CO_BETA, s)) != hipSuccess) return e;
    // p = s + beta p
    const size_t n = (size_t)g.W * g.H * g.D;
    const bool vp = aligned16(p) && aligned16(sv);
    hipLaunchKernelGGL(cgls_update_p_kernel, dim3(kCglsVecBlocks), dim3(256), 0, s, p,
                       (const float *)sv, n, vp, (const double *)state);
    return hipGetLastError();
}

}  // namespace ctp
