// ct_fbp.hip -- analytical FBP (parallel2d, fan2d) and FDK (cone) on a flat
// detector: pre-weights and ramp filter, then the voxel-driven interpolating
// weighted backprojection, and that backprojection's transpose.
//
// diffct documentation, "Differentiable analytical reconstruction" and the
// "Analytical Reconstruction Helpers" / "Ramp Filter Options" sections of its
// API reference: cosine (and, for short scans, Parker) pre-weights, a ramp
// filter along u zero-padded to pad_factor * U samples and applied as a real
// multiplier, angular quadrature weights (a full fan/cone turn carries the 1/2
// redundancy factor), and a voxel-driven interpolating backprojection that is
// not the Siddon adjoint; its transpose scatters the same coefficients.
//
// Readings where the pages give no formula: the Ram-Lak filter is the
// band-limited ramp of Ramachandran and Lakshminarayanan sampled in space
// (Kak and Slaney, "Principles of Computerized Tomographic Imaging", ch. 3),
// taken P-periodic; windows of f = k / P: Shepp-Logan sin(pi f)/(pi f), cosine
// cos(pi f), Hamming 0.54 + 0.46 cos(2 pi f), Hann 0.5 + 0.5 cos(2 pi f).  The
// FDK distance weight is R D / U(x)^2 (U(x) = (x - a).n, D = (c - a).n,
// R = (iso - a).n).  Parker weights follow Parker (1982).  Detector samples
// outside the detector read as 0.
//
// Overrides and the helical approximation (same page, the paragraph on the
// complete APIs and "Helical approximation"): a caller's filter response and
// pre-weights stand in for the windowed ramp and the cosine weight, and
// per-slice view weights (the helical full-turn windows, or the caller's) take
// the place of the angular weights inside the gather.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <type_traits>
#include <vector>

#include "ct_internal.h"

using namespace ctp;

namespace {

constexpr uint64_t kFbpMagic = 0x43544642'50303031ull;   // "CTFBP001"
constexpr int kBpViews = 128;      // views whose constants one LDS batch holds
constexpr int kBpConst = 40;       // floats per view in that batch
constexpr int kZRun = 4;           // 3D backprojection: voxels per thread along z
constexpr int64_t kStagingBytes = int64_t(4) << 30;   // cone backprojection staging cap

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const float *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0, (int)bytes, 0x00020000);
}

// Workgroups are dispatched to the 8 XCDs in turn (block i to XCD i mod 8),
// and each XCD has its own L2.  Logical block ids remapped so that XCD x runs
// one contiguous range: neighbouring blocks, which share cache lines of the
// sinogram rows, then share an L2.
__device__ __forceinline__ int xcd_block(int hw, int nblocks) {
    constexpr int kXcd = 8;
    const int q = nblocks / kXcd, r = nblocks % kXcd;
    const int x = hw % kXcd, k = hw / kXcd;
    return x * q + min(x, r) + k;
}

__device__ __forceinline__ float buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}

// Four consecutive floats at byte offset off (one 16-byte load).
__device__ __forceinline__ float4 buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return make_float4(buffer_load(r, off), buffer_load(r, off + 4u), buffer_load(r, off + 8u),
                       buffer_load(r, off + 12u));
}

// floor(x) as an integer in one instruction (|x| < 2^31).
__device__ __forceinline__ int floor_i32(float x) {
    int r;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// a * b + c with a and b signed 24-bit, in one instruction (the compiler
// otherwise splits it around a three-operand add).
__device__ __forceinline__ int mad_i24(int a, int b, int c) {
    int r;
    asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

ct_status_t ffail(ct_status_t st, const char *msg) {
    set_error(msg);
    return st;
}

ct_status_t fhip(hipError_t e, const char *where) {
    char buf[400];
    std::snprintf(buf, sizeof buf, "%s: %s", where, hipGetErrorString(e));
    set_error(buf);
    return CT_E_HIP;
}

// ---------------------------------------------------------------------------
// filter: pre-weights, circular convolution with the P-periodic filter kernel
// (equal to the zero-padded real-FFT multiplier), angular weight
// ---------------------------------------------------------------------------

// Per view, float: D, (c - a) (3), e_u du (3), e_v dv (3), angular weight, perspective.
constexpr int kFv = 12;

struct FilterArgs {
    const float *sino;
    float *out;
    const float *taps;     // 2 * U8 taps, tap j (|j| <= U8) at j + U8
    const float *fview;    // kFv floats per view
    const float *parker;   // n_views x U, or null
    const float *pw;       // pre-weights replacing the cosine weight (index view * pw_stride + u V + v), or null
    size_t pw_stride;      // 0 (one U x V array for every view) or U V
    int U, V, n_views, U8, VT, S;   // S: LDS row stride of the tile (floats)
    int two_d;
};

// One block filters VT rows: VT consecutive v of one view (3D), or VT
// consecutive views (2D).  Each thread owns 8 consecutive outputs of one row
// and keeps them in registers while it sweeps the row's samples eight at a
// time (16 taps per sweep step cover the 8 x 8 products).
__global__ __launch_bounds__(256) void fbp_filter_kernel(FilterArgs a) {
    extern __shared__ float lds[];
    float *taps = lds;                    // 2 * U8
    float *tile = lds + 2 * a.U8;         // VT rows of S floats
    const int U = a.U, V = a.V, U8 = a.U8, VT = a.VT, S = a.S;
    int view0, v0;
    if (a.two_d) {
        view0 = xcd_block(blockIdx.x, gridDim.x) * VT;
        v0 = 0;
    } else {
        const int nvt = (V + VT - 1) / VT;
        const int b = xcd_block(blockIdx.x, gridDim.x);
        view0 = b / nvt;
        v0 = (b % nvt) * VT;
    }
    for (int i = threadIdx.x; i < 2 * U8; i += 256) taps[i] = a.taps[i];
    // load the rows with their pre-weights; samples past U (or past the last
    // row) are zero
    for (int i = threadIdx.x; i < VT * U8; i += 256) {
        int r, u;
        if (a.two_d) {
            r = i / U8;
            u = i - r * U8;
        } else {
            u = i / VT;
            r = i - u * VT;
        }
        const int view = a.two_d ? view0 + r : view0;
        const int v = a.two_d ? 0 : v0 + r;
        float val = 0.f;
        if (u < U && view < a.n_views && v < V) {
            const float *fv = a.fview + (size_t)view * kFv;
            val = a.sino[((size_t)view * U + u) * V + v];
            if (a.pw) {   // the caller's pre-weights
                val *= a.pw[(size_t)view * a.pw_stride + (size_t)u * V + v];
            } else if (fv[11] != 0.f) {   // fan/cone: cosine weight
                const float ou = (float)u - 0.5f * (float)(U - 1);
                const float ov = a.two_d ? 0.f : (float)v - 0.5f * (float)(V - 1);
                const float px = fv[1] + ou * fv[4] + ov * fv[7];
                const float py = fv[2] + ou * fv[5] + ov * fv[8];
                const float pz = fv[3] + ou * fv[6] + ov * fv[9];
                val *= fabsf(fv[0]) / sqrtf(px * px + py * py + pz * pz);
            }
            if (a.parker) val *= a.parker[(size_t)view * U + u];
        }
        tile[r * S + u] = val;
    }
    __syncthreads();
    const int nb = U8 / 8;   // VT * nb <= 1024: at most four tasks per thread
    float res[4][8];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int task = threadIdx.x + 256 * it;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const int r = task / nb, n0 = (task - r * nb) * 8;
        const float *prow = tile + r * S;
        for (int m0 = 0; task < VT * nb && m0 < U8; m0 += 8) {
            const float4 p0 = *(const float4 *)(prow + m0);
            const float4 p1 = *(const float4 *)(prow + m0 + 4);
            const float *tb = taps + (n0 - m0 - 8 + U8);   // taps n0 - m0 - 8 .. + 15
            const float4 t0 = *(const float4 *)(tb);
            const float4 t1 = *(const float4 *)(tb + 4);
            const float4 t2 = *(const float4 *)(tb + 8);
            const float4 t3 = *(const float4 *)(tb + 12);
            const float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            const float t[16] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w,
                                 t2.x, t2.y, t2.z, t2.w, t3.x, t3.y, t3.z, t3.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[j] = fmaf(p[i], t[j - i + 8], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) res[it][j] = acc[j];
    }
    __syncthreads();   // every read of the tile is done: reuse it for the outputs
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int task = threadIdx.x + 256 * it;
        const int r = task / nb, n0 = (task - r * nb) * 8;
        if (task < VT * nb) {
            *(float4 *)(tile + r * S + n0) = make_float4(res[it][0], res[it][1], res[it][2], res[it][3]);
            *(float4 *)(tile + r * S + n0 + 4) = make_float4(res[it][4], res[it][5], res[it][6], res[it][7]);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < VT * U8; i += 256) {
        int r, u;
        if (a.two_d) {
            r = i / U8;
            u = i - r * U8;
        } else {
            u = i / VT;
            r = i - u * VT;
        }
        const int view = a.two_d ? view0 + r : view0;
        const int v = a.two_d ? 0 : v0 + r;
        if (u < U && view < a.n_views && v < V)
            a.out[((size_t)view * U + u) * V + v] = a.fview[(size_t)view * kFv + 10] * tile[r * S + u];
    }
}

// The same filter through FFTs, for power-of-two P <= 4096: the circular
// convolution with the P-periodic kernel is the inverse DFT of the product of
// the DFT and the multiplier.  Two real rows travel as the real and imaginary
// parts of one complex row (the multiplier is real and even, so each part is
// filtered on its own).  A block holds NPAIR complex rows in LDS: a radix-2
// decimation-in-time transform in place (bit-reversed input, written so by the
// load), the multiplier, then a radix-2 decimation-in-frequency inverse in
// place (natural input, bit-reversed output, read so by the store).
struct FftArgs {
    const float *sino;
    float *out;
    const float2 *tw;      // exp(-2 pi i t / P), t < P / 2
    const float *mul;      // multiplier M_k, k = 0..P/2
    const float *fview;
    const float *parker;
    const float *pw;
    size_t pw_stride;
    int U, V, n_views, P, L, npair;
    int two_d;
};

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}

__global__ __launch_bounds__(256) void fbp_fft_filter_kernel(FftArgs a) {
    extern __shared__ float2 sh[];
    const int P = a.P, L = a.L, NP = a.npair, C = 2 * NP, U = a.U, V = a.V;
    float2 *x = sh;                   // NP rows of P complex
    float2 *tw = sh + NP * P;         // P / 2
    float *mul = (float *)(tw + P / 2);   // P / 2 + 1
    int view0, v0;
    if (a.two_d) {
        view0 = xcd_block(blockIdx.x, gridDim.x) * C;
        v0 = 0;
    } else {
        const int nvt = (V + C - 1) / C;
        const int b = xcd_block(blockIdx.x, gridDim.x);
        view0 = b / nvt;
        v0 = (b % nvt) * C;
    }
    for (int i = threadIdx.x; i < P / 2; i += 256) tw[i] = a.tw[i];
    for (int i = threadIdx.x; i <= P / 2; i += 256) mul[i] = a.mul[i];
    float *xf = (float *)x;
    for (int i = threadIdx.x; i < C * P; i += 256) {
        int c, u;
        if (a.two_d) {
            c = i / P;
            u = i - c * P;
        } else {
            u = i / C;
            c = i - u * C;
        }
        const int view = a.two_d ? view0 + c : view0;
        const int v = a.two_d ? 0 : v0 + c;
        float val = 0.f;
        if (u < U && view < a.n_views && v < V) {
            const float *fv = a.fview + (size_t)view * kFv;
            val = a.sino[((size_t)view * U + u) * V + v];
            if (a.pw) {   // the caller's pre-weights
                val *= a.pw[(size_t)view * a.pw_stride + (size_t)u * V + v];
            } else if (fv[11] != 0.f) {
                const float ou = (float)u - 0.5f * (float)(U - 1);
                const float ov = a.two_d ? 0.f : (float)v - 0.5f * (float)(V - 1);
                const float px = fv[1] + ou * fv[4] + ov * fv[7];
                const float py = fv[2] + ou * fv[5] + ov * fv[8];
                const float pz = fv[3] + ou * fv[6] + ov * fv[9];
                val *= fabsf(fv[0]) / sqrtf(px * px + py * py + pz * pz);
            }
            if (a.parker) val *= a.parker[(size_t)view * U + u];
        }
        const int br = (int)(__builtin_bitreverse32((uint32_t)u) >> (32 - L));
        xf[2 * ((c >> 1) * P + br) + (c & 1)] = val;
    }
    __syncthreads();
    // Forward, decimation in time, two stages per pass: stages s and s + 1
    // touch the four elements i, i + h, i + 2h, i + 3h (h = 2^(s-1)) of a group
    // of 4h and no others, so a thread takes them through both stages in
    // registers (half the LDS traffic and barriers of one stage per pass).
    // An odd count of stages starts with one single stage.
    const int nbf = NP * (P / 2), nq = NP * (P / 4);
    int st = 1;
    if (L & 1) {
        for (int b = threadIdx.x; b < nbf; b += 256) {   // stage 1: h = 1, twiddle 1
            const float2 u0 = x[2 * b], u1 = x[2 * b + 1];
            x[2 * b] = make_float2(u0.x + u1.x, u0.y + u1.y);
            x[2 * b + 1] = make_float2(u0.x - u1.x, u0.y - u1.y);
        }
        __syncthreads();
        st = 2;
    }
    for (; st < L; st += 2) {
        const int h = 1 << (st - 1);
        for (int b = threadIdx.x; b < nq; b += 256) {
            const int pr = b >> (L - 2), bb = b & (P / 4 - 1);
            const int j = bb & (h - 1);
            const int i0 = pr * P + ((bb >> (st - 1)) << (st + 1)) + j;
            const float2 w1 = tw[j << (L - st)];
            const float2 w2a = tw[j << (L - st - 1)], w2b = tw[(j + h) << (L - st - 1)];
            const float2 x0 = x[i0], x1 = x[i0 + h], x2 = x[i0 + 2 * h], x3 = x[i0 + 3 * h];
            float2 t = cmul(w1, x1);
            const float2 y0 = make_float2(x0.x + t.x, x0.y + t.y), y1 = make_float2(x0.x - t.x, x0.y - t.y);
            t = cmul(w1, x3);
            const float2 y2 = make_float2(x2.x + t.x, x2.y + t.y), y3 = make_float2(x2.x - t.x, x2.y - t.y);
            t = cmul(w2a, y2);
            x[i0] = make_float2(y0.x + t.x, y0.y + t.y);
            x[i0 + 2 * h] = make_float2(y0.x - t.x, y0.y - t.y);
            t = cmul(w2b, y3);
            x[i0 + h] = make_float2(y1.x + t.x, y1.y + t.y);
            x[i0 + 3 * h] = make_float2(y1.x - t.x, y1.y - t.y);
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < NP * P; i += 256) {
        const int k = i & (P - 1);
        const float m = mul[k <= P / 2 ? k : P - k];
        x[i] = make_float2(x[i].x * m, x[i].y * m);
    }
    __syncthreads();
    // Inverse, decimation in frequency, stages L down to 1, two per pass:
    // stages s and s - 1 touch i, i + h, i + 2h, i + 3h (h = 2^(s-2)); an odd
    // count ends with the single stage 1.
    for (st = L; st >= 2; st -= 2) {
        const int h = 1 << (st - 2);
        for (int b = threadIdx.x; b < nq; b += 256) {
            const int pr = b >> (L - 2), bb = b & (P / 4 - 1);
            const int j = bb & (h - 1);
            const int i0 = pr * P + ((bb >> (st - 2)) << st) + j;
            const float2 wa = tw[j << (L - st)], wb = tw[(j + h) << (L - st)], wc = tw[j << (L - st + 1)];
            const float2 x0 = x[i0], x1 = x[i0 + h], x2 = x[i0 + 2 * h], x3 = x[i0 + 3 * h];
            const float2 y0 = make_float2(x0.x + x2.x, x0.y + x2.y);
            const float2 y2 = cmul(make_float2(x0.x - x2.x, x0.y - x2.y), make_float2(wa.x, -wa.y));
            const float2 y1 = make_float2(x1.x + x3.x, x1.y + x3.y);
            const float2 y3 = cmul(make_float2(x1.x - x3.x, x1.y - x3.y), make_float2(wb.x, -wb.y));
            x[i0] = make_float2(y0.x + y1.x, y0.y + y1.y);
            x[i0 + h] = cmul(make_float2(y0.x - y1.x, y0.y - y1.y), make_float2(wc.x, -wc.y));
            x[i0 + 2 * h] = make_float2(y2.x + y3.x, y2.y + y3.y);
            x[i0 + 3 * h] = cmul(make_float2(y2.x - y3.x, y2.y - y3.y), make_float2(wc.x, -wc.y));
        }
        __syncthreads();
    }
    if (st == 1) {
        for (int b = threadIdx.x; b < nbf; b += 256) {   // stage 1: h = 1, twiddle 1
            const float2 p0 = x[2 * b], p1 = x[2 * b + 1];
            x[2 * b] = make_float2(p0.x + p1.x, p0.y + p1.y);
            x[2 * b + 1] = make_float2(p0.x - p1.x, p0.y - p1.y);
        }
        __syncthreads();
    }
    const float inv = 1.0f / (float)P;
    for (int i = threadIdx.x; i < C * P; i += 256) {
        int c, u;
        if (a.two_d) {
            c = i / P;
            u = i - c * P;
        } else {
            u = i / C;
            c = i - u * C;
        }
        const int view = a.two_d ? view0 + c : view0;
        const int v = a.two_d ? 0 : v0 + c;
        if (u < U && view < a.n_views && v < V) {
            const int br = (int)(__builtin_bitreverse32((uint32_t)u) >> (32 - L));
            a.out[((size_t)view * U + u) * V + v] =
                a.fview[(size_t)view * kFv + 10] * inv * xf[2 * ((c >> 1) * P + br) + (c & 1)];
        }
    }
}

// ---------------------------------------------------------------------------
// weighted backprojection B (gather) and its transpose (scatter)
// ---------------------------------------------------------------------------

// Per view, float64, in voxel-index coordinates (i, j, k) = (x, y, z) index:
// u_h = Pu . (i, j, k) + pu, v_h likewise, w_h likewise, then
// u = u_h / w_h, v = v_h / w_h, weight = K / w_h^2 (parallel: w_h = 1, K = 1).
constexpr int kBpv = 16;   // Pu(3) pu Pv(3) pv Pw(3) pw K pad pad pad

struct BpArgs {
    const double *bp;
    const float *q;      // B (2D): filtered sinogram in
    const float2 *pairs; // B (3D): views [view0, view1) of the filtered sinogram, pair-interleaved
    float *vol;          // B: volume out; B^T: volume in (read)
    float *sino_out;     // B^T: sinogram out
    int W, H, D, U, V, n_views;
    int view0, view1;    // the views this launch takes
    int accumulate;      // B: add to vol instead of overwriting it
    const float *zw;     // per-slice view weights, zw[view * D + z] (3D with slice weights), else null
    const int2 *zrange;  // per band of TZ slices: the views [x, y) with a nonzero weight there
    int nbx, nby, nbz;
    int two_d;
};

// Pair interleaving of nv views of a (views, U, V) sinogram, with a border
// of zeros: per view (U + 1) x (V + 2) pairs,
//   out[view][u + 1][v + 1] = (q[view][u][v], q[view][u + 1][v]),  u in [-1, U - 1], v in [-1, V],
// q being 0 outside the detector.  The four bilinear taps at (u, v), (u + 1, v),
// (u, v + 1), (u + 1, v + 1) are then the 16 bytes at out[view][u + 1][v + 1],
// one load, for every -1 <= u <= U - 1 and -1 <= v <= V - 1; taps off the
// detector read the zeros.
__global__ __launch_bounds__(256) void fbp_pair_kernel(const float *__restrict__ q, float2 *__restrict__ out,
                                                       int U, int V, size_t nv) {
    const int Vp = V + 2;
    const size_t per = (size_t)(U + 1) * Vp, n = nv * per;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const size_t view = i / per;
        const int r = (int)(i - view * per);
        const int u = r / Vp - 1, v = r % Vp - 1;   // u in [-1, U - 1], v in [-1, V]
        const float *qv = q + view * U * V;
        const bool vin = v >= 0 && v < V;
        out[i] = make_float2(vin && u >= 0 ? qv[(size_t)u * V + v] : 0.f,
                             vin && u + 1 < U ? qv[(size_t)(u + 1) * V + v] : 0.f);
    }
}

// Block-relative constants of one view, for a tile of ZR sub-blocks stacked
// along z (sub-block r centred at X_r = (x0, y0, zc0 + 16 r)).  For a voxel at
// X_r + d (d the same offset in every sub-block):
//   w = Aw_r + Pw . d,   u - u0 = (Au_r + Pu . d - u0 Pw . d) / w,   v likewise
// with integer anchors: v0_r the projection of X_r rounded down, and one u0
// for the whole tile (u barely moves along z); Au_r = u_h(X_r) - u0 w_h(X_r),
// computed in float64: the float32 arithmetic then only meets numbers of the
// size of a sub-block's footprint.  (The u0 slots repeat the tile's anchor.)
// Layout: Pu(3) Pv(3) Pw(3) 1 fast 0 | Au[4] | Av[4] | Aw[4] | u0[4] | v0[4]
// | o0[4] | 0[4], o0 = 8 ((u0 + 1)(V + 2) + v0 + 1) the byte offset of the
// anchor pixel in the view's padded pair-interleaved sinogram (int bits; used
// only for offsets that are in range).  Every P and A is scaled by
// 1 / sqrt(K), which leaves u and v unchanged and makes the weight K / w^2
// the square of the reciprocal of the scaled w.
// fast = 1 when the whole tile (half extents hx, hy, hz about its centre
// (x0, y0, zt)) lies in front of the source and projects inside the detector
// (padded: inside the zero border), so every bilinear tap exists: the
// projection of a box lies inside the hull of its corners' projections.
template <int ZR>
__device__ __forceinline__ void view_consts(const double *p, double x0, double y0, double zc0, double zt,
                                            double hx, double hy, double hz, int U, int V, bool two_d,
                                            bool padded, float *c) {
    const double sk = 1.0 / sqrt(p[12]);   // K > 0 (checked when the plan is made)
    for (int k = 0; k < 3; ++k) {
        c[k] = (float)(sk * p[k]);
        c[3 + k] = (float)(sk * p[4 + k]);
        c[6 + k] = (float)(sk * p[8 + k]);
    }
    c[9] = 1.f;
    c[11] = 0.f;
    // one u anchor for the tile, from the sub-block farthest in front of the
    // source (u hardly changes along z: the tile's u range is a few bins)
    double ubest = 0.0, wbest = 0.0;
#pragma unroll 1
    for (int r = 0; r < ZR; ++r) {
        const double z = zc0 + 16.0 * r;
        const double wh = p[8] * x0 + p[9] * y0 + p[10] * z + p[11];
        if (wh > wbest) {
            wbest = wh;
            ubest = p[0] * x0 + p[1] * y0 + p[2] * z + p[3];
        }
    }
    const double u0 = wbest > 0.0 ? fmin(fmax(floor(ubest / wbest), -1e9), 1e9) : 0.0;
#pragma unroll 1
    for (int r = 0; r < 4; ++r) {
        const double z = zc0 + 16.0 * (r < ZR ? r : 0);
        const double uh = p[0] * x0 + p[1] * y0 + p[2] * z + p[3];
        const double vh = p[4] * x0 + p[5] * y0 + p[6] * z + p[7];
        const double wh = p[8] * x0 + p[9] * y0 + p[10] * z + p[11];
        const double v0 = wh > 0.0 ? fmin(fmax(floor(vh / wh), -1e9), 1e9) : 0.0;
        c[12 + r] = (float)(sk * (uh - u0 * wh));
        c[16 + r] = (float)(sk * (vh - v0 * wh));
        c[20 + r] = (float)(sk * wh);
        c[24 + r] = (float)u0;
        c[28 + r] = (float)v0;
        c[32 + r] = __uint_as_float((uint32_t)((int64_t)(u0 + 1) * (V + 2) + (int64_t)(v0 + 1)) * 8u);
        c[36 + r] = 0.f;
    }
    bool in = true;
#pragma unroll 1
    for (int k = 0; k < 8 && in; ++k) {
        const double X = x0 + ((k & 1) ? hx : -hx), Y = y0 + ((k & 2) ? hy : -hy), Z = zt + ((k & 4) ? hz : -hz);
        const float w = (float)(p[8] * X + p[9] * Y + p[10] * Z + p[11]);
        if (!(w > 0.f)) {
            in = false;
            break;
        }
        // float32 corners (errors ~1e-4 bin, far inside the 0.01 margin).
        // Plain layout: both taps on the detector; padded pairs: floor(u) in
        // [-1, U - 1] and floor(v) in [-1, V - 1] (the border holds the zeros)
        const float u = (float)(p[0] * X + p[1] * Y + p[2] * Z + p[3]) / w;
        const float v = (float)(p[4] * X + p[5] * Y + p[6] * Z + p[7]) / w;
        if (padded)
            in = u >= -0.99f && u <= (float)U - 0.01f && v >= -0.99f && v <= (float)V - 0.01f;
        else
            in = u >= 0.01f && u <= (float)(U - 1) - 0.01f &&
                 (two_d || (v >= 0.01f && v <= (float)(V - 1) - 0.01f));
    }
    c[10] = in ? 1.f : 0.f;
}

// One thread takes ZR voxels of a z column, 16 planes apart (the 16 lanes of
// a row of the wave hold 16 consecutive planes, which for the usual cone
// geometries land on neighbouring detector rows).  Views are taken in LDS
// batches of kBpViews whose block-relative constants the first kBpViews
// threads compute.  SLICEW (3D): each view's term for a voxel of slice z also
// carries the weight zw[view][z] (16 lanes read 16 consecutive floats of the
// view's row), and a block takes only the views of its band's range.
template <bool TRANSPOSE, bool TWO_D, int ZR, bool SLICEW = false>
__global__ __launch_bounds__(256) void fbp_bp_kernel(BpArgs a) {
    static_assert(!(SLICEW && TWO_D), "slice weights are for 3D volumes");
    __shared__ float cst[kBpViews * kBpConst];
    // tile: 3D 4 x 4 x (16 ZR) voxels (x, y, z); 2D 16 x 16
    constexpr int TX = TWO_D ? 16 : 4, TY = TWO_D ? 16 : 4, TZ = TWO_D ? 1 : 16 * ZR;
    // Tile order: z bands outermost, so the blocks resident at one time, on
    // every XCD, read the same detector rows per view; within a band, squares
    // of 8 x 8 tiles, so they also read a narrow range of detector columns
    // (512^3 cone: 105 ms in plain order, 98 / 96 / 99 ms with squares of
    // 16 / 8 / 4 tiles).
    // (Giving each XCD a contiguous range of tiles instead spreads the XCDs over
    // eight bands of z and measured 27% slower at 512^3.)
    constexpr int ST = 8;
    const int b = blockIdx.x, nxy = a.nbx * a.nby;
    const int bz = b / nxy, rem = b - bz * nxy;
    const int sy = rem / (ST * a.nbx), rows_in = min(ST, a.nby - sy * ST), r2 = rem - sy * ST * a.nbx;
    const int sx = r2 / (ST * rows_in), cols_in = min(ST, a.nbx - sx * ST), r3 = r2 - sx * ST * rows_in;
    const int ty = r3 / cols_in;
    const int bx = sx * ST + (r3 - ty * cols_in), by = sy * ST + ty;
    int lx, ly, lz;
    if (TWO_D) {
        lx = threadIdx.x & 15;
        ly = threadIdx.x >> 4;
        lz = 0;
    } else {
        lz = threadIdx.x & 15;
        ly = (threadIdx.x >> 4) & 3;
        lx = threadIdx.x >> 6;
    }
    const int ix = bx * TX + lx, iy = by * TY + ly, iz0 = bz * TZ + lz;
    const bool col_in = ix < a.W && iy < a.H && iz0 < a.D;
    const double X0 = bx * TX + 0.5 * (TX - 1), Y0 = by * TY + 0.5 * (TY - 1);
    const double ZC0 = bz * TZ + (TWO_D ? 0.0 : 7.5);          // centre of sub-block 0
    const double ZT = bz * TZ + 0.5 * (TZ - 1);                // centre of the tile
    const float dx = (float)lx - 0.5f * (TX - 1), dy = (float)ly - 0.5f * (TY - 1),
                dz = TWO_D ? 0.f : (float)lz - 7.5f;
    const size_t plane = (size_t)a.H * a.W;
    const size_t vidx0 = ((size_t)iz0 * a.H + iy) * a.W + ix;
    float fz[ZR], acc[ZR];
#pragma unroll
    for (int r = 0; r < ZR; ++r) {
        const bool in = col_in && iz0 + 16 * r < a.D;
        fz[r] = (TRANSPOSE && in) ? a.vol[vidx0 + (size_t)(16 * r) * plane] : 0.f;
        acc[r] = 0.f;
    }
    bool any = col_in;
    if (TRANSPOSE) {
        any = false;
#pragma unroll
        for (int r = 0; r < ZR; ++r) any = any || fz[r] != 0.f;
    }
    const int U = a.U, V = a.V;
    // One view's contribution to the thread's voxels.  fast_tag: the tile lies
    // in front of the source and every tap of its voxels exists (on the
    // detector, or for the 3D gather within the staging's zero border), so no
    // voxel needs a test.
    auto one_view = [&](int vb, int k, auto fast_tag) {
        const float *ck = cst + k * kBpConst;
        const float4 c0 = *(const float4 *)(ck);        // Pu.x Pu.y Pu.z Pv.x
        const float4 c1 = *(const float4 *)(ck + 4);    // Pv.y Pv.z Pw.x Pw.y
        const float4 c2 = *(const float4 *)(ck + 8);    // Pw.z 1 fast 0
        const float4 au4 = *(const float4 *)(ck + 12);
        const float4 av4 = *(const float4 *)(ck + 16);
        const float4 aw4 = *(const float4 *)(ck + 20);
        const float4 u04 = *(const float4 *)(ck + 24);
        const float4 v04 = *(const float4 *)(ck + 28);
        const float Au[4] = {au4.x, au4.y, au4.z, au4.w}, Av[4] = {av4.x, av4.y, av4.z, av4.w};
        const float Aw[4] = {aw4.x, aw4.y, aw4.z, aw4.w};
        const float U0[4] = {u04.x, u04.y, u04.z, u04.w}, V0[4] = {v04.x, v04.y, v04.z, v04.w};
        const float pud = fmaf(c0.z, dz, fmaf(c0.y, dy, c0.x * dx));
        const float pvd = fmaf(c1.y, dz, fmaf(c1.x, dy, c0.w * dx));
        const float pwd = fmaf(c2.x, dz, fmaf(c1.w, dy, c1.z * dx));
        constexpr bool fast = decltype(fast_tag)::value;
        const size_t vbase = (size_t)(vb + k) * U;
        // slice weights of the thread's voxels (a voxel past the last slice,
        // which is neither read nor written, takes the last slice's)
        float wz[ZR];
#pragma unroll
        for (int r = 0; r < ZR; ++r) wz[r] = 1.f;
        if constexpr (SLICEW) {
            const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(a.zw + (size_t)(vb + k) * a.D, (uint32_t)a.D * 4u);
#pragma unroll
            for (int r = 0; r < ZR; ++r) wz[r] = buffer_load(rz, (uint32_t)min(iz0 + 16 * r, a.D - 1) * 4u);
        }
        if constexpr (!TWO_D && !TRANSPOSE) {
            // 3D gather from the view's padded pair-interleaved copy
            const uint32_t pv = (uint32_t)(U + 1) * (uint32_t)(V + 2) * 8u;
            const __amdgpu_buffer_rsrc_t rq =
                buffer_rsrc((const float *)(a.pairs + (size_t)(vb + k - a.view0) * (U + 1) * (V + 2)), pv);
            const int4 o4 = *(const int4 *)(ck + 32);
            const int O0[4] = {o4.x, o4.y, o4.z, o4.w};
            const int row = 8 * (V + 2);
            const float pud0 = fmaf(-U0[0], pwd, pud);   // the tile's one u anchor
#pragma unroll
            for (int r = 0; r < ZR; ++r) {
                const float w = Aw[r] + pwd;
                const float rw = __builtin_amdgcn_rcpf(w);
                const float su = (Au[r] + pud0) * rw;
                const float sv = fmaf(-V0[r], pwd, Av[r] + pvd) * rw;
                // offsets from the anchor pixel: small signed integers, so a
                // 24-bit multiply-add forms the byte offset
                const float au = __builtin_amdgcn_fractf(su), av = __builtin_amdgcn_fractf(sv);
                uint32_t o = (uint32_t)mad_i24(floor_i32(su), row, floor_i32(sv) * 8 + O0[r]);
                // outside the fast tiles: voxels at or behind the source, or whose
                // taps fall beyond the zero border, add nothing (and read a safe
                // address); near the border a rounding of the test reads zeros
                bool in = true;
                if constexpr (!fast) {
                    const float fu = su + U0[r], fv = sv + V0[r];
                    in = w > 0.f && fu >= -1.f && fu < (float)U && fv >= -1.f && fv < (float)V;
                    o = in ? o : 0u;
                }
                // q(u, v), q(u + 1, v), q(u, v + 1), q(u + 1, v + 1) in one load
                const float4 t = buffer_load4(rq, o);
                const float s0 = fmaf(au, t.y - t.x, t.x), s1 = fmaf(au, t.w - t.z, t.z);
                const float wq = SLICEW ? rw * rw * wz[r] : rw * rw;
                const float nacc = fmaf(wq, fmaf(av, s1 - s0, s0), acc[r]);
                acc[r] = in ? nacc : acc[r];
            }
            return;
        }
        // 2D gather: this view's filtered sinogram, addressed with 32-bit offsets
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(a.q + vbase * V, (uint32_t)U * V * 4u);
#pragma unroll
        for (int r = 0; r < ZR; ++r) {
            const float w = Aw[r] + pwd;
            if (!fast && !(w > 0.f)) continue;   // at or behind the source
            const float rw = __builtin_amdgcn_rcpf(w);
            const float su = fmaf(-U0[r], pwd, Au[r] + pud) * rw;
            const float flu = floorf(su);
            const float au = su - flu;
            const int iu = (int)flu + (int)U0[r];
            const float wgt = rw * rw;   // K / w^2: K is folded into the scaled w
            if (TWO_D) {
                bool ok0 = true, ok1 = true;
                if (!fast) {
                    ok0 = (unsigned)iu < (unsigned)U;
                    ok1 = (unsigned)(iu + 1) < (unsigned)U;
                }
                const float k0 = ok0 ? 1.f - au : 0.f, k1 = ok1 ? au : 0.f;
                const int j0 = ok0 ? iu : 0, j1 = ok1 ? iu + 1 : 0;
                if (TRANSPOSE) {
                    const float g = wgt * fz[r];
                    if (g != 0.f && k0 != 0.f) atomicAdd(a.sino_out + vbase + j0, g * k0);
                    if (g != 0.f && k1 != 0.f) atomicAdd(a.sino_out + vbase + j1, g * k1);
                } else {
                    const float q0 = buffer_load(rq, (uint32_t)j0 * 4u), q1 = buffer_load(rq, (uint32_t)j1 * 4u);
                    acc[r] = fmaf(wgt, fmaf(k0, q0, k1 * q1), acc[r]);
                }
            } else {
                // 3D reaches here for the transpose only (the gather returned above)
                const float sv = fmaf(-V0[r], pwd, Av[r] + pvd) * rw;
                const float flv = floorf(sv);
                const float av = sv - flv;
                const int iv = (int)flv + (int)V0[r];
                bool u0k = true, u1k = true, v0k = true, v1k = true;
                if (!fast) {
                    u0k = (unsigned)iu < (unsigned)U;
                    u1k = (unsigned)(iu + 1) < (unsigned)U;
                    v0k = (unsigned)iv < (unsigned)V;
                    v1k = (unsigned)(iv + 1) < (unsigned)V;
                }
                const float ku0 = u0k ? 1.f - au : 0.f, ku1 = u1k ? au : 0.f;
                const float kv0 = v0k ? 1.f - av : 0.f, kv1 = v1k ? av : 0.f;
                const int ju0 = u0k ? iu : 0, ju1 = u1k ? iu + 1 : 0;
                const int jv0 = v0k ? iv : 0, jv1 = v1k ? iv + 1 : 0;
                const size_t r0 = (vbase + ju0) * V, r1 = (vbase + ju1) * V;
                const float g = SLICEW ? wgt * wz[r] * fz[r] : wgt * fz[r];
                if (g != 0.f) {
                    if (ku0 * kv0 != 0.f) atomicAdd(a.sino_out + r0 + jv0, g * ku0 * kv0);
                    if (ku0 * kv1 != 0.f) atomicAdd(a.sino_out + r0 + jv1, g * ku0 * kv1);
                    if (ku1 * kv0 != 0.f) atomicAdd(a.sino_out + r1 + jv0, g * ku1 * kv0);
                    if (ku1 * kv1 != 0.f) atomicAdd(a.sino_out + r1 + jv1, g * ku1 * kv1);
                }
            }
        }
    };
    __shared__ unsigned char vorder[kBpViews];   // 3D B: the batch's views, fast ones first
    __shared__ int vfast;
    int vlo = a.view0, vhi = a.view1;
    if constexpr (SLICEW) {
        const int2 zr = a.zrange[bz];
        vlo = max(vlo, zr.x);
        vhi = min(vhi, zr.y);
    }
    for (int vb = vlo; vb < vhi; vb += kBpViews) {
        const int nvb = min(kBpViews, vhi - vb);
        __syncthreads();
        if ((int)threadIdx.x < nvb)
            view_consts<ZR>(a.bp + (size_t)(vb + threadIdx.x) * kBpv, X0, Y0, ZC0, ZT, 0.5 * (TX - 1),
                            0.5 * (TY - 1), 0.5 * (TZ - 1), U, V, TWO_D, !TWO_D && !TRANSPOSE,
                            cst + threadIdx.x * kBpConst);
        __syncthreads();
        if constexpr (!TWO_D && !TRANSPOSE) {
            // order the batch: views whose fast flag is set first (each lane of
            // wave 0 ranks views l and l + 64 with ballots), so the two loops
            // below carry no per-view branch
            if (threadIdx.x < 64) {
                const int l = threadIdx.x;
                const bool in0 = l < nvb, in1 = l + 64 < nvb;
                const bool f0 = in0 && cst[l * kBpConst + 10] != 0.f;
                const bool f1 = in1 && cst[(l + 64) * kBpConst + 10] != 0.f;
                const uint64_t bf0 = __ballot(f0), bf1 = __ballot(f1);
                const uint64_t bs0 = __ballot(in0 && !f0), bs1 = __ballot(in1 && !f1);
                const uint64_t below = (1ull << l) - 1ull;
                const int nf0 = __popcll(bf0), nf = nf0 + __popcll(bf1), ns0 = __popcll(bs0);
                if (f0) vorder[__popcll(bf0 & below)] = (unsigned char)l;
                if (f1) vorder[nf0 + __popcll(bf1 & below)] = (unsigned char)(l + 64);
                if (in0 && !f0) vorder[nf + __popcll(bs0 & below)] = (unsigned char)l;
                if (in1 && !f1) vorder[nf + ns0 + __popcll(bs1 & below)] = (unsigned char)(l + 64);
                if (l == 0) vfast = nf;
            }
            __syncthreads();
            if (!any) continue;
            const int nf = vfast;
            for (int i = 0; i < nf; ++i) one_view(vb, vorder[i], std::true_type{});
            for (int i = nf; i < nvb; ++i) one_view(vb, vorder[i], std::false_type{});
        } else {
            if (!any) continue;
            for (int k = 0; k < nvb; ++k) {
                // uniform over the block: a scalar branch
                if (__builtin_amdgcn_readfirstlane(cst[k * kBpConst + 10] != 0.f ? 1 : 0) != 0)
                    one_view(vb, k, std::true_type{});
                else
                    one_view(vb, k, std::false_type{});
            }
        }
    }
    // (a later batch of views that adds nothing to this band leaves it alone)
    if (!TRANSPOSE && !(SLICEW && a.accumulate && vlo >= vhi)) {
#pragma unroll
        for (int r = 0; r < ZR; ++r)
            if (col_in && iz0 + 16 * r < a.D) {
                float *o = a.vol + vidx0 + (size_t)(16 * r) * plane;
                *o = a.accumulate ? *o + acc[r] : acc[r];
            }
    }
}

__global__ void fbp_zero_kernel(float *p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// host: the plan
// ---------------------------------------------------------------------------

struct V3 {
    double x, y, z;
};
V3 operator-(V3 a, V3 b) { return {a.x - b.x, a.y - b.y, a.z - b.z}; }
V3 operator+(V3 a, V3 b) { return {a.x + b.x, a.y + b.y, a.z + b.z}; }
V3 operator*(double s, V3 a) { return {s * a.x, s * a.y, s * a.z}; }
double dot(V3 a, V3 b) { return a.x * b.x + a.y * b.y + a.z * b.z; }
V3 cross(V3 a, V3 b) { return {a.y * b.z - a.z * b.y, a.z * b.x - a.x * b.z, a.x * b.y - a.y * b.x}; }
double norm(V3 a) { return std::sqrt(dot(a, a)); }

struct ViewFrame {
    V3 a, c, eu, ev, n;   // n: unit detector normal, from the source side toward the detector
};

// Windowed Ram-Lak multiplier M_k (k = 0..P/2) for sample spacing d.
std::vector<double> multiplier(int P, double d, int window) {
    std::vector<double> cosT(P);
    for (int j = 0; j < P; ++j) cosT[j] = std::cos(2.0 * M_PI * j / P);
    std::vector<double> h(P, 0.0);
    for (int j = 0; j < P; ++j) {
        const long n = j >= P / 2 + (P % 2) ? (long)j - P : j;   // signed index in [-P/2, P/2)
        if (n == 0) h[j] = 1.0 / (4.0 * d * d);
        else if (n % 2 != 0) h[j] = -1.0 / ((M_PI * (double)n * d) * (M_PI * (double)n * d));
    }
    std::vector<double> M(P / 2 + 1);
    for (int k = 0; k <= P / 2; ++k) {
        double s = 0.0;
        for (int j = 0; j < P; ++j) s += h[j] * cosT[(long)k * j % P];
        const double f = (double)k / P;
        double w = 1.0;
        switch (window) {
            case CT_WINDOW_SHEPP_LOGAN: w = f == 0.0 ? 1.0 : std::sin(M_PI * f) / (M_PI * f); break;
            case CT_WINDOW_COSINE: w = std::cos(M_PI * f); break;
            case CT_WINDOW_HAMMING: w = 0.54 + 0.46 * std::cos(2.0 * M_PI * f); break;
            case CT_WINDOW_HANN: w = 0.5 + 0.5 * std::cos(2.0 * M_PI * f); break;
            default: break;
        }
        M[k] = d * s * w;
    }
    return M;
}

// Spatial taps k[n] = inverse real DFT of M (length P), for n in [-U8, U8).
std::vector<float> filter_taps(int P, int U8, const std::vector<double> &M) {
    std::vector<double> cosT(P);
    for (int j = 0; j < P; ++j) cosT[j] = std::cos(2.0 * M_PI * j / P);
    const int kmax = (P + 1) / 2 - 1;   // bins doubled by the Hermitian symmetry
    std::vector<float> t(2 * (size_t)U8);
    for (int i = 0; i < 2 * U8; ++i) {
        const long n = i - U8;
        const long nm = ((n % P) + P) % P;
        double s = M[0];
        for (int k = 1; k <= kmax; ++k) s += 2.0 * M[k] * cosT[(long)k * nm % P];
        if (P % 2 == 0) s += M[P / 2] * ((nm % 2) ? -1.0 : 1.0);
        t[i] = (float)(s / P);
    }
    return t;
}

bool solve(int n, double A[3][3], double b[3], double x[3]) {
    int piv[3] = {0, 1, 2};
    double M[3][4];
    for (int i = 0; i < n; ++i) {
        for (int j = 0; j < n; ++j) M[i][j] = A[i][j];
        M[i][n] = b[i];
    }
    double scale = 0.0;
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) scale = std::max(scale, std::fabs(A[i][j]));
    for (int c = 0; c < n; ++c) {
        int p = c;
        for (int r = c + 1; r < n; ++r)
            if (std::fabs(M[r][c]) > std::fabs(M[p][c])) p = r;
        if (!(std::fabs(M[p][c]) > 1e-9 * scale)) return false;
        for (int j = 0; j <= n; ++j) std::swap(M[c][j], M[p][j]);
        std::swap(piv[c], piv[p]);
        for (int r = c + 1; r < n; ++r) {
            const double m = M[r][c] / M[c][c];
            for (int j = c; j <= n; ++j) M[r][j] -= m * M[c][j];
        }
    }
    for (int i = n - 1; i >= 0; --i) {
        double s = M[i][n];
        for (int j = i + 1; j < n; ++j) s -= M[i][j] * x[j];
        x[i] = s / M[i][i];
    }
    return true;
}

}  // namespace

struct ct_fbp_s {
    uint64_t magic = 0;
    GeomHost h;
    int device = 0;
    int U8 = 8, VT = 1, S = 8;
    double iso[3] = {0, 0, 0};
    std::vector<double> ang;
    float *d_taps = nullptr;
    int P = 0, L = 0, npair = 0;   // FFT filter: P a power of two <= 4096, else 0
    float2 *d_tw = nullptr;
    float *d_mul = nullptr;
    float *d_fview = nullptr;
    float *d_parker = nullptr;
    double *d_bp = nullptr;
    // 3D backprojection: the pair-interleaved copy of one batch of views
    float2 *d_pairs = nullptr;
    int pair_views = 0;
    bool direct = false;          // step 2 by direct convolution even where the FFT path applies
    float *d_pw = nullptr;        // the caller's pre-weights, or null
    size_t pw_stride = 0;
    float *d_zw = nullptr;        // slice weights, [view][z], or null
    int2 *d_zrange = nullptr;     // per band of 16 kZRun slices: views with a nonzero weight
};

namespace {

void free_plan(ct_fbp_s *f) {
    if (f->d_taps) (void)hipFree(f->d_taps);
    if (f->d_tw) (void)hipFree(f->d_tw);
    if (f->d_mul) (void)hipFree(f->d_mul);
    if (f->d_fview) (void)hipFree(f->d_fview);
    if (f->d_parker) (void)hipFree(f->d_parker);
    if (f->d_bp) (void)hipFree(f->d_bp);
    if (f->d_pairs) (void)hipFree(f->d_pairs);
    if (f->d_pw) (void)hipFree(f->d_pw);
    if (f->d_zw) (void)hipFree(f->d_zw);
    if (f->d_zrange) (void)hipFree(f->d_zrange);
    delete f;
}

bool valid_plan(ct_fbp_t f) { return f && f->magic == kFbpMagic; }

ct_status_t plan_device(ct_fbp_t f) {
    int cur = -1;
    const hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fhip(e, "hipGetDevice");
    if (cur != f->device) return ffail(CT_E_ARG, "current HIP device differs from the plan's device");
    return CT_OK;
}

}  // namespace

extern "C" {

ct_status_t ct_fbp_create(const ct_geom_desc_t *desc, const double *angles, const double *angular_weights,
                          const ct_fbp_opts_t *opts, ct_fbp_t *out) {
    return ct_fbp_create_ext(desc, angles, angular_weights, opts, nullptr, out);
}

ct_status_t ct_fbp_create_ext(const ct_geom_desc_t *desc, const double *angles, const double *angular_weights,
                              const ct_fbp_opts_t *opts, const ct_fbp_ext_t *ext_in, ct_fbp_t *out) {
    if (!out) return ffail(CT_E_NULL, "output plan pointer is NULL");
    *out = nullptr;
    if (!opts) return ffail(CT_E_NULL, "opts is NULL");
    ct_fbp_ext_t ext{};
    if (ext_in) ext = *ext_in;
    for (int k = 0; k < 4; ++k)
        if (ext.reserved[k] != 0) return ffail(CT_E_ARG, "ext reserved fields must be 0");
    if (ext.projection_weights_per_view != 0 && ext.projection_weights_per_view != 1)
        return ffail(CT_E_ARG, "projection_weights_per_view must be 0 or 1");
    if (ext.direct_filter != 0 && ext.direct_filter != 1) return ffail(CT_E_ARG, "direct_filter must be 0 or 1");
    const bool slicew = ext.slice_weights != nullptr;
    GeomHost h;
    const char *why = "";
    ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return ffail(st, why);
    if (h.beam != CT_PARALLEL2D && h.beam != CT_FAN2D && h.beam != CT_CONE)
        return ffail(CT_E_ARG, "FBP/FDK covers parallel2d, fan2d and cone beams");
    if (opts->window < CT_WINDOW_RAMLAK || opts->window > CT_WINDOW_HANN) return ffail(CT_E_ARG, "unknown window");
    if (opts->pad_factor < 1 || opts->pad_factor > 16) return ffail(CT_E_ARG, "pad_factor must be in [1, 16]");
    if (opts->reserved != 0) return ffail(CT_E_ARG, "reserved must be 0");
    const bool persp = h.beam != CT_PARALLEL2D;
    if (opts->short_scan && !persp) return ffail(CT_E_ARG, "short scans (Parker weights) need a fan or cone beam");
    if (h.U < 2 || (h.beam == CT_CONE && h.V < 2)) return ffail(CT_E_SHAPE, "interpolation needs >= 2 detector bins per axis");
    if (slicew && h.beam != CT_CONE) return ffail(CT_E_ARG, "slice weights are for cone beams");
    if (slicew && (angular_weights || opts->short_scan))
        return ffail(CT_E_ARG, "slice weights replace the angular weights; no angular_weights or short_scan with them");
    if (h.U > 4096) return ffail(CT_E_RANGE, "the filter supports U <= 4096");
    if ((int64_t)opts->pad_factor * h.U > 16384) return ffail(CT_E_RANGE, "pad_factor * U must be <= 16384");
    if (h.D * h.H * h.W >= (int64_t(1) << 30) || h.n_views * h.U * h.V >= (int64_t(1) << 31) ||
        h.U * h.V >= (int64_t(1) << 30))
        return ffail(CT_E_RANGE, "volume or sinogram too large for one buffer");
    // cone staging: one view's (U + 1)(V + 2) 8-byte pairs take 32-bit byte offsets
    if (h.beam == CT_CONE && (h.U + 1) * (h.V + 2) >= (int64_t(1) << 29))
        return ffail(CT_E_RANGE, "cone detector too large: (U + 1)(V + 2) must be < 2^29");
    // the gather forms its byte offsets with a signed 24-bit multiply-add whose
    // row operand is 8 (V + 2)
    if (h.beam == CT_CONE && h.V + 2 >= (int64_t(1) << 20))
        return ffail(CT_E_RANGE, "cone detector too large: V + 2 must be < 2^20");
    if (!angular_weights && !angles && !slicew)
        return ffail(CT_E_NULL, "angles (or angular_weights, or slice weights) must be given");
    if (opts->short_scan && !angles) return ffail(CT_E_NULL, "short scans need the angles");
    const int64_t nv = h.n_views;
    if (angles)
        for (int64_t i = 0; i < nv; ++i)
            if (!std::isfinite(angles[i])) return ffail(CT_E_NONFINITE, "angle not finite");
    if (angular_weights)
        for (int64_t i = 0; i < nv; ++i)
            if (!std::isfinite(angular_weights[i])) return ffail(CT_E_NONFINITE, "angular weight not finite");
    if (opts->iso_given)
        for (int k = 0; k < 3; ++k)
            if (!std::isfinite(opts->iso[k])) return ffail(CT_E_NONFINITE, "isocentre not finite");
    const int64_t n_resp = (int64_t)opts->pad_factor * h.U / 2 + 1;
    const int64_t n_pw = (ext.projection_weights_per_view ? nv : 1) * h.U * h.V;
    const int64_t n_sw = h.D * nv;
    auto all_finite = [](const double *p, int64_t n) {
        for (int64_t i = 0; i < n; ++i)
            if (!std::isfinite(p[i])) return false;
        return true;
    };
    if (ext.filter_response && !all_finite(ext.filter_response, n_resp))
        return ffail(CT_E_NONFINITE, "filter response not finite");
    if (ext.projection_weights && !all_finite(ext.projection_weights, n_pw))
        return ffail(CT_E_NONFINITE, "projection weight not finite");
    if (slicew && !all_finite(ext.slice_weights, n_sw)) return ffail(CT_E_NONFINITE, "slice weight not finite");

    // frames and unit normals
    std::vector<ViewFrame> fr(nv);
    for (int64_t i = 0; i < nv; ++i) {
        const double *r = desc->frames + 12 * i;
        ViewFrame &v = fr[i];
        v.a = {r[0], r[1], r[2]};
        v.c = {r[3], r[4], r[5]};
        v.eu = {r[6], r[7], r[8]};
        v.ev = {r[9], r[10], r[11]};
        if (h.beam == CT_CONE) v.n = cross(v.eu, v.ev);
        else v.n = {v.eu.y, -v.eu.x, 0.0};
        v.n = (1.0 / norm(v.n)) * v.n;
        const double toward = persp ? dot(v.c - v.a, v.n) : dot(v.a, v.n);
        if (toward < 0) v.n = -1.0 * v.n;
    }

    ct_fbp_s *f = new (std::nothrow) ct_fbp_s();
    if (!f) return ffail(CT_E_NOMEM, "host allocation failed");
    f->h = h;
    // isocentre: given, or the least-squares point nearest the lines a + t n
    if (opts->iso_given) {
        for (int k = 0; k < 3; ++k) f->iso[k] = opts->iso[k];
        if (h.is2d) f->iso[2] = 0.0;
    } else if (persp) {
        const int dim = h.is2d ? 2 : 3;
        double A[3][3] = {{0}}, b[3] = {0}, x[3] = {0};
        for (const ViewFrame &v : fr) {
            const double nn[3] = {v.n.x, v.n.y, v.n.z}, aa[3] = {v.a.x, v.a.y, v.a.z};
            for (int i = 0; i < dim; ++i)
                for (int j = 0; j < dim; ++j) {
                    const double pij = (i == j ? 1.0 : 0.0) - nn[i] * nn[j];
                    A[i][j] += pij;
                    b[i] += pij * aa[j];
                }
        }
        if (!solve(dim, A, b, x)) {
            delete f;
            return ffail(CT_E_ARG, "the isocentre cannot be estimated from these views; pass it");
        }
        for (int k = 0; k < dim; ++k) f->iso[k] = x[k];
    }
    // angular weights: given, or half the gaps to the neighbouring views
    f->ang.assign(nv, 0.0);
    const bool redundant = persp && !opts->short_scan;
    if (slicew) {
        f->ang.assign(nv, 1.0);   // the slice weights carry the quadrature
    } else if (angular_weights) {
        for (int64_t i = 0; i < nv; ++i) f->ang[i] = angular_weights[i];
    } else if (nv == 1) {
        f->ang[0] = M_PI;
    } else if (opts->short_scan) {
        for (int64_t i = 0; i < nv; ++i) {
            const double lo = angles[i > 0 ? i - 1 : 0], hi = angles[i + 1 < nv ? i + 1 : nv - 1];
            f->ang[i] = 0.5 * std::fabs(hi - lo);
        }
    } else {
        const double period = persp ? 2.0 * M_PI : M_PI;
        const double sgn = angles[nv - 1] >= angles[0] ? 1.0 : -1.0;
        for (int64_t i = 0; i < nv; ++i) {
            const double nx = i + 1 < nv ? angles[i + 1] : angles[0] + sgn * period;
            const double pv = i > 0 ? angles[i - 1] : angles[nv - 1] - sgn * period;
            f->ang[i] = 0.5 * std::fabs(nx - pv) * (redundant ? 0.5 : 1.0);
        }
    }
    const int U = (int)h.U, V = (int)h.V;
    // Parker weights
    std::vector<float> parker;
    if (opts->short_scan) {
        double rot = 0.0;
        for (int64_t i = 0; i + 1 < nv; ++i) rot += fr[i].a.x * fr[i + 1].a.y - fr[i].a.y * fr[i + 1].a.x;
        const double sense = rot >= 0 ? 1.0 : -1.0;
        std::vector<double> gam((size_t)nv * U);
        double delta = 0.0;
        for (int64_t i = 0; i < nv; ++i)
            for (int u = 0; u < U; ++u) {
                const V3 p = fr[i].c + ((u - 0.5 * (U - 1)) * h.du) * fr[i].eu;
                const V3 d = p - fr[i].a;
                const double cr = fr[i].n.x * d.y - fr[i].n.y * d.x, dt = fr[i].n.x * d.x + fr[i].n.y * d.y;
                const double g = sense * std::atan2(cr, dt);
                gam[(size_t)i * U + u] = g;
                delta = std::max(delta, std::fabs(g));
            }
        double span = 0.0;
        for (int64_t i = 0; i < nv; ++i) span = std::max(span, std::fabs(angles[i] - angles[0]));
        if (span < M_PI + 2.0 * delta - 1e-9 * (M_PI + 2.0 * delta)) {
            delete f;
            return ffail(CT_E_ARG, "a short scan needs an angular span of at least pi + 2 x half fan angle");
        }
        parker.resize((size_t)nv * U);
        for (int64_t i = 0; i < nv; ++i) {
            const double be = std::fabs(angles[i] - angles[0]);
            for (int u = 0; u < U; ++u) {
                const double g = gam[(size_t)i * U + u];
                double w = 0.0;
                if (be >= 0 && be < 2.0 * (delta - g)) {
                    const double s = std::sin(M_PI / 4.0 * be / (delta - g));
                    w = s * s;
                } else if (be >= 2.0 * (delta - g) && be <= M_PI - 2.0 * g) {
                    w = 1.0;
                } else if (be > M_PI - 2.0 * g && be <= M_PI + 2.0 * delta) {
                    const double s = std::sin(M_PI / 4.0 * (M_PI + 2.0 * delta - be) / (delta + g));
                    w = s * s;
                }
                parker[(size_t)i * U + u] = (float)w;
            }
        }
    }
    // filter: taps, launch shape
    const int P = opts->pad_factor * U;
    f->U8 = (U + 7) / 8 * 8;
    // rows per block: at most four tasks of 8 outputs per thread, LDS under 64 KB
    f->VT = f->U8 <= 512 ? 16 : (f->U8 <= 1024 ? 8 : (f->U8 <= 2048 ? 2 : 1));
    f->S = f->U8 + 4;
    const std::vector<double> mult = ext.filter_response
                                         ? std::vector<double>(ext.filter_response, ext.filter_response + n_resp)
                                         : multiplier(P, h.du, opts->window);
    const std::vector<float> taps = filter_taps(P, f->U8, mult);
    // FFT path: P a power of two in [64, 4096]
    std::vector<float2> twf;
    std::vector<float> mulf;
    if ((P & (P - 1)) == 0 && P >= 64 && P <= 4096) {
        f->P = P;
        f->L = 0;
        while ((1 << f->L) < P) ++f->L;
        f->npair = std::max(1, std::min(8, 4096 / P));
        twf.resize(P / 2);
        for (int t = 0; t < P / 2; ++t)
            twf[t] = make_float2((float)std::cos(2.0 * M_PI * t / P), (float)-std::sin(2.0 * M_PI * t / P));
        mulf.resize(P / 2 + 1);
        for (int k = 0; k <= P / 2; ++k) mulf[k] = (float)mult[k];
    }
    std::vector<float> fview((size_t)nv * kFv, 0.f);
    std::vector<double> bp((size_t)nv * kBpv, 0.0);
    // voxel centre of index (i, j, k): lo + (idx + 0.5) s per axis; 2D: z = 0
    const double sx = h.sx, sy = h.sy, sz = h.is2d ? 1.0 : h.sz;
    const V3 lo = {-0.5 * h.W * sx + 0.5 * sx, -0.5 * h.H * sy + 0.5 * sy,
                   h.is2d ? 0.0 : -0.5 * h.D * sz + 0.5 * sz};
    const V3 iso = {f->iso[0], f->iso[1], f->iso[2]};
    for (int64_t i = 0; i < nv; ++i) {
        const ViewFrame &v = fr[i];
        float *fv = fview.data() + i * kFv;
        double *t = bp.data() + i * kBpv;
        V3 Pu, Pv, Pw;
        double pu, pv, pw, K;
        if (persp) {
            const double D = dot(v.c - v.a, v.n), R = dot(iso - v.a, v.n);
            if (!(R > 0.0)) {
                delete f;
                return ffail(CT_E_ARG, "the isocentre must lie in front of every source");
            }
            const V3 ca = v.c - v.a;
            fv[0] = (float)D;
            fv[1] = (float)ca.x; fv[2] = (float)ca.y; fv[3] = (float)ca.z;
            fv[11] = 1.f;
            // w(X) = (X - a).n ; u_h = alpha_u w + (D / du) (X - a).e_u
            const double au = dot(v.a - v.c, v.eu) / h.du + 0.5 * (U - 1);
            const double av = h.is2d ? 0.0 : dot(v.a - v.c, v.ev) / h.dv + 0.5 * (V - 1);
            Pw = v.n;
            pw = -dot(v.a, v.n);
            Pu = au * v.n + (D / h.du) * v.eu;
            pu = -au * dot(v.a, v.n) - (D / h.du) * dot(v.a, v.eu);
            if (h.is2d) {
                Pv = {0, 0, 0};
                pv = 0.0;
            } else {
                Pv = av * v.n + (D / h.dv) * v.ev;
                pv = -av * dot(v.a, v.n) - (D / h.dv) * dot(v.a, v.ev);
            }
            K = R * D;
        } else {
            fv[11] = 0.f;
            Pw = {0, 0, 0};
            pw = 1.0;
            Pu = (1.0 / h.du) * v.eu;
            pu = -dot(v.c, v.eu) / h.du + 0.5 * (U - 1);
            Pv = {0, 0, 0};
            pv = 0.0;
            K = 1.0;
        }
        fv[4] = (float)(v.eu.x * h.du); fv[5] = (float)(v.eu.y * h.du); fv[6] = (float)(v.eu.z * h.du);
        fv[7] = (float)(v.ev.x * h.dv); fv[8] = (float)(v.ev.y * h.dv); fv[9] = (float)(v.ev.z * h.dv);
        fv[10] = (float)f->ang[i];
        // to index coordinates: X = lo + idx * s
        auto put = [&](int off, V3 P, double p) {
            t[off + 0] = P.x * sx;
            t[off + 1] = P.y * sy;
            t[off + 2] = P.z * sz;
            t[off + 3] = dot(P, lo) + p;
        };
        put(0, Pu, pu);
        put(4, Pv, pv);
        put(8, Pw, pw);
        t[12] = K;
    }
    hipError_t e = hipGetDevice(&f->device);
    if (e == hipSuccess) e = hipMalloc((void **)&f->d_taps, taps.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void **)&f->d_fview, fview.size() * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void **)&f->d_bp, bp.size() * sizeof(double));
    if (e == hipSuccess && !parker.empty()) e = hipMalloc((void **)&f->d_parker, parker.size() * sizeof(float));
    if (e == hipSuccess && f->P) e = hipMalloc((void **)&f->d_tw, twf.size() * sizeof(float2));
    if (e == hipSuccess && f->P) e = hipMalloc((void **)&f->d_mul, mulf.size() * sizeof(float));
    // overrides: pre-weights as float; slice weights transposed to [view][z], and
    // per band of 16 kZRun slices the range of views with a nonzero weight there
    std::vector<float> pwf, zwf;
    std::vector<int2> zr;
    if (ext.projection_weights) {
        pwf.assign(ext.projection_weights, ext.projection_weights + n_pw);
        f->pw_stride = ext.projection_weights_per_view ? (size_t)(h.U * h.V) : 0;
        if (e == hipSuccess) e = hipMalloc((void **)&f->d_pw, pwf.size() * sizeof(float));
    }
    if (slicew) {
        const int64_t D = h.D, TZ = 16 * kZRun, nbz = (D + TZ - 1) / TZ;
        zwf.resize((size_t)(nv * D));
        zr.assign((size_t)nbz, make_int2(0, 0));
        for (int64_t b = 0; b < nbz; ++b) {
            int64_t lo = nv, hi = 0;
            for (int64_t z = b * TZ; z < std::min(D, (b + 1) * TZ); ++z)
                for (int64_t i = 0; i < nv; ++i)
                    if (ext.slice_weights[z * nv + i] != 0.0) {
                        lo = std::min(lo, i);
                        hi = std::max(hi, i + 1);
                    }
            if (lo < hi) zr[(size_t)b] = make_int2((int)lo, (int)hi);
        }
        for (int64_t z = 0; z < D; ++z)
            for (int64_t i = 0; i < nv; ++i) zwf[(size_t)(i * D + z)] = (float)ext.slice_weights[z * nv + i];
        if (e == hipSuccess) e = hipMalloc((void **)&f->d_zw, zwf.size() * sizeof(float));
        if (e == hipSuccess) e = hipMalloc((void **)&f->d_zrange, zr.size() * sizeof(int2));
    }
    f->direct = ext.direct_filter != 0;
    if (!h.is2d) {
        // equal batches of at most kBpViews views, and of at most kStagingBytes
        // of staging (large detectors take smaller batches)
        const int64_t per_view = (h.U + 1) * (h.V + 2) * (int64_t)sizeof(float2);
        const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(kBpViews, kStagingBytes / per_view));
        const int64_t nb = (h.n_views + cap - 1) / cap;
        f->pair_views = (int)((h.n_views + nb - 1) / nb);
        if (e == hipSuccess)
            e = hipMalloc((void **)&f->d_pairs, (size_t)f->pair_views * (h.U + 1) * (h.V + 2) * sizeof(float2));
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        free_plan(f);
        return ffail(CT_E_NOMEM, "hipMalloc of the FBP tables failed");
    }
    e = hipMemcpy(f->d_taps, taps.data(), taps.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(f->d_fview, fview.data(), fview.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(f->d_bp, bp.data(), bp.size() * sizeof(double), hipMemcpyHostToDevice);
    if (e == hipSuccess && !parker.empty())
        e = hipMemcpy(f->d_parker, parker.data(), parker.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && f->P) e = hipMemcpy(f->d_tw, twf.data(), twf.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e == hipSuccess && f->P) e = hipMemcpy(f->d_mul, mulf.data(), mulf.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && f->d_pw) e = hipMemcpy(f->d_pw, pwf.data(), pwf.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && f->d_zw) e = hipMemcpy(f->d_zw, zwf.data(), zwf.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess && f->d_zrange)
        e = hipMemcpy(f->d_zrange, zr.data(), zr.size() * sizeof(int2), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        free_plan(f);
        return fhip(e, "upload of the FBP tables");
    }
    f->magic = kFbpMagic;
    *out = f;
    set_error("");
    return CT_OK;
}

ct_status_t ct_fbp_destroy(ct_fbp_t f) {
    if (!f) return CT_OK;
    if (!valid_plan(f)) return ffail(CT_E_ARG, "invalid FBP plan");
    f->magic = 0;
    free_plan(f);
    set_error("");
    return CT_OK;
}

ct_status_t ct_fbp_info(ct_fbp_t f, double *iso, double *angular_weights) {
    if (!valid_plan(f)) return ffail(CT_E_ARG, "invalid FBP plan");
    if (iso)
        for (int k = 0; k < 3; ++k) iso[k] = f->iso[k];
    if (angular_weights) std::memcpy(angular_weights, f->ang.data(), f->ang.size() * sizeof(double));
    set_error("");
    return CT_OK;
}

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const char *x = (const char *)a, *y = (const char *)b;
    return x < y + nb && y < x + na;
}

ct_status_t ct_fbp_filter(ct_fbp_t f, const float *sino, float *filtered, ct_stream_t stream) {
    if (!valid_plan(f)) return ffail(CT_E_ARG, "invalid FBP plan");
    if (!sino || !filtered) return ffail(CT_E_NULL, "sino and filtered must be non-NULL");
    const GeomHost &h = f->h;
    const size_t sb = (size_t)h.n_views * h.U * h.V * sizeof(float);
    if (overlaps(sino, sb, filtered, sb)) return ffail(CT_E_ALIAS, "filtered overlaps sino");
    ct_status_t st = plan_device(f);
    if (st != CT_OK) return st;
    if (f->P && !f->direct) {
        FftArgs b;
        b.sino = sino;
        b.out = filtered;
        b.tw = f->d_tw;
        b.mul = f->d_mul;
        b.fview = f->d_fview;
        b.parker = f->d_parker;
        b.pw = f->d_pw;
        b.pw_stride = f->pw_stride;
        b.U = (int)h.U;
        b.V = (int)h.V;
        b.n_views = (int)h.n_views;
        b.P = f->P;
        b.L = f->L;
        b.npair = f->npair;
        b.two_d = h.is2d ? 1 : 0;
        const int C = 2 * f->npair;
        const unsigned blocks = h.is2d ? (unsigned)((h.n_views + C - 1) / C)
                                       : (unsigned)(h.n_views * ((h.V + C - 1) / C));
        const size_t lds = (size_t)f->npair * f->P * sizeof(float2) + (size_t)(f->P / 2) * sizeof(float2) +
                           (size_t)(f->P / 2 + 1) * sizeof(float);
        hipLaunchKernelGGL(fbp_fft_filter_kernel, dim3(blocks), dim3(256), lds, (hipStream_t)stream, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fhip(e, "ct_fbp_filter launch");
        set_error("");
        return CT_OK;
    }
    FilterArgs a;
    a.sino = sino;
    a.out = filtered;
    a.taps = f->d_taps;
    a.fview = f->d_fview;
    a.parker = f->d_parker;
    a.pw = f->d_pw;
    a.pw_stride = f->pw_stride;
    a.U = (int)h.U;
    a.V = (int)h.V;
    a.n_views = (int)h.n_views;
    a.U8 = f->U8;
    a.VT = f->VT;
    a.S = f->S;
    a.two_d = h.is2d ? 1 : 0;
    const unsigned blocks = h.is2d ? (unsigned)((h.n_views + f->VT - 1) / f->VT)
                                   : (unsigned)(h.n_views * ((h.V + f->VT - 1) / f->VT));
    const size_t lds = (2 * (size_t)f->U8 + (size_t)f->VT * f->S) * sizeof(float);
    hipLaunchKernelGGL(fbp_filter_kernel, dim3(blocks), dim3(256), lds, (hipStream_t)stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fhip(e, "ct_fbp_filter launch");
    set_error("");
    return CT_OK;
}

static BpArgs bp_args(ct_fbp_t f) {
    const GeomHost &h = f->h;
    BpArgs a;
    a.bp = f->d_bp;
    a.W = (int)h.W;
    a.H = (int)h.H;
    a.D = (int)h.D;
    a.U = (int)h.U;
    a.V = (int)h.V;
    a.n_views = (int)h.n_views;
    a.two_d = h.is2d ? 1 : 0;
    const int TX = h.is2d ? 16 : 4, TY = h.is2d ? 16 : 4, TZ = h.is2d ? 1 : 16 * kZRun;
    a.nbx = (a.W + TX - 1) / TX;
    a.nby = (a.H + TY - 1) / TY;
    a.nbz = (a.D + TZ - 1) / TZ;
    a.q = nullptr;
    a.pairs = nullptr;
    a.vol = nullptr;
    a.sino_out = nullptr;
    a.view0 = 0;
    a.view1 = a.n_views;
    a.accumulate = 0;
    a.zw = f->d_zw;
    a.zrange = f->d_zrange;
    return a;
}

ct_status_t ct_fbp_backproject(ct_fbp_t f, const float *filtered, float *vol, ct_stream_t stream) {
    if (!valid_plan(f)) return ffail(CT_E_ARG, "invalid FBP plan");
    if (!filtered || !vol) return ffail(CT_E_NULL, "filtered and vol must be non-NULL");
    const GeomHost &h = f->h;
    const size_t sb = (size_t)h.n_views * h.U * h.V * sizeof(float), vb = (size_t)h.D * h.H * h.W * sizeof(float);
    if (overlaps(filtered, sb, vol, vb)) return ffail(CT_E_ALIAS, "vol overlaps filtered");
    ct_status_t st = plan_device(f);
    if (st != CT_OK) return st;
    BpArgs a = bp_args(f);
    a.q = filtered;
    a.vol = vol;
    const dim3 grid((unsigned)(a.nbx * a.nby * a.nbz));
    if (h.is2d) {
        hipLaunchKernelGGL((fbp_bp_kernel<false, true, 1>), grid, dim3(256), 0, (hipStream_t)stream, a);
    } else {
        // batches of views: pair-interleave the batch, then gather from it
        // (the first batch writes the volume, the others add to it)
        const size_t per_view = (size_t)h.U * h.V, per_pairs = (size_t)(h.U + 1) * (h.V + 2);
        for (int v0 = 0; v0 < (int)h.n_views; v0 += f->pair_views) {
            const int v1 = (int)std::min<int64_t>(h.n_views, (int64_t)v0 + f->pair_views);
            const size_t n = (size_t)(v1 - v0) * per_pairs;
            hipLaunchKernelGGL(fbp_pair_kernel, dim3((unsigned)std::min<size_t>((n + 255) / 256, 65536)), dim3(256),
                               0, (hipStream_t)stream, filtered + (size_t)v0 * per_view, f->d_pairs, a.U, a.V,
                               (size_t)(v1 - v0));
            a.pairs = f->d_pairs;
            a.view0 = v0;
            a.view1 = v1;
            a.accumulate = v0 > 0 ? 1 : 0;
            if (f->d_zw)
                hipLaunchKernelGGL((fbp_bp_kernel<false, false, kZRun, true>), grid, dim3(256), 0,
                                   (hipStream_t)stream, a);
            else
                hipLaunchKernelGGL((fbp_bp_kernel<false, false, kZRun>), grid, dim3(256), 0, (hipStream_t)stream, a);
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fhip(e, "ct_fbp_backproject launch");
    set_error("");
    return CT_OK;
}

ct_status_t ct_fbp_backproject_transpose(ct_fbp_t f, const float *vol, float *sino, ct_stream_t stream) {
    if (!valid_plan(f)) return ffail(CT_E_ARG, "invalid FBP plan");
    if (!vol || !sino) return ffail(CT_E_NULL, "vol and sino must be non-NULL");
    const GeomHost &h = f->h;
    const size_t sn = (size_t)h.n_views * h.U * h.V, vb = (size_t)h.D * h.H * h.W * sizeof(float);
    if (overlaps(sino, sn * sizeof(float), vol, vb)) return ffail(CT_E_ALIAS, "sino overlaps vol");
    ct_status_t st = plan_device(f);
    if (st != CT_OK) return st;
    hipLaunchKernelGGL(fbp_zero_kernel, dim3(2048), dim3(256), 0, (hipStream_t)stream, sino, sn);
    BpArgs a = bp_args(f);
    a.vol = const_cast<float *>(vol);   // read only in the transpose
    a.sino_out = sino;
    const dim3 grid((unsigned)(a.nbx * a.nby * a.nbz));
    if (h.is2d) hipLaunchKernelGGL((fbp_bp_kernel<true, true, 1>), grid, dim3(256), 0, (hipStream_t)stream, a);
    else if (f->d_zw)
        hipLaunchKernelGGL((fbp_bp_kernel<true, false, kZRun, true>), grid, dim3(256), 0, (hipStream_t)stream, a);
    else hipLaunchKernelGGL((fbp_bp_kernel<true, false, kZRun>), grid, dim3(256), 0, (hipStream_t)stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fhip(e, "ct_fbp_backproject_transpose launch");
    set_error("");
    return CT_OK;
}

ct_status_t ct_fbp_run(ct_fbp_t f, const float *sino, float *work, float *vol, ct_stream_t stream) {
    if (!valid_plan(f)) return ffail(CT_E_ARG, "invalid FBP plan");
    if (!sino || !work || !vol) return ffail(CT_E_NULL, "sino, work and vol must be non-NULL");
    const GeomHost &h = f->h;
    const size_t vb = (size_t)h.D * h.H * h.W * sizeof(float), sb = (size_t)h.n_views * h.U * h.V * sizeof(float);
    if (overlaps(sino, sb, vol, vb) || overlaps(sino, sb, work, sb) || overlaps(work, sb, vol, vb))
        return ffail(CT_E_ALIAS, "sino, work and vol must not overlap");
    ct_status_t st = ct_fbp_filter(f, sino, work, stream);
    if (st != CT_OK) return st;
    return ct_fbp_backproject(f, work, vol, stream);
}

// Helical approximation: per slice, the full turn centred at the angle where
// the source crosses the slice centre, integrated by the trapezoidal rule on the
// sampled angles (the hat functions of the linear interpolation), times 1/2.
ct_status_t ct_helical_view_weights(const ct_geom_desc_t *desc, const double *angles, double *weights) {
    if (!angles || !weights) return ffail(CT_E_NULL, "angles and weights must be non-NULL");
    GeomHost h;
    const char *why = "";
    const ct_status_t st = validate_desc(desc, &h, &why);
    if (st != CT_OK) return ffail(st, why);
    if (h.beam != CT_CONE) return ffail(CT_E_ARG, "the helical approximation is a cone-beam method");
    const int64_t nv = h.n_views, D = h.D;
    if (nv < 2) return ffail(CT_E_ARG, "the helical weights need at least two views");
    for (int64_t i = 0; i < nv; ++i)
        if (!std::isfinite(angles[i])) return ffail(CT_E_NONFINITE, "angle not finite");
    // work in increasing t = sa * angle and increasing key = sz * source z
    const double sa = angles[nv - 1] > angles[0] ? 1.0 : -1.0;
    const double sz = desc->frames[12 * (nv - 1) + 2] > desc->frames[2] ? 1.0 : -1.0;
    std::vector<double> t((size_t)nv), zs((size_t)nv);
    for (int64_t i = 0; i < nv; ++i) {
        t[(size_t)i] = sa * angles[i];
        zs[(size_t)i] = desc->frames[12 * i + 2];
    }
    for (int64_t i = 1; i < nv; ++i) {
        if (!(t[(size_t)i] > t[(size_t)i - 1])) return ffail(CT_E_ARG, "the unwrapped angles must be strictly monotone");
        if (!(sz * zs[(size_t)i] > sz * zs[(size_t)i - 1]))
            return ffail(CT_E_ARG, "the source z must be strictly monotone");
    }
    const double tol = 1e-9 * (1.0 + std::max(std::fabs(t[0]), std::fabs(t[(size_t)nv - 1])));
    std::vector<double> w((size_t)(D * nv), 0.0);
    char msg[160];
    for (int64_t s = 0; s < D; ++s) {
        const double zc = -0.5 * (double)D * h.sz + ((double)s + 0.5) * h.sz;
        const double key = sz * zc;
        if (key < sz * zs[0] || key > sz * zs[(size_t)nv - 1]) {
            std::snprintf(msg, sizeof msg, "slice %lld (z = %g) lies outside the source's z range", (long long)s, zc);
            return ffail(CT_E_RANGE, msg);
        }
        int64_t lo = 0, hi = nv - 1;   // the last sample at or below the slice, at most nv - 2
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) / 2;
            if (sz * zs[(size_t)mid] <= key) lo = mid;
            else hi = mid;
        }
        const double fz = (zc - zs[(size_t)lo]) / (zs[(size_t)lo + 1] - zs[(size_t)lo]);
        const double tc = t[(size_t)lo] + fz * (t[(size_t)lo + 1] - t[(size_t)lo]);
        double a = tc - M_PI, b = tc + M_PI;
        if (a < t[0] - tol || b > t[(size_t)nv - 1] + tol) {
            std::snprintf(msg, sizeof msg, "slice %lld: the full turn about its crossing angle leaves the scan",
                          (long long)s);
            return ffail(CT_E_RANGE, msg);
        }
        a = std::max(a, t[0]);
        b = std::min(b, t[(size_t)nv - 1]);
        for (int64_t i = 0; i < nv; ++i) {
            double acc = 0.0;
            if (i > 0) {   // rising side: (x - t[i-1]) / L over [l, r]
                const double tp = t[(size_t)i - 1], l = std::max(a, tp), r = std::min(b, t[(size_t)i]);
                if (r > l) acc += (r - l) * ((r - tp) + (l - tp)) / (2.0 * (t[(size_t)i] - tp));
            }
            if (i + 1 < nv) {   // falling side: (t[i+1] - x) / L over [l, r]
                const double tn = t[(size_t)i + 1], l = std::max(a, t[(size_t)i]), r = std::min(b, tn);
                if (r > l) acc += (r - l) * ((tn - l) + (tn - r)) / (2.0 * (tn - t[(size_t)i]));
            }
            w[(size_t)(s * nv + i)] = 0.5 * acc;
        }
    }
    std::memcpy(weights, w.data(), w.size() * sizeof(double));
    set_error("");
    return CT_OK;
}

}  // extern "C"
