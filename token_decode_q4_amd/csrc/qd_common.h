// qd_common.h -- device helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#define QD_DEV __device__ __forceinline__

namespace qd {

constexpr int WAVE = 64;

QD_DEV float f16_to_f32(uint16_t h) { return __half2float(__ushort_as_half(h)); }
// round to nearest even
QD_DEV uint16_t f32_to_f16(float f) { return __half_as_ushort(__float2half_rn(f)); }

// Cross-lane steps without LDS traffic: DPP moves inside rows of 16 lanes and
// the gfx950 permlane swaps across rows.  Each step pairs lanes symmetrically
// (lane a reads b exactly when b reads a), so a reduction built from them
// leaves the identical value in every lane of a group.
namespace lanes {
template <int CTRL>
QD_DEV float mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int HMIRROR = 0x141;  // row_half_mirror: lane i <-> 7-i within 8
constexpr int MIRROR = 0x140;   // row_mirror: lane i <-> 15-i within 16
// v of this lane's row and of the partner row (16 or 32 lanes away); r[0] is
// always the lower row's value and r[1] the upper row's
QD_DEV void swap16(float v, float& lo, float& hi)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
QD_DEV void swap32(float v, float& lo, float& hi)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
}  // namespace lanes

// sum over aligned groups of WIDTH consecutive lanes (WIDTH a power of two
// <= 64); every lane of a group ends with the group's sum.  Fixed order, so
// deterministic.  All lanes of the wave must be active.
template <int WIDTH>
QD_DEV float group_sum(float v)
{
    if (WIDTH >= 2)
        v += lanes::mov<lanes::XOR1>(v);
    if (WIDTH >= 4)
        v += lanes::mov<lanes::XOR2>(v);
    if (WIDTH >= 8)
        v += lanes::mov<lanes::HMIRROR>(v);
    if (WIDTH >= 16)
        v += lanes::mov<lanes::MIRROR>(v);
    if (WIDTH >= 32) {
        float lo, hi;
        lanes::swap16(v, lo, hi);
        v = lo + hi;
    }
    if (WIDTH >= 64) {
        float lo, hi;
        lanes::swap32(v, lo, hi);
        v = lo + hi;
    }
    return v;
}

template <int WIDTH>
QD_DEV float group_max(float v)
{
    if (WIDTH >= 2)
        v = fmaxf(v, lanes::mov<lanes::XOR1>(v));
    if (WIDTH >= 4)
        v = fmaxf(v, lanes::mov<lanes::XOR2>(v));
    if (WIDTH >= 8)
        v = fmaxf(v, lanes::mov<lanes::HMIRROR>(v));
    if (WIDTH >= 16)
        v = fmaxf(v, lanes::mov<lanes::MIRROR>(v));
    if (WIDTH >= 32) {
        float lo, hi;
        lanes::swap16(v, lo, hi);
        v = fmaxf(lo, hi);
    }
    if (WIDTH >= 64) {
        float lo, hi;
        lanes::swap32(v, lo, hi);
        v = fmaxf(lo, hi);
    }
    return v;
}

QD_DEV float slab_add(float a, float b) { return a + b; }
QD_DEV float2 slab_add(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
QD_DEV float4 slab_add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }

// p[0] + p[stride] + .. + p[(n-1) stride], n >= 1 partial products (K
// slices) of one value, added in that order.  The loads of each group of G
// are all issued before any is used (indexes clamped, no branch around a
// load): adding each term as its load arrived would wait out one memory
// latency per term.
template <int G, class T>
QD_DEV T slab_sum(const T* p, int n, size_t stride)
{
    T r{};   // set by the first term
    for (int k0 = 0; k0 < n; k0 += G) {
        T t[G];
#pragma unroll
        for (int u = 0; u < G; ++u)
            t[u] = p[(size_t)min(k0 + u, n - 1) * stride];
#pragma unroll
        for (int u = 0; u < G; ++u)
            if (k0 + u < n)
                r = (k0 + u == 0) ? t[0] : slab_add(r, t[u]);
    }
    return r;
}

// Timeline marks for profiling builds only: with QD_TIMELINE defined, thread 0
// of every workgroup stores the 100 MHz real-time counter for mark k (0..7) at
// qd_tl[8 * w + k], w = the linear workgroup index; the profiling host points
// qd_tl at a buffer of 8 entries per workgroup before each launch (a
// __constant__ pointer: read with a scalar load, so a mark never waits on the
// kernel's vector loads).  Without QD_TIMELINE a mark is nothing.
#ifdef QD_TIMELINE
__constant__ uint64_t* qd_tl;
#define QD_MARK(k)                                                          \
    do {                                                                    \
        if (threadIdx.x == 0 && qd_tl)                                      \
            qd_tl[8 * (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)) + (k)] = \
                __builtin_amdgcn_s_memrealtime();                              \
    } while (0)
#else
#define QD_MARK(k) \
    do {           \
    } while (0)
#endif

}  // namespace qd
