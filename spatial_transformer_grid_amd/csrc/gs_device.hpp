// gs_device.hpp -- device-side building blocks of libgsample (gfx950).
//
// Coordinates: every helper that decides a pixel index (base positions of the
// grid generator, un-normalisation, padding of a location) is written as a
// sequence of individually rounded fp32 operations.  The library is compiled
// with -ffp-contract=off so none of them is fused into an FMA; interpolation
// uses explicit fmaf where it wants one.
//
// Memory: X and Y are addressed through raw buffer resources, one per
// (image, channel) plane, with num_records = plane bytes.  Y is written once
// and never read back, so its stores are non-temporal (they stream through L2
// without displacing the input rows that neighbouring tiles still need).  A tap whose
// location is outside the image gets the offset GS_OOB (>= any plane size),
// which the buffer unit turns into a read of 0 (zeros padding) or a dropped
// store, without touching memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

enum : int { MODE_LINEAR = 0, MODE_NEAREST = 1, MODE_CUBIC = 2 };
enum : int { PAD_ZEROS = 0, PAD_BORDER = 1, PAD_REFLECTION = 2 };

constexpr int kBlock = 256;              // threads per block: 4 wave64s
constexpr uint32_t GS_OOB = 0x80000000u; // buffer offset that is always out of range
constexpr float kCoordLimit = 16777216.0f;  // |p| clamp before float->int (2^24)
constexpr float kCubicA = -0.75f;        // cubic convolution coefficient
constexpr int kStoreNT = 2;              // buffer cache-policy bit: non-temporal

// Word 3 of a gfx9-family buffer resource: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// ------------------------------------------------------------------ types

struct F32 {
    static constexpr int bytes = 4;
    typedef uint32_t raw_t;
    __device__ __forceinline__ static float load(rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    __device__ __forceinline__ static uint32_t load_raw(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
    }
    __device__ __forceinline__ static void store(float v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, kStoreNT);
    }
    __device__ __forceinline__ static void store_raw(uint32_t v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kStoreNT);
    }
    __device__ __forceinline__ static float from_raw(uint32_t v) {
        return __builtin_bit_cast(float, v);
    }
};

// The fp32 value as computed: an empty asm statement the compiler cannot look
// through.  Without it the FMA that produced a value can be fused with its
// conversion to fp16 / bf16 (v_fma_mix*), which rounds the exact result once
// to the half type instead of rounding the fp32 result, and the last bit of
// a half output then depends on how a kernel was scheduled.
__device__ __forceinline__ float settle(float v) {
    __asm__ volatile("" : "+v"(v));
    return v;
}

struct Half16Base {
    static constexpr int bytes = 2;
    typedef uint16_t raw_t;
    __device__ __forceinline__ static uint16_t load_raw(rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    }
    __device__ __forceinline__ static void store_raw(uint16_t v, rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, (int)off, 0, kStoreNT);
    }
};

struct F16 : Half16Base {
    __device__ __forceinline__ static float from_raw(uint16_t v) {
        return (float)__builtin_bit_cast(_Float16, v);
    }
    __device__ __forceinline__ static float load(rsrc_t r, uint32_t off) {
        return from_raw(load_raw(r, off));
    }
    // round to nearest even (v_cvt_f16_f32)
    __device__ __forceinline__ static void store(float v, rsrc_t r, uint32_t off) {
        store_raw(__builtin_bit_cast(uint16_t, (_Float16)settle(v)), r, off);
    }
};

struct BF16 : Half16Base {
    __device__ __forceinline__ static float from_raw(uint16_t v) {
        return __builtin_bit_cast(float, (uint32_t)v << 16);
    }
    __device__ __forceinline__ static float load(rsrc_t r, uint32_t off) {
        return from_raw(load_raw(r, off));
    }
    // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    __device__ __forceinline__ static void store(float v, rsrc_t r, uint32_t off) {
        store_raw(__builtin_bit_cast(uint16_t, (__bf16)settle(v)), r, off);
    }
};

// ------------------------------------------------------- integer division

// Division of non-negative 31-bit integers by a divisor fixed at launch
// (Granlund & Montgomery): q = (umulhi(n, m) + n) >> s.
struct FastDiv {
    uint32_t d, m, s;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.m) + n) >> f.s;
}

// ------------------------------------------------------------ coordinates

// Position of sample i of m evenly spaced samples over [-1, 1]
// (AffineGrid page, Summary; align_corners as described there), in the
// computation type F of the grid (float, or double for a double theta).
template <typename F = float>
__device__ __forceinline__ F base_position(int i, int m, int align_corners) {
    if (align_corners) {
        if (m == 1) return F(0);
        return (F)(2 * i) / (F)(m - 1) - F(1);
    }
    return (F)(2 * i + 1) / (F)m - F(1);
}

// The coordinate steps below are written once for the grid's coordinate
// type F: float (fp32, fp16 and bf16 grids) or double (double grids).
template <typename F>
__device__ __forceinline__ F floor_t(F v) {
    if constexpr (sizeof(F) == 4) return floorf(v);
    else return floor(v);
}
template <typename F>
__device__ __forceinline__ F fabs_t(F v) {
    if constexpr (sizeof(F) == 4) return fabsf(v);
    else return fabs(v);
}

// Normalised location -> pixel coordinate along an axis of n pixels
// (GridSample page, Attributes: align_corners).  (g+1)/2 is computed as
// (g+1)*0.5, which rounds identically.
template <typename F>
__device__ __forceinline__ F unnormalize(F g, int n, int align_corners) {
    if (align_corners) {
        F u = (g + F(1)) * F(0.5);
        return u * (F)(n - 1);
    }
    F v = (g + F(1)) * (F)n;
    return (v - F(1)) * F(0.5);
}

template <typename F>
__device__ __forceinline__ F clampf(F v, F lo, F hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

// Fold p into [lo, hi] by repeated reflection (GridSample page, padding_mode).
template <typename F>
__device__ __forceinline__ F reflect(F p, F lo, F hi) {
    F span = hi - lo;
    if (span <= F(0)) return F(0);
    F d = fabs_t(p - lo);
    F f = floor_t(d / span);
    F fs = f * span;
    F e = d - fs;
    F half = floor_t(f * F(0.5));
    bool odd = (f - F(2) * half) != F(0);
    return odd ? hi - e : lo + e;
}

template <typename F>
__device__ __forceinline__ void reflect_bounds(int n, int align_corners, F &lo, F &hi) {
    if (align_corners) {
        lo = F(0);
        hi = (F)(n - 1);
    } else {
        lo = F(-0.5);
        hi = (F)n - F(0.5);
    }
}

// Location padding of nearest and linear modes.
template <int PAD, typename F>
__device__ __forceinline__ F pad_coordinate(F p, int n, int align_corners) {
    if (PAD == PAD_BORDER) return clampf(p, F(0), (F)(n - 1));
    if (PAD == PAD_REFLECTION) {
        F lo, hi;
        reflect_bounds(n, align_corners, lo, hi);
        return clampf(reflect(p, lo, hi), F(0), (F)(n - 1));
    }
    return p;
}

// Keys' cubic convolution kernel for the four taps of fractional offset t:
// w[0..3] weight pixels floor(p) - 1 .. floor(p) + 2.
__device__ __forceinline__ void cubic_weights(float t, float w[4]) {
    const float a = kCubicA;
    float x0 = t + 1.0f;   // in [1, 2)
    float x1 = t;          // in [0, 1)
    float x2 = 1.0f - t;   // in (0, 1]
    float x3 = 2.0f - t;   // in (1, 2]
    w[0] = fmaf(fmaf(fmaf(a, x0, -5.0f * a), x0, 8.0f * a), x0, -4.0f * a);
    w[1] = fmaf(fmaf(a + 2.0f, x1, -(a + 3.0f)), x1 * x1, 1.0f);
    w[2] = fmaf(fmaf(a + 2.0f, x2, -(a + 3.0f)), x2 * x2, 1.0f);
    w[3] = fmaf(fmaf(fmaf(a, x3, -5.0f * a), x3, 8.0f * a), x3, -4.0f * a);
}

// Tap index of cubic mode after per-tap padding (border / reflection), the
// reflection folded in the coordinate type F.
template <int PAD, typename F = float>
__device__ __forceinline__ int pad_tap(int i, int n, int align_corners) {
    if (PAD == PAD_BORDER) return i < 0 ? 0 : (i > n - 1 ? n - 1 : i);
    F lo, hi;
    reflect_bounds(n, align_corners, lo, hi);
    return (int)clampf(reflect((F)i, lo, hi), F(0), (F)(n - 1));
}

// ----------------------------------------------------------- block order

// Workgroups are handed to the 8 XCDs round-robin by launch index.  Remap so
// that each XCD receives one contiguous run of logical tiles: neighbouring
// tiles then share their halo rows in that XCD's L2.  The launch holds
// 8 * ceil(n / 8) blocks; the surplus ones exit.
__device__ __forceinline__ int xcd_logical_block(int nblocks) {
    int per = (nblocks + 7) >> 3;
    int b = blockIdx.x;
    return (b & 7) * per + (b >> 3);
}

// As above, but the runs are kRun logical blocks long and are dealt to the
// XCDs round-robin, so every XCD works on every part of the launch at once
// (the sampler measured faster this way than with one run per XCD, whose
// co-resident blocks then all read a single image).  Launch 8*kRun*ceil(n/(8*kRun))
// blocks; the surplus ones exit.
constexpr int kRun = 16;
__device__ __forceinline__ int xcd_logical_block_runs(int nblocks) {
    (void)nblocks;
    const int b = blockIdx.x;
    const int grp = b / (8 * kRun), r = b - grp * (8 * kRun);
    return grp * (8 * kRun) + (r & 7) * kRun + (r >> 3);
}

// As xcd_logical_block_runs with runs of `run` logical blocks (the launch
// holds a multiple of 8 * run blocks).
__device__ __forceinline__ int xcd_logical_block_run_of(int run) {
    const int b = blockIdx.x;
    const int grp = b / (8 * run), r = b - grp * (8 * run);
    return grp * (8 * run) + (r & 7) * run + (r >> 3);
}


// ------------------------------------------------------- block reduction

// DPP lane moves within a row of 16 lanes (no LDS round trip, unlike a
// shuffle): quad permutations, half-row and row mirrors, shift right by n
// (lanes with no source keep `old`).
template <int CTRL>
__device__ __forceinline__ int dpp_move(int old, int v) {
    return __builtin_amdgcn_update_dpp(old, v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppQuad1032 = 0xb1, kDppQuad2301 = 0x4e, kDppHalfMirror = 0x141,
              kDppMirror = 0x140, kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114,
              kDppShr8 = 0x118;

// Minimum over the wave, uniform (every lane and an SGPR hold it).
__device__ __forceinline__ int wave_min(int v) {
    v = min(v, dpp_move<kDppQuad1032>(v, v));
    v = min(v, dpp_move<kDppQuad2301>(v, v));
    v = min(v, dpp_move<kDppHalfMirror>(v, v));
    v = min(v, dpp_move<kDppMirror>(v, v));
    const int a = min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16));
    const int b = min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48));
    return min(a, b);
}

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += dpp_move<kDppShr1>(0, v);
    v += dpp_move<kDppShr2>(0, v);
    v += dpp_move<kDppShr4>(0, v);
    v += dpp_move<kDppShr8>(0, v);
    // add the totals of the rows before this lane's row
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

template <int NV>
__device__ __forceinline__ void block_min(int (&v)[NV], int (*red)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = wave_min(v[i]);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int i = 0; i < NV; ++i) red[wave][i] = v[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int m = red[0][i];
#pragma unroll
        for (int wv = 1; wv < kBlock / 64; ++wv) m = min(m, red[wv][i]);
        v[i] = __builtin_amdgcn_readfirstlane(m);
    }
}

// q = f / d for 0 <= f < 2^16, 1 <= d: fp32 estimate, then one correction.
__device__ __forceinline__ int div_small(int f, int d, float inv_d) {
    int q = (int)((float)f * inv_d);
    int r = f - q * d;
    q += (r < 0) ? -1 : (r >= d ? 1 : 0);
    return q;
}

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

// Store the Q outputs of one lane for one channel: one vector store of
// Q elements when the row layout allows it, else Q stores.
template <typename T, int Q>
__device__ __forceinline__ void store_outputs(const typename T::raw_t (&v)[Q], rsrc_t yr,
                                              const uint32_t (&yoff)[Q], bool vec) {
    if constexpr (Q == 2) {
        if (vec) {
            if constexpr (T::bytes == 4) {
                u32x2 pk = {(uint32_t)v[0], (uint32_t)v[1]};
                __builtin_amdgcn_raw_buffer_store_b64(pk, yr, (int)yoff[0], 0, kStoreNT);
            } else {
                __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v[0] | ((uint32_t)v[1] << 16), yr,
                                                      (int)yoff[0], 0, kStoreNT);
            }
            return;
        }
    }
    if constexpr (Q == 4) {
        if (vec) {
            if constexpr (T::bytes == 4) {
                u32x4 pk = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
                __builtin_amdgcn_raw_buffer_store_b128(pk, yr, (int)yoff[0], 0, kStoreNT);
            } else {
                u32x2 pk = {(uint32_t)v[0] | ((uint32_t)v[1] << 16),
                            (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
                __builtin_amdgcn_raw_buffer_store_b64(pk, yr, (int)yoff[0], 0, kStoreNT);
            }
            return;
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) T::store_raw(v[q], yr, yoff[q]);
}

template <typename T>
__device__ __forceinline__ typename T::raw_t to_raw(float v);
template <>
__device__ __forceinline__ uint32_t to_raw<F32>(float v) { return __builtin_bit_cast(uint32_t, v); }
template <>
__device__ __forceinline__ uint16_t to_raw<F16>(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)settle(v));
}
template <>
__device__ __forceinline__ uint16_t to_raw<BF16>(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)settle(v));
}

// ------------------------------------------------------------------ taps

template <int MODE>
struct AxisK {
    static constexpr int K = MODE == MODE_NEAREST ? 1 : (MODE == MODE_LINEAR ? 2 : 4);
};

template <int K>
struct AxisTaps {
    int idx[K];
    bool ok[K];
    float w[K];
};

// Taps of one axis of n pixels for pixel coordinate pc (finite, |pc| <= 2^24).
template <int MODE, int PAD>
__device__ __forceinline__ void axis_taps(float pc, int n, int ac, AxisTaps<AxisK<MODE>::K> &a) {
    if constexpr (MODE == MODE_NEAREST) {
        float q = pad_coordinate<PAD>(pc, n, ac);
        int i = (int)rintf(q);
        a.idx[0] = i;
        a.ok[0] = (uint32_t)i < (uint32_t)n;
        a.w[0] = 1.0f;
    } else if constexpr (MODE == MODE_LINEAR) {
        float q = pad_coordinate<PAD>(pc, n, ac);
        float fl = floorf(q);
        int i0 = (int)fl;
        float t = q - fl;
        a.idx[0] = i0;
        a.idx[1] = i0 + 1;
        a.ok[0] = (uint32_t)i0 < (uint32_t)n;
        a.ok[1] = (uint32_t)(i0 + 1) < (uint32_t)n;
        a.w[0] = 1.0f - t;
        a.w[1] = t;
    } else {
        // cubic: the location is not padded; each tap is
        float fl = floorf(pc);
        int i0 = (int)fl;
        cubic_weights(pc - fl, a.w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int i = i0 - 1 + j;
            if constexpr (PAD == PAD_ZEROS) {
                a.idx[j] = i;
                a.ok[j] = (uint32_t)i < (uint32_t)n;
            } else {
                a.idx[j] = pad_tap<PAD>(i, n, ac);
                a.ok[j] = true;
            }
        }
    }
}

// ---------------------------------------------------- gather path choice

// Tiles the 2D gather path probes; its verdicts (1 = the tile's locations are
// scattered beyond what LDS staging holds) are kProbes words in device memory.
constexpr int kProbes = 64;

// True when at least half of the probed tiles are scattered.  Uniform across
// the block (the 64 words load through the scalar cache).
__device__ __forceinline__ bool gather_chosen(const int *verdicts) {
    int count = 0;
#pragma unroll
    for (int i = 0; i < kProbes; ++i) count += verdicts[i];
    return count * 2 >= kProbes;
}

}  // namespace gs
