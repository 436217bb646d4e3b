// gs_nd.hip -- GridSample of any rank (1 to 6 spatial axes) and any numeric
// element type, for gfx950.
//
// The GridSample page defines the operator for X of rank r+2 in general
// (Summary), for X of every numeric type -- an integer input is interpolated
// in floating point and only the result is converted back to the integer
// type (Outputs) -- and for fp16,
// fp32 and double grids (Type Constraints; bfloat16 from version 22).  The
// tuned 2D/3D kernels cover fp32 / fp16 / bf16 X with fp32 grids; this kernel
// covers the rest.
//
// One lane owns one output location of one image and loops over a group of
// channels.  Per axis it computes the location's taps once: the coordinate
// steps in the grid's coordinate type (fp32 for fp32, fp16 and bf16 grids,
// double for double grids), the weights in double.  Each output is the sum
// over the product of the per-axis taps, innermost axis fastest, of
// (product of the axis weights, outermost axis first) * X[tap], every product
// and sum rounded in double one operation at a time: the order of the plain
// definition, so the integer cast lands on the same side of every integer as
// that definition does.  X is gathered straight through buffer loads; a tap
// outside the image (zeros padding) is skipped.
#include "gs_device.hpp"
#include "gs_launch.hpp"

#include <stdint.h>

#include <limits>

namespace gs {

// ------------------------------------------------------------ element types

struct NdF32 {
    static constexpr int bytes = 4;
    __device__ static double load(rsrc_t r, uint32_t o) {
        return (double)__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)o, 0, 0));
    }
    __device__ static void store(double v, rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, (float)v), r, (int)o, 0,
                                              kStoreNT);
    }
};

struct NdF16 {
    static constexpr int bytes = 2;
    __device__ static double load(rsrc_t r, uint32_t o) {
        const uint16_t b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0);
        return (double)(float)__builtin_bit_cast(_Float16, b);
    }
    // double -> fp32 -> fp16, each step to nearest even
    __device__ static void store(double v, rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)(float)v), r,
                                              (int)o, 0, kStoreNT);
    }
};

struct NdBF16 {
    static constexpr int bytes = 2;
    __device__ static double load(rsrc_t r, uint32_t o) {
        const uint32_t b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0);
        return (double)__builtin_bit_cast(float, b << 16);
    }
    __device__ static void store(double v, rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)(float)v), r,
                                              (int)o, 0, kStoreNT);
    }
};

struct NdF64 {
    static constexpr int bytes = 8;
    __device__ static double load(rsrc_t r, uint32_t o) {
        return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, 0));
    }
    __device__ static void store(double v, rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)o, 0, kStoreNT);
    }
};

// The final cast of integer inputs (GridSample page, Outputs): truncation
// toward zero, saturated to the range of I; NaN becomes 0.
template <typename I>
__device__ __forceinline__ I cast_to_int(double v) {
    constexpr I kMin = std::numeric_limits<I>::min();
    constexpr I kMax = std::numeric_limits<I>::max();
    if (v != v) return (I)0;
    const double tv = trunc(v);
    if (tv <= (double)kMin) return kMin;
    if (tv >= (double)kMax) return kMax;
    return (I)tv;
}

// Integer element I: loaded exactly into double (64-bit values beyond 2^53
// round to nearest), stored through cast_to_int.
template <typename I>
struct NdInt {
    static constexpr int bytes = sizeof(I);
    __device__ static double load(rsrc_t r, uint32_t o) {
        if constexpr (sizeof(I) == 1) {
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(r, (int)o, 0, 0);
            return (double)(I)(uint8_t)b;
        } else if constexpr (sizeof(I) == 2) {
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0);
            return (double)(I)(uint16_t)b;
        } else if constexpr (sizeof(I) == 4) {
            return (double)(I)__builtin_amdgcn_raw_buffer_load_b32(r, (int)o, 0, 0);
        } else {
            return (double)__builtin_bit_cast(I, __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, 0));
        }
    }
    __device__ static void store(double v, rsrc_t r, uint32_t o) {
        const I c = cast_to_int<I>(v);
        if constexpr (sizeof(I) == 1) {
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)c, r, (int)o, 0, kStoreNT);
        } else if constexpr (sizeof(I) == 2) {
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)c, r, (int)o, 0, kStoreNT);
        } else if constexpr (sizeof(I) == 4) {
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)c, r, (int)o, 0, kStoreNT);
        } else {
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, c), r, (int)o, 0,
                                                  kStoreNT);
        }
    }
};

// ------------------------------------------------------------- coordinates

// taps per axis: nearest 1, linear 2, cubic 4
template <int MODE>
struct NdK {
    static constexpr int K = MODE == MODE_NEAREST ? 1 : (MODE == MODE_LINEAR ? 2 : 4);
};

// Cubic convolution kernel of Keys (1981, Eq. 4) with a = -0.75, in double,
// each operation rounded on its own in the order written.
__device__ __forceinline__ double keys_d(double s) {
    const double a = (double)kCubicA;
    const double x = fabs(s);
    if (x <= 1.0) return ((a + 2.0) * x - (a + 3.0)) * x * x + 1.0;
    if (x < 2.0) return ((a * x - 5.0 * a) * x + 8.0 * a) * x - 4.0 * a;
    return 0.0;
}

template <typename F>
__device__ __forceinline__ F rint_t(F v) {
    if constexpr (sizeof(F) == 4) return rintf(v);
    else return rint(v);
}

template <typename F>
__device__ __forceinline__ F pad_location(F p, int n, int padding, int ac) {
    switch (padding) {
    case PAD_BORDER: return pad_coordinate<PAD_BORDER>(p, n, ac);
    case PAD_REFLECTION: return pad_coordinate<PAD_REFLECTION>(p, n, ac);
    default: return p;
    }
}

// Taps of one axis of n pixels for pixel coordinate pc (finite, clamped to
// +-2^24): indices, validity and double weights (GridSample page,
// Attributes mode and padding_mode).
template <int MODE, typename F, int K>
__device__ __forceinline__ void nd_axis_taps(F pc, int n, int padding, int ac, int (&idx)[K],
                                             bool (&ok)[K], double (&w)[K]) {
    if constexpr (MODE == MODE_NEAREST) {
        const F q = pad_location(pc, n, padding, ac);
        const int i = (int)rint_t(q);  // ties to even
        idx[0] = i;
        ok[0] = i >= 0 && i < n;
        w[0] = 1.0;
    } else if constexpr (MODE == MODE_LINEAR) {
        const F q = pad_location(pc, n, padding, ac);
        const F fl = floor_t(q);
        const double frac = (double)q - (double)fl;  // exact
        const int i0 = (int)fl;
        idx[0] = i0;
        idx[1] = i0 + 1;
        w[0] = 1.0 - frac;
        w[1] = frac;
#pragma unroll
        for (int j = 0; j < 2; ++j) ok[j] = idx[j] >= 0 && idx[j] < n;
    } else {
        // the location itself is not padded; each of the four taps is
        const F fl = floor_t(pc);
        const double frac = (double)pc - (double)fl;
        const int i0 = (int)fl;
        w[0] = keys_d(frac + 1.0);
        w[1] = keys_d(frac);
        w[2] = keys_d(1.0 - frac);
        w[3] = keys_d(2.0 - frac);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i = i0 - 1 + j;
            if (padding == PAD_ZEROS) {
                idx[j] = i;
                ok[j] = i >= 0 && i < n;
            } else if (padding == PAD_BORDER) {
                idx[j] = pad_tap<PAD_BORDER, F>(i, n, ac);
                ok[j] = true;
            } else {
                idx[j] = pad_tap<PAD_REFLECTION, F>(i, n, ac);
                ok[j] = true;
            }
        }
    }
}

// One component of the location vector (grid element `at`), in the
// coordinate type F.
template <typename F>
__device__ __forceinline__ F grid_component(const void *grid, int grid_dtype, size_t at) {
    if constexpr (sizeof(F) == 8) {
        return ((const double *)grid)[at];
    } else {
        if (grid_dtype == 1) return (float)((const _Float16 *)grid)[at];
        if (grid_dtype == 2)
            return __builtin_bit_cast(float, (uint32_t)((const uint16_t *)grid)[at] << 16);
        return ((const float *)grid)[at];
    }
}

// element s of a per-axis array of K entries, s in [0, K): selects, no
// dynamic register indexing
template <int K, typename V>
__device__ __forceinline__ V pick(const V (&a)[K], int s) {
    if constexpr (K == 1) return a[0];
    else if constexpr (K == 2) return s ? a[1] : a[0];
    else return (s & 2) ? ((s & 1) ? a[3] : a[2]) : ((s & 1) ? a[1] : a[0]);
}

// ------------------------------------------------------------------ kernel

// A lane's location slot past the end of the output (its stores are dropped).
constexpr uint32_t kNoLocation = 0xFFFFFFFFu;

// The channel loop of one lane for element type T, over the lane's L output
// locations yo (kNoLocation: none).  Tap t
// selects, on axis a, digit a of t in base K (the innermost axis is the least
// significant digit, so it runs fastest).
template <int R, int MODE, typename T, int L>
__device__ __forceinline__ void nd_channels(const NdParams &p, int n, int cbeg, int cend,
                                            const uint32_t (&yo)[L],
                                            const int (&idx)[L][R][NdK<MODE>::K],
                                            const bool (&ok)[L][R][NdK<MODE>::K],
                                            const double (&w)[L][R][NdK<MODE>::K]) {
    constexpr int K = NdK<MODE>::K;
    constexpr int LK = K == 1 ? 0 : (K == 2 ? 1 : 2);
    constexpr int TAPS = 1 << (LK * R);
    const uint32_t ip = p.in_plane_bytes, op = p.out_plane_bytes;
    const char *xn = (const char *)p.X + ((size_t)n * p.C) * ip;
    char *yn = (char *)p.Y + ((size_t)n * p.C) * op;
    uint32_t yb[L];  // byte offsets of the outputs in a plane
#pragma unroll
    for (int l = 0; l < L; ++l) yb[l] = yo[l] == kNoLocation ? GS_OOB : yo[l] * (uint32_t)T::bytes;
    // weight, validity and offset of tap t of location l
    auto tap_of = [&](int l, int t, double &ww, bool &valid, uint32_t &off) {
        ww = 1.0;
        valid = true;
        off = 0;
#pragma unroll
        for (int a = 0; a < R; ++a) {
            const int s = (t >> (LK * (R - 1 - a))) & (K - 1);
            ww = ww * pick(w[l][a], s);
            valid = valid && pick(ok[l][a], s);
            off = off * (uint32_t)p.in_ext[a] + (uint32_t)pick(idx[l][a], s);
        }
    };
    int c = cbeg;
    if constexpr (TAPS <= 8) {
        // With few taps the taps' weights and offsets are kept, and UC
        // channels at a time have every load issued before the first sum:
        // a lane keeps 8 to 16 loads in flight (one channel of 2 taps left
        // it waiting on 2; 4 channels of 4 taps were slower than 2).  Each
        // channel's sum is the same, term by term, as the loop below.
        constexpr int UC = L > 1 ? (8 / (TAPS * L) > 1 ? 8 / (TAPS * L) : 1)
                                 : (TAPS == 8 ? 2 : 8 / TAPS);
        double tw[L][TAPS];
        bool tv[L][TAPS];
        uint32_t to[L][TAPS];
#pragma unroll
        for (int l = 0; l < L; ++l)
#pragma unroll
            for (int t = 0; t < TAPS; ++t) {
                uint32_t off;
                tap_of(l, t, tw[l][t], tv[l][t], off);
                to[l][t] = tv[l][t] ? off * (uint32_t)T::bytes : GS_OOB;
            }
        auto channels = [&](auto ucc) {
            constexpr int U = decltype(ucc)::value;
            double xv[U][L][TAPS];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const rsrc_t r = make_rsrc(xn + (size_t)(c + u) * ip, ip);
#pragma unroll
                for (int l = 0; l < L; ++l)
#pragma unroll
                    for (int t = 0; t < TAPS; ++t) xv[u][l][t] = T::load(r, to[l][t]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const rsrc_t yr = make_rsrc(yn + (size_t)(c + u) * op, op);
#pragma unroll
                for (int l = 0; l < L; ++l) {
                    double acc = 0.0;
#pragma unroll
                    for (int t = 0; t < TAPS; ++t)
                        acc = tv[l][t] ? acc + tw[l][t] * xv[u][l][t] : acc;
                    T::store(acc, yr, yb[l]);
                }
            }
        };
        if constexpr (UC > 1)
            for (; c + UC <= cend; c += UC) channels(std::integral_constant<int, UC>());
        for (; c < cend; ++c) channels(std::integral_constant<int, 1>());
    } else {
        static_assert(L == 1, "many taps: one location per lane");
        for (; c < cend; ++c) {
            const rsrc_t r = make_rsrc(xn + (size_t)c * ip, ip);
            double acc = 0.0;
            auto tap = [&](int t) {
                double ww;
                bool valid;
                uint32_t off;
                tap_of(0, t, ww, valid, off);
                const double x = T::load(r, valid ? off * (uint32_t)T::bytes : GS_OOB);
                acc = valid ? acc + ww * x : acc;
            };
            if constexpr (TAPS <= 64) {
#pragma unroll
                for (int t = 0; t < TAPS; ++t) tap(t);
            } else {
                for (int t = 0; t < TAPS; ++t) tap(t);
            }
            T::store(acc, make_rsrc(yn + (size_t)c * op, op), yb[0]);
        }
    }
}

// L output locations per lane, 256 apart (each load and store instruction of
// a wave stays contiguous): the per-wave set-up and the buffer resources of
// each channel serve L times the outputs.
template <int R, int MODE, typename F, int L>
__global__ __launch_bounds__(kBlock) void grid_sample_nd_kernel(NdParams p) {
    constexpr int K = NdK<MODE>::K;
    const int lb = xcd_logical_block_runs(p.nblocks);
    if (lb >= p.nblocks) return;
    const int tile = lb % p.tiles;
    const int ncg = lb / p.tiles;
    const int cg = ncg % p.cgroups;
    const int n = ncg / p.cgroups;
    const uint32_t o0 = (uint32_t)tile * (kBlock * L) + threadIdx.x;
    if (o0 >= p.out_count) return;  // no barrier in this kernel

    int idx[L][R][K];
    bool ok[L][R][K];
    double w[L][R][K];
    uint32_t yo[L];
#pragma unroll
    for (int l = 0; l < L; ++l) {
        const uint32_t ol = o0 + (uint32_t)(l * kBlock);
        const bool in = ol < p.out_count;
        const uint32_t o = in ? ol : p.out_count - 1;   // a valid grid element
        yo[l] = in ? o : kNoLocation;
        bool live = true;
#pragma unroll
        for (int a = 0; a < R; ++a) {
            // component k of the location vector addresses axis R-1-k
            const F g = grid_component<F>(p.grid, p.grid_dtype,
                                          ((size_t)n * p.out_count + o) * R + (R - 1 - a));
            const F u = unnormalize(g, p.in_ext[a], p.align_corners);
            const bool fin = __builtin_isfinite(u);
            live = live && fin;
            const F pc = fin ? clampf(u, F(-kCoordLimit), F(kCoordLimit)) : F(0);
            nd_axis_taps<MODE, F, K>(pc, p.in_ext[a], p.padding, p.align_corners, idx[l][a],
                                     ok[l][a], w[l][a]);
        }
        // a location that is not finite on some axis reads nothing (output 0)
#pragma unroll
        for (int a = 0; a < R; ++a)
#pragma unroll
            for (int j = 0; j < K; ++j) ok[l][a][j] = ok[l][a][j] && live;
    }

    const int cbeg = cg * p.cpg;
    const int cend = min(p.C, cbeg + p.cpg);
    switch (p.x_dtype) {
    case 0: nd_channels<R, MODE, NdF32, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 1: nd_channels<R, MODE, NdF16, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 2: nd_channels<R, MODE, NdBF16, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 3: nd_channels<R, MODE, NdF64, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 4: nd_channels<R, MODE, NdInt<int8_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 5: nd_channels<R, MODE, NdInt<uint8_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 6: nd_channels<R, MODE, NdInt<int16_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 7: nd_channels<R, MODE, NdInt<uint16_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 8: nd_channels<R, MODE, NdInt<int32_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 9: nd_channels<R, MODE, NdInt<uint32_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    case 10: nd_channels<R, MODE, NdInt<int64_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    default: nd_channels<R, MODE, NdInt<uint64_t>, L>(p, n, cbeg, cend, yo, idx, ok, w); break;
    }
}

// --------------------------------------------------------------- dispatch

template <int R, int MODE>
static int nd_launch(const NdParams &p, bool double_grid, hipStream_t s) {
    constexpr int L = nd_locs_per_lane(R, MODE);
    const dim3 grid(8 * kRun * ((p.nblocks + 8 * kRun - 1) / (8 * kRun)));
    if (double_grid)
        hipLaunchKernelGGL((grid_sample_nd_kernel<R, MODE, double, L>), grid, dim3(kBlock), 0, s, p);
    else
        hipLaunchKernelGGL((grid_sample_nd_kernel<R, MODE, float, L>), grid, dim3(kBlock), 0, s, p);
    return (int)hipGetLastError();
}

template <int R>
static int nd_by_mode(const NdParams &p, int mode, bool double_grid, hipStream_t s) {
    switch (mode) {
    case MODE_LINEAR: return nd_launch<R, MODE_LINEAR>(p, double_grid, s);
    case MODE_NEAREST: return nd_launch<R, MODE_NEAREST>(p, double_grid, s);
    default: return nd_launch<R, MODE_CUBIC>(p, double_grid, s);
    }
}

int launch_grid_sample_nd(const NdParams &p, int rank, int mode, bool double_grid,
                          hipStream_t stream) {
    switch (rank) {
    case 1: return nd_by_mode<1>(p, mode, double_grid, stream);
    case 2: return nd_by_mode<2>(p, mode, double_grid, stream);
    case 3: return nd_by_mode<3>(p, mode, double_grid, stream);
    case 4: return nd_by_mode<4>(p, mode, double_grid, stream);
    case 5: return nd_by_mode<5>(p, mode, double_grid, stream);
    default: return nd_by_mode<6>(p, mode, double_grid, stream);
    }
}

}  // namespace gs
