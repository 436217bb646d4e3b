// gs_gather.hip -- 2D GridSample for grids that are not locally smooth, on a
// channels-last copy of X, for gfx950.
//
// The tuned sampler stages each tile's input box in LDS; when the grid
// scatters a tile's locations over the whole image (a random flow) the box
// does not fit, and gathering every tap of every channel from the planes of
// X costs one scattered load per (tap, channel).  With a caller-provided
// workspace the library instead:
//
//  1. probes 64 of the sampler's tiles spread over the batch: a tile counts
//     as scattered when the bounding box of its locations (plus the tap
//     window) cannot be staged -- more than 256 input rows or more than the
//     16 KB slot;
//  2. if most probed tiles are scattered, copies X to channels-last slices
//     (N, C / CS, H, W, CS) of SB = 64 bytes of channels (32 when C does not
//     fill 64-byte slices) in the workspace and samples from it: SB / 16
//     lanes share an output location and each loads VW = 16 / sizeof(T)
//     channels of a tap in one 16-byte load.  One slice plane of an image
//     (H * W * SB bytes, 4 MB for 256 x 256) is about an XCD's L2, and the
//     blocks are ordered so that each XCD walks its own (image, slice)
//     planes one after another: the random taps mostly hit L2;
//  3. otherwise the tuned sampler runs as usual.
//
// All four launches (probe, tuned sampler, copy, gather, in that order) are
// enqueued every time; the ones the probe does not choose return at once.
// The copy and the gather go after the sampler: a launch that returns at
// once costs about 1 us there, against about 2.5 us ahead of it, where the
// sampler waits for it.  The per-output arithmetic is the tuned sampler's:
// the same taps and weights (GridSample page: Summary; Attributes
// align_corners, mode, padding_mode), the same fp32 sum in the same tap
// order, one rounding to T at the store.
#include "gs_device.hpp"
#include "gs_launch.hpp"
#include "gs_layout.hpp"

#include <limits.h>
#include <stdint.h>


namespace gs {

// SB bytes of channels per pixel slice (64, or 32 when the channels do not
// fill 64); SB / 16 lanes per output location, kBlock * 16 / SB locations
// per block (one row segment).

// Tile counters of the gather kernel (below): 64 on separate 128-byte lines.
constexpr int kGatherGrab = 2;
constexpr int kCounterStride = 32;  // ints: 128 bytes
constexpr int kCounters = 64;       // 8 sequences x 8 counters

// Block b probes tile (b * tiles) / 64 of the sampler's tiling (geometry in
// p) and writes verdicts[b]: 1 when the tile's locations are scattered.
template <int MODE>
__global__ __launch_bounds__(kBlock) void gather_probe(SampleParams p, int elem_bytes, int *verdicts,
                                                      int *counters) {
    __shared__ int red[kBlock / 64][4];
    // the gather kernel's tile counters (it runs after this launch)
    if (blockIdx.x == 0 && threadIdx.x < kCounters) counters[threadIdx.x * kCounterStride] = 0;
    const int64_t total = (int64_t)p.N * p.tiles_per_n;
    const int64_t tb = ((int64_t)blockIdx.x * total) / kProbes;
    const int n = (int)(tb / p.tiles_per_n);
    const int tile = (int)(tb - (int64_t)n * p.tiles_per_n);
    const int tx = tile % p.tiles_w, ty = tile / p.tiles_w;
    const int count = p.tile_w * p.tile_h;
    int mm[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};  // min x, -max x, min y, -max y
    for (int i = threadIdx.x; i < count; i += kBlock) {
        const int ox = tx * p.tile_w + i % p.tile_w, oy = ty * p.tile_h + i / p.tile_w;
        if (ox >= p.out_w || oy >= p.out_h) continue;
        const float *g = p.grid + ((size_t)n * p.out_count + (uint32_t)oy * (uint32_t)p.out_w + ox) * 2;
        const float u = unnormalize(g[0], p.in_w, p.align_corners);
        const float v = unnormalize(g[1], p.in_h, p.align_corners);
        if (!__builtin_isfinite(u) || !__builtin_isfinite(v)) continue;
        const int xi = (int)floorf(fminf(fmaxf(u, -1.0e6f), 1.0e6f));
        const int yi = (int)floorf(fminf(fmaxf(v, -1.0e6f), 1.0e6f));
        mm[0] = min(mm[0], xi);
        mm[1] = min(mm[1], -xi);
        mm[2] = min(mm[2], yi);
        mm[3] = min(mm[3], -yi);
    }
    block_min<4>(mm, red);
    if (threadIdx.x == 0) {
        int verdict = 0;
        if (mm[0] != INT_MAX) {
            constexpr int K = AxisK<MODE>::K;
            const int64_t sx = (int64_t)(-mm[1]) - mm[0] + K, sy = (int64_t)(-mm[3]) - mm[2] + K;
            verdict = (sy > 256 || sx * sy * elem_bytes > 16384) ? 1 : 0;
        }
        verdicts[blockIdx.x] = verdict;
    }
}

// The copy of X, which the probe may not choose, uses one block per resident
// slot of the device (one round of blocks covers it) and strides over its
// tiles, so that skipping it costs little.

// The sliced channels-last copy, when the probe chose gathering: tiles
// blockIdx.x, + gridDim.x, ...
template <typename raw_t, bool VEC, int SB>
__global__ __launch_bounds__(kBlock) void gather_prepare(const raw_t *__restrict__ X,
                                                        raw_t *__restrict__ Xt, int C, int S,
                                                        int c_tiles, int s_tiles, int tiles,
                                                        const int *verdicts) {
    if (!gather_chosen(verdicts)) return;
    constexpr int CS = SB / sizeof(raw_t);
    for (int b = blockIdx.x; b < tiles; b += gridDim.x) {
        if constexpr (VEC) to_channels_last_tile<raw_t>(X, Xt, C, S, c_tiles, s_tiles, b, CS);
        else to_channels_last_scalar<raw_t>(X, Xt, C, S, c_tiles, s_tiles, b, CS);
        __syncthreads();  // the tile's LDS reads are done before the next tile's writes
    }
}

// VW elements of type T from one 16-byte load, widened.
template <typename T>
__device__ __forceinline__ void widen16(const u32x4 &v, float *x) {
    if constexpr (T::bytes == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t u = v[e];
            x[e] = __builtin_bit_cast(float, u);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = T::from_raw((uint16_t)(v[e] & 0xffffu));
            x[2 * e + 1] = T::from_raw((uint16_t)(v[e] >> 16));
        }
    }
}

// Raw element e of a 16-byte vector of T.
template <typename T>
__device__ __forceinline__ typename T::raw_t raw_at(const u32x4 &v, int e) {
    if constexpr (T::bytes == 4) return v[e];
    else return (uint16_t)(e & 1 ? v[e >> 1] >> 16 : v[e >> 1] & 0xffffu);
}

// One logical block b: with `xcd_pairs`, b % 8 is the XCD whose sequence it
// belongs to, and that XCD's sequence walks (image, slice) pairs x, x + 8,
// x + 16, and so on, all row segments of a pair before the next; otherwise
// the logical blocks walk the pairs in order.  A logical block owns
// kBlock * 16 / SB consecutive output locations of one row; lane t serves
// location t / (SB / 16) and channels VW * (t % (SB / 16)) .. + VW - 1 of
// the slice.
template <int MODE, int PAD, typename T, int SB>
__device__ __forceinline__ void gather_block(const SampleParams &p, const void *Xt, int pairs,
                                             int tiles_per_pair, int xcd_pairs, int b);

// One block per resident slot of the device.  The logical blocks form one
// sequence per XCD (8 with xcd_pairs: blocks b % 8 == x serve XCD x's), or
// one; a sequence is dealt in grabs of kGatherGrab consecutive logical
// blocks by S = min(8, its blocks) counters that take turns (counter j hands
// out grabs j, j + S, j + 2S, ...), so the sequence advances in order, as a
// full grid would be dispatched, and no counter sees more than a few
// blocks' atomics.  Counters sit on separate 128-byte lines; the probe zeroes
// them.  A block asks for its next grab while it works on the current one.
// When the probe keeps the staged sampler, only one round of blocks starts
// and exits.
template <int MODE, int PAD, typename T, int SB>
__global__ __launch_bounds__(kBlock) void grid_sample_gather(SampleParams p, const void *Xt,
                                                            const int *verdicts, int *counters,
                                                            int pairs, int tiles_per_pair,
                                                            int xcd_pairs, int blocks) {
    __shared__ int next[2];
    if (!gather_chosen(verdicts)) return;
    const int nseq = xcd_pairs ? 8 : 1;
    const int x = (int)blockIdx.x % nseq;                 // sequence
    const int rank = (int)blockIdx.x / nseq;              // block's rank among its sequence's
    const int S = min(8, (int)gridDim.x / nseq);          // gridDim.x is a multiple of 8
    const int jc = rank % S;
    const int steps = blocks / nseq;                      // logical blocks per sequence
    int *ctr = counters + (x * 8 + jc) * kCounterStride;
    if (threadIdx.x == 0) next[0] = atomicAdd(ctr, 1);
    __syncthreads();
    int m = __builtin_amdgcn_readfirstlane(next[0]);
    for (int it = 0;; ++it) {
        // (m outside [0, steps) only from a counter the probe did not reset;
        // below steps <= 2^27 the product does not overflow)
        if (m < 0 || m >= steps) break;
        const int k0 = (m * S + jc) * kGatherGrab;
        if (k0 >= steps) break;
        if (threadIdx.x == 0) next[(it + 1) & 1] = atomicAdd(ctr, 1);
#pragma unroll
        for (int i = 0; i < kGatherGrab; ++i) {
            const int k = k0 + i;
            if (k < steps)
                gather_block<MODE, PAD, T, SB>(p, Xt, pairs, tiles_per_pair, xcd_pairs,
                                               xcd_pairs ? k * 8 + x : k);
        }
        __syncthreads();  // the next grab is visible
        m = __builtin_amdgcn_readfirstlane(next[(it + 1) & 1]);
    }
}

template <int MODE, int PAD, typename T, int SB>
__device__ __forceinline__ void gather_block(const SampleParams &p, const void *Xt, int pairs,
                                             int tiles_per_pair, int xcd_pairs, int b) {
    constexpr int K = AxisK<MODE>::K;
    constexpr int TAPS = K * K;
    constexpr int VW = 16 / T::bytes;
    constexpr int CS = SB / T::bytes;
    constexpr int kLanesPerLoc = SB / 16;
    constexpr int kGatherLocs = kBlock / kLanesPerLoc;
    int pair, tile;
    if (xcd_pairs) {
        const int k = b >> 3;
        const int pl = k / tiles_per_pair;
        tile = k - pl * tiles_per_pair;
        pair = pl * 8 + (b & 7);
    } else {
        pair = b / tiles_per_pair;
        tile = b - pair * tiles_per_pair;
    }
    if (pair >= pairs) return;
    const int nsl = p.C / CS;
    const int n = pair / nsl, sl = pair - (pair / nsl) * nsl;
    const int segs = (p.out_w + kGatherLocs - 1) / kGatherLocs;
    const int oy = tile / segs, seg = tile - (tile / segs) * segs;
    const int t = threadIdx.x;
    const int slot = t & (kLanesPerLoc - 1);
    const int ox = seg * kGatherLocs + t / kLanesPerLoc;
    const bool live = ox < p.out_w;
    const int cx = live ? ox : p.out_w - 1;

    // taps and weights of the location (the tuned sampler's steps)
    const float *gp = p.grid + ((size_t)n * p.out_count + (uint32_t)oy * (uint32_t)p.out_w + cx) * 2;
    const float g[2] = {gp[0], gp[1]};
    const int ext[2] = {p.in_w, p.in_h};
    AxisTaps<K> ax[2];
    bool any = true;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float u = unnormalize(g[k], ext[k], p.align_corners);
        const bool fin = __builtin_isfinite(u);
        const float pc = fin ? clampf(u, -kCoordLimit, kCoordLimit) : 0.0f;
        axis_taps<MODE, PAD>(pc, ext[k], p.align_corners, ax[k]);
        bool axis_any = false;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            ax[k].ok[j] = ax[k].ok[j] && fin;
            axis_any = axis_any || ax[k].ok[j];
        }
        any = any && axis_any;
    }
    const uint32_t lane_bytes = (uint32_t)slot * 16;
    uint32_t off[TAPS];
    float w[TAPS];
#pragma unroll
    for (int tap = 0; tap < TAPS; ++tap) {
        const int jx = tap % K, jy = tap / K;
        const bool ok = any && ax[0].ok[jx] && ax[1].ok[jy];
        off[tap] = ok ? (uint32_t)(ax[1].idx[jy] * p.in_w + ax[0].idx[jx]) * SB + lane_bytes
                      : GS_OOB;
        w[tap] = (1.0f * ax[0].w[jx]) * ax[1].w[jy];
    }

    // the slice plane of (n, sl): H * W pixels of SB bytes
    const uint32_t plane_bytes = (uint32_t)p.in_h * (uint32_t)p.in_w * SB;
    const rsrc_t xr = make_rsrc((const char *)Xt + (size_t)pair * plane_bytes, plane_bytes);
    // one resource over the image's C output planes (< 2^31 bytes); a lane's
    // channels are per-lane offsets into it
    const rsrc_t yr = make_rsrc((char *)p.Y + (size_t)n * p.C * p.out_plane_bytes,
                                (uint32_t)p.C * p.out_plane_bytes);
    const uint32_t yoff = ((uint32_t)oy * (uint32_t)p.out_w + ox) * T::bytes;
    const int c = sl * CS + VW * slot;
    // every tap's load is issued before any is used
    u32x4 v[TAPS];
#pragma unroll
    for (int tap = 0; tap < TAPS; ++tap) v[tap] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)off[tap], 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE == MODE_NEAREST) {
#pragma unroll
        for (int e = 0; e < VW; ++e)
            T::store_raw(raw_at<T>(v[0], e), yr, live ? (uint32_t)(c + e) * p.out_plane_bytes + yoff : GS_OOB);
    } else {
        float acc[VW], x[VW];
        widen16<T>(v[0], x);
#pragma unroll
        for (int e = 0; e < VW; ++e) acc[e] = w[0] * x[e];
#pragma unroll
        for (int tap = 1; tap < TAPS; ++tap) {
            widen16<T>(v[tap], x);
#pragma unroll
            for (int e = 0; e < VW; ++e) acc[e] = fmaf(w[tap], x[e], acc[e]);
        }
#pragma unroll
        for (int e = 0; e < VW; ++e)
            T::store(acc[e], yr, live ? (uint32_t)(c + e) * p.out_plane_bytes + yoff : GS_OOB);
    }
}

// --------------------------------------------------------------- dispatch

// Blocks of `kernel` the device holds at once, a multiple of 8 (whole XCD
// rounds), at least 8.
static int resident_blocks(const void *kernel) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess)
        return 2048;
    return max(8, (per_cu * cus) / 8 * 8);
}

template <int MODE, int PAD, typename T, int SB>
static int gather_launch(const SampleParams &p, const GatherParams &g, bool vec_in, int part,
                         hipStream_t s) {
    using raw_t = typename T::raw_t;
    if (part == 0) {
        hipLaunchKernelGGL((gather_probe<MODE>), dim3(kProbes), dim3(kBlock), 0, s, p, (int)T::bytes,
                           g.verdicts, g.counters);
        return (int)hipGetLastError();
    }
    const int S = p.in_h * p.in_w;
    const int c_tiles = (p.C + 63) / 64, s_tiles = (S + 63) / 64;
    const int tiles = p.N * c_tiles * s_tiles;
    // (the occupancy queries run once per kernel: each costs host time that
    // the launches after the sampler would otherwise wait for)
    static const int res_vec = resident_blocks((const void *)gather_prepare<raw_t, true, SB>);
    static const int res_scalar = resident_blocks((const void *)gather_prepare<raw_t, false, SB>);
    const dim3 xg((unsigned)min(tiles, vec_in ? res_vec : res_scalar));
    if (vec_in)
        hipLaunchKernelGGL((gather_prepare<raw_t, true, SB>), xg, dim3(kBlock), 0, s, (const raw_t *)p.X,
                           (raw_t *)g.Xt, p.C, S, c_tiles, s_tiles, tiles, (const int *)g.verdicts);
    else
        hipLaunchKernelGGL((gather_prepare<raw_t, false, SB>), xg, dim3(kBlock), 0, s, (const raw_t *)p.X,
                           (raw_t *)g.Xt, p.C, S, c_tiles, s_tiles, tiles, (const int *)g.verdicts);
    // one round of resident blocks, a multiple of 8 (one counter per XCD)
    static const int res_gather = resident_blocks((const void *)grid_sample_gather<MODE, PAD, T, SB>);
    const int want = (g.gather_blocks + 7) / 8 * 8;
    const dim3 gg((unsigned)min(want, res_gather));
    hipLaunchKernelGGL((grid_sample_gather<MODE, PAD, T, SB>), gg, dim3(kBlock), 0, s, p,
                       (const void *)g.Xt, (const int *)g.verdicts, g.counters, g.pairs,
                       g.tiles_per_pair, g.xcd_pairs, g.gather_blocks);
    return (int)hipGetLastError();
}

template <int MODE, int PAD>
static int gather_by_dtype(const SampleParams &p, const GatherParams &g, int dtype, bool vec_in,
                           int part, hipStream_t s) {
    const bool wide = g.slice_bytes == 64;
    switch (dtype) {
    case 0: return wide ? gather_launch<MODE, PAD, F32, 64>(p, g, vec_in, part, s)
                        : gather_launch<MODE, PAD, F32, 32>(p, g, vec_in, part, s);
    case 1: return wide ? gather_launch<MODE, PAD, F16, 64>(p, g, vec_in, part, s)
                        : gather_launch<MODE, PAD, F16, 32>(p, g, vec_in, part, s);
    default: return wide ? gather_launch<MODE, PAD, BF16, 64>(p, g, vec_in, part, s)
                         : gather_launch<MODE, PAD, BF16, 32>(p, g, vec_in, part, s);
    }
}

template <int MODE>
static int gather_by_padding(const SampleParams &p, const GatherParams &g, int padding, int dtype,
                             bool vec_in, int part, hipStream_t s) {
    switch (padding) {
    case PAD_ZEROS: return gather_by_dtype<MODE, PAD_ZEROS>(p, g, dtype, vec_in, part, s);
    case PAD_BORDER: return gather_by_dtype<MODE, PAD_BORDER>(p, g, dtype, vec_in, part, s);
    default: return gather_by_dtype<MODE, PAD_REFLECTION>(p, g, dtype, vec_in, part, s);
    }
}

int launch_grid_gather(const SampleParams &p, const GatherParams &g, int mode, int padding,
                       int dtype, bool vec_in, int part, hipStream_t s) {
    switch (mode) {
    case MODE_LINEAR: return gather_by_padding<MODE_LINEAR>(p, g, padding, dtype, vec_in, part, s);
    case MODE_NEAREST: return gather_by_padding<MODE_NEAREST>(p, g, padding, dtype, vec_in, part, s);
    default: return gather_by_padding<MODE_CUBIC>(p, g, padding, dtype, vec_in, part, s);
    }
}

}  // namespace gs
