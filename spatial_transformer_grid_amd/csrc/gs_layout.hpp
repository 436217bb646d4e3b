// gs_layout.hpp -- channels-last copies of X for the gathering kernels.
//
// A sampler that gathers at scattered locations reads every channel of a
// pixel: in the (N, C, spatial) layout the pages give, those are C loads
// from C planes; in a channels-last copy they are a few 16-byte loads of one
// contiguous run.  These device functions make that copy, one 64 x 64
// (channel x pixel) tile per 256-thread block, through LDS, in slices of CS
// channels: Xt (N, C / CS, S, CS), element (n, c, s) at
// ((n * C / CS + c / CS) * S + s) * CS + c % CS.  CS = C is plain
// (N, S, C); a smaller CS keeps one slice plane small enough for L2.
#pragma once

#include "gs_device.hpp"

#include <stdint.h>

namespace gs {

// Offset of element (c, s) of one image of Xt in slices of CS channels.
__device__ __forceinline__ size_t sliced_index(int c, int s, int S, int CS) {
    const int sl = c / CS;
    return ((size_t)sl * S + s) * CS + (c - sl * CS);
}

// X (N, C, S) -> Xt, S = H * W: 64 x 64 tiles through LDS.
template <typename raw_t>
__device__ __forceinline__ void to_channels_last_scalar(const raw_t *__restrict__ X,
                                                        raw_t *__restrict__ Xt, int C, int S,
                                                        int c_tiles, int s_tiles, int b, int CS) {
    __shared__ raw_t tile[64][65];
    const int st = b % s_tiles;
    const int ct = (b / s_tiles) % c_tiles;
    const int n = b / (s_tiles * c_tiles);
    const int t = threadIdx.x, col = t & 63, r4 = t >> 6;
    const raw_t *src = X + (size_t)n * C * S;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int c = ct * 64 + r4 + 4 * i, sp = st * 64 + col;
        tile[r4 + 4 * i][col] = (c < C && sp < S) ? src[(size_t)c * S + sp] : (raw_t)0;
    }
    __syncthreads();
    raw_t *dst = Xt + (size_t)n * S * C;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int sp = st * 64 + r4 + 4 * i, c = ct * 64 + col;
        if (sp < S && c < C) dst[sliced_index(c, sp, S, CS)] = tile[col][r4 + 4 * i];
    }
}

// As to_channels_last_scalar with 16-byte accesses on both sides: VW = 16 /
// sizeof(raw_t) spatial elements per load, VW channels per store.  Needs S,
// C and CS to be multiples of VW (and 16-byte aligned X, Xt).
template <typename raw_t>
__device__ __forceinline__ void to_channels_last_tile(const raw_t *__restrict__ X,
                                                      raw_t *__restrict__ Xt, int C, int S,
                                                      int c_tiles, int s_tiles, int b, int CS) {
    constexpr int VW = 16 / sizeof(raw_t);
    constexpr int P = 64 + 2;                       // LDS row pitch (elements)
    __shared__ raw_t tile[64 * P];                  // [c][s]
    const int st = b % s_tiles;
    const int ct = (b / s_tiles) % c_tiles;
    const int n = b / (s_tiles * c_tiles);
    const int t = threadIdx.x;
    const raw_t *src = X + (size_t)n * C * S;
    constexpr int PER = 64 / VW;                    // vectors per tile row
#pragma unroll
    for (int i = 0; i < 64 * PER / kBlock; ++i) {
        const int idx = t + i * kBlock;
        const int cl = idx / PER, sv = idx - (idx / PER) * PER;
        const int c = ct * 64 + cl, sp = st * 64 + sv * VW;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c < C && sp < S) v = *(const u32x4 *)(src + (size_t)c * S + sp);
        const raw_t *e = (const raw_t *)&v;
#pragma unroll
        for (int k = 0; k < VW; ++k) tile[cl * P + sv * VW + k] = e[k];
    }
    __syncthreads();
    raw_t *dst = Xt + (size_t)n * S * C;
#pragma unroll
    for (int i = 0; i < 64 * PER / kBlock; ++i) {
        const int idx = t + i * kBlock;
        const int sl = idx / PER, cv = idx - (idx / PER) * PER;
        const int sp = st * 64 + sl, c = ct * 64 + cv * VW;
        u32x4 v;
        raw_t *e = (raw_t *)&v;
#pragma unroll
        for (int k = 0; k < VW; ++k) e[k] = tile[(cv * VW + k) * P + sl];
        if (sp < S && c < C) *(u32x4 *)(dst + sliced_index(c, sp, S, CS)) = v;
    }
}

}  // namespace gs
