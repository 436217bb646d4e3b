// gs_deform.hip -- DeformConv (version 22) for gfx950.
//
// Y[n, oc, o] = B[oc] + sum over the input channels c of oc's group and the
// kernel positions k of W[oc, c, k] * mask[n, g(c), k, o] *
// linear_sample(X[n, c], regular(o, k) + offset[n, g(c), k, o])
// (DeformConv page: Inputs X, W, offset, B, mask; Summary).  Per image and
// group this is a matrix product of W (oC/group x K, K = C/group * kernel
// size) with the sampled "columns" (K x output positions).
//
// 2-D fp32 / fp16 / bf16 run an implicit GEMM on the matrix cores: a block
// owns TM output channels x 64 output positions of one image and group and
// walks K in chunks of 32.  Per chunk it stages the W tile in LDS and samples
// the 32 x 64 column tile straight into LDS (the columns never reach HBM),
// then each wave multiplies its 32-row blocks with MFMA 32x32 instructions
// (fp32: 32x32x2; fp16 / bf16: 32x32x16, fp32 accumulation).  The sampling of
// a (kernel position, output position) pair is the same for every channel of
// an offset group, so the block first computes, for its 64 positions, every
// such pair's four corner offsets and mask-folded weights into an LDS table.
// Everything else (double data, 1-D and 3-D) runs a direct kernel: one lane
// per output, summed in double.
#include "gs_device.hpp"
#include "gs_launch.hpp"
#include "gs_layout.hpp"

#include <stdint.h>

#include <type_traits>

namespace gs {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

constexpr int DC_TN = 64;   // output positions per block
constexpr int DC_TK = 32;   // K per chunk
constexpr int DC_TABLE = 16;  // kernel positions x offset groups the LDS table holds

// ------------------------------------------------------------ sampling

// Corner element offsets (-1 = outside the image) and weights of the linear
// sample of an H x W plane at (lh, lw), the mask folded into the weights; a
// corner outside the image has weight 0 and is read through the out-of-range
// offset (so it loads 0 and adds exactly 0).
struct Corners {
    int off[4];
    float w[4];
};

__device__ __forceinline__ Corners corners_of(float lh, float lw, float m, int H, int W) {
    Corners c;
    if (!__builtin_isfinite(lh) || !__builtin_isfinite(lw) || fabsf(lh) > kCoordLimit ||
        fabsf(lw) > kCoordLimit) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            c.off[q] = -1;
            c.w[q] = 0.0f;
        }
        return c;
    }
    const float fh0 = floorf(lh), fw0 = floorf(lw);
    const float fh = lh - fh0, fw = lw - fw0;  // exact
    const int h0 = (int)fh0, w0 = (int)fw0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int dy = q >> 1, dx = q & 1;
        const int h = h0 + dy, w = w0 + dx;
        const bool ok = h >= 0 && h < H && w >= 0 && w < W;
        c.off[q] = ok ? h * W + w : -1;
        c.w[q] = ok ? (dy ? fh : 1.0f - fh) * (dx ? fw : 1.0f - fw) * m : 0.0f;
    }
    return c;
}

// Element (index i) of a DeformConv operand of type T, widened to float.
template <typename T>
__device__ __forceinline__ float ld(const void *p, size_t i) {
    if constexpr (T::bytes == 4) return ((const float *)p)[i];
    else return T::from_raw(((const uint16_t *)p)[i]);
}

// Corners of the sample that kernel position `tap` of offset group g takes
// for output position o = (oh, ow) of image n.  No offset or mask is read for
// a position past the end of the plane or an offset group past the last one
// (a conv group may span fewer offset groups than the widest one).
template <typename T>
__device__ __forceinline__ Corners sample_corners(const DeformParams &p, int n, int o, bool o_ok,
                                                  int oh, int ow, int g, int tap) {
    Corners none;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        none.off[q] = -1;
        none.w[q] = 0.0f;
    }
    if (!o_ok || g >= p.og) return none;
    const int npos = p.OH * p.OW, KK = p.KH * p.KW;
    const int i = tap / p.KW, j = tap - (tap / p.KW) * p.KW;
    const size_t oc2 = (size_t)n * p.og * KK * 2 * npos + ((size_t)(g * KK + tap) * 2) * npos + o;
    const float dy = ld<T>(p.offset, oc2), dx = ld<T>(p.offset, oc2 + npos);
    const float m =
        p.mask ? ld<T>(p.mask, (size_t)n * p.og * KK * npos + (size_t)(g * KK + tap) * npos + o) : 1.0f;
    // regular position + offset, in fp32
    const float lh = (float)(oh * p.sh - p.pt + i * p.dh) + dy;
    const float lw = (float)(ow * p.sw - p.pl + j * p.dw) + dx;
    return corners_of(lh, lw, m, p.H, p.W);
}

// --------------------------------------------------------- implicit GEMM

// MFMA over one K chunk held in LDS: wave `wave` owns rows
// [wave * 32 * MB, +32 * MB) of the W tile As ([m][k], pitch LK) and all 64
// positions of the column tile Bs ([position][k], pitch LK).
template <typename T, int MB, int LK>
__device__ __forceinline__ void mfma_chunk(const typename T::raw_t *As, const typename T::raw_t *Bs,
                                           floatx16 (&acc)[MB][2], int wave, int lane) {
    if constexpr (T::bytes == 4) {
#pragma unroll
        for (int ks = 0; ks < DC_TK / 2; ++ks) {
            const int kk = 2 * ks + (lane >> 5);
            float b[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                b[nb] = __builtin_bit_cast(float, (uint32_t)Bs[(32 * nb + (lane & 31)) * LK + kk]);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = (wave * MB + mb) * 32 + (lane & 31);
                const float a = __builtin_bit_cast(float, (uint32_t)As[m * LK + kk]);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b[nb], acc[mb][nb], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < DC_TK / 16; ++ks) {
            const int kk = 16 * ks + 8 * (lane >> 5);
            u32x4 bv[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                bv[nb] = *(const u32x4 *)&Bs[(32 * nb + (lane & 31)) * LK + kk];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = (wave * MB + mb) * 32 + (lane & 31);
                const u32x4 av = *(const u32x4 *)&As[m * LK + kk];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    if constexpr (__is_same(T, BF16))
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv[nb]),
                            acc[mb][nb], 0, 0, 0);
                    else
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(halfx8, av), __builtin_bit_cast(halfx8, bv[nb]),
                            acc[mb][nb], 0, 0, 0);
                }
            }
        }
    }
}

// Bias and store of a block's TM x 64 tile of Y (image n, output channels
// oc0.., positions nt * 64..): lane holds column (lane & 31) + 32 nb and rows
// 8 (r / 4) + 4 (lane / 32) + (r % 4) of each 32 x 32 block.
template <typename T, int MB>
__device__ __forceinline__ void store_tile(const DeformParams &p, const floatx16 (&acc)[MB][2], int n,
                                           int oc0, int m_valid, int nt, int wave, int lane) {
    const int npos = p.OH * p.OW;
    const rsrc_t yr = make_rsrc((char *)p.Y + (size_t)n * p.OC * npos * T::bytes,
                                (uint32_t)((size_t)p.OC * npos * T::bytes));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = (wave * MB + mb) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const bool mok = m < m_valid;
            const float bias = (mok && p.B) ? ld<T>(p.B, oc0 + m) : 0.0f;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int oo = nt * DC_TN + 32 * nb + (lane & 31);
                const bool ok = mok && oo < npos;
                const uint32_t yo =
                    ok ? (uint32_t)(((size_t)(oc0 + m) * npos + oo) * T::bytes) : GS_OOB;
                T::store(acc[mb][nb][r] + bias, yr, yo);
            }
        }
}

// MB: 32-row blocks of output channels per wave (TM = 4 waves * 32 * MB).
template <typename T, int MB, bool TABLE>
__global__ __launch_bounds__(kBlock) void deform_conv2d_mfma(DeformParams p) {
    using raw_t = typename T::raw_t;
    constexpr int TM = 4 * 32 * MB;
    constexpr int PAD = 16 / T::bytes;      // row padding against LDS bank conflicts
    constexpr int LK = DC_TK + PAD;         // LDS row pitch (elements)
    constexpr int TE = DC_TABLE * DC_TN;    // table entries
    __shared__ __align__(16) raw_t As[TM * LK];      // W tile, [m][k]
    __shared__ __align__(16) raw_t Bs[DC_TN * LK];   // column tile, [position][k]
    __shared__ int tb_off[TABLE ? 4 * TE : 1];
    __shared__ float tb_w[TABLE ? 4 * TE : 1];

    const int lb = xcd_logical_block_runs(p.nblocks);
    if (lb >= p.nblocks) return;
    const int nt = lb % p.n_tiles;
    int rest = lb / p.n_tiles;
    const int mt = rest % p.m_tiles;
    rest /= p.m_tiles;
    const int G = rest % p.group;
    const int n = rest / p.group;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int npos = p.OH * p.OW;
    const int KK = p.KH * p.KW;
    const int g_first = (G * p.Cg) / p.Cog;

    // this thread's output position in the column tile
    const int pos = t & (DC_TN - 1);
    const int o = nt * DC_TN + pos;
    const bool o_ok = o < npos;
    const int oh = o_ok ? o / p.OW : 0, ow = o_ok ? o - (o / p.OW) * p.OW : 0;

    auto sample_of = [&](int g, int tap) -> Corners {
        return sample_corners<T>(p, n, o, o_ok, oh, ow, g, tap);
    };

    if constexpr (TABLE) {
        const int entries = p.og_span * KK * DC_TN;
        for (int e = t; e < entries; e += kBlock) {
            // e = (gi * KK + tap) * 64 + pos, and pos == t & 63 here
            const int gt = e / DC_TN;
            const int gi = gt / KK, tap = gt - gi * KK;
            const Corners c = sample_of(g_first + gi, tap);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tb_off[q * TE + e] = c.off[q];
                tb_w[q * TE + e] = c.w[q];
            }
        }
    }

    // X of image n: one buffer resource; channel c's plane starts at
    // c * plane_bytes (every offset stays below 2^31)
    const rsrc_t xr = make_rsrc((const char *)p.X + (size_t)n * p.C * p.x_plane_bytes,
                                (uint32_t)p.C * p.x_plane_bytes);
    // W rows of this block: output channels G*OCg + mt*TM + m
    const int oc0 = G * p.OCg + mt * TM;
    const int m_valid = min(TM, p.OCg - mt * TM);
    const rsrc_t wr = make_rsrc(p.Wt, p.w_bytes);

    floatx16 acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

    // Software pipeline: the next chunk's W tile (16-byte loads when the rows
    // allow) and column gathers are in flight while the current chunk runs on
    // the matrix cores.  Items past K or past the block's rows load through
    // the out-of-range offset (zeros), so the loads carry no branch.
    constexpr int CPR = DC_TK * T::bytes / 16;      // 16-byte parts per W row
    constexpr int WV = TM * CPR / kBlock;           // vector W parts per thread
    constexpr int NS = DC_TK / (kBlock / DC_TN);    // column slots per thread
    const bool wvec = p.w_vec != 0;
    u32x4 wpre[WV];
    float xpre[NS][4];
    float cw[NS][4];  // corner weights of the non-table path
    auto prefetch = [&](int k0) {
        if (wvec) {
#pragma unroll
            for (int j = 0; j < WV; ++j) {
                const int i = t + j * kBlock;
                const int row = i / CPR, part = i - (i / CPR) * CPR;
                const int k = k0 + part * (16 / T::bytes);
                const bool ok = row < m_valid && k < p.Ktot;
                const uint32_t wo =
                    ok ? (uint32_t)(((size_t)(oc0 + row) * p.Ktot + k) * T::bytes) : GS_OOB;
                wpre[j] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)wo, 0, 0);
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int k = k0 + (t >> 6) + (kBlock / DC_TN) * s;
            const bool kin = k < p.Ktot;
            const int kc = kin ? k : 0;
            const int cl = kc / KK, tap = kc - (kc / KK) * KK;
            const int c = G * p.Cg + cl;
            const int g = c / p.Cog;
            int off[4];
            if constexpr (TABLE) {
                const int e = ((g - g_first) * KK + tap) * DC_TN + pos;
#pragma unroll
                for (int q = 0; q < 4; ++q) off[q] = tb_off[q * TE + e];
            } else {
                const Corners cr = sample_of(g, tap);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    off[q] = cr.off[q];
                    cw[s][q] = cr.w[q];
                }
            }
            const uint32_t pb = (uint32_t)c * p.x_plane_bytes;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xpre[s][q] = T::load(xr, (kin && off[q] >= 0) ? pb + (uint32_t)off[q] * T::bytes
                                                              : GS_OOB);
        }
    };

    if constexpr (TABLE) __syncthreads();  // the table is complete before the first gathers
    prefetch(0);
    for (int k0 = 0; k0 < p.Ktot; k0 += DC_TK) {
        __syncthreads();  // the previous chunk's LDS reads are done
        // ---- W tile: TM x 32 into LDS
        if (wvec) {
#pragma unroll
            for (int j = 0; j < WV; ++j) {
                const int i = t + j * kBlock;
                const int row = i / CPR, part = i - (i / CPR) * CPR;
                *(u32x4 *)&As[row * LK + part * (16 / T::bytes)] = wpre[j];
            }
        } else {
            for (int e = t; e < TM * DC_TK; e += kBlock) {
                const int m = e / DC_TK, kk = e - m * DC_TK;
                const int k = k0 + kk;
                const bool ok = m < m_valid && k < p.Ktot;
                const uint32_t wo =
                    ok ? (uint32_t)(((size_t)(oc0 + m) * p.Ktot + k) * T::bytes) : GS_OOB;
                As[m * LK + kk] = T::load_raw(wr, wo);
            }
        }
        // ---- column tile: 32 x 64, this thread's position, NS of the K slots
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int kk = (t >> 6) + (kBlock / DC_TN) * s;
            float w4[4];
            if constexpr (TABLE) {
                const int k = k0 + kk;
                const int kc = k < p.Ktot ? k : 0;
                const int cl = kc / KK, tap = kc - (kc / KK) * KK;
                const int g = (G * p.Cg + cl) / p.Cog;
                const int e = ((g - g_first) * KK + tap) * DC_TN + pos;
#pragma unroll
                for (int q = 0; q < 4; ++q) w4[q] = tb_w[q * TE + e];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) w4[q] = cw[s][q];
            }
            float v = w4[0] * xpre[s][0];
#pragma unroll
            for (int q = 1; q < 4; ++q) v = fmaf(w4[q], xpre[s][q], v);
            Bs[pos * LK + kk] = to_raw<T>(v);
        }
        __syncthreads();
        prefetch(k0 + DC_TK);
        mfma_chunk<T, MB, LK>(As, Bs, acc, wave, lane);
    }
    store_tile<T, MB>(p, acc, n, oc0, m_valid, nt, wave, lane);
}

// ------------------------------------------- channels-last implicit GEMM
//
// When every conv group and offset group holds a multiple of 8 channels, the
// sampled columns come from a channels-last copy of X, (N, H, W, C): the 8
// consecutive channels a thread samples at one corner are one 16-byte load
// (two for fp32), instead of 8 scalar gathers from 8 planes.  K is walked in
// chunks of one kernel position and 32 channels of the conv group (Cgp = Cg
// rounded up to 32), so one set of corners serves a whole chunk.  W is copied
// to match the chunk order, zero beyond Cg.  Summing K in another order than the
// oracle only changes fp32 rounding order.

// Chunk i of the channels-last kernel covers one kernel position and tk (32
// or 64) channels of the conv group (Cgp = Cg rounded up to tk).  The table
// path walks the channel slices outermost (a slice's corners stay in L1
// across the kernel positions), the other path the kernel positions
// outermost (its corners change once per position).
__device__ __forceinline__ void chunk_coords(int i, int KK, int cpt, bool slice_major, int tk,
                                             int &tap, int &c0) {
    const int sl = slice_major ? i / KK : i - (i / cpt) * cpt;
    tap = slice_major ? i - sl * KK : i / cpt;
    c0 = sl * tk;
}

// As chunk_coords, dividing by KK and cpt with the launch's multipliers
// (i < 2^31).
__device__ __forceinline__ void chunk_coords_fd(int i, int KK, int cpt, FastDiv kk_div,
                                                FastDiv cpt_div, bool slice_major, int tk,
                                                int &tap, int &c0) {
    if (slice_major) {
        const int sl = (int)fdiv((uint32_t)i, kk_div);
        tap = i - sl * KK;
        c0 = sl * tk;
    } else {
        tap = (int)fdiv((uint32_t)i, cpt_div);
        c0 = (i - tap * cpt) * tk;
    }
}

// W (OC, Cg, KK) -> W2, packed in the order the matrix cores take the A
// operand: for conv group G, 32-row block R of its OCg rows (rounded up to
// 32), chunk i and load v, lane l's 16 bytes at
// ((((G * Rg + R) * nch + i) * AV + v) * 64 + l) * 16.  Lane l holds row
// R * 32 + l % 32 and, within the chunk, k = 16 v + 8 (l / 32) + 0..7 for
// fp16 / bf16 (AV = tk / 16), k = 16 (l / 32) + 4 v + 0..3 for fp32 (tk =
// 32, AV = 4).  Rows past OCg and channels past Cg are zero.  One thread per
// 16-byte unit.
template <typename raw_t, int AV>
__device__ __forceinline__ void w_pack_unit(const raw_t *__restrict__ W, raw_t *__restrict__ W2,
                                            int group, int OCg, int Cg, int KK, int Cgp,
                                            int slice_major, uint32_t j) {
    constexpr int EPL = 16 / sizeof(raw_t);         // elements per lane and load
    constexpr int TKC = EPL == 4 ? 32 : 16 * AV;    // chunk size
    const int Rg = (OCg + 31) / 32;
    const int cpt = Cgp / TKC, nch = KK * cpt;
    // W2 holds fewer than 2^31 bytes, so 32-bit indices suffice
    const uint32_t units = (uint32_t)group * Rg * nch * AV * 64;
    if (j >= units) return;
    const int l = (int)(j % 64);
    uint32_t u = j / 64;
    const int v = (int)(u % AV);
    u /= AV;
    const int i = (int)(u % (uint32_t)nch);
    u /= (uint32_t)nch;
    const int R = (int)(u % (uint32_t)Rg);
    const int G = (int)(u / (uint32_t)Rg);
    const int row = R * 32 + (l & 31);
    int tap, c0;
    chunk_coords(i, KK, cpt, slice_major != 0, TKC, tap, c0);
    const int k0 = EPL == 4 ? 16 * (l >> 5) + 4 * v : 16 * v + 8 * (l >> 5);
    const raw_t *wrow = W + (((size_t)G * OCg + row) * Cg) * KK + tap;
    u32x4 out;
    raw_t *e = (raw_t *)&out;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
        const int cl = c0 + k0 + k;
        e[k] = (row < OCg && cl < Cg) ? wrow[(size_t)cl * KK] : (raw_t)0;
    }
    *(u32x4 *)(W2 + (size_t)j * EPL) = out;
}

// The channels-last kernel's preparation in one launch: blocks below
// x_blocks transpose 64 x 64 tiles of X, the rest pack W (one 16-byte unit
// per thread); the two halves touch disjoint memory.
template <typename raw_t, int AV, bool VEC>
__global__ __launch_bounds__(kBlock) void cl_prepare(const raw_t *__restrict__ X, raw_t *__restrict__ Xt,
                                                    int C, int S, int c_tiles, int s_tiles, int x_blocks,
                                                    const raw_t *__restrict__ W, raw_t *__restrict__ W2,
                                                    int group, int OCg, int Cg, int KK, int Cgp,
                                                    int slice_major) {
    const int b = blockIdx.x;
    if (b < x_blocks) {
        if constexpr (VEC) to_channels_last_tile<raw_t>(X, Xt, C, S, c_tiles, s_tiles, b, C);
        else to_channels_last_scalar<raw_t>(X, Xt, C, S, c_tiles, s_tiles, b, C);
    } else {
        w_pack_unit<raw_t, AV>(W, W2, group, OCg, Cg, KK, Cgp, slice_major,
                               (uint32_t)(b - x_blocks) * kBlock + threadIdx.x);
    }
}

// Eight elements of type T from 8 * T::bytes consecutive bytes, widened.
template <typename T>
__device__ __forceinline__ void unpack8(const u32x4 *v, float (&x)[8]) {
    if constexpr (T::bytes == 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // through a scalar: a bit cast of the vector element itself
                // reads element 0 with this compiler
                const uint32_t u = v[h][e];
                x[4 * h + e] = __builtin_bit_cast(float, u);
            }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = T::from_raw((uint16_t)(v[0][e] & 0xffffu));
            x[2 * e + 1] = T::from_raw((uint16_t)(v[0][e] >> 16));
        }
    }
}

template <typename T>
__device__ __forceinline__ void pack8(const float (&x)[8], u32x4 *v) {
    if constexpr (T::bytes == 4) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[h][e] = __builtin_bit_cast(uint32_t, x[4 * h + e]);
    } else if constexpr (__is_same(T, BF16)) {
        // one v_cvt_pk_bf16_f32 per pair (round to nearest even, as to_raw)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2 pr = {settle(x[2 * e]), settle(x[2 * e + 1])};
            v[0][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[0][e] = (uint32_t)to_raw<T>(x[2 * e]) | ((uint32_t)to_raw<T>(x[2 * e + 1]) << 16);
    }
}

// MFMA over one chunk with the A operand (W rows) in registers, loaded in
// the instruction's layout, and the column tile Bs ([position][k], pitch LK)
// in LDS.  Inside a chunk the k of an fp32 step ks is 16 * (lane / 32) + ks
// for both operands (any pairing of A and B columns sums the same terms);
// fp16 / bf16 keep the native order, k = 16 ks + 8 (lane / 32) + 0..7.
template <typename T, int MB, int LK, int AV>
__device__ __forceinline__ void mfma_chunk_regs(const u32x4 (&a)[MB][AV], const typename T::raw_t *Bs,
                                                floatx16 (&acc)[MB][2], int lane) {
    if constexpr (T::bytes == 4) {
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
            u32x4 b[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                b[nb] = *(const u32x4 *)&Bs[(32 * nb + (lane & 31)) * LK + 16 * (lane >> 5) + 4 * kq];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const uint32_t au = a[mb][kq][e];
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const uint32_t bu = b[nb][e];
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            __builtin_bit_cast(float, au), __builtin_bit_cast(float, bu), acc[mb][nb],
                            0, 0, 0);
                    }
                }
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < AV; ++ks) {
            u32x4 bv[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                bv[nb] = *(const u32x4 *)&Bs[(32 * nb + (lane & 31)) * LK + 16 * ks + 8 * (lane >> 5)];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    if constexpr (__is_same(T, BF16))
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a[mb][ks]), __builtin_bit_cast(bf16x8, bv[nb]),
                            acc[mb][nb], 0, 0, 0);
                    else
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(halfx8, a[mb][ks]), __builtin_bit_cast(halfx8, bv[nb]),
                            acc[mb][nb], 0, 0, 0);
                }
        }
    }
}

// NW waves per block (4, or 8 for fp16 / bf16 with 256 output channels per
// block), chunks of TK = 8 * NW channels, loads DEPTH chunks ahead (8 waves:
// corner gathers two chunks ahead and A one, so that four waves fit a SIMD).
template <typename T, int MB, bool TABLE, int NW>
__global__ __launch_bounds__(64 * NW) void deform_conv2d_cl(DeformParams p) {
    using raw_t = typename T::raw_t;
    constexpr int NT = 64 * NW;                     // threads
    constexpr int TK = 8 * NW;                      // channels per chunk
    constexpr int DEPTH = NW == 8 ? 1 : 2;
    constexpr int TM = NW * 32 * MB;
    constexpr int PAD = 16 / T::bytes;
    constexpr int LK = TK + PAD;
    constexpr int TE = DC_TABLE * DC_TN;
    constexpr int VPC = 8 * T::bytes / 16;          // 16-byte loads per corner
    constexpr int AV = T::bytes == 4 ? 4 : TK / 16; // 16-byte A loads per 32-row block and chunk
    static_assert(T::bytes == 2 || NW == 4, "fp32 runs four waves");
    __shared__ __align__(16) raw_t Bs[2][DC_TN * LK];  // column tiles, double-buffered
    // corner byte offsets of the pixel's channel run in Xt (out-of-range
    // offset for corners outside the image) and mask-folded weights
    __shared__ uint32_t tb_off[TABLE ? 4 * TE : 1];
    __shared__ float tb_w[TABLE ? 4 * TE : 1];
    const uint32_t pix_bytes = (uint32_t)p.C * T::bytes;

    const int lb = xcd_logical_block_runs(p.nblocks);
    if (lb >= p.nblocks) return;
    const int nt = lb % p.n_tiles;
    int rest = lb / p.n_tiles;
    const int mt = rest % p.m_tiles;
    rest /= p.m_tiles;
    const int G = rest % p.group;
    const int n = rest / p.group;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int npos = p.OH * p.OW;
    const int KK = p.KH * p.KW;
    const int g_first = (G * p.Cg) / p.Cog;

    // This thread samples output position pos and channels c0 + 8 cgp ..
    // +7 of each chunk: the four lanes of a position read one 64-byte run of
    // a pixel, so a wave's load touches 16 pixels.
    const int cgp = (t & 3) + 4 * (t >> 8);
    const int pos = (t >> 2) & (DC_TN - 1);
    const int o = nt * DC_TN + pos;
    const bool o_ok = o < npos;
    const int oh = o_ok ? o / p.OW : 0, ow = o_ok ? o - (o / p.OW) * p.OW : 0;

    if constexpr (TABLE) {
        const int entries = p.og_span * KK * DC_TN;
        for (int e = t; e < entries; e += NT) {
            const int gt = e / DC_TN;
            const int gi = gt / KK, tap = gt - gi * KK;
            const int oe = nt * DC_TN + (e & (DC_TN - 1));
            const bool oe_ok = oe < npos;
            const int ohe = oe_ok ? oe / p.OW : 0, owe = oe_ok ? oe - (oe / p.OW) * p.OW : 0;
            const Corners c = sample_corners<T>(p, n, oe, oe_ok, ohe, owe, g_first + gi, tap);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tb_off[q * TE + e] = c.off[q] >= 0 ? (uint32_t)c.off[q] * pix_bytes : GS_OOB;
                tb_w[q * TE + e] = c.w[q];
            }
        }
        __syncthreads();
    }

    // channels-last X of image n; pixel s, channel c at (s * C + c) * bytes
    const rsrc_t xr = make_rsrc((const char *)p.Xt + (size_t)n * p.x_img_bytes, p.x_img_bytes);
    const int oc0 = G * p.OCg + mt * TM;
    const int m_valid = min(TM, p.OCg - mt * TM);
    // packed W of conv group G; 32-row blocks past the group's last read zeros
    const rsrc_t wr = make_rsrc((const char *)p.W2 + (size_t)G * p.w2_group_bytes, p.w2_group_bytes);

    floatx16 acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

    const int cpt = p.Cgp / TK;                     // chunks per kernel position
    const int nch = KK * cpt;
    // DEPTH register sets: chunk i's loads were issued DEPTH chunks earlier,
    // into set i % DEPTH.
    u32x4 a0[MB][AV], a1[DEPTH == 2 ? MB : 1][AV];
    u32x4 x0[4][VPC], x1[DEPTH == 2 ? 4 : 1][VPC];
    float q0[4], q1[4];
    u32x4 x8[NW == 8 ? 4 : 1][VPC];                 // eight waves: the second corner set
    float q8[4];
    Corners cc;                                     // corners of (ctap, cg), non-table path
    int ctap = -1, cg = -1;
    // Past the last chunk the loads fetch the last chunk again (unused):
    // issuing the same loads every chunk keeps the waits counted, not full.
    // This wave's packed A of chunk i: one coalesced 1 KB load per 32-row
    // block and v.
    auto load_a = [&](int i, u32x4 (&a)[MB][AV]) {
        i = min(i, nch - 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int R = mt * (TM / 32) + wave * MB + mb;
#pragma unroll
            for (int v = 0; v < AV; ++v) {
                const uint32_t wo =
                    R < p.Rg ? (uint32_t)((((size_t)R * nch + i) * AV + v) * 64 + lane) * 16 : GS_OOB;
                a[mb][v] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)wo, 0, 0);
            }
        }
    };
    // The four corners of this thread's position for channels c0 + 8 cgp ..
    // +7 of chunk i, and their weights.
    auto load_x = [&](int i, u32x4 (&xpre)[4][VPC], float (&wq)[4]) {
        i = min(i, nch - 1);
        int tap, c0;
        chunk_coords_fd(i, KK, cpt, FastDiv{0, p.kk_m, p.kk_s}, FastDiv{0, p.cpt_m, p.cpt_s}, TABLE,
                        TK, tap, c0);
        const int cl = c0 + 8 * cgp;
        const bool cv = cl < p.Cg;                  // past Cg: padding, W2 is zero there
        const int c = G * p.Cg + (cv ? cl : 0);
        const int g = (int)fdiv((uint32_t)c, FastDiv{0, p.cog_m, p.cog_s});
        uint32_t off[4];
        if constexpr (TABLE) {
            const int e = ((g - g_first) * KK + tap) * DC_TN + pos;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                off[q] = tb_off[q * TE + e];
                wq[q] = tb_w[q * TE + e];
            }
        } else {
            if (tap != ctap || g != cg) {
                cc = sample_corners<T>(p, n, o, o_ok, oh, ow, g, tap);
                ctap = tap;
                cg = g;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                off[q] = cc.off[q] >= 0 ? (uint32_t)cc.off[q] * pix_bytes : GS_OOB;
                wq[q] = cc.w[q];
            }
        }
        // an out-of-range corner offset stays out of range (below 2^32) with
        // the channel's bytes added
        const uint32_t cbytes = (uint32_t)c * T::bytes;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t xo = cv ? off[q] + cbytes : GS_OOB;
#pragma unroll
            for (int v = 0; v < VPC; ++v)
                xpre[q][v] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(xo + 16 * v), 0, 0);
        }
    };

    // loads issued per chunk: chunk i's are complete once no more than
    // DEPTH - 1 chunks' worth is outstanding
    constexpr int kLoads = (DEPTH - 1) * (MB * AV + 4 * VPC);
    static_assert(kLoads < 64, "vmcnt field");
    // One chunk: sample its columns into this chunk's LDS buffer; issue the
    // corner loads of the chunk two ahead into the registers just read;
    // multiply; then issue that chunk's A loads into the A registers just
    // used.
    auto step = [&](int i, u32x4 (&a)[MB][AV], u32x4 (&xpre)[4][VPC], float (&wq)[4]) {
        raw_t *bs = Bs[i & 1];
        // keep the scheduler from pulling this chunk's work above the
        // previous chunk's loads (it would then wait for those loads)
        __builtin_amdgcn_sched_barrier(0);
        // vmcnt(kLoads), expcnt and lgkmcnt left free
        __builtin_amdgcn_s_waitcnt((kLoads & 15) | ((kLoads >> 4) << 14) | 0x0f70);
        {
            float v[8], x[8];
            unpack8<T>(xpre[0], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = wq[0] * x[e];
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                unpack8<T>(xpre[q], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fmaf(wq[q], x[e], v[e]);
            }
            u32x4 packed[VPC];
            pack8<T>(v, packed);
#pragma unroll
            for (int h = 0; h < VPC; ++h)
                *(u32x4 *)&bs[pos * LK + 8 * cgp + h * (16 / T::bytes)] = packed[h];
        }
        // Every wave's column writes of chunk i are visible, and every wave
        // has finished reading the other buffer (chunk i - 1).
        __syncthreads();
        load_x(i + DEPTH, xpre, wq);
        mfma_chunk_regs<T, MB, LK, AV>(a, bs, acc, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_a(i + DEPTH, a);
    };

    // Eight waves: the corner gathers (scattered, the long wait) run two
    // chunks ahead and A one.  Issue order per step: A of the next chunk,
    // then the corners of the one after, so a step finds (oldest first) its
    // corners, its A, the next chunk's corners outstanding.  It waits for its
    // corners, samples, and waits for its A only before the MFMAs.
    constexpr int kCornerLoads = 4 * VPC;
    constexpr int kCornersDone = kCornerLoads + MB * AV;  // A and next corners may be out
    static_assert(kCornersDone < 64, "vmcnt field");
    auto step8 = [&](int i, u32x4 (&xpre)[4][VPC], float (&wq)[4]) {
        raw_t *bs = Bs[i & 1];
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((kCornersDone & 15) | ((kCornersDone >> 4) << 14) | 0x0f70);
        {
            float v[8], x[8];
            unpack8<T>(xpre[0], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = wq[0] * x[e];
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                unpack8<T>(xpre[q], x);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fmaf(wq[q], x[e], v[e]);
            }
            u32x4 packed[VPC];
            pack8<T>(v, packed);
#pragma unroll
            for (int h = 0; h < VPC; ++h)
                *(u32x4 *)&bs[pos * LK + 8 * cgp + h * (16 / T::bytes)] = packed[h];
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((kCornerLoads & 15) | ((kCornerLoads >> 4) << 14) | 0x0f70);
        mfma_chunk_regs<T, MB, LK, AV>(a0, bs, acc, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_a(i + 1, a0);
        load_x(i + 2, xpre, wq);
    };

    if constexpr (NW == 8) {
        load_x(0, x0, q0);
        load_a(0, a0);
        load_x(1, x8, q8);
        int i = 0;
        for (; i + 1 < nch; i += 2) {
            step8(i, x0, q0);
            step8(i + 1, x8, q8);
        }
        if (i < nch) step8(i, x0, q0);
        store_tile<T, MB>(p, acc, n, oc0, m_valid, nt, wave, lane);
        return;
    }
    load_x(0, x0, q0);
    load_a(0, a0);
    if constexpr (DEPTH == 2) {
        load_x(1, x1, q1);
        load_a(1, a1);
        int i = 0;
        for (; i + 1 < nch; i += 2) {
            step(i, a0, x0, q0);
            step(i + 1, a1, x1, q1);
        }
        if (i < nch) step(i, a0, x0, q0);
    } else {
        for (int i = 0; i < nch; ++i) step(i, a0, x0, q0);
    }
    store_tile<T, MB>(p, acc, n, oc0, m_valid, nt, wave, lane);
}

// ----------------------------------------------------------- direct kernel

// Linear sample of one plane (r axes) at the location with per-axis floor
// `base` and fraction `frac`, zero outside, in double: corners innermost
// axis fastest, weights as products over the axes (outermost first).
template <int R, typename T>
__device__ __forceinline__ double sample_direct(rsrc_t xr, uint32_t plane_byte, const int *ext,
                                                const int *base, const double *frac) {
    double acc = 0.0;
#pragma unroll
    for (int tcorner = 0; tcorner < (1 << R); ++tcorner) {
        double w = 1.0;
        bool valid = true;
        uint32_t off = 0;
#pragma unroll
        for (int a = 0; a < R; ++a) {
            const int bit = (tcorner >> (R - 1 - a)) & 1;
            const int i = base[a] + bit;
            w = w * (bit ? frac[a] : 1.0 - frac[a]);
            valid = valid && i >= 0 && i < ext[a];
            off = off * (uint32_t)ext[a] + (uint32_t)i;
        }
        const double x = T::load(xr, valid ? plane_byte + off * (uint32_t)T::bytes : GS_OOB);
        acc = valid ? acc + w * x : acc;
    }
    return acc;
}

// Element types of the direct kernel: loads widen to double, stores round.
struct DcF32 {
    static constexpr int bytes = 4;
    __device__ static double load(rsrc_t r, uint32_t o) { return (double)F32::load(r, o); }
    __device__ static double at(const void *p, size_t i) { return ((const float *)p)[i]; }
    __device__ static void store(double v, rsrc_t r, uint32_t o) { F32::store((float)v, r, o); }
};
struct DcF16 {
    static constexpr int bytes = 2;
    __device__ static double load(rsrc_t r, uint32_t o) { return (double)F16::load(r, o); }
    __device__ static double at(const void *p, size_t i) {
        return (double)F16::from_raw(((const uint16_t *)p)[i]);
    }
    __device__ static void store(double v, rsrc_t r, uint32_t o) { F16::store((float)v, r, o); }
};
struct DcBF16 {
    static constexpr int bytes = 2;
    __device__ static double load(rsrc_t r, uint32_t o) { return (double)BF16::load(r, o); }
    __device__ static double at(const void *p, size_t i) {
        return (double)BF16::from_raw(((const uint16_t *)p)[i]);
    }
    __device__ static void store(double v, rsrc_t r, uint32_t o) { BF16::store((float)v, r, o); }
};
struct DcF64 {
    static constexpr int bytes = 8;
    __device__ static double load(rsrc_t r, uint32_t o) {
        return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, (int)o, 0, 0));
    }
    __device__ static double at(const void *p, size_t i) { return ((const double *)p)[i]; }
    __device__ static void store(double v, rsrc_t r, uint32_t o) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)o, 0, kStoreNT);
    }
};

// One lane per output (n, oc, o); locations in fp32 (double for double data).
template <int R, typename T>
__global__ __launch_bounds__(kBlock) void deform_conv_direct(DeformParams p) {
    const size_t idx = (size_t)blockIdx.x * kBlock + threadIdx.x;
    const size_t npos = p.npos;
    const size_t total = (size_t)p.N * p.OC * npos;
    if (idx >= total) return;
    const size_t o = idx % npos;
    const int oc = (int)((idx / npos) % p.OC);
    const int n = (int)(idx / (npos * p.OC));
    const int G = oc / p.OCg;
    int oi[3];
    size_t rem = o;
#pragma unroll
    for (int a = R - 1; a >= 0; --a) {
        oi[a] = (int)(rem % (size_t)p.out_ext[a]);
        rem /= (size_t)p.out_ext[a];
    }
    const rsrc_t xr = make_rsrc((const char *)p.X + (size_t)n * p.C * p.x_plane_bytes,
                                (uint32_t)p.C * p.x_plane_bytes);
    const int K = p.Ktot / p.Cg;
    double acc = 0.0;
    for (int cl = 0; cl < p.Cg; ++cl) {
        const int c = G * p.Cg + cl;
        const int g = c / p.Cog;
        for (int k = 0; k < K; ++k) {
            int ki[3];
            int kr = k;
#pragma unroll
            for (int a = R - 1; a >= 0; --a) {
                ki[a] = kr % p.k_ext[a];
                kr /= p.k_ext[a];
            }
            int base[3];
            double frac[3];
            bool finite = true;
#pragma unroll
            for (int a = 0; a < R; ++a) {
                const int regular = oi[a] * p.stride[a] - p.pad[a] + ki[a] * p.dil[a];
                const double d =
                    T::at(p.offset, (((size_t)n * p.og + g) * K * R + (size_t)k * R + a) * npos + o);
                double loc;
                if constexpr (T::bytes == 8) loc = (double)regular + d;
                else loc = (double)((float)regular + (float)d);
                if (!__builtin_isfinite(loc) || fabs(loc) > (double)kCoordLimit) finite = false;
                const double fl = finite ? floor(loc) : 0.0;
                base[a] = (int)fl;
                frac[a] = finite ? loc - fl : 0.0;
            }
            if (!finite) continue;
            double v = sample_direct<R, T>(xr, (uint32_t)c * p.x_plane_bytes, p.in_ext, base, frac);
            if (p.mask) v = v * T::at(p.mask, (((size_t)n * p.og + g) * K + k) * npos + o);
            acc = acc + T::at(p.Wt, ((size_t)oc * p.Cg + cl) * K + k) * v;
        }
    }
    if (p.B) acc = acc + T::at(p.B, oc);
    const rsrc_t yr = make_rsrc((char *)p.Y + (size_t)n * p.OC * npos * T::bytes,
                                (uint32_t)((size_t)p.OC * npos * T::bytes));
    T::store(acc, yr, (uint32_t)(((size_t)oc * npos + o) * T::bytes));
}

// --------------------------------------------------------------- dispatch

template <typename T>
static int mfma_launch(const DeformParams &p, hipStream_t s) {
    const dim3 grid(8 * kRun * ((p.nblocks + 8 * kRun - 1) / (8 * kRun)));
    const bool table = p.og_span * p.KH * p.KW <= DC_TABLE;
    const bool wide = p.OCg > 128;
    if (wide) {
        if (table) hipLaunchKernelGGL((deform_conv2d_mfma<T, 2, true>), grid, dim3(kBlock), 0, s, p);
        else hipLaunchKernelGGL((deform_conv2d_mfma<T, 2, false>), grid, dim3(kBlock), 0, s, p);
    } else {
        if (table) hipLaunchKernelGGL((deform_conv2d_mfma<T, 1, true>), grid, dim3(kBlock), 0, s, p);
        else hipLaunchKernelGGL((deform_conv2d_mfma<T, 1, false>), grid, dim3(kBlock), 0, s, p);
    }
    return (int)hipGetLastError();
}

template <typename T>
static int cl_launch(const DeformParams &p, hipStream_t s) {
    using raw_t = typename T::raw_t;
    const int S = p.H * p.W, KK = p.KH * p.KW;
    const int c_tiles = (p.C + 63) / 64, s_tiles = (S + 63) / 64;
    const int x_blocks = (int)((size_t)p.N * c_tiles * s_tiles);
    const bool table = p.og_span * KK <= DC_TABLE;
    const bool wide = p.OCg > 128;
    const bool eight = T::bytes == 2 && wide;       // 8 waves, chunks of 64 channels
    const int w_blocks = (int)(((size_t)p.w2_bytes / 16 + kBlock - 1) / kBlock);
    constexpr int VW = 16 / sizeof(raw_t);
    // C is a multiple of 8 on this path
    const dim3 pgrid((unsigned)(x_blocks + w_blocks));
    const bool vec = S % VW == 0 && (uintptr_t)p.X % 16 == 0;
    constexpr int AV4 = T::bytes == 4 ? 4 : 2;      // chunks of 32 channels
    auto prepare = [&](auto av) {
        constexpr int AV = decltype(av)::value;
        if (vec)
            hipLaunchKernelGGL((cl_prepare<raw_t, AV, true>), pgrid, dim3(kBlock), 0, s, (const raw_t *)p.X,
                               (raw_t *)p.Xt, p.C, S, c_tiles, s_tiles, x_blocks, (const raw_t *)p.Wt,
                               (raw_t *)p.W2, p.group, p.OCg, p.Cg, KK, p.Cgp, (int)table);
        else
            hipLaunchKernelGGL((cl_prepare<raw_t, AV, false>), pgrid, dim3(kBlock), 0, s, (const raw_t *)p.X,
                               (raw_t *)p.Xt, p.C, S, c_tiles, s_tiles, x_blocks, (const raw_t *)p.Wt,
                               (raw_t *)p.W2, p.group, p.OCg, p.Cg, KK, p.Cgp, (int)table);
    };
    const dim3 grid(8 * kRun * ((p.nblocks + 8 * kRun - 1) / (8 * kRun)));
    if constexpr (T::bytes == 2) {
        if (eight) {
            prepare(std::integral_constant<int, 4>());
            if (table) hipLaunchKernelGGL((deform_conv2d_cl<T, 1, true, 8>), grid, dim3(512), 0, s, p);
            else hipLaunchKernelGGL((deform_conv2d_cl<T, 1, false, 8>), grid, dim3(512), 0, s, p);
            return (int)hipGetLastError();
        }
    }
    prepare(std::integral_constant<int, AV4>());
    if (wide) {
        if (table) hipLaunchKernelGGL((deform_conv2d_cl<T, 2, true, 4>), grid, dim3(kBlock), 0, s, p);
        else hipLaunchKernelGGL((deform_conv2d_cl<T, 2, false, 4>), grid, dim3(kBlock), 0, s, p);
    } else {
        if (table) hipLaunchKernelGGL((deform_conv2d_cl<T, 1, true, 4>), grid, dim3(kBlock), 0, s, p);
        else hipLaunchKernelGGL((deform_conv2d_cl<T, 1, false, 4>), grid, dim3(kBlock), 0, s, p);
    }
    return (int)hipGetLastError();
}

template <int R, typename T>
static int direct_launch(const DeformParams &p, hipStream_t s) {
    const size_t total = (size_t)p.N * p.OC * p.npos;
    const dim3 grid((unsigned)((total + kBlock - 1) / kBlock));
    hipLaunchKernelGGL((deform_conv_direct<R, T>), grid, dim3(kBlock), 0, s, p);
    return (int)hipGetLastError();
}

template <typename T>
static int direct_by_rank(const DeformParams &p, int rank, hipStream_t s) {
    switch (rank) {
    case 1: return direct_launch<1, T>(p, s);
    case 2: return direct_launch<2, T>(p, s);
    default: return direct_launch<3, T>(p, s);
    }
}

int launch_deform_conv(const DeformParams &p, int rank, int dtype, int path, hipStream_t s) {
    if (path == DC_PATH_CL) {
        switch (dtype) {
        case 0: return cl_launch<F32>(p, s);
        case 1: return cl_launch<F16>(p, s);
        default: return cl_launch<BF16>(p, s);
        }
    }
    if (path == DC_PATH_GATHER) {
        switch (dtype) {
        case 0: return mfma_launch<F32>(p, s);
        case 1: return mfma_launch<F16>(p, s);
        default: return mfma_launch<BF16>(p, s);
        }
    }
    switch (dtype) {
    case 0: return direct_by_rank<DcF32>(p, rank, s);
    case 1: return direct_by_rank<DcF16>(p, rank, s);
    case 2: return direct_by_rank<DcBF16>(p, rank, s);
    default: return direct_by_rank<DcF64>(p, rank, s);
    }
}

}  // namespace gs
