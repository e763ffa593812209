// gemm.h -- LDS-tiled GEMM kernels over a LayerArgs "problem" (layer.h).
//
//   gemm_mfma_kernel<P>: bf16 operands, fp32 accumulate on
//     v_mfma_f32_32x32x16_bf16.  Tile 128 x 128 x 64, 256 threads as 2 x 2
//     waves of 64 x 64.  Global -> registers -> LDS, double-buffered, with
//     the next k-tile's global loads in flight during the current tile's
//     MFMAs.  LDS rows are 64 bf16 = 8 chunks of 16 B; chunk c of row r sits
//     at c ^ (r & 7), so both the 16-byte row writes and the 16-byte fragment
//     reads of 8 consecutive rows hit 8 distinct bank groups.
//   gemm_simt_kernel<P>: float32 everywhere, 64 x 64 x 16 tiles, 4 x 4
//     outputs per thread on the vector ALUs.
//
// grid.x walks the problem's row tiles, grid.y its column tiles.
#pragma once

#include "layer.h"

namespace lmoe {

constexpr int kTileM = 128, kTileN = 128, kTileK = 64;
constexpr int kSimtM = 64, kSimtN = 64, kSimtK = 16;

template <class P>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(LayerArgs a) {
    int grp, row0, row_end;
    if (!P::tile(a, blockIdx.x, kTileM, grp, row0, row_end)) return;
    const int col0 = blockIdx.y * kTileN;
    const int ncols = P::ncols(a);
    if (col0 >= ncols) return;
    const int K = P::kdim(a);

    __shared__ uint4 As[2][kTileM * 8];
    __shared__ uint4 Bs[2][kTileN * 8];

    const int tid = threadIdx.x;
    const int ch = tid & 7;       // 16-byte chunk within a 64-element k-slice
    const int lrow = tid >> 3;    // 0..31; rows lrow + 32*i
    const bf16* ap[4];
    const bf16* bp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = row0 + lrow + 32 * i;
        ap[i] = r < row_end ? P::a_row(a, grp, r) + ch * 8 : nullptr;
        const int c = col0 + lrow + 32 * i;
        bp[i] = c < ncols ? P::b_row(a, grp, c) + ch * 8 : nullptr;
    }
    uint4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = ap[i] ? ldg16(ap[i] + k0) : kZero16;
            rb[i] = bp[i] ? ldg16(bp[i] + k0) : kZero16;
        }
    };
    auto swrite = [&](int st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = lrow + 32 * i;
            As[st][r * 8 + (ch ^ (r & 7))] = ra[i];
            Bs[st][r * 8 + (ch ^ (r & 7))] = rb[i];
        }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gload(0);
    swrite(0);
    __syncthreads();
    const int nk = K / kTileK;
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kTileK);
#pragma unroll
        for (int kk = 0; kk < kTileK / 16; ++kk) {
            const int chunk = kk * 2 + (lane >> 5);
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                af[i] = as_bf16x8(As[st][r * 8 + (chunk ^ (r & 7))]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = wn * 64 + j * 32 + (lane & 31);
                bfr[j] = as_bf16x8(Bs[st][c * 8 + (chunk ^ (c & 7))]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < nk) swrite(st ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = col0 + wn * 64 + j * 32 + (lane & 31);
                if (row < row_end && col < ncols) P::store(a, grp, row, col, acc[i][j][r]);
            }
}

template <class P>
__global__ __launch_bounds__(256) void gemm_simt_kernel(LayerArgs a) {
    int grp, row0, row_end;
    if (!P::tile(a, blockIdx.x, kSimtM, grp, row0, row_end)) return;
    const int col0 = blockIdx.y * kSimtN;
    const int ncols = P::ncols(a);
    if (col0 >= ncols) return;
    const int K = P::kdim(a);

    __shared__ float As[kSimtK][kSimtM + 4];
    __shared__ float Bs[kSimtK][kSimtN + 4];
    const int tid = threadIdx.x;
    const int lr = tid >> 2;          // row of the tile this thread loads
    const int lk = (tid & 3) * 4;     // first of its 4 k values
    const float* ap = (row0 + lr < row_end) ? P::a_row(a, grp, row0 + lr) : nullptr;
    const float* bp = (col0 + lr < ncols) ? P::b_row(a, grp, col0 + lr) : nullptr;
    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kSimtK) {
        float4 va = ap ? *reinterpret_cast<const float4*>(ap + k0 + lk) : make_float4(0, 0, 0, 0);
        float4 vb = bp ? *reinterpret_cast<const float4*>(bp + k0 + lk) : make_float4(0, 0, 0, 0);
        As[lk + 0][lr] = va.x; As[lk + 1][lr] = va.y; As[lk + 2][lr] = va.z; As[lk + 3][lr] = va.w;
        Bs[lk + 0][lr] = vb.x; Bs[lk + 1][lr] = vb.y; Bs[lk + 2][lr] = vb.z; Bs[lk + 3][lr] = vb.w;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kSimtK; ++k) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = As[k][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = row0 + ty * 4 + i, col = col0 + tx * 4 + j;
            if (row < row_end && col < ncols) P::store(a, grp, row, col, acc[i][j]);
        }
}

}  // namespace lmoe
