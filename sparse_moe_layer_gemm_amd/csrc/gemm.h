// gemm.h -- the float32 GEMM over a LayerArgs "problem" (layer.h).
//
//   gemm_simt_kernel<P>: float32 everywhere, 64 x 64 x 16 tiles, 4 x 4
//     outputs per thread on the vector ALUs.  (bf16 products run on the
//     MFMA kernel of gemm2.h.)
//
// grid.x walks the problem's row tiles, grid.y its column tiles.
#pragma once

#include "layer.h"

namespace lmoe {

constexpr int kSimtM = 64, kSimtN = 64, kSimtK = 16;

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
