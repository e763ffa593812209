// combine.h -- the gate-weighted sum of a token's K expert outputs,
// accumulated in fp32 in a fixed order (aggregation in the latent space before the
// projection back: 10100.com article, section 2.2).  Latent mode writes s
// [T, l]; standard mode adds the residual and writes out [T, d] directly.
//
// The expert outputs sit in `nsplit` partial planes (the streaming FFN's
// m-slices; 1 for the tiled FFN) of [T*K, l] each.  `gated`: multiply by the
// gate here (streaming FFN) or not (the tiled FFN already did).
#pragma once

#include "layer.h"

namespace lmoe {

// Work item = (token t, 16-byte column chunk q of its l values): VPC = 8
// values for bf16 expert outputs, 4 for fp32.  A workgroup of 256 threads
// holds 256 / RS items, and RS rank groups per item: group g sums the ranks
// k = g, g + RS, ... in increasing order; the groups' sums are then added in
// group order through LDS, so the result does not depend on scheduling.
// RS = 1 (one thread per item) when there are enough tokens to fill the GPU,
// 4 or 16 for decode-sized batches.  The rank loop is unrolled so the loads
// of several ranks (and partial planes) are in flight together; no store
// happens before the last load.
template <class E, class YT, int RS>
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a, int nsplit, int gated) {
    constexpr int VPC = 16 / (int)sizeof(YT);
    constexpr int IPB = 256 / RS;
    const int cpt = a.l / VPC;
    const int item = blockIdx.x * IPB + (int)threadIdx.x % IPB;
    const int g = (int)threadIdx.x / IPB;
    const bool live = item < a.T * cpt;
    const int t = live ? item / cpt : 0, c0 = (live ? item % cpt : 0) * VPC;
    const size_t plane = (size_t)a.T * a.K * a.l;
    const YT* Y = static_cast<const YT*>(a.ybuf) + c0;
    float acc[VPC];
#pragma unroll
    for (int i = 0; i < VPC; ++i) acc[i] = 0.0f;
    if (live) {
        const int* so = a.slot_of + (size_t)t * a.K;
        const float* gt = a.gates + (size_t)t * a.K;
#pragma unroll 4
        for (int k = g; k < a.K; k += RS) {
            const YT* yp = Y + (size_t)so[k] * a.l;
            uint4 raw = ldg16(yp);
            float part[VPC];
            if constexpr (VPC == 8) {
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    part[2 * i] = __uint_as_float(w[i] << 16);
                    part[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                }
            } else {
                part[0] = __uint_as_float(raw.x);
                part[1] = __uint_as_float(raw.y);
                part[2] = __uint_as_float(raw.z);
                part[3] = __uint_as_float(raw.w);
                for (int sp = 1; sp < nsplit; ++sp) {
                    const uint4 q = ldg16(yp + sp * plane);
                    part[0] += __uint_as_float(q.x);
                    part[1] += __uint_as_float(q.y);
                    part[2] += __uint_as_float(q.z);
                    part[3] += __uint_as_float(q.w);
                }
            }
            const float gk = gated ? gt[k] : 1.0f;
#pragma unroll
            for (int i = 0; i < VPC; ++i) acc[i] = fmaf(gk, part[i], acc[i]);
        }
    }
    if constexpr (RS > 1) {
        __shared__ float red[RS][VPC][IPB];
#pragma unroll
        for (int i = 0; i < VPC; ++i) red[g][i][threadIdx.x % IPB] = acc[i];
        __syncthreads();
        if (g != 0) return;
#pragma unroll
        for (int i = 0; i < VPC; ++i) {
            float v = red[0][i][threadIdx.x];
            for (int r = 1; r < RS; ++r) v += red[r][i][threadIdx.x];
            acc[i] = v;
        }
    }
    if (!live) return;
    E* dst;
    if (a.standard) {
        // out = x + s (+ the shared expert's float32 output), rounded once
        const size_t o = (size_t)t * a.d + c0;
        const E* xp = static_cast<const E*>(a.x) + o;
#pragma unroll
        for (int i = 0; i < VPC; ++i) acc[i] += to_f32(xp[i]);
        if (a.y_s) {
#pragma unroll
            for (int i = 0; i < VPC; ++i) acc[i] += a.y_s[o + i];
        }
        dst = static_cast<E*>(a.out) + o;
    } else {
        dst = static_cast<E*>(a.s) + (size_t)t * a.l + c0;
    }
    // one vector store of the VPC values (rows are 16-byte aligned: l and d
    // are multiples of 64)
    E v[VPC];
#pragma unroll
    for (int i = 0; i < VPC; ++i) v[i] = from_f32<E>(acc[i]);
    if constexpr (sizeof(E) * VPC == 16)
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(v);
    else
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(v);
}

}  // namespace lmoe
