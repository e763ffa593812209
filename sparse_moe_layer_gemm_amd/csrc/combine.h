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

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
    p[0] = (bf16)v.x;
    p[1] = (bf16)v.y;
    p[2] = (bf16)v.z;
    p[3] = (bf16)v.w;
}

// One workgroup per (token, 256-column chunk): its 4 waves take the ranks
// k = w, w+4, ... and their partial sums are added in wave order through LDS,
// so the result does not depend on scheduling.
template <class E, class YT>
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a, int nsplit, int gated) {
    const int l = a.l;
    const int chunks = l / 256 + (l % 256 ? 1 : 0);
    const int t = blockIdx.x / chunks;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i0 = (blockIdx.x % chunks) * 256 + lane * 4;
    const bool live = i0 < l;
    const size_t plane = (size_t)a.T * a.K * l;
    const YT* Y = static_cast<const YT*>(a.ybuf);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        for (int k = wave; k < a.K; k += 4) {
            const size_t flat = (size_t)t * a.K + k;
            const YT* yp = Y + (size_t)a.slot_of[flat] * l + i0;
            float4 part = load4(yp);
            for (int sp = 1; sp < nsplit; ++sp) {
                const float4 q = load4(yp + sp * plane);
                part.x += q.x;
                part.y += q.y;
                part.z += q.z;
                part.w += q.w;
            }
            const float g = gated ? a.gates[flat] : 1.0f;
            acc.x = fmaf(g, part.x, acc.x);
            acc.y = fmaf(g, part.y, acc.y);
            acc.z = fmaf(g, part.z, acc.z);
            acc.w = fmaf(g, part.w, acc.w);
        }
    }
    __shared__ float4 red[4][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0 || !live) return;
    float4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const float4 q = red[w][lane];
        s.x += q.x;
        s.y += q.y;
        s.z += q.z;
        s.w += q.w;
    }
    if (a.standard) {
        const size_t o = (size_t)t * a.d + i0;
        const float4 xv = load4(static_cast<const E*>(a.x) + o);
        store4(static_cast<E*>(a.out) + o, make_float4(xv.x + s.x, xv.y + s.y, xv.z + s.z, xv.w + s.w));
    } else {
        store4(static_cast<E*>(a.s) + (size_t)t * l + i0, s);
    }
}

}  // namespace lmoe
