// combine.h -- the gate-weighted sum of a token's K expert outputs,
// accumulated in fp32 in a fixed order (aggregation in the latent space before the
// projection back: 10100.com article, section 2.2).  Latent mode writes s
// [T, l]; standard mode adds the residual and writes out [T, d] directly.
//
// PL: the streaming FFN's outputs, `nsplit` partial planes (its m-slices)
// of [T*K, l] each, multiplied by the gate here; otherwise the tiled FFN's
// single plane, already gate-scaled.  (A separate instantiation: the plane
// loop in the rank loop keeps the compiler from batching the ranks' loads.)
// YT: float (the float32 layer, tiled only) or f16 times kYScale (the bf16
// layer: the streaming FFN's partials, the tiled FFN's gate-scaled outputs;
// summed as they are, then scaled back once: a power of two, so no extra
// rounding).
// A rank's expert output is at its slot (slot_of, after a dispatch), or at
// row t*K + k of each plane when the streaming FFN routed itself
// (self_route).  Zero-computation experts (ids >= n_ffn) have no expert
// output.  After a dispatch their slots are the last ones (ids sort after
// the FFN experts), so a rank is theirs when its slot is at or past
// offsets[n_ffn], and such ranks read the planes' zero row; self-routed, a
// rank is theirs by its id, and its row (never written) is read and then
// discarded.  Either way the loads of all ranks stay unconditional, and a
// second pass over just those ranks adds their own g * y: nothing for a zero
// expert, g * z for a copy expert, g * its vector for a constant expert
// (MoE++'s three kinds: 10100.com article, section 3.2).
#pragma once

#include <type_traits>

#include "layer.h"

namespace lmoe {

// g * y of zero-computation expert q (counted from id n_ffn) for the VPC
// columns from c0 of token t, added to acc.
template <class E, int VPC>
__device__ inline void zc_add(const LayerArgs& a, int q, int t, int c0, float g, float* acc) {
    if (q < a.n_zero) return;   // zero expert: y = 0
    q -= a.n_zero;
    const E* y = q < a.n_copy ? static_cast<const E*>(a.z) + (size_t)t * a.l + c0                 // copy: z
                              : static_cast<const E*>(a.zc) + (size_t)(q - a.n_copy) * a.l + c0;  // constant
#pragma unroll
    for (int i = 0; i < VPC; ++i) acc[i] = fmaf(g, to_f32(y[i]), acc[i]);
}

// Work item = (token t, 16-byte column chunk q of its l values): VPC = 8
// values for bf16 expert outputs, 4 for fp32.  A workgroup of 256 threads
// holds 256 / RS items, and RS rank groups per item: group g sums the ranks
// k = g, g + RS, ... in increasing order; the groups' sums are then added in
// group order through LDS, so the result does not depend on scheduling.
// RS = 1 (one thread per item) when there are enough tokens to fill the GPU,
// 4 or 16 for decode-sized batches.  The rank loop is unrolled so the loads
// of several ranks (and partial planes) are in flight together; no store
// happens before the last load.
template <class E, class YT, int RS, bool PL>
__global__ __launch_bounds__(256) void combine_kernel(LayerArgs a, int nsplit) {
    static_assert(!PL || std::is_same<YT, f16>::value, "the streaming FFN's partials are scaled half precision");
    constexpr int VPC = 16 / (int)sizeof(YT);
    constexpr int IPB = 256 / RS;
    const int cpt = a.l / VPC;
    const int item = blockIdx.x * IPB + (int)threadIdx.x % IPB;
    const int g = (int)threadIdx.x / IPB;
    const bool live = item < a.T * cpt;
    const int t = live ? item / cpt : 0, c0 = (live ? item % cpt : 0) * VPC;
    const size_t plane = y_plane_elems(a);
    const YT* Y = static_cast<const YT*>(a.ybuf) + c0;
    float acc[VPC];
#pragma unroll
    for (int i = 0; i < VPC; ++i) acc[i] = 0.0f;
    if (live) {
        const int* so = a.slot_of + (size_t)t * a.K;
        const int* idk = a.ids + (size_t)t * a.K;
        const float* gt = a.gates + (size_t)t * a.K;
        const bool has_zc = a.N > a.n_ffn;
        const int nf = has_zc && !a.self_route ? a.offsets[a.n_ffn] : INT_MAX;   // FFN slots: [0, nf)
        const size_t zrow = (size_t)a.T * a.K;
        unsigned long long zranks = 0;   // ranks of zero-computation experts (K <= 64)
        if constexpr (!PL) {
            // (after a dispatch) the slots of a batch of 8 ranks are loaded
            // first, then their outputs: loads that alternated with the
            // slot loads would each wait for all the loads before them.
            // Ranks past K take the last rank's row (a cached re-read) and
            // are not added.
            constexpr int B = 8;
            for (int k0 = g; k0 < a.K; k0 += RS * B) {
                size_t row[B];
                bool z[B];
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int sl = so[min(k0 + u * RS, a.K - 1)];
                    z[u] = sl >= nf;
                    row[u] = z[u] ? zrow : (size_t)sl;
                }
                uint4 raw[B];
#pragma unroll
                for (int u = 0; u < B; ++u) raw[u] = ldg16(Y + row[u] * a.l);
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int k = k0 + u * RS;
                    if (k < a.K) {
                        zranks |= (unsigned long long)z[u] << k;
                        float part[VPC];
                        if constexpr (VPC == 8) {
                            const f32x8 f = __builtin_convertvector(__builtin_bit_cast(f16x8, raw[u]), f32x8);
#pragma unroll
                            for (int i = 0; i < 8; ++i) part[i] = f[i];
                        } else {
                            part[0] = __uint_as_float(raw[u].x);
                            part[1] = __uint_as_float(raw[u].y);
                            part[2] = __uint_as_float(raw[u].z);
                            part[3] = __uint_as_float(raw[u].w);
                        }
#pragma unroll
                        for (int i = 0; i < VPC; ++i) acc[i] += z[u] ? 0.0f : part[i];
                    }
                }
            }
        } else
#pragma unroll 4
        for (int k = g; k < a.K; k += RS) {
            size_t row;
            bool z;
            if (a.self_route) {
                row = (size_t)t * a.K + k;
                z = has_zc && idk[k] >= a.n_ffn;
            } else {
                const int sl = so[k];
                z = sl >= nf;
                row = z ? zrow : (size_t)sl;
            }
            zranks |= (unsigned long long)z << k;
            const YT* yp = Y + row * a.l;
            uint4 raw = ldg16(yp);
            float part[VPC];
            if constexpr (VPC == 8) {
                static_assert(std::is_same<YT, f16>::value, "2-byte expert outputs are scaled half precision");
                const f32x8 f = __builtin_convertvector(__builtin_bit_cast(f16x8, raw), f32x8);
#pragma unroll
                for (int i = 0; i < 8; ++i) part[i] = f[i];
                if constexpr (PL) {
                    // the other planes, loaded 8 at a time before they are
                    // added (in plane order)
                    for (int sp0 = 1; sp0 < nsplit; sp0 += 8) {
                        uint4 q[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            q[i] = sp0 + i < nsplit ? ldg16(yp + (sp0 + i) * plane) : kZero16;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            if (sp0 + i < nsplit) {
                                const f32x8 g8 = __builtin_convertvector(__builtin_bit_cast(f16x8, q[i]), f32x8);
#pragma unroll
                                for (int c = 0; c < 8; ++c) part[c] += g8[c];
                            }
                    }
                }
            } else {
                part[0] = __uint_as_float(raw.x);
                part[1] = __uint_as_float(raw.y);
                part[2] = __uint_as_float(raw.z);
                part[3] = __uint_as_float(raw.w);
            }
            const float gk = PL ? gt[k] : 1.0f;
#pragma unroll
            for (int i = 0; i < VPC; ++i) acc[i] = fmaf(gk, z ? 0.0f : part[i], acc[i]);
        }
        if constexpr (std::is_same<YT, f16>::value) {
#pragma unroll
            for (int i = 0; i < VPC; ++i) acc[i] *= kYUnscale;
        }
        while (zranks) {
            const int k = __builtin_ctzll(zranks);
            zranks &= zranks - 1;
            zc_add<E, VPC>(a, idk[k] - a.n_ffn, t, c0, gt[k], acc);
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
