// stream.h -- kernels for few rows per weight matrix (decode shapes).
//
// With a handful of tokens per expert the layer is bound by reading weights
// from HBM once.  These kernels load MFMA operand fragments straight from
// global memory (both operands are contiguous along the reduction index, so
// a lane's 8 bf16 of a v_mfma_f32_16x16x32_bf16 operand are one 16-byte
// load) and keep many such loads in flight per wave.  The 16-row MFMA pads
// the few real rows; the extra arithmetic is free next to the weight stream.
//
//   skinny_kernel<P>: a product with T <= 256 rows.  One workgroup of 16
//     waves owns 16 output columns of a group of 64 rows; the waves split the
//     reduction and add their partial tiles through LDS.
//   skinny_part_kernel<P, NRB>: the same, with the reduction also split over
//     workgroups (fp32 partial tiles added by the consumer).
//   ffn_stream_kernel<MS, F>: the expert FFN.  Workgroup (s, a) takes
//     active expert a (from the dispatch, or, at T <= 256, found by the
//     workgroup itself from the top-K ids: expert_rows()) and the m-slice
//     [s*MS, (s+1)*MS) (MS = 64, 128, or 256 when there are enough
//     workgroups to go round): it computes
//     relu(W1[e][slice] z)^2 for up to 16 routed rows at a time, keeps it in
//     LDS, and multiplies it by the matching column slice of W2[e], writing
//     a partial expert output per slice (fp16 scaled by kYScale, like the
//     tiled path's outputs: half the bytes of fp32, 11 significant bits).  Every weight byte of an
//     active expert is read once per 16 rows; no atomics: the combine adds
//     the slices in a fixed order.  F: bf16, FP8 or MXFP4 weights.
//   ffn_stream_mx_kernel<MS>: the same for MXFP4 weights with 16-byte code
//     loads (32 codes per lane), for the usual shapes; MS = 128 or 256.
#pragma once

#include <type_traits>

#include "layer.h"

namespace lmoe {

constexpr int kSkinnyWaves = 16;
constexpr int kSkinnyMaxRows = 256;   // rows of a skinny product (in groups of 64)

template <class P>
__global__ __launch_bounds__(1024) void skinny_kernel(LayerArgs a) {
    const int c0 = blockIdx.x * 16, r0 = blockIdx.y * 64;   // 16 columns x a group of 64 rows
    const int ncols = P::ncols(a), K = P::kdim(a);
    const int K1 = k_first<P>(a);   // terms of the first operand pair (a multiple of 32)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nrb = min(4, cdiv(a.T - r0, 16));
    const int c = c0 + (lane & 15);
    const int koff = 8 * (lane >> 4);
    const bf16* bp = c < ncols ? P::b_row(a, 0, c) + koff : nullptr;
    const bf16* ap[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        const int r = r0 + rb * 16 + (lane & 15);
        ap[rb] = (rb < nrb && r < a.T) ? P::a_row(a, 0, r) + koff : nullptr;
    }
    f32x4 acc[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // k-steps [kb, ke) of 32 terms from rows b / ar (offset so that row + k0
    // addresses term k0)
    auto run = [&](const bf16* b, const bf16* const* ar, int kb, int ke) {
        for (int ks = kb; ks < ke; ks += 4) {
            uint4 bv[4], av[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k0 = (ks + u) * 32;
                const bool ok = ks + u < ke;
                bv[u] = (ok && b) ? ldg16(b + k0) : kZero16;
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) av[u][rb] = (ok && ar[rb]) ? ldg16(ar[rb] + k0) : kZero16;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    if (rb < nrb) acc[rb] = mfma16(as_bf16x8(av[u][rb]), as_bf16x8(bv[u]), acc[rb]);
        }
    };
    // the residual of this thread's outputs, loaded now so that its latency
    // overlaps the weight stream (the first nrb waves store the results)
    [[maybe_unused]] float res[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (HasResidual<P>::value) {
        if (threadIdx.x < nrb * 64) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = r0 + (threadIdx.x >> 6) * 16 + 4 * (lane >> 4) + r;
                if (row < a.T && c < ncols) res[r] = P::residual(a, row, c);
            }
        }
    }
    // the waves split each operand pair's k-steps evenly (the first pair's
    // split is the same as without a second pair)
    const int k1s = K1 / 32, per1 = cdiv(k1s, kSkinnyWaves);
    run(bp, ap, wave * per1, min(k1s, wave * per1 + per1));
    if constexpr (HasKSplit<P>::value) {
        const bf16* bp2 = bp ? P::b_row2(a, 0, c) + koff - K1 : nullptr;
        const bf16* ap2[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int r = r0 + rb * 16 + (lane & 15);
            ap2[rb] = ap[rb] ? P::a_row2(a, 0, r) + koff - K1 : nullptr;
        }
        const int k2s = (K - K1) / 32, per2 = cdiv(k2s, kSkinnyWaves);
        run(bp2, ap2, k1s + wave * per2, min(k1s + k2s, k1s + wave * per2 + per2));
    }

    __shared__ f32x4 red[kSkinnyWaves][4][64];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
        if (rb < nrb) red[wave][rb][lane] = acc[rb];
    __syncthreads();
    if (threadIdx.x < nrb * 64) {
        const int rb = threadIdx.x >> 6;
        f32x4 s = red[0][rb][lane];
        for (int w = 1; w < kSkinnyWaves; ++w) s += red[w][rb][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + rb * 16 + 4 * (lane >> 4) + r;
            if (row < a.T && c < ncols) {
                if constexpr (HasResidual<P>::value)
                    P::store_total(a, row, c, res[r] + s[r]);
                else
                    P::store(a, 0, row, c, s[r]);
            }
        }
    }
}

// z and the router logits for T <= 256 rows, split over the reduction so
// that enough workgroups stream the weights: workgroup (g, s, q) takes the
// 16 columns of group g, k-range s of `nsplit` and the NRB * 16 rows from
// q * NRB * 16 (NRB = 1, 2 or 4 row blocks, the fewest that hold min(T, 64)
// rows: no registers or MFMAs for row blocks that cannot hold a row); its 4
// waves split that range further and add their partial tiles through LDS,
// and the fp32 partial tile goes to part[s][T][stride].  A wave issues the
// loads of UB = 8 k-steps (4 with 4 row blocks) before their MFMAs, so the
// usual decode split (7 k-steps per wave) takes one round trip to memory.
// The top-K kernel adds the partials in split order (then the bias) and
// writes z.
template <class P, int NRB>
__global__ __launch_bounds__(256) void skinny_part_kernel(LayerArgs a, float* part, int nsplit, int stride) {
    constexpr int UB = NRB <= 2 ? 8 : 4;
    const int c0 = blockIdx.x * 16, s = blockIdx.y, r0 = blockIdx.z * (16 * NRB);
    const int ncols = P::ncols(a), K = P::kdim(a);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nrb = min(NRB, cdiv(a.T - r0, 16));
    const int ksteps = K / 32;
    const int kc = cdiv(ksteps, nsplit);
    const int kb = s * kc, ke = min(ksteps, kb + kc);
    const int per = cdiv(kc, 4);
    const int ks0 = kb + wave * per, ks1 = min(ke, ks0 + per);
    const int c = c0 + (lane & 15);
    const int koff = 8 * (lane >> 4);
    const bf16* bp = c < ncols ? P::b_row(a, 0, c) + koff : nullptr;
    const bf16* ap[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int r = r0 + rb * 16 + (lane & 15);
        ap[rb] = (rb < nrb && r < a.T) ? P::a_row(a, 0, r) + koff : nullptr;
    }
    f32x4 acc[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = ks0; ks < ks1; ks += UB) {
        uint4 bv[UB], av[UB][NRB];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int k0 = (ks + u) * 32;
            const bool ok = ks + u < ks1;
            bv[u] = (ok && bp) ? ldg16(bp + k0) : kZero16;
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) av[u][rb] = (ok && ap[rb]) ? ldg16(ap[rb] + k0) : kZero16;
        }
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb)
                if (rb < nrb) acc[rb] = mfma16(as_bf16x8(av[u][rb]), as_bf16x8(bv[u]), acc[rb]);
    }
    __shared__ f32x4 red[4][NRB][64];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
        if (rb < nrb) red[wave][rb][lane] = acc[rb];
    __syncthreads();
    const int rb = threadIdx.x >> 6;
    if (rb < nrb) {
        f32x4 v = red[0][rb][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) v += red[w][rb][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = r0 + rb * 16 + 4 * (lane >> 4) + r;
            if (row < a.T && c < ncols) part[((size_t)s * a.T + row) * stride + c] = v[r];
        }
    }
}

// The expert weights in 64-wide k blocks: lane group g = lane / 16 takes k =
// 16g .. 16g+15 of a block, its first 8 terms going to one MFMA and the next
// 8 to a second (the same grouping of the dot product for every weight
// format).  W64<F>::load takes the element offset of the lane's first term
// in the flattened weight matrix.
//   F = 0, bf16: two 16-byte loads per lane.
//   F = 1, FP8 E4M3: one 16-byte load of 16 codes, decoded to bf16 in
//          registers (the row scale is applied to the fp32 result).
//   F = 2, MXFP4: one 8-byte load of 16 E2M1 codes and their block's E8M0
//          scale byte (16 consecutive terms lie in one 32-element block),
//          decoded and scaled to bf16 in registers.
template <int F>
struct W64;

template <>
struct W64<0> {
    uint4 v[2];
    __device__ __forceinline__ static W64 load(const void* W, const uint8_t*, size_t off) {
        const bf16* p = static_cast<const bf16*>(W) + off;
        return W64{{ldg16(p), ldg16(p + 8)}};
    }
    __device__ __forceinline__ static W64 zero() { return W64{{kZero16, kZero16}}; }
    __device__ __forceinline__ bf16x8 frag(int h) const { return as_bf16x8(v[h]); }
};

template <>
struct W64<1> {
    uint4 v;
    __device__ __forceinline__ static W64 load(const void* W, const uint8_t*, size_t off) {
        return W64{ldg16(static_cast<const uint8_t*>(W) + off)};
    }
    __device__ __forceinline__ static W64 zero() { return W64{kZero16}; }
    __device__ __forceinline__ bf16x8 frag(int h) const {
        return as_bf16x8(e4m3x8_to_bf16x8(h ? uint2{v.z, v.w} : uint2{v.x, v.y}));
    }
};

template <>
struct W64<2> {
    uint2 c;
    float s;
    __device__ __forceinline__ static W64 load(const void* W, const uint8_t* S, size_t off) {
        return W64{ldg8(static_cast<const uint8_t*>(W) + off / 2), e8m0_to_f32(ldg1(S + off / 32))};
    }
    __device__ __forceinline__ static W64 zero() { return W64{uint2{0u, 0u}, 1.0f}; }
    __device__ __forceinline__ bf16x8 frag(int h) const { return as_bf16x8(fp4x8_to_bf16x8(h ? c.y : c.x, s)); }
};

// Workgroup -> (slice, active expert) for MXFP4 experts.  With an even
// slice count, slices 2k and 2k+1 of an expert are placed 8 workgroups
// apart -- on the same XCD (workgroups go to the 8 XCDs in turn): a 128-wide
// slice of an MXFP4 W2 row is 64 bytes, half a 128-byte line, and that
// XCD's L2 then fetches each line once.  The grid's y extent is a multiple
// of 8 (every chunk of 16 workgroups whole).
__device__ inline void paired_slices(int& slice, int& ai) {
    const int ns = gridDim.x;
    if (ns % 2 == 0) {
        const int L = blockIdx.y * ns + blockIdx.x;
        const int q = (L / 16) * 8 + (L % 8);   // (expert, slice pair) index
        ai = q / (ns / 2);
        slice = 2 * (q % (ns / 2)) + (L % 16) / 8;
    } else {
        slice = blockIdx.x, ai = blockIdx.y;
    }
}

// The rows of one streaming-FFN workgroup's expert.  With a dispatch: the
// expert is active expert ai (active experts in ascending id order), its
// rows the slots offsets[e] .. offsets[e+1] (perm gives each slot's pair
// t*K + k, and the output row is the slot).
// Self-routed (T <= 256, no dispatch): the workgroup reads all T*K routed ids
// (coalesced, into LDS) and finds the same active-expert order itself: a bit
// per FFN expert that any token names, then the ai-th set bit.  So the grid
// maps to active experts exactly as after a dispatch (workgroups past the
// active count return at once, and every XCD gets an even share of the real
// work).  A token names an expert at most once, so list[t] = the pair t*K + k
// naming e (or none) gives the expert's rows in token order; compacted with
// a ballot per wave, the pair indices are both the row's token (pair / K)
// and its output row.
struct ExpertRows {
    int e, n, base;
    const int* list;   // self-routed: n pair indices in LDS; else nullptr
    __device__ int pair(const LayerArgs& a, int i) const { return list ? list[i] : a.perm[base + i]; }
    __device__ int out_row(int i) const { return list ? list[i] : base + i; }
};

constexpr int kSelfRouteMaskWords = 64;   // FFN experts / 32 (at most 2048 experts)

struct SelfRouteLds {
    uint32_t amask[kSelfRouteMaskWords];   // FFN experts named by any token
    int list[kSkinnyMaxRows];
    int wcnt[4];
    int e, n_active;
};

// Dynamic LDS bytes of a streaming-FFN launch: the routed ids as 16-bit
// values when self-routed.
inline size_t self_route_lds_bytes(int T, int K, bool self_route) {
    return self_route ? ((size_t)T * K * 2 + 15) / 16 * 16 : 0;
}

// false: the workgroup has no rows (the same in every thread: return).
// L: LDS; ids16: dynamic LDS of T*K 16-bit ids (self-routed).  256 threads.
__device__ inline bool expert_rows(const LayerArgs& a, int ai, SelfRouteLds& L, uint16_t* ids16,
                                   ExpertRows& r) {
    if (!a.self_route) {
        if (ai >= *a.n_active) return false;
        r.e = a.active[ai];
        r.base = a.offsets[r.e];
        r.n = a.offsets[r.e + 1] - r.base;
        r.list = nullptr;
        return true;
    }
    if (ai >= a.n_ffn) return false;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int tk = a.T * a.K, nw = cdiv(a.n_ffn, 32);
    if (t < kSelfRouteMaskWords) L.amask[t] = 0u;
    L.list[t] = -1;
    __syncthreads();
    // the ids, 8 coalesced loads per thread in flight at a time
    for (int p0 = t; p0 < tk; p0 += 8 * 256) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = a.ids[min(p0 + 256 * u, tk - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = p0 + 256 * u;
            if (p < tk) {
                ids16[p] = (uint16_t)v[u];
                if (v[u] < a.n_ffn) atomicOr(&L.amask[v[u] >> 5], 1u << (v[u] & 31));
            }
        }
    }
    __syncthreads();
    // wave 0: the ai-th set bit of the mask (prefix count of set bits over
    // the words, one word per lane)
    if (wave == 0) {
        const uint32_t w = lane < nw ? L.amask[lane] : 0u;
        const int c = __popc(w);
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (lane == 63) L.n_active = incl;
        if (ai >= incl - c && ai < incl) {
            uint32_t x = w;
            for (int i = incl - c; i < ai; ++i) x &= x - 1;   // drop the lower set bits
            L.e = lane * 32 + __builtin_ctz(x);
        }
    }
    __syncthreads();
    if (ai >= L.n_active) return false;
    const int e = L.e;
    for (int p = t; p < tk; p += 256)
        if (ids16[p] == e) L.list[p / a.K] = p;
    __syncthreads();
    const int pair = L.list[t];
    __syncthreads();
    const unsigned long long m = __ballot(pair >= 0);
    if (lane == 0) L.wcnt[wave] = __popcll(m);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int c = L.wcnt[w];
        before += w < wave ? c : 0;
        total += c;
    }
    if (pair >= 0) {
        const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
        L.list[before + __popcll(m & below)] = pair;
    }
    __syncthreads();
    r.e = e;
    r.n = total;
    r.base = 0;
    r.list = L.list;
    return true;
}

// F: the expert weights' format (0 bf16, 1 FP8 E4M3 with one float32 scale
// per weight row applied to that row's fp32 result, 2 MXFP4 -- the shapes
// ffn_stream_mx_kernel does not take).
template <int MS, int F>
__global__ __launch_bounds__(256) void ffn_stream_kernel(LayerArgs a) {
    using WB = W64<F>;
    int slice, ai;
    if constexpr (F == 2)
        paired_slices(slice, ai);
    else
        slice = blockIdx.x, ai = blockIdx.y;
    __shared__ SelfRouteLds srl;
    extern __shared__ uint16_t ids16[];
    ExpertRows er;
    if (!expert_rows(a, ai, srl, ids16, er)) return;
    const int e = er.e;
    const int j0 = slice * MS;
    const int l = a.l, m = a.m;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 15, k16 = 16 * (lane >> 4);
    const bf16* Z = static_cast<const bf16*>(a.z);
    f16* Yp = static_cast<f16*>(a.ybuf) + (size_t)slice * y_plane_elems(a);   // scaled by kYScale

    constexpr int NB = MS / 16;        // 16-column blocks of the slice
    constexpr int NBW = NB / 4;        // per wave
    constexpr int AST = MS + 8;        // LDS row stride (bf16), padded
    // 64-wide k blocks per batch of phase-1 loads (MXFP4 loads move a
    // quarter of the bf16 bytes per block: more blocks per batch)
    constexpr int NKB = F == 2 ? 4 : 2;
    __shared__ bf16 As[16 * AST];

    for (int rc = 0; rc < er.n; rc += 16) {
        const int nr = min(16, er.n - rc);
        // ---- phase 1: H[16 x MS] = Z[rows] . W1[e][j0 : j0+MS]^T, reduce over l
        const int my_row = rc + min(lr, nr - 1);
        const size_t orow = (size_t)er.out_row(my_row) * l;   // the lane's output row (lanes lr < nr)
        const bf16* zp = Z + (size_t)(er.pair(a, my_row) / a.K) * l + k16;
        size_t w1o[NBW];   // element offset of the lane's W1 row, at its k16
#pragma unroll
        for (int b = 0; b < NBW; ++b) w1o[b] = ((size_t)e * m + j0 + (wave + 4 * b) * 16 + lr) * l + k16;
        f32x4 acc[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < l; k0 += 64 * NKB) {
            uint4 zv[NKB][2];
            WB wv[NKB][NBW];
#pragma unroll
            for (int p = 0; p < NKB; ++p) {
                const int kb = k0 + 64 * p;
                const bool ok = kb < l;   // l is a multiple of 64
                zv[p][0] = ok ? ldg16(zp + kb) : kZero16;
                zv[p][1] = ok ? ldg16(zp + kb + 8) : kZero16;
#pragma unroll
                for (int b = 0; b < NBW; ++b) wv[p][b] = ok ? WB::load(a.W1, a.w1x, w1o[b] + kb) : WB::zero();
            }
#pragma unroll
            for (int p = 0; p < NKB; ++p)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int b = 0; b < NBW; ++b)
                        acc[b] = mfma16(as_bf16x8(zv[p][h]), wv[p][b].frag(h), acc[b]);
        }
        if constexpr (F == 1) {
            // lane's column j0 + (wave + 4b) * 16 + lr: one W1 row scale
#pragma unroll
            for (int b = 0; b < NBW; ++b) acc[b] *= a.w1s[(size_t)e * m + j0 + (wave + 4 * b) * 16 + lr];
        }
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float h = acc[b][r] > 0.0f ? acc[b][r] : 0.0f;
                As[(4 * (lane >> 4) + r) * AST + (wave + 4 * b) * 16 + lr] = (bf16)(h * h);
            }
        // FP8: the first pass's W2 blocks do not depend on phase 1, so their
        // loads are issued before the barrier and the phase change does not
        // wait for them (for bf16 and MXFP4 weights the extra registers would
        // cost a wave per SIMD; measured slower for bf16)
        constexpr int KB = MS / 64;        // 64-wide k blocks of the slice
        constexpr int NU = MS == 256 ? 2 : 4;   // blocks per pass (fewer for the wider slice's k blocks)
        constexpr bool kPre = F == 1;
        const int nblk = l / 16;
        [[maybe_unused]] WB w0[NU][KB];
        [[maybe_unused]] f32x4 sc0[NU];
#pragma unroll
        for (int u = 0; u < NU && kPre; ++u) {
            const int ib = wave + 4 * u;
            const bool ok = ib < nblk;
            const size_t w2o = ((size_t)e * l + ib * 16 + lr) * m + j0 + k16;
#pragma unroll
            for (int q = 0; q < KB; ++q) w0[u][q] = ok ? WB::load(a.W2, a.w2x, w2o + 64 * q) : WB::zero();
            if constexpr (F == 1)
                sc0[u] = ok ? *reinterpret_cast<const f32x4*>(a.w2s + (size_t)e * l + ib * 16 + 4 * (lane >> 4))
                            : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        // ---- phase 2: Y[16 x l] = A[16 x MS] . W2[e][:, j0 : j0+MS]^T.  The
        // weight fragment is the MFMA's first operand, so lane l holds output
        // columns i0 + 4 (l / 16) .. +3 of row l % 16: one 16-byte store.
        // A pass loads NU blocks of 16 output columns; the results of NP
        // passes are stored together, since a load issued behind pending
        // stores waits for them to complete (the stores cost the kernel more
        // time than their bytes: without them the decode FFN ran 17 µs
        // faster).  bf16 weights in 256-wide slices: 8 passes, a wave's 16
        // blocks of the usual l = 1024 in one batch, so that its stores come
        // after all of its loads; 128-wide slices: 4 (their 4 blocks per pass
        // would need 128 more registers); fewer for FP8 (4 at 256-wide
        // slices, else 2) and MXFP4, whose decode registers would otherwise
        // cut the waves per SIMD.
        constexpr int NP = F == 0 ? (MS == 256 ? 8 : 4) : (F == 1 ? (MS == 256 ? 4 : 2) : 1);
        bf16x8 af[KB][2];
#pragma unroll
        for (int q = 0; q < KB; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                af[q][h] = *reinterpret_cast<const bf16x8*>(&As[lr * AST + 64 * q + k16 + 8 * h]);
        // a wave takes blocks wave + 4 (NU it + u), NP passes it per batch
        for (int ib0 = wave; ib0 < nblk; ib0 += 4 * NU * NP) {
            f32x4 yb[NP][NU];
#pragma unroll
            for (int it = 0; it < NP; ++it) {
                WB wv[NU][KB];
                f32x4 sc[NU];
                if (kPre && it == 0 && ib0 == wave) {
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
#pragma unroll
                        for (int q = 0; q < KB; ++q) wv[u][q] = w0[u][q];
                        if constexpr (F == 1) sc[u] = sc0[u];
                    }
                } else
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const int ib = ib0 + 4 * (NU * it + u);
                    const bool ok = ib < nblk;
                    const size_t w2o = ((size_t)e * l + ib * 16 + lr) * m + j0 + k16;
#pragma unroll
                    for (int q = 0; q < KB; ++q) wv[u][q] = ok ? WB::load(a.W2, a.w2x, w2o + 64 * q) : WB::zero();
                    if constexpr (F == 1) {
                        // the lane's 4 output rows ib*16 + 4 (lane/16) .. +3 of W2
                        sc[u] = ok ? *reinterpret_cast<const f32x4*>(a.w2s + (size_t)e * l + ib * 16 + 4 * (lane >> 4))
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
                    }
                }
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < KB; ++q)
#pragma unroll
                        for (int h = 0; h < 2; ++h) y = mfma16(wv[u][q].frag(h), af[q][h], y);
                    if constexpr (F == 1) y *= sc[u];
                    yb[it][u] = y;
                }
            }
            if (lr < nr) {
#pragma unroll
                for (int it = 0; it < NP; ++it)
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        const int ib = ib0 + 4 * (NU * it + u);
                        if (ib < nblk)
                            *reinterpret_cast<uint2*>(&Yp[orow + ib * 16 + 4 * (lane >> 4)]) =
                                pack4_f16_sat(yb[it][u] * kYScale);
                    }
            }
        }
        __syncthreads();
    }
}

// MXFP4 experts, 16-byte code loads: lane group g = lane / 16 takes the 32
// consecutive terms 32g .. 32g+31 of each 128-wide k block -- 16 code bytes,
// all in one 32-element scale block -- and word q of them (terms 32g + 8q ..
// +7) goes to MFMA q of the block.  Each load instruction then reads 64
// contiguous bytes of each of 16 weight rows, with as many bytes per
// instruction as the FP8 kernel.  (This groups the dot products' terms
// differently from ffn_stream_kernel.)  Needs l % 256 == 0 and m % MS == 0;
// in phase 2 a W2 row's slice is MS / 128 such blocks.  The scale bytes of a
// lane's row come as one vector per batch (8 bytes in phase 1, MS / 32 in
// phase 2).  With MS = 256 a W2 row's slice is a whole 128-byte line, so no
// slice pairing across XCDs is needed (paired_slices() keeps the plain
// order for the odd slice count of m = 768, and pairs otherwise).
template <int MS>
__global__ __launch_bounds__(256) void ffn_stream_mx_kernel(LayerArgs a) {
    constexpr int NBW = MS / 64, AST = MS + 8;
    constexpr int KC = MS / 128;   // 128-term chunks of a W2 row's slice
    constexpr int NSB = 2;   // 128-wide k blocks per batch of phase-1 loads
    int slice, ai;
    paired_slices(slice, ai);
    __shared__ SelfRouteLds srl;
    extern __shared__ uint16_t ids16[];
    ExpertRows er;
    if (!expert_rows(a, ai, srl, ids16, er)) return;
    const int e = er.e;
    const int j0 = slice * MS;
    const int l = a.l, m = a.m;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & 15, g = lane >> 4;
    const uint8_t* W1 = static_cast<const uint8_t*>(a.W1);
    const uint8_t* W2 = static_cast<const uint8_t*>(a.W2);
    const bf16* Z = static_cast<const bf16*>(a.z);
    f16* Yp = static_cast<f16*>(a.ybuf) + (size_t)slice * y_plane_elems(a);   // scaled by kYScale
    __shared__ bf16 As[16 * AST];
    auto decode = [](uint32_t word, uint32_t scale_byte) {
        return as_bf16x8(fp4x8_to_bf16x8(word, e8m0_to_f32(scale_byte & 0xffu)));
    };

    for (int rc = 0; rc < er.n; rc += 16) {
        const int nr = min(16, er.n - rc);
        // ---- phase 1: H[16 x MS] = Z[rows] . W1[e][j0 : j0+MS]^T, reduce over l
        const int my_row = rc + min(lr, nr - 1);
        const size_t orow = (size_t)er.out_row(my_row) * l;   // the lane's output row (lanes lr < nr)
        const bf16* zp = Z + (size_t)(er.pair(a, my_row) / a.K) * l + 32 * g;
        size_t w1e[NBW];   // element offset of the lane's W1 row
#pragma unroll
        for (int b = 0; b < NBW; ++b) w1e[b] = ((size_t)e * m + j0 + (wave + 4 * b) * 16 + lr) * l;
        f32x4 acc[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < l; k0 += 128 * NSB) {   // l % 256 == 0: every block is whole
            uint2 sv[NBW];          // the row's 8 scale bytes of these 256 terms
            uint4 cv[NSB][NBW];     // 32 codes per block and row
            uint4 zv[NSB][4];       // the matching 32 terms of z
#pragma unroll
            for (int b = 0; b < NBW; ++b) sv[b] = ldg8(a.w1x + (w1e[b] + k0) / 32);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const int kb = k0 + 128 * sb;
#pragma unroll
                for (int q = 0; q < 4; ++q) zv[sb][q] = ldg16(zp + kb + 8 * q);
#pragma unroll
                for (int b = 0; b < NBW; ++b) cv[sb][b] = ldg16(W1 + (w1e[b] + kb) / 2 + 16 * g);
            }
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int b = 0; b < NBW; ++b) {
                    // block sb, lane group g: scale byte 4 sb + g
                    const uint32_t sc = (sb == 0 ? sv[b].x : sv[b].y) >> (8 * g);
                    const uint32_t w[4] = {cv[sb][b].x, cv[sb][b].y, cv[sb][b].z, cv[sb][b].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[b] = mfma16(as_bf16x8(zv[sb][q]), decode(w[q], sc), acc[b]);
                }
        }
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float h = acc[b][r] > 0.0f ? acc[b][r] : 0.0f;
                As[(4 * (lane >> 4) + r) * AST + (wave + 4 * b) * 16 + lr] = (bf16)(h * h);
            }
        __syncthreads();
        // ---- phase 2: Y[16 x l] = A[16 x MS] . W2[e][:, j0 : j0+MS]^T, the
        // weight fragment as the MFMA's first operand (lane l: output columns
        // i0 + 4 (l / 16) .. +3 of row l % 16, one 16-byte store), one pass
        // of NU blocks of 16 output columns per batch of stores
        constexpr int NU = 4;
        bf16x8 af[KC][4];
#pragma unroll
        for (int c = 0; c < KC; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                af[c][q] = *reinterpret_cast<const bf16x8*>(&As[lr * AST + 128 * c + 32 * g + 8 * q]);
        const int nblk = l / 16;
        for (int ib0 = wave; ib0 < nblk; ib0 += 4 * NU) {
            uint4 cv[NU][KC];
            uint2 sb[NU];   // the row slice's scale bytes (4 per 128-term chunk)
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int ib = ib0 + 4 * u;
                const bool ok = ib < nblk;
                const size_t w2e = ((size_t)e * l + ib * 16 + lr) * m + j0;   // the row's slice
#pragma unroll
                for (int c = 0; c < KC; ++c) cv[u][c] = ok ? ldg16(W2 + (w2e + 128 * c) / 2 + 16 * g) : kZero16;
                if constexpr (KC == 1)
                    sb[u] = uint2{ok ? ldg4(a.w2x + w2e / 32) : 0x7f7f7f7fu, 0u};
                else
                    sb[u] = ok ? ldg8(a.w2x + w2e / 32) : uint2{0x7f7f7f7fu, 0x7f7f7f7fu};
            }
            f32x4 yb[NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < KC; ++c) {
                    const uint32_t sc = (c == 0 ? sb[u].x : sb[u].y) >> (8 * g);
                    const uint32_t w[4] = {cv[u][c].x, cv[u][c].y, cv[u][c].z, cv[u][c].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) y = mfma16(decode(w[q], sc), af[c][q], y);
                }
                yb[u] = y;
            }
            if (lr < nr) {
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const int ib = ib0 + 4 * u;
                    if (ib < nblk)
                        *reinterpret_cast<uint2*>(&Yp[orow + ib * 16 + 4 * (lane >> 4)]) =
                            pack4_f16_sat(yb[u] * kYScale);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace lmoe
