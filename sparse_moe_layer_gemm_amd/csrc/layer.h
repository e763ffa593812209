// layer.h -- the arguments every kernel of the layer sees, and the four
// matrix products of the layer expressed as "problems" that the GEMM kernels
// (tiled MFMA for bf16, SIMT for float32) instantiate.
//
// Every product has the form C[r, c] = epilogue(sum_k A[r, k] * B[c, k]):
// both operands are read along their contiguous reduction index.
#pragma once

#include <type_traits>
#include <utility>

#include "common.h"

namespace lmoe {

struct LayerArgs {
    // caller tensors
    const void* x;         // [T, d]
    const void* W_down;    // [l, d] or NULL (standard mode)
    const void* W_router;  // [N, d]: one row per routed id
    const void* W1;        // [N, m, l]
    const void* W2;        // [N, l, m]
    const void* W_up;      // [d, l] or NULL (standard mode)
    const void* W_s1;      // [m_s, d] shared expert, or NULL
    const void* W_s2;      // [d, m_s]
    const float* bias;     // [N] or NULL
    const void* zc;        // [n_const, l] constant experts' vectors, or NULL
    const float* w1s;      // [N, m] row scales of FP8 W1 (FP8 experts only)
    const float* w2s;      // [N, l] row scales of FP8 W2
    const uint8_t* w1x;    // [N, m, l/32] E8M0 block scales of MXFP4 W1 (MXFP4 experts only)
    const uint8_t* w2x;    // [N, l, m/32] E8M0 block scales of MXFP4 W2
    void* out;             // [T, d]
    int T, d, l, N, m, K;  // N: routed ids (FFN experts, then zero-computation experts)
    int n_ffn;             // FFN experts: ids < n_ffn have W1 / W2
    int n_zero, n_copy;    // zero experts, then copy experts, then constant experts
    int standard;
    int m_s;               // shared expert width (0: none)
    // workspace
    const void* z;         // [T, l] latent tokens (== x in standard mode)
    void* z_w;             // writable view of z (latent mode)
    float* logits;         // [T, N]
    int32_t* ids;          // [T, K]
    float* gates;          // [T, K]
    int32_t* counts;       // [N]
    int32_t* offsets;      // [N + 1]
    int32_t* perm;         // [T*K] slot -> t*K + k
    int32_t* slot_of;      // [T*K] t*K + k -> slot
    int32_t* blk_counts;   // [nblk, N]
    int32_t* blk_offsets;  // [nblk, N]
    int2* tiles;           // grouped-GEMM row tiles: (expert, first slot)
    int32_t* n_tiles;
    // tall_rows > 0: `tiles` lists only the experts with at most tile_rows
    // rows; the others get row tiles of tall_rows rows in tiles_tall, run on
    // the larger GEMM tile (their weights and gathered rows are then read by
    // half as many tiles)
    int2* tiles_tall;
    int32_t* n_tiles_tall;
    int tall_rows;
    int32_t* active;       // experts with rows, ascending
    int32_t* n_active;
    void* abuf;            // [T*K, m] relu(h)^2
    void* ybuf;            // expert outputs: fp16 times kYScale in the bf16 layer (the streaming
                           // FFN's per-slice partials, the tiled FFN's gate-scaled outputs),
                           // float32 in the float32 layer
    void* s;               // [T, l] gate-weighted latent sum (latent mode)
    void* part;            // split-reduction partial tiles of the skinny projection
    void* a_s;             // [T, m_s] relu(W_s1 x)^2 (shared expert)
    float* y_s;            // [T, d] W_s2 a_s, float32 (shared expert)
    // split-reduction tail of a tiled product (gemm2.h, Tail<P>): its last
    // tiles, from tile tail_base on, each reduced by tail_s workgroups into
    // fp32 partial tiles that tail_fixup_kernel adds and finishes
    float* tail_part;      // [tiles][tail_s][BM][BN]
    int tail_base, tail_s, tail_ncol;   // first split tile, split count, column tiles
    int tile_rows;         // rows per grouped-GEMM tile
    int y_planes;          // partial planes of ybuf (the streaming FFN's m-slices; 1 for the tiled FFN)
    int y_row_bytes;       // bytes of one ybuf row (l elements)
    // The streaming FFN for T <= 256 finds each expert's rows from ids
    // itself (no dispatch arrays): expert outputs are then stored at row
    // t*K + k of each plane, which the combine reads directly.
    int self_route;
};

// Elements of one ybuf plane: a row per slot (per pair t*K + k when
// self_route) and one more (row T*K), kept at zero when there are
// zero-computation experts and a dispatch, whose ranks read it in place of an
// expert output.
__device__ inline size_t y_plane_elems(const LayerArgs& a) { return ((size_t)a.T * a.K + 1) * a.l; }

// ---------------------------------------------------------------------------
// z = W_down x, the shared expert's a_s = relu(W_s1 x)^2 and logits =
// W_router x (+ bias): one product of x over the concatenated columns
// [z | h_s | logits] (z: l columns, none in standard mode; h_s: m_s
// columns, none without a shared expert; both multiples of 64, so no group
// of 4 columns straddles two parts).

__device__ inline int proj_lz(const LayerArgs& a) { return a.standard ? 0 : a.l; }

template <class E>
struct ProjRouter {
    using BElem = E;   // element type of the B (weight) rows
    __device__ static bool tile(const LayerArgs& a, int bx, int bm, int& grp, int& row0, int& row_end) {
        grp = 0;
        row0 = bx * bm;
        row_end = a.T;
        return row0 < row_end;
    }
    // row tiles of this launch: the host's count
    __device__ static int row_tiles(const LayerArgs&, int host_count) { return host_count; }
    __device__ static int ncols(const LayerArgs& a) { return proj_lz(a) + a.m_s + a.N; }
    __device__ static int kdim(const LayerArgs& a) { return a.d; }
    __device__ static const E* a_row(const LayerArgs& a, int, int r) {
        return static_cast<const E*>(a.x) + (size_t)r * a.d;
    }
    __device__ static const E* b_row(const LayerArgs& a, int, int c) {
        const int lz = proj_lz(a), le = lz + a.m_s;
        return c < lz   ? static_cast<const E*>(a.W_down) + (size_t)c * a.d
               : c < le ? static_cast<const E*>(a.W_s1) + (size_t)(c - lz) * a.d
                        : static_cast<const E*>(a.W_router) + (size_t)(c - le) * a.d;
    }
    __device__ static void store(const LayerArgs& a, int, int r, int c, float v) {
        const int lz = proj_lz(a), le = lz + a.m_s;
        if (c < lz) {
            static_cast<E*>(a.z_w)[(size_t)r * a.l + c] = from_f32<E>(v);
        } else if (c < le) {
            const float t = v > 0.0f ? v : 0.0f;
            static_cast<E*>(a.a_s)[(size_t)r * a.m_s + (c - lz)] = from_f32<E>(t * t);
        } else {
            const int e = c - le;
            a.logits[(size_t)r * a.N + e] = v + (a.bias ? a.bias[e] : 0.0f);
        }
    }
};

// Expert FFN, first product: h = W1[e] z for the rows routed to e, then
// relu(h)^2.  Row r of a tile is slot r; its token is perm[r] / K.
template <class E>
struct Ffn1 {
    using BElem = E;   // element type of the B (weight) rows
    __device__ static bool tile(const LayerArgs& a, int bx, int, int& grp, int& row0, int& row_end) {
        if (bx >= *a.n_tiles) return false;
        const int2 t = a.tiles[bx];
        grp = t.x;
        row0 = t.y;
        row_end = a.offsets[grp + 1];
        return true;
    }
    // the tile list's length, known only on the device (the host passes a bound)
    __device__ static int row_tiles(const LayerArgs& a, int) { return *a.n_tiles; }
    __device__ static int ncols(const LayerArgs& a) { return a.m; }
    __device__ static int kdim(const LayerArgs& a) { return a.l; }
    __device__ static const E* a_row(const LayerArgs& a, int, int slot) {
        const int t = a.perm[slot] / a.K;
        return static_cast<const E*>(a.z) + (size_t)t * a.l;
    }
    __device__ static const E* b_row(const LayerArgs& a, int e, int c) {
        return static_cast<const E*>(a.W1) + ((size_t)e * a.m + c) * a.l;
    }
    __device__ static void store(const LayerArgs& a, int, int slot, int c, float v) {
        const float r = v > 0.0f ? v : 0.0f;
        static_cast<E*>(a.abuf)[(size_t)slot * a.m + c] = from_f32<E>(r * r);
    }
};

// Expert FFN, second product: y = W2[e] a, scaled by the slot's gate
// (so the combine only sums).  YT: storage type of the expert outputs
// (float for the float32 layer; f16 scaled by kYScale for the bf16 layer's
// tiled path, whose epilogue is RowCtx<Ffn2<bf16, f16>> in gemm2.h).
template <class E, class YT>
struct Ffn2 {
    using BElem = E;
    __device__ static bool tile(const LayerArgs& a, int bx, int bm, int& grp, int& row0, int& row_end) {
        return Ffn1<E>::tile(a, bx, bm, grp, row0, row_end);
    }
    __device__ static int row_tiles(const LayerArgs& a, int b) { return Ffn1<E>::row_tiles(a, b); }
    __device__ static int ncols(const LayerArgs& a) { return a.l; }
    __device__ static int kdim(const LayerArgs& a) { return a.m; }
    __device__ static const E* a_row(const LayerArgs& a, int, int slot) {
        return static_cast<const E*>(a.abuf) + (size_t)slot * a.m;
    }
    __device__ static const E* b_row(const LayerArgs& a, int e, int c) {
        return static_cast<const E*>(a.W2) + ((size_t)e * a.l + c) * a.m;
    }
    __device__ static void store(const LayerArgs& a, int, int slot, int c, float v) {
        const float g = a.gates[a.perm[slot]];
        static_cast<YT*>(a.ybuf)[(size_t)slot * a.l + c] = from_f32<YT>(g * v);
    }
};

// out = x + W_up s.
template <class E>
struct Up {
    using BElem = E;   // element type of the B (weight) rows
    __device__ static bool tile(const LayerArgs& a, int bx, int bm, int& grp, int& row0, int& row_end) {
        grp = 0;
        row0 = bx * bm;
        row_end = a.T;
        return row0 < row_end;
    }
    __device__ static int row_tiles(const LayerArgs&, int host_count) { return host_count; }
    __device__ static int ncols(const LayerArgs& a) { return a.d; }
    __device__ static int kdim(const LayerArgs& a) { return a.l; }
    __device__ static const E* a_row(const LayerArgs& a, int, int r) {
        return static_cast<const E*>(a.s) + (size_t)r * a.l;
    }
    __device__ static const E* b_row(const LayerArgs& a, int, int c) {
        return static_cast<const E*>(a.W_up) + (size_t)c * a.l;
    }
    __device__ static void store(const LayerArgs& a, int, int r, int c, float v) {
        const size_t i = (size_t)r * a.d + c;
        static_cast<E*>(a.out)[i] = from_f32<E>(to_f32(static_cast<const E*>(a.x)[i]) + v);
    }
    // the same split in two, for kernels that load the residual early
    __device__ static float residual(const LayerArgs& a, int r, int c) {
        return to_f32(static_cast<const E*>(a.x)[(size_t)r * a.d + c]);
    }
    __device__ static void store_total(const LayerArgs& a, int r, int c, float t) {
        static_cast<E*>(a.out)[(size_t)r * a.d + c] = from_f32<E>(t);
    }
};

// Problems whose output adds a residual that a kernel may load early
// (residual(a, r, c), then store_total(a, r, c, residual + v)).
template <class P, class = void>
struct HasResidual : std::false_type {};
template <class P>
struct HasResidual<P, decltype((void)P::residual(std::declval<const LayerArgs&>(), 0, 0))> : std::true_type {};

// Shared expert, second product: y_s = W_s2 a_s, kept in float32 so that the
// layer's output is still rounded once (in the up-projection or combine).
template <class E>
struct Shared2 {
    using BElem = E;   // element type of the B (weight) rows
    __device__ static bool tile(const LayerArgs& a, int bx, int bm, int& grp, int& row0, int& row_end) {
        return Up<E>::tile(a, bx, bm, grp, row0, row_end);
    }
    __device__ static int row_tiles(const LayerArgs&, int host_count) { return host_count; }
    __device__ static int ncols(const LayerArgs& a) { return a.d; }
    __device__ static int kdim(const LayerArgs& a) { return a.m_s; }
    __device__ static const E* a_row(const LayerArgs& a, int, int r) {
        return static_cast<const E*>(a.a_s) + (size_t)r * a.m_s;
    }
    __device__ static const E* b_row(const LayerArgs& a, int, int c) {
        return static_cast<const E*>(a.W_s2) + (size_t)c * a.m_s;
    }
    __device__ static void store(const LayerArgs& a, int, int r, int c, float v) { a.y_s[(size_t)r * a.d + c] = v; }
};

// Problems whose reduction runs over two operand pairs (UpCat): k_split(a)
// terms from a_row / b_row, then the rest from a_row2 / b_row2.
template <class P, class = void>
struct HasKSplit : std::false_type {};
template <class P>
struct HasKSplit<P, decltype((void)P::k_split(std::declval<const LayerArgs&>()))> : std::true_type {};
template <class P>
__device__ inline int k_first(const LayerArgs& a) {
    if constexpr (HasKSplit<P>::value)
        return P::k_split(a);
    else
        return P::kdim(a);
}

// out = x + W_up s + W_s2 a_s (latent mode with a shared expert): one
// product whose reduction runs over l terms of [W_up | s], then m_s terms of
// [W_s2 | a_s] (k_split = l), residual added and rounded once.
template <class E>
struct UpCat : Up<E> {
    __device__ static int kdim(const LayerArgs& a) { return a.l + a.m_s; }
    __device__ static int k_split(const LayerArgs& a) { return a.l; }
    __device__ static const E* a_row2(const LayerArgs& a, int, int r) {
        return static_cast<const E*>(a.a_s) + (size_t)r * a.m_s;
    }
    __device__ static const E* b_row2(const LayerArgs& a, int, int c) {
        return static_cast<const E*>(a.W_s2) + (size_t)c * a.m_s;
    }
};

// out = x + W_up s + y_s (latent mode with a shared expert, float32 path:
// y_s computed beforehand), one rounding.
template <class E>
struct UpShared : Up<E> {
    __device__ static void store(const LayerArgs& a, int, int r, int c, float v) {
        const size_t i = (size_t)r * a.d + c;
        static_cast<E*>(a.out)[i] = from_f32<E>(to_f32(static_cast<const E*>(a.x)[i]) + a.y_s[i] + v);
    }
};

// The expert FFN with FP8 (E4M3) weights: the same products on bf16
// activations, the weight rows being one byte per element with one float32
// scale per row (applied to the row's fp32 dot product in the epilogue).
struct Ffn1Q : Ffn1<bf16> {
    using BElem = uint8_t;
    __device__ static const uint8_t* b_row(const LayerArgs& a, int e, int c) {
        return static_cast<const uint8_t*>(a.W1) + ((size_t)e * a.m + c) * a.l;
    }
    __device__ static float row_scale(const LayerArgs& a, int e, int c) { return a.w1s[(size_t)e * a.m + c]; }
};

struct Ffn2Q : Ffn2<bf16, f16> {
    using BElem = uint8_t;
    __device__ static const uint8_t* b_row(const LayerArgs& a, int e, int c) {
        return static_cast<const uint8_t*>(a.W2) + ((size_t)e * a.l + c) * a.m;
    }
    __device__ static float row_scale(const LayerArgs& a, int e, int c) { return a.w2s[(size_t)e * a.l + c]; }
};

// The expert FFN with MXFP4 weights: two E2M1 codes per byte, one E8M0
// scale per 32 elements along the reduction.  x_codes / x_scales give an
// expert's code and scale bytes; within an expert, the scale of the
// 32-element block holding code byte o is scale byte o / 16 (a row of n
// elements has n / 2 code bytes and n / 32 scale bytes).
struct MxFp4 {};   // BElem tag of MXFP4 weight rows

struct Ffn1X : Ffn1<bf16> {
    using BElem = MxFp4;
    __device__ static const uint8_t* x_codes(const LayerArgs& a, int e) {
        return static_cast<const uint8_t*>(a.W1) + (size_t)e * a.m * (a.l / 2);
    }
    __device__ static const uint8_t* x_scales(const LayerArgs& a, int e) { return a.w1x + (size_t)e * a.m * (a.l / 32); }
};

struct Ffn2X : Ffn2<bf16, f16> {
    using BElem = MxFp4;
    __device__ static const uint8_t* x_codes(const LayerArgs& a, int e) {
        return static_cast<const uint8_t*>(a.W2) + (size_t)e * a.l * (a.m / 2);
    }
    __device__ static const uint8_t* x_scales(const LayerArgs& a, int e) { return a.w2x + (size_t)e * a.l * (a.m / 32); }
};

}  // namespace lmoe