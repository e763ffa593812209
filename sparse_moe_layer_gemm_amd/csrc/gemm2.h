// gemm2.h -- the large-tile bf16 MFMA GEMM used by the tiled path.
//
// C[r, c] = epilogue(sum_k A[r, k] * B[c, k]) over a LayerArgs problem
// (layer.h), A rows = tokens or slots, B rows = weight rows.
//
// Tile BM x BN x 64 with NWM x NWN waves (2 x 2 for 128 x 128, 2 x 4 for
// 256 x 256); a wave owns (BM/NWM) x (BN/NWN) outputs as 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16.  The weight fragment is the MFMA's first
// operand, so a lane's 16 accumulators of a block are 4 groups of 4
// consecutive output columns of one row.  After a tile's last k-step its
// accumulators go through LDS so that the stores cover whole rows: as bf16
// after the epilogue for the expert FFN's problems and the up-projection
// (their epilogues need only the element, its row's gate, its column's scale
// or the residual element, which each lane loads in the accumulators'
// layout), as fp32 before it for the projection (mixed bf16 / fp32 outputs
// and a per-column bias, applied in the store layout).
//
// Pipeline: global -> registers two k-tiles ahead, registers -> LDS one
// k-tile ahead (two LDS buffers).  A k-tile is four MFMA groups (16 deep
// each); group q writes part q of the next k-tile to LDS and then loads
// part q of the k-tile after it into the freed registers, so every group
// carries the same LDS work (fragment reads plus a quarter of the staging
// writes) beside its MFMAs.  Within a group the MFMAs are interleaved with
// the LDS reads (two per MFMA) and then the writes and loads
// (sched_group_barrier), so each wave keeps the matrix cores and the LDS
// busy at once instead of alternating between them.
//
// LDS rows are 64 bf16 = 8 units of 16 bytes; unit c of row r is stored at
// c ^ sw(r), sw(r) = (r & 7) ^ ((r >> 3) & 1).  A 16-byte fragment read
// serves 16 lanes (16 consecutive rows, one unit) per cycle from 64 banks;
// two rows share a 256-byte bank window, so the 16 rows must land in 16
// distinct 16-byte slots (r & 1, c ^ sw(r)): sw takes 8 distinct values on
// the even rows and on the odd rows of any 16 aligned rows.  (The plain
// r & 7 repeats at r + 8 and costs a 2-way conflict on every read.)
//
// The grid is one-dimensional.  Consecutive workgroup ids go to different
// XCDs (round robin over 8), so ids are remapped such that each XCD gets a
// contiguous range of logical tiles; logical tiles run row-tile-major, so
// the tiles of one expert (its rows x all column tiles) share one XCD's L2.
#pragma once

#include <type_traits>

#include "layer.h"

namespace lmoe {

constexpr int kG2K = 64;     // k-tile
constexpr int kXcds = 8;

template <int BM, int BN, int NWM, int NWN>
struct G2Shape {
    static constexpr int NT = 64 * NWM * NWN;            // threads
    static constexpr int WM = BM / NWM, WN = BN / NWN;   // wave tile
    static constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 blocks per wave
    static constexpr int RSTEP = NT / 8;                 // rows one load instruction covers
    static constexpr int LA = BM / RSTEP, LB = BN / RSTEP;  // 16B loads per thread per k-tile
    static_assert(FM >= 1 && FN >= 1 && BM % RSTEP == 0 && BN % RSTEP == 0, "tile shape");
};

__device__ __forceinline__ int g2_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 4 consecutive output columns of one row (c0 .. c0+3), epilogue per problem.
// kStream: streaming stores, for the expert FFN's intermediates (A and the
// gate-scaled outputs: hundreds of MB at prefill, read once by the next
// kernel).  They shorten the wait of the next tile's operand loads, which
// are counted behind the stores; measured slower for the projections'
// outputs, which the next kernel reads while they may still be cached.
template <class E, bool kStream = false>
__device__ __forceinline__ void store_cols(E* dst, int c0, int ncols, const f32x4& v) {
    if (c0 + 3 < ncols && (reinterpret_cast<uintptr_t>(dst) & (4 * sizeof(E) - 1)) == 0) {
        if constexpr (sizeof(E) == 2) {
            bf16 b[4] = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            if constexpr (kStream)
                st_nt8(dst, *reinterpret_cast<const uint2*>(b));
            else
                *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(b);
        } else {
            const uint4 u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
            if constexpr (kStream)
                st_nt16(dst, u);
            else
                *reinterpret_cast<uint4*>(dst) = u;
        }
    } else {
        for (int i = 0; i < 4; ++i)
            if (c0 + i < ncols) dst[i] = from_f32<E>(v[i]);
    }
}

// Per-problem epilogue of 4 consecutive columns c0 .. c0+3 of one row.
// Loads in the epilogue sit behind the tile's stores in the one vector
// memory counter, so a load issued after a store waits for that store to
// complete.  The operands are therefore loaded early:
//   row_value(): one float per row (the gate), loaded by one thread per row
//     when the tile starts and passed through LDS (kRowVal);
//   col_load():  per-column data of the thread's 4 columns (the router
//     bias), loaded when the tile starts;
//   load():      per-element data (the residual), loaded for all passes of
//     an epilogue round before the round's first store.
struct NoPre {};

template <class P>
struct RowCtx;

// RowCtx<P>::kBf16Tile, false where a problem does not define it
template <class R, class = void>
struct Bf16Tile : std::false_type {};
template <class R>
struct Bf16Tile<R, std::void_t<decltype(R::kBf16Tile)>> : std::integral_constant<bool, R::kBf16Tile> {};
// RowCtx<P>::kElem (a per-element operand, elem_load(), added to the
// accumulator before the epilogue) and kNtStores (streaming stores; true
// where a problem does not say), for bf16 tiles
template <class R, class = void>
struct ElemOp : std::false_type {};
template <class R>
struct ElemOp<R, std::void_t<decltype(R::kElem)>> : std::integral_constant<bool, R::kElem> {};
template <class R, class = void>
struct NtStores : std::true_type {};
template <class R>
struct NtStores<R, std::void_t<decltype(R::kNtStores)>> : std::integral_constant<bool, R::kNtStores> {};
// RowCtx<P>::kColScale (a float per output column, applied first), false
// where a problem does not define it
// RowCtx<P>::kHalfOut: the 2-byte tile holds scaled half precision
// (pack4_f16_sat) instead of bfloat16
template <class R, class = void>
struct HalfOut : std::false_type {};
template <class R>
struct HalfOut<R, std::void_t<decltype(R::kHalfOut)>> : std::integral_constant<bool, R::kHalfOut> {};
template <class R, class = void>
struct ColScale : std::false_type {};
template <class R>
struct ColScale<R, std::void_t<decltype(R::kColScale)>> : std::integral_constant<bool, R::kColScale> {};

template <>
struct RowCtx<ProjRouter<bf16>> {
    static constexpr bool kRowVal = false;
    __device__ static float row_value(const LayerArgs&, int, int) { return 0.0f; }
    using ColPre = f32x4;
    __device__ static f32x4 col_load(const LayerArgs& a, int, int c0) {
        f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
        const int e0 = c0 - proj_lz(a) - a.m_s;
        if (a.bias && e0 >= 0)
            for (int i = 0; i < 4; ++i)
                if (e0 + i < a.N) b[i] = a.bias[e0 + i];
        return b;
    }
    using Pre = NoPre;
    __device__ static NoPre load(const LayerArgs&, int, int, int) { return NoPre{}; }
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4 v, const NoPre&, const f32x4& b,
                                 float) {
        const int lz = proj_lz(a), le = lz + a.m_s;
        if (c0 < lz) {
            store_cols(static_cast<bf16*>(a.z_w) + (size_t)r * a.l + c0, c0, lz, v);
        } else if (c0 < le) {   // the shared expert's relu(h_s)^2
            for (int i = 0; i < 4; ++i) {
                const float t = v[i] > 0.0f ? v[i] : 0.0f;
                v[i] = t * t;
            }
            store_cols(static_cast<bf16*>(a.a_s) + (size_t)r * a.m_s + (c0 - lz), c0 - lz, a.m_s, v);
        } else {
            const int e0 = c0 - le;
            store_cols(a.logits + (size_t)r * a.N + e0, e0, a.N, v + b);
        }
    }
};

// The FFN problems' epilogues depend only on the element and its row (relu^2;
// the slot's gate), so they run in registers and the tile goes through LDS
// as bf16 (kBf16Tile): tile_op() is the epilogue, tile_row() the row's
// destination.
template <>
struct RowCtx<Ffn1<bf16>> {
    static constexpr bool kRowVal = false;
    static constexpr bool kBf16Tile = true;
    __device__ static f32x4 tile_op(f32x4 v, float) {
        for (int i = 0; i < 4; ++i) {
            const float t = v[i] > 0.0f ? v[i] : 0.0f;
            v[i] = t * t;
        }
        return v;
    }
    __device__ static bf16* tile_row(const LayerArgs& a, int slot) { return static_cast<bf16*>(a.abuf) + (size_t)slot * a.m; }
    __device__ static float row_value(const LayerArgs&, int, int) { return 0.0f; }
    using ColPre = NoPre;
    __device__ static NoPre col_load(const LayerArgs&, int, int) { return NoPre{}; }
    using Pre = NoPre;
    __device__ static NoPre load(const LayerArgs&, int, int, int) { return NoPre{}; }
    __device__ static void store(const LayerArgs& a, int, int slot, int c0, f32x4 v, const NoPre&, const NoPre&,
                                 float) {
        for (int i = 0; i < 4; ++i) {
            const float t = v[i] > 0.0f ? v[i] : 0.0f;
            v[i] = t * t;
        }
        store_cols<bf16, true>(static_cast<bf16*>(a.abuf) + (size_t)slot * a.m + c0, c0, a.m, v);
    }
};

template <>
struct RowCtx<Ffn2<bf16, f16>> {
    static constexpr bool kRowVal = true;   // the slot's gate (times kYScale)
    static constexpr bool kBf16Tile = true;
    static constexpr bool kHalfOut = true;  // the tile is stored as scaled half precision
    __device__ static f32x4 tile_op(f32x4 v, float g) { return v * g; }
    __device__ static f16* tile_row(const LayerArgs& a, int slot) { return static_cast<f16*>(a.ybuf) + (size_t)slot * a.l; }
    __device__ static float row_value(const LayerArgs& a, int, int slot) { return a.gates[a.perm[slot]] * kYScale; }
    using ColPre = NoPre;
    __device__ static NoPre col_load(const LayerArgs&, int, int) { return NoPre{}; }
    using Pre = NoPre;
    __device__ static NoPre load(const LayerArgs&, int, int, int) { return NoPre{}; }
    __device__ static void store(const LayerArgs& a, int, int slot, int c0, f32x4 v, const NoPre&, const NoPre&,
                                 float g) {
        st_nt8(static_cast<f16*>(a.ybuf) + (size_t)slot * a.l + c0, pack4_f16_sat(v * g));   // l % 64 == 0
    }
};

template <>
struct RowCtx<Up<bf16>> {
    static constexpr bool kRowVal = false;
    // bf16 tile: the residual (4 bf16 of x per granule) is loaded per lane in
    // the accumulators' layout and added before the single rounding; plain
    // stores (the output is the layer's, read by the caller)
    static constexpr bool kBf16Tile = true, kElem = true, kNtStores = false;
    __device__ static uint2 elem_load(const LayerArgs& a, int r, int c0) {
        return *reinterpret_cast<const uint2*>(static_cast<const bf16*>(a.x) + (size_t)r * a.d + c0);
    }
    __device__ static f32x4 tile_op(f32x4 v, float) { return v; }
    __device__ static bf16* tile_row(const LayerArgs& a, int r) { return static_cast<bf16*>(a.out) + (size_t)r * a.d; }
    __device__ static float row_value(const LayerArgs&, int, int) { return 0.0f; }
    using ColPre = NoPre;
    __device__ static NoPre col_load(const LayerArgs&, int, int) { return NoPre{}; }
    using Pre = uint2;   // 4 bf16 of the residual row (d is a multiple of 64, so never ragged)
    __device__ static uint2 load(const LayerArgs& a, int, int r, int c0) {
        return *reinterpret_cast<const uint2*>(static_cast<const bf16*>(a.x) + (size_t)r * a.d + c0);
    }
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4 v, const uint2& u, const NoPre&,
                                 float) {
        v[0] += __uint_as_float(u.x << 16);
        v[1] += __uint_as_float(u.x & 0xffff0000u);
        v[2] += __uint_as_float(u.y << 16);
        v[3] += __uint_as_float(u.y & 0xffff0000u);
        store_cols(static_cast<bf16*>(a.out) + (size_t)r * a.d + c0, c0, a.d, v);
    }
};

// FP8 experts: the bf16 problems' epilogues after the column's scale (the
// scale of that weight row), which each tile loads once per column
// (kColScale) and passes through LDS.
template <>
struct RowCtx<Ffn1Q> : RowCtx<Ffn1<bf16>> {
    static constexpr bool kColScale = true;
    __device__ static float col_scale(const LayerArgs& a, int e, int c) { return Ffn1Q::row_scale(a, e, c); }
};

template <>
struct RowCtx<Ffn2Q> : RowCtx<Ffn2<bf16, f16>> {
    static constexpr bool kColScale = true;
    __device__ static float col_scale(const LayerArgs& a, int e, int c) { return Ffn2Q::row_scale(a, e, c); }
};

// MXFP4 experts: the block scales are applied when the codes are decoded,
// so the epilogues are the bf16 problems' own.
template <>
struct RowCtx<Ffn1X> : RowCtx<Ffn1<bf16>> {};
template <>
struct RowCtx<Ffn2X> : RowCtx<Ffn2<bf16, f16>> {};

template <>
struct RowCtx<Shared2<bf16>> {
    static constexpr bool kRowVal = false;
    __device__ static float row_value(const LayerArgs&, int, int) { return 0.0f; }
    using ColPre = NoPre;
    __device__ static NoPre col_load(const LayerArgs&, int, int) { return NoPre{}; }
    using Pre = NoPre;
    __device__ static NoPre load(const LayerArgs&, int, int, int) { return NoPre{}; }
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4 v, const NoPre&, const NoPre&,
                                 float) {
        store_cols(a.y_s + (size_t)r * a.d + c0, c0, a.d, v);
    }
};

// out = x + W_up s + W_s2 a_s: the epilogue of the up-projection (the
// reduction covers both products).
template <>
struct RowCtx<UpCat<bf16>> : RowCtx<Up<bf16>> {};

// Problems that map a logical tile index themselves (Tail<P>):
// item(a, logical, grp, row0, row_end, col0).
template <class P, class = void>
struct HasItem : std::false_type {};
template <class P>
struct HasItem<P, decltype((void)P::item(std::declval<const LayerArgs&>(), 0, std::declval<int&>(),
                                          std::declval<int&>(), std::declval<int&>(), std::declval<int&>()))>
    : std::true_type {};

template <class P, int BM, int BN, int NWM, int NWN>
__global__ __launch_bounds__(64 * NWM * NWN) void gemm2_kernel(LayerArgs a, int nrow_tiles, int ncol_tiles,
                                                                int g_limit) {
    using S = G2Shape<BM, BN, NWM, NWN>;
    // Persistent workgroups.  Logical tiles (row-tile-major) are split into
    // 8 contiguous ranges, one per XCD (workgroup b runs on XCD b % 8); the
    // gridDim / 8 workgroups of an XCD take its range's tiles round robin,
    // so the tiles in flight on an XCD at any time are neighbours (the rows
    // of one expert against all its weight columns) and share that XCD's
    // L2.  The actual tile count is read on the device for the FFN (the
    // host only knows a bound).
    // logical tiles: the problem's row tiles x column tiles, the first g_limit
    // of them (the rest, if any, run as a split-reduction tail)
    const int G = min(P::row_tiles(a, nrow_tiles) * ncol_tiles, g_limit);
    const int per_xcd = (G + kXcds - 1) / kXcds;
    const int xcd = blockIdx.x % kXcds, nslot = gridDim.x / kXcds;
    const int ncols = P::ncols(a);
    const int nk = P::kdim(a) / kG2K;
    struct Tile {
        int grp, row0, row_end, col0;
    };
    auto tile_at = [&](int slot, Tile& t) -> bool {
        if (slot >= per_xcd) return false;
        const int logical = xcd * per_xcd + slot;
        if (logical >= G) return false;
        if constexpr (HasItem<P>::value) {
            return P::item(a, logical, t.grp, t.row0, t.row_end, t.col0);
        } else {
            if (!P::tile(a, logical / ncol_tiles, BM, t.grp, t.row0, t.row_end)) return false;
            t.col0 = (logical % ncol_tiles) * BN;
            return t.col0 < ncols;
        }
    };

    // Two LDS stages, each [A rows | B rows] contiguous; after a tile's last
    // k-step its stage also stages the output tile.
    constexpr int kStageU4 = (BM + BN) * 8;
    __shared__ uint4 smem[2 * kStageU4];
    __shared__ float rowval[RowCtx<P>::kRowVal ? BM : 1];
    constexpr bool kColS = ColScale<RowCtx<P>>::value;
    __shared__ float colval[kColS ? BN : 1];
    auto As = [&](int st) { return smem + st * kStageU4; };
    auto Bs = [&](int st) { return smem + st * kStageU4 + BM * 8; };

    const int tid = threadIdx.x;
    const int ch = tid & 7;   // 16-byte unit within a row's k-slice
    const int lrow = tid >> 3;

    // The load cursor runs two k-steps ahead of the MFMAs, across tile
    // boundaries: (lslot, lkt) is the next k-step to load, ap/bp its rows.
    // Rows past a tile's end (and columns past ncols) read a valid row
    // instead: each output element depends only on its own row and column,
    // and those outputs are never stored.  No load is conditional, so the
    // compiler can count the loads in flight exactly.
    int lslot = blockIdx.x / kXcds, lkt = 0;
    Tile ct;  // the tile the MFMAs work on
    if (!tile_at(lslot, ct)) return;
    int cslot = lslot;
    // B rows: bf16; FP8 E4M3 codes (one byte each); or MXFP4 (two E2M1
    // codes per byte, a scale byte per 32 elements) -- the codes are decoded
    // to bf16 when they are written to LDS, so the LDS layout and the MFMAs
    // are the same.  A thread stages 8 elements of a row per k-step: 16
    // bytes, 8 code bytes, or 4 code bytes and their scale byte.
    using BE = typename P::BElem;
    constexpr int kFmt = std::is_same<BE, MxFp4>::value ? 2 : (sizeof(BE) == 1 ? 1 : 0);
    using BStage = typename std::conditional<kFmt == 0, uint4, uint2>::type;
    using BPtr = typename std::conditional<kFmt == 0, const bf16*, const uint8_t*>::type;
    const bf16* ap[S::LA];
    BPtr bp[kFmt == 2 ? 1 : S::LB];
    // MXFP4: the loading tile's expert's code and scale bytes, and each
    // staged row's byte offset within the expert (32-bit: fewer registers)
    const uint8_t* xc = nullptr;
    const uint8_t* xs = nullptr;
    uint32_t bo[kFmt == 2 ? S::LB : 1];
    auto set_rows = [&](const Tile& t) {
#pragma unroll
        for (int i = 0; i < S::LA; ++i) {
            const int r = t.row0 + lrow + S::RSTEP * i;
            ap[i] = P::a_row(a, t.grp, r < t.row_end ? r : t.row0) + ch * 8;
        }
        if constexpr (kFmt == 2) {
            xc = P::x_codes(a, t.grp);
            xs = P::x_scales(a, t.grp);
#pragma unroll
            for (int i = 0; i < S::LB; ++i) {
                const int c = t.col0 + lrow + S::RSTEP * i;
                bo[i] = (uint32_t)(c < ncols ? c : t.col0) * (uint32_t)(nk * (kG2K / 2)) + ch * 4;
            }
        } else {
#pragma unroll
            for (int i = 0; i < S::LB; ++i) {
                const int c = t.col0 + lrow + S::RSTEP * i;
                bp[i] = P::b_row(a, t.grp, c < ncols ? c : t.col0) + ch * 8;
            }
        }
    };
    set_rows(ct);
    // Two-segment reductions: at k-step nk1 the cursor's rows switch to the
    // second operand pair, offset by -k_split so that row + k0 addresses
    // term k0 - k_split of it (k_split is a multiple of the k-tile).
    constexpr bool kSeg = HasKSplit<P>::value;
    [[maybe_unused]] Tile lt = ct;   // the tile the load cursor is on
    [[maybe_unused]] int nk1 = nk;
    if constexpr (kSeg) nk1 = P::k_split(a) / kG2K;
    auto set_rows2 = [&](const Tile& t) {
        if constexpr (kSeg) {
            const int ks = P::k_split(a);
#pragma unroll
            for (int i = 0; i < S::LA; ++i) {
                const int r = t.row0 + lrow + S::RSTEP * i;
                ap[i] = P::a_row2(a, t.grp, r < t.row_end ? r : t.row0) + ch * 8 - ks;
            }
#pragma unroll
            for (int i = 0; i < S::LB; ++i) {
                const int c = t.col0 + lrow + S::RSTEP * i;
                bp[i] = P::b_row2(a, t.grp, c < ncols ? c : t.col0) + ch * 8 - ks;
            }
        }
    };
    // past the last tile the cursor stays on a valid k-step that is loaded
    // again and never used
    auto advance_load = [&]() {
        if (++lkt < nk) {
            if constexpr (kSeg)
                if (lkt == nk1) set_rows2(lt);
            return;
        }
        Tile nt;
        if (tile_at(lslot + nslot, nt)) {
            lslot += nslot;
            lkt = 0;
            set_rows(nt);
            if constexpr (kSeg) lt = nt;
        } else {
            lkt = nk - 1;
        }
    };

    uint4 ra[S::LA];
    BStage rb[S::LB];
    // Staged loads are split in 4 parts (load index i belongs to part i % 4),
    // so that part q of the next k-step can go to LDS, and part q of the
    // k-step after it can be loaded, in MFMA group q.
    auto in_part = [](int i, int n, int q) { return n >= 4 ? (i % 4 == q) : (q == 0); };
    // loads of the parts in `mask` (bit q: part q)
    auto gload_parts = [&](int mask) {
        auto in_mask = [&](int i, int n) {
            bool r = false;
#pragma unroll
            for (int q = 0; q < 4; ++q) r = r || (((mask >> q) & 1) && in_part(i, n, q));
            return r;
        };
        const int k0 = lkt * kG2K;
#pragma unroll
        for (int i = 0; i < S::LA; ++i)
            if (in_mask(i, S::LA)) ra[i] = ldg16(ap[i] + k0);
#pragma unroll
        for (int i = 0; i < S::LB; ++i)
            if (in_mask(i, S::LB)) {
                if constexpr (kFmt == 2) {
                    const uint32_t o = bo[i] + k0 / 2;
                    rb[i] = uint2{ldg4(xc + o), ldg1(xs + (o >> 4))};
                } else if constexpr (kFmt == 1) {
                    rb[i] = ldg8(bp[i] + k0);
                } else {
                    rb[i] = ldg16(bp[i] + k0);
                }
            }
    };
    auto swrite_part = [&](int st, int q) {
        uint4* as = As(st);
        uint4* bs = Bs(st);
#pragma unroll
        for (int i = 0; i < S::LA; ++i)
            if (in_part(i, S::LA, q)) {
                const int r = lrow + S::RSTEP * i;
                as[r * 8 + (ch ^ g2_swz(r))] = ra[i];
            }
#pragma unroll
        for (int i = 0; i < S::LB; ++i)
            if (in_part(i, S::LB, q)) {
                const int r = lrow + S::RSTEP * i;
                if constexpr (kFmt == 2)
                    bs[r * 8 + (ch ^ g2_swz(r))] = fp4x8_to_bf16x8(rb[i].x, e8m0_to_f32(rb[i].y));
                else if constexpr (kFmt == 1)
                    bs[r * 8 + (ch ^ g2_swz(r))] = e4m3x8_to_bf16x8(rb[i]);
                else
                    bs[r * 8 + (ch ^ g2_swz(r))] = rb[i];
            }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / NWN, wn = wave % NWN;
    f32x16 acc[S::FM][S::FN];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    };
    zero_acc();

    // prologue: k-step 0 into stage 0, k-step 1 into the registers
    gload_parts(15);
    advance_load();
#pragma unroll
    for (int q = 0; q < 4; ++q) swrite_part(0, q);
    __syncthreads();
    gload_parts(15);
    advance_load();

    // Fragments of MFMA group kk+1 are read from LDS while the MFMAs of
    // group kk are issued (two register sets), so LDS latency overlaps them.
    auto read_frags = [&](int st, int kk, bf16x8* af, bf16x8* bfr) {
        const int chunk = kk * 2 + (lane >> 5);
        const uint4* as = As(st);
        const uint4* bs = Bs(st);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
            const int r = wm * S::WM + i * 32 + (lane & 31);
            af[i] = as_bf16x8(as[r * 8 + (chunk ^ g2_swz(r))]);
        }
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int c = wn * S::WN + j * 32 + (lane & 31);
            bfr[j] = as_bf16x8(bs[c * 8 + (chunk ^ g2_swz(c))]);
        }
    };
    auto mfma_group = [&](const bf16x8* af, const bf16x8* bfr) {
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    };

    // Epilogue of tile ct from stage st (free once its last k-step is done;
    // the other stage already holds the next tile's first k-step).  The
    // fp32 tile goes through LDS row-major, in rounds of kEpiRows rows
    // (16-byte unit u of local row r at u ^ (r & 15), so 16 lanes on 16 rows
    // of one unit and 16 lanes on 16 units of one row both hit distinct bank
    // slots), and is read back 4 columns per lane with consecutive lanes on
    // consecutive columns: each store instruction covers whole rows instead
    // of 16 bytes of 32 rows.  Each round is written by the waves that own
    // its rows.
    constexpr int kEpiFit = kStageU4 * 16 / (BN * 4) / 32 * 32;   // fp32 rows one stage holds, in 32s
    constexpr int kEpiRows = kEpiFit < BM ? kEpiFit : BM;
    constexpr int kUpr = BN / 4, kPasses = kEpiRows * kUpr / S::NT;
    static_assert(!RowCtx<P>::kRowVal || BM <= S::NT, "one thread per row for the row values");
    // per-tile operands, loaded when the compute cursor enters a tile
    float rv = 0.0f;
    typename RowCtx<P>::ColPre colpre;
    float cs = 1.0f;
    static_assert(!kColS || (BN <= S::NT && Bf16Tile<RowCtx<P>>::value), "one thread per column for the scales");
    auto tile_loads = [&]() {
        if constexpr (RowCtx<P>::kRowVal) {
            if (tid < BM && ct.row0 + tid < ct.row_end) rv = RowCtx<P>::row_value(a, ct.grp, ct.row0 + tid);
        }
        if constexpr (kColS) {
            if (tid < BN) cs = ct.col0 + tid < ncols ? RowCtx<P>::col_scale(a, ct.grp, ct.col0 + tid) : 1.0f;
        }
        const int c = ct.col0 + 4 * (tid % kUpr);
        if (c < ncols) colpre = RowCtx<P>::col_load(a, ct.grp, c);
    };
    tile_loads();
    static_assert(kEpiRows % 32 == 0 && BM % kEpiRows == 0 && kUpr >= 16, "epilogue tiling");
    static_assert(kEpiRows * kUpr % S::NT == 0 && S::NT % kUpr == 0, "epilogue passes");
    // bf16 tiles (kBf16Tile): the epilogue runs on the accumulators, and the
    // rounded tile goes through LDS in rounds of kRowsB rows -- round h takes
    // the 32-row blocks h*FM/R .. of every wave row, so all waves write in
    // every round.  8-byte granule q (4 columns) of local row r is stored at
    // q ^ (r & 31): the 32 rows of one write instruction (one granule each)
    // hit 32 distinct bank pairs.  A 16-byte unit p (granules 2p, 2p+1) is
    // then unit p ^ ((r & 31) >> 1), its halves swapped when r is odd; each
    // thread stores whole units, consecutive threads on consecutive units.
    constexpr int kRowsFit = kStageU4 * 16 / (BN * 2) / 32 * 32;   // bf16 rows one stage holds
    constexpr int kRowsB = kRowsFit < BM ? kRowsFit : BM;
    constexpr int kRounds = BM / kRowsB, kWRows = S::WM / kRounds;   // a wave's rows per round
    constexpr int kUnits = BN / 8, kPassB = kRowsB * kUnits / S::NT;
    static_assert(kRowsB % 32 == 0 && BM % kRowsB == 0 && S::FM % kRounds == 0, "bf16 epilogue rounds");
    static_assert(S::NT % kUnits == 0 && kRowsB * kUnits % S::NT == 0, "bf16 epilogue passes");
    auto epilogue_bf16 = [&](int st) {
      if constexpr (Bf16Tile<RowCtx<P>>::value) {
        int etid = tid;
        asm volatile("" : "+v"(etid));
        const int lane = etid & 63;
        uint2* tg = reinterpret_cast<uint2*>(As(st));
        if constexpr (RowCtx<P>::kRowVal) {
            if (etid < BM) rowval[etid] = rv;
        }
        if constexpr (kColS) {
            if (etid < BN) colval[etid] = cs;
        }
        if constexpr (RowCtx<P>::kRowVal || kColS) __syncthreads();
        const int x = lane & 31;   // = local row & 31 of every row this lane writes
#pragma unroll
        for (int h = 0; h < kRounds; ++h) {
            if (h > 0) __syncthreads();   // the previous round's reads are done
            // per-element operands of this round, all loaded before the first
            // LDS write (rows past the tile's end and columns past ncols read
            // valid ones; their results are not stored)
            [[maybe_unused]] uint2 el[S::FM / kRounds][S::FN][4];
            if constexpr (ElemOp<RowCtx<P>>::value) {
#pragma unroll
                for (int ii = 0; ii < S::FM / kRounds; ++ii) {
                    const int i = h * (S::FM / kRounds) + ii;
                    const int row = min(ct.row0 + wm * S::WM + i * 32 + x, ct.row_end - 1);
#pragma unroll
                    for (int j = 0; j < S::FN; ++j)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int col = min(ct.col0 + wn * S::WN + j * 32 + 8 * q4 + 4 * (lane >> 5), ncols - 4);
                            el[ii][j][q4] = RowCtx<P>::elem_load(a, row, col);
                        }
                }
            }
#pragma unroll
            for (int ii = 0; ii < S::FM / kRounds; ++ii) {
                const int i = h * (S::FM / kRounds) + ii;
                const int rl = wm * kWRows + ii * 32 + x;
                const float g = RowCtx<P>::kRowVal ? rowval[wm * S::WM + i * 32 + x] : 0.0f;
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int q = (wn * S::WN + j * 32 + 8 * q4 + 4 * (lane >> 5)) >> 2;
                        f32x4 v = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
                        if constexpr (kColS) v *= *reinterpret_cast<const f32x4*>(&colval[4 * q]);
                        if constexpr (ElemOp<RowCtx<P>>::value) {
                            const uint2 u = el[ii][j][q4];
                            v[0] += __uint_as_float(u.x << 16);
                            v[1] += __uint_as_float(u.x & 0xffff0000u);
                            v[2] += __uint_as_float(u.y << 16);
                            v[3] += __uint_as_float(u.y & 0xffff0000u);
                        }
                        v = RowCtx<P>::tile_op(v, g);
                        tg[rl * (BN / 4) + (q ^ x)] =
                            HalfOut<RowCtx<P>>::value ? pack4_f16_sat(v) : pack4_bf16(v);
                    }
            }
            __syncthreads();
            const int p = etid % kUnits, c = ct.col0 + 8 * p;
#pragma unroll
            for (int it = 0; it < kPassB; ++it) {
                const int rl = it * (S::NT / kUnits) + etid / kUnits;
                const int row = ct.row0 + (rl / kWRows) * S::WM + h * kWRows + rl % kWRows;
                if (row < ct.row_end && c < ncols) {
                    const int y = rl & 31;
                    uint4 w = reinterpret_cast<const uint4*>(tg)[rl * kUnits + (p ^ (y >> 1))];
                    if (y & 1) w = uint4{w.z, w.w, w.x, w.y};
                    if constexpr (NtStores<RowCtx<P>>::value)
                        st_nt16(RowCtx<P>::tile_row(a, row) + c, w);
                    else
                        *reinterpret_cast<uint4*>(RowCtx<P>::tile_row(a, row) + c) = w;
                }
            }
        }
        __syncthreads();  // the stage is free for the k-step after next
      }
    };
    auto epilogue = [&](int st) {
        if constexpr (Bf16Tile<RowCtx<P>>::value) {
            epilogue_bf16(st);
            return;
        }
        // the epilogue's lane-dependent offsets are recomputed from an opaque
        // copy of the thread id, so they are not hoisted out of the tile loop
        // and kept live (in registers) across the k-steps
        int etid = tid;
        asm volatile("" : "+v"(etid));
        const int lane = etid & 63;
        float* tile = reinterpret_cast<float*>(As(st));
        const int u = etid % kUpr, c = ct.col0 + 4 * u;
        if constexpr (RowCtx<P>::kRowVal) {
            if (etid < BM) rowval[etid] = rv;   // read after the round's barrier
        }
#pragma unroll
        for (int h = 0; h < BM / kEpiRows; ++h) {
            if (h > 0) __syncthreads();  // the previous round's reads are done
#pragma unroll
            for (int i = 0; i < S::FM; ++i) {
                if ((wm * S::WM + i * 32) / kEpiRows != h) continue;
                const int rl = wm * S::WM + i * 32 + (lane & 31) - h * kEpiRows;
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int uu = (wn * S::WN + j * 32 + 8 * g + 4 * (lane >> 5)) >> 2;
                        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                         acc[i][j][4 * g + 3]};
                        *reinterpret_cast<f32x4*>(tile + rl * BN + ((uu ^ (rl & 15)) << 2)) = v;
                    }
            }
            // row of this thread's unit in pass it: it * (NT / kUpr) + tid / kUpr;
            // the per-element operands of all passes are loaded before the stores
            typename RowCtx<P>::Pre pre[kPasses];
#pragma unroll
            for (int it = 0; it < kPasses; ++it) {
                const int row = ct.row0 + h * kEpiRows + it * (S::NT / kUpr) + etid / kUpr;
                if (row < ct.row_end && c < ncols) pre[it] = RowCtx<P>::load(a, ct.grp, row, c);
            }
            __syncthreads();
#pragma unroll
            for (int it = 0; it < kPasses; ++it) {
                const int rl = it * (S::NT / kUpr) + etid / kUpr;
                const int row = ct.row0 + h * kEpiRows + rl;
                if (row < ct.row_end && c < ncols) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(tile + rl * BN + ((u ^ (rl & 15)) << 2));
                    RowCtx<P>::store(a, ct.grp, row, c, v, pre[it], colpre,
                                     RowCtx<P>::kRowVal ? rowval[h * kEpiRows + rl] : 0.0f);
                }
            }
        }
        __syncthreads();  // the stage is free for the k-step after next
    };

    // One barrier per k-step, in the last MFMA group: by then every wave
    // has written the next k-step to the other stage (parts 0-2 in groups
    // 0-2, part 3 just before the barrier) and read its last fragments of
    // this stage (in group 2).  After the barrier group 3 reads the next
    // k-step's first fragments from the other stage, so the next k-step
    // starts its MFMAs without waiting for the LDS.  After a tile's last
    // k-step those fragments are read again after the epilogue (which uses
    // only this stage), so that no fragment is live across the epilogue.
    bf16x8 a0[S::FM], b0[S::FN], a1[S::FM], b1[S::FN];
    read_frags(0, 0, a0, b0);
    for (int step = 0, ckt = 0;; ++step) {
        const int st = step & 1;
#pragma unroll
        for (int kk = 0; kk < kG2K / 16; ++kk) {
            bf16x8* ac = (kk & 1) ? a1 : a0;
            bf16x8* bc = (kk & 1) ? b1 : b0;
            bf16x8* an = (kk & 1) ? a0 : a1;
            bf16x8* bn = (kk & 1) ? b0 : b1;
            // part kk of the next k-step goes to LDS, then the same
            // registers take part kk of the k-step after
            if (kk + 1 < kG2K / 16) {
                read_frags(st, kk + 1, an, bn);
                swrite_part(st ^ 1, kk);
                gload_parts(1 << kk);
            } else {
                swrite_part(st ^ 1, kk);
                gload_parts(1 << kk);
                __syncthreads();
                read_frags(st ^ 1, 0, an, bn);
            }
            mfma_group(ac, bc);
            // Issue order of the group: each MFMA followed by two fragment
            // reads until they are all issued, then by one staging write and
            // one global load (masks: 0x008 MFMA, 0x100 LDS read, 0x200 LDS
            // write, 0x020 global load).  Group 3's write and load sit before
            // its barrier, outside this region.
            {
                constexpr int NM = S::FM * S::FN, NR = S::FM + S::FN;
#pragma unroll
                for (int i = 0; i < NM; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (2 * i + 1 < NR) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    } else if (2 * i < NR) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    } else if (kk < 3) {
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        advance_load();
        if (++ckt == nk) {
            epilogue(st);
            cslot += nslot;
            if (!tile_at(cslot, ct)) break;
            ckt = 0;
            zero_acc();
            tile_loads();
            read_frags(st ^ 1, 0, a0, b0);   // the next tile's first k-step
        }
    }
}

// ---------------------------------------------------------------------------
// Split-reduction tail.  A persistent launch of G tiles on R resident
// workgroups runs ceil(G / R) rounds; when the last round is partly empty
// (the projection at prefill: 384 tiles on 256 CUs), its r = G mod R tiles
// instead run as s = R / r (>= 2) workgroups each, workgroup p reducing k-range
// p of s into an fp32 partial tile (Tail<P>, a launch of its own after the
// full rounds), and tail_fixup_kernel adds the s partials in order and
// applies P's epilogue: ceil(G / R) rounds become floor(G / R) + 1/s.
// P: a problem with one row group (grp 0) and a one-segment reduction
// (the projection ProjRouter).
template <class P, int BM, int BN>
struct Tail {
    using BElem = typename P::BElem;
    __device__ static int kpart(const LayerArgs& a) { return P::kdim(a) / a.tail_s; }
    __device__ static bool item(const LayerArgs& a, int logical, int& grp, int& row0, int& row_end, int& col0) {
        const int t = a.tail_base + logical / a.tail_s;
        grp = logical % a.tail_s;   // the k-range
        int g;
        if (!P::tile(a, t / a.tail_ncol, BM, g, row0, row_end)) return false;
        col0 = (t % a.tail_ncol) * BN;
        return col0 < P::ncols(a);
    }
    __device__ static int row_tiles(const LayerArgs&, int host_count) { return host_count; }
    __device__ static int ncols(const LayerArgs& a) { return P::ncols(a); }
    __device__ static int kdim(const LayerArgs& a) { return kpart(a); }
    __device__ static const bf16* a_row(const LayerArgs& a, int p, int r) {
        return P::a_row(a, 0, r) + (size_t)p * kpart(a);
    }
    __device__ static const bf16* b_row(const LayerArgs& a, int p, int c) {
        return P::b_row(a, 0, c) + (size_t)p * kpart(a);
    }
    // partial tile of (row, column): [tile - tail_base][p][row - row0][column - col0]
    __device__ static float* part(const LayerArgs& a, int p, int r, int c) {
        const int t = (r / BM) * a.tail_ncol + c / BN - a.tail_base;
        return a.tail_part + (((size_t)t * a.tail_s + p) * BM + r % BM) * BN + c % BN;
    }
};

template <class P, int BM, int BN>
struct RowCtx<Tail<P, BM, BN>> {
    static constexpr bool kRowVal = false;
    __device__ static float row_value(const LayerArgs&, int, int) { return 0.0f; }
    using ColPre = NoPre;
    __device__ static NoPre col_load(const LayerArgs&, int, int) { return NoPre{}; }
    using Pre = NoPre;
    __device__ static NoPre load(const LayerArgs&, int, int, int) { return NoPre{}; }
    __device__ static void store(const LayerArgs& a, int p, int r, int c0, f32x4 v, const NoPre&, const NoPre&,
                                 float) {
        *reinterpret_cast<f32x4*>(Tail<P, BM, BN>::part(a, p, r, c0)) = v;   // BN, c0 multiples of 4
    }
};

// One thread per 4 consecutive columns of a row of a split tile: the s
// partials added in k-range order, then P's epilogue (its fp32-path
// RowCtx: per-element operand, per-column operand, store).
template <class P, int BM, int BN>
__global__ __launch_bounds__(256) void tail_fixup_kernel(LayerArgs a, int ntail) {
    const int item = blockIdx.x * 256 + threadIdx.x;
    const int per_tile = BM * (BN / 4);
    if (item >= ntail * per_tile) return;
    const int t = a.tail_base + item / per_tile;
    const int r = (t / a.tail_ncol) * BM + (item % per_tile) / (BN / 4);
    const int c = (t % a.tail_ncol) * BN + 4 * (item % (BN / 4));
    if (r >= a.T || c >= P::ncols(a)) return;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.tail_s; ++p) v += *reinterpret_cast<const f32x4*>(Tail<P, BM, BN>::part(a, p, r, c));
    const typename RowCtx<P>::Pre pre = RowCtx<P>::load(a, 0, r, c);
    const typename RowCtx<P>::ColPre cp = RowCtx<P>::col_load(a, 0, c);
    RowCtx<P>::store(a, 0, r, c, v, pre, cp, 0.0f);
}

}  // namespace lmoe
