// gemm2.h -- the large-tile bf16 MFMA GEMM used by the tiled path.
//
// C[r, c] = epilogue(sum_k A[r, k] * B[c, k]) over a LayerArgs problem
// (layer.h), A rows = tokens or slots, B rows = weight rows.
//
// Tile BM x BN x 64 with NWM x NWN waves (2 x 2 for 128 x 128, 2 x 4 for
// 256 x 256); a wave owns (BM/NWM) x (BN/NWN) outputs as 32 x 32 blocks of
// v_mfma_f32_32x32x16_bf16.  The weight fragment is the MFMA's first
// operand, so a lane's 16 accumulators of a block are 4 groups of 4
// consecutive output columns of one row: the epilogue reads per-row data
// (gate, token, residual row) once per lane and stores 4 columns at a time.
//
// Pipeline: global -> registers two k-tiles ahead, registers -> LDS one
// k-tile ahead (two LDS buffers).  In MFMA groups 0 and 1 of a k-tile,
// group g writes parts 2g and 2g+1 of the next k-tile to LDS and then loads
// the same parts of the k-tile after it into the freed registers, so each
// load is at least two groups old when the next k-tile starts.
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
template <class E>
__device__ __forceinline__ void store_cols(E* dst, int c0, int ncols, const f32x4& v) {
    if (c0 + 3 < ncols && (reinterpret_cast<uintptr_t>(dst) & (4 * sizeof(E) - 1)) == 0) {
        if constexpr (sizeof(E) == 2) {
            bf16 b[4] = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(b);
        } else {
            *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
        for (int i = 0; i < 4; ++i)
            if (c0 + i < ncols) dst[i] = from_f32<E>(v[i]);
    }
}

// Per-problem epilogue of 4 consecutive columns c0 .. c0+3 of one row:
// load() fetches what the row contributes (bias, gate, residual) and store()
// applies it and writes.  All load()s of a thread are issued before its
// first store(), so they overlap instead of each waiting behind the stores
// that the compiler cannot prove disjoint from them.
template <class P>
struct RowCtx;

template <>
struct RowCtx<ProjRouter<bf16>> {
    __device__ static f32x4 load(const LayerArgs& a, int, int, int c0) {
        f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
        const int e0 = c0 - (a.standard ? 0 : a.l);
        if (a.bias && e0 >= 0)
            for (int i = 0; i < 4; ++i)
                if (e0 + i < a.N) b[i] = a.bias[e0 + i];
        return b;
    }
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4 v, const f32x4& b) {
        const int lz = a.standard ? 0 : a.l;
        if (c0 < lz) {
            store_cols(static_cast<bf16*>(a.z_w) + (size_t)r * a.l + c0, c0, lz, v);
        } else {
            const int e0 = c0 - lz;
            store_cols(a.logits + (size_t)r * a.N + e0, e0, a.N, v + b);
        }
    }
};

template <>
struct RowCtx<Ffn1<bf16>> {
    __device__ static f32x4 load(const LayerArgs&, int, int, int) { return f32x4{}; }
    __device__ static void store(const LayerArgs& a, int, int slot, int c0, f32x4 v, const f32x4&) {
        for (int i = 0; i < 4; ++i) {
            const float t = v[i] > 0.0f ? v[i] : 0.0f;
            v[i] = t * t;
        }
        store_cols(static_cast<bf16*>(a.abuf) + (size_t)slot * a.m + c0, c0, a.m, v);
    }
};

template <>
struct RowCtx<Ffn2<bf16, bf16>> {
    __device__ static f32x4 load(const LayerArgs& a, int, int slot, int) {
        const float g = a.gates[a.perm[slot]];
        return f32x4{g, g, g, g};
    }
    __device__ static void store(const LayerArgs& a, int, int slot, int c0, f32x4 v, const f32x4& g) {
        store_cols(static_cast<bf16*>(a.ybuf) + (size_t)slot * a.l + c0, c0, a.l, v * g);
    }
};

template <>
struct RowCtx<Up<bf16>> {
    __device__ static f32x4 load(const LayerArgs& a, int, int r, int c0) {
        const bf16* xr = static_cast<const bf16*>(a.x) + (size_t)r * a.d + c0;
        f32x4 x;
        if (c0 + 3 < a.d) {
            const uint2 u = *reinterpret_cast<const uint2*>(xr);
            x[0] = __uint_as_float(u.x << 16);
            x[1] = __uint_as_float(u.x & 0xffff0000u);
            x[2] = __uint_as_float(u.y << 16);
            x[3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
            for (int i = 0; i < 4; ++i) x[i] = c0 + i < a.d ? (float)xr[i] : 0.0f;
        }
        return x;
    }
    __device__ static void store(const LayerArgs& a, int, int r, int c0, f32x4 v, const f32x4& x) {
        store_cols(static_cast<bf16*>(a.out) + (size_t)r * a.d + c0, c0, a.d, v + x);
    }
};

template <class P, int BM, int BN, int NWM, int NWN>
__global__ __launch_bounds__(64 * NWM * NWN) void gemm2_kernel(LayerArgs a, int nrow_tiles, int ncol_tiles) {
    using S = G2Shape<BM, BN, NWM, NWN>;
    // XCD-aware remap of the workgroup id to a logical tile.  The grid holds
    // kXcds * ceil(bound / kXcds) workgroups for the host's bound on the tile
    // count; the remap spreads the actual count (the tile list's length for
    // the FFN) over the 8 XCDs, so no XCD is left with only empty tiles, and
    // every logical tile still gets exactly one workgroup.
    const int G = P::row_tiles(a, nrow_tiles) * ncol_tiles;
    const int per_xcd = (G + kXcds - 1) / kXcds;
    const int slot = blockIdx.x / kXcds;
    if (slot >= per_xcd) return;
    const int logical = (blockIdx.x % kXcds) * per_xcd + slot;
    if (logical >= G) return;
    const int rt = logical / ncol_tiles, ct = logical % ncol_tiles;
    int grp, row0, row_end;
    if (!P::tile(a, rt, BM, grp, row0, row_end)) return;
    const int col0 = ct * BN;
    const int ncols = P::ncols(a);
    if (col0 >= ncols) return;
    const int K = P::kdim(a);
    const int nk = K / kG2K;

    // two LDS stages of both operands; after the k-loop the same memory
    // stages the output tile
    constexpr int kStageU4 = 2 * (BM + BN) * 8;
    __shared__ uint4 smem[kStageU4];
    uint4(*As)[BM * 8] = reinterpret_cast<uint4(*)[BM * 8]>(smem);
    uint4(*Bs)[BN * 8] = reinterpret_cast<uint4(*)[BN * 8]>(smem + 2 * BM * 8);

    const int tid = threadIdx.x;
    const int ch = tid & 7;   // 16-byte unit within a row's k-slice
    const int lrow = tid >> 3;
    // Rows past the tile's end (and columns past ncols) read a valid row
    // instead: each output element depends only on its own row and column,
    // and those outputs are never stored.  No load is conditional, so the
    // compiler can count the loads in flight exactly.
    const bf16* ap[S::LA];
    const bf16* bp[S::LB];
#pragma unroll
    for (int i = 0; i < S::LA; ++i) {
        const int r = row0 + lrow + S::RSTEP * i;
        ap[i] = P::a_row(a, grp, r < row_end ? r : row0) + ch * 8;
    }
#pragma unroll
    for (int i = 0; i < S::LB; ++i) {
        const int c = col0 + lrow + S::RSTEP * i;
        bp[i] = P::b_row(a, grp, c < ncols ? c : col0) + ch * 8;
    }
    uint4 ra[S::LA], rb[S::LB];
    // Staged loads are split in 4 parts (load index i belongs to part i % 4),
    // so that part q of the next k-tile can go to LDS, and part q of the
    // k-tile after it can be loaded, right after MFMA group q.
    auto in_part = [](int i, int n, int q) { return n >= 4 ? (i % 4 == q) : (q == 0); };
    // the loads of a k-tile are issued during the first two MFMA groups, so
    // that they are at least two groups old when the next k-tile starts
    auto gload_group = [&](int kt, int g) {
        const int k0 = kt * kG2K;
#pragma unroll
        for (int i = 0; i < S::LA; ++i)
            if (in_part(i, S::LA, 2 * g) || in_part(i, S::LA, 2 * g + 1)) ra[i] = ldg16(ap[i] + k0);
#pragma unroll
        for (int i = 0; i < S::LB; ++i)
            if (in_part(i, S::LB, 2 * g) || in_part(i, S::LB, 2 * g + 1)) rb[i] = ldg16(bp[i] + k0);
    };
    auto swrite_part = [&](int st, int q) {
#pragma unroll
        for (int i = 0; i < S::LA; ++i)
            if (in_part(i, S::LA, q)) {
                const int r = lrow + S::RSTEP * i;
                As[st][r * 8 + (ch ^ g2_swz(r))] = ra[i];
            }
#pragma unroll
        for (int i = 0; i < S::LB; ++i)
            if (in_part(i, S::LB, q)) {
                const int r = lrow + S::RSTEP * i;
                Bs[st][r * 8 + (ch ^ g2_swz(r))] = rb[i];
            }
    };

    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave / NWN, wn = wave % NWN;
    f32x16 acc[S::FM][S::FN];
#pragma unroll
    for (int i = 0; i < S::FM; ++i)
#pragma unroll
        for (int j = 0; j < S::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    gload_group(0, 0);
    gload_group(0, 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) swrite_part(0, q);
    __syncthreads();
    gload_group(min(1, nk - 1), 0);
    gload_group(min(1, nk - 1), 1);

    // Fragments of MFMA group kk+1 are read from LDS before the MFMAs of
    // group kk are issued (two register sets), so LDS latency overlaps them.
    auto read_frags = [&](int st, int kk, bf16x8* af, bf16x8* bfr) {
        const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < S::FM; ++i) {
            const int r = wm * S::WM + i * 32 + (lane & 31);
            af[i] = as_bf16x8(As[st][r * 8 + (chunk ^ g2_swz(r))]);
        }
#pragma unroll
        for (int j = 0; j < S::FN; ++j) {
            const int c = wn * S::WN + j * 32 + (lane & 31);
            bfr[j] = as_bf16x8(Bs[st][c * 8 + (chunk ^ g2_swz(c))]);
        }
    };
    auto mfma_group = [&](const bf16x8* af, const bf16x8* bfr) {
#pragma unroll
        for (int i = 0; i < S::FM; ++i)
#pragma unroll
            for (int j = 0; j < S::FN; ++j) acc[i][j] = mfma32(bfr[j], af[i], acc[i][j]);
    };
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        // the loop body is straight-line: the last iterations stage and load
        // a clamped k-tile that is never read
        const int kpre = min(kt + 2, nk - 1);
        bf16x8 a0[S::FM], b0[S::FN], a1[S::FM], b1[S::FN];
        read_frags(st, 0, a0, b0);
#pragma unroll
        for (int kk = 0; kk < kG2K / 16; ++kk) {
            bf16x8* ac = (kk & 1) ? a1 : a0;
            bf16x8* bc = (kk & 1) ? b1 : b0;
            bf16x8* an = (kk & 1) ? a0 : a1;
            bf16x8* bn = (kk & 1) ? b0 : b1;
            if (kk + 1 < kG2K / 16) read_frags(st, kk + 1, an, bn);
            if (kk < 2) {
                // parts 2kk, 2kk+1 of k-tile kt+1 go to LDS, then the same
                // registers take parts 2kk, 2kk+1 of k-tile kt+2
                swrite_part(st ^ 1, 2 * kk);
                swrite_part(st ^ 1, 2 * kk + 1);
                gload_group(kpre, kk);
            }
            mfma_group(ac, bc);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }

    // Epilogue through LDS: the fp32 tile is written row-major (16-byte unit
    // u of local row r at u ^ (r & 15), so 16 lanes on 16 rows of one unit
    // and 16 lanes on 16 units of one row both hit distinct bank slots),
    // then read back 4 columns per lane with consecutive lanes on
    // consecutive columns: each store instruction covers whole rows instead
    // of 16 bytes of 32 rows.  A tile larger than the LDS goes in rounds of
    // kEpiRows rows, each round written by the waves that own those rows.
    constexpr int kEpiRows = (kStageU4 * 16 / (BN * 4)) < BM ? (kStageU4 * 16 / (BN * 4)) : BM;
    static_assert(kEpiRows % S::WM == 0 && BM % kEpiRows == 0 && BN / 4 >= 16, "epilogue tiling");
    float* tile = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int h = 0; h < BM / kEpiRows; ++h) {
        __syncthreads();  // the k-loop (or the previous round) is done with the LDS
        if (wm * S::WM / kEpiRows == h) {
#pragma unroll
            for (int i = 0; i < S::FM; ++i) {
                const int rl = wm * S::WM + i * 32 + (lane & 31) - h * kEpiRows;
#pragma unroll
                for (int j = 0; j < S::FN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int u = (wn * S::WN + j * 32 + 8 * g + 4 * (lane >> 5)) >> 2;
                        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                         acc[i][j][4 * g + 3]};
                        *reinterpret_cast<f32x4*>(tile + rl * BN + ((u ^ (rl & 15)) << 2)) = v;
                    }
            }
        }
        // row/column of this thread's unit in pass it: rl = it * (NT / (BN/4)) + tid / (BN/4)
        constexpr int kUpr = BN / 4, kPasses = kEpiRows * kUpr / S::NT;
        static_assert(kEpiRows * kUpr % S::NT == 0 && S::NT % kUpr == 0, "epilogue passes");
        const int u = tid % kUpr, c = col0 + 4 * u;
        f32x4 pre[kPasses];
#pragma unroll
        for (int it = 0; it < kPasses; ++it) {
            const int row = row0 + h * kEpiRows + it * (S::NT / kUpr) + tid / kUpr;
            if (row < row_end && c < ncols) pre[it] = RowCtx<P>::load(a, grp, row, c);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kPasses; ++it) {
            const int rl = it * (S::NT / kUpr) + tid / kUpr;
            const int row = row0 + h * kEpiRows + rl;
            if (row < row_end && c < ncols) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(tile + rl * BN + ((u ^ (rl & 15)) << 2));
                RowCtx<P>::store(a, grp, row, c, v, pre[it]);
            }
        }
    }
}

}  // namespace lmoe
