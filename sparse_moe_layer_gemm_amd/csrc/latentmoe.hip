// latentmoe.hip -- the C ABI (include/latentmoe.h) and the launch plan.
//
// One forward enqueues, on the caller's stream:
//   1. z = W_down x and the router logits   (skinny / tiled MFMA / SIMT GEMM)
//   2. top-K + softmax renormalisation      (one wavefront per token)
//   3. dispatch: counting sort by expert    (1 or 3 launches; none on the
//                                            streaming path at T <= 256,
//                                            whose FFN routes itself)
//   4. expert FFN                           (streaming kernel, or two grouped
//                                            GEMMs with ReLU^2 and the gate
//                                            fused into their epilogues)
//   5. gate-weighted combine                (+ residual in standard mode)
//   6. out = x + W_up s                     (latent mode)
// No host synchronisation and no allocation happen inside a forward.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <type_traits>

#include "../../include/latentmoe.h"
#include "combine.h"
#include "common.h"
#include "gemm.h"
#include "gemm2.h"
#include "layer.h"
#include "route.h"
#include "stream.h"

using namespace lmoe;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

constexpr size_t kAlign = 256;

// Tiled bf16 GEMM shapes: rows x columns per workgroup and its wave grid.
// PER_CU: workgroups resident per CU (the LDS stages bound it).
template <int BM_, int BN_, int NWM_, int NWN_, int PER_CU_>
struct G2Cfg {
    static constexpr int BM = BM_, BN = BN_, NWM = NWM_, NWN = NWN_, PER_CU = PER_CU_;
};
using G2Large = G2Cfg<256, 256, 2, 4, 1>;   // 8 waves, 128 KB LDS
using G2Small = G2Cfg<128, 128, 2, 2, 2>;   // 4 waves, 64 KB LDS
// The expert FFN takes the large tile when experts hold many rows on average
// (the tile list, shared by both FFN GEMMs, is cut at that height); with few
// rows per expert the 256-row tile would be mostly padding.
constexpr int kFfnLargeMinMeanRows = 512;
constexpr long long kProjLargeMinTiles = 256;   // see proj_uses_large()
// the self-routed streaming FFN (T <= kSkinnyMaxRows): one mask bit per FFN
// expert, the T*K ids in at most 32 KB of dynamic LDS
static_assert(kSelfRouteMaskWords * 32 >= kMaxExperts, "self-route mask too small");
static_assert((size_t)kSkinnyMaxRows * kMaxK * 2 <= 32768, "self-route ids exceed 32 KB of LDS");
using UpTile = G2Large;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// The skinny projection's reduction is split into enough k-ranges that the
// (16-column group, k-range) workgroups fill the CUs once: 768 for T <= 32
// (the kernel with at most two row blocks fits three workgroups per CU),
// else 512; its partial tiles are part[split][T][stride], stride = columns
// rounded up to 4 floats.
constexpr int kMaxProjSplit = kMaxSplit;   // the top-K kernel adds at most this many partials
int proj_split(int ncols, int T) {
    const int target = T <= 32 ? 768 : 512;
    return std::max(1, std::min(kMaxProjSplit, target / (cdiv(ncols, 16) * cdiv(T, 64))));
}
int proj_stride(int ncols) { return (ncols + 3) / 4 * 4; }
size_t proj_part_floats(int ncols, int T) {  // per token row
    return (size_t)proj_split(ncols, T) * proj_stride(ncols);
}

// mean rows per expert at or below which the streaming FFN is chosen
constexpr int kStreamMaxMeanRows = 16;
// The streaming FFN's m-slice: 128 (64 where m is not a multiple of 128),
// or 256 (bf16, FP8, and MXFP4 experts with l % 256 == 0, which take
// ffn_stream_mx_kernel) when the expected (active expert, slice)
// workgroups under uniform routing number at least kWideSliceMinWgs (four
// per CU) and the active experts average at most kWideSliceMaxRows rows
// (one 16-row pass, as a rule), or when the 256-wide workgroups fill most
// of one round of the GPU's kOneRoundWgs (two per CU), which the 128-wide
// ones would overflow (decode at 8 tokens: 462 against 924).
// Wider slices halve the partial planes (the FFN's stores, the
// combine's reads) but also the workgroups that stream the weights.  With
// bf16 experts and fewer than kNarrowSliceMaxWgs such workgroups at 128
// (a few tokens on few, large experts) the slice is 64 wide: twice the
// workgroups, each streaming half as much.
constexpr double kWideSliceMinWgs = 1024;
constexpr double kWideSliceMaxRows = 16;
constexpr double kOneRoundWgs = 512;
constexpr double kOneRoundMinFill = 0.8;
constexpr double kNarrowSliceMaxWgs = 128;

struct Plan {
    int status = LMOE_OK;
    bool bf16 = false;
    int path = LMOE_PATH_TILED;   // resolved: STREAM or TILED
    bool skinny = false;          // projections on the skinny kernel
    int tile_rows = G2Small::BM;
    bool ffn_large = false;       // tiled FFN on G2Large
    int wfmt = 0;                 // expert weights: 0 dense, 1 FP8 E4M3 rows, 2 MXFP4
    int nr = 0;                   // routed ids: FFN and zero-computation experts
    int nblk = 1;                 // dispatch blocks
    int ms = 128;                 // streaming FFN m-slice
    int nsplit = 1;               // streaming FFN partial planes
    long long max_tiles = 0;
    int tall_rows = 0;            // > 0: experts over tile_rows rows take G2Large tiles (tiles_tall)
    long long max_tiles_tall = 0;
    size_t es = 2;
    size_t z, logits, ids, gates, counts, offsets, perm, slot_of, blk_counts, blk_offsets, tiles, n_tiles,
        tiles_tall, n_tiles_tall, active, n_active, abuf, ybuf, s, part, a_s, y_s, tail, total;
};

bool mult64(int v) { return v > 0 && v % 64 == 0; }

size_t tiled_tail_bytes(const lmoe_dims& d, const Plan& p);

// The tiled projection takes the large tile when it still makes at least one
// tile per CU (many rows and columns: the latent layer's [z | logits] at
// prefill), else the small one (the standard layer's few router columns).
bool proj_uses_large(int T, int ncols) {
    return (long long)cdiv(T, G2Large::BM) * cdiv(ncols, G2Large::BN) >= kProjLargeMinTiles;
}

Plan make_plan(const lmoe_dims* dm, int32_t K) {
    Plan p;
    if (!dm) {
        p.status = fail(LMOE_EINVAL, "dims is NULL");
        return p;
    }
    const lmoe_dims& d = *dm;
    if (d.T < 1 || d.T > (1 << 24)) {
        p.status = fail(LMOE_EINVAL, "T=%d must be in [1, 2^24]", d.T);
        return p;
    }
    if (!mult64(d.d) || !mult64(d.l) || !mult64(d.m)) {
        p.status = fail(LMOE_EINVAL, "d=%d, l=%d, m=%d must be positive multiples of 64", d.d, d.l, d.m);
        return p;
    }
    if (d.N < 1 || d.n_zero < 0 || d.n_copy < 0 || d.n_const < 0 ||
        (long long)d.N + d.n_zero + d.n_copy + d.n_const > kMaxExperts) {
        p.status = fail(LMOE_EINVAL, "N=%d >= 1 and n_zero=%d, n_copy=%d, n_const=%d >= 0 with at most %d ids in all",
                        d.N, d.n_zero, d.n_copy, d.n_const, kMaxExperts);
        return p;
    }
    p.nr = d.N + d.n_zero + d.n_copy + d.n_const;
    if (K < 1 || K > p.nr || K > kMaxK) {
        p.status = fail(LMOE_EINVAL, "K=%d must be in [1, min(Nr=%d, %d)]", K, p.nr, kMaxK);
        return p;
    }
    if ((long long)d.T * K > (1ll << 30)) {
        p.status = fail(LMOE_EUNSUPPORTED, "T*K=%lld exceeds 2^30", (long long)d.T * K);
        return p;
    }
    if (d.dtype != LMOE_F32 && d.dtype != LMOE_BF16) {
        p.status = fail(LMOE_EINVAL, "dtype=%d is not LMOE_F32 or LMOE_BF16", d.dtype);
        return p;
    }
    if (d.expert_format != LMOE_EXPERTS_DENSE && d.expert_format != LMOE_EXPERTS_FP8_E4M3 &&
        d.expert_format != LMOE_EXPERTS_MXFP4) {
        p.status = fail(LMOE_EINVAL, "expert_format=%d is not a lmoe_expert_format", d.expert_format);
        return p;
    }
    if (d.expert_format != LMOE_EXPERTS_DENSE && d.dtype != LMOE_BF16) {
        p.status = fail(LMOE_EUNSUPPORTED, "FP8 / MXFP4 experts need a bfloat16 layer");
        return p;
    }
    p.wfmt = d.expert_format == LMOE_EXPERTS_FP8_E4M3 ? 1 : (d.expert_format == LMOE_EXPERTS_MXFP4 ? 2 : 0);
    if (p.wfmt == 2 && (long long)d.m * d.l / 2 >= (1ll << 31)) {
        p.status = fail(LMOE_EUNSUPPORTED, "MXFP4 experts of more than 2^31 code bytes (m=%d, l=%d)", d.m, d.l);
        return p;
    }
    if (d.m_shared < 0 || d.m_shared % 64 != 0) {
        p.status = fail(LMOE_EINVAL, "m_shared=%d must be 0 or a positive multiple of 64", d.m_shared);
        return p;
    }
    if (d.path != LMOE_PATH_AUTO && d.path != LMOE_PATH_STREAM && d.path != LMOE_PATH_TILED) {
        p.status = fail(LMOE_EINVAL, "path=%d is not a lmoe_path", d.path);
        return p;
    }
    p.bf16 = d.dtype == LMOE_BF16;
    p.es = p.bf16 ? 2 : 4;
    const long long TK = (long long)d.T * K;
    if (!p.bf16) {
        if (d.path == LMOE_PATH_STREAM) {
            p.status = fail(LMOE_EUNSUPPORTED, "the streaming FFN is bf16 only");
            return p;
        }
        p.path = LMOE_PATH_TILED;
        p.tile_rows = kSimtM;
    } else {
        if (d.path == LMOE_PATH_AUTO)
            p.path = (TK <= (long long)kStreamMaxMeanRows * d.N) ? LMOE_PATH_STREAM : LMOE_PATH_TILED;
        else
            p.path = d.path;
        p.ffn_large = TK >= (long long)kFfnLargeMinMeanRows * d.N;
        p.tile_rows = p.ffn_large ? G2Large::BM : G2Small::BM;
        p.ms = (d.m % 128 == 0) ? 128 : 64;
        const double ffn_slots = (double)TK * d.N / p.nr;   // routed rows of FFN experts
        const double active = d.N * (1.0 - std::pow(1.0 - (double)K / p.nr, (double)d.T));   // expected
        const double wide_wgs = active * (d.m / 256);
        const bool many = wide_wgs >= kWideSliceMinWgs && ffn_slots <= kWideSliceMaxRows * active;
        const bool one_round = wide_wgs >= kOneRoundMinFill * kOneRoundWgs && wide_wgs <= kOneRoundWgs;
        if ((p.wfmt <= 1 || d.l % 256 == 0) && d.m % 256 == 0 && (many || one_round))
            p.ms = 256;
        else if (p.wfmt == 0 && p.ms == 128 && active * (d.m / 128) < kNarrowSliceMaxWgs)
            p.ms = 64;
        p.nsplit = p.path == LMOE_PATH_STREAM ? d.m / p.ms : 1;
        p.skinny = p.path == LMOE_PATH_STREAM && d.T <= kSkinnyMaxRows;
    }
    p.nblk = cdiv(d.T, kRouteTok);
    p.max_tiles = TK / p.tile_rows + std::min<long long>(d.N, TK);
    // On the 128-row FFN tiles, experts with more than 128 rows (possible
    // only when T > 128) take 256-row tiles on the large GEMM tile instead:
    // with skewed routing most rows belong to a few heavy experts, whose
    // weights are then read by half as many row tiles.
    if (p.bf16 && p.path == LMOE_PATH_TILED && !p.ffn_large && d.T > G2Small::BM) {
        p.tall_rows = G2Large::BM;
        p.max_tiles_tall = TK / p.tall_rows + std::min<long long>(d.N, TK);
    }

    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    p.z = take((size_t)d.T * d.l * p.es);
    p.logits = take((size_t)d.T * p.nr * 4);
    p.ids = take((size_t)TK * 4);
    p.gates = take((size_t)TK * 4);
    p.counts = take((size_t)p.nr * 4);
    p.offsets = take((size_t)(p.nr + 1) * 4);
    p.perm = take((size_t)TK * 4);
    p.slot_of = take((size_t)TK * 4);
    p.blk_counts = take((size_t)p.nblk * p.nr * 4);
    p.blk_offsets = take((size_t)p.nblk * p.nr * 4);
    p.tiles = take((size_t)p.max_tiles * 8);
    p.n_tiles = take(4);
    p.tiles_tall = take((size_t)p.max_tiles_tall * 8);
    p.n_tiles_tall = take(4);
    p.active = take((size_t)d.N * 4);
    p.n_active = take(4);
    if (p.path == LMOE_PATH_STREAM) {
        p.abuf = take(0);
        p.ybuf = take((size_t)p.nsplit * (TK + 1) * d.l * 2);   // fp16 partials, + the zero row of each plane
    } else {
        p.abuf = take((size_t)TK * d.m * p.es);
        p.ybuf = take((size_t)(TK + 1) * d.l * p.es);
    }
    p.s = take((size_t)d.T * d.l * p.es);
    // partial tiles of the split projection, for either mode (standard mode,
    // W_down == NULL, is only known at the call: m_s + Nr instead of
    // l + m_s + Nr columns)
    size_t part_bytes = 0;
    if (p.skinny)
        part_bytes = std::max(proj_part_floats(d.l + d.m_shared + p.nr, d.T),
                              proj_part_floats(d.m_shared + p.nr, d.T)) * d.T * 4;
    p.part = take(part_bytes);
    p.a_s = take((size_t)d.T * d.m_shared * p.es);
    p.y_s = take(d.m_shared > 0 ? (size_t)d.T * d.d * 4 : 0);
    p.tail = take(tiled_tail_bytes(d, p));
    p.total = o;
    return p;
}

size_t dispatch_lds_bytes(int N) { return (size_t)N * 32 + (size_t)N * 12 + 17 * 4; }

// Once per device (kernel attributes belong to a device): the dispatch
// kernels may use more dynamic LDS than the default limit.
void init_once() {
    constexpr int kMaxDevices = 64;
    static std::once_flag flags[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    std::call_once(flags[dev], [] {
        const int bytes = (int)dispatch_lds_bytes(kMaxExperts);
        (void)hipFuncSetAttribute((const void*)dispatch_one_block_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        (void)hipFuncSetAttribute((const void*)dispatch_count_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        (void)hipFuncSetAttribute((const void*)dispatch_scan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        (void)hipFuncSetAttribute((const void*)dispatch_scatter_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        (void)hipGetLastError();
    });
}

// Compute units of the current device (cached per device ordinal).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Resident workgroups of a tiled-GEMM configuration (a multiple of 8).
template <class C>
long long g2_resident() {
    return (long long)device_cus() * C::PER_CU / kXcds * kXcds;
}

// Persistent launch: one wave of resident workgroups (a multiple of 8, one
// range of tiles per XCD), or fewer when there are fewer tiles.  g_limit:
// only the first g_limit logical tiles (the rest run as a tail).
template <class P, class C>
void launch_g2(const LayerArgs& a, int nrow_tiles, int ncol_tiles, hipStream_t st, int g_limit = INT_MAX) {
    const long long tiles = std::min<long long>((long long)nrow_tiles * ncol_tiles, g_limit);
    const long long resident = g2_resident<C>();
    const long long g = std::max<long long>(kXcds, std::min<long long>((tiles + kXcds - 1) / kXcds * kXcds, resident));
    gemm2_kernel<P, C::BM, C::BN, C::NWM, C::NWN>
        <<<(unsigned)g, dim3(64 * C::NWM * C::NWN), 0, st>>>(a, nrow_tiles, ncol_tiles, g_limit);
}

// Split-reduction tail of a product of G tiles on R resident workgroups
// (Tail<P> in gemm2.h): when the last round would hold r = G mod R tiles
// with r <= R / 2, those tiles are split over s = min(4, R / r) k-ranges
// (s dividing the k-steps).  s = 1: no tail.
constexpr int kMaxTailSplit = 4;
struct TailPlan {
    long long base = 0;   // tiles before the tail
    int s = 1, ntail = 0;
};
TailPlan tail_plan(long long G, long long R, int ksteps) {
    TailPlan t;
    const long long r = G % R;
    if (G <= 0 || r == 0) return t;
    int s = (int)std::min<long long>(kMaxTailSplit, R / r);
    while (s > 1 && ksteps % s != 0) --s;
    if (s < 2) return t;
    t.base = G - r;
    t.s = s;
    t.ntail = (int)r;
    return t;
}
template <class C>
size_t tail_bytes(long long G, int ksteps) {
    const TailPlan t = tail_plan(G, g2_resident<C>(), ksteps);
    return t.s > 1 ? (size_t)t.ntail * t.s * C::BM * C::BN * 4 : 0;
}

// Bytes of the tail partials the bf16 tiled path's projection may need (its
// columns depend on the mode, only known at the call: the larger of the
// two).  The up-projection has no tail: its reduction (l) is short, and the
// half tiles' fp32 partials and the fixup cost what the shorter last round
// saves (skewed workload: 249 -> 258 us with a tail).
size_t tiled_tail_bytes(const lmoe_dims& d, const Plan& p) {
    if (!p.bf16 || p.skinny) return 0;
    size_t t = 0;
    for (int lz : {d.l, 0}) {
        const int nc = lz + d.m_shared + p.nr;
        t = std::max(t, proj_uses_large(d.T, nc)
                            ? tail_bytes<G2Large>((long long)cdiv(d.T, G2Large::BM) * cdiv(nc, G2Large::BN), d.d / 64)
                            : tail_bytes<G2Small>((long long)cdiv(d.T, G2Small::BM) * cdiv(nc, G2Small::BN), d.d / 64));
    }
    return t;
}

// A tiled product with its split-reduction tail, if any: the full rounds,
// then the tail's partial tiles, then the fixup that adds them and applies
// P's epilogue.  The workspace's tail buffer holds the partials.
template <class P, class C>
void launch_g2_tail(LayerArgs a, int nrow_tiles, int ncol_tiles, int ksteps, hipStream_t st) {
    const TailPlan t = tail_plan((long long)nrow_tiles * ncol_tiles, g2_resident<C>(), ksteps);
    if (t.s < 2) {
        launch_g2<P, C>(a, nrow_tiles, ncol_tiles, st);
        return;
    }
    a.tail_base = (int)t.base;
    a.tail_s = t.s;
    a.tail_ncol = ncol_tiles;
    if (t.base > 0) launch_g2<P, C>(a, nrow_tiles, ncol_tiles, st, (int)t.base);
    launch_g2<Tail<P, C::BM, C::BN>, C>(a, t.s * t.ntail, 1, st);
    const long long items = (long long)t.ntail * C::BM * (C::BN / 4);
    tail_fixup_kernel<P, C::BM, C::BN><<<(unsigned)((items + 255) / 256), dim3(256), 0, st>>>(a, t.ntail);
}

// Rank groups per combine item: enough threads to fill the GPU.
template <class E, class YT, bool PL>
void launch_combine(const LayerArgs& a, int nsplit, hipStream_t st) {
    const long long items = (long long)a.T * (a.l / (16 / (int)sizeof(YT)));
    if (items >= 131072) {
        combine_kernel<E, YT, 1, PL><<<(unsigned)((items + 255) / 256), dim3(256), 0, st>>>(a, nsplit);
    } else if (items >= 16384) {
        combine_kernel<E, YT, 4, PL><<<(unsigned)((items + 63) / 64), dim3(256), 0, st>>>(a, nsplit);
    } else {
        combine_kernel<E, YT, 16, PL><<<(unsigned)((items + 15) / 16), dim3(256), 0, st>>>(a, nsplit);
    }
}

template <class E, class YT>
hipError_t launch_all(const Plan& p, LayerArgs& a, hipStream_t st, void* const* events) {
    hipError_t ext_err = hipSuccess;   // the one launch whose status is returned, not left as the last error
    auto mark = [&](int i) {
        if (events && events[i]) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
    };
    const dim3 b256(256), b1024(1024);
    // projection columns: [z | the shared expert's h_s | logits]
    const int ncols_pr = (a.standard ? 0 : a.l) + a.m_s + a.N;
    PartIn pin{nullptr, 0, 0, 0};
    float* part = reinterpret_cast<float*>(a.part);
    // 1. projection + router logits
    mark(0);
    if constexpr (sizeof(E) == 2) {
        if (p.skinny) {
            const int split = proj_split(ncols_pr, a.T), stride = proj_stride(ncols_pr);
            const dim3 grid(cdiv(ncols_pr, 16), split, cdiv(a.T, 64));
            if (a.T <= 16)
                skinny_part_kernel<ProjRouter<bf16>, 1><<<dim3(grid.x, split, cdiv(a.T, 16)), b256, 0, st>>>(
                    a, part, split, stride);
            else if (a.T <= 32)
                skinny_part_kernel<ProjRouter<bf16>, 2><<<dim3(grid.x, split, cdiv(a.T, 32)), b256, 0, st>>>(
                    a, part, split, stride);
            else
                skinny_part_kernel<ProjRouter<bf16>, 4><<<grid, b256, 0, st>>>(a, part, split, stride);
            pin = PartIn{part, split, stride, a.standard ? 0 : a.l};
        } else {
            if (proj_uses_large(a.T, ncols_pr))
                launch_g2_tail<ProjRouter<bf16>, G2Large>(a, cdiv(a.T, G2Large::BM), cdiv(ncols_pr, G2Large::BN),
                                                          a.d / 64, st);
            else
                launch_g2_tail<ProjRouter<bf16>, G2Small>(a, cdiv(a.T, G2Small::BM), cdiv(ncols_pr, G2Small::BN),
                                                          a.d / 64, st);
        }
    } else {
        gemm_simt_kernel<ProjRouter<float>><<<dim3(cdiv(a.T, kSimtM), cdiv(ncols_pr, kSimtN)), b256, 0, st>>>(a);
    }
    // The shared expert's a_s = relu(W_s1 x)^2 comes out of the projection
    // (its h_s columns).  Its second product: in the bf16 latent layer, part
    // of the up-projection's reduction (UpCat); otherwise y_s = W_s2 a_s in
    // float32, added by the up-projection (float32) or the combine
    // (standard mode).
    const bool shared_y = a.m_s > 0 && (sizeof(E) == 4 || a.standard);
    // 2. top-K gates
    mark(1);
    {
        auto launch_topk = [&](auto npl) {
            constexpr int NPL = decltype(npl)::value;
            if (pin.nsplit > 0)
                topk_part_kernel<NPL><<<dim3(a.T, 2), b256, 0, st>>>(a, pin);
            else
                topk_kernel<NPL><<<dim3(cdiv(a.T, 4)), b256, 0, st>>>(a);
        };
        // logits per lane: the smallest tier that holds the routed ids
        if (a.N <= 256)
            launch_topk(std::integral_constant<int, 4>{});
        else if (a.N <= 512)
            launch_topk(std::integral_constant<int, 8>{});
        else if (a.N <= 768)
            launch_topk(std::integral_constant<int, 12>{});
        else if (a.N <= 1024)
            launch_topk(std::integral_constant<int, 16>{});
        else if (a.N <= 1536)
            launch_topk(std::integral_constant<int, 24>{});
        else
            launch_topk(std::integral_constant<int, 32>{});
    }
    if (shared_y) {
        if constexpr (sizeof(E) == 2) {
            if (p.skinny)
                skinny_kernel<Shared2<bf16>><<<dim3(cdiv(a.d, 16), cdiv(a.T, 64)), b1024, 0, st>>>(a);
            else
                launch_g2<Shared2<bf16>, G2Small>(a, cdiv(a.T, G2Small::BM), cdiv(a.d, G2Small::BN), st);
        } else {
            gemm_simt_kernel<Shared2<float>><<<dim3(cdiv(a.T, kSimtM), cdiv(a.d, kSimtN)), b256, 0, st>>>(a);
        }
    }
    // 3. dispatch
    mark(2);
    const size_t lds = dispatch_lds_bytes(a.N);
    if (a.self_route) {
        // none: the streaming FFN finds its rows from the ids
    } else if (p.nblk == 1) {
        dispatch_one_block_kernel<<<1, b1024, lds, st>>>(a);
    } else {
        dispatch_count_kernel<<<p.nblk, b1024, lds, st>>>(a);
        dispatch_scan_kernel<<<1, b1024, lds, st>>>(a, p.nblk);
        dispatch_scatter_kernel<<<p.nblk, b1024, lds, st>>>(a);
    }
    // 4. expert FFN
    const unsigned mt = (unsigned)p.max_tiles;
    if constexpr (sizeof(E) == 2) {
        if (p.path == LMOE_PATH_STREAM) {
            // The streaming FFN is one kernel; when both of its stage events
            // are given (and the stream is not being captured) they are the
            // kernel's own start and end, recorded with its launch, rather
            // than separate event packets around it.
            hipEvent_t ev0 = events ? static_cast<hipEvent_t>(events[3]) : nullptr;
            hipEvent_t ev1 = events ? static_cast<hipEvent_t>(events[4]) : nullptr;
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            if (ev0 && ev1 && hipStreamIsCapturing(st, &cap) != hipSuccess) cap = hipStreamCaptureStatusActive;
            const bool own = ev0 && ev1 && cap == hipStreamCaptureStatusNone;
            if (!own) mark(3);
            // (self-routed: the routed ids staged in dynamic LDS)
            const size_t dyn = self_route_lds_bytes(a.T, a.K, a.self_route != 0);
            auto launch = [&](auto kernel, dim3 grid) {
                if (own) {
                    void* args[] = {&a};
                    const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, b256, args,
                                                            dyn, st, ev0, ev1, 0);
                    if (e != hipSuccess) ext_err = e;
                } else {
                    kernel<<<grid, b256, dyn, st>>>(a);
                }
            };
            // One grid row per possibly active expert: at most min(n_ffn,
            // T*K) experts receive rows, so small batches launch no
            // workgroups that could only return.  (MXFP4 pairs slices across
            // the grid in chunks of 16 workgroups: a multiple of 8 experts
            // keeps every chunk whole.)
            const int rows_g = (int)std::min<long long>(a.n_ffn, (long long)a.T * a.K);
            const dim3 g(p.nsplit, p.wfmt == 2 ? (unsigned)(cdiv(rows_g, 8) * 8) : (unsigned)rows_g);
            auto stream = [&](auto fmt) {
                constexpr int F = decltype(fmt)::value;
                if (F <= 1 && p.ms == 256)
                    launch(ffn_stream_kernel<256, F <= 1 ? F : 0>, g);
                else if (p.ms == 128)
                    launch(ffn_stream_kernel<128, F>, g);
                else
                    launch(ffn_stream_kernel<64, F>, g);
            };
            if (p.wfmt == 1)
                stream(std::integral_constant<int, 1>{});
            else if (p.wfmt == 2 && p.ms == 256 && a.l % 256 == 0)
                launch(ffn_stream_mx_kernel<256>, g);   // 16-byte code loads
            else if (p.wfmt == 2 && p.ms == 128 && a.l % 256 == 0 && a.m % 128 == 0)
                launch(ffn_stream_mx_kernel<128>, g);
            else if (p.wfmt == 2)
                stream(std::integral_constant<int, 2>{});
            else
                stream(std::integral_constant<int, 0>{});
            if (!own) mark(4);
        } else {
            mark(3);
            auto ffn = [&](auto f1, auto f2) {
                using F1 = decltype(f1);
                using F2 = decltype(f2);
                if (p.ffn_large) {
                    launch_g2<F1, G2Large>(a, (int)mt, cdiv(a.m, G2Large::BN), st);
                    mark(4);
                    launch_g2<F2, G2Large>(a, (int)mt, cdiv(a.l, G2Large::BN), st);
                } else if (p.tall_rows > 0) {
                    // each product: the heavy experts' tall tiles, then the
                    // light experts' tiles
                    LayerArgs at = a;
                    at.tiles = a.tiles_tall;
                    at.n_tiles = a.n_tiles_tall;
                    const int mtt = (int)p.max_tiles_tall;
                    launch_g2<F1, G2Large>(at, mtt, cdiv(a.m, G2Large::BN), st);
                    launch_g2<F1, G2Small>(a, (int)mt, cdiv(a.m, G2Small::BN), st);
                    mark(4);
                    launch_g2<F2, G2Large>(at, mtt, cdiv(a.l, G2Large::BN), st);
                    launch_g2<F2, G2Small>(a, (int)mt, cdiv(a.l, G2Small::BN), st);
                } else {
                    launch_g2<F1, G2Small>(a, (int)mt, cdiv(a.m, G2Small::BN), st);
                    mark(4);
                    launch_g2<F2, G2Small>(a, (int)mt, cdiv(a.l, G2Small::BN), st);
                }
            };
            if (p.wfmt == 1)
                ffn(Ffn1Q{}, Ffn2Q{});
            else if (p.wfmt == 2)
                ffn(Ffn1X{}, Ffn2X{});
            else
                ffn(Ffn1<bf16>{}, Ffn2<bf16, YT>{});
        }
    } else {
        mark(3);
        gemm_simt_kernel<Ffn1<float>><<<dim3(mt, cdiv(a.m, kSimtN)), b256, 0, st>>>(a);
        mark(4);
        gemm_simt_kernel<Ffn2<float, float>><<<dim3(mt, cdiv(a.l, kSimtN)), b256, 0, st>>>(a);
    }
    // 5. combine
    mark(5);
    if constexpr (sizeof(E) == 2) {
        if (p.path == LMOE_PATH_STREAM)
            launch_combine<E, f16, true>(a, p.nsplit, st);   // the streaming FFN's fp16 partials
        else
            launch_combine<E, YT, false>(a, 1, st);
    } else {
        launch_combine<E, YT, false>(a, 1, st);   // (the float32 layer has no streaming path)
    }
    // 6. back to d with the residual
    mark(6);
    if (!a.standard && a.m_s == 0) {
        if constexpr (sizeof(E) == 2) {
            if (p.skinny)
                skinny_kernel<Up<bf16>><<<dim3(cdiv(a.d, 16), cdiv(a.T, 64)), b1024, 0, st>>>(a);
            else
                launch_g2<Up<bf16>, UpTile>(a, cdiv(a.T, UpTile::BM), cdiv(a.d, UpTile::BN), st);
        } else {
            gemm_simt_kernel<Up<float>><<<dim3(cdiv(a.T, kSimtM), cdiv(a.d, kSimtN)), b256, 0, st>>>(a);
        }
    } else if (!a.standard) {
        // with the shared expert: its second product is the rest of the
        // up-projection's reduction (bf16), or its float32 output is added
        // in the epilogue (float32)
        if constexpr (sizeof(E) == 2) {
            if (p.skinny)
                skinny_kernel<UpCat<bf16>><<<dim3(cdiv(a.d, 16), cdiv(a.T, 64)), b1024, 0, st>>>(a);
            else
                launch_g2<UpCat<bf16>, UpTile>(a, cdiv(a.T, UpTile::BM), cdiv(a.d, UpTile::BN), st);
        } else {
            gemm_simt_kernel<UpShared<float>><<<dim3(cdiv(a.T, kSimtM), cdiv(a.d, kSimtN)), b256, 0, st>>>(a);
        }
    }
    mark(7);
    return ext_err;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
}

// The buffers a forward writes (out, the routing buffers, the workspace) must
// not overlap one another or any array it reads; a NULL pointer spans nothing.
int check_aliasing(const Plan& p, const lmoe_dims& d, int K, bool standard, const void* x, const void* W_down,
                   const void* W_router, const void* W1, const void* W2, const void* W_up, const void* W_s1,
                   const void* W_s2, const void* w1s, const void* w2s, const void* zc_const, const float* bias,
                   const void* out, const int32_t* ids, const float* gates, const void* workspace) {
    struct Span {
        const void* ptr;
        size_t bytes;
        const char* name;
    };
    const size_t es = p.es, T = d.T, dd = d.d, l = d.l, N = d.N, m = d.m, nr = p.nr, ms = d.m_shared;
    // expert weight bytes per element: the layer's type, an FP8 code, half an MXFP4 byte
    const double wb = p.wfmt == 0 ? (double)es : (p.wfmt == 1 ? 1.0 : 0.5);
    const size_t wexp = (size_t)(wb * (double)(N * m * l));
    const size_t s1b = p.wfmt == 1 ? N * m * 4 : N * m * (l / 32), s2b = p.wfmt == 1 ? N * l * 4 : N * l * (m / 32);
    const Span in[] = {
        {x, T * dd * es, "x"},
        {standard ? nullptr : W_down, l * dd * es, "W_down"},
        {W_router, nr * dd * es, "W_router"},
        {W1, wexp, "W1"},
        {W2, wexp, "W2"},
        {standard ? nullptr : W_up, dd * l * es, "W_up"},
        {W_s1, ms * dd * es, "W_shared1"},
        {W_s2, dd * ms * es, "W_shared2"},
        {p.wfmt ? w1s : nullptr, s1b, "W1_scale"},
        {p.wfmt ? w2s : nullptr, s2b, "W2_scale"},
        {zc_const, (size_t)d.n_const * l * es, "zc_const"},
        {bias, nr * 4, "router_bias"},
    };
    const size_t tk = T * (size_t)K;
    const Span wr[] = {
        {out, T * dd * es, "out"},
        {ids, tk * 4, "topk_ids"},
        {gates, tk * 4, "topk_gates"},
        {workspace, p.total, "the workspace"},
    };
    for (size_t i = 0; i < sizeof wr / sizeof wr[0]; ++i) {
        if (!wr[i].ptr) continue;
        for (const Span& r : in)
            if (r.ptr && overlaps(wr[i].ptr, wr[i].bytes, r.ptr, r.bytes))
                return fail(LMOE_EINVAL, "%s must not alias %s", wr[i].name, r.name);
        for (size_t j = 0; j < i; ++j)
            if (wr[j].ptr && overlaps(wr[i].ptr, wr[i].bytes, wr[j].ptr, wr[j].bytes))
                return fail(LMOE_EINVAL, "%s must not alias %s", wr[i].name, wr[j].name);
    }
    return LMOE_OK;
}

// Device memory of latentmoe_forward_noalloc, for callers that cannot
// allocate: one copy of this array per device, held until the process ends.
// In host code `scratch` names a host-side stand-in, not the device array:
// host code uses only the address hipGetSymbolAddress gives for the current
// device (scratch_address()).
constexpr size_t kScratchBytes = LMOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on the current device, taken once per
// device (with that device current), or NULL with the failure recorded.
void* scratch_address() {
    constexpr int kMaxDevices = 64;
    static std::once_flag flags[kMaxDevices];
    static void* addr[kMaxDevices];
    static hipError_t err[kMaxDevices];
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(LMOE_EHIP, "hipGetDevice failed or device %d is out of range: %s", dev, hipGetErrorString(e));
        return nullptr;
    }
    std::call_once(flags[dev], [dev] {
        void* p = nullptr;
        err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        addr[dev] = err[dev] == hipSuccess ? p : nullptr;
    });
    if (err[dev] != hipSuccess || !addr[dev]) {
        fail(LMOE_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(err[dev]));
        return nullptr;
    }
    return addr[dev];
}

}  // namespace

extern "C" {

size_t latentmoe_workspace_bytes(const lmoe_dims* dims, int32_t K) {
    const Plan p = make_plan(dims, K);
    return p.status == LMOE_OK ? p.total : 0;
}

int latentmoe_resolved_path(const lmoe_dims* dims, int32_t K) {
    const Plan p = make_plan(dims, K);
    return p.status == LMOE_OK ? p.path : p.status;
}

int latentmoe_workspace_layout(const lmoe_dims* dims, int32_t K, lmoe_ws_layout* layout) {
    if (!layout) return fail(LMOE_EINVAL, "layout is NULL");
    const Plan p = make_plan(dims, K);
    if (p.status != LMOE_OK) return p.status;
    layout->counts = p.counts;
    layout->offsets = p.offsets;
    layout->perm = p.perm;
    layout->slot_of = p.slot_of;
    layout->n_active = p.n_active;
    layout->written = p.skinny ? 0 : 1;
    return LMOE_OK;
}

static int forward_impl(const void* x, const void* W_down, const void* W_router, const void* W1, const void* W2,
                        const void* W_up, const void* W_s1, const void* W_s2, const void* w1s, const void* w2s,
                        const void* zc_const, int32_t K, void* out, const lmoe_dims* dims, const float* router_bias,
                        int32_t* topk_ids, float* topk_gates, void* workspace, size_t workspace_bytes,
                        void* stream, void* const* events) {
    g_last_error.clear();
    const Plan p = make_plan(dims, K);
    if (p.status != LMOE_OK) return p.status;
    const lmoe_dims& d = *dims;
    if (!x || !W_router || !W1 || !W2 || !out)
        return fail(LMOE_EINVAL, "x, W_router, W1, W2 and out must be non-NULL");
    if ((W_down == nullptr) != (W_up == nullptr))
        return fail(LMOE_EINVAL, "W_down and W_up must be both NULL (standard MoE) or both set");
    const bool standard = W_down == nullptr;
    if ((d.m_shared > 0) != (W_s1 != nullptr) || (W_s1 == nullptr) != (W_s2 == nullptr))
        return fail(LMOE_EINVAL, "W_shared1 and W_shared2 must be both set when m_shared > 0 and both NULL when "
                                 "m_shared == 0 (m_shared=%d)", d.m_shared);
    if (standard && d.l != d.d) return fail(LMOE_EINVAL, "standard mode (no projections) needs l == d");
    if ((p.wfmt != 0) != (w1s != nullptr) || (w1s == nullptr) != (w2s == nullptr))
        return fail(LMOE_EINVAL, "W1_scale and W2_scale must be both set for FP8 / MXFP4 experts and both NULL "
                                 "otherwise");
    if (p.wfmt == 1 && ((reinterpret_cast<uintptr_t>(w1s) & 15) != 0 || (reinterpret_cast<uintptr_t>(w2s) & 15) != 0))
        return fail(LMOE_EINVAL, "FP8 W1_scale and W2_scale must be 16-byte aligned");
    if ((d.n_const > 0) != (zc_const != nullptr))
        return fail(LMOE_EINVAL, "zc_const must be set when n_const > 0 and NULL otherwise (n_const=%d)", d.n_const);
    if (p.wfmt == 2 && ((reinterpret_cast<uintptr_t>(w1s) & 7) != 0 || (reinterpret_cast<uintptr_t>(w2s) & 7) != 0))
        return fail(LMOE_EINVAL, "MXFP4 W1_scale and W2_scale must be 8-byte aligned");
    if (!workspace) return fail(LMOE_EWORKSPACE, "workspace is NULL");
    if (const int rc = check_aliasing(p, d, K, standard, x, W_down, W_router, W1, W2, W_up, W_s1, W_s2, w1s, w2s,
                                      zc_const, router_bias, out, topk_ids, topk_gates, workspace))
        return rc;
    if (workspace_bytes < p.total)
        return fail(LMOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, p.total);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(LMOE_EINVAL, "workspace must be 256-byte aligned");
    const void* ptrs[] = {x, W_down, W_router, W1, W2, W_up, W_s1, W_s2, zc_const, out};
    for (const void* q : ptrs)
        if (q && (reinterpret_cast<uintptr_t>(q) & 15) != 0)
            return fail(LMOE_EINVAL, "tensor pointers must be 16-byte aligned");

    init_once();
    char* ws = static_cast<char*>(workspace);
    LayerArgs a{};
    a.x = x;
    a.W_down = W_down;
    a.W_router = W_router;
    a.W1 = W1;
    a.W2 = W2;
    a.W_up = W_up;
    a.W_s1 = W_s1;
    a.W_s2 = W_s2;
    a.m_s = d.m_shared;
    a.bias = router_bias;
    a.w1s = p.wfmt == 1 ? static_cast<const float*>(w1s) : nullptr;
    a.w2s = p.wfmt == 1 ? static_cast<const float*>(w2s) : nullptr;
    a.w1x = p.wfmt == 2 ? static_cast<const uint8_t*>(w1s) : nullptr;
    a.w2x = p.wfmt == 2 ? static_cast<const uint8_t*>(w2s) : nullptr;
    a.out = out;
    a.T = d.T;
    a.d = d.d;
    a.l = d.l;
    a.N = p.nr;
    a.n_ffn = d.N;
    a.n_zero = d.n_zero;
    a.n_copy = d.n_copy;
    a.zc = zc_const;
    a.m = d.m;
    a.K = K;
    a.standard = standard ? 1 : 0;
    a.z_w = ws + p.z;
    a.z = standard ? x : (const void*)(ws + p.z);
    a.logits = reinterpret_cast<float*>(ws + p.logits);
    a.ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + p.ids);
    a.gates = topk_gates ? topk_gates : reinterpret_cast<float*>(ws + p.gates);
    a.counts = reinterpret_cast<int32_t*>(ws + p.counts);
    a.offsets = reinterpret_cast<int32_t*>(ws + p.offsets);
    a.perm = reinterpret_cast<int32_t*>(ws + p.perm);
    a.slot_of = reinterpret_cast<int32_t*>(ws + p.slot_of);
    a.blk_counts = reinterpret_cast<int32_t*>(ws + p.blk_counts);
    a.blk_offsets = reinterpret_cast<int32_t*>(ws + p.blk_offsets);
    a.tiles = reinterpret_cast<int2*>(ws + p.tiles);
    a.n_tiles = reinterpret_cast<int32_t*>(ws + p.n_tiles);
    a.tiles_tall = reinterpret_cast<int2*>(ws + p.tiles_tall);
    a.n_tiles_tall = reinterpret_cast<int32_t*>(ws + p.n_tiles_tall);
    a.tall_rows = p.tall_rows;
    a.active = reinterpret_cast<int32_t*>(ws + p.active);
    a.n_active = reinterpret_cast<int32_t*>(ws + p.n_active);
    a.abuf = ws + p.abuf;
    a.ybuf = ws + p.ybuf;
    a.s = ws + p.s;
    a.part = ws + p.part;
    a.a_s = d.m_shared > 0 ? ws + p.a_s : nullptr;
    // y_s (the shared expert's float32 output) only where it is kept apart:
    // float32 layers and standard mode
    a.y_s = (d.m_shared > 0 && (!p.bf16 || standard)) ? reinterpret_cast<float*>(ws + p.y_s) : nullptr;
    a.tail_part = reinterpret_cast<float*>(ws + p.tail);
    a.tile_rows = p.tile_rows;
    a.y_planes = p.nsplit;
    a.y_row_bytes = d.l * (int)p.es;   // fp16 (scaled) outputs or partials, or float32
    a.self_route = p.skinny ? 1 : 0;

    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const hipError_t launch_err =
        p.bf16 ? launch_all<bf16, f16>(p, a, st, events) : launch_all<float, float>(p, a, st, events);
    const hipError_t last_err = hipGetLastError();
    const hipError_t err = launch_err != hipSuccess ? launch_err : last_err;
    if (err != hipSuccess) return fail(LMOE_EHIP, "HIP launch failed: %s", hipGetErrorString(err));
    return LMOE_OK;
}

// The entry points other than latentmoe_forward_ex take no FP8 / MXFP4 experts and
// no zero-computation experts.
static int plain_options_only(const lmoe_dims* dims) {
    if (dims && dims->expert_format != LMOE_EXPERTS_DENSE)
        return fail(LMOE_EINVAL, "FP8 / MXFP4 experts go through latentmoe_forward_ex");
    if (dims && (dims->n_zero | dims->n_copy | dims->n_const) != 0)
        return fail(LMOE_EINVAL, "zero-computation experts go through latentmoe_forward_ex");
    return LMOE_OK;
}

int latentmoe_forward(const void* x, const void* W_down, const void* W_router, const void* W1, const void* W2,
                      const void* W_up, int32_t K, void* out, const lmoe_dims* dims, const float* router_bias,
                      int32_t* topk_ids, float* topk_gates, void* workspace, size_t workspace_bytes,
                      void* stream) {
    if (dims && dims->m_shared != 0)
        return fail(LMOE_EINVAL, "m_shared=%d: a shared expert goes through latentmoe_forward_shared",
                    dims->m_shared);
    if (const int rc = plain_options_only(dims)) return rc;
    return forward_impl(x, W_down, W_router, W1, W2, W_up, nullptr, nullptr, nullptr, nullptr, nullptr, K, out, dims,
                        router_bias, topk_ids, topk_gates, workspace, workspace_bytes, stream, nullptr);
}

int latentmoe_forward_shared(const void* x, const void* W_down, const void* W_router, const void* W1,
                             const void* W2, const void* W_up, const void* W_shared1, const void* W_shared2,
                             int32_t K, void* out, const lmoe_dims* dims, const float* router_bias,
                             int32_t* topk_ids, float* topk_gates, void* workspace, size_t workspace_bytes,
                             void* stream) {
    if (dims && dims->m_shared <= 0)
        return fail(LMOE_EINVAL, "latentmoe_forward_shared needs m_shared > 0 (got %d)", dims->m_shared);
    if (const int rc = plain_options_only(dims)) return rc;
    return forward_impl(x, W_down, W_router, W1, W2, W_up, W_shared1, W_shared2, nullptr, nullptr, nullptr, K, out, dims,
                        router_bias, topk_ids, topk_gates, workspace, workspace_bytes, stream, nullptr);
}

int latentmoe_forward_timed(const void* x, const void* W_down, const void* W_router, const void* W1,
                            const void* W2, const void* W_up, const void* W_shared1, const void* W_shared2,
                            int32_t K, void* out, const lmoe_dims* dims, const float* router_bias,
                            int32_t* topk_ids, float* topk_gates, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events) {
    if (!events) return fail(LMOE_EINVAL, "events is NULL");
    if (const int rc = plain_options_only(dims)) return rc;
    return forward_impl(x, W_down, W_router, W1, W2, W_up, W_shared1, W_shared2, nullptr, nullptr, nullptr, K, out, dims,
                        router_bias, topk_ids, topk_gates, workspace, workspace_bytes, stream, events);
}

int latentmoe_forward_noalloc(const void* x, const void* W_down, const void* W_router, const void* W1,
                              const void* W2, const void* W_up, int32_t K, void* out, const lmoe_dims* dims,
                              const float* router_bias, int32_t* topk_ids, float* topk_gates, void* stream) {
    if (dims && dims->m_shared != 0)
        return fail(LMOE_EINVAL, "m_shared=%d: a shared expert goes through latentmoe_forward_shared",
                    dims->m_shared);
    if (const int rc = plain_options_only(dims)) return rc;
    const Plan p = make_plan(dims, K);
    if (p.status != LMOE_OK) return p.status;
    if (p.total > kScratchBytes)
        return fail(LMOE_EUNSUPPORTED, "these dims need %zu bytes of workspace; latentmoe_forward_noalloc has %zu",
                    p.total, kScratchBytes);
    void* ws = scratch_address();
    if (!ws) return LMOE_EHIP;
    return forward_impl(x, W_down, W_router, W1, W2, W_up, nullptr, nullptr, nullptr, nullptr, nullptr, K, out, dims,
                        router_bias, topk_ids, topk_gates, ws, kScratchBytes, stream, nullptr);
}

int latentmoe_forward_ex(const lmoe_args* g, int32_t K, const lmoe_dims* dims) {
    if (!g) return fail(LMOE_EINVAL, "args is NULL");
    return forward_impl(g->x, g->W_down, g->W_router, g->W1, g->W2, g->W_up, g->W_shared1, g->W_shared2,
                        g->W1_scale, g->W2_scale, g->zc_const, K, g->out, dims, g->router_bias, g->topk_ids, g->topk_gates,
                        g->workspace, g->workspace_bytes, g->stream, g->events);
}

const char* latentmoe_status_string(int status) {
    switch (status) {
        case LMOE_OK: return "ok";
        case LMOE_EINVAL: return "invalid argument";
        case LMOE_EUNSUPPORTED: return "unsupported arguments";
        case LMOE_EWORKSPACE: return "workspace missing or too small";
        case LMOE_EHIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

const char* latentmoe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
