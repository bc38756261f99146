// Shape-grouped, batched Newton-Schulz chain on gfx950 MFMA.
//
// Method: "Record: Combined 3-Layer Recurrence + Parallel Residuals + Polar
// Express + Brotli" (PR #1396), "Techniques Combined": the Muon update is
// orthogonalised by a Newton-Schulz iteration with a per-step coefficient
// schedule.  Iteration k with row (a, b, c) of the table:
//     A = X X^T            (kGram,   m x m, contraction over n)
//     B = b A + c A A      (kSquare, m x m, contraction over m)
//     X <- a X + B X       (kUpdate, m x n, contraction over m)
// with X short-side-first (m <= n).
//
// bf16 numerics.  X is kept to ~16 significant bits as hi = rne(X) in bf16
// plus its remainder: one byte per element in units of 2^-15 of hi's binade
// for the base groups (lo8_insert), a second bf16 plane for the compensated
// ones, whose products use it as an MFMA operand.  MFMA operands are bf16 and
// accumulate in fp32.  A is split into hi + lo and A A is formed as
// hi*hi + hi*lo + lo*hi, because the plain bf16 square loses the small
// singular directions that the iteration amplifies; the a X term always uses
// hi + lo.  In the base groups the two cross products run on e4m3 operands
// (fp8 MFMA, see below).
//   base:        A = Xh Xh^T,  B X = Bh Xh
//   compensated: A = Xh Xh^T + Xh Xl^T + Xl Xh^T,  B X = Bh Xh + Bl Xh + Bh Xl
// The base products keep the error within 2e-2 of float64 once the short side
// has enough singular values to average the bf16 rounding (>= 192); smaller
// groups, or every group on request, run compensated (~1e-4).  The fp32
// precision runs the same phases on fp32 MFMA (v_mfma_f32_32x32x2_f32).
//
// Tiling.  One workgroup per 128 x 128 output tile, 64 x 64 per wave as 2 x 2
// v_mfma_f32_32x32x16_bf16 accumulators: 4 wave64s (2 x 2) for the update, and
// two such groups splitting the K stages for the Gram and square, whose few
// (upper-triangle) tiles would otherwise leave one wave per SIMD.  K is staged
// through LDS 128 or 256 bytes per row at a time with the next stage's global
// loads in flight during the MFMAs: through registers, or for the Gram
// straight into LDS (global_load_lds_dwordx4).  A and B are symmetric:
// only tiles with ti <= tj are computed and each is written twice (as is and
// mirrored).  Epilogues go through LDS so that every global access is 16
// bytes wide.  All work of one phase for the matrices of one stream (every
// shape group the host put there) is one launch; job indices are remapped so
// that the tiles of one matrix share an XCD (and its L2).  Workspace dimensions are padded to 128 with zeros,
// which the iteration keeps at zero, so no loop needs a bounds check.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "ns_device.h"

namespace muon {

namespace {

template <int PHASE>
__device__ inline bool decode_job(const NsArgs& args, Job& j) {
    const int job = xcd_job_index();
    if (job >= args.total_jobs) return false;
    int g = 0;
    while (g + 1 < args.ngroups && job >= args.g[g + 1].job_begin) ++g;
    const NsGroup& G = args.g[g];
    const int tm = G.M / kTile, tn = G.N / kTile;
    const int local = job - G.job_begin;
    if (PHASE == kUpdate) {
        // column-panel-major: the tm row tiles that read the same X column panel
        // are neighbours in job order (and so on one XCD at about the same time)
        const int per = tm * tn;
        j.slot = local / per;
        const int t = local - j.slot * per;
        j.tj = t / tm;
        j.ti = t - j.tj * tm;
    } else {
        const int per = tm * (tm + 1) / 2;
        j.slot = local / per;
        int t = local - j.slot * per;
        int ti = 0;
        while (t >= tm - ti) { t -= tm - ti; ++ti; }
        j.ti = ti;
        j.tj = ti + t;
    }
    j.g = g;
    return true;
}

// The update X' = s (a X + B X) of one phase: one 128 x 128 tile of X' per
// workgroup (update_tile), jobs in column-panel order.
template <int PREC, bool COMP, bool FUSE>
__global__ __launch_bounds__(kThreads, (PREC == kNsBf16 && !COMP && !FUSE) ? 3 : 1) void ns_update_kernel(
    const NsArgs args) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    Job job;
    if (!decode_job<kUpdate>(args, job)) return;
    const NsGroup& G = args.g[job.g];
    const UpdateCtx c{args.a, args.first, args.src, args.keep, args.decay, args.one_minus_decay};
    update_tile<PREC, COMP, FUSE>(G, job, c, args.apply[G.apply_begin + job.slot], lds);
}

// Gram and square with two K groups per workgroup.  These phases have few
// output tiles (the upper triangle of m x m), so a launch leaves one wave per
// SIMD and its LDS and MFMA latencies exposed.  Here 8 waves share a tile:
// waves 0-3 take the even K stages and waves 4-7 the odd ones, each group
// with its own LDS stage, so every SIMD holds two waves that interleave.  The
// two partial accumulators meet in a full-tile fp32 LDS staging buffer
// (group 0 writes, group 1 adds) before the 512-thread epilogue.
constexpr int kSymThreads = 2 * kThreads;
constexpr int kSymStageBytes = kTile * kStagePitch * 4;   // a full tile of fp32
// epilogue LDS: the staged tile, then the partial-sum exchange (2 groups x 4
// waves x 8 chunks x 64 lanes x 16 bytes)
constexpr int kSymEpilogueBytes = kSymStageBytes + 2 * 4 * 8 * kWave * 16;

template <int PHASE, int PREC, bool COMP>
__global__ __launch_bounds__(kSymThreads) void ns_sym_kernel(const NsArgs args) {
    static_assert(PHASE == kGram || PHASE == kSquare, "symmetric phases only");
    typedef typename Elem<PREC>::T T;
    constexpr bool kSplit = (PREC == kNsBf16) && (PHASE == kSquare || COMP);
    constexpr bool kDma = ns_sym_dma(PHASE, PREC, COMP);
    constexpr int kRB = ns_sym_stage_bytes(PHASE, PREC, COMP, kDma);
    constexpr int kBK = kRB / (int)sizeof(T);
    constexpr int kSlot = Stage<kRB>::kSlot;
    constexpr int kStageTiles = kSplit ? 4 : 2;
    // base bf16: A lo is an e4m3 byte plane and the square's cross terms run on the fp8 MFMA
    constexpr bool kF8 = NS_SQ_FP8 != 0 && PREC == kNsBf16 && !COMP;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    Job job;
    if (!decode_job<PHASE>(args, job)) return;   // uniform over the workgroup
    const NsGroup& G = args.g[job.g];
    const int M = G.M, N = G.N;
    const int tid = threadIdx.x;
    const int kg = tid / kThreads;                 // K group
    const int lane = tid % kWave, wave = (tid % kThreads) / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const bool diag = job.ti == job.tj;
    const size_t xplane = (size_t)job.slot * M * N;
    const size_t aplane = (size_t)job.slot * M * M;

    auto tile = [&](int which) -> uint8_t* {
        if (diag && which == 1) which = 0;
        if (diag && which == 3) which = 2;
        return lds + (kg * kStageTiles + which) * kSlot;
    };
    const uint8_t *ga, *gb, *gal, *gbl;
    size_t ld_bytes;
    int K;
    if (PHASE == kGram) {
        const T* xh = static_cast<const T*>(G.x[args.src]) + xplane;
        const T* xl = static_cast<const T*>(G.xl[args.src]) + xplane;
        ld_bytes = (size_t)N * sizeof(T);
        ga = reinterpret_cast<const uint8_t*>(xh + (size_t)job.ti * kTile * N);
        gb = reinterpret_cast<const uint8_t*>(xh + (size_t)job.tj * kTile * N);
        gal = reinterpret_cast<const uint8_t*>(xl + (size_t)job.ti * kTile * N);
        gbl = reinterpret_cast<const uint8_t*>(xl + (size_t)job.tj * kTile * N);
        K = N;
    } else {
        const T* ah = static_cast<const T*>(G.a_hi) + aplane;
        const T* al = static_cast<const T*>(G.a_lo) + aplane;
        ld_bytes = (size_t)M * sizeof(T);
        ga = reinterpret_cast<const uint8_t*>(ah + (size_t)job.ti * kTile * M);
        gb = reinterpret_cast<const uint8_t*>(ah + (size_t)job.tj * kTile * M);
        gal = reinterpret_cast<const uint8_t*>(al + (size_t)job.ti * kTile * M);
        gbl = reinterpret_cast<const uint8_t*>(al + (size_t)job.tj * kTile * M);
        K = M;
    }

    floatx16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
    // zeroed here, ahead of the first operand loads (otherwise the zeros are
    // rematerialised into registers that still wait for those loads)
    asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));

    // MFMAs of one LDS stage.  frag(t, row, kc) is the lane's 16-byte operand
    // chunk (K chunk kc of 16 elements) of row `row` of tile t.
    auto compute_with = [&](auto frag, const uint8_t* t_a, const uint8_t* t_b, const uint8_t* t_al,
                            const uint8_t* t_bl) {
        constexpr int kKC = kRB / 32;
        if constexpr (PREC == kNsBf16 && !kSplit) {
            // bf16 base: the fragments of chunk kc + 2 are read while the MFMAs
            // of chunk kc run.  The scheduling groups (one fragment read after
            // each MFMA) keep the compiler from moving the reads next to the
            // MFMAs that use them.
            constexpr int kDist = 2, kBufs = kDist + 1;
            static_assert(kKC >= kDist, "at least kDist chunks per stage");
            u32x4 f[kBufs][4];
            auto read = [&](int kc, u32x4* d) {
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) d[mi] = frag(t_a, wm * 64 + mi * 32 + lane % 32, kc);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) d[2 + ni] = frag(t_b, wn * 64 + ni * 32 + lane % 32, kc);
            };
#pragma unroll
            for (int kc = 0; kc < kDist; ++kc) read(kc, f[kc]);
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * kDist, 0);   // DS reads
#pragma unroll
            for (int kc = 0; kc < kKC; ++kc) {
                if (kc + kDist < kKC) read(kc + kDist, f[(kc + kDist) % kBufs]);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        mfma_chunk<PREC>(acc[mi][ni], f[kc % kBufs][mi], f[kc % kBufs][2 + ni]);
                if (kc + kDist < kKC) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                    }
                } else {
                    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) fa[mi] = frag(t_a, wm * 64 + mi * 32 + lane % 32, kc);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) fb[ni] = frag(t_b, wn * 64 + ni * 32 + lane % 32, kc);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) mfma_chunk<PREC>(acc[mi][ni], fa[mi], fb[ni]);
            if (kSplit) {
                u32x4 fal[2], fbl[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) fal[mi] = frag(t_al, wm * 64 + mi * 32 + lane % 32, kc);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) fbl[ni] = frag(t_bl, wn * 64 + ni * 32 + lane % 32, kc);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        mfma_chunk<PREC>(acc[mi][ni], fa[mi], fbl[ni]);
                        mfma_chunk<PREC>(acc[mi][ni], fal[mi], fb[ni]);
                    }
            }
        }
    };
    const int nk = K / kBK;
    // First Gram: the Frobenius scale of X0 from the per-row sums of squares
    // (every tile of a matrix computes the same bits; tile (0, 0) stores it for
    // the later phases).  Its 8 floats of LDS (at red_off, clear of the first
    // stage's LDS) are read before the barrier that precedes the first LDS
    // write of operands.
    float fscale = 0.f, fv[4];
    const bool fold = PHASE == kGram && args.first && args.fold_frob;
    const FrobSlot fs = fold ? args.frob[G.frob_begin + job.slot] : FrobSlot{0, 0};
    if (fold) frob_prefetch(args.rowsq + fs.off, fs.rows, fv);
    auto fold_frob = [&](int red_off) {
        if (fold) {
            fscale = frob_finish(args.rowsq + fs.off, fs.rows, fv, reinterpret_cast<float*>(lds + red_off));
            if (job.ti == 0 && job.tj == 0 && tid == 0) G.scale[job.slot] = fscale;
        }
    };

    if constexpr (kDma) {
        // Direct global -> LDS loads (global_load_lds_dwordx4, lane l writes the
        // 16 bytes at block base + 16 l).  Two LDS buffers; buffer b holds, per
        // group, the tiles [A hi, B hi, A lo, B lo] of one stage, rows of kRB
        // bytes without padding and the 16-byte chunk c of row r at c ^ swz(r),
        // which keeps the fragment reads free of bank conflicts.  Both groups
        // load and compute at the same time (group g: stages 2p + g); waits are
        // explicit: each wave waits for its own loads of the stage (vmcnt), a
        // barrier publishes them, and a second barrier frees the buffer for the
        // loads two stages ahead.
        constexpr int kC = kRB / 16;                       // 16-byte chunks per row
        constexpr int kTileBytes = kTile * kRB;
        constexpr int kBufBytes = 2 * kStageTiles * kTileBytes;
        constexpr int kPerTile = kTileBytes / 1024 / 4;    // loads per wave per tile
        auto swz = [](int row) { return (row / (16 / kC)) % kC; };
        auto dtile = [&](int buf, int which) -> const uint8_t* {
            if (diag && which == 1) which = 0;
            if (diag && which == 3) which = 2;
            return lds + buf * kBufBytes + (kg * kStageTiles + which) * kTileBytes;
        };
        auto dma_tile = [&](const uint8_t* src, int kt, int buf, int which) {
            uint8_t* dst = lds + buf * kBufBytes + (kg * kStageTiles + which) * kTileBytes;
#pragma unroll
            for (int j = 0; j < kPerTile; ++j) {
                const int q = j * 4 + wave;                      // 1 KB block: rows q*1024/kRB ..
                const int row = q * (1024 / kRB) + lane / kC;
                const int c = (lane % kC) ^ swz(row);
                __builtin_amdgcn_global_load_lds(src + (size_t)row * ld_bytes + (size_t)kt * kRB + c * 16,
                                                 (lds_ptr)(dst + q * 1024), 16, 0, 0);
            }
        };
        auto dma_stage = [&](int kt, int buf) {
            dma_tile(ga, kt, buf, 0);
            if (kSplit) dma_tile(gal, kt, buf, 2);
            if (!diag) {
                dma_tile(gb, kt, buf, 1);
                if (kSplit) dma_tile(gbl, kt, buf, 3);
            }
        };
        // loads per wave of one stage, by diagonal and off-diagonal tiles
        constexpr int kLoadsDiag = kPerTile * (kSplit ? 2 : 1);
        constexpr int kLoadsOff = 2 * kLoadsDiag;
        auto frag = [&](const uint8_t* t, int row, int kc) -> u32x4 {
            const int c = (2 * kc + lane / 32) ^ swz(row);
            return *reinterpret_cast<const u32x4*>(t + row * kRB + c * 16);
        };
        const int np = nk / 2;   // nk is even: K is a multiple of 128
        // the folded Frobenius sum first: no loads into registers may be in
        // flight once the direct loads start (waiting for them would also wait
        // for every direct load issued before)
        fold_frob(2 * kBufBytes);
        dma_stage(kg, 0);
        for (int p = 0; p < np; ++p) {
            const int buf = p & 1;
            if (p + 1 < np) {
                dma_stage(2 * (p + 1) + kg, buf ^ 1);
                if (diag) wait_vmcnt<kLoadsDiag>();
                else wait_vmcnt<kLoadsOff>();
            } else {
                wait_vmcnt<0>();
            }
            barrier_only();
            compute_with(frag, dtile(buf, 0), dtile(buf, 1), dtile(buf, 2), dtile(buf, 3));
            wait_lgkmcnt0();
            barrier_only();
        }
    } else if constexpr (kF8 && PHASE == kSquare) {
        // Base square, cross terms on the fp8 MFMA.  Per group and stage (64 K):
        // the bf16 Ah row tiles of both sides (for Ah Ah) and the e4m3 tiles of
        // Ah and Al of both sides (the byte planes the Gram stored), 80-byte
        // rows, K in natural order.  Same half-step schedule as the register
        // path below.
        static_assert(kRB == 128, "64 K per stage");
        const int sa = args.f8_sa, sl = args.f8_sl;
        uint8_t* const f8base = lds + 2 * 2 * kSlot;   // after both groups' bf16 tiles
        auto btile = [&](int side) -> uint8_t* { return lds + (kg * 2 + (diag ? 0 : side)) * kSlot; };
        auto ftile = [&](int which) -> uint8_t* {      // 0: Ah ti, 1: Ah tj, 2: Al ti, 3: Al tj
            if (diag && which == 1) which = 0;
            if (diag && which == 3) which = 2;
            return f8base + (kg * 4 + which) * kF8TileBytes;
        };
        const uint8_t* g8a = static_cast<const uint8_t*>(G.a_lo) + aplane + (size_t)job.ti * kTile * M;
        const uint8_t* g8b = static_cast<const uint8_t*>(G.a_lo) + aplane + (size_t)job.tj * kTile * M;
        const uint8_t* h8a = static_cast<const uint8_t*>(G.b_lo) + aplane + (size_t)job.ti * kTile * M;
        const uint8_t* h8b = static_cast<const uint8_t*>(G.b_lo) + aplane + (size_t)job.tj * kTile * M;
        const int t = tid % kThreads;
        NtLoader<kRB> la, lb;
        u32x4 l8a[2], l8b[2];   // Al bytes: row t/4 + 64q, 16-byte chunk t%4 of the stage's 64
        u32x4 h8va[2], h8vb[2]; // Ah e4m3 bytes, same mapping
        auto issue = [&](int kt) {
            la.load(ga, ld_bytes, kt * kRB);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const size_t o = (size_t)(t / 4 + 64 * q) * M + kt * 64 + (t % 4) * 16;
                l8a[q] = *reinterpret_cast<const u32x4*>(g8a + o);
                h8va[q] = *reinterpret_cast<const u32x4*>(h8a + o);
            }
            if (!diag) {
                lb.load(gb, ld_bytes, kt * kRB);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const size_t o = (size_t)(t / 4 + 64 * q) * M + kt * 64 + (t % 4) * 16;
                    l8b[q] = *reinterpret_cast<const u32x4*>(g8b + o);
                    h8vb[q] = *reinterpret_cast<const u32x4*>(h8b + o);
                }
            }
        };
        auto commit_side = [&](const NtLoader<kRB>& lh, const u32x4* l8, const u32x4* h8, int side) {
            lh.store(btile(side));
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *reinterpret_cast<u32x4*>(ftile(side) + (t / 4 + 64 * q) * kF8Pitch + (t % 4) * 16) = h8[q];
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *reinterpret_cast<u32x4*>(ftile(2 + side) + (t / 4 + 64 * q) * kF8Pitch + (t % 4) * 16) = l8[q];
        };
        auto commit = [&]() {
            commit_side(la, l8a, h8va, 0);
            if (!diag) commit_side(lb, l8b, h8vb, 1);
        };
        auto f8frag = [&](const uint8_t* tl, int row) -> v8i {
            const uint8_t* p = tl + row * kF8Pitch + (lane / 32) * 32;
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(p);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(p + 16);
            return v8i{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        };
        auto compute = [&]() {
            const uint8_t* ta = btile(0);
            const uint8_t* tb = btile(1);
#pragma unroll
            for (int kc = 0; kc < kRB / 32; ++kc) {
                u32x4 fa[2], fb[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) fa[mi] = lds_frag<kRB>(ta, wm * 64 + mi * 32 + lane % 32, kc, lane);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) fb[ni] = lds_frag<kRB>(tb, wn * 64 + ni * 32 + lane % 32, kc, lane);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) mfma_chunk<PREC>(acc[mi][ni], fa[mi], fb[ni]);
            }
            // Ah_i Al_j^T, then Al_i Ah_j^T: two A-side fragments and one B-side
            // fragment live at a time
#pragma unroll
            for (int term = 0; term < 2; ++term) {
                const int sx = term == 0 ? sa : sl, sy = term == 0 ? sl : sa;
                v8i fx[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) fx[mi] = f8frag(ftile(term == 0 ? 0 : 2), wm * 64 + mi * 32 + lane % 32);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const v8i fy = f8frag(ftile(term == 0 ? 3 : 1), wn * 64 + ni * 32 + lane % 32);
#pragma unroll
                    for (int mi = 0; mi < 2; ++mi)
                        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fx[mi], fy, acc[mi][ni], 0, 0, 0,
                                                                                     127 - sx, 0, 127 - sy);
                }
            }
        };
        if (kg < nk) issue(kg);
        __syncthreads();
        for (int h = 0; h <= nk; ++h) {
            if ((h & 1) == kg) {
                if (h < nk) {
                    commit();
                    if (h + 2 < nk) issue(h + 2);
                }
            } else if (h > 0 && h - 1 < nk) {
                compute();
            }
            __syncthreads();
        }
    } else {
        NtLoader<kRB> la, lb, lal, lbl;
        auto issue = [&](int kt) {
            const int kbyte = kt * kRB;
            la.load(ga, ld_bytes, kbyte);
            if (kSplit) lal.load(gal, ld_bytes, kbyte);
            if (!diag) {
                lb.load(gb, ld_bytes, kbyte);
                if (kSplit) lbl.load(gbl, ld_bytes, kbyte);
            }
        };
        auto commit = [&]() {
            la.store(tile(0));
            if (kSplit) lal.store(tile(2));
            if (!diag) {
                lb.store(tile(1));
                if (kSplit) lbl.store(tile(3));
            }
        };
        auto frag = [&](const uint8_t* t, int row, int kc) -> u32x4 { return lds_frag<kRB>(t, row, kc, lane); };
        // Group g takes the K stages kt = 2j + g.  The groups run half a step
        // apart: in half-step h, group 0 stores stage h (h even) into its LDS
        // slot or computes stage h - 1 (h odd), and group 1 stores stage h (h
        // odd) or computes stage h - 1 (h even), so one group's LDS stores and
        // load waits overlap the other group's MFMAs.  A barrier ends every
        // half-step; a group's store and the reads of that slot are always a
        // half-step apart.
        if (kg < nk) issue(kg);
        fold_frob(0);
        __syncthreads();
        for (int h = 0; h <= nk; ++h) {
            if ((h & 1) == kg) {
                if (h < nk) {                       // stage h: registers -> LDS, next loads
                    commit();
                    if (h + 2 < nk) issue(h + 2);
                }
            } else if (h > 0 && h - 1 < nk) {       // stage h - 1 of this group
                compute_with(frag, tile(0), tile(1), tile(2), tile(3));
            }
            __syncthreads();
        }
    }

    // ------------------------------------------------------- epilogue
    // thread tid -> rows tid/16 + 32p (p < 4) of the tile, columns 8*(tid%16) .. +7
    const int lc = 8 * (tid % 16);
    constexpr bool kPreA = (PHASE == kSquare) && (PREC == kNsBf16);
    u32x4 a_pre[4][2];
    if constexpr (kPreA) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const size_t idx = aplane + (size_t)(job.ti * kTile + tid / 16 + 32 * p) * M + job.tj * kTile + lc;
            a_pre[p][0] = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(G.a_hi) + idx);
            if constexpr (kF8) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(G.a_lo) + idx);
                a_pre[p][1] = u32x4{w[0], w[1], 0u, 0u};
            } else {
                a_pre[p][1] = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(G.a_lo) + idx);
            }
        }
    }
    // The two groups hold partial sums of the same tile.  Group g finishes the
    // 32-row blocks mi = g of every wave: it hands its partial of block 1 - g to
    // the same wave of the other group through LDS (16-byte chunks in register
    // order), adds the partial it receives, and stages its finished block.
    float* stage = reinterpret_cast<float*>(lds);
    u32x4* xbuf = reinterpret_cast<u32x4*>(lds + kSymStageBytes);   // [group][wave][8 chunks][lane]
    auto send = [&](auto mi_c) {
        constexpr int mi = decltype(mi_c)::value;
        u32x4* out = xbuf + ((kg * 4 + wave) * 8) * kWave + lane;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                floatx4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[mi][ni][4 * q + e];
                out[(ni * 4 + q) * kWave] = __builtin_bit_cast(u32x4, v);
            }
    };
    auto finish = [&](auto mi_c) {
        constexpr int mi = decltype(mi_c)::value;
        const u32x4* in = xbuf + (((1 - kg) * 4 + wave) * 8) * kWave + lane;
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const floatx4 v = __builtin_bit_cast(floatx4, in[(ni * 4 + q) * kWave]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[mi][ni][4 * q + e] += v[e];
            }
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + mi * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                const int col = wn * 64 + ni * 32 + (lane % 32);
                stage[row * kStagePitch + stage_col(row, col)] = acc[mi][ni][r];
            }
    };
    if (kg == 0) send(std::integral_constant<int, 1>{});
    else send(std::integral_constant<int, 0>{});
    __syncthreads();
    if (kg == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, 1>{});
    __syncthreads();
    const float s = fold ? fscale : G.scale[job.slot];
    const float sc = args.first ? s * s : 1.0f;
    const float f8_lo_scale = ldexpf(1.0f, args.f8_sl), f8_lo_inv = ldexpf(1.0f, -args.f8_sl);
    const float f8_hi_scale = ldexpf(1.0f, args.f8_sa);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int lr = tid / 16 + 32 * p;
        float* sp = stage + lr * kStagePitch + stage_col(lr, lc);
        float v[8];
        {
            const floatx4 a = *reinterpret_cast<const floatx4*>(sp);
            const floatx4 b = *reinterpret_cast<const floatx4*>(sp + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
        }
        const size_t idx = (size_t)(job.ti * kTile + lr) * M + job.tj * kTile + lc;
        if (PHASE == kGram) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= sc;
            if constexpr (kF8)
                store8_hi_f8lo(static_cast<bf16*>(G.a_hi) + aplane, static_cast<uint8_t*>(G.a_lo) + aplane,
                               static_cast<uint8_t*>(G.b_lo) + aplane, idx, v, f8_lo_scale, f8_hi_scale);
            else
                store8<PREC>(static_cast<T*>(G.a_hi) + aplane, static_cast<T*>(G.a_lo) + aplane, idx, v);
        } else {
            float ah[8], al[8];
            if constexpr (kPreA) {
                unpack8(a_pre[p][0], ah);
                if constexpr (kF8) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) al[e] = f8_decode(a_pre[p][1][e / 4], e % 4) * f8_lo_inv;
                } else {
                    unpack8(a_pre[p][1], al);
                }
            } else {
                load8<PREC>(static_cast<const T*>(G.a_hi) + aplane, idx, ah);
                if constexpr (PREC == kNsBf16) load8<PREC>(static_cast<const T*>(G.a_lo) + aplane, idx, al);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = (PREC == kNsBf16) ? ah[e] + al[e] : ah[e];
                v[e] = fmaf(args.b, a, args.c * v[e]);
            }
            store8<PREC>(static_cast<T*>(G.b) + aplane, COMP ? static_cast<T*>(G.b_lo) + aplane : nullptr, idx, v);
        }
        if (!diag) {
            floatx4 a, b;
#pragma unroll
            for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[4 + e]; }
            *reinterpret_cast<floatx4*>(sp) = a;
            *reinterpret_cast<floatx4*>(sp + 4) = b;
        }
    }
    if (!diag) {
        __syncthreads();
        // mirrored tile: output row tj*128 + c, columns ti*128 + 8*chunk .. +7.  A wave
        // takes 8 rows c x 8 chunks (8 lanes write one row's 128 contiguous bytes).
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int l = tid % kWave;
            const int chunk = l % 8 + 8 * (p % 2);
            const int c = l / 8 + 8 * (tid / kWave) + 64 * (p / 2);
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = stage[(chunk * 8 + e) * kStagePitch + stage_col(chunk * 8 + e, c)];
            const size_t idx = (size_t)(job.tj * kTile + c) * M + job.ti * kTile + chunk * 8;
            if (PHASE == kGram && kF8)
                store8_hi_f8lo(static_cast<bf16*>(G.a_hi) + aplane, static_cast<uint8_t*>(G.a_lo) + aplane,
                               static_cast<uint8_t*>(G.b_lo) + aplane, idx, v, f8_lo_scale, f8_hi_scale);
            else if (PHASE == kGram)
                store8<PREC>(static_cast<T*>(G.a_hi) + aplane, static_cast<T*>(G.a_lo) + aplane, idx, v);
            else
                store8<PREC>(static_cast<T*>(G.b) + aplane, COMP ? static_cast<T*>(G.b_lo) + aplane : nullptr,
                             idx, v);
        }
    }
}

// Dynamic LDS beyond the default 64 KiB must be requested for each kernel
// (gfx950 has 160 KiB per CU); done once per kernel and device.
template <auto Kernel>
hipError_t request_lds(size_t lds) {
    if (lds <= 65536) return hipSuccess;
    static std::mutex mu;
    static uint64_t done = 0;   // bit d: requested on device d
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    if (dev < 64 && ((done >> dev) & 1u)) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess && dev < 64) done |= (uint64_t)1 << dev;
    return e;
}

size_t ns_update_lds_bytes(int precision, bool comp) {
    return (size_t)((precision == kNsBf16 && comp) ? 4 : 2) * Stage<128>::kSlot;
}

template <int PREC, bool COMP, bool FUSE>
hipError_t launch_update(const NsArgs& a, hipStream_t s) {
    const size_t lds = ns_update_lds_bytes(PREC, COMP);
    const hipError_t attr = request_lds<&ns_update_kernel<PREC, COMP, FUSE>>(lds);
    if (attr != hipSuccess) return attr;
    const int grid = (a.total_jobs + kXcds - 1) / kXcds * kXcds;
    ns_update_kernel<PREC, COMP, FUSE><<<grid, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

size_t ns_sym_lds_bytes(int phase, int precision, bool comp) {
    const bool split = precision == kNsBf16 && (phase == kSquare || comp);
    const bool dma = ns_sym_dma(phase, precision, comp);
    if (NS_SQ_FP8 != 0 && phase == kSquare && precision == kNsBf16 && !comp)
        // both groups: bf16 Ah tiles of both sides, e4m3 Ah and Al tiles of both sides
        return std::max((size_t)2 * 2 * Stage<128>::kSlot + (size_t)2 * 4 * kF8TileBytes, (size_t)kSymEpilogueBytes);
    const int rb = ns_sym_stage_bytes(phase, precision, comp, dma);
    if (dma) {
        // two buffers x two groups x tiles, plus the 8 floats of the folded Frobenius sum
        const size_t bufs = (size_t)2 * 2 * (split ? 4 : 2) * kTile * rb;
        return std::max(bufs + 32, (size_t)kSymEpilogueBytes);
    }
    const int slot = rb == 256 ? Stage<256>::kSlot : Stage<128>::kSlot;
    return std::max((size_t)2 * (split ? 4 : 2) * slot, (size_t)kSymEpilogueBytes);
}

template <int PHASE, int PREC, bool COMP>
hipError_t launch_sym(const NsArgs& a, hipStream_t s) {
    const size_t lds = ns_sym_lds_bytes(PHASE, PREC, COMP);
    const hipError_t attr = request_lds<&ns_sym_kernel<PHASE, PREC, COMP>>(lds);
    if (attr != hipSuccess) return attr;
    const int grid = (a.total_jobs + kXcds - 1) / kXcds * kXcds;
    ns_sym_kernel<PHASE, PREC, COMP><<<grid, kSymThreads, lds, s>>>(a);
    return hipGetLastError();
}

template <int PHASE>
hipError_t launch_sym_phase(const NsArgs& a, int precision, bool comp, hipStream_t s) {
    if (precision == kNsFp32) return launch_sym<PHASE, kNsFp32, false>(a, s);
    return comp ? launch_sym<PHASE, kNsBf16, true>(a, s) : launch_sym<PHASE, kNsBf16, false>(a, s);
}

template <bool FUSE>
hipError_t launch_update_phase(const NsArgs& a, int precision, bool comp, hipStream_t s) {
    if (precision == kNsFp32) return launch_update<kNsFp32, false, FUSE>(a, s);
    return comp ? launch_update<kNsBf16, true, FUSE>(a, s) : launch_update<kNsBf16, false, FUSE>(a, s);
}

}  // namespace

hipError_t launch_ns(const NsArgs& a, int phase, int precision, bool comp, hipStream_t s) {
    if (phase == kGram) return launch_sym_phase<kGram>(a, precision, comp, s);
    if (phase == kSquare) return launch_sym_phase<kSquare>(a, precision, comp, s);
    return a.fuse_apply ? launch_update_phase<true>(a, precision, comp, s)
                        : launch_update_phase<false>(a, precision, comp, s);
}

const char* ns_kernel_name(int phase, int precision, bool comp, bool fused) {
    static const char* names[3][4] = {
        {"ns_gram_bf16", "ns_square_bf16", "ns_update_bf16", "ns_update_apply_bf16"},
        {"ns_gram_bf16x3", "ns_square_bf16x3", "ns_update_bf16x3", "ns_update_apply_bf16x3"},
        {"ns_gram_fp32", "ns_square_fp32", "ns_update_fp32", "ns_update_apply_fp32"}};
    const int v = precision == kNsFp32 ? 2 : (comp ? 1 : 0);
    return names[v][(phase == kUpdate && fused) ? 3 : phase];
}

}  // namespace muon
