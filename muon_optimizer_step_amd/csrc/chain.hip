// Persistent Newton-Schulz chain: every iteration of every base-precision bf16
// matrix of a call in one launch.
//
// Method: "Record: Combined 3-Layer Recurrence + Parallel Residuals + Polar
// Express + Brotli" (PR #1396), "Techniques Combined": the Muon update is
// orthogonalised by a Newton-Schulz iteration with a per-step coefficient
// schedule; "Record: Improved Parallel Residuals + Systems Optimization"
// (PR #1584), "Summary": the Muon step as one fused kernel.  Iteration k:
//     A = X X^T;   B = b_k A + c_k A A;   X <- a_k X + B X
// with the numerics of the base bf16 groups in ns.hip (bf16 hi operands, the
// square's cross terms on e4m3, X carried as bf16 hi + byte lo, fp32
// accumulation); the per-phase kernels there and this chain compute the same
// products with the same roundings.
//
// Schedule.  The launch has two resident workgroups per CU.  The host binds
// every matrix to one of the 8 XCDs (longest work first onto the least loaded
// XCD); a workgroup reads the XCD it runs on from the XCC_ID hardware register
// and only takes tiles of that XCD's matrices.  A matrix's tiles form one
// sequence: iteration 0's Gram tiles, its square tiles, its update tiles, then
// iteration 1's, ...  A tile may start once every tile of the phase before it
// in that sequence is done; per matrix, a grab counter hands out the next tile
// and a done counter counts finished ones (both monotonic, so "done >= first
// tile of my phase" is the whole dependency test).  A free workgroup scans its
// XCD's matrices (one lane per matrix, largest first) for one whose next tile
// is ready, takes it with one atomic add, waits if a race handed it a tile of
// the next phase, runs it, and counts it done.  No tile waits for a matrix
// other than its own, so one matrix's square runs while others are still in
// their Gram, and no grid-wide phase boundary exists.
//
// Memory ordering.  Producer and consumer of every plane are on the same XCD
// and so share its L2, the coherence point of that XCD's CUs (the vector L1
// writes through).  A finished tile waits for its stores (vmcnt(0)) in every
// wave, meets at a barrier, and then bumps the done counter; a consumer that
// sees the counter invalidates its CU's L1 (buffer_inv sc1) before loading.
// No plane crosses XCDs inside the launch, so no L2 writeback is needed; the
// kernel boundaries before (prep) and after (the caller's next work) order
// everything else.
//
// Termination.  Every wait is bounded by timeout_ticks of the 100 MHz real-time
// counter; a wait that runs out sets kChainStatusTimeout in the status word and
// the workgroup leaves, so a fault in the schedule cannot hang the GPU.  A
// workgroup leaves when every matrix of its XCD has handed out all its tiles.
#include "common.h"
#include "kernels.h"
#define NS_OPAQUE_TID 1
#include "ns_device.h"

namespace muon {

namespace {

constexpr int kChainThreads = kThreads;   // 4 waves of 64 x 64 per 128 x 128 tile
// LDS of the largest tile (the square: bf16 A hi tiles of both sides and the
// e4m3 tiles of A hi and A lo of both sides); the Gram's two direct-load
// buffers and every epilogue's fp32 staging fit inside it.
constexpr int kChainTileLds = 2 * Stage<128>::kSlot + 4 * kF8TileBytes;
constexpr int kChainSchedOff = kChainTileLds;          // scheduler broadcast (4 ints)
constexpr int kChainLds = kChainTileLds + 64;
constexpr int kGramBufBytes = 2 * kTile * 128;         // one direct-load buffer: two 128 x 128 B tiles
static_assert(2 * kGramBufBytes + 32 <= kChainTileLds, "Gram buffers and the Frobenius sum fit");
static_assert(kTile * kStagePitch * 4 <= kChainTileLds, "full-tile fp32 staging fits");
static_assert(2 * kChainLds <= 160 * 1024, "two chain workgroups per CU");

__device__ inline uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t add_relaxed(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int xcc_id() {
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return (int)(x & 0xFu) % kXcds;
}
__device__ inline uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Position of tile g in its matrix's sequence.
struct Item {
    int phase;        // kGram, kSquare or kUpdate
    int k;            // NS iteration
    int tile;         // index inside the phase
    uint32_t start;   // first tile of this phase instance in the sequence
};
__device__ inline Item decode_item(uint32_t g, int ts, int tu) {
    const uint32_t per = 2u * ts + tu;
    const uint32_t k = g / per;
    const uint32_t r = g - k * per;
    Item it;
    it.k = (int)k;
    if (r < (uint32_t)ts) { it.phase = kGram; it.tile = (int)r; it.start = k * per; }
    else if (r < 2u * ts) { it.phase = kSquare; it.tile = (int)r - ts; it.start = k * per + ts; }
    else { it.phase = kUpdate; it.tile = (int)r - 2 * ts; it.start = k * per + 2 * ts; }
    return it;
}

// (ti, tj) of an upper-triangle tile index (row-major over ti <= tj).
__device__ inline void sym_tile(int t, int tm, int& ti, int& tj) {
    int i = 0;
    while (t >= tm - i) { t -= tm - i; ++i; }
    ti = i;
    tj = i + t;
}

// Frobenius scale 1 / (sqrt(sum of rows[0 .. n)) + eps) with 256 threads in a
// fixed order (thread t sums rows t, t + 256, ...; wave butterflies; the four
// wave totals in order): every Gram tile of a matrix gets the same bits.
__device__ inline float frob256(const float* rows, int n, float* red) {
    float s = 0.f;
    for (int r = tid_x(); r < n; r += kChainThreads) s += rows[r];
    s = wave_sum(s);
    if (tid_x() % kWave == 0) red[tid_x() / kWave] = s;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return 1.0f / (sqrtf(t) + kEps);
}

// Accumulators of a 128 x 128 tile (4 waves, 64 x 64 each) -> fp32 staging.
__device__ inline void stage_acc(float* stage, const floatx16 (&acc)[2][2], int wm, int wn, int lane) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + mi * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                const int col = wn * 64 + ni * 32 + (lane % 32);
                stage[row * kStagePitch + stage_col(row, col)] = acc[mi][ni][r];
            }
}

// Mirror pass of a symmetric tile: output row tj*128 + c, columns ti*128 +
// 8*chunk .. +7, read from the staged (final) values column-wise.  A wave
// takes 8 rows c x 8 chunks; store(idx, v) writes 8 values at element idx.
template <typename Store>
__device__ inline void mirror_pass(const float* stage, int ti, int tj, int M, Store store) {
    const int tid = tid_x(), l = tid % kWave, wave = tid / kWave;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int chunk = l % 8 + 8 * (p % 2);
        const int c = l / 8 + 8 * wave + 32 * (p / 2);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = stage[(chunk * 8 + e) * kStagePitch + stage_col(chunk * 8 + e, c)];
        store((size_t)(tj * kTile + c) * M + ti * kTile + chunk * 8, v);
    }
}

__device__ inline void zero_acc(floatx16 (&acc)[2][2]) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
}

// A = s^2 Xh Xh^T (s on iteration 0 only): tile (ti, tj), K = N.  Operands go
// straight into LDS (global_load_lds_dwordx4) in two buffers of 128 K bytes
// per row, rows unpadded with the 16-byte chunk c of row r at c ^ ((r/2) % 8)
// (conflict-free fragment reads).  Stores A hi (bf16) and the e4m3 planes
// A lo * 2^sl (a_lo) and A hi * 2^sa (b_lo) that the square reads.
__device__ inline void gram_tile(const NsGroup& G, const Job job, int src, bool first, const float* rowsq,
                                 int rows, int sa, int sl, uint8_t* lds) {
    constexpr int kRB = 128, kC = kRB / 16, kTileBytes = kTile * kRB;
    constexpr int kPerTile = kTileBytes / 1024 / 4;   // 1 KB direct loads per wave per tile
    const int M = G.M, N = G.N;
    const int tid = tid_x(), lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const bool diag = job.ti == job.tj;
    const size_t xplane = (size_t)job.slot * M * N;
    const size_t aplane = (size_t)job.slot * M * M;
    const size_t ld_bytes = (size_t)N * 2;
    const uint8_t* xh = reinterpret_cast<const uint8_t*>(static_cast<const bf16*>(G.x[src]) + xplane);
    const uint8_t* ga = xh + (size_t)job.ti * kTile * ld_bytes;
    const uint8_t* gb = xh + (size_t)job.tj * kTile * ld_bytes;

    // the Frobenius sum first: no register loads may be in flight once the
    // direct loads start (a wait for them would also wait for those)
    float fscale = 1.f;
    if (first) {
        fscale = frob256(rowsq, rows, reinterpret_cast<float*>(lds + 2 * kGramBufBytes));
        if (job.ti == 0 && job.tj == 0 && tid == 0) G.scale[job.slot] = fscale;
    }

    floatx16 acc[2][2];
    zero_acc(acc);
    asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));

    auto swz = [](int row) { return (row / (16 / kC)) % kC; };
    auto dma_tile = [&](const uint8_t* g, int kt, int buf, int which) {
        uint8_t* dst = lds + buf * kGramBufBytes + which * kTileBytes;
#pragma unroll
        for (int j = 0; j < kPerTile; ++j) {
            const int q = j * 4 + wave;                      // 1 KB block: rows 8q .. 8q + 7
            const int row = q * (1024 / kRB) + lane / kC;
            const int c = (lane % kC) ^ swz(row);
            __builtin_amdgcn_global_load_lds(g + (size_t)row * ld_bytes + (size_t)kt * kRB + c * 16,
                                             (lds_ptr)(dst + q * 1024), 16, 0, 0);
        }
    };
    auto dma_stage = [&](int kt, int buf) {
        dma_tile(ga, kt, buf, 0);
        if (!diag) dma_tile(gb, kt, buf, 1);
    };
    auto frag = [&](const uint8_t* t, int row, int kc) -> u32x4 {
        const int c = (2 * kc + lane / 32) ^ swz(row);
        return *reinterpret_cast<const u32x4*>(t + row * kRB + c * 16);
    };
    // MFMAs of one stage; the fragments of chunk kc + 2 are read while the
    // MFMAs of chunk kc run (one fragment read scheduled after each MFMA)
    auto compute = [&](const uint8_t* t_a, const uint8_t* t_b) {
        constexpr int kKC = kRB / 32, kDist = 2, kBufs = kDist + 1;
        u32x4 f[kBufs][4];
        auto read = [&](int kc, u32x4* d) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) d[mi] = frag(t_a, wm * 64 + mi * 32 + lane % 32, kc);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) d[2 + ni] = frag(t_b, wn * 64 + ni * 32 + lane % 32, kc);
        };
#pragma unroll
        for (int kc = 0; kc < kDist; ++kc) read(kc, f[kc]);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * kDist, 0);
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
            if (kc + kDist < kKC) read(kc + kDist, f[(kc + kDist) % kBufs]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    mfma_chunk<kNsBf16>(acc[mi][ni], f[kc % kBufs][mi], f[kc % kBufs][2 + ni]);
            if (kc + kDist < kKC) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
        }
    };
    const int nk = N / (kRB / 2);
    dma_stage(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) {
            dma_stage(kt + 1, buf ^ 1);
            if (diag) wait_vmcnt<kPerTile>();
            else wait_vmcnt<2 * kPerTile>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_only();
        const uint8_t* t_a = lds + buf * kGramBufBytes;
        compute(t_a, diag ? t_a : t_a + kTileBytes);
        wait_lgkmcnt0();
        barrier_only();
    }

    // epilogue: full tile through fp32 staging, row pass then mirror pass
    float* stage = reinterpret_cast<float*>(lds);
    stage_acc(stage, acc, wm, wn, lane);
    __syncthreads();
    const float sc = first ? fscale * fscale : 1.0f;
    const float lo_scale = ldexpf(1.0f, sl), hi_scale = ldexpf(1.0f, sa);
    bf16* a_hi = static_cast<bf16*>(G.a_hi) + aplane;
    uint8_t* a_lo8 = static_cast<uint8_t*>(G.a_lo) + aplane;
    uint8_t* a_hi8 = static_cast<uint8_t*>(G.b_lo) + aplane;
    const int lc = 8 * (tid % 16);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int lr = tid / 16 + 16 * p;
        float* sp = stage + lr * kStagePitch + stage_col(lr, lc);
        const floatx4 x0 = *reinterpret_cast<const floatx4*>(sp);
        const floatx4 x1 = *reinterpret_cast<const floatx4*>(sp + 4);
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = sc * x0[e]; v[4 + e] = sc * x1[e]; }
        store8_hi_f8lo(a_hi, a_lo8, a_hi8, (size_t)(job.ti * kTile + lr) * M + job.tj * kTile + lc, v, lo_scale,
                       hi_scale);
        if (!diag) {
            floatx4 y0, y1;
#pragma unroll
            for (int e = 0; e < 4; ++e) { y0[e] = v[e]; y1[e] = v[4 + e]; }
            *reinterpret_cast<floatx4*>(sp) = y0;
            *reinterpret_cast<floatx4*>(sp + 4) = y1;
        }
    }
    if (!diag) {
        __syncthreads();
        mirror_pass(stage, job.ti, job.tj, M, [&](size_t idx, const float* v) {
            store8_hi_f8lo(a_hi, a_lo8, a_hi8, idx, v, lo_scale, hi_scale);
        });
    }
}

// B = b A + c (Ah Ah + Ah Al + Al Ah): tile (ti, tj), K = M.  Ah Ah on the bf16
// MFMA from the A hi plane, the cross terms on the scaled fp8 MFMA from the two
// e4m3 planes the Gram wrote (E8M0 scales 2^-sa and 2^-sl undo their
// scaling).  One LDS stage of 64 K per operand, staged through registers with
// the next stage's loads in flight during the MFMAs.
__device__ inline void square_tile(const NsGroup& G, const Job job, float b, float c, int sa, int sl,
                                   uint8_t* lds) {
    constexpr int kRB = 128;
    constexpr int kSlot = Stage<kRB>::kSlot;
    const int M = G.M;
    const int tid = tid_x(), lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const bool diag = job.ti == job.tj;
    const size_t aplane = (size_t)job.slot * M * M;
    const size_t ld_bytes = (size_t)M * 2;
    const uint8_t* ah = reinterpret_cast<const uint8_t*>(static_cast<const bf16*>(G.a_hi) + aplane);
    const uint8_t* ga = ah + (size_t)job.ti * kTile * ld_bytes;
    const uint8_t* gb = ah + (size_t)job.tj * kTile * ld_bytes;
    const uint8_t* g8a = static_cast<const uint8_t*>(G.a_lo) + aplane + (size_t)job.ti * kTile * M;
    const uint8_t* g8b = static_cast<const uint8_t*>(G.a_lo) + aplane + (size_t)job.tj * kTile * M;
    const uint8_t* h8a = static_cast<const uint8_t*>(G.b_lo) + aplane + (size_t)job.ti * kTile * M;
    const uint8_t* h8b = static_cast<const uint8_t*>(G.b_lo) + aplane + (size_t)job.tj * kTile * M;
    uint8_t* const f8base = lds + 2 * kSlot;
    auto btile = [&](int side) -> uint8_t* { return lds + (diag ? 0 : side) * kSlot; };
    auto ftile = [&](int which) -> uint8_t* {   // 0: Ah ti, 1: Ah tj, 2: Al ti, 3: Al tj
        if (diag && which == 1) which = 0;
        if (diag && which == 3) which = 2;
        return f8base + which * kF8TileBytes;
    };

    floatx16 acc[2][2];
    zero_acc(acc);
    asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1]));

    NtLoader<kRB> la, lb;
    u32x4 l8a[2], l8b[2];    // Al bytes: row tid/4 + 64q, 16-byte chunk tid%4 of the stage's 64
    u32x4 h8va[2], h8vb[2];  // Ah e4m3 bytes, same mapping
    auto issue = [&](int kt) {
        la.load(ga, ld_bytes, kt * kRB);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const size_t o = (size_t)(tid / 4 + 64 * q) * M + kt * 64 + (tid % 4) * 16;
            l8a[q] = *reinterpret_cast<const u32x4*>(g8a + o);
            h8va[q] = *reinterpret_cast<const u32x4*>(h8a + o);
        }
        if (!diag) {
            lb.load(gb, ld_bytes, kt * kRB);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const size_t o = (size_t)(tid / 4 + 64 * q) * M + kt * 64 + (tid % 4) * 16;
                l8b[q] = *reinterpret_cast<const u32x4*>(g8b + o);
                h8vb[q] = *reinterpret_cast<const u32x4*>(h8b + o);
            }
        }
    };
    auto commit_side = [&](const NtLoader<kRB>& lh, const u32x4* l8, const u32x4* h8, int side) {
        lh.store(btile(side));
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<u32x4*>(ftile(side) + (tid / 4 + 64 * q) * kF8Pitch + (tid % 4) * 16) = h8[q];
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<u32x4*>(ftile(2 + side) + (tid / 4 + 64 * q) * kF8Pitch + (tid % 4) * 16) = l8[q];
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
                for (int ni = 0; ni < 2; ++ni) mfma_chunk<kNsBf16>(acc[mi][ni], fa[mi], fb[ni]);
        }
#pragma unroll
        for (int term = 0; term < 2; ++term) {   // Ah_i Al_j^T, then Al_i Ah_j^T
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
    const int nk = M / 64;
    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        commit_side(la, l8a, h8va, 0);
        if (!diag) commit_side(lb, l8b, h8vb, 1);
        __syncthreads();
        if (kt + 1 < nk) issue(kt + 1);
        compute();
    }

    // epilogue: half of this tile's A (for the b A term) is loaded while the
    // accumulators are staged, the other half during the first rows
    const int lc = 8 * (tid % 16);
    u32x4 a_pre[8];
    u32x2 a8_pre[8];
    auto load_a = [&](int p) {
        const size_t idx = aplane + (size_t)(job.ti * kTile + tid / 16 + 16 * p) * M + job.tj * kTile + lc;
        a_pre[p] = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(G.a_hi) + idx);
        a8_pre[p] = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(G.a_lo) + idx);
    };
#pragma unroll
    for (int p = 0; p < 4; ++p) load_a(p);
    __syncthreads();
    float* stage = reinterpret_cast<float*>(lds);
    stage_acc(stage, acc, wm, wn, lane);
#pragma unroll
    for (int p = 4; p < 8; ++p) load_a(p);
    __syncthreads();
    const float lo_inv = ldexpf(1.0f, -sl);
    bf16* bp = static_cast<bf16*>(G.b) + aplane;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int lr = tid / 16 + 16 * p;
        float* sp = stage + lr * kStagePitch + stage_col(lr, lc);
        const floatx4 x0 = *reinterpret_cast<const floatx4*>(sp);
        const floatx4 x1 = *reinterpret_cast<const floatx4*>(sp + 4);
        float ahv[8], v[8];
        unpack8(a_pre[p], ahv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float al = f8_decode(a8_pre[p][e / 4], e % 4) * lo_inv;
            const float acc_v = e < 4 ? x0[e] : x1[e - 4];
            v[e] = fmaf(b, ahv[e] + al, c * acc_v);
        }
        store8<kNsBf16>(bp, nullptr, (size_t)(job.ti * kTile + lr) * M + job.tj * kTile + lc, v);
        if (!diag) {
            floatx4 y0, y1;
#pragma unroll
            for (int e = 0; e < 4; ++e) { y0[e] = v[e]; y1[e] = v[4 + e]; }
            *reinterpret_cast<floatx4*>(sp) = y0;
            *reinterpret_cast<floatx4*>(sp + 4) = y1;
        }
    }
    if (!diag) {
        __syncthreads();
        mirror_pass(stage, job.ti, job.tj, M, [&](size_t idx, const float* v) {
            store8<kNsBf16>(bp, nullptr, idx, v);
        });
    }
}

// The update tile with its fused weight apply taken from the matrix record.
template <bool FUSE>
__device__ inline void chain_update_tile(const NsGroup& G, const Job job, const UpdateCtx uc,
                                                            const ChainMat& R, float lr, uint8_t* lds) {
    FusedApply F{};
    if constexpr (FUSE) {
        F.param = R.param;
        F.out = R.out;
        F.ema = R.ema;
        F.rows = R.rows;
        F.cols = R.cols;
        F.lr_s = lr * R.shape_scale;   // the float product the per-phase path forms on the host
        F.flags = R.flags;
    }
    update_tile<kNsBf16, false, FUSE, true>(G, job, uc, F, lds);
}

// Workgroup-uniform scheduler state, broadcast through LDS by wave 0.
struct Pick {
    int mat;        // matrix, or -1: leave
    uint32_t g;     // tile index in the matrix's sequence
};

// Wave 0: the next ready tile of this XCD's matrices [m0, m1), taken with an
// atomic add on its grab counter (a compare-and-swap that only hands out
// ready tiles was measured slower: its retries under contention cost more
// than the occasional wait for a tile of the next phase).  mat = -1 once every
// matrix has handed out all its tiles (or a wait ran out of time).
__device__ inline Pick pick_next(const ChainArgs& A, int m0, int m1, uint64_t t0) {
    const int lane = tid_x() % kWave;
    const uint32_t steps = (uint32_t)A.ns_steps;
    for (;;) {
        bool any_left = false;
        int chosen = -1;
        for (int base = m0; base < m1 && chosen < 0; base += kWave) {
            const int j = base + lane;
            bool left = false, ready = false;
            if (j < m1) {
                const int ts = A.mats[j].tiles_sym, tu = A.mats[j].tiles_upd;
                const uint32_t total = steps * (2u * ts + tu);
                const uint32_t g = ld_relaxed(A.ctr + (size_t)j * kChainCtrWords);
                if (g < total) {
                    left = true;
                    const uint32_t d = ld_relaxed(A.ctr + (size_t)j * kChainCtrWords + 32);
                    ready = d >= decode_item(g, ts, tu).start;
                }
            }
            any_left = any_left || __ballot(left) != 0;
            const uint64_t rb = __ballot(ready);
            if (rb) chosen = base + __ffsll((long long)rb) - 1;
        }
        if (chosen >= 0) {
            uint32_t g = 0;
            if (lane == 0) g = add_relaxed(A.ctr + (size_t)chosen * kChainCtrWords, 1u);
            g = __shfl(g, 0);
            const uint32_t total = steps * (2u * A.mats[chosen].tiles_sym + A.mats[chosen].tiles_upd);
            if (g < total) return Pick{chosen, g};
            continue;   // another workgroup took the last tile
        }
        if (!any_left) return Pick{-1, 0};
        __builtin_amdgcn_s_sleep(2);
        if (now_ticks() - t0 > A.timeout_ticks) {
            if (lane == 0) __hip_atomic_fetch_or(A.ctr + (size_t)A.nmat * kChainCtrWords, kChainStatusTimeout,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return Pick{-1, 0};
        }
    }
}

__global__ __launch_bounds__(kChainThreads) __attribute__((amdgpu_waves_per_eu(2)))
void ns_chain_kernel(const ChainArgs args) {
    // The arguments through the kernarg segment pointer: the out-of-line tiles
    // take references into it, which the by-value parameter would have copied
    // to scratch first.
    (void)args;
    const ChainArgs& A = *(const ChainArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    int* sched = reinterpret_cast<int*>(lds + kChainSchedOff);
    const int tid = tid_x(), wave = tid / kWave;
    const int xcc = xcc_id();
    const int m0 = A.xcd_begin[xcc], m1 = A.xcd_begin[xcc + 1];
    const uint64_t t0 = now_ticks();
    uint32_t* const status = A.ctr + (size_t)A.nmat * kChainCtrWords;
    for (;;) {
        if (wave == 0) {
            const Pick pk = pick_next(A, m0, m1, t0);
            int go = pk.mat;
            if (go >= 0) {
                // wait until every tile of the phase before this one is done
                const ChainMat& R = A.mats[go];
                const uint32_t start = decode_item(pk.g, R.tiles_sym, R.tiles_upd).start;
                uint32_t* done = A.ctr + (size_t)go * kChainCtrWords + 32;
                while (ld_relaxed(done) < start) {
                    __builtin_amdgcn_s_sleep(1);
                    if (now_ticks() - t0 > A.timeout_ticks) {
                        if (tid == 0)
                            __hip_atomic_fetch_or(status, kChainStatusTimeout, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
                        go = -1;
                        break;
                    }
                }
            }
            if (tid == 0) {
                sched[0] = go;
                sched[1] = (int)pk.g;
            }
        }
        __syncthreads();
        // workgroup-uniform: scalar registers, scalar loads of the record
        const int j = __builtin_amdgcn_readfirstlane(sched[0]);
        const uint32_t g = (uint32_t)__builtin_amdgcn_readfirstlane(sched[1]);
        if (j < 0) break;
        // acquire: every wave drops its CU's L1 copies before its first load of
        // the tile (lines cached before the producers' stores reached the L2).
        // The agent-scope invalidate: the workgroup-scope one (sc0) leaves the
        // L1 alone outside threadgroup-split mode, and stale tiles were
        // measured with it.
        asm volatile("buffer_inv sc1\n\ts_waitcnt vmcnt(0)" ::: "memory");
        const ChainMat& R = A.mats[j];
        const NsGroup& G = A.g[R.group];
        const Item it = decode_item(g, R.tiles_sym, R.tiles_upd);
        const int tm = G.M / kTile;
        Job job;
        job.g = R.group;
        job.slot = R.slot;
        const int src = it.k & 1;
        const bool first = it.k == 0;
        if (it.phase == kGram) {
            sym_tile(it.tile, tm, job.ti, job.tj);
            gram_tile(G, job, src, first, A.rowsq + R.rowsq_off, R.rows, A.f8_sa[it.k], A.f8_sa[it.k] + 8, lds);
        } else if (it.phase == kSquare) {
            sym_tile(it.tile, tm, job.ti, job.tj);
            square_tile(G, job, A.b[it.k], A.c[it.k], A.f8_sa[it.k], A.f8_sa[it.k] + 8, lds);
        } else {
            // column-panel-major: the row tiles that read one X column panel are neighbours
            job.tj = it.tile / tm;
            job.ti = it.tile - job.tj * tm;
            const UpdateCtx uc{A.a[it.k], first ? 1 : 0, src, A.keep, A.decay, A.one_minus_decay};
            if (A.fuse_apply && it.k == A.ns_steps - 1) chain_update_tile<true>(G, job, uc, R, A.lr, lds);
            else chain_update_tile<false>(G, job, uc, R, A.lr, lds);
        }
        // every wave's stores have reached L2 before the tile counts as done
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) add_relaxed(A.ctr + (size_t)j * kChainCtrWords + 32, 1u);
    }
}

// Writes the per-matrix records of a chain launch and, in the first launch of
// a call, clears the grab / done counters and the status word.
__global__ __launch_bounds__(256) void chain_setup_kernel(const ChainSetupArgs a) {
    const int tid = tid_x();
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.rec);
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.dst);
    const int words = a.n * (int)(sizeof(ChainMat) / 4);
    for (int i = tid; i < words; i += 256) dst[i] = src[i];
    if (a.zero)
        for (int i = tid; i < a.nzero; i += 256) a.zero[i] = 0u;
}

}  // namespace

hipError_t launch_chain_setup(const ChainSetupArgs& a, hipStream_t s) {
    chain_setup_kernel<<<1, 256, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_chain(const ChainArgs& a, int workgroups, hipStream_t s) {
    static bool attr_done[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 64 || !attr_done[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ns_chain_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kChainLds);
        if (e != hipSuccess) return e;
        if (dev < 64) attr_done[dev] = true;
    }
    ns_chain_kernel<<<workgroups, kChainThreads, kChainLds, s>>>(a);
    return hipGetLastError();
}

}  // namespace muon
