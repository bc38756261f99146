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
// bf16 numerics: X is kept to ~16 significant bits as a pair of bf16 planes
// (hi = rne(X), lo = rne(X - hi)); MFMA operands are bf16 and accumulate in
// fp32.  A is likewise split, and A A is formed as hi*hi + hi*lo + lo*hi,
// because the plain bf16 square loses the small singular directions that the
// iteration amplifies.  The a X term uses hi + lo.  The fp32 precision runs the
// same three phases on fp32 MFMA (v_mfma_f32_32x32x2_f32).
//
// Tiling: one workgroup (4 wave64s, 2 x 2) per 128 x 128 output tile, 64 x 64
// per wave as 2 x 2 v_mfma_f32_32x32x16_bf16 accumulators; K is staged through
// LDS 128 bytes per row at a time (64 bf16 or 32 fp32), with the next stage's
// global loads in flight during the MFMAs.  A and B are symmetric: only tiles
// with ti <= tj are computed and each is also written mirrored.  All work of
// one phase for every matrix of every shape group is one launch; job indices
// are remapped so that the tiles of one matrix share an XCD (and its L2).
// Workspace dimensions are padded to 128 with zeros, which the iteration keeps
// at zero, so the inner loops need no bounds checks.
#include "common.h"
#include "kernels.h"

namespace muon {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;              // K bytes per LDS stage per row
constexpr int kPitch = kRowBytes + 16;      // padded LDS row pitch (conflict-free b128 reads)
constexpr int kTileBytes = kTile * kPitch;  // one 128-row operand tile

template <int PREC> struct Elem;
template <> struct Elem<kNsBf16> { typedef bf16 T; static constexpr int kBK = 64; };
template <> struct Elem<kNsFp32> { typedef float T; static constexpr int kBK = 32; };

// Accumulate one 16-byte operand chunk per lane: bf16 -> one 32x32x16 MFMA;
// fp32 -> four 32x32x2 MFMAs over the four components (the k permutation is the
// same for both operands, so the contraction is unchanged).
template <int PREC>
__device__ inline void mfma_chunk(floatx16& acc, const u32x4& a, const u32x4& b) {
    if constexpr (PREC == kNsBf16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    } else {
        const floatx4 fa = __builtin_bit_cast(floatx4, a);
        const floatx4 fb = __builtin_bit_cast(floatx4, b);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
    }
}

// 128 rows x 128 bytes of a row-major operand whose K index is contiguous
// ("NT" operand).  Thread t moves 16 bytes of row t/8 + 32q, chunk t%8.
struct NtLoader {
    u32x4 r[4];
    __device__ inline void load(const uint8_t* base, size_t ld_bytes, int kbyte) {
        const int t = threadIdx.x;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint8_t* p = base + (size_t)(t / 8 + 32 * q) * ld_bytes + kbyte + (t % 8) * 16;
            r[q] = *reinterpret_cast<const u32x4*>(p);
        }
    }
    __device__ inline void store(uint8_t* lds) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<u32x4*>(lds + (t / 8 + 32 * q) * kPitch + (t % 8) * 16) = r[q];
    }
};

// X[k][j] (j contiguous in memory) staged as LDS[j][k] so that K is contiguous
// per lane for the MFMA B operand.  bf16: thread t reads 8 k-rows x 4 j
// (8-byte loads, 256 contiguous bytes per half wave) and transposes in
// registers with v_perm; fp32: 4 k-rows x 4 j (16-byte loads).
template <int PREC> struct TLoader;

template <> struct TLoader<kNsBf16> {
    u32x2 v[8];
    __device__ inline void load(const bf16* x, size_t ld, int k0, int j0) {
        const int t = threadIdx.x;
        const int jq = t % 32, kb = t / 32;
#pragma unroll
        for (int r = 0; r < 8; ++r)
            v[r] = *reinterpret_cast<const u32x2*>(x + (size_t)(k0 + 8 * kb + r) * ld + j0 + 4 * jq);
    }
    __device__ inline void store(uint8_t* lds) const {
        const int t = threadIdx.x;
        const int jq = t % 32, kb = t / 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // column c of the 8 x 4 block: element c of every k-row, packed two k per dword
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            u32x4 w;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t lo_row = (c < 2) ? v[2 * p].x : v[2 * p].y;
                const uint32_t hi_row = (c < 2) ? v[2 * p + 1].x : v[2 * p + 1].y;
                w[p] = __builtin_amdgcn_perm(hi_row, lo_row, sel);
            }
            *reinterpret_cast<u32x4*>(lds + (4 * jq + c) * kPitch + kb * 16) = w;
        }
    }
};

template <> struct TLoader<kNsFp32> {
    floatx4 v[4];
    __device__ inline void load(const float* x, size_t ld, int k0, int j0) {
        const int t = threadIdx.x;
        const int jq = t % 32, kb = t / 32;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = *reinterpret_cast<const floatx4*>(x + (size_t)(k0 + 4 * kb + r) * ld + j0 + 4 * jq);
    }
    __device__ inline void store(uint8_t* lds) const {
        const int t = threadIdx.x;
        const int jq = t % 32, kb = t / 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            floatx4 w;
            w[0] = v[0][c]; w[1] = v[1][c]; w[2] = v[2][c]; w[3] = v[3][c];
            *reinterpret_cast<floatx4*>(lds + (4 * jq + c) * kPitch + kb * 16) = w;
        }
    }
};

__device__ inline u32x4 lds_frag(const uint8_t* tile, int row, int kc, int lane) {
    return *reinterpret_cast<const u32x4*>(tile + row * kPitch + kc * 32 + (lane / 32) * 16);
}

// acc element (mi, ni, r) -> tile-local (row, col) for the 32x32 MFMA layout.
__device__ inline int acc_row(int wm, int mi, int r, int lane) { return wm * 64 + mi * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4); }
__device__ inline int acc_col(int wn, int ni, int lane) { return wn * 64 + ni * 32 + (lane % 32); }

struct Job {
    int g, slot, ti, tj;
};

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
        const int per = tm * tn;
        j.slot = local / per;
        const int t = local - j.slot * per;
        j.ti = t / tn;
        j.tj = t - j.ti * tn;
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

template <int PHASE, int PREC>
__global__ __launch_bounds__(kThreads) void ns_kernel(const NsArgs args) {
    typedef typename Elem<PREC>::T T;
    constexpr int kBK = Elem<PREC>::kBK;
    constexpr bool kSplitSquare = (PHASE == kSquare && PREC == kNsBf16);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    Job job;
    if (!decode_job<PHASE>(args, job)) return;
    const NsGroup& G = args.g[job.g];
    const int M = G.M, N = G.N;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const bool diag = (PHASE != kUpdate) && job.ti == job.tj;

    const size_t xplane = (size_t)job.slot * M * N;
    const size_t aplane = (size_t)job.slot * M * M;
    const T* x_src = static_cast<const T*>(G.x[args.src]) + xplane;

    // Operand tiles in LDS: [0] A-operand (rows ti), [1] B-operand (rows tj),
    // and for the split square [2] lo of rows ti, [3] lo of rows tj.
    uint8_t* t_a = lds;
    uint8_t* t_b = diag ? lds : lds + kTileBytes;
    uint8_t* t_al = lds + 2 * kTileBytes;
    uint8_t* t_bl = diag ? t_al : lds + 3 * kTileBytes;

    const uint8_t *ga = nullptr, *gb = nullptr, *gal = nullptr, *gbl = nullptr;
    size_t ld_bytes = 0;
    int K = 0;
    if (PHASE == kGram) {
        ld_bytes = (size_t)N * sizeof(T);
        ga = reinterpret_cast<const uint8_t*>(x_src + (size_t)job.ti * kTile * N);
        gb = reinterpret_cast<const uint8_t*>(x_src + (size_t)job.tj * kTile * N);
        K = N;
    } else if (PHASE == kSquare) {
        const T* ah = static_cast<const T*>(G.a_hi) + aplane;
        ld_bytes = (size_t)M * sizeof(T);
        ga = reinterpret_cast<const uint8_t*>(ah + (size_t)job.ti * kTile * M);
        gb = reinterpret_cast<const uint8_t*>(ah + (size_t)job.tj * kTile * M);
        if (kSplitSquare) {
            const T* al = static_cast<const T*>(G.a_lo) + aplane;
            gal = reinterpret_cast<const uint8_t*>(al + (size_t)job.ti * kTile * M);
            gbl = reinterpret_cast<const uint8_t*>(al + (size_t)job.tj * kTile * M);
        }
        K = M;
    } else {
        const T* bm = static_cast<const T*>(G.b) + aplane;
        ld_bytes = (size_t)M * sizeof(T);
        ga = reinterpret_cast<const uint8_t*>(bm + (size_t)job.ti * kTile * M);
        K = M;
    }

    floatx16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    NtLoader la, lb, lal, lbl;
    TLoader<PREC> lt;
    auto issue = [&](int k0) {
        const int kbyte = k0 * (int)sizeof(T);
        la.load(ga, ld_bytes, kbyte);
        if (PHASE == kUpdate) {
            lt.load(x_src, (size_t)N, k0, job.tj * kTile);
        } else {
            if (!diag) lb.load(gb, ld_bytes, kbyte);
            if (kSplitSquare) {
                lal.load(gal, ld_bytes, kbyte);
                if (!diag) lbl.load(gbl, ld_bytes, kbyte);
            }
        }
    };
    auto commit = [&]() {
        la.store(t_a);
        if (PHASE == kUpdate) {
            lt.store(t_b);
        } else {
            if (!diag) lb.store(t_b);
            if (kSplitSquare) {
                lal.store(t_al);
                if (!diag) lbl.store(t_bl);
            }
        }
    };

    const int nk = K / kBK;
    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        commit();
        __syncthreads();
        if (kt + 1 < nk) issue((kt + 1) * kBK);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) fa[mi] = lds_frag(t_a, wm * 64 + mi * 32 + lane % 32, kc, lane);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) fb[ni] = lds_frag(t_b, wn * 64 + ni * 32 + lane % 32, kc, lane);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) mfma_chunk<PREC>(acc[mi][ni], fa[mi], fb[ni]);
            if (kSplitSquare) {
                u32x4 fal[2], fbl[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) fal[mi] = lds_frag(t_al, wm * 64 + mi * 32 + lane % 32, kc, lane);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) fbl[ni] = lds_frag(t_bl, wn * 64 + ni * 32 + lane % 32, kc, lane);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni) {
                        mfma_chunk<PREC>(acc[mi][ni], fa[mi], fbl[ni]);
                        mfma_chunk<PREC>(acc[mi][ni], fal[mi], fb[ni]);
                    }
            }
        }
    }

    // ------------------------------------------------------------ epilogues
    const float s = G.scale[job.slot];
    if (PHASE == kGram) {
        const float sc = args.first ? s * s : 1.0f;
        T* ah = static_cast<T*>(G.a_hi) + aplane;
        T* al = static_cast<T*>(G.a_lo) + aplane;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = job.tj * kTile + acc_col(wn, ni, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row0 = job.ti * kTile + acc_row(wm, mi, 4 * q, lane);
                    T hv[4], lv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = acc[mi][ni][4 * q + e] * sc;
                        if constexpr (PREC == kNsBf16) {
                            split_bf16(v, hv[e], lv[e]);
                            ah[(size_t)(row0 + e) * M + col] = hv[e];
                            al[(size_t)(row0 + e) * M + col] = lv[e];
                        } else {
                            hv[e] = v;
                            ah[(size_t)(row0 + e) * M + col] = v;
                        }
                    }
                    if (job.ti != job.tj) {
                        // mirror: A[col][row0..row0+3] is contiguous
                        if constexpr (PREC == kNsBf16) {
                            u32x2 ph, pl;
                            ph.x = bf16_bits(hv[0]) | (bf16_bits(hv[1]) << 16);
                            ph.y = bf16_bits(hv[2]) | (bf16_bits(hv[3]) << 16);
                            pl.x = bf16_bits(lv[0]) | (bf16_bits(lv[1]) << 16);
                            pl.y = bf16_bits(lv[2]) | (bf16_bits(lv[3]) << 16);
                            *reinterpret_cast<u32x2*>(ah + (size_t)col * M + row0) = ph;
                            *reinterpret_cast<u32x2*>(al + (size_t)col * M + row0) = pl;
                        } else {
                            floatx4 pv;
                            pv[0] = hv[0]; pv[1] = hv[1]; pv[2] = hv[2]; pv[3] = hv[3];
                            *reinterpret_cast<floatx4*>(ah + (size_t)col * M + row0) = pv;
                        }
                    }
                }
            }
    } else if (PHASE == kSquare) {
        const T* ah = static_cast<const T*>(G.a_hi) + aplane;
        const T* al = static_cast<const T*>(G.a_lo) + aplane;
        T* bm = static_cast<T*>(G.b) + aplane;
        const float cb = args.b, cc = args.c;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = job.tj * kTile + acc_col(wn, ni, lane);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row0 = job.ti * kTile + acc_row(wm, mi, 4 * q, lane);
                    T bv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const size_t idx = (size_t)(row0 + e) * M + col;
                        float a;
                        if constexpr (PREC == kNsBf16) a = from_bf16(ah[idx]) + from_bf16(al[idx]);
                        else a = ah[idx];
                        const float v = fmaf(cb, a, cc * acc[mi][ni][4 * q + e]);
                        bv[e] = (T)v;
                        bm[idx] = bv[e];
                    }
                    if (job.ti != job.tj) {
                        if constexpr (PREC == kNsBf16) {
                            u32x2 pb;
                            pb.x = bf16_bits(bv[0]) | (bf16_bits(bv[1]) << 16);
                            pb.y = bf16_bits(bv[2]) | (bf16_bits(bv[3]) << 16);
                            *reinterpret_cast<u32x2*>(bm + (size_t)col * M + row0) = pb;
                        } else {
                            floatx4 pv;
                            pv[0] = bv[0]; pv[1] = bv[1]; pv[2] = bv[2]; pv[3] = bv[3];
                            *reinterpret_cast<floatx4*>(bm + (size_t)col * M + row0) = pv;
                        }
                    }
                }
            }
    } else {
        const float sc = args.first ? s : 1.0f;
        const float ca = args.a;
        const int dst = args.src ^ 1;
        const T* xh = x_src;
        const bf16* xl = static_cast<const bf16*>(G.xl[args.src]) + xplane;
        T* yh = static_cast<T*>(G.x[dst]) + xplane;
        bf16* yl = static_cast<bf16*>(G.xl[dst]) + xplane;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
                const int col = job.tj * kTile + acc_col(wn, ni, lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = job.ti * kTile + acc_row(wm, mi, r, lane);
                    const size_t idx = (size_t)row * N + col;
                    float x;
                    if constexpr (PREC == kNsBf16) x = from_bf16(xh[idx]) + from_bf16(xl[idx]);
                    else x = xh[idx];
                    const float v = sc * fmaf(ca, x, acc[mi][ni][r]);
                    if constexpr (PREC == kNsBf16) {
                        bf16 h, l;
                        split_bf16(v, h, l);
                        yh[idx] = h;
                        yl[idx] = l;
                    } else {
                        yh[idx] = v;
                    }
                }
            }
    }
}

size_t ns_lds_bytes(int phase, int precision) {
    return (phase == kSquare && precision == kNsBf16) ? 4 * kTileBytes : 2 * kTileBytes;
}

template <int PHASE, int PREC>
hipError_t launch_one(const NsArgs& a, hipStream_t s) {
    const size_t lds = ns_lds_bytes(PHASE, PREC);
    if (lds > 65536) {
        // more than the default 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU)
        static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&ns_kernel<PHASE, PREC>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess) return attr;
    }
    const int grid = (a.total_jobs + kXcds - 1) / kXcds * kXcds;
    ns_kernel<PHASE, PREC><<<grid, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns(const NsArgs& a, int phase, int precision, hipStream_t s) {
    if (precision == kNsBf16) {
        if (phase == kGram) return launch_one<kGram, kNsBf16>(a, s);
        if (phase == kSquare) return launch_one<kSquare, kNsBf16>(a, s);
        return launch_one<kUpdate, kNsBf16>(a, s);
    }
    if (phase == kGram) return launch_one<kGram, kNsFp32>(a, s);
    if (phase == kSquare) return launch_one<kSquare, kNsFp32>(a, s);
    return launch_one<kUpdate, kNsFp32>(a, s);
}

const char* ns_kernel_name(int phase, int precision) {
    static const char* names[2][3] = {{"ns_gram_bf16", "ns_square_bf16", "ns_update_bf16"},
                                      {"ns_gram_fp32", "ns_square_fp32", "ns_update_fp32"}};
    return names[precision == kNsBf16 ? 0 : 1][phase];
}

}  // namespace muon
