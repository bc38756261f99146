// Device-side building blocks of the Newton-Schulz tiles on gfx950: LDS
// staging layouts, operand loaders, MFMA fragment reads, the bf16 / e4m3 /
// byte-lo encodings of the workspace planes, the fused weight apply, and the
// update tile.  Shared by the per-phase kernels (ns.hip) and the persistent
// chain kernel (chain.hip); see ns.hip for the numerics and the tiling.
#pragma once

#include "common.h"
#include "kernels.h"

namespace muon {
namespace {   // internal linkage: every kernel file compiles its own copy

// The thread index the tiles compute their addresses from.  The persistent
// chain kernel sets NS_OPAQUE_TID: read through an opaque move inside every
// tile, the per-thread address terms of all three tile kinds are not hoisted
// out of its scheduling loop (where they would all stay live at once and
// spill).
#ifndef NS_OPAQUE_TID
#define NS_OPAQUE_TID 0
#endif
__device__ inline int tid_x() {
    if constexpr (NS_OPAQUE_TID != 0) {
        int t;
        asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)__builtin_amdgcn_workitem_id_x()));
        return t;
    } else {
        return (int)__builtin_amdgcn_workitem_id_x();
    }
}

constexpr int kThreads = 256;
constexpr int kXPitch = 256 + 32;           // row pitch of a natural-layout X stage (see XLoader)
// K bytes per LDS stage per operand row: RB = 128 (64 bf16 / 32 fp32) or 256.
// Rows are padded by 16 bytes, which keeps the b128 fragment reads conflict-free.
template <int RB> struct Stage {
    static constexpr int kPitch = RB + 16;
    static constexpr int kBK = RB / 2;      // bf16 elements of K per stage
    // one operand slot: 128 rows of K, or kBK rows of natural-layout X
    static constexpr int kSlot = (kTile * kPitch > kBK * kXPitch) ? kTile * kPitch : kBK * kXPitch;
};
constexpr int kStagePitch = kTile + 4;      // fp32 epilogue staging row pitch
constexpr int kStageBytes = 64 * kStagePitch * 4;  // half a tile (64 rows) of fp32
// Column of element (row, col) in the fp32 staging buffer: aligned 8-column
// blocks are permuted per group of 8 rows, so the transposed (column) reads of
// the mirror and tall-apply passes, 8 rows x 8 columns per wave, hit 64
// distinct banks; rows keep their 8-column blocks contiguous and 16-byte aligned.
__device__ inline int stage_col(int row, int col) { return col ^ (((row >> 3) & 7) << 3); }
static_assert(kStageBytes <= 2 * Stage<128>::kSlot, "epilogue staging must fit in the operand LDS");

#ifndef NS_SYM_DMA
#define NS_SYM_DMA 1   // Gram operands loaded straight into LDS (double-buffered)
#endif
#ifndef NS_SQ_FP8
#define NS_SQ_FP8 1    // base bf16 square: cross terms Ah Al + Al Ah on the fp8 MFMA
#endif

// Direct loads for the phases with two operand tiles per stage (the split
// phases stage four, which would need 64-byte stages to fit two buffers).
constexpr bool ns_sym_dma(int phase, int precision, bool comp) {
    return NS_SYM_DMA != 0 && !(precision == kNsBf16 && (phase == kSquare || comp));
}

// K bytes per LDS stage of the Gram and square.  Register staging: 256 for the
// bf16 base Gram, whose long contraction gains from fewer, larger stages, 128
// otherwise.  Direct loads (two buffers per group): 128.
constexpr int ns_sym_stage_bytes(int phase, int precision, bool comp, bool dma) {
    if (dma) return 128;
    return (precision == kNsBf16 && !comp && phase == kGram) ? 256 : 128;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Explicit waits and a bare barrier for the direct-load K loop: the compiler
// does not count global_load_lds against later LDS reads, so the loop waits
// for its own loads (vmcnt) and publishes them with s_barrier.  The empty asm
// statements with memory clobbers keep LDS accesses on their side.
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ inline void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int PREC> struct Elem;
template <> struct Elem<kNsBf16> { typedef bf16 T; };
template <> struct Elem<kNsFp32> { typedef float T; };

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

// 128 rows x RB bytes of a row-major operand whose K index is contiguous
// ("NT" operand).  Thread t moves 16 bytes of row t/C + (256/C)q, chunk t%C,
// with C = RB/16 chunks per row.
template <int RB>
struct NtLoader {
    static constexpr int C = RB / 16, Q = RB / 32;
    u32x4 r[Q];
    __device__ inline void load(const uint8_t* base, size_t ld_bytes, int kbyte) {
        const int t = tid_x() % 256;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint8_t* p = base + (size_t)(t / C + (256 / C) * q) * ld_bytes + kbyte + (t % C) * 16;
            r[q] = *reinterpret_cast<const u32x4*>(p);
        }
    }
    __device__ inline void store(uint8_t* lds) const {
        const int t = tid_x() % 256;
#pragma unroll
        for (int q = 0; q < Q; ++q)
            *reinterpret_cast<u32x4*>(lds + (t / C + (256 / C) * q) * Stage<RB>::kPitch + (t % C) * 16) = r[q];
    }
};

// fp32 X[k][j] (j contiguous in memory) staged as LDS[j][k] so that K is
// contiguous per lane for the MFMA B operand: thread t reads 4 k-rows x 4 j
// (16-byte loads) and transposes in registers.
template <int PREC> struct TLoader;

template <> struct TLoader<kNsFp32> {
    floatx4 v[4];
    __device__ inline void load(const float* x, size_t ld, int k0, int j0) {
        const int t = tid_x();
        const int jq = t % 32, kb = t / 32;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = *reinterpret_cast<const floatx4*>(x + (size_t)(k0 + 4 * kb + r) * ld + j0 + 4 * jq);
    }
    __device__ inline void store(uint8_t* lds) const {
        const int t = tid_x();
        const int jq = t % 32, kb = t / 32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            floatx4 w;
            w[0] = v[0][c]; w[1] = v[1][c]; w[2] = v[2][c]; w[3] = v[3][c];
            *reinterpret_cast<floatx4*>(lds + (4 * jq + c) * Stage<128>::kPitch + kb * 16) = w;
        }
    }
};

// bf16 X[k][j] tile for the update's B operand kept in its natural layout:
// BK k-rows x 128 j (256 bytes) per stage, rows padded to kXPitch so that the
// transposing LDS reads below are free of bank conflicts.  Thread t moves 16
// bytes: row t/16 + 16q, column chunk t%16.
template <int BK>
struct XLoader {
    static constexpr int Q = BK / 16;
    u32x4 r[Q];
    __device__ inline void load(const bf16* x, size_t ld, int k0, int j0) {
        const int t = tid_x();
#pragma unroll
        for (int q = 0; q < Q; ++q)
            r[q] = *reinterpret_cast<const u32x4*>(x + (size_t)(k0 + t / 16 + 16 * q) * ld + j0 + 8 * (t % 16));
    }
    __device__ inline void store(uint8_t* lds) const {
        const int t = tid_x();
#pragma unroll
        for (int q = 0; q < Q; ++q)
            *reinterpret_cast<u32x4*>(lds + (t / 16 + 16 * q) * kXPitch + (t % 16) * 16) = r[q];
    }
};

typedef short short4v __attribute__((ext_vector_type(4)));

// B-operand fragment of v_mfma_f32_32x32x16_bf16 from the natural [k][j] tile:
// lane l needs X[k0 + 8(l/32) + e][j0 + l%32], e = 0..7.  ds_read_b64_tr_b16
// hands lane l' of each 16-lane group element l'%4 of the 8-byte chunk read by
// lane 4e + l'/4, so lane l points at row k0 + 8(l/32) + 4h + (l%16)/4,
// columns j0 + 16((l/16)%2) + 4(l%4) .. +3, for the halves h = 0, 1.
__device__ inline u32x4 lds_frag_tr(const uint8_t* tile, int k0, int j0, int lane) {
    const int row = k0 + 8 * (lane / 32) + (lane % 16) / 4;
    const int col = j0 + 16 * ((lane / 16) % 2) + 4 * (lane % 4);
    typedef __attribute__((address_space(3))) short4v lds_short4;
    const uint8_t* p0 = tile + row * kXPitch + col * 2;
    const short4v a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
    const short4v b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0 + 4 * kXPitch));
    u32x4 r;
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    r[0] = ua[0]; r[1] = ua[1]; r[2] = ub[0]; r[3] = ub[1];
    return r;
}

template <int RB>
__device__ inline u32x4 lds_frag(const uint8_t* tile, int row, int kc, int lane) {
    return *reinterpret_cast<const u32x4*>(tile + row * Stage<RB>::kPitch + kc * 32 + (lane / 32) * 16);
}

struct Job {
    int g, slot, ti, tj;
};

__device__ inline void unpack8(const u32x4& w, float* v) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        v[2 * p] = from_bf16(bits_bf16(w[p] & 0xFFFFu));
        v[2 * p + 1] = from_bf16(bits_bf16(w[p] >> 16));
    }
}

// 8 consecutive elements of a plane <-> 8 floats.
template <int PREC>
__device__ inline void load8(const void* plane, size_t idx, float* v) {
    if constexpr (PREC == kNsBf16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(plane) + idx);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v[2 * p] = from_bf16(bits_bf16(w[p] & 0xFFFFu));
            v[2 * p + 1] = from_bf16(bits_bf16(w[p] >> 16));
        }
    } else {
        const floatx4* s = reinterpret_cast<const floatx4*>(static_cast<const float*>(plane) + idx);
        const floatx4 a = s[0], b = s[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    }
}

// Store 8 values: bf16 -> hi plane (and lo plane when lo != nullptr); fp32 -> plane `hi`.
template <int PREC>
__device__ inline void store8(void* hi, void* lo, size_t idx, const float* v) {
    if constexpr (PREC == kNsBf16) {
        u32x4 wh, wl;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            wh[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
            wl[p] = pack_bf16x2(v[2 * p] - bf16_lo_f(wh[p]), v[2 * p + 1] - bf16_hi_f(wh[p]));
        }
        *reinterpret_cast<u32x4*>(static_cast<bf16*>(hi) + idx) = wh;
        if (lo) *reinterpret_cast<u32x4*>(static_cast<bf16*>(lo) + idx) = wl;
    } else {
        floatx4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[4 + e]; }
        floatx4* d = reinterpret_cast<floatx4*>(static_cast<float*>(hi) + idx);
        d[0] = a;
        d[1] = b;
    }
}

// fp8 cross terms of the base square.  A = Ah + Al with Ah = rne_bf16(A); the
// square needs Ah Ah + Ah Al + Al Ah, and the cross terms are ~2^-8 of A A, so
// OCP e4m3 operands (3 mantissa bits) carry them with an error far below the
// bf16 rounding of B that follows; what the base precision cannot drop is the
// cross term as a whole.  The Gram stores, besides Ah in bf16, e4m3(Al * 2^sl)
// and e4m3(Ah * 2^sa), one byte per element each; the square runs
// v_mfma_scale_f32_32x32x64_f8f6f4 on them with E8M0 scales 2^-sa and 2^-sl,
// so the cross products land unscaled in the same accumulators as Ah Ah.  sa
// and sl (= sa + 8) come from the host's bound on |A| for the iteration, which
// keeps every scaled operand under 224 (e4m3's largest value is 448).
typedef int v8i __attribute__((ext_vector_type(8)));
constexpr int kF8Pitch = 64 + 16;              // LDS row pitch of an e4m3 tile (64 K bytes per stage)
constexpr int kF8TileBytes = kTile * kF8Pitch;

// Four floats -> four e4m3 bytes (round to nearest even), a first.  Inputs
// are clamped to the e4m3 range first: the scales keep them under 224, and a
// table that drives X far past its bound then saturates instead of producing
// NaN codes (the conversion writes NaN from 480 up).
__device__ inline uint32_t f8_pack4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
__device__ inline float f8_decode(uint32_t word, int byte) {
    switch (byte) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
    }
}

// Store 8 A values of the base Gram: the bf16 hi plane, and two e4m3 byte
// planes for the square's cross terms, lo * 2^sl and hi * 2^sa.
__device__ inline void store8_hi_f8lo(void* hi, void* lo, void* hi8, size_t idx, const float* v, float lo_scale,
                                      float hi_scale) {
    u32x4 wh;
    float r[8], q[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        wh[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
        const float h0 = bf16_lo_f(wh[p]), h1 = bf16_hi_f(wh[p]);
        r[2 * p] = (v[2 * p] - h0) * lo_scale;
        r[2 * p + 1] = (v[2 * p + 1] - h1) * lo_scale;
        q[2 * p] = h0 * hi_scale;
        q[2 * p + 1] = h1 * hi_scale;
    }
    u32x2 wl;
    wl[0] = f8_pack4(r[0], r[1], r[2], r[3]);
    wl[1] = f8_pack4(r[4], r[5], r[6], r[7]);
    *reinterpret_cast<u32x4*>(static_cast<bf16*>(hi) + idx) = wh;
    *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(lo) + idx) = wl;
    u32x2 w8;
    w8[0] = f8_pack4(q[0], q[1], q[2], q[3]);
    w8[1] = f8_pack4(q[4], q[5], q[6], q[7]);
    *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(hi8) + idx) = w8;
}

// Store 8 X values as a bf16 hi plane and a byte lo plane (lo8_insert).
__device__ inline void store8_lo8(void* hi, void* lo, size_t idx, const float* v) {
    u32x4 wh;
    u32x2 wl = {0u, 0u};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        wh[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
        wl[p / 2] = lo8_insert(v[2 * p], bf16_lo_f(wh[p]), wl[p / 2], 2 * (p % 2));
        wl[p / 2] = lo8_insert(v[2 * p + 1], bf16_hi_f(wh[p]), wl[p / 2], 2 * (p % 2) + 1);
    }
    *reinterpret_cast<u32x4*>(static_cast<bf16*>(hi) + idx) = wh;
    *reinterpret_cast<u32x2*>(static_cast<uint8_t*>(lo) + idx) = wl;
}

// Fused weight update for up to 8 consecutive stored elements starting at idx:
// W' = keep*W - lr_s*O, the optional copy of O, and the optional weight EMA
// E' = d*E + (1-d)*W'.  apply_load fetches W (and E) early, into registers, so
// that the epilogue issues every load of a half tile before its first store
// (a store to W could otherwise alias the next load in the compiler's view and
// serialise one memory latency per row).
__device__ inline void apply_load(const FusedApply& F, size_t idx, int count, floatx4* w, floatx4* e) {
    if (count >= 8 && (F.flags & kApplyVec)) {
        const floatx4* w4 = reinterpret_cast<const floatx4*>(F.param + idx);
        w[0] = w4[0];
        w[1] = w4[1];
        if (F.ema) {
            const floatx4* e4 = reinterpret_cast<const floatx4*>(F.ema + idx);
            e[0] = e4[0];
            e[1] = e4[1];
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k < count) {
            w[k / 4][k % 4] = F.param[idx + k];
            if (F.ema) e[k / 4][k % 4] = F.ema[idx + k];
        }
    }
}

__device__ inline void apply_store(const FusedApply& F, size_t idx, int count, const float* v, const floatx4* w,
                                   const floatx4* e, float keep, float d, float omd) {
    floatx4 wn[2], en[2];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        wn[k / 4][k % 4] = fmaf(-F.lr_s, v[k], keep * w[k / 4][k % 4]);
        en[k / 4][k % 4] = fmaf(d, e[k / 4][k % 4], omd * wn[k / 4][k % 4]);
    }
    if (count >= 8 && (F.flags & kApplyVec)) {
        // W' and E' are not read again in the step: streaming stores
        floatx4* w4 = reinterpret_cast<floatx4*>(F.param + idx);
        __builtin_nontemporal_store(wn[0], w4);
        __builtin_nontemporal_store(wn[1], w4 + 1);
        if (F.out) {
            floatx4 o0, o1;
#pragma unroll
            for (int k = 0; k < 4; ++k) { o0[k] = v[k]; o1[k] = v[4 + k]; }
            floatx4* o4 = reinterpret_cast<floatx4*>(F.out + idx);
            o4[0] = o0;
            o4[1] = o1;
        }
        if (F.ema) {
            floatx4* e4 = reinterpret_cast<floatx4*>(F.ema + idx);
            __builtin_nontemporal_store(en[0], e4);
            __builtin_nontemporal_store(en[1], e4 + 1);
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if (k < count) {
            F.param[idx + k] = wn[k / 4][k % 4];
            if (F.out) F.out[idx + k] = v[k];
            if (F.ema) F.ema[idx + k] = en[k / 4][k % 4];
        }
    }
}

// The update X' = s (a X + B X), s the Frobenius scale on the first iteration
// and 1 after: one 128 x 128 tile of X' per workgroup, 4 waves of 64 x 64.  The
// rows ti*128 .. +127 of B (K contiguous) are the A operand and the column
// panel tj*128 .. +127 of X the B operand.  With FUSE, the last iteration
// writes W' = keep W - lr_s X' (and the EMA) instead of X' (F_ is read only then).
// Scalars of one update tile: the iteration's a, whether X is X0 (then the
// Frobenius scale of the slot multiplies the result), the ping-pong plane
// holding X, and the weight-apply / EMA factors of a fused last iteration.
struct UpdateCtx {
    float a;
    int first;
    int src;
    float keep, decay, one_minus_decay;
};

// IN_KERNEL: X and the Frobenius scale were written earlier in the same
// launch (the persistent chain), so the X lo plane is read with a plain load
// (a streaming load may go past the L2 that holds the freshly written lines)
// and the scale through the vector path (never a scalar-cache line).
template <int PREC, bool COMP, bool FUSE, bool IN_KERNEL = false>
__device__ inline void update_tile(const NsGroup& G, const Job& job, const UpdateCtx& args, const FusedApply& F_,
                                   uint8_t* lds) {
    typedef typename Elem<PREC>::T T;
    // operands carry a lo plane (and the MFMAs run hi*hi + hi*lo + lo*hi)
    constexpr bool kSplit = (PREC == kNsBf16) && COMP;
    // bf16 keeps the X tile in its natural [k][j] layout and reads it with
    // transposing LDS loads; fp32 transposes into LDS
    constexpr bool kTr = PREC == kNsBf16;
    constexpr int kRB = 128;                      // K bytes per stage per row
    constexpr int kBK = kRB / (int)sizeof(T);     // K elements per stage
    constexpr int kSlot = Stage<kRB>::kSlot;
    const int M = G.M, N = G.N;
    const int lane = tid_x() % kWave, wave = tid_x() / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const size_t xplane = (size_t)job.slot * M * N;
    const size_t aplane = (size_t)job.slot * M * M;
    const int src = args.src;
    const int K = M;

    // LDS operand tiles: [0] B hi rows, [1] X hi, [2] / [3] their lo planes
    auto tile = [&](int which) -> uint8_t* { return lds + which * kSlot; };

    const size_t ld_bytes = (size_t)M * sizeof(T);
    const uint8_t* ga = reinterpret_cast<const uint8_t*>(static_cast<const T*>(G.b) + aplane + (size_t)job.ti * kTile * M);
    const uint8_t* gal = reinterpret_cast<const uint8_t*>(static_cast<const T*>(G.b_lo) + aplane + (size_t)job.ti * kTile * M);
    const T* xb = static_cast<const T*>(G.x[src]) + xplane;
    const T* xbl = static_cast<const T*>(G.xl[src]) + xplane;

    floatx16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

    // Registers staging one K stage from global memory into LDS.
    NtLoader<kRB> la, lal;
    TLoader<kNsFp32> lt;
    XLoader<kBK> lx, lxl;
    auto issue = [&](int k0) {
        la.load(ga, ld_bytes, k0 * (int)sizeof(T));
        if (kSplit) lal.load(gal, ld_bytes, k0 * (int)sizeof(T));
        if constexpr (kTr) {
            lx.load(reinterpret_cast<const bf16*>(xb), (size_t)N, k0, job.tj * kTile);
            if (kSplit) lxl.load(reinterpret_cast<const bf16*>(xbl), (size_t)N, k0, job.tj * kTile);
        } else {
            lt.load(reinterpret_cast<const float*>(xb), (size_t)N, k0, job.tj * kTile);
        }
    };
    auto commit = [&]() {
        la.store(tile(0));
        if (kSplit) lal.store(tile(2));
        if constexpr (kTr) {
            lx.store(tile(1));
            if (kSplit) lxl.store(tile(3));
        } else {
            lt.store(tile(1));
        }
    };
    auto bfrag = [&](const uint8_t* tb, int ni, int kc) -> u32x4 {
        if constexpr (kTr) return lds_frag_tr(tb, kc * 16, wn * 64 + ni * 32, lane);
        else return lds_frag<kRB>(tb, wn * 64 + ni * 32 + lane % 32, kc, lane);
    };
    auto compute = [&]() {
        const uint8_t* t_a = tile(0);
        const uint8_t* t_b = tile(1);
        const uint8_t* t_al = tile(2);
        const uint8_t* t_bl = tile(3);
#pragma unroll
        for (int kc = 0; kc < kRB / 32; ++kc) {
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) fa[mi] = lds_frag<kRB>(t_a, wm * 64 + mi * 32 + lane % 32, kc, lane);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) fb[ni] = bfrag(t_b, ni, kc);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) mfma_chunk<PREC>(acc[mi][ni], fa[mi], fb[ni]);
            if (kSplit) {
                u32x4 fal[2], fbl[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) fal[mi] = lds_frag<kRB>(t_al, wm * 64 + mi * 32 + lane % 32, kc, lane);
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) fbl[ni] = bfrag(t_bl, ni, kc);
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

    // The tile's own rows ti*128 .. +127 of X pass through the K loop as the B
    // operand.  With bf16 the K loop starts right after them and wraps around,
    // so they are its last two stages; the XLoader thread mapping (row t/16 +
    // 16q, columns 8(t%16)) is the epilogue's row mapping, so each thread keeps
    // those registers instead of reloading X from HBM.
    constexpr bool kKeep = kTr;
    static_assert(!kKeep || kTile == 2 * kBK, "the own rows are the last two stages");
    u32x4 keep_h[2][4], keep_l[2][4];
    const int nk = K / kBK;   // >= 2: K is padded to a multiple of 128
    auto kstart = [&](int kt) -> int {
        if constexpr (kKeep) return ((job.ti + 1) * kTile + kt * kBK) % K;
        else return kt * kBK;
    };
    issue(kstart(0));
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        commit();
        if constexpr (kKeep) {
            if (kt == nk - 2) {   // rows ti*128 .. +63
#pragma unroll
                for (int q = 0; q < 4; ++q) { keep_h[0][q] = lx.r[q]; if (kSplit) keep_l[0][q] = lxl.r[q]; }
            }
        }
        __syncthreads();
        if (kt + 1 < nk) issue(kstart(kt + 1));
        compute();
    }
    if constexpr (kKeep) {   // the last stage: rows ti*128 + 64 .. +127
#pragma unroll
        for (int q = 0; q < 4; ++q) { keep_h[1][q] = lx.r[q]; if (kSplit) keep_l[1][q] = lxl.r[q]; }
    }

    // ---------------------------------------------------------- epilogue
    // Two passes of 64 rows: the waves holding those rows park their fp32
    // accumulators in LDS, then all threads finish 8 consecutive columns of a
    // row each with 16-byte global accesses.
    float* stage = reinterpret_cast<float*>(lds);
    // Base-precision bf16 updates carry X's low part as bytes (lo8_insert);
    // that plane for both halves is fetched before the accumulators are
    // staged, so one memory latency overlaps the LDS work.
    constexpr bool kLo8 = (PREC == kNsBf16) && !COMP;
    u32x2 xl_pre[2][4];
    if constexpr (kLo8) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const size_t idx = xplane + (size_t)(job.ti * kTile + h * 64 + tid_x() / 16 + 16 * p) * N +
                                   job.tj * kTile + 8 * (tid_x() % 16);
                const u32x2* q = reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(G.xl[src]) + idx);
                if constexpr (IN_KERNEL) xl_pre[h][p] = *q;
                else xl_pre[h][p] = __builtin_nontemporal_load(q);   // read by this tile only: streaming
            }
    }
    float s;
    if constexpr (IN_KERNEL) s = __hip_atomic_load(G.scale + job.slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else s = G.scale[job.slot];
    const float sc = args.first ? s : 1.0f;
    const int t = tid_x();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bool tall = FUSE && (F_.flags & kApplyTransposed);   // stored W is X^T
        const int row_base = job.ti * kTile + h * 64;
        // fused apply: W and E of this half's outputs are in flight while the
        // accumulators are staged (row pass mapping for stored rows = X rows,
        // column pass mapping for tall matrices)
        floatx4 w_pre[4][2], e_pre[4][2];
        if constexpr (FUSE) {
            const FusedApply& F = F_;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int wr = tall ? job.tj * kTile + t / 8 + 32 * p : row_base + t / 16 + 16 * p;
                const int wc = tall ? row_base + 8 * (t % 8) : job.tj * kTile + 8 * (t % 16);
                if (wr < F.rows && wc < F.cols) apply_load(F, (size_t)wr * F.cols + wc, F.cols - wc, w_pre[p], e_pre[p]);
            }
        }
        __syncthreads();
        if (wm == h) {
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = mi * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                        const int col = wn * 64 + ni * 32 + (lane % 32);
                        stage[row * kStagePitch + stage_col(row, col)] = acc[mi][ni][r];
                    }
        }
        __syncthreads();
        // row pass: thread -> (row t/16 + 16p, columns 8*(t%16) .. +7)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int lr = t / 16 + 16 * p;
            const int lc = 8 * (t % 16);
            float* sp = stage + lr * kStagePitch + stage_col(lr, lc);
            float v[8];
            {
                const floatx4 a = *reinterpret_cast<const floatx4*>(sp);
                const floatx4 b = *reinterpret_cast<const floatx4*>(sp + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
            }
            const size_t idx = xplane + (size_t)(row_base + lr) * N + job.tj * kTile + lc;
            float xh[8], xl[8], x[8];
            if constexpr (kKeep) unpack8(keep_h[h][p], xh);
            else load8<PREC>(G.x[src], idx, xh);
            if constexpr (kLo8) {
                const u32x2 q = xl_pre[h][p];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = lo8_decode(xh[e], q[e / 4], e % 4);
            } else if constexpr (PREC == kNsBf16) {
                unpack8(keep_l[h][p], xl);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = xh[e] + xl[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = xh[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = sc * fmaf(args.a, x[e], v[e]);
            if constexpr (!FUSE) {
                if constexpr (kLo8) store8_lo8(G.x[src ^ 1], G.xl[src ^ 1], idx, v);
                else store8<PREC>(G.x[src ^ 1], G.xl[src ^ 1], idx, v);
            } else if (!tall) {
                // X row = stored row, X column = stored column
                const FusedApply& F = F_;
                const int gi = row_base + lr, gj = job.tj * kTile + lc;
                if (gi < F.rows && gj < F.cols)
                    apply_store(F, (size_t)gi * F.cols + gj, F.cols - gj, v, w_pre[p], e_pre[p], args.keep,
                                args.decay, args.one_minus_decay);
            } else {
                // keep the final value for the column pass
                floatx4 a, b;
#pragma unroll
                for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[4 + e]; }
                *reinterpret_cast<floatx4*>(sp) = a;
                *reinterpret_cast<floatx4*>(sp + 4) = b;
            }
        }
        if (tall) {
            __syncthreads();
            // stored W is X^T: W row tj*128 + c, columns row_base + 8*chunk .. +7
            const FusedApply& F = F_;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int chunk = t % 8;
                const int c = t / 8 + 32 * p;
                const int wr = job.tj * kTile + c, wc = row_base + chunk * 8;
                if (wr < F.rows && wc < F.cols) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = stage[(chunk * 8 + e) * kStagePitch + stage_col(chunk * 8 + e, c)];
                    apply_store(F, (size_t)wr * F.cols + wc, F.cols - wc, v, w_pre[p], e_pre[p], args.keep,
                                args.decay, args.one_minus_decay);
                }
            }
        }
    }
}

}  // namespace
}  // namespace muon
