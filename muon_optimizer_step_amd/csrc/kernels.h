// Kernel argument blocks and launchers of the Muon step library (host + device).
//
// Every multi-tensor kernel takes its tensor table by value as a kernel
// argument (no device-side table, no upload); tables are chunked on the host so
// that each argument block stays under 4 KiB.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

constexpr int kMaxGroups = 12;    // NS shape groups per NS launch
constexpr int kPrepChunk = 50;    // tensors per prep launch
constexpr int kFrobChunk = 256;   // matrices per Frobenius-scale launch
constexpr int kEmaChunk = 144;    // table entries per EMA / swap launch (24 bytes each)
constexpr int64_t kEmaEntryElems = (int64_t)1 << 30;  // a longer tensor takes several entries
constexpr int kRowsPerWaveBlock = 4;  // stored rows per workgroup when no transpose is needed
constexpr size_t kTransposeLdsBytes = 64 * 1024;  // LDS budget of the transposing prep / apply

// ---------------------------------------------------------------- prep (K1)
// Momentum update, optional row normalisation, per-row sum of squares, and the
// NS input written short-side-first into the zero-padded workspace planes.
struct PrepTensor {
    const float* grad;
    float* mom;
    void* xh;        // bf16: hi plane of X0; fp32: the X0 plane.  [M_pad][N_pad]
    void* xl;        // bf16: lo plane of X0; fp32: unused
    float* rowsq;    // one float per stored row
    int rows, cols;  // stored shape
    int m_pad, n_pad;
    int transposed;  // rows > cols: X0 = U^T
    int rb;          // stored rows per workgroup
    int block_begin; // first workgroup of this tensor
    int vec;         // grad/mom 16-byte aligned and cols % 4 == 0
    int lo8;         // bf16: the lo plane holds bytes (base-precision group)
};
struct PrepArgs {
    PrepTensor t[kPrepChunk];
    int n;
    float mu;
    int nesterov;
    int row_norm;
};

// ------------------------------------------------------- Frobenius scale
struct FrobArgs {
    const float* rowsq;          // base of the per-row sums
    float* scale;                // base of the per-matrix scales
    int rowsq_off[kFrobChunk];
    int rows[kFrobChunk];
    int scale_idx[kFrobChunk];
    int n;
};

// ------------------------------------------------------------- NS phases
// Weight update folded into the last NS update launch (one entry per matrix of
// the launch): W' = keep*W - lr_s*O with O the final X, written in stored layout.
constexpr int kMaxFused = 72;
struct FusedApply {
    float* param;
    float* out;          // optional copy of O
    float* ema;          // optional weight EMA advanced with W'
    int rows, cols;      // stored shape
    float lr_s;
    int flags;           // kApplyTransposed | kApplyVec
};
constexpr int kApplyTransposed = 1;  // stored W is X^T
constexpr int kApplyVec = 2;         // param/out/ema 16-byte aligned and cols % 4 == 0
// First Gram launch with the Frobenius scale folded in: where each matrix's
// per-row sums of squares are (one entry per matrix of the launch).
struct FrobSlot {
    int off;    // offset into the row-sum array, in floats
    int rows;   // stored rows
};
constexpr int kMaxFrobSlots = kMaxFused * (int)sizeof(FusedApply) / (int)sizeof(FrobSlot);

struct NsGroup {
    void* x[2];      // bf16: hi planes (ping-pong); fp32: X planes.  [count][M][N]
    void* xl[2];     // bf16: lo planes; fp32: unused
    void* a_hi;      // bf16: hi of A; fp32: A.  [count][M][M]
    void* a_lo;      // compensated: bf16 lo of A; base: e4m3 bytes of lo * 2^sl; fp32: unused
    void* b;         // bf16: hi of B; fp32: B.  [count][M][M]
    void* b_lo;      // compensated: bf16 lo of B; base: e4m3 bytes of A hi * 2^sa (for the square)
    float* scale;        // [count] Frobenius scale of X0 (written by a folding first Gram)
    int count, M, N;     // padded, multiples of 128
    int job_begin;
    int apply_begin;     // fused apply: entry of slot 0 in NsArgs::apply
    int frob_begin;      // folded Frobenius scale: entry of slot 0 in NsArgs::frob
};
struct NsArgs {
    NsGroup g[kMaxGroups];
    int ngroups;
    int total_jobs;
    int src;         // ping-pong plane holding the current X
    int first;       // iteration 0: fold the Frobenius scale in
    float a, b, c;
    int fuse_apply;  // last update: write W' (and O) instead of X
    float keep;      // 1 - lr*wd
    float decay, one_minus_decay;  // weight EMA
    int f8_sa, f8_sl;      // base bf16 Gram / square: e4m3 scale exponents of A hi and A lo
    int fold_frob;         // first Gram: compute the Frobenius scale from the row sums
    const float* rowsq;    // base of the per-row sums (fold_frob)
    union {
        FusedApply apply[kMaxFused];    // last update (fuse_apply)
        FrobSlot frob[kMaxFrobSlots];   // first Gram (fold_frob)
    };
};

enum NsPhase { kGram = 0, kSquare = 1, kUpdate = 2 };
enum NsMode { kModeBf16 = 0, kModeFp32 = 1, kModeBf16x3 = 2 };  // the ns_precision argument

// ------------------------------------------------------- NS chain (persistent)
// One launch runs every Newton-Schulz iteration of every base-precision bf16
// matrix of a call.  Each matrix is bound to one XCD; the workgroups of an XCD
// take the tiles of its matrices in dependency order (Gram, square, update of
// iteration 0, then of iteration 1, ...), so a matrix's planes are only ever
// shared through that XCD's L2.  Per-matrix records and counters live in the
// workspace; chain_setup writes them before the chain launch.
struct ChainMat {
    float* param;        // fused apply (last iteration): W, optional O copy, optional EMA
    float* out;
    float* ema;
    float shape_scale;   // sqrt(max(1, rows / cols)); the apply uses lr * shape_scale
    int flags;           // kApplyTransposed | kApplyVec
    int rows, cols;      // stored shape
    int group, slot;     // NsGroup of the launch and slot in it
    int rowsq_off;       // first per-row sum of squares (floats)
    int tiles_sym;       // Gram / square tiles per iteration (upper triangle)
    int tiles_upd;       // update tiles per iteration
    int pad;
};
static_assert(sizeof(ChainMat) == 64, "ChainMat is one 64-byte record");
constexpr int kChainCtrWords = 64;   // per matrix: grab counter at [0], done counter at [32] (own 128-byte lines)
constexpr int kChainMaxSteps = 16;
struct ChainArgs {
    NsGroup g[kMaxGroups];
    const ChainMat* mats;     // ordered by XCD, highest priority first within an XCD
    uint32_t* ctr;            // [nmat][kChainCtrWords], then the status word
    const float* rowsq;
    int xcd_begin[kXcds + 1]; // matrices [xcd_begin[x], xcd_begin[x + 1]) run on XCD x
    int nmat;
    int ns_steps;
    int fuse_apply;           // the last update writes W' (and O, E') instead of X
    float keep;               // 1 - lr*wd
    float lr;
    float decay, one_minus_decay;
    float a[kChainMaxSteps], b[kChainMaxSteps], c[kChainMaxSteps];
    int f8_sa[kChainMaxSteps];  // e4m3 scale exponent of A hi per iteration (A lo: + 8)
    uint64_t timeout_ticks;   // bound on any wait, in s_memrealtime ticks (100 MHz)
};
constexpr int kChainSetupChunk = 60;
struct ChainSetupArgs {
    ChainMat rec[kChainSetupChunk];
    ChainMat* dst;
    uint32_t* zero;           // counters to clear (first setup launch of a call), or NULL
    int n;
    int nzero;
};
constexpr uint32_t kChainStatusTimeout = 1u;   // a wait ran past timeout_ticks

// ------------------------------------------------------------- apply (K3)
struct ApplyTensor {
    float* param;
    float* out;          // optional copy of O (stored layout)
    float* ema;          // optional weight EMA advanced with W'
    const void* xh;      // final X: bf16 hi plane or fp32 plane
    const void* xl;      // bf16 lo plane
    const float* scale;  // Frobenius scale (used when no NS step ran)
    float lr_s;          // lr * shape scale
    int rows, cols;
    int n_pad;           // leading dimension of X
    int transposed;
    int rb;
    int block_begin;
    int vec;             // param/out/ema 16-byte aligned and cols % 4 == 0
    int lo8;             // bf16: the lo plane holds bytes (base-precision group)
};
constexpr int kApplyChunk = 44;    // tensors per apply launch
struct ApplyArgs {
    ApplyTensor t[kApplyChunk];
    int n;
    float keep;          // 1 - lr*wd
    float decay, one_minus_decay;  // weight EMA
    int use_scale;       // 1 when ns_steps == 0
};

// ------------------------------------------------------------------ EMA (K4)
struct EmaTensor {
    float* ema;
    const float* param;
    int numel;           // <= kEmaEntryElems
    int block_begin;
};
struct EmaArgs {
    EmaTensor t[kEmaChunk];
    int n;
    float decay;
    float one_minus_decay;
};
constexpr int kEmaThreads = 256;
constexpr int kEmaVec = 4;                                    // float4 per thread per operand
constexpr int kEmaElemsPerBlock = kEmaThreads * 4 * kEmaVec;

// Swap of two fp32 buffers per tensor (the EMA swap-in), same chunking as the EMA
struct SwapTensor {
    float* a;
    float* b;
    int numel;           // <= kEmaEntryElems
    int block_begin;
};
struct SwapArgs {
    SwapTensor t[kEmaChunk];
    int n;
};

// AdamW over a chunk of tensors (one workgroup per kAdamElemsPerBlock elements)
constexpr int kAdamChunk = 64;
struct AdamTensor {
    float* param;
    const float* grad;
    float* m;
    float* v;
    float* ema;          // nullable
    int64_t numel;
    int block_begin;
    int vec;             // every pointer 16-byte aligned
};
struct AdamArgs {
    AdamTensor t[kAdamChunk];
    int n;
    float keep;          // 1 - lr*wd
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float step_size;     // lr / (1 - beta1^t)
    float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
    float eps;
    float decay, one_minus_decay;
};
constexpr int kAdamThreads = 256;
constexpr int kAdamElemsPerBlock = kAdamThreads * 4 * 2;  // float4 x 2 per thread

static_assert(sizeof(PrepArgs) <= 4096, "prep kernel arguments exceed 4 KiB");
static_assert(sizeof(AdamArgs) <= 4096, "AdamW kernel arguments exceed 4 KiB");
static_assert(sizeof(SwapArgs) <= 4096, "swap kernel arguments exceed 4 KiB");
static_assert(sizeof(FrobArgs) <= 4096, "frob kernel arguments exceed 4 KiB");
static_assert(sizeof(NsArgs) <= 4096, "NS kernel arguments exceed 4 KiB");
static_assert(sizeof(ChainArgs) <= 4096, "chain kernel arguments exceed 4 KiB");
static_assert(sizeof(ChainSetupArgs) <= 4096, "chain setup arguments exceed 4 KiB");
static_assert(sizeof(ApplyArgs) <= 4096, "apply kernel arguments exceed 4 KiB");
static_assert(sizeof(EmaArgs) <= 4096, "EMA kernel arguments exceed 4 KiB");

// Launchers: enqueue on `s`, return hipGetLastError() of the launch.
hipError_t launch_prep(const PrepArgs& a, int precision, int blocks, size_t lds_bytes, hipStream_t s);
hipError_t launch_frob(const FrobArgs& a, hipStream_t s);
hipError_t launch_ns(const NsArgs& a, int phase, int precision, bool compensated, hipStream_t s);
hipError_t launch_apply(const ApplyArgs& a, int precision, int blocks, size_t lds_bytes, hipStream_t s);
hipError_t launch_ema(const EmaArgs& a, int blocks, hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, int blocks, hipStream_t s);
hipError_t launch_swap(const SwapArgs& a, int blocks, hipStream_t s);
hipError_t launch_chain_setup(const ChainSetupArgs& a, hipStream_t s);
hipError_t launch_chain(const ChainArgs& a, int workgroups, hipStream_t s);
constexpr int kChainWgPerCu = 2;   // resident chain workgroups per CU (LDS-bound)

const char* ns_kernel_name(int phase, int precision, bool compensated, bool fused_apply);

// Short side below which the bf16 precision runs the compensated products:
// with fewer singular values the bf16 rounding of the base products no longer
// averages out and the error can pass 2e-2.
constexpr int kCompensateBelow = 192;

}  // namespace muon
