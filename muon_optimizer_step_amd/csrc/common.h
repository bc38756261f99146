// Shared device-side definitions for the gfx950 Muon step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int kTile = 128;        // NS output tile edge; workspace dims are padded to it
constexpr float kEps = 1e-7f;     // added to the row and Frobenius norms

// Storage precision of the NS workspace planes (X, A, B): bf16 hi/lo pairs or fp32.
enum NsPrecision { kNsBf16 = 0, kNsFp32 = 1 };

__host__ __device__ inline int pad_to_tile(int x) { return (x + kTile - 1) / kTile * kTile; }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ inline bf16 to_bf16(float x) { return (bf16)x; }
__device__ inline float from_bf16(bf16 x) { return (float)x; }

// Two floats -> two bf16 in one word, a in the low half (round to nearest
// even; one v_cvt_pk_bf16_f32 for the pair), and the two halves back as floats.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ inline float bf16_lo_f(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi_f(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }


// Base-precision groups keep the low part of X as one byte per element
// instead of a second bf16.  With hi = m 2^e (m in [0.5, 1), the frexp
// exponent), |x - hi| is at most half a bf16 ulp, 2^(e - 9), so the byte
// u = round((x - hi) 2^(16 - e)) + 128, clamped to [0, 255], holds it in
// steps of 2^(e - 16): hi + lo keeps x to 2^-16 of its magnitude (2^-15 where
// the code clamps, |x - hi| within a step of half an ulp), as a bf16 pair
// does, in 3 bytes instead of 4.  Both directions are exact apart from the
// one rounding to the byte (ldexp scales by a power of two; x - hi is exact).
// lo8_insert returns word with byte b set to the code of x (v_cvt_pk_u8_f32:
// round to nearest even, clamp to [0, 255]); lo8_decode reads byte b back.
__device__ inline uint32_t lo8_insert(float x, float hi, uint32_t word, int b) {
    const int e = __builtin_amdgcn_frexp_expf(hi);
    return __builtin_amdgcn_cvt_pk_u8_f32(ldexpf(x - hi, 16 - e) + 128.0f, b, word);
}
__device__ inline float lo8_decode(float hi, uint32_t word, int b) {
    const float u = (float)((word >> (8 * b)) & 0xFFu);
    return hi + ldexpf(u - 128.0f, __builtin_amdgcn_frexp_expf(hi) - 16);
}

__device__ inline uint32_t bf16_bits(bf16 x) { return (uint32_t)__builtin_bit_cast(uint16_t, x); }
__device__ inline bf16 bits_bf16(uint32_t b) { return __builtin_bit_cast(bf16, (uint16_t)b); }

__device__ inline float wave_sum(float v) {
    // Butterfly over the 64 lanes; every lane ends with the same total and the
    // order of additions is fixed, so results are reproducible.
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Frobenius scale 1 / (sqrt(sum of rows[0 .. n)) + eps) over a 512-thread
// workgroup in a fixed order: thread t sums rows t, t + 512, ...; each wave
// reduces with wave_sum; every thread adds the 8 wave totals in wave order.
// The frob kernel and the first Gram launch that folds it in both use this,
// so the scale is the same bits either way.  Split in two so that a caller can
// put other loads between them: frob_prefetch loads the first 4 rows of the
// thread, frob_finish adds them (0 for rows past n, which leaves the sum's
// bits unchanged) and any further rows.  red: 8 floats of LDS; every thread of the
// workgroup must call frob_finish; the result is valid in every thread.  The
// caller separates red from later LDS writes with a barrier of its own.
__device__ inline void frob_prefetch(const float* rows, int n, float v[4]) {
    // straight-line loads of rows in range (n >= 1; frob_finish drops the
    // values past n), so the compiler can wait for exactly these loads later
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = (int)threadIdx.x + 512 * k;
        v[k] = rows[r < n ? r : n - 1];
    }
}
__device__ inline float frob_finish(const float* rows, int n, const float v[4], float* red) {
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += ((int)threadIdx.x + 512 * k < n) ? v[k] : 0.f;
    for (int r = (int)threadIdx.x + 2048; r < n; r += 512) s += rows[r];
    s = wave_sum(s);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = s;
    // LDS-only barrier: waits for this wave's LDS write, not for other memory
    // operations in flight (the caller's direct LDS loads may be)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) t += red[w];
    return 1.0f / (sqrtf(t) + kEps);
}

// Remap blockIdx so that consecutive job indices land on the same XCD (blocks
// are dispatched round-robin over the XCDs).  grid must be a multiple of kXcds.
__device__ inline int xcd_job_index() {
    const int b = blockIdx.x;
    const int per_xcd = gridDim.x / kXcds;
    return (b % kXcds) * per_xcd + b / kXcds;
}

}  // namespace muon
