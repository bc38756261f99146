// Streaming kernels of the Muon step: momentum / row-norm / NS-input preparation
// (prep), the per-matrix Frobenius scale (frob, when the first Gram launch
// cannot fold it in), the weight update (apply), the multi-tensor weight EMA
// (ema), the EMA swap-in (swap) and AdamW for the non-matrix parameters
// (adamw).  All are HBM-bound: coalesced fp32 streams, float4 where the
// pointers allow, wavefront-shuffle reductions in a fixed order.
//
// Method: "Record: L_ParallelResiduals_UNetSkips_DepthRecur_Muon_ 1.0901"
// (PR #1893), "Architecture and training stack" (Muon with momentum, weight
// EMA); "Record: Combined 3-Layer Recurrence + Parallel Residuals + Polar
// Express + Brotli" (PR #1396), "Techniques Combined" (MuonEq-R row norm before
// NS, WD 0.105); "Record: Improved Parallel Residuals + Systems Optimization"
// (PR #1584), "Summary" (batched EMA over all parameters).
#include "common.h"
#include "kernels.h"

namespace muon {

namespace {

template <typename Tab>
__device__ inline int find_tensor(const Tab* t, int n, int blk) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t[mid].block_begin <= blk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Momentum: M' = mu*M + G;  U = G + mu*M' (Nesterov) or M'.
__device__ inline float momentum_u(float g, float m, float mu, int nesterov, float& m_new) {
    m_new = fmaf(mu, m, g);
    return nesterov ? fmaf(mu, m_new, g) : m_new;
}

// X element stores and loads.  bf16: hi plane plus either a bf16 lo plane or,
// for base-precision groups (lo8), a byte plane (see lo8_insert); fp32: one plane.
template <int PREC>
__device__ inline void store_x(void* xh, void* xl, size_t idx, float v, bool lo8) {
    if (PREC == kNsBf16) {
        const bf16 h = to_bf16(v);
        static_cast<bf16*>(xh)[idx] = h;
        if (lo8) static_cast<uint8_t*>(xl)[idx] = (uint8_t)lo8_insert(v, from_bf16(h), 0u, 0);
        else static_cast<bf16*>(xl)[idx] = to_bf16(v - from_bf16(h));
    } else {
        static_cast<float*>(xh)[idx] = v;
    }
}

template <int PREC>
__device__ inline float load_x(const void* xh, const void* xl, size_t idx, bool lo8) {
    if (PREC == kNsBf16) {
        const float h = from_bf16(static_cast<const bf16*>(xh)[idx]);
        if (lo8) return lo8_decode(h, static_cast<const uint8_t*>(xl)[idx], 0);
        return h + from_bf16(static_cast<const bf16*>(xl)[idx]);
    } else {
        return static_cast<const float*>(xh)[idx];
    }
}

// Four consecutive X elements (idx a multiple of 4).
template <int PREC>
__device__ inline void store_x4(void* xh, void* xl, size_t idx, float4 v, bool lo8) {
    if (PREC == kNsBf16) {
        const float x[4] = {v.x, v.y, v.z, v.w};
        u32x2 ph;
        ph.x = pack_bf16x2(x[0], x[1]);
        ph.y = pack_bf16x2(x[2], x[3]);
        const float h[4] = {bf16_lo_f(ph.x), bf16_hi_f(ph.x), bf16_lo_f(ph.y), bf16_hi_f(ph.y)};
        *reinterpret_cast<u32x2*>(static_cast<bf16*>(xh) + idx) = ph;
        if (lo8) {
            uint32_t q = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) q = lo8_insert(x[e], h[e], q, e);
            *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(xl) + idx) = q;
        } else {
            u32x2 pl;
            pl.x = pack_bf16x2(x[0] - h[0], x[1] - h[1]);
            pl.y = pack_bf16x2(x[2] - h[2], x[3] - h[3]);
            *reinterpret_cast<u32x2*>(static_cast<bf16*>(xl) + idx) = pl;
        }
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(xh) + idx) = v;
    }
}

template <int PREC>
__device__ inline float4 load_x4(const void* xh, const void* xl, size_t idx, bool lo8) {
    if (PREC == kNsBf16) {
        const u32x2 h = *reinterpret_cast<const u32x2*>(static_cast<const bf16*>(xh) + idx);
        const float hf[4] = {from_bf16(bits_bf16(h.x & 0xFFFFu)), from_bf16(bits_bf16(h.x >> 16)),
                             from_bf16(bits_bf16(h.y & 0xFFFFu)), from_bf16(bits_bf16(h.y >> 16))};
        float r[4];
        if (lo8) {
            const uint32_t q = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(xl) + idx);
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = lo8_decode(hf[e], q, e);
        } else {
            const u32x2 l = *reinterpret_cast<const u32x2*>(static_cast<const bf16*>(xl) + idx);
            r[0] = hf[0] + from_bf16(bits_bf16(l.x & 0xFFFFu));
            r[1] = hf[1] + from_bf16(bits_bf16(l.x >> 16));
            r[2] = hf[2] + from_bf16(bits_bf16(l.y & 0xFFFFu));
            r[3] = hf[3] + from_bf16(bits_bf16(l.y >> 16));
        }
        return make_float4(r[0], r[1], r[2], r[3]);
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(xh) + idx);
    }
}

// One stored row of up to 4 * 64 * RV floats (cols % 4 == 0, 16-byte
// aligned), one wavefront, a single pass over G and M: M' is written at once,
// U stays in registers until the row norm is known, then r = U/(|U|+eps) (or U)
// is handed to emit4 four elements at a time.  Returns sum(r^2) on every lane.
template <int RV, typename Emit4>
__device__ inline float process_row_regs(const float* __restrict__ g, float* __restrict__ m, int cols, float mu,
                                         int nesterov, int row_norm, int lane, Emit4 emit4) {
    const float4* g4 = reinterpret_cast<const float4*>(g);
    float4* m4 = reinterpret_cast<float4*>(m);
    const int nv = cols / 4;
    float4 u[RV];
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < RV; ++v) {
        const int j = lane + v * kWave;
        if (j < nv) {
            // G and M are read once and M' is not read again in the step: streaming
            // (non-temporal) accesses leave the caches to the NS chain's planes
            const floatx4 gx = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(g4 + j));
            const floatx4 mx = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(m4 + j));
            const float4 gv = make_float4(gx[0], gx[1], gx[2], gx[3]), mv = make_float4(mx[0], mx[1], mx[2], mx[3]);
            float4 mn;
            u[v].x = momentum_u(gv.x, mv.x, mu, nesterov, mn.x);
            u[v].y = momentum_u(gv.y, mv.y, mu, nesterov, mn.y);
            u[v].z = momentum_u(gv.z, mv.z, mu, nesterov, mn.z);
            u[v].w = momentum_u(gv.w, mv.w, mu, nesterov, mn.w);
            const floatx4 mnx = {mn.x, mn.y, mn.z, mn.w};
            __builtin_nontemporal_store(mnx, reinterpret_cast<floatx4*>(m4 + j));
            ss = fmaf(u[v].x, u[v].x, ss); ss = fmaf(u[v].y, u[v].y, ss);
            ss = fmaf(u[v].z, u[v].z, ss); ss = fmaf(u[v].w, u[v].w, ss);
        }
    }
    ss = wave_sum(ss);
    const float denom = sqrtf(ss) + kEps;
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < RV; ++v) {
        const int j = lane + v * kWave;
        if (j < nv) {
            float4 r = u[v];
            if (row_norm) { r.x /= denom; r.y /= denom; r.z /= denom; r.w /= denom; }
            rs = fmaf(r.x, r.x, rs); rs = fmaf(r.y, r.y, rs); rs = fmaf(r.z, r.z, rs); rs = fmaf(r.w, r.w, rs);
            emit4(4 * j, r);
        }
    }
    return wave_sum(rs);
}

// One stored row, one wavefront.  Pass 1 reduces sum(U^2) (no writes); pass 2
// recomputes U, writes M', and hands r = U/(|U|+eps) (or U) to `emit`.
// Returns sum(r^2) on every lane.
template <typename Emit>
__device__ inline float process_row(const float* __restrict__ g, float* __restrict__ m, int cols, int vec,
                                    float mu, int nesterov, int row_norm, int lane, Emit emit) {
    float ss = 0.f;
    if (vec) {
        const float4* g4 = reinterpret_cast<const float4*>(g);
        const float4* m4 = reinterpret_cast<const float4*>(m);
        for (int j = lane; j < cols / 4; j += kWave) {
            const float4 gv = g4[j], mv = m4[j];
            float t;
            const float u0 = momentum_u(gv.x, mv.x, mu, nesterov, t);
            const float u1 = momentum_u(gv.y, mv.y, mu, nesterov, t);
            const float u2 = momentum_u(gv.z, mv.z, mu, nesterov, t);
            const float u3 = momentum_u(gv.w, mv.w, mu, nesterov, t);
            ss = fmaf(u0, u0, ss); ss = fmaf(u1, u1, ss); ss = fmaf(u2, u2, ss); ss = fmaf(u3, u3, ss);
        }
    } else {
        for (int j = lane; j < cols; j += kWave) {
            float t;
            const float u = momentum_u(g[j], m[j], mu, nesterov, t);
            ss = fmaf(u, u, ss);
        }
    }
    ss = wave_sum(ss);
    const float denom = sqrtf(ss) + kEps;
    float rs = 0.f;
    if (vec) {
        const float4* g4 = reinterpret_cast<const float4*>(g);
        float4* m4 = reinterpret_cast<float4*>(m);
        for (int j = lane; j < cols / 4; j += kWave) {
            const float4 gv = g4[j], mv = m4[j];
            float4 mn;
            float4 u;
            u.x = momentum_u(gv.x, mv.x, mu, nesterov, mn.x);
            u.y = momentum_u(gv.y, mv.y, mu, nesterov, mn.y);
            u.z = momentum_u(gv.z, mv.z, mu, nesterov, mn.z);
            u.w = momentum_u(gv.w, mv.w, mu, nesterov, mn.w);
            m4[j] = mn;
            if (row_norm) { u.x /= denom; u.y /= denom; u.z /= denom; u.w /= denom; }
            rs = fmaf(u.x, u.x, rs); rs = fmaf(u.y, u.y, rs); rs = fmaf(u.z, u.z, rs); rs = fmaf(u.w, u.w, rs);
            emit(4 * j + 0, u.x); emit(4 * j + 1, u.y); emit(4 * j + 2, u.z); emit(4 * j + 3, u.w);
        }
    } else {
        for (int j = lane; j < cols; j += kWave) {
            float mn;
            float u = momentum_u(g[j], m[j], mu, nesterov, mn);
            m[j] = mn;
            if (row_norm) u /= denom;
            rs = fmaf(u, u, rs);
            emit(j, u);
        }
    }
    return wave_sum(rs);
}

// RV: float4 per lane a row may keep in registers (rows of up to 256 * RV floats
// take the single-pass path; longer rows re-read G and M).
template <int PREC, int RV>
__global__ __launch_bounds__(256) void prep_kernel(const PrepArgs a) {
    extern __shared__ float lds_rows[];
    const int ti = find_tensor(a.t, a.n, blockIdx.x);
    const PrepTensor& T = a.t[ti];
    const int blk = blockIdx.x - T.block_begin;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const size_t ld = (size_t)T.n_pad;

    if (!T.transposed) {
        // X0 row i is stored row i; rows in [rows, m_pad) and cols in [cols, n_pad) are zero.
        const int row = blk * kRowsPerWaveBlock + wave;
        if (row >= T.m_pad) return;
        const size_t xrow = (size_t)row * ld;
        if (row < T.rows) {
            const float* g = T.grad + (size_t)row * T.cols;
            float* m = T.mom + (size_t)row * T.cols;
            float rs;
            if (T.vec && T.cols <= 4 * kWave * RV) {
                rs = process_row_regs<RV>(g, m, T.cols, a.mu, a.nesterov, a.row_norm, lane,
                                          [&](int j, float4 r) { store_x4<PREC>(T.xh, T.xl, xrow + j, r, T.lo8); });
                const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int j = T.cols + 4 * lane; j < T.n_pad; j += 4 * kWave) store_x4<PREC>(T.xh, T.xl, xrow + j, z, T.lo8);
            } else {
                rs = process_row(g, m, T.cols, T.vec, a.mu, a.nesterov, a.row_norm, lane,
                                 [&](int j, float r) { store_x<PREC>(T.xh, T.xl, xrow + j, r, T.lo8); });
                for (int j = T.cols + lane; j < T.n_pad; j += kWave) store_x<PREC>(T.xh, T.xl, xrow + j, 0.f, T.lo8);
            }
            if (lane == 0) T.rowsq[row] = rs;
        } else {
            const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int j = 4 * lane; j < T.n_pad; j += 4 * kWave) store_x4<PREC>(T.xh, T.xl, xrow + j, z, T.lo8);
        }
        return;
    }

    // Transposed: X0[j][i] = r[i][j].  The workgroup owns stored rows
    // [blk*rb, blk*rb + rb), stages r in LDS, then writes X0 columns
    // [blk*rb, blk*rb + rb) for every X0 row j in [0, m_pad).
    const int rb = T.rb;
    const int pitch = T.cols + 1;
    const int row0 = blk * rb;
    for (int rr = wave; rr < rb; rr += 4) {
        const int row = row0 + rr;
        float* dst = lds_rows + (size_t)rr * pitch;
        if (row < T.rows) {
            const float* g = T.grad + (size_t)row * T.cols;
            float* m = T.mom + (size_t)row * T.cols;
            float rs;
            if (T.vec && T.cols <= 4 * kWave * RV) {
                rs = process_row_regs<RV>(g, m, T.cols, a.mu, a.nesterov, a.row_norm, lane, [&](int j, float4 r) {
                    dst[j] = r.x; dst[j + 1] = r.y; dst[j + 2] = r.z; dst[j + 3] = r.w;
                });
            } else {
                rs = process_row(g, m, T.cols, T.vec, a.mu, a.nesterov, a.row_norm, lane,
                                 [&](int j, float r) { dst[j] = r; });
            }
            if (lane == 0) T.rowsq[row] = rs;
        } else {
            for (int j = lane; j < T.cols; j += kWave) dst[j] = 0.f;
        }
    }
    __syncthreads();
    if (rb % 4 == 0) {
        // four consecutive X0 columns (= stored rows) per item: 8-byte bf16 stores
        const int rq = rb / 4;
        const int items = T.m_pad * rq;
        for (int it = threadIdx.x; it < items; it += blockDim.x) {
            const int j = it / rq;
            const int rr = 4 * (it - j * rq);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < T.cols) {
                v.x = lds_rows[(size_t)(rr + 0) * pitch + j];
                v.y = lds_rows[(size_t)(rr + 1) * pitch + j];
                v.z = lds_rows[(size_t)(rr + 2) * pitch + j];
                v.w = lds_rows[(size_t)(rr + 3) * pitch + j];
            }
            store_x4<PREC>(T.xh, T.xl, (size_t)j * ld + row0 + rr, v, T.lo8);
        }
    } else {
        const int items = T.m_pad * rb;
        for (int it = threadIdx.x; it < items; it += blockDim.x) {
            const int j = it / rb;
            const int rr = it - j * rb;
            const float v = (j < T.cols) ? lds_rows[(size_t)rr * pitch + j] : 0.f;
            store_x<PREC>(T.xh, T.xl, (size_t)j * ld + row0 + rr, v, T.lo8);
        }
    }
}

// One workgroup per matrix: scale = 1 / (sqrt(sum of the row sums) + eps),
// summed in the fixed order of frob_prefetch / frob_finish.
__global__ __launch_bounds__(512) void frob_kernel(const FrobArgs a) {
    __shared__ float red[8];
    const int i = blockIdx.x;
    const float* rs = a.rowsq + a.rowsq_off[i];
    float v[4];
    frob_prefetch(rs, a.rows[i], v);
    const float s = frob_finish(rs, a.rows[i], v, red);
    if (threadIdx.x == 0) a.scale[a.scale_idx[i]] = s;
}

// W' = keep*W - lr_s*O with O = fac*X (fac = Frobenius scale when no NS step ran).
template <int PREC>
__global__ __launch_bounds__(256) void apply_kernel(const ApplyArgs a) {
    extern __shared__ float lds_o[];
    const int ti = find_tensor(a.t, a.n, blockIdx.x);
    const ApplyTensor& T = a.t[ti];
    const int blk = blockIdx.x - T.block_begin;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const float fac = a.use_scale ? *T.scale : 1.0f;
    const float keep = a.keep;
    const float lr_s = T.lr_s;
    const float d = a.decay, omd = a.one_minus_decay;
    const size_t ld = (size_t)T.n_pad;

    if (!T.transposed) {
        const int row = blk * kRowsPerWaveBlock + wave;
        if (row >= T.rows) return;
        float* w = T.param + (size_t)row * T.cols;
        float* out = T.out ? T.out + (size_t)row * T.cols : nullptr;
        float* ema = T.ema ? T.ema + (size_t)row * T.cols : nullptr;
        const size_t xrow = (size_t)row * ld;
        if (T.vec) {
            float4* w4 = reinterpret_cast<float4*>(w);
            float4* o4 = reinterpret_cast<float4*>(out);
            float4* e4 = reinterpret_cast<float4*>(ema);
            for (int j = lane; j < T.cols / 4; j += kWave) {
                float4 o = load_x4<PREC>(T.xh, T.xl, xrow + 4 * j, T.lo8);
                o.x *= fac; o.y *= fac; o.z *= fac; o.w *= fac;
                float4 wv = w4[j];
                wv.x = fmaf(-lr_s, o.x, keep * wv.x);
                wv.y = fmaf(-lr_s, o.y, keep * wv.y);
                wv.z = fmaf(-lr_s, o.z, keep * wv.z);
                wv.w = fmaf(-lr_s, o.w, keep * wv.w);
                w4[j] = wv;
                if (o4) o4[j] = o;
                if (e4) {
                    float4 ev = e4[j];
                    ev.x = fmaf(d, ev.x, omd * wv.x);
                    ev.y = fmaf(d, ev.y, omd * wv.y);
                    ev.z = fmaf(d, ev.z, omd * wv.z);
                    ev.w = fmaf(d, ev.w, omd * wv.w);
                    e4[j] = ev;
                }
            }
        } else {
            for (int j = lane; j < T.cols; j += kWave) {
                const float o = fac * load_x<PREC>(T.xh, T.xl, xrow + j, T.lo8);
                const float wv = fmaf(-lr_s, o, keep * w[j]);
                w[j] = wv;
                if (out) out[j] = o;
                if (ema) ema[j] = fmaf(d, ema[j], omd * wv);
            }
        }
        return;
    }

    // Transposed: O[i][j] = X[j][i].  Stage X columns [row0, row0+rb) in LDS.
    const int rb = T.rb;
    const int pitch = T.cols + 1;
    const int row0 = blk * rb;
    if (rb % 4 == 0) {
        // X columns row0 .. row0+rb lie in the zero-padded plane (n_pad >= row0 + rb)
        const int rq = rb / 4;
        const int items = T.cols * rq;
        for (int it = threadIdx.x; it < items; it += blockDim.x) {
            const int j = it / rq;
            const int rr = 4 * (it - j * rq);
            const float4 v = load_x4<PREC>(T.xh, T.xl, (size_t)j * ld + row0 + rr, T.lo8);
            lds_o[(size_t)(rr + 0) * pitch + j] = fac * v.x;
            lds_o[(size_t)(rr + 1) * pitch + j] = fac * v.y;
            lds_o[(size_t)(rr + 2) * pitch + j] = fac * v.z;
            lds_o[(size_t)(rr + 3) * pitch + j] = fac * v.w;
        }
    } else {
        const int items = T.cols * rb;
        for (int it = threadIdx.x; it < items; it += blockDim.x) {
            const int j = it / rb;
            const int rr = it - j * rb;
            lds_o[(size_t)rr * pitch + j] = fac * load_x<PREC>(T.xh, T.xl, (size_t)j * ld + row0 + rr, T.lo8);
        }
    }
    __syncthreads();
    for (int rr = wave; rr < rb; rr += 4) {
        const int row = row0 + rr;
        if (row >= T.rows) break;
        float* w = T.param + (size_t)row * T.cols;
        float* out = T.out ? T.out + (size_t)row * T.cols : nullptr;
        float* ema = T.ema ? T.ema + (size_t)row * T.cols : nullptr;
        const float* o = lds_o + (size_t)rr * pitch;
        for (int j = lane; j < T.cols; j += kWave) {
            const float wv = fmaf(-lr_s, o[j], keep * w[j]);
            w[j] = wv;
            if (out) out[j] = o[j];
            if (ema) ema[j] = fmaf(d, ema[j], omd * wv);
        }
    }
}

// E' = d*E + (1-d)*P over a chunk of kEmaElemsPerBlock elements of one tensor.
__global__ __launch_bounds__(kEmaThreads) void ema_kernel(const EmaArgs a) {
    const int ti = find_tensor(a.t, a.n, blockIdx.x);
    const EmaTensor& T = a.t[ti];
    const int64_t base = (int64_t)(blockIdx.x - T.block_begin) * kEmaElemsPerBlock;
    const int64_t end = min(base + (int64_t)kEmaElemsPerBlock, (int64_t)T.numel);
    const float d = a.decay, omd = a.one_minus_decay;
    const bool vec = ((reinterpret_cast<uintptr_t>(T.ema) | reinterpret_cast<uintptr_t>(T.param)) & 15) == 0;
    if (vec && end - base == kEmaElemsPerBlock) {
        floatx4* e4 = reinterpret_cast<floatx4*>(T.ema + base);
        const floatx4* p4 = reinterpret_cast<const floatx4*>(T.param + base);
        floatx4 ev[kEmaVec], pv[kEmaVec];
#pragma unroll
        for (int k = 0; k < kEmaVec; ++k) {
            ev[k] = __builtin_nontemporal_load(e4 + threadIdx.x + k * kEmaThreads);
            pv[k] = __builtin_nontemporal_load(p4 + threadIdx.x + k * kEmaThreads);
        }
#pragma unroll
        for (int k = 0; k < kEmaVec; ++k) {
            floatx4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = fmaf(d, ev[k][e], omd * pv[k][e]);
            __builtin_nontemporal_store(r, e4 + threadIdx.x + k * kEmaThreads);
        }
        return;
    }
    for (int64_t i = base + threadIdx.x; i < end; i += kEmaThreads) {
        T.ema[i] = fmaf(d, T.ema[i], omd * T.param[i]);
    }
}

// Exchange a chunk of kEmaElemsPerBlock elements of two buffers (bit for bit).
__global__ __launch_bounds__(kEmaThreads) void swap_kernel(const SwapArgs a) {
    const int ti = find_tensor(a.t, a.n, blockIdx.x);
    const SwapTensor& T = a.t[ti];
    const int64_t base = (int64_t)(blockIdx.x - T.block_begin) * kEmaElemsPerBlock;
    const int64_t end = min(base + (int64_t)kEmaElemsPerBlock, (int64_t)T.numel);
    const bool vec = ((reinterpret_cast<uintptr_t>(T.a) | reinterpret_cast<uintptr_t>(T.b)) & 15) == 0;
    if (vec && end - base == kEmaElemsPerBlock) {
        floatx4* a4 = reinterpret_cast<floatx4*>(T.a + base);
        floatx4* b4 = reinterpret_cast<floatx4*>(T.b + base);
        floatx4 av[kEmaVec], bv[kEmaVec];
#pragma unroll
        for (int k = 0; k < kEmaVec; ++k) {
            av[k] = __builtin_nontemporal_load(a4 + threadIdx.x + k * kEmaThreads);
            bv[k] = __builtin_nontemporal_load(b4 + threadIdx.x + k * kEmaThreads);
        }
#pragma unroll
        for (int k = 0; k < kEmaVec; ++k) {
            __builtin_nontemporal_store(bv[k], a4 + threadIdx.x + k * kEmaThreads);
            __builtin_nontemporal_store(av[k], b4 + threadIdx.x + k * kEmaThreads);
        }
        return;
    }
    for (int64_t i = base + threadIdx.x; i < end; i += kEmaThreads) {
        const float x = T.a[i];
        T.a[i] = T.b[i];
        T.b[i] = x;
    }
}

// AdamW on one element: decoupled decay of the pre-update parameter, moment
// updates, bias-corrected step (the host folds 1/(1 - beta1^t) into step_size
// and 1/sqrt(1 - beta2^t) into inv_sqrt_bc2).
__device__ inline float adamw_elem(const AdamArgs& a, float p, float g, float& m, float& v) {
    m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
    v = fmaf(a.beta2, v, a.one_minus_beta2 * (g * g));
    const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
    return fmaf(-a.step_size, m / denom, a.keep * p);
}

// AdamW (then the EMA on the updated parameter, where one is given) over a
// chunk of kAdamElemsPerBlock elements of one tensor.  Streaming: every
// operand is read and written once, with 16-byte non-temporal accesses.
__global__ __launch_bounds__(kAdamThreads) void adamw_kernel(const AdamArgs a) {
    const int ti = find_tensor(a.t, a.n, blockIdx.x);
    const AdamTensor& T = a.t[ti];
    const int64_t base = (int64_t)(blockIdx.x - T.block_begin) * kAdamElemsPerBlock;
    const int64_t end = min(base + (int64_t)kAdamElemsPerBlock, T.numel);
    const float d = a.decay, omd = a.one_minus_decay;
    if (T.vec && end - base == kAdamElemsPerBlock) {
        floatx4* p4 = reinterpret_cast<floatx4*>(T.param + base);
        const floatx4* g4 = reinterpret_cast<const floatx4*>(T.grad + base);
        floatx4* m4 = reinterpret_cast<floatx4*>(T.m + base);
        floatx4* v4 = reinterpret_cast<floatx4*>(T.v + base);
        floatx4* e4 = T.ema ? reinterpret_cast<floatx4*>(T.ema + base) : nullptr;
        floatx4 pv[2], gv[2], mv[2], vv[2], ev[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int j = threadIdx.x + k * kAdamThreads;
            pv[k] = __builtin_nontemporal_load(p4 + j);
            gv[k] = __builtin_nontemporal_load(g4 + j);
            mv[k] = __builtin_nontemporal_load(m4 + j);
            vv[k] = __builtin_nontemporal_load(v4 + j);
            if (e4) ev[k] = __builtin_nontemporal_load(e4 + j);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int j = threadIdx.x + k * kAdamThreads;
            floatx4 pn, mn, vn;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float m = mv[k][e], v = vv[k][e];
                pn[e] = adamw_elem(a, pv[k][e], gv[k][e], m, v);
                mn[e] = m;
                vn[e] = v;
            }
            __builtin_nontemporal_store(pn, p4 + j);
            __builtin_nontemporal_store(mn, m4 + j);
            __builtin_nontemporal_store(vn, v4 + j);
            if (e4) {
                floatx4 en;
#pragma unroll
                for (int e = 0; e < 4; ++e) en[e] = fmaf(d, ev[k][e], omd * pn[e]);
                __builtin_nontemporal_store(en, e4 + j);
            }
        }
        return;
    }
    for (int64_t i = base + threadIdx.x; i < end; i += kAdamThreads) {
        float m = T.m[i], v = T.v[i];
        const float p = adamw_elem(a, T.param[i], T.grad[i], m, v);
        T.param[i] = p;
        T.m[i] = m;
        T.v[i] = v;
        if (T.ema) T.ema[i] = fmaf(d, T.ema[i], omd * p);
    }
}

}  // namespace

template <typename K>
hipError_t allow_lds(K kernel, size_t lds_bytes) {
    // dynamic LDS beyond the default 64 KiB must be requested (gfx950: 160 KiB per CU)
    if (lds_bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds_bytes);
}

template <int PREC, int RV>
hipError_t launch_prep_rv(const PrepArgs& a, int blocks, size_t lds_bytes, hipStream_t s) {
    hipError_t e = allow_lds(&prep_kernel<PREC, RV>, lds_bytes);
    if (e != hipSuccess) return e;
    prep_kernel<PREC, RV><<<blocks, 256, lds_bytes, s>>>(a);
    return hipGetLastError();
}

template <int PREC>
hipError_t launch_prep_prec(const PrepArgs& a, int max_cols, int blocks, size_t lds_bytes, hipStream_t s) {
    // the register row buffer sized to the widest row of the launch keeps occupancy up
    if (max_cols <= 1024) return launch_prep_rv<PREC, 4>(a, blocks, lds_bytes, s);
    if (max_cols <= 2048) return launch_prep_rv<PREC, 8>(a, blocks, lds_bytes, s);
    return launch_prep_rv<PREC, 16>(a, blocks, lds_bytes, s);
}

hipError_t launch_prep(const PrepArgs& a, int precision, int blocks, size_t lds_bytes, hipStream_t s) {
    int max_cols = 0;
    for (int i = 0; i < a.n; ++i) max_cols = max(max_cols, a.t[i].cols);
    if (precision == kNsBf16) return launch_prep_prec<kNsBf16>(a, max_cols, blocks, lds_bytes, s);
    return launch_prep_prec<kNsFp32>(a, max_cols, blocks, lds_bytes, s);
}

hipError_t launch_frob(const FrobArgs& a, hipStream_t s) {
    frob_kernel<<<a.n, 512, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_apply(const ApplyArgs& a, int precision, int blocks, size_t lds_bytes, hipStream_t s) {
    hipError_t e;
    if (precision == kNsBf16) {
        if ((e = allow_lds(&apply_kernel<kNsBf16>, lds_bytes)) != hipSuccess) return e;
        apply_kernel<kNsBf16><<<blocks, 256, lds_bytes, s>>>(a);
    } else {
        if ((e = allow_lds(&apply_kernel<kNsFp32>, lds_bytes)) != hipSuccess) return e;
        apply_kernel<kNsFp32><<<blocks, 256, lds_bytes, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_ema(const EmaArgs& a, int blocks, hipStream_t s) {
    ema_kernel<<<blocks, kEmaThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_swap(const SwapArgs& a, int blocks, hipStream_t s) {
    swap_kernel<<<blocks, kEmaThreads, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamArgs& a, int blocks, hipStream_t s) {
    adamw_kernel<<<blocks, kAdamThreads, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace muon
